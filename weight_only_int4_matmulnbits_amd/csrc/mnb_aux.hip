// The kernels around the matmul on the vocabulary and import side.
//
// Page "Qwen3 CPU Inference Critical Path":
//  * "Export contract", qwen3-int4-qdq: a projection is a logical UINT4[K][N]
//    in ONNX row-major, low-nibble-first storage whose DequantizeLinear blocks
//    run along axis 0; the tied embedding / LM-head weight is a logical
//    UINT4[vocabulary][hidden] blocked along axis 1; an artifact in another
//    layout is normalized before it is matched.  import_* normalize either
//    into the MatMulNBits storage (a one-time preparation, like packing).
//  * The same section and "Operator priority" (Gather): the optimized plan
//    dequantizes only the selected embedding rows of the tied weight and
//    streams the same packed bytes for the LM head (N = vocabulary): row v of
//    the embedding is column v of the MatMulNBits B.  gather_rows_kernel.
//  * "Phase Q2" (final RMSNorm, LM-head GEMV and greedy ArgMax):
//    argmax_kernel, the greedy choice over the logits.
#include <math.h>

#include "mnb_internal.h"

namespace mnb {
namespace {

__device__ __forceinline__ uint32_t nibble_at(const uint8_t* p, int64_t i) {
    const uint8_t b = p[i >> 1];
    return (i & 1) ? (uint32_t)(b >> 4) : (uint32_t)(b & 0xF);
}

// ---- QDQ import ----------------------------------------------------------------
// One workgroup moves 64 columns x 128 values of K through LDS: the reads
// follow the QDQ element order (n fastest for axis 0, k fastest for axis 1),
// the writes the MatMulNBits one (the bytes of a column are contiguous; byte
// j of a column holds k = 2j in the low nibble and 2j + 1 in the high one).
// Values past K (the partial last block) are written as zeros.
constexpr int kTileN = 64, kTileK = 128;

__global__ __launch_bounds__(256) void import_weights_kernel(const uint8_t* __restrict__ wq,
                                                             uint8_t* __restrict__ out, int64_t K,
                                                             int64_t N, int64_t col_bytes, int axis) {
    __shared__ uint8_t tile[kTileK][kTileN + 1];
    const int64_t n0 = (int64_t)blockIdx.x * kTileN;
    const int64_t k0 = (int64_t)blockIdx.y * kTileK;
    for (int i = threadIdx.x; i < kTileK * kTileN; i += blockDim.x) {
        const int kk = axis == 0 ? i / kTileN : i % kTileK;
        const int nn = axis == 0 ? i % kTileN : i / kTileK;
        const int64_t k = k0 + kk, n = n0 + nn;
        uint32_t v = 0;
        if (k < K && n < N) v = nibble_at(wq, axis == 0 ? k * N + n : n * K + k);
        tile[kk][nn] = (uint8_t)v;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < kTileN * (kTileK / 2); i += blockDim.x) {
        const int nn = i / (kTileK / 2), jj = i % (kTileK / 2);
        const int64_t n = n0 + nn, j = k0 / 2 + jj;
        if (n < N && j < col_bytes) out[n * col_bytes + j] = (uint8_t)(tile[2 * jj][nn] | (tile[2 * jj + 1][nn] << 4));
    }
}

// One thread per packed zero-point byte (blocks 2j and 2j + 1 of column n).
// Without a zero-point tensor DequantizeLinear uses 0, written explicitly.
__global__ __launch_bounds__(256) void import_zero_points_kernel(const uint8_t* __restrict__ zq,
                                                                 uint8_t* __restrict__ out, int64_t N,
                                                                 int nb, int row, int axis, int64_t total) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total) return;
    const int64_t n = i / row;
    const int j = (int)(i - n * row);
    uint32_t v[2] = {0, 0};
    for (int h = 0; h < 2; h++) {
        const int b = 2 * j + h;
        if (zq && b < nb) v[h] = nibble_at(zq, axis == 0 ? (int64_t)b * N + n : n * nb + b);
    }
    out[i] = (uint8_t)(v[0] | (v[1] << 4));
}

// One thread per scale: [nb][N] (axis 0) or [N][nb] (axis 1) into [N][nb].
template <typename T>
__global__ __launch_bounds__(256) void import_scales_kernel(const T* __restrict__ in, T* __restrict__ out,
                                                            int64_t N, int nb, int axis, int64_t total) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total) return;
    const int64_t n = i / nb;
    const int b = (int)(i - n * nb);
    out[i] = in[axis == 0 ? (int64_t)b * N + n : i];
}

// ---- tied-embedding gather ------------------------------------------------------
// out[t][k] = dequant(B)[k][ids[t]], one thread per packed byte (k = 2j and
// 2j + 1), rounded once to the output type exactly as the dequantization hook
// does: float32 by one rounding of (q - zp) * s, bfloat16 by one rounding of
// the exact product (a bfloat16 scale times a 5-bit integer is exact in
// float32).  A negative id counts from the end (ids in [-N, N)); a row whose
// id lies outside is written as NaN and reads nothing.
__global__ __launch_bounds__(256) void gather_rows_kernel(Problem p, const int64_t* __restrict__ ids,
                                                          int64_t n_ids, void* __restrict__ out) {
    const int64_t pairs = (p.K + 1) / 2;
    const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= pairs) return;
    for (int64_t t = blockIdx.y; t < n_ids; t += gridDim.y) {
        int64_t id = ids[t];
        if (id < 0) id += p.N;
        const bool ok = id >= 0 && id < p.N;
        const uint8_t byte = ok ? p.b[id * p.col_bytes + j] : 0;
        for (int h = 0; h < 2; h++) {
            const int64_t k = 2 * j + h;
            if (k >= p.K) break;
            const int64_t o = t * p.K + k;
            if (!ok) {
                if (p.bf16)
                    static_cast<uint16_t*>(out)[o] = 0x7FC0;
                else
                    static_cast<uint32_t*>(out)[o] = 0x7FC00000u;
                continue;
            }
            const int b = (int)(k / p.bs);
            const int qv = h ? (byte >> 4) : (byte & 0xF);
            int zv = 8;
            if (p.zp) {
                const uint8_t zb = p.zp[id * p.zp_row + (b >> 1)];
                zv = (b & 1) ? (zb >> 4) : (zb & 0xF);
            }
            const float d = (float)(qv - zv);
            if (p.bf16) {
                const float s = bf16_to_f32(static_cast<const uint16_t*>(p.scales)[id * p.nb + b]);
                static_cast<uint16_t*>(out)[o] = f32_to_bf16_rtne(d * s);
            } else {
                const float s = static_cast<const float*>(p.scales)[id * p.nb + b];
                static_cast<float*>(out)[o] = __fmul_rn(d, s);
            }
        }
    }
}

// ---- greedy ArgMax -----------------------------------------------------------------
// Row m of x [M][N]: the first index holding the largest value, a NaN counting
// as larger than every number (the first NaN wins).  One workgroup per row;
// (value, index) pairs are compared by a total order (NaN first, then value,
// then the smaller index), so the answer does not depend on how the row is
// split among threads.
constexpr int64_t kNoIndex = INT64_MAX;

__device__ __forceinline__ bool better(float v, int64_t i, float bv, int64_t bi) {
    if (i == kNoIndex) return false;
    if (bi == kNoIndex) return true;
    const bool vn = isnan(v), bn = isnan(bv);
    if (vn != bn) return vn;
    if (!vn && v != bv) return v > bv;
    return i < bi;
}

// The best (value, index) pair of a wavefront, in every lane: an XOR
// butterfly under the total order above (the result does not depend on the
// pairing).
__device__ __forceinline__ void wave_best(float& v, int64_t& i) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const float ov = __shfl_xor(v, off, 64);
        const int64_t oi = __shfl_xor(i, off, 64);
        if (better(ov, oi, v, i)) {
            v = ov;
            i = oi;
        }
    }
}

// The best pair of a workgroup (blockDim.x a multiple of 64, at most 1024):
// per wavefront, then the wavefronts' bests in order; every thread returns it.
__device__ __forceinline__ void block_best(float& v, int64_t& i) {
    __shared__ float sv[16];
    __shared__ int64_t si[16];
    wave_best(v, i);
    const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        sv[w] = v;
        si[w] = i;
    }
    __syncthreads();
    v = sv[0];
    i = si[0];
    for (int k = 1; k < nw; k++)
        if (better(sv[k], si[k], v, i)) {
            v = sv[k];
            i = si[k];
        }
}

// Best (value, index) of row m over [n0, n1) by one workgroup: each thread
// reads 16-byte pieces (4 float32 or 8 bfloat16 values), eight pieces in
// flight per round, when the row starts 16-byte aligned and has a whole number
// of pieces (then n0 and n1 are multiples of the piece); otherwise one value
// at a time.  Every thread of the block returns the block's best.
template <bool BF16>
__device__ void best_of_range(const void* __restrict__ x, int64_t N, int64_t m, int64_t n0, int64_t n1,
                              int vec, float& out_v, int64_t& out_i) {
    const int t = threadIdx.x, T = blockDim.x;
    float bv = -INFINITY;
    int64_t bi = kNoIndex;
    if (vec) {
        constexpr int PER = BF16 ? 8 : 4;        // values per 16-byte piece
        constexpr int R = 8;                     // pieces in flight per thread
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        const u32x4* row = reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(x) + m * N * (BF16 ? 2 : 4));
        const int64_t p1 = n1 / PER;
        for (int64_t p0 = n0 / PER + t; p0 < p1; p0 += (int64_t)R * T) {
            u32x4 v[R];
#pragma unroll
            for (int r = 0; r < R; r++) {
                const int64_t pc = p0 + (int64_t)r * T;
                v[r] = pc < p1 ? row[pc] : u32x4{0, 0, 0, 0};
            }
#pragma unroll
            for (int r = 0; r < R; r++) {
                const int64_t pc = p0 + (int64_t)r * T;
                if (pc >= p1) break;
#pragma unroll
                for (int e = 0; e < PER; e++) {
                    const uint32_t w = v[r][BF16 ? e / 2 : e];
                    const float f = BF16 ? __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16)) : __uint_as_float(w);
                    if (better(f, pc * PER + e, bv, bi)) {
                        bv = f;
                        bi = pc * PER + e;
                    }
                }
            }
        }
    } else {
        for (int64_t n = n0 + t; n < n1; n += T) {
            const float v = BF16 ? bf16_to_f32(static_cast<const uint16_t*>(x)[m * N + n])
                                 : static_cast<const float*>(x)[m * N + n];
            if (better(v, n, bv, bi)) {
                bv = v;
                bi = n;
            }
        }
    }
    block_best(bv, bi);
    out_v = bv;
    out_i = bi;
}

// One workgroup per row (short rows, or no workspace).
template <bool BF16>
__global__ __launch_bounds__(1024) void argmax_kernel(const void* __restrict__ x, int64_t N, int vec,
                                                      int64_t* __restrict__ idx) {
    float v;
    int64_t i;
    best_of_range<BF16>(x, N, blockIdx.x, 0, N, vec, v, i);
    if (threadIdx.x == 0) idx[blockIdx.x] = i;
}

// Long rows: S workgroups per row write the best of their segment (segment
// boundaries are multiples of 8 values), then one workgroup per row picks
// the best of the S partials by the same total order.
struct Partial {
    float v;
    int32_t pad;
    int64_t i;
};

template <bool BF16>
__global__ __launch_bounds__(256) void argmax_partial_kernel(const void* __restrict__ x, int64_t N, int vec,
                                                             int64_t seg, Partial* __restrict__ part) {
    const int64_t m = blockIdx.y, s = blockIdx.x;
    const int64_t n0 = s * seg, n1 = n0 + seg < N ? n0 + seg : N;
    float v;
    int64_t i;
    best_of_range<BF16>(x, N, m, n0, n1, vec, v, i);
    if (threadIdx.x == 0) part[m * gridDim.x + s] = Partial{v, 0, i};
}

__global__ __launch_bounds__(256) void argmax_final_kernel(const Partial* __restrict__ part, int S,
                                                           int64_t* __restrict__ idx) {
    const int64_t m = blockIdx.x;
    const int t = threadIdx.x;
    float bv = -INFINITY;
    int64_t bi = kNoIndex;
    for (int s = t; s < S; s += blockDim.x) {
        const Partial p = part[m * S + s];
        if (better(p.v, p.i, bv, bi)) {
            bv = p.v;
            bi = p.i;
        }
    }
    block_best(bv, bi);
    if (t == 0) idx[m] = bi;
}

constexpr int64_t kArgmaxSeg = 2048;     // values per partial workgroup
constexpr int64_t kArgmaxMaxSeg = 256;   // partials per row

int64_t argmax_segments(int64_t N) {
    int64_t S = (N + kArgmaxSeg - 1) / kArgmaxSeg;
    return S > kArgmaxMaxSeg ? kArgmaxMaxSeg : S;
}

inline unsigned blocks_for(int64_t items, int threads) { return (unsigned)((items + threads - 1) / threads); }

int launched(const char* what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(MNB_E_HIP, "%s launch: %s", what, hipGetErrorString(e));
    return MNB_OK;
}

}  // namespace

int launch_import_qdq(const Problem& p, int axis, const uint8_t* w_q, const void* scales_q, const uint8_t* zp_q,
                      uint8_t* b_packed, void* scales, uint8_t* zp_packed, hipStream_t s) {
    const dim3 grid(blocks_for(p.N, kTileN), blocks_for(2 * p.col_bytes, kTileK));
    hipLaunchKernelGGL(import_weights_kernel, grid, dim3(256), 0, s, w_q, b_packed, p.K, p.N, p.col_bytes, axis);
    int st = launched("QDQ weight import");
    if (st != MNB_OK) return st;
    const int64_t ts = p.N * p.nb;
    if (p.bf16)
        hipLaunchKernelGGL(import_scales_kernel<uint16_t>, dim3(blocks_for(ts, 256)), dim3(256), 0, s,
                           static_cast<const uint16_t*>(scales_q), static_cast<uint16_t*>(scales), p.N, p.nb,
                           axis, ts);
    else
        hipLaunchKernelGGL(import_scales_kernel<uint32_t>, dim3(blocks_for(ts, 256)), dim3(256), 0, s,
                           static_cast<const uint32_t*>(scales_q), static_cast<uint32_t*>(scales), p.N, p.nb,
                           axis, ts);
    st = launched("QDQ scale import");
    if (st != MNB_OK) return st;
    const int64_t tz = p.N * p.zp_row;
    hipLaunchKernelGGL(import_zero_points_kernel, dim3(blocks_for(tz, 256)), dim3(256), 0, s, zp_q, zp_packed,
                       p.N, p.nb, p.zp_row, axis, tz);
    return launched("QDQ zero-point import");
}

int launch_gather_rows(const Problem& p, const int64_t* ids, int64_t n_ids, void* out, hipStream_t s) {
    const int64_t pairs = (p.K + 1) / 2;
    const unsigned gy = (unsigned)(n_ids < 65535 ? n_ids : 65535);
    hipLaunchKernelGGL(gather_rows_kernel, dim3(blocks_for(pairs, 256), gy), dim3(256), 0, s, p, ids, n_ids, out);
    return launched("row gather");
}

// Rows longer than one segment (up to 65,535 rows: grid.y) keep their
// per-segment partials in the caller's workspace; otherwise one workgroup
// takes a row and no workspace is used.
size_t argmax_workspace_bytes(int64_t M, int64_t N) {
    const int64_t S = argmax_segments(N);
    return S > 1 && M <= 65535 ? (size_t)(M * S) * sizeof(Partial) : 0;
}

int launch_argmax(bool bf16, int64_t M, int64_t N, const void* x, int64_t* idx, hipStream_t s, void* ws,
                  size_t ws_bytes) {
    const int per = bf16 ? 8 : 4;
    const int vec = (reinterpret_cast<uintptr_t>(x) & 15) == 0 && N % per == 0;
    const int64_t S = argmax_segments(N);
    const size_t need = argmax_workspace_bytes(M, N);
    if (need > 0 && ws && ws_bytes >= need) {
        // segment length: a multiple of 8 values (whole 16-byte pieces)
        const int64_t seg = ((N + S - 1) / S + 7) / 8 * 8;
        const int64_t Sused = (N + seg - 1) / seg;
        Partial* part = static_cast<Partial*>(ws);
        if (bf16)
            hipLaunchKernelGGL(argmax_partial_kernel<true>, dim3((unsigned)Sused, (unsigned)M), dim3(256), 0, s, x,
                               N, vec, seg, part);
        else
            hipLaunchKernelGGL(argmax_partial_kernel<false>, dim3((unsigned)Sused, (unsigned)M), dim3(256), 0, s, x,
                               N, vec, seg, part);
        int st = launched("argmax partials");
        if (st != MNB_OK) return st;
        hipLaunchKernelGGL(argmax_final_kernel, dim3((unsigned)M), dim3(256), 0, s, part, (int)Sused, idx);
        return launched("argmax");
    }
    if (bf16)
        hipLaunchKernelGGL(argmax_kernel<true>, dim3((unsigned)M), dim3(1024), 0, s, x, N, vec, idx);
    else
        hipLaunchKernelGGL(argmax_kernel<false>, dim3((unsigned)M), dim3(1024), 0, s, x, N, vec, idx);
    return launched("argmax");
}

}  // namespace mnb
