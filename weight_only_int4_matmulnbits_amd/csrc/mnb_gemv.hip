// Decode GEMV (M == 1): y[n] = sum_k a[k] * (q[n][k] - zp[n][b]) * s[n][b] + bias[n].
//
// Page "Qwen3 CPU Inference Critical Path", "INT4 MatMul is first": batch-1
// projections have one activation row and are dominated by weight traffic;
// int4_gemv partitions output columns so every weight byte is streamed once;
// decode unpacks in registers, applies zero point and scale, accumulates in
// float32, and never expands the matrix.
//
// Mapping on CDNA4.  The packed weights are N-major: column n is one run of
// col_bytes contiguous bytes.  A "chunk" is CB = min(16, bs/2) bytes of one
// column (CK = 2*CB values of K, inside one quantization block); a column has
// S = ceil(K / CK) chunks.  Each column is handled by L lanes of one
// wavefront (L a power of two <= 64, G = 64 / L columns per wavefront at a
// time); lane p owns chunks p, p + L, ..., p + (J-1)L of EVERY column it
// visits, so its J*CK activations are loaded once into registers and reused
// for all of the wavefront's columns.  For a fixed column the L lanes read L
// consecutive chunks: one fully coalesced 16-byte-per-lane load.  Per chunk a
// lane forms dot = sum a_k q_k (nibbles -> float via v_cvt_f32_ubyte), then
// acc += s * (dot - zp * sum a_k); the L partial sums of a column meet in a
// fixed butterfly across lanes.  L and J depend only on (K, block_size), so
// the float32 summation order of a column is the same whatever N is and
// wherever the column sits: concatenated launches (fused QKV, gate||up) are
// bit-identical to separate ones.  No atomics, no workspace.
#include "mnb_internal.h"

namespace mnb {
namespace {

constexpr int kJMax = 5;          // chunks per lane held in registers
constexpr int kWavesPerBlock = 4;

struct GemvArgs {
    const void* a;
    const uint8_t* b;
    const void* scales;
    const uint8_t* zp;
    const float* bias;
    void* y;
    int64_t K, N, col_bytes, n_groups;
    int nb, zp_row, S, log2_bs, log2_L;
};

template <int CB>
struct ChunkT;
template <>
struct ChunkT<16> { using type = uint4; };
template <>
struct ChunkT<8> { using type = uint2; };

template <int NW>
__device__ __forceinline__ float dot_words(const uint32_t (&w)[NW], const float* av) {
    // av[i] is the activation of value i of the chunk; word d holds values
    // 8d..8d+7, two per byte, the even one in the low nibble.
    const uint32_t m = 0x0F0F0F0Fu;
    float de = 0.f, dd = 0.f;
#pragma unroll
    for (int d = 0; d < NW; d++) {
        uint32_t lo = opaque_and(w[d], m);        // values 8d, 8d+2, 8d+4, 8d+6
        uint32_t hi = opaque_and(w[d] >> 4, m);   // values 8d+1, 8d+3, ...
        de = fmaf(av[8 * d + 0], ubyte_to_f32<0>(lo), de);
        dd = fmaf(av[8 * d + 1], ubyte_to_f32<0>(hi), dd);
        de = fmaf(av[8 * d + 2], ubyte_to_f32<1>(lo), de);
        dd = fmaf(av[8 * d + 3], ubyte_to_f32<1>(hi), dd);
        de = fmaf(av[8 * d + 4], ubyte_to_f32<2>(lo), de);
        dd = fmaf(av[8 * d + 5], ubyte_to_f32<2>(hi), dd);
        de = fmaf(av[8 * d + 6], ubyte_to_f32<3>(lo), de);
        dd = fmaf(av[8 * d + 7], ubyte_to_f32<3>(hi), dd);
    }
    return de + dd;
}

template <bool BF16, bool HAS_ZP, int CB, int J, int U>
__global__ __launch_bounds__(64 * kWavesPerBlock) void gemv_kernel(GemvArgs g) {
    constexpr int CK = 2 * CB;        // values of K per chunk
    constexpr int NW = CB / 4;        // 32-bit words per chunk
    using Chunk = typename ChunkT<CB>::type;

    const int lane = threadIdx.x & 63;
    const int L = 1 << g.log2_L;
    const int p = lane & (L - 1);     // position of this lane within its column
    const int G = 64 >> g.log2_L;     // columns per wavefront step
    const int gsub = lane >> g.log2_L;
    const int64_t wave = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
    const int64_t n_waves = (int64_t)gridDim.x * kWavesPerBlock;

    // ---- activations of this lane's chunks, kept in registers ----
    float av[J][CK];
    float asum[J];
#pragma unroll
    for (int j = 0; j < J; j++) {
        const int64_t k0 = (int64_t)(p + j * L) * CK;
        if (k0 + CK <= g.K) {
            if constexpr (BF16) {
                const uint4* src = reinterpret_cast<const uint4*>(
                    static_cast<const uint16_t*>(g.a) + k0);
#pragma unroll
                for (int v = 0; v < CK / 8; v++) {
                    uint4 x = src[v];
                    const uint32_t xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
                    for (int h = 0; h < 4; h++) {
                        av[j][8 * v + 2 * h] = __uint_as_float(xs[h] << 16);
                        av[j][8 * v + 2 * h + 1] = __uint_as_float(xs[h] & 0xFFFF0000u);
                    }
                }
            } else {
                const float4* src = reinterpret_cast<const float4*>(
                    static_cast<const float*>(g.a) + k0);
#pragma unroll
                for (int v = 0; v < CK / 4; v++) {
                    float4 x = src[v];
                    av[j][4 * v] = x.x; av[j][4 * v + 1] = x.y;
                    av[j][4 * v + 2] = x.z; av[j][4 * v + 3] = x.w;
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < CK; i++) {
                const int64_t k = k0 + i;
                float v = 0.f;
                if (k < g.K)
                    v = BF16 ? bf16_to_f32(static_cast<const uint16_t*>(g.a)[k])
                             : static_cast<const float*>(g.a)[k];
                av[j][i] = v;
            }
        }
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < CK; i++) s += av[j][i];
        asum[j] = s;
    }

    // ---- columns: U groups of G columns per iteration ----
    for (int64_t base = wave * U; base < g.n_groups; base += n_waves * U) {
        Chunk w[U][J];
        float sc[U][J];
        float zf[U][J];
        int64_t col[U];
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int64_t gi = base + u;
            col[u] = gi * G + gsub;
            const bool ok = gi < g.n_groups && col[u] < g.N;
            const uint8_t* bc = g.b + col[u] * g.col_bytes;
#pragma unroll
            for (int j = 0; j < J; j++) {
                const int c = p + j * L;
                if (ok && c < g.S) {
                    w[u][j] = *reinterpret_cast<const Chunk*>(bc + (int64_t)c * CB);
                    const int blk = (c * CK) >> g.log2_bs;
                    const int64_t si = col[u] * g.nb + blk;
                    sc[u][j] = BF16 ? bf16_to_f32(static_cast<const uint16_t*>(g.scales)[si])
                                    : static_cast<const float*>(g.scales)[si];
                    if constexpr (HAS_ZP) {
                        const uint8_t zb = g.zp[col[u] * g.zp_row + (blk >> 1)];
                        zf[u][j] = (float)((blk & 1) ? (zb >> 4) : (zb & 0xF));
                    } else {
                        zf[u][j] = 8.f;
                    }
                } else {
                    w[u][j] = Chunk{};
                    sc[u][j] = 0.f;
                    zf[u][j] = 0.f;
                }
            }
        }
        float acc[U];
#pragma unroll
        for (int u = 0; u < U; u++) {
            float s = 0.f;
#pragma unroll
            for (int j = 0; j < J; j++) {
                uint32_t words[NW];
                const uint32_t* wp = reinterpret_cast<const uint32_t*>(&w[u][j]);
#pragma unroll
                for (int d = 0; d < NW; d++) words[d] = wp[d];
                const float dot = dot_words<NW>(words, av[j]);
                const float t = fmaf(-zf[u][j], asum[j], dot);
                s = fmaf(sc[u][j], t, s);
            }
            acc[u] = s;
        }
        // butterfly over the L lanes of each column: fixed order, every lane
        // of the column ends with the same bits
        for (int off = L >> 1; off > 0; off >>= 1) {
#pragma unroll
            for (int u = 0; u < U; u++) acc[u] += __shfl_xor(acc[u], off, 64);
        }
        if (p == 0) {
#pragma unroll
            for (int u = 0; u < U; u++) {
                const int64_t gi = base + u;
                if (gi < g.n_groups && col[u] < g.N) {
                    float v = acc[u];
                    if (g.bias) v += g.bias[col[u]];
                    if constexpr (BF16)
                        static_cast<uint16_t*>(g.y)[col[u]] = f32_to_bf16_rtne(v);
                    else
                        static_cast<float*>(g.y)[col[u]] = v;
                }
            }
        }
    }
}

int ilog2(int64_t v) {
    int r = 0;
    while ((int64_t(1) << r) < v) r++;
    return r;
}

// Lanes per column and chunks per lane: a function of S = ceil(K / CK) only.
void geometry(int64_t S, int* log2_L, int* J) {
    int lL = S >= 64 ? 6 : ilog2(S);
    *log2_L = lL;
    *J = (int)((S + (1 << lL) - 1) >> lL);
}

// Columns unrolled per iteration: enough independent loads in flight with
// few chunks per lane, fewer registers with many.
constexpr int unroll_for(int J) { return J == 1 ? 4 : J == 2 ? 2 : 1; }

template <bool BF16, bool HAS_ZP, int CB>
hipError_t dispatch_j(int J, dim3 grid, hipStream_t s, const GemvArgs& a) {
    switch (J) {
        case 1: hipLaunchKernelGGL((gemv_kernel<BF16, HAS_ZP, CB, 1, unroll_for(1)>), grid, dim3(256), 0, s, a); break;
        case 2: hipLaunchKernelGGL((gemv_kernel<BF16, HAS_ZP, CB, 2, unroll_for(2)>), grid, dim3(256), 0, s, a); break;
        case 3: hipLaunchKernelGGL((gemv_kernel<BF16, HAS_ZP, CB, 3, unroll_for(3)>), grid, dim3(256), 0, s, a); break;
        case 4: hipLaunchKernelGGL((gemv_kernel<BF16, HAS_ZP, CB, 4, unroll_for(4)>), grid, dim3(256), 0, s, a); break;
        case 5: hipLaunchKernelGGL((gemv_kernel<BF16, HAS_ZP, CB, 5, unroll_for(5)>), grid, dim3(256), 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <bool BF16, bool HAS_ZP>
hipError_t dispatch_cb(int CB, int J, dim3 grid, hipStream_t s, const GemvArgs& a) {
    return CB == 16 ? dispatch_j<BF16, HAS_ZP, 16>(J, grid, s, a)
                    : dispatch_j<BF16, HAS_ZP, 8>(J, grid, s, a);
}

}  // namespace

int64_t gemv_max_k(int bs) {
    const int CK = bs >= 32 ? 32 : 16;
    return (int64_t)64 * kJMax * CK;
}

int launch_gemv(const Problem& p, hipStream_t s) {
    const int CB = p.bs >= 32 ? 16 : 8;
    const int CK = 2 * CB;
    GemvArgs a;
    a.a = p.a; a.b = p.b; a.scales = p.scales; a.zp = p.has_zp ? p.zp : nullptr;
    a.bias = p.bias; a.y = p.y;
    a.K = p.K; a.N = p.N; a.col_bytes = p.col_bytes;
    a.nb = p.nb; a.zp_row = p.zp_row;
    a.S = (int)((p.K + CK - 1) / CK);
    a.log2_bs = ilog2(p.bs);
    int J;
    geometry(a.S, &a.log2_L, &J);
    if (J > kJMax) return fail(MNB_E_UNSUPPORTED, "gemv: K=%lld beyond the register kernel", (long long)p.K);
    const int G = 64 >> a.log2_L;
    a.n_groups = (p.N + G - 1) / G;
    // at most about 2048 wavefronts (8 per CU); each takes U groups per pass
    const int U = unroll_for(J);
    int64_t waves = (a.n_groups + U - 1) / U;
    if (waves > 2048) waves = 2048;
    const unsigned blocks = (unsigned)((waves + kWavesPerBlock - 1) / kWavesPerBlock);
    hipError_t e;
    if (p.bf16)
        e = p.has_zp ? dispatch_cb<true, true>(CB, J, dim3(blocks), s, a)
                     : dispatch_cb<true, false>(CB, J, dim3(blocks), s, a);
    else
        e = p.has_zp ? dispatch_cb<false, true>(CB, J, dim3(blocks), s, a)
                     : dispatch_cb<false, false>(CB, J, dim3(blocks), s, a);
    if (e != hipSuccess) return fail(MNB_E_HIP, "gemv launch: %s", hipGetErrorString(e));
    return MNB_OK;
}

}  // namespace mnb
