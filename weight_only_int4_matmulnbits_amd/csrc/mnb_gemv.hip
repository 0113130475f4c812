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
// S = ceil(K / CK) chunks.  A column is handled by a team of W wavefronts
// (split-K across wavefronts, W in {1, 2, 4}) with L lanes each (L a power
// of two <= 64; G = 64 / L columns per wavefront step when W == 1).  Team
// lane p owns chunks p, p + L*W, ..., p + (J-1)*L*W of EVERY column it
// visits, so its J*CK activations are loaded once into registers and reused
// for all of the team's columns.  For a fixed column the lanes read
// consecutive chunks: fully coalesced 16-byte-per-lane loads, marked
// non-temporal (each weight byte is read once).
//
// Inner product in float32 on the vector ALU, about 2.25 instructions per
// weight: per 32-bit word (8 nibbles) one AND keeps the even nibbles and one
// AND keeps the odd nibbles in place (16*q), v_cvt_f32_ubyte{0..3} turn each
// byte into a float, and one FMA per weight accumulates; odd-k activations
// are held pre-multiplied by 1/16 so that (16q)(a/16) = q*a exactly.  Per
// chunk a lane forms dot = sum a_k q_k and t = dot - zp * sum a_k, then
// acc += s * t.  The L partial sums of a wavefront meet in
// a fixed DPP tree (quad_perm, row_half_mirror, row_mirror, ds_swizzle,
// readlane); the W wavefront sums meet in LDS in wavefront order.  Grid
// size, unroll and prefetch only change which wavefront handles a column,
// never the arithmetic: (L, J, W) depend only on (K, block_size), so the
// float32 summation order of a column is the same whatever N is and wherever
// the column sits -- concatenated launches (fused QKV, gate||up) are
// bit-identical to separate ones.  No atomics, no workspace.
#include "mnb_internal.h"

namespace mnb {
namespace {

constexpr int kJMax = 4;          // chunks per lane held in registers
constexpr int kWMax = 4;          // wavefronts per column (split-K)
constexpr int kWavesPerBlock = 4;
constexpr size_t kMaxLds = 64 * 1024;    // staged activations per workgroup

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

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int CB>
struct ChunkT;
template <>
struct ChunkT<16> { using type = u32x4; };
template <>
struct ChunkT<8> { using type = u32x2; };

// One 32-bit word of a chunk holds values 8d..8d+7, two per byte, the even
// one in the low nibble.  av[] holds the chunk's activations with the odd
// ones pre-multiplied by 1/16.
template <int NW>
__device__ __forceinline__ float dot_words(const uint32_t (&w)[NW], const float* av) {
    float de = 0.f, dd = 0.f;
#pragma unroll
    for (int d = 0; d < NW; d++) {
        const uint32_t lo = opaque_and(w[d], 0x0F0F0F0Fu);   // q(8d), q(8d+2), ...
        const uint32_t hi = opaque_and(w[d], 0xF0F0F0F0u);   // 16*q(8d+1), ...
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

template <int CTRL>
__device__ __forceinline__ float add_dpp(float v) {
    const int t = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true);
    return v + __builtin_bit_cast(float, t);
}

// Sum over aligned groups of 2^log2_L lanes; every lane of a group ends with
// the same bits.  The tree is fixed: pairs, quads, eights, sixteens,
// thirty-twos, then the two halves of the wavefront.
__device__ __forceinline__ float reduce_lanes(float v, int log2_L) {
    if (log2_L >= 1) v = add_dpp<0xB1>(v);     // quad_perm [1,0,3,2]
    if (log2_L >= 2) v = add_dpp<0x4E>(v);     // quad_perm [2,3,0,1]
    if (log2_L >= 3) v = add_dpp<0x141>(v);    // row_half_mirror
    if (log2_L >= 4) v = add_dpp<0x140>(v);    // row_mirror
    if (log2_L >= 5)                           // lanes i, i^16 of each half
        v += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
    if (log2_L >= 6)
        v = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0)) +
            __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    return v;
}

// One iteration's loads, kept raw: decoding a scale or a zero-point nibble
// here would make the wavefront wait for the load it just issued.
template <bool BF16, bool HAS_ZP, int CB, int J, int U>
struct Group {
    using Chunk = typename ChunkT<CB>::type;
    Chunk w[U][J];
    uint32_t sc[U][J];   // float32 bits, or bfloat16 bits in the low half
    uint32_t zb[U][J];   // packed zero-point byte (HAS_ZP)
};

template <bool BF16, bool HAS_ZP, int CB, int J, int U>
__device__ __forceinline__ void load_group(const GemvArgs& g, int64_t base, int p, int LT, int G,
                                           int gsub, Group<BF16, HAS_ZP, CB, J, U>& r) {
    using Chunk = typename ChunkT<CB>::type;
    constexpr int CK = 2 * CB;
#pragma unroll
    for (int u = 0; u < U; u++) {
        const int64_t gi = base + u;
        const int64_t col = gi * G + gsub;
        const bool ok = gi < g.n_groups && col < g.N;
        const uint8_t* bc = g.b + col * g.col_bytes;
#pragma unroll
        for (int j = 0; j < J; j++) {
            const int c = p + j * LT;
            if (ok && c < g.S) {
                r.w[u][j] = __builtin_nontemporal_load(
                    reinterpret_cast<const Chunk*>(bc + (int64_t)c * CB));
                const int blk = (c * CK) >> g.log2_bs;
                const int64_t si = col * g.nb + blk;
                r.sc[u][j] = BF16 ? (uint32_t)static_cast<const uint16_t*>(g.scales)[si]
                                  : static_cast<const uint32_t*>(g.scales)[si];
                if constexpr (HAS_ZP) r.zb[u][j] = g.zp[col * g.zp_row + (blk >> 1)];
            } else {
                r.w[u][j] = Chunk{};
                r.sc[u][j] = 0;
                if constexpr (HAS_ZP) r.zb[u][j] = 0x88;
            }
        }
    }
}

// W wavefronts per column team, U column groups per team per iteration,
// PF: load the next iteration's weights before computing the current one.
template <bool BF16, bool HAS_ZP, int CB, int J, int U, int W, bool PF>
__global__ __launch_bounds__(64 * kWavesPerBlock) void gemv_kernel(GemvArgs g) {
    constexpr int CK = 2 * CB;        // values of K per chunk
    constexpr int NW = CB / 4;        // 32-bit words per chunk
    constexpr int TEAMS = kWavesPerBlock / W;
    static_assert(W == 1 || U == 1, "split-K teams take one column at a time");
    __shared__ float red[kWavesPerBlock];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int team = wave / W;
    const int wt = wave - team * W;   // wavefront index within the team
    const int L = 1 << g.log2_L;      // lanes per column in one wavefront
    const int LT = L * W;             // lanes per column in the team
    const int p = wt * L + (lane & (L - 1));
    const int G = 64 >> g.log2_L;
    const int gsub = lane >> g.log2_L;

    // iteration space: WG-uniform, so barriers (W > 1) are reached by all
    const int64_t stride = (int64_t)gridDim.x * TEAMS * U;
    int64_t base = ((int64_t)blockIdx.x * TEAMS + team) * U;
    const int64_t team0 = (int64_t)blockIdx.x * TEAMS * U;

    Group<BF16, HAS_ZP, CB, J, U> cur;
    load_group(g, base, p, LT, G, gsub, cur);     // weights first: they do not wait on A

    // ---- activations: staged once per workgroup in LDS (coalesced loads,
    // converted to float32, chunk rows padded to CK+4 floats so that the
    // per-lane 16-byte reads below hit distinct banks), then each lane copies
    // its chunks into registers ----
    extern __shared__ __attribute__((aligned(16))) float a_lds[];
    constexpr int ROW = CK + 4;
    {
        const int64_t nvec = (int64_t)g.S * (CK / 4);       // float4 slots
        const bool vec = (g.K & 3) == 0;
        for (int64_t i = threadIdx.x; i < nvec; i += 64 * kWavesPerBlock) {
            const int64_t k = 4 * i;
            float4 v;
            if (vec && k + 4 <= g.K) {
                if constexpr (BF16) {
                    const uint2 x = *reinterpret_cast<const uint2*>(
                        static_cast<const uint16_t*>(g.a) + k);
                    v = make_float4(__uint_as_float(x.x << 16), __uint_as_float(x.x & 0xFFFF0000u),
                                    __uint_as_float(x.y << 16), __uint_as_float(x.y & 0xFFFF0000u));
                } else {
                    v = *reinterpret_cast<const float4*>(static_cast<const float*>(g.a) + k);
                }
            } else {
                float e[4];
#pragma unroll
                for (int h = 0; h < 4; h++) {
                    e[h] = 0.f;
                    if (k + h < g.K)
                        e[h] = BF16 ? bf16_to_f32(static_cast<const uint16_t*>(g.a)[k + h])
                                    : static_cast<const float*>(g.a)[k + h];
                }
                v = make_float4(e[0], e[1], e[2], e[3]);
            }
            const int64_t c = k / CK;
            *reinterpret_cast<float4*>(&a_lds[c * ROW + (k - c * CK)]) = v;
        }
    }
    __syncthreads();
    // this lane's chunks of A in registers (odd k pre-scaled by 1/16) and
    // the chunk sums of the unscaled values
    float av[J][CK];
    float asum[J];
#pragma unroll
    for (int j = 0; j < J; j++) {
        const int c = p + j * LT;
        if (c < g.S) {
#pragma unroll
            for (int v = 0; v < CK / 4; v++) {
                const float4 x = *reinterpret_cast<const float4*>(&a_lds[c * ROW + 4 * v]);
                av[j][4 * v] = x.x; av[j][4 * v + 1] = x.y;
                av[j][4 * v + 2] = x.z; av[j][4 * v + 3] = x.w;
            }
        } else {
#pragma unroll
            for (int i = 0; i < CK; i++) av[j][i] = 0.f;
        }
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < CK; i++) s += av[j][i];
        asum[j] = s;
#pragma unroll
        for (int i = 1; i < CK; i += 2) av[j][i] *= 0.0625f;
    }

    for (int64_t it0 = team0; it0 < g.n_groups; it0 += stride, base += stride) {
        // groups past the end load as zeros, so every register is defined
        Group<BF16, HAS_ZP, CB, J, U> nxt;
        if constexpr (PF) load_group(g, base + stride, p, LT, G, gsub, nxt);
        float acc[U];
#pragma unroll
        for (int u = 0; u < U; u++) {
            float s = 0.f;
#pragma unroll
            for (int j = 0; j < J; j++) {
                uint32_t words[NW];
#pragma unroll
                for (int d = 0; d < NW; d++) words[d] = cur.w[u][j][d];
                const float dot = dot_words<NW>(words, av[j]);
                float zf = 8.f;
                if constexpr (HAS_ZP) {
                    const int blk = ((p + j * LT) * CK) >> g.log2_bs;
                    const uint32_t zb = cur.zb[u][j];
                    zf = (float)((blk & 1) ? (zb >> 4) : (zb & 0xF));
                }
                const float sc = BF16 ? __uint_as_float(cur.sc[u][j] << 16)
                                      : __uint_as_float(cur.sc[u][j]);
                const float t = fmaf(-zf, asum[j], dot);
                s = fmaf(sc, t, s);
            }
            acc[u] = reduce_lanes(s, g.log2_L);
        }
        if constexpr (W > 1) {
            if (lane == 0) red[wave] = acc[0];
            __syncthreads();
            if (wt == 0) {
                float v = red[team * W];
#pragma unroll
                for (int w2 = 1; w2 < W; w2++) v += red[team * W + w2];
                acc[0] = v;
            }
            __syncthreads();
        }
        if (wt == 0 && (lane & (L - 1)) == 0) {
#pragma unroll
            for (int u = 0; u < U; u++) {
                const int64_t gi = base + u;
                const int64_t col = gi * G + gsub;
                if (gi < g.n_groups && col < g.N) {
                    float v = acc[u];
                    if (g.bias) v += g.bias[col];
                    if constexpr (BF16)
                        static_cast<uint16_t*>(g.y)[col] = f32_to_bf16_rtne(v);
                    else
                        static_cast<float*>(g.y)[col] = v;
                }
            }
        }
        if constexpr (PF)
            cur = nxt;
        else
            load_group(g, base + stride, p, LT, G, gsub, cur);
    }
}

int ilog2(int64_t v) {
    int r = 0;
    while ((int64_t(1) << r) < v) r++;
    return r;
}

struct Geometry {
    int log2_L, J, W;
};

// Lanes per wavefront, chunks per lane and wavefronts per column: a function
// of S = ceil(K / CK) only.  Highest lane efficiency S / (L*W*J) first, then
// fewer wavefronts, then fewer chunks per lane.  J == 0: no register kernel.
Geometry geometry(int64_t S, bool allow_split) {
    Geometry best{0, 0, 0};
    double best_eff = -1.0;
    for (int W = 1; W <= (allow_split ? kWMax : 1); W *= 2) {
        for (int lL = 0; lL <= 6; lL++) {
            if (W > 1 && lL != 6) continue;    // split-K teams use whole wavefronts
            const int64_t LT = (int64_t(1) << lL) * W;
            if (LT > 2 * S && lL > 0) continue; // more than twice the lanes needed
            const int64_t J = (S + LT - 1) / LT;
            if (J > kJMax) continue;
            const double eff = (double)S / (double)(LT * J);
            const bool better = eff > best_eff + 1e-9 ||
                                (eff > best_eff - 1e-9 && (W < best.W || (W == best.W && J < best.J)));
            if (better) {
                best = Geometry{lL, (int)J, W};
                best_eff = eff;
            }
        }
    }
    return best;
}

// Columns unrolled per iteration when there are plenty of columns.
constexpr int unroll_for(int J) { return J == 1 ? 4 : J == 2 ? 2 : 1; }
// Resident wavefronts per SIMD that the register use of (J, U) allows
// (from the compiler's resource report for gfx950).
constexpr int occupancy_for(int J, int U) {
    return U == 1 ? (J == 1 ? 7 : J == 2 ? 4 : 2) : (J == 1 ? 3 : 2);
}

template <bool BF16, bool HAS_ZP, int CB, int J>
hipError_t launch_j(int U, int W, unsigned blocks, size_t lds, hipStream_t s, const GemvArgs& a) {
    constexpr int UJ = unroll_for(J);
    constexpr bool PF = J <= 3;
    if (W == 1 && U == 1)
        hipLaunchKernelGGL((gemv_kernel<BF16, HAS_ZP, CB, J, 1, 1, PF>), dim3(blocks), dim3(256), lds, s, a);
    else if (W == 1)
        hipLaunchKernelGGL((gemv_kernel<BF16, HAS_ZP, CB, J, UJ, 1, PF>), dim3(blocks), dim3(256), lds, s, a);
    else if constexpr (CB == 16) {
        if (W == 2)
            hipLaunchKernelGGL((gemv_kernel<BF16, HAS_ZP, CB, J, 1, 2, PF>), dim3(blocks), dim3(256), lds, s, a);
        else
            hipLaunchKernelGGL((gemv_kernel<BF16, HAS_ZP, CB, J, 1, 4, PF>), dim3(blocks), dim3(256), lds, s, a);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <bool BF16, bool HAS_ZP, int CB>
hipError_t launch_cb(int J, int U, int W, unsigned blocks, size_t lds, hipStream_t s, const GemvArgs& a) {
    switch (J) {
        case 1: return launch_j<BF16, HAS_ZP, CB, 1>(U, W, blocks, lds, s, a);
        case 2: return launch_j<BF16, HAS_ZP, CB, 2>(U, W, blocks, lds, s, a);
        case 3: return launch_j<BF16, HAS_ZP, CB, 3>(U, W, blocks, lds, s, a);
        case 4: return launch_j<BF16, HAS_ZP, CB, 4>(U, W, blocks, lds, s, a);
        default: return hipErrorInvalidValue;
    }
}

template <bool BF16, bool HAS_ZP>
hipError_t launch_dt(int CB, int J, int U, int W, unsigned blocks, size_t lds, hipStream_t s,
                     const GemvArgs& a) {
    return CB == 16 ? launch_cb<BF16, HAS_ZP, 16>(J, U, W, blocks, lds, s, a)
                    : launch_cb<BF16, HAS_ZP, 8>(J, U, W, blocks, lds, s, a);
}

int compute_units() {
    static thread_local int cached_dev = -1, cached_cus = 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (dev != cached_dev) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        cached_dev = dev;
        cached_cus = cus;
    }
    return cached_cus;
}

}  // namespace

int64_t gemv_max_k(int bs) {
    // limited by the register geometry (S <= 64 * W * kJMax chunks) and by
    // the staged activations (S rows of CK + 4 floats in kMaxLds bytes)
    const int CK = bs >= 32 ? 32 : 16;
    const int W = bs >= 32 ? kWMax : 1;
    int64_t s_max = (int64_t)64 * W * kJMax;
    const int64_t s_lds = (int64_t)(kMaxLds / ((CK + 4) * sizeof(float)));
    if (s_lds < s_max) s_max = s_lds;
    return s_max * CK;
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
    const Geometry geo = geometry(a.S, CB == 16);
    if (geo.J == 0)
        return fail(MNB_E_UNSUPPORTED, "gemv: K=%lld beyond the register kernel", (long long)p.K);
    a.log2_L = geo.log2_L;
    const int G = geo.W == 1 ? (64 >> geo.log2_L) : 1;
    a.n_groups = (p.N + G - 1) / G;
    // Fill the chip: resident wavefronts = CUs x 4 SIMDs x occupancy; each
    // team of W wavefronts takes U groups per iteration.  Unroll only when
    // there are enough groups to give every resident team U of them.
    const int64_t simds = (int64_t)compute_units() * 4;
    const int UJ = unroll_for(geo.J);
    int U = 1;
    int64_t slots = simds * occupancy_for(geo.J, 1) / geo.W;
    if (geo.W == 1 && UJ > 1 && a.n_groups >= simds * occupancy_for(geo.J, UJ) * UJ) {
        U = UJ;
        slots = simds * occupancy_for(geo.J, UJ);
    }
    int64_t teams = (a.n_groups + U - 1) / U;
    if (teams > slots) teams = slots;
    const int teams_per_block = kWavesPerBlock / geo.W;
    const unsigned blocks = (unsigned)((teams + teams_per_block - 1) / teams_per_block);
    // staged activations: S chunk rows of CK + 4 floats
    const size_t lds = (size_t)a.S * (CK + 4) * sizeof(float);
    if (lds > kMaxLds)
        return fail(MNB_E_UNSUPPORTED, "gemv: K=%lld needs %zu bytes of LDS", (long long)p.K, lds);
    hipError_t e;
    if (p.bf16)
        e = p.has_zp ? launch_dt<true, true>(CB, geo.J, U, geo.W, blocks, lds, s, a)
                     : launch_dt<true, false>(CB, geo.J, U, geo.W, blocks, lds, s, a);
    else
        e = p.has_zp ? launch_dt<false, true>(CB, geo.J, U, geo.W, blocks, lds, s, a)
                     : launch_dt<false, false>(CB, geo.J, U, geo.W, blocks, lds, s, a);
    if (e != hipSuccess) return fail(MNB_E_HIP, "gemv launch: %s", hipGetErrorString(e));
    return MNB_OK;
}

}  // namespace mnb
