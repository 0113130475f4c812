// Prefill GEMM (any M): Y[M][N] = A[M][K] x dequant(B)[K][N] (+ bias).
//
// Page "Qwen3 CPU Inference Critical Path", "INT4 MatMul is first", int4_gemm:
// prompt prefill packs activation panels and reuses weight blocks; the
// weights stay packed in HBM ("Prepared weight-only plan": no expanded
// matrix).  On CDNA4 this is a dense contraction, so it runs on the bf16
// matrix cores (v_mfma_f32_32x32x16_bf16):
//
//  * a 128x128 output tile per workgroup (4 wavefronts, 64x64 each);
//  * per K step of 32 the workgroup stages in LDS
//      - the activation panel as bf16; a float32 activation is split into
//        hi = bf16(a) and lo = bf16(a - hi) (two MFMAs per product; the split
//        keeps 16 significant bits, relative error <= 2^-16 per product),
//      - the weight panel unpacked on chip to the EXACT integers q - zp
//        (|q - zp| <= 15 is exact in bf16);
//  * MFMA partial sums of one quantization block are accumulated separately
//    in float32 and folded into the running result with that block's scale:
//    acc += s[n][b] * partial.  In the 32x32 MFMA result layout every lane's
//    16 values belong to one output column, so this is one scale per lane.
//
// Tails: rows past M and values past K are zero in the staged panels;
// columns past N are never stored; pad nibbles past K multiply zeros.
#include "mnb_internal.h"

namespace mnb {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;

constexpr int BM = 128, BN = 128, BK = 32;
constexpr int PAD = 8;              // bf16 elements of padding per LDS row
constexpr int LDR = BK + PAD;       // LDS row stride in bf16 elements

struct GemmArgs {
    const void* a;
    const uint8_t* b;
    const void* scales;
    const uint8_t* zp;
    const float* bias;
    void* y;
    int64_t M, K, N, col_bytes, k_pad;
    int nb, zp_row, bs;
    bool vec_a;                      // rows of A are 16-byte aligned
};

__device__ __forceinline__ uint32_t pack2(uint16_t lo, uint16_t hi) {
    return (uint32_t)lo | ((uint32_t)hi << 16);
}

// bf16 bits of the small integer d (|d| <= 15): exact.
__device__ __forceinline__ uint16_t int_to_bf16(int d) {
    return (uint16_t)(__float_as_uint((float)d) >> 16);
}

template <bool BF16>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs g) {
    __shared__ __attribute__((aligned(16))) uint16_t As_hi[BM * LDR];
    __shared__ __attribute__((aligned(16))) uint16_t As_lo[BF16 ? 8 : BM * LDR];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[BN * LDR];

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t m0 = (int64_t)blockIdx.y * BM;
    const int64_t n0 = (int64_t)blockIdx.x * BN;

    f32x16 acc[2][2], blk[2][2];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) { acc[i][j][r] = 0.f; blk[i][j][r] = 0.f; }

    // staging roles: thread t stages 16 K-values of A row (t>>1) and of
    // weight column (t>>1), half (t&1) of the 32-wide K step
    const int sr = t >> 1;
    const int sh = (t & 1) * 16;
    const int64_t arow = m0 + sr;
    const int64_t bcol = n0 + sr;

    for (int64_t k0 = 0; k0 < g.k_pad; k0 += BK) {
        // ---- A panel -> LDS (bf16 hi [, lo]) ----
        {
            float av[16];
            const int64_t kb = k0 + sh;
            if (arow < g.M && g.vec_a && kb + 16 <= g.K) {
                if constexpr (BF16) {
                    const uint4* src = reinterpret_cast<const uint4*>(
                        static_cast<const uint16_t*>(g.a) + arow * g.K + kb);
                    uint4 x0 = src[0], x1 = src[1];
                    uint4* dh = reinterpret_cast<uint4*>(&As_hi[sr * LDR + sh]);
                    dh[0] = x0; dh[1] = x1;
                } else {
                    const float4* src = reinterpret_cast<const float4*>(
                        static_cast<const float*>(g.a) + arow * g.K + kb);
#pragma unroll
                    for (int v = 0; v < 4; v++) {
                        float4 x = src[v];
                        av[4 * v] = x.x; av[4 * v + 1] = x.y;
                        av[4 * v + 2] = x.z; av[4 * v + 3] = x.w;
                    }
                }
            } else {
#pragma unroll
                for (int i = 0; i < 16; i++) {
                    const int64_t k = kb + i;
                    float v = 0.f;
                    if (arow < g.M && k < g.K)
                        v = BF16 ? bf16_to_f32(static_cast<const uint16_t*>(g.a)[arow * g.K + k])
                                 : static_cast<const float*>(g.a)[arow * g.K + k];
                    av[i] = v;
                }
                if constexpr (BF16) {
                    uint32_t hv[8];
#pragma unroll
                    for (int i = 0; i < 8; i++)
                        hv[i] = pack2((uint16_t)(__float_as_uint(av[2 * i]) >> 16),
                                      (uint16_t)(__float_as_uint(av[2 * i + 1]) >> 16));
                    uint4* dh = reinterpret_cast<uint4*>(&As_hi[sr * LDR + sh]);
                    dh[0] = make_uint4(hv[0], hv[1], hv[2], hv[3]);
                    dh[1] = make_uint4(hv[4], hv[5], hv[6], hv[7]);
                }
            }
            if constexpr (!BF16) {
                uint32_t hv[8], lv[8];
#pragma unroll
                for (int i = 0; i < 8; i++) {
                    uint16_t h0 = f32_to_bf16_rtne(av[2 * i]);
                    uint16_t h1 = f32_to_bf16_rtne(av[2 * i + 1]);
                    uint16_t l0 = f32_to_bf16_rtne(av[2 * i] - bf16_to_f32(h0));
                    uint16_t l1 = f32_to_bf16_rtne(av[2 * i + 1] - bf16_to_f32(h1));
                    hv[i] = pack2(h0, h1);
                    lv[i] = pack2(l0, l1);
                }
                uint4* dh = reinterpret_cast<uint4*>(&As_hi[sr * LDR + sh]);
                uint4* dl = reinterpret_cast<uint4*>(&As_lo[sr * LDR + sh]);
                dh[0] = make_uint4(hv[0], hv[1], hv[2], hv[3]);
                dh[1] = make_uint4(hv[4], hv[5], hv[6], hv[7]);
                dl[0] = make_uint4(lv[0], lv[1], lv[2], lv[3]);
                dl[1] = make_uint4(lv[4], lv[5], lv[6], lv[7]);
            }
        }
        // ---- weight panel -> LDS as exact bf16 integers q - zp ----
        {
            const int64_t kb = k0 + sh;
            uint32_t wv[8];
            if (bcol < g.N && kb < g.k_pad) {
                const uint2 x = *reinterpret_cast<const uint2*>(
                    g.b + bcol * g.col_bytes + kb / 2);
                const int blkid = (int)(kb / g.bs);
                int z = 8;
                if (g.zp) {
                    const uint8_t zb = g.zp[bcol * g.zp_row + (blkid >> 1)];
                    z = (blkid & 1) ? (zb >> 4) : (zb & 0xF);
                }
                const uint32_t xw[2] = {x.x, x.y};
#pragma unroll
                for (int d = 0; d < 2; d++)
#pragma unroll
                    for (int byte = 0; byte < 4; byte++) {
                        const uint32_t bv = (xw[d] >> (8 * byte)) & 0xFF;
                        wv[4 * d + byte] = pack2(int_to_bf16((int)(bv & 0xF) - z),
                                                 int_to_bf16((int)(bv >> 4) - z));
                    }
            } else {
#pragma unroll
                for (int i = 0; i < 8; i++) wv[i] = 0;
            }
            uint4* db = reinterpret_cast<uint4*>(&Bs[sr * LDR + sh]);
            db[0] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
            db[1] = make_uint4(wv[4], wv[5], wv[6], wv[7]);
        }
        __syncthreads();

        // ---- MFMA over the two 16-wide substeps ----
#pragma unroll
        for (int ks = 0; ks < 2; ks++) {
            const int64_t kk = k0 + ks * 16;
            if (kk >= g.k_pad) break;
            const int koff = ks * 16 + 8 * (lane >> 5);
            bf16x8 ah[2], al[2], bf[2];
#pragma unroll
            for (int i = 0; i < 2; i++) {
                const int r = wm * 64 + i * 32 + (lane & 31);
                ah[i] = *reinterpret_cast<const bf16x8*>(&As_hi[r * LDR + koff]);
                if constexpr (!BF16)
                    al[i] = *reinterpret_cast<const bf16x8*>(&As_lo[r * LDR + koff]);
            }
#pragma unroll
            for (int j = 0; j < 2; j++) {
                const int c = wn * 64 + j * 32 + (lane & 31);
                bf[j] = *reinterpret_cast<const bf16x8*>(&Bs[c * LDR + koff]);
            }
#pragma unroll
            for (int i = 0; i < 2; i++)
#pragma unroll
                for (int j = 0; j < 2; j++) {
                    blk[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[i], bf[j], blk[i][j], 0, 0, 0);
                    if constexpr (!BF16)
                        blk[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[i], bf[j], blk[i][j], 0, 0, 0);
                }
            // end of a quantization block: fold the partial sums with the scale
            if (((kk + 16) % g.bs) == 0) {
                const int blkid = (int)(kk / g.bs);
#pragma unroll
                for (int j = 0; j < 2; j++) {
                    const int64_t n = n0 + wn * 64 + j * 32 + (lane & 31);
                    float s = 0.f;
                    if (n < g.N)
                        s = BF16 ? bf16_to_f32(static_cast<const uint16_t*>(g.scales)[n * g.nb + blkid])
                                 : static_cast<const float*>(g.scales)[n * g.nb + blkid];
#pragma unroll
                    for (int i = 0; i < 2; i++)
#pragma unroll
                        for (int r = 0; r < 16; r++) {
                            acc[i][j][r] = fmaf(s, blk[i][j][r], acc[i][j][r]);
                            blk[i][j][r] = 0.f;
                        }
                }
            }
        }
        __syncthreads();
    }

    // ---- epilogue: + bias, round, store ----
#pragma unroll
    for (int j = 0; j < 2; j++) {
        const int64_t n = n0 + wn * 64 + j * 32 + (lane & 31);
        if (n >= g.N) continue;
        const float bv = g.bias ? g.bias[n] : 0.f;
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int64_t m = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (m >= g.M) continue;
                const float v = acc[i][j][r] + bv;
                if constexpr (BF16)
                    static_cast<uint16_t*>(g.y)[m * g.N + n] = f32_to_bf16_rtne(v);
                else
                    static_cast<float*>(g.y)[m * g.N + n] = v;
            }
    }
}


// ---------------------------------------------------------------------------
// bfloat16 activations: scaled bf16 weight tiles, one MFMA per product.
//
// For bf16 activations the scales are bf16 too, so (q - zp) * s is exact in
// float32 (at most 5 + 8 significant bits) and its bf16 rounding is a single
// rounding of the exact weight -- the same value mnb_dequant's bf16 output
// gives.  The weight panel is therefore dequantized once per workgroup into
// LDS as bf16 and multiplied directly: no per-block partial sums, one MFMA per
// product.
//
// Tile BM x BN x 64 per workgroup of 8 wavefronts (2 along M x 4 along N;
// each wavefront (BM/2) x (BN/4) = TM x TN MFMA 32x32x16 tiles).  LDS is
// double-buffered (A and B panels as bf16, rows padded by 16 bytes so that the
// lanes' 16-byte operand reads fall in distinct banks); the next K step is
// fetched into registers while the current one is multiplied, so one barrier
// per K step suffices.  Global reads go through buffer resources: 32-bit
// offsets advanced by a constant per K step, and reads past a tensor's end
// return zeros (rows past M, columns past N; values past K are zeroed
// explicitly and pad nibbles only ever meet zero activations).  Workgroups
// are remapped so that consecutive output tiles (the row tiles sharing one
// weight panel first) run on the same XCD and share its L2.
// ---------------------------------------------------------------------------
constexpr int B2_K = 64;
constexpr int B2_LDR = B2_K + 8;                  // bf16 per LDS row

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// bijective remap of block ids: the blocks that land on XCD x (bid % 8 == x)
// take a contiguous range of virtual indices
__device__ __forceinline__ int xcd_index(int bid, int nblk) {
    const int q = nblk / 8, r = nblk % 8;
    const int x = bid % 8, j = bid / 8;
    return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + j;
}

__device__ __forceinline__ int2 xcd_tile(int bid, int nblk, int mt) {
    // bijective remap: the blocks that land on XCD x (bid % 8 == x) take a
    // contiguous range of tiles; tile t -> (m = t % mt, n = t / mt)
    const int q = nblk / 8, r = nblk % 8;
    const int x = bid % 8, j = bid / 8;
    const int t = (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + j;
    return make_int2(t % mt, t / mt);
}

struct Bf16Args {
    const void* a;
    const uint8_t* b;
    const void* scales;
    const uint8_t* zp;
    const float* bias;
    void* y;
    int M, K, N, col_bytes, k_pad, nb, zp_row, log2_bs;
    uint32_t a_bytes, b_bytes, s_bytes, z_bytes;
    // split-K: workgroup w of tiles * splits takes K steps [split * sps,
    // split * sps + sps) and, when part is set, stores its float32 partial
    // tile to part[split][M][N] instead of Y (the reduction adds the bias)
    int splits, sps;
    float* part;
    // tail split (wide kernel): workgroups past full_tiles take the last
    // tail_tiles tiles, each split into tail_splits parts of tail_sps K steps,
    // and store float32 partial tiles to tail_part[split][tail tile][256][256]
    int full_tiles, tail_tiles, tail_splits, tail_sps;
    float* tail_part;
    // gated gate||up (wide kernel, SILU): I = N / 2; the 256 weight columns of
    // a tile are 128 gate columns and the matching 128 up columns, and Y is
    // h[M][I] = silu(gate) * up
    int silu_half;
};

template <int BM, int BN, int WAVES>
__global__ __launch_bounds__(64 * WAVES, 1) void gemm_bf16_kernel(Bf16Args g) {
    constexpr int T = 64 * WAVES;
    constexpr int WN = WAVES / 2;                       // wavefronts along N (2 along M)
    constexpr int TM = BM / 64, TN = BN / WN / 32;      // MFMA tiles per wavefront
    constexpr int AR = BM * 8 / T;                      // 16-byte A chunks per thread
    constexpr int BR = (BN * 2 + T - 1) / T;            // 16-byte packed-B chunks per thread
    static_assert(AR >= 1 && TN >= 1, "tile too small for the wavefront count");
    __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * B2_LDR];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * B2_LDR];

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int mt = (g.M + BM - 1) / BM;
    const int nt = (g.N + BN - 1) / BN;
    const int2 tile = xcd_tile(blockIdx.x, mt * nt, mt);
    const int m0 = tile.x * BM;
    const int n0 = tile.y * BN;

    const __amdgpu_buffer_rsrc_t ra_rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(g.a), (short)0, (int)g.a_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rb_rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(g.b), (short)0, (int)g.b_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(g.scales), (short)0, (int)g.s_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rz_rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(g.zp ? g.zp : g.b), (short)0, (int)(g.zp ? g.z_bytes : 0), 0x00020000);

    // staging roles: A chunk q = t + T*i is row q/8, 16-byte chunk q%8 of the
    // 64-wide K step; packed-B chunk q = t + T*i is column q/2, 16 bytes (32
    // values) half q%2
    const int a_r = t >> 3, a_c = t & 7;
    const uint32_t a_base = (uint32_t)(m0 + a_r) * (uint32_t)g.K * 2u + 16u * a_c;
    const uint32_t a_step = (uint32_t)(T / 8) * (uint32_t)g.K * 2u;   // rows between a thread's chunks

    struct StageA {
        u32x4 a[AR];
    };
    struct StageB {
        u32x4 b[BR];
        uint32_t s[BR][2], z[BR][2];   // scale bits and zero point of values 0-15, 16-31
    };

    auto fetch_a = [&](int k0, StageA& st) {
        const bool k_in = k0 + 8 * a_c < g.K;            // K % 8 == 0: whole chunk in or out
#pragma unroll
        for (int i = 0; i < AR; i++) {
            st.a[i] = __builtin_amdgcn_raw_buffer_load_b128(ra_rs, a_base + a_step * i + 2u * k0, 0, 0);
            if (!k_in) st.a[i] = u32x4{0, 0, 0, 0};
        }
    };
    auto fetch_b = [&](int k0, StageB& st) {
#pragma unroll
        for (int i = 0; i < BR; i++) {
            const int q = t + T * i;
            if (q < 2 * BN) {
                const int col = n0 + (q >> 1), half = q & 1;
                const int kb = k0 + 32 * half;
                st.b[i] = __builtin_amdgcn_raw_buffer_load_b128(
                    rb_rs, (uint32_t)col * (uint32_t)g.col_bytes + (uint32_t)kb / 2u, 0, 0);
#pragma unroll
                for (int h = 0; h < 2; h++) {
                    const uint32_t blk = (uint32_t)(kb + 16 * h) >> g.log2_bs;
                    st.s[i][h] = __builtin_amdgcn_raw_buffer_load_b16(
                        rs_rs, 2u * ((uint32_t)col * (uint32_t)g.nb + blk), 0, 0);
                    st.z[i][h] = g.zp ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(
                                            rz_rs, (uint32_t)col * (uint32_t)g.zp_row + (blk >> 1), 0, 0)
                                            | ((blk & 1u) << 8)
                                      : 0x8u;
                }
            }
        }
    };

    auto stash_a = [&](const StageA& st, int buf) {
#pragma unroll
        for (int i = 0; i < AR; i++)
            *reinterpret_cast<u32x4*>(&As[buf][(a_r + (T / 8) * i) * B2_LDR + 8 * a_c]) = st.a[i];
    };
    auto stash_b = [&](const StageB& st, int buf) {
#pragma unroll
        for (int i = 0; i < BR; i++) {
            const int q = t + T * i;
            if (q < 2 * BN) {
                const int c = q >> 1, half = q & 1;
#pragma unroll
                for (int d = 0; d < 4; d++) {
                    // (q - zp) * s exact in float32, then one RTNE rounding to bf16
                    const uint32_t zraw = st.z[i][d >> 1];
                    const uint32_t zq = g.zp ? ((zraw & 0x100u) ? ((zraw >> 4) & 0xFu) : (zraw & 0xFu)) : 8u;
                    const float s = __uint_as_float(st.s[i][d >> 1] << 16);
                    const float zs = (float)zq * s;
                    const uint32_t lo = opaque_and(st.b[i][d], 0x0F0F0F0Fu);
                    const uint32_t hi = opaque_and(st.b[i][d] >> 4, 0x0F0F0F0Fu);
                    float v[8];
                    v[0] = fmaf(ubyte_to_f32<0>(lo), s, -zs); v[1] = fmaf(ubyte_to_f32<0>(hi), s, -zs);
                    v[2] = fmaf(ubyte_to_f32<1>(lo), s, -zs); v[3] = fmaf(ubyte_to_f32<1>(hi), s, -zs);
                    v[4] = fmaf(ubyte_to_f32<2>(lo), s, -zs); v[5] = fmaf(ubyte_to_f32<2>(hi), s, -zs);
                    v[6] = fmaf(ubyte_to_f32<3>(lo), s, -zs); v[7] = fmaf(ubyte_to_f32<3>(hi), s, -zs);
                    uint32_t o[4];
#pragma unroll
                    for (int h = 0; h < 4; h++) {
                        bf16x2 pr;
                        pr[0] = (__bf16)v[2 * h];
                        pr[1] = (__bf16)v[2 * h + 1];
                        o[h] = __builtin_bit_cast(uint32_t, pr);
                    }
                    *reinterpret_cast<u32x4*>(&Bs[buf][c * B2_LDR + 32 * half + 8 * d]) =
                        u32x4{o[0], o[1], o[2], o[3]};
                }
            }
        }
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0.f;

    auto multiply = [&](int buf) {
#pragma unroll 1
        for (int ks = 0; ks < B2_K / 16; ks++) {
            const int koff = ks * 16 + 8 * (lane >> 5);
            bf16x8 af[TM], bfr[TN];
#pragma unroll
            for (int i = 0; i < TM; i++)
                af[i] = *reinterpret_cast<const bf16x8*>(
                    &As[buf][(wm * (BM / 2) + i * 32 + (lane & 31)) * B2_LDR + koff]);
#pragma unroll
            for (int j = 0; j < TN; j++)
                bfr[j] = *reinterpret_cast<const bf16x8*>(
                    &Bs[buf][(wn * (BN / WN) + j * 32 + (lane & 31)) * B2_LDR + koff]);
#pragma unroll
            for (int i = 0; i < TM; i++)
#pragma unroll
                for (int j = 0; j < TN; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
    };

    // Pipeline over K steps (one barrier per step).  While step s is
    // multiplied from LDS buffer s % 2, step s + 1 is moved from registers to
    // the other buffer, the weights of step s + 2 and the activations of step
    // s + 1 are requested.  Each half of the unrolled loop is one basic block
    // (reads past the end return zeros or are never used, and the last,
    // redundant stash goes to a buffer that is not read again) so the
    // scheduler can interleave the unpacking and LDS traffic with the MFMAs.
    const int steps = (g.k_pad + B2_K - 1) / B2_K;
    StageA sa;
    StageB sb0, sb1;
    fetch_a(0, sa);
    fetch_b(0, sb0);
    stash_a(sa, 0);
    stash_b(sb0, 0);
    fetch_a(B2_K, sa);
    fetch_b(B2_K, sb1);
    __syncthreads();
    for (int st = 0; st < steps; st += 2) {
        fetch_b((st + 2) * B2_K, sb0);
        multiply(0);
        stash_a(sa, 1);
        stash_b(sb1, 1);
        fetch_a((st + 2) * B2_K, sa);
        __syncthreads();
        if (st + 1 >= steps) break;
        fetch_b((st + 3) * B2_K, sb1);
        multiply(1);
        stash_a(sa, 0);
        stash_b(sb0, 0);
        fetch_a((st + 3) * B2_K, sa);
        __syncthreads();
    }

    // epilogue: + bias, RTNE to bf16, store
#pragma unroll
    for (int j = 0; j < TN; j++) {
        const int n = n0 + wn * (BN / WN) + j * 32 + (lane & 31);
        if (n >= g.N) continue;
        const float bv = g.bias ? g.bias[n] : 0.f;
#pragma unroll
        for (int i = 0; i < TM; i++)
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int m = m0 + wm * (BM / 2) + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (m < g.M)
                    static_cast<uint16_t*>(g.y)[(int64_t)m * g.N + n] = f32_to_bf16_rtne(acc[i][j][r] + bv);
            }
    }
}


// ---------------------------------------------------------------------------
// bf16 activations, large grids: 256 x 256 x 64 tiles on 8 wavefronts of
// 128 x 64 (8 MFMA 32x32x16 tiles each), in two groups that take turns on
// the matrix cores (a ping-pong schedule).
//
//  * Both operand panels of a K step live in LDS as bf16, double-buffered
//    (4 x 32 KiB): the activations as loaded, the weights unpacked to
//    bf16((q - zp) * s).  Rows are 128 bytes (64 K values); the eight
//    16-byte chunks of row r sit at chunk ^ ((r >> 1) & 7), so the operand
//    reads of 16 consecutive rows (one 256-byte bank sweep) are conflict-free.
//  * Group g (wavefronts 4g .. 4g + 3, one per SIMD) computes rows 128 g ..
//    128 g + 127 of the tile and moves half of every K step: activation rows
//    and weight columns 128 g .. 128 g + 127.  Every step j is "multiply j
//    from LDS; barrier; write this group's half of step j + 1 + g into the
//    other buffer and request step j + 2 + g; barrier", with group 1 one
//    barrier behind group 0.  So on every SIMD one wavefront multiplies
//    while the other unpacks weights, writes LDS and issues global loads;
//    both halves of a step are in LDS before group 0 reads it, and no
//    buffer is written while it is read.
//  * The barriers wait only for LDS: global loads stay in flight across
//    them (the compiler tracks every buffer load and waits precisely where
//    the registers are used, one step later).
//  * The bf16 tile leaves through LDS (free after the last barrier): each
//    wavefront writes its 128 x 64 tile as 128-byte rows and stores 16-byte
//    pieces of whole rows.
//  * SILU (the gate||up projection with the gated product fused into the
//    epilogue; page "Qwen3 CPU Inference Critical Path", "Phase Q5:
//    scheduling and fusion"): a tile's 256 weight columns are 128 gate
//    columns and the matching 128 up columns, placed so that each
//    wavefront's two 32-column MFMA tiles are gate columns c .. c + 31 and
//    up columns c .. c + 31: every lane then holds the gate and the up sums
//    of the same column and rows, and writes h = silu(gate + bias) * (up +
//    bias), evaluated in float32 and rounded once to bf16.  Y is h[M][N/2]:
//    half the bytes of the unfused gate||up output.
// Requires K % 64 == 0 and K % block_size == 0 (no partial K step or block).
// ---------------------------------------------------------------------------
constexpr int B4_M = 256, B4_N = 256, B4_K = 64;

// byte offset of 16-byte chunk c of 128-byte row r
__device__ __forceinline__ int swz(int r, int c) { return r * 128 + ((c ^ ((r >> 1) & 7)) << 4); }

// Barrier for LDS traffic only: this wavefront's LDS reads and writes are
// complete, global loads may still be in flight.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");
}

template <bool HAS_ZP, bool BS16, bool SILU = false>
__global__ __launch_bounds__(512, 1) void gemm_bf16_wide_kernel(Bf16Args g) {
    constexpr int TM = 4, TN = 2;
    constexpr int PANEL = 256 * B4_K * 2;               // one K step of one operand: 32 KiB
    constexpr int AR = 4;                               // activation chunks per thread per step
    __shared__ __attribute__((aligned(16))) uint8_t lds[4 * PANEL];
    uint8_t* const As = lds;                            // [2][PANEL]
    uint8_t* const Bs = lds + 2 * PANEL;                // [2][PANEL]

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;
    const int wm = wave >> 2, wn = wave & 3;
    const int grp = __builtin_amdgcn_readfirstlane(wm);  // wave-uniform group
    const int tg = t & 255;                             // thread within the group
    const int mt = (g.M + B4_M - 1) / B4_M;
    const int nt = (g.N + B4_N - 1) / B4_N;
    const int tiles = mt * nt;
    // whole tiles (remapped so that each XCD takes a contiguous range), then
    // the tail tiles split along K, dispatched last
    int split, tt, sps, tail_idx = -1;
    if (g.tail_tiles && (int)blockIdx.x >= g.full_tiles) {
        const int w = blockIdx.x - g.full_tiles;
        tail_idx = w % g.tail_tiles;
        split = w / g.tail_tiles;
        tt = g.full_tiles + tail_idx;
        sps = g.tail_sps;
    } else {
        const int v = xcd_index(blockIdx.x, g.tail_tiles ? g.full_tiles : tiles * g.splits);
        split = v / tiles;
        tt = v - split * tiles;
        sps = g.sps;
    }
    const int m0 = (tt % mt) * B4_M;
    const int n0 = (tt / mt) * B4_N;
    const int kbase = split * sps * B4_K;                   // this split's first K value

    const __amdgpu_buffer_rsrc_t ra_rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(g.a), (short)0, (int)g.a_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rb_rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(g.b), (short)0, (int)g.b_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(g.scales), (short)0, (int)g.s_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rz_rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(HAS_ZP ? g.zp : g.b), (short)0, (int)(HAS_ZP ? g.z_bytes : 0), 0x00020000);

    // this group's half of a step: activation rows 128 grp + tg / 8 + 32 i,
    // chunk tg % 8 (rows past M read as zeros); weight column 128 grp + tg / 2,
    // K half tg % 2, with its scale(s) and zero point(s).  With 16-value
    // blocks the 32-value chunk spans an even block and the next one: their
    // two scales are one aligned 32-bit word (K % 64 == 0 makes the blocks
    // per column even) and their zero points the two nibbles of one byte.
    const int a_r = 128 * grp + (tg >> 3), a_c = tg & 7;
    const uint32_t a_off = (uint32_t)(m0 + a_r) * (uint32_t)g.K * 2u + 16u * a_c;
    const uint32_t a_rows32 = 32u * (uint32_t)g.K * 2u;
    const int b_col = 128 * grp + (tg >> 1), b_half = tg & 1;
    // (z stays a byte: widening it where it is loaded would make the
    // compiler wait for the load there, ahead of the next step's requests)
    struct Stage {
        u32x4 a[AR];
        u32x4 b;
        uint32_t s;
        uint8_t z;
        uint32_t zsh;   // bit offset of the zero-point nibble (larger blocks)
    };
    auto fetch = [&](int k0, Stage& st) {
#pragma unroll
        for (int i = 0; i < AR; i++)
            st.a[i] = __builtin_amdgcn_raw_buffer_load_b128(ra_rs, a_off + a_rows32 * i + 2u * (kbase + k0), 0, 0);
        int col = n0 + b_col;
        if constexpr (SILU)   // wavefront block b_col / 64: gate columns, then the matching up columns
            col = ((b_col >> 5) & 1 ? g.silu_half : 0) + (n0 >> 1) + 32 * (b_col >> 6) + (b_col & 31);
        const int kb = kbase + k0 + 32 * b_half;
        st.b = __builtin_amdgcn_raw_buffer_load_b128(
            rb_rs, (uint32_t)col * (uint32_t)g.col_bytes + (uint32_t)kb / 2u, 0, 0);
        const uint32_t blk = (uint32_t)kb >> g.log2_bs;
        const uint32_t s_off = 2u * ((uint32_t)col * (uint32_t)g.nb + blk);
        if constexpr (BS16)
            st.s = __builtin_amdgcn_raw_buffer_load_b32(rs_rs, s_off, 0, 0);
        else
            st.s = __builtin_amdgcn_raw_buffer_load_b16(rs_rs, s_off, 0, 0);
        if constexpr (HAS_ZP) {
            st.z = __builtin_amdgcn_raw_buffer_load_b8(rz_rs, (uint32_t)col * (uint32_t)g.zp_row + (blk >> 1), 0, 0);
            if constexpr (!BS16) st.zsh = 4u * (blk & 1u);
        }
    };
    // the activations as loaded; the weights unpacked 8 values (one word of
    // the chunk) at a time: (q - zp) * s is exact in float32, one RTNE
    // rounding to bf16
    auto stash = [&](const Stage& st, int buf) {
#pragma unroll
        for (int i = 0; i < AR; i++)
            *reinterpret_cast<u32x4*>(As + buf * PANEL + swz(a_r + 32 * i, a_c)) = st.a[i];
#pragma unroll
        for (int d = 0; d < 4; d++) {
            const int h = BS16 ? (d >> 1) : 0;
            uint32_t zq = 8u;
            if constexpr (HAS_ZP) zq = __builtin_amdgcn_ubfe((uint32_t)st.z, BS16 ? 4u * h : st.zsh, 4);
            const float sc = __uint_as_float(BS16 && h ? (st.s & 0xFFFF0000u) : (st.s << 16));
            const float zs = (float)zq * sc;
            const uint32_t lo = opaque_and(st.b[d], 0x0F0F0F0Fu);
            const uint32_t hi = opaque_and(st.b[d] >> 4, 0x0F0F0F0Fu);
            float v[8];
            v[0] = fmaf(ubyte_to_f32<0>(lo), sc, -zs); v[1] = fmaf(ubyte_to_f32<0>(hi), sc, -zs);
            v[2] = fmaf(ubyte_to_f32<1>(lo), sc, -zs); v[3] = fmaf(ubyte_to_f32<1>(hi), sc, -zs);
            v[4] = fmaf(ubyte_to_f32<2>(lo), sc, -zs); v[5] = fmaf(ubyte_to_f32<2>(hi), sc, -zs);
            v[6] = fmaf(ubyte_to_f32<3>(lo), sc, -zs); v[7] = fmaf(ubyte_to_f32<3>(hi), sc, -zs);
            uint32_t o[4];
#pragma unroll
            for (int e = 0; e < 4; e++) {
                bf16x2 pr;
                pr[0] = (__bf16)v[2 * e];
                pr[1] = (__bf16)v[2 * e + 1];
                o[e] = __builtin_bit_cast(uint32_t, pr);
            }
            *reinterpret_cast<u32x4*>(Bs + buf * PANEL + swz(b_col, 4 * b_half + d)) = u32x4{o[0], o[1], o[2], o[3]};
        }
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0.f;

    // Multiply the step in LDS buffer buf: 4 sub-steps of 8 MFMAs, the
    // operands of the next sub-step read ahead, at raised issue priority.
    auto compute = [&](int buf) {
        const uint8_t* a = As + buf * PANEL;
        const uint8_t* b = Bs + buf * PANEL;
        bf16x8 af[2][TM], bfr[2][TN];
        auto load_frags = [&](int ks, int p) {
            const int chunk = 2 * ks + (lane >> 5);
#pragma unroll
            for (int i = 0; i < TM; i++)
                af[p][i] = *reinterpret_cast<const bf16x8*>(a + swz(wm * 128 + i * 32 + (lane & 31), chunk));
#pragma unroll
            for (int j = 0; j < TN; j++)
                bfr[p][j] = *reinterpret_cast<const bf16x8*>(b + swz(wn * 64 + j * 32 + (lane & 31), chunk));
        };
        __builtin_amdgcn_s_setprio(1);
        load_frags(0, 0);
#pragma unroll
        for (int ks = 0; ks < B4_K / 16; ks++) {
            const int p = ks & 1;
            if (ks + 1 < B4_K / 16) load_frags(ks + 1, p ^ 1);
            // keep the next sub-step's reads ahead of this sub-step's MFMAs:
            // left alone, the scheduler sinks each read to just before its
            // first use and the MFMAs then wait for LDS
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < TM; i++)
#pragma unroll
                for (int j = 0; j < TN; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[p][i], bfr[p][j], acc[i][j], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_setprio(0);
    };

    const int steps = min(sps, g.K / B4_K - split * sps);
    // One code path for both groups (divergent paths would double the live
    // registers), group 1 one barrier behind.  Past the last step the loads
    // read zeros or unused bytes inside the operands, and the buffer written
    // is never read again, so neither needs a guard.
    Stage su, sl;
    {
        Stage s0;
        fetch(0, s0);
        if (grp) fetch(B4_K, sl);
        stash(s0, 0);
        if (grp) stash(sl, 1);
        fetch((1 + grp) * B4_K, su);
    }
    lds_barrier();
    if (grp) lds_barrier();
    auto step = [&](int j, const Stage& use, Stage& ld) {
        __builtin_amdgcn_sched_barrier(0);
        compute(j & 1);
        __builtin_amdgcn_sched_barrier(0);
        lds_barrier();
        __builtin_amdgcn_sched_barrier(0);
        fetch((j + 2 + grp) * B4_K, ld);
        stash(use, (j + 1 + grp) & 1);
        __builtin_amdgcn_sched_barrier(0);
        lds_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };
    int j = 0;
    for (; j + 1 < steps; j += 2) {
        step(j, su, sl);
        step(j + 1, sl, su);
    }
    if (j < steps) step(j, su, sl);
    if (!grp) lds_barrier();
    // every wavefront is past its last LDS access of the operands here

    // epilogue: the float32 partial (of the whole product for split-K, of the
    // tile for the tail split), or + bias and RTNE to bf16
    if (tail_idx >= 0) {
        float* const tp = g.tail_part + ((int64_t)split * g.tail_tiles + tail_idx) * (B4_M * B4_N);
#pragma unroll
        for (int jj = 0; jj < TN; jj++) {
            const int c = wn * 64 + jj * 32 + (lane & 31);
#pragma unroll
            for (int i = 0; i < TM; i++)
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    const int rr = wm * 128 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                    tp[rr * B4_N + c] = acc[i][jj][r];
                }
        }
        return;
    }
    if constexpr (SILU) {
        // lane c of this wavefront holds, for its 16 rows of each MFMA row
        // tile i, the gate sums of h column hc (acc[i][0]) and the up sums
        // of the same column (acc[i][1]).  Rows R and R + 1 are packed into a
        // dword and lanes c and c ^ 1 swap halves (two adjacent columns of
        // one row per lane); with I % 8 == 0 the dwords go through this
        // wavefront's 8 KiB of LDS (64-byte rows) and leave as 16-byte
        // pieces, otherwise they are stored directly.  Rows past M are
        // dropped by the output's range check.
        const int I = g.silu_half;
        const int c = lane & 31;
        const int hc = (n0 >> 1) + 32 * wn + c;
        const bool ok = hc < I;
        const float bg = g.bias && ok ? g.bias[hc] : 0.f;
        const float bu = g.bias && ok ? g.bias[I + hc] : 0.f;
        const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(
            g.y, (short)0, (int)((uint32_t)g.M * (uint32_t)I * 2u), 0x00020000);
        const bool staged = (I & 7) == 0;
        uint8_t* const wt = lds + wave * 8192;
        const int odd = lane & 1;
        const uint32_t sel = odd ? 0x03020706u : 0x05040100u;
        const uint32_t rowb = 2u * (uint32_t)I;
        const uint32_t vb = (uint32_t)(m0 + wm * 128 + 4 * (lane >> 5) + odd) * rowb + 2u * (uint32_t)(hc & ~1);
        const bool pair_ok = (hc | 1) < I;
#pragma unroll
        for (int i = 0; i < TM; i++)
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const float g0 = acc[i][0][r] + bg, g1 = acc[i][0][r + 1] + bg;
                const float u0 = acc[i][1][r] + bu, u1 = acc[i][1][r + 1] + bu;
                bf16x2 pr;
                pr[0] = (__bf16)(g0 / (1.0f + expf(-g0)) * u0);
                pr[1] = (__bf16)(g1 / (1.0f + expf(-g1)) * u1);
                const uint32_t own = __builtin_bit_cast(uint32_t, pr);
                const uint32_t oth = (uint32_t)__builtin_amdgcn_mov_dpp((int)own, 0xB1, 0xF, 0xF, false);
                const uint32_t out = __builtin_amdgcn_perm(oth, own, sel);
                const int row = i * 32 + 8 * (r >> 2) + (r & 3);   // + 4 (lane >> 5) + odd
                if (staged)
                    *reinterpret_cast<uint32_t*>(wt + (row + 4 * (lane >> 5) + odd) * 64 + 2 * (c & ~1)) = out;
                else if (pair_ok)
                    __builtin_amdgcn_raw_buffer_store_b32(out, ry, vb + (uint32_t)row * rowb, 0, 0);
            }
        if (staged) {
            __builtin_amdgcn_s_waitcnt(0xC07F);                 // lgkmcnt(0): this wavefront's LDS writes
            const int pc = lane & 3;                            // 16-byte piece of a 64-byte row
            const int hcol = (n0 >> 1) + 32 * wn + 8 * pc;
            const uint32_t vb2 = (uint32_t)(m0 + wm * 128 + (lane >> 2)) * rowb + 2u * (uint32_t)hcol;
#pragma unroll
            for (int q = 0; q < 8; q++) {
                const u32x4 v = *reinterpret_cast<const u32x4*>(wt + (16 * q + (lane >> 2)) * 64 + 16 * pc);
                if (hcol < I)
                    __builtin_amdgcn_raw_buffer_store_b128(v, ry, vb2 + (uint32_t)(16 * q) * rowb, 0, 0);
            }
        }
        return;
    }
    float* const part = g.part ? g.part + (int64_t)split * g.M * g.N : nullptr;
    if (!part && (g.N & 1) == 0) {
        // In the MFMA result a lane holds 16 rows of one column.  Rows R and
        // R + 1 of a column are packed into one dword and lanes c and c ^ 1
        // swap halves, so that each lane holds two adjacent columns of one
        // row.  With N % 8 == 0 these dwords go through this wavefront's own
        // 16 KiB of LDS (rows of 128 bytes) and leave as 16-byte pieces of
        // whole rows; otherwise they are stored directly.  Rows past M fall
        // outside the output buffer and are dropped by its range check (the
        // whole offset is in the VGPR operand, which the check covers).
        const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(
            g.y, (short)0, (int)((uint32_t)g.M * (uint32_t)g.N * 2u), 0x00020000);
        const bool staged = (g.N & 7) == 0;
        uint8_t* const wt = lds + wave * 16384;
        const int odd = lane & 1;
        const uint32_t sel = odd ? 0x03020706u : 0x05040100u;
        const uint32_t rowb = 2u * (uint32_t)g.N;
#pragma unroll
        for (int jj = 0; jj < TN; jj++) {
            const int c = jj * 32 + (lane & 31);                // column in the wavefront's 64
            const int n = n0 + wn * 64 + c;
            const float bv = g.bias && n < g.N ? g.bias[n] : 0.f;
            const uint32_t vb = (uint32_t)(m0 + wm * 128 + 4 * (lane >> 5) + odd) * rowb + 2u * (uint32_t)(n & ~1);
            const bool col_ok = (n | 1) < g.N;                  // both columns of the pair
#pragma unroll
            for (int i = 0; i < TM; i++)
#pragma unroll
                for (int r = 0; r < 16; r += 2) {
                    bf16x2 pr;
                    pr[0] = (__bf16)(acc[i][jj][r] + bv);
                    pr[1] = (__bf16)(acc[i][jj][r + 1] + bv);
                    const uint32_t own = __builtin_bit_cast(uint32_t, pr);
                    const uint32_t oth = (uint32_t)__builtin_amdgcn_mov_dpp((int)own, 0xB1, 0xF, 0xF, false);
                    const uint32_t out = __builtin_amdgcn_perm(oth, own, sel);
                    const int row = i * 32 + 8 * (r >> 2) + (r & 3);   // + 4 (lane >> 5) + odd
                    if (staged)
                        *reinterpret_cast<uint32_t*>(wt + (row + 4 * (lane >> 5) + odd) * 128 + 2 * (c & ~1)) = out;
                    else if (col_ok)
                        __builtin_amdgcn_raw_buffer_store_b32(out, ry, vb + (uint32_t)row * rowb, 0, 0);
                }
        }
        if (staged) {
            __builtin_amdgcn_s_waitcnt(0xC07F);                 // lgkmcnt(0): this wavefront's LDS writes
            const int pc = lane & 7;                            // 16-byte piece of a row
            const int ncol = n0 + wn * 64 + 8 * pc;
            const uint32_t vb = (uint32_t)(m0 + wm * 128 + (lane >> 3)) * rowb + 2u * (uint32_t)ncol;
#pragma unroll
            for (int q = 0; q < 16; q++) {
                const u32x4 v = *reinterpret_cast<const u32x4*>(wt + (8 * q + (lane >> 3)) * 128 + 16 * pc);
                if (ncol < g.N)
                    __builtin_amdgcn_raw_buffer_store_b128(v, ry, vb + (uint32_t)(8 * q) * rowb, 0, 0);
            }
        }
        return;
    }
#pragma unroll
    for (int jj = 0; jj < TN; jj++) {
        const int n = n0 + wn * 64 + jj * 32 + (lane & 31);
        if (n >= g.N) continue;
        const float bv = (!part && g.bias) ? g.bias[n] : 0.f;
#pragma unroll
        for (int i = 0; i < TM; i++)
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int m = m0 + wm * 128 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (m >= g.M) continue;
                if (part)
                    part[(int64_t)m * g.N + n] = acc[i][jj][r];
                else
                    static_cast<uint16_t*>(g.y)[(int64_t)m * g.N + n] = f32_to_bf16_rtne(acc[i][jj][r] + bv);
            }
    }
}

// ---------------------------------------------------------------------------
// float32 activations and scales: exact-integer weights on the matrix cores.
//
// The weight panel holds the exact integers q - zp (|q - zp| <= 15 is exact
// in bf16), the activation panel a float32 value split into a bf16 head and
// tail (a = hi + lo, lo = bf16(a - hi): about 16 significant bits), so one
// product is two MFMAs and the only weight rounding is the scale's.  The
// partial sums of one scale period (one quantization block, or the part of
// it in one K step) are accumulated separately and folded in with that
// block's scale, acc += s * partial: each lane's 16 MFMA results belong to
// one output column, so that is one scale per lane.  With A the identity
// the result is float32((q - zp) * s), the dequantized weight, exactly.
//
// Tiles of BT x BT x KS on 4 wavefronts of BT/2 x BT/2 (T x T MFMA 32x32x16
// tiles each, BT = 64 T): T = 2 for large products, T = 1 for short ones,
// whose 64 x 64 tiles give four times as many workgroups (more of them per
// CU, far fewer K splits).  K steps of KS = 32 values, or 64 for T = 1 when
// K and the blocks allow (half the barriers per K); P 16-value sub-steps
// make one scale period.  The three panels (A hi, A lo, B) and the step's
// scales sit in LDS, double-buffered.  Rows are 2 KS bytes with the 16-byte
// pieces of row r XOR-swizzled (piece ^ ((r >> 2) & 3) for 64-byte rows,
// piece ^ ((r >> 1) & 7) for 128-byte rows), so the operand reads of 16
// consecutive rows are conflict-free.  Activations (full 128-byte lines)
// and packed weights are read two K steps ahead into registers and staged
// one step ahead, interleaved with the MFMAs; one barrier per K step; a
// two-step loop body with alternating register stages.
// Requires K % KS == 0 and K % block_size == 0.
// ---------------------------------------------------------------------------
constexpr int F_K = 32;

template <int V> struct IntC { static constexpr int value = V; };

__device__ __forceinline__ int swz64(int r, int piece) { return r * 64 + ((piece ^ ((r >> 2) & 3)) << 4); }

// bf16 head and tail of four floats, packed two per 32-bit word
__device__ __forceinline__ void split4(const u32x4& x, uint2& hi, uint2& lo) {
    uint32_t h[2], l[2];
#pragma unroll
    for (int e = 0; e < 2; e++) {
        const float a0 = __uint_as_float(x[2 * e]), a1 = __uint_as_float(x[2 * e + 1]);
        bf16x2 ph;
        ph[0] = (__bf16)a0;
        ph[1] = (__bf16)a1;
        const uint32_t hb = __builtin_bit_cast(uint32_t, ph);
        bf16x2 pl;
        pl[0] = (__bf16)(a0 - __uint_as_float(hb << 16));
        pl[1] = (__bf16)(a1 - __uint_as_float(hb & 0xFFFF0000u));
        h[e] = hb;
        l[e] = __builtin_bit_cast(uint32_t, pl);
    }
    hi = make_uint2(h[0], h[1]);
    lo = make_uint2(l[0], l[1]);
}

template <int KS>
__device__ __forceinline__ int swz_k(int r, int piece) {
    if constexpr (KS == 32) return swz64(r, piece);
    else return r * 128 + ((piece ^ ((r >> 1) & 7)) << 4);
}

template <bool HAS_ZP, int KS, int P, int T>
__global__ __launch_bounds__(256, T == 2 ? 2 : KS == 64 ? 3 : 4) void gemm_f32_int_kernel(Bf16Args g) {
    constexpr int TM = T, TN = T;
    constexpr int BT = 64 * T;                          // tile rows and columns
    constexpr int PANEL = BT * KS * 2;                  // one K step of one operand
    constexpr int SPAN = BT * 16;                       // the step's scales: up to 4 per column
    constexpr int CPR = KS / 4;                         // 16-byte activation chunks per row
    constexpr int RPP = 256 / CPR;                      // activation rows per pass
    constexpr int AP = BT / RPP;                        // activation chunks per thread and step
    constexpr int BQ = 256 / BT;                        // threads per weight column and step
    constexpr int VPT = BT * KS / 256;                  // weights per thread and step
    constexpr int NWB = VPT / 8;                        // 32-bit weight words per thread and step
    constexpr int NSUB = KS / 16;                       // MFMA sub-steps per K step
    constexpr int BUF = 3 * PANEL + SPAN;               // A hi, A lo, B, scales
    static_assert(AP % NSUB == 0 || NSUB % AP == 0, "activation chunks per sub-step");
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * BUF];

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int mt = (g.M + BT - 1) / BT;
    const int nt = (g.N + BT - 1) / BT;
    const int tiles = mt * nt;
    const int v = xcd_index(blockIdx.x, tiles * g.splits);
    const int split = v / tiles, tt = v - split * tiles;
    const int m0 = (tt % mt) * BT;
    const int n0 = (tt / mt) * BT;
    const int kbase = split * g.sps * KS;                  // this split's first K value

    const __amdgpu_buffer_rsrc_t ra_rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(g.a), (short)0, (int)g.a_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rb_rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(g.b), (short)0, (int)g.b_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(g.scales), (short)0, (int)g.s_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rz_rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(HAS_ZP ? g.zp : g.b), (short)0, (int)(HAS_ZP ? g.z_bytes : 0), 0x00020000);

    // activations: thread t moves four floats (chunk t % CPR) of rows
    // t / CPR + RPP i
    const int a_r = t / CPR, a_c = t % CPR;
    const uint32_t a_off = (uint32_t)(m0 + a_r) * (uint32_t)g.K * 4u + 16u * a_c;
    const uint32_t a_rows = (uint32_t)RPP * (uint32_t)g.K * 4u;
    struct StageA {
        u32x4 v[AP];
    };
    auto fetch_a = [&](int k0, StageA& st) {
#pragma unroll
        for (int i = 0; i < AP; i++)
            st.v[i] = __builtin_amdgcn_raw_buffer_load_b128(ra_rs, a_off + a_rows * i + 4u * (kbase + k0), 0, 0);
    };
    auto stash_a = [&](const StageA& st, int buf, int i) {
        uint2 hi, lo;
        split4(st.v[i], hi, lo);
        const int off = swz_k<KS>(a_r + RPP * i, a_c >> 1) + 8 * (a_c & 1);
        *reinterpret_cast<uint2*>(lds + buf * BUF + off) = hi;
        *reinterpret_cast<uint2*>(lds + buf * BUF + PANEL + off) = lo;
    };

    // weights: thread t takes VPT values (NWB words) of column t / BQ, part
    // t % BQ of the step, which lie in one quantization block
    const int b_c = t / BQ, b_h = t % BQ;
    struct StageB {
        uint32_t b[NWB];
        uint32_t s;
        uint8_t z;
        uint32_t zsh;
    };
    auto fetch_b = [&](int k0, StageB& st) {
        const int col = n0 + b_c;
        const uint32_t kq = (uint32_t)(kbase + k0) + (uint32_t)(VPT * b_h);   // first K value of the part
        const uint32_t boff = (uint32_t)col * (uint32_t)g.col_bytes + kq / 2u;
        if constexpr (NWB == 2) {
            const uint2 x = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rb_rs, boff, 0, 0));
            st.b[0] = x.x;
            st.b[1] = x.y;
        } else {
            st.b[0] = __builtin_amdgcn_raw_buffer_load_b32(rb_rs, boff, 0, 0);
        }
        const uint32_t blk = kq >> g.log2_bs;
        st.s = __builtin_amdgcn_raw_buffer_load_b32(rs_rs, 4u * ((uint32_t)col * (uint32_t)g.nb + blk), 0, 0);
        if constexpr (HAS_ZP) {
            st.z = __builtin_amdgcn_raw_buffer_load_b8(rz_rs, (uint32_t)col * (uint32_t)g.zp_row + (blk >> 1), 0, 0);
            st.zsh = 4u * (blk & 1u);
        }
    };
    // word d (8 values) of a staged weight as the exact bf16 integers q - zp
    // (piece NWB h + d of the column): even and odd nibbles masked into
    // bytes, v_cvt_f32_ubyte, the zero point subtracted in float32 (exact),
    // the upper halves of two results packed in one v_perm.  The part's scale
    // goes to its scale period's slot of the step's scale row (parts of one
    // period write the same value).
    auto stash_b = [&](const StageB& st, int buf, int d) {
        const float zf = HAS_ZP ? (float)__builtin_amdgcn_ubfe((uint32_t)st.z, st.zsh, 4) : 8.f;
        const uint32_t word = st.b[d];
        const uint32_t lo = opaque_and(word, 0x0F0F0F0Fu);
        const uint32_t hi = opaque_and(word >> 4, 0x0F0F0F0Fu);
        const float w[8] = {ubyte_to_f32<0>(lo) - zf, ubyte_to_f32<0>(hi) - zf, ubyte_to_f32<1>(lo) - zf,
                            ubyte_to_f32<1>(hi) - zf, ubyte_to_f32<2>(lo) - zf, ubyte_to_f32<2>(hi) - zf,
                            ubyte_to_f32<3>(lo) - zf, ubyte_to_f32<3>(hi) - zf};
        uint32_t v[4];
#pragma unroll
        for (int e = 0; e < 4; e++)
            v[e] = __builtin_amdgcn_perm(__float_as_uint(w[2 * e + 1]), __float_as_uint(w[2 * e]), 0x07060302u);
        *reinterpret_cast<u32x4*>(lds + buf * BUF + 2 * PANEL + swz_k<KS>(b_c, NWB * b_h + d)) =
            u32x4{v[0], v[1], v[2], v[3]};
        if (d == 0)
            *reinterpret_cast<uint32_t*>(lds + buf * BUF + 3 * PANEL + 16 * b_c + 4 * ((VPT * b_h) / (16 * P))) = st.s;
    };

    f32x16 acc[TM][TN], part[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0.f;
    const f32x16 zero = {};

    // one K step from buffer buf: per scale period, the period's MFMAs (the
    // first of each tile starting from zero) and the fold with the period's
    // scale; the next step (held in na, nb) is staged into buf ^ 1 in between
    auto step_body = [&](int buf, const StageA& na, const StageB& nb) {
        const uint8_t* base = lds + buf * BUF;
#pragma unroll
        for (int ks = 0; ks < NSUB; ks++) {
            const int piece = 2 * ks + (lane >> 5);
            bf16x8 ah[TM], al[TM], bw[TN];
#pragma unroll
            for (int i = 0; i < TM; i++) {
                const int r = wm * (32 * TM) + i * 32 + (lane & 31);
                ah[i] = *reinterpret_cast<const bf16x8*>(base + swz_k<KS>(r, piece));
                al[i] = *reinterpret_cast<const bf16x8*>(base + PANEL + swz_k<KS>(r, piece));
            }
#pragma unroll
            for (int j = 0; j < TN; j++) {
                const int c = wn * (32 * TN) + j * 32 + (lane & 31);
                bw[j] = *reinterpret_cast<const bf16x8*>(base + 2 * PANEL + swz_k<KS>(c, piece));
            }
#pragma unroll
            for (int i = 0; i < AP / NSUB; i++) stash_a(na, buf ^ 1, (AP / NSUB) * ks + i);
            if (ks < NWB) stash_b(nb, buf ^ 1, ks);
            const bool first = ks % P == 0;
#pragma unroll
            for (int i = 0; i < TM; i++)
#pragma unroll
                for (int j = 0; j < TN; j++) {
                    part[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[i], bw[j], first ? zero : part[i][j], 0, 0, 0);
                    part[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[i], bw[j], part[i][j], 0, 0, 0);
                }
            if (ks % P == P - 1) {
                // fold: this lane's column and the period's scale
#pragma unroll
                for (int j = 0; j < TN; j++) {
                    const int c = wn * (32 * TN) + j * 32 + (lane & 31);
                    const float sc = *reinterpret_cast<const float*>(base + 3 * PANEL + 16 * c + 4 * (ks / P));
#pragma unroll
                    for (int i = 0; i < TM; i++)
#pragma unroll
                        for (int r = 0; r < 16; r++) acc[i][j][r] = fmaf(sc, part[i][j][r], acc[i][j][r]);
                }
            }
        }
    };

    const int steps = min(g.sps, g.K / KS - split * g.sps);
    // D register stages: step st stages step st + 1 (requested D - 1 steps
    // earlier) into LDS and requests step st + D into the stage it frees
    constexpr int D = 2;
    int buf = 0;
    auto one_step = [&](int st, const StageA& ua, const StageB& ub, StageA& la, StageB& lb) {
        fetch_a((st + D) * KS, la);
        fetch_b((st + D) * KS, lb);
        __builtin_amdgcn_sched_barrier(0);    // issue the requests first
        step_body(buf, ua, ub);
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        buf ^= 1;
    };
    // Step j's data lives in stage (j - r) mod D, r = steps mod D: the loop
    // then runs whole groups of D steps with fixed stage roles (no tail,
    // whose conditional steps would keep every stage live past the loop);
    // the r leading steps run before it.
    StageA sa[D];
    StageB sb[D];
    auto lead = [&](auto rc) {
        constexpr int R = decltype(rc)::value;
#pragma unroll
        for (int j = 0; j < D; j++) {
            fetch_a(j * KS, sa[(j - R + D) % D]);
            fetch_b(j * KS, sb[(j - R + D) % D]);
        }
#pragma unroll
        for (int i = 0; i < AP; i++) stash_a(sa[(D - R) % D], 0, i);
#pragma unroll
        for (int d = 0; d < NWB; d++) stash_b(sb[(D - R) % D], 0, d);
        __syncthreads();
#pragma unroll
        for (int j = 0; j < R; j++)
            one_step(j, sa[(j + 1 - R + D) % D], sb[(j + 1 - R + D) % D], sa[(j - R + D) % D], sb[(j - R + D) % D]);
    };
    const int r = steps % D;
    if (D == 2) {
        if (r == 0) lead(IntC<0>{}); else lead(IntC<1>{});
    } else {
        switch (r) {
            case 0: lead(IntC<0>{}); break;
            case 1: lead(IntC<1 % D>{}); break;
            case 2: lead(IntC<2 % D>{}); break;
            default: lead(IntC<3 % D>{}); break;
        }
    }
    for (int st = r; st < steps; st += D) {
#pragma unroll
        for (int u = 0; u < D; u++) one_step(st + u, sa[(u + 1) % D], sb[(u + 1) % D], sa[u], sb[u]);
    }

    // epilogue: + bias, float32 store (or the partial, without bias)
    float* const out = g.part ? g.part + (int64_t)split * g.M * g.N : static_cast<float*>(g.y);
#pragma unroll
    for (int j = 0; j < TN; j++) {
        const int n = n0 + wn * (32 * TN) + j * 32 + (lane & 31);
        if (n >= g.N) continue;
        const float bv = (!g.part && g.bias) ? g.bias[n] : 0.f;
#pragma unroll
        for (int i = 0; i < TM; i++)
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int m = m0 + wm * (32 * TM) + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (m < g.M) out[(int64_t)m * g.N + n] = acc[i][j][r] + bv;
            }
    }
}

// ---------------------------------------------------------------------------
// split-K reduction: Y = sum over the splits of the float32 partials, in
// split order (deterministic), + bias, rounded to Y's type.
// ---------------------------------------------------------------------------
template <bool BF16>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part, int splits,
                                                            int64_t mn, int N, const float* __restrict__ bias,
                                                            void* __restrict__ y, int vec) {
    const int64_t stride = (int64_t)gridDim.x * 256 * 4;
    for (int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4; i < mn; i += stride) {
        float v[4];
        if (vec && i + 4 <= mn) {
            // four columns of one row (N % 4 == 0); the slices are requested
            // ahead of the additions, which stay in split order
            float4 x = *reinterpret_cast<const float4*>(part + i);
            int sp = 1;
            for (; sp + 1 < splits; sp += 2) {
                const float4 z0 = *reinterpret_cast<const float4*>(part + (int64_t)sp * mn + i);
                const float4 z1 = *reinterpret_cast<const float4*>(part + (int64_t)(sp + 1) * mn + i);
                x.x += z0.x; x.y += z0.y; x.z += z0.z; x.w += z0.w;
                x.x += z1.x; x.y += z1.y; x.z += z1.z; x.w += z1.w;
            }
            if (sp < splits) {
                const float4 z = *reinterpret_cast<const float4*>(part + (int64_t)sp * mn + i);
                x.x += z.x; x.y += z.y; x.z += z.z; x.w += z.w;
            }
            v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
            if (bias) {
                const int c = (int)(i % N);
#pragma unroll
                for (int e = 0; e < 4; e++) v[e] += bias[c + e];
            }
            if constexpr (BF16) {
                const uint32_t lo = (uint32_t)f32_to_bf16_rtne(v[0]) | ((uint32_t)f32_to_bf16_rtne(v[1]) << 16);
                const uint32_t hi = (uint32_t)f32_to_bf16_rtne(v[2]) | ((uint32_t)f32_to_bf16_rtne(v[3]) << 16);
                *reinterpret_cast<uint2*>(static_cast<uint16_t*>(y) + i) = make_uint2(lo, hi);
            } else {
                *reinterpret_cast<float4*>(static_cast<float*>(y) + i) = make_float4(v[0], v[1], v[2], v[3]);
            }
            continue;
        }
#pragma unroll
        for (int e = 0; e < 4; e++) {
            v[e] = 0.f;
            if (i + e < mn) {
                float x = part[i + e];
                for (int sp = 1; sp < splits; sp++) x += part[(int64_t)sp * mn + i + e];
                v[e] = x;
            }
        }
#pragma unroll
        for (int e = 0; e < 4; e++) {
            if (i + e >= mn) break;
            const float o = bias ? v[e] + bias[(i + e) % N] : v[e];
            if constexpr (BF16)
                static_cast<uint16_t*>(y)[i + e] = f32_to_bf16_rtne(o);
            else
                static_cast<float*>(y)[i + e] = o;
        }
    }
}

// The tail split's partial tiles: element (r, c) of tail tile t is the sum of
// its splits in split order, + bias, rounded to bf16; four columns per thread.
__global__ __launch_bounds__(256) void tail_reduce_kernel(const float* __restrict__ tp, int splits, int tail_tiles,
                                                          int full_tiles, int mt, int M, int N,
                                                          const float* __restrict__ bias, uint16_t* __restrict__ y,
                                                          int vec) {
    constexpr int TILE = B4_M * B4_N;
    const int64_t total = (int64_t)tail_tiles * TILE / 4;
    for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < total; q += (int64_t)gridDim.x * blockDim.x) {
        const int64_t e0 = q * 4;
        const int t = (int)(e0 / TILE);
        const int rc = (int)(e0 - (int64_t)t * TILE);
        const int r = rc / B4_N, c = rc % B4_N;
        const int tt = full_tiles + t;
        const int m = (tt % mt) * B4_M + r, n0 = (tt / mt) * B4_N + c;
        if (m >= M) continue;
        float4 x = *reinterpret_cast<const float4*>(tp + e0);
        for (int sp = 1; sp < splits; sp++) {
            const float4 z = *reinterpret_cast<const float4*>(tp + ((int64_t)sp * tail_tiles) * TILE + e0);
            x.x += z.x; x.y += z.y; x.z += z.z; x.w += z.w;
        }
        const float v[4] = {x.x, x.y, x.z, x.w};
        if (vec && n0 + 4 <= N) {          // four bf16 in one 8-byte store
            uint16_t o[4];
#pragma unroll
            for (int e = 0; e < 4; e++) o[e] = f32_to_bf16_rtne(bias ? v[e] + bias[n0 + e] : v[e]);
            *reinterpret_cast<uint2*>(y + (int64_t)m * N + n0) =
                make_uint2((uint32_t)o[0] | ((uint32_t)o[1] << 16), (uint32_t)o[2] | ((uint32_t)o[3] << 16));
            continue;
        }
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const int n = n0 + e;
            if (n < N) y[(int64_t)m * N + n] = f32_to_bf16_rtne(bias ? v[e] + bias[n] : v[e]);
        }
    }
}

// The gated tail split: tail tile t's partials are in the wide kernel's
// column order (wavefront block w: gate columns 32 w .. 32 w + 31 at tile
// columns 64 w .., the matching up columns at 64 w + 32 ..); h column
// 32 w + c of the tile is silu(gate + bias) * (up + bias) of the split sums
// (in split order), rounded to bf16; four h columns per thread.
__global__ __launch_bounds__(256) void tail_reduce_silu_kernel(const float* __restrict__ tp, int splits,
                                                               int tail_tiles, int full_tiles, int mt, int M, int I,
                                                               const float* __restrict__ bias,
                                                               uint16_t* __restrict__ h) {
    constexpr int TILE = B4_M * B4_N;
    constexpr int HT = B4_N / 2;                        // h columns per tile
    const int64_t total = (int64_t)tail_tiles * B4_M * HT / 4;
    for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < total; q += (int64_t)gridDim.x * blockDim.x) {
        const int64_t e0 = q * 4;
        const int t = (int)(e0 / (B4_M * HT));
        const int rc = (int)(e0 - (int64_t)t * (B4_M * HT));
        const int r = rc / HT, hl = rc % HT;
        const int tt = full_tiles + t;
        const int m = (tt % mt) * B4_M + r, hc0 = (tt / mt) * HT + hl;
        if (m >= M) continue;
        const int gcol = (hl >> 5) * 64 + (hl & 31);     // gate column in the tile; up at + 32
        const int64_t base = (int64_t)t * TILE + (int64_t)r * B4_N + gcol;
        float4 gs = *reinterpret_cast<const float4*>(tp + base);
        float4 us = *reinterpret_cast<const float4*>(tp + base + 32);
        for (int sp = 1; sp < splits; sp++) {
            const int64_t o = (int64_t)sp * tail_tiles * TILE + base;
            const float4 zg = *reinterpret_cast<const float4*>(tp + o);
            const float4 zu = *reinterpret_cast<const float4*>(tp + o + 32);
            gs.x += zg.x; gs.y += zg.y; gs.z += zg.z; gs.w += zg.w;
            us.x += zu.x; us.y += zu.y; us.z += zu.z; us.w += zu.w;
        }
        const float gv[4] = {gs.x, gs.y, gs.z, gs.w}, uv[4] = {us.x, us.y, us.z, us.w};
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const int hc = hc0 + e;
            if (hc >= I) break;
            const float gg = gv[e] + (bias ? bias[hc] : 0.f);
            const float uu = uv[e] + (bias ? bias[I + hc] : 0.f);
            h[(int64_t)m * I + hc] = f32_to_bf16_rtne(gg / (1.0f + expf(-gg)) * uu);
        }
    }
}

// The unfused path's second step: h[m][i] = silu(y[m][i]) * y[m][I + i] on
// the product y (already rounded to the activation type), in float32.
template <bool BF16>
__global__ __launch_bounds__(256) void silu_mul_rows_kernel(const void* __restrict__ y, int64_t M, int64_t I,
                                                            void* __restrict__ h) {
    const int64_t total = M * I;
    for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < total; q += (int64_t)gridDim.x * blockDim.x) {
        const int64_t m = q / I, i = q - m * I;
        float gg, uu;
        if constexpr (BF16) {
            gg = bf16_to_f32(static_cast<const uint16_t*>(y)[m * 2 * I + i]);
            uu = bf16_to_f32(static_cast<const uint16_t*>(y)[m * 2 * I + I + i]);
        } else {
            gg = static_cast<const float*>(y)[m * 2 * I + i];
            uu = static_cast<const float*>(y)[m * 2 * I + I + i];
        }
        const float v = gg / (1.0f + expf(-gg)) * uu;
        if constexpr (BF16)
            static_cast<uint16_t*>(h)[q] = f32_to_bf16_rtne(v);
        else
            static_cast<float*>(h)[q] = v;
    }
}

}  // namespace

namespace {

// Which kernel a problem takes, its output tiles and its K split.
struct Plan {
    enum Kind { LEGACY_BF16, WIDE, REG128, F32_INT, LEGACY_F32 } kind;
    int64_t tiles = 1;
    int f32_t = 2;                 // F32_INT: MFMA tiles per wavefront side (tile 64 f32_t)
    int f32_ks = F_K;              // F32_INT: K values per step (32 or 64)
    int splits = 1, sps = 1;
    int tail_tiles = 0, tail_splits = 1, tail_sps = 0;   // wide kernel: split of the last round
    size_t ws = 0;                 // workspace bytes for the split partials
};

// Wide kernel over more than one round of tiles: when the last round would
// leave more than half of the CUs idle, split its tiles along K (at least
// four K steps per part) so that it finishes sooner.
void choose_tail_split(Plan& pl, int64_t cus, int steps) {
    if (pl.splits > 1 || pl.tiles <= cus) return;
    const int64_t rem = pl.tiles % cus;
    if (rem == 0 || rem > cus / 2) return;
    int ts = (int)(cus / rem);
    if (ts > 4) ts = 4;
    if (ts > steps / 4) ts = steps / 4;
    if (ts < 2) return;
    pl.tail_sps = (steps + ts - 1) / ts;
    pl.tail_splits = (steps + pl.tail_sps - 1) / pl.tail_sps;
    if (pl.tail_splits < 2) return;
    pl.tail_tiles = (int)rem;
    pl.ws = (size_t)pl.tail_splits * (size_t)rem * B4_M * B4_N * 4;
}

constexpr size_t kMaxWorkspace = size_t(1) << 30;

// Split K only when the output tiles leave resident workgroup slots idle,
// keeping at least four K steps per split and at most max_sp splits.
void choose_split(Plan& pl, const Problem& p, int64_t resident, int steps, int64_t max_sp = 1 << 20) {
    pl.splits = 1;
    pl.sps = steps;
    if (pl.tiles >= resident) return;
    int64_t sp = resident / pl.tiles;
    if (sp > steps / 4) sp = steps / 4;
    if (sp > max_sp) sp = max_sp;
    while (sp > 1 && (size_t)sp * (size_t)(p.M * p.N) * 4 > kMaxWorkspace) sp--;
    if (sp <= 1) return;
    pl.sps = (int)((steps + sp - 1) / sp);
    pl.splits = (steps + pl.sps - 1) / pl.sps;
    if (pl.splits > 1) pl.ws = (size_t)pl.splits * (size_t)(p.M * p.N) * 4;
}

// The plan is a function of the problem's shape alone (the ABI layer has
// checked the alignment of A and of the scales), sized for the 256 CUs of an
// MI355X whatever the device reports: the K split fixes the float32
// summation order, so results do not depend on the partition mode, and the
// workspace a caller must provide is known on the host before any HIP call.
constexpr int64_t kPlanCUs = 256;

Plan plan_gemm(const Problem& p) {
    Plan pl;
    const int esz = p.bf16 ? 2 : 4;
    const bool vec_a = (p.K * esz) % 16 == 0;
    const int64_t a_bytes = p.M * p.K * esz, b_bytes = p.N * p.col_bytes;
    const int64_t lim = int64_t(1) << 31;
    const int64_t cus = kPlanCUs;
    if (p.bf16 && vec_a && (p.K % 8) == 0 && a_bytes + 256 * p.K * esz < lim &&
        b_bytes + 256 * p.col_bytes < lim && p.M * p.N < lim) {
        const int64_t big = ((p.M + 255) / 256) * ((p.N + 255) / 256);
        if (p.M > 128 && p.K % B4_K == 0 && p.K % p.bs == 0) {
            pl.kind = Plan::WIDE;
            pl.tiles = big;
            choose_split(pl, p, cus, (int)(p.K / B4_K));   // one 256 x 256 workgroup per CU
            choose_tail_split(pl, cus, (int)(p.K / B4_K));
        } else {
            pl.kind = Plan::REG128;
            pl.tiles = ((p.M + 127) / 128) * ((p.N + 127) / 128);
        }
    } else if (p.bf16) {
        pl.kind = Plan::LEGACY_BF16;
    } else if (vec_a && p.K % F_K == 0 && p.K % p.bs == 0 && p.M * p.K * 4 + 128 * p.K * 4 < lim &&
               b_bytes + 128 * p.col_bytes < lim && p.M * p.N < lim) {
        pl.kind = Plan::F32_INT;
        const int64_t big = ((p.M + 127) / 128) * ((p.N + 127) / 128);
        if (big >= 2 * cus) {                               // two 128 x 128 workgroups per CU
            pl.f32_t = 2;
            pl.tiles = big;
            choose_split(pl, p, 2 * cus, (int)(p.K / F_K));
        } else {                                            // 64 x 64 tiles, at most 4 K splits
            pl.f32_t = 1;
            // 64-value K steps where the blocks allow (a block of 32 or
            // more values holds each thread's 16 weights of a step)
            pl.f32_ks = (p.K % 64 == 0 && p.bs >= 32) ? 64 : F_K;
            pl.tiles = ((p.M + 63) / 64) * ((p.N + 63) / 64);
            choose_split(pl, p, 2 * cus, (int)(p.K / pl.f32_ks), 4);
        }
    } else {
        pl.kind = Plan::LEGACY_F32;
    }
    return pl;
}

}  // namespace

namespace {

Bf16Args bf16_args(const Problem& p, const Plan& pl, void* ws) {
    const int esz = p.bf16 ? 2 : 4;
    Bf16Args b;
    b.a = p.a; b.b = p.b; b.scales = p.scales; b.zp = p.has_zp ? p.zp : nullptr;
    b.bias = p.bias; b.y = p.y;
    b.M = (int)p.M; b.K = (int)p.K; b.N = (int)p.N; b.col_bytes = (int)p.col_bytes;
    b.k_pad = (int)((int64_t)p.nb * p.bs); b.nb = p.nb; b.zp_row = p.zp_row;
    int l2 = 0;
    while ((1 << l2) < p.bs) l2++;
    b.log2_bs = l2;
    b.a_bytes = (uint32_t)(p.M * p.K * esz); b.b_bytes = (uint32_t)(p.N * p.col_bytes);
    b.s_bytes = (uint32_t)(p.N * p.nb * esz); b.z_bytes = (uint32_t)(p.N * p.zp_row);
    b.splits = pl.splits;
    b.sps = pl.sps;
    b.part = pl.splits > 1 ? static_cast<float*>(ws) : nullptr;
    b.full_tiles = (int)(pl.tiles - pl.tail_tiles);
    b.tail_tiles = pl.tail_tiles;
    b.tail_splits = pl.tail_splits;
    b.tail_sps = pl.tail_sps;
    b.tail_part = pl.tail_tiles ? static_cast<float*>(ws) : nullptr;
    b.silu_half = 0;
    return b;
}

// The gated gate||up product on the wide kernel: no K split (the gated
// epilogue needs whole sums); the last round of tiles may still be split
// along K, its partials reduced by the gated tail kernel.
Plan plan_gemm_silu(const Problem& p) {
    Plan pl = plan_gemm(p);
    if (pl.kind != Plan::WIDE) return pl;
    Plan q;
    q.kind = Plan::WIDE;
    q.tiles = pl.tiles;
    q.splits = 1;
    q.sps = (int)(p.K / B4_K);
    choose_tail_split(q, kPlanCUs, q.sps);
    return q;
}

bool silu_decode(const Problem& p) { return p.M == 1 && p.K <= gemv_max_k(p.bs); }

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

}  // namespace

size_t gemm_workspace_bytes(const Problem& p) { return gemv_rows_ok(p) || smallm_ok(p) ? 0 : plan_gemm(p).ws; }

size_t gemm_silu_workspace_bytes(const Problem& p) {
    if (silu_decode(p)) return 0;
    const Plan pl = plan_gemm_silu(p);
    if (pl.kind == Plan::WIDE) return pl.ws;
    // the unfused path: the product's own workspace, then y [M][N]
    return align256(gemm_workspace_bytes(p)) + (size_t)(p.M * p.N) * (p.bf16 ? 2 : 4);
}

int launch_gemm_silu(const Problem& p, hipStream_t s, void* ws, size_t ws_bytes) {
    if (silu_decode(p)) return launch_gemv_silu(p, s);
    const Plan pl = plan_gemm_silu(p);
    const size_t need = gemm_silu_workspace_bytes(p);
    if (need && (!ws || ws_bytes < need))
        return fail(MNB_E_ARG, "gemm_silu: workspace of %zu bytes, %zu needed", ws ? ws_bytes : (size_t)0, need);
    const int64_t I = p.N / 2;
    if (pl.kind == Plan::WIDE) {
        Bf16Args b = bf16_args(p, pl, ws);
        b.silu_half = (int)I;
        const unsigned grid = (unsigned)(pl.tail_tiles ? b.full_tiles + (int64_t)pl.tail_tiles * pl.tail_splits
                                                       : pl.tiles);
        const bool bs16 = p.bs == 16;
        auto kern = p.has_zp
                        ? (bs16 ? gemm_bf16_wide_kernel<true, true, true> : gemm_bf16_wide_kernel<true, false, true>)
                        : (bs16 ? gemm_bf16_wide_kernel<false, true, true> : gemm_bf16_wide_kernel<false, false, true>);
        hipLaunchKernelGGL(kern, dim3(grid), dim3(512), 0, s, b);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return fail(MNB_E_HIP, "gated gemm launch: %s", hipGetErrorString(e));
        if (pl.tail_tiles) {
            const int64_t q = (int64_t)pl.tail_tiles * B4_M * (B4_N / 2) / 4;
            int64_t blocks = (q + 255) / 256;
            const int64_t cap = (int64_t)device_compute_units() * 8;
            if (blocks > cap) blocks = cap;
            hipLaunchKernelGGL(tail_reduce_silu_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                               static_cast<const float*>(ws), pl.tail_splits, pl.tail_tiles, b.full_tiles,
                               (int)((p.M + B4_M - 1) / B4_M), (int)p.M, (int)I, p.bias,
                               static_cast<uint16_t*>(p.y));
            e = hipGetLastError();
            if (e != hipSuccess) return fail(MNB_E_HIP, "gated tail reduction launch: %s", hipGetErrorString(e));
        }
        return MNB_OK;
    }
    // the unfused standard graph: the product into the workspace, then the
    // gated rows
    const size_t gws = align256(gemm_workspace_bytes(p));
    Problem q = p;
    q.y = static_cast<uint8_t*>(ws) + gws;
    int st = launch_gemm(q, s, gws ? ws : nullptr, gws);
    if (st != MNB_OK) return st;
    int64_t blocks = (p.M * I + 255) / 256;
    const int64_t cap = (int64_t)device_compute_units() * 8;
    if (blocks > cap) blocks = cap;
    if (p.bf16)
        hipLaunchKernelGGL(silu_mul_rows_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, s, q.y, p.M, I, p.y);
    else
        hipLaunchKernelGGL(silu_mul_rows_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, s, q.y, p.M, I, p.y);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(MNB_E_HIP, "gated rows launch: %s", hipGetErrorString(e));
    return MNB_OK;
}

int launch_gemm(const Problem& p, hipStream_t s, void* ws, size_t ws_bytes) {
    if (gemv_rows_ok(p)) return launch_gemv_rows(p, s);
    if (smallm_ok(p)) return launch_smallm(p, s);
    const Plan pl = plan_gemm(p);
    if (pl.ws && (!ws || ws_bytes < pl.ws))                 // the ABI layer checked this
        return fail(MNB_E_ARG, "gemm: workspace of %zu bytes, %zu needed", ws ? ws_bytes : (size_t)0, pl.ws);
    GemmArgs a;
    a.a = p.a; a.b = p.b; a.scales = p.scales; a.zp = p.has_zp ? p.zp : nullptr;
    a.bias = p.bias; a.y = p.y;
    a.M = p.M; a.K = p.K; a.N = p.N; a.col_bytes = p.col_bytes;
    a.k_pad = (int64_t)p.nb * p.bs;
    a.nb = p.nb; a.zp_row = p.zp_row; a.bs = p.bs;
    const int esz = p.bf16 ? 2 : 4;
    a.vec_a = ((p.K * esz) % 16 == 0) && ((reinterpret_cast<uintptr_t>(p.a) & 15) == 0);
    const Bf16Args b = bf16_args(p, pl, ws);
    const bool bs16 = p.bs == 16;
    const unsigned grid = (unsigned)(pl.tail_tiles ? b.full_tiles + (int64_t)pl.tail_tiles * pl.tail_splits
                                                   : pl.tiles * pl.splits);
    switch (pl.kind) {
        case Plan::WIDE: {
            auto kern = p.has_zp ? (bs16 ? gemm_bf16_wide_kernel<true, true> : gemm_bf16_wide_kernel<true, false>)
                                 : (bs16 ? gemm_bf16_wide_kernel<false, true> : gemm_bf16_wide_kernel<false, false>);
            hipLaunchKernelGGL(kern, dim3(grid), dim3(512), 0, s, b);
            break;
        }
        case Plan::REG128:
            hipLaunchKernelGGL((gemm_bf16_kernel<128, 128, 8>), dim3(grid), dim3(512), 0, s, b);
            break;
        case Plan::F32_INT: {
            // P: 16-value MFMA sub-steps per scale period
            decltype(&gemm_f32_int_kernel<true, 32, 1, 2>) kern;
            if (pl.f32_t == 2)
                kern = p.has_zp ? (bs16 ? gemm_f32_int_kernel<true, 32, 1, 2> : gemm_f32_int_kernel<true, 32, 2, 2>)
                                : (bs16 ? gemm_f32_int_kernel<false, 32, 1, 2> : gemm_f32_int_kernel<false, 32, 2, 2>);
            else if (pl.f32_ks == 64)
                kern = p.has_zp ? (p.bs == 32 ? gemm_f32_int_kernel<true, 64, 2, 1> : gemm_f32_int_kernel<true, 64, 4, 1>)
                                : (p.bs == 32 ? gemm_f32_int_kernel<false, 64, 2, 1> : gemm_f32_int_kernel<false, 64, 4, 1>);
            else
                kern = p.has_zp ? (bs16 ? gemm_f32_int_kernel<true, 32, 1, 1> : gemm_f32_int_kernel<true, 32, 2, 1>)
                                : (bs16 ? gemm_f32_int_kernel<false, 32, 1, 1> : gemm_f32_int_kernel<false, 32, 2, 1>);
            hipLaunchKernelGGL(kern, dim3(grid), dim3(256), 0, s, b);
            break;
        }
        case Plan::LEGACY_BF16:
        case Plan::LEGACY_F32: {
            const dim3 g2((unsigned)((p.N + BN - 1) / BN), (unsigned)((p.M + BM - 1) / BM));
            if (pl.kind == Plan::LEGACY_BF16)
                hipLaunchKernelGGL(gemm_kernel<true>, g2, dim3(256), 0, s, a);
            else
                hipLaunchKernelGGL(gemm_kernel<false>, g2, dim3(256), 0, s, a);
            break;
        }
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(MNB_E_HIP, "gemm launch: %s", hipGetErrorString(e));
    if (pl.splits > 1) {
        const int64_t mn = p.M * p.N;
        int64_t blocks = (mn / 4 + 255) / 256;
        const int64_t cap = (int64_t)device_compute_units() * 8;
        if (blocks > cap) blocks = cap;
        if (blocks < 1) blocks = 1;
        // whole vectors of four: N % 4 == 0 and Y aligned to four elements
        // (the workspace slices are)
        const int vec = (p.N % 4 == 0) && (reinterpret_cast<uintptr_t>(p.y) % (p.bf16 ? 8 : 16) == 0);
        if (p.bf16)
            hipLaunchKernelGGL(splitk_reduce_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, s,
                               static_cast<const float*>(ws), pl.splits, mn, (int)p.N, p.bias, p.y, vec);
        else
            hipLaunchKernelGGL(splitk_reduce_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, s,
                               static_cast<const float*>(ws), pl.splits, mn, (int)p.N, p.bias, p.y, vec);
        e = hipGetLastError();
        if (e != hipSuccess) return fail(MNB_E_HIP, "gemm split-K reduction launch: %s", hipGetErrorString(e));
    }
    if (pl.tail_tiles) {
        const int64_t q = (int64_t)pl.tail_tiles * B4_M * B4_N / 4;
        int64_t blocks = (q + 255) / 256;
        const int64_t cap = (int64_t)device_compute_units() * 8;
        if (blocks > cap) blocks = cap;
        hipLaunchKernelGGL(tail_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                           static_cast<const float*>(ws), pl.tail_splits, pl.tail_tiles, b.full_tiles,
                           (int)((p.M + B4_M - 1) / B4_M), (int)p.M, (int)p.N, p.bias, static_cast<uint16_t*>(p.y),
                           (int)(p.N % 4 == 0 && reinterpret_cast<uintptr_t>(p.y) % 8 == 0));
        e = hipGetLastError();
        if (e != hipSuccess) return fail(MNB_E_HIP, "gemm tail reduction launch: %s", hipGetErrorString(e));
    }
    return MNB_OK;
}

}  // namespace mnb
