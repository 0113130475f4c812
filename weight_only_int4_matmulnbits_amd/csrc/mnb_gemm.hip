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

}  // namespace

int launch_gemm(const Problem& p, hipStream_t s) {
    GemmArgs a;
    a.a = p.a; a.b = p.b; a.scales = p.scales; a.zp = p.has_zp ? p.zp : nullptr;
    a.bias = p.bias; a.y = p.y;
    a.M = p.M; a.K = p.K; a.N = p.N; a.col_bytes = p.col_bytes;
    a.k_pad = (int64_t)p.nb * p.bs;
    a.nb = p.nb; a.zp_row = p.zp_row; a.bs = p.bs;
    const int esz = p.bf16 ? 2 : 4;
    a.vec_a = ((p.K * esz) % 16 == 0) && ((reinterpret_cast<uintptr_t>(p.a) & 15) == 0);
    const dim3 grid((unsigned)((p.N + BN - 1) / BN), (unsigned)((p.M + BM - 1) / BM));
    if (p.bf16)
        hipLaunchKernelGGL(gemm_kernel<true>, grid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(gemm_kernel<false>, grid, dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(MNB_E_HIP, "gemm launch: %s", hipGetErrorString(e));
    return MNB_OK;
}

}  // namespace mnb
