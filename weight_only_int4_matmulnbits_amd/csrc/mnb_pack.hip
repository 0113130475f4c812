// Preparation kernels: packing logical uint4 weights and zero points into the
// MatMulNBits storage, and the dequantization test hook.
//
// Storage (page "Qwen3 CPU Inference Critical Path", "Export contract",
// qwen3-int4-qdq: low nibble first, per-block scales and zero points along K;
// "Exact kernel inventory": packed UINT8 storage of 4-bit weights).  Column n
// is one run of col_bytes = nb * bs / 2 bytes; within it value k sits in byte
// k / 2 (low nibble when k is even), so the blocked layout is the K stream
// padded to whole blocks.  Pad nibbles are written 0.
#include "mnb_internal.h"

namespace mnb {
namespace {

// One thread writes 8 packed bytes (16 values of K) of one column.
__global__ __launch_bounds__(256) void pack_weights_kernel(
    const uint8_t* __restrict__ q, uint8_t* __restrict__ out, int64_t K,
    int64_t words_per_col, int64_t total_words, bool vec16) {
    int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (w >= total_words) return;
    int64_t n = w / words_per_col;
    int64_t j = w - n * words_per_col;
    int64_t k0 = j * 16;
    const uint8_t* qc = q + n * K;
    uint8_t v[16];
    if (vec16 && k0 + 16 <= K) {
        uint4 x = *reinterpret_cast<const uint4*>(qc + k0);
        const uint8_t* xb = reinterpret_cast<const uint8_t*>(&x);
#pragma unroll
        for (int i = 0; i < 16; i++) v[i] = xb[i];
    } else {
#pragma unroll
        for (int i = 0; i < 16; i++) v[i] = (k0 + i < K) ? qc[k0 + i] : 0;
    }
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        lo |= (uint32_t)((v[2 * i] & 0xF) | ((v[2 * i + 1] & 0xF) << 4)) << (8 * i);
        hi |= (uint32_t)((v[8 + 2 * i] & 0xF) | ((v[8 + 2 * i + 1] & 0xF) << 4))
              << (8 * i);
    }
    *reinterpret_cast<uint2*>(out + n * words_per_col * 8 + j * 8) = make_uint2(lo, hi);
}

// One thread writes one packed zero-point byte (two blocks).
__global__ __launch_bounds__(256) void pack_zero_points_kernel(
    const uint8_t* __restrict__ zp, uint8_t* __restrict__ out, int nb,
    int row, int64_t total) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total) return;
    int64_t n = i / row;
    int j = (int)(i - n * row);
    uint8_t lo = zp[n * nb + 2 * j] & 0xF;
    uint8_t hi = (2 * j + 1 < nb) ? (zp[n * nb + 2 * j + 1] & 0xF) : 0;
    out[i] = (uint8_t)(lo | (hi << 4));
}

__device__ __forceinline__ int zero_point(const uint8_t* zp, int zp_row,
                                          int64_t n, int b) {
    if (!zp) return 8;
    uint8_t byte = zp[n * zp_row + (b >> 1)];
    return (b & 1) ? (byte >> 4) : (byte & 0xF);
}

// Dequantization test hook: one thread per pair of K values.
__global__ __launch_bounds__(256) void dequant_kernel(Problem p, int out_kind,
                                                      void* __restrict__ w) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    int64_t pairs = (p.K + 1) / 2;
    if (i >= p.N * pairs) return;
    int64_t n = i / pairs;
    int64_t k0 = (i - n * pairs) * 2;
    uint8_t byte = p.b[n * p.col_bytes + k0 / 2];
    for (int h = 0; h < 2; h++) {
        int64_t k = k0 + h;
        if (k >= p.K) break;
        int b = (int)(k / p.bs);
        int qv = h ? (byte >> 4) : (byte & 0xF);
        int d = qv - zero_point(p.zp, p.zp_row, n, b);
        int64_t o = n * p.K + k;
        if (out_kind == 2) {
            static_cast<int8_t*>(w)[o] = (int8_t)d;
            continue;
        }
        float s = p.bf16 ? bf16_to_f32(static_cast<const uint16_t*>(p.scales)[n * p.nb + b])
                         : static_cast<const float*>(p.scales)[n * p.nb + b];
        if (out_kind == 0) {
            static_cast<float*>(w)[o] = __fmul_rn((float)d, s);
        } else {
            // One rounding of the exact product to bfloat16: the product is
            // exact in binary64; round it to odd in binary32 (toward zero,
            // then set the last bit if anything was dropped), which leaves
            // more than two spare bits, then round to nearest even.
            double e = (double)d * (double)s;
            float f = __double2float_rz(e);
            if ((double)f != e) f = __uint_as_float(__float_as_uint(f) | 1u);
            static_cast<uint16_t*>(w)[o] = f32_to_bf16_rtne(f);
        }
    }
}

inline unsigned grid_for(int64_t items, int threads) {
    return (unsigned)((items + threads - 1) / threads);
}

}  // namespace

int launch_pack(int64_t K, int64_t N, int bs, const uint8_t* q,
                const uint8_t* zp, uint8_t* b_packed, uint8_t* zp_packed,
                hipStream_t s) {
    int nb = (int)((K + bs - 1) / bs);
    int64_t words_per_col = (int64_t)nb * bs / 16;  // 8-byte words per column
    int64_t total = N * words_per_col;
    bool vec16 = (K % 16 == 0) && ((reinterpret_cast<uintptr_t>(q) & 15) == 0);
    hipLaunchKernelGGL(pack_weights_kernel, dim3(grid_for(total, 256)), dim3(256),
                       0, s, q, b_packed, K, words_per_col, total, vec16);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(MNB_E_HIP, "pack launch: %s", hipGetErrorString(e));
    if (zp) {
        int row = (nb + 1) / 2;
        int64_t tz = N * row;
        hipLaunchKernelGGL(pack_zero_points_kernel, dim3(grid_for(tz, 256)),
                           dim3(256), 0, s, zp, zp_packed, nb, row, tz);
        e = hipGetLastError();
        if (e != hipSuccess)
            return fail(MNB_E_HIP, "zero-point pack launch: %s", hipGetErrorString(e));
    }
    return MNB_OK;
}

int launch_dequant(const Problem& p, int out_kind, void* w, hipStream_t s) {
    int64_t items = p.N * ((p.K + 1) / 2);
    hipLaunchKernelGGL(dequant_kernel, dim3(grid_for(items, 256)), dim3(256), 0, s,
                       p, out_kind, w);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(MNB_E_HIP, "dequant launch: %s", hipGetErrorString(e));
    return MNB_OK;
}

}  // namespace mnb
