// Internal declarations shared by the libmnb translation units (not part of
// the public ABI, which is include/mnb.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mnb.h"

namespace mnb {

// Fully validated, derived parameters of one matmul launch.
struct Problem {
    int64_t M, K, N;
    int bs;               // block_size
    int nb;               // ceil(K / bs)
    int64_t col_bytes;    // nb * bs / 2: bytes of one packed column
    int zp_row;           // ceil(nb / 2): bytes of one packed zero-point row
    bool bf16;            // activations, scales and Y are bfloat16
    bool has_zp;
    const void* a;
    const uint8_t* b;
    const void* scales;
    const uint8_t* zp;
    const float* bias;
    void* y;
};

// Records `detail` as the calling thread's last error and returns `status`.
int fail(int status, const char* fmt, ...);

// Kernel launchers (one per translation unit).  They return MNB_OK or
// MNB_E_HIP and never validate: the ABI layer has already done so.
int launch_pack(int64_t K, int64_t N, int bs, const uint8_t* q,
                const uint8_t* zp, uint8_t* b_packed, uint8_t* zp_packed,
                hipStream_t s);
int launch_dequant(const Problem& p, int out_kind, void* w, hipStream_t s);
int launch_gemv(const Problem& p, hipStream_t s);
// 2 <= M <= 4 rows through the decode GEMV (each weight unpacked once for all
// rows) when the shape allows it and is no LM head (gemv_rows_ok);
// launch_gemm takes it then.
bool gemv_rows_ok(const Problem& p);
int launch_gemv_rows(const Problem& p, hipStream_t s);
// p.N = 2 * half: the gate half then the up half; y [half] = silu(gate) * up.
int launch_gemv_silu(const Problem& p, hipStream_t s);
// One row whose input is RMS-normalized on the fly: a = x / sqrt(mean x^2 +
// eps) * gamma (gamma [K] in the activation type, 16-byte aligned).
int launch_gemv_rmsnorm(const Problem& p, const void* gamma, float eps, hipStream_t s);
// QDQ normalization (axis 0: W[K][N], scales/zp [nb][N]; axis 1: W[N][K],
// scales/zp [N][nb]) into the MatMulNBits storage of p (p.has_zp is true).
int launch_import_qdq(const Problem& p, int axis, const uint8_t* w_q, const void* scales_q, const uint8_t* zp_q,
                      uint8_t* b_packed, void* scales, uint8_t* zp_packed, hipStream_t s);
int launch_gather_rows(const Problem& p, const int64_t* ids, int64_t n_ids, void* out, hipStream_t s);
// ws: the caller's workspace for per-segment partials of long rows, at least
// argmax_workspace_bytes (the ABI layer checks it).
int launch_argmax(bool bf16, int64_t M, int64_t N, const void* x, int64_t* idx, hipStream_t s, void* ws,
                  size_t ws_bytes);
size_t argmax_workspace_bytes(int64_t M, int64_t N);
// ws: the caller's float32 workspace for split-K partials, at least
// gemm_workspace_bytes (a function of the shape alone; the ABI layer checks
// it, and launch_gemm refuses a smaller one).
int launch_gemm(const Problem& p, hipStream_t s, void* ws, size_t ws_bytes);
size_t gemm_workspace_bytes(const Problem& p);
// The gated gate||up product (p.N = 2 * I, p.y = h [M][I]): the gated decode
// GEMV at M == 1, the wide prefill kernel with its gated epilogue where it
// applies, otherwise the product into the workspace and then the gated rows.
int launch_gemm_silu(const Problem& p, hipStream_t s, void* ws, size_t ws_bytes);
size_t gemm_silu_workspace_bytes(const Problem& p);
// 1 <= M <= 16 on the matrix cores (K % 32 == 0, block_size >= 32, A 16-byte
// aligned); launch_gemm takes it whenever smallm_ok holds.
bool smallm_ok(const Problem& p);
int launch_smallm(const Problem& p, hipStream_t s);
int64_t gemv_max_k(int bs);
// The persistent decode step (mnb_step.hip): every entry M == 1.  Workspace
// bytes for n entries (arrival counters and the entry table); whether the
// step kernel takes problem p (MNB_E_UNSUPPORTED with the reason if not);
// the grid (one workgroup per CU; HIP calls); writing the table for that grid
// into ws (synchronous); one cooperative launch (trace: the optional phase
// timestamps, grid * n * 5 uint64, or NULL); and, after the stream, the
// error word (a wait that ran out).
size_t step_workspace_bytes(int64_t n_ops);
int step_supports(const Problem& p, int64_t idx);
int step_grid(bool bf16, int* grid);
int step_prepare(const Problem* probs, int64_t n, int grid, void* ws);
int step_launch(bool bf16, int grid, void* ws, int64_t n, void* trace, hipStream_t s);
int step_check(void* ws, hipStream_t s);
int device_compute_units();   // CUs of the current device (cached); sizes grids only

// ---- device helpers ---------------------------------------------------------

// float32 -> bfloat16 bit pattern, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16_rtne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float((uint32_t)h << 16);
}

// A 32-bit AND whose result the compiler cannot see through, so that byte
// extraction of the result maps onto v_cvt_f32_ubyte{0,1,2,3} instead of a
// bit-field extract followed by a conversion.
__device__ __forceinline__ uint32_t opaque_and(uint32_t x, uint32_t m) {
    uint32_t r;
    asm("v_and_b32 %0, %1, %2" : "=v"(r) : "v"(x), "v"(m));
    return r;
}

template <int B>
__device__ __forceinline__ float ubyte_to_f32(uint32_t x) {
    return (float)((x >> (8 * B)) & 0xFFu);
}

// (x & m) | e in one v_and_or_b32.  gfx9 VOP3 encodings take no literal
// constants, so the compiler otherwise splits this into an AND and an OR; the
// masks are loop invariants that live in VGPRs.
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t e) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(m), "v"(e));
    return r;
}

}  // namespace mnb
