/*
 * mnb.h -- C ABI of libmnb, a weight-only block-INT4 MatMul for AMD MI355X
 * (gfx950), following the com.microsoft::MatMulNBits contract.
 *
 *   Y[M][N] = A[M][K] x dequant(B)[K][N] (+ bias[N])
 *   dequant(B)[k][n] = (q[n][k] - zp[n][k / block_size]) * scale[n][k / block_size]
 *
 * Sources (page "Qwen3 CPU Inference Critical Path"):
 *   "Exact kernel inventory", com.microsoft::MatMulNBits v1 row -- FP32
 *     activations, packed UINT8 storage of 4-bit weights, FP32 scales,
 *     block_size 32; weights stay compressed; GEMV decode and GEMM prefill.
 *   "INT4 MatMul is first", "Prepared weight-only plan" -- the plan captures
 *     K, N, nibble order, signedness, block size, tails, per-block scales and
 *     optional zero points, and packed storage aligned for the kernel; decode
 *     kernels unpack in registers, apply zero point and scale, accumulate in
 *     float32, and never expand the whole matrix.
 *   "INT4 MatMul is first", int4_gemv / int4_gemm -- decode (M == 1) and
 *     prefill are separate algorithms.
 *   "Export contract", qwen3-int4-qdq -- UINT4 stored low nibble first, one
 *     scale and zero point per block along K; BF16 activations and scales.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory.   Every tensor argument is a DEVICE pointer (memory of the current
 *           HIP device), row-major and contiguous, allocated and owned by the
 *           caller.  The library allocates no device memory (apart from the
 *           static array behind mnb_gemm_noalloc, loaded with the library's
 *           device code) and keeps no pointer to caller memory after a call
 *           returns (graph handles,
 *           below, are the one documented exception: they record the
 *           pointers given at creation).  Products that split K across
 *           workgroups (too few output tiles to fill the GPU) and ArgMax over
 *           long rows keep partial results in a caller-provided WORKSPACE
 *           ("Prepared weight-only plan": the plan captures a bounded
 *           workspace): its size is a pure function of the shape, returned
 *           by mnb_workspace_bytes / mnb_argmax_workspace_bytes /
 *           mnb_sequence_workspace_bytes on the host before any HIP call;
 *           0 means none is needed and NULL may be passed.  A workspace must
 *           be 256-byte aligned and at least that size, else the call
 *           returns MNB_E_ARG (MNB_E_ALIGN) and launches nothing; its
 *           contents on entry do not matter and are undefined on return.
 *           Calls that may overlap on the device (different streams, or a
 *           graph replayed beside eager calls) must not share a workspace.
 *           The choice of kernel and K split depends on the shape alone
 *           (never on the workspace offered, the pointers, or the device's
 *           compute-unit count), so results are a function of the inputs.
 * Ordering. Work is enqueued on `stream` (a hipStream_t passed as void*;
 *           NULL is the null stream) and the call returns once it is
 *           enqueued.  Results are valid after the stream is synchronized.
 * Errors.   Every call returns an mnb_status.  Arguments are validated on the
 *           host BEFORE any HIP call, so validation errors are reported even
 *           on a machine without a GPU and leave every buffer untouched.  A
 *           kernel-launch failure returns MNB_E_HIP; faults inside a kernel
 *           surface at the caller's next synchronization.  After any error the
 *           output buffers are undefined.  No call aborts the process or
 *           throws across the ABI.  mnb_last_error() gives a human-readable
 *           detail of the most recent error on the calling thread.
 * Threads.  The library's only mutable global state is the per-device
 *           address of mnb_gemm_noalloc's array (looked up once, under a
 *           lock): calls are reentrant, and concurrent calls on different
 *           streams are safe when they do not share output buffers or a
 *           workspace (mnb_gemm_noalloc calls on one GPU share one).
 *
 * Data layouts (N-major: every column of B is one contiguous run of bytes)
 * ------------------------------------------------------------------------
 *   nb           = ceil(K / block_size)
 *   q (logical)  uint8 [N][K], values 0..15 (bits above the low nibble are
 *                ignored)
 *   B (packed)   uint8 [N][nb][block_size/2].  Value k of column n is in byte
 *                n*nb*(block_size/2) + k/2, low nibble for even k, high
 *                nibble for odd k; nibbles past K in the last, partial block
 *                are written as 0 by mnb_pack and never affect results.
 *   zp (logical) uint8 [N][nb], values 0..15
 *   zp (packed)  uint8 [N][ceil(nb/2)].  Block b of column n is in byte
 *                n*ceil(nb/2) + b/2, low nibble for even b; when absent every
 *                zero point is 8.
 *   scales       [N][nb] in the activation dtype (float32 or bfloat16).
 *   A            [M][K] float32 or bfloat16;  Y [M][N] in the same dtype.
 *   bias         float32 [N], optional, added after the K reduction and
 *                before the output is rounded.
 * bfloat16 values are raw 16-bit patterns; float32 -> bfloat16 output rounding
 * is round-to-nearest-even.
 */
#ifndef MNB_H
#define MNB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mnb_status {
    MNB_OK = 0,
    MNB_E_ARG = -1,          /* null pointer, bad shape, M out of range      */
    MNB_E_UNSUPPORTED = -2,  /* bits != 4, block size, dtype, reserved != 0  */
    MNB_E_ALIGN = -3,        /* a pointer violates its alignment rule        */
    MNB_E_OVERFLOW = -4,     /* a size does not fit the index arithmetic     */
    MNB_E_HIP = -5           /* the HIP runtime reported an error            */
} mnb_status;

typedef enum mnb_dtype { MNB_F32 = 0, MNB_BF16 = 1 } mnb_dtype;

/* The prepared-plan description ("Prepared weight-only plan": logical K and
 * N, block size, signedness and nibble order are fixed by this ABI: unsigned
 * 4-bit, low nibble first). */
typedef struct mnb_desc {
    int64_t K;               /* reduction length, >= 1                        */
    int64_t N;               /* output columns, >= 1                          */
    int32_t bits;            /* must be 4                                     */
    int32_t block_size;      /* 16, 32, 64, 128 or 256                        */
    int32_t act_dtype;       /* mnb_dtype of A, scales and Y                  */
    int32_t has_zero_points; /* 0: every zero point is 8                      */
    int32_t accuracy_level;  /* MatMulNBits attribute; recorded, never lowers
                                the precision of any computation              */
    int32_t reserved;        /* must be 0                                     */
} mnb_desc;

/* Checks `d` (and M >= 1) on the host; no HIP call.  MNB_OK or an error. */
int mnb_validate(const mnb_desc* d, int64_t M);

/* Buffer sizes in bytes for a valid descriptor; 0 when `d` is invalid or a
 * size overflows.  Packed weights: N*nb*block_size/2.  Scales: N*nb*(4 or 2).
 * Packed zero points: N*ceil(nb/2) when has_zero_points, else 0. */
size_t mnb_packed_weight_bytes(const mnb_desc* d);
size_t mnb_scale_bytes(const mnb_desc* d);
size_t mnb_zero_point_bytes(const mnb_desc* d);

/* Largest K that mnb_gemv serves with its register-resident decode kernel
 * for this descriptor's block size; larger K is served, with the same
 * results contract, by mnb_gemm at M = 1 (the tiled prefill kernel). */
int64_t mnb_gemv_max_k(const mnb_desc* d);

/* mnb_pack -- the preparation step ("Prepared weight-only plan": packed
 * constant storage aligned for the kernel; first-use packing time).
 *   q_nk        uint8 [N][K] logical weights (device).
 *   zp_nb       uint8 [N][nb] logical zero points (device); must be NULL iff
 *               d->has_zero_points == 0.
 *   b_packed    out, mnb_packed_weight_bytes(d) bytes, 16-byte aligned.
 *   zp_packed   out, mnb_zero_point_bytes(d) bytes; NULL iff no zero points.
 * Pad nibbles are written as 0.  The call writes every byte of both outputs. */
int mnb_pack(const mnb_desc* d, const uint8_t* q_nk, const uint8_t* zp_nb,
             uint8_t* b_packed, uint8_t* zp_packed, void* stream);

/* mnb_gemv -- decode, M == 1 ("int4_gemv": output columns partitioned so
 * each weight byte is streamed once; unpack in registers; float32
 * accumulation).
 *   a           [1][K] act_dtype, 16-byte aligned.
 *   b_packed    packed weights, 16-byte aligned.
 *   scales      [N][nb] act_dtype, aligned to its element size.
 *   zp_packed   packed zero points or NULL (iff !has_zero_points).
 *   bias        float32 [N] or NULL.
 *   y           [1][N] act_dtype, aligned to its element size.
 * M must be 1 (MNB_E_ARG otherwise) and K at most mnb_gemv_max_k
 * (MNB_E_UNSUPPORTED otherwise; mnb_gemm serves any K).  No workspace.
 * Each product is a * (q - zp) with the
 * exact integer q - zp, so weights equal to their zero points contribute
 * exactly nothing.  For a given (K, block_size) the float32 summation order
 * of a column does not depend on N or on the column's position, so a launch
 * over concatenated weights (fused QKV, gate||up) is bit-identical to
 * separate launches. */
int mnb_gemv(const mnb_desc* d, int64_t M, const void* a,
             const uint8_t* b_packed, const void* scales,
             const uint8_t* zp_packed, const float* bias, void* y,
             void* stream);

/* Bytes of workspace mnb_gemm needs for this descriptor and M (0: none;
 * 0 also for an invalid descriptor or M).  Host-only, no HIP call; a
 * function of the shape alone. */
size_t mnb_workspace_bytes(const mnb_desc* d, int64_t M);

/* mnb_gemm -- prefill, any M >= 1 ("int4_gemm": activation panels and
 * weight blocks reused on chip).  Same arguments as mnb_gemv with A [M][K]
 * and Y [M][N]; `a` and `b_packed` 16-byte aligned (bfloat16 scales of
 * 16-value blocks 4-byte aligned), plus the workspace: at least
 * mnb_workspace_bytes(d, M) bytes, 256-byte aligned (NULL when that is 0).
 * Products run on the bf16 matrix cores with float32 accumulation.
 * bfloat16 activations meet weight tiles unpacked on chip to
 * bf16((q - zp) * s) (one rounding of the exact weight, the bits
 * mnb_dequant's bf16 output gives).  float32 activations are split into two
 * bfloat16 terms (hi + lo) and meet the exact bfloat16 integers (q - zp); the
 * float32 per-block scale is applied to the float32 partial sums, so results
 * stay within float32 tolerance.  Products with too few output tiles to fill
 * the GPU split K across workgroups, keep the float32 partials in the
 * workspace and add them in a fixed order.
 * Short row blocks (page "Qwen3 CPU Inference Critical Path", int4_small_m)
 * unpack every weight once for all rows, with no workspace.  2 <= M <= 4
 * (block_size >= 32, K * element size a multiple of 16; K up to 8192 for
 * two rows and 4096 for three or four with float32 activations, twice that
 * with bfloat16) go through the decode GEMV: each unpacked weight feeds one
 * float32 FMA per row; but N > 32768 (an LM head), where the matrix-core
 * kernel takes the shape, goes there.  Otherwise 1 <= M <= 16 (K % 32 == 0,
 * block_size >= 32) take a matrix-core kernel: the exact integers (q - zp)
 * meet the activations (float32 as bf16 head + tail) and each 32-value
 * partial sum is scaled in float32.  In both, as in mnb_gemv, a column's
 * float32 summation order depends only on K (and the row count class), so
 * concatenated launches are bit-identical to separate ones (at 2 <= M <= 4,
 * launches on the same side of N = 32768). */
int mnb_gemm(const mnb_desc* d, int64_t M, const void* a,
             const uint8_t* b_packed, const void* scales,
             const uint8_t* zp_packed, const float* bias, void* y,
             void* workspace, size_t workspace_bytes, void* stream);

/* mnb_gemm_noalloc -- mnb_gemm for callers that cannot allocate device
 * memory (code under HIP graph capture that must not call hipMalloc, tight
 * serving loops, harnesses that forbid allocation): the same kernels, plan
 * and results as mnb_gemm, but the split-K partials live in a static device
 * array of MNB_NOALLOC_SCRATCH_BYTES inside the library (one per GPU, held
 * from the library's first use on that GPU until the process ends) instead
 * of a caller workspace.  Arguments and validation as for mnb_gemm, without
 * the workspace.  A product needing more than MNB_NOALLOC_SCRATCH_BYTES
 * returns MNB_E_UNSUPPORTED (no current plan does: a K split never holds
 * more than 256 float32 tiles of 256 x 256 = 64 MiB).  The call itself
 * allocates nothing; the first call on a device looks up that device's array
 * (hipGetSymbolAddress).  Every call on one GPU shares its array: calls that
 * may overlap on the device (different streams, graphs replayed beside other
 * work) race on it and must be ordered by the caller. */
#define MNB_NOALLOC_SCRATCH_BYTES (64u << 20)
int mnb_gemm_noalloc(const mnb_desc* d, int64_t M, const void* a,
                     const uint8_t* b_packed, const void* scales,
                     const uint8_t* zp_packed, const float* bias, void* y,
                     void* stream);

/* mnb_dequant -- test hook: writes the dequantized weights w[N][K] (the
 * transposed logical B) so they can be compared bit-for-bit.
 *   out_kind 0: float32, one round-to-nearest-even rounding of (q-zp)*scale;
 *   out_kind 1: bfloat16, one round-to-nearest-even rounding of the exact
 *               (q-zp)*scale;
 *   out_kind 2: int8, the exact integer q - zp (what the prefill kernel
 *               places in its bf16 weight tiles).
 *   w_nk        [N][K] of the chosen type. */
int mnb_dequant(const mnb_desc* d, const uint8_t* b_packed, const void* scales,
                const uint8_t* zp_packed, int32_t out_kind, void* w_nk,
                void* stream);

/* ---- QDQ import ---------------------------------------------------------------
 * mnb_import_qdq -- normalizes a weight in the blocked UINT4 DequantizeLinear
 * encoding into the storage above (page "Qwen3 CPU Inference Critical Path",
 * "Export contract", qwen3-int4-qdq: a projection is a logical UINT4[K,N]
 * in row-major, low-nibble-first storage, blocked along axis 0; the tied
 * embedding / LM-head weight is a logical UINT4[vocabulary,hidden] blocked
 * along axis 1; another layout is normalized before it is matched).  A
 * one-time preparation step, like mnb_pack.
 *   axis        0: W is [K][N] (the MatMul B), scales and zero points [nb][N];
 *               1: W is [N][K] (N = vocabulary, K = hidden), scales and zero
 *                  points [N][nb].  nb = ceil(K / block_size).
 *   w_q         ceil(K*N/2) bytes: W's elements in row-major order, element i
 *               in byte i/2, the low nibble when i is even.
 *   scales_q    nb*N elements of act_dtype in the axis's shape.
 *   zp_q        ceil(nb*N/2) bytes packed like w_q, or NULL: DequantizeLinear
 *               then uses zero point 0 (not the MatMulNBits default 8), which
 *               is written to zp_packed explicitly.
 *   b_packed, scales, zp_packed   outputs in the storage above (sizes from the
 *               mnb_*_bytes queries; b_packed 16-byte aligned).
 * d->has_zero_points must be 1 (the result always carries zero points).
 * Inputs and outputs must not overlap (MNB_E_ARG).  All device pointers. */
int mnb_import_qdq(const mnb_desc* d, int32_t axis, const uint8_t* w_q,
                   const void* scales_q, const uint8_t* zp_q,
                   uint8_t* b_packed, void* scales, uint8_t* zp_packed,
                   void* stream);

/* Nonzero when an axis-1 QDQ weight with zero points already is the storage
 * above byte for byte (K % block_size == 0 and an even number of blocks per
 * row): then w_q, scales_q and zp_q serve every entry point as they are, and
 * the tied embedding and LM head share one copy ("initializer aliasing": no
 * duplicated weight).  Host-only; 0 for an invalid descriptor. */
int mnb_qdq_is_native(const mnb_desc* d, int32_t axis);

/* ---- tied embedding and the LM head -------------------------------------------
 * mnb_gather_rows -- the embedding lookup on the tied weight (same page,
 * "Export contract" and "Operator priority", Gather: dequantize only the
 * selected rows of the tied quantized initializer).  With N = vocabulary and
 * K = hidden, embedding row v is column v of B:
 *   out[t][k] = (q[v][k] - zp[v][k / bs]) * s[v][k / bs],  v = ids[t],
 * rounded once to act_dtype exactly like mnb_dequant (out_kind 0 for float32,
 * 1 for bfloat16).  ids: int64 [n_ids] (device, 8-byte aligned); a negative
 * id counts from the end (ids in [-N, N)); a row whose id lies outside that
 * range is written as NaN and reads no weight.  out: [n_ids][K] act_dtype.
 * n_ids == 0 does nothing. */
int mnb_gather_rows(const mnb_desc* d, const int64_t* ids, int64_t n_ids,
                    const uint8_t* b_packed, const void* scales,
                    const uint8_t* zp_packed, void* out, void* stream);

/* Bytes of workspace mnb_argmax needs for M rows of N values (0: none, or
 * invalid sizes).  Host-only. */
size_t mnb_argmax_workspace_bytes(int64_t M, int64_t N);

/* mnb_argmax -- greedy ArgMax per row (same page, "Phase Q5: scheduling and
 * fusion": the final RMSNorm, LM-head GEMV and greedy ArgMax chain):
 * idx[m] = the first n holding the largest x[m][n]; a NaN counts as larger
 * than every number, so the first NaN wins.  x: [M][N] float32 or bfloat16
 * (dtype, an mnb_dtype); idx: int64 [M].  Rows longer than 2048 values (and
 * at most 65,535 rows) are split over up to 256 workgroups whose partial
 * maxima go to the workspace (at least mnb_argmax_workspace_bytes(M, N),
 * 256-byte aligned; NULL when that is 0) and are then reduced per row;
 * otherwise one workgroup takes a row.  Comparisons use a total order on
 * (value, index), so the answer does not depend on the split. */
int mnb_argmax(int32_t dtype, int64_t M, int64_t N, const void* x,
               int64_t* idx, void* workspace, size_t workspace_bytes,
               void* stream);

/* ---- gated MLP epilogue --------------------------------------------------------
 * mnb_gemv_silu_mul -- the fused gate||up decode projection (same page,
 * "Operator priority": the SiLU-gated MLP, Sigmoid(x) * x times the up
 * projection; "Phase Q5: scheduling and fusion": the gate projection, its
 * SiLU and the gate/up product as one fusion).
 * B holds N = 2I columns, gate columns 0..I-1 then the matching up columns
 * I..2I-1 (one concatenated weight, as for the unfused fused-N launch);
 * bias, when given, has N entries.  With y = a x dequant(B) + bias:
 *   h[i] = silu(y[i]) * y[I + i],  silu(x) = x / (1 + exp(-x)),
 * evaluated in float32 on y before any rounding, then stored in act_dtype
 * (RTNE for bfloat16).  y[i] and y[I + i] are summed exactly as mnb_gemv
 * sums those columns (the same lane geometry, split-K wavefront teams
 * included).  M must be 1, N even and K at most mnb_gemv_max_k
 * (MNB_E_UNSUPPORTED otherwise); h: [1][I]. */
int mnb_gemv_silu_mul(const mnb_desc* d, int64_t M, const void* a,
                      const uint8_t* b_packed, const void* scales,
                      const uint8_t* zp_packed, const float* bias, void* h,
                      void* stream);

/* mnb_gemm_silu_mul -- the gated gate||up projection for any M (same page
 * and passage as mnb_gemv_silu_mul; "INT4 MatMul is first", int4_gemm for
 * prompt prefill).  B, bias and h as for mnb_gemv_silu_mul with A [M][K] and
 * h [M][I], I = N / 2; plus a workspace of at least
 * mnb_gemm_silu_workspace_bytes(d, M) bytes (256-byte aligned; NULL when
 * that is 0).  Routes, by shape alone:
 *   M == 1, K <= mnb_gemv_max_k: mnb_gemv_silu_mul (no workspace);
 *   bfloat16, M > 128, K a multiple of 64 and of block_size: the prefill
 *     kernel with the gated product in its epilogue -- each tile pairs 128
 *     gate columns with the matching up columns, h is evaluated in float32 on
 *     the unrounded sums and rounded once (only h [M][I] is written);
 *   otherwise the unfused standard graph ("Phase Q5": each unfused graph
 *     remains a correctness fallback): y = mnb_gemm into the workspace, then
 *     h = silu(y_gate) * y_up in float32 on y rounded to act_dtype.
 * N must be even (MNB_E_ARG otherwise). */
size_t mnb_gemm_silu_workspace_bytes(const mnb_desc* d, int64_t M);
int mnb_gemm_silu_mul(const mnb_desc* d, int64_t M, const void* a,
                      const uint8_t* b_packed, const void* scales,
                      const uint8_t* zp_packed, const float* bias, void* h,
                      void* workspace, size_t workspace_bytes, void* stream);

/* ---- RMSNorm into the projection input ------------------------------------------
 * mnb_gemv_rmsnorm -- the decode projection of an RMS-normalized row (same
 * page, "Phase Q5: scheduling and fusion": RMSNorm fused into the packed
 * projection input; "Phase Q2": SimplifiedLayerNormalization lowered to the
 * RMSNormalization engine):
 *   a[k] = x[k] / sqrt(sum_k x[k]^2 / K + epsilon) * gamma[k],
 *   y = a x dequant(B) (+ bias),
 * the normalization computed by every workgroup from the staged row in
 * float32 (fixed summation order) and applied as the row enters registers, so
 * the normalized row never goes to memory.  x: [1][K] and gamma: [K] in
 * act_dtype, both 16-byte aligned; epsilon finite and >= 0.  M must be 1 and
 * K * element size a multiple of 16 with K * element size * 2 <= 64 KiB
 * (MNB_E_UNSUPPORTED otherwise); the other arguments as for mnb_gemv. */
int mnb_gemv_rmsnorm(const mnb_desc* d, int64_t M, const void* x,
                     const void* gamma, float epsilon,
                     const uint8_t* b_packed, const void* scales,
                     const uint8_t* zp_packed, const float* bias, void* y,
                     void* stream);

/* ---- decode-step driver ------------------------------------------------------
 * One projection of a step: mnb_gemv when M == 1 and K <= mnb_gemv_max_k,
 * mnb_gemm otherwise.  A fused QKV or gate||up projection is one entry whose
 * weights are concatenated along N.  (Page "Qwen3 CPU Inference Critical
 * Path", "Phase Q1": the plan-owned packed weights serve every token; the
 * decode GEMV and the prefill GEMM are the two algorithms of "INT4 MatMul is
 * first".) */
typedef struct mnb_matmul_args {
    mnb_desc desc;
    int64_t M;
    const void* a;
    const uint8_t* b_packed;
    const void* scales;
    const uint8_t* zp_packed;
    const float* bias;
    void* y;
} mnb_matmul_args;

/* Workspace bytes a sequence needs: the largest any entry needs (its
 * entries run in order on one stream and share it).  0 when none is needed
 * or an entry is invalid.  Host-only. */
size_t mnb_sequence_workspace_bytes(const mnb_matmul_args* ops, int64_t n_ops);

/* Validates every entry and the workspace first (nothing is launched if one
 * is invalid; the error detail names the entry), then enqueues them in order
 * on `stream`. */
int mnb_matmul_sequence(const mnb_matmul_args* ops, int64_t n_ops,
                        void* workspace, size_t workspace_bytes,
                        void* stream);

/* A captured HIP graph of a sequence, replayed with one launch.  The handle
 * records the pointers in `ops` and the workspace; the caller keeps those
 * buffers alive until mnb_graph_destroy, and does not use that workspace
 * for other work that may run while a replay does.  Creation captures on a
 * private stream of default priority and launches nothing on the device. */
typedef struct mnb_graph mnb_graph;
int mnb_graph_create(const mnb_matmul_args* ops, int64_t n_ops,
                     void* workspace, size_t workspace_bytes,
                     mnb_graph** out);
int mnb_graph_launch(mnb_graph* g, void* stream);
int mnb_graph_destroy(mnb_graph* g);

/* ---- persistent decode step ---------------------------------------------------
 * A decode step (every entry M == 1) as ONE cooperative launch that stays
 * resident for the whole step: one workgroup per compute unit, each of whose
 * compute wavefronts requests the next entry's packed weights before it waits
 * for the previous entry to finish.  (Page "Qwen3 CPU Inference Critical
 * Path", "Phase Q5: scheduling and fusion": the step is a chain of
 * projections whose only dependence is the activation row; "INT4 MatMul is
 * first": batch-1 projections are bound by the weight stream.)
 *
 * Ordering.  Entry i + 1 reads its activation row only after EVERY
 * workgroup has written its part of entry i's y (write-through stores,
 * acknowledged before a device-wide arrival counter is raised), so an entry
 * whose input `a` is an earlier entry's `y` sees that output.  The outputs
 * are those of mnb_gemv: every column has the same float32 bits (same
 * geometry, loads and summation order).
 *
 * Supported entries: M == 1, one activation type for all entries, block_size
 * >= 32, K * element size a multiple of 16, a K whose decode-GEMV geometry
 * keeps each column in one wavefront (at most 10,240; the few K below that
 * for which split-K teams sum more efficiently are refused), and at most
 * 4,096 outputs per workgroup and entry (N up to about a million columns on
 * 256 compute units).  Others
 * return MNB_E_UNSUPPORTED naming the entry; use mnb_matmul_sequence or
 * mnb_graph_* for them.
 *
 * Workspace.  mnb_step_workspace_bytes(ops, n) bytes (a function of n alone;
 * 0 if an entry is invalid or unsupported), 256-byte aligned, owned by the
 * caller, not overlapping any y: it holds the arrival counters and the entry
 * table.  mnb_step_create validates everything, then (synchronously, with
 * hipMemset / hipMemcpy on the current device) writes the table for the
 * current device's compute-unit count; the workspace must stay untouched and
 * alive until mnb_step_destroy.  The handle records the entries' pointers.
 * Launches that may overlap on the device must not share a step.
 *
 * mnb_step_launch enqueues one cooperative launch on `stream` (the device
 * current at creation must be current).  mnb_step_check synchronizes the
 * stream and reports whether any launch since the last check stopped waiting
 * for the other workgroups (a bounded wait ran out: the grid was not
 * co-resident); that launch's outputs are then undefined and the call
 * returns MNB_E_HIP.  Every wait is bounded, so a launch always completes. */
typedef struct mnb_step mnb_step;
size_t mnb_step_workspace_bytes(const mnb_matmul_args* ops, int64_t n_ops);
int mnb_step_create(const mnb_matmul_args* ops, int64_t n_ops,
                    void* workspace, size_t workspace_bytes, mnb_step** out);
int mnb_step_launch(mnb_step* step, void* stream);
int mnb_step_check(mnb_step* step, void* stream);
int mnb_step_destroy(mnb_step* step);

/* Phase timestamps of later launches, for profiling (page "Qwen3 CPU
 * Inference Critical Path", "INT4 MatMul is first": the kernel corpus reports
 * where the time of a matmul goes).  `trace` is device memory of at least
 * mnb_step_trace_bytes(step) bytes (8-byte aligned; NULL turns tracing off),
 * owned by the caller and overwritten by every launch: uint64 values
 * [workgroup][entry][5] of the 100 MHz s_memrealtime counter, taken by each
 * workgroup's control wavefront before it waits for entry i - 1, after that
 * wait, with entry i's activation row staged, with the workgroup's sums of
 * entry i complete, and with its outputs of entry i acknowledged.
 * mnb_step_trace_bytes returns 0 for NULL; mnb_step_set_trace returns
 * MNB_E_ARG for a short buffer, MNB_E_ALIGN for a misaligned one. */
size_t mnb_step_trace_bytes(const mnb_step* step);
int mnb_step_set_trace(mnb_step* step, void* trace, size_t trace_bytes);

/* Text for a status code (static storage). */
const char* mnb_status_string(int status);
/* Detail of the most recent error on the calling thread ("" if none). */
const char* mnb_last_error(void);
/* Library version string. */
const char* mnb_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MNB_H */
