// The C ABI of libmnb (declared and documented in include/mnb.h): host-side
// validation, derived sizes, dispatch to the kernels, the step driver and
// captured graphs.  Validation runs before any HIP call.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <new>
#include <vector>

#include "mnb_internal.h"

#define MNB_VERSION_STRING "mnb 0.1 (gfx950)"

namespace mnb {

static thread_local char g_last_error[512];

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return status;
}

namespace {

constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;   // K, N: int32 block math
constexpr int64_t kMaxM = int64_t(65535) * 128;       // grid.y of the GEMM

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int check_desc(const mnb_desc* d, const char* who) {
    if (!d) return fail(MNB_E_ARG, "%s: descriptor is NULL", who);
    if (d->bits != 4) return fail(MNB_E_UNSUPPORTED, "%s: bits=%d, only 4 is supported", who, d->bits);
    const int bs = d->block_size;
    if (bs != 16 && bs != 32 && bs != 64 && bs != 128 && bs != 256)
        return fail(MNB_E_UNSUPPORTED, "%s: block_size=%d, must be 16, 32, 64, 128 or 256", who, bs);
    if (d->act_dtype != MNB_F32 && d->act_dtype != MNB_BF16)
        return fail(MNB_E_UNSUPPORTED, "%s: act_dtype=%d unknown", who, d->act_dtype);
    if (d->has_zero_points != 0 && d->has_zero_points != 1)
        return fail(MNB_E_ARG, "%s: has_zero_points=%d, must be 0 or 1", who, d->has_zero_points);
    if (d->accuracy_level < 0 || d->accuracy_level > 4)
        return fail(MNB_E_ARG, "%s: accuracy_level=%d, must be 0..4", who, d->accuracy_level);
    if (d->reserved != 0) return fail(MNB_E_UNSUPPORTED, "%s: reserved field must be 0", who);
    if (d->K < 1 || d->N < 1)
        return fail(MNB_E_ARG, "%s: K=%lld N=%lld, both must be >= 1", who, (long long)d->K, (long long)d->N);
    if (d->K > kMaxDim || d->N > kMaxDim)
        return fail(MNB_E_OVERFLOW, "%s: K=%lld N=%lld exceed 2^31-1", who, (long long)d->K, (long long)d->N);
    return MNB_OK;
}

void fill_problem(const mnb_desc* d, int64_t M, Problem* p) {
    p->M = M;
    p->K = d->K;
    p->N = d->N;
    p->bs = d->block_size;
    p->nb = (int)((d->K + d->block_size - 1) / d->block_size);
    p->col_bytes = (int64_t)p->nb * (d->block_size / 2);
    p->zp_row = (p->nb + 1) / 2;
    p->bf16 = d->act_dtype == MNB_BF16;
    p->has_zp = d->has_zero_points != 0;
}

// Shared validation of gemv / gemm arguments.
int check_matmul(const char* who, const mnb_desc* d, int64_t M, const void* a,
                 const uint8_t* b, const void* scales, const uint8_t* zp,
                 const float* bias, void* y, bool gemv, Problem* p) {
    int st = check_desc(d, who);
    if (st != MNB_OK) return st;
    if (gemv && M != 1) return fail(MNB_E_ARG, "%s: M=%lld, the decode GEMV takes M == 1", who, (long long)M);
    if (M < 1) return fail(MNB_E_ARG, "%s: M=%lld, must be >= 1", who, (long long)M);
    if (M > kMaxM) return fail(MNB_E_OVERFLOW, "%s: M=%lld exceeds %lld", who, (long long)M, (long long)kMaxM);
    if (!a || !b || !scales || !y) return fail(MNB_E_ARG, "%s: a, b_packed, scales and y must be non-NULL", who);
    if ((zp != nullptr) != (d->has_zero_points != 0))
        return fail(MNB_E_ARG, "%s: zp_packed must be given iff has_zero_points", who);
    const uintptr_t esz = d->act_dtype == MNB_BF16 ? 2 : 4;
    if (!aligned(a, 16)) return fail(MNB_E_ALIGN, "%s: a must be 16-byte aligned", who);
    if (!aligned(b, 16)) return fail(MNB_E_ALIGN, "%s: b_packed must be 16-byte aligned", who);
    if (!aligned(scales, esz)) return fail(MNB_E_ALIGN, "%s: scales must be %d-byte aligned", who, (int)esz);
    if (!aligned(y, esz)) return fail(MNB_E_ALIGN, "%s: y must be %d-byte aligned", who, (int)esz);
    if (bias && !aligned(bias, 4)) return fail(MNB_E_ALIGN, "%s: bias must be 4-byte aligned", who);
    // the prefill kernel reads the two bfloat16 scales of a 16-value block
    // pair as one 32-bit word
    if (!gemv && esz == 2 && d->block_size == 16 && !aligned(scales, 4))
        return fail(MNB_E_ALIGN, "%s: bfloat16 scales of 16-value blocks must be 4-byte aligned", who);
    fill_problem(d, M, p);
    p->a = a; p->b = b; p->scales = scales; p->zp = zp; p->bias = bias; p->y = y;
    return MNB_OK;
}

bool takes_gemv(const Problem& p) { return p.M == 1 && p.K <= gemv_max_k(p.bs); }

size_t workspace_of(const Problem& p) { return takes_gemv(p) ? 0 : gemm_workspace_bytes(p); }

// The caller's workspace must hold what the product's plan needs: a split
// never changes with the workspace offered, so results depend on the shape
// alone.
int check_workspace(const char* who, size_t need, const void* ws, size_t ws_bytes) {
    if (need == 0) return MNB_OK;
    if (!ws || ws_bytes < need)
        return fail(MNB_E_ARG, "%s: needs a workspace of %zu bytes (given %zu%s)", who, need,
                    ws ? ws_bytes : (size_t)0, ws ? "" : ", NULL");
    if (!aligned(ws, 256)) return fail(MNB_E_ALIGN, "%s: workspace must be 256-byte aligned", who);
    return MNB_OK;
}

int run(const Problem& p, hipStream_t s, void* ws, size_t ws_bytes) {
    if (takes_gemv(p)) return launch_gemv(p, s);
    return launch_gemm(p, s, ws, ws_bytes);
}

}  // namespace
}  // namespace mnb

using namespace mnb;

// ---- the workspace of mnb_gemm_noalloc ---------------------------------------
// A file-scope device array: each GPU the library runs on holds its own copy
// from module load until the process ends.  Host code never passes its name to
// a kernel (on the host it is only a stand-in for the symbol): its device
// address is looked up once per device with hipGetSymbolAddress and that
// pointer is what the kernels get.
static __device__ __align__(256) unsigned char scratch[MNB_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];      // device address of `scratch`, per device

// The current device's copy of `scratch`; looked up on the first call on
// that device (the device is current), then cached.
int scratch_for_current_device(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(MNB_E_HIP, "mnb_gemm_noalloc: hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(MNB_E_UNSUPPORTED, "mnb_gemm_noalloc: device %d", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(MNB_E_HIP, "mnb_gemm_noalloc: hipGetSymbolAddress(scratch) on device %d: %s", dev,
                        hipGetErrorString(e));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return MNB_OK;
}

}  // namespace

struct mnb_graph {
    hipGraph_t graph;
    hipGraphExec_t exec;
};

struct mnb_step {
    int device;         // the device the table was written for
    int grid;           // workgroups (one per CU of that device)
    bool bf16;
    int64_t n_ops;
    void* workspace;    // the caller's: counters and the entry table
    void* trace;        // the caller's phase-timestamp buffer, or NULL
};

extern "C" {

int mnb_validate(const mnb_desc* d, int64_t M) {
    int st = check_desc(d, "mnb_validate");
    if (st != MNB_OK) return st;
    if (M < 1) return fail(MNB_E_ARG, "mnb_validate: M=%lld, must be >= 1", (long long)M);
    if (M > kMaxM) return fail(MNB_E_OVERFLOW, "mnb_validate: M=%lld too large", (long long)M);
    return MNB_OK;
}

size_t mnb_packed_weight_bytes(const mnb_desc* d) {
    if (check_desc(d, "mnb_packed_weight_bytes") != MNB_OK) return 0;
    Problem p;
    fill_problem(d, 1, &p);
    return (size_t)(p.N * p.col_bytes);
}

size_t mnb_scale_bytes(const mnb_desc* d) {
    if (check_desc(d, "mnb_scale_bytes") != MNB_OK) return 0;
    Problem p;
    fill_problem(d, 1, &p);
    return (size_t)(p.N * p.nb * (p.bf16 ? 2 : 4));
}

size_t mnb_zero_point_bytes(const mnb_desc* d) {
    if (check_desc(d, "mnb_zero_point_bytes") != MNB_OK) return 0;
    if (!d->has_zero_points) return 0;
    Problem p;
    fill_problem(d, 1, &p);
    return (size_t)(p.N * p.zp_row);
}

int64_t mnb_gemv_max_k(const mnb_desc* d) {
    if (check_desc(d, "mnb_gemv_max_k") != MNB_OK) return 0;
    return gemv_max_k(d->block_size);
}

int mnb_pack(const mnb_desc* d, const uint8_t* q_nk, const uint8_t* zp_nb,
             uint8_t* b_packed, uint8_t* zp_packed, void* stream) {
    int st = check_desc(d, "mnb_pack");
    if (st != MNB_OK) return st;
    if (!q_nk || !b_packed) return fail(MNB_E_ARG, "mnb_pack: q_nk and b_packed must be non-NULL");
    const bool zp = d->has_zero_points != 0;
    if ((zp_nb != nullptr) != zp || (zp_packed != nullptr) != zp)
        return fail(MNB_E_ARG, "mnb_pack: zp_nb and zp_packed must be given iff has_zero_points");
    if (!aligned(b_packed, 16)) return fail(MNB_E_ALIGN, "mnb_pack: b_packed must be 16-byte aligned");
    return launch_pack(d->K, d->N, d->block_size, q_nk, zp_nb, b_packed, zp_packed,
                       static_cast<hipStream_t>(stream));
}

int mnb_gemv(const mnb_desc* d, int64_t M, const void* a, const uint8_t* b_packed,
             const void* scales, const uint8_t* zp_packed, const float* bias, void* y,
             void* stream) {
    Problem p;
    int st = check_matmul("mnb_gemv", d, M, a, b_packed, scales, zp_packed, bias, y, true, &p);
    if (st != MNB_OK) return st;
    if (!takes_gemv(p))
        return fail(MNB_E_UNSUPPORTED, "mnb_gemv: K=%lld exceeds mnb_gemv_max_k=%lld (use mnb_gemm)",
                    (long long)p.K, (long long)gemv_max_k(p.bs));
    return launch_gemv(p, static_cast<hipStream_t>(stream));
}

size_t mnb_workspace_bytes(const mnb_desc* d, int64_t M) {
    if (mnb_validate(d, M) != MNB_OK) return 0;
    // the choice of kernel depends on the shape alone (A's 16-byte alignment
    // is a precondition of every product)
    Problem p;
    fill_problem(d, M, &p);
    p.a = nullptr; p.b = nullptr; p.scales = nullptr; p.zp = nullptr; p.bias = nullptr; p.y = nullptr;
    return gemm_workspace_bytes(p);
}

int mnb_gemm(const mnb_desc* d, int64_t M, const void* a, const uint8_t* b_packed,
             const void* scales, const uint8_t* zp_packed, const float* bias, void* y,
             void* workspace, size_t workspace_bytes, void* stream) {
    Problem p;
    int st = check_matmul("mnb_gemm", d, M, a, b_packed, scales, zp_packed, bias, y, false, &p);
    if (st != MNB_OK) return st;
    st = check_workspace("mnb_gemm", gemm_workspace_bytes(p), workspace, workspace_bytes);
    if (st != MNB_OK) return st;
    return launch_gemm(p, static_cast<hipStream_t>(stream), workspace, workspace_bytes);
}

int mnb_gemm_noalloc(const mnb_desc* d, int64_t M, const void* a, const uint8_t* b_packed,
                     const void* scales, const uint8_t* zp_packed, const float* bias, void* y,
                     void* stream) {
    Problem p;
    int st = check_matmul("mnb_gemm_noalloc", d, M, a, b_packed, scales, zp_packed, bias, y, false, &p);
    if (st != MNB_OK) return st;
    const size_t need = gemm_workspace_bytes(p);
    if (need > (size_t)MNB_NOALLOC_SCRATCH_BYTES)
        return fail(MNB_E_UNSUPPORTED,
                    "mnb_gemm_noalloc: this product needs %zu bytes of workspace, beyond the %u-byte static "
                    "scratch (use mnb_gemm with a caller workspace)", need, (unsigned)MNB_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    st = scratch_for_current_device(&ws);
    if (st != MNB_OK) return st;
    // the split partials are written in full before they are read: nothing in
    // the scratch needs clearing between calls
    return launch_gemm(p, static_cast<hipStream_t>(stream), ws, (size_t)MNB_NOALLOC_SCRATCH_BYTES);
}

int mnb_dequant(const mnb_desc* d, const uint8_t* b_packed, const void* scales,
                const uint8_t* zp_packed, int32_t out_kind, void* w_nk, void* stream) {
    int st = check_desc(d, "mnb_dequant");
    if (st != MNB_OK) return st;
    if (out_kind < 0 || out_kind > 2) return fail(MNB_E_ARG, "mnb_dequant: out_kind=%d, must be 0, 1 or 2", out_kind);
    if (!b_packed || !w_nk || (out_kind != 2 && !scales))
        return fail(MNB_E_ARG, "mnb_dequant: b_packed, w_nk (and scales unless out_kind 2) must be non-NULL");
    if ((zp_packed != nullptr) != (d->has_zero_points != 0))
        return fail(MNB_E_ARG, "mnb_dequant: zp_packed must be given iff has_zero_points");
    const uintptr_t esz = d->act_dtype == MNB_BF16 ? 2 : 4;
    if (scales && !aligned(scales, esz)) return fail(MNB_E_ALIGN, "mnb_dequant: scales misaligned");
    const uintptr_t osz = out_kind == 0 ? 4 : out_kind == 1 ? 2 : 1;
    if (!aligned(w_nk, osz)) return fail(MNB_E_ALIGN, "mnb_dequant: w_nk misaligned");
    Problem p;
    fill_problem(d, 1, &p);
    p.a = nullptr; p.b = b_packed; p.scales = scales; p.zp = zp_packed; p.bias = nullptr; p.y = nullptr;
    return launch_dequant(p, out_kind, w_nk, static_cast<hipStream_t>(stream));
}

namespace {

// [p, p + n) and [q, q + m) share a byte
bool overlap(const void* p, size_t n, const void* q, size_t m) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
    return n && m && a < b + m && b < a + n;
}

}  // namespace

int mnb_import_qdq(const mnb_desc* d, int32_t axis, const uint8_t* w_q, const void* scales_q,
                   const uint8_t* zp_q, uint8_t* b_packed, void* scales, uint8_t* zp_packed,
                   void* stream) {
    int st = check_desc(d, "mnb_import_qdq");
    if (st != MNB_OK) return st;
    if (axis != 0 && axis != 1) return fail(MNB_E_ARG, "mnb_import_qdq: axis=%d, must be 0 or 1", axis);
    if (!d->has_zero_points)
        return fail(MNB_E_ARG, "mnb_import_qdq: has_zero_points must be 1 (the normalized weight always "
                               "carries zero points; a missing QDQ zero point means 0)");
    if (!w_q || !scales_q || !b_packed || !scales || !zp_packed)
        return fail(MNB_E_ARG, "mnb_import_qdq: w_q, scales_q, b_packed, scales and zp_packed must be non-NULL");
    const uintptr_t esz = d->act_dtype == MNB_BF16 ? 2 : 4;
    if (!aligned(b_packed, 16)) return fail(MNB_E_ALIGN, "mnb_import_qdq: b_packed must be 16-byte aligned");
    if (!aligned(scales_q, esz) || !aligned(scales, esz))
        return fail(MNB_E_ALIGN, "mnb_import_qdq: scales_q and scales must be %d-byte aligned", (int)esz);
    Problem p;
    fill_problem(d, 1, &p);
    const size_t wq_bytes = (size_t)((d->K * d->N + 1) / 2), zq_bytes = (size_t)((p.nb * d->N + 1) / 2);
    const size_t s_bytes = (size_t)(p.nb * d->N) * esz, b_bytes = (size_t)(d->N * p.col_bytes),
                 z_bytes = (size_t)(d->N * p.zp_row);
    const void* ins[3] = {w_q, scales_q, zp_q};
    const size_t in_sz[3] = {wq_bytes, s_bytes, zp_q ? zq_bytes : 0};
    const void* outs[3] = {b_packed, scales, zp_packed};
    const size_t out_sz[3] = {b_bytes, s_bytes, z_bytes};
    for (int i = 0; i < 3; i++)
        for (int j = 0; j < 3; j++)
            if (overlap(ins[i], in_sz[i], outs[j], out_sz[j]) || (i < j && overlap(outs[i], out_sz[i], outs[j], out_sz[j])))
                return fail(MNB_E_ARG, "mnb_import_qdq: inputs and outputs must not overlap");
    p.has_zp = true;
    return launch_import_qdq(p, axis, w_q, scales_q, zp_q, b_packed, scales, zp_packed,
                             static_cast<hipStream_t>(stream));
}

int mnb_qdq_is_native(const mnb_desc* d, int32_t axis) {
    if (check_desc(d, "mnb_qdq_is_native") != MNB_OK) return 0;
    const int64_t nb = (d->K + d->block_size - 1) / d->block_size;
    return axis == 1 && d->has_zero_points && d->K % d->block_size == 0 && nb % 2 == 0;
}

int mnb_gather_rows(const mnb_desc* d, const int64_t* ids, int64_t n_ids, const uint8_t* b_packed,
                    const void* scales, const uint8_t* zp_packed, void* out, void* stream) {
    int st = check_desc(d, "mnb_gather_rows");
    if (st != MNB_OK) return st;
    if (n_ids < 0) return fail(MNB_E_ARG, "mnb_gather_rows: n_ids=%lld < 0", (long long)n_ids);
    if (n_ids == 0) return MNB_OK;
    if (!ids || !b_packed || !scales || !out)
        return fail(MNB_E_ARG, "mnb_gather_rows: ids, b_packed, scales and out must be non-NULL");
    if ((zp_packed != nullptr) != (d->has_zero_points != 0))
        return fail(MNB_E_ARG, "mnb_gather_rows: zp_packed must be given iff has_zero_points");
    const uintptr_t esz = d->act_dtype == MNB_BF16 ? 2 : 4;
    if (!aligned(ids, 8)) return fail(MNB_E_ALIGN, "mnb_gather_rows: ids must be 8-byte aligned");
    if (!aligned(scales, esz) || !aligned(out, esz))
        return fail(MNB_E_ALIGN, "mnb_gather_rows: scales and out must be %d-byte aligned", (int)esz);
    if (n_ids > (int64_t(1) << 40) / d->K)
        return fail(MNB_E_OVERFLOW, "mnb_gather_rows: n_ids * K too large");
    Problem p;
    fill_problem(d, 1, &p);
    p.a = nullptr; p.b = b_packed; p.scales = scales; p.zp = zp_packed; p.bias = nullptr; p.y = nullptr;
    return launch_gather_rows(p, ids, n_ids, out, static_cast<hipStream_t>(stream));
}

size_t mnb_argmax_workspace_bytes(int64_t M, int64_t N) {
    if (M < 1 || N < 1 || M > kMaxDim) return 0;
    return argmax_workspace_bytes(M, N);
}

int mnb_argmax(int32_t dtype, int64_t M, int64_t N, const void* x, int64_t* idx, void* workspace,
               size_t workspace_bytes, void* stream) {
    if (dtype != MNB_F32 && dtype != MNB_BF16) return fail(MNB_E_UNSUPPORTED, "mnb_argmax: dtype=%d unknown", dtype);
    if (M < 1 || N < 1) return fail(MNB_E_ARG, "mnb_argmax: M=%lld N=%lld, both must be >= 1", (long long)M, (long long)N);
    if (M > kMaxDim) return fail(MNB_E_OVERFLOW, "mnb_argmax: M=%lld exceeds 2^31-1", (long long)M);
    if (!x || !idx) return fail(MNB_E_ARG, "mnb_argmax: x and idx must be non-NULL");
    if (!aligned(x, dtype == MNB_BF16 ? 2 : 4) || !aligned(idx, 8))
        return fail(MNB_E_ALIGN, "mnb_argmax: x or idx misaligned");
    int st = check_workspace("mnb_argmax", argmax_workspace_bytes(M, N), workspace, workspace_bytes);
    if (st != MNB_OK) return st;
    return launch_argmax(dtype == MNB_BF16, M, N, x, idx, static_cast<hipStream_t>(stream), workspace,
                         workspace_bytes);
}

int mnb_gemv_silu_mul(const mnb_desc* d, int64_t M, const void* a, const uint8_t* b_packed,
                      const void* scales, const uint8_t* zp_packed, const float* bias, void* h,
                      void* stream) {
    Problem p;
    int st = check_matmul("mnb_gemv_silu_mul", d, M, a, b_packed, scales, zp_packed, bias, h, true, &p);
    if (st != MNB_OK) return st;
    if (d->N % 2 != 0)
        return fail(MNB_E_ARG, "mnb_gemv_silu_mul: N=%lld must be even (gate half, then up half)", (long long)d->N);
    if (!takes_gemv(p))
        return fail(MNB_E_UNSUPPORTED, "mnb_gemv_silu_mul: K=%lld beyond the decode kernel", (long long)d->K);
    return launch_gemv_silu(p, static_cast<hipStream_t>(stream));
}

int mnb_gemv_rmsnorm(const mnb_desc* d, int64_t M, const void* x, const void* gamma, float epsilon,
                     const uint8_t* b_packed, const void* scales, const uint8_t* zp_packed, const float* bias,
                     void* y, void* stream) {
    Problem p;
    int st = check_matmul("mnb_gemv_rmsnorm", d, M, x, b_packed, scales, zp_packed, bias, y, true, &p);
    if (st != MNB_OK) return st;
    if (!gamma) return fail(MNB_E_ARG, "mnb_gemv_rmsnorm: gamma must be non-NULL");
    if (!aligned(gamma, 16)) return fail(MNB_E_ALIGN, "mnb_gemv_rmsnorm: gamma must be 16-byte aligned");
    if (!(epsilon >= 0.f) || epsilon > 3.0e38f)
        return fail(MNB_E_ARG, "mnb_gemv_rmsnorm: epsilon must be finite and >= 0");
    const int esz = d->act_dtype == MNB_BF16 ? 2 : 4;
    if ((d->K * esz) % 16 != 0)
        return fail(MNB_E_UNSUPPORTED, "mnb_gemv_rmsnorm: K * element size must be a multiple of 16");
    if (!takes_gemv(p))
        return fail(MNB_E_UNSUPPORTED, "mnb_gemv_rmsnorm: K=%lld exceeds mnb_gemv_max_k=%lld", (long long)p.K,
                    (long long)gemv_max_k(p.bs));
    return launch_gemv_rmsnorm(p, gamma, epsilon, static_cast<hipStream_t>(stream));
}

size_t mnb_gemm_silu_workspace_bytes(const mnb_desc* d, int64_t M) {
    if (mnb_validate(d, M) != MNB_OK || d->N % 2 != 0) return 0;
    Problem p;
    fill_problem(d, M, &p);
    p.a = nullptr; p.b = nullptr; p.scales = nullptr; p.zp = nullptr; p.bias = nullptr; p.y = nullptr;
    return gemm_silu_workspace_bytes(p);
}

int mnb_gemm_silu_mul(const mnb_desc* d, int64_t M, const void* a, const uint8_t* b_packed,
                      const void* scales, const uint8_t* zp_packed, const float* bias, void* h,
                      void* workspace, size_t workspace_bytes, void* stream) {
    Problem p;
    int st = check_matmul("mnb_gemm_silu_mul", d, M, a, b_packed, scales, zp_packed, bias, h, false, &p);
    if (st != MNB_OK) return st;
    if (d->N % 2 != 0)
        return fail(MNB_E_ARG, "mnb_gemm_silu_mul: N=%lld must be even (gate half, then up half)", (long long)d->N);
    st = check_workspace("mnb_gemm_silu_mul", gemm_silu_workspace_bytes(p), workspace, workspace_bytes);
    if (st != MNB_OK) return st;
    return launch_gemm_silu(p, static_cast<hipStream_t>(stream), workspace, workspace_bytes);
}

static int check_sequence(const mnb_matmul_args* ops, int64_t n_ops, std::vector<Problem>* out) {
    if (n_ops < 0 || (n_ops > 0 && !ops)) return fail(MNB_E_ARG, "sequence: ops NULL or n_ops < 0");
    out->resize((size_t)n_ops);
    for (int64_t i = 0; i < n_ops; i++) {
        const mnb_matmul_args& o = ops[i];
        int st = check_matmul("sequence entry", &o.desc, o.M, o.a, o.b_packed, o.scales, o.zp_packed,
                              o.bias, o.y, false, &(*out)[(size_t)i]);
        if (st != MNB_OK) {
            char msg[512];
            snprintf(msg, sizeof msg, "%s", g_last_error);
            return fail(st, "entry %lld: %s", (long long)i, msg);
        }
    }
    return MNB_OK;
}

// The products of a sequence run in order on one stream, so they share one
// workspace: the largest any of them needs.
static size_t sequence_workspace(const std::vector<Problem>& probs) {
    size_t need = 0;
    for (const Problem& p : probs) {
        const size_t b = workspace_of(p);
        if (b > need) need = b;
    }
    return need;
}

size_t mnb_sequence_workspace_bytes(const mnb_matmul_args* ops, int64_t n_ops) {
    std::vector<Problem> probs;
    try {
        if (check_sequence(ops, n_ops, &probs) != MNB_OK) return 0;
    } catch (const std::bad_alloc&) {
        return 0;
    }
    return sequence_workspace(probs);
}

int mnb_matmul_sequence(const mnb_matmul_args* ops, int64_t n_ops, void* workspace, size_t workspace_bytes,
                        void* stream) {
    std::vector<Problem> probs;
    int st;
    try {
        st = check_sequence(ops, n_ops, &probs);
    } catch (const std::bad_alloc&) {
        return fail(MNB_E_ARG, "sequence: out of host memory");
    }
    if (st != MNB_OK) return st;
    st = check_workspace("mnb_matmul_sequence", sequence_workspace(probs), workspace, workspace_bytes);
    if (st != MNB_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    for (size_t i = 0; i < probs.size(); i++) {
        st = run(probs[i], s, workspace, workspace_bytes);
        if (st != MNB_OK) return st;
    }
    return MNB_OK;
}

int mnb_graph_create(const mnb_matmul_args* ops, int64_t n_ops, void* workspace, size_t workspace_bytes,
                     mnb_graph** out) {
    if (!out) return fail(MNB_E_ARG, "mnb_graph_create: out is NULL");
    *out = nullptr;
    std::vector<Problem> probs;
    int st;
    try {
        st = check_sequence(ops, n_ops, &probs);
    } catch (const std::bad_alloc&) {
        return fail(MNB_E_ARG, "mnb_graph_create: out of host memory");
    }
    if (st != MNB_OK) return st;
    st = check_workspace("mnb_graph_create", sequence_workspace(probs), workspace, workspace_bytes);
    if (st != MNB_OK) return st;
    hipStream_t cs;
    hipError_t e = hipStreamCreateWithFlags(&cs, hipStreamNonBlocking);
    if (e != hipSuccess) return fail(MNB_E_HIP, "mnb_graph_create: stream: %s", hipGetErrorString(e));
    e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
    if (e != hipSuccess) {
        (void)hipStreamDestroy(cs);
        return fail(MNB_E_HIP, "mnb_graph_create: begin capture: %s", hipGetErrorString(e));
    }
    for (size_t i = 0; i < probs.size() && st == MNB_OK; i++)
        st = run(probs[i], cs, workspace, workspace_bytes);
    hipGraph_t graph = nullptr;
    e = hipStreamEndCapture(cs, &graph);
    (void)hipStreamDestroy(cs);
    if (st != MNB_OK || e != hipSuccess) {
        if (graph) (void)hipGraphDestroy(graph);
        if (st != MNB_OK) return st;
        return fail(MNB_E_HIP, "mnb_graph_create: end capture: %s", hipGetErrorString(e));
    }
    hipGraphExec_t exec = nullptr;
    e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
    if (e != hipSuccess) {
        (void)hipGraphDestroy(graph);
        return fail(MNB_E_HIP, "mnb_graph_create: instantiate: %s", hipGetErrorString(e));
    }
    mnb_graph* g = new (std::nothrow) mnb_graph{graph, exec};
    if (!g) {
        (void)hipGraphExecDestroy(exec);
        (void)hipGraphDestroy(graph);
        return fail(MNB_E_ARG, "mnb_graph_create: out of host memory");
    }
    *out = g;
    return MNB_OK;
}

int mnb_graph_launch(mnb_graph* g, void* stream) {
    if (!g) return fail(MNB_E_ARG, "mnb_graph_launch: graph is NULL");
    hipError_t e = hipGraphLaunch(g->exec, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(MNB_E_HIP, "mnb_graph_launch: %s", hipGetErrorString(e));
    return MNB_OK;
}

int mnb_graph_destroy(mnb_graph* g) {
    if (!g) return MNB_OK;
    hipError_t e1 = hipGraphExecDestroy(g->exec);
    hipError_t e2 = hipGraphDestroy(g->graph);
    delete g;
    if (e1 != hipSuccess || e2 != hipSuccess)
        return fail(MNB_E_HIP, "mnb_graph_destroy: %s",
                    hipGetErrorString(e1 != hipSuccess ? e1 : e2));
    return MNB_OK;
}

// Entries of a persistent step: each a valid product with M == 1 that the
// step kernel takes, all of one activation type.
static int check_step(const mnb_matmul_args* ops, int64_t n_ops, std::vector<Problem>* probs) {
    if (n_ops < 1) return fail(MNB_E_ARG, "step: n_ops=%lld, must be >= 1", (long long)n_ops);
    if (n_ops > (int64_t(1) << 20)) return fail(MNB_E_OVERFLOW, "step: n_ops=%lld too large", (long long)n_ops);
    int st = check_sequence(ops, n_ops, probs);
    if (st != MNB_OK) return st;
    for (int64_t i = 0; i < n_ops; i++) {
        const Problem& p = (*probs)[(size_t)i];
        if (p.bf16 != (*probs)[0].bf16)
            return fail(MNB_E_UNSUPPORTED, "step entry %lld: every entry must have the activation type of entry 0",
                        (long long)i);
        st = step_supports(p, i);
        if (st != MNB_OK) return st;
    }
    return MNB_OK;
}

size_t mnb_step_workspace_bytes(const mnb_matmul_args* ops, int64_t n_ops) {
    std::vector<Problem> probs;
    try {
        if (check_step(ops, n_ops, &probs) != MNB_OK) return 0;
    } catch (const std::bad_alloc&) {
        return 0;
    }
    return step_workspace_bytes(n_ops);
}

int mnb_step_create(const mnb_matmul_args* ops, int64_t n_ops, void* workspace, size_t workspace_bytes,
                    mnb_step** out) {
    if (!out) return fail(MNB_E_ARG, "mnb_step_create: out is NULL");
    *out = nullptr;
    std::vector<Problem> probs;
    int st;
    try {
        st = check_step(ops, n_ops, &probs);
    } catch (const std::bad_alloc&) {
        return fail(MNB_E_ARG, "mnb_step_create: out of host memory");
    }
    if (st != MNB_OK) return st;
    st = check_workspace("mnb_step_create", step_workspace_bytes(n_ops), workspace, workspace_bytes);
    if (st != MNB_OK) return st;
    const size_t ws_need = step_workspace_bytes(n_ops);
    for (int64_t i = 0; i < n_ops; i++) {
        const Problem& p = probs[(size_t)i];
        if (overlap(workspace, ws_need, p.y, (size_t)p.N * (p.bf16 ? 2 : 4)))
            return fail(MNB_E_ARG, "mnb_step_create: entry %lld: y overlaps the workspace", (long long)i);
    }
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(MNB_E_HIP, "mnb_step_create: hipGetDevice: %s", hipGetErrorString(e));
    int grid = 0;
    st = step_grid(probs[0].bf16, &grid);
    if (st != MNB_OK) return st;
    try {
        st = step_prepare(probs.data(), n_ops, grid, workspace);
    } catch (const std::bad_alloc&) {
        return fail(MNB_E_ARG, "mnb_step_create: out of host memory");
    }
    if (st != MNB_OK) return st;
    mnb_step* h = new (std::nothrow) mnb_step{dev, grid, probs[0].bf16, n_ops, workspace, nullptr};
    if (!h) return fail(MNB_E_ARG, "mnb_step_create: out of host memory");
    *out = h;
    return MNB_OK;
}

int mnb_step_launch(mnb_step* h, void* stream) {
    if (!h) return fail(MNB_E_ARG, "mnb_step_launch: step is NULL");
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(MNB_E_HIP, "mnb_step_launch: hipGetDevice: %s", hipGetErrorString(e));
    if (dev != h->device)
        return fail(MNB_E_ARG, "mnb_step_launch: created on device %d, current device %d", h->device, dev);
    return step_launch(h->bf16, h->grid, h->workspace, h->n_ops, h->trace, static_cast<hipStream_t>(stream));
}

size_t mnb_step_trace_bytes(const mnb_step* h) {
    return h ? (size_t)h->grid * (size_t)h->n_ops * 5 * sizeof(uint64_t) : 0;
}

int mnb_step_set_trace(mnb_step* h, void* trace, size_t trace_bytes) {
    if (!h) return fail(MNB_E_ARG, "mnb_step_set_trace: step is NULL");
    if (trace) {
        if (trace_bytes < mnb_step_trace_bytes(h))
            return fail(MNB_E_ARG, "mnb_step_set_trace: %zu bytes given, %zu needed", trace_bytes,
                        mnb_step_trace_bytes(h));
        if (!aligned(trace, 8)) return fail(MNB_E_ALIGN, "mnb_step_set_trace: trace must be 8-byte aligned");
    }
    h->trace = trace;
    return MNB_OK;
}

int mnb_step_check(mnb_step* h, void* stream) {
    if (!h) return fail(MNB_E_ARG, "mnb_step_check: step is NULL");
    return step_check(h->workspace, static_cast<hipStream_t>(stream));
}

int mnb_step_destroy(mnb_step* h) {
    delete h;
    return MNB_OK;
}

const char* mnb_status_string(int status) {
    switch (status) {
        case MNB_OK: return "MNB_OK";
        case MNB_E_ARG: return "MNB_E_ARG: invalid argument";
        case MNB_E_UNSUPPORTED: return "MNB_E_UNSUPPORTED: unsupported configuration";
        case MNB_E_ALIGN: return "MNB_E_ALIGN: misaligned pointer";
        case MNB_E_OVERFLOW: return "MNB_E_OVERFLOW: size out of range";
        case MNB_E_HIP: return "MNB_E_HIP: HIP runtime error";
        default: return "unknown mnb status";
    }
}

const char* mnb_last_error(void) { return g_last_error; }

const char* mnb_version(void) { return MNB_VERSION_STRING; }

}  // extern "C"
