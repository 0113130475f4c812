// Decode GEMV launcher (M == 1, or up to four rows): geometry, kernel
// instance and grid.  The kernel, and what it computes, is in
// mnb_gemv_kernel.h.
#include "mnb_gemv_kernel.h"

namespace mnb {
namespace {

constexpr size_t kMaxLds = kGemvMaxLds;

GemvFn pick(bool bf16, bool has_zp, bool has_bias, int CB, int J, int W, bool silu, int input, bool nts) {
    return bf16 ? gemv_pick_bf16(has_zp, has_bias, CB, J, W, silu, input, nts)
                : gemv_pick_f32(has_zp, has_bias, CB, J, W, silu, input, nts);
}

GemvFn pick_rows(bool bf16, bool has_zp, bool has_bias, int MR, int J, int W, bool nts) {
    return bf16 ? gemv_pick_rows_bf16(has_zp, has_bias, MR, J, W, nts)
                : gemv_pick_rows_f32(has_zp, has_bias, MR, J, W, nts);
}

int compute_units() { return device_compute_units(); }

}  // namespace

int device_compute_units() {
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

namespace {

// Workgroups of kernel f with lds bytes of staged activations resident per
// CU (the compiler's register use and the LDS decide), cached per thread.
int resident_per_cu(GemvFn f, size_t lds) {
    struct Entry { GemvFn f; size_t lds; int n; };
    static thread_local Entry cache[64];
    static thread_local int used = 0;
    for (int i = 0; i < used; i++)
        if (cache[i].f == f && cache[i].lds == lds) return cache[i].n;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(f),
                                                     64 * kGemvWavesPerBlock, lds) != hipSuccess || n < 1)
        n = 1;
    cache[used % 64] = Entry{f, lds, n};
    if (used < 64) used++;
    return n;
}

}  // namespace

int64_t gemv_max_k(int bs) {
    // limited by the register geometry (S <= 64 * W * kJMax chunks) and by
    // the staged activations (S rows of CK float32 in kMaxLds bytes)
    const int CK = bs >= 32 ? 32 : 16;
    const int W = bs >= 32 ? kWMax : 1;
    int64_t s_max = (int64_t)64 * W * kJMax;
    const int64_t s_lds = (int64_t)(kMaxLds / (CK * sizeof(float)));
    if (s_lds < s_max) s_max = s_lds;
    return s_max * CK;
}

namespace {

// Rows per launch of the row kernel for M rows (2 <= M <= 4), and whether
// it takes the problem: 16-byte chunks (block >= 32), activations staged with
// LDS-direct loads, one chunk per lane and row (two for M == 2), and the MR
// rows' staged activations within kMaxLds.
int rows_mr(int64_t M) { return M <= 2 ? 2 : 4; }

size_t rows_lds(const Problem& p, int MR) {
    const int esz = p.bf16 ? 2 : 4;
    const int64_t S = (p.K + 31) / 32;
    return (size_t)MR * (size_t)((S * 32 * esz + 1023) / 1024) * 1024;
}

// silu: p.N = 2 * half columns (gate half, then up half), y receives half
// values of silu(gate) * up.  MR > 1: the row kernel (p.M rows, p.M <= MR).
int launch(const Problem& p, hipStream_t s, bool silu, int MR = 1, const void* gamma = nullptr, float eps = 0.f) {
    const int CB = p.bs >= 32 ? 16 : 8;
    const int CK = 2 * CB;
    GemvArgs a;
    a.a = p.a; a.b = p.b; a.scales = p.scales; a.zp = p.has_zp ? p.zp : nullptr;
    a.bias = p.bias; a.y = p.y;
    a.K = p.K; a.N = p.N; a.col_bytes = p.col_bytes;
    a.nb = p.nb; a.zp_row = p.zp_row;
    a.S = (int)((p.K + CK - 1) / CK);
    a.log2_bs = ilog2(p.bs);
    a.half = silu ? p.N / 2 : 0;
    a.M = (int)p.M;
    a.gamma = gamma;
    a.eps = eps;
    // the gated kernel takes the plain geometry: its sums are mnb_gemv's
    const Geometry geo = MR == 1 ? geometry(a.S, CB == 16, kJMax) : geometry(a.S, true, 4 / MR);
    if (geo.J == 0)
        return fail(MNB_E_UNSUPPORTED, "gemv: K=%lld beyond the register kernel", (long long)p.K);
    a.log2_L = geo.log2_L;
    const int G = geo.W == 1 ? (64 >> geo.log2_L) : 1;
    const int64_t cols = silu ? a.half : p.N;       // columns whose groups are walked
    a.n_groups = (cols + G - 1) / G;
    // staged activations: S chunk rows of CK elements
    const int esz = p.bf16 ? 2 : 4;
    a.a16 = ((p.K * esz) % 16 == 0) && ((reinterpret_cast<uintptr_t>(p.a) & 15) == 0) &&
            p.K * esz < (int64_t(1) << 31);
    // The staging writes whole 1 KiB requests (nreq per row in the kernel),
    // so every row is rounded up to a whole KiB of LDS; the row kernel stages
    // row m at m * ceil(S * CK * esz / 1 KiB) KiB.
    size_t lds = MR == 1 ? (size_t)(((int64_t)a.S * CK * esz + 1023) / 1024) * 1024 : rows_lds(p, MR);
    if (gamma) {
        if (!a.a16) return fail(MNB_E_UNSUPPORTED, "gemv rmsnorm: K * element size must be a multiple of 16");
        lds *= 2;                                   // gamma staged after A
    }
    if (lds > kMaxLds)
        return fail(MNB_E_UNSUPPORTED, "gemv: K=%lld needs %zu bytes of LDS", (long long)p.K, lds);
    // Fill the chip with resident teams of W wavefronts (the kernel's real
    // occupancy), one column group per team per iteration: unrolling several
    // groups per iteration costs more in occupancy than it saves.  For the
    // kernels that hold activations in registers (rows, RMSNorm, one chunk
    // per lane, the LM heads): when two workgroups per CU already leave each
    // team at most 2.5 groups, use only
    // those (a team with two groups has the second in flight while it
    // reduces the first, 2-7 % faster on the few-MB decode projections).  The
    // one-row kernel that reads them from LDS (several chunks per lane) fills
    // every resident slot: with it the 4B decode step ran 1.8 % faster than
    // with registers for every shape, the 0.6B step 2.6 %.
    const int64_t cus = compute_units();
    const int teams_per_block = kGemvWavesPerBlock / geo.W;
    // Weights are read non-temporally (each byte once): streamed past the
    // caches, they leave the activations and the scales resident, 4-9 % per
    // decode step.  With blocks of at most 32 values every chunk has its own
    // scale and zero point, a stream of 20-28 % of the bytes read once like
    // the weights, read non-temporally too (the 0.6B step 7 % faster); with
    // larger blocks several lanes and neighbouring columns share the scale
    // lines, which stay cached (non-temporal scales slowed the 4B step 3 %).
    // (RMSNorm: exactly with 8-byte chunks, the instances there are)
    const bool nts = gamma ? CB != 16 : p.bs <= 32;
    bool actl = MR == 1 && !gamma && geo.J > 1;
    GemvFn f = MR == 1 ? pick(p.bf16, p.has_zp, p.bias != nullptr, CB, geo.J, geo.W, silu,
                              gamma ? kInputRms : kInputLds, nts)
                       : pick_rows(p.bf16, p.has_zp, p.bias != nullptr, MR, geo.J, geo.W, nts);
    if (!f) return fail(MNB_E_UNSUPPORTED, "gemv: no kernel for J=%d W=%d", geo.J, geo.W);
    // A launch whose resident teams would each walk more than four column
    // groups (the LM heads) reads its activations once into registers: read
    // from LDS per chunk they would be read again for every group (the 4B LM
    // head, cold, 49.5 us that way and 43.9 us with registers on one box).
    if (actl && !silu && nts == (CB != 16)) {
        const int64_t resident_teams = cus * resident_per_cu(f, lds) * teams_per_block;
        if (a.n_groups > 4 * resident_teams) {
            const GemvFn fr = pick(p.bf16, p.has_zp, p.bias != nullptr, CB, geo.J, geo.W, false, kInputRegs, nts);
            if (fr) {
                f = fr;
                actl = false;
            }
        }
    }
    const int64_t teams = a.n_groups;
    int64_t blocks = (teams + teams_per_block - 1) / teams_per_block;
    // Where one column group per team takes at most twice the workgroups
    // that the single-stage kernel keeps resident (every per-layer decode
    // projection), that kernel on that grid: with the registers of the second
    // stage free, more workgroups are resident and each team's loads go out
    // at once (the 4B decode step 0.908 -> 0.828 ms, the 0.6B step 0.379 ->
    // 0.365 ms on one box; the 4B gate||up's 1216 workgroups all resident).
    bool one = false;
    if (actl && !silu) {
        const GemvFn f1 = pick(p.bf16, p.has_zp, p.bias != nullptr, CB, geo.J, geo.W, false, kInputLdsOne, nts);
        if (f1 && blocks <= 2 * cus * resident_per_cu(f1, lds)) {
            f = f1;
            one = true;
        }
    }
    int64_t max_blocks = cus * resident_per_cu(f, lds);
    if (!actl && max_blocks > 2 * cus && 2 * teams <= 5 * (2 * cus * teams_per_block)) max_blocks = 2 * cus;
    // The LDS-reading kernel gives every team one column group where that
    // takes at most twice the resident workgroups (the rest start as the
    // first ones finish): the 4B gate||up, 1.6 groups per resident team,
    // made the step 0.4 % faster so; the same grid with two groups for every
    // team (fewer workgroups, each walking the same number of groups) made
    // it 4 % slower.
    if (!one && blocks > max_blocks && !(actl && blocks <= 2 * max_blocks)) blocks = max_blocks;
    hipLaunchKernelGGL(f, dim3((unsigned)blocks), dim3(64 * kGemvWavesPerBlock), lds, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(MNB_E_HIP, "gemv launch: %s", hipGetErrorString(e));
    return MNB_OK;
}

}  // namespace

int launch_gemv(const Problem& p, hipStream_t s) { return launch(p, s, false); }

bool gemv_rows_ok(const Problem& p) {
    if (p.M < 2 || p.M > 4 || p.bs < 32) return false;
    // The LM heads (more than 32768 columns; every per-layer projection of
    // these models has at most 19456) go to the matrix-core kernel where it
    // takes them: there the row kernel's teams walk dozens of column groups
    // each, and the 0.6B step at 4 rows took 0.588 instead of 0.610 ms so
    // (its LM head 62 us in the row kernel, about 39 us on the matrix cores).
    if (p.N > 32768 && smallm_ok(p)) return false;
    const int esz = p.bf16 ? 2 : 4;
    if ((p.K * esz) % 16 != 0 || p.M * p.K * esz >= (int64_t(1) << 31))
        return false;
    const int MR = rows_mr(p.M);
    return geometry((p.K + 31) / 32, true, 4 / MR).J > 0 && rows_lds(p, MR) <= kMaxLds;
}

int launch_gemv_rows(const Problem& p, hipStream_t s) { return launch(p, s, false, rows_mr(p.M)); }

int launch_gemv_silu(const Problem& p, hipStream_t s) { return launch(p, s, true); }

int launch_gemv_rmsnorm(const Problem& p, const void* gamma, float eps, hipStream_t s) {
    return launch(p, s, false, 1, gamma, eps);
}

}  // namespace mnb
