// Persistent decode step (M == 1): every projection of a decode step in ONE
// cooperative launch.
//
// Page "Qwen3 CPU Inference Critical Path", "Phase Q5: scheduling and
// fusion": a step is a chain of projections, each one's input available only
// after the previous one (with the model's other operators between them) has
// finished; "INT4 MatMul is first": batch-1 projections are dominated by the
// weight stream.  Launched one by one, every projection pays a fill and a
// drain of the whole chip.  Here one workgroup per CU stays resident for the
// whole step, and only the activation row of a projection waits for the
// previous projection: the weights never depend on it, so each wavefront
// requests the next projection's weights before the wait.
//
// Workgroup = 8 compute wavefronts + 1 control wavefront.
//  * Compute wavefront t (t = wave * G + workgroup, T = 8 G in all) takes
//    column groups t, t + T, t + 2T, ... of every projection, with the
//    geometry, loads and arithmetic of the per-projection decode GEMV
//    (mnb_gemv_core.h): a column's sum has the same float32 bits as
//    mnb_gemv's.  Its items (projection, column group) form one stream across
//    projections; two register stages hold the next two items' weights,
//    scales, zero points and bias, refilled as each item is reduced, so the
//    requests for projection i + 1 are in flight while projection i ends and
//    while the barrier below is waited for.  A compute wavefront issues no
//    memory instruction besides those loads (vector memory operations retire
//    in order: a store or an activation load queued behind prefetched
//    weights could only be waited for with them); its column sums go to LDS.
//  * The control wavefront stages each projection's activation row into LDS
//    (LDS-direct loads that read at device coherence), then, once the compute
//    wavefronts have finished the projection, stores the workgroup's sums to
//    y with write-through stores, waits for their acknowledgement, and adds
//    one to one of 16 arrival counters (workgroup b to counter b % 16, each in
//    its own 128-byte line).  Before staging the next row it polls the
//    counters until every workgroup has arrived: the outputs of projection i
//    are in memory before any workgroup reads projection i + 1's input, so a
//    step whose input i + 1 is (or is computed from) output i is ordered.
//    Every poll is bounded: a wavefront that waits too long records an error
//    word and stops waiting, so every wavefront always finishes.
//  * Two workgroup barriers per projection order the LDS hand-offs:
//    S(i) (row i staged) and D(i) (sums of projection i written).
//  * The last workgroup to finish clears the counters for the next launch.
#include <type_traits>
#include <vector>

#include "mnb_gemv_core.h"

namespace mnb {
namespace {

constexpr int kComputeWaves = 8;
constexpr int kThreads = 64 * (kComputeWaves + 1);
constexpr int kCounters = 16;
constexpr int kCounterStride = 32;             // 32-bit words: one 128-byte line per counter
constexpr size_t kDoneOffset = 2048;           // bytes: after the 16 counter lines
constexpr size_t kErrorOffset = 2176;
constexpr size_t kHeaderBytes = 2304;          // multiple of 256: the table follows
constexpr size_t kActLds = 40 * 1024;          // one staged activation row
constexpr int kOutValues = 4096;               // a workgroup's sums of one projection
constexpr size_t kLdsBytes = 96 * 1024;        // more than half of a CU's LDS: one workgroup per CU
constexpr uint32_t kSpinMax = 1u << 20;        // polls (each a device-coherent round trip, ~1 us)
constexpr uint32_t kCoherent = 16;             // cache policy of a device-coherent load (sc1)

static_assert(kActLds + sizeof(float) * kOutValues <= kLdsBytes, "LDS layout");

// One projection as the kernel reads it (device memory, written at creation).
struct StepOp {
    const void* a;
    const uint8_t* b;
    const void* scales;
    const uint8_t* zp;          // NULL without zero points
    const float* bias;          // NULL without bias
    void* y;
    int64_t N, col_bytes;
    int32_t K, nb, zp_row, S, log2_bs, log2_L, J, n_groups, n_items, nreq, has_zp, has_bias;
};

// The table is read-only for the whole launch: read through the constant
// address space, its fields come in with scalar loads, which wait on their
// own counter (a vector load of a field would queue behind the weights in
// flight and could only be waited for with them).
typedef const __attribute__((address_space(4))) StepOp* OpTable;

// A projection's fields, read one by one through the table (scalar loads).
__device__ __forceinline__ StepOp op_at(OpTable t, int i) {
    StepOp o;
    o.a = t[i].a; o.b = t[i].b; o.scales = t[i].scales; o.zp = t[i].zp; o.bias = t[i].bias; o.y = t[i].y;
    o.N = t[i].N; o.col_bytes = t[i].col_bytes;
    o.K = t[i].K; o.nb = t[i].nb; o.zp_row = t[i].zp_row; o.S = t[i].S; o.log2_bs = t[i].log2_bs;
    o.log2_L = t[i].log2_L; o.J = t[i].J; o.n_groups = t[i].n_groups; o.n_items = t[i].n_items;
    o.nreq = t[i].nreq; o.has_zp = t[i].has_zp; o.has_bias = t[i].has_bias;
    return o;
}

struct StepArgs {
    OpTable ops;
    uint32_t* counters;
    uint32_t* done;
    uint32_t* error;
    int n_ops;
    // optional phase timestamps (s_memrealtime, 100 MHz): for workgroup w and
    // entry i, trace[(w * n_ops + i) * 5 + k] at k = 0 before the wait for
    // entry i - 1, 1 after it, 2 with row i staged, 3 with the workgroup's
    // sums of entry i complete, 4 with its outputs acknowledged; or NULL
    uint64_t* trace;
};

// One item's loads, kept raw (decoding them here would wait for them).
struct Item {
    u32x4 w[kJMax];
    uint32_t sc[kJMax];
    uint32_t zb[kJMax];
    uint32_t bias;
};

struct Cursor {
    int op;       // projection
    int item;     // index among this wavefront's column groups of the projection
};

// A workgroup barrier.  Each call site passes its own tag (an assembler
// comment), so the compiler never merges the barrier blocks of different
// sites: the vector-memory wait counts it derives at a merged block would
// have to assume the worst of every path into it.
template <int SITE>
__device__ __forceinline__ void wg_barrier() { asm volatile("s_barrier ; site %0" : : "i"(SITE) : "memory"); }

// LDS writes and reads of this wavefront done (vector memory loads may stay
// in flight): vmcnt 63, expcnt 7, lgkmcnt 0
__device__ __forceinline__ void lds_done() { __builtin_amdgcn_s_waitcnt(0xC07F); }

__device__ __forceinline__ int items_of(const StepOp& o, int t, int T) {
    return t < o.n_groups ? (o.n_groups - 1 - t) / T + 1 : 0;
}

// first projection at or after `op` in which wavefront t has a column group
__device__ __forceinline__ int next_op(const StepArgs& s, int op, int t) {
    while (op < s.n_ops && t >= s.ops[op].n_groups) op++;
    return op;
}

__device__ __forceinline__ void advance(const StepArgs& s, Cursor& c, int t, int T) {
    const StepOp o = op_at(s.ops, c.op);
    if (++c.item >= items_of(o, t, T)) {
        c.op = next_op(s, c.op + 1, t);
        c.item = 0;
    }
}

// Requests the loads of item c (or, past the last projection, loads that read
// nothing): always 16 memory instructions, so the waits before each stage's
// use count exactly the other stage's requests.
template <bool BF16>
__device__ __forceinline__ void request(const StepArgs& s, const Cursor& c, int t, int T, int lane, Item& r) {
    constexpr int SSZ = BF16 ? 2 : 4;
    const bool live = c.op < s.n_ops;
    const StepOp o = op_at(s.ops, live ? c.op : 0);
    const int Gc = 64 >> o.log2_L;
    const int64_t col0 = (int64_t)(t + (int64_t)c.item * T) * Gc;
    const int64_t left = o.N - col0;
    const int ncol = live ? (left < Gc ? (int)left : Gc) : 0;
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(o.b) + (ncol ? col0 * o.col_bytes : 0), (short)0, (int)(ncol * o.col_bytes), 0x00020000);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        static_cast<uint8_t*>(const_cast<void*>(o.scales)) + (ncol ? col0 * o.nb * SSZ : 0), (short)0,
        ncol * o.nb * SSZ, 0x00020000);
    const __amdgpu_buffer_rsrc_t rz = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(o.has_zp ? o.zp : o.b) + (ncol && o.has_zp ? col0 * o.zp_row : 0), (short)0,
        o.has_zp ? ncol * o.zp_row : 0, 0x00020000);
    const __amdgpu_buffer_rsrc_t rbias = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(o.has_bias ? o.bias : reinterpret_cast<const float*>(o.b)) +
            (ncol && o.has_bias ? col0 : 0), (short)0, o.has_bias ? ncol * 4 : 0, 0x00020000);
    const int L = 1 << o.log2_L;
    const int p = lane & (L - 1), gsub = lane >> o.log2_L;
#pragma unroll
    for (int j = 0; j < kJMax; j++) {
        const int ch = p + j * L;
        const uint32_t out = (j < o.J && ch < o.S) ? 0u : kOob;
        const int blk = (ch * 32) >> o.log2_bs;
        const uint32_t os = (uint32_t)((gsub * o.nb + blk) * SSZ) | out;
        r.sc[j] = BF16 ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs, os, 0, 0)
                       : __builtin_amdgcn_raw_buffer_load_b32(rs, os, 0, 0);
        r.zb[j] = __builtin_amdgcn_raw_buffer_load_b8(rz, (uint32_t)(gsub * o.zp_row + (blk >> 1)) | out, 0, 0);
    }
    r.bias = __builtin_amdgcn_raw_buffer_load_b32(rbias, (uint32_t)(4 * gsub), 0, 0);
#pragma unroll
    for (int j = 0; j < kJMax; j++) {
        const int ch = p + j * L;
        const uint32_t out = (j < o.J && ch < o.S) ? 0u : kOob;
        r.w[j] = __builtin_amdgcn_raw_buffer_load_b128(rb, (uint32_t)(gsub * o.col_bytes + ch * 16) | out, 0,
                                                       kNonTemporal);
    }
}

// Column sums of item c from its loads and the staged row, exactly as the
// decode GEMV forms them; the writer lane of each column puts y (with bias)
// into the workgroup's output slots.
template <bool BF16>
__device__ __forceinline__ void reduce_item(const StepArgs& s, const Cursor& c, int wave, int lane,
                                            const uint8_t* act, float* out, const Item& r, const NibbleMasks& nk) {
    constexpr int ESZ = BF16 ? 2 : 4;
    constexpr int RB = 32 * ESZ;          // bytes per staged chunk row
    constexpr int NV = RB / 16;
    constexpr int RPS = 256 / RB;
    const StepOp o = op_at(s.ops, c.op);
    const int L = 1 << o.log2_L;
    const int p = lane & (L - 1), gsub = lane >> o.log2_L;
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < kJMax; j++) {
        if (j < o.J) {
            const int ch = p + j * L;
            // a chunk past K contributes an exact zero (its scale reads 0)
            float dot = 0.f;
            if (ch < o.S) {
                float av[32];
#pragma unroll
                for (int v = 0; v < NV; v++) {
                    const u32x4 x = *reinterpret_cast<const u32x4*>(act + ch * RB + 16 * (v ^ ((ch / RPS) % NV)));
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        if constexpr (BF16) {
                            av[8 * v + 2 * e] = __uint_as_float(x[e] << 16);
                            av[8 * v + 2 * e + 1] = __uint_as_float(x[e] & 0xFFFF0000u);
                        } else {
                            av[4 * v + e] = __uint_as_float(x[e]);
                        }
                    }
                }
                uint32_t words[4];
#pragma unroll
                for (int d = 0; d < 4; d++) words[d] = r.w[j][d];
                uint32_t zq = 8u;
                if (o.has_zp) {
                    const int blk = (ch * 32) >> o.log2_bs;
                    zq = (blk & 1) ? ((r.zb[j] >> 4) & 0xFu) : (r.zb[j] & 0xFu);
                }
                uint32_t ze, zo;
                zero_point_pairs(zq, ze, zo);
                dot = dot_words<4>(words, av, ze, zo, nk);
            }
            const float sc = BF16 ? __uint_as_float(r.sc[j] << 16) : __uint_as_float(r.sc[j]);
            acc = fmaf(sc, dot, acc);
        }
    }
    acc = reduce_lanes(acc, o.log2_L);
    if ((lane & (L - 1)) == L - 1) {
        const int Gc = 64 >> o.log2_L;
        const int64_t g = (int64_t)(wave * (int)gridDim.x + (int)blockIdx.x) + (int64_t)c.item * (kComputeWaves * gridDim.x);
        if (g * Gc + gsub < o.N) {
            float v = acc;
            if (o.has_bias) v += __uint_as_float(r.bias);
            out[(wave * o.n_items + c.item) * Gc + gsub] = v;
        }
    }
}

template <bool BF16>
__device__ void compute_wave(const StepArgs& s, const uint8_t* act, float* out, int wave, int lane) {
    const int G = (int)gridDim.x, T = kComputeWaves * G;
    const int t = wave * G + (int)blockIdx.x;
    const int n = s.n_ops;
    Cursor lc{next_op(s, 0, t), 0};       // next item to request
    Cursor cc = lc;                       // next item to reduce
    Item A, B;
    request<BF16>(s, lc, t, T, lane, A);
    if (lc.op < n) advance(s, lc, t, T);
    request<BF16>(s, lc, t, T, lane, B);
    if (lc.op < n) advance(s, lc, t, T);
    const NibbleMasks nk = nibble_masks();
    int cur = -1;     // projection whose S barrier this wavefront has passed
    // passes the barriers up to S(op); SITE tells the call sites apart
    auto enter = [&](int op, auto site) {
        constexpr int S0 = decltype(site)::value;
        while (cur < op) {
            if (cur >= 0) {
                lds_done();
                wg_barrier<S0>();      // D(cur)
            }
            cur++;
            wg_barrier<S0 + 1>();      // S(cur)
        }
    };
    // Items in pairs: stage A, then stage B.  Both stages are requested in
    // every iteration and the loop leaves only at its top or after B's
    // request, so every use of a stage finds exactly the other stage's 16
    // requests issued after its own.
    for (;;) {
        if (cc.op >= n) break;
        enter(cc.op, std::integral_constant<int, 10>());
        reduce_item<BF16>(s, cc, wave, lane, act, out, A, nk);
        request<BF16>(s, lc, t, T, lane, A);
        if (lc.op < n) advance(s, lc, t, T);
        advance(s, cc, t, T);
        const bool more = cc.op < n;
        if (more) {
            enter(cc.op, std::integral_constant<int, 20>());
            reduce_item<BF16>(s, cc, wave, lane, act, out, B, nk);
        }
        request<BF16>(s, lc, t, T, lane, B);
        if (lc.op < n) advance(s, lc, t, T);
        if (!more) break;
        advance(s, cc, t, T);
    }
    // the barriers of the projections left
    if (cur >= 0) {
        lds_done();
        wg_barrier<30>();              // D(cur)
    }
    for (int i = cur + 1; i < n; i++) {
        wg_barrier<31>();              // S(i)
        wg_barrier<32>();              // D(i)
    }
}

// Until every workgroup has arrived `target` times in all; false (and the
// error word set) if the bounded wait runs out.
__device__ bool wait_arrivals(const StepArgs& s, uint32_t target, int lane) {
    for (uint32_t it = 0;; it++) {
        uint32_t v = 0;
        if (lane < kCounters)
            v = __hip_atomic_load(s.counters + lane * kCounterStride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        v += __shfl_xor(v, 1);
        v += __shfl_xor(v, 2);
        v += __shfl_xor(v, 4);
        v += __shfl_xor(v, 8);
        const uint32_t total = __builtin_amdgcn_readfirstlane(v);
        if (total >= target) return true;
        if (it >= kSpinMax) {
            if (lane == 0) __hip_atomic_fetch_or(s.error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return false;
        }
        __builtin_amdgcn_s_sleep(1);
    }
}

template <bool BF16>
__device__ void control_wave(const StepArgs& s, uint8_t* act, const float* out, int lane) {
    constexpr int ESZ = BF16 ? 2 : 4;
    constexpr int RB = 32 * ESZ;
    constexpr int NV = RB / 16;
    constexpr int RPS = 256 / RB;
    const int G = (int)gridDim.x, T = kComputeWaves * G;
    const int n = s.n_ops;
    bool waiting = true;
    for (int i = 0; i < n; i++) {
        const StepOp o = op_at(s.ops, i);
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        // every workgroup's outputs of projection i - 1 are in memory
        if (i > 0 && waiting) waiting = wait_arrivals(s, (uint32_t)i * (uint32_t)G, lane);
        const uint64_t t1 = __builtin_amdgcn_s_memrealtime();
        // stage row i: 1 KiB requests, the swizzle of the decode GEMV
        const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<void*>(o.a), (short)0, o.K * ESZ, 0x00020000);
        for (int r = 0; r < o.nreq; r++) {
            const int row = r * (64 / NV) + lane / NV;
            const int pos = lane % NV;
            const int piece = pos ^ ((row / RPS) % NV);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                ra, (void __attribute__((address_space(3)))*)(act + 1024 * r), 16, (uint32_t)(row * RB + 16 * piece),
                0, 0, kCoherent);
        }
        __builtin_amdgcn_s_waitcnt(0);
        const uint64_t t2 = __builtin_amdgcn_s_memrealtime();
        wg_barrier<40>();              // S(i)
        wg_barrier<41>();              // D(i)
        const uint64_t t3 = __builtin_amdgcn_s_memrealtime();
        // the workgroup's sums of projection i, written through to memory
        const int Gc = 64 >> o.log2_L;
        const int per_wave = o.n_items * Gc;
        for (int idx = lane; idx < kComputeWaves * per_wave; idx += 64) {
            const int w = idx / per_wave, rem = idx - w * per_wave;
            const int c = rem / Gc, gsub = rem - c * Gc;
            const int64_t g = (int64_t)(w * G + (int)blockIdx.x) + (int64_t)c * T;
            const int64_t col = g * Gc + gsub;
            if (g < o.n_groups && col < o.N) {
                const float v = out[idx];
                if constexpr (BF16)
                    __hip_atomic_store(static_cast<uint16_t*>(o.y) + col, f32_to_bf16_rtne(v), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                else
                    __hip_atomic_store(static_cast<float*>(o.y) + col, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        __builtin_amdgcn_s_waitcnt(0);     // acknowledged
        const uint64_t t4 = __builtin_amdgcn_s_memrealtime();
        if (s.trace && lane < 5)
            s.trace[((size_t)blockIdx.x * n + i) * 5 + lane] =
                lane == 0 ? t0 : lane == 1 ? t1 : lane == 2 ? t2 : lane == 3 ? t3 : t4;
        if (i + 1 < n && lane == 0)
            __hip_atomic_fetch_add(s.counters + (blockIdx.x % kCounters) * kCounterStride, 1u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
    }
    // the last workgroup to get here clears the counters for the next launch
    // (every other one has finished all its waits)
    if (lane == 0) {
        const uint32_t before = __hip_atomic_fetch_add(s.done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (before == (uint32_t)G - 1) {
            for (int c = 0; c < kCounters; c++)
                __hip_atomic_store(s.counters + c * kCounterStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(s.done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void step_kernel(StepArgs s) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    float* out = reinterpret_cast<float*>(lds + kActLds);
    if (wave == kComputeWaves)
        control_wave<BF16>(s, lds, out, lane);
    else
        compute_wave<BF16>(s, lds, out, wave, lane);
}

}  // namespace

size_t step_workspace_bytes(int64_t n_ops) {
    return kHeaderBytes + (((size_t)n_ops * sizeof(StepOp) + 255) / 256) * 256;
}

// Host-side checks of one projection against what the step kernel takes;
// MNB_OK or MNB_E_UNSUPPORTED with the reason.
int step_supports(const Problem& p, int64_t idx) {
    const int esz = p.bf16 ? 2 : 4;
    if (p.M != 1) return fail(MNB_E_UNSUPPORTED, "step entry %lld: M=%lld, the decode step takes M == 1", (long long)idx, (long long)p.M);
    if (p.bs < 32)
        return fail(MNB_E_UNSUPPORTED, "step entry %lld: block_size=%d, the decode step takes >= 32", (long long)idx, p.bs);
    if ((p.K * esz) % 16 != 0)
        return fail(MNB_E_UNSUPPORTED, "step entry %lld: K * element size must be a multiple of 16", (long long)idx);
    const int64_t S = (p.K + 31) / 32;
    const Geometry geo = geometry(S, true, kJMax);
    if (geo.J == 0 || geo.W != 1)
        return fail(MNB_E_UNSUPPORTED, "step entry %lld: K=%lld needs split-K wavefront teams (decode step: W == 1)",
                    (long long)idx, (long long)p.K);
    if ((size_t)((S * 32 * esz + 1023) / 1024) * 1024 > kActLds)
        return fail(MNB_E_UNSUPPORTED, "step entry %lld: K=%lld, the staged row exceeds %zu bytes", (long long)idx,
                    (long long)p.K, kActLds);
    return MNB_OK;
}

namespace {

struct StepKernel {
    const void* fn;
};

const void* step_fn(bool bf16) {
    return bf16 ? reinterpret_cast<const void*>(step_kernel<true>) : reinterpret_cast<const void*>(step_kernel<false>);
}

}  // namespace

// Fills the table for a grid of `grid` workgroups and writes it (and a zero
// header) into ws.  The problems passed step_supports.
int step_prepare(const Problem* probs, int64_t n, int grid, void* ws) {
    std::vector<StepOp> table((size_t)n);
    const int64_t T = (int64_t)kComputeWaves * grid;
    for (int64_t i = 0; i < n; i++) {
        const Problem& p = probs[i];
        const int esz = p.bf16 ? 2 : 4;
        const int64_t S = (p.K + 31) / 32;
        const Geometry geo = geometry(S, true, kJMax);
        const int Gc = 64 >> geo.log2_L;
        const int64_t n_groups = (p.N + Gc - 1) / Gc;
        const int64_t n_items = (n_groups + T - 1) / T;
        if ((int64_t)kComputeWaves * n_items * Gc > kOutValues)
            return fail(MNB_E_UNSUPPORTED, "step entry %lld: N=%lld gives a workgroup more than %d outputs on %d "
                        "workgroups", (long long)i, (long long)p.N, kOutValues, grid);
        StepOp& o = table[(size_t)i];
        o.a = p.a; o.b = p.b; o.scales = p.scales; o.zp = p.has_zp ? p.zp : nullptr; o.bias = p.bias; o.y = p.y;
        o.N = p.N; o.col_bytes = p.col_bytes;
        o.K = (int32_t)p.K; o.nb = p.nb; o.zp_row = p.zp_row; o.S = (int32_t)S;
        o.log2_bs = ilog2(p.bs); o.log2_L = geo.log2_L; o.J = geo.J;
        o.n_groups = (int32_t)n_groups; o.n_items = (int32_t)n_items;
        o.nreq = (int32_t)((S * 32 * esz + 1023) / 1024);
        o.has_zp = p.has_zp ? 1 : 0; o.has_bias = p.bias ? 1 : 0;
    }
    hipError_t e = hipMemset(ws, 0, kHeaderBytes);
    if (e == hipSuccess)
        e = hipMemcpy(static_cast<uint8_t*>(ws) + kHeaderBytes, table.data(), (size_t)n * sizeof(StepOp),
                      hipMemcpyHostToDevice);
    if (e != hipSuccess) return fail(MNB_E_HIP, "step: writing the projection table: %s", hipGetErrorString(e));
    return MNB_OK;
}

// Workgroups of the step kernel: one per CU, all resident (cooperative).
int step_grid(bool bf16, int* grid) {
    int dev = 0, coop = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return fail(MNB_E_HIP, "step: device attributes: %s", hipGetErrorString(e));
    if (!coop) return fail(MNB_E_UNSUPPORTED, "step: device %d has no cooperative launch", dev);
    e = hipFuncSetAttribute(step_fn(bf16), hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytes);
    if (e != hipSuccess) return fail(MNB_E_HIP, "step: LDS attribute: %s", hipGetErrorString(e));
    int per_cu = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, step_fn(bf16), kThreads, kLdsBytes);
    if (e != hipSuccess) return fail(MNB_E_HIP, "step: occupancy: %s", hipGetErrorString(e));
    if (per_cu < 1) return fail(MNB_E_UNSUPPORTED, "step: the kernel does not fit a CU");
    *grid = cus;
    return MNB_OK;
}

int step_launch(bool bf16, int grid, void* ws, int64_t n, void* trace, hipStream_t s) {
    StepArgs a;
    uint8_t* base = static_cast<uint8_t*>(ws);
    a.ops = (OpTable)(base + kHeaderBytes);
    a.counters = reinterpret_cast<uint32_t*>(base);
    a.done = reinterpret_cast<uint32_t*>(base + kDoneOffset);
    a.error = reinterpret_cast<uint32_t*>(base + kErrorOffset);
    a.n_ops = (int)n;
    a.trace = static_cast<uint64_t*>(trace);
    void* args[] = {&a};
    const hipError_t e = hipLaunchCooperativeKernel(step_fn(bf16), dim3((unsigned)grid), dim3(kThreads), args,
                                                    (unsigned)kLdsBytes, s);
    if (e != hipSuccess) return fail(MNB_E_HIP, "step launch: %s", hipGetErrorString(e));
    return MNB_OK;
}

// Reads (and clears) the error word after the stream has finished.
int step_check(void* ws, hipStream_t s) {
    uint32_t err = 0;
    hipError_t e = hipStreamSynchronize(s);
    if (e == hipSuccess)
        e = hipMemcpy(&err, static_cast<uint8_t*>(ws) + kErrorOffset, sizeof err, hipMemcpyDeviceToHost);
    if (e == hipSuccess && err) e = hipMemset(static_cast<uint8_t*>(ws) + kErrorOffset, 0, sizeof err);
    if (e != hipSuccess) return fail(MNB_E_HIP, "step check: %s", hipGetErrorString(e));
    if (err)
        return fail(MNB_E_HIP, "step: a workgroup stopped waiting for the others (the grid was not co-resident); "
                               "the outputs of that launch are undefined");
    return MNB_OK;
}

}  // namespace mnb
