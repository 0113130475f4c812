// Small M (1 <= M <= 16): Y = A x dequant(B) (+ bias) on the matrix cores.
//
// Page "Qwen3 CPU Inference Critical Path", "INT4 MatMul is first": short
// speculative blocks of a few rows (int4_small_m) sit between the decode GEMV
// and the prefill GEMM; the weights dominate the traffic, so each weight byte
// is still read once and unpacked once, and all rows share the unpacked
// values.
//
// Mapping on CDNA4.  One v_mfma_f32_16x16x32_bf16 multiplies 16 rows of A (rows
// past M are zeros) by 32 K values of 16 columns (a "column group").  K is cut
// into spans of 128 values; wavefront w of a workgroup owns spans w, w + WV,
// ... (P of them) and keeps their activations in registers as MFMA operands.
// The workgroup then walks over column groups (grid-stride, the next groups'
// weights in flight in two register stages).  For a span, lane l = c + 16 g
// reads the 16 packed bytes (32 values, K offset 32 g of the span) of column c
// of the group; a 4 x 4 word transpose across the four 16-lane rows
// (v_permlane32_swap, v_permlane16_swap) gives lane (c, g) word t = values
// 32 t + 8 g .. 32 t + 8 g + 7: exactly the B operand of MFMA t, whose 32
// values all lie in one quantization block (block_size >= 32, K % 32 == 0).
//
// Arithmetic.  The B operand holds the exact integers q - zp (|q - zp| <= 15
// is exact in bf16).  float32 activations are split into a bf16 head and
// tail (a = hi + lo), two MFMAs; bfloat16 activations are one term.  Each
// MFMA starts from zero and its float32 result, one column per lane, is
// folded into the accumulators with that column's block scale:
// acc += s * partial.  The wavefronts' partial sums meet in LDS and are added
// in wavefront order.  P and WV depend only on K, so a column's summation
// order does not depend on N or on the column's position: concatenated
// launches (fused QKV, gate||up) are bit-identical to separate ones.  No
// atomics, no workspace.
#include "mnb_internal.h"

namespace mnb {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kSpan = 128;          // K values per span
constexpr int kMaxWaves = 8;        // wavefronts per workgroup (split K)
constexpr uint32_t kOob = 0x80000000u;    // offset past any resource: reads zero

struct SmallArgs {
    const void* a;
    const uint8_t* b;
    const void* scales;
    const uint8_t* zp;
    const float* bias;
    void* y;
    int M, K, N;
    int col_bytes, nb, zp_row, log2_bs;
    int spans, n_groups;
    uint32_t a_bytes, b_bytes, s_bytes, z_bytes;
};

// The weight loads of one column group over a wavefront's P spans, kept raw
// (decoding here would make the wavefront wait for the loads it just issued).
template <int NG, int P>
struct Stage {
    u32x4 w[NG][P];              // 32 packed values per lane, group and span
    uint32_t s[NG][P][4];        // scale bits of slice t
    uint8_t z[NG][P][4];         // zero-point byte of slice t
    uint32_t bias;               // wavefront u < NG: float32 bits of the bias of
                                 // group u's column c (0 without a bias)
};

// groups gi .. gi + NG - 1 (those past the last read zeros)
template <bool BF16, bool HAS_ZP, int NG, int P>
__device__ __forceinline__ void load_stage(const SmallArgs& g, int64_t gi, int wave, int WV, int lane,
                                           __amdgpu_buffer_rsrc_t rb, __amdgpu_buffer_rsrc_t rs,
                                           __amdgpu_buffer_rsrc_t rz, __amdgpu_buffer_rsrc_t rbias,
                                           Stage<NG, P>& st) {
    constexpr int ESZ = BF16 ? 2 : 4;
    const int c = lane & 15, grp = lane >> 4;
    // the bias goes with the weights: a load issued late and consumed at once
    // would wait for every load in flight (they complete in order)
    {
        const int col = (int)(gi + (wave < NG ? wave : 0)) * 16 + c;
        st.bias = __builtin_amdgcn_raw_buffer_load_b32(rbias, (uint32_t)col * 4u | (col < g.N ? 0u : kOob), 0, 0);
    }
#pragma unroll
    for (int u = 0; u < NG; u++) {
    const int col = (int)(gi + u) * 16 + c;
    const uint32_t c_out = col < g.N ? 0u : kOob;
#pragma unroll
    for (int j = 0; j < P; j++) {
        const int sp = wave + j * WV;
        const uint32_t w_out = (sp * kSpan + 32 * grp < g.K ? 0u : kOob) | c_out;
        st.w[u][j] = __builtin_amdgcn_raw_buffer_load_b128(
            rb, ((uint32_t)col * (uint32_t)g.col_bytes + (uint32_t)(sp * 64 + 16 * grp)) | w_out, 0, 0);
#pragma unroll
        for (int t = 0; t < 4; t++) {
            const int k0 = sp * kSpan + 32 * t;
            const uint32_t out = (k0 < g.K ? 0u : kOob) | c_out;
            const uint32_t blk = (uint32_t)k0 >> g.log2_bs;
            const uint32_t os = (((uint32_t)col * (uint32_t)g.nb + blk) * ESZ) | out;
            st.s[u][j][t] = BF16 ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs, os, 0, 0)
                                 : __builtin_amdgcn_raw_buffer_load_b32(rs, os, 0, 0);
            if constexpr (HAS_ZP)
                st.z[u][j][t] = __builtin_amdgcn_raw_buffer_load_b8(
                    rz, ((uint32_t)col * (uint32_t)g.zp_row + (blk >> 1)) | out, 0, 0);
        }
    }
    }
}

// 4 x 4 transpose of 32-bit words across the four 16-lane rows: afterwards
// row r word t is what row t word r was.
__device__ __forceinline__ void transpose_rows(u32x4& w) {
    const auto p02 = __builtin_amdgcn_permlane32_swap(w[0], w[2], false, false);
    const auto p13 = __builtin_amdgcn_permlane32_swap(w[1], w[3], false, false);
    const auto q01 = __builtin_amdgcn_permlane16_swap(p02[0], p13[0], false, false);
    const auto q23 = __builtin_amdgcn_permlane16_swap(p02[1], p13[1], false, false);
    w = u32x4{q01[0], q01[1], q23[0], q23[1]};
}

template <bool BF16, bool HAS_ZP, int NG, int P>
__global__ __launch_bounds__(64 * kMaxWaves) void smallm_kernel(SmallArgs g) {
    __shared__ f32x4 red[2][NG][kMaxWaves * 64];    // partial sums, two buffers in turn

    const int WV = blockDim.x >> 6;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = lane & 15, grp = lane >> 4;

    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(g.a), (short)0, (int)g.a_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(g.b), (short)0, (int)g.b_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(g.scales), (short)0, (int)g.s_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rz = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(HAS_ZP ? g.zp : g.b), (short)0, (int)(HAS_ZP ? g.z_bytes : 0), 0x00020000);
    const __amdgpu_buffer_rsrc_t rbias = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(g.bias ? g.bias : reinterpret_cast<const float*>(g.b)), (short)0,
        g.bias ? (int)(4 * g.N) : 0, 0x00020000);

    // this wavefront's activations (requested first, so that waiting for them
    // leaves the weights below in flight): row c, values 32 t + 8 g .. + 7 of
    // each of its spans; rows past M and values past K read zeros
    constexpr int ESZ = BF16 ? 2 : 4;
    constexpr int AV = BF16 ? 1 : 2;              // 16-byte pieces per slice
    u32x4 araw[P][4][AV];
#pragma unroll
    for (int j = 0; j < P; j++) {
        const int sp = wave + j * WV;
#pragma unroll
        for (int t = 0; t < 4; t++) {
            const int k0 = sp * kSpan + 32 * t;
            const uint32_t out = k0 < g.K ? 0u : kOob;
            const uint32_t off = ((uint32_t)c * (uint32_t)g.K + (uint32_t)(k0 + 8 * grp)) * ESZ;
#pragma unroll
            for (int v = 0; v < AV; v++)
                araw[j][t][v] = __builtin_amdgcn_raw_buffer_load_b128(ra, (off + 16 * v) | out, 0, 0);
        }
    }
    __builtin_amdgcn_sched_barrier(0);    // keep the activation requests first

    // the first two iterations' weights; an iteration takes NG consecutive
    // column groups.  Every stage is loaded, also past the last group (its
    // loads read zeros): conditional loads would make the compiler wait for
    // all loads in flight wherever the paths meet
    const int64_t stride = (int64_t)gridDim.x * NG;
    int64_t gi = (int64_t)blockIdx.x * NG;
    Stage<NG, P> s0, s1;
    load_stage<BF16, HAS_ZP, NG, P>(g, gi, wave, WV, lane, rb, rs, rz, rbias, s0);
    load_stage<BF16, HAS_ZP, NG, P>(g, gi + stride, wave, WV, lane, rb, rs, rz, rbias, s1);
    __builtin_amdgcn_sched_barrier(0);

    // the activations as MFMA A operands (float32: bf16 head and tail)
    bf16x8 ahi[P][4], alo[P][4];
#pragma unroll
    for (int j = 0; j < P; j++) {
#pragma unroll
        for (int t = 0; t < 4; t++) {
            float v[8];
            if constexpr (BF16) {
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    v[2 * e] = __uint_as_float(araw[j][t][0][e] << 16);
                    v[2 * e + 1] = __uint_as_float(araw[j][t][0][e] & 0xFFFF0000u);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    v[e] = __uint_as_float(araw[j][t][0][e]);
                    v[4 + e] = __uint_as_float(araw[j][t][AV - 1][e]);
                }
            }
#pragma unroll
            for (int e = 0; e < 8; e++) {
                ahi[j][t][e] = (__bf16)v[e];
                if constexpr (!BF16) alo[j][t][e] = (__bf16)(v[e] - (float)ahi[j][t][e]);
            }
        }
    }

    // NG column groups: this wavefront's partial sums over its spans, then
    // the wavefronts' sums meet in LDS buffer `buf`
    auto group = [&](const Stage<NG, P>& st, int64_t gcur, int buf) {
#pragma unroll
        for (int u = 0; u < NG; u++) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < P; j++) {
            const int sp = wave + j * WV;
            u32x4 w = st.w[u][j];
            transpose_rows(w);
#pragma unroll
            for (int t = 0; t < 4; t++) {
                const uint32_t blk = (uint32_t)(sp * kSpan + 32 * t) >> g.log2_bs;
                float zf = 8.f;
                if constexpr (HAS_ZP) zf = (float)__builtin_amdgcn_ubfe((uint32_t)st.z[u][j][t], 4u * (blk & 1u), 4);
                const uint32_t lo = opaque_and(w[t], 0x0F0F0F0Fu);
                const uint32_t hi = opaque_and(w[t] >> 4, 0x0F0F0F0Fu);
                bf16x8 bq;
                bq[0] = (__bf16)(ubyte_to_f32<0>(lo) - zf); bq[1] = (__bf16)(ubyte_to_f32<0>(hi) - zf);
                bq[2] = (__bf16)(ubyte_to_f32<1>(lo) - zf); bq[3] = (__bf16)(ubyte_to_f32<1>(hi) - zf);
                bq[4] = (__bf16)(ubyte_to_f32<2>(lo) - zf); bq[5] = (__bf16)(ubyte_to_f32<2>(hi) - zf);
                bq[6] = (__bf16)(ubyte_to_f32<3>(lo) - zf); bq[7] = (__bf16)(ubyte_to_f32<3>(hi) - zf);
                const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
                f32x4 d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi[j][t], bq, zero, 0, 0, 0);
                if constexpr (!BF16) d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo[j][t], bq, d, 0, 0, 0);
                const float sc = BF16 ? __uint_as_float(st.s[u][j][t] << 16) : __uint_as_float(st.s[u][j][t]);
#pragma unroll
                for (int i = 0; i < 4; i++) acc[i] = fmaf(sc, d[i], acc[i]);
            }
        }
        red[buf][u][wave * 64 + lane] = acc;
        }
        // LDS writes done, then meet (a fenced barrier would also wait for
        // the weight loads in flight)
        __builtin_amdgcn_s_waitcnt(0xC07F);     // lgkmcnt(0)
        asm volatile("s_barrier" : : : "memory");
        // wavefront u < NG adds up group u in wavefront order and stores it:
        // lane (c, g) holds rows 4 g .. 4 g + 3 of column c
        if (wave < NG) {
            // unrolled to the largest team with the missing slots added as
            // +0 (x + 0 == x): a loop here would cost precise waits for the
            // weights in flight
            f32x4 v = red[buf][wave][lane];
#pragma unroll
            for (int w2 = 1; w2 < kMaxWaves; w2++) {
                const f32x4 x = red[buf][wave][w2 * 64 + lane];
                const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
                v += w2 < WV ? x : zero;
            }
            const int col = (int)(gcur + wave) * 16 + c;
            const float bv = __uint_as_float(st.bias);
            if (col < g.N) {
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int m = 4 * grp + i;
                    if (m < g.M) {
                        if constexpr (BF16)
                            static_cast<uint16_t*>(g.y)[(int64_t)m * g.N + col] = f32_to_bf16_rtne(v[i] + bv);
                        else
                            static_cast<float*>(g.y)[(int64_t)m * g.N + col] = v[i] + bv;
                    }
                }
            }
        }
    };

    // gi is workgroup-uniform, so every wavefront reaches every barrier; the
    // two LDS buffers alternate, so one barrier per group suffices (buffer b
    // is rewritten only after the next group's barrier)
    for (; gi < g.n_groups; gi += 2 * stride) {
        group(s0, gi, 0);
        load_stage<BF16, HAS_ZP, NG, P>(g, gi + 2 * stride, wave, WV, lane, rb, rs, rz, rbias, s0);
        __builtin_amdgcn_sched_barrier(0);
        if (gi + stride < g.n_groups) group(s1, gi + stride, 1);
        load_stage<BF16, HAS_ZP, NG, P>(g, gi + 3 * stride, wave, WV, lane, rb, rs, rz, rbias, s1);
        __builtin_amdgcn_sched_barrier(0);
    }
}

using SmallFn = void (*)(SmallArgs);

// spans per wavefront: the activations of P spans stay in registers
constexpr int kMaxP32 = 3, kMaxP16 = 4;

int spans_per_wave(int64_t K) {
    const int64_t spans = (K + kSpan - 1) / kSpan;
    return (int)((spans + kMaxWaves - 1) / kMaxWaves);
}

template <bool BF16, bool HAS_ZP>
SmallFn pick(int P, int NG) {
    (void)NG;
    switch (P) {
        case 1: return smallm_kernel<BF16, HAS_ZP, 1, 1>;
        case 2: return smallm_kernel<BF16, HAS_ZP, 1, 2>;
        case 3: return smallm_kernel<BF16, HAS_ZP, 1, 3>;
        default:
            if constexpr (BF16) return smallm_kernel<BF16, HAS_ZP, 1, 4>;
            return nullptr;
    }
}

int ilog2(int v) {
    int r = 0;
    while ((1 << r) < v) r++;
    return r;
}

// Workgroups of f with `threads` threads resident per CU, cached per thread.
int resident_per_cu(SmallFn f, int threads) {
    struct Entry { SmallFn f; int threads; int n; };
    static thread_local Entry cache[32];
    static thread_local int used = 0;
    for (int i = 0; i < used; i++)
        if (cache[i].f == f && cache[i].threads == threads) return cache[i].n;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(f), threads, 0) !=
            hipSuccess || n < 1)
        n = 1;
    cache[used % 32] = Entry{f, threads, n};
    if (used < 32) used++;
    return n;
}

}  // namespace

bool smallm_ok(const Problem& p) {
    const int esz = p.bf16 ? 2 : 4;
    const int64_t lim = int64_t(1) << 31;
    return p.M >= 1 && p.M <= 16 && p.K % 32 == 0 && p.bs >= 32 &&
           spans_per_wave(p.K) <= (p.bf16 ? kMaxP16 : kMaxP32) &&
           p.M * p.K * esz < lim &&
           p.N * p.col_bytes < lim && (int64_t)p.N * p.nb * esz < lim;
}

int launch_smallm(const Problem& p, hipStream_t s) {
    SmallArgs a;
    a.a = p.a; a.b = p.b; a.scales = p.scales; a.zp = p.has_zp ? p.zp : nullptr;
    a.bias = p.bias; a.y = p.y;
    a.M = (int)p.M; a.K = (int)p.K; a.N = (int)p.N;
    a.col_bytes = (int)p.col_bytes; a.nb = p.nb; a.zp_row = p.zp_row;
    a.log2_bs = ilog2(p.bs);
    a.spans = (int)((p.K + kSpan - 1) / kSpan);
    a.n_groups = (int)((p.N + 15) / 16);
    const int esz = p.bf16 ? 2 : 4;
    a.a_bytes = (uint32_t)(p.M * p.K * esz);
    a.b_bytes = (uint32_t)(p.N * p.col_bytes);
    a.s_bytes = (uint32_t)((int64_t)p.N * p.nb * esz);
    a.z_bytes = p.has_zp ? (uint32_t)((int64_t)p.N * p.zp_row) : 0u;
    // P and WV from K alone (they fix the summation order); the grid only
    // decides which workgroup takes a column group
    const int P = spans_per_wave(p.K);
    const int WV = (a.spans + P - 1) / P;
    // one column group per iteration: more per iteration (more bytes in
    // flight, fewer barriers) measured slower, the larger LDS and register
    // footprint costing more occupancy than it saves
    const int64_t cus = device_compute_units();
    const int ng = 1;
    SmallFn f = p.bf16 ? (p.has_zp ? pick<true, true>(P, ng) : pick<true, false>(P, ng))
                       : (p.has_zp ? pick<false, true>(P, ng) : pick<false, false>(P, ng));
    if (!f) return fail(MNB_E_UNSUPPORTED, "small-M: K=%lld beyond the register kernel", (long long)p.K);
    int64_t blocks = cus * resident_per_cu(f, 64 * WV);
    if (blocks > (a.n_groups + ng - 1) / ng) blocks = (a.n_groups + ng - 1) / ng;
    hipLaunchKernelGGL(f, dim3((unsigned)blocks), dim3(64 * WV), 0, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(MNB_E_HIP, "small-M launch: %s", hipGetErrorString(e));
    return MNB_OK;
}

}  // namespace mnb
