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
// into spans of 128 values (four MFMA slices of 32).  A workgroup of WV
// wavefronts walks over column groups (a "set" each); wavefront w takes spans
// w, w + WV, ... of the group, so each weight byte is read by exactly one
// wavefront.  Each wavefront stages the rows of A for its own spans in LDS,
// already in the MFMA operand layout (float32 activations as a bf16 head and
// tail, a = hi + lo), once for as many spans as fit (a "pass"; longer K is
// staged pass by pass, again for each set), so one staged slice serves every
// column group the workgroup takes and no wavefront waits for another's
// staging.  (Sets of several column groups, sharing each staged slice within
// an item, needed twice the registers, one workgroup per CU, and were slower.)
// Weights stream through two register stages (the next item's loads are in
// flight while one is multiplied), read non-temporally: each byte is read
// once, and streamed past the caches it leaves A resident.  For a span, lane l = c + 16 g reads the 16
// packed bytes (32 values, K offset 32 g of the span) of column c; a 4 x 4
// word transpose across the four 16-lane rows (v_permlane32_swap,
// v_permlane16_swap) gives lane (c, g) word t = values 32 t + 8 g ..
// 32 t + 8 g + 7: exactly the B operand of slice t, whose 32 values all lie
// in one quantization block (block_size >= 32, K % 32 == 0).  The wavefronts'
// partial sums of a set meet in LDS once, at the end of the set.
//
// Arithmetic.  The B operand holds the exact integers q - zp (|q - zp| <= 15
// is exact in bf16).  Each slice's MFMA (two for float32: head, then tail)
// starts from zero and its float32 result, one column per lane, is folded
// into the accumulators with that column's block scale: acc += s * partial,
// slice by slice in K order within a wavefront; the WV wavefront sums are
// then added in wavefront order.  WV depends only on K, so a column's
// summation order does not depend on N or on the column's position:
// concatenated launches (fused QKV, gate||up) are bit-identical to separate
// ones.  With one nonzero activation the result is float32((q - zp) * s)
// exactly.  No atomics, no workspace.

#include "mnb_internal.h"

namespace mnb {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kSpan = 128;                  // K values per span
constexpr int kMaxWV = 8;                   // wavefronts per workgroup
constexpr int kStageMax = 128 * 1024;       // LDS for staged activations
static_assert(kStageMax / (256 * 16 * 2) >= kMaxWV, "a pass holds at least one span per wavefront");
constexpr uint32_t kOob = 0x80000000u;      // offset past any resource: reads zero
constexpr int kNonTemporal = 2;             // cache policy of the weight loads: each byte is read once

struct SmallArgs {
    const void* a;
    const uint8_t* b;
    const void* scales;
    const uint8_t* zp;
    const float* bias;
    void* y;
    int M, K, N;
    int col_bytes, nb, zp_row, log2_bs;
    int spans;              // ceil(K / 128)
    int n_sets;             // column groups: ceil(N / 16)
    int pass_spans;         // spans staged per pass, a multiple of WV
    int passes;             // ceil(spans / pass_spans)
    int ipw;                // items per wavefront per set: ceil(spans / WV)
    int ipp;                // items per wavefront per pass: pass_spans / WV
    int log2_mr;            // rows of A staged: 8 (M <= 8) or 16
    uint32_t a_bytes, b_bytes, s_bytes, z_bytes;
};

// NSB distinct scale blocks per span (4 for 32-value blocks, 2 for 64, 1 for
// larger), NZB zero-point bytes per span (two blocks per byte).  With SV the
// NSB scales of a span are one aligned vector load and its zero-point bytes
// one load (nb a multiple of NSB); otherwise one load each.
template <int NSB>
struct Item {
    static constexpr int NZB = (NSB + 1) / 2;
    u32x4 w;                 // 32 packed values per lane
    uint32_t s[NSB];         // scale bits
    uint32_t z[NZB];         // zero-point bytes
    uint32_t bias;           // float32 bits of the bias of column c
};

struct Res {
    __amdgpu_buffer_rsrc_t a, b, s, z, bias;
};

// Where item f of a wavefront lies: set r of the workgroup (f / ipw), item i
// of the set (f % ipw), and for staged passes the pass and the item within it
// (i / ipp, i % ipp).  Items are visited in order, so the position advances
// by counting (wavefront-uniform scalar operations, no divisions).
struct Pos {
    int r, i, pass, ip;
};

__device__ __forceinline__ void advance(const SmallArgs& g, Pos& p) {
    p.i++;
    p.ip++;
    if (p.ip == g.ipp) {
        p.ip = 0;
        p.pass++;
    }
    if (p.i == g.ipw) {
        p.i = 0;
        p.ip = 0;
        p.pass = 0;
        p.r++;
    }
}

// The loads of the item at position p of this wavefront: set p.r of this
// workgroup (a column group), span wave + p.i * WV.  Items past the last
// set or span, values past K and columns past N read zeros (offsets forced
// past the resources), so every lane issues the same loads whatever the
// shape.
template <bool BF16, bool HAS_ZP, int NSB, bool SV>
__device__ __forceinline__ void load_item(const SmallArgs& g, const Res& rr, const Pos& p, int wave, int WV, int lane,
                                          Item<NSB>& it) {
    constexpr int ESZ = BF16 ? 2 : 4;
    constexpr int SPB = 4 / NSB;                 // slices per scale block
    const int c = lane & 15, grp = lane >> 4;
    const int span = wave + p.i * WV;
    const int set = (int)blockIdx.x + p.r * (int)gridDim.x;
    const uint32_t set_out = set < g.n_sets ? 0u : kOob;
    const uint32_t span_out = span < g.spans ? 0u : kOob;
    const int col = set * 16 + c;
    it.bias = __builtin_amdgcn_raw_buffer_load_b32(rr.bias, (uint32_t)col * 4u | set_out | (col < g.N ? 0u : kOob), 0, 0);
    {
        const uint32_t o = (col < g.N ? set_out : kOob) | span_out;
        const uint32_t kw = (span * kSpan + 32 * grp < g.K) ? 0u : kOob;
        it.w = __builtin_amdgcn_raw_buffer_load_b128(
            rr.b, ((uint32_t)col * (uint32_t)g.col_bytes + (uint32_t)(span * 64 + 16 * grp)) | o | kw, 0, kNonTemporal);
        if constexpr (SV) {
            // the span's NSB consecutive scales and NZB consecutive zero-point
            // bytes, each as one load (aligned: nb is a multiple of NSB)
            const int k0 = span * kSpan;
            const uint32_t blk = (uint32_t)k0 >> g.log2_bs;
            const uint32_t os = (((uint32_t)col * (uint32_t)g.nb + blk) * ESZ) | o | (k0 < g.K ? 0u : kOob);
            if constexpr (NSB * ESZ == 16) {
                const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rr.s, os, 0, 0);
#pragma unroll
                for (int b = 0; b < 4; b++) it.s[b] = v[b];
            } else if constexpr (NSB * ESZ == 8) {
                const uint64_t v = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(rr.s, os, 0, 0));
                if constexpr (BF16) {
#pragma unroll
                    for (int b = 0; b < 4; b++) it.s[b] = (uint32_t)(v >> (16 * b)) & 0xFFFFu;
                } else {
                    it.s[0] = (uint32_t)v;
                    it.s[1] = (uint32_t)(v >> 32);
                }
            } else if constexpr (NSB * ESZ == 4) {
                const uint32_t v = __builtin_amdgcn_raw_buffer_load_b32(rr.s, os, 0, 0);
                if constexpr (BF16 && NSB == 2) {
                    it.s[0] = v & 0xFFFFu;
                    it.s[1] = v >> 16;
                } else {
                    it.s[0] = v;
                }
            } else {
                it.s[0] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rr.s, os, 0, 0);
            }
            if constexpr (HAS_ZP) {
                const uint32_t oz = ((uint32_t)col * (uint32_t)g.zp_row + (blk >> 1)) | o | (k0 < g.K ? 0u : kOob);
                if constexpr (Item<NSB>::NZB == 2) {
                    const uint32_t v = __builtin_amdgcn_raw_buffer_load_b16(rr.z, oz, 0, 0);
                    it.z[0] = v & 0xFFu;
                    it.z[1] = v >> 8;
                } else {
                    it.z[0] = __builtin_amdgcn_raw_buffer_load_b8(rr.z, oz, 0, 0);
                }
            }
        } else {
#pragma unroll
            for (int b = 0; b < NSB; b++) {
                const int k0 = span * kSpan + 32 * SPB * b;
                const uint32_t blk = (uint32_t)k0 >> g.log2_bs;
                const uint32_t os = (((uint32_t)col * (uint32_t)g.nb + blk) * ESZ) | o | (k0 < g.K ? 0u : kOob);
                it.s[b] = BF16 ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rr.s, os, 0, 0)
                                  : __builtin_amdgcn_raw_buffer_load_b32(rr.s, os, 0, 0);
            }
            if constexpr (HAS_ZP) {
#pragma unroll
                for (int b = 0; b < Item<NSB>::NZB; b++) {
                    const int k0 = span * kSpan + 64 * SPB * b;
                    const uint32_t blk = (uint32_t)k0 >> g.log2_bs;
                    it.z[b] = __builtin_amdgcn_raw_buffer_load_b8(
                        rr.z, ((uint32_t)col * (uint32_t)g.zp_row + (blk >> 1)) | o | (k0 < g.K ? 0u : kOob), 0, 0);
                }
            }
        }
    }
}

// bf16(a) in the low half and bf16(b) in the high half (round to nearest
// even; exact here: the values are small integers).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16_pair(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
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

// Activations in LDS: for the first mr rows of A (8 when M <= 8, else 16),
// slice j (32 values) of a pass at hi[(j * 4 + g) * mr + row] (and lo): values
// 8 g .. 8 g + 7 of the slice for that row, the A operand of MFMA lane
// row + 16 g; rows past M and values past K are zeros (rows past mr are not
// staged: their lanes read row c mod mr, and their products land in output
// rows that are never stored).

// One piece (8 values of a row) as the bf16 head h and, for float32
// activations, the bf16 tail t = bf16(a - h).
template <bool BF16>
__device__ __forceinline__ void convert_piece(const u32x4 (&x)[BF16 ? 1 : 2], u32x4& hv, u32x4& tv) {
    float v[8];
    if constexpr (BF16) {
#pragma unroll
        for (int e = 0; e < 4; e++) {
            v[2 * e] = __uint_as_float(x[0][e] << 16);
            v[2 * e + 1] = __uint_as_float(x[0][e] & 0xFFFF0000u);
        }
    } else {
#pragma unroll
        for (int e = 0; e < 4; e++) {
            v[e] = __uint_as_float(x[0][e]);
            v[4 + e] = __uint_as_float(x[1][e]);
        }
    }
    bf16x8 h, t;
#pragma unroll
    for (int e = 0; e < 8; e++) {
        h[e] = (__bf16)v[e];
        if constexpr (!BF16) t[e] = (__bf16)(v[e] - (float)h[e]);
    }
    hv = __builtin_bit_cast(u32x4, h);
    if constexpr (!BF16) tv = __builtin_bit_cast(u32x4, t);
}

// Each wavefront stages only the spans it multiplies (w, w + WV, ...) of a
// pass, into their places of the layout above, so no other wavefront waits
// for it and none overwrites it.  Of its items i0, i0 + 1, ... (spans
// w + i WV), lane l takes pieces q = 0 .. nq - 1 of the list: item
// i0 + q / P, piece j = (q % P) * 64 + l of that span's 16 mr in row order
// (row j / 16, values 8 (j % 16) .. 8 (j % 16) + 7 of the span), so that 16
// lanes read one row's span contiguously; P = mr / 4 pieces per lane and
// span.  Only the pieces of the list are requested, up to U at a time (8 for
// the first pass, which covers a pass of up to four spans per wavefront at 8
// rows; 4 for later passes, staged while both register stages of weights are
// live).
template <bool BF16, int U>
struct OwnRegs {
    u32x4 x[U][BF16 ? 1 : 2];
};

struct OwnList {
    int i0;         // first item of the list
    int base;       // first span of the pass (its LDS position 0)
    int nq;         // pieces per lane
};

// Staged index (LDS position) and source of piece q of the list.
__device__ __forceinline__ void own_piece(const SmallArgs& g, int wave, int WV, int lane, const OwnList& o, int q,
                                          int& idx, int& row, int& k0) {
    const int l2p = g.log2_mr - 2;
    const int span = wave + (o.i0 + (q >> l2p)) * WV;
    const int j = ((q & ((1 << l2p) - 1)) << 6) + lane;
    row = j >> 4;
    k0 = span * kSpan + 8 * (j & 15);
    idx = ((span - o.base) << (g.log2_mr + 4)) + ((j & 15) << g.log2_mr) + row;
}

template <bool BF16, int U>
__device__ __forceinline__ void own_issue(const SmallArgs& g, const Res& rr, int wave, int WV, int lane,
                                          const OwnList& o, int q0, OwnRegs<BF16, U>& st) {
    constexpr int ESZ = BF16 ? 2 : 4;
#pragma unroll
    for (int j = 0; j < U; j++) {
        if (q0 + j < o.nq) {
            int idx, row, k0;
            own_piece(g, wave, WV, lane, o, q0 + j, idx, row, k0);
            const uint32_t out = (row < g.M && k0 < g.K) ? 0u : kOob;
            const uint32_t off = (((uint32_t)row * (uint32_t)g.K + (uint32_t)k0) * ESZ) | out;
#pragma unroll
            for (int v = 0; v < (BF16 ? 1 : 2); v++)
                st.x[j][v] = __builtin_amdgcn_raw_buffer_load_b128(rr.a, off + 16 * v, 0, 0);
        }
    }
}

template <bool BF16, int U>
__device__ __forceinline__ void own_finish(const SmallArgs& g, int wave, int WV, int lane, const OwnList& o, int q0,
                                           const OwnRegs<BF16, U>& st, u32x4* hi, u32x4* lo) {
#pragma unroll
    for (int j = 0; j < U; j++) {
        if (q0 + j < o.nq) {
            int idx, row, k0;
            own_piece(g, wave, WV, lane, o, q0 + j, idx, row, k0);
            u32x4 h, t;
            convert_piece<BF16>(st.x[j], h, t);
            hi[idx] = h;
            if constexpr (!BF16) lo[idx] = t;
        }
    }
}

// The list of pass `pass` of this wavefront: its items pass * ipp .. below
// (pass + 1) * ipp whose spans lie below K.
__device__ __forceinline__ OwnList own_list(const SmallArgs& g, int wave, int WV, int pass) {
    const int own = (g.spans - wave + WV - 1) / WV;      // items with a span below K
    const int i0 = pass * g.ipp;
    const int i1 = i0 + g.ipp < own ? i0 + g.ipp : own;
    return OwnList{i0, pass * g.pass_spans, (i1 > i0 ? i1 - i0 : 0) << (g.log2_mr - 2)};
}

// Stages pieces q0 .. of the list, U at a time.
template <bool BF16, int U>
__device__ __forceinline__ void own_stage(const SmallArgs& g, const Res& rr, int wave, int WV, int lane,
                                          const OwnList& o, int q0, u32x4* hi, u32x4* lo) {
    for (; q0 < o.nq; q0 += U) {
        OwnRegs<BF16, U> st;
        own_issue<BF16, U>(g, rr, wave, WV, lane, o, q0, st);
        own_finish<BF16, U>(g, wave, WV, lane, o, q0, st, hi, lo);
    }
}

// MP: K takes several passes (a separate instance, so that the single-pass
// loop carries no staging code: its register use and waits stay lean).
template <bool BF16, bool HAS_ZP, int NSB, bool SV, bool MP>
__global__ __launch_bounds__(64 * kMaxWV) void smallm_kernel(SmallArgs g) {
    extern __shared__ __attribute__((aligned(16))) u32x4 lds[];
    const int WV = blockDim.x >> 6;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = lane & 15, grp = lane >> 4;
    const int mr = 1 << g.log2_mr;
    const int pieces = (g.pass_spans * 16) << g.log2_mr;    // staged 16-byte pieces per term
    u32x4* hi = lds;
    u32x4* lo = lds + pieces;
    f32x4* red = reinterpret_cast<f32x4*>(lds + pieces * (BF16 ? 1 : 2));   // [WV][64]

    Res rr;
    rr.a = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(g.a), (short)0, (int)g.a_bytes, 0x00020000);
    rr.b = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(g.b), (short)0, (int)g.b_bytes, 0x00020000);
    rr.s = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(g.scales), (short)0, (int)g.s_bytes, 0x00020000);
    rr.z = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(HAS_ZP ? g.zp : g.b), (short)0,
                                             (int)(HAS_ZP ? g.z_bytes : 0), 0x00020000);
    rr.bias = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(g.bias ? g.bias : reinterpret_cast<const float*>(g.b)), (short)0,
        g.bias ? (int)(4 * g.N) : 0, 0x00020000);

    // this workgroup's sets and items (workgroup-uniform)
    const int my_sets = (int)blockIdx.x < g.n_sets ? (g.n_sets - 1 - (int)blockIdx.x) / (int)gridDim.x + 1 : 0;
    const int total = my_sets * g.ipw;

    // the positions of the next item to multiply and of the next to request
    Pos ps{0, 0, 0, 0};
    Pos pl = ps;

    // The first pass of this wavefront's own spans: its first pieces are
    // requested before the first item's weights and converted after (loads
    // complete in order: the weights stay in flight while A is written); the
    // second item's weights follow (both at once could exceed the 63 loads
    // the wait counter tracks).  A wavefront reads only what it wrote, so
    // waiting for its own LDS writes is enough.
    Item<NSB> s0, s1;
    {
        constexpr int U = 8;
        const OwnList o = own_list(g, wave, WV, 0);
        OwnRegs<BF16, U> st;
        own_issue<BF16, U>(g, rr, wave, WV, lane, o, 0, st);
        load_item<BF16, HAS_ZP, NSB, SV>(g, rr, pl, wave, WV, lane, s0);
        advance(g, pl);
        own_finish<BF16, U>(g, wave, WV, lane, o, 0, st, hi, lo);
        own_stage<BF16, U>(g, rr, wave, WV, lane, o, U, hi, lo);
        load_item<BF16, HAS_ZP, NSB, SV>(g, rr, pl, wave, WV, lane, s1);
        advance(g, pl);
        __builtin_amdgcn_s_waitcnt(0xC07F);
    }
    __builtin_amdgcn_sched_barrier(0);

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};

    auto step = [&](const Item<NSB>& it, const Pos& p) {
        const int r = p.r;
        const int i = p.i;
        // the first item of a later pass (or the first pass of a later set):
        // this wavefront restages its own spans of that pass (this waits for
        // the weights in flight too); no other wavefront reads them
        if constexpr (MP) {
            if (p.ip == 0 && (p.pass > 0 || r > 0)) {
                own_stage<BF16, 4>(g, rr, wave, WV, lane, own_list(g, wave, WV, p.pass), 0, hi, lo);
                __builtin_amdgcn_s_waitcnt(0xC07F);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        const int span = wave + i * WV;
        if (span < g.spans) {
            const int ls = (span - p.pass * g.pass_spans) * 4;     // its first slice in LDS
            // lanes of rows past mr read staged row c mod mr: MFMA output
            // rows depend only on their own A rows, so those products land
            // in rows >= mr, which are never stored
            const int pos = grp * mr + (c & (mr - 1));
            bf16x8 ah[4], al[4];
#pragma unroll
            for (int t = 0; t < 4; t++) {
                ah[t] = __builtin_bit_cast(bf16x8, hi[(ls + t) * 4 * mr + pos]);
                if constexpr (!BF16) al[t] = __builtin_bit_cast(bf16x8, lo[(ls + t) * 4 * mr + pos]);
            }
            u32x4 w = it.w;
            transpose_rows(w);
#pragma unroll
            for (int t = 0; t < 4; t++) {
                constexpr int SPB = 4 / NSB;
                const int b = t / SPB;
                float zf = 8.f;
                if constexpr (HAS_ZP) {
                    const uint32_t blk = (uint32_t)(span * kSpan + 32 * t) >> g.log2_bs;
                    constexpr int NZB = Item<NSB>::NZB;
                    zf = (float)__builtin_amdgcn_ubfe(it.z[b / 2 < NZB ? b / 2 : 0], 4u * (blk & 1u), 4);
                }
                const uint32_t lo4 = opaque_and(w[t], 0x0F0F0F0Fu);
                const uint32_t hi4 = opaque_and(w[t] >> 4, 0x0F0F0F0Fu);
                // values 2e and 2e + 1 (byte e, low then high nibble) as one
                // packed conversion each
                const bf16x8 bq = __builtin_bit_cast(
                    bf16x8, u32x4{bf16_pair(ubyte_to_f32<0>(lo4) - zf, ubyte_to_f32<0>(hi4) - zf),
                                  bf16_pair(ubyte_to_f32<1>(lo4) - zf, ubyte_to_f32<1>(hi4) - zf),
                                  bf16_pair(ubyte_to_f32<2>(lo4) - zf, ubyte_to_f32<2>(hi4) - zf),
                                  bf16_pair(ubyte_to_f32<3>(lo4) - zf, ubyte_to_f32<3>(hi4) - zf)});
                const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
                f32x4 d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[t], bq, zero, 0, 0, 0);
                if constexpr (!BF16) d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[t], bq, d, 0, 0, 0);
                const float sc = BF16 ? __uint_as_float(it.s[b] << 16) : __uint_as_float(it.s[b]);
#pragma unroll
                for (int e = 0; e < 4; e++) acc[e] = fmaf(sc, d[e], acc[e]);
            }
        }
        // the end of a set: the wavefronts' sums meet in LDS (in wavefront
        // order) and wavefront 0 stores them; the first barrier keeps the
        // buffer from being rewritten while the previous set is read
        if (i == g.ipw - 1) {
            asm volatile("s_barrier" : : : "memory");
            red[wave * 64 + lane] = acc;
            acc = f32x4{0.f, 0.f, 0.f, 0.f};
            __builtin_amdgcn_s_waitcnt(0xC07F);
            asm volatile("s_barrier" : : : "memory");
            if (wave == 0) {
                f32x4 v = red[lane];
                // unrolled to the largest workgroup, the missing wavefronts
                // adding +0 (x + 0 == x): a loop would cost precise waits for
                // the weights in flight
#pragma unroll
                for (int w2 = 1; w2 < kMaxWV; w2++) {
                    const f32x4 x = red[(w2 < WV ? w2 : 0) * 64 + lane];
                    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
                    v += w2 < WV ? x : zero;
                }
                const int set = (int)blockIdx.x + r * (int)gridDim.x;
                const int col = set * 16 + c;
                const float bv = __uint_as_float(it.bias);
                if (col < g.N) {
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        const int m = 4 * grp + e;
                        if (m < g.M) {
                            if constexpr (BF16)
                                static_cast<uint16_t*>(g.y)[(int64_t)m * g.N + col] = f32_to_bf16_rtne(v[e] + bv);
                            else
                                static_cast<float*>(g.y)[(int64_t)m * g.N + col] = v[e] + bv;
                        }
                    }
                }
            }
        }
    };

    // f is workgroup-uniform, so every wavefront reaches every barrier
    for (int f = 0; f < total; f += 2) {
        step(s0, ps);
        advance(g, ps);
        load_item<BF16, HAS_ZP, NSB, SV>(g, rr, pl, wave, WV, lane, s0);
        advance(g, pl);
        __builtin_amdgcn_sched_barrier(0);
        if (f + 1 < total) step(s1, ps);
        advance(g, ps);
        load_item<BF16, HAS_ZP, NSB, SV>(g, rr, pl, wave, WV, lane, s1);
        advance(g, pl);
        __builtin_amdgcn_sched_barrier(0);
    }
}

using SmallFn = void (*)(SmallArgs);

template <bool BF16, bool HAS_ZP, bool SV, bool MP>
SmallFn pick_nsb(int nsb) {
    switch (nsb) {
        case 4: return smallm_kernel<BF16, HAS_ZP, 4, SV, MP>;
        case 2: return smallm_kernel<BF16, HAS_ZP, 2, SV, MP>;
        default: return smallm_kernel<BF16, HAS_ZP, 1, SV, MP>;
    }
}

template <bool BF16, bool HAS_ZP>
SmallFn pick(int nsb, bool sv, bool mp) {
    if (mp) return sv ? pick_nsb<BF16, HAS_ZP, true, true>(nsb) : pick_nsb<BF16, HAS_ZP, false, true>(nsb);
    return sv ? pick_nsb<BF16, HAS_ZP, true, false>(nsb) : pick_nsb<BF16, HAS_ZP, false, false>(nsb);
}

int ilog2(int v) {
    int r = 0;
    while ((1 << r) < v) r++;
    return r;
}

// Workgroups of f with `threads` threads and `lds` bytes resident per CU,
// cached per thread; raises f's dynamic LDS limit first.
int resident_per_cu(SmallFn f, int threads, size_t lds) {
    struct Entry { SmallFn f; int threads; size_t lds; int n; };
    static thread_local Entry cache[32];
    static thread_local int used = 0;
    for (int i = 0; i < used; i++)
        if (cache[i].f == f && cache[i].threads == threads && cache[i].lds == lds) return cache[i].n;
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(f), hipFuncAttributeMaxDynamicSharedMemorySize,
                              160 * 1024);
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(f), threads, lds) !=
            hipSuccess || n < 1)
        n = 1;
    (void)hipGetLastError();
    cache[used % 32] = Entry{f, threads, lds, n};
    if (used < 32) used++;
    return n;
}

// Wavefronts per workgroup: a function of K alone (it fixes the summation
// order), one span per wavefront up to eight.
int waves_for(int64_t K) {
    const int64_t spans = (K + kSpan - 1) / kSpan;
    return (int)(spans < kMaxWV ? spans : kMaxWV);
}

}  // namespace

bool smallm_ok(const Problem& p) {
    const int esz = p.bf16 ? 2 : 4;
    const int64_t lim = int64_t(1) << 31;
    return p.M >= 1 && p.M <= 16 && p.K % 32 == 0 && p.bs >= 32 && p.M * p.K * esz < lim &&
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
    const int esz = p.bf16 ? 2 : 4;
    a.a_bytes = (uint32_t)(p.M * p.K * esz);
    a.b_bytes = (uint32_t)(p.N * p.col_bytes);
    a.s_bytes = (uint32_t)((int64_t)p.N * p.nb * esz);
    a.z_bytes = p.has_zp ? (uint32_t)((int64_t)p.N * p.zp_row) : 0u;
    const int WV = waves_for(p.K);
    a.log2_mr = p.M <= 8 ? 3 : 4;
    // passes: as many spans as the staging LDS holds, a multiple of WV
    const int span_bytes = (256 << a.log2_mr) * (p.bf16 ? 1 : 2);
    int ps = (kStageMax / span_bytes) / WV * WV;
    const int need = (a.spans + WV - 1) / WV * WV;
    if (ps > need) ps = need;
    a.pass_spans = ps;
    a.passes = (a.spans + ps - 1) / ps;
    a.ipw = (a.spans + WV - 1) / WV;
    a.ipp = ps / WV;
    // one set per column group; the grid only decides which workgroup takes a
    // set
    const int64_t cus = device_compute_units();
    a.n_sets = (int)((p.N + 15) / 16);
    const int nsb = p.bs >= 128 ? 1 : p.bs == 64 ? 2 : 4;
    // vector scale / zero-point loads when a span's blocks are aligned
    // (scales [N][nb] and zero points [N][ceil(nb/2)] are element-aligned)
    const bool sv = p.nb % nsb == 0 && (nsb < 4 || p.zp_row % 2 == 0);
    const bool mp = a.passes > 1;
    SmallFn f = p.bf16 ? (p.has_zp ? pick<true, true>(nsb, sv, mp) : pick<true, false>(nsb, sv, mp))
                       : (p.has_zp ? pick<false, true>(nsb, sv, mp) : pick<false, false>(nsb, sv, mp));
    const size_t lds = (size_t)ps * span_bytes + (size_t)WV * 64 * 16;
    int64_t blocks = cus * resident_per_cu(f, 64 * WV, lds);
    if (blocks > a.n_sets) blocks = a.n_sets;
    hipLaunchKernelGGL(f, dim3((unsigned)blocks), dim3(64 * WV), lds, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(MNB_E_HIP, "small-M launch: %s", hipGetErrorString(e));
    return MNB_OK;
}

}  // namespace mnb
