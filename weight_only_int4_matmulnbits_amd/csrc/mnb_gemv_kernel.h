// The decode GEMV kernel (M == 1, or up to four rows) and the choice of its
// instance; the launcher is mnb_gemv.hip, and each activation type's
// instances are compiled in a translation unit of their own
// (mnb_gemv_f32.hip, mnb_gemv_bf16.hip).
//
// Decode GEMV (M == 1): y[n] = sum_k a[k] * (q[n][k] - zp[n][b]) * s[n][b] + bias[n].
//
// Page "Qwen3 CPU Inference Critical Path", "INT4 MatMul is first": batch-1
// projections have one activation row and are dominated by weight traffic;
// int4_gemv partitions output columns so every weight byte is streamed once;
// decode unpacks in registers, applies zero point and scale, accumulates in
// float32, and never expands the matrix.
//
// Mapping on CDNA4.  The packed weights are N-major: column n is one run of
// col_bytes contiguous bytes.  A "chunk" is CB = min(16, bs/2) bytes of one
// column (CK = 2*CB values of K, inside one quantization block); a column has
// S = ceil(K / CK) chunks.  A column is handled by a team of W wavefronts
// (split-K across wavefronts, W in {1, 2, 4}) with L lanes each (L a power
// of two <= 64; G = 64 / L columns per wavefront step when W == 1).  Team
// lane p owns chunks p, p + L*W, ..., p + (J-1)*L*W of EVERY column it
// visits; the activations are staged once per workgroup in LDS and the lane
// reads its J*CK of them from there for every column (one chunk ahead of
// its use).  For a fixed column the lanes read
// consecutive chunks: fully coalesced 16-byte-per-lane loads, marked
// non-temporal (each weight byte is read once).
//
// Inner product in float32 on the vector ALU, about 2.1 instructions per
// weight: per 32-bit word (8 nibbles) one shift and four masks build f16
// pairs 1024 + q (1024 + 16 q for odd k), one packed f16 addition or FMA per
// pair leaves the exact integers q - zp, and one mixed-precision FMA (f16
// weight, float32 activation and sum) per weight accumulates.  Per chunk a lane forms
// t = sum a_k (q_k - zp), then acc += s * t; a weight equal to its zero point
// adds exactly nothing.  The L partial sums of a wavefront meet in a fixed
// all-DPP tree; the W wavefront sums meet in LDS in wavefront order.  Grid
// size, unroll and prefetch only change which wavefront handles a column,
// never the arithmetic: (L, J, W) depend only on (K, block_size), so the
// float32 summation order of a column is the same whatever N is and wherever
// the column sits -- concatenated launches (fused QKV, gate||up) are
// bit-identical to separate ones.  No atomics, no workspace.
#pragma once

#include "mnb_gemv_core.h"

namespace mnb {

constexpr int kGemvWavesPerBlock = 4;
constexpr size_t kGemvMaxLds = 64 * 1024;    // staged activations per workgroup

struct GemvArgs {
    const void* a;
    const uint8_t* b;
    const void* scales;
    const uint8_t* zp;
    const float* bias;
    void* y;
    int64_t K, N, col_bytes, n_groups;
    int nb, zp_row, S, log2_bs, log2_L;
    int a16;                  // K * element size is a multiple of 16 and A is 16-byte aligned
    int64_t half;             // gated epilogue: columns per half (gate | up); 0 otherwise
    int M;                    // rows of A and Y (1 for the decode GEMV; up to MR)
    const void* gamma;        // RMSNorm fused into the input (one row): gamma [K], or NULL
    float eps;
};

using GemvFn = void (*)(GemvArgs);

// How the one-row kernel takes its activations: read from the staged row in
// LDS chunk by chunk where a lane holds several chunks (else registers; a
// form with a single register stage, for grids that give every team at
// most one column group), held in registers for all columns, or held in
// registers RMS-normalized.
enum GemvInput { kInputLds = 0, kInputRegs = 1, kInputRms = 2, kInputLdsOne = 3 };

// The kernel for one activation type (defined once per type, in
// mnb_gemv_f32.hip and mnb_gemv_bf16.hip): one row (silu: gated gate||up;
// input: a GemvInput) or MR rows; nullptr where no kernel has that shape.
// nts: scales, zero points and bias read non-temporally.
GemvFn gemv_pick_f32(bool has_zp, bool has_bias, int CB, int J, int W, bool silu, int input, bool nts);
GemvFn gemv_pick_bf16(bool has_zp, bool has_bias, int CB, int J, int W, bool silu, int input, bool nts);
GemvFn gemv_pick_rows_f32(bool has_zp, bool has_bias, int MR, int J, int W, bool nts);
GemvFn gemv_pick_rows_bf16(bool has_zp, bool has_bias, int MR, int J, int W, bool nts);

namespace {

constexpr int kWavesPerBlock = kGemvWavesPerBlock;

// The same for MR rows of activations: each weight is unpacked once and
// multiplied into every row (per row the additions are those of dot_words).
template <int NW, int MR>
__device__ __forceinline__ void dot_words_rows(const uint32_t (&w)[NW], const float (*av)[32], uint32_t ze,
                                               uint32_t zo, const NibbleMasks& k, float (&out)[MR]) {
    float de[MR], dd[MR];
#pragma unroll
    for (int r = 0; r < MR; r++) de[r] = dd[r] = 0.f;
#pragma unroll
    for (int d = 0; d < NW; d++) {
        const uint32_t w8 = w[d] >> 8;
        const half2_t p0 = nibble_pair(w[d], k.lo, k.magic, ze);
        const half2_t p1 = nibble_pair_hi(w[d], k.hi, k.magic, zo);
        const half2_t p2 = nibble_pair(w8, k.lo, k.magic, ze);
        const half2_t p3 = nibble_pair_hi(w8, k.hi, k.magic, zo);
        const float q[8] = {(float)p0[0], (float)p1[0], (float)p2[0], (float)p3[0],
                            (float)p0[1], (float)p1[1], (float)p2[1], (float)p3[1]};
#pragma unroll
        for (int e = 0; e < 8; e += 2)
#pragma unroll
            for (int r = 0; r < MR; r++) {
                de[r] = fmaf(av[r][8 * d + e], q[e], de[r]);
                dd[r] = fmaf(av[r][8 * d + e + 1], q[e + 1], dd[r]);
            }
    }
#pragma unroll
    for (int r = 0; r < MR; r++) out[r] = de[r] + dd[r];
}


// One iteration's loads, kept raw: decoding a scale or a zero-point nibble
// here would make the wavefront wait for the load it just issued.
template <bool BF16, bool HAS_ZP, int CB, int J>
struct Group {
    using Chunk = typename ChunkT<CB>::type;
    Chunk w[J];
    uint32_t sc[J];      // float32 bits, or bfloat16 bits in the low half
    uint32_t zb[J];      // packed zero-point byte (HAS_ZP)
    uint32_t bias;       // float32 bits of the column's bias (0 without one)
};

// One iteration's loads through buffer resources based at the group's
// first column: every load is issued (a chunk past K or a column past N reads
// zeros, which contribute nothing), so a wavefront issues the same number of
// memory instructions on every path (kOob: an offset past any resource).

// Column group gi of the `width` columns starting at column col_off (the
// whole of B, or the gate or the up half of a gated gate||up weight).
template <bool BF16, bool HAS_ZP, bool HAS_BIAS, int CB, int J, bool NTS>
__device__ __forceinline__ void load_group(const GemvArgs& g, int64_t gi, int64_t col_off, int64_t width, int p,
                                           int LT, int G, int gsub, Group<BF16, HAS_ZP, CB, J>& r) {
    constexpr int CK = 2 * CB;
    constexpr int SSZ = BF16 ? 2 : 4;
    constexpr int kSmallPolicy = NTS ? kNonTemporal : 0;
    const int64_t col0 = col_off + gi * G;
    const int64_t ncol = gi < g.n_groups ? (width - gi * G < G ? width - gi * G : G) : 0;
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(g.b) + (ncol ? col0 * g.col_bytes : 0), (short)0,
        (int)(ncol * g.col_bytes), 0x00020000);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        static_cast<uint8_t*>(const_cast<void*>(g.scales)) + (ncol ? col0 * g.nb * SSZ : 0), (short)0,
        (int)(ncol * g.nb * SSZ), 0x00020000);
    // the bias goes with the weights: a load issued late and consumed at
    // once would wait for every load in flight (they complete in order)
    const __amdgpu_buffer_rsrc_t rbias = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(g.bias ? g.bias : reinterpret_cast<const float*>(g.b)) + (ncol && g.bias ? col0 : 0),
        (short)0, g.bias ? (int)(ncol * 4) : 0, 0x00020000);
    r.bias = HAS_BIAS ? __builtin_amdgcn_raw_buffer_load_b32(rbias, (uint32_t)(4 * gsub), 0, kSmallPolicy) : 0u;
    __amdgpu_buffer_rsrc_t rz;
    if constexpr (HAS_ZP)
        rz = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(g.zp) + (ncol ? col0 * g.zp_row : 0),
                                               (short)0, (int)(ncol * g.zp_row), 0x00020000);
    // scales and zero points first: loads complete in order, so they are in
    // registers by the time the weights arrive
#pragma unroll
    for (int j = 0; j < J; j++) {
        const int c = p + j * LT;
        // offsets of chunks past K forced past the resource (branch-free, so
        // that every lane issues the same single load)
        const uint32_t out = c < g.S ? 0u : kOob;
        const int blk = (c * CK) >> g.log2_bs;
        const uint32_t os = (uint32_t)((gsub * g.nb + blk) * SSZ) | out;
        r.sc[j] = BF16 ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs, os, 0, kSmallPolicy)
                       : __builtin_amdgcn_raw_buffer_load_b32(rs, os, 0, kSmallPolicy);
        if constexpr (HAS_ZP)
            r.zb[j] = __builtin_amdgcn_raw_buffer_load_b8(rz, (uint32_t)(gsub * g.zp_row + (blk >> 1)) | out, 0,
                                                          kSmallPolicy);
    }
#pragma unroll
    for (int j = 0; j < J; j++) {
        const int c = p + j * LT;
        const uint32_t out = c < g.S ? 0u : kOob;
        const uint32_t ow = (uint32_t)(gsub * g.col_bytes + c * CB) | out;
        if constexpr (CB == 16) {
            r.w[j] = __builtin_amdgcn_raw_buffer_load_b128(rb, ow, 0, kNonTemporal);
        } else {
            const uint64_t x =
                __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(rb, ow, 0, kNonTemporal));
            r.w[j] = u32x2{(uint32_t)x, (uint32_t)(x >> 32)};
        }
    }
}

// W wavefronts per column team, one column group per team per iteration.
// SILU: the gate||up projection with the gated product fused into the
// epilogue (page "Qwen3 CPU Inference Critical Path", "Phase Q5: scheduling
// and fusion": the gate projection, its SiLU and the gate/up product as one
// fusion): the two register stages hold column group g of the gate half and
// the same group of the up half; both go through exactly the geometry and
// arithmetic of unfused columns (the sums are those mnb_gemv computes), and h
// = silu(gate) * up is written for the gate columns only.
// MR > 1: rows 0 .. M - 1 of A (M <= MR; the rows past M read zeros) with
// one chunk of K per lane (J == 1, or 2 for two rows): every weight byte is
// still read and unpacked once and serves all rows.
// RMS: one row normalized on the fly (gamma staged after A in LDS).
// Activations: one row without RMSNorm and with several chunks per lane
// (ACTL) reads each chunk's values from the staged copy in LDS as the chunk
// is reduced, one chunk ahead of its use, which leaves room for more
// resident wavefronts (144 instead of 236 VGPRs at five float32 chunks per
// lane).  The row kernel, RMS (normalized once), one chunk per lane (no next
// chunk to read ahead, and few registers anyway) and REGS (launches with
// many column groups per team, where the LDS reads would repeat for every
// group) hold the lane's chunks in registers for all columns.
// ONE: the LDS-reading kernel on a grid that gives every team at most one
// column group: no second register stage (90 instead of 144 VGPRs at five
// float32 chunks per lane, five workgroups per CU instead of three).
template <bool BF16, bool HAS_ZP, bool HAS_BIAS, int CB, int J, int W, bool SILU, int MR, bool NTS, bool RMS,
          bool REGS, bool ONE>
__global__ __launch_bounds__(64 * kWavesPerBlock) void gemv_kernel(GemvArgs g) {
    constexpr int CK = 2 * CB;        // values of K per chunk
    constexpr int NW = CB / 4;        // 32-bit words per chunk
    constexpr int TEAMS = kWavesPerBlock / W;
    static_assert(MR == 1 || (!SILU && J * MR <= 4 && CB == 16), "row kernel: <= 4 row chunks");
    static_assert(!RMS || (MR == 1 && !SILU), "RMSNorm: one row, plain epilogue");
    static_assert(!REGS || (MR == 1 && !SILU && !RMS && J > 1), "register input: the plain one-row kernel");
    constexpr bool ACTL = MR == 1 && !RMS && !REGS && J > 1;
    static_assert(!ONE || (ACTL && !SILU), "one group per team: the plain LDS-reading kernel");
    __shared__ float red[kWavesPerBlock * MR];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int team = wave / W;
    const int wt = wave - team * W;   // wavefront index within the team
    const int L = 1 << g.log2_L;      // lanes per column in one wavefront
    const int LT = L * W;             // lanes per column in the team
    const int p = wt * L + (lane & (L - 1));
    const int G = 64 >> g.log2_L;
    const int gsub = lane >> g.log2_L;

    // iteration space: WG-uniform, so barriers (W > 1) are reached by all
    const int64_t stride = (int64_t)gridDim.x * TEAMS;
    int64_t base = (int64_t)blockIdx.x * TEAMS + team;
    const int64_t team0 = (int64_t)blockIdx.x * TEAMS;
    // the columns the groups index: all of B, or (gated) each half
    const int64_t width = SILU ? g.half : g.N;

    // ---- activations: staged once per workgroup in LDS as they are (float32
    // or bfloat16), one RB-byte row per chunk; the 16-byte pieces of row c sit
    // at v ^ ((c / (256 / RB)) % NV), so that the per-lane 16-byte reads of 16
    // consecutive rows below cover all 64 banks once.  The requests go out
    // before the weights': loads complete in order, so activations queued
    // behind HBM weight loads would be late ----
    constexpr int ESZ = BF16 ? 2 : 4;
    constexpr int RB = CK * ESZ;                 // bytes per chunk row
    constexpr int NV = RB / 16;                  // 16-byte pieces per row
    constexpr int RPS = 256 / RB;                // rows per 256-byte bank sweep
    extern __shared__ __attribute__((aligned(16))) uint8_t a_lds[];
    const int nthr = 64 * kWavesPerBlock;
    const int nreq = (g.S * RB + 1023) / 1024;   // 1 KiB requests per row of A
    if (g.a16) {
        // LDS-direct loads: request r of row m puts 64 pieces (1 KiB) at
        // a_lds + 1024 (m nreq + r); lane l fills chunk row r * 64 / NV + l / NV,
        // position l % NV, with the piece that the swizzle assigns there;
        // reads past K (and rows past M) return zeros
#pragma unroll
        for (int m = 0; m < MR; m++) {
            const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
                static_cast<uint8_t*>(const_cast<void*>(g.a)) + (m < g.M ? (int64_t)m * g.K * ESZ : 0), (short)0,
                m < g.M ? (int)(g.K * ESZ) : 0, 0x00020000);
            for (int r = wave; r < nreq; r += kWavesPerBlock) {
                const int row = r * (64 / NV) + lane / NV;
                const int pos = lane % NV;
                const int piece = pos ^ ((row / RPS) % NV);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    ra, (void __attribute__((address_space(3)))*)(a_lds + 1024 * (m * nreq + r)), 16,
                    (uint32_t)(row * RB + 16 * piece), 0, 0, 0);
            }
        }
        if constexpr (RMS) {
            // the RMSNorm weights, staged like A after it
            const __amdgpu_buffer_rsrc_t rg = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<void*>(g.gamma), (short)0, (int)(g.K * ESZ), 0x00020000);
            for (int r = wave; r < nreq; r += kWavesPerBlock) {
                const int row = r * (64 / NV) + lane / NV;
                const int pos = lane % NV;
                const int piece = pos ^ ((row / RPS) % NV);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rg, (void __attribute__((address_space(3)))*)(a_lds + 1024 * (MR * nreq + r)), 16,
                    (uint32_t)(row * RB + 16 * piece), 0, 0, 0);
            }
        }
    } else {
        // K * element size not a multiple of 16: element-wise loads
        for (int i = threadIdx.x; i < g.S * NV; i += nthr) {
            const int row = i / NV, piece = i % NV;
            const int64_t k0 = (int64_t)row * CK + piece * (16 / ESZ);
            uint32_t w[4];
#pragma unroll
            for (int e = 0; e < 4; e++) {
                if constexpr (BF16) {
                    const int64_t k = k0 + 2 * e;
                    const uint32_t lo = k < g.K ? static_cast<const uint16_t*>(g.a)[k] : 0u;
                    const uint32_t hi = k + 1 < g.K ? static_cast<const uint16_t*>(g.a)[k + 1] : 0u;
                    w[e] = lo | (hi << 16);
                } else {
                    const int64_t k = k0 + e;
                    w[e] = k < g.K ? static_cast<const uint32_t*>(g.a)[k] : 0u;
                }
            }
            *reinterpret_cast<u32x4*>(a_lds + row * RB + 16 * (piece ^ ((row / RPS) % NV))) =
                u32x4{w[0], w[1], w[2], w[3]};
        }
    }

    // the first two stages' weights: the first two iterations (the second
    // only if this team has one), or (gated) the gate and the up group of
    // the first iteration
    Group<BF16, HAS_ZP, CB, J> g0, g1;
    const bool two = !ONE && (SILU || base + stride < g.n_groups);     // wave-uniform
    load_group<BF16, HAS_ZP, HAS_BIAS, CB, J, NTS>(g, base, 0, width, p, LT, G, gsub, g0);
    if constexpr (!ONE) {
        if (two)
            load_group<BF16, HAS_ZP, HAS_BIAS, CB, J, NTS>(g, SILU ? base : base + stride, SILU ? g.half : 0, width,
                                                      p, LT, G, gsub, g1);
    }

    // wait for this wavefront's staging (all memory instructions but the
    // weight loads just issued, and the LDS writes), then meet the others.
    // A plain barrier: a fenced one would also wait for the weights.
    {
        constexpr int NL = J * (HAS_ZP ? 3 : 2) + (HAS_BIAS ? 1 : 0);     // loads per group
        static_assert(2 * NL < 64, "vmcnt range");
        constexpr int W1 = (NL & 15) | (7 << 4) | (0 << 8) | ((NL >> 4) << 14);
        constexpr int W2 = ((2 * NL) & 15) | (7 << 4) | (0 << 8) | (((2 * NL) >> 4) << 14);
        if (two)
            __builtin_amdgcn_s_waitcnt(W2);
        else
            __builtin_amdgcn_s_waitcnt(W1);
        asm volatile("s_barrier" : : : "memory");
    }
    const NibbleMasks nk = nibble_masks();
    // RMSNorm fused into the input (page "Qwen3 CPU Inference Critical
    // Path", "Phase Q5": RMSNorm into the packed projection input; one row):
    // the sum of squares over this lane's chunks -- the team's lanes of a
    // column cover K once -- reduced by the lane tree (and the team's
    // wavefronts in order), then a = (x * r) * gamma with r = 1 / sqrt(mean +
    // eps), all in float32
    const uint8_t* const g_lds = a_lds + 1024 * (MR * nreq);
    float inv_rms = 1.f;
    if constexpr (RMS) {
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < J; j++) {
            const int c = p + j * LT;
            if (c < g.S) {
#pragma unroll
                for (int v = 0; v < NV; v++) {
                    const u32x4 x = *reinterpret_cast<const u32x4*>(a_lds + c * RB + 16 * (v ^ ((c / RPS) % NV)));
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        if constexpr (BF16) {
                            const float x0 = __uint_as_float(x[e] << 16), x1 = __uint_as_float(x[e] & 0xFFFF0000u);
                            ss = fmaf(x0, x0, ss);
                            ss = fmaf(x1, x1, ss);
                        } else {
                            const float x0 = __uint_as_float(x[e]);
                            ss = fmaf(x0, x0, ss);
                        }
                    }
                }
            }
        }
        ss = reduce_lanes(ss, g.log2_L);
        // every lane takes its lane group's sum (held by the group's last lane)
        ss = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((lane | (L - 1)) << 2, __builtin_bit_cast(int, ss)));
        if constexpr (W > 1) {
            if (lane == 63) red[wave] = ss;
            __syncthreads();
            float v = red[team * W];
#pragma unroll
            for (int w2 = 1; w2 < W; w2++) v += red[team * W + w2];
            ss = v;
            __syncthreads();
        }
        inv_rms = 1.0f / sqrtf(ss / (float)g.K + g.eps);
    }
    // this lane's chunks of A in registers, for each row (not with ACTL)
    float av[ACTL ? 1 : MR * J][CK];
#pragma unroll
    for (int mj = 0; mj < (ACTL ? 0 : MR * J); mj++) {          // [chunk j][row m]
        const int j = mj / MR, m = mj % MR;
        const int c = p + j * LT;
        if (c < g.S) {
#pragma unroll
            for (int v = 0; v < NV; v++) {
                const u32x4 x = *reinterpret_cast<const u32x4*>(a_lds + 1024 * m * nreq + c * RB +
                                                                16 * (v ^ ((c / RPS) % NV)));
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    if constexpr (BF16) {
                        av[mj][8 * v + 2 * e] = __uint_as_float(x[e] << 16);
                        av[mj][8 * v + 2 * e + 1] = __uint_as_float(x[e] & 0xFFFF0000u);
                    } else {
                        av[mj][4 * v + e] = __uint_as_float(x[e]);
                    }
                }
                if constexpr (RMS) {
                    const u32x4 gw = *reinterpret_cast<const u32x4*>(g_lds + c * RB + 16 * (v ^ ((c / RPS) % NV)));
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        if constexpr (BF16) {
                            av[mj][8 * v + 2 * e] = (av[mj][8 * v + 2 * e] * inv_rms) * __uint_as_float(gw[e] << 16);
                            av[mj][8 * v + 2 * e + 1] =
                                (av[mj][8 * v + 2 * e + 1] * inv_rms) * __uint_as_float(gw[e] & 0xFFFF0000u);
                        } else {
                            av[mj][4 * v + e] = (av[mj][4 * v + e] * inv_rms) * __uint_as_float(gw[e]);
                        }
                    }
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < CK; i++) av[mj][i] = 0.f;
        }
    }
    // ACTL: chunk c of the row into a1.  A lane past K reads the last chunk
    // (its sum is replaced by zero below).  The opaque chunk index keeps the
    // reads inside the column loop: hoisted out of it, they would hold every
    // chunk in registers again.
    auto act_chunk = [&](int c, float (&a1)[CK]) {
        c = c < g.S ? c : g.S - 1;
        asm volatile("" : "+v"(c));
#pragma unroll
        for (int v = 0; v < NV; v++) {
            const u32x4 x = *reinterpret_cast<const u32x4*>(a_lds + c * RB + 16 * (v ^ ((c / RPS) % NV)));
#pragma unroll
            for (int e = 0; e < 4; e++) {
                if constexpr (BF16) {
                    a1[8 * v + 2 * e] = __uint_as_float(x[e] << 16);
                    a1[8 * v + 2 * e + 1] = __uint_as_float(x[e] & 0xFFFF0000u);
                } else {
                    a1[4 * v + e] = __uint_as_float(x[e]);
                }
            }
        }
    };

    // Two register stages used alternately (copying a stage would make the
    // wavefront wait for the loads just issued into it): while one
    // iteration is reduced, the next one's weights are in flight, and its
    // own stage is refilled with the iteration after.  reduce() leaves the
    // column sums (before the bias) in the last lane of each column's lane
    // group of the team's first wavefront.
    auto reduce = [&](const Group<BF16, HAS_ZP, CB, J>& cur, float (&acc)[MR]) {
        float s[MR];
#pragma unroll
        for (int r = 0; r < MR; r++) s[r] = 0.f;
        float a_buf[2][ACTL ? CK : 1];
        if constexpr (ACTL) act_chunk(p, a_buf[0]);
#pragma unroll
        for (int j = 0; j < J; j++) {
            if constexpr (ACTL) {
                if (j + 1 < J) act_chunk(p + (j + 1) * LT, a_buf[(j + 1) & 1]);
            }
            uint32_t words[NW];
#pragma unroll
            for (int d = 0; d < NW; d++) words[d] = cur.w[j][d];
            uint32_t zq = 8u;
            if constexpr (HAS_ZP) {
                const int blk = ((p + j * LT) * CK) >> g.log2_bs;
                const uint32_t zb = cur.zb[j];
                zq = (blk & 1) ? ((zb >> 4) & 0xFu) : (zb & 0xFu);
            }
            uint32_t ze, zo;
            zero_point_pairs(zq, ze, zo);
            float dot[MR];
            if constexpr (ACTL) {
                // a chunk past K: exactly the zero sum of zero activations
                dot[0] = dot_words<NW>(words, a_buf[j & 1], ze, zo, nk);
                dot[0] = p + j * LT < g.S ? dot[0] : 0.f;
            } else if constexpr (MR == 1) {
                dot[0] = dot_words<NW>(words, av[j], ze, zo, nk);
            } else {
                dot_words_rows<NW, MR>(words, &av[j * MR], ze, zo, nk, dot);
            }
            const float sc = BF16 ? __uint_as_float(cur.sc[j] << 16) : __uint_as_float(cur.sc[j]);
#pragma unroll
            for (int r = 0; r < MR; r++) s[r] = fmaf(sc, dot[r], s[r]);
            if constexpr (ACTL) __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int r = 0; r < MR; r++) acc[r] = reduce_lanes(s[r], g.log2_L);
        if constexpr (W > 1) {
            if (lane == 63) {
#pragma unroll
                for (int r = 0; r < MR; r++) red[wave * MR + r] = acc[r];
            }
            __syncthreads();
            if (wt == 0) {
#pragma unroll
                for (int r = 0; r < MR; r++) {
                    float v = red[team * W * MR + r];
#pragma unroll
                    for (int w2 = 1; w2 < W; w2++) v += red[(team * W + w2) * MR + r];
                    acc[r] = v;
                }
            }
            __syncthreads();
        }
    };
    const bool writer = wt == 0 && (lane & (L - 1)) == L - 1;
    if constexpr (SILU) {
        // one column group per iteration: its gate half in g0, its up half
        // in g1; the next group's halves are requested as each is reduced.
        // base is workgroup-uniform in it0, so split-K barriers are reached
        // by all
        for (int64_t it0 = team0; it0 < g.n_groups; it0 += stride, base += stride) {
            float gate[MR], up[MR];
            reduce(g0, gate);
            const float gbias = HAS_BIAS ? __uint_as_float(g0.bias) : 0.f;
            if (base + stride < g.n_groups)
                load_group<BF16, HAS_ZP, HAS_BIAS, CB, J, NTS>(g, base + stride, 0, width, p, LT, G, gsub, g0);
            __builtin_amdgcn_sched_barrier(0);
            reduce(g1, up);
            if (writer) {
                const int64_t col = base * G + gsub;
                if (base < g.n_groups && col < g.half) {
                    const float gv = gate[0] + gbias;
                    const float uv = up[0] + (HAS_BIAS ? __uint_as_float(g1.bias) : 0.f);
                    const float h = gv / (1.0f + expf(-gv)) * uv;
                    if constexpr (BF16)
                        static_cast<uint16_t*>(g.y)[col] = f32_to_bf16_rtne(h);
                    else
                        static_cast<float*>(g.y)[col] = h;
                }
            }
            if (base + stride < g.n_groups)
                load_group<BF16, HAS_ZP, HAS_BIAS, CB, J, NTS>(g, base + stride, g.half, width, p, LT, G, gsub, g1);
            __builtin_amdgcn_sched_barrier(0);
        }
    } else {
        auto store = [&](const Group<BF16, HAS_ZP, CB, J>& cur, const float (&acc)[MR], int64_t gi) {
            if (!writer) return;
            const int64_t col = gi * G + gsub;
            if (gi < g.n_groups && col < g.N) {
#pragma unroll
                for (int r = 0; r < MR; r++) {
                    if (r >= g.M) break;
                    float v = acc[r];
                    if (HAS_BIAS) v += __uint_as_float(cur.bias);
                    if constexpr (BF16)
                        static_cast<uint16_t*>(g.y)[r * g.N + col] = f32_to_bf16_rtne(v);
                    else
                        static_cast<float*>(g.y)[r * g.N + col] = v;
                }
            }
        };
        // it0 is WG-uniform, so the barriers of split-K teams are reached by
        // all.  No exit between the halves (it would cost precise waits): the
        // second half past the end loads zeros and skips its work.
        if constexpr (ONE) {
            // every team has at most one column group (the grid covers them all)
            float acc[MR];
            reduce(g0, acc);
            store(g0, acc, base);
            return;
        }
        for (int64_t it0 = team0; it0 < g.n_groups; it0 += 2 * stride, base += 2 * stride) {
            float acc[MR];
            reduce(g0, acc);
            store(g0, acc, base);
            if (base + 2 * stride < g.n_groups)
                load_group<BF16, HAS_ZP, HAS_BIAS, CB, J, NTS>(g, base + 2 * stride, 0, width, p, LT, G, gsub, g0);
            __builtin_amdgcn_sched_barrier(0);
            if (it0 + stride < g.n_groups) {
                reduce(g1, acc);
                store(g1, acc, base + stride);
            }
            if (base + 3 * stride < g.n_groups)
                load_group<BF16, HAS_ZP, HAS_BIAS, CB, J, NTS>(g, base + 3 * stride, 0, width, p, LT, G, gsub, g1);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}


// ---- kernel choice for one activation type ----
// (the plain and the gated kernel at every geometry; RMSNorm and the
// register-held input with the scale policy the launcher gives them:
// non-temporal exactly for 8-byte chunks)

template <bool BF16, bool HAS_ZP, bool HAS_BIAS, int CB, int J, bool SILU, bool NTS, bool RMS, bool REGS,
          bool ONE = false>
GemvFn pick_js(int W) {
    if (W == 1) return gemv_kernel<BF16, HAS_ZP, HAS_BIAS, CB, J, 1, SILU, 1, NTS, RMS, REGS, ONE>;
    if constexpr (CB == 16) {
        if (W == 2) return gemv_kernel<BF16, HAS_ZP, HAS_BIAS, CB, J, 2, SILU, 1, NTS, RMS, REGS, ONE>;
        if (W == 4) return gemv_kernel<BF16, HAS_ZP, HAS_BIAS, CB, J, 4, SILU, 1, NTS, RMS, REGS, ONE>;
    }
    return nullptr;
}

template <bool BF16, bool HAS_ZP, bool HAS_BIAS, int CB, int J, bool NTS>
GemvFn pick_j(int W, bool silu, int input) {
    if (silu) return pick_js<BF16, HAS_ZP, HAS_BIAS, CB, J, true, NTS, false, false>(W);
    if (input == kInputRms) {
        if constexpr (NTS == (CB != 16)) return pick_js<BF16, HAS_ZP, HAS_BIAS, CB, J, false, NTS, true, false>(W);
        return nullptr;
    }
    if (input == kInputLdsOne) {
        if constexpr (J > 1) return pick_js<BF16, HAS_ZP, HAS_BIAS, CB, J, false, NTS, false, false, true>(W);
        return nullptr;
    }
    if (input == kInputRegs) {
        if constexpr (J > 1 && NTS == (CB != 16))
            return pick_js<BF16, HAS_ZP, HAS_BIAS, CB, J, false, NTS, false, true>(W);
        return nullptr;
    }
    return pick_js<BF16, HAS_ZP, HAS_BIAS, CB, J, false, NTS, false, false>(W);
}

template <bool BF16, bool HAS_ZP, bool HAS_BIAS, int CB, bool NTS>
GemvFn pick_cb(int J, int W, bool silu, int input) {
    switch (J) {
        case 1: return pick_j<BF16, HAS_ZP, HAS_BIAS, CB, 1, NTS>(W, silu, input);
        case 2: return pick_j<BF16, HAS_ZP, HAS_BIAS, CB, 2, NTS>(W, silu, input);
        case 3: return pick_j<BF16, HAS_ZP, HAS_BIAS, CB, 3, NTS>(W, silu, input);
        case 4: return pick_j<BF16, HAS_ZP, HAS_BIAS, CB, 4, NTS>(W, silu, input);
        case 5: return pick_j<BF16, HAS_ZP, HAS_BIAS, CB, 5, NTS>(W, silu, input);
        default: return nullptr;
    }
}

// 8-byte chunks come with 16-value blocks only, where the small loads are
// always non-temporal
template <bool BF16, bool HAS_ZP, bool HAS_BIAS>
GemvFn pick_b(int CB, int J, int W, bool silu, int input, bool nts) {
    if (CB != 16) return pick_cb<BF16, HAS_ZP, HAS_BIAS, 8, true>(J, W, silu, input);
    return nts ? pick_cb<BF16, HAS_ZP, HAS_BIAS, 16, true>(J, W, silu, input)
               : pick_cb<BF16, HAS_ZP, HAS_BIAS, 16, false>(J, W, silu, input);
}

template <bool BF16>
GemvFn pick_type(bool has_zp, bool has_bias, int CB, int J, int W, bool silu, int input, bool nts) {
    if (has_zp) return has_bias ? pick_b<BF16, true, true>(CB, J, W, silu, input, nts)
                                : pick_b<BF16, true, false>(CB, J, W, silu, input, nts);
    return has_bias ? pick_b<BF16, false, true>(CB, J, W, silu, input, nts)
                    : pick_b<BF16, false, false>(CB, J, W, silu, input, nts);
}

// MR rows of A (block >= 32, so 16-byte chunks), J * MR <= 4
template <bool BF16, bool HAS_ZP, bool HAS_BIAS, int MR, int J, bool NTS>
GemvFn pick_rows_j(int W) {
    if (W == 1) return gemv_kernel<BF16, HAS_ZP, HAS_BIAS, 16, J, 1, false, MR, NTS, false, false, false>;
    if (W == 2) return gemv_kernel<BF16, HAS_ZP, HAS_BIAS, 16, J, 2, false, MR, NTS, false, false, false>;
    if (W == 4) return gemv_kernel<BF16, HAS_ZP, HAS_BIAS, 16, J, 4, false, MR, NTS, false, false, false>;
    return nullptr;
}

template <bool BF16, bool HAS_ZP, bool HAS_BIAS, bool NTS>
GemvFn pick_rows_n(int MR, int J, int W) {
    if (MR == 2) return J == 1 ? pick_rows_j<BF16, HAS_ZP, HAS_BIAS, 2, 1, NTS>(W)
                               : J == 2 ? pick_rows_j<BF16, HAS_ZP, HAS_BIAS, 2, 2, NTS>(W) : nullptr;
    if (MR == 4 && J == 1) return pick_rows_j<BF16, HAS_ZP, HAS_BIAS, 4, 1, NTS>(W);
    return nullptr;
}

template <bool BF16, bool HAS_ZP, bool HAS_BIAS>
GemvFn pick_rows_b(int MR, int J, int W, bool nts) {
    return nts ? pick_rows_n<BF16, HAS_ZP, HAS_BIAS, true>(MR, J, W)
               : pick_rows_n<BF16, HAS_ZP, HAS_BIAS, false>(MR, J, W);
}

template <bool BF16>
GemvFn pick_rows_type(bool has_zp, bool has_bias, int MR, int J, int W, bool nts) {
    if (has_zp) return has_bias ? pick_rows_b<BF16, true, true>(MR, J, W, nts)
                                : pick_rows_b<BF16, true, false>(MR, J, W, nts);
    return has_bias ? pick_rows_b<BF16, false, true>(MR, J, W, nts) : pick_rows_b<BF16, false, false>(MR, J, W, nts);
}

}  // namespace
}  // namespace mnb
