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
// visits, so its J*CK activations are loaded once into registers and reused
// for all of the team's columns.  For a fixed column the lanes read
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
#include "mnb_gemv_core.h"

namespace mnb {
namespace {

constexpr int kWavesPerBlock = 4;
constexpr size_t kMaxLds = 64 * 1024;    // staged activations per workgroup

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
template <bool BF16, bool HAS_ZP, bool HAS_BIAS, int CB, int J, int W, bool SILU, int MR, bool NTS>
__global__ __launch_bounds__(64 * kWavesPerBlock) void gemv_kernel(GemvArgs g) {
    constexpr int CK = 2 * CB;        // values of K per chunk
    constexpr int NW = CB / 4;        // 32-bit words per chunk
    constexpr int TEAMS = kWavesPerBlock / W;
    static_assert(MR == 1 || (!SILU && J * MR <= 4 && CB == 16), "row kernel: <= 4 row chunks");
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
        if (g.gamma) {
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
    const bool two = SILU || base + stride < g.n_groups;     // wave-uniform
    load_group<BF16, HAS_ZP, HAS_BIAS, CB, J, NTS>(g, base, 0, width, p, LT, G, gsub, g0);
    if (two)
        load_group<BF16, HAS_ZP, HAS_BIAS, CB, J, NTS>(g, SILU ? base : base + stride, SILU ? g.half : 0, width, p,
                                                  LT, G, gsub, g1);

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
    if (g.gamma) {
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
    // this lane's chunks of A in registers, for each row
    float av[MR * J][CK];
#pragma unroll
    for (int mj = 0; mj < MR * J; mj++) {          // [chunk j][row m]
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
                if (g.gamma) {
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
#pragma unroll
        for (int j = 0; j < J; j++) {
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
            if constexpr (MR == 1)
                dot[0] = dot_words<NW>(words, av[j], ze, zo, nk);
            else
                dot_words_rows<NW, MR>(words, &av[j * MR], ze, zo, nk, dot);
            const float sc = BF16 ? __uint_as_float(cur.sc[j] << 16) : __uint_as_float(cur.sc[j]);
#pragma unroll
            for (int r = 0; r < MR; r++) s[r] = fmaf(sc, dot[r], s[r]);
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


using GemvFn = void (*)(GemvArgs);

template <bool BF16, bool HAS_ZP, bool HAS_BIAS, int CB, int J, bool SILU, bool NTS>
GemvFn pick_js(int W) {
    if (W == 1) return gemv_kernel<BF16, HAS_ZP, HAS_BIAS, CB, J, 1, SILU, 1, NTS>;
    if constexpr (CB == 16) {
        if (W == 2) return gemv_kernel<BF16, HAS_ZP, HAS_BIAS, CB, J, 2, SILU, 1, NTS>;
        if (W == 4) return gemv_kernel<BF16, HAS_ZP, HAS_BIAS, CB, J, 4, SILU, 1, NTS>;
    }
    return nullptr;
}

template <bool BF16, bool HAS_ZP, bool HAS_BIAS, int CB, int J, bool NTS>
GemvFn pick_j(int W, bool silu) {
    return silu ? pick_js<BF16, HAS_ZP, HAS_BIAS, CB, J, true, NTS>(W)
                : pick_js<BF16, HAS_ZP, HAS_BIAS, CB, J, false, NTS>(W);
}

template <bool BF16, bool HAS_ZP, bool HAS_BIAS, int CB, bool NTS>
GemvFn pick_cb(int J, int W, bool silu) {
    switch (J) {
        case 1: return pick_j<BF16, HAS_ZP, HAS_BIAS, CB, 1, NTS>(W, silu);
        case 2: return pick_j<BF16, HAS_ZP, HAS_BIAS, CB, 2, NTS>(W, silu);
        case 3: return pick_j<BF16, HAS_ZP, HAS_BIAS, CB, 3, NTS>(W, silu);
        case 4: return pick_j<BF16, HAS_ZP, HAS_BIAS, CB, 4, NTS>(W, silu);
        case 5: return pick_j<BF16, HAS_ZP, HAS_BIAS, CB, 5, NTS>(W, silu);
        default: return nullptr;
    }
}

// nts: scales, zero points and bias read non-temporally like the weights
// (8-byte chunks come with 16-value blocks only, where they always are)
template <bool BF16, bool HAS_ZP, bool HAS_BIAS>
GemvFn pick_b(int CB, int J, int W, bool silu, bool nts) {
    if (CB != 16) return pick_cb<BF16, HAS_ZP, HAS_BIAS, 8, true>(J, W, silu);
    return nts ? pick_cb<BF16, HAS_ZP, HAS_BIAS, 16, true>(J, W, silu)
               : pick_cb<BF16, HAS_ZP, HAS_BIAS, 16, false>(J, W, silu);
}

// MR rows of A (block >= 32, so 16-byte chunks), J * MR <= 4
template <bool BF16, bool HAS_ZP, bool HAS_BIAS, int MR, int J, bool NTS>
GemvFn pick_rows_j(int W) {
    if (W == 1) return gemv_kernel<BF16, HAS_ZP, HAS_BIAS, 16, J, 1, false, MR, NTS>;
    if (W == 2) return gemv_kernel<BF16, HAS_ZP, HAS_BIAS, 16, J, 2, false, MR, NTS>;
    if (W == 4) return gemv_kernel<BF16, HAS_ZP, HAS_BIAS, 16, J, 4, false, MR, NTS>;
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

GemvFn pick_rows(bool bf16, bool has_zp, bool has_bias, int MR, int J, int W, bool nts) {
    if (bf16) {
        if (has_zp) return has_bias ? pick_rows_b<true, true, true>(MR, J, W, nts)
                                    : pick_rows_b<true, true, false>(MR, J, W, nts);
        return has_bias ? pick_rows_b<true, false, true>(MR, J, W, nts) : pick_rows_b<true, false, false>(MR, J, W, nts);
    }
    if (has_zp) return has_bias ? pick_rows_b<false, true, true>(MR, J, W, nts)
                                : pick_rows_b<false, true, false>(MR, J, W, nts);
    return has_bias ? pick_rows_b<false, false, true>(MR, J, W, nts) : pick_rows_b<false, false, false>(MR, J, W, nts);
}

// silu: the gated gate||up kernel
GemvFn pick(bool bf16, bool has_zp, bool has_bias, int CB, int J, int W, bool silu, bool nts) {
    if (bf16) {
        if (has_zp) return has_bias ? pick_b<true, true, true>(CB, J, W, silu, nts)
                                    : pick_b<true, true, false>(CB, J, W, silu, nts);
        return has_bias ? pick_b<true, false, true>(CB, J, W, silu, nts) : pick_b<true, false, false>(CB, J, W, silu, nts);
    }
    if (has_zp) return has_bias ? pick_b<false, true, true>(CB, J, W, silu, nts)
                                : pick_b<false, true, false>(CB, J, W, silu, nts);
    return has_bias ? pick_b<false, false, true>(CB, J, W, silu, nts) : pick_b<false, false, false>(CB, J, W, silu, nts);
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
                                                     64 * kWavesPerBlock, lds) != hipSuccess || n < 1)
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
    // groups per iteration costs more in occupancy than it saves.  When two
    // workgroups per CU already leave each team at most 2.5 groups, use only
    // those: a team with two groups has the second in flight while it reduces
    // the first, which measured 2-7 % faster than one group per team on the
    // few-MB decode projections (and slower on the large ones).
    const int64_t cus = compute_units();
    const int teams_per_block = kWavesPerBlock / geo.W;
    // Weights are read non-temporally (each byte once): streamed past the
    // caches, they leave the activations and the scales resident, 4-9 % per
    // decode step.  With blocks of at most 32 values every chunk has its own
    // scale and zero point, a stream of 20-28 % of the bytes read once like
    // the weights, read non-temporally too (the 0.6B step 7 % faster); with
    // larger blocks several lanes and neighbouring columns share the scale
    // lines, which stay cached (non-temporal scales slowed the 4B step 3 %).
    const bool nts = p.bs <= 32;
    GemvFn f = MR == 1 ? pick(p.bf16, p.has_zp, p.bias != nullptr, CB, geo.J, geo.W, silu, nts)
                       : pick_rows(p.bf16, p.has_zp, p.bias != nullptr, MR, geo.J, geo.W, nts);
    if (!f) return fail(MNB_E_UNSUPPORTED, "gemv: no kernel for J=%d W=%d", geo.J, geo.W);
    const int64_t teams = a.n_groups;
    int64_t blocks = (teams + teams_per_block - 1) / teams_per_block;
    int64_t max_blocks = cus * resident_per_cu(f, lds);
    if (max_blocks > 2 * cus && 2 * teams <= 5 * (2 * cus * teams_per_block)) max_blocks = 2 * cus;
    if (blocks > max_blocks) blocks = max_blocks;
    hipLaunchKernelGGL(f, dim3((unsigned)blocks), dim3(64 * kWavesPerBlock), lds, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(MNB_E_HIP, "gemv launch: %s", hipGetErrorString(e));
    return MNB_OK;
}

}  // namespace

int launch_gemv(const Problem& p, hipStream_t s) { return launch(p, s, false); }

bool gemv_rows_ok(const Problem& p) {
    if (p.M < 2 || p.M > 4 || p.bs < 32) return false;
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
