// The decode GEMV's arithmetic, shared by the per-projection kernel
// (mnb_gemv.hip) and the persistent decode-step kernel (mnb_step.hip): the
// nibble-to-f16 unpacking, the per-chunk dot product, the lane reduction tree
// and the choice of lanes, chunks per lane and wavefronts per column.  Both
// kernels take a column's geometry from geometry() and sum it with these
// functions, so a column computed by either has the same float32 bits.
#pragma once

#include "mnb_internal.h"

namespace mnb {
namespace {

constexpr int kJMax = 5;          // chunks per lane held in registers
constexpr int kWMax = 4;          // wavefronts per column (split-K)
constexpr uint32_t kOob = 0x80000000u;    // buffer offset past any resource: the load reads zero
constexpr int kNonTemporal = 2;           // cache policy of a load whose bytes are read once (nt)

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int CB>
struct ChunkT;
template <>
struct ChunkT<16> { using type = u32x4; };
template <>
struct ChunkT<8> { using type = u32x2; };

// One 32-bit word of a chunk holds values 8d..8d+7, two per byte, the even
// one in the low nibble.  Two nibbles 16 bits apart are masked into the
// mantissas of a packed f16 pair with one v_and_or_b32: nibbles at bits 0..3
// of a half give 1024 + q, nibbles at bits 4..7 give 1024 + 16 q.  One packed
// f16 operation leaves the exact integers q - zp: v_pk_add_f16 of
// -(1024 + zp) for the first kind, v_pk_fma_f16 times 1/16 plus -(64 + zp)
// for the second.  v_fma_mix_f32 multiplies each f16 half into a float32 FMA,
// so every product is exactly a (q - zp) before the FMA rounding, a weight
// equal to its zero point adds exactly nothing, and the chunk sum is the
// float32 sum of the products a_k (q_k - zp) (about 2.1 instructions per
// weight).  ze holds -(1024 + zp) and zo holds -(64 + zp) in both halves.
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// The masks and the f16 exponent pattern live in VGPRs whose values the
// compiler cannot see, so (w & mask) | magic becomes one v_and_or_b32 (gfx9
// VOP3 encodings take no literal constants) without an opaque asm statement
// at every use.
struct NibbleMasks {
    uint32_t lo, hi, magic;      // 0x000F000F, 0x00F000F0, 0x64006400
};

__device__ __forceinline__ NibbleMasks nibble_masks() {
    NibbleMasks k{0x000F000Fu, 0x00F000F0u, 0x64006400u};
    asm volatile("" : "+v"(k.lo), "+v"(k.hi), "+v"(k.magic));
    return k;
}

// nibbles at bits 0..3 of each half: q - zp
__device__ __forceinline__ half2_t nibble_pair(uint32_t w, uint32_t mask, uint32_t magic, uint32_t ze) {
    const uint32_t m = (w & mask) | magic;
    return __builtin_bit_cast(half2_t, m) + __builtin_bit_cast(half2_t, ze);
}

// nibbles at bits 4..7 of each half: (1024 + 16 q) / 16 - (64 + zp) = q - zp
__device__ __forceinline__ half2_t nibble_pair_hi(uint32_t w, uint32_t mask, uint32_t magic, uint32_t zo) {
    const uint32_t m = (w & mask) | magic;
    const half2_t sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
    return __builtin_elementwise_fma(__builtin_bit_cast(half2_t, m), sixteenth, __builtin_bit_cast(half2_t, zo));
}

// f16 pairs -(1024 + zp) and -(64 + zp)
__device__ __forceinline__ void zero_point_pairs(uint32_t zp, uint32_t& ze, uint32_t& zo) {
    const uint32_t he = 0xE400u | zp, ho = 0xD400u | (zp << 4);
    ze = he | (he << 16);
    zo = ho | (ho << 16);
}

template <int NW>
__device__ __forceinline__ float dot_words(const uint32_t (&w)[NW], const float* av, uint32_t ze, uint32_t zo,
                                           const NibbleMasks& k) {
    float de = 0.f, dd = 0.f;
#pragma unroll
    for (int d = 0; d < NW; d++) {
        const uint32_t w8 = w[d] >> 8;
        const half2_t p0 = nibble_pair(w[d], k.lo, k.magic, ze);   // values 8d + 0, 8d + 4
        const half2_t p1 = nibble_pair_hi(w[d], k.hi, k.magic, zo);   // 8d + 1, 8d + 5
        const half2_t p2 = nibble_pair(w8, k.lo, k.magic, ze);     // 8d + 2, 8d + 6
        const half2_t p3 = nibble_pair_hi(w8, k.hi, k.magic, zo);     // 8d + 3, 8d + 7
        de = fmaf(av[8 * d + 0], (float)p0[0], de);
        dd = fmaf(av[8 * d + 1], (float)p1[0], dd);
        de = fmaf(av[8 * d + 2], (float)p2[0], de);
        dd = fmaf(av[8 * d + 3], (float)p3[0], dd);
        de = fmaf(av[8 * d + 4], (float)p0[1], de);
        dd = fmaf(av[8 * d + 5], (float)p1[1], dd);
        de = fmaf(av[8 * d + 6], (float)p2[1], de);
        dd = fmaf(av[8 * d + 7], (float)p3[1], dd);
    }
    return de + dd;
}

template <int CTRL>
__device__ __forceinline__ float add_dpp(float v) {
    const int t = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true);
    return v + __builtin_bit_cast(float, t);
}

template <int CTRL, int ROWS>
__device__ __forceinline__ float add_dpp_rows(float v) {
    const int t = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROWS, 0xF, false);
    return v + __builtin_bit_cast(float, t);
}

// Sum over aligned groups of 2^log2_L lanes, valid in the LAST lane of each
// group.  The tree is fixed and all DPP: pairs, quads, eights, sixteens
// (after which every lane of a 16-lane row holds the row sum), then the
// row sums are added by row broadcasts (rows 1 and 3 take the last lane of
// rows 0 and 2; row 3 then takes the last lane of row 1).
__device__ __forceinline__ float reduce_lanes(float v, int log2_L) {
    if (log2_L >= 1) v = add_dpp<0xB1>(v);            // quad_perm [1,0,3,2]
    if (log2_L >= 2) v = add_dpp<0x4E>(v);            // quad_perm [2,3,0,1]
    if (log2_L >= 3) v = add_dpp<0x141>(v);           // row_half_mirror
    if (log2_L >= 4) v = add_dpp<0x140>(v);           // row_mirror
    if (log2_L >= 5) v = add_dpp_rows<0x142, 0xA>(v);  // row_bcast:15 into rows 1, 3
    if (log2_L >= 6) v = add_dpp_rows<0x143, 0x8>(v);  // row_bcast:31 into row 3
    return v;
}

int ilog2(int64_t v) {
    int r = 0;
    while ((int64_t(1) << r) < v) r++;
    return r;
}

struct Geometry {
    int log2_L, J, W;
};

// Lanes per wavefront, chunks per lane and wavefronts per column: a function
// of S = ceil(K / CK) (and of the chunks a lane may hold) only.  Highest lane
// efficiency S / (L*W*J) first, then fewer wavefronts, then fewer chunks per
// lane.  J == 0: no register kernel.
Geometry geometry(int64_t S, bool allow_split, int jmax = kJMax) {
    Geometry best{0, 0, 0};
    double best_eff = -1.0;
    for (int W = 1; W <= (allow_split ? kWMax : 1); W *= 2) {
        for (int lL = 0; lL <= 6; lL++) {
            if (W > 1 && lL != 6) continue;    // split-K teams use whole wavefronts
            const int64_t LT = (int64_t(1) << lL) * W;
            if (LT > 2 * S && lL > 0) continue; // more than twice the lanes needed
            const int64_t J = (S + LT - 1) / LT;
            if (J > jmax) continue;
            const double eff = (double)S / (double)(LT * J);
            const bool better = eff > best_eff + 1e-9 ||
                                (eff > best_eff - 1e-9 && (W < best.W || (W == best.W && J < best.J)));
            if (better) {
                best = Geometry{lL, (int)J, W};
                best_eff = eff;
            }
        }
    }
    return best;
}

}  // namespace
}  // namespace mnb
