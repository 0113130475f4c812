/*
 * mnb_oracle.c -- plain CPU oracle for the weight-only block-INT4 MatMul
 * (the MatMulNBits contract).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no code, header,
 * table or helper with the GPU library; it is slow on purpose and written so
 * that each function can be checked against its definition by eye.
 *
 * What it follows (page "Qwen3 CPU Inference Critical Path"):
 *   - "Exact kernel inventory", com.microsoft::MatMulNBits row: FP32
 *     activations, packed UINT8 storage of 4-bit weights, FP32 scales,
 *     block_size 32; the implementation keeps weights compressed.
 *   - "INT4 MatMul is first", "Prepared weight-only plan": per-block scales
 *     and optional zero points; decode applies the zero-point correction and
 *     the scales and accumulates; nibble order and tails are part of the plan.
 *   - "Export contract", qwen3-int4-qdq: 4-bit values stored low nibble first;
 *     one scale and one zero point per block of K; partial K blocks, odd N and
 *     packed-byte tails must be handled.
 *
 * The operation (one reading of the pages, see the design notes):
 *
 *   w[k][n] = (q[n][k] - zp[n][k / bs]) * s[n][k / bs]
 *   y[m][n] = sum_{k < K} a[m][k] * w[k][n]  (+ bias[n])
 *
 * with zp = 8 for every block when no zero-point tensor is supplied.
 *
 * Exactness: q - zp is an integer in [-15, 15] (at most 4 significant bits)
 * and s is a binary32 or bfloat16 value (at most 24 bits), so (q - zp) * s is
 * exact in binary64.  a is binary32 or bfloat16 (at most 24 bits), so every
 * product a * w (at most 53 bits) is exact too.  The only rounding in y is the
 * k-sequential binary64 summation.
 *
 * Layouts (the MatMulNBits storage, N-major with K contiguous per column):
 *   packed weights   [N][nb][bs/2] bytes, nb = ceil(K / bs);
 *                    k lives in byte n*nb*(bs/2) + (k/bs)*(bs/2) + (k%bs)/2,
 *                    in the low nibble when k is even, the high one when odd;
 *                    nibbles past K (the partial last block) are written 0.
 *   packed zero pts  [N][ceil(nb/2)] bytes; block b of column n lives in byte
 *                    n*ceil(nb/2) + b/2, low nibble when b is even; a pad
 *                    nibble is written 0.
 *   scales           [N][nb], binary32 or bfloat16 (raw 16-bit patterns).
 *   activations      [M][K], binary32 or bfloat16.
 *   bias             [N] binary32, optional.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1

int64_t oracle_n_blocks(int64_t K, int64_t bs) { return (K + bs - 1) / bs; }

/* The accepted contract: 4-bit weights, K >= 1, N >= 1, and a
 * block size that is a power of two from 16 to 256 (the pages use 32 and
 * 128; the public MatMulNBits schema requires a power of two >= 16). */
int oracle_contract_ok(int64_t K, int64_t N, int64_t bits, int64_t bs) {
    if (bits != 4 || K < 1 || N < 1) return 0;
    if (bs < 16 || bs > 256) return 0;
    for (int64_t p = 16; p <= 256; p *= 2)
        if (bs == p) return 1;
    return 0;
}

/* ---- packing ------------------------------------------------------------ */

void oracle_pack_weights(int64_t K, int64_t N, int64_t bs, const uint8_t *q,
                         uint8_t *packed) {
    int64_t nb = oracle_n_blocks(K, bs);
    int64_t col_bytes = nb * (bs / 2);
    memset(packed, 0, (size_t)(N * col_bytes));
    for (int64_t n = 0; n < N; n++) {
        for (int64_t k = 0; k < K; k++) {
            uint8_t v = q[n * K + k] & 0x0F;
            int64_t byte = n * col_bytes + (k / bs) * (bs / 2) + (k % bs) / 2;
            if (k % 2 == 0)
                packed[byte] |= v;          /* even k: low nibble */
            else
                packed[byte] |= (uint8_t)(v << 4); /* odd k: high nibble */
        }
    }
}

void oracle_unpack_weights(int64_t K, int64_t N, int64_t bs,
                           const uint8_t *packed, uint8_t *q) {
    int64_t nb = oracle_n_blocks(K, bs);
    int64_t col_bytes = nb * (bs / 2);
    for (int64_t n = 0; n < N; n++) {
        for (int64_t k = 0; k < K; k++) {
            uint8_t byte =
                packed[n * col_bytes + (k / bs) * (bs / 2) + (k % bs) / 2];
            q[n * K + k] = (k % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
        }
    }
}

void oracle_pack_zero_points(int64_t N, int64_t nb, const uint8_t *zp,
                             uint8_t *packed) {
    int64_t row = (nb + 1) / 2;
    memset(packed, 0, (size_t)(N * row));
    for (int64_t n = 0; n < N; n++) {
        for (int64_t b = 0; b < nb; b++) {
            uint8_t v = zp[n * nb + b] & 0x0F;
            if (b % 2 == 0)
                packed[n * row + b / 2] |= v;
            else
                packed[n * row + b / 2] |= (uint8_t)(v << 4);
        }
    }
}

void oracle_unpack_zero_points(int64_t N, int64_t nb, const uint8_t *packed,
                               uint8_t *zp) {
    int64_t row = (nb + 1) / 2;
    for (int64_t n = 0; n < N; n++) {
        for (int64_t b = 0; b < nb; b++) {
            uint8_t byte = packed[n * row + b / 2];
            zp[n * nb + b] = (b % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
        }
    }
}

/* ---- scalar conversions --------------------------------------------------- */

static double bf16_bits_to_double(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double load_value(int dtype, const void *base, int64_t idx) {
    if (dtype == ORACLE_F32) return (double)((const float *)base)[idx];
    return bf16_bits_to_double(((const uint16_t *)base)[idx]);
}

/* Round a binary64 value to the nearest bfloat16 (8 significant bits, the
 * binary32 exponent range, subnormal spacing 2^-133), ties to even, in ONE
 * rounding straight from binary64. */
static uint16_t double_to_bf16_rtne(double x) {
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (isnan(x)) return 0x7FC0;
    double ax = fabs(x);
    if (isinf(ax)) return sign | 0x7F80;
    if (ax == 0.0) return sign;
    int e;
    frexp(ax, &e);               /* ax in [2^(e-1), 2^e) */
    int quantum = e - 8;         /* spacing of 8-bit significands there */
    if (quantum < -133) quantum = -133;
    double r = nearbyint(ldexp(ax, -quantum)); /* default mode: ties-to-even */
    double v = ldexp(r, quantum);
    if (v >= 0x1p128) return sign | 0x7F80;    /* rounds past the largest */
    float f = (float)v;          /* exact: v has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return sign | (uint16_t)(u >> 16);
}

void oracle_round_to_f32(int64_t n, const double *x, float *out) {
    for (int64_t i = 0; i < n; i++) out[i] = (float)x[i]; /* one RTNE rounding */
}

void oracle_round_to_bf16(int64_t n, const double *x, uint16_t *out) {
    for (int64_t i = 0; i < n; i++) out[i] = double_to_bf16_rtne(x[i]);
}

/* ---- dequantization --------------------------------------------------------
 * w[n][k] = (q[n][k] - zp[n][k/bs]) * s[n][k/bs], exact in binary64.
 * q and zp are the logical (unpacked) values; zp == NULL means 8 everywhere. */
void oracle_dequant(int64_t K, int64_t N, int64_t bs, const uint8_t *q,
                    const uint8_t *zp, int scale_dtype, const void *scales,
                    double *w) {
    int64_t nb = oracle_n_blocks(K, bs);
    for (int64_t n = 0; n < N; n++) {
        for (int64_t k = 0; k < K; k++) {
            int64_t b = k / bs;
            int zero = zp ? zp[n * nb + b] : 8;
            double s = load_value(scale_dtype, scales, n * nb + b);
            w[n * K + k] = (double)((int)q[n * K + k] - zero) * s;
        }
    }
}

/* The integer part alone, q - zp, for checking exact-integer weight tiles. */
void oracle_dequant_int(int64_t K, int64_t N, int64_t bs, const uint8_t *q,
                        const uint8_t *zp, int8_t *out) {
    int64_t nb = oracle_n_blocks(K, bs);
    for (int64_t n = 0; n < N; n++)
        for (int64_t k = 0; k < K; k++)
            out[n * K + k] =
                (int8_t)((int)q[n * K + k] - (zp ? zp[n * nb + k / bs] : 8));
}

/* ---- matmul ----------------------------------------------------------------
 * y[m][n] = sum_k a[m][k] * w[n][k] + bias[n]      (binary64, k sequential)
 * S[m][n] = sum_k |a[m][k] * w[n][k]| + |bias[n]|  (the tolerance scale)
 * Columns are independent; with nthreads > 1 they are split across OpenMP
 * threads, which does not change the order of any sum. */
void oracle_matmul(int64_t M, int64_t K, int64_t N, int64_t bs, int act_dtype,
                   const void *a, const uint8_t *q, const uint8_t *zp,
                   const void *scales, const float *bias, double *y, double *S,
                   int nthreads) {
    int64_t nb = oracle_n_blocks(K, bs);
    (void)nthreads;
#pragma omp parallel num_threads(nthreads > 0 ? nthreads : 1)
    {
        double *wcol = (double *)malloc(sizeof(double) * (size_t)K);
#pragma omp for schedule(static)
        for (int64_t n = 0; n < N; n++) {
            for (int64_t k = 0; k < K; k++) {
                int64_t b = k / bs;
                int zero = zp ? zp[n * nb + b] : 8;
                double s = load_value(act_dtype, scales, n * nb + b);
                wcol[k] = (double)((int)q[n * K + k] - zero) * s;
            }
            for (int64_t m = 0; m < M; m++) {
                double acc = 0.0, mag = 0.0;
                for (int64_t k = 0; k < K; k++) {
                    double p = load_value(act_dtype, a, m * K + k) * wcol[k];
                    acc += p;
                    mag += fabs(p);
                }
                if (bias) {
                    acc += (double)bias[n];
                    mag += fabs((double)bias[n]);
                }
                y[m * N + n] = acc;
                if (S) S[m * N + n] = mag;
            }
        }
        free(wcol);
    }
}

/* ---- the QDQ encoding (page "Qwen3 CPU Inference Critical Path", "Export
 * contract", qwen3-int4-qdq) ------------------------------------------------
 * A logical UINT4 tensor is stored in ONNX row-major element order, two
 * elements per byte, the even-numbered element in the low nibble.  Scales and
 * zero points are blocked along one axis of the weight:
 *   axis 0 (a projection):      W[K][N], scale/zp [nb][N], block of k = k/bs;
 *   axis 1 (tied embedding/LM): W[N][K], scale/zp [N][nb], block of k = k/bs.
 * A missing zero-point tensor means zero point 0 (the DequantizeLinear
 * default), unlike the MatMulNBits default of 8. */

/* element i of a flat packed UINT4 stream */
static uint8_t qdq_nibble(const uint8_t *packed, int64_t i) {
    uint8_t byte = packed[i / 2];
    return (i % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
}

void oracle_qdq_unpack(int64_t count, const uint8_t *packed, uint8_t *out) {
    for (int64_t i = 0; i < count; i++) out[i] = qdq_nibble(packed, i);
}

/* flat element index of w[k][n] (the MatMulNBits B[k][n]) in the QDQ tensor */
static int64_t qdq_w_index(int axis, int64_t K, int64_t N, int64_t k, int64_t n) {
    return axis == 0 ? k * N + n : n * K + k;
}

static int64_t qdq_s_index(int axis, int64_t nb, int64_t N, int64_t b, int64_t n) {
    return axis == 0 ? b * N + n : n * nb + b;
}

/* DequantizeLinear on the QDQ layout, straight from the definition:
 * out[k][n] = (w - zp) * scale, exact in binary64. */
void oracle_qdq_dequant(int64_t K, int64_t N, int64_t bs, int axis,
                        const uint8_t *w_q, const uint8_t *zp_q,
                        int scale_dtype, const void *scales_q, double *out) {
    int64_t nb = oracle_n_blocks(K, bs);
    for (int64_t k = 0; k < K; k++) {
        for (int64_t n = 0; n < N; n++) {
            int64_t b = k / bs;
            int64_t si = qdq_s_index(axis, nb, N, b, n);
            int w = qdq_nibble(w_q, qdq_w_index(axis, K, N, k, n));
            int zero = zp_q ? qdq_nibble(zp_q, si) : 0;
            out[k * N + n] = (double)(w - zero) * load_value(scale_dtype, scales_q, si);
        }
    }
}

/* The normalization into the MatMulNBits storage: gather the logical
 * q[n][k] and zp[n][b] from the QDQ tensors, then pack them with the packers
 * above; scales are moved element by element (scale_size bytes each) into
 * [N][nb]. */
void oracle_qdq_import(int64_t K, int64_t N, int64_t bs, int axis,
                       const uint8_t *w_q, const uint8_t *zp_q,
                       int64_t scale_size, const void *scales_q,
                       uint8_t *b_packed, void *scales, uint8_t *zp_packed) {
    int64_t nb = oracle_n_blocks(K, bs);
    uint8_t *q = (uint8_t *)malloc((size_t)(N * K));
    uint8_t *zp = (uint8_t *)malloc((size_t)(N * nb));
    for (int64_t n = 0; n < N; n++) {
        for (int64_t k = 0; k < K; k++)
            q[n * K + k] = qdq_nibble(w_q, qdq_w_index(axis, K, N, k, n));
        for (int64_t b = 0; b < nb; b++) {
            int64_t si = qdq_s_index(axis, nb, N, b, n);
            zp[n * nb + b] = zp_q ? qdq_nibble(zp_q, si) : 0;
            memcpy((uint8_t *)scales + (n * nb + b) * scale_size,
                   (const uint8_t *)scales_q + si * scale_size, (size_t)scale_size);
        }
    }
    oracle_pack_weights(K, N, bs, q, b_packed);
    oracle_pack_zero_points(N, nb, zp, zp_packed);
    free(q);
    free(zp);
}

/* ---- the gated MLP product (page "Qwen3 CPU Inference Critical Path",
 * "Operator priority": the SiLU-gated MLP, Sigmoid(x) * x times the up
 * projection) ------------------------------------------------------------- */
void oracle_silu_mul(int64_t n, const double *gate, const double *up, double *h) {
    for (int64_t i = 0; i < n; i++) {
        double g = gate[i];
        double sig = 1.0 / (1.0 + exp(-g));
        h[i] = g * sig * up[i];
    }
}

/* ---- RMS normalization of a projection's input (page "Qwen3 CPU Inference
 * Critical Path", "Phase Q2": SimplifiedLayerNormalization lowered to the
 * RMSNormalization engine; "Phase Q5": RMSNorm into the packed projection
 * input).  The RMSNormalization definition over the last axis:
 *   a[m][k] = x[m][k] / sqrt(mean_k x[m][k]^2 + eps) * gamma[k]
 * in binary64 (x and gamma binary32 or bfloat16, gamma of length K). */
void oracle_rmsnorm(int64_t M, int64_t K, int dtype, const void *x, const void *gamma, double eps,
                    double *a) {
    for (int64_t m = 0; m < M; m++) {
        double ss = 0.0;
        for (int64_t k = 0; k < K; k++) {
            double v = load_value(dtype, x, m * K + k);
            ss += v * v;
        }
        double rms = sqrt(ss / (double)K + eps);
        for (int64_t k = 0; k < K; k++)
            a[m * K + k] = load_value(dtype, x, m * K + k) / rms * load_value(dtype, gamma, k);
    }
}

/* The matmul above on binary64 activations (the normalized input), scales
 * in their own type: y and S as in oracle_matmul, k-sequential. */
void oracle_matmul_f64a(int64_t M, int64_t K, int64_t N, int64_t bs, int scale_dtype, const double *a,
                        const uint8_t *q, const uint8_t *zp, const void *scales, const float *bias,
                        double *y, double *S) {
    int64_t nb = oracle_n_blocks(K, bs);
    for (int64_t n = 0; n < N; n++) {
        for (int64_t m = 0; m < M; m++) {
            double acc = 0.0, mag = 0.0;
            for (int64_t k = 0; k < K; k++) {
                int64_t b = k / bs;
                int zero = zp ? zp[n * nb + b] : 8;
                double w = (double)((int)q[n * K + k] - zero) * load_value(scale_dtype, scales, n * nb + b);
                double p = a[m * K + k] * w;
                acc += p;
                mag += fabs(p);
            }
            if (bias) {
                acc += (double)bias[n];
                mag += fabs((double)bias[n]);
            }
            y[m * N + n] = acc;
            S[m * N + n] = mag;
        }
    }
}

/* ---- greedy ArgMax ("final RMSNorm, LM-head GEMV, and greedy ArgMax"):
 * per row, the first index holding the largest value; a NaN counts as larger
 * than every number, so the first NaN wins. */
void oracle_argmax(int64_t M, int64_t N, int dtype, const void *x, int64_t *idx) {
    for (int64_t m = 0; m < M; m++) {
        int64_t best = 0;
        double bv = load_value(dtype, x, m * N);
        for (int64_t n = 1; n < N && !isnan(bv); n++) {
            double v = load_value(dtype, x, m * N + n);
            if (isnan(v) || v > bv) {
                best = n;
                bv = v;
            }
        }
        idx[m] = best;
    }
}
