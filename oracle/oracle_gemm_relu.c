/*
 * CPU oracle for C = ReLU(A * B) with fp16 operands, fp32 accumulation and an
 * fp16 result.  TEST INFRASTRUCTURE ONLY: the product library never links,
 * loads or calls this file; only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark do.  It shares no code with the GPU path.
 *
 * What it computes (one element at a time, written out plainly):
 *
 *   1. Widen each fp16 operand to fp32.  Every binary16 value, subnormals
 *      included, is exactly representable in binary32.
 *   2. acc = +0.0f; for k = 0, 1, ..., K-1 in that order:
 *          acc = fl32(acc + a[i][k] * b[k][j]).
 *      The accumulator starts cleared and is fp32, as in the TileLang tutorial
 *      chapter "GEMM walkthrough and parameter derivation" (T.clear of the fp32
 *      fragment, then one tile product accumulated per K strip) and the blog
 *      "TileLang programming basics", section 2 (fp32 fragment, fp16 storage).
 *      The product of two fp16 numbers needs at most 22 significand bits and
 *      lies well inside the fp32 normal range, so it is exact in fp32: the only
 *      rounding in the loop is the addition.  The build flags forbid
 *      reassociation (-fno-fast-math) and contraction (-ffp-contract=off).
 *   3. ReLU on the fp32 accumulator: r = acc > 0 ? acc : +0.0f.  The epilogue
 *      in both GEMM+ReLU listings (blog section 2, and "Writing
 *      high-performance kernels in TileLang", section "Writing a GEMM") takes
 *      max(C_local, 0) on the fp32 fragment before the write-back.  Negative
 *      values, -0 and NaN all map to +0 (the pages leave these open; this is
 *      the reading stated in the design notes).
 *   4. Round r to fp16, to nearest with ties to even; values too large become
 *      +Inf.  The pages only say the cast happens on write-back; RNE is the
 *      IEEE default and the reading taken here.
 *
 * Loop order: the full/rows variants run i, then k, then j with a row of fp32
 * accumulators.  Each element still sees exactly the sequence of step 2, so
 * the result is bit-identical to the i-j-k order.  OpenMP (when compiled with
 * -fopenmp) splits rows only, never k.
 *
 * The fp16 <-> fp32 conversions below are written from the IEEE 754 binary16
 * and binary32 encodings, not taken from any library.
 *
 * The same computation is offered for bfloat16 operands and result (the
 * *_bf16_* entry points): bfloat16 is the upper half of a binary32 pattern (8
 * exponent bits, 7 fraction bits), so widening is exact and only step 4
 * changes: round r to bfloat16, nearest with ties to even.  The product of two
 * bfloat16 numbers needs at most 16 significand bits and stays in the fp32
 * range only if the exponents allow; the tests use magnitudes where it is
 * exact, as for fp16.
 *
 * The *_epi_* entry points generalise steps 3 and 4 to C = act(A*B + bias):
 *   3'. x = acc, plus fl32(acc + bias[j]) when a bias (one value per output
 *       column, in the operands' format) is given: the bias is broadcast down
 *       the columns, one of the elementwise operations of "Tilelang Cuda
 *       Patterns", section 1.
 *   4'. y = act(x) for one of the activations that section lists (relu,
 *       sigmoid, tanh, gelu), plus SiLU and the tanh form of GELU, evaluated
 *       in double precision with the C library (erf, tanh, exp); then y is
 *       rounded once to the output format, nearest with ties to even.  ReLU
 *       and the identity stay in fp32 (they are exact) and round as in step 4.
 * The *_fp8_* entry points take A (M x K) and Bt (N x K) in OCP fp8 E4M3
 * (decoded exactly to fp32 below), B given transposed: acc = sum over k of
 * a[i][k] * bt[j][k] in fp32, k increasing (a product of two E4M3 values has
 * at most 8 significant bits and stays in the fp32 normal range, so it is
 * exact); then x = fl32(acc * s) with s = fl32(scale_a * scale_b), the
 * per-tensor dequantisation scales, and steps 3' and 4' as above.
 *
 * The *_mxfp8_* entry points take the same E4M3 operands in OCP MX form:
 * every run of 32 consecutive k of a row of A (of Bt) shares one E8M0 scale
 * (8 exponent bits, value 2^(x - 127); x = 255 is NaN), sa[i][k/32] and
 * sb[j][k/32].  Each product is a[i][k] * 2^(sa - 127) * bt[j][k] * 2^(sb -
 * 127), formed exactly in double and converted to fp32 (exact while it stays
 * in the fp32 range, as in the tests), then added in fp32, k increasing; then
 * steps 3' and 4' with no further scale.  The pages point to block-scaled
 * GEMMs (per-block scales on quantised operands) as examples; MX is the
 * block format the gfx950 matrix cores scale in hardware.
 *
 * The *_mxfp4_* entry points are the same with OCP fp4 E2M1 elements (1 sign
 * bit, 2 exponent bits with bias 1, 1 fraction bit: 0, 0.5, 1, 1.5, 2, 3, 4,
 * 6), two per byte: element k of a row is the low nibble of byte k/2 when k
 * is even, the high nibble when k is odd; K counts elements, the pitches
 * count bytes.
 *
 * The single rounding from double goes through fp32 with round-to-odd (the
 * nearest fp32 toward zero with its last bit forced to 1 when inexact), which
 * keeps two or more spare bits over the fp16 and bfloat16 significands, so
 * the final round-to-nearest-even sees the same side of every midpoint as the
 * exact double would.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- IEEE 754 binary16 <-> binary32 -------------------------------------- */

static float bits_to_f32(uint32_t u) {
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static uint32_t f32_to_bits(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return u;
}

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
float oracle_f16_to_f32(uint16_t h) {
    uint32_t sign = (uint32_t)(h >> 15) << 31;
    uint32_t exp = (h >> 10) & 0x1Fu;
    uint32_t frac = h & 0x3FFu;
    if (exp == 0x1Fu) {
        /* Inf (frac == 0) or NaN: keep the payload, widen it by 13 bits. */
        return bits_to_f32(sign | 0x7F800000u | (frac << 13));
    }
    if (exp == 0) {
        /* zero or subnormal: value = frac * 2^-24, exact in binary32. */
        float mag = (float)frac * 0x1p-24f;
        return sign ? -mag : mag;
    }
    /* normal: (1 + frac/1024) * 2^(exp-15); rebias the exponent to 127. */
    return bits_to_f32(sign | ((exp - 15u + 127u) << 23) | (frac << 13));
}

/* Round a binary32 value to binary16, nearest, ties to even. */
uint16_t oracle_f32_to_f16_rne(float f) {
    uint32_t u = f32_to_bits(f);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    uint32_t exp = (u >> 23) & 0xFFu;
    uint32_t frac = u & 0x7FFFFFu;

    if (exp == 0xFFu) {
        if (frac == 0) return (uint16_t)(sign | 0x7C00u);          /* Inf */
        return (uint16_t)(sign | 0x7E00u | (frac >> 13));          /* quiet NaN */
    }
    int e = (int)exp - 127; /* unbiased exponent of a normal binary32 */
    if (exp == 0) {
        /* binary32 subnormals are below 2^-126, far under half of the
           smallest binary16 subnormal (2^-25): they round to zero. */
        return sign;
    }
    if (e >= 16) return (uint16_t)(sign | 0x7C00u); /* >= 2^16: overflow */

    uint32_t sig = frac | 0x800000u; /* 24-bit significand, value sig*2^(e-23) */
    if (e >= -14) {
        /* binary16 normal range: keep 10 fraction bits, round off 13. */
        uint32_t h = ((uint32_t)(e + 15) << 10) | (frac >> 13);
        uint32_t rem = frac & 0x1FFFu;
        if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h += 1u; /* carry may reach Inf: correct */
        return (uint16_t)(sign | h);
    }
    /* binary16 subnormal range: result is q * 2^-24 with q an integer.
       value / 2^-24 = sig * 2^(e+1), a right shift by s = -(e+1) >= 14. */
    int s = -(e + 1);
    if (s >= 25) return sign; /* value < 2^-25: below half the smallest subnormal */
    uint32_t q = sig >> s;
    uint32_t rem = sig & ((1u << s) - 1u);
    uint32_t half = 1u << (s - 1);
    if (rem > half || (rem == half && (q & 1u))) q += 1u; /* q may become 0x400: the smallest normal */
    return (uint16_t)(sign | q);
}

/* bfloat16: the upper 16 bits of a binary32 pattern. */
float oracle_bf16_to_f32(uint16_t h) { return bits_to_f32((uint32_t)h << 16); }

/* Round a binary32 value to bfloat16, nearest, ties to even.  The kept part is
   the upper 16 bits; the discarded lower 16 bits decide the rounding.  A carry
   out of the fraction increments the exponent, which is the correct result,
   up to +-Inf for the largest finite values. */
uint16_t oracle_f32_to_bf16_rne(float f) {
    uint32_t u = f32_to_bits(f);
    uint32_t exp = (u >> 23) & 0xFFu;
    uint32_t frac = u & 0x7FFFFFu;
    if (exp == 0xFFu && frac != 0) return (uint16_t)((u >> 16) | 0x0040u); /* quiet NaN */
    uint32_t keep = u >> 16;
    uint32_t rem = u & 0xFFFFu;
    if (rem > 0x8000u || (rem == 0x8000u && (keep & 1u))) keep += 1u;
    return (uint16_t)keep;
}

/* OCP fp8 E4M3: sign, 4 exponent bits (bias 7), 3 fraction bits.  Exponent
   field 0 is the subnormal range (m / 8 * 2^-6); S.1111.111 is NaN; there is
   no infinity (S.1111.110 = 448 is the largest finite value). */
float oracle_e4m3_to_f32(uint8_t b) {
    const uint32_t sign = (uint32_t)(b >> 7) << 31;
    const uint32_t e = (b >> 3) & 0xFu, m = b & 7u;
    if (e == 15u && m == 7u) return bits_to_f32(sign | 0x7FC00000u);
    float v;
    if (e == 0u) v = (float)m * 0.001953125f; /* m * 2^-9, exact */
    else v = bits_to_f32(((e - 7u + 127u) << 23) | (m << 20));
    return sign ? -v : v;
}

void oracle_e4m3_to_f32_array(const uint8_t* in, float* out, int64_t n) {
    for (int64_t e = 0; e < n; ++e) out[e] = oracle_e4m3_to_f32(in[e]);
}

/* Array forms of the conversions (used by the conversion pins). */
void oracle_bf16_to_f32_array(const uint16_t* in, float* out, int64_t n) {
    for (int64_t e = 0; e < n; ++e) out[e] = oracle_bf16_to_f32(in[e]);
}

void oracle_f32_to_bf16_array(const float* in, uint16_t* out, int64_t n) {
    for (int64_t e = 0; e < n; ++e) out[e] = oracle_f32_to_bf16_rne(in[e]);
}

void oracle_f16_to_f32_array(const uint16_t* in, float* out, int64_t n) {
    for (int64_t e = 0; e < n; ++e) out[e] = oracle_f16_to_f32(in[e]);
}

void oracle_f32_to_f16_array(const float* in, uint16_t* out, int64_t n) {
    for (int64_t e = 0; e < n; ++e) out[e] = oracle_f32_to_f16_rne(in[e]);
}

/* Element formats of A, B and C. */
enum { FMT_F16 = 0, FMT_BF16 = 1 };

/* Activations (the same codes as the library's GR_ACT_*). */
enum { ACT_NONE = 0, ACT_RELU = 1, ACT_GELU = 2, ACT_GELU_TANH = 3, ACT_SILU = 4, ACT_SIGMOID = 5, ACT_TANH = 6,
       ACT_COUNT = 7 };

/* The epilogue of one call: bias (N values, or NULL) and activation. */
typedef struct {
    const uint16_t* bias;
    int act;
    float scale; /* multiplies the fp32 sum first (1 except for the fp8 entry points) */
} Epi;

static const Epi kRelu = {NULL, ACT_RELU, 1.0f};

static float widen(int fmt, uint16_t h) { return fmt == FMT_BF16 ? oracle_bf16_to_f32(h) : oracle_f16_to_f32(h); }

static uint16_t round_to(int fmt, float r) {
    return fmt == FMT_BF16 ? oracle_f32_to_bf16_rne(r) : oracle_f32_to_f16_rne(r);
}

/* Nearest fp32 toward zero, last bit forced to 1 when d is not exact in fp32
   (round-to-odd).  Beyond the fp32 range this gives the largest finite fp32
   with that sign, which still rounds to Inf in both 16-bit formats. */
static float f64_to_f32_odd(double d) {
    float f = (float)d;
    if (isnan(d) || isinf(d) || (double)f == d) return f;
    if (fabs((double)f) > fabs(d)) f = nextafterf(f, 0.0f);
    return bits_to_f32(f32_to_bits(f) | 1u);
}

/* The activations in double precision, from their definitions.  For x far
   below zero, 1 + erf(x/sqrt 2) and 1 + tanh(u) cancel to nothing; the same
   values are written with functions that keep their precision there:
   1 + erf(z) = erfc(-z), and (1 + tanh u) / 2 = 1 / (1 + e^(-2u)). */
static double act_f64(int act, double x) {
    switch (act) {
        case ACT_GELU: return 0.5 * x * erfc(-x * 0.70710678118654752440);          /* x Phi(x) */
        case ACT_GELU_TANH: {
            const double u = 0.79788456080286535588 * (x + 0.044715 * x * x * x);   /* sqrt(2/pi) */
            return x / (1.0 + exp(-2.0 * u));
        }
        case ACT_SILU: return x / (1.0 + exp(-x));
        case ACT_SIGMOID: return 1.0 / (1.0 + exp(-x));
        case ACT_TANH: return tanh(x);
        default: return x;
    }
}

/* Steps 3 and 4 (or 3' and 4') for output column j. */
static uint16_t epilogue(int fmt, const Epi* ep, int64_t j, float acc) {
    float x = acc * ep->scale; /* exact when the scale is 1 */
    if (ep->bias) x = x + widen(fmt, ep->bias[j]);
    if (ep->act == ACT_RELU) return round_to(fmt, (x > 0.0f) ? x : 0.0f); /* NaN compares false -> +0 */
    if (ep->act == ACT_NONE) return round_to(fmt, x);
    return round_to(fmt, f64_to_f32_odd(act_f64(ep->act, (double)x)));
}

/* ---- thread control (used only to time the oracle) ----------------------- */

void oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---- the four entry points (fp16 and bf16) -------------------------------- */

/* One full output row i.  bf holds B widened to fp32, packed K x N. */
static void one_row(int fmt, const Epi* ep, int64_t i, int64_t N, int64_t K, const uint16_t* A, int64_t lda,
                    const float* bf, float* acc, uint16_t* out) {
    for (int64_t j = 0; j < N; ++j) acc[j] = 0.0f;
    for (int64_t k = 0; k < K; ++k) {
        float a = widen(fmt, A[i * lda + k]);
        const float* brow = bf + k * N;
        for (int64_t j = 0; j < N; ++j) acc[j] = acc[j] + a * brow[j];
    }
    for (int64_t j = 0; j < N; ++j) out[j] = epilogue(fmt, ep, j, acc[j]);
}

static float* widen_b(int fmt, int64_t N, int64_t K, const uint16_t* B, int64_t ldb) {
    float* bf = (float*)malloc((size_t)(K > 0 ? K : 1) * (size_t)(N > 0 ? N : 1) * sizeof(float));
    if (!bf) return NULL;
    for (int64_t k = 0; k < K; ++k)
        for (int64_t j = 0; j < N; ++j) bf[k * N + j] = widen(fmt, B[k * ldb + j]);
    return bf;
}

/* C[i*ldc + j] for all 0 <= i < M, 0 <= j < N.  Returns 0, or -1 on allocation
   failure.  Columns j >= N of C are not touched. */
static int gemm_full(int fmt, const Epi* ep, int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda,
                     const uint16_t* B, int64_t ldb, uint16_t* C, int64_t ldc) {
    if (M <= 0 || N <= 0) return 0;
    float* bf = widen_b(fmt, N, K, B, ldb);
    if (!bf) return -1;
    int failed = 0;
#pragma omp parallel
    {
        float* acc = (float*)malloc((size_t)N * sizeof(float));
        if (!acc) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t i = 0; i < M; ++i) one_row(fmt, ep, i, N, K, A, lda, bf, acc, C + i * ldc);
            free(acc);
        }
    }
    free(bf);
    return failed ? -1 : 0;
}

/* Full rows: out[r*N + j] = C[rows[r]][j] for r < nrows. */
static int gemm_rows(int fmt, const Epi* ep, int64_t N, int64_t K, const uint16_t* A, int64_t lda, const uint16_t* B,
                     int64_t ldb, const int64_t* rows, int64_t nrows, uint16_t* out) {
    if (nrows <= 0 || N <= 0) return 0;
    float* bf = widen_b(fmt, N, K, B, ldb);
    if (!bf) return -1;
    int failed = 0;
#pragma omp parallel
    {
        float* acc = (float*)malloc((size_t)N * sizeof(float));
        if (!acc) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t r = 0; r < nrows; ++r) one_row(fmt, ep, rows[r], N, K, A, lda, bf, acc, out + r * N);
            free(acc);
        }
    }
    free(bf);
    return failed ? -1 : 0;
}

/* Full columns: out[c*M + i] = C[i][cols[c]] for c < ncols. */
static int gemm_cols(int fmt, const Epi* ep, int64_t M, int64_t K, const uint16_t* A, int64_t lda, const uint16_t* B,
                     int64_t ldb, const int64_t* cols, int64_t ncols, uint16_t* out) {
    if (ncols <= 0 || M <= 0) return 0;
    int failed = 0;
#pragma omp parallel
    {
        float* bcol = (float*)malloc((size_t)(K > 0 ? K : 1) * sizeof(float));
        if (!bcol) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t c = 0; c < ncols; ++c) {
                int64_t j = cols[c];
                for (int64_t k = 0; k < K; ++k) bcol[k] = widen(fmt, B[k * ldb + j]);
                for (int64_t i = 0; i < M; ++i) {
                    float acc = 0.0f;
                    for (int64_t k = 0; k < K; ++k) acc = acc + widen(fmt, A[i * lda + k]) * bcol[k];
                    out[c * M + i] = epilogue(fmt, ep, j, acc);
                }
            }
            free(bcol);
        }
    }
    return failed ? -1 : 0;
}

/* Single elements: out[e] = C[ii[e]][jj[e]] for e < n. */
static int gemm_elems(int fmt, const Epi* ep, int64_t K, const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                      const int64_t* ii, const int64_t* jj, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t e = 0; e < n; ++e) {
        float acc = 0.0f;
        for (int64_t k = 0; k < K; ++k)
            acc = acc + widen(fmt, A[ii[e] * lda + k]) * widen(fmt, B[k * ldb + jj[e]]);
        out[e] = epilogue(fmt, ep, jj[e], acc);
    }
    return 0;
}

int oracle_gemm_relu_f16_full(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda,
                              const uint16_t* B, int64_t ldb, uint16_t* C, int64_t ldc) {
    return gemm_full(FMT_F16, &kRelu, M, N, K, A, lda, B, ldb, C, ldc);
}

int oracle_gemm_relu_f16_rows(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda,
                              const uint16_t* B, int64_t ldb, const int64_t* rows, int64_t nrows, uint16_t* out) {
    (void)M;
    return gemm_rows(FMT_F16, &kRelu, N, K, A, lda, B, ldb, rows, nrows, out);
}

int oracle_gemm_relu_f16_cols(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda,
                              const uint16_t* B, int64_t ldb, const int64_t* cols, int64_t ncols, uint16_t* out) {
    (void)N;
    return gemm_cols(FMT_F16, &kRelu, M, K, A, lda, B, ldb, cols, ncols, out);
}

int oracle_gemm_relu_f16_elems(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda,
                               const uint16_t* B, int64_t ldb, const int64_t* ii, const int64_t* jj, int64_t n,
                               uint16_t* out) {
    (void)M;
    (void)N;
    return gemm_elems(FMT_F16, &kRelu, K, A, lda, B, ldb, ii, jj, n, out);
}

int oracle_gemm_relu_bf16_full(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda,
                               const uint16_t* B, int64_t ldb, uint16_t* C, int64_t ldc) {
    return gemm_full(FMT_BF16, &kRelu, M, N, K, A, lda, B, ldb, C, ldc);
}

int oracle_gemm_relu_bf16_rows(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda,
                               const uint16_t* B, int64_t ldb, const int64_t* rows, int64_t nrows, uint16_t* out) {
    (void)M;
    return gemm_rows(FMT_BF16, &kRelu, N, K, A, lda, B, ldb, rows, nrows, out);
}

int oracle_gemm_relu_bf16_cols(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda,
                               const uint16_t* B, int64_t ldb, const int64_t* cols, int64_t ncols, uint16_t* out) {
    (void)N;
    return gemm_cols(FMT_BF16, &kRelu, M, K, A, lda, B, ldb, cols, ncols, out);
}

int oracle_gemm_relu_bf16_elems(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda,
                                const uint16_t* B, int64_t ldb, const int64_t* ii, const int64_t* jj, int64_t n,
                                uint16_t* out) {
    (void)M;
    (void)N;
    return gemm_elems(FMT_BF16, &kRelu, K, A, lda, B, ldb, ii, jj, n, out);
}

/* C = act(A*B + bias) in format fmt (0 = fp16, 1 = bfloat16); bias holds N
   values or is NULL.  Returns -2 for an unknown format or activation. */
static int epi_check(int fmt, int act) {
    return (fmt == FMT_F16 || fmt == FMT_BF16) && act >= 0 && act < ACT_COUNT;
}

int oracle_gemm_epi_full(int fmt, const uint16_t* bias, int act, int64_t M, int64_t N, int64_t K, const uint16_t* A,
                         int64_t lda, const uint16_t* B, int64_t ldb, uint16_t* C, int64_t ldc) {
    if (!epi_check(fmt, act)) return -2;
    const Epi ep = {bias, act, 1.0f};
    return gemm_full(fmt, &ep, M, N, K, A, lda, B, ldb, C, ldc);
}

int oracle_gemm_epi_rows(int fmt, const uint16_t* bias, int act, int64_t M, int64_t N, int64_t K, const uint16_t* A,
                         int64_t lda, const uint16_t* B, int64_t ldb, const int64_t* rows, int64_t nrows,
                         uint16_t* out) {
    (void)M;
    if (!epi_check(fmt, act)) return -2;
    const Epi ep = {bias, act, 1.0f};
    return gemm_rows(fmt, &ep, N, K, A, lda, B, ldb, rows, nrows, out);
}

int oracle_gemm_epi_cols(int fmt, const uint16_t* bias, int act, int64_t M, int64_t N, int64_t K, const uint16_t* A,
                         int64_t lda, const uint16_t* B, int64_t ldb, const int64_t* cols, int64_t ncols,
                         uint16_t* out) {
    (void)N;
    if (!epi_check(fmt, act)) return -2;
    const Epi ep = {bias, act, 1.0f};
    return gemm_cols(fmt, &ep, M, K, A, lda, B, ldb, cols, ncols, out);
}

int oracle_gemm_epi_elems(int fmt, const uint16_t* bias, int act, int64_t M, int64_t N, int64_t K,
                          const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, const int64_t* ii,
                          const int64_t* jj, int64_t n, uint16_t* out) {
    (void)M;
    (void)N;
    if (!epi_check(fmt, act)) return -2;
    const Epi ep = {bias, act, 1.0f};
    return gemm_elems(fmt, &ep, K, A, lda, B, ldb, ii, jj, n, out);
}

/* ---- fp8 (E4M3) operands, B given transposed ---------------------------------- */

/* One output element of the fp8 product. */
static uint16_t fp8_element(int fmt, const Epi* ep, int64_t i, int64_t j, int64_t K, const uint8_t* A, int64_t lda,
                            const uint8_t* Bt, int64_t ldbt) {
    float acc = 0.0f;
    for (int64_t k = 0; k < K; ++k)
        acc = acc + oracle_e4m3_to_f32(A[i * lda + k]) * oracle_e4m3_to_f32(Bt[j * ldbt + k]);
    return epilogue(fmt, ep, j, acc);
}

/* C[i*ldc + j] for all i < M, j < N.  fmt: output format (0 fp16, 1 bf16).
   Returns -2 for an unknown format or activation. */
int oracle_gemm_fp8_bt_full(int fmt, const uint16_t* bias, int act, float scale_a, float scale_b, int64_t M,
                            int64_t N, int64_t K, const uint8_t* A, int64_t lda, const uint8_t* Bt, int64_t ldbt,
                            uint16_t* C, int64_t ldc) {
    if (!epi_check(fmt, act)) return -2;
    const Epi ep = {bias, act, scale_a * scale_b};
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j) C[i * ldc + j] = fp8_element(fmt, &ep, i, j, K, A, lda, Bt, ldbt);
    return 0;
}

/* Single elements: out[e] = C[ii[e]][jj[e]]. */
int oracle_gemm_fp8_bt_elems(int fmt, const uint16_t* bias, int act, float scale_a, float scale_b, int64_t M,
                             int64_t N, int64_t K, const uint8_t* A, int64_t lda, const uint8_t* Bt, int64_t ldbt,
                             const int64_t* ii, const int64_t* jj, int64_t n, uint16_t* out) {
    (void)M;
    (void)N;
    if (!epi_check(fmt, act)) return -2;
    const Epi ep = {bias, act, scale_a * scale_b};
#pragma omp parallel for schedule(static)
    for (int64_t e = 0; e < n; ++e) out[e] = fp8_element(fmt, &ep, ii[e], jj[e], K, A, lda, Bt, ldbt);
    return 0;
}

/* ---- MX fp8: E4M3 elements with one E8M0 scale per 32 consecutive k --------- */

/* E8M0: 2^(x - 127) for x = 0 .. 254 (2^-127 .. 2^127), NaN for 255. */
double oracle_e8m0_to_f64(uint8_t x) {
    if (x == 255u) return NAN;
    return ldexp(1.0, (int)x - 127);
}

void oracle_e8m0_to_f64_array(const uint8_t* in, double* out, int64_t n) {
    for (int64_t e = 0; e < n; ++e) out[e] = oracle_e8m0_to_f64(in[e]);
}

/* One output element of the MX product: scaled products formed exactly in
   double, converted to fp32, added in fp32 in increasing k. */
static uint16_t mx_element(int fmt, const Epi* ep, int64_t i, int64_t j, int64_t K, const uint8_t* A, int64_t lda,
                           const uint8_t* SA, int64_t ldsa, const uint8_t* Bt, int64_t ldbt, const uint8_t* SB,
                           int64_t ldsb) {
    float acc = 0.0f;
    for (int64_t k = 0; k < K; ++k) {
        const double a = (double)oracle_e4m3_to_f32(A[i * lda + k]) * oracle_e8m0_to_f64(SA[i * ldsa + k / 32]);
        const double b = (double)oracle_e4m3_to_f32(Bt[j * ldbt + k]) * oracle_e8m0_to_f64(SB[j * ldsb + k / 32]);
        acc = acc + (float)(a * b);
    }
    return epilogue(fmt, ep, j, acc);
}

/* C[i*ldc + j] for all i < M, j < N.  K is a multiple of 32; SA is M x K/32
   (pitch ldsa), SB is N x K/32 (pitch ldsb).  Returns -2 for an unknown
   format or activation, -3 when K is not a multiple of 32. */
int oracle_gemm_mxfp8_bt_full(int fmt, const uint16_t* bias, int act, int64_t M, int64_t N, int64_t K,
                              const uint8_t* A, int64_t lda, const uint8_t* SA, int64_t ldsa, const uint8_t* Bt,
                              int64_t ldbt, const uint8_t* SB, int64_t ldsb, uint16_t* C, int64_t ldc) {
    if (!epi_check(fmt, act)) return -2;
    if (K % 32 != 0) return -3;
    const Epi ep = {bias, act, 1.0f};
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j)
            C[i * ldc + j] = mx_element(fmt, &ep, i, j, K, A, lda, SA, ldsa, Bt, ldbt, SB, ldsb);
    return 0;
}

/* Single elements: out[e] = C[ii[e]][jj[e]]. */
int oracle_gemm_mxfp8_bt_elems(int fmt, const uint16_t* bias, int act, int64_t M, int64_t N, int64_t K,
                               const uint8_t* A, int64_t lda, const uint8_t* SA, int64_t ldsa, const uint8_t* Bt,
                               int64_t ldbt, const uint8_t* SB, int64_t ldsb, const int64_t* ii, const int64_t* jj,
                               int64_t n, uint16_t* out) {
    (void)M;
    (void)N;
    if (!epi_check(fmt, act)) return -2;
    if (K % 32 != 0) return -3;
    const Epi ep = {bias, act, 1.0f};
#pragma omp parallel for schedule(static)
    for (int64_t e = 0; e < n; ++e)
        out[e] = mx_element(fmt, &ep, ii[e], jj[e], K, A, lda, SA, ldsa, Bt, ldbt, SB, ldsb);
    return 0;
}

/* ---- MX fp4: E2M1 elements (two per byte) with one E8M0 scale per 32 k ------- */

/* E2M1: bit 3 sign, bits 2..1 exponent (bias 1), bit 0 fraction; exponent 0
   is the subnormal 0.5 * m.  No infinity or NaN. */
float oracle_e2m1_to_f32(uint8_t nib) {
    const int sign = (nib >> 3) & 1, e = (nib >> 1) & 3, m = nib & 1;
    const float v = e == 0 ? 0.5f * (float)m : ldexpf(1.0f + 0.5f * (float)m, e - 1);
    return sign ? -v : v;
}

void oracle_e2m1_to_f32_array(const uint8_t* in, float* out, int64_t n) {
    for (int64_t e = 0; e < n; ++e) out[e] = oracle_e2m1_to_f32(in[e] & 15u);
}

/* Element k of a row of packed E2M1. */
static float e2m1_at(const uint8_t* row, int64_t k) {
    const uint8_t b = row[k >> 1];
    return oracle_e2m1_to_f32((k & 1) ? (uint8_t)(b >> 4) : (uint8_t)(b & 15u));
}

static uint16_t mx4_element(int fmt, const Epi* ep, int64_t i, int64_t j, int64_t K, const uint8_t* A,
                            int64_t lda, const uint8_t* SA, int64_t ldsa, const uint8_t* Bt, int64_t ldbt,
                            const uint8_t* SB, int64_t ldsb) {
    float acc = 0.0f;
    for (int64_t k = 0; k < K; ++k) {
        const double a = (double)e2m1_at(A + i * lda, k) * oracle_e8m0_to_f64(SA[i * ldsa + k / 32]);
        const double b = (double)e2m1_at(Bt + j * ldbt, k) * oracle_e8m0_to_f64(SB[j * ldsb + k / 32]);
        acc = acc + (float)(a * b);
    }
    return epilogue(fmt, ep, j, acc);
}

/* As oracle_gemm_mxfp8_bt_full with packed E2M1 operands (lda, ldbt in
   bytes, at least K/2). */
int oracle_gemm_mxfp4_bt_full(int fmt, const uint16_t* bias, int act, int64_t M, int64_t N, int64_t K,
                              const uint8_t* A, int64_t lda, const uint8_t* SA, int64_t ldsa, const uint8_t* Bt,
                              int64_t ldbt, const uint8_t* SB, int64_t ldsb, uint16_t* C, int64_t ldc) {
    if (!epi_check(fmt, act)) return -2;
    if (K % 32 != 0) return -3;
    const Epi ep = {bias, act, 1.0f};
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j)
            C[i * ldc + j] = mx4_element(fmt, &ep, i, j, K, A, lda, SA, ldsa, Bt, ldbt, SB, ldsb);
    return 0;
}

int oracle_gemm_mxfp4_bt_elems(int fmt, const uint16_t* bias, int act, int64_t M, int64_t N, int64_t K,
                               const uint8_t* A, int64_t lda, const uint8_t* SA, int64_t ldsa, const uint8_t* Bt,
                               int64_t ldbt, const uint8_t* SB, int64_t ldsb, const int64_t* ii, const int64_t* jj,
                               int64_t n, uint16_t* out) {
    (void)M;
    (void)N;
    if (!epi_check(fmt, act)) return -2;
    if (K % 32 != 0) return -3;
    const Epi ep = {bias, act, 1.0f};
#pragma omp parallel for schedule(static)
    for (int64_t e = 0; e < n; ++e)
        out[e] = mx4_element(fmt, &ep, ii[e], jj[e], K, A, lda, SA, ldsa, Bt, ldbt, SB, ldsb);
    return 0;
}
