/*
 * Plain fp64 CPU oracle for the block-wise INT4 MatMulNBits decode GEMV.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file or the library built from it; only the test suite, the
 * smoke check and the CPU-baseline leg of the benchmark use it.  It shares no
 * code, header, table or helper with the HIP implementation.
 *
 * What it computes (the definition, written out without blocking or fusion):
 *
 *   y[r][n] = sum_k a[r][k] * w[n][k],   w[n][k] = (q[n][k] - z[n][k/32]) * s[n][k/32]
 *
 * as described on the onnx-genai pages "perf(cuda): let the split-K decode
 * GEMV store bf16 directly" (first paragraphs: block-32 INT4 weights, fp32
 * accumulator rounded to fp16 in the epilogue) and "PORT-1 (offline
 * bias+interleave)" (the asymmetric zero-point subtract and the +8 bias of
 * the symmetric case, in "Why the premise fails here", item 1).
 *
 * Steps, in order:
 *   1. activations: an fp16 input is widened exactly; a bf16 input is first
 *      rounded to fp16 (round to nearest, ties to even), then widened;
 *   2. dequantisation of every weight to fp64, which is exact; with
 *      weights_f16 set, each weight is then rounded to fp16 (RNE, gradual
 *      underflow), the packed-half dequant of the second page's GEMV ("Why
 *      the premise fails here", item 3) that the prefill kernel follows;
 *   3. the dot product in fp64 in ascending k (every product is exact);
 *   4. one rounding of that fp64 sum to fp16 (RNE, gradual underflow,
 *      overflow to infinity);
 *   5. for bf16 output, the fp16 value is narrowed to bf16 (RNE): the
 *      fp32 -> fp16 -> bf16 double rounding that the first page's second
 *      paragraph states the bf16 arm must reproduce.
 *
 * Layout readings (the pages do not print them):
 *   Bpacked     [N][K/2] bytes, byte k/2 of row n holds k (even k: low nibble,
 *               odd k: high nibble);
 *   scales      [N][K/32] fp16 bit patterns;
 *   zero_points [N][ceil(K/64)] bytes, block b in byte b/2 (even b: low
 *               nibble, odd b: high nibble); NULL means every zero point is 8;
 *   A           [m][K] fp16 or bf16 bit patterns, row-major;
 *   outputs     [m][ncols] row-major over the requested columns.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- rounding, from the IEEE-754 definition ----------------------------- */

/* Round x to the nearest number with p significand bits (implicit bit
 * included) whose exponent is at least emin (gradual underflow below it);
 * ties go to the candidate with an even last significand bit.  The result is
 * returned exactly as a double.  Range overflow is left to the encoder. */
static double round_to_format(double x, int p, int emin)
{
    if (x == 0.0 || isnan(x) || isinf(x)) return x;
    double ax = fabs(x);
    int ex;
    frexp(ax, &ex);              /* ax in [2^(ex-1), 2^ex) */
    int e = ex - 1;
    if (e < emin) e = emin;      /* subnormal: the quantum stops shrinking */
    int qexp = e - (p - 1);      /* spacing of representable numbers: 2^qexp */
    double r = ldexp(ax, -qexp); /* exact: scaling by a power of two */
    double n = floor(r);
    double frac = r - n;         /* exact */
    if (frac > 0.5 || (frac == 0.5 && fmod(n, 2.0) != 0.0)) n += 1.0;
    return copysign(ldexp(n, qexp), x);
}

/* Encode a value that is already representable (or beyond the largest
 * finite value, which becomes infinity) into a binary format with p
 * significand bits, exponent bias `bias`, w exponent bits. */
static uint32_t encode_format(double v, int p, int bias, int w, double maxfinite)
{
    uint32_t sign = signbit(v) ? 1u : 0u;
    uint32_t sbit = sign << (p - 1 + w);
    uint32_t expall = (1u << w) - 1u;
    if (isnan(v)) return sbit | (expall << (p - 1)) | (1u << (p - 2)); /* quiet NaN */
    double av = fabs(v);
    if (isinf(v) || av > maxfinite) return sbit | (expall << (p - 1));
    if (av == 0.0) return sbit;
    int ex;
    frexp(av, &ex);
    int e = ex - 1;
    int emin = 1 - bias;
    if (e < emin) { /* subnormal: exponent field 0, significand = av / 2^(emin-(p-1)) */
        double mant = ldexp(av, -(emin - (p - 1)));
        return sbit | (uint32_t)mant;
    }
    double mant = ldexp(av, -(e - (p - 1))) - ldexp(1.0, p - 1);
    return sbit | ((uint32_t)(e + bias) << (p - 1)) | (uint32_t)mant;
}

/* fp16: 11 significand bits, 5 exponent bits, bias 15, largest finite 65504. */
uint16_t mnb_oracle_f64_to_f16(double x)
{
    double v = round_to_format(x, 11, -14);
    return (uint16_t)encode_format(v, 11, 15, 5, 65504.0);
}

/* bf16: 8 significand bits, 8 exponent bits, bias 127. */
static uint16_t f64_to_bf16(double x)
{
    double v = round_to_format(x, 8, -126);
    return (uint16_t)encode_format(v, 8, 127, 8, ldexp(255.0, 120));
}

/* Exact value of an fp16 bit pattern. */
double mnb_oracle_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1F;
    int mant = h & 0x3FF;
    double v;
    if (expo == 0) v = ldexp((double)mant, -24);
    else if (expo == 31) v = mant ? NAN : INFINITY;
    else v = ldexp((double)(mant + 1024), expo - 25);
    return sign ? -v : v;
}

/* Exact value of a bf16 bit pattern (the upper half of an fp32). */
double mnb_oracle_bf16_to_f64(uint16_t b)
{
    int sign = (b >> 15) & 1;
    int expo = (b >> 7) & 0xFF;
    int mant = b & 0x7F;
    double v;
    if (expo == 0) v = ldexp((double)mant, -133);
    else if (expo == 255) v = mant ? NAN : INFINITY;
    else v = ldexp((double)(mant + 128), expo - 134);
    return sign ? -v : v;
}

/* Narrowing of an fp16 result to bf16: the fp16 value (exact in fp32 and in
 * fp64) is rounded once to bf16, ties to even.  A NaN stays a quiet NaN with
 * its sign; infinities stay infinities. */
uint16_t mnb_oracle_f16_to_bf16(uint16_t h)
{
    double v = mnb_oracle_f16_to_f64(h);
    if (isnan(v)) return (uint16_t)(((h >> 15) << 15) | 0x7FC0);
    return f64_to_bf16(v);
}

/* A bf16 activation converted to fp16 for the dot product (RNE). */
uint16_t mnb_oracle_bf16_to_f16(uint16_t b)
{
    double v = mnb_oracle_bf16_to_f64(b);
    if (isnan(v)) return (uint16_t)(((b >> 15) << 15) | 0x7E00);
    return mnb_oracle_f64_to_f16(v);
}

/* Array forms, for the exhaustive checks of the rounding routines. */
void mnb_oracle_f64_to_f16_array(const double* x, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = mnb_oracle_f64_to_f16(x[i]);
}
void mnb_oracle_f16_to_bf16_array(const uint16_t* h, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = mnb_oracle_f16_to_bf16(h[i]);
}
void mnb_oracle_bf16_to_f16_array(const uint16_t* b, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = mnb_oracle_bf16_to_f16(b[i]);
}

/* ---- the GEMV ------------------------------------------------------------ */

/* Weight q[n][k]: byte k/2 of row n, low nibble for even k. */
static int weight_nibble(const uint8_t* B, int64_t K, int64_t n, int64_t k)
{
    uint8_t byte = B[n * (K / 2) + k / 2];
    return (k % 2 == 0) ? (byte & 0xF) : (byte >> 4);
}

/* Zero point of block b of column n; 8 when no zero points are given. */
static int zero_point(const uint8_t* zp, int64_t nblocks, int64_t n, int64_t b)
{
    if (zp == NULL) return 8;
    int64_t zrow = (nblocks + 1) / 2;
    uint8_t byte = zp[n * zrow + b / 2];
    return (b % 2 == 0) ? (byte & 0xF) : (byte >> 4);
}

/*
 * Compute the requested columns of y.
 *   A_bits      m*K activation bit patterns, a_is_bf16 selects the format
 *   cols        ncols column indices into [0, N), or NULL for all N columns
 *   y_f16       [m][ncols] fp16 results (step 4)
 *   y_bf16      [m][ncols] narrowed results (step 5), may be NULL
 *   y_f64       [m][ncols] unrounded fp64 sums, may be NULL
 *   abs_sum     [m][ncols] sum of |a*w| (for the tolerance), may be NULL
 *   nthreads    OpenMP threads over columns (<=0: the runtime's default)
 *   weights_f16 nonzero: round each dequantised weight to fp16 (step 2)
 * Returns 0, or -1 for arguments it cannot use.
 */
int mnb_oracle_matmul_nbits(const uint16_t* A_bits, int a_is_bf16,
                            int64_t m, int64_t K, int64_t N,
                            const uint8_t* B, const uint16_t* scales,
                            const uint8_t* zp,
                            const int64_t* cols, int64_t ncols,
                            uint16_t* y_f16, uint16_t* y_bf16,
                            double* y_f64, double* abs_sum, int nthreads,
                            int weights_f16)
{
    if (m < 0 || K < 0 || N < 0 || K % 32 != 0) return -1;
    if (cols == NULL) ncols = N;
    if (m == 0 || ncols == 0) return 0;
    int64_t nblocks = K / 32;

    /* step 1: activations as exact fp64 values of their fp16 form */
    double* a = (double*)malloc(sizeof(double) * (size_t)(m * K > 0 ? m * K : 1));
    if (!a) return -1;
    for (int64_t i = 0; i < m * K; ++i) {
        uint16_t h = a_is_bf16 ? mnb_oracle_bf16_to_f16(A_bits[i]) : A_bits[i];
        a[i] = mnb_oracle_f16_to_f64(h);
    }

#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 16) num_threads(nthreads)
#endif
    for (int64_t c = 0; c < ncols; ++c) {
        int64_t n = cols ? cols[c] : c;
        for (int64_t r = 0; r < m; ++r) {
            double sum = 0.0, asum = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                int64_t b = k / 32;
                double s = mnb_oracle_f16_to_f64(scales[n * nblocks + b]);
                int z = zero_point(zp, nblocks, n, b);
                int q = weight_nibble(B, K, n, k);
                double w = (double)(q - z) * s;      /* step 2, exact */
                if (weights_f16) w = mnb_oracle_f16_to_f64(mnb_oracle_f64_to_f16(w));
                double p = a[r * K + k] * w;         /* exact product */
                sum += p;                            /* step 3 */
                asum += fabs(p);
            }
            int64_t o = r * ncols + c;
            uint16_t h = mnb_oracle_f64_to_f16(sum); /* step 4 */
            y_f16[o] = h;
            if (y_bf16) y_bf16[o] = mnb_oracle_f16_to_bf16(h); /* step 5 */
            if (y_f64) y_f64[o] = sum;
            if (abs_sum) abs_sum[o] = asum;
        }
    }
    free(a);
    return 0;
}

int mnb_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
