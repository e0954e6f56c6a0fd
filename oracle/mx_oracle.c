/*
 * mx_oracle.c -- CPU oracle for the W4A4 microscaling linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the plain, slow definition that the GPU
 * library is checked against.  Only the test suite, the package smoke check
 * and the benchmark's CPU-baseline leg load it.  The GPU library never links,
 * includes or calls this file, and the two share no code, header or table.
 *
 * All arithmetic is exact: every quantity below is either an integer, a value
 * with at most a few dozen significant bits held in an IEEE double, or a
 * comparison between such values.  Where a result is fixed by a plain
 * definition ("the nearest grid point", "the smallest exponent such that"),
 * the code writes that definition out as a search rather than a closed form;
 * the closed forms live in the tests, which pin this file against them.
 *
 * Sources (titles of the model-card pages this build follows):
 *  [MX-27B]  Qwen3.5-27B-MXFP4-QAD-W4A4-LR1e-5-s1000, "How this checkpoint was
 *            produced" (Training row: MXFP4 weights, E2M1 elements, block-32,
 *            EVEN-rule E8M0 scales).
 *  [MX-9B]   Qwen3.5-9B-MXFP4-QAD-W4A4-LR1e-5-s3000, "Training mode" paragraph
 *            (activations quantized per token, block-32 E2M1, CEIL-rule UE8M0,
 *            distinct from the EVEN weight rule) and "Serving" (block-32 E8M0,
 *            dynamic per-token activations, FP4 GEMM).
 *  [NV-RTN]  Qwen3.5-27B-NVFP4-RTN-weight-only, introduction and "How this
 *            checkpoint was produced" (round-to-nearest onto the lattice,
 *            per-tensor input global scales).
 *  [NV-GPTQ] Qwen3.5-27B-NVFP4-GPTQ, introduction (NVFP4 with per-tensor input
 *            global scales) and the Serving-KL table (running-max input scales).
 *  [AR]      Qwen3.8-27B-MXFP8Attn-MXFP4MLP-lmheadMXFP4 (Intel AutoRound card),
 *            introduction (MXFP8 = E4M3 + E8M0 per group, MXFP4 = E2M1 + E8M0),
 *            section 2 (group_size 32, symmetric, dynamic activations) and
 *            section 7 (formats follow the OCP Microscaling specification).
 * Bit layouts of E2M1, E4M3 and E8M0 are those of the OCP Microscaling
 * Formats specification v1.0, which [AR] section 7 names.
 *
 * Readings where the pages are silent (each is listed with its reason in the
 * design notes of this repository):
 *  - a block is 32 consecutive elements along K of one row (16 for NVFP4);
 *  - element rounding is round-to-nearest, ties to the even code, and values
 *    beyond the largest magnitude saturate to it;
 *  - the sign bit of a code always copies the sign of the input, so a negative
 *    input that rounds to zero encodes as negative zero;
 *  - an all-zero block gets scale byte 0 (exponent -127);
 *  - scale exponents are clamped to [-127, 127];
 *  - NVFP4: global scale g = RNE_fp32(448*6 / tensor_amax) (1 if amax is 0),
 *    block scale s = RNE_E4M3(block_amax * g / 6) in exact reals, element code
 *    = RNE_E2M1(x * g / s) in exact reals, s == 0 gives signed zeros;
 *  - Y = A * W^T with W stored [N, K] (nn.Linear orientation).
 *  - fake quantization rounds the exact dequantized value once to bf16
 *    (nearest, ties to even; infinity from the largest finite bf16 plus half
 *    an ulp upward); a zero keeps its code's sign.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

/* element kinds and scale rules, matching the public enum values so the
 * Python side can pass the same integers (values only; no header is shared) */
enum { ORC_E2M1 = 0, ORC_E4M3 = 1 };
enum { ORC_FLOOR = 0, ORC_CEIL = 1, ORC_EVEN = 2 };

/* ------------------------------------------------------------------------ */
/* Decoders (OCP MX v1.0 bit layouts)                                        */
/* ------------------------------------------------------------------------ */

/* bf16: the upper 16 bits of an IEEE binary32. */
double orc_bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* E2M1: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0.  Exponent
 * field 0 is the subnormal range (0 or 0.5).  No Inf, no NaN. */
double orc_e2m1_value(int code)
{
    int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -mag : mag;
}

/* E4M3 ("FN" variant of OCP MX): sign bit 7, exponent bits 6..3 (bias 7),
 * mantissa bits 2..0.  Exponent field 0 is subnormal (m * 2^-9).  S.1111.111
 * is NaN; there is no Inf, so 1111.110 = 448 is the largest finite value. */
double orc_e4m3_value(int code)
{
    int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
    double mag;
    if (e == 15 && m == 7) return NAN;
    mag = (e == 0) ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
    return s ? -mag : mag;
}

/* E8M0: an unsigned biased exponent, value 2^(c-127); 255 is NaN. */
double orc_e8m0_value(int code)
{
    if (code == 255) return NAN;
    return ldexp(1.0, code - 127);
}

/* ------------------------------------------------------------------------ */
/* Element encoders: nearest grid point, ties to the even code, saturating   */
/* ------------------------------------------------------------------------ */

/* Positive magnitudes of an element type, indexed by their (unsigned) code:
 * 8 for E2M1 (0 .. 6), 127 for E4M3 (0 .. 448; code 127 is NaN).  The values
 * are the decoders' own outputs, tabulated once. */
static double grid_tab[2][128];
static int grid_ready = 0;
static void grid_init(void)
{
    int c;
    if (grid_ready) return;
    for (c = 0; c < 8; c++) grid_tab[0][c] = orc_e2m1_value(c);
    for (c = 0; c < 127; c++) grid_tab[1][c] = orc_e4m3_value(c);
    grid_ready = 1;
}
static int grid_size(int elem) { return elem == ORC_E2M1 ? 8 : 127; }
static double grid_value(int elem, int code) { return grid_tab[elem][code]; }

/*
 * Encode the exact real num/den (den > 0, num >= 0 or -0) onto the grid.
 * All comparisons are made as num <=> v*den, which is exact because every
 * grid value and every midpoint has at most 5 significant bits and den has
 * at most 24, so the product fits a double.  A plain linear search over the
 * grid finds the bracket [g_i, g_{i+1}] that holds the value; the midpoint of
 * the bracket decides, and an exact tie goes to the code with an even LSB.
 * Values above the largest magnitude saturate to it.
 */
static int encode_ratio_mag(int elem, double num, double den)
{
    int n = grid_size(elem), i;
    double top = grid_value(elem, n - 1);
    if (num >= top * den) return n - 1;
    for (i = 0; i + 1 < n; i++) {
        double lo = grid_value(elem, i), hi = grid_value(elem, i + 1);
        if (num >= lo * den && num < hi * den) {
            double mid = 0.5 * (lo + hi);
            if (num < mid * den) return i;
            if (num > mid * den) return i + 1;
            return (i % 2 == 0) ? i : i + 1;
        }
    }
    return 0; /* unreachable for num >= 0 */
}

/* Encode an exact real r (held exactly in a double). */
int orc_encode(int elem, double r)
{
    grid_init();
    int sign = signbit(r) ? 1 : 0;
    int mag = encode_ratio_mag(elem, fabs(r), 1.0);
    return elem == ORC_E2M1 ? (sign << 3) | mag : (sign << 7) | mag;
}

/* ------------------------------------------------------------------------ */
/* Shared block-32 scale rules ([MX-27B] EVEN for weights, [MX-9B] CEIL for  */
/* activations, OCP's own rule FLOOR)                                         */
/* ------------------------------------------------------------------------ */

static double elem_max(int elem) { return elem == ORC_E2M1 ? 6.0 : 448.0; }
static int elem_emax(int elem) { return elem == ORC_E2M1 ? 2 : 8; }
static int elem_mbits(int elem) { return elem == ORC_E2M1 ? 1 : 3; }

/* floor(log2(v)) for finite v > 0: frexp gives v = f * 2^x with f in
 * [0.5, 1), exactly. */
static int floor_log2(double v)
{
    int x;
    frexp(v, &x);
    return x - 1;
}

/*
 * Scale exponent e (scale = 2^e) of one block with maximum magnitude amax.
 *  FLOOR: the largest e with 2^(e + emax) <= amax (the OCP v1.0 rule).
 *  CEIL:  the smallest e with amax <= max_elem * 2^e: the tightest power of
 *         two at which no element needs clipping.
 *  EVEN:  amax rounded to the element's mantissa width (round half to even),
 *         then the FLOOR rule applied to the rounded value.
 * The exponent is clamped to [-127, 127]; amax == 0 yields -127.
 */
int orc_scale_exponent(double amax, int elem, int rule)
{
    int e;
    if (!(amax > 0.0)) return -127;
    if (rule == ORC_FLOOR) {
        e = floor_log2(amax) - elem_emax(elem);
    } else if (rule == ORC_CEIL) {
        /* start below the answer: max_elem < 2^(emax+1), so at this e the
         * bound max_elem * 2^e < 2^(floor_log2(amax) - 1) < amax fails */
        e = floor_log2(amax) - elem_emax(elem) - 2;
        while (!(amax <= elem_max(elem) * ldexp(1.0, e))) e++;
    } else {
        int E = floor_log2(amax);
        double mant = ldexp(amax, -E);                    /* in [1, 2) */
        double steps = ldexp(mant, elem_mbits(elem));      /* exact */
        double rounded = ldexp(nearbyint(steps), E - elem_mbits(elem));
        e = floor_log2(rounded) - elem_emax(elem);
    }
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e;
}

/* ------------------------------------------------------------------------ */
/* MX quantization: rows x k bf16 -> codes + one E8M0 byte per 32 along k    */
/* ------------------------------------------------------------------------ */

static void put_code(uint8_t* q, int elem, int64_t idx, int code)
{
    if (elem == ORC_E4M3) {
        q[idx] = (uint8_t)code;
    } else if (idx % 2 == 0) { /* element 2j -> low nibble of byte j */
        q[idx / 2] = (uint8_t)((q[idx / 2] & 0xF0) | (code & 0xF));
    } else {                   /* element 2j+1 -> high nibble */
        q[idx / 2] = (uint8_t)((q[idx / 2] & 0x0F) | ((code & 0xF) << 4));
    }
}

static int get_code(const uint8_t* q, int elem, int64_t idx)
{
    if (elem == ORC_E4M3) return q[idx];
    return (idx % 2 == 0) ? (q[idx / 2] & 0xF) : (q[idx / 2] >> 4);
}

/*
 * For every row and every block of 32 consecutive k: amax -> exponent by the
 * rule -> scale byte e + 127; each element encoded as x * 2^-e (exact).
 * Output: q is rows x k/2 bytes (E2M1) or rows x k bytes (E4M3), s is
 * rows x k/32 bytes.  Returns 0, or -1 if k is not a multiple of 32.
 */
int orc_mx_quantize(int elem, int rule, const uint16_t* x, int64_t rows, int64_t k,
                    uint8_t* q, uint8_t* s, int nthreads)
{
    int64_t r;
    if (k % 32 != 0 || rows < 0) return -1;
    grid_init();
#pragma omp parallel for schedule(static) num_threads(nthreads)
    for (r = 0; r < rows; r++) {
        int64_t b, i;
        for (b = 0; b < k / 32; b++) {
            double amax = 0.0;
            int e;
            for (i = 0; i < 32; i++) {
                double v = fabs(orc_bf16_value(x[r * k + b * 32 + i]));
                if (v > amax) amax = v;
            }
            e = orc_scale_exponent(amax, elem, rule);
            s[r * (k / 32) + b] = (uint8_t)(e + 127);
            for (i = 0; i < 32; i++) {
                double v = orc_bf16_value(x[r * k + b * 32 + i]);
                put_code(q, elem, r * k + b * 32 + i, orc_encode(elem, ldexp(v, -e)));
            }
        }
    }
    return 0;
}

/* Dequantize MX codes back to reals (for tests and the GEMM below). */
int orc_mx_dequantize(int elem, const uint8_t* q, const uint8_t* s, int64_t rows, int64_t k,
                      double* out, int nthreads)
{
    int64_t r;
    if (k % 32 != 0) return -1;
#pragma omp parallel for schedule(static) num_threads(nthreads)
    for (r = 0; r < rows; r++) {
        int64_t i;
        for (i = 0; i < k; i++) {
            int c = get_code(q, elem, r * k + i);
            double v = elem == ORC_E2M1 ? orc_e2m1_value(c) : orc_e4m3_value(c);
            out[r * k + i] = v * orc_e8m0_value(s[r * (k / 32) + i / 32]);
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* NVFP4 ([NV-RTN], [NV-GPTQ]): E2M1 elements, an E4M3 scale per 16 along k, */
/* and a per-tensor fp32 global scale                                        */
/* ------------------------------------------------------------------------ */

/* Largest |x| over a bf16 tensor. */
double orc_bf16_amax(const uint16_t* x, int64_t count)
{
    double m = 0.0;
    int64_t i;
    for (i = 0; i < count; i++) {
        double v = fabs(orc_bf16_value(x[i]));
        if (v > m) m = v;
    }
    return m;
}

/*
 * g = RNE_fp32(448 * 6 / amax); amax == 0 gives 1; a quotient beyond the
 * fp32 range saturates to the largest finite fp32.  The correctly rounded
 * quotient is found by testing the float candidates around the double
 * quotient: |c - 2688/amax| is compared as |c * amax - 2688|, which is exact
 * in a double (24 + 8 significant bits).  A tie goes to the even mantissa.
 */
float orc_nv_global_scale(double amax)
{
    float best, c0;
    double bestd;
    int i;
    if (!(amax > 0.0)) return 1.0f;
    /* a tensor so small that the quotient leaves the fp32 range gets the
     * largest finite fp32 (saturating reading; unreachable for amax above
     * about 8e-36) */
    if (2688.0 / amax > (double)FLT_MAX) return FLT_MAX;
    c0 = (float)(2688.0 / amax);
    best = c0;
    bestd = fabs((double)c0 * amax - 2688.0);
    for (i = -2; i <= 2; i++) {
        float c = c0;
        int j;
        for (j = 0; j < (i < 0 ? -i : i); j++) c = nextafterf(c, i < 0 ? 0.0f : INFINITY);
        {
            double d = fabs((double)c * amax - 2688.0);
            uint32_t cu, bu;
            memcpy(&cu, &c, 4);
            memcpy(&bu, &best, 4);
            if (d < bestd || (d == bestd && (cu & 1u) == 0 && (bu & 1u) == 1)) {
                best = c;
                bestd = d;
            }
        }
    }
    return best;
}

/*
 * rows x k bf16 -> q (rows x k/2, E2M1 nibbles) + s (rows x k/16, E4M3 bytes).
 * Per block of 16: s = RNE_E4M3(amax_blk * g / 6) (saturating at 448), then
 * each element is RNE_E2M1(x * g / s) (saturating at 6); s == 0 gives signed
 * zeros.  Both roundings are of exact reals (compared exactly, see
 * encode_ratio_mag).  Returns -1 if k is not a multiple of 16.
 */
int orc_nv_quantize(const uint16_t* x, int64_t rows, int64_t k, float g, uint8_t* q, uint8_t* s,
                    int nthreads)
{
    int64_t r;
    if (k % 16 != 0 || rows < 0) return -1;
    grid_init();
#pragma omp parallel for schedule(static) num_threads(nthreads)
    for (r = 0; r < rows; r++) {
        int64_t b, i;
        for (b = 0; b < k / 16; b++) {
            double amax = 0.0, sv;
            int sc;
            for (i = 0; i < 16; i++) {
                double v = fabs(orc_bf16_value(x[r * k + b * 16 + i]));
                if (v > amax) amax = v;
            }
            sc = encode_ratio_mag(ORC_E4M3, amax * (double)g, 6.0); /* amax*g exact */
            s[r * (k / 16) + b] = (uint8_t)sc;
            sv = orc_e4m3_value(sc);
            for (i = 0; i < 16; i++) {
                double v = orc_bf16_value(x[r * k + b * 16 + i]);
                int sign = signbit(v) ? 1 : 0, mag;
                mag = (sv == 0.0) ? 0 : encode_ratio_mag(ORC_E2M1, fabs(v) * (double)g, sv);
                put_code(q, ORC_E2M1, r * k + b * 16 + i, (sign << 3) | mag);
            }
        }
    }
    return 0;
}

/* Dequantized NVFP4 value: e2m1 * s / g. */
int orc_nv_dequantize(const uint8_t* q, const uint8_t* s, int64_t rows, int64_t k, float g,
                      double* out, int nthreads)
{
    int64_t r;
    if (k % 16 != 0) return -1;
#pragma omp parallel for schedule(static) num_threads(nthreads)
    for (r = 0; r < rows; r++) {
        int64_t i;
        for (i = 0; i < k; i++) {
            double v = orc_e2m1_value(get_code(q, ORC_E2M1, r * k + i));
            out[r * k + i] = v * orc_e4m3_value(s[r * (k / 16) + i / 16]) / (double)g;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* GEMM: Y[m, n] = sum_k A[m, k] * W[n, k] over the dequantized operands     */
/* ([MX-9B] "Serving": block-scaled FP4 GEMM; output is compared before any  */
/* bf16 rounding).  Also returns S[m, n] = sum_k |A[m, k] * W[n, k]|.        */
/* ------------------------------------------------------------------------ */

/* Plain dot products over dequantized rows.  For MX operands every product is
 * exact in a double; the sum is exact while the exponent spread plus log2(k)
 * stays under 53 bits. */
static void dot_rows(const double* a, const double* w, int64_t k, double* y, double* sa)
{
    double acc = 0.0, accabs = 0.0;
    int64_t i;
    for (i = 0; i < k; i++) {
        double p = a[i] * w[i];
        acc += p;
        accabs += fabs(p);
    }
    *y = acc;
    *sa = accabs;
}

/* Full product of two dequantized matrices A (m x k) and W (n x k). */
int orc_gemm_dq(const double* a, const double* w, int64_t m, int64_t n, int64_t k, double* y,
                double* sabs, int nthreads)
{
    int64_t i;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (i = 0; i < m; i++) {
        int64_t j;
        for (j = 0; j < n; j++) dot_rows(a + i * k, w + j * k, k, &y[i * n + j], &sabs[i * n + j]);
    }
    return 0;
}

/* Selected entries (mi[t], ni[t]) of the same product. */
int orc_gemm_dq_pairs(const double* a, const double* w, int64_t k, const int64_t* mi,
                      const int64_t* ni, int64_t npairs, double* y, double* sabs, int nthreads)
{
    int64_t t;
#pragma omp parallel for schedule(static) num_threads(nthreads)
    for (t = 0; t < npairs; t++) dot_rows(a + mi[t] * k, w + ni[t] * k, k, &y[t], &sabs[t]);
    return 0;
}

/*
 * The MX GEMM straight from codes, without materialising dequantized
 * matrices: each product is decoded on the fly.  Rows of A are processed
 * independently (OpenMP over m), which makes it the CPU baseline as well.
 */
int orc_mx_gemm(int a_elem, const uint8_t* aq, const uint8_t* as, int w_elem, const uint8_t* wq,
                const uint8_t* ws, int64_t m, int64_t n, int64_t k, double* y, double* sabs,
                int nthreads)
{
    int64_t i;
    if (k % 32 != 0) return -1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (i = 0; i < m; i++) {
        int64_t j, t;
        for (j = 0; j < n; j++) {
            double acc = 0.0, accabs = 0.0;
            for (t = 0; t < k; t++) {
                int ca = get_code(aq, a_elem, i * k + t), cw = get_code(wq, w_elem, j * k + t);
                double va = (a_elem == ORC_E2M1 ? orc_e2m1_value(ca) : orc_e4m3_value(ca)) *
                            orc_e8m0_value(as[i * (k / 32) + t / 32]);
                double vw = (w_elem == ORC_E2M1 ? orc_e2m1_value(cw) : orc_e4m3_value(cw)) *
                            orc_e8m0_value(ws[j * (k / 32) + t / 32]);
                acc += va * vw;
                accabs += fabs(va * vw);
            }
            y[i * n + j] = acc;
            sabs[i * n + j] = accabs;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Fake quantization: the quantize -> dequantize round trip written back as  */
/* bf16, the op that quantization-aware training runs in place of the        */
/* serving quantizer ([MX-27B] "How this checkpoint was produced": weights   */
/* and activations fake-quantized during training; [MX-9B] "Training mode": */
/* the same CEIL rule as serving).  Each output is the bf16 nearest to the   */
/* exact dequantized value, ties to the even pattern.                        */
/* ------------------------------------------------------------------------ */

/* bf16 bits (sign clear) of the value nearest to the exact ratio p / g, for
 * p >= 0 and g > 0 finite, ties to the even pattern; from the largest finite
 * bf16 plus half an ulp upward the result is infinity.  The candidates are
 * the patterns around the truncation of the double quotient, each compared
 * by its distance |b * g - p| (b * g has at most 8 + 24 significant bits, so
 * it is exact; near the quotient the difference is exact too). */
uint16_t orc_bf16_nearest_ratio(double p, double g)
{
    const double top = orc_bf16_value(0x7F7F), half_ulp = ldexp(1.0, 127 - 8);
    double q = p / g, bestd = -1.0;
    float f = (float)q;
    uint32_t fb;
    int32_t u, c;
    uint16_t best = 0;
    if (p != p) return 0x7FC0;
    if (p >= (top + half_ulp) * g) return 0x7F80;
    memcpy(&fb, &f, 4);
    u = (int32_t)(fb >> 16);
    for (c = u - 2; c <= u + 2; c++) {
        double d;
        if (c < 0 || c > 0x7F7F) continue;
        d = fabs(orc_bf16_value((uint16_t)c) * g - p);
        if (bestd < 0.0 || d < bestd || (d == bestd && (c & 1) == 0)) {
            best = (uint16_t)c;
            bestd = d;
        }
    }
    return best;
}

/*
 * rows x k bf16 -> rows x k bf16 fake-quantized values.  fmt 0: MXFP4 (E2M1,
 * E8M0 per 32 by `rule`); 1: MXFP8 (E4M3, E8M0 per 32 by `rule`); 2: NVFP4
 * (E2M1, E4M3 per 16, global scale g; `rule` unused).  The codes and scales
 * are those of orc_mx_quantize / orc_nv_quantize; MX values e * 2^(s - 127)
 * and NVFP4 values e2m1 * s / g are rounded once to bf16.  A zero value keeps
 * the sign of its code.  Returns -1 on a bad fmt or a k that is not a
 * multiple of the block, -2 if scratch memory is unavailable.
 */
int orc_fake_quant(int fmt, int rule, const uint16_t* x, int64_t rows, int64_t k, float g, uint16_t* out,
                   int nthreads)
{
    const int elem = fmt == 1 ? ORC_E4M3 : ORC_E2M1;
    const int block = fmt == 2 ? 16 : 32;
    const int64_t qbytes = elem == ORC_E2M1 ? rows * k / 2 : rows * k;
    uint8_t *q, *sc;
    int64_t i;
    int rc;
    if (fmt < 0 || fmt > 2 || k % block != 0 || rows < 0) return -1;
    q = (uint8_t*)malloc((size_t)(qbytes > 0 ? qbytes : 1));
    sc = (uint8_t*)malloc((size_t)(rows * k / block > 0 ? rows * k / block : 1));
    if (!q || !sc) {
        free(q);
        free(sc);
        return -2;
    }
    rc = fmt == 2 ? orc_nv_quantize(x, rows, k, g, q, sc, nthreads)
                  : orc_mx_quantize(elem, rule, x, rows, k, q, sc, nthreads);
    if (rc == 0) {
#pragma omp parallel for schedule(static) num_threads(nthreads)
        for (i = 0; i < rows * k; i++) {
            const int code = get_code(q, elem, i);
            const int sign = elem == ORC_E2M1 ? (code >> 3) & 1 : (code >> 7) & 1;
            double v;
            uint16_t bits;
            if (fmt == 2) {
                v = fabs(orc_e2m1_value(code) * orc_e4m3_value(sc[i / 16]));   /* exact */
                bits = v == 0.0 ? 0 : orc_bf16_nearest_ratio(v, (double)g);
            } else {
                v = fabs((elem == ORC_E2M1 ? orc_e2m1_value(code) : orc_e4m3_value(code)) *
                         orc_e8m0_value(sc[i / 32]));                          /* exact */
                bits = v == 0.0 ? 0 : orc_bf16_nearest_ratio(v, 1.0);
            }
            out[i] = (uint16_t)(bits | (sign << 15));
        }
    }
    free(q);
    free(sc);
    return rc;
}
