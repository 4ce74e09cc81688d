/*
 * CPU oracle for the quantized linear layer: TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, obviously correct loops that state what the layer computes.
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * call this file; the GPU library never links or includes it, and this file
 * includes nothing of the GPU library.  Floating point is fp64 unless the
 * definition fixes a single fp32 operation (written fl32 below); those are
 * plain C float operations, compiled with -ffp-contract=off so each one is a
 * single IEEE round-to-nearest-even operation.
 *
 * Sources (web pages, cited by title and section):
 *   [Q4]  bitorch-engine API docs, "Q4LinearFunction" - forward.
 *   [BL]  LLaMA-BitNet utils.py, "Class BitLinear" - forward docstring
 *         steps 1-5 and the forward body.
 *   [PT]  Ascend CANN ATB docs, "Per-token Quantization for Matmul" -
 *         Parameters, Input, Output and Example.
 *   [CA]  frankenstein-transformer docs, "Common Attention Utilities" -
 *         activation_quant, weight_quant, BitLinear.bake_ternary_weights.
 *   [L4]  docs.rs vyre-libs 0.7.2, "linear_4bit/mod.rs" - module doc
 *         comment and the QuantizedLinear4BitPlannerEvidence fields.
 *
 * Every function returns 0 on success and a negative value when an integer
 * accumulator would not fit in int32 (the definition asserts that it does).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* O1: per-token absmax int8 activation quantization.                  */
/* ------------------------------------------------------------------ */
/*
 * [BL] forward steps 1-2 (parameter-free RMSNorm, then 8-bit per-token
 * quantization) and step 5 (the activation scale multiplies the output);
 * [CA] activation_quant (scale the last dimension into [-128, 127], round,
 * rescale).
 *
 * For each token row m of X[m, k] (fp32 values, exact copies of the bf16 /
 * fp16 input):
 *   r   = 1                               without RMSNorm
 *   r   = 1 / sqrt(sum_k X^2 / K + eps_n) with RMSNorm (fp64)
 *   a   = max_k |X|                       (exact)
 *   t   = fl32(eps_q / r)                 (t = eps_q exactly without RMSNorm)
 *   a'  = max(a, t)                       (division guard)
 *   s   = fl32(127 / a')
 *   q   = clamp(rne(fl32(X * s)), -128, 127)
 *   pts = fp32(a' * r / 127)              (fp64, one final rounding)
 *   rowsum = sum_k q                      (int32)
 * RMSNorm multiplies the whole row by r > 0 and absmax quantization is
 * invariant under a positive per-row factor, so the codes are those of X
 * and the norm survives as the factor r in the dequant scale.  The guard
 * belongs to the quantizer, which sees the normalized row Y = r X: it takes
 * max(max|Y|, eps_q), and max(r a, eps_q) / r = max(a, eps_q / r) = a'.
 * Only rows with r a < eps_q reach the guard; their codes depend on r.
 */
int oracle_quant_act(const float *x, int64_t m, int64_t k, int rmsnorm,
                     double eps_norm, float eps_q, int8_t *q, float *pts,
                     int32_t *rowsum)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < m; i++) {
        const float *row = x + i * k;
        float a = 0.0f;
        for (int64_t j = 0; j < k; j++) {
            float v = fabsf(row[j]);
            if (v > a) a = v;
        }
        double rr = 1.0;
        if (rmsnorm) {
            double ss = 0.0;
            for (int64_t j = 0; j < k; j++) ss += (double)row[j] * (double)row[j];
            rr = 1.0 / sqrt(ss / (double)k + eps_norm);
        }
        float t = rmsnorm ? (float)((double)eps_q / rr) : eps_q;
        float ap = a > t ? a : t;
        float s = 127.0f / ap;
        int64_t sum = 0;
        for (int64_t j = 0; j < k; j++) {
            float v = row[j] * s;
            float r = nearbyintf(v);
            if (r > 127.0f) r = 127.0f;
            if (r < -128.0f) r = -128.0f;
            int8_t c = (int8_t)r;
            q[i * k + j] = c;
            sum += c;
        }
        pts[i] = (float)((double)ap * rr / 127.0);
        if (rowsum) rowsum[i] = (int32_t)sum;
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* O2: absmean ternary weight quantization and its 2-bit packing.      */
/* ------------------------------------------------------------------ */
/*
 * [BL] forward step 3 (ternary {-1, 0, +1} via absmean) and step 5 (a
 * scalar weight scale); [CA] weight_quant (scale by the inverse mean
 * absolute value, round to the nearest integer in [-1, 1]).
 *
 *   S      = sum |W|                      (exact, then rounded once to fp64)
 *   gamma  = S / count                    (one fp64 division)
 *   gamma' = max(gamma, eps)
 *   q      = sign(W) if |W| > gamma'/2 else 0
 * The comparison is exact in fp64 (halving is exact); |W| == gamma'/2
 * gives 0, which is round-half-to-even of W/gamma' = +-0.5.  Values whose
 * quotient is 1.5 or more clamp to +-1, so this equals
 * clamp(rne(W / gamma'), -1, 1) in exact arithmetic.
 *
 * w is read in its stored layout: layout 1 = [n][k] (nn.Linear weight),
 * layout 0 = [k][n].  codes are always written [n][k].
 */
/*
 * Exact sum of |w| over fp32 values.  A finite fp32 magnitude is
 * mant * 2^(e - 149) with mant < 2^24 and e = max(biased exponent - 1, 0)
 * in [0, 253], so it is an integer below 2^277 in units of 2^-149, and a sum
 * of fewer than 2^40 of them is an integer below 2^317: five 64-bit limbs
 * hold it with no rounding at all.  Non-finite inputs are not summed.
 */
typedef struct { uint64_t limb[5]; } exact_sum;

static void exact_add_limb(exact_sum *a, int i, uint64_t v)
{
    for (; i < 5 && v; i++) {
        uint64_t old = a->limb[i];
        a->limb[i] = old + v;
        v = a->limb[i] < old ? 1u : 0u;   /* carry into the next limb */
    }
}

static void exact_add_abs(exact_sum *a, float v)
{
    uint32_t bits;
    memcpy(&bits, &v, sizeof bits);
    bits &= 0x7fffffffu;
    uint32_t be = bits >> 23, frac = bits & 0x7fffffu;
    if (be == 255) return;
    uint64_t mant = be ? (frac | 0x800000u) : frac;
    int e = be ? (int)be - 1 : 0;
    int i = e / 64, off = e % 64;
    exact_add_limb(a, i, mant << off);
    if (off > 40) exact_add_limb(a, i + 1, mant >> (64 - off));
}

/* The exact sum rounded to the nearest fp64, ties to even. */
static double exact_to_double(const exact_sum *a)
{
    int top = -1;
    for (int b = 319; b >= 0; b--)
        if ((a->limb[b / 64] >> (b % 64)) & 1u) { top = b; break; }
    if (top < 0) return 0.0;
    if (top < 53) {
        /* below 2^53 units: the integer itself is exact in fp64 */
        return ldexp((double)a->limb[0], -149);
    }
    /* keep bits [top-52, top]; round on bit top-53 and the bits below it */
    int low = top - 52;
    uint64_t m = 0;
    for (int b = top; b >= low; b--) m = (m << 1) | ((a->limb[b / 64] >> (b % 64)) & 1u);
    int guard = (int)((a->limb[(low - 1) / 64] >> ((low - 1) % 64)) & 1u);
    int sticky = 0;
    for (int b = low - 2; b >= 0 && !sticky; b--) sticky = (int)((a->limb[b / 64] >> (b % 64)) & 1u);
    if (guard && (sticky || (m & 1u))) m++;   /* m may become 2^53: still exact */
    return ldexp((double)m, low - 149);
}

int oracle_ternary_quant(const float *w, int layout, int64_t n, int64_t k,
                         double eps, int8_t *codes, double *gamma_out)
{
    int64_t count = n * k;
    exact_sum acc = {{0, 0, 0, 0, 0}};
    for (int64_t i = 0; i < count; i++) exact_add_abs(&acc, w[i]);
    double g = exact_to_double(&acc) / (double)count;
    if (g < eps) g = eps;
    double half = g / 2.0;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; r++) {
        for (int64_t c = 0; c < k; c++) {
            float v = layout == 1 ? w[r * k + c] : w[c * n + r];
            double av = fabs((double)v);
            int8_t t = 0;
            if (av > half) t = v > 0.0f ? 1 : -1;
            codes[r * k + c] = t;
        }
    }
    *gamma_out = g;
    return 0;
}

/*
 * Count of weights within rel * gamma' of the rounding threshold gamma'/2:
 * the only weights whose code could depend on the summation order of the
 * absmean.
 */
int64_t oracle_ternary_tie_band(const float *w, int64_t count, double gamma,
                                double rel)
{
    int64_t c = 0;
    for (int64_t i = 0; i < count; i++)
        if (fabs(fabs((double)w[i]) - gamma / 2.0) <= rel * gamma) c++;
    return c;
}

/*
 * Ternary pack layout version 1 (our definition; the pages fix only that
 * codes are ternary and BitNet stores them in 2 bits).  Requires
 * n % 16 == 0 and k % 256 == 0.
 *   The [n][k] code matrix is cut into blocks of 16 columns x 256 k; block
 *   (nb, kb) is 256 consecutive u32 words starting at word
 *   (nb * (k / 256) + kb) * 256.
 *   Word 4*l + t of a block (l in [0, 64), t in [0, 4)) holds column
 *   16*nb + l % 16 and the 16 consecutive k starting at
 *   k0 = 256*kb + 64*(l / 16) + 16*t.
 *   Element k0 + 4*a + b (a, b in [0, 4)) sits in bits [8b + 2a, 8b + 2a + 1]
 *   as the code c = q + 1 in {0, 1, 2}.
 */
static int64_t tern_word_index(int64_t n, int64_t k, int64_t col, int64_t kk,
                               int *bitpos)
{
    int64_t nb = col / 16, kb = kk / 256;
    int64_t within = kk % 256;
    int64_t lgrp = within / 64;          /* l / 16 */
    int64_t t = (within % 64) / 16;
    int64_t e = within % 16;             /* 4a + b */
    int64_t a = e / 4, b = e % 4;
    int64_t l = lgrp * 16 + col % 16;
    (void)n;
    *bitpos = (int)(8 * b + 2 * a);
    return (nb * (k / 256) + kb) * 256 + 4 * l + t;
}

int oracle_pack_ternary_v1(const int8_t *codes, int64_t n, int64_t k,
                           uint32_t *packed)
{
    if (n % 16 || k % 256) return -2;
    memset(packed, 0, (size_t)(n * k / 16) * sizeof(uint32_t));
    for (int64_t r = 0; r < n; r++)
        for (int64_t c = 0; c < k; c++) {
            int bit;
            int64_t wi = tern_word_index(n, k, r, c, &bit);
            uint32_t code = (uint32_t)(codes[r * k + c] + 1);
            packed[wi] |= code << bit;
        }
    return 0;
}

int oracle_unpack_ternary_v1(const uint32_t *packed, int64_t n, int64_t k,
                             int8_t *codes)
{
    if (n % 16 || k % 256) return -2;
    for (int64_t r = 0; r < n; r++)
        for (int64_t c = 0; c < k; c++) {
            int bit;
            int64_t wi = tern_word_index(n, k, r, c, &bit);
            codes[r * k + c] = (int8_t)((int)((packed[wi] >> bit) & 3u) - 1);
        }
    return 0;
}

/* ------------------------------------------------------------------ */
/* O3: 4-bit packing and the grouped affine INT4 product.              */
/* ------------------------------------------------------------------ */
/*
 * [L4] module doc: the packed weight is u32 words holding eight nibbles;
 * the grouped path applies a per-group scale and zero-point (the
 * "scale plus zero-point sidecar").
 *
 * Weight layout version 1 (our definition).  Requires n % 16 == 0 and
 * k % 128 == 0.  Blocks of 16 columns x 128 k; block (nb, kb) is 256 words
 * from word (nb * (k / 128) + kb) * 256.  Word 4*l + t holds column
 * 16*nb + l % 16 and the 8 k starting at k0 = 128*kb + 32*(l / 16) + 8*t.
 * Nibble p (bits [4p, 4p + 3]) holds k-offset 2p for p < 4 and 2(p - 4) + 1
 * for p >= 4.  Only the low nibble of each input code is used.
 */
static int64_t int4_word_index(int64_t k, int64_t col, int64_t kk, int *bitpos)
{
    int64_t nb = col / 16, kb = kk / 128;
    int64_t within = kk % 128;
    int64_t lgrp = within / 32;
    int64_t t = (within % 32) / 8;
    int64_t off = within % 8;
    int64_t p = (off % 2 == 0) ? off / 2 : off / 2 + 4;
    int64_t l = lgrp * 16 + col % 16;
    *bitpos = (int)(4 * p);
    return (nb * (k / 128) + kb) * 256 + 4 * l + t;
}

int oracle_pack_int4_v1(const uint8_t *q, int64_t n, int64_t k,
                        uint32_t *packed)
{
    if (n % 16 || k % 128) return -2;
    memset(packed, 0, (size_t)(n * k / 8) * sizeof(uint32_t));
    for (int64_t r = 0; r < n; r++)
        for (int64_t c = 0; c < k; c++) {
            int bit;
            int64_t wi = int4_word_index(k, r, c, &bit);
            packed[wi] |= ((uint32_t)(q[r * k + c] & 15u)) << bit;
        }
    return 0;
}

int oracle_unpack_int4_v1(const uint32_t *packed, int64_t n, int64_t k,
                          uint8_t *q)
{
    if (n % 16 || k % 128) return -2;
    for (int64_t r = 0; r < n; r++)
        for (int64_t c = 0; c < k; c++) {
            int bit;
            int64_t wi = int4_word_index(k, r, c, &bit);
            q[r * k + c] = (uint8_t)((packed[wi] >> bit) & 15u);
        }
    return 0;
}

/*
 * Zero-points z[n][g] (g = number of groups) are stored group-major:
 * word (gi, col / 8) of a [g][n / 8] array, column col in nibble col % 8.
 * Requires n % 8 == 0.
 */
int oracle_pack_int4_zeros(const uint8_t *z, int64_t n, int64_t g,
                           uint32_t *packed)
{
    if (n % 8) return -2;
    memset(packed, 0, (size_t)(g * n / 8) * sizeof(uint32_t));
    for (int64_t r = 0; r < n; r++)
        for (int64_t gi = 0; gi < g; gi++)
            packed[gi * (n / 8) + r / 8] |= ((uint32_t)(z[r * g + gi] & 15u))
                                            << (4 * (r % 8));
    return 0;
}

/*
 * y[m][n] = sum_g s[n][g] * sum_{k in g} x[m][k] * (q[n][k] - z[n][g])
 * in fp64; also bound[m][n] = sum_k |x[m][k] * w[n][k]| with the dequantized
 * weight w = s * (q - z), the scale of the error allowed for this path.
 * x and s hold the fp16 input values widened exactly to fp64.
 */
int oracle_grouped_int4(const double *x, const uint8_t *q, const double *s,
                        const uint8_t *z, int64_t group_size, int64_t m,
                        int64_t n, int64_t k, double *y, double *bound)
{
    int64_t ng = k / group_size;
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < n; c++) {
        for (int64_t r = 0; r < m; r++) {
            double acc = 0.0, ab = 0.0;
            for (int64_t gi = 0; gi < ng; gi++) {
                double sg = s[c * ng + gi];
                int zg = z[c * ng + gi] & 15;
                double part = 0.0;
                for (int64_t j = gi * group_size; j < (gi + 1) * group_size; j++) {
                    int d = (int)(q[c * k + j] & 15) - zg;
                    part += x[r * k + j] * (double)d;
                    ab += fabs(x[r * k + j] * sg * (double)d);
                }
                acc += sg * part;
            }
            y[r * n + c] = acc;
            if (bound) bound[r * n + c] = ab;
        }
    }
    return 0;
}

/*
 * The same grouped affine INT4 linear with int8 activation codes and their
 * per-token scale ([L4] module doc for the weight side; the per-token int8
 * activation of [BL] steps 2 and 5 for the input side):
 *   y[m][n] = pts[m] * sum_g s[n][g] * sum_{k in g} xq[m][k] * (q[n][k] - z[n][g])
 * The inner sums are exact integers (int64); the rest is fp64.
 *   bound[m][n] = |pts[m]| * sum_k |xq[m][k] * s[n][g(k)] * (q[n][k] - z[n][g(k)])|
 */
int oracle_grouped_int4_i8(const int8_t *xq, const float *pts, const uint8_t *q,
                           const double *s, const uint8_t *z, int64_t group_size,
                           int64_t m, int64_t n, int64_t k, double *y, double *bound)
{
    int64_t ng = k / group_size;
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < n; c++) {
        for (int64_t r = 0; r < m; r++) {
            double acc = 0.0, ab = 0.0;
            for (int64_t gi = 0; gi < ng; gi++) {
                double sg = s[c * ng + gi];
                int zg = z[c * ng + gi] & 15;
                int64_t part = 0, apart = 0;
                for (int64_t j = gi * group_size; j < (gi + 1) * group_size; j++) {
                    int64_t d = (int64_t)xq[r * k + j] * ((int)(q[c * k + j] & 15) - zg);
                    part += d;
                    apart += d < 0 ? -d : d;
                }
                acc += sg * (double)part;
                ab += fabs(sg) * (double)apart;
            }
            y[r * n + c] = (double)pts[r] * acc;
            if (bound) bound[r * n + c] = fabs((double)pts[r]) * ab;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* O4: integer GEMM and the per-token dequant epilogue.                */
/* ------------------------------------------------------------------ */
/*
 * [PT] Input (x int8 [m,k], weight int8 [k,n], deqScale [n],
 * perTokenScale [m]), Parameters (transposeB), Output ([m,n] fp16 / bf16)
 * and Example: out[m][n] = (sum_k x[m][k] * w[k][n]) * deqScale[n] *
 * perTokenScale[m].
 * acc is accumulated in int64 and must fit int32.
 * layout 0: w is [k][n]; layout 1: w is [n][k] (transposeB).
 */
int oracle_gemm_i8(const int8_t *x, const int8_t *w, int layout, int64_t m,
                   int64_t n, int64_t k, int32_t *acc)
{
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t r = 0; r < m; r++) {
        for (int64_t c = 0; c < n; c++) {
            int64_t s = 0;
            for (int64_t j = 0; j < k; j++) {
                int64_t wv = layout == 1 ? w[c * k + j] : w[j * n + c];
                s += (int64_t)x[r * k + j] * wv;
            }
            if (s > INT32_MAX || s < INT32_MIN) bad = 1;
            acc[r * n + c] = (int32_t)s;
        }
    }
    return bad ? -1 : 0;
}

/* y[m][n] = acc[m][n] * pts[m] * deq[n] in fp64 ([PT] Example; [BL] step 5). */
int oracle_dequant(const int32_t *acc, const float *pts, const float *deq,
                   int64_t m, int64_t n, double *y)
{
    for (int64_t r = 0; r < m; r++)
        for (int64_t c = 0; c < n; c++)
            y[r * n + c] = (double)acc[r * n + c] * (double)pts[r] * (double)deq[c];
    return 0;
}

/* ------------------------------------------------------------------ */
/* O5: A4W4 per-tensor 4-bit quantization ([Q4] forward).             */
/* ------------------------------------------------------------------ */
/*
 * [Q4] forward: inputs and weights are quantized to 4 bits with the given
 * scale factors; eps avoids division by zero.
 *   s' = max(scale, eps)
 *   q  = clamp(rne(fl32(X / s')), -8, 7)
 * The product is then oracle_gemm_i8 (layout [n][k]) and the dequant is
 * acc * s'_a * s'_w in fp64.
 */
int oracle_quant_int4_tensor(const float *x, int64_t count, float scale,
                             float eps, int8_t *q)
{
    float sp = scale > eps ? scale : eps;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; i++) {
        float v = x[i] / sp;
        float r = nearbyintf(v);
        if (r > 7.0f) r = 7.0f;
        if (r < -8.0f) r = -8.0f;
        q[i] = (int8_t)r;
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Q4Linear backward.                                                   */
/* ------------------------------------------------------------------ */
/*
 * [Q4] backward: gradients for the input, the weight and the activation
 * scale from the output gradient, "adjusted to the quantization ranges";
 * none for scale_w and eps.  The page states it only in words; this is
 * the straight-through reading with the clipping range and the learned
 * step size term for the scale:
 *   forward  y = Xh Wh^T, Xh = s'_a q_a, Wh = s'_w q_w (the codes of
 *            oracle_quant_int4_tensor), v = fl32(X / s') the quotient the
 *            code rounds
 *   dXh = G Wh       [m, n] x [n, k]          (fp64)
 *   dWh = G^T Xh     [n, m] x [m, k]          (fp64)
 *   in  = (-8 <= v <= 7)                      (the clip range)
 *   grad_x = dXh * in_a,  grad_w = dWh * in_w (round passes the gradient)
 *   grad_scale_a = sum dXh * (q_a - v_a * in_a) when scale_a > eps, else 0
 *                  (d(s round(x/s))/ds = round(v) - v inside the range,
 *                  the clamp bound outside; s' = eps does not depend on s)
 * G [m, n] fp64 (exact copies of the fp16 / bf16 gradient), X [m, k],
 * W [n, k] fp32 (exact copies).  Also returns, for tolerances,
 *   bx = s'_w sum_n |G q_w|, bw = s'_a sum_m |G q_a|,
 *   bs = sum |bx (q_a - v_a in_a)|.
 */
static float q4_quotient(float x, float sp) { return x / sp; }

int oracle_q4_backward(const double *g, const float *x, const float *w, float scale_a, float scale_w,
                       float eps, int64_t m, int64_t n, int64_t k, double *grad_x, double *grad_w,
                       double *grad_sa, double *bx, double *bw, double *bs)
{
    float spa = scale_a > eps ? scale_a : eps, spw = scale_w > eps ? scale_w : eps;
    int8_t *qa = malloc((size_t)(m * k)), *qw = malloc((size_t)(n * k));
    unsigned char *ina = malloc((size_t)(m * k)), *inw = malloc((size_t)(n * k));
    float *va = malloc(sizeof(float) * (size_t)(m * k));
    double total = 0.0, abs_total = 0.0;
    if (!qa || !qw || !ina || !inw || !va) return -2;
    oracle_quant_int4_tensor(x, m * k, scale_a, eps, qa);
    oracle_quant_int4_tensor(w, n * k, scale_w, eps, qw);
    for (int64_t i = 0; i < m * k; i++) {
        va[i] = q4_quotient(x[i], spa);
        ina[i] = (va[i] >= -8.0f && va[i] <= 7.0f);
    }
    for (int64_t i = 0; i < n * k; i++) {
        float v = q4_quotient(w[i], spw);
        inw[i] = (v >= -8.0f && v <= 7.0f);
    }
#pragma omp parallel for schedule(static) reduction(+ : total, abs_total)
    for (int64_t i = 0; i < m; i++)
        for (int64_t c = 0; c < k; c++) {
            double d = 0.0, a = 0.0;
            for (int64_t j = 0; j < n; j++) {
                d += g[i * n + j] * (double)qw[j * k + c];
                a += fabs(g[i * n + j] * (double)qw[j * k + c]);
            }
            d *= (double)spw;
            bx[i * k + c] = a * (double)spw;
            grad_x[i * k + c] = ina[i * k + c] ? d : 0.0;
            double t = (double)qa[i * k + c] - (ina[i * k + c] ? (double)va[i * k + c] : 0.0);
            total += d * t;
            abs_total += a * (double)spw * fabs(t);
        }
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; j++)
        for (int64_t c = 0; c < k; c++) {
            double d = 0.0, a = 0.0;
            for (int64_t i = 0; i < m; i++) {
                d += g[i * n + j] * (double)qa[i * k + c];
                a += fabs(g[i * n + j] * (double)qa[i * k + c]);
            }
            d *= (double)spa;
            bw[j * k + c] = a * (double)spa;
            grad_w[j * k + c] = inw[j * k + c] ? d : 0.0;
        }
    *grad_sa = scale_a > eps ? total : 0.0;
    *bs = abs_total;
    free(qa); free(qw); free(ina); free(inw); free(va);
    return 0;
}

/* ------------------------------------------------------------------ */
/* A4W4 operand tiles: 4-bit codes written as FP6 E3M2 values.          */
/* ------------------------------------------------------------------ */
/*
 * Not a format of the pages: this project's packed operand for the 4-bit
 * product ("Q4LinearFunction" forward multiplies 4-bit codes in [-8, 7]).
 * Each code is written as the FP6 E3M2 number of the same value (OCP
 * Microscaling Formats v1.0: 1 sign bit, 3 exponent bits with bias 3, 2
 * mantissa bits; every integer in [-8, 7] is exact).  Rows are padded with
 * zero codes to a multiple of 32 and k to a multiple of 128.  Tile (rb, ks)
 * covers rows 32rb .. 32rb+31 and k 64ks .. 64ks+63 and occupies 1536 bytes
 * at (rb * (kp / 64) + ks) * 1536.  Slot l (0..63) of a tile holds row
 * 32rb + l % 32 and k 64ks + 32(l / 32) + j for j = 0..31 as a 192-bit
 * little-endian string with element j in bits 6j .. 6j+5; its bytes 0..15
 * sit at tile byte 16l and bytes 16..23 at tile byte 1024 + 8l.
 * Parity unpinned beyond its definition: tests decode it and compare codes.
 */
static unsigned e3m2_of_code(int c)
{
    unsigned sign = c < 0 ? 1u : 0u;
    unsigned a = (unsigned)(c < 0 ? -c : c);
    unsigned e = 0, m;
    if (a == 0) return 0u;
    /* a = 2^p * (1 + m/4) with p = floor(log2 a); biased exponent p + 3 */
    while ((2u << e) <= a) e++;
    m = (a * 4u) / (1u << e) - 4u;
    return (sign << 5) | ((e + 3u) << 2) | m;
}

int64_t oracle_a4w4_operand_bytes(int64_t rows, int64_t k)
{
    int64_t rp = (rows + 31) / 32 * 32, kp = (k + 127) / 128 * 128;
    return rp * kp * 3 / 4;
}

int oracle_pack_a4w4_fp6(const int8_t *codes, int64_t rows, int64_t k, uint8_t *out)
{
    int64_t rp = (rows + 31) / 32 * 32, kp = (k + 127) / 128 * 128;
    int64_t kt = kp / 64;
    for (int64_t rb = 0; rb < rp / 32; rb++)
        for (int64_t ks = 0; ks < kt; ks++) {
            uint8_t *tile = out + (rb * kt + ks) * 1536;
            for (int l = 0; l < 64; l++) {
                uint8_t img[24] = {0};
                int64_t row = 32 * rb + l % 32;
                for (int j = 0; j < 32; j++) {
                    int64_t kk = 64 * ks + 32 * (l / 32) + j;
                    int c = (row < rows && kk < k) ? codes[row * k + kk] : 0;
                    unsigned v = e3m2_of_code(c);
                    for (int b = 0; b < 6; b++)
                        if ((v >> b) & 1u) img[(6 * j + b) / 8] |= (uint8_t)(1u << ((6 * j + b) % 8));
                }
                for (int b = 0; b < 16; b++) tile[16 * l + b] = img[b];
                for (int b = 0; b < 8; b++) tile[1024 + 8 * l + b] = img[16 + b];
            }
        }
    return 0;
}

/* ------------------------------------------------------------------ */
/* A4W4 packed operand: two 4-bit codes per byte.                       */
/* ------------------------------------------------------------------ */
/*
 * Not a format of the pages: this project's 4-bit storage of the codes of
 * "Q4LinearFunction" forward, 0.5 byte per code.  Same tiling as the FP6
 * operand above (rows padded with zero codes to a multiple of 32, k to a
 * multiple of 128; tile (rb, ks) = rows 32rb .. 32rb+31, k 64ks .. 64ks+63),
 * but a tile is 1024 bytes at (rb * (kp / 64) + ks) * 1024 and slot l
 * (0..63) is the 16 bytes at tile byte 16l: row 32rb + l % 32, k
 * 64ks + 32(l / 32) + j for j = 0..31.  Element j of a slot is in the
 * little-endian 32-bit word j / 8 of the slot, in nibble p (bits 4p .. 4p+3)
 * with p = e / 2 for even e = j % 8 and p = 4 + e / 2 for odd e, stored as
 * code + 8 (in [0, 15]).
 * Parity unpinned beyond its definition: tests decode it and compare codes.
 */
int64_t oracle_a4w4_packed_bytes(int64_t rows, int64_t k)
{
    int64_t rp = (rows + 31) / 32 * 32, kp = (k + 127) / 128 * 128;
    return rp * kp / 2;
}

int oracle_pack_a4w4_int4(const int8_t *codes, int64_t rows, int64_t k, uint8_t *out)
{
    int64_t rp = (rows + 31) / 32 * 32, kp = (k + 127) / 128 * 128;
    int64_t kt = kp / 64;
    for (int64_t rb = 0; rb < rp / 32; rb++)
        for (int64_t ks = 0; ks < kt; ks++) {
            uint8_t *tile = out + (rb * kt + ks) * 1024;
            for (int l = 0; l < 64; l++) {
                uint32_t word[4] = {0, 0, 0, 0};
                int64_t row = 32 * rb + l % 32;
                for (int j = 0; j < 32; j++) {
                    int64_t kk = 64 * ks + 32 * (l / 32) + j;
                    int c = (row < rows && kk < k) ? codes[row * k + kk] : 0;
                    int e = j % 8;
                    int p = (e % 2 == 0) ? e / 2 : 4 + e / 2;
                    word[j / 8] |= (uint32_t)(c + 8) << (4 * p);
                }
                for (int w = 0; w < 4; w++)
                    for (int b = 0; b < 4; b++)
                        tile[16 * l + 4 * w + b] = (uint8_t)(word[w] >> (8 * b));
            }
        }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Output rounding: fp64 -> fp16 / bf16, round to nearest, ties to even. */
/* ------------------------------------------------------------------ */
/*
 * [PT] Parameters / Output: the result is written as float16 or bf16.
 * Direct single rounding from fp64 (no fp32 intermediate).  fp16 overflow
 * gives +-inf as in IEEE.  Returns the 16-bit pattern.
 */
static uint16_t round_to_16(double v, int mant_bits, int exp_bits)
{
    int bias = (1 << (exp_bits - 1)) - 1;
    uint16_t sign = (uint16_t)(signbit(v) ? 1u << 15 : 0u);
    double a = fabs(v);
    uint16_t expmask = (uint16_t)(((1u << exp_bits) - 1u) << mant_bits);
    if (isnan(v)) return (uint16_t)(expmask | (1u << (mant_bits - 1)));
    if (isinf(v)) return (uint16_t)(sign | expmask);
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);                 /* a = f * 2^e, f in [0.5, 1) */
    int ue = e - 1;               /* a in [2^ue, 2^(ue+1)) */
    int emin = 1 - bias;
    if (ue < emin) ue = emin;     /* subnormal range uses the minimum exponent */
    double quantum = ldexp(1.0, ue - mant_bits);
    double units = nearbyint(a / quantum);   /* exact scaling by a power of 2 */
    if (units == 0.0) return sign;           /* rounds to a signed zero */
    /* units may have carried into the next binade; recompose. */
    double r = units * quantum;
    int e2;
    frexp(r, &e2);
    int rexp = e2 - 1;
    uint32_t bits;
    if (r >= ldexp(1.0, bias + 1)) return (uint16_t)(sign | expmask);  /* overflow */
    if (rexp < emin) {
        bits = (uint32_t)units;                  /* subnormal */
    } else {
        uint32_t biased = (uint32_t)(rexp + bias);
        uint32_t mant = (uint32_t)(r / ldexp(1.0, rexp - mant_bits)) - (1u << mant_bits);
        bits = (biased << mant_bits) | mant;
    }
    return (uint16_t)(sign | bits);
}

void oracle_round_f16(const double *v, int64_t count, uint16_t *out)
{
    for (int64_t i = 0; i < count; i++) out[i] = round_to_16(v[i], 10, 5);
}

void oracle_round_bf16(const double *v, int64_t count, uint16_t *out)
{
    for (int64_t i = 0; i < count; i++) out[i] = round_to_16(v[i], 7, 8);
}
