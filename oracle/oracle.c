/*
 * oracle.c -- plain, slow, loop-based CPU reference of one GPU's MoE layer
 * forward (softmax top-k gate -> expert histogram / permutation -> SwiGLU
 * expert FFN -> gate-weighted combine).
 *
 * THIS IS TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load it.  It shares no code, header, table or
 * helper with the HIP library; the two meet only through the seeded input
 * generators.
 *
 * Sources followed:
 *   - FlashMoE Kernel page, opening paragraph: the layer is
 *     gate -> dispatch -> expert FFN -> combine.
 *   - FlashMoE Kernel page, "Architecture" section (unified task abstraction):
 *     the combine is a Hadamard (per-token gate weight) weighted sum of expert
 *     outputs.
 *   - MegaMoE-vs-MoE-systems page, section 2.4 (routing index drives the write
 *     address): every expert-pool slot records its source (token, top-k slot).
 *   - MegaMoE-vs-MoE-systems page, section 2.6 (dropless): no capacity factor,
 *     every routed token is computed.
 *   - The stated workloads: renormalised top-k softmax gate, SwiGLU experts,
 *     bf16 activations/weights with fp32 accumulation, and an FP8 variant with
 *     e4m3 weights scaled per 128x128 block and activations quantised per
 *     1x128 group with scale = amax/448, the SwiGLU output requantised the same
 *     way before the down projection.
 *
 * Readings taken where the pages are silent (each one is a choice; the GPU
 * side must follow the same choice):
 *   - Logits are fp32: acc = +0.0f, then acc = fmaf(x[i], w[i][e], acc) for
 *     i ascending, then one fp32 add of the bias.  Selection is done on these
 *     logits, not on probabilities (softmax is monotone).
 *   - Top-k order: descending logit, equal logits ranked by lower expert index.
 *   - Weights: softmax over the k selected logits (equal to renormalising the
 *     full softmax over the selected experts), computed in fp64, stored fp32.
 *   - Slot order inside an expert is increasing q = t*k + j (stable).
 *   - SwiGLU: h = SiLU(x.W1) * (x.W3), SiLU(a) = a / (1 + exp(-a)); y = h.W2.
 *   - h is an activation: it is rounded to the activation type before W2
 *     (fp32 for fp32 layers, bf16 RNE for bf16 layers, fp32 then FP8 1x128
 *     requantisation for FP8 layers).
 *   - FP8 is OCP E4M3FN (max 448, no infinity), round-to-nearest-even with
 *     saturation; the group scale is the fp32 quotient amax/448 (1 if amax is
 *     0) and the code is e4m3(v / s) with an fp32 quotient.
 *   - All sums of products are exact-order fp64 loops with the contraction
 *     index ascending.
 *   - MXFP4 layers (the FP8 x FP4 expert variant of the MegaMoE-vs-MoE-systems
 *     page, sections 1 and 4): weights are OCP MX FP4, i.e. E2M1 codes
 *     (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6) sharing one E8M0 power-of-two
 *     scale per 32 consecutive elements along the contraction axis; x and h
 *     are OCP MX FP8 (E4M3 codes, one E8M0 scale per 32 consecutive
 *     elements).  A block's scale exponent is floor(log2(amax)) minus the
 *     element format's largest exponent (2 for E2M1, 8 for E4M3), clamped to
 *     [-127, 127], and 0 for an all-zero block; each element is v * 2^-X
 *     (exact) rounded to nearest, ties to even, saturating at the format's
 *     largest magnitude.  h is requantised from fp32(h).
 *   - Shared experts (MegaMoE-vs-MoE-systems page, section 2.7: shared-expert
 *     GEMMs are phases of the same task queue as the routed ones) see every
 *     token and are added with weight 1 after the gate-weighted routed sum:
 *     out = sum_j w_j y_j (j ascending) + sum_s ys_s (s ascending).  Their
 *     weights follow the E routed experts' in the weight lists.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fno-fast-math -shared -fPIC.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_FP8 = 2, ORC_MXFP4 = 3 };
enum { ORC_MX_E4M3 = 0, ORC_MX_E2M1 = 1 }; /* element formats of the MX blocks */

typedef struct {
    int64_t T, d, f;
    int32_t E, k;
    int32_t act_dtype; /* x and gate_w: ORC_F32 or ORC_BF16                 */
    int32_t w_dtype;   /* W1, W3, W2: ORC_F32, ORC_BF16, ORC_FP8, ORC_MXFP4 */
    int32_t n_shared;  /* shared experts, weights at list index E + s       */
} orc_problem;

/* ------------------------------------------------------------------ */
/* number formats                                                      */
/* ------------------------------------------------------------------ */

static float bf16_bits_to_float(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float v;
    memcpy(&v, &u, sizeof v);
    return v;
}

/* Value of element i of an array stored as fp32 or bf16. */
static float load_f(const void *p, int dtype, int64_t i)
{
    if (dtype == ORC_BF16)
        return bf16_bits_to_float(((const uint16_t *)p)[i]);
    return ((const float *)p)[i];
}

/* OCP E4M3FN decode: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits;
 * exponent field 0 is subnormal (m * 2^-9); S.1111.111 is NaN. */
double orc_e4m3_decode(uint8_t q)
{
    int s = q >> 7, e = (q >> 3) & 15, m = q & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    v = (e == 0) ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
    return s ? -v : v;
}

/* OCP E4M3FN encode, round to nearest (ties to even), saturating at 448. */
static uint8_t e4m3_encode_d(double v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs(v), quantum, r;
    int e, ex, m;
    if (isnan(v))
        return 0x7f;
    if (a >= 448.0)
        return sign | 0x7e;
    /* binade of a: a in [2^ex, 2^(ex+1)); below 2^-6 the spacing is 2^-9 */
    frexp(a, &e);
    ex = e - 1;
    if (ex < -6)
        ex = -6;
    quantum = ldexp(1.0, ex - 3);
    r = nearbyint(a / quantum) * quantum; /* exact scaling; RNE */
    if (r == 0.0)
        return sign;
    if (r > 448.0)
        r = 448.0;
    frexp(r, &e);
    ex = e - 1;
    if (ex < -6) /* subnormal code */
        return sign | (uint8_t)(r / ldexp(1.0, -9));
    m = (int)(r / ldexp(1.0, ex - 3)) - 8;
    return sign | (uint8_t)(((ex + 7) << 3) | m);
}

uint8_t orc_e4m3_encode(float v) { return e4m3_encode_d((double)v); }

/* OCP E2M1 (FP4) decode: 1 sign bit (bit 3), 2 exponent bits (bias 1), 1
 * mantissa bit; exponent field 0 is subnormal (m * 0.5).  No inf or NaN. */
double orc_e2m1_decode(uint8_t q)
{
    int s = (q >> 3) & 1, e = (q >> 1) & 3, m = q & 1;
    double v = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -v : v;
}

/* E2M1 encode, round to nearest (ties to even), saturating at 6. */
static uint8_t e2m1_encode_d(double v)
{
    uint8_t sign = signbit(v) ? 0x8 : 0x0;
    double a = fabs(v), r;
    int e, ex;
    if (isnan(v) || a >= 6.0)
        return sign | 0x7;
    /* binade of a: a in [2^ex, 2^(ex+1)); below 1 the spacing is 0.5 */
    frexp(a, &e);
    ex = e - 1;
    if (ex < 0)
        ex = 0;
    r = nearbyint(a / ldexp(1.0, ex - 1)) * ldexp(1.0, ex - 1); /* exact scaling; RNE */
    if (r == 0.0)
        return sign;
    if (r < 1.0) /* 0.5: the subnormal code */
        return sign | 0x1;
    frexp(r, &e);
    ex = e - 1; /* 0, 1 or 2 */
    return sign | (uint8_t)(((ex + 1) << 1) | (r > ldexp(1.0, ex) ? 1 : 0));
}

uint8_t orc_e2m1_encode(float v) { return e2m1_encode_d((double)v); }

/* Shared exponent X of one MX block (scale 2^X, stored as the E8M0 byte
 * X + 127): floor(log2(amax)) - emax, emax = 2 for E2M1 and 8 for E4M3,
 * clamped to [-127, 127]; 0 for an all-zero block. */
int orc_mx_exponent(float amax, int elem)
{
    int e, x;
    if (amax == 0.0f)
        return 0;
    frexp((double)amax, &e); /* amax in [2^(e-1), 2^e) */
    x = (e - 1) - (elem == ORC_MX_E2M1 ? 2 : 8);
    return x < -127 ? -127 : (x > 127 ? 127 : x);
}

/* MX quantisation of a [rows x cols] fp32 matrix along its rows (cols a
 * multiple of 32): codes [rows x cols], one per byte; scales
 * [rows x cols/32] E8M0 bytes. */
void orc_mx_quant_rows(int64_t rows, int64_t cols, int elem, const float *v,
                       uint8_t *q, uint8_t *s)
{
    int64_t nb = cols / 32;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            const float *vb = v + r * cols + b * 32;
            float amax = 0.0f;
            int i, x;
            for (i = 0; i < 32; ++i)
                if (fabsf(vb[i]) > amax)
                    amax = fabsf(vb[i]);
            x = orc_mx_exponent(amax, elem);
            s[r * nb + b] = (uint8_t)(x + 127);
            for (i = 0; i < 32; ++i) {
                double u = ldexp((double)vb[i], -x);
                q[r * cols + b * 32 + i] =
                    elem == ORC_MX_E2M1 ? e2m1_encode_d(u) : e4m3_encode_d(u);
            }
        }
}

/* Decoded value of one MX element: code value times 2^(scale byte - 127). */
double orc_mx_value(int elem, uint8_t code, uint8_t scale)
{
    double c = elem == ORC_MX_E2M1 ? orc_e2m1_decode(code) : orc_e4m3_decode(code);
    return ldexp(c, (int)scale - 127);
}

/* Round an fp64 value to the nearest bfloat16 value (ties to even), returned
 * as fp64.  bfloat16 has 8 significant bits and fp32's exponent range. */
double orc_round_bf16(double h)
{
    double a, quantum, r;
    int e, ex;
    if (h == 0.0 || !isfinite(h))
        return h;
    a = fabs(h);
    frexp(a, &e);
    ex = e - 1;
    if (ex < -126)
        ex = -126;
    quantum = ldexp(1.0, ex - 7);
    r = nearbyint(a / quantum) * quantum;
    if (r > ldexp(255.0, 120)) /* beyond the largest finite bf16 */
        r = INFINITY;
    return copysign(r, h);
}

/* Quantise one group of n values (n <= 128) to e4m3 with one fp32 scale:
 * amax over the group, s = amax / 448 as an fp32 quotient (1 if amax == 0),
 * code = e4m3(v / s) with an fp32 quotient. */
static void quant_group(const float *v, int n, uint8_t *q, float *s_out)
{
    float amax = 0.0f, s;
    int i;
    for (i = 0; i < n; ++i) {
        float a = fabsf(v[i]);
        if (a > amax)
            amax = a;
    }
    s = (amax == 0.0f) ? 1.0f : amax / 448.0f;
    for (i = 0; i < n; ++i)
        q[i] = orc_e4m3_encode(v[i] / s);
    *s_out = s;
}

/* Row-wise 1x128 group quantisation of a [rows x cols] fp32 matrix. */
void orc_fp8_quant_rows(int64_t rows, int64_t cols, const float *v,
                        uint8_t *q, float *s)
{
    int64_t ng = (cols + 127) / 128;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t g = 0; g < ng; ++g) {
            int64_t c0 = g * 128;
            int n = (int)((cols - c0) < 128 ? (cols - c0) : 128);
            quant_group(v + r * cols + c0, n, q + r * cols + c0, s + r * ng + g);
        }
}

/* Array helpers so tests can pin the number formats directly. */
void orc_e4m3_encode_array(int64_t n, const float *v, uint8_t *q)
{
    for (int64_t i = 0; i < n; ++i)
        q[i] = orc_e4m3_encode(v[i]);
}

void orc_e4m3_decode_array(int64_t n, const uint8_t *q, double *v)
{
    for (int64_t i = 0; i < n; ++i)
        v[i] = orc_e4m3_decode(q[i]);
}

void orc_e2m1_encode_array(int64_t n, const float *v, uint8_t *q)
{
    for (int64_t i = 0; i < n; ++i)
        q[i] = orc_e2m1_encode(v[i]);
}

void orc_e2m1_decode_array(int64_t n, const uint8_t *q, double *v)
{
    for (int64_t i = 0; i < n; ++i)
        v[i] = orc_e2m1_decode(q[i]);
}

void orc_round_bf16_array(int64_t n, const double *in, double *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_round_bf16(in[i]);
}

/* ------------------------------------------------------------------ */
/* gate: logits, top-k, renormalised softmax weights                    */
/* ------------------------------------------------------------------ */

/* Logit of token t for expert e: fp32 fused multiply-add chain over the
 * hidden index ascending from +0, then the bias as one fp32 add. */
static float logit(const orc_problem *p, const void *x, const void *gate_w,
                   const float *bias, int64_t t, int e)
{
    float acc = 0.0f;
    for (int64_t i = 0; i < p->d; ++i)
        acc = fmaf(load_f(x, p->act_dtype, t * p->d + i),
                   load_f(gate_w, p->act_dtype, i * p->E + e), acc);
    if (bias)
        acc = acc + bias[e];
    return acc;
}

/* a ranks before b: larger logit first, equal logits by lower index. */
static int ranks_before(const float *l, int a, int b)
{
    return l[a] > l[b] || (l[a] == l[b] && a < b);
}

/* Route one token given its E logits: ids in rank order and weights. */
static void route_one(int E, int k, const float *l, int32_t *ids, float *w)
{
    char *taken = (char *)calloc((size_t)E, 1);
    double u[512], sum = 0.0, m;
    int j, e;
    for (j = 0; j < k; ++j) {
        int best = -1;
        for (e = 0; e < E; ++e)
            if (!taken[e] && (best < 0 || ranks_before(l, e, best)))
                best = e;
        taken[best] = 1;
        ids[j] = best;
    }
    free(taken);
    m = (double)l[ids[0]];
    for (j = 0; j < k; ++j) {
        u[j] = exp((double)l[ids[j]] - m);
        sum += u[j];
    }
    for (j = 0; j < k; ++j)
        w[j] = (float)(u[j] / sum);
}

/* Gate for every token: logits [T x E] (nullable), ids and weights [T x k]. */
int orc_route(const orc_problem *p, const void *x, const void *gate_w,
              const float *bias, float *logits, int32_t *ids, float *w)
{
    if (p->k < 1 || p->k > p->E || p->k > 512)
        return 1;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t t = 0; t < p->T; ++t) {
        float *l = (float *)malloc(sizeof(float) * (size_t)p->E);
        for (int e = 0; e < p->E; ++e)
            l[e] = logit(p, x, gate_w, bias, t, e);
        if (logits)
            memcpy(logits + t * p->E, l, sizeof(float) * (size_t)p->E);
        route_one(p->E, p->k, l, ids + t * p->k, w + t * p->k);
        free(l);
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* dispatch: histogram, exclusive scan, stable counting-sort scatter    */
/* ------------------------------------------------------------------ */

int orc_permute(int64_t T, int k, int E, const int32_t *ids, int32_t *counts,
                int32_t *offsets, int32_t *slot_token, int32_t *slot_k,
                int32_t *token_slot)
{
    int64_t n = T * k, q;
    int32_t *fill;
    int e;
    for (q = 0; q < n; ++q)
        if (ids[q] < 0 || ids[q] >= E)
            return 1;
    for (e = 0; e < E; ++e)
        counts[e] = 0;
    for (q = 0; q < n; ++q)
        counts[ids[q]]++;
    offsets[0] = 0;
    for (e = 0; e < E; ++e)
        offsets[e + 1] = offsets[e] + counts[e];
    fill = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
    memcpy(fill, offsets, sizeof(int32_t) * (size_t)E);
    for (q = 0; q < n; ++q) {
        int32_t s = fill[ids[q]]++;
        slot_token[s] = (int32_t)(q / k);
        slot_k[s] = (int32_t)(q % k);
        token_slot[q] = s;
    }
    free(fill);
    return 0;
}

/* ------------------------------------------------------------------ */
/* expert FFN and combine                                               */
/* ------------------------------------------------------------------ */

/* Decoded value of every E4M3FN code, filled from orc_e4m3_decode once
 * (a lookup only to make the loops below faster). */
static double e4m3_value[256];
static int e4m3_value_ready = 0;

static void init_e4m3_values(void)
{
    if (!e4m3_value_ready) {
        for (int c = 0; c < 256; ++c)
            e4m3_value[c] = orc_e4m3_decode((uint8_t)c);
        e4m3_value_ready = 1;
    }
}

/* Value of weight element (r, c) of one expert's [R x C] matrix.  FP8:
 * Ws = fp32 [R/128 x C/128] block scales; MXFP4: W holds one E2M1 code per
 * byte and Ws = E8M0 bytes [R/32 x C] (blocks of 32 along the contraction
 * axis r). */
static double load_w(const orc_problem *p, const void *W, const void *Ws,
                     int64_t C, int64_t r, int64_t c)
{
    if (p->w_dtype == ORC_FP8) {
        int64_t ncb = (C + 127) / 128;
        return e4m3_value[((const uint8_t *)W)[r * C + c]] *
               (double)((const float *)Ws)[(r / 128) * ncb + c / 128];
    }
    if (p->w_dtype == ORC_MXFP4)
        return orc_mx_value(ORC_MX_E2M1, ((const uint8_t *)W)[r * C + c],
                            ((const uint8_t *)Ws)[(r / 32) * C + c]);
    return (double)load_f(W, p->w_dtype, r * C + c);
}

/* MX FP8 round trip of n fp32 values (n a multiple of 32), into fp64. */
static void mx_fp8_roundtrip(int64_t n, const float *v, double *out)
{
    uint8_t *q = (uint8_t *)malloc((size_t)n);
    uint8_t *s = (uint8_t *)malloc((size_t)(n / 32));
    orc_mx_quant_rows(1, n, ORC_MX_E4M3, v, q, s);
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_mx_value(ORC_MX_E4M3, q[i], s[i / 32]);
    free(q);
    free(s);
}

/* Activation row of token t as the experts consume it (fp64).  For FP8 layers
 * the bf16 row is quantised per 1x128 group and dequantised. */
static void expert_input_row(const orc_problem *p, const void *x, int64_t t,
                             double *row)
{
    int64_t i;
    if (p->w_dtype == ORC_FP8) {
        float *v = (float *)malloc(sizeof(float) * (size_t)p->d);
        uint8_t *q = (uint8_t *)malloc((size_t)p->d);
        float *s = (float *)malloc(sizeof(float) * (size_t)((p->d + 127) / 128));
        for (i = 0; i < p->d; ++i)
            v[i] = load_f(x, p->act_dtype, t * p->d + i);
        orc_fp8_quant_rows(1, p->d, v, q, s);
        for (i = 0; i < p->d; ++i)
            row[i] = orc_e4m3_decode(q[i]) * (double)s[i / 128];
        free(v);
        free(q);
        free(s);
    } else if (p->w_dtype == ORC_MXFP4) {
        float *v = (float *)malloc(sizeof(float) * (size_t)p->d);
        for (i = 0; i < p->d; ++i)
            v[i] = load_f(x, p->act_dtype, t * p->d + i);
        mx_fp8_roundtrip(p->d, v, row);
        free(v);
    } else {
        for (i = 0; i < p->d; ++i)
            row[i] = (double)load_f(x, p->act_dtype, t * p->d + i);
    }
}

/* Round the SwiGLU output of one slot to the activation format seen by W2. */
static void mirror_h(const orc_problem *p, double *h)
{
    int64_t n;
    if (p->w_dtype == ORC_FP8) {
        int64_t ng = (p->f + 127) / 128;
        float *v = (float *)malloc(sizeof(float) * (size_t)p->f);
        uint8_t *q = (uint8_t *)malloc((size_t)p->f);
        float *s = (float *)malloc(sizeof(float) * (size_t)ng);
        for (n = 0; n < p->f; ++n)
            v[n] = (float)h[n];
        orc_fp8_quant_rows(1, p->f, v, q, s);
        for (n = 0; n < p->f; ++n)
            h[n] = orc_e4m3_decode(q[n]) * (double)s[n / 128];
        free(v);
        free(q);
        free(s);
    } else if (p->w_dtype == ORC_MXFP4) {
        float *v = (float *)malloc(sizeof(float) * (size_t)p->f);
        for (n = 0; n < p->f; ++n)
            v[n] = (float)h[n];
        mx_fp8_roundtrip(p->f, v, h);
        free(v);
    } else if (p->act_dtype == ORC_BF16) {
        for (n = 0; n < p->f; ++n)
            h[n] = orc_round_bf16(h[n]);
    } else {
        for (n = 0; n < p->f; ++n)
            h[n] = (double)(float)h[n];
    }
}

#define ORC_BLOCK 8 /* slots of one expert evaluated together */
#define SCALED(p) ((p)->w_dtype == ORC_FP8 || (p)->w_dtype == ORC_MXFP4)

/* SwiGLU hidden rows h = SiLU(rows W1) * (rows W3) in fp64, before any
 * rounding to the format W2 reads (FlashMoE Kernel page, the FFN stage).
 * rows: [nr x d]; h: [nr x f].  Each product is an fp64 sum over the
 * contraction index ascending. */
static void swiglu_rows(const orc_problem *p, int nr, const double *rows,
                        const void *W1, const void *W3, const void *W1s,
                        const void *W3s, double *h)
{
    int64_t d = p->d, f = p->f, i, n;
    int r;
    double *b = (double *)calloc((size_t)(nr * f), sizeof(double));
    memset(h, 0, sizeof(double) * (size_t)(nr * f));
    for (i = 0; i < d; ++i)
        for (n = 0; n < f; ++n) {
            double w1 = load_w(p, W1, W1s, f, i, n);
            double w3 = load_w(p, W3, W3s, f, i, n);
            for (r = 0; r < nr; ++r) {
                h[r * f + n] += rows[r * d + i] * w1;
                b[r * f + n] += rows[r * d + i] * w3;
            }
        }
    for (r = 0; r < nr; ++r)
        for (n = 0; n < f; ++n) /* SiLU(a) * b */
            h[r * f + n] = h[r * f + n] / (1.0 + exp(-h[r * f + n])) * b[r * f + n];
    free(b);
}

/* Expert FFN for up to ORC_BLOCK activation rows of one expert.
 * rows: [nr x d]; y: [nr x d].  Each output element is an fp64 sum over the
 * contraction index ascending. */
static void expert_ffn(const orc_problem *p, int nr, const double *rows,
                       const void *W1, const void *W3, const void *W2,
                       const void *W1s, const void *W3s, const void *W2s,
                       double *y)
{
    int64_t d = p->d, f = p->f, n, m;
    int r;
    double *a = (double *)malloc(sizeof(double) * (size_t)(nr * f));
    swiglu_rows(p, nr, rows, W1, W3, W1s, W3s, a);
    for (r = 0; r < nr; ++r)
        mirror_h(p, a + r * f);
    memset(y, 0, sizeof(double) * (size_t)(nr * d));
    for (n = 0; n < f; ++n)
        for (m = 0; m < d; ++m) {
            double w2 = load_w(p, W2, W2s, d, n, m);
            for (r = 0; r < nr; ++r)
                y[r * d + m] += a[r * f + n] * w2;
        }
    free(a);
}

/* The exact SwiGLU output (fp64, before rounding to W2's input format) of
 * token t through one expert's W1, W3 (and their scales for FP8 and MXFP4
 * weights, else NULL): h [f].  The activation row is the one the experts
 * consume (quantised and dequantised on FP8 and MXFP4 layers).  Returns 0,
 * or 1 for a token out of range. */
int orc_expert_hidden(const orc_problem *p, const void *x, int64_t t,
                      const void *W1, const void *W3, const void *W1s,
                      const void *W3s, double *h)
{
    if (t < 0 || t >= p->T)
        return 1;
    init_e4m3_values();
    double *row = (double *)malloc(sizeof(double) * (size_t)p->d);
    expert_input_row(p, x, t, row);
    swiglu_rows(p, 1, row, W1, W3, W1s, W3s, h);
    free(row);
    return 0;
}

/* Layer forward for a list of tokens.
 *
 * W1[e], W3[e]: [d x f]; W2[e]: [f x d], one pointer per expert (an expert no
 * listed token routes to may be NULL); entries E .. E + n_shared - 1 are the
 * shared experts (never NULL when n_shared > 0).  For FP8 weights
 * W1s/W3s/W2s[e] point to the [K/128 x N/128] fp32 block scales of that
 * expert's [K x N] matrix; for MXFP4 weights W holds one E2M1 code per byte
 * and W1s/W3s/W2s[e] the [K/32 x N] E8M0 scale bytes; otherwise they are
 * NULL.  x is the full [T x d] activation matrix, gate_w is
 * [d x E], bias is [E] or NULL.
 *
 * out:   [ntok x d] fp64, the unrounded combine of each listed token.
 * ids, w (nullable): [ntok x k] routing of each listed token.
 * Returns 0, or nonzero for an invalid argument or a missing expert.
 */
int orc_forward(const orc_problem *p, const void *x, const void *gate_w,
                const float *bias, const void *const *W1,
                const void *const *W3, const void *const *W2,
                const void *const *W1s, const void *const *W3s,
                const void *const *W2s, const int64_t *tokens, int64_t ntok,
                double *out, int32_t *ids_out, float *w_out)
{
    int64_t d = p->d, k = p->k, npair = ntok * k, it;
    int32_t *ids = (int32_t *)malloc(sizeof(int32_t) * (size_t)npair);
    float *w = (float *)malloc(sizeof(float) * (size_t)npair);
    double *y = (double *)malloc(sizeof(double) * (size_t)(npair * d));
    int64_t *order = (int64_t *)malloc(sizeof(int64_t) * (size_t)npair);
    int64_t *start = (int64_t *)calloc((size_t)p->E + 1, sizeof(int64_t));
    int64_t nitems = 0, *item_e, *item_beg, *item_len;
    int bad = 0;
    init_e4m3_values();
    if (k < 1 || k > p->E || k > 512 || p->n_shared < 0)
        bad = 1;
    for (int s = 0; s < p->n_shared && !bad; ++s) {
        int e = p->E + s;
        if (!W1[e] || !W3[e] || !W2[e] ||
            (SCALED(p) && (!W1s[e] || !W3s[e] || !W2s[e])))
            bad = 1;
    }

    /* gate, token by token */
    for (it = 0; it < ntok && !bad; ++it) {
        float *l = (float *)malloc(sizeof(float) * (size_t)p->E);
        if (tokens[it] < 0 || tokens[it] >= p->T)
            bad = 1;
        else {
            for (int e = 0; e < p->E; ++e)
                l[e] = logit(p, x, gate_w, bias, tokens[it], e);
            route_one(p->E, (int)k, l, ids + it * k, w + it * k);
        }
        free(l);
    }
    /* group (token, j) pairs by expert, pair order increasing */
    if (!bad) {
        int64_t *fill = (int64_t *)malloc(sizeof(int64_t) * (size_t)p->E);
        for (it = 0; it < npair; ++it)
            start[ids[it] + 1]++;
        for (int e = 0; e < p->E; ++e)
            start[e + 1] += start[e];
        memcpy(fill, start, sizeof(int64_t) * (size_t)p->E);
        for (it = 0; it < npair; ++it)
            order[fill[ids[it]]++] = it;
        free(fill);
        for (int e = 0; e < p->E; ++e)
            if (start[e + 1] > start[e] && (!W1[e] || !W3[e] || !W2[e] ||
                (SCALED(p) && (!W1s[e] || !W3s[e] || !W2s[e]))))
                bad = 1;
    }
    if (bad) {
        free(ids); free(w); free(y); free(order); free(start);
        return 1;
    }
    /* work items: blocks of up to ORC_BLOCK pairs of one expert */
    item_e = (int64_t *)malloc(sizeof(int64_t) * (size_t)(npair + p->E));
    item_beg = (int64_t *)malloc(sizeof(int64_t) * (size_t)(npair + p->E));
    item_len = (int64_t *)malloc(sizeof(int64_t) * (size_t)(npair + p->E));
    for (int e = 0; e < p->E; ++e)
        for (it = start[e]; it < start[e + 1]; it += ORC_BLOCK) {
            item_e[nitems] = e;
            item_beg[nitems] = it;
            item_len[nitems] = (start[e + 1] - it) < ORC_BLOCK ? (start[e + 1] - it) : ORC_BLOCK;
            nitems++;
        }

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t wi = 0; wi < nitems; ++wi) {
        int e = (int)item_e[wi], nr = (int)item_len[wi], r;
        double *rows = (double *)malloc(sizeof(double) * (size_t)(nr * d));
        double *yb = (double *)malloc(sizeof(double) * (size_t)(nr * d));
        for (r = 0; r < nr; ++r)
            expert_input_row(p, x, tokens[order[item_beg[wi] + r] / k], rows + r * d);
        expert_ffn(p, nr, rows, W1[e], W3[e], W2[e],
                   SCALED(p) ? W1s[e] : NULL, SCALED(p) ? W3s[e] : NULL,
                   SCALED(p) ? W2s[e] : NULL, yb);
        for (r = 0; r < nr; ++r)
            memcpy(y + order[item_beg[wi] + r] * d, yb + r * d, sizeof(double) * (size_t)d);
        free(rows);
        free(yb);
    }

    /* shared experts: every listed token, blocks of ORC_BLOCK tokens */
    double *ys = NULL;
    if (p->n_shared > 0) {
        int64_t nsb = (ntok + ORC_BLOCK - 1) / ORC_BLOCK;
        ys = (double *)malloc(sizeof(double) * (size_t)(p->n_shared * ntok * d));
#pragma omp parallel for schedule(dynamic, 1)
        for (int64_t wi = 0; wi < p->n_shared * nsb; ++wi) {
            int e = p->E + (int)(wi / nsb);
            int64_t t0 = (wi % nsb) * ORC_BLOCK;
            int nr = (int)((ntok - t0) < ORC_BLOCK ? (ntok - t0) : ORC_BLOCK), r;
            double *rows = (double *)malloc(sizeof(double) * (size_t)(nr * d));
            for (r = 0; r < nr; ++r)
                expert_input_row(p, x, tokens[t0 + r], rows + r * d);
            expert_ffn(p, nr, rows, W1[e], W3[e], W2[e],
                       SCALED(p) ? W1s[e] : NULL, SCALED(p) ? W3s[e] : NULL,
                       SCALED(p) ? W2s[e] : NULL,
                       ys + ((int64_t)(e - p->E) * ntok + t0) * d);
            free(rows);
        }
    }

    /* combine: gate-weighted sum over the k slots of each token, j ascending,
     * then the shared experts, s ascending */
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < ntok; ++t)
        for (int64_t m = 0; m < d; ++m) {
            double acc = 0.0;
            for (int64_t j = 0; j < k; ++j)
                acc += (double)w[t * k + j] * y[(t * k + j) * d + m];
            for (int s = 0; s < p->n_shared; ++s)
                acc += ys[((int64_t)s * ntok + t) * d + m];
            out[t * d + m] = acc;
        }
    free(ys);
    if (ids_out)
        memcpy(ids_out, ids, sizeof(int32_t) * (size_t)npair);
    if (w_out)
        memcpy(w_out, w, sizeof(float) * (size_t)npair);
    free(ids); free(w); free(y); free(order); free(start);
    free(item_e); free(item_beg); free(item_len);
    return 0;
}
