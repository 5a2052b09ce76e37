/*
 * CPU oracle for FlashOptim's compressed optimizer step.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this file's library.  It shares no
 * source with the HIP library (include/flashopt.h, compressed_adamw_state_amd/
 * csrc), and neither side includes or links the other.
 *
 * What it computes follows the FlashOptim digest ("FlashOptim: Optimizers for
 * Memory Efficient Training", arXiv 2602.23349v1):
 *   - weight splitting, section "Core method > Weight splitting: ULP-based
 *     error correction" (Eq. 1-2, Alg. 1): theta' = BF16(theta), and the error
 *     theta - theta', normalised by ULP(theta')/2, uniformly quantised to an
 *     INT8 code rho;
 *   - companding quantisation, section "Core method > Optimizer-state
 *     quantisation with companding" (Alg. 2-3): phi_m(x) = 2x/(1+|x|),
 *     phi_m^-1(z) = z/(2-|z|), phi_v(x) = sqrt(x), phi_v^-1(z) = z^2, groups of
 *     G = 32 with one FP16 scale each, momentum INT8, variance UINT8;
 *   - the fused step, section "Core method > Fused optimizer step" (Alg. 4):
 *     dequantise, rebuild the master weight, standard AdamW (or SGD with
 *     momentum, named in the background section), requantise, re-split;
 *   - compression switched off for a layer, section "Practical advice": the
 *     same updates over an FP32 master weight and FP32 moments, with the BF16
 *     weight the model computes with rounded from the new master weight.
 *
 * The page prints the companding formulas but not the algorithms, so the
 * arithmetic order below is the plainest reading, one IEEE binary32 operation
 * per line (round to nearest even, no fused multiply-add, subnormals kept):
 *   K8   = RN(1/127), K255 = RN(1/255)
 *   h    = ULP(theta')/2 = 2^(max(E,1) - 135), E = biased exponent of theta'
 *   unsplit: theta_hat = theta' + (rho * K8) * h            (Inf/NaN: theta')
 *   split:   theta' = bf16_rne(theta), e = (theta - theta')/h (exact),
 *            rho = clamp(rne(e * 127), -127, 127)           (non-finite: 0)
 *   dequant m: d = s*K8, z = q*d, m = z/(2-|z|)
 *   dequant v: d = s*K255, z = q*d, v = z*z
 *   AdamW:   m' = b1*m + c1*g; v' = b2*v + c2*(g*g); w = sqrt(v');
 *            u = m'/(w*kappa + eps); theta_n = lambda*theta_hat - alpha*u
 *   SGD:     g' = g + omega*theta_hat; b' = mu*b + g'; theta_n = theta_hat - eta*b'
 *   requant: z = (2*m')/(1+|m'|) (or w for v); a = max|z| over the group's
 *            valid elements; s16 = f16_rne(a) (clamped to 0x3FFF for m,
 *            0x7BFF for v); q = 0 if s16 = 0, else clamp(rne(z * (127/s)))
 *            (255/s and [0,255] for v).
 * Host scalars (per call, in double, rounded to binary32 once):
 *   p1 = beta1^t, p2 = beta2^t by repeated multiplication; alpha = lr/(1-p1);
 *   kappa = 1/sqrt(1-p2); lambda = 1 - lr*wd; b1, c1 = 1-beta1, b2, c2 = 1-beta2.
 *
 * Build: gcc -std=c11 -O2 -ffp-contract=off -fno-fast-math (no FTZ/DAZ).
 */
#include <fenv.h>
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "flashopt_oracle.h"

_Static_assert(FLT_EVAL_METHOD == 0, "binary32 operations must round to binary32");
_Static_assert(sizeof(float) == 4 && sizeof(double) == 8, "IEEE binary32/binary64 expected");

#define GROUP 32

static uint32_t bits_of(float x) { uint32_t u; memcpy(&u, &x, 4); return u; }
static float float_of(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }

/* RN(1/127), RN(1/255): the compiler rounds these constant quotients once. */
static const float K8 = 1.0f / 127.0f;
static const float K255 = 1.0f / 255.0f;

int orc_env_ok(void)
{
    volatile float tiny = 1.0e-38f;
    volatile float r = tiny * 1.0e-3f;   /* 1e-41: representable only as a subnormal */
    if (r == 0.0f) return 0;             /* flush-to-zero active */
    volatile float sub = float_of(1u);   /* 2^-149 */
    if (sub * 2.0f == 0.0f) return 0;    /* denormals-are-zero active */
    if (fegetround() != FE_TONEAREST) return 0;
    return 1;
}

/* ------------------------------------------------------------------------ */
/* Conversions, written from the IEEE-754 definition of the formats.          */

/* Round half to even of a non-negative double that holds an exact value. */
static double round_half_even(double n)
{
    double fl = floor(n);
    double frac = n - fl;                 /* exact: n < 2^53 and fl = floor(n) */
    if (frac > 0.5) return fl + 1.0;
    if (frac < 0.5) return fl;
    return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
}

/* Nearest value of a binary format with `mant` stored mantissa bits, exponent
 * bias `bias`, ties to even; returns the bit pattern without sign.  The
 * magnitude `a` is finite and non-negative.  Overflow gives the Inf pattern
 * because the carry out of the largest finite value lands on it. */
static uint32_t encode_rne(double a, int mant, int bias)
{
    if (a == 0.0) return 0;
    int e;
    (void)frexp(a, &e);                   /* a = f * 2^e, f in [0.5, 1) */
    int unbiased = e - 1;                 /* a in [2^unbiased, 2^(unbiased+1)) */
    int emin = 1 - bias;
    if (unbiased < emin) unbiased = emin; /* subnormal range: fixed quantum */
    double quantum = ldexp(1.0, unbiased - mant);
    double k = round_half_even(a / quantum);   /* a / quantum is exact */
    if (unbiased == emin && k < ldexp(1.0, mant))
        return (uint32_t)k;                    /* subnormal (or zero) */
    /* normal: k in [2^mant, 2^(mant+1)]; k == 2^(mant+1) carries into the exponent */
    return ((uint32_t)(unbiased + bias) << mant) + (uint32_t)(k - ldexp(1.0, mant));
}

uint16_t orc_bf16_rne(float x)
{
    uint32_t b = bits_of(x);
    uint32_t sign = (b >> 16) & 0x8000u;
    if (isnan(x)) return (uint16_t)((b >> 16) | 0x0040u);   /* keep payload, make quiet */
    if (isinf(x)) return (uint16_t)(sign | 0x7F80u);
    return (uint16_t)(sign | encode_rne(fabs((double)x), 7, 127));
}

float orc_bf16_to_f32(uint16_t b)
{
    return float_of((uint32_t)b << 16);   /* bf16 is the upper half of binary32 */
}

uint16_t orc_f16_rne(float x)
{
    uint32_t b = bits_of(x);
    uint32_t sign = (b >> 16) & 0x8000u;
    if (isnan(x)) return (uint16_t)(sign | 0x7E00u);
    if (isinf(x)) return (uint16_t)(sign | 0x7C00u);
    uint32_t mag = encode_rne(fabs((double)x), 10, 15);
    if (mag > 0x7C00u) mag = 0x7C00u;     /* beyond the largest binade: Inf */
    return (uint16_t)(sign | mag);
}

float orc_f16_to_f32(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int m = h & 0x3FF;
    double v;
    if (e == 0x1F) {
        if (m) return NAN;
        v = INFINITY;
    } else if (e == 0) {
        v = ldexp((double)m, -24);
    } else {
        v = ldexp((double)(1024 + m), e - 25);
    }
    return (float)(sign ? -v : v);        /* exact: every fp16 value is a binary32 value */
}

/* ------------------------------------------------------------------------ */
/* Weight splitting.                                                         */

/* ULP(theta')/2 with ULP the spacing above |theta'| in its binade; zero and
 * subnormal bf16 use the minimum-normal spacing. */
static float half_ulp(uint16_t tb)
{
    int E = (tb >> 7) & 0xFF;
    if (E < 1) E = 1;
    return ldexpf(1.0f, E - 135);         /* 2^(E-127) * 2^-7 / 2, exact */
}

/* Nearest integer, ties to even.  NaN gives 0: non-finite gradients are
 * outside the method's contract, and 0 keeps the code well defined. */
static float rne_to_int(float y)
{
    if (isnan(y)) return 0.0f;
    if (isinf(y)) return y;
    return (float)round_half_even(fabs((double)y)) * (y < 0.0f ? -1.0f : 1.0f);
}

static float clampf(float x, float lo, float hi)
{
    if (x < lo) return lo;
    if (x > hi) return hi;
    return x;
}

/* rne(qmax * e) of an exact |e| <= 1 with the product itself exact (in double:
 * 24 + 16 bits), for any code width up to 16 bits.  With qmax = 127 and a BF16
 * base the binary32 product is already exact, so this equals split1's code. */
static int32_t code_of(float e, int32_t qmax)
{
    double y = (double)e * (double)qmax;
    double r = round_half_even(fabs(y)) * (y < 0 ? -1.0 : 1.0);
    if (r > qmax) r = qmax;
    if (r < -qmax) r = -qmax;
    return (int32_t)r;
}

void orc_split_q(const float* theta, int64_t n, int32_t qmax, uint16_t* tb, int32_t* rho)
{
    for (int64_t i = 0; i < n; ++i) {
        float x = theta[i];
        uint16_t b = orc_bf16_rne(x);
        float t = orc_bf16_to_f32(b);
        tb[i] = b;
        if (!isfinite(t)) { rho[i] = 0; continue; }
        float h = half_ulp(b);
        float diff = x - t;               /* exact (Sterbenz; or t == 0) */
        float e = diff / h;               /* exact: h is a power of two, |e| <= 1 */
        rho[i] = code_of(e, qmax);
    }
}

void orc_unsplit_q(const uint16_t* tb, const int32_t* rho, int64_t n, int32_t qmax, float* out)
{
    float k = 1.0f / (float)qmax;         /* RN(1/qmax) */
    for (int64_t i = 0; i < n; ++i) {
        float t = orc_bf16_to_f32(tb[i]);
        if (!isfinite(t)) { out[i] = t; continue; }
        float h = half_ulp(tb[i]);
        float c = (float)rho[i] * k;
        float d = c * h;
        out[i] = t + d;
    }
}

/* FP16 base (10 stored mantissa bits, bias 15): ULP(theta')/2 with the same
 * convention -- the spacing above |theta'|, zero and subnormal FP16 using the
 * minimum-normal spacing 2^-24. */
static float half_ulp_f16(uint16_t hb)
{
    int E = (hb >> 10) & 0x1F;
    if (E < 1) E = 1;
    return ldexpf(1.0f, E - 26);          /* 2^(E-15) * 2^-10 / 2, exact */
}

void orc_split_f16_q(const float* theta, int64_t n, int32_t qmax, uint16_t* hb, int32_t* rho)
{
    for (int64_t i = 0; i < n; ++i) {
        float x = theta[i];
        uint16_t b = orc_f16_rne(x);
        float t = orc_f16_to_f32(b);
        hb[i] = b;
        if (!isfinite(t)) { rho[i] = 0; continue; }
        float h = half_ulp_f16(b);
        float diff = x - t;               /* exact (Sterbenz; or t == 0) */
        float e = diff / h;               /* exact: h is a power of two, |e| <= 1 */
        rho[i] = code_of(e, qmax);
    }
}

void orc_unsplit_f16_q(const uint16_t* hb, const int32_t* rho, int64_t n, int32_t qmax,
                       float* out)
{
    float k = 1.0f / (float)qmax;         /* RN(1/qmax) */
    for (int64_t i = 0; i < n; ++i) {
        float t = orc_f16_to_f32(hb[i]);
        if (!isfinite(t)) { out[i] = t; continue; }
        float h = half_ulp_f16(hb[i]);
        float c = (float)rho[i] * k;
        float d = c * h;
        out[i] = t + d;
    }
}

static float unsplit1(uint16_t b, int8_t r)
{
    float t = orc_bf16_to_f32(b);
    if (!isfinite(t)) return t;
    float h = half_ulp(b);
    float c = (float)r * K8;
    float d = c * h;
    return t + d;
}

static void split1(float x, uint16_t* tb, int8_t* rho)
{
    uint16_t b = orc_bf16_rne(x);
    float t = orc_bf16_to_f32(b);
    *tb = b;
    if (!isfinite(t)) { *rho = 0; return; }
    float h = half_ulp(b);
    float diff = x - t;
    float e = diff / h;
    float y = e * 127.0f;
    float r = clampf(rne_to_int(y), -127.0f, 127.0f);
    *rho = (int8_t)r;
}

void orc_split(const float* theta, int64_t n, uint16_t* tb, int8_t* rho)
{
    for (int64_t i = 0; i < n; ++i) split1(theta[i], &tb[i], &rho[i]);
}

void orc_unsplit(const uint16_t* tb, const int8_t* rho, int64_t n, float* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = unsplit1(tb[i], rho[i]);
}

/* ------------------------------------------------------------------------ */
/* Companding.                                                               */

float orc_phi_m(float x)
{
    float num = 2.0f * x;
    float den = 1.0f + fabsf(x);
    return num / den;
}

float orc_phi_m_inv(float z)
{
    float den = 2.0f - fabsf(z);
    return z / den;
}

float orc_phi_v(float x) { return sqrtf(x); }

float orc_phi_v_inv(float z) { return z * z; }

/* ------------------------------------------------------------------------ */
/* Group quantiser.  z[] are companded values of one group (n <= 32).        */

static uint16_t group_scale(const float* z, int n, uint16_t smax)
{
    uint32_t amax = 0;
    for (int j = 0; j < n; ++j) {
        uint32_t a = bits_of(z[j]) & 0x7FFFFFFFu;   /* |z| as an ordered integer */
        if (a > amax) amax = a;
    }
    uint16_t s16 = orc_f16_rne(float_of(amax));
    if (s16 > smax) s16 = smax;
    return s16;
}

static void quant_group_m(const float* z, int n, int8_t* q, uint16_t* s)
{
    uint16_t s16 = group_scale(z, n, 0x3FFF);   /* 0x3FFF = 1.999..., keeps 2-|z| > 0 */
    *s = s16;
    if (s16 == 0) {
        for (int j = 0; j < n; ++j) q[j] = 0;
        return;
    }
    float sc = orc_f16_to_f32(s16);
    float r = 127.0f / sc;
    for (int j = 0; j < n; ++j) {
        float y = z[j] * r;
        q[j] = (int8_t)clampf(rne_to_int(y), -127.0f, 127.0f);
    }
}

static void quant_group_v(const float* w, int n, uint8_t* q, uint16_t* s)
{
    uint16_t s16 = group_scale(w, n, 0x7BFF);   /* 0x7BFF = 65504, largest finite */
    *s = s16;
    if (s16 == 0) {
        for (int j = 0; j < n; ++j) q[j] = 0;
        return;
    }
    float sc = orc_f16_to_f32(s16);
    float r = 255.0f / sc;
    for (int j = 0; j < n; ++j) {
        float y = w[j] * r;
        q[j] = (uint8_t)clampf(rne_to_int(y), 0.0f, 255.0f);
    }
}

static float dequant_m1(int8_t q, uint16_t s16)
{
    float s = orc_f16_to_f32(s16);
    float d = s * K8;
    float z = (float)q * d;
    return orc_phi_m_inv(z);
}

static float dequant_v1(uint8_t q, uint16_t s16)
{
    float s = orc_f16_to_f32(s16);
    float d = s * K255;
    float z = (float)q * d;
    return orc_phi_v_inv(z);
}

static int group_len(int64_t n, int64_t g)
{
    int64_t rem = n - g * GROUP;
    return rem < GROUP ? (int)rem : GROUP;
}

void orc_quant_m(const float* m, int64_t n, int8_t* q, uint16_t* s)
{
    for (int64_t g = 0; g * GROUP < n; ++g) {
        int len = group_len(n, g);
        float z[GROUP];
        for (int j = 0; j < len; ++j) z[j] = orc_phi_m(m[g * GROUP + j]);
        quant_group_m(z, len, q + g * GROUP, s + g);
    }
}

void orc_dequant_m(const int8_t* q, const uint16_t* s, int64_t n, float* m)
{
    for (int64_t i = 0; i < n; ++i) m[i] = dequant_m1(q[i], s[i / GROUP]);
}

void orc_quant_v(const float* v, int64_t n, uint8_t* q, uint16_t* s)
{
    for (int64_t g = 0; g * GROUP < n; ++g) {
        int len = group_len(n, g);
        float w[GROUP];
        for (int j = 0; j < len; ++j) w[j] = orc_phi_v(v[g * GROUP + j]);
        quant_group_v(w, len, q + g * GROUP, s + g);
    }
}

void orc_dequant_v(const uint8_t* q, const uint16_t* s, int64_t n, float* v)
{
    for (int64_t i = 0; i < n; ++i) v[i] = dequant_v1(q[i], s[i / GROUP]);
}

/* Linear quantisers (no companding): z = m or z = v. */
void orc_quant_lin_m(const float* m, int64_t n, int8_t* q, uint16_t* s)
{
    for (int64_t g = 0; g * GROUP < n; ++g) {
        int len = group_len(n, g);
        const float* z = m + g * GROUP;
        uint16_t s16 = group_scale(z, len, 0x7BFF);
        s[g] = s16;
        float r = s16 ? 127.0f / orc_f16_to_f32(s16) : 0.0f;
        for (int j = 0; j < len; ++j) {
            float y = z[j] * r;
            q[g * GROUP + j] = s16 ? (int8_t)clampf(rne_to_int(y), -127.0f, 127.0f) : 0;
        }
    }
}

void orc_dequant_lin_m(const int8_t* q, const uint16_t* s, int64_t n, float* m)
{
    for (int64_t i = 0; i < n; ++i) {
        float d = orc_f16_to_f32(s[i / GROUP]) * K8;
        m[i] = (float)q[i] * d;
    }
}

void orc_quant_lin_v(const float* v, int64_t n, uint8_t* q, uint16_t* s)
{
    for (int64_t g = 0; g * GROUP < n; ++g)
        quant_group_v(v + g * GROUP, group_len(n, g), q + g * GROUP, s + g);
}

void orc_dequant_lin_v(const uint8_t* q, const uint16_t* s, int64_t n, float* v)
{
    for (int64_t i = 0; i < n; ++i) {
        float d = orc_f16_to_f32(s[i / GROUP]) * K255;
        v[i] = (float)q[i] * d;
    }
}

/* ------------------------------------------------------------------------ */
/* Host scalars.                                                             */

void orc_adamw_scalars(double lr, double beta1, double beta2, double eps, double wd,
                       int64_t t, float out[8])
{
    double p1 = 1.0, p2 = 1.0;
    for (int64_t k = 0; k < t; ++k) {
        p1 = p1 * beta1;
        p2 = p2 * beta2;
    }
    out[0] = (float)beta1;                 /* b1 */
    out[1] = (float)(1.0 - beta1);         /* c1 */
    out[2] = (float)beta2;                 /* b2 */
    out[3] = (float)(1.0 - beta2);         /* c2 */
    out[4] = (float)(lr / (1.0 - p1));     /* alpha: lr with the first-moment bias correction */
    out[5] = (float)(1.0 / sqrt(1.0 - p2));/* kappa: second-moment bias correction of sqrt(v) */
    out[6] = (float)eps;
    out[7] = (float)(1.0 - lr * wd);       /* lambda: decoupled weight decay factor */
}

/* ------------------------------------------------------------------------ */
/* The updates of one element, shared by the compressed and the FP32 steps.  */

/* AdamW (reading of "standard AdamW"): returns theta_n; sc from
 * orc_adamw_scalars. */
static float adam1(const float sc[8], float theta_hat, float m, float v, float gr,
                   float* m_new, float* v_new, float* root)
{
    const float b1 = sc[0], c1 = sc[1], b2 = sc[2], c2 = sc[3];
    const float alpha = sc[4], kappa = sc[5], epsf = sc[6], lambda = sc[7];
    float bm = b1 * m;
    float cg = c1 * gr;
    float mn = bm + cg;
    float bv = b2 * v;
    float gg = gr * gr;
    float cgg = c2 * gg;
    float vn = bv + cgg;
    float w = sqrtf(vn);
    float denom_a = w * kappa;
    float denom = denom_a + epsf;
    float u = mn / denom;
    float decayed = lambda * theta_hat;
    float step = alpha * u;
    *m_new = mn;
    *v_new = vn;
    *root = w;
    return decayed - step;
}

/* SGD with momentum: L2 decay added to the gradient, no dampening. */
static float sgd1(float mu, float eta, float omega, float theta_hat, float b, float gr,
                  float* b_new)
{
    float decay = omega * theta_hat;
    float g2 = gr + decay;
    float mb = mu * b;
    float bn = mb + g2;
    float step = eta * bn;
    *b_new = bn;
    return theta_hat - step;
}

/* Lion (see orc_lion_step): lc = {b1, c1, b2, c2, eta, lambda}. */
static float sign1(float c);
static void lion_scalars(double lr, double beta1, double beta2, double wd, float lc[6])
{
    lc[0] = (float)beta1;
    lc[1] = (float)(1.0 - beta1);
    lc[2] = (float)beta2;
    lc[3] = (float)(1.0 - beta2);
    lc[4] = (float)lr;
    lc[5] = (float)(1.0 - lr * wd);
}

static float lion1(const float lc[6], float theta_hat, float m, float gr, float* m_new)
{
    float bm = lc[0] * m;
    float cg = lc[1] * gr;
    float c = bm + cg;
    float sgn = sign1(c);
    if (sgn == 0.0f) sgn = 0.0f;           /* a zero direction is +0 */
    float decayed = lc[5] * theta_hat;
    float step = lc[4] * sgn;
    float b2m = lc[2] * m;
    float c2g = lc[3] * gr;
    *m_new = b2m + c2g;
    return decayed - step;
}

/* ------------------------------------------------------------------------ */
/* Fused steps over one tensor.                                              */

/* linear_v = 0: the method.  linear_v = 1: the Fig. 5 ablation, the variance
 * stored by the linear quantiser (read as q*RN(s*K255); written as the
 * group scale and codes of v' itself, no square root). */
static void adamw_step(int64_t n, uint16_t* tb, int8_t* rho, int8_t* qm, uint16_t* sm,
                       uint8_t* qv, uint16_t* sv, const uint16_t* grad,
                       double lr, double beta1, double beta2, double eps, double wd, int64_t t,
                       float* theta_out, float* m_out, float* v_out, int linear_v)
{
    float sc[8];
    orc_adamw_scalars(lr, beta1, beta2, eps, wd, t, sc);

    for (int64_t g = 0; g * GROUP < n; ++g) {
        int len = group_len(n, g);
        int64_t o = g * GROUP;
        float mn[GROUP], w[GROUP], z[GROUP], tn[GROUP];
        for (int j = 0; j < len; ++j) {
            float theta_hat = unsplit1(tb[o + j], rho[o + j]);
            float m = dequant_m1(qm[o + j], sm[g]);
            float v = linear_v ? (float)qv[o + j] * (orc_f16_to_f32(sv[g]) * K255)
                               : dequant_v1(qv[o + j], sv[g]);
            float gr = orc_bf16_to_f32(grad[o + j]);
            float m_new, v_new, root;
            float theta_new = adam1(sc, theta_hat, m, v, gr, &m_new, &v_new, &root);

            mn[j] = m_new;
            w[j] = linear_v ? v_new : root;    /* what the variance codes quantise */
            tn[j] = theta_new;
            if (theta_out) theta_out[o + j] = theta_new;
            if (m_out) m_out[o + j] = m_new;
            if (v_out) v_out[o + j] = v_new;
        }
        for (int j = 0; j < len; ++j) z[j] = orc_phi_m(mn[j]);
        quant_group_m(z, len, qm + o, sm + g);
        quant_group_v(w, len, qv + o, sv + g);
        for (int j = 0; j < len; ++j) split1(tn[j], &tb[o + j], &rho[o + j]);
    }
}

void orc_adamw_step(int64_t n, uint16_t* tb, int8_t* rho, int8_t* qm, uint16_t* sm,
                    uint8_t* qv, uint16_t* sv, const uint16_t* grad,
                    double lr, double beta1, double beta2, double eps, double wd, int64_t t,
                    float* theta_out, float* m_out, float* v_out)
{
    adamw_step(n, tb, rho, qm, sm, qv, sv, grad, lr, beta1, beta2, eps, wd, t, theta_out, m_out,
               v_out, 0);
}

void orc_adamw_step_linv(int64_t n, uint16_t* tb, int8_t* rho, int8_t* qm, uint16_t* sm,
                         uint8_t* qv, uint16_t* sv, const uint16_t* grad,
                         double lr, double beta1, double beta2, double eps, double wd, int64_t t,
                         float* theta_out, float* m_out, float* v_out)
{
    adamw_step(n, tb, rho, qm, sm, qv, sv, grad, lr, beta1, beta2, eps, wd, t, theta_out, m_out,
               v_out, 1);
}

void orc_sgd_step(int64_t n, uint16_t* tb, int8_t* rho, int8_t* qb, uint16_t* sb,
                  const uint16_t* grad, double lr, double momentum, double wd, int64_t t,
                  float* theta_out, float* b_out)
{
    (void)t;                               /* SGD with momentum has no step-dependent scalar */
    const float mu = (float)momentum;
    const float eta = (float)lr;
    const float omega = (float)wd;
    for (int64_t g = 0; g * GROUP < n; ++g) {
        int len = group_len(n, g);
        int64_t o = g * GROUP;
        float bn[GROUP], z[GROUP], tn[GROUP];
        for (int j = 0; j < len; ++j) {
            float theta_hat = unsplit1(tb[o + j], rho[o + j]);
            float b = dequant_m1(qb[o + j], sb[g]);
            float gr = orc_bf16_to_f32(grad[o + j]);
            float b_new;
            float theta_new = sgd1(mu, eta, omega, theta_hat, b, gr, &b_new);

            bn[j] = b_new;
            tn[j] = theta_new;
            if (theta_out) theta_out[o + j] = theta_new;
            if (b_out) b_out[o + j] = b_new;
        }
        for (int j = 0; j < len; ++j) z[j] = orc_phi_m(bn[j]);
        quant_group_m(z, len, qb + o, sb + g);
        for (int j = 0; j < len; ++j) split1(tn[j], &tb[o + j], &rho[o + j]);
    }
}

/* Lion (named by the FlashOptim page as FlashLion; its update rule is the
 * published Lion algorithm, not printed on the page): with one compressed
 * momentum m per parameter,
 *     c = b1*m + c1*g,  theta_new = lambda*theta_hat - eta*sign(c),
 *     m_new = b2*m + c2*g,
 * sign(0) = 0, lambda = 1 - lr*wd (decoupled decay), every line one binary32
 * operation rounded to nearest.  m is stored like the AdamW momentum:
 * phi_m companding, INT8 codes, one FP16 scale per group. */
static float sign1(float c)
{
    if (c > 0.0f) return 1.0f;
    if (c < 0.0f) return -1.0f;
    return c;                              /* +-0 -> 0 (sign of a zero is dropped below); NaN stays NaN */
}

void orc_lion_step(int64_t n, uint16_t* tb, int8_t* rho, int8_t* qm, uint16_t* sm,
                   const uint16_t* grad, double lr, double beta1, double beta2, double wd,
                   float* theta_out, float* m_out)
{
    float lc[6];
    lion_scalars(lr, beta1, beta2, wd, lc);
    for (int64_t g = 0; g * GROUP < n; ++g) {
        int len = group_len(n, g);
        int64_t o = g * GROUP;
        float mn[GROUP], z[GROUP], tn[GROUP];
        for (int j = 0; j < len; ++j) {
            float theta_hat = unsplit1(tb[o + j], rho[o + j]);
            float m = dequant_m1(qm[o + j], sm[g]);
            float gr = orc_bf16_to_f32(grad[o + j]);
            float m_new;
            float theta_new = lion1(lc, theta_hat, m, gr, &m_new);

            mn[j] = m_new;
            tn[j] = theta_new;
            if (theta_out) theta_out[o + j] = theta_new;
            if (m_out) m_out[o + j] = m_new;
        }
        for (int j = 0; j < len; ++j) z[j] = orc_phi_m(mn[j]);
        quant_group_m(z, len, qm + o, sm + g);
        for (int j = 0; j < len; ++j) split1(tn[j], &tb[o + j], &rho[o + j]);
    }
}

/* ------------------------------------------------------------------------ */
/* Compression disabled (Practical advice: compression can be switched off  */
/* per layer).  The same updates over an FP32 master weight and FP32        */
/* moments, in place; tb receives theta' = bf16_rne(theta_n), the weight    */
/* the model computes with.                                                 */

void orc_adamw_step_fp32(int64_t n, float* theta, float* m, float* v, uint16_t* tb,
                         const uint16_t* grad, double lr, double beta1, double beta2,
                         double eps, double wd, int64_t t)
{
    float sc[8];
    orc_adamw_scalars(lr, beta1, beta2, eps, wd, t, sc);
    for (int64_t i = 0; i < n; ++i) {
        float m_new, v_new, root;
        float theta_new = adam1(sc, theta[i], m[i], v[i], orc_bf16_to_f32(grad[i]), &m_new,
                                &v_new, &root);
        theta[i] = theta_new;
        m[i] = m_new;
        v[i] = v_new;
        tb[i] = orc_bf16_rne(theta_new);
    }
}

void orc_sgd_step_fp32(int64_t n, float* theta, float* b, uint16_t* tb, const uint16_t* grad,
                       double lr, double momentum, double wd)
{
    const float mu = (float)momentum, eta = (float)lr, omega = (float)wd;
    for (int64_t i = 0; i < n; ++i) {
        float b_new;
        float theta_new = sgd1(mu, eta, omega, theta[i], b[i], orc_bf16_to_f32(grad[i]), &b_new);
        theta[i] = theta_new;
        b[i] = b_new;
        tb[i] = orc_bf16_rne(theta_new);
    }
}

void orc_lion_step_fp32(int64_t n, float* theta, float* m, uint16_t* tb, const uint16_t* grad,
                        double lr, double beta1, double beta2, double wd)
{
    float lc[6];
    lion_scalars(lr, beta1, beta2, wd, lc);
    for (int64_t i = 0; i < n; ++i) {
        float m_new;
        float theta_new = lion1(lc, theta[i], m[i], orc_bf16_to_f32(grad[i]), &m_new);
        theta[i] = theta_new;
        m[i] = m_new;
        tb[i] = orc_bf16_rne(theta_new);
    }
}

/* ------------------------------------------------------------------------ */
/* Array helpers for exhaustive checks.                                      */

void orc_bf16_rne_array(const float* x, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_rne(x[i]);
}

void orc_f16_rne_array(const float* x, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_f16_rne(x[i]);
}

void orc_f16_to_f32_array(const uint16_t* h, int64_t n, float* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_f16_to_f32(h[i]);
}

void orc_phi_m_array(const float* x, int64_t n, float* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_phi_m(x[i]);
}

void orc_phi_m_inv_array(const float* z, int64_t n, float* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_phi_m_inv(z[i]);
}

void orc_phi_v_array(const float* x, int64_t n, float* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_phi_v(x[i]);
}

void orc_phi_v_inv_array(const float* z, int64_t n, float* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_phi_v_inv(z[i]);
}
