// Device-side codec of FlashOptim's compressed state for gfx950.
//
// Method: "FlashOptim: Optimizers for Memory Efficient Training" (digest
// page), section "Core method": weight splitting (Eq. 1-2, Alg. 1),
// optimizer-state quantisation with companding (Alg. 2-3), fused step
// (Alg. 4).  The exact binary32 operation order is the one documented in
// include/flashopt.h; every function here performs those operations one by
// one (this file is compiled with -ffp-contract=off and correctly rounded
// division / square root).
//
// Lane layout used by every kernel: a wavefront of 64 lanes covers 512
// consecutive elements per sub-tile, lane l owning elements [8l, 8l+8).
// A quantisation group (32 elements) is therefore exactly one quad of lanes
// (4l..4l+3), so the group max is two DPP quad-permute steps, with no LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flashopt {

constexpr int kGroup = 32;
constexpr int kWave = 64;
constexpr int kLaneElems = 8;                       // elements per lane per sub-tile
constexpr int kSubTile = kWave * kLaneElems;        // 512 elements
constexpr int kSubTiles = 4;
constexpr int kTile = kSubTile * kSubTiles;         // 2048 elements per wave

// RN(1/127) and RN(1/255) as bit patterns.
constexpr uint32_t kK8Bits = 0x3C010204u;
constexpr uint32_t kK255Bits = 0x3B808081u;

__device__ __forceinline__ float as_f32(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t as_u32(float f) { return __float_as_uint(f); }

// ---- format conversions ---------------------------------------------------

// BF16 is the upper half of a binary32 pattern.
__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return as_f32(b << 16); }

// binary32 -> BF16, round to nearest even; NaN keeps its payload, made quiet.
__device__ __forceinline__ uint32_t f32_to_bf16(float x) {
    uint32_t b = as_u32(x);
    uint32_t rounded = (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
    bool nan = (b & 0x7FFFFFFFu) > 0x7F800000u;
    return nan ? ((b >> 16) | 0x40u) : rounded;
}

// binary32 -> FP16 (v_cvt_f16_f32: round to nearest even, FP16 subnormals kept).
__device__ __forceinline__ uint32_t f32_to_f16(float x) {
    _Float16 h = (_Float16)x;
    return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float f16_to_f32(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// ---- weight split (Eq. 1-2) -----------------------------------------------

// ULP(theta')/2 from the exponent bits of theta' (as binary32 bits): the
// power of two 2^(E-127) times 2^-8, where E is clamped to [1, 254] (zero and
// subnormal theta' use the smallest normal spacing; for Inf/NaN theta' any
// finite h leaves theta' unchanged).  The product is exact, also when it is
// subnormal.
__device__ __forceinline__ float half_ulp(uint32_t theta_bits) {
    uint32_t e = theta_bits & 0x7F800000u;
    e = min(max(e, 0x00800000u), 0x7F000000u);
    return as_f32(e) * 0x1p-8f;
}

// Rebuilt master weight: theta' + (rho * K8) * h, from theta' as binary32 bits.
// Computed as (rho * (K8 * 2^-8)) * 2^(E-127): K8 * 2^-8 is exact, and for
// |rho| >= 1 the first product is at least 2^-15, so scaling by 2^-8 commutes
// with its rounding; the second product rounds once, like (rho*K8) * h.
__device__ __forceinline__ float unsplit_bits(uint32_t tbits, int32_t rho) {
    const float t = as_f32(tbits);
    const uint32_t e = min(max(tbits & 0x7F800000u, 0x00800000u), 0x7F000000u);
    const float c = (float)rho * as_f32(kK8Bits - 0x04000000u);   // K8 * 2^-8
    const float d = c * as_f32(e);
    return t + d;
}

// The same rebuild as one FMA: (rho*K8*2^-8) * 2^(E-127) is a power-of-two
// scaling of the first product, exact when the field E is at least 16 (|rho|
// >= 1 makes the first product at least 2^-15), so fma rounds once to the same
// t + d.  The field is taken unclamped and folded into emin / emax: for E in
// [16, 254] the clamp of unsplit_bits() changes nothing, and the caller redoes
// the lane with unsplit_bits() when any field falls outside.
__device__ __forceinline__ float unsplit_fma(uint32_t tbits, int32_t rho, uint32_t& emin,
                                             uint32_t& emax) {
    const float t = as_f32(tbits);
    const uint32_t e = tbits & 0x7F800000u;
    emin = min(emin, e);
    emax = max(emax, e);
    const float c = (float)rho * as_f32(kK8Bits - 0x04000000u);   // K8 * 2^-8
    return __builtin_fmaf(c, as_f32(e), t);
}

__device__ __forceinline__ bool unsplit_fma_ok(uint32_t emin, uint32_t emax) {
    return emin >= (16u << 23) && emax <= 0x7F000000u;             // E in [16, 254]
}

__device__ __forceinline__ float unsplit(uint32_t tb, int32_t rho) {
    return unsplit_bits(tb << 16, rho);
}

// Split: theta' = BF16(x); rho = clamp(rne(127 * (x - theta') / h), +-127).
// (x - theta') is exact, and dividing by the power of two h is done exactly by
// ldexp with the negated exponent.
struct Split { uint32_t tb; int32_t rho; };

__device__ __forceinline__ Split split(float x) {
    uint32_t tb = f32_to_bf16(x);
    uint32_t tbits = tb << 16;
    float t = as_f32(tbits);
    uint32_t E = (tbits >> 23) & 0xFFu;
    int shift = 135 - (int)max(E, 1u);
    float e = __builtin_amdgcn_ldexpf(x - t, shift);
    float y = e * 127.0f;
    float r = __builtin_rintf(y);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    Split s;
    s.tb = tb;
    s.rho = (E == 0xFFu) ? 0 : (int32_t)r;
    return s;
}

// ---- companding (Alg. 2-3) ------------------------------------------------

__device__ __forceinline__ float phi_m(float x) {
    float num = 2.0f * x;
    float den = 1.0f + fabsf(x);
    return num / den;
}

__device__ __forceinline__ float phi_m_inv(float z) {
    float den = 2.0f - fabsf(z);
    return z / den;
}

// Per-group dequantisation factors: s*K8 (momentum), s*K255 (variance).
__device__ __forceinline__ float m_step(uint32_t s16) { return f16_to_f32(s16) * as_f32(kK8Bits); }
__device__ __forceinline__ float v_step(uint32_t s16) { return f16_to_f32(s16) * as_f32(kK255Bits); }

__device__ __forceinline__ float dequant_m(int32_t q, float d) {
    float z = (float)q * d;
    return phi_m_inv(z);
}

__device__ __forceinline__ float dequant_v(uint32_t q, float d) {
    float z = (float)q * d;
    return z * z;
}

// ---- group maximum over a quad of lanes (DPP quad_perm) --------------------

__device__ __forceinline__ uint32_t quad_max_u32(uint32_t a) {
    // quad_perm [1,0,3,2] then [2,3,0,1]; every lane of the quad ends with the
    // max.  The DPP moves take 0 (the identity of the max) as the old value, so
    // each step compiles to a single v_max_u32 with a DPP source.
    uint32_t b = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, 0xB1, 0xF, 0xF, false);
    a = max(a, b);
    b = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, 0x4E, 0xF, 0xF, false);
    return max(a, b);
}

// Scale of a group from the quad-reduced max |z| bit pattern, capped.
__device__ __forceinline__ uint32_t group_scale(uint32_t amax_bits, uint32_t cap) {
    uint32_t s16 = f32_to_f16(as_f32(amax_bits));
    return min(s16, cap);
}

// Reciprocal factor 127/s (or 255/s); 0 when the scale is 0 (all codes 0).
__device__ __forceinline__ float code_factor(uint32_t s16, float qmax) {
    float s = f16_to_f32(s16);
    float r = qmax / s;
    return s16 == 0u ? 0.0f : r;
}

__device__ __forceinline__ int32_t code_m(float z, float r) {
    float y = z * r;
    float q = __builtin_rintf(y);
    q = fminf(fmaxf(q, -127.0f), 127.0f);
    return (int32_t)q;
}

__device__ __forceinline__ uint32_t code_v(float w, float r) {
    float y = w * r;
    float q = __builtin_rintf(y);
    q = fminf(fmaxf(q, 0.0f), 255.0f);
    return (uint32_t)q;
}

// ---- short exactly rounded sequences ----------------------------------------
//
// Each function below returns the same bits as the IEEE operation it replaces
// (the compiler's correctly rounded division / square root above) on the
// whole domain where it is used; the GPU test suite checks this exhaustively
// over all 2^32 binary32 inputs (and all 2^16 FP16 scales).  They cost 4-9
// instructions instead of ~11 (division) and ~17 (square root).

// RN(a/b) from the hardware reciprocal estimate and one FMA correction of
// the quotient.  Exact for phi_m (a = 2x, b = 1+|x|, all x), phi_m^-1
// (a = z, b = 2-|z|, |z| < 2) and the code factors 127/s, 255/s.
__device__ __forceinline__ float div_rcp1(float a, float b) {
    const float y = __builtin_amdgcn_rcpf(b);
    const float q = a * y;
    const float r = __builtin_fmaf(-b, q, a);
    return __builtin_fmaf(r, y, q);
}

__device__ __forceinline__ float phi_m_fast(float x) {
    const float num = 2.0f * x;
    const float den = 1.0f + fabsf(x);
    return div_rcp1(num, den);
}

// phi_m(x) / 2 = x / (1+|x|) by the same sequence: every step of phi_m_fast
// scaled by 1/2, so 2 * phi_m_half_fast(x) == phi_m(x) wherever the halved
// value is normal (|phi_m(x)| >= 2^-125).  Below that both are too small to
// move a code or a scale (codes round |z| * 127/s < 2^-94 to 0; the FP16 scale
// of a group maximum below 2^-25 is 0).  The fused step keeps z/2 and folds
// the factor 2 into the group maximum and the code factor 254/s.
__device__ __forceinline__ float phi_m_half_fast(float x) {
    const float den = 1.0f + fabsf(x);
    return div_rcp1(x, den);
}

__device__ __forceinline__ float phi_m_inv_fast(float z) {
    const float den = 2.0f - fabsf(z);
    return div_rcp1(z, den);
}

__device__ __forceinline__ float code_factor_fast(uint32_t s16, float qmax) {
    const float r = div_rcp1(qmax, f16_to_f32(s16));
    return s16 == 0u ? 0.0f : r;
}

// Square root from the hardware reciprocal square root y = rsq(x) by one
// correction in the coupled form of the Newton-Raphson iteration for sqrt(x)
// and 1/(2 sqrt(x)) (the final step of Markstein's square root: P. Markstein,
// "IA-64 and Elementary Functions: Speed and Precision", 2000, chapter on
// square root): g = x*y approximates sqrt(x), the residual x - g*g is exact
// in one FMA, and g + residual*(y/2) in one more FMA rounds once.  Checked
// exhaustively to return the correctly rounded root for every finite x >=
// 2^-96; sqrt_fast_bad() flags 0 <= x < 2^-96 (x = 0 gives 0 * Inf = NaN,
// tiny x lose bits in the residual), and Inf or NaN x give NaN (the fused
// step's quotient guard catches those lanes).
__device__ __forceinline__ float sqrt_fast(float x) {
    const float q = __builtin_amdgcn_rsqf(x);
    const float g = x * q;
    const float d = __builtin_fmaf(-g, g, x);
    return __builtin_fmaf(d, 0.5f * q, g);
}

__device__ __forceinline__ bool sqrt_fast_bad(float x) {
    return as_u32(x) < 0x0F800000u;               // +0 <= x < 2^-96 (x >= +0)
}

// Re-split of two weights with the gfx950 BF16 convert (RNE).  For theta'
// with exponent field E in [14, 254], F = 127 * 2^(135-E) is a normal binary32
// built from the exponent bits, and (x - theta') * F is exactly e * 127 with
// |e| <= 1 (no clamp needed); adding 128 is exact too, so one FMA gives
// e*127 + 128 without rounding, and the packed u8 convert rounds it to
// nearest even: that byte is rho + 128 (the caller flips bit 7 of each byte).
// Returns the packed BF16 pair, writes the two biased codes into bytes kByte
// and kByte + 1 of `codes`, and folds the two exponent fields into emin/emax;
// the results are exact when split_fast_ok(emin, emax) holds.
template <int kByte>
__device__ __forceinline__ uint32_t split2_fast(float x0, float x1, uint32_t& codes,
                                                uint32_t& emin, uint32_t& emax) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const f32x2 v = {x0, x1};
    const uint32_t packed = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
    const uint32_t t0b = packed << 16, t1b = packed & 0xFFFF0000u;
    const uint32_t e0 = t0b & 0x7F800000u, e1 = t1b & 0x7F800000u;
    const float y0 = __builtin_fmaf(x0 - as_f32(t0b), as_f32(0x867E0000u - e0), 128.0f);
    const float y1 = __builtin_fmaf(x1 - as_f32(t1b), as_f32(0x867E0000u - e1), 128.0f);
    codes = __builtin_amdgcn_cvt_pk_u8_f32(y0, kByte, codes);
    codes = __builtin_amdgcn_cvt_pk_u8_f32(y1, kByte + 1, codes);
    emin = min(emin, min(e0, e1));
    emax = max(emax, max(e0, e1));
    return packed;
}

__device__ __forceinline__ bool split_fast_ok(uint32_t emin, uint32_t emax) {
    return emin >= 0x07000000u && emax <= 0x7F000000u;    // E in [14, 254]
}

// Momentum code clamp(rne(z * r), -127, 127) as the low byte of the result:
// clamping first is the same (rounding is monotone, +-127 are integers), and
// adding 1.5 * 2^23 rounds to nearest even, leaving the integer in the low
// mantissa bits (two's complement in the low byte).
__device__ __forceinline__ uint32_t code_m_bits(float z, float r) {
    const float y = z * r;
    const float c = __builtin_amdgcn_fmed3f(y, -127.0f, 127.0f);
    return as_u32(c + 12582912.0f);
}

// RN(1/b) for every positive normal b whose reciprocal is normal: the
// hardware estimate refined by one Newton step.
__device__ __forceinline__ float rcp_rn(float b) {
    const float y = __builtin_amdgcn_rcpf(b);
    const float e = __builtin_fmaf(-b, y, 1.0f);
    return __builtin_fmaf(e, y, y);
}

// RN(a/b) from r = RN(1/b) by Markstein's correction: q0 = RN(a*r), the
// residual a - b*q0 in one FMA, then RN(q0 + residual*r).  Exact whenever
// nothing leaves the normal range: b and 1/b normal, the residual
// representable (e(b) + e(q0) >= -103) and 2^-125 <= |q0| < 2^126.  The
// caller bounds e(b) from below, turns that into a window [2^L, 2^126) for
// |q0|, and tests quot_key(q0) < span, a single unsigned compare.
__device__ __forceinline__ float div_rn(float a, float b, float r, float& q0) {
    q0 = a * r;
    const float res = __builtin_fmaf(-b, q0, a);
    return __builtin_fmaf(res, r, q0);
}

// 2|q0| - 2^(L+1) as bit patterns (mod 2^32); below span = 2(bits(2^126) -
// bits(2^L)) exactly when |q0| is in [2^L, 2^126).  neg_lo2 = -2 bits(2^L).
__device__ __forceinline__ uint32_t quot_key(float q0, uint32_t neg_lo2) {
    return (as_u32(q0) << 1) + neg_lo2;
}

// The window for the Adam quotient u = m' / (w*kappa + eps): the denominator
// is at least eps and below 2^92 (w < 2^64, kappa <= 2^27) or not finite, so
// with e(b) >= e(eps) the residual is exact once e(q0) >= -103 - e(eps):
// L = max(-125, -103 - e(eps)).  eps subnormal or >= 2^100 gives span 0
// (every element takes the IEEE division).
__host__ __device__ inline void quot_window(float eps, uint32_t& neg_lo2, uint32_t& span) {
    const uint32_t eb = (__builtin_bit_cast(uint32_t, eps) >> 23) & 0xFFu;
    neg_lo2 = 0u;
    span = 0u;
    if (eb >= 1u && eb <= 127u + 99u) {
        int L = -103 - ((int)eb - 127);
        if (L < -125) L = -125;
        const uint32_t lo = (uint32_t)(L + 127) << 23, hi = (uint32_t)(126 + 127) << 23;
        neg_lo2 = 0u - 2u * lo;
        span = 2u * (hi - lo);
    }
}

// ---- the update rules (fused-step section) -----------------------------------

// quot_neg_lo2 / quot_span: the fast-quotient window for u = m' / (w*kappa +
// eps) (see div_rn); span 0 sends every element to the IEEE division.
struct AdamScalars {
    float b1, c1, b2, c2, alpha, kappa, eps, lambda;
    uint32_t quot_neg_lo2, quot_span;
};
static_assert(sizeof(AdamScalars) == 40, "ten 32-bit words");

// The binary32 AdamW scalars of step t from the double hyper-parameters and
// p1 = beta1^t, p2 = beta2^t: each value formed in binary64 (correctly
// rounded division and square root) and rounded once.  The host call and the
// device-scheduled call both use this one definition.
__host__ __device__ inline AdamScalars adam_scalars_from(double lr, double beta1, double beta2,
                                                         double eps, double wd, double p1,
                                                         double p2) {
    AdamScalars a;
    a.b1 = (float)beta1;
    a.c1 = (float)(1.0 - beta1);
    a.b2 = (float)beta2;
    a.c2 = (float)(1.0 - beta2);
    a.alpha = (float)(lr / (1.0 - p1));
    a.kappa = (float)(1.0 / sqrt(1.0 - p2));
    a.eps = (float)eps;
    a.lambda = (float)(1.0 - lr * wd);
    quot_window(a.eps, a.quot_neg_lo2, a.quot_span);
    return a;
}

struct SgdScalars { float mu, eta, omega; };
// Lion: b1, c1 = 1-beta1 (direction), b2, c2 = 1-beta2 (momentum), eta = lr,
// lambda = 1 - lr*wd.
struct LionScalars { float b1, c1, b2, c2, eta, lambda; };

// The SGD and Lion scalars from the double hyper-parameters, each rounded
// once (one definition for the host call and the device-scheduled call).
__host__ __device__ inline SgdScalars sgd_scalars_from(double lr, double momentum, double wd) {
    return SgdScalars{(float)momentum, (float)lr, (float)wd};
}
__host__ __device__ inline LionScalars lion_scalars_from(double lr, double beta1, double beta2,
                                                         double wd) {
    LionScalars l;
    l.b1 = (float)beta1;
    l.c1 = (float)(1.0 - beta1);
    l.b2 = (float)beta2;
    l.c2 = (float)(1.0 - beta2);
    l.eta = (float)lr;
    l.lambda = (float)(1.0 - lr * wd);
    return l;
}
// One kernel argument for every optimizer; each instantiation reads its own.
struct StepScalars {
    AdamScalars a;
    SgdScalars s;
    LionScalars l;
};

// Lion's step direction sign(c): +1, -1, +0 for a zero c (of either sign),
// NaN for NaN.
__device__ __forceinline__ float lion_sign(float c) {
    return c > 0.0f ? 1.0f : (c < 0.0f ? -1.0f : (c == c ? 0.0f : c));
}

}  // namespace flashopt
