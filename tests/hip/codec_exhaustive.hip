// Exhaustive device checks of the short exactly rounded sequences in
// compressed_adamw_state_amd/csrc/codec.hpp: on every binary32 input of the
// domain where the fused kernel uses them, each must return the same bits as
// the general sequence it replaces (correctly rounded division and square
// root, the emulated BF16 round-to-nearest-even, the float clamp-and-round
// of the variance codes).  Test infrastructure: the tests load this library
// and read back one mismatch counter per check and per thread.  A second
// kernel checks the Adam quotient sequence (div_rn) against the IEEE division
// on every pair of significands.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "codec.hpp"

using namespace flashopt;

constexpr int kChecks = 12;

__global__ void __launch_bounds__(256) all_inputs(uint32_t* count, uint32_t* example) {
    const uint64_t tid = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const uint64_t nth = (uint64_t)gridDim.x * blockDim.x;
    uint32_t c[kChecks] = {0};
    uint32_t ex[kChecks] = {0};
    for (uint64_t i = tid; i < (1ull << 32); i += nth) {
        const uint32_t bits = (uint32_t)i;
        const float x = as_f32(bits);
        const bool finite = (bits & 0x7F800000u) != 0x7F800000u;
        const float ax = fabsf(x);
        if (!finite) {
            // 2: the square root turns +Inf and every NaN into NaN (caught by the step's guard)
            if ((!(bits >> 31) || (bits & 0x007FFFFFu)) && !__builtin_isnan(sqrt_fast(x))) {
                c[2]++; ex[2] = bits;
            }
            continue;
        }
        // 0: phi_m, every x with |x| <= 2^125 except -0 (a momentum is never -0)
        if (ax <= 0x1p125f && bits != 0x80000000u && as_u32(phi_m_fast(x)) != as_u32(phi_m(x))) {
            c[0]++; ex[0] = bits;
        }
        // 1: phi_m^-1, every |z| < 2 except -0
        if (ax < 2.0f && bits != 0x80000000u &&
            as_u32(phi_m_inv_fast(x)) != as_u32(phi_m_inv(x))) {
            c[1]++; ex[1] = bits;
        }
        // 2: square root, every x >= 0 not flagged for the general path
        if (!(bits >> 31) && !sqrt_fast_bad(x) &&
            as_u32(sqrt_fast(x)) != as_u32(__builtin_sqrtf(x))) {
            c[2]++; ex[2] = bits;
        }
        // 3: re-split of x (paired with -x), when the exponent range is fast
        {
            uint32_t codes = 0x5A5A5A5Au;                 // bytes 0, 1 must be overwritten
            uint32_t emin = 0xFFFFFFFFu, emax = 0u;
            const uint32_t packed = split2_fast<0>(x, -x, codes, emin, emax);
            const bool bad = !split_fast_ok(emin, emax);
            const Split s0 = split(x), s1 = split(-x);
            const int32_t r0 = (int32_t)(int8_t)(uint8_t)((codes ^ 0x80u) & 0xFFu);
            const int32_t r1 = (int32_t)(int8_t)(uint8_t)(((codes >> 8) ^ 0x80u) & 0xFFu);
            if (!bad && (packed != (s0.tb | (s1.tb << 16)) || r0 != s0.rho || r1 != s1.rho ||
                         (codes >> 16) != 0x5A5Au)) {
                c[3]++; ex[3] = bits;
            }
            // 4: the flag is raised exactly outside theta' exponent [14, 254]
            const uint32_t E = (s0.tb >> 7) & 0xFFu;
            if (bad != (E < 14u || E == 255u)) { c[4]++; ex[4] = bits; }
        }
        // 5: variance code via the packed convert == clamp(rne(y), 0, 255), y in [0, 512]
        if (!(bits >> 31) && x <= 512.0f) {
            const uint32_t got = __builtin_amdgcn_cvt_pk_u8_f32(x, 0, 0u) & 0xFFu;
            if (got != code_v(x, 1.0f)) { c[5]++; ex[5] = bits; }
        }
        // 7: momentum code from the rounding add == clamp(rne(y), +-127), y in [-1000, 1000]
        if (ax <= 1000.0f && (code_m_bits(x, 1.0f) & 0xFFu) != ((uint32_t)code_m(x, 1.0f) & 0xFFu)) {
            c[7]++; ex[7] = bits;
        }
        // 8: Newton-refined reciprocal == RN(1/x) for every x in [2^-126, 2^126)
        if (!(bits >> 31) && bits >= 0x00800000u && bits < 0x7E800000u &&
            as_u32(rcp_rn(x)) != as_u32(1.0f / x)) {
            c[8]++; ex[8] = bits;
        }
        // 9: Adam quotient x / b inside the window of a pseudo-random eps, with
        //    b >= eps of any exponent up to 2^100 (plus Inf), against IEEE
        {
            uint32_t h = bits * 0x9E3779B1u;
            h ^= h >> 15; h *= 0x85EBCA77u; h ^= h >> 13;
            const uint32_t ee = 1u + (h & 0xFFu) % 226u;             // eps exponent field
            const float eps = as_f32((ee << 23) | ((h >> 8) & 0x7FFFFFu));
            uint32_t neg_lo2, span;
            quot_window(eps, neg_lo2, span);
            uint32_t h2 = h * 0xC2B2AE35u; h2 ^= h2 >> 16;
            const uint32_t be = ee + (h2 & 0xFFu) % (227u - ee);      // up to 2^100
            float b = as_f32((be << 23) | ((h2 * 0x27D4EB2Fu) >> 9));
            if (b < eps) b = eps;
            if ((h2 >> 24) == 0u) b = __builtin_inff();
            float q0;
            const float q = div_rn(x, b, rcp_rn(b), q0);
            if (quot_key(q0, neg_lo2) < span && as_u32(q) != as_u32(x / b)) {
                c[9]++; ex[9] = bits;
            }
        }
        // 10: halved phi_m: 2 * phi_m_half_fast(x) == phi_m(x) where |phi_m(x)| >= 2^-125,
        //     and below that the halved value stays below 2^-125 too
        if (ax <= 0x1p125f && bits != 0x80000000u) {
            const float z = phi_m(x), h = phi_m_half_fast(x);
            if (fabsf(z) >= 0x1p-125f ? as_u32(2.0f * h) != as_u32(z) : !(fabsf(h) < 0x1p-125f)) {
                c[10]++; ex[10] = bits;
            }
        }
        // 11: unsplit as one FMA == unsplit_bits for every BF16 theta' and code
        //     byte (first 2^24 inputs: theta' = bits >> 8, rho = low byte), when
        //     the flag allows it; the flag is raised exactly for fields outside
        //     [16, 254]
        if (bits < (1u << 24)) {
            const uint32_t tbits = (bits >> 8) << 16;
            const int32_t rho = (int32_t)(int8_t)(uint8_t)(bits & 0xFFu);
            uint32_t emin = 0xFFFFFFFFu, emax = 0u;
            const float f = unsplit_fma(tbits, rho, emin, emax);
            const float g = unsplit_bits(tbits, rho);
            const uint32_t E = (tbits >> 23) & 0xFFu;
            const bool ok = unsplit_fma_ok(emin, emax);
            if ((ok && as_u32(f) != as_u32(g)) || ok != (E >= 16u && E <= 254u)) {
                c[11]++; ex[11] = bits;
            }
        }
        // 6: the general path is used for +0 <= x < 2^-96 only
        if (!(bits >> 31) && sqrt_fast_bad(x) != (x >= 0.0f && x < 0x1p-96f)) {
            c[6]++; ex[6] = bits;
        }
    }
    for (int k = 0; k < kChecks; ++k) {
        count[tid * kChecks + k] = c[k];
        example[tid * kChecks + k] = ex[k];
    }
}

// per-group code factors 127/s and 255/s for every FP16 scale pattern
__global__ void all_scales(uint32_t* bad) {
    const uint32_t s16 = blockIdx.x * blockDim.x + threadIdx.x;    // grid covers 2^16 exactly
    uint32_t b = 0;
    const uint32_t mag = s16 & 0x7FFFu;
    if (mag < 0x7C00u) {
        if (as_u32(code_factor_fast(mag, 127.0f)) != as_u32(code_factor(mag, 127.0f))) b |= 1u;
        if (as_u32(code_factor_fast(mag, 255.0f)) != as_u32(code_factor(mag, 255.0f))) b |= 2u;
        if (as_u32(code_factor_fast(mag, 254.0f)) != as_u32(2.0f * code_factor(mag, 127.0f)))
            b |= 4u;
    }
    bad[s16] = b;
}

// div_rn(a, b) == a / b for every pair of significands: b = 1.j (one thread
// per j, 2^23 threads) and a = 1.i for i in [i0, i0 + n).  Both operations
// scale exactly by powers of two while the window conditions hold, so this
// covers every exponent inside the window.
__global__ void __launch_bounds__(256) all_quotients(uint32_t i0, uint32_t n, uint32_t* bad) {
    const uint32_t j = blockIdx.x * blockDim.x + threadIdx.x;      // grid covers 2^23 exactly
    const float b = as_f32(0x3F800000u | j);
    const float r = rcp_rn(b);
    uint32_t c = 0;
    for (uint32_t i = i0; i < i0 + n; ++i) {
        const float a = as_f32(0x3F800000u | i);
        float q0;
        c += as_u32(div_rn(a, b, r, q0)) != as_u32(a / b);
    }
    bad[j] += c;
}

extern "C" int codec_exhaustive_checks(void) { return kChecks; }

// one slice of the significand pairs: a = 1.i for i in [i0, i0 + n), n > 0,
// i0 + n <= 2^23; bad has 2^23 counters (accumulated)
extern "C" int codec_quotient_slice(uint32_t i0, uint32_t n, uint32_t* bad) {
    if (n == 0 || i0 + n > (1u << 23)) return -3;
    hipLaunchKernelGGL(all_quotients, dim3((1u << 23) / 256), dim3(256), 0, 0, i0, n, bad);
    if (hipGetLastError() != hipSuccess) return -1;
    return hipDeviceSynchronize() == hipSuccess ? 0 : -2;
}

extern "C" int codec_exhaustive_run(uint32_t* count, uint32_t* example, int blocks,
                                    uint32_t* scale_bad) {
    hipLaunchKernelGGL(all_inputs, dim3(blocks), dim3(256), 0, 0, count, example);
    hipLaunchKernelGGL(all_scales, dim3(256), dim3(256), 0, 0, scale_bad);
    if (hipGetLastError() != hipSuccess) return -1;
    return hipDeviceSynchronize() == hipSuccess ? 0 : -2;
}
