// Codec ablations of "FlashOptim: Optimizers for Memory Efficient Training"
// (digest page): the weight split with a BF16 or FP16 base and 1-16-bit
// corrections ("Weight splitting", Eq. 1-2, Fig. 3) and the linear group
// quantiser without companding ("Optimizer-state quantisation", Fig. 4-5).
#include "host.hpp"
#include "quant.hpp"

namespace flashopt {

// ---- codec ablations: BF16 / FP16 base, code widths up to 16 bits -----------
//
// The split of Eq. 1-2 with the base rounded to BF16 (base 0) or FP16 (base
// 1) and codes in [-qmax, qmax]: rho = clamp(rne(qmax * e)), e = (x - t)/h
// exact and the product exact (double); the rebuild t + (rho*RN(1/qmax))*h.
// h = ULP/2 above |t|, zero and subnormal bases using the minimum-normal
// spacing; a non-finite base gets rho = 0 and rebuilds to itself.

template <int kBase>
__device__ __forceinline__ void base_of(float x, uint32_t& bits, float& t, float& h) {
    if (kBase == 0) {
        bits = f32_to_bf16(x);
        t = bf16_to_f32(bits);
        h = half_ulp(bits << 16);
    } else {
        bits = f32_to_f16(x);
        t = f16_to_f32(bits);
        const int E = max((int)((bits >> 10) & 0x1Fu), 1);
        h = __builtin_amdgcn_ldexpf(1.0f, E - 26);
    }
}

template <int kBase>
__device__ __forceinline__ void base_h(uint32_t bits, float& t, float& h) {
    if (kBase == 0) {
        t = bf16_to_f32(bits);
        h = half_ulp(bits << 16);
    } else {
        t = f16_to_f32(bits);
        const int E = max((int)((bits >> 10) & 0x1Fu), 1);
        h = __builtin_amdgcn_ldexpf(1.0f, E - 26);
    }
}

template <int kBase>
__global__ __launch_bounds__(256) void split_ex_kernel(const float* x, int64_t n, int32_t qmax,
                                                        uint16_t* base, int16_t* rho) {
    FLAT_LOOP(n) {
        const int64_t e0 = c * kSubTile + lane * kLaneElems;
        for (int j = 0; j < 8; ++j) {
            const int64_t i = e0 + j;
            if (i >= n) break;
            uint32_t bits;
            float t, h;
            base_of<kBase>(x[i], bits, t, h);
            base[i] = (uint16_t)bits;
            int32_t r = 0;
            if (__builtin_isfinite(t)) {
                const float diff = x[i] - t;                      // exact
                const float ee = diff / h;                        // exact (power of two)
                double y = (double)ee * (double)qmax;             // exact
                y = __builtin_rint(y);
                y = y > qmax ? qmax : (y < -qmax ? -qmax : y);
                r = (int32_t)y;
            }
            rho[i] = (int16_t)r;
        }
    }
}

template <int kBase>
__global__ __launch_bounds__(256) void unsplit_ex_kernel(const uint16_t* base, const int16_t* rho,
                                                          int64_t n, float k, float* out) {
    FLAT_LOOP(n) {
        const int64_t e0 = c * kSubTile + lane * kLaneElems;
        for (int j = 0; j < 8; ++j) {
            const int64_t i = e0 + j;
            if (i >= n) break;
            float t, h;
            base_h<kBase>(base[i], t, h);
            if (!__builtin_isfinite(t)) { out[i] = t; continue; }
            const float cc = (float)rho[i] * k;
            const float d = cc * h;
            out[i] = t + d;
        }
    }
}

}  // namespace flashopt

using namespace flashopt;

extern "C" {

int flashopt_split_ex(const float* theta, int64_t n, int32_t base, int32_t qmax,
                      uint16_t* theta_base, int16_t* rho, void* stream) {
    if (n < 0 || n > kMaxNumel) return FLASHOPT_ERR_SIZE;
    if ((base != 0 && base != 1) || qmax < 1 || qmax > 32767) return FLASHOPT_ERR_ARG;
    if (n == 0) return FLASHOPT_OK;
    if (!theta || !theta_base || !rho) return FLASHOPT_ERR_NULL;
    if (!aligned(theta, 4) || !aligned(theta_base, 2) || !aligned(rho, 2)) return FLASHOPT_ERR_ALIGN;
    const int64_t chunks = (n + kSubTile - 1) / kSubTile;
    if (base == 0)
        hipLaunchKernelGGL(split_ex_kernel<0>, dim3(grid_for(chunks)), dim3(kBlock), 0,
                           (hipStream_t)stream, theta, n, qmax, theta_base, rho);
    else
        hipLaunchKernelGGL(split_ex_kernel<1>, dim3(grid_for(chunks)), dim3(kBlock), 0,
                           (hipStream_t)stream, theta, n, qmax, theta_base, rho);
    return launch_status();
}

int flashopt_unsplit_ex(const uint16_t* theta_base, const int16_t* rho, int64_t n, int32_t base,
                        int32_t qmax, float* out, void* stream) {
    if (n < 0 || n > kMaxNumel) return FLASHOPT_ERR_SIZE;
    if ((base != 0 && base != 1) || qmax < 1 || qmax > 32767) return FLASHOPT_ERR_ARG;
    if (n == 0) return FLASHOPT_OK;
    if (!theta_base || !rho || !out) return FLASHOPT_ERR_NULL;
    if (!aligned(theta_base, 2) || !aligned(rho, 2) || !aligned(out, 4)) return FLASHOPT_ERR_ALIGN;
    const float k = 1.0f / (float)qmax;                          // RN(1/qmax)
    const int64_t chunks = (n + kSubTile - 1) / kSubTile;
    if (base == 0)
        hipLaunchKernelGGL(unsplit_ex_kernel<0>, dim3(grid_for(chunks)), dim3(kBlock), 0,
                           (hipStream_t)stream, theta_base, rho, n, k, out);
    else
        hipLaunchKernelGGL(unsplit_ex_kernel<1>, dim3(grid_for(chunks)), dim3(kBlock), 0,
                           (hipStream_t)stream, theta_base, rho, n, k, out);
    return launch_status();
}

static int quantize_lin(int kind, const float* x, int64_t n, void* q, uint16_t* scale,
                        void* stream) {
    if (n < 0 || n > kMaxNumel) return FLASHOPT_ERR_SIZE;
    if (n == 0) return FLASHOPT_OK;
    if (!x || !q || !scale) return FLASHOPT_ERR_NULL;
    if (!aligned(x, 16) || !aligned(q, 8) || !aligned(scale, 2)) return FLASHOPT_ERR_ALIGN;
    const int64_t chunks = (n + kSubTile - 1) / kSubTile;
    if (kind == 0)
        hipLaunchKernelGGL((quantize_kernel<0, false>), dim3(grid_for(chunks)), dim3(kBlock), 0,
                           (hipStream_t)stream, x, n, (uint8_t*)q, scale);
    else
        hipLaunchKernelGGL((quantize_kernel<1, false>), dim3(grid_for(chunks)), dim3(kBlock), 0,
                           (hipStream_t)stream, x, n, (uint8_t*)q, scale);
    return launch_status();
}

static int dequantize_lin(int kind, const void* q, const uint16_t* scale, int64_t n, float* out,
                          void* stream) {
    if (n < 0 || n > kMaxNumel) return FLASHOPT_ERR_SIZE;
    if (n == 0) return FLASHOPT_OK;
    if (!q || !scale || !out) return FLASHOPT_ERR_NULL;
    if (!aligned(q, 8) || !aligned(scale, 2) || !aligned(out, 16)) return FLASHOPT_ERR_ALIGN;
    const int64_t chunks = (n + kSubTile - 1) / kSubTile;
    if (kind == 0)
        hipLaunchKernelGGL((dequantize_kernel<0, false>), dim3(grid_for(chunks)), dim3(kBlock), 0,
                           (hipStream_t)stream, (const uint8_t*)q, scale, n, out);
    else
        hipLaunchKernelGGL((dequantize_kernel<1, false>), dim3(grid_for(chunks)), dim3(kBlock), 0,
                           (hipStream_t)stream, (const uint8_t*)q, scale, n, out);
    return launch_status();
}

int flashopt_quantize_lin_m(const float* m, int64_t n, int8_t* q, uint16_t* scale, void* stream) {
    return quantize_lin(0, m, n, q, scale, stream);
}
int flashopt_dequantize_lin_m(const int8_t* q, const uint16_t* scale, int64_t n, float* m,
                              void* stream) {
    return dequantize_lin(0, q, scale, n, m, stream);
}
int flashopt_quantize_lin_v(const float* v, int64_t n, uint8_t* q, uint16_t* scale,
                            void* stream) {
    return quantize_lin(1, v, n, q, scale, stream);
}
int flashopt_dequantize_lin_v(const uint8_t* q, const uint16_t* scale, int64_t n, float* v,
                              void* stream) {
    return dequantize_lin(1, q, scale, n, v, stream);
}

}  // extern "C"
