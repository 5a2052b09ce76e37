// Flat group quantiser kernels (momentum INT8 / variance UINT8 with one FP16
// scale per 32 elements): "FlashOptim: Optimizers for Memory Efficient
// Training" (digest page), "Core method > Optimizer-state quantisation with
// companding", Alg. 2-3; kCompand = false gives the linear quantiser of the
// companding ablation (Fig. 4-5).  Instantiated by tensor.hip and ablation.hip.
#pragma once

#include "device.hpp"

namespace flashopt {

// kind 0: momentum (INT8), kind 1: variance (UINT8); kCompand: phi_m / sqrt
// first (the method), or the values themselves (the linear ablation, whose
// momentum scale may reach the largest finite FP16)
template <int kKind, bool kCompand = true>
__global__ __launch_bounds__(256) void quantize_kernel(const float* x, int64_t n, uint8_t* q,
                                                        uint16_t* scale) {
    FLAT_LOOP(n) {
        const int64_t e = c * kSubTile + lane * kLaneElems;
        const bool full = (c + 1) * kSubTile <= n;
        float v[8];
        if (full) {
            const float4 a = *reinterpret_cast<const float4*>(x + e);
            const float4 b = *reinterpret_cast<const float4*>(x + e + 4);
            v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
            v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = (e + j < n) ? x[e + j] : 0.0f;
        }
        float z[8];
        uint32_t amax = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            z[j] = !kCompand ? v[j] : (kKind == 0) ? phi_m(v[j]) : __builtin_sqrtf(v[j]);
            amax = max(amax, as_u32(z[j]) & 0x7FFFFFFFu);
        }
        const uint32_t s16 =
            group_scale(quad_max_u32(amax), (kKind == 0 && kCompand) ? 0x3FFFu : 0x7BFFu);
        const float r = code_factor(s16, kKind == 0 ? 127.0f : 255.0f);
        uint32_t o[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            o[j] = (kKind == 0) ? (uint32_t)code_m(z[j], r) : code_v(z[j], r);
        if (full) {
            *reinterpret_cast<uint2*>(q + e) = pack_u8x8(o);
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) if (e + j < n) q[e + j] = (uint8_t)o[j];
        }
        if ((lane & 3) == 0 && e < n) scale[e >> 5] = (uint16_t)s16;
    }
}

template <int kKind, bool kCompand = true>
__global__ __launch_bounds__(256) void dequantize_kernel(const uint8_t* q, const uint16_t* scale,
                                                          int64_t n, float* out) {
    FLAT_LOOP(n) {
        const int64_t e = c * kSubTile + lane * kLaneElems;
        const bool full = (c + 1) * kSubTile <= n;
        uint32_t u[8];
        if (full) {
            unpack_u8x8(*reinterpret_cast<const uint2*>(q + e), u);
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) u[j] = (e + j < n) ? q[e + j] : 0u;
        }
        const uint32_t s16 = (e < n) ? scale[e >> 5] : 0u;
        float o[8];
        if (kKind == 0) {
            const float d = m_step(s16);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int32_t code = (int32_t)(int8_t)(uint8_t)u[j];
                o[j] = kCompand ? dequant_m(code, d) : (float)code * d;
            }
        } else {
            const float d = v_step(s16);
#pragma unroll
            for (int j = 0; j < 8; ++j) o[j] = kCompand ? dequant_v(u[j], d) : (float)u[j] * d;
        }
        if (full) {
            *reinterpret_cast<float4*>(out + e) = make_float4(o[0], o[1], o[2], o[3]);
            *reinterpret_cast<float4*>(out + e + 4) = make_float4(o[4], o[5], o[6], o[7]);
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) if (e + j < n) out[e + j] = o[j];
        }
    }
}

}  // namespace flashopt
