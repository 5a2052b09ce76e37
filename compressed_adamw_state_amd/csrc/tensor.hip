// One tensor's compressed state: flat split / unsplit (Eq. 1-2, Alg. 1) and
// group quantisation (Alg. 2-3) of "FlashOptim: Optimizers for Memory
// Efficient Training" (digest page, "Core method"), state init from FP32,
// export to FP32, list zeroing and gradient pointers.
#include <algorithm>

#include "host.hpp"
#include "quant.hpp"

namespace flashopt {

__global__ __launch_bounds__(256) void split_kernel(const float* x, int64_t n, uint16_t* tb,
                                                     int8_t* rho) {
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
        uint32_t otb[8], orho[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const Split sp = split(v[j]);
            otb[j] = sp.tb;
            orho[j] = (uint32_t)sp.rho;
        }
        if (full) {
            *reinterpret_cast<uint4*>(tb + e) = pack_u16x8(otb);
            *reinterpret_cast<uint2*>(rho + e) = pack_u8x8(orho);
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (e + j < n) { tb[e + j] = (uint16_t)otb[j]; rho[e + j] = (int8_t)orho[j]; }
        }
    }
}

__global__ __launch_bounds__(256) void unsplit_kernel(const uint16_t* tb, const int8_t* rho,
                                                       int64_t n, float* out) {
    FLAT_LOOP(n) {
        const int64_t e = c * kSubTile + lane * kLaneElems;
        const bool full = (c + 1) * kSubTile <= n;
        uint32_t th[8];
        int32_t r[8];
        if (full) {
            unpack_bf16x8(*reinterpret_cast<const uint4*>(tb + e), th);
            unpack_s8x8(*reinterpret_cast<const uint2*>(rho + e), r);
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                th[j] = (e + j < n) ? tb[e + j] : 0u;
                r[j] = (e + j < n) ? rho[e + j] : 0;
            }
        }
        float o[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j] = unsplit(th[j], r[j]);
        if (full) {
            *reinterpret_cast<float4*>(out + e) = make_float4(o[0], o[1], o[2], o[3]);
            *reinterpret_cast<float4*>(out + e + 4) = make_float4(o[4], o[5], o[6], o[7]);
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) if (e + j < n) out[e + j] = o[j];
        }
    }
}

// ---- list maintenance kernels ----------------------------------------------

// Zero the momentum / variance codes and the scales of a list (rho kept), one
// tile per wave.
template <int kOpt>
__global__ __launch_bounds__(256) void zero_kernel(const DevTensor* __restrict__ table,
                                                   const int64_t* __restrict__ tile_begin,
                                                   int32_t count, int64_t total_tiles) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t wave = uniform((int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x / kWave));
    const int64_t nwaves = (int64_t)gridDim.x * kWavesPerBlock;
    if (wave >= total_tiles) return;
    TileCursor cur;
    cur.start(table, tile_begin, count, kNoTensor, total_tiles, wave);
    for (int64_t tile = wave; tile < total_tiles; tile += nwaves) {
        cur.seek(table, tile_begin, tile);
        const GTensor& T = cur.T;
        const int64_t e0 = (tile - cur.begin) * kTile;
        for (int k = 0; k < kSubTiles; ++k) {
            const int64_t e = e0 + k * kSubTile + lane * kLaneElems;
            for (int j = 0; j < 8; ++j) {
                if (e + j < T.numel) {
                    *code_at<kOpt>(T, e + j, kM) = 0;
                    if (kOpt == kAdamW) *code_at<kOpt>(T, e + j, kV) = 0;
                }
            }
            if ((lane & 3) == 0 && e < T.numel) {
                T.scales[(e >> 5) * Layout<kOpt>::kScl] = 0;
                if (kOpt == kAdamW) T.scales[(e >> 5) * Layout<kOpt>::kScl + 1] = 0;
            }
        }
    }
}

// ---- one tensor: initialise from / export to FP32 ----------------------------

// theta' and rho from the FP32 weights (Eq. 1-2), momentum and variance codes
// and scales zero.
template <int kOpt>
__global__ __launch_bounds__(256) void init_kernel(DevTensor d, const float* x) {
    const GTensor T = view(d);
    const int64_t n = T.numel;
    FLAT_LOOP(n) {
        const int64_t e = c * kSubTile + lane * kLaneElems;
        for (int j = 0; j < 8; ++j) {
            if (e + j < n) {
                const Split sp = split(x[e + j]);
                T.theta[e + j] = (uint16_t)sp.tb;
                *code_at<kOpt>(T, e + j, kRho) = (uint8_t)sp.rho;
                *code_at<kOpt>(T, e + j, kM) = 0;
                if (kOpt == kAdamW) *code_at<kOpt>(T, e + j, kV) = 0;
            }
        }
        if ((lane & 3) == 0 && e < n) {
            T.scales[(e >> 5) * Layout<kOpt>::kScl] = 0;
            if (kOpt == kAdamW) T.scales[(e >> 5) * Layout<kOpt>::kScl + 1] = 0;
        }
    }
}

// The rebuilt FP32 master weight, momentum and (AdamW) variance; any output
// pointer may be null.
template <int kOpt, bool kLinV = false>
__global__ __launch_bounds__(256) void export_kernel(DevTensor d, float* theta_out, float* m_out,
                                                     float* v_out) {
    const GTensor T = view(d);
    const int64_t n = T.numel;
    FLAT_LOOP(n) {
        const int64_t e = c * kSubTile + lane * kLaneElems;
        if (e >= n) continue;
        const int64_t g = e >> 5;
        const float dm = m_step(T.scales[g * Layout<kOpt>::kScl]);
        const float dv = kOpt == kAdamW ? v_step(T.scales[g * Layout<kOpt>::kScl + 1]) : 0.0f;
        for (int j = 0; j < 8; ++j) {
            const int64_t i = e + j;
            if (i >= n) break;
            if (theta_out)
                theta_out[i] = unsplit(T.theta[i], (int8_t)*code_at<kOpt>(T, i, kRho));
            if (m_out) m_out[i] = dequant_m((int8_t)*code_at<kOpt>(T, i, kM), dm);
            if (kOpt == kAdamW && v_out) {
                const uint32_t q = *code_at<kOpt>(T, i, kV);
                v_out[i] = kLinV ? (float)q * dv : dequant_v(q, dv);
            }
        }
    }
}

constexpr int kGradBatch = 200;
struct GradBatch {
    int32_t first, count;
    const uint16_t* ptr[kGradBatch];
};

__global__ void set_grads_kernel(DevTensor* table, GradBatch b) {
    const int i = threadIdx.x;
    if (i < b.count) table[b.first + i].grad = (uint64_t)b.ptr[i];
}

int launch_set_grads(DevTensor* table, int32_t first, int32_t count,
                     const uint16_t* const* grads, hipStream_t st) {
    for (int32_t off = 0; off < count; off += kGradBatch) {
        GradBatch b;
        b.first = first + off;
        b.count = std::min<int32_t>(kGradBatch, count - off);
        for (int i = 0; i < b.count; ++i) b.ptr[i] = grads[off + i];
        hipLaunchKernelGGL(set_grads_kernel, dim3(1), dim3(kGradBatch), 0, st, table, b);
        const int s = launch_status();
        if (s != FLASHOPT_OK) return s;
    }
    return FLASHOPT_OK;
}

}  // namespace flashopt

using namespace flashopt;

extern "C" {

int flashopt_split(const float* theta, int64_t n, uint16_t* theta_bf16, int8_t* rho,
                   void* stream) {
    if (n < 0 || n > kMaxNumel) return FLASHOPT_ERR_SIZE;
    if (n == 0) return FLASHOPT_OK;
    if (!theta || !theta_bf16 || !rho) return FLASHOPT_ERR_NULL;
    if (!aligned(theta, 16) || !aligned(theta_bf16, 16) || !aligned(rho, 8))
        return FLASHOPT_ERR_ALIGN;
    const int64_t chunks = (n + kSubTile - 1) / kSubTile;
    hipLaunchKernelGGL(split_kernel, dim3(grid_for(chunks)), dim3(kBlock), 0,
                       (hipStream_t)stream, theta, n, theta_bf16, rho);
    return launch_status();
}

int flashopt_unsplit(const uint16_t* theta_bf16, const int8_t* rho, int64_t n, float* out,
                     void* stream) {
    if (n < 0 || n > kMaxNumel) return FLASHOPT_ERR_SIZE;
    if (n == 0) return FLASHOPT_OK;
    if (!theta_bf16 || !rho || !out) return FLASHOPT_ERR_NULL;
    if (!aligned(theta_bf16, 16) || !aligned(rho, 8) || !aligned(out, 16))
        return FLASHOPT_ERR_ALIGN;
    const int64_t chunks = (n + kSubTile - 1) / kSubTile;
    hipLaunchKernelGGL(unsplit_kernel, dim3(grid_for(chunks)), dim3(kBlock), 0,
                       (hipStream_t)stream, theta_bf16, rho, n, out);
    return launch_status();
}

static int quantize_common(int kind, const float* x, int64_t n, void* q, uint16_t* scale,
                           void* stream) {
    if (n < 0 || n > kMaxNumel) return FLASHOPT_ERR_SIZE;
    if (n == 0) return FLASHOPT_OK;
    if (!x || !q || !scale) return FLASHOPT_ERR_NULL;
    if (!aligned(x, 16) || !aligned(q, 8) || !aligned(scale, 2)) return FLASHOPT_ERR_ALIGN;
    const int64_t chunks = (n + kSubTile - 1) / kSubTile;
    if (kind == 0)
        hipLaunchKernelGGL(quantize_kernel<0>, dim3(grid_for(chunks)), dim3(kBlock), 0,
                           (hipStream_t)stream, x, n, (uint8_t*)q, scale);
    else
        hipLaunchKernelGGL(quantize_kernel<1>, dim3(grid_for(chunks)), dim3(kBlock), 0,
                           (hipStream_t)stream, x, n, (uint8_t*)q, scale);
    return launch_status();
}

static int dequantize_common(int kind, const void* q, const uint16_t* scale, int64_t n,
                             float* out, void* stream) {
    if (n < 0 || n > kMaxNumel) return FLASHOPT_ERR_SIZE;
    if (n == 0) return FLASHOPT_OK;
    if (!q || !scale || !out) return FLASHOPT_ERR_NULL;
    if (!aligned(q, 8) || !aligned(scale, 2) || !aligned(out, 16)) return FLASHOPT_ERR_ALIGN;
    const int64_t chunks = (n + kSubTile - 1) / kSubTile;
    if (kind == 0)
        hipLaunchKernelGGL(dequantize_kernel<0>, dim3(grid_for(chunks)), dim3(kBlock), 0,
                           (hipStream_t)stream, (const uint8_t*)q, scale, n, out);
    else
        hipLaunchKernelGGL(dequantize_kernel<1>, dim3(grid_for(chunks)), dim3(kBlock), 0,
                           (hipStream_t)stream, (const uint8_t*)q, scale, n, out);
    return launch_status();
}

int flashopt_quantize_m(const float* m, int64_t n, int8_t* q, uint16_t* scale, void* stream) {
    return quantize_common(0, m, n, q, scale, stream);
}
int flashopt_dequantize_m(const int8_t* q, const uint16_t* scale, int64_t n, float* m,
                          void* stream) {
    return dequantize_common(0, q, scale, n, m, stream);
}
int flashopt_quantize_v(const float* v, int64_t n, uint8_t* q, uint16_t* scale, void* stream) {
    return quantize_common(1, v, n, q, scale, stream);
}
int flashopt_dequantize_v(const uint8_t* q, const uint16_t* scale, int64_t n, float* v,
                          void* stream) {
    return dequantize_common(1, q, scale, n, v, stream);
}

size_t flashopt_codes_bytes(int32_t kind, int64_t numel) {
    if (!valid_kind(kind) || numel < 0 || numel > kMaxNumel) return 0;
    const bool adam = opt_of(kind) == kAdamW;
    if (is_fp32(kind))                           // whole 512-element blocks of FP32 fields
        return (size_t)((numel + kSubTile - 1) / kSubTile) * kSubTile * 4 * (adam ? 3 : 2);
    if (adam) return (size_t)((numel + kSubTile - 1) / kSubTile) * 1536;   // whole blocks
    return (size_t)((numel + 7) / 8) * 16;
}

size_t flashopt_scales_bytes(int32_t kind, int64_t numel) {
    if (!valid_kind(kind) || is_fp32(kind) || numel < 0 || numel > kMaxNumel) return 0;
    return (size_t)((numel + 31) / 32) * (opt_of(kind) == kAdamW ? 4 : 2);
}

int flashopt_tensor_init(const flashopt_tensor* t, int32_t kind, const float* theta,
                         void* stream) {
    if (!t) return FLASHOPT_ERR_NULL;
    if (!valid_kind(kind)) return FLASHOPT_ERR_ARG;
    const int st = check_tensor(*t, kind);
    if (st != FLASHOPT_OK) return st;
    if (t->numel == 0) return FLASHOPT_OK;
    if (!theta) return FLASHOPT_ERR_NULL;
    const int64_t chunks = (t->numel + kSubTile - 1) / kSubTile;
    const dim3 grid(grid_for(chunks));
    hipStream_t s = (hipStream_t)stream;
    if (kind == FLASHOPT_KIND_ADAMW || is_linv(kind))          // same layout, all codes zero
        hipLaunchKernelGGL(init_kernel<kAdamW>, grid, dim3(kBlock), 0, s, to_dev(*t), theta);
    else if (is_fp32(kind))
        return launch_init_fp32(opt_of(kind), to_dev(*t), theta, s);
    else
        hipLaunchKernelGGL(init_kernel<kSgd>, grid, dim3(kBlock), 0, s, to_dev(*t), theta);
    return launch_status();
}

int flashopt_tensor_export(const flashopt_tensor* t, int32_t kind, float* theta, float* m,
                           float* v, void* stream) {
    if (!t) return FLASHOPT_ERR_NULL;
    if (!valid_kind(kind)) return FLASHOPT_ERR_ARG;
    const int st = check_tensor(*t, kind);
    if (st != FLASHOPT_OK) return st;
    if (opt_of(kind) != kAdamW) v = nullptr;                // one-momentum layouts have no v
    if (t->numel == 0 || (!theta && !m && !v)) return FLASHOPT_OK;
    const int64_t chunks = (t->numel + kSubTile - 1) / kSubTile;
    const dim3 grid(grid_for(chunks));
    hipStream_t s = (hipStream_t)stream;
    if (kind == FLASHOPT_KIND_ADAMW)
        hipLaunchKernelGGL(export_kernel<kAdamW>, grid, dim3(kBlock), 0, s, to_dev(*t), theta, m,
                           v);
    else if (is_linv(kind))
        hipLaunchKernelGGL((export_kernel<kAdamW, true>), grid, dim3(kBlock), 0, s, to_dev(*t),
                           theta, m, v);
    else if (is_fp32(kind))
        return launch_export_fp32(opt_of(kind), to_dev(*t), theta, m, v, s);
    else
        hipLaunchKernelGGL(export_kernel<kSgd>, grid, dim3(kBlock), 0, s, to_dev(*t), theta, m,
                           v);
    return launch_status();
}

int flashopt_state_zero(const flashopt_list* L, void* stream) {
    if (!L) return FLASHOPT_ERR_NULL;
    if (L->total_tiles == 0) return FLASHOPT_OK;
    const dim3 grid(grid_for(L->total_tiles));
    hipStream_t s = (hipStream_t)stream;
    const DevTensor* tab = L->d_table;
    const int64_t* tb = L->d_tile_begin;
    if (L->kind == FLASHOPT_KIND_ADAMW || is_linv(L->kind))
        hipLaunchKernelGGL(zero_kernel<kAdamW>, grid, dim3(kBlock), 0, s, tab, tb, L->count,
                           L->total_tiles);
    else if (is_fp32(L->kind))
        return launch_zero_fp32(opt_of(L->kind), tab, tb, L->count, L->total_tiles, s);
    else
        hipLaunchKernelGGL(zero_kernel<kSgd>, grid, dim3(kBlock), 0, s, tab, tb, L->count,
                           L->total_tiles);
    return launch_status();
}

}  // extern "C"
