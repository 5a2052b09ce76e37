// The uncompressed state kinds (_FP32) for gfx950: a layer with compression
// switched off keeps its FP32 master weight and moments and takes the same
// update as the fused step ("FlashOptim: Optimizers for Memory Efficient
// Training", digest page, "Practical advice": compression may be disabled per
// layer).  Step, one-tensor init / export and list zeroing.
#include "host.hpp"

namespace flashopt {

// ---- the uncompressed step (_FP32 kinds) -------------------------------------
//
// Compression switched off for a layer: the FP32 master weight and moments in
// blocks of 512 elements [theta[512] | m[512] | v[512]] (6 KB, AdamW) or
// [theta[512] | m[512]] (4 KB), the update above on the stored values, and
// theta' = bf16_rne(theta_n) for the model.  The same tiles and launch shape
// as the compressed step; in a 512-element sub-tile lane l owns elements
// [4l, 4l+4) and [256+4l, 256+4l+4), so every 16-byte load and store of a
// wave covers one contiguous kilobyte of a field (a per-lane record of 8
// elements would spread each access over 96-byte strides).
template <int kOpt> struct LayoutF {
    static constexpr int kFields = kOpt == kAdamW ? 3 : 2;
    static constexpr int kBlock = kSubTile * 4 * kFields;   // bytes per 512-element block
};

// field f (0 theta, 1 m, 2 v) of element i
template <int kOpt>
__device__ __forceinline__ GLOBAL float* f32_at(const GTensor& T, int64_t i, int f) {
    return (GLOBAL float*)(T.codes + (i >> 9) * LayoutF<kOpt>::kBlock) + f * kSubTile + (i & 511);
}

// Every access of the uncompressed step covers whole lines, each touched once
// per step: all carry the non-temporal hint (2.5-3.2 % faster than without on
// the Llama-3.1-8B list).

struct RawF {
    uint4 th[2], m[2], v[2];        // a lane's 2 x 4 FP32 values of each field
    uint2 gr[2];                    // and its 2 x 4 BF16 gradients
};

// e: a sub-tile's first element (a multiple of 512)
template <int kOpt>
__device__ __forceinline__ void load_raw_f(const GTensor& T, int64_t e, int lane, RawF& R) {
    const GLOBAL uint8_t* blk = T.codes + (e >> 9) * LayoutF<kOpt>::kBlock + 16 * lane;
    R.gr[0] = ld2nt(T.grad + e + 4 * lane);
    R.gr[1] = ld2nt(T.grad + e + 256 + 4 * lane);
    R.th[0] = ld4nt(blk);
    R.th[1] = ld4nt(blk + 1024);
    R.m[0] = ld4nt(blk + 2048);
    R.m[1] = ld4nt(blk + 3072);
    if (kOpt == kAdamW) {
        R.v[0] = ld4nt(blk + 4096);
        R.v[1] = ld4nt(blk + 5120);
    }
}

__device__ __forceinline__ float f_at(const uint4* v, int j) { return as_f32(word(v[j >> 2], j & 3)); }

__device__ __forceinline__ float g_at(const uint2* v, int j) {
    const uint32_t w = word(v[j >> 2], (j & 3) >> 1);
    return as_f32((j & 1) ? (w & 0xFFFF0000u) : (w << 16));
}

template <int kOpt>
__device__ __forceinline__ void step_f(const GTensor& T, int64_t e, int lane, const RawF& R,
                                       const StepScalars& P) {
    uint32_t th[8], mo[8], vo[8], tb[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float v = (kOpt == kAdamW) ? f_at(R.v, j) : 0.0f;
        const Upd u = update<kOpt>(f_at(R.th, j), f_at(R.m, j), v, g_at(R.gr, j), P);
        th[j] = as_u32(u.theta);
        mo[j] = as_u32(u.m);
        vo[j] = as_u32(u.v);
        tb[j] = f32_to_bf16(u.theta);
    }
    GLOBAL uint8_t* blk = T.codes + (e >> 9) * LayoutF<kOpt>::kBlock + 16 * lane;
    st2nt(T.theta + e + 4 * lane, make_uint2(tb[0] | (tb[1] << 16), tb[2] | (tb[3] << 16)));
    st2nt(T.theta + e + 256 + 4 * lane, make_uint2(tb[4] | (tb[5] << 16), tb[6] | (tb[7] << 16)));
    st4nt(blk, make_uint4(th[0], th[1], th[2], th[3]));
    st4nt(blk + 1024, make_uint4(th[4], th[5], th[6], th[7]));
    st4nt(blk + 2048, make_uint4(mo[0], mo[1], mo[2], mo[3]));
    st4nt(blk + 3072, make_uint4(mo[4], mo[5], mo[6], mo[7]));
    if (kOpt == kAdamW) {
        st4nt(blk + 4096, make_uint4(vo[0], vo[1], vo[2], vo[3]));
        st4nt(blk + 5120, make_uint4(vo[4], vo[5], vo[6], vo[7]));
    }
}

// a sub-tile that runs past the tensor's end: the lane's 8 elements one by one
template <int kOpt>
__device__ __forceinline__ void step_f_partial(const GTensor& T, int64_t e, int lane,
                                               const StepScalars& P) {
    for (int j = 0; j < 8; ++j) {
        const int64_t i = e + (j >> 2) * 256 + 4 * lane + (j & 3);
        if (i >= T.numel) continue;
        GLOBAL float* th = f32_at<kOpt>(T, i, 0);
        const float v = (kOpt == kAdamW) ? th[2 * kSubTile] : 0.0f;
        const Upd u = update<kOpt>(th[0], th[kSubTile], v, bf16_to_f32(T.grad[i]), P);
        th[0] = u.theta;
        th[kSubTile] = u.m;
        if (kOpt == kAdamW) th[2 * kSubTile] = u.v;
        T.theta[i] = (uint16_t)f32_to_bf16(u.theta);
    }
}

// kSplit: one wave per 512-element sub-tile (small launches), as in the
// compressed step.
template <int kOpt, bool kSplit>
__global__ __launch_bounds__(256) void step_fp32_kernel(const DevTensor* __restrict__ table,
                                                        const int64_t* __restrict__ tile_begin,
                                                        int32_t count, int64_t tile0,
                                                        int64_t ntiles, DevTensor one,
                                                        StepScalars P) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t wave = uniform((int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x / kWave));
    const int64_t nwaves = (int64_t)gridDim.x * kWavesPerBlock;
    if (kSplit) {
        const int64_t nitems = ntiles * kSubTiles;
        if (wave >= nitems) return;
        TileCursor cur;
        cur.start(table, tile_begin, count, one, ntiles, tile0 + wave / kSubTiles);
        for (int64_t item = wave; item < nitems; item += nwaves) {
            const int64_t tile = tile0 + item / kSubTiles;
            cur.seek(table, tile_begin, tile);
            const GTensor& T = cur.T;
            const int64_t e = (tile - cur.begin) * kTile + (item % kSubTiles) * kSubTile;
            if (e + kSubTile <= T.numel) {
                RawF R;
                load_raw_f<kOpt>(T, e, lane, R);
                step_f<kOpt>(T, e, lane, R, P);
            } else if (e < T.numel) {
                step_f_partial<kOpt>(T, e, lane, P);
            }
        }
        return;
    }
    if (wave >= ntiles) return;
    TileCursor cur;
    cur.start(table, tile_begin, count, one, ntiles, tile0 + wave);
    for (int64_t tile = tile0 + wave; tile < tile0 + ntiles; tile += nwaves) {
        cur.seek(table, tile_begin, tile);
        const GTensor& T = cur.T;
        const int64_t e0 = (tile - cur.begin) * kTile;
        if (e0 + kTile <= T.numel) {
            RawF R[2];
            load_raw_f<kOpt>(T, e0, lane, R[0]);
            if (kSubTiles > 1) load_raw_f<kOpt>(T, e0 + kSubTile, lane, R[1]);
#pragma unroll
            for (int k = 0; k < kSubTiles; ++k) {
                step_f<kOpt>(T, e0 + k * kSubTile, lane, R[k & 1], P);
                if (k + 2 < kSubTiles)
                    load_raw_f<kOpt>(T, e0 + (k + 2) * kSubTile, lane, R[k & 1]);
            }
        } else {
            for (int k = 0; k < kSubTiles; ++k) {
                const int64_t e = e0 + k * kSubTile;
                if (e + kSubTile <= T.numel) {
                    RawF R;
                    load_raw_f<kOpt>(T, e, lane, R);
                    step_f<kOpt>(T, e, lane, R, P);
                } else if (e < T.numel) {
                    step_f_partial<kOpt>(T, e, lane, P);
                }
            }
        }
    }
}

// _FP32 kinds: master weight = x, theta' = bf16_rne(x), m = v = 0.
template <int kOpt>
__global__ __launch_bounds__(256) void init_fp32_kernel(DevTensor d, const float* x) {
    const GTensor T = view(d);
    const int64_t n = T.numel;
    FLAT_LOOP(n) {
        const int64_t e = c * kSubTile + lane * kLaneElems;
        for (int j = 0; j < 8; ++j) {
            if (e + j >= n) break;
            GLOBAL float* th = f32_at<kOpt>(T, e + j, 0);
            const float v = x[e + j];
            th[0] = v;
            th[kSubTile] = 0.0f;
            if (kOpt == kAdamW) th[2 * kSubTile] = 0.0f;
            T.theta[e + j] = (uint16_t)f32_to_bf16(v);
        }
    }
}

template <int kOpt>
__global__ __launch_bounds__(256) void export_fp32_kernel(DevTensor d, float* theta_out,
                                                          float* m_out, float* v_out) {
    const GTensor T = view(d);
    const int64_t n = T.numel;
    FLAT_LOOP(n) {
        const int64_t e = c * kSubTile + lane * kLaneElems;
        for (int j = 0; j < 8; ++j) {
            if (e + j >= n) break;
            const GLOBAL float* th = f32_at<kOpt>(T, e + j, 0);
            if (theta_out) theta_out[e + j] = th[0];
            if (m_out) m_out[e + j] = th[kSubTile];
            if (kOpt == kAdamW && v_out) v_out[e + j] = th[2 * kSubTile];
        }
    }
}

// m = v = 0 over a list of _FP32 tensors (master weights kept), one tile per wave.
template <int kOpt>
__global__ __launch_bounds__(256) void zero_fp32_kernel(const DevTensor* __restrict__ table,
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
                if (e + j >= T.numel) break;
                GLOBAL float* th = f32_at<kOpt>(T, e + j, 0);
                th[kSubTile] = 0.0f;
                if (kOpt == kAdamW) th[2 * kSubTile] = 0.0f;
            }
        }
    }
}

template <int kOpt>
static int launch_fp32(const DevTensor* table, const int64_t* tile_begin, int32_t count,
                       int64_t tile0, int64_t ntiles, const DevTensor& one, const StepScalars& P,
                       hipStream_t st) {
    if (ntiles < kSplitTiles)
        hipLaunchKernelGGL((step_fp32_kernel<kOpt, true>), dim3(grid_for(ntiles * kSubTiles)),
                           dim3(kBlock), 0, st, table, tile_begin, count, tile0, ntiles, one, P);
    else
        hipLaunchKernelGGL((step_fp32_kernel<kOpt, false>), dim3(grid_for(ntiles)),
                           dim3(kBlock), 0, st, table, tile_begin, count, tile0, ntiles, one, P);
    return launch_status();
}

int launch_step_fp32(int opt, const DevTensor* table, const int64_t* tile_begin, int32_t count,
                     int64_t tile0, int64_t ntiles, const DevTensor& one, const StepScalars& P,
                     hipStream_t st) {
    if (opt == kAdamW)
        return launch_fp32<kAdamW>(table, tile_begin, count, tile0, ntiles, one, P, st);
    if (opt == kSgd)
        return launch_fp32<kSgd>(table, tile_begin, count, tile0, ntiles, one, P, st);
    return launch_fp32<kLion>(table, tile_begin, count, tile0, ntiles, one, P, st);
}

// SGD and Lion share the one-momentum block layout.
int launch_init_fp32(int opt, const DevTensor& d, const float* x, hipStream_t st) {
    const dim3 grid(grid_for((d.numel + kSubTile - 1) / kSubTile));
    if (opt == kAdamW)
        hipLaunchKernelGGL(init_fp32_kernel<kAdamW>, grid, dim3(kBlock), 0, st, d, x);
    else
        hipLaunchKernelGGL(init_fp32_kernel<kSgd>, grid, dim3(kBlock), 0, st, d, x);
    return launch_status();
}

int launch_export_fp32(int opt, const DevTensor& d, float* theta, float* m, float* v,
                       hipStream_t st) {
    const dim3 grid(grid_for((d.numel + kSubTile - 1) / kSubTile));
    if (opt == kAdamW)
        hipLaunchKernelGGL(export_fp32_kernel<kAdamW>, grid, dim3(kBlock), 0, st, d, theta, m, v);
    else
        hipLaunchKernelGGL(export_fp32_kernel<kSgd>, grid, dim3(kBlock), 0, st, d, theta, m, v);
    return launch_status();
}

int launch_zero_fp32(int opt, const DevTensor* table, const int64_t* tile_begin, int32_t count,
                     int64_t total_tiles, hipStream_t st) {
    const dim3 grid(grid_for(total_tiles));
    if (opt == kAdamW)
        hipLaunchKernelGGL(zero_fp32_kernel<kAdamW>, grid, dim3(kBlock), 0, st, table, tile_begin,
                           count, total_tiles);
    else
        hipLaunchKernelGGL(zero_fp32_kernel<kSgd>, grid, dim3(kBlock), 0, st, table, tile_begin,
                           count, total_tiles);
    return launch_status();
}

}  // namespace flashopt
