// Measurement aids (include/flashopt_probe.h): the fused step's own access
// pattern with the arithmetic taken out.
#include "host.hpp"
#include "flashopt_probe.h"

namespace flashopt {

// ---- bandwidth probe ---------------------------------------------------------
//
// The AdamW step's memory traffic with the arithmetic taken out: the same
// tiles, launch shape, loads (with the same two-buffer pipeline) and stores,
// and one XOR per word in place of the update (theta' ^= g, rho ^= q_m,
// q_m ^= q_v, q_v ^= rho, both scales ^= 1).  Its time is the practical floor
// of the step's access pattern on this device.
__device__ __forceinline__ uint2 xor2(const uint2 a, const uint2 b) {
    return make_uint2(a.x ^ b.x, a.y ^ b.y);
}

__device__ __forceinline__ void probe_sub(const TileAddr<kAdamW>& A, int k, int lane,
                                          const Raw& R) {
    GLOBAL uint8_t* rec = A.rc(k);
    st4(A.th(k), make_uint4(R.th.x ^ R.gr.x, R.th.y ^ R.gr.y, R.th.z ^ R.gr.z,
                            R.th.w ^ R.gr.w));
    st2(rec + kRhoOff, xor2(R.rho, R.qm));
    st2(rec + kMOff, xor2(R.qm, R.qv));
    st2(rec + kVOff, xor2(R.qv, R.rho));
    if ((lane & 3) == 0)
        *(GLOBAL uint32_t*)A.sc(k) = (R.ms | (R.vs << 16)) ^ 0x00010001u;
}

__global__ __launch_bounds__(256) void probe_kernel(const DevTensor* __restrict__ table,
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
        if (e0 + kTile <= T.numel) {
            const TileAddr<kAdamW> A(T, e0, lane);
            Raw R[2];
            load_raw<kAdamW>(A, 0, R[0]);
            if (kSubTiles > 1) load_raw<kAdamW>(A, 1, R[1]);
#pragma unroll
            for (int k = 0; k < kSubTiles; ++k) {
                probe_sub(A, k, lane, R[k & 1]);
                if (k + 2 < kSubTiles) load_raw<kAdamW>(A, k + 2, R[k & 1]);
            }
        } else {
            for (int k = 0; k < kSubTiles; ++k) {
                const int64_t e = e0 + k * kSubTile + lane * kLaneElems;
                for (int j = 0; j < 8; ++j) {
                    const int64_t i = e + j;
                    if (i < T.numel) {
                        GLOBAL uint8_t* r = code_at<kAdamW>(T, i, kRhoOff);
                        GLOBAL uint8_t* m = code_at<kAdamW>(T, i, kMOff);
                        GLOBAL uint8_t* v = code_at<kAdamW>(T, i, kVOff);
                        const uint8_t rho = *r, qm = *m, qv = *v;
                        T.theta[i] = (uint16_t)(T.theta[i] ^ T.grad[i]);
                        *r = (uint8_t)(rho ^ qm);
                        *m = (uint8_t)(qm ^ qv);
                        *v = (uint8_t)(qv ^ rho);
                    }
                }
                if ((lane & 3) == 0 && e < T.numel) {
                    GLOBAL uint32_t* w = (GLOBAL uint32_t*)(T.scales + 2 * (e >> 5));
                    *w = *w ^ 0x00010001u;
                }
            }
        }
    }
}

// ---- ceiling of the step's byte mix -------------------------------------------
//
// The same bytes per parameter as the AdamW step (read 7.125, write 5.125)
// over four streams read and three written, in place like the step -- theta'
// (2 bytes, read and written), the gradient (2, read), the codes (3, read and
// written) and the scales (0.125, read and written) -- but over flat buffers
// with every access a fully coalesced 16 bytes per lane: a wave takes one
// 2048-parameter tile, issues all of its loads (4 KB of theta', 4 KB of
// gradient, 6 KB of codes, 256 B of scales), then writes theta' ^ grad, the
// codes ^ 0x5A per byte and the scales ^ 1 per FP16.  It is the practical
// ceiling for the step's traffic with the best access pattern the byte mix
// allows, independent of the code-record layout.
constexpr int kMixTile = 2048;
constexpr int kMixThetaUnits = kMixTile * 2 / 16 / kWave;     // 16-byte units per lane: 4
constexpr int kMixCodeUnits = kMixTile * 3 / 16 / kWave;      // 6
constexpr int kMixScaleLanes = kMixTile / kGroup * 4 / 16;    // lanes holding scales: 16

__global__ __launch_bounds__(256) void mix_ceiling_kernel(GLOBAL uint8_t* theta,
                                                          const GLOBAL uint8_t* grad,
                                                          GLOBAL uint8_t* codes,
                                                          GLOBAL uint8_t* scales, int64_t ntiles) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t wave = uniform((int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x / kWave));
    const int64_t nwaves = (int64_t)gridDim.x * kWavesPerBlock;
    for (int64_t tile = wave; tile < ntiles; tile += nwaves) {
        GLOBAL uint8_t* th = theta + tile * (kMixTile * 2) + lane * 16;
        const GLOBAL uint8_t* gr = grad + tile * (kMixTile * 2) + lane * 16;
        GLOBAL uint8_t* cd = codes + tile * (kMixTile * 3) + lane * 16;
        GLOBAL uint8_t* sc = scales + tile * (kMixTile / kGroup * 4) + lane * 16;
        uint4 t[kMixThetaUnits], g[kMixThetaUnits], c[kMixCodeUnits], s = make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int u = 0; u < kMixThetaUnits; ++u) {
            t[u] = ld4(th + u * kWave * 16);
            g[u] = ld4(gr + u * kWave * 16);
        }
#pragma unroll
        for (int u = 0; u < kMixCodeUnits; ++u) c[u] = ld4(cd + u * kWave * 16);
        if (lane < kMixScaleLanes) s = ld4(sc);
#pragma unroll
        for (int u = 0; u < kMixThetaUnits; ++u)
            st4(th + u * kWave * 16, make_uint4(t[u].x ^ g[u].x, t[u].y ^ g[u].y, t[u].z ^ g[u].z,
                                                t[u].w ^ g[u].w));
#pragma unroll
        for (int u = 0; u < kMixCodeUnits; ++u)
            st4(cd + u * kWave * 16, make_uint4(c[u].x ^ 0x5A5A5A5Au, c[u].y ^ 0x5A5A5A5Au,
                                                c[u].z ^ 0x5A5A5A5Au, c[u].w ^ 0x5A5A5A5Au));
        if (lane < kMixScaleLanes)
            st4(sc, make_uint4(s.x ^ 0x00010001u, s.y ^ 0x00010001u, s.z ^ 0x00010001u,
                               s.w ^ 0x00010001u));
    }
}

// ---- stream-count sweep ---------------------------------------------------------
//
// R buffers read and W buffers written, all of the same size, one 16-byte
// unit of each per thread: the XOR of the R units read is written to every
// written buffer (XOR the buffer's index); with W = 0 the XOR stays in
// registers.  In place: the W written buffers are the first W of the R read.
struct SweepPtrs {
    const GLOBAL u32x4* r[8];
    GLOBAL u32x4* w[8];
};

template <int R, int W>
__global__ __launch_bounds__(256) void sweep_kernel(SweepPtrs p, int64_t units) {
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < units; i += stride) {
        uint4 acc = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const u32x4 v = p.r[r][i];
            acc = make_uint4(acc.x ^ v.x, acc.y ^ v.y, acc.z ^ v.z, acc.w ^ v.w);
        }
#pragma unroll
        for (int w = 0; w < W; ++w) {
            const u32x4 v = {acc.x ^ (uint32_t)w, acc.y, acc.z, acc.w};
            p.w[w][i] = v;
        }
        if (W == 0)      // keep the loads: the values are consumed, nothing is written
            asm volatile("" ::"v"(acc.x), "v"(acc.y), "v"(acc.z), "v"(acc.w));
    }
}

template <int R, int W>
static int launch_sweep(const SweepPtrs& p, int64_t units, hipStream_t st) {
    hipLaunchKernelGGL((sweep_kernel<R, W>), dim3(grid_for(units / kWave)), dim3(kBlock), 0, st,
                       p, units);
    return launch_status();
}

}  // namespace flashopt

using namespace flashopt;

extern "C" {

int flashopt_stream_probe(const flashopt_list* L, void* stream) {
    if (!L) return FLASHOPT_ERR_NULL;
    if (L->kind != FLASHOPT_KIND_ADAMW) return FLASHOPT_ERR_ARG;
    if (!L->all_have_grad) return FLASHOPT_ERR_NULL;
    if (L->total_tiles == 0) return FLASHOPT_OK;
    hipLaunchKernelGGL(probe_kernel, dim3(grid_for(L->total_tiles)), dim3(kBlock), 0,
                       (hipStream_t)stream, (const DevTensor*)L->d_table,
                       (const int64_t*)L->d_tile_begin, L->count, L->total_tiles);
    return launch_status();
}

int flashopt_mix_ceiling(uint16_t* theta, const uint16_t* grad, uint8_t* codes, uint16_t* scales,
                         int64_t n, void* stream) {
    if (n < 0 || n > kMaxNumel || n % kMixTile != 0) return FLASHOPT_ERR_SIZE;
    if (n == 0) return FLASHOPT_OK;
    if (!theta || !grad || !codes || !scales) return FLASHOPT_ERR_NULL;
    if (!aligned(theta, 16) || !aligned(grad, 16) || !aligned(codes, 16) || !aligned(scales, 16))
        return FLASHOPT_ERR_ALIGN;
    const int64_t ntiles = n / kMixTile;
    hipLaunchKernelGGL(mix_ceiling_kernel, dim3(grid_for(ntiles)), dim3(kBlock), 0,
                       (hipStream_t)stream, (GLOBAL uint8_t*)theta, (const GLOBAL uint8_t*)grad,
                       (GLOBAL uint8_t*)codes, (GLOBAL uint8_t*)scales, ntiles);
    return launch_status();
}

int flashopt_stream_sweep(int32_t nread, int32_t nwrite, const void* const* reads,
                          void* const* writes, int32_t in_place, int64_t bytes, void* stream) {
    if (bytes < 0 || bytes > kMaxNumel || bytes % 16 != 0) return FLASHOPT_ERR_SIZE;
    if (nread < 0 || nwrite < 0 || nread > 8 || nwrite > 8 || (in_place && nwrite > nread))
        return FLASHOPT_ERR_ARG;
    if ((nread > 0 && !reads) || (nwrite > 0 && !in_place && !writes)) return FLASHOPT_ERR_NULL;
    SweepPtrs p{};
    for (int32_t r = 0; r < nread; ++r) {
        if (!reads[r]) return FLASHOPT_ERR_NULL;
        if (!aligned(reads[r], 16)) return FLASHOPT_ERR_ALIGN;
        p.r[r] = (const GLOBAL u32x4*)reads[r];
    }
    for (int32_t w = 0; w < nwrite; ++w) {
        void* q = in_place ? const_cast<void*>(reads[w]) : writes[w];
        if (!q) return FLASHOPT_ERR_NULL;
        if (!aligned(q, 16)) return FLASHOPT_ERR_ALIGN;
        p.w[w] = (GLOBAL u32x4*)q;
    }
    const int64_t units = bytes / 16;
    if (units == 0) return FLASHOPT_OK;
    hipStream_t st = (hipStream_t)stream;
#define FLASHOPT_SWEEP(R, W) \
    if (nread == R && nwrite == W) return launch_sweep<R, W>(p, units, st);
    FLASHOPT_SWEEP(1, 0) FLASHOPT_SWEEP(0, 1) FLASHOPT_SWEEP(1, 1) FLASHOPT_SWEEP(2, 1)
    FLASHOPT_SWEEP(1, 2) FLASHOPT_SWEEP(3, 2) FLASHOPT_SWEEP(4, 3) FLASHOPT_SWEEP(7, 5)
    FLASHOPT_SWEEP(2, 2) FLASHOPT_SWEEP(4, 0) FLASHOPT_SWEEP(0, 4)
#undef FLASHOPT_SWEEP
    return FLASHOPT_ERR_ARG;
}

}  // extern "C"
