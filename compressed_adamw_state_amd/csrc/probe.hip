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

}  // extern "C"
