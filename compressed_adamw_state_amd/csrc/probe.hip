// Measurement aids (include/flashopt_probe.h): the fused step's own access
// pattern with the arithmetic taken out.
#include "host.hpp"
#include "flashopt_probe.h"

namespace flashopt {

#define LDS __attribute__((address_space(3)))

// ---- bandwidth probe ---------------------------------------------------------
//
// A step's memory traffic with the arithmetic taken out: the same tiles,
// launch shape, loads (with the same two-buffer pipeline) and stores, and one
// XOR per word in place of the update.  AdamW: theta' ^= g, rho ^= q_m,
// q_m ^= q_v, q_v ^= rho, both scales ^= 1; SGD and Lion: theta' ^= g,
// rho ^= q_m, q_m = ~q_m, the scale ^= 1.  Its time is the practical floor of
// the step's access pattern on this device.
__device__ __forceinline__ uint2 xor2(const uint2 a, const uint2 b) {
    return make_uint2(a.x ^ b.x, a.y ^ b.y);
}

template <int kOpt>
__device__ __forceinline__ void probe_sub(const TileAddr<kOpt>& A, int k, int lane,
                                          const Raw& R) {
    GLOBAL uint8_t* rec = A.rc(k);
    st4nt(A.th(k), make_uint4(R.th.x ^ R.gr.x, R.th.y ^ R.gr.y, R.th.z ^ R.gr.z,
                              R.th.w ^ R.gr.w));
    const uint2 rho = xor2(R.rho, R.qm);
    if (kOpt == kAdamW) {
        st2nt(rec, rho);
        st2nt(rec + Layout<kOpt>::kField, xor2(R.qm, R.qv));
        st2nt(rec + 2 * Layout<kOpt>::kField, xor2(R.qv, R.rho));
        if ((lane & 3) == 0)
            *(GLOBAL uint32_t*)A.sc(k) = (R.ms | (R.vs << 16)) ^ 0x00010001u;
    } else {
        st4nt(rec, make_uint4(rho.x, rho.y, ~R.qm.x, ~R.qm.y));
        if ((lane & 3) == 0) *(GLOBAL uint16_t*)A.sc(k) = (uint16_t)(R.ms ^ 1u);
    }
}

template <int kOpt>
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
            const TileAddr<kOpt> A(T, e0);
            Raw R[2];
            load_raw<kOpt>(A, 0, R[0]);
            if (kSubTiles > 1) load_raw<kOpt>(A, 1, R[1]);
#pragma unroll
            for (int k = 0; k < kSubTiles; ++k) {
                probe_sub<kOpt>(A, k, lane, R[k & 1]);
                if (k + 2 < kSubTiles) load_raw<kOpt>(A, k + 2, R[k & 1]);
            }
        } else {
            for (int k = 0; k < kSubTiles; ++k) {
                const int64_t e = e0 + k * kSubTile + lane * kLaneElems;
                for (int j = 0; j < 8; ++j) {
                    const int64_t i = e + j;
                    if (i < T.numel) {
                        GLOBAL uint8_t* r = code_at<kOpt>(T, i, kRho);
                        GLOBAL uint8_t* m = code_at<kOpt>(T, i, kM);
                        const uint8_t rho = *r, qm = *m;
                        T.theta[i] = (uint16_t)(T.theta[i] ^ T.grad[i]);
                        *r = (uint8_t)(rho ^ qm);
                        if (kOpt == kAdamW) {
                            GLOBAL uint8_t* v = code_at<kOpt>(T, i, kV);
                            const uint8_t qv = *v;
                            *m = (uint8_t)(qm ^ qv);
                            *v = (uint8_t)(qv ^ rho);
                        } else {
                            *m = (uint8_t)~qm;
                        }
                    }
                }
                if ((lane & 3) == 0 && e < T.numel) {
                    if (kOpt == kAdamW) {
                        GLOBAL uint32_t* w = (GLOBAL uint32_t*)(T.scales + 2 * (e >> 5));
                        *w = *w ^ 0x00010001u;
                    } else {
                        T.scales[e >> 5] = (uint16_t)(T.scales[e >> 5] ^ 1u);
                    }
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
// with every access a fully coalesced 16 bytes per lane, all with the
// non-temporal hint (on this byte mix 4 % faster than without): a wave takes one
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
            t[u] = ld4nt(th + u * kWave * 16);
            g[u] = ld4nt(gr + u * kWave * 16);
        }
#pragma unroll
        for (int u = 0; u < kMixCodeUnits; ++u) c[u] = ld4nt(cd + u * kWave * 16);
        if (lane < kMixScaleLanes) s = ld4nt(sc);
#pragma unroll
        for (int u = 0; u < kMixThetaUnits; ++u)
            st4nt(th + u * kWave * 16, make_uint4(t[u].x ^ g[u].x, t[u].y ^ g[u].y,
                                                  t[u].z ^ g[u].z, t[u].w ^ g[u].w));
#pragma unroll
        for (int u = 0; u < kMixCodeUnits; ++u)
            st4nt(cd + u * kWave * 16, make_uint4(c[u].x ^ 0x5A5A5A5Au, c[u].y ^ 0x5A5A5A5Au,
                                                  c[u].z ^ 0x5A5A5A5Au, c[u].w ^ 0x5A5A5A5Au));
        if (lane < kMixScaleLanes)
            st4nt(sc, make_uint4(s.x ^ 0x00010001u, s.y ^ 0x00010001u, s.z ^ 0x00010001u,
                                 s.w ^ 0x00010001u));
    }
}

// ---- access-pattern variants over the same flat buffers --------------------------
//
// The step's traffic (same bytes, streams and 2048-parameter tiles as the
// ceiling above) with the access patterns the fused kernel could use, to
// isolate the pattern from the byte mix.  Per tile, four 512-parameter
// sub-tiles; lane l owns parameters [8l, 8l+8) of a sub-tile.
//   0: the fused kernel's own pattern: theta' and the gradient 16 bytes per
//      lane, the codes of the lane's 8 parameters as three 8-byte runs, one
//      in each 512-byte plane of the sub-tile's 1536 code bytes, a quad
//      leader's 4-byte scale pair; every theta', gradient and code access
//      hinted non-temporal; sub-tile k+2 loaded once sub-tile k is stored
//      (two register buffers).
//   1: as 0, but the 1536 code bytes of a sub-tile as 16-byte units (lane l
//      unit l, lanes 0-31 also unit 64 + l) and the 64 scale bytes as 16
//      lanes x 4 bytes, the codes not hinted.
//   2: the units of 1, loaded by global-to-LDS DMA (global_load_lds_dwordx4)
//      into a two-slot ring per wave and read back from LDS: no VGPR holds a
//      load in flight.
//   3: as 0 with three register buffers: the loads of sub-tile k+2 are issued
//      before sub-tile k is stored.
//   4: as 0 with the tiles in a hashed order: wave w takes tile
//      (w * mult) mod ntiles (mult a prime not dividing ntiles, so every tile
//      once), so the tiles in flight at any moment are spread over the whole
//      buffers instead of one window: separates an effect of which addresses
//      are accessed together from one of where the buffers lie.
//   5: as 0, but the lane's codes as one interleaved 24-byte record (lane l
//      at bytes [24l, 24l+24) of the sub-tile's 1536), three 8-byte accesses
//      without the hint: the layout the fused kernel used before the planes.
// Results: theta' ^= grad in every variant; codes: variants 0, 3, 4 and 5
// replace each lane's three 8-byte code words (a, b, c) with (a^b, b^c,
// c^a), variants 1 and 2 XOR every code byte with 0x5A; every scale word
// (the pair of a 32-parameter group) ^= 0x00010001.
struct PatternPtrs {
    GLOBAL uint8_t* th;
    const GLOBAL uint8_t* gr;
    GLOBAL uint8_t* rec;
    GLOBAL uint8_t* sc;
    int64_t ntiles;
    int64_t mult;       // variant 4's tile order; 0: tile = wave
};

struct PRec { u32x4 th, gr; u32x2 a, b, c; uint32_t s; };

// the lane's three 8-byte code words of sub-tile k: plane runs (kPlanes) or
// one interleaved record
template <bool kPlanes>
__device__ __forceinline__ GLOBAL uint8_t* prec_codes(const PatternPtrs& p, int64_t w, int k,
                                                      int lane) {
    return p.rec + w * 6144 + k * 1536 + lane * (kPlanes ? 8 : 24);
}
template <bool kPlanes> constexpr int kPrecWord = kPlanes ? 512 : 8;    // bytes between words

template <bool kPlanes>
__device__ __forceinline__ void prec_load(const PatternPtrs& p, int64_t w, int k, int lane,
                                          PRec& r) {
    r.th = __builtin_nontemporal_load((const GLOBAL u32x4*)(p.th + w * 4096 + k * 1024 + lane * 16));
    r.gr = __builtin_nontemporal_load((const GLOBAL u32x4*)(p.gr + w * 4096 + k * 1024 + lane * 16));
    const GLOBAL uint8_t* c = prec_codes<kPlanes>(p, w, k, lane);
    constexpr int d = kPrecWord<kPlanes>;
    if (kPlanes) {
        r.a = __builtin_nontemporal_load((const GLOBAL u32x2*)c);
        r.b = __builtin_nontemporal_load((const GLOBAL u32x2*)(c + d));
        r.c = __builtin_nontemporal_load((const GLOBAL u32x2*)(c + 2 * d));
    } else {
        r.a = *(const GLOBAL u32x2*)c;
        r.b = *(const GLOBAL u32x2*)(c + d);
        r.c = *(const GLOBAL u32x2*)(c + 2 * d);
    }
    r.s = *(const GLOBAL uint32_t*)(p.sc + w * 256 + k * 64 + (lane >> 2) * 4);
}

template <bool kPlanes>
__device__ __forceinline__ void prec_store(const PatternPtrs& p, int64_t w, int k, int lane,
                                           const PRec& r) {
    __builtin_nontemporal_store(r.th ^ r.gr, (GLOBAL u32x4*)(p.th + w * 4096 + k * 1024 + lane * 16));
    GLOBAL uint8_t* c = prec_codes<kPlanes>(p, w, k, lane);
    constexpr int d = kPrecWord<kPlanes>;
    if (kPlanes) {
        __builtin_nontemporal_store(r.a ^ r.b, (GLOBAL u32x2*)c);
        __builtin_nontemporal_store(r.b ^ r.c, (GLOBAL u32x2*)(c + d));
        __builtin_nontemporal_store(r.c ^ r.a, (GLOBAL u32x2*)(c + 2 * d));
    } else {
        *(GLOBAL u32x2*)c = r.a ^ r.b;
        *(GLOBAL u32x2*)(c + d) = r.b ^ r.c;
        *(GLOBAL u32x2*)(c + 2 * d) = r.c ^ r.a;
    }
    if ((lane & 3) == 0)
        *(GLOBAL uint32_t*)(p.sc + w * 256 + k * 64 + (lane >> 2) * 4) = r.s ^ 0x00010001u;
}

template <int kBuffers, bool kPlanes>
__global__ __launch_bounds__(256) void pattern_records_kernel(PatternPtrs p) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t wave = uniform((int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x / kWave));
    if (wave >= p.ntiles) return;
    const int64_t w = p.mult ? wave * p.mult % p.ntiles : wave;
    PRec r[kBuffers];
    prec_load<kPlanes>(p, w, 0, lane, r[0]);
    prec_load<kPlanes>(p, w, 1, lane, r[1]);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        if (kBuffers == 3 && k + 2 < 4) prec_load<kPlanes>(p, w, k + 2, lane, r[(k + 2) % kBuffers]);
        prec_store<kPlanes>(p, w, k, lane, r[k % kBuffers]);
        if (kBuffers == 2 && k + 2 < 4) prec_load<kPlanes>(p, w, k + 2, lane, r[k % kBuffers]);
    }
}

struct PUnits { u32x4 th, gr, c0, c1; uint32_t s; };

__global__ __launch_bounds__(256) void pattern_units_kernel(PatternPtrs p) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t w = uniform((int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x / kWave));
    if (w >= p.ntiles) return;
    GLOBAL uint8_t* th = p.th + w * 4096;
    const GLOBAL uint8_t* gr = p.gr + w * 4096;
    GLOBAL uint8_t* rec = p.rec + w * 6144;
    GLOBAL uint8_t* sc = p.sc + w * 256;
    auto ld = [&](int k, PUnits& r) {
        r.th = __builtin_nontemporal_load((const GLOBAL u32x4*)(th + k * 1024 + lane * 16));
        r.gr = __builtin_nontemporal_load((const GLOBAL u32x4*)(gr + k * 1024 + lane * 16));
        r.c0 = *(const GLOBAL u32x4*)(rec + k * 1536 + lane * 16);
        if (lane < 32) r.c1 = *(const GLOBAL u32x4*)(rec + k * 1536 + 1024 + lane * 16);
        if (lane < 16) r.s = *(const GLOBAL uint32_t*)(sc + k * 64 + lane * 4);
    };
    auto st = [&](int k, const PUnits& r) {
        __builtin_nontemporal_store(r.th ^ r.gr, (GLOBAL u32x4*)(th + k * 1024 + lane * 16));
        *(GLOBAL u32x4*)(rec + k * 1536 + lane * 16) = r.c0 ^ 0x5A5A5A5Au;
        if (lane < 32) *(GLOBAL u32x4*)(rec + k * 1536 + 1024 + lane * 16) = r.c1 ^ 0x5A5A5A5Au;
        if (lane < 16) *(GLOBAL uint32_t*)(sc + k * 64 + lane * 4) = r.s ^ 0x00010001u;
    };
    PUnits r[2];
    ld(0, r[0]);
    ld(1, r[1]);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        st(k, r[k & 1]);
        if (k + 2 < 4) ld(k + 2, r[k & 1]);
    }
}

// Variant 2.  Per wave a ring of two LDS slots of 3648 bytes (theta' 1024,
// gradient 1024, codes 1536, scales 64); one batch of DMA loads is five
// instructions (theta', gradient, codes in two, scales), the stores of a
// sub-tile four.  The vmcnt waits below count the memory instructions
// issued after the batch being consumed (vmcnt counts loads and stores of a
// wave in issue order on this architecture).
constexpr int kSlot = 3648;
#define FLASHOPT_VMCNT(N) \
    __builtin_amdgcn_s_waitcnt(((N) & 0xF) | (0x7 << 4) | (0xF << 8) | (((N) >> 4) << 14))
#define FLASHOPT_LGKMCNT0() __builtin_amdgcn_s_waitcnt(0xC07F)

__device__ __forceinline__ void dma16(const GLOBAL uint8_t* src, LDS uint8_t* dst) {
    __builtin_amdgcn_global_load_lds((const GLOBAL uint32_t*)src, (LDS uint32_t*)dst, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const GLOBAL uint8_t* src, LDS uint8_t* dst) {
    __builtin_amdgcn_global_load_lds((const GLOBAL uint32_t*)src, (LDS uint32_t*)dst, 4, 0, 0);
}

__global__ __launch_bounds__(256) void pattern_dma_kernel(PatternPtrs p) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[kWavesPerBlock * 2 * kSlot];
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t w = uniform((int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x / kWave));
    if (w >= p.ntiles) return;
    GLOBAL uint8_t* th = p.th + w * 4096;
    const GLOBAL uint8_t* gr = p.gr + w * 4096;
    GLOBAL uint8_t* rec = p.rec + w * 6144;
    GLOBAL uint8_t* sc = p.sc + w * 256;
    LDS uint8_t* base = (LDS uint8_t*)lds + (threadIdx.x / kWave) * 2 * kSlot;
    auto issue = [&](int k) {
        LDS uint8_t* s = base + (k & 1) * kSlot;
        dma16(th + k * 1024 + lane * 16, s);
        dma16(gr + k * 1024 + lane * 16, s + 1024);
        dma16(rec + k * 1536 + lane * 16, s + 2048);
        if (lane < 32) dma16(rec + k * 1536 + 1024 + lane * 16, s + 3072);
        if (lane < 16) dma4(sc + k * 64 + lane * 4, s + 3584);
    };
    auto consume = [&](int k) {
        LDS uint8_t* s = base + (k & 1) * kSlot;
        const u32x4 t = *(LDS u32x4*)(s + lane * 16);
        const u32x4 g = *(LDS u32x4*)(s + 1024 + lane * 16);
        const u32x4 c0 = *(LDS u32x4*)(s + 2048 + lane * 16);
        u32x4 c1 = {0u, 0u, 0u, 0u};
        uint32_t sv = 0u;
        if (lane < 32) c1 = *(LDS u32x4*)(s + 3072 + lane * 16);
        if (lane < 16) sv = *(LDS uint32_t*)(s + 3584 + lane * 4);
        FLASHOPT_LGKMCNT0();              // the slot's data is in registers: it may be refilled
        return [=]() {
            *(GLOBAL u32x4*)(th + k * 1024 + lane * 16) = t ^ g;
            *(GLOBAL u32x4*)(rec + k * 1536 + lane * 16) = c0 ^ 0x5A5A5A5Au;
            if (lane < 32) *(GLOBAL u32x4*)(rec + k * 1536 + 1024 + lane * 16) = c1 ^ 0x5A5A5A5Au;
            if (lane < 16) *(GLOBAL uint32_t*)(sc + k * 64 + lane * 4) = sv ^ 0x00010001u;
        };
    };
    issue(0);
    issue(1);
    FLASHOPT_VMCNT(5);                    // batch 0 landed (batch 1 may be in flight)
    auto s0 = consume(0);
    issue(2);
    s0();
    FLASHOPT_VMCNT(5 + 4);                // batch 1 (then batch 2, stores 0)
    auto s1 = consume(1);
    issue(3);
    s1();
    FLASHOPT_VMCNT(4 + 5 + 4);            // batch 2 (then stores 0, batch 3, stores 1)
    auto s2 = consume(2);
    s2();
    FLASHOPT_VMCNT(4 + 4);                // batch 3 (then stores 1, stores 2)
    auto s3 = consume(3);
    s3();
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
    if (is_fp32(L->kind)) return FLASHOPT_ERR_ARG;
    if (!L->all_have_grad) return FLASHOPT_ERR_NULL;
    if (L->total_tiles == 0) return FLASHOPT_OK;
    const dim3 grid(grid_for(L->total_tiles)), block(kBlock);
    const hipStream_t s = (hipStream_t)stream;
    const DevTensor* table = (const DevTensor*)L->d_table;
    const int64_t* begin = (const int64_t*)L->d_tile_begin;
    switch (opt_of(L->kind)) {
    case kAdamW:
        hipLaunchKernelGGL(probe_kernel<kAdamW>, grid, block, 0, s, table, begin, L->count,
                           L->total_tiles);
        break;
    case kSgd:
        hipLaunchKernelGGL(probe_kernel<kSgd>, grid, block, 0, s, table, begin, L->count,
                           L->total_tiles);
        break;
    default:
        hipLaunchKernelGGL(probe_kernel<kLion>, grid, block, 0, s, table, begin, L->count,
                           L->total_tiles);
        break;
    }
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

int flashopt_pattern_probe(int32_t variant, uint16_t* theta, const uint16_t* grad,
                           uint8_t* codes, uint16_t* scales, int64_t n, void* stream) {
    if (variant < 0 || variant > 5) return FLASHOPT_ERR_ARG;
    if (n < 0 || n > kMaxNumel || n % kMixTile != 0) return FLASHOPT_ERR_SIZE;
    if (n == 0) return FLASHOPT_OK;
    if (!theta || !grad || !codes || !scales) return FLASHOPT_ERR_NULL;
    if (!aligned(theta, 16) || !aligned(grad, 16) || !aligned(codes, 16) || !aligned(scales, 16))
        return FLASHOPT_ERR_ALIGN;
    PatternPtrs p{(GLOBAL uint8_t*)theta, (const GLOBAL uint8_t*)grad, (GLOBAL uint8_t*)codes,
                  (GLOBAL uint8_t*)scales, n / kMixTile, 0};
    if (variant == 4) {
        // the first of these primes that does not divide ntiles (ntiles <= 2^25
        // with one wave per tile, so at most one of them divides it, and
        // wave * mult stays far below 2^63)
        static const int64_t kPrimes[] = {1000003, 1000033, 1000037, 1000039};
        for (int64_t q : kPrimes)
            if (p.ntiles % q != 0) { p.mult = q; break; }
    }
    const dim3 grid(grid_for(p.ntiles)), block(kBlock);
    if (p.ntiles > kMaxBlocks * kWavesPerBlock) return FLASHOPT_ERR_SIZE;   // one wave per tile
    hipStream_t s = (hipStream_t)stream;
    if (variant == 0 || variant == 4)
        hipLaunchKernelGGL((pattern_records_kernel<2, true>), grid, block, 0, s, p);
    else if (variant == 1) hipLaunchKernelGGL(pattern_units_kernel, grid, block, 0, s, p);
    else if (variant == 2) hipLaunchKernelGGL(pattern_dma_kernel, grid, block, 0, s, p);
    else if (variant == 3) hipLaunchKernelGGL((pattern_records_kernel<3, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((pattern_records_kernel<2, false>), grid, block, 0, s, p);
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
