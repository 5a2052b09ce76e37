// Device-side building blocks shared by the kernels of libflashopt.so.
//
// Method: "FlashOptim: Optimizers for Memory Efficient Training" (digest
// page), section "Core method": the state layout of the compressed optimizer
// (weight splitting, Eq. 1-2; companded group quantisation, Alg. 2-3) and the
// per-element update of the fused step (Alg. 4).  This header holds the state
// descriptors, the tile walk over a ragged tensor list, the vector loads and
// stores, and the optimizer update on FP32 values; the kernels live in the
// .hip files beside it.
#pragma once

#include <hip/hip_runtime.h>

#include "codec.hpp"

namespace flashopt {

#define GLOBAL __attribute__((address_space(1)))

enum Opt { kAdamW = 0, kSgd = 1, kLion = 2 };

// Every tiled kernel runs blocks of kBlock threads (the launch bounds below and
// every launch say so); kernels use the constant, not blockDim.
constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / kWave;

// State layout of one tensor (see include/flashopt.h).  Codes, per
// 512-element block: AdamW keeps three 512-byte planes, rho, m_code and
// v_code, each in element order; SGD and Lion keep 64 16-byte records, one
// per 8-element run, rho[8] then m_code[8].  Either way a lane's codes in a
// full sub-tile are whole accesses that, with the other lanes', cover whole
// lines.  Scales: per 32-element group the FP16 m scale followed, for AdamW,
// by the v scale.
enum Field { kRho = 0, kM = 1, kV = 2 };
template <int kOpt> struct Layout {
    static constexpr int kLaneCode = kOpt == kAdamW ? 8 : 16;    // bytes between 8-element runs
    static constexpr int kField = kOpt == kAdamW ? 512 : 8;      // bytes between fields
    static constexpr int kBlockBytes = kOpt == kAdamW ? 1536 : 1024;   // per 512 elements
    static constexpr int kScl = kOpt == kAdamW ? 2 : 1;           // FP16 scales per group
};

// Device descriptor of one tensor as it sits in the table and in kernel
// arguments: plain 64-bit addresses (64 bytes per tensor).
struct DevTensor {
    uint64_t theta, codes, scales, grad;
    int64_t numel;
    uint64_t reserved[3];
};
static_assert(sizeof(DevTensor) == 64, "descriptor layout");

// The same descriptor as global-address-space pointers: with these every
// element access compiles to global_load / global_store (not flat), so the
// waits only count vector memory traffic.
struct GTensor {
    GLOBAL uint16_t* theta;
    GLOBAL uint8_t* codes;
    GLOBAL uint16_t* scales;
    const GLOBAL uint16_t* grad;
    int64_t numel;
};

__device__ __forceinline__ GTensor view(const DevTensor& d) {
    GTensor t;
    t.theta = (GLOBAL uint16_t*)d.theta;
    t.codes = (GLOBAL uint8_t*)d.codes;
    t.scales = (GLOBAL uint16_t*)d.scales;
    t.grad = (const GLOBAL uint16_t*)d.grad;
    t.numel = d.numel;
    return t;
}

// byte address of field f of element i's code
template <int kOpt>
__device__ __forceinline__ GLOBAL uint8_t* code_at(const GTensor& T, int64_t i, int f) {
    return T.codes + (i >> 9) * Layout<kOpt>::kBlockBytes +
           ((i & 511) >> 3) * Layout<kOpt>::kLaneCode + f * Layout<kOpt>::kField + (i & 7);
}


typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// 16- and 8-byte global accesses (clang vectors: no HIP vector-type
// constructors, which do not take address-space-qualified references)
__device__ __forceinline__ uint4 ld4(const GLOBAL void* p) {
    const u32x4 v = *(const GLOBAL u32x4*)p;
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ld2(const GLOBAL void* p) {
    const u32x2 v = *(const GLOBAL u32x2*)p;
    return make_uint2(v.x, v.y);
}
__device__ __forceinline__ void st4(GLOBAL void* p, uint4 v) {
    const u32x4 w = {v.x, v.y, v.z, v.w};
    *(GLOBAL u32x4*)p = w;
}
__device__ __forceinline__ void st2(GLOBAL void* p, uint2 v) {
    const u32x2 w = {v.x, v.y};
    *(GLOBAL u32x2*)p = w;
}
// The same accesses with the non-temporal hint (the `nt` bit), for the
// streams a step touches once, each access covering whole lines with the
// other lanes': theta' (read and written), the gradient (read) and the code
// planes or records.  Measured on the Llama-3.1-8B step against plain
// accesses in the same process: 1.5-2.2 % faster on theta' and the gradient
// whatever the placement of the state, 2.6-3.3 % on Lion's records.  Where a
// lane's access covers only part of each line (AdamW's earlier interleaved
// 24-byte records, two accesses over the same lines) the hint made the step
// slower.
__device__ __forceinline__ uint4 ld4nt(const GLOBAL void* p) {
    const u32x4 v = __builtin_nontemporal_load((const GLOBAL u32x4*)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st4nt(GLOBAL void* p, uint4 v) {
    const u32x4 w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, (GLOBAL u32x4*)p);
}
__device__ __forceinline__ uint2 ld2nt(const GLOBAL void* p) {
    const u32x2 v = __builtin_nontemporal_load((const GLOBAL u32x2*)p);
    return make_uint2(v.x, v.y);
}
__device__ __forceinline__ void st2nt(GLOBAL void* p, uint2 v) {
    const u32x2 w = {v.x, v.y};
    __builtin_nontemporal_store(w, (GLOBAL u32x2*)p);
}

__device__ __forceinline__ int64_t uniform(int64_t x) {
    uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)x);
    uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Largest i in [0, count) with tile_begin[i] <= tile (skips empty tensors).
__device__ __forceinline__ int32_t find_tensor(const int64_t* __restrict__ tile_begin,
                                               int32_t count, int64_t tile) {
    int32_t lo = 0, hi = count - 1;
    while (lo < hi) {
        int32_t mid = (lo + hi + 1) >> 1;
        if (tile_begin[mid] <= tile) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Walks a wave's increasing tile indices through the tensor list: one binary
// search for the first tile, then a forward scan (scalar loads of the small
// tile_begin table; a wave's next tile is at most a few tensors further).
// Pins a descriptor read from the (wave-uniform) table in scalar registers
// and keeps the compiler from merging that read with the read of a by-value
// kernel argument into one load through a generic pointer (a flat load into
// vector registers, which then carried every tile address as 64-bit vector
// arithmetic).
__device__ __forceinline__ void scalar_fence(GTensor& T) {
    asm volatile("" : "+s"(T.theta), "+s"(T.codes), "+s"(T.scales), "+s"(T.grad), "+s"(T.numel));
}

struct TileCursor {
    int32_t i;
    int64_t begin, end;
    GTensor T;

    __device__ __forceinline__ void start(const DevTensor* __restrict__ table,
                                          const int64_t* __restrict__ tile_begin, int32_t count,
                                          const DevTensor& one, int64_t total, int64_t tile) {
        if (table != nullptr) {
            i = find_tensor(tile_begin, count, tile);
            begin = tile_begin[i];
            end = tile_begin[i + 1];
            T = view(table[i]);
            scalar_fence(T);
        } else {
            i = 0;
            begin = 0;
            end = total;
            T = view(one);
        }
    }

    // tile < total; for the single-tensor form end == total, so no advance
    __device__ __forceinline__ void seek(const DevTensor* __restrict__ table,
                                         const int64_t* __restrict__ tile_begin, int64_t tile) {
        if (tile >= end) {
            do {
                ++i;
                begin = end;
                end = tile_begin[i + 1];
            } while (tile >= end);
            T = view(table[i]);
        }
    }
};

// ---- per-lane element staging ------------------------------------------------

struct Lane8 {                      // one lane's 8 elements of one sub-tile
    uint32_t th[8];                 // BF16 theta' bits
    uint32_t gr[8];                 // BF16 grad bits
    int32_t rho[8];
    int32_t qm[8];
    uint32_t qv[8];
    uint32_t ms, vs;                // the group's FP16 scales
};

__device__ __forceinline__ void unpack_bf16x8(const uint4 v, uint32_t* o) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) { o[2 * i] = w[i] & 0xFFFFu; o[2 * i + 1] = w[i] >> 16; }
}

__device__ __forceinline__ void unpack_s8x8(const uint2 v, int32_t* o) {
    const uint32_t w[2] = {v.x, v.y};
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = (int32_t)(int8_t)(uint8_t)(w[i >> 2] >> (8 * (i & 3)));
}

__device__ __forceinline__ void unpack_u8x8(const uint2 v, uint32_t* o) {
    const uint32_t w[2] = {v.x, v.y};
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = (w[i >> 2] >> (8 * (i & 3))) & 0xFFu;
}

__device__ __forceinline__ uint4 pack_u16x8(const uint32_t* v) {
    return make_uint4(v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16),
                      v[6] | (v[7] << 16));
}

__device__ __forceinline__ uint2 pack_u8x8(const uint32_t* v) {
    return make_uint2((v[0] & 0xFF) | ((v[1] & 0xFF) << 8) | ((v[2] & 0xFF) << 16) | (v[3] << 24),
                      (v[4] & 0xFF) | ((v[5] & 0xFF) << 8) | ((v[6] & 0xFF) << 16) | (v[7] << 24));
}

// One lane's 8 elements of a partial sub-tile, loaded element by element
// with bounds checks (the last tile of a tensor).
template <int kOpt>
__device__ __forceinline__ void load_lane(const GTensor& T, int64_t e, Lane8& L) {
    const int64_t n = T.numel;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const bool ok = e + j < n;
        L.th[j] = ok ? T.theta[e + j] : 0u;
        L.gr[j] = ok ? T.grad[e + j] : 0u;
        L.rho[j] = ok ? (int8_t)*code_at<kOpt>(T, e + j, kRho) : 0;
        L.qm[j] = ok ? (int8_t)*code_at<kOpt>(T, e + j, kM) : 0;
        if (kOpt == kAdamW) L.qv[j] = ok ? *code_at<kOpt>(T, e + j, kV) : 0u;
    }
    const int64_t g = e >> 5;
    const bool gok = (e & ~int64_t(31)) < n;           // the lane's group has valid elements
    L.ms = gok ? T.scales[g * Layout<kOpt>::kScl] : 0u;
    if (kOpt == kAdamW) L.vs = gok ? T.scales[g * Layout<kOpt>::kScl + 1] : 0u;
}

// ---- the update of one element ---------------------------------------------
//
// The optimizer arithmetic on FP32 values, one IEEE binary32 operation per
// line with the division and square root correctly rounded: the compressed
// step's general path applies it to the rebuilt weight and dequantised
// moments, the uncompressed (_FP32) step to the stored FP32 values.
struct Upd {
    float theta, m, v, root;        // new weight, momentum, variance, sqrt(variance)
};

template <int kOpt>
__device__ __forceinline__ Upd update(float theta_hat, float m, float v, float g,
                                      const StepScalars& P) {
    Upd r;
    r.v = 0.0f;
    r.root = 0.0f;
    if (kOpt == kAdamW) {
        const AdamScalars& a = P.a;
        const float bm = a.b1 * m;
        const float cg = a.c1 * g;
        r.m = bm + cg;
        const float bv = a.b2 * v;
        const float gg = g * g;
        const float cgg = a.c2 * gg;
        r.v = bv + cgg;
        r.root = __builtin_sqrtf(r.v);
        const float den0 = r.root * a.kappa;
        const float den = den0 + a.eps;
        const float u = r.m / den;
        const float decayed = a.lambda * theta_hat;
        const float stp = a.alpha * u;
        r.theta = decayed - stp;
    } else if (kOpt == kSgd) {
        const SgdScalars& s = P.s;
        const float decay = s.omega * theta_hat;
        const float g2 = g + decay;
        const float mb = s.mu * m;
        r.m = mb + g2;
        const float stp = s.eta * r.m;
        r.theta = theta_hat - stp;
    } else {
        const LionScalars& l = P.l;
        const float bm = l.b1 * m;
        const float cg = l.c1 * g;
        const float c = bm + cg;
        const float decayed = l.lambda * theta_hat;
        const float stp = l.eta * lion_sign(c);
        r.theta = decayed - stp;
        const float b2m = l.b2 * m;
        const float c2g = l.c2 * g;
        r.m = b2m + c2g;
    }
    return r;
}

// ---- whole sub-tiles: short exact sequences on the packed registers --------

struct Raw {                        // one lane's packed loads of one sub-tile
    uint4 th, gr;                   // 8 BF16 theta', 8 BF16 grads
    uint2 rho, qm, qv;              // the code record: 8 rho, 8 momentum, 8 variance codes
    uint32_t ms, vs;                // the group's FP16 scales
};

// The lane's index in its wave, read where a tile's addresses are formed.  The
// asm is volatile so that the compiler cannot hoist it (and the per-lane
// offsets derived from it) out of a kernel's tile loop: hoisted, those offsets
// stay live as 64-bit pairs across the whole loop body, and under the step's
// register budget one of them went to scratch memory, 512 bytes written and
// read back per wave.
__device__ __forceinline__ uint32_t lane_here() {
    uint32_t l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
}

// Addresses inside one full tile: the wave-uniform byte address of the tile's
// first element in each array, and the lane's constant byte offsets within a
// sub-tile.  Every access is a scalar base plus a 32-bit lane offset, so no
// per-lane 64-bit address arithmetic is issued per sub-tile.
template <int kOpt>
struct TileAddr {
    static constexpr int kSubEl = kSubTile * 2;                               // BF16 bytes
    static constexpr int kSubRec = Layout<kOpt>::kBlockBytes;
    static constexpr int kSubScl = kSubTile / kGroup * Layout<kOpt>::kScl * 2;
    GLOBAL uint8_t* theta;
    const GLOBAL uint8_t* grad;
    GLOBAL uint8_t* codes;
    GLOBAL uint8_t* scales;
    uint32_t el, rec, scl;          // lane offsets: 8 BF16, its code run, the group's scales

    __device__ __forceinline__ TileAddr(const GTensor& T, int64_t e0)
        : theta((GLOBAL uint8_t*)(T.theta + e0)),
          grad((const GLOBAL uint8_t*)(T.grad + e0)),
          codes(T.codes + (e0 >> 9) * Layout<kOpt>::kBlockBytes),
          scales((GLOBAL uint8_t*)(T.scales + (e0 >> 5) * Layout<kOpt>::kScl)) {
        const uint32_t lane = lane_here();
        el = lane * (kLaneElems * 2);
        rec = lane * Layout<kOpt>::kLaneCode;
        scl = (lane >> 2) * (Layout<kOpt>::kScl * 2);
    }

    __device__ __forceinline__ GLOBAL uint8_t* th(int k) const { return theta + k * kSubEl + el; }
    __device__ __forceinline__ const GLOBAL uint8_t* gr(int k) const {
        return grad + k * kSubEl + el;
    }
    __device__ __forceinline__ GLOBAL uint8_t* rc(int k) const { return codes + k * kSubRec + rec; }
    __device__ __forceinline__ GLOBAL uint8_t* sc(int k) const {
        return scales + k * kSubScl + scl;
    }
};

template <int kOpt>
__device__ __forceinline__ void load_raw(const TileAddr<kOpt>& A, int k, Raw& R) {
    const GLOBAL uint8_t* rec = A.rc(k);
    R.th = ld4nt(A.th(k));
    R.gr = ld4nt(A.gr(k));
    if (kOpt == kAdamW) {
        R.rho = ld2nt(rec);
        R.qm = ld2nt(rec + Layout<kOpt>::kField);
        R.qv = ld2nt(rec + 2 * Layout<kOpt>::kField);
        const uint32_t w = *(const GLOBAL uint32_t*)A.sc(k);             // m | v << 16
        R.ms = w & 0xFFFFu;
        R.vs = w >> 16;
    } else {
        const uint4 r = ld4nt(rec);                        // one 16-byte record
        R.rho = make_uint2(r.x, r.y);
        R.qm = make_uint2(r.z, r.w);
        R.ms = *(const GLOBAL uint16_t*)A.sc(k);
    }
}

__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}
__device__ __forceinline__ uint32_t word(const uint2& v, int i) { return i == 0 ? v.x : v.y; }

// binary32 bits of the j-th BF16 of a lane's 8 (low half first)
__device__ __forceinline__ uint32_t bf16_bits(const uint4& v, int j) {
    const uint32_t w = word(v, j >> 1);
    return (j & 1) ? (w & 0xFFFF0000u) : (w << 16);
}
__device__ __forceinline__ int32_t s8(const uint2& v, int j) {
    return (int32_t)(int8_t)(uint8_t)(word(v, j >> 2) >> (8 * (j & 3)));
}
__device__ __forceinline__ uint32_t u8(const uint2& v, int j) {
    return (word(v, j >> 2) >> (8 * (j & 3))) & 0xFFu;
}

// low bytes of four words, packed into one word
__device__ __forceinline__ uint32_t pack_lo_bytes(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    const uint32_t ab = __builtin_amdgcn_perm(b, a, 0x0C0C0400u);     // a0 b0 0 0
    const uint32_t cd = __builtin_amdgcn_perm(d, c, 0x0C0C0400u);     // c0 d0 0 0
    return __builtin_amdgcn_perm(cd, ab, 0x05040100u);                 // a0 b0 c0 d0
}

// A list's steps never read the single-tensor descriptor; this zero one gives
// step_body an address that is not a per-wave local (which would live in
// scratch memory).
__device__ const DevTensor kNoTensor = {};

// ---- flat-buffer kernels: split / unsplit / quantise / dequantise ----------

// Each wave walks 512-element chunks; lane l owns chunk elements [8l, 8l+8).
#define FLAT_LOOP(n)                                                                   \
    const int lane = threadIdx.x & (kWave - 1);                                          \
    const int64_t wave = uniform((int64_t)blockIdx.x * kWavesPerBlock +            \
                                 (threadIdx.x / kWave));                                 \
    const int64_t nwaves = (int64_t)gridDim.x * kWavesPerBlock;                    \
    for (int64_t c = wave; c * kSubTile < (n); c += nwaves)

}  // namespace flashopt
