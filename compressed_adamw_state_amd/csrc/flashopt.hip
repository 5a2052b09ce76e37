// HIP kernels for gfx950 and the C ABI declared in include/flashopt.h.
//
// Method: "FlashOptim: Optimizers for Memory Efficient Training" (digest
// page), section "Core method" -- weight splitting (Eq. 1-2, Alg. 1),
// companded group quantisation (Alg. 2-3) and the fused optimizer step
// (Alg. 4), including gradient release.
//
// Design (MI355X): the step is an elementwise read-modify-write stream with a
// 32-element group reduction, bound by HBM bandwidth (12.25 bytes per
// parameter for AdamW).  One launch covers a whole ragged tensor list, one
// wavefront per 2048-element tile; a tile never crosses a tensor boundary,
// and the tile -> tensor lookup is a scalar binary search over per-tensor
// tile offsets kept in a small device table.  Within a tile, lane l owns 8
// consecutive elements of each 512-element sub-tile: one 16-byte BF16 load
// each for theta' and the gradient, and one 8-element code record (rho, m
// and v codes interleaved, so the state is one stream rather than three) read
// as three 8-byte loads; a quantisation group is one quad of lanes reduced
// with DPP, its two FP16 scales one 32-bit word.  Whole tiles take an
// unguarded vector path; the last tile of a tensor takes a guarded
// element-wise path.
//
// Also here: the uncompressed step for layers with compression switched off
// (FP32 master weight and moments in 512-element blocks), the scheduled steps
// whose scalars live in device memory (so a HIP graph can replay them), the
// flat split / quantise kernels, the codec-ablation kernels, list maintenance
// and a bandwidth probe of the step's access pattern.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <new>
#include <vector>

#include "codec.hpp"
#include "flashopt.h"
#include "flashopt_probe.h"

namespace flashopt {

#define GLOBAL __attribute__((address_space(1)))

enum Opt { kAdamW = 0, kSgd = 1, kLion = 2 };

// Every tiled kernel runs blocks of kBlock threads (the launch bounds below and
// every launch say so); kernels use the constant, not blockDim.
constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / kWave;

// State layout of one tensor (see include/flashopt.h): a code record per 8
// elements -- rho[8], m_code[8] and, for AdamW, v_code[8] -- and per 32-element
// group the FP16 m scale followed, for AdamW, by the v scale.  SGD and Lion
// keep one momentum, so they share the 16-byte record.
template <int kOpt> struct Layout {
    static constexpr int kRec = kOpt == kAdamW ? 24 : 16;   // bytes per 8-element record
    static constexpr int kScl = kOpt == kAdamW ? 2 : 1;     // FP16 scales per group
};
constexpr int kRhoOff = 0, kMOff = 8, kVOff = 16;          // field offsets in a record

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

// byte address of field `off` of element i's record entry
template <int kOpt>
__device__ __forceinline__ GLOBAL uint8_t* code_at(const GTensor& T, int64_t i, int off) {
    return T.codes + (i >> 3) * Layout<kOpt>::kRec + off + (i & 7);
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
        L.rho[j] = ok ? (int8_t)*code_at<kOpt>(T, e + j, kRhoOff) : 0;
        L.qm[j] = ok ? (int8_t)*code_at<kOpt>(T, e + j, kMOff) : 0;
        if (kOpt == kAdamW) L.qv[j] = ok ? *code_at<kOpt>(T, e + j, kVOff) : 0u;
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

// ---- the fused step on one sub-tile of one lane ----------------------------

// kLinV (AdamW only): the variance codes are the linear quantiser of v'
// itself (the companding ablation), read back as q * RN(s*K255).
template <int kOpt, bool kLinV = false>
__device__ __forceinline__ void step_lane(const GTensor& T, int64_t e, int lane,
                                          const Lane8& L, const StepScalars& P) {
    float z[8], w[8], tn[8];
    uint32_t amax_m = 0, amax_v = 0;
    const float dm = m_step(L.ms);
    const float dv = (kOpt == kAdamW) ? v_step(L.vs) : 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float theta_hat = unsplit(L.th[j], L.rho[j]);
        const float m = dequant_m(L.qm[j], dm);
        const float g = bf16_to_f32(L.gr[j]);
        const float v = (kOpt != kAdamW) ? 0.0f
                        : kLinV ? (float)L.qv[j] * dv : dequant_v(L.qv[j], dv);
        const Upd u = update<kOpt>(theta_hat, m, v, g, P);
        if (kOpt == kAdamW) {
            w[j] = kLinV ? u.v : u.root;              // what the variance codes quantise
            amax_v = max(amax_v, as_u32(w[j]));
        }
        z[j] = phi_m(u.m);
        tn[j] = u.theta;
        amax_m = max(amax_m, as_u32(z[j]) & 0x7FFFFFFFu);
    }
    // group scales: every lane of the quad computes the same value
    const uint32_t sm16 = group_scale(quad_max_u32(amax_m), 0x3FFFu);
    const float rm = code_factor(sm16, 127.0f);
    uint32_t sv16 = 0;
    float rv = 0.0f;
    if (kOpt == kAdamW) {
        sv16 = group_scale(quad_max_u32(amax_v), 0x7BFFu);
        rv = code_factor(sv16, 255.0f);
    }
    uint32_t otb[8], orho[8], oqm[8], oqv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        oqm[j] = (uint32_t)code_m(z[j], rm);
        if (kOpt == kAdamW) oqv[j] = code_v(w[j], rv);
        const Split sp = split(tn[j]);
        otb[j] = sp.tb;
        orho[j] = (uint32_t)sp.rho;
    }
    const int64_t g = e >> 5;
    const int64_t n = T.numel;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        if (e + j < n) {
            T.theta[e + j] = (uint16_t)otb[j];
            *code_at<kOpt>(T, e + j, kRhoOff) = (uint8_t)orho[j];
            *code_at<kOpt>(T, e + j, kMOff) = (uint8_t)oqm[j];
            if (kOpt == kAdamW) *code_at<kOpt>(T, e + j, kVOff) = (uint8_t)oqv[j];
        }
    }
    if ((lane & 3) == 0 && e < n) {
        T.scales[g * Layout<kOpt>::kScl] = (uint16_t)sm16;
        if (kOpt == kAdamW) T.scales[g * Layout<kOpt>::kScl + 1] = (uint16_t)sv16;
    }
}

// ---- whole sub-tiles: short exact sequences on the packed registers --------

struct Raw {                        // one lane's packed loads of one sub-tile
    uint4 th, gr;                   // 8 BF16 theta', 8 BF16 grads
    uint2 rho, qm, qv;              // the code record: 8 rho, 8 momentum, 8 variance codes
    uint32_t ms, vs;                // the group's FP16 scales
};

// Addresses inside one full tile: the wave-uniform byte address of the tile's
// first element in each array, and the lane's constant byte offsets within a
// sub-tile.  Every access is a scalar base plus a 32-bit lane offset, so no
// per-lane 64-bit address arithmetic is issued per sub-tile.
template <int kOpt>
struct TileAddr {
    static constexpr int kSubEl = kSubTile * 2;                               // BF16 bytes
    static constexpr int kSubRec = kSubTile / 8 * Layout<kOpt>::kRec;
    static constexpr int kSubScl = kSubTile / kGroup * Layout<kOpt>::kScl * 2;
    GLOBAL uint8_t* theta;
    const GLOBAL uint8_t* grad;
    GLOBAL uint8_t* codes;
    GLOBAL uint8_t* scales;
    uint32_t el, rec, scl;          // lane offsets: 8 BF16, one record, the group's scales

    __device__ __forceinline__ TileAddr(const GTensor& T, int64_t e0, int lane)
        : theta((GLOBAL uint8_t*)(T.theta + e0)),
          grad((const GLOBAL uint8_t*)(T.grad + e0)),
          codes(T.codes + (e0 >> 3) * Layout<kOpt>::kRec),
          scales((GLOBAL uint8_t*)(T.scales + (e0 >> 5) * Layout<kOpt>::kScl)),
          el((uint32_t)lane * (kLaneElems * 2)),
          rec((uint32_t)lane * Layout<kOpt>::kRec),
          scl((uint32_t)(lane >> 2) * (Layout<kOpt>::kScl * 2)) {}

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
    R.th = ld4(A.th(k));
    R.gr = ld4(A.gr(k));
    R.rho = ld2(rec + kRhoOff);
    R.qm = ld2(rec + kMOff);
    if (kOpt == kAdamW) {
        R.qv = ld2(rec + kVOff);
        const uint32_t w = *(const GLOBAL uint32_t*)A.sc(k);             // m | v << 16
        R.ms = w & 0xFFFFu;
        R.vs = w >> 16;
    } else {
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

// One lane's 8 elements of a full sub-tile.  The per-element part (rebuilt
// weight, dequantised moments, update, the new weight's split) uses short
// exact sequences; each one's condition of exactness is folded into a flag,
// and a lane with a raised flag redoes that operation for its eight elements
// with the general sequence.  The group part (maxima over the quad of lanes,
// FP16 scales, code factors, codes) follows once the new weight is stored.
template <int kOpt, bool kLinV = false>
__device__ __forceinline__ void step_fast(const TileAddr<kOpt>& A, int k, int lane, const Raw& R,
                                          const StepScalars& P) {
    const AdamScalars& a = P.a;
    const SgdScalars& s = P.s;
    const LionScalars& l = P.l;
    float z[8], w[8], tn[8], m_new[8], v_new[8], theta_hat[8];
    const float dm = m_step(R.ms);
    const float dv = (kOpt == kAdamW) ? v_step(R.vs) : 0.0f;
    uint32_t vmin = 0xFFFFFFFFu;           // min over (bits(v') - 1): flags 0 < v' < 2^-96
    uint32_t tmin = 0xFFFFFFFFu, tmax = 0u;  // exponent fields of theta'
#pragma unroll
    for (int j = 0; j < 8; ++j)
        theta_hat[j] = unsplit_fma(bf16_bits(R.th, j), s8(R.rho, j), tmin, tmax);
    if (__builtin_expect(!unsplit_fma_ok(tmin, tmax), 0)) {
#pragma unroll
        for (int j = 0; j < 8; ++j) theta_hat[j] = unsplit_bits(bf16_bits(R.th, j), s8(R.rho, j));
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float m = phi_m_inv_fast((float)s8(R.qm, j) * dm);
        const float g = as_f32(bf16_bits(R.gr, j));
        if (kOpt == kAdamW) {
            const float zv = (float)u8(R.qv, j) * dv;
            const float v = kLinV ? zv : zv * zv;
            const float bm = a.b1 * m;
            const float cg = a.c1 * g;
            m_new[j] = bm + cg;
            const float bv = a.b2 * v;
            const float gg = g * g;
            const float cgg = a.c2 * gg;
            v_new[j] = bv + cgg;
            w[j] = sqrt_fast(v_new[j]);
            vmin = min(vmin, as_u32(v_new[j]) - 1u);
        } else if (kOpt == kSgd) {
            const float decay = s.omega * theta_hat[j];
            const float g2 = g + decay;
            const float mb = s.mu * m;
            m_new[j] = mb + g2;
            const float stp = s.eta * m_new[j];
            tn[j] = theta_hat[j] - stp;
        } else {
            const float bm = l.b1 * m;
            const float cg = l.c1 * g;
            const float c = bm + cg;
            const float decayed = l.lambda * theta_hat[j];
            const float stp = l.eta * lion_sign(c);
            tn[j] = decayed - stp;
            const float b2m = l.b2 * m;
            const float c2g = l.c2 * g;
            m_new[j] = b2m + c2g;
        }
    }
    if (kOpt == kAdamW) {
        if (__builtin_expect(vmin < 0x0F7FFFFFu, 0)) {
#pragma unroll
            for (int j = 0; j < 8; ++j)                 // 0 < v' < 2^-96: IEEE square root
                if (sqrt_fast_bad(v_new[j])) w[j] = __builtin_sqrtf(v_new[j]);
        }
        // u = m' / (w*kappa + eps) by div_rn; a lane with any quotient outside
        // the window redoes its eight with the IEEE division
        float u[8];
        uint32_t qkey = 0u;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float den0 = w[j] * a.kappa;
            const float den = den0 + a.eps;
            float q0;
            u[j] = div_rn(m_new[j], den, rcp_rn(den), q0);
            qkey = max(qkey, quot_key(q0, a.quot_neg_lo2));
        }
        if (__builtin_expect(qkey >= a.quot_span, 0)) {
            // also where v' is Inf or NaN: sqrt_fast returned NaN there
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                w[j] = __builtin_sqrtf(v_new[j]);
                const float den0 = w[j] * a.kappa;
                const float den = den0 + a.eps;
                u[j] = m_new[j] / den;
            }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float decayed = a.lambda * theta_hat[j];
            const float stp = a.alpha * u[j];
            tn[j] = decayed - stp;
            if (kLinV) w[j] = v_new[j];                // the codes quantise v' itself
        }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) z[j] = phi_m_half_fast(m_new[j]);   // phi_m(m') / 2
    // new theta' and rho: BF16 RNE convert and the biased code of the remainder
    uint32_t otb[4];
    uint32_t rc[2] = {0u, 0u};                      // rho + 128, four per word
    uint32_t emin = 0xFFFFFFFFu, emax = 0u;         // exponent fields of the new theta'
    otb[0] = split2_fast<0>(tn[0], tn[1], rc[0], emin, emax);
    otb[1] = split2_fast<2>(tn[2], tn[3], rc[0], emin, emax);
    otb[2] = split2_fast<0>(tn[4], tn[5], rc[1], emin, emax);
    otb[3] = split2_fast<2>(tn[6], tn[7], rc[1], emin, emax);
    if (__builtin_expect(!split_fast_ok(emin, emax), 0)) {
        // some theta' exponent outside [14, 254] (tiny, zero or non-finite): general split
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const Split s0 = split(tn[2 * p]), s1 = split(tn[2 * p + 1]);
            otb[p] = s0.tb | (s1.tb << 16);
            const int sh = 16 * (p & 1);
            const uint32_t pair = ((uint32_t)(s0.rho + 128) & 0xFFu) |
                                  (((uint32_t)(s1.rho + 128) & 0xFFu) << 8);
            rc[p >> 1] = (rc[p >> 1] & ~(0xFFFFu << sh)) | (pair << sh);
        }
    }
    st4(A.th(k), make_uint4(otb[0], otb[1], otb[2], otb[3]));
    // group maxima of |z| and w as floats (== the integer max of the bit patterns
    // for every finite value)
    float amax_m = 0.0f, amax_v = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        amax_m = fmaxf(amax_m, fabsf(z[j]));
        if (kOpt == kAdamW) amax_v = fmaxf(amax_v, w[j]);
    }
    const uint32_t sm16 =
        group_scale(as_u32(2.0f * as_f32(quad_max_u32(as_u32(amax_m)))), 0x3FFFu);
    const float rm = code_factor_fast(sm16, 254.0f);   // 2 * 127/s, exactly
    uint32_t sv16 = 0;
    uint32_t qv0 = 0, qv1 = 0;
    if (kOpt == kAdamW) {
        sv16 = group_scale(quad_max_u32(as_u32(amax_v)), 0x7BFFu);
        const float rv = code_factor_fast(sv16, 255.0f);
        // clamp(rne(w * 255/s), 0, 255), packed four per word
        qv0 = __builtin_amdgcn_cvt_pk_u8_f32(w[0] * rv, 0, qv0);
        qv0 = __builtin_amdgcn_cvt_pk_u8_f32(w[1] * rv, 1, qv0);
        qv0 = __builtin_amdgcn_cvt_pk_u8_f32(w[2] * rv, 2, qv0);
        qv0 = __builtin_amdgcn_cvt_pk_u8_f32(w[3] * rv, 3, qv0);
        qv1 = __builtin_amdgcn_cvt_pk_u8_f32(w[4] * rv, 0, qv1);
        qv1 = __builtin_amdgcn_cvt_pk_u8_f32(w[5] * rv, 1, qv1);
        qv1 = __builtin_amdgcn_cvt_pk_u8_f32(w[6] * rv, 2, qv1);
        qv1 = __builtin_amdgcn_cvt_pk_u8_f32(w[7] * rv, 3, qv1);
    }
    uint32_t mb[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) mb[j] = code_m_bits(z[j], rm);
    const uint2 oqm = make_uint2(pack_lo_bytes(mb[0], mb[1], mb[2], mb[3]),
                                 pack_lo_bytes(mb[4], mb[5], mb[6], mb[7]));
    const uint2 orho = make_uint2(rc[0] ^ 0x80808080u, rc[1] ^ 0x80808080u);
    GLOBAL uint8_t* rec = A.rc(k);
    st2(rec + kRhoOff, orho);
    st2(rec + kMOff, oqm);
    if (kOpt == kAdamW) st2(rec + kVOff, make_uint2(qv0, qv1));
    if ((lane & 3) == 0) {
        if (kOpt == kAdamW)                          // m | v << 16 in one v_perm
            *(GLOBAL uint32_t*)A.sc(k) = __builtin_amdgcn_perm(sv16, sm16, 0x05040100u);
        else *(GLOBAL uint16_t*)A.sc(k) = (uint16_t)sm16;
    }
}

// A full tile streams its sub-tiles through two register buffers: the loads
// of sub-tile k+2 are issued as soon as sub-tile k is done, so one sub-tile's
// loads are always in flight behind the arithmetic.  The partial last tile of
// a tensor goes one bounds-checked sub-tile at a time.
template <int kOpt, bool kFull, bool kLinV>
__device__ __forceinline__ void step_tile(const GTensor& T, int64_t e0, int lane,
                                          const StepScalars& P) {
    if (kFull) {
        const TileAddr<kOpt> A(T, e0, lane);
        Raw R[2];
        load_raw<kOpt>(A, 0, R[0]);
        if (kSubTiles > 1) load_raw<kOpt>(A, 1, R[1]);
#pragma unroll
        for (int k = 0; k < kSubTiles; ++k) {
            step_fast<kOpt, kLinV>(A, k, lane, R[k & 1], P);
            if (k + 2 < kSubTiles) load_raw<kOpt>(A, k + 2, R[k & 1]);
        }
    } else {
        for (int k = 0; k < kSubTiles; ++k) {
            Lane8 L;
            load_lane<kOpt>(T, e0 + k * kSubTile + lane * kLaneElems, L);
            step_lane<kOpt, kLinV>(T, e0 + k * kSubTile + lane * kLaneElems, lane, L, P);
        }
    }
}

// Five waves per SIMD: the AdamW instantiation fits in 96 VGPRs without
// spilling, and the fifth wave covers more memory latency (measured ~0.5 %).
// Sub-tile k of the tile at e0, alone: the full fast path with its own
// loads, or the bounds-checked path for the part of a tensor's last tile
// that holds elements.
template <int kOpt, bool kLinV>
__device__ __forceinline__ void step_sub(const GTensor& T, int64_t e0, int k, int lane,
                                         const StepScalars& P) {
    const int64_t e = e0 + (int64_t)k * kSubTile;
    if (e + kSubTile <= T.numel) {
        const TileAddr<kOpt> A(T, e0, lane);
        Raw R;
        load_raw<kOpt>(A, k, R);
        step_fast<kOpt, kLinV>(A, k, lane, R, P);
    } else if (e < T.numel) {
        Lane8 L;
        load_lane<kOpt>(T, e + lane * kLaneElems, L);
        step_lane<kOpt, kLinV>(T, e + lane * kLaneElems, lane, L, P);
    }
}

// The launch covers the list's tiles [tile0, tile0 + ntiles) (a range of
// whole tensors: the whole list, or a bucket of consecutive tensors).  kSplit
// (launches of few tiles): one wave per 512-element sub-tile instead of one
// per tile, so a small launch spreads over four times as many waves; the
// arithmetic per element is the same.
template <int kOpt, bool kLinV, bool kSplit>
__device__ __forceinline__ void step_body(const DevTensor* __restrict__ table,
                                          const int64_t* __restrict__ tile_begin, int32_t count,
                                          int64_t tile0, int64_t ntiles, const DevTensor& one,
                                          const StepScalars& P) {
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
            step_sub<kOpt, kLinV>(cur.T, (tile - cur.begin) * kTile, (int)(item % kSubTiles),
                                  lane, P);
        }
        return;
    }
    if (wave >= ntiles) return;
    TileCursor cur;
    cur.start(table, tile_begin, count, one, ntiles, tile0 + wave);
    for (int64_t tile = tile0 + wave; tile < tile0 + ntiles; tile += nwaves) {
        cur.seek(table, tile_begin, tile);
        const int64_t e0 = (tile - cur.begin) * kTile;
        if (e0 + kTile <= cur.T.numel) step_tile<kOpt, true, kLinV>(cur.T, e0, lane, P);
        else step_tile<kOpt, false, kLinV>(cur.T, e0, lane, P);
    }
}

template <int kOpt, bool kLinV, bool kSplit>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(5))) void step_kernel(const DevTensor* __restrict__ table,
                                                   const int64_t* __restrict__ tile_begin,
                                                   int32_t count, int64_t tile0, int64_t ntiles,
                                                   DevTensor one, StepScalars P) {
    step_body<kOpt, kLinV, kSplit>(table, tile_begin, count, tile0, ntiles, one, P);
}

// ---- graph-capturable AdamW: the step's scalars from a device schedule -------

// Advances the schedule by one step (t + 1, p1 * beta1, p2 * beta2: the same
// successive multiplications as the host) and writes the step's scalars.
__global__ void schedule_advance_kernel(flashopt_adamw_schedule* S) {
    if (threadIdx.x != 0 || blockIdx.x != 0) return;
    const double p1 = S->p1 * S->beta1;
    const double p2 = S->p2 * S->beta2;
    S->t = S->t + 1;
    S->p1 = p1;
    S->p2 = p2;
    const AdamScalars a =
        adam_scalars_from(S->lr, S->beta1, S->beta2, S->eps, S->weight_decay, p1, p2);
    uint32_t w[10];
    __builtin_memcpy(w, &a, sizeof a);
    for (int i = 0; i < 10; ++i) S->scalars[i] = w[i];
}

__global__ void schedule_init_kernel(flashopt_adamw_schedule* S, flashopt_adamw_hparams hp,
                                     int64_t t, double p1, double p2) {
    if (threadIdx.x != 0 || blockIdx.x != 0) return;
    S->lr = hp.lr;
    S->eps = hp.eps;
    S->weight_decay = hp.weight_decay;
    S->beta1 = hp.beta1;
    S->beta2 = hp.beta2;
    S->t = t;
    S->p1 = p1;
    S->p2 = p2;
    for (int i = 0; i < 10; ++i) S->scalars[i] = 0u;
    S->pad[0] = S->pad[1] = 0u;
}

__global__ void sgd_schedule_advance_kernel(flashopt_sgd_schedule* S) {
    if (threadIdx.x != 0 || blockIdx.x != 0) return;
    S->t = S->t + 1;
    const SgdScalars a = sgd_scalars_from(S->lr, S->momentum, S->weight_decay);
    uint32_t w[3];
    __builtin_memcpy(w, &a, sizeof a);
    for (int i = 0; i < 3; ++i) S->scalars[i] = w[i];
    S->scalars[3] = 0u;
}

__global__ void lion_schedule_advance_kernel(flashopt_lion_schedule* S) {
    if (threadIdx.x != 0 || blockIdx.x != 0) return;
    S->t = S->t + 1;
    const LionScalars a = lion_scalars_from(S->lr, S->beta1, S->beta2, S->weight_decay);
    uint32_t w[6];
    __builtin_memcpy(w, &a, sizeof a);
    for (int i = 0; i < 6; ++i) S->scalars[i] = w[i];
}

__global__ void sgd_schedule_init_kernel(flashopt_sgd_schedule* S, flashopt_sgd_hparams hp,
                                         int64_t t) {
    if (threadIdx.x != 0 || blockIdx.x != 0) return;
    S->lr = hp.lr;
    S->momentum = hp.momentum;
    S->weight_decay = hp.weight_decay;
    S->t = t;
    for (int i = 0; i < 4; ++i) S->scalars[i] = 0u;
}

__global__ void lion_schedule_init_kernel(flashopt_lion_schedule* S, flashopt_lion_hparams hp,
                                          int64_t t) {
    if (threadIdx.x != 0 || blockIdx.x != 0) return;
    S->lr = hp.lr;
    S->beta1 = hp.beta1;
    S->beta2 = hp.beta2;
    S->weight_decay = hp.weight_decay;
    S->t = t;
    for (int i = 0; i < 6; ++i) S->scalars[i] = 0u;
}

// A list's steps never read the single-tensor descriptor; this zero one gives
// step_body an address that is not a per-wave local (which would live in
// scratch memory).
__device__ const DevTensor kNoTensor = {};

// The step with its scalars read from a schedule's `scalars` words (written
// by the advance kernel launched just before on the same stream).
template <int kOpt, bool kSplit>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(5))) void step_kernel_scheduled(
    const DevTensor* __restrict__ table, const int64_t* __restrict__ tile_begin, int32_t count,
    int64_t total_tiles, const uint32_t* __restrict__ scalars) {
    // typed loads of the kernel-argument pointer (uniform: scalar loads into
    // registers; a copy through the address of a local would go to scratch)
    StepScalars P;
    if (kOpt == kAdamW) P.a = *reinterpret_cast<const AdamScalars*>(scalars);
    else if (kOpt == kSgd) P.s = *reinterpret_cast<const SgdScalars*>(scalars);
    else P.l = *reinterpret_cast<const LionScalars*>(scalars);
    step_body<kOpt, false, kSplit>(table, tile_begin, count, 0, total_tiles, kNoTensor, P);
}

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

struct RawF {
    uint4 th[2], m[2], v[2];        // a lane's 2 x 4 FP32 values of each field
    uint2 gr[2];                    // and its 2 x 4 BF16 gradients
};

// e: a sub-tile's first element (a multiple of 512)
template <int kOpt>
__device__ __forceinline__ void load_raw_f(const GTensor& T, int64_t e, int lane, RawF& R) {
    const GLOBAL uint8_t* blk = T.codes + (e >> 9) * LayoutF<kOpt>::kBlock + 16 * lane;
    R.gr[0] = ld2(T.grad + e + 4 * lane);
    R.gr[1] = ld2(T.grad + e + 256 + 4 * lane);
    R.th[0] = ld4(blk);
    R.th[1] = ld4(blk + 1024);
    R.m[0] = ld4(blk + 2048);
    R.m[1] = ld4(blk + 3072);
    if (kOpt == kAdamW) {
        R.v[0] = ld4(blk + 4096);
        R.v[1] = ld4(blk + 5120);
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
    st2(T.theta + e + 4 * lane, make_uint2(tb[0] | (tb[1] << 16), tb[2] | (tb[3] << 16)));
    st2(T.theta + e + 256 + 4 * lane, make_uint2(tb[4] | (tb[5] << 16), tb[6] | (tb[7] << 16)));
    st4(blk, make_uint4(th[0], th[1], th[2], th[3]));
    st4(blk + 1024, make_uint4(th[4], th[5], th[6], th[7]));
    st4(blk + 2048, make_uint4(mo[0], mo[1], mo[2], mo[3]));
    st4(blk + 3072, make_uint4(mo[4], mo[5], mo[6], mo[7]));
    if (kOpt == kAdamW) {
        st4(blk + 4096, make_uint4(vo[0], vo[1], vo[2], vo[3]));
        st4(blk + 5120, make_uint4(vo[4], vo[5], vo[6], vo[7]));
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

// ---- flat-buffer kernels: split / unsplit / quantise / dequantise ----------

// Each wave walks 512-element chunks; lane l owns chunk elements [8l, 8l+8).
#define FLAT_LOOP(n)                                                                   \
    const int lane = threadIdx.x & (kWave - 1);                                          \
    const int64_t wave = uniform((int64_t)blockIdx.x * kWavesPerBlock +            \
                                 (threadIdx.x / kWave));                                 \
    const int64_t nwaves = (int64_t)gridDim.x * kWavesPerBlock;                    \
    for (int64_t c = wave; c * kSubTile < (n); c += nwaves)

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
                    *code_at<kOpt>(T, e + j, kMOff) = 0;
                    if (kOpt == kAdamW) *code_at<kOpt>(T, e + j, kVOff) = 0;
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
                *code_at<kOpt>(T, e + j, kRhoOff) = (uint8_t)sp.rho;
                *code_at<kOpt>(T, e + j, kMOff) = 0;
                if (kOpt == kAdamW) *code_at<kOpt>(T, e + j, kVOff) = 0;
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
                theta_out[i] = unsplit(T.theta[i], (int8_t)*code_at<kOpt>(T, i, kRhoOff));
            if (m_out) m_out[i] = dequant_m((int8_t)*code_at<kOpt>(T, i, kMOff), dm);
            if (kOpt == kAdamW && v_out) {
                const uint32_t q = *code_at<kOpt>(T, i, kVOff);
                v_out[i] = kLinV ? (float)q * dv : dequant_v(q, dv);
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

constexpr int kGradBatch = 200;
struct GradBatch {
    int32_t first, count;
    const uint16_t* ptr[kGradBatch];
};

__global__ void set_grads_kernel(DevTensor* table, GradBatch b) {
    const int i = threadIdx.x;
    if (i < b.count) table[b.first + i].grad = (uint64_t)b.ptr[i];
}

// ---- host side -------------------------------------------------------------

// One wave per work item (tile or chunk) up to kMaxBlocks blocks; the kernels
// fall back to a wave-stride loop beyond that.  Many short-lived waves let the
// dispatcher refill a CU the moment one finishes, which keeps every SIMD busy
// to the end of the launch (a fixed resident grid left a tail of idle SIMDs).
constexpr int64_t kMaxBlocks = int64_t(1) << 23;    // 2^31 threads

static unsigned grid_for(int64_t wave_items) {
    int64_t blocks = (wave_items + kWavesPerBlock - 1) / kWavesPerBlock;
    if (blocks > kMaxBlocks) blocks = kMaxBlocks;
    if (blocks < 1) blocks = 1;
    return (unsigned)blocks;
}

static bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

static int64_t tiles_of(int64_t n) { return (n + kTile - 1) / kTile; }

static constexpr int64_t kMaxNumel = int64_t(1) << 60;

static int launch_status() {
    return hipGetLastError() == hipSuccess ? FLASHOPT_OK : FLASHOPT_ERR_HIP;
}

static AdamScalars adam_scalars(const flashopt_adamw_hparams& hp, int64_t t, double* p1c,
                                double* p2c, int64_t* tc, double* b1c, double* b2c) {
    // p1 = beta1^t and p2 = beta2^t by t successive multiplications; continue
    // from the cached power when t does not go backwards (same operation
    // sequence, so the same value), stop early once both are zero.
    double p1 = 1.0, p2 = 1.0;
    int64_t k = 0;
    if (*tc > 0 && *tc <= t && *b1c == hp.beta1 && *b2c == hp.beta2) {
        p1 = *p1c; p2 = *p2c; k = *tc;
    }
    for (; k < t; ++k) {
        if (p1 == 0.0 && p2 == 0.0) { k = t; break; }
        p1 = p1 * hp.beta1;
        p2 = p2 * hp.beta2;
    }
    *p1c = p1; *p2c = p2; *tc = t; *b1c = hp.beta1; *b2c = hp.beta2;
    return adam_scalars_from(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, p1, p2);
}

static int check_adam(const flashopt_adamw_hparams* hp, int64_t step) {
    if (!hp) return FLASHOPT_ERR_NULL;
    if (step < 1) return FLASHOPT_ERR_STEP;
    // eps is used as its binary32 rounding: it must not round to 0 (below
    // 2^-150), or a zero second moment would divide 0 by 0
    if (!(hp->lr >= 0.0) || !(hp->beta1 >= 0.0 && hp->beta1 < 1.0) ||
        !(hp->beta2 >= 0.0 && hp->beta2 < 1.0) || !((float)hp->eps > 0.0f) ||
        !(hp->weight_decay >= 0.0) || !std::isfinite(hp->lr) || !std::isfinite(hp->eps) ||
        !std::isfinite(hp->weight_decay))
        return FLASHOPT_ERR_ARG;
    return FLASHOPT_OK;
}

static int check_sgd(const flashopt_sgd_hparams* hp, int64_t step) {
    if (!hp) return FLASHOPT_ERR_NULL;
    if (step < 1) return FLASHOPT_ERR_STEP;
    if (!(hp->lr >= 0.0) || !(hp->momentum >= 0.0 && hp->momentum < 1.0) ||
        !(hp->weight_decay >= 0.0) || !std::isfinite(hp->lr) || !std::isfinite(hp->weight_decay))
        return FLASHOPT_ERR_ARG;
    return FLASHOPT_OK;
}

static bool valid_kind(int32_t kind) {
    return kind >= FLASHOPT_KIND_ADAMW && kind <= FLASHOPT_KIND_ADAMW_LINEAR_V;
}

// the optimizer of a kind (kAdamW, kSgd, kLion), whether its state is FP32,
// and whether its variance codes are linear (the companding ablation)
static int opt_of(int32_t kind) {
    return kind == FLASHOPT_KIND_ADAMW_LINEAR_V ? kAdamW : kind % 3;
}
static bool is_fp32(int32_t kind) {
    return kind >= FLASHOPT_KIND_ADAMW_FP32 && kind <= FLASHOPT_KIND_LION_FP32;
}
static bool is_linv(int32_t kind) { return kind == FLASHOPT_KIND_ADAMW_LINEAR_V; }

static int check_lion(const flashopt_lion_hparams* hp, int64_t step) {
    if (!hp) return FLASHOPT_ERR_NULL;
    if (step < 1) return FLASHOPT_ERR_STEP;
    if (!(hp->lr >= 0.0) || !(hp->beta1 >= 0.0 && hp->beta1 < 1.0) ||
        !(hp->beta2 >= 0.0 && hp->beta2 < 1.0) || !(hp->weight_decay >= 0.0) ||
        !std::isfinite(hp->lr) || !std::isfinite(hp->weight_decay))
        return FLASHOPT_ERR_ARG;
    return FLASHOPT_OK;
}

static SgdScalars sgd_scalars(const flashopt_sgd_hparams& hp) {
    return sgd_scalars_from(hp.lr, hp.momentum, hp.weight_decay);
}

static LionScalars lion_scalars(const flashopt_lion_hparams& hp) {
    return lion_scalars_from(hp.lr, hp.beta1, hp.beta2, hp.weight_decay);
}

static int check_tensor(const flashopt_tensor& t, int32_t kind) {
    if (t.numel < 0 || t.numel > kMaxNumel) return FLASHOPT_ERR_SIZE;
    if (t.numel == 0) return FLASHOPT_OK;
    if (is_fp32(kind)) {                         // FP32 records, no scales
        if (!t.theta || !t.codes) return FLASHOPT_ERR_NULL;
        if (!aligned(t.theta, 16) || !aligned(t.codes, 16) || (t.grad && !aligned(t.grad, 16)))
            return FLASHOPT_ERR_ALIGN;
        return FLASHOPT_OK;
    }
    if (!t.theta || !t.codes || !t.scales) return FLASHOPT_ERR_NULL;
    if (!aligned(t.theta, 16) || !aligned(t.codes, 8) ||
        !aligned(t.scales, opt_of(kind) == kAdamW ? 4 : 2) || (t.grad && !aligned(t.grad, 16)))
        return FLASHOPT_ERR_ALIGN;
    return FLASHOPT_OK;
}

static DevTensor to_dev(const flashopt_tensor& t) {
    DevTensor d{};
    d.theta = (uint64_t)t.theta;
    d.codes = (uint64_t)t.codes;
    d.scales = (uint64_t)t.scales;
    d.grad = (uint64_t)t.grad;
    d.numel = t.numel;
    return d;
}

}  // namespace flashopt

using namespace flashopt;

struct flashopt_list {
    int32_t count = 0;
    int64_t total_tiles = 0;
    int64_t numel = 0;
    DevTensor* d_table = nullptr;
    int64_t* d_tile_begin = nullptr;
    std::vector<flashopt_tensor> host;
    std::vector<int64_t> tile_begin;
    int32_t kind = FLASHOPT_KIND_ADAMW;
    bool all_have_grad = true;
    // cached bias-correction powers (see adam_scalars)
    double p1 = 1.0, p2 = 1.0, b1 = -1.0, b2 = -1.0;
    int64_t t = 0;
};

extern "C" {

const char* flashopt_status_string(int s) {
    switch (s) {
        case FLASHOPT_OK: return "ok";
        case FLASHOPT_ERR_NULL: return "required pointer is NULL";
        case FLASHOPT_ERR_SIZE: return "element or tensor count out of range";
        case FLASHOPT_ERR_ALIGN: return "pointer misaligned";
        case FLASHOPT_ERR_ARG: return "argument out of range or state array missing";
        case FLASHOPT_ERR_STEP: return "step counter must be >= 1";
        case FLASHOPT_ERR_WORKSPACE: return "device workspace too small or misaligned";
        case FLASHOPT_ERR_HIP: return "HIP runtime error";
        case FLASHOPT_ERR_INDEX: return "tensor index out of range";
        case FLASHOPT_ERR_HOST_MEMORY: return "host memory allocation failed";
        default: return "unknown status";
    }
}

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

size_t flashopt_list_workspace_bytes(int32_t count) {
    if (count < 0) return 0;
    const size_t tb = ((size_t)count + 1) * sizeof(int64_t);
    const size_t tb_padded = (tb + 255) / 256 * 256;
    return tb_padded + (size_t)count * sizeof(DevTensor);
}

size_t flashopt_codes_bytes(int32_t kind, int64_t numel) {
    if (!valid_kind(kind) || numel < 0 || numel > kMaxNumel) return 0;
    const bool adam = opt_of(kind) == kAdamW;
    if (is_fp32(kind))                           // whole 512-element blocks of FP32 fields
        return (size_t)((numel + kSubTile - 1) / kSubTile) * kSubTile * 4 * (adam ? 3 : 2);
    return (size_t)((numel + 7) / 8) * (adam ? 24 : 16);
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
    else if (kind == FLASHOPT_KIND_ADAMW_FP32)
        hipLaunchKernelGGL(init_fp32_kernel<kAdamW>, grid, dim3(kBlock), 0, s, to_dev(*t), theta);
    else if (is_fp32(kind))
        hipLaunchKernelGGL(init_fp32_kernel<kSgd>, grid, dim3(kBlock), 0, s, to_dev(*t), theta);
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
    else if (kind == FLASHOPT_KIND_ADAMW_FP32)
        hipLaunchKernelGGL(export_fp32_kernel<kAdamW>, grid, dim3(kBlock), 0, s, to_dev(*t),
                           theta, m, v);
    else if (is_fp32(kind))
        hipLaunchKernelGGL(export_fp32_kernel<kSgd>, grid, dim3(kBlock), 0, s, to_dev(*t), theta,
                           m, v);
    else
        hipLaunchKernelGGL(export_kernel<kSgd>, grid, dim3(kBlock), 0, s, to_dev(*t), theta, m,
                           v);
    return launch_status();
}

int flashopt_list_create(const flashopt_tensor* tensors, int32_t count, int32_t kind,
                         void* workspace, size_t workspace_bytes, void* stream,
                         flashopt_list** out) {
    if (!out) return FLASHOPT_ERR_NULL;
    *out = nullptr;
    if (!valid_kind(kind)) return FLASHOPT_ERR_ARG;
    if (count < 0) return FLASHOPT_ERR_SIZE;
    if (count > 0 && !tensors) return FLASHOPT_ERR_NULL;
    const size_t need = flashopt_list_workspace_bytes(count);
    if (count > 0) {
        if (!workspace) return FLASHOPT_ERR_NULL;
        if (workspace_bytes < need || !aligned(workspace, 256)) return FLASHOPT_ERR_WORKSPACE;
    }
    for (int32_t i = 0; i < count; ++i) {
        const int st = check_tensor(tensors[i], kind);
        if (st != FLASHOPT_OK) return st;
    }
    flashopt_list* L = new (std::nothrow) flashopt_list();
    if (!L) return FLASHOPT_ERR_HOST_MEMORY;
    std::vector<DevTensor> dev;
    try {                                        // no exception crosses the C interface
        L->host.assign(tensors, tensors + count);
        L->tile_begin.resize((size_t)count + 1);
        dev.resize((size_t)count);
    } catch (...) {
        delete L;
        return FLASHOPT_ERR_HOST_MEMORY;
    }
    L->count = count;
    L->kind = kind;
    int64_t tiles = 0;
    for (int32_t i = 0; i < count; ++i) {
        L->tile_begin[i] = tiles;
        tiles += tiles_of(tensors[i].numel);
        L->numel += tensors[i].numel;
        if (tensors[i].numel > 0 && !tensors[i].grad) L->all_have_grad = false;
        dev[i] = to_dev(tensors[i]);
    }
    L->tile_begin[count] = tiles;
    L->total_tiles = tiles;
    if (count > 0) {
        const size_t tb = ((size_t)count + 1) * sizeof(int64_t);
        const size_t tb_padded = (tb + 255) / 256 * 256;
        L->d_tile_begin = (int64_t*)workspace;
        L->d_table = (DevTensor*)((char*)workspace + tb_padded);
        hipStream_t s = (hipStream_t)stream;
        if (hipMemcpyAsync(L->d_tile_begin, L->tile_begin.data(), tb, hipMemcpyHostToDevice, s) !=
                hipSuccess ||
            hipMemcpyAsync(L->d_table, dev.data(), dev.size() * sizeof(DevTensor),
                           hipMemcpyHostToDevice, s) != hipSuccess ||
            hipStreamSynchronize(s) != hipSuccess) {
            delete L;
            return FLASHOPT_ERR_HIP;
        }
    }
    *out = L;
    return FLASHOPT_OK;
}

int flashopt_list_destroy(flashopt_list* L) {
    delete L;
    return FLASHOPT_OK;
}

int64_t flashopt_list_numel(const flashopt_list* L) { return L ? L->numel : -1; }

// Writes the gradient pointers of tensors [first, first + count) into the
// device table (one small kernel per kGradBatch tensors) and the host mirror.
static int set_grads_range(flashopt_list* L, int32_t first, int32_t count,
                           const uint16_t* const* grads, void* stream) {
    for (int32_t i = 0; i < count; ++i)
        if (grads[i] && !aligned(grads[i], 16)) return FLASHOPT_ERR_ALIGN;
    for (int32_t off = 0; off < count; off += kGradBatch) {
        GradBatch b;
        b.first = first + off;
        b.count = std::min<int32_t>(kGradBatch, count - off);
        for (int i = 0; i < b.count; ++i) b.ptr[i] = grads[off + i];
        hipLaunchKernelGGL(set_grads_kernel, dim3(1), dim3(kGradBatch), 0, (hipStream_t)stream,
                           L->d_table, b);
        const int st = launch_status();
        if (st != FLASHOPT_OK) return st;
    }
    for (int32_t i = 0; i < count; ++i) L->host[first + i].grad = grads[i];
    bool all = true;
    for (int32_t i = 0; i < L->count; ++i)
        if (!L->host[i].grad && L->host[i].numel > 0) all = false;
    L->all_have_grad = all;
    return FLASHOPT_OK;
}

int flashopt_list_set_grads(flashopt_list* L, const uint16_t* const* grads, void* stream) {
    if (!L) return FLASHOPT_ERR_NULL;
    if (L->count == 0) return FLASHOPT_OK;
    if (!grads) return FLASHOPT_ERR_NULL;
    return set_grads_range(L, 0, L->count, grads, stream);
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
    else if (L->kind == FLASHOPT_KIND_ADAMW_FP32)
        hipLaunchKernelGGL(zero_fp32_kernel<kAdamW>, grid, dim3(kBlock), 0, s, tab, tb, L->count,
                           L->total_tiles);
    else if (is_fp32(L->kind))
        hipLaunchKernelGGL(zero_fp32_kernel<kSgd>, grid, dim3(kBlock), 0, s, tab, tb, L->count,
                           L->total_tiles);
    else
        hipLaunchKernelGGL(zero_kernel<kSgd>, grid, dim3(kBlock), 0, s, tab, tb, L->count,
                           L->total_tiles);
    return launch_status();
}

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

// Launches of fewer tiles than this run one wave per 512-element sub-tile
// (the kSplit form of the step kernels).  Measured on MI355X (AdamW, one
// tensor): the split form takes 6.4 instead of 9.2 us at 64 tiles, 11.8
// instead of 14.9 at 1279, 42.4 instead of 43.9 at 8192 (and 63 instead of
// 66 us on the 161-tensor ResNet-50 list); the two are even around 16K-32K
// tiles, and from 64K tiles on one wave per tile is ~2 % faster.
constexpr int64_t kSplitTiles = 16384;

extern "C++" {   // templates, inside the C-linkage block
template <int kOpt, bool kLinV>
static int launch_fused(const DevTensor* table, const int64_t* tile_begin, int32_t count,
                        int64_t tile0, int64_t ntiles, const DevTensor& one, const StepScalars& P,
                        hipStream_t st) {
    if (ntiles < kSplitTiles)
        hipLaunchKernelGGL((step_kernel<kOpt, kLinV, true>), dim3(grid_for(ntiles * kSubTiles)),
                           dim3(kBlock), 0, st, table, tile_begin, count, tile0, ntiles, one, P);
    else
        hipLaunchKernelGGL((step_kernel<kOpt, kLinV, false>), dim3(grid_for(ntiles)),
                           dim3(kBlock), 0, st, table, tile_begin, count, tile0, ntiles, one, P);
    return launch_status();
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
}  // extern "C++"

// One launch of the step over the tiles [tile0, tile0 + ntiles) of a list
// (table, tile_begin) or, with table == nullptr, of the single tensor `one`.
static int launch_step(int opt, int32_t kind, const DevTensor* table, const int64_t* tile_begin,
                       int32_t count, int64_t tile0, int64_t ntiles, const DevTensor& one,
                       const StepScalars& P, void* stream) {
    if (ntiles == 0) return FLASHOPT_OK;
    hipStream_t st = (hipStream_t)stream;
    if (is_linv(kind))
        return launch_fused<kAdamW, true>(table, tile_begin, count, tile0, ntiles, one, P, st);
    if (is_fp32(kind)) {
        if (opt == kAdamW)
            return launch_fp32<kAdamW>(table, tile_begin, count, tile0, ntiles, one, P, st);
        if (opt == kSgd)
            return launch_fp32<kSgd>(table, tile_begin, count, tile0, ntiles, one, P, st);
        return launch_fp32<kLion>(table, tile_begin, count, tile0, ntiles, one, P, st);
    }
    if (opt == kAdamW)
        return launch_fused<kAdamW, false>(table, tile_begin, count, tile0, ntiles, one, P, st);
    if (opt == kSgd)
        return launch_fused<kSgd, false>(table, tile_begin, count, tile0, ntiles, one, P, st);
    return launch_fused<kLion, false>(table, tile_begin, count, tile0, ntiles, one, P, st);
}
// The scheduled step kernel over a whole list, in the same launch form as
// launch_fused chooses.
extern "C++" {
template <int kOpt>
static int launch_scheduled(const flashopt_list* L, const uint32_t* scalars, hipStream_t st) {
    const DevTensor* table = (const DevTensor*)L->d_table;
    const int64_t* tile_begin = (const int64_t*)L->d_tile_begin;
    if (L->total_tiles < kSplitTiles)
        hipLaunchKernelGGL((step_kernel_scheduled<kOpt, true>),
                           dim3(grid_for(L->total_tiles * kSubTiles)), dim3(kBlock), 0, st, table,
                           tile_begin, L->count, L->total_tiles, scalars);
    else
        hipLaunchKernelGGL((step_kernel_scheduled<kOpt, false>), dim3(grid_for(L->total_tiles)),
                           dim3(kBlock), 0, st, table, tile_begin, L->count, L->total_tiles,
                           scalars);
    return launch_status();
}
}  // extern "C++"

static int launch_list(int opt, const flashopt_list* L, const StepScalars& P, void* stream) {
    return launch_step(opt, L->kind, L->d_table, L->d_tile_begin, L->count, 0, L->total_tiles,
                       DevTensor{}, P, stream);
}

static int launch_one(int opt, const flashopt_list* L, int32_t index, const uint16_t* grad,
                      const StepScalars& P, void* stream) {
    const flashopt_tensor& t = L->host[index];
    if (t.numel == 0) return FLASHOPT_OK;
    DevTensor one = to_dev(t);
    one.grad = (uint64_t)grad;
    return launch_step(opt, L->kind, nullptr, nullptr, 1, 0, tiles_of(t.numel), one, P, stream);
}

static int check_one(const flashopt_list* L, int32_t index, const uint16_t* grad) {
    if (index < 0 || index >= L->count) return FLASHOPT_ERR_INDEX;
    if (L->host[index].numel > 0) {
        if (!grad) return FLASHOPT_ERR_NULL;
        if (!aligned(grad, 16)) return FLASHOPT_ERR_ALIGN;
    }
    return FLASHOPT_OK;
}

int flashopt_adamw_step(const flashopt_list* L, const flashopt_adamw_hparams* hp, int64_t step,
                        void* stream) {
    if (!L) return FLASHOPT_ERR_NULL;
    int st = check_adam(hp, step);
    if (st != FLASHOPT_OK) return st;
    if (opt_of(L->kind) != kAdamW) return FLASHOPT_ERR_ARG;
    if (!L->all_have_grad) return FLASHOPT_ERR_NULL;
    flashopt_list* M = const_cast<flashopt_list*>(L);   // only the scalar cache changes
    StepScalars P{};
    P.a = adam_scalars(*hp, step, &M->p1, &M->p2, &M->t, &M->b1, &M->b2);
    return launch_list(kAdamW, L, P, stream);
}

int flashopt_sgd_step(const flashopt_list* L, const flashopt_sgd_hparams* hp, int64_t step,
                      void* stream) {
    if (!L) return FLASHOPT_ERR_NULL;
    int st = check_sgd(hp, step);
    if (st != FLASHOPT_OK) return st;
    if (opt_of(L->kind) != kSgd) return FLASHOPT_ERR_ARG;
    if (!L->all_have_grad) return FLASHOPT_ERR_NULL;
    StepScalars P{};
    P.s = sgd_scalars(*hp);
    return launch_list(kSgd, L, P, stream);
}

int flashopt_lion_step(const flashopt_list* L, const flashopt_lion_hparams* hp, int64_t step,
                       void* stream) {
    if (!L) return FLASHOPT_ERR_NULL;
    int st = check_lion(hp, step);
    if (st != FLASHOPT_OK) return st;
    if (opt_of(L->kind) != kLion) return FLASHOPT_ERR_ARG;
    if (!L->all_have_grad) return FLASHOPT_ERR_NULL;
    StepScalars P{};
    P.l = lion_scalars(*hp);
    return launch_list(kLion, L, P, stream);
}

int flashopt_adamw_schedule_init(flashopt_adamw_schedule* S, const flashopt_adamw_hparams* hp,
                                 int64_t t, void* stream) {
    if (!S) return FLASHOPT_ERR_NULL;
    if (!aligned(S, 8)) return FLASHOPT_ERR_ALIGN;
    if (t < 0) return FLASHOPT_ERR_STEP;
    const int st = check_adam(hp, t + 1);
    if (st != FLASHOPT_OK) return st;
    // beta^t by t successive multiplications, as every host step computes it
    double p1 = 1.0, p2 = 1.0;
    for (int64_t k = 0; k < t && !(p1 == 0.0 && p2 == 0.0); ++k) {
        p1 = p1 * hp->beta1;
        p2 = p2 * hp->beta2;
    }
    hipLaunchKernelGGL(schedule_init_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, S, *hp, t,
                       p1, p2);
    return launch_status();
}

int flashopt_adamw_step_scheduled(const flashopt_list* L, flashopt_adamw_schedule* S,
                                  void* stream) {
    if (!L || !S) return FLASHOPT_ERR_NULL;
    if (!aligned(S, 8)) return FLASHOPT_ERR_ALIGN;
    if (L->kind != FLASHOPT_KIND_ADAMW) return FLASHOPT_ERR_ARG;
    if (!L->all_have_grad) return FLASHOPT_ERR_NULL;
    hipStream_t st = (hipStream_t)stream;
    hipLaunchKernelGGL(schedule_advance_kernel, dim3(1), dim3(64), 0, st, S);
    int r = launch_status();
    if (r != FLASHOPT_OK || L->total_tiles == 0) return r;
    return launch_scheduled<kAdamW>(L, (const uint32_t*)S->scalars, st);
}

int flashopt_sgd_schedule_init(flashopt_sgd_schedule* S, const flashopt_sgd_hparams* hp,
                               int64_t t, void* stream) {
    if (!S) return FLASHOPT_ERR_NULL;
    if (!aligned(S, 8)) return FLASHOPT_ERR_ALIGN;
    if (t < 0) return FLASHOPT_ERR_STEP;
    const int st = check_sgd(hp, t + 1);
    if (st != FLASHOPT_OK) return st;
    hipLaunchKernelGGL(sgd_schedule_init_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, S,
                       *hp, t);
    return launch_status();
}

int flashopt_sgd_step_scheduled(const flashopt_list* L, flashopt_sgd_schedule* S, void* stream) {
    if (!L || !S) return FLASHOPT_ERR_NULL;
    if (!aligned(S, 8)) return FLASHOPT_ERR_ALIGN;
    if (L->kind != FLASHOPT_KIND_SGD) return FLASHOPT_ERR_ARG;
    if (!L->all_have_grad) return FLASHOPT_ERR_NULL;
    hipStream_t st = (hipStream_t)stream;
    hipLaunchKernelGGL(sgd_schedule_advance_kernel, dim3(1), dim3(64), 0, st, S);
    int r = launch_status();
    if (r != FLASHOPT_OK || L->total_tiles == 0) return r;
    return launch_scheduled<kSgd>(L, (const uint32_t*)S->scalars, st);
}

int flashopt_lion_schedule_init(flashopt_lion_schedule* S, const flashopt_lion_hparams* hp,
                                int64_t t, void* stream) {
    if (!S) return FLASHOPT_ERR_NULL;
    if (!aligned(S, 8)) return FLASHOPT_ERR_ALIGN;
    if (t < 0) return FLASHOPT_ERR_STEP;
    const int st = check_lion(hp, t + 1);
    if (st != FLASHOPT_OK) return st;
    hipLaunchKernelGGL(lion_schedule_init_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, S,
                       *hp, t);
    return launch_status();
}

int flashopt_lion_step_scheduled(const flashopt_list* L, flashopt_lion_schedule* S,
                                 void* stream) {
    if (!L || !S) return FLASHOPT_ERR_NULL;
    if (!aligned(S, 8)) return FLASHOPT_ERR_ALIGN;
    if (L->kind != FLASHOPT_KIND_LION) return FLASHOPT_ERR_ARG;
    if (!L->all_have_grad) return FLASHOPT_ERR_NULL;
    hipStream_t st = (hipStream_t)stream;
    hipLaunchKernelGGL(lion_schedule_advance_kernel, dim3(1), dim3(64), 0, st, S);
    int r = launch_status();
    if (r != FLASHOPT_OK || L->total_tiles == 0) return r;
    return launch_scheduled<kLion>(L, (const uint32_t*)S->scalars, st);
}

int flashopt_adamw_step_one(const flashopt_list* L, int32_t index, const uint16_t* grad,
                            const flashopt_adamw_hparams* hp, int64_t step, void* stream) {
    if (!L) return FLASHOPT_ERR_NULL;
    if (index < 0 || index >= L->count) return FLASHOPT_ERR_INDEX;
    int st = check_adam(hp, step);
    if (st != FLASHOPT_OK) return st;
    if (opt_of(L->kind) != kAdamW) return FLASHOPT_ERR_ARG;
    st = check_one(L, index, grad);
    if (st != FLASHOPT_OK) return st;
    flashopt_list* M = const_cast<flashopt_list*>(L);
    StepScalars P{};
    P.a = adam_scalars(*hp, step, &M->p1, &M->p2, &M->t, &M->b1, &M->b2);
    return launch_one(kAdamW, L, index, grad, P, stream);
}

int flashopt_sgd_step_one(const flashopt_list* L, int32_t index, const uint16_t* grad,
                          const flashopt_sgd_hparams* hp, int64_t step, void* stream) {
    if (!L) return FLASHOPT_ERR_NULL;
    if (index < 0 || index >= L->count) return FLASHOPT_ERR_INDEX;
    int st = check_sgd(hp, step);
    if (st != FLASHOPT_OK) return st;
    if (opt_of(L->kind) != kSgd) return FLASHOPT_ERR_ARG;
    st = check_one(L, index, grad);
    if (st != FLASHOPT_OK) return st;
    StepScalars P{};
    P.s = sgd_scalars(*hp);
    return launch_one(kSgd, L, index, grad, P, stream);
}

int flashopt_lion_step_one(const flashopt_list* L, int32_t index, const uint16_t* grad,
                           const flashopt_lion_hparams* hp, int64_t step, void* stream) {
    if (!L) return FLASHOPT_ERR_NULL;
    if (index < 0 || index >= L->count) return FLASHOPT_ERR_INDEX;
    int st = check_lion(hp, step);
    if (st != FLASHOPT_OK) return st;
    if (opt_of(L->kind) != kLion) return FLASHOPT_ERR_ARG;
    st = check_one(L, index, grad);
    if (st != FLASHOPT_OK) return st;
    StepScalars P{};
    P.l = lion_scalars(*hp);
    return launch_one(kLion, L, index, grad, P, stream);
}

// ---- bucketed gradient release: one launch over consecutive tensors ----------

static int check_range(const flashopt_list* L, int32_t first, int32_t count) {
    if (!L) return FLASHOPT_ERR_NULL;
    if (first < 0 || count < 0 || first > L->count - count) return FLASHOPT_ERR_INDEX;
    return FLASHOPT_OK;
}

static int check_range_grads(const flashopt_list* L, int32_t first, int32_t count,
                             const uint16_t* const* grads) {
    if (count > 0 && !grads) return FLASHOPT_ERR_NULL;
    for (int32_t i = 0; i < count; ++i) {
        if (!grads[i] && L->host[first + i].numel > 0) return FLASHOPT_ERR_NULL;
        if (grads[i] && !aligned(grads[i], 16)) return FLASHOPT_ERR_ALIGN;
    }
    return FLASHOPT_OK;
}

// The gradients of a range launch serve that launch only (the caller may
// free them once it has run): afterwards the list holds no gradient for
// those tensors, so a whole-list step needs flashopt_list_set_grads first.
static int launch_range(int opt, flashopt_list* L, int32_t first, int32_t count,
                        const uint16_t* const* grads, const StepScalars& P, void* stream) {
    if (count == 0) return FLASHOPT_OK;
    int st = set_grads_range(L, first, count, grads, stream);
    if (st != FLASHOPT_OK) return st;
    const int64_t t0 = L->tile_begin[first], t1 = L->tile_begin[first + count];
    st = launch_step(opt, L->kind, L->d_table, L->d_tile_begin, L->count, t0, t1 - t0,
                     DevTensor{}, P, stream);
    for (int32_t i = 0; i < count; ++i) L->host[first + i].grad = nullptr;
    for (int32_t i = 0; i < count; ++i)
        if (L->host[first + i].numel > 0) L->all_have_grad = false;
    return st;
}

int flashopt_adamw_step_range(flashopt_list* L, int32_t first, int32_t count,
                              const uint16_t* const* grads, const flashopt_adamw_hparams* hp,
                              int64_t step, void* stream) {
    int st = check_range(L, first, count);
    if (st != FLASHOPT_OK) return st;
    st = check_adam(hp, step);
    if (st != FLASHOPT_OK) return st;
    if (opt_of(L->kind) != kAdamW) return FLASHOPT_ERR_ARG;
    st = check_range_grads(L, first, count, grads);
    if (st != FLASHOPT_OK) return st;
    StepScalars P{};
    P.a = adam_scalars(*hp, step, &L->p1, &L->p2, &L->t, &L->b1, &L->b2);
    return launch_range(kAdamW, L, first, count, grads, P, stream);
}

int flashopt_sgd_step_range(flashopt_list* L, int32_t first, int32_t count,
                            const uint16_t* const* grads, const flashopt_sgd_hparams* hp,
                            int64_t step, void* stream) {
    int st = check_range(L, first, count);
    if (st != FLASHOPT_OK) return st;
    st = check_sgd(hp, step);
    if (st != FLASHOPT_OK) return st;
    if (opt_of(L->kind) != kSgd) return FLASHOPT_ERR_ARG;
    st = check_range_grads(L, first, count, grads);
    if (st != FLASHOPT_OK) return st;
    StepScalars P{};
    P.s = sgd_scalars(*hp);
    return launch_range(kSgd, L, first, count, grads, P, stream);
}

int flashopt_lion_step_range(flashopt_list* L, int32_t first, int32_t count,
                             const uint16_t* const* grads, const flashopt_lion_hparams* hp,
                             int64_t step, void* stream) {
    int st = check_range(L, first, count);
    if (st != FLASHOPT_OK) return st;
    st = check_lion(hp, step);
    if (st != FLASHOPT_OK) return st;
    if (opt_of(L->kind) != kLion) return FLASHOPT_ERR_ARG;
    st = check_range_grads(L, first, count, grads);
    if (st != FLASHOPT_OK) return st;
    StepScalars P{};
    P.l = lion_scalars(*hp);
    return launch_range(kLion, L, first, count, grads, P, stream);
}

}  // extern "C"
