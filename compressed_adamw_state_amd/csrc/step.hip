// The fused compressed optimizer step for gfx950: the hot path of
// libflashopt.so.
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
// each for theta' and the gradient, and its codes: one 8-byte run in each of
// the sub-tile's three 512-byte code planes (AdamW: rho, m, v codes; the
// planes of a sub-tile are contiguous, so the codes stay one stream) or one
// 16-byte record (SGD, Lion: rho and m codes); a quantisation group is one
// quad of lanes reduced with DPP, its two FP16 scales one 32-bit word.  Whole tiles take an
// unguarded vector path; the last tile of a tensor takes a guarded
// element-wise path.
#include <algorithm>

#include "host.hpp"

namespace flashopt {

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
            *code_at<kOpt>(T, e + j, kRho) = (uint8_t)orho[j];
            *code_at<kOpt>(T, e + j, kM) = (uint8_t)oqm[j];
            if (kOpt == kAdamW) *code_at<kOpt>(T, e + j, kV) = (uint8_t)oqv[j];
        }
    }
    if ((lane & 3) == 0 && e < n) {
        T.scales[g * Layout<kOpt>::kScl] = (uint16_t)sm16;
        if (kOpt == kAdamW) T.scales[g * Layout<kOpt>::kScl + 1] = (uint16_t)sv16;
    }
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
    uint32_t vmin = 0xFFFFFFFFu;           // min over bits(v') >= +0: flags v' < 2^-96
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
            vmin = min(vmin, as_u32(v_new[j]));
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
        if (__builtin_expect(vmin < 0x0F800000u, 0)) {
            // v' = +0 (a zero gradient over a variance coded 0): sqrt_fast gave
            // NaN (0 * Inf), the root is +0; 0 < v' < 2^-96: the IEEE square root
            uint32_t tiny = 0xFFFFFFFFu;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (as_u32(v_new[j]) == 0u) w[j] = 0.0f;
                tiny = min(tiny, as_u32(v_new[j]) - 1u);
            }
            if (__builtin_expect(tiny < 0x0F7FFFFFu, 0)) {
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (as_u32(v_new[j]) - 1u < 0x0F7FFFFFu) w[j] = __builtin_sqrtf(v_new[j]);
            }
        }
        // u = m' / (w*kappa + eps) by div_rn; a lane with any quotient outside
        // the window rechecks its eight (below)
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
            // the elements whose quotient is outside the window (the same q0 as
            // above): a zero m' over a finite denominator gives u = m' exactly
            // (0 / den keeps the sign of m'), the others (tiny or huge
            // quotients; v' Inf or NaN, where sqrt_fast returned NaN) the IEEE
            // square root and division
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float den0 = w[j] * a.kappa;
                const float den = den0 + a.eps;
                const float q0 = m_new[j] * rcp_rn(den);
                if (quot_key(q0, a.quot_neg_lo2) >= a.quot_span) {
                    if (m_new[j] == 0.0f && __builtin_isfinite(den)) {
                        u[j] = m_new[j];
                    } else {
                        w[j] = __builtin_sqrtf(v_new[j]);
                        const float d0 = w[j] * a.kappa;
                        const float d = d0 + a.eps;
                        u[j] = m_new[j] / d;
                    }
                }
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
    st4nt(A.th(k), make_uint4(otb[0], otb[1], otb[2], otb[3]));
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
    if (kOpt == kAdamW) {                            // three 8-byte plane runs
        st2nt(rec, orho);
        st2nt(rec + Layout<kOpt>::kField, oqm);
        st2nt(rec + 2 * Layout<kOpt>::kField, make_uint2(qv0, qv1));
    } else {                                         // one 16-byte record
        st4nt(rec, make_uint4(orho.x, orho.y, oqm.x, oqm.y));
    }
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
        const TileAddr<kOpt> A(T, e0);
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
        const TileAddr<kOpt> A(T, e0);
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

// The hybrid form of a launch (gradient release: one launch per tensor or per
// bucket): waves [0, nbulk) take one whole tile each, as in step_body, and
// the last ntiles - nbulk tiles go to one wave per 512-element sub-tile.
// Waves are dispatched in order, so the launch ends on short waves: its tail
// (the time the last waves run while SIMDs fall idle) is about a quarter of a
// whole tile's.  The grid covers every wave (no stride loop).
template <int kOpt, bool kLinV>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(5))) void step_kernel_hybrid(
    const DevTensor* __restrict__ table, const int64_t* __restrict__ tile_begin, int32_t count,
    int64_t tile0, int64_t ntiles, int64_t nbulk, DevTensor one, StepScalars P) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t wave = uniform((int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x / kWave));
    TileCursor cur;
    if (wave < nbulk) {
        cur.start(table, tile_begin, count, one, ntiles, tile0 + wave);
        const int64_t e0 = (tile0 + wave - cur.begin) * kTile;
        if (e0 + kTile <= cur.T.numel) step_tile<kOpt, true, kLinV>(cur.T, e0, lane, P);
        else step_tile<kOpt, false, kLinV>(cur.T, e0, lane, P);
        return;
    }
    const int64_t item = wave - nbulk;
    if (item >= (ntiles - nbulk) * kSubTiles) return;
    const int64_t tile = tile0 + nbulk + item / kSubTiles;
    cur.start(table, tile_begin, count, one, ntiles, tile);
    step_sub<kOpt, kLinV>(cur.T, (tile - cur.begin) * kTile, (int)(item % kSubTiles), lane, P);
}

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

template <int kOpt, bool kLinV>
static int launch_fused(const DevTensor* table, const int64_t* tile_begin, int32_t count,
                        int64_t tile0, int64_t ntiles, const DevTensor& one, const StepScalars& P,
                        int64_t tail, hipStream_t st) {
    const int64_t nbulk = ntiles - std::min(tail, ntiles);
    if (ntiles >= kSplitTiles && tail > 0 &&
        nbulk + (ntiles - nbulk) * kSubTiles <= kMaxBlocks * kWavesPerBlock) {
        hipLaunchKernelGGL((step_kernel_hybrid<kOpt, kLinV>),
                           dim3(grid_for(nbulk + (ntiles - nbulk) * kSubTiles)), dim3(kBlock), 0,
                           st, table, tile_begin, count, tile0, ntiles, nbulk, one, P);
        return launch_status();
    }
    if (ntiles < kSplitTiles)
        hipLaunchKernelGGL((step_kernel<kOpt, kLinV, true>), dim3(grid_for(ntiles * kSubTiles)),
                           dim3(kBlock), 0, st, table, tile_begin, count, tile0, ntiles, one, P);
    else
        hipLaunchKernelGGL((step_kernel<kOpt, kLinV, false>), dim3(grid_for(ntiles)),
                           dim3(kBlock), 0, st, table, tile_begin, count, tile0, ntiles, one, P);
    return launch_status();
}

// One launch of the compressed step (see host.hpp).
int launch_step_compressed(int opt, bool linv, const DevTensor* table, const int64_t* tile_begin,
                           int32_t count, int64_t tile0, int64_t ntiles, const DevTensor& one,
                           const StepScalars& P, int64_t tail, hipStream_t st) {
    if (linv)
        return launch_fused<kAdamW, true>(table, tile_begin, count, tile0, ntiles, one, P, tail,
                                          st);
    if (opt == kAdamW)
        return launch_fused<kAdamW, false>(table, tile_begin, count, tile0, ntiles, one, P, tail,
                                           st);
    if (opt == kSgd)
        return launch_fused<kSgd, false>(table, tile_begin, count, tile0, ntiles, one, P, tail,
                                         st);
    return launch_fused<kLion, false>(table, tile_begin, count, tile0, ntiles, one, P, tail, st);
}

// The scheduled step kernel over a whole list, in the same launch form as
// launch_fused chooses.
template <int kOpt>
static int launch_scheduled(const DevTensor* table, const int64_t* tile_begin, int32_t count,
                            int64_t total_tiles, const uint32_t* scalars, hipStream_t st) {
    if (total_tiles < kSplitTiles)
        hipLaunchKernelGGL((step_kernel_scheduled<kOpt, true>),
                           dim3(grid_for(total_tiles * kSubTiles)), dim3(kBlock), 0, st, table,
                           tile_begin, count, total_tiles, scalars);
    else
        hipLaunchKernelGGL((step_kernel_scheduled<kOpt, false>), dim3(grid_for(total_tiles)),
                           dim3(kBlock), 0, st, table, tile_begin, count, total_tiles, scalars);
    return launch_status();
}

int launch_step_scheduled(int opt, const DevTensor* table, const int64_t* tile_begin,
                          int32_t count, int64_t total_tiles, const uint32_t* scalars,
                          hipStream_t st) {
    if (opt == kAdamW)
        return launch_scheduled<kAdamW>(table, tile_begin, count, total_tiles, scalars, st);
    if (opt == kSgd)
        return launch_scheduled<kSgd>(table, tile_begin, count, total_tiles, scalars, st);
    return launch_scheduled<kLion>(table, tile_begin, count, total_tiles, scalars, st);
}

}  // namespace flashopt
