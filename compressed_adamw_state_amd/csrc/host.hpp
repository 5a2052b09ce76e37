// Host-side helpers of libflashopt.so shared by its translation units: launch
// shapes, argument checks, the per-call optimizer scalars, the list handle,
// and the launch functions each kernel file exports to the C ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <vector>

#include "device.hpp"
#include "flashopt.h"

namespace flashopt {

// One wave per work item (tile or chunk) up to kMaxBlocks blocks; the kernels
// fall back to a wave-stride loop beyond that.  Many short-lived waves let the
// dispatcher refill a CU the moment one finishes, which keeps every SIMD busy
// to the end of the launch (a fixed resident grid left a tail of idle SIMDs).
constexpr int64_t kMaxBlocks = int64_t(1) << 23;    // 2^31 threads

static inline unsigned grid_for(int64_t wave_items) {
    int64_t blocks = (wave_items + kWavesPerBlock - 1) / kWavesPerBlock;
    if (blocks > kMaxBlocks) blocks = kMaxBlocks;
    if (blocks < 1) blocks = 1;
    return (unsigned)blocks;
}

static inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

static inline int64_t tiles_of(int64_t n) { return (n + kTile - 1) / kTile; }

static constexpr int64_t kMaxNumel = int64_t(1) << 60;

static inline int launch_status() {
    return hipGetLastError() == hipSuccess ? FLASHOPT_OK : FLASHOPT_ERR_HIP;
}

static inline AdamScalars adam_scalars(const flashopt_adamw_hparams& hp, int64_t t, double* p1c,
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

static inline int check_adam(const flashopt_adamw_hparams* hp, int64_t step) {
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

static inline int check_sgd(const flashopt_sgd_hparams* hp, int64_t step) {
    if (!hp) return FLASHOPT_ERR_NULL;
    if (step < 1) return FLASHOPT_ERR_STEP;
    if (!(hp->lr >= 0.0) || !(hp->momentum >= 0.0 && hp->momentum < 1.0) ||
        !(hp->weight_decay >= 0.0) || !std::isfinite(hp->lr) || !std::isfinite(hp->weight_decay))
        return FLASHOPT_ERR_ARG;
    return FLASHOPT_OK;
}

static inline bool valid_kind(int32_t kind) {
    return kind >= FLASHOPT_KIND_ADAMW && kind <= FLASHOPT_KIND_ADAMW_LINEAR_V;
}

// the optimizer of a kind (kAdamW, kSgd, kLion), whether its state is FP32,
// and whether its variance codes are linear (the companding ablation)
static inline int opt_of(int32_t kind) {
    return kind == FLASHOPT_KIND_ADAMW_LINEAR_V ? kAdamW : kind % 3;
}
static inline bool is_fp32(int32_t kind) {
    return kind >= FLASHOPT_KIND_ADAMW_FP32 && kind <= FLASHOPT_KIND_LION_FP32;
}
static inline bool is_linv(int32_t kind) { return kind == FLASHOPT_KIND_ADAMW_LINEAR_V; }

static inline int check_lion(const flashopt_lion_hparams* hp, int64_t step) {
    if (!hp) return FLASHOPT_ERR_NULL;
    if (step < 1) return FLASHOPT_ERR_STEP;
    if (!(hp->lr >= 0.0) || !(hp->beta1 >= 0.0 && hp->beta1 < 1.0) ||
        !(hp->beta2 >= 0.0 && hp->beta2 < 1.0) || !(hp->weight_decay >= 0.0) ||
        !std::isfinite(hp->lr) || !std::isfinite(hp->weight_decay))
        return FLASHOPT_ERR_ARG;
    return FLASHOPT_OK;
}

static inline SgdScalars sgd_scalars(const flashopt_sgd_hparams& hp) {
    return sgd_scalars_from(hp.lr, hp.momentum, hp.weight_decay);
}

static inline LionScalars lion_scalars(const flashopt_lion_hparams& hp) {
    return lion_scalars_from(hp.lr, hp.beta1, hp.beta2, hp.weight_decay);
}

static inline int check_tensor(const flashopt_tensor& t, int32_t kind) {
    if (t.numel < 0 || t.numel > kMaxNumel) return FLASHOPT_ERR_SIZE;
    if (t.numel == 0) return FLASHOPT_OK;
    if (is_fp32(kind)) {                         // FP32 records, no scales
        if (!t.theta || !t.codes) return FLASHOPT_ERR_NULL;
        if (!aligned(t.theta, 16) || !aligned(t.codes, 16) || (t.grad && !aligned(t.grad, 16)))
            return FLASHOPT_ERR_ALIGN;
        return FLASHOPT_OK;
    }
    if (!t.theta || !t.codes || !t.scales) return FLASHOPT_ERR_NULL;
    // codes: SGD's and Lion's 16-byte records are read and written whole
    if (!aligned(t.theta, 16) || !aligned(t.codes, 16) ||
        !aligned(t.scales, opt_of(kind) == kAdamW ? 4 : 2) || (t.grad && !aligned(t.grad, 16)))
        return FLASHOPT_ERR_ALIGN;
    return FLASHOPT_OK;
}

static inline DevTensor to_dev(const flashopt_tensor& t) {
    DevTensor d{};
    d.theta = (uint64_t)t.theta;
    d.codes = (uint64_t)t.codes;
    d.scales = (uint64_t)t.scales;
    d.grad = (uint64_t)t.grad;
    d.numel = t.numel;
    return d;
}

// Launches of fewer tiles than this run one wave per 512-element sub-tile
// (the kSplit form of the step kernels).  Measured on MI355X (AdamW, one
// tensor): the split form takes 6.4 instead of 9.2 us at 64 tiles, 11.8
// instead of 14.9 at 1279, 42.4 instead of 43.9 at 8192 (and 63 instead of
// 66 us on the 161-tensor ResNet-50 list); the two are even around 16K-32K
// tiles, and from 64K tiles on one wave per tile is ~2 % faster.
constexpr int64_t kSplitTiles = 16384;

// Tiles at the end of a gradient-release launch (one tensor, or a bucket of
// them) that run as sub-tile waves (the hybrid form): about one round of the
// waves the GPU holds at once (256 CUs x 4 SIMDs x 5 waves = 5120).
#ifndef FLASHOPT_RELEASE_TAIL
#define FLASHOPT_RELEASE_TAIL 2560
#endif
constexpr int64_t kReleaseTail = FLASHOPT_RELEASE_TAIL;

// ---- launches exported by the kernel files ----------------------------------

// step.hip: one launch of the compressed step (opt kAdamW / kSgd / kLion;
// linv: AdamW with linear variance codes) over tiles [tile0, tile0 + ntiles)
// of a list (table, tile_begin) or, with table == nullptr, of the single
// tensor `one`; a launch of at least kSplitTiles tiles with tail > 0 takes the
// hybrid form, its last `tail` tiles as 512-element sub-tile waves (gradient
// release passes kReleaseTail); and the scheduled step over a whole list.
int launch_step_compressed(int opt, bool linv, const DevTensor* table, const int64_t* tile_begin,
                           int32_t count, int64_t tile0, int64_t ntiles, const DevTensor& one,
                           const StepScalars& P, int64_t tail, hipStream_t st);
int launch_step_scheduled(int opt, const DevTensor* table, const int64_t* tile_begin,
                          int32_t count, int64_t total_tiles, const uint32_t* scalars,
                          hipStream_t st);

// step_fp32.hip: the same for the uncompressed (_FP32) kinds, and their
// one-tensor init / export and list zeroing.
int launch_step_fp32(int opt, const DevTensor* table, const int64_t* tile_begin, int32_t count,
                     int64_t tile0, int64_t ntiles, const DevTensor& one, const StepScalars& P,
                     hipStream_t st);
int launch_init_fp32(int opt, const DevTensor& d, const float* x, hipStream_t st);
int launch_export_fp32(int opt, const DevTensor& d, float* theta, float* m, float* v,
                       hipStream_t st);
int launch_zero_fp32(int opt, const DevTensor* table, const int64_t* tile_begin, int32_t count,
                     int64_t total_tiles, hipStream_t st);

// tensor.hip: gradient pointers of tensors [first, first + count) into a
// device table.
int launch_set_grads(DevTensor* table, int32_t first, int32_t count,
                     const uint16_t* const* grads, hipStream_t st);

}  // namespace flashopt

struct flashopt_list {
    int32_t count = 0;
    int64_t total_tiles = 0;
    int64_t numel = 0;
    flashopt::DevTensor* d_table = nullptr;
    int64_t* d_tile_begin = nullptr;
    std::vector<flashopt_tensor> host;
    std::vector<int64_t> tile_begin;
    int32_t kind = FLASHOPT_KIND_ADAMW;
    bool all_have_grad = true;
    // cached bias-correction powers (see adam_scalars)
    double p1 = 1.0, p2 = 1.0, b1 = -1.0, b2 = -1.0;
    int64_t t = 0;
};
