// Device schedules: the fused step with its step counter and scalars in device
// memory, so that a captured HIP graph can replay it (an MI355X-side addition
// around the step of "FlashOptim: Optimizers for Memory Efficient Training",
// digest page, "Core method > Fused optimizer step").
#include "host.hpp"

namespace flashopt {

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

}  // namespace flashopt

using namespace flashopt;

extern "C" {

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
    return launch_step_scheduled(kAdamW, L->d_table, L->d_tile_begin, L->count, L->total_tiles,
                                 (const uint32_t*)S->scalars, st);
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
    return launch_step_scheduled(kSgd, L->d_table, L->d_tile_begin, L->count, L->total_tiles,
                                 (const uint32_t*)S->scalars, st);
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
    return launch_step_scheduled(kLion, L->d_table, L->d_tile_begin, L->count, L->total_tiles,
                                 (const uint32_t*)S->scalars, st);
}

}  // extern "C"
