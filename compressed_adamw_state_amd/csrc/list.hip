// The C ABI of include/flashopt.h for tensor lists: handles, gradient
// pointers, and the step entry points (whole list, one tensor, a range of
// tensors) that launch the kernels of step.hip and step_fp32.hip.  Host code
// only.
#include <algorithm>
#include <new>

#include "host.hpp"

using namespace flashopt;

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

size_t flashopt_list_workspace_bytes(int32_t count) {
    if (count < 0) return 0;
    const size_t tb = ((size_t)count + 1) * sizeof(int64_t);
    const size_t tb_padded = (tb + 255) / 256 * 256;
    return tb_padded + (size_t)count * sizeof(DevTensor);
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
// device table (launch_set_grads) and the host mirror.
static int set_grads_range(flashopt_list* L, int32_t first, int32_t count,
                           const uint16_t* const* grads, void* stream) {
    for (int32_t i = 0; i < count; ++i)
        if (grads[i] && !aligned(grads[i], 16)) return FLASHOPT_ERR_ALIGN;
    const int st = launch_set_grads(L->d_table, first, count, grads, (hipStream_t)stream);
    if (st != FLASHOPT_OK) return st;
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

// One launch of the step over the tiles [tile0, tile0 + ntiles) of a list
// (table, tile_begin) or, with table == nullptr, of the single tensor `one`;
// tail > 0: the compressed step's hybrid form (gradient-release launches).
static int launch_step(int opt, int32_t kind, const DevTensor* table, const int64_t* tile_begin,
                       int32_t count, int64_t tile0, int64_t ntiles, const DevTensor& one,
                       const StepScalars& P, int64_t tail, void* stream) {
    if (ntiles == 0) return FLASHOPT_OK;
    hipStream_t st = (hipStream_t)stream;
    if (is_fp32(kind))
        return launch_step_fp32(opt, table, tile_begin, count, tile0, ntiles, one, P, st);
    return launch_step_compressed(opt, is_linv(kind), table, tile_begin, count, tile0, ntiles, one,
                                  P, tail, st);
}

static int launch_list(int opt, const flashopt_list* L, const StepScalars& P, void* stream) {
    return launch_step(opt, L->kind, L->d_table, L->d_tile_begin, L->count, 0, L->total_tiles,
                       DevTensor{}, P, 0, stream);
}

static int launch_one(int opt, const flashopt_list* L, int32_t index, const uint16_t* grad,
                      const StepScalars& P, void* stream) {
    const flashopt_tensor& t = L->host[index];
    if (t.numel == 0) return FLASHOPT_OK;
    DevTensor one = to_dev(t);
    one.grad = (uint64_t)grad;
    return launch_step(opt, L->kind, nullptr, nullptr, 1, 0, tiles_of(t.numel), one, P,
                       kReleaseTail, stream);
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
                     DevTensor{}, P, kReleaseTail, stream);
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
