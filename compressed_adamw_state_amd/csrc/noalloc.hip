// The whole-list AdamW step for callers that cannot allocate device memory
// (include/flashopt.h, flashopt_adamw_step_noalloc): the list's descriptor
// table and tile offsets live in a fixed array of this library's own device
// memory instead of a caller workspace, filled in stream order by a small
// kernel whose arguments carry the descriptors (no host staging buffer that
// would have to outlive the call), then the step kernel of step.hip runs over
// it.
#include <algorithm>
#include <mutex>

#include "host.hpp"

namespace flashopt {

// Layout of the array: tile offsets (int64[count + 1]) in the first
// kTileBytes, then the 64-byte descriptors.
constexpr int32_t kNoallocMax = FLASHOPT_NOALLOC_MAX_TENSORS;
constexpr size_t kTileBytes = ((size_t)(kNoallocMax + 1) * sizeof(int64_t) + 255) / 256 * 256;
constexpr size_t kScratchBytes = kTileBytes + (size_t)kNoallocMax * sizeof(DevTensor);

// Every GPU the library runs on holds its own copy until the process ends.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

// Descriptors per fill launch: the kernel-argument block stays under 4 KB.
constexpr int kFillBatch = 56;
struct FillBatch {
    int32_t first, count;
    int64_t tile_begin[kFillBatch + 1];    // tile offsets of tensors first .. first + count
    DevTensor d[kFillBatch];
};
static_assert(sizeof(FillBatch) <= 4096, "kernel arguments");

__global__ void fill_kernel(uint8_t* base, FillBatch b) {
    int64_t* tile_begin = (int64_t*)base;
    DevTensor* table = (DevTensor*)(base + kTileBytes);
    const int i = threadIdx.x;
    if (i < b.count) table[b.first + i] = b.d[i];
    if (i <= b.count) tile_begin[b.first + i] = b.tile_begin[i];
}

// The array's device address, looked up once per device with that device
// current (in host code `scratch` is only a stand-in for the symbol).
constexpr int kMaxDevices = 64;
static void* g_scratch[kMaxDevices];
static std::mutex g_scratch_mutex;

static int scratch_of_current_device(uint8_t** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FLASHOPT_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return FLASHOPT_ERR_HIP;
        g_scratch[dev] = p;
    }
    *out = (uint8_t*)g_scratch[dev];
    return FLASHOPT_OK;
}

}  // namespace flashopt

using namespace flashopt;

extern "C" {

int flashopt_adamw_step_noalloc(const flashopt_tensor* tensors, int32_t count,
                                const flashopt_adamw_hparams* hp, int64_t step, void* stream) {
    if (count < 0 || count > kNoallocMax) return FLASHOPT_ERR_SIZE;
    if (count > 0 && !tensors) return FLASHOPT_ERR_NULL;
    int st = check_adam(hp, step);
    if (st != FLASHOPT_OK) return st;
    int64_t total = 0;
    for (int32_t i = 0; i < count; ++i) {
        st = check_tensor(tensors[i], FLASHOPT_KIND_ADAMW);
        if (st != FLASHOPT_OK) return st;
        if (tensors[i].numel > 0 && !tensors[i].grad) return FLASHOPT_ERR_NULL;
        total += tiles_of(tensors[i].numel);
    }
    if (total == 0) return FLASHOPT_OK;
    uint8_t* base = nullptr;
    st = scratch_of_current_device(&base);
    if (st != FLASHOPT_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    int64_t tiles = 0;
    for (int32_t first = 0; first < count; first += kFillBatch) {
        FillBatch b;
        b.first = first;
        b.count = std::min<int32_t>(kFillBatch, count - first);
        for (int32_t k = 0; k < b.count; ++k) {
            b.tile_begin[k] = tiles;
            tiles += tiles_of(tensors[first + k].numel);
            b.d[k] = to_dev(tensors[first + k]);
        }
        b.tile_begin[b.count] = tiles;
        hipLaunchKernelGGL(fill_kernel, dim3(1), dim3(kFillBatch + 1), 0, s, base, b);
        st = launch_status();
        if (st != FLASHOPT_OK) return st;
    }
    // the powers beta^t by t successive multiplications, continued from this
    // thread's previous call when its t and betas allow (host memory only)
    static thread_local double p1 = 1.0, p2 = 1.0, b1 = -1.0, b2 = -1.0;
    static thread_local int64_t tc = 0;
    StepScalars P{};
    P.a = adam_scalars(*hp, step, &p1, &p2, &tc, &b1, &b2);
    return launch_step_compressed(kAdamW, false, (const DevTensor*)(base + kTileBytes),
                                  (const int64_t*)base, count, 0, total, DevTensor{}, P, 0, s);
}

}  // extern "C"
