// A C++ consumer of the C ABI with no Python and no torch: device memory from
// hipMalloc, the stream from hipStreamCreate, every call through
// include/flashopt.h.  It steps a ragged list with AdamW (whole-list launch,
// gradient release per tensor and in buckets of consecutive tensors), Lion
// and SGD, and compares every theta', code and
// scale with the CPU oracle (oracle/flashopt_oracle.h, test infrastructure)
// stepping the same inputs.  Exit status 0 when everything matches.
//
// FlashOptim: Optimizers for Memory Efficient Training -- Core method, fused
// optimizer step (Alg. 4) and gradient release.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "flashopt.h"
#include "flashopt_oracle.h"

#define HIP_OK(x)                                                                   \
    do {                                                                            \
        hipError_t e_ = (x);                                                        \
        if (e_ != hipSuccess) {                                                     \
            std::fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));     \
            return 2;                                                               \
        }                                                                           \
    } while (0)

#define FO_OK(x)                                                                    \
    do {                                                                            \
        int s_ = (x);                                                               \
        if (s_ != FLASHOPT_OK) {                                                    \
            std::fprintf(stderr, "%s failed: %s\n", #x, flashopt_status_string(s_)); \
            return 3;                                                               \
        }                                                                           \
    } while (0)

namespace {

// seeded inputs: splitmix64 -> Box-Muller normals
struct Rng {
    uint64_t s;
    uint64_t next() {
        uint64_t z = (s += 0x9E3779B97F4A7C15ull);
        z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
        z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
        return z ^ (z >> 31);
    }
    double uniform() { return ((next() >> 11) + 0.5) * (1.0 / 9007199254740992.0); }
    float normal(double sd) {
        const double u = uniform(), v = uniform();
        return (float)(sd * __builtin_sqrt(-2.0 * __builtin_log(u)) * __builtin_cos(6.283185307179586 * v));
    }
};

struct Host {                       // one tensor's state as the oracle holds it
    int64_t n;
    std::vector<uint16_t> tb, sm, sv;
    std::vector<int8_t> rho, qm;
    std::vector<uint8_t> qv;
};

struct Dev {                        // the same tensor's state on the device
    uint16_t* theta = nullptr;
    uint8_t* codes = nullptr;
    uint16_t* scales = nullptr;
    uint16_t* grad = nullptr;
    size_t codes_bytes = 0, scales_bytes = 0;
};

// compare the device state of one tensor with the oracle's, element by element
int compare(const Host& h, const Dev& d, int32_t kind, const char* what) {
    const int64_t n = h.n;
    const bool adam = kind == FLASHOPT_KIND_ADAMW;
    std::vector<uint16_t> th((size_t)n);
    std::vector<uint8_t> codes(d.codes_bytes);
    std::vector<uint16_t> scales(d.scales_bytes / 2);
    if (n == 0) return 0;
    if (hipMemcpy(th.data(), d.theta, (size_t)n * 2, hipMemcpyDeviceToHost) != hipSuccess ||
        hipMemcpy(codes.data(), d.codes, d.codes_bytes, hipMemcpyDeviceToHost) != hipSuccess ||
        hipMemcpy(scales.data(), d.scales, d.scales_bytes, hipMemcpyDeviceToHost) != hipSuccess)
        return 2;
    const int64_t per_group = adam ? 2 : 1;
    int64_t bad = 0;
    for (int64_t i = 0; i < n; ++i) {
        // AdamW: 512-element blocks of rho, m and v planes; SGD, Lion: 16-byte
        // records of 8 elements (include/flashopt.h)
        const uint8_t* r = adam ? codes.data() + (i >> 9) * 1536 + (i & 511)
                                : codes.data() + (i >> 3) * 16 + (i & 7);
        const int64_t field = adam ? 512 : 8;
        bad += th[i] != h.tb[i];
        bad += (int8_t)r[0] != h.rho[i];
        bad += (int8_t)r[field] != h.qm[i];
        if (adam) bad += r[2 * field] != h.qv[i];
    }
    for (int64_t g = 0; g < (n + 31) / 32; ++g) {
        bad += scales[g * per_group] != h.sm[g];
        if (adam) bad += scales[g * per_group + 1] != h.sv[g];
    }
    if (bad) std::fprintf(stderr, "%s: tensor of %lld elements: %lld mismatches\n", what,
                          (long long)n, (long long)bad);
    return bad ? 1 : 0;
}

enum Mode { kList, kRelease, kBuckets };

int run(int32_t kind, Mode mode, hipStream_t stream) {
    const int64_t sizes[] = {4101, 33, 2048, 1, 0, 70000};
    const int count = (int)(sizeof sizes / sizeof sizes[0]);
    const char* name = kind == FLASHOPT_KIND_ADAMW
                           ? (mode == kRelease ? "adamw release"
                              : mode == kBuckets ? "adamw buckets" : "adamw")
                       : kind == FLASHOPT_KIND_LION ? "lion" : "sgd";
    Rng rng{0x5EEDull + (uint64_t)kind * 7 + (uint64_t)mode};
    std::vector<Host> host((size_t)count);
    std::vector<Dev> dev((size_t)count);
    std::vector<flashopt_tensor> desc((size_t)count);
    for (int i = 0; i < count; ++i) {
        const int64_t n = sizes[i];
        Host& h = host[(size_t)i];
        Dev& d = dev[(size_t)i];
        h.n = n;
        std::vector<float> theta((size_t)n);
        for (auto& x : theta) x = rng.normal(0.02);
        h.tb.resize((size_t)n);
        h.rho.resize((size_t)n);
        h.qm.assign((size_t)n, 0);
        h.qv.assign((size_t)n, 0);
        h.sm.assign((size_t)((n + 31) / 32), 0);
        h.sv.assign((size_t)((n + 31) / 32), 0);
        orc_split(theta.data(), n, h.tb.data(), h.rho.data());
        d.codes_bytes = flashopt_codes_bytes(kind, n);
        d.scales_bytes = flashopt_scales_bytes(kind, n);
        float* dtheta = nullptr;
        if (n > 0) {
            HIP_OK(hipMalloc(&d.theta, (size_t)n * 2));
            HIP_OK(hipMalloc(&d.codes, d.codes_bytes));
            HIP_OK(hipMalloc(&d.scales, d.scales_bytes));
            HIP_OK(hipMalloc(&d.grad, (size_t)n * 2));
            HIP_OK(hipMalloc(&dtheta, (size_t)n * 4));
            HIP_OK(hipMemcpy(dtheta, theta.data(), (size_t)n * 4, hipMemcpyHostToDevice));
        }
        desc[(size_t)i] = flashopt_tensor{n, d.theta, d.codes, d.scales, d.grad};
        FO_OK(flashopt_tensor_init(&desc[(size_t)i], kind, dtheta, stream));
        HIP_OK(hipStreamSynchronize(stream));
        if (dtheta) HIP_OK(hipFree(dtheta));
        if (compare(h, d, kind, name)) return 1;
    }
    void* ws = nullptr;
    const size_t ws_bytes = flashopt_list_workspace_bytes(count);
    HIP_OK(hipMalloc(&ws, ws_bytes));
    flashopt_list* list = nullptr;
    FO_OK(flashopt_list_create(desc.data(), count, kind, ws, ws_bytes, stream, &list));

    const flashopt_adamw_hparams adam{1e-3, 0.9, 0.999, 1e-8, 0.01};
    const flashopt_sgd_hparams sgd{0.1, 0.9, 1e-4};
    const flashopt_lion_hparams lion{1e-4, 0.9, 0.99, 0.1};
    for (int64_t t = 1; t <= 3; ++t) {
        for (int i = 0; i < count; ++i) {
            Host& h = host[(size_t)i];
            const int64_t n = h.n;
            std::vector<uint16_t> g((size_t)n);
            for (auto& x : g) x = orc_bf16_rne(rng.normal(kind == FLASHOPT_KIND_SGD ? 1e-2 : 1e-3));
            if (n > 0)
                HIP_OK(hipMemcpyAsync(dev[(size_t)i].grad, g.data(), (size_t)n * 2,
                                      hipMemcpyHostToDevice, stream));
            HIP_OK(hipStreamSynchronize(stream));
            if (kind == FLASHOPT_KIND_ADAMW)
                orc_adamw_step(n, h.tb.data(), h.rho.data(), h.qm.data(), h.sm.data(),
                               h.qv.data(), h.sv.data(), g.data(), adam.lr, adam.beta1,
                               adam.beta2, adam.eps, adam.weight_decay, t, nullptr, nullptr,
                               nullptr);
            else if (kind == FLASHOPT_KIND_LION)
                orc_lion_step(n, h.tb.data(), h.rho.data(), h.qm.data(), h.sm.data(), g.data(),
                              lion.lr, lion.beta1, lion.beta2, lion.weight_decay, nullptr,
                              nullptr);
            else
                orc_sgd_step(n, h.tb.data(), h.rho.data(), h.qm.data(), h.sm.data(), g.data(),
                             sgd.lr, sgd.momentum, sgd.weight_decay, t, nullptr, nullptr);
        }
        if (mode == kRelease) {
            for (int i = count - 1; i >= 0; --i)     // backward order, one launch per tensor
                FO_OK(flashopt_adamw_step_one(list, i, dev[(size_t)i].grad, &adam, t, stream));
        } else if (mode == kBuckets) {
            // backward order, one launch per bucket of consecutive tensors
            const int buckets[][2] = {{4, 2}, {1, 3}, {0, 1}};
            for (const auto& b : buckets) {
                const uint16_t* g[3];
                for (int i = 0; i < b[1]; ++i) g[i] = dev[(size_t)(b[0] + i)].grad;
                FO_OK(flashopt_adamw_step_range(list, b[0], b[1], g, &adam, t, stream));
            }
            // the ranges' gradients served those launches only: a whole-list
            // step is refused until the gradients are given again
            if (flashopt_adamw_step(list, &adam, t + 1, stream) != FLASHOPT_ERR_NULL) {
                std::fprintf(stderr, "%s: whole-list step accepted after range launches\n", name);
                return 1;
            }
        } else if (kind == FLASHOPT_KIND_ADAMW) {
            FO_OK(flashopt_adamw_step(list, &adam, t, stream));
        } else if (kind == FLASHOPT_KIND_LION) {
            FO_OK(flashopt_lion_step(list, &lion, t, stream));
        } else {
            FO_OK(flashopt_sgd_step(list, &sgd, t, stream));
        }
        HIP_OK(hipStreamSynchronize(stream));
        for (int i = 0; i < count; ++i)
            if (compare(host[(size_t)i], dev[(size_t)i], kind, name)) return 1;
    }
    FO_OK(flashopt_list_destroy(list));
    HIP_OK(hipFree(ws));
    for (auto& d : dev) {
        if (d.theta) HIP_OK(hipFree(d.theta));
        if (d.codes) HIP_OK(hipFree(d.codes));
        if (d.scales) HIP_OK(hipFree(d.scales));
        if (d.grad) HIP_OK(hipFree(d.grad));
    }
    std::printf("c_abi_check: %s: 3 steps over %d tensors match the oracle\n", name, count);
    std::fflush(stdout);
    return 0;
}

}  // namespace

int main() {
    if (orc_env_ok() != 1) {
        std::fprintf(stderr, "oracle: non-nearest rounding or flush-to-zero in effect\n");
        return 4;
    }
    hipStream_t stream = nullptr;
    HIP_OK(hipSetDevice(0));
    HIP_OK(hipStreamCreate(&stream));
    int rc = 0;
    if (!rc) rc = run(FLASHOPT_KIND_ADAMW, kList, stream);
    if (!rc) rc = run(FLASHOPT_KIND_ADAMW, kRelease, stream);
    if (!rc) rc = run(FLASHOPT_KIND_ADAMW, kBuckets, stream);
    if (!rc) rc = run(FLASHOPT_KIND_LION, kList, stream);
    if (!rc) rc = run(FLASHOPT_KIND_SGD, kList, stream);
    HIP_OK(hipStreamDestroy(stream));
    return rc;
}
