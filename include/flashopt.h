/*
 * flashopt.h -- C ABI of the MI355X (gfx950) implementation of FlashOptim's
 * fused compressed optimizer step.
 *
 * Method: "FlashOptim: Optimizers for Memory Efficient Training" (arXiv
 * 2602.23349v1), as summarised by its digest page:
 *   - section "Core method > Weight splitting: ULP-based error correction"
 *     (Eq. 1-2, Alg. 1): the FP32 master weight is stored as a BF16 weight
 *     theta' plus an INT8 code rho of the error theta - theta' normalised by
 *     ULP(theta')/2;
 *   - section "Core method > Optimizer-state quantisation with companding"
 *     (Alg. 2-3): momentum m is stored as INT8 codes of phi_m(m) = 2m/(1+|m|),
 *     variance v as UINT8 codes of phi_v(v) = sqrt(v), each with one FP16
 *     scale per group of 32 elements;
 *   - section "Core method > Fused optimizer step" (Alg. 4): one pass per
 *     parameter dequantises, rebuilds the master weight, applies AdamW (or
 *     SGD with momentum, or Lion), requantises the states and re-splits the
 *     weight; gradient release steps each tensor as soon as its gradient
 *     exists.
 *
 * Arithmetic (every operation IEEE binary32, round to nearest even, no fused
 * multiply-add, subnormals kept; K8 = RN(1/127), K255 = RN(1/255)) -- the
 * results are those of this operation sequence; the kernels reach the same
 * bits with shorter sequences (some with FMA) checked to be identical:
 *   h         = ULP(theta')/2 = 2^(max(E,1)-135), E = exponent field of theta'
 *   rebuild   theta_hat = theta' + (rho*K8)*h                 (theta' Inf/NaN: theta')
 *   dequant   m = z/(2-|z|), z = q*(s*K8);  v = z*z, z = q*(s*K255)
 *   AdamW     m' = b1*m + c1*g;  v' = b2*v + c2*(g*g);  w = sqrt(v');
 *             theta_n = lambda*theta_hat - alpha*(m'/(w*kappa + eps))
 *   SGD       g' = g + wd*theta_hat;  b' = mu*b + g';  theta_n = theta_hat - lr*b'
 *   Lion      c = b1*m + c1*g;  theta_n = lambda*theta_hat - lr*sign(c);
 *             m' = b2*m + c2*g  (flashopt_lion_hparams)
 *   requant   z = (2m')/(1+|m'|) (momentum) or w (variance); a = max |z| over
 *             the group's elements; s = FP16(a) capped at 0x3FFF (momentum) or
 *             0x7BFF (variance); q = 0 if s = 0 else clamp(rne(z*(127/s)), +-127)
 *             (variance: 255/s, [0,255])
 *   re-split  theta' = BF16_rne(theta_n); rho = clamp(rne(127*(theta_n-theta')/h), +-127)
 *             (0 when theta' is Inf/NaN)
 * with per-call scalars computed on the host in double and rounded once:
 *   p1 = beta1^t, p2 = beta2^t (t successive multiplications), b1 = beta1,
 *   c1 = 1-beta1, b2 = beta2, c2 = 1-beta2, alpha = lr/(1-p1),
 *   kappa = 1/sqrt(1-p2), lambda = 1-lr*wd.
 *
 * Memory and ownership.  Every array argument is DEVICE memory on the
 * current HIP device, owned by the caller (the library never allocates device
 * memory); streams are hipStream_t values passed as void* (NULL = the null
 * stream).  Element arrays are dense, 1-D, row-major flattenings of the
 * tensor.  Groups of 32 restart at element 0 of every tensor; a tensor of n
 * elements has ceil(n/32) scales per state, the last group possibly partial
 * (its scale covers only its valid elements).  BF16 and FP16 values are passed
 * as their uint16 bit patterns.
 *
 * Alignment: BF16 arrays (theta', grad) and a tensor's codes 16 bytes; flat
 * INT8/UINT8 code arrays 8 bytes; AdamW scale arrays 4 bytes, SGD / Lion and
 * flat scale arrays 2 bytes; FP32 arrays and the _FP32 kinds' state blocks 16
 * bytes (the ablation entry points, element by element: their element size).
 *
 * Errors.  Every call validates its arguments on the host before launching
 * anything and returns a flashopt_status; a failed validation launches
 * nothing.  FLASHOPT_ERR_HIP reports a launch failure (hipGetLastError).
 * Faults inside kernels surface asynchronously at the caller's next
 * synchronisation.  Calls are ordered on the given stream and never
 * synchronise the device, except flashopt_list_create (documented there).
 * Non-finite gradients are outside the contract (they propagate).
 * No C++ exception crosses this interface.  A list handle must not be used
 * from two host threads at once.
 */
#ifndef FLASHOPT_H
#define FLASHOPT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FLASHOPT_GROUP 32

typedef enum flashopt_status {
    FLASHOPT_OK = 0,
    FLASHOPT_ERR_NULL = -1,      /* a required pointer is NULL                         */
    FLASHOPT_ERR_SIZE = -2,      /* negative or too large element count / list count   */
    FLASHOPT_ERR_ALIGN = -3,     /* a pointer violates the alignment above             */
    FLASHOPT_ERR_ARG = -4,       /* hyper-parameter out of range, wrong kind           */
    FLASHOPT_ERR_STEP = -5,      /* step counter t < 1                                 */
    FLASHOPT_ERR_WORKSPACE = -6, /* device workspace too small                         */
    FLASHOPT_ERR_HIP = -7,       /* HIP runtime error (launch, copy, device query)     */
    FLASHOPT_ERR_INDEX = -8,     /* tensor index out of range                          */
    FLASHOPT_ERR_HOST_MEMORY = -9 /* host allocation for a list handle failed          */
} flashopt_status;

/* Optimizer kind of a tensor's state layout (and of a list).  The _FP32
 * kinds are the same optimizers with compression switched off (practical-
 * advice section: compression can be disabled per layer): an FP32 master
 * weight and FP32 moments, no codes, no scales. */
typedef enum flashopt_kind {
    FLASHOPT_KIND_ADAMW = 0,     /* rho, momentum and variance codes; two scales per group */
    FLASHOPT_KIND_SGD = 1,       /* rho and momentum codes; one scale per group            */
    FLASHOPT_KIND_LION = 2,      /* the SGD layout, holding Lion's momentum                */
    FLASHOPT_KIND_ADAMW_FP32 = 3,/* FP32 theta, m, v in 512-element blocks; no scales      */
    FLASHOPT_KIND_SGD_FP32 = 4,  /* FP32 theta and momentum buffer in blocks; no scales    */
    FLASHOPT_KIND_LION_FP32 = 5, /* FP32 theta and momentum in blocks; no scales           */
    FLASHOPT_KIND_ADAMW_LINEAR_V = 6 /* ablation only: the AdamW layout with linear variance
                                        codes (no square root; companding section, Fig. 5) */
} flashopt_kind;

/* One parameter tensor and its compressed state (all DEVICE pointers).
 *
 * State layout.  The per-element codes lie in blocks of 512 consecutive
 * elements, one block after another, so the fused step reads and writes them
 * as one stream (HBM bandwidth on this device falls with the number of
 * concurrent streams).  AdamW: a block is three 512-byte planes,
 *   codes[b*1536 + 0 + p]    = rho of element 512b+p             (INT8, two's complement)
 *   codes[b*1536 + 512 + p]  = momentum code of element 512b+p   (INT8)
 *   codes[b*1536 + 1024 + p] = variance code of element 512b+p   (UINT8)
 * with b < ceil(n/512), p < 512, so that each of a lane's three code accesses
 * in the step (8 bytes) covers whole lines together with its wave's other
 * lanes.  SGD, Lion: a record of 16 bytes per 8 consecutive elements,
 *   codes[r*16 + 0 + j] = rho of element 8r+j                    (INT8)
 *   codes[r*16 + 8 + j] = momentum code of element 8r+j          (INT8; SGD: momentum buffer)
 * with r < ceil(n/8), j < 8 (a lane's record is one 16-byte access).  In both
 * layouts the entries past n are padding (never read as state, may be
 * overwritten).
 *   scales[2g], scales[2g+1] = FP16 momentum and variance scales of group g (AdamW)
 *   scales[g]                = FP16 momentum scale of group g (SGD, Lion)
 * for g < ceil(n/32).  flashopt_codes_bytes / flashopt_scales_bytes give the
 * sizes.  The values are exactly those of the flat arrays the quantisers and
 * split below produce, only their placement differs.
 *
 * FLASHOPT_KIND_ADAMW_LINEAR_V has the AdamW layout, but its variance codes
 * are the linear quantiser of v' itself (scale f16_rne(max v'), codes
 * clamp(rne(v' * RN(255/s)), 0, 255), read back as q * RN(s*K255)): the
 * no-companding ablation, for experiments only.
 *
 * _FP32 kinds: `codes` holds blocks of 512 elements of FP32 fields (16-byte
 * aligned),
 *   ((float*)codes)[b*512*F + 0 + p]    = master weight theta of element 512b+p
 *   ((float*)codes)[b*512*F + 512 + p]  = momentum (SGD: momentum buffer)
 *   ((float*)codes)[b*512*F + 1024 + p] = variance (AdamW only)
 * with F = 3 (AdamW) or 2 (SGD, Lion), b < ceil(n/512), p < 512; the last
 * block's entries past n are padding.  `scales` is not used (may be NULL) and
 * theta' is written by every step as bf16_rne(theta), the weight the model
 * computes with (it is never read). */
typedef struct flashopt_tensor {
    int64_t numel;           /* n >= 0                                                   */
    uint16_t* theta;         /* [n] BF16 theta'; the model weight the forward pass reads */
    uint8_t* codes;          /* codes (planes or records), layout above                  */
    uint16_t* scales;        /* FP16 scales, layout above                                */
    const uint16_t* grad;    /* [n] BF16 gradient, read only; may be NULL when only the
                                *_step_one entry points (gradient release) are used    */
} flashopt_tensor;

typedef struct flashopt_adamw_hparams {
    double lr;            /* >= 0                                  */
    double beta1;         /* [0, 1)                                */
    double beta2;         /* [0, 1)                                */
    double eps;           /* > 0, and nonzero once rounded to binary32 (> 2^-150) */
    double weight_decay;  /* >= 0, decoupled (scaled by lr)        */
} flashopt_adamw_hparams;

typedef struct flashopt_sgd_hparams {
    double lr;            /* >= 0                                  */
    double momentum;      /* [0, 1); dampening 0, no Nesterov      */
    double weight_decay;  /* >= 0, L2 added to the gradient        */
} flashopt_sgd_hparams;

/* Lion (named by the FlashOptim page as FlashLion; the update is the published
 * Lion rule): c = b1*m + c1*g, theta_n = lambda*theta_hat - lr*sign(c) with
 * sign(0) = 0, m' = b2*m + c2*g; b1 = beta1, c1 = 1-beta1, b2 = beta2,
 * c2 = 1-beta2, lambda = 1-lr*wd, each rounded once to binary32.  m is stored
 * like the AdamW momentum (phi_m, INT8, FP16 group scale). */
typedef struct flashopt_lion_hparams {
    double lr;            /* >= 0                                  */
    double beta1;         /* [0, 1): interpolation for the direction */
    double beta2;         /* [0, 1): momentum decay                 */
    double weight_decay;  /* >= 0, decoupled (scaled by lr)        */
} flashopt_lion_hparams;

typedef struct flashopt_list flashopt_list;   /* opaque; host memory owned by the library */

const char* flashopt_status_string(int status);

/* ---- flat buffers: weight split / rebuild (weight-splitting section, Eq. 1-2,
 * Alg. 1).  split: theta (FP32 [n]) -> theta' (BF16 [n]) and rho (INT8 [n]),
 * used once at optimizer construction.  unsplit: the reverse, writing the
 * rebuilt FP32 master weight (export, checkpoint conversion). */
int flashopt_split(const float* theta, int64_t n, uint16_t* theta_bf16, int8_t* rho,
                   void* stream);
int flashopt_unsplit(const uint16_t* theta_bf16, const int8_t* rho, int64_t n,
                     float* theta_out, void* stream);

/* ---- flat buffers: companded group quantisers (companding section, Alg. 2-3).
 * Import an FP32 optimizer state into the compressed form, or export it.
 * quantize_v takes the variance v itself (it applies phi_v = sqrt). */
int flashopt_quantize_m(const float* m, int64_t n, int8_t* q, uint16_t* scale, void* stream);
int flashopt_dequantize_m(const int8_t* q, const uint16_t* scale, int64_t n, float* m,
                          void* stream);
int flashopt_quantize_v(const float* v, int64_t n, uint8_t* q, uint16_t* scale, void* stream);
int flashopt_dequantize_v(const uint8_t* q, const uint16_t* scale, int64_t n, float* v,
                          void* stream);

/* ---- codec ablations over flat buffers (weight-splitting section, Fig. 3:
 * BF16 versus FP16 base and the width of the correction; companding section,
 * Fig. 4-5: linear quantisation without companding).  Not used by the step.
 * split_ex: base 0 = BF16, 1 = FP16 (RNE; beyond 65504 FP16 rounds to Inf);
 * codes rho = clamp(rne(qmax*e)) in [-qmax, qmax], 1 <= qmax <= 32767, with
 * e = (theta - theta')/h exact, h = ULP(theta')/2 above |theta'| (zero and
 * subnormal bases: the minimum-normal spacing), the product qmax*e exact;
 * rho = 0 where theta' is not finite.  unsplit_ex: theta' + (rho*RN(1/qmax))*h.
 * theta_base and rho are [n] uint16 / int16 (2-byte aligned), theta [n] FP32. */
int flashopt_split_ex(const float* theta, int64_t n, int32_t base, int32_t qmax,
                      uint16_t* theta_base, int16_t* rho, void* stream);
int flashopt_unsplit_ex(const uint16_t* theta_base, const int16_t* rho, int64_t n, int32_t base,
                        int32_t qmax, float* theta_out, void* stream);
/* Linear group quantisers: the group scale and codes of the quantisers above
 * applied to m and v themselves (no phi); both scales capped at 0x7BFF.
 * Dequantisation: m = q*(s*K8), v = q*(s*K255). */
int flashopt_quantize_lin_m(const float* m, int64_t n, int8_t* q, uint16_t* scale,
                            void* stream);
int flashopt_dequantize_lin_m(const int8_t* q, const uint16_t* scale, int64_t n, float* m,
                              void* stream);
int flashopt_quantize_lin_v(const float* v, int64_t n, uint8_t* q, uint16_t* scale,
                            void* stream);
int flashopt_dequantize_lin_v(const uint8_t* q, const uint16_t* scale, int64_t n, float* v,
                              void* stream);

/* ---- one tensor's compressed state.
 * Sizes in bytes of the code records and the scale array for n elements
 * (0 for an unknown kind or n out of range). */
size_t flashopt_codes_bytes(int32_t kind, int64_t numel);
size_t flashopt_scales_bytes(int32_t kind, int64_t numel);
/* Initialise from FP32 master weights (device [n]): theta' and rho by the split
 * (weight-splitting section, Eq. 1-2), momentum and variance codes and all
 * scales zero (m = v = 0).  _FP32 kinds: the master weight is theta itself,
 * theta' = bf16_rne(theta), m = v = 0.  t->grad is not used. */
int flashopt_tensor_init(const flashopt_tensor* t, int32_t kind, const float* theta,
                         void* stream);
/* Export to FP32 (device [n] each; any may be NULL, v ignored for SGD and
 * Lion): the rebuilt master weight theta' + (rho*K8)*h, and the dequantised
 * momentum and variance (companding section, Alg. 2-3) -- checkpoint
 * conversion.  _FP32 kinds: copies of the stored values. */
int flashopt_tensor_export(const flashopt_tensor* t, int32_t kind, float* theta, float* m,
                           float* v, void* stream);

/* ---- ragged tensor lists (a flat buffer is a list of one).
 * The list keeps a device descriptor table in a caller-provided DEVICE
 * workspace of at least flashopt_list_workspace_bytes(count) bytes (256-byte
 * aligned), which must outlive the handle.  flashopt_list_create validates
 * every descriptor, uploads the table on `stream` and waits for that copy
 * (it is a set-up call); afterwards the descriptors' pointers are fixed,
 * except the gradients (flashopt_list_set_grads).  count may be 0. */
size_t flashopt_list_workspace_bytes(int32_t count);
/* kind: FLASHOPT_KIND_ADAMW[_FP32] (steps with flashopt_adamw_step*),
 * FLASHOPT_KIND_SGD[_FP32] (flashopt_sgd_step*) or FLASHOPT_KIND_LION[_FP32]
 * (flashopt_lion_step*); a step of another optimizer returns FLASHOPT_ERR_ARG.
 * Every tensor of a list has the list's kind: a model with some layers left
 * uncompressed keeps two lists and steps both. */
int flashopt_list_create(const flashopt_tensor* tensors, int32_t count, int32_t kind,
                         void* workspace, size_t workspace_bytes, void* stream,
                         flashopt_list** out);
int flashopt_list_destroy(flashopt_list* list);
int64_t flashopt_list_numel(const flashopt_list* list);
/* grads: HOST array of `count` device pointers (entries may be NULL).  The new
 * pointers are written into the device table in stream order (kernel
 * arguments, no host staging buffer), so steps enqueued later see them. */
int flashopt_list_set_grads(flashopt_list* list, const uint16_t* const* grads, void* stream);
/* Zero the momentum and variance codes and every scale of the list (m = v = 0;
 * theta' and rho, or the FP32 master weight, are kept). */
int flashopt_state_zero(const flashopt_list* list, void* stream);

/* ---- the fused step (fused-step section, Alg. 4): ONE launch over the whole
 * list.  step is the 1-based AdamW counter t shared by all tensors of one
 * optimizer step.  The list's kind must match the step.  On an _FP32 list
 * the same update runs on the FP32 values (no dequantisation, requantisation
 * or split) and theta' = bf16_rne(theta_n) is written. */
int flashopt_adamw_step(const flashopt_list* list, const flashopt_adamw_hparams* hp,
                        int64_t step, void* stream);
int flashopt_sgd_step(const flashopt_list* list, const flashopt_sgd_hparams* hp,
                      int64_t step, void* stream);
/* Lion has no step-dependent scalar; step must still be >= 1. */
int flashopt_lion_step(const flashopt_list* list, const flashopt_lion_hparams* hp,
                       int64_t step, void* stream);

/* ---- the whole-list AdamW step for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  The same result as flashopt_list_create over `tensors`
 * (kind FLASHOPT_KIND_ADAMW, every numel > 0 tensor with a gradient) followed
 * by flashopt_adamw_step, bit for bit, with the same kernel and launch shape,
 * but no handle and no workspace: the descriptor table and tile offsets live
 * in a fixed array of the library's own device memory (each GPU the library
 * runs on holds one, about 290 KB, until the process ends), written by a few
 * small kernels on `stream` (the descriptors travel as kernel arguments) and
 * then read by the step.  Calls on one stream are ordered; calls that overlap
 * on one GPU (other streams, other host threads) share that array and race.
 * Nothing is allocated, nothing synchronises.  tensors: HOST array of `count`
 * descriptors.  Errors: FLASHOPT_ERR_SIZE (count < 0 or above
 * FLASHOPT_NOALLOC_MAX_TENSORS), FLASHOPT_ERR_NULL (tensors NULL with count > 0,
 * a missing gradient), the checks of flashopt_list_create and
 * flashopt_adamw_step, FLASHOPT_ERR_HIP (no current device, the array's address
 * not found, a launch failure). */
#define FLASHOPT_NOALLOC_MAX_TENSORS 4096
int flashopt_adamw_step_noalloc(const flashopt_tensor* tensors, int32_t count,
                                const flashopt_adamw_hparams* hp, int64_t step, void* stream);

/* ---- graph-capturable AdamW.  The step counter, the bias-correction powers
 * and the schedulable hyper-parameters live in a DEVICE struct that each call
 * advances on the stream, so the launches of one call depend on no host value
 * that changes from step to step: capture them once (HIP graphs,
 * torch.cuda.graphs) and replay every step.  Each call gives exactly the
 * results of flashopt_adamw_step with the advanced t and the struct's
 * hyper-parameters. */
typedef struct flashopt_adamw_schedule {
    double lr, eps, weight_decay;  /* read on the device by every call: write new values
                                      between calls or replays (an lr schedule); not
                                      validated there -- keep them in the ranges of
                                      flashopt_adamw_hparams                          */
    double beta1, beta2;           /* fixed at init (p1 and p2 depend on them)        */
    int64_t t;                     /* steps taken; each call first adds one           */
    double p1, p2;                 /* beta1^t, beta2^t by t successive multiplications */
    uint32_t scalars[10];          /* the step's binary32 scalars, written by each call */
    uint32_t pad[2];
} flashopt_adamw_schedule;

/* Set up a schedule (DEVICE pointer, 8-byte aligned) for a state that has taken
 * t >= 0 steps: hp validated as for flashopt_adamw_step, p1 and p2 computed on
 * the host; written by a one-thread kernel on `stream` (no copy, no wait). */
int flashopt_adamw_schedule_init(flashopt_adamw_schedule* schedule,
                                 const flashopt_adamw_hparams* hp, int64_t t, void* stream);
/* One fused AdamW step over a FLASHOPT_KIND_ADAMW list: a one-thread kernel
 * advances the schedule and forms the scalars (adam_scalars_from, the host's
 * own definition), then the step launch reads them from device memory. */
int flashopt_adamw_step_scheduled(const flashopt_list* list,
                                  flashopt_adamw_schedule* schedule, void* stream);

/* SGD and Lion have no step-dependent scalar; their schedules hold the
 * hyper-parameters on the device so that a captured graph follows an lr (or
 * momentum, beta, weight-decay) schedule written between replays.  t counts
 * the calls.  Same results as flashopt_sgd_step / flashopt_lion_step. */
typedef struct flashopt_sgd_schedule {
    double lr, momentum, weight_decay;  /* read on the device by every call; not validated there */
    int64_t t;
    uint32_t scalars[4];                /* written by each call */
} flashopt_sgd_schedule;

typedef struct flashopt_lion_schedule {
    double lr, beta1, beta2, weight_decay;  /* read on the device by every call */
    int64_t t;
    uint32_t scalars[6];                    /* written by each call */
} flashopt_lion_schedule;

int flashopt_sgd_schedule_init(flashopt_sgd_schedule* schedule, const flashopt_sgd_hparams* hp,
                               int64_t t, void* stream);
int flashopt_sgd_step_scheduled(const flashopt_list* list, flashopt_sgd_schedule* schedule,
                                void* stream);
int flashopt_lion_schedule_init(flashopt_lion_schedule* schedule,
                                const flashopt_lion_hparams* hp, int64_t t, void* stream);
int flashopt_lion_step_scheduled(const flashopt_list* list, flashopt_lion_schedule* schedule,
                                 void* stream);

/* ---- gradient release (fused-step section): step tensor `index` of the list
 * now, reading `grad` (device BF16 [numel], overriding the descriptor's
 * pointer); the caller may free or reuse grad once this launch has run.
 * Same arithmetic and results as the whole-list step. */
int flashopt_adamw_step_one(const flashopt_list* list, int32_t index, const uint16_t* grad,
                            const flashopt_adamw_hparams* hp, int64_t step, void* stream);
int flashopt_sgd_step_one(const flashopt_list* list, int32_t index, const uint16_t* grad,
                          const flashopt_sgd_hparams* hp, int64_t step, void* stream);
int flashopt_lion_step_one(const flashopt_list* list, int32_t index, const uint16_t* grad,
                           const flashopt_lion_hparams* hp, int64_t step, void* stream);

/* Bucketed gradient release (fused-step section): one launch steps the
 * consecutive tensors [first, first + count) of the list.  grads: HOST array
 * of count device BF16 gradient pointers (16-byte aligned; NULL only for
 * empty tensors), written first into the list's descriptors by a small
 * kernel on `stream`.  They serve this launch only: the caller may free or
 * reuse the gradients once it has run, and afterwards the list holds no
 * gradient for these tensors (a whole-list step returns FLASHOPT_ERR_NULL
 * until flashopt_list_set_grads gives them again).  Ranges stepped from
 * different streams must not overlap.  Same arithmetic and results as
 * the whole-list step.  Errors: FLASHOPT_ERR_INDEX for a range outside the
 * list, then the hyper-parameter, kind and gradient checks of the other
 * calls; nothing is launched on error. */
int flashopt_adamw_step_range(flashopt_list* list, int32_t first, int32_t count,
                              const uint16_t* const* grads, const flashopt_adamw_hparams* hp,
                              int64_t step, void* stream);
int flashopt_sgd_step_range(flashopt_list* list, int32_t first, int32_t count,
                            const uint16_t* const* grads, const flashopt_sgd_hparams* hp,
                            int64_t step, void* stream);
int flashopt_lion_step_range(flashopt_list* list, int32_t first, int32_t count,
                             const uint16_t* const* grads, const flashopt_lion_hparams* hp,
                             int64_t step, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* FLASHOPT_H */
