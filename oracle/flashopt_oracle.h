/*
 * CPU oracle for FlashOptim's compressed optimizer step -- TEST INFRASTRUCTURE.
 * Declarations of oracle/flashopt_oracle.c.  This header belongs to the
 * oracle alone; the HIP library never includes it.
 *
 * All arrays are host memory owned by the caller.  Group size is 32; a tensor
 * of n elements has ceil(n/32) scales, the last group possibly partial.
 */
#ifndef FLASHOPT_ORACLE_H
#define FLASHOPT_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int orc_env_ok(void);  /* 1 if round-to-nearest and subnormals are in effect */

uint16_t orc_bf16_rne(float x);
float orc_bf16_to_f32(uint16_t b);
uint16_t orc_f16_rne(float x);
float orc_f16_to_f32(uint16_t h);

/* weight split / rebuild with INT8 codes (qmax = 127) */
void orc_split(const float* theta, int64_t n, uint16_t* tb, int8_t* rho);
void orc_unsplit(const uint16_t* tb, const int8_t* rho, int64_t n, float* out);
/* same algorithm with a general code range [-qmax, qmax] (b-bit: qmax = 2^(b-1)-1) */
void orc_split_q(const float* theta, int64_t n, int32_t qmax, uint16_t* tb, int32_t* rho);
void orc_unsplit_q(const uint16_t* tb, const int32_t* rho, int64_t n, int32_t qmax, float* out);

/* the same algorithm on an FP16 base weight (ablation: the weight-splitting
 * part compares BF16 and FP16 bases, Fig. 3) */
void orc_split_f16_q(const float* theta, int64_t n, int32_t qmax, uint16_t* hb, int32_t* rho);
void orc_unsplit_f16_q(const uint16_t* hb, const int32_t* rho, int64_t n, int32_t qmax,
                       float* out);

float orc_phi_m(float x);
float orc_phi_m_inv(float z);
float orc_phi_v(float x);
float orc_phi_v_inv(float z);

void orc_quant_m(const float* m, int64_t n, int8_t* q, uint16_t* s);
void orc_dequant_m(const int8_t* q, const uint16_t* s, int64_t n, float* m);
void orc_quant_v(const float* v, int64_t n, uint8_t* q, uint16_t* s);
void orc_dequant_v(const uint8_t* q, const uint16_t* s, int64_t n, float* v);

/* linear group quantisers without companding (ablation, Fig. 4-5): the same
 * group scale and codes applied to m and v themselves; both scales may reach
 * the largest finite FP16 */
void orc_quant_lin_m(const float* m, int64_t n, int8_t* q, uint16_t* s);
void orc_dequant_lin_m(const int8_t* q, const uint16_t* s, int64_t n, float* m);
void orc_quant_lin_v(const float* v, int64_t n, uint8_t* q, uint16_t* s);
void orc_dequant_lin_v(const uint8_t* q, const uint16_t* s, int64_t n, float* v);

/* out = {b1, c1, b2, c2, alpha, kappa, eps, lambda} */
void orc_adamw_scalars(double lr, double beta1, double beta2, double eps, double wd,
                       int64_t t, float out[8]);

/* One fused step over one tensor, in place.  theta_out / m_out / v_out
 * (nullable) receive the fp32 values before requantisation and re-split. */
void orc_adamw_step(int64_t n, uint16_t* tb, int8_t* rho, int8_t* qm, uint16_t* sm,
                    uint8_t* qv, uint16_t* sv, const uint16_t* grad,
                    double lr, double beta1, double beta2, double eps, double wd, int64_t t,
                    float* theta_out, float* m_out, float* v_out);
void orc_sgd_step(int64_t n, uint16_t* tb, int8_t* rho, int8_t* qb, uint16_t* sb,
                  const uint16_t* grad, double lr, double momentum, double wd, int64_t t,
                  float* theta_out, float* b_out);

/* Lion with the compressed single momentum (one scale per group): sign update
 * of the interpolated momentum, decoupled weight decay.  theta_out / m_out
 * (nullable) receive theta_new and m_new before requantisation and re-split. */
void orc_lion_step(int64_t n, uint16_t* tb, int8_t* rho, int8_t* qm, uint16_t* sm,
                   const uint16_t* grad, double lr, double beta1, double beta2, double wd,
                   float* theta_out, float* m_out);

void orc_bf16_rne_array(const float* x, int64_t n, uint16_t* out);
void orc_f16_rne_array(const float* x, int64_t n, uint16_t* out);
void orc_f16_to_f32_array(const uint16_t* h, int64_t n, float* out);
void orc_phi_m_array(const float* x, int64_t n, float* out);
void orc_phi_m_inv_array(const float* z, int64_t n, float* out);
void orc_phi_v_array(const float* x, int64_t n, float* out);
void orc_phi_v_inv_array(const float* z, int64_t n, float* out);

/* The AdamW step with the variance stored by the linear quantiser (no
 * companding; the ablation of the companding section, Fig. 5). */
void orc_adamw_step_linv(int64_t n, uint16_t* tb, int8_t* rho, int8_t* qm, uint16_t* sm,
                         uint8_t* qv, uint16_t* sv, const uint16_t* grad,
                         double lr, double beta1, double beta2, double eps, double wd, int64_t t,
                         float* theta_out, float* m_out, float* v_out);

/* Compression disabled for a tensor: FP32 master weight and moments, the
 * same updates, theta' = bf16_rne(theta_n) written to tb. */
void orc_adamw_step_fp32(int64_t n, float* theta, float* m, float* v, uint16_t* tb,
                         const uint16_t* grad, double lr, double beta1, double beta2,
                         double eps, double wd, int64_t t);
void orc_sgd_step_fp32(int64_t n, float* theta, float* b, uint16_t* tb, const uint16_t* grad,
                       double lr, double momentum, double wd);
void orc_lion_step_fp32(int64_t n, float* theta, float* m, uint16_t* tb, const uint16_t* grad,
                        double lr, double beta1, double beta2, double wd);

#ifdef __cplusplus
}
#endif
#endif
