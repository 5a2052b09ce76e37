/*
 * flashopt_probe.h -- measurement aid for the fused AdamW step of flashopt.h.
 *
 * The fused-step section of "FlashOptim: Optimizers for Memory Efficient
 * Training" (digest page, "Core method > Fused optimizer step", Alg. 4) fuses
 * the whole update into one pass so that it costs no more memory traffic than
 * a standard optimizer step: the step is meant to be bound by HBM bandwidth.
 * This probe measures that bound for the step's own access pattern.
 */
#ifndef FLASHOPT_PROBE_H
#define FLASHOPT_PROBE_H

#include "flashopt.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Moves exactly the bytes flashopt_adamw_step moves for `list` -- the same
 * tiles, launch shape, loads and stores (12.25 bytes per element plus the
 * partial-group scales) -- with the arithmetic replaced by one XOR per word:
 *   theta' ^= grad (16-bit words), rho ^= m_code, m_code ^= v_code,
 *   v_code ^= rho (bytes; right-hand sides are the values read), and
 *   m_scale ^= 1, v_scale ^= 1 (every group).
 * DESTRUCTIVE: the state then holds meaningless bits.  Requirements and
 * errors as flashopt_adamw_step (v_code / v_scale and a gradient on every
 * tensor: FLASHOPT_ERR_ARG / FLASHOPT_ERR_NULL otherwise); one launch on
 * `stream`, nothing allocated, no synchronisation. */
int flashopt_stream_probe(const flashopt_list* list, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FLASHOPT_PROBE_H */
