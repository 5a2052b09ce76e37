/*
 * flashopt_probe.h -- measurement aids for the fused steps of flashopt.h.
 *
 * The fused-step section of "FlashOptim: Optimizers for Memory Efficient
 * Training" (digest page, "Core method > Fused optimizer step", Alg. 4) fuses
 * the whole update into one pass so that it costs no more memory traffic than
 * a standard optimizer step: the step is meant to be bound by HBM bandwidth.
 * These probes measure that bound: for the step's own access pattern, for
 * the best pattern of the step's byte mix, and for plain streams.
 */
#ifndef FLASHOPT_PROBE_H
#define FLASHOPT_PROBE_H

#include "flashopt.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Moves exactly the bytes the list's step (flashopt_adamw_step,
 * flashopt_sgd_step or flashopt_lion_step, by the list's kind) moves for
 * `list` -- the same tiles, launch shape, loads and stores (12.25 bytes per
 * element for AdamW, 10.125 for SGD and Lion, plus the partial-group scales)
 * -- with the arithmetic replaced by one XOR per word:
 *   theta' ^= grad (16-bit words);
 *   AdamW: rho ^= m_code, m_code ^= v_code, v_code ^= rho (bytes; right-hand
 *          sides are the values read), m_scale ^= 1, v_scale ^= 1;
 *   SGD, Lion: rho ^= m_code, m_code = ~m_code, m_scale ^= 1 (every group).
 * DESTRUCTIVE: the state then holds meaningless bits (any bits may be probed,
 * the contents do not change the traffic).  Requirements and errors as the
 * step (a gradient on every tensor: FLASHOPT_ERR_NULL otherwise); the _FP32
 * kinds: FLASHOPT_ERR_ARG.  One launch on `stream`, nothing allocated, no
 * synchronisation. */
int flashopt_stream_probe(const flashopt_list* list, void* stream);

/* The practical ceiling of the AdamW step's traffic: the same bytes per
 * parameter (read 7.125, write 5.125) over the same four read and three
 * written streams, in place like the step, but over flat buffers with the
 * best access pattern the byte mix allows (every load and store a fully
 * coalesced 16 bytes per lane with the non-temporal hint; a wave loads one
 * 2048-parameter tile, then stores it).  Over n parameters (n a multiple of
 * 2048):
 *   theta   uint16[n]           theta ^= grad            (read and written)
 *   grad    uint16[n]           read only
 *   codes   uint8[3n]           every byte ^= 0x5A       (read and written)
 *   scales  uint16[n/16]        every 16-bit word ^= 1   (read and written)
 * (3n code bytes: rho, m and v codes; n/16 scale words: two FP16 per group
 * of 32).  DESTRUCTIVE.  Errors: FLASHOPT_ERR_SIZE (n < 0 or not a multiple
 * of 2048), FLASHOPT_ERR_NULL, FLASHOPT_ERR_ALIGN (any pointer not 16-byte
 * aligned).  One launch on `stream`, nothing allocated, no synchronisation. */
int flashopt_mix_ceiling(uint16_t* theta, const uint16_t* grad, uint8_t* codes, uint16_t* scales,
                         int64_t n, void* stream);

/* The step's traffic over the same flat buffers as flashopt_mix_ceiling
 * (theta 2n, grad 2n, codes 3n, scales n/8 bytes; n a multiple of 2048; one
 * wave per 2048-parameter tile of four 512-parameter sub-tiles, lane l owning
 * parameters [8l, 8l+8) of a sub-tile), with one of the access patterns the
 * fused kernel could use -- to tell the pattern's cost from the byte mix's:
 *   (theta' and the gradient carry the non-temporal hint in every variant, as
 *   in the fused kernel; variant 2's DMA loads do not)
 *   variant 0: the fused kernel's own: theta' and gradient 16 bytes per lane,
 *              the codes of a lane's 8 parameters as three 8-byte runs, one
 *              in each 512-byte plane of the sub-tile's 1536 code bytes, all
 *              hinted non-temporal, the group's 4-byte scale pair from one
 *              lane of four, two register buffers (sub-tile k+2 loaded once k
 *              is stored);
 *   variant 1: as 0 with the 1536 code bytes of a sub-tile as 16-byte units
 *              (not hinted) and the 64 scale bytes as 16 lanes x 4 bytes;
 *   variant 2: the units of 1 loaded by global-to-LDS DMA into a two-slot ring
 *              per wave (no register holds a load in flight);
 *   variant 3: as 0 with three register buffers (the loads of sub-tile k+2
 *              issued before sub-tile k is stored);
 *   variant 4: as 0 with the tiles taken in a hashed order (wave w takes tile
 *              w * q mod ntiles, q a prime near 10^6 that does not divide
 *              ntiles), so the tiles in flight are spread over the buffers;
 *   variant 5: as 0 with a lane's codes as one interleaved 24-byte record
 *              (bytes [24l, 24l+24) of the sub-tile's 1536) taken as three
 *              8-byte accesses without the hint: the fused kernel's earlier
 *              layout.
 * Results: theta ^= grad; codes: variants 0, 3, 4 and 5 replace each lane's
 * three 8-byte code words (a, b, c) -- at 8l, 512 + 8l and 1024 + 8l of each
 * 1536-byte sub-tile block for 0, 3 and 4, at 24l, 24l + 8 and 24l + 16 for 5
 * -- with (a^b, b^c, c^a), variants 1 and 2 XOR every code byte with 0x5A;
 * every 32-bit scale word ^= 0x00010001.  DESTRUCTIVE.  Errors:
 * FLASHOPT_ERR_ARG (variant outside 0-5) and those of flashopt_mix_ceiling.
 * One launch on `stream`, nothing allocated. */
int flashopt_pattern_probe(int32_t variant, uint16_t* theta, const uint16_t* grad,
                           uint8_t* codes, uint16_t* scales, int64_t n, void* stream);

/* Stream-count sweep: `nread` device buffers read and `nwrite` written, each
 * of `bytes` bytes (a multiple of 16), one 16-byte unit of each per thread.
 * Written value: the XOR of the units read, its first word XORed with the
 * written buffer's index w (so buffer w holds the XOR of the read buffers
 * with w in every fourth word); with nwrite = 0 nothing is written.
 * in_place != 0: the written buffers are reads[0 .. nwrite-1] (nwrite <=
 * nread) and `writes` is ignored; else writes[0 .. nwrite-1].  (nread,
 * nwrite) must be one of (1,0) (0,1) (1,1) (2,1) (1,2) (2,2) (3,2) (4,3)
 * (7,5) (4,0) (0,4), else FLASHOPT_ERR_ARG.  Host arrays of device
 * pointers; buffers 16-byte aligned (FLASHOPT_ERR_ALIGN) and non-NULL
 * (FLASHOPT_ERR_NULL).  One launch on `stream`, nothing allocated. */
int flashopt_stream_sweep(int32_t nread, int32_t nwrite, const void* const* reads,
                          void* const* writes, int32_t in_place, int64_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FLASHOPT_PROBE_H */
