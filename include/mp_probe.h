/*
 * libmp_probe — measurement probes for MI355X (gfx950), beside libmp.
 *
 * Not part of the method: these kernels measure the denominators its hot
 * path is judged against. The pages call point-wise operations and weight
 * updates bandwidth- or latency-limited and the dot products arithmetic-
 * limited ("Mixed Precision Training", long-form analysis page, §3.4 "FP16
 * Arithmetic with FP32 Accumulation" and §6.1 "Speedup Claims"); the
 * probes give the achievable HBM stream rates (read only, write only, and
 * the 1:1 read/write mix of the optimizer sweep) and the shader clock and
 * binary16 MFMA rate under a matrix-core load (constant or random operands),
 * next to the datasheet peaks.
 *
 * Same conventions as mp.h: device pointers unless stated, `stream` is a
 * hipStream_t passed as void*, every call is asynchronous on it, argument
 * errors are returned as mp_status before anything is launched.
 */
#ifndef MP_PROBE_H
#define MP_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include "mp.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MP_PROBE_READ = 0,      /* read `bytes` of src; one 4-byte word per block to dst     */
    MP_PROBE_WRITE = 1,     /* write `bytes` of a constant pattern to dst                 */
    MP_PROBE_COPY = 2       /* copy `bytes` from src to dst (one read, one write)         */
} mp_probe_mode;

/* Streams `bytes` (a positive multiple of 4096, both buffers 16-byte
 * aligned, not overlapping) through HBM in mode `mode` with 16-byte vector
 * accesses, four in flight per lane. blocks = 0: one 256-thread block per
 * 16 KiB; blocks > 0: that many blocks walk the buffer with a grid stride.
 * nontemporal != 0 marks the loads and stores non-temporal. In READ mode dst
 * receives one word per block (the XOR of what the block read), so dst must
 * hold 4 * (number of blocks) bytes; in the other modes dst holds `bytes`.
 * Errors: MP_ERR_INVALID_ARGUMENT (unknown mode, bad size or alignment, a null
 * pointer the mode needs), MP_ERR_HIP. */
mp_status mp_probe_hbm(int32_t mode, const void* src, void* dst, size_t bytes, int32_t blocks,
                       int32_t nontemporal, mp_stream stream);

typedef enum {
    MP_PROBE_OPERANDS_CONSTANT = 0,  /* every MFMA takes the same few small multiples of 2^-8   */
    MP_PROBE_OPERANDS_RANDOM = 1     /* random binary16 (sign, mantissa; exponent 2^-3..2^0),
                                        sixteen different registers per wave in rotation       */
} mp_probe_operands;

typedef enum {
    MP_PROBE_MFMA_32X32X16 = 0,      /* v_mfma_f32_32x32x16_f16, eight accumulator chains per wave  */
    MP_PROBE_MFMA_16X16X32 = 1       /* v_mfma_f32_16x16x32_f16 (the GEMMs' form), sixteen chains   */
} mp_probe_mfma_shape;

/* Runs `blocks` blocks of four waves; every wave issues `iters` rounds of
 * 16 * 32768 FLOP of binary16 MFMAs with FP32 sums, of the form `shape`, on
 * independent chains, with operands of the kind `operands`. The matrix
 * cores' power draw, and so the clock the chip holds, depends on the MFMA
 * form and on how many operand bits change between MFMAs: the CONSTANT load
 * shows the clock ceiling, the RANDOM load the MFMA rate the chip sustains on
 * data like a GEMM's. Wave 0 of each block records its shader clock counter
 * (s_memtime) and the constant-rate counter (s_memrealtime) before and after
 * the loop: out[4 b + 0..3] = {clock start, clock end, real start, real end}
 * (device uint64, 4 * blocks entries). *realtime_khz (host) receives the
 * constant counter's rate. The shader clock in MHz under this load is
 * (clock end - start) / (real end - start) * realtime_khz / 1000.
 * Errors: MP_ERR_INVALID_ARGUMENT (blocks < 1, iters < 1, unknown operand
 * kind or shape, null pointers), MP_ERR_HIP. */
mp_status mp_probe_mfma_clock(int32_t blocks, int32_t iters, int32_t operands, int32_t shape, uint64_t* out,
                              int32_t* realtime_khz, mp_stream stream);

#ifdef __cplusplus
}
#endif
#endif
