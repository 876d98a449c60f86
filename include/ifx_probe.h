/*
 * ifx_probe.h -- practical-ceiling probes of the device (part of libifx.so).
 *
 * Not part of the convolution path: these kernels measure what the device
 * reaches at all, so a measurement can report each convolution kernel both
 * against the published peaks (HBM 8 TB/s, dense int8 MFMA 5.0 POP/s) and
 * against what a plain kernel attains on the same box.  The pages time their
 * fused kernels against the memory and tensor-core limits of their GPUs
 * (Inspur conv-merge article, section 4); these probes give the MI355X
 * counterparts.  Return values are ifx_status codes (ifx.h): 0 ok, 1 null,
 * 2 bad size, 4 misaligned, 6 HIP launch failure.
 */
#ifndef IFX_PROBE_H
#define IFX_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Copy `bytes` (a multiple of 16) from src to dst, DEVICE pointers, 16-byte
 * aligned, not overlapping: 16-byte non-temporal vector loads and stores in a
 * grid-stride loop over at most 64 workgroups of 256 threads per CU.  Moves
 * 2 * bytes through HBM.  Enqueued on `stream` (hipStream_t as void*).
 */
int32_t ifx_probe_copy(const void *src, void *dst, size_t bytes, void *stream);

/*
 * `blocks` workgroups of four waves, each wave running `iters` rounds of a
 * 4 x 4 tile of independent v_mfma_i32_16x16x64_i8 (16 x 16 x 64 int8
 * products, 32768 ops each) on register operands, then writing one int32 per
 * wave to out (DEVICE, blocks * 4 elements).
 * Ops = blocks * 4 * iters * 16 * 32768.
 */
int32_t ifx_probe_mfma_i8(int32_t *out, int32_t blocks, int32_t iters, void *stream);

/*
 * The same with operands that change from one MFMA to the next: four sets of
 * random operand bits per lane (an integer hash of the lane and a counter),
 * cycled, so every instruction multiplies fresh bytes as a contraction's MFMAs
 * do (the matrix pipe's power, and with it its clock, depends on how many
 * operand bits toggle).  out: DEVICE, blocks * 4 elements.
 * Ops = blocks * 4 * iters * 4 * 16 * 32768.
 */
int32_t ifx_probe_mfma_i8_data(int32_t *out, int32_t blocks, int32_t iters, void *stream);

/*
 * Buffer->LDS DMA rate: `blocks` workgroups of four waves, each wave running
 * `iters` rounds of 8 DMAs of one contiguous 1 KB run each (16 bytes per lane)
 * from src into its own LDS, waiting for them at the end of the round -- the
 * way the convolution kernels stage their operands.  src is a DEVICE buffer of
 * `bytes` (a multiple of 1024, at most 2^31 - 1), 16-byte aligned; the runs
 * cycle through it, so a buffer that fits the L2 is read from L2.  Writes one
 * int32 per wave to out (DEVICE, blocks * 4 elements).
 * Bytes moved = blocks * 4 * iters * 8192.
 */
int32_t ifx_probe_dma_lds(const void *src, size_t bytes, int32_t blocks, int32_t iters, int32_t *out,
                          void *stream);

/*
 * LDS read rate of one lane pattern: `blocks` workgroups of four waves, each
 * wave running `iters` rounds of 8 independent ds_read_b128, lane l reading the
 * 16 bytes at LDS byte offset offsets[l] (+ j KB; offsets is a DEVICE array of
 * 64 int32, taken modulo 16 KB and rounded down to 16 bytes).  Bank conflicts
 * of the pattern show as a lower rate.  out: DEVICE, `blocks` int32 (written
 * only in a case that does not occur; it keeps the reads live).
 * Bytes read = blocks * 4 * iters * 8 * 1024.
 */
int32_t ifx_probe_lds_read(const int32_t *offsets, int32_t blocks, int32_t iters, int32_t *out, void *stream);

/*
 * VALU issue rate of one operation pair: `blocks` workgroups of four waves,
 * each lane running `iters` rounds of 8 independent chains of
 *   kind 0: v_mad_i64_i32 + an arithmetic shift of the high word (the
 *           fixed-point requantisation core of the fused epilogue),
 *   kind 1: an integer add + an xor (plain full-rate integer work),
 *   kind 2: int32 -> f64, an f64 fused multiply-add, f64 -> int32 (an exact
 *           double-precision form of the same requantisation, for comparison).
 * out: DEVICE, `blocks` int32 (written only for an impossible value).
 * Chain steps = blocks * 256 * iters * 8.
 */
int32_t ifx_probe_valu(int32_t kind, int32_t *out, int32_t blocks, int32_t iters, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* IFX_PROBE_H */
