/*
 * bitlinear_measure.h -- measurement probes shipped with the BitLinear
 * library for AMD Instinct MI355X (gfx950): the two hardware ceilings the
 * forward pass of bitlinear.h is measured against, each as a plain kernel
 * doing only that one thing.  They compute nothing of the method; their
 * outputs are checksums that keep the work from being optimized away.
 *
 * Conventions as in bitlinear.h: device pointers, caller-owned buffers, the
 * library allocates nothing, every call only queues work on `stream` (a
 * hipStream_t), arguments are validated before anything is queued and the
 * return is a BITLINEAR_* status.
 */
#ifndef BITLINEAR_MEASURE_H
#define BITLINEAR_MEASURE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes of the `sink` buffer both probes write (one 32-bit checksum per
 * workgroup; host only). */
size_t bitlinear_measure_sink_bytes(void);

/*
 * HBM streaming-read ceiling: read `bytes` bytes of `buf` exactly once (four
 * wavefronts per SIMD, each streaming one contiguous run with 16-byte
 * non-temporal loads, sixteen in flight per lane), fold them with XOR and
 * write one word per workgroup to `sink`.  Achieved bandwidth = bytes /
 * kernel time.
 *   buf    16-byte aligned device buffer (in); bytes a multiple of 16, > 0
 *   sink   bitlinear_measure_sink_bytes() bytes (out)
 * BITLINEAR_EINVAL for a null or misaligned pointer or a bad size.
 */
int bitlinear_measure_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);

/*
 * int8 matrix-core ceiling: two workgroups of four wavefronts per CU, each
 * wavefront issuing `iters` rounds of eight independent
 * v_mfma_i32_32x32x32_i8 (four accumulators, the tiling of the prefill
 * kernel's 64 x 64 wave tile) with nothing else in the loop.  The operands
 * are real data, so that the matrix cores toggle as many bits as in the
 * forward pass: A fragments from `xq` (int8 activations) and B fragments
 * expanded from `packed` (2-bit codes, field j of a word = (w >> 2j) & 3, as
 * the prefill kernel feeds them).  Int8 ops per call =
 * bitlinear_measure_mfma_ops(iters), for the workgroup count this device gets.
 *   xq      at least 8 KB of int8 data (in); packed at least 2 KB (in)
 *   iters   rounds per wavefront, 1 .. 2^24
 *   sink    bitlinear_measure_sink_bytes() bytes (out)
 * BITLINEAR_EINVAL for a null pointer or iters out of range.
 */
int bitlinear_measure_mfma_i8(const int8_t* xq, const uint8_t* packed, int32_t iters, int32_t* sink,
                              void* stream);

/* Int8 ops one bitlinear_measure_mfma_i8 call performs on the current device
 * (host only; 0 for iters out of range). */
double bitlinear_measure_mfma_ops(int32_t iters);

#ifdef __cplusplus
}
#endif

#endif /* BITLINEAR_MEASURE_H */
