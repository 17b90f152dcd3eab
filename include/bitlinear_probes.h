/*
 * bitlinear_probes.h -- C ABI of libbitlinear_probes.so: two measurement
 * kernels that give the achievable ceilings of the two bounds of the
 * BitLinear forward pass (bitlinear.h) on the GPU they run on:
 *
 *  - a streaming read of device memory: the decode contraction reads every
 *    packed weight byte once, so its bound is how fast memory can be read;
 *  - a loop of int8 matrix-core operations (v_mfma_i32_32x32x32_i8) on
 *    operands held in registers: the prefill contraction's bound.
 *
 * Nothing on the forward path calls them; they live in their own library.
 *
 * Conventions (as in bitlinear.h): pointers are DEVICE pointers owned by
 * the caller; work is only enqueued on `stream` (a hipStream_t, NULL = the
 * default stream); arguments are checked on the host before anything is
 * enqueued.  Return value: 0 = enqueued, 1 = invalid argument (nothing
 * enqueued), 5 = launch failed.
 */
#ifndef BITLINEAR_PROBES_H
#define BITLINEAR_PROBES_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Words of the stream-read probe's result array. */
#define BLPROBE_SINK_WORDS 256

/* Reads `bytes` bytes from `buf` (16-byte aligned, bytes a positive multiple
 * of 16) once, with 16-byte vector loads in a grid-stride loop over the whole
 * chip.  XORs every 32-bit word of the buffer into sink[0 ..
 * BLPROBE_SINK_WORDS) (int32s the caller zeroes beforehand; the XOR of those
 * words is the XOR of the buffer's words), so the result can be checked and
 * no load can be dropped.  Bytes moved: `bytes`. */
int blprobe_stream_read(const void* buf, int64_t bytes, int32_t* sink, void* stream);

/* `workgroups` workgroups of 256 threads (four waves) each run `iters`
 * rounds of eight independent v_mfma_i32_32x32x32_i8 per wave on operands
 * held in registers.  pattern 0: every operand byte is 1.  pattern 1: two
 * operand sets, alternating from one operation to the next, with
 * pseudo-random activation-like bytes (-127..127) for the first operand and
 * weight-code-like bytes (0..2) for the second, as in the prefill GEMM.
 * Thread t writes the sum of its 128 accumulator values to sink[t]
 * (workgroups * 256 int32); with pattern 0 that is 4096 * iters.
 * int8 operations: 65536 * 8 * iters * 4 * workgroups.
 * 1 <= workgroups <= 2^20, 1 <= iters <= 2^16. */
int blprobe_mfma_i8(int64_t workgroups, int32_t iters, int32_t pattern, int32_t* sink,
                    void* stream);

/* The lookup-table alternative to the decode contraction, for one token row
 * (M = 1): acc[n] = sum_k q[k] * u[n][k], like bitlinear_forward_acc, with a
 * per-workgroup LDS table of the 16 partial sums of every pair of activation
 * codes indexed by 4 bits of packed weights (the T-MAC idea the GeekNews
 * page on bitnet.cpp names); a workgroup covers 64 rows and 2048 weights of
 * each, the parts' sums are added atomically.  q: [K] int8; tiled: the
 * weights in the 16-row tiled layout of bitlinear.h; acc: [N] int32
 * (written; two kernels: clearing, then the contraction).  N % 16 == 0,
 * 256 <= K <= 8192, K % 256 == 0, pointers 16-byte aligned.  It exists to be
 * measured against the matrix-core decode; the library does not use it. */
int blprobe_lut_decode_acc(const int8_t* q, int64_t k, const uint8_t* tiled, int64_t n,
                           int32_t* acc, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BITLINEAR_PROBES_H */
