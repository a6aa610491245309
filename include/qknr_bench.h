/*
 * qknr_bench.h -- measurement helpers of the QK-Norm + RoPE benchmark (not part
 * of the operation; libqknr_bench.so).
 *
 * Plain streaming kernels that measure the achievable HBM bandwidth of one read
 * and one write stream (a copy) or of two reads and one write (the shape of the
 * backward's traffic), an empty kernel (the cost of a dispatch), and a fill that
 * evicts other data from L2 and the Infinity Cache between timed launches.  All calls are asynchronous on
 * `stream` (a hipStream_t, NULL for the default stream); buffers are device
 * memory the caller owns, 16-byte aligned, and `bytes` a multiple of 16.
 * Return values: 0 ok (also for bytes == 0, a no-op), 1 a null pointer,
 * 3 misaligned pointer or size, 5 a failed launch.
 */
#ifndef QKNR_BENCH_H
#define QKNR_BENCH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    QKNR_BENCH_OK = 0,
    QKNR_BENCH_ERR_INVALID_ARG = 1,
    QKNR_BENCH_ERR_MISALIGNED = 3,
    QKNR_BENCH_ERR_HIP = 5
};

/* dst[i] = src[i] for `bytes` bytes. */
int qknr_bench_copy(const void *src, void *dst, size_t bytes, void *stream);

/* dst[i] = a[i] ^ b[i] for `bytes` bytes (two reads, one write). */
int qknr_bench_stream2(const void *a, const void *b, void *dst, size_t bytes, void *stream);

/* Launches a kernel of one 64-thread workgroup that does nothing: the cost of
 * a dispatch, the floor under any kernel's duration. */
int qknr_bench_empty(void *stream);

/* Writes `bytes` bytes of a counter pattern (16-byte chunk i holds i ^ seed,
 * then +1, +2, +3 in its other words) into buf. */
int qknr_bench_flush(void *buf, size_t bytes, uint32_t seed, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QKNR_BENCH_H */
