/*
 * moe_bench.h -- measurement utilities that sit beside the MoE decode layer in the
 * same library.  They compute nothing of the layer; a benchmark uses them to state
 * what the layer's numbers are measured against, as the SM120 page ("Frontier MoE on
 * consumer Blackwell (SM120)", section "SM120 decode kernels") states the HBM floor
 * and the cold-cache rotation its decode-kernel figures are taken with:
 *   * the HBM read-stream ceiling of this device (the bandwidth a plain streaming
 *     read reaches, beside the 8 TB/s specification);
 *   * a write pass over a large buffer, which evicts the Infinity Cache and the L2
 *     before a cold measurement;
 *   * an empty kernel, whose back-to-back launches give the per-launch floor.
 * All pointers are device memory owned by the caller; `stream` is a hipStream_t as
 * void* (NULL = default stream).  Work is enqueued asynchronously; every function
 * returns 0 (MOE_OK) or MOE_ERR_INVALID_ARG / MOE_ERR_LAUNCH.
 */
#ifndef MOE_BENCH_H
#define MOE_BENCH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` (a positive multiple of 64 KiB, 16-byte aligned) of `buf` once with
 * 16-byte non-temporal loads from a grid of 4 workgroups per compute unit.  `sink`
 * (4 bytes, device) is written only if the data XOR to a value that never occurs in a
 * filled buffer, so the loads cannot be dropped.                                   */
int moe_bench_read_stream(const void* buf, size_t bytes, unsigned* sink, void* stream);

/* Writes `value` to every 4-byte word of `buf` (`bytes` a positive multiple of 16). */
int moe_bench_fill(void* buf, size_t bytes, unsigned value, void* stream);

/* One launch of an empty kernel of `workgroups` workgroups of 256 threads.          */
int moe_bench_empty(int workgroups, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_BENCH_H */
