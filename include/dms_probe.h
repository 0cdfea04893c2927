/*
 * dms_probe.h — machine-rate probes for the MI355X (gfx950) figures the DMS
 * kernels are measured against: HBM streaming-read bandwidth (decode
 * attention is bound by it: the pages put decode cost in the reading of the
 * KV cache, the FastDMS post's decode tables and the walkthrough's 为什么需要
 * DMS) and the dense bf16 matrix-core rate (chunked prefill attention, a
 * dense contraction per chunk: walkthrough, 高级选项 Chunked Prefill).
 *
 * libdms_probe.so; no DMS arithmetic.  Asynchronous on `stream` (a
 * hipStream_t as void*); the caller times the calls (events on that stream).
 * Returns 0, -1 for a bad argument (nothing launched), -5 for a launch error.
 */
#ifndef DMS_PROBE_H
#define DMS_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads dms_probe_read_bytes(bytes, grid, unroll) bytes of the device buffer
 * `buf` (16-byte aligned) once, with `grid` workgroups of 256 threads, each
 * thread keeping `unroll` (4, 8 or 16) 16-byte non-temporal loads in flight;
 * writes nothing to `sink` (device, >= grid words) in practice. */
int dms_probe_read(const void* buf, size_t bytes, int grid, int unroll, uint32_t* sink, void* stream);

/* Bytes dms_probe_read actually reads (rounded down to whole rounds). */
size_t dms_probe_read_bytes(size_t bytes, int grid, int unroll);

/* `grid` workgroups of 4 waves; each wave runs `iters` rounds of 8 independent
 * 16x16x32 bf16 matrix products with fp32 accumulation (register operands). */
int dms_probe_mfma_bf16(int grid, int iters, uint32_t* sink, void* stream);

/* Flops one dms_probe_mfma_bf16 call performs. */
double dms_probe_mfma_bf16_flops(int grid, int iters);

#ifdef __cplusplus
}
#endif

#endif /* DMS_PROBE_H */
