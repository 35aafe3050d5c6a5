/*
 * Measurement probes of libqlora: kernels whose work is known exactly, for
 * re-measuring on the machine itself the peaks that the layer's kernels are
 * judged against (dense matrix-core throughput, HBM streaming bandwidth) and
 * the cost of a launch. They compute nothing of the layer; benchmarks time
 * them with events on `stream` around the call.
 *
 * Conventions: device pointers, owned by the caller; nothing is allocated
 * or synchronized; a pending HIP error of the caller makes a call return 5
 * without launching. Returns 0 on success, 1 on a bad argument, 5 when the
 * runtime rejects the launch (the qlora_status values of qlora.h).
 */
#ifndef QLORA_PROBE_H
#define QLORA_PROBE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { QLORA_PROBE_BF16 = 0, QLORA_PROBE_I8 = 1 };

/* `blocks` blocks of four waves; each wave issues `iters` rounds of eight
 * independent dense MFMAs (v_mfma_f32_16x16x32_bf16 for QLORA_PROBE_BF16,
 * v_mfma_i32_16x16x64_i8 for QLORA_PROBE_I8). *ops receives the operations
 * (two per multiply-add) one launch performs. out: float32 [blocks * 256]
 * (one value per thread, so that no product is dropped). */
int qlora_probe_mfma(int kind, int blocks, int iters, void* out, void* stream,
                     double* ops);

/* Streaming copy of `bytes` (a multiple of 16384) from src to dst with
 * 16-byte loads and stores, `blocks` blocks of 256 threads. */
int qlora_probe_copy(const void* src, void* dst, size_t bytes, int blocks, void* stream);

/* Read-only stream over `bytes` (a multiple of 16384) of src; out receives
 * 16 bytes per thread (blocks * 256 * 16 bytes). */
int qlora_probe_read(const void* src, size_t bytes, int blocks, void* out, void* stream);

/* A kernel that does nothing: blocks x threads (threads <= 1024). */
int qlora_probe_empty(int blocks, int threads, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_PROBE_H */
