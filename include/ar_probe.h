/*
 * ar_probe.h -- C ABI of libar_probe.so: memory-traffic ceilings for the access
 * pattern of an Allreduce over P rank buffers in one GPU's HBM. Measurement
 * only: nothing here combines values, and the Allreduce library does not use it.
 *
 * The metric of the Allreduce library counts every input read once and every
 * output written once (2 P n elt bytes). Its direct kernel reads the P buffers
 * at one element offset and writes all P back: 2P concurrent streams. The probe
 * kernels move exactly those bytes with no arithmetic, so their bandwidth bounds
 * what any schedule's one-pass kernel can reach on the same buffers:
 *
 *  AR_PROBE_STREAMS  one launch reads every bufs[p] and writes it back unchanged
 *                    (in place, 2P streams of `bytes` each way per rank). Element
 *                    offsets are laid out like the direct kernel's: a thread takes
 *                    `vectors_per_thread` 16-byte vectors per rank, block-
 *                    interleaved so every wave-level access covers 1 KB. For 7 and
 *                    8 ranks the kernel is compiled for P and loads every rank
 *                    before any store; other P go 8 ranks at a time (load 8,
 *                    store 8). Bytes moved: 2 P bytes.
 *  AR_PROBE_COPY     bufs[1] = bufs[0] over `bytes` (P must be 2): one read and
 *                    one write stream. Bytes moved: 2 bytes.
 *  AR_PROBE_FOLD     the smallest one-pass Allreduce kernel: the fp32 sum of the
 *                    P ranks (P = 7 or 8, compiled for P) written back to every
 *                    rank, every load before any store, with no work items and
 *                    no rank table: the 2P streams of the direct kernel without
 *                    the library's generality. Bytes moved: 2 P bytes. Its
 *                    results are sums, not the ranks' data.
 *
 * Arguments: bufs is a host array of P device pointers, each 16-byte aligned and
 * holding at least `bytes` bytes; `bytes` must be a positive multiple of 16.
 * vectors_per_thread is 1, 2 or 4. stream is a hipStream_t (NULL: default).
 * start_event / stop_event are optional hipEvent_t recorded at the kernel's own
 * start and end (hipExtLaunchKernelGGL). The call enqueues one kernel and returns.
 * Returns 0 on success, 1 for invalid arguments (nothing enqueued), 2 when the
 * launch fails (the HIP code is in ar_probe_last_hip_error()).
 */
#ifndef AR_PROBE_H
#define AR_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { AR_PROBE_STREAMS = 0, AR_PROBE_COPY = 1, AR_PROBE_FOLD = 2 } ar_probe_kind;

int32_t ar_probe_stream(void* const* bufs, int32_t P, int64_t bytes, int32_t kind, int32_t vectors_per_thread,
                        void* stream, void* start_event, void* stop_event);
int32_t ar_probe_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif /* AR_PROBE_H */
