/*
 * lrsort_prof.h -- per-kernel timing hooks of the lrsort library, for
 * benchmarks.  Not part of the sort's semantics.
 *
 * While recording is on, every kernel the sort calls enqueue is bracketed by
 * two HIP events recorded on the same stream as the kernel, so the elapsed time
 * between them is that launch's duration on the device.  Recording state is
 * process-global.  Sorts may run from several host threads while it is on:
 * each launch reserves its own record under a lock (launches past the capacity
 * are not recorded), and with recording off a launch only reads one atomic
 * flag.  lrs_prof_start and lrs_prof_release discard the records and must not
 * run while another thread is inside lrs_prof_read.
 */
#ifndef LRSORT_PROF_H
#define LRSORT_PROF_H

#include "lrsort.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Kernel kinds a record can name. */
typedef enum lrs_kernel_kind {
    LRS_KERNEL_UPSWEEP = 0,    /* per-block digit counts */
    LRS_KERNEL_SCAN = 1,       /* exclusive scan of the count matrix */
    LRS_KERNEL_DOWNSWEEP = 2,  /* stable in-tile rank and scatter */
    LRS_KERNEL_COPY = 3,       /* plain device copy */
    LRS_KERNEL_FINALIZE = 4,   /* after the last pass of a sort with an in-place
                                  array: moves it back to the output if the
                                  passes left it in temp storage */
    LRS_KERNEL_TINY = 5,       /* a whole small sort in one workgroup */
    LRS_KERNEL_SMALL = 6       /* one whole pass of a small sort in one launch */
} lrs_kernel_kind;

/* Starts recording with room for `capacity` kernel launches (events are
 * created here, on the current device).  Launches beyond the capacity are not
 * recorded.  Any earlier recording is discarded.  LRS_ERR_INVALID_ARG if
 * capacity <= 0, LRS_ERR_HIP if event creation fails. */
lrs_status lrs_prof_start(int capacity);

/* Stops recording; records made so far stay readable.  Always LRS_OK. */
lrs_status lrs_prof_stop(void);

/* Number of launches recorded since the last lrs_prof_start. */
int lrs_prof_count(void);

/* Record i (0 <= i < lrs_prof_count()): kernel kind, and the device time in
 * milliseconds between the events around it.  Blocks until that launch has
 * finished.  LRS_ERR_INVALID_ARG for a bad index or NULL outputs,
 * LRS_ERR_HIP if the event query fails. */
lrs_status lrs_prof_read(int i, int *kind, float *ms);

/* Frees the events.  Always LRS_OK. */
lrs_status lrs_prof_release(void);

/* Streaming-read reference for benchmarks: reads `bytes` bytes of device
 * memory at d_src with the library's tuned read kernel (grid-stride 16-byte
 * non-temporal loads, eight 256-thread workgroups per CU).  Each lane folds
 * the words it read into one xor; a lane whose fold equals 0x9E3779B9 stores
 * it to *d_result (device memory, 4 bytes), which otherwise is left as it is:
 * the store only gives the loads an effect, it is not a checksum.  bytes must
 * be a multiple of 16 and d_src 16-byte aligned, d_result 4-byte aligned;
 * otherwise, or NULL pointers with bytes > 0, LRS_ERR_INVALID_ARG.  Recorded
 * as LRS_KERNEL_COPY while profiling is on. */
lrs_status lrs_bench_read(const void *d_src, size_t bytes, uint32_t *d_result, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LRSORT_PROF_H */
