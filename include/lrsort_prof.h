/*
 * lrsort_prof.h -- per-kernel timing hooks of the lrsort library, for
 * benchmarks.  Not part of the sort's semantics.
 *
 * While recording is on, every kernel the sort calls enqueue is bracketed by
 * two HIP events recorded on the same stream as the kernel, so the elapsed time
 * between them is that launch's duration on the device.  Recording state is
 * process-global and not thread-safe: enable it, run sorts from one host thread,
 * synchronize the stream, read the records, disable it.
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
    LRS_KERNEL_FINALIZE = 4,   /* after the last pass: moves data to the output
                                  if skipped passes left it elsewhere */
    LRS_KERNEL_TINY = 5        /* a whole small sort in one workgroup */
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

#ifdef __cplusplus
}
#endif

#endif /* LRSORT_PROF_H */
