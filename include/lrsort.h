/*
 * lrsort.h -- C ABI of a stable LSD radix sort for AMD MI355X (gfx950).
 *
 * The operation: sort n keys (and, for the pair calls, a uint32 value carried
 * with each key) ascending by the key bits [begin_bit, end_bit), from an input
 * array into an output array, stably (equal bit fields keep their input order).
 * The bit range is half-open, as in the library call of the page "GPU radix
 * sort: from the CUB implementation to performance tuning", section 2, and the
 * sort runs one pass per 8-bit digit from least to most significant, each pass a
 * histogram, a scan and a scatter (same page, section 3).  A last digit narrower
 * than 8 bits sorts only the bits left before end_bit (the quant67.com survey
 * "Parallel sorting: from merge networks to GPU bitonic sort", section 8.1:
 * the last few bits take one counting step).  Bits outside [begin_bit,
 * end_bit) play no part in the order but are kept in the output keys.
 *
 * Keys and values move together in one sort, never as a key sort followed by a
 * gather (same page, section 5.5).
 *
 * Key types.  Every key type is ordered as an unsigned word, the key's order
 * code, and [begin_bit, end_bit) indexes that word:
 *  - u32, u64: the key itself;
 *  - i32, i64 (two's complement): the key with its sign bit flipped (the page
 *    "GPU radix sort ...", section 5.2), so negative keys sort first;
 *  - f32, f64 (IEEE-754): non-negative floats get the sign bit set, negative
 *    floats get every bit inverted (same page, section 5.3; the kwkr.cn essay
 *    on bitonic vs. LSD radix sort, section 3.3).  Under it -0.0 sorts before
 *    +0.0, +NaN after +inf and -NaN before -inf.
 * The code is formed in registers to pick each digit; keys are stored and
 * returned as the caller's bit patterns, unchanged.
 *
 * Conventions shared by every sort call:
 *  - Two-phase temp storage (same page, section 2, and section 6, first
 *    pitfall): with d_temp == NULL the call writes the bytes it needs to
 *    *temp_bytes, returns LRS_OK and does no work.  Call it with the same
 *    pointers, n and bit range as the real call (in-place use can need more
 *    temp).  With d_temp != NULL, *temp_bytes is the size of d_temp; less than
 *    the requirement gives LRS_ERR_TEMP_TOO_SMALL and nothing is touched.
 *    d_temp may have any alignment: the library lays its temp out from the
 *    first 256-byte boundary at or after d_temp, and the size the query
 *    reports includes 255 bytes for that (an aligned d_temp needs 255 fewer).
 *  - All array pointers are device memory owned by the caller.  The library
 *    allocates nothing and enqueues its kernels on `stream` asynchronously:
 *    results are ready when the stream reaches them.  d_temp must stay
 *    allocated until then.  Between calls it keeps only per-device facts it
 *    looks up once (the CU count, its kernels' occupancy).
 *  - A call enqueues kernel launches only (no memset, copy engine or host
 *    synchronization), so a call with its temp storage already allocated can
 *    be captured into a HIP graph and replayed; the first call on a device is
 *    best made outside the capture, since it queries the device.
 *  - The input arrays are not modified, except when the caller passes the same
 *    pointer for input and output (in-place sort, same page section 6, third
 *    pitfall), which is allowed for keys and values independently.  Partial
 *    overlap of an input and an output gives LRS_ERR_INVALID_ARG; overlap of
 *    d_temp with any array is undefined.
 *  - 0 <= begin_bit <= end_bit <= 8 * sizeof(key); otherwise
 *    LRS_ERR_INVALID_ARG.  begin_bit == end_bit copies input to output.
 *  - 0 <= n <= 2^32 - 1 (offsets are 32-bit); n == 0 is a no-op.  Otherwise
 *    LRS_ERR_INVALID_ARG.
 *  - Arrays must be aligned to their element size; NULL array pointers with
 *    n > 0 give LRS_ERR_INVALID_ARG.
 *  - Ascending only.  The result is deterministic (identical on every run).
 *  - A failed kernel launch gives LRS_ERR_HIP.
 *  - Calls on different streams with different temp buffers may run
 *    concurrently; a temp buffer must not be shared by calls in flight.
 */
#ifndef LRSORT_H
#define LRSORT_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum lrs_status {
    LRS_OK = 0,
    LRS_ERR_INVALID_ARG = 1,
    LRS_ERR_TEMP_TOO_SMALL = 2,
    LRS_ERR_HIP = 3,
    LRS_ERR_TOO_LARGE = 4  /* lrs_sort_digits_noalloc only: the sort needs more
                              scratch than the library's static scratch holds */
} lrs_status;

/* Keys-only sorts: d_keys_in[0..n) -> d_keys_out[0..n). */
lrs_status lrs_sort_keys_u32(void *d_temp, size_t *temp_bytes,
                             const uint32_t *d_keys_in, uint32_t *d_keys_out,
                             int64_t n, int begin_bit, int end_bit, hipStream_t stream);
lrs_status lrs_sort_keys_u64(void *d_temp, size_t *temp_bytes,
                             const uint64_t *d_keys_in, uint64_t *d_keys_out,
                             int64_t n, int begin_bit, int end_bit, hipStream_t stream);
lrs_status lrs_sort_keys_f32(void *d_temp, size_t *temp_bytes,
                             const float *d_keys_in, float *d_keys_out,
                             int64_t n, int begin_bit, int end_bit, hipStream_t stream);
lrs_status lrs_sort_keys_i32(void *d_temp, size_t *temp_bytes,
                             const int32_t *d_keys_in, int32_t *d_keys_out,
                             int64_t n, int begin_bit, int end_bit, hipStream_t stream);
lrs_status lrs_sort_keys_i64(void *d_temp, size_t *temp_bytes,
                             const int64_t *d_keys_in, int64_t *d_keys_out,
                             int64_t n, int begin_bit, int end_bit, hipStream_t stream);
lrs_status lrs_sort_keys_f64(void *d_temp, size_t *temp_bytes,
                             const double *d_keys_in, double *d_keys_out,
                             int64_t n, int begin_bit, int end_bit, hipStream_t stream);

/* Pair sorts: (d_keys_in[i], d_values_in[i]) move together to the outputs.
 * Argument order follows the pair call of the page "GPU radix sort ...",
 * section 5.5. */
lrs_status lrs_sort_pairs_u32(void *d_temp, size_t *temp_bytes,
                              const uint32_t *d_keys_in, const uint32_t *d_values_in,
                              uint32_t *d_keys_out, uint32_t *d_values_out,
                              int64_t n, int begin_bit, int end_bit, hipStream_t stream);
lrs_status lrs_sort_pairs_u64(void *d_temp, size_t *temp_bytes,
                              const uint64_t *d_keys_in, const uint32_t *d_values_in,
                              uint64_t *d_keys_out, uint32_t *d_values_out,
                              int64_t n, int begin_bit, int end_bit, hipStream_t stream);
lrs_status lrs_sort_pairs_f32(void *d_temp, size_t *temp_bytes,
                              const float *d_keys_in, const uint32_t *d_values_in,
                              float *d_keys_out, uint32_t *d_values_out,
                              int64_t n, int begin_bit, int end_bit, hipStream_t stream);
lrs_status lrs_sort_pairs_i32(void *d_temp, size_t *temp_bytes,
                              const int32_t *d_keys_in, const uint32_t *d_values_in,
                              int32_t *d_keys_out, uint32_t *d_values_out,
                              int64_t n, int begin_bit, int end_bit, hipStream_t stream);
lrs_status lrs_sort_pairs_i64(void *d_temp, size_t *temp_bytes,
                              const int64_t *d_keys_in, const uint32_t *d_values_in,
                              int64_t *d_keys_out, uint32_t *d_values_out,
                              int64_t n, int begin_bit, int end_bit, hipStream_t stream);
lrs_status lrs_sort_pairs_f64(void *d_temp, size_t *temp_bytes,
                              const double *d_keys_in, const uint32_t *d_values_in,
                              double *d_keys_out, uint32_t *d_values_out,
                              int64_t n, int begin_bit, int end_bit, hipStream_t stream);

/* Key types of lrs_sort_digits, with the order codes of the typed calls. */
typedef enum lrs_key_type {
    LRS_KEY_U32 = 0,
    LRS_KEY_I32 = 1,
    LRS_KEY_F32 = 2,
    LRS_KEY_U64 = 3,
    LRS_KEY_I64 = 4,
    LRS_KEY_F64 = 5
} lrs_key_type;

/* The sort of the typed calls above, for any key type, with the digit width
 * chosen: digit_bits 8 is what the typed calls run; digit_bits 11 sorts by
 * 11-bit digits, 2048 buckets per pass, so ceil((end_bit - begin_bit) / 11)
 * passes (3 instead of 4 for 32-bit keys, the last digit taking what bits are
 * left), as the kwkr.cn essay on bitonic vs. LSD radix sort suggests in
 * sections 3.4 and 5.2 and the page "GPU radix sort ..." weighs in section 4
 * (fewer passes against larger histograms and scans).  The result is the same
 * for either width: a stable sort is determined by the keys' order.
 *  - key_type: an lrs_key_type; d_keys_in / d_keys_out point to arrays of that
 *    type.
 *  - d_values_in and d_values_out: both NULL for a keys-only sort, else both
 *    uint32 arrays of n values that move with the keys (pair sort).  One NULL
 *    and the other not, with n > 0, gives LRS_ERR_INVALID_ARG.
 *  - digit_bits other than 8 or 11 gives LRS_ERR_INVALID_ARG.
 *  - Sorts small enough for the library's one-workgroup path (some thousands
 *    of keys) take that path for either width.
 * Temp storage, streams, in-place use, bit range, n and alignment follow the
 * conventions at the top of this file; the temp query must pass the same
 * digit_bits (11-bit sorts need a count matrix 8 times larger, up to 32 MB). */
lrs_status lrs_sort_digits(lrs_key_type key_type, int digit_bits, void *d_temp, size_t *temp_bytes,
                           const void *d_keys_in, const uint32_t *d_values_in, void *d_keys_out,
                           uint32_t *d_values_out, int64_t n, int begin_bit, int end_bit,
                           hipStream_t stream);

/* The sort of lrs_sort_digits without temp storage from the caller and without
 * any allocation: for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * The library's count matrix and alternate buffers live instead in one static
 * device array of LRS_NOALLOC_SCRATCH_BYTES bytes per GPU (held by each GPU
 * the library runs on until the process ends); the call itself allocates
 * nothing, on the host or the device.
 *  - Arguments, results and errors as lrs_sort_digits, without d_temp and
 *    temp_bytes.
 *  - A sort whose temp storage (what lrs_sort_digits would ask for with
 *    d_temp == NULL) exceeds LRS_NOALLOC_SCRATCH_BYTES gives
 *    LRS_ERR_TOO_LARGE before any device call: at most about 15.6 million
 *    32-bit keys alone, 7.8 million 32-bit pairs or 64-bit keys, 5.2 million
 *    64-bit pairs with 8-bit digits (in-place sorts with an odd number of
 *    passes, three or more, need twice the alternate space).
 *  - The scratch is shared by every call on a GPU and keeps the last call's
 *    contents; no part of it needs to start at zero.  Calls that overlap on
 *    one GPU (other host threads, or other streams before the earlier call's
 *    work has finished) race on it and give undefined results: serialize
 *    them on one stream.
 *  - The first call on a device looks up that device's scratch address
 *    (hipGetSymbolAddress); it is best made outside any graph capture. */
#define LRS_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
lrs_status lrs_sort_digits_noalloc(lrs_key_type key_type, int digit_bits, const void *d_keys_in,
                                   const uint32_t *d_values_in, void *d_keys_out, uint32_t *d_values_out,
                                   int64_t n, int begin_bit, int end_bit, hipStream_t stream);

/* Static description of a status code (never NULL). */
const char *lrs_status_string(lrs_status status);

/* Plain device-to-device copy of `bytes` bytes on `stream` with the library's
 * own streaming kernel (the sort uses it when begin_bit == end_bit).  Also the
 * achievable-bandwidth reference a benchmark times beside the sort.  dst and
 * src must not overlap.  LRS_ERR_INVALID_ARG for NULL pointers with bytes > 0. */
lrs_status lrs_device_copy(void *d_dst, const void *d_src, size_t bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LRSORT_H */
