/*
 * lsd_oracle.c -- plain, single-threaded CPU oracle for the stable LSD radix
 * sort.  TEST INFRASTRUCTURE ONLY: the parity tests, the smoke check and the
 * benchmark's CPU-baseline leg load it.  The GPU library never links, includes
 * or calls anything here, and this file includes nothing from the GPU side.
 *
 * What it computes (the plain definition the GPU path must reproduce bit for
 * bit): with T(k) the identity for unsigned keys and the sign-flip encoding for
 * float32, and F(k) = (T(k) >> begin_bit) mod 2^(end_bit - begin_bit), the
 * output is the unique stable permutation of the input ordered by F.  Keys and
 * values move together; output keys are the original bit patterns.
 *
 * How it computes it: exactly the serial LSD loop of the kwkr.cn essay
 * (bitonic vs. LSD radix sort), section 3.1 "LSD baseline flow": for each digit
 * from least to most significant, (i) count the digit of every key, (ii) turn
 * the counts into an exclusive prefix, (iii) walk the input in order and drop
 * each key into the next free slot of its digit, (iv) swap source and
 * destination.  That page prints the loop for 32-bit keys with shifts
 * 0, 8, 16, 24; here the shift starts at begin_bit, steps by 8, and the last
 * digit is narrowed to the bits left before end_bit (the page "GPU radix sort:
 * from the CUB implementation to performance tuning", section 2, gives the
 * half-open [begin_bit, end_bit) range; the quant67.com survey "Parallel
 * sorting: from merge networks to GPU bitonic sort", section 8.1, finishes the
 * last few bits with one counting step).
 *
 * Keys are widened to 64-bit working words so one loop serves every key type;
 * that changes no result, only memory use.
 *
 * Parity pins (tests/test_oracle.py): the pages' worked 8-element example,
 * the float bit patterns the kwkr.cn essay prints, an exhaustive check of the
 * float transform against IEEE-754 ordering, brute-force stable sorts of every
 * short sequence over colliding alphabets, and numpy's stable argsort.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <time.h>

#define ORACLE_OK 0
#define ORACLE_ERR_ARG 1
#define ORACLE_ERR_NOMEM 2

/* Float32 -> order-preserving uint32 (kwkr.cn essay, section 3.3; page "GPU
 * radix sort ...", section 5.3): a clear sign bit gets the sign bit set, a set
 * sign bit gets every bit inverted. */
uint32_t oracle_f2s(uint32_t bits)
{
    uint32_t mask = (bits & 0x80000000u) ? 0xFFFFFFFFu : 0x80000000u;
    return bits ^ mask;
}

/* The reverse mapping the kwkr.cn essay (section 3.3) asks for after sorting
 * but does not print: an encoded word with its top bit set came from a
 * non-negative float (clear that bit again), otherwise from a negative one
 * (invert every bit again). */
uint32_t oracle_s2f(uint32_t u)
{
    return (u & 0x80000000u) ? (u ^ 0x80000000u) : ~u;
}

/* Signed keys (two's complement) -> order-preserving unsigned words: flip
 * the sign bit (page "GPU radix sort ...", section 5.2: the most negative
 * value becomes 0, the most positive all ones).  Flipping twice restores the
 * key, so the same function is its own inverse. */
uint32_t oracle_i32_code(uint32_t bits)
{
    return bits ^ 0x80000000u;
}

uint64_t oracle_i64_code(uint64_t bits)
{
    return bits ^ 0x8000000000000000ull;
}

/* Float64 -> order-preserving uint64: the float32 rule above on the 64-bit
 * pattern (sign clear: set the sign bit; sign set: invert every bit), and its
 * reverse mapping. */
uint64_t oracle_f64_code(uint64_t bits)
{
    uint64_t mask = (bits & 0x8000000000000000ull) ? 0xFFFFFFFFFFFFFFFFull : 0x8000000000000000ull;
    return bits ^ mask;
}

uint64_t oracle_f64_uncode(uint64_t u)
{
    return (u & 0x8000000000000000ull) ? (u ^ 0x8000000000000000ull) : ~u;
}

void oracle_f2s_array(const uint32_t *in, uint32_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f2s(in[i]);
}

void oracle_s2f_array(const uint32_t *in, uint32_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_s2f(in[i]);
}

/* One counting-sort pass over the digit (key >> shift) & mask, scattering in
 * input order so that equal digits keep their relative order. */
static void counting_pass(const uint64_t *src, uint64_t *dst,
                          const uint32_t *src_v, uint32_t *dst_v,
                          int64_t n, int shift, uint64_t mask)
{
    int64_t count[256];
    memset(count, 0, sizeof(count));

    /* (i) histogram of the digit */
    for (int64_t i = 0; i < n; ++i)
        count[(src[i] >> shift) & mask] += 1;

    /* (ii) exclusive prefix: count[d] becomes the first slot of digit d */
    int64_t total = 0;
    for (int d = 0; d < 256; ++d) {
        int64_t c = count[d];
        count[d] = total;
        total += c;
    }

    /* (iii) scatter in increasing input index */
    for (int64_t i = 0; i < n; ++i) {
        uint64_t digit = (src[i] >> shift) & mask;
        int64_t pos = count[digit];
        dst[pos] = src[i];
        if (dst_v) dst_v[pos] = src_v[i];
        count[digit] = pos + 1;
    }
}

/* Sorts n 64-bit working words (and optional values) in place over
 * [begin_bit, end_bit).  Returns ORACLE_OK or an error code. */
static int lsd_sort_words(uint64_t *words, uint32_t *vals, int64_t n,
                          int begin_bit, int end_bit)
{
    if (n <= 1 || begin_bit == end_bit) return ORACLE_OK;

    uint64_t *buf = (uint64_t *)malloc((size_t)n * sizeof(uint64_t));
    uint32_t *vbuf = NULL;
    if (!buf) return ORACLE_ERR_NOMEM;
    if (vals) {
        vbuf = (uint32_t *)malloc((size_t)n * sizeof(uint32_t));
        if (!vbuf) { free(buf); return ORACLE_ERR_NOMEM; }
    }

    uint64_t *src = words, *dst = buf;
    uint32_t *src_v = vals, *dst_v = vbuf;
    for (int shift = begin_bit; shift < end_bit; shift += 8) {
        int width = end_bit - shift < 8 ? end_bit - shift : 8;
        uint64_t mask = (1ull << width) - 1ull;
        counting_pass(src, dst, src_v, dst_v, n, shift, mask);
        /* (iv) the output of this pass is the input of the next */
        uint64_t *t = src; src = dst; dst = t;
        uint32_t *tv = src_v; src_v = dst_v; dst_v = tv;
    }
    if (src != words) {
        memcpy(words, src, (size_t)n * sizeof(uint64_t));
        if (vals) memcpy(vals, src_v, (size_t)n * sizeof(uint32_t));
    }
    free(buf);
    free(vbuf);
    return ORACLE_OK;
}

static int check_args(int64_t n, int begin_bit, int end_bit, int key_bits)
{
    if (n < 0) return ORACLE_ERR_ARG;
    if (begin_bit < 0 || end_bit < begin_bit || end_bit > key_bits) return ORACLE_ERR_ARG;
    return ORACLE_OK;
}

/* Key kinds: 0 = uint32, 1 = float32, 2 = uint64, 3 = int32, 4 = int64,
 * 5 = float64.  Each kind is sorted by its order-preserving unsigned word
 * (the identity, or one of the codes above) and written back through the
 * inverse, so keys come out as the caller's bit patterns. */
static int kind_bits(int key_kind)
{
    return (key_kind == 2 || key_kind == 4 || key_kind == 5) ? 64 : 32;
}

static uint64_t to_word(int key_kind, uint64_t raw)
{
    switch (key_kind) {
    case 1: return oracle_f2s((uint32_t)raw);
    case 3: return oracle_i32_code((uint32_t)raw);
    case 4: return oracle_i64_code(raw);
    case 5: return oracle_f64_code(raw);
    default: return raw;
    }
}

static uint64_t from_word(int key_kind, uint64_t w)
{
    switch (key_kind) {
    case 1: return oracle_s2f((uint32_t)w);
    case 3: return oracle_i32_code((uint32_t)w);
    case 4: return oracle_i64_code(w);
    case 5: return oracle_f64_uncode(w);
    default: return w;
    }
}

/* The order-preserving words of n keys of the given kind (as uint64). */
int oracle_code_array(int key_kind, const void *keys, uint64_t *words, int64_t n)
{
    if (key_kind < 0 || key_kind > 5 || n < 0) return ORACLE_ERR_ARG;
    for (int64_t i = 0; i < n; ++i) {
        uint64_t raw = kind_bits(key_kind) == 64 ? ((const uint64_t *)keys)[i]
                                                 : ((const uint32_t *)keys)[i];
        words[i] = to_word(key_kind, raw);
    }
    return ORACLE_OK;
}

/* keys_in/keys_out hold raw bit patterns (4 or 8 bytes per key).  vals_in and
 * vals_out are both NULL for a keys-only sort.  Inputs are never modified. */
int oracle_sort(int key_kind, const void *keys_in, const uint32_t *vals_in,
                void *keys_out, uint32_t *vals_out, int64_t n,
                int begin_bit, int end_bit)
{
    if (key_kind < 0 || key_kind > 5) return ORACLE_ERR_ARG;
    int key_bits = kind_bits(key_kind);
    int rc = check_args(n, begin_bit, end_bit, key_bits);
    if (rc) return rc;
    if ((vals_in == NULL) != (vals_out == NULL)) return ORACLE_ERR_ARG;
    if (n == 0) return ORACLE_OK;

    uint64_t *words = (uint64_t *)malloc((size_t)n * sizeof(uint64_t));
    uint32_t *vals = NULL;
    if (!words) return ORACLE_ERR_NOMEM;
    if (vals_in) {
        vals = (uint32_t *)malloc((size_t)n * sizeof(uint32_t));
        if (!vals) { free(words); return ORACLE_ERR_NOMEM; }
        memcpy(vals, vals_in, (size_t)n * sizeof(uint32_t));
    }

    if (key_bits == 64) {
        const uint64_t *k64 = (const uint64_t *)keys_in;
        for (int64_t i = 0; i < n; ++i) words[i] = to_word(key_kind, k64[i]);
    } else {
        const uint32_t *k32 = (const uint32_t *)keys_in;
        for (int64_t i = 0; i < n; ++i) words[i] = to_word(key_kind, k32[i]);
    }

    rc = lsd_sort_words(words, vals, n, begin_bit, end_bit);

    if (rc == ORACLE_OK) {
        if (key_bits == 64) {
            uint64_t *o64 = (uint64_t *)keys_out;
            for (int64_t i = 0; i < n; ++i) o64[i] = from_word(key_kind, words[i]);
        } else {
            uint32_t *o32 = (uint32_t *)keys_out;
            for (int64_t i = 0; i < n; ++i) o32[i] = (uint32_t)from_word(key_kind, words[i]);
        }
        if (vals_out) memcpy(vals_out, vals, (size_t)n * sizeof(uint32_t));
    }
    free(words);
    free(vals);
    return rc;
}

/* Runs oracle_sort `reps` times and stores each run's wall time in seconds
 * (steady clock) in times[]; used only to report the CPU baseline. */
int oracle_time_sort(int key_kind, const void *keys_in, const uint32_t *vals_in,
                     void *keys_out, uint32_t *vals_out, int64_t n,
                     int begin_bit, int end_bit, int reps, double *times)
{
    for (int r = 0; r < reps; ++r) {
        struct timespec t0, t1;
        clock_gettime(CLOCK_MONOTONIC, &t0);
        int rc = oracle_sort(key_kind, keys_in, vals_in, keys_out, vals_out, n,
                             begin_bit, end_bit);
        clock_gettime(CLOCK_MONOTONIC, &t1);
        if (rc) return rc;
        times[r] = (double)(t1.tv_sec - t0.tv_sec) + 1e-9 * (double)(t1.tv_nsec - t0.tv_nsec);
    }
    return ORACLE_OK;
}
