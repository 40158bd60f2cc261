// kernels.hpp -- gfx950 (CDNA4, wave64) kernels of the stable LSD radix sort.
//
// One pass sorts by one 8-bit digit and runs three kernels on the caller's
// stream (the page "GPU radix sort: from the CUB implementation to performance
// tuning", section 3: histogram, scan, scatter):
//
//   upsweep    each workgroup counts the digits of its block of keys
//              (a "block" = a contiguous run of whole tiles) in wave-private
//              LDS sub-histograms and stores the merged counts digit-major,
//              counts[d * num_blocks + b];
//   scan       one workgroup per digit row turns its row into exclusive
//              prefixes and stores the row total;
//   downsweep  each workgroup walks the tiles of its block in order: loads a
//              tile with coalesced reads, ranks every key stably inside the
//              tile with 64-lane match masks, reorders the tile through LDS so
//              that each digit's keys are contiguous, and writes them to
//              digit_start[d] + block_prefix[d] + (keys of digit d in earlier
//              tiles of the block) + rank.
//
// Counting per block of many tiles instead of per tile keeps the count matrix a
// few MB at any n (so the scan is cheap), and lets a workgroup continue each
// digit's output run from one tile to the next: it holds back the keys of the
// 128-byte line a run leaves open and writes that line whole once a later tile
// fills it.
//
// Stability: within a tile, key i's rank among equal digits counts only keys
// before it in input order (the page's section 3, last paragraphs: the stable
// in-block rank replaces the atomic cursor of the teaching scatter, whose order
// is the scheduler's).  Across tiles and blocks, offsets are assigned in input
// order by the scans.  So every pass is a stable counting sort, which is what
// least-significant-digit-first ordering needs (kwkr.cn essay on bitonic vs. LSD
// radix sort, section 3).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace lrs {

constexpr int kRadixBits = 8;
constexpr int kXcds = 8;  // accelerator complex dies of the part; used only to place work
constexpr int kRadix = 1 << kRadixBits;
constexpr int kWave = 64;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ key codes
//
// Keys stay as the caller gave them, in every buffer and every pass.  A pass
// orders keys by a digit of an order-preserving unsigned code of the key,
// formed in registers only to take that digit (the codes are those of the page
// "GPU radix sort: from the CUB implementation to performance tuning",
// sections 5.2-5.3, and of the kwkr.cn essay on bitonic vs. LSD radix sort,
// section 3.3):
//   unsigned   the key itself;
//   signed     two's complement with the sign bit flipped;
//   float      IEEE-754: sign clear -> sign bit set; sign set -> all bits
//              inverted (so -0.0 orders just below +0.0 and NaNs past the
//              infinities of their sign).
enum KeyCode { CODE_UNSIGNED = 0, CODE_SIGNED = 1, CODE_FLOAT = 2 };

template <typename K, int CODE>
__device__ __forceinline__ K order_code(K k)
{
    constexpr int kTop = 8 * (int)sizeof(K) - 1;
    constexpr K kSign = (K)1 << kTop;
    using S = typename std::conditional<sizeof(K) == 4, int32_t, int64_t>::type;
    if constexpr (CODE == CODE_SIGNED) {
        return k ^ kSign;
    } else if constexpr (CODE == CODE_FLOAT) {
        return k ^ ((K)((S)k >> kTop) | kSign);  // arithmetic shift: all ones if negative
    } else {
        return k;
    }
}

template <int CODE, typename K>
__device__ __forceinline__ uint32_t digit_of(K k, int shift, uint32_t mask)
{
    if constexpr (sizeof(K) == 4) {
        // one bitfield extract (mask is 2^width - 1, the same for all lanes)
        return __builtin_amdgcn_ubfe((uint32_t)order_code<K, CODE>(k), (uint32_t)shift, (uint32_t)__popc(mask));
    } else {
        return (uint32_t)(order_code<K, CODE>(k) >> shift) & mask;
    }
}

// A key whose code is all ones: its digit is the largest of any pass, so the
// padding slots of a short tile rank after every real key.
template <typename K, int CODE>
__device__ __forceinline__ K pad_key()
{
    return CODE == CODE_UNSIGNED ? ~(K)0 : (K)(~(K)0 >> 1);  // 0x7f..f: sign clear, code all ones
}

// --------------------------------------------------------------- wave helpers

// All-ones if bit b of d is set, else zero.  Written as the instruction itself
// so the compiler keeps one v_bfe_i32 per bit and derives the ballot from its
// result instead of re-testing d with an extra shift.
template <int B>
__device__ __forceinline__ uint32_t bit_mask(uint32_t d)
{
    uint32_t t;
    asm("v_bfe_i32 %0, %1, %2, 1" : "=v"(t) : "v"(d), "i"(B));
    return t;
}

// Lanes of the wave whose 8-bit digit equals this lane's: for each digit bit,
// keep the lanes whose ballot bit agrees with ours (the 64-lane form of the
// ballot / popcount / lanes-below rank of the warp partition walked through on
// the blog.csdn.net page about the qsort_warp sample).  All 64 lanes must be
// active.  v_bitop3 0x90 computes m & ~(ballot ^ t): with t all-ones when our
// bit is set it keeps the ballot, otherwise its complement.  Four VALU
// instructions per digit bit; BITS is the digit width.
template <int BITS, int B = 0>
__device__ __forceinline__ void match_bits(uint32_t d, uint32_t &lo, uint32_t &hi)
{
    if constexpr (B < BITS) {
        const uint32_t t = bit_mask<B>(d);
        const uint64_t bal = __ballot(t != 0u);
        lo = __builtin_amdgcn_bitop3_b32(lo, (uint32_t)bal, t, 0x90);
        hi = __builtin_amdgcn_bitop3_b32(hi, (uint32_t)(bal >> 32), t, 0x90);
        match_bits<BITS, B + 1>(d, lo, hi);
    }
}

template <int BITS = kRadixBits>
__device__ __forceinline__ void match_digit(uint32_t d, uint32_t &lo, uint32_t &hi)
{
    lo = 0xFFFFFFFFu;
    hi = 0xFFFFFFFFu;
    match_bits<BITS>(d, lo, hi);
}

// Number of set bits of (hi:lo) in lanes below this one.
__device__ __forceinline__ uint32_t lanes_below(uint32_t lo, uint32_t hi)
{
    return __builtin_amdgcn_mbcnt_hi(hi, __builtin_amdgcn_mbcnt_lo(lo, 0u));
}

// Inclusive prefix sum over the 64 lanes with DPP moves (no LDS): shifts of
// 1, 2, 4 and 8 lanes inside each row of 16, then row 0's and rows 0-1's
// last lanes broadcast into the rows above.  All lanes must be active.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x)
{
    x += __builtin_amdgcn_update_dpp(0u, x, 0x111, 0xf, 0xf, false);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0u, x, 0x112, 0xf, 0xf, false);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0u, x, 0x114, 0xf, 0xf, false);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0u, x, 0x118, 0xf, 0xf, false);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0u, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0u, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return x;
}

// Exclusive prefix sum of one value per thread over the whole workgroup.
// s_tmp needs THREADS/64 words.  Every thread must call it (it synchronizes).
template <int THREADS>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t *s_tmp, uint32_t &total)
{
    constexpr int WAVES = THREADS / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const uint32_t x = wave_inclusive_scan(v);
    if (lane == kWave - 1) s_tmp[wave] = x;
    __syncthreads();
    uint32_t before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
        const uint32_t t = s_tmp[w];
        before += (w < wave) ? t : 0u;
        all += t;
    }
    total = all;
    __syncthreads();
    return before + x - v;
}

// Exclusive prefix sum over the 256 digits, run by one wave: lane l owns
// digits 4l..4l+3 (one 16-byte vector).  Returns the lane's four exclusive
// prefixes.
__device__ __forceinline__ uint4 wave_scan_digits(uint4 c)
{
    const uint32_t p1 = c.x, p2 = p1 + c.y, p3 = p2 + c.z, sum = p3 + c.w;
    const uint32_t base = wave_inclusive_scan(sum) - sum;
    return make_uint4(base, base + p1, base + p2, base + p3);
}

// ------------------------------------------------------------------ routing
//
// Where a sort's data can be: the caller's input and output and two alternate
// buffers in temp storage, by index.  A pass whose digit is the same for every
// key leaves the order unchanged, so it moves nothing (the kwkr.cn essay on
// bitonic vs. LSD radix sort, section 3.4: a pass over a constant digit is
// wasted work).  Which passes those are follows from the bits in which the
// keys' order codes differ (their AND xor their OR), which the first pass
// records; from it, every kernel derives the same route for itself: the
// passes that run alternate between buffers so that the last of them writes
// the output.  Only an in-place array (input and output the same memory) can
// end elsewhere, and a copy after the last pass moves it.
enum BufIndex { BUF_IN = 0, BUF_OUT = 1, BUF_A = 2, BUF_B = 3 };

struct SortBufs {
    const void *keys[4];
    const uint32_t *vals[4];
};

// A sort's passes and where each array starts: BUF_IN, or BUF_OUT for an
// in-place array.  kb / vb: the second alternate buffer exists (in-place
// arrays with an odd number of passes, at least 3).
struct Route {
    int passes;
    int begin_bit, end_bit, digit_bits;
    int kstart, vstart;
    int kb, vb;
};

// Pass p sorts by bits [shift, shift + width) (the last digit takes what is
// left of the range).
__host__ __device__ __forceinline__ int pass_shift(const Route &rt, int p) { return rt.begin_bit + rt.digit_bits * p; }
__host__ __device__ __forceinline__ uint32_t pass_mask(const Route &rt, int p)
{
    const int left = rt.end_bit - pass_shift(rt, p);
    const int w = rt.digit_bits < left ? rt.digit_bits : left;
    return (1u << w) - 1u;
}

// Bit p set when pass p's digit is the same for every key, from the bits in
// which the keys' order codes differ.
__host__ __device__ __forceinline__ uint32_t skipped_passes(const Route &rt, unsigned long long diff)
{
    uint32_t skip = 0u;
    for (int p = 0; p < rt.passes; ++p)
        if (((diff >> pass_shift(rt, p)) & (unsigned long long)pass_mask(rt, p)) == 0ull) skip |= 1u << p;
    return skip;
}

// Destination of the k-th of R passes that run, for an array that starts in
// `start`.  An array that starts in the input alternates between the output
// and A so that pass R-1 writes the output.  An in-place array starts in the
// output, so it goes out first (to A, then B when R is odd and B exists) and
// comes back on the last pass; with R odd and no B it ends in A and is copied
// back.
__host__ __device__ __forceinline__ int run_dest(int start, bool has_b, int R, int k)
{
    if (start != BUF_OUT) return ((R - 1 - k) & 1) == 0 ? BUF_OUT : BUF_A;
    if ((R & 1) == 0 || !(has_b && R >= 3)) return (k & 1) == 0 ? BUF_A : BUF_OUT;
    if (k == 0) return BUF_A;
    if (k == 1) return BUF_B;
    return ((R - 1 - k) & 1) == 0 ? BUF_OUT : BUF_B;
}

// Where pass p of an array reads and writes (a skipped pass: the same buffer).
__host__ __device__ __forceinline__ void pass_route(int start, bool has_b, int passes, uint32_t skip, int p,
                                                    int &src, int &dst)
{
    const uint32_t run = ~skip & ((1u << passes) - 1u);
    const int R = __builtin_popcount(run);
    const int k = __builtin_popcount(run & ((1u << p) - 1u));  // passes that run before p
    src = k == 0 ? start : run_dest(start, has_b, R, k - 1);
    dst = (skip >> p) & 1u ? src : run_dest(start, has_b, R, k);
}

// Where an array is after the last pass.
__host__ __device__ __forceinline__ int final_buffer(int start, bool has_b, int passes, uint32_t skip)
{
    const int R = __builtin_popcount(~skip & ((1u << passes) - 1u));
    return R == 0 ? start : run_dest(start, has_b, R, R - 1);
}

// Grid-stride copy of n elements, 16 bytes per lane per step when both arrays
// are 16-byte aligned.
template <typename T>
__device__ __forceinline__ void grid_copy(const T *__restrict__ src, T *__restrict__ dst, int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t first = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    int64_t done = 0;
    if ((((uintptr_t)src | (uintptr_t)dst) & 15) == 0) {
        constexpr int PER = 16 / (int)sizeof(T);
        const int64_t nv = n / PER;
        const u32x4 *s4 = reinterpret_cast<const u32x4 *>(src);
        u32x4 *d4 = reinterpret_cast<u32x4 *>(dst);
        // non-temporal both ways: whole 16-byte vectors, written once
        for (int64_t i = first; i < nv; i += stride)
            __builtin_nontemporal_store(__builtin_nontemporal_load(&s4[i]), &d4[i]);
        done = nv * PER;
    }
    for (int64_t i = done + first; i < n; i += stride) dst[i] = src[i];
}

// Moves each array that `skip` leaves outside the output there.  Every thread
// of the grid takes part.
template <typename K, bool PAIRS>
__device__ __forceinline__ void move_to_output(const SortBufs &bufs, const Route &rt, uint32_t skip, int64_t n)
{
    const int k = final_buffer(rt.kstart, rt.kb != 0, rt.passes, skip);
    if (k != BUF_OUT) grid_copy<K>((const K *)bufs.keys[k], (K *)bufs.keys[BUF_OUT], n);
    if constexpr (PAIRS) {
        const int v = final_buffer(rt.vstart, rt.vb != 0, rt.passes, skip);
        if (v != BUF_OUT) grid_copy<uint32_t>(bufs.vals[v], (uint32_t *)bufs.vals[BUF_OUT], n);
    }
}

// -------------------------------------------------------------------- upsweep

// Adds the digits of keys [begin, end) into the LDS histogram h (atomics),
// THREADS lanes striding together.  16-byte loads, UNROLL in flight per lane,
// where the array and `begin` are 16-byte aligned; single keys otherwise.
// With SPREAD, it also folds the keys into code_and and code_or, from which
// the bits that differ between the keys' order codes follow (AND xor OR).
// Unsigned and signed codes differ from the key bits by a fixed xor, which
// leaves those bits unchanged, so only float keys are folded as codes.
template <typename K, int CODE, int THREADS, bool SPREAD = false, int UNROLL = 4>
__device__ __forceinline__ void count_range(const K *__restrict__ keys, int64_t begin, int64_t end,
                                            uint32_t *h, int tid, int shift, uint32_t mask, K &code_and,
                                            K &code_or)
{
    auto fold = [](K k) { return CODE == CODE_FLOAT ? order_code<K, CODE>(k) : k; };
    auto spread = [&](K k) {
        if constexpr (SPREAD) {
            code_and &= fold(k);
            code_or |= fold(k);
        }
    };
    // four keys at once: three-input AND and OR
    auto spread4 = [&](K a, K b, K c, K d) {
        if constexpr (SPREAD) {
            code_and = code_and & fold(a) & fold(b) & (fold(c) & fold(d));
            code_or = code_or | fold(a) | fold(b) | (fold(c) | fold(d));
        }
    };
    auto count_key = [&](K k) {
        spread(k);
        atomicAdd(&h[digit_of<CODE>(k, shift, mask)], 1u);
    };
    constexpr int PER = 16 / (int)sizeof(K);
    int64_t scalar_from = begin;
    if ((((uintptr_t)keys & 15) == 0) && begin % PER == 0) {
        using V = uint4;
        const V *vk = reinterpret_cast<const V *>(keys);
        const int64_t vbeg = begin / PER, vend = end / PER;
        for (int64_t base = vbeg; base < vend; base += (int64_t)THREADS * UNROLL) {
            V v[UNROLL];
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                const int64_t i = base + (int64_t)u * THREADS + tid;
                if (i < vend) {
                    const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(&vk[i]));
                    v[u] = make_uint4(t.x, t.y, t.z, t.w);
                }
            }
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                const int64_t i = base + (int64_t)u * THREADS + tid;
                if (i < vend) {
                    uint32_t d[PER];
                    if constexpr (sizeof(K) == 4) {
                        spread4((K)v[u].x, (K)v[u].y, (K)v[u].z, (K)v[u].w);
                        d[0] = digit_of<CODE>((K)v[u].x, shift, mask);
                        d[1] = digit_of<CODE>((K)v[u].y, shift, mask);
                        d[2] = digit_of<CODE>((K)v[u].z, shift, mask);
                        d[3] = digit_of<CODE>((K)v[u].w, shift, mask);
                    } else {
                        spread((K)(((uint64_t)v[u].y << 32) | v[u].x));
                        spread((K)(((uint64_t)v[u].w << 32) | v[u].z));
                        d[0] = digit_of<CODE>((K)(((uint64_t)v[u].y << 32) | v[u].x), shift, mask);
                        d[1] = digit_of<CODE>((K)(((uint64_t)v[u].w << 32) | v[u].z), shift, mask);
                    }
                    // When every key the wave holds here has one digit (constant
                    // keys, or a constant digit of this pass), one lane adds them
                    // all: otherwise 64 lanes would serialize on one LDS word.
                    const uint32_t f = __builtin_amdgcn_readfirstlane(d[0]);
                    bool same = true;
#pragma unroll
                    for (int k = 0; k < PER; ++k) same = same && d[k] == f;
                    if (__ballot(!same) == 0) {
                        const unsigned long long act = __ballot(1);
                        if ((int)(tid & (kWave - 1)) == __builtin_ffsll((long long)act) - 1)
                            atomicAdd(&h[f], (uint32_t)(PER * __popcll(act)));
                    } else {
#pragma unroll
                        for (int k = 0; k < PER; ++k) atomicAdd(&h[d[k]], 1u);
                    }
                }
            }
        }
        scalar_from = vend * PER;
    }
    for (int64_t i = scalar_from + tid; i < end; i += THREADS) count_key(__builtin_nontemporal_load(&keys[i]));
}


// Counts the digits of block b = keys [b * block_len, min(n, (b+1) * block_len)).
// Each wave adds into its own LDS sub-histograms, so atomics only contend
// within a wave (the kwkr.cn essay, section 3.2, and the quant67.com survey,
// section 8.1: per-block and per-warp counting instead of global atomics).
// The keys are read 16 bytes per lane when their array is 16-byte aligned.
// RB is the digit width: 8, or 11 for the 2048-digit passes.
// Bits that differ between the order codes of a sort's keys (their AND xor
// their OR) show which passes have a constant digit: the first pass records
// the AND and OR of each column (SPREAD), the first scan combines them, and a
// later pass whose digit bits are all equal there returns at once in every
// kernel (no key is read; its downsweep leaves the data where it is).
__device__ __forceinline__ bool digit_constant(const unsigned long long *diff, int shift, uint32_t mask)
{
    return ((*diff >> shift) & (unsigned long long)mask) == 0ull;
}

template <typename K, int CODE, int THREADS, int RB = kRadixBits, bool SPREAD = false>
__global__ __launch_bounds__(THREADS) void upsweep_kernel(
    SortBufs bufs, Route rt, int pass, uint32_t *__restrict__ counts, int64_t n, int64_t block_len, int num_blocks,
    int shift, uint32_t mask, unsigned long long *__restrict__ spread_out,
    const unsigned long long *__restrict__ diff_in)
{
    // The count matrix is digit-major, so a workgroup's 256 counts land in 256
    // different rows, 4 bytes in each 128-byte line.  Workgroups go to the
    // chip's XCDs in turn (workgroup i to XCD i mod kXcds); column c is counted
    // by workgroup (c mod per) * kXcds + c / per, so that each XCD counts a
    // contiguous range of columns and a line's 32 counts are merged in one L2
    // instead of reaching memory as partial writes from several.  (Any mapping
    // is correct; this one only places the writes.)
    const int per = (num_blocks + kXcds - 1) / kXcds;
    const int col = (int)(blockIdx.x % kXcds) * per + (int)(blockIdx.x / kXcds);
    if (col >= num_blocks) return;  // the launch rounds the grid up to kXcds * per
    // (read before the histograms are cleared, so the two latencies overlap)
    const unsigned long long diff = diff_in != nullptr ? *diff_in : ~0ull;
    constexpr int WAVES = THREADS / kWave;
    // COPIES sub-histograms (lane % COPIES picks one), padded by one word so
    // that equal digits in different copies fall in different banks: skewed
    // digits then serialize at most 64/COPIES lanes per atomic.  With 256
    // digits each wave has its own copies; with 2048 the workgroup's waves
    // share them (32 KB, against 256 KB for copies per wave), which leaves
    // room for four workgroups per CU.
    constexpr int RADIX = 1 << RB;
    constexpr int COPIES = 4;
    constexpr bool SHARED = RB != kRadixBits;
    constexpr int ROWS = SHARED ? COPIES : WAVES * COPIES;
    constexpr int STRIDE = RADIX + 1;
    __shared__ uint32_t hist[ROWS][STRIDE];
    const int tid = threadIdx.x;
    uint32_t *h = hist[SHARED ? (tid % COPIES) : (tid / kWave) * COPIES + (tid % COPIES)];
    for (int i = tid; i < ROWS * STRIDE; i += THREADS) (&hist[0][0])[i] = 0u;
    __syncthreads();
    // After the first pass: return at once when this pass's digit is constant;
    // otherwise read where the previous passes left the keys.
    int src = rt.kstart;
    if (diff_in != nullptr) {
        const uint32_t skip = skipped_passes(rt, diff);
        if ((skip >> pass) & 1u) return;
        int dst;
        pass_route(rt.kstart, rt.kb != 0, rt.passes, skip, pass, src, dst);
    }
    const K *__restrict__ keys = (const K *)bufs.keys[src];

    const int64_t begin = (int64_t)col * block_len;
    const int64_t end = begin + block_len < n ? begin + block_len : n;

    K code_and = ~(K)0, code_or = (K)0;
    count_range<K, CODE, THREADS, SPREAD>(keys, begin, end, h, tid, shift, mask, code_and, code_or);
    __shared__ unsigned long long wave_spread[SPREAD ? WAVES : 1][2];
    if constexpr (SPREAD) {
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            code_and &= __shfl_xor(code_and, o);
            code_or |= __shfl_xor(code_or, o);
        }
        if ((tid & (kWave - 1)) == 0) {
            wave_spread[tid / kWave][0] = (unsigned long long)code_and;
            wave_spread[tid / kWave][1] = (unsigned long long)code_or;
        }
    }
    __syncthreads();
    if constexpr (SPREAD) {
        if (tid == 0) {
            unsigned long long a = ~0ull, o = 0ull;
            for (int w = 0; w < WAVES; ++w) a &= wave_spread[w][0], o |= wave_spread[w][1];
            spread_out[2 * col] = a;
            spread_out[2 * col + 1] = o;
        }
    }

    for (int d = tid; d < RADIX; d += THREADS) {
        uint32_t s = 0;
#pragma unroll
        for (int w = 0; w < ROWS; ++w) s += hist[w][d];
        counts[(int64_t)d * num_blocks + col] = s;
    }
}

// ----------------------------------------------------------------------- scan

// Row d of the digit-major count matrix (num_blocks entries) becomes its
// exclusive prefix sums in place; row_total[d] gets the row's sum.  One
// workgroup per digit.  The digit starts (exclusive prefix of row_total) are
// formed by each downsweep workgroup from the 256 totals.
//
// The first scan of a sort that recorded its codes' spread (spread_cols, one
// AND and one OR per column) also combines them, in workgroup 0, into
// *diff_out; a later scan returns at once when its digit is constant.
template <int THREADS, int MAX_PER_THREAD>
__global__ __launch_bounds__(THREADS) void scan_kernel(uint32_t *__restrict__ counts,
                                                       uint32_t *__restrict__ row_total, int num_blocks,
                                                       const unsigned long long *__restrict__ spread_cols,
                                                       unsigned long long *__restrict__ diff_out,
                                                       const unsigned long long *__restrict__ diff_in, int shift,
                                                       uint32_t mask)
{
    if (spread_cols != nullptr && blockIdx.x == 0) {
        __shared__ unsigned long long s_spread[THREADS / kWave][2];
        unsigned long long a = ~0ull, o = 0ull;
        for (int c = threadIdx.x; c < num_blocks; c += THREADS) a &= spread_cols[2 * c], o |= spread_cols[2 * c + 1];
#pragma unroll
        for (int x = 1; x < kWave; x <<= 1) {
            a &= __shfl_xor(a, x);
            o |= __shfl_xor(o, x);
        }
        if ((threadIdx.x & (kWave - 1)) == 0) s_spread[threadIdx.x / kWave][0] = a, s_spread[threadIdx.x / kWave][1] = o;
        __syncthreads();
        if (threadIdx.x == 0) {
            for (int w = 1; w < THREADS / kWave; ++w) a &= s_spread[w][0], o |= s_spread[w][1];
            *diff_out = a ^ o;
        }
    }
    __shared__ uint32_t s_tmp[THREADS / kWave];
    uint32_t *row = counts + (int64_t)blockIdx.x * num_blocks;
    const int per = (num_blocks + THREADS - 1) / THREADS;
    const int first = threadIdx.x * per;
    uint32_t v[MAX_PER_THREAD];
#pragma unroll
    for (int i = 0; i < MAX_PER_THREAD; ++i) {
        const int idx = first + i;
        v[i] = (i < per && idx < num_blocks) ? row[idx] : 0u;
    }
    // (tested after the row's loads are issued, so the two latencies overlap)
    if (diff_in != nullptr && digit_constant(diff_in, shift, mask)) return;
    uint32_t sum = 0;
#pragma unroll
    for (int i = 0; i < MAX_PER_THREAD; ++i) sum += v[i];
    uint32_t total;
    uint32_t run = block_exclusive_scan<THREADS>(sum, s_tmp, total);
#pragma unroll
    for (int i = 0; i < MAX_PER_THREAD; ++i) {
        const int idx = first + i;
        if (i < per && idx < num_blocks) row[idx] = run;
        run += v[i];
    }
    if (threadIdx.x == 0) row_total[blockIdx.x] = total;
}

// ------------------------------------------------------------------ downsweep
//
// Stable rank and scatter of one digit, one workgroup per block (a contiguous
// run of tiles).  Tile layout: wave w owns keys [w*64*ITEMS, (w+1)*64*ITEMS)
// of the tile, item i of lane l is key w*64*ITEMS + i*64 + l, so each load
// instruction reads 64 consecutive keys and (item, lane) order is input order.
// Per tile: each wave ranks its keys among its own keys of the same digit
// (per-wave 16-bit counters in LDS, 64-lane match masks within an item), the
// waves' counts give every key its slot in the tile in digit order, the keys
// are written to LDS at those slots, and the tile is stored from LDS with
// consecutive threads on consecutive slots, so each digit's run goes out as
// consecutive addresses.
//
// Write combining.  A digit's run from one tile starts and ends inside 128-byte
// output lines.  Stored as is, the line it shares with the same digit's run
// from the next tile reaches HBM as two partial writes a tile apart, and
// partial line writes cost far more than their bytes (both in this kernel and
// in the next pass's reads of the lines).  So each workgroup holds, for every
// digit, the keys of the output line its run has opened but not filled (the
// carry: LINE positions per digit), and a tile stores only the carry keys and
// tile keys that complete a line.  The lines at the two ends of a block's range
// of a digit are shared with the neighbouring blocks and go out in parts; every
// other line is written whole, once.  The carry is in LDS for 32-bit keys
// alone and in registers otherwise (where the tile's LDS already allows only
// one workgroup per CU).
//
// Stores are buffer stores (outputs up to 2 GiB): a lane with nothing to store
// gives an offset past the output buffer, which the buffer's range check drops,
// so the carry stores and the register-carry path's stores sit in no branch.
// With the carry in LDS, a tile key is either stored or written to the carry,
// and one compare picks the side of an if/else (a select for the store offset
// cost a second compare and the select itself per key).  The wait for the next
// tile's loads stays exact: loads are issued on every path.  WIDE outputs use
// plain stores under a branch.

// Buffer resource over `bytes` bytes from `base`: buffer loads through it at
// byte offsets at or past `bytes` return zero without touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_over(const void *base, uint32_t bytes)
{
    // word 3: 32-bit data format, the setting for untyped loads on gfx9-family parts
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

constexpr int kNonTemporal = 2;  // cache-policy bit: streaming access

// A 4- or 8-byte buffer load with cache policy POLICY (0 or kNonTemporal).
template <typename K, int POLICY>
__device__ __forceinline__ K buffer_load_pol(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    if constexpr (sizeof(K) == 4) {
        return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, POLICY);
    } else {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, POLICY);
        return ((uint64_t)v[1] << 32) | v[0];
    }
}

// Issues the loads of one tile's keys (or values) for this lane: item i is
// element first + i*64 of the tile, which starts `tile_off` elements into the
// block that `r` covers.  The loads are non-temporal unless POLICY says
// otherwise: each key is read once per kernel, and keeping the stream out of
// L2 leaves it to the scattered output lines that are still being filled
// (64-bit pairs measured faster with ordinary loads: 0.355 ms per pass against
// 0.381 for 2^26 pairs; 32-bit keys, 32-bit pairs and 64-bit keys alone
// measured the same or slower).  Elements past the block's end
// (a short last tile, or a tile past the end) read as zero from the buffer's
// range check: there is no branch, so every call issues the same loads, and
// finish_tile overwrites such slots where they are used.  Nothing here waits
// for the loads.
template <typename K, int ITEMS, int POLICY = kNonTemporal>
__device__ __forceinline__ void issue_tile_loads(K (&k)[ITEMS], __amdgpu_buffer_rsrc_t r, uint32_t tile_off,
                                                 int first)
{
    const uint32_t off = (tile_off + (uint32_t)first) * (uint32_t)sizeof(K);
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) k[i] = buffer_load_pol<K, POLICY>(r, off + (uint32_t)(i * kWave * sizeof(K)));
}

// Gives slots past `valid` the padding key, whose digit is the largest of any
// pass, so they rank after every real key of the tile.
template <typename K, int CODE, int ITEMS>
__device__ __forceinline__ void finish_tile(K (&k)[ITEMS], int first, int valid, bool full)
{
    if (!full) {
#pragma unroll
        for (int i = 0; i < ITEMS; ++i)
            if (first + i * kWave >= valid) k[i] = pad_key<K, CODE>();
    }
}

constexpr uint32_t kStoreNowhere = 0x80000000u;  // byte offset past every narrow output buffer

template <typename K>
__device__ __forceinline__ void buffer_store(K x, __amdgpu_buffer_rsrc_t r, uint32_t off);
template <>
__device__ __forceinline__ void buffer_store<uint32_t>(uint32_t x, __amdgpu_buffer_rsrc_t r, uint32_t off)
{
    __builtin_amdgcn_raw_buffer_store_b32(x, r, off, 0, 0);
}
template <>
__device__ __forceinline__ void buffer_store<uint64_t>(uint64_t x, __amdgpu_buffer_rsrc_t r, uint32_t off)
{
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    u32x2 v;
    v[0] = (uint32_t)x;
    v[1] = (uint32_t)(x >> 32);
    __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, 0);
}

// Stores x at element `pos` of the output when `put`.
template <bool WIDE, typename T>
__device__ __forceinline__ void store_out(T x, T *out, __amdgpu_buffer_rsrc_t r, uint32_t pos, bool put)
{
    if constexpr (WIDE) {
        if (put) out[pos] = x;
    } else {
        buffer_store<T>(x, r, put ? pos * (uint32_t)sizeof(T) : kStoreNowhere);
    }
}

// Bits [a, b) of a lane mask, for 0 <= a and b <= 31 (empty when a >= b).
__device__ __forceinline__ uint32_t bit_range(uint32_t a, uint32_t b)
{
    return ((1u << b) - 1u) & ~((1u << a) - 1u);
}

// The lanes of the wave whose digit equals this lane's, through LDS: every
// lane clears its digit's 64-bit slot of the wave's table, sets its own bit
// there (an atomic OR on the slot's half that holds its bit, so the order of
// lanes does not matter) and reads the slot back.  DS operations of one wave
// complete in issue order, so the read sees every lane's bit.  Three LDS
// operations instead of the ballot form's 32 VALU instructions; the rank loop
// alternates the two forms so that neither the VALU nor the LDS pipe carries
// all of the matching.
__device__ __forceinline__ void match_digit_lds(unsigned long long *slot, uint32_t lane, uint32_t &lo,
                                                uint32_t &hi)
{
    *slot = 0ull;
    atomicOr(reinterpret_cast<uint32_t *>(slot) + (lane >> 5), 1u << (lane & 31u));
    const unsigned long long m = *slot;
    lo = (uint32_t)m;
    hi = (uint32_t)(m >> 32);
}

template <typename K, bool PAIRS>
constexpr bool carry_in_lds()
{
    return sizeof(K) == 4 && !PAIRS;
}

// Waves per SIMD the register allocation has to allow: 32-bit keys alone run
// 16 waves per CU (one 16-wave or two 8-wave workgroups); the other shapes 8.
template <typename K, bool PAIRS>
constexpr int downsweep_waves_per_simd()
{
    return carry_in_lds<K, PAIRS>() ? 4 : 2;
}

// Whether half of the rank's matching goes through the LDS table: everywhere
// except 8-wave workgroups of 32-bit keys alone, where the table's 16 KB would
// cost the second workgroup per CU.
template <typename K, bool PAIRS, int WAVES>
constexpr bool match_in_lds()
{
    return !(carry_in_lds<K, PAIRS>() && WAVES == 8);
}

template <typename K, bool PAIRS, int WAVES, int ITEMS>
struct DownsweepSmem {
    static constexpr int kThreads = WAVES * kWave;
    static constexpr int kTile = kThreads * ITEMS;
    static constexpr bool kCarryLds = carry_in_lds<K, PAIRS>();
    // Output line, in positions: 128 bytes of keys; with values, 128 bytes of
    // values (and 128 or 256 of keys).
    static constexpr uint32_t kLine = PAIRS ? 32u : 128u / (uint32_t)sizeof(K);
    // The carry, when in LDS: lane e of digit d holds output index (open line
    // of d) + e.  First, so that a lane's address is (d*kLine + e)*sizeof(K)
    // with no base.
    K carry[kCarryLds ? kRadix : 1][kCarryLds ? kLine : 1];
    K keys[kTile];                     // the tile in digit order
    uint32_t vals[PAIRS ? kTile : 1];  // payload in the same order
    // Per-wave 16-bit digit counters, two buffers alternating by tile: the
    // current tile counts in one; in the other, each wave's own row holds its
    // slot bases (tile slot of its first key of digit d) for the scatter.
    alignas(16) uint16_t wave_count[2][WAVES][kRadix];
    static constexpr bool kMatchLds = match_in_lds<K, PAIRS, WAVES>();
    alignas(16) unsigned long long match_table[kMatchLds ? WAVES : 1][kMatchLds ? kRadix : 1];  // match_digit_lds slots
    // Per digit d: {output index of tile slot 0 of d, end of the indices
    // stored from the tile}.
    alignas(16) uint2 place[kRadix];
    // Per digit d: {output index of d's open line, carry lanes to store} and,
    // for a carry in registers, {tile slot of the line left open after the
    // tile, carry lanes to reload from the tile}.
    alignas(16) std::conditional_t<kCarryLds, uint2, uint4> pend[kRadix];
};

template <typename K, bool PAIRS, int WAVES, int ITEMS, int CODE, bool WIDE>
__global__ __launch_bounds__(WAVES *kWave)
    __attribute__((amdgpu_waves_per_eu(downsweep_waves_per_simd<K, PAIRS>()))) void downsweep_kernel(
        SortBufs bufs, Route rt, int pass, int copy_if_idle, const uint32_t *__restrict__ counts,
        const uint32_t *__restrict__ row_total, int64_t n, int64_t block_len, int count_cols, int split, int shift,
        uint32_t mask, const unsigned long long *__restrict__ diff_in)
{
    using Smem = DownsweepSmem<K, PAIRS, WAVES, ITEMS>;
    constexpr int THREADS = Smem::kThreads;
    constexpr int TILE = Smem::kTile;
    constexpr int WAVE_KEYS = kWave * ITEMS;
    constexpr uint32_t LINE = Smem::kLine;
    constexpr bool CARRY_LDS = Smem::kCarryLds;
    constexpr int CARRY = (int)(kRadix * LINE) / THREADS;  // carry positions per thread
    // Units of place[]: byte offsets where the tile's stores use them directly
    // (32-bit keys alone, outputs below 2 GiB), else element indices.
    constexpr uint32_t PU = CARRY_LDS && !WIDE ? (uint32_t)sizeof(K) : 1u;
    constexpr uint32_t SB = sizeof(K) == 4 ? 4u : 1u;  // slot bases in bytes (4-byte keys) or slots
    constexpr int LOAD_POLICY = sizeof(K) == 8 && PAIRS ? 0 : kNonTemporal;  // see issue_tile_loads
    static_assert(THREADS >= kRadix, "one thread per digit is assumed");
    static_assert(TILE < 65536 && (TILE & (TILE - 1)) == 0, "16-bit ranks, power-of-two tile");
    static_assert(THREADS % LINE == 0 && (kRadix * LINE) % THREADS == 0, "carry lanes map evenly");
    __shared__ Smem s;

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // uniform: per-wave choices are scalar
    const int blk = blockIdx.x;
    const int64_t blk_begin = (int64_t)blk * block_len;
    const int64_t blk_end = blk_begin + block_len < n ? blk_begin + block_len : n;
    const uint32_t n32 = (uint32_t)n;

    // The codes' spread (more than one pass), read early.
    const unsigned long long diff = diff_in != nullptr ? *diff_in : 0ull;

    // Digit totals (4 digits per lane) and, for waves 0-3, this block's prefix
    // within one digit each: wave k owns digit 4*lane + k in the run
    // placement below.  The upsweep counted each block as `split` consecutive
    // sub-blocks (count_cols columns in all): the block's prefix is the one of
    // its first sub-block.
    const uint4 tot4 = reinterpret_cast<const uint4 *>(row_total)[lane];
    uint32_t before_own = 0u;
    if (wave < 4)
        before_own = counts[(int64_t)(4 * lane + wave) * count_cols + (int64_t)blk * split];

    // The skipped passes: from the codes' spread with more than one pass (a
    // later pass's counts are then never taken); a single pass is skipped when
    // one digit holds every key (every wave tests the totals itself, so the
    // decision is uniform without a barrier).
    const uint32_t skipset =
        diff_in != nullptr ? skipped_passes(rt, diff)
                           : (__ballot(tot4.x == n32 || tot4.y == n32 || tot4.z == n32 || tot4.w == n32) != 0 ? 1u : 0u);
    int ksrc, kdst, vsrc = 0, vdst = 0;
    pass_route(rt.kstart, rt.kb != 0, rt.passes, skipset, pass, ksrc, kdst);
    if constexpr (PAIRS) pass_route(rt.vstart, rt.vb != 0, rt.passes, skipset, pass, vsrc, vdst);
    if ((skipset >> pass) & 1u) {
        // Nothing to reorder.  The last pass's launch, when no copy follows
        // the sort, moves arrays that no pass moved to the output.
        if (copy_if_idle) move_to_output<K, PAIRS>(bufs, rt, skipset, n);
        return;
    }
    const K *__restrict__ keys_in = (const K *)bufs.keys[ksrc];
    K *__restrict__ keys_out = (K *)bufs.keys[kdst];
    const uint32_t *__restrict__ vals_in = PAIRS ? bufs.vals[vsrc] : nullptr;
    uint32_t *__restrict__ vals_out = PAIRS ? (uint32_t *)bufs.vals[vdst] : nullptr;

    // The block's first output index of its own digit (digit start plus the
    // block's prefix) and the next output index of that digit, in registers
    // of waves 0-3.
    uint32_t start_own = 0u;
    if (wave < 4) {
        const uint4 st = wave_scan_digits(tot4);
        start_own = (wave == 0 ? st.x : wave == 1 ? st.y : wave == 2 ? st.z : st.w) + before_own;
    }
    uint32_t run_own = start_own;

    // Makes the compiler wait here for a buffer's loads.
    auto ready = [](K(&kb)[ITEMS]) {
#pragma unroll
        for (int i = 0; i < ITEMS; ++i) asm volatile("" : "+v"(kb[i]));
    };

    // Lane's first key in a tile.  Re-derived from an opaque copy of the lane
    // index at each use: the per-item offsets built from it then fold into
    // the instructions that use them instead of being hoisted out of the loop
    // into ~50 registers.
    auto lane_first = [&]() {
        int tid_l = tid;
        asm volatile("" : "+v"(tid_l));
        return (tid_l / kWave) * WAVE_KEYS + (tid_l & (kWave - 1));
    };

    // The block's keys and values, as buffers: loads past the block's end
    // read zero.  A block holds at most 2^31 bytes of keys (the host keeps
    // blocks below that).  The outputs as buffers (used unless WIDE).
    const __amdgpu_buffer_rsrc_t keys_buf =
        buffer_over(keys_in + blk_begin, (uint32_t)((blk_end - blk_begin) * (int64_t)sizeof(K)));
    const __amdgpu_buffer_rsrc_t vals_buf =
        buffer_over(PAIRS ? vals_in + blk_begin : nullptr, PAIRS ? (uint32_t)((blk_end - blk_begin) * 4) : 0u);
    const __amdgpu_buffer_rsrc_t kout_buf = buffer_over(keys_out, WIDE ? 0u : (uint32_t)(n * (int64_t)sizeof(K)));
    const __amdgpu_buffer_rsrc_t vout_buf = buffer_over(vals_out, PAIRS && !WIDE ? n32 * 4u : 0u);

    // Issues the loads of the block's tile at tile_begin into kb.  The same
    // loads are issued whether or not the tile exists (past the block's end
    // they read zero and move no data): every path then has the same count of
    // memory operations in flight, so the compiler's wait counts stay exact
    // instead of falling back to waits that also cover the stores.
    auto prefetch = [&](K(&kb)[ITEMS], int64_t tile_begin) {
        issue_tile_loads<K, ITEMS, LOAD_POLICY>(kb, keys_buf, (uint32_t)(tile_begin - blk_begin), lane_first());
    };

    // A carry in registers: thread t holds positions (i*THREADS + t) % LINE
    // of digit (i*THREADS + t) / LINE, for i < CARRY.
    K ck[CARRY_LDS ? 1 : CARRY];
    uint32_t cv[PAIRS ? CARRY : 1];
#pragma unroll
    for (int i = 0; i < (CARRY_LDS ? 1 : CARRY); ++i) ck[i] = (K)0;
#pragma unroll
    for (int i = 0; i < (PAIRS ? CARRY : 1); ++i) cv[i] = 0u;

    // Ranks the tile at tile_begin (keys in kb) into LDS and writes out what it
    // completes.  `par` selects the counter buffer (tile parity in the block);
    // `final_tile` is set for the block's last tile, which also writes the
    // lines it leaves open.
    auto process_tile = [&](K(&kb)[ITEMS], int64_t tile_begin, int par, bool final_tile) {
        const int valid = blk_end - tile_begin < TILE ? (int)(blk_end - tile_begin) : TILE;
        const bool full = valid == TILE;
        const int first = lane_first();
        uint32_t v[ITEMS];
        if constexpr (PAIRS)
            issue_tile_loads<uint32_t, ITEMS, LOAD_POLICY>(v, vals_buf, (uint32_t)(tile_begin - blk_begin), first);
        finish_tile<K, CODE, ITEMS>(kb, first, valid, full);

        // This wave's digit counters start at zero for the tile.  Counters
        // alternate between two buffers by tile parity: the other waves read
        // this tile's counters after the barrier below, and the row being
        // cleared was last read by other waves in the tile before the
        // previous one (finished before the previous barrier) and by this
        // wave itself, as slot bases, in the previous tile.
        uint16_t(&count)[WAVES][kRadix] = s.wave_count[par];
        // This wave's counter row and slot-base row, addressed from one base
        // so that each item's address serves both.
        uint16_t *const row0 = &s.wave_count[0][wave][0];
        constexpr int kBufStride = WAVES * kRadix;
        reinterpret_cast<uint2 *>(count[wave])[lane] = make_uint2(0u, 0u);

        // Rank within the wave: keys of earlier items (all lanes), then keys of
        // this item in lower lanes with the same digit.  Every lane of a
        // same-digit group writes the group's new count (the same value), so
        // no lane has to be picked to do it.  The counter read is issued
        // before the match so its latency hides under it; the scheduling
        // fence keeps the compiler from hoisting every item's match at once
        // (which costs registers, not time).
        uint32_t r[ITEMS];
#pragma unroll
        for (int i = 0; i < ITEMS; ++i) {
            const uint32_t d = digit_of<CODE>(kb[i], shift, mask);
            uint16_t *counter = row0 + (par * kBufStride + (int)d);
            const uint32_t prior = *counter;
            uint32_t lo, hi;
            if ((i & 1) && Smem::kMatchLds)
                match_digit_lds(&s.match_table[Smem::kMatchLds ? wave : 0][Smem::kMatchLds ? d : 0], (uint32_t)lane,
                                lo, hi);
            else
                match_digit(d, lo, hi);
            // (the lane-count instructions add their accumulator operand for free)
            uint32_t part = __popc(lo) + prior;
            asm volatile("" : "+v"(part));  // keeps the two adds in the popcounts' accumulators
            *counter = (uint16_t)(__popc(hi) + part);
            r[i] = __builtin_amdgcn_mbcnt_hi(hi, __builtin_amdgcn_mbcnt_lo(lo, prior));
            asm volatile("" : "+v"(r[i]));  // formed here, so d and the masks die here
            __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();

        // With the carry in LDS: this thread's carry lanes, read now.  The
        // carry holds what the previous tile left (its writes came before the
        // barrier above), and every read here precedes the next barrier, after
        // which this tile's held-back keys overwrite it.
        K cx[CARRY_LDS ? CARRY : 1];
        if constexpr (CARRY_LDS) {
            int tid_c = tid;
            asm volatile("" : "+v"(tid_c));
#pragma unroll
            for (int i = 0; i < CARRY; ++i)
                cx[i] = s.carry[(uint32_t)i * (THREADS / LINE) + (uint32_t)tid_c / LINE][(uint32_t)tid_c % LINE];
        }

        // Every wave forms the digit offsets itself (4 digits per lane): its
        // own prefix over the waves before it, and the tile's exclusive prefix
        // over digits.  Redundant across waves, but it needs no second barrier
        // and no wave waits for another.
        uint4 tot, off;
        {
            // Two 16-bit counts per word: a tile's total per digit is below
            // 2^16, so the packed sums never carry into each other.
            uint2 sum = make_uint2(0u, 0u), pre = make_uint2(0u, 0u);
#pragma unroll
            for (int w = 0; w < WAVES; ++w) {
                const uint2 c = reinterpret_cast<const uint2 *>(count[w])[lane];
                if (w == wave) pre = sum;
                sum.x += c.x;
                sum.y += c.y;
            }
            tot = make_uint4(sum.x & 0xFFFFu, sum.x >> 16, sum.y & 0xFFFFu, sum.y >> 16);
            const uint4 before = make_uint4(pre.x & 0xFFFFu, pre.x >> 16, pre.y & 0xFFFFu, pre.y >> 16);
            off = wave_scan_digits(tot);
            // As byte offsets for 4-byte keys (below 2^16: a tile holds at
            // most 2^14 keys), so the scatter address is one shift-add.
            reinterpret_cast<uint2 *>(row0 + (par ^ 1) * kBufStride)[lane] =
                make_uint2(((before.x + off.x) * SB & 0xFFFFu) | ((before.y + off.y) * SB << 16),
                           ((before.z + off.z) * SB & 0xFFFFu) | ((before.w + off.w) * SB << 16));
        }

        // Reorder the tile in LDS: slot = tile offset of the digit + rank.
#pragma unroll
        for (int i = 0; i < ITEMS; ++i)
            r[i] = r[i] * SB + row0[(par ^ 1) * kBufStride + (int)digit_of<CODE>(kb[i], shift, mask)];
#pragma unroll
        for (int i = 0; i < ITEMS; ++i) {
            if constexpr (SB == 1) {
                s.keys[r[i]] = kb[i];
                if constexpr (PAIRS) s.vals[r[i]] = v[i];
            } else {
                *reinterpret_cast<K *>(reinterpret_cast<char *>(s.keys) + r[i]) = kb[i];
                if constexpr (PAIRS) *reinterpret_cast<uint32_t *>(reinterpret_cast<char *>(s.vals) + r[i]) = v[i];
            }
        }

        // Waves 0-3 place this tile's runs and plan its stores, wave k taking
        // digit 4*lane + k (the offsets are in every wave, 4 digits per lane).
        if (wave < 4) {
            const int k = wave;
            const uint32_t d = 4u * (uint32_t)lane + (uint32_t)k;
            const uint32_t tt = k == 0 ? tot.x : k == 1 ? tot.y : k == 2 ? tot.z : tot.w;
            const uint32_t of = k == 0 ? off.x : k == 1 ? off.y : k == 2 ? off.z : off.w;
            // The padding slots of a short last tile were counted under digit
            // `mask`; they sit after that digit's real keys and are never
            // stored.
            const uint32_t lo = run_own;
            const uint32_t hi = lo + tt - (d == mask ? (uint32_t)(TILE - valid) : 0u);
            const uint32_t base = lo - of;               // output index of tile slot 0 of the digit
            const uint32_t open = lo & ~(LINE - 1u);     // line holding the carry
            const uint32_t next = hi & ~(LINE - 1u);     // line left open after this tile
            // Carry lanes before the block's first index belong to the
            // previous block.
            const uint32_t first_idx = start_own;
            const uint32_t mine = first_idx > open ? first_idx - open : 0u;
            // The carry goes out when its line fills, or at the block's end
            // (never past n: only a key array changed under a running sort
            // could make the counts say otherwise).
            const uint32_t put_to = (final_tile || next > open) ? min(lo, n32) - min(open, n32) : 0u;
            // Lanes kept from the old carry (line still open) and loaded from
            // the tile.
            const uint32_t keep = next == open ? lo - open : 0u;
            const uint32_t fill = final_tile ? 0u : hi - next;
            s.place[d] = make_uint2(base * PU, min(final_tile ? hi : next, n32) * PU);
            if constexpr (CARRY_LDS)
                s.pend[d] = make_uint2(open, bit_range(mine, put_to));
            else
                s.pend[d] = make_uint4(open, bit_range(mine, put_to), next - base, bit_range(keep, fill));
            run_own = hi;
        }
        __syncthreads();

        // Stores: the carry lanes whose line fills, then the tile's keys up to
        // the last full line of their digit (all of them in the final tile),
        // then the new carry.  No barrier follows: LDS is next written after
        // the next tile's rank barrier.
        int tid_l = tid;
        asm volatile("" : "+v"(tid_l));
        const uint32_t e = (uint32_t)tid_l % LINE;
        const uint32_t drow = (uint32_t)tid_l / LINE;
        if constexpr (CARRY_LDS) {
            // Consecutive threads take consecutive lanes of a digit's carry
            // line: a wave stores whole lines.
            uint2 pe[CARRY];
#pragma unroll
            for (int i = 0; i < CARRY; ++i) pe[i] = s.pend[(uint32_t)i * (THREADS / LINE) + drow];
#pragma unroll
            for (int i = 0; i < CARRY; ++i)
                store_out<WIDE>(cx[i], keys_out, kout_buf, pe[i].x + e, ((pe[i].y >> e) & 1u) != 0u);
            // In phases, so that the LDS reads of all items are in flight
            // together rather than one item's at a time: the keys, then their
            // digits' placements, then the stores.  Keys past their digit's
            // last full line join the carry instead (in the final tile these
            // are padding slots, and the carry is dead).  Only those lanes
            // write (all lanes writing, the others to a spare row, measured
            // slower).
            K xk[ITEMS];
            uint2 pl[ITEMS];
#pragma unroll
            for (int i = 0; i < ITEMS; ++i) xk[i] = s.keys[i * THREADS + tid_l];
#pragma unroll
            for (int i = 0; i < ITEMS; ++i) pl[i] = s.place[digit_of<CODE>(xk[i], shift, mask)];
#pragma unroll
            for (int i = 0; i < ITEMS; ++i) {
                const uint32_t at = pl[i].x + (uint32_t)(i * THREADS + tid_l) * PU;  // in place[] units
                const bool held = at >= pl[i].y;
                if constexpr (WIDE) {
                    store_out<true>(xk[i], keys_out, kout_buf, at, !held);
                    if (held) s.carry[digit_of<CODE>(xk[i], shift, mask)][at & (LINE - 1u)] = xk[i];
                } else {
                    // stored, or kept at byte offset (lane (at / PU) % LINE) of
                    // the digit's carry row
                    if (!held)
                        buffer_store<K>(xk[i], kout_buf, at);
                    else
                        *reinterpret_cast<K *>(reinterpret_cast<char *>(&s.carry[0][0]) +
                                               ((digit_of<CODE>(xk[i], shift, mask) * LINE * PU) |
                                                (at & (LINE * PU - 1u)))) = xk[i];
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < CARRY; ++i) {
                const uint4 pe = s.pend[(uint32_t)i * (THREADS / LINE) + drow];
                const bool put = ((pe.y >> e) & 1u) != 0u;
                store_out<WIDE>(ck[i], keys_out, kout_buf, pe.x + e, put);
                if constexpr (PAIRS) store_out<WIDE>(cv[i], vals_out, vout_buf, pe.x + e, put);
            }
#pragma unroll
            for (int i = 0; i < ITEMS; ++i) {
                const uint32_t j = (uint32_t)(i * THREADS + tid_l);
                const K x = s.keys[j];
                const uint2 pl = s.place[digit_of<CODE>(x, shift, mask)];
                const uint32_t pos = pl.x + j;
                const bool put = pos < pl.y;
                store_out<WIDE>(x, keys_out, kout_buf, pos, put);
                if constexpr (PAIRS) store_out<WIDE>(s.vals[j], vals_out, vout_buf, pos, put);
            }
            // Re-read the carry descriptors rather than keep them live across
            // the stores (registers bound the workgroups per CU here).
            asm volatile("" ::: "memory");
#pragma unroll
            for (int i = 0; i < CARRY; ++i) {
                const uint4 pe = s.pend[(uint32_t)i * (THREADS / LINE) + drow];
                const bool take = ((pe.w >> e) & 1u) != 0u;
                const uint32_t slot = (pe.z + e) & (uint32_t)(TILE - 1);
                // Read unconditionally (the slot is always in the tile), so the
                // reload is a select rather than a branch per carry register.
                K x = s.keys[slot];
                asm volatile("" : "+v"(x));
                ck[i] = take ? x : ck[i];
                if constexpr (PAIRS) {
                    uint32_t y = s.vals[slot];
                    asm volatile("" : "+v"(y));
                    cv[i] = take ? y : cv[i];
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    // One tile ahead: tile t+1's loads are issued before tile t is ranked, so
    // they are in flight during its rank and ahead of its stores; the memory
    // counter is in order, so the wait for them (before tile t+1) never waits
    // for those stores.  Buffers a and b alternate, unrolled by two so each
    // stays in fixed registers, and a is ready at the loop head.
    K a[ITEMS], b[ITEMS];
    prefetch(a, blk_begin);
    ready(a);
    const int tiles = (int)((blk_end - blk_begin + TILE - 1) / TILE);
    const int pairs = (tiles - 1) / 2;
    int64_t ta = blk_begin;
    for (int p = 0; p < pairs; ++p, ta += 2 * TILE) {
        prefetch(b, ta + TILE);
        process_tile(a, ta, 0, false);
        ready(b);
        prefetch(a, ta + 2 * TILE);
        process_tile(b, ta + TILE, 1, false);
        ready(a);
    }
    if (tiles - 2 * pairs == 1) {
        process_tile(a, ta, 0, true);
    } else {
        prefetch(b, ta + TILE);
        process_tile(a, ta, 0, false);
        ready(b);
        process_tile(b, ta + TILE, 1, true);
    }
}

// ------------------------------------------------------ 2048-digit downsweep
//
// The downsweep of an 11-bit pass (2048 digits; three passes cover 32 bits
// instead of four: the kwkr.cn essay on bitonic vs. LSD radix sort, sections
// 3.4 and 5.2, and the page "GPU radix sort: from the CUB implementation to
// performance tuning", section 4, on the pass count against the cost of more
// buckets).  Same tile order and stable rank as the 8-bit downsweep, with
// what 2048 digits change:
//  - the match takes 11 ballots;
//  - per-wave counters cover 2048 digits (4 KB per wave), one buffer;
//  - the digit offsets of a tile come from a workgroup-wide scan, each thread
//    owning 4 digits and keeping their running output indices in registers;
//  - there is no write-combining carry (one open line per digit would take
//    256 KB of LDS): a tile's keys go from LDS straight to their output
//    positions, a digit's run of about 4 keys at a time.
// Eight waves, 16 keys per lane: 8,192-key tiles.
constexpr int kWideDigitWaves = 8;
constexpr int kWideDigitItems = 16;

template <typename K, bool PAIRS, int RB>
struct WideDigitSmem {
    static constexpr int kRadixW = 1 << RB;
    static constexpr int kTile = kWideDigitWaves * kWave * kWideDigitItems;
    K keys[kTile];                     // the tile in digit order
    uint32_t vals[PAIRS ? kTile : 1];  // payload in the same order
    // Per wave and digit: the tile's 16-bit counts, then (after the tile's
    // scan) the tile slot of the wave's first key of the digit.
    alignas(16) uint16_t wave_count[kWideDigitWaves][kRadixW];
    alignas(16) uint32_t place[kRadixW];  // output index of tile slot 0 of digit d (mod 2^32)
    uint32_t scan_tmp[kWideDigitWaves];
};

// Waves per SIMD for the register allocation: 32-bit keys alone fit two
// workgroups per CU in LDS.
template <typename K, bool PAIRS>
constexpr int wide_digit_waves_per_simd()
{
    return sizeof(K) == 4 && !PAIRS ? 4 : 2;
}

template <typename K, bool PAIRS, int RB, int CODE, bool WIDE>
__global__ __launch_bounds__(kWideDigitWaves *kWave)
    __attribute__((amdgpu_waves_per_eu(wide_digit_waves_per_simd<K, PAIRS>()))) void wide_digit_downsweep_kernel(
        SortBufs bufs, Route rt, int pass, int copy_if_idle, const uint32_t *__restrict__ counts,
        const uint32_t *__restrict__ row_total, int64_t n, int64_t block_len, int count_cols, int split, int shift,
        uint32_t mask, const unsigned long long *__restrict__ diff_in)
{
    using Smem = WideDigitSmem<K, PAIRS, RB>;
    constexpr int RADIX = Smem::kRadixW;
    constexpr int THREADS = kWideDigitWaves * kWave;
    constexpr int ITEMS = kWideDigitItems;
    constexpr int TILE = Smem::kTile;
    constexpr int WAVE_KEYS = kWave * ITEMS;
    static_assert(RADIX == 4 * THREADS, "each thread owns four digits");
    static_assert(TILE < 65536, "16-bit counts and slots");
    __shared__ Smem s;

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int blk = blockIdx.x;
    const int64_t blk_begin = (int64_t)blk * block_len;
    const int64_t blk_end = blk_begin + block_len < n ? blk_begin + block_len : n;
    const uint32_t n32 = (uint32_t)n;

    const unsigned long long diff = diff_in != nullptr ? *diff_in : 0ull;

    // This thread's digits 4*tid .. 4*tid+3: their totals, and the block's
    // prefix within each (the count column of the block's first sub-block).
    const uint4 tot4 = reinterpret_cast<const uint4 *>(row_total)[tid];
    uint32_t run[4];
    {
        const int64_t col = (int64_t)blk * split;
#pragma unroll
        for (int k = 0; k < 4; ++k) run[k] = counts[(int64_t)(4 * tid + k) * count_cols + col];
    }
    // The skipped passes, as in the 8-bit downsweep.
    const uint32_t skipset =
        diff_in != nullptr
            ? skipped_passes(rt, diff)
            : (__syncthreads_or(tot4.x == n32 || tot4.y == n32 || tot4.z == n32 || tot4.w == n32) != 0 ? 1u : 0u);
    int ksrc, kdst, vsrc = 0, vdst = 0;
    pass_route(rt.kstart, rt.kb != 0, rt.passes, skipset, pass, ksrc, kdst);
    if constexpr (PAIRS) pass_route(rt.vstart, rt.vb != 0, rt.passes, skipset, pass, vsrc, vdst);
    if ((skipset >> pass) & 1u) {
        if (copy_if_idle) move_to_output<K, PAIRS>(bufs, rt, skipset, n);
        return;
    }
    const K *__restrict__ keys_in = (const K *)bufs.keys[ksrc];
    K *__restrict__ keys_out = (K *)bufs.keys[kdst];
    const uint32_t *__restrict__ vals_in = PAIRS ? bufs.vals[vsrc] : nullptr;
    uint32_t *__restrict__ vals_out = PAIRS ? (uint32_t *)bufs.vals[vdst] : nullptr;

    // The block's first output index of each owned digit: the digit's start
    // (exclusive prefix of the totals over all digits) plus the block prefix.
    {
        uint32_t all;
        const uint32_t start = block_exclusive_scan<THREADS>(tot4.x + tot4.y + tot4.z + tot4.w, s.scan_tmp, all);
        run[0] += start;
        run[1] += start + tot4.x;
        run[2] += start + tot4.x + tot4.y;
        run[3] += start + tot4.x + tot4.y + tot4.z;
    }

    auto ready = [](K(&kb)[ITEMS]) {
#pragma unroll
        for (int i = 0; i < ITEMS; ++i) asm volatile("" : "+v"(kb[i]));
    };
    auto lane_first = [&]() {
        int tid_l = tid;
        asm volatile("" : "+v"(tid_l));
        return (tid_l / kWave) * WAVE_KEYS + (tid_l & (kWave - 1));
    };
    const __amdgpu_buffer_rsrc_t keys_buf =
        buffer_over(keys_in + blk_begin, (uint32_t)((blk_end - blk_begin) * (int64_t)sizeof(K)));
    const __amdgpu_buffer_rsrc_t vals_buf =
        buffer_over(PAIRS ? vals_in + blk_begin : nullptr, PAIRS ? (uint32_t)((blk_end - blk_begin) * 4) : 0u);
    const __amdgpu_buffer_rsrc_t kout_buf = buffer_over(keys_out, WIDE ? 0u : (uint32_t)(n * (int64_t)sizeof(K)));
    const __amdgpu_buffer_rsrc_t vout_buf = buffer_over(vals_out, PAIRS && !WIDE ? n32 * 4u : 0u);
    auto prefetch = [&](K(&kb)[ITEMS], int64_t tile_begin) {
        issue_tile_loads<K, ITEMS>(kb, keys_buf, (uint32_t)(tile_begin - blk_begin), lane_first());
    };

    auto process_tile = [&](K(&kb)[ITEMS], int64_t tile_begin) {
        const int valid = blk_end - tile_begin < TILE ? (int)(blk_end - tile_begin) : TILE;
        const bool full = valid == TILE;
        const int first = lane_first();
        uint32_t v[ITEMS];
        if constexpr (PAIRS) issue_tile_loads<uint32_t, ITEMS>(v, vals_buf, (uint32_t)(tile_begin - blk_begin), first);
        finish_tile<K, CODE, ITEMS>(kb, first, valid, full);

        // This wave's counters start at zero.  Its row was last read by this
        // wave's scatter in the previous tile, and by every thread's scan
        // before that tile's second barrier.
        uint16_t *const row = s.wave_count[wave];
#pragma unroll
        for (int q = 0; q < RADIX / (8 * kWave); ++q)
            reinterpret_cast<uint4 *>(row)[q * kWave + lane] = make_uint4(0u, 0u, 0u, 0u);

        // Rank within the wave, as in the 8-bit downsweep.
        uint32_t r[ITEMS];
#pragma unroll
        for (int i = 0; i < ITEMS; ++i) {
            const uint32_t d = digit_of<CODE>(kb[i], shift, mask);
            uint16_t *counter = row + d;
            const uint32_t prior = *counter;
            uint32_t lo, hi;
            match_digit<RB>(d, lo, hi);
            uint32_t part = __popc(lo) + prior;
            asm volatile("" : "+v"(part));
            *counter = (uint16_t)(__popc(hi) + part);
            r[i] = __builtin_amdgcn_mbcnt_hi(hi, __builtin_amdgcn_mbcnt_lo(lo, prior));
            asm volatile("" : "+v"(r[i]));
            __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();

        // Thread t's digits 4t..4t+3: each wave's prefix over the waves before
        // it (two 16-bit counts per word; a digit's tile total is below 2^16),
        // the tile's totals, and their exclusive prefix over all digits.
        uint2 pre[kWideDigitWaves];
        uint2 sum = make_uint2(0u, 0u);
#pragma unroll
        for (int w = 0; w < kWideDigitWaves; ++w) {
            const uint2 c = reinterpret_cast<const uint2 *>(s.wave_count[w])[tid];
            pre[w] = sum;
            sum.x += c.x;
            sum.y += c.y;
        }
        const uint32_t t0 = sum.x & 0xFFFFu, t1 = sum.x >> 16, t2 = sum.y & 0xFFFFu, t3 = sum.y >> 16;
        uint32_t all;
        const uint32_t o0 = block_exclusive_scan<THREADS>(t0 + t1 + t2 + t3, s.scan_tmp, all);
        const uint32_t o1 = o0 + t0, o2 = o1 + t1, o3 = o2 + t2;
        // Slot bases (only this thread touches these four columns), and the
        // output index of tile slot 0 of each digit.
        const uint2 off = make_uint2(o0 | (o1 << 16), o2 | (o3 << 16));
#pragma unroll
        for (int w = 0; w < kWideDigitWaves; ++w)
            reinterpret_cast<uint2 *>(s.wave_count[w])[tid] = make_uint2(off.x + pre[w].x, off.y + pre[w].y);
        reinterpret_cast<uint4 *>(s.place)[tid] = make_uint4(run[0] - o0, run[1] - o1, run[2] - o2, run[3] - o3);
        run[0] += t0;
        run[1] += t1;
        run[2] += t2;
        run[3] += t3;
        __syncthreads();

        // Reorder the tile in LDS.
#pragma unroll
        for (int i = 0; i < ITEMS; ++i) r[i] += row[digit_of<CODE>(kb[i], shift, mask)];
#pragma unroll
        for (int i = 0; i < ITEMS; ++i) {
            s.keys[r[i]] = kb[i];
            if constexpr (PAIRS) s.vals[r[i]] = v[i];
        }
        __syncthreads();

        // Store: consecutive threads take consecutive tile slots, so each
        // digit's run goes out as consecutive addresses.  Slots past `valid`
        // hold the padding keys (largest digit, after every real key).
#pragma unroll
        for (int i = 0; i < ITEMS; ++i) {
            const int j = i * THREADS + tid;
            const K x = s.keys[j];
            const uint32_t pos = s.place[digit_of<CODE>(x, shift, mask)] + (uint32_t)j;
            const bool put = j < valid;
            store_out<WIDE>(x, keys_out, kout_buf, pos, put);
            if constexpr (PAIRS) store_out<WIDE>(s.vals[j], vals_out, vout_buf, pos, put);
        }
    };

    // One tile ahead, as in the 8-bit downsweep.
    K a[ITEMS], b[ITEMS];
    prefetch(a, blk_begin);
    ready(a);
    const int tiles = (int)((blk_end - blk_begin + TILE - 1) / TILE);
    const int pairs = (tiles - 1) / 2;
    int64_t ta = blk_begin;
    for (int p = 0; p < pairs; ++p, ta += 2 * TILE) {
        prefetch(b, ta + TILE);
        process_tile(a, ta);
        ready(b);
        prefetch(a, ta + 2 * TILE);
        process_tile(b, ta + TILE);
        ready(a);
    }
    if (tiles - 2 * pairs == 1) {
        process_tile(a, ta);
    } else {
        prefetch(b, ta + TILE);
        process_tile(a, ta);
        ready(b);
        process_tile(b, ta + TILE);
    }
}

// ------------------------------------------------- small sorts: one launch a pass
//
// Below a few hundred thousand keys a sort is bound by launch latency and
// kernel-boundary drains, not bandwidth (the page "GPU radix sort: from the
// CUB implementation to performance tuning", sections 1 and 6, second
// pitfall: small inputs are dominated by launch overhead).  This pass does the
// histogram, scan and scatter of one digit in one launch, with no waiting
// between workgroups: every workgroup reads the whole input of the pass (a
// few hundred KB, held in L2) and counts its digits itself, those before its
// own chunk (its prefix) and those from its chunk on (the rest of the
// totals).  The totals' exclusive prefix gives each digit's start.  It then
// ranks its chunk of 1024 * ITEMS keys stably, as the downsweep does (ballot
// match within a wave, per-wave counters that follow input order, a prefix
// over the waves), and writes each key to digit start + prefix + rank.  The
// counting is repeated by every workgroup, which is what makes the pass need
// no upsweep, scan or second launch; it is cheap only while the input is
// small.
//
// Histograms: 32 copies, digit-major with the copy (lane % 32) minor, so the
// atomics of a wave's lanes fall in distinct banks except lanes l and l + 32.
constexpr int kSmallCopies = 32;

// Counts the digits of keys [0, n) into two banked histograms: keys before
// `split` into `before`, the others into `rest` (THREADS lanes striding
// together, 16-byte loads, four in flight per lane, where the array is 16-byte
// aligned and `split` a multiple of the keys per vector).
template <typename K, int CODE, int THREADS>
__device__ __forceinline__ void count_keys_banked(const K *__restrict__ keys, int n, int split, uint32_t *before,
                                                  uint32_t *rest, int tid, int shift, uint32_t mask)
{
    const int copy = tid & (kSmallCopies - 1);
    auto add = [&](K k, bool early) {
        atomicAdd((early ? before : rest) + digit_of<CODE>(k, shift, mask) * kSmallCopies + copy, 1u);
    };
    constexpr int PER = 16 / (int)sizeof(K);
    int from = 0;
    if ((((uintptr_t)keys & 15) == 0) && split % PER == 0) {
        const u32x4 *vk = reinterpret_cast<const u32x4 *>(keys);
        const int ve = n / PER, vsplit = split / PER;
        constexpr int UNROLL = 4;
        for (int base = 0; base < ve; base += THREADS * UNROLL) {
            u32x4 v[UNROLL];
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                const int i = base + u * THREADS + tid;
                v[u] = i < ve ? vk[i] : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                const int i = base + u * THREADS + tid;
                if (i < ve) {
                    const bool early = i < vsplit;
                    if constexpr (sizeof(K) == 4) {
                        add((K)v[u].x, early);
                        add((K)v[u].y, early);
                        add((K)v[u].z, early);
                        add((K)v[u].w, early);
                    } else {
                        add((K)(((uint64_t)v[u].y << 32) | v[u].x), early);
                        add((K)(((uint64_t)v[u].w << 32) | v[u].z), early);
                    }
                }
            }
        }
        from = ve * PER;
    }
    for (int i = from + tid; i < n; i += THREADS) add(keys[i], i < split);
}

template <typename K, bool PAIRS, int CODE, int ITEMS>
__global__ __launch_bounds__(1024) void small_pass_kernel(const K *__restrict__ keys_in,
                                                         const uint32_t *__restrict__ vals_in, K *__restrict__ keys_out,
                                                         uint32_t *__restrict__ vals_out, int n, int shift, uint32_t mask)
{
    constexpr int THREADS = 1024, WAVES = THREADS / kWave;
    constexpr int CHUNK = THREADS * ITEMS, WAVE_KEYS = kWave * ITEMS;
    __shared__ uint32_t before[kRadix * kSmallCopies];  // keys before the chunk
    __shared__ uint32_t rest[kRadix * kSmallCopies];    // keys from the chunk on
    __shared__ alignas(16) uint16_t wcount[WAVES][kRadix];
    __shared__ uint32_t base[kRadix];  // output index of the chunk's first key of each digit
    __shared__ uint32_t scan_tmp[WAVES];
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int start = blockIdx.x * CHUNK;

    for (int i = tid; i < kRadix * kSmallCopies; i += THREADS) before[i] = 0u, rest[i] = 0u;
    for (int i = tid; i < WAVES * kRadix / 2; i += THREADS) reinterpret_cast<uint32_t *>(&wcount[0][0])[i] = 0u;
    // this chunk's keys (and values), item i of lane l of wave w being key
    // start + w * WAVE_KEYS + i * 64 + l, so (item, lane) order is input order
    K k[ITEMS];
    uint32_t v[PAIRS ? ITEMS : 1];
    const int first = start + wave * WAVE_KEYS + lane;
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
        const int j = first + i * kWave;
        k[i] = j < n ? keys_in[j] : (K)0;
        if constexpr (PAIRS) v[i] = j < n ? vals_in[j] : 0u;
    }
    __syncthreads();
    count_keys_banked<K, CODE, THREADS>(keys_in, n, start, before, rest, tid, shift, mask);

    // rank within the wave, in input order
    uint32_t r[ITEMS];
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
        const bool valid = first + i * kWave < n;
        const uint32_t d = digit_of<CODE>(k[i], shift, mask);
        uint32_t lo, hi;
        match_digit(d, lo, hi);
        const uint64_t vm = __ballot(valid);
        lo &= (uint32_t)vm;
        hi &= (uint32_t)(vm >> 32);
        uint16_t *counter = &wcount[wave][d];
        const uint32_t prior = *counter;
        // every lane of a digit's group writes the same new count (a lane
        // past n writes its group's, or the unchanged count)
        *counter = (uint16_t)(prior + __popc(lo) + __popc(hi));
        r[i] = lanes_below(lo, hi) + prior;
    }
    __syncthreads();

    // thread t < 256, digit t: its count before the chunk and its total (the
    // copies read from a rotated start, so a wave's lanes spread over the
    // banks), and the waves' exclusive prefixes within the chunk (in place)
    uint32_t pre = 0u, all = 0u;
    if (tid < kRadix) {
#pragma unroll 8
        for (int c = 0; c < kSmallCopies; ++c) {
            pre += before[tid * kSmallCopies + ((c + tid) & (kSmallCopies - 1))];
            all += rest[tid * kSmallCopies + ((c + tid) & (kSmallCopies - 1))];
        }
        all += pre;
        uint32_t run = 0u;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) {
            const uint32_t c = wcount[w][tid];
            wcount[w][tid] = (uint16_t)run;
            run += c;
        }
    }
    uint32_t total;
    const uint32_t dstart = block_exclusive_scan<THREADS>(tid < kRadix ? all : 0u, scan_tmp, total);
    if (tid < kRadix) base[tid] = dstart + pre;
    __syncthreads();

#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
        if (first + i * kWave < n) {
            const uint32_t d = digit_of<CODE>(k[i], shift, mask);
            const uint32_t pos = base[d] + wcount[wave][d] + r[i];
            keys_out[pos] = k[i];
            if constexpr (PAIRS) vals_out[pos] = v[i];
        }
    }
}

// ---------------------------------------------------------------- tiny sorts
//
// A sort of at most NMAX keys in one launch and one workgroup, with the keys
// (and values) held in LDS for all passes: below some tens of thousands of
// keys a sort is dominated by launch latency (the page "GPU radix sort: from
// the CUB implementation to performance tuning", sections 1 and 6), and this
// takes one launch instead of three per pass.  The 16 waves each own a
// contiguous segment of the keys.  Per pass: each wave counts the digits of its
// segment; wave 0 turns the (digit, wave) counts into every wave's first slot
// per digit; then each wave walks its segment in input order, 64 keys at a
// time, ranking them with the ballot match and its own running offsets.  The
// walk needs no barrier, and equal digits keep input order: earlier waves hold
// earlier segments, and a wave ranks its keys in order.
template <typename K, bool PAIRS, int CODE, int NMAX>
__global__ __launch_bounds__(1024) void tiny_sort_kernel(const K *__restrict__ keys_in,
                                                        const uint32_t *__restrict__ vals_in,
                                                        K *__restrict__ keys_out, uint32_t *__restrict__ vals_out,
                                                        int n, int begin_bit, int end_bit)
{
    constexpr int THREADS = 1024, WAVES = THREADS / kWave;
    __shared__ K sk[2][NMAX];
    __shared__ uint32_t sv[PAIRS ? 2 : 1][PAIRS ? NMAX : 1];
    __shared__ alignas(16) uint32_t off[WAVES][kRadix];  // per wave: digit counts, then next slot per digit
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;

    for (int i = tid; i < n; i += THREADS) {
        sk[0][i] = keys_in[i];
        if constexpr (PAIRS) sv[0][i] = vals_in[i];
    }
    const int seg = ((n + WAVES - 1) / WAVES + kWave - 1) / kWave * kWave;
    const int sb = min(wave * seg, n), se = min(sb + seg, n);
    __syncthreads();

    int cur = 0;
    for (int shift = begin_bit; shift < end_bit; shift += kRadixBits, cur ^= 1) {
        const int width = min(kRadixBits, end_bit - shift);
        const uint32_t mask = (1u << width) - 1u;

        // counts of this wave's segment, in its own row
        for (int d = lane; d < kRadix; d += kWave) off[wave][d] = 0u;
        for (int i = sb + lane; i < se; i += kWave) atomicAdd(&off[wave][digit_of<CODE>(sk[cur][i], shift, mask)], 1u);
        __syncthreads();

        if (wave == 0) {
            uint32_t c[4][WAVES];
            uint4 tot = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
            for (int w = 0; w < WAVES; ++w) {
                const uint4 x = reinterpret_cast<const uint4 *>(off[w])[lane];
                c[0][w] = x.x; c[1][w] = x.y; c[2][w] = x.z; c[3][w] = x.w;
                tot.x += x.x; tot.y += x.y; tot.z += x.z; tot.w += x.w;
            }
            uint4 run = wave_scan_digits(tot);
#pragma unroll
            for (int w = 0; w < WAVES; ++w) {
                reinterpret_cast<uint4 *>(off[w])[lane] = run;
                run.x += c[0][w]; run.y += c[1][w]; run.z += c[2][w]; run.w += c[3][w];
            }
        }
        __syncthreads();

        for (int base = sb; base < se; base += kWave) {
            const int i = base + lane;
            const bool valid = i < se;
            const K k = valid ? sk[cur][i] : (K)0;
            uint32_t v = 0;
            if constexpr (PAIRS) v = valid ? sv[cur][i] : 0u;
            const uint32_t d = digit_of<CODE>(k, shift, mask);
            uint32_t lo, hi;
            match_digit(d, lo, hi);
            const uint64_t vm = __ballot(valid);
            lo &= (uint32_t)vm;
            hi &= (uint32_t)(vm >> 32);
            const uint32_t below = lanes_below(lo, hi);
            const uint32_t same = __popc(lo) + __popc(hi);
            uint32_t *counter = &off[wave][d];
            const uint32_t slot = *counter + below;
            if (valid) {
                sk[cur ^ 1][slot] = k;
                if constexpr (PAIRS) sv[cur ^ 1][slot] = v;
                if (below + 1u == same) *counter = slot + 1u;  // the group's last lane advances it
            }
        }
        __syncthreads();
    }

    for (int i = tid; i < n; i += THREADS) {
        keys_out[i] = sk[cur][i];
        if constexpr (PAIRS) vals_out[i] = sv[cur][i];
    }
}

// ------------------------------------------------------------------- finalize

// After the last pass of a sort with an in-place array: moves each array that
// ended outside the output there (an in-place array after an odd number of
// passes that run, when the second alternate buffer does not exist or only one
// pass runs).  Otherwise every workgroup returns at once.  With one pass the
// skip decision comes from the totals (one digit holding every key).
template <typename K, bool PAIRS>
__global__ __launch_bounds__(256) void finalize_kernel(SortBufs bufs, Route rt, const uint32_t *__restrict__ row_total,
                                                       int64_t n, const unsigned long long *__restrict__ diff_in)
{
    uint32_t skip;
    if (diff_in != nullptr) {
        skip = skipped_passes(rt, *diff_in);
    } else {
        bool all_one = false;
        for (int d = threadIdx.x; d < (1 << rt.digit_bits); d += blockDim.x) all_one |= row_total[d] == (uint32_t)n;
        skip = __syncthreads_or(all_one) ? 1u : 0u;
    }
    move_to_output<K, PAIRS>(bufs, rt, skip, n);
}

// ----------------------------------------------------------------------- copy

// Grid-stride copy of n16 16-byte vectors: each lane moves one vector per
// step, the grid sized to the chip's resident waves (16 per CU), loads and
// stores non-temporal.  Measured on MI355X for 400 MB: 6.2 TB/s, against 5.3
// for plain stores with eight times the workgroups, and the next kernel reads
// the copy at full speed (lines written with plain stores stay in the
// memory-side cache and slow the next reader by a fifth).
__global__ __launch_bounds__(256) void copy16_kernel(const uint4 *__restrict__ src, uint4 *__restrict__ dst,
                                                     int64_t n16)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const u32x4 *s4 = reinterpret_cast<const u32x4 *>(src);
    u32x4 *d4 = reinterpret_cast<u32x4 *>(dst);
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
        __builtin_nontemporal_store(__builtin_nontemporal_load(&s4[i]), &d4[i]);
}

// Reads n16 16-byte vectors (grid-stride, non-temporal) and folds each lane's
// words into one xor: the streaming-read reference a benchmark times beside
// the sort.  A lane whose fold equals kReadMarker writes it to *result, so the
// loads have an effect the compiler must keep (one shared atomic per wave
// instead would serialize thousands of atomics on one address and time those).
constexpr uint32_t kReadMarker = 0x9E3779B9u;
__global__ __launch_bounds__(256) void read16_kernel(const uint4 *__restrict__ src, int64_t n16,
                                                     uint32_t *__restrict__ result)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const u32x4 *s4 = reinterpret_cast<const u32x4 *>(src);
    uint32_t acc = 0u;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
        const u32x4 v = __builtin_nontemporal_load(&s4[i]);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == kReadMarker) *result = acc;
}

// Grid-stride byte copy (unaligned heads and tails).
__global__ __launch_bounds__(256) void copy1_kernel(const uint8_t *__restrict__ src, uint8_t *__restrict__ dst,
                                                    int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

}  // namespace lrs
