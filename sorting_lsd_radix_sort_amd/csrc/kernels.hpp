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
//              tile with 64-lane ballots, reorders the tile through LDS so that
//              each digit's keys are contiguous, and writes them to
//              digit_start[d] + block_prefix[d] + (keys of digit d in earlier
//              tiles of the block) + rank.
//
// Counting per block of many tiles instead of per tile keeps the count matrix a
// few MB at any n (so the scan is cheap), and lets a workgroup continue each
// digit's output run from one tile to the next, so partial cache lines at a
// run's end are completed by the same workgroup through its own L2.
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

namespace lrs {

constexpr int kRadixBits = 8;
constexpr int kRadix = 1 << kRadixBits;
constexpr int kWave = 64;

// ------------------------------------------------------------------ key codes

// Float32 bit pattern -> order-preserving unsigned word (kwkr.cn essay,
// section 3.3): sign clear -> set the sign bit; sign set -> invert all bits.
__device__ __forceinline__ uint32_t encode_f32(uint32_t b)
{
    return b ^ ((uint32_t)((int32_t)b >> 31) | 0x80000000u);
}

// Inverse of encode_f32: top bit set -> clear it; top bit clear -> invert all.
__device__ __forceinline__ uint32_t decode_f32(uint32_t u)
{
    return u ^ (~(uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

template <typename K>
__device__ __forceinline__ uint32_t digit_of(K k, int shift, uint32_t mask)
{
    return (uint32_t)(k >> shift) & mask;
}

// --------------------------------------------------------------- wave helpers

// Lanes of the wave whose 8-bit digit equals this lane's: for each digit bit,
// keep the lanes whose ballot bit agrees with ours.  All 64 lanes must be
// active.  v_bitop3 0x90 computes m & ~(ballot ^ t): with t all-ones when our
// bit is set it keeps the ballot, otherwise its complement.
__device__ __forceinline__ void match_digit(uint32_t d, uint32_t &lo, uint32_t &hi)
{
    lo = 0xFFFFFFFFu;
    hi = 0xFFFFFFFFu;
#pragma unroll
    for (int b = 0; b < kRadixBits; ++b) {
        const uint32_t t = (uint32_t)((int32_t)(d << (31 - b)) >> 31);
        const uint64_t bal = __ballot(t != 0u);
        lo = __builtin_amdgcn_bitop3_b32(lo, (uint32_t)bal, t, 0x90);
        hi = __builtin_amdgcn_bitop3_b32(hi, (uint32_t)(bal >> 32), t, 0x90);
    }
}

// Number of set bits of (hi:lo) in lanes below this one.
__device__ __forceinline__ uint32_t lanes_below(uint32_t lo, uint32_t hi)
{
    return __builtin_amdgcn_mbcnt_hi(hi, __builtin_amdgcn_mbcnt_lo(lo, 0u));
}

// Exclusive prefix sum of one value per thread over the whole workgroup.
// s_tmp needs THREADS/64 words.  Every thread must call it (it synchronizes).
template <int THREADS>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t *s_tmp, uint32_t &total)
{
    constexpr int WAVES = THREADS / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    uint32_t x = v;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const uint32_t y = __shfl_up(x, off, kWave);
        if (lane >= off) x += y;
    }
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

// -------------------------------------------------------------------- upsweep

// Counts the digits of block b = keys [b * block_len, min(n, (b+1) * block_len)).
// Each wave adds into its own 256-bin LDS histogram, so atomics only contend
// within a wave (the kwkr.cn essay, section 3.2, and the quant67.com survey,
// section 8.1: per-block and per-warp counting instead of global atomics).
// VEC loads 16 bytes per lane when the key array is 16-byte aligned.
template <typename K, bool ENCODE, int THREADS, bool VEC>
__global__ __launch_bounds__(THREADS) void upsweep_kernel(
    const K *__restrict__ keys, uint32_t *__restrict__ counts, int64_t n, int64_t block_len,
    int num_blocks, int shift, uint32_t mask)
{
    constexpr int WAVES = THREADS / kWave;
    __shared__ uint32_t hist[WAVES][kRadix];
    const int tid = threadIdx.x;
    uint32_t *h = hist[tid / kWave];
    for (int i = tid; i < WAVES * kRadix; i += THREADS) (&hist[0][0])[i] = 0u;
    __syncthreads();

    const int64_t begin = (int64_t)blockIdx.x * block_len;
    const int64_t end = begin + block_len < n ? begin + block_len : n;

    auto count_key = [&](K k) {
        if constexpr (ENCODE) k = (K)encode_f32((uint32_t)k);
        atomicAdd(&h[digit_of(k, shift, mask)], 1u);
    };

    int64_t scalar_from = begin;
    if constexpr (VEC) {
        // 16-byte vectors: 4 uint32 or 2 uint64 keys each.  `begin` is a whole
        // number of tiles, hence of vectors.
        constexpr int PER = 16 / (int)sizeof(K);
        constexpr int UNROLL = 4;
        using V = uint4;
        const V *vk = reinterpret_cast<const V *>(keys);
        const int64_t vbeg = begin / PER, vend = end / PER;
        for (int64_t base = vbeg; base < vend; base += (int64_t)THREADS * UNROLL) {
            V v[UNROLL];
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                const int64_t i = base + (int64_t)u * THREADS + tid;
                if (i < vend) v[u] = vk[i];
            }
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                const int64_t i = base + (int64_t)u * THREADS + tid;
                if (i < vend) {
                    if constexpr (sizeof(K) == 4) {
                        count_key((K)v[u].x); count_key((K)v[u].y);
                        count_key((K)v[u].z); count_key((K)v[u].w);
                    } else {
                        count_key((K)(((uint64_t)v[u].y << 32) | v[u].x));
                        count_key((K)(((uint64_t)v[u].w << 32) | v[u].z));
                    }
                }
            }
        }
        scalar_from = vend * PER;
    }
    for (int64_t i = scalar_from + tid; i < end; i += THREADS) count_key(keys[i]);
    __syncthreads();

    for (int d = tid; d < kRadix; d += THREADS) {
        uint32_t s = 0;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) s += hist[w][d];
        counts[(int64_t)d * num_blocks + blockIdx.x] = s;
    }
}

// ----------------------------------------------------------------------- scan

// Row d of the digit-major count matrix (num_blocks entries) becomes its
// exclusive prefix sums in place; row_total[d] gets the row's sum.  One
// workgroup per digit.  The digit starts (exclusive prefix of row_total) are
// formed by each downsweep workgroup from the 256 totals.
template <int THREADS, int MAX_PER_THREAD>
__global__ __launch_bounds__(THREADS) void scan_kernel(uint32_t *__restrict__ counts,
                                                       uint32_t *__restrict__ row_total, int num_blocks)
{
    __shared__ uint32_t s_tmp[THREADS / kWave];
    uint32_t *row = counts + (int64_t)blockIdx.x * num_blocks;
    const int per = (num_blocks + THREADS - 1) / THREADS;
    const int first = threadIdx.x * per;
    uint32_t v[MAX_PER_THREAD];
    uint32_t sum = 0;
#pragma unroll
    for (int i = 0; i < MAX_PER_THREAD; ++i) {
        const int idx = first + i;
        v[i] = (i < per && idx < num_blocks) ? row[idx] : 0u;
        sum += v[i];
    }
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

template <typename K, int WAVES, int ITEMS>
struct DownsweepSmem {
    static constexpr int kThreads = WAVES * kWave;
    static constexpr int kTile = kThreads * ITEMS;
    union {
        K keys[kTile];
        uint32_t vals[kTile];
    } x;
    uint32_t wave_count[WAVES][kRadix];  // per-wave digit counters, then offsets
    uint32_t out_base[kRadix];           // global index of tile slot 0 of digit d
    uint32_t run[kRadix];                // next global index of digit d in this block
    uint32_t scan_tmp[WAVES];
};

// Stable rank + scatter of block b's tiles for one digit.  Tile layout: wave w
// owns keys [w*64*ITEMS, (w+1)*64*ITEMS) of the tile, item i of lane l is key
// w*64*ITEMS + i*64 + l, so each load instruction reads 64 consecutive keys and
// (item, lane) order is input order.  Slots past the end of the input (only in
// the last tile) take digit 255 and rank after every real key, so they land in
// the tile's last slots and are never written.
template <typename K, bool PAIRS, int WAVES, int ITEMS, bool ENCODE, bool DECODE>
__global__ __launch_bounds__(WAVES * kWave) void downsweep_kernel(
    const K *__restrict__ keys_in, K *__restrict__ keys_out, const uint32_t *__restrict__ vals_in,
    uint32_t *__restrict__ vals_out, const uint32_t *__restrict__ counts,
    const uint32_t *__restrict__ row_total, int64_t n, int64_t block_len, int num_blocks, int shift,
    uint32_t mask)
{
    using Smem = DownsweepSmem<K, WAVES, ITEMS>;
    constexpr int THREADS = Smem::kThreads;
    constexpr int TILE = Smem::kTile;
    constexpr int WAVE_KEYS = kWave * ITEMS;
    static_assert(THREADS >= kRadix, "one thread per digit is assumed");
    __shared__ Smem s;

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int blk = blockIdx.x;
    const int64_t blk_begin = (int64_t)blk * block_len;
    const int64_t blk_end = blk_begin + block_len < n ? blk_begin + block_len : n;

    {   // digit starts, then this block's first output index per digit
        uint32_t total;
        const uint32_t t = tid < kRadix ? row_total[tid] : 0u;
        const uint32_t start = block_exclusive_scan<THREADS>(t, s.scan_tmp, total);
        if (tid < kRadix) s.run[tid] = start + counts[(int64_t)tid * num_blocks + blk];
    }

    for (int64_t tile_begin = blk_begin; tile_begin < blk_end; tile_begin += TILE) {
        const int valid = blk_end - tile_begin < TILE ? (int)(blk_end - tile_begin) : TILE;
        const int wave_first = wave * WAVE_KEYS;

        K k[ITEMS];
        uint32_t d[ITEMS];
        uint32_t v[ITEMS];
        if (valid == TILE) {
#pragma unroll
            for (int i = 0; i < ITEMS; ++i) {
                const int local = wave_first + i * kWave + lane;
                k[i] = keys_in[tile_begin + local];
                if constexpr (PAIRS) v[i] = vals_in[tile_begin + local];
            }
#pragma unroll
            for (int i = 0; i < ITEMS; ++i) {
                if constexpr (ENCODE) k[i] = (K)encode_f32((uint32_t)k[i]);
                d[i] = digit_of(k[i], shift, mask);
            }
        } else {
#pragma unroll
            for (int i = 0; i < ITEMS; ++i) {
                const int local = wave_first + i * kWave + lane;
                if (local < valid) {
                    K x = keys_in[tile_begin + local];
                    if constexpr (ENCODE) x = (K)encode_f32((uint32_t)x);
                    k[i] = x;
                    d[i] = digit_of(x, shift, mask);
                    if constexpr (PAIRS) v[i] = vals_in[tile_begin + local];
                } else {
                    k[i] = 0;
                    d[i] = kRadix - 1;
                    if constexpr (PAIRS) v[i] = 0u;
                }
            }
        }

        // This wave's digit counters start at zero for the tile.
#pragma unroll
        for (int j = 0; j < kRadix / kWave; ++j) s.wave_count[wave][lane + j * kWave] = 0u;

        // Rank within the wave: keys of earlier items (all lanes), then keys of
        // this item in lower lanes with the same digit.  The last lane of each
        // same-digit group advances the wave's counter for that digit.
        uint32_t r[ITEMS];
#pragma unroll
        for (int i = 0; i < ITEMS; ++i) {
            uint32_t lo, hi;
            match_digit(d[i], lo, hi);
            const uint32_t below = lanes_below(lo, hi);
            const uint32_t same = __popc(lo) + __popc(hi);
            const uint32_t prior = s.wave_count[wave][d[i]];
            if (below + 1u == same) s.wave_count[wave][d[i]] = prior + same;
            r[i] = prior + below;
        }
        __syncthreads();

        // Per digit: exclusive prefix over waves, tile count, tile offset.
        uint32_t tile_count = 0;
        if (tid < kRadix) {
#pragma unroll
            for (int w = 0; w < WAVES; ++w) {
                const uint32_t c = s.wave_count[w][tid];
                s.wave_count[w][tid] = tile_count;
                tile_count += c;
            }
        }
        uint32_t tile_total;
        const uint32_t tile_off = block_exclusive_scan<THREADS>(tile_count, s.scan_tmp, tile_total);
        if (tid < kRadix) {
#pragma unroll
            for (int w = 0; w < WAVES; ++w) s.wave_count[w][tid] += tile_off;
            const uint32_t run = s.run[tid];
            s.out_base[tid] = run - tile_off;
            const uint32_t pad = (tid == kRadix - 1) ? (uint32_t)(TILE - valid) : 0u;
            s.run[tid] = run + tile_count - pad;
        }
        __syncthreads();

        // Reorder the tile in LDS: slot = tile offset of the digit + rank.
        uint32_t slot[ITEMS];
#pragma unroll
        for (int i = 0; i < ITEMS; ++i) {
            slot[i] = s.wave_count[wave][d[i]] + r[i];
            s.x.keys[slot[i]] = k[i];
        }
        __syncthreads();

        // Consecutive threads take consecutive slots: each digit's run of slots
        // goes to consecutive global addresses.  The dest < n test never fails
        // when the counts of upsweep and downsweep agree (same keys, same
        // digit); it keeps a key array changed between the two kernels (a
        // caller race) from turning into stores outside the output.
        const uint32_t n32 = (uint32_t)n;
        uint32_t dest[ITEMS];
#pragma unroll
        for (int i = 0; i < ITEMS; ++i) {
            const int j = i * THREADS + tid;
            dest[i] = n32;
            if (j < valid) {
                const K x = s.x.keys[j];
                dest[i] = s.out_base[digit_of(x, shift, mask)] + (uint32_t)j;
                K y = x;
                if constexpr (DECODE) y = (K)decode_f32((uint32_t)x);
                if (dest[i] < n32) keys_out[dest[i]] = y;
            }
        }
        if constexpr (PAIRS) {
            __syncthreads();
#pragma unroll
            for (int i = 0; i < ITEMS; ++i) s.x.vals[slot[i]] = v[i];
            __syncthreads();
#pragma unroll
            for (int i = 0; i < ITEMS; ++i) {
                const int j = i * THREADS + tid;
                if (j < valid && dest[i] < n32) vals_out[dest[i]] = s.x.vals[j];
            }
        }
        __syncthreads();
    }
}

// ----------------------------------------------------------------------- copy

// Grid-stride copy of n16 16-byte vectors.
__global__ __launch_bounds__(256) void copy16_kernel(const uint4 *__restrict__ src, uint4 *__restrict__ dst,
                                                     int64_t n16)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

// Grid-stride byte copy (unaligned heads and tails).
__global__ __launch_bounds__(256) void copy1_kernel(const uint8_t *__restrict__ src, uint8_t *__restrict__ dst,
                                                    int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

}  // namespace lrs
