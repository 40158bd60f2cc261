// lrsort.hip -- host side of the C ABI in include/lrsort.h: argument checks,
// pass plan, temp-storage layout and kernel launches on the caller's stream.
//
// A sort over [begin_bit, end_bit) runs P = ceil((end_bit - begin_bit) / 8)
// passes, pass p sorting by bits [begin_bit + 8p, min(begin_bit + 8p + 8,
// end_bit)) (the page "GPU radix sort: from the CUB implementation to
// performance tuning", section 2: one call over [0, 32) equals four 8-bit calls
// with the source and destination swapped after each).  Each pass enqueues
// upsweep -> scan -> downsweep with no host synchronization.
//
// Buffers: pass 0 reads the input and the last pass writes the output; the
// passes in between ping-pong through an alternate buffer A in temp storage, the
// first destination being chosen by the parity of P so that the last pass lands
// in the output (same page, section 6, third pitfall: know which buffer holds
// the last pass).  When input and output are the same array and P is odd, pass 0
// cannot write the output it is still reading, so a second alternate buffer B is
// used (P >= 3) or the result is copied from A (P == 1).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <map>
#include <mutex>
#include <vector>

#include "kernels.hpp"
#include "lrsort.h"
#include "lrsort_prof.h"

#define LRS_API extern "C" __attribute__((visibility("default")))

namespace {

using namespace lrs;

// Key types; each selects a storage width and an order code (order_code in
// kernels.hpp) through run_kind's template arguments.
enum KeyKind { KIND_U32, KIND_I32, KIND_F32, KIND_U64, KIND_I64, KIND_F64 };
int key_bytes(KeyKind k) { return k == KIND_U64 || k == KIND_I64 || k == KIND_F64 ? 8 : 4; }

constexpr int kMaxBlocks = 4096;  // count-matrix width cap (scan: 256 threads x 16)
constexpr int kWideDigitBits = 11;  // the other digit width lrs_sort_digits takes
constexpr int kMaxSplit = 8;      // upsweep sub-blocks per downsweep block
constexpr int kUpsweepThreads = 512;
constexpr int kScanThreads = 256;
constexpr int kScanPerThread = kMaxBlocks / kScanThreads;
constexpr size_t kAlign = 256;

// The most keys the one-workgroup sort (tiny_sort_kernel) can hold: two
// copies of the keys and values in 128 KB of LDS.  It is used up to the
// smaller of this and kTinyMaxKeys.
template <typename K, bool PAIRS>
constexpr int tiny_max()
{
    return (64 * 1024) / (int)(sizeof(K) + (PAIRS ? 4 : 0)) >= 16384 ? 16384
           : (64 * 1024) / (int)(sizeof(K) + (PAIRS ? 4 : 0)) >= 8192 ? 8192
                                                                       : 4096;
}

// Downsweep tile shapes, 16 keys per lane throughout.  32-bit keys alone run
// 16 waves (16,384-key tiles; the carry of the write-combining stores fits in
// LDS beside the tile, one workgroup per CU) from 2^21 keys; longer tiles give
// each digit longer runs and spread the per-tile work (the digit scan, the
// carry stores) over more keys.  Below that (where the 8-wave shape measured
// faster: more workgroups for the same n), and for pairs and 64-bit keys, 8
// waves (8,192-key tiles).
// Up to 2^17 keys the sort is latency-bound (a few tiles per pass), and
// 2,048-key tiles (8 waves x 4 keys per lane) give it more workgroups: 50 us
// instead of 58 for 65,536 uint32 keys.
constexpr int kItems = 16;
constexpr int kSmallItems = 4;
constexpr int64_t kWideTileMinKeys = (int64_t)1 << 21;
constexpr int64_t kSmallTileMaxKeys = (int64_t)1 << 17;
// Sorts of up to kSmallPassMaxBytes of keys (8-bit digits) take one launch per
// pass (small_pass_kernel), whose workgroups each reread the whole input, 1024
// keys per workgroup.  Measured on MI355X (uint32 keys / pairs): 65,536 keys in
// 30 / 33 us against 48 / 54 on the three-kernel path; even at 200,000 keys
// (58 / 63 against 61 / 70); slower from about 225,000.
constexpr int64_t kSmallPassMaxBytes = 800000;
// The one-workgroup sort wins below this many keys (6,144 uint32 keys: 16.9 us
// against 18.6 for four small passes; 8,192: 20.9 against 19.2).
constexpr int64_t kTinyMaxKeys = 6144;
constexpr bool wide_tiles(int kbytes, bool pairs, int64_t n) { return kbytes == 4 && !pairs && n >= kWideTileMinKeys; }
int tile_keys(KeyKind kind, bool pairs, int64_t n)
{
    if (n <= kSmallTileMaxKeys) return 8 * 64 * kSmallItems;
    return (wide_tiles(key_bytes(kind), pairs, n) ? 16 : 8) * 64 * kItems;
}

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// ------------------------------------------------------------------ profiling

// Recording is off unless a benchmark turns it on.  A launch only tests the
// flag; while it is on, each launch takes the mutex, reserves its record slot
// (bounds-checked) and records its events under it, so threads that launch
// concurrently, or that start, read or release the records meanwhile, never
// share a slot or touch a vector being reassigned.
struct Prof {
    std::atomic<bool> on{false};
    std::mutex mu;
    int cap = 0;
    int count = 0;
    std::vector<hipEvent_t> ev;  // 2 per record
    std::vector<int> kind;
};
Prof g_prof;

template <typename F>
hipError_t launch(int kind, hipStream_t stream, F &&f)
{
    if (!g_prof.on.load(std::memory_order_acquire)) {
        f();
        return hipGetLastError();
    }
    std::lock_guard<std::mutex> lock(g_prof.mu);
    const int slot = g_prof.on.load(std::memory_order_relaxed) && g_prof.count < g_prof.cap ? g_prof.count++ : -1;
    if (slot >= 0) (void)hipEventRecord(g_prof.ev[2 * slot], stream);
    f();
    const hipError_t err = hipGetLastError();
    if (slot >= 0) {
        (void)hipEventRecord(g_prof.ev[2 * slot + 1], stream);
        g_prof.kind[slot] = kind;
    }
    return err;
}

// --------------------------------------------------------------- device info

struct DevInfo {
    bool ready = false;
    int cus = 0;
};
std::mutex g_dev_mu;
DevInfo g_dev[64];

hipError_t device_cus(int *cus)
{
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_dev_mu);
    if (!g_dev[dev].ready) {
        int n = 0;
        err = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
        if (err != hipSuccess) return err;
        g_dev[dev].cus = n;
        g_dev[dev].ready = true;
    }
    *cus = g_dev[dev].cus;
    return hipSuccess;
}

// Resident workgroups per CU of a kernel, cached per kernel and device.  The
// cache is keyed by the kernel's address: kernels of one signature (keys only
// and pairs, say) share a function type but not an occupancy.
hipError_t occupancy(const void *kern, int threads, int *per_cu)
{
    static std::mutex mu;
    static std::map<std::pair<int, const void *>, int> cache;
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find({dev, kern});
    if (it == cache.end()) {
        int nb = 0;
        err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kern, threads, 0);
        if (err != hipSuccess) return err;
        it = cache.emplace(std::make_pair(dev, kern), nb > 0 ? nb : 1).first;
    }
    *per_cu = it->second;
    return hipSuccess;
}

// -------------------------------------------------------------------- plan

// Which alternate buffers a sort needs in temp storage.  The passes alternate
// between buffers so that, with no pass skipped, the last one writes the
// output (the kernels derive each pass's buffers from the same rule, with the
// skipped passes left out; run_dest in kernels.hpp):
//  - an array that starts in the input needs A when it runs two passes or more;
//  - an in-place array (input and output the same memory) goes out to A and
//    comes back, and with an odd number of passes, three or more, it also uses
//    B so that its last pass still writes the output (with one pass, the pass
//    writes A and a copy moves the result back).
struct Plan {
    bool need_a = false;
    bool need_b = false;
};

Plan make_plan(int passes, bool in_place)
{
    Plan pl;
    if (passes == 0) return pl;
    pl.need_a = in_place || passes >= 2;
    pl.need_b = in_place && passes % 2 == 1 && passes >= 3;
    return pl;
}

bool overlap_partial(const void *a, const void *b, size_t bytes)
{
    if (a == b || bytes == 0) return false;
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + bytes && y < x + bytes;
}

struct Request {
    KeyKind kind;
    const void *keys_in;
    void *keys_out;
    const uint32_t *vals_in;  // NULL for keys only
    uint32_t *vals_out;
    int64_t n;
    int begin_bit, end_bit;
    int digit_bits = kRadixBits;  // 8, or 11 (2048-digit passes)
};

struct Layout {
    int passes = 0;
    int tile = 0;
    int64_t tiles = 0;
    int max_cols = 0;  // count-matrix columns (upsweep sub-blocks) at most
    Plan kplan, vplan;
    size_t off_counts = 0, off_rowtot = 0, off_spread = 0, off_diff = 0, off_ka = 0, off_kb = 0,
           off_va = 0, off_vb = 0;
    size_t total = 0;
};

Layout make_layout(const Request &rq)
{
    Layout L;
    const size_t ksz = (size_t)key_bytes(rq.kind);
    const size_t radix = (size_t)1 << rq.digit_bits;
    L.passes = (rq.end_bit - rq.begin_bit + rq.digit_bits - 1) / rq.digit_bits;
    L.tile = rq.digit_bits == kRadixBits ? tile_keys(rq.kind, rq.vals_in != nullptr, rq.n)
                                         : kWideDigitWaves * 64 * kWideDigitItems;
    L.tiles = (rq.n + L.tile - 1) / L.tile;
    L.max_cols = (int)std::min<int64_t>(L.tiles * kMaxSplit, kMaxBlocks);
    L.kplan = make_plan(L.passes, rq.keys_in == rq.keys_out);
    L.vplan = make_plan(L.passes, rq.vals_in != nullptr && rq.vals_in == rq.vals_out);
    size_t off = 0;
    L.off_counts = off;
    off += align_up(radix * L.max_cols * 4);
    L.off_rowtot = off;
    off += align_up(radix * 4);
    L.off_spread = off;  // AND and OR of the order codes, per column of the first pass
    off += align_up((size_t)2 * L.max_cols * 8);
    L.off_diff = off;  // their combination over all columns
    off += align_up(8);
    const size_t kbytes = align_up((size_t)rq.n * ksz), vbytes = align_up((size_t)rq.n * 4);
    if (L.kplan.need_a) { L.off_ka = off; off += kbytes; }
    if (L.kplan.need_b) { L.off_kb = off; off += kbytes; }
    if (rq.vals_in) {
        if (L.vplan.need_a) { L.off_va = off; off += vbytes; }
        if (L.vplan.need_b) { L.off_vb = off; off += vbytes; }
    }
    L.total = off;
    return L;
}

lrs_status copy_bytes(void *dst, const void *src, size_t bytes, hipStream_t stream)
{
    if (bytes == 0 || dst == src) return LRS_OK;
    const uintptr_t d = (uintptr_t)dst, s = (uintptr_t)src;
    hipError_t err;
    if ((d % 16) == 0 && (s % 16) == 0) {
        const int64_t n16 = (int64_t)(bytes / 16);
        if (n16 > 0) {
            int cus = 0;
            if (device_cus(&cus) != hipSuccess) return LRS_ERR_HIP;
            // four 256-thread workgroups per CU (16 waves), one vector per lane per step
            const int grid = (int)std::min<int64_t>((n16 + 255) / 256, (int64_t)4 * cus);
            err = launch(LRS_KERNEL_COPY, stream, [&] {
                copy16_kernel<<<grid, 256, 0, stream>>>((const uint4 *)src, (uint4 *)dst, n16);
            });
            if (err != hipSuccess) return LRS_ERR_HIP;
        }
        const size_t done = (size_t)n16 * 16;
        if (done < bytes) {
            err = launch(LRS_KERNEL_COPY, stream, [&] {
                copy1_kernel<<<1, 256, 0, stream>>>((const uint8_t *)src + done, (uint8_t *)dst + done,
                                                   (int64_t)(bytes - done));
            });
            if (err != hipSuccess) return LRS_ERR_HIP;
        }
        return LRS_OK;
    }
    const int grid = (int)std::min<int64_t>(((int64_t)bytes + 255) / 256, 8192);
    err = launch(LRS_KERNEL_COPY, stream, [&] {
        copy1_kernel<<<grid, 256, 0, stream>>>((const uint8_t *)src, (uint8_t *)dst, (int64_t)bytes);
    });
    return err == hipSuccess ? LRS_OK : LRS_ERR_HIP;
}

// ------------------------------------------------------------ pass launchers

// The codes' spread: where the first pass records it (spread_out, AND and OR
// per column, and diff_out, their combination) and where later passes read
// the combination (diff_in); each null where it does not apply.
struct SpreadArgs {
    unsigned long long *spread_out = nullptr;
    unsigned long long *diff_out = nullptr;
    const unsigned long long *diff_in = nullptr;
};

template <typename K, int CODE, int RB>
hipError_t launch_upsweep(const SortBufs &bufs, const Route &rt, int pass, uint32_t *counts, int64_t n,
                          int64_t block_len, int blocks, int shift, uint32_t mask, const SpreadArgs &sp,
                          hipStream_t stream)
{
    return launch(LRS_KERNEL_UPSWEEP, stream, [&] {
        const int grid = (blocks + kXcds - 1) / kXcds * kXcds;  // see upsweep_kernel's column mapping
        if (sp.spread_out != nullptr)
            upsweep_kernel<K, CODE, kUpsweepThreads, RB, true><<<grid, kUpsweepThreads, 0, stream>>>(
                bufs, rt, pass, counts, n, block_len, blocks, shift, mask, sp.spread_out, sp.diff_in);
        else
            upsweep_kernel<K, CODE, kUpsweepThreads, RB, false><<<grid, kUpsweepThreads, 0, stream>>>(
                bufs, rt, pass, counts, n, block_len, blocks, shift, mask, nullptr, sp.diff_in);
    });
}

// One workgroup per digit (row of the count matrix).
hipError_t launch_scan(uint32_t *counts, uint32_t *rowtot, int blocks, int radix, int shift, uint32_t mask,
                       const SpreadArgs &sp, hipStream_t stream)
{
    return launch(LRS_KERNEL_SCAN, stream, [&] {
        scan_kernel<kScanThreads, kScanPerThread><<<radix, kScanThreads, 0, stream>>>(
            counts, rowtot, blocks, sp.spread_out, sp.diff_out, sp.diff_in, shift, mask);
    });
}

// Outputs past 2 GiB take the downsweep with plain stores: the buffer stores'
// byte offsets are 32-bit.
template <typename K>
bool wide_output(int64_t n)
{
    return n * (int64_t)sizeof(K) > ((int64_t)1 << 31);
}

template <typename K, bool PAIRS, int WAVES, int ITEMS, int CODE, int RB = kRadixBits>
auto downsweep_fn(bool wide)
{
    if constexpr (RB != kRadixBits) {
        static_assert(WAVES == kWideDigitWaves && ITEMS == kWideDigitItems, "the 2048-digit downsweep's shape");
        return wide ? wide_digit_downsweep_kernel<K, PAIRS, RB, CODE, true>
                    : wide_digit_downsweep_kernel<K, PAIRS, RB, CODE, false>;
    } else if constexpr (ITEMS == kSmallItems) {
        return downsweep_kernel<K, PAIRS, WAVES, ITEMS, CODE, false>;  // small n: never wide
    } else {
        return wide ? downsweep_kernel<K, PAIRS, WAVES, ITEMS, CODE, true>
                    : downsweep_kernel<K, PAIRS, WAVES, ITEMS, CODE, false>;
    }
}

// copy_if_idle: this launch (the last pass's) also moves arrays that no pass
// moved to the output, when no finalize launch follows.
template <typename K, bool PAIRS, int WAVES, int ITEMS, int CODE, int RB>
hipError_t launch_downsweep(const SortBufs &bufs, const Route &rt, int pass, bool copy_if_idle,
                            const uint32_t *counts, const uint32_t *rowtot, int64_t n, int64_t block_len,
                            int blocks, int cols, int split, int shift, uint32_t mask,
                            const unsigned long long *diff_in, hipStream_t stream)
{
    return launch(LRS_KERNEL_DOWNSWEEP, stream, [&] {
        downsweep_fn<K, PAIRS, WAVES, ITEMS, CODE, RB>(wide_output<K>(n))<<<blocks, WAVES * 64, 0, stream>>>(
            bufs, rt, pass, copy_if_idle ? 1 : 0, counts, rowtot, n, block_len, cols, split, shift, mask, diff_in);
    });
}

// The kernel whose occupancy sets the number of blocks for this key type.
template <typename K, bool PAIRS, int WAVES, int ITEMS, int CODE, int RB>
hipError_t blocks_for(int64_t n, int64_t tiles, int *blocks)
{
    int cus = 0, per_cu = 0;
    hipError_t err = device_cus(&cus);
    if (err != hipSuccess) return err;
    err = occupancy((const void *)downsweep_fn<K, PAIRS, WAVES, ITEMS, CODE, RB>(wide_output<K>(n)), WAVES * 64,
                    &per_cu);
    if (err != hipSuccess) return err;
    // The downsweep reads a block's keys through a buffer whose size field is
    // 32-bit: keep every block below 2^30 bytes (at least 32 blocks at the
    // largest n of 64-bit keys, well inside the count-matrix width).
    constexpr int64_t kMaxBlockTiles = ((int64_t)1 << 30) / ((int64_t)WAVES * 64 * ITEMS * (int64_t)sizeof(K));
    const int64_t want = std::max<int64_t>(std::max<int64_t>(1, (int64_t)cus * per_cu),
                                           (tiles + kMaxBlockTiles - 1) / kMaxBlockTiles);
    *blocks = (int)std::min<int64_t>(std::min<int64_t>(tiles, want), kMaxBlocks);
    return hipSuccess;
}

// The buffers a sort's data can be in, by BufIndex.
template <bool PAIRS>
SortBufs sort_bufs(const Request &rq, const Layout &L, char *temp)
{
    SortBufs bufs;
    bufs.keys[BUF_IN] = rq.keys_in;
    bufs.keys[BUF_OUT] = rq.keys_out;
    bufs.keys[BUF_A] = L.kplan.need_a ? temp + L.off_ka : nullptr;
    bufs.keys[BUF_B] = L.kplan.need_b ? temp + L.off_kb : nullptr;
    bufs.vals[BUF_IN] = rq.vals_in;
    bufs.vals[BUF_OUT] = rq.vals_out;
    bufs.vals[BUF_A] = PAIRS && L.vplan.need_a ? (const uint32_t *)(temp + L.off_va) : nullptr;
    bufs.vals[BUF_B] = PAIRS && L.vplan.need_b ? (const uint32_t *)(temp + L.off_vb) : nullptr;
    return bufs;
}

// RB: digit width (8, or 11 with the 2048-digit downsweep).
template <typename K, bool PAIRS, int WAVES, int ITEMS, int CODE, int RB = kRadixBits>
lrs_status run_passes(const Request &rq, const Layout &L, char *temp, hipStream_t stream)
{
    constexpr int TILE = WAVES * 64 * ITEMS;
    int want_blocks = 0;
    if (blocks_for<K, PAIRS, WAVES, ITEMS, CODE, RB>(rq.n, L.tiles, &want_blocks) != hipSuccess) return LRS_ERR_HIP;
    const int64_t tiles_per_block = (L.tiles + want_blocks - 1) / want_blocks;
    const int64_t block_len = tiles_per_block * TILE;
    const int blocks = (int)((rq.n + block_len - 1) / block_len);
    // The upsweep counts each block as `split` sub-blocks, so that it runs as
    // many workgroups as fill the chip however few blocks the downsweep's
    // occupancy allows; the count matrix has one column per sub-block.  The
    // split doubles while the sub-blocks still fit one round of resident
    // upsweep workgroups: more columns than that make the scan longer without
    // a faster upsweep (1e8 keys: 1020 columns sort 6 us faster than 2040).
    int cus = 0, up_per_cu = 0;
    if (device_cus(&cus) != hipSuccess) return LRS_ERR_HIP;
    if (occupancy((const void *)upsweep_kernel<K, CODE, kUpsweepThreads, RB>, kUpsweepThreads, &up_per_cu) !=
        hipSuccess)
        return LRS_ERR_HIP;
    int split = 1;
    while (split < kMaxSplit && (int64_t)blocks * split * 2 <= kMaxBlocks &&
           (int64_t)blocks * split * 2 <= (int64_t)cus * up_per_cu)
        split *= 2;
    const int64_t sub_len = block_len / split;  // TILE is a multiple of kMaxSplit
    const int cols = (int)((rq.n + sub_len - 1) / sub_len);

    uint32_t *counts = (uint32_t *)(temp + L.off_counts);
    uint32_t *rowtot = (uint32_t *)(temp + L.off_rowtot);
    unsigned long long *spread = (unsigned long long *)(temp + L.off_spread);
    unsigned long long *diff = (unsigned long long *)(temp + L.off_diff);
    const SortBufs bufs = sort_bufs<PAIRS>(rq, L, temp);
    // An in-place array starts in the output buffer (the same memory).
    Route rt;
    rt.passes = L.passes;
    rt.begin_bit = rq.begin_bit;
    rt.end_bit = rq.end_bit;
    rt.digit_bits = RB;
    rt.kstart = rq.keys_in == rq.keys_out ? BUF_OUT : BUF_IN;
    rt.vstart = PAIRS && rq.vals_in == rq.vals_out ? BUF_OUT : BUF_IN;
    rt.kb = L.kplan.need_b ? 1 : 0;
    rt.vb = PAIRS && L.vplan.need_b ? 1 : 0;
    // Only an in-place array can end outside the output (and then a copy
    // launch follows the passes); otherwise the last pass's downsweep moves the
    // data itself when every pass was skipped.
    const bool finalize = rt.kstart == BUF_OUT || rt.vstart == BUF_OUT;
    // With more than one pass, the first records the codes' spread, and every
    // later kernel derives the skipped passes and the route from it.
    const bool spread_on = L.passes > 1;

    for (int p = 0; p < L.passes; ++p) {
        const int shift = rq.begin_bit + RB * p;
        const int width = std::min(RB, rq.end_bit - shift);
        const uint32_t mask = (1u << width) - 1u;
        SpreadArgs sp;
        if (spread_on) {
            if (p == 0) {
                sp.spread_out = spread;
                sp.diff_out = diff;
            } else {
                sp.diff_in = diff;
            }
        }
        hipError_t err = launch_upsweep<K, CODE, RB>(bufs, rt, p, counts, rq.n, sub_len, cols, shift, mask, sp, stream);
        if (err != hipSuccess) return LRS_ERR_HIP;
        if (launch_scan(counts, rowtot, cols, 1 << RB, shift, mask, sp, stream) != hipSuccess) return LRS_ERR_HIP;
        err = launch_downsweep<K, PAIRS, WAVES, ITEMS, CODE, RB>(bufs, rt, p, p == L.passes - 1 && !finalize, counts,
                                                                 rowtot, rq.n, block_len, blocks, cols, split, shift,
                                                                 mask, spread_on ? diff : nullptr, stream);
        if (err != hipSuccess) return LRS_ERR_HIP;
    }
    if (!finalize) return LRS_OK;
    const int fin_grid = (int)std::min<int64_t>(((int64_t)sizeof(K) * rq.n + 4095) / 4096, 4096);
    const hipError_t err = launch(LRS_KERNEL_FINALIZE, stream, [&] {
        finalize_kernel<K, PAIRS><<<fin_grid, 256, 0, stream>>>(bufs, rt, rowtot, rq.n, spread_on ? diff : nullptr);
    });
    return err == hipSuccess ? LRS_OK : LRS_ERR_HIP;
}

// Sorts above the one-workgroup limit and up to kSmallPassMaxBytes of keys (8-bit
// digits): one small_pass_kernel launch per pass, every pass running (a pass
// over a constant digit reorders nothing, so the result is the same), the
// buffers alternating as run_dest plans them with no pass skipped.  An
// in-place array that ends in A is copied back by the device copy.
template <typename K, bool PAIRS, int CODE, int ITEMS>
lrs_status run_small_passes(const Request &rq, const Layout &L, char *temp, hipStream_t stream)
{
    const SortBufs bufs = sort_bufs<PAIRS>(rq, L, temp);
    const int kstart = rq.keys_in == rq.keys_out ? BUF_OUT : BUF_IN;
    const int vstart = PAIRS && rq.vals_in == rq.vals_out ? BUF_OUT : BUF_IN;
    const bool kb = L.kplan.need_b, vb = PAIRS && L.vplan.need_b;
    const int grid = (int)((rq.n + 1024 * ITEMS - 1) / (1024 * ITEMS));
    for (int p = 0; p < L.passes; ++p) {
        const int shift = rq.begin_bit + kRadixBits * p;
        const int width = std::min(kRadixBits, rq.end_bit - shift);
        const uint32_t mask = (1u << width) - 1u;
        int ks, kd, vs = 0, vd = 0;
        pass_route(kstart, kb, L.passes, 0u, p, ks, kd);
        if (PAIRS) pass_route(vstart, vb, L.passes, 0u, p, vs, vd);
        const hipError_t err = launch(LRS_KERNEL_SMALL, stream, [&] {
            small_pass_kernel<K, PAIRS, CODE, ITEMS><<<grid, 1024, 0, stream>>>(
                (const K *)bufs.keys[ks], PAIRS ? bufs.vals[vs] : nullptr, (K *)bufs.keys[kd],
                PAIRS ? (uint32_t *)bufs.vals[vd] : nullptr, (int)rq.n, shift, mask);
        });
        if (err != hipSuccess) return LRS_ERR_HIP;
    }
    const int kf = final_buffer(kstart, kb, L.passes, 0u);
    if (kf != BUF_OUT) {
        const lrs_status st = copy_bytes(rq.keys_out, bufs.keys[kf], (size_t)rq.n * sizeof(K), stream);
        if (st != LRS_OK) return st;
    }
    if (PAIRS) {
        const int vf = final_buffer(vstart, vb, L.passes, 0u);
        if (vf != BUF_OUT) return copy_bytes(rq.vals_out, bufs.vals[vf], (size_t)rq.n * 4, stream);
    }
    return LRS_OK;
}

template <typename K, bool PAIRS, int CODE>
lrs_status run_tiny(const Request &rq, hipStream_t stream)
{
    constexpr int NMAX = tiny_max<K, PAIRS>();
    const hipError_t err = launch(LRS_KERNEL_TINY, stream, [&] {
        tiny_sort_kernel<K, PAIRS, CODE, NMAX><<<1, 1024, 0, stream>>>(
            (const K *)rq.keys_in, rq.vals_in, (K *)rq.keys_out, rq.vals_out, (int)rq.n, rq.begin_bit, rq.end_bit);
    });
    return err == hipSuccess ? LRS_OK : LRS_ERR_HIP;
}

template <typename K, int CODE>
lrs_status run_kind(bool pairs, const Request &r, const Layout &L, char *temp, hipStream_t stream)
{
    if (pairs && r.n <= std::min<int64_t>(tiny_max<K, true>(), kTinyMaxKeys)) return run_tiny<K, true, CODE>(r, stream);
    if (!pairs && r.n <= std::min<int64_t>(tiny_max<K, false>(), kTinyMaxKeys)) return run_tiny<K, false, CODE>(r, stream);
    if (r.digit_bits == kWideDigitBits) {
        if (pairs) return run_passes<K, true, kWideDigitWaves, kWideDigitItems, CODE, kWideDigitBits>(r, L, temp, stream);
        return run_passes<K, false, kWideDigitWaves, kWideDigitItems, CODE, kWideDigitBits>(r, L, temp, stream);
    }
    if (r.n * (int64_t)sizeof(K) <= kSmallPassMaxBytes) {
        if (pairs) return run_small_passes<K, true, CODE, 1>(r, L, temp, stream);
        return run_small_passes<K, false, CODE, 1>(r, L, temp, stream);
    }
    if (r.n <= kSmallTileMaxKeys) {
        if (pairs) return run_passes<K, true, 8, kSmallItems, CODE>(r, L, temp, stream);
        return run_passes<K, false, 8, kSmallItems, CODE>(r, L, temp, stream);
    }
    if (pairs) return run_passes<K, true, 8, kItems, CODE>(r, L, temp, stream);
    if constexpr (sizeof(K) == 4) {
        if (wide_tiles(4, false, r.n)) return run_passes<K, false, 16, kItems, CODE>(r, L, temp, stream);
    }
    return run_passes<K, false, 8, kItems, CODE>(r, L, temp, stream);
}

lrs_status sort_entry(const Request &rq, void *d_temp, size_t *temp_bytes, hipStream_t stream)
{
    // All checks happen before any HIP call, so they need no device.
    if (temp_bytes == nullptr) return LRS_ERR_INVALID_ARG;
    if (rq.digit_bits != kRadixBits && rq.digit_bits != kWideDigitBits) return LRS_ERR_INVALID_ARG;
    const int key_bits = 8 * key_bytes(rq.kind);
    const size_t ksz = key_bits / 8;
    if (rq.n < 0 || rq.n > (int64_t)0xFFFFFFFFll) return LRS_ERR_INVALID_ARG;
    if (rq.begin_bit < 0 || rq.end_bit < rq.begin_bit || rq.end_bit > key_bits) return LRS_ERR_INVALID_ARG;
    if (rq.n > 0) {
        if (!rq.keys_in || !rq.keys_out) return LRS_ERR_INVALID_ARG;
        if (((uintptr_t)rq.keys_in % ksz) || ((uintptr_t)rq.keys_out % ksz)) return LRS_ERR_INVALID_ARG;
        if (overlap_partial(rq.keys_in, rq.keys_out, (size_t)rq.n * ksz)) return LRS_ERR_INVALID_ARG;
    }
    const bool pairs = rq.vals_in != nullptr || rq.vals_out != nullptr;
    if (pairs && rq.n > 0) {
        if (!rq.vals_in || !rq.vals_out) return LRS_ERR_INVALID_ARG;
        if (((uintptr_t)rq.vals_in % 4) || ((uintptr_t)rq.vals_out % 4)) return LRS_ERR_INVALID_ARG;
        if (overlap_partial(rq.vals_in, rq.vals_out, (size_t)rq.n * 4)) return LRS_ERR_INVALID_ARG;
    }
    Request r = rq;
    if (!pairs || rq.n == 0) r.vals_in = nullptr, r.vals_out = nullptr;
    const Layout L = make_layout(r);
    // d_temp may have any alignment: the layout starts at its first kAlign
    // boundary, and the size reported covers the worst case of that padding.
    if (d_temp == nullptr) {
        *temp_bytes = L.total + (kAlign - 1);
        return LRS_OK;
    }
    const size_t pad = (kAlign - (uintptr_t)d_temp % kAlign) % kAlign;
    if (*temp_bytes < L.total + pad) return LRS_ERR_TEMP_TOO_SMALL;
    if (r.n == 0) return LRS_OK;
    if (L.passes == 0) {
        lrs_status st = copy_bytes(r.keys_out, r.keys_in, (size_t)r.n * ksz, stream);
        if (st == LRS_OK && pairs) st = copy_bytes(r.vals_out, r.vals_in, (size_t)r.n * 4, stream);
        return st;
    }
    char *temp = (char *)d_temp + pad;
    switch (r.kind) {
    case KIND_U32: return run_kind<uint32_t, CODE_UNSIGNED>(pairs, r, L, temp, stream);
    case KIND_I32: return run_kind<uint32_t, CODE_SIGNED>(pairs, r, L, temp, stream);
    case KIND_F32: return run_kind<uint32_t, CODE_FLOAT>(pairs, r, L, temp, stream);
    case KIND_U64: return run_kind<uint64_t, CODE_UNSIGNED>(pairs, r, L, temp, stream);
    case KIND_I64: return run_kind<uint64_t, CODE_SIGNED>(pairs, r, L, temp, stream);
    case KIND_F64: return run_kind<uint64_t, CODE_FLOAT>(pairs, r, L, temp, stream);
    }
    return LRS_ERR_INVALID_ARG;
}

}  // namespace

// ------------------------------------------------------------------- exports

LRS_API lrs_status lrs_sort_keys_u32(void *d_temp, size_t *temp_bytes, const uint32_t *d_keys_in,
                                     uint32_t *d_keys_out, int64_t n, int begin_bit, int end_bit,
                                     hipStream_t stream)
{
    return sort_entry({KIND_U32, d_keys_in, d_keys_out, nullptr, nullptr, n, begin_bit, end_bit}, d_temp,
                      temp_bytes, stream);
}

LRS_API lrs_status lrs_sort_keys_u64(void *d_temp, size_t *temp_bytes, const uint64_t *d_keys_in,
                                     uint64_t *d_keys_out, int64_t n, int begin_bit, int end_bit,
                                     hipStream_t stream)
{
    return sort_entry({KIND_U64, d_keys_in, d_keys_out, nullptr, nullptr, n, begin_bit, end_bit}, d_temp,
                      temp_bytes, stream);
}

LRS_API lrs_status lrs_sort_keys_f32(void *d_temp, size_t *temp_bytes, const float *d_keys_in, float *d_keys_out,
                                     int64_t n, int begin_bit, int end_bit, hipStream_t stream)
{
    return sort_entry({KIND_F32, d_keys_in, d_keys_out, nullptr, nullptr, n, begin_bit, end_bit}, d_temp,
                      temp_bytes, stream);
}

LRS_API lrs_status lrs_sort_pairs_u32(void *d_temp, size_t *temp_bytes, const uint32_t *d_keys_in,
                                      const uint32_t *d_values_in, uint32_t *d_keys_out, uint32_t *d_values_out,
                                      int64_t n, int begin_bit, int end_bit, hipStream_t stream)
{
    if (n > 0 && (!d_values_in || !d_values_out)) return LRS_ERR_INVALID_ARG;
    return sort_entry({KIND_U32, d_keys_in, d_keys_out, d_values_in, d_values_out, n, begin_bit, end_bit}, d_temp,
                      temp_bytes, stream);
}

LRS_API lrs_status lrs_sort_pairs_u64(void *d_temp, size_t *temp_bytes, const uint64_t *d_keys_in,
                                      const uint32_t *d_values_in, uint64_t *d_keys_out, uint32_t *d_values_out,
                                      int64_t n, int begin_bit, int end_bit, hipStream_t stream)
{
    if (n > 0 && (!d_values_in || !d_values_out)) return LRS_ERR_INVALID_ARG;
    return sort_entry({KIND_U64, d_keys_in, d_keys_out, d_values_in, d_values_out, n, begin_bit, end_bit}, d_temp,
                      temp_bytes, stream);
}

LRS_API lrs_status lrs_sort_pairs_f32(void *d_temp, size_t *temp_bytes, const float *d_keys_in,
                                      const uint32_t *d_values_in, float *d_keys_out, uint32_t *d_values_out,
                                      int64_t n, int begin_bit, int end_bit, hipStream_t stream)
{
    if (n > 0 && (!d_values_in || !d_values_out)) return LRS_ERR_INVALID_ARG;
    return sort_entry({KIND_F32, d_keys_in, d_keys_out, d_values_in, d_values_out, n, begin_bit, end_bit}, d_temp,
                      temp_bytes, stream);
}

LRS_API lrs_status lrs_sort_keys_i32(void *d_temp, size_t *temp_bytes, const int32_t *d_keys_in, int32_t *d_keys_out,
                                     int64_t n, int begin_bit, int end_bit, hipStream_t stream)
{
    return sort_entry({KIND_I32, d_keys_in, d_keys_out, nullptr, nullptr, n, begin_bit, end_bit}, d_temp,
                      temp_bytes, stream);
}

LRS_API lrs_status lrs_sort_keys_i64(void *d_temp, size_t *temp_bytes, const int64_t *d_keys_in, int64_t *d_keys_out,
                                     int64_t n, int begin_bit, int end_bit, hipStream_t stream)
{
    return sort_entry({KIND_I64, d_keys_in, d_keys_out, nullptr, nullptr, n, begin_bit, end_bit}, d_temp,
                      temp_bytes, stream);
}

LRS_API lrs_status lrs_sort_keys_f64(void *d_temp, size_t *temp_bytes, const double *d_keys_in, double *d_keys_out,
                                     int64_t n, int begin_bit, int end_bit, hipStream_t stream)
{
    return sort_entry({KIND_F64, d_keys_in, d_keys_out, nullptr, nullptr, n, begin_bit, end_bit}, d_temp,
                      temp_bytes, stream);
}

LRS_API lrs_status lrs_sort_pairs_i32(void *d_temp, size_t *temp_bytes, const int32_t *d_keys_in,
                                      const uint32_t *d_values_in, int32_t *d_keys_out, uint32_t *d_values_out,
                                      int64_t n, int begin_bit, int end_bit, hipStream_t stream)
{
    if (n > 0 && (!d_values_in || !d_values_out)) return LRS_ERR_INVALID_ARG;
    return sort_entry({KIND_I32, d_keys_in, d_keys_out, d_values_in, d_values_out, n, begin_bit, end_bit}, d_temp,
                      temp_bytes, stream);
}

LRS_API lrs_status lrs_sort_pairs_i64(void *d_temp, size_t *temp_bytes, const int64_t *d_keys_in,
                                      const uint32_t *d_values_in, int64_t *d_keys_out, uint32_t *d_values_out,
                                      int64_t n, int begin_bit, int end_bit, hipStream_t stream)
{
    if (n > 0 && (!d_values_in || !d_values_out)) return LRS_ERR_INVALID_ARG;
    return sort_entry({KIND_I64, d_keys_in, d_keys_out, d_values_in, d_values_out, n, begin_bit, end_bit}, d_temp,
                      temp_bytes, stream);
}

LRS_API lrs_status lrs_sort_pairs_f64(void *d_temp, size_t *temp_bytes, const double *d_keys_in,
                                      const uint32_t *d_values_in, double *d_keys_out, uint32_t *d_values_out,
                                      int64_t n, int begin_bit, int end_bit, hipStream_t stream)
{
    if (n > 0 && (!d_values_in || !d_values_out)) return LRS_ERR_INVALID_ARG;
    return sort_entry({KIND_F64, d_keys_in, d_keys_out, d_values_in, d_values_out, n, begin_bit, end_bit}, d_temp,
                      temp_bytes, stream);
}

LRS_API lrs_status lrs_sort_digits(lrs_key_type key_type, int digit_bits, void *d_temp, size_t *temp_bytes,
                                   const void *d_keys_in, const uint32_t *d_values_in, void *d_keys_out,
                                   uint32_t *d_values_out, int64_t n, int begin_bit, int end_bit, hipStream_t stream)
{
    KeyKind kind;
    switch (key_type) {
    case LRS_KEY_U32: kind = KIND_U32; break;
    case LRS_KEY_I32: kind = KIND_I32; break;
    case LRS_KEY_F32: kind = KIND_F32; break;
    case LRS_KEY_U64: kind = KIND_U64; break;
    case LRS_KEY_I64: kind = KIND_I64; break;
    case LRS_KEY_F64: kind = KIND_F64; break;
    default: return LRS_ERR_INVALID_ARG;
    }
    if (n > 0 && (d_values_in == nullptr) != (d_values_out == nullptr)) return LRS_ERR_INVALID_ARG;
    Request rq{kind, d_keys_in, d_keys_out, d_values_in, d_values_out, n, begin_bit, end_bit};
    rq.digit_bits = digit_bits;
    return sort_entry(rq, d_temp, temp_bytes, stream);
}

// ------------------------------------------------------- allocation-free sort

// The scratch of lrs_sort_digits_noalloc: one array per GPU the library runs
// on.  In host code `scratch` is only a handle for hipGetSymbolAddress, never
// a device address: kernels get the per-device address looked up below.
static __device__ __align__(256) unsigned char scratch[LRS_NOALLOC_SCRATCH_BYTES];

namespace {
std::mutex g_scratch_mu;
void *g_scratch_ptr[64];  // per device, looked up once

hipError_t scratch_address(void **ptr)
{
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void *p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess) return err;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}
}  // namespace

LRS_API lrs_status lrs_sort_digits_noalloc(lrs_key_type key_type, int digit_bits, const void *d_keys_in,
                                           const uint32_t *d_values_in, void *d_keys_out, uint32_t *d_values_out,
                                           int64_t n, int begin_bit, int end_bit, hipStream_t stream)
{
    // The size query makes every argument check first (no device call).
    size_t need = 0;
    lrs_status st = lrs_sort_digits(key_type, digit_bits, nullptr, &need, d_keys_in, d_values_in, d_keys_out,
                                    d_values_out, n, begin_bit, end_bit, stream);
    if (st != LRS_OK) return st;
    // The scratch is 256-byte aligned, so the layout needs none of the 255
    // bytes of padding the query includes.
    if (need - (kAlign - 1) > LRS_NOALLOC_SCRATCH_BYTES) return LRS_ERR_TOO_LARGE;
    if (n == 0) return LRS_OK;  // nothing to do, on the device either
    void *ptr = nullptr;
    if (scratch_address(&ptr) != hipSuccess) return LRS_ERR_HIP;
    size_t bytes = LRS_NOALLOC_SCRATCH_BYTES;
    return lrs_sort_digits(key_type, digit_bits, ptr, &bytes, d_keys_in, d_values_in, d_keys_out, d_values_out, n,
                           begin_bit, end_bit, stream);
}

LRS_API const char *lrs_status_string(lrs_status status)
{
    switch (status) {
    case LRS_OK: return "LRS_OK: success";
    case LRS_ERR_INVALID_ARG: return "LRS_ERR_INVALID_ARG: invalid argument";
    case LRS_ERR_TEMP_TOO_SMALL: return "LRS_ERR_TEMP_TOO_SMALL: temp storage smaller than required";
    case LRS_ERR_HIP: return "LRS_ERR_HIP: a HIP call or kernel launch failed";
    case LRS_ERR_TOO_LARGE:
        return "LRS_ERR_TOO_LARGE: the sort needs more than the library's static scratch "
               "(LRS_NOALLOC_SCRATCH_BYTES) holds";
    }
    return "unknown lrs_status";
}

LRS_API lrs_status lrs_device_copy(void *d_dst, const void *d_src, size_t bytes, hipStream_t stream)
{
    if (bytes > 0 && (!d_dst || !d_src)) return LRS_ERR_INVALID_ARG;
    return copy_bytes(d_dst, d_src, bytes, stream);
}

namespace {
void prof_release_locked()
{
    g_prof.on.store(false, std::memory_order_release);
    for (auto &e : g_prof.ev)
        if (e) (void)hipEventDestroy(e);
    g_prof.ev.clear();
    g_prof.kind.clear();
    g_prof.cap = 0;
    g_prof.count = 0;
}
}  // namespace

LRS_API lrs_status lrs_bench_read(const void *d_src, size_t bytes, uint32_t *d_result, hipStream_t stream)
{
    if (bytes % 16 != 0 || (uintptr_t)d_src % 16 != 0 || (uintptr_t)d_result % 4 != 0) return LRS_ERR_INVALID_ARG;
    if (bytes > 0 && (!d_src || !d_result)) return LRS_ERR_INVALID_ARG;
    if (bytes == 0) return LRS_OK;
    int cus = 0;
    if (device_cus(&cus) != hipSuccess) return LRS_ERR_HIP;
    const int64_t n16 = (int64_t)(bytes / 16);
    // eight 256-thread workgroups per CU: the fastest read measured
    const int grid = (int)std::min<int64_t>((n16 + 255) / 256, (int64_t)8 * cus);
    const hipError_t err = launch(LRS_KERNEL_COPY, stream, [&] {
        read16_kernel<<<grid, 256, 0, stream>>>((const uint4 *)d_src, n16, d_result);
    });
    return err == hipSuccess ? LRS_OK : LRS_ERR_HIP;
}

LRS_API lrs_status lrs_prof_start(int capacity)
{
    if (capacity <= 0) return LRS_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> lock(g_prof.mu);
    prof_release_locked();
    g_prof.ev.assign(2 * (size_t)capacity, nullptr);
    g_prof.kind.assign(capacity, 0);
    for (auto &e : g_prof.ev) {
        if (hipEventCreate(&e) != hipSuccess) {
            e = nullptr;
            prof_release_locked();
            return LRS_ERR_HIP;
        }
    }
    g_prof.cap = capacity;
    g_prof.count = 0;
    g_prof.on.store(true, std::memory_order_release);
    return LRS_OK;
}

LRS_API lrs_status lrs_prof_stop(void)
{
    std::lock_guard<std::mutex> lock(g_prof.mu);
    g_prof.on.store(false, std::memory_order_release);
    return LRS_OK;
}

LRS_API int lrs_prof_count(void)
{
    std::lock_guard<std::mutex> lock(g_prof.mu);
    return g_prof.count;
}

LRS_API lrs_status lrs_prof_read(int i, int *kind, float *ms)
{
    hipEvent_t a, b;
    int k;
    {
        std::lock_guard<std::mutex> lock(g_prof.mu);
        if (i < 0 || i >= g_prof.count || !kind || !ms) return LRS_ERR_INVALID_ARG;
        a = g_prof.ev[2 * i];
        b = g_prof.ev[2 * i + 1];
        k = g_prof.kind[i];
    }
    // (waits outside the lock; the events stay valid until lrs_prof_release,
    // which the caller must not run concurrently with a read)
    if (hipEventSynchronize(b) != hipSuccess) return LRS_ERR_HIP;
    float t = 0.f;
    if (hipEventElapsedTime(&t, a, b) != hipSuccess) return LRS_ERR_HIP;
    *kind = k;
    *ms = t;
    return LRS_OK;
}

LRS_API lrs_status lrs_prof_release(void)
{
    std::lock_guard<std::mutex> lock(g_prof.mu);
    prof_release_locked();
    return LRS_OK;
}
