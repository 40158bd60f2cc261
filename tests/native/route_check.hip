// Exhaustive host-side check of the pass routing the sort's kernels derive
// (kernels.hpp: pass_route, final_buffer, skipped_passes): for every pass
// count, every set of skipped passes and in-place or not, each pass reads the
// buffer the previous one left the data in, a pass that runs writes another
// buffer that exists in temp storage (never the caller's input), a skipped pass
// moves nothing, and the data ends in the output (an in-place array may end in
// A, from which the sort's last launch copies it back).  Exit status 0 on
// success.
#include <stdio.h>

#include "../../sorting_lsd_radix_sort_amd/csrc/kernels.hpp"

using namespace lrs;

static int fails = 0;
#define CHECK(c, ...)                                  \
    do {                                               \
        if (!(c)) {                                    \
            if (fails++ < 20) printf(__VA_ARGS__);     \
        }                                              \
    } while (0)

int main()
{
    long cases = 0;
    for (int passes = 1; passes <= 12; ++passes) {
        for (int in_place = 0; in_place <= 1; ++in_place) {
            // the alternate buffers the host reserves (make_plan in lrsort.hip)
            const bool has_a = in_place || passes >= 2;
            const bool has_b = in_place && passes % 2 == 1 && passes >= 3;
            const int start = in_place ? BUF_OUT : BUF_IN;
            for (uint32_t skip = 0; skip < (1u << passes); ++skip) {
                ++cases;
                int at = start;
                int runs = 0;
                for (int p = 0; p < passes; ++p) {
                    int src, dst;
                    pass_route(start, has_b, passes, skip, p, src, dst);
                    CHECK(src == at, "P=%d ip=%d skip=%x p=%d: reads %d, data in %d\n", passes, in_place, skip, p, src, at);
                    if ((skip >> p) & 1u) {
                        CHECK(dst == src, "P=%d ip=%d skip=%x p=%d: skipped pass moves data\n", passes, in_place, skip, p);
                    } else {
                        ++runs;
                        CHECK(dst != src, "P=%d ip=%d skip=%x p=%d: writes its source\n", passes, in_place, skip, p);
                        CHECK(dst != BUF_IN, "P=%d ip=%d skip=%x p=%d: writes the input\n", passes, in_place, skip, p);
                        CHECK(dst != BUF_A || has_a, "P=%d ip=%d skip=%x p=%d: A not reserved\n", passes, in_place, skip, p);
                        CHECK(dst != BUF_B || has_b, "P=%d ip=%d skip=%x p=%d: B not reserved\n", passes, in_place, skip, p);
                    }
                    at = dst;
                }
                const int fin = final_buffer(start, has_b, passes, skip);
                CHECK(fin == at, "P=%d ip=%d skip=%x: final %d, data in %d\n", passes, in_place, skip, fin, at);
                if (in_place)
                    CHECK(at == BUF_OUT || at == BUF_A, "P=%d ip=1 skip=%x: ends in %d\n", passes, skip, at);
                else
                    CHECK(at == BUF_OUT || (runs == 0 && at == BUF_IN), "P=%d ip=0 skip=%x: ends in %d\n", passes, skip, at);
                // an in-place array needs the copy back only when an odd number
                // of passes run and B cannot take the middle one
                if (in_place && at == BUF_A)
                    CHECK(runs % 2 == 1 && (runs == 1 || !has_b), "P=%d ip=1 skip=%x: avoidable copy\n", passes, skip);
            }
        }
    }
    // skipped_passes against the digit fields of a spread value
    for (int bits = 8; bits <= 11; bits += 3) {
        for (int begin = 0; begin < 64; begin += 5) {
            for (int end = begin; end <= 64; end += 7) {
                Route rt{};
                rt.begin_bit = begin;
                rt.end_bit = end;
                rt.digit_bits = bits;
                rt.passes = (end - begin + bits - 1) / bits;
                for (int b = 0; b < 64; ++b) {
                    const unsigned long long diff = 1ull << b;
                    const uint32_t skip = skipped_passes(rt, diff);
                    for (int p = 0; p < rt.passes; ++p) {
                        const int lo = begin + bits * p, hi = lo + bits < end ? lo + bits : end;
                        const bool differs = b >= lo && b < hi;
                        CHECK(((skip >> p) & 1u) == (differs ? 0u : 1u),
                              "bits=%d [%d,%d) diff bit %d pass %d: skip %u\n", bits, begin, end, b, p, (skip >> p) & 1u);
                        ++cases;
                    }
                }
            }
        }
    }
    printf("%ld cases, %d failures\n", cases, fails);
    return fails == 0 ? 0 : 1;
}
