/*
 * Exhaustive check of the oracle's float32 transform (test code, CPU only).
 * For every 32-bit word u, in increasing order:
 *   - oracle_f2s(oracle_s2f(u)) == u and oracle_s2f(oracle_f2s(u)) == u
 *     (the two maps are inverse bijections);
 *   - the decoded float of u is NaN exactly when u lies below the word of -inf
 *     or above the word of +inf;
 *   - between those words the decoded floats strictly increase under the
 *     hardware's IEEE-754 '<', except one step from -0.0 to +0.0 (equal
 *     under '<', ordered by sign).
 * The ordering it checks against is the FPU's comparison, not the encoding.
 * Optional arguments LO HI (hex) restrict the walk to words [LO, HI); the
 * ordering step from LO-1 to LO is still checked, so contiguous ranges run in
 * parallel cover every step exactly once.
 * Prints "ok" and the number of -0.0 -> +0.0 steps seen, and exits 0, or
 * prints the first failing word and exits 1.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

uint32_t oracle_f2s(uint32_t bits);
uint32_t oracle_s2f(uint32_t u);

static float as_float(uint32_t w) { float f; memcpy(&f, &w, 4); return f; }

int main(int argc, char **argv)
{
    uint64_t lo = 0, hi = 1ull << 32;
    if (argc == 3) {
        lo = strtoull(argv[1], NULL, 16);
        hi = strtoull(argv[2], NULL, 16);
    }
    const uint32_t neg_inf_word = oracle_f2s(0xFF800000u);
    const uint32_t pos_inf_word = oracle_f2s(0x7F800000u);
    int have_prev = 0, zero_steps = 0;
    float prev = 0.0f;
    for (uint64_t w = lo ? lo - 1 : 0; w < hi; ++w) {
        uint32_t u = (uint32_t)w;
        int counted = w >= lo; /* the word before LO only seeds 'prev' */
        uint32_t x = oracle_s2f(u);
        if (oracle_f2s(x) != u) { printf("f2s(s2f(%08x)) != itself\n", u); return 1; }
        if (oracle_s2f(oracle_f2s(u)) != u) { printf("s2f(f2s(%08x)) != itself\n", u); return 1; }
        float f = as_float(x);
        int outside = u < neg_inf_word || u > pos_inf_word;
        if (outside) {
            if (!isnan(f)) { printf("word %08x outside [-inf,+inf] decodes to non-NaN\n", u); return 1; }
        } else {
            if (isnan(f)) { printf("word %08x inside [-inf,+inf] decodes to NaN\n", u); return 1; }
            if (have_prev) {
                if (prev < f) {
                    /* strictly increasing: fine */
                } else if (prev == 0.0f && f == 0.0f && signbit(prev) && !signbit(f)) {
                    zero_steps += counted;
                } else {
                    printf("order broken at word %08x: %a then %a\n", u, (double)prev, (double)f);
                    return 1;
                }
            }
            prev = f;
            have_prev = 1;
        }
    }
    printf("ok zero_steps=%d neg_inf_word=%08x pos_inf_word=%08x\n", zero_steps,
           neg_inf_word, pos_inf_word);
    return 0;
}
