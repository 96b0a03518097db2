/* oracle/philox_ref.c built with AddressSanitizer and UndefinedBehaviorSanitizer:
 * the batch entry point over a buffer of counters, checked against the
 * published Philox4x32-10 known-answer vectors (Salmon et al., SC'11, and its
 * Random123 distribution).  Built and run by tests/test_host_sanitizers.py. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void philox4x32_10_batch(const uint32_t* ctr, size_t n, uint32_t k0, uint32_t k1, uint32_t* out);

static const uint32_t KAT[3][10] = {
    {0x00000000, 0x00000000, 0x00000000, 0x00000000, 0x00000000, 0x00000000,
     0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8},
    {0xffffffff, 0xffffffff, 0xffffffff, 0xffffffff, 0xffffffff, 0xffffffff,
     0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd},
    {0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344, 0xa4093822, 0x299f31d0,
     0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1},
};

int main(void) {
    for (int v = 0; v < 3; ++v) {
        /* a heap buffer of exactly n counters, so an overrun is reported */
        const size_t n = 37;
        uint32_t* ctr = malloc(n * 4 * sizeof(uint32_t));
        uint32_t* out = malloc(n * 4 * sizeof(uint32_t));
        if (!ctr || !out) return 2;
        for (size_t i = 0; i < n; ++i)
            for (int w = 0; w < 4; ++w) ctr[4 * i + w] = KAT[v][w];
        philox4x32_10_batch(ctr, n, KAT[v][4], KAT[v][5], out);
        for (size_t i = 0; i < n; ++i)
            for (int w = 0; w < 4; ++w)
                if (out[4 * i + w] != KAT[v][6 + w]) {
                    fprintf(stderr, "vector %d word %d: %08x\n", v, w, out[4 * i + w]);
                    return 1;
                }
        free(ctr);
        free(out);
    }
    printf("philox sanitize ok\n");
    return 0;
}
