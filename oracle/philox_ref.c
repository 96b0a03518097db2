/* Philox4x32-10 in plain C (oracle side, test infrastructure only).
 *
 * An independent second implementation of the generator defined in Salmon,
 * Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11),
 * used by the tests to cross-check the vectorised numpy version bit for bit.
 * One round: the two 32x32->64-bit products of words 0 and 2 with the round
 * multipliers; the new words are (hi(word2 product) ^ c1 ^ k0, lo(word2
 * product), hi(word0 product) ^ c3 ^ k1, lo(word0 product)); then the key
 * advances by the two Weyl increments.  Ten rounds.
 */
#include <stdint.h>
#include <stddef.h>

static void philox_round(uint32_t c[4], const uint32_t k[2]) {
    const uint64_t a = (uint64_t)0xD2511F53u * c[0];
    const uint64_t b = (uint64_t)0xCD9E8D57u * c[2];
    const uint32_t n0 = (uint32_t)(b >> 32) ^ c[1] ^ k[0];
    const uint32_t n1 = (uint32_t)b;
    const uint32_t n2 = (uint32_t)(a >> 32) ^ c[3] ^ k[1];
    const uint32_t n3 = (uint32_t)a;
    c[0] = n0; c[1] = n1; c[2] = n2; c[3] = n3;
}

void philox4x32_10_ref(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
    uint32_t c[4] = {ctr_in[0], ctr_in[1], ctr_in[2], ctr_in[3]};
    uint32_t k[2] = {key_in[0], key_in[1]};
    for (int r = 0; r < 10; ++r) {
        philox_round(c, k);
        k[0] += 0x9E3779B9u;
        k[1] += 0xBB67AE85u;
    }
    out[0] = c[0]; out[1] = c[1]; out[2] = c[2]; out[3] = c[3];
}

/* Batch form: n counters (4 words each) with one key; out gets 4 words each. */
void philox4x32_10_batch(const uint32_t* ctr, size_t n, uint32_t k0, uint32_t k1, uint32_t* out) {
    const uint32_t key[2] = {k0, k1};
    for (size_t i = 0; i < n; ++i) philox4x32_10_ref(ctr + 4 * i, key, out + 4 * i);
}
