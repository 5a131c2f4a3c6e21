/*
 * Seeded synthetic inputs, host side.
 *
 * Holds none of the optimizer's arithmetic: it only turns (seed, stream,
 * block, purpose, step, index) into numbers.  The oracle's inputs come from
 * here; the device generator in csrc/synth_fill.hip implements the same
 * published generator independently, and a GPU test checks that the two
 * agree bit for bit.
 *
 * Generator: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
 * numbers: as easy as 1, 2, 3", SC'11), a counter-based generator: ten
 * rounds of two 32x32->64 multiplies whose halves are mixed into the
 * counter words, with a Weyl-sequence key schedule.
 *
 * Normal deviates: Irwin-Hall sum of the eight 16-bit halves of one Philox
 * output, centred (integer arithmetic, exact) and scaled by one FP32
 * multiply, so any two conforming implementations give identical bits.
 * Mean 0, standard deviation = the requested sigma (to FP32 rounding of the
 * scale), support +-4.9 sigma.
 *
 * Build: gcc -O2 -ffp-contract=off -shared -fPIC
 */
#include <stdint.h>
#include <string.h>

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

void synth_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4])
{
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int r = 0; r < 10; ++r) {
        uint64_t p0 = (uint64_t)PHILOX_M0 * c0;
        uint64_t p1 = (uint64_t)PHILOX_M1 * c2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
        k0 += PHILOX_W0; k1 += PHILOX_W1;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* Centred Irwin-Hall(8) integer of one Philox output: in [-262140, 262140]. */
static int32_t irwin_hall8(uint64_t index, uint32_t seed, uint32_t stream,
                           uint32_t block, uint32_t purpose, uint32_t step)
{
    uint32_t ctr[4] = { (uint32_t)index, (uint32_t)(index >> 32), block,
                        (purpose << 24) | (step & 0x00FFFFFFu) };
    uint32_t key[2] = { seed, stream };
    uint32_t r[4];
    synth_philox4x32_10(ctr, key, r);
    int32_t s = 0;
    for (int k = 0; k < 4; ++k) s += (int32_t)(r[k] & 0xFFFFu) + (int32_t)(r[k] >> 16);
    return s - 262140;   /* 8 * 65535 / 2 */
}

/* out[k] = normal deviate for index i0 + k, as FP32.  scale = sigma / sd of
 * the centred sum, already rounded to FP32 by the caller. */
void synth_normal_f32(float* out, uint64_t i0, uint64_t n, uint32_t seed, uint32_t stream,
                      uint32_t block, uint32_t purpose, uint32_t step, float scale)
{
    for (uint64_t k = 0; k < n; ++k)
        out[k] = (float)irwin_hall8(i0 + k, seed, stream, block, purpose, step) * scale;
}

/* The same deviates truncated to BF16 (upper 16 bits of the FP32 pattern). */
void synth_normal_bf16(uint16_t* out, uint64_t i0, uint64_t n, uint32_t seed, uint32_t stream,
                       uint32_t block, uint32_t purpose, uint32_t step, float scale)
{
    for (uint64_t k = 0; k < n; ++k) {
        float f = (float)irwin_hall8(i0 + k, seed, stream, block, purpose, step) * scale;
        uint32_t u;
        memcpy(&u, &f, 4);
        out[k] = (uint16_t)(u >> 16);
    }
}

/* Gathered forms: deviates at arbitrary indices (for sampled checks). */
void synth_normal_f32_at(float* out, const uint64_t* idx, uint64_t n, uint32_t seed,
                         uint32_t stream, uint32_t block, uint32_t purpose, uint32_t step,
                         float scale)
{
    for (uint64_t k = 0; k < n; ++k)
        out[k] = (float)irwin_hall8(idx[k], seed, stream, block, purpose, step) * scale;
}

void synth_normal_bf16_at(uint16_t* out, const uint64_t* idx, uint64_t n, uint32_t seed,
                          uint32_t stream, uint32_t block, uint32_t purpose, uint32_t step,
                          float scale)
{
    for (uint64_t k = 0; k < n; ++k) {
        float f = (float)irwin_hall8(idx[k], seed, stream, block, purpose, step) * scale;
        uint32_t u;
        memcpy(&u, &f, 4);
        out[k] = (uint16_t)(u >> 16);
    }
}

/* The four raw Philox words of indices i0 .. i0 + n - 1 (out[4k .. 4k+3]),
 * same counter and key as the deviates above. */
void synth_philox_words(uint32_t* out, uint64_t i0, uint64_t n, uint32_t seed, uint32_t stream,
                        uint32_t block, uint32_t purpose, uint32_t step)
{
    for (uint64_t k = 0; k < n; ++k) {
        const uint64_t index = i0 + k;
        uint32_t ctr[4] = { (uint32_t)index, (uint32_t)(index >> 32), block,
                            (purpose << 24) | (step & 0x00FFFFFFu) };
        uint32_t key[2] = { seed, stream };
        synth_philox4x32_10(ctr, key, out + 4 * k);
    }
}
