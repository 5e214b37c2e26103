/*
 * Host side of the counter-based normal generator used for synthetic
 * weights, inputs and caches of the large workloads (input generation only;
 * none of the decode method's arithmetic is here).
 *
 * Generator (the same definition is implemented, separately, in the HIP
 * library's dv_fill_normal):
 *   Philox-4x32-10 (J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw,
 *   "Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011): 10 rounds of
 *     (c0, c1, c2, c3) <- (hi(M1*c2) ^ c1 ^ k0, lo(M1*c2), hi(M0*c0) ^ c3 ^ k1, lo(M0*c0))
 *   with M0 = 0xD2511F53, M1 = 0xCD9E8D57, and the key bumped by
 *   (0x9E3779B9, 0xBB67AE85) between rounds.
 *   Stream (seed, stream id), element i: block b = i / 4 has counter
 *   (b_lo, b_hi, stream_lo, stream_hi) and key (seed_lo, seed_hi); its four
 *   words x0..x3 give two Box-Muller pairs (x0, x1) and (x2, x3):
 *     u = (x_a + 1) / 2^32,  v = x_b / 2^32,  r = sqrt(-2 ln u)
 *     z_a = r cos(2 pi v),   z_b = r sin(2 pi v)          (in double)
 *   element 4b + j takes z_j; the value is mean + std * z in double,
 *   rounded to float (to half afterwards for half storage).
 *
 * Built with gcc into libsynth.so next to synth.py, which loads it.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>

static void philox4x32_10(uint32_t c[4], uint32_t k0, uint32_t k1) {
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
        const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c[1] ^ k0;
        const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c[3] ^ k1;
        c[0] = n0;
        c[1] = (uint32_t)p1;
        c[2] = n2;
        c[3] = (uint32_t)p0;
    }
}

/* One Philox block: out[4] from counter ctr[4] and key[2]. */
void synth_philox_block(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
    uint32_t c[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
    philox4x32_10(c, key[0], key[1]);
    for (int i = 0; i < 4; ++i) out[i] = c[i];
}

static void block_words(uint64_t b, uint64_t seed, uint64_t stream, uint32_t x[4]) {
    x[0] = (uint32_t)b;
    x[1] = (uint32_t)(b >> 32);
    x[2] = (uint32_t)stream;
    x[3] = (uint32_t)(stream >> 32);
    philox4x32_10(x, (uint32_t)seed, (uint32_t)(seed >> 32));
}

/* Raw words of elements [offset, offset + n) of the stream. */
void synth_philox_words(uint32_t* out, uint64_t n, uint64_t offset, uint64_t seed, uint64_t stream, int threads) {
    const int64_t b0 = (int64_t)(offset >> 2), b1 = (int64_t)((offset + n + 3) >> 2);
#pragma omp parallel for num_threads(threads) schedule(static)
    for (int64_t b = b0; b < b1; ++b) {
        uint32_t x[4];
        block_words((uint64_t)b, seed, stream, x);
        for (int j = 0; j < 4; ++j) {
            const uint64_t i = (uint64_t)b * 4 + (uint64_t)j;
            if (i >= offset && i < offset + n) out[i - offset] = x[j];
        }
    }
}

/* mean + std * z of elements [offset, offset + n) of the stream, as float. */
void synth_philox_normal(float* out, uint64_t n, uint64_t offset, uint64_t seed, uint64_t stream, float mean, float std,
                         int threads) {
    const int64_t b0 = (int64_t)(offset >> 2), b1 = (int64_t)((offset + n + 3) >> 2);
    const double two_pi = 6.283185307179586;
    const double inv32 = 1.0 / 4294967296.0;
#pragma omp parallel for num_threads(threads) schedule(static)
    for (int64_t b = b0; b < b1; ++b) {
        uint32_t x[4];
        block_words((uint64_t)b, seed, stream, x);
        double z[4];
        for (int p = 0; p < 2; ++p) {
            const double u = ((double)x[2 * p] + 1.0) * inv32;
            const double v = (double)x[2 * p + 1] * inv32;
            const double r = sqrt(-2.0 * log(u));
            const double t = two_pi * v;
            z[2 * p] = r * cos(t);
            z[2 * p + 1] = r * sin(t);
        }
        for (int j = 0; j < 4; ++j) {
            const uint64_t i = (uint64_t)b * 4 + (uint64_t)j;
            if (i >= offset && i < offset + n) out[i - offset] = (float)((double)mean + (double)std * z[j]);
        }
    }
}
