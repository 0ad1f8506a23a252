/*
 * Seeded, counter-based normal deviates for the synthetic MoE-layer inputs.
 *
 * This file is input generation only: it draws numbers and rounds them to the
 * storage precision. It computes nothing of the MoE layer itself. Both the
 * fp64 CPU oracle and the GPU library read the arrays it writes.
 *
 * Generator: Philox4x32-10 as published by Salmon, Moraes, Dror and Shaw,
 * "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11): a 4x32-bit counter,
 * a 2x32-bit key, ten rounds of two 32x32->64 multiplies with the published
 * multipliers and Weyl key increments.
 *
 * Element i of stream (seed, tensor_id, attempt) uses counter block
 * (i/2 low word, i/2 high word, attempt, 0) with key (seed, tensor_id).
 * The four output words form two 53-bit uniforms u1, u2 in (0,1); the
 * Box-Muller transform (Box & Muller 1958) gives r*cos(theta) for even i and
 * r*sin(theta) for odd i, r = sqrt(-2 ln u1), theta = 2*pi*u2. The deviate is
 * scaled by `std` in double precision, rounded to fp32 (round-to-nearest-even)
 * and, for bf16 storage, rounded again from fp32 to bf16 (RNE).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

static inline void philox_round(uint32_t c[4], const uint32_t k[2]) {
    uint64_t p0 = (uint64_t)PHILOX_M0 * c[0];
    uint64_t p1 = (uint64_t)PHILOX_M1 * c[2];
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t n0 = hi1 ^ c[1] ^ k[0];
    uint32_t n2 = hi0 ^ c[3] ^ k[1];
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
}

/* Philox4x32 with ten rounds; `ctr` and `key` are not modified. */
void moegen_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
    uint32_t c[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
    uint32_t k[2] = {key[0], key[1]};
    for (int r = 0; r < 10; ++r) {
        philox_round(c, k);
        k[0] += PHILOX_W0;
        k[1] += PHILOX_W1;
    }
    memcpy(out, c, sizeof(c));
}

static inline double unit53(uint32_t hi, uint32_t lo) {
    uint64_t v = (((uint64_t)hi << 32) | lo) >> 11; /* 53 random bits */
    return ((double)v + 0.5) * (1.0 / 9007199254740992.0);
}


/* fp32 -> bf16 bits, round to nearest even (inputs are finite). */
static inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

/* Both deviates of Philox block `blk`: element 2*blk is rad*cos(th), element 2*blk+1 is rad*sin(th)
   (Box-Muller on the block's two 53-bit uniforms); one Philox evaluation serves both. */
static inline void normal_pair(uint32_t seed, uint32_t tensor_id, uint32_t attempt, uint64_t blk, double* d0,
                               double* d1) {
    uint32_t ctr[4] = {(uint32_t)blk, (uint32_t)(blk >> 32), attempt, 0u};
    uint32_t key[2] = {seed, tensor_id};
    uint32_t r[4];
    moegen_philox4x32_10(ctr, key, r);
    double u1 = unit53(r[0], r[1]);
    double u2 = unit53(r[2], r[3]);
    double rad = sqrt(-2.0 * log(u1));
    double th = 6.283185307179586476925286766559 * u2;
    *d0 = rad * cos(th);
    *d1 = rad * sin(th);
}

/* Elements [i0, i0+n) of a stream through a per-element store callback, one Philox block per pair. */
#define MOEGEN_FILL(STORE)                                                                     \
    do {                                                                                       \
        uint64_t b0 = i0 >> 1, b1 = (i0 + n + 1) >> 1;                                        \
        _Pragma("omp parallel for schedule(static)")                                           \
        for (int64_t b = (int64_t)b0; b < (int64_t)b1; ++b) {                                  \
            double v[2];                                                                       \
            normal_pair(seed, tensor_id, attempt, (uint64_t)b, &v[0], &v[1]);                  \
            for (int h = 0; h < 2; ++h) {                                                      \
                uint64_t i = 2 * (uint64_t)b + (uint64_t)h;                                    \
                if (i >= i0 && i < i0 + n) { STORE(i - i0, v[h] * std); }                      \
            }                                                                                  \
        }                                                                                      \
    } while (0)

/* Unrounded deviates (scaled by std), elements [i0, i0+n). */
void moegen_normal_f64(uint32_t seed, uint32_t tensor_id, uint32_t attempt, uint64_t i0,
                       uint64_t n, double std, double* out) {
#define ST_F64(j, v) out[j] = (v)
    MOEGEN_FILL(ST_F64);
#undef ST_F64
}

/* Deviates rounded to fp32. */
void moegen_normal_f32(uint32_t seed, uint32_t tensor_id, uint32_t attempt, uint64_t i0,
                       uint64_t n, double std, float* out) {
#define ST_F32(j, v) out[j] = (float)(v)
    MOEGEN_FILL(ST_F32);
#undef ST_F32
}

/* Deviates rounded to fp32, then to bf16; written as raw bf16 bit patterns. */
void moegen_normal_bf16(uint32_t seed, uint32_t tensor_id, uint32_t attempt, uint64_t i0,
                        uint64_t n, double std, uint16_t* out) {
#define ST_BF16(j, v) out[j] = f32_to_bf16_rne((float)(v))
    MOEGEN_FILL(ST_BF16);
#undef ST_BF16
}

/* Raw Philox words for a block range, for known-answer checks. */
void moegen_philox_blocks(uint32_t seed, uint32_t tensor_id, uint32_t attempt, uint64_t b0,
                          uint64_t nb, uint32_t* out /* [nb*4] */) {
    for (uint64_t j = 0; j < nb; ++j) {
        uint64_t blk = b0 + j;
        uint32_t ctr[4] = {(uint32_t)blk, (uint32_t)(blk >> 32), attempt, 0u};
        uint32_t key[2] = {seed, tensor_id};
        moegen_philox4x32_10(ctr, key, out + 4 * j);
    }
}

/* Philox with an arbitrary counter and key, for the published known-answer vectors. */
void moegen_philox_raw(const uint32_t* ctr, const uint32_t* key, uint32_t* out) {
    moegen_philox4x32_10(ctr, key, out);
}
