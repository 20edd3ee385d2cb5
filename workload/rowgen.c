/* Seeded synthetic KV rows: N(0,1) values rounded to bf16.
 *
 * Test and benchmark infrastructure, not part of the resolve path and holding
 * none of its arithmetic.  The value of every element is a pure function of
 * (data seed, request b, layer l, row p, element e), so any subset of rows can
 * be filled, in any order and on any number of threads, with identical bytes.
 *
 * Generator (published definitions, written out here):
 *   - Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
 *     easy as 1, 2, 3", SC 2011): key (seed, b), counter (e/4, p lo, p hi, l),
 *     giving four 32-bit words per group of four elements.
 *   - Box-Muller: words (x0, x1) and (x2, x3) each give two normals
 *     r cos(2 pi u2), r sin(2 pi u2) with r = sqrt(-2 ln u1),
 *     u1 = (x + 1) / 2^32 in (0, 1], u2 = x / 2^32 in [0, 1), in float64.
 *   - float64 -> float32 (round to nearest) -> bf16 (round to nearest even).
 *
 * The row shape is the sparse-MLA latent row: 576 bf16 per token (512 latent +
 * 64 rope); a page row is 16 token rows back to back.  Rows must be a multiple
 * of four elements.
 */
#include <math.h>
#include <stdint.h>

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

static inline void philox4x32_10(uint32_t c[4], uint32_t k0, uint32_t k1) {
  for (int r = 0; r < 10; ++r) {
    uint64_t p0 = (uint64_t)PHILOX_M0 * c[0];
    uint64_t p1 = (uint64_t)PHILOX_M1 * c[2];
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t n0 = hi1 ^ c[1] ^ k0;
    uint32_t n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
    k0 += PHILOX_W0;
    k1 += PHILOX_W1;
  }
}

static inline uint16_t f32_to_bf16_rne(float f) {
  union { float f; uint32_t u; } x;
  x.f = f;
  uint32_t u = x.u;
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

static void fill_one_row(uint16_t* d, int64_t row_elems, int64_t p, uint32_t seed,
                         uint32_t b, uint32_t l) {
  const double inv32 = 1.0 / 4294967296.0;
  const double two_pi = 6.283185307179586476925;
  for (int64_t e = 0; e < row_elems; e += 4) {
    uint32_t c[4] = {(uint32_t)(e >> 2), (uint32_t)p, (uint32_t)((uint64_t)p >> 32), l};
    philox4x32_10(c, seed, b);
    double u1 = ((double)c[0] + 1.0) * inv32, u2 = (double)c[1] * inv32;
    double u3 = ((double)c[2] + 1.0) * inv32, u4 = (double)c[3] * inv32;
    double r1 = sqrt(-2.0 * log(u1)), r2 = sqrt(-2.0 * log(u3));
    d[e + 0] = f32_to_bf16_rne((float)(r1 * cos(two_pi * u2)));
    d[e + 1] = f32_to_bf16_rne((float)(r1 * sin(two_pi * u2)));
    d[e + 2] = f32_to_bf16_rne((float)(r2 * cos(two_pi * u4)));
    d[e + 3] = f32_to_bf16_rne((float)(r2 * sin(two_pi * u4)));
  }
}

/* Fill rows [p0, p0 + n) of a stream whose row 0 starts at `base`. */
int hsw_fill_range(uint16_t* base, int64_t row_elems, int64_t p0, int64_t n,
                   uint32_t seed, uint32_t b, uint32_t l) {
  if (row_elems % 4 != 0 || n < 0 || p0 < 0) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n; ++r)
    fill_one_row(base + (p0 + r) * row_elems, row_elems, p0 + r, seed, b, l);
  return 0;
}

/* Fill the listed rows of a stream whose row 0 starts at `base`. */
int hsw_fill_rows(uint16_t* base, int64_t row_elems, const int64_t* rows, int64_t n,
                  uint32_t seed, uint32_t b, uint32_t l) {
  if (row_elems % 4 != 0 || n < 0) return -1;
  for (int64_t i = 0; i < n; ++i)
    if (rows[i] < 0) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i)
    fill_one_row(base + rows[i] * row_elems, row_elems, rows[i], seed, b, l);
  return 0;
}

/* Write the bytes of row p into `dst` (one row, for appends). */
int hsw_make_row(uint16_t* dst, int64_t row_elems, int64_t p, uint32_t seed, uint32_t b,
                 uint32_t l) {
  if (row_elems % 4 != 0 || p < 0) return -1;
  fill_one_row(dst, row_elems, p, seed, b, l);
  return 0;
}
