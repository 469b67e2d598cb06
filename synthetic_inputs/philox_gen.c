/*
 * Seeded synthetic Q/K/V generator for the SSTA workloads.
 *
 * This file holds no part of the attention method: it only draws numbers.
 * Both the CPU oracle (oracle/) and the GPU library receive the arrays it
 * writes; neither links this code into its own arithmetic.
 *
 * Random bits: Philox4x32-10, from its published definition (Salmon, Moraes,
 * Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC'11): a
 * 4x32-bit counter and a 2x32-bit key, ten rounds of two 32x32->64 bit
 * multiplies with the constants 0xD2511F53 / 0xCD9E8D57, key bumped by the
 * Weyl constants 0x9E3779B9 / 0xBB67AE85 between rounds.
 *
 * Normals: Box-Muller on pairs of 32-bit uniforms u = (x + 0.5) / 2^32, so
 * u is never 0 or 1.
 *
 * Output: bf16 bit patterns (uint16), rounded to nearest-even from the fp32
 * rounding of the fp64 value.  Layout [batch, heads, T*H*W, head_dim], tokens
 * row-major over (t, y, x).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

typedef struct { uint32_t v[4]; } ctr4;

static inline void mulhilo32(uint32_t a, uint32_t b, uint32_t* hi, uint32_t* lo) {
  uint64_t p = (uint64_t)a * (uint64_t)b;
  *hi = (uint32_t)(p >> 32);
  *lo = (uint32_t)p;
}

ctr4 synth_philox4x32_10(ctr4 c, uint32_t k0, uint32_t k1) {
  for (int round = 0; round < 10; ++round) {
    uint32_t hi0, lo0, hi1, lo1;
    mulhilo32(0xD2511F53u, c.v[0], &hi0, &lo0);
    mulhilo32(0xCD9E8D57u, c.v[2], &hi1, &lo1);
    ctr4 n;
    n.v[0] = hi1 ^ c.v[1] ^ k0;
    n.v[1] = lo1;
    n.v[2] = hi0 ^ c.v[3] ^ k1;
    n.v[3] = lo0;
    c = n;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

/* Exported for the known-answer test of the generator itself. */
void synth_philox_block(const uint32_t ctr_in[4], const uint32_t key[2], uint32_t out[4]) {
  ctr4 c;
  memcpy(c.v, ctr_in, sizeof c.v);
  ctr4 r = synth_philox4x32_10(c, key[0], key[1]);
  memcpy(out, r.v, sizeof r.v);
}

static inline double u01(uint32_t x) { return ((double)x + 0.5) * (1.0 / 4294967296.0); }

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u) {       /* inf / nan: keep, quiet nan */
    uint16_t h = (uint16_t)(u >> 16);
    if (u & 0x007FFFFFu) h |= 0x0040u;
    return h;
  }
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

/* Stream ids inside one (seed, tensor) key: noise, frequencies, phases. */
enum { STREAM_NOISE = 0, STREAM_FREQ = 1, STREAM_PHASE = 2 };

static void noise4(uint64_t group, uint32_t tensor, uint32_t seed, double out[4]) {
  ctr4 c = {{(uint32_t)group, (uint32_t)(group >> 32), tensor, STREAM_NOISE}};
  ctr4 r = synth_philox4x32_10(c, seed, 0x53535441u);
  for (int p = 0; p < 2; ++p) {
    double u1 = u01(r.v[2 * p]), u2 = u01(r.v[2 * p + 1]);
    double rad = sqrt(-2.0 * log(u1));
    double ang = 6.283185307179586476925 * u2;
    out[2 * p] = rad * cos(ang);
    out[2 * p + 1] = rad * sin(ang);
  }
}

static double uniform_at(uint32_t stream, uint64_t idx, uint32_t tensor, uint32_t seed) {
  ctr4 c = {{(uint32_t)idx, (uint32_t)(idx >> 32), tensor, stream}};
  ctr4 r = synth_philox4x32_10(c, seed, 0x53535441u);
  return u01(r.v[0]);
}

/*
 * kind 0: x = noise_std * N(0,1)                          (i.i.d. Gaussian)
 * kind 1: x = sin(2*pi*(ft*t/T + fy*y/H + fx*x/W) + phi[h,d]) + noise_std * N(0,1)
 *         with (ft, fy, fx) ~ U[fmin, fmax] per (batch, head) and phi ~ U[0, 2*pi)
 *         per (batch, head, channel).
 * Element index e = ((b*heads + h)*N + n)*D + d; noise for e comes from
 * counter group e/4, lane e%4.
 */
int synth_generate(uint16_t* out, int32_t batch, int32_t heads, int32_t T, int32_t H, int32_t W,
                   int32_t D, int32_t kind, uint32_t seed, uint32_t tensor, double noise_std,
                   double fmin, double fmax) {
  if (!out || batch <= 0 || heads <= 0 || T <= 0 || H <= 0 || W <= 0 || D <= 0 || (D % 4) != 0)
    return -1;
  const int64_t N = (int64_t)T * H * W;
  const int64_t BH = (int64_t)batch * heads;
  for (int64_t bh = 0; bh < BH; ++bh) {
    double ft = 0, fy = 0, fx = 0;
    double cphi[1024], sphi[1024];
    if (D > 1024) return -1;
    if (kind == 1) {
      ft = fmin + (fmax - fmin) * uniform_at(STREAM_FREQ, (uint64_t)bh * 3 + 0, tensor, seed);
      fy = fmin + (fmax - fmin) * uniform_at(STREAM_FREQ, (uint64_t)bh * 3 + 1, tensor, seed);
      fx = fmin + (fmax - fmin) * uniform_at(STREAM_FREQ, (uint64_t)bh * 3 + 2, tensor, seed);
      for (int d = 0; d < D; ++d) {
        double phi = 6.283185307179586476925 *
                     uniform_at(STREAM_PHASE, (uint64_t)bh * D + d, tensor, seed);
        cphi[d] = cos(phi);
        sphi[d] = sin(phi);
      }
    }
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
      const int64_t t = n / ((int64_t)H * W);
      const int64_t y = (n / W) % H;
      const int64_t x = n % W;
      double sa = 0, ca = 0;
      if (kind == 1) {
        double a = 6.283185307179586476925 *
                   (ft * (double)t / T + fy * (double)y / H + fx * (double)x / W);
        sa = sin(a);
        ca = cos(a);
      }
      const int64_t e0 = (bh * N + n) * D;
      uint16_t* row = out + e0;
      for (int d = 0; d < D; d += 4) {
        double z[4];
        noise4((uint64_t)(e0 + d) >> 2, tensor, seed, z);
        for (int q = 0; q < 4; ++q) {
          double v = noise_std * z[q];
          if (kind == 1) v += sa * cphi[d + q] + ca * sphi[d + q];   /* sin(a + phi) */
          row[d + q] = f32_to_bf16_rne((float)v);
        }
      }
    }
  }
  return 0;
}
