/* Synthetic model weights of the oracle, in plain C.
 *
 * TEST INFRASTRUCTURE ONLY (part of the oracle): computes exactly what
 * oracle/weights.py computes (stored_rows), for the full-width parity tests,
 * where the numpy version's rate (a few million values per second) cannot
 * cover every layer.  It shares no code with the HIP library.
 *
 * Definition (same as the numpy oracle): element n of tensor tau is
 * 0.02 * z, z from Box-Muller in fp64 over Philox4x32-10 (Salmon et al.,
 * SC'11; key = seed, counter = (n/4 low 32 bits, n/4 high 32 bits, tau,
 * 1 << 24)): words (r0, r1) feed elements 4q and 4q+1, words (r2, r3) feed
 * 4q+2 and 4q+3, u1 = (r_a + 1) / 2^32, u2 = r_b / 2^32,
 * z = sqrt(-2 ln u1) * (cos, sin)(2 pi u2).  The value is then rounded once
 * to its storage format, round to nearest even:
 *   fmt 0: fp32;   fmt 1: bf16 (8 significant bits);
 *   fmt 2: E4M3FN with a per-row bf16 scale s = bf16(max|w| / 448),
 *          stored value e4m3(w / s) * s (saturating at 448);
 *   fmt 3: MXFP4, one shared exponent per 32 columns,
 *          e = clamp(floor(log2 max|w|) - 2, -126, 127) (0 for an all-zero
 *          block), stored value e2m1(w / 2^e) * 2^e (saturating at 6);
 *   fmt 4: the unrounded fp64 value.
 * Pinned bit-exactly against oracle/weights.py in tests/test_oracle_wgen.py.
 *
 * Built with gcc without fast-math or FMA contraction, so every operation is
 * the IEEE double operation the numpy expressions perform, in their order.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

static void philox4x32_10(const uint32_t ctr[4], uint32_t k0, uint32_t k1, uint32_t out[4]) {
  uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    const uint32_t n1 = (uint32_t)p1;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    const uint32_t n3 = (uint32_t)p0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* round x to `sig` significant bits, ties to even, with a quantum of at
 * least 2^minq (frexp and ldexp are exact, nearbyint rounds to even) */
static double round_sig(double x, int sig, int minq) {
  int e;
  frexp(x, &e);
  int q = e - sig;
  if (q < minq) q = minq;
  return ldexp(nearbyint(ldexp(x, -q)), q);
}

static double round_bf16(double x) {
  const double out = round_sig(x, 8, -133);
  if (fabs(out) >= ldexp(1.0, 128)) return copysign(INFINITY, out);
  return out;
}

static double clampd(double x, double m) { return x > m ? m : (x < -m ? -m : x); }
static double round_e4m3(double x) { return clampd(round_sig(x, 4, -9), 448.0); }
static double round_e2m1(double x) { return clampd(round_sig(x, 2, -1), 6.0); }

static int mx_scale_exp(double amax) {
  if (!(amax > 0)) return 0;
  int e;
  frexp(amax, &e);
  int s = e - 1 - 2;
  if (s < -126) s = -126;
  if (s > 127) s = 127;
  return s;
}

/* 0.02 * z for elements [0, n_in) of row `row` of tensor tau (fp64); the
 * two elements of a Box-Muller pair share their radius and angle */
static void raw_row(uint64_t seed, uint32_t tau, int64_t row, int64_t n_in, double* w) {
  const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  const double two_pi = 2.0 * 3.141592653589793;   /* the double nearest pi */
  const int64_t beg = row * n_in, end = beg + n_in;
  for (int64_t q = beg >> 2; 4 * q < end; ++q) {
    const uint32_t ctr[4] = {(uint32_t)q, (uint32_t)((uint64_t)q >> 32), tau, 1u << 24};
    uint32_t r[4];
    philox4x32_10(ctr, k0, k1, r);
    for (int p = 0; p < 2; ++p) {
      const double u1 = ((double)r[2 * p] + 1.0) * 0x1p-32;
      const double u2 = (double)r[2 * p + 1] * 0x1p-32;
      const double rad = sqrt(-2.0 * log(u1));
      const double ang = two_pi * u2;
      const int64_t n0 = 4 * q + 2 * p;
      if (n0 >= beg && n0 < end) w[n0 - beg] = 0.02 * (rad * cos(ang));
      if (n0 + 1 >= beg && n0 + 1 < end) w[n0 + 1 - beg] = 0.02 * (rad * sin(ang));
    }
  }
}

/* Stored values of rows[0..n_rows) of tensor tau ([out][n_in]) in `out`
 * (n_rows x n_in, fp64).  aux: fmt 2 the row scales (n_rows), fmt 3 the
 * block exponents (n_rows x n_in/32); may be NULL.  Returns 0, or -1 for a
 * bad format or an MXFP4 row length that is not a multiple of 32. */
int wgen_rows(uint64_t seed, uint32_t tau, int64_t n_in, const int64_t* rows, int64_t n_rows, int fmt,
              double* out, double* aux) {
  if (fmt < 0 || fmt > 4 || (fmt == 3 && n_in % 32)) return -1;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < n_rows; ++i) {
    double* w = out + i * n_in;
    raw_row(seed, tau, rows[i], n_in, w);
    if (fmt == 0) {
      for (int64_t j = 0; j < n_in; ++j) w[j] = (double)(float)w[j];
    } else if (fmt == 1) {
      for (int64_t j = 0; j < n_in; ++j) w[j] = round_bf16(w[j]);
    } else if (fmt == 2) {
      double amax = 0.0;
      for (int64_t j = 0; j < n_in; ++j) amax = fmax(amax, fabs(w[j]));
      const double s = round_bf16(amax / 448.0);
      for (int64_t j = 0; j < n_in; ++j) w[j] = round_e4m3(w[j] / s) * s;
      if (aux) aux[i] = s;
    } else if (fmt == 3) {
      for (int64_t b = 0; b < n_in / 32; ++b) {
        double amax = 0.0;
        for (int j = 0; j < 32; ++j) amax = fmax(amax, fabs(w[b * 32 + j]));
        const int e = mx_scale_exp(amax);
        for (int j = 0; j < 32; ++j) w[b * 32 + j] = ldexp(round_e2m1(ldexp(w[b * 32 + j], -e)), e);
        if (aux) aux[i * (n_in / 32) + b] = (double)e;
      }
    }
  }
  return 0;
}
