// Exact query sums and MixKVQ channel ranking, shared by the prefill
// selection, the query accumulator and the flush that reselects per page
// (MixKVQ "方法细节": A_d = I_d * S_d; the system section: a running
// accumulator of query magnitudes, tiers refreshed at each flush).
#pragma once
#include "kvq_internal.h"

namespace kvq {

typedef unsigned __int128 u128;

// round_half_even(|bf16| * 2^64) as an integer (|x| < 2^63 assumed)
__device__ inline u128 psi_bf16(uint16_t bits) {
  int e = (bits >> 7) & 0xFF;
  uint32_t sig = (bits & 0x7F) | (e ? 0x80u : 0u);
  int ex = (e ? e : 1) - 134;          // value = sig * 2^ex
  int s = ex + 64;
  if (sig == 0) return 0;
  if (s >= 0) return (u128)sig << s;
  int rs = -s;
  if (rs > 9) return 0;
  uint32_t q = sig >> rs;
  uint32_t rem = sig & ((1u << rs) - 1);
  uint32_t half = 1u << (rs - 1);
  if (rem > half || (rem == half && (q & 1))) q += 1;
  return (u128)q;
}

// round_half_even(y * 2^64) for a finite double y >= 0 (y < 2^63)
__device__ inline u128 psi_f64(double y) {
  if (y <= 0.0) return 0;
  double z = y * 18446744073709551616.0;     // exact scaling by 2^64
  if (z < 9007199254740992.0) return (u128)(uint64_t)rint(z);
  union { double d; uint64_t u; } c;
  c.d = z;
  int e = (int)((c.u >> 52) & 0x7FF) - 1023;
  uint64_t sig = (c.u & 0xFFFFFFFFFFFFFull) | (1ull << 52);
  return (u128)sig << (e - 52);
}

// 128 x 128 -> 256-bit product as four 64-bit limbs (little end first)
__device__ inline void mul128(u128 a, u128 b, uint64_t out[4]) {
  uint64_t a0 = (uint64_t)a, a1 = (uint64_t)(a >> 64), b0 = (uint64_t)b, b1 = (uint64_t)(b >> 64);
  u128 p00 = (u128)a0 * b0, p01 = (u128)a0 * b1, p10 = (u128)a1 * b0, p11 = (u128)a1 * b1;
  u128 mid = (p00 >> 64) + (uint64_t)p01 + (uint64_t)p10;
  out[0] = (uint64_t)p00;
  out[1] = (uint64_t)mid;
  u128 hi = (mid >> 64) + (p01 >> 64) + (p10 >> 64) + p11;
  out[2] = (uint64_t)hi;
  out[3] = (uint64_t)(hi >> 64);
}
__device__ inline int cmp256(const uint64_t x[4], const uint64_t y[4]) {
  for (int i = 3; i >= 0; --i) {
    if (x[i] != y[i]) return x[i] > y[i] ? 1 : -1;
  }
  return 0;
}


// double-double key (kh + kl) = sq * range: sq = hi + lo exactly, the product
// from one fused multiply-add and the low part's product, renormalised.
__device__ inline void dd_key(u128 sq, double range, double& kh, double& kl) {
  const double hi = (double)sq;
  const double lo = (double)(__int128)(sq - (u128)hi);
  const double p = hi * range;
  const double e = fma(hi, range, -p) + lo * range;
  kh = p + e;
  kl = e - (kh - p);
}

// rank of channel d among the D keys: larger keys first, ties to the lower
// channel
__device__ inline int key_rank(const double* key_hi, const double* key_lo, int d) {
  int r = 0;
  for (int o = 0; o < D; ++o) {
    const bool better = key_hi[o] > key_hi[d] || (key_hi[o] == key_hi[d] && key_lo[o] > key_lo[d]);
    const bool same = key_hi[o] == key_hi[d] && key_lo[o] == key_lo[d];
    if (better || (same && o < d)) ++r;
  }
  return r;
}

// ---------------------------------------------------------------- threshold tiers
// Exact sign of a sum of doubles: the terms are added one by one into a
// nonoverlapping expansion (Shewchuk, "Adaptive Precision Floating-Point
// Arithmetic and Fast Robust Geometric Predicates", grow-expansion with the
// error-free two-sum), whose largest nonzero component carries the sign.
__device__ inline void two_sum_exact(double a, double b, double& s, double& e) {
#pragma clang fp contract(off)
  s = a + b;
  const double bb = s - a;
  e = (a - (s - bb)) + (b - bb);
}
template <int N>
__device__ inline int exact_sign(const double (&t)[N]) {
  double h[N];
  int m = 0;
  for (int i = 0; i < N; ++i) {
    double q = t[i];
    for (int j = 0; j < m; ++j) {
      double s, e;
      two_sum_exact(q, h[j], s, e);
      h[j] = e;
      q = s;
    }
    h[m++] = q;
  }
  for (int j = m - 1; j >= 0; --j)
    if (h[j] != 0.0) return h[j] > 0.0 ? 1 : -1;
  return 0;
}

// Sign of A_d - tau for the MixKVQ salience A_d = I_d * S_d (MixKVQ
// "方法细节"): I_d = SQ_d 2^-64 / (g l_q), S_d = (mx - mn) / 3 (B = 2), so
// A_d - tau has the sign of SQ_d (mx - mn) - tau * 3 g l_q * 2^64, evaluated
// exactly: SQ_d in three 43-bit pieces, mx - mn as an exact two-sum, every
// product as an exact fused-multiply-add pair. n3 = 3 g l_q < 2^53; tau is 0
// or 2^-900 <= |tau| <= 2^900, so no partial product underflows.
__device__ inline int salience_vs_tau(u128 sq, float mx, float mn, double n3, double tau) {
#pragma clang fp contract(off)
  double rh, rl;
  two_sum_exact((double)mx, -(double)mn, rh, rl);
  const double c[3] = {(double)(uint64_t)(sq & ((((u128)1) << 43) - 1)),
                       (double)(uint64_t)((sq >> 43) & ((((u128)1) << 43) - 1)) * 0x1p43,
                       (double)(uint64_t)(sq >> 86) * 0x1p86};
  double t[14];
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    t[4 * i] = c[i] * rh;
    t[4 * i + 1] = fma(c[i], rh, -t[4 * i]);
    t[4 * i + 2] = c[i] * rl;
    t[4 * i + 3] = fma(c[i], rl, -t[4 * i + 2]);
  }
  const double th = tau * n3;
  const double tl = fma(tau, n3, -th);
  t[12] = -th * 0x1p64;
  t[13] = -tl * 0x1p64;
  return exact_sign(t);
}

// Tier counts of a head under the thresholds: c16 channels have A_d >
// tau_bf16, c4 have tau_u4 < A_d <= tau_bf16. The tiers are contiguous in the
// ranking; capacities cap16 / cap4 keep the highest-ranked channels of a tier
// that overflows and pass the rest down one tier.
__device__ inline void threshold_counts(int c16, int c4, int cap16, int cap4, int& n16, int& n4) {
  n16 = min(c16, cap16);
  n4 = min(c16 - n16 + c4, cap4);
}

}  // namespace kvq
