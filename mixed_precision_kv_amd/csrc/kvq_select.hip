// Precision selection at prefill.
//
// MixKVQ ("方法细节" salience A_d = I_d * S_d; "MixKVQ的系统级实现细节": the
// importance aggregates every query head sharing the KV head): channels are
// ranked by SQ_d * range_d, where SQ_d = sum |Q_{t,d}| over the group's
// prefill queries and range_d = max - min of the Key tokens to be quantized;
// the positive factors 1/L_q and 1/(2^B - 1) do not change the order.
// PN-Mix (Eq.6): RoPE pairs ranked by sum ||q pair|| * sum ||k pair||.
//
// Sums are exact: every |q| (or pair norm, the correctly rounded double
// sqrt(a^2 + b^2)) is rounded to the grid 2^-64 and added as a 128-bit
// integer, so the result does not depend on how the work is split. One
// workgroup of 1024 threads handles one (batch, kv head): 64 column lanes x
// 16 row lanes stream the rows with coalesced loads.
#include "kvq_internal.h"
#include "kvq_rank.h"

namespace kvq {

// ------------------------------------------------------------------ MixKVQ
__global__ __launch_bounds__(1024) void select_mixkvq_kernel(SelectArgs A) {
  __shared__ u128 part[16][D];                 // 32 KB
  __shared__ float kmin[16][D], kmax[16][D];
  __shared__ double key_hi[D], key_lo[D];
  __shared__ int rank_s[D];
  __shared__ uint8_t tier_s[D];
  __shared__ uint8_t over_s[D];                // threshold tiers: 2 if A_d > tau_bf16, 1 if tau_u4 < A_d <= tau_bf16
  __shared__ int count_s[2];
  const int kvh = blockIdx.x, b = blockIdx.y;
  const int g = A.n_q_heads / A.n_kv_heads;
  const int j = threadIdx.x & 63, rl = threadIdx.x >> 6;   // channel pair, row lane

  u128 s0 = 0, s1 = 0;
  const int64_t rows = (int64_t)g * A.l_q;
  for (int64_t R = rl; R < rows; R += 16) {
    int hh = (int)(R / A.l_q);
    int64_t t = R - (int64_t)hh * A.l_q;
    const uint16_t* row = A.q + (((int64_t)b * A.n_q_heads + (int64_t)kvh * g + hh) * A.q_stride + t) * D;
    uint32_t w = reinterpret_cast<const uint32_t*>(row)[j];
    s0 += psi_bf16((uint16_t)(w & 0x7FFF));
    s1 += psi_bf16((uint16_t)((w >> 16) & 0x7FFF));
  }
  part[rl][2 * j] = s0;
  part[rl][2 * j + 1] = s1;

  float mn0 = INFINITY, mn1 = INFINITY, mx0 = -INFINITY, mx1 = -INFINITY;
  for (int64_t t = rl; t < A.l_k; t += 16) {
    const uint16_t* row = A.k + (((int64_t)b * A.n_kv_heads + kvh) * A.k_stride + t) * D;
    uint32_t w = reinterpret_cast<const uint32_t*>(row)[j];
    float v0 = bf16_to_f32((uint16_t)w), v1 = bf16_to_f32((uint16_t)(w >> 16));
    mn0 = fminf(mn0, v0); mx0 = fmaxf(mx0, v0);
    mn1 = fminf(mn1, v1); mx1 = fmaxf(mx1, v1);
  }
  kmin[rl][2 * j] = mn0; kmin[rl][2 * j + 1] = mn1;
  kmax[rl][2 * j] = mx0; kmax[rl][2 * j + 1] = mx1;
  __syncthreads();

  if (threadIdx.x < D) {
    int d = threadIdx.x;
    u128 sq = 0;
    float mn = INFINITY, mx = -INFINITY;
    for (int r = 0; r < 16; ++r) {
      sq += part[r][d];
      mn = fminf(mn, kmin[r][d]);
      mx = fmaxf(mx, kmax[r][d]);
    }
    const double range = (A.l_k > 0) ? (double)mx - (double)mn : 0.0;
    dd_key(sq, range, key_hi[d], key_lo[d]);
    if (A.threshold) {
      // the salience A_d against both thresholds, exactly (MixKVQ three-tier rule)
      const double n3 = 3.0 * (double)g * (double)A.l_q;
      const bool b16 = A.l_k > 0 && salience_vs_tau(sq, mx, mn, n3, A.tau_bf16) > 0;
      const bool b4 = A.l_k > 0 && salience_vs_tau(sq, mx, mn, n3, A.tau_u4) > 0;
      over_s[d] = b16 ? 2 : (b4 ? 1 : 0);
    }
    if (d < 2) count_s[d] = 0;
  }
  __syncthreads();
  // better(o, d): channel o ranks above channel d (larger key, ties to the lower channel)
  auto better = [&](int o, int d) {
    return key_hi[o] > key_hi[d] || (key_hi[o] == key_hi[d] && (key_lo[o] > key_lo[d] || (key_lo[o] == key_lo[d] && o < d)));
  };
  if (threadIdx.x < D) {
    const int d = threadIdx.x, r = key_rank(key_hi, key_lo, d);
    rank_s[d] = r;
    if (!A.threshold) {
      tier_s[d] = r < A.n16 ? 2 : (r < A.n16 + A.n4 ? 1 : 0);
    } else {
      // BF16: above tau_bf16 and among the n16 best of those
      int r16 = 0;
      for (int o = 0; o < D; ++o) r16 += over_s[o] == 2 && better(o, d);
      tier_s[d] = over_s[d] == 2 && r16 < A.n16 ? 2 : 0;
    }
  }
  __syncthreads();
  if (A.threshold && threadIdx.x < D) {
    // UINT4: the n4 best of the channels above tau_u4 only and those the
    // BF16 tier had no room for
    const int d = threadIdx.x;
    auto cand = [&](int o) { return tier_s[o] != 2 && over_s[o] != 0; };
    int r4 = 0;
    for (int o = 0; o < D; ++o) r4 += cand(o) && better(o, d);
    if (cand(d) && r4 < A.n4) over_s[d] = 3;   // marked; tier_s is still read by the other threads
  }
  __syncthreads();
  if (A.threshold && threadIdx.x < D && over_s[threadIdx.x] == 3) tier_s[threadIdx.x] = 1;
  __syncthreads();
  if (threadIdx.x < D && tier_s[threadIdx.x] != 0) atomicAdd(&count_s[2 - tier_s[threadIdx.x]], 1);
  __syncthreads();
  uint8_t* rec = A.out + ((int64_t)b * A.n_kv_heads + kvh) * MIX_RECORD;
  if (threadIdx.x < D) {
    int d = threadIdx.x, t = tier_s[d];
    const int n16 = count_s[0], n4 = count_s[1];   // the head's own counts (the configured ones by rank)
    int base = t == 2 ? 0 : (t == 1 ? n16 : n16 + n4);
    int pos = base;
    for (int o = 0; o < d; ++o) pos += tier_s[o] == t;
    rec[pos] = (uint8_t)d;
  } else if (threadIdx.x < D + 32) {
    int q = threadIdx.x - D;
    rec[D + q] = (uint8_t)(tier_s[4 * q] | (tier_s[4 * q + 1] << 2) | (tier_s[4 * q + 2] << 4) | (tier_s[4 * q + 3] << 6));
  }
}

// ------------------------------------------------------------------ PN-Mix
__global__ __launch_bounds__(1024) void select_pnmix_kernel(SelectArgs A) {
  __shared__ u128 qpart[16][64], kpart[16][64];
  __shared__ u128 qn[64], kn[64];
  __shared__ uint8_t hi_s[64];
  const int kvh = blockIdx.x, b = blockIdx.y;
  const int g = A.n_q_heads / A.n_kv_heads;
  const int i = threadIdx.x & 63, rl = threadIdx.x >> 6;
  const int d0 = A.pair_layout == KVQ_PAIR_HALF_SPLIT ? i : 2 * i;
  const int d1 = A.pair_layout == KVQ_PAIR_HALF_SPLIT ? i + 64 : 2 * i + 1;

  u128 sq = 0;
  const int64_t rows = (int64_t)g * A.l_q;
  for (int64_t R = rl; R < rows; R += 16) {
    int hh = (int)(R / A.l_q);
    int64_t t = R - (int64_t)hh * A.l_q;
    const uint16_t* row = A.q + (((int64_t)b * A.n_q_heads + (int64_t)kvh * g + hh) * A.q_stride + t) * D;
    double x = bf16_to_f64(row[d0]), y = bf16_to_f64(row[d1]);
    sq += psi_f64(sqrt(fma(x, x, y * y)));
  }
  u128 sk = 0;
  for (int64_t t = rl; t < A.l_k; t += 16) {
    const uint16_t* row = A.k + (((int64_t)b * A.n_kv_heads + kvh) * A.k_stride + t) * D;
    double x = bf16_to_f64(row[d0]), y = bf16_to_f64(row[d1]);
    sk += psi_f64(sqrt(fma(x, x, y * y)));
  }
  qpart[rl][i] = sq;
  kpart[rl][i] = sk;
  __syncthreads();
  if (threadIdx.x < 64) {
    u128 a = 0, c = 0;
    for (int r = 0; r < 16; ++r) {
      a += qpart[r][threadIdx.x];
      c += kpart[r][threadIdx.x];
    }
    qn[threadIdx.x] = a;
    kn[threadIdx.x] = c;
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    int me = threadIdx.x, r = 0;
    uint64_t kme[4];
    mul128(qn[me], kn[me], kme);
    for (int o = 0; o < 64; ++o) {
      uint64_t ko[4];
      mul128(qn[o], kn[o], ko);
      int c = cmp256(ko, kme);
      if (c > 0 || (c == 0 && o < me)) ++r;
    }
    hi_s[me] = r < A.n_hi_pairs;
  }
  __syncthreads();
  if (threadIdx.x < 8) {
    uint8_t byte = 0;
    for (int k = 0; k < 8; ++k) byte |= hi_s[8 * threadIdx.x + k] << k;
    A.out[((int64_t)b * A.n_kv_heads + kvh) * PN_RECORD + threadIdx.x] = byte;
  }
}

// ------------------------------------------------------------------ QJL outlier channels
// QJL outlier handling (Figure 2 orders channels by their mean magnitude
// over tokens): channels ranked by the exact sum of psi(|K_{t,d}|) over the
// prompt's Key tokens, ties to the lower channel; the n_out largest are the
// head's outlier channels, written as a 128-bit record (bit d % 8 of byte d / 8).
__global__ __launch_bounds__(1024) void select_qjl_outliers_kernel(SelectArgs A) {
  __shared__ u128 part[16][D];
  __shared__ u128 sum_s[D];
  __shared__ uint8_t out_s[D];
  const int kvh = blockIdx.x, b = blockIdx.y;
  const int j = threadIdx.x & 63, rl = threadIdx.x >> 6;
  u128 s0 = 0, s1 = 0;
  for (int64_t t = rl; t < A.l_k; t += 16) {
    const uint16_t* row = A.k + (((int64_t)b * A.n_kv_heads + kvh) * A.k_stride + t) * D;
    const uint32_t w = reinterpret_cast<const uint32_t*>(row)[j];
    s0 += psi_bf16((uint16_t)(w & 0x7FFF));
    s1 += psi_bf16((uint16_t)((w >> 16) & 0x7FFF));
  }
  part[rl][2 * j] = s0;
  part[rl][2 * j + 1] = s1;
  __syncthreads();
  if (threadIdx.x < D) {
    u128 s = 0;
    for (int r = 0; r < 16; ++r) s += part[r][threadIdx.x];
    sum_s[threadIdx.x] = s;
  }
  __syncthreads();
  if (threadIdx.x < D) {
    const int d = threadIdx.x;
    const u128 me = sum_s[d];
    int rank = 0;
    for (int o = 0; o < D; ++o) rank += (sum_s[o] > me) || (sum_s[o] == me && o < d);
    out_s[d] = rank < A.n_out;
  }
  __syncthreads();
  if (threadIdx.x < QJL_RECORD) {
    uint8_t byte = 0;
    for (int k = 0; k < 8; ++k) byte |= out_s[8 * threadIdx.x + k] << k;
    A.out[((int64_t)b * A.n_kv_heads + kvh) * QJL_RECORD + threadIdx.x] = byte;
  }
}

// ------------------------------------------------------------------ query accumulator
// acc[(b Hkv + h) D + d] += sum of psi(|q|) over the l_q query rows of every
// query head of the group: the running query-magnitude accumulator of the
// MixKVQ system section, exact and independent of how the rows are split
// between calls. One 1024-thread workgroup per (batch, kv head), the same
// row / column lanes as the selection.
__global__ __launch_bounds__(1024) void accumulate_query_kernel(SelectArgs A, u128* acc) {
  __shared__ u128 part[16][D];
  const int kvh = blockIdx.x, b = blockIdx.y;
  const int g = A.n_q_heads / A.n_kv_heads;
  const int j = threadIdx.x & 63, rl = threadIdx.x >> 6;
  u128 s0 = 0, s1 = 0;
  const int64_t rows = (int64_t)g * A.l_q;
  for (int64_t R = rl; R < rows; R += 16) {
    const int hh = (int)(R / A.l_q);
    const int64_t t = R - (int64_t)hh * A.l_q;
    const uint16_t* row = A.q + (((int64_t)b * A.n_q_heads + (int64_t)kvh * g + hh) * A.q_stride + t) * D;
    const uint32_t w = reinterpret_cast<const uint32_t*>(row)[j];
    s0 += psi_bf16((uint16_t)(w & 0x7FFF));
    s1 += psi_bf16((uint16_t)((w >> 16) & 0x7FFF));
  }
  part[rl][2 * j] = s0;
  part[rl][2 * j + 1] = s1;
  __syncthreads();
  if (threadIdx.x < D) {
    u128 sq = 0;
    for (int r = 0; r < 16; ++r) sq += part[r][threadIdx.x];
    acc[((int64_t)b * A.n_kv_heads + kvh) * D + threadIdx.x] += sq;
  }
}

hipError_t launch_accumulate(const SelectArgs& a, void* acc, int batch, hipStream_t stream) {
  hipLaunchKernelGGL(accumulate_query_kernel, dim3(a.n_kv_heads, batch), dim3(1024), 0, stream, a, (u128*)acc);
  return hipGetLastError();
}

hipError_t launch_select(int key_mode, const SelectArgs& a, int batch, hipStream_t stream) {
  dim3 grid(a.n_kv_heads, batch);
  if (key_mode == KVQ_KEY_MIXKVQ)
    hipLaunchKernelGGL(select_mixkvq_kernel, grid, dim3(1024), 0, stream, a);
  else if (key_mode == KVQ_KEY_PNMIX)
    hipLaunchKernelGGL(select_pnmix_kernel, grid, dim3(1024), 0, stream, a);
  else
    hipLaunchKernelGGL(select_qjl_outliers_kernel, grid, dim3(1024), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kvq
