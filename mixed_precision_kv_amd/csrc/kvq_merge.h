// The log-sum-exp merge of a decode call's split partials, shared by the
// merge kernel of the decode call and the kernel that runs it beside a flush.
#pragma once
#include "kvq_internal.h"

namespace kvq {

__device__ inline float wave_max64(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

__device__ inline float wave_sum64(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// What a merge adds beyond the split partials: NoWindow nothing.
struct NoWindow {
  __device__ inline void issue(int) {}
  __device__ inline void apply(float, float&, float&, int) {}
};

// KIVI Value FIFO on the pipelined kernels (KIVI blog sections 4-5): the
// window tokens inside the pages, n_tok of them from token t_lo of the first
// window page on, whose logits the split kernel left in spare records (one
// per window page, float = token in the page) and whose Values are the
// window's first n_tok rows. They add 2^(x_t - M) v_t to the output sum;
// their probabilities are already in the splits' l. A batch of 64 tokens:
// lane t loads token t's logit, and sixteen 16-byte loads per lane bring the
// rows, four per load (lane group g = lane / 16 row 4k + g, eight channels
// 8 (lane % 16) ..); the sums over the four row groups and the move to the
// merge's layout (lane l: channels 2l, 2l + 1) go through lane shuffles.
// The first batch is issued with the merge's first loads (17 loads, so that
// with a batch of up to 40 parts they stay within the 63 a wave keeps in
// flight).
struct FifoWindow {
  const float* logits;     // this query head's record of the first window page
  int64_t rec_stride;      // floats from one window page's record to the next
  const uint8_t* vrow0;    // the head's window row 0 (bf16 rows of 256 bytes)
  int t_lo, n_tok;         // n_tok >= 1
  float x;
  uint4 v[16];
  __device__ inline void load(int t0, int lane) {
    const int p = t_lo + min(t0 + lane, n_tok - 1);
    x = t0 + lane < n_tok ? logits[(int64_t)(p >> 7) * rec_stride + (p & 127)] : -INFINITY;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int t = min(t0 + 4 * k + (lane >> 4), n_tok - 1);
      v[k] = *reinterpret_cast<const uint4*>(vrow0 + (int64_t)t * (2 * D) + 16 * (lane & 15));
    }
  }
  __device__ inline void issue(int lane) { load(0, lane); }
  __device__ inline void apply(float M, float& o0, float& o1, int lane) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int t0 = 0;;) {
      const float w = x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(x - M);   // tokens past n_tok weigh 0
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const float wk = __shfl(w, 4 * k + (lane >> 4));
        const uint32_t d[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[2 * q] = fmaf(wk, __uint_as_float(d[q] << 16), acc[2 * q]);
          acc[2 * q + 1] = fmaf(wk, __uint_as_float(d[q] & 0xFFFF0000u), acc[2 * q + 1]);
        }
      }
      t0 += 64;
      if (t0 >= n_tok) break;
      load(t0, lane);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      acc[e] += __shfl_xor(acc[e], 16);
      acc[e] += __shfl_xor(acc[e], 32);
    }
    // channels 2 lane, 2 lane + 1 are elements 2 (lane % 4), + 1 of lane (lane / 4)'s block
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float a0 = __shfl(acc[2 * q], lane >> 2), a1 = __shfl(acc[2 * q + 1], lane >> 2);
      if ((lane & 3) == q) {
        s0 = a0;
        s1 = a1;
      }
    }
    o0 += s0;
    o1 += s1;
  }
};

// Merge of one query head's split partials (m, l, out[128] per split, out
// scaled by 2^-m) by one wave, lane l owning channels 2l and 2l+1:
//   M = max_j m_j, w_j = 2^(m_j - M), out = (sum_j w_j out_j) / (sum_j w_j l_j).
// M and the l sum come first, lane-parallel over the parts (lane i takes
// parts i, i + 64, ...), then out is one fused multiply-add chain over the
// parts in order, NB value rows at a time (NB <= 64), the weights reaching
// the lanes as lane reads (no LDS, no barrier). The result does not depend
// on NB, bit for bit. The first batch's loads are issued with the (m, l)
// loads, before any reduction, so up to min(NB, 64) parts cost one memory
// round trip. Zero parts give zero output. win adds its terms to the output
// sum before the division (its loads issued with the first batch's).
template <int NB, class Win = NoWindow>
__device__ inline void merge_row(const float* partial, float* out, int n_parts, int rows, int row,
                                 Win win = Win()) {
  static_assert(NB == 16 || NB == 32 || NB == 40 || NB == 48 || NB == 64, "batch of parts");
  const int lane = threadIdx.x & 63;
  float* dst = out + (int64_t)row * D + 2 * lane;
  if (n_parts <= 0) {
    dst[0] = 0.f;
    dst[1] = 0.f;
    return;
  }
  const int64_t stride = (int64_t)rows * RECORD;           // from one part's record to the next
  const float* base = partial + (int64_t)row * RECORD;
  const int last = n_parts - 1;                             // loads are clamped to parts that exist
  const float2 ml = *reinterpret_cast<const float2*>(base + min(lane, last) * stride);
  float2 v[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) v[j] = *reinterpret_cast<const float2*>(base + min(j, last) * stride + REC_OUT + 2 * lane);
  win.issue(lane);
  auto weight = [](float m, float Mx) { return m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - Mx); };
  float mloc = lane <= last ? ml.x : -INFINITY;
  for (int p = lane + 64; p <= last; p += 64) mloc = fmaxf(mloc, base[p * stride]);
  const float M = wave_max64(mloc);
  float lloc = lane <= last ? weight(ml.x, M) * ml.y : 0.f;
  for (int p = lane + 64; p <= last; p += 64) {
    const float2 t = *reinterpret_cast<const float2*>(base + p * stride);
    lloc += weight(t.x, M) * t.y;
  }
  const float l = wave_sum64(lloc);
  float o0 = 0.f, o1 = 0.f;
  float w = weight(ml.x, M);                                // lane j < NB: part j
  for (int s0 = 0;;) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if (s0 + j <= last) {                                 // uniform: parts past the end are skipped
        const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), j));
        o0 = fmaf(wj, v[j].x, o0);
        o1 = fmaf(wj, v[j].y, o1);
      }
    }
    s0 += NB;
    if (s0 > last) break;
#pragma unroll
    for (int j = 0; j < NB; ++j)
      v[j] = *reinterpret_cast<const float2*>(base + min(s0 + j, last) * stride + REC_OUT + 2 * lane);
    w = weight(base[min(s0 + lane % NB, last) * stride], M);
  }
  win.apply(M, o0, o1, lane);
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  dst[0] = o0 * inv;
  dst[1] = o1 * inv;
}

// NB for a call with n_parts parts: one batch whenever n_parts <= 64, and
// the smallest that covers the call (a wave keeps at most 63 loads in
// flight: NB + 1 loads of a batch past that wait for a second round trip).
inline int merge_batch(int n_parts) {
  return n_parts <= 16 ? 16 : n_parts <= 32 ? 32 : n_parts <= 40 ? 40 : n_parts <= 48 ? 48 : 64;
}

}  // namespace kvq
