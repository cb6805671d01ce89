// Split-K single-token decode attention over the packed cache.
//
// Computes, with one global softmax over [sinks | pages | residual] (KIVI
// blog section 6; MixKVQ Algorithm 1 Decoding; PN-Mix cache.attention; QJL
// EstimateScores + softmax), out = sum_t softmax(logit)_t * v^_t.
//
// Work split: workgroup = one wave64 = one (page range, kv head, batch); the
// last split of every (batch, kv head) handles the BF16 segment (sinks and
// residual). Each split writes (max, sum, unnormalised output) per query
// head; the last split to finish for a (batch, kv head) merges them
// (log-sum-exp) in the same launch.
//
// Per page, per kv head, the g query heads of the GQA group are processed
// together on MFMA v_mfma_f32_16x16x32_f16 (16x16 tiles, 64 lanes):
//  * Keys: logits[token][col] = sum_slot code[token][slot] * B[slot][col].
//    Codes (2-bit or 1-bit) become exact f16 integers through the fp4
//    converter (an fp4 nibble 0b00cc is c/2; the converter's power-of-two
//    scale 2 restores c). The per-page, per-channel Key scale is folded into
//    the query (B = q * s, split into f16 hi + lo parts for ~22-bit
//    precision) and the offsets into a per-head bias q . z, the InnerQ idea
//    of folding Key factors into the query. BF16-tier channels and the
//    BF16 segment use the bf16 MFMA with the raw bf16 query (exact products).
//  * Values: out[ch][col] = sum_t code[t][ch] * (p_t * s_{t,j}) + sum_t p_t z_{t,j};
//    the per-token value scale rides on the probabilities (B operand), the
//    offset term is accumulated per lane. Columns hold (value group j, head):
//    16 / g copies of each head's logits so every lane owns one (j, head).
// Lane conventions (verified on gfx950): lane l, a = l / 16, r = l % 16;
// A[row r][k 8a..8a+7], B[k 8a..8a+7][col r], D[row 4a..4a+3][col r].
#include "kvq_internal.h"

namespace kvq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float B_SCALE = 0.015625f;   // 2^-6 applied to every Key B operand (f16 range headroom)
constexpr float B_UNSCALE = 64.0f;
constexpr int MAX_KS = 8;              // max Key k-steps of 32 slots
constexpr int RECORD = 130;            // partial record per query head: m, l, out[128]


__device__ inline uint32_t rd(const u32x4& v, int i) { return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w)); }

__device__ inline u32x4 ld16(const uint8_t* p) { return *reinterpret_cast<const u32x4*>(p); }

__device__ inline uint32_t h2u(half2v h) {
  uint32_t u;
  __builtin_memcpy(&u, &h, 4);
  return u;
}

// fp4 pair conversion: byte `sel` of w (two nibbles 0b00cc / 0b000c) -> f16 (c_lo, c_hi)
template <int SEL>
__device__ inline uint32_t cvt2(uint32_t w) {
  return h2u(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 2.0f, SEL));
}

__device__ inline half8 u4_to_h8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  u32x4 v = {a, b, c, d};
  half8 h;
  __builtin_memcpy(&h, &v, 16);
  return h;
}

// 2-bit block dword w (tiles 2w, 2w+1 of one row) -> A fragments of both tiles
__device__ inline void expand2(uint32_t w, half8& t0, half8& t1) {
  uint32_t we = w & 0x33333333u, wo = (w >> 2) & 0x33333333u;
  t0 = u4_to_h8(cvt2<0>(we), cvt2<0>(wo), cvt2<1>(we), cvt2<1>(wo));
  t1 = u4_to_h8(cvt2<2>(we), cvt2<2>(wo), cvt2<3>(we), cvt2<3>(wo));
}

// 1-bit dword (tiles 4q..4q+3 of one row) -> A fragments of 4 tiles
__device__ inline void expand1(uint32_t w, half8* t) {
  uint32_t m0 = w & 0x11111111u, m1 = (w >> 1) & 0x11111111u, m2 = (w >> 2) & 0x11111111u,
           m3 = (w >> 3) & 0x11111111u;
  t[0] = u4_to_h8(cvt2<0>(m0), cvt2<0>(m1), cvt2<0>(m2), cvt2<0>(m3));
  t[1] = u4_to_h8(cvt2<1>(m0), cvt2<1>(m1), cvt2<1>(m2), cvt2<1>(m3));
  t[2] = u4_to_h8(cvt2<2>(m0), cvt2<2>(m1), cvt2<2>(m2), cvt2<2>(m3));
  t[3] = u4_to_h8(cvt2<3>(m0), cvt2<3>(m1), cvt2<3>(m2), cvt2<3>(m3));
}

__device__ inline f32x4 mfma(half8 a, half8 b, f32x4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0); }
__device__ inline f32x4 mfma_bf(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ inline float lo_bf(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float hi_bf(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// hi/lo f16 split of 8 products
__device__ inline void split8(const float* x, half8& hi, half8& lo) {
  for (int e = 0; e < 8; ++e) {
    _Float16 h = (_Float16)x[e];
    hi[e] = h;
    lo[e] = (_Float16)(x[e] - (float)h);
  }
}

__device__ inline float wave_max_groups(float v) {   // max over the 4 lane groups sharing a column
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}
__device__ inline float wave_sum_groups(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

// Online-softmax state of one lane (one head; one value group per pass).
template <int NPASS>
struct SoftState {
  float m;          // running max (log2 domain)
  float l;          // partial sum of p over this lane's tokens
  float z[NPASS];   // partial sum of p * value offset, per pass
  f32x4 acc[8];     // value accumulators of the 8 value tiles (16 channels each)
};

// Consume one page: logit[i][e] is the raw Key accumulator of tile i row e
// (token 16 i + 4 a + e); the log2-domain logit is logit * xs + xb.
template <int G, int NPASS>
__device__ inline void consume_values(SoftState<NPASS>& st, const f32x4 (&logit)[8], float xs, float xb,
                                      const u32x4 (&vc)[4], const uint8_t* vmeta, int a, int col) {
  constexpr int C = 16 / G;
  float pm = -INFINITY;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) pm = fmaxf(pm, logit[i][e]);
  pm = fmaf(wave_max_groups(pm), xs, xb);
  const float mn = fmaxf(st.m, pm);
  if (__any(mn > st.m)) {
    const float alpha = (st.m == -INFINITY) ? 0.f : exp2f(st.m - mn);
    st.l *= alpha;
#pragma unroll
    for (int P = 0; P < NPASS; ++P) st.z[P] *= alpha;
#pragma unroll
    for (int u = 0; u < 8; ++u) st.acc[u] *= alpha;
    st.m = mn;
  }
  const float shift = xb - st.m;
  float p[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      p[i][e] = exp2f(fmaf(logit[i][e], xs, shift));
      st.l += p[i][e];
    }
  const int jl = col / G;
#pragma unroll
  for (int P = 0; P < NPASS; ++P) {
    const int j = (jl + P * C) & 3;            // this lane's value group in pass P
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const uint8_t* mb = vmeta + 512 * ks + 128 * a + 32 * j;
      const u32x4 sw = ld16(mb), zw = ld16(mb + 16);
      half8 B;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t w = rd(sw, e >> 1), zz = rd(zw, e >> 1);
        const float s = (e & 1) ? hi_bf(w) : lo_bf(w);
        const float z = (e & 1) ? hi_bf(zz) : lo_bf(zz);
        const float pe = p[2 * ks + (e >> 2)][e & 3];     // token pi(ks, a, e)
        B[e] = (_Float16)(pe * s);
        st.z[P] = fmaf(pe, z, st.z[P]);
      }
#pragma unroll
      for (int w = 0; w < 4; ++w) {            // value tiles 2w, 2w+1 hold group w
        if (w / C != P) continue;
        half8 A0, A1;
        expand2(rd(vc[ks], w), A0, A1);
        st.acc[2 * w] = mfma(A0, B, st.acc[2 * w]);
        st.acc[2 * w + 1] = mfma(A1, B, st.acc[2 * w + 1]);
      }
    }
  }
}

// Write this split's (m, l, out) for the lane's head.
template <int G, int NPASS>
__device__ inline void write_partial(const DecodeArgs& A, SoftState<NPASS>& st, int split, int b, int kvh, int a,
                                     int col) {
  constexpr int C = 16 / G;
  const int h = col % G, jl = col / G;
  const float l = wave_sum_groups(st.l);
  float z[NPASS];
#pragma unroll
  for (int P = 0; P < NPASS; ++P) z[P] = wave_sum_groups(st.z[P]);
  float* rec = A.partial + (((int64_t)split * A.batch + b) * A.n_q_heads + kvh * G + h) * RECORD;
  if (a == 0 && jl == 0) {
    rec[0] = st.m;
    rec[1] = l;
  }
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int P = w / C;
    if (P >= NPASS || jl != w - P * C) continue;
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      const int u = 2 * w + t2;
#pragma unroll
      for (int e = 0; e < 4; ++e) rec[2 + 16 * u + 4 * a + e] = st.acc[u][e] + z[P];
    }
  }
}

constexpr int QJL_MAX_KS = 8;   // m <= 256

struct DecodeSmem {
  float qf[8][D];                              // the group's query heads (float)
  union {
    float qslot[MAX_KS][4][8][8];              // [k-step][lane group][head][e]: query value of a Key slot
    float p_lds[256][8];                       // BF16 segment: probabilities [token][head]
    half8 bq[2][QJL_MAX_KS][4][8];             // QJL: S q hi/lo [k-step][lane group][head]
  } u;
  int slot_ch[256];
  float mh[16];
};

// Key slot operand for k-step ks: B = q * s * 2^-6 (hi/lo), bias += q . z
__device__ inline void key_operand(const float* qv, const u32x4& sw, const u32x4& zw, half8& hi, half8& lo,
                                   float& bias) {
  float prod[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t w = rd(sw, e >> 1), z = rd(zw, e >> 1);
    prod[e] = qv[e] * ((e & 1) ? hi_bf(w) : lo_bf(w)) * B_SCALE;
    bias = fmaf(qv[e], (e & 1) ? hi_bf(z) : lo_bf(z), bias);
  }
  split8(prod, hi, lo);
}

// The split that arrives last for a (batch, kv head) merges all partials of
// its G query heads (log-sum-exp) and resets the arrival counter, so one
// launch produces the final output. Release: every split fences its partial
// stores before counting in; acquire: the last split fences before reading.
template <int G>
__device__ inline void finish_split(const DecodeArgs& A, int b, int kvh, int lane) {
  __threadfence();
  const int total = A.n_page_splits + 1;
  unsigned* ctr = A.counter + (int64_t)b * A.n_kv_heads + kvh;
  int old = 0;
  if (lane == 0) old = (int)atomicAdd(ctr, 1u);
  old = __shfl(old, 0);
  if (old != total - 1) return;
  __threadfence();
  const int64_t rows = (int64_t)A.batch * A.n_q_heads;
#pragma unroll 1
  for (int hh = 0; hh < G; ++hh) {
    const int64_t row = (int64_t)b * A.n_q_heads + kvh * G + hh;
    float M = -INFINITY;
    for (int s = 0; s < total; ++s) M = fmaxf(M, A.partial[(s * rows + row) * RECORD]);
    float l = 0.f, o0 = 0.f, o1 = 0.f;
    if (M != -INFINITY) {
      for (int s = 0; s < total; ++s) {
        const float* rec = A.partial + (s * rows + row) * RECORD;
        const float ms = rec[0];
        if (ms == -INFINITY) continue;
        const float w = exp2f(ms - M);
        l = fmaf(w, rec[1], l);
        o0 = fmaf(w, rec[2 + 2 * lane], o0);
        o1 = fmaf(w, rec[3 + 2 * lane], o1);
      }
    }
    const float inv = l > 0.f ? 1.f / l : 0.f;
    A.out[row * D + 2 * lane] = o0 * inv;
    A.out[row * D + 2 * lane + 1] = o1 * inv;
  }
  if (lane == 0) *ctr = 0u;
}

// ------------------------------------------------------------------ decode kernel
template <int MODE, int G>
__global__ __launch_bounds__(64) void decode_kernel(DecodeArgs A) {
  constexpr int C = 16 / G;
  constexpr int NPASS = (4 + C - 1) / C;
  __shared__ DecodeSmem S;
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x, a = lane >> 4, r = lane & 15, col = r;
  const int h = col % G;
  const int64_t head = (int64_t)b * A.n_kv_heads + kvh;
  const int hq = kvh * G + h;
  const uint16_t* qrow = A.q + ((int64_t)b * A.n_q_heads + hq) * D;

  // ---------------------------------------------------------------- BF16 segment
  if (split == A.n_page_splits) {
    const int T = A.n_sink + A.n_resid;
    bf16x8 Bq[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4 raw = ld16(reinterpret_cast<const uint8_t*>(qrow + 32 * ks + 8 * a));
      __builtin_memcpy(&Bq[ks], &raw, 16);
    }
    float mloc = -INFINITY;
    const int nt = (T + 15) / 16;
    for (int i = 0; i < nt; ++i) {
      const int t = 16 * i + r;                // A row = token
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        u32x4 raw = {0u, 0u, 0u, 0u};
        if (t < A.n_sink)
          raw = ld16(reinterpret_cast<const uint8_t*>(A.sink_k + (head * A.n_sink + t) * D + 32 * ks + 8 * a));
        else if (t < T)
          raw = ld16(reinterpret_cast<const uint8_t*>(A.resid_k + (head * A.resid_stride + (t - A.n_sink)) * D +
                                                      32 * ks + 8 * a));
        bf16x8 Ak;
        __builtin_memcpy(&Ak, &raw, 16);
        acc = mfma_bf(Ak, Bq[ks], acc);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int tok = 16 * i + 4 * a + e;
        const float x = tok < T ? acc[e] * A.scale_log2 : -INFINITY;
        mloc = fmaxf(mloc, x);
        if (col < G) S.u.p_lds[tok][col] = x;
      }
    }
    const float m = wave_max_groups(mloc);
    if (a == 0 && col < G) S.mh[col] = m;
    __syncthreads();
    for (int idx = lane; idx < 16 * nt * G; idx += 64) {
      const int tok = idx / G, hh = idx % G;
      S.u.p_lds[tok][hh] = tok < T ? exp2f(S.u.p_lds[tok][hh] - S.mh[hh]) : 0.f;
    }
    __syncthreads();
    float o[G][2], lsum[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) o[hh][0] = o[hh][1] = lsum[hh] = 0.f;
    for (int t = 0; t < T; ++t) {              // lane owns channels 2 lane, 2 lane + 1
      const uint16_t* vrow = t < A.n_sink ? A.sink_v + (head * A.n_sink + t) * D
                                          : A.resid_v + (head * A.resid_stride + (t - A.n_sink)) * D;
      const uint32_t w = reinterpret_cast<const uint32_t*>(vrow)[lane];
      const float v0 = lo_bf(w), v1 = hi_bf(w);
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float pp = S.u.p_lds[t][hh];
        o[hh][0] = fmaf(pp, v0, o[hh][0]);
        o[hh][1] = fmaf(pp, v1, o[hh][1]);
        lsum[hh] += pp;
      }
    }
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      float* rec = A.partial + (((int64_t)split * A.batch + b) * A.n_q_heads + kvh * G + hh) * RECORD;
      if (lane == 0) {
        rec[0] = T > 0 ? S.mh[hh] : -INFINITY;
        rec[1] = lsum[hh];
      }
      rec[2 + 2 * lane] = o[hh][0];
      rec[2 + 2 * lane + 1] = o[hh][1];
    }
    finish_split<G>(A, b, kvh, lane);
    return;
  }

  // ---------------------------------------------------------------- page splits
  for (int i = lane; i < G * D; i += 64)
    S.qf[i / D][i % D] = bf16_to_f32(A.q[((int64_t)b * A.n_q_heads + kvh * G + i / D) * D + i % D]);
  SoftState<NPASS> st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int P = 0; P < NPASS; ++P) st.z[P] = 0.f;
#pragma unroll
  for (int u = 0; u < 8; ++u) st.acc[u] = (f32x4){0.f, 0.f, 0.f, 0.f};
  const int p0 = split * A.pps;
  const int p1 = min(A.n_pages, p0 + A.pps);
  const uint8_t* pages = A.arena + head * A.max_pages * A.page_stride;

  if constexpr (MODE == KVQ_KEY_MIXKVQ) {
    const MixGeo g = mix_geo(A.n16, A.n4);
    const int NKS = (g.F + 3) / 4;
    const uint8_t* rec = A.mask + head * MIX_RECORD;
    for (int s = lane; s < 32 * NKS; s += 64) {
      int ch = -1;
      if (s < 2 * g.n4) ch = rec[g.n16 + (s >> 1)];
      else if (s >= g.s4 && s < g.s4 + g.n2) ch = rec[g.n16 + g.n4 + (s - g.s4)];
      S.slot_ch[s] = ch;
    }
    __syncthreads();
    for (int idx = lane; idx < NKS * 4 * G * 8; idx += 64) {
      const int e = idx & 7, hh = (idx >> 3) % G, aa = (idx >> 3) / G % 4, ks = (idx >> 3) / G / 4;
      const int ch = S.slot_ch[8 * (4 * ks + aa) + e];
      S.u.qslot[ks][aa][hh][e] = ch >= 0 ? S.qf[hh][ch] : 0.f;
    }
    const int NKB = (g.n16 + 31) / 32;
    bf16x8 Bq[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c = 32 * kb + 8 * a + e;
        Bq[kb][e] = (__bf16)(c < g.n16 ? S.qf[h][rec[c]] * B_SCALE : 0.f);
      }
    __syncthreads();
    const float xs = A.scale_log2 * B_UNSCALE;

    for (int pg = p0; pg < p1; ++pg) {
      const uint8_t* page = pages + (int64_t)pg * A.page_stride;
      u32x4 vc[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) vc[ks] = ld16(page + g.off_v + 1024 * ks + 256 * a + 16 * r);
      f32x4 logit[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) logit[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
      float bias = 0.f;
#pragma unroll
      for (int ks = 0; ks < MAX_KS; ++ks) {
        if (ks >= NKS) break;
        const int f = 4 * ks + a;
        u32x4 kc = {0u, 0u, 0u, 0u}, sw = {0u, 0u, 0u, 0u}, zw = {0u, 0u, 0u, 0u};
        if (f < g.F) {
          kc = ld16(page + g.off_codes + 256 * f + 16 * r);
          sw = ld16(page + g.off_meta + 32 * f);
          zw = ld16(page + g.off_meta + 32 * f + 16);
        }
        half8 Bhi, Blo;
        key_operand(S.u.qslot[ks][a][h], sw, zw, Bhi, Blo, bias);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          half8 A0, A1;
          expand2(rd(kc, w), A0, A1);
          logit[2 * w] = mfma(A0, Bhi, logit[2 * w]);
          logit[2 * w] = mfma(A0, Blo, logit[2 * w]);
          logit[2 * w + 1] = mfma(A1, Bhi, logit[2 * w + 1]);
          logit[2 * w + 1] = mfma(A1, Blo, logit[2 * w + 1]);
        }
      }
      for (int kb = 0; kb < NKB; ++kb) {        // BF16 tier, exact bf16 products
        u32x4 raw[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int c = 32 * kb + 8 * a + e;
          raw[e] = c < g.n16 ? ld16(page + 256 * c + 16 * r) : (u32x4){0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          uint16_t tmp[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) tmp[e] = (uint16_t)(rd(raw[e], i >> 1) >> (16 * (i & 1)));
          bf16x8 Ak;
          __builtin_memcpy(&Ak, tmp, 16);
          logit[i] = mfma_bf(Ak, Bq[kb], logit[i]);
        }
      }
      bias = wave_sum_groups(bias);
      consume_values<G, NPASS>(st, logit, xs, bias * A.scale_log2, vc, page + g.off_v + V_CODE_BYTES, a, col);
    }
  } else if constexpr (MODE == KVQ_KEY_PNMIX) {
    const PnGeo g = pn_geo(A.n_hi);
    const uint8_t* rec = A.mask + head * PN_RECORD;
    if (lane == 0) {                      // slot order: high channels ascending, then low ones
      int nh = 0;
      for (int d = 0; d < D; ++d) {
        const int pair = A.pair_layout == KVQ_PAIR_HALF_SPLIT ? (d & 63) : (d >> 1);
        if ((rec[pair >> 3] >> (pair & 7)) & 1) S.slot_ch[nh++] = d;
      }
      int nl = nh;
      for (int d = 0; d < D; ++d) {
        const int pair = A.pair_layout == KVQ_PAIR_HALF_SPLIT ? (d & 63) : (d >> 1);
        if (!((rec[pair >> 3] >> (pair & 7)) & 1)) S.slot_ch[nl++] = d;
      }
    }
    __syncthreads();
    for (int idx = lane; idx < 4 * 4 * G * 8; idx += 64) {
      const int e = idx & 7, hh = (idx >> 3) % G, aa = (idx >> 3) / G % 4, ks = (idx >> 3) / G / 4;
      S.u.qslot[ks][aa][hh][e] = S.qf[hh][S.slot_ch[8 * (4 * ks + aa) + e]];
    }
    __syncthreads();
    const int NUP = (g.n_hi + 31) / 32;
    const float xs = A.scale_log2 * B_UNSCALE;
    for (int pg = p0; pg < p1; ++pg) {
      const uint8_t* page = pages + (int64_t)pg * A.page_stride;
      u32x4 vc[4], lsb[2];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) vc[ks] = ld16(page + g.off_v + 1024 * ks + 256 * a + 16 * r);
#pragma unroll
      for (int P2 = 0; P2 < 2; ++P2) lsb[P2] = ld16(page + 1024 * P2 + 256 * a + 16 * r);
      f32x4 logit[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) logit[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
      float bias = 0.f;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int f = 4 * ks + a;
        const u32x4 sw = ld16(page + g.off_meta + 32 * f), zw = ld16(page + g.off_meta + 32 * f + 16);
        half8 Bhi, Blo;
        key_operand(S.u.qslot[ks][a][h], sw, zw, Bhi, Blo, bias);
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2) {       // LSB plane: 1-bit codes, weight s
          half8 At[4];
          expand1(rd(lsb[ks >> 1], 2 * (ks & 1) + q2), At);
#pragma unroll
          for (int T = 0; T < 4; ++T) {
            logit[4 * q2 + T] = mfma(At[T], Bhi, logit[4 * q2 + T]);
            logit[4 * q2 + T] = mfma(At[T], Blo, logit[4 * q2 + T]);
          }
        }
        if (ks < NUP) {                          // upper 2 bits of high channels, weight 2 s
          const u32x4 up = f < g.n_up_frag ? ld16(page + g.off_up + 256 * f + 16 * r) : (u32x4){0u, 0u, 0u, 0u};
          const half8 Uh = Bhi * (_Float16)2.0f, Ul = Blo * (_Float16)2.0f;
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            half8 A0, A1;
            expand2(rd(up, w), A0, A1);
            logit[2 * w] = mfma(A0, Uh, logit[2 * w]);
            logit[2 * w] = mfma(A0, Ul, logit[2 * w]);
            logit[2 * w + 1] = mfma(A1, Uh, logit[2 * w + 1]);
            logit[2 * w + 1] = mfma(A1, Ul, logit[2 * w + 1]);
          }
        }
      }
      bias = wave_sum_groups(bias);
      consume_values<G, NPASS>(st, logit, xs, bias * A.scale_log2, vc, page + g.off_v + V_CODE_BYTES, a, col);
    }
  } else {   // QJL
    const QjlGeo g = qjl_geo(A.qjl_m);
    const int NKS = A.qjl_m / 32;
    const float* sqrow = A.sq + ((int64_t)b * A.n_q_heads + hq) * A.qjl_m;
    float ssum = 0.f;
    for (int ks = 0; ks < NKS; ++ks) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = sqrow[32 * ks + 8 * a + e] * B_SCALE;
      half8 hi, lo;
      split8(x, hi, lo);
      if (col < G) {
        S.u.bq[0][ks][a][h] = hi;
        S.u.bq[1][ks][a][h] = lo;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) ssum += (float)hi[e] + (float)lo[e];
    }
    ssum = wave_sum_groups(ssum);          // sum_i (S q)_i * 2^-6 as seen by the MFMA
    __syncthreads();
    const float xs = A.scale_log2 * A.qjl_coef * B_UNSCALE;
    for (int pg = p0; pg < p1; ++pg) {
      const uint8_t* page = pages + (int64_t)pg * A.page_stride;
      u32x4 vc[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) vc[ks] = ld16(page + g.off_v + 1024 * ks + 256 * a + 16 * r);
      f32x4 logit[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) logit[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
      for (int P2 = 0; P2 < NKS / 2; ++P2) {
        const u32x4 v = ld16(page + 1024 * P2 + 256 * a + 16 * r);
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int ks = 2 * P2 + hf;
          const half8 Bh = S.u.bq[0][ks][a][h], Bl = S.u.bq[1][ks][a][h];
#pragma unroll
          for (int q2 = 0; q2 < 2; ++q2) {
            half8 At[4];
            expand1(rd(v, 2 * hf + q2), At);
#pragma unroll
            for (int T = 0; T < 4; ++T) {
              logit[4 * q2 + T] = mfma(At[T], Bh, logit[4 * q2 + T]);
              logit[4 * q2 + T] = mfma(At[T], Bl, logit[4 * q2 + T]);
            }
          }
        }
      }
      // estimator: nu_t * (2 <Sq, bits> - sum Sq); the norms of tokens 16 i + 4 a + e sit at 32 a + 4 i + e
      const uint8_t* nb = page + g.off_norm + 64 * a;
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const u32x4 nw = ld16(nb + 16 * qd);
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
          const int i = 2 * qd + ii;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t w = rd(nw, 2 * ii + (e >> 1));
            const uint16_t hb = (uint16_t)(w >> (16 * (e & 1)));
            _Float16 hv;
            __builtin_memcpy(&hv, &hb, 2);
            logit[i][e] = (float)hv * (2.0f * logit[i][e] - ssum);
          }
        }
      }
      consume_values<G, NPASS>(st, logit, xs, 0.f, vc, page + g.off_v + V_CODE_BYTES, a, col);
    }
  }
  write_partial<G, NPASS>(A, st, split, b, kvh, a, col);
  finish_split<G>(A, b, kvh, lane);
}

// QJL projection: S q for every query head (float accumulation of bf16 products).
__global__ __launch_bounds__(256) void qjl_project_kernel(const uint16_t* q, const uint16_t* S, float* sq, int m,
                                                          int n_rows) {
  const int row = blockIdx.x;          // (b, hq)
  if (row >= n_rows) return;
  __shared__ float qs[D];
  if (threadIdx.x < D) qs[threadIdx.x] = bf16_to_f32(q[(int64_t)row * D + threadIdx.x]);
  __syncthreads();
  for (int i = threadIdx.x; i < m; i += blockDim.x) {
    const uint16_t* srow = S + (int64_t)i * D;
    float acc = 0.f;
    for (int d = 0; d < D; ++d) acc = fmaf(bf16_to_f32(srow[d]), qs[d], acc);
    sq[(int64_t)row * m + i] = acc;
  }
}

int decode_pages_per_split(int n_pages, int batch, int n_kv_heads) {
  const int64_t units = (int64_t)n_pages * batch * n_kv_heads;
  int pps = (int)((units + 4095) / 4096);
  if (pps < 2) pps = 2;
  if (pps > 16) pps = 16;
  return pps;
}

template <int MODE>
static hipError_t launch_mode(const DecodeArgs& a, int g, dim3 grid, hipStream_t s) {
  switch (g) {
    case 1: hipLaunchKernelGGL((decode_kernel<MODE, 1>), grid, dim3(64), 0, s, a); break;
    case 2: hipLaunchKernelGGL((decode_kernel<MODE, 2>), grid, dim3(64), 0, s, a); break;
    case 4: hipLaunchKernelGGL((decode_kernel<MODE, 4>), grid, dim3(64), 0, s, a); break;
    case 8: hipLaunchKernelGGL((decode_kernel<MODE, 8>), grid, dim3(64), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode(int key_mode, const DecodeArgs& a, const uint16_t* qjl_s, hipStream_t s) {
  const int g = a.n_q_heads / a.n_kv_heads;
  if (key_mode == KVQ_KEY_QJL) {
    hipLaunchKernelGGL(qjl_project_kernel, dim3(a.batch * a.n_q_heads), dim3(256), 0, s, a.q, qjl_s,
                       const_cast<float*>(a.sq), a.qjl_m, a.batch * a.n_q_heads);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  dim3 grid(a.n_page_splits + 1, a.n_kv_heads, a.batch);
  hipError_t e;
  if (key_mode == KVQ_KEY_MIXKVQ) e = launch_mode<KVQ_KEY_MIXKVQ>(a, g, grid, s);
  else if (key_mode == KVQ_KEY_PNMIX) e = launch_mode<KVQ_KEY_PNMIX>(a, g, grid, s);
  else e = launch_mode<KVQ_KEY_QJL>(a, g, grid, s);
  return e;
}

}  // namespace kvq
