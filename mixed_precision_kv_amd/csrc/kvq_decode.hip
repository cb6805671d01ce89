// Split-K single-token decode attention over the packed cache.
//
// Computes, with one global softmax over [sinks | pages | residual] (KIVI
// blog section 6; MixKVQ Algorithm 1 Decoding; PN-Mix cache.attention; QJL
// EstimateScores + softmax), out = sum_t softmax(logit)_t * v^_t.
//
// Work split: workgroup = one wave64 = one (page range, kv head, batch); the
// last split of every (batch, kv head) handles the BF16 segment (sinks and
// residual). Each split writes (max, sum, unnormalised output) per query
// head; a small combine kernel merges them (log-sum-exp). Keeping the merge
// in its own launch lets the kernel boundary order the partial writes; an
// in-kernel merge needs device-scope fences that write back the whole L2.
//
// Per page, per kv head, the g query heads of the GQA group are processed
// together on MFMA v_mfma_f32_16x16x32_f16 (16x16 tiles, 64 lanes):
//  * Keys: logits[token][col] = sum_slot code[token][slot] * B[slot][col].
//    Codes (2-bit or 1-bit) are masked straight out of the packed words as
//    binary16 subnormals c * 2^(l - 24), one power of two l per 16-token
//    tile, which the f16 MFMA multiplies exactly; the power is divided out
//    of each tile's sums (no conversion instruction per code). The
//    per-page, per-channel Key scale is folded into the query (B = q * s, split into f16 hi + lo parts for ~22-bit
//    precision) and the offsets into a per-head bias q . z, the InnerQ idea
//    of folding Key factors into the query. BF16-tier channels and the
//    BF16 segment use the bf16 MFMA with the raw bf16 query (exact products).
//  * Values: out[ch][col] = sum_t code[t][ch] * (p_t * s_{t,j}) + sum_t p_t z_{t,j};
//    the per-token value scale rides on the probabilities (B operand), the
//    offset term is accumulated per lane. Columns hold (value group j, head):
//    16 / g copies of each head's logits so every lane owns one (j, head).
// Lane conventions (verified on gfx950): lane l, a = l / 16, r = l % 16;
// A[row r][k 8a..8a+7], B[k 8a..8a+7][col r], D[row 4a..4a+3][col r].
#include "kvq_decode_common.h"
#include "kvq_merge.h"

namespace kvq {

constexpr int QJL_MAX_KS = 12;  // m + mo <= 384

struct DecodeSmem {
  float qf[8][D];                              // the group's query heads (float)
  union {
    float qslot[MAX_KS][4][8][8];              // [k-step][lane group][head][e]: query value of a Key slot
    float p_lds[256][8];                       // BF16 segment: probabilities [token][head]
    half8 bq[2][QJL_MAX_KS][4][8];             // QJL: S q hi/lo [k-step][lane group][head]
  } u;
  int slot_ch[256];
  float mh[16];
  alignas(16) uint8_t rec[MIX_RECORD];         // MixKVQ: the head's record (one record per head)
};

// KIVI Value FIFO (KIVI blog sections 4-5): tokens of page pg from vlim on
// have sealed Keys but their Values still in the full-precision window (row
// pg * 128 + t - vq_end). Their probabilities, staged in hp by the HYB
// consume_values, weight those rows here; lane l owns channels 2l, 2l+1 of
// every head. Sixteen rows' loads are issued together (one wait per chunk,
// not one memory latency per token); past the page's end a lane reloads row
// PAGE - 1, which is in the window since vlim < PAGE, and adds nothing.
template <int G>
__device__ inline void fifo_values(const DecodeArgs& A, int64_t head, int pg, int vlim, float (*hp)[8],
                                   float (&ow)[8][2], int lane) {
  __syncthreads();   // hp written
  const uint32_t* win = reinterpret_cast<const uint32_t*>(A.vwin + head * A.vwin_stride * D) + lane;
  for (int t0 = max(vlim, 0); t0 < PAGE; t0 += 16) {
    uint32_t w[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int64_t row = (int64_t)pg * PAGE + min(t0 + j, PAGE - 1) - A.vq_end;
      w[j] = win[row * (D / 2)];
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (t0 + j < PAGE) {
        const float v0 = lo_bf(w[j]), v1 = hi_bf(w[j]);
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          ow[hh][0] = fmaf(hp[t0 + j][hh], v0, ow[hh][0]);
          ow[hh][1] = fmaf(hp[t0 + j][hh], v1, ow[hh][1]);
        }
      }
    }
  }
  __syncthreads();   // hp free for the next page
}

// The page's first token whose Value is not quantized yet (PAGE: all are).
__device__ inline int fifo_vlim(const DecodeArgs& A, int pg) {
  return (int)min((int64_t)PAGE, max((int64_t)0, (int64_t)A.vq_end - (int64_t)pg * PAGE));
}

// After a page's consume_values: ow follows the running maximum like the
// value accumulators, then takes the page's full-precision Values. A lane's
// st.m is its own column's head's maximum, while ow holds every head's
// channels, so head hh's factor comes from lane hh (column hh, head hh).
template <int G, int NPASS>
__device__ inline void fifo_after(const DecodeArgs& A, const SoftState<NPASS>& st, float m0, int64_t head, int pg,
                                  int vlim, float (*hp)[8], float (&ow)[8][2], int lane) {
  if (__any(st.m != m0)) {
    const float alpha = m0 == -INFINITY ? 0.f : fast_exp2(m0 - st.m);   // 1 where the maximum held
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const float ah = __shfl(alpha, hh);
      ow[hh][0] *= ah;
      ow[hh][1] *= ah;
    }
  }
  if (vlim < PAGE) fifo_values<G>(A, head, pg, vlim, hp, ow, lane);
}

// ------------------------------------------------------------------ decode kernel
// FIFO: KIVI Value-FIFO decodes (tokens from A.vq_end on take full-precision
// Values); their probability staging hp[PAGE][8] is the launch's dynamic LDS.
template <int MODE, int G, bool FIFO>
__global__ __launch_bounds__(64) void decode_kernel(DecodeArgs A) {
  constexpr int C = 16 / G;
  constexpr int NPASS = (4 + C - 1) / C;
  __shared__ DecodeSmem S;
  extern __shared__ float fifo_lds[];
  float (*hp)[8] = reinterpret_cast<float (*)[8]>(fifo_lds);
  const DecodeBlock blk = decode_block(A);
  const int split = blk.split, kvh = blk.kvh, b = blk.b;
  const int lane = threadIdx.x, a = lane >> 4, r = lane & 15, col = r;
  const int h = col % G;
  const int64_t head = (int64_t)b * A.n_kv_heads + kvh;
  const int hq = kvh * G + h;
  const uint16_t* qrow = A.q + ((int64_t)b * A.n_q_heads + hq) * D;

  if (split >= A.n_page_splits) {
    bf16_segment<G>(A, split, b, kvh, lane, S.u.p_lds, S.mh);
    return;
  }

  // ---------------------------------------------------------------- page splits
  // The set-up's loads are issued together: the group's query rows (G x 128
  // bf16, contiguous: one 16-byte piece per lane and step) and, for MixKVQ
  // with one record per head, that record (staged in LDS).
  {
    constexpr int QP = G * D / 8;
    constexpr int QS = (QP + 63) / 64;
    const uint8_t* qg = reinterpret_cast<const uint8_t*>(A.q + ((int64_t)b * A.n_q_heads + kvh * G) * D);
    u32x4 qv[QS];
#pragma unroll
    for (int j = 0; j < QS; ++j) qv[j] = lane + 64 * j < QP ? ld16(qg + 16 * (lane + 64 * j)) : (u32x4){0u, 0u, 0u, 0u};
    const bool rec_lds = MODE == KVQ_KEY_MIXKVQ && A.rec_stride == 0 && lane < MIX_RECORD / 16;
    const u32x4 rv = rec_lds ? ld16(A.mask + head * MIX_RECORD + 16 * lane) : (u32x4){0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < QS; ++j) {
      const int i = lane + 64 * j;
      if (i < QP) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t w = rd(qv[j], k);
          S.qf[(8 * i) / D][(8 * i) % D + 2 * k] = lo_bf(w);
          S.qf[(8 * i) / D][(8 * i) % D + 2 * k + 1] = hi_bf(w);
        }
      }
    }
    if (rec_lds) *reinterpret_cast<u32x4*>(S.rec + 16 * lane) = rv;
    __syncthreads();
  }
  SoftState<NPASS> st;
  init_state(st);
  float ow[8][2];   // KIVI Value FIFO: full-precision Values of the split's pages, lane's channels
#pragma unroll
  for (int hh = 0; hh < 8; ++hh) ow[hh][0] = ow[hh][1] = 0.f;
  const int p0 = split * A.pps;
  const int p1 = min(A.n_pages, p0 + A.pps);

  if constexpr (MODE == KVQ_KEY_MIXKVQ) {
    const uint8_t* hrec = A.rec_stride == 0 ? S.rec : A.mask + head * MIX_RECORD;   // the head's record
    int hn16 = A.n16, hn4 = A.n4;
    if (A.head_tiers) mix_record_counts(hrec, hn16, hn4);   // threshold tiers: the head's counts
    const MixGeo g = mix_geo(hn16, hn4);
    const int NKS = (g.F + 3) / 4;
    const int NKB = (g.n16 + 31) / 32;
    bf16x8 Bq[4];
    // slot -> channel and the query tables of a record: once per split, or
    // at every page when every page has its own record (per-flush reselection)
    auto tables = [&](const uint8_t* rec) {
      __syncthreads();
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
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int c = 32 * kb + 8 * a + e;
          Bq[kb][e] = (__bf16)(c < g.n16 ? S.qf[h][rec[c]] * B_SCALE : 0.f);
        }
      __syncthreads();
    };
    if (A.rec_stride == 0) tables(hrec);
    const float xs = A.scale_log2 * B_UNSCALE;

    for (int pg = p0; pg < p1; ++pg) {
      if (A.rec_stride) tables(A.mask + (head * A.rec_stride + pg) * MIX_RECORD);
      const uint8_t* page = page_ptr(A, head, pg);
      // the page's loads are issued together: Value codes and metadata, the
      // first BF16 block and four Key k-steps at a time
      u32x4 vc[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) vc[ks] = ld16(page + g.off_v + 1024 * ks + 256 * a + 16 * r);
      const uint8_t *vlo = page + g.off_v + V_CODE_BYTES, *vhi = vlo + 1024;
      VMeta<G, NPASS> vm;
      load_vmeta<G, NPASS>(vm, vlo, vhi, a, col);
      u32x4 raw0[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c = 8 * a + e;
        raw0[e] = c < g.n16 ? ld16(page + 256 * c + 16 * r) : (u32x4){0u, 0u, 0u, 0u};
      }
      f32x4 logit[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) logit[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
      float bias = 0.f;
      for (int k0 = 0; k0 < NKS; k0 += 4) {
        u32x4 kc[4], sw[4], zw[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int f = 4 * (k0 + j) + a;
          kc[j] = sw[j] = zw[j] = (u32x4){0u, 0u, 0u, 0u};
          if (k0 + j < NKS && f < g.F) {
            kc[j] = ld16(page + g.off_codes + 256 * f + 16 * r);
            sw[j] = ld16(page + g.off_meta + 32 * f);
            zw[j] = ld16(page + g.off_meta + 32 * f + 16);
          }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int ks = k0 + j;
          if (ks >= NKS) break;
          half8 Bhi, Blo;
          key_operand(S.u.qslot[ks][a][h], sw[j], zw[j], Bhi, Blo, bias);
          const u32x4 kc8 = kc[j] >> 8u;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const half8 At = tile2(kc[j], kc8, i);
            logit[i] = mfma(At, Bhi, logit[i]);
            logit[i] = mfma(At, Blo, logit[i]);
          }
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) logit[i] *= tile_unscale(i);
      for (int kb = 0; kb < NKB; ++kb) {        // BF16 tier, exact bf16 products
        u32x4 raw[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int c = 32 * kb + 8 * a + e;
          raw[e] = kb == 0 ? raw0[e] : c < g.n16 ? ld16(page + 256 * c + 16 * r) : (u32x4){0u, 0u, 0u, 0u};
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
      if constexpr (FIFO) {
        const int vlim = fifo_vlim(A, pg);
        const float m0 = st.m;
        if (vlim >= PAGE) consume_values<G, NPASS>(st, logit, xs, bias * A.scale_log2, vc, vm, a, col);
        else consume_values<G, NPASS, true>(st, logit, xs, bias * A.scale_log2, vc, vm, a, col, vlim, hp);
        fifo_after<G, NPASS>(A, st, m0, head, pg, vlim, hp, ow, lane);
      } else {
        consume_values<G, NPASS>(st, logit, xs, bias * A.scale_log2, vc, vm, a, col);
      }
    }
  } else if constexpr (MODE == KVQ_KEY_PNMIX) {
    const PnGeo g = pn_geo(A.n_hi);
    // the 64 pair bits, bit i of byte i / 8 (one 8-byte load; records are 8-byte aligned)
    const uint64_t pbits = *reinterpret_cast<const uint64_t*>(A.mask + head * PN_RECORD);
    if (lane == 0) {                      // slot order: high channels ascending, then low ones
      int nh = 0;
      for (int d = 0; d < D; ++d) {
        const int pair = A.pair_layout == KVQ_PAIR_HALF_SPLIT ? (d & 63) : (d >> 1);
        if ((pbits >> pair) & 1) S.slot_ch[nh++] = d;
      }
      int nl = nh;
      for (int d = 0; d < D; ++d) {
        const int pair = A.pair_layout == KVQ_PAIR_HALF_SPLIT ? (d & 63) : (d >> 1);
        if (!((pbits >> pair) & 1)) S.slot_ch[nl++] = d;
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
      const uint8_t* page = page_ptr(A, head, pg);
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
        {                                        // LSB plane: 1-bit codes, weight s
          const Row1 x = row1(rd(lsb[ks >> 1], 2 * (ks & 1)), rd(lsb[ks >> 1], 2 * (ks & 1) + 1));
#pragma unroll
          for (int T = 0; T < 8; ++T) {
            const half8 At = tile1(x, T);
            logit[T] = mfma(At, Bhi, logit[T]);
            logit[T] = mfma(At, Blo, logit[T]);
          }
        }
        if (ks < NUP) {                          // upper 2 bits of high channels, weight 2 s
          const u32x4 up = f < g.n_up_frag ? ld16(page + g.off_up + 256 * f + 16 * r) : (u32x4){0u, 0u, 0u, 0u};
          const u32x4 up8 = up >> 8u;
          const half8 Uh = Bhi * (_Float16)2.0f, Ul = Blo * (_Float16)2.0f;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const half8 At = tile2(up, up8, i);
            logit[i] = mfma(At, Uh, logit[i]);
            logit[i] = mfma(At, Ul, logit[i]);
          }
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) logit[i] *= tile_unscale(i);
      bias = wave_sum_groups(bias);
      const uint8_t *vlo = page + g.off_v + V_CODE_BYTES, *vhi = vlo + 1024;
      if constexpr (FIFO) {
        const int vlim = fifo_vlim(A, pg);
        const float m0 = st.m;
        if (vlim >= PAGE) consume_values<G, NPASS>(st, logit, xs, bias * A.scale_log2, vc, VMetaAt{vlo, vhi}, a, col);
        else consume_values<G, NPASS, true>(st, logit, xs, bias * A.scale_log2, vc, VMetaAt{vlo, vhi}, a, col, vlim, hp);
        fifo_after<G, NPASS>(A, st, m0, head, pg, vlim, hp, ow, lane);
      } else {
        consume_values<G, NPASS>(st, logit, xs, bias * A.scale_log2, vc, VMetaAt{vlo, vhi}, a, col);
      }
    }
  } else {   // QJL
    // with the outlier split, k-steps NKI.. are the outlier instance: its
    // estimate is accumulated apart and added with its own norm and factor
    const QjlGeo g = qjl_geo(A.qjl_m, A.qjl_mo);
    const int NKS = (A.qjl_m + A.qjl_mo) / 32, NKI = A.qjl_m / 32;
    const float* sqrow = A.sq + ((int64_t)b * A.n_q_heads + hq) * (A.qjl_m + A.qjl_mo);
    float ssum = 0.f, ssum_o = 0.f;
    for (int k0 = 0; k0 < NKS; k0 += 4) {  // four k-steps' S q loads issued together
      float sqv[4][8];
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) sqv[j][e] = k0 + j < NKS ? sqrow[32 * (k0 + j) + 8 * a + e] : 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int ks = k0 + j;
        if (ks >= NKS) break;
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = sqv[j][e] * B_SCALE;
        half8 hi, lo;
        split8(x, hi, lo);
        if (col < G) {
          S.u.bq[0][ks][a][h] = hi;
          S.u.bq[1][ks][a][h] = lo;
        }
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) part += (float)hi[e] + (float)lo[e];
        if (ks < NKI) ssum += part;
        else ssum_o += part;
      }
    }
    ssum = wave_sum_groups(ssum);          // sum_i (S q)_i * 2^-6 as seen by the MFMA
    ssum_o = wave_sum_groups(ssum_o);
    const float ratio = A.qjl_mo ? (float)A.qjl_m / (float)A.qjl_mo : 0.f;   // the instances' sqrt(pi/2)/m factors
    __syncthreads();
    const float xs = A.scale_log2 * A.qjl_coef * B_UNSCALE;
    for (int pg = p0; pg < p1; ++pg) {
      const uint8_t* page = page_ptr(A, head, pg);
      u32x4 vc[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) vc[ks] = ld16(page + g.off_v + 1024 * ks + 256 * a + 16 * r);
      f32x4 logit[8], logit_o[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) logit[i] = logit_o[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
      auto sketch = [&](int P2b, int P2e, f32x4* acc) {
        for (int P2 = P2b; P2 < P2e; ++P2) {
          const u32x4 v = ld16(page + 1024 * P2 + 256 * a + 16 * r);
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            const int ks = 2 * P2 + hf;
            const half8 Bh = S.u.bq[0][ks][a][h], Bl = S.u.bq[1][ks][a][h];
            const Row1 x = row1(rd(v, 2 * hf), rd(v, 2 * hf + 1));
#pragma unroll
            for (int T = 0; T < 8; ++T) {
              const half8 At = tile1(x, T);
              acc[T] = mfma(At, Bh, acc[T]);
              acc[T] = mfma(At, Bl, acc[T]);
            }
          }
        }
      };
      sketch(0, NKI / 2, logit);
      sketch(NKI / 2, NKS / 2, logit_o);
      // estimator: nu_t * (2 <Sq, bits> - sum Sq); the norms of tokens 16 i + 4 a + e sit at 32 a + 4 i + e
      const uint8_t* nb = page + g.off_norm + 64 * a;
      const uint8_t* nbo = page + g.off_norm_o + 64 * a;
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const u32x4 nw = ld16(nb + 16 * qd);
        const u32x4 nwo = A.qjl_mo ? ld16(nbo + 16 * qd) : (u32x4){0u, 0u, 0u, 0u};
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
          const int i = 2 * qd + ii;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t w = rd(nw, 2 * ii + (e >> 1)), wo = rd(nwo, 2 * ii + (e >> 1));
            const uint16_t hb = (uint16_t)(w >> (16 * (e & 1))), hbo = (uint16_t)(wo >> (16 * (e & 1)));
            _Float16 hv, hvo;
            __builtin_memcpy(&hv, &hb, 2);
            __builtin_memcpy(&hvo, &hbo, 2);
            const float est_o = ratio * (float)hvo * fmaf(2.0f * tile_unscale(i), logit_o[i][e], -ssum_o);
            logit[i][e] = fmaf((float)hv, fmaf(2.0f * tile_unscale(i), logit[i][e], -ssum), est_o);
          }
        }
      }
      const uint8_t *vlo = page + g.off_v + V_CODE_BYTES, *vhi = vlo + 1024;
      if constexpr (FIFO) {
        const int vlim = fifo_vlim(A, pg);
        const float m0 = st.m;
        if (vlim >= PAGE) consume_values<G, NPASS>(st, logit, xs, 0.f, vc, VMetaAt{vlo, vhi}, a, col);
        else consume_values<G, NPASS, true>(st, logit, xs, 0.f, vc, VMetaAt{vlo, vhi}, a, col, vlim, hp);
        fifo_after<G, NPASS>(A, st, m0, head, pg, vlim, hp, ow, lane);
      } else {
        consume_values<G, NPASS>(st, logit, xs, 0.f, vc, VMetaAt{vlo, vhi}, a, col);
      }
    }
  }
  __syncthreads();
  write_partial<G, NPASS>(A, st, split, b, kvh, a, col, stage_buf(S), FIFO ? ow : nullptr);
}

// S q on the bf16 MFMA (QJL Algorithm 1 step 4, the projection of the query):
// sq[row][i] = sum_d S[i][d] q[row][d] for the query rows (batch, head) and
// the m + mo sketch rows, as a [rows x 128] x [128 x (m + mo)] product. A wave
// takes 16 query rows (the A operand: rows = query heads, k = channels) and
// QJL_PROJ_TILES tiles of 16 sketch rows (the B operand: k = channels,
// columns = sketch rows, read straight from S's rows). With the outlier split
// the rows below m see q's normal channels and the rest its outlier channels;
// m and mo are multiples of 64, so a tile belongs to one instance. Products
// of bf16 are exact and the sums are float, as in the scalar form. Every
// load (the query rows and all of the wave's sketch tiles) is issued before
// the first product, so a wave waits for memory once; a tile past m + mo
// reloads the last sketch row and stores nothing.
constexpr int QJL_PROJ_TILES = 4;
__global__ __launch_bounds__(64) void qjl_project_mfma(const uint16_t* q, const uint16_t* S, float* sq, int m, int mo,
                                                       const uint8_t* mask, int n_rows, int n_q_heads, int group) {
  const int lane = threadIdx.x, a = lane >> 4, r = lane & 15;
  const int row0 = blockIdx.x * 16;
  const int mt = m + mo;
  const int qrow = min(row0 + r, n_rows - 1);                 // A row r: query row row0 + r
  const int tile0 = blockIdx.y * QJL_PROJ_TILES;
  bf16x8 bs[QJL_PROJ_TILES][4];                                // B column r of each tile: sketch row
#pragma unroll
  for (int t = 0; t < QJL_PROJ_TILES; ++t) {
    const int srow = min(16 * (tile0 + t) + r, mt - 1);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      bs[t][ks] = as_bf16x8(ld16(reinterpret_cast<const uint8_t*>(S + (int64_t)srow * D + 32 * ks + 8 * a)));
  }
  bf16x8 an[4], ao[4];
  uint32_t obits = 0;                                          // outlier bits of channels 32 ks + 8 a + e
  if (mo > 0 && mask != nullptr) {
    const int b = qrow / n_q_heads, kvh = (qrow - b * n_q_heads) / group;
    const uint8_t* rec = mask + ((int64_t)b * (n_q_heads / group) + kvh) * QJL_RECORD;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) obits |= (uint32_t)rec[4 * ks + a] << (8 * ks);
  }
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const u32x4 raw = ld16(reinterpret_cast<const uint8_t*>(q + (int64_t)qrow * D + 32 * ks + 8 * a));
    uint16_t hv[8], nv[8], ov[8];
    __builtin_memcpy(hv, &raw, 16);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const bool out = (obits >> (8 * ks + e)) & 1;
      nv[e] = out ? (uint16_t)0 : hv[e];
      ov[e] = out ? hv[e] : (uint16_t)0;
    }
    __builtin_memcpy(&an[ks], nv, 16);
    __builtin_memcpy(&ao[ks], ov, 16);
  }
#pragma unroll
  for (int t = 0; t < QJL_PROJ_TILES; ++t) {
    const int tile = tile0 + t;
    if (16 * tile >= mt) break;                                // uniform
    const int srow = 16 * tile + r;
    const bool outlier = 16 * tile >= m;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) acc = mfma_bf(outlier ? ao[ks] : an[ks], bs[t][ks], acc);
#pragma unroll
    for (int e = 0; e < 4; ++e) {                              // D row 4 a + e: query row row0 + 4 a + e
      const int row = row0 + 4 * a + e;
      if (row < n_rows) sq[(int64_t)row * mt + srow] = acc[e];
    }
  }
}

// Split merge: one single-wave workgroup per query head (merge_row).
template <int NB>
__global__ __launch_bounds__(64) void combine_kernel(const float* partial, float* out, int n_parts, int rows) {
  merge_row<NB>(partial, out, n_parts, rows, blockIdx.x);
}

// The window of a Value-FIFO decode on the pipelined kernels, for its merge.
struct FifoMerge {
  int wsplit;                 // record of the first window page's logits
  int t_lo, n_tok;            // first window token in that page, window tokens inside the pages
  const uint16_t* vwin;
  int vwin_stride;
  int n_q_heads, n_kv_heads;
};

// Split merge plus the window tokens inside the pages (FifoWindow).
template <int NB>
__global__ __launch_bounds__(64) void combine_fifo_kernel(const float* partial, float* out, int n_parts, int rows,
                                                          FifoMerge f) {
  const int row = blockIdx.x;
  const int b = row / f.n_q_heads, hq = row - b * f.n_q_heads;
  const int64_t head = (int64_t)b * f.n_kv_heads + hq / (f.n_q_heads / f.n_kv_heads);
  FifoWindow w;
  w.logits = partial + ((int64_t)f.wsplit * rows + row) * RECORD;
  w.rec_stride = (int64_t)rows * RECORD;
  w.vrow0 = reinterpret_cast<const uint8_t*>(f.vwin + head * f.vwin_stride * D);
  w.t_lo = f.t_lo;
  w.n_tok = f.n_tok;
  merge_row<NB>(partial, out, n_parts, rows, row, w);
}

bool launch_decode_fast(int key_mode, DecodeArgs& a, hipStream_t s, bool fifo);

// Pages per split: the page splits of every (batch, kv head) are sized to
// fill `slots` resident workgroups in one round, with the pages spread
// evenly, but never fewer than MIN_PAGES_PER_SPLIT pages; the BF16-segment
// workgroups are dispatched after them (see decode_block). DECODE_SLOTS (256
// CUs x 8 resident single-wave workgroups on MI355X) bounds every kernel's
// split count, and the workspace is sized for it. The floor matters for short
// contexts: llama8b_8k's 64 pages per (batch, kv head) as 16 splits of 4
// pages (1024 split waves, the 256 segment workgroups resident beside them)
// measured 19.5 us per decode call against 20.3 us as 32 splits of 2 pages
// (every slot taken, the segment workgroups waiting for the splits); 3, 6 or
// 8 pages measured 21.4, 22.1 and 25.2 us. Longer contexts keep the
// two-waves-per-SIMD split count (qwen32b_32k: 16 splits of 16 pages, 82.5
// against 89.1 us as 8 of 32).
constexpr int MIN_PAGES_PER_SPLIT = 4;
int decode_pages_per_split_slots(int n_pages, int batch, int n_kv_heads, int slots) {
  const int64_t pairs = (int64_t)batch * n_kv_heads;
  const int64_t budget = slots;
  int64_t splits = budget / pairs;
  if (splits < 1) splits = 1;
  int64_t pps = (n_pages + splits - 1) / splits;
  if (pps < MIN_PAGES_PER_SPLIT) pps = MIN_PAGES_PER_SPLIT;
  return (int)pps;
}

int decode_pages_per_split(int n_pages, int batch, int n_kv_heads) {
  return decode_pages_per_split_slots(n_pages, batch, n_kv_heads, DECODE_SLOTS);
}

template <int MODE, bool FIFO>
static hipError_t launch_mode_f(const DecodeArgs& a, int g, dim3 grid, hipStream_t s) {
  const size_t dyn = FIFO ? (size_t)PAGE * 8 * sizeof(float) : 0;
  switch (g) {
    case 1: hipLaunchKernelGGL((decode_kernel<MODE, 1, FIFO>), grid, dim3(64), dyn, s, a); break;
    case 2: hipLaunchKernelGGL((decode_kernel<MODE, 2, FIFO>), grid, dim3(64), dyn, s, a); break;
    case 4: hipLaunchKernelGGL((decode_kernel<MODE, 4, FIFO>), grid, dim3(64), dyn, s, a); break;
    case 8: hipLaunchKernelGGL((decode_kernel<MODE, 8, FIFO>), grid, dim3(64), dyn, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
template <int MODE>
static hipError_t launch_mode(const DecodeArgs& a, int g, dim3 grid, hipStream_t s) {
  return a.vq_end != INT32_MAX ? launch_mode_f<MODE, true>(a, g, grid, s) : launch_mode_f<MODE, false>(a, g, grid, s);
}

int decode_parts(const DecodeArgs& a) { return a.n_page_splits + a.n_seg_splits; }

static hipError_t launch_generic(int key_mode, const DecodeArgs& a, int g, hipStream_t s) {
  const dim3 grid(decode_parts(a) * a.n_kv_heads * a.batch);
  if (key_mode == KVQ_KEY_MIXKVQ) return launch_mode<KVQ_KEY_MIXKVQ>(a, g, grid, s);
  if (key_mode == KVQ_KEY_PNMIX) return launch_mode<KVQ_KEY_PNMIX>(a, g, grid, s);
  return launch_mode<KVQ_KEY_QJL>(a, g, grid, s);
}

// KIVI Value FIFO on the pipelined kernels (KIVI blog sections 4-5): every
// page and the Key residual go to the FIFO variant of the pipelined kernel
// as an ordinary decode. The pages the full-precision Value window reaches
// into (from vq_end / 128 on; at most two, as the window holds at most 256
// tokens) keep their window tokens' Value rows as the Key seal left them
// (zero), so the split kernel adds nothing for those tokens but counts their
// probabilities; it leaves their logits in spare partial records (the last
// n_win records the workspace holds per query head), and the merge adds
// their window Values (combine_fifo_kernel). Returns false, having launched
// nothing, when no pipelined kernel covers the configuration; otherwise
// `win` is set when the merge has window tokens to add.
static bool launch_fifo_fast(int key_mode, DecodeArgs& a, hipStream_t s, FifoMerge& fm, bool& win, hipError_t& err) {
  const int n_clean = (int)min((int64_t)a.n_pages, (int64_t)a.vq_end / PAGE);
  const int n_win = a.n_pages - n_clean;
  const int cap = a.n_page_splits + MAX_SEG_SPLITS;   // records per query head in the workspace
  if (a.n_seg_splits + n_win > MAX_SEG_SPLITS) return false;   // spare records for the window pages
  a.fifo_clean = n_clean;
  a.fifo_wsplit = cap - n_win;
  if (!launch_decode_fast(key_mode, a, s, n_win > 0)) return false;
  err = hipGetLastError();
  win = n_win > 0;
  fm.wsplit = a.fifo_wsplit;
  fm.t_lo = a.vq_end - n_clean * PAGE;
  fm.n_tok = a.n_pages * PAGE - a.vq_end;
  fm.vwin = a.vwin;
  fm.vwin_stride = a.vwin_stride;
  fm.n_q_heads = a.n_q_heads;
  fm.n_kv_heads = a.n_kv_heads;
  return true;
}

hipError_t launch_decode(int key_mode, DecodeArgs& args, const uint16_t* qjl_s, hipStream_t s, bool with_merge,
                         int path) {
  DecodeArgs a = args;
  const bool generic = path == KVQ_DECODE_GENERIC;
  const int g = a.n_q_heads / a.n_kv_heads;
  const int n_parts = decode_parts(a);
  const int rows = a.batch * a.n_q_heads;
  FifoMerge fm{};
  bool win = false;   // the merge adds a Value-FIFO window (launch_fifo_fast)
  if (n_parts > 0) {
    if (key_mode == KVQ_KEY_QJL) {
      const int tiles = (a.qjl_m + a.qjl_mo) / 16;
      const dim3 pgrid((rows + 15) / 16, (tiles + QJL_PROJ_TILES - 1) / QJL_PROJ_TILES);
      hipLaunchKernelGGL(qjl_project_mfma, pgrid, dim3(64), 0, s, a.q, qjl_s, const_cast<float*>(a.sq), a.qjl_m,
                         a.qjl_mo, a.n_pages > 0 ? a.mask : nullptr, rows, a.n_q_heads, g);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    hipError_t e = hipSuccess;
    // The software-pipelined kernels cover the common shapes; the config's
    // decode path can ask for the generic kernel (same results within the
    // decode bound). (Merging the splits inside the split kernel, by
    // workgroups that wait for a slice's parts, measured slower than this
    // separate pass: the waits' device-scope polls slow the page stream, and
    // a store-acknowledge, count, poll, load chain costs about a launch.)
    bool done = false;
    if (!generic && a.vq_end != INT32_MAX) {   // the window is added by the merge below
      if (with_merge) done = launch_fifo_fast(key_mode, a, s, fm, win, e);
    } else if (!generic && launch_decode_fast(key_mode, a, s, false)) {
      done = true;
      e = hipGetLastError();
    }
    if (done) {
      args.pps = a.pps;   // the kernels' own split geometry, for the caller's merge
      args.n_page_splits = a.n_page_splits;
    } else {
      e = launch_generic(key_mode, a, g, s);
    }
    if (e != hipSuccess) return e;
  }
  if (!with_merge) return hipSuccess;
  // with nothing to attend to (no part) every output row is zero; a kernel
  // may have chosen its own split count (in a)
  const int parts = decode_parts(a);
  const dim3 cgrid(rows);
  if (win) {
    switch (merge_batch(parts)) {
      case 16: hipLaunchKernelGGL(combine_fifo_kernel<16>, cgrid, dim3(64), 0, s, a.partial, a.out, parts, rows, fm); break;
      case 32: hipLaunchKernelGGL(combine_fifo_kernel<32>, cgrid, dim3(64), 0, s, a.partial, a.out, parts, rows, fm); break;
      case 40: hipLaunchKernelGGL(combine_fifo_kernel<40>, cgrid, dim3(64), 0, s, a.partial, a.out, parts, rows, fm); break;
      case 48: hipLaunchKernelGGL(combine_fifo_kernel<48>, cgrid, dim3(64), 0, s, a.partial, a.out, parts, rows, fm); break;
      default: hipLaunchKernelGGL(combine_fifo_kernel<64>, cgrid, dim3(64), 0, s, a.partial, a.out, parts, rows, fm); break;
    }
    return hipGetLastError();
  }
  switch (merge_batch(parts)) {
    case 16: hipLaunchKernelGGL(combine_kernel<16>, cgrid, dim3(64), 0, s, a.partial, a.out, parts, rows); break;
    case 32: hipLaunchKernelGGL(combine_kernel<32>, cgrid, dim3(64), 0, s, a.partial, a.out, parts, rows); break;
    case 40: hipLaunchKernelGGL(combine_kernel<40>, cgrid, dim3(64), 0, s, a.partial, a.out, parts, rows); break;
    case 48: hipLaunchKernelGGL(combine_kernel<48>, cgrid, dim3(64), 0, s, a.partial, a.out, parts, rows); break;
    default: hipLaunchKernelGGL(combine_kernel<64>, cgrid, dim3(64), 0, s, a.partial, a.out, parts, rows); break;
  }
  return hipGetLastError();
}

}  // namespace kvq
