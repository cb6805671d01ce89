// Flush kernels: quantize and pack full 128-token segments into pages.
//
// MixKVQ Algorithm 1 (KeyQuant / GroupQuant at a buffer flush) with the
// KIVI blog grouping axes: Keys per channel over the 128 tokens of the page,
// Values per token over groups of 32 channels. PN-Mix Eq.2/Eq.7 and
// Appendix G planes. QJL Algorithm 1 steps 2-3 (sign(S k) and ||k||).
//
// Several workgroups of 256 threads write one (page, kv head, batch): one per
// value k-step and one per Key part (see "Work split" below). Each stages its
// tokens in LDS, reduces every group's min / max (wave reductions), then
// every thread produces one 32-bit word of packed output, so consecutive
// threads store consecutive words.
//
// Exactness. Codes are round-half-even of the exact (2^b-1)(x-m)/(M-m): an
// estimate from a reciprocal is corrected by comparing 2(2^b-1)(x-m) with
// (2c+-1)(M-m) in double precision, exact while a group spans at most 38
// binades (checked; KVQ_FLAG_SPAN otherwise). Scales and offsets are the
// binary16 nearest to the exact values (one rounding from a double that is
// either exact or correctly rounded and never a binary16 midpoint); values
// beyond the binary16 range are stored as infinity with KVQ_FLAG_RANGE.
#include "kvq_internal.h"
#include "kvq_merge.h"
#include "kvq_rank.h"

namespace kvq {


// 16 bytes per group; M - m is recomputed exactly in double from m and M.
struct GroupParam {
  float m;         // group minimum (exact bf16 value)
  float M;         // group maximum
  float inv;       // levels / (M - m) (2 / (M - m) for a midpoint group); NaN sends every code to the exact path
  uint16_t scale;  // stored binary16 scale
  uint16_t offset; // stored binary16 offset
};

// A group's finite minimum and maximum, the smallest nonzero magnitude and
// whether a non-finite value occurred. The exponent span the exact code path
// needs follows from them: the largest exponent field is that of
// max(|mn|, |mx|), the smallest that of the smallest nonzero magnitude
// (subnormals count as field 1).
struct Scan {
  float mn, mx;      // over finite values
  uint32_t am1;      // min over the values of (|bits| - 1) mod 2^16: 0xFFFF with no nonzero value,
                     // >= 0x7F7F with no finite nonzero value
  bool nonfinite;
};

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Scan of N words, each two bf16 values (low half first). The fast pass is
// two values per step: three-operand float min / max over both halves and
// 16-bit packed integer min / max of the magnitude bits; a word with a
// non-finite value only marks the group, whose minimum and maximum are then
// taken again over the finite values alone.
template <int N>
__device__ inline Scan scan_words(const uint32_t (&w)[N]) {
  float mn = INFINITY, mx = -INFINITY;
  u16x2 am1 = {0xFFFF, 0xFFFF}, amax = {0, 0};
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const u16x2 a = __builtin_bit_cast(u16x2, w[i] & 0x7FFF7FFFu);
    am1 = __builtin_elementwise_min(am1, a - (u16x2){1, 1});   // zero wraps to 0xFFFF
    amax = __builtin_elementwise_max(amax, a);
    const float lo = __uint_as_float(w[i] << 16), hi = __uint_as_float(w[i] & 0xFFFF0000u);
    mn = fminf(mn, fminf(lo, hi));
    mx = fmaxf(mx, fmaxf(lo, hi));
  }
  Scan s;
  s.am1 = min((uint32_t)am1.x, (uint32_t)am1.y);
  s.nonfinite = max(amax.x, amax.y) >= 0x7F80;
  if (s.nonfinite) {   // rare: minimum and maximum over the finite values
    mn = INFINITY;
    mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 2 * N; ++i) {
      const uint32_t b = (w[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
      const bool fin = (b & 0x7FFF) < 0x7F80;
      const float v = __uint_as_float(b << 16);
      mn = fminf(mn, fin ? v : INFINITY);
      mx = fmaxf(mx, fin ? v : -INFINITY);
    }
  }
  s.mn = mn;
  s.mx = mx;
  return s;
}

// Exponent span of the group's nonzero finite values beyond 38 binades.
__device__ inline bool scan_span(const Scan& s) {
  if (s.am1 >= 0x7F7Fu) return false;   // no nonzero finite value
  const int emin = max((int)((s.am1 + 1) >> 7), 1);
  const int emax = (int)((__float_as_uint(fmaxf(fabsf(s.mn), fabsf(s.mx))) >> 23) & 0xFF);
  return emax - emin > 38;
}

// Merge with a partner lane through a DPP lane move (one VALU instruction,
// no LDS round trip). Applied for W = 1, 2, 4 in turn it reduces over 2, 4 or
// 8 consecutive lanes: the xor-1 and xor-2 quad permutations, then the
// half-row mirror (lane i with 7 - i of its 8), which pairs each lane with
// the other quad.
template <int W>
__device__ inline int dpp_partner(int v) {
  constexpr int ctrl = W == 1 ? 0xB1 : (W == 2 ? 0x4E : 0x141);   // quad_perm [1,0,3,2], [2,3,0,1]; row_half_mirror
  static_assert(W == 1 || W == 2 || W == 4, "lane distance");
  return __builtin_amdgcn_update_dpp(0, v, ctrl, 0xF, 0xF, false);
}
template <int W>
__device__ inline void scan_merge(Scan& s) {
  s.mn = fminf(s.mn, __int_as_float(dpp_partner<W>(__float_as_int(s.mn))));
  s.mx = fmaxf(s.mx, __int_as_float(dpp_partner<W>(__float_as_int(s.mx))));
  s.am1 = min(s.am1, (uint32_t)dpp_partner<W>((int)s.am1));
  // not `||`: a short circuit would run the lane move only in the lanes
  // without a non-finite value, and a DPP move reads nothing from lanes that
  // are switched off, so the partner's flag would be lost
  const int partner_nonfinite = dpp_partner<W>((int)s.nonfinite);
  s.nonfinite = s.nonfinite | (partner_nonfinite != 0);
}

__device__ inline bool f16_is_inf(uint16_t h) { return (h & 0x7FFF) == 0x7C00; }

// the status bits a group raises, OR-ed into *flags with one atomic
__device__ inline void raise_flags(const Scan& s, const GroupParam& p, unsigned* flags) {
  const unsigned f = (s.nonfinite ? KVQ_FLAG_NONFINITE : 0u) | (scan_span(s) ? KVQ_FLAG_SPAN : 0u) |
                     (f16_is_inf(p.scale) || f16_is_inf(p.offset) ? KVQ_FLAG_RANGE : 0u);
  if (f && flags) atomicOr(flags, f);
}

// min-max quantizer parameters for `levels` = 2^b - 1
__device__ inline GroupParam make_param(const Scan& s, int levels, unsigned* flags) {
  GroupParam p;
  p.m = s.mn;
  p.M = s.mn;
  p.offset = s.mn == INFINITY ? (uint16_t)0 : f64_to_f16_rne((double)s.mn);
  p.inv = 0.0f;
  p.scale = 0;
  if (s.mx > s.mn) {
    p.M = s.mx;
    const double den = (double)s.mx - (double)s.mn;
    p.inv = (float)((double)levels / den);
    if (!(p.inv >= 0x1.0p-126f && p.inv <= 0x1.0p126f)) p.inv = NAN;   // outside the fast path's bound
    p.scale = f64_to_f16_rne(den / (double)levels);
  }
  raise_flags(s, p, flags);
  return p;
}

// PN-Mix Eq.7 parameters: s = (M-m)/2, z = (3m+M)/4; code = 2(x-m) > M-m
__device__ inline GroupParam make_param_mid(const Scan& s, unsigned* flags) {
  GroupParam p;
  p.m = s.mn;
  p.M = s.mn;
  p.inv = 0.0f;
  p.scale = 0;
  p.offset = s.mn == INFINITY ? (uint16_t)0 : f64_to_f16_rne((double)s.mn);
  if (s.mx > s.mn) {
    p.M = s.mx;
    const double den = (double)s.mx - (double)s.mn;
    p.inv = (float)(2.0 / den);
    if (!(p.inv >= 0x1.0p-126f && p.inv <= 0x1.0p126f)) p.inv = NAN;
    p.scale = f64_to_f16_rne(0.5 * den);
    p.offset = f64_to_f16_rne(0.25 * (3.0 * (double)s.mn + (double)s.mx));
  }
  raise_flags(s, p, flags);
  return p;
}

// Exact round-half-even code of x for levels = 2^b - 1. The double estimate
// is within one of the true code; the fix-up compares 2*levels*(x-m) with
// (2c -+ 1)(M-m), all exact in double for groups spanning <= 38 binades.
__device__ inline int quant_code_exact(const GroupParam& p, int levels, float x) {
  if (!(p.M > p.m)) return 0;
  double den = (double)p.M - (double)p.m;
  double two_num = 2.0 * (double)levels * ((double)x - (double)p.m);
  int c = (int)rint(0.5 * two_num / den);   // within one of the exact code
  c = max(0, min(levels, c));
  if (c > 0) {
    double lo = (double)(2 * c - 1) * den;
    if (two_num < lo || (two_num == lo && (c & 1))) return c - 1;   // tie -> even c-1
  }
  if (c < levels) {
    double hi = (double)(2 * c + 1) * den;
    if (two_num > hi || (two_num == hi && (c & 1))) return c + 1;   // tie -> even c+1
  }
  return c;
}

// Fast path: t = (x - m) * levels / (M - m) in float is within 4 ulp of the
// exact quotient (x - m and levels / (M - m) each rounded once, then the
// product), i.e. within 2^-20 for t <= 15. If t is farther than 0.5 - 2^-14
// from a half-integer boundary its nearest integer is the exact code;
// otherwise (ties and near-ties) the double-precision path decides. A
// constant group has inv = 0, so t = 0.
__device__ inline int quant_code(const GroupParam& p, int levels, float x) {
  const float t = (x - p.m) * p.inv;
  const float c = rintf(t);
  if (fabsf(t - c) < 0.49993896f) return (int)c;
  return quant_code_exact(p, levels, x);
}

// The fast path on its own, for straight-line loops: `amb` collects the
// codes that the exact path has to redo.
__device__ inline int fast_code(float m, float inv, float x, bool& amb) {
  const float t = (x - m) * inv;
  const float c = rintf(t);
  amb = !(fabsf(t - c) < 0.49993896f);
  return (int)c;
}

// PN-Mix Eq.7 code: 1 iff 2(x - m) > M - m (the exact midpoint rounds to 0).
// inv = 2 / (M - m) here; the double comparison settles t within 2^-14 of 1.
__device__ inline int mid_code(const GroupParam& p, float x) {
  if (!(p.M > p.m)) return 0;
  const float t = (x - p.m) * p.inv;
  if (fabsf(t - 1.0f) > 0x1.0p-14f) return t > 1.0f ? 1 : 0;
  return 2.0 * ((double)x - (double)p.m) > ((double)p.M - (double)p.m) ? 1 : 0;
}

__device__ inline void store16(uint8_t* dst, uint4 v) { *reinterpret_cast<uint4*>(dst) = v; }

__device__ inline void store4(uint8_t* dst, uint32_t v) { *reinterpret_cast<uint32_t*>(dst) = v; }

// rows row0 .. row0 + NROWS - 1 of a [*, 128] bf16 source into LDS, by the
// 256 threads of the workgroup: every load is issued before the first LDS
// store, so the staging costs one memory latency.
template <int NROWS>
__device__ inline void stage_rows(uint16_t* lds, const uint16_t* src, int64_t row0) {
  constexpr int N = NROWS * D / 8 / 256;
  static_assert(N * 256 * 8 == NROWS * D, "whole 16-byte chunks per thread");
  const uint4* s = reinterpret_cast<const uint4*>(src + row0 * D);
  uint4* d = reinterpret_cast<uint4*>(lds);
  uint4 v[N];
#pragma unroll
  for (int j = 0; j < N; ++j) v[j] = s[threadIdx.x + 256 * j];
#pragma unroll
  for (int j = 0; j < N; ++j) d[threadIdx.x + 256 * j] = v[j];
}

__device__ inline uint4 pack8(const uint16_t* v) {
  return make_uint4(v[0] | ((uint32_t)v[1] << 16), v[2] | ((uint32_t)v[3] << 16), v[4] | ((uint32_t)v[5] << 16),
                    v[6] | ((uint32_t)v[7] << 16));
}

// Work split. A page is written by several workgroups of 256 threads: one
// per value k-step (32 tokens, V_PARTS of them) and one or more Key parts.
// Every thread produces one 32-bit word of packed output, so a page takes
// a few microseconds of latency rather than a long serial loop.
constexpr int V_PARTS = 4;

// ------------------------------------------------------------------ values
struct VPartSmem {
  uint16_t tile[32 * D];        // the k-step's 32 tokens
  GroupParam vp[32 * 4];        // their per-token group parameters
};

// Value k-step s of a page (tokens 32 s .. 32 s + 31, per-token groups of 32
// channels): code units (a, r) of the code region and the k-step's 512
// bytes of scales / offsets.
__device__ __attribute__((always_inline)) inline void flush_value_part(uint8_t* page_v, const uint16_t* v_src, int64_t row0, int s,
                                        unsigned* flags, VPartSmem& S) {
  stage_rows<32>(S.tile, v_src, row0 + 32 * s);
  __syncthreads();
  {  // 128 groups, two threads each
    const int gi = threadIdx.x >> 1, half = threadIdx.x & 1, tl = gi >> 2, j = gi & 3;
    const uint4* src = reinterpret_cast<const uint4*>(S.tile + tl * D + GV * j + 16 * half);
    const uint4 c0 = src[0], c1 = src[1];
    const uint32_t cw[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
    Scan sc = scan_words(cw);
    scan_merge<1>(sc);
    if (half == 0) S.vp[gi] = make_param(sc, 3, flags);
  }
  __syncthreads();
  {  // code unit (a, r), word w: every V-tile u (channel 16 u + r) of the two tokens pi(s, a, 2w + hh);
     // the code of (u, hh) sits at bits 2 u + 16 hh
    const int t = threadIdx.x, a = t >> 6, r = (t >> 2) & 15, w = t & 3;
    float m[2][4], inv[2][4], x[16];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int k = 2 * w + hh, tl = 16 * (k >> 2) + 4 * a + (k & 3);   // pi(s, a, k) - 32 s
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        m[hh][j] = S.vp[tl * 4 + j].m;
        inv[hh][j] = S.vp[tl * 4 + j].inv;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) x[8 * hh + u] = bf16_to_f32(S.tile[tl * D + 16 * u + r]);
    }
    uint32_t word = 0, redo = 0;
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      const int u = p & 7, hh = p >> 3;
      bool amb;
      // cut to the code's field: an infinite input (t infinite, redone below)
      // converts to a full-width integer that would reach the other codes
      word |= ((uint32_t)fast_code(m[hh][u >> 1], inv[hh][u >> 1], x[p], amb) & 3u) << (2 * p);
      redo |= (uint32_t)amb << p;
    }
    while (redo) {   // the few codes within 2^-14 of a rounding midpoint, one by one
      const int p = __builtin_ctz(redo);
      redo &= redo - 1;
      const int u = p & 7, k = 2 * w + (p >> 3);
      const int tl = 16 * (k >> 2) + 4 * a + (k & 3);
      const uint32_t c = quant_code_exact(S.vp[tl * 4 + (u >> 1)], 3, bf16_to_f32(S.tile[tl * D + 16 * u + r]));
      word = (word & ~(3u << (2 * p))) | c << (2 * p);
    }
    store4(page_v + 1024 * s + 256 * a + 16 * r + 4 * w, word);
  }
  if (threadIdx.x < 128) {  // meta unit (a, j, half), dword w: tokens pi(s, a, 2w) and pi(s, a, 2w + 1)
    const int t = threadIdx.x, a = t >> 5, j = (t >> 3) & 3, half = (t >> 2) & 1, w = t & 3;
    const int t0 = 16 * ((2 * w) >> 2) + 4 * a + ((2 * w) & 3);
    const int t1 = 16 * ((2 * w + 1) >> 2) + 4 * a + ((2 * w + 1) & 3);
    const GroupParam& p0 = S.vp[t0 * 4 + j];
    const GroupParam& p1 = S.vp[t1 * 4 + j];
    const uint16_t lo = half ? p0.offset : p0.scale, hi = half ? p1.offset : p1.scale;
    store4(page_v + V_CODE_BYTES + 512 * s + 128 * a + 32 * j + 16 * half + 4 * w, (uint32_t)lo | ((uint32_t)hi << 16));
  }
}

// KIVI Value FIFO seal (KIVI blog section 4): the Keys of a full residual are
// quantized into the page and its value k-step s is cleared (codes, scales,
// offsets all zero); each token's Value row is ORed in later by the value
// push, when it leaves the full-precision window.
__device__ inline void zero_value_part(uint8_t* page_v, int s) {
  store4(page_v + 1024 * s + 4 * threadIdx.x, 0u);
  if (threadIdx.x < 128) store4(page_v + V_CODE_BYTES + 512 * s + 4 * threadIdx.x, 0u);
}

// Key tiles are read down columns (one channel over many tokens); rows of
// 130 elements (65 dwords) put the 64 rows a wave reads in 64 different banks.
constexpr int KS = D + 2;

// rows row0 .. row0 + PAGE - 1 into an LDS tile with row stride KS (dword stores)
__device__ inline void stage_rows_padded(uint16_t* lds, const uint16_t* src, int64_t row0) {
  constexpr int N = PAGE * D / 8 / 256;
  const uint4* s = reinterpret_cast<const uint4*>(src + row0 * D);
  uint4 v[N];
#pragma unroll
  for (int j = 0; j < N; ++j) v[j] = s[threadIdx.x + 256 * j];
#pragma unroll
  for (int j = 0; j < N; ++j) {
    const int i = threadIdx.x + 256 * j, row = i >> 4, c = i & 15;
    uint32_t* d = reinterpret_cast<uint32_t*>(lds + row * KS + 8 * c);
    d[0] = v[j].x;
    d[1] = v[j].y;
    d[2] = v[j].z;
    d[3] = v[j].w;
  }
}

struct KPartSmem {
  uint16_t tile[PAGE * KS];     // the page's Keys, row stride KS
  double key_hi[D], key_lo[D];  // per-flush reselection: the channels' rank keys
  uint8_t tier[D];
  GroupParam kp[D];             // Key group parameters (by slot or channel position)
  uint8_t ch[D];                // channel order (MixKVQ) / slot -> channel (PN-Mix)
  int kinfo[32];                // MixKVQ slot of the part: channel | shift << 8 | mask << 10 | param << 12 | u4 << 20
};

// ------------------------------------------------------------------ MixKVQ keys
// Slot -> channel position (into the record's channel order), its levels and
// whether it owns the channel's parameters (the low half of a UINT4 code).
__device__ inline int mix_slot_pos(const MixGeo& g, int slot, int& levels, bool& primary) {
  if (slot < 2 * g.n4) {
    levels = 15;
    primary = !(slot & 1);
    return g.n16 + (slot >> 1);
  }
  if (slot >= g.s4 && slot < g.s4 + g.n2) {
    levels = 3;
    primary = true;
    return g.n16 + g.n4 + (slot - g.s4);
  }
  return -1;
}

// Key part fg: fragments 4 fg .. 4 fg + 3 (codes and scales / offsets); part
// 0 also writes the BF16-tier rows.
// Per-flush reselection of one page (MixKVQ: I_d from the running
// accumulator of query magnitudes, S_d from the page's own Keys; tiers
// refreshed at each flush): rank keys SQ_d * range_d exactly as the prefill
// selection, tiers by rank, the channel order into S.ch; `write` also stores
// the page's record (order, then 2-bit tiers). Keys must be finite.
__device__ inline void reselect_page(const FlushArgs& A, int64_t head, int lpage, bool write, KPartSmem& S) {
  const int d = threadIdx.x >> 1, half = threadIdx.x & 1;   // two threads per channel, 64 tokens each
  float mn = INFINITY, mx = -INFINITY;
#pragma unroll 16
  for (int t = 64 * half; t < 64 * half + 64; ++t) {
    const float v = bf16_to_f32(S.tile[t * KS + d]);
    mn = fminf(mn, v);
    mx = fmaxf(mx, v);
  }
  mn = fminf(mn, __int_as_float(dpp_partner<1>(__float_as_int(mn))));
  mx = fmaxf(mx, __int_as_float(dpp_partner<1>(__float_as_int(mx))));
  if (half == 0) {
    const u128 sq = reinterpret_cast<const u128*>(A.q_accum)[head * D + d];
    dd_key(sq, (double)mx - (double)mn, S.key_hi[d], S.key_lo[d]);
  }
  __syncthreads();
  {  // rank of channel d: both of its threads count half of the other channels
    const double kh = S.key_hi[d], kl = S.key_lo[d];
    int r = 0;
#pragma unroll 16
    for (int o = 64 * half; o < 64 * half + 64; ++o) {
      const double oh = S.key_hi[o], ol = S.key_lo[o];
      r += (oh > kh || (oh == kh && (ol > kl || (ol == kl && o < d)))) ? 1 : 0;
    }
    r += dpp_partner<1>(r);
    if (half == 0) S.tier[d] = r < A.n16 ? 2 : (r < A.n16 + A.n4 ? 1 : 0);
  }
  __syncthreads();
  uint8_t* rec = A.rec_out + (head * A.rec_stride + lpage) * MIX_RECORD;
  if (threadIdx.x < D) {
    // position in the channel order: the tier's base plus the lower channels
    // of the same tier, counted four tier bytes at a time
    const int c = threadIdx.x, t = S.tier[c];
    const uint32_t pat = 0x01010101u * (uint32_t)t;
    const uint32_t* tw = reinterpret_cast<const uint32_t*>(S.tier);
    int pos = t == 2 ? 0 : (t == 1 ? A.n16 : A.n16 + A.n4);
    for (int q = 0; q < (c >> 2); ++q) {
      const uint32_t x = tw[q] ^ pat;   // tier bytes use bits 0-1: a zero byte is the same tier
      pos += 4 - __builtin_popcount((x | (x >> 1)) & 0x01010101u);
    }
    for (int o = c & ~3; o < c; ++o) pos += S.tier[o] == t;
    S.ch[pos] = (uint8_t)c;
    if (write) rec[pos] = (uint8_t)c;
  } else if (write && threadIdx.x < D + 32) {
    const int q = threadIdx.x - D;
    rec[D + q] = (uint8_t)(S.tier[4 * q] | (S.tier[4 * q + 1] << 2) | (S.tier[4 * q + 2] << 4) | (S.tier[4 * q + 3] << 6));
  }
  __syncthreads();
}

__device__ __attribute__((always_inline)) inline void flush_mix_key_part(const FlushArgs& A, uint8_t* page, int64_t head, int64_t row0, int fg,
                                          int lpage, KPartSmem& S) {
  int hn16 = A.n16, hn4 = A.n4;
  if (A.head_tiers) mix_record_counts(A.mask + head * MIX_RECORD, hn16, hn4);   // threshold tiers: the head's counts
  const MixGeo g = mix_geo(hn16, hn4);
  const bool resel = A.q_accum != nullptr;
  const uint8_t chv = resel ? (uint8_t)0 : A.mask[head * MIX_RECORD + (threadIdx.x & (D - 1))];   // in flight with the staging
  stage_rows_padded(S.tile, A.k_src, row0);
  if (!resel && threadIdx.x < D) S.ch[threadIdx.x] = chv;
  __syncthreads();
  if (resel) reselect_page(A, head, lpage, fg == 0, S);
  {  // parameters of the group's 32 slots, eight threads per slot (16 tokens each)
    const int ls = threadIdx.x >> 3, part = threadIdx.x & 7;
    int levels = 0;
    bool primary = false;
    const int pos = mix_slot_pos(g, 32 * fg + ls, levels, primary);
    uint32_t cw[8];
    const int dd = pos >= 0 ? S.ch[pos] : 0;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      cw[i] = (uint32_t)S.tile[(16 * part + 2 * i) * KS + dd] | ((uint32_t)S.tile[(16 * part + 2 * i + 1) * KS + dd] << 16);
    Scan sc = scan_words(cw);
    if (!(pos >= 0 && primary)) sc = Scan{INFINITY, -INFINITY, 0xFFFFu, false};   // no parameters of its own
    scan_merge<1>(sc);
    scan_merge<2>(sc);
    scan_merge<4>(sc);
    if (part == 0 && pos >= 0 && primary) S.kp[ls] = make_param(sc, levels, A.flags);
    if (part == 0 && pos < 0) S.kp[ls] = GroupParam{0.f, 0.f, 0.f, 0, 0};   // empty slot: code 0
    if (part == 1) {
      const bool u4 = levels == 15;
      const int d = pos >= 0 ? S.ch[pos] : 0;
      const int shift = u4 && !primary ? 2 : 0;           // high half of a UINT4 code
      const int mask = pos >= 0 ? 3 : 0;
      const int pidx = u4 ? (ls & ~1) : ls;               // the UINT4 pair's parameters sit at its even slot
      S.kinfo[ls] = d | shift << 8 | mask << 10 | pidx << 12 | (int)u4 << 20;
    }
  }
  __syncthreads();
  {  // code fragment f, token row r, word w: slots 8f + 2w + hh of every tile u (token 16 u + r);
     // the code of (u, hh) sits at bits 2 u + 16 hh
    const int t = threadIdx.x, f = 4 * fg + (t >> 6), r = (t >> 2) & 15, w = t & 3;
    if (f < g.F) {
      int info[2];
      float m[2], inv[2], x[16];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        info[hh] = S.kinfo[8 * (t >> 6) + 2 * w + hh];
        const GroupParam& q = S.kp[(info[hh] >> 12) & 255];
        m[hh] = q.m;
        inv[hh] = q.inv;
#pragma unroll
        for (int u = 0; u < 8; ++u) x[8 * hh + u] = bf16_to_f32(S.tile[(16 * u + r) * KS + (info[hh] & 255)]);
      }
      uint32_t word = 0, redo = 0;
#pragma unroll
      for (int pp = 0; pp < 16; ++pp) {
        const int hh = pp >> 3;
        bool amb;
        const int full = fast_code(m[hh], inv[hh], x[pp], amb);
        word |= (uint32_t)((full >> ((info[hh] >> 8) & 3)) & ((info[hh] >> 10) & 3)) << (2 * pp);
        redo |= (uint32_t)amb << pp;
      }
      while (redo) {   // the few codes within 2^-14 of a rounding midpoint, one by one
        const int pp = __builtin_ctz(redo);
        redo &= redo - 1;
        const int in = S.kinfo[8 * (t >> 6) + 2 * w + (pp >> 3)];
        const int tok = 16 * (pp & 7) + r;
        const float xv = bf16_to_f32(S.tile[tok * KS + (in & 255)]);
        const int full = quant_code_exact(S.kp[(in >> 12) & 255], (in >> 20) ? 15 : 3, xv);
        const uint32_t c = (uint32_t)((full >> ((in >> 8) & 3)) & ((in >> 10) & 3));
        word = (word & ~(3u << (2 * pp))) | c << (2 * pp);
      }
      store4(page + g.off_codes + 256 * f + 16 * r + 4 * w, word);
    }
  }
  if (threadIdx.x < 32) {  // scales (half 0) / offsets (half 1) of fragment f, dword w: slots 8f + 2w, 8f + 2w + 1
    const int t = threadIdx.x, f = 4 * fg + (t >> 3), half = (t >> 2) & 1, w = t & 3;
    if (f < g.F) {
      uint16_t v[2];
      for (int k = 0; k < 2; ++k) {
        const int slot = 8 * f + 2 * w + k;
        int levels = 0;
        bool primary = false;
        const int pos = mix_slot_pos(g, slot, levels, primary);
        uint16_t sc = 0, of = 0;
        if (pos >= 0) {
          const GroupParam& q = S.kp[(slot - 32 * fg) & (levels == 15 ? ~1 : ~0)];
          if (levels == 15 && (slot & 1)) {   // high half of a UINT4 code: 4 s, no offset
            sc = q.scale == 0 ? 0 : f64_to_f16_rne(4.0 * f16_to_f64(q.scale));
            if (f16_is_inf(sc) && !half) atomicOr(A.flags, KVQ_FLAG_RANGE);
          } else {
            sc = q.scale;
            of = q.offset;
          }
        }
        v[k] = half ? of : sc;
      }
      store4(page + g.off_meta + 32 * f + 16 * half + 4 * w, (uint32_t)v[0] | ((uint32_t)v[1] << 16));
    }
  }
  if (fg == 0) {  // BF16 tier: channel row c, token row r, 8 tiles
    bool bad = false;
    for (int u = threadIdx.x; u < 16 * g.n16; u += blockDim.x) {
      const int c = u >> 4, r = u & 15, d = S.ch[c];
      uint16_t v[8];
      for (int i = 0; i < 8; ++i) {
        v[i] = S.tile[(16 * i + r) * KS + d];
        bad = bad || bf16_exp_field(v[i]) == 0xFF;
      }
      store16(page + 256 * c + 16 * r, pack8(v));
    }
    if (bad) atomicOr(A.flags, KVQ_FLAG_NONFINITE);
  }
}

// ------------------------------------------------------------------ PN-Mix keys
// Key part 0: LSB plane; part 1: upper-2-bit plane and slot scales / offsets.
__device__ __attribute__((always_inline)) inline void flush_pn_key_part(const FlushArgs& A, uint8_t* page, int64_t head, int64_t row0, int part,
                                         KPartSmem& S) {
  const PnGeo g = pn_geo(A.n_hi);
  const uint8_t* rec = A.mask + head * PN_RECORD;   // bit p of the 8 bytes: pair p is high
  uint64_t pm = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) pm |= (uint64_t)rec[i] << (8 * i);
  stage_rows_padded(S.tile, A.k_src, row0);
  const int np_hi = __builtin_popcountll(pm);
  const int nhs = 2 * np_hi;                         // high channels
  if (threadIdx.x < D) {   // slot order: high channels ascending, then low ones
    const int d = threadIdx.x;
    const bool halfsplit = A.pair_layout == KVQ_PAIR_HALF_SPLIT;
    const int pair = halfsplit ? (d & 63) : (d >> 1);
    const bool hi = (pm >> pair) & 1;
    const int cnt = __builtin_popcountll(pair == 0 ? 0ull : (pm & ((1ull << pair) - 1)));
    const int below = hi ? cnt : pair - cnt;         // channels of d's class with a lower pair
    const int before = halfsplit ? below + (d >= 64 ? (hi ? np_hi : 64 - np_hi) : 0) : 2 * below + (d & 1);
    S.ch[hi ? before : nhs + before] = (uint8_t)d;
  }
  if (threadIdx.x == 0 && nhs != A.n_hi) atomicOr(A.flags, KVQ_FLAG_MASK);
  __syncthreads();
  const int n_hi = min(nhs, A.n_hi);
  {
    const int slot = threadIdx.x >> 1, half = threadIdx.x & 1;
    const int d = S.ch[slot];
    uint32_t cw[32];
#pragma unroll
    for (int i = 0; i < 32; ++i)
      cw[i] = (uint32_t)S.tile[(half * 64 + 2 * i) * KS + d] | ((uint32_t)S.tile[(half * 64 + 2 * i + 1) * KS + d] << 16);
    Scan sc = scan_words(cw);
    scan_merge<1>(sc);
    if (half == 0) S.kp[slot] = slot < nhs ? make_param(sc, 7, A.flags) : make_param_mid(sc, A.flags);
  }
  __syncthreads();
  if (part == 0) {   // LSB plane: 128 units (pair P, lane group a, row r) x 4 words
    for (int wi = threadIdx.x; wi < 512; wi += blockDim.x) {
      const int u = wi >> 2, wq = wi & 3;
      const int P = u >> 6, a = (u >> 4) & 3, r = u & 15, half = wq >> 1, q = wq & 1;
      const int f = 4 * (2 * P + half) + a;
      uint32_t word = 0;
      for (int bit = 0; bit < 32; ++bit) {   // tile T, element 4 z + 2 q + h at bit 16 h + 8 (T / 4) + 2 (T % 4) + z
        const int slot = 8 * f + 4 * (bit & 1) + 2 * q + (bit >> 4);
        const int t = 16 * (4 * ((bit >> 3) & 1) + ((bit >> 1) & 3)) + r;
        const float x = bf16_to_f32(S.tile[t * KS + S.ch[slot]]);
        const int code = slot < nhs ? quant_code(S.kp[slot], 7, x) : mid_code(S.kp[slot], x);
        word |= (uint32_t)(code & 1) << bit;
      }
      store4(page + 1024 * P + 256 * a + 16 * r + 4 * wq, word);
    }
  } else {           // upper plane units (fragment f, row r) x 4 words, then 32 meta units x 4 dwords
    const int n_up = 16 * g.n_up_frag * 4;
    for (int wi = threadIdx.x; wi < n_up + 128; wi += blockDim.x) {
      if (wi < n_up) {
        const int f = wi >> 6, r = (wi >> 2) & 15, w = wi & 3;
        uint32_t word = 0;
        for (int pp = 0; pp < 16; ++pp) {   // tile pp & 7, element 2 w + pp / 8 at bits 2 pp
          const int t = 16 * (pp & 7) + r;
          const int slot = 8 * f + 2 * w + (pp >> 3);
          int code = 0;
          if (slot < n_hi) code = quant_code(S.kp[slot], 7, bf16_to_f32(S.tile[t * KS + S.ch[slot]])) >> 1;
          word |= (uint32_t)code << (2 * pp);
        }
        store4(page + g.off_up + 256 * f + 16 * r + 4 * w, word);
      } else {
        const int m = wi - n_up, f = m >> 3, half = (m >> 2) & 1, w = m & 3;
        const GroupParam& p0 = S.kp[8 * f + 2 * w];
        const GroupParam& p1 = S.kp[8 * f + 2 * w + 1];
        const uint16_t lo = half ? p0.offset : p0.scale, hi = half ? p1.offset : p1.scale;
        store4(page + g.off_meta + 32 * f + 16 * half + 4 * w, (uint32_t)lo | ((uint32_t)hi << 16));
      }
    }
  }
}

// ------------------------------------------------------------------ QJL keys
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

struct QPartSmem {
  uint16_t tile[PAGE * D];
  uint16_t srow[64 * D];        // the part's 64 sketch rows of S
  union {
    uint32_t bits[64 * 4];      // the part's 64 sketch rows x 128 tokens (bit t of row i: word 4 i + t / 32)
    uint16_t bits16[64 * 8];    // the same, written 16 tokens at a time
  };
  float snorm[64];
  float knorm[PAGE];
  double ksq[PAGE];
  double ksq_o[PAGE];           // outlier split: squared norm over the outlier channels
};

// Key part P: sketch rows 64 P .. 64 P + 63 (fragment pair P of the sign
// region); part 0 also writes the norms. sign(S_i . k_t) comes from a bf16
// MFMA (exact products, float accumulation) and is accepted when |dot| >
// 2^-16 ||S_i|| ||k_t||, which exceeds the float summation error bound;
// otherwise the dot product is recomputed in double.
// Outlier split (QJL outlier handling): parts of the normal instance (rows
// below qjl_m) zero the head's outlier columns of their S rows and parts of
// the outlier instance the other columns, so each dot product runs over its
// instance's channels only; part 0 writes ||k_normal|| and ||k_outlier||.
__device__ __attribute__((always_inline)) inline void flush_qjl_key_part(const FlushArgs& A, uint8_t* page, int64_t head,
                                                                         int64_t row0, int P, QPartSmem& S) {
  const QjlGeo g = qjl_geo(A.qjl_m, A.qjl_mo);
  const bool split = A.qjl_mo > 0;
  uint32_t om[4] = {0u, 0u, 0u, 0u};          // outlier channel bits
  if (split) {
    const uint8_t* rec = A.mask + head * QJL_RECORD;
    for (int k = 0; k < QJL_RECORD; ++k) om[k >> 2] |= (uint32_t)rec[k] << (8 * (k & 3));
  }
  stage_rows<64>(S.srow, A.qjl_s, 64 * P);    // S is [m + mo][128] bf16
  stage_rows<PAGE>(S.tile, A.k_src, row0);
  __syncthreads();
  if (split) {
    const uint32_t outlier_rows = 64 * P >= A.qjl_m ? 1u : 0u;
    for (int i = threadIdx.x; i < 64 * D; i += blockDim.x) {
      const int d = i & (D - 1);
      if (((om[d >> 5] >> (d & 31)) & 1u) != outlier_rows) S.srow[i] = 0;
    }
    __syncthreads();
  }
  for (int i = threadIdx.x; i < 64 + PAGE; i += blockDim.x) {
    const uint16_t* row = i < 64 ? S.srow + i * D : S.tile + (i - 64) * D;
    double acc = 0.0, acc_o = 0.0;
    bool bad = false;
    for (int c = 0; c < D / 8; ++c) {
      const uint4 w8 = reinterpret_cast<const uint4*>(row)[c];
      const uint32_t wv[4] = {w8.x, w8.y, w8.z, w8.w};
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const uint16_t v = (uint16_t)(wv[k >> 1] >> (16 * (k & 1)));
        if (bf16_exp_field(v) == 0xFF) bad = true;
        const double x = bf16_to_f64(v);
        const int d = 8 * c + k;
        if ((om[d >> 5] >> (d & 31)) & 1u) acc_o = fma(x, x, acc_o);
        else acc = fma(x, x, acc);
      }
    }
    if (bad) atomicOr(A.flags, KVQ_FLAG_NONFINITE);
    if (i < 64) {
      S.snorm[i] = (float)sqrt(acc + acc_o);
    } else {   // acc: the normal channels (every channel without the split)
      S.knorm[i - 64] = (float)sqrt(acc + acc_o);
      S.ksq[i - 64] = acc;
      S.ksq_o[i - 64] = acc_o;
    }
  }
  __syncthreads();
  {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int a = lane >> 4, r = lane & 15;
    for (int tile = wave; tile < 32; tile += 4) {   // 4 row tiles x 8 token tiles
      const int ti = tile >> 3, tt = tile & 7;
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8_t av = *reinterpret_cast<const bf16x8_t*>(S.srow + (16 * ti + r) * D + 32 * ks + 8 * a);
        const bf16x8_t bv = *reinterpret_cast<const bf16x8_t*>(S.tile + (16 * tt + r) * D + 32 * ks + 8 * a);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc, 0, 0, 0);
      }
      for (int e = 0; e < 4; ++e) {        // D[row = sketch 16 ti + 4 a + e][col = token 16 tt + r]
        const int il = 16 * ti + 4 * a + e, t = 16 * tt + r;
        const float dot = acc[e];
        bool pos;
        if (fabsf(dot) > 0x1.0p-16f * S.snorm[il] * S.knorm[t]) {
          pos = dot >= 0.f;
        } else if (S.ksq[t] + S.ksq_o[t] == 0.0) {    // k = 0: the dot product is exactly 0
          pos = true;
        } else {
          double x = 0.0;
          for (int d = 0; d < D; ++d) x = fma(bf16_to_f64(S.srow[il * D + d]), bf16_to_f64(S.tile[t * D + d]), x);
          pos = x >= 0.0;
        }
        // the 16 lanes of row group a hold tokens 16 tt .. 16 tt + 15 of sketch row il
        const uint64_t bal = __ballot(pos);
        if (r == 0) S.bits16[il * 8 + tt] = (uint16_t)(bal >> (16 * a));
      }
    }
  }
  __syncthreads();
  {  // unit (aa, rr) of pair P, word wq = 2 half + q
    const int t = threadIdx.x, u = t >> 2, wq = t & 3, aa = u >> 4, rr = u & 15, half = wq >> 1, q = wq & 1;
    const int fl = 4 * half + aa;         // fragment 8 P + fl, local rows 8 fl .. 8 fl + 7
    uint32_t word = 0;
    for (int bit = 0; bit < 32; ++bit) {   // tile T, element 4 z + 2 q + h at bit 16 h + 8 (T / 4) + 2 (T % 4) + z
      const int il = 8 * fl + 4 * (bit & 1) + 2 * q + (bit >> 4);
      const int tok = 16 * (4 * ((bit >> 3) & 1) + ((bit >> 1) & 3)) + rr;
      word |= ((S.bits[il * 4 + (tok >> 5)] >> (tok & 31)) & 1u) << bit;
    }
    store4(page + 1024 * P + 256 * aa + 16 * rr + 4 * wq, word);
  }
  if (P == 0 && threadIdx.x < 64) {   // norms: position 32 a + 4 i + e holds token 16 i + 4 a + e
    const int qd = threadIdx.x >> 2, w = threadIdx.x & 3;
    uint16_t v[2], vo[2];
    for (int k = 0; k < 2; ++k) {
      const int pos = 8 * qd + 2 * w + k;
      const int aa = pos >> 5, i = (pos >> 2) & 7, e = pos & 3;
      v[k] = sqrt_to_f16_rne(S.ksq[16 * i + 4 * aa + e]);
      vo[k] = sqrt_to_f16_rne(S.ksq_o[16 * i + 4 * aa + e]);
    }
    store4(page + g.off_norm + 16 * qd + 4 * w, (uint32_t)v[0] | ((uint32_t)v[1] << 16));
    if (split) store4(page + g.off_norm_o + 16 * qd + 4 * w, (uint32_t)vo[0] | ((uint32_t)vo[1] << 16));
  }
}

// ------------------------------------------------------------------ kernels
// Block `lin` of a flush: part lin / units of page unit lin % units (unit:
// head-major, page-minor). Part-major order puts the parts of one page
// `units` blocks apart, so with units a multiple of 8 they land on the same
// XCD (blocks go round-robin over the 8) and the Key parts, which each stage
// the page's whole Key tile, share that XCD's L2 rather than each fetching
// the tile from memory.
__device__ inline void part_coords(const FlushArgs& A, int parts, int lin, int& part, int64_t& head, int64_t& row0,
                                   uint8_t*& page, int& lpage) {
  (void)parts;
  part = lin / A.units;
  const int unit = lin - part * A.units;
  head = unit / A.n_pages;
  const int p = unit - (int)head * A.n_pages;
  lpage = A.first_page + p;
  row0 = head * A.src_stride + (int64_t)p * PAGE;
  if (A.table == nullptr) {
    page = A.arena + (head * A.max_pages + A.first_page + p) * A.page_stride;
  } else {   // an entry outside the pool: the page is not written (KVQ_FLAG_TABLE)
    const int v = A.table[head * A.table_stride + A.first_page + p];
    page = (v >= 0 && v < A.pool_pages) ? A.arena + (int64_t)v * A.page_stride : nullptr;
  }
}

// One flush block (256 threads): value k-step `part` (< V_PARTS) or a Key
// part of its page.
template <int MODE>
__device__ inline void flush_block(const FlushArgs& A, int parts, int lin) {
  int part, lpage;
  int64_t head, row0;
  uint8_t* page;
  part_coords(A, parts, lin, part, head, row0, page, lpage);
  if (page == nullptr) {   // uniform over the block: no barrier is reached
    if (threadIdx.x == 0 && part == 0) atomicOr(A.flags, KVQ_FLAG_TABLE);
    return;
  }
  if constexpr (MODE == KVQ_KEY_MIXKVQ) {
    __shared__ union {
      VPartSmem v;
      KPartSmem k;
    } S;
    int hn16 = A.n16, hn4 = A.n4;
    if (A.head_tiers && part < V_PARTS) mix_record_counts(A.mask + head * MIX_RECORD, hn16, hn4);
    const MixGeo g = mix_geo(hn16, hn4);
    if (part < V_PARTS && A.keys_only) zero_value_part(page + g.off_v, part);
    else if (part < V_PARTS) flush_value_part(page + g.off_v, A.v_src, row0, part, A.flags, S.v);
    else flush_mix_key_part(A, page, head, row0, part - V_PARTS, lpage, S.k);
  } else if constexpr (MODE == KVQ_KEY_PNMIX) {
    __shared__ union {
      VPartSmem v;
      KPartSmem k;
    } S;
    const PnGeo g = pn_geo(A.n_hi);
    if (part < V_PARTS && A.keys_only) zero_value_part(page + g.off_v, part);
    else if (part < V_PARTS) flush_value_part(page + g.off_v, A.v_src, row0, part, A.flags, S.v);
    else flush_pn_key_part(A, page, head, row0, part - V_PARTS, S.k);
  } else {
    __shared__ union {
      VPartSmem v;
      QPartSmem q;
    } S;
    const QjlGeo g = qjl_geo(A.qjl_m, A.qjl_mo);
    if (part < V_PARTS && A.keys_only) zero_value_part(page + g.off_v, part);
    else if (part < V_PARTS) flush_value_part(page + g.off_v, A.v_src, row0, part, A.flags, S.v);
    else flush_qjl_key_part(A, page, head, row0, part - V_PARTS, S.q);
  }
}

__global__ __launch_bounds__(256) void flush_mixkvq_kernel(FlushArgs A, int parts) {
  flush_block<KVQ_KEY_MIXKVQ>(A, parts, blockIdx.x);
}
__global__ __launch_bounds__(256) void flush_pnmix_kernel(FlushArgs A, int parts) {
  flush_block<KVQ_KEY_PNMIX>(A, parts, blockIdx.x);
}
__global__ __launch_bounds__(256) void flush_qjl_kernel(FlushArgs A, int parts) {
  flush_block<KVQ_KEY_QJL>(A, parts, blockIdx.x);
}

// A decode call's split merge beside a flush, in one launch (the two are
// independent): blocks [0, n_flush) are flush blocks, the rest merge four
// query heads each, one per wave. The merge waves touch no LDS and reach no
// barrier, so blocks of either kind run the same code as on their own.
template <int MODE, int NB>
__global__ __launch_bounds__(256) void merge_flush_kernel(FlushArgs A, int parts, int n_flush, const float* partial,
                                                          float* out, int n_parts, int rows) {
  const int blk = blockIdx.x;
  if (blk < n_flush) {
    flush_block<MODE>(A, parts, blk);
    return;
  }
  const int row = 4 * (blk - n_flush) + (threadIdx.x >> 6);
  if (row < rows) merge_row<NB>(partial, out, n_parts, rows, row);
}

// ------------------------------------------------------------------ launchers
// ------------------------------------------------------------------ value push
// KIVI Value FIFO (KIVI blog section 4): the Value rows of tokens that leave
// the full-precision window are quantized per token (four groups of 32
// channels, 2 bits, the flush's exact quantizer) and ORed into their pages,
// whose value part the Key seal has cleared. One wave per (head, row): lane
// l holds channels 2l, 2l+1; a group is 16 lanes. In the page's value layout
// the token's 128 codes fill bits 2u + 16hh of 16 dwords (one per channel
// residue r = c % 16, u = c / 16) and its 4 scales and offsets the 16-bit
// half hh of 8 metadata dwords.
__global__ __launch_bounds__(64) void value_push_kernel(FlushArgs A, int key_mode) {
  const int lane = threadIdx.x;
  const int64_t head = blockIdx.x / A.push_rows;
  const int j = blockIdx.x - (int)head * A.push_rows;
  const int tok = A.push_first + j, lpage = tok / PAGE, rr = tok % PAGE;
  uint8_t* page;
  if (A.table == nullptr) {
    page = A.arena + (head * A.max_pages + lpage) * A.page_stride;
  } else {
    const int v = A.table[head * A.table_stride + lpage];
    if (v < 0 || v >= A.pool_pages) {   // uniform: nothing written
      if (lane == 0) atomicOr(A.flags, KVQ_FLAG_TABLE);
      return;
    }
    page = A.arena + (int64_t)v * A.page_stride;
  }
  int off_v;
  if (key_mode == KVQ_KEY_MIXKVQ) {
    int hn16 = A.n16, hn4 = A.n4;
    if (A.head_tiers) mix_record_counts(A.mask + head * MIX_RECORD, hn16, hn4);
    off_v = mix_geo(hn16, hn4).off_v;
  } else if (key_mode == KVQ_KEY_PNMIX) {
    off_v = pn_geo(A.n_hi).off_v;
  } else {
    off_v = qjl_geo(A.qjl_m, A.qjl_mo).off_v;
  }
  const uint32_t w = reinterpret_cast<const uint32_t*>(A.v_src + (head * A.src_stride + j) * D)[lane];
  const uint32_t cw[1] = {w};
  Scan sc = scan_words(cw);
  scan_merge<1>(sc);
  scan_merge<2>(sc);
  scan_merge<4>(sc);
  {   // lanes 8 apart within the group of 16
    sc.mn = fminf(sc.mn, __shfl_xor(sc.mn, 8));
    sc.mx = fmaxf(sc.mx, __shfl_xor(sc.mx, 8));
    sc.am1 = min(sc.am1, (uint32_t)__shfl_xor((int)sc.am1, 8));
    const int partner_nonfinite = __shfl_xor((int)sc.nonfinite, 8);   // every lane (see scan_merge)
    sc.nonfinite = sc.nonfinite | (partner_nonfinite != 0);
  }
  const int grp = lane >> 4;
  const GroupParam p = make_param(sc, 3, (lane & 15) == 0 ? A.flags : nullptr);   // one status write per group
  const int c0 = quant_code(p, 3, bf16_to_f32((uint16_t)w)), c1 = quant_code(p, 3, bf16_to_f32((uint16_t)(w >> 16)));
  // token -> (k-step s, lane group a, element k = 2 w + hh) of the value layout
  const int s = rr >> 5, rem = rr & 31, a = (rem & 15) >> 2, k = 4 * (rem >> 4) + (rem & 3);
  const int wd = k >> 1, hh = k & 1;
  uint8_t* pv = page + off_v;
  // the dword of channel residue r = lane % 16: codes of channels 16 u + r,
  // held by lane 8 u + r / 2 (gathered with every lane active, stored by 16)
  uint32_t word = 0;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int src = 8 * u + ((lane & 15) >> 1);
    const int x0 = __shfl(c0, src), x1 = __shfl(c1, src);
    word |= (uint32_t)((lane & 1) ? x1 : x0) << (2 * u + 16 * hh);
  }
  if (lane < 16) atomicOr(reinterpret_cast<unsigned*>(pv + 1024 * s + 256 * a + 16 * lane + 4 * wd), word);
  if ((lane & 15) == 0) {   // group grp's scale (half 0) and offset (half 1)
    uint8_t* m = pv + V_CODE_BYTES + 512 * s + 128 * a + 32 * grp + 4 * wd;
    atomicOr(reinterpret_cast<unsigned*>(m), (uint32_t)p.scale << (16 * hh));
    atomicOr(reinterpret_cast<unsigned*>(m + 16), (uint32_t)p.offset << (16 * hh));
  }
}

hipError_t launch_value_push(int key_mode, const FlushArgs& a, int batch, hipStream_t stream) {
  const int64_t heads = (int64_t)batch * a.n_kv_heads;
  hipLaunchKernelGGL(value_push_kernel, dim3((unsigned)(heads * a.push_rows)), dim3(64), 0, stream, a, key_mode);
  return hipGetLastError();
}

// most code fragments a MixKVQ page can have: the configured counts, or with
// threshold tiers any counts within the capacities (fewer BF16 channels leave
// more UINT2 slots)
int mix_max_fragments(int n16, int n4, bool head_tiers) {
  if (!head_tiers) return mix_geo(n16, n4).F;
  int f = 0;
  for (int a = 0; a <= n16; ++a)
    for (int c = 0; c <= n4 && a + c <= D; ++c) f = max(f, mix_geo(a, c).F);
  return f;
}

static int flush_parts(int key_mode, const FlushArgs& a) {
  if (key_mode == KVQ_KEY_MIXKVQ)   // part 0 also writes the BF16 rows
    return V_PARTS + max(1, (mix_max_fragments(a.n16, a.n4, a.head_tiers) + 3) / 4);
  if (key_mode == KVQ_KEY_PNMIX) return V_PARTS + 2;
  return V_PARTS + (a.qjl_m + a.qjl_mo) / 64;
}

hipError_t launch_flush(int key_mode, const FlushArgs& a, int batch, hipStream_t stream) {
  const int parts = flush_parts(key_mode, a);
  const dim3 grid(a.units * parts);
  (void)batch;
  if (key_mode == KVQ_KEY_MIXKVQ)
    hipLaunchKernelGGL(flush_mixkvq_kernel, grid, dim3(256), 0, stream, a, parts);
  else if (key_mode == KVQ_KEY_PNMIX)
    hipLaunchKernelGGL(flush_pnmix_kernel, grid, dim3(256), 0, stream, a, parts);
  else
    hipLaunchKernelGGL(flush_qjl_kernel, grid, dim3(256), 0, stream, a, parts);
  return hipGetLastError();
}

template <int MODE>
static void launch_mf(dim3 grid, hipStream_t s, const FlushArgs& f, int parts, int n_flush, const DecodeArgs& d,
                      int n_parts, int rows) {
  hipLaunchKernelGGL((merge_flush_kernel<MODE, 16>), grid, dim3(256), 0, s, f, parts, n_flush, d.partial, d.out,
                     n_parts, rows);
}

hipError_t launch_merge_flush(int key_mode, const DecodeArgs& d, const FlushArgs& f, int batch, hipStream_t s) {
  const int parts = flush_parts(key_mode, f);
  const int n_flush = f.units * parts;
  (void)batch;
  const int rows = d.batch * d.n_q_heads;
  const int n_parts = decode_parts(d);
  const dim3 grid(n_flush + (rows + 3) / 4);
  // merge batches of 16 parts: the merge's result does not depend on the
  // batch, and larger batches' registers would be the whole kernel's and cut
  // the flush blocks' occupancy; the merge hides behind the flush either way
  if (key_mode == KVQ_KEY_MIXKVQ) launch_mf<KVQ_KEY_MIXKVQ>(grid, s, f, parts, n_flush, d, n_parts, rows);
  else if (key_mode == KVQ_KEY_PNMIX) launch_mf<KVQ_KEY_PNMIX>(grid, s, f, parts, n_flush, d, n_parts, rows);
  else launch_mf<KVQ_KEY_QJL>(grid, s, f, parts, n_flush, d, n_parts, rows);
  return hipGetLastError();
}

}  // namespace kvq
