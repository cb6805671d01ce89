// Flush kernels: quantize and pack full 128-token segments into pages.
//
// MixKVQ Algorithm 1 (KeyQuant / GroupQuant at a buffer flush) with the
// KIVI blog grouping axes: Keys per channel over the 128 tokens of the page,
// Values per token over groups of 32 channels. PN-Mix Eq.2/Eq.7 and
// Appendix G planes. QJL Algorithm 1 steps 2-3 (sign(S k) and ||k||).
//
// One workgroup of 256 threads handles one (page, kv head, batch). The page
// tokens are staged in LDS; phase 1 reduces each group's min/max, phase 2
// lets every thread produce whole 16-byte output units, so all global stores
// are coalesced dwordx4 stores.
//
// Exactness. Codes are round-half-even of the exact (2^b-1)(x-m)/(M-m): an
// estimate from a reciprocal is corrected by comparing 2(2^b-1)(x-m) with
// (2c+-1)(M-m) in double precision, exact while a group spans at most 38
// binades (checked; KVQ_FLAG_SPAN otherwise). Scales and offsets are the
// binary16 nearest to the exact values (one rounding from a double that is
// either exact or correctly rounded and never a binary16 midpoint); values
// beyond the binary16 range are stored as infinity with KVQ_FLAG_RANGE.
#include "kvq_internal.h"

namespace kvq {

__constant__ int c_swap[8] = {0, 2, 1, 3, 4, 6, 5, 7};

// 16 bytes per group; M - m is recomputed exactly in double from m and M.
struct GroupParam {
  float m;         // group minimum (exact bf16 value)
  float M;         // group maximum
  float inv;       // levels / (M - m), an estimate used before the exact fix-up
  uint16_t scale;  // stored binary16 scale
  uint16_t offset; // stored binary16 offset
};

// value token t of a page lives at src[(base + t) * 128 + d]
__device__ inline void stage_page(uint16_t* lds, const uint16_t* src, int64_t row0) {
  const uint4* s = reinterpret_cast<const uint4*>(src + row0 * D);
  uint4* d = reinterpret_cast<uint4*>(lds);
  for (int i = threadIdx.x; i < PAGE * D / 8; i += blockDim.x) d[i] = s[i];
}

// min / max / flags over n values read by a strided accessor (all in LDS)
struct Scan {
  float mn, mx;
  int emin, emax;  // exponent fields of nonzero |x|
  bool nonfinite;
};
__device__ inline void scan_init(Scan& s) {
  s.mn = INFINITY;
  s.mx = -INFINITY;
  s.emin = 1000;
  s.emax = -1000;
  s.nonfinite = false;
}
__device__ inline void scan_add(Scan& s, uint16_t b) {
  int e = bf16_exp_field(b);
  if (e == 0xFF) { s.nonfinite = true; return; }
  float v = bf16_to_f32(b);
  s.mn = fminf(s.mn, v);
  s.mx = fmaxf(s.mx, v);
  if ((b & 0x7FFF) != 0) {
    int ee = e == 0 ? 1 : e;
    s.emin = min(s.emin, ee);
    s.emax = max(s.emax, e);
  }
}
__device__ inline void scan_merge_xor(Scan& s, int mask) {
  s.mn = fminf(s.mn, __shfl_xor(s.mn, mask));
  s.mx = fmaxf(s.mx, __shfl_xor(s.mx, mask));
  s.emin = min(s.emin, __shfl_xor(s.emin, mask));
  s.emax = max(s.emax, __shfl_xor(s.emax, mask));
  s.nonfinite = s.nonfinite || __shfl_xor((int)s.nonfinite, mask);
}

__device__ inline bool f16_is_inf(uint16_t h) { return (h & 0x7FFF) == 0x7C00; }

__device__ inline void flag_range(const GroupParam& p, unsigned* flags) {
  if (f16_is_inf(p.scale) || f16_is_inf(p.offset)) atomicOr(flags, KVQ_FLAG_RANGE);
}

// min-max quantizer parameters for `levels` = 2^b - 1
__device__ inline GroupParam make_param(const Scan& s, int levels, unsigned* flags) {
  GroupParam p;
  p.m = s.mn;
  p.M = s.mn;
  p.offset = s.mn == INFINITY ? (uint16_t)0 : f64_to_f16_rne((double)s.mn);
  p.inv = 0.0f;
  p.scale = 0;
  if (s.nonfinite) atomicOr(flags, KVQ_FLAG_NONFINITE);
  if (s.emax - s.emin > 38) atomicOr(flags, KVQ_FLAG_SPAN);
  if (s.mx > s.mn) {
    p.M = s.mx;
    const double den = (double)s.mx - (double)s.mn;
    p.inv = (float)((double)levels / den);
    p.scale = f64_to_f16_rne(den / (double)levels);
  }
  flag_range(p, flags);
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
  if (s.nonfinite) atomicOr(flags, KVQ_FLAG_NONFINITE);
  if (s.emax - s.emin > 38) atomicOr(flags, KVQ_FLAG_SPAN);
  if (s.mx > s.mn) {
    p.M = s.mx;
    const double den = (double)s.mx - (double)s.mn;
    p.scale = f64_to_f16_rne(0.5 * den);
    p.offset = f64_to_f16_rne(0.25 * (3.0 * (double)s.mn + (double)s.mx));
  }
  flag_range(p, flags);
  return p;
}

// Exact round-half-even code of x for levels = 2^b - 1. The float estimate
// is within one of the true code; the fix-up compares 2*levels*(x-m) with
// (2c -+ 1)(M-m), all exact in double for groups spanning <= 38 binades.
__device__ inline int quant_code(const GroupParam& p, int levels, float x) {
  if (!(p.M > p.m)) return 0;
  double den = (double)p.M - (double)p.m;
  double two_num = 2.0 * (double)levels * ((double)x - (double)p.m);
  int c = __float2int_rn((x - p.m) * p.inv);
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

// PN-Mix Eq.7 code: 1 iff 2(x - m) > M - m (the exact midpoint rounds to 0)
__device__ inline int mid_code(const GroupParam& p, float x) {
  if (!(p.M > p.m)) return 0;
  return 2.0 * ((double)x - (double)p.m) > ((double)p.M - (double)p.m) ? 1 : 0;
}

__device__ inline void store16(uint8_t* dst, uint4 v) { *reinterpret_cast<uint4*>(dst) = v; }

// ------------------------------------------------------------------ values
// Per-token value parameters: 128 tokens x 4 groups, thread t -> groups 2t, 2t+1.
__device__ inline void value_params(const uint16_t* sv, GroupParam* vp, unsigned* flags) {
  for (int g = threadIdx.x; g < PAGE * 4; g += blockDim.x) {
    int t = g >> 2, j = g & 3;
    Scan s;
    scan_init(s);
    for (int c = 0; c < GV; ++c) scan_add(s, sv[t * D + GV * j + c]);
    vp[g] = make_param(s, 3, flags);
  }
}

__device__ inline int pi_token(int s, int a, int k) { return 32 * s + 16 * (k >> 2) + 4 * a + (k & 3); }

// value code region unit (s, a, r): 16 bytes = V-tiles u = 0..7, 8 tokens each
__device__ inline uint4 value_code_unit(const uint16_t* sv, const GroupParam* vp, int s, int a, int r) {
  uint32_t w4[4];
  for (int w = 0; w < 4; ++w) {
    uint32_t word = 0;
    for (int p = 0; p < 16; ++p) {
      int u = 2 * w + (p >> 3);
      int k = c_swap[p & 7];
      int t = pi_token(s, a, k);
      int ch = 16 * u + r;
      int code = quant_code(vp[t * 4 + (ch >> 5)], 3, bf16_to_f32(sv[t * D + ch]));
      word |= (uint32_t)code << (2 * p);
    }
    w4[w] = word;
  }
  return make_uint4(w4[0], w4[1], w4[2], w4[3]);
}

// value meta unit (s, a, j, half): 8 scales (half 0) or 8 offsets (half 1)
__device__ inline uint4 value_meta_unit(const GroupParam* vp, int s, int a, int j, int half) {
  uint32_t w4[4];
  for (int w = 0; w < 4; ++w) {
    uint16_t lo, hi;
    const GroupParam& p0 = vp[pi_token(s, a, 2 * w) * 4 + j];
    const GroupParam& p1 = vp[pi_token(s, a, 2 * w + 1) * 4 + j];
    lo = half ? p0.offset : p0.scale;
    hi = half ? p1.offset : p1.scale;
    w4[w] = (uint32_t)lo | ((uint32_t)hi << 16);
  }
  return make_uint4(w4[0], w4[1], w4[2], w4[3]);
}

// Stage the page's Values in `tile`, quantize per token and write the value
// code region (256 units) and value meta region (128 units).
__device__ inline void value_part(uint8_t* page, uint16_t* tile, GroupParam* vp, const uint16_t* v_src,
                                  int64_t row0, unsigned* flags) {
  __syncthreads();                      // the tile may still be read by the Key phase
  stage_page(tile, v_src, row0);
  __syncthreads();
  value_params(tile, vp, flags);
  __syncthreads();
  const uint16_t* sv = tile;
  for (int u = threadIdx.x; u < 384; u += blockDim.x) {
    if (u < 256) {
      int s = u >> 6, a = (u >> 4) & 3, r = u & 15;
      store16(page + 1024 * s + 256 * a + 16 * r, value_code_unit(sv, vp, s, a, r));
    } else {
      int m = u - 256;
      int s = m >> 5, a = (m >> 3) & 3, j = (m >> 1) & 3, half = m & 1;
      store16(page + V_CODE_BYTES + 512 * s + 128 * a + 32 * j + 16 * half, value_meta_unit(vp, s, a, j, half));
    }
  }
}

// ------------------------------------------------------------------ MixKVQ

struct FlushSmem {
  uint16_t tile[PAGE * D];      // staged Keys, then Values
  GroupParam kp[D];             // Key group parameters
  GroupParam vp[PAGE * 4];      // Value group parameters
};

__device__ inline uint4 pack8(const uint16_t* v) {
  return make_uint4(v[0] | ((uint32_t)v[1] << 16), v[2] | ((uint32_t)v[3] << 16), v[4] | ((uint32_t)v[5] << 16),
                    v[6] | ((uint32_t)v[7] << 16));
}

__global__ __launch_bounds__(256) void flush_mixkvq_kernel(FlushArgs A) {
  __shared__ FlushSmem S;
  __shared__ uint8_t perm[D];
  const int p = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int64_t head = (int64_t)b * A.n_kv_heads + h;
  const int64_t row0 = head * A.src_stride + (int64_t)p * PAGE;
  uint8_t* page = A.arena + (head * A.max_pages + A.first_page + p) * A.page_stride;
  const MixGeo g = mix_geo(A.n16, A.n4);
  uint16_t* sk = S.tile;

  if (threadIdx.x < D) perm[threadIdx.x] = A.mask[head * MIX_RECORD + threadIdx.x];
  stage_page(sk, A.k_src, row0);
  __syncthreads();

  // Key channel parameters, two threads per channel position
  {
    int c = threadIdx.x >> 1, half = threadIdx.x & 1;
    int d = perm[c];
    Scan s;
    scan_init(s);
    for (int t = half * 64; t < half * 64 + 64; ++t) scan_add(s, sk[t * D + d]);
    scan_merge_xor(s, 1);
    if (half == 0) {
      if (c < g.n16) {
        if (s.nonfinite) atomicOr(A.flags, KVQ_FLAG_NONFINITE);
      } else {
        S.kp[c] = make_param(s, c < g.n16 + g.n4 ? 15 : 3, A.flags);
      }
    }
  }
  __syncthreads();

  const int n_bf = 16 * g.n16, n_codes = 16 * g.F, n_meta = 2 * g.F;
  for (int u = threadIdx.x; u < n_bf + n_codes + n_meta; u += blockDim.x) {
    if (u < n_bf) {                       // BF16 tier: channel row c, token row r, 8 tiles
      int c = u >> 4, r = u & 15, d = perm[c];
      uint16_t v[8];
      for (int i = 0; i < 8; ++i) v[i] = sk[(16 * i + r) * D + d];
      store16(page + 256 * c + 16 * r, pack8(v));
    } else if (u < n_bf + n_codes) {      // code fragment f, token row r
      int f = (u - n_bf) >> 4, r = (u - n_bf) & 15;
      uint32_t w4[4];
      for (int w = 0; w < 4; ++w) {
        uint32_t word = 0;
        for (int pp = 0; pp < 16; ++pp) {
          int t = 16 * (2 * w + (pp >> 3)) + r;
          int slot = 8 * f + c_swap[pp & 7];
          int code = 0;
          if (slot < 2 * g.n4) {
            int c = g.n16 + (slot >> 1);
            int full = quant_code(S.kp[c], 15, bf16_to_f32(sk[t * D + perm[c]]));
            code = (slot & 1) ? (full >> 2) : (full & 3);
          } else if (slot >= g.s4 && slot < g.s4 + g.n2) {
            int c = g.n16 + g.n4 + (slot - g.s4);
            code = quant_code(S.kp[c], 3, bf16_to_f32(sk[t * D + perm[c]]));
          }
          word |= (uint32_t)code << (2 * pp);
        }
        w4[w] = word;
      }
      store16(page + g.off_codes + 256 * f + 16 * r, make_uint4(w4[0], w4[1], w4[2], w4[3]));
    } else {                              // slot scales (half 0) / offsets (half 1)
      int m = u - n_bf - n_codes;
      int f = m >> 1, half = m & 1;
      uint16_t v[8];
      for (int k = 0; k < 8; ++k) {
        int slot = 8 * f + k;
        uint16_t sc = 0, of = 0;
        if (slot < 2 * g.n4) {
          const GroupParam& q = S.kp[g.n16 + (slot >> 1)];
          if (slot & 1) {
            sc = q.scale == 0 ? 0 : f64_to_f16_rne(4.0 * f16_to_f64(q.scale));   // 4s, no offset
            if (f16_is_inf(sc) && !half) atomicOr(A.flags, KVQ_FLAG_RANGE);
          } else {
            sc = q.scale;
            of = q.offset;
          }
        } else if (slot >= g.s4 && slot < g.s4 + g.n2) {
          const GroupParam& q = S.kp[g.n16 + g.n4 + (slot - g.s4)];
          sc = q.scale;
          of = q.offset;
        }
        v[k] = half ? of : sc;
      }
      store16(page + g.off_meta + 32 * f + 16 * half, pack8(v));
    }
  }
  value_part(page + g.off_v, S.tile, S.vp, A.v_src, row0, A.flags);
}

// ------------------------------------------------------------------ PN-Mix
__global__ __launch_bounds__(256) void flush_pnmix_kernel(FlushArgs A) {
  __shared__ FlushSmem S;
  __shared__ uint8_t slot_ch[D];
  __shared__ uint8_t is_hi[D];
  __shared__ int n_hi_s;
  const int p = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int64_t head = (int64_t)b * A.n_kv_heads + h;
  const int64_t row0 = head * A.src_stride + (int64_t)p * PAGE;
  uint8_t* page = A.arena + (head * A.max_pages + A.first_page + p) * A.page_stride;
  const PnGeo g = pn_geo(A.n_hi);
  uint16_t* sk = S.tile;

  if (threadIdx.x < D) {
    int d = threadIdx.x;
    int pair = A.pair_layout == KVQ_PAIR_HALF_SPLIT ? (d & 63) : (d >> 1);
    is_hi[d] = (A.mask[head * PN_RECORD + (pair >> 3)] >> (pair & 7)) & 1;
  }
  stage_page(sk, A.k_src, row0);
  __syncthreads();
  if (threadIdx.x == 0) {   // slot order: high channels ascending, then low ones
    int nh = 0;
    for (int d = 0; d < D; ++d)
      if (is_hi[d]) slot_ch[nh++] = (uint8_t)d;
    int nl = nh;
    for (int d = 0; d < D; ++d)
      if (!is_hi[d]) slot_ch[nl++] = (uint8_t)d;
    n_hi_s = nh;
    if (nh != A.n_hi) atomicOr(A.flags, KVQ_FLAG_MASK);
  }
  __syncthreads();
  const int n_hi = min(n_hi_s, A.n_hi);

  {
    int slot = threadIdx.x >> 1, half = threadIdx.x & 1;
    int d = slot_ch[slot];
    Scan s;
    scan_init(s);
    for (int t = half * 64; t < half * 64 + 64; ++t) scan_add(s, sk[t * D + d]);
    scan_merge_xor(s, 1);
    if (half == 0) S.kp[slot] = slot < n_hi_s ? make_param(s, 7, A.flags) : make_param_mid(s, A.flags);
  }
  __syncthreads();

  const int n_lsb = 128, n_up = 16 * g.n_up_frag, n_meta = 32;
  for (int u = threadIdx.x; u < n_lsb + n_up + n_meta; u += blockDim.x) {
    if (u < n_lsb) {                     // LSB plane: fragment pair P, lane group a, row r
      int P = u >> 6, a = (u >> 4) & 3, r = u & 15;
      uint32_t w4[4];
      for (int half = 0; half < 2; ++half) {
        int f = 4 * (2 * P + half) + a;
        for (int q = 0; q < 2; ++q) {
          uint32_t word = 0;
          for (int bit = 0; bit < 32; ++bit) {
            int bb = bit & 7;
            int slot = 8 * f + 2 * (bb & 3) + (bb >> 2);
            int t = 16 * (4 * q + (bit >> 3)) + r;
            float x = bf16_to_f32(sk[t * D + slot_ch[slot]]);
            int code = slot < n_hi_s ? quant_code(S.kp[slot], 7, x) : mid_code(S.kp[slot], x);
            word |= (uint32_t)(code & 1) << bit;
          }
          w4[2 * half + q] = word;
        }
      }
      store16(page + 1024 * P + 256 * a + 16 * r, make_uint4(w4[0], w4[1], w4[2], w4[3]));
    } else if (u < n_lsb + n_up) {       // upper-2-bit plane of the high channels
      int f = (u - n_lsb) >> 4, r = (u - n_lsb) & 15;
      uint32_t w4[4];
      for (int w = 0; w < 4; ++w) {
        uint32_t word = 0;
        for (int pp = 0; pp < 16; ++pp) {
          int t = 16 * (2 * w + (pp >> 3)) + r;
          int slot = 8 * f + c_swap[pp & 7];
          int code = 0;
          if (slot < n_hi) code = quant_code(S.kp[slot], 7, bf16_to_f32(sk[t * D + slot_ch[slot]])) >> 1;
          word |= (uint32_t)code << (2 * pp);
        }
        w4[w] = word;
      }
      store16(page + g.off_up + 256 * f + 16 * r, make_uint4(w4[0], w4[1], w4[2], w4[3]));
    } else {                             // per-slot scale / offset
      int m = u - n_lsb - n_up;
      int f = m >> 1, half = m & 1;
      uint16_t v[8];
      for (int k = 0; k < 8; ++k) v[k] = half ? S.kp[8 * f + k].offset : S.kp[8 * f + k].scale;
      store16(page + g.off_meta + 32 * f + 16 * half, pack8(v));
    }
  }
  value_part(page + g.off_v, S.tile, S.vp, A.v_src, row0, A.flags);
}

// ------------------------------------------------------------------ QJL
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int QJL_MAX_M = 512;

// sign(S_i . k_t) for i < m, t < 128 with bf16 MFMA (products exact, float
// accumulation). A sign is accepted when |dot| > 2^-16 ||S_i|| ||k_t||, which
// exceeds the float summation error bound; otherwise the dot product is
// recomputed in double.
__global__ __launch_bounds__(256) void flush_qjl_kernel(FlushArgs A) {
  __shared__ FlushSmem S;
  __shared__ uint32_t bits[QJL_MAX_M * 4];
  __shared__ float snorm[QJL_MAX_M];
  __shared__ float knorm[PAGE];
  __shared__ double ksq[PAGE];
  const int p = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int64_t head = (int64_t)b * A.n_kv_heads + h;
  const int64_t row0 = head * A.src_stride + (int64_t)p * PAGE;
  uint8_t* page = A.arena + (head * A.max_pages + A.first_page + p) * A.page_stride;
  const int m = A.qjl_m;
  const QjlGeo g = qjl_geo(m);
  const uint16_t* ss = A.qjl_s;         // S [m][128] stays in L2
  uint16_t* sk = S.tile;

  stage_page(sk, A.k_src, row0);
  for (int i = threadIdx.x; i < m * 4; i += blockDim.x) bits[i] = 0;
  __syncthreads();
  for (int i = threadIdx.x; i < m + PAGE; i += blockDim.x) {
    const uint16_t* row = i < m ? ss + (size_t)i * D : sk + (i - m) * D;
    double acc = 0.0;
    bool bad = false;
    for (int d = 0; d < D; ++d) {
      uint16_t v = row[d];
      if (bf16_exp_field(v) == 0xFF) bad = true;
      double x = bf16_to_f64(v);
      acc = fma(x, x, acc);
    }
    if (bad) atomicOr(A.flags, KVQ_FLAG_NONFINITE);
    if (i < m) {
      snorm[i] = (float)sqrt(acc);
    } else {
      knorm[i - m] = (float)sqrt(acc);
      ksq[i - m] = acc;
    }
  }
  __syncthreads();

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int a = lane >> 4, r = lane & 15;
  const int n_tiles = (m / 16) * 8;
  for (int tile = wave; tile < n_tiles; tile += 4) {
    int ti = tile >> 3, tt = tile & 7;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8_t av = *reinterpret_cast<const bf16x8_t*>(ss + (size_t)(16 * ti + r) * D + 32 * ks + 8 * a);
      bf16x8_t bv = *reinterpret_cast<const bf16x8_t*>(sk + (16 * tt + r) * D + 32 * ks + 8 * a);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc, 0, 0, 0);
    }
    for (int e = 0; e < 4; ++e) {        // D[row = sketch 16 ti + 4 a + e][col = token 16 tt + r]
      int i = 16 * ti + 4 * a + e, t = 16 * tt + r;
      float dot = acc[e];
      bool pos;
      if (fabsf(dot) > 0x1.0p-16f * snorm[i] * knorm[t]) {
        pos = dot >= 0.f;
      } else {
        double x = 0.0;
        for (int d = 0; d < D; ++d) x = fma(bf16_to_f64(ss[(size_t)i * D + d]), bf16_to_f64(sk[t * D + d]), x);
        pos = x >= 0.0;
      }
      if (pos) atomicOr(&bits[i * 4 + (t >> 5)], 1u << (t & 31));
    }
  }
  __syncthreads();

  const int n_bit_units = m;               // (m / 64) pairs x 4 lane groups x 16 rows
  for (int u = threadIdx.x; u < n_bit_units + 16; u += blockDim.x) {
    if (u < n_bit_units) {
      int P = u >> 6, aa = (u >> 4) & 3, rr = u & 15;
      uint32_t w4[4];
      for (int half = 0; half < 2; ++half) {
        int f = 4 * (2 * P + half) + aa;
        for (int q = 0; q < 2; ++q) {
          uint32_t word = 0;
          for (int bit = 0; bit < 32; ++bit) {
            int bb = bit & 7;
            int srow = 8 * f + 2 * (bb & 3) + (bb >> 2);
            int t = 16 * (4 * q + (bit >> 3)) + rr;
            word |= ((bits[srow * 4 + (t >> 5)] >> (t & 31)) & 1u) << bit;
          }
          w4[2 * half + q] = word;
        }
      }
      store16(page + 1024 * P + 256 * aa + 16 * rr, make_uint4(w4[0], w4[1], w4[2], w4[3]));
    } else {                               // norms: position 32 a + 4 i + e holds token 16 i + 4 a + e
      int q = u - n_bit_units;
      uint16_t v[8];
      for (int k = 0; k < 8; ++k) {
        int pos = 8 * q + k;
        int aa = pos >> 5, i = (pos >> 2) & 7, e = pos & 3;
        v[k] = sqrt_to_f16_rne(ksq[16 * i + 4 * aa + e]);
      }
      store16(page + g.off_norm + 16 * q, pack8(v));
    }
  }
  value_part(page + g.off_v, S.tile, S.vp, A.v_src, row0, A.flags);
}

// ------------------------------------------------------------------ launcher
hipError_t launch_flush(int key_mode, const FlushArgs& a, int n_pages, int batch, hipStream_t stream) {
  dim3 grid(n_pages, a.n_kv_heads, batch);
  if (key_mode == KVQ_KEY_MIXKVQ)
    hipLaunchKernelGGL(flush_mixkvq_kernel, grid, dim3(256), 0, stream, a);
  else if (key_mode == KVQ_KEY_PNMIX)
    hipLaunchKernelGGL(flush_pnmix_kernel, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(flush_qjl_kernel, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kvq
