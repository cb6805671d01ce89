// Decode helpers shared by the generic and the pipelined decode kernels:
// MFMA operand expansion, online softmax with the value MFMA, partial writes
// and the BF16 (sink + residual) segment.
#pragma once

#include "kvq_internal.h"

namespace kvq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float B_SCALE = 0.015625f;   // 2^-6 applied to every Key B operand (f16 range headroom)
constexpr float B_UNSCALE = 64.0f;
constexpr int MAX_KS = 8;              // max Key k-steps of 32 slots


__device__ inline uint32_t rd(const u32x4& v, int i) { return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w)); }

__device__ inline u32x4 ld16(const uint8_t* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ inline uint32_t ld4(const uint8_t* p) { return *reinterpret_cast<const uint32_t*>(p); }

// Byte idx of a record held one dword per lane (lane l: bytes 4l .. 4l+3);
// every lane of the wave must execute it.
__device__ inline int rec_byte(uint32_t recw, int idx) {
  const uint32_t w = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * (idx >> 2), (int)recw);
  return (int)((w >> (8 * (idx & 3))) & 0xffu);
}

__device__ inline uint32_t h2u(half2v h) {
  uint32_t u;
  __builtin_memcpy(&u, &h, 4);
  return u;
}

__device__ inline half8 u4_to_h8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  u32x4 v = {a, b, c, d};
  half8 h;
  __builtin_memcpy(&h, &v, 16);
  return h;
}

// Codes as MFMA operands without a conversion. In a 2-bit block row (four
// dwords, see the page layout) the eight codes of tile T sit at bits 2T and
// 16 + 2T of every dword; masking them out leaves binary16 subnormals
// c * 2^(2T - 24), which the f16 MFMA multiplies exactly (gfx950 keeps f16
// denormals). Tiles 4..7 are taken from the dwords shifted right by 8, so
// tile T carries the factor 4^(T & 3) * 2^-24; tile_unscale undoes it.
__device__ inline half8 tile2(const u32x4& w, const u32x4& w8, int T) {
  const u32x4& s = T < 4 ? w : w8;
  const uint32_t m = 0x00030003u << (2 * (T & 3));
  return u4_to_h8(s.x & m, s.y & m, s.z & m, s.w & m);
}
__device__ constexpr float tile_unscale(int T) { return 16777216.0f / (float)(1 << (2 * (T & 3))); }

// A 1-bit block row (two dwords) with the shifted copies its tiles need:
// tile T's bits sit at 16 h + 8 (T / 4) + 2 (T % 4) + z, so the same masks as
// for 2-bit codes give b * 4^(T & 3) * 2^-24 (the same tile factor).
struct Row1 {
  uint32_t w0, w1, w0s1, w1s1, w0s8, w1s8, w0s9, w1s9;
};
__device__ inline Row1 row1(uint32_t w0, uint32_t w1) {
  return Row1{w0, w1, w0 >> 1, w1 >> 1, w0 >> 8, w1 >> 8, w0 >> 9, w1 >> 9};
}
__device__ inline half8 tile1(const Row1& x, int T) {
  const uint32_t m = 0x00010001u << (2 * (T & 3));
  return T < 4 ? u4_to_h8(x.w0 & m, x.w1 & m, x.w0s1 & m, x.w1s1 & m)
               : u4_to_h8(x.w0s8 & m, x.w1s8 & m, x.w0s9 & m, x.w1s9 & m);
}

__device__ inline f32x4 mfma(half8 a, half8 b, f32x4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0); }
__device__ inline f32x4 mfma_bf(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 2^x on the transcendental unit (v_exp_f32). Softmax weights below 2^-126
// flush to zero, which changes no result at float precision.
__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ inline float lo_bf(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float hi_bf(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// 8 binary16 values (scales or offsets of 8 slots / tokens) from 16 bytes
__device__ inline half8 as_half8(const u32x4& v) {
  half8 h;
  __builtin_memcpy(&h, &v, 16);
  return h;
}

// hi/lo f16 split of 8 products
__device__ inline void split8(const float* x, half8& hi, half8& lo) {
  for (int e = 0; e < 8; ++e) {
    _Float16 h = (_Float16)x[e];
    hi[e] = h;
    lo[e] = (_Float16)(x[e] - (float)h);
  }
}

// Reductions over the 4 lane groups sharing a column (lanes 16 apart), with
// the cross-row lane swaps: after a swap of v with itself the two results
// hold v and its partner row's v, in one order or the other.
__device__ inline float wave_max_groups(float v) {
  const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(s16[0]), __uint_as_float(s16[1]));
  const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(s32[0]), __uint_as_float(s32[1]));
}
__device__ inline float wave_sum_groups(float v) {
  const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
  const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
}

// Online-softmax state of one lane (one head; one value group per pass).
// zl accumulates rows 4a..4a+3 of the offset MFMA (A rows 0-3: the value
// offsets of groups 0-3, row 4: ones; B: the probabilities), so lane group 0
// holds sum p * offset of value groups 0-3 and lane group 1 (row 4) sum p,
// each for the head of the lane's column.
template <int NPASS>
struct SoftState {
  float m;          // running max (log2 domain)
  f32x4 zl;
  f32x4 acc[8];     // value accumulators of the 8 value tiles (16 channels each)
};

template <int NPASS>
__device__ inline void init_state(SoftState<NPASS>& st) {
  st.m = -INFINITY;
  st.zl = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < 8; ++u) st.acc[u] = (f32x4){0.f, 0.f, 0.f, 0.f};
}

// Where consume_values takes a page's Value scale and offset words from, per
// k-step ks: the offset row zr of the lane's value group, and the scale row
// of value group j. VMetaAt reads them from the page's metadata halves
// vm_lo / vm_hi where they are used; VMeta holds them loaded beforehand
// (load_vmeta), with the page's other loads, so that a page waits for
// memory once.
// The constant rows of the offset MFMA's A operand, in LDS: ones, then
// zeros. Written once per workgroup before the page loop's first barrier.
struct ZConst {
  u32x4 v[2];
  __device__ inline void init(int lane) {
    if (lane < 2) v[lane] = lane == 0 ? (u32x4){0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u}
                                      : (u32x4){0u, 0u, 0u, 0u};
  }
  __device__ inline const uint8_t* ptr() const { return reinterpret_cast<const uint8_t*>(v); }
};

struct VMetaAt {
  const uint8_t* lo;
  const uint8_t* hi;
  const uint8_t* zc;   // 32 bytes: eight binary16 ones, then zeros (ZConst)
  __device__ inline const uint8_t* row(int ks, int a) const { return (ks < 2 ? lo : hi) + 512 * (ks & 1) + 128 * a; }
  __device__ inline u32x4 z(int ks, int a, int zr) const { return ld16(row(ks, a) + 32 * zr + 16); }
  // the offset MFMA's A operand of column col: the offsets of head col
  // (col < 4), ones (col 4: the probability sum) or zeros, each lane
  // reading its own 16 bytes
  __device__ inline u32x4 za(int ks, int a, int col) const {
    return ld16(col < 4 ? row(ks, a) + 32 * col + 16 : zc + (col == 4 ? 0 : 16));
  }
  __device__ inline u32x4 s(int ks, int, int a, int j) const { return ld16(row(ks, a) + 32 * j); }
};
template <int G, int NPASS>
struct VMeta {
  u32x4 zw[4];
  u32x4 sw[4][NPASS];
  __device__ inline u32x4 z(int ks, int, int) const { return zw[ks]; }
  __device__ inline u32x4 s(int ks, int P, int, int) const { return sw[ks][P]; }
};
template <int G, int NPASS>
__device__ inline void load_vmeta(VMeta<G, NPASS>& m, const uint8_t* vm_lo, const uint8_t* vm_hi, int a, int col) {
  constexpr int C = 16 / G;
  const VMetaAt at{vm_lo, vm_hi};
  const int jl = col / G, zr = col < 4 ? col : 3;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    m.zw[ks] = at.z(ks, a, zr);
#pragma unroll
    for (int P = 0; P < NPASS; ++P) m.sw[ks][P] = at.s(ks, P, a, (jl + P * C) & 3);
  }
}

// Consume one page: logit[i][e] is the raw Key accumulator of tile i row e
// (token 16 i + 4 a + e); the log2-domain logit is logit * xs + xb; vm gives
// the page's Value metadata words (VMetaAt or VMeta).
// HYB (KIVI Value FIFO): page tokens from vlim on have no quantized Value
// yet: their scales and offsets are masked out of the value MFMAs (their
// probabilities still count in the normaliser) and their binary16
// probabilities go to hp[token][head] for the caller to weight the
// full-precision Values with.
template <int G, int NPASS, bool HYB = false, class Meta>
__device__ inline void consume_values(SoftState<NPASS>& st, const f32x4 (&logit)[8], float xs, float xb,
                                      const u32x4 (&vc)[4], const Meta& vm, int a, int col, int vlim = PAGE,
                                      float (*hp)[8] = nullptr) {
  constexpr int C = 16 / G;
  float pm = -INFINITY;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) pm = fmaxf(pm, logit[i][e]);
  pm = fmaf(wave_max_groups(pm), xs, xb);
  const float mn = fmaxf(st.m, pm);
  if (__any(mn > st.m)) {
    const float alpha = (st.m == -INFINITY) ? 0.f : fast_exp2(st.m - mn);
    st.zl *= alpha;
#pragma unroll
    for (int u = 0; u < 8; ++u) st.acc[u] *= alpha;
    st.m = mn;
  }
  const float shift = xb - st.m;
  const int jl = col / G;
  // offset-MFMA A rows: row r < 4 reads the offsets of value group r, row 4
  // is binary16 ones, rows 5-15 zero
  const int zr = col < 4 ? col : 3;
  const uint32_t zconst = col == 4 ? 0x3C003C00u : 0u;
  // k-step outer: the 8 probabilities of tiles 2ks, 2ks+1 are formed right
  // before they are used (in every pass), so only 8 stay live at a time.
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    float p[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      p[e] = fast_exp2(fmaf(logit[2 * ks + (e >> 2)][e & 3], xs, shift));   // token pi(ks, a, e)
    // p as binary16: the B operand of the offset MFMA, and p s of the value
    // MFMAs as one packed multiply per two tokens (two roundings of p s)
    half8 ph;
#pragma unroll
    for (int e = 0; e < 8; ++e) ph[e] = (_Float16)p[e];
    u32x4 keep = {~0u, ~0u, ~0u, ~0u};   // HYB: binary16 lanes of tokens with a quantized Value
    if constexpr (HYB) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int tok = 32 * ks + 16 * (e >> 2) + 4 * a + (e & 3);   // pi(ks, a, e)
        if (tok >= vlim) {
          if (col < G) hp[tok][col] = (float)ph[e];
          const uint32_t m = ~(0xFFFFu << (16 * (e & 1)));
          if ((e >> 1) == 0) keep.x &= m;
          else if ((e >> 1) == 1) keep.y &= m;
          else if ((e >> 1) == 2) keep.z &= m;
          else keep.w &= m;
        }
      }
    }
    {
      // sum p * offset per value group and sum p, on the MFMA (p as binary16)
      const u32x4 zw = vm.z(ks, a, zr) & keep;
      u32x4 za;
      za.x = col < 4 ? zw.x : zconst;
      za.y = col < 4 ? zw.y : zconst;
      za.z = col < 4 ? zw.z : zconst;
      za.w = col < 4 ? zw.w : zconst;
      st.zl = mfma(as_half8(za), ph, st.zl);
    }
#pragma unroll
    for (int P = 0; P < NPASS; ++P) {
      const int j = (jl + P * C) & 3;            // this lane's value group in pass P
      const half8 s8 = as_half8(vm.s(ks, P, a, j) & keep);
      const half8 B = ph * s8;
      const u32x4 v8 = vc[ks] >> 8u;
#pragma unroll
      for (int w = 0; w < 4; ++w) {            // value tiles 2w, 2w+1 hold group w
        if (w / C != P) continue;
        st.acc[2 * w] = mfma(tile2(vc[ks], v8, 2 * w), B, st.acc[2 * w]);
        st.acc[2 * w + 1] = mfma(tile2(vc[ks], v8, 2 * w + 1), B, st.acc[2 * w + 1]);
      }
    }
  }
}

// DPP within each 16-lane row (ctrl 0x128 = rotate by 8: lane c reads lane
// c ^ 8, its partner across the hi/lo Key operand halves); lanes outside the
// bank mask keep `old`.
template <int CTRL, int BANKS>
__device__ inline uint32_t dpp_u(uint32_t old, uint32_t src) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)src, CTRL, 0xF, BANKS, false);
}
template <int CTRL, int BANKS>
__device__ inline float dpp_f(float old, float src) {
  return __uint_as_float(dpp_u<CTRL, BANKS>(__float_as_uint(old), __float_as_uint(src)));
}

// lane col ^ 8's value (row rotate by 8)
__device__ inline float from_partner8(float v) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false));
}

// Hi/lo column split (pipelined kernels): columns col < 8 carry the f16 hi
// part of the Key operand, columns col >= 8 the lo part, so one MFMA per
// tile covers both, leaving the two partial logits in lanes col and col ^ 8.
// Rather than both lanes of a pair adding all 32 values, each forms half of
// them: lanes col < 8 the joined logits of tiles 0-3, lanes col >= 8 those
// of tiles 4-7, in J[0..3].
__device__ inline void half_join(const f32x4 (&L)[8], f32x4 (&J)[4], bool hi) {
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float own = hi ? L[t][e] : L[t + 4][e];    // the tile this lane joins
      const float give = hi ? L[t + 4][e] : L[t][e];   // the tile its partner joins
      J[t][e] = own + from_partner8(give);
    }
}

// consume_values for logits joined by half_join: the softmax maximum, the
// exponentials and their binary16 conversion run on the lane's 16 tokens
// (tiles 0-3 or 4-7); the two k-steps' binary16 probabilities the partner
// lane formed arrive by DPP, so every lane then holds all four k-steps'
// operands as before. Same results as consume_values on the fully joined
// logits, bit for bit.
template <int G, int NPASS, class Meta>
__device__ inline void consume_own(SoftState<NPASS>& st, const f32x4 (&J)[4], float xs, float xb,
                                   const u32x4 (&vc)[4], const Meta& vm, int a, int col) {
  constexpr int C = 16 / G;
  float pm = -INFINITY;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) pm = fmaxf(pm, J[t][e]);
  pm = fmaxf(pm, dpp_f<0x128, 0xF>(pm, pm));
  pm = fmaf(wave_max_groups(pm), xs, xb);
  const float mn = fmaxf(st.m, pm);
  if (__any(mn > st.m)) {
    const float alpha = (st.m == -INFINITY) ? 0.f : fast_exp2(st.m - mn);
    st.zl *= alpha;
#pragma unroll
    for (int u = 0; u < 8; ++u) st.acc[u] *= alpha;
    st.m = mn;
  }
  const float shift = xb - st.m;
  // own k-steps: lanes < 8 hold k-steps 0, 1 (tiles 0-3), lanes >= 8 k-steps
  // 2, 3. Every lane needs all four: k-step k2 (k2 < 2) is lane col - 8's own
  // in lanes 8-15 of each row (DPP banks 2-3) and k-step 2 + k2 lane col + 8's
  // in lanes 0-7 (banks 0-1); a row rotate by 8 written to those banks only
  // leaves the own value in the others.
  u32x4 pk[4];
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2) {
    half8 ph;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      ph[e] = (_Float16)fast_exp2(fmaf(J[2 * k2 + (e >> 2)][e & 3], xs, shift));   // token pi(ks, a, e)
    u32x4 own;
    __builtin_memcpy(&own, &ph, 16);
    pk[k2].x = dpp_u<0x128, 0xC>(own.x, own.x);
    pk[k2].y = dpp_u<0x128, 0xC>(own.y, own.y);
    pk[k2].z = dpp_u<0x128, 0xC>(own.z, own.z);
    pk[k2].w = dpp_u<0x128, 0xC>(own.w, own.w);
    pk[2 + k2].x = dpp_u<0x128, 0x3>(own.x, own.x);
    pk[2 + k2].y = dpp_u<0x128, 0x3>(own.y, own.y);
    pk[2 + k2].z = dpp_u<0x128, 0x3>(own.z, own.z);
    pk[2 + k2].w = dpp_u<0x128, 0x3>(own.w, own.w);
  }
  const int jl = col / G;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const half8 ph = as_half8(pk[ks]);
    st.zl = mfma(as_half8(vm.za(ks, a, col)), ph, st.zl);
#pragma unroll
    for (int P = 0; P < NPASS; ++P) {
      const int j = (jl + P * C) & 3;
      const half8 s8 = as_half8(vm.s(ks, P, a, j));
      const half8 B = ph * s8;
      const u32x4 v8 = vc[ks] >> 8u;
#pragma unroll
      for (int w2 = 0; w2 < 4; ++w2) {
        if (w2 / C != P) continue;
        st.acc[2 * w2] = mfma(tile2(vc[ks], v8, 2 * w2), B, st.acc[2 * w2]);
        st.acc[2 * w2 + 1] = mfma(tile2(vc[ks], v8, 2 * w2 + 1), B, st.acc[2 * w2 + 1]);
      }
    }
  }
}

// LDS staging area (8 KB) for write_partial: the BF16-segment buffer, free
// once a split's page loop has ended.
template <class Smem>
__device__ inline float* stage_buf(Smem& S) {
  return &S.u.p_lds[0][0];
}

// Write this split's (m, l, out) for the lane's head. Lane (a, col) holds
// rows 4a..4a+3 of all 8 value tiles for column col = (copy jl, head h);
// only tiles of value group jl + P*C are meaningful. The tiles go through
// LDS with static indices (stage: 64 lanes x 32 floats), then every lane
// writes 2 channels of each head's record, coalesced.
// extra (optional): per head, two channels 2 lane, 2 lane + 1 added to the
// output (the full-precision Values of a KIVI FIFO page).
template <int G, int NPASS>
__device__ inline void write_partial(const DecodeArgs& A, SoftState<NPASS>& st, int split, int b, int kvh, int a,
                                     int col, float* stage, const float (*extra)[2] = nullptr) {
  constexpr int C = 16 / G;
  const int lane = threadIdx.x & 63;   // lane within the calling wave
  // sum p (row 4: lane group 1) and sum p * offset of value group j (row j:
  // lane group 0), for the head of this lane's column
  const float l = __shfl(st.zl[0], 16 + col);
  float zg[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) zg[j] = __shfl(st.zl[j], col);
  float z[NPASS];
#pragma unroll
  for (int P = 0; P < NPASS; ++P) {
    const int j = (col / G + P * C) & 3;
    z[P] = j == 0 ? zg[0] : (j == 1 ? zg[1] : (j == 2 ? zg[2] : zg[3]));
  }
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int P = (u >> 1) / C;
#pragma unroll
    for (int e = 0; e < 4; ++e)   // value tiles carry the operand factor 4^(u & 3) * 2^-24
      stage[(col * 8 + u) * 4 * 4 + a * 4 + e] = fmaf(st.acc[u][e], tile_unscale(u), P < NPASS ? z[P] : 0.f);
  }
  __syncthreads();
  const int h = col % G, jl = col / G;
  float* base = A.partial + (((int64_t)split * A.batch + b) * A.n_q_heads + kvh * G) * RECORD;
  // streaming stores: the records are read once, by the combine pass, after
  // the kernel has ended
  if (a == 0 && jl == 0) {
    __builtin_nontemporal_store(st.m, &base[h * RECORD]);
    __builtin_nontemporal_store(l, &base[h * RECORD + 1]);
  }
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int ch = 2 * lane + k;                 // channel = 16 u + 4 a' + e
      const int u = ch >> 4, aa = (ch >> 2) & 3, e = ch & 3;
      const int j = u >> 1, c = (j % C) * G + hh;  // column holding (group j, head hh)
      const float v = stage[(c * 8 + u) * 16 + aa * 4 + e] + (extra ? extra[hh][k] : 0.f);
      __builtin_nontemporal_store(v, &base[hh * RECORD + REC_OUT + ch]);
    }
  }
}


// write_partial without the LDS staging: each lane stores its meaningful
// tiles straight from the accumulators. Lane (a, col), col = (copy jl, head
// h), holds channels 16 u + 4 a .. + 3 of head h for the value tiles u whose
// group u / 2 it covers ((u / 2) % C == jl); each such tile is one 16-byte
// store (the four lane groups fill 64 contiguous bytes of the record), so
// every (head, channel) is written once, with no barrier and no LDS traffic.
template <int G, int NPASS>
__device__ inline void write_partial_direct(const DecodeArgs& A, const SoftState<NPASS>& st, int split, int b,
                                            int kvh, int a, int col) {
  constexpr int C = 16 / G;
  const int h = col % G, jl = col / G;
  const float l = __shfl(st.zl[0], 16 + col);   // row 4 (lane group 1): sum p
  float zg[4];                                   // rows 0-3 (lane group 0): sum p * offset of group j
#pragma unroll
  for (int j = 0; j < 4; ++j) zg[j] = __shfl(st.zl[j], col);
  float* rec = A.partial + (((int64_t)split * A.batch + b) * A.n_q_heads + kvh * G + h) * RECORD;
  if (a == 0 && jl == 0) __builtin_nontemporal_store((f32x2){st.m, l}, reinterpret_cast<f32x2*>(rec));
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int j = u >> 1;
    if (j % C != jl) continue;                   // this lane's column carries another group's scale
    const float z = j == 0 ? zg[0] : (j == 1 ? zg[1] : (j == 2 ? zg[2] : zg[3]));
    const float sc = tile_unscale(u);            // value tiles carry the operand factor 4^(u & 3) * 2^-24
    __builtin_nontemporal_store((f32x4){fmaf(st.acc[u][0], sc, z), fmaf(st.acc[u][1], sc, z),
                                        fmaf(st.acc[u][2], sc, z), fmaf(st.acc[u][3], sc, z)},
                                reinterpret_cast<f32x4*>(rec + REC_OUT + 16 * u + 4 * a));
  }
}

// Key slot operand for k-step ks: B = q * s * 2^-6 (hi/lo), bias += q . z
// (s, z binary16; q * s has at most 8 + 11 significant bits, so hi + lo
// carry it exactly unless it leaves the binary16 range)
__device__ inline void key_operand(const float* qv, const u32x4& sw, const u32x4& zw, half8& hi, half8& lo,
                                   float& bias) {
  const half8 s8 = as_half8(sw), z8 = as_half8(zw);
  float prod[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    prod[e] = qv[e] * (float)s8[e] * B_SCALE;
    bias = fmaf(qv[e], (float)z8[e], bias);
  }
  split8(prod, hi, lo);
}

// Key slot operand from pre-scaled query values (q * 2^-6): B = q * s (hi/lo)
__device__ inline void key_operand_scaled(const float* qv, const u32x4& sw, half8& hi, half8& lo) {
  const half8 s8 = as_half8(sw);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    // q * s is exact in float (8 + 11 bits); both halves are single v_fma_mix
    const _Float16 h = (_Float16)fmaf(qv[e], (float)s8[e], 0.0f);
    hi[e] = h;
    lo[e] = (_Float16)fmaf(qv[e], (float)s8[e], -(float)h);
  }
}

// KIVI Value FIFO on the pipelined kernels (KIVI blog sections 4-5): pages
// from A.fifo_clean on hold tokens whose Values are still in the
// full-precision window. Their page rows are as the Key seal left them
// (codes, scales and offsets zero), so the page's Value pass adds nothing
// for them while their probabilities count in the split's l. Their
// log2-domain logits (J * xs + xb, as the softmax forms them) go to a spare
// partial record of the query head, record A.fifo_wsplit + pg -
// A.fifo_clean, float = token in the page, for the merge to weight the
// window's Values with. After half_join, lanes (col & 7) < G hold head
// col & 7's logits of tiles 0-3 (col < 8) or 4-7 (col >= 8); records are
// 8-byte aligned.
template <int G>
__device__ inline void fifo_store_own(const DecodeArgs& A, int b, int kvh, int pg, const f32x4 (&J)[4], float xs,
                                      float xb, int a, int col) {
  if (pg < A.fifo_clean || (col & 7) >= G) return;
  const int h = col & 7, t0 = col >= 8 ? 4 : 0;
  float* rec = A.partial + ((int64_t)(A.fifo_wsplit + pg - A.fifo_clean) * A.batch * A.n_q_heads +
                            (int64_t)b * A.n_q_heads + kvh * G + h) * RECORD;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    float2* d = reinterpret_cast<float2*>(rec + 16 * (t0 + t) + 4 * a);
    d[0] = make_float2(fmaf(J[t][0], xs, xb), fmaf(J[t][1], xs, xb));
    d[1] = make_float2(fmaf(J[t][2], xs, xb), fmaf(J[t][3], xs, xb));
  }
}

// This lane's half of B = q * s, with qh = binary16(q * 2^-6): the hi part
// binary16(qh s) (columns 0-7) or its rounding error binary16(qh s - hi)
// (columns 8-15, one fused rounding), both as fma(qh, s, binary16(qn s)):
// qn = 0 in columns 0-7 (the exact product rounded once) and qn = -qh in
// columns 8-15 (binary16(-qh s) = -hi, rounding being symmetric), read from
// a table whose head G is zero, so no per-lane select is needed. Packed
// half-precision arithmetic, two slots per instruction.
__device__ inline half8 key_operand_half(const half8& qh, const half8& qn, const u32x4& sw) {
  const half8 s8 = as_half8(sw);
  return __builtin_elementwise_fma(qh, s8, qn * s8);
}

__device__ inline bf16x8 as_bf16x8(const u32x4& v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

// Workgroup -> (batch, kv head, split) of a decode launch (one dimension):
// every page split first, slice by slice, then the BF16-segment workgroups.
// The page splits fill the resident slots; the short segment workgroups are
// dispatched after them and take the slots page splits release.
// Address of logical page p of head `head`: through the page table when
// there is one (the entry clamped into the pool), else contiguous.
__device__ inline const uint8_t* page_ptr(const DecodeArgs& A, int64_t head, int p) {
  if (A.table == nullptr) return A.arena + (head * A.max_pages + p) * A.page_stride;
  const int v = A.table[head * A.table_stride + p];
  return A.arena + (int64_t)min(max(v, 0), A.pool_pages - 1) * A.page_stride;
}

struct DecodeBlock {
  int b, kvh, split;
};
__device__ inline DecodeBlock decode_block(const DecodeArgs& A) {
  const int n_pw = A.batch * A.n_kv_heads * A.n_page_splits;
  int w = blockIdx.x, slice, split;
  if (w < n_pw) {
    slice = w / A.n_page_splits;
    split = w - slice * A.n_page_splits;
  } else {
    w -= n_pw;
    slice = w / A.n_seg_splits;
    split = A.n_page_splits + (w - slice * A.n_seg_splits);
  }
  return {slice / A.n_kv_heads, slice % A.n_kv_heads, split};
}

// BF16 segment (attention sinks + residual): workgroup split - n_page_splits
// takes segment tokens [SEG_TOKENS c, SEG_TOKENS (c + 1)), so the segment's
// memory latency is paid once, in parallel, rather than once per chunk.
// One wave, in chunks of 32 tokens: all Key and Value loads of a chunk are
// issued together; q.k runs on the bf16 MFMA (exact products); each lane
// turns its own 8 logits into probabilities against the running per-head
// maximum and stages them in LDS; p.V runs on the VALU with each lane owning
// two channels of every head. Writes the split's partial record. p_lds needs
// 32 x 8 floats, mh 16.
template <int G>
__device__ inline void bf16_segment(const DecodeArgs& A, int split, int b, int kvh, int lane, float (*p_lds)[8],
                                    float* mh) {
  const int a = lane >> 4, r = lane & 15, col = r, h = col % G;
  const int64_t head = (int64_t)b * A.n_kv_heads + kvh;
  const uint16_t* qrow = A.q + ((int64_t)b * A.n_q_heads + kvh * G + h) * D;
  const int t_lo = SEG_TOKENS * (split - A.n_page_splits);
  const int T = min(A.n_sink + A.n_resid, t_lo + SEG_TOKENS);   // end of this workgroup's tokens
  bf16x8 Bq[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    u32x4 raw = ld16(reinterpret_cast<const uint8_t*>(qrow + 32 * ks + 8 * a));
    __builtin_memcpy(&Bq[ks], &raw, 16);
  }
  float m_run = -INFINITY;                   // running max of this lane's head (log2 domain)
  float o[G][2], lsum[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) o[hh][0] = o[hh][1] = lsum[hh] = 0.f;
  for (int t0 = t_lo; t0 < T; t0 += 32) {
    // Unconditional loads (straight-line issue, one wait): a token past T
    // reads token T-1 again; its logit is -inf, so its probability is 0 and
    // its finite row adds nothing.
    u32x4 kr[2][4];
    uint32_t vr[32];
#pragma unroll
    for (int i2 = 0; i2 < 2; ++i2) {
      const int t = min(t0 + 16 * i2 + r, T - 1);   // A row = token
      const uint16_t* krow = t < A.n_sink ? A.sink_k + (head * A.n_sink + t) * D
                                          : A.resid_k + (head * A.resid_stride + (t - A.n_sink)) * D;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kr[i2][ks] = ld16(reinterpret_cast<const uint8_t*>(krow + 32 * ks + 8 * a));
    }
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const int t = min(t0 + j, T - 1);
      const uint16_t* vrow = t < A.n_sink ? A.sink_v + (head * A.n_sink + t) * D
                                          : A.resid_v + (head * A.resid_v_stride + (t - A.n_sink)) * D;
      vr[j] = reinterpret_cast<const uint32_t*>(vrow)[lane];
    }
    float x[2][4];
    float cm = -INFINITY;
#pragma unroll
    for (int i2 = 0; i2 < 2; ++i2) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        bf16x8 Ak;
        __builtin_memcpy(&Ak, &kr[i2][ks], 16);
        acc = mfma_bf(Ak, Bq[ks], acc);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int tok = t0 + 16 * i2 + 4 * a + e;
        x[i2][e] = tok < T ? acc[e] * A.scale_log2 : -INFINITY;
        cm = fmaxf(cm, x[i2][e]);
      }
    }
    const float m_new = fmaxf(m_run, wave_max_groups(cm));   // finite: the chunk has a token
    const float alpha = m_run == -INFINITY ? 0.f : fast_exp2(m_run - m_new);
    m_run = m_new;
    if (col < G) {
#pragma unroll
      for (int i2 = 0; i2 < 2; ++i2)
#pragma unroll
        for (int e = 0; e < 4; ++e) p_lds[16 * i2 + 4 * a + e][col] = fast_exp2(x[i2][e] - m_new);
      if (a == 0) mh[col] = alpha;
    }
    __syncthreads();
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const float al = mh[hh];
      o[hh][0] *= al;
      o[hh][1] *= al;
      lsum[hh] *= al;
    }
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const float v0 = lo_bf(vr[j]), v1 = hi_bf(vr[j]);
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float pp = p_lds[j][hh];
        o[hh][0] = fmaf(pp, v0, o[hh][0]);
        o[hh][1] = fmaf(pp, v1, o[hh][1]);
        lsum[hh] += pp;
      }
    }
    __syncthreads();
  }
  if (a == 0 && col < G) mh[8 + col] = m_run;
  __syncthreads();
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    float* rec = A.partial + (((int64_t)split * A.batch + b) * A.n_q_heads + kvh * G + hh) * RECORD;
    if (lane == 0) {
      rec[0] = mh[8 + hh];
      rec[1] = lsum[hh];
    }
    rec[REC_OUT + 2 * lane] = o[hh][0];
    rec[REC_OUT + 2 * lane + 1] = o[hh][1];
  }
}

}  // namespace kvq
