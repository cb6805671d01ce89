// Internal definitions shared by the libkvq translation units: page geometry,
// bf16/f16 helpers and the exact-rounding primitives the flush kernels use.
// gfx950 (CDNA4) only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kvq.h"

namespace kvq {

constexpr int D = 128;            // head dimension
constexpr int PAGE = 128;         // tokens per page (Key group along time)
constexpr int GV = 32;            // value channels per group
constexpr int V_CODE_BYTES = 4096;
constexpr int V_META_BYTES = 2048;

__host__ __device__ inline int round_up(int x, int m) { return (x + m - 1) / m * m; }

// ---------------------------------------------------------------- geometry
// MixKVQ page: [K_BF16 | K_CODES | K_META | V_CODES | V_META]
//  K_BF16 : n16 channel rows of 256 B, token 16*i + r at byte 16*r + 2*i
//  K_CODES: fragments of 8 slots x 128 tokens x 2 bits (256 B); slots are
//           the low/high halves of every UINT4 code (padded to a multiple of
//           8 slots) followed by the UINT2 codes
//  K_META : per fragment 8 binary16 slot scales then 8 binary16 slot offsets
struct MixGeo {
  int n16, n4, n2, s4, n_slots, F, off_codes, off_meta, off_v, used, stride;
};
__host__ __device__ inline MixGeo mix_geo(int n16, int n4) {
  MixGeo g;
  g.n16 = n16;
  g.n4 = n4;
  g.n2 = D - n16 - n4;
  g.s4 = round_up(2 * n4, 8);
  g.n_slots = g.s4 + g.n2;
  g.F = (g.n_slots + 7) / 8;
  g.off_codes = 256 * n16;
  g.off_meta = g.off_codes + 256 * g.F;
  g.off_v = g.off_meta + 32 * g.F;
  g.used = g.off_v + V_CODE_BYTES + V_META_BYTES;
  g.stride = round_up(g.used, 256);
  return g;
}

// PN-Mix page: [LSB plane (2048) | UP plane | K_META (512) | V_CODES | V_META]
struct PnGeo {
  int n_hi, n_up_frag, off_up, off_meta, off_v, used, stride;
};
__host__ __device__ inline PnGeo pn_geo(int n_hi) {
  PnGeo g;
  g.n_hi = n_hi;
  g.n_up_frag = (n_hi + 7) / 8;
  g.off_up = 2048;
  g.off_meta = g.off_up + 256 * g.n_up_frag;
  g.off_v = g.off_meta + 512;
  g.used = g.off_v + V_CODE_BYTES + V_META_BYTES;
  g.stride = round_up(g.used, 256);
  return g;
}

// QJL page: [sign bits (16*(m + mo)) | norms (256) | outlier norms (256, mo > 0) | V_CODES | V_META];
// with the outlier split (mo > 0) sign rows m .. m + mo - 1 are the outlier instance's
struct QjlGeo {
  int m, mo, off_norm, off_norm_o, off_v, used, stride;
};
__host__ __device__ inline QjlGeo qjl_geo(int m, int mo = 0) {
  QjlGeo g;
  g.m = m;
  g.mo = mo;
  g.off_norm = 16 * (m + mo);
  g.off_norm_o = g.off_norm + 256;
  g.off_v = g.off_norm + (mo ? 512 : 256);
  g.used = g.off_v + V_CODE_BYTES + V_META_BYTES;
  g.stride = round_up(g.used, 256);
  return g;
}

constexpr int MIX_RECORD = 160;   // channel order u8[128] + 2-bit tiers [32]

// Tier counts a MixKVQ record holds in its 2-bit codes (2 = BF16, 1 = UINT4):
// with threshold tiers every head has its own counts, and its pages are laid
// out by them. rec must be 4-byte aligned.
__device__ inline void mix_record_counts(const uint8_t* rec, int& n16, int& n4) {
  const uint32_t* tw = reinterpret_cast<const uint32_t*>(rec + 128);
  int c2 = 0, c1 = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t w = tw[i], hi = (w >> 1) & 0x55555555u, lo = w & 0x55555555u;
    c2 += __builtin_popcount(hi & ~lo);
    c1 += __builtin_popcount(lo & ~hi);
  }
  n16 = c2;
  n4 = c1;
}
constexpr int PN_RECORD = 8;      // 64 pair bits
constexpr int QJL_RECORD = 16;    // outlier-channel bits (QJL outlier split)

// ---------------------------------------------------------------- number formats
__host__ __device__ inline float bf16_to_f32(uint16_t b) {
  union { uint32_t u; float f; } c;
  c.u = (uint32_t)b << 16;
  return c.f;
}
__host__ __device__ inline double bf16_to_f64(uint16_t b) { return (double)bf16_to_f32(b); }

// Correctly rounded (ties-to-even) IEEE binary16 of a double: subnormals
// down to 2^-24, +-infinity past the largest finite value (65504), and +0.0
// for a result that rounds to zero. A non-finite input maps to infinity of
// its sign (NaN is not produced here: callers flag non-finite groups).
__host__ __device__ inline uint16_t f64_to_f16_rne(double v) {
  union { double d; uint64_t u; } c;
  c.d = v;
  const uint64_t u = c.u;
  const uint16_t sign = (uint16_t)((u >> 48) & 0x8000);
  const int ef = (int)((u >> 52) & 0x7FF);
  if (ef == 0x7FF) return (uint16_t)(sign | 0x7C00);
  if (v == 0.0 || ef == 0) return 0;                      // zero and double subnormals (far below 2^-25)
  const int e = ef - 1023;
  if (e > 15) return (uint16_t)(sign | 0x7C00);
  const uint64_t sig = (u & 0xFFFFFFFFFFFFFull) | (1ull << 52);   // value = sig * 2^(e-52)
  const int q_exp = e >= -14 ? e - 10 : -24;             // exponent of the result quantum
  const int shift = q_exp - (e - 52);                    // >= 42
  uint64_t q;
  if (shift >= 64) {
    q = 0;
  } else {
    q = sig >> shift;
    const uint64_t rem = sig & ((1ull << shift) - 1);
    const uint64_t half = 1ull << (shift - 1);
    if (rem > half || (rem == half && (q & 1))) q += 1;
  }
  if (q == 0) return 0;
  if (e >= -14) {
    int ex = e;
    if (q == 2048) { q = 1024; ex += 1; }
    if (ex > 15) return (uint16_t)(sign | 0x7C00);
    return (uint16_t)(sign | ((uint16_t)(ex + 15) << 10) | (uint16_t)(q - 1024));
  }
  return (uint16_t)(sign | (uint16_t)q);   // q == 1024 encodes the smallest normal
}

__host__ __device__ inline double f16_to_f64(uint16_t h) {
  const int e = (h >> 10) & 0x1F, m = h & 0x3FF;
  const double s = (h & 0x8000) ? -1.0 : 1.0;
  if (e == 0x1F) return m ? NAN : s * INFINITY;
  if (e == 0) return s * (double)m * 0x1p-24;
  return s * (double)(1024 + m) * __builtin_ldexp(1.0, e - 25);
}

// binary16 bit pattern of the correctly rounded sqrt(s) for an exact s >= 0
// given in double. Midpoints are decided on their squares (exact in double).
__device__ inline uint16_t sqrt_to_f16_rne(double s) {
  if (s <= 0.0) return 0;
  double r = sqrt(s);
  _Float16 h = (_Float16)(float)r;   // candidate, fixed below
  uint16_t c;
  __builtin_memcpy(&c, &h, 2);
  for (int it = 0; it < 4; ++it) {
    _Float16 hv, hu, hd;
    uint16_t cu = (uint16_t)(c + 1), cd = (uint16_t)(c - 1);
    __builtin_memcpy(&hv, &c, 2);
    __builtin_memcpy(&hu, &cu, 2);
    __builtin_memcpy(&hd, &cd, 2);
    double v = (double)(float)hv;
    if (c < 0x7BFF) {
      double mid = 0.5 * (v + (double)(float)hu);
      double m2 = mid * mid;                 // 13-bit mid -> exact square
      if (s > m2 || (s == m2 && (c & 1))) { c = cu; continue; }
    }
    if (c > 0) {
      double mid = 0.5 * (v + (double)(float)hd);
      double m2 = mid * mid;
      if (s < m2 || (s == m2 && (c & 1))) { c = cd; continue; }
    }
    break;
  }
  return c;
}

__host__ __device__ inline int bf16_exp_field(uint16_t b) { return (b >> 7) & 0xFF; }

// ---------------------------------------------------------------- kernel argument blocks
// Flush (kvq_flush.hip): source rows, selection records, arena geometry.
struct FlushArgs {
  const uint16_t* k_src;
  const uint16_t* v_src;
  int64_t src_stride;
  const uint8_t* mask;
  const uint16_t* qjl_s;
  uint8_t* arena;
  int64_t page_stride;
  const int32_t* table;           // pool index of logical page p of head h: table[h * table_stride + p]; null: contiguous
  int table_stride;
  int pool_pages;                 // pages in the arena: batch * n_kv_heads * max_pages
  int max_pages;
  int first_page;
  int n_pages;                    // pages written per (batch, kv head)
  int units;                      // pages written in all: n_pages * n_kv_heads * batch
  int n_kv_heads;
  int n16, n4;
  int n_hi;
  int pair_layout;
  int qjl_m;
  int qjl_mo;                     // outlier-instance sketch rows (0: no outlier split)
  unsigned* flags;
  const void* q_accum;            // MixKVQ reselection: query sums (128-bit) per (head, channel); null: the mask records
  uint8_t* rec_out;               // with q_accum: record of logical page p of head h at rec_out + (h rec_stride + p) * 160
  int rec_stride;
  int head_tiers;                 // MixKVQ threshold tiers: each head's counts come from its record (n16, n4: capacities)
  int keys_only;                  // KIVI Value FIFO: seal the Keys, zero the Value part (rows arrive by value push)
  int push_first, push_rows;      // value push: tokens push_first .. push_first + push_rows - 1 of every head
};
struct SelectArgs {
  const uint16_t* q;
  const uint16_t* k;
  int64_t l_q, q_stride, l_k, k_stride;
  int n_q_heads, n_kv_heads;
  int n16, n4;
  int n_hi_pairs, pair_layout;
  int n_out;                      // QJL: outlier channels
  uint8_t* out;
  int threshold;                  // MixKVQ: tiers by the salience thresholds (n16, n4: capacities)
  double tau_bf16, tau_u4;
};
struct DecodeArgs {
  const uint16_t* q;
  const uint8_t* arena;
  int64_t page_stride;
  const int32_t* table;           // as FlushArgs::table
  int table_stride;
  int pool_pages;
  int max_pages, n_pages, pps, n_page_splits;
  int n_seg_splits;               // BF16-segment workgroups per (batch, kv head), SEG_TOKENS tokens each
  int rec_stride;                 // 0: one record per head; > 0: record of page p of head h at mask + (h rec_stride + p) * 160
  const uint8_t* mask;
  const float* sq;
  const uint16_t* sink_k;
  const uint16_t* sink_v;
  int n_sink;
  const uint16_t* resid_k;
  const uint16_t* resid_v;
  int n_resid, resid_stride;
  int resid_v_stride;             // row stride of resid_v (resid_stride, or the Value window's in FIFO decodes)
  int vq_end;                     // KIVI Value FIFO: tokens from vq_end on take their Value from vwin (else INT32_MAX)
  const uint16_t* vwin;           // [batch][n_kv_heads][vwin_stride][128] bf16: Value of token vq_end + j at row j
  int vwin_stride;
  float scale_log2;
  float qjl_coef;
  float* partial;                 // [n_splits][B][Hq][RECORD]: m, l, unused, out[128] (from REC_OUT)
  float* out;                     // [B][Hq][128]
  int batch, n_kv_heads, n_q_heads;
  int n16, n4;
  int n_hi, pair_layout;
  int qjl_m;
  int qjl_mo;                     // as FlushArgs::qjl_mo; the estimate's outlier term is scaled by qjl_m / qjl_mo
  int head_tiers;                 // as FlushArgs::head_tiers
  int fifo_clean;                 // FIFO on the pipelined kernels: pages from here on hold window tokens
  int fifo_wsplit;                // ... whose logits go to partial record fifo_wsplit + page - fifo_clean
};

hipError_t launch_flush(int key_mode, const FlushArgs& a, int batch, hipStream_t stream);
hipError_t launch_value_push(int key_mode, const FlushArgs& a, int batch, hipStream_t stream);
hipError_t launch_select(int key_mode, const SelectArgs& a, int batch, hipStream_t stream);
hipError_t launch_accumulate(const SelectArgs& a, void* acc, int batch, hipStream_t stream);
// with_merge false: the split kernels only; the caller launches the merge
// (launch_merge_flush) with the same DecodeArgs
// path: kvq_decode_path. A pipelined kernel may choose its own split count:
// a.pps and a.n_page_splits are updated to what was launched (the merge that
// follows, in the call or from the caller, uses them).
hipError_t launch_decode(int key_mode, DecodeArgs& a, const uint16_t* qjl_s, hipStream_t s, bool with_merge,
                         int path);
int decode_parts(const DecodeArgs& a);
hipError_t launch_merge_flush(int key_mode, const DecodeArgs& d, const FlushArgs& f, int batch, hipStream_t s);
constexpr int RECORD = 144;       // partial record per query head: m, l, 14 unused, out[128]
constexpr int REC_OUT = 16;       // out[] offset: records and out[] are 64-byte aligned (whole-line stores)
constexpr int DECODE_SLOTS = 2048;
// Sink + residual tokens per BF16-segment workgroup; at most 256 segment
// tokens (128 sinks + 128 residual) make MAX_SEG_SPLITS workgroups.
constexpr int SEG_TOKENS = 32;
constexpr int MAX_SEG_SPLITS = 2 * PAGE / SEG_TOKENS;
inline int seg_splits(int n_tokens) { return (n_tokens + SEG_TOKENS - 1) / SEG_TOKENS; }
int decode_pages_per_split(int n_pages, int batch, int n_kv_heads);
int mix_max_fragments(int n16, int n4, bool head_tiers);
int decode_pages_per_split_slots(int n_pages, int batch, int n_kv_heads, int slots);

}  // namespace kvq
