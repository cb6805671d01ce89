// Software-pipelined decode kernels for the common shapes (GQA group 4 or 8,
// the workloads' Key layouts). Same arithmetic as the generic kernel in
// kvq_decode.hip (see there for the method and the MFMA conventions); what
// differs is the memory pipeline and the MFMA column layout:
//  * every loop index is a compile-time constant (templates on the number
//    of Key k-steps and BF16-tier loads), so no runtime selects remain;
//  * MFMA columns 0-7 carry the f16 hi part of the Key operand and columns
//    8-15 the lo part, so one MFMA per tile covers both halves; the partial
//    logits are joined across lanes col and col ^ 8 (DPP);
//  * while page p is computed, page p+1 is in flight. PN-Mix and QJL split
//    the next page into a Key part (codes + metadata, requested before the
//    Key phase) and a value part (requested between the phases, into the
//    registers the previous value phase released); every load is
//    unconditional and the metadata reaches LDS through registers, which
//    keeps the compiler's wait counts exact. MixKVQ, whose larger Key part
//    leaves no registers for that, copies its metadata straight into a
//    double-buffered LDS slot with global_load_lds_dwordx4 and prefetches
//    its codes into registers, one wait per page;
//  * the first page's loads are issued before the per-split set-up (query
//    staging, slot tables), so set-up and the first memory latency overlap;
//  * LDS holds only what one split needs (about 14 KB for GQA group 8), so
//    eight single-wave workgroups stay resident per CU.
// LDS metadata slot of a page: [0, 1024) Key meta (MixKVQ, PN-Mix) or norms
// (QJL), [1024, 3072) value meta.
#include "kvq_decode_common.h"

namespace kvq {

typedef __attribute__((address_space(3))) void* lds_void_ptr;

__device__ inline void async16(const uint8_t* src, uint8_t* lds_base) {
  __builtin_amdgcn_global_load_lds(src, (lds_void_ptr)lds_base, 16, 0, 0);
}

// Buffer resource over [base, base + bytes): a buffer load at an offset past
// the range returns zero without a memory request, so loads of absent
// fragments / rows stay unconditional (exact wait counts) and cost no
// traffic. bytes is a multiple of 16 at every use.
__device__ inline __amdgpu_buffer_rsrc_t range_rsrc(const uint8_t* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), 0, bytes, 0x00020000);
}
__device__ inline u32x4 ld16_in(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ inline void async16_in(__amdgpu_buffer_rsrc_t r, int off, uint8_t* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_ptr)lds_base, 16, off, 0, 0, 0);
}

// Where a split's pages are. PAGED false: contiguous from the split's first
// page. PAGED true: through the page table, lane i of register j holding the
// pool index of page p0 + 64 j + i (np <= 64 NT; range-limited loads, lanes
// past np read zero), clamped into the pool; page `it` (uniform) is then one
// lane read away.
template <bool PAGED, int NT = 1>
struct PageSet {
  const uint8_t* base;
  int64_t stride;
  int tab[NT];
  __device__ const uint8_t* at(int it) const {
    if constexpr (PAGED) {
      const int t = NT == 1 || it < 64 ? __builtin_amdgcn_readlane(tab[0], it)
                                       : __builtin_amdgcn_readlane(tab[NT - 1], it - 64);
      return base + (int64_t)t * stride;
    } else {
      return base + (int64_t)it * stride;
    }
  }
};
template <bool PAGED, int NT = 1>
__device__ inline PageSet<PAGED, NT> page_set(const DecodeArgs& A, int64_t head, int p0, int np, int lane) {
  static_assert(NT == 1 || NT == 2, "up to 128 pages per split");
  PageSet<PAGED, NT> s;
  s.stride = A.page_stride;
  if constexpr (PAGED) {
    const auto r = range_rsrc(reinterpret_cast<const uint8_t*>(A.table + head * A.table_stride + p0), 4 * np);
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int v = (int)__builtin_amdgcn_raw_buffer_load_b32(r, 4 * (lane + 64 * j), 0, 0);
      s.tab[j] = min(max(v, 0), A.pool_pages - 1);
    }
    s.base = A.arena;
  } else {
#pragma unroll
    for (int j = 0; j < NT; ++j) s.tab[j] = 0;
    s.base = A.arena + (head * A.max_pages + p0) * A.page_stride;
  }
  return s;
}

// Wait until at most N vector-memory operations of this wave are in flight.
// Emitted through the builtin (not inline asm) so that the compiler's own
// wait insertion knows which loads have completed: otherwise, with an
// asynchronous LDS copy in flight, it drains every load before the first use
// of a register loaded earlier. gfx9 encoding: vmcnt in bits 3:0 and 15:14,
// expcnt (7) and lgkmcnt (15) left at "no wait".
template <int N>
__device__ inline void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Wait for this wave's LDS operations (orders plain LDS stores before an
// asynchronous global->LDS copy into the same bytes).
__device__ inline void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

__device__ inline u32x4 lds16(const uint8_t* p) { return *reinterpret_cast<const u32x4*>(p); }

constexpr int META_SLOT = 3072;

// Wave priority by progress through the split: waves with more pages left
// issue first, so the two waves sharing a SIMD tend to finish together
// rather than one running alone (with no latency hiding) at the end.
__device__ inline void progress_prio(int it, int np) {
  const int q = (4 * it) / (np > 0 ? np : 1);
  if (q == 0) __builtin_amdgcn_s_setprio(3);
  else if (q == 1) __builtin_amdgcn_s_setprio(2);
  else if (q == 2) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

// Shared memory of the MixKVQ / PN-Mix kernels. The page-loop tables and the
// BF16-segment / partial staging buffer (8 KB) share one union; the bf16
// query is staged in the value-meta half of slot 1 during set-up.
template <int G, int NKS>
struct PgSmem {
  union {
    struct {
      half8 qh[NKS][4][G];         // [k-step][lane group][head]: binary16 q * 2^-6 of the slot's channel
      half8 qz[NKS][4][G];         // q of the slot's channel as binary16 (offset MFMA operand)
      half8 qn[NKS][4][G + 1];     // -qh, and zero at head G (the Key operand's correction term)
      uint8_t meta[2][META_SLOT];  // double-buffered page metadata
    } pg;
    float p_lds[256][8];
  } u;
  int slot_ch[32 * NKS];
  float mh[16];
  ZConst zc;                     // constant rows of the offset MFMA operand
};

// Shared memory of the MixKVQ kernel. The page metadata lives in six
// separate 1 KB arrays (MixMeta), one per asynchronous copy: distinct LDS
// objects let the compiler see that a copy in flight for the next page does
// not alias this page's metadata, so its waits stay exact.
template <int G, int NKS>
struct MixSmem {
  union {
    struct {
      half8 qh[NKS][4][G];         // [k-step][lane group][head]: binary16 q * 2^-6 of the slot's channel
      half8 qz[NKS][4][G];         // q of the slot's channel as binary16 (offset MFMA operand)
      half8 qn[NKS][4][G + 1];     // -qh, and zero at head G (the Key operand's correction term)
    } pg;
    float p_lds[256][8];
  } u;
  float mh[16];
  ZConst zc;                     // constant rows of the offset MFMA operand
};

template <int G, int NK = 8>
struct QjSmem {
  union {
    struct {
      half8 bq[2][NK][4][G];       // S q hi/lo [k-step][lane group][head]
      uint8_t meta[2][META_SLOT];
    } qj;
    float p_lds[256][8];
  } u;
  float mh[16];
  ZConst zc;                     // constant rows of the offset MFMA operand
};

// value meta (2048 B) of a page -> LDS slot + 1024: two async loads
__device__ inline void issue_vmeta(const uint8_t* vmeta_g, uint8_t* slot, int lane) {
  async16(vmeta_g + 16 * lane, slot + 1024);
  async16(vmeta_g + 1024 + 16 * lane, slot + 2048);
}

// query heads kvh*G .. kvh*G+G-1 of batch b as 16-byte chunks (8 bf16), G/4 per lane
template <int G>
__device__ inline void load_q(const DecodeArgs& A, int b, int kvh, int lane, u32x4 (&qv)[G / 4]) {
  const uint8_t* qg = reinterpret_cast<const uint8_t*>(A.q + ((int64_t)b * A.n_q_heads + kvh * G) * D);
#pragma unroll
  for (int j = 0; j < G / 4; ++j) qv[j] = ld16(qg + 16 * (lane + 64 * j));
}

template <int G>
__device__ inline void stage_q(const u32x4 (&qv)[G / 4], uint8_t* qb, int lane) {
#pragma unroll
  for (int j = 0; j < G / 4; ++j) *reinterpret_cast<u32x4*>(qb + 16 * (lane + 64 * j)) = qv[j];
}

__device__ inline float qb_at(const uint8_t* qb, int h, int ch) {
  return bf16_to_f32(reinterpret_cast<const uint16_t*>(qb)[h * D + ch]);
}

// A page's metadata in registers: 16 bytes of Key meta (or norms) and 32
// bytes of value meta per lane, written to an LDS slot by commit_meta.
__device__ inline void load_vmeta(u32x4 (&m)[3], const uint8_t* vmeta_g, int lane) {
  m[1] = ld16(vmeta_g + 16 * lane);
  m[2] = ld16(vmeta_g + 1024 + 16 * lane);
}

__device__ inline void commit_meta(const u32x4 (&m)[3], uint8_t* slot, int lane) {
  *reinterpret_cast<u32x4*>(slot + 16 * lane) = m[0];
  *reinterpret_cast<u32x4*>(slot + 1024 + 16 * lane) = m[1];
  *reinterpret_cast<u32x4*>(slot + 2048 + 16 * lane) = m[2];
}

// ------------------------------------------------------------------ page loop
// Two register sets per part, used alternately: the Key part of page p+1
// (codes + metadata) is requested before page p's Key phase, the Value part
// (value codes) between page p's Key and Value phases, i.e. into registers
// that page p-1's Value phase has just released. Each part is in flight for
// about one page of compute, and only one Value set is live in the Key phase.
// Every load is unconditional (same count per page), which keeps the
// compiler's wait counts exact. page(k, v, slot, p, mid): p is the page's
// index in the split.
template <class KP, class VP, class LK, class LV, class PG>
__device__ inline void page_loop(int np, KP (&k)[2], VP (&v)[2], LK load_k, LV load_v, PG page) {
  for (int it = 0; it < np; it += 2) {
    progress_prio(it, np);
    if (it + 1 < np) load_k(k[1], it + 1);
    page(k[0], v[0], 0, it, [&] {
      if (it + 1 < np) load_v(v[1], it + 1);
    });
    if (it + 1 >= np) break;
    if (it + 2 < np) load_k(k[0], it + 2);
    page(k[1], v[1], 1, it + 1, [&] {
      if (it + 2 < np) load_v(v[0], it + 2);
    });
  }
}

struct ValCodes {
  u32x4 vc[4];
};

__device__ inline void load_vcodes(ValCodes& v, const uint8_t* page, int off_v, int a, int r) {
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) v.vc[ks] = ld16(page + off_v + 1024 * ks + 256 * a + 16 * r);
}

// ------------------------------------------------------------------ MixKVQ
template <int NKS, int NB>
struct MixCodes {
  u32x4 kc[NKS];
  u32x4 vc[4];
  u32x4 bf[NB > 0 ? NB : 1];
};

// The metadata slot of one page: Key meta, value meta of k-steps 0-1 and 2-3.
struct MixSlot {
  uint8_t* k;
  uint8_t* v_lo;
  uint8_t* v_hi;
};

// Every load is unconditional, so the issue is straight-line code the
// compiler counts exactly (a conditional load makes it wait for everything in
// flight). Fragments past F and BF16 rows past n16 are read through range-
// limited buffer resources: they load as zero (zero codes, zero BF16 values)
// and request nothing from memory.
template <int NKS, int NB>
__device__ inline void mix_load(MixCodes<NKS, NB>& c, const uint8_t* page, const MixGeo& g, int a, int r) {
  const auto rk = range_rsrc(page + g.off_codes, 256 * g.F);
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) c.kc[ks] = ld16_in(rk, 256 * (4 * ks + a) + 16 * r);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) c.vc[ks] = ld16(page + g.off_v + 1024 * ks + 256 * a + 16 * r);
  const auto rb = range_rsrc(page, 256 * g.n16);
#pragma unroll
  for (int e = 0; e < NB; ++e) c.bf[e] = ld16_in(rb, 256 * (8 * a + e) + 16 * r);
}

// Key meta: the page's 32 F bytes into the first 1 KB of the slot, the rest
// of that 1 KB zero (range-limited copy: zero scales and offsets past F).
__device__ inline void mix_issue_meta(const uint8_t* page, const MixSlot& slot, const MixGeo& g, int lane) {
  async16_in(range_rsrc(page + g.off_meta, 32 * g.F), 16 * lane, slot.k);
  async16(page + g.off_v + V_CODE_BYTES + 16 * lane, slot.v_lo);
  async16(page + g.off_v + V_CODE_BYTES + 1024 + 16 * lane, slot.v_hi);
}

// win(J, xb): sees the page's logits as half_join leaves them (log2 domain:
// J * xs + xb) before the softmax takes them (the FIFO's window logits);
// NoLogits ignores them.
struct NoLogits {
  __device__ inline void operator()(const f32x4 (&)[4], float) const {}
};
// NQ = 4: Bq[k] is the BF16-tier operand of the tiles i with i & 3 = k,
// scaled like their code operands, and the tile factor is undone after the
// join on the lane's 16 logits. NQ = 1 (fewer registers, for the per-page
// record variant): Bq[0] in true units, the factor undone on all 32 raw
// logits before the BF16 tier is added.
template <int G, int NKS, int NB, int NPASS, int NQ, class Win>
__device__ inline void mix_page(SoftState<NPASS>& st, const MixCodes<NKS, NB>& c, const MixSlot& slot,
                                const MixSmem<G, NKS>& S, const bf16x8 (&Bq)[NQ], float xs, float scale_log2, int a,
                                int h, int col, Win win) {
  f32x4 logit[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) logit[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
  f32x4 zacc = {0.f, 0.f, 0.f, 0.f};       // sum_slot q * offset, identical in every row
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    const uint8_t* km = slot.k + 32 * (4 * ks + a);   // past F: zero meta
    const u32x4 sw = lds16(km), zw = lds16(km + 16);
    const half8 B = key_operand_half(S.u.pg.qh[ks][a][h], S.u.pg.qn[ks][a][col >= 8 ? h : G], sw);
    zacc = mfma(as_half8(zw), S.u.pg.qz[ks][a][h], zacc);
    const u32x4 k8 = c.kc[ks] >> 8u;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      logit[2 * w] = mfma(tile2(c.kc[ks], k8, 2 * w), B, logit[2 * w]);
      logit[2 * w + 1] = mfma(tile2(c.kc[ks], k8, 2 * w + 1), B, logit[2 * w + 1]);
    }
  }
  // the code operands carry 4^(i & 3) * 2^-24
  if constexpr (NQ == 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i) logit[i] *= tile_unscale(i);
  }
  if constexpr (NB > 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint16_t tmp[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        tmp[e] = e < NB ? (uint16_t)(rd(c.bf[e < NB ? e : 0], i >> 1) >> (16 * (i & 1))) : (uint16_t)0;
      bf16x8 Ak;
      __builtin_memcpy(&Ak, tmp, 16);
      logit[i] = mfma_bf(Ak, Bq[NQ == 4 ? (i & 3) : 0], logit[i]);   // Bq is zero in the lo columns
    }
  }
  f32x4 J[4];
  half_join(logit, J, col < 8);
  if constexpr (NQ == 4) {
#pragma unroll
    for (int t = 0; t < 4; ++t) J[t] *= tile_unscale(t);   // tiles t and t + 4 carry the same factor
  }
  win(J, zacc[0] * scale_log2);
  consume_own<G, NPASS>(st, J, xs, zacc[0] * scale_log2, c.vc, VMetaAt{slot.v_lo, slot.v_hi, S.zc.ptr()}, a, col);
}

// The record's tables for the page loop: slot -> channel of this lane's slots
// and the BF16-tier channels of its lane group (bytes of the record, one
// dword per lane in recw), the query of each slot's channel per head into
// S.u.pg (q * 2^-6 as the Key operand, binary16 q as the offset operand) and
// the BF16-tier operands Bq4. The staged bf16 query rows qb are read first,
// then the tables written: interleaved, each read would wait for the writes
// before it.
// NE: BF16-tier elements a lane group can hold (0, 1 or 8: the kernel's NB),
// the rest of Bq left zero.
template <int G, int NKS, int NQ, int NE>
__device__ inline void mix_tables(uint32_t recw, const MixGeo& g, const uint8_t* qb, MixSmem<G, NKS>& S,
                                  bf16x8 (&Bq)[NQ], int lane, int a, int h, int col) {
  constexpr int NJ = (32 * NKS + 63) / 64;
  int sch[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int s = lane + 64 * j;
    int idx = -1;
    if (s < 2 * g.n4) idx = g.n16 + (s >> 1);
    else if (s >= g.s4 && s < g.s4 + g.n2) idx = g.n16 + g.n4 + (s - g.s4);
    const int ch = rec_byte(recw, idx < 0 ? 0 : idx);
    sch[j] = idx < 0 ? -1 : ch;
  }
  int bch[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int ch = e < NE ? rec_byte(recw, 8 * a + e) : 0;
    bch[e] = e < NE && 8 * a + e < g.n16 ? ch : -1;
  }
  float qsl[NJ][G], qbf[8];
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int hh = 0; hh < G; ++hh) qsl[j][hh] = qb_at(qb, hh, sch[j] >= 0 ? sch[j] : 0);
#pragma unroll
  for (int e = 0; e < 8; ++e) qbf[e] = e < NE ? qb_at(qb, h, bch[e] >= 0 ? bch[e] : 0) : 0.f;
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int s = lane + 64 * j;
    if (s < 32 * NKS) {
      const int ks = s >> 5, aa = (s >> 3) & 3, e = s & 7;
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float qf = sch[j] >= 0 ? qsl[j][hh] : 0.f;
        const _Float16 qhv = (_Float16)(qf * B_SCALE);   // exact unless |q| < 2^-11
        S.u.pg.qh[ks][aa][hh][e] = qhv;
        S.u.pg.qn[ks][aa][hh][e] = -qhv;
        S.u.pg.qz[ks][aa][hh][e] = (_Float16)qf;   // exact for bf16 q inside the binary16 range
      }
    }
  }
  if (lane < 4 * NKS) S.u.pg.qn[lane >> 2][lane & 3][G] = half8{};
  // the BF16-tier operand: q * 2^-6, for NQ = 4 also times 4^k * 2^-24 for the
  // tiles with i & 3 = k (exact power-of-two scalings of the bf16 query)
#pragma unroll
  for (int k = 0; k < NQ; ++k)
#pragma unroll
    for (int e = 0; e < 8; ++e)
      Bq[k][e] = e < NE ? (__bf16)(bch[e] >= 0 && col < 8 ? qbf[e] * (NQ == 4 ? B_SCALE / tile_unscale(k) : B_SCALE) : 0.f)
                        : (__bf16)0.f;
}

// Registers of 256 VGPRs (two waves per SIMD) fit every variant except the
// eight-channel BF16 tier, which keeps one wave per SIMD rather than spill.
// PREC: every page has its own record (per-flush reselection). Page p's
// record dword comes with the page's loads; its tables are rebuilt at the
// top of the page, after the wait that covers them. FIFO: the KIVI Value
// FIFO's window pages store their logits (fifo_store_own).
template <int G, int NKS, int NB, bool PAGED, bool PREC, bool FIFO>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(NB == 8 ? 1 : 2))) void decode_mix_fast(
    DecodeArgs A) {
  constexpr int C = 16 / G;
  constexpr int NPASS = (4 + C - 1) / C;
  __shared__ MixSmem<G, NKS> S;
  __shared__ __attribute__((aligned(16))) uint8_t km0[1024], km1[1024], vl0[1024], vh0[1024], vl1[1024], vh1[1024];
  __shared__ __attribute__((aligned(16))) uint8_t qb[G * D * 2];   // bf16 query rows of the group
  const MixSlot slot0 = {km0, vl0, vh0}, slot1 = {km1, vl1, vh1};
  const DecodeBlock blk = decode_block(A);
  const int split = blk.split, kvh = blk.kvh, b = blk.b;
  const int lane = threadIdx.x, a = lane >> 4, r = lane & 15, col = r, h = col % G;
  if (split >= A.n_page_splits) {
    bf16_segment<G>(A, split, b, kvh, lane, S.u.p_lds, S.mh);
    return;
  }
  const int64_t head = (int64_t)b * A.n_kv_heads + kvh;
  int hn16 = A.n16, hn4 = A.n4;
  if (A.head_tiers) mix_record_counts(A.mask + head * MIX_RECORD, hn16, hn4);   // threshold tiers: the head's counts
  const MixGeo g = mix_geo(hn16, hn4);
  const int p0 = split * A.pps, np = min(A.n_pages, p0 + A.pps) - p0;
  const PageSet<PAGED> pset = page_set<PAGED>(A, head, p0, np, lane);

  // Set-up loads first (loads return in issue order, so they arrive before
  // the page): the selection record as one dword per lane, the query rows.
  // Then the first page, its metadata into registers: while an asynchronous
  // LDS copy is in flight every wait the compiler inserts drains all loads,
  // so the set-up issues none and its waits stay partial.
  auto rec_word = [&](int p) {   // this lane's dword of the record page p (split-relative) uses
    const uint8_t* r0 = PREC ? A.mask + (head * A.rec_stride + p0 + p) * MIX_RECORD : A.mask + head * MIX_RECORD;
    return ld4(r0 + 4 * min(lane, MIX_RECORD / 4 - 1));
  };
  const uint32_t recw = rec_word(0);
  u32x4 qv[G / 4];
  load_q<G>(A, b, kvh, lane, qv);
  const uint8_t* pages = pset.at(0);   // paged: waits for the table load only
  u32x4 m0[3];
  m0[0] = ld16_in(range_rsrc(pages + g.off_meta, 32 * g.F), 16 * lane);   // zero past the page's 32 F bytes
  m0[1] = ld16(pages + g.off_v + V_CODE_BYTES + 16 * lane);
  m0[2] = ld16(pages + g.off_v + V_CODE_BYTES + 1024 + 16 * lane);
  MixCodes<NKS, NB> c0, c1;
  mix_load(c0, pages, g, a, r);
  __builtin_amdgcn_sched_barrier(0);
  stage_q<G>(qv, qb, lane);
  __syncthreads();
  constexpr int NQ = PREC ? 1 : 4;
  bf16x8 Bq[NQ];
  mix_tables<G, NKS, NQ, NB>(recw, g, qb, S, Bq, lane, a, h, col);
  *reinterpret_cast<u32x4*>(km0 + 16 * lane) = m0[0];
  *reinterpret_cast<u32x4*>(vl0 + 16 * lane) = m0[1];
  *reinterpret_cast<u32x4*>(vh0 + 16 * lane) = m0[2];
  S.zc.init(lane);
  __syncthreads();

  SoftState<NPASS> st;
  init_state(st);
  const float xs = A.scale_log2 * B_UNSCALE;

  // Each half: wait for everything in flight (all of it is the page about to
  // be computed, requested one page earlier), then request the next page and
  // compute this one. Draining before the copies are issued keeps the
  // compiler from draining after them, which would wait for the next page.
  // (Two pages in flight, the next one requested before this one arrives,
  // measured slower: the memory then serves each split's pages back to back,
  // so the splits served last start computing last; with one page ahead,
  // every split's first page comes before any split's second.)
  uint32_t recn = 0;   // PREC: the next page's record dword
  for (int it = 0; it < np; it += 2) {
    progress_prio(it, np);
    // page it: codes c0, meta slot 0; prefetch page it + 1 into c1 / slot 1
    wait_vm<0>();
    if constexpr (PREC) {
      if (it > 0) mix_tables<G, NKS, NQ, NB>(recn, g, qb, S, Bq, lane, a, h, col);
    }
    if (it + 1 < np) {
      mix_issue_meta(pset.at(it + 1), slot1, g, lane);
      mix_load(c1, pset.at(it + 1), g, a, r);
      if constexpr (PREC) recn = rec_word(it + 1);
    }
    if constexpr (FIFO)
      mix_page<G, NKS, NB, NPASS, NQ>(st, c0, slot0, S, Bq, xs, A.scale_log2, a, h, col,
                                  [&](const f32x4 (&lg)[4], float xb) {
                                    fifo_store_own<G>(A, b, kvh, p0 + it, lg, xs, xb, a, col);
                                  });
    else
      mix_page<G, NKS, NB, NPASS, NQ>(st, c0, slot0, S, Bq, xs, A.scale_log2, a, h, col, NoLogits{});
    if (it + 1 >= np) break;
    wait_vm<0>();
    if constexpr (PREC) mix_tables<G, NKS, NQ, NB>(recn, g, qb, S, Bq, lane, a, h, col);
    if (it + 2 < np) {
      mix_issue_meta(pset.at(it + 2), slot0, g, lane);
      mix_load(c0, pset.at(it + 2), g, a, r);
      if constexpr (PREC) recn = rec_word(it + 2);
    }
    if constexpr (FIFO)
      mix_page<G, NKS, NB, NPASS, NQ>(st, c1, slot1, S, Bq, xs, A.scale_log2, a, h, col,
                                  [&](const f32x4 (&lg)[4], float xb) {
                                    fifo_store_own<G>(A, b, kvh, p0 + it + 1, lg, xs, xb, a, col);
                                  });
    else
      mix_page<G, NKS, NB, NPASS, NQ>(st, c1, slot1, S, Bq, xs, A.scale_log2, a, h, col, NoLogits{});
  }
  write_partial_direct<G, NPASS>(A, st, split, b, kvh, a, col);
}

// ------------------------------------------------------------------ PN-Mix
struct PnKey {
  u32x4 m[3];
  u32x4 lsb[2];
  u32x4 up[2];
};

__device__ inline void pn_load_key(PnKey& c, const uint8_t* page, const PnGeo& g, int lane, int a, int r) {
  c.m[0] = ld16(page + g.off_meta + 16 * (lane & 31));   // 512 B of slot scales/offsets (lanes 32+ repeat them)
  load_vmeta(c.m, page + g.off_v + V_CODE_BYTES, lane);
#pragma unroll
  for (int P2 = 0; P2 < 2; ++P2) c.lsb[P2] = ld16(page + 1024 * P2 + 256 * a + 16 * r);
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) c.up[ks] = ld16(page + g.off_up + 256 * min(4 * ks + a, g.n_up_frag - 1) + 16 * r);
}

template <int G>
__device__ inline void pn_keys(f32x4 (&J)[4], f32x4& zacc, const PnKey& c, const uint8_t* slot,
                               const PgSmem<G, 4>& S, int a, int h, int col) {
  f32x4 logit[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) logit[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
  zacc = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const uint8_t* km = slot + 32 * (4 * ks + a);
    const u32x4 sw = lds16(km), zw = lds16(km + 16);
    const half8 B = key_operand_half(S.u.pg.qh[ks][a][h], S.u.pg.qn[ks][a][col >= 8 ? h : G], sw);
    zacc = mfma(as_half8(zw), S.u.pg.qz[ks][a][h], zacc);
    {                                       // LSB plane: 1-bit codes, weight s
      const Row1 x = row1(rd(c.lsb[ks >> 1], 2 * (ks & 1)), rd(c.lsb[ks >> 1], 2 * (ks & 1) + 1));
#pragma unroll
      for (int T = 0; T < 8; ++T) logit[T] = mfma(tile1(x, T), B, logit[T]);
    }
    if (ks < 2) {                           // upper two bits of the high channels, weight 2 s
      const half8 U = B * (_Float16)2.0f;
      const u32x4 u8 = c.up[ks] >> 8u;
#pragma unroll
      for (int i = 0; i < 8; ++i) logit[i] = mfma(tile2(c.up[ks], u8, i), U, logit[i]);
    }
  }
  half_join(logit, J, col < 8);
#pragma unroll
  for (int t = 0; t < 4; ++t) J[t] *= tile_unscale(t);   // code operands carry 4^(t & 3) * 2^-24
}

template <int G, bool PAGED, bool FIFO>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void decode_pn_fast(DecodeArgs A) {
  constexpr int C = 16 / G;
  constexpr int NPASS = (4 + C - 1) / C;
  __shared__ PgSmem<G, 4> S;
  const DecodeBlock blk = decode_block(A);
  const int split = blk.split, kvh = blk.kvh, b = blk.b;
  const int lane = threadIdx.x, a = lane >> 4, r = lane & 15, col = r, h = col % G;
  if (split >= A.n_page_splits) {
    bf16_segment<G>(A, split, b, kvh, lane, S.u.p_lds, S.mh);
    return;
  }
  const int64_t head = (int64_t)b * A.n_kv_heads + kvh;
  const PnGeo g = pn_geo(A.n_hi);
  const uint8_t* rec = A.mask + head * PN_RECORD;
  const int p0 = split * A.pps, np = min(A.n_pages, p0 + A.pps) - p0;
  const PageSet<PAGED> pset = page_set<PAGED>(A, head, p0, np, lane);

  // set-up loads (the record, the query rows), then the first page, before
  // any of them is waited for
  const uint64_t mask = *reinterpret_cast<const uint64_t*>(rec);   // pair p is high iff bit p
  u32x4 qv[G / 4];
  load_q<G>(A, b, kvh, lane, qv);
  const uint8_t* pages = pset.at(0);   // paged: waits for the table load only

  PnKey kp[2];
  ValCodes vp[2];
  pn_load_key(kp[0], pages, g, lane, a, r);
  load_vcodes(vp[0], pages, g.off_v, a, r);
  __builtin_amdgcn_sched_barrier(0);

  uint8_t* qb = S.u.pg.meta[1] + 1024;
  stage_q<G>(qv, qb, lane);
  {
    // slot order: high channels ascending, then low ones; the slot of
    // channel d counts the channels before it in its class
    const int nh = __builtin_popcountll(mask);                            // high pairs
    for (int d = lane; d < D; d += 64) {
      const bool half = A.pair_layout == KVQ_PAIR_HALF_SPLIT;
      const int pair = half ? (d & 63) : (d >> 1);
      const bool hi = (mask >> pair) & 1;
      const uint64_t below = pair == 0 ? 0ull : (mask & ((1ull << pair) - 1));
      const int cnt = __builtin_popcountll(below);
      int before;
      if (half) before = (hi ? cnt : pair - cnt) + (d >= 64 ? (hi ? nh : 64 - nh) : 0);
      else before = 2 * (hi ? cnt : pair - cnt) + (d & 1);
      S.slot_ch[hi ? before : 2 * nh + before] = d;
    }
  }
  __syncthreads();
  // q of each of this lane's two slots (s = lane, lane + 64), per head; every
  // read comes before the table writes
  int sch[2];
  sch[0] = S.slot_ch[lane];
  sch[1] = S.slot_ch[lane + 64];
  float qsl[2][G];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int hh = 0; hh < G; ++hh) qsl[j][hh] = qb_at(qb, hh, sch[j]);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int s = lane + 64 * j, ks = s >> 5, aa = (s >> 3) & 3, e = s & 7;
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const _Float16 qhv = (_Float16)(qsl[j][hh] * B_SCALE);   // exact unless |q| < 2^-11
      S.u.pg.qh[ks][aa][hh][e] = qhv;
      S.u.pg.qn[ks][aa][hh][e] = -qhv;
      S.u.pg.qz[ks][aa][hh][e] = (_Float16)qsl[j][hh];
    }
  }
  if (lane < 4 * 4) S.u.pg.qn[lane >> 2][lane & 3][G] = half8{};
  S.zc.init(lane);
  __syncthreads();

  SoftState<NPASS> st;
  init_state(st);
  const float xs = A.scale_log2 * B_UNSCALE;
  page_loop(
      np, kp, vp, [&](PnKey& k, int p) { pn_load_key(k, pset.at(p), g, lane, a, r); },
      [&](ValCodes& v, int p) { load_vcodes(v, pset.at(p), g.off_v, a, r); },
      [&](const PnKey& k, const ValCodes& v, int s, int p, auto mid) {
        uint8_t* slot = S.u.pg.meta[s];
        commit_meta(k.m, slot, lane);
        f32x4 J[4], zacc;
        pn_keys<G>(J, zacc, k, slot, S, a, h, col);
        if constexpr (FIFO) fifo_store_own<G>(A, b, kvh, p0 + p, J, xs, zacc[0] * A.scale_log2, a, col);
        mid();
        consume_own<G, NPASS>(st, J, xs, zacc[0] * A.scale_log2, v.vc, VMetaAt{slot + 1024, slot + 2048, S.zc.ptr()}, a, col);
      });
  write_partial_direct<G, NPASS>(A, st, split, b, kvh, a, col);
}

// ------------------------------------------------------------------ QJL (m = 256)
// OUT: the outlier split (m = 256 inlier and 64 outlier sketch rows): a fifth
// 1 KB block of sign bits, the outlier norms beside the inlier ones, and the
// outlier instance's estimate added with its own norm and factor m / mo.
template <bool OUT>
struct QjKey {
  u32x4 m[3];
  u32x4 bits[OUT ? 5 : 4];
};

template <bool OUT>
__device__ inline void qj_load_key(QjKey<OUT>& c, const uint8_t* page, const QjlGeo& g, int lane, int a, int r) {
  // 256 B of norms (OUT: 512 B, the outlier norms after them); the lanes past
  // them repeat them
  c.m[0] = ld16(page + g.off_norm + 16 * (lane & (OUT ? 31 : 15)));
  load_vmeta(c.m, page + g.off_v + V_CODE_BYTES, lane);
#pragma unroll
  for (int P2 = 0; P2 < (OUT ? 5 : 4); ++P2) c.bits[P2] = ld16(page + 1024 * P2 + 256 * a + 16 * r);
}

// Estimator logits nu_t * (2 <Sq, bits_t> - sum Sq) of one page (before the
// sqrt(pi/2)/m and softmax factors, which ride on xs); OUT adds
// (m / mo) nu'_t * (2 <S'q, bits'_t> - sum S'q) of the outlier instance, whose
// MFMAs run one tile at a time once the inlier tiles are done (four more
// accumulator registers, not 32).
template <int G, bool OUT>
__device__ inline void qj_keys(f32x4 (&J)[4], const QjKey<OUT>& c, const uint8_t* slot,
                               const QjSmem<G, OUT ? 10 : 8>& S, float ssum, float ssum_o, float ratio, int a, int h,
                               int col) {
  f32x4 logit[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) logit[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int P2 = 0; P2 < 4; ++P2) {
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int ks = 2 * P2 + hf;
      const half8 B = S.u.qj.bq[col >> 3][ks][a][h];   // hi part in columns < 8, lo part above
      const Row1 x = row1(rd(c.bits[P2], 2 * hf), rd(c.bits[P2], 2 * hf + 1));
#pragma unroll
      for (int T = 0; T < 8; ++T) logit[T] = mfma(tile1(x, T), B, logit[T]);
    }
  }
  const bool hi = col < 8;
  half_join(logit, J, hi);   // this lane's tiles: t (lanes < 8) or t + 4
  // tokens 16 i + 4 a + e have their norms at 32 a + 4 i + e; the lane's
  // tiles 2 q2, 2 q2 + 1 (own numbering) are one 16-byte read
  const uint8_t* nb = slot + 64 * a + (hi ? 0 : 32);
#pragma unroll
  for (int q2 = 0; q2 < 2; ++q2) {
    const u32x4 nw = lds16(nb + 16 * q2);
    u32x4 nwo = {0u, 0u, 0u, 0u};
    if constexpr (OUT) nwo = lds16(nb + 256 + 16 * q2);
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
      const int t = 2 * q2 + ii;   // tiles t and t + 4 carry the same factor
      f32x4 jo = {0.f, 0.f, 0.f, 0.f};
      if constexpr (OUT) {
        // the outlier instance's tiles t and t + 4, joined like the inlier ones
        f32x4 oa = {0.f, 0.f, 0.f, 0.f}, ob4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const half8 B = S.u.qj.bq[col >> 3][8 + hf][a][h];
          const u32x4& ob = c.bits[OUT ? 4 : 0];   // the outlier block
          const Row1 x = row1(rd(ob, 2 * hf), rd(ob, 2 * hf + 1));
          oa = mfma(tile1(x, t), B, oa);
          ob4 = mfma(tile1(x, t + 4), B, ob4);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) jo[e] = (hi ? oa[e] : ob4[e]) + from_partner8(hi ? ob4[e] : oa[e]);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t w = rd(nw, 2 * ii + (e >> 1));
        const uint16_t hb = (uint16_t)(w >> (16 * (e & 1)));
        _Float16 hv;
        __builtin_memcpy(&hv, &hb, 2);
        float est_o = 0.f;
        if constexpr (OUT) {
          const uint16_t hbo = (uint16_t)(rd(nwo, 2 * ii + (e >> 1)) >> (16 * (e & 1)));
          _Float16 hvo;
          __builtin_memcpy(&hvo, &hbo, 2);
          est_o = ratio * (float)hvo * fmaf(2.0f * tile_unscale(t), jo[e], -ssum_o);
        }
        J[t][e] = fmaf((float)hv, fmaf(2.0f * tile_unscale(t), J[t][e], -ssum), est_o);
      }
    }
  }
}

template <int G, bool PAGED, bool OUT, bool FIFO>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(OUT ? 1 : 2))) void decode_qjl_fast(DecodeArgs A) {
  constexpr int C = 16 / G;
  constexpr int NPASS = (4 + C - 1) / C;
  constexpr int NK = OUT ? 10 : 8;   // k-steps of 32 sketch rows
  __shared__ QjSmem<G, NK> S;
  const DecodeBlock blk = decode_block(A);
  const int split = blk.split, kvh = blk.kvh, b = blk.b;
  const int lane = threadIdx.x, a = lane >> 4, r = lane & 15, col = r, h = col % G;
  if (split >= A.n_page_splits) {
    bf16_segment<G>(A, split, b, kvh, lane, S.u.p_lds, S.mh);
    return;
  }
  const int64_t head = (int64_t)b * A.n_kv_heads + kvh;
  const QjlGeo g = qjl_geo(A.qjl_m, OUT ? A.qjl_mo : 0);
  const int p0 = split * A.pps, np = min(A.n_pages, p0 + A.pps) - p0;
  const PageSet<PAGED, OUT ? 2 : 1> pset = page_set<PAGED, OUT ? 2 : 1>(A, head, p0, np, lane);

  // S q of this lane's head first (the inlier rows, so the set-up waits
  // once; OUT: the outlier rows after the first page's loads), then the
  // first page, before any load is waited for
  const int hq = kvh * G + h;
  const float* sqrow = A.sq + ((int64_t)b * A.n_q_heads + hq) * (A.qjl_m + (OUT ? A.qjl_mo : 0));
  float4 sqv[NK][2];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) sqv[ks][hf] = *reinterpret_cast<const float4*>(sqrow + 32 * ks + 8 * a + 4 * hf);
  const uint8_t* pages = pset.at(0);   // paged: waits for the table load only
  QjKey<OUT> kp[2];
  ValCodes vp[2];
  qj_load_key(kp[0], pages, g, lane, a, r);
  load_vcodes(vp[0], pages, g.off_v, a, r);
  __builtin_amdgcn_sched_barrier(0);

  float ssum = 0.f, ssum_o = 0.f;   // sum_i (S q)_i * 2^-6 as the MFMA sees it, per instance
#pragma unroll
  for (int ks = 0; ks < NK; ++ks) {
    if (ks >= 8) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) sqv[ks][hf] = *reinterpret_cast<const float4*>(sqrow + 32 * ks + 8 * a + 4 * hf);
    }
    const float x[8] = {sqv[ks][0].x * B_SCALE, sqv[ks][0].y * B_SCALE, sqv[ks][0].z * B_SCALE, sqv[ks][0].w * B_SCALE,
                        sqv[ks][1].x * B_SCALE, sqv[ks][1].y * B_SCALE, sqv[ks][1].z * B_SCALE, sqv[ks][1].w * B_SCALE};
    half8 hi, lo;
    split8(x, hi, lo);
    if (col < G) {
      S.u.qj.bq[0][ks][a][h] = hi;
      S.u.qj.bq[1][ks][a][h] = lo;
    }
    float part = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) part += (float)hi[e] + (float)lo[e];
    if (ks < 8) ssum += part;
    else ssum_o += part;
  }
  ssum = wave_sum_groups(ssum);
  if constexpr (OUT) ssum_o = wave_sum_groups(ssum_o);
  const float ratio = OUT ? (float)A.qjl_m / (float)A.qjl_mo : 0.f;   // the instances' sqrt(pi/2)/m factors
  S.zc.init(lane);
  __syncthreads();

  SoftState<NPASS> st;
  init_state(st);
  const float xs = A.scale_log2 * A.qjl_coef * B_UNSCALE;
  page_loop(
      np, kp, vp, [&](QjKey<OUT>& k, int p) { qj_load_key(k, pset.at(p), g, lane, a, r); },
      [&](ValCodes& v, int p) { load_vcodes(v, pset.at(p), g.off_v, a, r); },
      [&](const QjKey<OUT>& k, const ValCodes& v, int s, int p, auto mid) {
        uint8_t* slot = S.u.qj.meta[s];
        commit_meta(k.m, slot, lane);
        f32x4 J[4];
        qj_keys<G, OUT>(J, k, slot, S, ssum, ssum_o, ratio, a, h, col);
        if constexpr (FIFO) fifo_store_own<G>(A, b, kvh, p0 + p, J, xs, 0.f, a, col);
        mid();
        consume_own<G, NPASS>(st, J, xs, 0.f, v.vc, VMetaAt{slot + 1024, slot + 2048, S.zc.ptr()}, a, col);
      });
  write_partial_direct<G, NPASS>(A, st, split, b, kvh, a, col);
}

// ------------------------------------------------------------------ dispatch
template <class K>
static void launch1(K kernel, const DecodeArgs& a, hipStream_t s) {
  const int n_parts = a.n_page_splits + a.n_seg_splits;
  hipLaunchKernelGGL(kernel, dim3(n_parts * a.n_kv_heads * a.batch), dim3(64), 0, s, a);
}

template <int G, int NKS, bool PAGED, bool PREC, bool FIFO>
static void launch_mix_nb(const DecodeArgs& a, int nb, hipStream_t s) {
  if (nb == 0) launch1(decode_mix_fast<G, NKS, 0, PAGED, PREC, FIFO>, a, s);
  else if (nb == 1) launch1(decode_mix_fast<G, NKS, 1, PAGED, PREC, FIFO>, a, s);
  else if constexpr (!PREC) launch1(decode_mix_fast<G, NKS, 8, PAGED, false, FIFO>, a, s);
}
template <int G, int NKS, bool FIFO>
static void launch_mix_nb(const DecodeArgs& a, int nb, hipStream_t s) {
  if constexpr (FIFO) {   // no per-page records with the Value FIFO
    if (a.table) launch_mix_nb<G, NKS, true, false, true>(a, nb, s);
    else launch_mix_nb<G, NKS, false, false, true>(a, nb, s);
  } else if (a.rec_stride) {
    if (a.table) launch_mix_nb<G, NKS, true, true, false>(a, nb, s);
    else launch_mix_nb<G, NKS, false, true, false>(a, nb, s);
  } else {
    if (a.table) launch_mix_nb<G, NKS, true, false, false>(a, nb, s);
    else launch_mix_nb<G, NKS, false, false, false>(a, nb, s);
  }
}

template <bool FIFO>
static bool launch_fast(int key_mode, DecodeArgs& a, hipStream_t s) {
  const int g = a.n_q_heads / a.n_kv_heads;
  if (g != 4 && g != 8) return false;
  if (a.table && a.pps > 64) return false;   // the split's page indices live in one register
  if (a.rec_stride && (FIFO || key_mode != KVQ_KEY_MIXKVQ || a.n16 > 1)) return false;   // per-page records: no eight-row BF16 tier
  if (key_mode == KVQ_KEY_MIXKVQ) {
    const int nks = (mix_max_fragments(a.n16, a.n4, a.head_tiers) + 3) / 4;
    if (a.n16 > 8) return false;   // the fast path keeps the BF16 tier in lane group 0 (<= 8 channels)
    const int nb = a.n16 == 0 ? 0 : (a.n16 == 1 ? 1 : 8);
    if (nks == 5) {
      if (g == 4) launch_mix_nb<4, 5, FIFO>(a, nb, s);
      else launch_mix_nb<8, 5, FIFO>(a, nb, s);
      return true;
    }
    if (nks == 4) {
      if (g == 4) launch_mix_nb<4, 4, FIFO>(a, nb, s);
      else launch_mix_nb<8, 4, FIFO>(a, nb, s);
      return true;
    }
    return false;
  }
  if (key_mode == KVQ_KEY_PNMIX) {
    if (a.n_hi != 64) return false;
    if (a.table) {
      if (g == 4) launch1(decode_pn_fast<4, true, FIFO>, a, s);
      else launch1(decode_pn_fast<8, true, FIFO>, a, s);
    } else {
      if (g == 4) launch1(decode_pn_fast<4, false, FIFO>, a, s);
      else launch1(decode_pn_fast<8, false, FIFO>, a, s);
    }
    return true;
  }
  if (a.qjl_m != 256 || (a.qjl_mo != 0 && a.qjl_mo != 64)) return false;   // other sketch sizes: the generic kernel
  if (a.qjl_mo) {
    // one wave per SIMD (the outlier split's registers): half the splits, so
    // that one round of resident waves covers every page; never more splits
    // than the caller's geometry (a.pps), which the workspace is sized for
    const int pps = max(a.pps, a.n_pages > 0 ? decode_pages_per_split_slots(a.n_pages, a.batch, a.n_kv_heads,
                                                                               DECODE_SLOTS / 2)
                                             : 1);
    if (a.table && pps > 128) return false;   // the split's page indices live in two registers
    a.pps = pps;
    a.n_page_splits = a.n_pages > 0 ? (a.n_pages + pps - 1) / pps : 0;
    if (a.table) {
      if (g == 4) launch1(decode_qjl_fast<4, true, true, FIFO>, a, s);
      else launch1(decode_qjl_fast<8, true, true, FIFO>, a, s);
    } else {
      if (g == 4) launch1(decode_qjl_fast<4, false, true, FIFO>, a, s);
      else launch1(decode_qjl_fast<8, false, true, FIFO>, a, s);
    }
    return true;
  }
  if (a.table) {
    if (g == 4) launch1(decode_qjl_fast<4, true, false, FIFO>, a, s);
    else launch1(decode_qjl_fast<8, true, false, FIFO>, a, s);
  } else {
    if (g == 4) launch1(decode_qjl_fast<4, false, false, FIFO>, a, s);
    else launch1(decode_qjl_fast<8, false, false, FIFO>, a, s);
  }
  return true;
}

// Launches the pipelined kernel when one covers the configuration (with the
// split geometry in `a`); returns false (nothing launched) otherwise. fifo:
// the KIVI Value FIFO variant, whose window pages store their logits
// (fifo_store_own; a.fifo_clean and a.fifo_wsplit set by the caller).
bool launch_decode_fast(int key_mode, DecodeArgs& a, hipStream_t s, bool fifo) {
  return fifo ? launch_fast<true>(key_mode, a, s) : launch_fast<false>(key_mode, a, s);
}

}  // namespace kvq
