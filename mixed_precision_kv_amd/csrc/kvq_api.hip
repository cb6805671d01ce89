// libkvq C ABI: host-side validation, geometry queries, storage accounting
// and kernel dispatch. Every entry point checks its arguments before it
// launches anything; on error nothing is launched and no output is touched.
#include <math.h>
#include <stddef.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "kvq_internal.h"

// the layout every binding mirrors (18 int32, then the two thresholds)
static_assert(sizeof(kvq_config) == 88 && offsetof(kvq_config, tau_bf16) == 72, "kvq_config layout");

namespace kvq {

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

static kvq_status check_config(const kvq_config* c) {
  if (!c) return KVQ_INVALID_ARG;
  if (c->abi_version != KVQ_ABI_VERSION) return KVQ_INVALID_ARG;
  if (c->reserved != 0) return KVQ_INVALID_ARG;
  if (c->key_mode != KVQ_KEY_QJL && (c->qjl_outliers != 0 || c->qjl_m_out != 0)) return KVQ_INVALID_ARG;
  if (c->page_records != 0 && c->page_records != 1) return KVQ_INVALID_ARG;
  if (c->page_records && c->key_mode != KVQ_KEY_MIXKVQ) return KVQ_UNSUPPORTED;
  if (c->decode_path != KVQ_DECODE_AUTO && c->decode_path != KVQ_DECODE_GENERIC) return KVQ_INVALID_ARG;
  if (c->select_mode != KVQ_SELECT_COUNT && c->select_mode != KVQ_SELECT_THRESHOLD) return KVQ_INVALID_ARG;
  if (c->select_mode == KVQ_SELECT_THRESHOLD) {
    if (c->key_mode != KVQ_KEY_MIXKVQ) return KVQ_INVALID_ARG;
    for (double t : {c->tau_bf16, c->tau_u4})   // the exact comparison's domain
      if (!isfinite(t) || (t != 0.0 && (fabs(t) < 0x1p-900 || fabs(t) > 0x1p900))) return KVQ_INVALID_ARG;
    if (c->page_records) return KVQ_UNSUPPORTED;   // the query accumulator keeps no row count for the mean
  }
  if (c->head_dim != D) return c->head_dim > 0 ? KVQ_UNSUPPORTED : KVQ_INVALID_ARG;
  if (c->batch < 1 || c->n_kv_heads < 1 || c->n_q_heads < 1 || c->max_pages < 1) return KVQ_INVALID_ARG;
  if ((int64_t)c->batch * c->n_kv_heads * c->max_pages > INT32_MAX) return KVQ_INVALID_ARG;   // pool indices are int32
  if (c->n_q_heads % c->n_kv_heads) return KVQ_INVALID_ARG;
  const int g = c->n_q_heads / c->n_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8 && g != 16) return KVQ_UNSUPPORTED;
  switch (c->key_mode) {
    case KVQ_KEY_MIXKVQ:
      if (c->n_bf16 < 0 || c->n_u4 < 0 || c->n_bf16 + c->n_u4 > D) return KVQ_INVALID_ARG;
      break;
    case KVQ_KEY_PNMIX:
      if (c->pair_layout != KVQ_PAIR_HALF_SPLIT && c->pair_layout != KVQ_PAIR_ADJACENT) return KVQ_INVALID_ARG;
      if (c->n_hi_pairs < 0 || c->n_hi_pairs > D / 2) return KVQ_INVALID_ARG;
      break;
    case KVQ_KEY_QJL:
      if (c->qjl_m < 64 || c->qjl_m % 64) return KVQ_INVALID_ARG;
      if (c->qjl_m > 256) return KVQ_UNSUPPORTED;
      if (c->qjl_outliers < 0 || c->qjl_outliers > 64 || c->qjl_m_out < 0 || c->qjl_m_out % 64) return KVQ_INVALID_ARG;
      if ((c->qjl_outliers == 0) != (c->qjl_m_out == 0)) return KVQ_INVALID_ARG;
      if (c->qjl_m + c->qjl_m_out > 384) return KVQ_UNSUPPORTED;
      break;
    default:
      return KVQ_INVALID_ARG;
  }
  return KVQ_OK;
}

// pages in the arena: the pool a page table indexes
static int pool_pages(const kvq_config* c) { return c->batch * c->n_kv_heads * c->max_pages; }

static bool head_tiers(const kvq_config* c) {
  return c->key_mode == KVQ_KEY_MIXKVQ && c->select_mode == KVQ_SELECT_THRESHOLD;
}

static size_t page_stride(const kvq_config* c) {
  if (c->key_mode == KVQ_KEY_MIXKVQ) {
    if (!head_tiers(c)) return (size_t)mix_geo(c->n_bf16, c->n_u4).stride;
    int st = 0;   // threshold tiers: the largest page of any counts within the capacities
    for (int a = 0; a <= c->n_bf16; ++a)
      for (int b = 0; b <= c->n_u4 && a + b <= D; ++b) st = st > mix_geo(a, b).stride ? st : mix_geo(a, b).stride;
    return (size_t)st;
  }
  if (c->key_mode == KVQ_KEY_PNMIX) return (size_t)pn_geo(2 * c->n_hi_pairs).stride;
  return (size_t)qjl_geo(c->qjl_m, c->qjl_m_out).stride;
}

static size_t record_bytes(const kvq_config* c) {
  if (c->key_mode == KVQ_KEY_MIXKVQ) return MIX_RECORD;
  if (c->key_mode == KVQ_KEY_PNMIX) return PN_RECORD;
  return c->qjl_outliers ? QJL_RECORD : 0;
}

static int n_page_splits(const kvq_config* c, int n_pages) {
  if (n_pages <= 0) return 0;
  const int pps = decode_pages_per_split(n_pages, c->batch, c->n_kv_heads);
  return (n_pages + pps - 1) / pps;
}

// Workspace of a decode call: [split partials | QJL S q]. The partials hold
// the page splits plus the most segment workgroups any call can have.
static size_t partial_bytes(const kvq_config* c, int n_pages) {
  size_t splits = (size_t)n_page_splits(c, n_pages) + MAX_SEG_SPLITS;
  return splits * (size_t)c->batch * c->n_q_heads * RECORD * sizeof(float);
}
static size_t sq_bytes(const kvq_config* c) {
  if (c->key_mode != KVQ_KEY_QJL) return 0;
  return (size_t)c->batch * c->n_q_heads * (size_t)(c->qjl_m + c->qjl_m_out) * sizeof(float);
}
static size_t workspace_for(const kvq_config* c, int n_pages) {
  size_t bytes = partial_bytes(c, n_pages) + sq_bytes(c);
  return (bytes + 255) / 256 * 256;
}

// Checks of kvq_flush_quantize and its kernel arguments (a is filled when
// the result is KVQ_OK, also for n_pages == 0).
static kvq_status flush_prepare(const kvq_config* cfg, const void* k_src, const void* v_src, int64_t src_stride,
                                int32_t n_pages, const void* mask, const void* qjl_s, void* page_arena,
                                const int32_t* page_table, int32_t table_stride, int32_t first_page,
                                uint32_t* status_flags, FlushArgs& a) {
  kvq_status st = check_config(cfg);
  if (st != KVQ_OK) return st;
  if (!k_src || !v_src || !page_arena || !status_flags) return KVQ_INVALID_ARG;
  if (!aligned16(k_src) || !aligned16(v_src) || !aligned16(page_arena)) return KVQ_INVALID_ARG;
  if (page_table && (table_stride < 1 || ((uintptr_t)page_table & 3u))) return KVQ_INVALID_ARG;
  if (n_pages < 0 || first_page < 0 || src_stride < (int64_t)n_pages * PAGE) return KVQ_INVALID_ARG;
  if ((int64_t)first_page + n_pages > (page_table ? table_stride : cfg->max_pages)) return KVQ_CAPACITY;
  const bool needs_mask = cfg->key_mode != KVQ_KEY_QJL || cfg->qjl_outliers > 0;
  if (needs_mask && !mask) return KVQ_INVALID_ARG;
  if (head_tiers(cfg) && !aligned16(mask)) return KVQ_INVALID_ARG;   // the tier codes are read as dwords
  if (cfg->key_mode == KVQ_KEY_QJL && (!qjl_s || !aligned16(qjl_s))) return KVQ_INVALID_ARG;
  // one block per (page, part, kv head, batch) on a one-dimensional grid
  if ((int64_t)n_pages * 16 * cfg->n_kv_heads * cfg->batch > INT32_MAX / 2) return KVQ_INVALID_ARG;
  a.k_src = (const uint16_t*)k_src;
  a.v_src = (const uint16_t*)v_src;
  a.src_stride = src_stride;
  a.mask = (const uint8_t*)mask;
  a.qjl_s = (const uint16_t*)qjl_s;
  a.arena = (uint8_t*)page_arena;
  a.page_stride = (int64_t)page_stride(cfg);
  a.table = page_table;
  a.table_stride = page_table ? table_stride : 0;
  a.pool_pages = pool_pages(cfg);
  a.max_pages = cfg->max_pages;
  a.first_page = first_page;
  a.n_pages = n_pages;
  a.units = n_pages * cfg->n_kv_heads * cfg->batch;
  a.n_kv_heads = cfg->n_kv_heads;
  a.n16 = cfg->n_bf16;
  a.n4 = cfg->n_u4;
  a.n_hi = 2 * cfg->n_hi_pairs;
  a.pair_layout = cfg->pair_layout;
  a.qjl_m = cfg->qjl_m;
  a.qjl_mo = cfg->qjl_m_out;
  a.flags = status_flags;
  a.q_accum = nullptr;
  a.rec_out = nullptr;
  a.rec_stride = 0;
  a.head_tiers = head_tiers(cfg) ? 1 : 0;
  a.keys_only = 0;
  a.push_first = 0;
  a.push_rows = 0;
  return KVQ_OK;
}

// Checks of kvq_decode_attention and its kernel arguments.
static kvq_status decode_prepare(const kvq_config* cfg, const void* q, const void* page_arena,
                                 const int32_t* page_table, int32_t table_stride, int32_t n_pages,
                                 const void* mask, const void* qjl_s, const void* sink_k, const void* sink_v,
                                 int32_t n_sink, const void* resid_k, const void* resid_v, int32_t n_resid,
                                 int32_t resid_stride, float softmax_scale, float* out, void* workspace,
                                 size_t workspace_bytes, DecodeArgs& a) {
  kvq_status st = check_config(cfg);
  if (st != KVQ_OK) return st;
  const int g = cfg->n_q_heads / cfg->n_kv_heads;
  if (g > 8) return KVQ_UNSUPPORTED;
  if (!q || !out || !workspace || !aligned16(q) || !aligned16(out) || !aligned16(workspace)) return KVQ_INVALID_ARG;
  if (page_table && (table_stride < 1 || ((uintptr_t)page_table & 3u))) return KVQ_INVALID_ARG;
  if (n_pages < 0 || n_pages > (page_table ? table_stride : cfg->max_pages)) return KVQ_INVALID_ARG;
  if (n_pages > 0 && (!page_arena || !aligned16(page_arena))) return KVQ_INVALID_ARG;
  const bool needs_mask = cfg->key_mode != KVQ_KEY_QJL || cfg->qjl_outliers > 0;
  if (n_pages > 0 && needs_mask && (!mask || !aligned16(mask))) return KVQ_INVALID_ARG;
  if (cfg->key_mode == KVQ_KEY_QJL && (!qjl_s || !aligned16(qjl_s))) return KVQ_INVALID_ARG;
  if (n_sink < 0 || n_sink > PAGE || n_resid < 0 || n_resid > PAGE) return KVQ_INVALID_ARG;
  if (n_sink > 0 && (!sink_k || !sink_v || !aligned16(sink_k) || !aligned16(sink_v))) return KVQ_INVALID_ARG;
  if (n_resid > 0 && (!resid_k || !resid_v || !aligned16(resid_k) || !aligned16(resid_v) || resid_stride < n_resid))
    return KVQ_INVALID_ARG;
  if (!(softmax_scale > 0.f) || !isfinite(softmax_scale)) return KVQ_INVALID_ARG;
  if (workspace_bytes < workspace_for(cfg, n_pages)) return KVQ_WORKSPACE_TOO_SMALL;
  a.q = (const uint16_t*)q;
  a.arena = (const uint8_t*)page_arena;
  a.page_stride = (int64_t)page_stride(cfg);
  a.table = page_table;
  a.table_stride = page_table ? table_stride : 0;
  a.pool_pages = pool_pages(cfg);
  a.max_pages = cfg->max_pages;
  a.n_pages = n_pages;
  a.n_seg_splits = seg_splits(n_sink + n_resid);
  a.rec_stride = cfg->page_records ? (page_table ? table_stride : cfg->max_pages) : 0;
  a.pps = n_pages > 0 ? decode_pages_per_split(n_pages, cfg->batch, cfg->n_kv_heads) : 1;
  a.n_page_splits = n_page_splits(cfg, n_pages);
  a.mask = (const uint8_t*)mask;
  a.partial = (float*)workspace;
  a.sq = (const float*)((uint8_t*)workspace + partial_bytes(cfg, n_pages));
  a.vq_end = INT32_MAX;   // no KIVI Value FIFO: every page token's Value is quantized
  a.vwin = nullptr;
  a.vwin_stride = 0;
  a.fifo_clean = INT32_MAX;
  a.fifo_wsplit = 0;
  a.out = out;
  a.sink_k = (const uint16_t*)sink_k;
  a.sink_v = (const uint16_t*)sink_v;
  a.n_sink = n_sink;
  a.resid_k = (const uint16_t*)resid_k;
  a.resid_v = (const uint16_t*)resid_v;
  a.n_resid = n_resid;
  a.resid_stride = resid_stride;
  a.resid_v_stride = resid_stride;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.qjl_coef = cfg->key_mode == KVQ_KEY_QJL ? (float)(sqrt(M_PI / 2.0) / cfg->qjl_m) : 0.f;
  a.batch = cfg->batch;
  a.n_kv_heads = cfg->n_kv_heads;
  a.n_q_heads = cfg->n_q_heads;
  a.n16 = cfg->n_bf16;
  a.n4 = cfg->n_u4;
  a.n_hi = 2 * cfg->n_hi_pairs;
  a.pair_layout = cfg->pair_layout;
  a.qjl_m = cfg->qjl_m;
  a.qjl_mo = cfg->qjl_m_out;
  a.head_tiers = head_tiers(cfg) ? 1 : 0;
  return KVQ_OK;
}


// ------------------------------------------------------------------ allocation-free decode
// The decode's scratch (split partials, QJL S q) for callers that cannot
// allocate: one array per GPU, kept until the process ends. In host code the
// array's name is only a stand-in; its device address, different on every
// GPU, is looked up once per device (with that device current) and used
// wherever the host needs the array.
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)KVQ_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];
constexpr int MAX_DEVICES = 64;
static std::atomic<void*> scratch_ptr[MAX_DEVICES];
static std::mutex scratch_mu;

static hipError_t scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  void* p = scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(scratch_mu);
    p = scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || p == nullptr) return e != hipSuccess ? e : hipErrorInvalidSymbol;
      scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}
}  // namespace kvq

using namespace kvq;

extern "C" {

int32_t kvq_abi_version(void) { return KVQ_ABI_VERSION; }

const char* kvq_status_string(kvq_status s) {
  switch (s) {
    case KVQ_OK: return "ok";
    case KVQ_INVALID_ARG: return "invalid argument";
    case KVQ_UNSUPPORTED: return "unsupported configuration";
    case KVQ_WORKSPACE_TOO_SMALL: return "workspace too small";
    case KVQ_CAPACITY: return "page index beyond max_pages";
    case KVQ_HIP_ERROR: return "HIP launch error";
  }
  return "unknown status";
}

kvq_status kvq_page_bytes(const kvq_config* cfg, size_t* bytes) {
  kvq_status st = check_config(cfg);
  if (st != KVQ_OK) return st;
  if (!bytes) return KVQ_INVALID_ARG;
  *bytes = page_stride(cfg);
  return KVQ_OK;
}

kvq_status kvq_mask_bytes(const kvq_config* cfg, size_t* bytes) {
  kvq_status st = check_config(cfg);
  if (st != KVQ_OK) return st;
  if (!bytes) return KVQ_INVALID_ARG;
  *bytes = record_bytes(cfg);
  return KVQ_OK;
}

kvq_status kvq_workspace_bytes(const kvq_config* cfg, int32_t n_pages, size_t* bytes) {
  kvq_status st = check_config(cfg);
  if (st != KVQ_OK) return st;
  if (!bytes || n_pages < 0 || n_pages > cfg->max_pages) return KVQ_INVALID_ARG;
  *bytes = workspace_for(cfg, n_pages);
  return KVQ_OK;
}

// KIVI blog section 7 / PN-Mix storage(): logical bytes, 2-byte metadata.
kvq_status kvq_storage_bytes(const kvq_config* cfg, int64_t n_quant, int32_t n_resid, int32_t n_sink,
                             kvq_storage_breakdown* out) {
  kvq_status st = check_config(cfg);
  if (st != KVQ_OK) return st;
  if (!out || n_quant < 0 || n_quant % PAGE || n_resid < 0 || n_sink < 0) return KVQ_INVALID_ARG;
  const uint64_t H = (uint64_t)cfg->batch * cfg->n_kv_heads;
  const uint64_t pages = (uint64_t)(n_quant / PAGE);
  const uint64_t T = (uint64_t)n_quant;
  kvq_storage_breakdown o;
  memset(&o, 0, sizeof(o));
  o.value_codes = H * T * D * 2 / 8;
  o.value_meta = H * T * (D / GV) * 2 * 2;
  o.residual = H * 2 * (uint64_t)n_resid * D * 2;
  o.sink = H * 2 * (uint64_t)n_sink * D * 2;
  double key_bits_quant = 0.0;   // Key bits per element of a quantized token
  if (cfg->key_mode == KVQ_KEY_MIXKVQ) {
    const int n2 = D - cfg->n_bf16 - cfg->n_u4;
    o.key_full = H * T * cfg->n_bf16 * 2;
    o.key_codes = H * T * (4 * (uint64_t)cfg->n_u4 + 2 * (uint64_t)n2) / 8;
    o.key_meta = H * pages * (uint64_t)(cfg->n_u4 + n2) * 2 * 2;
    o.selection = H * (cfg->page_records ? pages : 1) * (D + D / 4);   // a record per page when re-selected
    key_bits_quant = (16.0 * cfg->n_bf16 + 4.0 * cfg->n_u4 + 2.0 * n2 + 32.0 * (cfg->n_u4 + n2) / PAGE) / D;
  } else if (cfg->key_mode == KVQ_KEY_PNMIX) {
    const uint64_t n_hi = 2 * (uint64_t)cfg->n_hi_pairs;
    o.key_codes = H * (T * D + T * n_hi * 2) / 8;
    o.key_meta = H * pages * D * 2 * 2;
    o.selection = H * ((D / 2 + 7) / 8);
    key_bits_quant = (D + 2.0 * n_hi + 32.0 * D / PAGE) / D;
  } else {
    const int n_norms = cfg->qjl_m_out ? 2 : 1;   // the outlier split keeps a second norm
    o.key_codes = H * T * (uint64_t)(cfg->qjl_m + cfg->qjl_m_out) / 8;
    o.key_meta = H * T * 2 * n_norms;
    o.selection = cfg->qjl_outliers ? H * QJL_RECORD : 0;
    key_bits_quant = ((double)cfg->qjl_m + cfg->qjl_m_out + 16.0 * n_norms) / D;
  }
  o.total = o.key_full + o.key_codes + o.key_meta + o.value_codes + o.value_meta + o.residual + o.sink + o.selection;
  const double toks = (double)n_quant + n_sink;
  o.key_bits_per_element = toks > 0 ? (key_bits_quant * n_quant + 16.0 * n_sink) / toks : 0.0;
  *out = o;
  return KVQ_OK;
}

kvq_status kvq_select_channels(const kvq_config* cfg, const void* q_pre, int64_t l_q, int64_t q_stride,
                               const void* k_pre, int64_t l_k, int64_t k_stride, void* mask_out, void* stream) {
  kvq_status st = check_config(cfg);
  if (st != KVQ_OK) return st;
  const bool qjl = cfg->key_mode == KVQ_KEY_QJL;
  if (qjl && cfg->qjl_outliers == 0) return KVQ_UNSUPPORTED;
  if ((!qjl && !q_pre) || !k_pre || !mask_out) return KVQ_INVALID_ARG;
  if ((!qjl && !aligned16(q_pre)) || !aligned16(k_pre)) return KVQ_INVALID_ARG;
  if ((!qjl && (l_q < 1 || q_stride < l_q)) || l_k < 1 || k_stride < l_k) return KVQ_INVALID_ARG;
  SelectArgs a;
  memset(&a, 0, sizeof(a));
  a.q = (const uint16_t*)q_pre;
  a.k = (const uint16_t*)k_pre;
  a.l_q = l_q;
  a.q_stride = q_stride;
  a.l_k = l_k;
  a.k_stride = k_stride;
  a.n_q_heads = cfg->n_q_heads;
  a.n_kv_heads = cfg->n_kv_heads;
  a.n16 = cfg->n_bf16;
  a.n4 = cfg->n_u4;
  a.n_hi_pairs = cfg->n_hi_pairs;
  a.pair_layout = cfg->pair_layout;
  a.n_out = cfg->qjl_outliers;
  a.out = (uint8_t*)mask_out;
  a.threshold = head_tiers(cfg) ? 1 : 0;
  a.tau_bf16 = cfg->tau_bf16;
  a.tau_u4 = cfg->tau_u4;
  if (a.threshold && 3.0 * (double)(cfg->n_q_heads / cfg->n_kv_heads) * (double)l_q >= 0x1p53) return KVQ_INVALID_ARG;
  return launch_select(cfg->key_mode, a, cfg->batch, (hipStream_t)stream) == hipSuccess ? KVQ_OK : KVQ_HIP_ERROR;
}

kvq_status kvq_accumulate_query(const kvq_config* cfg, const void* q, int64_t l_q, int64_t q_stride, void* q_accum,
                                void* stream) {
  kvq_status st = check_config(cfg);
  if (st != KVQ_OK) return st;
  if (cfg->key_mode != KVQ_KEY_MIXKVQ) return KVQ_UNSUPPORTED;
  if (!q || !q_accum || !aligned16(q) || !aligned16(q_accum)) return KVQ_INVALID_ARG;
  if (l_q < 1 || q_stride < l_q) return KVQ_INVALID_ARG;
  SelectArgs a;
  memset(&a, 0, sizeof(a));
  a.q = (const uint16_t*)q;
  a.l_q = l_q;
  a.q_stride = q_stride;
  a.n_q_heads = cfg->n_q_heads;
  a.n_kv_heads = cfg->n_kv_heads;
  return launch_accumulate(a, q_accum, cfg->batch, (hipStream_t)stream) == hipSuccess ? KVQ_OK : KVQ_HIP_ERROR;
}

kvq_status kvq_flush_quantize(const kvq_config* cfg, const void* k_src, const void* v_src, int64_t src_stride,
                              int32_t n_pages, const void* mask, const void* qjl_s, void* page_arena,
                              const int32_t* page_table, int32_t table_stride, int32_t first_page,
                              uint32_t* status_flags, void* stream) {
  FlushArgs a;
  const kvq_status st = flush_prepare(cfg, k_src, v_src, src_stride, n_pages, mask, qjl_s, page_arena, page_table,
                                      table_stride, first_page, status_flags, a);
  if (st != KVQ_OK || n_pages == 0) return st;
  if (cfg->page_records) return KVQ_UNSUPPORTED;   // per-page records come from kvq_flush_reselect
  return launch_flush(cfg->key_mode, a, cfg->batch, (hipStream_t)stream) == hipSuccess ? KVQ_OK : KVQ_HIP_ERROR;
}

kvq_status kvq_flush_reselect(const kvq_config* cfg, const void* k_src, const void* v_src, int64_t src_stride,
                              int32_t n_pages, const void* q_accum, void* page_records, void* page_arena,
                              const int32_t* page_table, int32_t table_stride, int32_t first_page,
                              uint32_t* status_flags, void* stream) {
  if (cfg && cfg->key_mode == KVQ_KEY_MIXKVQ && !cfg->page_records) return KVQ_INVALID_ARG;
  FlushArgs a;
  const kvq_status st = flush_prepare(cfg, k_src, v_src, src_stride, n_pages, page_records, nullptr, page_arena,
                                      page_table, table_stride, first_page, status_flags, a);
  if (st != KVQ_OK) return st;
  if (cfg->key_mode != KVQ_KEY_MIXKVQ) return KVQ_UNSUPPORTED;
  if (!q_accum || !aligned16(q_accum) || !aligned16(page_records)) return KVQ_INVALID_ARG;
  if (n_pages == 0) return KVQ_OK;
  a.q_accum = q_accum;
  a.rec_out = (uint8_t*)page_records;
  a.rec_stride = page_table ? table_stride : cfg->max_pages;
  return launch_flush(cfg->key_mode, a, cfg->batch, (hipStream_t)stream) == hipSuccess ? KVQ_OK : KVQ_HIP_ERROR;
}

kvq_status kvq_decode_attention(const kvq_config* cfg, const void* q, const void* page_arena,
                                const int32_t* page_table, int32_t table_stride, int32_t n_pages,
                                const void* mask, const void* qjl_s, const void* sink_k, const void* sink_v,
                                int32_t n_sink, const void* resid_k, const void* resid_v, int32_t n_resid,
                                int32_t resid_stride, float softmax_scale, float* out, void* workspace,
                                size_t workspace_bytes, void* stream) {
  DecodeArgs a;
  const kvq_status st = decode_prepare(cfg, q, page_arena, page_table, table_stride, n_pages, mask, qjl_s, sink_k,
                                       sink_v, n_sink, resid_k, resid_v, n_resid, resid_stride, softmax_scale, out,
                                       workspace, workspace_bytes, a);
  if (st != KVQ_OK) return st;
  return launch_decode(cfg->key_mode, a, (const uint16_t*)qjl_s, (hipStream_t)stream, true, cfg->decode_path) ==
                 hipSuccess
             ? KVQ_OK
             : KVQ_HIP_ERROR;
}

kvq_status kvq_flush_keys(const kvq_config* cfg, const void* k_src, const void* v_src, int64_t src_stride,
                          int32_t n_pages, const void* mask, const void* qjl_s, void* page_arena,
                          const int32_t* page_table, int32_t table_stride, int32_t first_page,
                          uint32_t* status_flags, void* stream) {
  FlushArgs a;
  const kvq_status st = flush_prepare(cfg, k_src, v_src, src_stride, n_pages, mask, qjl_s, page_arena, page_table,
                                      table_stride, first_page, status_flags, a);
  if (st != KVQ_OK || n_pages == 0) return st;
  if (cfg->page_records) return KVQ_UNSUPPORTED;
  a.keys_only = 1;
  return launch_flush(cfg->key_mode, a, cfg->batch, (hipStream_t)stream) == hipSuccess ? KVQ_OK : KVQ_HIP_ERROR;
}

kvq_status kvq_value_push(const kvq_config* cfg, const void* v_src, int64_t src_stride, int32_t n_rows,
                          int32_t first_token, const void* mask, void* page_arena, const int32_t* page_table,
                          int32_t table_stride, uint32_t* status_flags, void* stream) {
  kvq_status st = check_config(cfg);
  if (st != KVQ_OK) return st;
  if (cfg->page_records) return KVQ_UNSUPPORTED;
  if (!v_src || !page_arena || !status_flags || !aligned16(v_src) || !aligned16(page_arena)) return KVQ_INVALID_ARG;
  if (page_table && (table_stride < 1 || ((uintptr_t)page_table & 3u))) return KVQ_INVALID_ARG;
  if (n_rows < 0 || first_token < 0 || src_stride < n_rows) return KVQ_INVALID_ARG;
  if (n_rows == 0) return KVQ_OK;
  const int64_t last_page = ((int64_t)first_token + n_rows - 1) / PAGE;
  if (last_page >= (page_table ? table_stride : cfg->max_pages)) return KVQ_CAPACITY;
  if (head_tiers(cfg) && (!mask || !aligned16(mask))) return KVQ_INVALID_ARG;
  if ((int64_t)cfg->batch * cfg->n_kv_heads * n_rows > INT32_MAX) return KVQ_INVALID_ARG;
  FlushArgs a;
  memset(&a, 0, sizeof(a));
  a.v_src = (const uint16_t*)v_src;
  a.src_stride = src_stride;
  a.mask = (const uint8_t*)mask;
  a.arena = (uint8_t*)page_arena;
  a.page_stride = (int64_t)page_stride(cfg);
  a.table = page_table;
  a.table_stride = page_table ? table_stride : 0;
  a.pool_pages = pool_pages(cfg);
  a.max_pages = cfg->max_pages;
  a.n_kv_heads = cfg->n_kv_heads;
  a.n16 = cfg->n_bf16;
  a.n4 = cfg->n_u4;
  a.n_hi = 2 * cfg->n_hi_pairs;
  a.qjl_m = cfg->qjl_m;
  a.qjl_mo = cfg->qjl_m_out;
  a.flags = status_flags;
  a.head_tiers = head_tiers(cfg) ? 1 : 0;
  a.push_first = first_token;
  a.push_rows = n_rows;
  return launch_value_push(cfg->key_mode, a, cfg->batch, (hipStream_t)stream) == hipSuccess ? KVQ_OK
                                                                                            : KVQ_HIP_ERROR;
}

kvq_status kvq_decode_attention_fifo(const kvq_config* cfg, const void* q, const void* page_arena,
                                     const int32_t* page_table, int32_t table_stride, int32_t n_pages,
                                     int32_t n_vq, const void* mask, const void* qjl_s, const void* resid_k,
                                     int32_t n_kres, int32_t kres_stride, const void* vwin, int32_t n_vwin,
                                     int32_t vwin_stride, float softmax_scale, float* out, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  kvq_status st = check_config(cfg);
  if (st != KVQ_OK) return st;
  if (cfg->page_records) return KVQ_UNSUPPORTED;
  if (n_pages < 0 || n_vq < 0 || n_kres < 0 || n_kres > PAGE || n_vwin < 0 || n_vwin > 2 * PAGE)
    return KVQ_INVALID_ARG;
  if (n_vq > (int64_t)n_pages * PAGE || (int64_t)n_pages * PAGE + n_kres != (int64_t)n_vq + n_vwin)
    return KVQ_INVALID_ARG;
  if (n_vwin > 0 && (!vwin || !aligned16(vwin) || vwin_stride < n_vwin)) return KVQ_INVALID_ARG;
  if (n_kres > 0 && kres_stride < n_kres) return KVQ_INVALID_ARG;
  // the Key residual's Values are the window's last n_kres rows (256-byte steps: alignment kept)
  const int kres_row = n_pages * PAGE - n_vq;
  const void* resid_v = n_kres > 0 ? (const void*)((const uint16_t*)vwin + (size_t)kres_row * D) : nullptr;
  DecodeArgs a;
  st = decode_prepare(cfg, q, page_arena, page_table, table_stride, n_pages, mask, qjl_s, nullptr, nullptr, 0,
                      resid_k, resid_v, n_kres, n_kres > 0 ? kres_stride : 0, softmax_scale, out, workspace,
                      workspace_bytes, a);
  if (st != KVQ_OK) return st;
  a.resid_v_stride = vwin_stride;
  a.vq_end = n_vq;
  a.vwin = (const uint16_t*)vwin;
  a.vwin_stride = vwin_stride;
  return launch_decode(cfg->key_mode, a, (const uint16_t*)qjl_s, (hipStream_t)stream, true, cfg->decode_path) ==
                 hipSuccess
             ? KVQ_OK
             : KVQ_HIP_ERROR;
}

kvq_status kvq_decode_attention_noalloc(const kvq_config* cfg, const void* q, const void* page_arena,
                                        const int32_t* page_table, int32_t table_stride, int32_t n_pages,
                                        const void* mask, const void* qjl_s, const void* sink_k, const void* sink_v,
                                        int32_t n_sink, const void* resid_k, const void* resid_v, int32_t n_resid,
                                        int32_t resid_stride, float softmax_scale, float* out, void* stream) {
  kvq_status st = check_config(cfg);
  if (st != KVQ_OK) return st;
  if (n_pages < 0 || n_pages > (page_table ? table_stride : cfg->max_pages)) return KVQ_INVALID_ARG;
  if (workspace_for(cfg, n_pages) > NOALLOC_SCRATCH_BYTES) return KVQ_WORKSPACE_TOO_SMALL;
  void* ws = nullptr;
  if (scratch_of_current_device(&ws) != hipSuccess) return KVQ_HIP_ERROR;
  DecodeArgs a;
  st = decode_prepare(cfg, q, page_arena, page_table, table_stride, n_pages, mask, qjl_s, sink_k, sink_v, n_sink,
                      resid_k, resid_v, n_resid, resid_stride, softmax_scale, out, ws, NOALLOC_SCRATCH_BYTES, a);
  if (st != KVQ_OK) return st;
  return launch_decode(cfg->key_mode, a, (const uint16_t*)qjl_s, (hipStream_t)stream, true, cfg->decode_path) ==
                 hipSuccess
             ? KVQ_OK
             : KVQ_HIP_ERROR;
}

kvq_status kvq_decode_attention_flush(const kvq_config* cfg, const void* q, void* page_arena,
                                      const int32_t* page_table, int32_t table_stride, int32_t n_pages,
                                      const void* mask, const void* qjl_s, const void* sink_k, const void* sink_v,
                                      int32_t n_sink, const void* resid_k, const void* resid_v, int32_t n_resid,
                                      int32_t resid_stride, float softmax_scale, float* out, void* workspace,
                                      size_t workspace_bytes, const void* flush_k_src, const void* flush_v_src,
                                      int64_t flush_src_stride, int32_t n_flush_pages, int32_t flush_first_page,
                                      uint32_t* status_flags, void* stream) {
  DecodeArgs d;
  kvq_status st = decode_prepare(cfg, q, page_arena, page_table, table_stride, n_pages, mask, qjl_s, sink_k, sink_v,
                                 n_sink, resid_k, resid_v, n_resid, resid_stride, softmax_scale, out, workspace,
                                 workspace_bytes, d);
  if (st != KVQ_OK) return st;
  FlushArgs f;
  st = flush_prepare(cfg, flush_k_src, flush_v_src, flush_src_stride, n_flush_pages, mask, qjl_s, page_arena,
                     page_table, table_stride, flush_first_page, status_flags, f);
  if (st != KVQ_OK) return st;
  if (cfg->page_records) return KVQ_UNSUPPORTED;
  const hipStream_t s = (hipStream_t)stream;
  // the split kernels, then one launch holding the flush and the split merge
  if (launch_decode(cfg->key_mode, d, (const uint16_t*)qjl_s, s, false, cfg->decode_path) != hipSuccess)
    return KVQ_HIP_ERROR;
  return launch_merge_flush(cfg->key_mode, d, f, cfg->batch, s) == hipSuccess ? KVQ_OK : KVQ_HIP_ERROR;
}

}  // extern "C"
