/*
 * libkvq - mixed-precision low-bit KV cache for single-token decode on
 * AMD Instinct MI355X (gfx950).
 *
 * Plain C ABI: every argument is a host pointer, a device pointer or a size.
 * The caller owns every buffer and the HIP stream; the library never
 * allocates, frees or synchronizes, keeps no mutable global state (apart from
 * the per-GPU scratch array of kvq_decode_attention_noalloc) and is safe to
 * call from several threads. Every call validates its arguments on
 * the host first; on an error it returns a status and launches nothing, and
 * no output is touched. Device pointers must be 16-byte aligned (page tables:
 * 4-byte). Kernels are
 * launched asynchronously on `stream` (a hipStream_t; NULL = default stream);
 * a launch failure is reported as KVQ_HIP_ERROR.
 *
 * Sources of the operations (cited by page title and section):
 *  - MixKVQ (ACL 2026) summary: salience score A_d = I_d * S_d, the
 *    BF16 / UINT4 / UINT2 Key tiers ("方法细节"), GQA aggregation, lazy
 *    update with a 128-token full-precision residual ("MixKVQ的系统级实现
 *    细节", "通过延迟更新进行摊销调度"), Algorithm 1 (Prefill, Decoding,
 *    KeyQuant, GroupQuant); the running accumulator of query magnitudes
 *    ("高效的在线显著性估计") behind the per-flush reselection; the runtime
 *    evaluation in vLLM's setting and the limitation on non-contiguous
 *    blocks behind the page table.
 *  - PN-Mix reproduction notes: RoPE-pair score (Eq.6), min-max (Eq.2) and
 *    1-bit midpoint correction (Eq.7), H3/L1 bit planes (Appendix G), sinks
 *    and residual, the cache API (from_prefill / append / attention /
 *    storage).
 *  - QJL (AAAI 2025) summary: Definition 3.1, Algorithm 1 (sign sketch,
 *    norm, EstimateScores), orthogonalised S, and its outlier handling
 *    ("处理异常值（Outliers）" with Figure 2: outlier channels fixed at the
 *    prompt, two independent QJL instances, more sketch rows per outlier
 *    coordinate).
 *  - KIVI quantization-axes blog: per-channel Keys / per-token Values,
 *    round-half-to-even, low-bits-first packing, one global softmax,
 *    storage formula.
 *
 * Fixed geometry: head_dim D = 128; a page holds G_K = R = 128 tokens (one
 * Key group per channel per page); Values use 32-channel groups at 2 bits.
 * All model tensors are bfloat16. Quantization scales/offsets are IEEE
 * binary16, as the PN-Mix GPU run ("本地复现") and the KIVI storage budget
 * (section 7) keep them: scale = the binary16 nearest to the exact
 * (max-min)/(2^b-1), offset = the binary16 nearest to the group minimum
 * (exact for bf16 inputs inside the binary16 range); a constant group stores
 * scale +0.0, codes 0; a scale or offset beyond the binary16 range is stored
 * as infinity and reported with KVQ_FLAG_RANGE. QJL norms are binary16.
 * Decode outputs are float32.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVQ_ABI_VERSION 4
#define KVQ_HEAD_DIM 128
#define KVQ_PAGE_TOKENS 128
#define KVQ_VALUE_GROUP 32

typedef enum kvq_status {
  KVQ_OK = 0,
  KVQ_INVALID_ARG = 1,        /* null/misaligned pointer, bad size or count */
  KVQ_UNSUPPORTED = 2,        /* valid request this build does not implement */
  KVQ_WORKSPACE_TOO_SMALL = 3,
  KVQ_CAPACITY = 4,           /* page index beyond max_pages */
  KVQ_HIP_ERROR = 5           /* a kernel launch failed */
} kvq_status;

typedef enum kvq_key_mode {
  KVQ_KEY_MIXKVQ = 0,         /* query-aware 3-tier per-channel Keys */
  KVQ_KEY_PNMIX = 1,          /* RoPE-pair mask, 3-bit / 1-bit midpoint planes */
  KVQ_KEY_QJL = 2             /* 1-bit sign sketch sign(S k) plus ||k||_2 */
} kvq_key_mode;

typedef enum kvq_select_mode {
  KVQ_SELECT_COUNT = 0,       /* MixKVQ tiers by rank: the n_bf16 most salient channels BF16, the next n_u4 UINT4 */
  KVQ_SELECT_THRESHOLD = 1    /* MixKVQ tiers by the salience thresholds tau_bf16 / tau_u4 */
} kvq_select_mode;

typedef enum kvq_decode_path {
  KVQ_DECODE_AUTO = 0,        /* the software-pipelined kernel where one covers the shape, else the generic one */
  KVQ_DECODE_GENERIC = 1      /* always the generic kernel (same results within the decode bound) */
} kvq_decode_path;

typedef enum kvq_pair_layout {
  KVQ_PAIR_HALF_SPLIT = 0,    /* RoPE pair i = (i, i + 64): Llama-style rotate-half */
  KVQ_PAIR_ADJACENT = 1       /* RoPE pair i = (2i, 2i + 1) */
} kvq_pair_layout;

/* Status bits written (OR-ed) into *status_flags by kvq_flush_quantize. */
#define KVQ_FLAG_NONFINITE 1u   /* a non-finite input was seen; that group's codes are unspecified */
#define KVQ_FLAG_SPAN 2u        /* a group spans more than 38 binades; its codes may be off by one */
#define KVQ_FLAG_MASK 4u        /* a PN-Mix record selects a pair count other than n_hi_pairs */
#define KVQ_FLAG_RANGE 8u       /* a group's scale or offset exceeds the binary16 range (stored as inf); a
                                   decode over that page gives non-finite outputs (NaN or inf) for every
                                   query head of its (batch, kv head), and only for those */
#define KVQ_FLAG_TABLE 16u      /* a page-table entry of a flushed page lies outside the pool; that page is not written */

/* Plain-old-data configuration, passed by pointer to every call. */
typedef struct kvq_config {
  int32_t abi_version;        /* must equal KVQ_ABI_VERSION */
  int32_t key_mode;           /* kvq_key_mode */
  int32_t batch;              /* B >= 1 */
  int32_t n_q_heads;          /* Hq, a multiple of Hkv; Hq/Hkv in {1,2,4,8,16} */
  int32_t n_kv_heads;         /* Hkv >= 1 */
  int32_t head_dim;           /* must be 128 */
  int32_t max_pages;          /* page slots per (batch, kv head) in the arena */
  int32_t n_bf16;             /* MixKVQ: channels kept in BF16 (tier 1) */
  int32_t n_u4;               /* MixKVQ: channels at UINT4 (tier 2); the rest UINT2 */
  int32_t pair_layout;        /* PN-Mix: kvq_pair_layout */
  int32_t n_hi_pairs;         /* PN-Mix: high-precision pairs, floor(r*D/2) (32 at r=0.5) */
  int32_t qjl_m;              /* QJL: sketch rows m, a multiple of 64, at most 512 */
  int32_t page_records;       /* MixKVQ: 0, one selection record per (batch, kv head) (selection at
                                 prefill); 1, one record per page, written by kvq_flush_reselect
                                 (tiers re-selected at every flush) and read per page by the decode */
  int32_t qjl_outliers;       /* QJL: 0, one sketch instance; 1..64, outlier channels per (batch, kv head)
                                 found by kvq_select_channels, sketched by a second instance */
  int32_t qjl_m_out;          /* QJL with outliers: that instance's sketch rows, a multiple of 64,
                                 qjl_m + qjl_m_out <= 384 (else 0) */
  int32_t select_mode;        /* MixKVQ: kvq_select_mode. With KVQ_SELECT_THRESHOLD every (batch, kv head)
                                 gets its own tier counts from its selection record, and n_bf16 / n_u4 are the
                                 most BF16 / UINT4 channels a head may hold (they fix the page stride) */
  int32_t decode_path;        /* kvq_decode_path */
  int32_t reserved;           /* must be zero */
  double tau_bf16;            /* THRESHOLD: A_d > tau_bf16 -> BF16 */
  double tau_u4;              /* THRESHOLD: tau_u4 < A_d <= tau_bf16 -> UINT4, else UINT2; finite, and 0 or
                                 2^-900 <= |tau| <= 2^900 */
} kvq_config;

/* Persistent cache bytes of one layer for all (batch, kv head) pairs, by
 * region; logical sizes (codes at their bit width, 2-byte metadata), as in
 * the KIVI blog storage formula and the PN-Mix storage() accounting. */
typedef struct kvq_storage_breakdown {
  uint64_t key_full;          /* BF16-tier Key channels (MixKVQ) */
  uint64_t key_codes;         /* packed Key codes / sign bits */
  uint64_t key_meta;          /* Key scales+offsets (MixKVQ, PN-Mix) or norms (QJL) */
  uint64_t value_codes;
  uint64_t value_meta;
  uint64_t residual;          /* BF16 residual tokens, K and V */
  uint64_t sink;              /* BF16 attention-sink tokens, K and V */
  uint64_t selection;         /* selection records (channel order + tiers, or pair mask) */
  uint64_t total;
  double key_bits_per_element;/* Key bits per element over quantized + sink tokens */
} kvq_storage_breakdown;

/* ABI version of the loaded library. */
int32_t kvq_abi_version(void);

/* Static, never-freed description of a status code. */
const char* kvq_status_string(kvq_status status);

/* Byte stride of one page in the arena (a multiple of 256) for this
 * configuration. The arena is [batch][n_kv_heads][max_pages] pages. With
 * KVQ_SELECT_THRESHOLD it is the largest page any tier counts within the
 * capacities n_bf16 / n_u4 need; a head's page then uses the first bytes of
 * its slot, as its own counts lay them out, and the bytes after them are not
 * written. */
kvq_status kvq_page_bytes(const kvq_config* cfg, size_t* bytes);

/* Bytes of the selection record of one (batch, kv head); the mask buffer of
 * kvq_select_channels holds batch*n_kv_heads records back to back.
 * MixKVQ: 160 bytes = channel order u8[128] (BF16 tier, then UINT4, then
 * UINT2, each ascending) + 2-bit tier codes (0 UINT2, 1 UINT4, 2 BF16, low
 * bits first). PN-Mix: 8 bytes, bit i = RoPE pair i kept at 3 bits.
 * QJL: 0 (S is an input); with qjl_outliers, 16 bytes: bit d % 8 of byte
 * d / 8 set for outlier channel d. */
kvq_status kvq_mask_bytes(const kvq_config* cfg, size_t* bytes);

/* Device workspace kvq_decode_attention needs for n_pages pages. */
kvq_status kvq_workspace_bytes(const kvq_config* cfg, int32_t n_pages, size_t* bytes);

/* Host-only and pure: persistent bytes of a cache holding n_quant_tokens
 * quantized tokens (a multiple of 128), n_resid residual and n_sink sink
 * tokens per (batch, kv head). KIVI blog section 7; PN-Mix storage(). With
 * cfg->page_records the MixKVQ selection counts one record per page. With
 * KVQ_SELECT_THRESHOLD the counts are the data's, not the configuration's:
 * the breakdown is that of heads filled to the capacities n_bf16 / n_u4. */
kvq_status kvq_storage_bytes(const kvq_config* cfg, int64_t n_quant_tokens, int32_t n_resid,
                             int32_t n_sink, kvq_storage_breakdown* out);

/* Precision selection at prefill, once per (batch, kv head).
 *  MixKVQ ("方法细节", "MixKVQ的系统级实现细节"): for every channel d,
 *    SQ_d = sum of |Q| over the l_q prefill queries of all query heads that
 *    share the kv head, range_d = max - min of K over the l_k Key tokens to be
 *    quantized; channels ranked by SQ_d * range_d (ties: lower d first);
 *    KVQ_SELECT_COUNT: the n_bf16 best are BF16, the next n_u4 UINT4, the
 *    rest UINT2.
 *    KVQ_SELECT_THRESHOLD (the three-tier rule with Algorithm 1's tau_BF16,
 *    tau_UINT4): the salience A_d = I_d * S_d with I_d = SQ_d / (g * l_q) (the
 *    mean |Q| over the group's prefill queries) and S_d = range_d / (2^B - 1),
 *    B = 2, is compared exactly with the thresholds: A_d > tau_bf16 is BF16,
 *    tau_u4 < A_d <= tau_bf16 UINT4 (empty when tau_bf16 <= tau_u4), the
 *    rest UINT2. A tier that receives more channels than its capacity
 *    (n_bf16, n_u4) keeps the highest-ranked ones and passes the rest down
 *    one tier. The tiers are contiguous in the ranking, so the record has the
 *    same form, with the head's own counts in its tier codes.
 *  PN-Mix (Eq.6): pairs ranked by sum_t ||q pair|| * sum_s ||k pair||
 *    (query sum over the whole GQA group), top n_hi_pairs kept at 3 bits.
 *  QJL with qjl_outliers > 0 (outlier handling of the QJL page, Figure 2):
 *    channels ranked by sum over the l_k Key tokens of |K| (ties: lower d
 *    first), the qjl_outliers largest are the head's outlier channels;
 *    q_pre is not read (may be NULL).
 *  All rank on exact integer sums of the per-element values rounded to a
 *  2^-64 grid, so the result does not depend on summation order.
 * q_pre: device bf16, element (b, h, t, d) at q_pre[((b*Hq + h)*q_stride + t)*128 + d]
 * k_pre: device bf16, element (b, h, t, d) at k_pre[((b*Hkv + h)*k_stride + t)*128 + d]
 * mask_out: device, batch*n_kv_heads records of kvq_mask_bytes bytes.
 * Preconditions: finite inputs with |q|, |k| < 2^30.
 * QJL without outliers returns KVQ_UNSUPPORTED (S is generated by the caller). */
kvq_status kvq_select_channels(const kvq_config* cfg, const void* q_pre, int64_t l_q, int64_t q_stride,
                               const void* k_pre, int64_t l_k, int64_t k_stride, void* mask_out,
                               void* stream);

/* Quantize and pack n_pages full 128-token segments into pages
 * first_page .. first_page + n_pages - 1 of every (batch, kv head)
 * (MixKVQ Algorithm 1 KeyQuant/GroupQuant at a buffer flush; PN-Mix
 * append; QJL Algorithm 1 steps 2-3). Keys: per channel over the 128
 * tokens (tier per the MixKVQ record; 3-bit or 1-bit-midpoint per the PN-Mix
 * mask; sign sketch + binary16 norm for QJL). Values: per token, 4 groups of
 * 32 channels, 2 bits.
 * k_src/v_src: device bf16, token t of page p of (b, h) at
 *   src[((b*Hkv + h)*src_stride + p*128 + t)*128 + d].
 * mask: the records of kvq_select_channels (ignored for QJL without outliers).
 * qjl_s: device bf16 [qjl_m + qjl_m_out][128] (QJL only, else may be NULL).
 *   With outliers, rows < qjl_m sketch the key's normal channels (the row
 *   restricted to them) and rows >= qjl_m its outlier channels; the page
 *   keeps both instances' sign bits and the two binary16 norms ||k_normal||
 *   and ||k_outlier||.
 * page_arena: device, batch * n_kv_heads * max_pages pages of kvq_page_bytes
 *   (the page pool).
 * page_table: NULL, or device int32 [batch][n_kv_heads][table_stride], 4-byte
 *   aligned: entry p of (b, h) is the pool index of logical page p (a block
 *   table as in vLLM, whose serving setup the MixKVQ runtime evaluation
 *   follows; the pages leave the managing of non-contiguous blocks open).
 *   NULL: logical page p of (b, h) is pool page (b * n_kv_heads + h) *
 *   max_pages + p. An entry outside [0, pool) is not written to: that page
 *   is skipped and KVQ_FLAG_TABLE raised.
 * status_flags: device uint32 (not NULL) the kernels OR KVQ_FLAG_* bits into.
 * Returns KVQ_CAPACITY if first_page + n_pages exceeds max_pages (no table)
 * or table_stride (with a table). */
/* (With cfg->page_records set, kvq_flush_quantize and kvq_decode_attention_flush
 * return KVQ_UNSUPPORTED: the records then come from kvq_flush_reselect.
 * With KVQ_SELECT_THRESHOLD every page of a head is laid out by the tier
 * counts its record holds.) */
kvq_status kvq_flush_quantize(const kvq_config* cfg, const void* k_src, const void* v_src,
                              int64_t src_stride, int32_t n_pages, const void* mask,
                              const void* qjl_s, void* page_arena, const int32_t* page_table,
                              int32_t table_stride, int32_t first_page,
                              uint32_t* status_flags, void* stream);

/* MixKVQ's running accumulator of query magnitudes (system section: at each
 * decode step the current query's magnitude is added; I_d is refreshed from
 * it every R tokens). Adds, for every (batch, kv head) and channel d, the
 * exact sum of psi(|q|) (|q| rounded half-even to the grid 2^-64) over the
 * l_q query rows of every query head of the group, as an unsigned 128-bit
 * integer. Sums of several calls are the sum of one call over all the rows.
 * Call it on the prefill queries (as kvq_select_channels reads them) and on
 * every decode query (l_q = 1, q_stride = 1) to accumulate the whole history;
 * zero the accumulator after each flush for the window-only reading.
 * q: device bf16, element (b, h, t, d) at q[((b*Hq + h)*q_stride + t)*128 + d].
 * q_accum: device, 16-byte aligned, [batch][n_kv_heads][128] uint128
 *   (little-endian), read and written.
 * MixKVQ only (else KVQ_UNSUPPORTED). */
kvq_status kvq_accumulate_query(const kvq_config* cfg, const void* q, int64_t l_q, int64_t q_stride,
                                void* q_accum, void* stream);

/* kvq_flush_quantize with the MixKVQ tiers re-selected for every flushed page
 * (MixKVQ: I_d and S_d are updated every R tokens, channel selection and group
 * quantization run when the residual fills): channels are ranked by
 * SQ_d * range_d, SQ_d from q_accum and range_d = max - min of the page's own
 * 128 Keys, exactly as kvq_select_channels ranks (ties to the lower channel),
 * and the page is packed with that order. The page's 160-byte record goes to
 * page_records + ((b*Hkv + h)*rec_stride + p)*160 for logical page p, with
 * rec_stride = table_stride with a page table, else max_pages.
 * Requires cfg->page_records == 1 (MixKVQ only, KVQ_SELECT_COUNT: the
 * accumulator keeps no row count for the mean |Q| a threshold needs); other
 * arguments as kvq_flush_quantize. Keys must be finite for the ranking. */
kvq_status kvq_flush_reselect(const kvq_config* cfg, const void* k_src, const void* v_src,
                              int64_t src_stride, int32_t n_pages, const void* q_accum,
                              void* page_records, void* page_arena, const int32_t* page_table,
                              int32_t table_stride, int32_t first_page, uint32_t* status_flags,
                              void* stream);

/* Single-token decode attention over [sinks | pages 0..n_pages-1 | residual]
 * with one global softmax (KIVI blog section 6; MixKVQ Algorithm 1
 * Decoding; PN-Mix cache.attention; QJL EstimateScores + softmax):
 *   out[b, h, :] = sum_t softmax_t(logit_t) * v^_t,
 *   logit_t = softmax_scale * q . k^_t for BF16 and dequantized keys,
 *   logit_t = softmax_scale * sqrt(pi/2)/m * nu_t * <S q, sign(S k_t)> for QJL pages;
 *   with the outlier split the sum of that estimate over the normal channels
 *   (m = qjl_m rows) and over the outlier channels (m = qjl_m_out rows).
 * q: device bf16 [batch][n_q_heads][128]; query head h uses kv head h / (Hq/Hkv).
 * page_arena, page_table, table_stride: as for kvq_flush_quantize; pages
 *   0 .. n_pages - 1 are read (n_pages <= max_pages without a table, <=
 *   table_stride with one). A table entry outside the pool is clamped into
 *   it (that page's contribution is then unspecified).
 * mask: the records of kvq_select_channels, 16-byte aligned (ignored for QJL
 *   without outliers and when n_pages is 0); with cfg->page_records, the per-page records of
 *   kvq_flush_reselect (same indexing as there), read page by page.
 * sink_k/sink_v: device bf16 [batch][n_kv_heads][n_sink][128] (n_sink <= 128; may be NULL if 0).
 * resid_k/resid_v: device bf16 [batch][n_kv_heads][resid_stride][128], first
 *   n_resid tokens visible (0 <= n_resid <= 128; may be NULL if 0).
 * out: device float32 [batch][n_q_heads][128].
 * workspace: device, at least kvq_workspace_bytes(cfg, n_pages) bytes (split
 *   partials; for QJL also S q). Calls sharing one workspace must be ordered
 *   on one stream; concurrent calls on the same workspace race. */
kvq_status kvq_decode_attention(const kvq_config* cfg, const void* q, const void* page_arena,
                                const int32_t* page_table, int32_t table_stride,
                                int32_t n_pages, const void* mask, const void* qjl_s,
                                const void* sink_k, const void* sink_v, int32_t n_sink,
                                const void* resid_k, const void* resid_v, int32_t n_resid,
                                int32_t resid_stride, float softmax_scale, float* out,
                                void* workspace, size_t workspace_bytes, void* stream);

/* KIVI's Value FIFO (KIVI blog sections 4-5), the residual policy in which
 * Keys are sealed a whole 128-token segment at a time but Values leave the
 * full-precision residual one token at a time, once R = 128 newer tokens
 * follow. A Value's codes (per token, 32-channel groups) do not depend on when
 * it is quantized, so pages keep their layout: kvq_flush_keys seals the Keys
 * of full segments and clears the pages' Value parts, kvq_value_push
 * quantizes the Value rows that leave the window into their pages, and
 * kvq_decode_attention_fifo attends with the Key boundary and the Value
 * boundary apart (one global softmax). Not with cfg->page_records. */

/* kvq_flush_quantize for the Value FIFO: the Keys of pages first_page ..
 * first_page + n_pages - 1 quantized and packed as kvq_flush_quantize does,
 * their Value parts cleared (codes, scales and offsets zero); v_src is not
 * read (may equal k_src). Same arguments, errors and flags. */
kvq_status kvq_flush_keys(const kvq_config* cfg, const void* k_src, const void* v_src, int64_t src_stride,
                          int32_t n_pages, const void* mask, const void* qjl_s, void* page_arena,
                          const int32_t* page_table, int32_t table_stride, int32_t first_page,
                          uint32_t* status_flags, void* stream);

/* The Value rows of tokens first_token .. first_token + n_rows - 1 of every
 * (batch, kv head), leaving the full-precision window: each quantized per token
 * (four groups of 32 channels, 2 bits, the flush's quantizer, flags as there)
 * and ORed into its page (logical page token / 128, row token % 128). The
 * pages must hold sealed Keys (kvq_flush_keys) and these rows must not have
 * been pushed before: the push adds bits to the cleared Value part.
 * v_src: device bf16 [batch][n_kv_heads][src_stride][128], row j = token
 * first_token + j. mask, page_arena, page_table, table_stride, status_flags:
 * as kvq_flush_quantize. KVQ_CAPACITY if a row's page is past max_pages (or
 * table_stride). */
kvq_status kvq_value_push(const kvq_config* cfg, const void* v_src, int64_t src_stride, int32_t n_rows,
                          int32_t first_token, const void* mask, void* page_arena, const int32_t* page_table,
                          int32_t table_stride, uint32_t* status_flags, void* stream);

/* Decode attention with the Value FIFO: the visible tokens are n_pages * 128
 * sealed Keys (pages) followed by n_kres Key-residual rows (resid_k,
 * [batch][n_kv_heads][kres_stride][128] bf16); the Values of tokens 0 ..
 * n_vq - 1 are the pages' quantized rows and those of tokens n_vq .. T - 1
 * the window rows (vwin, [batch][n_kv_heads][vwin_stride][128] bf16, row j =
 * token n_vq + j), T = n_pages * 128 + n_kres = n_vq + n_vwin. Constraints:
 * n_vq <= n_pages * 128, 0 <= n_kres <= 128, n_vwin <= 256. The pages'
 * Value rows of tokens n_vq and later must be as kvq_flush_keys left them
 * (cleared; the FIFO pushes a row only when it leaves the window). Logits
 * and the global softmax as kvq_decode_attention. Where a pipelined kernel
 * covers the configuration it runs over every page and the Key residual;
 * the window tokens inside the pages add nothing there (cleared rows), and
 * the split merge adds their window Values, weighted by their logits, which
 * that kernel leaves in spare workspace records. cfg->decode_path =
 * KVQ_DECODE_GENERIC runs the generic kernel, which takes those Values
 * inside the page pass (results within the same bound). Other arguments and
 * the workspace as kvq_decode_attention. */
kvq_status kvq_decode_attention_fifo(const kvq_config* cfg, const void* q, const void* page_arena,
                                     const int32_t* page_table, int32_t table_stride, int32_t n_pages,
                                     int32_t n_vq, const void* mask, const void* qjl_s, const void* resid_k,
                                     int32_t n_kres, int32_t kres_stride, const void* vwin, int32_t n_vwin,
                                     int32_t vwin_stride, float softmax_scale, float* out, void* workspace,
                                     size_t workspace_bytes, void* stream);

/* kvq_decode_attention without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). The split partials (and QJL's S q) go to
 * a scratch array of KVQ_NOALLOC_SCRATCH_BYTES that the library keeps on
 * every GPU it runs on until the process ends; this call allocates nothing
 * and calls no allocating routine. Arguments and results as
 * kvq_decode_attention. Returns KVQ_WORKSPACE_TOO_SMALL when the call would
 * need more scratch than that (kvq_workspace_bytes(cfg, n_pages) >
 * KVQ_NOALLOC_SCRATCH_BYTES), KVQ_HIP_ERROR if the array's device address
 * cannot be found. All calls on one GPU share its array: calls that overlap
 * on one GPU (on different streams, or from several threads) race. */
#define KVQ_NOALLOC_SCRATCH_BYTES (16u << 20)
kvq_status kvq_decode_attention_noalloc(const kvq_config* cfg, const void* q, const void* page_arena,
                                        const int32_t* page_table, int32_t table_stride, int32_t n_pages,
                                        const void* mask, const void* qjl_s, const void* sink_k, const void* sink_v,
                                        int32_t n_sink, const void* resid_k, const void* resid_v, int32_t n_resid,
                                        int32_t resid_stride, float softmax_scale, float* out, void* stream);

/* kvq_decode_attention, then kvq_flush_quantize, in one call: the decode step
 * at which the residual has filled and is packed into the next page (KIVI
 * blog section 6: the residual holds up to R tokens and is quantized when
 * full; MixKVQ Algorithm 1, KeyQuant / GroupQuant at that flush). The flush
 * does not depend on the decode's output, so it runs in the same launch as
 * the decode's split merge rather than after it.
 * Arguments: those of kvq_decode_attention (q .. workspace_bytes), then the
 *   flush's source, count and target (flush_k_src, flush_v_src,
 *   flush_src_stride, n_flush_pages, flush_first_page, status_flags: as
 *   k_src, v_src, src_stride, n_pages, first_page, status_flags of
 *   kvq_flush_quantize); cfg, mask, qjl_s, page_arena, page_table,
 *   table_stride and stream serve both.
 * Results: out, the written pages and the status bits are bit-identical to
 *   the two calls made in that order on one stream; the flush writes after
 *   the decode has read the arena, so the page ranges may overlap.
 * Errors: any check of either call fails the whole call and launches
 *   nothing. The workspace rule of kvq_decode_attention applies. */
kvq_status kvq_decode_attention_flush(const kvq_config* cfg, const void* q, void* page_arena,
                                      const int32_t* page_table, int32_t table_stride,
                                      int32_t n_pages, const void* mask, const void* qjl_s,
                                      const void* sink_k, const void* sink_v, int32_t n_sink,
                                      const void* resid_k, const void* resid_v, int32_t n_resid,
                                      int32_t resid_stride, float softmax_scale, float* out,
                                      void* workspace, size_t workspace_bytes,
                                      const void* flush_k_src, const void* flush_v_src,
                                      int64_t flush_src_stride, int32_t n_flush_pages,
                                      int32_t flush_first_page, uint32_t* status_flags,
                                      void* stream);

/* Measurement helper, not part of the method: the read-stream reference a
 * decode's fraction of the HBM peak is read against. Reads the `bytes` bytes
 * at src (device, 16-byte aligned, bytes a multiple of 16) with the load
 * shape of the decode kernels (16-byte lane loads, 1 KB per wave
 * instruction, 16 KB per workgroup, all of a workgroup's loads in flight
 * together) and writes, for chunk c of 16384 bytes (the last one possibly
 * short), the XOR of its 32-bit little-endian words to sink[c] (device,
 * sink_bytes >= 4 * ceil(bytes / 16384), else KVQ_WORKSPACE_TOO_SMALL).
 * bytes == 0 launches nothing. Asynchronous on `stream`. */
kvq_status kvq_read_stream(const void* src, size_t bytes, uint32_t* sink, size_t sink_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
