/*
 * kvq.h -- C ABI of the mixed-format paged KV decode-attention library
 * (libkvq.so, MI355X / gfx950).
 *
 * What it computes. Single-token decode attention over a paged KV cache
 * whose logical pages come in different physical formats (Minima-KV, arxiv
 * 2608.23834, section 3.1 and section 3.3): Recent and Anchor pages hold FP8
 * E4M3 codes with one fp32 scale per (token, KV head, role); Stale pages hold
 * packed 3-bit TurboQuant-MSE-style codes (one fp16 norm correction per
 * vector, a seeded Hadamard-sign rotation, an fp16 Gaussian Lloyd-Max
 * codebook), or their 2-bit form, or grouped mixed-rate keys whose RoPE
 * blocks of equal width form TQ segments of 2, 3 and 4 bits next to TQ3
 * values (Block-GTQ appendix A.7). Each format is scanned by its own pass producing a partial
 * maximum, exponential sum and normalized partial output; the partials are
 * merged by the stable online-softmax recurrence of Minima-KV Eq. 11-13, with
 * TQ values accumulated in rotated coordinates and rotated back once
 * (Block-GTQ, paperpeel 2606.24033, appendix H.2). No dense decoded copy of
 * the cache is written to device memory.
 *
 * Conventions for every call:
 *  - pointers are DEVICE pointers unless marked [host];
 *  - every call is asynchronous on `stream` (hipStream_t, may be 0) and never
 *    synchronizes, allocates, or frees; the caller owns every buffer and keeps
 *    it alive until the stream work is done;
 *  - host-side validation runs before any launch; an invalid or unsupported
 *    argument returns an error and launches nothing ("fail closed", Minima-KV
 *    section 4.1);
 *  - supported geometry: head_dim d in {128, 256}, page_size P in {16, 32},
 *    num_q_heads % num_kv_heads == 0, group size G = Hq/Hkv <= 16;
 *  - device-side bad data (unknown format tag, page id outside its pool,
 *    seq_len > max_pages * P) cannot be an error code without a sync: the
 *    entry is masked out and counted in kvq_counters.invalid_entries.
 *
 * Page layout (one pool per format, [pool pages][page bytes]; a page holds
 * all KV heads, [Hkv][head block]); tiles are 16 tokens of one role:
 *   FP8 head block: K tiles | V tiles | K scale f32[P] | V scale f32[P]
 *                   = 2*P*d + 8*P bytes
 *   TQb head block: K tiles | V tiles | K sigma f16[P] | V sigma f16[P]
 *                   = 2*P*d*b/8 + 4*P bytes   (b = 3 for TQ3, 2 for TQ2)
 *   TQK head block: K tiles | V tiles | K sigma f16[3][P] | V sigma f16[P]
 *                   = P*(3*d/4 + 8) bytes (d = 128: 104 B per token and head)
 * Inside a tile, 64 "lanes" own d/4 elements each:
 *   K: lane l, element i = token l%16, dim (l/16)*(d/4) + i
 *   V: lane l, element i = token 4*(l/16) + i%4, dim l%16 + 16*(i/4)
 * FP8 element (l, i) is byte ((i/16)*64 + l)*16 + i%16 of the tile. TQb codes
 * of a lane fill (d/4)*b/32 32-bit words, stored in 16/8/4-byte per-lane
 * regions; groups of four consecutive elements share a byte lane (element
 * i sits in byte i%4 of its word). For b = 3, each triple of words holds
 * eight groups q = 0..7: q = 0..5 at bits 0-2 / 3-5 of words 0, 0, 1, 1, 2, 2;
 * q = 6 and q = 7 keep code bits 0-1 at bits 6-7 of words 0 and 1 and code
 * bit 2 at bits 6 and 7 of word 2. For b = 2, group g sits at bits 2*(g%4)
 * of word g/4.
 *
 * TQK (grouped mixed-rate keys, Block-GTQ appendix A.7, H.1-H.2): the key is
 * stored in a permuted coordinate order (tqk_perm) made of three segments,
 * [0, d/4) at 2 bits, [d/4, 3d/4) at 3 bits and [3d/4, d) at 4 bits; each
 * segment is the TQ codec above at its own length d_s with its own fp16
 * sigma and the K sign bits at its positions (K signs are indexed in
 * permuted order). Values are uniform TQ3 (the TQ3 V tile rule). A TQK K tile
 * deals 32-coordinate chunks: lane l, element i = token l%16, permuted dim
 * 32*(i/8) + 8*(l/16) + i%8, so one chunk never mixes segments. A lane's
 * groups g (four elements each) are n2 = d/64 2-bit groups, then n3 = d/32
 * 3-bit, then d/64 4-bit; the 3d/128 words go in triples, triple m holding
 * at byte i%4: word 3m the 4-bit groups n2+n3+2m (bits 0-3) and +1 (bits
 * 4-7); word 3m+1 the 3-bit groups n2+4m (bits 0-2) and +1 (bits 3-5) and
 * the 2-bit group 2m (bits 6-7); word 3m+2 the 3-bit groups n2+4m+2, +3 and
 * the 2-bit group 2m+1. Words use the per-lane regions of TQ3.
 *
 * TQF5 / TQF6 (fractional-level codes, SemKV section 4.1 "Memory
 * accounting" and section 4.9): the TQ codec below with a 5- or 6-level
 * codebook. A head block is P key rows | P value rows | K sigma f16[P] | V
 * sigma f16[P]; row t holds the codes of slot t as one little-endian
 * bitstream of ceil(d / k) groups of nbits bits (L = 5: k = 3, nbits = 7;
 * L = 6: k = 5, nbits = 13), group j = sum_i c_{kj+i} L^i (codes past d are
 * 0), R = ceil(groups * nbits / 8) bytes: 38 / 76 bytes (L = 5) and 43 / 85
 * bytes (L = 6) at d = 128 / 256. A token-head takes 2 R + 4 bytes.
 *
 * TQ codec (Minima-KV section 4.3 "normalize-rotate-pack"; Block-GTQ B.1):
 * for a vector x of length d in fp32: n = sqrt(halving-tree sum of x*x);
 * w = FWHT(s * x) with the role's sign vector s (unnormalized, butterfly
 * stages 1, 2, 4, ...); code_j = #{k : w_j > n * t_k}; sigma = fp16(n /
 * sqrt(halving-tree sum of c[code]^2)); a zero vector gets codes 0 and sigma
 * 0. Decoded x = sigma * s * FWHT(c[code]) / sqrt(d).
 * Input range of the TQ encoders: sigma is an fp16 number, so a vector whose
 * ratio n / ||c[code]|| rounds to 65520 or more (a norm above roughly
 * 6.4e4 * sqrt(d_s) for Gaussian-like rows, d_s the segment length) stores
 * sigma = +inf, exactly as the definition above says, and decodes to
 * inf / NaN. Callers keep rows below that norm (activations in bf16 / fp16
 * models are far below it); the encoders do not clamp.
 */
#ifndef KVQ_H_
#define KVQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *hipStream_t;

typedef enum {
  KVQ_OK = 0,
  KVQ_ERR_INVALID = -1,      /* bad pointer, size, alignment or workspace */
  KVQ_ERR_UNSUPPORTED = -2,  /* geometry outside the supported set */
  KVQ_ERR_HIP = -3           /* a HIP launch failed (kvq_last_error has it) */
} kvq_status;

/* Per-page format tags (one byte per logical page of a request). */
typedef enum {
  KVQ_FMT_FP8 = 0,   /* Recent / Anchor pages: E4M3 codes + fp32 scales */
  KVQ_FMT_TQ3 = 1,   /* Stale pages: 3-bit TQ codes + fp16 sigma */
  KVQ_FMT_TQ2 = 2,   /* Stale pages at 2 bits (same codec, 4 levels) */
  KVQ_FMT_TQK = 3,   /* Stale pages: grouped mixed-rate keys, TQ3 values (d = 128) */
  KVQ_FMT_TQF5 = 4,  /* Stale pages: 5-level codes, three to 7 bits (2.33 bits a value) */
  KVQ_FMT_TQF6 = 5,  /* Stale pages: 6-level codes, five to 13 bits (2.6 bits a value) */
  KVQ_FMT_COUNT = 6
} kvq_format;

/* Source of kv_encode_tq3 / kv_encode_tq2 / kv_encode_tqk. */
typedef enum {
  KVQ_SRC_F32_ROWS = 0,   /* float [n_pages][P][Hkv][2][d] */
  KVQ_SRC_FP8_PAGES = 1   /* pages of the cache's FP8 pool (demotion) */
} kvq_source;

/* One layer's cache. The struct itself is read on the host ([host]); the
 * pool pointers are device pointers. Pools may be NULL when empty. */
typedef struct {
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t page_size;
  int32_t reserved0;
  uint8_t *fp8_pages;       int64_t fp8_num_pages;
  uint8_t *tq3_pages;       int64_t tq3_num_pages;
  uint8_t *tq2_pages;       int64_t tq2_num_pages;
  /* Rotation signs, uint32 [Hkv][2][d/32]; role 0 = K, role 1 = V; bit j of
   * word j/32 set means coordinate j is negated before the Hadamard
   * transform (Block-GTQ B.1: one rotation per group from a fixed seed,
   * reused for every token). Required when any TQ pool is used. */
  const uint32_t *rot_signs;
  /* Grouped mixed-rate key pool (KVQ_FMT_TQK) and its key coordinate order,
   * uint16 [Hkv][d]: entry j is the original coordinate stored at permuted
   * position j (Block-GTQ H.1: blocks of one rate permuted into a contiguous
   * segment). Entries are used modulo d; a table that is not a permutation
   * gives meaningless but in-bounds results. Required with a TQK pool, which
   * also needs head_dim 128. */
  uint8_t *tqk_pages;       int64_t tqk_num_pages;
  const uint16_t *tqk_perm;
  /* Fractional-level pools (KVQ_FMT_TQF5 / KVQ_FMT_TQF6); they use rot_signs. */
  uint8_t *tqf5_pages;      int64_t tqf5_num_pages;
  uint8_t *tqf6_pages;      int64_t tqf6_num_pages;
} kvq_layer_cache;

/* Route counters (Minima-KV section 3.3 and Table 4: route and fallback
 * instrumentation). Device memory; the library only adds to them.
 * pages_* count (page, KV head) pairs scanned by decode calls;
 * invalid_entries counts masked table entries (plan calls, and decode calls
 * whose cache holds fewer pages than a table entry names) and decode calls
 * handed a plan built for another geometry; fallbacks is never incremented --
 * there is no generic path to fall back to. */
typedef struct {
  unsigned long long pages_fp8;
  unsigned long long pages_tq3;
  unsigned long long pages_tq2;
  unsigned long long pages_tqk;
  unsigned long long invalid_entries;
  unsigned long long fallbacks;
  unsigned long long pages_tqf5;
  unsigned long long pages_tqf6;
} kvq_counters;

/* [host] Static description of a status code. */
const char *kvq_status_string(int32_t status);
/* [host] Detail of the last error on the calling thread ("" if none). */
const char *kvq_last_error(void);
/* [host] ABI version (bumped on any layout or signature change). */
int32_t kvq_abi_version(void);
/* [host] Measurement hook; nothing it does changes a result. While `event`
 * (a hipEvent_t) is not NULL, every decode call made on the calling thread
 * records it on the call's stream between the call's scan kernel and its
 * merge kernel, so a caller can time the two kernels apart with HIP events
 * on the stream they run on. NULL (the default) turns it off. */
void kvq_set_scan_end_event(void *event);
/* [host] Bytes of one page (all KV heads) of a format; 0 if unsupported. */
size_t kvq_page_bytes(int32_t format, int32_t num_kv_heads, int32_t head_dim, int32_t page_size);

/* Append / Anchor write (Minima-KV algorithm 1 "Append"; section 3.1
 * "Recent"): FP8-encode n_tok tokens into FP8 pages.
 *   src       float (src_is_bf16 = 0) or bf16 (1) rows [n_tok][Hkv][2][d],
 *             role 0 = K, role 1 = V
 *   dst_page  int32 [n_tok] page id in c->fp8_pages
 *   dst_slot  int32 [n_tok] slot 0..P-1 inside that page
 * Per (token, head, role): amax = max|x|; amax = 0 -> codes 0, scale 0;
 * else y = x * fp32(448 / amax) rounded to E4M3 (nearest, ties to even),
 * scale = fp32(amax / 448). Writes only the given slots. Two tokens must not
 * target the same slot in one call. */
kvq_status kv_encode_fp8(const kvq_layer_cache *c, const void *src, int32_t src_is_bf16, int64_t n_tok,
                         const int32_t *dst_page, const int32_t *dst_slot, hipStream_t stream);

/* Stale conversion (Minima-KV algorithm 1 "Retier", section 4.3 batched
 * FP8-to-TQ3 normalize-rotate-pack): encode whole pages into c->tq3_pages.
 *   src_kind  KVQ_SRC_F32_ROWS: src = float [n_pages][P][Hkv][2][d]
 *             KVQ_SRC_FP8_PAGES: src ignored, src_page int32 [n_pages] =
 *             FP8 page ids; rows are fp32(value(e) * scale)
 *   dst_page  int32 [n_pages] page ids in c->tq3_pages
 *   page_valid int32 [n_pages] number of filled slots (1..P), or NULL for P;
 *             slots past it are written as codes 0, sigma 0
 * The source page is only read; freeing it is the caller's business. */
kvq_status kv_encode_tq3(const kvq_layer_cache *c, int32_t src_kind, const void *src, const int32_t *src_page,
                         int64_t n_pages, const int32_t *dst_page, const int32_t *page_valid, hipStream_t stream);
/* Same for the 2-bit pool c->tq2_pages. */
kvq_status kv_encode_tq2(const kvq_layer_cache *c, int32_t src_kind, const void *src, const int32_t *src_page,
                         int64_t n_pages, const int32_t *dst_page, const int32_t *page_valid, hipStream_t stream);
/* Same for the grouped mixed-rate pool c->tqk_pages (Block-GTQ A.7, H.1):
 * keys are permuted by c->tqk_perm and each segment is TQ-encoded at its own
 * rate and length with one fp16 sigma; values are TQ3. head_dim must be 128. */
kvq_status kv_encode_tqk(const kvq_layer_cache *c, int32_t src_kind, const void *src, const int32_t *src_page,
                         int64_t n_pages, const int32_t *dst_page, const int32_t *page_valid, hipStream_t stream);
/* Same for the fractional-level pools c->tqf5_pages and c->tqf6_pages (SemKV
 * section 4.1: 5- and 6-level codes, mixed-radix packed). */
kvq_status kv_encode_tqf5(const kvq_layer_cache *c, int32_t src_kind, const void *src, const int32_t *src_page,
                          int64_t n_pages, const int32_t *dst_page, const int32_t *page_valid, hipStream_t stream);
kvq_status kv_encode_tqf6(const kvq_layer_cache *c, int32_t src_kind, const void *src, const int32_t *src_page,
                          int64_t n_pages, const int32_t *dst_page, const int32_t *page_valid, hipStream_t stream);

/* Promote (Minima-KV algorithm 1 "Promote"; section 3.1 "Anchor" and figure
 * 2: a Stale page re-entering the protected budget is reconstructed into a
 * newly allocated FP8 page before its mapping is published).
 *   src_format KVQ_FMT_TQ3, KVQ_FMT_TQ2, KVQ_FMT_TQK, KVQ_FMT_TQF5 or
 *              KVQ_FMT_TQF6: the pool that is read
 *   src_page   int32 [n_pages] page ids in that pool
 *   dst_page   int32 [n_pages] page ids in c->fp8_pages (distinct)
 * Each (token, head, role) row is rebuilt in fp32 in this order: F =
 * FWHT(c[code]) (exact in fp32), u = fp32(F * r) with r the fp32 value
 * nearest 1/sqrt(d_s), x = fp32(sigma * u), then the sign flip; grouped keys
 * segment by segment (d_s = the segment's width), the permutation undone.
 * The row is then FP8-encoded as by kv_encode_fp8. Empty slots (sigma 0)
 * become codes 0, scale 0. A page whose source or destination id is out of
 * range is skipped (its destination is left as it was). The source page is
 * only read; retiring it is the caller's business. */
kvq_status kv_promote_fp8(const kvq_layer_cache *c, int32_t src_format, const int32_t *src_page, int64_t n_pages,
                          const int32_t *dst_page, hipStream_t stream);

/* Format partition (Minima-KV section 4.1: compact per-request page-index
 * arrays that partition the logical block table by format, order kept).
 * Built once per decode step and shared by every layer with the same page
 * table and geometry.
 *   block_table int32 [batch][max_pages] physical page id in the pool of the
 *               page's format; page_format uint8 [batch][max_pages];
 *   seq_lens    int32 [batch] cached tokens N_b (the query's own K/V already
 *               appended); pages past ceil(N_b / P) are ignored
 *   plan        device buffer of paged_decode_plan_bytes(...) bytes, fully
 *               written by the call (no initial contents needed). Its first
 *               64 bytes record the geometry it was built for (batch,
 *               max_pages, num_kv_heads, page_size, head_dim); it also holds
 *               the work dispenser of the decode grid, which every decode call
 *               counts up and returns to zero, so decode calls sharing one plan
 *               must be ordered on one stream
 *   counters    optional (NULL): invalid_entries += masked entries
 * An entry is masked when its tag is unknown or its id is outside the pool
 * that c names for its format. */
size_t paged_decode_plan_bytes(int32_t batch, int32_t max_pages, const kvq_layer_cache *c);
kvq_status paged_decode_plan(const kvq_layer_cache *c, int32_t batch, const int32_t *block_table,
                             const uint8_t *page_format, int32_t max_pages, const int32_t *seq_lens,
                             void *plan, size_t plan_bytes, kvq_counters *counters, hipStream_t stream);

/* Decode attention for one layer from a plan (Minima-KV section 3.3 Eq. 11-13,
 * section 4.1 fused scans + merge; Block-GTQ H.2-H.4).
 *   plan, plan_bytes  a buffer written by paged_decode_plan; plan_bytes below
 *            paged_decode_plan_bytes(batch, max_pages, c) is an error
 *   q_bf16   bf16 [batch][num_q_heads][d]; q-head h reads KV head h / G
 *   out      float [batch][num_q_heads][d]
 *   lse      float [batch][num_q_heads] natural-log sum-exp, or NULL
 *   workspace  device scratch of paged_decode_attn_planned_workspace_size(...)
 *              bytes (partials only; no initial contents needed)
 *   sm_scale   multiplies q.k (1/sqrt(d) in the usual setting)
 * A request with no tokens gets out = 0 and lse = -inf. The grid is fixed
 * by (batch, max_pages, geometry); sequence lengths are read on the device,
 * so the call can be captured in a HIP graph.
 * Checks on the device (they cannot be return codes without a sync): a plan
 * whose recorded geometry differs from this call's leaves every out and lse
 * element NaN and adds 1 to counters->invalid_entries; a planned entry whose
 * page id is outside the pool c names (c may describe fewer pages than the
 * cache the plan was built with) is masked like an invalid entry and
 * counted once per KV head. */
size_t paged_decode_attn_planned_workspace_size(int32_t batch, int32_t num_q_heads, int32_t max_pages,
                                                const kvq_layer_cache *c);
kvq_status paged_decode_attn_planned(const kvq_layer_cache *c, const void *plan, size_t plan_bytes,
                                     const void *q_bf16, int32_t batch, int32_t num_q_heads, int32_t max_pages,
                                     float sm_scale, float *out, float *lse, void *workspace,
                                     size_t workspace_bytes, kvq_counters *counters, hipStream_t stream);

/* Decode with the step's new token appended in the same launch (Minima-KV
 * algorithm 1 "Append": new KV is written in FP8 to a Recent page; section
 * 3.1 "Recent"). The plan covers the N_b tokens already cached; attention
 * covers those and the new token (N_b + 1 keys), and the new token's K and V
 * are written to (new_page[b], new_slot[b]) of c->fp8_pages with exactly the
 * codes and scales kv_encode_fp8 would write.
 *   new_kv       float (new_kv_is_bf16 = 0) or bf16 (1) [batch][Hkv][2][d]
 *   new_page     int32 [batch] FP8 page id; new_slot int32 [batch] slot 0..P-1
 * The new token is attended from the call's own registers, so the scan never
 * reads its slot; a page or slot out of range skips the write (counted in
 * counters->invalid_entries once per KV head) but the token is still
 * attended. Publishing the page in the table for the next step is the
 * caller's business. Other arguments as paged_decode_attn_planned. */
kvq_status paged_decode_attn_append(const kvq_layer_cache *c, const void *plan, size_t plan_bytes,
                                    const void *q_bf16, int32_t batch, int32_t num_q_heads, int32_t max_pages,
                                    float sm_scale, const void *new_kv, int32_t new_kv_is_bf16,
                                    const int32_t *new_page, const int32_t *new_slot, float *out, float *lse,
                                    void *workspace, size_t workspace_bytes, kvq_counters *counters,
                                    hipStream_t stream);

/* Chunked prefill (Block-GTQ appendix H.5, packed chunked prefill over the
 * compressed cache): each request's next `chunk` tokens attend causally to
 * the cache, their own K/V already appended (any format; normally FP8 by
 * kv_encode_fp8). The plan's seq_lens count them: request b's chunk holds
 * positions N_b - chunk .. N_b - 1, and token c sees cache tokens 0 ..
 * N_b - chunk + c (a token whose position is negative sees none: out 0,
 * lse -inf). With R = chunk * (num_q_heads / num_kv_heads) query rows per
 * KV head:
 *   R <= 16: the rows are one MFMA group of the decode scan (split-K items
 *            and the merge kernel; chunk = 1 is paged_decode_attn_planned);
 *   R > 16:  the packed prefill: a workgroup takes 128 rows (token x GQA
 *            head) of one request and KV head and scans every page they can
 *            see, each decoded K/V tile serving all 128 rows; one launch per
 *            format whose pool is present (TQ formats, then FP8), the rows'
 *            running softmax state passing between launches in the
 *            workspace (batch x chunk x num_q_heads x (d + 2) floats when
 *            more than one pool is present; else none is needed and a NULL
 *            workspace is accepted). chunk can be thousands of tokens.
 *   q_bf16  bf16 [batch][chunk][num_q_heads][d], 16-byte aligned
 *   out     float [batch][chunk][num_q_heads][d], 16-byte aligned;
 *           lse float [batch][chunk][num_q_heads] or NULL
 *   workspace  paged_prefill_attn_workspace_size(...) bytes
 * Other arguments as paged_decode_attn_planned. */
size_t paged_prefill_attn_workspace_size(int32_t batch, int32_t num_q_heads, int32_t chunk, int32_t max_pages,
                                         const kvq_layer_cache *c);
kvq_status paged_prefill_attn_planned(const kvq_layer_cache *c, const void *plan, size_t plan_bytes,
                                      const void *q_bf16, int32_t batch, int32_t num_q_heads, int32_t chunk,
                                      int32_t max_pages, float sm_scale, float *out, float *lse, void *workspace,
                                      size_t workspace_bytes, kvq_counters *counters, hipStream_t stream);

/* Scored decode (Minima-KV section 3.1 Eq. 6-8 and section 4.2: a direct
 * mixed-format collector rescales each local page mass by the global softmax).
 * Same as paged_decode_attn_planned (identical out and lse), and also writes
 *   tile_lmass float [batch][num_q_heads][max_pages][page_size/16]: for each
 *              16-token tile of each logical page, ln q~ with q~ the tile's
 *              globally normalized, page-addressable attention mass: the scan
 *              takes ln sum_{i in tile} e^{s_i} (s_i = sm_scale q.k_i, the
 *              decode's own scores: a one-tile partition's Eq. 6 statistics
 *              in one number), the merge subtracts lse (Eq. 8) and the log of
 *              the head's total over the request's tiles, so the exp of a
 *              head's row sums to 1. -inf for tiles the scan does not reach
 *              (pages past N_b, masked entries), and for every tile of a
 *              request with no token.
 * lse must not be NULL. A page's mass q~_{h,p} is the sum of exp over its
 * page_size/16 tiles. */
kvq_status paged_decode_attn_scored(const kvq_layer_cache *c, const void *plan, size_t plan_bytes,
                                    const void *q_bf16, int32_t batch, int32_t num_q_heads, int32_t max_pages,
                                    float sm_scale, float *out, float *lse, float *tile_lmass, void *workspace,
                                    size_t workspace_bytes, kvq_counters *counters, hipStream_t stream);

/* Running page score (Minima-KV Eq. 9) from a scored decode: for each request
 * b and live page p (p < ceil(N_b / P)): r_p = mean over the head set of
 * q~_{h,p}; score[b][p] = beta * score[b][p] + (1 - beta) * r_p.
 *   seq_lens    int32 [batch] as given to the plan (clamped to max_pages * P)
 *   tile_lmass  the scored decode's output
 *   heads       [host] int32 [n_heads] q-head ids (the sampled set H), at most
 *               256; n_heads = 0 leaves score as it is
 *   beta        EWMA weight in [0, 1]
 *   score       float [batch][max_pages], read and written on live pages only
 *   r_out       float [batch][max_pages] r_p (0 on pages that are not live),
 *               or NULL */
kvq_status page_mass_collect(int32_t batch, int32_t num_q_heads, int32_t max_pages, int32_t page_size,
                             const int32_t *seq_lens, const float *tile_lmass, const int32_t *heads, int32_t n_heads,
                             float beta, float *score, float *r_out, hipStream_t stream);

/* Decode attention in one call, as the pages state the problem: a page table,
 * per-page format tags, the query, the softmax scale and the GQA shape
 * (Minima-KV section 3.3 and section 4.1: the format partition, the
 * format-specific scans and the merge of their partials, Eq. 11-13; Block-GTQ
 * H.2-H.4: query rotation in the prologue, one inverse V rotation, a fixed
 * grid with device-side lengths). It is paged_decode_plan into the front of
 * `workspace` followed by paged_decode_attn_planned on the rest.
 *   workspace  paged_decode_attn_workspace_size(batch, num_q_heads, max_pages,
 *              c) bytes, no initial contents needed; that size is exactly
 *              paged_decode_plan_bytes rounded up to 256 plus
 *              paged_decode_attn_planned_workspace_size
 * Other arguments as paged_decode_plan and paged_decode_attn_planned. */
size_t paged_decode_attn_workspace_size(int32_t batch, int32_t num_q_heads, int32_t max_pages,
                                        const kvq_layer_cache *c);
kvq_status paged_decode_attn(const kvq_layer_cache *c, const void *q_bf16, int32_t batch, int32_t num_q_heads,
                             const int32_t *block_table, const uint8_t *page_format, int32_t max_pages,
                             const int32_t *seq_lens, float sm_scale, float *out, float *lse,
                             void *workspace, size_t workspace_bytes, kvq_counters *counters,
                             hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * call as paged_decode_attn, with the workspace taken from a fixed device
 * array the library holds on each GPU it runs on (KVQ_NOALLOC_SCRATCH_BYTES
 * bytes per GPU, kept until the process ends; its address is looked up the
 * first time the call runs on a device, so make that first call outside a
 * graph capture). The call allocates and frees nothing. A geometry whose
 * paged_decode_attn_workspace_size exceeds the array returns
 * KVQ_ERR_UNSUPPORTED before any launch. Every call on one GPU uses the same
 * array and needs none of its old contents: calls ordered on one stream are
 * fine, calls that overlap on one GPU (other streams, other threads) race
 * and must not be issued. Arguments and results as paged_decode_attn. */
#define KVQ_NOALLOC_SCRATCH_BYTES (32u << 20)
kvq_status paged_decode_attn_noalloc(const kvq_layer_cache *c, const void *q_bf16, int32_t batch,
                                     int32_t num_q_heads, const int32_t *block_table, const uint8_t *page_format,
                                     int32_t max_pages, const int32_t *seq_lens, float sm_scale, float *out,
                                     float *lse, kvq_counters *counters, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* KVQ_H_ */
