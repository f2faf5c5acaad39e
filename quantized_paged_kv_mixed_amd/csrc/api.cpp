// extern "C" entry points of libkvq: argument validation (fail closed before
// any launch, Minima-KV section 4.1), workspace sizing, and kernel launches on
// the caller's stream. No allocation, no synchronization.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>

#include "kvq_internal.h"

using namespace kvq;

// Workspace of paged_decode_attn_noalloc: one fixed array per GPU (every GPU
// the library runs on holds its own copy until the process ends). In host
// code this name is only a stand-in for the symbol; the device address comes
// from hipGetSymbolAddress, once per device, and only that address is used.
__device__ __align__(256) uint8_t scratch[KVQ_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_last_error;
thread_local hipEvent_t g_scan_end_event = nullptr;   // measurement hook (kvq_set_scan_end_event)

kvq_status fail(kvq_status s, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

kvq_status ok() {
  g_last_error.clear();
  return KVQ_OK;
}

kvq_status from_hip(hipError_t e, const char *what) {
  if (e == hipSuccess) return ok();
  return fail(KVQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxScratchDevices] = {};

// Device address of `scratch` on the current device, looked up on the first
// call made with that device current and kept.
hipError_t scratch_of_current_device(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

// The pool and page count the cache names for a format.
uint8_t *pool_of(const kvq_layer_cache *c, int fmt) {
  switch (fmt) {
    case FMT_FP8: return c->fp8_pages;
    case FMT_TQ3: return c->tq3_pages;
    case FMT_TQ2: return c->tq2_pages;
    case FMT_TQK: return c->tqk_pages;
    case FMT_TQF5: return c->tqf5_pages;
    case FMT_TQF6: return c->tqf6_pages;
    default: return nullptr;
  }
}
int64_t pool_pages_of(const kvq_layer_cache *c, int fmt) {
  switch (fmt) {
    case FMT_FP8: return c->fp8_num_pages;
    case FMT_TQ3: return c->tq3_num_pages;
    case FMT_TQ2: return c->tq2_num_pages;
    case FMT_TQK: return c->tqk_num_pages;
    case FMT_TQF5: return c->tqf5_num_pages;
    case FMT_TQF6: return c->tqf6_num_pages;
    default: return 0;
  }
}

kvq_status check_cache(const kvq_layer_cache *c) {
  if (!c) return fail(KVQ_ERR_INVALID, "cache descriptor is NULL");
  if (c->head_dim != 128 && c->head_dim != 256)
    return fail(KVQ_ERR_UNSUPPORTED, "head_dim %d not in {128, 256}", c->head_dim);
  if (c->page_size != 16 && c->page_size != 32)
    return fail(KVQ_ERR_UNSUPPORTED, "page_size %d not in {16, 32}", c->page_size);
  if (c->num_kv_heads < 1 || c->num_kv_heads > 1024)
    return fail(KVQ_ERR_UNSUPPORTED, "num_kv_heads %d out of range", c->num_kv_heads);
  bool any_tq = false;
  for (int f = 0; f < NFMT; ++f) {
    const uint8_t *pool = pool_of(c, f);
    const int64_t n = pool_pages_of(c, f);
    if (n < 0) return fail(KVQ_ERR_INVALID, "pool %d has a negative page count", f);
    if (n > 0 && !pool) return fail(KVQ_ERR_INVALID, "pool %d has pages but a NULL pointer", f);
    if (pool && !aligned(pool, 16)) return fail(KVQ_ERR_INVALID, "pool %d is not 16-byte aligned", f);
    if (n > (int64_t)INT32_MAX) return fail(KVQ_ERR_UNSUPPORTED, "pool %d has more than 2^31-1 pages", f);
    any_tq = any_tq || (f != FMT_FP8 && n > 0);
  }
  if (any_tq && !c->rot_signs) return fail(KVQ_ERR_INVALID, "TQ pools need rot_signs");
  if (c->tqk_num_pages > 0) {
    if (c->head_dim != 128) return fail(KVQ_ERR_UNSUPPORTED, "the TQK pool needs head_dim 128, not %d", c->head_dim);
    if (!c->tqk_perm) return fail(KVQ_ERR_INVALID, "the TQK pool needs tqk_perm");
    if (!aligned(c->tqk_perm, 4)) return fail(KVQ_ERR_INVALID, "tqk_perm is not 4-byte aligned");
  }
  return KVQ_OK;
}

int64_t page_bytes_of(const kvq_layer_cache *c, int fmt) {
  return (int64_t)c->num_kv_heads * head_block_bytes(fmt, c->page_size, c->head_dim);
}

kvq_status encode_tq(const kvq_layer_cache *c, int fmt, int32_t src_kind, const void *src, const int32_t *src_page,
                     int64_t n_pages, const int32_t *dst_page, const int32_t *page_valid, hipStream_t stream) {
  kvq_status st = check_cache(c);
  if (st != KVQ_OK) return st;
  uint8_t *pool = pool_of(c, fmt);
  const int64_t pool_pages = pool_pages_of(c, fmt);
  if (n_pages < 0) return fail(KVQ_ERR_INVALID, "n_pages < 0");
  if (n_pages == 0) return ok();
  if (n_pages * c->num_kv_heads * 2 > (int64_t)INT32_MAX) return fail(KVQ_ERR_UNSUPPORTED, "too many pages in one call");
  if (!pool || pool_pages <= 0) return fail(KVQ_ERR_INVALID, "destination pool is empty");
  if (!dst_page) return fail(KVQ_ERR_INVALID, "dst_page is NULL");
  if (!c->rot_signs) return fail(KVQ_ERR_INVALID, "rot_signs is NULL");
  if (src_kind == KVQ_SRC_F32_ROWS) {
    if (!src) return fail(KVQ_ERR_INVALID, "src rows are NULL");
    if (!aligned(src, 4)) return fail(KVQ_ERR_INVALID, "src rows not 4-byte aligned");
  } else if (src_kind == KVQ_SRC_FP8_PAGES) {
    if (!src_page) return fail(KVQ_ERR_INVALID, "src_page is NULL");
    if (!c->fp8_pages || c->fp8_num_pages <= 0) return fail(KVQ_ERR_INVALID, "FP8 source pool is empty");
  } else {
    return fail(KVQ_ERR_INVALID, "unknown src_kind %d", src_kind);
  }
  EncodeTqParams p{};
  p.pool = pool;
  p.pool_pages = pool_pages;
  p.page_bytes = page_bytes_of(c, fmt);
  p.head_bytes = head_block_bytes(fmt, c->page_size, c->head_dim);
  p.fp8_pool = c->fp8_pages;
  p.fp8_pool_pages = c->fp8_num_pages;
  p.fp8_page_bytes = page_bytes_of(c, FMT_FP8);
  p.fp8_head_bytes = head_block_bytes(FMT_FP8, c->page_size, c->head_dim);
  p.src_rows = (const float *)src;
  p.src_page = src_page;
  p.dst_page = dst_page;
  p.page_valid = page_valid;
  p.signs = c->rot_signs;
  p.tqk_perm = fmt == FMT_TQK ? c->tqk_perm : nullptr;
  p.n_pages = n_pages;
  p.Hkv = c->num_kv_heads;
  p.P = c->page_size;
  p.src_kind = src_kind;
  return from_hip(launch_encode_tq(p, c->head_dim, fmt, stream), "kv_encode_tq launch");
}

kvq_status check_plan_args(const kvq_layer_cache *c, int32_t batch, int32_t max_pages) {
  kvq_status st = check_cache(c);
  if (st != KVQ_OK) return st;
  if (batch < 0) return fail(KVQ_ERR_INVALID, "batch < 0");
  if (max_pages < 1) return fail(KVQ_ERR_INVALID, "max_pages < 1");
  if ((int64_t)max_pages * c->page_size > (int64_t)INT32_MAX) return fail(KVQ_ERR_UNSUPPORTED, "max_pages too large");
  int S[NFMT];
  split_pages(batch, c->num_kv_heads, max_pages, c->page_size, c->head_dim, S);
  if (max_items(batch, max_pages, S) * c->num_kv_heads > (int64_t)INT32_MAX)
    return fail(KVQ_ERR_UNSUPPORTED, "grid too large");
  return KVQ_OK;
}

}  // namespace

extern "C" {

const char *kvq_status_string(int32_t s) {
  switch (s) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_INVALID: return "invalid argument";
    case KVQ_ERR_UNSUPPORTED: return "unsupported geometry";
    case KVQ_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

const char *kvq_last_error(void) { return g_last_error.c_str(); }

void kvq_set_scan_end_event(void *event) { g_scan_end_event = (hipEvent_t)event; }

int32_t kvq_abi_version(void) { return 10; }

size_t kvq_page_bytes(int32_t format, int32_t num_kv_heads, int32_t head_dim, int32_t page_size) {
  if (format < 0 || format >= NFMT || num_kv_heads < 1) return 0;
  if ((head_dim != 128 && head_dim != 256) || (page_size != 16 && page_size != 32)) return 0;
  if (format == FMT_TQK && head_dim != 128) return 0;
  return (size_t)num_kv_heads * (size_t)head_block_bytes(format, page_size, head_dim);
}

kvq_status kv_encode_fp8(const kvq_layer_cache *c, const void *src, int32_t src_is_bf16, int64_t n_tok,
                         const int32_t *dst_page, const int32_t *dst_slot, hipStream_t stream) {
  kvq_status st = check_cache(c);
  if (st != KVQ_OK) return st;
  if (n_tok < 0) return fail(KVQ_ERR_INVALID, "n_tok < 0");
  if (n_tok == 0) return ok();
  if (!c->fp8_pages || c->fp8_num_pages <= 0) return fail(KVQ_ERR_INVALID, "FP8 pool is empty");
  if (!src || !dst_page || !dst_slot) return fail(KVQ_ERR_INVALID, "NULL src / dst_page / dst_slot");
  if (!aligned(src, src_is_bf16 ? 2 : 4)) return fail(KVQ_ERR_INVALID, "src not aligned");
  if ((n_tok * c->num_kv_heads * 2 + 3) / 4 > (int64_t)INT32_MAX) return fail(KVQ_ERR_UNSUPPORTED, "n_tok too large");
  EncodeFp8Params p{};
  p.pool = c->fp8_pages;
  p.pool_pages = c->fp8_num_pages;
  p.page_bytes = page_bytes_of(c, FMT_FP8);
  p.head_bytes = head_block_bytes(FMT_FP8, c->page_size, c->head_dim);
  p.src = src;
  p.dst_page = dst_page;
  p.dst_slot = dst_slot;
  p.n_tok = n_tok;
  p.Hkv = c->num_kv_heads;
  p.P = c->page_size;
  return from_hip(launch_encode_fp8(p, c->head_dim, src_is_bf16 ? 1 : 0, stream), "kv_encode_fp8 launch");
}

kvq_status kv_encode_tq3(const kvq_layer_cache *c, int32_t src_kind, const void *src, const int32_t *src_page,
                         int64_t n_pages, const int32_t *dst_page, const int32_t *page_valid, hipStream_t stream) {
  return encode_tq(c, FMT_TQ3, src_kind, src, src_page, n_pages, dst_page, page_valid, stream);
}

kvq_status kv_encode_tq2(const kvq_layer_cache *c, int32_t src_kind, const void *src, const int32_t *src_page,
                         int64_t n_pages, const int32_t *dst_page, const int32_t *page_valid, hipStream_t stream) {
  return encode_tq(c, FMT_TQ2, src_kind, src, src_page, n_pages, dst_page, page_valid, stream);
}

kvq_status kv_encode_tqk(const kvq_layer_cache *c, int32_t src_kind, const void *src, const int32_t *src_page,
                         int64_t n_pages, const int32_t *dst_page, const int32_t *page_valid, hipStream_t stream) {
  return encode_tq(c, FMT_TQK, src_kind, src, src_page, n_pages, dst_page, page_valid, stream);
}

kvq_status kv_encode_tqf5(const kvq_layer_cache *c, int32_t src_kind, const void *src, const int32_t *src_page,
                          int64_t n_pages, const int32_t *dst_page, const int32_t *page_valid, hipStream_t stream) {
  return encode_tq(c, FMT_TQF5, src_kind, src, src_page, n_pages, dst_page, page_valid, stream);
}

kvq_status kv_encode_tqf6(const kvq_layer_cache *c, int32_t src_kind, const void *src, const int32_t *src_page,
                          int64_t n_pages, const int32_t *dst_page, const int32_t *page_valid, hipStream_t stream) {
  return encode_tq(c, FMT_TQF6, src_kind, src, src_page, n_pages, dst_page, page_valid, stream);
}

kvq_status kv_promote_fp8(const kvq_layer_cache *c, int32_t src_format, const int32_t *src_page, int64_t n_pages,
                          const int32_t *dst_page, hipStream_t stream) {
  kvq_status st = check_cache(c);
  if (st != KVQ_OK) return st;
  if (src_format <= FMT_FP8 || src_format >= NFMT)
    return fail(KVQ_ERR_INVALID, "src_format %d is not a compressed format", src_format);
  if (n_pages < 0) return fail(KVQ_ERR_INVALID, "n_pages < 0");
  if (n_pages == 0) return ok();
  if (n_pages * c->num_kv_heads * 2 > (int64_t)INT32_MAX) return fail(KVQ_ERR_UNSUPPORTED, "too many pages in one call");
  const uint8_t *pool = pool_of(c, src_format);
  const int64_t pool_pages = pool_pages_of(c, src_format);
  if (!pool || pool_pages <= 0) return fail(KVQ_ERR_INVALID, "source pool is empty");
  if (!c->fp8_pages || c->fp8_num_pages <= 0) return fail(KVQ_ERR_INVALID, "FP8 destination pool is empty");
  if (!src_page || !dst_page) return fail(KVQ_ERR_INVALID, "NULL src_page / dst_page");
  PromoteParams p{};
  p.src_pool = pool;
  p.src_pool_pages = pool_pages;
  p.src_page_bytes = page_bytes_of(c, src_format);
  p.src_head_bytes = head_block_bytes(src_format, c->page_size, c->head_dim);
  p.fp8_pool = c->fp8_pages;
  p.fp8_pool_pages = c->fp8_num_pages;
  p.fp8_page_bytes = page_bytes_of(c, FMT_FP8);
  p.fp8_head_bytes = head_block_bytes(FMT_FP8, c->page_size, c->head_dim);
  p.src_page = src_page;
  p.dst_page = dst_page;
  p.signs = c->rot_signs;
  p.tqk_perm = src_format == FMT_TQK ? c->tqk_perm : nullptr;
  p.n_pages = n_pages;
  p.Hkv = c->num_kv_heads;
  p.P = c->page_size;
  return from_hip(launch_promote_fp8(p, c->head_dim, src_format, stream), "kv_promote_fp8 launch");
}

size_t paged_decode_plan_bytes(int32_t batch, int32_t max_pages, const kvq_layer_cache *c) {
  if (!c || batch < 0 || max_pages < 1 || c->num_kv_heads < 1) return 0;
  if (c->head_dim != 128 && c->head_dim != 256) return 0;
  if (c->page_size != 16 && c->page_size != 32) return 0;
  return (size_t)PlanLayout(batch, max_pages, c->num_kv_heads, c->page_size, c->head_dim).total;
}

kvq_status paged_decode_plan(const kvq_layer_cache *c, int32_t batch, const int32_t *block_table,
                             const uint8_t *page_format, int32_t max_pages, const int32_t *seq_lens,
                             void *plan, size_t plan_bytes, kvq_counters *counters, hipStream_t stream) {
  kvq_status st = check_plan_args(c, batch, max_pages);
  if (st != KVQ_OK) return st;
  if (batch == 0) return ok();
  if (!block_table || !page_format || !seq_lens || !plan)
    return fail(KVQ_ERR_INVALID, "NULL block_table / page_format / seq_lens / plan");
  if (!aligned(plan, 16)) return fail(KVQ_ERR_INVALID, "plan not 16-byte aligned");
  const PlanLayout L(batch, max_pages, c->num_kv_heads, c->page_size, c->head_dim);
  if (plan_bytes < (size_t)L.total) return fail(KVQ_ERR_INVALID, "plan buffer %zu < %lld bytes", plan_bytes, (long long)L.total);
  if (L.n_slots > (int64_t)INT32_MAX) return fail(KVQ_ERR_UNSUPPORTED, "too many work items");
  PlanParams p{};
  p.hdr = (PlanHeader *)plan;
  p.block_table = block_table;
  p.page_format = page_format;
  p.seq_lens = seq_lens;
  for (int f = 0; f < NFMT; ++f) p.pool_pages[f] = pool_pages_of(c, f);
  uint8_t *base = (uint8_t *)plan;
  p.seq = (int32_t *)(base + L.seq_off);
  p.counts = (int32_t *)(base + L.counts_off);
  p.req = (ReqItems *)(base + L.req_off);
  p.entries = (int2 *)(base + L.entries_off);
  p.packets = base + L.packets_off;
  p.packet_stride = L.packet_stride;
  p.n_slots = L.n_slots;
  p.ticket = (uint32_t *)(base + L.ticket_off);
  split_pages(batch, c->num_kv_heads, max_pages, c->page_size, c->head_dim, p.S);
  p.counters = counters;
  p.B = batch;
  p.max_pages = max_pages;
  p.P = c->page_size;
  p.Hkv = c->num_kv_heads;
  p.d = c->head_dim;
  return from_hip(launch_plan(p, stream), "paged_decode_plan launch");
}

size_t paged_decode_attn_planned_workspace_size(int32_t batch, int32_t num_q_heads, int32_t max_pages,
                                                const kvq_layer_cache *c) {
  if (!c || batch < 0 || max_pages < 1 || c->num_kv_heads < 1 || num_q_heads < c->num_kv_heads) return 0;
  if (c->head_dim != 128 && c->head_dim != 256) return 0;
  if (c->page_size != 16 && c->page_size != 32) return 0;
  const int G = num_q_heads / c->num_kv_heads;
  int S[NFMT];
  split_pages(batch, c->num_kv_heads, max_pages, c->page_size, c->head_dim, S);
  const int64_t slots = max_items(batch, max_pages, S) * c->num_kv_heads;
  return (size_t)WorkspaceLayout(slots, G, c->head_dim).total;
}

namespace {

struct NewToken {
  const void *kv = nullptr;
  int bf16 = 0;
  const int32_t *page = nullptr, *slot = nullptr;
};

kvq_status decode_planned(const kvq_layer_cache *c, const void *plan, size_t plan_bytes, const void *q_bf16,
                          int32_t batch,
                          int32_t num_q_heads, int32_t max_pages, float sm_scale, float *out, float *lse,
                          float *tile_lmass, void *workspace, size_t workspace_bytes, kvq_counters *counters,
                          hipStream_t stream, const NewToken &nt = NewToken(), int chunk = 1) {
  kvq_status st = check_plan_args(c, batch, max_pages);
  if (st != KVQ_OK) return st;
  if (num_q_heads < 1 || num_q_heads % c->num_kv_heads != 0)
    return fail(KVQ_ERR_UNSUPPORTED, "num_q_heads %d is not a multiple of num_kv_heads %d", num_q_heads, c->num_kv_heads);
  const int Gr = num_q_heads / c->num_kv_heads;
  if (chunk < 1) return fail(KVQ_ERR_INVALID, "chunk %d < 1", chunk);
  if ((int64_t)Gr * chunk > 16)
    return fail(KVQ_ERR_UNSUPPORTED, "GQA group %d x chunk %d > 16 rows", Gr, chunk);
  const int G = Gr * chunk;                      // rows of the MFMA group: C tokens x Gr heads
  if (!isfinite(sm_scale)) return fail(KVQ_ERR_INVALID, "sm_scale is not finite");
  if (batch == 0) return ok();
  if (!plan || !q_bf16 || !out || !workspace) return fail(KVQ_ERR_INVALID, "NULL plan / q / out / workspace");
  if (!aligned(plan, 16) || !aligned(workspace, 16) || !aligned(q_bf16, 16) || !aligned(out, 4))
    return fail(KVQ_ERR_INVALID, "misaligned plan / workspace / q / out");
  const size_t need = paged_decode_attn_planned_workspace_size(batch, num_q_heads * chunk, max_pages, c);
  if (workspace_bytes < need) return fail(KVQ_ERR_INVALID, "workspace %zu < %zu bytes", workspace_bytes, need);
  const PlanLayout L(batch, max_pages, c->num_kv_heads, c->page_size, c->head_dim);
  if (plan_bytes < (size_t)L.total)
    return fail(KVQ_ERR_INVALID, "plan buffer %zu < %lld bytes for this geometry", plan_bytes, (long long)L.total);
  const WorkspaceLayout W(L.n_slots * c->num_kv_heads, G, c->head_dim);
  DecodeParams p{};
  for (int f = 0; f < NFMT; ++f) {
    p.pool[f] = pool_of(c, f);
    p.pool_pages[f] = pool_pages_of(c, f);
  }
  for (int f = 0; f < NFMT; ++f) {
    p.head_bytes[f] = head_block_bytes(f, c->page_size, c->head_dim);
    p.page_bytes[f] = page_bytes_of(c, f);
  }
  p.signs = c->rot_signs;
  p.tqk_perm = c->tqk_perm;
  p.q = (const uint16_t *)q_bf16;
  p.out = out;
  p.lse = lse;
  uint8_t *pb = (uint8_t *)plan;
  p.plan_hdr = (const PlanHeader *)pb;
  p.req = (const ReqItems *)(pb + L.req_off);
  p.packets = pb + L.packets_off;
  p.packet_stride = L.packet_stride;
  p.n_slots = L.n_slots;
  p.ticket = (uint32_t *)(pb + L.ticket_off);
  uint8_t *wb = (uint8_t *)workspace;
  p.part_o = (float *)(wb + W.o_off);
  p.part_ml = (float *)(wb + W.ml_off);
  p.counters = counters;
  p.B = batch;
  p.Hq = num_q_heads * chunk;
  p.Hkv = c->num_kv_heads;
  p.max_pages = max_pages;
  p.D = c->head_dim;
  p.G = G;
  p.chunk = chunk;
  p.Gr = Gr;
  p.Hq_r = num_q_heads;
  p.P = c->page_size;
  {
    int S[NFMT];
    split_pages(batch, c->num_kv_heads, max_pages, c->page_size, c->head_dim, S);
    p.mi = max_items_per_request(max_pages, S);
  }
  p.scale_log2 = sm_scale * 1.4426950408889634f;
  p.tile_lmass = tile_lmass;
  p.tlm_stride = (int64_t)max_pages * (c->page_size / 16);
  p.new_kv = nt.kv;
  p.new_kv_bf16 = nt.bf16;
  p.new_page = nt.page;
  p.new_slot = nt.slot;
  p.fp8_pool_w = c->fp8_pages;
  return from_hip(launch_decode(p, c->head_dim, stream, g_scan_end_event), "paged_decode_attn launch");
}

// Chunks whose chunk x G query rows exceed one MFMA group (16 rows) take the
// packed prefill: query-row tiles of 128 rows instead of one group per scan.
bool packed_prefill(const kvq_layer_cache *c, int32_t num_q_heads, int32_t chunk) {
  return (int64_t)chunk * (num_q_heads / c->num_kv_heads) > 16;
}
// Launches of a packed prefill: one per format whose pool is present.
int prefill_launches(const kvq_layer_cache *c) {
  int n = 0;
  for (int f = 0; f < NFMT; ++f) n += (pool_of(c, f) && pool_pages_of(c, f) > 0) ? 1 : 0;
  return n;
}

kvq_status prefill_packed(const kvq_layer_cache *c, const void *plan, size_t plan_bytes, const void *q_bf16,
                          int32_t batch, int32_t num_q_heads, int32_t chunk, int32_t max_pages, float sm_scale,
                          float *out, float *lse, void *workspace, size_t workspace_bytes, kvq_counters *counters,
                          hipStream_t stream) {
  kvq_status st = check_plan_args(c, batch, max_pages);
  if (st != KVQ_OK) return st;
  if (num_q_heads < 1 || num_q_heads % c->num_kv_heads != 0)
    return fail(KVQ_ERR_UNSUPPORTED, "num_q_heads %d is not a multiple of num_kv_heads %d", num_q_heads, c->num_kv_heads);
  const int G = num_q_heads / c->num_kv_heads;
  if (!isfinite(sm_scale)) return fail(KVQ_ERR_INVALID, "sm_scale is not finite");
  const int64_t rows = (int64_t)chunk * G;
  if ((int64_t)batch * chunk * num_q_heads > ((int64_t)1 << 40) || rows > ((int64_t)1 << 30))
    return fail(KVQ_ERR_UNSUPPORTED, "chunk %d too large", chunk);
  if (batch > 65535) return fail(KVQ_ERR_UNSUPPORTED, "batch %d > 65535", batch);
  if (batch == 0) return ok();
  if (!plan || !q_bf16 || !out) return fail(KVQ_ERR_INVALID, "NULL plan / q / out");
  if (!aligned(plan, 16) || !aligned(q_bf16, 16) || !aligned(out, 16) || !aligned(lse, 4))
    return fail(KVQ_ERR_INVALID, "misaligned plan / q / out / lse");
  const PlanLayout L(batch, max_pages, c->num_kv_heads, c->page_size, c->head_dim);
  if (plan_bytes < (size_t)L.total)
    return fail(KVQ_ERR_INVALID, "plan buffer %zu < %lld bytes for this geometry", plan_bytes, (long long)L.total);
  const int n_launch = prefill_launches(c);
  const int64_t need = n_launch > 1 ? prefill_ws_bytes(batch, chunk, num_q_heads, c->head_dim) : 0;
  if (need > 0 && (!workspace || !aligned(workspace, 16) || workspace_bytes < (size_t)need))
    return fail(KVQ_ERR_INVALID, "workspace %zu < %lld bytes (or misaligned)", workspace_bytes, (long long)need);
  PrefillParams p{};
  for (int f = 0; f < NFMT; ++f) {
    p.pool[f] = pool_of(c, f);
    p.pool_pages[f] = pool_pages_of(c, f);
    p.head_bytes[f] = head_block_bytes(f, c->page_size, c->head_dim);
    p.page_bytes[f] = page_bytes_of(c, f);
  }
  p.signs = c->rot_signs;
  p.tqk_perm = c->tqk_perm;
  p.q = (const uint16_t *)q_bf16;
  p.out = out;
  p.lse = lse;
  const uint8_t *pb = (const uint8_t *)plan;
  p.plan_hdr = (const PlanHeader *)pb;
  p.seq = (const int32_t *)(pb + L.seq_off);
  p.counts = (const int32_t *)(pb + L.counts_off);
  p.entries = (const int2 *)(pb + L.entries_off);
  p.counters = counters;
  p.B = batch;
  p.Hq = num_q_heads;
  p.Hkv = c->num_kv_heads;
  p.G = G;
  p.P = c->page_size;
  p.max_pages = max_pages;
  p.D = c->head_dim;
  p.chunk = chunk;
  p.row_blocks = (int)((rows + kPfBlockRows - 1) / kPfBlockRows);
  p.scale_log2 = sm_scale * 1.4426950408889634f;
  if (need > 0) {
    const int64_t nrow = (int64_t)batch * chunk * num_q_heads;
    p.ws_o = (float *)workspace;
    p.ws_ml = (float *)((uint8_t *)workspace + ((nrow * c->head_dim * 4 + 255) & ~255LL));
  }
  return from_hip(launch_prefill(p, stream), "paged_prefill_attn launch");
}

}  // namespace

kvq_status paged_decode_attn_planned(const kvq_layer_cache *c, const void *plan, size_t plan_bytes,
                                     const void *q_bf16, int32_t batch, int32_t num_q_heads, int32_t max_pages,
                                     float sm_scale, float *out, float *lse, void *workspace,
                                     size_t workspace_bytes, kvq_counters *counters, hipStream_t stream) {
  return decode_planned(c, plan, plan_bytes, q_bf16, batch, num_q_heads, max_pages, sm_scale, out, lse, nullptr,
                        workspace, workspace_bytes, counters, stream);
}

kvq_status paged_decode_attn_scored(const kvq_layer_cache *c, const void *plan, size_t plan_bytes,
                                    const void *q_bf16, int32_t batch, int32_t num_q_heads, int32_t max_pages,
                                    float sm_scale, float *out, float *lse, float *tile_lmass, void *workspace,
                                    size_t workspace_bytes, kvq_counters *counters, hipStream_t stream) {
  if (!tile_lmass || !lse) return fail(KVQ_ERR_INVALID, "a scored call needs tile_lmass and lse");
  if (!aligned(tile_lmass, 4) || !aligned(lse, 4)) return fail(KVQ_ERR_INVALID, "misaligned tile_lmass / lse");
  return decode_planned(c, plan, plan_bytes, q_bf16, batch, num_q_heads, max_pages, sm_scale, out, lse,
                        tile_lmass, workspace, workspace_bytes, counters, stream);
}

kvq_status paged_decode_attn_append(const kvq_layer_cache *c, const void *plan, size_t plan_bytes,
                                    const void *q_bf16, int32_t batch, int32_t num_q_heads, int32_t max_pages,
                                    float sm_scale, const void *new_kv, int32_t new_kv_is_bf16,
                                    const int32_t *new_page, const int32_t *new_slot, float *out, float *lse,
                                    void *workspace, size_t workspace_bytes, kvq_counters *counters,
                                    hipStream_t stream) {
  if (!new_kv || !new_page || !new_slot) return fail(KVQ_ERR_INVALID, "NULL new_kv / new_page / new_slot");
  if (!aligned(new_kv, new_kv_is_bf16 ? 2 : 4) || !aligned(new_page, 4) || !aligned(new_slot, 4))
    return fail(KVQ_ERR_INVALID, "misaligned new_kv / new_page / new_slot");
  if (c && (!c->fp8_pages || c->fp8_num_pages <= 0)) return fail(KVQ_ERR_INVALID, "fused append needs an FP8 pool");
  NewToken nt;
  nt.kv = new_kv;
  nt.bf16 = new_kv_is_bf16 ? 1 : 0;
  nt.page = new_page;
  nt.slot = new_slot;
  return decode_planned(c, plan, plan_bytes, q_bf16, batch, num_q_heads, max_pages, sm_scale, out, lse, nullptr,
                        workspace, workspace_bytes, counters, stream, nt);
}

size_t paged_prefill_attn_workspace_size(int32_t batch, int32_t num_q_heads, int32_t chunk, int32_t max_pages,
                                         const kvq_layer_cache *c) {
  if (chunk < 1 || (int64_t)num_q_heads * chunk > INT32_MAX) return 0;
  if (!c || c->num_kv_heads < 1 || num_q_heads < c->num_kv_heads) return 0;
  if (packed_prefill(c, num_q_heads, chunk)) {
    if (batch < 0 || max_pages < 1) return 0;
    return prefill_launches(c) > 1 ? (size_t)prefill_ws_bytes(batch, chunk, num_q_heads, c->head_dim) : 256;
  }
  return paged_decode_attn_planned_workspace_size(batch, num_q_heads * chunk, max_pages, c);
}

kvq_status paged_prefill_attn_planned(const kvq_layer_cache *c, const void *plan, size_t plan_bytes,
                                      const void *q_bf16, int32_t batch, int32_t num_q_heads, int32_t chunk,
                                      int32_t max_pages, float sm_scale, float *out, float *lse, void *workspace,
                                      size_t workspace_bytes, kvq_counters *counters, hipStream_t stream) {
  if (chunk < 1) return fail(KVQ_ERR_INVALID, "chunk %d < 1", chunk);
  if (c && c->num_kv_heads >= 1 && num_q_heads >= c->num_kv_heads && packed_prefill(c, num_q_heads, chunk))
    return prefill_packed(c, plan, plan_bytes, q_bf16, batch, num_q_heads, chunk, max_pages, sm_scale, out, lse,
                          workspace, workspace_bytes, counters, stream);
  return decode_planned(c, plan, plan_bytes, q_bf16, batch, num_q_heads, max_pages, sm_scale, out, lse, nullptr,
                        workspace, workspace_bytes, counters, stream, NewToken(), chunk);
}

kvq_status page_mass_collect(int32_t batch, int32_t num_q_heads, int32_t max_pages, int32_t page_size,
                             const int32_t *seq_lens, const float *tile_lmass, const int32_t *heads, int32_t n_heads,
                             float beta, float *score, float *r_out, hipStream_t stream) {
  if (batch < 0 || num_q_heads < 1 || max_pages < 1) return fail(KVQ_ERR_INVALID, "bad batch / heads / max_pages");
  if (page_size != 16 && page_size != 32) return fail(KVQ_ERR_UNSUPPORTED, "page_size %d not in {16, 32}", page_size);
  if (n_heads < 0 || n_heads > kMaxCollectHeads)
    return fail(KVQ_ERR_UNSUPPORTED, "n_heads %d outside 0..%d", n_heads, kMaxCollectHeads);
  if (n_heads > 0 && !heads) return fail(KVQ_ERR_INVALID, "heads is NULL");
  for (int k = 0; k < n_heads; ++k)
    if (heads[k] < 0 || heads[k] >= num_q_heads) return fail(KVQ_ERR_INVALID, "head %d out of range", heads[k]);
  if (!(beta >= 0.f && beta <= 1.f)) return fail(KVQ_ERR_INVALID, "beta outside [0, 1]");
  if (batch == 0) return ok();
  if (!seq_lens || !tile_lmass || !score) return fail(KVQ_ERR_INVALID, "NULL seq_lens / tile_lmass / score");
  if (!aligned(tile_lmass, 4) || !aligned(score, 4) || !aligned(r_out, 4) || !aligned(seq_lens, 4))
    return fail(KVQ_ERR_INVALID, "misaligned argument");
  CollectParams p{};
  p.seq_lens = seq_lens;
  p.tile_lmass = tile_lmass;
  p.score = score;
  p.r_out = r_out;
  p.tlm_stride = (int64_t)max_pages * (page_size / 16);
  p.beta = beta;
  p.B = batch;
  p.Hq = num_q_heads;
  p.max_pages = max_pages;
  p.P = page_size;
  p.n_heads = n_heads;
  for (int k = 0; k < n_heads; ++k) p.heads[k] = heads[k];
  return from_hip(launch_collect(p, stream), "page_mass_collect launch");
}

size_t paged_decode_attn_workspace_size(int32_t batch, int32_t num_q_heads, int32_t max_pages,
                                        const kvq_layer_cache *c) {
  if (!c) return 0;
  const size_t a = paged_decode_plan_bytes(batch, max_pages, c);
  const size_t b = paged_decode_attn_planned_workspace_size(batch, num_q_heads, max_pages, c);
  if (!a || !b) return 0;
  return ((a + 255) & ~(size_t)255) + b;
}

kvq_status paged_decode_attn(const kvq_layer_cache *c, const void *q_bf16, int32_t batch, int32_t num_q_heads,
                             const int32_t *block_table, const uint8_t *page_format, int32_t max_pages,
                             const int32_t *seq_lens, float sm_scale, float *out, float *lse,
                             void *workspace, size_t workspace_bytes, kvq_counters *counters,
                             hipStream_t stream) {
  kvq_status st = check_plan_args(c, batch, max_pages);
  if (st != KVQ_OK) return st;
  if (batch == 0) return ok();
  if (!workspace) return fail(KVQ_ERR_INVALID, "workspace is NULL");
  const size_t need = paged_decode_attn_workspace_size(batch, num_q_heads, max_pages, c);
  if (need == 0) return fail(KVQ_ERR_UNSUPPORTED, "unsupported geometry for the workspace");
  if (workspace_bytes < need) return fail(KVQ_ERR_INVALID, "workspace %zu < %zu bytes", workspace_bytes, need);
  const size_t plan_sz = (paged_decode_plan_bytes(batch, max_pages, c) + 255) & ~(size_t)255;
  st = paged_decode_plan(c, batch, block_table, page_format, max_pages, seq_lens, workspace, plan_sz, counters, stream);
  if (st != KVQ_OK) return st;
  return paged_decode_attn_planned(c, workspace, plan_sz, q_bf16, batch, num_q_heads, max_pages, sm_scale, out, lse,
                                   (uint8_t *)workspace + plan_sz, workspace_bytes - plan_sz, counters, stream);
}

kvq_status paged_decode_attn_noalloc(const kvq_layer_cache *c, const void *q_bf16, int32_t batch,
                                     int32_t num_q_heads, const int32_t *block_table, const uint8_t *page_format,
                                     int32_t max_pages, const int32_t *seq_lens, float sm_scale, float *out,
                                     float *lse, kvq_counters *counters, hipStream_t stream) {
  kvq_status st = check_plan_args(c, batch, max_pages);
  if (st != KVQ_OK) return st;
  if (batch == 0) return ok();
  const size_t need = paged_decode_attn_workspace_size(batch, num_q_heads, max_pages, c);
  if (need == 0) return fail(KVQ_ERR_UNSUPPORTED, "unsupported geometry for the workspace");
  if (need > (size_t)KVQ_NOALLOC_SCRATCH_BYTES)
    return fail(KVQ_ERR_UNSUPPORTED, "this call needs %zu bytes of workspace, more than the %zu bytes of the "
                "library's fixed array; use paged_decode_attn with a caller-owned workspace", need,
                (size_t)KVQ_NOALLOC_SCRATCH_BYTES);
  void *ws = nullptr;
  const hipError_t e = scratch_of_current_device(&ws);
  if (e != hipSuccess) return from_hip(e, "locating the fixed workspace array");
  return paged_decode_attn(c, q_bf16, batch, num_q_heads, block_table, page_format, max_pages, seq_lens, sm_scale,
                           out, lse, ws, (size_t)KVQ_NOALLOC_SCRATCH_BYTES, counters, stream);
}

}  // extern "C"
