// Internal geometry shared by the host API and the gfx950 kernels of libkvq.
// (Not part of the public ABI; the public contract is include/kvq.h.)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kvq.h"

namespace kvq {

enum : int { FMT_FP8 = 0, FMT_TQ3 = 1, FMT_TQ2 = 2, NFMT = 3, FMT_EMPTY = 7 };

constexpr int kDecodeWaves = 4;                 // waves per decode workgroup
constexpr int kDecodeThreads = 64 * kDecodeWaves;
constexpr int64_t kWaveTargetBytes = 48 * 1024;  // KV bytes one wave streams per item

__host__ __device__ inline int tq_bits(int fmt) { return fmt == FMT_TQ3 ? 3 : (fmt == FMT_TQ2 ? 2 : 0); }

// Bytes of one (page, KV head) block of a format.
__host__ __device__ inline int64_t head_block_bytes(int fmt, int P, int d) {
  if (fmt == FMT_FP8) return 2LL * P * d + 8LL * P;
  if (fmt == FMT_TQ3 || fmt == FMT_TQ2) return 2LL * P * d * tq_bits(fmt) / 8 + 4LL * P;
  return 0;
}

// Pages of one format a single decode wave scans per work item: about
// kWaveTargetBytes of KV, so every wave of a workgroup moves a similar
// number of bytes whatever the page format (byte-balanced splits).
__host__ __device__ inline int pages_per_wave(int fmt, int P, int d) {
  const int64_t hb = head_block_bytes(fmt, P, d);
  if (hb <= 0) return 1;
  int64_t n = (kWaveTargetBytes + hb / 2) / hb;
  return n < 1 ? 1 : (int)n;
}
__host__ __device__ inline int pages_per_item(int fmt, int P, int d) {
  return kDecodeWaves * pages_per_wave(fmt, P, d);
}

// Upper bound on work items of a batch: per request, sum_f ceil(n_f / S_f)
// <= max_pages / min_f S_f + NFMT, and an empty request still has one item.
inline int64_t max_items(int B, int max_pages, int P, int d) {
  int smin = 1 << 30;
  for (int f = 0; f < NFMT; ++f) {
    int s = pages_per_item(f, P, d);
    smin = s < smin ? s : smin;
  }
  return (int64_t)B * ((max_pages + smin - 1) / smin + NFMT + 1);
}

// Plan buffer: per-request clamped lengths, per-(request, format) entry
// counts, per-(request, KV head) merge counters, and the compact entry lists
// entries[b][k] = (logical page, physical id), formats in tag order, logical
// order kept inside each format.
struct PlanLayout {
  int64_t seq_off, counts_off, merge_off, entries_off, total;
  __host__ __device__ PlanLayout(int B, int max_pages, int Hkv) {
    int64_t o = 64;
    seq_off = o;
    o += 4LL * B;
    o = (o + 15) & ~15LL;
    counts_off = o;
    o += 16LL * B;
    merge_off = o;
    o += 4LL * B * Hkv;
    o = (o + 15) & ~15LL;
    entries_off = o;
    o += 8LL * B * (int64_t)max_pages;
    total = (o + 255) & ~255LL;
  }
};

// Decode workspace: per (item, KV head) normalized partial outputs O_bar
// [G][d] and (m, l) [G][2] (m in log2 units).
struct WorkspaceLayout {
  int64_t o_off, ml_off, total;
  WorkspaceLayout(int64_t n_slots, int G, int d) {
    o_off = 0;
    int64_t o = 4LL * n_slots * G * d;
    o = (o + 255) & ~255LL;
    ml_off = o;
    o += 8LL * n_slots * G;
    total = (o + 255) & ~255LL;
  }
};

struct DecodeParams {
  const uint8_t *pool[NFMT];
  int64_t pool_pages[NFMT];
  int64_t page_bytes[NFMT];
  int64_t head_bytes[NFMT];
  int S[NFMT];                 // pages per item, per format
  const uint32_t *signs;       // [Hkv][2][d/32]
  const uint16_t *q;           // bf16 [B][Hq][d]
  float *out;                  // [B][Hq][d]
  float *lse;                  // [B][Hq] or null
  const int32_t *seq;          // plan: clamped N_b
  const int32_t *counts;       // plan: [B][4]
  uint32_t *merge_ctr;         // plan: [B][Hkv]
  const int2 *entries;         // plan: [B][max_pages]
  float *part_o;
  float *part_ml;
  kvq_counters *counters;
  int B, Hq, Hkv, G, P, max_pages;
  float scale_log2;            // sm_scale * log2(e)
};

struct PlanParams {
  const int32_t *block_table;
  const uint8_t *page_format;
  const int32_t *seq_lens;
  int64_t pool_pages[NFMT];
  int32_t *seq;
  int32_t *counts;
  uint32_t *merge_ctr;
  int2 *entries;
  kvq_counters *counters;
  int B, max_pages, P, Hkv;
};

struct EncodeFp8Params {
  uint8_t *pool;
  int64_t pool_pages, page_bytes, head_bytes;
  const void *src;
  const int32_t *dst_page, *dst_slot;
  int64_t n_tok;
  int Hkv, P;
};

struct EncodeTqParams {
  uint8_t *pool;
  int64_t pool_pages, page_bytes, head_bytes;
  const uint8_t *fp8_pool;
  int64_t fp8_pool_pages, fp8_page_bytes, fp8_head_bytes;
  const float *src_rows;
  const int32_t *src_page, *dst_page, *page_valid;
  const uint32_t *signs;
  int64_t n_pages;
  int Hkv, P, src_kind;
};

// Launchers (return hipSuccess or the launch error).
hipError_t launch_plan(const PlanParams &p, hipStream_t s);
hipError_t launch_decode(const DecodeParams &p, int d, int64_t n_items, hipStream_t s);
hipError_t launch_encode_fp8(const EncodeFp8Params &p, int d, int src_is_bf16, hipStream_t s);
hipError_t launch_encode_tq(const EncodeTqParams &p, int d, int bits, hipStream_t s);

}  // namespace kvq
