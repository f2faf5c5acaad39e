// Internal geometry shared by the host API and the gfx950 kernels of libkvq.
// (Not part of the public ABI; the public contract is include/kvq.h.)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kvq.h"

namespace kvq {

enum : int { FMT_FP8 = 0, FMT_TQ3 = 1, FMT_TQ2 = 2, FMT_TQK = 3, FMT_TQF5 = 4, FMT_TQF6 = 5, NFMT = 6,
              FMT_EMPTY = 7 };

#ifndef KVQ_DECODE_WAVES
#define KVQ_DECODE_WAVES 8
#endif
constexpr int kDecodeWaves = KVQ_DECODE_WAVES;  // waves per decode workgroup
constexpr int kDecodeThreads = 64 * kDecodeWaves;
constexpr int kWorkgroupsPerCU = 8 / kDecodeWaves;   // two waves per SIMD either way
constexpr int kMaxPagesPerWave = 64;            // one entry per lane of a wave
constexpr int kCUs = 256 * kWorkgroupsPerCU;    // workgroup slots of an MI355X (work sizing only)
constexpr int kTargetWorkgroups = 230 * kWorkgroupsPerCU;   // items of a one-item-per-slot split
constexpr int kMaxUnitTiles = 64 * kDecodeWaves;  // 16-token tiles of one KV head in the largest unit
constexpr int kMinUnitTiles = 32;               // and in the smallest

__host__ __device__ inline int tq_bits(int fmt) {
  return fmt == FMT_TQ3 || fmt == FMT_TQK ? 3 : (fmt == FMT_TQ2 ? 2 : 0);
}

// Fractional-level codes: level count, codes per mixed-radix group, bits per
// group, and the bytes of one token row (ceil(d / k) groups, whole bytes).
__host__ __device__ constexpr int tqf_levels(int fmt) { return fmt == FMT_TQF5 ? 5 : (fmt == FMT_TQF6 ? 6 : 0); }
__host__ __device__ constexpr int tqf_group_codes(int L) { return L == 5 ? 3 : 5; }
__host__ __device__ constexpr int tqf_group_bits(int L) { return L == 5 ? 7 : 13; }
__host__ __device__ constexpr int tqf_row_bytes(int d, int L) {
  return ((d + tqf_group_codes(L) - 1) / tqf_group_codes(L) * tqf_group_bits(L) + 7) / 8;
}

// Bytes of one (page, KV head) block of a format.
__host__ __device__ inline int64_t head_block_bytes(int fmt, int P, int d) {
  if (fmt == FMT_FP8) return 2LL * P * d + 8LL * P;
  if (fmt == FMT_TQ3 || fmt == FMT_TQ2) return 2LL * P * d * tq_bits(fmt) / 8 + 4LL * P;
  if (fmt == FMT_TQK) return 2LL * P * d * 3 / 8 + 8LL * P;   // three K sigmas, one V sigma
  if (fmt == FMT_TQF5 || fmt == FMT_TQF6) return 2LL * P * tqf_row_bytes(d, tqf_levels(fmt)) + 4LL * P;
  return 0;
}

// Split-K sizing. A work item is a run of pages of one format of one request
// for one KV head, scanned by one workgroup; a persistent grid of one
// workgroup per CU takes items from a dispenser. Wave w of a workgroup scans
// the item's pages w, w + kW, .... A TQ scan costs about the same per
// 16-token tile whatever the code width (the code decode dominates), so TQ
// items of every width hold the same number of pages; an FP8 page reads ~2.6x
// the bytes of a TQ3 page, so FP8 items hold the pages of an equal byte
// count. Items are sized from the largest cache the batch can describe: a
// little under one item per CU (kTargetWorkgroups, which leaves room for each
// list's remainder item), or k equal items per CU when one would exceed
// kMaxUnitTiles. On the 2 x 59,008-token d = 256 layer this gives 248 units
// (TQ3 items of ~127 pages, FP8 items of ~45); filling all 256 CUs exactly
// (TQ3 items of ~118 pages, FP8 items of 68) measured 1 us slower per call.
// Fixed by host-known sizes only, so the grid can be captured in a graph; at
// most kMaxPagesPerWave pages per wave.
inline int clamp_pages(int64_t n) {
  if (n < kDecodeWaves) n = kDecodeWaves;
  if (n > (int64_t)kDecodeWaves * kMaxPagesPerWave) n = (int64_t)kDecodeWaves * kMaxPagesPerWave;
  return (int)n;
}
inline void split_pages(int B, int Hkv, int max_pages, int P, int d, int S[NFMT]) {
  const int64_t T = P / 16;
  const int64_t total = (int64_t)B * Hkv * max_pages * T;      // tiles if every page were live
  int64_t tiles = total / kTargetWorkgroups;
  if (tiles > kMaxUnitTiles) {
    const int64_t k = (total + (int64_t)kCUs * kMaxUnitTiles - 1) / ((int64_t)kCUs * kMaxUnitTiles);
    tiles = (total + k * kCUs - 1) / (k * kCUs);
  }
  tiles = tiles < kMinUnitTiles ? kMinUnitTiles : (tiles > kMaxUnitTiles ? kMaxUnitTiles : tiles);
  const int s_tq = clamp_pages(tiles / T);
  for (int f = 0; f < NFMT; ++f) S[f] = s_tq;
  S[FMT_FP8] = clamp_pages((int64_t)s_tq * head_block_bytes(FMT_TQ3, P, d) / head_block_bytes(FMT_FP8, P, d));
}

// A list of n pages (one format of one request) splits into k items of
// near-equal size: k = n / S rounded to nearest (at least 1), and at least
// enough items to keep every item within kDecodeWaves * kMaxPagesPerWave
// pages. Item j covers pages [j n / k, (j + 1) n / k); k <= ceil(n / S), and
// an item holds fewer than 1.5 S pages.
__host__ __device__ inline int items_in_list(int n, int S) {
  if (n <= 0) return 0;
  int k = (2 * n + S) / (2 * S);
  const int kmin = (n + kDecodeWaves * kMaxPagesPerWave - 1) / (kDecodeWaves * kMaxPagesPerWave);
  k = k < kmin ? kmin : k;
  return k < 1 ? 1 : k;
}

// Upper bound on work items of one request: sum_f ceil(n_f / S_f) <=
// max_pages / min_f S_f + NFMT, and an empty request still has one item. The
// partial rows of q-head hq of request b sit at [(b Hq + hq) MI, (b Hq + hq +
// 1) MI) (MI = this bound, local item order), so the merge of one head reads
// one contiguous run found from (b, hq) alone.
inline int max_items_per_request(int max_pages, const int S[NFMT]) {
  int smin = S[0];
  for (int f = 1; f < NFMT; ++f) smin = S[f] < smin ? S[f] : smin;
  return (max_pages + smin - 1) / smin + NFMT + 1;
}
inline int64_t max_items(int B, int max_pages, const int S[NFMT]) {
  return (int64_t)B * max_items_per_request(max_pages, S);
}

// A work item's packet, written by the plan for every item slot of the batch
// (slots past the last item carry valid = 0): the header and the item's page
// entries sit together so a decode workgroup reads both in one round trip.
struct ItemHeader {
  int32_t b;          // request
  int32_t fmt;        // page format of the item
  int32_t cnt;        // pages in the item
  int32_t seq;        // clamped N_b
  int32_t n_items;    // items of request b (all formats)
  int32_t item_base;  // global id of request b's first item
  int32_t n8;         // FP8 items of request b (they come first)
  int32_t valid;
};

inline int max_pages_per_item(const int S[NFMT]) {
  int m = S[0];
  for (int f = 1; f < NFMT; ++f) m = S[f] > m ? S[f] : m;
  m = m + m / 2 + 1;
  return m > kDecodeWaves * kMaxPagesPerWave ? kDecodeWaves * kMaxPagesPerWave : m;
}

// Plan buffer: per-request clamped lengths, per-(request, format) entry
// counts, per-request item ranges (ReqItems), the compact entry lists
// entries[b][k] = (logical page, physical id) (formats in tag order, logical
// order kept inside each format), and one packet per item slot:
// [ItemHeader][S_max x int2 entries].
// Items of one request: global id of the first, how many, and how many of
// them (the first ones) are FP8 items.
struct ReqItems {
  int32_t item_base, n_items, n8, pad;
};

// The plan's first 64 bytes record the geometry it was built for; decode
// kernels compare it with their own arguments before reading anything else.
constexpr int32_t kPlanMagic = 0x4B565150;   // "PQVK" in memory order
struct PlanHeader {
  int32_t magic, B, max_pages, Hkv, P, d, pad0, pad1;
};

struct PlanLayout {
  int64_t seq_off, counts_off, req_off, entries_off, packets_off, packet_stride, n_slots, ticket_off, total;
  PlanLayout(int B, int max_pages, int Hkv, int P, int d) {
    int S[NFMT];
    split_pages(B, Hkv, max_pages, P, d, S);
    n_slots = max_items(B, max_pages, S);
    packet_stride = (int64_t)sizeof(ItemHeader) + 8LL * max_pages_per_item(S);
    int64_t o = 64;
    seq_off = o;
    o += 4LL * B;
    o = (o + 15) & ~15LL;
    counts_off = o;
    o += 4LL * NFMT * B;
    o = (o + 15) & ~15LL;
    req_off = o;
    o += 16LL * B;
    entries_off = o;
    o += 8LL * B * (int64_t)max_pages;
    o = (o + 255) & ~255LL;
    packets_off = o;
    o += n_slots * packet_stride;
    o = (o + 255) & ~255LL;
    ticket_off = o;                    // [0] next unit for a workgroup that finished one (zero between
                                       // calls), [1] the batch's item count
    o += 256;
    total = o;
  }
};

// Decode workspace: per (request slot, item of the request, KV head)
// normalized partial outputs O_bar [G][d] and (m, l) [G][2] (m in log2 units).
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
  const uint32_t *signs;       // [Hkv][2][d/32]
  const uint16_t *tqk_perm;    // [Hkv][d] key coordinate order of TQK pages, or null
  const uint16_t *q;           // bf16 [B][Hq][d]
  float *out;                  // [B][Hq][d]
  float *lse;                  // [B][Hq] or null
  const PlanHeader *plan_hdr;  // plan: the geometry it was built for
  const uint8_t *packets;      // plan: item packets
  int64_t packet_stride;
  int64_t n_slots;             // item slots (valid ones form a prefix)
  const ReqItems *req;         // plan: [B]
  float *part_o;
  float *part_ml;
  uint32_t *ticket;            // plan: unit dispenser of the persistent grid, then the item count
  kvq_counters *counters;
  int B, Hq, Hkv, G, P;
  int max_pages, D;            // with B, Hkv, P: must match the plan's header
  int mi;                      // partial slots per request (max_items_per_request)
  float scale_log2;            // sm_scale * log2(e)
  float *tile_lmass;           // scored calls: [B][Hq][tlm_stride] tile log-mass, else null
  int64_t tlm_stride;          // max_pages * (P / 16)
  int mass_lds_off;            // scored scan: float offset of the tile log-mass stage in LDS
  // chunked prefill: C query tokens per request; the kernels see C * Gr
  // virtual heads per KV head (G = C * Gr, Hq = C * Hq_r), row c * Gr + n
  // being head g * Gr + n of token c. Decode: chunk 1, Gr = G, Hq_r = Hq.
  int chunk, Gr, Hq_r;
  // fused append: the step's new token, [B][Hkv][2][d] float or bf16, else null
  const void *new_kv;
  const int32_t *new_page;     // [B] FP8 page of the new token
  const int32_t *new_slot;     // [B] its slot
  uint8_t *fp8_pool_w;         // the FP8 pool, writable
  int new_kv_bf16;
};

constexpr int kMaxCollectHeads = 256;   // head set of one page_mass_collect call

struct CollectParams {
  const int32_t *seq_lens;     // [B]
  const float *tile_lmass;     // [B][Hq][tlm_stride]
  float *score;                // [B][max_pages] running score a (in / out)
  float *r_out;                // [B][max_pages] or null
  int64_t tlm_stride;
  float beta;
  int B, Hq, max_pages, P, n_heads;
  int32_t heads[kMaxCollectHeads];
};

struct PlanParams {
  PlanHeader *hdr;
  const int32_t *block_table;
  const uint8_t *page_format;
  const int32_t *seq_lens;
  int64_t pool_pages[NFMT];
  int32_t *seq;
  int32_t *counts;
  ReqItems *req;
  int2 *entries;
  uint8_t *packets;
  int64_t packet_stride;
  int64_t n_slots;
  uint32_t *ticket;
  int S[NFMT];
  kvq_counters *counters;
  int B, max_pages, P, Hkv, d;
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
  const uint16_t *tqk_perm;    // grouped keys (TQK pool), else null
  int64_t n_pages;
  int Hkv, P, src_kind;
};

struct PromoteParams {
  const uint8_t *src_pool;     // TQ3, TQ2 or TQK pool
  int64_t src_pool_pages, src_page_bytes, src_head_bytes;
  uint8_t *fp8_pool;
  int64_t fp8_pool_pages, fp8_page_bytes, fp8_head_bytes;
  const int32_t *src_page, *dst_page;
  const uint32_t *signs;
  const uint16_t *tqk_perm;    // grouped keys (TQK source), else null
  int64_t n_pages;
  int Hkv, P;
};

// Packed chunked prefill: one workgroup per (request, KV head, 128 query
// rows); the plan's per-format entry lists give the pages.
constexpr int kPfThreads = 256;                  // four waves
constexpr int kPfBlockRows = 128;                // query rows (token x GQA head) of a workgroup
struct PrefillParams {
  const uint8_t *pool[NFMT];
  int64_t pool_pages[NFMT];
  int64_t page_bytes[NFMT];
  int64_t head_bytes[NFMT];
  const uint32_t *signs;       // [Hkv][2][d/32]
  const uint16_t *tqk_perm;    // [Hkv][d] or null
  const uint16_t *q;           // bf16 [B][C][Hq][d]
  float *out;                  // [B][C][Hq][d]
  float *lse;                  // [B][C][Hq] or null
  const PlanHeader *plan_hdr;
  const int32_t *seq;          // plan: clamped N_b [B]
  const int32_t *counts;       // plan: [B][NFMT]
  const int2 *entries;         // plan: [B][max_pages] (logical page, pool id), per format in tag order
  kvq_counters *counters;
  int B, Hq, Hkv, G, P, max_pages, D, chunk;
  int row_blocks;              // ceil(chunk * G / kPfBlockRows)
  float scale_log2;            // sm_scale * log2(e)
  float *ws_o;                 // [B][C][Hq][d] the rows' running O between launches (workspace)
  float *ws_ml;                // [B][C][Hq][2] their (m, l)
  int first, last, unrot_out;  // set per launch by launch_prefill
};
// Workspace of a packed prefill that takes more than one launch.
inline int64_t prefill_ws_bytes(int B, int C, int Hq, int d) {
  const int64_t rows = (int64_t)B * C * Hq;
  return ((rows * d * 4 + 255) & ~255LL) + rows * 8;
}

// Launchers (return hipSuccess or the launch error).
hipError_t launch_plan(const PlanParams &p, hipStream_t s);
// Decode = scan kernel (partials) followed by the merge kernel (Eq. 11-13 and
// the inverse V rotation), both on stream s.
// scan_end: if not null, recorded on s between the two kernels (measurement).
hipError_t launch_decode(const DecodeParams &p, int d, hipStream_t s, hipEvent_t scan_end = nullptr);
// Packed chunked prefill (chunk * G query rows per request and KV head).
hipError_t launch_prefill(const PrefillParams &p, hipStream_t s);
// Page mass and running score from a scored decode (one workgroup per request).
hipError_t launch_collect(const CollectParams &c, hipStream_t s);
hipError_t launch_encode_fp8(const EncodeFp8Params &p, int d, int src_is_bf16, hipStream_t s);
// fmt: FMT_TQ3, FMT_TQ2 or FMT_TQK.
hipError_t launch_encode_tq(const EncodeTqParams &p, int d, int fmt, hipStream_t s);
// fmt: FMT_TQ3, FMT_TQ2 or FMT_TQK (the source pool's format).
hipError_t launch_promote_fp8(const PromoteParams &p, int d, int fmt, hipStream_t s);

}  // namespace kvq
