// Mixed-format paged decode attention for gfx950 (MI355X).
//
// Minima-KV (arxiv 2608.23834) section 3.3: pages are partitioned by format,
// each format-specific pass yields (m_j, l_j, O_bar_j), and Eq. 11-13 merge
// them; section 4.1: compact per-request page-index arrays partition the
// block table by format, the scans reuse each unpacked tile across the GQA
// group, write a normalized partial plus its statistics, and a separate stage
// merges all splits. Block-GTQ (paperpeel 2606.24033) appendix H.2-H.4: the
// query is rotated into codec coordinates in the prologue, values are
// accumulated in rotated space and rotated back once after the merge, and
// the launch grid is fixed with sequence lengths read on the device.
//
// gfx950 design:
//  * one workgroup (8 waves, two per SIMD) = one work item (request, format,
//    run of S_f pages of that format) for one KV head; the waves take the
//    item's pages round-robin; items of all formats carry about the same
//    number of KV bytes (byte-balanced split-K);
//  * a wave consumes 16-token tiles with fully coalesced global loads (the
//    page layout deals a tile to lanes in MFMA operand order, so K/V never
//    pass through LDS); the loads of the next DEPTH tiles are in flight while
//    a tile is computed (register ring, one slot per tile);
//  * the wave's page ids sit one per lane and are read with v_readlane, so
//    every tile address is scalar;
//  * QK^T: tokens x GQA heads (padded to 16) x d as 16x16x32 MFMAs (bf16 for
//    FP8 pages, f16 for TQ pages against the rotated query);
//  * PV: dims x heads x 16 tokens as 16x16x16 f16 MFMAs; the QK accumulator
//    layout is the PV B-operand layout, so P never leaves registers;
//  * TQ codes turn into fp16 centroids with byte-permute lookups (v_perm_b32
//    on 8-byte tables), FP8 codes with the gfx950 scaled converts (exact);
//  * online softmax in fp32 / log2 units; the accumulator is rescaled only
//    when a head's running maximum grows by more than kRescaleSlack (the
//    deferred maximum keeps every exponent <= 2^kRescaleSlack);
//  * the 8 waves merge by a tree in LDS; one release fence per workgroup
//    publishes its partial; the last workgroup of a (request, KV head)
//    acquires, merges every partial (Eq. 11-13) with all loads in flight,
//    applies the single inverse V rotation to the TQ part and writes O, lse.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int kW = kDecodeWaves;
constexpr float kRescaleSlack = 8.0f;   // log2 units

// fp16 bit patterns of the Gaussian Lloyd-Max centroids (rounded to fp16),
// ascending code order.
constexpr uint16_t kC3[8] = {0xC04E, 0xBD60, 0xBA0C, 0xB3D8, 0x33D8, 0x3A0C, 0x3D60, 0x404E};
constexpr uint16_t kC2[4] = {0xBE0B, 0xB73F, 0x373F, 0x3E0B};

constexpr uint32_t pack_bytes(uint32_t b0, uint32_t b1, uint32_t b2, uint32_t b3) {
  return b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
}
// v_perm tables: low / high bytes of the centroids, entries 0-3 and 4-7.
constexpr uint32_t kT3LoA = pack_bytes(kC3[0] & 255, kC3[1] & 255, kC3[2] & 255, kC3[3] & 255);
constexpr uint32_t kT3LoB = pack_bytes(kC3[4] & 255, kC3[5] & 255, kC3[6] & 255, kC3[7] & 255);
constexpr uint32_t kT3HiA = pack_bytes(kC3[0] >> 8, kC3[1] >> 8, kC3[2] >> 8, kC3[3] >> 8);
constexpr uint32_t kT3HiB = pack_bytes(kC3[4] >> 8, kC3[5] >> 8, kC3[6] >> 8, kC3[7] >> 8);
constexpr uint32_t kT2Lo = pack_bytes(kC2[0] & 255, kC2[1] & 255, kC2[2] & 255, kC2[3] & 255);
constexpr uint32_t kT2Hi = pack_bytes(kC2[0] >> 8, kC2[1] >> 8, kC2[2] >> 8, kC2[3] >> 8);

// Byte-spread selector of group g (four codes, one per byte) from a lane's
// code words, following the page layout rule.
template <int BITS>
__device__ __forceinline__ uint32_t group_sel(const uint32_t *w, int g) {
  if constexpr (BITS == 3) {
    const uint32_t a = w[3 * (g >> 3)], b = w[3 * (g >> 3) + 1], c = w[3 * (g >> 3) + 2];
    switch (g & 7) {
      case 0: return a & 0x07070707u;
      case 1: return (a >> 3) & 0x07070707u;
      case 2: return b & 0x07070707u;
      case 3: return (b >> 3) & 0x07070707u;
      case 4: return c & 0x07070707u;
      case 5: return (c >> 3) & 0x07070707u;
      case 6: return ((a >> 6) & 0x03030303u) | ((c >> 4) & 0x04040404u);
      default: return ((b >> 6) & 0x03030303u) | ((c >> 5) & 0x04040404u);
    }
  } else {
    return (w[g >> 2] >> (2 * (g & 3))) & 0x03030303u;
  }
}

// Four codes -> four fp16 centroids as two dwords (codes 0,1 | codes 2,3).
template <int BITS>
__device__ __forceinline__ uint2 decode_group(uint32_t sel) {
  uint32_t lo, hi;
  if constexpr (BITS == 3) {
    lo = __builtin_amdgcn_perm(kT3LoB, kT3LoA, sel);
    hi = __builtin_amdgcn_perm(kT3HiB, kT3HiA, sel);
  } else {
    lo = __builtin_amdgcn_perm(0u, kT2Lo, sel);
    hi = __builtin_amdgcn_perm(0u, kT2Hi, sel);
  }
  uint2 r;
  r.x = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
  r.y = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
  return r;
}

__device__ __forceinline__ half8_t as_half8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  uint4 v = make_uint4(a, b, c, d);
  return __builtin_bit_cast(half8_t, v);
}
__device__ __forceinline__ half4_t as_half4(uint2 v) { return __builtin_bit_cast(half4_t, v); }

__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w, bool hi_word) {
  bf16x2_t r = hi_word ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)
                       : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ uint32_t fp8x2_to_f16x2(uint32_t w, bool hi_word) {
  half2_t r = hi_word ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true)
                      : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float kNegInf = -__builtin_inff();

// ------------------------------------------------------------------------
// plan: per-request compact lists by format (order kept), counts, lengths
// ------------------------------------------------------------------------
constexpr int kPlanThreads = 1024;

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanParams p) {
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int NWAVE = kPlanThreads / 64;
  __shared__ int s_wsum[NWAVE][NFMT + 1];
  __shared__ int s_base[NWAVE][NFMT + 1];
  int N = p.seq_lens[b];
  if (N < 0) N = 0;
  int n_pages = (N + p.P - 1) / p.P;
  int clamp_invalid = 0;
  if (n_pages > p.max_pages) {
    n_pages = p.max_pages;
    N = p.max_pages * p.P;
    clamp_invalid = 1;
  }
  if (tid == 0) p.seq[b] = N;
  for (int h = tid; h < p.Hkv; h += kPlanThreads) p.merge_ctr[(int64_t)b * p.Hkv + h] = 0u;
  const int32_t *bt = p.block_table + (int64_t)b * p.max_pages;
  const uint8_t *pf = p.page_format + (int64_t)b * p.max_pages;
  // each thread owns a contiguous run of pages
  const int chunk = (n_pages + kPlanThreads - 1) / kPlanThreads;
  const int k0 = min(n_pages, tid * chunk), k1 = min(n_pages, k0 + chunk);
  int cnt[NFMT + 1] = {0, 0, 0, 0};   // [NFMT] = invalid entries
  for (int k = k0; k < k1; ++k) {
    const int f = pf[k];
    const int pid = bt[k];
    const bool ok = f < NFMT && pid >= 0 && pid < p.pool_pages[f < NFMT ? f : 0];
    cnt[ok ? f : NFMT]++;
  }
  // block-wide exclusive scan of the four counters
  int incl[NFMT + 1];
#pragma unroll
  for (int f = 0; f <= NFMT; ++f) {
    int v = cnt[f];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(v, off);
      if (lane >= off) v += t;
    }
    incl[f] = v;
    if (lane == 63) s_wsum[wave][f] = v;
  }
  __syncthreads();
  if (tid <= NFMT) {
    int run = 0;
    for (int w = 0; w < NWAVE; ++w) {
      s_base[w][tid] = run;
      run += s_wsum[w][tid];
    }
    s_wsum[0][tid] = run;   // totals (s_wsum row 0 is no longer needed as a wave sum)
  }
  __syncthreads();
  int tot[NFMT + 1];
#pragma unroll
  for (int f = 0; f <= NFMT; ++f) tot[f] = s_wsum[0][f];
  if (tid == 0) {
    for (int f = 0; f < NFMT; ++f) p.counts[b * 4 + f] = tot[f];
    p.counts[b * 4 + 3] = 0;
    const int bad = tot[NFMT] + clamp_invalid;
    if (p.counters && bad) atomicAdd(&p.counters->invalid_entries, (unsigned long long)bad);
  }
  int pos[NFMT];
  {
    int off = 0;
#pragma unroll
    for (int f = 0; f < NFMT; ++f) {
      pos[f] = off + s_base[wave][f] + incl[f] - cnt[f];
      off += tot[f];
    }
  }
  int2 *ent = p.entries + (int64_t)b * p.max_pages;
  for (int k = k0; k < k1; ++k) {
    const int f = pf[k];
    const int pid = bt[k];
    const bool ok = f < NFMT && pid >= 0 && pid < p.pool_pages[f < NFMT ? f : 0];
    if (ok) {
      const int at = f == 0 ? pos[0]++ : (f == 1 ? pos[1]++ : pos[2]++);
      ent[at] = make_int2(k, pid);
    }
  }
}

// ------------------------------------------------------------------------
// decode
// ------------------------------------------------------------------------
struct ItemInfo {
  int b, fmt, start, cnt, list_off, n_items, item_base;
};

__device__ __forceinline__ int items_of(const int32_t *cnt4, const int *S) {
  int n = 0;
  for (int f = 0; f < NFMT; ++f) n += (cnt4[f] + S[f] - 1) / S[f];
  return n > 0 ? n : 1;
}

// Locate work item `it`; run by one full wave, result broadcast to all lanes.
__device__ bool find_item(const DecodeParams &p, int it, ItemInfo &info) {
  const int lane = threadIdx.x & 63;
  int base = 0;
  for (int b0 = 0; b0 < p.B; b0 += 64) {
    const int b = b0 + lane;
    int n = 0;
    if (b < p.B) n = items_of(p.counts + 4 * b, p.S);
    int incl = n;
    for (int off = 1; off < 64; off <<= 1) {
      int t = __shfl_up(incl, off);
      if (lane >= off) incl += t;
    }
    const int excl = incl - n;
    const bool mine = b < p.B && it >= base + excl && it < base + incl;
    const uint64_t m = __ballot(mine);
    if (m) {
      const int src = __ffsll((unsigned long long)m) - 1;
      info.b = __shfl(b, src);
      info.n_items = __shfl(n, src);
      info.item_base = base + __shfl(excl, src);
      int local = it - info.item_base;
      const int32_t *c4 = p.counts + 4 * info.b;
      info.fmt = FMT_EMPTY;
      info.start = 0;
      info.cnt = 0;
      info.list_off = 0;
      int off = 0;
      for (int f = 0; f < NFMT; ++f) {
        const int nf = (c4[f] + p.S[f] - 1) / p.S[f];
        if (local < nf) {
          info.fmt = f;
          info.start = local * p.S[f];
          info.cnt = min(p.S[f], c4[f] - info.start);
          info.list_off = off;
          break;
        }
        local -= nf;
        off += c4[f];
      }
      return true;
    }
    base += __shfl(incl, 63);
  }
  return false;
}

// ---- tiles held in registers: one 16-token K tile and V tile of a page ----
template <int FMT, int D>
struct Tile;

template <int D>
struct Tile<FMT_FP8, D> {
  uint4 k[D / 64], v[D / 64];
  float4 ks, vs;
};
template <int D>
struct Tile<FMT_TQ3, D> {
  uint32_t k[D * 3 / 128], v[D * 3 / 128];
  uint2 ks, vs;
};
template <int D>
struct Tile<FMT_TQ2, D> {
  uint32_t k[D / 64], v[D / 64];
  uint2 ks, vs;
};

// Words of one role of a TQ tile for lane `lane`, following the region rule
// of the page layout (regions of 4, then 2, then 1 words per lane).
template <int WN>
__device__ __forceinline__ void load_tq_words(uint32_t (&w)[WN], const uint8_t *t, int lane) {
  if constexpr (WN == 6) {
    const uint4 a = *(const uint4 *)(t + lane * 16);
    const uint2 b = *(const uint2 *)(t + 1024 + lane * 8);
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w; w[4] = b.x; w[5] = b.y;
  } else if constexpr (WN == 3) {
    const uint2 a = *(const uint2 *)(t + lane * 8);
    w[0] = a.x; w[1] = a.y; w[2] = *(const uint32_t *)(t + 512 + lane * 4);
  } else if constexpr (WN == 4) {
    const uint4 a = *(const uint4 *)(t + lane * 16);
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
  } else {
    static_assert(WN == 2, "unsupported TQ word count");
    const uint2 a = *(const uint2 *)(t + lane * 8);
    w[0] = a.x; w[1] = a.y;
  }
}

// head: this (page, KV head) block; tau: tile index inside the page.
template <int FMT, int D>
__device__ __forceinline__ void load_tile(Tile<FMT, D> &t, const uint8_t *head, int tau, int T, int P, int lane) {
  const int grp = lane >> 4;
  if constexpr (FMT == FMT_FP8) {
    const uint8_t *kt = head + (int64_t)tau * 16 * D;
    const uint8_t *vt = head + (int64_t)(T + tau) * 16 * D;
#pragma unroll
    for (int r = 0; r < D / 64; ++r) {
      t.k[r] = *(const uint4 *)(kt + (r * 64 + lane) * 16);
      t.v[r] = *(const uint4 *)(vt + (r * 64 + lane) * 16);
    }
    t.ks = *(const float4 *)(head + 2LL * P * D + 4 * (tau * 16 + 4 * grp));
    t.vs = *(const float4 *)(head + 2LL * P * D + 4LL * P + 4 * (tau * 16 + 4 * grp));
  } else {
    constexpr int BITS = FMT == FMT_TQ3 ? 3 : 2;
    constexpr int64_t tile_bytes = 16LL * D * BITS / 8;
    load_tq_words(t.k, head + tau * tile_bytes, lane);
    load_tq_words(t.v, head + (T + tau) * tile_bytes, lane);
    const uint8_t *sig = head + 2LL * T * tile_bytes;
    t.ks = *(const uint2 *)(sig + 2 * (tau * 16 + 4 * grp));
    t.vs = *(const uint2 *)(sig + 2LL * P + 2 * (tau * 16 + 4 * grp));
  }
}

// One tile: scores, online softmax (deferred rescale), P V.
template <int FMT, int D>
__device__ __forceinline__ void process_tile(const Tile<FMT, D> &t, int nvalid, const uint32_t *qb, float scale_log2,
                                             float4_t (&acc)[D / 16], float &m_run, float &l_run) {
  constexpr int NKK = D / 32;
  constexpr int NGV = D / 16;
  const int lane = threadIdx.x & 63;
  const int grp = lane >> 4;
  float4_t s = {0.f, 0.f, 0.f, 0.f};
  float ks[4], vs[4];
  if constexpr (FMT == FMT_FP8) {
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const uint4 v = t.k[kk >> 1];
      const uint32_t w0 = (kk & 1) ? v.z : v.x;
      const uint32_t w1 = (kk & 1) ? v.w : v.y;
      uint4 a;
      a.x = fp8x2_to_bf16x2(w0, false);
      a.y = fp8x2_to_bf16x2(w0, true);
      a.z = fp8x2_to_bf16x2(w1, false);
      a.w = fp8x2_to_bf16x2(w1, true);
      const uint4 bq = make_uint4(qb[4 * kk], qb[4 * kk + 1], qb[4 * kk + 2], qb[4 * kk + 3]);
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, bq),
                                                  s, 0, 0, 0);
    }
    ks[0] = t.ks.x; ks[1] = t.ks.y; ks[2] = t.ks.z; ks[3] = t.ks.w;
    vs[0] = t.vs.x; vs[1] = t.vs.y; vs[2] = t.vs.z; vs[3] = t.vs.w;
  } else {
    constexpr int BITS = FMT == FMT_TQ3 ? 3 : 2;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const uint2 lo = decode_group<BITS>(group_sel<BITS>(t.k, 2 * kk));
      const uint2 hi = decode_group<BITS>(group_sel<BITS>(t.k, 2 * kk + 1));
      const half8_t a = as_half8(lo.x, lo.y, hi.x, hi.y);
      const half8_t bq = as_half8(qb[4 * kk], qb[4 * kk + 1], qb[4 * kk + 2], qb[4 * kk + 3]);
      s = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bq, s, 0, 0, 0);
    }
    ks[0] = half_bits_to_float(t.ks.x & 0xFFFF); ks[1] = half_bits_to_float(t.ks.x >> 16);
    ks[2] = half_bits_to_float(t.ks.y & 0xFFFF); ks[3] = half_bits_to_float(t.ks.y >> 16);
    vs[0] = half_bits_to_float(t.vs.x & 0xFFFF); vs[1] = half_bits_to_float(t.vs.x >> 16);
    vs[2] = half_bits_to_float(t.vs.y & 0xFFFF); vs[3] = half_bits_to_float(t.vs.y >> 16);
  }
  // scores in log2 units; tokens past the sequence end are masked
  float sc[4];
  float mx = kNegInf;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    sc[r] = (4 * grp + r < nvalid) ? s[r] * ks[r] * scale_log2 : kNegInf;
    mx = fmaxf(mx, sc[r]);
  }
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  // deferred rescale: only when some head's maximum grew by more than the slack
  if (__builtin_amdgcn_ballot_w64(mx > m_run + kRescaleSlack) != 0) {
    const float mnew = fmaxf(m_run, mx);
    const float alpha = mnew == kNegInf ? 1.f : fast_exp2(m_run - mnew);
    l_run *= alpha;
#pragma unroll
    for (int gv = 0; gv < NGV; ++gv) acc[gv] *= alpha;
    m_run = mnew;
  }
  float pr[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) pr[r] = m_run == kNegInf ? 0.f : fast_exp2(sc[r] - m_run);
  l_run += (pr[0] + pr[1]) + (pr[2] + pr[3]);
  half4_t pb;
#pragma unroll
  for (int r = 0; r < 4; ++r) pb[r] = (_Float16)(4 * grp + r < nvalid ? pr[r] * vs[r] : 0.f);
  if constexpr (FMT == FMT_FP8) {
#pragma unroll
    for (int gv = 0; gv < NGV; ++gv) {
      const uint4 v = t.v[gv >> 2];
      const uint32_t w = (gv & 3) == 0 ? v.x : (gv & 3) == 1 ? v.y : (gv & 3) == 2 ? v.z : v.w;
      uint2 a;
      a.x = fp8x2_to_f16x2(w, false);
      a.y = fp8x2_to_f16x2(w, true);
      acc[gv] = __builtin_amdgcn_mfma_f32_16x16x16f16(as_half4(a), pb, acc[gv], 0, 0, 0);
    }
  } else {
    constexpr int BITS = FMT == FMT_TQ3 ? 3 : 2;
#pragma unroll
    for (int gv = 0; gv < NGV; ++gv) {
      const uint2 a = decode_group<BITS>(group_sel<BITS>(t.v, gv));
      acc[gv] = __builtin_amdgcn_mfma_f32_16x16x16f16(as_half4(a), pb, acc[gv], 0, 0, 0);
    }
  }
}

// Per-wave scan over this wave's pages of the item (pages wave, wave + kW, ...)
// with DEPTH tiles of loads in flight.
template <int FMT, int D, int DEPTH>
__device__ __forceinline__ void wave_scan(const DecodeParams &p, int my_pages, int2 my_ent, int g, int N,
                                          const uint32_t *qb, float4_t (&acc)[D / 16], float &m_run, float &l_run) {
  const int lane = threadIdx.x & 63;
  const int P = p.P, T = P / 16;
  const int n_tiles = my_pages * T;
  const uint8_t *pool = p.pool[FMT] + (int64_t)g * p.head_bytes[FMT];
  const int64_t page_bytes = p.page_bytes[FMT];
  auto head_of = [&](int j) {
    const int pid = __builtin_amdgcn_readlane(my_ent.y, j);
    return pool + (int64_t)pid * page_bytes;
  };
  auto tok0_of = [&](int tt) {
    const int lp = __builtin_amdgcn_readlane(my_ent.x, tt / T);
    return lp * P + (tt % T) * 16;
  };
  Tile<FMT, D> buf[DEPTH];
#pragma unroll
  for (int j = 0; j < DEPTH; ++j)
    if (j < n_tiles) load_tile<FMT, D>(buf[j], head_of(j / T), j % T, T, P, lane);
  for (int t0 = 0; t0 < n_tiles; t0 += DEPTH) {
#pragma unroll
    for (int j = 0; j < DEPTH; ++j) {
      const int tt = t0 + j;
      if (tt < n_tiles) {
        const Tile<FMT, D> cur = buf[j];
        const int nx = tt + DEPTH;
        if (nx < n_tiles) load_tile<FMT, D>(buf[j], head_of(nx / T), nx % T, T, P, lane);
        const int nvalid = N - tok0_of(tt);
        if (nvalid > 0) process_tile<FMT, D>(cur, nvalid, qb, p.scale_log2, acc, m_run, l_run);
      }
    }
  }
}

// In-LDS unnormalized Walsh-Hadamard transform of `rows` vectors of length D
// (stride D floats), all threads of the block.
template <int D>
__device__ void lds_fwht(float *buf, int rows) {
  for (int h = 1; h < D; h <<= 1) {
    __syncthreads();
    for (int t = threadIdx.x; t < rows * (D / 2); t += blockDim.x) {
      const int r = t / (D / 2), k = t % (D / 2);
      const int i = (k / h) * (2 * h) + (k % h);
      float *v = buf + r * D;
      const float a = v[i], c = v[i + h];
      v[i] = a + c;
      v[i + h] = a - c;
    }
  }
  __syncthreads();
}

// LDS bytes of the tree merge of the waves' accumulators.
__host__ __device__ constexpr int merge_chunk_dims(int D, int G) {
  // 4 slots x G heads x Dc dims x 4 B <= 48 KB
  return (4 * G * D * 4 <= 48 * 1024) ? D : (4 * G * (D / 2) * 4 <= 48 * 1024 ? D / 2 : D / 4);
}

// Last-workgroup merge of every partial of request b, KV head g.
template <int D>
__device__ void merge_request_head(const DecodeParams &p, const ItemInfo &info, int g, float *smem) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = p.G;
  const int32_t *c4 = p.counts + 4 * info.b;
  const int n8 = (c4[FMT_FP8] + p.S[FMT_FP8] - 1) / p.S[FMT_FP8];
  const int n_real = n8 + (c4[FMT_TQ3] + p.S[FMT_TQ3] - 1) / p.S[FMT_TQ3] +
                     (c4[FMT_TQ2] + p.S[FMT_TQ2] - 1) / p.S[FMT_TQ2];
  const int64_t slot0 = (int64_t)info.item_base * p.Hkv + g;     // slot of item i: slot0 + i * Hkv
  const float *ml_g = p.part_ml + slot0 * G * 2;
  const float *o_g = p.part_o + slot0 * G * D;
  const int64_t ml_stride = (int64_t)p.Hkv * G * 2, o_stride = (int64_t)p.Hkv * G * D;

  float *stat = smem;                       // [16][4]: M_rot, L_rot, M_nat, L_nat
  float *orot = smem + 64;                  // [G][D] rotated-space TQ merge
  float *onat = orot + G * D;               // [G][D] natural-space FP8 merge
  float *wt = onat + G * D;                 // [kChunk][16] weights of the current item chunk
  constexpr int kChunk = 64;

  // statistics per head: wave w takes heads w, w + kW; lanes over items
  for (int n = wave; n < G; n += kW) {
    float Mr = kNegInf, Mn = kNegInf;
    for (int i = lane; i < n_real; i += 64) {
      const float2 ml = *(const float2 *)(ml_g + i * ml_stride + 2 * n);
      if (ml.y > 0.f) {
        if (i < n8) Mn = fmaxf(Mn, ml.x); else Mr = fmaxf(Mr, ml.x);
      }
    }
    for (int off = 32; off >= 1; off >>= 1) {
      Mr = fmaxf(Mr, __shfl_xor(Mr, off));
      Mn = fmaxf(Mn, __shfl_xor(Mn, off));
    }
    float Lr = 0.f, Ln = 0.f;
    for (int i = lane; i < n_real; i += 64) {
      const float2 ml = *(const float2 *)(ml_g + i * ml_stride + 2 * n);
      if (ml.y > 0.f) {
        if (i < n8) Ln += fast_exp2(ml.x - Mn) * ml.y; else Lr += fast_exp2(ml.x - Mr) * ml.y;
      }
    }
    for (int off = 32; off >= 1; off >>= 1) {
      Lr += __shfl_xor(Lr, off);
      Ln += __shfl_xor(Ln, off);
    }
    if (lane == 0) {
      stat[4 * n] = Mr; stat[4 * n + 1] = Lr; stat[4 * n + 2] = Mn; stat[4 * n + 3] = Ln;
    }
  }
  // weighted sums over items, in chunks of kChunk items; each thread owns
  // float4 slots (head n, dims 4c..4c+3). Items [0, n8) are FP8 partials
  // (natural space), [n8, n_real) TQ partials (rotated V space).
  constexpr int D4 = D / 4;
  const int n_slots = G * D4;
  float4 acc_s[2][2];   // [slot][0 = natural, 1 = rotated]
#pragma unroll
  for (int s = 0; s < 2; ++s) acc_s[s][0] = acc_s[s][1] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int i0 = 0; i0 < n_real; i0 += kChunk) {
    const int ni = min(kChunk, n_real - i0);
    __syncthreads();   // stat ready (first chunk) / previous weights consumed
    for (int t = tid; t < ni * G; t += kDecodeThreads) {
      const int i = i0 + t / G, n = t % G;
      const float2 ml = *(const float2 *)(ml_g + i * ml_stride + 2 * n);
      const bool nat = i < n8;
      const float M = stat[4 * n + (nat ? 2 : 0)], L = stat[4 * n + (nat ? 3 : 1)];
      wt[(t / G) * 16 + n] = (ml.y > 0.f && L > 0.f) ? fast_exp2(ml.x - M) * ml.y / L : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int slot = tid + s * kDecodeThreads;
      if (slot < n_slots) {
        const int n = slot / D4, c = slot % D4;
        const float *src = o_g + n * D + 4 * c;
        constexpr int U = 16;
        for (int j0 = 0; j0 < ni; j0 += U) {
          float4 v[U];
#pragma unroll
          for (int u = 0; u < U; ++u)
            if (j0 + u < ni) v[u] = *(const float4 *)(src + (int64_t)(i0 + j0 + u) * o_stride);
#pragma unroll
          for (int u = 0; u < U; ++u) {
            if (j0 + u < ni) {
              const float w = wt[(j0 + u) * 16 + n];
              const float wn = i0 + j0 + u < n8 ? w : 0.f;
              const float wr = w - wn;
              acc_s[s][0].x += wn * v[u].x; acc_s[s][0].y += wn * v[u].y;
              acc_s[s][0].z += wn * v[u].z; acc_s[s][0].w += wn * v[u].w;
              acc_s[s][1].x += wr * v[u].x; acc_s[s][1].y += wr * v[u].y;
              acc_s[s][1].z += wr * v[u].z; acc_s[s][1].w += wr * v[u].w;
            }
          }
        }
      }
    }
  }
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int slot = tid + s * kDecodeThreads;
    if (slot < n_slots) {
      const int n = slot / D4, c = slot % D4;
      *(float4 *)(orot + n * D + 4 * c) = acc_s[s][1];
      *(float4 *)(onat + n * D + 4 * c) = acc_s[s][0];
    }
  }
  // single inverse V rotation of the TQ part: R_V^T y = s_V * FWHT(y) / sqrt(D)
  lds_fwht<D>(orot, G);
  const uint32_t *sv = p.signs + ((int64_t)g * 2 + 1) * (D / 32);
  const float rs = 1.0f / sqrtf((float)D);
  for (int t = tid; t < G * D; t += kDecodeThreads) {
    const int n = t / D, j = t % D;
    const float Mr = stat[4 * n], Lr = stat[4 * n + 1], Mn = stat[4 * n + 2], Ln = stat[4 * n + 3];
    const float M = fmaxf(Mr, Mn);
    float num = 0.f, L = 0.f;
    if (M != kNegInf) {
      if (Lr > 0.f) {
        float vr = orot[t] * rs;
        if ((sv[j >> 5] >> (j & 31)) & 1u) vr = -vr;
        const float er = fast_exp2(Mr - M) * Lr;
        L += er;
        num += er * vr;
      }
      if (Ln > 0.f) {
        const float en = fast_exp2(Mn - M) * Ln;
        L += en;
        num += en * onat[t];
      }
    }
    const int64_t orow = ((int64_t)info.b * p.Hq + (int64_t)g * G + n);
    p.out[orow * D + j] = L > 0.f ? num / L : 0.f;
    if (j == 0 && p.lse) p.lse[orow] = L > 0.f ? (M + log2f(L)) * 0.69314718055994531f : kNegInf;
  }
  if (tid == 0) p.merge_ctr[(int64_t)info.b * p.Hkv + g] = 0u;
}

template <int D>
__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(DecodeParams p) {
  constexpr int DL = D / 4;
  constexpr int NKK = D / 32;
  constexpr int NGV = D / 16;
  extern __shared__ float smem[];
  __shared__ ItemInfo s_info;
  __shared__ int s_found, s_last;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int it = blockIdx.x / p.Hkv, g = blockIdx.x % p.Hkv;
  const int G = p.G;

  if (wave == 0) {
    ItemInfo info;
    const bool ok = find_item(p, it, info);
    if (lane == 0) {
      s_found = ok;
      if (ok) s_info = info;
    }
  }
  __syncthreads();
  if (!s_found) return;
  const ItemInfo info = s_info;

  // this wave's page entries, one per lane: pages wave, wave + kW, ...
  const int my_pages = info.cnt > wave ? (info.cnt - wave + kW - 1) / kW : 0;
  int2 my_ent = make_int2(0, 0);
  if (lane < my_pages)
    my_ent = p.entries[(int64_t)info.b * p.max_pages + info.list_off + info.start + wave + kW * lane];

  // ---- prologue: query operand in LDS (16 head rows x D), rows >= G zero ----
  uint16_t *qs = (uint16_t *)smem;                 // [16][D] f16 or bf16 bits
  float *qf = smem + 16 * D / 2;                   // [G][D] fp32 scratch (TQ rotation)
  const uint16_t *qsrc = p.q + ((int64_t)info.b * p.Hq + (int64_t)g * G) * D;
  const bool tq = info.fmt == FMT_TQ3 || info.fmt == FMT_TQ2;
  if (info.fmt != FMT_EMPTY) {
    if (!tq) {
      for (int t = tid; t < 16 * D; t += kDecodeThreads) {
        const int n = t / D;
        qs[t] = n < G ? qsrc[t] : (uint16_t)0;
      }
    } else {
      const uint32_t *sg = p.signs + (int64_t)g * 2 * (D / 32);   // K role signs
      for (int t = tid; t < G * D; t += kDecodeThreads) {
        const int j = t % D;
        float v = __builtin_bit_cast(float, (uint32_t)qsrc[t] << 16);
        if ((sg[j >> 5] >> (j & 31)) & 1u) v = -v;
        qf[t] = v;
      }
      lds_fwht<D>(qf, G);
      const float rs = 1.0f / sqrtf((float)D);
      for (int t = tid; t < 16 * D; t += kDecodeThreads) {
        const int n = t / D;
        const _Float16 h = n < G ? (_Float16)(qf[t] * rs) : (_Float16)0.f;
        qs[t] = __builtin_bit_cast(uint16_t, h);
      }
    }
  }
  __syncthreads();
  // B operand: lane (head n = lane%16, k-block lane/16): dims (lane/16)*DL + 8kk + e
  uint32_t qb[NKK * 4];
  {
    const uint4 *src = (const uint4 *)(qs + (lane & 15) * D + (lane >> 4) * DL);
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const uint4 v = src[kk];
      qb[4 * kk] = v.x; qb[4 * kk + 1] = v.y; qb[4 * kk + 2] = v.z; qb[4 * kk + 3] = v.w;
    }
  }
  __syncthreads();   // qs / qf are reused below

  float4_t acc[NGV];
#pragma unroll
  for (int gv = 0; gv < NGV; ++gv) acc[gv] = (float4_t){0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf, l_run = 0.f;
  const int N = p.seq[info.b];
  switch (info.fmt) {
    case FMT_FP8: wave_scan<FMT_FP8, D, 2>(p, my_pages, my_ent, g, N, qb, acc, m_run, l_run); break;
    case FMT_TQ3: wave_scan<FMT_TQ3, D, 4>(p, my_pages, my_ent, g, N, qb, acc, m_run, l_run); break;
    case FMT_TQ2: wave_scan<FMT_TQ2, D, 4>(p, my_pages, my_ent, g, N, qb, acc, m_run, l_run); break;
    default: break;
  }
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);

  // ---- tree merge of the 8 waves in LDS (dims in chunks of DC) ----
  // A lane holds head n = lane % 16 and dims 16 gv + 4 (lane / 16) + r.
  const int DC = merge_chunk_dims(D, G);
  float *mo = smem;                                   // [4][G][DC]
  float *mml = smem + 4 * G * DC;                     // [4][16][2]
  const int n = lane & 15;
  for (int half = kW / 2; half >= 1; half >>= 1) {
    // waves [half, 2 half) hand their state to waves [0, half)
    const bool writer = wave >= half && wave < 2 * half;
    const bool reader = wave < half;
    float alpha_self = 1.f, alpha_other = 1.f;
    if (writer && lane < 16) {
      mml[((wave - half) * 16 + n) * 2] = m_run;
      mml[((wave - half) * 16 + n) * 2 + 1] = l_run;
    }
    __syncthreads();
    if (reader) {
      const float mo_ = mml[(wave * 16 + n) * 2], lo_ = mml[(wave * 16 + n) * 2 + 1];
      const float M = fmaxf(m_run, mo_);
      if (M != kNegInf) {
        alpha_self = fast_exp2(m_run - M);
        alpha_other = fast_exp2(mo_ - M);
      }
      l_run = l_run * alpha_self + lo_ * alpha_other;
      m_run = M;
#pragma unroll
      for (int gv = 0; gv < NGV; ++gv) acc[gv] *= alpha_self;
    }
    for (int c0 = 0; c0 < D; c0 += DC) {
      if (writer && n < G) {
#pragma unroll
        for (int gv = 0; gv < NGV; ++gv)
          if (16 * gv >= c0 && 16 * gv < c0 + DC)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              mo[((wave - half) * G + n) * DC + 16 * gv - c0 + 4 * (lane >> 4) + r] = acc[gv][r];
      }
      __syncthreads();
      if (reader && n < G) {
#pragma unroll
        for (int gv = 0; gv < NGV; ++gv)
          if (16 * gv >= c0 && 16 * gv < c0 + DC)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              acc[gv][r] += alpha_other * mo[(wave * G + n) * DC + 16 * gv - c0 + 4 * (lane >> 4) + r];
      }
      __syncthreads();
    }
  }
  // ---- wave 0 writes the normalized partial ----
  const int64_t slot = (int64_t)it * p.Hkv + g;
  if (wave == 0 && n < G) {
    float *po = p.part_o + (slot * G + n) * D;
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
#pragma unroll
    for (int gv = 0; gv < NGV; ++gv) {
      float4 v;
      v.x = acc[gv][0] * inv; v.y = acc[gv][1] * inv; v.z = acc[gv][2] * inv; v.w = acc[gv][3] * inv;
      *(float4 *)(po + 16 * gv + 4 * (lane >> 4)) = v;
    }
    if (lane < 16) {
      float2 ml;
      ml.x = l_run > 0.f ? m_run : kNegInf;
      ml.y = l_run;
      *(float2 *)(p.part_ml + (slot * G + n) * 2) = ml;
    }
  }
  if (tid == 0 && p.counters && info.cnt > 0) {
    unsigned long long *c = info.fmt == FMT_FP8 ? &p.counters->pages_fp8
                          : info.fmt == FMT_TQ3 ? &p.counters->pages_tq3 : &p.counters->pages_tq2;
    atomicAdd(c, (unsigned long long)info.cnt);
  }

  // ---- publish (release); the last workgroup of (request, KV head) merges ----
  __syncthreads();
  if (tid == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const uint32_t old = __hip_atomic_fetch_add(&p.merge_ctr[(int64_t)info.b * p.Hkv + g], 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
    const bool last = old == (uint32_t)(info.n_items - 1);
    if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    s_last = last;
  }
  __syncthreads();
  if (!s_last) return;
  merge_request_head<D>(p, info, g, smem);
}

}  // namespace

hipError_t launch_plan(const PlanParams &p, hipStream_t s) {
  if (p.B <= 0) return hipSuccess;
  hipLaunchKernelGGL(plan_kernel, dim3(p.B), dim3(kPlanThreads), 0, s, p);
  return hipGetLastError();
}

size_t decode_lds_bytes(int d, int G) {
  const size_t q = 16 * (size_t)d * 2 + (size_t)G * d * 4;
  const int dc = merge_chunk_dims(d, G);
  const size_t tree = 4 * (size_t)G * dc * 4 + 4 * 16 * 2 * 4;
  const size_t fin = 64 * 4 + 2 * (size_t)G * d * 4 + 64 * 16 * 4;
  size_t m = q > tree ? q : tree;
  return m > fin ? m : fin;
}

hipError_t launch_decode(const DecodeParams &p, int d, int64_t n_items, hipStream_t s) {
  const int64_t blocks = n_items * p.Hkv;
  if (blocks <= 0) return hipSuccess;
  const size_t lds = decode_lds_bytes(d, p.G);
  if (d == 256) {
    hipLaunchKernelGGL(decode_kernel<256>, dim3((unsigned)blocks), dim3(kDecodeThreads), lds, s, p);
  } else {
    hipLaunchKernelGGL(decode_kernel<128>, dim3((unsigned)blocks), dim3(kDecodeThreads), lds, s, p);
  }
  return hipGetLastError();
}

}  // namespace kvq
