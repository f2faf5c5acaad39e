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
//  * one workgroup = one work item (request, format, run of that format's
//    pages) for one KV head; 4 waves split the item's pages round-robin;
//  * a wave consumes a 16-token tile with page-granular, fully coalesced
//    global loads (the page layout deals the tile to lanes in the MFMA
//    operand order, so no LDS staging of K/V is needed);
//  * QK^T: tokens x GQA heads (padded to 16) x d as 16x16x32 MFMAs (bf16 for
//    FP8 pages, f16 for TQ pages against the rotated query);
//  * PV: dims x heads x 16 tokens as 16x16x16 f16 MFMAs; the QK accumulator
//    layout is exactly the PV B-operand layout, so P never leaves registers;
//  * TQ codes turn into fp16 centroids with two byte-permute lookups per four
//    codes (v_perm_b32 on an 8-byte table), FP8 codes with the gfx950
//    scaled-convert instructions (exact, scale 1);
//  * online softmax in fp32 / log2 units per lane, 4-lane-group max by
//    cross-lane shuffles; per-workgroup merge in LDS; the last workgroup of
//    a (request, KV head) merges all partials (Eq. 11-13), applies the single
//    inverse V rotation to the TQ part and writes O and lse.
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

template <int BITS>
struct TqWords {
  static constexpr int kW(int D) { return D / 4 * BITS / 32; }
};

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
__global__ __launch_bounds__(256) void plan_kernel(PlanParams p) {
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ int s_cnt[4][4];     // [wave][format]
  __shared__ int s_run[4];        // running offset per format
  __shared__ int s_tot[4];
  __shared__ int s_invalid;
  int N = p.seq_lens[b];
  if (N < 0) N = 0;
  int n_pages = (N + p.P - 1) / p.P;
  int clamp_invalid = 0;
  if (n_pages > p.max_pages) {
    n_pages = p.max_pages;
    N = p.max_pages * p.P;
    clamp_invalid = 1;
  }
  if (tid == 0) {
    p.seq[b] = N;
    s_invalid = clamp_invalid;
  }
  for (int h = tid; h < p.Hkv; h += blockDim.x) p.merge_ctr[(int64_t)b * p.Hkv + h] = 0u;
  if (tid < 4) s_tot[tid] = 0;
  __syncthreads();
  const int32_t *bt = p.block_table + (int64_t)b * p.max_pages;
  const uint8_t *pf = p.page_format + (int64_t)b * p.max_pages;
  // pass 1: counts per format
  int my[NFMT] = {0, 0, 0};
  int my_invalid = 0;
  for (int k = tid; k < n_pages; k += blockDim.x) {
    int f = pf[k];
    int pid = bt[k];
    bool ok = f < NFMT && pid >= 0 && pid < p.pool_pages[f < NFMT ? f : 0];
    if (ok) my[f]++; else my_invalid++;
  }
  for (int f = 0; f < NFMT; ++f) {
    int v = my[f];
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    if (lane == 0) atomicAdd(&s_tot[f], v);
  }
  {
    int v = my_invalid;
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    if (lane == 0 && v) atomicAdd(&s_invalid, v);
  }
  __syncthreads();
  if (tid == 0) {
    int off = 0;
    for (int f = 0; f < NFMT; ++f) {
      p.counts[b * 4 + f] = s_tot[f];
      s_run[f] = off;
      off += s_tot[f];
    }
    p.counts[b * 4 + 3] = 0;
    if (p.counters && s_invalid) atomicAdd(&p.counters->invalid_entries, (unsigned long long)s_invalid);
  }
  __syncthreads();
  // pass 2: ordered compaction, 256 pages per round
  int2 *ent = p.entries + (int64_t)b * p.max_pages;
  for (int k0 = 0; k0 < n_pages; k0 += blockDim.x) {
    const int k = k0 + tid;
    int f = -1, pid = 0;
    if (k < n_pages) {
      f = pf[k];
      pid = bt[k];
      if (!(f < NFMT && pid >= 0 && pid < p.pool_pages[f < NFMT ? f : 0])) f = -1;
    }
    int rank[NFMT];
    for (int ff = 0; ff < NFMT; ++ff) {
      uint64_t m = __ballot(f == ff);
      rank[ff] = __popcll(m & ((1ull << lane) - 1ull));
      if (lane == 0) s_cnt[wave][ff] = __popcll(m);
    }
    __syncthreads();
    if (f >= 0) {
      int pos = s_run[f] + rank[f];
      for (int w = 0; w < wave; ++w) pos += s_cnt[w][f];
      ent[pos] = make_int2(k, pid);
    }
    __syncthreads();
    if (tid < NFMT) {
      int add = 0;
      for (int w = 0; w < kDecodeWaves; ++w) add += s_cnt[w][tid];
      s_run[tid] += add;
    }
    __syncthreads();
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

// Per-wave scan over the item's pages of one format.
// FMT: FMT_FP8 or a TQ format; D: head dim.
template <int FMT, int D>
__device__ __forceinline__ void wave_scan(const DecodeParams &p, const ItemInfo &it, int g, const uint32_t *qb,
                                          float4_t (&acc)[D / 16], float &m_run, float &l_run) {
  constexpr int DL = D / 4;
  constexpr int NKK = D / 32;
  constexpr int NGV = D / 16;
  constexpr int BITS = FMT == FMT_TQ3 ? 3 : 2;
  constexpr int W = (FMT == FMT_FP8) ? 0 : DL * BITS / 32;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = lane >> 4;                          // 4-token group of the QK output rows
  const int P = p.P, T = P / 16;
  const int64_t tile_bytes = (FMT == FMT_FP8) ? 16LL * D : 16LL * D * BITS / 8;
  const int N = p.seq[it.b];
  const uint8_t *pool = p.pool[FMT];
  const int2 *ent = p.entries + (int64_t)it.b * p.max_pages + it.list_off + it.start;

  for (int k = wave; k < it.cnt; k += kDecodeWaves) {
    const int2 e = ent[k];
    const int lp = e.x;
    const uint8_t *head = pool + (int64_t)e.y * p.page_bytes[FMT] + (int64_t)g * p.head_bytes[FMT];
    for (int tau = 0; tau < T; ++tau) {
      const int tok0 = lp * P + tau * 16;
      const int nvalid = N - tok0;
      if (nvalid <= 0) break;
      const uint8_t *kt = head + tau * tile_bytes;
      const uint8_t *vt = head + (T + tau) * tile_bytes;
      float4_t s = {0.f, 0.f, 0.f, 0.f};
      float ks[4], vs[4];
      if constexpr (FMT == FMT_FP8) {
        uint4 kw[DL / 16], vw[DL / 16];
#pragma unroll
        for (int r = 0; r < DL / 16; ++r) {
          kw[r] = *(const uint4 *)(kt + (r * 64 + lane) * 16);
          vw[r] = *(const uint4 *)(vt + (r * 64 + lane) * 16);
        }
        const float4 kf = *(const float4 *)(head + 2LL * P * D + 4 * (tau * 16 + 4 * grp));
        const float4 vf = *(const float4 *)(head + 2LL * P * D + 4LL * P + 4 * (tau * 16 + 4 * grp));
        ks[0] = kf.x; ks[1] = kf.y; ks[2] = kf.z; ks[3] = kf.w;
        vs[0] = vf.x; vs[1] = vf.y; vs[2] = vf.z; vs[3] = vf.w;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          const uint4 v = kw[kk >> 1];
          const uint32_t w0 = (kk & 1) ? v.z : v.x;
          const uint32_t w1 = (kk & 1) ? v.w : v.y;
          uint4 a;
          a.x = fp8x2_to_bf16x2(w0, false);
          a.y = fp8x2_to_bf16x2(w0, true);
          a.z = fp8x2_to_bf16x2(w1, false);
          a.w = fp8x2_to_bf16x2(w1, true);
          const uint4 bq = make_uint4(qb[4 * kk], qb[4 * kk + 1], qb[4 * kk + 2], qb[4 * kk + 3]);
          s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                      __builtin_bit_cast(bf16x8_t, bq), s, 0, 0, 0);
        }
        // softmax + PV below uses vw
        float mx = kNegInf;
        float sc[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          sc[r] = (4 * grp + r < nvalid) ? s[r] * ks[r] * p.scale_log2 : kNegInf;
          mx = fmaxf(mx, sc[r]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mnew = fmaxf(m_run, mx);
        float alpha = 1.f, pr[4] = {0.f, 0.f, 0.f, 0.f};
        if (mnew != kNegInf) {
          alpha = fast_exp2(m_run - mnew);
#pragma unroll
          for (int r = 0; r < 4; ++r) pr[r] = fast_exp2(sc[r] - mnew);
        }
        l_run = l_run * alpha + (pr[0] + pr[1]) + (pr[2] + pr[3]);
        m_run = mnew;
#pragma unroll
        for (int gv = 0; gv < NGV; ++gv) acc[gv] *= alpha;
        half4_t pb;
#pragma unroll
        for (int r = 0; r < 4; ++r) pb[r] = (_Float16)(pr[r] * vs[r]);
#pragma unroll
        for (int gv = 0; gv < NGV; ++gv) {
          const uint4 v = vw[gv >> 2];
          const uint32_t w = (gv & 3) == 0 ? v.x : (gv & 3) == 1 ? v.y : (gv & 3) == 2 ? v.z : v.w;
          uint2 a;
          a.x = fp8x2_to_f16x2(w, false);
          a.y = fp8x2_to_f16x2(w, true);
          acc[gv] = __builtin_amdgcn_mfma_f32_16x16x16f16(as_half4(a), pb, acc[gv], 0, 0, 0);
        }
      } else {
        uint32_t kw[W], vw[W];
        if constexpr (W == 6) {
          const uint4 a = *(const uint4 *)(kt + lane * 16);
          const uint2 b = *(const uint2 *)(kt + 1024 + lane * 8);
          kw[0] = a.x; kw[1] = a.y; kw[2] = a.z; kw[3] = a.w; kw[4] = b.x; kw[5] = b.y;
          const uint4 c = *(const uint4 *)(vt + lane * 16);
          const uint2 d = *(const uint2 *)(vt + 1024 + lane * 8);
          vw[0] = c.x; vw[1] = c.y; vw[2] = c.z; vw[3] = c.w; vw[4] = d.x; vw[5] = d.y;
        } else if constexpr (W == 3) {
          const uint2 a = *(const uint2 *)(kt + lane * 8);
          kw[0] = a.x; kw[1] = a.y; kw[2] = *(const uint32_t *)(kt + 512 + lane * 4);
          const uint2 c = *(const uint2 *)(vt + lane * 8);
          vw[0] = c.x; vw[1] = c.y; vw[2] = *(const uint32_t *)(vt + 512 + lane * 4);
        } else if constexpr (W == 4) {
          const uint4 a = *(const uint4 *)(kt + lane * 16);
          kw[0] = a.x; kw[1] = a.y; kw[2] = a.z; kw[3] = a.w;
          const uint4 c = *(const uint4 *)(vt + lane * 16);
          vw[0] = c.x; vw[1] = c.y; vw[2] = c.z; vw[3] = c.w;
        } else {
          static_assert(W == 2, "unsupported TQ word count");
          const uint2 a = *(const uint2 *)(kt + lane * 8);
          kw[0] = a.x; kw[1] = a.y;
          const uint2 c = *(const uint2 *)(vt + lane * 8);
          vw[0] = c.x; vw[1] = c.y;
        }
        const uint8_t *sig = head + 2LL * T * tile_bytes;
        const uint2 kh = *(const uint2 *)(sig + 2 * (tau * 16 + 4 * grp));
        const uint2 vh = *(const uint2 *)(sig + 2LL * P + 2 * (tau * 16 + 4 * grp));
        ks[0] = half_bits_to_float(kh.x & 0xFFFF); ks[1] = half_bits_to_float(kh.x >> 16);
        ks[2] = half_bits_to_float(kh.y & 0xFFFF); ks[3] = half_bits_to_float(kh.y >> 16);
        vs[0] = half_bits_to_float(vh.x & 0xFFFF); vs[1] = half_bits_to_float(vh.x >> 16);
        vs[2] = half_bits_to_float(vh.y & 0xFFFF); vs[3] = half_bits_to_float(vh.y >> 16);
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          const uint2 lo = decode_group<BITS>(group_sel<BITS>(kw, 2 * kk));
          const uint2 hi = decode_group<BITS>(group_sel<BITS>(kw, 2 * kk + 1));
          const half8_t a = as_half8(lo.x, lo.y, hi.x, hi.y);
          const half8_t bq = as_half8(qb[4 * kk], qb[4 * kk + 1], qb[4 * kk + 2], qb[4 * kk + 3]);
          s = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bq, s, 0, 0, 0);
        }
        float mx = kNegInf;
        float sc[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          sc[r] = (4 * grp + r < nvalid) ? s[r] * ks[r] * p.scale_log2 : kNegInf;
          mx = fmaxf(mx, sc[r]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mnew = fmaxf(m_run, mx);
        float alpha = 1.f, pr[4] = {0.f, 0.f, 0.f, 0.f};
        if (mnew != kNegInf) {
          alpha = fast_exp2(m_run - mnew);
#pragma unroll
          for (int r = 0; r < 4; ++r) pr[r] = fast_exp2(sc[r] - mnew);
        }
        l_run = l_run * alpha + (pr[0] + pr[1]) + (pr[2] + pr[3]);
        m_run = mnew;
#pragma unroll
        for (int gv = 0; gv < NGV; ++gv) acc[gv] *= alpha;
        half4_t pb;
#pragma unroll
        for (int r = 0; r < 4; ++r) pb[r] = (_Float16)(pr[r] * vs[r]);
#pragma unroll
        for (int gv = 0; gv < NGV; ++gv) {
          const uint2 a = decode_group<BITS>(group_sel<BITS>(vw, gv));
          acc[gv] = __builtin_amdgcn_mfma_f32_16x16x16f16(as_half4(a), pb, acc[gv], 0, 0, 0);
        }
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

  // ---- prologue: query operand in LDS (16 head rows x D), rows >= G zero ----
  uint16_t *qs = (uint16_t *)smem;                 // [16][D] f16 or bf16 bits
  float *qf = smem + 16 * D / 2;                   // [G][D] fp32 scratch (TQ rotation)
  const uint16_t *qsrc = p.q + ((int64_t)info.b * p.Hq + (int64_t)g * G) * D;
  const bool tq = info.fmt == FMT_TQ3 || info.fmt == FMT_TQ2;
  if (info.fmt != FMT_EMPTY) {
    if (!tq) {
      for (int t = tid; t < 16 * D; t += blockDim.x) {
        const int n = t / D;
        qs[t] = n < G ? qsrc[t] : (uint16_t)0;
      }
    } else {
      const uint32_t *sg = p.signs + (int64_t)g * 2 * (D / 32);   // K role signs
      for (int t = tid; t < G * D; t += blockDim.x) {
        const int j = t % D;
        float v = __builtin_bit_cast(float, (uint32_t)qsrc[t] << 16);
        if ((sg[j >> 5] >> (j & 31)) & 1u) v = -v;
        qf[t] = v;
      }
      lds_fwht<D>(qf, G);
      const float rs = 1.0f / sqrtf((float)D);
      for (int t = tid; t < 16 * D; t += blockDim.x) {
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
  switch (info.fmt) {
    case FMT_FP8: wave_scan<FMT_FP8, D>(p, info, g, qb, acc, m_run, l_run); break;
    case FMT_TQ3: wave_scan<FMT_TQ3, D>(p, info, g, qb, acc, m_run, l_run); break;
    case FMT_TQ2: wave_scan<FMT_TQ2, D>(p, info, g, qb, acc, m_run, l_run); break;
    default: break;
  }
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);

  // ---- merge the 4 waves in LDS ----
  float *mo = smem;                                   // [4][G][D] unnormalized
  float *mml = smem + kDecodeWaves * G * D;           // [4][G][2]
  {
    const int n = lane & 15;
    if (n < G) {
#pragma unroll
      for (int gv = 0; gv < NGV; ++gv)
#pragma unroll
        for (int r = 0; r < 4; ++r) mo[(wave * G + n) * D + 16 * gv + 4 * (lane >> 4) + r] = acc[gv][r];
      if (lane < 16) {
        mml[(wave * G + n) * 2] = m_run;
        mml[(wave * G + n) * 2 + 1] = l_run;
      }
    }
  }
  __syncthreads();
  const int64_t slot = (int64_t)it * p.Hkv + g;
  float *po = p.part_o + slot * G * D;
  float *pml = p.part_ml + slot * G * 2;
  for (int t = tid; t < G * D; t += blockDim.x) {
    const int n = t / D, j = t % D;
    float M = kNegInf;
    for (int w = 0; w < kDecodeWaves; ++w) M = fmaxf(M, mml[(w * G + n) * 2]);
    float L = 0.f, O = 0.f;
    if (M != kNegInf) {
      for (int w = 0; w < kDecodeWaves; ++w) {
        const float lw = mml[(w * G + n) * 2 + 1];
        if (lw > 0.f) {
          const float e = fast_exp2(mml[(w * G + n) * 2] - M);
          L += e * lw;
          O += e * mo[(w * G + n) * D + j];
        }
      }
    }
    po[t] = L > 0.f ? O / L : 0.f;
    if (j == 0) {
      pml[2 * n] = L > 0.f ? M : kNegInf;
      pml[2 * n + 1] = L;
    }
  }
  if (tid == 0 && p.counters && info.cnt > 0) {
    unsigned long long *c = info.fmt == FMT_FP8 ? &p.counters->pages_fp8
                          : info.fmt == FMT_TQ3 ? &p.counters->pages_tq3 : &p.counters->pages_tq2;
    atomicAdd(c, (unsigned long long)info.cnt);
  }

  // ---- last workgroup of (request, KV head) merges every partial ----
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const uint32_t old = atomicAdd(&p.merge_ctr[(int64_t)info.b * p.Hkv + g], 1u);
    s_last = (old == (uint32_t)(info.n_items - 1));
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();

  // Items of a request are ordered FP8, TQ3, TQ2: FP8 partials (natural
  // space) are items [0, n8), TQ partials (rotated V space) [n8, n_real).
  const int32_t *c4 = p.counts + 4 * info.b;
  const int n8 = (c4[FMT_FP8] + p.S[FMT_FP8] - 1) / p.S[FMT_FP8];
  const int n_real = n8 + (c4[FMT_TQ3] + p.S[FMT_TQ3] - 1) / p.S[FMT_TQ3] +
                     (c4[FMT_TQ2] + p.S[FMT_TQ2] - 1) / p.S[FMT_TQ2];
  const float *ml_b = p.part_ml + (int64_t)info.item_base * p.Hkv * G * 2;
  const float *o_b = p.part_o + (int64_t)info.item_base * p.Hkv * G * D;
  const int64_t ml_stride = (int64_t)p.Hkv * G * 2, o_stride = (int64_t)p.Hkv * G * D;
  const float *ml_g = ml_b + (int64_t)g * G * 2;
  const float *o_g = o_b + (int64_t)g * G * D;

  float *stat = smem;                  // [16][4]: M_rot, L_rot, M_nat, L_nat
  float *orot = smem + 4 * 16;         // [G][D] rotated-space TQ merge
  for (int n = tid; n < G; n += blockDim.x) {
    float Mr = kNegInf, Mn = kNegInf;
    for (int i = 0; i < n_real; ++i) {
      const float *ml = ml_g + i * ml_stride;
      if (ml[2 * n + 1] <= 0.f) continue;
      if (i < n8) Mn = fmaxf(Mn, ml[2 * n]); else Mr = fmaxf(Mr, ml[2 * n]);
    }
    float Lr = 0.f, Ln = 0.f;
    for (int i = 0; i < n_real; ++i) {
      const float *ml = ml_g + i * ml_stride;
      const float li = ml[2 * n + 1];
      if (li <= 0.f) continue;
      if (i < n8) Ln += fast_exp2(ml[2 * n] - Mn) * li;
      else Lr += fast_exp2(ml[2 * n] - Mr) * li;
    }
    stat[4 * n] = Mr; stat[4 * n + 1] = Lr; stat[4 * n + 2] = Mn; stat[4 * n + 3] = Ln;
  }
  __syncthreads();
  // rotated-space merge of the TQ partials (Eq. 11-13 inside the TQ set)
  for (int t = tid; t < G * D; t += blockDim.x) {
    const int n = t / D;
    const float Mr = stat[4 * n], Lr = stat[4 * n + 1];
    float O = 0.f;
    if (Lr > 0.f) {
      for (int i = n8; i < n_real; ++i) {
        const float *ml = ml_g + i * ml_stride;
        const float li = ml[2 * n + 1];
        if (li <= 0.f) continue;
        O += fast_exp2(ml[2 * n] - Mr) * li * o_g[i * o_stride + t];
      }
      O /= Lr;
    }
    orot[t] = O;
  }
  // single inverse V rotation: R_V^T y = s_V * FWHT(y) / sqrt(D)
  lds_fwht<D>(orot, G);
  const uint32_t *sv = p.signs + ((int64_t)g * 2 + 1) * (D / 32);
  const float rs = 1.0f / sqrtf((float)D);
  for (int t = tid; t < G * D; t += blockDim.x) {
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
        L += fast_exp2(Mn - M) * Ln;
        for (int i = 0; i < n8; ++i) {
          const float *ml = ml_g + i * ml_stride;
          const float li = ml[2 * n + 1];
          if (li <= 0.f) continue;
          num += fast_exp2(ml[2 * n] - M) * li * o_g[i * o_stride + t];
        }
      }
    }
    const int64_t orow = ((int64_t)info.b * p.Hq + (int64_t)g * G + n);
    p.out[orow * D + j] = L > 0.f ? num / L : 0.f;
    if (j == 0 && p.lse) p.lse[orow] = L > 0.f ? (M + log2f(L)) * 0.69314718055994531f : kNegInf;
  }
  if (tid == 0) p.merge_ctr[(int64_t)info.b * p.Hkv + g] = 0u;
}

}  // namespace

hipError_t launch_plan(const PlanParams &p, hipStream_t s) {
  if (p.B <= 0) return hipSuccess;
  hipLaunchKernelGGL(plan_kernel, dim3(p.B), dim3(256), 0, s, p);
  return hipGetLastError();
}

size_t decode_lds_bytes(int d, int G) {
  size_t q = 16 * (size_t)d * 2 + (size_t)G * d * 4;
  size_t merge = (size_t)kDecodeWaves * G * d * 4 + (size_t)kDecodeWaves * G * 2 * 4;
  size_t fin = 4 * 16 * 4 + (size_t)G * d * 4;
  size_t m = q > merge ? q : merge;
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
