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
//    item's pages round-robin; TQ items of every width hold the same number
//    of pages and FP8 items the pages of an equal byte count (cost-balanced
//    split-K); a persistent grid draws further items from a dispenser;
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
//  * the query rotation (a length-D FWHT per GQA head) stays in registers:
//    DPP row permutes and the gfx950 lane-swap moves for the cross-lane
//    butterflies; the waves sharing a SIMD balance their progress through
//    the issue priority;
//  * online softmax in fp32 / log2 units; the accumulator is rescaled only
//    when a head's running maximum grows by more than kRescaleSlack (the
//    deferred maximum keeps every exponent <= 2^kRescaleSlack);
//  * grouped mixed-rate keys (TQK, Block-GTQ A.7 / H.1-H.2): the query is
//    permuted and rotated per key segment, the K tile is dealt in 32-coordinate
//    chunks so each MFMA stays inside one segment, and the three segment dot
//    products get their own sigma before the softmax;
//  * the 8 waves merge their partials in LDS and the workgroup writes one
//    normalized partial per (item, KV head); a second kernel merges every
//    partial of a (request, q-head) (Eq. 11-13), applies the single inverse V
//    rotation to the TQ part and writes O and lse;
//  * variants (separate template instantiations, the plain path unchanged):
//    the scored scan also stores each 16-token tile's log-mass per head and
//    the scored merge turns it into ln q~ (Minima-KV Eq. 6-8); the appending
//    merge FP8-encodes the step's new token, attends it as one more
//    partition and writes its slot (Minima-KV algorithm 1 "Append"); a small
//    collector kernel updates the running page score (Eq. 9).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "codebook.h"
#include "kvq_internal.h"
#include "lane_ops.h"

namespace kvq {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int kW = kDecodeWaves;
// sched_barrier mask: ALU, VALU, SALU, MFMA, LDS and transcendental
// instructions may cross; vector-memory instructions may not (their issue
// order must match the ring order for exact in-order waits).
constexpr int kKeepVmemOrder = 0x0F | 0x380 | 0x400;
constexpr float kRescaleSlack = 8.0f;   // log2 units

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

// Grouped mixed-rate keys (TQK): a lane's groups are D/64 2-bit groups, D/32
// 3-bit groups, then D/64 4-bit groups; word triple m holds the 4-bit groups
// of the triple in word 3m (bits 0-3 / 4-7), and the 3-bit pairs plus one
// 2-bit group in words 3m+1 and 3m+2 (bits 0-2 / 3-5 / 6-7).
template <int D>
__host__ __device__ constexpr int tqk_group_bits(int g) {
  return g < D / 64 ? 2 : (g < D / 64 + D / 32 ? 3 : 4);
}
template <int D>
__device__ __forceinline__ uint32_t tqk_group_sel(const uint32_t *w, int g) {
  constexpr int n2 = D / 64, n3 = D / 32;
  if (g < n2) return (w[3 * (g >> 1) + 1 + (g & 1)] >> 6) & 0x03030303u;
  if (g < n2 + n3) {
    const int q = g - n2, m = q >> 2, qq = q & 3;
    const uint32_t word = w[3 * m + 1 + (qq >> 1)];
    return ((qq & 1) ? (word >> 3) : word) & 0x07070707u;
  }
  const int q = g - n2 - n3;
  return (w[3 * (q >> 1)] >> (4 * (q & 1))) & 0x0F0F0F0Fu;
}
template <int D>
__device__ __forceinline__ uint2 tqk_decode_group(const uint32_t *w, int g) {
  const uint32_t sel = tqk_group_sel<D>(w, g);
  const int bits = tqk_group_bits<D>(g);
  return bits == 2 ? decode_group<2>(sel) : (bits == 3 ? decode_group<3>(sel) : decode_group4(sel));
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

// x times the fp16 value in half K (0 low, 1 high) of w: one mixed-precision
// FMA (v_fma_mix) instead of a convert and a multiply. The product is exact
// but for the sign of a zero (the +0 addend, which also keeps the FMA from
// being folded back into a multiply); the callers feed it to exp2 and to
// sums, where the sign of a zero does not matter.
template <int K>
__device__ __forceinline__ float mul_half(float x, uint32_t w) {
  const _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)(K ? (w >> 16) : (w & 0xFFFFu)));
  return __builtin_fmaf(x, (float)h, 0.0f);
}

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Maximum over lanes l, l ^ 16, l ^ 32, l ^ 48 (the four lane groups that hold
// one MFMA column). Each step takes the partner's value with lane_xor (a
// lane-swap move and a per-lane pick of its result, converted by value) and
// keeps the larger. (A __builtin_bit_cast applied directly to an element of
// an ext_vector_type value, such as a lane swap's result, reads element 0's
// bits whatever the index: fmaxf over bit_cast(r[0]) and bit_cast(r[1]) saw
// one value twice.)
__device__ __forceinline__ float lane_max4(float x) {
  const int lane = (int)(threadIdx.x & 63);
  const float m1 = fmaxf(x, lane_xor<32>(x, lane));
  return fmaxf(m1, lane_xor<16>(m1, lane));
}

// One butterfly stage between lanes at distance M: the lower lane keeps
// a + b, the upper one a - b.
template <int M, int E>
__device__ __forceinline__ void lane_butterfly(float (&x)[E], int lane) {
  const bool upper = (lane & M) != 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const float o = lane_xor<M>(x[e], lane);
    x[e] = upper ? (o - x[e]) : (x[e] + o);
  }
}

// Unnormalized Walsh-Hadamard transform of one length-D row held by a wave,
// lane l holding elements E l + e (E = D / 64): the in-register stages, then
// the six lane stages.
template <int D>
__device__ __forceinline__ void wave_fwht_rows(float (&x)[D / 64], int lane) {
  constexpr int E = D / 64;
#pragma unroll
  for (int h = 1; h < E; h <<= 1) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if ((e & h) == 0) {
        const float a = x[e], c = x[e + h];
        x[e] = a + c;
        x[e + h] = a - c;
      }
    }
  }
  lane_butterfly<1, E>(x, lane);
  lane_butterfly<2, E>(x, lane);
  lane_butterfly<4, E>(x, lane);
  lane_butterfly<8, E>(x, lane);
  lane_butterfly<16, E>(x, lane);
  lane_butterfly<32, E>(x, lane);
}

constexpr float kNegInf = -__builtin_inff();

// Whether the plan was built for this call's geometry (read once per
// workgroup; the plan's header is its first 32 bytes, a and c).
__device__ __forceinline__ bool header_matches(const DecodeParams &p, int4 a, int4 c) {
  const bool ok = a.x == kPlanMagic && a.y == p.B && a.z == p.max_pages && a.w == p.Hkv && c.x == p.P && c.y == p.D;
  return __builtin_amdgcn_readfirstlane((int)ok) != 0;
}

// One unit's packet as a wave reads it: the item header and the wave's page
// entries (entry wave + kW lane), one round trip.
struct PacketRaw {
  int4 h0, h1;
  int2 ent;
};
__device__ __forceinline__ PacketRaw load_packet(const DecodeParams &p, int64_t it, int wave, int lane, int s_max) {
  const uint8_t *pk = p.packets + it * p.packet_stride;
  PacketRaw r;
  r.h0 = *(const int4 *)pk;
  r.h1 = *(const int4 *)(pk + 16);
  const int ei = wave + kW * lane;
  r.ent = make_int2(0, 0);
  if (ei < s_max) r.ent = *(const int2 *)(pk + sizeof(ItemHeader) + 8 * ei);
  return r;
}

// Lane index as a value the optimizer cannot treat as loop-invariant: in the
// persistent loop this keeps per-lane address math inside the loop body
// instead of hoisting dozens of live registers across it.
__device__ __forceinline__ int fresh_lane() {
  int l = (int)(threadIdx.x & 63);
  asm volatile("" : "+v"(l));
  return l;
}

// ------------------------------------------------------------------------
// plan: per-request compact lists by format (order kept), counts, lengths
// ------------------------------------------------------------------------
constexpr int kPlanThreads = 1024;
constexpr int kPlanRegs = 8;          // table entries per thread held in registers

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
  if (b == 0 && tid == 0) {
    *p.ticket = 0u;
    PlanHeader hd;
    hd.magic = kPlanMagic; hd.B = p.B; hd.max_pages = p.max_pages; hd.Hkv = p.Hkv; hd.P = p.P; hd.d = p.d;
    hd.pad0 = 0; hd.pad1 = 0;
    *p.hdr = hd;
  }
  const int32_t *bt = p.block_table + (int64_t)b * p.max_pages;
  const uint8_t *pf = p.page_format + (int64_t)b * p.max_pages;
  // each thread owns a contiguous run of pages; up to kPlanRegs of them are
  // loaded at once into registers (one round trip) and reused by the second pass
  const int chunk = (n_pages + kPlanThreads - 1) / kPlanThreads;
  const int k0 = min(n_pages, tid * chunk), k1 = min(n_pages, k0 + chunk);
  int rf[kPlanRegs], rp[kPlanRegs];
#pragma unroll
  for (int u = 0; u < kPlanRegs; ++u) {
    rf[u] = k0 + u < k1 ? (int)pf[k0 + u] : 255;
    rp[u] = k0 + u < k1 ? bt[k0 + u] : -1;
  }
  auto fmt_of = [&](int f, int pid) {   // the entry's format, or NFMT if it is masked
    return (f < NFMT && pid >= 0 && pid < p.pool_pages[f < NFMT ? f : 0]) ? f : NFMT;
  };
  int cnt[NFMT + 1] = {};             // [NFMT] = invalid entries
#pragma unroll
  for (int u = 0; u < kPlanRegs; ++u)
    if (k0 + u < k1) cnt[fmt_of(rf[u], rp[u])]++;
  for (int k = k0 + kPlanRegs; k < k1; ++k) cnt[fmt_of(pf[k], bt[k])]++;
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
    for (int f = 0; f < NFMT; ++f) p.counts[b * NFMT + f] = tot[f];
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
  auto place = [&](int k, int f, int pid) {
    if (fmt_of(f, pid) == NFMT) return;
    int at = 0;
#pragma unroll
    for (int ff = 0; ff < NFMT; ++ff)
      if (ff == f) at = pos[ff]++;
    ent[at] = make_int2(k, pid);
  };
#pragma unroll
  for (int u = 0; u < kPlanRegs; ++u)
    if (k0 + u < k1) place(k0 + u, rf[u], rp[u]);
  for (int k = k0 + kPlanRegs; k < k1; ++k) place(k, pf[k], bt[k]);
}

// ------------------------------------------------------------------------
// items: one wave per item slot. Items of a request are its FP8 runs, then
// TQ3, TQ2 and TQK runs (equal runs of about S_f pages); requests follow each other. The
// wave locates item k (prefix over the requests' item counts), then writes
// its packet: header plus the item's page entries.
// ------------------------------------------------------------------------
__device__ __forceinline__ int items_of(const int32_t *cnt4, const int *S, int *n8) {
  int n = 0;
  for (int f = 0; f < NFMT; ++f) {
    const int nf = items_in_list(cnt4[f], S[f]);
    if (f == FMT_FP8) *n8 = nf;
    n += nf;
  }
  return n > 0 ? n : 1;
}

__global__ __launch_bounds__(64) void items_kernel(PlanParams p) {
  const int lane = threadIdx.x;
  const int64_t k = blockIdx.x;
  if (k == 0) {
    // the batch's item count, next to the dispenser
    int tot = 0;
    for (int b = lane; b < p.B; b += 64) {
      int n8 = 0;
      tot += items_of(p.counts + NFMT * b, p.S, &n8);
    }
    for (int off = 32; off >= 1; off >>= 1) tot += __shfl_xor(tot, off);
    if (lane == 0) p.ticket[1] = (uint32_t)tot;
  }
  ItemHeader h;
  h.b = 0; h.fmt = FMT_EMPTY; h.cnt = 0; h.seq = 0; h.n_items = 0; h.item_base = 0; h.n8 = 0; h.valid = 0;
  int list_off = 0, start = 0;
  int64_t base = 0;
  for (int b0 = 0; b0 < p.B; b0 += 64) {
    const int b = b0 + lane;
    int n = 0, n8 = 0;
    if (b < p.B) n = items_of(p.counts + NFMT * b, p.S, &n8);
    int incl = n;
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(incl, off);
      if (lane >= off) incl += t;
    }
    const int excl = incl - n;
    const bool mine = b < p.B && k >= base + excl && k < base + incl;
    const uint64_t m = __ballot(mine);
    if (m) {
      const int src = __ffsll((unsigned long long)m) - 1;
      h.b = __shfl(b, src);
      h.n_items = __shfl(n, src);
      h.n8 = __shfl(n8, src);
      h.item_base = (int)(base + __shfl(excl, src));
      h.seq = p.seq[h.b];
      h.valid = 1;
      int local = (int)(k - h.item_base);
      const int32_t *c4 = p.counts + NFMT * h.b;
      int off = 0;
      for (int f = 0; f < NFMT; ++f) {
        const int nf = items_in_list(c4[f], p.S[f]);
        if (local < nf) {
          h.fmt = f;
          start = (int)((int64_t)local * c4[f] / nf);
          h.cnt = (int)((int64_t)(local + 1) * c4[f] / nf) - start;
          list_off = off;
          break;
        }
        local -= nf;
        off += c4[f];
      }
      break;
    }
    base += __shfl(incl, 63);
  }
  uint8_t *pk = p.packets + k * p.packet_stride;
  if (lane == 0) {
    *(ItemHeader *)pk = h;
    if (h.valid && k == h.item_base) {
      ReqItems r;
      r.item_base = h.item_base;
      r.n_items = h.n_items;
      r.n8 = h.n8;
      r.pad = 0;
      p.req[h.b] = r;
    }
  }
  int2 *pe = (int2 *)(pk + sizeof(ItemHeader));
  const int2 *src = p.entries + (int64_t)h.b * p.max_pages + list_off + start;
  // the first 4 x 64 entries in one round trip, then the rest
  int2 e4[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) e4[u] = lane + 64 * u < h.cnt ? src[lane + 64 * u] : make_int2(0, 0);
#pragma unroll
  for (int u = 0; u < 4; ++u)
    if (lane + 64 * u < h.cnt) pe[lane + 64 * u] = e4[u];
  for (int i = lane + 256; i < h.cnt; i += 64) pe[i] = src[i];
}

// ---- tiles held in registers: one 16-token K tile and V tile of a page ----
template <int FMT, int D>
struct Tile;

template <int D>
struct Tile<FMT_FP8, D> {
  uint4 k[D / 64], v[D / 64];
  uint4 ks, vs;      // fp32 scale bits of the lane's four tokens
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
template <int D>
struct Tile<FMT_TQK, D> {
  uint32_t k[D * 3 / 128], v[D * 3 / 128];
  uint2 ks[3], vs;   // K sigma of the lane's four tokens per segment; V sigma
};

// Fractional-level tiles: the raw bytes of the K and V tile (16 rows of R
// bytes) dealt to lanes in 16-byte slices (the first 1024 bytes), then 8-byte
// slices (the rest, d = 256), plus the sigmas of the lane's four tokens.
__host__ __device__ constexpr bool is_tqf(int fmt) { return fmt == FMT_TQF5 || fmt == FMT_TQF6; }
template <int D>
constexpr int tqf_raw_words() { return D == 128 ? 4 : 6; }
template <int D>
struct TileTqf {
  uint32_t k[tqf_raw_words<D>()], v[tqf_raw_words<D>()];
  uint2 ks, vs;
};
template <int D>
struct Tile<FMT_TQF5, D> : TileTqf<D> {};
template <int D>
struct Tile<FMT_TQF6, D> : TileTqf<D> {};

// Buffer resource of one (page, KV head) block: scalar base, range-checked
// to the block (a read past it returns zeros instead of faulting).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(const uint8_t *head, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void *)head, (short)0, bytes, 0x00020000);
}

// The float with these bits (for the words buffer loads return).
__device__ __forceinline__ float f32_bits(uint32_t x) { return __builtin_bit_cast(float, x); }

// Cache policy of the scans' KV tile loads: non-temporal. A call reads each
// (page, KV head) block once, so the tiles are not worth keeping in L2 or in
// the memory-side cache; streaming them past both leaves those to the plan's
// packets, the queries and the partial rows that the merge reads back.
constexpr int kStreamLoad = 2;

// Words of one role of a TQ tile for lane `lane` (tile at byte `t0` of the
// block), following the region rule of the page layout (regions of 4, then
// 2, then 1 words per lane).
template <int WN>
__device__ __forceinline__ void load_tq_words(uint32_t (&w)[WN], __amdgpu_buffer_rsrc_t r, int t0, int lane) {
  if constexpr (WN == 6) {
    const auto a = __builtin_amdgcn_raw_buffer_load_b128(r, lane * 16, t0, kStreamLoad);
    const auto b = __builtin_amdgcn_raw_buffer_load_b64(r, lane * 8, t0 + 1024, kStreamLoad);
    w[0] = a[0]; w[1] = a[1]; w[2] = a[2]; w[3] = a[3]; w[4] = b[0]; w[5] = b[1];
  } else if constexpr (WN == 3) {
    const auto a = __builtin_amdgcn_raw_buffer_load_b64(r, lane * 8, t0, kStreamLoad);
    w[0] = a[0]; w[1] = a[1];
    w[2] = __builtin_amdgcn_raw_buffer_load_b32(r, lane * 4, t0 + 512, kStreamLoad);
  } else if constexpr (WN == 4) {
    const auto a = __builtin_amdgcn_raw_buffer_load_b128(r, lane * 16, t0, kStreamLoad);
    w[0] = a[0]; w[1] = a[1]; w[2] = a[2]; w[3] = a[3];
  } else {
    static_assert(WN == 2, "unsupported TQ word count");
    const auto a = __builtin_amdgcn_raw_buffer_load_b64(r, lane * 8, t0, kStreamLoad);
    w[0] = a[0]; w[1] = a[1];
  }
}

// Tile tau of the (page, KV head) block described by r.
template <int FMT, int D>
__device__ __forceinline__ void load_tile(Tile<FMT, D> &t, __amdgpu_buffer_rsrc_t r, int tau, int T, int P, int lane) {
  const int grp = lane >> 4;
  if constexpr (FMT == FMT_FP8) {
    const int kt = tau * 16 * D, vt = (T + tau) * 16 * D;
#pragma unroll
    for (int i = 0; i < D / 64; ++i) {
      const auto a = __builtin_amdgcn_raw_buffer_load_b128(r, lane * 16, kt + i * 1024, kStreamLoad);
      const auto b = __builtin_amdgcn_raw_buffer_load_b128(r, lane * 16, vt + i * 1024, kStreamLoad);
      t.k[i] = make_uint4(a[0], a[1], a[2], a[3]);
      t.v[i] = make_uint4(b[0], b[1], b[2], b[3]);
    }
    const auto ks = __builtin_amdgcn_raw_buffer_load_b128(r, 16 * grp, 2 * P * D + 64 * tau, kStreamLoad);
    const auto vs = __builtin_amdgcn_raw_buffer_load_b128(r, 16 * grp, 2 * P * D + 4 * P + 64 * tau, kStreamLoad);
    t.ks = make_uint4(ks[0], ks[1], ks[2], ks[3]);
    t.vs = make_uint4(vs[0], vs[1], vs[2], vs[3]);
  } else if constexpr (is_tqf(FMT)) {
    constexpr int RT = 16 * tqf_row_bytes(D, tqf_levels(FMT));   // one tile of rows
    const int k0 = tau * RT, v0 = T * RT + tau * RT;
    // lanes whose slice lies past the tile read with an offset outside the
    // block: the buffer returns zeros without a memory request
    constexpr int kOff = 1 << 30;
    const int o16 = lane * 16 < (D == 256 ? 1024 : RT) ? lane * 16 : kOff;
    const auto a = __builtin_amdgcn_raw_buffer_load_b128(r, o16, k0, kStreamLoad);
    const auto b = __builtin_amdgcn_raw_buffer_load_b128(r, o16, v0, kStreamLoad);
    t.k[0] = a[0]; t.k[1] = a[1]; t.k[2] = a[2]; t.k[3] = a[3];
    t.v[0] = b[0]; t.v[1] = b[1]; t.v[2] = b[2]; t.v[3] = b[3];
    if constexpr (D == 256) {
      const int o8 = lane * 8 < RT - 1024 ? lane * 8 : kOff;
      const auto c = __builtin_amdgcn_raw_buffer_load_b64(r, o8, k0 + 1024, kStreamLoad);
      const auto e = __builtin_amdgcn_raw_buffer_load_b64(r, o8, v0 + 1024, kStreamLoad);
      t.k[4] = c[0]; t.k[5] = c[1];
      t.v[4] = e[0]; t.v[5] = e[1];
    }
    const int sig = 2 * T * RT;
    const auto ks = __builtin_amdgcn_raw_buffer_load_b64(r, 8 * grp, sig + 32 * tau, kStreamLoad);
    const auto vs = __builtin_amdgcn_raw_buffer_load_b64(r, 8 * grp, sig + 2 * P + 32 * tau, kStreamLoad);
    t.ks = make_uint2(ks[0], ks[1]);
    t.vs = make_uint2(vs[0], vs[1]);
  } else if constexpr (FMT == FMT_TQK) {
    constexpr int tile_bytes = 16 * D * 3 / 8;
    load_tq_words(t.k, r, tau * tile_bytes, lane);
    load_tq_words(t.v, r, (T + tau) * tile_bytes, lane);
    const int sig = 2 * T * tile_bytes;
#pragma unroll
    for (int sgm = 0; sgm < 3; ++sgm) {
      const auto ks = __builtin_amdgcn_raw_buffer_load_b64(r, 8 * grp, sig + sgm * 2 * P + 32 * tau, kStreamLoad);
      t.ks[sgm] = make_uint2(ks[0], ks[1]);
    }
    const auto vs = __builtin_amdgcn_raw_buffer_load_b64(r, 8 * grp, sig + 6 * P + 32 * tau, kStreamLoad);
    t.vs = make_uint2(vs[0], vs[1]);
  } else {
    constexpr int BITS = FMT == FMT_TQ3 ? 3 : 2;
    constexpr int tile_bytes = 16 * D * BITS / 8;
    load_tq_words(t.k, r, tau * tile_bytes, lane);
    load_tq_words(t.v, r, (T + tau) * tile_bytes, lane);
    const int sig = 2 * T * tile_bytes;
    const auto ks = __builtin_amdgcn_raw_buffer_load_b64(r, 8 * grp, sig + 32 * tau, kStreamLoad);
    const auto vs = __builtin_amdgcn_raw_buffer_load_b64(r, 8 * grp, sig + 2 * P + 32 * tau, kStreamLoad);
    t.ks = make_uint2(ks[0], ks[1]);
    t.vs = make_uint2(vs[0], vs[1]);
  }
}

// Natural log of one 16-token tile's unnormalized attention mass per head,
// ln sum_i e^{s_i} = (m + log2 sum_i 2^{s_i - m}) ln 2 from the scan's
// log2-unit probabilities pr (masked tokens are 0): summed over the four lane
// groups of the head's column, stored by the head's lane into the wave's LDS
// stage (mrow is null in every other lane, and mi < 0 marks a tile past the
// list); the workgroup writes the unit's stage out after the scan.
__device__ __forceinline__ void tile_mass_store(const float *pr, float m_run, float *mrow, int mi, int lane) {
  float s = (pr[0] + pr[1]) + (pr[2] + pr[3]);
  s += lane_xor<16>(s, lane);
  s += lane_xor<32>(s, lane);
  if (mrow != nullptr && mi >= 0) mrow[mi] = (m_run + __builtin_amdgcn_logf(s)) * 0.69314718055994531f;
}

// One tile: scores, online softmax (deferred rescale), P V. MASS: also the
// tile's log-mass per head (tile_mass_store).
// Per-wave LDS of the fractional-level scan, after the query staging: the
// raw tile (16-byte then 8-byte lane slices, as loaded) and the code bytes,
// row-major [token][D + 8] for K (8-byte operand reads) or transposed
// [dim][kTqfVStride] for V (4-byte reads of four tokens).
constexpr int kTqfVStride = 20;
__host__ __device__ constexpr int tqf_raw_bytes(int D) { return D == 128 ? 1024 : 1536; }
__host__ __device__ constexpr int tqf_code_bytes(int D) {
  return 16 * (D + 8) > D * kTqfVStride ? 16 * (D + 8) : D * kTqfVStride;
}
__host__ __device__ constexpr int tqf_wave_bytes(int D) { return tqf_raw_bytes(D) + tqf_code_bytes(D); }
__host__ __device__ constexpr int query_stage_bytes(int D) { return ((16 * (D + 8) * 2) + 15) & ~15; }

template <int D>
__device__ __forceinline__ void tqf_stage_raw(uint32_t *raw, const uint32_t (&w)[tqf_raw_words<D>()], int lane) {
  *(uint4 *)(raw + 4 * lane) = make_uint4(w[0], w[1], w[2], w[3]);
  if constexpr (D == 256) *(uint2 *)(raw + 256 + 2 * lane) = make_uint2(w[4], w[5]);
}

template <int FMT, int D, bool MASS = false>
__device__ __forceinline__ void process_tile(const Tile<FMT, D> &t, int nvalid, const uint32_t *qb, float scale_log2,
                                             float4_t (&acc)[D / 16], float &m_run, float &l_run, int lane,
                                             float *mrow = nullptr, int mi = -1, int dn = 0, uint8_t *wl = nullptr) {
  constexpr int NKK = D / 32;
  constexpr int NGV = D / 16;
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
    ks[0] = __builtin_bit_cast(float, t.ks.x) * scale_log2; ks[1] = __builtin_bit_cast(float, t.ks.y) * scale_log2;
    ks[2] = __builtin_bit_cast(float, t.ks.z) * scale_log2; ks[3] = __builtin_bit_cast(float, t.ks.w) * scale_log2;
    vs[0] = __builtin_bit_cast(float, t.vs.x); vs[1] = __builtin_bit_cast(float, t.vs.y);
    vs[2] = __builtin_bit_cast(float, t.vs.z); vs[3] = __builtin_bit_cast(float, t.vs.w);
  } else if constexpr (is_tqf(FMT)) {
    // the K rows go to LDS, their mixed-radix groups become code bytes
    // there, and each lane reads its operand's codes (eight at a time)
    constexpr int L = tqf_levels(FMT);
    uint32_t *raw = (uint32_t *)wl;
    uint8_t *codes = wl + tqf_raw_bytes(D);
    tqf_stage_raw<D>(raw, t.k, lane);
    wave_lds_sync();
    tqf_unpack_tile<D, L, true>(raw, codes, D + 8, lane);
    wave_lds_sync();
    const uint8_t *crow = codes + (lane & 15) * (D + 8) + (lane >> 4) * (D / 4);
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const uint2 c8 = *(const uint2 *)(crow + 8 * kk);
      const uint2 lo = decode_group_levels<L>(c8.x);
      const uint2 hi = decode_group_levels<L>(c8.y);
      const half8_t bq = as_half8(qb[4 * kk], qb[4 * kk + 1], qb[4 * kk + 2], qb[4 * kk + 3]);
      s = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(lo.x, lo.y, hi.x, hi.y), bq, s, 0, 0, 0);
    }
    ks[0] = half_bits_to_float(t.ks.x & 0xFFFF); ks[1] = half_bits_to_float(t.ks.x >> 16);
    ks[2] = half_bits_to_float(t.ks.y & 0xFFFF); ks[3] = half_bits_to_float(t.ks.y >> 16);
    vs[0] = half_bits_to_float(t.vs.x & 0xFFFF); vs[1] = half_bits_to_float(t.vs.x >> 16);
    vs[2] = half_bits_to_float(t.vs.y & 0xFFFF); vs[3] = half_bits_to_float(t.vs.y >> 16);
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
    sc[r] = (4 * grp + r < nvalid - dn) ? s[r] * ks[r] : kNegInf;
    mx = fmaxf(mx, sc[r]);
  }
  mx = lane_max4(mx);
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
  if constexpr (MASS) tile_mass_store(pr, m_run, mrow, mi, lane);
  half4_t pb;
#pragma unroll
  for (int r = 0; r < 4; ++r) pb[r] = (_Float16)(4 * grp + r < nvalid - dn ? pr[r] * vs[r] : 0.f);
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
  } else if constexpr (is_tqf(FMT)) {
    // V rows the same way, codes transposed: a lane's operand is four tokens
    // of one dim, one 4-byte read (the K reads above are done first: the
    // wave's LDS accesses execute in order)
    constexpr int L = tqf_levels(FMT);
    uint32_t *raw = (uint32_t *)wl;
    uint8_t *codes = wl + tqf_raw_bytes(D);
    wave_lds_sync();
    tqf_stage_raw<D>(raw, t.v, lane);
    wave_lds_sync();
    tqf_unpack_tile<D, L, false>(raw, codes, kTqfVStride, lane);
    wave_lds_sync();
#pragma unroll
    for (int gv = 0; gv < NGV; ++gv) {
      const uint32_t c4 = *(const uint32_t *)(codes + (16 * gv + (lane & 15)) * kTqfVStride + 4 * (lane >> 4));
      const uint2 a = decode_group_levels<L>(c4);
      acc[gv] = __builtin_amdgcn_mfma_f32_16x16x16f16(as_half4(a), pb, acc[gv], 0, 0, 0);
    }
    wave_lds_sync();
  } else {
    constexpr int BITS = FMT == FMT_TQ3 ? 3 : 2;
#pragma unroll
    for (int gv = 0; gv < NGV; ++gv) {
      const uint2 a = decode_group<BITS>(group_sel<BITS>(t.v, gv));
      acc[gv] = __builtin_amdgcn_mfma_f32_16x16x16f16(as_half4(a), pb, acc[gv], 0, 0, 0);
    }
  }
}

// Two TQ tiles at once (32 tokens): two independent QK chains, one softmax
// update for both, and P V as 16x16x32 MFMAs whose contraction runs over the
// 32 tokens: k = 8 (lane/16) + i holds tile i/4, token 4 (lane/16) + i%4,
// which is exactly how the QK accumulators of the two tiles sit in a lane.
// A tile with nvalid <= 0 contributes nothing (every score masked). MASK =
// false is the steady state: both tiles hold 16 live tokens, so no score is
// masked and the running maximum is finite after the rescale step.
template <int FMT, int D, bool MASK = true, bool MASS = false>
__device__ __forceinline__ void process_pair(const Tile<FMT, D> &t0, const Tile<FMT, D> &t1, int nv0, int nv1,
                                             const uint32_t *qb, float4_t (&acc)[D / 16], float &m_run,
                                             float &l_run, int lane, float *mrow = nullptr, int mi0 = -1,
                                             int mi1 = -1, int dn = 0) {
  static_assert(FMT != FMT_FP8, "pairs are for TQ tiles");
  constexpr int NKK = D / 32;
  constexpr int NGV = D / 16;
  constexpr int BITS = FMT == FMT_TQ2 ? 2 : 3;     // uniform keys; every V tile
  const int grp = lane >> 4;
  float sk0[4], sk1[4];                            // sigma-scaled scores of the two tiles
  if constexpr (FMT == FMT_TQK) {
    // one accumulator per key segment: chunk kk (32 permuted coordinates) is
    // in segment 0 for kk < D/128, segment 1 for kk < 3D/128, else segment 2
    float4_t a0[3], a1[3];
#pragma unroll
    for (int sgm = 0; sgm < 3; ++sgm) a0[sgm] = a1[sgm] = (float4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const int sgm = kk < D / 128 ? 0 : (kk < 3 * D / 128 ? 1 : 2);
      const half8_t bq = as_half8(qb[4 * kk], qb[4 * kk + 1], qb[4 * kk + 2], qb[4 * kk + 3]);
      const uint2 x0 = tqk_decode_group<D>(t0.k, 2 * kk), y0 = tqk_decode_group<D>(t0.k, 2 * kk + 1);
      a0[sgm] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(x0.x, x0.y, y0.x, y0.y), bq, a0[sgm], 0, 0, 0);
      const uint2 x1 = tqk_decode_group<D>(t1.k, 2 * kk), y1 = tqk_decode_group<D>(t1.k, 2 * kk + 1);
      a1[sgm] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(x1.x, x1.y, y1.x, y1.y), bq, a1[sgm], 0, 0, 0);
    }
    // sum over segments of sigma_s * S_s, one mixed-precision FMA per term
    auto sig_dot = [](const float4_t (&a)[3], const uint2 (&k)[3], int r) {
      float v = 0.f;
#pragma unroll
      for (int sgm = 0; sgm < 3; ++sgm) {
        const uint32_t w = r < 2 ? k[sgm].x : k[sgm].y;
        const _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)((r & 1) ? (w >> 16) : (w & 0xFFFFu)));
        v = __builtin_fmaf(a[sgm][r], (float)h, v);
      }
      return v;
    };
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sk0[r] = sig_dot(a0, t0.ks, r);
      sk1[r] = sig_dot(a1, t1.ks, r);
    }
  } else {
    float4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const half8_t bq = as_half8(qb[4 * kk], qb[4 * kk + 1], qb[4 * kk + 2], qb[4 * kk + 3]);
      const uint2 a0 = decode_group<BITS>(group_sel<BITS>(t0.k, 2 * kk));
      const uint2 b0 = decode_group<BITS>(group_sel<BITS>(t0.k, 2 * kk + 1));
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(a0.x, a0.y, b0.x, b0.y), bq, s0, 0, 0, 0);
      const uint2 a1 = decode_group<BITS>(group_sel<BITS>(t1.k, 2 * kk));
      const uint2 b1 = decode_group<BITS>(group_sel<BITS>(t1.k, 2 * kk + 1));
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(a1.x, a1.y, b1.x, b1.y), bq, s1, 0, 0, 0);
    }
    sk0[0] = mul_half<0>(s0[0], t0.ks.x); sk0[1] = mul_half<1>(s0[1], t0.ks.x);
    sk0[2] = mul_half<0>(s0[2], t0.ks.y); sk0[3] = mul_half<1>(s0[3], t0.ks.y);
    sk1[0] = mul_half<0>(s1[0], t1.ks.x); sk1[1] = mul_half<1>(s1[1], t1.ks.x);
    sk1[2] = mul_half<0>(s1[2], t1.ks.y); sk1[3] = mul_half<1>(s1[3], t1.ks.y);
  }
  // scores in log2 units (the rotated query carries sm_scale * log2 e)
  float sc[8];
  float mx = kNegInf;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    sc[r] = (!MASK || 4 * grp + r < nv0 - dn) ? sk0[r] : kNegInf;
    sc[4 + r] = (!MASK || 4 * grp + r < nv1 - dn) ? sk1[r] : kNegInf;
  }
#pragma unroll
  for (int r = 0; r < 8; ++r) mx = fmaxf(mx, sc[r]);
  mx = lane_max4(mx);
  if (__builtin_amdgcn_ballot_w64(mx > m_run + kRescaleSlack) != 0) {
    const float mnew = fmaxf(m_run, mx);
    const float alpha = mnew == kNegInf ? 1.f : fast_exp2(m_run - mnew);
    l_run *= alpha;
#pragma unroll
    for (int gv = 0; gv < NGV; ++gv) acc[gv] *= alpha;
    m_run = mnew;
  }
  float pr[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) pr[r] = (MASK && m_run == kNegInf) ? 0.f : fast_exp2(sc[r] - m_run);
  l_run += ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
  if constexpr (MASS) {
    tile_mass_store(pr, m_run, mrow, mi0, lane);
    tile_mass_store(pr + 4, m_run, mrow, mi1, lane);
  }
  // P times the tokens' V sigma, as the f16 B operand
  float pv[8];
  pv[0] = mul_half<0>(pr[0], t0.vs.x); pv[1] = mul_half<1>(pr[1], t0.vs.x);
  pv[2] = mul_half<0>(pr[2], t0.vs.y); pv[3] = mul_half<1>(pr[3], t0.vs.y);
  pv[4] = mul_half<0>(pr[4], t1.vs.x); pv[5] = mul_half<1>(pr[5], t1.vs.x);
  pv[6] = mul_half<0>(pr[6], t1.vs.y); pv[7] = mul_half<1>(pr[7], t1.vs.y);
  half8_t pb;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    pb[r] = (_Float16)((!MASK || 4 * grp + r < nv0 - dn) ? pv[r] : 0.f);
    pb[4 + r] = (_Float16)((!MASK || 4 * grp + r < nv1 - dn) ? pv[4 + r] : 0.f);
  }
#pragma unroll
  for (int gv = 0; gv < NGV; ++gv) {
    const uint2 a = decode_group<BITS>(group_sel<BITS>(t0.v, gv));
    const uint2 b = decode_group<BITS>(group_sel<BITS>(t1.v, gv));
    acc[gv] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(a.x, a.y, b.x, b.y), pb, acc[gv], 0, 0, 0);
  }
}

// Unnormalized Walsh-Hadamard transform of segments of a D-vector held by a
// wave, E = D / 64 consecutive elements per lane (element e of lane l is
// index E l + e), butterfly stages h = 1, 2, 4, ...: in-lane for h < E, across
// lanes above. A lane's segment is lanes [lane0, lane0 + nl): the whole wave
// (lane0 0, nl 64) for a uniform TQ query, three segments for grouped keys.
template <int D>
__device__ __forceinline__ void wave_fwht(float (&x)[D / 64], int lane, int lane0 = 0, int nl = 64) {
  constexpr int E = D / 64;
#pragma unroll
  for (int h = 1; h < E; h <<= 1) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if ((e & h) == 0) {
        const float a = x[e], c = x[e + h];
        x[e] = a + c;
        x[e + h] = a - c;
      }
    }
  }
  const int ll = lane - lane0;
#pragma unroll
  for (int h = E; h < D; h <<= 1) {
    const int dl = h / E;
    const bool upper = (ll & dl) != 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float o = __shfl(x[e], lane0 + (ll ^ dl));
      if (dl < nl) x[e] = upper ? (o - x[e]) : (x[e] + o);
    }
  }
}

// Query operand modes: the bf16 query (FP8 items), the rotated query q_r =
// H (s_K * q) / sqrt(D) (uniform TQ items), or the grouped-key query: q
// permuted by the key coordinate order, then rotated segment by segment,
// R_s q_s = H_s (s_s * q_s) / sqrt(d_s) (Block-GTQ H.2).
enum : int { QM_BF16 = 0, QM_ROT = 1, QM_GROUPED = 2 };
constexpr int kQPad = 8;   // halves of padding per staged query row (keeps LDS reads conflict-free)

// Raw bf16 words of rows wave and wave + kW of the query group, the K sign
// bits of this lane's elements and (grouped keys) the lane's entries of the
// key coordinate order; fetched first so the loads return ahead of the tile
// loads issued after them.
constexpr int kQRows = 16 / kW;   // query rows (heads) a wave rotates: wave, wave + kW, ...
template <int D>
struct QueryRaw {
  uint32_t w[kQRows][D / 128];
  uint32_t sw;
  uint32_t perm[D / 128];
};

template <int D, int QM, bool CAUSAL>
__device__ __forceinline__ QueryRaw<D> fetch_query(const DecodeParams &p, int b, int g) {
  constexpr int E = D / 64;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = p.G;
  QueryRaw<D> r;
#pragma unroll
  for (int i = 0; i < kQRows; ++i) {
    const int n = wave + i * kW;
    if (n < G) {
      // row n: head g G + n (decode), or head g Gr + nn of the request's
      // token c for row n = c Gr + nn (chunked prefill)
      const uint16_t *qrow = p.q + ((int64_t)b * p.Hq + (int64_t)g * G + n) * D;
      if constexpr (CAUSAL) {
        const int c = n / p.Gr, nn = n - c * p.Gr;
        qrow = p.q + (((int64_t)b * p.chunk + c) * p.Hq_r + (int64_t)g * p.Gr + nn) * D;
      }
      if constexpr (E == 4) {
        const uint2 v = *(const uint2 *)(qrow + E * lane);
        r.w[i][0] = v.x; r.w[i][1] = v.y;
      } else {
        r.w[i][0] = *(const uint32_t *)(qrow + E * lane);
      }
    } else {
#pragma unroll
      for (int k = 0; k < E / 2; ++k) r.w[i][k] = 0u;
    }
  }
  r.sw = QM != QM_BF16 ? p.signs[(int64_t)g * 2 * (D / 32) + (E * lane) / 32] >> ((E * lane) & 31) : 0u;
#pragma unroll
  for (int k = 0; k < E / 2; ++k)
    r.perm[k] = QM == QM_GROUPED ? *(const uint32_t *)(p.tqk_perm + (int64_t)g * D + E * lane + 2 * k) : 0u;
  return r;
}

// Query operand of KV head g for this wave's MFMAs: lane (head n = lane % 16,
// k-block lane / 16) holds, for MFMA kk, dims (lane/16) D/4 + 8 kk + e (the
// uniform K tile order) or 32 kk + 8 (lane/16) + e (grouped keys: one
// 32-coordinate chunk per MFMA). The rotated forms carry sm_scale * log2(e)
// so TQ scores need only sigma_K; wave w rotates heads w and w + 8 with
// shuffles. Rows >= G are zero. Every thread calls it.
template <int D, int QM>
__device__ __forceinline__ void finish_query(const DecodeParams &p, const QueryRaw<D> &raw, float *smem,
                                             uint32_t (&qb)[D / 8]) {
  constexpr int DL = D / 4;
  constexpr int NKK = D / 32;
  constexpr int E = D / 64;
  constexpr int RS = D + kQPad;                    // staged row stride (halves)
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = p.G;
  uint16_t *qs = (uint16_t *)smem;                 // [16][RS] f16 or bf16 bits
#pragma unroll
  for (int i = 0; i < kQRows; ++i) {
    const int n = wave + i * kW;
    uint32_t outw[E / 2];
    if (n >= G) {                                  // padding row of the MFMA (wave-uniform)
#pragma unroll
      for (int k = 0; k < E / 2; ++k) outw[k] = 0u;
    } else if constexpr (QM == QM_BF16) {
#pragma unroll
      for (int k = 0; k < E / 2; ++k) outw[k] = raw.w[i][k];
    } else {
      float x[E];
#pragma unroll
      for (int k = 0; k < E / 2; ++k) {
        x[2 * k] = __builtin_bit_cast(float, raw.w[i][k] << 16);
        x[2 * k + 1] = __builtin_bit_cast(float, raw.w[i][k] & 0xFFFF0000u);
      }
      int lane0 = 0, nl = 64;
      if constexpr (QM == QM_GROUPED) {
        // gather q[perm[j]]: element perm % E of lane perm / E
        float y[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int src = (int)((raw.perm[e >> 1] >> (16 * (e & 1))) & (D - 1));
          float v = 0.f;
#pragma unroll
          for (int k = 0; k < E; ++k) {
            const float o = __shfl(x[k], src / E);
            v = (src % E == k) ? o : v;
          }
          y[e] = v;
        }
#pragma unroll
        for (int e = 0; e < E; ++e) x[e] = y[e];
        lane0 = lane < 16 ? 0 : (lane < 48 ? 16 : 48);
        nl = (lane >= 16 && lane < 48) ? 32 : 16;
      }
#pragma unroll
      for (int e = 0; e < E; ++e)
        if ((raw.sw >> e) & 1u) x[e] = -x[e];
      if constexpr (QM == QM_GROUPED) wave_fwht<D>(x, lane, lane0, nl);
      else wave_fwht_rows<D>(x, lane);
      const float rs = p.scale_log2 / sqrtf((float)(E * nl));
#pragma unroll
      for (int k = 0; k < E / 2; ++k) {
        half2_t hv = {(_Float16)(x[2 * k] * rs), (_Float16)(x[2 * k + 1] * rs)};
        outw[k] = n < G ? __builtin_bit_cast(uint32_t, hv) : 0u;
      }
    }
    if constexpr (E == 4) *(uint2 *)(qs + n * RS + E * lane) = make_uint2(outw[0], outw[1]);
    else *(uint32_t *)(qs + n * RS + E * lane) = outw[0];
  }
  __syncthreads();
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    const int col = QM == QM_GROUPED ? 32 * kk + 8 * (lane >> 4) : (lane >> 4) * DL + 8 * kk;
    const uint4 v = *(const uint4 *)(qs + (lane & 15) * RS + col);
    qb[4 * kk] = v.x; qb[4 * kk + 1] = v.y; qb[4 * kk + 2] = v.z; qb[4 * kk + 3] = v.w;
  }
}

// Issue balance between the waves of a workgroup. Every wave owns the same
// share of a unit's tiles, but a SIMD's arbiter favours its oldest wave, so
// the two waves that share a SIMD would finish far apart and the SIMD would
// run one wave alone at the end of the unit. After each step a wave
// publishes its progress in LDS and runs at low issue priority while it is
// ahead of the workgroup mean, at raised priority otherwise. Only the issue
// order changes: every wave still computes its own tiles in the same order,
// so results stay bitwise reproducible.
__device__ __forceinline__ void balance_step(int *prog, int wave, int done) {
  int sum = 0;
#pragma unroll
  for (int k = 0; k < kW; k += 4) {
    const int4 a = *(const int4 *)(prog + k);
    sum += a.x + a.y + a.z + a.w;
  }
  prog[wave] = done;
  sum = __builtin_amdgcn_readfirstlane(sum);
  if (done * kW > sum) __builtin_amdgcn_s_setprio(0);
  else __builtin_amdgcn_s_setprio(1);
}

// One work unit (item, KV head) of format FMT: the first tile of this wave's
// pages (pages wave, wave + kW, ...) is requested with the query, the rest of
// the ring's DEPTH tiles right after the query prologue (a smaller burst when
// every workgroup starts at once lets the queries return sooner); then the
// ring streams the rest: slot j is computed, then refilled with the tile
// DEPTH ahead, so DEPTH - 1 tiles of loads are in flight during compute. Tiles past the wave's list get an
// empty buffer range: their loads are issued (every load is unconditional,
// so the in-order load counter stays exact for the waits) but return zeros
// without touching memory. my_pages and the loop counters are wave-uniform.
template <int FMT, int D, int DEPTH, int T, bool MASS, bool CAUSAL>
__device__ __forceinline__ void scan_unit(const DecodeParams &p, const ItemHeader &h, int g, int my_pages,
                                          int2 my_ent, float *smem, int *prog, float4_t (&acc)[D / 16],
                                          float &m_run, float &l_run) {
  const int lane = fresh_lane();
  constexpr int P = 16 * T;
  const int n_tiles = my_pages * T;
  const uint8_t *pool = p.pool[FMT] + (int64_t)g * p.head_bytes[FMT];
  const int64_t page_bytes = p.page_bytes[FMT];
  const int hb = (int)p.head_bytes[FMT];
  const int N = h.seq;
  // An entry whose id is outside this cache's pool (the plan may have been
  // built against a larger pool) is masked: its loads get an empty range and
  // its logical page is moved past N_b, so every token of it is masked.
  const bool ent_bad = lane < my_pages && (my_ent.y < 0 || (int64_t)my_ent.y >= p.pool_pages[FMT]);
  const uint64_t bad_mask = __builtin_amdgcn_ballot_w64(ent_bad);
  const int2 ent = ent_bad ? make_int2(N / P + 1, -1) : my_ent;
  if (bad_mask != 0 && lane == 0 && p.counters)
    atomicAdd(&p.counters->invalid_entries, (unsigned long long)__builtin_popcountll(bad_mask));
  auto rsrc_of = [&](int tt) {
    const bool live = tt < n_tiles;
    const int pid = __builtin_amdgcn_readlane(ent.y, live ? tt / T : 0);
    const bool ok = live && pid >= 0;
    return block_rsrc(pool + (int64_t)(ok ? pid : 0) * page_bytes, ok ? hb : 0);
  };
  constexpr int QM = FMT == FMT_FP8 ? QM_BF16 : (FMT == FMT_TQK ? QM_GROUPED : QM_ROT);
  const QueryRaw<D> qraw = fetch_query<D, QM, CAUSAL>(p, h.b, g);
  __builtin_amdgcn_sched_barrier(kKeepVmemOrder);
  Tile<FMT, D> buf[DEPTH];
  load_tile<FMT, D>(buf[0], rsrc_of(0), 0, T, P, lane);
  __builtin_amdgcn_sched_barrier(kKeepVmemOrder);
  uint32_t qb[D / 8];
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  prog[wave] = 0;                                  // published before the query barrier
  int done = 0;
  finish_query<D, QM>(p, qraw, smem, qb);
  __builtin_amdgcn_sched_barrier(kKeepVmemOrder);
#pragma unroll
  for (int j = 1; j < DEPTH; ++j) {
    load_tile<FMT, D>(buf[j], rsrc_of(j), j % T, T, P, lane);
    __builtin_amdgcn_sched_barrier(kKeepVmemOrder);
  }
  auto nvalid_of = [&](int tt) {
    const int lp = __builtin_amdgcn_readlane(ent.x, (tt < n_tiles ? tt : 0) / T);
    return tt < n_tiles ? N - (lp * P + (tt % T) * 16) : 0;
  };
  // tile log-mass (scored calls): staged in LDS, [wave][local tile][head],
  // the head's lane writing element (tt, lane); the logical page of each of
  // the unit's entries goes next to it for the write-out after the scan
  float *mrow = nullptr;
  if constexpr (MASS) {
    const int s_max = (int)((p.packet_stride - (int64_t)sizeof(ItemHeader)) / 8);
    const int cap = ((s_max + kW - 1) / kW) * T;
    float *stage = smem + p.mass_lds_off;
    const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    if (lane < p.G) mrow = stage + (int64_t)wv * cap * p.G + lane;
    int *lps = (int *)(stage + (int64_t)kW * cap * p.G);
    if (lane < my_pages) lps[wv + kW * lane] = my_ent.x;
  }
  // chunked prefill: row c Gr + nn of the lane's column sees C - 1 - c tokens
  // fewer at the end of the list than the chunk's last token (0 in decode)
  int dn = 0;
  if constexpr (CAUSAL) {
    const int row = lane & 15;
    dn = row < p.G ? p.chunk - 1 - row / p.Gr : 0;
  }
  auto mi_of = [&](int tt) { return tt < n_tiles ? tt * p.G : -1; };
  uint8_t *wl = nullptr;                          // fractional-level scans: the wave's LDS area
  if constexpr (is_tqf(FMT)) wl = (uint8_t *)smem + query_stage_bytes(D) + wave * tqf_wave_bytes(D);
  if constexpr (FMT == FMT_FP8 || is_tqf(FMT)) {
    // steady state: every slot holds a tile of the list (no per-tile branch,
    // so tile t's tail and tile t+1's decode can interleave)
    int t0 = 0;
    for (; t0 + DEPTH <= n_tiles; t0 += DEPTH) {
#pragma unroll
      for (int j = 0; j < DEPTH; ++j) {
        const int tt = t0 + j;
        process_tile<FMT, D, MASS>(buf[j], nvalid_of(tt), qb, p.scale_log2, acc, m_run, l_run, lane, mrow, mi_of(tt), dn,
                                   wl);
        balance_step(prog, wave, ++done);
        __builtin_amdgcn_sched_barrier(kKeepVmemOrder);
        load_tile<FMT, D>(buf[j], rsrc_of(tt + DEPTH), (tt + DEPTH) % T, T, P, lane);
        __builtin_amdgcn_sched_barrier(kKeepVmemOrder);
      }
    }
    // tail: fewer than DEPTH tiles left, already loaded
#pragma unroll
    for (int j = 0; j < DEPTH; ++j)
      if (t0 + j < n_tiles)
        process_tile<FMT, D, MASS>(buf[j], nvalid_of(t0 + j), qb, p.scale_log2, acc, m_run, l_run, lane, mrow,
                                   mi_of(t0 + j), dn, wl);
  } else {
    // TQ tiles go in pairs: slots (0, 1) and (2, 3) hold two pairs; a pair
    // is computed, then refilled with the pair two ahead. The second tile of
    // an odd list's last pair is an empty-range tile with nvalid 0.
    static_assert(DEPTH == 4, "two pairs in flight");
    const int n_pairs = (n_tiles + 1) / 2;
    // only the request's last page can be partial, and it is the last page
    // of whichever wave holds it: every earlier tile of the list is full
    int full_tiles = n_tiles;
    if constexpr (CAUSAL) {
      // a tile is unmasked only if every row sees all of it: its tokens end
      // at least C - 1 before the chunk's last token
      while (full_tiles > 0 && nvalid_of(full_tiles - 1) - (p.chunk - 1) < 16) --full_tiles;
    } else {
      if (n_tiles > 0 && nvalid_of(n_tiles - 1) < 16) full_tiles = n_tiles - 1;
      if (T == 2 && n_tiles >= 2 && nvalid_of(n_tiles - 2) < 16) full_tiles = n_tiles - 2;
    }
    if (bad_mask != 0) full_tiles = 0;   // masked entries anywhere: every pair takes the masked path
    const int full_pairs = full_tiles / 2;
    // steady state (no masking), then the remaining pairs with masks
    int q0 = 0;
    for (; q0 + 2 <= full_pairs; q0 += 2) {
      const int ta = 2 * q0, tb = 2 * q0 + 2;
      process_pair<FMT, D, false, MASS>(buf[0], buf[1], 16, 16, qb, acc, m_run, l_run, lane, mrow, mi_of(ta),
                                        mi_of(ta + 1));
      balance_step(prog, wave, ++done);
      __builtin_amdgcn_sched_barrier(kKeepVmemOrder);
      load_tile<FMT, D>(buf[0], rsrc_of(ta + 4), (ta + 4) % T, T, P, lane);
      load_tile<FMT, D>(buf[1], rsrc_of(ta + 5), (ta + 5) % T, T, P, lane);
      __builtin_amdgcn_sched_barrier(kKeepVmemOrder);
      process_pair<FMT, D, false, MASS>(buf[2], buf[3], 16, 16, qb, acc, m_run, l_run, lane, mrow, mi_of(tb),
                                        mi_of(tb + 1));
      balance_step(prog, wave, ++done);
      __builtin_amdgcn_sched_barrier(kKeepVmemOrder);
      load_tile<FMT, D>(buf[2], rsrc_of(tb + 4), (tb + 4) % T, T, P, lane);
      load_tile<FMT, D>(buf[3], rsrc_of(tb + 5), (tb + 5) % T, T, P, lane);
      __builtin_amdgcn_sched_barrier(kKeepVmemOrder);
    }
    for (; q0 + 2 <= n_pairs; q0 += 2) {
      const int ta = 2 * q0, tb = 2 * q0 + 2;
      process_pair<FMT, D, true, MASS>(buf[0], buf[1], nvalid_of(ta), nvalid_of(ta + 1), qb, acc, m_run, l_run, lane,
                                       mrow, mi_of(ta), mi_of(ta + 1), dn);
      balance_step(prog, wave, ++done);
      __builtin_amdgcn_sched_barrier(kKeepVmemOrder);
      load_tile<FMT, D>(buf[0], rsrc_of(ta + 4), (ta + 4) % T, T, P, lane);
      load_tile<FMT, D>(buf[1], rsrc_of(ta + 5), (ta + 5) % T, T, P, lane);
      __builtin_amdgcn_sched_barrier(kKeepVmemOrder);
      process_pair<FMT, D, true, MASS>(buf[2], buf[3], nvalid_of(tb), nvalid_of(tb + 1), qb, acc, m_run, l_run, lane,
                                       mrow, mi_of(tb), mi_of(tb + 1), dn);
      balance_step(prog, wave, ++done);
      __builtin_amdgcn_sched_barrier(kKeepVmemOrder);
      load_tile<FMT, D>(buf[2], rsrc_of(tb + 4), (tb + 4) % T, T, P, lane);
      load_tile<FMT, D>(buf[3], rsrc_of(tb + 5), (tb + 5) % T, T, P, lane);
      __builtin_amdgcn_sched_barrier(kKeepVmemOrder);
    }
    if (q0 < n_pairs)
      process_pair<FMT, D, true, MASS>(buf[0], buf[1], nvalid_of(2 * q0), nvalid_of(2 * q0 + 1), qb, acc, m_run, l_run,
                                       lane, mrow, mi_of(2 * q0), mi_of(2 * q0 + 1), dn);
  }
  __builtin_amdgcn_s_setprio(0);
}

// Persistent decode: workgroup w takes unit w first, then the next unit of
// the plan's dispenser (grid + a ticket) whenever it finishes one, so the
// CUs stay busy whatever the mix of item sizes; unit u = item * Hkv + g. A
// workgroup stops at the first item slot that holds no item. Each unit's
// result depends only on the unit, so the output does not depend on which
// workgroup ran it.
template <int D, bool MASS, bool CAUSAL>
__global__ __launch_bounds__(kDecodeThreads) __attribute__((amdgpu_waves_per_eu(2))) void decode_kernel(DecodeParams p) {
  constexpr int NGV = D / 16;
  // 16-byte aligned: the static variables come first, and the b64 / b128
  // LDS accesses of the query staging and the merge need the alignment
  extern __shared__ __align__(16) float smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = p.G;
  const int s_max = (int)((p.packet_stride - (int64_t)sizeof(ItemHeader)) / 8);
  __shared__ uint32_t s_next;
  __shared__ __align__(16) int s_prog[kW];                 // per-wave progress (issue balance)
  // The plan header, the item count and the first unit's packet are read
  // together, one round trip: the grid never exceeds the unit slots of this
  // geometry's plan (whose size the host checked), so that packet exists
  // whatever the header says.
  const int4 hdr_a = *(const int4 *)p.plan_hdr;
  const int4 hdr_c = *((const int4 *)p.plan_hdr + 1);
  const uint32_t n_items_raw = p.ticket[1];
  PacketRaw pkt = load_packet(p, (int64_t)blockIdx.x / p.Hkv, wave, lane, s_max);
  if (!header_matches(p, hdr_a, hdr_c)) return;       // the merge kernel reports it
  const uint32_t n_items_plan = (uint32_t)__builtin_amdgcn_readfirstlane((int)n_items_raw);
  const int64_t n_units = (int64_t)(n_items_plan < (uint64_t)p.n_slots ? n_items_plan : p.n_slots) * p.Hkv;
  for (int64_t u = blockIdx.x; u < n_units;) {
    const int64_t it = u / p.Hkv;
    const int g = (int)(u % p.Hkv);
    const int4 h0 = pkt.h0, h1 = pkt.h1;
    const int2 my_ent = pkt.ent;
    ItemHeader h;
    h.b = __builtin_amdgcn_readfirstlane(h0.x);
    h.fmt = __builtin_amdgcn_readfirstlane(h0.y);
    h.cnt = __builtin_amdgcn_readfirstlane(h0.z);
    h.seq = __builtin_amdgcn_readfirstlane(h0.w);
    h.n_items = __builtin_amdgcn_readfirstlane(h1.x);
    h.item_base = __builtin_amdgcn_readfirstlane(h1.y);
    h.n8 = __builtin_amdgcn_readfirstlane(h1.z);
    h.valid = __builtin_amdgcn_readfirstlane(h1.w);
    if (!h.valid || h.b < 0 || h.b >= p.B) break;
    h.cnt = h.cnt < 0 ? 0 : (h.cnt > s_max ? s_max : h.cnt);
    const int my_pages = h.cnt > wave ? (h.cnt - wave + kW - 1) / kW : 0;

    float4_t acc[NGV];
#pragma unroll
    for (int gv = 0; gv < NGV; ++gv) acc[gv] = (float4_t){0.f, 0.f, 0.f, 0.f};
    float m_run = kNegInf, l_run = 0.f;
    if (p.P == 16) {
      switch (h.fmt) {
        case FMT_FP8: scan_unit<FMT_FP8, D, 2, 1, MASS, CAUSAL>(p, h, g, my_pages, my_ent, smem, s_prog, acc, m_run, l_run); break;
        case FMT_TQ3: scan_unit<FMT_TQ3, D, 4, 1, MASS, CAUSAL>(p, h, g, my_pages, my_ent, smem, s_prog, acc, m_run, l_run); break;
        case FMT_TQ2: scan_unit<FMT_TQ2, D, 4, 1, MASS, CAUSAL>(p, h, g, my_pages, my_ent, smem, s_prog, acc, m_run, l_run); break;
        case FMT_TQK:
          if constexpr (D == 128) scan_unit<FMT_TQK, D, 4, 1, MASS, CAUSAL>(p, h, g, my_pages, my_ent, smem, s_prog, acc, m_run, l_run);
          break;
        case FMT_TQF5: scan_unit<FMT_TQF5, D, 2, 1, MASS, CAUSAL>(p, h, g, my_pages, my_ent, smem, s_prog, acc, m_run, l_run); break;
        case FMT_TQF6: scan_unit<FMT_TQF6, D, 2, 1, MASS, CAUSAL>(p, h, g, my_pages, my_ent, smem, s_prog, acc, m_run, l_run); break;
        default: break;
      }
    } else {
      switch (h.fmt) {
        case FMT_FP8: scan_unit<FMT_FP8, D, 2, 2, MASS, CAUSAL>(p, h, g, my_pages, my_ent, smem, s_prog, acc, m_run, l_run); break;
        case FMT_TQ3: scan_unit<FMT_TQ3, D, 4, 2, MASS, CAUSAL>(p, h, g, my_pages, my_ent, smem, s_prog, acc, m_run, l_run); break;
        case FMT_TQ2: scan_unit<FMT_TQ2, D, 4, 2, MASS, CAUSAL>(p, h, g, my_pages, my_ent, smem, s_prog, acc, m_run, l_run); break;
        case FMT_TQK:
          if constexpr (D == 128) scan_unit<FMT_TQK, D, 4, 2, MASS, CAUSAL>(p, h, g, my_pages, my_ent, smem, s_prog, acc, m_run, l_run);
          break;
        case FMT_TQF5: scan_unit<FMT_TQF5, D, 2, 2, MASS, CAUSAL>(p, h, g, my_pages, my_ent, smem, s_prog, acc, m_run, l_run); break;
        case FMT_TQF6: scan_unit<FMT_TQF6, D, 2, 2, MASS, CAUSAL>(p, h, g, my_pages, my_ent, smem, s_prog, acc, m_run, l_run); break;
        default: break;
      }
    }
    // the next unit is requested now and read after the workgroup merge: an
    // increment that returns the old ticket is not turned into a wave-wide
    // add whose result is waited for at once (as a single-lane fetch_add
    // is), so its round trip overlaps the merge
    uint32_t next = 0x7FFFFFFFu;
    const bool dispense = n_units > (int64_t)gridDim.x;   // some workgroup runs a second unit
    if (dispense) {
      next = 0u;
      if (tid == 0) next = __builtin_amdgcn_atomic_inc32(p.ticket, 0xFFFFFFFFu, __ATOMIC_RELAXED, "agent");
    }
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);

    // ---- merge of the waves in LDS ----
    // A lane holds head n = lane % 16 and dims 16 gv + 4 (lane / 16) + r.
    // Every wave stores its (m, l) per head and its unscaled rows; wave v
    // then merges head v over the waves: M = max m_w, L = sum l_w e^(m_w -
    // M), O_bar[d] = sum_w (e^(m_w - M) / L) acc_w[d], holding dims E lane ..
    // E lane + E - 1 (E = D / 64). A unit of a TQ format turns its row back
    // from rotated V space here, R_V^T y = s_V * FWHT(y) / sqrt(D) (the
    // rotation is linear, so rotating each partial before the merge equals
    // rotating the merged result), and every partial row leaves in natural
    // space. The merge area lies past the query staging; the scan's other
    // LDS (fractional-level areas, the tile log-mass stage) is free only once
    // every wave is done.
    {
      constexpr int DP = D + 4;                           // padded row (floats)
      float2 *mls = (float2 *)(smem + query_stage_bytes(D) / 4);   // [kW][16]
      float *mo = smem + query_stage_bytes(D) / 4 + kW * 16 * 2;    // [kW][G][DP]
      const int n = lane & 15, grp = lane >> 4;
      // partial rows of q-head hq sit at [(b Hq + hq) MI + local item]: the
      // final merge of a head reads one contiguous run of rows
      const int64_t row0 = ((int64_t)h.b * p.Hq + (int64_t)g * G) * p.mi + (it - h.item_base);
      if (MASS || h.fmt == FMT_TQF5 || h.fmt == FMT_TQF6) __syncthreads();
      if constexpr (MASS) {
        // the unit's staged tile log-masses, one contiguous run per head and
        // format run (entry k of the unit: wave k % kW, its (k / kW)-th page)
        const int T = p.P / 16;
        const int cap = ((s_max + kW - 1) / kW) * T;
        const float *stage = smem + p.mass_lds_off;
        const int *lps = (const int *)(stage + (int64_t)kW * cap * G);
        const int n_t = h.cnt * T;
        float *rows = p.tile_lmass + ((int64_t)h.b * p.Hq + (int64_t)g * G) * p.tlm_stride;
        for (int e = tid; e < G * n_t; e += kDecodeThreads) {
          const int hn = e / n_t, r = e - hn * n_t;
          const int k = r / T, t = r - k * T;
          rows[(int64_t)hn * p.tlm_stride + (int64_t)lps[k] * T + t] =
              stage[((int64_t)(k % kW) * cap + (k / kW) * T + t) * G + hn];
        }
      }
      if (lane < 16) mls[wave * 16 + n] = make_float2(m_run, l_run);
      if (n < G) {
#pragma unroll
        for (int gv = 0; gv < NGV; ++gv)
          *(float4 *)(mo + (wave * G + n) * DP + 16 * gv + 4 * grp) =
              make_float4(acc[gv][0], acc[gv][1], acc[gv][2], acc[gv][3]);
      }
      __syncthreads();
      constexpr int E = D / 64;
      const bool rotated = h.fmt != FMT_FP8;         // TQ caches always carry their signs
      const uint32_t sv = rotated ? p.signs[((int64_t)g * 2 + 1) * (D / 32) + (E * lane) / 32] >> ((E * lane) & 31) : 0u;
      for (int ne = wave; ne < G; ne += kW) {
        float2 st[kW];
#pragma unroll
        for (int w = 0; w < kW; ++w) st[w] = mls[w * 16 + ne];
        float M = kNegInf;
#pragma unroll
        for (int w = 0; w < kW; ++w) M = st[w].y > 0.f ? fmaxf(M, st[w].x) : M;
        float L = 0.f, wt[kW];
#pragma unroll
        for (int w = 0; w < kW; ++w) {
          wt[w] = st[w].y > 0.f ? fast_exp2(st[w].x - M) : 0.f;
          L += st[w].y * wt[w];
        }
        const float inv = L > 0.f ? 1.f / L : 0.f;
        float x[E];
#pragma unroll
        for (int e = 0; e < E; ++e) x[e] = 0.f;
#pragma unroll
        for (int w = 0; w < kW; ++w) {
          const float ww = wt[w] * inv;
          const float *src = mo + (w * G + ne) * DP + E * lane;
          if constexpr (E == 4) {
            const float4 v = *(const float4 *)src;
            x[0] += v.x * ww; x[1] += v.y * ww; x[2] += v.z * ww; x[3] += v.w * ww;
          } else {
            const float2 v = *(const float2 *)src;
            x[0] += v.x * ww; x[1] += v.y * ww;
          }
        }
        if (rotated) {
          wave_fwht_rows<D>(x, lane);
          constexpr float rs = D == 256 ? 0.0625f : 0.08838834764831845f;   // 1 / sqrt(D)
#pragma unroll
          for (int e = 0; e < E; ++e) x[e] = ((sv >> e) & 1u) ? -(x[e] * rs) : x[e] * rs;
        }
        float *dst = p.part_o + (row0 + (int64_t)ne * p.mi) * D + E * lane;
        if constexpr (E == 4) *(float4 *)dst = make_float4(x[0], x[1], x[2], x[3]);
        else *(float2 *)dst = make_float2(x[0], x[1]);
        if (lane == 0) *(float2 *)(p.part_ml + (row0 + (int64_t)ne * p.mi) * 2) = make_float2(L > 0.f ? M : kNegInf, L);
      }
      __syncthreads();                                    // LDS free for the next unit
    }
    if (tid == 0 && p.counters && h.cnt > 0) {
      unsigned long long *c = h.fmt == FMT_FP8 ? &p.counters->pages_fp8
                            : h.fmt == FMT_TQ3 ? &p.counters->pages_tq3
                            : h.fmt == FMT_TQ2 ? &p.counters->pages_tq2
                            : h.fmt == FMT_TQK ? &p.counters->pages_tqk
                            : h.fmt == FMT_TQF5 ? &p.counters->pages_tqf5 : &p.counters->pages_tqf6;
      atomicAdd(c, (unsigned long long)h.cnt);
    }
    if (tid == 0) s_next = next;
    __syncthreads();
    u = (int64_t)gridDim.x + s_next;
    if (u >= n_units) break;
    pkt = load_packet(p, u / p.Hkv, wave, lane, s_max);
  }
}

// Combine two (m, l) partial statistics (log2 units); an empty one has l = 0.
__device__ __forceinline__ void ml_combine(float &m, float &l, float m2, float l2) {
  if (l2 <= 0.f) return;
  if (l <= 0.f) { m = m2; l = l2; return; }
  const float M = fmaxf(m, m2);
  l = l * fast_exp2(m - M) + l2 * fast_exp2(m2 - M);
  m = M;
}

// Wave-wide maximum and sum by butterflies: every lane gets the same value
// (both lanes of a pair add the same two operands).
__device__ __forceinline__ float wave_max(float x, int lane) {
  x = fmaxf(x, lane_xor<1>(x, lane));
  x = fmaxf(x, lane_xor<2>(x, lane));
  x = fmaxf(x, lane_xor<4>(x, lane));
  x = fmaxf(x, lane_xor<8>(x, lane));
  x = fmaxf(x, lane_xor<16>(x, lane));
  return fmaxf(x, lane_xor<32>(x, lane));
}
__device__ __forceinline__ float wave_sum(float x, int lane) {
  x += lane_xor<1>(x, lane);
  x += lane_xor<2>(x, lane);
  x += lane_xor<4>(x, lane);
  x += lane_xor<8>(x, lane);
  x += lane_xor<16>(x, lane);
  return x + lane_xor<32>(x, lane);
}

constexpr int kMergeChunk = 32;   // partial rows one thread has in flight
constexpr int kMassRegs = 16;     // tile log-masses per thread held in registers (scored merge)

// Merge of every partial of one (request, q-head) (Minima-KV Eq. 11-13):
// thread j owns dim j. Every partial row is in natural space (a TQ unit
// rotates its rows back before it writes them), so the merge is one
// softmax-weighted sum. Every wave loads the (m, l) of the first 64 items
// (item i in lane i) next to its first chunk of partial rows and derives the
// maximum, the sum and the item weights itself with lane butterflies, so no
// LDS exchange or barrier precedes the accumulation; a weight reaches the
// whole wave with v_readlane.
template <int D, bool MASS, bool APPEND>
__global__ __launch_bounds__(D) void merge_kernel(DecodeParams p) {
  __shared__ float s_x[D];
  __shared__ float s_red[8];
  const int j = threadIdx.x, lane = j & 63;
  const int b = blockIdx.x / p.Hq, hq = blockIdx.x % p.Hq;
  if (blockIdx.x == 0 && j == 0) *p.ticket = 0u;     // the dispenser is free again for the next call
  const int g = hq / p.G;
  // The plan header and the request's item count are read through the
  // scalar cache (constant memory: the plan was written before this launch
  // and nothing writes it during it). Vector loads would add to the partial
  // rows' loads below, and past about 35 vector loads in flight a wave's
  // next load waits for one to return.
  typedef __attribute__((address_space(4))) const int32_t const_i32;
  const const_i32 *hw = (const const_i32 *)p.plan_hdr;
  const int4 hdr_a = make_int4(hw[0], hw[1], hw[2], hw[3]);
  const int4 hdr_c = make_int4(hw[4], hw[5], hw[6], hw[7]);
  if (!header_matches(p, hdr_a, hdr_c)) {
    // a plan built for another geometry: the scan did nothing; poison the
    // outputs and count the call once
    const int hrem = hq - g * p.G, hc = hrem / p.Gr;
    const int64_t orow = ((int64_t)b * p.chunk + hc) * p.Hq_r + (int64_t)g * p.Gr + (hrem - hc * p.Gr);
    p.out[orow * D + j] = __builtin_nanf("");
    if (j == 0 && p.lse) p.lse[orow] = __builtin_nanf("");
    if (blockIdx.x == 0 && j == 0 && p.counters) atomicAdd(&p.counters->invalid_entries, 1ull);
    return;
  }
  // the head's partial rows sit at [(b Hq + hq) MI, (b Hq + hq + 1) MI):
  // statistics first, then the first chunk of rows, then the item count
  // (loads past MI are skipped; values past the count are discarded)
  const int64_t row0 = ((int64_t)b * p.Hq + hq) * p.mi;
  const float *ml = p.part_ml + row0 * 2;
  // the head's MI rows and statistics as range-checked buffers: a read past
  // them returns zero, so every load below is issued without a branch
  const __amdgpu_buffer_rsrc_t rrows = block_rsrc((const uint8_t *)(p.part_o + row0 * D), (int)(p.mi * D * 4));
  const __amdgpu_buffer_rsrc_t rstat = block_rsrc((const uint8_t *)ml, (int)(p.mi * 8));
  // fused append: the new token's K and V coordinate j and the query's, issued
  // first, so the append's arithmetic below waits for them alone (loads
  // return in issue order) while the partial rows are still in flight
  float kx = 0.f, vx = 0.f, qj = 0.f;
  if constexpr (APPEND) {
    const int64_t kv = ((int64_t)b * p.Hkv + hq / p.G) * 2 * D;
    if (p.new_kv_bf16) {
      const uint16_t *src = (const uint16_t *)p.new_kv;
      kx = __builtin_bit_cast(float, (uint32_t)src[kv + j] << 16);
      vx = __builtin_bit_cast(float, (uint32_t)src[kv + D + j] << 16);
    } else {
      const float *src = (const float *)p.new_kv;
      kx = src[kv + j];
      vx = src[kv + D + j];
    }
    qj = __builtin_bit_cast(float, (uint32_t)p.q[((int64_t)b * p.Hq + hq) * D + j] << 16);
  }
  float2 mine;
  {
    const auto st = __builtin_amdgcn_raw_buffer_load_b64(rstat, 8 * lane, 0, 0);
    mine = make_float2(f32_bits((uint32_t)st[0]), f32_bits((uint32_t)st[1]));
  }
  float v[kMergeChunk];
#pragma unroll
  for (int u = 0; u < kMergeChunk; ++u)
    v[u] = f32_bits(__builtin_amdgcn_raw_buffer_load_b32(rrows, 4 * (u * D + j), 0, 0));
  // scored call: the head's first tile log-masses, in flight with the partials
  float mv[MASS ? kMassRegs : 1];
  float *mrow = nullptr;
  if constexpr (MASS) {
    mrow = p.tile_lmass + ((int64_t)b * p.Hq + hq) * p.tlm_stride;
#pragma unroll
    for (int u = 0; u < kMassRegs; ++u) {
      const int64_t t = j + (int64_t)u * D;
      mv[u] = t < p.tlm_stride ? mrow[t] : kNegInf;
    }
  }
  // fused append (Minima-KV algorithm 1 "Append" in the decode launch): the
  // step's new token is FP8-encoded exactly as kv_encode_fp8 does, joins the
  // softmax as one more partition (m = its score, l = 1, O = its decoded V)
  // and is written to its FP8 slot by the first q-head of each group
  float s_new = kNegInf, vhat = 0.f;
  if constexpr (APPEND) {
    float ak = wave_max(fabsf(kx), lane), av = wave_max(fabsf(vx), lane);
    if (lane == 0) {
      s_red[j >> 6] = ak;
      s_red[4 + (j >> 6)] = av;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < D / 64; ++w) {
      ak = fmaxf(ak, s_red[w]);
      av = fmaxf(av, s_red[4 + w]);
    }
    uint32_t ek = 0, ev = 0;
    float sk = 0.f, svl = 0.f;
    if (ak > 0.f) {
      const float inv = 448.0f / ak;
      ek = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(kx * inv, 0.f, 0, false) & 255u;
      sk = ak / 448.0f;
    }
    if (av > 0.f) {
      const float inv = 448.0f / av;
      ev = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(vx * inv, 0.f, 0, false) & 255u;
      svl = av / 448.0f;
    }
    const float khat = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(ek, 1.0f, false)[0] * sk;
    vhat = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(ev, 1.0f, false)[0] * svl;
    const float dot = wave_sum(qj * khat, lane);
    __syncthreads();                                     // s_red is read above
    if (lane == 0) s_red[j >> 6] = dot;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < D / 64; ++w) tot += s_red[w];
    s_new = tot * p.scale_log2;
    if (hq % p.G == 0) {
      const int pid = p.new_page[b], slot = p.new_slot[b];
      if (pid >= 0 && pid < p.pool_pages[FMT_FP8] && slot >= 0 && slot < p.P) {
        constexpr int DL = D / 4;
        const int T = p.P / 16, tau = slot / 16, t16 = slot % 16;
        uint8_t *head = p.fp8_pool_w + (int64_t)pid * p.page_bytes[FMT_FP8] + (int64_t)g * p.head_bytes[FMT_FP8];
        const int lk = t16 + 16 * (j / DL), ik = j % DL;
        head[(int64_t)tau * 16 * D + ((ik / 16) * 64 + lk) * 16 + ik % 16] = (uint8_t)ek;
        const int lv = j % 16 + 16 * (t16 / 4), iv = 4 * (j / 16) + t16 % 4;
        head[(int64_t)(T + tau) * 16 * D + ((iv / 16) * 64 + lv) * 16 + iv % 16] = (uint8_t)ev;
        if (j == 0) {
          float *sc = (float *)(head + 2LL * p.P * D);
          sc[slot] = sk;
          sc[p.P + slot] = svl;
        }
      } else if (j == 0 && p.counters) {
        atomicAdd(&p.counters->invalid_entries, 1ull);
      }
    }
  }
  const int n_items = ((const const_i32 *)(p.req + b))[1];          // ReqItems::n_items
#pragma unroll
  for (int u = 0; u < kMergeChunk; ++u) v[u] = u < n_items ? v[u] : 0.f;
  // statistics over items lane, lane + 64, ..., then the maxima and sums
  // across the wave (every partial row is in natural space)
  if (lane >= n_items) mine = make_float2(0.f, 0.f);
  float mr = 0.f, lr = 0.f;
  ml_combine(mr, lr, mine.x, mine.y);
  for (int i = lane + 64; i < n_items; i += 64) {
    const float2 x = *(const float2 *)(ml + 2 * i);
    ml_combine(mr, lr, x.x, x.y);
  }
  const float Mr = wave_max(lr > 0.f ? mr : kNegInf, lane);
  const float Lr = wave_sum(lr > 0.f ? lr * fast_exp2(mr - Mr) : 0.f, lane);
  const float inv_r = Lr > 0.f ? 1.f / Lr : 0.f;
  // weight of item lane
  const float w_mine = mine.y > 0.f ? fast_exp2(mine.x - Mr) * mine.y * inv_r : 0.f;
  float acc = 0.f;
  for (int i0 = 0; i0 < n_items; i0 += kMergeChunk) {
    if (i0 > 0) {
#pragma unroll
      for (int u = 0; u < kMergeChunk; ++u)
        v[u] = i0 + u < n_items ? f32_bits(__builtin_amdgcn_raw_buffer_load_b32(rrows, 4 * ((i0 + u) * D + j), 0, 0)) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kMergeChunk; ++u) {
      const int i = i0 + u;
      float w;
      if (i < 64) {
        w = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w_mine), i));
      } else if (i < n_items) {
        const float2 x = *(const float2 *)(ml + 2 * i);
        w = x.y > 0.f ? fast_exp2(x.x - Mr) * x.y * inv_r : 0.f;
      } else {
        w = 0.f;
      }
      acc += w * v[u];
    }
  }
  const float M = fmaxf(Mr, s_new);
  float num = 0.f, L = 0.f;
  if (M != kNegInf) {
    if (Lr > 0.f) {
      const float er = fast_exp2(Mr - M) * Lr;
      L += er;
      num += er * acc;
    }
    if (APPEND && s_new != kNegInf) {
      const float ea = fast_exp2(s_new - M);
      L += ea;
      num += ea * vhat;
    }
  }
  // output row: head g Gr + nn of token c (virtual head hq = g G + c Gr + nn)
  const int hrem = hq - g * p.G, hc = hrem / p.Gr;
  const int64_t orow_out = ((int64_t)b * p.chunk + hc) * p.Hq_r + (int64_t)g * p.Gr + (hrem - hc * p.Gr);
  // without an appended token the result is the merged rows themselves
  p.out[orow_out * D + j] = L > 0.f ? (APPEND ? num / L : acc) : 0.f;
  const float lse_h = L > 0.f ? (M + log2f(L)) * 0.69314718055994531f : kNegInf;
  if (j == 0 && p.lse) p.lse[orow_out] = lse_h;
  if constexpr (MASS) {
    // Scored call: the head's tile log-masses become ln q~ (Minima-KV Eq. 8,
    // then the page-addressable normalization): ln q = lambda - lse, and
    // q~ = q / sum over the request's tiles (tiles not reached hold -inf).
    // The first kMassRegs D tiles were loaded with the partials.
    float part = 0.f;
    if (lse_h != kNegInf) {
#pragma unroll
      for (int u = 0; u < kMassRegs; ++u) part += expf(mv[u] - lse_h);
      // the rest of the row kMassRegs loads at a time (all in flight together)
      for (int64_t t0 = j + (int64_t)kMassRegs * D; t0 < p.tlm_stride; t0 += (int64_t)kMassRegs * D) {
        float w[kMassRegs];
#pragma unroll
        for (int u = 0; u < kMassRegs; ++u) {
          const int64_t t = t0 + (int64_t)u * D;
          w[u] = t < p.tlm_stride ? mrow[t] : kNegInf;
        }
#pragma unroll
        for (int u = 0; u < kMassRegs; ++u) part += expf(w[u] - lse_h);
      }
    }
    part = wave_sum(part, lane);
    __syncthreads();                                     // s_x is free
    if (lane == 0) s_x[j >> 6] = part;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < D / 64; ++w) tot += s_x[w];
    const float shift = tot > 0.f ? lse_h + logf(tot) : kNegInf;
#pragma unroll
    for (int u = 0; u < kMassRegs; ++u) {
      const int64_t t = j + (int64_t)u * D;
      if (t < p.tlm_stride) mrow[t] = shift == kNegInf ? kNegInf : mv[u] - shift;
    }
    for (int64_t t0 = j + (int64_t)kMassRegs * D; t0 < p.tlm_stride; t0 += (int64_t)kMassRegs * D) {
      float w[kMassRegs];
#pragma unroll
      for (int u = 0; u < kMassRegs; ++u) {
        const int64_t t = t0 + (int64_t)u * D;
        w[u] = t < p.tlm_stride ? mrow[t] : kNegInf;
      }
#pragma unroll
      for (int u = 0; u < kMassRegs; ++u) {
        const int64_t t = t0 + (int64_t)u * D;
        if (t < p.tlm_stride) mrow[t] = shift == kNegInf ? kNegInf : w[u] - shift;
      }
    }
  }
}

// Fill of a float buffer (the tile log-mass rows before a scored scan).
__global__ __launch_bounds__(256) void fill_kernel(float *x, int64_t n, float v) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) x[i] = v;
}

// Running page score (Minima-KV Eq. 9), one thread per (request, page): the
// scored call left ln q~ per tile, so r_p = mean over the head set of
// sum_t e^{ln q~_{h,p,t}}, and a_p = beta a_p + (1 - beta) r_p on live pages;
// r_out (if given) is 0 on the others.
__global__ __launch_bounds__(256) void collect_kernel(CollectParams c) {
  const int b = blockIdx.y;
  const int pg = blockIdx.x * 256 + threadIdx.x;
  if (pg >= c.max_pages) return;
  int N = c.seq_lens[b];
  if (N < 0) N = 0;
  int n_pages = (N + c.P - 1) / c.P;
  if (n_pages > c.max_pages) n_pages = c.max_pages;
  const int T = c.P / 16;
  const int64_t o = (int64_t)b * c.max_pages + pg;
  if (pg < n_pages && c.n_heads > 0) {
    // eight heads' loads in flight at a time
    constexpr int KH = 8;
    float r = 0.f;
    for (int k0 = 0; k0 < c.n_heads; k0 += KH) {
      float w[KH][2];
#pragma unroll
      for (int u = 0; u < KH; ++u) {
        const int k = k0 + u < c.n_heads ? k0 + u : k0;
        const float *row = c.tile_lmass + ((int64_t)b * c.Hq + c.heads[k]) * c.tlm_stride + (int64_t)pg * T;
        w[u][0] = k0 + u < c.n_heads ? row[0] : kNegInf;
        w[u][1] = (k0 + u < c.n_heads && T == 2) ? row[1] : kNegInf;
      }
#pragma unroll
      for (int u = 0; u < KH; ++u) r += expf(w[u][0]) + expf(w[u][1]);
    }
    r *= 1.f / (float)c.n_heads;
    c.score[o] = c.beta * c.score[o] + (1.f - c.beta) * r;
    if (c.r_out) c.r_out[o] = r;
  } else if (c.r_out) {
    c.r_out[o] = 0.f;
  }
}

// ------------------------------------------------------------------------
// Packed chunked prefill (Block-GTQ appendix H.5: a prompt chunk attends
// causally to the packed cache with an online softmax, no dense attention
// matrix and no decoded copy of the cache). One workgroup takes 128 query
// rows (row r = token r / G, head r % G of KV head g) of one request; wave w
// owns rows 32 w .. 32 w + 31, one row per lane (lane l and l ^ 32 share
// row l % 32 and split its keys). The request's pages are scanned per
// format, 32 keys a step: each wave decodes one (tile, role) of the step
// into LDS as f16 in the format's own coordinates (K row-major, V
// transposed) with one scale per key (FP8 scale or TQ sigma), and every
// wave then runs S^T = K Q^T and O^T += V^T P^T on 32 x 32 x 16 MFMAs, so a
// decoded tile serves all 128 rows. Keys past N_b or after a row's position
// are masked. TQ pages score against the rotated query and accumulate V in
// rotated space; they come first, then the accumulator is turned back once
// (R_V^T, a register FWHT per row) and the FP8 pages follow in natural space.
// ------------------------------------------------------------------------
typedef float floatx16 __attribute__((ext_vector_type(16)));
constexpr int kPfKeys = 32;                          // keys per step (two 16-token tiles)
constexpr int kPfVS = kPfKeys + 4;                   // V^T row stride (halves): 18 dwords, conflict-free b64 reads
__host__ __device__ constexpr int pf_ks(int D) { return D + 8; }   // K row stride (halves)
// byte offsets inside one step buffer
__host__ __device__ constexpr int pf_vt_off(int D) { return kPfKeys * pf_ks(D) * 2; }
__host__ __device__ constexpr int pf_ksc_off(int D) { return pf_vt_off(D) + D * kPfVS * 2; }   // f32 [3][32]
__host__ __device__ constexpr int pf_vsc_off(int D) { return pf_ksc_off(D) + 3 * kPfKeys * 4; }  // f32 [32]
__host__ __device__ constexpr int pf_kp_off(int D) { return pf_vsc_off(D) + kPfKeys * 4; }      // i32 [32]
__host__ __device__ constexpr int pf_buf_bytes(int D) { return (pf_kp_off(D) + kPfKeys * 4 + 15) & ~15; }
__host__ __device__ constexpr int pf_tqf_wave_bytes(int D) { return 16 * D + 1536; }   // raw rows, then codes
// Workgroup shapes. The TQ3 / TQ2 scans at d = 256 give a 32-row block two
// waves, one per half of the head dim (eight waves a workgroup, two a SIMD):
// each holds half the query fragments and half the accumulator, and the two
// halves of every score are added through LDS (the exchange area:
// [wave][4][64] float4). The other formats at d = 256 (wider raw tiles) keep
// one wave per 32-row block and SIMD, four a workgroup. At d = 128 a
// workgroup has eight waves of 32 rows, two a SIMD: each step's tiles are
// decoded once (by waves 0..3) for 256 rows.
template <int D, int FMT> struct PfShape {
  static constexpr bool SPLIT = D == 256 && (FMT == FMT_TQ3 || FMT == FMT_TQ2);
  static constexpr int WAVES = (SPLIT || D == 128) ? 8 : 4;
  static constexpr int DW = SPLIT ? D / 2 : D;       // head dims one wave holds
  static constexpr int WPE = (D == 256 && !SPLIT) ? 1 : 2;   // waves per SIMD
  static constexpr int RBW = SPLIT ? WAVES / 2 : WAVES;     // 32-row blocks a workgroup
  static constexpr int ROWS = 32 * RBW;                     // query rows a workgroup
};
__host__ __device__ constexpr int pf_sx_off(int D) { return 2 * pf_buf_bytes(D) + 4 * pf_tqf_wave_bytes(D); }
// the scan's areas; before the scan the query staging and after it the
// unrotation staging reuse the start of the allocation
__host__ __device__ constexpr int pf_lds_bytes(int D, bool split, int rbw) {
  const int scan = pf_sx_off(D) + (split ? 8 * 4 * 64 * 16 : 0);
  const int qst = rbw * 32 * pf_ks(D) * 2;
  const int ust = rbw * 16 * (D + 4) * 4;
  const int m = scan > qst ? scan : qst;
  return m > ust ? m : ust;
}
constexpr int kPfNoKey = 0x7FFFFFFF;                 // position of a key no row may see

// Number of entries ent[0 .. n) with logical page <= lp_max (ent ascending in
// logical page): a 64-way search by the wave, two or three rounds.
__device__ __forceinline__ int pf_count_visible(const int2 *ent, int n, int lp_max, int lane) {
  int lo = 0, len = n;
  while (len > 0) {
    const int step = (len + 63) / 64;
    const bool probe = lane * step < len;
    const bool ok = probe && ent[lo + lane * step].x <= lp_max;
    const int cnt = __builtin_popcountll(__builtin_amdgcn_ballot_w64(ok));
    if (cnt == 0) break;
    const int nlo = lo + (cnt - 1) * step + 1;
    const int end = (cnt * step < len) ? lo + cnt * step : lo + len;   // first index known (or assumed) > lp_max
    len = end - nlo;
    lo = nlo;
  }
  return lo;
}

// The query operand of this wave's 32 rows for one format: each row is
// transformed like the decode's (FP8: sm_scale log2 e q; TQ: the K rotation;
// TQK: the grouped rotation) one row at a time across the wave (lane l holds
// dims E l .. E l + E - 1), staged in LDS as f16, then read back as MFMA B
// fragments: lane l, MFMA kk: row l % 32, dims 16 kk + 8 (l / 32) + 0..7.
template <int D, int QM>
__device__ __forceinline__ void pf_query_stage(const PrefillParams &p, int b, int g, int row0, uint16_t *qs,
                                               int lane) {
  constexpr int E = D / 64;
  const int G = p.G, C = p.chunk;
  const uint32_t sw = QM != QM_BF16 ? p.signs[(int64_t)g * 2 * (D / 32) + (E * lane) / 32] >> ((E * lane) & 31) : 0u;
  uint32_t perm[E / 2];
#pragma unroll
  for (int k = 0; k < E / 2; ++k)
    perm[k] = QM == QM_GROUPED ? *(const uint32_t *)(p.tqk_perm + (int64_t)g * D + E * lane + 2 * k) : 0u;
  for (int r = 0; r < 32; ++r) {
    const int row = row0 + r;
    const int c = row / G, n = row - (row / G) * G;
    float x[E];
    if (c < C) {
      const uint16_t *qrow = p.q + (((int64_t)b * C + c) * p.Hq + (int64_t)g * G + n) * D + E * lane;
      uint32_t w[E / 2];
      if constexpr (E == 4) {
        const uint2 v = *(const uint2 *)qrow;
        w[0] = v.x; w[1] = v.y;
      } else {
        w[0] = *(const uint32_t *)qrow;
      }
#pragma unroll
      for (int k = 0; k < E / 2; ++k) {
        x[2 * k] = __builtin_bit_cast(float, w[k] << 16);
        x[2 * k + 1] = __builtin_bit_cast(float, w[k] & 0xFFFF0000u);
      }
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) x[e] = 0.f;
    }
    float rs = p.scale_log2;
    if constexpr (QM != QM_BF16) {
      int lane0 = 0, nl = 64;
      if constexpr (QM == QM_GROUPED) {
        float y[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int src = (int)((perm[e >> 1] >> (16 * (e & 1))) & (D - 1));
          float v = 0.f;
#pragma unroll
          for (int k = 0; k < E; ++k) {
            const float o = __shfl(x[k], src / E);
            v = (src % E == k) ? o : v;
          }
          y[e] = v;
        }
#pragma unroll
        for (int e = 0; e < E; ++e) x[e] = y[e];
        lane0 = lane < 16 ? 0 : (lane < 48 ? 16 : 48);
        nl = (lane >= 16 && lane < 48) ? 32 : 16;
      }
#pragma unroll
      for (int e = 0; e < E; ++e)
        if ((sw >> e) & 1u) x[e] = -x[e];
      if constexpr (QM == QM_GROUPED) wave_fwht<D>(x, lane, lane0, nl);
      else wave_fwht_rows<D>(x, lane);
      rs = p.scale_log2 / sqrtf((float)(E * nl));
    }
#pragma unroll
    for (int k = 0; k < E / 2; ++k) {
      half2_t hv = {(_Float16)(x[2 * k] * rs), (_Float16)(x[2 * k + 1] * rs)};
      *(uint32_t *)(qs + r * pf_ks(D) + E * lane + 2 * k) = __builtin_bit_cast(uint32_t, hv);
    }
  }
}

// The wave's MFMA B fragments from the staged rows: fragment kk (dims
// 16 (kk0 + kk) .. + 15) of lane l is row l % 32, dims + 8 (l / 32) + 0..7.
template <int D, int NKK>
__device__ __forceinline__ void pf_query_frags(const uint16_t *qs, int kk0, int lane, uint32_t (&qb)[4 * NKK]) {
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    const uint4 v = *(const uint4 *)(qs + (lane & 31) * pf_ks(D) + 16 * (kk0 + kk) + 8 * (lane >> 5));
    qb[4 * kk] = v.x; qb[4 * kk + 1] = v.y; qb[4 * kk + 2] = v.z; qb[4 * kk + 3] = v.w;
  }
}

// Raw bytes of one (tile, role) of a format as a wave loads them, and the
// role's per-token scales (lane t < 16: token t; three key sigmas for TQK)
// as stored: f32 bits (FP8) or f16 bits (sigmas). They are converted only
// when the tile is decoded, so nothing waits for a tile load before then.
template <int FMT, int D>
struct PfRaw {
  static constexpr int NW = FMT == FMT_FP8 ? D / 16
                          : (is_tqf(FMT) ? tqf_raw_words<D>() : (FMT == FMT_TQ2 ? D / 64 : 3 * D / 128));
  uint32_t w[NW];
  uint32_t sc[FMT == FMT_TQK ? 3 : 1];
};

template <int FMT>
__device__ __forceinline__ float pf_scale(uint32_t bits) {
  if constexpr (FMT == FMT_FP8) return __builtin_bit_cast(float, bits);
  else return half_bits_to_float(bits);
}

template <int FMT, int D>
__device__ __forceinline__ void pf_load(PfRaw<FMT, D> &r, __amdgpu_buffer_rsrc_t rs, int tau, int T, int P, int role,
                                        int lane) {
  const int t = lane & 15;
  if constexpr (FMT == FMT_FP8) {
    const int base = (role * T + tau) * 16 * D;
#pragma unroll
    for (int i = 0; i < D / 64; ++i) {
      const auto a = __builtin_amdgcn_raw_buffer_load_b128(rs, lane * 16, base + i * 1024, 0);
      r.w[4 * i] = a[0]; r.w[4 * i + 1] = a[1]; r.w[4 * i + 2] = a[2]; r.w[4 * i + 3] = a[3];
    }
    r.sc[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, 4 * t, 2 * P * D + role * 4 * P + 64 * tau, 0);
  } else if constexpr (is_tqf(FMT)) {
    constexpr int RT = 16 * tqf_row_bytes(D, tqf_levels(FMT));
    const int base = (role * T + tau) * RT;
    constexpr int kOff = 1 << 30;
    const int o16 = lane * 16 < (D == 256 ? 1024 : RT) ? lane * 16 : kOff;
    const auto a = __builtin_amdgcn_raw_buffer_load_b128(rs, o16, base, 0);
    r.w[0] = a[0]; r.w[1] = a[1]; r.w[2] = a[2]; r.w[3] = a[3];
    if constexpr (D == 256) {
      const int o8 = lane * 8 < RT - 1024 ? lane * 8 : kOff;
      const auto c = __builtin_amdgcn_raw_buffer_load_b64(rs, o8, base + 1024, 0);
      r.w[4] = c[0]; r.w[5] = c[1];
    }
    const uint32_t h = __builtin_amdgcn_raw_buffer_load_b16(rs, 2 * t, 2 * T * RT + role * 2 * P + 32 * tau, 0);
    r.sc[0] = h;
  } else {
    constexpr int BITS = FMT == FMT_TQ2 ? 2 : 3;
    constexpr int tile_bytes = 16 * D * BITS / 8;
    load_tq_words<PfRaw<FMT, D>::NW>(r.w, rs, (role * T + tau) * tile_bytes, lane);
    const int sig = 2 * T * tile_bytes;
    if constexpr (FMT == FMT_TQK) {
      if (role == 0) {
#pragma unroll
        for (int sgm = 0; sgm < 3; ++sgm)
          r.sc[sgm] = __builtin_amdgcn_raw_buffer_load_b16(rs, 2 * t, sig + sgm * 2 * P + 32 * tau, 0);
      } else {
        r.sc[0] = __builtin_amdgcn_raw_buffer_load_b16(rs, 2 * t, sig + 6 * P + 32 * tau, 0);
        r.sc[1] = r.sc[2] = 0u;
      }
    } else {
      r.sc[0] = __builtin_amdgcn_raw_buffer_load_b16(rs, 2 * t, sig + role * 2 * P + 32 * tau, 0);
    }
  }
}

// One (tile j, role) of a step into the step buffer: K rows kt[16 j + t][dim]
// (TQK: permuted dims), V columns vt[dim][16 j + t], scales, key positions
// (role 0). tw: the wave's fractional-level LDS area.
template <int FMT, int D>
__device__ __forceinline__ void pf_store(const PfRaw<FMT, D> &r, uint8_t *buf, int j, int role, int kpos0, int N,
                                         int lane, uint8_t *tw) {
  constexpr int DL = D / 4;
  uint16_t *kt = (uint16_t *)buf;
  uint16_t *vt = (uint16_t *)(buf + pf_vt_off(D));
  float *ksc = (float *)(buf + pf_ksc_off(D));
  float *vsc = (float *)(buf + pf_vsc_off(D));
  int *kp = (int *)(buf + pf_kp_off(D));
  const int g4 = lane >> 4, t = lane & 15;
  if (role == 0) {
    uint16_t *row = kt + (16 * j + t) * pf_ks(D);
    if constexpr (FMT == FMT_FP8) {
#pragma unroll
      for (int c = 0; c < D / 64; ++c) {
        uint32_t h[8];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          h[2 * u] = fp8x2_to_f16x2(r.w[4 * c + u], false);
          h[2 * u + 1] = fp8x2_to_f16x2(r.w[4 * c + u], true);
        }
        *(uint4 *)(row + g4 * DL + 16 * c) = make_uint4(h[0], h[1], h[2], h[3]);
        *(uint4 *)(row + g4 * DL + 16 * c + 8) = make_uint4(h[4], h[5], h[6], h[7]);
      }
    } else if constexpr (FMT == FMT_TQK) {
#pragma unroll
      for (int m = 0; m < D / 32; ++m) {
        const uint2 a = tqk_decode_group<D>(r.w, 2 * m), c = tqk_decode_group<D>(r.w, 2 * m + 1);
        *(uint4 *)(row + 32 * m + 8 * g4) = make_uint4(a.x, a.y, c.x, c.y);
      }
    } else if constexpr (is_tqf(FMT)) {
      constexpr int L = tqf_levels(FMT);
      uint32_t *raw = (uint32_t *)tw;
      uint8_t *codes = tw + 1536;
      *(uint4 *)(raw + 4 * lane) = make_uint4(r.w[0], r.w[1], r.w[2], r.w[3]);
      if constexpr (D == 256) *(uint2 *)(raw + 256 + 2 * lane) = make_uint2(r.w[4], r.w[5]);
      wave_lds_sync();
      tqf_unpack_tile<D, L, true>(raw, codes, D, lane);
      wave_lds_sync();
#pragma unroll
      for (int m = 0; m < DL / 8; ++m) {
        const uint2 c8 = *(const uint2 *)(codes + t * D + g4 * DL + 8 * m);
        const uint2 a = decode_group_levels<L>(c8.x), c = decode_group_levels<L>(c8.y);
        *(uint4 *)(row + g4 * DL + 8 * m) = make_uint4(a.x, a.y, c.x, c.y);
      }
      wave_lds_sync();
    } else {
      constexpr int BITS = FMT == FMT_TQ2 ? 2 : 3;
#pragma unroll
      for (int m = 0; m < DL / 8; ++m) {
        const uint2 a = decode_group<BITS>(group_sel<BITS>(r.w, 2 * m));
        const uint2 c = decode_group<BITS>(group_sel<BITS>(r.w, 2 * m + 1));
        *(uint4 *)(row + g4 * DL + 8 * m) = make_uint4(a.x, a.y, c.x, c.y);
      }
    }
    if (lane < 16) {
      const int pos = kpos0 + t;
      kp[16 * j + t] = (kpos0 >= 0 && pos < N) ? pos : kPfNoKey;
#pragma unroll
      for (int sgm = 0; sgm < (FMT == FMT_TQK ? 3 : 1); ++sgm) ksc[sgm * kPfKeys + 16 * j + t] = pf_scale<FMT>(r.sc[sgm]);
    }
  } else {
    // V lane layout: group q = four tokens 4 g4 .. 4 g4 + 3 of dim t + 16 q
    uint16_t *col = vt + 16 * j + 4 * g4;
    if constexpr (FMT == FMT_FP8) {
#pragma unroll
      for (int q = 0; q < D / 16; ++q) {
        const uint32_t w = r.w[q];
        *(uint2 *)(col + (t + 16 * q) * kPfVS) = make_uint2(fp8x2_to_f16x2(w, false), fp8x2_to_f16x2(w, true));
      }
    } else if constexpr (is_tqf(FMT)) {
      constexpr int L = tqf_levels(FMT);
      uint32_t *raw = (uint32_t *)tw;
      uint8_t *codes = tw + 1536;
      *(uint4 *)(raw + 4 * lane) = make_uint4(r.w[0], r.w[1], r.w[2], r.w[3]);
      if constexpr (D == 256) *(uint2 *)(raw + 256 + 2 * lane) = make_uint2(r.w[4], r.w[5]);
      wave_lds_sync();
      tqf_unpack_tile<D, L, false>(raw, codes, 16, lane);
      wave_lds_sync();
#pragma unroll
      for (int q = 0; q < D / 16; ++q) {
        const uint32_t c4 = *(const uint32_t *)(codes + (t + 16 * q) * 16 + 4 * g4);
        const uint2 a = decode_group_levels<L>(c4);
        *(uint2 *)(col + (t + 16 * q) * kPfVS) = a;
      }
      wave_lds_sync();
    } else {
      constexpr int BITS = FMT == FMT_TQ2 ? 2 : 3;        // TQK values are TQ3
#pragma unroll
      for (int q = 0; q < D / 16; ++q) {
        const uint2 a = decode_group<BITS>(group_sel<BITS>(r.w, q));
        *(uint2 *)(col + (t + 16 * q) * kPfVS) = a;
      }
    }
    if (lane < 16) vsc[16 * j + t] = pf_scale<FMT>(r.sc[0]);
  }
}

// One step's attention for this wave's rows from a step buffer. The rows'
// reference maxima stay fixed during a scan (the accumulator is never
// rescaled here): a row takes its first visible score as its reference, and
// the probabilities 2^(s - m) stay below 2^kRescaleSlack while no score
// exceeds the reference by more; the step reports (true) when one does, and
// m_seen keeps the largest score the row has seen for the scan's restart.
template <int FMT, int D>
__device__ __forceinline__ bool pf_compute(const uint8_t *buf, const uint32_t (&qb)[PfShape<D, FMT>::DW / 4],
                                           floatx16 (&acc)[PfShape<D, FMT>::DW / 32], float &m_run, float &l_run,
                                           float &m_seen, int pos, int lane, float4 *sx, int wave) {
  constexpr bool SPLIT = PfShape<D, FMT>::SPLIT;
  constexpr int NKK = PfShape<D, FMT>::DW / 16, NJD = PfShape<D, FMT>::DW / 32;
  static_assert(!SPLIT || FMT != FMT_TQK, "grouped keys exist at d = 128 only");
  const int dh = SPLIT ? (wave >> 2) : 0;              // this wave's half of the head dim
  constexpr int NSEG = FMT == FMT_TQK ? 3 : 1;
  const uint16_t *kt = (const uint16_t *)buf;
  const uint16_t *vt = (const uint16_t *)(buf + pf_vt_off(D));
  const float *ksc = (const float *)(buf + pf_ksc_off(D));
  const float *vsc = (const float *)(buf + pf_vsc_off(D));
  const int *kp = (const int *)(buf + pf_kp_off(D));
  const int h = lane >> 5;
  floatx16 s[NSEG];
#pragma unroll
  for (int sgm = 0; sgm < NSEG; ++sgm)
#pragma unroll
    for (int i = 0; i < 16; ++i) s[sgm][i] = 0.f;
  const uint16_t *krow = kt + (lane & 31) * pf_ks(D) + 8 * h;
  // every K fragment is requested before the first MFMA, so the LDS latency
  // is paid once per step rather than once per MFMA
  uint4 kf[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) kf[kk] = *(const uint4 *)(krow + 16 * (dh * NKK + kk));
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    const int sgm = FMT == FMT_TQK ? (kk < D / 64 ? 0 : (kk < 3 * D / 64 ? 1 : 2)) : 0;
    const uint4 a = kf[kk];
    s[sgm] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_half8(a.x, a.y, a.z, a.w),
                                                    as_half8(qb[4 * kk], qb[4 * kk + 1], qb[4 * kk + 2], qb[4 * kk + 3]),
                                                    s[sgm], 0, 0, 0);
  }
  if constexpr (SPLIT) {
    // the other half of every score: both waves add the same two partials,
    // so they hold bitwise equal scores from here on
#pragma unroll
    for (int q = 0; q < 4; ++q)
      sx[(wave * 4 + q) * 64 + lane] = make_float4(s[0][4 * q], s[0][4 * q + 1], s[0][4 * q + 2], s[0][4 * q + 3]);
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 o = sx[((wave ^ 4) * 4 + q) * 64 + lane];
      s[0][4 * q] += o.x; s[0][4 * q + 1] += o.y; s[0][4 * q + 2] += o.z; s[0][4 * q + 3] += o.w;
    }
  }
  // lane's keys: i -> key 8 (i / 4) + 4 h + i % 4
  float sc[16], vs[16];
  float mx = kNegInf;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int k0 = 8 * q + 4 * h;
    const int4 kq = *(const int4 *)(kp + k0);
    const float4 v4 = *(const float4 *)(vsc + k0);
    float4 k4[NSEG];
#pragma unroll
    for (int sgm = 0; sgm < NSEG; ++sgm) k4[sgm] = *(const float4 *)(ksc + sgm * kPfKeys + k0);
    const int kpv[4] = {kq.x, kq.y, kq.z, kq.w};
    const float vv[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float x = 0.f;
#pragma unroll
      for (int sgm = 0; sgm < NSEG; ++sgm) {
        const float kv = u == 0 ? k4[sgm].x : (u == 1 ? k4[sgm].y : (u == 2 ? k4[sgm].z : k4[sgm].w));
        x = __builtin_fmaf(s[sgm][4 * q + u], kv, x);
      }
      sc[4 * q + u] = kpv[u] <= pos ? x : kNegInf;
      vs[4 * q + u] = vv[u];
      mx = fmaxf(mx, sc[4 * q + u]);
    }
  }
  // the V fragments of the PV MFMAs are requested before the softmax, whose
  // ALU work then covers their LDS latency
  const uint16_t *vrow = vt + (lane & 31) * kPfVS + 4 * h;
  uint2 vf[NJD][2][2];
#pragma unroll
  for (int jd = 0; jd < NJD; ++jd)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      vf[jd][hf][0] = *(const uint2 *)(vrow + 32 * (dh * NJD + jd) * kPfVS + 16 * hf);
      vf[jd][hf][1] = *(const uint2 *)(vrow + 32 * (dh * NJD + jd) * kPfVS + 16 * hf + 8);
    }
  __builtin_amdgcn_sched_barrier(0);
  mx = fmaxf(mx, lane_xor<32>(mx, lane));
  m_seen = fmaxf(m_seen, mx);
  if (m_run == kNegInf) m_run = mx;                 // nothing accumulated yet: take this step's maximum
  const bool over = __builtin_amdgcn_ballot_w64(mx > m_run + kRescaleSlack) != 0;
  half8_t pb[2];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float pr = m_run == kNegInf ? 0.f : fast_exp2(sc[i] - m_run);
    l_run += pr;
    pb[i >> 3][i & 7] = (_Float16)(pr * vs[i]);
  }
  // O^T[dim][row] += V^T[dim][key] P^T[key][row]; the two 16-key halves take
  // keys {4h .. 4h+3, 8+4h .. 8+4h+3} (+16) in the lane's own P order
#pragma unroll
  for (int jd = 0; jd < NJD; ++jd) {
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const uint2 a0 = vf[jd][hf][0], a1 = vf[jd][hf][1];
      acc[jd] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_half8(a0.x, a0.y, a1.x, a1.y), pb[hf], acc[jd], 0, 0, 0);
    }
  }
  return over;
}

// All visible pages of one format: steps of two tiles, each wave loading
// and decoding tile (wave & 1), role (wave >> 1) two steps ahead. If some
// row's score exceeds its reference by more than the slack, the workgroup
// scans the format again from the state it started with (reload), each row
// now referenced to the largest score it has seen: rare (references are set
// by each row's first visible scores), and it keeps the common path free of
// accumulator rescales.
template <int FMT, int D, typename Reload>
__device__ __forceinline__ void pf_scan(const PrefillParams &p, int g, const int2 *ent, int n_vis, int N,
                                        uint8_t *lds, const uint32_t (&qb)[PfShape<D, FMT>::DW / 4],
                                        floatx16 (&acc)[PfShape<D, FMT>::DW / 32], float &m_run, float &l_run, int pos,
                                        int lane, int wave, uint32_t *flag, Reload reload) {
  const int P = p.P, T = P / 16;
  const int tiles = n_vis * T;
  const int steps = (tiles + 1) / 2;
  // waves 0..3 load and decode the steps (at d = 256 the other four only
  // compute)
  const bool dec = wave < 4;
  const int j = wave & 1, role = (wave >> 1) & 1;
  float4 *sx = (float4 *)(lds + pf_sx_off(D));
  const uint8_t *pool = p.pool[FMT] + (int64_t)g * p.head_bytes[FMT];
  const int64_t page_bytes = p.page_bytes[FMT];
  const int hb = (int)p.head_bytes[FMT];
  uint8_t *tw = lds + 2 * pf_buf_bytes(D) + (wave & 3) * pf_tqf_wave_bytes(D);
  // The entries are read through the scalar cache (constant address space:
  // the plan wrote them before this launch, and nothing writes them during
  // it), with a scalar index. A vector load of an entry would be waited for
  // with every tile load in flight.
  typedef __attribute__((address_space(4))) const uint64_t const_u64;
  const const_u64 *ent_c = (const const_u64 *)ent;
  auto entry = [&](int s, int &kpos0, int &tau) {
    const int tt = 2 * s + j;
    tau = tt % T;
    if (tt >= tiles) { kpos0 = -1; return block_rsrc(pool, 0); }
    const uint64_t ev = ent_c[__builtin_amdgcn_readfirstlane(tt / T)];   // (logical page, id)
    const int2 e = make_int2((int)(uint32_t)ev, (int)(uint32_t)(ev >> 32));
    kpos0 = e.x * P + tau * 16;
    return block_rsrc(pool + (int64_t)e.y * page_bytes, hb);
  };
  float m_seen = m_run;
  // Grouped keys decode ahead: a step first decodes the next step's tiles
  // into the other buffer (free since the barrier that ended the step
  // before), then computes its own, so the decoding waves' ALU work overlaps
  // the other waves' MFMAs. Measured faster for this format only: at d = 256
  // the split waves meet again at the score exchange, and the other d = 128
  // codes spill with both steps' registers live.
  constexpr bool AHEAD = FMT == FMT_TQK;
  for (;;) {
    bool again = false;
    if constexpr (AHEAD) {
      // raw slot k holds the tiles of step s with s % 2 == k, two steps
      // before their decode
      PfRaw<FMT, D> raw[2];
      int kpos[2] = {-1, -1}, tau;
      if (dec) {
        __amdgpu_buffer_rsrc_t rs = entry(0, kpos[0], tau);
        pf_load<FMT, D>(raw[0], rs, tau, T, P, role, lane);
        if (steps > 1) {
          rs = entry(1, kpos[1], tau);
          pf_load<FMT, D>(raw[1], rs, tau, T, P, role, lane);
        }
        pf_store<FMT, D>(raw[0], lds, j, role, kpos[0], N, lane, tw);
        if (steps > 2) {
          rs = entry(2, kpos[0], tau);
          pf_load<FMT, D>(raw[0], rs, tau, T, P, role, lane);
        }
      }
      __syncthreads();
      // step s computes from its buffer; r / kp are the slot of step s + 1
      auto step = [&](int s, PfRaw<FMT, D> &r, int &kp) {
        // the flag step s - 1 may have set was final at the barrier that
        // ended it; step s sets only the other
        if (s > 0 && ((volatile uint32_t *)flag)[(s - 1) & 1]) return true;   // every wave stops here
        if (dec && s + 1 < steps) {
          pf_store<FMT, D>(r, lds + ((s + 1) & 1) * pf_buf_bytes(D), j, role, kp, N, lane, tw);
          if (s + 3 < steps) {
            int t3;
            const __amdgpu_buffer_rsrc_t r3 = entry(s + 3, kp, t3);
            pf_load<FMT, D>(r, r3, t3, T, P, role, lane);
          }
        }
        const bool over = pf_compute<FMT, D>(lds + (s & 1) * pf_buf_bytes(D), qb, acc, m_run, l_run, m_seen, pos,
                                             lane, sx, wave);
        if (over && lane == 0) ((volatile uint32_t *)flag)[s & 1] = 1u;
        __syncthreads();
        return false;
      };
      int s = 0;
      for (; s + 2 <= steps && !again; s += 2) {
        again = step(s, raw[1], kpos[1]);
        if (!again) again = step(s + 1, raw[0], kpos[0]);
      }
      if (!again && s < steps) again = step(s, raw[1], kpos[1]);
    } else {
      // two steps of raw tiles in flight: slot k holds step s with s % 2 == k
      PfRaw<FMT, D> raw[2];
      int kpos[2] = {-1, -1}, tau;
      if (dec) {
        __amdgpu_buffer_rsrc_t rs = entry(0, kpos[0], tau);
        pf_load<FMT, D>(raw[0], rs, tau, T, P, role, lane);
        if (steps > 1) {
          rs = entry(1, kpos[1], tau);
          pf_load<FMT, D>(raw[1], rs, tau, T, P, role, lane);
        }
      }
      auto step = [&](int s, PfRaw<FMT, D> &r, int &kp) {
        uint8_t *buf = lds + (s & 1) * pf_buf_bytes(D);
        if (dec) pf_store<FMT, D>(r, buf, j, role, kp, N, lane, tw);
        __syncthreads();
        // the flags alternate by step: the one step s - 1 may have set was
        // final at this barrier, and step s sets only the other (the flag's
        // read waits for every load in flight, so step s + 2's tiles are
        // requested after it)
        if (s > 0 && ((volatile uint32_t *)flag)[(s - 1) & 1]) return true;   // every wave stops here
        if (dec && s + 2 < steps) {
          int t2;
          const __amdgpu_buffer_rsrc_t r2 = entry(s + 2, kp, t2);
          pf_load<FMT, D>(r, r2, t2, T, P, role, lane);
        }
        if (pf_compute<FMT, D>(buf, qb, acc, m_run, l_run, m_seen, pos, lane, sx, wave) && lane == 0)
          ((volatile uint32_t *)flag)[s & 1] = 1u;
        return false;
      };
      int s = 0;
      for (; s + 2 <= steps && !again; s += 2) {
        again = step(s, raw[0], kpos[0]);
        if (!again) again = step(s + 1, raw[1], kpos[1]);
      }
      if (!again && s < steps) again = step(s, raw[0], kpos[0]);
    }
    __syncthreads();                                // the buffers are free again, every step done
    if (!again) again = (((volatile uint32_t *)flag)[0] | ((volatile uint32_t *)flag)[1]) != 0u;
    if (!again) break;
    __syncthreads();                                // every wave has read the flags
    if (threadIdx.x == 0) {
      ((volatile uint32_t *)flag)[0] = 0u;
      ((volatile uint32_t *)flag)[1] = 0u;
    }
    // again from the starting state, referenced to the largest score seen
    float m0, l0;
    reload(acc, m0, l0);
    const float m_new = fmaxf(m_seen, m0);
    const float f = (m0 == kNegInf || m_new == kNegInf) ? 0.f : fast_exp2(m0 - m_new);
#pragma unroll
    for (int jd = 0; jd < PfShape<D, FMT>::DW / 32; ++jd) acc[jd] *= f;
    l_run = l0 * f;
    m_run = m_new;
    m_seen = m_new;
  }
}

// R_V^T of the accumulator of this wave's rows (O^T element (jd, i) of lane
// l is dim 32 (jd0 + jd) + 8 (i / 4) + 4 (l / 32) + i % 4 of row l % 32,
// jd0 the first 32-dim block the wave holds), through the row block's LDS
// area st (16 rows of D + 4 floats) in two halves of 16 rows: the rows go to
// LDS, each row is transformed across a wave like the query (lane l holds
// dims E l .. E l + E - 1: s_V * FWHT / sqrt(D)), and the lanes read their
// elements back. With the head dim split over two waves, both write their
// halves and each transforms eight of the sixteen rows.
template <int D, int FMT>
__device__ __forceinline__ void pf_unrotate(const PrefillParams &p, floatx16 (&acc)[PfShape<D, FMT>::DW / 32], int g,
                                            float *st, int lane, int dh) {
  constexpr bool SPLIT = PfShape<D, FMT>::SPLIT;
  constexpr int NJD = PfShape<D, FMT>::DW / 32;
  constexpr int E = D / 64;
  constexpr int RS = D + 4;
  const uint32_t sv = p.signs[((int64_t)g * 2 + 1) * (D / 32) + (E * lane) / 32] >> ((E * lane) & 31);
  constexpr float rs = D == 256 ? 0.0625f : 0.08838834764831845f;   // 1 / sqrt(D)
  const int r = lane & 31, h = lane >> 5;
  const int jd0 = dh * NJD;
  auto sync = [] {
    if constexpr (SPLIT) __syncthreads();
    else wave_lds_sync();
  };
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const bool mine = (r >> 4) == hf;
    if (mine) {
#pragma unroll
      for (int jd = 0; jd < NJD; ++jd)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *(float4 *)(st + (r - 16 * hf) * RS + 32 * (jd0 + jd) + 8 * q + 4 * h) =
              make_float4(acc[jd][4 * q], acc[jd][4 * q + 1], acc[jd][4 * q + 2], acc[jd][4 * q + 3]);
    }
    sync();
    for (int rr = SPLIT ? 8 * dh : 0; rr < (SPLIT ? 8 * dh + 8 : 16); ++rr) {
      float x[E];
      if constexpr (E == 4) {
        const float4 v = *(const float4 *)(st + rr * RS + 4 * lane);
        x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
      } else {
        const float2 v = *(const float2 *)(st + rr * RS + 2 * lane);
        x[0] = v.x; x[1] = v.y;
      }
      wave_fwht_rows<D>(x, lane);
#pragma unroll
      for (int e = 0; e < E; ++e) x[e] = ((sv >> e) & 1u) ? -(x[e] * rs) : x[e] * rs;
      if constexpr (E == 4) *(float4 *)(st + rr * RS + 4 * lane) = make_float4(x[0], x[1], x[2], x[3]);
      else *(float2 *)(st + rr * RS + 2 * lane) = make_float2(x[0], x[1]);
    }
    sync();
    if (mine) {
#pragma unroll
      for (int jd = 0; jd < NJD; ++jd)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 v = *(const float4 *)(st + (r - 16 * hf) * RS + 32 * (jd0 + jd) + 8 * q + 4 * h);
          acc[jd][4 * q] = v.x; acc[jd][4 * q + 1] = v.y; acc[jd][4 * q + 2] = v.z; acc[jd][4 * q + 3] = v.w;
        }
    }
    sync();
  }
}

// One format's pass of the packed prefill (one launch per format the cache
// holds: the TQ formats, then FP8). The running state of every row (m, l
// and O, unnormalized) passes between the launches through the workspace:
// the first launch starts from the empty state, a TQ launch keeps O in
// rotated V space unless the next launch is FP8 or it is the last one (then
// it turns O back, R_V^T), and the last launch writes out and lse.
// One format per kernel keeps each scan's registers to its own format.
template <int D, int FMT>
__global__ __launch_bounds__((64 * PfShape<D, FMT>::WAVES))
__attribute__((amdgpu_waves_per_eu(PfShape<D, FMT>::WPE, PfShape<D, FMT>::WPE)))
void prefill_kernel(PrefillParams p) {
  constexpr bool SPLIT = PfShape<D, FMT>::SPLIT;
  constexpr int NJD = PfShape<D, FMT>::DW / 32;
  constexpr int ROWS = PfShape<D, FMT>::ROWS;
  constexpr int TPR = 64 * PfShape<D, FMT>::WAVES / ROWS;   // threads per row
  extern __shared__ __align__(16) uint8_t pf_lds[];
  __shared__ uint32_t s_over[2];                            // a scan step saw a score past a row's reference
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int rbw = SPLIT ? (wave & 3) : wave;                // the wave's 32-row block
  const int dh = SPLIT ? (wave >> 2) : 0;                   // and half of the head dim (d = 256)
  const int rb = p.row_blocks - 1 - (int)blockIdx.x;       // the longest rows first
  if (threadIdx.x < 2) s_over[threadIdx.x] = 0u;            // read after the scan's barriers
  const int g = blockIdx.y, b = blockIdx.z;
  {
    const int4 a = *(const int4 *)p.plan_hdr;
    const int4 c = *((const int4 *)p.plan_hdr + 1);
    const bool ok = a.x == kPlanMagic && a.y == p.B && a.z == p.max_pages && a.w == p.Hkv && c.x == p.P && c.y == p.D;
    if (!__builtin_amdgcn_readfirstlane((int)ok)) {
      // a plan built for another geometry: the last launch poisons the rows,
      // the first counts the call once
      const int r = rb * ROWS + (int)threadIdx.x / TPR;
      if (p.last && r < p.chunk * p.G && (threadIdx.x % TPR) == 0) {
        const int64_t orow = ((int64_t)b * p.chunk + r / p.G) * p.Hq + (int64_t)g * p.G + r % p.G;
        for (int d = 0; d < D; ++d) p.out[orow * D + d] = __builtin_nanf("");
        if (p.lse) p.lse[orow] = __builtin_nanf("");
      }
      if (p.first && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x == 0 && p.counters)
        atomicAdd(&p.counters->invalid_entries, 1ull);
      return;
    }
  }
  const int G = p.G, C = p.chunk;
  int N = p.seq[b];
  N = N < 0 ? 0 : N;
  const int n0 = N - C;
  const int row0 = rb * ROWS + rbw * 32;
  const int row = row0 + (lane & 31);
  const int c = row / G, n = row - (row / G) * G;
  const bool valid = c < C;
  const int pos = valid ? n0 + c : -1;
  const int c_last = min(C - 1, (rb * ROWS + ROWS - 1) / G);
  const int maxpos = n0 + c_last;                           // the block's last row sees up to here
  const int64_t orow = ((int64_t)b * C + (valid ? c : 0)) * p.Hq + (int64_t)g * G + n;
  const int h = lane >> 5;
  // this format's visible pages
  const int32_t *cnt = p.counts + (int64_t)b * NFMT;
  int start = 0;
#pragma unroll
  for (int f = 0; f < FMT; ++f) start += cnt[f];
  const int nf = __builtin_amdgcn_readfirstlane(cnt[FMT]);
  const int2 *ent = p.entries + (int64_t)b * p.max_pages + start;
  const int n_vis = (maxpos >= 0 && nf > 0)
                        ? __builtin_amdgcn_readfirstlane(pf_count_visible(ent, nf, maxpos / p.P, lane)) : 0;
  if (blockIdx.x == 0 && threadIdx.x == 0 && p.counters && n_vis > 0) {
    unsigned long long *ctr = FMT == FMT_FP8 ? &p.counters->pages_fp8 : FMT == FMT_TQ3 ? &p.counters->pages_tq3
                            : FMT == FMT_TQ2 ? &p.counters->pages_tq2 : FMT == FMT_TQK ? &p.counters->pages_tqk
                            : FMT == FMT_TQF5 ? &p.counters->pages_tqf5 : &p.counters->pages_tqf6;
    atomicAdd(ctr, (unsigned long long)n_vis);
  }
  // nothing to scan, nothing to start, turn or write: the state stays as it is
  if (n_vis == 0 && !p.first && !p.last && !p.unrot_out) return;
  // the rows' state at the start of this launch (also the restart point of
  // the scan)
  auto reload = [&](floatx16 (&a)[NJD], float &m0, float &l0) {
    m0 = kNegInf;
    l0 = 0.f;
    if (p.first || !valid) {
#pragma unroll
      for (int jd = 0; jd < NJD; ++jd)
#pragma unroll
        for (int i = 0; i < 16; ++i) a[jd][i] = 0.f;
    } else {
      const float *so = p.ws_o + orow * D + 32 * dh * NJD + 4 * h;
#pragma unroll
      for (int jd = 0; jd < NJD; ++jd)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 v = *(const float4 *)(so + 32 * jd + 8 * q);
          a[jd][4 * q] = v.x; a[jd][4 * q + 1] = v.y; a[jd][4 * q + 2] = v.z; a[jd][4 * q + 3] = v.w;
        }
      const float2 ml = *(const float2 *)(p.ws_ml + orow * 2);
      m0 = ml.x;
      l0 = h == 0 ? ml.y : 0.f;                             // the row's l, counted once
    }
  };
  floatx16 acc[NJD];
  float m_run, l_run;
  reload(acc, m_run, l_run);
  if (n_vis > 0) {
    uint32_t qb[PfShape<D, FMT>::DW / 4];
    uint16_t *qs = (uint16_t *)pf_lds + rbw * 32 * pf_ks(D);
    constexpr int QM = FMT == FMT_FP8 ? QM_BF16 : (FMT == FMT_TQK ? QM_GROUPED : QM_ROT);
    if constexpr (FMT != FMT_TQK || D == 128) {
      // one wave of each row block stages the block's query rows; every wave
      // takes the fragments of its dims
      if (dh == 0) pf_query_stage<D, QM>(p, b, g, row0, qs, lane);
      if constexpr (SPLIT) __syncthreads();
      else wave_lds_sync();
      pf_query_frags<D, PfShape<D, FMT>::DW / 16>(qs, dh * (PfShape<D, FMT>::DW / 16), lane, qb);
      // with one wave a SIMD (d = 256, unsplit) the query fragments sit in
      // the accumulation registers (MFMAs read their operands there): that
      // leaves the vector registers to the fragments read ahead from LDS
      if constexpr (PfShape<D, FMT>::WPE == 1) {
#pragma unroll
        for (int i = 0; i < D / 4; ++i) asm volatile("" : "+a"(qb[i]));
      }
      __syncthreads();                                      // every wave holds its query fragments
      pf_scan<FMT, D>(p, g, ent, n_vis, N, pf_lds, qb, acc, m_run, l_run, pos, lane, wave, s_over, reload);
    }
  }
  if (FMT != FMT_FP8 && p.unrot_out) {
    float *ust = (float *)pf_lds + rbw * 16 * (D + 4);
    pf_unrotate<D, FMT>(p, acc, g, ust, lane, dh);
  }
  const float l_tot = l_run + lane_xor<32>(l_run, lane);
  if (!valid) return;
  if (p.last) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    float *o = p.out + orow * D + 32 * dh * NJD + 4 * h;
#pragma unroll
    for (int jd = 0; jd < NJD; ++jd)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *(float4 *)(o + 32 * jd + 8 * q) = make_float4(acc[jd][4 * q] * inv, acc[jd][4 * q + 1] * inv,
                                                       acc[jd][4 * q + 2] * inv, acc[jd][4 * q + 3] * inv);
    if (h == 0 && dh == 0 && p.lse) p.lse[orow] = l_tot > 0.f ? (m_run + log2f(l_tot)) * 0.69314718055994531f : kNegInf;
  } else {
    float *so = p.ws_o + orow * D + 32 * dh * NJD + 4 * h;
#pragma unroll
    for (int jd = 0; jd < NJD; ++jd)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *(float4 *)(so + 32 * jd + 8 * q) = make_float4(acc[jd][4 * q], acc[jd][4 * q + 1], acc[jd][4 * q + 2],
                                                        acc[jd][4 * q + 3]);
    if (h == 0 && dh == 0) *(float2 *)(p.ws_ml + orow * 2) = make_float2(m_run, l_tot);
  }
}

}  // namespace

hipError_t launch_plan(const PlanParams &p, hipStream_t s) {
  if (p.B <= 0) return hipSuccess;
  hipLaunchKernelGGL(plan_kernel, dim3(p.B), dim3(kPlanThreads), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(items_kernel, dim3((unsigned)p.n_slots), dim3(64), 0, s, p);
  return hipGetLastError();
}

size_t decode_lds_bytes(int d, int G) {
  // the query staging, then each wave's fractional-level scan area
  const size_t q = (size_t)query_stage_bytes(d) + (size_t)kW * (d == 256 ? tqf_wave_bytes(256) : tqf_wave_bytes(128));
  // the in-workgroup merge past the query staging: (m, l) per wave and
  // head, then every wave's G rows of d + 4 floats (at most 8 x 16 x 260 x 4
  // = 133,120 bytes)
  const size_t wmerge = (size_t)query_stage_bytes(d) + (size_t)kW * 16 * 2 * 4 + (size_t)kW * G * (d + 4) * 4;
  return q > wmerge ? q : wmerge;
}

// Dynamic LDS above 64 KB must be allowed per kernel (and device) first.
static hipError_t allow_lds(const void *kernel, int slot, size_t lds) {
  if (lds <= 65536) return hipSuccess;
  static size_t allowed[64][8] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (allowed[dev][slot] >= lds) return hipSuccess;
  const hipError_t e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e == hipSuccess) allowed[dev][slot] = lds;
  return e;
}

// Workgroups of the persistent grid: one per CU of the current device.
static int decode_grid(int64_t units) {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cus[dev] <= 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev] = n * kWorkgroupsPerCU;
  }
  return (int)(units < cus[dev] ? units : cus[dev]);
}

hipError_t launch_decode(const DecodeParams &pin, int d, hipStream_t s, hipEvent_t scan_end) {
  DecodeParams p = pin;
  const int64_t units = p.n_slots * p.Hkv;
  if (units <= 0) return hipSuccess;
  size_t lds = decode_lds_bytes(d, p.G);
  const dim3 grid((unsigned)decode_grid(units));
  const bool mass = p.tile_lmass != nullptr;
  if (mass) {
    // scored scan: the tile log-mass stage after the scan's LDS
    const int s_max = (int)((p.packet_stride - (int64_t)sizeof(ItemHeader)) / 8);
    const int cap = ((s_max + kW - 1) / kW) * (p.P / 16);
    const size_t base = (lds + 15) & ~(size_t)15;
    p.mass_lds_off = (int)(base / 4);
    lds = base + (size_t)kW * cap * p.G * 4 + (size_t)s_max * 4;
  }
  const bool causal = p.chunk > 1;
  {
    const void *k = d == 256 ? (mass ? (const void *)decode_kernel<256, true, false>
                                     : causal ? (const void *)decode_kernel<256, false, true>
                                              : (const void *)decode_kernel<256, false, false>)
                             : (mass ? (const void *)decode_kernel<128, true, false>
                                     : causal ? (const void *)decode_kernel<128, false, true>
                                              : (const void *)decode_kernel<128, false, false>);
    const hipError_t e = allow_lds(k, (d == 256 ? 3 : 0) + (mass ? 1 : causal ? 2 : 0), lds);
    if (e != hipSuccess) return e;
  }
  if (mass) {
    // tiles the scan does not reach (masked entries, pages past N_b) hold -inf
    const int64_t n = (int64_t)p.B * p.Hq * p.tlm_stride;
    const int64_t blocks = (n + 255) / 256 < 2048 ? (n + 255) / 256 : 2048;
    hipLaunchKernelGGL(fill_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p.tile_lmass, n, kNegInf);
  }
  if (d == 256) {
    if (mass) hipLaunchKernelGGL((decode_kernel<256, true, false>), grid, dim3(kDecodeThreads), lds, s, p);
    else if (causal) hipLaunchKernelGGL((decode_kernel<256, false, true>), grid, dim3(kDecodeThreads), lds, s, p);
    else hipLaunchKernelGGL((decode_kernel<256, false, false>), grid, dim3(kDecodeThreads), lds, s, p);
  } else {
    if (mass) hipLaunchKernelGGL((decode_kernel<128, true, false>), grid, dim3(kDecodeThreads), lds, s, p);
    else if (causal) hipLaunchKernelGGL((decode_kernel<128, false, true>), grid, dim3(kDecodeThreads), lds, s, p);
    else hipLaunchKernelGGL((decode_kernel<128, false, false>), grid, dim3(kDecodeThreads), lds, s, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (scan_end) {
    e = hipEventRecord(scan_end, s);
    if (e != hipSuccess) return e;
  }
  const dim3 mgrid((unsigned)((int64_t)p.B * p.Hq));
  const bool append = p.new_kv != nullptr;
  if (d == 256) {
    if (mass) hipLaunchKernelGGL((merge_kernel<256, true, false>), mgrid, dim3(256), 0, s, p);
    else if (append) hipLaunchKernelGGL((merge_kernel<256, false, true>), mgrid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((merge_kernel<256, false, false>), mgrid, dim3(256), 0, s, p);
  } else {
    if (mass) hipLaunchKernelGGL((merge_kernel<128, true, false>), mgrid, dim3(128), 0, s, p);
    else if (append) hipLaunchKernelGGL((merge_kernel<128, false, true>), mgrid, dim3(128), 0, s, p);
    else hipLaunchKernelGGL((merge_kernel<128, false, false>), mgrid, dim3(128), 0, s, p);
  }
  return hipGetLastError();
}

template <int D, int FMT>
static hipError_t launch_prefill_fmt(const PrefillParams &p, hipStream_t s) {
  const size_t lds = (size_t)pf_lds_bytes(D, PfShape<D, FMT>::SPLIT, PfShape<D, FMT>::RBW);
  const void *k = (const void *)prefill_kernel<D, FMT>;
  static size_t allowed[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (lds > 65536 && allowed[dev] < lds) {
    const hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    allowed[dev] = lds;
  }
  // this shape's row blocks (the workspace holds per-row state, so the
  // formats' launches may block rows differently)
  PrefillParams q = p;
  const int64_t rows = (int64_t)p.chunk * p.G;
  q.row_blocks = (int)((rows + PfShape<D, FMT>::ROWS - 1) / PfShape<D, FMT>::ROWS);
  const dim3 grid((unsigned)q.row_blocks, (unsigned)q.Hkv, (unsigned)q.B);
  hipLaunchKernelGGL((prefill_kernel<D, FMT>), grid, dim3(64 * PfShape<D, FMT>::WAVES), lds, s, q);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_prefill_d(const PrefillParams &p, int fmt, hipStream_t s) {
  switch (fmt) {
    case FMT_FP8: return launch_prefill_fmt<D, FMT_FP8>(p, s);
    case FMT_TQ3: return launch_prefill_fmt<D, FMT_TQ3>(p, s);
    case FMT_TQ2: return launch_prefill_fmt<D, FMT_TQ2>(p, s);
    case FMT_TQK: return D == 128 ? launch_prefill_fmt<D, FMT_TQK>(p, s) : hipErrorInvalidValue;
    case FMT_TQF5: return launch_prefill_fmt<D, FMT_TQF5>(p, s);
    default: return launch_prefill_fmt<D, FMT_TQF6>(p, s);
  }
}

hipError_t launch_prefill(const PrefillParams &pin, hipStream_t s) {
  if (pin.B <= 0 || pin.row_blocks <= 0) return hipSuccess;
  // one launch per format the cache holds: the TQ formats, then FP8
  int order[NFMT], n = 0;
  for (int k = 0; k < NFMT; ++k) {
    const int f = k < NFMT - 1 ? k + 1 : FMT_FP8;
    if (pin.pool[f] && pin.pool_pages[f] > 0) order[n++] = f;
  }
  if (n == 0) order[n++] = FMT_FP8;                       // no pool at all: one launch writes the empty rows
  for (int k = 0; k < n; ++k) {
    PrefillParams p = pin;
    const int f = order[k];
    p.first = k == 0;
    p.last = k == n - 1;
    p.unrot_out = f != FMT_FP8 && (p.last || order[k + 1] == FMT_FP8);
    const hipError_t e = pin.D == 256 ? launch_prefill_d<256>(p, f, s) : launch_prefill_d<128>(p, f, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_collect(const CollectParams &c, hipStream_t s) {
  if (c.B <= 0) return hipSuccess;
  hipLaunchKernelGGL(collect_kernel, dim3((unsigned)((c.max_pages + 255) / 256), (unsigned)c.B), dim3(256), 0, s, c);
  return hipGetLastError();
}

}  // namespace kvq
