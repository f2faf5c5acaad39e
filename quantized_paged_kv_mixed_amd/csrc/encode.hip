// Encoders of the paged KV pools for gfx950 (MI355X).
//
// FP8 (Minima-KV, arxiv 2608.23834, section 3.1 "Recent" and algorithm 1
// "Append"): one fp32 scale per (token, KV head, role), codes E4M3 with
// round-to-nearest-even, converted by the hardware v_cvt_pk_fp8_f32 (OCP
// E4M3 on gfx950).
// TQ (Minima-KV section 4.3 "normalize-rotate-pack"; Block-GTQ, paperpeel
// 2606.24033, appendix B.1): per vector, the norm by a fixed halving tree,
// Hadamard-sign rotation by an unnormalized butterfly FWHT, threshold
// comparison against norm-scaled fp32 midpoints of the fp16 Gaussian
// Lloyd-Max centroids, and an fp16 norm correction sigma = ||x|| / ||c||.
// Every step is fp32 round-to-nearest-even with contraction off, so codes and
// sigmas are bit-identical to the plain CPU definition.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kvq_internal.h"

#pragma clang fp contract(off)

namespace kvq {
namespace {

typedef float float2_t __attribute__((ext_vector_type(2)));

// Thresholds (ascending): fp32 midpoints of adjacent fp16 centroids.
__constant__ float kTh3[7] = {-1.748046875f, -1.0498046875f, -0.50048828125f, 0.0f,
                              0.50048828125f, 1.0498046875f, 1.748046875f};
__constant__ float kTh2[3] = {-0.9818115234375f, 0.0f, 0.9818115234375f};
// Centroids (fp16 values, exactly representable in fp32), ascending codes.
__constant__ float kCb3[8] = {-2.15234375f, -1.34375f, -0.755859375f, -0.2451171875f,
                              0.2451171875f, 0.755859375f, 1.34375f, 2.15234375f};
__constant__ float kCb2[4] = {-1.5107421875f, -0.452880859375f, 0.452880859375f, 1.5107421875f};
__constant__ float kTh4[15] = {-2.400390625f, -1.84326171875f, -1.43701171875f, -1.09912109375f,
                               -0.799560546875f, -0.5223388671875f, -0.2581787109375f, 0.0f,
                               0.2581787109375f, 0.5223388671875f, 0.799560546875f, 1.09912109375f,
                               1.43701171875f, 1.84326171875f, 2.400390625f};
__constant__ float kCb4[16] = {-2.732421875f, -2.068359375f, -1.6181640625f, -1.255859375f,
                               -0.9423828125f, -0.65673828125f, -0.387939453125f, -0.12841796875f,
                               0.12841796875f, 0.387939453125f, 0.65673828125f, 0.9423828125f,
                               1.255859375f, 1.6181640625f, 2.068359375f, 2.732421875f};

// fp32 -> fp16 bits, round to nearest even, subnormals kept, overflow to inf.
__device__ __forceinline__ uint16_t f32_to_f16_rne(float f) {
  const uint32_t x = __builtin_bit_cast(uint32_t, f);
  const uint32_t sign = (x >> 16) & 0x8000u;
  const uint32_t ax = x & 0x7FFFFFFFu;
  if (ax >= 0x7F800000u) return (uint16_t)(sign | 0x7C00u | (ax > 0x7F800000u ? 0x200u : 0u));
  if (ax >= 0x477FF000u) return (uint16_t)(sign | 0x7C00u);           // >= 65520 rounds to inf
  if (ax < 0x38800000u) {                                               // below 2^-14: subnormal
    const float m = __builtin_bit_cast(float, ax) * 16777216.0f;        // / 2^-24, exact
    return (uint16_t)(sign | (uint32_t)__builtin_rintf(m));
  }
  const uint32_t r = ax + 0xFFFu + ((ax >> 13) & 1u);
  return (uint16_t)(sign | ((r - 0x38000000u) >> 13));
}

__device__ __forceinline__ float wave_max(float v) {
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

// FP8 codes and scale of one (token, KV head, role) vector held by a wave,
// lane l holding coordinates E l .. E l + E - 1, stored at `slot` of the
// role's tiles in `head` (an FP8 head block): amax = max |x| (vector_amax);
// amax = 0 gives
// codes 0 and scale 0; else y = x * fp32(448 / amax) rounded to E4M3 by
// v_cvt_pk_fp8_f32 (nearest, ties to even, saturating), scale = amax / 448.
template <int D>
__device__ __forceinline__ float vector_amax(const float (&x)[D / 64]) {
  float a = 0.f;
#pragma unroll
  for (int e = 0; e < D / 64; ++e) a = fmaxf(a, fabsf(x[e]));
  return wave_max(a);
}

template <int D>
__device__ __forceinline__ void fp8_store_vector(const float (&x)[D / 64], float amax, uint8_t *head, int P, int role,
                                                 int slot, int lane) {
  constexpr int E = D / 64;          // elements per lane
  constexpr int DL = D / 4;
  uint32_t packed = 0;
  float scale = 0.f;
  if (amax > 0.f) {
    const float inv = 448.0f / amax;
    float y[E];
#pragma unroll
    for (int e = 0; e < E; ++e) y[e] = x[e] * inv;
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
    if constexpr (E == 4) w = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w, true);
    packed = (uint32_t)w;
    scale = amax / 448.0f;
  }
  const int T = P / 16, tau = slot / 16, t16 = slot % 16;
  const int j0 = E * lane;
  if (role == 0) {
    uint8_t *tile = head + (int64_t)tau * 16 * D;
    const int lp = t16 + 16 * (j0 / DL), i = j0 % DL;
    uint8_t *dst = tile + ((i / 16) * 64 + lp) * 16 + i % 16;
    if constexpr (E == 4) *(uint32_t *)dst = packed;
    else *(uint16_t *)dst = (uint16_t)packed;
  } else {
    uint8_t *tile = head + (int64_t)(T + tau) * 16 * D;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int j = j0 + e;
      const int lp = j % 16 + 16 * (t16 / 4), i = 4 * (j / 16) + t16 % 4;
      tile[((i / 16) * 64 + lp) * 16 + i % 16] = (uint8_t)(packed >> (8 * e));
    }
  }
  if (lane == 0) *(float *)(head + 2LL * P * D + (int64_t)role * 4 * P + 4 * slot) = scale;
}

// ------------------------------------------------------------------------
// FP8 append: one wave per (token, KV head, role) vector
// ------------------------------------------------------------------------
template <int D, bool BF16>
__global__ __launch_bounds__(256) void encode_fp8_kernel(EncodeFp8Params p) {
  constexpr int E = D / 64;          // elements per lane
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t v = (int64_t)blockIdx.x * 4 + wave;
  if (v >= p.n_tok * p.Hkv * 2) return;
  const int role = (int)(v & 1);
  const int h = (int)((v >> 1) % p.Hkv);
  const int64_t tok = (v >> 1) / p.Hkv;
  const int64_t row = ((tok * p.Hkv + h) * 2 + role) * D + (int64_t)E * lane;
  float x[E];
  if constexpr (BF16) {
    const uint16_t *s = (const uint16_t *)p.src + row;
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = __builtin_bit_cast(float, (uint32_t)s[e] << 16);
  } else {
    const float *s = (const float *)p.src + row;
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = s[e];
  }
  // amax before the destination check keeps the row's loads ahead of the
  // destination's (two independent round trips, not one after the other)
  const float amax = vector_amax<D>(x);
  const int pid = p.dst_page[tok], slot = p.dst_slot[tok];
  if (pid < 0 || pid >= p.pool_pages || slot < 0 || slot >= p.P) return;   // the whole wave
  uint8_t *head = p.pool + (int64_t)pid * p.page_bytes + (int64_t)h * p.head_bytes;
  fp8_store_vector<D>(x, amax, head, p.P, role, slot, lane);
}

// ------------------------------------------------------------------------
// TQ encode: one workgroup per (page, KV head, role)
// ------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ int tile_word_offset(int l, int w, int W) {
  if (W == 6) return w < 4 ? l * 16 + 4 * w : 1024 + l * 8 + 4 * (w - 4);
  if (W == 3) return w < 2 ? l * 8 + 4 * w : 512 + l * 4;
  if (W == 4) return l * 16 + 4 * w;
  return l * 8 + 4 * w;  // W == 2
}

// Segment of a lane inside its wave's vector: lanes [lane0, lane0 + nl) hold
// coordinates [E lane0, E (lane0 + nl)) of one TQ-coded vector of width E nl
// at `bits` bits. A uniform format is one segment of 64 lanes; a TQK key is
// three (d/4 at 2 bits, d/2 at 3, d/4 at 4: lanes 0-15, 16-47, 48-63).
struct Seg {
  int lane0, nl, bits, idx;
};

__device__ __forceinline__ float threshold(int bits, int k) {
  return bits == 2 ? kTh2[k] : (bits == 3 ? kTh3[k] : kTh4[k]);
}
__device__ __forceinline__ float centroid(int bits, int c) {
  return bits == 2 ? kCb2[c] : (bits == 3 ? kCb3[c] : kCb4[c]);
}

// Halving-tree sum over a lane's segment, E values per lane: for h = d_s/2,
// d_s/4, .., 1: t[0:h] += t[h:2h] in the segment's own element order. The
// total ends in element 0 of the segment's first lane; every lane gets it.
template <int D>
__device__ __forceinline__ float segment_tree_sum(float (&t)[D / 64], const Seg &sg) {
  constexpr int E = D / 64;
#pragma unroll
  for (int hh = D / 2; hh >= E; hh >>= 1) {
    const int dl = hh / E;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float o = __shfl_down(t[e], dl);
      if (dl < sg.nl) t[e] = t[e] + o;
    }
  }
#pragma unroll
  for (int hh = E / 2; hh >= 1; hh >>= 1)
#pragma unroll
    for (int e = 0; e < hh; ++e) t[e] = t[e] + t[e + hh];
  return __shfl(t[0], sg.lane0);
}

// Unnormalized FWHT of every segment of a vector held by a wave (E
// consecutive coordinates per lane), stages 1, 2, 4, ...: the in-register
// stages, then lane butterflies inside the segment.
template <int D>
__device__ __forceinline__ void segment_fwht(float (&u)[D / 64], const Seg &sg, int lane) {
  constexpr int E = D / 64;
#pragma unroll
  for (int hh = 1; hh < E; hh <<= 1) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if ((e & hh) == 0) {
        const float a = u[e], b = u[e + hh];
        u[e] = a + b;
        u[e + hh] = a - b;
      }
    }
  }
  const int ll = lane - sg.lane0;
#pragma unroll
  for (int hh = E; hh < D; hh <<= 1) {
    const int dl = hh / E;
    const int partner = sg.lane0 + (ll ^ dl);
    const bool upper = (ll & dl) != 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float o = __shfl(u[e], partner);
      if (dl < sg.nl) u[e] = upper ? (o - u[e]) : (u[e] + o);
    }
  }
}

// TQ encode of every segment of one vector held by a wave (E consecutive
// coordinates per lane): norm, sign flips, unnormalized FWHT inside the
// segment, threshold count, norm correction. Returns the lane's codes and,
// for the segment, sigma bits (valid in every lane).
template <int D>
__device__ __forceinline__ uint16_t tq_encode_segment(const float (&x)[D / 64], uint32_t sign_bits, const Seg &sg,
                                                      int lane, int (&code)[D / 64]) {
  constexpr int E = D / 64;
  float t[E], u[E];
  // 1. norm by the halving tree
#pragma unroll
  for (int e = 0; e < E; ++e) t[e] = x[e] * x[e];
  const float n2 = segment_tree_sum<D>(t, sg);
  const float n = sqrtf(n2);
  // 2. sign flips
#pragma unroll
  for (int e = 0; e < E; ++e) u[e] = ((sign_bits >> e) & 1u) ? -x[e] : x[e];
  // 3. unnormalized FWHT inside the segment, stages 1, 2, 4, ...
  segment_fwht<D>(u, sg, lane);
  // 4. codes: thresholds strictly below w
  const int nt = (1 << sg.bits) - 1;
  float c2[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    int c = 0;
    for (int k = 0; k < nt; ++k) {
      const float Tk = n * threshold(sg.bits, k);
      c += u[e] > Tk ? 1 : 0;
    }
    code[e] = n2 > 0.f ? c : 0;
    const float cv = centroid(sg.bits, code[e]);
    c2[e] = cv * cv;
  }
  // 5. norm correction
  const float cn2 = segment_tree_sum<D>(c2, sg);
  const float ratio = n / sqrtf(cn2);
  return n2 > 0.f ? f32_to_f16_rne(ratio) : (uint16_t)0;
}

// One workgroup per (page, KV head, role). FMT = FMT_TQ3 / FMT_TQ2 (uniform
// codes) or FMT_TQK (keys: permuted, three segments; values: TQ3).
template <int D, int FMT>
__global__ __launch_bounds__(256) void encode_tq_kernel(EncodeTqParams p) {
  constexpr int E = D / 64;
  constexpr int DL = D / 4;
  constexpr int BITS = FMT == FMT_TQ2 ? 2 : 3;     // uniform rows (TQK values are TQ3)
  constexpr int W = DL * 3 / 32;                    // words per lane of TQ3 and TQK tiles
  extern __shared__ float xs[];                     // [P][D] fp32, then codes [P][D] bytes
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int P = p.P, T = P / 16;
  const int role = blockIdx.x & 1;
  const int h = (blockIdx.x >> 1) % p.Hkv;
  const int64_t ip = (blockIdx.x >> 1) / p.Hkv;
  uint8_t *cb = (uint8_t *)(xs + P * D);
  const int dst = p.dst_page[ip];
  if (dst < 0 || dst >= p.pool_pages) return;
  int nvalid = P;
  if (p.page_valid) nvalid = min(max(p.page_valid[ip], 0), P);
  const bool grouped = FMT == FMT_TQK && role == 0;

  // stage the fp32 rows of this (page, head, role)
  if (p.src_kind == KVQ_SRC_F32_ROWS) {
    for (int t = tid; t < P * D; t += blockDim.x) {
      const int s = t / D, j = t % D;
      xs[t] = s < nvalid ? p.src_rows[(((ip * P + s) * p.Hkv + h) * 2 + role) * D + j] : 0.f;
    }
  } else {
    const int sp = p.src_page[ip];
    const bool ok = sp >= 0 && sp < p.fp8_pool_pages;
    const uint8_t *fh = p.fp8_pool + (int64_t)(ok ? sp : 0) * p.fp8_page_bytes + (int64_t)h * p.fp8_head_bytes;
    const float *sc = (const float *)(fh + 2LL * P * D + (int64_t)role * 4 * P);
    for (int t = tid; t < P * D; t += blockDim.x) {
      const int s = t / D, j = t % D;
      float x = 0.f;
      if (ok && s < nvalid) {
        const int tau = s / 16, t16 = s % 16;
        int lp, i;
        if (role == 0) { lp = t16 + 16 * (j / DL); i = j % DL; }
        else { lp = j % 16 + 16 * (t16 / 4); i = 4 * (j / 16) + t16 % 4; }
        const uint8_t byte = fh[(int64_t)(role * T + tau) * 16 * D + ((i / 16) * 64 + lp) * 16 + i % 16];
        const float2_t f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((uint32_t)byte, 1.0f, false);
        x = f[0] * sc[s];
      }
      xs[t] = x;
    }
  }
  __syncthreads();

  uint8_t *head = p.pool + (int64_t)dst * p.page_bytes + (int64_t)h * p.head_bytes;
  const int64_t tile_bytes = 16LL * D * BITS / 8;
  const uint32_t *sgw = p.signs + ((int64_t)h * 2 + role) * (D / 32);
  const int64_t sig0 = 2LL * T * tile_bytes;
  uint16_t *sig_out = (uint16_t *)(head + sig0 + (int64_t)role * (FMT == FMT_TQK ? 6 : 2) * P);

  Seg sg{0, 64, BITS, 0};
  int perm[E];
#pragma unroll
  for (int e = 0; e < E; ++e) perm[e] = E * lane + e;
  if (grouped) {
    sg.idx = lane < 16 ? 0 : (lane < 48 ? 1 : 2);
    sg.lane0 = sg.idx == 0 ? 0 : (sg.idx == 1 ? 16 : 48);
    sg.nl = sg.idx == 1 ? 32 : 16;
    sg.bits = 2 + sg.idx;
    const uint16_t *pm = p.tqk_perm + (int64_t)h * D;
#pragma unroll
    for (int e = 0; e < E; ++e) perm[e] = pm[E * lane + e] & (D - 1);
  }
  const int j0 = E * lane;
  const uint32_t sign_bits = (sgw[j0 >> 5] >> (j0 & 31)) & ((1u << E) - 1u);

  for (int s = wave; s < P; s += 4) {
    float x[E];
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = xs[s * D + perm[e]];
    int code[E];
    const uint16_t sig = tq_encode_segment<D>(x, sign_bits, sg, lane, code);
#pragma unroll
    for (int e = 0; e < E; ++e) cb[s * D + E * lane + e] = (uint8_t)code[e];
    if (lane == sg.lane0) sig_out[sg.idx * P + s] = sig;
  }
  __syncthreads();

  // pack every word of the role's tiles
  constexpr int WU = FMT == FMT_TQ2 ? DL * 2 / 32 : W;
  for (int t = tid; t < T * 64 * WU; t += blockDim.x) {
    const int tau = t / (64 * WU), r = t % (64 * WU), l = r / WU, w = r % WU;
    auto code_of = [&](int i) -> uint32_t {
      int tok, dim;
      if (grouped) { tok = 16 * tau + (l & 15); dim = 32 * (i >> 3) + 8 * (l >> 4) + (i & 7); }
      else if (role == 0) { tok = 16 * tau + (l & 15); dim = (l >> 4) * DL + i; }
      else { tok = 16 * tau + 4 * (l >> 4) + (i & 3); dim = (l & 15) + 16 * (i >> 2); }
      return cb[tok * D + dim];
    };
    uint32_t word = 0;
#pragma unroll
    for (int s8 = 0; s8 < 4; ++s8) {
      uint32_t byte;
      const int m = w / 3, pp = w % 3;
      auto c = [&](int g) { return code_of(4 * g + s8); };
      if (grouped) {
        constexpr int n2 = D / 64, n3 = D / 32;
        if (pp == 0) byte = c(n2 + n3 + 2 * m) | (c(n2 + n3 + 2 * m + 1) << 4);
        else if (pp == 1) byte = c(n2 + 4 * m) | (c(n2 + 4 * m + 1) << 3) | (c(2 * m) << 6);
        else byte = c(n2 + 4 * m + 2) | (c(n2 + 4 * m + 3) << 3) | (c(2 * m + 1) << 6);
      } else if constexpr (BITS == 3) {
        auto c3 = [&](int q) { return c(8 * m + q); };
        if (pp == 0) byte = c3(0) | (c3(1) << 3) | ((c3(6) & 3u) << 6);
        else if (pp == 1) byte = c3(2) | (c3(3) << 3) | ((c3(7) & 3u) << 6);
        else byte = c3(4) | (c3(5) << 3) | ((c3(6) >> 2) << 6) | ((c3(7) >> 2) << 7);
      } else {
        byte = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) byte |= c(4 * w + k) << (2 * k);
      }
      word |= (byte & 255u) << (8 * s8);
    }
    *(uint32_t *)(head + (int64_t)(role * T + tau) * tile_bytes + tile_word_offset<D>(l, w, WU)) = word;
  }
}


// ------------------------------------------------------------------------
// Promote (Minima-KV algorithm 1 "Promote", figure 2): a compressed page is
// rebuilt in fp32 and written as a new FP8 page. One workgroup per (page, KV
// head, role). The rebuild is the TQ decode x = sigma * s (.) FWHT(c) / sqrt(d_s)
// in this order: centroids (exact), unnormalized FWHT (every partial sum is a
// multiple of 2^-13 below 2^23, so exact in any order), u = fp32(F * r) with
// r the fp32 value nearest 1/sqrt(d_s), x = fp32(sigma * u), then the sign
// flip; grouped keys per segment, the permutation undone on the way to LDS.
// ------------------------------------------------------------------------
__device__ __forceinline__ float inv_sqrt_width(int ds) {
  // fp32 values nearest 1/sqrt(32), 1/8, 1/sqrt(128), 1/16
  return ds == 32 ? 0x1.6a09e6p-3f : (ds == 64 ? 0x1p-3f : (ds == 128 ? 0x1.6a09e6p-4f : 0x1p-4f));
}

template <int D, int FMT>
__global__ __launch_bounds__(256) void promote_fp8_kernel(PromoteParams p) {
  constexpr int E = D / 64;
  constexpr int DL = D / 4;
  constexpr int BITS = FMT == FMT_TQ2 ? 2 : 3;
  constexpr int WU = FMT == FMT_TQ2 ? DL * 2 / 32 : DL * 3 / 32;   // words per lane of a tile
  constexpr int GW = FMT == FMT_TQ2 ? 1 : 3;                        // words read together
  constexpr int NG = WU / GW;
  extern __shared__ float xs[];                     // [P][D] fp32 rows, then codes [P][D] bytes
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int P = p.P, T = P / 16;
  const int role = blockIdx.x & 1;
  const int h = (blockIdx.x >> 1) % p.Hkv;
  const int64_t ip = (blockIdx.x >> 1) / p.Hkv;
  const int src = p.src_page[ip], dst = p.dst_page[ip];
  if (src < 0 || src >= p.src_pool_pages || dst < 0 || dst >= p.fp8_pool_pages) return;   // whole workgroup
  uint8_t *cb = (uint8_t *)(xs + P * D);
  const bool grouped = FMT == FMT_TQK && role == 0;
  const uint8_t *sh = p.src_pool + (int64_t)src * p.src_page_bytes + (int64_t)h * p.src_head_bytes;
  const int64_t tile_bytes = 16LL * D * BITS / 8;

  // 1. codes of the role's tiles into cb[token][dim] (dim in stored order:
  //    permuted for grouped keys); the inverse of the encoder's packing
  for (int t = tid; t < T * 64 * NG; t += blockDim.x) {
    const int tau = t / (64 * NG), r = t % (64 * NG), l = r / NG, m = r % NG;
    const uint8_t *tile = sh + (int64_t)(role * T + tau) * tile_bytes;
    uint32_t wd[GW];
#pragma unroll
    for (int k = 0; k < GW; ++k) wd[k] = *(const uint32_t *)(tile + tile_word_offset<D>(l, GW * m + k, WU));
#pragma unroll
    for (int s8 = 0; s8 < 4; ++s8) {
      auto put = [&](int g, uint32_t code) {
        const int i = 4 * g + s8;
        int tok, dim;
        if (grouped) { tok = 16 * tau + (l & 15); dim = 32 * (i >> 3) + 8 * (l >> 4) + (i & 7); }
        else if (role == 0) { tok = 16 * tau + (l & 15); dim = (l >> 4) * DL + i; }
        else { tok = 16 * tau + 4 * (l >> 4) + (i & 3); dim = (l & 15) + 16 * (i >> 2); }
        cb[tok * D + dim] = (uint8_t)code;
      };
      if constexpr (GW == 3) {
        const uint32_t b0 = (wd[0] >> (8 * s8)) & 255u, b1 = (wd[1] >> (8 * s8)) & 255u,
                       b2 = (wd[2] >> (8 * s8)) & 255u;
        if (grouped) {
          constexpr int n2 = D / 64, n3 = D / 32;
          put(n2 + n3 + 2 * m, b0 & 15u);
          put(n2 + n3 + 2 * m + 1, b0 >> 4);
          put(n2 + 4 * m, b1 & 7u);
          put(n2 + 4 * m + 1, (b1 >> 3) & 7u);
          put(2 * m, b1 >> 6);
          put(n2 + 4 * m + 2, b2 & 7u);
          put(n2 + 4 * m + 3, (b2 >> 3) & 7u);
          put(2 * m + 1, b2 >> 6);
        } else {
          put(8 * m + 0, b0 & 7u);
          put(8 * m + 1, (b0 >> 3) & 7u);
          put(8 * m + 2, b1 & 7u);
          put(8 * m + 3, (b1 >> 3) & 7u);
          put(8 * m + 4, b2 & 7u);
          put(8 * m + 5, (b2 >> 3) & 7u);
          put(8 * m + 6, (b0 >> 6) | (((b2 >> 6) & 1u) << 2));
          put(8 * m + 7, (b1 >> 6) | (((b2 >> 7) & 1u) << 2));
        }
      } else {
        const uint32_t b = (wd[0] >> (8 * s8)) & 255u;
#pragma unroll
        for (int k = 0; k < 4; ++k) put(4 * m + k, (b >> (2 * k)) & 3u);
      }
    }
  }
  __syncthreads();

  // 2. rebuild each token's row in fp32 (one wave per token), natural order into LDS
  const uint16_t *sig_in = (const uint16_t *)(sh + 2LL * T * tile_bytes + (int64_t)role * (FMT == FMT_TQK ? 6 : 2) * P);
  const uint32_t *sgw = p.signs + ((int64_t)h * 2 + role) * (D / 32);
  Seg sg{0, 64, BITS, 0};
  int perm[E];
#pragma unroll
  for (int e = 0; e < E; ++e) perm[e] = E * lane + e;
  if (grouped) {
    sg.idx = lane < 16 ? 0 : (lane < 48 ? 1 : 2);
    sg.lane0 = sg.idx == 0 ? 0 : (sg.idx == 1 ? 16 : 48);
    sg.nl = sg.idx == 1 ? 32 : 16;
    sg.bits = 2 + sg.idx;
    const uint16_t *pm = p.tqk_perm + (int64_t)h * D;
#pragma unroll
    for (int e = 0; e < E; ++e) perm[e] = pm[E * lane + e] & (D - 1);
  }
  const int j0 = E * lane;
  const uint32_t sign_bits = (sgw[j0 >> 5] >> (j0 & 31)) & ((1u << E) - 1u);
  const float r = inv_sqrt_width(E * sg.nl);
  for (int s = wave; s < P; s += 4) {
    float u[E];
#pragma unroll
    for (int e = 0; e < E; ++e) u[e] = centroid(sg.bits, cb[s * D + E * lane + e]);
    segment_fwht<D>(u, sg, lane);
    const float sigma = (float)__builtin_bit_cast(_Float16, sig_in[sg.idx * P + s]);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float x = sigma * (u[e] * r);
      xs[s * D + perm[e]] = ((sign_bits >> e) & 1u) ? -x : x;
    }
  }
  __syncthreads();

  // 3. FP8 append of the rebuilt rows
  uint8_t *head = p.fp8_pool + (int64_t)dst * p.fp8_page_bytes + (int64_t)h * p.fp8_head_bytes;
  for (int s = wave; s < P; s += 4) {
    float x[E];
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = xs[s * D + E * lane + e];
    fp8_store_vector<D>(x, vector_amax<D>(x), head, P, role, s, lane);
  }
}

}  // namespace

hipError_t launch_encode_fp8(const EncodeFp8Params &p, int d, int src_is_bf16, hipStream_t s) {
  const int64_t nvec = p.n_tok * p.Hkv * 2;
  if (nvec <= 0) return hipSuccess;
  const dim3 grid((unsigned)((nvec + 3) / 4));
  if (d == 256) {
    if (src_is_bf16) hipLaunchKernelGGL((encode_fp8_kernel<256, true>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((encode_fp8_kernel<256, false>), grid, dim3(256), 0, s, p);
  } else {
    if (src_is_bf16) hipLaunchKernelGGL((encode_fp8_kernel<128, true>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((encode_fp8_kernel<128, false>), grid, dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_encode_tq(const EncodeTqParams &p, int d, int fmt, hipStream_t s) {
  const int64_t nwg = p.n_pages * p.Hkv * 2;
  if (nwg <= 0) return hipSuccess;
  const size_t lds = (size_t)p.P * d * 4 + (size_t)p.P * d;
  const dim3 grid((unsigned)nwg);
  if (d == 256) {
    if (fmt == FMT_TQ3) hipLaunchKernelGGL((encode_tq_kernel<256, FMT_TQ3>), grid, dim3(256), lds, s, p);
    else if (fmt == FMT_TQ2) hipLaunchKernelGGL((encode_tq_kernel<256, FMT_TQ2>), grid, dim3(256), lds, s, p);
    else return hipErrorInvalidValue;
  } else {
    if (fmt == FMT_TQ3) hipLaunchKernelGGL((encode_tq_kernel<128, FMT_TQ3>), grid, dim3(256), lds, s, p);
    else if (fmt == FMT_TQ2) hipLaunchKernelGGL((encode_tq_kernel<128, FMT_TQ2>), grid, dim3(256), lds, s, p);
    else hipLaunchKernelGGL((encode_tq_kernel<128, FMT_TQK>), grid, dim3(256), lds, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_promote_fp8(const PromoteParams &p, int d, int fmt, hipStream_t s) {
  const int64_t nwg = p.n_pages * p.Hkv * 2;
  if (nwg <= 0) return hipSuccess;
  const size_t lds = (size_t)p.P * d * 4 + (size_t)p.P * d;
  const dim3 grid((unsigned)nwg);
  if (d == 256) {
    if (fmt == FMT_TQ3) hipLaunchKernelGGL((promote_fp8_kernel<256, FMT_TQ3>), grid, dim3(256), lds, s, p);
    else if (fmt == FMT_TQ2) hipLaunchKernelGGL((promote_fp8_kernel<256, FMT_TQ2>), grid, dim3(256), lds, s, p);
    else return hipErrorInvalidValue;
  } else {
    if (fmt == FMT_TQ3) hipLaunchKernelGGL((promote_fp8_kernel<128, FMT_TQ3>), grid, dim3(256), lds, s, p);
    else if (fmt == FMT_TQ2) hipLaunchKernelGGL((promote_fp8_kernel<128, FMT_TQ2>), grid, dim3(256), lds, s, p);
    else hipLaunchKernelGGL((promote_fp8_kernel<128, FMT_TQK>), grid, dim3(256), lds, s, p);
  }
  return hipGetLastError();
}

}  // namespace kvq
