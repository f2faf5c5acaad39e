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

#include "codebook.h"
#include "kvq_internal.h"
#include "lane_ops.h"

#pragma clang fp contract(off)

namespace kvq {
namespace {

typedef float float2_t __attribute__((ext_vector_type(2)));

// Centroids (fp16 values, exactly representable in fp32), ascending codes
// (the grouped-key promotion decodes through these; the encoders count
// thresholds with the level books below).
__constant__ float kCb3[8] = {-2.15234375f, -1.34375f, -0.755859375f, -0.2451171875f,
                              0.2451171875f, 0.755859375f, 1.34375f, 2.15234375f};
__constant__ float kCb2[4] = {-1.5107421875f, -0.452880859375f, 0.452880859375f, 1.5107421875f};
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

// A vector's four (D = 256) or two (D = 128) codes per lane, packed as
// v_cvt_pk_fp8_f32 leaves them, and its scale.
struct Fp8Codes {
  uint32_t packed;
  float scale;
};
template <int D>
__device__ __forceinline__ Fp8Codes fp8_encode_vector(const float (&x)[D / 64], float amax) {
  constexpr int E = D / 64;
  Fp8Codes c{0u, 0.f};
  if (amax > 0.f) {
    const float inv = 448.0f / amax;
    float y[E];
#pragma unroll
    for (int e = 0; e < E; ++e) y[e] = x[e] * inv;
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
    if constexpr (E == 4) w = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w, true);
    c.packed = (uint32_t)w;
    c.scale = amax / 448.0f;
  }
  return c;
}

// One vector's codes into `slot` of its role's tiles (K: four bytes a lane,
// V: one byte per coordinate, the V tile being token-minor), and its scale.
template <int D>
__device__ __forceinline__ void fp8_store_codes(const Fp8Codes &c, uint8_t *head, int P, int role, int slot,
                                                int lane) {
  constexpr int E = D / 64;          // elements per lane
  constexpr int DL = D / 4;
  const int T = P / 16, tau = slot / 16, t16 = slot % 16;
  const int j0 = E * lane;
  if (role == 0) {
    uint8_t *tile = head + (int64_t)tau * 16 * D;
    const int lp = t16 + 16 * (j0 / DL), i = j0 % DL;
    uint8_t *dst = tile + ((i / 16) * 64 + lp) * 16 + i % 16;
    if constexpr (E == 4) *(uint32_t *)dst = c.packed;
    else *(uint16_t *)dst = (uint16_t)c.packed;
  } else {
    uint8_t *tile = head + (int64_t)(T + tau) * 16 * D;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int j = j0 + e;
      const int lp = j % 16 + 16 * (t16 / 4), i = 4 * (j / 16) + t16 % 4;
      tile[((i / 16) * 64 + lp) * 16 + i % 16] = (uint8_t)(c.packed >> (8 * e));
    }
  }
  if (lane == 0) *(float *)(head + 2LL * P * D + (int64_t)role * 4 * P + 4 * slot) = c.scale;
}

template <int D>
__device__ __forceinline__ void fp8_store_vector(const float (&x)[D / 64], float amax, uint8_t *head, int P, int role,
                                                 int slot, int lane) {
  fp8_store_codes<D>(fp8_encode_vector<D>(x, amax), head, P, role, slot, lane);
}

// ------------------------------------------------------------------------
// FP8 append: one wave per (group of four consecutive tokens, KV head,
// role). The four V vectors of slots 4m .. 4m + 3 of one page put their
// codes of coordinate j into four adjacent bytes of the V tile, so such a
// group is stored as one word per coordinate instead of one byte.
// ------------------------------------------------------------------------
constexpr int kFp8Group = 4;
template <int D, bool BF16>
__global__ __launch_bounds__(256) void encode_fp8_kernel(EncodeFp8Params p) {
  constexpr int E = D / 64;          // elements per lane
  constexpr int R = kFp8Group;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t w = (int64_t)blockIdx.x * 4 + wave;        // ((group, head), role)
  const int64_t n_groups = (p.n_tok + R - 1) / R;
  if (w >= n_groups * p.Hkv * 2) return;
  const int role = (int)(w & 1);
  const int64_t gh = w >> 1;
  const int64_t grp = gh / p.Hkv;
  const int h = (int)(gh - grp * p.Hkv);
  const int64_t t0 = grp * R;
  const int nt = (int)(p.n_tok - t0 < R ? p.n_tok - t0 : R);
  // the group's rows (a token past the end rereads the first, not stored)
  // and their destinations, all requested before any row is reduced
  float x[R][E];
  int pid[R], slot[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t tk = t0 + (r < nt ? r : 0);
    const int64_t row = ((tk * p.Hkv + h) * 2 + role) * D + (int64_t)E * lane;
    if constexpr (BF16) {
      const uint16_t *s = (const uint16_t *)p.src + row;
#pragma unroll
      for (int e = 0; e < E; ++e) x[r][e] = __builtin_bit_cast(float, (uint32_t)s[e] << 16);
    } else {
      const float *s = (const float *)p.src + row;
#pragma unroll
      for (int e = 0; e < E; ++e) x[r][e] = s[e];
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t tk = t0 + (r < nt ? r : 0);
    pid[r] = p.dst_page[tk];
    slot[r] = p.dst_slot[tk];
  }
  Fp8Codes c[R];
#pragma unroll
  for (int r = 0; r < R; ++r) c[r] = fp8_encode_vector<D>(x[r], vector_amax<D>(x[r]));
  auto ok = [&](int r) { return pid[r] >= 0 && pid[r] < p.pool_pages && slot[r] >= 0 && slot[r] < p.P; };
  bool grouped = role == 1 && nt == R && ok(0) && slot[0] % R == 0;
#pragma unroll
  for (int r = 1; r < R; ++r) grouped = grouped && pid[r] == pid[0] && slot[r] == slot[0] + r;
  if (grouped) {
    uint8_t *head = p.pool + (int64_t)pid[0] * p.page_bytes + (int64_t)h * p.head_bytes;
    const int T = p.P / 16, tau = slot[0] / 16, q4 = (slot[0] % 16) / 4;
    uint8_t *tile = head + (int64_t)(T + tau) * 16 * D;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int j = E * lane + e;
      const int lp = j % 16 + 16 * q4, i = 4 * (j / 16);
      uint32_t word = 0;
#pragma unroll
      for (int r = 0; r < R; ++r) word |= ((c[r].packed >> (8 * e)) & 255u) << (8 * r);
      *(uint32_t *)(tile + ((i / 16) * 64 + lp) * 16 + i % 16) = word;
    }
    if (lane < R) {
      const float sc = lane == 0 ? c[0].scale : lane == 1 ? c[1].scale : lane == 2 ? c[2].scale : c[3].scale;
      *(float *)(head + 2LL * p.P * D + 4LL * p.P + 4 * (slot[0] + lane)) = sc;
    }
    return;
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (r >= nt || !ok(r)) continue;                        // the whole wave
    uint8_t *head = p.pool + (int64_t)pid[r] * p.page_bytes + (int64_t)h * p.head_bytes;
    fp8_store_codes<D>(c[r], head, p.P, role, slot[r], lane);
  }
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

__device__ __forceinline__ float centroid(int bits, int c) {
  return bits == 2 ? kCb2[c] : (bits == 3 ? kCb3[c] : kCb4[c]);
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

// ------------------------------------------------------------------------
// Register-resident TQ encoder for the uniform formats (TQ3, TQ2): one wave
// per 16-token tile of one role of one (page, KV head). The FP8 tile and the
// TQ tile deal a tile to the 64 lanes the same way (K: lane l holds token
// l%16, dims (l/16) DL + i; V: lane l holds tokens 4 (l/16) + i%4, dims
// l%16 + 16 (i/4); DL = d/4 elements per lane), so every lane reads, encodes
// and writes its own elements: no LDS, no barrier. The definition's fixed
// orders are kept exactly:
//  * the halving-tree sums pair the same elements in the same order: in the
//    K layout the first stages pair lanes (a permlane swap per stage that
//    also halves the values each lane keeps), the last ones run in-lane or
//    as lane butterflies, which give the tree's value in every lane;
//  * the butterfly FWHT runs its stages 1, 2, 4, ... in order, in-lane where
//    the partner is in the lane and across lanes otherwise; an upper partner
//    computes a - b as fma(b, -1, a), one rounding like the subtraction;
//  * the sign flip of s * x is done on the FP8 bytes (bit 7) before they are
//    widened: fp32(-v * scale) = -fp32(v * scale), and the norm squares x.
// Codes count the thresholds strictly below w: with a = |w|, w > 0 gives
// 2^(b-1) + #{k : a > T_k} and w <= 0 gives 2^(b-1) - 1 - #{k : a >= T_k}
// (T_k the positive thresholds, T_-k = -T_k exactly), and a >= T is
// nextup(a) > T for a >= 0, so one comparison chain serves both signs.
// ------------------------------------------------------------------------

// Halving-tree sum of the D values of a K-layout token (DL in each of the
// lanes r, r + 16, r + 32, r + 48); every lane gets the total. Stage h = D/2
// pairs lanes 32 apart, h = D/4 lanes 16 apart, and so on alternately; each
// of the first log2(DL) stages keeps half of the lane's values (lower lanes
// the first half), the last two are butterflies.
template <int DL>
__device__ __forceinline__ float ktree_sum(float (&t)[DL]) {
  int st = 0;
#pragma unroll
  for (int n = DL; n > 1; n >>= 1, ++st) {
    const int half = n / 2;
#pragma unroll
    for (int e = 0; e < half; ++e) {
      float d, s;
      if ((st & 1) == 0) lane_swap<32>(t[e], t[e + half], d, s);
      else lane_swap<16>(t[e], t[e + half], d, s);
      t[e] = d + s;
    }
  }
#pragma unroll
  for (int k = 0; k < 2; ++k, ++st) {
    float d, s;
    if ((st & 1) == 0) lane_swap<32>(t[0], t[0], d, s);
    else lane_swap<16>(t[0], t[0], d, s);
    t[0] = d + s;
  }
  return t[0];
}

// Halving-tree sums of the four V-layout tokens of a lane (token tt = element
// i % 4, dims l%16 + 16 (i/4)): stages D/2 .. 16 in-lane, then 8, 4, 2, 1 as
// lane butterflies inside the 16-lane row; every lane of the row gets them.
template <int DL>
__device__ __forceinline__ void vtree_sum(const float (&t)[DL], float (&out)[4], int lane) {
  constexpr int K = DL / 4;
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    float u[K];
#pragma unroll
    for (int k = 0; k < K; ++k) u[k] = t[4 * k + tt];
#pragma unroll
    for (int hk = K / 2; hk >= 1; hk >>= 1)
#pragma unroll
      for (int k = 0; k < hk; ++k) u[k] = u[k] + u[k + hk];
    float v = u[0];
    v = v + lane_xor<8>(v, lane);
    v = v + lane_xor<4>(v, lane);
    v = v + lane_xor<2>(v, lane);
    v = v + lane_xor<1>(v, lane);
    out[tt] = v;
  }
}

// Unnormalized FWHT of K-layout rows: stages 1 .. DL/2 in-lane, DL across
// lanes 16 apart, 2 DL across lanes 32 apart.
template <int DL>
__device__ __forceinline__ void kfwht(float (&x)[DL], int lane) {
#pragma unroll
  for (int h = 1; h < DL; h <<= 1)
#pragma unroll
    for (int i = 0; i < DL; ++i)
      if ((i & h) == 0) {
        const float a = x[i], b = x[i + h];
        x[i] = a + b;
        x[i + h] = a - b;
      }
  const float sg16 = (lane & 16) ? -1.0f : 1.0f, sg32 = (lane & 32) ? -1.0f : 1.0f;
#pragma unroll
  for (int i = 0; i < DL; ++i) x[i] = __builtin_fmaf(x[i], sg16, lane_xor_ds<16>(x[i], lane));
#pragma unroll
  for (int i = 0; i < DL; ++i) x[i] = __builtin_fmaf(x[i], sg32, lane_xor_ds<32>(x[i], lane));
}

// Unnormalized FWHT of V-layout rows: stages 1, 2, 4, 8 across lanes of a
// row, 16 .. D/2 in-lane (element i = 4 k + tt, dim l%16 + 16 k).
template <int DL>
__device__ __forceinline__ void vfwht(float (&x)[DL], int lane) {
  constexpr int K = DL / 4;
  const float s1 = (lane & 1) ? -1.0f : 1.0f, s2 = (lane & 2) ? -1.0f : 1.0f;
  const float s4 = (lane & 4) ? -1.0f : 1.0f, s8 = (lane & 8) ? -1.0f : 1.0f;
#pragma unroll
  for (int i = 0; i < DL; ++i) x[i] = __builtin_fmaf(x[i], s1, lane_xor_ds<1>(x[i], lane));
#pragma unroll
  for (int i = 0; i < DL; ++i) x[i] = __builtin_fmaf(x[i], s2, lane_xor_ds<2>(x[i], lane));
#pragma unroll
  for (int i = 0; i < DL; ++i) x[i] = __builtin_fmaf(x[i], s4, lane_xor_ds<4>(x[i], lane));
#pragma unroll
  for (int i = 0; i < DL; ++i) x[i] = __builtin_fmaf(x[i], s8, lane_xor_ds<8>(x[i], lane));
#pragma unroll
  for (int hk = 1; hk < K; hk <<= 1)
#pragma unroll
    for (int k = 0; k < K; ++k)
      if ((k & hk) == 0)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          const int i = 4 * k + tt, j = 4 * (k + hk) + tt;
          const float a = x[i], b = x[j];
          x[i] = a + b;
          x[j] = a - b;
        }
}

// Positive nonzero thresholds (ascending) and the squared centroids by
// magnitude index m of an L-level codebook (L = 4: TQ2, 8: TQ3, 5 and 6: the
// fractional levels, 16: the 4-bit segment of grouped keys). With m = #{k : |w| beats T_k} (see quantize), the code
// is L/2 + m for w > 0, and L/2 - m (odd L) or L/2 - 1 - m (even L) else.
template <int L>
struct LevelBook;
template <>
struct LevelBook<8> {
  static constexpr int NT = 3;
  static constexpr float t[3] = {0.50048828125f, 1.0498046875f, 1.748046875f};
  static constexpr float c2[4] = {0.2451171875f * 0.2451171875f, 0.755859375f * 0.755859375f,
                                  1.34375f * 1.34375f, 2.15234375f * 2.15234375f};
};
template <>
struct LevelBook<4> {
  static constexpr int NT = 1;
  static constexpr float t[1] = {0.9818115234375f};
  static constexpr float c2[2] = {0.452880859375f * 0.452880859375f, 1.5107421875f * 1.5107421875f};
};
template <>
struct LevelBook<5> {
  static constexpr int NT = 2;
  static constexpr float t[2] = {0.38232421875f, 1.24462890625f};
  static constexpr float c2[3] = {0.0f, 0.7646484375f * 0.7646484375f, 1.724609375f * 1.724609375f};
};
template <>
struct LevelBook<6> {
  static constexpr int NT = 2;
  static constexpr float t[2] = {0.6588134765625f, 1.44677734375f};
  static constexpr float c2[3] = {0.317626953125f * 0.317626953125f, 1.0f, 1.8935546875f * 1.8935546875f};
};

template <>
struct LevelBook<16> {
  static constexpr int NT = 7;
  static constexpr float t[7] = {0.2581787109375f, 0.5223388671875f, 0.799560546875f, 1.09912109375f,
                                 1.43701171875f, 1.84326171875f, 2.400390625f};
  static constexpr float c2[8] = {0.12841796875f * 0.12841796875f, 0.387939453125f * 0.387939453125f,
                                  0.65673828125f * 0.65673828125f, 0.9423828125f * 0.9423828125f,
                                  1.255859375f * 1.255859375f, 1.6181640625f * 1.6181640625f,
                                  2.068359375f * 2.068359375f, 2.732421875f * 2.732421875f};
};

// Code of one rotated coordinate w against the norm-scaled positive
// thresholds T (ascending), and the square of its centroid.
template <int L>
__device__ __forceinline__ uint32_t quantize(float w, const float *T, float &cc) {
  using B = LevelBook<L>;
  const bool pos = w > 0.0f;
  // |w|, one ulp up unless w > 0 (the bits plus a carry of !pos)
  const float ap = __builtin_bit_cast(float, (__builtin_bit_cast(uint32_t, w) & 0x7FFFFFFFu) + (pos ? 0u : 1u));
  uint32_t m = 0;
  cc = B::c2[0];
#pragma unroll
  for (int j = 0; j < B::NT; ++j) {
    const bool gt = ap > T[j];
    m += gt ? 1u : 0u;
    cc = gt ? B::c2[j + 1] : cc;
  }
  constexpr uint32_t H = L / 2;
  if constexpr ((L & (L - 1)) == 0) {
    // H a power of two and m < H: H + m = m ^ H and H - 1 - m = m ^ (H - 1)
    return m ^ (pos ? H : H - 1u);
  } else {
    return pos ? H + m : ((L & 1) ? H - m : H - 1u - m);
  }
}

// Four codes per group word (element 4 q + j in byte j) -> the lane's packed
// words in the tile's bit rule, stored to the lane's regions of the tile.
template <int D, int BITS>
__device__ __forceinline__ void store_codes(uint8_t *tile, const uint32_t (&G)[D / 16], int lane) {
  constexpr int NG = D / 16;   // groups of four elements per lane
  if constexpr (BITS == 3) {
    constexpr int NWD = 3 * NG / 8;
    uint32_t w[NWD];
#pragma unroll
    for (int m = 0; m < NG / 8; ++m) {
      const uint32_t *q = G + 8 * m;
      w[3 * m] = q[0] | (q[1] << 3) | ((q[6] & 0x03030303u) << 6);
      w[3 * m + 1] = q[2] | (q[3] << 3) | ((q[7] & 0x03030303u) << 6);
      w[3 * m + 2] = q[4] | (q[5] << 3) | (((q[6] >> 2) & 0x01010101u) << 6) | (((q[7] >> 2) & 0x01010101u) << 7);
    }
    if constexpr (NWD == 6) {
      *(uint4 *)(tile + lane * 16) = make_uint4(w[0], w[1], w[2], w[3]);
      *(uint2 *)(tile + 1024 + lane * 8) = make_uint2(w[4], w[5]);
    } else {
      *(uint2 *)(tile + lane * 8) = make_uint2(w[0], w[1]);
      *(uint32_t *)(tile + 512 + lane * 4) = w[2];
    }
  } else {
    constexpr int NWD = NG / 4;
    uint32_t w[NWD];
#pragma unroll
    for (int k = 0; k < NWD; ++k)
      w[k] = G[4 * k] | (G[4 * k + 1] << 2) | (G[4 * k + 2] << 4) | (G[4 * k + 3] << 6);
    if constexpr (NWD == 4) *(uint4 *)(tile + lane * 16) = make_uint4(w[0], w[1], w[2], w[3]);
    else *(uint2 *)(tile + lane * 8) = make_uint2(w[0], w[1]);
  }
}

// Fractional-level output of one tile: the lane's code bytes go to LDS as
// [token][d]; each lane then builds mixed-radix groups (group j of row t =
// sum_i c_{kj+i} L^i, codes past d count 0) and ORs them into the row
// bitstreams staged in LDS (zeroed first); the wave writes the tile's 16 rows
// out as dwords. wl: the wave's LDS area, 16 d code bytes then the tile.
template <int D, int L, int ROLE>
__device__ __forceinline__ void store_rows(uint8_t *tile, const uint32_t (&G)[D / 16], int lane, uint8_t *wl) {
  constexpr int DL = D / 4, NG = D / 16;
  constexpr int K = tqf_group_codes(L), NB = tqf_group_bits(L);
  constexpr int NGR = (D + K - 1) / K, R = tqf_row_bytes(D, L), RT = 16 * R;
  uint8_t *codes = wl;
  uint32_t *rows = (uint32_t *)(wl + 16 * D);
  const int g = lane >> 4, r = lane & 15;
  if constexpr (ROLE == 0) {
#pragma unroll
    for (int c = 0; c < NG / 4; ++c)
      *(uint4 *)(codes + r * D + g * DL + 16 * c) = make_uint4(G[4 * c], G[4 * c + 1], G[4 * c + 2], G[4 * c + 3]);
  } else {
#pragma unroll
    for (int q = 0; q < NG; ++q)
#pragma unroll
      for (int j = 0; j < 4; ++j) codes[(4 * g + j) * D + r + 16 * q] = (uint8_t)(G[q] >> (8 * j));
  }
  for (int w = lane; w < RT / 4; w += 64) rows[w] = 0u;
  wave_lds_sync();
  for (int gi = lane; gi < 16 * NGR; gi += 64) {
    const int row = gi / NGR, grp = gi - row * NGR;
    uint32_t v = 0u;
#pragma unroll
    for (int i = K - 1; i >= 0; --i) {
      const int dim = K * grp + i;
      v = v * L + (dim < D ? (uint32_t)codes[row * D + dim] : 0u);
    }
    const int bit = row * R * 8 + grp * NB;
    atomicOr(rows + (bit >> 5), v << (bit & 31));
    if ((bit & 31) + NB > 32) atomicOr(rows + (bit >> 5) + 1, v >> (32 - (bit & 31)));
  }
  wave_lds_sync();
  for (int w = lane; w < RT / 4; w += 64) *(uint32_t *)(tile + 4 * w) = rows[w];
}

// Byte masks of the sign flips of a lane's elements (0x80 in byte j of word
// q when element 4 q + j is negated): K: the lane's DL consecutive dims;
// V: word q holds four tokens of dim l%16 + 16 q, one sign for the word.
template <int D, int ROLE>
__device__ __forceinline__ void sign_masks(const uint32_t *sgw, int lane, uint32_t (&mk)[D / 16]) {
  constexpr int DL = D / 4;
  const int g = lane >> 4, r = lane & 15;
#pragma unroll
  for (int q = 0; q < D / 16; ++q) {
    if constexpr (ROLE == 0) {
      const uint32_t bits = sgw[(g * DL + 4 * q) >> 5] >> ((4 * q) & 31);
      mk[q] = ((bits & 15u) * 0x10204080u) & 0x80808080u;
    } else {
      const uint32_t bit = (sgw[q >> 1] >> (r + 16 * (q & 1))) & 1u;
      mk[q] = (0u - bit) & 0x80808080u;
    }
  }
}

// Encode one tile (16 tokens) of one role of one (page, KV head) and store
// its codes and sigmas. nvalid = filled slots of the page; ok = the source is
// readable (else the rows are zero).
// KSIG: bytes per token of the key sigma region that precedes the value
// sigmas (2: one fp16; 6: the three segment sigmas of grouped keys).
template <int D, int L, int ROLE, bool FP8SRC, int KSIG = 2>
__device__ __forceinline__ void encode_tile(const EncodeTqParams &p, int64_t ip, int h, int tau, int nvalid, bool ok,
                                            uint8_t *head, int lane, uint8_t *wl) {
  constexpr int DL = D / 4, NG = D / 16;
  const int P = p.P, T = P / 16;
  const int g = lane >> 4, r = lane & 15;
  const uint32_t *sgw = p.signs + ((int64_t)h * 2 + ROLE) * (D / 32);
  float x[DL];
  if constexpr (FP8SRC) {
    const int sp = p.src_page[ip];
    const uint8_t *fh = p.fp8_pool + (int64_t)sp * p.fp8_page_bytes + (int64_t)h * p.fp8_head_bytes;
    const uint8_t *tile = fh + (int64_t)(ROLE * T + tau) * 16 * D;
    const float *scl = (const float *)(fh + 2LL * P * D + (int64_t)ROLE * 4 * P);
    uint32_t wv[NG];
    float s4[4];
    uint32_t keep = 0xFFFFFFFFu;      // byte mask of valid tokens (V: byte j = token 4g + j)
    if constexpr (ROLE == 0) {
      const bool valid = ok && 16 * tau + r < nvalid;
      s4[0] = valid ? scl[16 * tau + r] : 0.0f;
      keep = valid ? 0xFFFFFFFFu : 0u;
    } else {
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (ok) v = *(const float4 *)(scl + 16 * tau + 4 * g);
      const float vv[4] = {v.x, v.y, v.z, v.w};
      keep = 0u;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool valid = ok && 16 * tau + 4 * g + j < nvalid;
        s4[j] = valid ? vv[j] : 0.0f;
        keep |= valid ? (0xFFu << (8 * j)) : 0u;
      }
    }
#pragma unroll
    for (int c = 0; c < DL / 16; ++c) {
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (ok) v = *(const uint4 *)(tile + c * 1024 + lane * 16);
      wv[4 * c] = v.x; wv[4 * c + 1] = v.y; wv[4 * c + 2] = v.z; wv[4 * c + 3] = v.w;
    }
    uint32_t mk[NG];
    sign_masks<D, ROLE>(sgw, lane, mk);
#pragma unroll
    for (int q = 0; q < NG; ++q) {
      const uint32_t wq = (wv[q] & keep) ^ mk[q];
      const auto lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(wq, 1.0f, false);
      const auto hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(wq, 1.0f, true);
      x[4 * q] = lo[0] * s4[ROLE == 0 ? 0 : 0];
      x[4 * q + 1] = lo[1] * s4[ROLE == 0 ? 0 : 1];
      x[4 * q + 2] = hi[0] * s4[ROLE == 0 ? 0 : 2];
      x[4 * q + 3] = hi[1] * s4[ROLE == 0 ? 0 : 3];
    }
  } else {
    auto row = [&](int s) { return p.src_rows + (((ip * P + s) * p.Hkv + h) * 2 + ROLE) * D; };
    if constexpr (ROLE == 0) {
      const int s = 16 * tau + r;
      const bool valid = s < nvalid;
#pragma unroll
      for (int c = 0; c < DL / 4; ++c) {
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (valid) v = *(const float4 *)(row(s) + g * DL + 4 * c);
        x[4 * c] = v.x; x[4 * c + 1] = v.y; x[4 * c + 2] = v.z; x[4 * c + 3] = v.w;
      }
#pragma unroll
      for (int i = 0; i < DL; ++i) {
        const uint32_t bit = (sgw[(g * DL + i) >> 5] >> ((g * DL + i) & 31)) & 1u;
        x[i] = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, x[i]) ^ (bit << 31));
      }
    } else {
#pragma unroll
      for (int i = 0; i < DL; ++i) {
        const int s = 16 * tau + 4 * g + (i & 3), dim = r + 16 * (i >> 2);
        const float v = s < nvalid ? row(s)[dim] : 0.0f;
        const uint32_t bit = (sgw[dim >> 5] >> (dim & 31)) & 1u;
        x[i] = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, v) ^ (bit << 31));
      }
    }
  }

  // norms (halving trees of x^2; x carries the signs, which squaring drops)
  constexpr int NTK = ROLE == 0 ? 1 : 4;        // tokens per lane
  float n2[NTK];
  {
    float t[DL];
#pragma unroll
    for (int i = 0; i < DL; ++i) t[i] = x[i] * x[i];
    if constexpr (ROLE == 0) n2[0] = ktree_sum<DL>(t);
    else vtree_sum<DL>(t, n2, lane);
  }
  // rotation (x is s * x already)
  if constexpr (ROLE == 0) kfwht<DL>(x, lane);
  else vfwht<DL>(x, lane);
  // thresholds, codes, squared centroids
  constexpr int NT = LevelBook<L>::NT;
  float n[NTK], thr[NTK][NT];
#pragma unroll
  for (int k = 0; k < NTK; ++k) {
    n[k] = sqrtf(n2[k]);
#pragma unroll
    for (int j = 0; j < NT; ++j) thr[k][j] = n[k] * LevelBook<L>::t[j];
  }
  uint32_t G[NG];
  float cc[DL];
#pragma unroll
  for (int q = 0; q < NG; ++q) {
    uint32_t word = 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k = ROLE == 0 ? 0 : j;
      word |= quantize<L>(x[4 * q + j], thr[k], cc[4 * q + j]) << (8 * j);
    }
    // materialize the group's code word here: left to itself the compiler
    // computes every squared centroid first and keeps all the comparison
    // masks (SGPR pairs) alive for the codes, spilling them into VGPR lanes
    asm volatile("" : "+v"(word));
    G[q] = word;
  }
  float cn2[NTK];
  if constexpr (ROLE == 0) cn2[0] = ktree_sum<DL>(cc);
  else vtree_sum<DL>(cc, cn2, lane);
  uint16_t sig[NTK];
  uint32_t zero_mask = 0xFFFFFFFFu;               // zero vectors get codes 0
#pragma unroll
  for (int k = 0; k < NTK; ++k) {
    const bool nz = n2[k] > 0.0f;
    sig[k] = nz ? f32_to_f16_rne(n[k] / sqrtf(cn2[k])) : (uint16_t)0;
    if (!nz) zero_mask &= ROLE == 0 ? 0u : ~(0xFFu << (8 * k));
  }
#pragma unroll
  for (int q = 0; q < NG; ++q) G[q] &= zero_mask;

  constexpr bool FRAC = L == 5 || L == 6;
  const int64_t tile_bytes = FRAC ? 16LL * tqf_row_bytes(D, L) : 16LL * D * (L == 8 ? 3 : 2) / 8;
  if constexpr (FRAC) store_rows<D, L, ROLE>(head + (int64_t)(ROLE * T + tau) * tile_bytes, G, lane, wl);
  else store_codes<D, L == 8 ? 3 : 2>(head + (int64_t)(ROLE * T + tau) * tile_bytes, G, lane);
  uint16_t *so = (uint16_t *)(head + 2LL * T * tile_bytes + (int64_t)ROLE * KSIG * P);
  if constexpr (ROLE == 0) {
    if (g == 0) so[16 * tau + r] = sig[0];
  } else {
    if (r == 0)
      *(uint2 *)(so + 16 * tau + 4 * g) =
          make_uint2((uint32_t)sig[0] | ((uint32_t)sig[1] << 16), (uint32_t)sig[2] | ((uint32_t)sig[3] << 16));
  }
}

constexpr int kEncWaves = 4;   // waves (tiles) per encoder workgroup

// Wave w of the grid encodes tile tau of role `role` of KV head h of page ip,
// with tau fastest, then role, head and page (the waves of a workgroup read
// neighbouring tiles of one source page).
// LDS of the fractional-level output stage, per wave: 16 d code bytes, then
// the tile's rows (at most 16 x 85 bytes, rounded up to dwords).
__host__ __device__ constexpr int tqf_encode_wave_bytes(int D) { return 16 * D + 1376; }

template <int D, int L, bool FP8SRC>
__global__ __launch_bounds__(64 * kEncWaves) __attribute__((amdgpu_waves_per_eu(D == 256 ? 3 : 4))) void encode_tq_tiles_kernel(EncodeTqParams p) {
  extern __shared__ __align__(16) uint8_t enc_lds[];
  const int lane = threadIdx.x & 63;
  const int64_t wid = (int64_t)blockIdx.x * kEncWaves + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int T = p.P / 16;
  if (wid >= p.n_pages * p.Hkv * 2 * T) return;
  const int tau = (int)(wid % T);
  const int role = (int)((wid / T) & 1);
  const int h = (int)((wid / (2 * T)) % p.Hkv);
  const int64_t ip = wid / (2 * T * p.Hkv);
  const int dst = p.dst_page[ip];
  if (dst < 0 || dst >= p.pool_pages) return;      // the whole wave
  int nvalid = p.P;
  if (p.page_valid) nvalid = min(max(p.page_valid[ip], 0), p.P);
  bool ok = true;
  if constexpr (FP8SRC) {
    const int sp = p.src_page[ip];
    ok = sp >= 0 && sp < p.fp8_pool_pages;
  }
  uint8_t *head = p.pool + (int64_t)dst * p.page_bytes + (int64_t)h * p.head_bytes;
  uint8_t *wl = enc_lds + (threadIdx.x >> 6) * tqf_encode_wave_bytes(D);
  if (role == 0) encode_tile<D, L, 0, FP8SRC>(p, ip, h, tau, nvalid, ok, head, lane, wl);
  else encode_tile<D, L, 1, FP8SRC>(p, ip, h, tau, nvalid, ok, head, lane, wl);
}

// ------------------------------------------------------------------------
// Register-resident demotion to grouped mixed-rate keys (TQK, Block-GTQ
// appendix A.7, H.1-H.2; d = 128): one wave per 16-token tile, as for the
// uniform formats; value tiles are uniform TQ3 (encode_tile). A key tile's
// FP8 rows (lane l: token l % 16, dims 32 (l / 16) + i) pass once through the
// wave's LDS, and each lane reads back its token's permuted coordinates in
// the key tile's own order: chunk k holds coordinates 32 k + 8 (l / 16) + j,
// j < 8 (k = 0: the 2-bit segment, 1 and 2: the 3-bit one, 3: the 4-bit
// one). Each chunk is then a K-layout row of 8 values per lane, so the
// segment's halving-tree sums and FWHT keep the definition's orders through
// ktree_sum<8> and kfwht<8>; the 3-bit segment first adds (tree) or
// combines (FWHT, its last stage) its two chunks in-lane. Codes count the
// thresholds below each coordinate as in the uniform encoder (the tables are
// symmetric), and a segment of norm 0 gets codes 0 and sigma 0.
// ------------------------------------------------------------------------
template <bool FP8SRC>
__device__ __forceinline__ void encode_tqk_key_tile(const EncodeTqParams &p, int64_t ip, int h, int tau, int nvalid,
                                                    bool ok, uint8_t *head, int lane, float *xs) {
  // every product and sum rounds on its own, as in the definition (the
  // 3-bit segment's first tree stage adds two squares in-lane)
#pragma clang fp contract(off)
  constexpr int D = 128, DL = 32;
  const int P = p.P, T = P / 16;
  const int g = lane >> 4, r = lane & 15;
  const int s = 16 * tau + r;
  const bool valid = ok && s < nvalid;
  float x[DL];
  if constexpr (FP8SRC) {
    const int sp = p.src_page[ip];
    const uint8_t *fh = p.fp8_pool + (int64_t)sp * p.fp8_page_bytes + (int64_t)h * p.fp8_head_bytes;
    const uint8_t *tile = fh + (int64_t)tau * 16 * D;
    const float sc = valid ? ((const float *)(fh + 2LL * P * D))[s] : 0.0f;
    uint32_t wv[8];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (valid) v = *(const uint4 *)(tile + c * 1024 + lane * 16);
      wv[4 * c] = v.x; wv[4 * c + 1] = v.y; wv[4 * c + 2] = v.z; wv[4 * c + 3] = v.w;
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const auto lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(wv[q], 1.0f, false);
      const auto hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(wv[q], 1.0f, true);
      x[4 * q] = lo[0] * sc;
      x[4 * q + 1] = lo[1] * sc;
      x[4 * q + 2] = hi[0] * sc;
      x[4 * q + 3] = hi[1] * sc;
    }
  } else {
    const float *row = p.src_rows + (((ip * P + s) * p.Hkv + h) * 2) * D + g * DL;
#pragma unroll
    for (int c = 0; c < DL / 4; ++c) {
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (s < nvalid) v = *(const float4 *)(row + 4 * c);
      x[4 * c] = v.x; x[4 * c + 1] = v.y; x[4 * c + 2] = v.z; x[4 * c + 3] = v.w;
    }
  }
  // the token's row through LDS into the permuted order, with the sign flip
  // of each permuted coordinate
  float *xr = xs + r * D;
#pragma unroll
  for (int c = 0; c < DL / 4; ++c)
    *(float4 *)(xr + g * DL + 4 * c) = make_float4(x[4 * c], x[4 * c + 1], x[4 * c + 2], x[4 * c + 3]);
  wave_lds_sync();
  const uint32_t *pm = (const uint32_t *)(p.tqk_perm + (int64_t)h * D);
  const uint32_t *sgw = p.signs + (int64_t)h * 2 * (D / 32);
  float u[DL];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t sb = sgw[k] >> (8 * g);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const uint32_t pw = pm[(32 * k + 8 * g) / 2 + jj];
#pragma unroll
      for (int hlf = 0; hlf < 2; ++hlf) {
        const int j = 2 * jj + hlf;
        const float v = xr[(hlf ? (pw >> 16) : pw) & (D - 1)];
        u[8 * k + j] = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, v) ^ (((sb >> j) & 1u) << 31));
      }
    }
  }
  // segment norms (halving trees; the 3-bit segment adds its chunks first)
  float n2[3];
  {
    float t[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) t[j] = u[j] * u[j];
    n2[0] = ktree_sum<8>(t);
#pragma unroll
    for (int j = 0; j < 8; ++j) t[j] = u[8 + j] * u[8 + j] + u[16 + j] * u[16 + j];
    n2[1] = ktree_sum<8>(t);
#pragma unroll
    for (int j = 0; j < 8; ++j) t[j] = u[24 + j] * u[24 + j];
    n2[2] = ktree_sum<8>(t);
  }
  // rotation inside each segment, stages 1, 2, 4, ... (the 3-bit segment's
  // stage 32 pairs its two chunks, in-lane)
  {
    float c0[8], c1[8], c2v[8], c3[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) { c0[j] = u[j]; c1[j] = u[8 + j]; c2v[j] = u[16 + j]; c3[j] = u[24 + j]; }
    kfwht<8>(c0, lane);
    kfwht<8>(c1, lane);
    kfwht<8>(c2v, lane);
    kfwht<8>(c3, lane);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      u[j] = c0[j];
      u[8 + j] = c1[j] + c2v[j];
      u[16 + j] = c1[j] - c2v[j];
      u[24 + j] = c3[j];
    }
  }
  // codes, squared centroids, segment sigmas
  float n[3], th0[LevelBook<4>::NT], th1[LevelBook<8>::NT], th2[LevelBook<16>::NT];
#pragma unroll
  for (int k = 0; k < 3; ++k) n[k] = sqrtf(n2[k]);
#pragma unroll
  for (int j = 0; j < LevelBook<4>::NT; ++j) th0[j] = n[0] * LevelBook<4>::t[j];
#pragma unroll
  for (int j = 0; j < LevelBook<8>::NT; ++j) th1[j] = n[1] * LevelBook<8>::t[j];
#pragma unroll
  for (int j = 0; j < LevelBook<16>::NT; ++j) th2[j] = n[2] * LevelBook<16>::t[j];
  uint32_t cw[8];                                  // codes of elements 4 q .. 4 q + 3, one per byte
  float cc[DL];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    uint32_t word = 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = 4 * q + j;
      uint32_t c;
      if (i < 8) c = quantize<4>(u[i], th0, cc[i]);
      else if (i < 24) c = quantize<8>(u[i], th1, cc[i]);
      else c = quantize<16>(u[i], th2, cc[i]);
      word |= c << (8 * j);
    }
    asm volatile("" : "+v"(word));
    cw[q] = word;
  }
  float cn2[3];
  {
    float t[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) t[j] = cc[j];
    cn2[0] = ktree_sum<8>(t);
#pragma unroll
    for (int j = 0; j < 8; ++j) t[j] = cc[8 + j] + cc[16 + j];
    cn2[1] = ktree_sum<8>(t);
#pragma unroll
    for (int j = 0; j < 8; ++j) t[j] = cc[24 + j];
    cn2[2] = ktree_sum<8>(t);
  }
  uint16_t sig[3];
#pragma unroll
  for (int k = 0; k < 3; ++k) sig[k] = n2[k] > 0.0f ? f32_to_f16_rne(n[k] / sqrtf(cn2[k])) : (uint16_t)0;
  // zero segments get codes 0 (words 0-1: segment 0, 2-5: segment 1, 6-7: segment 2)
  const uint32_t z0 = n2[0] > 0.0f ? 0xFFFFFFFFu : 0u, z1 = n2[1] > 0.0f ? 0xFFFFFFFFu : 0u,
                 z2 = n2[2] > 0.0f ? 0xFFFFFFFFu : 0u;
  cw[0] &= z0; cw[1] &= z0;
  cw[2] &= z1; cw[3] &= z1; cw[4] &= z1; cw[5] &= z1;
  cw[6] &= z2; cw[7] &= z2;
  // the tile's words (byte s8 of each: element s8 of the groups named):
  // word 0 = 4-bit groups 6, 7; word 1 = 3-bit groups 2, 3 and 2-bit group 0;
  // word 2 = 3-bit groups 4, 5 and 2-bit group 1
  uint8_t *tile = head + (int64_t)tau * 16 * D * 3 / 8;
  *(uint2 *)(tile + lane * 8) = make_uint2(cw[6] | (cw[7] << 4), cw[2] | (cw[3] << 3) | (cw[0] << 6));
  *(uint32_t *)(tile + 512 + lane * 4) = cw[4] | (cw[5] << 3) | (cw[1] << 6);
  uint16_t *so = (uint16_t *)(head + 2LL * T * 16 * D * 3 / 8);
  if (g < 3) so[g * P + s] = sig[g];
}

template <bool FP8SRC>
__global__ __launch_bounds__(64 * kEncWaves) void encode_tqk_tiles_kernel(EncodeTqParams p) {
  extern __shared__ __align__(16) uint8_t enc_lds[];
  constexpr int D = 128;
  const int lane = threadIdx.x & 63;
  const int64_t wid = (int64_t)blockIdx.x * kEncWaves + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int T = p.P / 16;
  if (wid >= p.n_pages * p.Hkv * 2 * T) return;
  const int tau = (int)(wid % T);
  const int role = (int)((wid / T) & 1);
  const int h = (int)((wid / (2 * T)) % p.Hkv);
  const int64_t ip = wid / (2 * T * p.Hkv);
  const int dst = p.dst_page[ip];
  if (dst < 0 || dst >= p.pool_pages) return;      // the whole wave
  int nvalid = p.P;
  if (p.page_valid) nvalid = min(max(p.page_valid[ip], 0), p.P);
  bool ok = true;
  if constexpr (FP8SRC) {
    const int sp = p.src_page[ip];
    ok = sp >= 0 && sp < p.fp8_pool_pages;
  }
  uint8_t *head = p.pool + (int64_t)dst * p.page_bytes + (int64_t)h * p.head_bytes;
  if (role == 0) {
    float *xs = (float *)enc_lds + (threadIdx.x >> 6) * 16 * D;
    encode_tqk_key_tile<FP8SRC>(p, ip, h, tau, nvalid, ok, head, lane, xs);
  } else {
    encode_tile<D, 8, 1, FP8SRC, 6>(p, ip, h, tau, nvalid, ok, head, lane, nullptr);
  }
}

// ------------------------------------------------------------------------
// Register-resident promotion of uniform TQ tiles (TQ3, TQ2) to FP8: one
// wave per tile of one role of one (page, KV head), in the shared lane
// layout. Rebuild x = sigma * fp32(F * r) with F = FWHT(c[code]) (exact in
// fp32 whatever the order), then the FP8 codec of the Append path: amax over
// the token's row, inv = fp32(448 / amax), codes E4M3(x * inv), scale =
// amax / 448. The sign flip s * x is applied to the FP8 bytes (bit 7) after
// the conversion: E4M3(-y) = E4M3(y) with the sign bit set, zero included;
// an all-zero row keeps codes 0.
// ------------------------------------------------------------------------
template <int D, int BITS>
__device__ __forceinline__ void tq_tile_groups(const uint8_t *tile, int lane, uint32_t (&G)[D / 16]) {
  constexpr int NG = D / 16;
  if constexpr (BITS == 3) {
    constexpr int NWD = 3 * NG / 8;
    uint32_t w[NWD];
    if constexpr (NWD == 6) {
      const uint4 a = *(const uint4 *)(tile + lane * 16);
      const uint2 b = *(const uint2 *)(tile + 1024 + lane * 8);
      w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w; w[4] = b.x; w[5] = b.y;
    } else {
      const uint2 a = *(const uint2 *)(tile + lane * 8);
      w[0] = a.x; w[1] = a.y;
      w[2] = *(const uint32_t *)(tile + 512 + lane * 4);
    }
#pragma unroll
    for (int m = 0; m < NG / 8; ++m) {
      const uint32_t a = w[3 * m], b = w[3 * m + 1], c = w[3 * m + 2];
      uint32_t *q = G + 8 * m;
      q[0] = a & 0x07070707u;
      q[1] = (a >> 3) & 0x07070707u;
      q[2] = b & 0x07070707u;
      q[3] = (b >> 3) & 0x07070707u;
      q[4] = c & 0x07070707u;
      q[5] = (c >> 3) & 0x07070707u;
      q[6] = ((a >> 6) & 0x03030303u) | ((c >> 4) & 0x04040404u);
      q[7] = ((b >> 6) & 0x03030303u) | ((c >> 5) & 0x04040404u);
    }
  } else {
    constexpr int NWD = NG / 4;
    uint32_t w[NWD];
    if constexpr (NWD == 4) {
      const uint4 a = *(const uint4 *)(tile + lane * 16);
      w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    } else {
      const uint2 a = *(const uint2 *)(tile + lane * 8);
      w[0] = a.x; w[1] = a.y;
    }
#pragma unroll
    for (int g = 0; g < NG; ++g) G[g] = (w[g >> 2] >> (2 * (g & 3))) & 0x03030303u;
  }
}

// Codes of a fractional-level tile in the lane layout of role ROLE: the
// tile's rows are staged in the wave's LDS area wl (raw rows, then 16 d code
// bytes), split into codes there (row-major for keys, dim-major for values),
// and each lane reads its groups of four back as words.
template <int D, int L, int ROLE>
__device__ __forceinline__ void tqf_tile_groups(const uint8_t *tile, int lane, uint32_t (&G)[D / 16], uint8_t *wl) {
  constexpr int DL = D / 4, NG = D / 16, RT = 16 * tqf_row_bytes(D, L);
  uint32_t *raw = (uint32_t *)wl;
  uint8_t *codes = wl + 1376;
  for (int w = lane; w < RT / 4; w += 64) raw[w] = *(const uint32_t *)(tile + 4 * w);
  wave_lds_sync();
  tqf_unpack_tile<D, L, ROLE == 0>(raw, codes, ROLE == 0 ? D : 16, lane);
  wave_lds_sync();
  const int g = lane >> 4, r = lane & 15;
  if constexpr (ROLE == 0) {
#pragma unroll
    for (int c = 0; c < NG / 4; ++c) {
      const uint4 v = *(const uint4 *)(codes + r * D + g * DL + 16 * c);
      G[4 * c] = v.x; G[4 * c + 1] = v.y; G[4 * c + 2] = v.z; G[4 * c + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int q = 0; q < NG; ++q) G[q] = *(const uint32_t *)(codes + (r + 16 * q) * 16 + 4 * g);
  }
}

template <int D, int L, int ROLE>
__device__ __forceinline__ void promote_tile(const PromoteParams &p, const uint8_t *sh, uint8_t *fh, int h, int tau,
                                             int lane, uint8_t *wl) {
  constexpr int DL = D / 4, NG = D / 16;
  constexpr bool FRAC = L == 5 || L == 6;
  constexpr int BITS = L == 8 ? 3 : 2;
  const int P = p.P, T = P / 16;
  const int g = lane >> 4, r = lane & 15;
  const int64_t tile_bytes = FRAC ? 16LL * tqf_row_bytes(D, L) : 16LL * D * BITS / 8;
  uint32_t G[NG];
  if constexpr (FRAC) tqf_tile_groups<D, L, ROLE>(sh + (int64_t)(ROLE * T + tau) * tile_bytes, lane, G, wl);
  else tq_tile_groups<D, BITS>(sh + (int64_t)(ROLE * T + tau) * tile_bytes, lane, G);
  const uint16_t *si = (const uint16_t *)(sh + 2LL * T * tile_bytes + (int64_t)ROLE * 2 * P);
  constexpr int NTK = ROLE == 0 ? 1 : 4;
  float sig[NTK];
  if constexpr (ROLE == 0) {
    sig[0] = (float)__builtin_bit_cast(_Float16, si[16 * tau + r]);
  } else {
    const uint2 v = *(const uint2 *)(si + 16 * tau + 4 * g);
    sig[0] = (float)__builtin_bit_cast(_Float16, (uint16_t)(v.x & 0xFFFFu));
    sig[1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(v.x >> 16));
    sig[2] = (float)__builtin_bit_cast(_Float16, (uint16_t)(v.y & 0xFFFFu));
    sig[3] = (float)__builtin_bit_cast(_Float16, (uint16_t)(v.y >> 16));
  }
  float x[DL];
#pragma unroll
  for (int q = 0; q < NG; ++q) {
    uint2 hc;                                       // fp16 centroids of elements 4q .. 4q + 3
    if constexpr (FRAC) hc = decode_group_levels<L>(G[q]);
    else hc = decode_group<BITS>(G[q]);
    x[4 * q] = (float)__builtin_bit_cast(_Float16, (uint16_t)(hc.x & 0xFFFFu));
    x[4 * q + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(hc.x >> 16));
    x[4 * q + 2] = (float)__builtin_bit_cast(_Float16, (uint16_t)(hc.y & 0xFFFFu));
    x[4 * q + 3] = (float)__builtin_bit_cast(_Float16, (uint16_t)(hc.y >> 16));
  }
  if constexpr (ROLE == 0) kfwht<DL>(x, lane);
  else vfwht<DL>(x, lane);
  const float rs = D == 256 ? 0x1p-4f : 0x1.6a09e6p-4f;   // fp32 nearest 1/sqrt(D)
  float amax[NTK];
#pragma unroll
  for (int k = 0; k < NTK; ++k) amax[k] = 0.0f;
#pragma unroll
  for (int i = 0; i < DL; ++i) {
    const int k = ROLE == 0 ? 0 : (i & 3);
    const float u = x[i] * rs;
    x[i] = sig[k] * u;
    amax[k] = fmaxf(amax[k], fabsf(x[i]));
  }
  if constexpr (ROLE == 0) {
    amax[0] = fmaxf(amax[0], lane_xor<16>(amax[0], lane));
    amax[0] = fmaxf(amax[0], lane_xor<32>(amax[0], lane));
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      amax[k] = fmaxf(amax[k], lane_xor<8>(amax[k], lane));
      amax[k] = fmaxf(amax[k], lane_xor<4>(amax[k], lane));
      amax[k] = fmaxf(amax[k], lane_xor<2>(amax[k], lane));
      amax[k] = fmaxf(amax[k], lane_xor<1>(amax[k], lane));
    }
  }
  float inv[NTK], scale[NTK];
  uint32_t live = 0u;                               // byte mask of rows with amax > 0
#pragma unroll
  for (int k = 0; k < NTK; ++k) {
    const bool nz = amax[k] > 0.0f;
    inv[k] = nz ? 448.0f / amax[k] : 0.0f;
    scale[k] = nz ? amax[k] / 448.0f : 0.0f;
    live |= nz ? (ROLE == 0 ? 0xFFFFFFFFu : (0xFFu << (8 * k))) : 0u;
  }
  uint32_t mk[NG];
  sign_masks<D, ROLE>(p.signs + ((int64_t)h * 2 + ROLE) * (D / 32), lane, mk);
  uint8_t *tile = fh + (int64_t)(ROLE * T + tau) * 16 * D;
#pragma unroll
  for (int c = 0; c < DL / 16; ++c) {
    uint32_t w4[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int q = 4 * c + u;
      const float y0 = x[4 * q] * inv[ROLE == 0 ? 0 : 0], y1 = x[4 * q + 1] * inv[ROLE == 0 ? 0 : 1];
      const float y2 = x[4 * q + 2] * inv[ROLE == 0 ? 0 : 2], y3 = x[4 * q + 3] * inv[ROLE == 0 ? 0 : 3];
      int w = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
      w = __builtin_amdgcn_cvt_pk_fp8_f32(y2, y3, w, true);
      w4[u] = ((uint32_t)w ^ mk[q]) & live;
    }
    *(uint4 *)(tile + c * 1024 + lane * 16) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
  }
  float *so = (float *)(fh + 2LL * P * D + (int64_t)ROLE * 4 * P);
  if constexpr (ROLE == 0) {
    if (g == 0) so[16 * tau + r] = scale[0];
  } else {
    if (r == 0) *(float4 *)(so + 16 * tau + 4 * g) = make_float4(scale[0], scale[1], scale[2], scale[3]);
  }
}

template <int D, int L>
__global__ __launch_bounds__(64 * kEncWaves) void promote_tiles_kernel(PromoteParams p) {
  extern __shared__ __align__(16) uint8_t pro_lds[];
  const int lane = threadIdx.x & 63;
  const int64_t wid = (int64_t)blockIdx.x * kEncWaves + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int T = p.P / 16;
  if (wid >= p.n_pages * p.Hkv * 2 * T) return;
  const int tau = (int)(wid % T);
  const int role = (int)((wid / T) & 1);
  const int h = (int)((wid / (2 * T)) % p.Hkv);
  const int64_t ip = wid / (2 * T * p.Hkv);
  const int src = p.src_page[ip], dst = p.dst_page[ip];
  if (src < 0 || src >= p.src_pool_pages || dst < 0 || dst >= p.fp8_pool_pages) return;   // the whole wave
  const uint8_t *sh = p.src_pool + (int64_t)src * p.src_page_bytes + (int64_t)h * p.src_head_bytes;
  uint8_t *fh = p.fp8_pool + (int64_t)dst * p.fp8_page_bytes + (int64_t)h * p.fp8_head_bytes;
  uint8_t *wl = pro_lds + (threadIdx.x >> 6) * tqf_encode_wave_bytes(D);
  if (role == 0) promote_tile<D, L, 0>(p, sh, fh, h, tau, lane, wl);
  else promote_tile<D, L, 1>(p, sh, fh, h, tau, lane, wl);
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
  const int64_t waves = (p.n_tok + kFp8Group - 1) / kFp8Group * p.Hkv * 2;   // (group, head, role)
  const dim3 grid((unsigned)((waves + 3) / 4));
  if (d == 256) {
    if (src_is_bf16) hipLaunchKernelGGL((encode_fp8_kernel<256, true>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((encode_fp8_kernel<256, false>), grid, dim3(256), 0, s, p);
  } else {
    if (src_is_bf16) hipLaunchKernelGGL((encode_fp8_kernel<128, true>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((encode_fp8_kernel<128, false>), grid, dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

template <int D, int L>
static void launch_tiles(const EncodeTqParams &p, dim3 grid, hipStream_t s) {
  const size_t lds = (L == 5 || L == 6) ? (size_t)kEncWaves * tqf_encode_wave_bytes(D) : 0;
  if (p.src_kind == KVQ_SRC_FP8_PAGES)
    hipLaunchKernelGGL((encode_tq_tiles_kernel<D, L, true>), grid, dim3(64 * kEncWaves), lds, s, p);
  else
    hipLaunchKernelGGL((encode_tq_tiles_kernel<D, L, false>), grid, dim3(64 * kEncWaves), lds, s, p);
}

hipError_t launch_encode_tq(const EncodeTqParams &p, int d, int fmt, hipStream_t s) {
  const int64_t nwg = p.n_pages * p.Hkv * 2;
  if (nwg <= 0) return hipSuccess;
  if (fmt != FMT_TQK) {
    const int64_t waves = nwg * (p.P / 16);
    const dim3 grid((unsigned)((waves + kEncWaves - 1) / kEncWaves));
    const int L = fmt == FMT_TQ3 ? 8 : (fmt == FMT_TQ2 ? 4 : tqf_levels(fmt));
    if (d == 256) {
      if (L == 8) launch_tiles<256, 8>(p, grid, s);
      else if (L == 4) launch_tiles<256, 4>(p, grid, s);
      else if (L == 5) launch_tiles<256, 5>(p, grid, s);
      else launch_tiles<256, 6>(p, grid, s);
    } else {
      if (L == 8) launch_tiles<128, 8>(p, grid, s);
      else if (L == 4) launch_tiles<128, 4>(p, grid, s);
      else if (L == 5) launch_tiles<128, 5>(p, grid, s);
      else launch_tiles<128, 6>(p, grid, s);
    }
    return hipGetLastError();
  }
  if (d != 128) return hipErrorInvalidValue;
  // one wave per tile; a key tile's rows pass through 16 x 128 floats of LDS
  const int64_t waves = nwg * (p.P / 16);
  const dim3 grid((unsigned)((waves + kEncWaves - 1) / kEncWaves));
  const size_t lds = (size_t)kEncWaves * 16 * 128 * 4;
  if (p.src_kind == KVQ_SRC_FP8_PAGES)
    hipLaunchKernelGGL((encode_tqk_tiles_kernel<true>), grid, dim3(64 * kEncWaves), lds, s, p);
  else
    hipLaunchKernelGGL((encode_tqk_tiles_kernel<false>), grid, dim3(64 * kEncWaves), lds, s, p);
  return hipGetLastError();
}

hipError_t launch_promote_fp8(const PromoteParams &p, int d, int fmt, hipStream_t s) {
  const int64_t nwg = p.n_pages * p.Hkv * 2;
  if (nwg <= 0) return hipSuccess;
  if (fmt != FMT_TQK) {
    const int64_t waves = nwg * (p.P / 16);
    const dim3 grid((unsigned)((waves + kEncWaves - 1) / kEncWaves)), block(64 * kEncWaves);
    const int L = fmt == FMT_TQ3 ? 8 : (fmt == FMT_TQ2 ? 4 : tqf_levels(fmt));
    const size_t lds = (L == 5 || L == 6) ? (size_t)kEncWaves * tqf_encode_wave_bytes(d) : 0;
    if (d == 256) {
      if (L == 8) hipLaunchKernelGGL((promote_tiles_kernel<256, 8>), grid, block, 0, s, p);
      else if (L == 4) hipLaunchKernelGGL((promote_tiles_kernel<256, 4>), grid, block, 0, s, p);
      else if (L == 5) hipLaunchKernelGGL((promote_tiles_kernel<256, 5>), grid, block, lds, s, p);
      else hipLaunchKernelGGL((promote_tiles_kernel<256, 6>), grid, block, lds, s, p);
    } else {
      if (L == 8) hipLaunchKernelGGL((promote_tiles_kernel<128, 8>), grid, block, 0, s, p);
      else if (L == 4) hipLaunchKernelGGL((promote_tiles_kernel<128, 4>), grid, block, 0, s, p);
      else if (L == 5) hipLaunchKernelGGL((promote_tiles_kernel<128, 5>), grid, block, lds, s, p);
      else hipLaunchKernelGGL((promote_tiles_kernel<128, 6>), grid, block, lds, s, p);
    }
    return hipGetLastError();
  }
  if (d != 128) return hipErrorInvalidValue;
  const size_t lds = (size_t)p.P * d * 4 + (size_t)p.P * d;
  hipLaunchKernelGGL((promote_fp8_kernel<128, FMT_TQK>), dim3((unsigned)nwg), dim3(256), lds, s, p);
  return hipGetLastError();
}

}  // namespace kvq
