// The fp16 Gaussian Lloyd-Max codebooks of the TQ formats and their v_perm
// lookup tables (gfx950 device code shared by the scans and the encoders).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_internal.h"

namespace kvq {

// fp16 bit patterns of the Gaussian Lloyd-Max centroids (rounded to fp16),
// ascending code order.
constexpr uint16_t kC3[8] = {0xC04E, 0xBD60, 0xBA0C, 0xB3D8, 0x33D8, 0x3A0C, 0x3D60, 0x404E};
constexpr uint16_t kC2[4] = {0xBE0B, 0xB73F, 0x373F, 0x3E0B};
constexpr uint16_t kC4[16] = {0xC177, 0xC023, 0xBE79, 0xBD06, 0xBB8A, 0xB941, 0xB635, 0xB01C,
                              0x301C, 0x3635, 0x3941, 0x3B8A, 0x3D06, 0x3E79, 0x4023, 0x4177};

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
constexpr uint32_t t4lo(int a) { return pack_bytes(kC4[a] & 255, kC4[a + 1] & 255, kC4[a + 2] & 255, kC4[a + 3] & 255); }
constexpr uint32_t t4hi(int a) { return pack_bytes(kC4[a] >> 8, kC4[a + 1] >> 8, kC4[a + 2] >> 8, kC4[a + 3] >> 8); }
constexpr uint32_t kT4Lo[4] = {t4lo(0), t4lo(4), t4lo(8), t4lo(12)};
constexpr uint32_t kT4Hi[4] = {t4hi(0), t4hi(4), t4hi(8), t4hi(12)};

// Fractional-level codebooks (5 and 6 levels), fp16 bits, ascending codes;
// the 5-level middle centroid is the fp16 -0 the Lloyd iteration rounds to.
constexpr uint16_t kC5[5] = {0xBEE6, 0xBA1E, 0x8000, 0x3A1E, 0x3EE6};
constexpr uint16_t kC6[6] = {0xBF93, 0xBC00, 0xB515, 0x3515, 0x3C00, 0x3F93};
template <int L>
constexpr uint16_t level_c16(int c) {
  return c >= L ? 0 : (L == 5 ? kC5[c] : kC6[c]);
}
template <int L>
constexpr uint32_t level_table(int a, int hi) {
  return pack_bytes((level_c16<L>(a) >> (8 * hi)) & 255, (level_c16<L>(a + 1) >> (8 * hi)) & 255,
                    (level_c16<L>(a + 2) >> (8 * hi)) & 255, (level_c16<L>(a + 3) >> (8 * hi)) & 255);
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

// Four codes of an L-level codebook (L = 5 or 6, one code per byte) -> four
// fp16 centroids as two dwords (codes 0,1 | codes 2,3).
template <int L>
__device__ __forceinline__ uint2 decode_group_levels(uint32_t sel) {
  const uint32_t lo = __builtin_amdgcn_perm(level_table<L>(4, 0), level_table<L>(0, 0), sel);
  const uint32_t hi = __builtin_amdgcn_perm(level_table<L>(4, 1), level_table<L>(0, 1), sel);
  uint2 r;
  r.x = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
  r.y = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
  return r;
}

// Four 4-bit codes (one per byte) -> four fp16 centroids: two 8-entry
// lookups per byte half, chosen by code bit 3 with a byte mask.
__device__ __forceinline__ uint2 decode_group4(uint32_t sel) {
  const uint32_t s7 = sel & 0x07070707u;
  const uint32_t b3 = (sel >> 3) & 0x01010101u;
  const uint32_t upper = (b3 << 8) - b3;          // 0xFF in every byte whose code is >= 8
  const uint32_t lo = (__builtin_amdgcn_perm(kT4Lo[3], kT4Lo[2], s7) & upper) |
                      (__builtin_amdgcn_perm(kT4Lo[1], kT4Lo[0], s7) & ~upper);
  const uint32_t hi = (__builtin_amdgcn_perm(kT4Hi[3], kT4Hi[2], s7) & upper) |
                      (__builtin_amdgcn_perm(kT4Hi[1], kT4Hi[0], s7) & ~upper);
  uint2 r;
  r.x = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
  r.y = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
  return r;
}

// ------------------------------------------------------------------------
// Fractional-level (TQF) tiles: 16 token rows of R bytes, each row the
// slot's codes as one little-endian bitstream of mixed-radix groups (group j
// = sum_i c_{kj+i} L^i, nbits bits). A wave stages a tile's raw bytes in LDS
// and turns every group into code bytes there.
// ------------------------------------------------------------------------
__device__ __forceinline__ uint32_t div_levels(uint32_t v, int L) {
  // floor(v / L) for v < 2^16: multiply by the rounded-up 2^18 / L
  return L == 5 ? (v * 52429u) >> 18 : (v * 43691u) >> 18;
}

// Raw bytes of a tile staged in LDS (dword aligned, 8 readable bytes past
// the tile) -> code bytes: ROWMAJOR puts code (row r, dim j) at codes[r cs +
// j], else at codes[j cs + r]. Lanes take groups lane, lane + 64, ...
template <int D, int L, bool ROWMAJOR>
__device__ __forceinline__ void tqf_unpack_tile(const uint32_t *raw, uint8_t *codes, int cs, int lane) {
  constexpr int K = tqf_group_codes(L), NB = tqf_group_bits(L);
  constexpr int NG = (D + K - 1) / K;
  constexpr int R = tqf_row_bytes(D, L);
  for (int gi = lane; gi < 16 * NG; gi += 64) {
    const int r = gi / NG, g = gi - r * NG;
    const int bit = r * R * 8 + g * NB;
    const uint32_t w0 = raw[bit >> 5], w1 = raw[(bit >> 5) + 1];
    uint32_t v = __builtin_amdgcn_alignbit(w1, w0, bit & 31) & ((1u << NB) - 1u);
#pragma unroll
    for (int i = 0; i < K; ++i) {
      const uint32_t q = div_levels(v, L);
      const int dim = K * g + i;
      if (dim < D) codes[ROWMAJOR ? r * cs + dim : dim * cs + r] = (uint8_t)(v - q * L);
      v = q;
    }
  }
}

}  // namespace kvq
