// The fp16 Gaussian Lloyd-Max codebooks of the TQ formats and their v_perm
// lookup tables (gfx950 device code shared by the scans and the encoders).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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

}  // namespace kvq
