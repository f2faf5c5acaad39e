// Cross-lane moves of a 64-lane gfx950 wave, without LDS.
//
// lane_xor<M>(x): the value of lane (lane ^ M). DPP row permutes for M < 16
// (quad permutes for 1 and 2; a half-row mirror followed by a quad reversal
// for 4; a row rotation by 8 for 8) and the gfx950 lane-swap moves for 16 and
// 32 (a self-swap leaves the lower half of each pair in the first result and
// the upper half in the second).
//
// lane_swap<X>(a, b, d, s): one v_permlane{16,32}_swap of the registers a, b
// (X = 16: odd rows of a trade places with even rows of b; X = 32: the upper
// half of a with the lower half of b). For a lane whose bit X is clear, d is
// its own a and s is the a of lane ^ X; for a lane whose bit X is set, d is
// the b of lane ^ X and s is its own b. With a = b that is (own, partner) in
// lower lanes and (partner, own) in upper lanes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

template <int M>
__device__ __forceinline__ float lane_xor(float x, int lane) {
  const int u = __builtin_bit_cast(int, x);
  int r;
  if constexpr (M == 1) {
    r = __builtin_amdgcn_update_dpp(0, u, 0xB1, 0xF, 0xF, true);
  } else if constexpr (M == 2) {
    r = __builtin_amdgcn_update_dpp(0, u, 0x4E, 0xF, 0xF, true);
  } else if constexpr (M == 4) {
    const int t = __builtin_amdgcn_update_dpp(0, u, 0x141, 0xF, 0xF, true);
    r = __builtin_amdgcn_update_dpp(0, t, 0x1B, 0xF, 0xF, true);
  } else if constexpr (M == 8) {
    r = __builtin_amdgcn_update_dpp(0, u, 0x128, 0xF, 0xF, true);
  } else if constexpr (M == 16) {
    const auto s = __builtin_amdgcn_permlane16_swap((uint32_t)u, (uint32_t)u, false, false);
    r = (int)((lane & 16) ? s[0] : s[1]);
  } else {
    static_assert(M == 32, "lane distance");
    const auto s = __builtin_amdgcn_permlane32_swap((uint32_t)u, (uint32_t)u, false, false);
    r = (int)((lane & 32) ? s[0] : s[1]);
  }
  return __builtin_bit_cast(float, r);
}

// The value of lane (lane ^ M) through the LDS crossbar (no LDS storage):
// ds_swizzle in its bit-mask mode for M < 32, ds_bpermute for M = 32. These
// issue on the LDS pipe, leaving the VALU to the arithmetic around them.
template <int M>
__device__ __forceinline__ float lane_xor_ds(float x, int lane) {
  const int u = __builtin_bit_cast(int, x);
  if constexpr (M < 32) {
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(u, 0x1F | (M << 10)));
  } else {
    static_assert(M == 32, "lane distance");
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, u));
  }
}

// Orders a wave's own LDS writes before its later LDS reads of other lanes'
// data: LDS executes one wave's operations in issue order, so what is needed
// is that the compiler keeps the order (wavefront-scope fences) and keeps the
// wave together (wave barrier).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int X>
__device__ __forceinline__ void lane_swap(float a, float b, float &d, float &s) {
  const uint32_t ua = __builtin_bit_cast(uint32_t, a), ub = __builtin_bit_cast(uint32_t, b);
  if constexpr (X == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(ua, ub, false, false);
    d = __builtin_bit_cast(float, (uint32_t)r[0]);
    s = __builtin_bit_cast(float, (uint32_t)r[1]);
  } else {
    static_assert(X == 32, "swap distance");
    const auto r = __builtin_amdgcn_permlane32_swap(ua, ub, false, false);
    d = __builtin_bit_cast(float, (uint32_t)r[0]);
    s = __builtin_bit_cast(float, (uint32_t)r[1]);
  }
}

}  // namespace kvq
