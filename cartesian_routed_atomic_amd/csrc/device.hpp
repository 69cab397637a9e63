// Device helpers shared by the gfx950 kernels: wave64 reductions, bf16
// widening, order-preserving float keys and the internal launch interface.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace omni {

constexpr int kWave = 64;

__device__ __forceinline__ int lane() { return static_cast<int>(__lane_id()); }

// bfloat16 bits -> float32 (exact): low / high half of a packed 32-bit word.
__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// DPP helpers: v from the lane selected by `ctrl` (lanes without a source,
// or in rows left out by `row_mask`, get `old`).
template <int ctrl, int row_mask>
__device__ __forceinline__ float dpp_f(float old, float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
      __builtin_bit_cast(int, old), __builtin_bit_cast(int, v), ctrl, row_mask, 0xf, false));
}
// Wave-wide sum with DPP: row_shr 1, 2, 4, 8 builds each 16-lane row's total
// in its lane 15; row_bcast:15 and row_bcast:31 carry the row totals up to
// lane 63, which is then broadcast.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<0x111, 0xf>(0.f, v);  // row_shr:1
  v += dpp_f<0x112, 0xf>(0.f, v);  // row_shr:2
  v += dpp_f<0x114, 0xf>(0.f, v);  // row_shr:4
  v += dpp_f<0x118, 0xf>(0.f, v);  // row_shr:8
  v += dpp_f<0x142, 0xa>(0.f, v);  // row_bcast:15 into rows 1 and 3
  v += dpp_f<0x143, 0xc>(0.f, v);  // row_bcast:31 into rows 2 and 3
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<0x111, 0xf>(-INFINITY, v));
  v = fmaxf(v, dpp_f<0x112, 0xf>(-INFINITY, v));
  v = fmaxf(v, dpp_f<0x114, 0xf>(-INFINITY, v));
  v = fmaxf(v, dpp_f<0x118, 0xf>(-INFINITY, v));
  v = fmaxf(v, dpp_f<0x142, 0xa>(-INFINITY, v));
  v = fmaxf(v, dpp_f<0x143, 0xc>(-INFINITY, v));
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
template <int ctrl, int row_mask>
__device__ __forceinline__ uint32_t dpp_u(uint32_t old, uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(
      static_cast<int>(old), static_cast<int>(v), ctrl, row_mask, 0xf, false));
}
__device__ __forceinline__ uint32_t wave_and32(uint32_t v) {
  v &= dpp_u<0x111, 0xf>(~0u, v);
  v &= dpp_u<0x112, 0xf>(~0u, v);
  v &= dpp_u<0x114, 0xf>(~0u, v);
  v &= dpp_u<0x118, 0xf>(~0u, v);
  v &= dpp_u<0x142, 0xa>(~0u, v);
  v &= dpp_u<0x143, 0xc>(~0u, v);
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 63));
}
__device__ __forceinline__ uint32_t wave_or32(uint32_t v) {
  v |= dpp_u<0x111, 0xf>(0u, v);
  v |= dpp_u<0x112, 0xf>(0u, v);
  v |= dpp_u<0x114, 0xf>(0u, v);
  v |= dpp_u<0x118, 0xf>(0u, v);
  v |= dpp_u<0x142, 0xa>(0u, v);
  v |= dpp_u<0x143, 0xc>(0u, v);
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 63));
}
__device__ __forceinline__ uint64_t wave_and64(uint64_t v) {
  return (static_cast<uint64_t>(wave_and32(static_cast<uint32_t>(v >> 32))) << 32) |
         wave_and32(static_cast<uint32_t>(v));
}
__device__ __forceinline__ uint64_t wave_or64(uint64_t v) {
  return (static_cast<uint64_t>(wave_or32(static_cast<uint32_t>(v >> 32))) << 32) |
         wave_or32(static_cast<uint32_t>(v));
}
// Inclusive prefix sum over the 64 lanes (Hillis-Steele inside each 16-lane
// row, then the row totals carried up with row_bcast).
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v) {
  v += dpp_u<0x111, 0xf>(0u, v);
  v += dpp_u<0x112, 0xf>(0u, v);
  v += dpp_u<0x114, 0xf>(0u, v);
  v += dpp_u<0x118, 0xf>(0u, v);
  v += dpp_u<0x142, 0xa>(0u, v);
  v += dpp_u<0x143, 0xc>(0u, v);
  return v;
}
// Inclusive suffix sum over lanes: sum of v over lanes >= this lane.
__device__ __forceinline__ uint32_t wave_suffix_sum(uint32_t v) {
  const uint32_t p = wave_inclusive_scan(v);
  const uint32_t total = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(p), 63));
  return total - p + v;
}
// Inclusive prefix sum over lanes.
__device__ __forceinline__ int wave_prefix_sum(int v) {
  return static_cast<int>(wave_inclusive_scan(static_cast<uint32_t>(v)));
}
// Number of set bits of m in lanes below this lane.
__device__ __forceinline__ int mbcnt(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0));
}
// Orders LDS traffic of one wave (the LDS unit serves a wave in order; this
// only stops the compiler from moving accesses across the point).
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Order-preserving map float32 -> uint32 (larger float -> larger key), with
// -0 folded onto +0 so the two compare equal, as float32 comparison does.
__device__ __forceinline__ uint32_t fkey(float f) {
  uint32_t u = __float_as_uint(f);
  u = (u == 0x80000000u) ? 0u : u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float fkey_inv(uint32_t k) {
  return (k & 0x80000000u) ? __uint_as_float(k & 0x7fffffffu) : __uint_as_float(~k);
}
// 64-bit selection key: value descending, then index ascending.  Keys of
// real items are never 0 (fkey(-inf) > 0), so 0 marks an empty slot.
__device__ __forceinline__ uint64_t sel_key(float v, uint32_t idx) {
  return (static_cast<uint64_t>(fkey(v)) << 32) | static_cast<uint64_t>(~idx);
}
__device__ __forceinline__ uint32_t sel_idx(uint64_t k) { return ~static_cast<uint32_t>(k); }
__device__ __forceinline__ float sel_val(uint64_t k) { return fkey_inv(static_cast<uint32_t>(k >> 32)); }

}  // namespace omni
