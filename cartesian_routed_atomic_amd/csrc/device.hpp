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

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ uint64_t wave_and64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v &= __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ uint64_t wave_or64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v |= __shfl_xor(v, o);
  return v;
}
// Inclusive suffix sum over lanes: sum of v over lanes >= this lane.
__device__ __forceinline__ uint32_t wave_suffix_sum(uint32_t v) {
  const int l = lane();
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t u = __shfl_down(v, o);
    if (l + o < 64) v += u;
  }
  return v;
}
// Inclusive prefix sum over lanes.
__device__ __forceinline__ int wave_prefix_sum(int v) {
  const int l = lane();
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int u = __shfl_up(v, o);
    if (l >= o) v += u;
  }
  return v;
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
