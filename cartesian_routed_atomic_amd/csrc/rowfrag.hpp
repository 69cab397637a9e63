// Row fragments shared by the executor and its backward: how one wave holds
// a d-long row of W, V or x (bf16 bits or float32) spread over its 64 lanes,
// the per-lane partial dot product, and the store of a float32 result row.
#pragma once
#include "device.hpp"

namespace omni {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// A plain load, or (NT) one with the nontemporal hint.  Rows that a kernel
// reads once (expert rows, a token's own x row) are streamed with the hint so
// they do not displace what is reused from the caches (x rows shared by a
// run of tasks, y, the task lists).
template <bool NT, typename V>
__device__ __forceinline__ V ld(const V* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

// A row fragment of one lane: EPL elements held raw (as loaded) so a load
// can stay in flight until the first use; element q = c * VEC + j maps to
// row[c * 64 * VEC + lane * VEC + j].  load() caches as usual; stream()
// carries the nontemporal hint.
template <typename T, int EPL> struct RowFrag;

template <int EPL> struct RowFrag<uint16_t, EPL> {  // bfloat16 bits
  static constexpr int VEC = EPL < 8 ? EPL : 8;
  static constexpr int NCH = EPL / VEC;
  static constexpr int NW = (EPL + 1) / 2;
  uint32_t w[NW];
  template <bool NT>
  __device__ __forceinline__ void fetch(const uint16_t* row, int l) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const uint16_t* p = row + c * 64 * VEC + l * VEC;
      if constexpr (VEC == 8) {
        const u32x4 v = ld<NT>(reinterpret_cast<const u32x4*>(p));
#pragma unroll
        for (int j = 0; j < 4; ++j) w[c * 4 + j] = v[j];
      } else if constexpr (VEC == 4) {
        const u32x2 v = ld<NT>(reinterpret_cast<const u32x2*>(p));
        w[c * 2] = v[0];
        w[c * 2 + 1] = v[1];
      } else if constexpr (VEC == 2) {
        w[c] = ld<NT>(reinterpret_cast<const uint32_t*>(p));
      } else {
        w[0] = static_cast<uint32_t>(ld<NT>(p));
      }
    }
  }
  __device__ __forceinline__ void load(const uint16_t* row, int l) { fetch<false>(row, l); }
  __device__ __forceinline__ void stream(const uint16_t* row, int l) { fetch<true>(row, l); }
  __device__ __forceinline__ float get(int q) const {
    if constexpr (VEC == 1) return bf_lo(w[0]);
    else return (q & 1) ? bf_hi(w[q >> 1]) : bf_lo(w[q >> 1]);
  }
};

template <int EPL> struct RowFrag<float, EPL> {
  static constexpr int VEC = EPL < 4 ? EPL : 4;
  static constexpr int NCH = EPL / VEC;
  float f[EPL];
  template <bool NT>
  __device__ __forceinline__ void fetch(const float* row, int l) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const float* p = row + c * 64 * VEC + l * VEC;
      if constexpr (VEC == 4) {
        const f32x4 v = ld<NT>(reinterpret_cast<const f32x4*>(p));
#pragma unroll
        for (int j = 0; j < 4; ++j) f[c * 4 + j] = v[j];
      } else if constexpr (VEC == 2) {
        const f32x2 v = ld<NT>(reinterpret_cast<const f32x2*>(p));
        f[c * 2] = v[0];
        f[c * 2 + 1] = v[1];
      } else {
        f[0] = ld<NT>(p);
      }
    }
  }
  __device__ __forceinline__ void load(const float* row, int l) { fetch<false>(row, l); }
  __device__ __forceinline__ void stream(const float* row, int l) { fetch<true>(row, l); }
  __device__ __forceinline__ float get(int q) const { return f[q]; }
};

// Partial dot product of this lane's fragment elements.
template <int EPL>
__device__ __forceinline__ float frag_dot(const RowFrag<uint16_t, EPL>& a,
                                          const RowFrag<uint16_t, EPL>& b) {
  float p = 0.f;
  if constexpr (EPL == 1) {
    p = a.get(0) * b.get(0);
  } else {
#pragma unroll
    for (int i = 0; i < RowFrag<uint16_t, EPL>::NW; ++i)
      p = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.w[i]),
                                          __builtin_bit_cast(bf16x2, b.w[i]), p, false);
  }
  return p;
}
template <int EPL>
__device__ __forceinline__ float frag_dot(const RowFrag<float, EPL>& a,
                                          const RowFrag<float, EPL>& b) {
  float p = 0.f;
#pragma unroll
  for (int q = 0; q < EPL; ++q) p = fmaf(a.f[q], b.f[q], p);
  return p;
}

__device__ __forceinline__ int rdlane(int v, int i) { return __builtin_amdgcn_readlane(v, i); }
__device__ __forceinline__ float rdlane(float v, int i) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), i));
}

// How store_row writes an output row (measured on MI355X, with the random
// 4 KiB expert-row reads of the executor running beside the writes):
//   kStorePlain   ordinary stores (the backward: its rows are re-read soon,
//                 and its 6.7 GB dW / dV stream lost 9 % with the
//                 nontemporal hint and 68 % with the sc1 bit);
//   kStoreNT      the nontemporal hint (executor y rows in most shapes);
//   kStoreDevice  buffer stores with the sc1 scope bit (executor y rows where
//                 the expert rows are streamed: 2 % faster than kStoreNT
//                 there, 9 % slower at heavy expert reuse).
// kStoreDevice builds a buffer descriptor from yrow, so yrow must be the
// same in every lane of the wave (one output row or row slice per wave).
enum StorePolicy { kStorePlain = 0, kStoreNT = 1, kStoreDevice = 2 };

// Store (or add) a lane's accumulators to its columns of a y row, in the
// RowFrag element layout, with 16-byte stores where the layout allows.
template <typename T, int EPL, int POL>
__device__ __forceinline__ void store_row(const float (&acc)[EPL], float* __restrict__ yrow,
                                          int accumulate) {
  constexpr int VEC = RowFrag<T, EPL>::VEC, NCH = RowFrag<T, EPL>::NCH;
  const int l = lane();
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    float* p = yrow + c * 64 * VEC + l * VEC;
    if constexpr (VEC >= 4) {
#pragma unroll
      for (int j = 0; j < VEC; j += 4) {
        float4 v = make_float4(acc[c * VEC + j], acc[c * VEC + j + 1], acc[c * VEC + j + 2],
                               acc[c * VEC + j + 3]);
        if (accumulate) {
          const float4 o = *reinterpret_cast<const float4*>(p + j);
          v.x += o.x; v.y += o.y; v.z += o.z; v.w += o.w;
        }
        if constexpr (POL == kStoreDevice) {
          const __amdgpu_buffer_rsrc_t rs =
              __builtin_amdgcn_make_buffer_rsrc(yrow, 0, NCH * 64 * VEC * 4, 0x00020000);
          const u32x4 nv = {__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z),
                            __float_as_uint(v.w)};
          __builtin_amdgcn_raw_buffer_store_b128(nv, rs, (c * 64 * VEC + l * VEC + j) * 4, 0,
                                                 16 /* sc1 */);
        } else if constexpr (POL == kStoreNT) {
          const f32x4 nv = {v.x, v.y, v.z, v.w};
          __builtin_nontemporal_store(nv, reinterpret_cast<f32x4*>(p + j));
        } else {
          *reinterpret_cast<float4*>(p + j) = v;
        }
      }
    } else {
#pragma unroll
      for (int q = 0; q < VEC; ++q) {
        const float v = acc[c * VEC + q] + (accumulate ? p[q] : 0.f);
        if constexpr (POL != kStorePlain) __builtin_nontemporal_store(v, p + q);
        else p[q] = v;
      }
    }
  }
}

// Wave-level row streaming shared by the token-centric kernels and the grouped
// form's cold tasks: the n (1 <= n <= 64) tasks of a chunk have their expert
// ids in lanes 0..n-1 (my_e), and rows stream through a ring of RING register
// slots with RING - 1 rows in flight.  Two ways to end the ring:
//   EXACT   loads and steps stop at task n - 1 (the loads past the chunk are
//           skipped under a condition, so the compiler's wait counts assume
//           the skipping path near the end);
//   !EXACT  every load is issued: positions past the chunk re-read its last
//           row (then in cache), and the steps past it compute on that row
//           into a lane past n (token_dots) or with a zero coefficient
//           (token_gather), so they change nothing.
// Measured (us per executor call): the token-centric kernels at 64 tasks per
// token run faster EXACT (large 665 against 682, mid 393 against 398, decode
// 23.1 against 23.6: the re-read rows cost more than the looser waits); the
// grouped form's cold tasks, about 13 per token, run faster !EXACT (its call
// at mid 357 against 365, at decode 73 against 80).  The chunked gather keeps
// !EXACT, the form it was built and measured with.

// h_k = x_t . M[e_k] for the n tasks of a chunk (expert e_k in lane k); h_k
// ends in lane k (lanes from n on hold unspecified finite values).
template <typename T, int EPL, bool NT, int RING, bool EXACT = true>
__device__ __forceinline__ float token_dots(const RowFrag<T, EPL>& xf, const T* __restrict__ M,
                                            int my_e, int n, int d, int l,
                                            RowFrag<T, EPL> (&f)[RING]) {
  float my_h = 0.f;
  const int last = n - 1;
#pragma unroll
  for (int s = 0; s < RING - 1; ++s) {
    if (EXACT && s >= n) break;
    f[s].template fetch<NT>(M + static_cast<size_t>(rdlane(my_e, min(s, last))) * d, l);
  }
  for (int i = 0; i < n; i += RING) {
#pragma unroll
    for (int s = 0; s < RING; ++s) {
      const int ii = i + s;
      if (EXACT && ii >= n) break;
      if (!EXACT || ii + RING - 1 < n)
        f[(s + RING - 1) % RING].template fetch<NT>(
            M + static_cast<size_t>(rdlane(my_e, min(ii + RING - 1, last))) * d, l);
      const float h = wave_sum(frag_dot<EPL>(xf, f[s]));
      if (l == ii) my_h = h;
    }
  }
  return my_h;
}

// y_t (+)= sum_k c_k V[e_k] over the n tasks of a chunk (c_k, e_k in lane k),
// the V rows streamed through the ring, fp32 accumulation in k order.
template <typename T, int EPL, bool NT, int RING, bool EXACT = true>
__device__ __forceinline__ void token_gather(const T* __restrict__ V, int my_e, float my_c, int n,
                                             int d, int l, RowFrag<T, EPL> (&f)[RING],
                                             float (&acc)[EPL]) {
  const int last = n - 1;
#pragma unroll
  for (int s = 0; s < RING - 1; ++s) {
    if (EXACT && s >= n) break;
    f[s].template fetch<NT>(V + static_cast<size_t>(rdlane(my_e, min(s, last))) * d, l);
  }
  for (int i = 0; i < n; i += RING) {
#pragma unroll
    for (int s = 0; s < RING; ++s) {
      const int ii = i + s;
      if (EXACT && ii >= n) break;
      if (!EXACT || ii + RING - 1 < n)
        f[(s + RING - 1) % RING].template fetch<NT>(
            V + static_cast<size_t>(rdlane(my_e, min(ii + RING - 1, last))) * d, l);
      const float c = ii < n ? rdlane(my_c, min(ii, 63)) : 0.f;
#pragma unroll
      for (int q = 0; q < EPL; ++q) acc[q] = fmaf(c, f[s].get(q), acc[q]);
    }
  }
}

}  // namespace omni
