// Flat router: the baseline the Cartesian Product Router replaces.  Pages:
// gist.science explainer §2.2 (a standard router scores all N experts with a
// d x N projection, O(N d) per token) and the interactive explainer's
// ablation table (the layer without its Cartesian router).
//
//   z = x Wf^T + bias over all N experts (the router GEMM kernels), then per
//   token: log p = z - LSE(z); exact top-K by (log p desc, e asc), values
//   compared as float32 numbers; gates = softmax over the K selected log p.
//
// flat_topk_kernel: one 1024-thread workgroup per token, two passes over the
// token's N logits in the common case:
//   1. online max / sum of exp (-> LSE) and each thread's two largest logits;
//   2. the K-th largest log p among those 2048 thread maxima is a lower bound
//      tau0 of the K-th largest overall (they are K real items); collect every
//      item with log p >= tau0 into LDS (ties at the K-th value included),
//      bitonic-sort them by (value desc, index asc) and keep the first K.
//   If more than kFlatCap items reach tau0 (rows with massive ties), an exact
//   fallback finds the K-th value key with a 4 x 8-bit radix select, then
//   collects the items above it and the lowest-index items equal to it.
#include <cmath>

#include "device.hpp"
#include "launch.hpp"

namespace omni {

constexpr int kFlatThreads = 1024;
constexpr int kFlatWaves = kFlatThreads / 64;
constexpr int kFlatCap = 2048;  // candidates sorted in LDS

struct FlatLds {
  uint64_t cand[kFlatCap];
  uint32_t hist[256];
  float rm[kFlatWaves], rs[kFlatWaves];
  int wcnt[kFlatWaves];
  int n_cand, n_above, digit, digit_above;
};

// Online (max, sum of exp) pair: s = sum exp(z - m).
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  const float mm = fmaxf(m, m2);
  if (mm == -INFINITY) return;
  s = s * __expf(m - mm) + s2 * __expf(m2 - mm);
  m = mm;
}

// Bitonic sort of P (a power of two, <= kFlatCap) 64-bit keys, descending.
__device__ void bitonic_desc(uint64_t* a, int P) {
  for (int k = 2; k <= P; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < P; i += kFlatThreads) {
        const int p = i ^ j;
        if (p > i) {
          const uint64_t x = a[i], y = a[p];
          const bool desc = (i & k) == 0;
          if (desc ? x < y : x > y) {
            a[i] = y;
            a[p] = x;
          }
        }
      }
      __syncthreads();
    }
  }
}

__global__ __launch_bounds__(kFlatThreads) void flat_topk_kernel(
    const float* __restrict__ z, int N, int K, float* __restrict__ logp_out,
    int32_t* __restrict__ expert_idx, float* __restrict__ score, float* __restrict__ gate) {
  __shared__ FlatLds sh;
  const int t = blockIdx.x;
  const int tid = threadIdx.x, w = tid >> 6, l = lane();
  const float* row = z + static_cast<size_t>(t) * N;

  // pass 1: online LSE and the thread's two largest logits
  float m = -INFINITY, s = 0.f, t1 = -INFINITY, t2 = -INFINITY;
  bool h1 = false, h2 = false;
  for (int i = tid; i < N; i += kFlatThreads) {
    const float v = row[i];
    if (v > m) {
      s = s * __expf(m - v) + 1.f;
      m = v;
    } else {
      s += __expf(v - m);
    }
    if (!h1 || v > t1) {
      t2 = t1;
      h2 = h1;
      t1 = v;
      h1 = true;
    } else if (!h2 || v > t2) {
      t2 = v;
      h2 = true;
    }
  }
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o), s2 = __shfl_xor(s, o);
    lse_merge(m, s, m2, s2);
  }
  if (l == 0) {
    sh.rm[w] = m;
    sh.rs[w] = s;
  }
  if (tid == 0) sh.n_cand = 0;
  __syncthreads();
  m = sh.rm[0];
  s = sh.rs[0];
  for (int q = 1; q < kFlatWaves; ++q) lse_merge(m, s, sh.rm[q], sh.rs[q]);
  const float lse = m + __logf(s);

  // tau0: the K-th largest value key among the 2048 thread maxima (bit by bit)
  const uint32_t k1 = h1 ? fkey(t1 - lse) : 0u, k2 = h2 ? fkey(t2 - lse) : 0u;
  uint32_t tau0 = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t c = tau0 | (1u << b);
    const int n = __syncthreads_count(k1 >= c) + __syncthreads_count(k2 >= c);
    if (n >= K) tau0 = c;
  }

  // pass 2: collect every item with a value key >= tau0 (optionally store log p)
  for (int i = tid; i < N; i += kFlatThreads) {
    const float lp = row[i] - lse;
    if (logp_out) logp_out[static_cast<size_t>(t) * N + i] = lp;
    if (fkey(lp) >= tau0) {
      const int slot = atomicAdd(&sh.n_cand, 1);
      if (slot < kFlatCap) sh.cand[slot] = sel_key(lp, static_cast<uint32_t>(i));
    }
  }
  __syncthreads();
  const int C = sh.n_cand;
  if (C <= kFlatCap) {
    int P = 64;
    while (P < C) P <<= 1;
    for (int i = C + tid; i < P; i += kFlatThreads) sh.cand[i] = 0;  // empty slots sort last
    __syncthreads();
    bitonic_desc(sh.cand, P);
  } else {
    // exact fallback: tau = the K-th largest value key, 8 bits per pass
    uint32_t prefix = 0, mask = 0;
    int need = K;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      if (tid < 256) sh.hist[tid] = 0;
      __syncthreads();
      for (int i = tid; i < N; i += kFlatThreads) {
        const uint32_t k = fkey(row[i] - lse);
        if ((k & mask) == prefix) atomicAdd(&sh.hist[(k >> shift) & 255], 1u);
      }
      __syncthreads();
      if (w == 0) {
        // lane l holds bins 4l .. 4l + 3; items in bins above bin b: 'above'
        uint32_t h[4];
        uint32_t s4 = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          h[q] = sh.hist[4 * l + q];
          s4 += h[q];
        }
        uint32_t above = wave_suffix_sum(s4) - s4;  // bins of the lanes above
#pragma unroll
        for (int q = 3; q >= 0; --q) {
          if (above < static_cast<uint32_t>(need) && above + h[q] >= static_cast<uint32_t>(need)) {
            sh.digit = 4 * l + q;
            sh.digit_above = static_cast<int>(above);
          }
          above += h[q];
        }
      }
      __syncthreads();
      prefix |= static_cast<uint32_t>(sh.digit) << shift;
      mask |= 255u << shift;
      need -= sh.digit_above;
      __syncthreads();
    }
    const uint32_t tau = prefix;  // K - need items lie above tau; take `need` ties
    if (tid == 0) sh.n_above = 0;
    __syncthreads();
    int taken = 0;
    for (int base = 0; base < N; base += kFlatThreads) {
      const int i = base + tid;
      uint32_t k = 0;
      float lp = 0.f;
      if (i < N) {
        lp = row[i] - lse;
        k = fkey(lp);
      }
      if (i < N && k > tau) {
        const int slot = atomicAdd(&sh.n_above, 1);  // K - need of them in all
        if (slot < 64) sh.cand[slot] = sel_key(lp, static_cast<uint32_t>(i));
      }
      // ties in index order: block-wide exclusive prefix count
      const bool eq = i < N && k == tau;
      const uint64_t bal = __ballot(eq);
      if (l == 0) sh.wcnt[w] = __popcll(bal);
      __syncthreads();
      int before = 0, total = 0;
      for (int q = 0; q < kFlatWaves; ++q) {
        before += q < w ? sh.wcnt[q] : 0;
        total += sh.wcnt[q];
      }
      const int pos = taken + before + mbcnt(bal);
      if (eq && pos < need) sh.cand[K - need + pos] = sel_key(lp, static_cast<uint32_t>(i));
      taken += total;
      __syncthreads();
    }
    for (int i = K + tid; i < 64; i += kFlatThreads) sh.cand[i] = 0;
    __syncthreads();
    bitonic_desc(sh.cand, 64);
  }
  // outputs: the first K keys; g_k = exp(S_k - S_0) / sum_j exp(S_j - S_0)
  if (w == 0) {
    const uint64_t best = l < K ? sh.cand[l] : 0;
    const float sv = l < K ? sel_val(best) : 0.f;
    const float s0 = __shfl(sv, 0);
    const float ex = l < K ? expf(sv - s0) : 0.f;
    const float den = wave_sum(ex);
    if (l < K) {
      const size_t o = static_cast<size_t>(t) * K + l;
      expert_idx[o] = static_cast<int32_t>(sel_idx(best));
      score[o] = sv;
      gate[o] = ex / den;
    }
  }
}

size_t flat_router_ws_bytes(int L, int N) {
  return (static_cast<size_t>(L > 0 ? L : 1) * N * 4 + 255) & ~static_cast<size_t>(255);
}

hipError_t launch_flat_router(int bf16, int L, int d, int N, int K, const void* x,
                              const void* wf, const float* bias, int32_t* expert_idx,
                              float* score, float* gate, float* logp, void* ws, hipStream_t s) {
  if (L == 0) return hipSuccess;
  float* z = static_cast<float*>(ws);
  const hipError_t e =
      bf16 ? launch_router_bf16(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(wf),
                                static_cast<const uint16_t*>(wf), bias, nullptr, z, z, L, d, N,
                                0, nullptr, s)
           : launch_router_f32(static_cast<const float*>(x), static_cast<const float*>(wf),
                               static_cast<const float*>(wf), bias, nullptr, z, z, L, d, N, 0, s);
  if (e != hipSuccess) return e;
  flat_topk_kernel<<<static_cast<unsigned>(L), kFlatThreads, 0, s>>>(z, N, K, logp, expert_idx,
                                                                    score, gate);
  return hipGetLastError();
}

}  // namespace omni
