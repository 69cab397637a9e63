// Cartesian Product Router, part 2: per-axis log-probabilities and top-k',
// top-K over the product cells, gates.  Pages: interactive explainer
// "Cartesian Product Router" (row and column distributions p_r, p_c; rows and
// columns are searched separately; the joint score S_ij = log p_r[i] +
// log p_c[j] is additive in log space and the N-entry score matrix is never
// formed) and "Expert-Centric Scheduling" (every decision carries a weight;
// the gate is the softmax over the K selected scores).
//
// One wave (64 lanes) serves one token end to end; four tokens per
// workgroup, no cross-wave synchronisation.
//
// Per axis the wave reads the logit row once, forms a = z - (m + ln sum
// exp(z - m)) in float32, optionally stores it, and selects the k' largest a
// with an MSB-first radix select over 32-bit order-preserving value keys
// (bits shared by all candidates are skipped; ties at the threshold value
// are taken in index order, which is the lane/slot order of the row).  The
// winners are sorted by a 64-lane bitonic sort on (value key << 32 | ~index).
//
// Product merge.  With rank-ordered axis lists R (rows) and C (columns),
// S(r, c) = fl32(a[R_r] + b[C_c]) is non-increasing in r and in c (float
// addition is monotone).  For any cell outside the staircase
// P = {(r, c) : (r+1)(c+1) <= K} at least K cells of P dominate it, so the
// K-th best value over P, tau, bounds everything outside P from above.  The
// kernel therefore selects the top K of P (|P| <= 280 for K, k' <= 64) and
// checks, per row, the first cell past the staircase: if none reaches tau
// the answer is exact.  Otherwise (a float32 tie at tau) the token is
// flagged and a second, plain kernel redoes its top K over all k'^2 cells.
#include "device.hpp"
#include "launch.hpp"

namespace omni {

// ---------------------------------------------------------------- selection

// Result of a value-key selection: the selected items are those with
// key > T plus the first `eq_take` items with key == T in index order, or,
// when eq_take < 0, every item with key >= T.
struct Sel32 {
  uint32_t T;
  int eq_take;
};

// k largest of the wave's 32-bit keys (NI per lane; bit j of `valid` marks
// slot j as an item).  Requires 1 <= k <= number of items.
// hist: 256 words of LDS owned by this wave.
template <int NI>
__device__ __forceinline__ Sel32 wave_select32(const uint32_t (&vk)[NI], uint32_t valid, int k,
                                               uint32_t* hist) {
  const int l = lane();
  uint32_t cand = valid;
  uint32_t need = static_cast<uint32_t>(k);
  for (int pass = 0; pass < 5; ++pass) {
    uint32_t a = ~0u, o = 0u;
#pragma unroll
    for (int j = 0; j < NI; ++j)
      if ((cand >> j) & 1u) {
        a &= vk[j];
        o |= vk[j];
      }
    a = wave_and32(a);
    o = wave_or32(o);
    const uint32_t diff = a ^ o;
    if (diff == 0) return Sel32{o, static_cast<int>(need)};  // equal keys left: ties
    const int h = 31 - __clz(diff);
    const int lo = h > 7 ? h - 7 : 0;
    *reinterpret_cast<uint4*>(&hist[4 * l]) = make_uint4(0, 0, 0, 0);
    wave_lds_fence();
#pragma unroll
    for (int j = 0; j < NI; ++j)
      if ((cand >> j) & 1u) atomicAdd(&hist[(vk[j] >> lo) & 255u], 1u);
    wave_lds_fence();
    const uint4 c = *reinterpret_cast<const uint4*>(&hist[4 * l]);
    const uint32_t s = c.x + c.y + c.z + c.w;
    const uint32_t S = wave_suffix_sum(s);
    const uint32_t above = S - s;
    const uint64_t hm = __ballot(above < need && need <= S);
    if (hm == 0) return Sel32{0u, -1};  // unreachable while k <= #items
    const int hl = __ffsll(static_cast<unsigned long long>(hm)) - 1;
    uint32_t dstar = 0, nneed = 0, bcnt = 0;
    if (l == hl) {
      uint32_t cum = above;
      if (cum + c.w >= need) { dstar = 4 * l + 3; nneed = need - cum; bcnt = c.w; }
      else if ((cum += c.w) + c.z >= need) { dstar = 4 * l + 2; nneed = need - cum; bcnt = c.z; }
      else if ((cum += c.z) + c.y >= need) { dstar = 4 * l + 1; nneed = need - cum; bcnt = c.y; }
      else { cum += c.y; dstar = 4 * l; nneed = need - cum; bcnt = c.x; }
    }
    dstar = __builtin_amdgcn_readlane(dstar, hl);
    nneed = __builtin_amdgcn_readlane(nneed, hl);
    bcnt = __builtin_amdgcn_readlane(bcnt, hl);
#pragma unroll
    for (int j = 0; j < NI; ++j)
      if (((cand >> j) & 1u) && ((vk[j] >> lo) & 255u) != dstar) cand &= ~(1u << j);
    need = nneed;
    wave_lds_fence();
    if (bcnt == need) {
      const uint32_t hi_mask = (h >= 31) ? 0u : (~0u << (h + 1));
      return Sel32{(a & hi_mask) | (dstar << lo), -1};
    }
  }
  return Sel32{0u, -1};  // not reached
}

// Threshold T such that exactly k of this wave's 64-bit keys are >= T.
// keys[j] is this lane's j-th key (0 = no item); keys are distinct.
template <int NI>
__device__ __forceinline__ uint64_t wave_select64(const uint64_t (&keys)[NI], int k,
                                                  uint32_t* hist) {
  const int l = lane();
  uint32_t cand = 0;
#pragma unroll
  for (int j = 0; j < NI; ++j)
    if (keys[j] != 0) cand |= (1u << j);
  uint32_t need = static_cast<uint32_t>(k);
  for (int pass = 0; pass < 9; ++pass) {
    uint64_t a = ~0ull, o = 0;
#pragma unroll
    for (int j = 0; j < NI; ++j)
      if ((cand >> j) & 1u) {
        a &= keys[j];
        o |= keys[j];
      }
    a = wave_and64(a);
    o = wave_or64(o);
    const uint64_t diff = a ^ o;
    if (diff == 0) return o;  // one candidate left
    const int h = 63 - __clzll(diff);
    const int lo = h > 7 ? h - 7 : 0;
    *reinterpret_cast<uint4*>(&hist[4 * l]) = make_uint4(0, 0, 0, 0);
    wave_lds_fence();
#pragma unroll
    for (int j = 0; j < NI; ++j)
      if ((cand >> j) & 1u) atomicAdd(&hist[(keys[j] >> lo) & 255], 1u);
    wave_lds_fence();
    const uint4 c = *reinterpret_cast<const uint4*>(&hist[4 * l]);
    const uint32_t s = c.x + c.y + c.z + c.w;
    const uint32_t S = wave_suffix_sum(s);
    const uint32_t above = S - s;
    const uint64_t hm = __ballot(above < need && need <= S);
    if (hm == 0) return 0;  // unreachable while k <= #items
    const int hl = __ffsll(static_cast<unsigned long long>(hm)) - 1;
    uint32_t dstar = 0, nneed = 0, bcnt = 0;
    if (l == hl) {
      uint32_t cum = above;
      if (cum + c.w >= need) { dstar = 4 * l + 3; nneed = need - cum; bcnt = c.w; }
      else if ((cum += c.w) + c.z >= need) { dstar = 4 * l + 2; nneed = need - cum; bcnt = c.z; }
      else if ((cum += c.z) + c.y >= need) { dstar = 4 * l + 1; nneed = need - cum; bcnt = c.y; }
      else { cum += c.y; dstar = 4 * l; nneed = need - cum; bcnt = c.x; }
    }
    dstar = __builtin_amdgcn_readlane(dstar, hl);
    nneed = __builtin_amdgcn_readlane(nneed, hl);
    bcnt = __builtin_amdgcn_readlane(bcnt, hl);
#pragma unroll
    for (int j = 0; j < NI; ++j)
      if (((cand >> j) & 1u) && static_cast<uint32_t>((keys[j] >> lo) & 255) != dstar)
        cand &= ~(1u << j);
    need = nneed;
    wave_lds_fence();
    if (bcnt == need) {
      const uint64_t hi_mask = (h >= 63) ? 0ull : (~0ull << (h + 1));
      return (a & hi_mask) | (static_cast<uint64_t>(dstar) << lo);
    }
  }
  return 0;  // not reached for distinct keys
}

// Descending bitonic sort of one 64-bit key per lane.
__device__ __forceinline__ uint64_t bitonic_desc(uint64_t key) {
  const int l = lane();
#pragma unroll
  for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const uint64_t o = __shfl_xor(key, stride);
      const bool take_max = ((l & stride) == 0) == ((l & size) == 0);
      key = take_max ? (key > o ? key : o) : (key < o ? key : o);
    }
  }
  return key;
}

// Compacts the selected axis items into buf as (value key << 32 | ~index)
// and returns them sorted, rank r in lane r (0 past k).  Item (j, lane) has
// index j * 64 + lane, so slot order is index order.
template <int NI>
__device__ __forceinline__ uint64_t axis_collect_sorted(const uint32_t (&vk)[NI], uint32_t valid,
                                                        Sel32 sel, int k, uint64_t* buf) {
  const int l = lane();
  int base = 0;
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const bool in = ((valid >> j) & 1u) && (sel.eq_take < 0 ? vk[j] >= sel.T : vk[j] > sel.T);
    const uint64_t m = __ballot(in);
    const int slot = base + mbcnt(m);
    if (in && slot < 64)
      buf[slot] = (static_cast<uint64_t>(vk[j]) << 32) | static_cast<uint32_t>(~(j * 64 + l));
    base += __popcll(m);
  }
  int rest = sel.eq_take;
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const bool eq = rest > 0 && ((valid >> j) & 1u) && vk[j] == sel.T;
    const uint64_t m = __ballot(eq);
    const int r = mbcnt(m);
    const int slot = base + r;
    if (eq && r < rest && slot < 64)
      buf[slot] = (static_cast<uint64_t>(vk[j]) << 32) | static_cast<uint32_t>(~(j * 64 + l));
    const int taken = min(__popcll(m), max(rest, 0));
    base += taken;
    rest -= taken;
  }
  wave_lds_fence();
  uint64_t key = (l < k) ? buf[l] : 0ull;
  wave_lds_fence();
  return bitonic_desc(key);
}

// The k keys >= T in descending order: lane r holds rank r (0 past k).
template <int NI>
__device__ __forceinline__ uint64_t wave_collect_sorted(const uint64_t (&keys)[NI], uint64_t T,
                                                        int k, uint64_t* buf) {
  const int l = lane();
  int base = 0;
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const bool p = keys[j] >= T && keys[j] != 0;
    const uint64_t m = __ballot(p);
    const int slot = base + mbcnt(m);
    if (p && slot < 64) buf[slot] = keys[j];
    base += __popcll(m);
  }
  wave_lds_fence();
  uint64_t key = (l < k) ? buf[l] : 0ull;
  wave_lds_fence();
  return bitonic_desc(key);
}

__device__ __forceinline__ void write_outputs(uint64_t best, int t, int K,
                                              int32_t* __restrict__ expert_idx,
                                              float* __restrict__ score,
                                              float* __restrict__ gate) {
  // g_k = exp(S_k - S_0) / sum_j exp(S_j - S_0), S_0 the largest
  const int l = lane();
  const float sv = (l < K) ? sel_val(best) : 0.f;
  const float s0 = __shfl(sv, 0);
  const float ex = (l < K) ? expf(sv - s0) : 0.f;
  const float den = wave_sum(ex);
  if (l < K) {
    const size_t o = static_cast<size_t>(t) * K + l;
    expert_idx[o] = static_cast<int32_t>(sel_idx(best));
    score[o] = sv;
    gate[o] = ex / den;
  }
}

// ln sum exp over one row held NI per lane (invalid slots excluded), as
// m + ln sum exp(z - m) with m the row maximum.
template <int NI>
__device__ __forceinline__ float row_lse(const float (&z)[NI], uint32_t valid) {
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < NI; ++j)
    if ((valid >> j) & 1u) m = fmaxf(m, z[j]);
  m = wave_max(m);
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < NI; ++j)
    if ((valid >> j) & 1u) s += expf(z[j] - m);
  s = wave_sum(s);
  return m + logf(s);
}

struct TopkLds {
  uint32_t hist[256];
  uint64_t buf[64];
  float av[64];
  float bv[64];
  uint32_t R[64];
  uint32_t C[64];
  int poff[68];
};

constexpr int kStairItems = 5;  // ceil(280 / 64): |P| <= 280 for K, k' <= 64

// Main pass.  tie_flag[t] = 1 marks a token whose K-th score ties a cell past
// the staircase; its outputs are then written by product_topk_fixup_kernel.
// lse[2t], lse[2t+1] keep the row / column normalisers for that kernel.
template <int NI>
__global__ __launch_bounds__(256) void product_topk_kernel(
    const float* __restrict__ Zr, const float* __restrict__ Zc, int L, int Nr, int Nc, int kp,
    int K, int32_t* __restrict__ expert_idx, float* __restrict__ score,
    float* __restrict__ gate, float* __restrict__ row_logp, float* __restrict__ col_logp,
    int32_t* __restrict__ row_sel, int32_t* __restrict__ col_sel,
    int32_t* __restrict__ tie_flag, float* __restrict__ lse_out) {
  static_assert(NI <= 32, "32 slots per lane at most");
  __shared__ TopkLds smem[4];
  const int w = threadIdx.x >> 6, l = lane();
  const int t = blockIdx.x * 4 + w;
  if (t >= L) return;  // the whole wave leaves together
  TopkLds& S = smem[w];

  // ---- per axis: log-softmax, then the k' best lines in rank order
#pragma unroll 1
  for (int axis = 0; axis < 2; ++axis) {
    const int n = axis ? Nc : Nr;
    const float* src = axis ? Zc + static_cast<size_t>(t) * Nc : Zr + static_cast<size_t>(t) * Nr;
    float* dst = axis ? col_logp : row_logp;
    float z[NI];
    uint32_t valid = 0;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int i = j * 64 + l;
      z[j] = 0.f;
      if (i < n) {
        z[j] = src[i];
        valid |= 1u << j;
      }
    }
    const float lse = row_lse<NI>(z, valid);
    uint32_t vk[NI];
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const float a = z[j] - lse;
      vk[j] = fkey(a);
      if (dst && ((valid >> j) & 1u)) dst[static_cast<size_t>(t) * n + j * 64 + l] = a;
    }
    if (l == 0) lse_out[2 * static_cast<size_t>(t) + axis] = lse;
    const Sel32 sel = wave_select32<NI>(vk, valid, kp, S.hist);
    const uint64_t kk = axis_collect_sorted<NI>(vk, valid, sel, kp, S.buf);
    int32_t* out = axis ? col_sel : row_sel;
    if (l < kp) {
      (axis ? S.bv : S.av)[l] = sel_val(kk);
      (axis ? S.C : S.R)[l] = sel_idx(kk);
      out[static_cast<size_t>(t) * kp + l] = static_cast<int32_t>(sel_idx(kk));
    }
  }
  wave_lds_fence();

  // ---- staircase P: row r contributes columns c < len_r = min(k', K / (r + 1))
  const int len = (l < kp) ? min(kp, K / (l + 1)) : 0;
  const int inc = wave_prefix_sum(len);
  if (l < kp) S.poff[l + 1] = inc;
  if (l == 0) S.poff[0] = 0;
  const int P = __builtin_amdgcn_readlane(inc, 63);
  wave_lds_fence();
  uint64_t pk[kStairItems];
#pragma unroll
  for (int j = 0; j < kStairItems; ++j) {
    const int p = l + 64 * j;
    pk[j] = 0ull;
    if (p < P) {
      int lo = 0, hi = kp;  // largest r with poff[r] <= p
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (S.poff[mid] <= p) lo = mid; else hi = mid;
      }
      const int r = lo, c = p - S.poff[r];
      const float sv = S.av[r] + S.bv[c];
      pk[j] = sel_key(sv, S.R[r] * static_cast<uint32_t>(Nc) + S.C[c]);
    }
  }
  const uint64_t Tp = wave_select64<kStairItems>(pk, K, S.hist);
  const uint64_t best = wave_collect_sorted<kStairItems>(pk, Tp, K, S.buf);
  const uint32_t tau = static_cast<uint32_t>(__shfl(best, K - 1) >> 32);

  // ---- a cell past the staircase can only tie at tau; check each row's first
  bool extra = false;
  if (l < kp && len < kp) extra = fkey(S.av[l] + S.bv[len]) >= tau;
  const bool tie = __ballot(extra) != 0ull;
  if (l == 0) tie_flag[t] = tie ? 1 : 0;
  if (!tie) write_outputs(best, t, K, expert_idx, score, gate);
}

// Exact top-K for the flagged tokens: K rounds, each taking the largest cell
// key below the previous round's, over all k' x k' cells.  Lane r owns row r
// (k' <= 64); columns are walked one at a time.  The axis values are rebuilt
// as z - lse with the main pass's float32 normalisers, so they are the same
// numbers the main pass selected on.
__global__ __launch_bounds__(256) void product_topk_fixup_kernel(
    const float* __restrict__ Zr, const float* __restrict__ Zc, int L, int Nr, int Nc, int kp,
    int K, const int32_t* __restrict__ row_sel, const int32_t* __restrict__ col_sel,
    const int32_t* __restrict__ tie_flag, const float* __restrict__ lse,
    int32_t* __restrict__ expert_idx, float* __restrict__ score, float* __restrict__ gate) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6), l = lane();
  if (t >= L || tie_flag[t] == 0) return;
  int ri = 0, ci = 0;
  float av = 0.f, bv = 0.f;
  if (l < kp) {
    ri = row_sel[static_cast<size_t>(t) * kp + l];
    ci = col_sel[static_cast<size_t>(t) * kp + l];
    ri = min(max(ri, 0), Nr - 1);
    ci = min(max(ci, 0), Nc - 1);
    av = Zr[static_cast<size_t>(t) * Nr + ri] - lse[2 * static_cast<size_t>(t)];
    bv = Zc[static_cast<size_t>(t) * Nc + ci] - lse[2 * static_cast<size_t>(t) + 1];
  }
  uint64_t prev = ~0ull, mine = 0;
  for (int k = 0; k < K; ++k) {
    uint64_t cur = 0;
    for (int c = 0; c < kp; ++c) {
      const float bc = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), c));
      const uint32_t cc = static_cast<uint32_t>(__builtin_amdgcn_readlane(ci, c));
      const uint64_t key = sel_key(av + bc, static_cast<uint32_t>(ri) * Nc + cc);
      if (l < kp && key < prev && key > cur) cur = key;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const uint64_t u = __shfl_xor(cur, o);
      cur = cur > u ? cur : u;
    }
    if (l == k) mine = cur;
    prev = cur;
  }
  write_outputs(mine, t, K, expert_idx, score, gate);
}

hipError_t launch_product_topk(const float* zr, const float* zc, int L, int Nr, int Nc, int kp,
                               int K, int32_t* expert_idx, float* score, float* gate,
                               float* row_logp, float* col_logp, int32_t* row_sel,
                               int32_t* col_sel, int32_t* tie_flag, float* lse,
                               hipStream_t s) {
  if (L == 0) return hipSuccess;
  const int n = Nr > Nc ? Nr : Nc;
  const int grid = (L + 3) / 4;
#define OMNI_TOPK(NI_)                                                                     \
  product_topk_kernel<NI_><<<grid, 256, 0, s>>>(zr, zc, L, Nr, Nc, kp, K, expert_idx, score, \
                                                gate, row_logp, col_logp, row_sel, col_sel,  \
                                                tie_flag, lse)
  if (n <= 64) OMNI_TOPK(1);
  else if (n <= 128) OMNI_TOPK(2);
  else if (n <= 256) OMNI_TOPK(4);
  else if (n <= 512) OMNI_TOPK(8);
  else if (n <= 1024) OMNI_TOPK(16);
  else OMNI_TOPK(32);
#undef OMNI_TOPK
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  product_topk_fixup_kernel<<<grid, 256, 0, s>>>(zr, zc, L, Nr, Nc, kp, K, row_sel, col_sel,
                                                 tie_flag, lse, expert_idx, score, gate);
  return hipGetLastError();
}

}  // namespace omni
