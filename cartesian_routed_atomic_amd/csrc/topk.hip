// Cartesian Product Router, part 2: per-axis log-probabilities and top-k',
// top-K over the product cells, gates.  Pages: interactive explainer
// "Cartesian Product Router" (row and column distributions p_r, p_c; rows and
// columns are searched separately; the joint score S_ij = log p_r[i] +
// log p_c[j] is additive in log space and the N-entry score matrix is never
// formed) and "Expert-Centric Scheduling" (every decision carries a weight;
// the gate is the softmax over the K selected scores).
//
// Two waves (64 lanes each) serve one token: one per axis, then one merges.
//
// Per axis the wave reads the logit row once, forms a = z - (m + ln sum
// exp(z - m)) in float32, optionally stores it, and selects the k' largest a
// with an MSB-first radix select over 32-bit order-preserving value keys
// (bits shared by all candidates are skipped; ties at the threshold value
// are taken in index order, which is the lane/slot order of the row).  The
// winners are put in (value key << 32 | ~index) order by a rank sort: each
// lane counts the keys above its own.
//
// Product merge.  With rank-ordered axis lists R (rows) and C (columns),
// S(r, c) = fl32(a[R_r] + b[C_c]) is non-increasing in r and in c (float
// addition is monotone).  For any cell outside the staircase
// P = {(r, c) : (r+1)(c+1) <= K} at least K cells of P dominate it, so the
// K-th best value over P, tau, bounds everything outside P from above.  The
// kernel therefore selects the top K of P (|P| <= 280 for K, k' <= 64) and
// checks, per row, the first cell past the staircase: if none reaches tau
// the answer is exact.  Otherwise (a float32 tie at tau) the token is
// flagged and its wave redoes its top K over all k'^2 cells, plainly: K
// rounds, each taking the largest cell key below the previous round's.
#include "device.hpp"
#include "launch.hpp"

namespace omni {

// ---------------------------------------------------------------- selection

// Number of the wave's keys >= c (NI keys per lane; key 0 is an empty slot
// and never counts, since every c used here is >= 1).  One compare and a
// ballot per slot; the counts are summed in scalar registers.
template <int NI>
__device__ __forceinline__ int wave_count_ge(const uint32_t (&vk)[NI], uint32_t c) {
  int n = 0;
#pragma unroll
  for (int j = 0; j < NI; ++j) n += __popcll(__ballot(vk[j] >= c));
  return n;
}

// State of an exact k-th-largest search over 32-bit keys: the answer is
// built bit by bit from the most significant bit where the keys differ.
// Invariant: n = #keys >= prefix >= k.  When n reaches k the k largest keys
// are exactly those >= prefix and the search stops early; otherwise it ends
// with prefix = the k-th largest key and n = #keys >= it (ties at it).
struct KthSearch {
  uint32_t prefix;
  int n, bit;  // bit < 0: finished
};

template <int NI>
__device__ __forceinline__ KthSearch kth_begin(const uint32_t (&vk)[NI], int k) {
  uint32_t a = ~0u, o = 0u;
  int items = 0;
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    a &= vk[j] ? vk[j] : ~0u;
    o |= vk[j];
    items += __popcll(__ballot(vk[j] != 0u));
  }
  a = wave_and32(a);
  o = wave_or32(o);
  const uint32_t diff = a ^ o;
  if (diff == 0u || items == k) return KthSearch{items == k ? a : o, items, -1};
  const int h = 31 - __clz(diff);
  const uint32_t low = (h == 31) ? ~0u : ((2u << h) - 1u);  // bits h..0
  return KthSearch{a & ~low, items, h};
}

template <int NI>
__device__ __forceinline__ void kth_step(KthSearch& s, const uint32_t (&vk)[NI], int k) {
  if (s.bit < 0) return;
  const uint32_t c = s.prefix | (1u << s.bit);
  const int n = wave_count_ge<NI>(vk, c);
  if (n >= k) {
    s.prefix = c;
    s.n = n;
  }
  s.bit = (s.n == k) ? -1 : s.bit - 1;
}

// Sort the k (<= 64) distinct keys buf[0..k) descending; buf[k..64) must be
// 0.  Each lane counts the keys above its own with broadcast LDS reads (no
// cross-lane shuffles on the critical path), then stores its key at that
// rank in `out`.  Returns rank r in lane r (0 past k).
__device__ __forceinline__ uint64_t rank_sort64(const uint64_t (&buf)[64], uint64_t (&out)[64],
                                                int k) {
  const int l = lane();
  const uint64_t mine = buf[l];
  int rank = 0;
#pragma unroll
  for (int i = 0; i < 64; i += 2) {
    const ulonglong2 p = *reinterpret_cast<const ulonglong2*>(&buf[i]);
    rank += (p.x > mine) + (p.y > mine);
  }
  if (l < k) out[rank] = mine;
  wave_lds_fence();
  const uint64_t r = (l < k) ? out[l] : 0ull;
  wave_lds_fence();
  return r;
}

// The k largest axis items (value key desc, index asc) into buf as
// (key << 32 | ~index), buf zero-padded to 64.  Slot j of lane l is index
// j * 64 + l, so slot order is index order and ties at the threshold are
// taken in index order.
template <int NI>
__device__ __forceinline__ void axis_collect(const uint32_t (&vk)[NI], const KthSearch& s, int k,
                                             uint64_t (&buf)[64]) {
  const int l = lane();
  buf[l] = 0ull;
  wave_lds_fence();
  const bool all_ge = s.n == k;  // no partial ties: take every key >= prefix
  int base = 0;
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const bool in = vk[j] != 0u && (all_ge ? vk[j] >= s.prefix : vk[j] > s.prefix);
    const uint64_t m = __ballot(in);
    if (in) buf[base + mbcnt(m)] = (static_cast<uint64_t>(vk[j]) << 32) |
                                   static_cast<uint32_t>(~(j * 64 + l));
    base += __popcll(m);
  }
  if (!all_ge) {
    int rest = k - base;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const bool eq = rest > 0 && vk[j] == s.prefix;
      const uint64_t m = __ballot(eq);
      const int r = mbcnt(m);
      if (eq && r < rest)
        buf[base + r] = (static_cast<uint64_t>(vk[j]) << 32) |
                        static_cast<uint32_t>(~(j * 64 + l));
      const int taken = min(__popcll(m), max(rest, 0));
      base += taken;
      rest -= taken;
    }
  }
  wave_lds_fence();
}

// The k largest of a wave's 64-bit keys held in two 32-bit words per slot
// (hi = value key, lo = ~index; 0/0 = empty; keys distinct), as a predicate
// per slot: first the k-th largest value word, then, if several slots tie at
// it, the split among the tied slots by their lo words.
struct Top64 {
  uint32_t T, T2;  // take hi > T, or hi == T && lo >= T2 (T2 = 0 takes every hi == T)
};

template <int NI>
__device__ __forceinline__ Top64 top64_finish(const uint32_t (&hi)[NI], const uint32_t (&lo)[NI],
                                              int k, const KthSearch& q) {
  if (q.n == k) return Top64{q.prefix, 0u};  // every key with hi >= prefix
  uint32_t tk[NI];
  int n_gt = 0;
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    tk[j] = (hi[j] == q.prefix) ? lo[j] : 0u;
    n_gt += __popcll(__ballot(hi[j] > q.prefix));
  }
  KthSearch qt = kth_begin<NI>(tk, k - n_gt);
  while (qt.bit >= 0) kth_step<NI>(qt, tk, k - n_gt);
  return Top64{q.prefix, qt.prefix};
}

template <int NI>
__device__ __forceinline__ bool top64_take(const Top64& s, uint32_t hi, uint32_t lo) {
  return hi != 0u && (hi > s.T || (hi == s.T && lo >= s.T2));
}

// Write the taken keys to buf[0..k) (slot order), buf zero-padded to 64.
template <int NI>
__device__ __forceinline__ void top64_collect(const uint32_t (&hi)[NI], const uint32_t (&lo)[NI],
                                              const Top64& s, uint64_t (&buf)[64]) {
  const int l = lane();
  buf[l] = 0ull;
  wave_lds_fence();
  int base = 0;
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const bool in = top64_take<NI>(s, hi[j], lo[j]);
    const uint64_t m = __ballot(in);
    if (in) buf[base + mbcnt(m)] = (static_cast<uint64_t>(hi[j]) << 32) | lo[j];
    base += __popcll(m);
  }
  wave_lds_fence();
}

// Items of one axis with value key >= v, compacted in index order into
// cand[0..128) as (key << 32 | ~index), zero-padded; returns them two per
// lane (cand[l], cand[64 + l]) and true, or false (hi, lo unset) when more
// than 128 items pass (then only the first 128 are written).
template <int NI>
__device__ __forceinline__ bool axis_compact(const uint32_t (&vk)[NI], uint32_t v,
                                             uint64_t (&cand)[128],
                                             uint32_t (&hi)[2], uint32_t (&lo)[2]) {
  const int l = lane();
  cand[l] = 0ull;
  cand[64 + l] = 0ull;
  wave_lds_fence();
  int base = 0;
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const bool in = vk[j] >= v && vk[j] != 0u;
    const uint64_t m = __ballot(in);
    const int at = base + mbcnt(m);
    if (in && at < 128)
      cand[at] = (static_cast<uint64_t>(vk[j]) << 32) | static_cast<uint32_t>(~(j * 64 + l));
    base += __popcll(m);
  }
  wave_lds_fence();
  if (base > 128) return false;
  const uint64_t a = cand[l], b = cand[64 + l];
  hi[0] = static_cast<uint32_t>(a >> 32);
  lo[0] = static_cast<uint32_t>(a);
  hi[1] = static_cast<uint32_t>(b >> 32);
  lo[1] = static_cast<uint32_t>(b);
  wave_lds_fence();
  return true;
}

// Per-lane two largest keys (0 = empty).
template <int NI>
__device__ __forceinline__ void lane_top2(const uint32_t (&vk)[NI], uint32_t (&t)[2]) {
  uint32_t t1 = 0u, t2 = 0u;
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const uint32_t v = vk[j];
    t2 = v > t1 ? t1 : (v > t2 ? v : t2);
    t1 = v > t1 ? v : t1;
  }
  t[0] = t1;
  t[1] = t2;
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

struct TopkLds {
  uint64_t cand[2][128]; // per axis: the items that pass the pre-filter
  uint64_t buf[2][64];   // per axis: selected items, then the merge's K cells
  uint64_t srt[2][64];   // rank-sorted copies
  float av[64];
  float bv[64];
  uint32_t R[64];
  uint32_t C[64];
  int poff[68];
  uint8_t rowstart[320];  // 1 at the first staircase cell of each row
};

constexpr int kStairItems = 5;  // ceil(280 / 64): |P| <= 280 for K, k' <= 64
static_assert(kStairItems * 64 <= 320, "one rowstart byte per staircase slot");

// The product merge of one token, by one wave, from the rank-ordered axis
// lists in S (av, R: rows; bv, C: columns): the staircase cells, their top K,
// the tie check against the first cell past the staircase in each row, the
// exact walk for a tied token, then gates and outputs.
__device__ __forceinline__ void product_merge(TopkLds& S, int kp, int K, int Nc, int t,
                                              int32_t* __restrict__ expert_idx,
                                              float* __restrict__ score,
                                              float* __restrict__ gate,
                                              int32_t* __restrict__ tie_flag) {
  const int l = lane();
  // ---- staircase P: row r contributes columns c < len_r = min(k', K / (r + 1))
  const int len = (l < kp) ? min(kp, K / (l + 1)) : 0;
  const int inc = wave_prefix_sum(len);
  if (l < kp) S.poff[l + 1] = inc;
  if (l == 0) S.poff[0] = 0;
  const int P = __builtin_amdgcn_readlane(inc, 63);
  // The row of cell p is the number of rows that begin at or before p, less
  // one (rows with cells begin at distinct offsets; empty rows come last):
  // each row marks its first cell, and the lanes of a block of 64 cells count
  // the marks with one ballot.
  uint32_t* rs = reinterpret_cast<uint32_t*>(S.rowstart);
  rs[l] = 0u;
  if (l < 320 / 4 - 64) rs[64 + l] = 0u;
  wave_lds_fence();
  if (len > 0) S.rowstart[inc - len] = 1;
  wave_lds_fence();
  uint32_t phi[kStairItems], plo[kStairItems];  // cell key = value key << 32 | ~expert
  int rows_before = 0;  // rows that begin in the blocks before this one
#pragma unroll
  for (int j = 0; j < kStairItems; ++j) {
    const int p = l + 64 * j;
    const bool first = p < P && S.rowstart[p] != 0;
    const uint64_t m = __ballot(first);
    const int r = rows_before + mbcnt(m) + (first ? 1 : 0) - 1;
    rows_before += __popcll(m);
    phi[j] = 0u;
    plo[j] = 0u;
    if (p < P) {
      const int c = p - S.poff[r];
      phi[j] = fkey(S.av[r] + S.bv[c]);
      plo[j] = ~(S.R[r] * static_cast<uint32_t>(Nc) + S.C[c]);
    }
  }
  // K best cells by (value desc, expert asc): value threshold first; cells
  // tied at it are split by a second search on ~expert among them.
  KthSearch qm = kth_begin<kStairItems>(phi, K);
  while (qm.bit >= 0) kth_step<kStairItems>(qm, phi, K);
  uint64_t (&mb)[64] = S.buf[0];
  top64_collect<kStairItems>(phi, plo, top64_finish<kStairItems>(phi, plo, K, qm), mb);
  const uint64_t best = rank_sort64(mb, S.srt[0], K);
  const uint32_t tau = static_cast<uint32_t>(__shfl(best, K - 1) >> 32);

  // ---- a cell past the staircase can only tie at tau; check each row's first
  bool extra = false;
  if (l < kp && len < kp) extra = fkey(S.av[l] + S.bv[len]) >= tau;
  const bool tie = __ballot(extra) != 0ull;
  if (l == 0) tie_flag[t] = tie ? 1 : 0;
  uint64_t out = best;
  if (tie) {
    // Exact top K over all k' x k' cells: K rounds, each taking the largest
    // cell key below the previous round's.  Lane r owns row r; the columns
    // are walked one at a time from LDS.  The axis values are the ones the
    // selection above used.
    const float av = (l < kp) ? S.av[l] : 0.f;
    const uint32_t rbase = (l < kp) ? S.R[l] * static_cast<uint32_t>(Nc) : 0u;
    uint64_t prev = ~0ull;
    out = 0ull;
    for (int k = 0; k < K; ++k) {
      uint64_t cur = 0ull;
      for (int c = 0; c < kp; ++c) {
        const uint64_t key = sel_key(av + S.bv[c], rbase + S.C[c]);
        if (l < kp && key < prev && key > cur) cur = key;
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const uint64_t u = __shfl_xor(cur, o);
        cur = cur > u ? cur : u;
      }
      if (l == k) out = cur;
      prev = cur;
    }
  }
  write_outputs(out, t, K, expert_idx, score, gate);
}

// Two waves per token: wave 0 takes the rows, wave 1 the columns (log-sum-exp,
// value keys, pre-filter, exact top-k', rank order), then wave 0 merges.  Per
// token the work is a chain of dependent steps (wave reductions, ballots, LDS
// round trips); splitting the two axes over two waves halves the axis part of
// that chain and doubles the waves that hide each other's latency.
// tie_flag[t] = 1 marks a token whose K-th score ties a cell past the
// staircase (its outputs then come from the exact walk over all cells);
// lse[2t], lse[2t+1] keep the row / column normalisers.  FULL: both axes
// have exactly NI * 64 lines (every slot holds a line; no per-slot guards).
template <int NI, bool FULL>
__global__ __launch_bounds__(128) void product_topk_kernel(
    const float* __restrict__ Zr, const float* __restrict__ Zc, int L, int Nr, int Nc, int kp,
    int K, int32_t* __restrict__ expert_idx, float* __restrict__ score,
    float* __restrict__ gate, float* __restrict__ row_logp, float* __restrict__ col_logp,
    int32_t* __restrict__ row_sel, int32_t* __restrict__ col_sel,
    int32_t* __restrict__ tie_flag, float* __restrict__ lse_out) {
  static_assert(NI <= 32, "32 slots per lane at most");
  __shared__ TopkLds S;
  const int w = threadIdx.x >> 6, l = lane();
  const int t = blockIdx.x;
  if (t >= L) return;  // the whole workgroup leaves together
  const int n = w ? Nc : Nr;
  const float* zrow = (w ? Zc : Zr) + static_cast<size_t>(t) * n;
  float z[NI];
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const int i = j * 64 + l;
    z[j] = (FULL || i < n) ? zrow[i] : -INFINITY;
  }
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < NI; ++j) m = fmaxf(m, z[j]);
  m = wave_max(m);
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < NI; ++j)
    if (FULL || j * 64 + l < n) sum += __expf(z[j] - m);
  sum = wave_sum(sum);
  const float lse = m + __logf(sum);
  if (l == 0) lse_out[2 * static_cast<size_t>(t) + w] = lse;
  float* logp = w ? col_logp : row_logp;
  uint32_t k[NI];
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const int i = j * 64 + l;
    const float a = z[j] - lse;
    k[j] = (FULL || i < n) ? fkey(a) : 0u;
    if (logp && (FULL || i < n)) logp[static_cast<size_t>(t) * n + i] = a;
  }
  // The k' best lines of this axis.  Pre-filter: v = the k'-th largest of the
  // per-lane top-2 keys is a lower bound of the k'-th largest key (k' keys
  // are >= v), and for Gaussian-like rows only ~70 keys reach it.  Those are
  // compacted two per lane and searched exactly; more than 128 fall back to
  // the search over all slots (both searches are exact).
  uint32_t tp[2];
  lane_top2<NI>(k, tp);
  KthSearch f = kth_begin<2>(tp, kp);
  while (f.bit >= 0) kth_step<2>(f, tp, kp);
  uint32_t h[2], lo[2];
  if (axis_compact<NI>(k, f.prefix, S.cand[w], h, lo)) {
    KthSearch q = kth_begin<2>(h, kp);
    while (q.bit >= 0) kth_step<2>(q, h, kp);
    top64_collect<2>(h, lo, top64_finish<2>(h, lo, kp, q), S.buf[w]);
  } else {
    KthSearch q = kth_begin<NI>(k, kp);
    while (q.bit >= 0) kth_step<NI>(q, k, kp);
    axis_collect<NI>(k, q, kp, S.buf[w]);
  }
  const uint64_t rk = rank_sort64(S.buf[w], S.srt[w], kp);
  if (l < kp) {
    (w ? S.bv : S.av)[l] = sel_val(rk);
    (w ? S.C : S.R)[l] = sel_idx(rk);
    (w ? col_sel : row_sel)[static_cast<size_t>(t) * kp + l] = static_cast<int32_t>(sel_idx(rk));
  }
  __syncthreads();
  if (w != 0) return;
  product_merge(S, kp, K, Nc, t, expert_idx, score, gate, tie_flag);
}

hipError_t launch_product_topk(const float* zr, const float* zc, int L, int Nr, int Nc, int kp,
                               int K, int32_t* expert_idx, float* score, float* gate,
                               float* row_logp, float* col_logp, int32_t* row_sel,
                               int32_t* col_sel, int32_t* tie_flag, float* lse,
                               hipStream_t s) {
  if (L == 0) return hipSuccess;
  const int n = Nr > Nc ? Nr : Nc;
#define OMNI_TOPK_F(NI_, F_)                                                                   \
  hipLaunchKernelGGL(HIP_KERNEL_NAME(product_topk_kernel<NI_, F_>), dim3(L), dim3(128), 0, s,  \
                     zr, zc, L, Nr, Nc, kp, K, expert_idx, score, gate, row_logp, col_logp,    \
                     row_sel, col_sel, tie_flag, lse)
#define OMNI_TOPK(NI_)                                 \
  do {                                                 \
    if (Nr == (NI_) * 64 && Nc == (NI_) * 64)          \
      OMNI_TOPK_F(NI_, true);                          \
    else                                               \
      OMNI_TOPK_F(NI_, false);                         \
  } while (0)
  if (n <= 64) OMNI_TOPK(1);
  else if (n <= 128) OMNI_TOPK(2);
  else if (n <= 256) OMNI_TOPK(4);
  else if (n <= 512) OMNI_TOPK(8);
  else if (n <= 1024) OMNI_TOPK(16);
  else OMNI_TOPK(32);
#undef OMNI_TOPK
#undef OMNI_TOPK_F
  return hipGetLastError();
}

}  // namespace omni
