// Expert-Centric Scheduling of a small batch (at most kSmallM = 16,384 tasks
// and as many groups) in one workgroup, one launch.  Pages: interactive
// explainer "Expert-Centric Scheduling" (flatten the L*K decisions into
// tasks; collect the unique active experts sorted by id and cut them into
// groups of B; order the tasks by group, then token) and gist.science
// explainer §2.2.  It writes exactly what the multi-kernel pipeline of
// schedule.hip writes; that pipeline costs six launches at decode sizes,
// which dominate there (a few thousand tasks).
//
// Everything happens in LDS (two 16,384-word buffers):
//   1. the task ids, invalid ones replaced by a sentinel above every valid id,
//      sorted by a stable LSD radix sort (8-bit digits, lanes with the same
//      digit found with 8 ballots, per-wave running counts);
//   2. the unique valid ids, by a block scan: the active list and n_active;
//   3. every task's group key (rank / B, or e / B for id windows; the rank
//      by binary search in the active list), packed with its flat index m as
//      (key << 14) | m, so a plain sort of the words orders by (group, m),
//      i.e. (group, token, k);
//   4. the words sorted by their key bits, then the task arrays and the CSR
//      group offsets written from them.
#include "device.hpp"
#include "launch.hpp"

namespace omni {

constexpr int kSmallM = 16384;        // tasks (and groups) the one-workgroup schedule takes
constexpr int kSmT = 1024;            // threads
constexpr int kSmR = kSmallM / kSmT;  // words per thread
constexpr int kSmW = kSmT / 64;       // waves
constexpr int kSmIdx = 14;            // bits of the flat index in a packed word

struct SmLds {
  uint32_t buf[2][kSmallM];  // ping-pong buffers, indexed (no pointers into LDS)
  uint32_t wh[kSmW][256];  // per-wave digit counts, then their bases
  uint32_t dbase[256];     // digit totals, then the digits' first positions
  uint32_t red[kSmW];
};

// Exclusive prefix over the workgroup of one value per thread (thread order);
// also returns the total.
__device__ __forceinline__ uint32_t sm_block_scan(uint32_t v, uint32_t* red, uint32_t& total) {
  const int w = threadIdx.x >> 6, l = lane();
  const uint32_t inc = wave_inclusive_scan(v);
  if (l == 63) red[w] = inc;
  __syncthreads();
  uint32_t before = 0, all = 0;
  for (int q = 0; q < kSmW; ++q) {
    const uint32_t r = red[q];
    before += q < w ? r : 0u;
    all += r;
  }
  __syncthreads();  // red is reused by the next call
  total = all;
  return before + inc - v;
}

// One stable pass of an LSD radix sort over all kSmallM words: digit
// (v >> shift) & 255, buf[cur] -> buf[cur ^ 1].  Wave w ranks words
// [1024 w, 1024 w + 1024) 64 at a time, in order.
__device__ __forceinline__ void sm_radix_pass(SmLds& S, int cur, int shift) {
  const int tid = threadIdx.x, w = tid >> 6, l = lane();
  const uint64_t lt = l == 0 ? 0ull : (~0ull >> (64 - l));
  for (int i = tid; i < kSmW * 256; i += kSmT) (&S.wh[0][0])[i] = 0;
  __syncthreads();
  uint32_t v[kSmR], dg[kSmR], lr[kSmR];
  const int base = w * (kSmR * 64);
#pragma unroll
  for (int r = 0; r < kSmR; ++r) v[r] = S.buf[cur][base + r * 64 + l];
#pragma unroll
  for (int r = 0; r < kSmR; ++r) {
    const uint32_t d = (v[r] >> shift) & 255u;
    uint64_t peers = ~0ull;
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
      const bool on = (d >> bit) & 1u;
      const uint64_t bm = __ballot(on);
      peers &= on ? bm : ~bm;
    }
    const uint64_t below = peers & lt;
    const uint32_t before = S.wh[w][d];
    wave_lds_fence();
    if (below == 0) S.wh[w][d] = before + static_cast<uint32_t>(__popcll(peers));
    wave_lds_fence();
    dg[r] = d;
    lr[r] = before + static_cast<uint32_t>(__popcll(below));
  }
  __syncthreads();
  uint32_t tot = 0;
  if (tid < 256) {  // exclusive prefix over the waves of each digit, and its total
#pragma unroll
    for (int q = 0; q < kSmW; ++q) {
      const uint32_t c = S.wh[q][tid];
      S.wh[q][tid] = tot;
      tot += c;
    }
  }
  // exclusive prefix of the digit totals (threads past 255 add nothing)
  uint32_t all;
  const uint32_t first = sm_block_scan(tid < 256 ? tot : 0u, S.red, all);
  if (tid < 256) S.dbase[tid] = first;
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kSmR; ++r) S.buf[cur ^ 1][S.dbase[dg[r]] + S.wh[w][dg[r]] + lr[r]] = v[r];
  __syncthreads();
}

// First index in [0, n) of list (ascending) holding a value >= v.
__device__ __forceinline__ int sm_lower_bound(const uint32_t (&list)[kSmallM], int n, uint32_t v) {
  int lo = 0;
  while (n > 0) {
    const int h = n >> 1;
    if (list[lo + h] < v) {
      lo += h + 1;
      n -= h + 1;
    } else {
      n = h;
    }
  }
  return lo;
}

// id_bits: 2^id_bits >= N (the sentinel 2^id_bits sorts after every valid
// id); key_bits: 2^key_bits >= G.
__global__ __launch_bounds__(kSmT) void schedule_small_kernel(
    int L, int K, int N, int B, int window, int G, int id_bits, int key_bits,
    const int32_t* __restrict__ expert_idx, const float* __restrict__ gate,
    int32_t* __restrict__ counts, int32_t* __restrict__ active,
    int32_t* __restrict__ group_offsets, int32_t* __restrict__ task_token,
    int32_t* __restrict__ task_expert, float* __restrict__ task_gate,
    int32_t* __restrict__ task_index) {
  __shared__ SmLds S;
  const int tid = threadIdx.x;
  const int M = L * K;
  const uint32_t sentinel = 1u << id_bits;
  // 1. the ids (task tid + 1024 j in ev[j]; all loads issued together), sorted
  int ev[kSmR];
#pragma unroll
  for (int j = 0; j < kSmR; ++j) {
    const int i = tid + j * kSmT;
    ev[j] = i < M ? expert_idx[i] : -1;
  }
#pragma unroll
  for (int j = 0; j < kSmR; ++j)
    S.buf[0][tid + j * kSmT] = static_cast<unsigned>(ev[j]) < static_cast<unsigned>(N)
                                   ? static_cast<uint32_t>(ev[j])
                                   : sentinel;
  __syncthreads();
  int cur = 0;
  for (int shift = 0; shift <= id_bits; shift += 8) {  // bits 0 .. id_bits
    sm_radix_pass(S, cur, shift);
    cur ^= 1;
  }
  // 2. the unique valid ids: thread tid takes sorted positions [16 tid, 16 tid + 16)
  uint32_t flags = 0, nflag = 0;
#pragma unroll
  for (int j = 0; j < kSmR; ++j) {
    const int i = tid * kSmR + j;
    const uint32_t v = S.buf[cur][i];
    const bool first = v < sentinel && (i == 0 || S.buf[cur][i - 1] != v);
    flags |= (first ? 1u : 0u) << j;
    nflag += first ? 1u : 0u;
  }
  uint32_t n_active;
  uint32_t r = sm_block_scan(nflag, S.red, n_active);
#pragma unroll
  for (int j = 0; j < kSmR; ++j) {
    if ((flags >> j) & 1u) {
      const uint32_t v = S.buf[cur][tid * kSmR + j];
      S.buf[cur ^ 1][r] = v;  // the active list, in LDS for the rank lookups
      active[r] = static_cast<int32_t>(v);
      ++r;
    }
  }
  __syncthreads();
  // 3. packed (group key, flat index) words, in buf[cur] (the sorted ids are done)
#pragma unroll
  for (int j = 0; j < kSmR; ++j) {
    const int m = tid + j * kSmT;
    uint32_t word = 0xffffffffu;  // the padding sorts last
    if (m < M) {
      const int e = ev[j];
      uint32_t key = 0;  // an invalid id goes to group 0
      if (static_cast<unsigned>(e) < static_cast<unsigned>(N))
        key = window ? static_cast<uint32_t>(e / B)
                     : static_cast<uint32_t>(sm_lower_bound(S.buf[cur ^ 1],
                                                            static_cast<int>(n_active),
                                                            static_cast<uint32_t>(e)) /
                                             B);
      word = (key << kSmIdx) | static_cast<uint32_t>(m);
    }
    S.buf[cur][m] = word;
  }
  __syncthreads();
  // 4. sort by the key bits, then write the tasks and the offsets
  for (int shift = kSmIdx; shift < kSmIdx + key_bits; shift += 8) {
    sm_radix_pass(S, cur, shift);
    cur ^= 1;
  }
  // the sorted words of positions tid + 1024 j, then every gather issued
  // before the first store
  int mv[kSmR], gv[kSmR], ex[kSmR];
  float gt[kSmR];
#pragma unroll
  for (int j = 0; j < kSmR; ++j) {
    const int p = tid + j * kSmT;
    const uint32_t w = S.buf[cur][p];  // padding words for p >= M
    mv[j] = static_cast<int>(w & ((1u << kSmIdx) - 1));
    gv[j] = static_cast<int>(w >> kSmIdx);
  }
#pragma unroll
  for (int j = 0; j < kSmR; ++j) {
    const int m = min(mv[j], M - 1);  // padding: any valid index, never stored
    ex[j] = expert_idx[m];
    gt[j] = gate[m];
  }
#pragma unroll
  for (int j = 0; j < kSmR; ++j) {
    const int p = tid + j * kSmT;
    if (p >= M) continue;
    const int m = mv[j], g = gv[j];
    task_token[p] = m / K;
    task_expert[p] = ex[j];
    task_gate[p] = gt[j];
    if (task_index) task_index[p] = m;
    // off[q] = first position of a group >= q, for q in (previous key, g]
    const int gp = p ? static_cast<int>(S.buf[cur][p - 1] >> kSmIdx) : -1;
    for (int q = gp + 1; q <= g && q <= G; ++q) group_offsets[q] = p;
    if (p == M - 1)
      for (int q = g + 1; q <= G; ++q) group_offsets[q] = M;
  }
  if (tid == 0) {
    counts[0] = static_cast<int32_t>(n_active);
    counts[1] = window ? static_cast<int32_t>((static_cast<long long>(N) + B - 1) / B)
                       : static_cast<int32_t>((n_active + B - 1) / B);
  }
}

bool schedule_small_fits(long long M, long long G) {
  return M >= 1 && M <= kSmallM && G <= kSmallM;
}

hipError_t launch_schedule_small(int L, int K, int N, int B, int window, int G,
                                 const int32_t* expert_idx, const float* gate, int32_t* counts,
                                 int32_t* active, int32_t* group_offsets, int32_t* task_token,
                                 int32_t* task_expert, float* task_gate, int32_t* task_index,
                                 hipStream_t s) {
  if (!schedule_small_fits(static_cast<long long>(L) * K, G)) return hipErrorInvalidValue;
  int id_bits = 0;
  while ((1ll << id_bits) < N) ++id_bits;
  int key_bits = 1;
  while ((1ll << key_bits) < G) ++key_bits;
  hipLaunchKernelGGL(schedule_small_kernel, dim3(1), dim3(kSmT), 0, s, L, K, N, B, window, G,
                     id_bits, key_bits, expert_idx, gate, counts, active, group_offsets,
                     task_token, task_expert, task_gate, task_index);
  return hipGetLastError();
}

}  // namespace omni
