// Expert-Centric Scheduling.  Pages: interactive explainer "Expert-Centric
// Scheduling" (flatten every (token, expert, weight) decision into M = L*K
// tasks; collect the unique active experts, sort them by id, cut them into
// groups of B; order the tasks by group first and token second) and
// gist.science explainer §2.2 (task collection, grouping and sorting).
//
// Device pipeline, no host synchronisation (n_active and n_groups stay on
// the device):
//   1. clear a byte flag per expert, then mark every expert some task uses
//      (read-before-write, so hot experts cause few stores);
//   2. count flags per 4096-expert tile; each tile sums the counts of the
//      tiles before it, scans its own flags and writes rank[e] (position
//      among active experts) and the ascending active list;
//   3. key[m] = rank[e_m] / B, the group of task m;
//   4. stable LSD radix sort of the tasks by group, 8 bits per pass.  Tasks
//      enter in flatten order m = t*K + k, which is already token-major, so a
//      stable sort by group alone yields (group, token) order with ties in
//      flatten order.  Each pass: per-tile digit histograms, one exclusive
//      scan, then a stable scatter ranked with 8 ballots per element;
//   5. CSR group offsets from the group boundaries of the sorted keys.
#include "device.hpp"
#include "launch.hpp"

namespace omni {

constexpr int kTile = 4096;  // elements per workgroup tile (256 threads x 16)

static inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

ScheduleWs schedule_ws_layout(int L, int K, int N, int B) {
  ScheduleWs w{};
  const long long M = static_cast<long long>(L) * K;
  w.n_ftiles = static_cast<int>((static_cast<long long>(N) + kTile - 1) / kTile);
  w.n_ttiles = static_cast<int>((M + kTile - 1) / kTile);
  const long long mn = M < N ? M : N;
  w.max_groups = static_cast<int>((mn + B - 1) / B);
  int bits = 0;
  while (bits < 31 && (1ll << bits) < w.max_groups) ++bits;  // groups are < max_groups
  w.passes = bits <= 8 ? 1 : (bits + 7) / 8;
  size_t o = 0;
  w.flags = o;    o = align256(o + static_cast<size_t>(w.n_ftiles) * kTile);
  w.tile_cnt = o; o = align256(o + static_cast<size_t>(w.n_ftiles) * 4);
  w.rank = o;     o = align256(o + static_cast<size_t>(N) * 4);
  w.key0 = o;     o = align256(o + static_cast<size_t>(M) * 4);
  w.val0 = o;     o = align256(o + static_cast<size_t>(M) * 4);
  w.key1 = o;     o = align256(o + static_cast<size_t>(M) * 4);
  w.val1 = o;     o = align256(o + static_cast<size_t>(M) * 4);
  w.hist = o;     o = align256(o + static_cast<size_t>(256) * (w.n_ttiles > 0 ? w.n_ttiles : 1) * 4);
  w.bytes = o;
  return w;
}

__global__ __launch_bounds__(256) void zero16_kernel(uint4* __restrict__ p, size_t n16) {
  const size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n16) p[i] = make_uint4(0, 0, 0, 0);
}

// Ids outside [0, N) are ignored here and sent to group 0 below: the result is
// then unspecified but every access stays in bounds.
__global__ __launch_bounds__(256) void mark_kernel(const int32_t* __restrict__ idx, int M, int N,
                                                   uint8_t* __restrict__ flags) {
  const int m = blockIdx.x * 256 + threadIdx.x;
  if (m >= M) return;
  const int e = idx[m];
  if (static_cast<unsigned>(e) < static_cast<unsigned>(N) && flags[e] == 0) flags[e] = 1;
}

// block-wide sum over 256 threads (4 waves); red: 4 ints of LDS
__device__ __forceinline__ int block_sum256(int v, int* red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  if (lane() == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  const int r = red[0] + red[1] + red[2] + red[3];
  __syncthreads();
  return r;
}

// popcount of a word whose bytes are each 0 or 1 = number of set flags
__device__ __forceinline__ int flag_count(uint4 v) {
  return __popc(v.x) + __popc(v.y) + __popc(v.z) + __popc(v.w);
}

__global__ __launch_bounds__(256) void tile_count_kernel(const uint8_t* __restrict__ flags,
                                                         int* __restrict__ tile_cnt) {
  __shared__ int red[4];
  const uint4 v = reinterpret_cast<const uint4*>(flags + static_cast<size_t>(blockIdx.x) * kTile)[threadIdx.x];
  const int s = block_sum256(flag_count(v), red);
  if (threadIdx.x == 0) tile_cnt[blockIdx.x] = s;
}

__global__ __launch_bounds__(256) void rank_kernel(const uint8_t* __restrict__ flags, int N,
                                                   const int* __restrict__ tile_cnt, int n_tiles,
                                                   int B, int* __restrict__ rank,
                                                   int* __restrict__ active,
                                                   int* __restrict__ counts) {
  __shared__ int red[4];
  __shared__ int wpre[4];
  const int b = blockIdx.x, tid = threadIdx.x, w = tid >> 6, l = lane();
  int part = 0;
  for (int i = tid; i < b; i += 256) part += tile_cnt[i];
  const int off = block_sum256(part, red);
  const uint4 v = reinterpret_cast<const uint4*>(flags + static_cast<size_t>(b) * kTile)[tid];
  const int c = flag_count(v);
  const int inc = wave_prefix_sum(c);
  if (l == 63) wpre[w] = inc;
  __syncthreads();
  int wbase = 0;
  for (int q = 0; q < w; ++q) wbase += wpre[q];
  int run = off + wbase + inc - c;
  const uint32_t words[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    if ((words[q >> 2] >> (8 * (q & 3))) & 0xff) {
      const int e = b * kTile + tid * 16 + q;
      rank[e] = run;
      active[run] = e;
      ++run;
    }
  }
  if (b == n_tiles - 1 && tid == 255) {
    counts[0] = run;
    counts[1] = (run + B - 1) / B;
  }
  (void)N;
}

__global__ __launch_bounds__(256) void group_key_kernel(const int32_t* __restrict__ idx,
                                                        const int* __restrict__ rank, int M, int N,
                                                        int B, int* __restrict__ key) {
  const int m = blockIdx.x * 256 + threadIdx.x;
  if (m >= M) return;
  const int e = idx[m];
  key[m] = static_cast<unsigned>(e) < static_cast<unsigned>(N) ? rank[e] / B : 0;
}

__global__ __launch_bounds__(256) void radix_up_kernel(const int* __restrict__ key, int M,
                                                       int shift, int n_tt,
                                                       int* __restrict__ hist) {
  __shared__ uint32_t h[256];
  h[threadIdx.x] = 0;
  __syncthreads();
  const int base = blockIdx.x * kTile;
#pragma unroll 4
  for (int r = 0; r < 16; ++r) {
    const int i = base + r * 256 + threadIdx.x;
    if (i < M) atomicAdd(&h[(static_cast<uint32_t>(key[i]) >> shift) & 255], 1u);
  }
  __syncthreads();
  hist[threadIdx.x * n_tt + blockIdx.x] = static_cast<int>(h[threadIdx.x]);
}

// Exclusive scan of n ints in place, one workgroup of 1024 threads.
__global__ __launch_bounds__(1024) void scan_kernel(int* __restrict__ a, int n) {
  __shared__ int wpre[16];
  __shared__ int total_s;
  const int tid = threadIdx.x, w = tid >> 6, l = lane();
  int carry = 0;
  for (int base = 0; base < n; base += 4096) {
    int v[4];
    int s = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = base + tid * 4 + q;
      v[q] = i < n ? a[i] : 0;
      s += v[q];
    }
    const int inc = wave_prefix_sum(s);
    if (l == 63) wpre[w] = inc;
    __syncthreads();
    if (tid == 0) {
      int acc = 0;
      for (int q = 0; q < 16; ++q) { const int t = wpre[q]; wpre[q] = acc; acc += t; }
      total_s = acc;
    }
    __syncthreads();
    int run = carry + wpre[w] + inc - s;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = base + tid * 4 + q;
      if (i < n) a[i] = run;
      run += v[q];
    }
    carry += total_s;
    __syncthreads();
  }
}

// Stable scatter of one radix pass.  Wave w of a tile ranks its 1024
// consecutive elements 64 at a time: lanes with the same digit find each
// other with 8 ballots, the lowest of them bumps the wave's running count.
__global__ __launch_bounds__(256) void radix_down_kernel(
    const int* __restrict__ kin, const int* __restrict__ vin, int M, int shift, int n_tt,
    const int* __restrict__ hscan, int* __restrict__ kout, int* __restrict__ vout, int K,
    const int32_t* __restrict__ expert_idx, const float* __restrict__ gate,
    int32_t* __restrict__ task_token, int32_t* __restrict__ task_expert,
    float* __restrict__ task_gate, int32_t* __restrict__ task_index) {
  __shared__ uint32_t wh[4][256];
  __shared__ uint32_t goff[256];
  const int tid = threadIdx.x, w = tid >> 6, l = lane();
  wh[0][tid] = 0; wh[1][tid] = 0; wh[2][tid] = 0; wh[3][tid] = 0;
  goff[tid] = static_cast<uint32_t>(hscan[tid * n_tt + blockIdx.x]);
  __syncthreads();
  const int base = blockIdx.x * kTile + w * 1024;
  const uint64_t lt = (l == 0) ? 0ull : (~0ull >> (64 - l));
  uint32_t dg[16], lr[16];
  int kv[16], vv[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int i = base + r * 64 + l;
    const bool valid = i < M;
    const int k = valid ? kin[i] : 0;
    const int v = valid ? (vin ? vin[i] : i) : 0;
    const uint32_t d = (static_cast<uint32_t>(k) >> shift) & 255;
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
      const bool on = (d >> bit) & 1;
      const uint64_t bm = __ballot(valid && on);
      peers &= on ? bm : ~bm;
    }
    const uint64_t below = peers & lt;
    const uint32_t before = wh[w][d];
    wave_lds_fence();
    if (valid && below == 0) wh[w][d] = before + static_cast<uint32_t>(__popcll(peers));
    wave_lds_fence();
    dg[r] = d;
    lr[r] = before + static_cast<uint32_t>(__popcll(below));
    kv[r] = k;
    vv[r] = v;
  }
  __syncthreads();
  {
    const uint32_t c0 = wh[0][tid], c1 = wh[1][tid], c2 = wh[2][tid];
    wh[0][tid] = 0;
    wh[1][tid] = c0;
    wh[2][tid] = c0 + c1;
    wh[3][tid] = c0 + c1 + c2;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int i = base + r * 64 + l;
    if (i >= M) continue;
    const uint32_t pos = goff[dg[r]] + wh[w][dg[r]] + lr[r];
    if (pos >= static_cast<uint32_t>(M)) continue;  // unreachable when counts agree
    kout[pos] = kv[r];
    vout[pos] = vv[r];
    if (task_token) {
      const int m = vv[r];
      task_token[pos] = m / K;
      task_expert[pos] = expert_idx[m];
      task_gate[pos] = gate[m];
      if (task_index) task_index[pos] = m;
    }
  }
}

// CSR offsets: off[g] = first sorted position of group g (groups are never
// empty); entries from n_groups to G hold M.
__global__ __launch_bounds__(256) void offsets_kernel(const int* __restrict__ skey, int M, int G,
                                                      const int* __restrict__ counts,
                                                      int* __restrict__ off) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < M) {
    const int g = min(skey[i], G - 1);
    const int gp = i ? min(skey[i - 1], G - 1) : -1;
    for (int j = gp + 1; j <= g; ++j) off[j] = i;
  }
  if (i <= G && i >= counts[1]) off[i] = M;
}

__global__ void empty_schedule_kernel(int* counts, int* off) {
  counts[0] = 0;
  counts[1] = 0;
  off[0] = 0;
}

static inline unsigned blocks_for(long long n, int per) {
  return static_cast<unsigned>((n + per - 1) / per);
}

hipError_t launch_schedule(int L, int K, int N, int B, const int32_t* expert_idx,
                           const float* gate, int32_t* counts, int32_t* active,
                           int32_t* group_offsets, int32_t* task_token, int32_t* task_expert,
                           float* task_gate, int32_t* task_index, void* ws, hipStream_t s) {
  const int M = L * K;
  const ScheduleWs lay = schedule_ws_layout(L, K, N, B);
  if (M == 0) {
    empty_schedule_kernel<<<1, 1, 0, s>>>(counts, group_offsets);
    return hipGetLastError();
  }
  char* base = static_cast<char*>(ws);
  uint8_t* flags = reinterpret_cast<uint8_t*>(base + lay.flags);
  int* tile_cnt = reinterpret_cast<int*>(base + lay.tile_cnt);
  int* rank = reinterpret_cast<int*>(base + lay.rank);
  int* key0 = reinterpret_cast<int*>(base + lay.key0);
  int* val0 = reinterpret_cast<int*>(base + lay.val0);
  int* key1 = reinterpret_cast<int*>(base + lay.key1);
  int* val1 = reinterpret_cast<int*>(base + lay.val1);
  int* hist = reinterpret_cast<int*>(base + lay.hist);

  const size_t n16 = static_cast<size_t>(lay.n_ftiles) * kTile / 16;
  zero16_kernel<<<blocks_for(static_cast<long long>(n16), 256), 256, 0, s>>>(
      reinterpret_cast<uint4*>(flags), n16);
  mark_kernel<<<blocks_for(M, 256), 256, 0, s>>>(expert_idx, M, N, flags);
  tile_count_kernel<<<lay.n_ftiles, 256, 0, s>>>(flags, tile_cnt);
  rank_kernel<<<lay.n_ftiles, 256, 0, s>>>(flags, N, tile_cnt, lay.n_ftiles, B, rank, active,
                                           counts);
  group_key_kernel<<<blocks_for(M, 256), 256, 0, s>>>(expert_idx, rank, M, N, B, key0);

  int* kin = key0;
  int* vin = nullptr;  // identity payload on the first pass
  int* kbuf[2] = {key1, key0};
  int* vbuf[2] = {val1, val0};
  for (int p = 0; p < lay.passes; ++p) {
    const int shift = 8 * p;
    const bool last = p == lay.passes - 1;
    int* ko = kbuf[p & 1];
    int* vo = vbuf[p & 1];
    radix_up_kernel<<<lay.n_ttiles, 256, 0, s>>>(kin, M, shift, lay.n_ttiles, hist);
    scan_kernel<<<1, 1024, 0, s>>>(hist, 256 * lay.n_ttiles);
    radix_down_kernel<<<lay.n_ttiles, 256, 0, s>>>(
        kin, vin, M, shift, lay.n_ttiles, hist, ko, vo, K, expert_idx, gate,
        last ? task_token : nullptr, task_expert, task_gate, task_index);
    kin = ko;
    vin = vo;
  }
  const long long nthr = M > lay.max_groups + 1 ? M : lay.max_groups + 1;
  offsets_kernel<<<blocks_for(nthr, 256), 256, 0, s>>>(kin, M, lay.max_groups, counts,
                                                       group_offsets);
  return hipGetLastError();
}

}  // namespace omni
