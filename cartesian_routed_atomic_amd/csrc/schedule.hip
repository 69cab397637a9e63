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
//   3. stable LSD radix sort of the tasks by group g = rank[e] / B (or, in
//      the fixed-window variant, g = e / B: the id window), 8 bits
//      per pass.  Tasks enter in flatten order m = t*K + k, which is already
//      token-major, so a stable sort by group alone yields (group, token)
//      order with ties in flatten order.  Each pass: per-tile digit
//      histograms (the first pass computes the group keys on the way), a
//      parallel scan of each digit's row of tile counts, then a stable
//      scatter ranked with 8 ballots per element.  Passes beyond the digits
//      that n_groups actually needs return at once;
//   4. CSR group offsets from the group boundaries of the sorted keys.
#include "device.hpp"
#include "launch.hpp"

namespace omni {

constexpr int kTile = 4096;   // experts per flag tile (256 threads x 16)
constexpr int kInlineCountTiles = 8;  // up to 32,768 experts: no separate tile-count launch
constexpr int kSTile = 2048;  // tasks per sort tile (512 threads x 4)
// Up to this many sort tiles (65,536 tasks) the down-sweep reads its digit
// rows of tile counts itself, one round of loads; measured: decode (8 tiles)
// 31 -> 27 us per schedule, tiny 30 -> 25 us; at 64 tiles (two rounds) it
// lost 3 us to the separate scan.
constexpr int kFuseTiles = 32;

static inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

ScheduleWs schedule_ws_layout(int L, int K, int N, int B, int window) {
  ScheduleWs w{};
  const long long M = static_cast<long long>(L) * K;
  w.n_ftiles = static_cast<int>((static_cast<long long>(N) + kTile - 1) / kTile);
  w.n_ttiles = static_cast<int>((M + kSTile - 1) / kSTile);
  const long long mn = window ? N : (M < N ? M : N);  // every id window is a group
  w.max_groups = static_cast<int>((mn + B - 1) / B);
  int bits = 0;
  while (bits < 31 && (1ll << bits) < w.max_groups) ++bits;  // groups are < max_groups
  w.passes = bits <= 8 ? 1 : (bits + 7) / 8;
  const size_t nt = static_cast<size_t>(w.n_ttiles > 0 ? w.n_ttiles : 1);
  size_t o = 0;
  w.flags = o;    o = align256(o + static_cast<size_t>(w.n_ftiles) * kTile);
  w.tile_cnt = o; o = align256(o + static_cast<size_t>(w.n_ftiles) * 4);
  w.rank = o;     o = align256(o + static_cast<size_t>(N) * 4);
  w.key0 = o;     o = align256(o + static_cast<size_t>(M) * 4);
  w.val0 = o;     o = align256(o + static_cast<size_t>(M) * 4);
  w.key1 = o;     o = align256(o + static_cast<size_t>(M) * 4);
  w.val1 = o;     o = align256(o + static_cast<size_t>(M) * 4);
  w.hist = o;     o = align256(o + 256 * nt * 4);
  w.dtot = o;     o = align256(o + 256 * 4);
  w.bytes = o;
  return w;
}

// Passes that n_groups actually needs: max group id n_groups - 1 < 256^eff.
__device__ __forceinline__ int effective_passes(int n_groups) {
  int eff = 1;
  long long lim = 256;
  while (static_cast<long long>(n_groups) > lim && eff < 4) {
    ++eff;
    lim <<= 8;
  }
  return eff;
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
  const uint4 v =
      reinterpret_cast<const uint4*>(flags + static_cast<size_t>(blockIdx.x) * kTile)[threadIdx.x];
  const int s = block_sum256(flag_count(v), red);
  if (threadIdx.x == 0) tile_cnt[blockIdx.x] = s;
}

// tile_cnt == NULL (few tiles): each block counts the flags of the tiles
// before it itself, in place of tile_count_kernel's per-tile counts.
__global__ __launch_bounds__(256) void rank_kernel(const uint8_t* __restrict__ flags, int N,
                                                   const int* __restrict__ tile_cnt, int n_tiles,
                                                   int B, int window, int* __restrict__ rank,
                                                   int* __restrict__ active,
                                                   int* __restrict__ counts) {
  __shared__ int red[4];
  __shared__ int wpre[4];
  const int b = blockIdx.x, tid = threadIdx.x, w = tid >> 6, l = lane();
  int part = 0;
  if (tile_cnt) {
    for (int i = tid; i < b; i += 256) part += tile_cnt[i];
  } else {
    for (int i = 0; i < b; ++i)
      part += flag_count(
          reinterpret_cast<const uint4*>(flags + static_cast<size_t>(i) * kTile)[tid]);
  }
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
    counts[1] = window ? static_cast<int>((static_cast<long long>(N) + B - 1) / B)
                       : (run + B - 1) / B;
  }
}

// Per-tile digit histogram, digit-major: hist[d * n_tt + tile].  The first
// pass computes the group key of each task (kout) on the way.
__global__ __launch_bounds__(512) void radix_up_kernel(
    const int* __restrict__ kin, const int32_t* __restrict__ idx, const int* __restrict__ rank,
    int* __restrict__ kout, int M, int N, int B, int window, int pass, int n_tt,
    const int* __restrict__ counts, int* __restrict__ hist) {
  if (pass >= effective_passes(counts[1])) return;
  __shared__ uint32_t h[256];
  if (threadIdx.x < 256) h[threadIdx.x] = 0;
  __syncthreads();
  const int shift = 8 * pass;
  const int base = blockIdx.x * kSTile;
#pragma unroll
  for (int r = 0; r < kSTile / 512; ++r) {
    const int i = base + r * 512 + threadIdx.x;
    if (i >= M) continue;
    int key;
    if (pass == 0) {
      const int e = idx[i];
      key = static_cast<unsigned>(e) < static_cast<unsigned>(N) ? (window ? e : rank[e]) / B : 0;
      kout[i] = key;
    } else {
      key = kin[i];
    }
    atomicAdd(&h[(static_cast<uint32_t>(key) >> shift) & 255], 1u);
  }
  __syncthreads();
  if (threadIdx.x < 256) hist[threadIdx.x * n_tt + blockIdx.x] = static_cast<int>(h[threadIdx.x]);
}

// Exclusive scan of each digit's row of tile counts; the row total goes to
// dtot[d].  One wave per digit.
__global__ __launch_bounds__(64) void radix_rowscan_kernel(int* __restrict__ hist, int n_tt,
                                                           int pass,
                                                           const int* __restrict__ counts,
                                                           int* __restrict__ dtot) {
  if (pass >= effective_passes(counts[1])) return;
  int* row = hist + static_cast<size_t>(blockIdx.x) * n_tt;
  const int l = lane();
  uint32_t carry = 0;
  for (int b0 = 0; b0 < n_tt; b0 += 64) {
    const int b = b0 + l;
    const uint32_t v = b < n_tt ? static_cast<uint32_t>(row[b]) : 0u;
    const uint32_t inc = wave_inclusive_scan(v);
    if (b < n_tt) row[b] = static_cast<int>(carry + inc - v);
    carry += static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(inc), 63));
  }
  if (l == 0) dtot[blockIdx.x] = static_cast<int>(carry);
}

// Stable scatter of one pass.  Wave w of a tile ranks its 256 consecutive
// elements 64 at a time: lanes with the same digit find each other with 8
// ballots, the lowest of them bumps the wave's running count.  The last
// effective pass also writes the task arrays.
// fused != 0 (few tiles): hist holds the raw tile counts and each block sums
// its digit rows itself (no radix_rowscan_kernel launch); a single-pass sort
// then also writes the group offsets (G + 1 entries, spread over the blocks:
// off[g] = tasks in groups below g), so no offsets_kernel launch either.
__global__ __launch_bounds__(512) void radix_down_kernel(
    const int* __restrict__ kin, const int* __restrict__ vin, int M, int pass, int n_tt,
    const int* __restrict__ hist, const int* __restrict__ dtot, const int* __restrict__ counts,
    int* __restrict__ kout, int* __restrict__ vout, int K,
    const int32_t* __restrict__ expert_idx, const float* __restrict__ gate,
    int32_t* __restrict__ task_token, int32_t* __restrict__ task_expert,
    float* __restrict__ task_gate, int32_t* __restrict__ task_index, int fused, int G,
    int32_t* __restrict__ group_offsets) {
  const int eff = effective_passes(counts[1]);
  if (pass >= eff) return;
  const bool last = pass == eff - 1;
  constexpr int kW = 8, kR = kSTile / (kW * 64);
  __shared__ uint32_t wh[kW][256];
  __shared__ uint32_t goff[256];
  __shared__ uint32_t tpre[256];
  __shared__ uint32_t red[4];
  const int tid = threadIdx.x, w = tid >> 6, l = lane();
  for (int q = 0; q < kW; ++q)
    if (tid < 256) wh[q][tid] = 0;
  // digit base: exclusive scan of the digit totals (first 4 waves, 64 each)
  if (tid < 256) {
    uint32_t v, before;
    if (fused) {  // this digit's tiles before this block, and all of them
      const int* row = hist + static_cast<size_t>(tid) * n_tt;
      uint32_t all = 0;
      before = 0;
      for (int b0 = 0; b0 < n_tt; b0 += 32) {  // 32 loads in flight per round
        uint32_t c[32];
#pragma unroll
        for (int j = 0; j < 32; ++j)
          c[j] = b0 + j < n_tt ? static_cast<uint32_t>(row[b0 + j]) : 0u;
#pragma unroll
        for (int j = 0; j < 32; ++j) {
          before += b0 + j < static_cast<int>(blockIdx.x) ? c[j] : 0u;
          all += c[j];
        }
      }
      v = all;
    } else {
      v = static_cast<uint32_t>(dtot[tid]);
      before = static_cast<uint32_t>(hist[tid * n_tt + blockIdx.x]);
    }
    tpre[tid] = before;
    const uint32_t inc = wave_inclusive_scan(v);
    if (l == 63) red[w] = inc;
    goff[tid] = inc - v;
  }
  __syncthreads();
  if (tid < 256) {
    uint32_t add = 0;
    for (int q = 0; q < w; ++q) add += red[q];
    goff[tid] += add;
  }
  __syncthreads();
  if (fused && eff == 1) {  // single pass: the digit is the group
    for (long long g = static_cast<long long>(blockIdx.x) * 512 + tid; g <= G;
         g += static_cast<long long>(gridDim.x) * 512)
      group_offsets[g] = g < 256 ? static_cast<int>(goff[g]) : M;
  }
  if (tid < 256) goff[tid] += tpre[tid];
  __syncthreads();
  const int shift = 8 * pass;
  const int base = blockIdx.x * kSTile + w * (kR * 64);
  const uint64_t lt = (l == 0) ? 0ull : (~0ull >> (64 - l));
  uint32_t dg[kR], lr[kR];
  int kv[kR], vv[kR];
#pragma unroll
  for (int r = 0; r < kR; ++r) {
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
  if (tid < 256) {  // exclusive prefix of the per-wave counts of each digit
    uint32_t run = 0;
#pragma unroll
    for (int q = 0; q < kW; ++q) {
      const uint32_t c = wh[q][tid];
      wh[q][tid] = run;
      run += c;
    }
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kR; ++r) {
    const int i = base + r * 64 + l;
    if (i >= M) continue;
    const uint32_t pos = goff[dg[r]] + wh[w][dg[r]] + lr[r];
    if (pos >= static_cast<uint32_t>(M)) continue;  // unreachable when counts agree
    kout[pos] = kv[r];
    vout[pos] = vv[r];
    if (last) {
      const int m = vv[r];
      task_token[pos] = m / K;
      task_expert[pos] = expert_idx[m];
      task_gate[pos] = gate[m];
      if (task_index) task_index[pos] = m;
    }
  }
}

// CSR offsets: off[g] = first sorted position of group g.  An empty group
// (only id windows can be empty) gets the position of the next non-empty
// one; entries past the last task's group, up to G, hold M.  The sorted keys
// are those of the last effective pass.
__global__ __launch_bounds__(256) void offsets_kernel(const int* __restrict__ skey_even,
                                                      const int* __restrict__ skey_odd, int M,
                                                      int G, const int* __restrict__ counts,
                                                      int* __restrict__ off) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  const int eff = effective_passes(counts[1]);
  const int* skey = ((eff - 1) & 1) ? skey_odd : skey_even;
  if (i < M) {
    const int g = min(skey[i], G - 1);
    const int gp = i ? min(skey[i - 1], G - 1) : -1;
    for (int j = gp + 1; j <= g; ++j) off[j] = i;
  }
  if (i <= G && i > min(skey[M - 1], G - 1)) off[i] = M;
}

// No tasks: no active expert; every group (only id windows exist without
// tasks) is empty.
__global__ __launch_bounds__(256) void empty_schedule_kernel(int* counts, int* off, int n_groups,
                                                             int G) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i == 0) {
    counts[0] = 0;
    counts[1] = n_groups;
  }
  if (i <= G) off[i] = 0;
}

static inline unsigned blocks_for(long long n, int per) {
  return static_cast<unsigned>((n + per - 1) / per);
}

hipError_t launch_schedule(int L, int K, int N, int B, int window, const int32_t* expert_idx,
                           const float* gate, int32_t* counts, int32_t* active,
                           int32_t* group_offsets, int32_t* task_token, int32_t* task_expert,
                           float* task_gate, int32_t* task_index, void* ws, hipStream_t s) {
  const int M = L * K;
  const ScheduleWs lay = schedule_ws_layout(L, K, N, B, window);
  if (M == 0) {
    const int ng = window ? lay.max_groups : 0;
    empty_schedule_kernel<<<blocks_for(static_cast<long long>(lay.max_groups) + 1, 256), 256, 0,
                            s>>>(counts, group_offsets, ng, lay.max_groups);
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
  int* dtot = reinterpret_cast<int*>(base + lay.dtot);

  const size_t n16 = static_cast<size_t>(lay.n_ftiles) * kTile / 16;
  zero16_kernel<<<blocks_for(static_cast<long long>(n16), 256), 256, 0, s>>>(
      reinterpret_cast<uint4*>(flags), n16);
  mark_kernel<<<blocks_for(M, 256), 256, 0, s>>>(expert_idx, M, N, flags);
  // few expert tiles: rank_kernel counts the flags before its tile itself
  const bool count_inline = lay.n_ftiles <= kInlineCountTiles;
  if (!count_inline) tile_count_kernel<<<lay.n_ftiles, 256, 0, s>>>(flags, tile_cnt);
  rank_kernel<<<lay.n_ftiles, 256, 0, s>>>(flags, N, count_inline ? nullptr : tile_cnt,
                                           lay.n_ftiles, B, window, rank, active, counts);
  // pass p reads (key, val) from buffer p & 1 and writes buffer (p + 1) & 1;
  // pass 0 reads the group keys it computes itself (key0) and identity values
  int* kb[2] = {key0, key1};
  int* vb[2] = {val0, val1};
  // few sort tiles: the down-sweep scans the tile counts itself
  const int fused = lay.n_ttiles <= kFuseTiles ? 1 : 0;
  for (int p = 0; p < lay.passes; ++p) {
    int* kin = kb[p & 1];
    const int* vin = p == 0 ? nullptr : vb[p & 1];
    radix_up_kernel<<<lay.n_ttiles, 512, 0, s>>>(kin, expert_idx, rank, key0, M, N, B, window,
                                                 p, lay.n_ttiles, counts, hist);
    if (!fused) radix_rowscan_kernel<<<256, 64, 0, s>>>(hist, lay.n_ttiles, p, counts, dtot);
    radix_down_kernel<<<lay.n_ttiles, 512, 0, s>>>(
        kin, vin, M, p, lay.n_ttiles, hist, dtot, counts, kb[(p + 1) & 1], vb[(p + 1) & 1], K,
        expert_idx, gate, task_token, task_expert, task_gate, task_index, fused,
        lay.max_groups, group_offsets);
  }
  // A fused single-pass sort has written the offsets; with more possible
  // passes the offsets come from the sorted keys (the last effective pass p
  // leaves them in kb[(p + 1) & 1]).
  if (!fused || lay.passes > 1) {
    const long long nthr = M > lay.max_groups + 1 ? M : lay.max_groups + 1;
    offsets_kernel<<<blocks_for(nthr, 256), 256, 0, s>>>(key1, key0, M, lay.max_groups, counts,
                                                         group_offsets);
  }
  return hipGetLastError();
}

}  // namespace omni
