// Cartesian Product Router, part 1: row / column logits.  Pages: gist.science
// explainer §2.2 "Cartesian Product Router" (two small projections give row
// and column logits over the Nr x Nc grid).
//
// The projection is one dense contraction z = x . [Wr | Wc] of shape
// L x d x (Nr + Nc), so the bf16 path runs it on the gfx950 matrix cores
// (v_mfma_f32_16x16x32_bf16, fp32 accumulation).  The per-axis log-softmax
// is fused into the selection kernel, which reads each row once anyway.
//
// The same MFMA kernels serve the other dense products of the layer: the
// backward's router products (launch_gemm_nt) and the shared dense MLP
// (launch_swiglu_up with a fused SwiGLU epilogue, then launch_gemm_nt).
#include "device.hpp"
#include "launch.hpp"

namespace omni {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Block tile 128 tokens x 128 grid lines x 64 features; 4 waves in 2 x 2,
// each wave owns a 64 x 64 sub-tile = 4 x 4 MFMA 16x16 tiles.  LDS rows are
// padded by 8 bf16 (16 bytes) to spread the 16-byte fragment reads over banks.
constexpr int RBM = 128, RBN = 128, RBK = 64, RLD = RBK + 8;

// Epilogues: grid-line logits (+ bias, or accumulated into the output), or
// the SwiGLU hidden activation of the shared dense MLP.  In SwiGLU mode the
// B operand is [Wg; Wu] seen through an interleave: logical columns come in
// blocks of 16, even blocks are gate rows and odd blocks the up rows of the
// same 16 hidden units, so one lane holds both halves of a hidden unit in
// its tiles j and j + 1.
constexpr int kEpiLogits = 0, kEpiSwiglu = 1;
// Split-K partial: the raw accumulators of K range blockIdx.y, no bias, into
// zr + blockIdx.y * L * (Nr + Nc) (summed in order by splitk_reduce_kernel).
constexpr int kEpiPartial = 2;

__device__ __forceinline__ int swiglu_hidden(int n) { return ((n >> 5) << 4) | (n & 15); }

// silu(g) * u rounded to bf16 (nearest even; finite values)
__device__ __forceinline__ uint16_t swiglu_bf16(float g, float u) {
  const float v = g / (1.f + __expf(-g)) * u;
  const uint32_t b = __float_as_uint(v);
  return static_cast<uint16_t>((b + 0x7fffu + ((b >> 16) & 1u)) >> 16);
}

template <int EPI>
__global__ __launch_bounds__(256) void router_gemm_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
    const uint16_t* __restrict__ wc, const float* __restrict__ rb,
    const float* __restrict__ cb, float* __restrict__ zr, float* __restrict__ zc,
    int L, int d, int Nr, int Nc, int n_mt, int n_nt, int acc_out, uint16_t* __restrict__ hout,
    int ksplit) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[RBM * RLD];
  __shared__ __attribute__((aligned(16))) uint16_t sB[RBN * RLD];

  const int tid = threadIdx.x, wv = tid >> 6, l = tid & 63;
  // Workgroup b runs on XCD b % 8.  Give every XCD a contiguous run of
  // logical tiles so one token tile is reused from that XCD's L2 across all
  // of its grid-line tiles.
  const int nblk = n_mt * n_nt;
  const int per = nblk >> 3, rem = nblk & 7;
  const int xcd = blockIdx.x & 7, loc = blockIdx.x >> 3;
  const int logical = xcd * per + min(xcd, rem) + loc;
  const int mt = logical / n_nt, nt = logical - mt * n_nt;
  const int m0 = mt * RBM, n0 = nt * RBN;
  const int NT = Nr + Nc;
  // K range of this workgroup: all of K, or split-K chunk blockIdx.y
  const int kb = blockIdx.y * ksplit, ke = min(d, kb + ksplit);

  // global -> register staging: 4 x 16 B of A and of B per thread
  const uint16_t* arow[4];
  const uint16_t* brow[4];
  int ach[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 256 * i, row = c >> 3;
    ach[i] = (c & 7) * 8;
    const int t = m0 + row;
    arow[i] = (t < L) ? x + static_cast<size_t>(t) * d : nullptr;
    const int n = n0 + row;
    if constexpr (EPI == kEpiSwiglu) {
      const int h = swiglu_hidden(n);
      brow[i] = h < Nr ? ((n >> 4) & 1 ? wc : wr) + static_cast<size_t>(h) * d : nullptr;
    } else {
      brow[i] = (n < Nr) ? wr + static_cast<size_t>(n) * d
                         : ((n < NT) ? wc + static_cast<size_t>(n - Nr) * d : nullptr);
    }
  }
  uint4 ra[4], rbv[4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k = k0 + ach[i];
      ra[i] = (arow[i] && k < ke) ? *reinterpret_cast<const uint4*>(arow[i] + k) : make_uint4(0, 0, 0, 0);
      rbv[i] = (brow[i] && k < ke) ? *reinterpret_cast<const uint4*>(brow[i] + k) : make_uint4(0, 0, 0, 0);
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int wm = wv >> 1, wn = wv & 1;
  const int fr = l & 15, fk = (l >> 4) * 8;

  gload(kb);
  for (int k0 = kb; k0 < ke; k0 += RBK) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i, row = c >> 3;
      *reinterpret_cast<uint4*>(&sA[row * RLD + ach[i]]) = ra[i];
      *reinterpret_cast<uint4*>(&sB[row * RLD + ach[i]]) = rbv[i];
    }
    __syncthreads();
    if (k0 + RBK < ke) gload(k0 + RBK);
#pragma unroll
    for (int kk = 0; kk < RBK; kk += 32) {
      bf16x8 af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(&sA[(wm * 64 + i * 16 + fr) * RLD + kk + fk]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8*>(&sB[(wn * 64 + j * 16 + fr) * RLD + kk + fk]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }

  // Accumulator lane layout (16x16 output tile): column = lane % 16,
  // rows 4 * (lane / 16) + q, q = 0..3.
  if constexpr (EPI == kEpiSwiglu) {
    // tiles j = 0, 2 hold gate columns and j = 1, 3 the up columns of the
    // same hidden units (the B rows were interleaved in blocks of 16)
#pragma unroll
    for (int jp = 0; jp < 2; ++jp) {
      const int h = (n0 + wn * 64) / 2 + jp * 16 + fr;
      if (h >= Nr) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int t = m0 + wm * 64 + i * 16 + (l >> 4) * 4 + q;
          if (t < L)
            hout[static_cast<size_t>(t) * Nr + h] =
                swiglu_bf16(acc[i][2 * jp][q], acc[i][2 * jp + 1][q]);
        }
    }
    return;
  }
  if constexpr (EPI == kEpiPartial) {
    float* part = zr + static_cast<size_t>(blockIdx.y) * L * NT;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + wn * 64 + j * 16 + fr;
      if (n >= NT) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int t = m0 + wm * 64 + i * 16 + (l >> 4) * 4 + q;
          if (t < L) part[static_cast<size_t>(t) * NT + n] = acc[i][j][q];
        }
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = n0 + wn * 64 + j * 16 + fr;
    if (n >= NT) continue;
    const bool is_row = n < Nr;
    const float bias = is_row ? (rb ? rb[n] : 0.f) : (cb ? cb[n - Nr] : 0.f);
    float* col = is_row ? zr + n : zc + (n - Nr);
    const size_t ld = is_row ? Nr : Nc;
    // accumulate: read this column's old values first, all loads in flight
    float old[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int t = m0 + wm * 64 + i * 16 + (l >> 4) * 4 + q;
        old[i][q] = (acc_out && t < L) ? col[static_cast<size_t>(t) * ld] : 0.f;
      }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int t = m0 + wm * 64 + i * 16 + (l >> 4) * 4 + q;
        if (t >= L) continue;
        col[static_cast<size_t>(t) * ld] = acc[i][j][q] + bias + old[i][q];
      }
    }
  }
}

// Large-shape path (d % 32 == 0): block tile 256 tokens x 256 grid lines,
// K step 32, 8 waves in 2 x 4, each wave a 128 x 64 sub-tile = 8 x 4 MFMA
// 16x16x32 tiles (128 float32 accumulators per lane).  Operands go straight
// from global memory into a 4-stage LDS ring with global_load_lds_dwordx4
// (three K steps in flight, no register staging).  An LDS row holds 32 bf16
// (64 B = four 16-B chunks); chunk c of row r is stored at position
// c ^ ((r >> 1) & 3).  A 16-byte-per-lane LDS read is served eight lanes at a
// time from one 128-byte bank window; the eight rows such a group of a
// fragment read touches (r .. r+7, same chunk) then land on eight distinct
// 16-byte bank groups (measured on gfx950: the (r >> 2) swizzle costs four
// conflict cycles per read, this one none).
constexpr int GBM = 256, GBN = 256, GBK = 32, GSTAGES = 4;
constexpr int GSTAGE_BYTES = (GBM + GBN) * GBK * 2;  // 32 KiB

__device__ __forceinline__ int swz_chunk(int row, int chunk) { return chunk ^ ((row >> 1) & 3); }
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * 64 + (swz_chunk(row, chunk) << 4);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// vmcnt <= N and every LDS access of this wave complete (lgkmcnt = 0)
template <int N>
__device__ __forceinline__ void wait_vmcnt_lds() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

// Issue the direct global->LDS loads of K step kt into its ring stage: each
// wave fills 2 KiB of A and 2 KiB of B with two 1-KiB instructions each.
__device__ __forceinline__ void gemm_issue(uint8_t* smem, const uint16_t* const (&asrc)[2],
                                           const uint16_t* const (&bsrc)[2], int wv, int kt) {
  uint8_t* st = smem + (kt % GSTAGES) * GSTAGE_BYTES;
  const int k0 = kt * GBK;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    __builtin_amdgcn_global_load_lds(asrc[u] + k0, st + (wv * 2 + u) * 1024, 16, 0, 0);
    __builtin_amdgcn_global_load_lds(bsrc[u] + k0, st + GBM * 64 + (wv * 2 + u) * 1024, 16, 0, 0);
  }
}

// Read one stage's MFMA fragments: 8 A tiles (16 rows each) and 4 B tiles.
__device__ __forceinline__ void gemm_read_frags(const uint8_t* smem, int kt, int wm, int wn,
                                                int fr, int fc, bf16x8 (&af)[8],
                                                bf16x8 (&bfr)[4]) {
  const uint8_t* st = smem + (kt % GSTAGES) * GSTAGE_BYTES;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    af[i] = *reinterpret_cast<const bf16x8*>(st + swz(wm * 128 + i * 16 + fr, fc));
#pragma unroll
  for (int j = 0; j < 4; ++j)
    bfr[j] = *reinterpret_cast<const bf16x8*>(st + GBM * 64 + swz(wn * 64 + j * 16 + fr, fc));
}

// One pipeline iteration (see the kernel): stage kt's fragments are in
// (ca, cb); stage kt+1's go to (na, nb).
__device__ __forceinline__ void gemm_step(uint8_t* smem, const uint16_t* const (&asrc)[2],
                                          const uint16_t* const (&bsrc)[2], int wv, int wm,
                                          int wn, int fr, int fc, int kt, int nk,
                                          const bf16x8 (&ca)[8], const bf16x8 (&cb)[4],
                                          bf16x8 (&na)[8], bf16x8 (&nb)[4],
                                          f32x4 (&acc)[8][4]) {
  if (kt + 1 < nk) {
    // stages issued so far: 0 .. min(kt + 3, nk - 1); those after kt + 1 may stay in flight
    // (and this wave's reads of stage kt's fragments complete, so the slot
    // can be refilled once every wave has passed the barrier)
    const int after = min(kt + 3, nk - 1) - (kt + 1);
    if (after >= 2) wait_vmcnt_lds<8>();
    else if (after == 1) wait_vmcnt_lds<4>();
    else wait_vmcnt_lds<0>();
    // a bare barrier: a fenced one would also wait for the stages in flight
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
    if (kt + GSTAGES < nk) gemm_issue(smem, asrc, bsrc, wv, kt + GSTAGES);
    gemm_read_frags(smem, kt + 1, wm, wn, fr, fc, na, nb);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ca[i], cb[j], acc[i][j], 0, 0, 0);
}

template <int EPI>
__global__ __launch_bounds__(512) void router_gemm_bf16_big_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
    const uint16_t* __restrict__ wc, const float* __restrict__ rb,
    const float* __restrict__ cb, float* __restrict__ zr, float* __restrict__ zc,
    int L, int d, int Nr, int Nc, int n_mt, int n_nt, int acc_out, uint16_t* __restrict__ hout) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[GSTAGES * GSTAGE_BYTES];
  const int tid = threadIdx.x, wv = tid >> 6, l = tid & 63;
  const int nblk = n_mt * n_nt;
  const int per = nblk >> 3, rem = nblk & 7;
  const int xcd = blockIdx.x & 7, loc = blockIdx.x >> 3;
  const int logical = xcd * per + min(xcd, rem) + loc;
  const int mt = logical / n_nt, nt = logical - mt * n_nt;
  const int m0 = mt * GBM, n0 = nt * GBN;
  const int NT = Nr + Nc;
  const int nk = d / GBK;
  if (nk == 0) return;

  // Direct loads: each wave fills 2 KiB of A (32 rows) and 2 KiB of B per
  // stage with two 1-KiB instructions each; lane i of an instruction lands
  // on row r = base + i / 4, stored chunk i % 4, so it fetches the logical
  // chunk that swz_chunk maps there (the map is its own inverse).  Rows past
  // the end re-read a valid row (their results are never stored).
  const uint16_t* asrc[2];
  const uint16_t* bsrc[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int r = (wv * 2 + u) * 16 + (l >> 2);
    const int c = swz_chunk(r, l & 3);
    const int t = min(m0 + r, L - 1);
    asrc[u] = x + static_cast<size_t>(t) * d + c * 8;
    if constexpr (EPI == kEpiSwiglu) {
      const int n = n0 + r;
      const int h = min(swiglu_hidden(n), Nr - 1);
      bsrc[u] = ((n >> 4) & 1 ? wc : wr) + static_cast<size_t>(h) * d + c * 8;
    } else {
      const int n = min(n0 + r, NT - 1);
      bsrc[u] = (n < Nr ? wr + static_cast<size_t>(n) * d : wc + static_cast<size_t>(n - Nr) * d) +
                c * 8;
    }
  }

  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int wm = wv >> 2, wn = wv & 3;  // 2 x 4 waves
  const int fr = l & 15, fc = l >> 4;
  // Software pipeline.  Iteration kt: wait until stage kt+1 has landed,
  // barrier, refill the slot of stage kt (its fragments are already in
  // registers) with stage kt+4, read stage kt+1's fragments into the other
  // register set, then run stage kt's MFMAs while those reads are in flight.
  // Three stages of global loads stay in flight behind the one being read.
  bf16x8 af[2][8], bfr[2][4];
#pragma unroll
  for (int u = 0; u < GSTAGES; ++u)
    if (u < nk) gemm_issue(smem, asrc, bsrc, wv, u);
  if (nk > 3) wait_vmcnt<12>();
  else if (nk == 3) wait_vmcnt<8>();
  else if (nk == 2) wait_vmcnt<4>();
  else wait_vmcnt<0>();
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
  gemm_read_frags(smem, 0, wm, wn, fr, fc, af[0], bfr[0]);
  for (int kt = 0; kt < nk; kt += 2) {
    gemm_step(smem, asrc, bsrc, wv, wm, wn, fr, fc, kt, nk, af[0], bfr[0], af[1], bfr[1], acc);
    if (kt + 1 < nk)
      gemm_step(smem, asrc, bsrc, wv, wm, wn, fr, fc, kt + 1, nk, af[1], bfr[1], af[0], bfr[0],
                acc);
  }

  // Accumulator lane layout (16x16 output tile): column = lane % 16,
  // rows 4 * (lane / 16) + q, q = 0..3.
  if constexpr (EPI == kEpiSwiglu) {
    // tiles j = 0, 2 hold gate columns and j = 1, 3 the up columns of the
    // same hidden units (the B rows were interleaved in blocks of 16)
#pragma unroll
    for (int jp = 0; jp < 2; ++jp) {
      const int h = (n0 + wn * 64) / 2 + jp * 16 + fr;
      if (h >= Nr) continue;
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int t = m0 + wm * 128 + i * 16 + fc * 4 + q;
          if (t < L)
            hout[static_cast<size_t>(t) * Nr + h] =
                swiglu_bf16(acc[i][2 * jp][q], acc[i][2 * jp + 1][q]);
        }
    }
    return;
  }
  // The logits go through LDS so that every store to HBM is part of a
  // contiguous row: in four rounds, the waves write the accumulators of 64
  // tile rows (row tiles 2r and 2r + 1 of both wave rows) into a 64 x 256
  // float tile, then the workgroup stores the tile row by row, 16 bytes per
  // thread, with the bias (and, with acc_out, the old values) added.
  // Storing straight from the accumulator layout wrote 4-byte pieces of 16
  // rows per instruction (18 us of the 80 us call at L = 8192, N = 2^20).
  constexpr int kCtLd = GBN + 4;  // floats per LDS row (16-byte pad)
  float* ct = reinterpret_cast<float*>(smem);
  const bool vec4 = (Nr & 3) == 0 && (Nc & 3) == 0;
  __syncthreads();  // the ring's last reads are done: smem is free
#pragma unroll
  for (int r = 0; r < 4; ++r) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          ct[(wm * 32 + h * 16 + fc * 4 + q) * kCtLd + wn * 64 + j * 16 + fr] =
              acc[2 * r + h][j][q];
    __syncthreads();
    for (int e = tid; e < 64 * (GBN / 4); e += 512) {
      const int rr = e / (GBN / 4), c = (e % (GBN / 4)) * 4;
      const int t = m0 + (rr >> 5) * 128 + r * 32 + (rr & 31);
      const int n = n0 + c;
      if (t >= L || n >= NT) continue;
      const float4 v = *reinterpret_cast<const float4*>(&ct[rr * kCtLd + c]);
      const float vv[4] = {v.x, v.y, v.z, v.w};
      if (vec4 && (n + 3 < Nr || (n >= Nr && n + 3 < NT))) {
        const bool is_row = n < Nr;
        const float* bias = is_row ? rb : cb;
        const int nb = is_row ? n : n - Nr;
        float* dst = (is_row ? zr + static_cast<size_t>(t) * Nr : zc + static_cast<size_t>(t) * Nc) + nb;
        float4 o = bias ? *reinterpret_cast<const float4*>(bias + nb)
                        : make_float4(0.f, 0.f, 0.f, 0.f);
        if (acc_out) {
          const float4 p = *reinterpret_cast<const float4*>(dst);
          o.x += p.x; o.y += p.y; o.z += p.z; o.w += p.w;
        }
        *reinterpret_cast<float4*>(dst) = make_float4(vv[0] + o.x, vv[1] + o.y, vv[2] + o.z,
                                                      vv[3] + o.w);
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int nu = n + u;
          if (nu >= NT) break;
          const bool is_row = nu < Nr;
          const float bias = is_row ? (rb ? rb[nu] : 0.f) : (cb ? cb[nu - Nr] : 0.f);
          float* dst = is_row ? zr + static_cast<size_t>(t) * Nr + nu
                              : zc + static_cast<size_t>(t) * Nc + (nu - Nr);
          *dst = vv[u] + bias + (acc_out ? *dst : 0.f);
        }
      }
    }
    __syncthreads();  // the tile is read before the next round overwrites it
  }
}

// fp32 path (small shapes): one thread per (token, grid line), features in
// ascending order, float4 loads.
__global__ __launch_bounds__(256) void router_gemm_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ wr, const float* __restrict__ wc,
    const float* __restrict__ rb, const float* __restrict__ cb, float* __restrict__ zr,
    float* __restrict__ zc, int L, int d, int Nr, int Nc, int acc_out) {
  const int NT = Nr + Nc;
  const size_t id = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (id >= static_cast<size_t>(L) * NT) return;
  const int t = static_cast<int>(id / NT), n = static_cast<int>(id - static_cast<size_t>(t) * NT);
  const float4* xr = reinterpret_cast<const float4*>(x + static_cast<size_t>(t) * d);
  const float4* wrow = reinterpret_cast<const float4*>(
      n < Nr ? wr + static_cast<size_t>(n) * d : wc + static_cast<size_t>(n - Nr) * d);
  float s = 0.f;
  for (int c = 0; c < d / 4; ++c) {
    const float4 a = xr[c], b = wrow[c];
    s = fmaf(a.x, b.x, s);
    s = fmaf(a.y, b.y, s);
    s = fmaf(a.z, b.z, s);
    s = fmaf(a.w, b.w, s);
  }
  float* out = n < Nr ? zr + static_cast<size_t>(t) * Nr + n
                      : zc + static_cast<size_t>(t) * Nc + (n - Nr);
  *out = s + (n < Nr ? (rb ? rb[n] : 0.f) : (cb ? cb[n - Nr] : 0.f)) + (acc_out ? *out : 0.f);
}

// Split-K count for the router product (1 = no split): shapes whose 128 x 128
// tiles number well under one per CU (few tokens, or few grid lines) split
// K so that about 256 workgroups run; chunks are multiples of 64 and at
// least 256 long.
static bool router_big(int L, int d, int NT) {
  return d % GBK == 0 && ((L + GBM - 1) / GBM) * ((NT + GBN - 1) / GBN) >= 192;
}

int router_split_count(int L, int d, int NT) {
  if (L <= 0 || router_big(L, d, NT)) return 1;
  const int tiles = ((L + RBM - 1) / RBM) * ((NT + RBN - 1) / RBN);
  if (tiles >= 192) return 1;
  int S = (256 + tiles - 1) / tiles;
  const int max_s = d / 256;
  if (S > max_s) S = max_s;
  if (S <= 1) return 1;
  const int chunk = ((d + S - 1) / S + RBK - 1) / RBK * RBK;
  return (d + chunk - 1) / chunk;
}

size_t router_ws_bytes(int bf16, int L, int d, int Nr, int Nc) {
  if (!bf16) return 0;
  const int S = router_split_count(L, d, Nr + Nc);
  return S > 1 ? static_cast<size_t>(S) * L * (Nr + Nc) * 4 : 0;
}

// z[t, n] = bias[n] + sum over the S partials of (t, n), in partial order
// (added to z as it stands when acc_out).
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part, int S,
                                                            int L, int Nr, int Nc,
                                                            const float* __restrict__ rb,
                                                            const float* __restrict__ cb,
                                                            float* __restrict__ zr,
                                                            float* __restrict__ zc, int acc_out) {
  const int NT = Nr + Nc;
  const size_t total = static_cast<size_t>(L) * NT;
  const size_t id = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (id >= total) return;
  const int t = static_cast<int>(id / NT), n = static_cast<int>(id - static_cast<size_t>(t) * NT);
  float v = 0.f;
  for (int z = 0; z < S; ++z) v += part[static_cast<size_t>(z) * total + id];
  float* out = n < Nr ? zr + static_cast<size_t>(t) * Nr + n
                      : zc + static_cast<size_t>(t) * Nc + (n - Nr);
  *out = v + (n < Nr ? (rb ? rb[n] : 0.f) : (cb ? cb[n - Nr] : 0.f)) + (acc_out ? *out : 0.f);
}

hipError_t launch_router_bf16(const uint16_t* x, const uint16_t* wr, const uint16_t* wc,
                              const float* rb, const float* cb, float* zr, float* zc, int L,
                              int d, int Nr, int Nc, void* ws, hipStream_t s) {
  if (L == 0) return hipSuccess;
  const int NT = Nr + Nc;
  if (router_big(L, d, NT)) {
    const int n_mt = (L + GBM - 1) / GBM, n_nt = (NT + GBN - 1) / GBN;
    router_gemm_bf16_big_kernel<kEpiLogits><<<n_mt * n_nt, 512, 0, s>>>(
        x, wr, wc, rb, cb, zr, zc, L, d, Nr, Nc, n_mt, n_nt, 0, nullptr);
    return hipGetLastError();
  }
  const int n_mt = (L + RBM - 1) / RBM, n_nt = (NT + RBN - 1) / RBN;
  const int S = ws ? router_split_count(L, d, NT) : 1;
  if (S > 1) {
    const int chunk = ((d + S - 1) / S + RBK - 1) / RBK * RBK;
    float* part = static_cast<float*>(ws);
    router_gemm_bf16_kernel<kEpiPartial><<<dim3(n_mt * n_nt, S), 256, 0, s>>>(
        x, wr, wc, nullptr, nullptr, part, part, L, d, Nr, Nc, n_mt, n_nt, 0, nullptr, chunk);
    const size_t n = static_cast<size_t>(L) * NT;
    splitk_reduce_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, s>>>(
        part, S, L, Nr, Nc, rb, cb, zr, zc, 0);
    return hipGetLastError();
  }
  router_gemm_bf16_kernel<kEpiLogits><<<n_mt * n_nt, 256, 0, s>>>(
      x, wr, wc, rb, cb, zr, zc, L, d, Nr, Nc, n_mt, n_nt, 0, nullptr, d);
  return hipGetLastError();
}

hipError_t launch_router_f32(const float* x, const float* wr, const float* wc, const float* rb,
                             const float* cb, float* zr, float* zc, int L, int d, int Nr, int Nc,
                             hipStream_t s) {
  if (L == 0) return hipSuccess;
  const size_t n = static_cast<size_t>(L) * (Nr + Nc);
  router_gemm_f32_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, s>>>(
      x, wr, wc, rb, cb, zr, zc, L, d, Nr, Nc, 0);
  return hipGetLastError();
}

// C[m][n] = sum_k A[m][k] B[n][k] (A [M, K], B [N, K], C [M, N] float32, all
// row-major): the 128 x 128 MFMA kernel (bf16, K a multiple of 8) or the
// float32 kernel, used as plain products by the backward pass.
size_t gemm_nt_ws_bytes(int bf16, int M, int N, int K) {
  if (!bf16 || M <= 0 || N <= 0) return 0;
  const int S = router_split_count(M, K, N);
  return S > 1 ? static_cast<size_t>(S) * M * N * 4 : 0;
}

hipError_t launch_gemm_nt(int bf16, const void* a, const void* b, float* c, int M, int N, int K,
                          int accumulate, void* ws, hipStream_t s) {
  if (M == 0 || N == 0) return hipSuccess;
  if (bf16) {
    const uint16_t* pa = static_cast<const uint16_t*>(a);
    const uint16_t* pb = static_cast<const uint16_t*>(b);
    const int n_mt = (M + RBM - 1) / RBM, n_nt = (N + RBN - 1) / RBN;
    const int S = ws ? router_split_count(M, K, N) : 1;
    if (router_big(M, K, N)) {  // the large tile only where it still fills the chip
      router_gemm_bf16_big_kernel<kEpiLogits><<<((M + GBM - 1) / GBM) * ((N + GBN - 1) / GBN),
                                               512, 0, s>>>(
          pa, pb, pb, nullptr, nullptr, c, c, M, K, N, 0, (M + GBM - 1) / GBM,
          (N + GBN - 1) / GBN, accumulate, nullptr);
    } else if (S > 1) {  // few tiles: split K, partials summed in order
      const int chunk = ((K + S - 1) / S + RBK - 1) / RBK * RBK;
      float* part = static_cast<float*>(ws);
      router_gemm_bf16_kernel<kEpiPartial><<<dim3(n_mt * n_nt, S), 256, 0, s>>>(
          pa, pb, pb, nullptr, nullptr, part, part, M, K, N, 0, n_mt, n_nt, 0, nullptr, chunk);
      const size_t n = static_cast<size_t>(M) * N;
      splitk_reduce_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, s>>>(
          part, S, M, N, 0, nullptr, nullptr, c, c, accumulate);
    } else {
      router_gemm_bf16_kernel<kEpiLogits><<<n_mt * n_nt, 256, 0, s>>>(
          pa, pb, pb, nullptr, nullptr, c, c, M, K, N, 0, n_mt, n_nt, accumulate, nullptr, K);
    }
  } else {
    const size_t n = static_cast<size_t>(M) * N;
    router_gemm_f32_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, s>>>(
        static_cast<const float*>(a), static_cast<const float*>(b), static_cast<const float*>(b),
        nullptr, nullptr, c, c, M, K, N, 0, accumulate);
  }
  return hipGetLastError();
}

// Shared dense MLP, first product: h[t, j] = silu(x_t . Wg[j]) * (x_t . Wu[j]),
// float32 path: one thread per (token, hidden unit), features in ascending
// order, float4 loads.
__global__ __launch_bounds__(256) void swiglu_f32_kernel(const float* __restrict__ x,
                                                         const float* __restrict__ wg,
                                                         const float* __restrict__ wu, int L,
                                                         int d, int d_ff, float* __restrict__ h) {
  const size_t id = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (id >= static_cast<size_t>(L) * d_ff) return;
  const int t = static_cast<int>(id / d_ff), j = static_cast<int>(id - static_cast<size_t>(t) * d_ff);
  const float4* xr = reinterpret_cast<const float4*>(x + static_cast<size_t>(t) * d);
  const float4* gr = reinterpret_cast<const float4*>(wg + static_cast<size_t>(j) * d);
  const float4* ur = reinterpret_cast<const float4*>(wu + static_cast<size_t>(j) * d);
  float g = 0.f, u = 0.f;
  for (int c = 0; c < d / 4; ++c) {
    const float4 a = xr[c], b = gr[c], e = ur[c];
    g = fmaf(a.x, b.x, g); g = fmaf(a.y, b.y, g); g = fmaf(a.z, b.z, g); g = fmaf(a.w, b.w, g);
    u = fmaf(a.x, e.x, u); u = fmaf(a.y, e.y, u); u = fmaf(a.z, e.z, u); u = fmaf(a.w, e.w, u);
  }
  h[id] = g / (1.f + __expf(-g)) * u;
}

hipError_t launch_swiglu_up(int bf16, const void* x, const void* wg, const void* wu, void* h,
                            int L, int d, int d_ff, hipStream_t s) {
  if (L == 0 || d_ff == 0) return hipSuccess;
  if (bf16) {
    const uint16_t* px = static_cast<const uint16_t*>(x);
    const uint16_t* pg = static_cast<const uint16_t*>(wg);
    const uint16_t* pu = static_cast<const uint16_t*>(wu);
    uint16_t* ph = static_cast<uint16_t*>(h);
    const int n_log = 2 * ((d_ff + 15) / 16 * 16);  // interleaved gate / up columns
    const int big_mt = (L + GBM - 1) / GBM, big_nt = (n_log + GBN - 1) / GBN;
    if (d % GBK == 0 && big_mt * big_nt >= 192) {
      router_gemm_bf16_big_kernel<kEpiSwiglu><<<big_mt * big_nt, 512, 0, s>>>(
          px, pg, pu, nullptr, nullptr, nullptr, nullptr, L, d, d_ff, 0, big_mt, big_nt, 0, ph);
    } else {
      const int n_mt = (L + RBM - 1) / RBM, n_nt = (n_log + RBN - 1) / RBN;
      router_gemm_bf16_kernel<kEpiSwiglu><<<n_mt * n_nt, 256, 0, s>>>(
          px, pg, pu, nullptr, nullptr, nullptr, nullptr, L, d, d_ff, 0, n_mt, n_nt, 0, ph, d);
    }
  } else {
    const size_t n = static_cast<size_t>(L) * d_ff;
    swiglu_f32_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, s>>>(
        static_cast<const float*>(x), static_cast<const float*>(wg), static_cast<const float*>(wu),
        L, d, d_ff, static_cast<float*>(h));
  }
  return hipGetLastError();
}

}  // namespace omni
