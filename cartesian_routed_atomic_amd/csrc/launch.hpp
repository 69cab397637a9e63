// Internal host-side launch interface between the C ABI (api.hip) and the
// kernel files.  Every function enqueues on `s` and returns the launch error.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace omni {

// router.hip
// ws: split-K partials (router_ws_bytes of them); NULL runs without a split
size_t router_ws_bytes(int bf16, int L, int d, int Nr, int Nc);
hipError_t launch_router_bf16(const uint16_t* x, const uint16_t* wr, const uint16_t* wc,
                              const float* rb, const float* cb, float* zr, float* zc,
                              int L, int d, int Nr, int Nc, void* ws, hipStream_t s);
hipError_t launch_router_f32(const float* x, const float* wr, const float* wc,
                             const float* rb, const float* cb, float* zr, float* zc,
                             int L, int d, int Nr, int Nc, hipStream_t s);
// c[M, N] (+)= a[M, K] b[N, K]^T, row-major, fp32 accumulation; a, b bf16
// bits (bf16 != 0, K a multiple of 8) or float32 (K a multiple of 4).
// ws: split-K partials for shapes with few tiles (gemm_nt_ws_bytes of them),
// or NULL to run without a split.
size_t gemm_nt_ws_bytes(int bf16, int M, int N, int K);
hipError_t launch_gemm_nt(int bf16, const void* a, const void* b, float* c, int M, int N, int K,
                          int accumulate, void* ws, hipStream_t s);
// h[L, d_ff] = silu(x Wg^T) * (x Wu^T); x [L, d], wg / wu [d_ff, d]; h is bf16
// bits (bf16 != 0, d a multiple of 8) or float32 (d a multiple of 4).
hipError_t launch_swiglu_up(int bf16, const void* x, const void* wg, const void* wu, void* h,
                            int L, int d, int d_ff, hipStream_t s);

// topk.hip
hipError_t launch_product_topk(const float* zr, const float* zc, int L, int Nr, int Nc, int kp,
                               int K, int32_t* expert_idx, float* score, float* gate,
                               float* row_logp, float* col_logp, int32_t* row_sel,
                               int32_t* col_sel, int32_t* tie_flag, float* lse,
                               hipStream_t s);

// schedule.hip
struct ScheduleWs {
  size_t bytes;
  size_t flags, tile_cnt, rank, key0, val0, key1, val1, hist, dtot;  // byte offsets
  int n_ftiles, n_ttiles, passes, max_groups;
  int dbits;  // digit bits per radix pass
};
// window = 0: groups of B active experts in id order; window != 0: group g
// is the id window [g B, (g + 1) B), every window a group.
ScheduleWs schedule_ws_layout(int L, int K, int N, int B, int window);
hipError_t launch_schedule(int L, int K, int N, int B, int window, const int32_t* expert_idx,
                           const float* gate, int32_t* counts, int32_t* active,
                           int32_t* group_offsets, int32_t* task_token, int32_t* task_expert,
                           float* task_gate, int32_t* task_index, void* ws, hipStream_t s);

// execute.hip
size_t atomic_forward_ws_bytes(int L, int K);
// true: read expert rows with the nontemporal hint (M tasks over N experts)
bool stream_rows(long long M, long long N);
// the token-centric kernels that hold a row per wave: d a power of two, rows
// of at most 4 KiB (other widths run the chunked kernels)
bool token_rows_in_registers(int bf16, int d);
// schedule order -> flatten order: le[task_index[m]] = task_expert[m] (ids
// outside [0, N) mapped to 0), lg[task_index[m]] = task_gate[m]
hipError_t launch_unpermute(const int32_t* texp, const float* tgate, const int32_t* tidx, int M,
                            int N, int32_t* le, float* lg, hipStream_t s);
// 1 expert-centric, 2 token-centric, 3 grouped
int auto_exec_mode(int bf16, int L, int d, int N, int K);
// workspace of one form (mode 1, 2 or 3)
size_t exec_ws_bytes(int mode, int L, int d, int N, int K);
// flat_expert / flat_gate: the selection in flatten order, or NULL (the
// token-centric and grouped forms then invert the sorted order through
// task_index); sched_counts / active: the schedule's (grouped form only)
hipError_t launch_atomic_forward(int bf16, int mode, int L, int d, int N, int K, const void* x,
                                 const void* w, const void* v, const int32_t* task_token,
                                 const int32_t* task_expert, const float* task_gate,
                                 const int32_t* task_index, const int32_t* flat_expert,
                                 const float* flat_gate, float* y, bool accumulate, void* ws,
                                 hipStream_t s);
// SwiGLU-gated variant (third matrix u), token-centric form only
hipError_t launch_atomic_forward_glu(int bf16, int L, int d, int N, int K, const void* x,
                                     const void* w, const void* u, const void* v,
                                     const int32_t* task_expert, const float* task_gate,
                                     const int32_t* task_index, const int32_t* flat_expert,
                                     const float* flat_gate, float* y, bool accumulate,
                                     void* ws, hipStream_t s);

// chunked.hip: the expert-centric (form 1) and token-centric (form 2) forms
// for any d = 64 m up to 16384, the row taken in chunks; glu: the gated
// variant (form 2 only).  ws: atomic_forward_ws_bytes(L, K).
bool chunked_supported(int d);
hipError_t launch_chunked(int bf16, int form, bool glu, int L, int d, int N, int K,
                          const void* x, const void* w, const void* u, const void* v,
                          const int32_t* task_token, const int32_t* task_expert,
                          const float* task_gate, const int32_t* task_index,
                          const int32_t* flat_expert, const float* flat_gate, float* y,
                          bool accumulate, void* ws, hipStream_t s);

// grouped.hip: the grouped form (bf16, K <= 64, rows of at most 4 KiB).  The
// hot set comes from the sorted schedule (counts, active, task_expert); the
// token tiles read the flattened selection fe / fg.  gws: grouped_ws_bytes.
size_t grouped_ws_bytes(int L, int K, int d, int N);
bool grouped_supported(int bf16, int d, int K);
hipError_t launch_grouped(const uint16_t* x, const uint16_t* w, const uint16_t* v,
                          const int32_t* task_expert, const int32_t* fe, const float* fg, int L,
                          int K, int d, int N, float* y, int accumulate, void* gws,
                          hipStream_t s);

// flat_router.hip: the d x N router baseline
size_t flat_router_ws_bytes(int L, int N);
hipError_t launch_flat_router(int bf16, int L, int d, int N, int K, const void* x,
                              const void* wf, const float* bias, int32_t* expert_idx,
                              float* score, float* gate, float* logp, void* ws, hipStream_t s);

// backward.hip
size_t routed_backward_ws_bytes(int bf16, int L, int d, int Nr, int Nc, int K);
bool routed_backward_supported(int bf16, int d, int K);
hipError_t launch_routed_backward(int bf16, int L, int d, int Nr, int Nc, int K, const void* x,
                                  const void* wr, const void* wc, const void* w, const void* v,
                                  const int32_t* expert_idx, const float* gate, const float* dy,
                                  float* dx, float* dwr, float* dwc, float* drb, float* dcb,
                                  int32_t* counts, int32_t* active, float* dw, float* dv,
                                  float* dgate, void* ws, hipStream_t s);

}  // namespace omni
