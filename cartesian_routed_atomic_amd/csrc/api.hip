// C ABI of the routed atomic-expert layer: argument validation, workspace
// sizing and dispatch to the gfx950 kernels.  Every check runs on the host
// before anything is enqueued; nothing here allocates or synchronises.
#include <stdint.h>

#include <mutex>

#include "../../include/omni.h"
#include "launch.hpp"

namespace {

constexpr int kAbiVersion = 14;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned256(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }
bool fits_i32(long long v) { return v >= 0 && v < (1ll << 31); }

omni_status hip_status(hipError_t e) { return e == hipSuccess ? OMNI_OK : OMNI_ERR_HIP; }

}  // namespace

extern "C" {

int omni_abi_version(void) { return kAbiVersion; }

const char* omni_status_string(omni_status s) {
  switch (s) {
    case OMNI_OK: return "ok";
    case OMNI_ERR_INVALID_ARG: return "invalid argument";
    case OMNI_ERR_WORKSPACE: return "workspace missing or too small";
    case OMNI_ERR_UNSUPPORTED: return "shape or type not covered by the kernels";
    case OMNI_ERR_HIP: return "kernel launch failed";
    default: return "unknown status";
  }
}

size_t omni_router_logits_workspace(omni_dtype dt, int L, int d, int Nr, int Nc) {
  if (dt != OMNI_F32 && dt != OMNI_BF16) return 0;
  if (L < 0 || d < 1 || Nr < 1 || Nc < 1) return 0;
  if (!fits_i32(static_cast<long long>(L) * (Nr + static_cast<long long>(Nc)))) return 0;
  return omni::router_ws_bytes(dt == OMNI_BF16, L, d, Nr, Nc);
}

omni_status omni_router_logits(omni_dtype dt, int L, int d, int Nr, int Nc, const void* x,
                               const void* wr_t, const void* wc_t, const float* row_bias,
                               const float* col_bias, float* row_logits, float* col_logits,
                               void* ws, size_t ws_bytes, hipStream_t stream) {
  if (dt != OMNI_F32 && dt != OMNI_BF16) return OMNI_ERR_INVALID_ARG;
  if (L < 0 || d < 1 || Nr < 1 || Nc < 1) return OMNI_ERR_INVALID_ARG;
  if (!wr_t || !wc_t) return OMNI_ERR_INVALID_ARG;
  if (L > 0 && (!x || !row_logits || !col_logits)) return OMNI_ERR_INVALID_ARG;
  if (!fits_i32(static_cast<long long>(L) * d) || !fits_i32(static_cast<long long>(L) * Nr) ||
      !fits_i32(static_cast<long long>(L) * Nc) ||
      !fits_i32(static_cast<long long>(Nr + static_cast<long long>(Nc)) * d))
    return OMNI_ERR_UNSUPPORTED;
  if ((L > 0 && !aligned16(x)) || !aligned16(wr_t) || !aligned16(wc_t))
    return OMNI_ERR_INVALID_ARG;
  if (dt == OMNI_BF16 && d % 8 != 0) return OMNI_ERR_UNSUPPORTED;
  if (dt == OMNI_F32 && d % 4 != 0) return OMNI_ERR_UNSUPPORTED;
  const size_t need = omni_router_logits_workspace(dt, L, d, Nr, Nc);
  if (need > 0 && (!ws || ws_bytes < need || !aligned256(ws))) return OMNI_ERR_WORKSPACE;
  if (L == 0) return OMNI_OK;
  hipError_t e;
  if (dt == OMNI_BF16)
    e = omni::launch_router_bf16(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(wr_t),
                                 static_cast<const uint16_t*>(wc_t), row_bias, col_bias,
                                 row_logits, col_logits, L, d, Nr, Nc, need > 0 ? ws : nullptr,
                                 stream);
  else
    e = omni::launch_router_f32(static_cast<const float*>(x), static_cast<const float*>(wr_t),
                                static_cast<const float*>(wc_t), row_bias, col_bias, row_logits,
                                col_logits, L, d, Nr, Nc, stream);
  return hip_status(e);
}

static size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Workspace of omni_product_topk: a tie flag and the two float32 normalisers
// per token, then room for the per-axis lists the caller does not ask for.
struct TopkWs {
  size_t lse, rsel, csel, bytes;  // byte offsets (the flags start at 0)
};
static TopkWs topk_ws_layout(int L, int kprime, bool lists_r, bool lists_c) {
  const size_t list = align256(static_cast<size_t>(L) * static_cast<size_t>(kprime) * 4);
  TopkWs w;
  w.lse = align256(static_cast<size_t>(L) * 4);
  w.rsel = w.lse + align256(static_cast<size_t>(L) * 8);
  w.csel = w.rsel + (lists_r ? list : 0);
  w.bytes = w.csel + (lists_c ? list : 0);
  return w;
}

size_t omni_product_topk_workspace(int L, int Nr, int Nc, int kprime, int K) {
  (void)Nr; (void)Nc; (void)K;
  if (L <= 0 || kprime < 1) return 0;
  return topk_ws_layout(L, kprime, true, true).bytes;
}

// Argument checks shared by both top-K entry points.
static omni_status topk_args(int L, int Nr, int Nc, int kprime, int K, const float* row_logits,
                             const float* col_logits, const int32_t* expert_idx,
                             const float* score, const float* gate) {
  if (L < 0 || Nr < 1 || Nc < 1) return OMNI_ERR_INVALID_ARG;
  if (kprime < 1 || kprime > Nr || kprime > Nc) return OMNI_ERR_INVALID_ARG;
  if (K < 1 || static_cast<long long>(K) > static_cast<long long>(kprime) * kprime)
    return OMNI_ERR_INVALID_ARG;
  if (!fits_i32(static_cast<long long>(Nr) * Nc)) return OMNI_ERR_INVALID_ARG;
  if (L > 0 && (!row_logits || !col_logits || !expert_idx || !score || !gate))
    return OMNI_ERR_INVALID_ARG;
  if (kprime > 64 || K > 64 || Nr > 2048 || Nc > 2048) return OMNI_ERR_UNSUPPORTED;
  if (!fits_i32(static_cast<long long>(L) * Nr) || !fits_i32(static_cast<long long>(L) * Nc) ||
      !fits_i32(static_cast<long long>(L) * K) || !fits_i32(static_cast<long long>(L) * kprime))
    return OMNI_ERR_UNSUPPORTED;
  return OMNI_OK;
}

static omni_status topk_run(int L, int Nr, int Nc, int kprime, int K, const float* row_logits,
                            const float* col_logits, int32_t* expert_idx, float* score,
                            float* gate, float* row_logp, float* col_logp, int32_t* row_sel,
                            int32_t* col_sel, char* base, const TopkWs& w, hipStream_t stream) {
  int32_t* flags = reinterpret_cast<int32_t*>(base);
  float* lse = reinterpret_cast<float*>(base + w.lse);
  int32_t* rsel = row_sel ? row_sel : reinterpret_cast<int32_t*>(base + w.rsel);
  int32_t* csel = col_sel ? col_sel : reinterpret_cast<int32_t*>(base + w.csel);
  return hip_status(omni::launch_product_topk(row_logits, col_logits, L, Nr, Nc, kprime, K,
                                              expert_idx, score, gate, row_logp, col_logp, rsel,
                                              csel, flags, lse, stream));
}

omni_status omni_product_topk(int L, int Nr, int Nc, int kprime, int K, const float* row_logits,
                              const float* col_logits, int32_t* expert_idx, float* score,
                              float* gate, float* row_logp, float* col_logp, int32_t* row_sel,
                              int32_t* col_sel, void* ws, size_t ws_bytes, hipStream_t stream) {
  const omni_status a = topk_args(L, Nr, Nc, kprime, K, row_logits, col_logits, expert_idx,
                                  score, gate);
  if (a != OMNI_OK) return a;
  if (L == 0) return OMNI_OK;
  const TopkWs w = topk_ws_layout(L, kprime, true, true);
  if (!ws || ws_bytes < w.bytes || !aligned256(ws)) return OMNI_ERR_WORKSPACE;
  return topk_run(L, Nr, Nc, kprime, K, row_logits, col_logits, expert_idx, score, gate,
                  row_logp, col_logp, row_sel, col_sel, static_cast<char*>(ws), w, stream);
}

// omni_product_topk_static: the same call with its workspace in a fixed
// device array (one per GPU, held until the process ends).  Host code never
// passes the array's name to a kernel: the device address comes from
// hipGetSymbolAddress, once per device, on the first call there.
static __device__ __align__(256) uint8_t scratch[OMNI_TOPK_STATIC_SCRATCH_BYTES];

static std::mutex g_scratch_mu;
static void* g_scratch_ptr[256];

static omni_status scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 256) return OMNI_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return OMNI_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return OMNI_OK;
}

omni_status omni_product_topk_static(int L, int Nr, int Nc, int kprime, int K,
                                     const float* row_logits, const float* col_logits,
                                     int32_t* expert_idx, float* score, float* gate,
                                     float* row_logp, float* col_logp, int32_t* row_sel,
                                     int32_t* col_sel, hipStream_t stream) {
  const omni_status a = topk_args(L, Nr, Nc, kprime, K, row_logits, col_logits, expert_idx,
                                  score, gate);
  if (a != OMNI_OK) return a;
  if (L == 0) return OMNI_OK;
  const TopkWs w = topk_ws_layout(L, kprime, row_sel == nullptr, col_sel == nullptr);
  if (w.bytes > OMNI_TOPK_STATIC_SCRATCH_BYTES) return OMNI_ERR_WORKSPACE;
  void* p = nullptr;
  const omni_status e = scratch_ptr(&p);
  if (e != OMNI_OK) return e;
  return topk_run(L, Nr, Nc, kprime, K, row_logits, col_logits, expert_idx, score, gate,
                  row_logp, col_logp, row_sel, col_sel, static_cast<char*>(p), w, stream);
}

static bool grouping_ok(omni_grouping g) {
  return g == OMNI_GROUP_ACTIVE || g == OMNI_GROUP_ID_WINDOW;
}

int omni_schedule_max_groups(int L, int K, int N, int B, omni_grouping grouping) {
  if (L < 0 || K < 1 || N < 1 || B < 1 || !grouping_ok(grouping)) return 0;
  const long long M = static_cast<long long>(L) * K;
  const long long mn = grouping == OMNI_GROUP_ID_WINDOW ? N : (M < N ? M : N);
  return static_cast<int>((mn + B - 1) / B);
}

static bool schedule_args_ok(int L, int K, int N, int B) {
  return L >= 0 && K >= 1 && N >= 1 && B >= 1 && fits_i32(static_cast<long long>(L) * K);
}

size_t omni_schedule_workspace(int L, int K, int N, int B, omni_grouping grouping) {
  if (!schedule_args_ok(L, K, N, B) || !grouping_ok(grouping)) return 0;
  return omni::schedule_ws_layout(L, K, N, B, grouping == OMNI_GROUP_ID_WINDOW).bytes;
}

omni_status omni_schedule_tasks(int L, int K, int N, int B, omni_grouping grouping,
                                const int32_t* expert_idx, const float* gate,
                                const omni_schedule* out, void* ws, size_t ws_bytes,
                                hipStream_t stream) {
  if (!schedule_args_ok(L, K, N, B) || !grouping_ok(grouping)) return OMNI_ERR_INVALID_ARG;
  if (!out || !out->counts || !out->group_offsets) return OMNI_ERR_INVALID_ARG;
  const long long M = static_cast<long long>(L) * K;
  if (M > 0 && (!expert_idx || !gate || !out->active || !out->task_token || !out->task_expert ||
                !out->task_gate))
    return OMNI_ERR_INVALID_ARG;
  const size_t need = omni_schedule_workspace(L, K, N, B, grouping);
  if (M > 0 && (!ws || ws_bytes < need)) return OMNI_ERR_WORKSPACE;
  if (M > 0 && !aligned256(ws)) return OMNI_ERR_WORKSPACE;
  return hip_status(omni::launch_schedule(L, K, N, B, grouping == OMNI_GROUP_ID_WINDOW,
                                          expert_idx, gate, out->counts, out->active,
                                          out->group_offsets, out->task_token, out->task_expert,
                                          out->task_gate, out->task_index, ws, stream));
}

int omni_atomic_forward_mode(omni_dtype dt, int L, int d, int N, int K, int B) {
  if (dt != OMNI_F32 && dt != OMNI_BF16) return 0;
  if (!schedule_args_ok(L, K, N, B) || d < 1) return 0;
  return omni::auto_exec_mode(dt == OMNI_BF16, L, d, N, K);
}

static bool exec_mode_ok(omni_exec_mode m) {
  return m == OMNI_EXEC_AUTO || m == OMNI_EXEC_EXPERT_CENTRIC || m == OMNI_EXEC_TOKEN_CENTRIC ||
         m == OMNI_EXEC_GROUPED;
}

// The form a call runs: AUTO resolved the way omni_atomic_forward resolves it.
static int resolve_form(omni_dtype dt, int L, int d, int N, int K, omni_exec_mode mode) {
  return mode == OMNI_EXEC_AUTO ? omni::auto_exec_mode(dt == OMNI_BF16, L, d, N, K)
                                : static_cast<int>(mode);
}

size_t omni_atomic_forward_workspace(omni_dtype dt, int L, int d, int N, int K, int B,
                                     omni_exec_mode mode) {
  (void)B;
  if (dt != OMNI_F32 && dt != OMNI_BF16) return 0;
  if (!exec_mode_ok(mode) || N < 1 || d < 1) return 0;
  if (L <= 0 || K < 1 || !fits_i32(static_cast<long long>(L) * K)) return 0;
  return omni::exec_ws_bytes(resolve_form(dt, L, d, N, K, mode), L, d, N, K);
}

omni_status omni_atomic_forward(omni_dtype dt, int L, int d, int N, int K, int B, const void* x,
                                const void* w, const void* v, const omni_schedule* sched,
                                float* y, int accumulate, omni_exec_mode mode, void* ws,
                                size_t ws_bytes, hipStream_t stream) {
  if (dt != OMNI_F32 && dt != OMNI_BF16) return OMNI_ERR_INVALID_ARG;
  if (!exec_mode_ok(mode)) return OMNI_ERR_INVALID_ARG;
  if (!schedule_args_ok(L, K, N, B) || d < 1) return OMNI_ERR_INVALID_ARG;
  if (!w || !v || !sched) return OMNI_ERR_INVALID_ARG;
  const long long M = static_cast<long long>(L) * K;
  if (L > 0 && (!x || !y)) return OMNI_ERR_INVALID_ARG;
  if (M > 0 && (!sched->task_token || !sched->task_expert || !sched->task_gate ||
                !sched->task_index))
    return OMNI_ERR_INVALID_ARG;
  if ((sched->flat_expert == nullptr) != (sched->flat_gate == nullptr))
    return OMNI_ERR_INVALID_ARG;
  if (!omni::chunked_supported(d)) return OMNI_ERR_UNSUPPORTED;
  const int bf16 = dt == OMNI_BF16;
  const int form = resolve_form(dt, L, d, N, K, mode);
  if (form == OMNI_EXEC_GROUPED && !omni::grouped_supported(bf16, d, K))
    return OMNI_ERR_UNSUPPORTED;
  if ((L > 0 && !aligned16(x)) || !aligned16(w) || !aligned16(v)) return OMNI_ERR_INVALID_ARG;
  if (L > 0 && !aligned16(y)) return OMNI_ERR_INVALID_ARG;
  if (!fits_i32(static_cast<long long>(L) * d)) return OMNI_ERR_UNSUPPORTED;
  if (L == 0) return OMNI_OK;
  const size_t need = omni_atomic_forward_workspace(dt, L, d, N, K, B,
                                                    static_cast<omni_exec_mode>(form));
  if (need > 0 && (!ws || ws_bytes < need || !aligned256(ws))) return OMNI_ERR_WORKSPACE;
  return hip_status(omni::launch_atomic_forward(bf16, form, L, d, N, K, x, w, v,
                                                sched->task_token, sched->task_expert,
                                                sched->task_gate, sched->task_index,
                                                sched->flat_expert, sched->flat_gate, y,
                                                accumulate != 0, ws, stream));
}

omni_status omni_atomic_forward_glu(omni_dtype dt, int L, int d, int N, int K, int B,
                                    const void* x, const void* w, const void* u, const void* v,
                                    const omni_schedule* sched, float* y, int accumulate,
                                    void* ws, size_t ws_bytes, hipStream_t stream) {
  if (dt != OMNI_F32 && dt != OMNI_BF16) return OMNI_ERR_INVALID_ARG;
  if (!schedule_args_ok(L, K, N, B) || d < 1) return OMNI_ERR_INVALID_ARG;
  if (!w || !u || !v || !sched) return OMNI_ERR_INVALID_ARG;
  const long long M = static_cast<long long>(L) * K;
  if (L > 0 && (!x || !y)) return OMNI_ERR_INVALID_ARG;
  if (M > 0 && (!sched->task_expert || !sched->task_gate || !sched->task_index))
    return OMNI_ERR_INVALID_ARG;
  if ((sched->flat_expert == nullptr) != (sched->flat_gate == nullptr))
    return OMNI_ERR_INVALID_ARG;
  const int bf16 = dt == OMNI_BF16;
  if (!omni::chunked_supported(d)) return OMNI_ERR_UNSUPPORTED;
  if ((L > 0 && !aligned16(x)) || !aligned16(w) || !aligned16(u) || !aligned16(v))
    return OMNI_ERR_INVALID_ARG;
  if (L > 0 && !aligned16(y)) return OMNI_ERR_INVALID_ARG;
  if (!fits_i32(static_cast<long long>(L) * d)) return OMNI_ERR_UNSUPPORTED;
  if (L == 0) return OMNI_OK;
  const size_t need = omni_atomic_forward_workspace(dt, L, d, N, K, B, OMNI_EXEC_TOKEN_CENTRIC);
  if (need > 0 && (!ws || ws_bytes < need || !aligned256(ws))) return OMNI_ERR_WORKSPACE;
  return hip_status(omni::launch_atomic_forward_glu(bf16, L, d, N, K, x, w, u, v,
                                                    sched->task_expert, sched->task_gate,
                                                    sched->task_index, sched->flat_expert,
                                                    sched->flat_gate, y, accumulate != 0, ws,
                                                    stream));
}

size_t omni_flat_router_workspace(omni_dtype dt, int L, int N) {
  if (dt != OMNI_F32 && dt != OMNI_BF16) return 0;
  if (L < 0 || N < 1) return 0;
  return omni::flat_router_ws_bytes(L, N);
}

omni_status omni_flat_router_topk(omni_dtype dt, int L, int d, int N, int K, const void* x,
                                  const void* wf, const float* bias, int32_t* expert_idx,
                                  float* score, float* gate, float* logp, void* ws,
                                  size_t ws_bytes, hipStream_t stream) {
  if (dt != OMNI_F32 && dt != OMNI_BF16) return OMNI_ERR_INVALID_ARG;
  if (L < 0 || d < 1 || N < 1 || K < 1 || K > N) return OMNI_ERR_INVALID_ARG;
  if (!wf) return OMNI_ERR_INVALID_ARG;
  if (L > 0 && (!x || !expert_idx || !score || !gate)) return OMNI_ERR_INVALID_ARG;
  if (K > 64) return OMNI_ERR_UNSUPPORTED;
  // the kernels index rows of wf and of the logits in 64 bits
  if (!fits_i32(static_cast<long long>(L) * d) || !fits_i32(static_cast<long long>(L) * K))
    return OMNI_ERR_UNSUPPORTED;
  if (dt == OMNI_BF16 && d % 8 != 0) return OMNI_ERR_UNSUPPORTED;
  if (dt == OMNI_F32 && d % 4 != 0) return OMNI_ERR_UNSUPPORTED;
  if ((L > 0 && !aligned16(x)) || !aligned16(wf)) return OMNI_ERR_INVALID_ARG;
  if (L == 0) return OMNI_OK;
  const size_t need = omni_flat_router_workspace(dt, L, N);
  if (!ws || ws_bytes < need || !aligned256(ws)) return OMNI_ERR_WORKSPACE;
  return hip_status(omni::launch_flat_router(dt == OMNI_BF16, L, d, N, K, x, wf, bias,
                                             expert_idx, score, gate, logp, ws, stream));
}

size_t omni_routed_backward_workspace(omni_dtype dt, int L, int d, int Nr, int Nc, int K) {
  if (dt != OMNI_F32 && dt != OMNI_BF16) return 0;
  if (L < 0 || d < 1 || Nr < 1 || Nc < 1 || K < 1 || K > 64) return 0;
  if (!fits_i32(static_cast<long long>(Nr) * Nc) || !fits_i32(static_cast<long long>(L) * K))
    return 0;
  return omni::routed_backward_ws_bytes(dt == OMNI_BF16, L, d, Nr, Nc, K);
}

omni_status omni_routed_backward(omni_dtype dt, int L, int d, int Nr, int Nc, int K,
                                 const void* x, const void* wr_t, const void* wc_t,
                                 const void* w, const void* v, const int32_t* expert_idx,
                                 const float* gate, const float* dy, float* dx, float* dwr_t,
                                 float* dwc_t, float* drow_bias, float* dcol_bias,
                                 int32_t* counts, int32_t* active, float* dw, float* dv,
                                 float* dgate, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (dt != OMNI_F32 && dt != OMNI_BF16) return OMNI_ERR_INVALID_ARG;
  if (L < 0 || d < 1 || Nr < 1 || Nc < 1 || K < 1) return OMNI_ERR_INVALID_ARG;
  if (!fits_i32(static_cast<long long>(Nr) * Nc) || !fits_i32(static_cast<long long>(L) * K) ||
      !fits_i32(static_cast<long long>(L) * d))
    return OMNI_ERR_INVALID_ARG;
  if (!wr_t || !wc_t || !w || !v || !dwr_t || !dwc_t || !counts || !active || !dw || !dv)
    return OMNI_ERR_INVALID_ARG;
  if (L > 0 && (!x || !expert_idx || !gate || !dy || !dx)) return OMNI_ERR_INVALID_ARG;
  if (!omni::routed_backward_supported(dt == OMNI_BF16, d, K)) return OMNI_ERR_UNSUPPORTED;
  const void* rows[] = {x, wr_t, wc_t, w, v, dy, dx, dwr_t, dwc_t, dw, dv};
  for (const void* p : rows)
    if (p && !aligned16(p)) return OMNI_ERR_INVALID_ARG;
  const size_t need = omni_routed_backward_workspace(dt, L, d, Nr, Nc, K);
  if (!ws || ws_bytes < need || !aligned256(ws)) return OMNI_ERR_WORKSPACE;
  return hip_status(omni::launch_routed_backward(
      dt == OMNI_BF16, L, d, Nr, Nc, K, x, wr_t, wc_t, w, v, expert_idx, gate, dy, dx, dwr_t,
      dwc_t, drow_bias, dcol_bias, counts, active, dw, dv, dgate, ws, stream));
}

// The hidden activation, then the split-K partials of the down product.
static size_t mlp_hidden_bytes(omni_dtype dt, int L, int d_ff) {
  const size_t n = static_cast<size_t>(L > 0 ? L : 1) * d_ff * (dt == OMNI_BF16 ? 2 : 4);
  return (n + 255) & ~static_cast<size_t>(255);
}

size_t omni_shared_mlp_workspace(omni_dtype dt, int L, int d, int d_ff) {
  if (dt != OMNI_F32 && dt != OMNI_BF16) return 0;
  if (L < 0 || d < 1 || d_ff < 1 || !fits_i32(static_cast<long long>(L) * d_ff)) return 0;
  return mlp_hidden_bytes(dt, L, d_ff) + omni::gemm_nt_ws_bytes(dt == OMNI_BF16, L, d, d_ff);
}

omni_status omni_shared_mlp(omni_dtype dt, int L, int d, int d_ff, const void* x,
                            const void* w_gate, const void* w_up, const void* w_down, float* y,
                            int accumulate, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (dt != OMNI_F32 && dt != OMNI_BF16) return OMNI_ERR_INVALID_ARG;
  if (L < 0 || d < 1 || d_ff < 1) return OMNI_ERR_INVALID_ARG;
  if (!fits_i32(static_cast<long long>(L) * d) || !fits_i32(static_cast<long long>(L) * d_ff) ||
      !fits_i32(static_cast<long long>(d) * d_ff))
    return OMNI_ERR_INVALID_ARG;
  if (!w_gate || !w_up || !w_down) return OMNI_ERR_INVALID_ARG;
  if (L > 0 && (!x || !y)) return OMNI_ERR_INVALID_ARG;
  const int mult = dt == OMNI_BF16 ? 8 : 4;
  if (d % mult != 0 || d_ff % mult != 0) return OMNI_ERR_UNSUPPORTED;
  const void* rows[] = {x, w_gate, w_up, w_down, y};
  for (const void* p : rows)
    if (p && !aligned16(p)) return OMNI_ERR_INVALID_ARG;
  if (L == 0) return OMNI_OK;
  const size_t need = omni_shared_mlp_workspace(dt, L, d, d_ff);
  if (!ws || ws_bytes < need || !aligned256(ws)) return OMNI_ERR_WORKSPACE;
  const int bf16 = dt == OMNI_BF16;
  hipError_t e = omni::launch_swiglu_up(bf16, x, w_gate, w_up, ws, L, d, d_ff, stream);
  if (e != hipSuccess) return hip_status(e);
  void* part = omni::gemm_nt_ws_bytes(bf16, L, d, d_ff) > 0
                   ? static_cast<char*>(ws) + mlp_hidden_bytes(dt, L, d_ff)
                   : nullptr;
  return hip_status(omni::launch_gemm_nt(bf16, ws, w_down, y, L, d, d_ff, accumulate, part,
                                         stream));
}

}  // extern "C"
