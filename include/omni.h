/*
 * omni.h — C ABI of the MI355X (gfx950) OmniMoE routed atomic-expert layer,
 * forward pass.
 *
 * The layer (pages: "OmniMoE: An Efficient MoE by Orchestrating Atomic
 * Experts at Scale", gist.science explainer §2.1-§2.2, and the OmniMoE
 * interactive explainer, sections "Atomic Expert / DEA", "Cartesian Product
 * Router", "Expert-Centric Scheduling"):
 *
 *   1. omni_router_logits   row / column logits of the Cartesian Product
 *                           Router over an Nr x Nc expert grid;
 *   2. omni_product_topk    per-axis log-softmax and top-k', then top-K over
 *                           the k' x k' product cells with
 *                           S = log p_r[i] + log p_c[j], plus the gates
 *                           (softmax over the K selected S);
 *   3. omni_schedule_tasks  Expert-Centric Scheduling: flatten the L*K
 *                           (token, expert, gate) tasks, group the unique
 *                           active experts B at a time, order the tasks by
 *                           (group, token);
 *   4. omni_atomic_forward  execution of the schedule:
 *                           y_t = sum_k g_tk * silu(x_t . W[e_tk]) * V[e_tk],
 *                           expert-centric or token-centric (same result);
 *   5. omni_routed_backward gradients of the whole routed layer.
 *
 * Conventions shared by every call
 *   - All pointers except the `omni_schedule` descriptor itself are DEVICE
 *     pointers owned by the caller.  The library never allocates, frees or
 *     synchronises; every call only enqueues kernels on `stream` and returns.
 *   - Matrices are dense row-major.  bf16 data is raw bfloat16 bits.
 *   - Shapes and pointers are validated on the host before anything is
 *     enqueued; a failed check returns a non-OK status and enqueues nothing.
 *     A failed launch returns OMNI_ERR_HIP.  Faults during execution surface
 *     at the caller's next synchronisation.
 *   - Inputs must be finite; NaN / Inf inputs give unspecified results.
 *   - Expert ids: grid cell (i, j) is expert e = i * Nc + j (row-major).
 *   - Tie rule everywhere: larger value first, then lower index; values are
 *     compared as float32 numbers (-0 == +0).
 *   - L == 0 is accepted and enqueues only what writes the (empty) outputs.
 *     A call that then enqueues nothing takes a null workspace; the backward
 *     still writes its (zero) router gradients through its workspace.
 */
#ifndef OMNI_H
#define OMNI_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum omni_status {
  OMNI_OK = 0,
  OMNI_ERR_INVALID_ARG = 1,   /* bad shape, null or misaligned pointer      */
  OMNI_ERR_WORKSPACE = 2,     /* workspace pointer null or smaller than asked */
  OMNI_ERR_UNSUPPORTED = 3,   /* valid request outside what the kernels cover */
  OMNI_ERR_HIP = 4            /* a kernel launch failed                      */
} omni_status;

typedef enum omni_dtype {
  OMNI_F32 = 0,               /* float32 x, weights                          */
  OMNI_BF16 = 1               /* bfloat16 x, weights; float32 accumulation   */
} omni_dtype;

/* ABI revision of this header. */
int omni_abi_version(void);  /* 14 */

/* Human-readable name of a status code (static string, never NULL). */
const char* omni_status_string(omni_status s);

/*
 * omni_router_logits — Cartesian Product Router, row and column logits.
 * Pages: gist.science explainer §2.2 "Cartesian Product Router" (two small
 * projections give independent low-dimensional row and column logits over
 * the Nr x Nc grid).
 *
 *   row_logits[t, i] = x[t,:] . Wr[:, i] + row_bias[i]
 *   col_logits[t, j] = x[t,:] . Wc[:, j] + col_bias[j]
 *
 * dt          OMNI_BF16 (MFMA path, float32 accumulation) or OMNI_F32.
 * x           [L, d] of dt.
 * wr_t        [Nr, d] of dt: row i holds the d weights that score grid row i
 *             (Wr of the pages, Wr in R^{d x Nr}, stored transposed).
 * wc_t        [Nc, d] of dt, likewise for grid columns.
 * row_bias    [Nr] float32 or NULL;  col_bias [Nc] float32 or NULL.
 * row_logits  [L, Nr] float32 out;   col_logits [L, Nc] float32 out.
 * ws          workspace of at least omni_router_logits_workspace(...) bytes,
 *             256-byte aligned, or NULL with ws_bytes 0 when that is 0.  Shapes
 *             with few tokens or few grid lines split the contraction over d
 *             (partial products summed in a fixed order, so the result is
 *             deterministic); the workspace holds the partials.
 * Requires L >= 0, d >= 1, Nr >= 1, Nc >= 1; for bf16 d % 8 == 0 and
 * x, wr_t, wc_t 16-byte aligned; for f32 d % 4 == 0 and 16-byte aligned.
 */
size_t omni_router_logits_workspace(omni_dtype dt, int L, int d, int Nr, int Nc);
omni_status omni_router_logits(omni_dtype dt, int L, int d, int Nr, int Nc,
                               const void* x, const void* wr_t, const void* wc_t,
                               const float* row_bias, const float* col_bias,
                               float* row_logits, float* col_logits, void* ws,
                               size_t ws_bytes, hipStream_t stream);

/*
 * omni_product_topk — per-axis log-probabilities, top-K over the product
 * grid, and the gates.
 * Pages: interactive explainer, "Cartesian Product Router" (p(i,j|x) is
 * taken as p_r(i|x) p_c(j|x); rows and columns are searched separately; the
 * joint score S_ij = log p_r[i] + log p_c[j] is additive in log space and the
 * N-entry score matrix is never formed) and "Expert-Centric Scheduling"
 * (each routing decision carries a weight).
 *
 * Per token t: a = row_logits[t] - LSE(row_logits[t]) and b likewise for the
 * columns (float32, LSE = m + ln sum exp(z - m)); R = the k' best rows of a
 * (value desc, index asc), C = the k' best columns of b; over the k' x k'
 * cells S = fl32(a[R_r] + b[C_c]), e = R_r * Nc + C_c, keep the K best by
 * (S desc, e asc) in rank order.
 *
 * expert_idx [L, K] int32 out (rank order); score [L, K] float32 out (S);
 * gate [L, K] float32 out: g_k = exp(S_k - S_0) / sum_j exp(S_j - S_0).
 * row_logp [L, Nr], col_logp [L, Nc] float32 out (a and b), each may be NULL.
 * row_sel, col_sel: [L, k'] int32 out (R and C in rank order), each may be
 * NULL.
 * ws / ws_bytes: workspace of at least omni_product_topk_workspace(...)
 * bytes, 256-byte aligned (a tie flag and two normalisers per token and, for
 * NULL row_sel / col_sel, the per-axis lists).
 * Requires 1 <= k' <= min(Nr, Nc), 1 <= K <= k'^2, Nr * Nc < 2^31.
 * Kernels cover k' <= 64, K <= 64 and Nr, Nc <= 2048 (else UNSUPPORTED).
 * Given a and b, selection and scores are exact functions of them (the same
 * a and b are written to row_logp / col_logp); gates are float32 (expf,
 * wave-order sum).
 */
size_t omni_product_topk_workspace(int L, int Nr, int Nc, int kprime, int K);
omni_status omni_product_topk(int L, int Nr, int Nc, int kprime, int K,
                              const float* row_logits, const float* col_logits,
                              int32_t* expert_idx, float* score, float* gate,
                              float* row_logp, float* col_logp,
                              int32_t* row_sel, int32_t* col_sel,
                              void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * omni_product_topk_static — omni_product_topk for callers that cannot
 * allocate device memory: code being captured into a HIP graph, tight
 * serving loops, harnesses that forbid allocation.  Arguments, results and
 * errors as omni_product_topk, without the workspace: the call uses a fixed
 * array of OMNI_TOPK_STATIC_SCRATCH_BYTES bytes in device memory that the
 * library holds on every GPU it runs on until the process ends.  It calls
 * no allocator.
 *
 * Limit: the call needs, in bytes,
 *   A(4 L) + A(8 L) + (row_sel ? 0 : A(4 L k')) + (col_sel ? 0 : A(4 L k'))
 * with A(n) = n rounded up to a multiple of 256 (a tie flag and two
 * normalisers per token, then the per-axis lists the caller does not ask
 * for); more than OMNI_TOPK_STATIC_SCRATCH_BYTES returns OMNI_ERR_WORKSPACE
 * before anything is enqueued.  8 MiB holds 16,008 tokens with both lists
 * at k' = 64, and 699,040 tokens when the caller passes row_sel and col_sel.
 * The array is per GPU and shared by every call on that GPU: calls that
 * overlap on one GPU (two streams, two threads) race and give unspecified
 * results.  Nothing in it needs to start at zero (the kernels write every
 * entry they read).  The GPU is the caller's current device.
 */
#define OMNI_TOPK_STATIC_SCRATCH_BYTES (8u << 20)
omni_status omni_product_topk_static(int L, int Nr, int Nc, int kprime, int K,
                                     const float* row_logits, const float* col_logits,
                                     int32_t* expert_idx, float* score, float* gate,
                                     float* row_logp, float* col_logp,
                                     int32_t* row_sel, int32_t* col_sel,
                                     hipStream_t stream);

/*
 * How omni_schedule_tasks forms its groups.
 *   OMNI_GROUP_ACTIVE     the unique active experts in id order, B per group
 *                         (the last group may be short); n_groups =
 *                         ceil(n_active / B).  Interactive explainer,
 *                         "Expert-Centric Scheduling".
 *   OMNI_GROUP_ID_WINDOW  fixed windows of the id space: group g holds the
 *                         experts with ids in [g B, (g + 1) B), every window a
 *                         group (empty ones too); n_groups = ceil(N / B).
 *                         gist.science explainer §2.2 (tasks grouped by
 *                         contiguous ranges of expert ids).
 * Either way the tasks are ordered by (group, token), ties in flatten order.
 */
typedef enum omni_grouping {
  OMNI_GROUP_ACTIVE = 0,
  OMNI_GROUP_ID_WINDOW = 1
} omni_grouping;

/*
 * Schedule produced by omni_schedule_tasks (all members device pointers).
 * G = omni_schedule_max_groups(L, K, N, B, grouping): ceil(min(N, L*K) / B)
 * for OMNI_GROUP_ACTIVE, ceil(N / B) for OMNI_GROUP_ID_WINDOW.
 *   counts        [2]      int32: n_active, n_groups.
 *   active        [min(N, L*K)] int32: the active expert ids ascending
 *                          (entries >= n_active unspecified).
 *   group_offsets [G + 1]  int32: tasks of group g are [off[g], off[g+1]);
 *                          every entry past n_groups equals L*K.
 *   task_token, task_expert [L*K] int32, task_gate [L*K] float32: the tasks
 *                          sorted by (group, token), ties in flatten order.
 *   task_index    [L*K] int32: flat id m = t*K + k of each sorted task, or
 *                          NULL if not wanted.
 *   flat_expert   [L*K] int32, flat_gate [L*K] float32, optional (NULL, or
 *                          both set): the flattened selection the tasks were
 *                          built from, in flatten order m = t*K + k (the
 *                          expert_idx / gate given to omni_schedule_tasks).
 *                          omni_schedule_tasks neither reads nor writes them;
 *                          the token-centric executor reads each token's list
 *                          from them instead of inverting the sorted order.
 *                          They must hold the arrays the schedule was built
 *                          from, else y is unspecified.
 */
typedef struct omni_schedule {
  int32_t* counts;
  int32_t* active;
  int32_t* group_offsets;
  int32_t* task_token;
  int32_t* task_expert;
  float* task_gate;
  int32_t* task_index;
  const int32_t* flat_expert;
  const float* flat_gate;
} omni_schedule;

/* G above: the number of groups the schedule can hold (0 for invalid args). */
int omni_schedule_max_groups(int L, int K, int N, int B, omni_grouping grouping);

/*
 * omni_schedule_tasks — Expert-Centric Scheduling.
 * Pages: interactive explainer, "Expert-Centric Scheduling" (flatten all
 * (token, expert, weight) triples into M = L x K tasks; collect the unique
 * active experts, sort them by id, B per group; order by group id, then
 * token id) and gist.science explainer §2.2 (task collection, grouping and
 * sorting, grouped execution).
 *
 * grouping: OMNI_GROUP_ACTIVE (the pages' B active experts per group) or
 * OMNI_GROUP_ID_WINDOW (fixed id windows), see omni_grouping; anything else
 * is INVALID_ARG.
 * expert_idx [L, K] int32 in (each id in [0, N)); gate [L, K] float32 in.
 * out: host pointer to a descriptor whose members point to device buffers
 * of the sizes listed above.  ws / ws_bytes: workspace of at least
 * omni_schedule_workspace(...) bytes, 256-byte aligned.
 * Requires N >= 1, K >= 1, B >= 1, L*K < 2^31.  Ids outside [0, N) give
 * unspecified results (the ids are produced on the device and not checked).
 * Bit-exact: the result is a pure function of the inputs.
 */
size_t omni_schedule_workspace(int L, int K, int N, int B, omni_grouping grouping);
omni_status omni_schedule_tasks(int L, int K, int N, int B, omni_grouping grouping,
                                const int32_t* expert_idx, const float* gate,
                                const omni_schedule* out,
                                void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * omni_atomic_forward — execution of a schedule.
 * Pages: gist.science explainer §2.1 (atomic expert E_i(x) = sigma(x w_in^T)
 * w_out; all N experts live in two global matrices W, V in R^{N x d}; per
 * token the selected rows are assembled into one block: Dynamic Expert
 * Assembly) and interactive explainer "Expert-Centric Scheduling" (each
 * group's parameters are loaded once and reused for all tokens assigned to
 * it; traffic 2d*|E_active| instead of 2d*L*K).  sigma = SiLU.
 *
 *   y[t, :] = sum over scheduled tasks (t, e, g): g * silu(x[t,:] . W[e,:]) * V[e,:]
 *
 * Three execution forms, selected by `mode`:
 *   OMNI_EXEC_EXPERT_CENTRIC: two kernels; the first walks the tasks in the
 *     schedule's (group, token) order and computes c = g * silu(x_t . W[e])
 *     per task, the second gathers y_t = sum_k c_tk V[e_tk] per token, so y
 *     is written once, without atomics.
 *   OMNI_EXEC_TOKEN_CENTRIC: the per-token task lists are the schedule's
 *     flat_expert / flat_gate when present, else the schedule's sorted order
 *     inverted through task_index (one more kernel); then one wave per
 *     token assembles its experts: x_t stays in registers, the token's W
 *     rows give the K coefficients, its V rows are summed into y_t.  Below
 *     4096 tokens each token gets several waves: its tasks are split over
 *     them for the coefficients, the columns of y_t for the sum.
 *   Both forms hold a whole row per wave in registers where they can (d a
 *   power of two; token-centric: rows of at most 4 KiB; expert-centric:
 *   d <= 4096).  Every other width d = 64 m (m >= 1, d <= 16384) runs a pair
 *   of chunked kernels: the coefficients with the rows taken in chunks of
 *   64 * 2^j elements (2^j the largest power of two dividing m, at most 16
 *   bytes per lane), then one wave per (token, chunk of columns) summing the
 *   token's tasks in k order.
 *   OMNI_EXEC_GROUPED (bf16 only, K <= 64, d = 64 * 2^p <= 2048, else
 *     UNSUPPORTED): the pages' grouped execution on the matrix cores.  From
 *     the sorted schedule's task_expert the tasks of every expert are
 *     counted; the experts with at least tau tasks form
 *     the hot set H (tau = max(2, ceil(L / 64)), doubled until at most 512
 *     experts reach it; H in id order).  Each tile of 64 consecutive tokens
 *     then computes S = x_tile W_H^T and y_tile = C V_H with two bf16 MFMA
 *     products, C[t, h] = g * silu(S[t, h]) rounded to bf16 on the tile's
 *     hot tasks and 0 elsewhere, so every hot expert's W and V rows are read
 *     once per tile and reused by all its tokens; the tile's other (cold)
 *     tasks run token by token in float32 as in the token-centric form, and
 *     the hot product is added to the rows they wrote.  Meant for skewed
 *     routing, where a few hundred experts take most tasks (measured on
 *     MI355X with Zipf(1.1) routing, L = 16384, N = 2^18: 0.334 ms against
 *     0.352 ms for the token-centric form).  With no hot expert it computes
 *     every task that way, slower than the other forms.  Agrees with the
 *     other forms within the bf16 rounding of the hot coefficients;
 *     deterministic.
 *   OMNI_EXEC_AUTO: the form omni_atomic_forward_mode() names for the shape
 *     (the one that measured faster on MI355X).
 * The token-centric form with flat_expert / flat_gate set reads no other
 * member of sched (those must still be non-null): such a call may run while
 * the omni_schedule_tasks call that fills the rest is still running on
 * another stream.  The expert-centric and grouped forms read the sorted
 * schedule (the grouped form its task_expert), so they must follow it on the
 * stream.
 * The expert- and token-centric forms evaluate every coefficient and every y
 * element with the same operations in the same order (k = 0..K-1), so they
 * give bit-identical y; the grouped form agrees with them within the bf16
 * rounding of its hot coefficients.
 *
 * x [L, d], w [N, d], v [N, d] of dt; sched: a schedule produced by
 * omni_schedule_tasks for the same L, K, N, B, with task_index present;
 * y [L, d] float32 out, 16-byte aligned.  accumulate = 0: y is overwritten
 * with the routed output; accumulate != 0: the routed output is added to y as
 * it stands (e.g. onto the output of a shared dense branch).
 * ws / ws_bytes: at least omni_atomic_forward_workspace(..., mode) bytes for
 * the mode of the call, 256-byte aligned (8 bytes per task: a coefficient and
 * an expert id, or the per-token lists; the grouped form adds a task count
 * per expert id, 4 N bytes, 32 KiB of level lists and 2 KiB per column of d
 * for the gathered W_H and V_H^T).  Requires d = 64 m with 64 <= d <= 16384 (else UNSUPPORTED);
 * 16-byte aligned x, w, v.  Deterministic.
 */
typedef enum omni_exec_mode {
  OMNI_EXEC_AUTO = 0,
  OMNI_EXEC_EXPERT_CENTRIC = 1,
  OMNI_EXEC_TOKEN_CENTRIC = 2,
  OMNI_EXEC_GROUPED = 3
} omni_exec_mode;

/* The form OMNI_EXEC_AUTO runs for this shape (1, 2 or 3); 0 for invalid args. */
int omni_atomic_forward_mode(omni_dtype dt, int L, int d, int N, int K, int B);
/* Workspace of the call with this mode (AUTO: the form AUTO runs); 0 for
   invalid arguments. */
size_t omni_atomic_forward_workspace(omni_dtype dt, int L, int d, int N, int K, int B,
                                     omni_exec_mode mode);
omni_status omni_atomic_forward(omni_dtype dt, int L, int d, int N, int K, int B,
                                const void* x, const void* w, const void* v,
                                const omni_schedule* sched, float* y, int accumulate,
                                omni_exec_mode mode, void* ws, size_t ws_bytes,
                                hipStream_t stream);

/*
 * omni_atomic_forward_glu — variant: SwiGLU-gated atomic experts.  The
 * interactive explainer ("Atomic Expert") names SwiGLU as the expert's
 * activation while the expert has a single input vector; this variant gives
 * every expert a third vector, row e of u, and computes
 *
 *   y_t = sum_k g_tk * silu(x_t . W[e_tk]) * (x_t . U[e_tk]) * V[e_tk]
 *
 * (3d parameters per expert instead of 2d).  Arguments as omni_atomic_forward
 * plus u [N, d] of dt; the workspace is omni_atomic_forward_workspace(...,
 * OMNI_EXEC_TOKEN_CENTRIC).
 * Token-centric form only (the chunked kernels for the widths whose rows do
 * not fit in registers): requires d = 64 m with 64 <= d <= 16384, else
 * UNSUPPORTED.  Deterministic.
 */
omni_status omni_atomic_forward_glu(omni_dtype dt, int L, int d, int N, int K, int B,
                                    const void* x, const void* w, const void* u, const void* v,
                                    const omni_schedule* sched, float* y, int accumulate,
                                    void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * omni_flat_router_topk — variant: the flat router the Cartesian Product
 * Router replaces (gist.science explainer §2.2: a standard router scores all
 * N experts with a d x N projection; interactive explainer, ablation table).
 *
 *   z = x Wf^T (+ bias);  log p = z - LSE(z) over all N experts;
 *   top-K by (log p desc, e asc), values compared as float32 numbers;
 *   gate = softmax over the K selected log p.
 *
 * x [L, d] of dt; wf [N, d] of dt (row e: expert e's router weights); bias
 * [N] float32 or NULL.  Out: expert_idx [L, K] int32, score [L, K] float32
 * (log p of the selected experts), gate [L, K] float32, in rank order;
 * logp [L, N] float32 (NULL if not wanted).  ws / ws_bytes: at least
 * omni_flat_router_workspace(dt, L, N) bytes (the L x N logits), 256-byte
 * aligned.  Requires 1 <= K <= min(64, N); d a multiple of 8 (bf16) or 4
 * (float32).  Bit-exact selection for given log p: ties go to the lower id.
 */
size_t omni_flat_router_workspace(omni_dtype dt, int L, int N);
omni_status omni_flat_router_topk(omni_dtype dt, int L, int d, int N, int K, const void* x,
                                  const void* wf, const float* bias, int32_t* expert_idx,
                                  float* score, float* gate, float* logp, void* ws,
                                  size_t ws_bytes, hipStream_t stream);

/*
 * omni_routed_backward — gradients of the routed layer for a given upstream
 * gradient dy = dL/dy.  The pages train models with this layer but print no
 * backward pass; the gradients follow from the forward above by the chain rule
 * (gist.science explainer §2.1-§2.2; interactive explainer "Cartesian Product
 * Router", "Expert-Centric Scheduling").  The expert selection is piecewise
 * constant and passes no gradient; sigma = SiLU, gate = softmax of the K
 * selected scores, as in the forward.
 *
 *   per task (t, e = i * Nc + j, gate g): u = dy_t . V[e], h = x_t . W[e]
 *     dV[e] += g silu(h) dy_t      dW[e] += g silu'(h) u x_t
 *     dx_t  += g silu'(h) u W[e]   dgate = silu(h) u
 *   dS_k = g_k (dgate_k - sum_j g_j dgate_j);  dz_r[t, i_k] += dS_k, dz_c[t, j_k] += dS_k
 *   (the log-softmax backward adds nothing more because sum_k dS_k = 0)
 *   dx += dz_r Wr + dz_c Wc;  dWr = dz_r^T x;  dWc = dz_c^T x;  d bias = column sums
 *
 * Inputs: x [L, d], wr_t [Nr, d], wc_t [Nc, d], w [N, d], v [N, d] of dt
 * (N = Nr * Nc); expert_idx, gate [L, K]: the forward's omni_product_topk
 * output; dy [L, d] float32.
 * Outputs (float32, overwritten): dx [L, d]; dwr_t [Nr, d]; dwc_t [Nc, d];
 * drow_bias [Nr], dcol_bias [Nc] (either may be null); counts[0] = number of
 * active experts n (counts[1] = n as well); active [min(N, L*K)] ascending
 * active expert ids; dw, dv [min(N, L*K), d]: row r is the gradient of
 * W[active[r]] / V[active[r]] for r < n (rows from n on are left untouched);
 * dgate [L, K] (may be null).
 * ws / ws_bytes: at least omni_routed_backward_workspace(...) bytes, 256-byte
 * aligned.  Requires K <= 64, d = 64 * 2^p with rows of at most 4 KiB
 * (bf16 d <= 2048, float32 d <= 1024), else UNSUPPORTED; 16-byte aligned
 * row arrays.  Deterministic: every sum runs in a fixed order.
 */
size_t omni_routed_backward_workspace(omni_dtype dt, int L, int d, int Nr, int Nc, int K);
omni_status omni_routed_backward(omni_dtype dt, int L, int d, int Nr, int Nc, int K,
                                 const void* x, const void* wr_t, const void* wc_t,
                                 const void* w, const void* v, const int32_t* expert_idx,
                                 const float* gate, const float* dy, float* dx, float* dwr_t,
                                 float* dwc_t, float* drow_bias, float* dcol_bias,
                                 int32_t* counts, int32_t* active, float* dw, float* dv,
                                 float* dgate, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * omni_shared_mlp — the shared dense MLP branch of the OmniMoE layer: the
 * dense branch every token passes through, next to the routed atomic experts
 * (gist.science explainer §2 and §2.1 "Shared Dense MLP"; interactive
 * explainer "Atomic Expert").  The pages print no formula for it; this is the
 * gated SwiGLU form (the activation the pages name):
 *
 *   y_t (+)= Wd (silu(Wg x_t) * (Wu x_t))
 *
 * x [L, d], w_gate [d_ff, d], w_up [d_ff, d] (row j: hidden unit j's input
 * weights), w_down [d, d_ff] (row c: output feature c's weights), all of dt;
 * y [L, d] float32.  accumulate = 0 overwrites y; accumulate != 0 adds the
 * branch onto y as it stands, which is the layer's hybrid sum when y holds
 * the routed output of omni_atomic_forward (or call omni_atomic_forward with
 * its accumulate flag after this one).  The bf16 path runs both products on
 * MFMA with fp32 accumulation and keeps the hidden activation in bf16; the
 * float32 path computes it in float32.
 * ws / ws_bytes: at least omni_shared_mlp_workspace(dt, L, d, d_ff) bytes,
 * 256-byte aligned (the hidden activation, L * d_ff elements of dt, and for
 * few tokens the split-K partials of the down product).
 * Requires d and d_ff multiples of 8 (bf16) or 4 (float32), else
 * UNSUPPORTED; 16-byte aligned arrays.  Deterministic.
 */
size_t omni_shared_mlp_workspace(omni_dtype dt, int L, int d, int d_ff);
omni_status omni_shared_mlp(omni_dtype dt, int L, int d, int d_ff, const void* x,
                            const void* w_gate, const void* w_up, const void* w_down, float* y,
                            int accumulate, void* ws, size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* OMNI_H */
