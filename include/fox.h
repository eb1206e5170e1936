/*
 * fox.h — C ABI of the Forgetting Attention library (libfox.so, gfx950 / MI355X).
 *
 * Forgetting Attention is causal softmax attention whose logits carry the bias
 * D_ij = c_i - c_j, with c the per-head prefix sum of log forget gates
 * (arXiv 2503.02130, "Forgetting Transformer: Softmax Attention with a Forget Gate";
 * paper-graph-ui summary, section 3.4, parts "The Mathematical Form of Forgetting
 * Attention" and "Hardware-Aware Implementation (Modified FlashAttention)").
 *
 * Conventions shared by every entry point
 *   - Every data pointer is a DEVICE pointer owned by the caller. The library never
 *     allocates, frees or keeps a pointer after the call returns; the caller keeps the
 *     buffers alive until the queued work on `stream` has finished.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream). Every call only
 *     enqueues kernels on it: no host synchronisation, no host<->device copies.
 *   - Layouts are dense and row-major, last index fastest:
 *       q, k, v, o, dO, dq, dk, dv : [B, H, L, D]
 *       log_f, c, lse, dlog_f       : [B, H, L]
 *       x (gate input)              : [B, L, d_model];  w_f: [H, d_model];  b_f: [H]
 *     Positions are 0-indexed; c is the inclusive prefix sum c_i = sum_{l<=i} log f_l.
 *   - Every pointer must be 16-byte aligned. D must be 64 or 128; 1 <= L <= 2^23; B, H >= 1.
 *   - Arguments are validated on the host before anything is launched. A bad argument
 *     returns FOX_E_INVALID (or FOX_E_UNSUPPORTED for a well-formed request this library does
 *     not implement) and enqueues nothing; fox_last_error() then describes it. A failed
 *     launch returns FOX_E_LAUNCH. No C++ exception or abort crosses this boundary.
 *   - Preconditions not checked on the device: log f must be finite (the pages' log 0 = -inf
 *     would make c_i - c_j undefined); NaN inputs propagate to NaN outputs. A hard reset is a
 *     large finite negative log f: -200 already cuts every earlier weight exactly (exp
 *     underflows in fp32), and deeper values only cost precision, in two ways. (1) |c| grows:
 *     fp32 c is spaced 2^-11 at |c| ~ 4e3 and 2^-7 at 1e5, and that rounding shows in the
 *     gradients once |c| passes about 1e4 (many resets, or strong decay over a long context);
 *     fp64 c (FOX_C_F64) removes it. (2) Within a tile the kernels hold c differences in fp32
 *     against one reference, so a fall of c by F inside one tile leaves errors of about
 *     2^-24 F (log2 units) in the weights on one side of it, whatever the type of c: keep a
 *     single reset within about -2000 (at -1e4 d log f can reach 2e-2 on bf16 inputs).
 *   - Size queries (the *_bytes calls) return 0 for sizes outside these limits; every size
 *     check is made without an intermediate product that could overflow.
 *   - Calls are reentrant: the library holds no mutable global state apart from the
 *     thread-local error message and the per-device scratch array of fox_attn_bwd_noalloc.
 */
#ifndef FOX_H
#define FOX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fox_status {
  FOX_OK = 0,
  FOX_E_INVALID = 1,      /* bad pointer, size, alignment, dtype combination or workspace */
  FOX_E_UNSUPPORTED = 2,  /* valid request outside what is implemented (e.g. non-causal) */
  FOX_E_LAUNCH = 3        /* the HIP runtime rejected a kernel launch */
} fox_status;

typedef enum fox_dtype { FOX_F32 = 0, FOX_BF16 = 1 } fox_dtype;

/* Flags of fox_attn_fwd / fox_attn_bwd and the backward steps. FOX_CAUSAL is required: the
 * method is defined for causal sequence modelling only (paperlayer.ai summary, section 6
 * "CONCLUSION", limitations: the non-causal case is future work).
 * FOX_C_F64: c holds fp64 values (from fox_logf_cumsum_f64) instead of fp32. The kernels then
 * form every c_i - c_j in fp64 and round the difference once, so it keeps full precision however
 * far c has fallen; with fp32 c each value carries a rounding of up to half the fp32 spacing at
 * |c| (2^-9 at |c| ~ 2^14, 2^-7 at |c| ~ 2^17), which hard resets (log f ~ -1e4) reach within a
 * few positions. Not taken together with a skip plan (FOX_E_UNSUPPORTED). */
enum { FOX_CAUSAL = 1u, FOX_C_F64 = 2u, FOX_QK_RMSNORM = 4u, FOX_K_RMSNORM = 8u };

/* Cumulative log decay (paper-graph-ui summary, "Hardware-Aware Implementation": c is the
 * cumulative sum of log f, computed once per head before attention and kept in HBM).
 *   log_f : [BH, L] fp32 input;  c : [BH, L] fp32 output, c[r, i] = sum_{l<=i} log_f[r, l].
 * Accumulates in fp64 and rounds once to fp32. c may not alias log_f. */
fox_status fox_logf_cumsum(const float* log_f, float* c, int64_t BH, int64_t L, void* stream);
/* The same prefix sum kept in fp64 (c : [BH, L] fp64 output; the accumulation is fp64 either
 * way), for the attention calls with FOX_C_F64. */
fox_status fox_logf_cumsum_f64(const float* log_f, double* c, int64_t BH, int64_t L, void* stream);

/* Scalar per-head forget gate in log space (paper-graph-ui summary, "Forget Gate Computation";
 * Pro block Step 4): log_f[b, h, t] = log sigmoid(sum_d x[b, t, d] * w_f[h, d] + b_f[h]).
 *   x   : [B, L, d_model], dtype x_dt (FOX_BF16 or FOX_F32)
 *   w_f : [H, d_model] fp32;  b_f : [H] fp32;  log_f : [B, H, L] fp32 output.
 * fp32 accumulation; log sigmoid is evaluated stably (never as log of a rounded sigmoid).
 * d_model must be a multiple of 8 and at most 8192; H at most 64. */
fox_status fox_gate_logf(const void* x, fox_dtype x_dt, const float* w_f, const float* b_f,
                         float* log_f, int64_t B, int64_t L, int64_t d_model, int64_t H,
                         void* stream);

/* QK-norm (Pro block Steps 1-2: RMSNorm over the head dimension of each query and key):
 *   y[r, :] = x[r, :] / sqrt(mean_d x[r, d]^2 + eps) * (weight ? weight[:] : 1)
 *   x, y : [rows, D] in dtype dt (same dtype in and out; y may equal x for in-place);
 *   weight : [D] fp32 or NULL for unit weights. fp32 arithmetic, one rounding on output.
 * Call once for q and once for k ([B*H*L, D] each). */
fox_status fox_qk_rmsnorm(const void* x, void* y, fox_dtype dt, int64_t rows, int64_t D,
                          float eps, const float* weight, void* stream);

/* Backward of the gate (paper-graph-ui summary, "Forget Gate Computation"; Pro block Step 4),
 * for the loss whose gradient with respect to log_f is dlog_f ([B, H, L] fp32):
 *   dz[b, h, t] = dlog_f[b, h, t] * sigmoid(-z[b, h, t])
 *   dx[b, t, :] = sum_h dz[b, h, t] w_f[h, :]              [B, L, d_model] fp32 output
 *   dw_f[h, :]  = sum_{b,t} dz[b, h, t] x[b, t, :]         [H, d_model] fp32 output
 *   db_f[h]     = sum_{b,t} dz[b, h, t]                    [H] fp32 output
 * log_f: the forward's output [B, H, L] fp32 (fox_gate_logf of the same x, w_f, b_f), or NULL.
 * With it, sigmoid(-z) = 1 - f = -expm1(log f) comes from log_f and x is read once (for dw_f);
 * with NULL, z is recomputed from x, w_f and b_f (a second pass over x).
 * x, w_f, b_f, shapes and limits as for fox_gate_logf. workspace: device memory of at least
 * fox_gate_logf_bwd_workspace_bytes(B, L, d_model, H) bytes, 256-byte aligned, contents ignored.
 * fp32 arithmetic; sums over tokens run in a fixed order (deterministic, no atomics). */
size_t fox_gate_logf_bwd_workspace_bytes(int64_t B, int64_t L, int64_t d_model, int64_t H);
fox_status fox_gate_logf_bwd(const void* x, fox_dtype x_dt, const float* w_f, const float* b_f,
                             const float* dlog_f, const float* log_f, float* dx, float* dw_f,
                             float* db_f, void* workspace, size_t workspace_bytes, int64_t B,
                             int64_t L, int64_t d_model, int64_t H, void* stream);

/* Backward of the QK-norm (Pro block Steps 1-2), y = x / sqrt(mean x^2 + eps) * weight:
 *   x  : [rows, D] in dtype dt (the norm's input);  dy : [rows, D] fp32 (gradient of y)
 *   dx : [rows, D] fp32 output, dx = r (g - xh mean(g xh)) with r = 1 / sqrt(mean x^2 + eps),
 *        xh = x r, g = dy * weight (weight NULL: unit weights)
 *   dweight : [D] fp32 output sum_rows dy * xh, or NULL if not wanted (needs weight != NULL);
 *        then workspace must hold fox_qk_rmsnorm_bwd_workspace_bytes(rows, D) bytes, 256-byte
 *        aligned (it may be NULL when dweight is NULL). Deterministic (fixed-order sums). */
size_t fox_qk_rmsnorm_bwd_workspace_bytes(int64_t rows, int64_t D);
fox_status fox_qk_rmsnorm_bwd(const void* x, fox_dtype dt, const float* dy, float* dx,
                              const float* weight, float* dweight, void* workspace,
                              size_t workspace_bytes, int64_t rows, int64_t D, float eps,
                              void* stream);

/* Exact skipping of fully decayed tiles. The forget gate makes a key's weight decay with its
 * distance from the query; the pages name pruning of computation by the gate values as future
 * work (paperlayer.ai summary, section 6 "CONCLUSION", limitations and future work;
 * paper-graph-ui summary, "Follow-Up Research", KV-cache eviction). A plan records, for the
 * given q, k, c and scale, the tiles of the bf16 attention kernels in which every weight is
 * provably below 2^-160 of the row's largest, so that the kernels' exp2 already returns exactly
 * zero there; with the plan the kernels do not visit those tiles. For finite inputs the
 * results are bit-identical to those without a plan.
 * The bound: for a query i and an earlier key j,
 *   scale q_i.k_j + c_i - c_j - (scale q_i.k_i) <= scale |q_i| (|k_j| + |k_i|) - (c_j - c_i),
 * evaluated per tile with the largest row norms of q and k in each 64-row group, the smallest c
 * of the key tile and the largest c of the query tile (with gates in (0, 1), c at the key tile's
 * last and the query tile's first position), plus a slack for the fp32 rounding of c. The
 * extremes are taken per 64-row group, so the plan is exact for any finite c, rising or not.
 * The forward's running maximum and the backward's LSE are never below the diagonal logit
 * scale q_i.k_i.
 *   fox_attn_skip_plan_bytes : bytes of device memory a plan takes for these sizes.
 *   fox_attn_skip_plan       : fills `plan` (256-byte aligned, at least that many bytes) from
 *                              q, k (bf16, [B, H, L, D]), c and scale. Reads q and k once.
 *                              Supports B*H <= 65535 (FOX_E_UNSUPPORTED beyond).
 * Plan layout (arrays in this order, each starting at the next 256-byte boundary, BH = B * H):
 *   int32 q_skip[BH][ceil(L / 256)]   key tiles of 64 keys, counted from key 0, that the
 *                                     256-query tile skips (the forward and dq steps);
 *   int32 kv_tiles[BH][ceil(L / 128)] 64-query tiles, counted from the block's first key, that
 *                                     the 128-key block walks (the dk/dv step);
 *   fp32 qn[BH][ceil(L / 64)], kn[...] largest row norm of q and k in each 64-row group;
 *   fp32 cmin[BH][ceil(L / 64)], cmax[...] smallest and largest c in each 64-row group;
 *   int32 q_order[BH * ceil(L / 256)]  launch order of the query tiles (entry bh * ceil(L / 256)
 *                                     + tile), most work first; entries of equal work may come
 *                                     in a different order on each call (results do not depend
 *                                     on it);
 *   int32 kv_order[BH * ceil(L / 128)] the same for the key blocks.
 * Pass the plan as skip_plan to fox_attn_fwd and the backward calls made with the same q, k,
 * c, sizes and scale; a plan for other inputs gives wrong results. skip_plan = NULL visits
 * every tile. */
size_t fox_attn_skip_plan_bytes(int64_t B, int64_t H, int64_t L, int64_t D);
fox_status fox_attn_skip_plan(const void* q, const void* k, fox_dtype in_dt, const float* c,
                              void* plan, size_t plan_bytes, int64_t B, int64_t H, int64_t L,
                              int64_t D, float scale, void* stream);

/* The Pro block's token shift and output normalisation + gate (paper-graph-ui summary, section
 * 3.4, "The Pro Block Architecture", Steps 2-3, 5 and 7). The page's equations are missing;
 * these entry points take the plainest reading of its words:
 *   shift gate   alpha[b, h, t] = sigmoid(x[b, t, :] . w[h, :])  (one learned vector per head,
 *                no bias), in (0, 1);
 *   token shift  y_t = alpha_t x_{t-1} + (1 - alpha_t) x_t  (x_{-1} = 0; alpha weights the
 *                carried-forward previous candidate), then RMSNorm for keys (normalize = 1),
 *                none for values;
 *   output       y = RMSNorm(o) [* weight] * sigmoid(g)  (g = W_g x, the per-dimension output
 *                gate pre-activation), before the output projection.
 * The projections W_k x, W_v x, W_g x and W_o are plain GEMMs outside this library.
 *
 * fox_shift_gate: x [B, L, d_model] (x_dt FOX_BF16 or FOX_F32), w [H, d_model] fp32 ->
 *   alpha [B, H, L] fp32; limits as for fox_gate_logf.
 * fox_shift_gate_bwd: dalpha [B, H, L] fp32 -> dx [B, L, d_model], dw [H, d_model] (fp32);
 *   workspace of fox_gate_logf_bwd_workspace_bytes(B, L, d_model, H) bytes, 256-byte aligned.
 *   Deterministic (fixed-order sums).
 * fox_kv_shift: x, y [BH, L, D] in dt (FOX_BF16 or FOX_F32; y may not alias x); alpha [BH, L]
 *   fp32; with normalize != 0 the shifted rows are RMS-normalised with eps and weight ([D] fp32,
 *   or NULL for unit weights). fp32 arithmetic, one rounding on output.
 * fox_kv_shift_bwd: dy [BH, L, D] fp32, the gradient of fox_kv_shift's output -> dx [BH, L, D]
 *   fp32 (may not alias dy) and dalpha [BH, L] fp32, with the same x, alpha, normalize, eps
 *   and weight (the weight is a constant here: no weight gradient).
 * fox_out_norm_gate: o [rows, D] (o_dt), g [rows, D] (g_dt), weight [D] fp32 or NULL -> y
 *   [rows, D] in g_dt.
 * fox_out_norm_gate_bwd: dy [rows, D] fp32 -> d_o and dg [rows, D] fp32 (no weight gradient). */
fox_status fox_shift_gate(const void* x, fox_dtype x_dt, const float* w, float* alpha, int64_t B,
                          int64_t L, int64_t d_model, int64_t H, void* stream);
fox_status fox_shift_gate_bwd(const void* x, fox_dtype x_dt, const float* w, const float* dalpha,
                              float* dx, float* dw, void* workspace, size_t workspace_bytes,
                              int64_t B, int64_t L, int64_t d_model, int64_t H, void* stream);
fox_status fox_kv_shift(const void* x, fox_dtype dt, const float* alpha, void* y, int normalize,
                        float eps, const float* weight, int64_t BH, int64_t L, int64_t D,
                        void* stream);
fox_status fox_kv_shift_bwd(const void* x, fox_dtype dt, const float* alpha, const float* dy,
                            float* dx, float* dalpha, int normalize, float eps,
                            const float* weight, int64_t BH, int64_t L, int64_t D, void* stream);
fox_status fox_out_norm_gate(const void* o, fox_dtype o_dt, const void* g, fox_dtype g_dt,
                             const float* weight, float eps, void* y, int64_t rows, int64_t D,
                             void* stream);
fox_status fox_out_norm_gate_bwd(const void* o, fox_dtype o_dt, const void* g, fox_dtype g_dt,
                                 const float* weight, float eps, const float* dy, float* d_o,
                                 float* dg, int64_t rows, int64_t D, void* stream);

/* Forward (paper-graph-ui summary, "Hardware-Aware Implementation", the forward pass;
 * paperlayer.ai summary, section E):
 *   O[i]   = sum_{j<=i} softmax_j(scale * q_i . k_j + c_i - c_j) v_j
 *   lse[i] = log sum_{j<=i} exp(scale * q_i . k_j + c_i - c_j)     (natural log, fp32)
 * The scale multiplies q.k only; the bias is added unscaled. Only differences of c matter,
 * so any per-(b,h) constant offset in c leaves O and lse unchanged.
 *   q, k, v : in_dt (FOX_BF16, or FOX_F32 for the full-fp32 path)
 *   c       : fp32, or fp64 with FOX_C_F64 in flags
 *   o       : o_dt (FOX_BF16 or FOX_F32; must be FOX_F32 when in_dt is FOX_F32)
 *   lse     : fp32, may be NULL if not wanted.
 * bf16 inputs run on bf16 MFMA with fp32 accumulation and an fp32 online softmax; fp32
 * inputs run fully in fp32. flags must contain FOX_CAUSAL. skip_plan: NULL, or a plan from
 * fox_attn_skip_plan for these q, k, c and scale (bf16 inputs only). */
fox_status fox_attn_fwd(const void* q, const void* k, const void* v, fox_dtype in_dt,
                        const void* c, void* o, fox_dtype o_dt, float* lse, int64_t B,
                        int64_t H, int64_t L, int64_t D, float scale, uint32_t flags,
                        const void* skip_plan, void* stream);

/* The forward with the Pro block's fusions (paper-graph-ui summary, section 3.4, "The Pro Block
 * Architecture": Step 1, QK-norm; Steps 2-3, the token shift of keys and values; Steps 5 and 7,
 * output norm and output gate), through one options struct. Everything else as fox_attn_fwd.
 *   flags: FOX_CAUSAL (required), FOX_C_F64, FOX_QK_RMSNORM and FOX_K_RMSNORM.
 *          FOX_QK_RMSNORM: each query row is normalised as it is loaded,
 *          q / sqrt(mean_d q^2 + q_norm_eps) [* q_norm_weight], in fp32 with one rounding to bf16,
 *          as fox_qk_rmsnorm would. FOX_K_RMSNORM: each key row (after its shift, if any) is
 *          normalised the same way with k_norm_eps [* k_norm_weight] as its tile is loaded.
 *   k_shift_alpha, v_shift_alpha: NULL, or the shift gate alpha ([B, H, L] fp32, from
 *          fox_shift_gate); k (v) then holds the raw candidates, and row t of the keys (values)
 *          the attention uses is alpha_t x_{t-1} + (1 - alpha_t) x_t, with x_{-1} = 0.
 *          With FOX_K_RMSNORM and k_shift_alpha, the keys are exactly the rows fox_kv_shift
 *          (normalize = 1, the same eps and weight) writes, and v_shift_alpha gives the rows of
 *          fox_kv_shift (normalize = 0): O, lse and y are bit-identical to that pass followed by
 *          this call without them. Every workgroup whose queries see a key tile repeats the shift
 *          and norm of that tile (its loads go through registers instead of direct copies), so
 *          this serves callers that must not write the shifted keys and values; the separate
 *          pass is faster.
 *   gate:  NULL, or the output gate's pre-activation g ([B, H, L, D], gate_dt FOX_BF16 or
 *          FOX_F32). Then y ([B, H, L, D], gate_dt) = RMSNorm(O) [* out_norm_weight] *
 *          sigmoid(g), RMSNorm over D with out_norm_eps, formed from the fp32 O in registers.
 *   o:     may be NULL when gate is given (inference, O not wanted); lse may be NULL.
 * bf16 inputs only for any of these (FOX_E_UNSUPPORTED otherwise); a skip plan is not taken with
 * FOX_QK_RMSNORM, FOX_K_RMSNORM or a shift (a plan is built from the q and k the attention
 * sees). The shift gates and k_norm_weight must be 4-byte aligned. */
typedef struct fox_fwd_opts {
  float scale;
  uint32_t flags;
  float q_norm_eps;
  const float* q_norm_weight;
  const void* gate;
  fox_dtype gate_dt;
  const float* out_norm_weight;
  float out_norm_eps;
  void* y;
  const void* skip_plan;
  const float* k_shift_alpha;
  const float* v_shift_alpha;
  float k_norm_eps;
  const float* k_norm_weight;
} fox_fwd_opts;
fox_status fox_attn_fwd_ex(const void* q, const void* k, const void* v, fox_dtype in_dt,
                           const void* c, void* o, fox_dtype o_dt, float* lse, int64_t B,
                           int64_t H, int64_t L, int64_t D, const fox_fwd_opts* opts,
                           void* stream);

/* The forward with the prefix sum fused in (paper-graph-ui summary, section 7 "Implications and
 * Future Directions", follow-up work: fuse the computation of c into the attention kernel). It
 * takes log f ([B, H, L] fp32) instead of c, computes the prefix sums itself in fp64, and writes
 * c_out ([B, H, L]; fp32, or fp64 with FOX_C_F64) for the backward: within one fp32 ulp of
 * fox_logf_cumsum (fox_logf_cumsum_f64 to fp64 rounding). O and lse as fox_attn_fwd; every bias
 * c_i - c_j is formed as an fp64 difference, so the forward does not carry the rounding of an
 * fp32 c. bf16 inputs run one fused kernel; fp32 inputs run the scan and then the fp32 forward.
 * No skip plan (a plan is built from c). c_out may not alias log_f. */
fox_status fox_attn_fwd_logf(const void* q, const void* k, const void* v, fox_dtype in_dt,
                             const float* log_f, void* c_out, void* o, fox_dtype o_dt, float* lse,
                             int64_t B, int64_t H, int64_t L, int64_t D, float scale,
                             uint32_t flags, void* stream);

/* Bytes of device workspace fox_attn_bwd needs for these sizes (caller-allocated). */
size_t fox_attn_bwd_workspace_bytes(int64_t B, int64_t H, int64_t L, int64_t D);

/* Backward of the loss sum(dO * O) (paper-graph-ui summary, "Hardware-Aware Implementation",
 * the backward pass; paperlayer.ai summary, section E): recomputes P from lse with the same
 * bias (c fp32, or fp64 with FOX_C_F64, as given to the forward), and returns
 *   dq, dk, dv : [B, H, L, D] fp32
 *   dlog_f     : [B, H, L] fp32, the reverse cumulative sum of dc = dc^q + dc^k with
 *                dc^q_i = sum_j dS_ij and dc^k_j = -sum_i dS_ij.
 * Inputs: q, k, v, dO in in_dt (FOX_BF16 on the matrix cores; FOX_F32 for the full-fp32 path
 * on the vector ALU, which takes no skip plan and B*H <= 65535); c and lse as given to / returned by
 * fox_attn_fwd; o is the forward output in fp32 (the row term Delta_i = dO_i . O_i is formed
 * from the fp32 output). workspace: device memory of at least
 * fox_attn_bwd_workspace_bytes(B, H, L, D) bytes, 256-byte aligned, contents ignored on
 * entry and clobbered. Deterministic: identical inputs give bit-identical outputs. skip_plan:
 * NULL, or the plan of these q, k, c and scale (see fox_attn_skip_plan). */
fox_status fox_attn_bwd(const void* q, const void* k, const void* v, fox_dtype in_dt,
                        const void* c, const float* o, const float* lse, const void* dO,
                        float* dq, float* dk, float* dv, float* dlog_f, void* workspace,
                        size_t workspace_bytes, int64_t B, int64_t H, int64_t L, int64_t D,
                        float scale, uint32_t flags, const void* skip_plan, void* stream);

/* fox_attn_bwd for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid an allocator). Same arguments, results and errors
 * as fox_attn_bwd, minus the workspace: the row term and the dc partial sums live in a static
 * device array of the library (32 MiB, fox_attn_bwd_noalloc_max_bytes()) that every GPU the
 * library runs on holds from the library's load until the process ends. Sizes whose workspace
 * (fox_attn_bwd_workspace_bytes) exceeds it, that is B*H*L above 2^21, return FOX_E_INVALID.
 * Calls no allocator. Every call on one GPU shares that GPU's array: calls that overlap in time
 * on one GPU (on different streams, or from different threads) race and give wrong results;
 * calls in order on one stream are safe. The array's contents are not read on entry. */
size_t fox_attn_bwd_noalloc_max_bytes(void);
fox_status fox_attn_bwd_noalloc(const void* q, const void* k, const void* v, fox_dtype in_dt,
                                const void* c, const float* o, const float* lse, const void* dO,
                                float* dq, float* dk, float* dv, float* dlog_f, int64_t B,
                                int64_t H, int64_t L, int64_t D, float scale, uint32_t flags,
                                const void* skip_plan, void* stream);

/* The four steps of fox_attn_bwd as separate calls, for callers that schedule them
 * themselves. Running them in this order with the same arguments gives exactly fox_attn_bwd's
 * results. fox_attn_bwd itself runs step 1 inside step 2 (step 2 with delta = NULL and o
 * given), which gives the same bits with one launch and one read of dO fewer.
 *
 * Step 1, Delta_i = sum_d dO[i, d] * O[i, d] (the FlashAttention row term that dS needs):
 *   dO : [rows, D] in dO_dt (FOX_BF16 or FOX_F32);  o : [rows, D] fp32;  delta : [rows] fp32. */
fox_status fox_attn_bwd_delta(const void* dO, fox_dtype dO_dt, const float* o, float* delta,
                              int64_t rows, int64_t D, void* stream);

/* Step 2, query-stationary: dq ([B,H,L,D] fp32), dc_q[i] = sum_j dS_ij ([B,H,L] fp32),
 * delta_out ([B,H,L] fp32, may equal delta) and lse_out ([B,H,L] fp32, must not alias lse).
 * delta_out is the row term refined so that each row of dS sums to zero under the P and dP this
 * library recomputes: the forward rounds P to bf16 before the PV product, so dO . O matches
 * sum_j P_ij dP_ij only to ~1e-3 relative, and d log f sums that residual over every row that
 * attends across a position. lse_out is the row offset that makes each recomputed row of P sum
 * to one: the forward's lse is the log of the sum of the bf16-rounded weights that built O, which
 * leaves exp(s - lse) summing to 1 + O(2^-9) over a row (most off where a few keys dominate, as
 * after a hard reset); the step scales dq and dc_q by the inverse of that sum and returns
 * lse + log(sum) for step 3. (The full-fp32 path's forward sums fp32 weights; it copies lse.)
 * The row term comes from delta (step 1's output) when it is not NULL, and o is then not read.
 * With delta = NULL, o ([B,H,L,D] fp32, the forward output) must be given and the step forms
 * Delta_i = dO_i . O_i itself, bit-identical to step 1 (the bf16 path in the same kernel; the
 * fp32 path as a launch of step 1 into delta_out first). Both NULL: FOX_E_INVALID. skip_plan as
 * for fox_attn_bwd. */
fox_status fox_attn_bwd_dq(const void* q, const void* k, const void* v, fox_dtype in_dt,
                           const void* c, const float* lse, const void* dO, const float* o,
                           const float* delta, float* dq, float* dc_q, float* delta_out,
                           float* lse_out, int64_t B, int64_t H, int64_t L, int64_t D,
                           float scale, uint32_t flags, const void* skip_plan, void* stream);

/* Step 3, key-stationary: dk, dv ([B,H,L,D] fp32) and dc_k[j] = -sum_i dS_ij ([B,H,L] fp32).
 * lse must be step 2's lse_out and delta step 2's delta_out; the other inputs (skip_plan too)
 * as for fox_attn_bwd. */
fox_status fox_attn_bwd_dkv(const void* q, const void* k, const void* v, fox_dtype in_dt,
                            const void* c, const float* lse, const void* dO, const float* delta,
                            float* dk, float* dv, float* dc_k, int64_t B, int64_t H, int64_t L,
                            int64_t D, float scale, uint32_t flags, const void* skip_plan,
                            void* stream);

/* Step 4, d log f[r, l] = sum_{t>=l} (dc_q[r, t] + dc_k[r, t]): the gradient of the prefix sum
 * fox_logf_cumsum computes, applied to dc = dc^q + dc^k ([BH, L] fp32 each; fp64 accumulation,
 * one rounding). dlog_f may not alias dc_q or dc_k. */
fox_status fox_dlogf_from_dc(const float* dc_q, const float* dc_k, float* dlog_f, int64_t BH,
                             int64_t L, void* stream);

/* Single-token decode against a KV cache. The last position t of a sequence attends to all of
 * its cached positions: o_t = sum_{j<=t} softmax_j(scale q_t.k_j + c_t - c_j) v_j, the forward's
 * row t (paper-graph-ui summary, section 3.4, "The Mathematical Form of Forgetting Attention"),
 * and appending a token extends c by the recurrence c_t = c_{t-1} + log f_t of the prefix sum
 * ("Hardware-Aware Implementation"). The cache has the forward's layout, so a prefill with
 * fox_logf_cumsum and fox_attn_fwd over the prompt leaves k, v, c ready for decoding.
 *   q       : [B, H, D] bf16, the query of the newest position of each sequence
 *   k_cache, v_cache : [B, H, T_max, D] bf16;  c_cache : [B, H, T_max] fp32
 *   lens    : [B] int32 on the device, the number of cached positions of each sequence
 *             (1 <= lens[b] <= T_max; the query sits at position lens[b] - 1, whose key and
 *             value must already be in the cache). A length above T_max is read as T_max; a
 *             sequence with lens[b] < 1 gets zeros and lse = -inf.
 *   k_norms : [B, H, ceil(T_max / 64)] fp32, the largest key norm of every 64 cached positions
 *             (fox_attn_decode_key_norms, kept current by fox_attn_decode_append), or NULL.
 *             With it, chunks of the cache whose every weight is provably below 2^-160 of the
 *             query's own-key weight (scale q.(k_j - k_t) - (c_j - c_t) <= scale |q| (|k_j| +
 *             |k_t|) - (c_min - c_t), c_min the chunk's smallest c, read from c_cache) have
 *             their keys and values not read; the result is bit-identical for any finite c,
 *             since such a chunk would enter the combination scaled by exactly 0 in fp32. A
 *             stale k_norms gives wrong results.
 *   o       : [B, H, D] in o_dt (FOX_BF16 or FOX_F32);  lse : [B, H] fp32 or NULL
 *   workspace : at least fox_attn_decode_workspace_bytes(B, H, T_max, D) bytes, 256-byte
 *             aligned, contents ignored and clobbered.
 * fp32 logits, exponentials and sums; no rounding of the weights. flags must contain
 * FOX_CAUSAL. Reads every cached key and value once (bound by HBM). Supports B*H <= 65535
 * (FOX_E_UNSUPPORTED beyond). */
size_t fox_attn_decode_workspace_bytes(int64_t B, int64_t H, int64_t T_max, int64_t D);
fox_status fox_attn_decode(const void* q, const void* k_cache, const void* v_cache,
                           fox_dtype in_dt, const float* c_cache, const int32_t* lens,
                           const float* k_norms, void* o, fox_dtype o_dt, float* lse,
                           void* workspace, size_t workspace_bytes, int64_t B, int64_t H,
                           int64_t T_max, int64_t D, float scale, uint32_t flags, void* stream);

/* The largest key norm of every 64 positions of a bf16 cache (positions at or past lens[b]
 * count as 0), rounded up: k_norms [B, H, ceil(T_max / 64)] fp32. Call it after filling a cache
 * by other means (a prefill); fox_attn_decode_append keeps it current afterwards. */
fox_status fox_attn_decode_key_norms(const void* k_cache, fox_dtype in_dt, const int32_t* lens,
                                     float* k_norms, int64_t B, int64_t H, int64_t T_max,
                                     int64_t D, void* stream);

/* Append one position to every sequence of the cache: at index p = lens[b], copy k_new and
 * v_new ([B, H, D] bf16) and set c_cache[b, h, p] = c_cache[b, h, p - 1] + log_f_new[b, h]
 * (log_f_new : [B, H] fp32; c starts at log f for p = 0), updates k_norms (or NULL) for the
 * group of p, then lens[b] += 1, all on the device. A sequence with lens[b] >= T_max (a full
 * cache) is left unchanged, lens included. */
fox_status fox_attn_decode_append(const void* k_new, const void* v_new, fox_dtype in_dt,
                                  const float* log_f_new, void* k_cache, void* v_cache,
                                  float* c_cache, float* k_norms, int32_t* lens, int64_t B,
                                  int64_t H, int64_t T_max, int64_t D, void* stream);

/* Static description of a status code. */
const char* fox_status_str(fox_status s);

/* Thread-local detail of the last non-OK status returned on this thread ("" if none). */
const char* fox_last_error(void);

/* Library version, "major.minor.patch". The minor number rises when a struct of this header
 * changes layout (0.2.0: fox_fwd_opts gained the key and value shift and the key norm fields at
 * its end), so a caller built against another layout can check it before passing one. */
const char* fox_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FOX_H */
