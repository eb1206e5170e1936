// abi.cpp — the C ABI of libfox (declared in include/fox.h).
//
// Each entry point validates its arguments on the host, returns FOX_E_INVALID /
// FOX_E_UNSUPPORTED before touching the GPU when they are wrong, and otherwise enqueues the
// kernels on the caller's stream and maps a failed launch to FOX_E_LAUNCH. Nothing here
// allocates device memory or synchronises the host with the device.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "fox.h"
#include "fox_launch.h"

namespace {

thread_local std::string g_last_error;

fox_status fail(fox_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

fox_status ok() {
  g_last_error.clear();
  return FOX_OK;
}

fox_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(FOX_E_LAUNCH, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Largest sequence length: the attention kernels address one (b, h) slab of L x D bf16 values
// with 32-bit byte offsets (buffer descriptors cover L * D * 2 bytes), so L * 128 * 2 < 2^32.
constexpr int64_t kMaxL = int64_t(1) << 23;
constexpr int64_t kMaxElems = int64_t(1) << 40;

// a * b <= lim for a, b >= 1, decided without forming a product that could overflow.
bool prod_le(int64_t a, int64_t b, int64_t lim) { return a <= lim / b; }

#define FOX_REQUIRE(cond, ...)                                   \
  do {                                                           \
    if (!(cond)) return fail(FOX_E_INVALID, __VA_ARGS__);        \
  } while (0)

#define FOX_REQUIRE_PTR(p)                                                          \
  do {                                                                              \
    FOX_REQUIRE((p) != nullptr, "%s must not be NULL", #p);                         \
    FOX_REQUIRE(aligned16(p), "%s must be 16-byte aligned", #p);                    \
  } while (0)

fox_status check_bhld(int64_t B, int64_t H, int64_t L, int64_t D) {
  FOX_REQUIRE(B >= 1 && H >= 1, "B and H must be >= 1 (got B=%lld H=%lld)", (long long)B,
              (long long)H);
  FOX_REQUIRE(L >= 1 && L <= kMaxL, "L must be in [1, %lld] (got %lld)", (long long)kMaxL,
              (long long)L);
  FOX_REQUIRE(D == 64 || D == 128, "D must be 64 or 128 (got %lld)", (long long)D);
  FOX_REQUIRE(prod_le(B, H, (int64_t(1) << 31) / 1024) && B * H * L * D <= kMaxElems,
              "B*H*L*D too large");
  return FOX_OK;
}

// Flags of the attention calls: FOX_CAUSAL is required; FOX_C_F64 says c holds fp64 values.
// A skip plan is built from fp32 c, so it is not taken together with FOX_C_F64.
fox_status check_flags(uint32_t flags, const void* skip_plan) {
  if (!(flags & FOX_CAUSAL))
    return fail(FOX_E_UNSUPPORTED, "only causal attention is defined (pass FOX_CAUSAL)");
  if (flags & ~uint32_t(FOX_CAUSAL | FOX_C_F64 | FOX_QK_RMSNORM | FOX_K_RMSNORM))
    return fail(FOX_E_UNSUPPORTED, "unknown flag bits 0x%x", flags);
  if (flags & (FOX_QK_RMSNORM | FOX_K_RMSNORM))
    return fail(FOX_E_UNSUPPORTED, "FOX_QK_RMSNORM and FOX_K_RMSNORM are taken by fox_attn_fwd_ex only");
  if ((flags & FOX_C_F64) && skip_plan)
    return fail(FOX_E_UNSUPPORTED, "a skip plan is built from fp32 c; it is not taken with FOX_C_F64");
  return FOX_OK;
}

fox::CPtr cptr(const void* c, uint32_t flags) {
  fox::CPtr r;
  r.p = c;
  r.f64 = (flags & FOX_C_F64) != 0;
  return r;
}

}  // namespace

extern "C" {

const char* fox_version(void) { return "0.2.0"; }

const char* fox_status_str(fox_status s) {
  switch (s) {
    case FOX_OK: return "ok";
    case FOX_E_INVALID: return "invalid argument";
    case FOX_E_UNSUPPORTED: return "unsupported request";
    case FOX_E_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

const char* fox_last_error(void) { return g_last_error.c_str(); }

fox_status fox_logf_cumsum(const float* log_f, float* c, int64_t BH, int64_t L, void* stream) {
  FOX_REQUIRE_PTR(log_f);
  FOX_REQUIRE_PTR(c);
  FOX_REQUIRE(log_f != c, "c must not alias log_f");
  FOX_REQUIRE(BH >= 1 && BH < (int64_t(1) << 31), "BH must be in [1, 2^31) (got %lld)",
              (long long)BH);
  FOX_REQUIRE(L >= 1 && L <= kMaxL, "L must be in [1, %lld] (got %lld)", (long long)kMaxL,
              (long long)L);
  return launched(fox::launch_cumsum(log_f, c, BH, L, (hipStream_t)stream), "fox_logf_cumsum");
}

fox_status fox_logf_cumsum_f64(const float* log_f, double* c, int64_t BH, int64_t L, void* stream) {
  FOX_REQUIRE_PTR(log_f);
  FOX_REQUIRE_PTR(c);
  FOX_REQUIRE((const void*)log_f != (const void*)c, "c must not alias log_f");
  FOX_REQUIRE(BH >= 1 && BH < (int64_t(1) << 31), "BH must be in [1, 2^31) (got %lld)",
              (long long)BH);
  FOX_REQUIRE(L >= 1 && L <= kMaxL, "L must be in [1, %lld] (got %lld)", (long long)kMaxL,
              (long long)L);
  return launched(fox::launch_cumsum64(log_f, c, BH, L, (hipStream_t)stream),
                  "fox_logf_cumsum_f64");
}

fox_status fox_gate_logf(const void* x, fox_dtype x_dt, const float* w_f, const float* b_f,
                         float* log_f, int64_t B, int64_t L, int64_t d_model, int64_t H,
                         void* stream) {
  FOX_REQUIRE_PTR(x);
  FOX_REQUIRE_PTR(w_f);
  FOX_REQUIRE(b_f != nullptr, "b_f must not be NULL");
  FOX_REQUIRE_PTR(log_f);
  FOX_REQUIRE(x_dt == FOX_BF16 || x_dt == FOX_F32, "x_dt must be FOX_BF16 or FOX_F32");
  FOX_REQUIRE(B >= 1 && L >= 1 && L <= kMaxL, "B >= 1 and 1 <= L <= 2^23 required");
  FOX_REQUIRE(H >= 1 && H <= 64, "H must be in [1, 64] (got %lld)", (long long)H);
  FOX_REQUIRE(d_model >= 8 && d_model <= 8192 && d_model % 8 == 0,
              "d_model must be a multiple of 8 in [8, 8192] (got %lld)", (long long)d_model);
  FOX_REQUIRE(prod_le(B, (L + 63) / 64, (int64_t(1) << 31) - 1), "B*L too large");
  return launched(fox::launch_gate(x, x_dt == FOX_BF16, w_f, b_f, log_f, B, L, d_model, H,
                                   fox::GateKind::kLogSigmoid, (hipStream_t)stream),
                  "fox_gate_logf");
}

fox_status fox_qk_rmsnorm(const void* x, void* y, fox_dtype dt, int64_t rows, int64_t D, float eps,
                          const float* weight, void* stream) {
  FOX_REQUIRE_PTR(x);
  FOX_REQUIRE_PTR(y);
  FOX_REQUIRE(dt == FOX_BF16 || dt == FOX_F32, "dt must be FOX_BF16 or FOX_F32");
  FOX_REQUIRE(D == 64 || D == 128, "D must be 64 or 128 (got %lld)", (long long)D);
  FOX_REQUIRE(rows >= 1 && prod_le(rows, D, kMaxElems) && rows * (D / 8) / 256 < (int64_t(1) << 31),
              "rows out of range");
  FOX_REQUIRE(eps >= 0.f, "eps must be >= 0");
  return launched(fox::launch_rmsnorm(x, y, dt == FOX_BF16, rows, D, eps, weight,
                                      (hipStream_t)stream),
                  "fox_qk_rmsnorm");
}

size_t fox_gate_logf_bwd_workspace_bytes(int64_t B, int64_t L, int64_t d_model, int64_t H) {
  if (B < 1 || L < 1 || L > kMaxL || d_model < 1 || d_model > 8192 || H < 1 || H > 64 ||
      !prod_le(B, L, (int64_t(1) << 31) / 64))
    return 0;
  return fox::gate_bwd_workspace_bytes(B, L, d_model, H);
}

fox_status fox_gate_logf_bwd(const void* x, fox_dtype x_dt, const float* w_f, const float* b_f,
                             const float* dlog_f, const float* log_f, float* dx, float* dw_f,
                             float* db_f, void* workspace, size_t workspace_bytes, int64_t B,
                             int64_t L, int64_t d_model, int64_t H, void* stream) {
  FOX_REQUIRE_PTR(x);
  FOX_REQUIRE_PTR(w_f);
  FOX_REQUIRE(b_f != nullptr, "b_f must not be NULL");
  FOX_REQUIRE_PTR(dlog_f);
  if (log_f) FOX_REQUIRE(aligned16(log_f), "log_f must be 16-byte aligned");
  FOX_REQUIRE_PTR(dx);
  FOX_REQUIRE_PTR(dw_f);
  FOX_REQUIRE(db_f != nullptr, "db_f must not be NULL");
  FOX_REQUIRE(workspace != nullptr, "workspace must not be NULL");
  FOX_REQUIRE((reinterpret_cast<uintptr_t>(workspace) & 255u) == 0,
              "workspace must be 256-byte aligned");
  FOX_REQUIRE(x_dt == FOX_BF16 || x_dt == FOX_F32, "x_dt must be FOX_BF16 or FOX_F32");
  FOX_REQUIRE(B >= 1 && L >= 1 && L <= kMaxL, "B >= 1 and 1 <= L <= 2^23 required");
  FOX_REQUIRE(H >= 1 && H <= 64, "H must be in [1, 64] (got %lld)", (long long)H);
  FOX_REQUIRE(d_model >= 8 && d_model <= 8192 && d_model % 8 == 0,
              "d_model must be a multiple of 8 in [8, 8192] (got %lld)", (long long)d_model);
  FOX_REQUIRE(prod_le(B, L, (int64_t(1) << 31) / 64) && B * L * d_model <= kMaxElems,
              "B*L*d_model too large");
  const size_t need = fox::gate_bwd_workspace_bytes(B, L, d_model, H);
  FOX_REQUIRE(workspace_bytes >= need, "workspace too small: %zu bytes given, %zu needed",
              workspace_bytes, need);
  return launched(fox::launch_gate_bwd(x, x_dt == FOX_BF16, w_f, b_f, dlog_f, log_f, dx, dw_f,
                                       db_f, workspace, B, L, d_model, H, fox::GateKind::kLogSigmoid,
                                       (hipStream_t)stream),
                  "fox_gate_logf_bwd");
}

size_t fox_qk_rmsnorm_bwd_workspace_bytes(int64_t rows, int64_t D) {
  if (rows < 1 || !(D == 64 || D == 128) || !prod_le(rows, D, kMaxElems)) return 0;
  return fox::rmsnorm_bwd_workspace_bytes(rows, D);
}

fox_status fox_qk_rmsnorm_bwd(const void* x, fox_dtype dt, const float* dy, float* dx,
                              const float* weight, float* dweight, void* workspace,
                              size_t workspace_bytes, int64_t rows, int64_t D, float eps,
                              void* stream) {
  FOX_REQUIRE_PTR(x);
  FOX_REQUIRE_PTR(dy);
  FOX_REQUIRE_PTR(dx);
  FOX_REQUIRE(dt == FOX_BF16 || dt == FOX_F32, "dt must be FOX_BF16 or FOX_F32");
  FOX_REQUIRE(D == 64 || D == 128, "D must be 64 or 128 (got %lld)", (long long)D);
  FOX_REQUIRE(rows >= 1 && prod_le(rows, D, kMaxElems), "rows out of range");
  FOX_REQUIRE(eps >= 0.f, "eps must be >= 0");
  FOX_REQUIRE(!(dweight && !weight), "dweight needs the weight it is the gradient of");
  if (dweight) {
    FOX_REQUIRE(workspace != nullptr, "workspace must not be NULL when dweight is wanted");
    FOX_REQUIRE((reinterpret_cast<uintptr_t>(workspace) & 255u) == 0,
                "workspace must be 256-byte aligned");
    const size_t need = fox::rmsnorm_bwd_workspace_bytes(rows, D);
    FOX_REQUIRE(workspace_bytes >= need, "workspace too small: %zu bytes given, %zu needed",
                workspace_bytes, need);
  }
  return launched(fox::launch_rmsnorm_bwd(x, dt == FOX_BF16, dy, weight, dx, dweight, workspace,
                                          rows, D, eps, (hipStream_t)stream),
                  "fox_qk_rmsnorm_bwd");
}

size_t fox_attn_skip_plan_bytes(int64_t B, int64_t H, int64_t L, int64_t D) {
  (void)D;
  if (B < 1 || H < 1 || L < 1 || L > kMaxL || !prod_le(B, H, int64_t(1) << 31)) return 0;
  return fox::skip_plan_layout(B * H, L).bytes;
}

fox_status fox_attn_skip_plan(const void* q, const void* k, fox_dtype in_dt, const float* c,
                              void* plan, size_t plan_bytes, int64_t B, int64_t H, int64_t L,
                              int64_t D, float scale, void* stream) {
  FOX_REQUIRE_PTR(q);
  FOX_REQUIRE_PTR(k);
  FOX_REQUIRE_PTR(c);
  FOX_REQUIRE(plan != nullptr, "plan must not be NULL");
  FOX_REQUIRE((reinterpret_cast<uintptr_t>(plan) & 255u) == 0, "plan must be 256-byte aligned");
  fox_status st = check_bhld(B, H, L, D);
  if (st != FOX_OK) return st;
  FOX_REQUIRE(scale > 0.f && scale < 1e30f, "scale must be positive and finite");
  if (in_dt != FOX_BF16)
    return fail(in_dt == FOX_F32 ? FOX_E_UNSUPPORTED : FOX_E_INVALID,
                "tile skipping serves the bf16 kernels (in_dt = FOX_BF16)");
  // the plan's kernels put B*H on the second grid axis and count items in 32-bit integers
  if (B * H > 65535 || B * H * ((L + 127) / 128 + (L + 255) / 256) > (int64_t(1) << 29))
    return fail(FOX_E_UNSUPPORTED, "tile skipping supports B*H <= 65535 and B*H*ceil(L/128) "
                "below 2^29 (got B*H=%lld, L=%lld)", (long long)(B * H), (long long)L);
  const size_t need = fox::skip_plan_layout(B * H, L).bytes;
  FOX_REQUIRE(plan_bytes >= need, "plan too small: %zu bytes given, %zu needed", plan_bytes, need);
  return launched(fox::launch_skip_plan(q, k, c, plan, B * H, L, D, scale, (hipStream_t)stream),
                  "fox_attn_skip_plan");
}

fox_status fox_attn_fwd(const void* q, const void* k, const void* v, fox_dtype in_dt,
                        const void* c, void* o, fox_dtype o_dt, float* lse, int64_t B, int64_t H,
                        int64_t L, int64_t D, float scale, uint32_t flags, const void* skip_plan,
                        void* stream) {
  FOX_REQUIRE_PTR(q);
  FOX_REQUIRE_PTR(k);
  FOX_REQUIRE_PTR(v);
  FOX_REQUIRE_PTR(c);
  FOX_REQUIRE_PTR(o);
  if (lse) FOX_REQUIRE(aligned16(lse), "lse must be 16-byte aligned");
  fox_status st = check_bhld(B, H, L, D);
  if (st != FOX_OK) return st;
  FOX_REQUIRE(in_dt == FOX_BF16 || in_dt == FOX_F32, "in_dt must be FOX_BF16 or FOX_F32");
  FOX_REQUIRE(o_dt == FOX_BF16 || o_dt == FOX_F32, "o_dt must be FOX_BF16 or FOX_F32");
  FOX_REQUIRE(!(in_dt == FOX_F32 && o_dt != FOX_F32), "fp32 inputs require an fp32 output");
  FOX_REQUIRE(scale > 0.f && scale < 1e30f, "scale must be positive and finite");
  st = check_flags(flags, skip_plan);
  if (st != FOX_OK) return st;
  FOX_REQUIRE((reinterpret_cast<uintptr_t>(skip_plan) & 255u) == 0,
              "skip_plan must be 256-byte aligned");
  if (skip_plan && in_dt != FOX_BF16)
    return fail(FOX_E_UNSUPPORTED, "tile skipping serves the bf16 kernels (in_dt = FOX_BF16)");
  if (in_dt == FOX_F32 && B * H > 65535)
    return fail(FOX_E_UNSUPPORTED, "the fp32 kernels take B*H <= 65535 (got %lld)", (long long)(B * H));
  const hipStream_t s = (hipStream_t)stream;
  if (in_dt == FOX_F32)
    return launched(fox::launch_fwd_f32((const float*)q, (const float*)k, (const float*)v,
                                        cptr(c, flags), (float*)o, lse, B * H, L, D, scale, s),
                    "fox_attn_fwd");
  return launched(fox::launch_fwd_bf16(q, k, v, cptr(c, flags), o, o_dt == FOX_F32, lse, B * H, L,
                                       D, scale,
                                       fox::skip_args(skip_plan, B * H, L), s),
                  "fox_attn_fwd");
}

fox_status fox_attn_fwd_ex(const void* q, const void* k, const void* v, fox_dtype in_dt,
                           const void* c, void* o, fox_dtype o_dt, float* lse, int64_t B,
                           int64_t H, int64_t L, int64_t D, const fox_fwd_opts* opts,
                           void* stream) {
  FOX_REQUIRE(opts != nullptr, "opts must not be NULL");
  const uint32_t flags = opts->flags;
  const bool qnorm = (flags & FOX_QK_RMSNORM) != 0;
  const bool gated = opts->gate != nullptr;
  const bool knorm = (flags & FOX_K_RMSNORM) != 0;
  const bool staged = knorm || opts->k_shift_alpha || opts->v_shift_alpha;  // K/V via registers
  if (!qnorm && !gated && !staged)  // nothing fused: the plain forward
    return fox_attn_fwd(q, k, v, in_dt, c, o, o_dt, lse, B, H, L, D, opts->scale, flags,
                        opts->skip_plan, stream);
  FOX_REQUIRE_PTR(q);
  FOX_REQUIRE_PTR(k);
  FOX_REQUIRE_PTR(v);
  FOX_REQUIRE_PTR(c);
  FOX_REQUIRE(o != nullptr || gated, "o may be NULL only when the output gate is given");
  if (o) FOX_REQUIRE(aligned16(o), "o must be 16-byte aligned");
  if (lse) FOX_REQUIRE(aligned16(lse), "lse must be 16-byte aligned");
  fox_status st = check_bhld(B, H, L, D);
  if (st != FOX_OK) return st;
  if (in_dt != FOX_BF16)
    return fail(FOX_E_UNSUPPORTED, "QK-norm, the token shift and the output gate serve the bf16 kernels");
  FOX_REQUIRE(o_dt == FOX_BF16 || o_dt == FOX_F32, "o_dt must be FOX_BF16 or FOX_F32");
  FOX_REQUIRE(opts->scale > 0.f && opts->scale < 1e30f, "scale must be positive and finite");
  if (!(flags & FOX_CAUSAL))
    return fail(FOX_E_UNSUPPORTED, "only causal attention is defined (pass FOX_CAUSAL)");
  if (flags & ~uint32_t(FOX_CAUSAL | FOX_C_F64 | FOX_QK_RMSNORM | FOX_K_RMSNORM))
    return fail(FOX_E_UNSUPPORTED, "unknown flag bits 0x%x", flags);
  if ((flags & FOX_C_F64) && opts->skip_plan)
    return fail(FOX_E_UNSUPPORTED, "a skip plan is built from fp32 c; it is not taken with FOX_C_F64");
  if (qnorm && opts->skip_plan)
    return fail(FOX_E_UNSUPPORTED, "a skip plan is built from the normalised q; it is not taken "
                                   "with FOX_QK_RMSNORM");
  if (staged && opts->skip_plan)
    return fail(FOX_E_UNSUPPORTED, "a skip plan is built from the keys the attention sees; it is "
                                   "not taken with the key shift or FOX_K_RMSNORM");
  if (knorm) FOX_REQUIRE(opts->k_norm_eps >= 0.f, "k_norm_eps must be >= 0");
  FOX_REQUIRE((reinterpret_cast<uintptr_t>(opts->k_shift_alpha) & 3u) == 0 &&
                  (reinterpret_cast<uintptr_t>(opts->v_shift_alpha) & 3u) == 0 &&
                  (reinterpret_cast<uintptr_t>(opts->k_norm_weight) & 3u) == 0,
              "the shift gates and k_norm_weight must be 4-byte aligned");
  FOX_REQUIRE((reinterpret_cast<uintptr_t>(opts->skip_plan) & 255u) == 0,
              "skip_plan must be 256-byte aligned");
  if (qnorm) FOX_REQUIRE(opts->q_norm_eps >= 0.f, "q_norm_eps must be >= 0");
  // the caller's struct may hold any int in gate_dt: read its bits, not an enum value
  static_assert(sizeof(fox_dtype) == sizeof(int), "fox_dtype is an int-sized enum");
  int gate_dt = 0;
  std::memcpy(&gate_dt, &opts->gate_dt, sizeof gate_dt);
  if (gated) {
    FOX_REQUIRE(aligned16(opts->gate), "gate must be 16-byte aligned");
    FOX_REQUIRE_PTR(opts->y);
    FOX_REQUIRE(gate_dt == FOX_BF16 || gate_dt == FOX_F32, "gate_dt must be FOX_BF16 or FOX_F32");
    FOX_REQUIRE(opts->out_norm_eps >= 0.f, "out_norm_eps must be >= 0");
  }
  fox::ProFwdArgs pa;
  pa.q_norm = qnorm;
  pa.q_w = opts->q_norm_weight;
  pa.q_eps = opts->q_norm_eps;
  pa.g = opts->gate;
  pa.g_f32 = gate_dt == FOX_F32;
  pa.out_w = opts->out_norm_weight;
  pa.out_eps = opts->out_norm_eps;
  pa.y = gated ? opts->y : nullptr;
  pa.k_alpha = opts->k_shift_alpha;
  pa.v_alpha = opts->v_shift_alpha;
  pa.k_norm = knorm;
  pa.k_w = opts->k_norm_weight;
  pa.k_eps = opts->k_norm_eps;
  return launched(fox::launch_fwd_bf16(q, k, v, cptr(c, flags), o, o_dt == FOX_F32, lse, B * H, L,
                                       D, opts->scale, fox::skip_args(opts->skip_plan, B * H, L),
                                       (hipStream_t)stream, &pa),
                  "fox_attn_fwd_ex");
}

fox_status fox_attn_fwd_logf(const void* q, const void* k, const void* v, fox_dtype in_dt,
                             const float* log_f, void* c_out, void* o, fox_dtype o_dt, float* lse,
                             int64_t B, int64_t H, int64_t L, int64_t D, float scale,
                             uint32_t flags, void* stream) {
  FOX_REQUIRE_PTR(q);
  FOX_REQUIRE_PTR(k);
  FOX_REQUIRE_PTR(v);
  FOX_REQUIRE_PTR(log_f);
  FOX_REQUIRE_PTR(c_out);
  FOX_REQUIRE_PTR(o);
  FOX_REQUIRE((const void*)log_f != c_out, "c_out must not alias log_f");
  if (lse) FOX_REQUIRE(aligned16(lse), "lse must be 16-byte aligned");
  fox_status st = check_bhld(B, H, L, D);
  if (st != FOX_OK) return st;
  FOX_REQUIRE(in_dt == FOX_BF16 || in_dt == FOX_F32, "in_dt must be FOX_BF16 or FOX_F32");
  FOX_REQUIRE(o_dt == FOX_BF16 || o_dt == FOX_F32, "o_dt must be FOX_BF16 or FOX_F32");
  FOX_REQUIRE(!(in_dt == FOX_F32 && o_dt != FOX_F32), "fp32 inputs require an fp32 output");
  FOX_REQUIRE(scale > 0.f && scale < 1e30f, "scale must be positive and finite");
  st = check_flags(flags, nullptr);
  if (st != FOX_OK) return st;
  if (in_dt == FOX_F32 && B * H > 65535)
    return fail(FOX_E_UNSUPPORTED, "the fp32 kernels take B*H <= 65535 (got %lld)", (long long)(B * H));
  const hipStream_t s = (hipStream_t)stream;
  const fox::CPtr c = cptr(c_out, flags);
  if (in_dt == FOX_F32) {  // the full-fp32 path: the scan, then the forward on its output
    const hipError_t e = c.f64 ? fox::launch_cumsum64(log_f, (double*)c_out, B * H, L, s)
                               : fox::launch_cumsum(log_f, (float*)c_out, B * H, L, s);
    if (e != hipSuccess) return launched(e, "fox_attn_fwd_logf");
    return launched(fox::launch_fwd_f32((const float*)q, (const float*)k, (const float*)v, c,
                                        (float*)o, lse, B * H, L, D, scale, s),
                    "fox_attn_fwd_logf");
  }
  return launched(fox::launch_fwd_bf16_logf(q, k, v, log_f, c, o, o_dt == FOX_F32, lse, B * H, L,
                                            D, scale, s),
                  "fox_attn_fwd_logf");
}

size_t fox_attn_bwd_workspace_bytes(int64_t B, int64_t H, int64_t L, int64_t D) {
  (void)D;
  if (B < 1 || H < 1 || L < 1 || L > kMaxL || !prod_le(B, H, int64_t(1) << 31)) return 0;
  return fox::bwd_workspace_bytes(B * H, L);
}

}  // extern "C"

namespace {

// fox_attn_bwd's validation and launches; the workspace comes from the caller or, with
// scratch set, from the library's static array (fox_attn_bwd_noalloc, named `what` in
// messages), whose address is looked up only once every argument has passed.
fox_status attn_bwd_impl(const void* q, const void* k, const void* v, fox_dtype in_dt,
                         const void* c, const float* o, const float* lse, const void* dO,
                         float* dq, float* dk, float* dv, float* dlog_f, void* workspace,
                         size_t workspace_bytes, int64_t B, int64_t H, int64_t L, int64_t D,
                         float scale, uint32_t flags, const void* skip_plan, void* stream,
                         const char* what, bool scratch) {
  FOX_REQUIRE_PTR(q);
  FOX_REQUIRE_PTR(k);
  FOX_REQUIRE_PTR(v);
  FOX_REQUIRE_PTR(c);
  FOX_REQUIRE_PTR(o);
  FOX_REQUIRE_PTR(lse);
  FOX_REQUIRE_PTR(dO);
  FOX_REQUIRE_PTR(dq);
  FOX_REQUIRE_PTR(dk);
  FOX_REQUIRE_PTR(dv);
  FOX_REQUIRE_PTR(dlog_f);
  if (!scratch) {
    FOX_REQUIRE(workspace != nullptr, "workspace must not be NULL");
    FOX_REQUIRE((reinterpret_cast<uintptr_t>(workspace) & 255u) == 0,
                "workspace must be 256-byte aligned");
  }
  fox_status st = check_bhld(B, H, L, D);
  if (st != FOX_OK) return st;
  FOX_REQUIRE(scale > 0.f && scale < 1e30f, "scale must be positive and finite");
  st = check_flags(flags, skip_plan);
  if (st != FOX_OK) return st;
  FOX_REQUIRE(in_dt == FOX_BF16 || in_dt == FOX_F32, "in_dt must be FOX_BF16 or FOX_F32");
  const size_t need = fox::bwd_workspace_bytes(B * H, L);
  if (scratch)
    FOX_REQUIRE(need <= fox::noalloc_scratch_bytes(),
                "B*H*L too large for the static scratch: %zu bytes needed, %zu held "
                "(fox_attn_bwd_noalloc_max_bytes; use fox_attn_bwd with a workspace)",
                need, fox::noalloc_scratch_bytes());
  else
    FOX_REQUIRE(workspace_bytes >= need, "workspace too small: %zu bytes given, %zu needed",
                workspace_bytes, need);
  FOX_REQUIRE((reinterpret_cast<uintptr_t>(skip_plan) & 255u) == 0,
              "skip_plan must be 256-byte aligned");
  if (in_dt == FOX_F32 && skip_plan)
    return fail(FOX_E_UNSUPPORTED, "tile skipping serves the bf16 kernels (in_dt = FOX_BF16)");
  if (in_dt == FOX_F32 && B * H > 65535)
    return fail(FOX_E_UNSUPPORTED, "the fp32 kernels take B*H <= 65535 (got %lld)",
                (long long)(B * H));
  if (scratch) {
    const hipError_t e = fox::noalloc_scratch(&workspace);
    if (e != hipSuccess)
      return fail(FOX_E_LAUNCH, "%s: scratch address: %s", what, hipGetErrorString(e));
  }
  if (in_dt == FOX_F32) {
    return launched(fox::launch_bwd_f32((const float*)q, (const float*)k, (const float*)v,
                                        cptr(c, flags), o, lse, (const float*)dO, dq, dk, dv,
                                        dlog_f, workspace, B * H, L, D, scale,
                                        (hipStream_t)stream),
                    what);
  }
  return launched(fox::launch_bwd_bf16(q, k, v, cptr(c, flags), o, lse, dO, dq, dk, dv, dlog_f,
                                       workspace,
                                       B * H, L, D, scale, skip_plan, (hipStream_t)stream),
                  what);
}

}  // namespace

extern "C" {

fox_status fox_attn_bwd(const void* q, const void* k, const void* v, fox_dtype in_dt,
                        const void* c, const float* o, const float* lse, const void* dO,
                        float* dq, float* dk, float* dv, float* dlog_f, void* workspace,
                        size_t workspace_bytes, int64_t B, int64_t H, int64_t L, int64_t D,
                        float scale, uint32_t flags, const void* skip_plan, void* stream) {
  return attn_bwd_impl(q, k, v, in_dt, c, o, lse, dO, dq, dk, dv, dlog_f, workspace,
                       workspace_bytes, B, H, L, D, scale, flags, skip_plan, stream,
                       "fox_attn_bwd", false);
}

size_t fox_attn_bwd_noalloc_max_bytes(void) { return fox::noalloc_scratch_bytes(); }

fox_status fox_attn_bwd_noalloc(const void* q, const void* k, const void* v, fox_dtype in_dt,
                                const void* c, const float* o, const float* lse, const void* dO,
                                float* dq, float* dk, float* dv, float* dlog_f, int64_t B,
                                int64_t H, int64_t L, int64_t D, float scale, uint32_t flags,
                                const void* skip_plan, void* stream) {
  return attn_bwd_impl(q, k, v, in_dt, c, o, lse, dO, dq, dk, dv, dlog_f, nullptr, 0, B, H, L, D,
                       scale, flags, skip_plan, stream, "fox_attn_bwd_noalloc", true);
}

namespace {
fox_status check_bwd_common(const void* q, const void* k, const void* v, fox_dtype in_dt,
                            const void* c, const float* lse, const void* dO, int64_t B, int64_t H,
                            int64_t L, int64_t D, float scale, uint32_t flags,
                            const void* skip_plan) {
  FOX_REQUIRE_PTR(q);
  FOX_REQUIRE_PTR(k);
  FOX_REQUIRE_PTR(v);
  FOX_REQUIRE_PTR(c);
  FOX_REQUIRE_PTR(lse);
  FOX_REQUIRE_PTR(dO);
  fox_status st = check_bhld(B, H, L, D);
  if (st != FOX_OK) return st;
  FOX_REQUIRE(scale > 0.f && scale < 1e30f, "scale must be positive and finite");
  st = check_flags(flags, skip_plan);
  if (st != FOX_OK) return st;
  FOX_REQUIRE(in_dt == FOX_BF16 || in_dt == FOX_F32, "in_dt must be FOX_BF16 or FOX_F32");
  if (in_dt == FOX_F32 && B * H > 65535)
    return fail(FOX_E_UNSUPPORTED, "the fp32 kernels take B*H <= 65535 (got %lld)", (long long)(B * H));
  return FOX_OK;
}
}  // namespace

fox_status fox_attn_bwd_delta(const void* dO, fox_dtype dO_dt, const float* o, float* delta,
                              int64_t rows, int64_t D, void* stream) {
  FOX_REQUIRE_PTR(dO);
  FOX_REQUIRE_PTR(o);
  FOX_REQUIRE_PTR(delta);
  FOX_REQUIRE(dO_dt == FOX_BF16 || dO_dt == FOX_F32, "dO_dt must be FOX_BF16 or FOX_F32");
  FOX_REQUIRE(D == 64 || D == 128, "D must be 64 or 128 (got %lld)", (long long)D);
  FOX_REQUIRE(rows >= 1 && prod_le(rows, D, kMaxElems) && rows * (D / 8) / 256 < (int64_t(1) << 31),
              "rows out of range");
  if (dO_dt == FOX_F32)
    return launched(fox::launch_bwd_delta_f32((const float*)dO, o, delta, rows, D,
                                              (hipStream_t)stream),
                    "fox_attn_bwd_delta");
  return launched(fox::launch_bwd_delta(dO, o, delta, rows, D, (hipStream_t)stream),
                  "fox_attn_bwd_delta");
}

fox_status fox_attn_bwd_dkv(const void* q, const void* k, const void* v, fox_dtype in_dt,
                            const void* c, const float* lse, const void* dO, const float* delta,
                            float* dk, float* dv, float* dc_k, int64_t B, int64_t H, int64_t L,
                            int64_t D, float scale, uint32_t flags, const void* skip_plan,
                            void* stream) {
  fox_status st = check_bwd_common(q, k, v, in_dt, c, lse, dO, B, H, L, D, scale, flags, skip_plan);
  if (st != FOX_OK) return st;
  FOX_REQUIRE_PTR(delta);
  FOX_REQUIRE((reinterpret_cast<uintptr_t>(skip_plan) & 255u) == 0,
              "skip_plan must be 256-byte aligned");
  FOX_REQUIRE_PTR(dk);
  FOX_REQUIRE_PTR(dv);
  FOX_REQUIRE_PTR(dc_k);
  if (in_dt == FOX_F32) {
    if (skip_plan)
      return fail(FOX_E_UNSUPPORTED, "tile skipping serves the bf16 kernels (in_dt = FOX_BF16)");
    return launched(fox::launch_bwd_dkv_f32((const float*)q, (const float*)k, (const float*)v,
                                            cptr(c, flags), lse,
                                            (const float*)dO, delta, dk, dv, dc_k, B * H, L, D,
                                            scale, (hipStream_t)stream),
                    "fox_attn_bwd_dkv");
  }
  return launched(fox::launch_bwd_dkv(q, k, v, cptr(c, flags), lse, dO, delta, dk, dv, dc_k, B * H, L, D, scale,
                                      fox::skip_args(skip_plan, B * H, L), (hipStream_t)stream),
                  "fox_attn_bwd_dkv");
}

fox_status fox_attn_bwd_dq(const void* q, const void* k, const void* v, fox_dtype in_dt,
                           const void* c, const float* lse, const void* dO, const float* o,
                           const float* delta, float* dq, float* dc_q, float* delta_out,
                           float* lse_out, int64_t B, int64_t H, int64_t L, int64_t D,
                           float scale, uint32_t flags, const void* skip_plan, void* stream) {
  fox_status st = check_bwd_common(q, k, v, in_dt, c, lse, dO, B, H, L, D, scale, flags, skip_plan);
  if (st != FOX_OK) return st;
  FOX_REQUIRE(delta != nullptr || o != nullptr, "one of delta and o must be given");
  if (delta) FOX_REQUIRE_PTR(delta);
  else FOX_REQUIRE_PTR(o);
  FOX_REQUIRE((reinterpret_cast<uintptr_t>(skip_plan) & 255u) == 0,
              "skip_plan must be 256-byte aligned");
  FOX_REQUIRE_PTR(dq);
  FOX_REQUIRE_PTR(dc_q);
  FOX_REQUIRE_PTR(delta_out);
  FOX_REQUIRE_PTR(lse_out);
  FOX_REQUIRE((const void*)lse_out != (const void*)lse, "lse_out must not alias lse");
  const float* o_used = delta ? nullptr : o;  // a given delta wins; o is then not read
  if (in_dt == FOX_F32) {
    if (skip_plan)
      return fail(FOX_E_UNSUPPORTED, "tile skipping serves the bf16 kernels (in_dt = FOX_BF16)");
    if (o_used) {  // the vector-ALU path keeps the row term as its own launch, into delta_out
      const hipError_t e = fox::launch_bwd_delta_f32((const float*)dO, o_used, delta_out, B * H * L,
                                                     D, (hipStream_t)stream);
      if (e != hipSuccess) return launched(e, "fox_attn_bwd_dq");
      delta = delta_out;
    }
    return launched(fox::launch_bwd_dq_f32((const float*)q, (const float*)k, (const float*)v,
                                           cptr(c, flags), lse, (const float*)dO, delta, dq, dc_q,
                                           delta_out, lse_out, B * H, L, D, scale,
                                           (hipStream_t)stream),
                    "fox_attn_bwd_dq");
  }
  return launched(fox::launch_bwd_dq(q, k, v, cptr(c, flags), lse, dO, delta, o_used, dq, dc_q,
                                     delta_out, lse_out, B * H, L, D, scale,
                                     fox::skip_args(skip_plan, B * H, L), (hipStream_t)stream),
                  "fox_attn_bwd_dq");
}

namespace {
fox_status check_shift_gate(const void* x, fox_dtype x_dt, const float* w, int64_t B, int64_t L,
                            int64_t d_model, int64_t H) {
  FOX_REQUIRE_PTR(x);
  FOX_REQUIRE_PTR(w);
  FOX_REQUIRE(x_dt == FOX_BF16 || x_dt == FOX_F32, "x_dt must be FOX_BF16 or FOX_F32");
  FOX_REQUIRE(B >= 1 && L >= 1 && L <= kMaxL, "B >= 1 and 1 <= L <= 2^23 required");
  FOX_REQUIRE(H >= 1 && H <= 64, "H must be in [1, 64] (got %lld)", (long long)H);
  FOX_REQUIRE(d_model >= 8 && d_model <= 8192 && d_model % 8 == 0,
              "d_model must be a multiple of 8 in [8, 8192] (got %lld)", (long long)d_model);
  FOX_REQUIRE(prod_le(B, L, (int64_t(1) << 31) / 64) && B * L * d_model <= kMaxElems,
              "B*L*d_model too large");
  return FOX_OK;
}

fox_status check_rows(const void* x, int64_t rows, int64_t D, float eps) {
  FOX_REQUIRE_PTR(x);
  FOX_REQUIRE(D == 64 || D == 128, "D must be 64 or 128 (got %lld)", (long long)D);
  FOX_REQUIRE(rows >= 1 && prod_le(rows, D, kMaxElems), "rows out of range");
  FOX_REQUIRE(eps >= 0.f, "eps must be >= 0");
  return FOX_OK;
}
}  // namespace

fox_status fox_shift_gate(const void* x, fox_dtype x_dt, const float* w, float* alpha, int64_t B,
                          int64_t L, int64_t d_model, int64_t H, void* stream) {
  fox_status st = check_shift_gate(x, x_dt, w, B, L, d_model, H);
  if (st != FOX_OK) return st;
  FOX_REQUIRE_PTR(alpha);
  return launched(fox::launch_gate(x, x_dt == FOX_BF16, w, nullptr, alpha, B, L, d_model, H,
                                   fox::GateKind::kSigmoid, (hipStream_t)stream),
                  "fox_shift_gate");
}

fox_status fox_shift_gate_bwd(const void* x, fox_dtype x_dt, const float* w, const float* dalpha,
                              float* dx, float* dw, void* workspace, size_t workspace_bytes,
                              int64_t B, int64_t L, int64_t d_model, int64_t H, void* stream) {
  fox_status st = check_shift_gate(x, x_dt, w, B, L, d_model, H);
  if (st != FOX_OK) return st;
  FOX_REQUIRE_PTR(dalpha);
  FOX_REQUIRE_PTR(dx);
  FOX_REQUIRE_PTR(dw);
  FOX_REQUIRE(workspace != nullptr, "workspace must not be NULL");
  FOX_REQUIRE((reinterpret_cast<uintptr_t>(workspace) & 255u) == 0,
              "workspace must be 256-byte aligned");
  const size_t need = fox::gate_bwd_workspace_bytes(B, L, d_model, H);
  FOX_REQUIRE(workspace_bytes >= need, "workspace too small: %zu bytes given, %zu needed",
              workspace_bytes, need);
  return launched(fox::launch_gate_bwd(x, x_dt == FOX_BF16, w, nullptr, dalpha, nullptr, dx, dw,
                                       nullptr, workspace, B, L, d_model, H, fox::GateKind::kSigmoid,
                                       (hipStream_t)stream),
                  "fox_shift_gate_bwd");
}

fox_status fox_kv_shift(const void* x, fox_dtype dt, const float* alpha, void* y, int normalize,
                        float eps, const float* weight, int64_t BH, int64_t L, int64_t D,
                        void* stream) {
  FOX_REQUIRE(BH >= 1 && L >= 1 && L <= kMaxL && prod_le(BH, L, kMaxElems),
              "BH >= 1, 1 <= L <= 2^23 and BH*L*D <= 2^40 required");
  fox_status st = check_rows(x, BH * L, D, eps);
  if (st != FOX_OK) return st;
  FOX_REQUIRE_PTR(alpha);
  FOX_REQUIRE_PTR(y);
  FOX_REQUIRE(dt == FOX_BF16 || dt == FOX_F32, "dt must be FOX_BF16 or FOX_F32");
  FOX_REQUIRE(BH >= 1 && L >= 1 && L <= kMaxL, "BH >= 1 and 1 <= L <= 2^23 required");
  FOX_REQUIRE(y != x, "y must not alias x (each row reads its predecessor)");
  return launched(fox::launch_kv_shift(x, dt == FOX_BF16, alpha, y, normalize != 0, eps, weight,
                                       BH * L, L, D, (hipStream_t)stream),
                  "fox_kv_shift");
}

fox_status fox_kv_shift_bwd(const void* x, fox_dtype dt, const float* alpha, const float* dy,
                            float* dx, float* dalpha, int normalize, float eps,
                            const float* weight, int64_t BH, int64_t L, int64_t D, void* stream) {
  FOX_REQUIRE(BH >= 1 && L >= 1 && L <= kMaxL && prod_le(BH, L, kMaxElems),
              "BH >= 1, 1 <= L <= 2^23 and BH*L*D <= 2^40 required");
  fox_status st = check_rows(x, BH * L, D, eps);
  if (st != FOX_OK) return st;
  FOX_REQUIRE_PTR(alpha);
  FOX_REQUIRE_PTR(dy);
  FOX_REQUIRE_PTR(dx);
  FOX_REQUIRE_PTR(dalpha);
  FOX_REQUIRE(dt == FOX_BF16 || dt == FOX_F32, "dt must be FOX_BF16 or FOX_F32");
  FOX_REQUIRE(BH >= 1 && L >= 1 && L <= kMaxL, "BH >= 1 and 1 <= L <= 2^23 required");
  FOX_REQUIRE(static_cast<const void*>(dx) != static_cast<const void*>(dy),
              "dx must not alias dy (each row reads its successor's gradient)");
  return launched(fox::launch_kv_shift_bwd(x, dt == FOX_BF16, alpha, dy, dx, dalpha,
                                           normalize != 0, eps, weight, BH * L, L, D,
                                           (hipStream_t)stream),
                  "fox_kv_shift_bwd");
}

fox_status fox_out_norm_gate(const void* o, fox_dtype o_dt, const void* g, fox_dtype g_dt,
                             const float* weight, float eps, void* y, int64_t rows, int64_t D,
                             void* stream) {
  fox_status st = check_rows(o, rows, D, eps);
  if (st != FOX_OK) return st;
  FOX_REQUIRE_PTR(g);
  FOX_REQUIRE_PTR(y);
  FOX_REQUIRE(o_dt == FOX_BF16 || o_dt == FOX_F32, "o_dt must be FOX_BF16 or FOX_F32");
  FOX_REQUIRE(g_dt == FOX_BF16 || g_dt == FOX_F32, "g_dt must be FOX_BF16 or FOX_F32");
  return launched(fox::launch_out_norm_gate(o, o_dt == FOX_BF16, g, g_dt == FOX_BF16, weight, eps,
                                            y, rows, D, (hipStream_t)stream),
                  "fox_out_norm_gate");
}

fox_status fox_out_norm_gate_bwd(const void* o, fox_dtype o_dt, const void* g, fox_dtype g_dt,
                                 const float* weight, float eps, const float* dy, float* d_o,
                                 float* dg, int64_t rows, int64_t D, void* stream) {
  fox_status st = check_rows(o, rows, D, eps);
  if (st != FOX_OK) return st;
  FOX_REQUIRE_PTR(g);
  FOX_REQUIRE_PTR(dy);
  FOX_REQUIRE_PTR(d_o);
  FOX_REQUIRE_PTR(dg);
  FOX_REQUIRE(o_dt == FOX_BF16 || o_dt == FOX_F32, "o_dt must be FOX_BF16 or FOX_F32");
  FOX_REQUIRE(g_dt == FOX_BF16 || g_dt == FOX_F32, "g_dt must be FOX_BF16 or FOX_F32");
  return launched(fox::launch_out_norm_gate_bwd(o, o_dt == FOX_BF16, g, g_dt == FOX_BF16, weight,
                                                eps, dy, d_o, dg, rows, D, (hipStream_t)stream),
                  "fox_out_norm_gate_bwd");
}

size_t fox_attn_decode_workspace_bytes(int64_t B, int64_t H, int64_t T_max, int64_t D) {
  if (B < 1 || H < 1 || T_max < 1 || T_max > kMaxL || (D != 64 && D != 128) ||
      !prod_le(B, H, int64_t(1) << 31))
    return 0;
  return fox::decode_workspace_bytes(B * H, T_max, D);
}

fox_status fox_attn_decode(const void* q, const void* k_cache, const void* v_cache,
                           fox_dtype in_dt, const float* c_cache, const int32_t* lens,
                           const float* k_norms, void* o, fox_dtype o_dt, float* lse,
                           void* workspace, size_t workspace_bytes, int64_t B, int64_t H,
                           int64_t T_max, int64_t D, float scale, uint32_t flags, void* stream) {
  FOX_REQUIRE_PTR(q);
  FOX_REQUIRE_PTR(k_cache);
  FOX_REQUIRE_PTR(v_cache);
  FOX_REQUIRE_PTR(c_cache);
  FOX_REQUIRE_PTR(lens);
  FOX_REQUIRE_PTR(o);
  if (lse) FOX_REQUIRE(aligned16(lse), "lse must be 16-byte aligned");
  if (k_norms) FOX_REQUIRE(aligned16(k_norms), "k_norms must be 16-byte aligned");
  FOX_REQUIRE(workspace != nullptr, "workspace must not be NULL");
  FOX_REQUIRE((reinterpret_cast<uintptr_t>(workspace) & 255u) == 0,
              "workspace must be 256-byte aligned");
  fox_status st = check_bhld(B, H, T_max, D);
  if (st != FOX_OK) return st;
  FOX_REQUIRE(o_dt == FOX_BF16 || o_dt == FOX_F32, "o_dt must be FOX_BF16 or FOX_F32");
  FOX_REQUIRE(scale > 0.f && scale < 1e30f, "scale must be positive and finite");
  if (!(flags & FOX_CAUSAL))
    return fail(FOX_E_UNSUPPORTED, "only causal attention is defined (pass FOX_CAUSAL)");
  if (flags & ~uint32_t(FOX_CAUSAL)) return fail(FOX_E_UNSUPPORTED, "unknown flag bits 0x%x", flags);
  if (in_dt != FOX_BF16)
    return fail(in_dt == FOX_F32 ? FOX_E_UNSUPPORTED : FOX_E_INVALID,
                "the decode step takes a bf16 cache (in_dt = FOX_BF16)");
  if (B * H > 65535)  // the second grid axis
    return fail(FOX_E_UNSUPPORTED, "decode supports B*H <= 65535 (got %lld)", (long long)(B * H));
  const size_t need = fox::decode_workspace_bytes(B * H, T_max, D);
  FOX_REQUIRE(workspace_bytes >= need, "workspace too small: %zu bytes given, %zu needed",
              workspace_bytes, need);
  return launched(fox::launch_decode(q, k_cache, v_cache, c_cache, lens, k_norms, o,
                                     o_dt == FOX_F32, lse, workspace, B, H, T_max, D, scale,
                                     (hipStream_t)stream),
                  "fox_attn_decode");
}

fox_status fox_attn_decode_key_norms(const void* k_cache, fox_dtype in_dt, const int32_t* lens,
                                     float* k_norms, int64_t B, int64_t H, int64_t T_max,
                                     int64_t D, void* stream) {
  FOX_REQUIRE_PTR(k_cache);
  FOX_REQUIRE_PTR(lens);
  FOX_REQUIRE_PTR(k_norms);
  fox_status st = check_bhld(B, H, T_max, D);
  if (st != FOX_OK) return st;
  if (in_dt != FOX_BF16)
    return fail(in_dt == FOX_F32 ? FOX_E_UNSUPPORTED : FOX_E_INVALID,
                "the decode cache is bf16 (in_dt = FOX_BF16)");
  if (B * H > 65535)  // the second grid axis
    return fail(FOX_E_UNSUPPORTED, "decode supports B*H <= 65535 (got %lld)", (long long)(B * H));
  return launched(fox::launch_decode_key_norms(k_cache, lens, k_norms, B, H, T_max, D,
                                               (hipStream_t)stream),
                  "fox_attn_decode_key_norms");
}

fox_status fox_attn_decode_append(const void* k_new, const void* v_new, fox_dtype in_dt,
                                  const float* log_f_new, void* k_cache, void* v_cache,
                                  float* c_cache, float* k_norms, int32_t* lens, int64_t B,
                                  int64_t H, int64_t T_max, int64_t D, void* stream) {
  FOX_REQUIRE_PTR(k_new);
  FOX_REQUIRE_PTR(v_new);
  FOX_REQUIRE_PTR(log_f_new);
  FOX_REQUIRE_PTR(k_cache);
  FOX_REQUIRE_PTR(v_cache);
  FOX_REQUIRE_PTR(c_cache);
  FOX_REQUIRE_PTR(lens);
  if (k_norms) FOX_REQUIRE(aligned16(k_norms), "k_norms must be 16-byte aligned");
  fox_status st = check_bhld(B, H, T_max, D);
  if (st != FOX_OK) return st;
  if (in_dt != FOX_BF16)
    return fail(in_dt == FOX_F32 ? FOX_E_UNSUPPORTED : FOX_E_INVALID,
                "the decode cache is bf16 (in_dt = FOX_BF16)");
  return launched(fox::launch_decode_append(k_new, v_new, log_f_new, k_cache, v_cache, c_cache,
                                            k_norms, lens, B, H, T_max, D, (hipStream_t)stream),
                  "fox_attn_decode_append");
}

fox_status fox_dlogf_from_dc(const float* dc_q, const float* dc_k, float* dlog_f, int64_t BH,
                             int64_t L, void* stream) {
  FOX_REQUIRE_PTR(dc_q);
  FOX_REQUIRE_PTR(dc_k);
  FOX_REQUIRE_PTR(dlog_f);
  FOX_REQUIRE(dlog_f != dc_q && dlog_f != dc_k, "dlog_f must not alias dc_q or dc_k");
  FOX_REQUIRE(BH >= 1 && BH < (int64_t(1) << 31), "BH must be in [1, 2^31)");
  FOX_REQUIRE(L >= 1 && L <= kMaxL, "L must be in [1, 2^23]");
  return launched(fox::launch_rev_cumsum2(dc_q, dc_k, dlog_f, BH, L, (hipStream_t)stream),
                  "fox_dlogf_from_dc");
}

}  // extern "C"
