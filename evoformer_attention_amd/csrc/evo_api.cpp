// C ABI of libevoattn.so (declared in include/evo_attn.h): argument
// validation, error reporting and dispatch to the kernel launchers.
// Every check runs before the first HIP call, so an invalid call enqueues
// nothing and touches no device state.
#include "evo_attn.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

#include "evo_kernels.h"

namespace {

thread_local std::string g_last_error;

evo_status_t fail(evo_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

evo_status_t ok() {
  g_last_error.clear();
  return EVO_OK;
}

// Test hook: EVO_FAULT_INJECT=launch makes every entry point report a HIP
// launch failure after validation, without touching the device.
bool fault_injected() {
  const char* e = std::getenv("EVO_FAULT_INJECT");
  return e && std::strcmp(e, "launch") == 0;
}

evo_status_t from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(EVO_EHIP, "%s: HIP error %d (%s)", what, (int)e,
              hipGetErrorString(e));
}

size_t elem_size(evo_dtype_t dt) { return dt == EVO_BF16 ? 2 : 4; }

bool aligned16(const void* p) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

// Largest element count any single tensor may have (kernel offsets are
// 64-bit, work-item counts 32-bit).
constexpr int64_t kMaxElems = int64_t(1) << 40;

evo_status_t check_dtype(evo_dtype_t dt) {
  if (dt != EVO_FP32 && dt != EVO_BF16)
    return fail(EVO_ENOTSUP, "dtype %d is not supported (EVO_FP32=0, "
                "EVO_BF16=1)", (int)dt);
  return EVO_OK;
}

evo_status_t check_core_sizes(evo_dtype_t dt, int64_t B, int64_t R, int64_t N,
                              int64_t H, int64_t C) {
  evo_status_t st = check_dtype(dt);
  if (st != EVO_OK) return st;
  if (B <= 0 || R <= 0 || N <= 0 || H <= 0 || C <= 0)
    return fail(EVO_EINVAL, "sizes must be positive (B=%lld R=%lld N=%lld "
                "H=%lld C=%lld)", (long long)B, (long long)R, (long long)N,
                (long long)H, (long long)C);
  if (C != evo::kHeadDim)
    return fail(EVO_ENOTSUP, "head dimension C=%lld is not supported (only "
                "C=32)", (long long)C);
  if (N > (int64_t(1) << 20) || H > 4096 || R > (int64_t(1) << 24) ||
      B > (int64_t(1) << 24))
    return fail(EVO_ENOTSUP, "problem too large (N<=2^20, H<=4096, R,B<=2^24)");
  if (B * R * N * H * C > kMaxElems || B * H * N * N > kMaxElems)
    return fail(EVO_ENOTSUP, "problem too large: tensors above 2^40 elements");
  return EVO_OK;
}

#define REQUIRE_PTR(p)                                                   \
  do {                                                                   \
    if (!(p)) return fail(EVO_EINVAL, "argument '%s' is NULL", #p);      \
    if (!aligned16(p))                                                   \
      return fail(EVO_ENOTSUP, "argument '%s' is not 16-byte aligned", #p); \
  } while (0)

#define OPTIONAL_PTR(p)                                                  \
  do {                                                                   \
    if ((p) && !aligned16(p))                                            \
      return fail(EVO_ENOTSUP, "argument '%s' is not 16-byte aligned", #p); \
  } while (0)

evo_status_t check_mask(const uint8_t* key_mask, int64_t mask_rows,
                        int64_t R) {
  if (!key_mask) return EVO_OK;
  if (mask_rows != 1 && mask_rows != R)
    return fail(EVO_EINVAL, "mask_rows=%lld must be 1 or R=%lld",
                (long long)mask_rows, (long long)R);
  return EVO_OK;
}

}  // namespace

extern "C" {

int evo_abi_version(void) { return 1; }

const char* evo_last_error(void) { return g_last_error.c_str(); }

evo_status_t evo_attn_fwd(evo_dtype_t dtype, int64_t B, int64_t R, int64_t N,
                          int64_t H, int64_t C, const void* q, const void* k,
                          const void* v, const void* gate,
                          const uint8_t* key_mask, int64_t mask_rows,
                          const void* bias, void* out, float* lse,
                          void* workspace, size_t workspace_bytes,
                          void* stream) {
  try {
    evo_status_t st = check_core_sizes(dtype, B, R, N, H, C);
    if (st != EVO_OK) return st;
    REQUIRE_PTR(q);
    REQUIRE_PTR(k);
    REQUIRE_PTR(v);
    REQUIRE_PTR(out);
    OPTIONAL_PTR(gate);
    OPTIONAL_PTR(bias);
    OPTIONAL_PTR(lse);
    OPTIONAL_PTR(key_mask);
    if ((st = check_mask(key_mask, mask_rows, R)) != EVO_OK) return st;
    if (bias || key_mask) {
      const size_t need = evo::attn_fwd_workspace((int)dtype, B, N, H);
      if (!workspace || workspace_bytes < need)
        return fail(EVO_EWORKSPACE, "workspace of %zu bytes needed, %zu given",
                    need, workspace ? workspace_bytes : (size_t)0);
      if (!aligned16(workspace))
        return fail(EVO_ENOTSUP, "argument 'workspace' is not 16-byte aligned");
    }
    if (fault_injected()) return fail(EVO_EHIP, "evo_attn_fwd: injected launch failure");
    evo::AttnFwdArgs a{(int)dtype, B, R, N, H, q, k, v, gate, key_mask,
                       mask_rows, bias, out, lse, workspace};
    return from_hip(evo::launch_attn_fwd(a, (hipStream_t)stream),
                    "evo_attn_fwd");
  } catch (...) {
    return fail(EVO_EINTERNAL, "evo_attn_fwd: internal error");
  }
}

evo_status_t evo_attn_fwd_noalloc(evo_dtype_t dtype, int64_t B, int64_t R,
                                  int64_t N, int64_t H, int64_t C, const void* q,
                                  const void* k, const void* v, const void* gate,
                                  const uint8_t* key_mask, int64_t mask_rows,
                                  const void* bias, void* out, float* lse,
                                  void* stream) {
  try {
    evo_status_t st = check_core_sizes(dtype, B, R, N, H, C);
    if (st != EVO_OK) return st;
    REQUIRE_PTR(q);
    REQUIRE_PTR(k);
    REQUIRE_PTR(v);
    REQUIRE_PTR(out);
    OPTIONAL_PTR(gate);
    OPTIONAL_PTR(bias);
    OPTIONAL_PTR(lse);
    OPTIONAL_PTR(key_mask);
    if ((st = check_mask(key_mask, mask_rows, R)) != EVO_OK) return st;
    void* scratch = nullptr;
    if (bias || key_mask) {
      const size_t need = evo::attn_fwd_workspace((int)dtype, B, N, H);
      size_t cap = 0;
      const hipError_t e = evo::fwd_static_scratch(&scratch, &cap);
      if (e != hipSuccess) return from_hip(e, "evo_attn_fwd_noalloc: scratch lookup");
      if (need > cap)
        return fail(EVO_ENOTSUP,
                    "evo_attn_fwd_noalloc: the prepared bias needs %zu bytes, more than "
                    "the library's static scratch of %zu bytes (call evo_attn_fwd with "
                    "a workspace instead)", need, cap);
    }
    if (fault_injected())
      return fail(EVO_EHIP, "evo_attn_fwd_noalloc: injected launch failure");
    evo::AttnFwdArgs a{(int)dtype, B, R, N, H, q, k, v, gate, key_mask,
                       mask_rows, bias, out, lse, scratch};
    return from_hip(evo::launch_attn_fwd(a, (hipStream_t)stream),
                    "evo_attn_fwd_noalloc");
  } catch (...) {
    return fail(EVO_EINTERNAL, "evo_attn_fwd_noalloc: internal error");
  }
}

evo_status_t evo_probe_issue_rate(int kind, int waves_per_simd, int iters, float* out,
                                  void* stream) {
  try {
    if (kind < 0 || kind > 2) return fail(EVO_EINVAL, "evo_probe_issue_rate: kind %d", kind);
    if (waves_per_simd < 1 || waves_per_simd > 8 || iters < 1)
      return fail(EVO_EINVAL, "evo_probe_issue_rate: waves_per_simd %d, iters %d",
                  waves_per_simd, iters);
    REQUIRE_PTR(out);
    return from_hip(evo::launch_probe(kind, waves_per_simd, iters, out, (hipStream_t)stream),
                    "evo_probe_issue_rate");
  } catch (...) {
    return fail(EVO_EINTERNAL, "evo_probe_issue_rate: internal error");
  }
}

size_t evo_attn_fwd_workspace_bytes(evo_dtype_t dtype, int64_t B, int64_t R,
                                    int64_t N, int64_t H, int64_t C) {
  const std::string saved = g_last_error;
  const evo_status_t st = check_core_sizes(dtype, B, R, N, H, C);
  g_last_error = saved;
  if (st != EVO_OK) return 0;
  return evo::attn_fwd_workspace((int)dtype, B, N, H);
}

size_t evo_attn_bwd_workspace_bytes(evo_dtype_t dtype, int64_t B, int64_t R,
                                    int64_t N, int64_t H, int64_t C) {
  const std::string saved = g_last_error;
  const evo_status_t st = check_core_sizes(dtype, B, R, N, H, C);
  g_last_error = saved;
  if (st != EVO_OK) return 0;
  return evo::attn_bwd_workspace((int)dtype, B, R, N, H);
}

evo_status_t evo_attn_bwd(evo_dtype_t dtype, int64_t B, int64_t R, int64_t N,
                          int64_t H, int64_t C, const void* q, const void* k,
                          const void* v, const void* gate,
                          const uint8_t* key_mask, int64_t mask_rows,
                          const void* bias, const void* out, const float* lse,
                          const void* dout, void* dq, void* dk, void* dv,
                          void* dgate, float* dbias, void* workspace,
                          size_t workspace_bytes, void* stream) {
  try {
    evo_status_t st = check_core_sizes(dtype, B, R, N, H, C);
    if (st != EVO_OK) return st;
    REQUIRE_PTR(q);
    REQUIRE_PTR(k);
    REQUIRE_PTR(v);
    REQUIRE_PTR(out);
    REQUIRE_PTR(lse);
    REQUIRE_PTR(dout);
    REQUIRE_PTR(dq);
    REQUIRE_PTR(dk);
    REQUIRE_PTR(dv);
    OPTIONAL_PTR(gate);
    OPTIONAL_PTR(dgate);
    OPTIONAL_PTR(bias);
    OPTIONAL_PTR(dbias);
    if ((gate == nullptr) != (dgate == nullptr))
      return fail(EVO_EINVAL, "dgate must be given exactly when gate is");
    OPTIONAL_PTR(key_mask);
    if ((st = check_mask(key_mask, mask_rows, R)) != EVO_OK) return st;
    const size_t need = evo::attn_bwd_workspace((int)dtype, B, R, N, H);
    if (need == 0)
      return fail(EVO_ENOTSUP, "evo_attn_bwd supports N <= 65536 (N=%lld)",
                  (long long)N);
    if (!workspace || workspace_bytes < need)
      return fail(EVO_EWORKSPACE, "workspace of %zu bytes needed, %zu given",
                  need, workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace))
      return fail(EVO_ENOTSUP, "argument 'workspace' is not 16-byte aligned");
    if (fault_injected()) return fail(EVO_EHIP, "evo_attn_bwd: injected launch failure");
    evo::AttnBwdArgs a{(int)dtype, B, R, N, H, q, k, v, gate, key_mask,
                       mask_rows, bias, out, lse, dout, dq, dk, dv, dgate,
                       dbias, workspace};
    return from_hip(evo::launch_attn_bwd(a, (hipStream_t)stream),
                    "evo_attn_bwd");
  } catch (...) {
    return fail(EVO_EINTERNAL, "evo_attn_bwd: internal error");
  }
}

static evo_status_t check_module_sizes(evo_dtype_t dtype, int64_t N,
                                       int64_t CZ, int64_t H, int64_t C) {
  evo_status_t st = check_core_sizes(dtype, 1, N, N, H, C);
  if (st != EVO_OK) return st;
  if (CZ <= 0) return fail(EVO_EINVAL, "CZ=%lld must be positive", (long long)CZ);
  if (N > 46340)  // N*N positions are indexed in 32 bits
    return fail(EVO_ENOTSUP, "N=%lld is not supported (at most 46340)", (long long)N);
  if (CZ % 32 != 0 || CZ > 256)
    return fail(EVO_ENOTSUP, "CZ=%lld is not supported (multiple of 32, at "
                "most 256)", (long long)CZ);
  if (H * C > 256)
    return fail(EVO_ENOTSUP, "H*C=%lld is not supported (at most 256)",
                (long long)(H * C));
  return EVO_OK;
}

evo_status_t tri_attn_project(evo_dtype_t dtype, int64_t N, int64_t CZ,
                              int64_t H, int64_t C, int ending, const void* z,
                              const void* ln_w, const void* ln_b, float ln_eps,
                              const void* w_q, const void* w_k,
                              const void* w_v, const void* w_g,
                              const void* b_g, const void* w_bias, void* q,
                              void* k, void* v, void* g, void* bias,
                              void* stream) {
  try {
    evo_status_t st = check_module_sizes(dtype, N, CZ, H, C);
    if (st != EVO_OK) return st;
    if (ending != 0 && ending != 1)
      return fail(EVO_EINVAL, "ending=%d must be 0 or 1", ending);
    if (!(ln_eps > 0.f)) return fail(EVO_EINVAL, "ln_eps must be > 0");
    REQUIRE_PTR(z);
    REQUIRE_PTR(ln_w);
    REQUIRE_PTR(ln_b);
    REQUIRE_PTR(w_q);
    REQUIRE_PTR(w_k);
    REQUIRE_PTR(w_v);
    REQUIRE_PTR(w_g);
    REQUIRE_PTR(w_bias);
    REQUIRE_PTR(q);
    REQUIRE_PTR(k);
    REQUIRE_PTR(v);
    REQUIRE_PTR(g);
    REQUIRE_PTR(bias);
    OPTIONAL_PTR(b_g);
    if (fault_injected()) return fail(EVO_EHIP, "tri_attn_project: injected launch failure");
    evo::ProjectArgs a{(int)dtype, N, CZ, H, ending, z, ln_w, ln_b, ln_eps,
                       w_q, w_k, w_v, w_g, b_g, w_bias, q, k, v, g, bias};
    return from_hip(evo::launch_project(a, (hipStream_t)stream),
                    "tri_attn_project");
  } catch (...) {
    return fail(EVO_EINTERNAL, "tri_attn_project: internal error");
  }
}

evo_status_t tri_attn_out_project(evo_dtype_t dtype, int64_t N, int64_t CZ,
                                  int64_t H, int64_t C, int ending,
                                  const void* o, const void* w_o,
                                  const void* b_o, void* out, void* stream) {
  try {
    evo_status_t st = check_module_sizes(dtype, N, CZ, H, C);
    if (st != EVO_OK) return st;
    if (ending != 0 && ending != 1)
      return fail(EVO_EINVAL, "ending=%d must be 0 or 1", ending);
    REQUIRE_PTR(o);
    REQUIRE_PTR(w_o);
    REQUIRE_PTR(out);
    OPTIONAL_PTR(b_o);
    if (fault_injected()) return fail(EVO_EHIP, "tri_attn_out_project: injected launch failure");
    evo::OutProjectArgs a{(int)dtype, N, CZ, H, ending, o, w_o, b_o, out};
    return from_hip(evo::launch_out_project(a, (hipStream_t)stream),
                    "tri_attn_out_project");
  } catch (...) {
    return fail(EVO_EINTERNAL, "tri_attn_out_project: internal error");
  }
}

// Workspace layout of tri_attn_module_fwd: q | k | v | g | o (each
// N*N*H*C elements) | bias (H*N*N elements) | the forward's fp32 bias,
// each region 256-byte aligned.
static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

size_t tri_attn_workspace_bytes(evo_dtype_t dtype, int64_t N, int64_t CZ,
                                int64_t H, int64_t C) {
  const std::string saved = g_last_error;
  const evo_status_t st = check_module_sizes(dtype, N, CZ, H, C);
  g_last_error = saved;
  if (st != EVO_OK) return 0;
  const size_t es = elem_size(dtype);
  const size_t t = align256((size_t)N * N * H * C * es);
  const size_t b = align256((size_t)H * N * N * es);
  return 5 * t + b + align256(evo::attn_fwd_workspace((int)dtype, 1, N, H));
}

evo_status_t tri_attn_module_fwd(evo_dtype_t dtype, int64_t N, int64_t CZ,
                                 int64_t H, int64_t C, int ending,
                                 const void* z, const uint8_t* residue_mask,
                                 const void* ln_w, const void* ln_b,
                                 float ln_eps, const void* w_q,
                                 const void* w_k, const void* w_v,
                                 const void* w_g, const void* b_g,
                                 const void* w_bias, const void* w_o,
                                 const void* b_o, void* out, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  try {
    evo_status_t st = check_module_sizes(dtype, N, CZ, H, C);
    if (st != EVO_OK) return st;
    if (ending != 0 && ending != 1)
      return fail(EVO_EINVAL, "ending=%d must be 0 or 1", ending);
    if (!(ln_eps > 0.f)) return fail(EVO_EINVAL, "ln_eps must be > 0");
    REQUIRE_PTR(z);
    REQUIRE_PTR(ln_w);
    REQUIRE_PTR(ln_b);
    REQUIRE_PTR(w_q);
    REQUIRE_PTR(w_k);
    REQUIRE_PTR(w_v);
    REQUIRE_PTR(w_g);
    REQUIRE_PTR(w_bias);
    REQUIRE_PTR(w_o);
    REQUIRE_PTR(out);
    OPTIONAL_PTR(b_g);
    OPTIONAL_PTR(b_o);
    OPTIONAL_PTR(residue_mask);
    const size_t need = tri_attn_workspace_bytes(dtype, N, CZ, H, C);
    if (!workspace || workspace_bytes < need)
      return fail(EVO_EWORKSPACE, "workspace of %zu bytes needed, %zu given",
                  need, workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace))
      return fail(EVO_ENOTSUP, "argument 'workspace' is not 16-byte aligned");
    if (fault_injected()) return fail(EVO_EHIP, "tri_attn_module_fwd: injected launch failure");

    const size_t es = elem_size(dtype);
    const size_t t = align256((size_t)N * N * H * C * es);
    char* ws = static_cast<char*>(workspace);
    void* q = ws;
    void* k = ws + t;
    void* v = ws + 2 * t;
    void* g = ws + 3 * t;
    void* o = ws + 4 * t;
    void* bias = ws + 5 * t;
    void* fwd_ws = ws + 5 * t + align256((size_t)H * N * N * es);
    hipStream_t s = (hipStream_t)stream;

    evo::ProjectArgs pa{(int)dtype, N, CZ, H, ending, z, ln_w, ln_b, ln_eps,
                        w_q, w_k, w_v, w_g, b_g, w_bias, q, k, v, g, bias};
    st = from_hip(evo::launch_project(pa, s), "tri_attn_module_fwd/project");
    if (st != EVO_OK) return st;
    evo::AttnFwdArgs fa{(int)dtype, 1, N, N, H, q, k, v, g, residue_mask, 1,
                        bias, o, nullptr, fwd_ws};
    st = from_hip(evo::launch_attn_fwd(fa, s), "tri_attn_module_fwd/attention");
    if (st != EVO_OK) return st;
    evo::OutProjectArgs oa{(int)dtype, N, CZ, H, ending, o, w_o, b_o, out};
    return from_hip(evo::launch_out_project(oa, s),
                    "tri_attn_module_fwd/out_project");
  } catch (...) {
    return fail(EVO_EINTERNAL, "tri_attn_module_fwd: internal error");
  }
}


// ---------------------------------------------------------------- backward

static evo_status_t check_module_bwd_sizes(evo_dtype_t dtype, int64_t N,
                                           int64_t CZ, int64_t H, int64_t C) {
  evo_status_t st = check_module_sizes(dtype, N, CZ, H, C);
  if (st != EVO_OK) return st;
  if (CZ > 128 || H * C > 128)
    return fail(EVO_ENOTSUP, "the module backward supports CZ <= 128 and "
                "H*C <= 128 (CZ=%lld, H*C=%lld)", (long long)CZ,
                (long long)(H * C));
  return EVO_OK;
}

size_t tri_attn_proj_bwd_workspace_bytes(evo_dtype_t dtype, int64_t N,
                                         int64_t CZ, int64_t H, int64_t C) {
  const std::string saved = g_last_error;
  const evo_status_t st = check_module_bwd_sizes(dtype, N, CZ, H, C);
  g_last_error = saved;
  if (st != EVO_OK) return 0;
  return evo::proj_bwd_workspace(N, CZ, H);
}

// Workspace layout of tri_attn_module_bwd: q | k | v | g | o | do | dq | dk
// | dv | dg (each N*N*H*C elements) | bias (H*N*N elements) | lse and dbias
// (fp32) | the attention forward's and backward's workspaces | the
// projection backward's workspace, each region 256-byte aligned.
struct ModuleBwdLayout {
  size_t t, bias, lse, dbias, fwd, bwd, proj, total;
};
static ModuleBwdLayout module_bwd_layout(evo_dtype_t dtype, int64_t N,
                                         int64_t CZ, int64_t H, int64_t C) {
  const size_t es = elem_size(dtype);
  ModuleBwdLayout L;
  L.t = align256((size_t)N * N * H * C * es);
  L.bias = 10 * L.t;
  L.lse = L.bias + align256((size_t)H * N * N * es);
  L.dbias = L.lse + align256((size_t)N * H * N * 4);
  L.fwd = L.dbias + align256((size_t)H * N * N * 4);
  L.bwd = L.fwd + align256(evo::attn_fwd_workspace((int)dtype, 1, N, H));
  L.proj = L.bwd + align256(evo::attn_bwd_workspace((int)dtype, 1, N, N, H));
  L.total = L.proj + align256(evo::proj_bwd_workspace(N, CZ, H));
  return L;
}

size_t tri_attn_bwd_workspace_bytes(evo_dtype_t dtype, int64_t N, int64_t CZ,
                                    int64_t H, int64_t C) {
  const std::string saved = g_last_error;
  const evo_status_t st = check_module_bwd_sizes(dtype, N, CZ, H, C);
  g_last_error = saved;
  if (st != EVO_OK) return 0;
  return module_bwd_layout(dtype, N, CZ, H, C).total;
}

static evo_status_t check_workspace(const char* fn, void* workspace,
                                    size_t workspace_bytes, size_t need) {
  if (!workspace || workspace_bytes < need)
    return fail(EVO_EWORKSPACE, "%s: workspace of %zu bytes needed, %zu given",
                fn, need, workspace ? workspace_bytes : (size_t)0);
  if (!aligned16(workspace))
    return fail(EVO_ENOTSUP, "argument 'workspace' is not 16-byte aligned");
  return EVO_OK;
}

evo_status_t tri_attn_out_project_bwd(evo_dtype_t dtype, int64_t N,
                                      int64_t CZ, int64_t H, int64_t C,
                                      int ending, const void* o,
                                      const void* w_o, const void* dout,
                                      void* d_o, float* dw_o, float* db_o,
                                      void* workspace, size_t workspace_bytes,
                                      void* stream) {
  try {
    evo_status_t st = check_module_bwd_sizes(dtype, N, CZ, H, C);
    if (st != EVO_OK) return st;
    if (ending != 0 && ending != 1)
      return fail(EVO_EINVAL, "ending=%d must be 0 or 1", ending);
    REQUIRE_PTR(o);
    REQUIRE_PTR(w_o);
    REQUIRE_PTR(dout);
    REQUIRE_PTR(d_o);
    REQUIRE_PTR(dw_o);
    REQUIRE_PTR(db_o);
    st = check_workspace("tri_attn_out_project_bwd", workspace, workspace_bytes,
                         evo::proj_bwd_workspace(N, CZ, H));
    if (st != EVO_OK) return st;
    if (fault_injected())
      return fail(EVO_EHIP, "tri_attn_out_project_bwd: injected launch failure");
    evo::OutProjectBwdArgs a{(int)dtype, N, CZ, H, ending, o, w_o, dout, d_o,
                             dw_o, db_o, workspace};
    return from_hip(evo::launch_out_project_bwd(a, (hipStream_t)stream),
                    "tri_attn_out_project_bwd");
  } catch (...) {
    return fail(EVO_EINTERNAL, "tri_attn_out_project_bwd: internal error");
  }
}

evo_status_t tri_attn_project_bwd(
    evo_dtype_t dtype, int64_t N, int64_t CZ, int64_t H, int64_t C, int ending,
    const void* z, const void* ln_w, const void* ln_b, float ln_eps,
    const void* w_q, const void* w_k, const void* w_v, const void* w_g,
    const void* w_bias, const void* dq, const void* dk, const void* dv,
    const void* dg, const float* dbias, void* dz, float* dln_w, float* dln_b,
    float* dw_q, float* dw_k, float* dw_v, float* dw_g, float* db_g,
    float* dw_bias, void* workspace, size_t workspace_bytes, void* stream) {
  try {
    evo_status_t st = check_module_bwd_sizes(dtype, N, CZ, H, C);
    if (st != EVO_OK) return st;
    if (ending != 0 && ending != 1)
      return fail(EVO_EINVAL, "ending=%d must be 0 or 1", ending);
    if (!(ln_eps > 0.f)) return fail(EVO_EINVAL, "ln_eps must be > 0");
    REQUIRE_PTR(z);
    REQUIRE_PTR(ln_w);
    REQUIRE_PTR(ln_b);
    REQUIRE_PTR(w_q);
    REQUIRE_PTR(w_k);
    REQUIRE_PTR(w_v);
    REQUIRE_PTR(w_g);
    REQUIRE_PTR(w_bias);
    REQUIRE_PTR(dq);
    REQUIRE_PTR(dk);
    REQUIRE_PTR(dv);
    REQUIRE_PTR(dg);
    REQUIRE_PTR(dbias);
    REQUIRE_PTR(dz);
    REQUIRE_PTR(dln_w);
    REQUIRE_PTR(dln_b);
    REQUIRE_PTR(dw_q);
    REQUIRE_PTR(dw_k);
    REQUIRE_PTR(dw_v);
    REQUIRE_PTR(dw_g);
    REQUIRE_PTR(db_g);
    REQUIRE_PTR(dw_bias);
    st = check_workspace("tri_attn_project_bwd", workspace, workspace_bytes,
                         evo::proj_bwd_workspace(N, CZ, H));
    if (st != EVO_OK) return st;
    if (fault_injected())
      return fail(EVO_EHIP, "tri_attn_project_bwd: injected launch failure");
    evo::ProjectBwdArgs a{(int)dtype, N, CZ, H, ending, z, ln_w, ln_b, ln_eps,
                          w_q, w_k, w_v, w_g, w_bias, dq, dk, dv, dg, dbias,
                          dz, dln_w, dln_b, dw_q, dw_k, dw_v, dw_g, db_g,
                          dw_bias, workspace};
    return from_hip(evo::launch_project_bwd(a, (hipStream_t)stream),
                    "tri_attn_project_bwd");
  } catch (...) {
    return fail(EVO_EINTERNAL, "tri_attn_project_bwd: internal error");
  }
}

evo_status_t tri_attn_module_bwd(
    evo_dtype_t dtype, int64_t N, int64_t CZ, int64_t H, int64_t C, int ending,
    const void* z, const uint8_t* residue_mask, const void* ln_w,
    const void* ln_b, float ln_eps, const void* w_q, const void* w_k,
    const void* w_v, const void* w_g, const void* b_g, const void* w_bias,
    const void* w_o, const void* dout, void* dz, float* dln_w, float* dln_b,
    float* dw_q, float* dw_k, float* dw_v, float* dw_g, float* db_g,
    float* dw_bias, float* dw_o, float* db_o, void* workspace,
    size_t workspace_bytes, void* stream) {
  try {
    evo_status_t st = check_module_bwd_sizes(dtype, N, CZ, H, C);
    if (st != EVO_OK) return st;
    if (ending != 0 && ending != 1)
      return fail(EVO_EINVAL, "ending=%d must be 0 or 1", ending);
    if (!(ln_eps > 0.f)) return fail(EVO_EINVAL, "ln_eps must be > 0");
    REQUIRE_PTR(z);
    REQUIRE_PTR(ln_w);
    REQUIRE_PTR(ln_b);
    REQUIRE_PTR(w_q);
    REQUIRE_PTR(w_k);
    REQUIRE_PTR(w_v);
    REQUIRE_PTR(w_g);
    REQUIRE_PTR(w_bias);
    REQUIRE_PTR(w_o);
    REQUIRE_PTR(dout);
    REQUIRE_PTR(dz);
    REQUIRE_PTR(dln_w);
    REQUIRE_PTR(dln_b);
    REQUIRE_PTR(dw_q);
    REQUIRE_PTR(dw_k);
    REQUIRE_PTR(dw_v);
    REQUIRE_PTR(dw_g);
    REQUIRE_PTR(db_g);
    REQUIRE_PTR(dw_bias);
    REQUIRE_PTR(dw_o);
    REQUIRE_PTR(db_o);
    OPTIONAL_PTR(b_g);
    OPTIONAL_PTR(residue_mask);
    const ModuleBwdLayout L = module_bwd_layout(dtype, N, CZ, H, C);
    st = check_workspace("tri_attn_module_bwd", workspace, workspace_bytes, L.total);
    if (st != EVO_OK) return st;
    if (fault_injected())
      return fail(EVO_EHIP, "tri_attn_module_bwd: injected launch failure");

    char* ws = static_cast<char*>(workspace);
    void* q = ws;
    void* k = ws + L.t;
    void* v = ws + 2 * L.t;
    void* g = ws + 3 * L.t;
    void* o = ws + 4 * L.t;
    void* d_o = ws + 5 * L.t;
    void* dq = ws + 6 * L.t;
    void* dk = ws + 7 * L.t;
    void* dv = ws + 8 * L.t;
    void* dg = ws + 9 * L.t;
    void* bias = ws + L.bias;
    float* lse = reinterpret_cast<float*>(ws + L.lse);
    float* dbias = reinterpret_cast<float*>(ws + L.dbias);
    hipStream_t s = (hipStream_t)stream;

    // the forward's activations, recomputed from z
    evo::ProjectArgs pa{(int)dtype, N, CZ, H, ending, z, ln_w, ln_b, ln_eps,
                        w_q, w_k, w_v, w_g, b_g, w_bias, q, k, v, g, bias};
    st = from_hip(evo::launch_project(pa, s), "tri_attn_module_bwd/project");
    if (st != EVO_OK) return st;
    evo::AttnFwdArgs fa{(int)dtype, 1, N, N, H, q, k, v, g, residue_mask, 1,
                        bias, o, lse, ws + L.fwd};
    st = from_hip(evo::launch_attn_fwd(fa, s), "tri_attn_module_bwd/attention");
    if (st != EVO_OK) return st;
    // backward, last step first
    evo::OutProjectBwdArgs ob{(int)dtype, N, CZ, H, ending, o, w_o, dout, d_o,
                              dw_o, db_o, ws + L.proj};
    st = from_hip(evo::launch_out_project_bwd(ob, s),
                  "tri_attn_module_bwd/out_project_bwd");
    if (st != EVO_OK) return st;
    evo::AttnBwdArgs ab{(int)dtype, 1, N, N, H, q, k, v, g, residue_mask, 1,
                        bias, o, lse, d_o, dq, dk, dv, dg, dbias, ws + L.bwd};
    st = from_hip(evo::launch_attn_bwd(ab, s), "tri_attn_module_bwd/attention_bwd");
    if (st != EVO_OK) return st;
    evo::ProjectBwdArgs pb{(int)dtype, N, CZ, H, ending, z, ln_w, ln_b, ln_eps,
                           w_q, w_k, w_v, w_g, w_bias, dq, dk, dv, dg, dbias,
                           dz, dln_w, dln_b, dw_q, dw_k, dw_v, dw_g, db_g,
                           dw_bias, ws + L.proj};
    return from_hip(evo::launch_project_bwd(pb, s),
                    "tri_attn_module_bwd/project_bwd");
  } catch (...) {
    return fail(EVO_EINTERNAL, "tri_attn_module_bwd: internal error");
  }
}

// ------------------------------------------- triangular multiplicative update

static evo_status_t check_opm_sizes(evo_dtype_t dtype, int64_t S, int64_t N,
                                    int64_t CM, int64_t C, int64_t CZ) {
  evo_status_t st = check_dtype(dtype);
  if (st != EVO_OK) return st;
  if (S <= 0 || N <= 0 || CM <= 0 || C <= 0 || CZ <= 0)
    return fail(EVO_EINVAL, "sizes must be positive (S=%lld N=%lld CM=%lld C=%lld CZ=%lld)",
                (long long)S, (long long)N, (long long)CM, (long long)C, (long long)CZ);
  if (S > INT32_MAX / N)  // sequence-residue positions are indexed in 32 bits
    return fail(EVO_ENOTSUP, "S*N=%lld*%lld is not supported (below 2^31)", (long long)S,
                (long long)N);
  if (CM % 32 != 0 || CM > 256)
    return fail(EVO_ENOTSUP, "CM=%lld must be a multiple of 32, at most 256", (long long)CM);
  if (CZ % 32 != 0 || CZ > 128 || C % 32 != 0 || C > 128)
    return fail(EVO_ENOTSUP, "CZ=%lld and C=%lld must be multiples of 32, at most "
                "128", (long long)CZ, (long long)C);
  if (N * C > 46340 || (N * C) * (N * C) > kMaxElems)  // product rows indexed in 32 bits
    return fail(EVO_ENOTSUP, "N*C=%lld is not supported (at most 46340)", (long long)(N * C));
  return EVO_OK;
}

static evo_status_t check_trimul_sizes(evo_dtype_t dtype, int64_t N, int64_t CZ,
                                       int64_t C) {
  evo_status_t st = check_dtype(dtype);
  if (st != EVO_OK) return st;
  if (N <= 0 || CZ <= 0 || C <= 0)
    return fail(EVO_EINVAL, "sizes must be positive (N=%lld CZ=%lld C=%lld)",
                (long long)N, (long long)CZ, (long long)C);
  if (N > 46340)  // N*N positions are indexed in 32 bits
    return fail(EVO_ENOTSUP, "N=%lld is not supported (at most 46340)", (long long)N);
  if (CZ % 32 != 0 || CZ > 128 || C % 32 != 0 || C > 128)
    return fail(EVO_ENOTSUP, "CZ=%lld and C=%lld must be multiples of 32, at most "
                "128", (long long)CZ, (long long)C);
  if (C * N * N > kMaxElems)
    return fail(EVO_ENOTSUP, "problem too large: tensors above 2^40 elements");
  return EVO_OK;
}

size_t tri_mul_workspace_bytes(evo_dtype_t dtype, int64_t N, int64_t CZ,
                               int64_t C) {
  const std::string saved = g_last_error;
  const evo_status_t st = check_trimul_sizes(dtype, N, CZ, C);
  g_last_error = saved;
  if (st != EVO_OK) return 0;
  return evo::trimul_workspace((int)dtype, N, C);
}

evo_status_t tri_mul_fwd(evo_dtype_t dtype, int64_t N, int64_t CZ, int64_t C,
                         int outgoing, const void* z,
                         const uint8_t* residue_mask, const void* ln_w,
                         const void* ln_b, float ln_eps, const void* w_a,
                         const void* w_b, const void* w_o, const void* b_o,
                         void* out, void* workspace, size_t workspace_bytes,
                         void* stream) {
  try {
    evo_status_t st = check_trimul_sizes(dtype, N, CZ, C);
    if (st != EVO_OK) return st;
    if (outgoing != 0 && outgoing != 1)
      return fail(EVO_EINVAL, "outgoing=%d must be 0 or 1", outgoing);
    if (!(ln_eps > 0.f)) return fail(EVO_EINVAL, "ln_eps must be > 0");
    REQUIRE_PTR(z);
    REQUIRE_PTR(ln_w);
    REQUIRE_PTR(ln_b);
    REQUIRE_PTR(w_a);
    REQUIRE_PTR(w_b);
    REQUIRE_PTR(w_o);
    REQUIRE_PTR(out);
    OPTIONAL_PTR(b_o);
    OPTIONAL_PTR(residue_mask);
    st = check_workspace("tri_mul_fwd", workspace, workspace_bytes,
                         evo::trimul_workspace((int)dtype, N, C));
    if (st != EVO_OK) return st;
    if (fault_injected()) return fail(EVO_EHIP, "tri_mul_fwd: injected launch failure");
    evo::TriMulArgs a{(int)dtype, N, CZ, C, outgoing, z, residue_mask, ln_w,
                      ln_b, ln_eps, w_a, w_b, w_o, b_o, out, workspace};
    return from_hip(evo::launch_trimul(a, (hipStream_t)stream), "tri_mul_fwd");
  } catch (...) {
    return fail(EVO_EINTERNAL, "tri_mul_fwd: internal error");
  }
}

size_t tri_mul_bwd_workspace_bytes(evo_dtype_t dtype, int64_t N, int64_t CZ,
                                   int64_t C) {
  const std::string saved = g_last_error;
  const evo_status_t st = check_trimul_sizes(dtype, N, CZ, C);
  g_last_error = saved;
  if (st != EVO_OK) return 0;
  return evo::trimul_bwd_workspace((int)dtype, N, CZ, C);
}

evo_status_t tri_mul_bwd(evo_dtype_t dtype, int64_t N, int64_t CZ, int64_t C,
                         int outgoing, const void* z,
                         const uint8_t* residue_mask, const void* ln_w,
                         const void* ln_b, float ln_eps, const void* w_a,
                         const void* w_b, const void* w_o, const void* dout,
                         void* dz, float* dln_w, float* dln_b, float* dw_a,
                         float* dw_b, float* dw_o, float* db_o, void* workspace,
                         size_t workspace_bytes, void* stream) {
  try {
    evo_status_t st = check_trimul_sizes(dtype, N, CZ, C);
    if (st != EVO_OK) return st;
    if (outgoing != 0 && outgoing != 1)
      return fail(EVO_EINVAL, "outgoing=%d must be 0 or 1", outgoing);
    if (!(ln_eps > 0.f)) return fail(EVO_EINVAL, "ln_eps must be > 0");
    REQUIRE_PTR(z);
    REQUIRE_PTR(ln_w);
    REQUIRE_PTR(ln_b);
    REQUIRE_PTR(w_a);
    REQUIRE_PTR(w_b);
    REQUIRE_PTR(w_o);
    REQUIRE_PTR(dout);
    REQUIRE_PTR(dz);
    REQUIRE_PTR(dln_w);
    REQUIRE_PTR(dln_b);
    REQUIRE_PTR(dw_a);
    REQUIRE_PTR(dw_b);
    REQUIRE_PTR(dw_o);
    REQUIRE_PTR(db_o);
    OPTIONAL_PTR(residue_mask);
    st = check_workspace("tri_mul_bwd", workspace, workspace_bytes,
                         evo::trimul_bwd_workspace((int)dtype, N, CZ, C));
    if (st != EVO_OK) return st;
    if (fault_injected()) return fail(EVO_EHIP, "tri_mul_bwd: injected launch failure");
    evo::TriMulBwdArgs a{(int)dtype, N, CZ, C, outgoing, z, residue_mask, ln_w, ln_b,
                         ln_eps, w_a, w_b, w_o, dout, dz, dln_w, dln_b, dw_a, dw_b,
                         dw_o, db_o, workspace};
    return from_hip(evo::launch_trimul_bwd(a, (hipStream_t)stream), "tri_mul_bwd");
  } catch (...) {
    return fail(EVO_EINTERNAL, "tri_mul_bwd: internal error");
  }
}

// ---------------------------------------------- LayerNorm + SwiGLU transition

static evo_status_t check_transition_sizes(evo_dtype_t dtype, int64_t N,
                                           int64_t CZ, int64_t HID) {
  evo_status_t st = check_dtype(dtype);
  if (st != EVO_OK) return st;
  if (N <= 0 || CZ <= 0 || HID <= 0)
    return fail(EVO_EINVAL, "sizes must be positive (N=%lld CZ=%lld HID=%lld)",
                (long long)N, (long long)CZ, (long long)HID);
  if (N > 46340)  // N*N positions are indexed in 32 bits
    return fail(EVO_ENOTSUP, "N=%lld is not supported (at most 46340)", (long long)N);
  if (CZ % 32 != 0 || CZ > 128)
    return fail(EVO_ENOTSUP, "CZ=%lld must be a multiple of 32, at most 128", (long long)CZ);
  if (HID % 64 != 0 || HID > 4096)
    return fail(EVO_ENOTSUP, "HID=%lld must be a multiple of 64, at most 4096",
                (long long)HID);
  return EVO_OK;
}

size_t pair_transition_workspace_bytes(evo_dtype_t dtype, int64_t N, int64_t CZ,
                                       int64_t HID) {
  const std::string saved = g_last_error;
  const evo_status_t st = check_transition_sizes(dtype, N, CZ, HID);
  g_last_error = saved;
  if (st != EVO_OK) return 0;
  return evo::transition_workspace((int)dtype, CZ, HID);
}

evo_status_t pair_transition_fwd(evo_dtype_t dtype, int64_t N, int64_t CZ,
                                 int64_t HID, const void* z, const void* ln_w,
                                 const void* ln_b, float ln_eps,
                                 const void* w_a, const void* w_b,
                                 const void* w_o, void* out, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  try {
    evo_status_t st = check_transition_sizes(dtype, N, CZ, HID);
    if (st != EVO_OK) return st;
    if (!(ln_eps > 0.f)) return fail(EVO_EINVAL, "ln_eps must be > 0");
    REQUIRE_PTR(z);
    REQUIRE_PTR(ln_w);
    REQUIRE_PTR(ln_b);
    REQUIRE_PTR(w_a);
    REQUIRE_PTR(w_b);
    REQUIRE_PTR(w_o);
    REQUIRE_PTR(out);
    st = check_workspace("pair_transition_fwd", workspace, workspace_bytes,
                         evo::transition_workspace((int)dtype, CZ, HID));
    if (st != EVO_OK) return st;
    if (fault_injected())
      return fail(EVO_EHIP, "pair_transition_fwd: injected launch failure");
    evo::TransitionArgs a{(int)dtype, N * N, CZ, HID, z, ln_w, ln_b, ln_eps,
                          w_a, w_b, w_o, out, workspace};
    return from_hip(evo::launch_transition(a, (hipStream_t)stream),
                    "pair_transition_fwd");
  } catch (...) {
    return fail(EVO_EINTERNAL, "pair_transition_fwd: internal error");
  }
}


size_t outer_product_mean_workspace_bytes(evo_dtype_t dtype, int64_t S, int64_t N,
                                          int64_t CM, int64_t C, int64_t CZ) {
  const std::string saved = g_last_error;
  const evo_status_t st = check_opm_sizes(dtype, S, N, CM, C, CZ);
  g_last_error = saved;
  if (st != EVO_OK) return 0;
  return evo::opm_workspace((int)dtype, S, N, C);
}

evo_status_t outer_product_mean_fwd(evo_dtype_t dtype, int64_t S, int64_t N, int64_t CM,
                                    int64_t C, int64_t CZ, const void* m, const void* ln_w,
                                    const void* ln_b, float ln_eps, const void* w_a,
                                    const void* w_b, const void* w_o, const void* b_o,
                                    void* out, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  try {
    evo_status_t st = check_opm_sizes(dtype, S, N, CM, C, CZ);
    if (st != EVO_OK) return st;
    if (!(ln_eps > 0.f)) return fail(EVO_EINVAL, "ln_eps must be > 0");
    REQUIRE_PTR(m);
    REQUIRE_PTR(ln_w);
    REQUIRE_PTR(ln_b);
    REQUIRE_PTR(w_a);
    REQUIRE_PTR(w_b);
    REQUIRE_PTR(w_o);
    REQUIRE_PTR(out);
    OPTIONAL_PTR(b_o);
    st = check_workspace("outer_product_mean_fwd", workspace, workspace_bytes,
                         evo::opm_workspace((int)dtype, S, N, C));
    if (st != EVO_OK) return st;
    if (fault_injected())
      return fail(EVO_EHIP, "outer_product_mean_fwd: injected launch failure");
    evo::OpmArgs a{(int)dtype, S, N, CM, C, CZ, m, ln_w, ln_b, ln_eps,
                   w_a, w_b, w_o, b_o, out, workspace};
    return from_hip(evo::launch_opm(a, (hipStream_t)stream), "outer_product_mean_fwd");
  } catch (...) {
    return fail(EVO_EINTERNAL, "outer_product_mean_fwd: internal error");
  }
}

size_t outer_product_mean_bwd_workspace_bytes(evo_dtype_t dtype, int64_t S, int64_t N,
                                              int64_t CM, int64_t C, int64_t CZ) {
  const std::string saved = g_last_error;
  evo_status_t st = check_opm_sizes(dtype, S, N, CM, C, CZ);
  if (st == EVO_OK && CM > 128 && CM != 256) st = EVO_ENOTSUP;
  g_last_error = saved;
  if (st != EVO_OK) return 0;
  return evo::opm_bwd_workspace((int)dtype, S, N, CM, C, CZ);
}

evo_status_t outer_product_mean_bwd(evo_dtype_t dtype, int64_t S, int64_t N, int64_t CM,
                                    int64_t C, int64_t CZ, const void* m, const void* ln_w,
                                    const void* ln_b, float ln_eps, const void* w_a,
                                    const void* w_b, const void* w_o, const void* dout,
                                    void* dm, float* dln_w, float* dln_b, float* dw_a,
                                    float* dw_b, float* dw_o, float* db_o, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  try {
    evo_status_t st = check_opm_sizes(dtype, S, N, CM, C, CZ);
    if (st != EVO_OK) return st;
    if (CM > 128 && CM != 256)
      return fail(EVO_ENOTSUP, "outer_product_mean_bwd: CM=%lld must be at most 128, or 256",
                  (long long)CM);
    if (!(ln_eps > 0.f)) return fail(EVO_EINVAL, "ln_eps must be > 0");
    REQUIRE_PTR(m);
    REQUIRE_PTR(ln_w);
    REQUIRE_PTR(ln_b);
    REQUIRE_PTR(w_a);
    REQUIRE_PTR(w_b);
    REQUIRE_PTR(w_o);
    REQUIRE_PTR(dout);
    REQUIRE_PTR(dm);
    REQUIRE_PTR(dln_w);
    REQUIRE_PTR(dln_b);
    REQUIRE_PTR(dw_a);
    REQUIRE_PTR(dw_b);
    REQUIRE_PTR(dw_o);
    REQUIRE_PTR(db_o);
    st = check_workspace("outer_product_mean_bwd", workspace, workspace_bytes,
                         evo::opm_bwd_workspace((int)dtype, S, N, CM, C, CZ));
    if (st != EVO_OK) return st;
    if (fault_injected())
      return fail(EVO_EHIP, "outer_product_mean_bwd: injected launch failure");
    evo::OpmBwdArgs a{(int)dtype, S, N, CM, C, CZ, m, ln_w, ln_b, ln_eps, w_a, w_b, w_o,
                      dout, dm, dln_w, dln_b, dw_a, dw_b, dw_o, db_o, workspace};
    return from_hip(evo::launch_opm_bwd(a, (hipStream_t)stream), "outer_product_mean_bwd");
  } catch (...) {
    return fail(EVO_EINTERNAL, "outer_product_mean_bwd: internal error");
  }
}

static evo_status_t check_transition_bwd_sizes(evo_dtype_t dtype, int64_t N, int64_t CZ,
                                               int64_t HID) {
  evo_status_t st = check_transition_sizes(dtype, N, CZ, HID);
  if (st != EVO_OK) return st;
  if (HID % 128 != 0)
    return fail(EVO_ENOTSUP, "HID=%lld must be a multiple of 128 for the backward",
                (long long)HID);
  return EVO_OK;
}

size_t pair_transition_bwd_workspace_bytes(evo_dtype_t dtype, int64_t N, int64_t CZ,
                                           int64_t HID) {
  const std::string saved = g_last_error;
  const evo_status_t st = check_transition_bwd_sizes(dtype, N, CZ, HID);
  g_last_error = saved;
  if (st != EVO_OK) return 0;
  return evo::transition_bwd_workspace((int)dtype, N * N, CZ, HID);
}

evo_status_t pair_transition_bwd(evo_dtype_t dtype, int64_t N, int64_t CZ, int64_t HID,
                                 const void* z, const void* ln_w, const void* ln_b,
                                 float ln_eps, const void* w_a, const void* w_b,
                                 const void* w_o, const void* dout, void* dz, float* dln_w,
                                 float* dln_b, float* dw_a, float* dw_b, float* dw_o,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  try {
    evo_status_t st = check_transition_bwd_sizes(dtype, N, CZ, HID);
    if (st != EVO_OK) return st;
    if (!(ln_eps > 0.f)) return fail(EVO_EINVAL, "ln_eps must be > 0");
    REQUIRE_PTR(z);
    REQUIRE_PTR(ln_w);
    REQUIRE_PTR(ln_b);
    REQUIRE_PTR(w_a);
    REQUIRE_PTR(w_b);
    REQUIRE_PTR(w_o);
    REQUIRE_PTR(dout);
    REQUIRE_PTR(dz);
    REQUIRE_PTR(dln_w);
    REQUIRE_PTR(dln_b);
    REQUIRE_PTR(dw_a);
    REQUIRE_PTR(dw_b);
    REQUIRE_PTR(dw_o);
    st = check_workspace("pair_transition_bwd", workspace, workspace_bytes,
                         evo::transition_bwd_workspace((int)dtype, N * N, CZ, HID));
    if (st != EVO_OK) return st;
    if (fault_injected())
      return fail(EVO_EHIP, "pair_transition_bwd: injected launch failure");
    evo::TransitionBwdArgs a{(int)dtype, N * N, CZ, HID, z, ln_w, ln_b, ln_eps, w_a, w_b,
                             w_o, dout, dz, dln_w, dln_b, dw_a, dw_b, dw_o, workspace};
    return from_hip(evo::launch_transition_bwd(a, (hipStream_t)stream), "pair_transition_bwd");
  } catch (...) {
    return fail(EVO_EINTERNAL, "pair_transition_bwd: internal error");
  }
}

}  // extern "C"
