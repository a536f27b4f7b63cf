// kda_abi.cpp -- the C ABI declared in include/kda.h: argument validation
// (before any launch, so an error enqueues nothing and writes nothing) and
// dispatch to the gfx950 kernels.  TensorFold issue #850 asks the shared KDA
// module to reject unsupported head widths and tap counts before launch; the
// checks here do that for every entry point.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <map>
#include <mutex>
#include <utility>

#include "kda.h"
#include "kda_launch.hpp"

namespace {

thread_local char g_err[512] = "";
thread_local hipEvent_t* g_events = nullptr;  // measurement hook (kda_set_timing_events)
thread_local int g_nevents = 0;

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return KDA_OK;
}

// Limits that keep every launch within a grid's extents: heads go on a grid axis of
// at most 65535, and the prompt path's workgroup counts (one per (record slot, head),
// one per 16 rows of the norm) on an axis of at most 2^31 - 1.
constexpr int kMaxHeads = 65535;
constexpr int64_t kMaxGridX = 2147483647;

int check_rows(const char* what, const kda_dims* d, int32_t num_seqs, int64_t t_tot) {
  if (t_tot > 2147483647) return fail(KDA_E_ARG, "%s: %lld rows exceed the int32 range of cu_seqlens", what,
                                      (long long)t_tot);
  const int64_t records = t_tot / 64 + num_seqs;  // record slots of the prompt path
  if (records * d->num_heads > kMaxGridX || (t_tot * d->num_heads) / 16 > kMaxGridX)
    return fail(KDA_E_ARG, "%s: %lld rows x %d heads exceed the launch grid", what, (long long)t_tot, d->num_heads);
  return KDA_OK;
}

bool aligned(const void* p, unsigned a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1u)) == 0; }
unsigned elem_bytes(int32_t dtype) { return dtype == KDA_DTYPE_BF16 ? 2u : 4u; }

int check_dims(const kda_dims* d) {
  if (!d) return fail(KDA_E_ARG, "dims is NULL");
  if (d->num_heads < 1) return fail(KDA_E_ARG, "num_heads must be >= 1 (got %d)", d->num_heads);
  if (d->num_heads > kMaxHeads)
    return fail(KDA_E_GEOMETRY, "num_heads %d unsupported: at most %d", d->num_heads, kMaxHeads);
  if (!((d->head_dim_k == 64 || d->head_dim_k == 128) && (d->head_dim_v == 64 || d->head_dim_v == 128)))
    return fail(KDA_E_GEOMETRY, "head dims (%d, %d) unsupported: d_k and d_v must be 64 or 128", d->head_dim_k,
                d->head_dim_v);
  if (d->conv_width != 4) return fail(KDA_E_GEOMETRY, "conv width %d unsupported: must be 4", d->conv_width);
  if (d->in_dtype != KDA_DTYPE_F32 && d->in_dtype != KDA_DTYPE_BF16)
    return fail(KDA_E_DTYPE, "unknown in_dtype %d", d->in_dtype);
  if (d->conv_act != KDA_ACT_NONE && d->conv_act != KDA_ACT_SILU)
    return fail(KDA_E_DTYPE, "unknown conv_act %d", d->conv_act);
  if (d->precision != KDA_PREC_FP32 && d->precision != KDA_PREC_BF16X3 && d->precision != KDA_PREC_FP16 &&
      d->precision != KDA_PREC_BF16X2)
    return fail(KDA_E_DTYPE, "unknown precision %d", d->precision);
  if (d->decay_shape != KDA_DECAY_PER_DIM && d->decay_shape != KDA_DECAY_PER_HEAD)
    return fail(KDA_E_GEOMETRY, "unknown decay shape %d", d->decay_shape);
  return KDA_OK;
}

int check_gate(int32_t gate_mode, float lb) {
  if (gate_mode == KDA_GATE_SOFTPLUS) return KDA_OK;  // the bound is ignored outside safe mode
  if (gate_mode != KDA_GATE_SAFE) return fail(KDA_E_GATE, "unknown gate mode %d", gate_mode);
  if (!std::isfinite(lb) || !(lb < 0.0f))
    return fail(KDA_E_GATE, "safe gate needs a finite lower bound < 0 (got %g)", (double)lb);
  return KDA_OK;
}

// all listed pointers non-null and aligned to `align` bytes (16 where the
// kernels use 128-bit accesses, else the element size)
int check_ptrs(const char* what, std::initializer_list<const void*> ps, unsigned align = 16) {
  int i = 0;
  for (const void* p : ps) {
    if (!p) return fail(KDA_E_ARG, "%s: pointer argument %d is NULL", what, i);
    if (!aligned(p, align)) return fail(KDA_E_ALIGN, "%s: pointer argument %d is not %u-byte aligned", what, i, align);
    ++i;
  }
  return KDA_OK;
}

int check_opt_ptr(const char* what, const void* p) {
  if (p && !aligned(p, 4)) return fail(KDA_E_ALIGN, "%s is not 4-byte aligned", what);
  return KDA_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(KDA_E_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

#define KDA_TRY(expr)          \
  do {                         \
    const int rc_ = (expr);    \
    if (rc_ != KDA_OK) return rc_; \
  } while (0)

}  // namespace

namespace kda {

hipError_t ensure_dynamic_lds(const void* kernel, size_t bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  static std::mutex mu;
  static std::map<std::pair<const void*, int>, size_t> set_to;  // (kernel, device) -> bytes allowed
  std::lock_guard<std::mutex> lock(mu);
  size_t& have = set_to[std::make_pair(kernel, dev)];
  if (have >= bytes) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess) have = bytes;
  return e;
}

hipError_t device_cus(int* cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  static std::mutex mu;
  static std::map<int, int> known;
  std::lock_guard<std::mutex> lock(mu);
  auto it = known.find(dev);
  if (it == known.end()) {
    int n = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    it = known.emplace(dev, n > 0 ? n : 1).first;
  }
  *cus = it->second;
  return hipSuccess;
}

static_assert(kNoAllocScratchBytes == KDA_NOALLOC_SCRATCH_BYTES, "scratch size as the header states it");

}  // namespace kda

extern "C" {

const char* kda_last_error(void) { return g_err; }

int kda_set_timing_events(hipEvent_t* events, int32_t count) {
  if (count < 0 || (count & 1)) return fail(KDA_E_ARG, "kda_set_timing_events: count must be even and >= 0");
  if (count > 0 && !events) return fail(KDA_E_ARG, "kda_set_timing_events: NULL events");
  g_events = count > 0 ? events : nullptr;
  g_nevents = count > 0 ? count : 0;
  return ok();
}

int kda_prep(const kda_dims* d, int32_t num_seqs, int64_t t_tot, const int32_t* cu_seqlens, const int32_t* slots,
             const void* q_raw, const void* k_raw, const void* v_raw, const float* conv_weight,
             const void* conv_state_in, void* conv_state_out, const void* g_raw, const void* beta_logit,
             int32_t gate_mode, float lower_bound, float* q_hat, float* k_hat, float* v_out, float* g_out,
             float* beta_out, hipStream_t stream) {
  KDA_TRY(check_dims(d));
  KDA_TRY(check_gate(gate_mode, lower_bound));
  if (num_seqs < 0 || t_tot < 0) return fail(KDA_E_ARG, "kda_prep: negative size");
  if (num_seqs == 0 && t_tot > 0) return fail(KDA_E_ARG, "kda_prep: rows without sequences");
  KDA_TRY(check_rows("kda_prep", d, num_seqs, t_tot));
  KDA_TRY(check_opt_ptr("kda_prep: slots", slots));
  const unsigned eb = elem_bytes(d->in_dtype);
  if (num_seqs > 0) {
    KDA_TRY(check_ptrs("kda_prep", {cu_seqlens, conv_weight}, 4));
    KDA_TRY(check_ptrs("kda_prep: conv state", {conv_state_in, conv_state_out}, eb));
  }
  if (t_tot > 0) {
    KDA_TRY(check_ptrs("kda_prep: q/k/v/g rows", {q_raw, k_raw, v_raw, g_raw}));
    KDA_TRY(check_ptrs("kda_prep: beta logits", {beta_logit}, eb));
    KDA_TRY(check_ptrs("kda_prep: outputs", {q_hat, k_hat, v_out, g_out}));
    KDA_TRY(check_ptrs("kda_prep: beta out", {beta_out}, 4));
  }
  kda::PrepLaunch L{d->num_heads, d->head_dim_k, d->head_dim_v, d->in_dtype, d->conv_act, gate_mode, num_seqs, t_tot,
                    lower_bound, cu_seqlens, slots, q_raw, k_raw, v_raw, g_raw, beta_logit, conv_weight,
                    conv_state_in, conv_state_out, q_hat, k_hat, v_out, g_out, beta_out};
  L.g_per_head = d->decay_shape == KDA_DECAY_PER_HEAD;
  return hip_status(kda::launch_prep(L, stream), "kda_prep");
}

size_t kda_prefill_workspace_bytes(const kda_dims* d, int32_t num_seqs, int64_t t_tot) {
  if (check_dims(d) != KDA_OK || num_seqs < 0 || t_tot < 0) return 0;
  return kda::prefill_workspace_bytes(d->num_heads, d->head_dim_k, d->head_dim_v, d->precision, num_seqs, t_tot);
}

// kda_prefill_varlen and its allocation-free variant: the same validation and launches; the
// variant takes the chunk records' scratch from the library's per-device array instead of the
// caller's workspace (noalloc, with workspace NULL on entry).
static int prefill_call(const char* fn, const kda_dims* d, int32_t num_seqs, int64_t t_tot, const int32_t* cu_seqlens,
                        const int32_t* slots, const float* q_hat, const float* k_hat, const float* v, const float* g,
                        const float* beta, const kda_raw_rows* raw, const kda_norm_args* norm, float* state, float* o,
                        void* workspace, size_t workspace_bytes, bool noalloc, hipStream_t stream) {
  KDA_TRY(check_dims(d));
  if (num_seqs < 0 || t_tot < 0) return fail(KDA_E_ARG, "%s: negative size", fn);
  KDA_TRY(check_rows(fn, d, num_seqs, t_tot));
  if (norm) {
    if ((norm->z_dtype != KDA_DTYPE_F32 && norm->z_dtype != KDA_DTYPE_BF16) ||
        (norm->y_dtype != KDA_DTYPE_F32 && norm->y_dtype != KDA_DTYPE_BF16))
      return fail(KDA_E_DTYPE, "%s: unknown norm z or y dtype", fn);
    if (!(norm->eps >= 0.0f) || !std::isfinite(norm->eps))
      return fail(KDA_E_ARG, "%s: norm eps must be finite and >= 0", fn);
    if (t_tot > 0) KDA_TRY(check_ptrs("prompt call: norm z/weight/y", {norm->z, norm->weight, norm->y}));
  }
  if (num_seqs == 0 && t_tot > 0) return fail(KDA_E_ARG, "%s: rows without sequences", fn);
  KDA_TRY(check_opt_ptr("prompt call: slots", slots));
  if (raw) KDA_TRY(check_gate(raw->gate_mode, raw->lower_bound));
  const unsigned eb = elem_bytes(d->in_dtype);
  if (num_seqs > 0) {
    KDA_TRY(check_ptrs("prompt call: cu_seqlens", {cu_seqlens}, 4));
    KDA_TRY(check_ptrs("prompt call: state", {state}));
    if (raw) {
      KDA_TRY(check_ptrs("prompt call: raw conv weight", {raw->conv_weight}, 4));
      KDA_TRY(check_ptrs("prompt call: raw conv state", {raw->conv_state_in, raw->conv_state_out}, eb));
    }
  }
  if (t_tot > 0) {
    if (raw) {
      KDA_TRY(check_ptrs("prompt call: raw q/k/v/g rows", {raw->q_raw, raw->k_raw, raw->v_raw, raw->g_raw}));
      KDA_TRY(check_ptrs("prompt call: raw beta logits", {raw->beta_logit}, eb));
    } else {
      KDA_TRY(check_ptrs("prompt call", {q_hat, k_hat, v, g}));
      KDA_TRY(check_ptrs("prompt call", {beta}, 4));
    }
    KDA_TRY(check_ptrs("prompt call: o", {o}));
  }
  const size_t need =
      kda::prefill_workspace_bytes(d->num_heads, d->head_dim_k, d->head_dim_v, d->precision, num_seqs, t_tot);
  if (num_seqs > 0 && noalloc) {
    if (need > kda::kNoAllocScratchBytes)
      return fail(KDA_E_WORKSPACE, "%s: this call needs %zu bytes of scratch, more than the %zu the library holds "
                  "per device; use kda_prefill_varlen with a workspace", fn, need, kda::kNoAllocScratchBytes);
    KDA_TRY(hip_status(kda::noalloc_scratch(&workspace), fn));
    workspace_bytes = kda::kNoAllocScratchBytes;
  }
  if (num_seqs > 0) {
    if (!workspace || workspace_bytes < need)
      return fail(KDA_E_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                  workspace ? workspace_bytes : (size_t)0);
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
      return fail(KDA_E_ALIGN, "%s: workspace must be 256-byte aligned", fn);
  }
  if (num_seqs == 0) return ok();
  kda::PrefillLaunch L{};
  L.H = d->num_heads; L.dk = d->head_dim_k; L.dv = d->head_dim_v; L.precision = d->precision;
  L.num_seqs = num_seqs; L.t_tot = t_tot; L.cu_seqlens = cu_seqlens; L.slots = slots;
  L.q_hat = q_hat; L.k_hat = k_hat; L.v = v; L.g = g; L.beta = beta; L.state = state; L.o = o;
  L.workspace = workspace; L.workspace_bytes = workspace_bytes;
  L.in_dtype = d->in_dtype; L.act = d->conv_act;
  L.events = g_events; L.nevents = g_nevents;
  if (raw) {
    L.fused = 1; L.gate_mode = raw->gate_mode; L.lb = raw->lower_bound;
    L.g_per_head = d->decay_shape == KDA_DECAY_PER_HEAD;
    L.raw_q = raw->q_raw; L.raw_k = raw->k_raw; L.raw_v = raw->v_raw; L.raw_g = raw->g_raw;
    L.raw_beta = raw->beta_logit; L.conv_w = raw->conv_weight; L.cs_in = raw->conv_state_in;
    L.cs_out = raw->conv_state_out;
  }
  KDA_TRY(hip_status(kda::launch_prefill(L, stream), fn));
  if (norm && t_tot > 0) {
    kda::NormLaunch N{t_tot * d->num_heads, d->head_dim_v, norm->z_dtype, norm->y_dtype, o, norm->z, norm->weight,
                      norm->eps, norm->y};
    N.cu = cu_seqlens; N.slots = slots; N.num_seqs = num_seqs; N.H = d->num_heads;
    const bool timed = g_nevents >= 6;
    if (timed) KDA_TRY(hip_status(hipEventRecord(g_events[4], stream), fn));
    KDA_TRY(hip_status(kda::launch_gated_rmsnorm(N, stream), fn));
    if (timed) KDA_TRY(hip_status(hipEventRecord(g_events[5], stream), fn));
  }
  return ok();
}

int kda_prefill_varlen(const kda_dims* d, int32_t num_seqs, int64_t t_tot, const int32_t* cu_seqlens,
                       const int32_t* slots, const float* q_hat, const float* k_hat, const float* v,
                       const float* g, const float* beta, const kda_raw_rows* raw, const kda_norm_args* norm,
                       float* state, float* o, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return prefill_call("kda_prefill_varlen", d, num_seqs, t_tot, cu_seqlens, slots, q_hat, k_hat, v, g, beta, raw,
                      norm, state, o, workspace, workspace_bytes, false, stream);
}

int kda_prefill_varlen_noalloc(const kda_dims* d, int32_t num_seqs, int64_t t_tot, const int32_t* cu_seqlens,
                               const int32_t* slots, const float* q_hat, const float* k_hat, const float* v,
                               const float* g, const float* beta, const kda_raw_rows* raw, const kda_norm_args* norm,
                               float* state, float* o, hipStream_t stream) {
  return prefill_call("kda_prefill_varlen_noalloc", d, num_seqs, t_tot, cu_seqlens, slots, q_hat, k_hat, v, g, beta,
                      raw, norm, state, o, nullptr, 0, true, stream);
}

int kda_decode(const kda_dims* d, int32_t batch, const int32_t* slots, float* state, void* conv_state,
               const float* conv_weight, const void* q_raw, const void* k_raw, const void* v_raw, const void* g_raw,
               const void* beta_logit, int32_t gate_mode, float lower_bound, float* o, hipStream_t stream) {
  KDA_TRY(check_dims(d));
  KDA_TRY(check_gate(gate_mode, lower_bound));
  if (batch < 0) return fail(KDA_E_ARG, "kda_decode: negative batch");
  if (batch == 0) return ok();
  KDA_TRY(check_opt_ptr("kda_decode: slots", slots));
  KDA_TRY(check_ptrs("kda_decode", {state, o}));
  KDA_TRY(check_ptrs("kda_decode: conv weight", {conv_weight}, 4));
  KDA_TRY(check_ptrs("kda_decode: rows", {conv_state, q_raw, k_raw, v_raw, g_raw, beta_logit}, elem_bytes(d->in_dtype)));
  kda::RowsLaunch L{};
  L.H = d->num_heads; L.dk = d->head_dim_k; L.dv = d->head_dim_v; L.in_dtype = d->in_dtype; L.act = d->conv_act;
  L.g_per_head = d->decay_shape == KDA_DECAY_PER_HEAD;
  L.gate_mode = gate_mode; L.batch = batch; L.window = 1; L.lb = lower_bound; L.slots = slots; L.state = state;
  L.conv_state = conv_state; L.conv_w = conv_weight; L.q = q_raw; L.k = k_raw; L.v = v_raw; L.g = g_raw;
  L.beta = beta_logit; L.o = o;
  return hip_status(kda::launch_rows(L, false, stream), "kda_decode");
}

int kda_verify_window(const kda_dims* d, int32_t batch, int32_t window, const int32_t* window_lens,
                      const int32_t* slots, float* state,
                      void* conv_state, const float* conv_weight, const int32_t* n_commit, const kda_log* log_in,
                      const kda_log* log_out, const void* q_raw, const void* k_raw, const void* v_raw,
                      const void* g_raw, const void* beta_logit, int32_t gate_mode, float lower_bound, float* o,
                      hipStream_t stream) {
  KDA_TRY(check_dims(d));
  KDA_TRY(check_gate(gate_mode, lower_bound));
  if (batch < 0) return fail(KDA_E_ARG, "kda_verify_window: negative batch");
  if (window < 0 || window > 8) return fail(KDA_E_GEOMETRY, "kda_verify_window: window %d not in [0, 8]", window);
  const bool commit = n_commit != nullptr;
  if (commit && !log_in) return fail(KDA_E_ARG, "kda_verify_window: n_commit given without log_in");
  if (commit && (log_in->window < 0 || log_in->window > 8))
    return fail(KDA_E_GEOMETRY, "kda_verify_window: log_in window %d not in [0, 8]", log_in->window);
  if (window > 0 && !log_out) return fail(KDA_E_ARG, "kda_verify_window: window rows need log_out");
  if (window > 0 && log_out->window != window)
    return fail(KDA_E_GEOMETRY, "kda_verify_window: log_out sized for %d rows, window is %d", log_out->window, window);
  if (batch == 0) return ok();
  KDA_TRY(check_opt_ptr("kda_verify_window: slots", slots));
  KDA_TRY(check_opt_ptr("kda_verify_window: window_lens", window_lens));
  const unsigned eb = elem_bytes(d->in_dtype);
  KDA_TRY(check_ptrs("kda_verify_window: state", {state}));
  KDA_TRY(check_ptrs("kda_verify_window: conv weight", {conv_weight}, 4));
  KDA_TRY(check_ptrs("kda_verify_window: conv state", {conv_state}, eb));
  if (commit) {
    KDA_TRY(check_ptrs("kda_verify_window: n_commit", {n_commit}, 4));
    if (log_in->window > 0) {
      KDA_TRY(check_ptrs("kda_verify_window: log_in", {log_in->a, log_in->k_hat}, 4));
      KDA_TRY(check_ptrs("kda_verify_window: log_in u", {log_in->u}));
      KDA_TRY(check_ptrs("kda_verify_window: log_in rows", {log_in->conv_rows}, eb));
    }
  }
  if (window > 0) {
    KDA_TRY(check_ptrs("kda_verify_window: rows", {q_raw, k_raw, v_raw, g_raw, beta_logit}, eb));
    KDA_TRY(check_ptrs("kda_verify_window: o", {o}));
    KDA_TRY(check_ptrs("kda_verify_window: log_out", {log_out->a, log_out->k_hat}, 4));
    KDA_TRY(check_ptrs("kda_verify_window: log_out u", {log_out->u}));
    KDA_TRY(check_ptrs("kda_verify_window: log_out rows", {log_out->conv_rows}, eb));
    if (commit && log_in->window > 0 &&
        (log_in->a == log_out->a || log_in->k_hat == log_out->k_hat || log_in->u == log_out->u ||
         log_in->conv_rows == log_out->conv_rows))
      return fail(KDA_E_ARG, "kda_verify_window: log_in and log_out must not share buffers");
  }
  if (!commit && window == 0) return ok();
  kda::RowsLaunch L{};
  L.H = d->num_heads; L.dk = d->head_dim_k; L.dv = d->head_dim_v; L.in_dtype = d->in_dtype; L.act = d->conv_act;
  L.g_per_head = d->decay_shape == KDA_DECAY_PER_HEAD;
  L.gate_mode = gate_mode; L.batch = batch; L.window = window; L.lb = lower_bound; L.slots = slots; L.state = state;
  L.conv_state = conv_state; L.conv_w = conv_weight; L.q = q_raw; L.k = k_raw; L.v = v_raw; L.g = g_raw;
  L.beta = beta_logit; L.o = o;
  L.n_commit = n_commit; L.window_lens = window > 0 ? window_lens : nullptr;
  if (commit) {
    L.in_a = log_in->a; L.in_k = log_in->k_hat; L.in_u = log_in->u; L.in_rows = log_in->conv_rows;
    L.in_window = log_in->window;
  }
  if (window > 0) {
    L.out_a = log_out->a; L.out_k = log_out->k_hat; L.out_u = log_out->u; L.out_rows = log_out->conv_rows;
  }
  return hip_status(kda::launch_rows(L, true, stream), "kda_verify_window");
}

int gated_rmsnorm_out(int64_t rows, int32_t d_v, const float* o, const void* z, int32_t z_dtype, const float* w,
                      float eps, void* y, int32_t y_dtype, hipStream_t stream) {
  if (rows < 0) return fail(KDA_E_ARG, "gated_rmsnorm_out: negative rows");
  if (rows / 16 > kMaxGridX) return fail(KDA_E_ARG, "gated_rmsnorm_out: %lld rows exceed the launch grid", (long long)rows);
  if (d_v != 64 && d_v != 128) return fail(KDA_E_GEOMETRY, "gated_rmsnorm_out: d_v %d not in {64, 128}", d_v);
  if ((z_dtype != KDA_DTYPE_F32 && z_dtype != KDA_DTYPE_BF16) || (y_dtype != KDA_DTYPE_F32 && y_dtype != KDA_DTYPE_BF16))
    return fail(KDA_E_DTYPE, "gated_rmsnorm_out: unknown dtype");
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return fail(KDA_E_ARG, "gated_rmsnorm_out: eps must be finite and >= 0");
  if (rows == 0) return ok();
  KDA_TRY(check_ptrs("gated_rmsnorm_out", {o, z, w, y}));
  kda::NormLaunch L{rows, d_v, z_dtype, y_dtype, o, z, w, eps, y};
  return hip_status(kda::launch_gated_rmsnorm(L, stream), "gated_rmsnorm_out");
}

}  // extern "C"
