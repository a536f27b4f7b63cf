// kda_launch.hpp -- internal launcher interface between the C ABI (kda_abi.cpp)
// and the kernels.  Host-side plain structs; arguments are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

// Raises `kernel`'s dynamic-LDS limit to at least `bytes` on the calling thread's
// current device.  The attribute is set once per (kernel, device) for the life of
// the process, under a lock, so host threads that make their first calls at the
// same time, or calls on several devices, each find it set before they launch.
hipError_t ensure_dynamic_lds(const void* kernel, size_t bytes);
// number of compute units of the calling thread's current device (queried once per device)
hipError_t device_cus(int* cus);

struct RowsLaunch {
  int H, dk, dv, in_dtype, act, gate_mode, batch, window;
  float lb;
  const int32_t* slots;
  float* state;
  void* conv_state;
  const float* conv_w;
  const void *q, *k, *v, *g, *beta;
  float* o;
  const int32_t* n_commit;
  const float *in_a, *in_k, *in_u;
  const void* in_rows;
  int in_window;
  float *out_a, *out_k, *out_u;
  void* out_rows;
  int g_per_head = 0;  // raw g rows [B, (window,) H]
  const int32_t* window_lens = nullptr;  // verify: rows per sequence, NULL = window
};
hipError_t launch_rows(const RowsLaunch& L, bool verify, hipStream_t s);

struct NormLaunch {
  int64_t rows;
  int dv, z_dtype, y_dtype;
  const float* o;
  const void* z;
  const float* w;
  float eps;
  void* y;
  // optional (prompt epilogue): rows are [t_tot, H]; with slots given, the rows of a
  // sequence whose slot is negative are left alone
  const int32_t* cu = nullptr;
  const int32_t* slots = nullptr;
  int num_seqs = 0, H = 1;
};
hipError_t launch_gated_rmsnorm(const NormLaunch& L, hipStream_t s);

struct PrepLaunch {
  int H, dk, dv, in_dtype, act, gate_mode, num_seqs;
  int64_t t_tot;
  float lb;
  const int32_t *cu_seqlens, *slots;
  const void *q, *k, *v, *g, *beta;
  const float* conv_w;
  const void* cs_in;
  void* cs_out;
  float *q_hat, *k_hat, *v_out, *g_out, *beta_out;
  int g_per_head = 0;  // raw g rows [T, H]: one decay per head, broadcast over d_k
};
hipError_t launch_prep(const PrepLaunch& L, hipStream_t s);

struct PrefillLaunch {
  int H, dk, dv, precision, num_seqs;
  int64_t t_tot;
  const int32_t *cu_seqlens, *slots;
  const float *q_hat, *k_hat, *v, *g, *beta;
  float* state;
  float* o;
  void* workspace;
  size_t workspace_bytes;
  // fused preamble (fused != 0): raw rows and conv / gate parameters
  int fused, in_dtype, act, gate_mode;
  float lb;
  const void *raw_q, *raw_k, *raw_v, *raw_g, *raw_beta;
  const float* conv_w;
  const void* cs_in;
  void* cs_out;
  // measurement hook: events[2i], events[2i+1] around kernel i (2i+1 < nevents)
  hipEvent_t* events;
  int nevents;
  int g_per_head = 0;  // raw g rows [T, H] (fused preamble)
};
size_t prefill_workspace_bytes(int H, int dk, int dv, int precision, int num_seqs, int64_t t_tot);
hipError_t launch_prefill(const PrefillLaunch& L, hipStream_t s);

// Scratch of the allocation-free prompt call: a device array of this many bytes, one per
// device; noalloc_scratch gives its address on the calling thread's current device
// (resolved on the first call on each device and kept for the life of the process).
constexpr size_t kNoAllocScratchBytes = (size_t)160 << 20;
hipError_t noalloc_scratch(void** ptr);

}  // namespace kda
