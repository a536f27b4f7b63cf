// kda_prep.hip -- preamble of the prompt path for packed varlen rows (gfx950).
//
// TensorFold issue #850 (shared KDA module: conv window, safe or softplus gate,
// beta, q/k L2 norms) and onnxruntime-genai PR #2843 (VarlenCausalConvWithState,
// GatedDeltaNet gate with gate_activation='sigmoid' and gate_lower_bound):
//   conv: c_t = sum_{j<4} w[c][j] x_{t-3+j}  (rows before a sequence's first row
//         come from its carried conv state), then SiLU;
//   q_hat = c_q / sqrt(|c_q|^2 + 1e-6), k_hat likewise, v = c_v;
//   g = -softplus(x_g) or lb * sigmoid(x_g);  beta = sigmoid(x_b).
// One wavefront per (row, head); each lane owns d/64 consecutive channels of q,
// k, g and v, so every load and store is coalesced.  The carried conv state is
// written by a second launch after every read of the old one, which lets the
// caller pass the same buffer for input and output.
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

template <typename RawT>
struct PrepArgs {
  int H, act, gate_mode, num_seqs;
  int64_t t_tot;
  float lb;
  const int32_t *cu, *slots;
  const RawT *q, *k, *v, *g, *beta;
  const float* conv_w;
  const RawT* cs_in;
  RawT* cs_out;
  float *q_hat, *k_hat, *v_out, *g_out, *beta_out;
  int g_per_head;  // raw g rows [T, H]: one decay per head and row, broadcast over d_k
};

// sequence n such that cu[n] <= row < cu[n+1] (cu non-decreasing; zero-length
// sequences are skipped by taking the last n with cu[n] <= row)
__device__ __forceinline__ int find_seq(const int32_t* cu, int num_seqs, int64_t row) {
  int lo = 0, hi = num_seqs;  // invariant: cu[lo] <= row < cu[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if ((int64_t)cu[mid] <= row) lo = mid; else hi = mid;
  }
  return lo;
}

template <int DK, int DV, typename RawT>
__global__ __launch_bounds__(256) void prep_kernel(PrepArgs<RawT> p) {
  constexpr int EK = DK / 64, EV = DV / 64;  // channels per lane
  const int lane = threadIdx.x & 63;
  const int64_t pair = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int H = p.H;
  if (pair >= p.t_tot * H) return;
  const int64_t row = pair / H;
  const int h = (int)(pair - row * H);
  const int n = find_seq(p.cu, p.num_seqs, row);
  const int slot = p.slots ? p.slots[n] : n;
  if (slot < 0) return;
  const int64_t t0 = p.cu[n];
  const int64_t rel = row - t0;
  const int64_t C = (int64_t)H * (2 * DK + DV);
  const RawT* cs = p.cs_in + (int64_t)slot * 3 * C;
  const int64_t wk = (int64_t)H * DK, wv = (int64_t)H * DV;
  // tap j of a channel: packed row t0+rel-3+j, or the carried conv state before the sequence start
  auto tap_of = [&](const RawT* src, int64_t width, int64_t col0, int64_t ch0) {
    return [=](int, int j, int d) {
      const int64_t pos = rel - 3 + j;
      return pos >= 0 ? to_f32(src[(t0 + pos) * width + col0 + d]) : to_f32(cs[(3 + pos) * C + ch0 + d]);
    };
  };
  float q[1][EK], k[1][EK], v[1][EV];
  conv_rows<DK, true, 1>(tap_of(p.q, wk, (int64_t)h * DK, (int64_t)h * DK), p.conv_w + (int64_t)h * DK * 4, p.act, q);
  conv_rows<DK, true, 1>(tap_of(p.k, wk, (int64_t)h * DK, wk + (int64_t)h * DK),
                         p.conv_w + (wk + (int64_t)h * DK) * 4, p.act, k);
  conv_rows<DV, false, 1>(tap_of(p.v, wv, (int64_t)h * DV, 2 * wk + (int64_t)h * DV),
                          p.conv_w + (2 * wk + (int64_t)h * DV) * 4, p.act, v);
  const int64_t ok = pair * DK + EK * lane, ov = pair * DV + EV * lane;
#pragma unroll
  for (int e = 0; e < EK; ++e) {
    p.q_hat[ok + e] = q[0][e];
    p.k_hat[ok + e] = k[0][e];
    p.g_out[ok + e] = log_decay(to_f32(p.g[p.g_per_head ? pair : ok + e]), p.gate_mode, p.lb);
  }
#pragma unroll
  for (int e = 0; e < EV; ++e) p.v_out[ov + e] = v[0][e];
  if (lane == 0) p.beta_out[pair] = sigmoid(to_f32(p.beta[pair]));
}

// conv_state_out[slot][r][c] = source row (len - 3 + r) of channel c, reaching
// back into conv_state_in for short sequences.  Rows are written in order
// r = 0, 1, 2 by the thread that reads them; with in == out, row r reads old
// row r + len >= r, so nothing is overwritten before it is read.
template <typename RawT>
__global__ __launch_bounds__(256) void conv_state_kernel(PrepArgs<RawT> p, int DK, int DV) {
  const int n = blockIdx.y;
  const int64_t C = (int64_t)p.H * (2 * DK + DV);
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= C) return;
  const int slot = p.slots ? p.slots[n] : n;
  if (slot < 0) return;
  const int64_t t0 = p.cu[n], len = (int64_t)p.cu[n + 1] - t0;
  const int64_t qk = (int64_t)p.H * DK;
  const RawT* in = p.cs_in + (int64_t)slot * 3 * C;
  RawT* out = p.cs_out + (int64_t)slot * 3 * C;
  for (int r = 0; r < 3; ++r) {
    const int64_t pos = len - 3 + r;
    RawT x;
    if (pos >= 0) {
      const int64_t row = t0 + pos;
      if (c < qk) x = p.q[row * qk + c];
      else if (c < 2 * qk) x = p.k[row * qk + (c - qk)];
      else x = p.v[row * (int64_t)p.H * DV + (c - 2 * qk)];
    } else {
      x = in[(3 + pos) * C + c];
    }
    out[r * C + c] = x;
  }
}

template <int DK, int DV, typename RawT>
static hipError_t launch_prep_t(const PrepLaunch& L, hipStream_t s) {
  PrepArgs<RawT> p;
  p.H = L.H; p.act = L.act; p.gate_mode = L.gate_mode; p.num_seqs = L.num_seqs; p.t_tot = L.t_tot; p.lb = L.lb;
  p.cu = L.cu_seqlens; p.slots = L.slots;
  p.q = static_cast<const RawT*>(L.q); p.k = static_cast<const RawT*>(L.k); p.v = static_cast<const RawT*>(L.v);
  p.g = static_cast<const RawT*>(L.g); p.beta = static_cast<const RawT*>(L.beta); p.conv_w = L.conv_w;
  p.g_per_head = L.g_per_head;
  p.cs_in = static_cast<const RawT*>(L.cs_in); p.cs_out = static_cast<RawT*>(L.cs_out);
  p.q_hat = L.q_hat; p.k_hat = L.k_hat; p.v_out = L.v_out; p.g_out = L.g_out; p.beta_out = L.beta_out;
  const int64_t waves = L.t_tot * L.H;
  if (waves > 0) {
    hipLaunchKernelGGL((prep_kernel<DK, DV, RawT>), dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t C = (int64_t)L.H * (2 * DK + DV);
  if (L.num_seqs > 0) {
    hipLaunchKernelGGL((conv_state_kernel<RawT>), dim3((unsigned)((C + 255) / 256), (unsigned)L.num_seqs), dim3(256),
                       0, s, p, DK, DV);
  }
  return hipGetLastError();
}

hipError_t launch_prep(const PrepLaunch& L, hipStream_t s) {
  const bool bf = L.in_dtype == 1;
#define KDA_PREP_CASE(DK_, DV_)                                                                   \
  if (L.dk == DK_ && L.dv == DV_)                                                                 \
    return bf ? launch_prep_t<DK_, DV_, uint16_t>(L, s) : launch_prep_t<DK_, DV_, float>(L, s);
  KDA_PREP_CASE(64, 64)
  KDA_PREP_CASE(64, 128)
  KDA_PREP_CASE(128, 64)
  KDA_PREP_CASE(128, 128)
#undef KDA_PREP_CASE
  return hipErrorInvalidValue;
}

}  // namespace kda
