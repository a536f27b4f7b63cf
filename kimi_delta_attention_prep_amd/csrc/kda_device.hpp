// kda_device.hpp -- device-side helpers shared by the KDA kernels (gfx950 only).
//
// Scalar functions of the layer (TensorFold issue #850, shared KDA module: conv
// window, safe or softplus gate, beta, q/k L2 norms; onnxruntime-genai PR #2843:
// gate_activation='sigmoid' with gate_lower_bound, GatedRMSNorm 'sigmoid').
// Every kernel takes these from here, so a value computed by two kernels (the
// prompt preamble and a fused variant, decode and a verify window) is computed
// by the same instructions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr float kL2Eps = 1e-6f;  // inside the square root of the q/k L2 norms
constexpr int kConvW = 4;        // conv taps; tap 3 multiplies the current row
constexpr int kChunk = 64;       // prompt rows per chunk

// ---------------------------------------------------------------------------
// Record slots, with no table: chunk i of sequence n lives in slot
// base(n) + i, base(n) = floor(cu[n] / 64) + n.  From one sequence to the next
// base grows by floor(cu[n+1] / 64) - floor(cu[n] / 64) + 1 >= ceil(len_n / 64),
// so no two chunks share a slot, and the last slot is below T / 64 + num_seqs.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int64_t slot_base(const int32_t* cu, int n) { return cu[n] / kChunk + n; }

// the sequence whose slots include slot c: the largest n < num_seqs with base(n) <= c
__device__ __forceinline__ int slot_seq(const int32_t* cu, int num_seqs, int64_t c) {
  int lo = 0, hi = num_seqs;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (slot_base(cu, mid) <= c) lo = mid; else hi = mid;
  }
  return lo;
}

inline int64_t max_chunks(int num_seqs, int64_t t_tot) { return t_tot / kChunk + num_seqs; }

// raw rows arrive as fp32 or as bf16 bit patterns (uint16_t); widening is exact
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(uint16_t x) { return __uint_as_float(static_cast<uint32_t>(x) << 16); }

// sigma(x) = 1 / (1 + e^-x) from the hardware exp2 and reciprocal (each within
// about one ulp); e^-x overflows to inf for x < -88, which gives exactly 0
__device__ __forceinline__ float sigmoid(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x * -1.4426950408889634f));
}

// per-key-dim log decay g: softplus gate g = -softplus(x) = -(max(x,0) + log1p(e^-|x|));
// safe gate g = lb * sigmoid(x), so a = e^g lies in (e^lb, 1).  The softplus term uses
// the hardware exp2 and log2 (each within about one ulp): with y = e^-|x| in (0, 1],
// log1p(y) = log2(1 + y) ln 2, whose only loss beyond those is the rounding of 1 + y,
// at most 2^-24 absolute in g
__device__ __forceinline__ float log_decay(float x, int gate_mode, float lb) {
  if (gate_mode == 1) return lb * sigmoid(x);
  const float y = __builtin_amdgcn_exp2f(fabsf(x) * -1.4426950408889634f);
  return -(fmaxf(x, 0.0f) + __builtin_amdgcn_logf(1.0f + y) * 0.6931471805599453f);
}

// depthwise causal conv over 4 taps (x0 oldest, x3 current row), then SiLU when ACT
template <bool ACT>
__device__ __forceinline__ float conv4(float w0, float w1, float w2, float w3, float x0, float x1, float x2, float x3) {
  float c = w0 * x0;
  c = fmaf(w1, x1, c);
  c = fmaf(w2, x2, c);
  c = fmaf(w3, x3, c);
  if constexpr (ACT) return c * sigmoid(c);
  return c;
}
__device__ __forceinline__ float conv4_act(float w0, float w1, float w2, float w3, float x0, float x1, float x2,
                                           float x3, int act) {
  return act ? conv4<true>(w0, w1, w2, w3, x0, x1, x2, x3) : conv4<false>(w0, w1, w2, w3, x0, x1, x2, x3);
}

// Sum over the 64 lanes of a wavefront, in registers: DPP within each 16-lane
// row (pairs lane^1, lane^2, then the mirrored half-rows and rows), then the
// four row sums read as uniform values and added in a fixed order.  At every
// DPP step each lane adds its own value and its partner's, and fp addition is
// commutative bit for bit, so all lanes end with identical bits.
template <int CTRL>
__device__ __forceinline__ float dpp_partner(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp_partner<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_partner<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_partner<0x141>(x);  // row_half_mirror
  x += dpp_partner<0x140>(x);  // row_mirror
  return x;
}
__device__ __forceinline__ float lane_value(float x, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}
// x holds its 16-lane row's sum in every lane of the row
__device__ __forceinline__ float rows_total(float x) {
  return (lane_value(x, 0) + lane_value(x, 16)) + (lane_value(x, 32) + lane_value(x, 48));
}
__device__ __forceinline__ float wave_sum(float x) { return rows_total(row_sum16(x)); }

// NR rows (of one head and stream) of the prompt preamble, computed by a whole
// wavefront: lane l owns channels E*l .. E*l+E-1 (E = D/64) of every row.
// tap(rr, j, d) returns conv input tap j (0 = oldest, 3 = current row) of
// channel d for row rr; wt holds the lane's conv weights (load_conv_w).
// out[rr] gets the conv output after the activation, L2-normalised over the D
// channels when NORM.  The rows are independent and computed side by side;
// each row's arithmetic does not depend on NR, so the standalone preamble
// kernel (one row, taps from HBM) and the fused prompt kernel (several rows,
// taps from LDS) produce the same bits.

// the conv weights lane l uses: channels E*l .. E*l+E-1 of the head's stream, 4 taps each
template <int D>
struct ConvW {
  float v[D / 64][4];
};
template <int D>
__device__ __forceinline__ ConvW<D> load_conv_w(const float* __restrict__ w) {
  constexpr int E = D / 64;
  const int lane = threadIdx.x & 63;
  ConvW<D> wt;
#pragma unroll
  for (int e = 0; e < E; ++e)
#pragma unroll
    for (int j = 0; j < 4; ++j) wt.v[e][j] = w[(int64_t)(E * lane + e) * 4 + j];
  return wt;
}
template <int D, bool NORM, int NR, bool ACT, class TAP>
__device__ __forceinline__ void conv_rows_t(TAP tap, const ConvW<D>& wt, float (&out)[NR][D / 64]) {
  constexpr int E = D / 64;
  const int lane = threadIdx.x & 63;
  float ss[NR];
#pragma unroll
  for (int rr = 0; rr < NR; ++rr) {
    ss[rr] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int d = E * lane + e;
      out[rr][e] = conv4<ACT>(wt.v[e][0], wt.v[e][1], wt.v[e][2], wt.v[e][3], tap(rr, 0, d), tap(rr, 1, d),
                              tap(rr, 2, d), tap(rr, 3, d));
      ss[rr] = fmaf(out[rr][e], out[rr][e], ss[rr]);
    }
  }
  if constexpr (NORM) {  // wave_sum of every row, side by side
#pragma unroll
    for (int rr = 0; rr < NR; ++rr) ss[rr] = row_sum16(ss[rr]);
#pragma unroll
    for (int rr = 0; rr < NR; ++rr) ss[rr] = rows_total(ss[rr]);
#pragma unroll
    for (int rr = 0; rr < NR; ++rr) {
      const float r = __builtin_amdgcn_rsqf(ss[rr] + kL2Eps);  // hardware 1/sqrt, about 1 ulp
#pragma unroll
      for (int e = 0; e < E; ++e) out[rr][e] *= r;
    }
  }
}
// the activation is chosen once for the whole batch of rows, so that the rows'
// loads and arithmetic interleave freely; the weights are either loaded here
// (w points at the head's first conv weight row of the stream) or loaded
// earlier by the caller
template <int D, bool NORM, int NR, class TAP>
__device__ __forceinline__ void conv_rows(TAP tap, const ConvW<D>& wt, int act, float (&out)[NR][D / 64]) {
  if (act) conv_rows_t<D, NORM, NR, true>(tap, wt, out);
  else conv_rows_t<D, NORM, NR, false>(tap, wt, out);
}
template <int D, bool NORM, int NR, class TAP>
__device__ __forceinline__ void conv_rows(TAP tap, const float* __restrict__ w, int act, float (&out)[NR][D / 64]) {
  conv_rows<D, NORM, NR>(tap, load_conv_w<D>(w), act, out);
}

// 16-byte state accesses marked non-temporal: every state tile is read once and
// written once per call, and the state pool is larger than the caches
__device__ __forceinline__ float4 load_nt4(const float* p) {
  const floatx4 x = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(p));
  return make_float4(x[0], x[1], x[2], x[3]);
}
__device__ __forceinline__ void store_nt4(float* p, const float4& v) {
  __builtin_nontemporal_store(floatx4{v.x, v.y, v.z, v.w}, reinterpret_cast<floatx4*>(p));
}

// one state element's step: S' = a * S, then S = S' + k * u (explicit fma).
// decode, verify windows and the commit replay all use exactly this.
__device__ __forceinline__ float decay(float s, float a) { return a * s; }
__device__ __forceinline__ float rank1(float s_decayed, float k, float u) { return fmaf(k, u, s_decayed); }

}  // namespace kda
