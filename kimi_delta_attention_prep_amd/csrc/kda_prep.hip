// kda_prep.hip -- preamble of the prompt path for packed varlen rows (gfx950).
//
// TensorFold issue #850 (shared KDA module: conv window, safe or softplus gate,
// beta, q/k L2 norms) and onnxruntime-genai PR #2843 (VarlenCausalConvWithState,
// GatedDeltaNet gate with gate_activation='sigmoid' and gate_lower_bound):
//   conv: c_t = sum_{j<4} w[c][j] x_{t-3+j}  (rows before a sequence's first row
//         come from its carried conv state), then SiLU;
//   q_hat = c_q / sqrt(|c_q|^2 + 1e-6), k_hat likewise, v = c_v;
//   g = -softplus(x_g) or lb * sigmoid(x_g);  beta = sigmoid(x_b).
// One workgroup per (64-row tile of a sequence, head, stream), its rows staged
// in LDS with 16-byte loads; each lane owns d/64 consecutive channels of a row.
// The carried conv state is written by a second launch after every read of the
// old one, which lets the caller pass the same buffer for input and output.
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

// 8 consecutive raw values (16 or 32 bytes, aligned) as fp32
__device__ __forceinline__ void load8_raw(const float* src, float (&x)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(src), b = *reinterpret_cast<const float4*>(src + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
__device__ __forceinline__ void load8_raw(const uint16_t* src, float (&x)[8]) {
  const uint4 v = *reinterpret_cast<const uint4*>(src);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// The conv of one stream (q, k or v: D channels per head) over one 64-row tile:
// the tile's rows and the 3 rows before it are staged in LDS with 16-byte loads
// (rows before the sequence's first row come from its carried conv state), then
// each wavefront convolves 16 consecutive rows side by side from there and writes
// a lane's D/64 channels of each row.  conv_rows computes each row on its own
// whatever the number of rows, so the bits are those of the fused prompt kernel.
template <int D, bool NORM, typename RawT>
__device__ __forceinline__ void prep_stream(const PrepArgs<RawT>& p, RawT* st, const RawT* src, const RawT* cs,
                                            int64_t C, int64_t ch0, float* dst, int h, int64_t t0, int64_t end,
                                            int64_t start, int len) {
  constexpr int L = kChunk, NT = 256, RW = L / (NT / 64);  // 16 rows per wavefront
  constexpr int VE = 16 / sizeof(RawT);                   // raw elements per 16-byte piece
  constexpr int PR = D / VE, NP = (L + 3) * PR;           // pieces per row, per staged tile
  constexpr int NI = (NP + NT - 1) / NT;                  // ... per thread
  constexpr int E = D / 64;                               // channels per lane
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, H = p.H;
  const int64_t width = (int64_t)H * D, col0 = (int64_t)h * D;
  // Loads are unconditional (clamped into the sequence) so that no branch makes a
  // wait count fewer loads; rows before the sequence start are overwritten below.
  uint4 x[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int idx = min(t + i * NT, NP - 1), sr = idx / PR;
    int64_t pos = start - 3 + sr;
    pos = pos < t0 ? t0 : (pos >= end ? end - 1 : pos);
    x[i] = *reinterpret_cast<const uint4*>(src + pos * width + col0 + (idx % PR) * VE);
  }
  const ConvW<D> wt = load_conv_w<D>(p.conv_w + ch0 * 4);
#pragma unroll
  for (int i = 0; i < NI; ++i)
    if (t + i * NT < NP) *reinterpret_cast<uint4*>(st + (t + i * NT) * VE) = x[i];
  if (start == t0) {  // the sequence's first tile (uniform over the workgroup): the 3 carried rows
    for (int idx = t; idx < 3 * PR; idx += NT) {
      const int sr = idx / PR, c0 = (idx % PR) * VE;
      const RawT* cr = cs + sr * C + ch0 + c0;  // the conv state is not 16-byte aligned per channel
#pragma unroll
      for (int e = 0; e < VE; ++e) st[idx * VE + e] = cr[e];
    }
  }
  __syncthreads();
  const int r0 = RW * wave;
  float y[RW][E];
  conv_rows<D, NORM, RW>([&](int rr, int j, int d) { return to_f32(st[(r0 + rr + j) * D + d]); }, wt, p.act, y);
#pragma unroll
  for (int rr = 0; rr < RW; ++rr) {
    if (r0 + rr < len) {
      float* o = dst + ((start + r0 + rr) * H + h) * D + E * lane;
      if constexpr (E == 2) *reinterpret_cast<float2*>(o) = make_float2(y[rr][0], y[rr][1]);
      else o[0] = y[rr][0];
    }
  }
}

// One workgroup (4 wavefronts) per (64-row tile of a sequence, head, stream),
// the tiles anchored at each sequence's first row as the prompt kernels' chunks
// are.  blockIdx.z picks the stream: 0 q, 1 k, 2 v (a staged conv each), 3 the
// decay and beta (no conv: rows to outputs, 8 values per lane).  Splitting the
// streams keeps each workgroup's LDS small, so several run per CU and one's
// loads overlap another's stores.
template <int DK, int DV, typename RawT>
__global__ __launch_bounds__(256) void prep_tile_kernel(PrepArgs<RawT> p) {
  constexpr int L = kChunk, NT = 256;
  extern __shared__ __align__(16) unsigned char prep_smem[];
  RawT* st = reinterpret_cast<RawT*>(prep_smem);  // [67][D] staged rows of the workgroup's stream
  const int t = threadIdx.x;
  const int c = blockIdx.x, h = blockIdx.y, z = blockIdx.z, H = p.H;
  const int n = slot_seq(p.cu, p.num_seqs, c);
  const int64_t t0 = p.cu[n], end = p.cu[n + 1];
  const int64_t start = t0 + (c - slot_base(p.cu, n)) * L;
  if (start >= end) return;  // a tile past the sequence's last row
  const int slot = p.slots ? p.slots[n] : n;
  if (slot < 0) return;
  const int len = (int)min((int64_t)L, end - start);
  const int64_t C = (int64_t)H * (2 * DK + DV), wk = (int64_t)H * DK;
  const RawT* cs = p.cs_in + (int64_t)slot * 3 * C;
  if (z == 0) {
    prep_stream<DK, true>(p, st, p.q, cs, C, (int64_t)h * DK, p.q_hat, h, t0, end, start, len);
  } else if (z == 1) {
    prep_stream<DK, true>(p, st, p.k, cs, C, wk + (int64_t)h * DK, p.k_hat, h, t0, end, start, len);
  } else if (z == 2) {
    prep_stream<DV, false>(p, st, p.v, cs, C, 2 * wk + (int64_t)h * DV, p.v_out, h, t0, end, start, len);
  } else {
    for (int idx = t; idx < L * (DK / 8); idx += NT) {
      const int r = idx / (DK / 8), c8 = 8 * (idx % (DK / 8));
      if (r >= len) break;  // rows ascend with idx
      const int64_t pr = (start + r) * H + h;
      float gv[8];
      if (p.g_per_head) {
        const float gh = log_decay(to_f32(p.g[pr]), p.gate_mode, p.lb);
#pragma unroll
        for (int e = 0; e < 8; ++e) gv[e] = gh;
      } else {
        load8_raw(p.g + pr * DK + c8, gv);
#pragma unroll
        for (int e = 0; e < 8; ++e) gv[e] = log_decay(gv[e], p.gate_mode, p.lb);
      }
      *reinterpret_cast<float4*>(p.g_out + pr * DK + c8) = make_float4(gv[0], gv[1], gv[2], gv[3]);
      *reinterpret_cast<float4*>(p.g_out + pr * DK + c8 + 4) = make_float4(gv[4], gv[5], gv[6], gv[7]);
    }
    if (t < len) p.beta_out[(start + t) * H + h] = sigmoid(to_f32(p.beta[(start + t) * H + h]));
  }
}

// conv_state_out[slot][r][c] = source row (len - 3 + r) of channel c, reaching
// back into conv_state_in for short sequences.  Rows are written in order
// r = 0, 1, 2 by the thread that reads them; with in == out, row r reads old
// row r + len >= r, so nothing is overwritten before it is read.
constexpr int kSeqGridY = 65535;  // the largest y extent of a grid: sequences beyond it continue in z

template <typename RawT>
__global__ __launch_bounds__(256) void conv_state_kernel(PrepArgs<RawT> p, int DK, int DV) {
  const int n = (int)(blockIdx.z * kSeqGridY + blockIdx.y);
  if (n >= p.num_seqs) return;
  const int64_t C = (int64_t)p.H * (2 * DK + DV);
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= C) return;
  const int slot = p.slots ? p.slots[n] : n;
  if (slot < 0) return;
  const int64_t t0 = p.cu[n], len = (int64_t)p.cu[n + 1] - t0;
  const int64_t qk = (int64_t)p.H * DK;
  const RawT* in = p.cs_in + (int64_t)slot * 3 * C;
  RawT* out = p.cs_out + (int64_t)slot * 3 * C;
  if (len >= 3) {  // (uniform over the workgroup) every row comes from the packed rows: three loads, then the stores
    const RawT* src = c < qk ? p.q + c : (c < 2 * qk ? p.k + (c - qk) : p.v + (c - 2 * qk));
    const int64_t width = c < 2 * qk ? qk : (int64_t)p.H * DV;
    RawT x[3];
#pragma unroll
    for (int r = 0; r < 3; ++r) x[r] = src[(t0 + len - 3 + r) * width];
#pragma unroll
    for (int r = 0; r < 3; ++r) out[r * C + c] = x[r];
    return;
  }
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
  const int64_t mc = max_chunks(L.num_seqs, L.t_tot);
  if (L.t_tot > 0 && L.num_seqs > 0) {
    constexpr size_t lds = (size_t)(kChunk + 3) * (DK > DV ? DK : DV) * sizeof(RawT);
    const hipError_t ea = ensure_dynamic_lds(reinterpret_cast<const void*>(&prep_tile_kernel<DK, DV, RawT>), lds);
    if (ea != hipSuccess) return ea;
    hipLaunchKernelGGL((prep_tile_kernel<DK, DV, RawT>), dim3((unsigned)mc, (unsigned)L.H, 4), dim3(256), lds, s, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t C = (int64_t)L.H * (2 * DK + DV);
  if (L.num_seqs > 0) {
    const unsigned gy = (unsigned)(L.num_seqs < kSeqGridY ? L.num_seqs : kSeqGridY);
    const unsigned gz = (unsigned)((L.num_seqs + kSeqGridY - 1) / kSeqGridY);
    hipLaunchKernelGGL((conv_state_kernel<RawT>), dim3((unsigned)((C + 255) / 256), gy, gz), dim3(256), 0, s, p, DK,
                       DV);
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
