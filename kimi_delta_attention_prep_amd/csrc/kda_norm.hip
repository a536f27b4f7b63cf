// kda_norm.hip -- sigmoid-gated output RMSNorm (onnxruntime-genai PR #2843:
// GatedRMSNorm with activation 'sigmoid'; TensorFold issue #850: the gated
// output norm closes the shared KDA module):
//     y = o / sqrt(mean(o^2) + eps) * w * sigmoid(z)   per row of d_v values.
// 8 values per lane with 16- and 32-byte accesses, the sum of squares reduced
// within each row's lanes by DPP; bound by HBM bytes (read o and z, write y).
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

// 8 consecutive values of a row, 16 or 32 bytes per lane
template <typename ZT>
__device__ __forceinline__ void load8(const ZT* p, float (&x)[8]);
template <>
__device__ __forceinline__ void load8<float>(const float* p, float (&x)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float (&x)[8]) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// fp32 -> bf16 bits, round to nearest even (finite inputs; NaN kept quiet)
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u) return (u >> 16) | ((u & 0xffffu) ? 0x40u : 0u);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

template <typename YT>
__device__ __forceinline__ void store8(YT* p, const float (&y)[8]);
template <>
__device__ __forceinline__ void store8<float>(float* p, const float (&y)[8]) {
  *reinterpret_cast<float4*>(p) = make_float4(y[0], y[1], y[2], y[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(y[4], y[5], y[6], y[7]);
}
template <>
__device__ __forceinline__ void store8<uint16_t>(uint16_t* p, const float (&y)[8]) {
  uint4 v;
  v.x = f32_to_bf16_bits(y[0]) | (f32_to_bf16_bits(y[1]) << 16);
  v.y = f32_to_bf16_bits(y[2]) | (f32_to_bf16_bits(y[3]) << 16);
  v.z = f32_to_bf16_bits(y[4]) | (f32_to_bf16_bits(y[5]) << 16);
  v.w = f32_to_bf16_bits(y[6]) | (f32_to_bf16_bits(y[7]) << 16);
  *reinterpret_cast<uint4*>(p) = v;
}

// DV/8 lanes per row (8 values each): 16 lanes at d_v = 128, 8 at 64; the sum of
// squares is reduced inside the lanes' 16-lane DPP row, so no LDS is touched
template <int DV, typename ZT, typename YT>
__global__ __launch_bounds__(256) void gated_rmsnorm_kernel(int64_t rows, const float* __restrict__ o,
                                                            const ZT* __restrict__ z, const float* __restrict__ w,
                                                            float eps, YT* __restrict__ y, const int32_t* cu,
                                                            const int32_t* slots, int num_seqs, int H) {
  constexpr int LPR = DV / 8;  // lanes per row
  static_assert(LPR == 8 || LPR == 16, "8 or 16 lanes per row");
  const int t = threadIdx.x;
  const int64_t row = (int64_t)blockIdx.x * (256 / LPR) + t / LPR;
  const int c = 8 * (t % LPR);
  float ov[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, zv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  bool live = row < rows;
  if (live) {
    load8<float>(o + row * DV + c, ov);
    load8<ZT>(z + row * DV + c, zv);
  }
  float ss = ov[0] * ov[0];
#pragma unroll
  for (int e = 1; e < 8; ++e) ss = fmaf(ov[e], ov[e], ss);
  ss += dpp_partner<0xB1>(ss);    // quad_perm [1,0,3,2]
  ss += dpp_partner<0x4E>(ss);    // quad_perm [2,3,0,1]
  ss += dpp_partner<0x141>(ss);   // row_half_mirror: the 8-lane sum
  if constexpr (LPR == 16) ss += dpp_partner<0x140>(ss);  // row_mirror: the 16-lane sum
  if (live && slots) {  // prompt epilogue with a slot map: the row's sequence n, largest with cu[n] <= token
    const int64_t tok = row / H;
    int lo = 0, hi = num_seqs;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (cu[mid] <= tok) lo = mid; else hi = mid;
    }
    live = slots[lo] >= 0;
  }
  if (!live) return;
  const float inv = 1.0f / sqrtf(ss / (float)DV + eps);
  float wa[8], yv[8];
  load8<float>(w + c, wa);
#pragma unroll
  for (int e = 0; e < 8; ++e) yv[e] = ov[e] * inv * wa[e] * sigmoid(zv[e]);
  store8<YT>(y + row * DV + c, yv);
}

template <int DV>
static hipError_t launch_norm_dv(const NormLaunch& L, hipStream_t s) {
  constexpr int RPB = 256 / (DV / 8);
  const dim3 grid((unsigned)((L.rows + RPB - 1) / RPB));
  const bool zb = L.z_dtype == 1, yb = L.y_dtype == 1;
#define KDA_NORM_CASE(ZT, YT)                                                                          \
  hipLaunchKernelGGL((gated_rmsnorm_kernel<DV, ZT, YT>), grid, dim3(256), 0, s, L.rows, L.o,           \
                     static_cast<const ZT*>(L.z), L.w, L.eps, static_cast<YT*>(L.y), L.cu, L.slots,    \
                     L.num_seqs, L.H)
  if (zb && yb) KDA_NORM_CASE(uint16_t, uint16_t);
  else if (zb) KDA_NORM_CASE(uint16_t, float);
  else if (yb) KDA_NORM_CASE(float, uint16_t);
  else KDA_NORM_CASE(float, float);
#undef KDA_NORM_CASE
  return hipGetLastError();
}

hipError_t launch_gated_rmsnorm(const NormLaunch& L, hipStream_t s) {
  if (L.rows == 0) return hipSuccess;
  if (L.dv == 64) return launch_norm_dv<64>(L, s);
  if (L.dv == 128) return launch_norm_dv<128>(L, s);
  return hipErrorInvalidValue;
}

}  // namespace kda
