// kda_norm.hip -- sigmoid-gated output RMSNorm (onnxruntime-genai PR #2843:
// GatedRMSNorm with activation 'sigmoid'; TensorFold issue #850: the gated
// output norm closes the shared KDA module):
//     y = o / sqrt(mean(o^2) + eps) * w * sigmoid(z)   per row of d_v values.
// One wavefront per row, 16-byte loads, a wavefront butterfly for the sum of
// squares; bound by HBM bytes (read o and z, write y).
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

template <typename ZT>
__device__ __forceinline__ void load4(const ZT* p, float (&x)[4]);
template <>
__device__ __forceinline__ void load4<float>(const float* p, float (&x)[4]) {
  const float4 v = *reinterpret_cast<const float4*>(p);
  x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
}
template <>
__device__ __forceinline__ void load4<uint16_t>(const uint16_t* p, float (&x)[4]) {
  const uint2 v = *reinterpret_cast<const uint2*>(p);
  x[0] = __uint_as_float(v.x << 16); x[1] = __uint_as_float(v.x & 0xffff0000u);
  x[2] = __uint_as_float(v.y << 16); x[3] = __uint_as_float(v.y & 0xffff0000u);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs; NaN kept quiet)
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u) return (u >> 16) | ((u & 0xffffu) ? 0x40u : 0u);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

template <typename YT>
__device__ __forceinline__ void store4(YT* p, const float (&y)[4]);
template <>
__device__ __forceinline__ void store4<float>(float* p, const float (&y)[4]) {
  *reinterpret_cast<float4*>(p) = make_float4(y[0], y[1], y[2], y[3]);
}
template <>
__device__ __forceinline__ void store4<uint16_t>(uint16_t* p, const float (&y)[4]) {
  uint2 v;
  v.x = f32_to_bf16_bits(y[0]) | (f32_to_bf16_bits(y[1]) << 16);
  v.y = f32_to_bf16_bits(y[2]) | (f32_to_bf16_bits(y[3]) << 16);
  *reinterpret_cast<uint2*>(p) = v;
}

// DV/4 lanes per row (4 values each); 64/(DV/4) rows per wavefront
template <int DV, typename ZT, typename YT>
__global__ __launch_bounds__(256) void gated_rmsnorm_kernel(int64_t rows, const float* __restrict__ o,
                                                            const ZT* __restrict__ z, const float* __restrict__ w,
                                                            float eps, YT* __restrict__ y) {
  constexpr int LPR = DV / 4;  // lanes per row
  const int t = threadIdx.x;
  const int64_t row = (int64_t)blockIdx.x * (256 / LPR) + t / LPR;
  const int c = 4 * (t % LPR);
  float ov[4] = {0.f, 0.f, 0.f, 0.f}, zv[4] = {0.f, 0.f, 0.f, 0.f};
  const bool live = row < rows;
  if (live) {
    load4<float>(o + row * DV + c, ov);
    load4<ZT>(z + row * DV + c, zv);
  }
  float ss = ov[0] * ov[0];
  ss = fmaf(ov[1], ov[1], ss);
  ss = fmaf(ov[2], ov[2], ss);
  ss = fmaf(ov[3], ov[3], ss);
#pragma unroll
  for (int off = 1; off < LPR; off <<= 1) ss += __shfl_xor(ss, off, 64);
  if (!live) return;
  const float inv = 1.0f / sqrtf(ss / (float)DV + eps);
  const float4 wv = *reinterpret_cast<const float4*>(w + c);
  const float wa[4] = {wv.x, wv.y, wv.z, wv.w};
  float yv[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) yv[e] = ov[e] * inv * wa[e] * sigmoid(zv[e]);
  store4<YT>(y + row * DV + c, yv);
}

template <int DV>
static hipError_t launch_norm_dv(const NormLaunch& L, hipStream_t s) {
  constexpr int RPB = 256 / (DV / 4);
  const dim3 grid((unsigned)((L.rows + RPB - 1) / RPB));
  const bool zb = L.z_dtype == 1, yb = L.y_dtype == 1;
#define KDA_NORM_CASE(ZT, YT)                                                                          \
  hipLaunchKernelGGL((gated_rmsnorm_kernel<DV, ZT, YT>), grid, dim3(256), 0, s, L.rows, L.o,           \
                     static_cast<const ZT*>(L.z), L.w, L.eps, static_cast<YT*>(L.y))
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
