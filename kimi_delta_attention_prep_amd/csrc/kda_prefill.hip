// kda_prefill.hip -- chunk-parallel prompt path of the gated delta rule (gfx950).
//
// The recurrence (per-key-dim gated delta rule; TensorFold issue #850, the
// shared KDA module's prompt rows "in chunks from a segment's first row")
//   S_t = Diag(a_t) S_{t-1} + k_t u_t^T,  u_t = b_t (v_t - (Diag(a_t) S_{t-1})^T k_t),  o_t = S_t^T q_t
// is unrolled over 64-row chunks anchored at each sequence's first row.  With
// G_r = sum_{i<=r} g_i (per key dim, g = log a) and a chunk entering with S0:
//   A_ri = b_r sum_d k_r[d] k_i[d] e^{G_r[d]-G_i[d]}   (i < r)
//   P_ri =     sum_d q_r[d] k_i[d] e^{G_r[d]-G_i[d]}   (i <= r)
//   X = (I + A)^{-1},  W = X Diag(b) K^gamma,  U~ = X Diag(b) V      (WY / UT form)
//   U = U~ - W S0,  O = Q^gamma S0 + P U,  S_L = Diag(gamma_L) S0 + K_<^T U
// where K^gamma = e^{G_r} k_r, Q^gamma = e^{G_r} q_r, K_< = e^{G_last - G_i} k_i.
//
// Kernels:
//   chunk_table  -- first chunk of every sequence (exclusive scan of ceil(len/64))
//   chunk_intra  -- one workgroup per (chunk, head), all chunks in parallel:
//                   G, A, P on the matrix cores, the 64x64 triangular solve,
//                   W and U~.  It writes W, Q^gamma, P and K_<^T as matrix-core
//                   operand fragments (each lane's 32-wide K slice, already
//                   converted to the policy's operand type), U~ in the result
//                   layout of 16-column slices, and gamma_L.
//   chunk_scan   -- one workgroup per (sequence, head, 16 state columns), a
//                   sequential pass over the sequence's chunks.  Each wavefront
//                   loads its own operand fragments straight into registers
//                   with 128-bit loads, one chunk ahead of use; only the small
//                   B operands (the state slice and U slice) go through LDS.
// The pairwise factors e^{G_r - G_i} are formed as e^{G_r - G_p} * e^{G_p - G_i}
// around pivot rows (below), so each 16x16 block of A and P is a plain matrix
// product; exponents come from block-local prefix sums, which keeps them
// accurate to a few ulp of the exponent itself.
//
// Precision policies of the matrix products (all accumulate in fp32; the
// intra-chunk products always use fp32 or split bf16):
//   FP32    fp32 operands, v_mfma_f32_16x16x4f32
//   BF16X3  operands split into bf16 hi + lo, hi*hi + hi*lo + lo*hi
//   FP16    A operands (W, Q^gamma, P, K_<^T: every entry bounded by 1) rounded
//           once to fp16; B operands (state, U) split into fp16 hi + lo
//   BF16X2  as FP16 with bf16 in place of fp16: A operands rounded once to bf16,
//           B operands split into bf16 hi + lo, so state and U keep the fp32 range
#include <mutex>
#include <type_traits>

#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

enum { POL_FP32 = 0, POL_BF16X3 = 1, POL_FP16 = 2, POL_BF16X2 = 3 };

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// 16x16 matrix-core tile product on the fly:  acc (16x16) += A (16xK) * B (Kx16)
// Fragment map of v_mfma_f32_16x16x4f32 / v_mfma_f32_16x16x32_{bf16,f16}: lane
// l holds row (l % 16) of A and column (l % 16) of B, with its K slice picked
// by l / 16; the result lane l holds column l % 16, rows 4*(l/16)..4*(l/16)+3.
// K is a multiple of 32.  Used by the intra-chunk kernel (FP32 or BF16X3).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void split_bf16(float x, __bf16& hi, __bf16& lo) {
  hi = static_cast<__bf16>(x);
  lo = static_cast<__bf16>(x - static_cast<float>(hi));
}
__device__ __forceinline__ void split_f16(float x, _Float16& hi, _Float16& lo) {
  hi = static_cast<_Float16>(x);
  lo = static_cast<_Float16>(x - static_cast<float>(hi));
}

template <int POL, class FA, class FB>
__device__ __forceinline__ void mma16(floatx4& acc, int K, FA fa, FB fb) {
  const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
  if constexpr (POL == POL_FP32) {
    for (int k0 = 0; k0 < K; k0 += 4)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(fa(r, k0 + g), fb(k0 + g, r), acc, 0, 0, 0);
  } else {
    for (int k0 = 0; k0 < K; k0 += 32) {
      bf16x8 ah, al, bh, bl;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        __bf16 h1, l1, h2, l2;
        split_bf16(fa(r, k0 + 8 * g + e), h1, l1);
        split_bf16(fb(k0 + 8 * g + e, r), h2, l2);
        ah[e] = h1; al[e] = l1; bh[e] = h2; bl[e] = l2;
      }
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
    }
  }
}

// ---------------------------------------------------------------------------
// Stored operand fragments.  A fragment is one lane's share of a 16-row x
// 32-wide K block; element e of lane l sits at K index kof(l/16, e).
// ---------------------------------------------------------------------------
template <int POL>
struct Frag;

template <>
struct Frag<POL_FP32> {
  static constexpr int BYTES = 32;
  __device__ static constexpr int kof(int g, int e) { return 4 * e + g; }
  struct A { float v[8]; };
  using B = A;
  __device__ static A load_a(const uint8_t* p) {
    A a;
    const float4 x = *reinterpret_cast<const float4*>(p), y = *reinterpret_cast<const float4*>(p + 16);
    a.v[0] = x.x; a.v[1] = x.y; a.v[2] = x.z; a.v[3] = x.w; a.v[4] = y.x; a.v[5] = y.y; a.v[6] = y.z; a.v[7] = y.w;
    return a;
  }
  __device__ static void store_a(uint8_t* p, const float (&x)[8]) {
    *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
    *reinterpret_cast<float4*>(p + 16) = make_float4(x[4], x[5], x[6], x[7]);
  }
  __device__ static B make_b(const float (&x)[8]) {
    B b;
#pragma unroll
    for (int e = 0; e < 8; ++e) b.v[e] = x[e];
    return b;
  }
  __device__ static floatx4 mma(floatx4 acc, const A& a, const B& b) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], acc, 0, 0, 0);
    return acc;
  }
  // the transposed product (A B)^T = B^T A^T from the same registers: a B fragment
  // holds B^T in the A layout and an A fragment holds A^T in the B layout
  __device__ static floatx4 mma_t(floatx4 acc, const B& b, const A& a) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(b.v[e], a.v[e], acc, 0, 0, 0);
    return acc;
  }
  // B operand kept in LDS as one fp32 plane [16 columns][K]: 4 consecutive K values per write
  using P = float;
  static constexpr int PLANES = 1;
  __device__ static void store_b4(P* hi, P*, const floatx4& x) { *reinterpret_cast<floatx4*>(hi) = x; }
  __device__ static B load_b(const P* hi, const P*, int g) {
    B b;
#pragma unroll
    for (int e = 0; e < 8; ++e) b.v[e] = hi[kof(g, e)];
    return b;
  }
};

template <>
struct Frag<POL_BF16X3> {
  static constexpr int BYTES = 32;
  __device__ static constexpr int kof(int g, int e) { return 8 * g + e; }
  struct A { bf16x8 hi, lo; };
  using B = A;
  __device__ static A load_a(const uint8_t* p) {
    A a;
    a.hi = *reinterpret_cast<const bf16x8*>(p);
    a.lo = *reinterpret_cast<const bf16x8*>(p + 16);
    return a;
  }
  __device__ static B make_b(const float (&x)[8]) {
    B b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      __bf16 h, l;
      split_bf16(x[e], h, l);
      b.hi[e] = h; b.lo[e] = l;
    }
    return b;
  }
  __device__ static void store_a(uint8_t* p, const float (&x)[8]) {
    const B b = make_b(x);
    *reinterpret_cast<bf16x8*>(p) = b.hi;
    *reinterpret_cast<bf16x8*>(p + 16) = b.lo;
  }
  // elements 4 half .. 4 half + 3 of an A fragment (two lanes write one fragment)
  __device__ static void store_a_half(uint8_t* p, int half, const float (&x)[4]) {
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    bf16x4 h, l;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      __bf16 a, b;
      split_bf16(x[e], a, b);
      h[e] = a; l[e] = b;
    }
    *reinterpret_cast<bf16x4*>(p + 8 * half) = h;
    *reinterpret_cast<bf16x4*>(p + 16 + 8 * half) = l;
  }
  __device__ static floatx4 mma(floatx4 acc, const A& a, const B& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.lo, b.hi, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.lo, acc, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.hi, acc, 0, 0, 0);
  }
  __device__ static floatx4 mma_t(floatx4 acc, const B& b, const A& a) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b.hi, a.lo, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b.lo, a.hi, acc, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(b.hi, a.hi, acc, 0, 0, 0);
  }
  // B operand kept in LDS already split: hi and lo planes [16 columns][K] of bf16
  using P = __bf16;
  static constexpr int PLANES = 2;
  __device__ static void store_b4(P* hi, P* lo, const floatx4& x) {
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    bf16x4 h, l;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      __bf16 a, b;
      split_bf16(x[e], a, b);
      h[e] = a; l[e] = b;
    }
    *reinterpret_cast<bf16x4*>(hi) = h;
    *reinterpret_cast<bf16x4*>(lo) = l;
  }
  __device__ static B load_b(const P* hi, const P* lo, int g) {
    B b;
    b.hi = *reinterpret_cast<const bf16x8*>(hi + 8 * g);
    b.lo = *reinterpret_cast<const bf16x8*>(lo + 8 * g);
    return b;
  }
};

template <>
struct Frag<POL_FP16> {
  static constexpr int BYTES = 16;
  __device__ static constexpr int kof(int g, int e) { return 8 * g + e; }
  struct A { f16x8 v; };
  struct B { f16x8 hi, lo; };
  __device__ static A load_a(const uint8_t* p) {
    A a;
    a.v = *reinterpret_cast<const f16x8*>(p);
    return a;
  }
  __device__ static void store_a(uint8_t* p, const float (&x)[8]) {
    f16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = static_cast<_Float16>(x[e]);
    *reinterpret_cast<f16x8*>(p) = v;
  }
  // elements 4 half .. 4 half + 3 of an A fragment (two lanes write one fragment)
  __device__ static void store_a_half(uint8_t* p, int half, const float (&x)[4]) {
    typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
    f16x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = static_cast<_Float16>(x[e]);
    *reinterpret_cast<f16x4*>(p + 8 * half) = v;
  }
  __device__ static B make_b(const float (&x)[8]) {
    B b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      _Float16 h, l;
      split_f16(x[e], h, l);
      b.hi[e] = h; b.lo[e] = l;
    }
    return b;
  }
  __device__ static floatx4 mma(floatx4 acc, const A& a, const B& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a.v, b.lo, acc, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a.v, b.hi, acc, 0, 0, 0);
  }
  __device__ static floatx4 mma_t(floatx4 acc, const B& b, const A& a) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(b.lo, a.v, acc, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(b.hi, a.v, acc, 0, 0, 0);
  }
  // B operand kept in LDS already split: hi and lo planes [16 columns][K] of fp16
  using P = _Float16;
  static constexpr int PLANES = 2;
  __device__ static void store_b4(P* hi, P* lo, const floatx4& x) {
    typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
    f16x4 h, l;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      _Float16 a, b;
      split_f16(x[e], a, b);
      h[e] = a; l[e] = b;
    }
    *reinterpret_cast<f16x4*>(hi) = h;
    *reinterpret_cast<f16x4*>(lo) = l;
  }
  __device__ static B load_b(const P* hi, const P* lo, int g) {
    B b;
    b.hi = *reinterpret_cast<const f16x8*>(hi + 8 * g);
    b.lo = *reinterpret_cast<const f16x8*>(lo + 8 * g);
    return b;
  }
};

// One-part bf16 A operands and two-part bf16 B operands: the record layout and the
// product count of FP16, with the fp32 range (bf16 keeps fp32's exponent) for the
// state and U; A entries are bounded by 1, so one bf16 part costs only precision
// (2^-9 relative, against fp16's 2^-11).
template <>
struct Frag<POL_BF16X2> {
  static constexpr int BYTES = 16;
  __device__ static constexpr int kof(int g, int e) { return 8 * g + e; }
  struct A { bf16x8 v; };
  struct B { bf16x8 hi, lo; };
  __device__ static A load_a(const uint8_t* p) {
    A a;
    a.v = *reinterpret_cast<const bf16x8*>(p);
    return a;
  }
  __device__ static void store_a(uint8_t* p, const float (&x)[8]) {
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = static_cast<__bf16>(x[e]);
    *reinterpret_cast<bf16x8*>(p) = v;
  }
  // elements 4 half .. 4 half + 3 of an A fragment (two lanes write one fragment)
  __device__ static void store_a_half(uint8_t* p, int half, const float (&x)[4]) {
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    bf16x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = static_cast<__bf16>(x[e]);
    *reinterpret_cast<bf16x4*>(p + 8 * half) = v;
  }
  __device__ static B make_b(const float (&x)[8]) {
    B b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      __bf16 h, l;
      split_bf16(x[e], h, l);
      b.hi[e] = h; b.lo[e] = l;
    }
    return b;
  }
  __device__ static floatx4 mma(floatx4 acc, const A& a, const B& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.lo, acc, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.hi, acc, 0, 0, 0);
  }
  __device__ static floatx4 mma_t(floatx4 acc, const B& b, const A& a) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b.lo, a.v, acc, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(b.hi, a.v, acc, 0, 0, 0);
  }
  // B operand kept in LDS already split: hi and lo planes [16 columns][K] of bf16
  using P = __bf16;
  static constexpr int PLANES = 2;
  __device__ static void store_b4(P* hi, P* lo, const floatx4& x) {
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    bf16x4 h, l;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      __bf16 a, b;
      split_bf16(x[e], a, b);
      h[e] = a; l[e] = b;
    }
    *reinterpret_cast<bf16x4*>(hi) = h;
    *reinterpret_cast<bf16x4*>(lo) = l;
  }
  __device__ static B load_b(const P* hi, const P* lo, int g) {
    B b;
    b.hi = *reinterpret_cast<const bf16x8*>(hi + 8 * g);
    b.lo = *reinterpret_cast<const bf16x8*>(lo + 8 * g);
    return b;
  }
};

// the intra-chunk kernel's own products: fp32 for the FP32 policy, split bf16 otherwise
template <int POL>
struct IntraPol { static constexpr int value = POL == POL_FP32 ? POL_FP32 : POL_BF16X3; };

// e^x: the accurate library exponential for the fp32 policy, the hardware
// exp2 for the others (whose products carry a larger rounding anyway)
template <int POL>
__device__ __forceinline__ float pexp(float x) {
  if constexpr (POL == POL_FP32) return expf(x);
  else return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

// Write the A-operand fragments of a (16*MT) x (32*KB) matrix given by acc(row, k)
// to dst[(mt * KB + kb) * 64 + lane], spread over the workgroup's threads.
template <int POL, int NT, class ACC>
__device__ __forceinline__ void write_afrags(uint8_t* dst, int MT, int KB, ACC acc) {
  using F = Frag<POL>;
  for (int item = threadIdx.x; item < MT * KB * 64; item += NT) {
    const int lane = item & 63, blk = item >> 6, mt = blk / KB, kb = blk % KB;
    const int row = 16 * mt + (lane & 15), g = lane >> 4;
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = acc(row, 32 * kb + F::kof(g, e));
    F::store_a(dst + (size_t)item * F::BYTES, x);
  }
}

// ---------------------------------------------------------------------------
// workspace layout
// ---------------------------------------------------------------------------
// Record of one (chunk, head), byte offsets; FB = fragment bytes per lane.
//   Wf  [4 mt][dk/32 kb][64 lanes]    W        (rows 16mt.., K = key dim)
//   Qf  [4 mt][dk/32 kb][64 lanes]    Q^gamma
//   Pf  [4 mt][2 kb][64 lanes]        P        (K = chunk row)
//   Kf  [dk/16 mt][2 kb][64 lanes]    K_<^T    (rows = key dim, K = chunk row)
//   Ut  [dv/16 slice][4 mt][64 lanes][4] fp32  U~ in the matrix-core result layout
//   gL  [dk] fp32                     gamma_L = e^{G_last}
struct RecLayout {
  int64_t Wf, Qf, Pf, Kf, Ut, gL, bytes;
};
__host__ __device__ inline RecLayout rec_layout(int dk, int dv, int fb) {
  RecLayout r;
  const int64_t fs = 64 * (int64_t)fb;
  r.Wf = 0;
  r.Qf = r.Wf + 4 * (dk / 32) * fs;
  r.Pf = r.Qf + 4 * (dk / 32) * fs;
  r.Kf = r.Pf + 4 * 2 * fs;
  r.Ut = r.Kf + (dk / 16) * 2 * fs;
  r.gL = r.Ut + (int64_t)64 * dv * 4;
  r.bytes = (r.gL + (int64_t)dk * 4 + 255) / 256 * 256;
  return r;
}
static inline int frag_bytes(int precision) { return precision == POL_FP16 || precision == POL_BF16X2 ? 16 : 32; }
// workspace: a 1 KiB sink that absorbs stores of rows past a sequence's end, then the records
constexpr size_t kSinkBytes = 1024;

size_t prefill_workspace_bytes(int H, int dk, int dv, int precision, int num_seqs, int64_t t_tot) {
  const RecLayout rl = rec_layout(dk, dv, frag_bytes(precision));
  return kSinkBytes + (size_t)max_chunks(num_seqs, t_tot) * H * (size_t)rl.bytes;
}

// The allocation-free prompt call's workspace: the sink and the chunk records live here instead of in
// a caller buffer.  Nothing in it has to start at zero (every record the scan reads is written by the
// intra-chunk kernel of the same call, and the sink is never read), so no call clears it.  Host code
// never passes this array's name to a kernel: its host-side symbol is not the device address.  Each
// device's address comes from hipGetSymbolAddress, once per device, with that device current.
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;

hipError_t noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

// raw rows and preamble parameters when the preamble runs inside the prompt kernels
struct RawRowsArgs {
  const void *q, *k, *v, *g, *beta;
  const float* conv_w;
  const void* cs_in;
  void* cs_out;
  int act, gate_mode;
  float lb;
  int esize;  // bytes per raw element; 0 without raw rows (nothing to carry)
  int g_per_head;  // raw g rows [T, H]: one decay per head and row, broadcast over d_k
};

struct PrefillArgs {
  int H, num_seqs;
  RawRowsArgs raw;
  const int32_t *cu, *slots;
  const float *q, *k, *v, *g, *beta;
  float *state, *o;
  float* sink;         // [256] target of stores that must not land in o
  uint8_t* recs;       // [max_chunks][H][rec bytes]
  int64_t rec_bytes;
  int lookahead;       // intra-chunk workgroups resident at once (one per CU): item b + lookahead
                       // runs after item b, on the same XCD
};

// ---------------------------------------------------------------------------
// intra-chunk kernel
//
// One workgroup (16 wavefronts) per (chunk, head).  Pivots: every 16-row block R
// is anchored at its first row, gl_r = G_r - G_{16R} (a block-local prefix sum,
// so exponents carry only the rounding of the decay they describe):
//   diagonal block (R,R):  left  x_r e^{gl_r}            (<= |x_r|, x = k or q)
//                          right k_i e^{-gl_i}           (<= |k_i| e^{span_R})
//   block (R,I), I < R:    left  x_r e^{gl_r}
//                          right k_i e^{D_RI - gl_i}     (<= |k_i|, D_RI = G_{16R} - G_{16I})
// Each operand is one exponential of a small exponent times a unit-norm row.
// While every block's decay span G_{16R} - G_{16R+15} stays within e^80, no
// factor overflows, and a right factor that underflows only drops terms below
// e^-87.  A chunk with a steeper block is recomputed pair by pair.  Q^gamma,
// K_< and K^gamma are single exponentials of block-local sums: e^{G_{16R}+gl_r},
// e^{G_last - G_{16I} - gl_i}, so they are exact to fp32 rounding whatever the decay.
//
// With a raw-row descriptor the kernel also runs the preamble (conv + SiLU, L2
// norms, gates, beta) itself, through the same per-row device function as the
// standalone preamble kernel, so the fused and unfused paths agree bit for bit.
// ---------------------------------------------------------------------------
constexpr float kSpanGuard = 80.0f;
// and a block's full decay T_I = G_{16I+16} - G_{16I} (one more row) must keep
// e^{T_I} a normal fp32 number, which the pivoted path multiplies by
constexpr float kBlockDecayGuard = 86.0f;

template <int DK, int DV>
struct IntraSmem {
  static constexpr int L = 64;
  static constexpr int DM = DK > DV ? DK : DV;
  static constexpr int PK = DM + 4;  // row stride of the 64 x d tiles
  static constexpr int PL = L + 4;   // row stride of the 64 x 64 tiles
  static constexpr int T0 = 0;                // k_hat; later W                      [L][PK]
  static constexpr int T1 = T0 + L * PK;      // q_hat; later b v                    [L][PK]
  static constexpr int T2 = T1 + L * PK;      // g, then gl; later b e^{G} k          [L][PK]
  static constexpr int TA = T2 + L * PK;      // A                                   [L][PL]
  static constexpr int TP = TA + L * PL;      // P, then X                           [L][PL]
  static constexpr int TB = TP + L * PL;      // beta                                [L]
  static constexpr int TD = TB + L;           // e^{G_{16R} - G_{16I+16}}, I + 1 < R  [6][DK]
  static constexpr int TG0 = TD + 6 * DK;     // g at each block's first row          [4][DK]
  static constexpr int TY = TG0 + 4 * DK;     // solve scratch, one per wavefront    [3][16][17]
  static constexpr int TFLAG = TY + 3 * 16 * 17;
  // pivoted path: e^{G_{16R}}, the K_<^T factor of block I, and e^{T_I}      [4][DK], [4][DK], [3][DK]
  static constexpr int TGFE = TFLAG + 4;
  static constexpr int TXE = TGFE + 4 * DK;
  static constexpr int TET = TXE + 4 * DK;
  static constexpr int FLOATS = TET + 3 * DK;
  static constexpr size_t BYTES = FLOATS * sizeof(float);
};

// element e of a 16-byte piece of raw rows (bf16 bit patterns or fp32)
template <typename RawT>
__device__ __forceinline__ float piece_elem(const uint4& x, int e) {
  if constexpr (sizeof(RawT) == 2) {
    const uint32_t w = e < 2 ? x.x : e < 4 ? x.y : e < 6 ? x.z : x.w;
    return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
  } else {
    return __uint_as_float(e == 0 ? x.x : e == 1 ? x.y : e == 2 ? x.z : x.w);
  }
}

__device__ __forceinline__ int pair_index(int R, int I) { return R * (R - 1) / 2 + I; }  // I < R

// Pivoted factor tiles of the intra-chunk kernel, [64 rows] x [row stride PK
// floats] in LDS.  With fp32 intra products an element is the float at
// [r * PK + d].  With split (bf16 x 3) products each row is a run of 8-column
// groups of 32 bytes, the 8 bf16 high parts and then the 8 bf16 low parts
// (hi + lo within about 2^-17 of the value), so the operands of a 32-wide K
// block load straight into the matrix-core registers and every element is
// split once per chunk instead of once per product that reads it.
template <int IP, int PK>
struct FacTile {
  static constexpr bool SPLIT = IP != POL_FP32;
  __device__ static uint8_t* at(float* base, int r, int d) {
    return reinterpret_cast<uint8_t*>(base + r * PK) + (d >> 3) * 32 + (d & 7) * 2;
  }
  __device__ static const uint8_t* at(const float* base, int r, int d) {
    return reinterpret_cast<const uint8_t*>(base + r * PK) + (d >> 3) * 32 + (d & 7) * 2;
  }
  // elements d4 .. d4 + 3 of row r (d4 a multiple of 4)
  __device__ static void store4(float* base, int r, int d4, const float (&x)[4]) {
    if constexpr (!SPLIT) {
      *reinterpret_cast<float4*>(&base[r * PK + d4]) = make_float4(x[0], x[1], x[2], x[3]);
    } else {
      // hi = x rounded to bf16, lo = (x - hi) rounded to bf16, two elements per packed
      // conversion; hi widens back to fp32 exactly from its bits
      typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
      typedef float floatx2 __attribute__((ext_vector_type(2)));
      uint32_t hb[2], lb[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const floatx2 v = {x[2 * j], x[2 * j + 1]};
        hb[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
        const floatx2 w = {v[0] - __uint_as_float(hb[j] << 16), v[1] - __uint_as_float(hb[j] & 0xffff0000u)};
        lb[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(w, bf16x2));
      }
      uint8_t* q = at(base, r, d4);
      *reinterpret_cast<uint2*>(q) = make_uint2(hb[0], hb[1]);
      *reinterpret_cast<uint2*>(q + 16) = make_uint2(lb[0], lb[1]);
    }
  }
  __device__ static float load1(const float* base, int r, int d) {
    if constexpr (!SPLIT) {
      return base[r * PK + d];
    } else {
      const uint8_t* q = at(base, r, d);
      return static_cast<float>(*reinterpret_cast<const __bf16*>(q)) +
             static_cast<float>(*reinterpret_cast<const __bf16*>(q + 16));
    }
  }
  // high and low parts of row r, columns kk .. kk + 7 (kk a multiple of 8)
  __device__ static void load8(const float* base, int r, int kk, bf16x8& hi, bf16x8& lo) {
    const uint8_t* q = at(base, r, kk);
    hi = *reinterpret_cast<const bf16x8*>(q);
    lo = *reinterpret_cast<const bf16x8*>(q + 16);
  }
};

// One block pair of A and P: acc_a += La (s . Rt)^T and acc_p += Lq (s . Rt)^T over
// K = DK, where La, Lq, Rt point at 16 factor rows (FacTile layout) and s is a
// per-K scale (none when null), applied to the right operand, which both
// products share.
template <int IP, int DK, int PK>
__device__ __forceinline__ void pair_mma(floatx4& acc_a, floatx4& acc_p, const float* La, const float* Lq,
                                         const float* Rt, const float* s) {
  using FT = FacTile<IP, PK>;
  const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
  if constexpr (IP == POL_FP32) {
    auto fa = [&](int i, int kk) { return La[i * PK + kk]; };
    auto fq = [&](int i, int kk) { return Lq[i * PK + kk]; };
    auto fb = [&](int kk, int j) { return s ? Rt[j * PK + kk] * s[kk] : Rt[j * PK + kk]; };
    mma16<IP>(acc_a, DK, fa, fb);
    mma16<IP>(acc_p, DK, fq, fb);
  } else {
#pragma unroll
    for (int k0 = 0; k0 < DK; k0 += 32) {
      const int kk = k0 + 8 * g;
      bf16x8 ah, al, qh, ql, bh, bl;
      FT::load8(La, r, kk, ah, al);
      FT::load8(Lq, r, kk, qh, ql);
      FT::load8(Rt, r, kk, bh, bl);
      if (s) {
        const float4 s0 = *reinterpret_cast<const float4*>(s + kk), s1 = *reinterpret_cast<const float4*>(s + kk + 4);
        const float sc[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          __bf16 h, l;
          split_bf16((static_cast<float>(bh[e]) + static_cast<float>(bl[e])) * sc[e], h, l);
          bh[e] = h; bl[e] = l;
        }
      }
      acc_a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc_a, 0, 0, 0);
      acc_a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc_a, 0, 0, 0);
      acc_a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc_a, 0, 0, 0);
      acc_p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ql, bh, acc_p, 0, 0, 0);
      acc_p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qh, bl, acc_p, 0, 0, 0);
      acc_p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qh, bh, acc_p, 0, 0, 0);
    }
  }
}

// 32-byte matrix-core fragments kept in LDS as two planes of 16-byte halves
// ([item] first halves, then [item] second halves), so that a wavefront's
// 16-byte accesses run at a 16-byte stride across lanes
struct FragHalves {
  uint4 a, b;
};
template <class FR>
__device__ __forceinline__ void put_frag(void* base, int nitems, int idx, const FR& f) {
  static_assert(sizeof(FR) == 32, "32-byte fragments");
  const FragHalves h = __builtin_bit_cast(FragHalves, f);
  reinterpret_cast<uint4*>(base)[idx] = h.a;
  reinterpret_cast<uint4*>(base)[nitems + idx] = h.b;
}
template <class FR>
__device__ __forceinline__ FR get_frag(const void* base, int nitems, int idx) {
  FragHalves h;
  h.a = reinterpret_cast<const uint4*>(base)[idx];
  h.b = reinterpret_cast<const uint4*>(base)[nitems + idx];
  return __builtin_bit_cast(FR, h);
}

constexpr int kIntraThreads = 1024;  // 16 wavefronts: 4 per SIMD with one workgroup per CU

template <int DK, int DV, int POL, typename RawT, bool FUSED>
__global__ __launch_bounds__(kIntraThreads) void chunk_intra_kernel(PrefillArgs p) {
  using SM = IntraSmem<DK, DV>;
  constexpr int IP = IntraPol<POL>::value;
  constexpr int L = SM::L, PK = SM::PK, PL = SM::PL, NT = kIntraThreads;
  constexpr int NW = NT / 64, RW = L / NW;  // wavefronts; consecutive rows per wavefront in the convolutions
  using FT = FacTile<IP, PK>;               // layout of the pivoted factors over T0, T1, T2 and A / P
  extern __shared__ __align__(16) float smem[];
  float* sK = smem + SM::T0;
  float* sQ = smem + SM::T1;
  float* sG = smem + SM::T2;
  float* sA = smem + SM::TA;
  float* sP = smem + SM::TP;
  float* sBeta = smem + SM::TB;
  float* sD = smem + SM::TD;
  float* sG0 = smem + SM::TG0;
  float* sGFe = smem + SM::TGFE;
  float* sXe = smem + SM::TXE;
  float* sET = smem + SM::TET;
  float* sY = smem + SM::TY;
  int* sFlag = reinterpret_cast<int*>(smem + SM::TFLAG);

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  // chunk-major order: the workgroups that start together cover every head of
  // consecutive chunks, so a round's first loads read whole rows of the packed
  // q, k, v and g tensors (about 1 µs per pass faster than head-major at T=4096, H=16)
  const int H = p.H, c = (int)(blockIdx.x / (unsigned)H), h = (int)(blockIdx.x % (unsigned)H);
  const int n = slot_seq(p.cu, p.num_seqs, c);
  const int64_t t0 = p.cu[n];
  const int64_t start = t0 + (c - slot_base(p.cu, n)) * L;
  if (start >= p.cu[n + 1]) return;  // a slot past the sequence's last chunk
  const int slot = p.slots ? p.slots[n] : n;
  if (slot < 0) return;  // the sequence is skipped: nothing of it is read or written
  const int len = (int)min((int64_t)L, (int64_t)p.cu[n + 1] - start);
  uint8_t* rec = p.recs + ((int64_t)c * H + h) * p.rec_bytes;
  const RecLayout rl = rec_layout(DK, DV, Frag<POL>::BYTES);
  const int64_t Cch = (int64_t)H * (2 * DK + DV);
  const RawT* raw_cs = FUSED ? static_cast<const RawT*>(p.raw.cs_in) + (int64_t)slot * 3 * Cch : nullptr;

  // 1. rows: k_hat, q_hat, g (zero past the chunk's last row) and beta
  // Fused: every raw row the chunk needs is loaded up front, 16 bytes per load.
  // The q and k streams are staged in LDS as 67 rows each (3 halo rows, then
  // the chunk's rows; halo rows come from the sequence's previous rows, or
  // from its carried conv state at the sequence start) and each wavefront
  // then runs the preamble of RW consecutive rows side by side, reading its taps there.
  constexpr int VE = 16 / sizeof(RawT);  // raw elements per 16-byte piece
  // piece idx of a staged stream (row sr = idx / (D / VE) of the 67).  Every load is
  // unconditional (pieces with nothing to load read the stream's first piece): a load
  // inside a branch is waited for where the branches join, which serialises the loads.
  auto load_staged = [&](const RawT* src, int D, int idx) {
    const int per_row = D / VE;
    const int sr = idx / per_row, c0 = (idx % per_row) * VE;
    const int64_t pos = start - 3 + sr;  // packed row of this staged row
    const bool live = idx < (L + 3) * per_row && sr < len + 3 && pos >= t0;
    return *reinterpret_cast<const uint4*>(src + (live ? pos * ((int64_t)H * D) + (int64_t)h * D + c0 : 0));
  };
  // the value that lands in LDS is chosen here, where it is needed anyway: the
  // loaded row, or zero past the chunk's last row
  auto store_staged = [&](RawT* st, int D, int idx, uint4 x) {
    const int per_row = D / VE;
    if (idx >= (L + 3) * per_row) return;
    if (idx / per_row >= len + 3) x = {0u, 0u, 0u, 0u};
    *reinterpret_cast<uint4*>(st + idx * VE) = x;
  };
  // the halo rows before a sequence's first row, from its carried conv state row
  // 3 + (pos - t0) (channels not 16-byte aligned in general), written over what
  // store_staged left there by the same thread.  Only the first chunk of a sequence
  // has such rows, and its workgroup alone takes this branch.
  auto store_halo = [&](RawT* st, int D, int64_t ch0, int idx) {
    const int per_row = D / VE;
    const int sr = idx / per_row, c0 = (idx % per_row) * VE;
    const int64_t pos = start - 3 + sr;
    if (idx >= (L + 3) * per_row || pos >= t0 || sr >= len + 3) return;
    const RawT* cr = raw_cs + (3 + (pos - t0)) * Cch + ch0 + c0;
    uint32_t wv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (sizeof(RawT) == 2) wv[e] = (uint32_t)cr[2 * e] | ((uint32_t)cr[2 * e + 1] << 16);
      else wv[e] = __float_as_uint(cr[e]);
    }
    *reinterpret_cast<uint4*>(st + idx * VE) = uint4{wv[0], wv[1], wv[2], wv[3]};
  };
  const bool seq_first = start == t0;  // uniform over the workgroup
  // Fused: the v rows are loaded with the preamble's rows and land long before step 7
  // (staged over T1 there where they fit; fp32 rows read their taps from HBM)
  constexpr bool kVStaged = FUSED && (L + 3) * DV * sizeof(RawT) <= (size_t)L * PK * sizeof(float);
  constexpr int NSV = kVStaged ? ((L + 3) * (DV / VE) + NT - 1) / NT : 1;
  const int64_t chv = 2 * (int64_t)H * DK + (int64_t)h * DV;
  uint4 xv[NSV];
  ConvW<DV> cwv;  // the v conv weights, loaded with the v rows
  if constexpr (FUSED) {
    constexpr int E = DK / 64;
    constexpr int NSK = ((L + 3) * (DK / VE) + NT - 1) / NT;  // pieces per thread of a staged q or k stream
    constexpr int NGK = (L * (DK / VE) + NT - 1) / NT;        // pieces per thread of the g rows
    static_assert(2 * (L + 3) * DK * sizeof(RawT) <= (size_t)(L * PK + 2 * L * PL) * sizeof(float),
                  "staged q and k rows fit over T2, A and P");
    RawT* stq = reinterpret_cast<RawT*>(sG);  // [67][DK] staged q rows, then k rows, over T2, A and P
    RawT* stk = stq + (L + 3) * DK;
    const int64_t wk = (int64_t)H * DK;
    const int64_t chq = (int64_t)h * DK, chk = wk + (int64_t)h * DK;
    // q and k load first (the workgroup that ran before on this XCD touched them
    // into L2, below); g, beta and v load once q is convolved and land while k is.
    uint4 xq[NSK], xk[NSK], xg[NGK];
    RawT xgh[NGK];
#pragma unroll
    for (int i = 0; i < NSK; ++i) xq[i] = load_staged(static_cast<const RawT*>(p.raw.q), DK, t + i * NT);
#pragma unroll
    for (int i = 0; i < NSK; ++i) xk[i] = load_staged(static_cast<const RawT*>(p.raw.k), DK, t + i * NT);
    // each stream's conv weights load right after its rows (a wait for them is then no
    // longer than the wait for the rows)
    const ConvW<DK> cwq = load_conv_w<DK>(p.raw.conv_w + chq * 4);
    // each wavefront takes RW consecutive rows, so its 4 RW taps per channel come
    // from RW + 3 staged rows, each read and widened once
    auto conv_stream = [&](const RawT* st, float* dst, const ConvW<DK>& wt) {  // rows RW wave + rr
      float x[RW][E];
      conv_rows<DK, true, RW>([&](int rr, int j, int d) { return to_f32(st[(RW * wave + rr + j) * DK + d]); },
                                 wt, p.raw.act, x);
#pragma unroll
      for (int rr = 0; rr < RW; ++rr) {
        const int r = RW * wave + rr;
#pragma unroll
        for (int e = 0; e < E; ++e) dst[r * PK + E * lane + e] = r < len ? x[rr][e] : 0.f;
      }
    };
#pragma unroll
    for (int i = 0; i < NSK; ++i) store_staged(stq, DK, t + i * NT, xq[i]);
    if (seq_first)
#pragma unroll
      for (int i = 0; i < NSK; ++i) store_halo(stq, DK, chq, t + i * NT);
    __syncthreads();
    const ConvW<DK> cwk = load_conv_w<DK>(p.raw.conv_w + chk * 4);
    conv_stream(stq, sQ, cwq);
#pragma unroll
    for (int i = 0; i < NSK; ++i) store_staged(stk, DK, t + i * NT, xk[i]);
    if (seq_first)
#pragma unroll
      for (int i = 0; i < NSK; ++i) store_halo(stk, DK, chk, t + i * NT);
    const RawT* rg = static_cast<const RawT*>(p.raw.g);
#pragma unroll
    for (int i = 0; i < NGK; ++i) {
      const int idx = t + i * NT, r = idx / (DK / VE), c0 = (idx % (DK / VE)) * VE;
      // both loads are unconditional: with one decay per head, the 16-byte piece reads
      // the q rows' first piece instead (g may hold fewer than 16 bytes) and the row's
      // own decay comes from the scalar load, which otherwise reads g's first element
      const bool ok = idx < L * (DK / VE) && r < len;
      xg[i] = *reinterpret_cast<const uint4*>(p.raw.g_per_head ? static_cast<const RawT*>(p.raw.q)
                                                               : rg + (ok ? ((start + r) * H + h) * DK + c0 : 0));
      xgh[i] = rg[p.raw.g_per_head && ok ? (start + r) * H + h : 0];
    }
    const RawT braw = static_cast<const RawT*>(p.raw.beta)[t < len ? (start + t) * H + h : 0];
    if constexpr (kVStaged) {
#pragma unroll
      for (int i = 0; i < NSV; ++i) xv[i] = load_staged(static_cast<const RawT*>(p.raw.v), DV, t + i * NT);
    }
    cwv = load_conv_w<DV>(p.raw.conv_w + chv * 4);
    __syncthreads();
    conv_stream(stk, sK, cwk);
    __syncthreads();  // the staged rows over T2 are consumed
#pragma unroll
    for (int i = 0; i < NGK; ++i) {
      const int idx = t + i * NT, r = idx / (DK / VE), c0 = (idx % (DK / VE)) * VE;
      if (idx < L * (DK / VE)) {
        float gv[VE];
#pragma unroll
        for (int e = 0; e < VE; ++e)
          gv[e] = r < len ? log_decay(p.raw.g_per_head ? to_f32(xgh[i]) : piece_elem<RawT>(xg[i], e),
                                      p.raw.gate_mode, p.raw.lb)
                          : 0.f;
#pragma unroll
        for (int e = 0; e < VE; e += 4)
          *reinterpret_cast<float4*>(&sG[r * PK + c0 + e]) = make_float4(gv[e], gv[e + 1], gv[e + 2], gv[e + 3]);
      }
    }
    if (t < L) sBeta[t] = t < len ? sigmoid(to_f32(braw)) : 0.f;
  } else {
    for (int idx = t; idx < L * (DK / 4); idx += NT) {
      const int r = idx / (DK / 4), c4 = 4 * (idx % (DK / 4));
      float4 kk = {0.f, 0.f, 0.f, 0.f}, qq = kk, gg = kk;
      if (r < len) {
        const int64_t off = ((start + r) * H + h) * DK + c4;
        kk = *reinterpret_cast<const float4*>(p.k + off);
        qq = *reinterpret_cast<const float4*>(p.q + off);
        gg = *reinterpret_cast<const float4*>(p.g + off);
      }
      *reinterpret_cast<float4*>(&sK[r * PK + c4]) = kk;
      *reinterpret_cast<float4*>(&sQ[r * PK + c4]) = qq;
      *reinterpret_cast<float4*>(&sG[r * PK + c4]) = gg;
    }
    if (t < L) sBeta[t] = t < len ? p.beta[(start + t) * H + h] : 0.f;
  }
  if (t == 0) sFlag[0] = 0;
  __syncthreads();

  // 2. per (block R, key dim d): gl_r = sum of g over rows 16R+1..r (block-local prefix)
  if (t < 4 * DK) {  // the block's 16 values are read at once, then summed in registers
    const int R = t / DK, d = t % DK;
    float gv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) gv[i] = sG[(16 * R + i) * PK + d];
    sG0[R * DK + d] = gv[0];
    sG[(16 * R) * PK + d] = 0.f;
    float run = 0.f;
#pragma unroll
    for (int i = 1; i < 16; ++i) {
      run += gv[i];
      sG[(16 * R + i) * PK + d] = run;
    }
    if (-run > kSpanGuard) atomicOr(sFlag, 1);  // the block's decay span G_{16R} - G_{16R+15}
  }
  __syncthreads();

  // 3. per key dim, from block-local sums: T_R = G_{16R+16} - G_{16R}, and the exponentials of the
  //    pivoted path: e^{G_{16R}}, e^{G_last - G_{16I+16}} (I < 3) or e^{G_last - G_48},
  //    e^{G_{16R} - G_{16I+16}} for the off-diagonal block pairs, e^{T_I}, and gamma_L (which
  //    the exact path rewrites from its own sums: which path the chunk takes is known after
  //    the barrier).  One thread per (block R, key dim d); every sum runs over J in order.
  if (t < 4 * DK) {
    const int R = t / DK, d = t % DK;
    float T[3];
#pragma unroll
    for (int J = 0; J < 3; ++J) T[J] = sG[(16 * J + 15) * PK + d] + sG0[(J + 1) * DK + d];
    const int Rl = (len - 1) / 16;
    const float glL = sG[(len - 1) * PK + d];
    const float g0 = sG0[d];
    float gf = g0;  // G_{16R}
    for (int J = 0; J < R; ++J) gf += T[J];
    sGFe[R * DK + d] = pexp<POL>(gf);
    float x = 0.f;  // G_last - G_{16R}: blocks past the last row hold only zero rows
    if (R <= Rl) {
      x = glL;
      for (int J = R; J < Rl; ++J) x += T[J];
    }
    sXe[R * DK + d] = pexp<POL>(R < 3 ? x - T[R] : x);
    for (int I = 0; I + 1 < R; ++I) {
      float dd = 0.f;
      for (int J = I + 1; J < R; ++J) dd += T[J];
      sD[pair_index(R, I) * DK + d] = pexp<POL>(dd);
    }
    if (R < 3) {
      sET[R * DK + d] = pexp<POL>(T[R]);
      if (-T[R] > kBlockDecayGuard) atomicOr(sFlag, 1);
    } else {
      float glast = g0;
      for (int J = 0; J < Rl; ++J) glast += T[J];
      reinterpret_cast<float*>(rec + rl.gL)[d] = pexp<POL>(glast + glL);
    }
  }
  __syncthreads();
  const bool exact = sFlag[0] != 0;

  // 4. exact path.  Its exponents are differences G_r - G_i of prefix sums over the chunk,
  //    G_r = g_0 + ... + g_r, which grow to thousands under steep decay; a prefix sum
  //    rounded to fp32 would carry that magnitude's rounding into every difference.  So
  //    each G_r is kept as an unevaluated sum hi + lo of two fp32 numbers, accumulated
  //    with Knuth's two-sum (the rounding error of every addition goes into lo), and a
  //    difference is (hi_r - hi_i) + (lo_r - lo_i), exact up to its own last rounding.
  //    The log decays are read again from their source and recomputed by the same
  //    function as in step 1, so they are the same values.  hi replaces gl in T2, lo
  //    lives over the A and P tiles until the pair products are stored.  Then the
  //    operand fragments of Q^gamma = e^{G_r} q_r and K_<^T (e^{G_last - G_i} k_i) and
  //    gamma_L, one exponential per element (the pivoted path forms them from its
  //    factors in step 5).
  float* sGlo = sA;  // [L][PK] over the A and P tiles (exact path only)
  static_assert(L * PK <= 2 * L * PL, "the low parts fit over the A and P tiles");
  const int last = len - 1;
  if (exact) {
    for (int idx = t; idx < L * DK; idx += NT) {
      const int r = idx / DK, d = idx % DK;
      float gr = 0.f;
      if (r < len) {
        if constexpr (FUSED) {
          const RawT* rg = static_cast<const RawT*>(p.raw.g);
          gr = log_decay(to_f32(p.raw.g_per_head ? rg[(start + r) * H + h] : rg[((start + r) * H + h) * DK + d]),
                         p.raw.gate_mode, p.raw.lb);
        } else {
          gr = p.g[((start + r) * H + h) * DK + d];
        }
      }
      sG[r * PK + d] = gr;
    }
    __syncthreads();
    if (t < DK) {  // one key dim per thread, rows in order
      float hi = 0.f, lo = 0.f;
      for (int r = 0; r < L; ++r) {
        const float gr = sG[r * PK + t];
        const float sum = hi + gr, bv = sum - hi;
        lo += (hi - (sum - bv)) + (gr - bv);
        hi = sum;
        sG[r * PK + t] = hi;
        sGlo[r * PK + t] = lo;
      }
    }
    __syncthreads();
    if (t >= 3 * DK && t < 4 * DK) {  // the thread that wrote gamma_L in step 3
      const int d = t - 3 * DK;
      reinterpret_cast<float*>(rec + rl.gL)[d] = pexp<POL>(sG[last * PK + d] + sGlo[last * PK + d]);
    }
    write_afrags<POL, NT>(rec + rl.Qf, 4, DK / 32, [&](int r, int d) {
      return sQ[r * PK + d] * pexp<POL>(sG[r * PK + d] + sGlo[r * PK + d]);
    });
    write_afrags<POL, NT>(rec + rl.Kf, DK / 16, 2, [&](int d, int r) {
      return sK[r * PK + d] *
             pexp<POL>((sG[last * PK + d] - sG[r * PK + d]) + (sGlo[last * PK + d] - sGlo[r * PK + d]));
    });
    __syncthreads();
  }

  // 5. A and P.  Per block pair (R, I <= R), with pivots at the blocks' first rows:
  //      A_ri = b_r sum_d [k_r e^{gl_r}] E_RI [k_i e^{T_I - gl_i}]     (I < R)
  //      A_ri = b_r sum_d [k_r e^{gl_r}]      [k_i e^{-gl_i}]          (I = R)
  //    with E_RI = e^{G_{16R} - G_{16I+16}} (1 for R = I + 1), and the same with q_r for P.
  //    Off the diagonal every factor is at most 1, so a factor that underflows
  //    belongs to a term below e^-87; on the diagonal the span guard keeps both
  //    factors within e^{+-80}.  The factors are formed once per chunk in place
  //    (already split for split products): T0 = k e^{gl}, T1 = q e^{gl},
  //    T2 = k e^{-gl}, and k e^{T_I - gl} for blocks 0..2 over the A / P tiles;
  //    each wavefront then computes whole block pairs, A and P together, sharing
  //    the right operand, which carries E_RI where it is not 1.
  //    Q^gamma and K_<^T come from the same factors, one product each:
  //      e^{G_r} q_r = e^{G_{16R}} (q_r e^{gl_r}),
  //      e^{G_last - G_i} k_i = e^{G_last - G_{16I+16}} (k_i e^{T_I - gl_i})   (I < 3)
  //                           = e^{G_last - G_48} (k_i e^{-gl_i})             (I = 3)
  //    (every factor at most 1, or within the span guard for the last block),
  //    with the per-(block, key dim) exponentials of step 3 in place of G_{16R}
  //    and G_last - G_{16I}, and
  //    k e^{T_I - gl} = (k e^{-gl}) e^{T_I}, one product.
  if (!exact) {
    float* sRk = sA;  // [48][PK] k e^{T_I - gl}, over the A and P tiles until the products are done
    // With record fragments of 8 consecutive key dims (fp16 and split-bf16 records), the two
    // lanes that hold the 4-dim halves of a group write its Q^gamma = e^{G_{16R}} (q e^{gl})
    // fragment from their registers, half each; fp32 records (strided K order) go through the
    // factor tile later.
    using FR = Frag<POL>;
    constexpr bool kQfDirect = FR::kof(1, 0) == 8;
    for (int idx = t; idx < L * (DK / 4); idx += NT) {
      const int r = idx / (DK / 4), d4 = 4 * (idx % (DK / 4));
      const float4 kk = *reinterpret_cast<const float4*>(&sK[r * PK + d4]);
      const float4 qq = *reinterpret_cast<const float4*>(&sQ[r * PK + d4]);
      const float4 gg = *reinterpret_cast<const float4*>(&sG[r * PK + d4]);
      const float4 ee = *reinterpret_cast<const float4*>(&sET[min(r >> 4, 2) * DK + d4]);  // used for r < 48
      const float kv[4] = {kk.x, kk.y, kk.z, kk.w}, qv[4] = {qq.x, qq.y, qq.z, qq.w}, gv[4] = {gg.x, gg.y, gg.z, gg.w};
      const float ev[4] = {ee.x, ee.y, ee.z, ee.w};
      float lk[4], lq[4], rd[4], rk[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float ep = pexp<POL>(gv[e]);
        lk[e] = kv[e] * ep;
        lq[e] = qv[e] * ep;
        rd[e] = kv[e] * pexp<POL>(-gv[e]);
        rk[e] = rd[e] * ev[e];  // k e^{T_I - gl}: e^{-gl} <= e^80 and e^{T_I} >= e^-86, both normal
      }
      FT::store4(sK, r, d4, lk);
      FT::store4(sQ, r, d4, lq);
      FT::store4(sG, r, d4, rd);
      if (r < 48) FT::store4(sRk, r, d4, rk);
      if constexpr (kQfDirect) {  // A fragment (row tile r / 16, K block d4 / 32), lane (r % 16) + 16 (d4 % 32) / 8
        const float4 gf = *reinterpret_cast<const float4*>(&sGFe[(r >> 4) * DK + d4]);
        const float qf[4] = {gf.x * lq[0], gf.y * lq[1], gf.z * lq[2], gf.w * lq[3]};
        const int item = ((r >> 4) * (DK / 32) + (d4 >> 5)) * 64 + (r & 15) + 16 * ((d4 & 31) >> 3);
        FR::store_a_half(rec + rl.Qf + (size_t)item * FR::BYTES, (d4 >> 2) & 1, qf);
      }
    }
    __syncthreads();
    constexpr int NJ = (10 + NW - 1) / NW;  // block pairs per wavefront
    // pair indices in order (0,0) (1,0) (1,1) (2,0) (2,1) (2,2) (3,0) (3,1) (3,2) (3,3);
    // the three that carry a scale, (2,0) (3,0) (3,1), go to wavefronts 0..2
    // (packed 4 bits per entry, so that the lookup is arithmetic: a constant table is read
    // with a vector load, and its wait would also drain the record stores in flight)
    constexpr uint64_t kPairOrder = 0x9854210763ull;  // 3, 6, 7, 0, 1, 2, 4, 5, 8, 9 from the low end
    auto pair_of = [&](int j) { const int w = wave + NW * j; return w < 10 ? (int)((kPairOrder >> (4 * w)) & 15) : 10; };
    floatx4 acc[NJ][2];  // [pair of this wavefront][A, P]
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int pr = pair_of(j);  // pairs in order (0,0) (1,0) (1,1) (2,0) (2,1) (2,2) (3,0) ...
      acc[j][0] = acc[j][1] = floatx4{0.f, 0.f, 0.f, 0.f};
      if (pr < 10) {
        int R = 0, I = pr;
        while (I > R) { I -= R + 1; ++R; }
        const float* right = I == R ? &sG[16 * I * PK] : &sRk[16 * I * PK];
        const float* scale = I + 1 < R ? &sD[pair_index(R, I) * DK] : nullptr;
        pair_mma<IP, DK, PK>(acc[j][0], acc[j][1], &sK[16 * R * PK], &sQ[16 * R * PK], right, scale);
      }
    }
    // the record's K_<^T (and, for fp32 records, Q^gamma) fragments from the same factors,
    // while the products run
    if constexpr (!kQfDirect)
      write_afrags<POL, NT>(rec + rl.Qf, 4, DK / 32, [&](int r, int d) {
        return sGFe[(r / 16) * DK + d] * FT::load1(sQ, r, d);
      });
    if constexpr (kQfDirect) {
      // an item's 8 chunk rows r0 .. r0 + 7 lie in one 16-row block: its factor e^{G_last - G_16I}
      // and its source tile are taken once
      for (int item = t; item < (DK / 16) * 2 * 64; item += NT) {
        const int ln = item & 63, blk = item >> 6;
        const int d = 16 * (blk >> 1) + (ln & 15), r0 = 32 * (blk & 1) + 8 * (ln >> 4), R = r0 >> 4;
        const float* src = R < 3 ? sRk : sG;
        const float xe = sXe[R * DK + d];
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = xe * FT::load1(src, r0 + e, d);
        FR::store_a(rec + rl.Kf + (size_t)item * FR::BYTES, x);
      }
    } else {
      write_afrags<POL, NT>(rec + rl.Kf, DK / 16, 2, [&](int d, int r) {
        return sXe[(r / 16) * DK + d] * FT::load1(r < 48 ? sRk : sG, r, d);
      });
    }
    __syncthreads();  // every wavefront is done with the factors over A and P
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int pr = pair_of(j);
      if (pr < 10) {
        int R = 0, I = pr;
        while (I > R) { I -= R + 1; ++R; }
        const int col = lane & 15, g4 = lane >> 4;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int rr = 16 * R + 4 * g4 + v, ii = 16 * I + col;
          sA[rr * PL + ii] = (ii < rr) ? sBeta[rr] * acc[j][0][v] : 0.f;
          sP[rr * PL + ii] = (ii <= rr) ? acc[j][1][v] : 0.f;
        }
      }
    }
    // P's strictly-upper blocks (0,1) (0,2) (0,3) (1,2) (1,3) (2,3) are zero in its record
    // fragments; A's are never read (the solve reads its diagonal and lower blocks only)
    for (int idx = t; idx < 6 * 256; idx += NT) {
      const int b = idx >> 8, R = b < 3 ? 0 : b < 5 ? 1 : 2, I = b < 3 ? b + 1 : b < 5 ? b - 1 : 3;
      sP[(16 * R + ((idx >> 4) & 15)) * PL + 16 * I + (idx & 15)] = 0.f;
    }
  } else {
    // exact path: every pair (r, i <= r) with one exponential of G_r - G_i per key dim, the
    // difference taken from the two-sum prefixes of step 4; the sums are kept in registers
    // until every thread is done reading the low parts over the A and P tiles
    constexpr int NPR = (L * L + NT - 1) / NT;
    float sa[NPR], sp[NPR];
#pragma unroll
    for (int j = 0; j < NPR; ++j) {
      const int pr = t + j * NT, r = pr / L, i = pr % L;
      sa[j] = sp[j] = 0.f;
      if (pr < L * L && i <= r) {
        for (int d = 0; d < DK; ++d) {
          const float dg = (sG[r * PK + d] - sG[i * PK + d]) + (sGlo[r * PK + d] - sGlo[i * PK + d]);
          const float e = expf(dg);
          sa[j] = fmaf(sK[r * PK + d] * sK[i * PK + d], e, sa[j]);
          sp[j] = fmaf(sQ[r * PK + d] * sK[i * PK + d], e, sp[j]);
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NPR; ++j) {
      const int pr = t + j * NT, r = pr / L, i = pr % L;
      if (pr < L * L) {
        sA[r * PL + i] = (i < r) ? sBeta[r] * sa[j] : 0.f;
        sP[r * PL + i] = (i <= r) ? sp[j] : 0.f;
      }
    }
  }
  // the v rows for step 7 go to T1, which nothing reads any more: fused, the staged raw rows
  // (16-byte pieces, loaded with the preamble's rows); unfused, the rows b_r v_r in fp32
  if constexpr (kVStaged) {
    static_assert((L + 3) * DV * sizeof(RawT) <= (size_t)L * PK * sizeof(float), "staged v rows fit in T1");
    RawT* stv = reinterpret_cast<RawT*>(sQ);
#pragma unroll
    for (int i = 0; i < NSV; ++i) store_staged(stv, DV, t + i * NT, xv[i]);
    if (seq_first)
#pragma unroll
      for (int i = 0; i < NSV; ++i) store_halo(stv, DV, chv, t + i * NT);
  } else if constexpr (!FUSED) {
    for (int idx = t; idx < L * (DV / 4); idx += NT) {
      const int r = idx / (DV / 4), c4 = 4 * (idx % (DV / 4));
      float4 vv = {0.f, 0.f, 0.f, 0.f};
      if (r < len) vv = *reinterpret_cast<const float4*>(p.v + ((start + r) * H + h) * DV + c4);
      const float b = sBeta[r];
      vv.x *= b; vv.y *= b; vv.z *= b; vv.w *= b;
      *reinterpret_cast<float4*>(&sQ[r * PK + c4]) = vv;
    }
  }
  __syncthreads();
  write_afrags<POL, NT>(rec + rl.Pf, 4, 2, [&](int r, int i) { return sP[r * PL + i]; });
  __syncthreads();  // P's last read: X takes its tile

  // 6 and 7 side by side.  X = (I + A)^{-1} goes into the P tile.  Only wavefronts 0..3 take
  // part in the solve, so the right-hand sides of step 8, which do not depend on X, are formed
  // by the other wavefronts meanwhile, as B-operand fragments of the intra products (an item
  // (column tile c, 32-row block kb, lane) holds 8 rows of one column):
  //   b_r e^{G_r} k_r (wavefronts 4..15, while the diagonal blocks are solved) into T2,
  //   b_r v_r (wavefronts 8..15, while the blocks below the diagonal are solved) into T0.
  // e^{G_r} k_r is e^{G_{16R}} (k_r e^{gl_r}) from the factors of step 5, or formed directly
  // from the chunk prefix G_r on the exact path.
  // X's strictly-upper blocks keep the zeros of P's (step 8 reads blocks (0,1) and (2,3));
  // the solve writes the diagonal and lower blocks only.
  float* sXi = sP;
  using FI = Frag<IP>;
  using FB = typename FI::B;
  constexpr int NFK = (DK / 16) * 2 * 64, NFV = (DV / 16) * 2 * 64;
  constexpr int EV = DV / 64, NKT = NT - 4 * 64, PFK = (NFK + NKT - 1) / NKT;  // b e^G k items per thread
  static_assert(NW == 16, "wavefront roles: 4 solve, 12 b e^G k, 8 of them b v");
  FB fk[PFK];
  if (wave < 4) {  // diagonal block R = wavefront, by forward substitution
    // lane 4 cc + qq owns column cc, rows 4 qq .. 4 qq + 3 of the block.  Right-looking:
    // once x_r is final it is broadcast in the lane quad and every later row takes its
    // term, in the order r = 0, 1, ... (rows at or above r see a zero of A's strictly
    // lower block and keep their value).
    const int R = wave, b0 = 16 * R, cc = lane >> 2, qq = lane & 3;
    float xv4[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) xv4[j] = (4 * qq + j == cc) ? 1.f : 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      constexpr int kQuad[4] = {0x00, 0x55, 0xAA, 0xFF};  // quad_perm broadcast of lane 0..3 of each quad
      float x = xv4[r & 3];
      if ((r >> 2) == 0) x = dpp_partner<kQuad[0]>(x);
      else if ((r >> 2) == 1) x = dpp_partner<kQuad[1]>(x);
      else if ((r >> 2) == 2) x = dpp_partner<kQuad[2]>(x);
      else x = dpp_partner<kQuad[3]>(x);
      x = (r >= cc) ? x : 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) xv4[j] = fmaf(-sA[(b0 + 4 * qq + j) * PL + b0 + r], x, xv4[j]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) sXi[(b0 + 4 * qq + j) * PL + b0 + cc] = xv4[j];
  } else {
    // exact path: T2 holds the chunk prefix G_r (its high part); else e^{G_{16R}} times the factor k e^{gl}
    auto fk_item = [&](int item, auto&& elem) {
      const int ln = item & 63, kb = (item >> 6) & 1, c = item >> 7;
      const int d = 16 * c + (ln & 15), g = ln >> 4;
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = elem(32 * kb + FI::kof(g, e), d);
      return FI::make_b(x);
    };
    if (exact) {
#pragma unroll
      for (int i = 0; i < PFK; ++i)
        if ((t - 256) + i * NKT < NFK)
          fk[i] = fk_item((t - 256) + i * NKT, [&](int r, int d) {
            return sBeta[r] * (sK[r * PK + d] * pexp<POL>(sG[r * PK + d]));
          });
    } else if constexpr (FI::kof(1, 0) == 8) {
      // an item's 8 rows r0 .. r0 + 7 are consecutive and lie in one 16-row block: its b_r
      // load as two 16-byte vectors and e^{G_{16R}} once
#pragma unroll
      for (int i = 0; i < PFK; ++i) {
        const int item = (t - 256) + i * NKT;
        if (item < NFK) {
          const int ln = item & 63, kb = (item >> 6) & 1, c = item >> 7;
          const int d = 16 * c + (ln & 15), r0 = 32 * kb + 8 * (ln >> 4);
          const float4 b0 = *reinterpret_cast<const float4*>(&sBeta[r0]);
          const float4 b1 = *reinterpret_cast<const float4*>(&sBeta[r0 + 4]);
          const float bb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
          const float ge = sGFe[(r0 >> 4) * DK + d];
          float x[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = bb[e] * (FT::load1(sK, r0 + e, d) * ge);
          fk[i] = FI::make_b(x);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < PFK; ++i)
        if ((t - 256) + i * NKT < NFK)
          fk[i] = fk_item((t - 256) + i * NKT, [&](int r, int d) {
            return sBeta[r] * (FT::load1(sK, r, d) * sGFe[(r >> 4) * DK + d]);
          });
    }
  }
  __syncthreads();  // the diagonal blocks of X are final; every read of T0 and T2 is done
  if (wave < 3) {
    // column I = wavefront of X below the diagonal, on the matrix cores (fp32), nearest block first:
    //   Y = sum_{J=I}^{R-1} A_RJ X_JI,  X_RI = -X_RR Y
    // Block (R, I) reads the blocks above it in its own column, which this wavefront wrote
    // (a wavefront's LDS accesses take effect in program order), and X_RR, final at the barrier.
    const int I = wave, col = lane & 15, g4 = lane >> 4;
    float* yb = sY + wave * 16 * 17;  // this wavefront's own scratch: written, then read back in order
    // block (I + D, I) with a compile-time K = 16 D, so that all of its operands are read from
    // LDS before the products that use them
    auto block = [&](auto dist) {
      constexpr int D = decltype(dist)::value;
      const int R = I + D;
      float ao[4 * D], xo[4 * D];
#pragma unroll
      for (int j = 0; j < 4 * D; ++j) {
        ao[j] = sA[(16 * R + col) * PL + 16 * I + 4 * j + g4];
        xo[j] = sXi[(16 * I + 4 * j + g4) * PL + 16 * I + col];
      }
      floatx4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4 * D; ++j) y = __builtin_amdgcn_mfma_f32_16x16x4f32(ao[j], xo[j], y, 0, 0, 0);
#pragma unroll
      for (int v = 0; v < 4; ++v) yb[(4 * g4 + v) * 17 + col] = y[v];
      float xr[4], yr[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        xr[j] = sXi[(16 * R + col) * PL + 16 * R + 4 * j + g4];
        yr[j] = yb[(4 * j + g4) * 17 + col];
      }
      floatx4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) x = __builtin_amdgcn_mfma_f32_16x16x4f32(xr[j], yr[j], x, 0, 0, 0);
#pragma unroll
      for (int v = 0; v < 4; ++v) sXi[(16 * R + 4 * g4 + v) * PL + 16 * I + col] = -x[v];
    };
    block(std::integral_constant<int, 1>{});
    if (I < 2) block(std::integral_constant<int, 2>{});
    if (I < 1) block(std::integral_constant<int, 3>{});
  } else {
    if constexpr (FUSED) {
      // Wavefronts 3..7 have little to do here: they read one word of every 128-byte line of
      // the raw q and k rows that item b + lookahead (the next to run on this XCD) reads
      // first, so that those rows wait in the XCD's L2 when its workgroup starts, instead
      // of every CU's first loads meeting in HBM at once.  The words are waited for here,
      // inside this interval, so no later wait on the in-order memory counter includes them.
      const int64_t it2 = (int64_t)blockIdx.x + p.lookahead;
      if (wave < 8 && p.lookahead > 0 && it2 < (int64_t)gridDim.x) {
        const int c2 = (int)(it2 / H), h2 = (int)(it2 % H);
        const int n2 = slot_seq(p.cu, p.num_seqs, c2);
        const int64_t t02 = p.cu[n2], s2 = t02 + (c2 - slot_base(p.cu, n2)) * L, e2 = p.cu[n2 + 1];
        if (s2 < e2) {
          constexpr int LPR = (int)(DK * sizeof(RawT) / 128);  // 128-byte lines per row of a stream
          constexpr int NL = 2 * (L + 3) * LPR;
          uint32_t acc = 0;
          for (int li = t - 192; li < NL; li += 320) {
            const int st = li / ((L + 3) * LPR), rem = li % ((L + 3) * LPR), sr = rem / LPR, part = rem % LPR;
            int64_t pos = s2 - 3 + sr;
            pos = pos < t02 ? t02 : (pos >= e2 ? e2 - 1 : pos);  // within the sequence's rows
            const RawT* src = static_cast<const RawT*>(st ? p.raw.k : p.raw.q);
            acc += *reinterpret_cast<const uint32_t*>(src + pos * ((int64_t)H * DK) + (int64_t)h2 * DK +
                                                      part * (128 / (int)sizeof(RawT)));
          }
          asm volatile("" ::"v"(acc));
        }
      }
    }
    if (wave >= 4) {
#pragma unroll
      for (int i = 0; i < PFK; ++i)
        if ((t - 256) + i * NKT < NFK) put_frag(sG, NFK, (t - 256) + i * NKT, fk[i]);
      if (wave >= 8) {
        // v wavefront 8 + 4 kb + g takes chunk rows 32 kb + kof(g, e), e < 8, and writes one
        // fragment per column; lane l holds columns EV l .. EV l + EV - 1
        const int vkb = (wave - 8) >> 2, vg = wave & 3;
        auto vrow = [&](int e) { return 32 * vkb + FI::kof(vg, e); };
        float x[8][EV];
        if constexpr (FUSED) {  // conv (no norm) of the wavefront's 8 rows, then b_r v_r
          if constexpr (kVStaged) {
            const RawT* stv = reinterpret_cast<const RawT*>(sQ);
            conv_rows<DV, false, 8>([&](int rr, int j, int d) { return to_f32(stv[(vrow(rr) + j) * DV + d]); }, cwv,
                                    p.raw.act, x);
          } else {
            const RawT* rv = static_cast<const RawT*>(p.raw.v);
            const int64_t wv = (int64_t)H * DV, rel0 = start - t0;
            conv_rows<DV, false, 8>([&](int rr, int j, int d) {
              const int64_t pos = rel0 + vrow(rr) - 3 + j;
              if (vrow(rr) >= len) return 0.f;
              return pos >= 0 ? to_f32(rv[(t0 + pos) * wv + (int64_t)h * DV + d]) : to_f32(raw_cs[(3 + pos) * Cch + chv + d]);
            }, cwv, p.raw.act, x);
          }
          float bb[8];
          if constexpr (FI::kof(1, 0) == 8) {  // 8 consecutive rows: b_r as two 16-byte vectors
            const float4 b0 = *reinterpret_cast<const float4*>(&sBeta[vrow(0)]);
            const float4 b1 = *reinterpret_cast<const float4*>(&sBeta[vrow(4)]);
            bb[0] = b0.x; bb[1] = b0.y; bb[2] = b0.z; bb[3] = b0.w; bb[4] = b1.x; bb[5] = b1.y; bb[6] = b1.z; bb[7] = b1.w;
          } else {
#pragma unroll
            for (int rr = 0; rr < 8; ++rr) bb[rr] = sBeta[vrow(rr)];
          }
#pragma unroll
          for (int rr = 0; rr < 8; ++rr)
#pragma unroll
            for (int e = 0; e < EV; ++e) x[rr][e] = vrow(rr) < len ? bb[rr] * x[rr][e] : 0.f;
        } else {
#pragma unroll
          for (int rr = 0; rr < 8; ++rr)
#pragma unroll
            for (int e = 0; e < EV; ++e) x[rr][e] = sQ[vrow(rr) * PK + EV * lane + e];
        }
#pragma unroll
        for (int e = 0; e < EV; ++e) {
          float y[8];
#pragma unroll
          for (int rr = 0; rr < 8; ++rr) y[rr] = x[rr][e];
          const int d = EV * lane + e;
          put_frag(sK, NFV, ((d >> 4) * 2 + vkb) * 64 + (d & 15) + 16 * vg, FI::make_b(y));
        }
      }
    }
  }
  __syncthreads();

  // 8. W = X (b K^gamma), U~ = X (b V).  X is lower triangular, so row block R
  //    needs K = 16(R+1) rounded up to 32.  NW / 4 wavefronts per row block R, each
  //    holding its split rows of X and taking an equal share of the W and U~ column tiles.
  //    U~ goes to the record in result layout; W through LDS (T1) into fragments.
  {
    constexpr int NTW = DK / 16, NTU = DV / 16, NTT = NTW + NTU;
    // right-hand side fragments: b e^{G} k in T2 (NFK items), b v in T0 (NFV items)
    float* sW = sQ;  // the v rows in T1 are consumed
    constexpr int WPR = NW / 4, TPW = NTT / WPR;  // wavefronts per row block, column tiles per wavefront
    static_assert(NTT % WPR == 0, "column tiles split evenly");
    const int R = 3 - wave / WPR, part = wave % WPR, KBR = (16 * (R + 1) + 31) / 32;
    const int col = lane & 15, g4 = lane >> 4;
    typename FI::A xa[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = sXi[(16 * R + col) * PL + 32 * kb + FI::kof(g4, e)];
      xa[kb] = FI::make_b(x);
    }
    for (int c = part * TPW; c < (part + 1) * TPW; ++c) {
      const bool isW = c < NTW;
      const int cb = isW ? c : c - NTW;
      const float* bsrc = isW ? sG : sK;
      const int nb = isW ? NFK : NFV;
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        if (kb < KBR) acc = FI::mma(acc, xa[kb], get_frag<FB>(bsrc, nb, (cb * 2 + kb) * 64 + lane));
      if (!isW) *reinterpret_cast<floatx4*>(rec + rl.Ut + ((int64_t)(cb * 4 + R) * 64 + lane) * 16) = acc;
      else {
#pragma unroll
        for (int v = 0; v < 4; ++v) sW[(16 * R + 4 * g4 + v) * PK + 16 * cb + col] = acc[v];
      }
    }
    __syncthreads();
    write_afrags<POL, NT>(rec + rl.Wf, 4, DK / 32, [&](int r, int d) { return sW[r * PK + d]; });
  }
}

// ---------------------------------------------------------------------------
// inter-chunk scan
//
// Workgroup = (sequence, head, CB blocks of 16 state columns from j0), 8
// wavefronts in two roles, so that only the state recurrence sits on the serial
// path.  State wavefront w (0..3) owns chunk rows 16w..16w+15 of U and state
// rows 16*(w*DK/64 + s) + 0..15 (s < DK/64), kept as fp32 matrix-core
// accumulators; output wavefront 4 + w owns chunk rows 16w..16w+15 of O.  Per chunk c, with
// S_c^T and U_c^T slices shared through LDS:
//   phase 1 (S_c complete):  U_c = U~_c - W_c S_c  (state),  O_c = Q^gamma_c S_c  (output)
//   phase 2 (U_c complete):  S_{c+1} = gamma_L . S_c + K_<^T U_c  (state),  O_c += P_c U_c  (output)
// Phase 1 reads S^T and writes U^T; phase 2 reads U^T and writes S^T; the two
// barriers per chunk order every write after the last read of the old
// contents, so one buffer of each suffices.  Each wavefront keeps NS register
// sets of its operand fragments and loads chunk c+NS-1 while chunk c computes.
//
// With CB = 2 or 4 a workgroup takes that many column blocks and each wavefront
// applies its W, K_<^T, Q^gamma and P fragments to all of them: 1/CB of the
// operand traffic per state column, for a chain CB times as long per chunk.
// Each column's arithmetic is the same for every CB, so all give the same bits.
// It pays where the operand loads bound the scan, that is where the workgroups
// fill every CU.
// ---------------------------------------------------------------------------
template <int DK, int POL, int CB>
struct ScanSmem {
  using P = typename Frag<POL>::P;
  static constexpr int NP = Frag<POL>::PLANES;
  // row strides padded by 32 bytes (16 bytes measured slower on the LDS)
  static constexpr int PS = DK + 32 / sizeof(P);  // S^T row stride (one row per state column)
  static constexpr int PU = 64 + 32 / sizeof(P);  // U^T row stride
  static constexpr int S_PLANE = 16 * CB * PS, U_PLANE = 16 * CB * PU;
  static constexpr size_t BYTES = (size_t)(NP * S_PLANE + NP * U_PLANE) * sizeof(P);
  static_assert(BYTES <= 65536, "the scan runs with the default LDS limit");
};

// one chunk's operand fragments of a state wavefront: the state chain's
// operands (W, U~, K_<^T, gamma_L)
template <int DK, int POL, int CB>
struct StateFrags {
  using F = Frag<POL>;
  static constexpr int KB = DK / 32, MS = DK / 64;
  typename F::A w[KB], k[MS][2];
  floatx4 ut[CB];
  float4 gl[MS];
  // in three groups, so that each iteration can spread its loads over the chunk
  __device__ void load_w(const uint8_t* rec, const RecLayout& rl, int w4, int lane) {
    constexpr int FB = F::BYTES;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) w[kb] = F::load_a(rec + rl.Wf + ((int64_t)(w4 * KB + kb) * 64 + lane) * FB);
  }
  // split0: the workgroup's first 16-column block
  __device__ void load_ug(const uint8_t* rec, const RecLayout& rl, int w4, int lane, int split0) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
      ut[cb] = *reinterpret_cast<const floatx4*>(rec + rl.Ut + ((int64_t)((split0 + cb) * 4 + w4) * 64 + lane) * 16);
#pragma unroll
    for (int s = 0; s < MS; ++s)
      gl[s] = *reinterpret_cast<const float4*>(rec + rl.gL + (int64_t)(16 * (w4 * MS + s) + 4 * (lane >> 4)) * 4);
  }
  __device__ void load_k(const uint8_t* rec, const RecLayout& rl, int w4, int lane) {
    constexpr int FB = F::BYTES;
#pragma unroll
    for (int s = 0; s < MS; ++s)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        k[s][kb] = F::load_a(rec + rl.Kf + ((int64_t)((w4 * MS + s) * 2 + kb) * 64 + lane) * FB);
  }
  __device__ void load(const uint8_t* rec, const RecLayout& rl, int w4, int lane, int split0) {
    load_w(rec, rl, w4, lane);
    load_ug(rec, rl, w4, lane, split0);
    load_k(rec, rl, w4, lane);
  }
};

// one chunk's operand fragments of an output wavefront (Q^gamma, and P up to
// the diagonal: row block w4 needs chunk rows < 16 (w4 + 1))
template <int DK, int POL>
struct OutFrags {
  using F = Frag<POL>;
  static constexpr int KB = DK / 32;
  typename F::A q[KB], pp[2];
  __device__ void load_q(const uint8_t* rec, const RecLayout& rl, int w4, int lane) {
    constexpr int FB = F::BYTES;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) q[kb] = F::load_a(rec + rl.Qf + ((int64_t)(w4 * KB + kb) * 64 + lane) * FB);
  }
  __device__ void load_p(const uint8_t* rec, const RecLayout& rl, int w4, int lane) {
    constexpr int FB = F::BYTES;
    pp[0] = F::load_a(rec + rl.Pf + ((int64_t)(w4 * 2) * 64 + lane) * FB);
    if (w4 >= 2) pp[1] = F::load_a(rec + rl.Pf + ((int64_t)(w4 * 2 + 1) * 64 + lane) * FB);
  }
  __device__ void load(const uint8_t* rec, const RecLayout& rl, int w4, int lane) {
    load_q(rec, rl, w4, lane);
    load_p(rec, rl, w4, lane);
  }
};

// Conv-state carry of a prompt pass with raw rows: conv_state_out[slot][r][c]
// = raw row (len - 3 + r) of channel c, reaching back into conv_state_in for
// sequences shorter than 3 rows.  Runs after every read of the old conv state
// (the intra-chunk kernel is done), so the two may be one buffer; the channels
// of a sequence are spread over its nwg scan workgroups, and each thread writes
// rows r = 0, 1, 2 of its channel in order (with in == out, row r reads old row
// r + len >= r, so nothing is overwritten before it is read).
template <typename E>
__device__ __forceinline__ void carry_rows(const PrefillArgs& p, int n, int slot, int64_t c, int64_t C, int64_t qk,
                                           int64_t vw) {
  const int64_t t0 = p.cu[n], len = (int64_t)p.cu[n + 1] - t0;
  const E* in = static_cast<const E*>(p.raw.cs_in) + (int64_t)slot * 3 * C;
  E* out = static_cast<E*>(p.raw.cs_out) + (int64_t)slot * 3 * C;
  if (len >= 3) {  // (uniform over the sequence) every row comes from the packed rows: three loads, then the stores
    const E* src = c < qk ? static_cast<const E*>(p.raw.q) + c
                 : c < 2 * qk ? static_cast<const E*>(p.raw.k) + (c - qk)
                              : static_cast<const E*>(p.raw.v) + (c - 2 * qk);
    const int64_t width = c < 2 * qk ? qk : vw;
    E x[3];
#pragma unroll
    for (int r = 0; r < 3; ++r) x[r] = src[(t0 + len - 3 + r) * width];
#pragma unroll
    for (int r = 0; r < 3; ++r) out[r * C + c] = x[r];
    return;
  }
  for (int r = 0; r < 3; ++r) {
    const int64_t pos = len - 3 + r;
    E x;
    if (pos >= 0) {
      const int64_t row = t0 + pos;
      if (c < qk) x = static_cast<const E*>(p.raw.q)[row * qk + c];
      else if (c < 2 * qk) x = static_cast<const E*>(p.raw.k)[row * qk + (c - qk)];
      else x = static_cast<const E*>(p.raw.v)[row * vw + (c - 2 * qk)];
    } else {
      x = in[(3 + pos) * C + c];
    }
    out[r * C + c] = x;
  }
}
template <int DK, int DV>
__device__ __forceinline__ void carry_conv_state(const PrefillArgs& p, int n, int slot, int wid, int nwg) {
  const int64_t C = (int64_t)p.H * (2 * DK + DV), qk = (int64_t)p.H * DK, vw = (int64_t)p.H * DV;
  const int64_t per = (C + nwg - 1) / nwg;
  for (int64_t e = threadIdx.x; e < per; e += blockDim.x) {
    const int64_t c = wid * per + e;
    if (c >= C) break;
    if (p.raw.esize == 2) carry_rows<uint16_t>(p, n, slot, c, C, qk, vw);
    else carry_rows<uint32_t>(p, n, slot, c, C, qk, vw);
  }
}

template <int DK, int DV, int POL, int CB>
__global__ __launch_bounds__(512) void chunk_scan_kernel(PrefillArgs p, int groups) {
  using SM = ScanSmem<DK, POL, CB>;
  using F = Frag<POL>;
  using P = typename F::P;
  constexpr int L = kChunk, PS = SM::PS, PU = SM::PU;
  constexpr int NSPLIT = DV / (16 * CB), KB = DK / 32, MS = DK / 64;
  constexpr int NS = F::BYTES == 16 && CB == 1 ? 3 : 2;  // register sets of operand fragments
  extern __shared__ __align__(16) float smem_f[];
  P* smem = reinterpret_cast<P*>(smem_f);

  // workgroups of one (sequence, head) share its chunk records: keep them on one XCD
  // (workgroups are dealt round-robin over the 8 XCDs by linear id)
  const int id = blockIdx.x, xcd = id % 8, kq = id / 8;
  const int grp = (kq / NSPLIT) * 8 + xcd, split = kq % NSPLIT;
  if (grp >= groups) return;
  const int H = p.H, n_seq = grp / H, h = grp % H;
  const int slot = p.slots ? p.slots[n_seq] : n_seq;
  if (slot < 0) return;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, w4 = wave & 3;
  const int col = lane & 15, g4 = lane >> 4;
  const int j0 = 16 * CB * split;
  if (p.raw.esize) carry_conv_state<DK, DV>(p, n_seq, slot, h * NSPLIT + split, H * NSPLIT);
  const RecLayout rl = rec_layout(DK, DV, F::BYTES);
  float* Sg = p.state + ((int64_t)slot * H + h) * DK * DV;
  P* sS0 = smem;
  P* sS1 = smem + (SM::NP - 1) * SM::S_PLANE;
  P* sU0 = smem + SM::NP * SM::S_PLANE;
  P* sU1 = sU0 + (SM::NP - 1) * SM::U_PLANE;
  // S^T and U^T rows per state column: column 16 cb + col of the workgroup's block (the row
  // offsets stay separate pointer steps, so that they fold into the LDS instructions' offsets)
  P* const sSc0 = sS0 + col * PS;
  P* const sSc1 = sS1 + col * PS;
  P* const sUc0 = sU0 + col * PU;
  P* const sUc1 = sU1 + col * PU;
  auto put_s = [&](int cb, int row0, const floatx4& x) {
    F::store_b4(sSc0 + 16 * cb * PS + row0, sSc1 + 16 * cb * PS + row0, x);
  };
  auto put_u = [&](int cb, int row0, const floatx4& x) {
    F::store_b4(sUc0 + 16 * cb * PU + row0, sUc1 + 16 * cb * PU + row0, x);
  };
  auto get_s = [&](int cb, int kb) {
    return F::load_b(sSc0 + 16 * cb * PS + 32 * kb, sSc1 + 16 * cb * PS + 32 * kb, g4);
  };
  auto get_u = [&](int cb, int kb) {
    return F::load_b(sUc0 + 16 * cb * PU + 32 * kb, sUc1 + 16 * cb * PU + 32 * kb, g4);
  };

  const int64_t c_begin = slot_base(p.cu, n_seq);
  const int n = (int)((p.cu[n_seq + 1] - p.cu[n_seq] + L - 1) / L);
  const int64_t seq_start = p.cu[n_seq], seq_end = p.cu[n_seq + 1];
  auto rec_of = [&](int i) { return p.recs + ((int64_t)(c_begin + i) * H + h) * p.rec_bytes; };
  // Every load is unconditional (indices clamped to the last chunk), so the
  // compiler can count outstanding loads exactly and wait only for the set a
  // chunk needs.
  auto clampc = [&](int j) { return j < n ? j : n - 1; };
  // Both roles walk the chunks in step, two barriers per chunk:
  //   A: S_c^T complete (and every read of U_{c-1}^T done),
  //   B: U_c^T complete (and every read of S_c^T done).
  // Each K block of a product accumulates on its own and the blocks are summed
  // as a tree, so a chain holds at most two dependent products and the matrix
  // cores have independent products to issue while one waits.
  const floatx4 z4 = {0.f, 0.f, 0.f, 0.f};
  if (wave < 4) {
    // state wavefronts: U_c = U~_c - W_c S_c, then S_{c+1} = gamma_L . S_c + K_<^T U_c
    floatx4 Sacc[CB][MS];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int s = 0; s < MS; ++s) {
        const int r0 = 16 * (w4 * MS + s) + 4 * g4;
#pragma unroll
        for (int v = 0; v < 4; ++v) Sacc[cb][s][v] = Sg[(int64_t)(r0 + v) * DV + j0 + 16 * cb + col];
        put_s(cb, r0, Sacc[cb][s]);
      }
    StateFrags<DK, POL, CB> fr[NS];
    if (n > 0) {
#pragma unroll
      for (int j = 0; j < NS - 1; ++j) fr[j].load(rec_of(clampc(j)), rl, w4, lane, CB * split);
    }
    auto iter = [&](int c, const StateFrags<DK, POL, CB>& cur, StateFrags<DK, POL, CB>& ahead) {
      // the next-but-one chunk's operands load in three groups (W right after A,
      // U~ and gamma after U is written, K_<^T while U_c^T is read), so no group
      // waits long for the CU's load path
      const uint8_t* nrec = rec_of(clampc(c + NS - 1));
      __syncthreads();  // A
      ahead.load_w(nrec, rl, w4, lane);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        typename F::B bs[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) bs[kb] = get_s(cb, kb);
        // one accumulator per K block (chains of one block's products), summed as a tree
        floatx4 acc[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) acc[kb] = F::mma(z4, cur.w[kb], bs[kb]);
        floatx4 ws = acc[0] + acc[1];
        if constexpr (KB == 4) ws = ws + (acc[2] + acc[3]);
        floatx4 u;
#pragma unroll
        for (int v = 0; v < 4; ++v) u[v] = cur.ut[cb][v] - ws[v];
        put_u(cb, 16 * w4 + 4 * g4, u);
      }
      __builtin_amdgcn_sched_barrier(0);
      ahead.load_ug(nrec, rl, w4, lane, CB * split);
      __syncthreads();  // B
      typename F::B u0[CB], u1[CB];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        u0[cb] = get_u(cb, 0);
        u1[cb] = get_u(cb, 1);
      }
      ahead.load_k(nrec, rl, w4, lane);
      __builtin_amdgcn_sched_barrier(0);
      floatx4 sk[CB][MS];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int s = 0; s < MS; ++s) {
          const float4 gl = cur.gl[s];
          floatx4& a = Sacc[cb][s];
          a[0] *= gl.x; a[1] *= gl.y; a[2] *= gl.z; a[3] *= gl.w;
          a = F::mma(a, cur.k[s][0], u0[cb]);
          sk[cb][s] = F::mma(z4, cur.k[s][1], u1[cb]);
        }
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int s = 0; s < MS; ++s) {
#pragma unroll
          for (int v = 0; v < 4; ++v) Sacc[cb][s][v] += sk[cb][s][v];
          put_s(cb, 16 * (w4 * MS + s) + 4 * g4, Sacc[cb][s]);
        }
    };
    const int full = n / NS * NS;
    for (int base = 0; base < full; base += NS) {
#pragma unroll
      for (int u = 0; u < NS; ++u) iter(base + u, fr[u], fr[(u + NS - 1) % NS]);
    }
#pragma unroll
    for (int u = 0; u < NS - 1; ++u)
      if (full + u < n) iter(full + u, fr[u], fr[(u + NS - 1) % NS]);
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int s = 0; s < MS; ++s) {
        const int r0 = 16 * (w4 * MS + s) + 4 * g4;
#pragma unroll
        for (int v = 0; v < 4; ++v) Sg[(int64_t)(r0 + v) * DV + j0 + 16 * cb + col] = Sacc[cb][s][v];
      }
  } else {
    // output wavefronts: O_c = Q^gamma_c S_c + P_c U_c for chunk rows 16 w4 .. 16 w4 + 15,
    // formed transposed, O^T = S^T Q^gamma^T + U^T P^T, from the same fragments: lane l
    // then holds 4 consecutive columns of row 16 w4 + l % 16 (one 16-byte store)
    OutFrags<DK, POL> fr[NS];
    if (n > 0) {
#pragma unroll
      for (int j = 0; j < NS - 1; ++j) fr[j].load(rec_of(clampc(j)), rl, w4, lane);
    }
    auto iter = [&](int c, const OutFrags<DK, POL>& cur, OutFrags<DK, POL>& ahead) {
      const uint8_t* nrec = rec_of(clampc(c + NS - 1));
      __syncthreads();  // A
      ahead.load_q(nrec, rl, w4, lane);  // the next-but-one chunk's Q^gamma right after A
      __builtin_amdgcn_sched_barrier(0);
      floatx4 ao[CB][2];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        typename F::B bs[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) bs[kb] = get_s(cb, kb);
        floatx4 aq[KB];  // one accumulator per K block, summed in pairs
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) aq[kb] = F::mma_t(z4, bs[kb], cur.q[kb]);
        ao[cb][0] = aq[0];
        ao[cb][1] = aq[1];
        if constexpr (KB == 4) {
          ao[cb][0] = ao[cb][0] + aq[2];
          ao[cb][1] = ao[cb][1] + aq[3];
        }
      }
      __syncthreads();  // B
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const typename F::B u0 = get_u(cb, 0);
        ao[cb][0] = F::mma_t(ao[cb][0], u0, cur.pp[0]);
        if (w4 >= 2) ao[cb][1] = F::mma_t(ao[cb][1], get_u(cb, 1), cur.pp[1]);  // P is lower triangular
      }
      const int64_t start = seq_start + (int64_t)c * L;
      const int len = (int)min((int64_t)L, seq_end - start);
      // stores are unconditional: rows past the sequence go to the sink
      const int rr = 16 * w4 + col;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        float* dst = rr < len ? &p.o[((start + rr) * H + h) * DV + j0 + 16 * cb + 4 * g4] : &p.sink[lane * 4];
        *reinterpret_cast<floatx4*>(dst) = ao[cb][0] + ao[cb][1];
      }
      __builtin_amdgcn_sched_barrier(0);
      ahead.load_p(nrec, rl, w4, lane);
    };
    const int full = n / NS * NS;
    for (int base = 0; base < full; base += NS) {
#pragma unroll
      for (int u = 0; u < NS; ++u) iter(base + u, fr[u], fr[(u + NS - 1) % NS]);
    }
#pragma unroll
    for (int u = 0; u < NS - 1; ++u)
      if (full + u < n) iter(full + u, fr[u], fr[(u + NS - 1) % NS]);
  }
}

// ---------------------------------------------------------------------------
// host launch
// ---------------------------------------------------------------------------
template <int DK, int DV, int POL, typename RawT, bool FUSED>
static hipError_t launch_prefill_t(const PrefillLaunch& Lc, hipStream_t s) {
  PrefillArgs p;
  p.H = Lc.H; p.num_seqs = Lc.num_seqs; p.cu = Lc.cu_seqlens; p.slots = Lc.slots;
  p.q = Lc.q_hat; p.k = Lc.k_hat; p.v = Lc.v; p.g = Lc.g; p.beta = Lc.beta; p.state = Lc.state; p.o = Lc.o;
  p.raw = {Lc.raw_q, Lc.raw_k, Lc.raw_v, Lc.raw_g, Lc.raw_beta, Lc.conv_w, Lc.cs_in, Lc.cs_out,
           Lc.act, Lc.gate_mode, Lc.lb, FUSED ? (int)sizeof(RawT) : 0, Lc.g_per_head};
  p.sink = static_cast<float*>(Lc.workspace);
  p.lookahead = 0;
  if (FUSED) {
    const hipError_t ec = device_cus(&p.lookahead);
    if (ec != hipSuccess) return ec;
  }
  p.recs = static_cast<uint8_t*>(Lc.workspace) + kSinkBytes;
  p.rec_bytes = rec_layout(DK, DV, Frag<POL>::BYTES).bytes;
  // measurement hook: an event just before / after kernel i
  auto mark = [&](int i, int end) -> hipError_t {
    return 2 * i + 1 < Lc.nevents ? hipEventRecord(Lc.events[2 * i + end], s) : hipSuccess;
  };
  hipError_t e = hipSuccess;
  const int64_t mc = max_chunks(Lc.num_seqs, Lc.t_tot);
  constexpr size_t intra_bytes = IntraSmem<DK, DV>::BYTES;
  e = ensure_dynamic_lds(reinterpret_cast<const void*>(&chunk_intra_kernel<DK, DV, POL, RawT, FUSED>), intra_bytes);
  if (e != hipSuccess) return e;
  e = mark(0, 0);
  if (e != hipSuccess) return e;
  if (mc > 0 && Lc.t_tot > 0 && Lc.num_seqs > 0) {
    hipLaunchKernelGGL((chunk_intra_kernel<DK, DV, POL, RawT, FUSED>), dim3((unsigned)(mc * Lc.H)), dim3(kIntraThreads),
                       intra_bytes, s, p);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = mark(0, 1);
  if (e != hipSuccess) return e;
  // (the conv-state carry of a fused call runs inside the scan kernel)
  const int groups = Lc.num_seqs * Lc.H;
  e = mark(1, 0);
  if (e != hipSuccess) return e;
  if (groups > 0) {
    // several column blocks per workgroup where the workgroups would still fill every
    // CU (the scan is then bound by its operand loads), one where they leave CUs idle
    // (it is then bound by the chain's latency); four blocks only with one-part A
    // fragments, whose registers leave room for them
    int cus = 0;
    e = device_cus(&cus);
    if (e != hipSuccess) return e;
    const int padded = (groups + 7) / 8 * 8;
    auto launch_scan = [&](auto blocks) {
      constexpr int CB = decltype(blocks)::value;
      hipLaunchKernelGGL((chunk_scan_kernel<DK, DV, POL, CB>), dim3((unsigned)(padded * (DV / (16 * CB)))),
                         dim3(512), (ScanSmem<DK, POL, CB>::BYTES), s, p, groups);
    };
    constexpr bool kFour = Frag<POL>::BYTES == 16 && DV % 64 == 0;
    const int cb = kFour && 2 * groups >= cus ? 4 : 4 * groups >= cus ? 2 : 1;
    if (cb == 1) launch_scan(std::integral_constant<int, 1>{});
    else if (cb == 2) launch_scan(std::integral_constant<int, 2>{});
    else if constexpr (kFour) launch_scan(std::integral_constant<int, 4>{});
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = mark(1, 1);
  return e;
}

template <int DK, int DV, int POL>
static hipError_t launch_prefill_pol(const PrefillLaunch& L, hipStream_t s) {
  if (!L.fused) return launch_prefill_t<DK, DV, POL, float, false>(L, s);
  if (L.in_dtype == 1) return launch_prefill_t<DK, DV, POL, uint16_t, true>(L, s);
  return launch_prefill_t<DK, DV, POL, float, true>(L, s);
}

hipError_t launch_prefill(const PrefillLaunch& L, hipStream_t s) {
#define KDA_PF_CASE(DK_, DV_)                                                       \
  if (L.dk == DK_ && L.dv == DV_) {                                                 \
    if (L.precision == POL_FP32) return launch_prefill_pol<DK_, DV_, POL_FP32>(L, s); \
    if (L.precision == POL_FP16) return launch_prefill_pol<DK_, DV_, POL_FP16>(L, s); \
    if (L.precision == POL_BF16X2) return launch_prefill_pol<DK_, DV_, POL_BF16X2>(L, s); \
    return launch_prefill_pol<DK_, DV_, POL_BF16X3>(L, s);                          \
  }
  KDA_PF_CASE(64, 64)
  KDA_PF_CASE(64, 128)
  KDA_PF_CASE(128, 64)
  KDA_PF_CASE(128, 128)
#undef KDA_PF_CASE
  return hipErrorInvalidValue;
}

}  // namespace kda
