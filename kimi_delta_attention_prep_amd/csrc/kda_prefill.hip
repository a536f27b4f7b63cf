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
//                   W and U~; writes W, U~, Q^gamma, K_<, P, gamma_L.
//   chunk_scan   -- one workgroup per (sequence, head, 16 state columns), a
//                   sequential pass over the sequence's chunks; the state slice
//                   lives in LDS and all three products run on the matrix cores.
// The pairwise factors e^{G_r - G_i} are formed as e^{G_r - G_p} * e^{G_p - G_i}
// around a pivot row p (the middle row of the 16-row block holding r), so each
// 16x16 block of A and P is a plain matrix product.  Exponents are taken from
// block-local prefix sums, which keeps them accurate to a few ulp of the
// exponent itself; a diagonal block whose half-span of decay exceeds e^80 in
// some key dim is recomputed exactly, pair by pair.
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

enum { POL_FP32 = 0, POL_BF16X3 = 1 };

// ---------------------------------------------------------------------------
// 16x16 matrix-core tile product:  acc (16x16 fp32) += A (16xK) * B (Kx16)
// Fragment map of v_mfma_f32_16x16x4f32 and v_mfma_f32_16x16x32_bf16: lane l
// holds row (l % 16) of A and column (l % 16) of B, with its K slice picked by
// l / 16 (one element for fp32, eight consecutive for bf16); the result lane l
// holds column l % 16, rows 4*(l/16) .. 4*(l/16)+3.  K is a multiple of 32.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void split_bf16(float x, __bf16& hi, __bf16& lo) {
  hi = static_cast<__bf16>(x);
  lo = static_cast<__bf16>(x - static_cast<float>(hi));
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

// e^x: the accurate library exponential for the fp32 policy, the hardware
// exp2 for the split-bf16 policy (whose products carry ~2^-17 error anyway)
template <int POL>
__device__ __forceinline__ float pexp(float x) {
  if constexpr (POL == POL_FP32) return expf(x);
  else return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

// ---------------------------------------------------------------------------
// workspace layout
// ---------------------------------------------------------------------------
struct RecLayout {
  int64_t W, Qg, Kl, Ut, P, gL, floats;  // offsets (floats) inside one (chunk, head) record
};
__host__ __device__ inline RecLayout rec_layout(int dk, int dv) {
  RecLayout r;
  r.W = 0;
  r.Qg = r.W + 64 * dk;
  r.Kl = r.Qg + 64 * dk;
  r.Ut = r.Kl + 64 * dk;
  r.P = r.Ut + 64 * dv;
  r.gL = r.P + 64 * 64;
  r.floats = (r.gL + dk + 63) / 64 * 64;  // 256-byte aligned records
  return r;
}
static inline int64_t max_chunks(int num_seqs, int64_t t_tot) { return t_tot / kChunk + num_seqs; }
static inline size_t table_bytes(int num_seqs) { return ((size_t)(num_seqs + 1) * 4 + 255) / 256 * 256; }

size_t prefill_workspace_bytes(int H, int dk, int dv, int num_seqs, int64_t t_tot) {
  const RecLayout rl = rec_layout(dk, dv);
  return table_bytes(num_seqs) + (size_t)max_chunks(num_seqs, t_tot) * H * rl.floats * sizeof(float);
}

struct PrefillArgs {
  int H, num_seqs;
  const int32_t *cu, *slots;
  const float *q, *k, *v, *g, *beta;
  float *state, *o;
  int32_t* chunk_off;  // [num_seqs + 1]
  float* recs;         // [max_chunks][H][rec floats]
  int64_t rec_floats;
};

// ---------------------------------------------------------------------------
// chunk table: chunk_off[n] = sum_{m<n} ceil(len_m / 64)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void chunk_table_kernel(const int32_t* cu, int num_seqs, int32_t* chunk_off) {
  __shared__ int32_t s[256];
  __shared__ int32_t carry;
  if (threadIdx.x == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < num_seqs; base += 256) {
    const int n = base + threadIdx.x;
    const int32_t c = (n < num_seqs) ? (cu[n + 1] - cu[n] + kChunk - 1) / kChunk : 0;
    s[threadIdx.x] = c;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {  // inclusive Hillis-Steele scan
      const int32_t x = threadIdx.x >= off ? s[threadIdx.x - off] : 0;
      __syncthreads();
      s[threadIdx.x] += x;
      __syncthreads();
    }
    if (n < num_seqs) chunk_off[n] = carry + s[threadIdx.x] - c;
    __syncthreads();
    if (threadIdx.x == 255) carry += s[255];
    __syncthreads();
  }
  if (threadIdx.x == 0) chunk_off[num_seqs] = carry;
}

__device__ __forceinline__ int chunk_seq(const int32_t* chunk_off, int num_seqs, int c) {
  int lo = 0, hi = num_seqs;  // largest n with chunk_off[n] <= c
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (chunk_off[mid] <= c) lo = mid; else hi = mid;
  }
  return lo;
}

// ---------------------------------------------------------------------------
// intra-chunk kernel
//
// Pivots.  Inside diagonal block R (rows 16R..16R+15) the pivot is its middle
// row m_R = 16R+8 and gloc_r = G_r - G_{m_R} (a block-local prefix difference):
//   A/P block (R,R): left k_r e^{gloc_r} (or q_r e^{gloc_r}), right k_i e^{-gloc_i}.
// For an off-diagonal block (R,I), I < R, the pivot is the first row 16R of R:
//   left  = k_r e^{gloc_r} * e^{-gloc_{16R}}            = k_r e^{G_r - G_{16R}}  <= |k_r|
//   right = k_i e^{-gloc_i} * e^{G_{16R} - G_{m_I}}      = k_i e^{G_{16R} - G_i}  <= |k_i|
// While every |gloc| <= 40 no factor overflows and a factor that underflows
// can only drop terms below e^-47, so the products are as exact as fp32
// allows.  A chunk with a wider half-block decay span (a key dim decaying by
// more than e^40 over 8 rows) is recomputed exactly from its raw rows.
// ---------------------------------------------------------------------------
constexpr float kSpanGuard = 40.0f;

template <int DK, int DV>
struct IntraSmem {
  static constexpr int L = 64;
  static constexpr int DM = DK > DV ? DK : DV;
  static constexpr int PK = DM + 4;  // row stride of the 64 x d tiles
  static constexpr int PL = L + 4;   // row stride of the 64 x 64 tiles
  static constexpr int T0 = 0;                 // k e^{gloc}; later b e^{G} k        [L][PK]
  static constexpr int T1 = T0 + L * PK;       // q e^{gloc}; later b v              [L][PK]
  static constexpr int T2 = T1 + L * PK;       // block prefix of g; then k e^{-gloc} [L][PK]
  static constexpr int TA = T2 + L * PK;       // A                                  [L][PL]
  static constexpr int TP = TA + L * PL;       // P, then X                          [L][PL]
  static constexpr int TB = TP + L * PL;       // beta                               [L]
  static constexpr int TPV = TB + L;           // block prefix at the pivot row      [4][DK]
  static constexpr int TEG = TPV + 4 * DK;     // e^{G_{m_R}}                        [4][DK]
  static constexpr int TEL = TEG + 4 * DK;     // e^{G_last - G_{m_R}}               [4][DK]
  static constexpr int TEF = TEL + 4 * DK;     // e^{-gloc_{16R}}                    [4][DK]
  static constexpr int TEE = TEF + 4 * DK;     // e^{G_{16R} - G_{m_I}}, I < R       [6][DK]
  static constexpr int TY = TEE + 6 * DK;      // 16x16 scratch of the solve         [16][17]
  static constexpr int TFLAG = TY + 16 * 17;   // 1 int: chunk takes the exact path
  static constexpr int FLOATS = TFLAG + 4;
  static constexpr size_t BYTES = FLOATS * sizeof(float);
};

__device__ __forceinline__ int pair_index(int R, int I) { return R * (R - 1) / 2 + I; }  // I < R

template <int DK, int DV, int POL>
__global__ __launch_bounds__(256) void chunk_intra_kernel(PrefillArgs p) {
  using SM = IntraSmem<DK, DV>;
  constexpr int L = SM::L, PK = SM::PK, PL = SM::PL;
  extern __shared__ __align__(16) float smem[];
  float* sKl = smem + SM::T0;
  float* sQl = smem + SM::T1;
  float* sKr = smem + SM::T2;
  float* sA = smem + SM::TA;
  float* sP = smem + SM::TP;
  float* sBeta = smem + SM::TB;
  float* sPv = smem + SM::TPV;
  float* sEG = smem + SM::TEG;
  float* sEL = smem + SM::TEL;
  float* sEF = smem + SM::TEF;
  float* sEE = smem + SM::TEE;
  float* sY = smem + SM::TY;
  int* sFlag = reinterpret_cast<int*>(smem + SM::TFLAG);

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int c = blockIdx.x, h = blockIdx.y, H = p.H;
  const int total = p.chunk_off[p.num_seqs];
  if (c >= total) return;
  const int n = chunk_seq(p.chunk_off, p.num_seqs, c);
  const int64_t start = (int64_t)p.cu[n] + (int64_t)(c - p.chunk_off[n]) * L;
  const int len = (int)min((int64_t)L, (int64_t)p.cu[n + 1] - start);
  float* rec = p.recs + ((int64_t)c * H + h) * p.rec_floats;
  const RecLayout rl = rec_layout(DK, DV);
  auto row_off = [&](int r, int d) -> int64_t { return ((start + r) * H + h) * DK + d; };

  // 1. rows of k, q, g (zero beyond the chunk's last row) and beta
  for (int idx = t; idx < L * (DK / 4); idx += 256) {
    const int r = idx / (DK / 4), c4 = 4 * (idx % (DK / 4));
    float4 kk = {0.f, 0.f, 0.f, 0.f}, qq = kk, gg = kk;
    if (r < len) {
      kk = *reinterpret_cast<const float4*>(p.k + row_off(r, c4));
      qq = *reinterpret_cast<const float4*>(p.q + row_off(r, c4));
      gg = *reinterpret_cast<const float4*>(p.g + row_off(r, c4));
    }
    *reinterpret_cast<float4*>(&sKl[r * PK + c4]) = kk;
    *reinterpret_cast<float4*>(&sQl[r * PK + c4]) = qq;
    *reinterpret_cast<float4*>(&sKr[r * PK + c4]) = gg;
  }
  if (t < L) sBeta[t] = t < len ? p.beta[(start + t) * H + h] : 0.f;
  if (t == 0) sFlag[0] = 0;
  __syncthreads();

  // 2. block-local inclusive prefix sums of g over each 16-row block (in place)
  for (int item = t; item < 4 * DK; item += 256) {
    const int R = item / DK, d = item % DK;
    float run = 0.f;
    for (int r = 16 * R; r < 16 * R + 16; ++r) {
      run += sKr[r * PK + d];
      sKr[r * PK + d] = run;
    }
  }
  __syncthreads();

  // 3. per key dim, from block prefixes only (no differences of large sums):
  //    pv[R] = prefix at m_R, tot[R] = block total, G at pivots and the last row
  if (t < DK) {
    const int d = t;
    float pv[4], tot[4], first[4];
#pragma unroll
    for (int R = 0; R < 4; ++R) {
      pv[R] = sKr[(16 * R + 8) * PK + d];
      tot[R] = sKr[(16 * R + 15) * PK + d];
      first[R] = sKr[(16 * R) * PK + d];
    }
    const int Rl = (len - 1) / 16;
    const float pl = sKr[(len - 1) * PK + d];
    float off = 0.f;  // G at the row before block R
    float gl = 0.f;   // G at the last row
#pragma unroll
    for (int R = 0; R < 4; ++R) {
      if (R == Rl) gl = off + pl;
      sPv[R * DK + d] = pv[R];
      sEG[R * DK + d] = pexp<POL>(off + pv[R]);
      // G_last - G_{m_R}: rows m_R+1 .. len-1 (zero when the pivot lies past the last row)
      float gLp = 0.f;
      if (R < Rl) {
        gLp = tot[R] - pv[R];
        for (int Rm = R + 1; Rm < Rl; ++Rm) gLp += tot[Rm];
        gLp += pl;
      } else if (R == Rl && 16 * R + 8 < len) {
        gLp = pl - pv[R];
      }
      sEL[R * DK + d] = pexp<POL>(gLp);
      sEF[R * DK + d] = pexp<POL>(-(first[R] - pv[R]));
      // G_{16R} - G_{m_I} for I < R: rows m_I+1 .. 16R
      for (int I = 0; I < R; ++I) {
        float e = tot[I] - pv[I];
        for (int Rm = I + 1; Rm < R; ++Rm) e += tot[Rm];
        e += first[R];
        sEE[pair_index(R, I) * DK + d] = pexp<POL>(e);
      }
      // the exponents inside block R span [gloc(last row), gloc(first row)]
      if (fmaxf(first[R] - pv[R], pv[R] - tot[R]) > kSpanGuard) atomicOr(sFlag, 1);
      off += tot[R];
    }
    rec[rl.gL + d] = pexp<POL>(gl);
  }
  __syncthreads();
  const bool exact = sFlag[0] != 0;

  // 4. elementwise: pivot operands, Q^gamma = e^{G_r} q_r and K_< = e^{G_last - G_r} k_r
  for (int idx = t; idx < L * DK; idx += 256) {
    const int r = idx / DK, d = idx % DK, R = r / 16;
    const float gloc = fminf(fmaxf(sKr[r * PK + d] - sPv[R * DK + d], -kSpanGuard), kSpanGuard);
    const float ep = pexp<POL>(gloc), em = pexp<POL>(-gloc);
    const float kk = sKl[r * PK + d], qq = sQl[r * PK + d];
    const float kl = kk * ep, ql = qq * ep, kr = kk * em;
    sKl[r * PK + d] = kl;
    sQl[r * PK + d] = ql;
    sKr[r * PK + d] = kr;
    rec[rl.Qg + r * DK + d] = sEG[R * DK + d] * ql;
    rec[rl.Kl + r * DK + d] = sEL[R * DK + d] * kr;
  }
  __syncthreads();

  if (!exact) {
    // 5. A and P, one 16x16 block pair (R >= I) at a time on the matrix cores
    for (int blk = wave; blk < 10; blk += 4) {
      int R = 0, I = blk;  // blocks in order (0,0) (1,0) (1,1) (2,0) (2,1) (2,2) (3,0) ...
      while (I > R) { I -= R + 1; ++R; }
      floatx4 accA = {0.f, 0.f, 0.f, 0.f}, accP = accA;
      if (I == R) {
        auto fr = [&](int kk, int j) { return sKr[(16 * I + j) * PK + kk]; };
        mma16<POL>(accA, DK, [&](int i, int kk) { return sKl[(16 * R + i) * PK + kk]; }, fr);
        mma16<POL>(accP, DK, [&](int i, int kk) { return sQl[(16 * R + i) * PK + kk]; }, fr);
      } else {
        const float* ee = &sEE[pair_index(R, I) * DK];
        const float* ef = &sEF[R * DK];
        auto fr = [&](int kk, int j) { return sKr[(16 * I + j) * PK + kk] * ee[kk]; };
        mma16<POL>(accA, DK, [&](int i, int kk) { return sKl[(16 * R + i) * PK + kk] * ef[kk]; }, fr);
        mma16<POL>(accP, DK, [&](int i, int kk) { return sQl[(16 * R + i) * PK + kk] * ef[kk]; }, fr);
      }
      const int col = lane & 15, g4 = lane >> 4;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int rr = 16 * R + 4 * g4 + v, ii = 16 * I + col;
        sA[rr * PL + ii] = (ii < rr) ? sBeta[rr] * accA[v] : 0.f;
        sP[rr * PL + ii] = (ii <= rr) ? accP[v] : 0.f;
      }
    }
    for (int idx = t; idx < L * L; idx += 256) {  // strictly-upper blocks are zero
      const int rr = idx / L, ii = idx % L;
      if ((ii >> 4) > (rr >> 4)) { sA[rr * PL + ii] = 0.f; sP[rr * PL + ii] = 0.f; }
    }
  } else {
    // 5'. exact path: G as a full-chunk prefix, every factor as one exponential
    float* sG = sKl;   // G_r            [L][PK]
    float* sK0 = sQl;  // k rows         [L][PK]
    float* sQ0 = sKr;  // q rows         [L][PK]
    for (int idx = t; idx < L * DK; idx += 256) {
      const int r = idx / DK, d = idx % DK;
      sK0[r * PK + d] = r < len ? p.k[row_off(r, d)] : 0.f;
      sQ0[r * PK + d] = r < len ? p.q[row_off(r, d)] : 0.f;
    }
    if (t < DK) {
      float run = 0.f;
      for (int r = 0; r < L; ++r) {
        run += r < len ? p.g[row_off(r, t)] : 0.f;
        sG[r * PK + t] = run;
      }
    }
    __syncthreads();
    for (int pr = t; pr < L * L; pr += 256) {
      const int r = pr / L, i = pr % L;
      float sa = 0.f, sp = 0.f;
      if (i <= r) {
        for (int d = 0; d < DK; ++d) {
          const float e = expf(sG[r * PK + d] - sG[i * PK + d]);
          sa = fmaf(sK0[r * PK + d] * sK0[i * PK + d], e, sa);
          sp = fmaf(sQ0[r * PK + d] * sK0[i * PK + d], e, sp);
        }
      }
      sA[r * PL + i] = (i < r) ? sBeta[r] * sa : 0.f;
      sP[r * PL + i] = (i <= r) ? sp : 0.f;
    }
    for (int idx = t; idx < L * DK; idx += 256) {
      const int r = idx / DK, d = idx % DK;
      const float G = sG[r * PK + d], GL = sG[(len - 1) * PK + d];
      rec[rl.Qg + r * DK + d] = expf(G) * sQ0[r * PK + d];
      rec[rl.Kl + r * DK + d] = expf(GL - G) * sK0[r * PK + d];
    }
  }
  __syncthreads();

  // 6. P to the record; then X = (I + A)^{-1} into the P tile
  for (int idx = t; idx < L * L; idx += 256) {
    const int rr = idx / L, ii = idx % L;
    rec[rl.P + rr * L + ii] = sP[rr * PL + ii];
  }
  __syncthreads();
  float* sX = sP;
  for (int idx = t; idx < L * L; idx += 256) sX[(idx / L) * PL + idx % L] = 0.f;
  __syncthreads();
  if (t < L) {  // diagonal blocks by forward substitution, one column per thread
    const int R = t / 16, cc = t % 16, b0 = 16 * R;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float s = (r == cc) ? 1.f : 0.f;
#pragma unroll
      for (int i = 0; i < r; ++i) s = fmaf(-sA[(b0 + r) * PL + b0 + i], x[i], s);
      x[r] = (r >= cc) ? s : 0.f;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) sX[(b0 + r) * PL + b0 + cc] = x[r];
  }
  __syncthreads();
  // off-diagonal blocks, nearest diagonals first: X_RI = -X_RR sum_{J=I}^{R-1} A_RJ X_JI
  for (int dist = 1; dist < 4; ++dist) {
    for (int I = 0; I + dist < 4; ++I) {
      const int R = I + dist;
      const int r = t / 16, cc = t % 16;
      float y = 0.f;
      for (int J = I; J < R; ++J)
        for (int kk = 0; kk < 16; ++kk)
          y = fmaf(sA[(16 * R + r) * PL + 16 * J + kk], sX[(16 * J + kk) * PL + 16 * I + cc], y);
      sY[r * 17 + cc] = y;
      __syncthreads();
      float x = 0.f;
      for (int kk = 0; kk <= r; ++kk) x = fmaf(sX[(16 * R + r) * PL + 16 * R + kk], sY[kk * 17 + cc], x);
      sX[(16 * R + r) * PL + 16 * I + cc] = -x;
      __syncthreads();
    }
  }

  // 7. right-hand sides: b_r e^{G_r} k_r into T0, b_r v_r into T1
  for (int idx = t; idx < L * DK; idx += 256) {
    const int r = idx / DK, d = idx % DK;
    const float kg = exact ? expf(sKl[r * PK + d]) * sQl[r * PK + d]   // exact path: T0 = G, T1 = k
                           : sEG[(r / 16) * DK + d] * sKl[r * PK + d];
    sKl[r * PK + d] = sBeta[r] * kg;
  }
  __syncthreads();
  for (int idx = t; idx < L * (DV / 4); idx += 256) {
    const int r = idx / (DV / 4), c4 = 4 * (idx % (DV / 4));
    float4 vv = {0.f, 0.f, 0.f, 0.f};
    if (r < len) vv = *reinterpret_cast<const float4*>(p.v + ((start + r) * H + h) * DV + c4);
    const float b = sBeta[r];
    vv.x *= b; vv.y *= b; vv.z *= b; vv.w *= b;
    *reinterpret_cast<float4*>(&sQl[r * PK + c4]) = vv;
  }
  __syncthreads();

  // 8. W = X (b K^gamma), U~ = X (b V); X is lower triangular, so row block R needs K = 16(R+1)
  constexpr int NTW = 4 * (DK / 16), NTU = 4 * (DV / 16);
  for (int tile = wave; tile < NTW + NTU; tile += 4) {
    const bool isW = tile < NTW;
    const int tt = isW ? tile : tile - NTW;
    const int R = tt % 4, cb = tt / 4;
    const int K = (16 * (R + 1) + 31) / 32 * 32;
    const float* B = isW ? sKl : sQl;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    mma16<POL>(acc, K, [&](int i, int kk) { return sX[(16 * R + i) * PL + kk]; },
               [&](int kk, int j) { return B[kk * PK + 16 * cb + j]; });
    const int col = lane & 15, g4 = lane >> 4;
    float* dst = rec + (isW ? rl.W : rl.Ut);
    const int ld = isW ? DK : DV;
#pragma unroll
    for (int v = 0; v < 4; ++v) dst[(16 * R + 4 * g4 + v) * ld + 16 * cb + col] = acc[v];
  }
}

// ---------------------------------------------------------------------------
// inter-chunk scan
// ---------------------------------------------------------------------------
template <int DK, int DV>
struct ScanSmem {
  static constexpr int L = 64;
  static constexpr int PK = DK + 4, PL = L + 4, PS = 16 + 4;
  static constexpr int TW = 0;               // W        [L][PK]
  static constexpr int TQ = TW + L * PK;     // Q^gamma  [L][PK]
  static constexpr int TK = TQ + L * PK;     // K_<      [L][PK]
  static constexpr int TP = TK + L * PK;     // P        [L][PL]
  static constexpr int TS = TP + L * PL;     // state slice [DK][PS]
  static constexpr int TU = TS + DK * PS;    // U slice  [L][PS]
  static constexpr int TUT = TU + L * PS;    // U~ slice [L][PS]
  static constexpr int TG = TUT + L * PS;    // gamma_L  [DK]
  static constexpr int FLOATS = TG + DK;
  static constexpr size_t BYTES = FLOATS * sizeof(float);
};

template <int DK, int DV, int POL>
__global__ __launch_bounds__(256) void chunk_scan_kernel(PrefillArgs p, int groups) {
  using SM = ScanSmem<DK, DV>;
  constexpr int L = SM::L, PK = SM::PK, PL = SM::PL, PS = SM::PS;
  constexpr int NSPLIT = DV / 16;
  extern __shared__ __align__(16) float smem[];
  float* sW = smem + SM::TW;
  float* sQ = smem + SM::TQ;
  float* sK = smem + SM::TK;
  float* sP = smem + SM::TP;
  float* sS = smem + SM::TS;
  float* sU = smem + SM::TU;
  float* sUt = smem + SM::TUT;
  float* sG = smem + SM::TG;

  // workgroups of one (sequence, head) share its chunk records: keep them on one XCD
  // (workgroups are dealt round-robin over the 8 XCDs by linear id)
  const int id = blockIdx.x, xcd = id % 8, k = id / 8;
  const int grp = (k / NSPLIT) * 8 + xcd, split = k % NSPLIT;
  if (grp >= groups) return;
  const int H = p.H, n = grp / H, h = grp % H;
  const int slot = p.slots ? p.slots[n] : n;
  if (slot < 0) return;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int col = lane & 15, g4 = lane >> 4;
  const int j0 = 16 * split;
  const RecLayout rl = rec_layout(DK, DV);
  float* Sg = p.state + ((int64_t)slot * H + h) * DK * DV;

  for (int idx = t; idx < DK * 4; idx += 256) {
    const int r = idx / 4, c4 = 4 * (idx % 4);
    *reinterpret_cast<float4*>(&sS[r * PS + c4]) = *reinterpret_cast<const float4*>(Sg + (int64_t)r * DV + j0 + c4);
  }
  const int c_begin = p.chunk_off[n], c_end = p.chunk_off[n + 1];
  for (int c = c_begin; c < c_end; ++c) {
    const float* rec = p.recs + ((int64_t)c * H + h) * p.rec_floats;
    const int64_t start = (int64_t)p.cu[n] + (int64_t)(c - c_begin) * L;
    const int len = (int)min((int64_t)L, (int64_t)p.cu[n + 1] - start);
    __syncthreads();  // previous chunk done with the tiles
    for (int idx = t; idx < L * (DK / 4); idx += 256) {
      const int r = idx / (DK / 4), c4 = 4 * (idx % (DK / 4));
      *reinterpret_cast<float4*>(&sW[r * PK + c4]) = *reinterpret_cast<const float4*>(rec + rl.W + r * DK + c4);
      *reinterpret_cast<float4*>(&sQ[r * PK + c4]) = *reinterpret_cast<const float4*>(rec + rl.Qg + r * DK + c4);
      *reinterpret_cast<float4*>(&sK[r * PK + c4]) = *reinterpret_cast<const float4*>(rec + rl.Kl + r * DK + c4);
    }
    for (int idx = t; idx < L * (L / 4); idx += 256) {
      const int r = idx / (L / 4), c4 = 4 * (idx % (L / 4));
      *reinterpret_cast<float4*>(&sP[r * PL + c4]) = *reinterpret_cast<const float4*>(rec + rl.P + r * L + c4);
    }
    {
      const int r = t / 4, c4 = 4 * (t % 4);  // 64 rows x 16 columns of U~
      *reinterpret_cast<float4*>(&sUt[r * PS + c4]) = *reinterpret_cast<const float4*>(rec + rl.Ut + r * DV + j0 + c4);
    }
    for (int d = t; d < DK; d += 256) sG[d] = rec[rl.gL + d];
    __syncthreads();

    // U = U~ - W S  (wave w: rows 16w .. 16w+15)
    {
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
      mma16<POL>(acc, DK, [&](int i, int kk) { return sW[(16 * wave + i) * PK + kk]; },
                 [&](int kk, int j) { return sS[kk * PS + j]; });
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int rr = 16 * wave + 4 * g4 + v;
        sU[rr * PS + col] = sUt[rr * PS + col] - acc[v];
      }
    }
    __syncthreads();
    // O = Q^gamma S + P U  (P is lower triangular: row block w needs K = 16(w+1))
    {
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
      mma16<POL>(acc, DK, [&](int i, int kk) { return sQ[(16 * wave + i) * PK + kk]; },
                 [&](int kk, int j) { return sS[kk * PS + j]; });
      mma16<POL>(acc, (16 * (wave + 1) + 31) / 32 * 32, [&](int i, int kk) { return sP[(16 * wave + i) * PL + kk]; },
                 [&](int kk, int j) { return sU[kk * PS + j]; });
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int rr = 16 * wave + 4 * g4 + v;
        if (rr < len) p.o[((start + rr) * H + h) * DV + j0 + col] = acc[v];
      }
    }
    // S_L = Diag(gamma_L) S + K_<^T U  (wave w: state rows 16*(2w+s) .. +15)
    floatx4 accS[DK / 64];
#pragma unroll
    for (int s = 0; s < DK / 64; ++s) {
      const int rb = 16 * (wave * (DK / 64) + s);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int rr = rb + 4 * g4 + v;
        accS[s][v] = sG[rr] * sS[rr * PS + col];
      }
      mma16<POL>(accS[s], L, [&](int i, int kk) { return sK[kk * PK + rb + i]; },
                 [&](int kk, int j) { return sU[kk * PS + j]; });
    }
    __syncthreads();  // every read of the old state is done
#pragma unroll
    for (int s = 0; s < DK / 64; ++s) {
      const int rb = 16 * (wave * (DK / 64) + s);
#pragma unroll
      for (int v = 0; v < 4; ++v) sS[(rb + 4 * g4 + v) * PS + col] = accS[s][v];
    }
  }
  __syncthreads();
  for (int idx = t; idx < DK * 4; idx += 256) {
    const int r = idx / 4, c4 = 4 * (idx % 4);
    *reinterpret_cast<float4*>(Sg + (int64_t)r * DV + j0 + c4) = *reinterpret_cast<const float4*>(&sS[r * PS + c4]);
  }
}

// ---------------------------------------------------------------------------
// host launch
// ---------------------------------------------------------------------------
template <int DK, int DV, int POL>
static hipError_t launch_prefill_t(const PrefillLaunch& Lc, hipStream_t s) {
  PrefillArgs p;
  p.H = Lc.H; p.num_seqs = Lc.num_seqs; p.cu = Lc.cu_seqlens; p.slots = Lc.slots;
  p.q = Lc.q_hat; p.k = Lc.k_hat; p.v = Lc.v; p.g = Lc.g; p.beta = Lc.beta; p.state = Lc.state; p.o = Lc.o;
  p.chunk_off = static_cast<int32_t*>(Lc.workspace);
  p.recs = reinterpret_cast<float*>(static_cast<char*>(Lc.workspace) + table_bytes(Lc.num_seqs));
  p.rec_floats = rec_layout(DK, DV).floats;
  hipLaunchKernelGGL(chunk_table_kernel, dim3(1), dim3(256), 0, s, Lc.cu_seqlens, Lc.num_seqs, p.chunk_off);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t mc = max_chunks(Lc.num_seqs, Lc.t_tot);
  if (mc > 0 && Lc.t_tot > 0) {
    constexpr size_t intra_bytes = IntraSmem<DK, DV>::BYTES;
    static bool attr_set = false;
    if (!attr_set) {
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(&chunk_intra_kernel<DK, DV, POL>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)intra_bytes);
      if (e != hipSuccess) return e;
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(&chunk_scan_kernel<DK, DV, POL>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)ScanSmem<DK, DV>::BYTES);
      if (e != hipSuccess) return e;
      attr_set = true;
    }
    hipLaunchKernelGGL((chunk_intra_kernel<DK, DV, POL>), dim3((unsigned)mc, (unsigned)Lc.H), dim3(256), intra_bytes,
                       s, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int groups = Lc.num_seqs * Lc.H;
  if (groups > 0) {
    const int nsplit = DV / 16;
    const int wgs = (groups + 7) / 8 * 8 * nsplit;
    constexpr size_t scan_bytes = ScanSmem<DK, DV>::BYTES;
    hipLaunchKernelGGL((chunk_scan_kernel<DK, DV, POL>), dim3((unsigned)wgs), dim3(256), scan_bytes, s, p, groups);
  }
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillLaunch& L, hipStream_t s) {
#define KDA_PF_CASE(DK_, DV_)                                                                        \
  if (L.dk == DK_ && L.dv == DV_)                                                                    \
    return L.precision == POL_FP32 ? launch_prefill_t<DK_, DV_, POL_FP32>(L, s)                      \
                                   : launch_prefill_t<DK_, DV_, POL_BF16X3>(L, s);
  KDA_PF_CASE(64, 64)
  KDA_PF_CASE(64, 128)
  KDA_PF_CASE(128, 64)
  KDA_PF_CASE(128, 128)
#undef KDA_PF_CASE
  return hipErrorInvalidValue;
}

}  // namespace kda
