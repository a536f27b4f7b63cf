// kda_rows.hip -- decode rows and speculative verify windows (gfx950).
//
// One workgroup per (sequence, head) streams that head's fp32 d_k x d_v state
// from HBM into registers with 128-bit loads, runs the fused row step
//   conv step on the carried conv state -> SiLU -> q/k L2 norm -> gates, beta
//   S' = Diag(a) S;  u = beta (v - S'^T k);  S = S' + k u^T;  o = S^T q
// (the gated delta rule with per-key-dim decay; TensorFold issue #850: "decode
// rows and verify windows", the shared KDA module) and streams the state back.
// The readout uses o = S'^T q + (q.k) u, so one pass over S' gives both
// reductions S'^T k and S'^T q.
//
// A verify window (same issue: a window logs each row's decay, normalised key
// and update; the next call replays the kept rows from that log) first commits
// n_commit rows of the previous window's log into the state and conv state,
// then runs its own rows through the very same row step on a register copy of
// the committed state, writing outputs and the log but not the state.  Decode
// and verify share the row step, the thread-to-element map and the reduction
// tree, and the replay applies the identical decay-then-fma update, so a
// committed window leaves the same bits as rows decoded one at a time.
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

template <int DK, int DV>
struct RowsShape {
  static constexpr int NT = 256;          // threads per workgroup (4 wavefronts)
  static constexpr int NW = NT / 64;      // wavefronts
  static constexpr int CG = DV / 4;       // threads across the d_v columns, 4 columns (16 B) each
  static constexpr int RG = NT / CG;      // row groups
  static constexpr int RPT = DK / RG;     // state rows held per thread
  static constexpr int GPW = 64 / CG;     // row groups inside one wavefront
  static_assert(DK + DV <= NT, "one preamble channel pair per thread");
  static_assert(RPT * RG == DK && CG * 4 == DV, "tile");
};

template <typename RawT>
struct RowsArgs {
  int H, gate_mode, act, batch, window;
  int g_per_head;  // raw g rows [B, (window,) H]: one decay per head and row, broadcast over d_k
  float lb;
  const int32_t* slots;
  float* state;
  RawT* conv_state;
  const float* conv_w;
  const RawT *q, *k, *v, *g, *beta;  // rows [B, window, H, d] (decode: window = 1)
  float* o;                          // [B, window, H, d_v]
  // verify only
  const int32_t* n_commit;
  const int32_t* wlen;  // rows of the window per sequence, or NULL (all `window`)
  const float *in_a, *in_k, *in_u;
  const RawT* in_rows;
  int in_window;
  float *out_a, *out_k, *out_u;
  RawT* out_rows;
};

// Conv history of the channels one thread owns: for t < DK the q and k channel
// t of this head, for DK <= t < DK+DV the v channel t-DK.  h[0] is the oldest.
template <typename RawT>
struct ChanHist {
  RawT hq[3], hk[3];  // q/k channel (or v channel in hq for v threads)
  float wq[4], wk[4];
};

template <int DK, int DV, typename RawT>
struct RowStep {
  using SH = RowsShape<DK, DV>;
  float* s_q;  // [DK] normalised q
  float* s_k;  // [DK] normalised k
  float* s_v;  // [DV] conv output of v
  float* s_a;  // [DK] decay
  float* s_red;  // [NW][8] wave partials of scalar reductions
  float* s_pk;   // [NW][DV]
  float* s_pq;   // [NW][DV]
  float* s_scal; // [4]: beta

  // The raw inputs of one row that this thread uses: q, k, g of channel t (t < DK),
  // v of channel t - DK (DK <= t < DK + DV), beta (t = 0).  Every thread loads all
  // five, from clamped indices, so that no load sits in a branch (a load inside a
  // branch is waited for where the branches join) and a row's inputs can be
  // loaded while the previous row computes.
  struct RowIn {
    RawT q, k, g, v, beta;
  };
  __device__ RowIn load_in(const RowsArgs<RawT>& p, int64_t row_hd_k, int64_t row_hd_v, int64_t row_h) {
    const int t = threadIdx.x;
    const int tk = t < DK ? t : 0, tv = (t >= DK && t < DK + DV) ? t - DK : 0;
    RowIn in;
    in.q = p.q[row_hd_k + tk];
    in.k = p.k[row_hd_k + tk];
    in.g = p.g[p.g_per_head ? row_h : row_hd_k + tk];
    in.v = p.v[row_hd_v + tv];
    in.beta = p.beta[row_h];
    return in;
  }

  // Preamble of one row: conv step (history shifts by the new raw row), gates,
  // norms.  Leaves normalised q, k, conv v, decay a and beta in LDS and returns q.k.
  __device__ float preamble(const RowsArgs<RawT>& p, ChanHist<RawT>& ch, const RowIn& in, RawT& raw_q,
                            RawT& raw_k) {
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    float cq = 0.f, ck = 0.f;
    if (t < DK) {
      raw_q = in.q;
      raw_k = in.k;
      cq = conv4_act(ch.wq[0], ch.wq[1], ch.wq[2], ch.wq[3], to_f32(ch.hq[0]), to_f32(ch.hq[1]),
                     to_f32(ch.hq[2]), to_f32(raw_q), p.act);
      ck = conv4_act(ch.wk[0], ch.wk[1], ch.wk[2], ch.wk[3], to_f32(ch.hk[0]), to_f32(ch.hk[1]),
                     to_f32(ch.hk[2]), to_f32(raw_k), p.act);
      ch.hq[0] = ch.hq[1]; ch.hq[1] = ch.hq[2]; ch.hq[2] = raw_q;
      ch.hk[0] = ch.hk[1]; ch.hk[1] = ch.hk[2]; ch.hk[2] = raw_k;
      s_a[t] = expf(log_decay(to_f32(in.g), p.gate_mode, p.lb));
    } else if (t < DK + DV) {
      const int j = t - DK;
      raw_q = in.v;
      const float cv = conv4_act(ch.wq[0], ch.wq[1], ch.wq[2], ch.wq[3], to_f32(ch.hq[0]), to_f32(ch.hq[1]),
                                 to_f32(ch.hq[2]), to_f32(raw_q), p.act);
      ch.hq[0] = ch.hq[1]; ch.hq[1] = ch.hq[2]; ch.hq[2] = raw_q;
      s_v[j] = cv;
    }
    if (t == 0) s_scal[0] = sigmoid(to_f32(in.beta));
    // L2 norms over d_k (only the DK/64 wavefronts holding q/k channels contribute)
    const float sq = wave_sum(cq * cq), sk = wave_sum(ck * ck);
    if (lane == 0) { s_red[wave * 8 + 0] = sq; s_red[wave * 8 + 1] = sk; }
    __syncthreads();
    float tq = 0.f, tk = 0.f;
#pragma unroll
    for (int w = 0; w < DK / 64; ++w) { tq += s_red[w * 8 + 0]; tk += s_red[w * 8 + 1]; }
    const float rq = 1.0f / sqrtf(tq + kL2Eps), rk = 1.0f / sqrtf(tk + kL2Eps);
    float qk = 0.f;
    if (t < DK) {
      const float qh = cq * rq, kh = ck * rk;
      s_q[t] = qh;
      s_k[t] = kh;
      qk = qh * kh;
    }
    qk = wave_sum(qk);
    if (lane == 0) s_red[wave * 8 + 2] = qk;
    __syncthreads();
    float dot = 0.f;
#pragma unroll
    for (int w = 0; w < DK / 64; ++w) dot += s_red[w * 8 + 2];
    return dot;
  }

  // State step on the register tile S (rows rg + RG*m, columns 4cg..4cg+3).
  // Returns u and o for this thread's 4 columns (valid in every row group).
  __device__ void step(float4 (&S)[SH::RPT], float qk, float4& u_out, float4& o_out) {
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int cg = t % SH::CG, rg = t / SH::CG;
    float4 pk = {0.f, 0.f, 0.f, 0.f}, pq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < SH::RPT; ++m) {
      const int i = rg + SH::RG * m;
      const float a = s_a[i], ki = s_k[i], qi = s_q[i];
      float4 s = S[m];
      s.x = decay(s.x, a); s.y = decay(s.y, a); s.z = decay(s.z, a); s.w = decay(s.w, a);
      S[m] = s;
      pk.x = fmaf(ki, s.x, pk.x); pk.y = fmaf(ki, s.y, pk.y); pk.z = fmaf(ki, s.z, pk.z); pk.w = fmaf(ki, s.w, pk.w);
      pq.x = fmaf(qi, s.x, pq.x); pq.y = fmaf(qi, s.y, pq.y); pq.z = fmaf(qi, s.z, pq.z); pq.w = fmaf(qi, s.w, pq.w);
    }
    // reduce over the row groups inside the wavefront (xor butterfly: both
    // partners add the same two values, so all lanes of a column agree bitwise)
#pragma unroll
    for (int off = SH::CG; off < 64; off <<= 1) {
      pk.x += __shfl_xor(pk.x, off, 64); pk.y += __shfl_xor(pk.y, off, 64);
      pk.z += __shfl_xor(pk.z, off, 64); pk.w += __shfl_xor(pk.w, off, 64);
      pq.x += __shfl_xor(pq.x, off, 64); pq.y += __shfl_xor(pq.y, off, 64);
      pq.z += __shfl_xor(pq.z, off, 64); pq.w += __shfl_xor(pq.w, off, 64);
    }
    if (lane < SH::CG) {
      *reinterpret_cast<float4*>(&s_pk[wave * DV + 4 * cg]) = pk;
      *reinterpret_cast<float4*>(&s_pq[wave * DV + 4 * cg]) = pq;
    }
    __syncthreads();
    // then over the wavefronts in a fixed order
    float4 ks = *reinterpret_cast<const float4*>(&s_pk[4 * cg]);
    float4 qs = *reinterpret_cast<const float4*>(&s_pq[4 * cg]);
#pragma unroll
    for (int w = 1; w < SH::NW; ++w) {
      const float4 a = *reinterpret_cast<const float4*>(&s_pk[w * DV + 4 * cg]);
      const float4 b = *reinterpret_cast<const float4*>(&s_pq[w * DV + 4 * cg]);
      ks.x += a.x; ks.y += a.y; ks.z += a.z; ks.w += a.w;
      qs.x += b.x; qs.y += b.y; qs.z += b.z; qs.w += b.w;
    }
    const float beta = s_scal[0];
    const float4 v = *reinterpret_cast<const float4*>(&s_v[4 * cg]);
    float4 u;
    u.x = beta * (v.x - ks.x); u.y = beta * (v.y - ks.y); u.z = beta * (v.z - ks.z); u.w = beta * (v.w - ks.w);
    float4 o;
    o.x = fmaf(qk, u.x, qs.x); o.y = fmaf(qk, u.y, qs.y); o.z = fmaf(qk, u.z, qs.z); o.w = fmaf(qk, u.w, qs.w);
#pragma unroll
    for (int m = 0; m < SH::RPT; ++m) {
      const float ki = s_k[rg + SH::RG * m];
      float4 s = S[m];
      s.x = rank1(s.x, ki, u.x); s.y = rank1(s.y, ki, u.y); s.z = rank1(s.z, ki, u.z); s.w = rank1(s.w, ki, u.w);
      S[m] = s;
    }
    u_out = u;
    o_out = o;
  }
};

constexpr int kRowsGridY = 65535;  // the largest y extent of a grid

template <int DK, int DV, typename RawT, bool VERIFY>
__global__ __launch_bounds__(256) void kda_rows_kernel(RowsArgs<RawT> p) {
  using SH = RowsShape<DK, DV>;
  // batches above the 65535 limit of a grid's y extent continue in z
  const int h = blockIdx.x, b = (int)(blockIdx.z * kRowsGridY + blockIdx.y);
  if (b >= p.batch) return;
  const int t = threadIdx.x;
  const int slot = p.slots ? p.slots[b] : b;
  if (slot < 0) return;
  const int H = p.H;
  const int64_t C = (int64_t)H * (2 * DK + DV);
  const int cg = t % SH::CG, rg = t / SH::CG;

  __shared__ __align__(16) float s_q[DK];
  __shared__ __align__(16) float s_k[DK];
  __shared__ __align__(16) float s_v[DV];
  __shared__ __align__(16) float s_a[DK];
  __shared__ float s_red[SH::NW * 8];
  __shared__ __align__(16) float s_pk[SH::NW * DV];
  __shared__ __align__(16) float s_pq[SH::NW * DV];
  __shared__ float s_scal[4];
  RowStep<DK, DV, RawT> rs{s_q, s_k, s_v, s_a, s_red, s_pk, s_pq, s_scal};

  // 1. issue the state loads first (64 KB per head at d=128), non-temporal
  float* Sg = p.state + ((int64_t)slot * H + h) * DK * DV;
  float4 S[SH::RPT];
#pragma unroll
  for (int m = 0; m < SH::RPT; ++m)
    S[m] = load_nt4(Sg + (int64_t)(rg + SH::RG * m) * DV + 4 * cg);

  // 2. conv weights and carried conv rows of the channels this thread owns
  ChanHist<RawT> ch;
  int64_t cq_ch = -1, ck_ch = -1;  // global conv channel indices owned (q/k or v)
  if (t < DK) {
    cq_ch = (int64_t)h * DK + t;
    ck_ch = (int64_t)H * DK + (int64_t)h * DK + t;
  } else if (t < DK + DV) {
    cq_ch = 2 * (int64_t)H * DK + (int64_t)h * DV + (t - DK);
  }
  RawT* cs = p.conv_state + (int64_t)slot * 3 * C;
  if (cq_ch >= 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) ch.wq[j] = p.conv_w[cq_ch * 4 + j];
#pragma unroll
    for (int r = 0; r < 3; ++r) ch.hq[r] = cs[r * C + cq_ch];
  }
  if (ck_ch >= 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) ch.wk[j] = p.conv_w[ck_ch * 4 + j];
#pragma unroll
    for (int r = 0; r < 3; ++r) ch.hk[r] = cs[r * C + ck_ch];
  }

  if constexpr (VERIFY) {
    // 3. commit n_commit rows of the previous window from its log.  A row's decay
    //    and key (one element per thread) and update (16 bytes per thread) go
    //    through LDS, and every thread reads back the entries of its state rows;
    //    the next row's log entries load while the current row is applied.
    int nc = (p.n_commit && p.in_window > 0) ? p.n_commit[b] : 0;
    nc = nc < 0 ? 0 : (nc > p.in_window ? p.in_window : nc);
    {
      const int tk = t < DK ? t : (t < 2 * DK ? t - DK : 0);  // a (t < DK) or k (DK <= t < 2 DK) of channel tk
      const int tu = t < DV / 4 ? t : 0;                      // 4 entries of u
      auto log_row = [&](int r, float& av, float4& uv, RawT& rq, RawT& rk) {
        const int rr = r < nc ? r : (nc > 0 ? nc - 1 : 0);  // clamped: every load is unconditional
        const int64_t base_k = (((int64_t)b * p.in_window + rr) * H + h) * DK;
        const int64_t base_v = (((int64_t)b * p.in_window + rr) * H + h) * DV;
        av = (t < DK ? p.in_a : p.in_k)[base_k + tk];
        uv = *reinterpret_cast<const float4*>(p.in_u + base_v + 4 * tu);
        const RawT* rows = p.in_rows + ((int64_t)b * p.in_window + rr) * C;
        rq = rows[cq_ch >= 0 ? cq_ch : 0];
        rk = rows[ck_ch >= 0 ? ck_ch : 0];
      };
      float av;
      float4 uv;
      RawT rq, rk;
      if (nc > 0) log_row(0, av, uv, rq, rk);
      for (int r = 0; r < nc; ++r) {
        if (t < DK) s_a[t] = av;
        else if (t < 2 * DK) s_k[t - DK] = av;
        if (t < DV / 4) *reinterpret_cast<float4*>(&s_v[4 * t]) = uv;
        const RawT cur_q = rq, cur_k = rk;
        log_row(r + 1, av, uv, rq, rk);
        __syncthreads();
        const float4 u = *reinterpret_cast<const float4*>(&s_v[4 * cg]);
#pragma unroll
        for (int m = 0; m < SH::RPT; ++m) {
          const int i = rg + SH::RG * m;
          const float a = s_a[i], ki = s_k[i];
          float4 s = S[m];
          s.x = rank1(decay(s.x, a), ki, u.x); s.y = rank1(decay(s.y, a), ki, u.y);
          s.z = rank1(decay(s.z, a), ki, u.z); s.w = rank1(decay(s.w, a), ki, u.w);
          S[m] = s;
        }
        if (cq_ch >= 0) { ch.hq[0] = ch.hq[1]; ch.hq[1] = ch.hq[2]; ch.hq[2] = cur_q; }
        if (ck_ch >= 0) { ch.hk[0] = ch.hk[1]; ch.hk[1] = ch.hk[2]; ch.hk[2] = cur_k; }
        __syncthreads();  // the next row overwrites the LDS entries this row read
      }
    }
    if (nc > 0) {
#pragma unroll
      for (int m = 0; m < SH::RPT; ++m)
        store_nt4(Sg + (int64_t)(rg + SH::RG * m) * DV + 4 * cg, S[m]);
      if (cq_ch >= 0)
        for (int r = 0; r < 3; ++r) cs[r * C + cq_ch] = ch.hq[r];
      if (ck_ch >= 0)
        for (int r = 0; r < 3; ++r) cs[r * C + ck_ch] = ch.hk[r];
    }
    // 4. the window's own rows, on the register copy of the committed state
    int nrow = p.window;  // uniform over the workgroup (one sequence)
    if (p.wlen) {
      const int wl = p.wlen[b];
      nrow = wl < 0 ? 0 : (wl > p.window ? p.window : wl);
    }
    auto row_in = [&](int r) {  // clamped: every load is unconditional
      const int64_t row_h = ((int64_t)b * p.window + (r < nrow ? r : (nrow > 0 ? nrow - 1 : 0))) * H + h;
      return rs.load_in(p, row_h * DK, row_h * DV, row_h);
    };
    typename RowStep<DK, DV, RawT>::RowIn nx{};
    if (nrow > 0) nx = row_in(0);
    for (int r = 0; r < nrow; ++r) {
      const int64_t row_h = ((int64_t)b * p.window + r) * H + h;
      const typename RowStep<DK, DV, RawT>::RowIn in = nx;
      nx = row_in(r + 1);  // the next row's inputs load while this row computes
      RawT raw_q{}, raw_k{};
      const float qk = rs.preamble(p, ch, in, raw_q, raw_k);
      float4 u, o;
      rs.step(S, qk, u, o);
      if (rg == 0) {
        *reinterpret_cast<float4*>(p.o + row_h * DV + 4 * cg) = o;
        *reinterpret_cast<float4*>(p.out_u + row_h * DV + 4 * cg) = u;
      }
      RawT* orow = p.out_rows + ((int64_t)b * p.window + r) * C;
      if (t < DK) {
        p.out_a[row_h * DK + t] = s_a[t];
        p.out_k[row_h * DK + t] = s_k[t];
        orow[cq_ch] = raw_q;
        orow[ck_ch] = raw_k;
      } else if (t < DK + DV) {
        orow[cq_ch] = raw_q;
      }
      __syncthreads();  // the next row overwrites the LDS vectors this row read
    }
  } else {
    // decode: one row, committed at once
    const int64_t row_h = (int64_t)b * H + h;
    RawT raw_q{}, raw_k{};
    const float qk = rs.preamble(p, ch, rs.load_in(p, row_h * DK, row_h * DV, row_h), raw_q, raw_k);
    float4 u, o;
    rs.step(S, qk, u, o);
#pragma unroll
    for (int m = 0; m < SH::RPT; ++m)
      store_nt4(Sg + (int64_t)(rg + SH::RG * m) * DV + 4 * cg, S[m]);
    if (rg == 0) *reinterpret_cast<float4*>(p.o + row_h * DV + 4 * cg) = o;
    if (cq_ch >= 0)
      for (int r = 0; r < 3; ++r) cs[r * C + cq_ch] = ch.hq[r];
    if (ck_ch >= 0)
      for (int r = 0; r < 3; ++r) cs[r * C + ck_ch] = ch.hk[r];
  }
}

template <int DK, int DV, typename RawT, bool VERIFY>
static hipError_t launch_rows_t(const RowsLaunch& L, hipStream_t s) {
  RowsArgs<RawT> p;
  p.H = L.H; p.gate_mode = L.gate_mode; p.act = L.act; p.batch = L.batch; p.window = L.window; p.lb = L.lb;
  p.slots = L.slots; p.state = L.state; p.conv_state = static_cast<RawT*>(L.conv_state); p.conv_w = L.conv_w;
  p.q = static_cast<const RawT*>(L.q); p.k = static_cast<const RawT*>(L.k); p.v = static_cast<const RawT*>(L.v);
  p.g = static_cast<const RawT*>(L.g); p.beta = static_cast<const RawT*>(L.beta); p.o = L.o;
  p.g_per_head = L.g_per_head;
  p.n_commit = L.n_commit; p.wlen = L.window_lens; p.in_a = L.in_a; p.in_k = L.in_k; p.in_u = L.in_u;
  p.in_rows = static_cast<const RawT*>(L.in_rows); p.in_window = L.in_window;
  p.out_a = L.out_a; p.out_k = L.out_k; p.out_u = L.out_u; p.out_rows = static_cast<RawT*>(L.out_rows);
  const int gy = L.batch < kRowsGridY ? L.batch : kRowsGridY;
  dim3 grid(L.H, gy, (L.batch + kRowsGridY - 1) / kRowsGridY);
  hipLaunchKernelGGL((kda_rows_kernel<DK, DV, RawT, VERIFY>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

template <bool VERIFY>
static hipError_t launch_rows_v(const RowsLaunch& L, hipStream_t s) {
  const bool bf = L.in_dtype == 1;
#define KDA_ROWS_CASE(DK_, DV_)                                                                  \
  if (L.dk == DK_ && L.dv == DV_)                                                                \
    return bf ? launch_rows_t<DK_, DV_, uint16_t, VERIFY>(L, s) : launch_rows_t<DK_, DV_, float, VERIFY>(L, s);
  KDA_ROWS_CASE(64, 64)
  KDA_ROWS_CASE(64, 128)
  KDA_ROWS_CASE(128, 64)
  KDA_ROWS_CASE(128, 128)
#undef KDA_ROWS_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_rows(const RowsLaunch& L, bool verify, hipStream_t s) {
  if (L.batch == 0 || L.H == 0) return hipSuccess;
  return verify ? launch_rows_v<true>(L, s) : launch_rows_v<false>(L, s);
}

}  // namespace kda
