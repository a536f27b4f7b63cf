/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention layer library.
 *
 * The layer (TensorFold issue #850, "Ling-3.1-flash on CUDA", the comment that
 * describes the shared KDA module; onnxruntime-genai PR #2843, the op list in
 * its description) takes a model's projected rows and runs, per head:
 *   1. a causal short conv over the q, k and v rows, with the last W-1 rows
 *      carried across calls in a conv state (CausalConvWithState /
 *      VarlenCausalConvWithState in PR #2843), then SiLU;
 *   2. L2 normalisation of q and k over the key dimension;
 *   3. a per-key-dimension log-decay gate g (softplus: g = -softplus(x); safe:
 *      g = lower_bound * sigmoid(x), PR #2843 gate_activation='sigmoid' with
 *      gate_lower_bound), decay a = e^g, and a per-head beta = sigmoid(x_b)
 *      (with KDA_DECAY_PER_HEAD, one decay per head and row: the scalar-decay
 *      gated delta rule);
 *   4. the gated delta rule on one fp32 d_k x d_v state per (sequence, head):
 *        S_t = (I - beta_t k_t k_t^T) Diag(a_t) S_{t-1} + beta_t k_t v_t^T,
 *        o_t = S_t^T q_t;
 *   5. the sigmoid-gated output RMSNorm y = o / sqrt(mean(o^2) + eps) * w *
 *      sigmoid(z) (GatedRMSNorm with activation 'sigmoid' in PR #2843).
 * Prompt rows run chunk-parallel (64-row chunks anchored at each sequence's
 * first row); decode rows and speculative verify windows run row by row, and a
 * verify window logs each row's decay, normalised key and update so that a
 * later call can commit the accepted rows (TensorFold #850: a window's rows
 * replay from that log with the same bits as rows decoded one at a time).
 *
 * Conventions shared by every entry point
 *   - Memory: the caller owns every buffer (device memory unless stated); the
 *     library never allocates.  Scratch comes from a caller workspace.
 *   - Streams: every call is enqueued on `stream` and returns without waiting.
 *   - Layouts: row-major, token-major packed rows.
 *       q, k, g rows      [T, H, d_k]      v, z, o rows   [T, H, d_v]
 *       (raw g rows [T, H] when decay_shape is KDA_DECAY_PER_HEAD)
 *       beta logits       [T, H]
 *       state             [S_slots, H, d_k, d_v]  fp32, d_v contiguous
 *       conv channels     C = H*(2*d_k + d_v), ordered [q: H*d_k | k: H*d_k | v: H*d_v]
 *       conv weight       [C, 4] fp32, tap 3 multiplies the current row
 *       conv state        [S_slots, 3, C] in the raw-row dtype, oldest row first
 *   - Slots: `slots` (int32 [num_seqs or batch], device) maps sequence n to its
 *     row of `state` / `conv_state`; NULL means slot n.  A negative slot skips
 *     the sequence: nothing of it is read or written.
 *   - Alignment: buffers the kernels move with 128-bit accesses must be 16-byte
 *     aligned: the state, the fp32 rows q_hat/k_hat/v/g of the prompt path, the
 *     raw q/k/v/g rows handed to kda_prefill_varlen in `raw`, the output o of
 *     every call, a log's u, the z, weight and y of the norm epilogue, and
 *     every buffer of gated_rmsnorm_out.  Every other pointer needs its
 *     element alignment.
 *   - Errors: each call returns KDA_OK or one KDA_E_* code.  All validation
 *     happens before the first launch; on error nothing is enqueued and no
 *     output is written.  kda_last_error() gives a message (thread-local).
 *   - Device-side contents (cu_seqlens monotone with cu[0]=0 and cu[N]=T, slots
 *     below the pool size, commit counts within the rows each sequence logged)
 *     are preconditions the library does not read back.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t;
typedef struct ihipEvent_t* hipEvent_t;

enum kda_status {
  KDA_OK = 0,
  KDA_E_ARG = 1,       /* null pointer, negative size, or more rows than cu_seqlens (int32) or a launch grid addresses */
  KDA_E_GEOMETRY = 2,  /* d_k or d_v not in {64, 128}, num_heads > 65535, conv width != 4, unknown decay shape,
                          window not in [0, 8] */
  KDA_E_ALIGN = 3,     /* a pointer is not aligned as its access needs (see Alignment) */
  KDA_E_GATE = 4,      /* unknown gate mode, or safe mode with a lower bound that is not finite and < 0 */
  KDA_E_DTYPE = 5,     /* unknown dtype, activation or precision policy */
  KDA_E_WORKSPACE = 6, /* workspace missing or smaller than kda_prefill_workspace_bytes() */
  KDA_E_HIP = 7        /* a HIP launch failed */
};

enum kda_dtype { KDA_DTYPE_F32 = 0, KDA_DTYPE_BF16 = 1 };
enum kda_gate { KDA_GATE_SOFTPLUS = 0, KDA_GATE_SAFE = 1 };
enum kda_act { KDA_ACT_NONE = 0, KDA_ACT_SILU = 1 };
/* Shape of the decay: one log decay per key dim (the KDA layer), or one per head
 * and row broadcast over the key dims (the scalar-decay gated delta rule); raw g
 * rows are then [.., H] instead of [.., H, d_k].  The recurrence is the same
 * with equal per-dim decays, and every entry point gives the bits it gives for
 * the broadcast rows. */
enum kda_decay { KDA_DECAY_PER_DIM = 0, KDA_DECAY_PER_HEAD = 1 };
/* Arithmetic of the chunked prompt path's matrix products (all accumulate in fp32):
 *   FP32   fp32 matrix-core products;
 *   BF16X3 each fp32 operand split into bf16 hi + lo and the product formed as
 *          hi*hi + hi*lo + lo*hi (relative error about 2^-16 per product);
 *          the fp32 range throughout;
 *   FP16   in the inter-chunk pass, the per-chunk operands (each entry bounded
 *          by 1) rounded once to fp16 and the state / update operands split
 *          into fp16 hi + lo (relative error about 2^-12 per product); the
 *          intra-chunk products as in BF16X3.
 *          Domain: each state and update entry x must satisfy |x| < 65504 (the
 *          largest finite fp16 value); the pair hi + lo then holds x to within
 *          max(2^-22 |x|, 2^-25), so entries much smaller than 2^-12 lose
 *          relative precision.  Outside the domain the split overflows and the
 *          call's o, y and state are not finite (never finite and wrong).  Use
 *          BF16X3, BF16X2 or FP32 for states or value rows that may leave it.
 *   BF16X2 FP16's layout with bf16 in place of fp16: the A operands rounded
 *          once to bf16 (relative error about 2^-10 per product), the state /
 *          update operands split into bf16 hi + lo, so every state and update
 *          entry keeps the fp32 range: the speed of FP16 with the domain of
 *          BF16X3, at about 8 times FP16's error (relative L2 of o about 1.6e-3
 *          over a 4096-row prompt with bf16 rows, near the 2e-3 of bf16 inputs'
 *          own rounding). */
enum kda_precision { KDA_PREC_FP32 = 0, KDA_PREC_BF16X3 = 1, KDA_PREC_FP16 = 2, KDA_PREC_BF16X2 = 3 };

typedef struct kda_dims {
  int32_t num_heads;  /* 1 <= H <= 65535 */
  int32_t head_dim_k; /* d_k in {64, 128} */
  int32_t head_dim_v; /* d_v in {64, 128} */
  int32_t conv_width; /* must be 4 */
  int32_t in_dtype;   /* kda_dtype of raw rows (q, k, v, g, beta logits) and of the conv state */
  int32_t conv_act;   /* kda_act applied after the conv */
  int32_t precision;  /* kda_precision of the prompt path's matrix products */
  int32_t decay_shape; /* kda_decay of the raw g rows */
} kda_dims;

/* Log of a verify window: everything a later call needs to commit its rows.
 * Device buffers; `window` is the row count they were written with. */
typedef struct kda_log {
  float* a;        /* [B, window, H, d_k] per-row decay e^g */
  float* k_hat;    /* [B, window, H, d_k] per-row L2-normalised key */
  float* u;        /* [B, window, H, d_v] per-row update beta*(v - (Diag(a)S)^T k_hat) */
  void* conv_rows; /* [B, window, C] raw conv input rows (in_dtype), conv channel order */
  int32_t window;  /* rows per sequence in this log, 0..8 */
} kda_log;

/* kda_prep -- preamble of the prompt path (parts 1-3 above) for packed varlen rows.
 *   cu_seqlens      int32 [num_seqs+1] device, packed row offsets
 *   slots           int32 [num_seqs] device or NULL (conv_state row of each sequence)
 *   q_raw,k_raw     [t_tot, H, d_k] in_dtype;  v_raw [t_tot, H, d_v];  g_raw [t_tot, H, d_k]
 *                   ([t_tot, H] with KDA_DECAY_PER_HEAD; g_out is then that decay repeated over d_k)
 *   beta_logit      [t_tot, H] in_dtype
 *   conv_weight     [C, 4] fp32
 *   conv_state_in   [slots, 3, C] in_dtype, read;  conv_state_out  same shape, written
 *                   after all reads (the two may be the same buffer)
 *   gate_mode       kda_gate;  lower_bound used in safe mode only (finite, < 0)
 *   outputs (fp32): q_hat, k_hat [t_tot,H,d_k]; v_out [t_tot,H,d_v]; g_out (log decay)
 *                   [t_tot,H,d_k]; beta_out [t_tot,H]
 * The outputs are what kda_prefill_varlen consumes.  q_raw, k_raw, v_raw, g_raw
 * and the four wide outputs move with 16-byte accesses and must be 16-byte
 * aligned (else KDA_E_ALIGN); beta_logit, beta_out and the conv state need only
 * element alignment. */
int kda_prep(const kda_dims* d, int32_t num_seqs, int64_t t_tot, const int32_t* cu_seqlens, const int32_t* slots,
             const void* q_raw, const void* k_raw, const void* v_raw, const float* conv_weight,
             const void* conv_state_in, void* conv_state_out, const void* g_raw, const void* beta_logit,
             int32_t gate_mode, float lower_bound, float* q_hat, float* k_hat, float* v_out, float* g_out,
             float* beta_out, hipStream_t stream);

/* Bytes of workspace kda_prefill_varlen needs for this geometry (an upper
 * bound that depends only on num_seqs and t_tot). */
size_t kda_prefill_workspace_bytes(const kda_dims* d, int32_t num_seqs, int64_t t_tot);

/* Raw projected rows and preamble parameters, for running the preamble inside
 * the prompt kernels (kda_prefill_varlen with a non-NULL `raw`).  Device
 * pointers; shapes and meaning as in kda_prep. */
typedef struct kda_raw_rows {
  const void* q_raw;          /* [t_tot, H, d_k] in_dtype */
  const void* k_raw;          /* [t_tot, H, d_k] */
  const void* v_raw;          /* [t_tot, H, d_v] */
  const void* g_raw;          /* [t_tot, H, d_k] */
  const void* beta_logit;     /* [t_tot, H] */
  const float* conv_weight;   /* [C, 4] fp32 */
  const void* conv_state_in;  /* [slots, 3, C] in_dtype, read */
  void* conv_state_out;       /* same shape, written after all reads (may equal conv_state_in) */
  int32_t gate_mode;          /* kda_gate */
  float lower_bound;          /* safe mode only: finite, < 0 */
} kda_raw_rows;

/* The gated output norm as the epilogue of a prompt call (kda_prefill_varlen
 * with a non-NULL `norm`): y = o / sqrt(mean(o^2) + eps) * weight * sigmoid(z)
 * over each row of d_v values, as gated_rmsnorm_out computes it.  Device
 * pointers, 16-byte aligned. */
typedef struct kda_norm_args {
  const void* z;              /* [t_tot, H, d_v] of z_dtype */
  int32_t z_dtype;            /* kda_dtype: F32 or BF16 */
  const float* weight;        /* [d_v] fp32 */
  float eps;                  /* finite, >= 0 */
  void* y;                    /* [t_tot, H, d_v] of y_dtype, written */
  int32_t y_dtype;            /* kda_dtype: F32 or BF16 */
} kda_norm_args;

/* kda_prefill_varlen -- the delta rule (part 4) over packed prompt rows, in
 * 64-row chunks anchored at each sequence's first row (WY/UT form with an
 * intra-chunk lower-triangular solve, then a sequential pass over chunks).
 *   q_hat, k_hat, v, g, beta   fp32 outputs of kda_prep (g is the log decay);
 *                              ignored (may be NULL) when `raw` is given
 *   raw     NULL, or raw rows + preamble parameters: the preamble (parts 1-3)
 *           then runs inside the prompt kernels, with the same bits as kda_prep,
 *           and the conv state is carried as kda_prep would carry it
 *   norm    NULL, or the output norm (part 5) as the call's epilogue: y gets
 *           the same bits as gated_rmsnorm_out on o would give.  A row's norm
 *           spans all d_v columns, which the scan spreads over up to eight
 *           workgroups (16, 32 or 64 columns each, by how many workgroups the
 *           call has), so the epilogue is one more launch on the stream, after
 *           the scan; rows of a skipped sequence (negative slot) keep their y.
 *   state   fp32 [slots, H, d_k, d_v], read as the initial state and
 *           overwritten with the final state of each sequence
 *   o       fp32 [t_tot, H, d_v], pre-norm output (written also when `norm` is given)
 *   workspace  device scratch of at least kda_prefill_workspace_bytes(), 256-byte aligned
 * A prompt cut at a multiple of 64 rows, with the state carried, gives the same
 * bits as the uncut prompt. */
int kda_prefill_varlen(const kda_dims* d, int32_t num_seqs, int64_t t_tot, const int32_t* cu_seqlens,
                       const int32_t* slots, const float* q_hat, const float* k_hat, const float* v,
                       const float* g, const float* beta, const kda_raw_rows* raw, const kda_norm_args* norm,
                       float* state, float* o, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* kda_prefill_varlen_noalloc -- for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The same call as kda_prefill_varlen (same arguments, kernels,
 * bits and errors) without the workspace argument: the sink and the chunk
 * records go to a scratch array the library holds in each device's memory,
 * KDA_NOALLOC_SCRATCH_BYTES (160 MiB; T=4096 rows at H=16, d=128 fit under
 * every precision policy), from the first use of the library on that device
 * until the process ends.  The call itself allocates nothing.
 *   Errors: KDA_E_WORKSPACE when kda_prefill_workspace_bytes() for the call's
 *   geometry exceeds KDA_NOALLOC_SCRATCH_BYTES (nothing is enqueued);
 *   KDA_E_HIP if the scratch's device address cannot be resolved (the first
 *   call on each device resolves it, before any launch).
 *   Sharing: every call on a device uses that device's one scratch, which keeps
 *   the last call's contents (nothing in it has to start at zero).  Calls that
 *   overlap on one device -- on two streams, or from two host threads without
 *   ordering between their streams -- race on it; the caller orders them. */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)160 << 20)
int kda_prefill_varlen_noalloc(const kda_dims* d, int32_t num_seqs, int64_t t_tot, const int32_t* cu_seqlens,
                               const int32_t* slots, const float* q_hat, const float* k_hat, const float* v,
                               const float* g, const float* beta, const kda_raw_rows* raw, const kda_norm_args* norm,
                               float* state, float* o, hipStream_t stream);

/* kda_decode -- one row per sequence (parts 1-4 fused): conv step on the conv
 * state, gates, norms, state step, readout.
 *   q_raw,k_raw,g_raw [batch,H,d_k], v_raw [batch,H,d_v], beta_logit [batch,H]  (in_dtype)
 *   state [slots,H,d_k,d_v] fp32 and conv_state [slots,3,C] (in_dtype) updated in place
 *   o     fp32 [batch, H, d_v] */
int kda_decode(const kda_dims* d, int32_t batch, const int32_t* slots, float* state, void* conv_state,
               const float* conv_weight, const void* q_raw, const void* k_raw, const void* v_raw, const void* g_raw,
               const void* beta_logit, int32_t gate_mode, float lower_bound, float* o, hipStream_t stream);

/* kda_verify_window -- speculative verify window on top of committed state.
 * First commits n_commit[b] rows (0..log_in->window) of the previous window
 * from log_in: S = Diag(a) S + k_hat u^T per row and the conv state advances
 * by those raw rows, bit for bit as kda_decode would have left them.  Then it
 * runs `window` new rows per sequence row by row on a private copy of the
 * committed state, writes their outputs o [batch, window, H, d_v] (same bits
 * as kda_decode on those rows) and their log to log_out.  The state and conv
 * state stay at the committed point.  window = 0 only commits.
 *   window_lens  int32 [batch] device, or NULL: sequence b runs only its first
 *             window_lens[b] rows of the window (clamped to [0, window]); its o
 *             and log rows past those are left alone, and a later commit of
 *             more rows than it ran is outside the preconditions
 *   n_commit  int32 [batch] device, or NULL when log_in is NULL (nothing to commit)
 *   rows      q_raw,k_raw,g_raw [batch,window,H,d_k], v_raw [batch,window,H,d_v],
 *             beta_logit [batch,window,H]  (in_dtype)
 *   log_out   buffers sized for `window`; must not overlap log_in. */
int kda_verify_window(const kda_dims* d, int32_t batch, int32_t window, const int32_t* window_lens,
                      const int32_t* slots, float* state,
                      void* conv_state, const float* conv_weight, const int32_t* n_commit, const kda_log* log_in,
                      const kda_log* log_out, const void* q_raw, const void* k_raw, const void* v_raw,
                      const void* g_raw, const void* beta_logit, int32_t gate_mode, float lower_bound, float* o,
                      hipStream_t stream);

/* gated_rmsnorm_out -- part 5: y = o / sqrt(mean(o^2) + eps) * w * sigmoid(z)
 * over rows of d_v values.
 *   o fp32 [rows, d_v];  z [rows, d_v] of z_dtype;  w fp32 [d_v];  y [rows, d_v] of y_dtype */
int gated_rmsnorm_out(int64_t rows, int32_t d_v, const float* o, const void* z, int32_t z_dtype, const float* w,
                      float eps, void* y, int32_t y_dtype, hipStream_t stream);

/* Message for the last error returned on this thread ("" if none). */
const char* kda_last_error(void);

/* kda_set_timing_events -- measurement hook for benchmarks.  Until the next
 * call, every kda_prefill_varlen call made by this thread records events[2i]
 * and events[2i+1] on its stream immediately before and after its kernel i,
 * for 2i+1 < count:
 *   i = 0 intra-chunk kernel,  1 inter-chunk scan (which also carries the conv
 *   state when `raw` is given),  2 the output norm when `norm` is given.
 * The events are caller-owned hipEvent_t handles, already created; the library
 * keeps only the pointer, which must stay valid while set.  count = 0 (events
 * may be NULL) turns the hook off.  Errors: KDA_E_ARG for a negative or odd
 * count, or NULL events with count > 0. */
int kda_set_timing_events(hipEvent_t* events, int32_t count);

#ifdef __cplusplus
}
#endif
#endif /* KDA_H */
