/*
 * libkda -- Kimi Delta Attention (KDA) on AMD Instinct MI355X (gfx950).
 *
 * The recurrence (per sequence, per head; state S is [K][V] fp32, rows are key
 * channels):
 *     q^ = q / sqrt(sum q^2 + 1e-6),  k^ = k / sqrt(sum k^2 + 1e-6)
 *     log alpha = lower_bound * sigmoid(exp(A_log[h]) * (g + dt_bias[h]))   (per key channel)
 *     beta      = sigmoid(beta_logit)
 *     S <- Diag(alpha) S;   S <- S + beta k^ (v - S^T k^)^T;   o = scale * S^T q^
 * The gate, the in-kernel q/k L2 norm and the raw beta logits are those of
 * vLLM PR #55737 "Use FlashKDA for KDA chunked prefill" (opening commit
 * message, "Purpose").  The one-launch multi-step verify with a read-only
 * state pool and one state row per draft step is that of TensorRT-LLM PR
 * #21179 "GLM-5.3-Flash FP8 performance fixes on Hopper" (fused-verify commit
 * message).  Supported shapes follow the same vLLM page: bf16 inputs,
 * head_dim 128, bounded gate.
 *
 * Conventions shared by every entry point:
 *  - Every buffer is caller-owned device memory.  The library never allocates
 *    or frees memory, never synchronises a stream and never reads device
 *    memory from the host.  Work is enqueued on `stream` (a hipStream_t cast
 *    to void*, NULL = the default stream) and is asynchronous.
 *  - bf16 tensors are passed as raw 16-bit words (void*), laid out token-major:
 *    element (token t, head h, channel c) sits at t*token_stride + h*128 + c.
 *    A token stride of 0 means the dense default (H*128, or H for beta logits);
 *    larger strides read rows in place from a fused projection.
 *  - States are fp32 [.., H, 128 (key), 128 (value)] row-major, value channel
 *    contiguous.
 *  - Only host-side arguments are validated; a failed check returns a status
 *    and sets a thread-local message (kda_last_error) without enqueuing work.
 *    Device-side contents (cu_seqlens monotone with cu[0] = 0 and
 *    cu[N] == total_tokens, indices in range, finite inputs) are preconditions.
 *  - Results are deterministic run to run (no atomics).
 *  - Prefill feeds fp16 MFMA operands with v, the state and values a small
 *    multiple of them (X = V - K_Gamma S and U = T X of the chunked form), so |v|
 *    and |state| must stay below 2^14.  Within that range the largest operand stays
 *    a few times below the fp16 maximum (65504); past it an operand can overflow,
 *    and out and final_state then hold inf or NaN while the call still returns
 *    KDA_OK (device contents are never checked).  The Python binding's check=True
 *    rejects |v| or |initial_state| >= 2^14.  Verify computes in fp32 throughout
 *    and has no such limit.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 2
#define KDA_HEAD_DIM 128
#define KDA_MAX_VERIFY_STEPS 64

typedef enum kda_status {
  KDA_OK = 0,
  KDA_ERR_INVALID_ARGUMENT = 1,   /* null pointer, negative size, bad stride, overlap */
  KDA_ERR_UNSUPPORTED = 2,        /* head_dim != 128, lower_bound outside [-5, 0], too many steps */
  KDA_ERR_WORKSPACE_TOO_SMALL = 3,
  KDA_ERR_HIP = 4                 /* a HIP runtime call or a kernel launch failed */
} kda_status;

/* Shapes and strides of one prefill call.  All values are host integers:
 * nothing is read back from the device (the lesson of TensorRT-LLM PR #21179,
 * host cu_seqlens commit: a device read of chunk counts stalls every layer). */
typedef struct kda_prefill_desc {
  int32_t num_seqs;          /* N; cu_seqlens holds N+1 entries */
  int32_t total_tokens;      /* T_total == cu_seqlens[N] */
  int32_t num_heads;         /* H >= 1 */
  int32_t head_dim;          /* must be 128 */
  float scale;               /* output scale; <= 0 selects 1/sqrt(128) */
  int32_t num_state_rows;    /* rows of initial_state (N when indexed directly, pool slots when indexed) */
  int64_t q_token_stride, k_token_stride, v_token_stride, g_token_stride;  /* elements, 0 = H*128 */
  int64_t beta_token_stride; /* elements, 0 = H */
  int64_t out_token_stride;  /* elements, 0 = H*128 */
  /* Scattered output (the mixed speculative step of vLLM PR #55737, "...code steps
   * too" commit: prefill outputs land in the layer buffer at non_spec_token_indx).
   * NULL: token t's output is row t of out.  Otherwise a device int32 [T_total]:
   * token t's output is row out_token_index[t] of out (rows out_token_stride
   * apart); an index outside [0, out_rows) is not written.  Indices must be
   * distinct (rows written twice hold either value). */
  const int32_t* out_token_index;
  int64_t out_rows;          /* rows of out when out_token_index is given */
} kda_prefill_desc;

typedef struct kda_verify_desc {
  int32_t batch;             /* B rows; token of row b, step t is b*num_steps + t */
  int32_t num_steps;         /* T draft steps per row, 1..KDA_MAX_VERIFY_STEPS */
  int32_t num_heads;         /* H */
  int32_t head_dim;          /* must be 128 */
  float scale;               /* <= 0 selects 1/sqrt(128) */
  int32_t num_slots;         /* rows of state_pool */
  int64_t q_token_stride, k_token_stride, v_token_stride, g_token_stride;
  int64_t beta_token_stride;
  int64_t out_token_stride;
  /* As in kda_prefill_desc, for token b*num_steps + t (spec_token_indx). */
  const int32_t* out_token_index;
  int64_t out_rows;
} kda_verify_desc;

typedef struct kda_commit_desc {
  int32_t batch;             /* B verify rows */
  int32_t num_steps;         /* T: rows per verify row in intermediate_state */
  int32_t num_heads;         /* H */
  int32_t head_dim;          /* must be 128 */
  int32_t num_slots;         /* rows of state_pool */
} kda_commit_desc;

/* Bytes of caller-provided workspace kda_chunk_prefill needs for these shapes.
 * Returns 0 for shapes the library does not support. */
size_t kda_chunk_prefill_workspace_size(int32_t num_seqs, int32_t total_tokens,
                                        int32_t num_heads, int32_t head_dim);

/*
 * Varlen chunked prefill of N packed sequences (vLLM PR #55737, the FlashKDA
 * role: output written straight into the caller's layer buffer, final state
 * returned).
 *   q, k, g, v      bf16 [T_total, H, 128] (token-strided, see desc)
 *   beta_logits     bf16 [T_total, H], raw logits
 *   A_log           fp32 [H];  dt_bias fp32 [H, 128]
 *   lower_bound     finite, in [-5, 0]
 *   cu_seqlens      device int32 [N+1]
 *   initial_state   fp32 [num_state_rows, H, 128, 128] or NULL (zero start)
 *   initial_state_idx  device int32 [N] or NULL.  When given, sequence n starts
 *                   from initial_state[initial_state_idx[n]]; an index < 0 or
 *                   >= num_state_rows starts from zero.  When NULL, sequence n
 *                   starts from initial_state[n].
 *   out             bf16 [T_total, H, 128]; must not overlap any input
 *   final_state     fp32 [N, H, 128, 128] or NULL (not written).  May alias
 *                   initial_state when both are indexed the same way.
 *   workspace       device scratch of at least kda_chunk_prefill_workspace_size bytes.
 * A zero-length sequence writes no output and copies its start state to final_state.
 * (T_total/64 + N) * H above 2^31 - 1 chunk-heads returns KDA_ERR_UNSUPPORTED.
 */
kda_status kda_chunk_prefill(const void* q, const void* k, const void* v, const void* g,
                             const void* beta_logits, const float* A_log, const float* dt_bias,
                             float lower_bound, const int32_t* cu_seqlens,
                             const float* initial_state, const int32_t* initial_state_idx,
                             void* out, float* final_state,
                             void* workspace, size_t workspace_bytes,
                             const kda_prefill_desc* desc, void* stream);

/*
 * The two phases of kda_chunk_prefill as separate calls, with the same
 * arguments and checks.  kda_chunk_prefill(...) is exactly
 * kda_chunk_prefill_intra(...) followed by kda_chunk_prefill_scan(...) on the
 * same stream with the same workspace: the intra phase (parallel over chunks
 * and heads) writes one record per (chunk, head) into the workspace, and the
 * scan phase (sequential over each sequence's chunks) reads them and writes
 * out and final_state.  Splitting lets a caller time or schedule the phases
 * on their own; the workspace contents between them are private to libkda.
 */
kda_status kda_chunk_prefill_intra(const void* q, const void* k, const void* v, const void* g,
                                   const void* beta_logits, const float* A_log,
                                   const float* dt_bias, float lower_bound,
                                   const int32_t* cu_seqlens, const float* initial_state,
                                   const int32_t* initial_state_idx, void* out,
                                   float* final_state, void* workspace, size_t workspace_bytes,
                                   const kda_prefill_desc* desc, void* stream);
kda_status kda_chunk_prefill_scan(const void* q, const void* k, const void* v, const void* g,
                                  const void* beta_logits, const float* A_log,
                                  const float* dt_bias, float lower_bound,
                                  const int32_t* cu_seqlens, const float* initial_state,
                                  const int32_t* initial_state_idx, void* out,
                                  float* final_state, void* workspace, size_t workspace_bytes,
                                  const kda_prefill_desc* desc, void* stream);

/*
 * kda_chunk_prefill without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Arguments, results and checks are those of kda_chunk_prefill;
 * the chunk records and segment states live in a fixed device array of
 * KDA_NOALLOC_SCRATCH_BYTES inside libkda instead.
 *  - Each GPU holds its own array, from the first call on that GPU until the process
 *    ends.  The call itself allocates and frees nothing.
 *  - Shapes whose kda_chunk_prefill_workspace_size exceeds KDA_NOALLOC_SCRATCH_BYTES
 *    return KDA_ERR_UNSUPPORTED without enqueuing work (e.g. H = 16 heads fit up to
 *    about 8K tokens per call).
 *  - Every call on one GPU shares that GPU's array and overwrites it before reading
 *    it; calls that overlap on one GPU (other streams, other threads) race and must
 *    be serialised by the caller.
 */
#define KDA_NOALLOC_SCRATCH_BYTES (128ll * 1024 * 1024)
kda_status kda_chunk_prefill_noalloc(const void* q, const void* k, const void* v, const void* g,
                                     const void* beta_logits, const float* A_log,
                                     const float* dt_bias, float lower_bound,
                                     const int32_t* cu_seqlens, const float* initial_state,
                                     const int32_t* initial_state_idx, void* out,
                                     float* final_state, const kda_prefill_desc* desc,
                                     void* stream);

/*
 * Fused multi-step verify (TensorRT-LLM PR #21179, fused-verify commit: the
 * fused_recurrent_kda role).  For each row b the state starts from
 * state_pool[state_idx[b]] (the pool is only read) and the T tokens of the row
 * are applied in order.
 *   q, k, g, v      bf16 [B*T, H, 128];  beta_logits bf16 [B*T, H]
 *   state_pool      fp32 [num_slots, H, 128, 128], read only
 *   state_idx       device int32 [B]; an index < 0 or >= num_slots marks a
 *                   padding row: its outputs are written as zeros and its
 *                   intermediate rows are left untouched.
 *   intermediate_state  fp32 [B, T, H, 128, 128]; row (b, t) receives the state
 *                   after token t of row b (0-based), so row (b, T-1) is the
 *                   state with every draft token accepted.  Must not overlap the pool.
 *   out             bf16 [B*T, H, 128]
 * B*T above 2^31 - 1 tokens returns KDA_ERR_UNSUPPORTED.
 * The arithmetic is fp32.  With few (row, head) pairs a call takes its tokens' sums
 * over the key channels from the state at the start of each block of 8 tokens (the
 * chunked form on 8 tokens), so a T-token call agrees with T one-token calls to fp32
 * rounding, not bit for bit; repeated calls are bitwise identical.
 */
kda_status kda_recurrent_verify(const void* q, const void* k, const void* v, const void* g,
                                const void* beta_logits, const float* A_log, const float* dt_bias,
                                float lower_bound, const float* state_pool,
                                const int32_t* state_idx, float* intermediate_state, void* out,
                                const kda_verify_desc* desc, void* stream);

/* The output-gate sigmoid RMSNorm applied to each output row before it is stored
 * (SGLang PR #42489 "Improve GLM-5.3-Flash DFlash decoding on B300": the sigmoid
 * RMSNorm of the attention output, tuned with the recurrence).  For output row r and
 * head h, with o the fp32 output of the recurrence (scale included):
 *     rstd = 1 / sqrt(mean(o^2) + eps),   y = o * rstd * weight * sigmoid(gate[r, h])
 * and y, rounded to bf16, is what lands in out.  Rows are the output rows (the token
 * index, or out_token_index[token] when the descriptor scatters). */
typedef struct kda_output_norm {
  const void* gate;            /* bf16 [out rows, H, 128], token-strided, 16-byte aligned */
  int64_t gate_token_stride;   /* elements, 0 = H*128; a multiple of 8 */
  const float* weight;         /* fp32 [128], shared by the heads, 16-byte aligned */
  float eps;                   /* finite, >= 0 */
  float* rstd;                 /* fp32 [out rows, H], or NULL (not written) */
} kda_output_norm;

/*
 * kda_recurrent_verify with the output-gate sigmoid RMSNorm fused into its output
 * store (one launch: the normalised rows never pass through memory unnormalised).
 * Arguments and checks are those of kda_recurrent_verify plus `norm` (not NULL); gate,
 * weight and rstd must not overlap out or the state buffers.  Padding rows store
 * y = 0 and rstd = 1/sqrt(eps).
 */
kda_status kda_recurrent_verify_gated(const void* q, const void* k, const void* v, const void* g,
                                      const void* beta_logits, const float* A_log,
                                      const float* dt_bias, float lower_bound,
                                      const float* state_pool, const int32_t* state_idx,
                                      float* intermediate_state, void* out,
                                      const kda_output_norm* norm, const kda_verify_desc* desc,
                                      void* stream);

/*
 * Commit after verify: the num_accepted_tokens rollback of vLLM PR #55737
 * ("...code steps too" commit message: spec-decode tokens keep the recurrent
 * kernel with num_accepted_tokens rollback).  For each row b whose slot
 * s = state_idx[b] lies in [0, num_slots) and whose count n = num_accepted[b]
 * lies in [1, T], state_pool[s] (all heads) becomes intermediate_state[b, n-1],
 * the state after the n accepted tokens.  Other rows leave the pool unchanged.
 *   intermediate_state  fp32 [B, T, H, 128, 128] as written by kda_recurrent_verify;
 *                       must not overlap the pool
 *   state_idx           device int32 [B] (the verify call's indices)
 *   num_accepted        device int32 [B]
 *   state_pool          fp32 [num_slots, H, 128, 128], updated in place
 * Rows of one call must name distinct slots.
 */
kda_status kda_commit_accepted(const float* intermediate_state, const int32_t* state_idx,
                               const int32_t* num_accepted, float* state_pool,
                               const kda_commit_desc* desc, void* stream);

typedef struct kda_norm_desc {
  int32_t tokens;            /* rows of x, gate and y */
  int32_t num_heads;         /* H: each token holds H rows of head_dim channels */
  int32_t head_dim;          /* must be 128 */
  float eps;                 /* added to mean(x^2); finite and >= 0 */
  int64_t x_token_stride, gate_token_stride, y_token_stride;   /* elements, 0 = H*128 */
} kda_norm_desc;

/*
 * Output-gate sigmoid RMSNorm (SGLang PR #42489 "Improve GLM-5.3-Flash DFlash decoding
 * on B300": the sigmoid RMSNorm of bf16, D = 128 rows, checked for output and rstd).
 * Per row of 128 channels (token t, head h):
 *     rstd = 1 / sqrt(mean(x^2) + eps),   y = x * rstd * weight * sigmoid(gate)
 *   x, gate         bf16 [tokens, H, 128] (token-strided)
 *   weight          fp32 [128], shared by the heads
 *   y               bf16 [tokens, H, 128]; may be x itself (same pointer and stride),
 *                   must not overlap gate
 *   rstd            fp32 [tokens, H] or NULL (not written)
 * tokens * H above 32 * (2^24 - 1) rows returns KDA_ERR_UNSUPPORTED.
 */
kda_status kda_gated_rmsnorm(const void* x, const void* gate, const float* weight, void* y,
                             float* rstd, const kda_norm_desc* desc, void* stream);

typedef struct kda_conv_desc {
  int32_t num_seqs;          /* prefill: N sequences (cu_seqlens has N+1); update: B rows */
  int32_t total_tokens;      /* prefill: T_total == cu_seqlens[N]; update: B * num_steps */
  int32_t num_steps;         /* update: T tokens per row (token b*T + t); prefill: unused */
  int32_t channels;          /* C, a positive multiple of 8 (3*H*128 for packed q|k|v) */
  int32_t width;             /* W taps, 1..4 */
  int32_t num_state_slots;   /* rows of the window pool */
  int32_t silu;              /* 1: y = SiLU(conv); 0: y = conv */
  int64_t x_token_stride;    /* elements between tokens of x; 0 = C */
  int64_t y_token_stride;    /* elements between tokens of y; 0 = C */
} kda_conv_desc;

/*
 * Short causal convolution of the q / k / v projections (TensorRT-LLM PR #21179,
 * fused-verify commit message; vLLM PR #55737, "Notes for review").  Depthwise, per
 * channel c:  y_t[c] = act(bias[c] + sum_{i<W} weight[c][i] * x_{t-W+1+i}[c]).
 * A window holds the W-1 inputs before a token, oldest first: bf16 [W-1, C].
 *
 * Prefill over N packed sequences:
 *   x           bf16 [T_total, C] (token-strided: e.g. the q|k|v columns of a fused
 *               projection); weight bf16 [C, W]; bias bf16 [C] or NULL
 *   conv_state  bf16 [slots, W-1, C] or NULL (zero windows, nothing written).  Sequence n
 *               starts from window state_idx[n] (row n when state_idx is NULL; zeros
 *               for an index outside [0, slots)), and that window is replaced by the
 *               one after its last token (kept when the sequence is empty).  Two
 *               sequences must not name one window.
 *   y           bf16 [T_total, C], token-strided; must not overlap x or conv_state
 * (T_total / 16 + N) * ceil(C / 2048) above 2^24 - 1 returns KDA_ERR_UNSUPPORTED.
 */
kda_status kda_causal_conv1d_prefill(const void* x, const void* weight, const void* bias,
                                     const int32_t* cu_seqlens, void* conv_state,
                                     const int32_t* state_idx, void* y,
                                     const kda_conv_desc* desc, void* stream);

/*
 * Multi-step update for verify (the packed causal_conv1d_update of TensorRT-LLM PR
 * #21179): B rows of T tokens (token b*T + t), each row starting from window
 * conv_state[state_idx[b]], which is only read.  An index outside [0, slots) marks a
 * padding row: zero outputs, its windows untouched.
 *   intermediate_window  bf16 [B, T, W-1, C]: (b, t) receives the window after token t
 *   y                    bf16 [B*T, C], token-strided
 */
kda_status kda_causal_conv1d_update(const void* x, const void* weight, const void* bias,
                                    const void* conv_state, const int32_t* state_idx,
                                    void* intermediate_window, void* y,
                                    const kda_conv_desc* desc, void* stream);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* kda_last_error(void);

/* KDA_ABI_VERSION of the loaded library. */
int kda_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
