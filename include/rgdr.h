/*
 * rgdr.h -- C ABI of the gfx950 (MI355X) gated-delta-rule decode library.
 *
 * Three operations:
 *
 *   rgdr_decode  The recurrent gated-delta-rule decode step of the MindSpore Lite API page
 *                "lite_boost.ops.recurrent_gated_delta_rule" (algorithm section, parameter
 *                list, returns, notes). For every batch entry b, every value head h and
 *                every valid token t, in token order, on the state S (D_k rows = key
 *                dimension, D_v columns = value dimension):
 *                  1. decay   S = S * exp(g[t]) * exp(gk[t][i])        (row i scaled)
 *                  2. read    kv = S^T k_t
 *                  3. update  S = S + k_t (x) ((v_t - kv) * beta[t])   (outer product)
 *                  4. output  o_t = S^T (q_t * scale)
 *                rgdr_decode_snapshots (and rgdr_decode_gated_snapshots, with the gate
 *                fused in) also store S after every token.
 *   rgdr_prefill The same recurrence over long sequences (T up to 65536): the page's notes
 *                limit the decode operator to T <= 8 and hand the parallel prefill to a
 *                chunk-level operator; this is that operator, with rgdr_decode's arguments.
 *                rgdr_prefill_ws (and rgdr_prefill_gated_ws) take a caller's workspace, with
 *                which calls of few sequences run all of a sequence's segments at once.
 *   la_gate      The gate front end of the kernel README "com.microsoft.LinearAttentionGate"
 *                (Description; Inputs, Outputs, Type constraints tables):
 *                  decay = decay_scale[h] * softplus(a + dt_bias[h]),  beta = sigmoid(b),
 *                computed in fp32 and narrowed only on store.
 *
 * Conventions for every call:
 *   - All tensor pointers are DEVICE pointers to row-major, contiguous buffers owned by
 *     the caller. The library allocates nothing and keeps no pointer after returning; a
 *     call that needs scratch memory takes it as a workspace argument, except
 *     rgdr_prefill_noalloc, which uses a fixed device array inside the library.
 *   - Calls are asynchronous on `stream` (0 = the null stream). The return value reports
 *     only errors that the host can see before launching (arguments, shapes, alignment,
 *     a failed launch); when it is not RGDR_OK nothing was launched.
 *   - bf16 is the 16-bit brain float (1 sign, 8 exponent, 7 fraction bits); outputs are
 *     rounded to it with round-to-nearest-even. Arithmetic is fp32.
 *   - Environment: RGDR_HOLD_READ_GBPS (a number, GB/s; 0 = off) sets the HBM read rate
 *     that single-token (T = 1) decode calls assume when they delay their state write-back
 *     until the call's reads could have completed. It is read once, at the process's first
 *     single-token call, and changes timing only, never results. Unset: the built-in rate
 *     for MI355X (6400).
 */
#ifndef RGDR_H
#define RGDR_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    RGDR_OK = 0,
    RGDR_ERR_NULL = 1,        /* a required pointer is NULL                                */
    RGDR_ERR_SHAPE = 2,       /* a size is negative, or zero where not allowed; T > 8
                                 (decode) or T > 65536 (prefill); H_v % H_q != 0; grid too
                                 large; beta requested without b                          */
    RGDR_ERR_UNSUPPORTED = 3, /* D_k not in {64, 128}, D_v not a multiple of 64 or above
                                 4096, or an unknown option bit                             */
    RGDR_ERR_RANGE = 4,       /* (validate) a length, count or slot index out of range     */
    RGDR_ERR_DUPLICATE = 5,   /* (validate) two batch entries name the same slot           */
    RGDR_ERR_DTYPE = 6,       /* a dtype code not allowed for that argument                 */
    RGDR_ERR_HIP = 7,         /* a HIP runtime call failed                                  */
    RGDR_ERR_ALIGN = 8,       /* a pointer is not aligned as its argument requires          */
    RGDR_ERR_SCRATCH = 9      /* (rgdr_prefill_noalloc) the call needs more scratch memory
                                 than the library's fixed array holds                       */
} rgdr_status;

typedef enum { RGDR_F32 = 0, RGDR_F16 = 1, RGDR_BF16 = 2 } rgdr_dtype;

/* Option bits of rgdr_decode_gated. */
enum { RGDR_NORMALIZE_QK = 1u /* L2-normalise each token's query and key head vector */ };

/*
 * rgdr_decode -- one decode step over a batch (MindSpore Lite page above; arguments keep
 * the page's names and meaning).
 *
 *   query               bf16 [B, H_q, T, D_k]  L2-normalised per head vector (caller's
 *                       precondition, not checked). 16-byte aligned.
 *   key                 bf16 [B, H_q, T, D_k]  as query (16-byte aligned). Value head h reads query/key head
 *                       h / (H_v / H_q), i.e. floor(h * H_q / H_v).
 *   value               bf16 [B, H_v, T, D_v]  16-byte aligned.
 *   beta                bf16 [B, H_v, T]       delta step size, in (0, 1) (not checked).
 *   state_pool          bf16 [N_slots, H_v, D_k, D_v]  the recurrent states; entry b uses
 *                       slot ssm_state_indices[b]. 16-byte aligned.
 *   actual_seq_lengths  int32 [B]  valid tokens L of entry b. Tokens t >= L are never read
 *                       and their out rows are written as +0.0. Values outside [0, T] act
 *                       as clamped to [0, T].
 *   ssm_state_indices   int32 [B]  slot of entry b. Must be distinct (two entries naming one
 *                       slot race). An index outside [0, N_slots) skips the entry: its out
 *                       rows are +0.0 and no state is read or written.
 *   g                   fp32 [B, H_v, T]        global log-decay, negative (not checked).
 *   gk                  fp32 [B, H_v, T, D_k]   per-key-dimension log-decay, negative.
 *                       16-byte aligned.
 *   num_accepted_tokens int32 [B]  n: the state committed for entry b is the state after
 *                       its first n tokens (clamped to [0, L]); n = L in ordinary decoding.
 *   scale               q is multiplied by it before step 4 (the page's scale_value).
 *   B, H_q, H_v, T, D_k, D_v, N_slots   sizes; T <= 8 (decode only), H_v % H_q == 0,
 *                       D_k in {64, 128}, D_v a multiple of 64 and at most 4096.
 *                       B = 0 is an empty batch: RGDR_OK, nothing is read or launched.
 *   out                 bf16 [B, H_v, T, D_v]  written entirely. 16-byte aligned.
 *   state_out           bf16 [N_slots, H_v, D_k, D_v]  receives the committed state of every
 *                       slot some entry names; other slots are not touched. It may be the
 *                       same buffer as state_pool (in-place update); any other overlap is
 *                       undefined. 16-byte aligned.
 *   stream              HIP stream the kernel is enqueued on.
 * Errors: RGDR_ERR_NULL, RGDR_ERR_SHAPE, RGDR_ERR_UNSUPPORTED, RGDR_ERR_ALIGN,
 * RGDR_ERR_HIP (launch failure). Device-side data (lengths, indices) never causes an
 * out-of-bounds access; rgdr_validate reports bad values.
 */
rgdr_status rgdr_decode(const void *query, const void *key, const void *value,
                        const void *beta, const void *state_pool,
                        const int32_t *actual_seq_lengths, const int32_t *ssm_state_indices,
                        const float *g, const float *gk, const int32_t *num_accepted_tokens,
                        float scale, int32_t B, int32_t H_q, int32_t H_v, int32_t T,
                        int32_t D_k, int32_t D_v, int32_t N_slots, void *out,
                        void *state_out, hipStream_t stream);

/*
 * rgdr_decode_snapshots -- rgdr_decode that also stores the state after every token.
 * The page's num_accepted_tokens parameter serves speculative decoding: a step evaluates
 * T drafted tokens and commits the state after the accepted prefix. A caller that learns
 * the accepted count only after the step needs the state after each candidate prefix;
 * this call writes all of them in the same pass.
 *
 *   state_snapshots  bf16 [B, T, H_v, D_k, D_v], 16-byte aligned, owned by the caller.
 *                    Entry (b, t, h) receives the state of value head h of batch entry b
 *                    after its first t + 1 tokens (after step 3 of token t), rounded as the
 *                    committed state is, for every t below the clamped length L of entry b
 *                    whose slot is valid. Other entries (t >= L, skipped entries) are not
 *                    written. With n = num_accepted_tokens[b] >= 1, entry (b, n - 1) holds
 *                    the same bytes as the committed slot.
 *   All other arguments, results and errors: as rgdr_decode (RGDR_ERR_NULL also for
 *   state_snapshots, RGDR_ERR_ALIGN for its alignment). The snapshots add D_k * D_v * 2
 *   bytes of HBM writes per written entry and value head (at most B * T * H_v * D_k * D_v * 2
 *   in all).
 */
rgdr_status rgdr_decode_snapshots(const void *query, const void *key, const void *value,
                                  const void *beta, const void *state_pool,
                                  const int32_t *actual_seq_lengths,
                                  const int32_t *ssm_state_indices, const float *g,
                                  const float *gk, const int32_t *num_accepted_tokens,
                                  float scale, int32_t B, int32_t H_q, int32_t H_v, int32_t T,
                                  int32_t D_k, int32_t D_v, int32_t N_slots, void *out,
                                  void *state_out, void *state_snapshots, hipStream_t stream);

/*
 * rgdr_decode_gated -- rgdr_decode with the gate front end fused in: instead of g and beta,
 * it takes the raw gate projections of the "com.microsoft.LinearAttentionGate" README and
 * computes, per token and value head, in fp32 and without storing them,
 *   g    = decay_scale[h] * softplus(gate_a[b, t, h] + dt_bias[h]),
 *   beta = sigmoid(gate_b[b, t, h]),
 * then runs the same four steps as rgdr_decode on them.
 *
 *   gate_a, gate_b  [B, T, H_v] (the README's head-axis-last layout) of gate_dtype, RGDR_F32
 *                   or RGDR_F16; element-aligned. Entries of padded tokens are not read.
 *   dt_bias, decay_scale  fp32 [H_v].
 *   All other arguments: as rgdr_decode (g and beta are not taken).
 * Unlike rgdr_decode fed by la_gate, beta is not rounded to bf16 in between.
 *
 *   flags  0, or RGDR_NORMALIZE_QK: establish the operator's unit-norm precondition on
 *          query and key (MindSpore Lite page, parameters query and key) in the kernel:
 *          each token's q and k head vector is divided by its L2 norm over D_k (fp32 sum
 *          of squares, reciprocal square root) before the four steps and before the scale;
 *          an all-zero vector stays zero. The inputs are not modified.
 * Errors: as rgdr_decode, plus RGDR_ERR_DTYPE for another gate_dtype and
 * RGDR_ERR_UNSUPPORTED for an unknown flag bit.
 */
rgdr_status rgdr_decode_gated(const void *query, const void *key, const void *value,
                              const void *gate_a, const void *gate_b, const float *dt_bias,
                              const float *decay_scale, rgdr_dtype gate_dtype,
                              const void *state_pool, const int32_t *actual_seq_lengths,
                              const int32_t *ssm_state_indices, const float *gk,
                              const int32_t *num_accepted_tokens, float scale, int32_t B,
                              int32_t H_q, int32_t H_v, int32_t T, int32_t D_k, int32_t D_v,
                              int32_t N_slots, void *out, void *state_out, uint32_t flags,
                              hipStream_t stream);

/*
 * rgdr_decode_gated_snapshots -- rgdr_decode_gated that also stores the state after every
 * token, as rgdr_decode_snapshots extends rgdr_decode (the same speculative-decoding use of
 * the page's num_accepted_tokens, with the gate computed in the kernel).
 *
 *   state_snapshots  bf16 [B, T, H_v, D_k, D_v], 16-byte aligned, owned by the caller;
 *                    written exactly as by rgdr_decode_snapshots.
 *   All other arguments, results and errors: as rgdr_decode_gated (RGDR_ERR_NULL also for
 *   state_snapshots, RGDR_ERR_ALIGN for its alignment).
 */
rgdr_status rgdr_decode_gated_snapshots(const void *query, const void *key, const void *value,
                                        const void *gate_a, const void *gate_b,
                                        const float *dt_bias, const float *decay_scale,
                                        rgdr_dtype gate_dtype, const void *state_pool,
                                        const int32_t *actual_seq_lengths,
                                        const int32_t *ssm_state_indices, const float *gk,
                                        const int32_t *num_accepted_tokens, float scale,
                                        int32_t B, int32_t H_q, int32_t H_v, int32_t T,
                                        int32_t D_k, int32_t D_v, int32_t N_slots, void *out,
                                        void *state_out, void *state_snapshots, uint32_t flags,
                                        hipStream_t stream);

/*
 * rgdr_prefill -- the recurrence of rgdr_decode over a long sequence per batch entry
 * (MindSpore Lite page above, notes: the prefill counterpart, a chunk-level operator, of the
 * T <= 8 decode operator). Arguments, layouts, ownership and semantics are rgdr_decode's
 * (state pool and slots, valid lengths with +0.0 padded rows, accepted counts, head
 * sharing, in-place update), with one difference:
 *   T  1 <= T <= 65536 (the padded sequence length), and T * H_v <= 2^29.
 * The state is read once and kept in fp32 across all of an entry's tokens; it is rounded to
 * bf16 once, when it is committed after the entry's first num_accepted_tokens tokens.
 * Tokens are evaluated in chunks of at most 32 in the exact closed form of the recurrence,
 * whose dense products run on the matrix cores with operands split into bf16 high parts and
 * remainders (about 16 bits of each operand, fp32 accumulation); a chunk whose decay
 * products span more than 2^192 is shortened. That costs time and moves rounding, since
 * chunk boundaries group the arithmetic, but leaves the precision unchanged.
 * Errors: as rgdr_decode (RGDR_ERR_SHAPE for T > 65536 or T * H_v > 2^29).
 */
rgdr_status rgdr_prefill(const void *query, const void *key, const void *value,
                         const void *beta, const void *state_pool,
                         const int32_t *actual_seq_lengths, const int32_t *ssm_state_indices,
                         const float *g, const float *gk, const int32_t *num_accepted_tokens,
                         float scale, int32_t B, int32_t H_q, int32_t H_v, int32_t T,
                         int32_t D_k, int32_t D_v, int32_t N_slots, void *out,
                         void *state_out, hipStream_t stream);

/*
 * rgdr_prefill_gated -- rgdr_prefill with the gate front end fused in, exactly as
 * rgdr_decode_gated extends rgdr_decode: raw gate projections gate_a, gate_b [B, T, H_v]
 * (RGDR_F32 or RGDR_F16) and fp32 dt_bias, decay_scale [H_v] instead of g and beta, and the
 * RGDR_NORMALIZE_QK option. Sizes and errors as rgdr_prefill, plus rgdr_decode_gated's.
 */
rgdr_status rgdr_prefill_gated(const void *query, const void *key, const void *value,
                               const void *gate_a, const void *gate_b, const float *dt_bias,
                               const float *decay_scale, rgdr_dtype gate_dtype,
                               const void *state_pool, const int32_t *actual_seq_lengths,
                               const int32_t *ssm_state_indices, const float *gk,
                               const int32_t *num_accepted_tokens, float scale, int32_t B,
                               int32_t H_q, int32_t H_v, int32_t T, int32_t D_k, int32_t D_v,
                               int32_t N_slots, void *out, void *state_out, uint32_t flags,
                               hipStream_t stream);

/*
 * rgdr_prefill_workspace_size -- the workspace rgdr_prefill_ws and rgdr_prefill_gated_ws
 * use for a call of these sizes on the current device: *bytes = 0 when such a call runs in
 * one pass (it then needs none). Sizes as rgdr_prefill; H_q does not matter.
 * Errors: RGDR_ERR_NULL (bytes NULL), RGDR_ERR_SHAPE, RGDR_ERR_UNSUPPORTED as rgdr_prefill;
 * RGDR_ERR_HIP if the device cannot be queried.
 */
rgdr_status rgdr_prefill_workspace_size(int32_t B, int32_t H_v, int32_t T, int32_t D_k,
                                        int32_t D_v, size_t *bytes);

/*
 * rgdr_prefill_ws -- rgdr_prefill (same arguments, results and errors) with a workspace.
 * The recurrence maps each segment of tokens affinely: a segment takes its incoming state S
 * to Phi S + Psi, where Psi is its end state from a zero state and Phi (D_k x D_k) is the
 * product of its tokens' factors (I - beta_t k_t k_t^T) diag(exp(g_t) exp(gk_t)) (MindSpore
 * Lite page above, algorithm section: steps 1 and 3 are linear in S, with v entering only
 * through Psi). Where a call has too few (entry, value head) pairs to fill the device, the
 * entries' tokens are cut into segments (at num_accepted_tokens too), every segment's Phi
 * and Psi are evaluated at once, a short sequential scan composes them in fp32 into each
 * segment's incoming state and commits the state after the accepted prefix, and every
 * segment then produces its outputs from its incoming state at once.
 *   workspace        device memory of at least rgdr_prefill_workspace_size's bytes, 256-byte
 *                    aligned, owned by the caller, not read before it is written; the call
 *                    uses it until it completes on `stream`. Calls that share a workspace
 *                    must be ordered (the same stream, or synchronised).
 *   workspace_bytes  its size.
 * With workspace NULL, or smaller than the size query, or where the size query gives 0, the
 * call runs rgdr_prefill's single pass. Both forms hold the same precision (fp32 state,
 * products of split bf16 operands); their rounding differs, since the segmented form
 * groups the arithmetic by segment.
 */
rgdr_status rgdr_prefill_ws(const void *query, const void *key, const void *value,
                            const void *beta, const void *state_pool,
                            const int32_t *actual_seq_lengths, const int32_t *ssm_state_indices,
                            const float *g, const float *gk, const int32_t *num_accepted_tokens,
                            float scale, int32_t B, int32_t H_q, int32_t H_v, int32_t T,
                            int32_t D_k, int32_t D_v, int32_t N_slots, void *out,
                            void *state_out, void *workspace, size_t workspace_bytes,
                            hipStream_t stream);

/*
 * rgdr_prefill_gated_ws -- rgdr_prefill_gated with a workspace, as rgdr_prefill_ws extends
 * rgdr_prefill.
 */
rgdr_status rgdr_prefill_gated_ws(const void *query, const void *key, const void *value,
                                  const void *gate_a, const void *gate_b, const float *dt_bias,
                                  const float *decay_scale, rgdr_dtype gate_dtype,
                                  const void *state_pool, const int32_t *actual_seq_lengths,
                                  const int32_t *ssm_state_indices, const float *gk,
                                  const int32_t *num_accepted_tokens, float scale, int32_t B,
                                  int32_t H_q, int32_t H_v, int32_t T, int32_t D_k,
                                  int32_t D_v, int32_t N_slots, void *out, void *state_out,
                                  uint32_t flags, void *workspace, size_t workspace_bytes,
                                  hipStream_t stream);

/*
 * rgdr_prefill_noalloc -- rgdr_prefill_ws for callers that cannot allocate device memory
 * (code under HIP graph capture, serving loops, harnesses that forbid hipMalloc): the same
 * arguments as rgdr_prefill, results as rgdr_prefill_ws with a workspace of 128 MiB. The
 * workspace is a fixed device array inside the library (128 MiB on every device the library
 * runs on, held until the process ends); the call allocates nothing. The segmented form's
 * workspace is written before it is read, so nothing in it needs clearing between calls.
 * Every call on one device uses the same array: calls that may overlap on one device (other
 * streams, other threads) race and must be ordered by the caller.
 * Errors: as rgdr_prefill; RGDR_ERR_SCRATCH where the segmented form would need more than
 * 128 MiB (no call of the library's current segment plan does: its largest takes
 * 108 MiB); RGDR_ERR_HIP if the array's device address cannot be looked up.
 */
rgdr_status rgdr_prefill_noalloc(const void *query, const void *key, const void *value,
                                 const void *beta, const void *state_pool,
                                 const int32_t *actual_seq_lengths,
                                 const int32_t *ssm_state_indices, const float *g,
                                 const float *gk, const int32_t *num_accepted_tokens,
                                 float scale, int32_t B, int32_t H_q, int32_t H_v, int32_t T,
                                 int32_t D_k, int32_t D_v, int32_t N_slots, void *out,
                                 void *state_out, hipStream_t stream);

/*
 * la_gate -- decay = decay_scale * softplus(a + dt_bias) and, when beta_out != NULL,
 * beta = sigmoid(b) ("com.microsoft.LinearAttentionGate" README, Description and tables).
 *
 *   a            [n_rows, H] of ab_dtype: the decay projection; any rank >= 1 with the head
 *                axis last, leading axes folded into n_rows.
 *   dt_bias      fp32 [H]  per-head bias added to a.
 *   decay_scale  fp32 [H]  per-head multiplier; for gated DeltaNet it is -exp(A_log).
 *   b            [n_rows, H] of ab_dtype: the update-rate projection. Required when
 *                beta_out != NULL; may be given (and is then unused) when it is NULL.
 *   ab_dtype     RGDR_F32 or RGDR_F16 (the README's T).
 *   n_rows, H    sizes; n_rows >= 0, H >= 1. n_rows = 0 returns RGDR_OK without reading
 *                any pointer or launching.
 *   decay_out    [n_rows, H] of decay_dtype (RGDR_F32 or RGDR_F16).
 *   beta_out     [n_rows, H] of beta_dtype (RGDR_F32, RGDR_F16, or RGDR_BF16 so that it can
 *                feed rgdr_decode's beta directly), or NULL.
 * Arithmetic is fp32 (precise expf/log1pf); values are narrowed once, on store, with
 * round-to-nearest-even. With T = 1, the gate's [B, 1, H] layout is the [B, H, 1] layout
 * rgdr_decode reads for g and beta.
 * Errors: RGDR_ERR_NULL, RGDR_ERR_SHAPE (also beta_out without b), RGDR_ERR_DTYPE,
 * RGDR_ERR_ALIGN (element alignment), RGDR_ERR_HIP.
 */
rgdr_status la_gate(const void *a, const float *dt_bias, const float *decay_scale,
                    const void *b, rgdr_dtype ab_dtype, int64_t n_rows, int32_t H,
                    void *decay_out, rgdr_dtype decay_dtype, void *beta_out,
                    rgdr_dtype beta_dtype, hipStream_t stream);

/*
 * rgdr_validate_host -- checks the index arrays of one rgdr_decode call, given as HOST
 * pointers: every length in [0, T], every accepted count in [0, length], every slot index
 * in [0, N_slots), no slot named twice. Returns RGDR_OK, RGDR_ERR_RANGE,
 * RGDR_ERR_DUPLICATE, RGDR_ERR_NULL or RGDR_ERR_SHAPE. Pure host code.
 */
rgdr_status rgdr_validate_host(const int32_t *actual_seq_lengths,
                               const int32_t *ssm_state_indices,
                               const int32_t *num_accepted_tokens, int32_t B, int32_t T,
                               int32_t N_slots);

/*
 * rgdr_validate -- the same checks for DEVICE pointers: copies the 3 x B int32 values to
 * the host on `stream` and waits for that stream (synchronous; not for the hot path).
 */
rgdr_status rgdr_validate(const int32_t *actual_seq_lengths, const int32_t *ssm_state_indices,
                          const int32_t *num_accepted_tokens, int32_t B, int32_t T,
                          int32_t N_slots, hipStream_t stream);

/* A static, human-readable name for a status code. */
const char *rgdr_status_string(rgdr_status s);

#ifdef __cplusplus
}
#endif

#endif /* RGDR_H */
