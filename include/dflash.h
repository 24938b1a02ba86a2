/*
 * dflash.h -- C ABI of the MI355X (gfx950) DFlash block-diffusion drafter forward.
 *
 * The drafter proposes a whole block of draft tokens in one forward (Ollama
 * "mlxrunner/dflash.go", type dflashDrafter and its session).  Two halves:
 *
 *  context path   target-layer hidden taps, concatenated per row, go through
 *                 fc and hidden_norm, then every layer's K/V projection; the
 *                 row is written to the draft KV cache at its own slot S and
 *                 depends on the features at S only.  Rows are buffered and
 *                 written in one context-only forward once flush_rows (256)
 *                 accumulate.
 *  block path     the anchor token plus n = min(maxTokens, blockSize-1) mask
 *                 tokens attend over that cache; row i predicts the token at
 *                 its own position, so rows 1..n are unembedded and sampled
 *                 from one batched distribution.
 *
 * The Laguna variant (mlxcel PR "feat(speculative): add the Laguna DFlash
 * drafter") adds per-tap aux norms, a per-layer input_layernorm on context
 * rows, fused QKV, a per-head sigmoid gate and a sliding window with the
 * drop-before-fc rule; each is a dflash_config switch.
 *
 * Conventions for every call:
 *  - Device memory is allocated by the caller (PyTorch) and borrowed: weights
 *    until dflash_destroy, the session arena and the workspace until
 *    dflash_session_close.  The library itself allocates no device memory.
 *  - Device work is enqueued on the session's HIP stream (hipStream_t passed
 *    as void*) and the call returns at once; device outputs are valid after
 *    that stream is synchronized.  Host-visible integers (n, offsets, states)
 *    are exact on return.  A call that flushes two chunks or more (a long
 *    committed run) also runs every second chunk read from the caller's rows
 *    on a second stream the session opens with itself (default priority,
 *    destroyed by dflash_session_close); that stream waits for the session's
 *    stream at the start of the call and the session's stream waits for it
 *    before the call returns, so the call's work is ordered with the
 *    session's stream as if it all ran there.
 *  - Return value 0 is success; a negative DFLASH_E_* code is an error, with a
 *    thread-local message from dflash_last_error().  A call that fails leaves
 *    every session's state (offsets, pending rows, cache length, outstanding
 *    block, committed-token history) as it was before the call.  Errors found
 *    on the host (E_ARG, E_CONFIG, E_SHAPE, E_CONTEXT_GAP, E_CAPACITY) are
 *    found before any device work is enqueued.  After E_HIP (the HIP runtime
 *    refused an enqueue) the host state is put back the same way, but device
 *    work enqueued earlier in the call may have written cache rows; a
 *    windowed session's ring can then hold partial rows at visible slots, so
 *    a session that saw E_HIP should be closed.
 *  - A session is not thread-safe.  Sessions that share a workspace must issue
 *    their calls on one stream (their calls are then serialized by it).
 *  - Linear weights are row-major [out_features, in_features]; all weights of
 *    a context share one dtype (fp32 or bf16).
 */
#ifndef DFLASH_H
#define DFLASH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    DFLASH_OK = 0,
    DFLASH_E_ARG = -1,          /* null or out-of-range argument */
    DFLASH_E_CONFIG = -2,       /* configuration outside the supported bounds */
    DFLASH_E_SHAPE = -3,        /* a weight's shape disagrees with the configuration */
    DFLASH_E_CONTEXT_GAP = -4,  /* committed run starts past the frontier */
    DFLASH_E_CAPACITY = -5,     /* cache arena, workspace or output too small */
    DFLASH_E_STATE = -6,        /* call not allowed in the current state */
    DFLASH_E_HIP = -7           /* a HIP runtime call failed */
};

enum { DFLASH_FP32 = 0, DFLASH_BF16 = 1 };

typedef struct dflash_ctx dflash_ctx;
typedef struct dflash_session dflash_session;

/* Drafter configuration.  block_size and mask_id are BlockParams(); window is
 * the sliding window (0 = dense context); flush_rows is the pending bound
 * (256 in dflash.go).  Bounds checked by dflash_create (E_CONFIG):
 * block_size in [2, 512]; window 0 or in [2, 2^20]; attention_bias must be 0;
 * q_heads a multiple of kv_heads; hidden, target_hidden <= 8192; at most 16
 * layers; (q_heads/kv_heads) * block_size <= 64; bf16 needs head_dim 128 and hidden,
 * intermediate, target_hidden, q_heads*head_dim multiples of 64; fp32 needs
 * head_dim <= 64 and even. */
typedef struct {
    int32_t dtype;           /* DFLASH_FP32 or DFLASH_BF16 */
    int32_t hidden;          /* H */
    int32_t layers;          /* L, at most 16 */
    int32_t q_heads;         /* Hq */
    int32_t kv_heads;        /* Hkv */
    int32_t head_dim;        /* D */
    int32_t taps;            /* target layers tapped (5) */
    int32_t target_hidden;   /* Ht; fc input width is taps * Ht */
    int32_t vocab;           /* V */
    int32_t block_size;      /* B; a round drafts n <= B-1 rows */
    int32_t mask_id;         /* token id of the mask rows */
    int32_t window;          /* W (0: none); key s visible to query p iff p - s < W */
    int32_t intermediate;    /* MLP width I */
    int32_t causal;          /* 1: row i sees block rows j <= i; 0: all block rows */
    int32_t qk_norm;         /* per-head RMSNorm of q and k before RoPE */
    int32_t gate;            /* per-head sigmoid gate from g_proj [Hq, H] */
    int32_t aux_norms;       /* per-tap RMSNorm of the features before fc */
    int32_t ctx_input_norm;  /* context rows pass each layer's input_layernorm before K/V */
    int32_t fused_qkv;       /* one qkv_proj with rows q | k | v */
    int32_t attention_bias;  /* refused when nonzero */
    int32_t flush_rows;      /* pending bound; in [1, 4096] */
    float rope_theta;        /* RoPE base */
    float rms_eps;           /* RMSNorm epsilon */
    int32_t sel_candidates;  /* DFlash2 selector: candidates per drafted row K (0: no selector; 1..16) */
    int32_t sel_dim;         /* DFlash2 selector: width Ds of its two token tables (1..256) */
} dflash_config;

/* One weight: device pointer plus its shape (ndim 1 or 2). */
typedef struct {
    const void* data;
    int32_t ndim;
    int64_t shape[2];
} dflash_tensor;

typedef struct {
    dflash_tensor input_layernorm;           /* [H] */
    dflash_tensor post_attention_layernorm;  /* [H] */
    dflash_tensor q_proj, k_proj, v_proj;    /* [Hq*D, H], [Hkv*D, H] x2 (split) */
    dflash_tensor qkv_proj;                  /* [(Hq+2Hkv)*D, H] (fused) */
    dflash_tensor q_norm, k_norm;            /* [D] (qk_norm) */
    dflash_tensor g_proj;                    /* [Hq, H] (gate) */
    dflash_tensor o_proj;                    /* [H, Hq*D] */
    dflash_tensor gate_proj, up_proj;        /* [I, H] */
    dflash_tensor down_proj;                 /* [H, I] */
} dflash_layer_weights;

typedef struct {
    dflash_tensor embed;        /* [V, H] */
    dflash_tensor lm_head;      /* [V, H] */
    dflash_tensor fc;           /* [H, taps*Ht] */
    dflash_tensor hidden_norm;  /* [H] */
    dflash_tensor norm;         /* [H], final norm before the unembedding */
    dflash_tensor aux_norms;    /* [taps, Ht] (aux_norms) */
    const dflash_layer_weights* layers;  /* host array of `layers` entries, copied */
    dflash_tensor sel_prev;     /* [V, Ds] selector table of the predecessor (sel_candidates > 0) */
    dflash_tensor sel_next;     /* [V, Ds] selector table of the candidate (sel_candidates > 0) */
} dflash_weights;

/* Sampler settings of one dflash_sample call.  temperature 0 is greedy
 * (argmax, lowest id on an exact tie; no probabilities).  rep_penalty is the
 * CTRL repetition penalty over the distinct tokens among each session's last
 * `history` committed tokens (history <= 512). */
typedef struct {
    float temperature;
    float rep_penalty;
    int32_t history;
    int32_t round;           /* Philox counter field: one value per round */
} dflash_sample_params;

/* Selector settings of one dflash_select call (temperature only, no
 * penalties: the DFlash2 draft samples with the request's temperature). */
typedef struct {
    float temperature;       /* 0: the best-scoring candidate */
    int32_t round;           /* Philox counter field: one value per round */
} dflash_select_params;

/* Verification settings of one dflash_verify call. */
typedef struct {
    float temperature;       /* 0: greedy (argmax) verification */
    int32_t round;           /* Philox counter field: one value per round */
} dflash_verify_params;

/* Thread-local text of the last error. */
const char* dflash_last_error(void);

/* Validate the configuration and every weight shape (dflash.go
 * newDFlashDrafter / BlockParams; Laguna PR review commits: block_size 2..512,
 * windows 2..2^20, attention_bias refused, projection rows, input widths and
 * per-head norm lengths checked at load).  Errors: E_ARG, E_CONFIG, E_SHAPE. */
int dflash_create(const dflash_config* cfg, const dflash_weights* weights, dflash_ctx** out);
void dflash_destroy(dflash_ctx* ctx);

/* blockSize - 1 (dflash.go draftLimit). */
int dflash_draft_limit(const dflash_ctx* ctx);

/* Bytes of a session arena holding `capacity` cache slots, the pending
 * buffer and the committed-token history.  Dense configs need
 * capacity >= final context + block_size; windowed ones use the arena as a
 * ring and need capacity >= window + block_size - 1.  Returns 0 on a bad
 * argument. */
size_t dflash_session_bytes(const dflash_ctx* ctx, int32_t capacity);

/* Bytes of a workspace serving batched calls of up to `max_sessions`
 * sessions (1 for single-session use), two sets of context-path buffers
 * included (the two streams of a long committed run).  Returns 0 on a bad
 * argument. */
size_t dflash_workspace_bytes(const dflash_ctx* ctx, int32_t max_sessions);

/* Open a session (dflash.go open): ctxOffset = restored_offset, i.e. the
 * arena already holds cache slots [0, restored_offset) from earlier work with
 * the same context and capacity.  seed and stream_id key the sampler's
 * Philox stream.  The session also opens its second HIP stream (see the
 * conventions); if the runtime refuses one, every flush chunk runs on
 * hip_stream.  Errors: E_ARG, E_CAPACITY. */
int dflash_session_open(dflash_ctx* ctx, void* arena, size_t arena_bytes, int32_t capacity,
                        void* workspace, size_t workspace_bytes, int32_t max_sessions,
                        int32_t restored_offset, uint64_t seed, uint64_t stream_id,
                        void* hip_stream, dflash_session** out);

/* Flush pending rows (dflash.go close) and release the host-side session.
 * Returns the flush status; the session is released either way. */
int dflash_session_close(dflash_session* s);

/* A committed run (dflash.go committed): tokens_host[T] at positions
 * position..position+T-1 and their tap features features_dev, a device
 * [T, taps*Ht] array of the config dtype.  start = ctxOffset + pending -
 * position; start < 0 is E_CONTEXT_GAP (nothing changes); rows [start, T)
 * join the pending rows and their tokens the history; reaching flush_rows
 * pending rows flushes (the history tokens of a flushing run are written to
 * the device ring when a sample or a one-step commit next uses it).  Rows that stay pending are copied into the pending
 * buffer; a flushed chunk made only of this run's rows (16-byte aligned) is
 * projected where it lies by the forward this call enqueues.  Either way the
 * caller may free its buffer on return, in stream order.  Errors: E_ARG,
 * E_CONTEXT_GAP, E_CAPACITY. */
int dflash_committed(dflash_session* s, const int32_t* tokens_host, const void* features_dev,
                     int32_t T, int32_t position);

/* dflash.go flush (also settle and close): rewind an outstanding block even
 * when nothing is pending, then write every pending row in one context-only
 * forward (in chunks of at most flush_rows rows, which the context path's
 * per-row locality makes equal to one pass). */
int dflash_flush(dflash_session* s);

/* dflash_committed for `count` sessions in one call (a server commits the
 * accepted run of every session after a batched round; dflash.go committed,
 * once per session).  Session k's run is tokens_host[token_offsets[k] ..
 * token_offsets[k+1]) (host) with feature rows features_dev[k] (device,
 * [T_k, taps*Ht], config dtype) starting at positions[k].  Every run is
 * checked before anything happens: a gap (E_CONTEXT_GAP), capacity
 * (E_CAPACITY) or argument error (E_ARG: null pointers, negative lengths, a
 * session twice, sessions on different contexts or streams) leaves every
 * session unchanged.  The result equals calling dflash_committed on the
 * sessions in order; runs that stay below the flush threshold are written in
 * one or two launches for all sessions together. */
int dflash_committed_batch(dflash_session* const* sessions, int32_t count, const int32_t* tokens_host,
                           const int32_t* token_offsets, const void* const* features_dev,
                           const int32_t* positions);

/* dflash_flush over `count` sessions in one context forward (the flush of
 * dflash.go, once per session, with every session's pending rows gathered
 * into one pass as the Batch of dflash.go gathers its sequences).  Each
 * session rewinds an outstanding block, writes its pending rows to its cache
 * and advances ctxOffset past them; since a context row depends only on the
 * features at its own slot, the result equals flushing the sessions one by
 * one.  The sessions share one context, workspace and stream, count <= the
 * workspace's max_sessions, and none appears twice.  Errors (state
 * unchanged): E_ARG, E_CAPACITY. */
int dflash_flush_batch(dflash_session* const* sessions, int32_t count);

/* dflash.go commitBlock: when a block is outstanding, cut the cache back to
 * ctxOffset; otherwise nothing.  Idempotent. */
int dflash_commit_block(dflash_session* s);

/* dflash.go propose + selectBlock: n = min(max_tokens, blockSize-1); when
 * n <= 0 or no context was ever committed, *n_out = 0 and nothing changes.
 * Otherwise: rewind, write the pending rows in the same pass, schedule the
 * block [current, mask x n] at the new frontier F, run the block forward and
 * unembed rows 1..n into logits_out (device fp32 [n, V], row r predicting
 * position F+1+r).  hidden_out, when not NULL, receives the last hidden state
 * of all n+1 rows (device fp32 [n+1, H], before the final norm).  Errors:
 * E_ARG, E_CAPACITY. */
int dflash_propose(dflash_session* s, int32_t current, int32_t max_tokens, float* logits_out,
                   float* hidden_out, int32_t* n_out);

/* propose over `count` sessions in one forward (the Batch of dflash.go with
 * SeqOffsets/SeqQueryLens).  All sessions share one context, workspace and
 * stream, and count <= the workspace's max_sessions.  Rows of session k are
 * logits_out rows [row_offsets_out[k], row_offsets_out[k+1]) (host array of
 * count+1 ints); a session with nothing to propose contributes no rows. */
int dflash_propose_batch(dflash_session* const* sessions, int32_t count, const int32_t* current,
                         const int32_t* max_tokens, float* logits_out, int32_t* row_offsets_out);

/* dflash.go selectBlock's Sampler.Distribution + SampleDistribution over the
 * drafted rows: rows [row_offsets[k], row_offsets[k+1]) of logits (device fp32
 * [R, V]) belong to sessions[k]; each row's penalty set comes from that
 * session's committed history only.  ids_out: device int32 [R]; probs_out:
 * device fp32 [R, V] or NULL (ignored when greedy).  The draw of row r of
 * session k is keyed by (seed, stream_id) of the session and counter
 * (t div 8, r - row_offsets[k], round, 0): word (t mod 8) div 2, bits 63..41
 * for even t and 40..18 for odd t.  Errors: E_ARG. */
int dflash_sample(dflash_session* const* sessions, int32_t count, const int32_t* row_offsets,
                  const float* logits, const dflash_sample_params* params, int32_t* ids_out,
                  float* probs_out);

/* DFlash2 candidate selector (Ollama dflash.go selectBlock, BlockSelector
 * branch; DFlash2 commit note: the selector proposes each token conditioned
 * on its predecessor and returns each position's candidate distribution,
 * which verification uses to keep the output exact).  Rows [row_offsets[k],
 * row_offsets[k+1]) of logits (device fp32 [R, V], as dflash_propose returns
 * them) are session k's drafted rows 1..n_k and current[k] (host) its anchor.
 * Position i's candidates are the K = sel_candidates highest logits of its
 * row (ties to the lower id), ranked by logit (a NaN logit counts as -inf,
 * and a row with fewer than K finite logits is filled with the lowest ids
 * among the rest: they score -inf and get probability 0); candidate c scores
 * s_i(c) = z_i(c) + <sel_prev[t_{i-1}], sel_next[c]> with t_0 the anchor and
 * t_{i-1} the token chosen at position i-1 (so the positions are chosen in
 * order); the position's distribution is softmax over its candidates of
 * s_i / T, and the token is the Gumbel-max draw (u of candidate rank j: top
 * 23 bits of word j mod 4 of Philox4x64-10 at counter (j div 4, i, round, 3)
 * under the session's (seed, stream_id), plus 1/2, times 2^-23), or the best
 * score when T = 0 (the lower rank on a tie).  Outputs (device): tokens_out
 * int32 [R]; cand_ids_out int32 [R, K]; cand_probs_out fp32 [R, K] (T > 0;
 * may be NULL); dense_probs_out fp32 [R, V] or NULL: the candidate
 * distribution as full rows, zero off the candidates, in the form
 * dflash_verify takes as draft probabilities (T > 0).  Session state is not
 * touched.  Sessions share context, workspace and stream.  Errors: E_ARG,
 * E_STATE (the drafter has no selector), E_CAPACITY. */
int dflash_select(dflash_session* const* sessions, int32_t count, const int32_t* row_offsets, const float* logits,
                  const int32_t* current, const dflash_select_params* params, int32_t* tokens_out,
                  int32_t* cand_ids_out, float* cand_probs_out, float* dense_probs_out);

/* Speculative verification of drafted blocks against the target's logits
 * (the round loop's check of a draft; Ollama dflash.go propose: verification
 * uses each position's actual proposal distribution to keep the output exact;
 * mlxcel Laguna PR review: the greedy round loop verifies by a raw
 * per-position argmax).  Session k drafted n_k = draft_offsets[k+1] -
 * draft_offsets[k] tokens (0 <= n_k <= blockSize-1), draft_ids[draft_offsets[k]
 * + i] for i < n_k, and supplies n_k + 1 target rows from row
 * draft_offsets[k] + k of target_logits (device fp32 [draft_offsets[count] +
 * count, V]): row i scores the token after block position i, row n_k is the
 * bonus position.
 *   temperature 0: accepted_k = the number of leading drafts equal to their
 *     row's argmax (lowest id on a tie); next_k = the argmax of row accepted_k.
 *   temperature T > 0 (speculative sampling): with p_i = softmax(row i / T) and
 *     q_i = draft_probs row draft_offsets[k] + i (device fp32 [rows, V], the
 *     distribution draft i was drawn from, as dflash_sample returns it), draft
 *     i is accepted while u_i * q_i(x_i) <= p_i(x_i); at the first rejection,
 *     row a, next_k is drawn from max(0, p_a - q_a) renormalised, and after n_k
 *     acceptances from p_{n_k}.  Every emitted token is then an exact draw from
 *     the target.  Draws are keyed by the session's (seed, stream_id):
 *     u_i from Philox4x64-10 counter (0, i, round, 1), the draw from row a by
 *     Gumbel-max with counter (t div 4, a, round, 2).
 * A draft id outside [0, V) is never accepted (greedy or not; nothing is read
 * at it) and next_k is drawn at its row as after any rejection.
 * accepted_out and next_out are device int32 [count].  The session state is
 * not touched (commit the accepted run with dflash_committed).  Sessions
 * share context, workspace and stream.  Errors: E_ARG. */
int dflash_verify(dflash_session* const* sessions, int32_t count, const int32_t* draft_offsets,
                  const float* target_logits, const int32_t* draft_ids, const float* draft_probs,
                  const dflash_verify_params* params, int32_t* accepted_out, int32_t* next_out);

/* dflash_verify for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same arguments, results and errors, but the verification's tables and
 * statistics live in a static 4 MiB device array of the library (one per
 * GPU, held until the process ends) instead of the sessions' workspace, so
 * the sessions need not share one.  The call allocates nothing.  It needs
 * 32 bytes per target row and 4096-token vocabulary chunk (2 KiB per row at
 * a 262144-token vocabulary: up to about 2000 target rows) plus its tables;
 * a call needing more fails with E_CAPACITY and does nothing.  Every call on one GPU uses the same array: calls that overlap on
 * one GPU (on different streams, or from several threads) race and must be
 * ordered by the caller. */
int dflash_verify_noalloc(dflash_session* const* sessions, int32_t count, const int32_t* draft_offsets,
                          const float* target_logits, const int32_t* draft_ids, const float* draft_probs,
                          const dflash_verify_params* params, int32_t* accepted_out, int32_t* next_out);

/* Draft width controller (host only).  The pages: DFlash2 drafts a fixed
 * seven tokens per round instead of following Ollama's depth controller, whose
 * shallower picks lose more accepted tokens than they save in verify time.
 * This controller makes that trade explicit: it keeps, per draft position i,
 * a decayed estimate of P(draft i accepted | drafts before it accepted)
 * (prior 1/2), and picks the width n in [1, max_width] that maximises the
 * expected tokens a round emits, 1 + sum_{j<=n} prod_{i<=j} alpha_i (accepted
 * drafts plus the correction or bonus token), per unit of round time
 * draft_fixed + draft_per_row * n + verify_fixed + verify_per_row * (n + 1)
 * (any time unit; bench.py measures the draft terms).  decay in (0, 1]
 * weights past rounds.  Errors: E_ARG. */
typedef struct dflash_width_policy dflash_width_policy;
int dflash_width_policy_create(int32_t max_width, float draft_fixed, float draft_per_row, float verify_fixed,
                               float verify_per_row, float decay, dflash_width_policy** out);
/* One round: `drafted` tokens were proposed and `accepted` of them accepted. */
int dflash_width_policy_observe(dflash_width_policy* p, int32_t drafted, int32_t accepted);
/* The width to draft next (>= 1), or a negative error code. */
int dflash_width_policy_choose(const dflash_width_policy* p);
/* Current acceptance estimates alpha_1..alpha_max_width into out[max_width]. */
int dflash_width_policy_rates(const dflash_width_policy* p, float* out);
void dflash_width_policy_destroy(dflash_width_policy* p);

/* Host-side state: ctxOffset, pending rows, cache length (Offset()), block
 * outstanding flag, and the number of context rows projected so far. */
int dflash_session_state(const dflash_session* s, int32_t* ctx_offset, int32_t* pending,
                         int32_t* cache_len, int32_t* outstanding, int64_t* rows_written);

/* Read `count` cache entries of `layer` starting at absolute position
 * position0 (within [0, cache_len), and for windowed configs within the last
 * capacity positions) into device fp32 k_out / v_out [count, Hkv, D]. */
int dflash_cache_read(const dflash_session* s, int32_t layer, int32_t position0, int32_t count,
                      float* k_out, float* v_out);

/* Kernel timing (tracing): while enabled, every launch of the named stage is
 * bracketed by HIP events on the stream it runs on.  Stages: "unembed" (the
 * lm_head GEMM), "attention" (partials + combine), "attention_partial" (the
 * partials kernel alone, bf16), "flush_fc" and "flush_kv" (the context-path
 * GEMMs), "layer_gemms" (the block path's per-layer projections: q|k|v(|g),
 * o_proj, gate|up, down), "sampler", "verify" (one pair per dflash_verify),
 * "select" (one pair per dflash_select).
 * dflash_profile_end waits for the
 * recorded events and returns the summed kernel time (ms) and the number of
 * launches since dflash_profile_begin.  Errors: E_ARG (unknown stage),
 * E_HIP. */
int dflash_profile_begin(dflash_ctx* ctx, const char* stage);
int dflash_profile_end(dflash_ctx* ctx, double* total_ms, int32_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* DFLASH_H */
