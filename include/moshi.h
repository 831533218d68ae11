/*
 * moshi.h -- C ABI of the MI355X Moshi/PersonaPlex frame-step library
 * (libmoshi.so).
 *
 * One call of moshi_step() advances every live session slot by one 80 ms
 * frame: one 17-row token column in (text, 8 agent codes, 8 user codes), one
 * text token and 16 audio codes out ("vLLM-Omni recipe: PersonaPlex", sections
 * "Why it is different" and "Architecture"). Sessions join and leave between
 * steps without disturbing the others ("When to use this recipe"; "Notes":
 * joins beyond the capacity are refused, a recycled slot behaves like a fresh
 * engine).
 *
 * Conventions shared by every entry point:
 *  - Every call returns an int status: MOSHI_OK (0) or a negative MOSHI_E_*.
 *    On any error nothing observable changes (no session state moves), except
 *    that a device failure makes the context sticky-failed (every later call
 *    returns MOSHI_E_DEVICE).
 *  - All pointers in the signatures are HOST pointers owned by the caller; the
 *    library copies what it needs before returning. The library owns all
 *    device memory and the context.
 *  - A context is not thread-safe: use one thread per context.
 *  - B below is the capacity `max_sessions` fixed at creation; per-slot arrays
 *    have B rows indexed by slot. Rows of slots that are not live are ignored
 *    on input and written as -1 on output.
 */
#ifndef MOSHI_H
#define MOSHI_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct moshi_ctx moshi_ctx;

enum {
  MOSHI_OK = 0,
  MOSHI_E_INVALID = -1,   /* bad argument, config or code; nothing changed */
  MOSHI_E_FULL = -2,      /* join with every slot taken */
  MOSHI_E_NOSESSION = -3, /* slot out of range or not live */
  MOSHI_E_DEVICE = -4,    /* HIP error; the context is now unusable */
  MOSHI_E_OOM = -5        /* device allocation failed at creation */
};

enum { MOSHI_F32 = 0, MOSHI_BF16 = 1 };

/* Reading flags (create-time; default off).
 * MOSHI_FLAG_MASK_OLDEST: once a session's ring is full, also mask the oldest
 *   key (W-1 keys attended instead of W) -- SGLang-Omni cookbook
 *   "PersonaPlex", "Known limitations": the temporal window follows the
 *   streaming ring, including the masked oldest slot once the cache fills.
 * MOSHI_FLAG_DEP_FINAL_NORM: each depformer head reads RMSNorm(y) times one
 *   more gain tensor (dep.out_norm [Dd], appended after the heads) instead of
 *   the residual y itself -- the other reading of where the depformer's
 *   norms stop (mobius PR #368, "P2 - Moshi LM", names pre-norm layers and
 *   no final depformer norm).
 * MOSHI_FLAG_DEP_REF_RING: the substep K/V behaves as a ring whose capacity
 *   is the number of substeps run; at the last substep, once it is full,
 *   entry 0 is masked -- cookbook "Reference parity": the last depformer step
 *   matches the reference only with its ring behaviour emulated. */
#define MOSHI_FLAG_MASK_OLDEST 1u
#define MOSHI_FLAG_DEP_FINAL_NORM 2u
#define MOSHI_FLAG_DEP_REF_RING 4u
/* MOSHI_FLAG_SAMPLING: the context can draw tokens by temperature + top-k
 *   (moshi_session_set_sampling; vocabularies up to 32768). Without it every
 *   head is greedy. Contexts with it run one kernel per operation (the
 *   capacity-1 step kernel is greedy only). */
#define MOSHI_FLAG_SAMPLING 8u

/* Model shape and engine capacity.
 * Temporal transformer: `dim`, `n_layers`, `n_heads` (head_dim = dim/n_heads
 * must be 32, 64 or 128; the same holds for the depformer), SwiGLU width
 * `ffn_hidden`, ring window `window` frames (mobius PR #368, "P2 - Moshi LM";
 * recipe "Architecture": 4096-d, 32 layers, 32 heads, window 3000).
 * Depformer: `dep_dim`, `dep_layers`, `dep_heads`, `dep_ffn_hidden`,
 * `n_substeps` substeps (1024-d, 6 layers, 16 heads, 16 substeps).
 * Vocabularies: `text_vocab` (32000), `audio_card` (2048); the token column
 * has 1 + n_substeps rows and every embedding table has card+1 rows.
 * `dtype` MOSHI_BF16 or MOSHI_F32 (weights, K/V and linear inputs);
 * `max_sessions` = capacity B (1..64), fixed for the life of the context.
 * `flags`: MOSHI_FLAG_* above. `dep_q`: depformer substeps run per frame,
 * 1..n_substeps, 0 = all (the cookbook's "Known limitations" runs 8: the
 * agent's codebooks; the recipe's "Architecture": 16 codebooks, 8 vocoded);
 * codes of substeps not run are returned as -1.
 * Every width (dim, ffn_hidden, dep_dim, dep_ffn_hidden) must be a multiple of
 * 8 (bf16) or 4 (fp32). */
typedef struct {
  int32_t dim, n_layers, n_heads, ffn_hidden, window;
  int32_t dep_dim, dep_layers, dep_heads, dep_ffn_hidden, n_substeps;
  int32_t text_vocab, audio_card;
  double rope_theta, norm_eps;
  int32_t dtype, max_sessions;
  uint32_t flags;
  int32_t dep_q;
} moshi_config;

/* Number of weight tensors moshi_create expects for this config (< 0 on a bad
 * config); the list is in moshi_create's comment. */
int32_t moshi_n_tensors(const moshi_config* cfg);

/* Creates a context and uploads the weights.
 * tensors: n_tensors host pointers in the order below, each row-major in the
 * config's dtype (uint16 bf16 bit patterns or float32); copied, so the caller
 * may free them afterwards. A matrix [N, K] maps a K-vector to N outputs.
 *   emb.text [Vt+1, D]; emb.audio.k [Va+1, D] for k < S;
 *   per temporal layer l: attn_norm [D], qkv [3D, D] (rows q|k|v),
 *     o [D, D], mlp_norm [D], gate_up [2F, D] (rows gate|up), down [D, F];
 *   out_norm [D]; text_head [Vt, D];
 *   dep.in.s [Dd, D] for s < S; dep.emb.0 [Vt+1, Dd]; dep.emb.s [Va+1, Dd];
 *   per depformer layer l: attn_norm [Dd], mlp_norm [Dd] (shared by substeps);
 *   per substep s, per layer l: qkv [3Dd, Dd], o [Dd, Dd],
 *     gate_up [2Fd, Dd], down [Dd, Fd];
 *   dep.head.s [Va, Dd] for s < S;
 *   dep.out_norm [Dd] (MOSHI_FLAG_DEP_FINAL_NORM only).
 * (Shapes: mobius PR #368, "P2 - Moshi LM": FusedGateUpMLP, weights_per_step
 * = 16; recipe "Architecture": the 17-row token column.)
 * hip_stream: a hipStream_t created by the caller (not the legacy default
 * stream) that every launch and copy uses, or NULL for a library-owned
 * stream. A borrowed stream is never destroyed.
 * Errors: MOSHI_E_INVALID (bad config / count / NULL), MOSHI_E_OOM,
 * MOSHI_E_DEVICE (no GPU or a HIP failure). *out is NULL on error. */
int moshi_create(const moshi_config* cfg, const void* const* tensors, int32_t n_tensors,
                 void* hip_stream, moshi_ctx** out);

/* Frees the context and its device memory (every call enqueued on it is
 * waited for first). NULL is accepted. */
int moshi_destroy(moshi_ctx* ctx);

/* The config a context was created with (*out; MOSHI_E_INVALID on NULL). */
int moshi_get_config(const moshi_ctx* ctx, moshi_config* out);

/* Opens a session in the lowest free slot: position 0, empty window
 * (recipe "When to use this recipe": sessions join on any tick; "Notes": a
 * recycled slot behaves exactly like a fresh engine).
 * MOSHI_E_FULL when all B slots are live ("Notes": connections beyond N are
 * rejected until a slot frees). Host bookkeeping only; it takes effect at the
 * next step, and steps already enqueued keep the slots they were enqueued
 * with. */
int moshi_session_join(moshi_ctx* ctx, int32_t* slot_out);

/* Sampling parameters of one session (SGLang-Omni cookbook "PersonaPlex",
 * "Request parameters": text temperature / top-k 0.7 / 25 by default,
 * temperature 0 = greedy; audio 0.8 / 250; a seed that makes both draws
 * reproducible, with a child seed each; mobius PR #368's sampling commit:
 * temperature + top-k instead of greedy). top_k <= 0 or >= the vocabulary:
 * no top-k filter.
 * The draw (the same definition as the repository's CPU reference): it is
 * decided on the fp32 logits; the candidates are the top_k largest (lowest
 * index first among equal values, -0 below +0); weights exp((l - l_max) / T)
 * in fp64; the token is the first candidate in ascending index order whose
 * running sum of weights exceeds u * (their sum), the last candidate if none
 * does. u = (output pos+1 of a splitmix64 generator seeded with the stream's
 * child seed) >> 11, times 2^-53, where the child seed is output stream+1 of
 * a splitmix64 generator seeded with `seed`, stream 0 is the text head and
 * 1 + s depformer substep s, and pos is the number of frames the session had
 * consumed before this one. Forced tokens (moshi_step_forced) win over
 * drawn ones. */
typedef struct {
  double text_temperature;
  int32_t text_top_k;
  double audio_temperature;
  int32_t audio_top_k;
  uint64_t seed;
} moshi_sampling;

/* Sets a live session's sampling (NULL: greedy, the default after a join).
 * Takes effect at the next step. MOSHI_E_INVALID without MOSHI_FLAG_SAMPLING
 * (unless NULL or both temperatures <= 0); MOSHI_E_NOSESSION if the slot is
 * not live. */
int moshi_session_set_sampling(moshi_ctx* ctx, int32_t slot, const moshi_sampling* p);

/* Closes a live session; its slot becomes free for the next join (recipe
 * "When to use this recipe": leaving does not disturb the other slots).
 * MOSHI_E_NOSESSION if the slot is out of range or not live. */
int moshi_session_leave(moshi_ctx* ctx, int32_t slot);

/* One frame for every live slot (synchronous: returns when the outputs are on
 * the host) -- recipe "Why it is different": one user frame in, one agent
 * frame and one text token out per 80 ms tick; mobius PR #368 "P3 - ONNX
 * Runtime example": the temporal step, greedy text, then the autoregressive
 * depformer substeps.
 * frames [B, 1+S] int32: row = slot; text code in [0, Vt], audio codes in
 *   [0, Va] (the last row of each table is the initial token). Any live row
 *   out of range -> MOSHI_E_INVALID before any device work, state unchanged.
 * text_token [B]: greedy text token (lowest index on ties).
 * audio_codes [B, S]: greedy code of each depformer substep; substep s
 *   consumes code s-1 (the text token at s = 0).
 * Each live slot's position advances by one; the frame's K/V are written into
 * the slot's ring at position mod W. */
int moshi_step(moshi_ctx* ctx, const int32_t* frames, int32_t* text_token, int32_t* audio_codes);

/* moshi_step with teacher forcing (mobius PR #368, the persona/voice commit:
 * the step teacher-forces the agent audio stream for priming; the sampling
 * commit: an explicitly supplied text token replaces the generated one).
 * forced [B, 1+S] int32 or NULL: where forced[b][0] >= 0 it is slot b's text
 * token (fed to depformer substep 0 and returned instead of the model's
 * choice); where forced[b][1+s] >= 0 it is code s (fed to substep s+1 and
 * returned). -1 = not forced. Forced text must lie in [0, Vt), forced codes
 * in [0, Va); anything else -> MOSHI_E_INVALID before any device work. The
 * logits stay the model's own. */
int moshi_step_forced(moshi_ctx* ctx, const int32_t* frames, const int32_t* forced,
                      int32_t* text_token, int32_t* audio_codes);

/* Device-resident step, for callers whose codes already live in HBM (a codec
 * on the same GPU; mobius PR #368, the device-resident KV commit: keep the
 * step's state on the device): enqueues one moshi_step on the context's
 * stream and returns without waiting.
 * d_frames: DEVICE pointer to [B, 1+S] int32 codes, read when the step runs.
 *   Codes are not checked on the host; a live code outside its table is
 *   clamped to the nearest valid row and reported by the next moshi_sync.
 * d_text_token [B], d_audio_codes [B, S]: DEVICE pointers that receive the
 *   outputs (either may be NULL; the last outputs also stay readable through
 *   moshi_read_logits). Live slots' positions advance by one per call. */
int moshi_step_enqueue(moshi_ctx* ctx, const int32_t* d_frames, int32_t* d_text_token,
                       int32_t* d_audio_codes);

/* moshi_step_enqueue for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * one-session step kernel and results, with its synchronisation scratch --
 * grid-barrier counters and the flagged hand-off arena -- in a static device
 * array of the library (40 MiB per GPU, held until the process ends) instead
 * of the context's buffers. The call allocates nothing.
 * Only for contexts that use the step kernel (moshi_uses_step_kernel == 1)
 * whose scratch fits the array (the PersonaPlex shape needs 29.7 MB);
 * otherwise MOSHI_E_INVALID with the sizes in moshi_last_error. Calls that
 * overlap on one GPU (other streams or threads using this entry point at the
 * same time) race: serialise them. Arguments, outputs and errors as for
 * moshi_step_enqueue; moshi_sync waits for it. A join, leave or prefill since
 * the last step enqueues one small host-to-device copy of the slot table. */
int moshi_step_enqueue_noalloc(moshi_ctx* ctx, const int32_t* d_frames, int32_t* d_text_token,
                               int32_t* d_audio_codes);

/* Waits for every enqueued step. MOSHI_E_INVALID if a clamped code was seen
 * since the last call (the flag is then cleared); MOSHI_E_DEVICE if a step
 * kernel gave up waiting (the context is then unusable). */
int moshi_sync(moshi_ctx* ctx);

/* ---- delayed-stream wrapper (host-side, over moshi_step_forced) ----
 * The user contract of the pages' runtime (mobius PR #368, "P3 - ONNX
 * Runtime example": the port of Kyutai's LMGen.step keeps a ring cache with
 * per-codebook delays [0,0,1,1,1,1,1,1,1,0,1,1,1,1,1,1,1] and collects the
 * delayed outputs; the persona/voice commit teacher-forces the agent audio
 * (codebooks 1..8) and the text stream to prime a conversation).
 * Channels: 0 text, 1..A the agent's codebooks (the depformer's first A
 * substeps), A+1..S the user's. Channel k of stream column c carries its
 * token of acoustic frame c - d_k, the initial token (row Vt of the text
 * table, row card of an audio table) where c - d_k < 0. Step t feeds column
 * t to moshi_step_forced, writes the generated text and agent codes into
 * column t+1 (column 0 of those channels is initial), and puts the user's
 * frame t into column t + d_k. After step t the acoustic frame
 * t + 1 - max(d) is complete and is returned when it is >= 1: with delays of
 * at most 1, n steps return n - 1 frames. The object is host memory; the
 * caller owns it and must not use it with other threads at the same time. */
typedef struct moshi_stream moshi_stream;

/* A wrapper over every slot of `ctx` (the context must outlive it).
 * n_agent = A, 1 <= A < n_substeps, A <= the substeps run (dep_q).
 * delays [1+S] (each 0..8) or NULL for the pages' pattern: 0 for the text,
 * and in each half of the audio channels 0 for the first codebook and 1 for
 * the others. MOSHI_E_INVALID on bad arguments. */
int moshi_stream_create(moshi_ctx* ctx, int32_t n_agent, const int32_t* delays,
                        moshi_stream** out);
int moshi_stream_destroy(moshi_stream* s);

/* Starts the stream of a live slot afresh (call after moshi_session_join,
 * and after moshi_session_prefill_kv if the session is primed from K/V).
 * MOSHI_E_NOSESSION if the slot is not live. */
int moshi_stream_reset(moshi_stream* s, int32_t slot);

/* One step of every live slot of the context.
 * user [B, S-A]: the user's codes of this acoustic frame, each in [0, card).
 * forced [B, 1+A] or NULL: what this step generates for column t+1, -1 = the
 *   model's own choice: [0] the text token (in [0, Vt); also depformer
 *   substep 0's input), [k] agent codebook k (in [0, card); substep k's input).
 * out_frames [B, 1+A]: the completed acoustic frame (text, agent codes) of
 *   slots whose out_ready [B] is 1; -1 elsewhere.
 * step_text [B], step_codes [B, S] (either may be NULL): the step's raw
 *   tokens (the user channels' substeps included; -1 past dep_q).
 * A live slot that was not reset since it joined (or that another caller
 * stepped) -> MOSHI_E_INVALID, nothing changes; see moshi_stream_last_error. */
int moshi_stream_step(moshi_stream* s, const int32_t* user, const int32_t* forced,
                      int32_t* out_frames, int32_t* out_ready, int32_t* step_text,
                      int32_t* step_codes);

/* Detail of the last error of a wrapper (never NULL). */
const char* moshi_stream_last_error(const moshi_stream* s);

/* ---- test and benchmark hooks (same kernels as moshi_step) ---- */

/* Temporal transformer and text head only (the depformer is not run); the
 * positions advance as in moshi_step. text_token [B]. (mobius PR #368, "P2 -
 * Moshi LM": the temporal task returns the hidden state and text logits.) */
int moshi_temporal_step(moshi_ctx* ctx, const int32_t* frames, int32_t* text_token);

/* Depformer only, from a given hidden state: hidden [B, D] in the config's
 * dtype (the temporal output after its final norm), text_in [B] in [0, Vt].
 * audio_codes [B, S]. Positions do not move. Rows of non-live slots ignored.
 * (mobius PR #368, "P2 - Moshi LM": the depformer task takes the hidden
 * state and the previous token.) */
int moshi_depformer_step(moshi_ctx* ctx, const void* hidden, const int32_t* text_in,
                         int32_t* audio_codes);

/* Loads K and V of positions 0..n-1 of a live slot (n in [0, W]) and sets its
 * position to n. k, v: [L][n][D] in the config's dtype, already rotated
 * (post-RoPE), head h at columns h*head_dim.. of each row. (A conversation
 * already n frames into the recipe's 3000-frame ring, "Architecture".)
 * MOSHI_E_INVALID for n outside [0, W] or NULL data; state unchanged. */
int moshi_session_prefill_kv(moshi_ctx* ctx, int32_t slot, int32_t n, const void* k,
                             const void* v);

/* Multi-frame prefill (mobius PR #368, "P2 - Moshi LM": the temporal task
 * takes input_frame[B, 17, S] with S > 1; the persona/voice commit primes a
 * conversation in about 2 s): runs the temporal transformer and text head
 * over n consecutive frames of one live session at once -- the same result
 * as n temporal-only steps (moshi_temporal_step) of that session, with every
 * projection an MFMA product over up to 64 frames at a time. The depformer
 * does not run. The frames' K/V are written into the session's ring and its
 * position advances by n; other slots are untouched.
 * frames [n, 1+S] int32 (codes as in moshi_step; any out of range ->
 *   MOSHI_E_INVALID before any device work); text_tokens [n] (greedy) and
 *   text_logits [n, Vt] float32 receive each frame's outputs (either may be
 *   NULL). A workspace (~60 MB at the PersonaPlex shape) is allocated at the
 *   first call. Synchronous. */
int moshi_session_prefill_frames(moshi_ctx* ctx, int32_t slot, int32_t n, const int32_t* frames,
                                 int32_t* text_tokens, float* text_logits);

/* Copies a live slot's whole ring out: k, v [L][W][D] in the config's dtype,
 * ring slot j (row j) holding the position congruent to j mod W; rows the
 * session has not written yet are unspecified. (The recipe's ring KV cache,
 * "Architecture".) */
int moshi_session_read_kv(moshi_ctx* ctx, int32_t slot, void* k, void* v);

/* Bookkeeping of a live slot's next step: absolute position (frames consumed;
 * the RoPE offset, which mobius PR #368 derives from the cache length),
 * fill = min(pos, W), ring write index = pos mod W (recipe "Notes": the ring
 * recycles beyond 3000 frames). */
int moshi_session_info(moshi_ctx* ctx, int32_t slot, int64_t* pos, int32_t* fill,
                       int32_t* write_idx);

/* Logits of the last step: text [B, Vt] and/or audio [B, S, Va] (float32;
 * either may be NULL). Rows of non-live slots, and of substeps not run, are
 * unspecified. Ordered after every step enqueued on the context's stream.
 * (mobius PR #368, "P2 - Moshi LM": text_logits and the depformer logits.) */
int moshi_read_logits(moshi_ctx* ctx, float* text, float* audio);

/* Temporal hidden state of the last step (after the final norm and rounding),
 * [B, D] float32 (the "hidden" output of mobius PR #368's temporal task). */
int moshi_read_hidden(moshi_ctx* ctx, float* hidden);

/* Kernel timing (measurement hook; the per-frame budget of the recipe's
 * "Notes" and of mobius PR #368's RTF reports). Runs `n_steps` full steps
 * (frames as in moshi_step, outputs
 * discarded; positions advance) launching every kernel eagerly with a HIP
 * event pair around it on the library's stream, and returns per kernel class
 * c < n_classes: the summed device time in ms (ms[c]), the launch count
 * (launches[c]) and the algorithmic bytes moved (bytes[c]: weights read once,
 * K/V attended and written). Class names: moshi_kernel_class_name(c).
 * Where a persistent kernel runs (moshi_uses_step_kernel or
 * moshi_uses_dep_kernel) its operations are instead timed from workgroup 0's
 * clock at each grid barrier or hand-off, under the class of the kernel each
 * replaces, and launches[c] counts those phases.
 * Returns the number of classes (>= 0) or an error. */
int moshi_time_kernels(moshi_ctx* ctx, const int32_t* frames, int32_t n_steps, double* ms,
                       int64_t* launches, double* bytes, int32_t n_classes);
const char* moshi_kernel_class_name(int32_t c);

/* Which implementation runs the step (measurement hook).
 * 1 if moshi_step / moshi_step_enqueue run the whole frame as one persistent
 * kernel (capacity 1 with a supported shape, unless the environment variable
 * MOSHI_STEP_KERNEL=0 was set at creation), 0 if they run one kernel per
 * operation; the results are identical. Negative on a NULL context. */
int32_t moshi_uses_step_kernel(const moshi_ctx* ctx);

/* 1 if the depformer of every step (the 16 substeps of "vLLM-Omni recipe:
 * PersonaPlex", "Architecture") runs as one persistent kernel for all slots:
 * capacity 2..64 with a supported shape and without MOSHI_FLAG_SAMPLING,
 * unless the environment variable MOSHI_DEP_MULTI=0 was set at creation;
 * 0 if it runs one kernel per operation. The results are identical.
 * Negative on a NULL context. */
int32_t moshi_uses_dep_kernel(const moshi_ctx* ctx);

/* Test hook of the persistent kernels' bounded waits (the failure path that
 * keeps a lost hand-off from hanging the GPU): every later launch of the step
 * kernel or of the multi-session depformer kernel on this context
 * gives up after `limit` polls (>= 1) of a grid barrier or flagged input,
 * raises the context's abort flag, and every workgroup leaves; the call then
 * fails with MOSHI_E_DEVICE and the context stays failed. MOSHI_E_INVALID if
 * the context uses neither. */
int moshi_test_set_spin_limit(moshi_ctx* ctx, int32_t limit);

/* Static text of a status code. */
const char* moshi_strerror(int status);

/* Detail of the last error on this context (never NULL). */
const char* moshi_last_error(const moshi_ctx* ctx);

#ifdef __cplusplus
}
#endif

#endif /* MOSHI_H */
