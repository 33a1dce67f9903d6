/*
 * mtp.h -- C ABI of libmtp, the MI355X (gfx950) implementation of the MTP
 * (multi-token-prediction) speculative-decoding round: the draft-head step, the
 * pending-pair flush, speculative verification and draft-KV rollback.
 *
 * Conventions for every entry point
 *  - Pointers named *_dev, and every tensor argument, are caller-owned DEVICE
 *    pointers; structs passed by pointer (config, weights, kv descriptor,
 *    sampling) are HOST memory read during the call only.
 *  - The library never allocates device memory.  Scratch lives in a caller-owned
 *    workspace sized by mtp_workspace_bytes / spec_verify_workspace_bytes.  No
 *    kernel relies on its previous contents (every scratch value is written
 *    before it is read in the same call); mtp_workspace_init zeroes one anyway
 *    so a fresh workspace holds no stale values from the allocator.
 *  - Every compute call is asynchronous on `stream` and does not synchronise.
 *  - Host-checkable problems return a negative mtp_status BEFORE anything is
 *    enqueued (fail closed).  Problems only the device can see (a device-side
 *    count above its host bound, a KV append past capacity, a rollback past the
 *    current length) set the sticky error word state[3] of the draft KV; every
 *    later kernel on that KV is then a no-op.  Read state[] at the round's host
 *    synchronisation.
 *  - Not thread-safe per workspace or per KV; distinct (workspace, KV) pairs are
 *    independent.  Calls that share a workspace must be ordered on one stream.
 *  - Layouts are row-major; weight matrices are [out, in] (nn.Linear).  Norm
 *    weights are the final multiplicative values (any +1.0 offset of a raw
 *    checkpoint already applied).  Tokens are int32; logits and uniforms fp32.
 *
 * The pages describing the method: "Ollama qwen3_5 MTP loader and SelfDraft
 * path" (Facts), "feat(inference): support the qwen3_5_mtp drafter for
 * Qwen3.5/3.6/3.8 MTP speculative decoding" (sections "Where the MTP weights
 * actually live", "Upstream contract to port", "Acceptance criteria"), and the
 * Ollama x/mlxrunner commit log.
 */
#ifndef MTP_H_
#define MTP_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MTP_OK = 0,
  MTP_E_INVALID_ARG = -1, /* null pointer, bad size, bad mode */
  MTP_E_UNSUPPORTED = -2, /* shape or option outside what the kernels implement */
  MTP_E_NOT_BOUND = -3,   /* embedding table or lm_head missing: the head borrows both */
  MTP_E_CAPACITY = -4,    /* host-visible KV capacity or flush-size bound exceeded */
  MTP_E_HIP = -5,         /* a HIP launch or runtime call failed */
  MTP_E_DEVICE = -6,      /* reported by callers that read a non-zero state[3] */
  MTP_E_WORKSPACE = -7    /* workspace smaller than the size function returns */
} mtp_status;

typedef enum { MTP_F32 = 0, MTP_BF16 = 1, MTP_I8G128 = 2 } mtp_dtype;

/* Device error codes stored in mtp_kv.state[3]: the append would pass the
 * capacity; a rollback target above the length; a device pair count outside
 * [0, n_max]; a pair's token outside [0, vocab).  Once set, every later kernel on
 * that cache is a no-op until the caller clears the word. */
enum { MTP_DEV_OK = 0, MTP_DEV_CAPACITY = 1, MTP_DEV_ROLLBACK = 2, MTP_DEV_COUNT = 3, MTP_DEV_TOKEN = 4 };

/* Shape and storage of the draft head.  Source: "Upstream contract to port"
 * (fc 2H->H, the two pre-fc RMSNorms, one full-attention layer with q/k norms,
 * final norm; embedding and lm_head borrowed from the target).
 * hidden, intermediate: multiples of 64; head_dim: 64, 128 or 256;
 * n_q_heads / n_kv_heads in {1, 2, 3, 4, 6, 8}.
 * weight_dtype (projections, norms, embedding): F32 or BF16.
 * act_dtype (hidden states crossing the ABI): F32 or BF16.
 * kv_dtype: F32 or BF16.  lm_head_dtype: F32, BF16 or I8G128 (int8 per row and
 * 128-column group, fp16 scales [vocab, hidden/128], value = q * s). */
typedef struct {
  int32_t hidden, n_q_heads, n_kv_heads, head_dim, intermediate, vocab;
  float rms_eps, rope_theta;
  int32_t weight_dtype, act_dtype, kv_dtype, lm_head_dtype;
} mtp_head_config;

/* The 15 head tensors ("Where the MTP weights actually live") plus the borrowed
 * embedding table [vocab, hidden] and lm_head [vocab, hidden].  Shapes:
 * fc [H, 2H] (columns: embedding half first); q_proj [Hq*D, H]; k_proj, v_proj
 * [Hkv*D, H]; o_proj [H, Hq*D]; gate_proj, up_proj [I, H]; down_proj [H, I];
 * q_norm, k_norm [D]; the five other norms [H].  Must outlive the mtp_head. */
typedef struct {
  const void *embed, *lm_head, *lm_head_scales;
  const void *pre_fc_norm_embedding, *pre_fc_norm_hidden, *fc, *input_layernorm;
  const void *q_proj, *k_proj, *v_proj, *q_norm, *k_norm, *o_proj;
  const void *post_attention_layernorm, *gate_proj, *up_proj, *down_proj, *norm;
} mtp_head_weights;

/* Opaque HOST object holding the validated config and weight pointers. */
typedef struct mtp_head mtp_head;

/* The head's own draft KV cache (separate from the target's; only the position
 * offset is shared: "Upstream contract to port").  k, v: [n_kv_heads, capacity,
 * head_dim] in kv_dtype, capacity <= 2^20.  state: device int32[4] = {len,
 * round_base, reserved, err}; slot S holds the pair (token S+1, target hidden S)
 * at RoPE position S. */
typedef struct {
  void *k, *v;
  int32_t capacity;
  int32_t *state;
} mtp_kv;

/* Sampler settings ("Ollama qwen3_5 MTP loader and SelfDraft path", Facts
 * "Verification": temperature, penalty, top-k/top-p/min-p).  temperature 0 means
 * greedy.  top_k 0 = off, top_p >= 1 = off, min_p 0 = off, repeat_penalty 1 = off.
 * window: length of the history ring the penalty looks at (1..1024). */
typedef struct {
  float temperature, repeat_penalty, top_p, min_p;
  int32_t top_k, window;
} spec_sampling;

enum { MTP_FLUSH_KV_ONLY = 0, MTP_FLUSH_LAST = 1, MTP_FLUSH_ALL = 2 };
#define MTP_TO_ROUND_BASE (-1)
#define MTP_MAX_FLUSH 256  /* pending-pair flush cap ("Facts": flush batches of up to 256) */
#define MTP_MAX_DRAFT 16   /* drafts per verify */
#define MTP_MAX_BATCH 16   /* sessions per batched call */

/* Library infrastructure (no passage of the pages defines these): the name of a
 * status code (static string, never NULL; "MTP_E_UNKNOWN" for other values). */
const char *mtp_status_string(int status);

/* Library infrastructure: text of the last HIP error this thread's calls
 * returned MTP_E_HIP for (static string owned by the HIP runtime). */
const char *mtp_last_error(void);

/* Validate the config and weights and build the host-side head object
 * ("feat(inference): support the qwen3_5_mtp drafter ...", section "Upstream
 * contract to port": the drafter holds its own layer, pre-fc norms, fc and final
 * norm, borrows the target's embedding table and lm_head through a bind step,
 * and its drafting raises when bind was skipped -- here that is creation).
 * Returns MTP_E_NOT_BOUND if embed or lm_head is NULL (the head owns neither),
 * MTP_E_INVALID_ARG for other NULL tensors or bad sizes, MTP_E_UNSUPPORTED for
 * shapes outside the kernels.  *out is set only on success; nothing is
 * allocated on the device and no HIP call is made.  The weight pointers are
 * borrowed: they must outlive the head.  mtp_head_destroy(NULL) is a no-op. */
int mtp_head_create(const mtp_head_config *cfg, const mtp_head_weights *w, mtp_head **out);
void mtp_head_destroy(mtp_head *head);

/* Library infrastructure: workspace bytes for calls with at most max_rows
 * pairs (1..256) on a KV of at most max_capacity slots.  It takes the config,
 * not a head, so a caller can size (and allocate) the workspace before the
 * weights are bound.  0 on invalid arguments. */
size_t mtp_workspace_bytes(const mtp_head_config *cfg, int32_t max_rows, int32_t max_capacity);

/* Library infrastructure: zero a workspace (either kind) with a fill kernel on
 * `stream` (asynchronous; no hipMemset node, so it may be graph-captured). */
int mtp_workspace_init(void *ws, size_t ws_bytes, hipStream_t stream);

/* One draft-head step ("Facts", MTP drafting: one head call per draft token) at
 * slot S = state[0]: the pair (token_dev[0], hidden_in_dev) is appended to the
 * draft KV at S and state[0] becomes S + 1.
 * token_dev: int32[1]; hidden_in_dev: [hidden] act_dtype; hidden_out_dev:
 * [hidden] act_dtype, the layer output before the final norm (the hidden a
 * chained step feeds back); logits_dev (nullable): fp32 [vocab];
 * argmax_dev (nullable): int32[1], lowest index among equal maxima.
 * hidden_out_dev must not alias hidden_in_dev. */
int mtp_draft_step(const mtp_head *head, const mtp_kv *kv, const int32_t *token_dev,
                   const void *hidden_in_dev, void *hidden_out_dev, float *logits_dev,
                   int32_t *argmax_dev, void *ws, size_t ws_bytes, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): mtp_draft_step
 * without a workspace argument.  Its scratch is a static array of
 * MTP_STATIC_SCRATCH_BYTES held by the library on each device it runs on (for
 * the life of the process); nothing is allocated and no allocating routine is
 * called.  Arguments, results and device errors are those of mtp_draft_step.
 * Returns MTP_E_WORKSPACE, before anything is enqueued, when the step needs more
 * scratch than the array holds (mtp_workspace_bytes(cfg, 1, capacity) >
 * MTP_STATIC_SCRATCH_BYTES; the 27B-shaped head at any capacity needs about
 * 2 MiB).  Every call on one device shares that device's array: calls that may
 * overlap on one device (two streams, two threads) race and give wrong results;
 * order them on one stream.  No scratch value survives from one call to the
 * next in any way that matters (each is written before it is read). */
#define MTP_STATIC_SCRATCH_BYTES (4 << 20)
int mtp_draft_step_static(const mtp_head *head, const mtp_kv *kv, const int32_t *token_dev,
                          const void *hidden_in_dev, void *hidden_out_dev, float *logits_dev,
                          int32_t *argmax_dev, hipStream_t stream);

/* Pending-pair flush ("Facts", MTP drafting: pending pairs flush in batches of
 * up to 256): n complete pairs (tokens_dev[j], hiddens_dev[j]) are appended at
 * slots state[0] + j, causal within the batch and over the whole prefix.
 * n = n_max, or min(*n_dev, n_max) when n_dev is given (device count; a count
 * above n_max or below 0 sets state[3] = MTP_DEV_COUNT).  n_max <= 256.
 * out_mode KV_ONLY: only K/V.  LAST: hidden_out [hidden] (last row's g), logits
 * and argmax of the last row.  ALL: hidden_out [n, hidden] for every row, logits
 * and argmax of the last row.  set_round_base != 0 records state[1] = state[0]
 * after the append (the first provisional slot of a round).  A device count of
 * 0 appends nothing and leaves every output untouched (state[1] is still set). */
int mtp_flush_pairs(const mtp_head *head, const mtp_kv *kv, const int32_t *tokens_dev,
                    const void *hiddens_dev, int32_t n_max, const int32_t *n_dev,
                    int32_t out_mode, int32_t set_round_base, void *hidden_out_dev,
                    float *logits_last_dev, int32_t *argmax_last_dev, void *ws,
                    size_t ws_bytes, hipStream_t stream);

/* A round's drafting in one call ("Facts", MTP drafting: the pending pairs are
 * flushed, then one head call per draft token): mtp_flush_pairs(pending, LAST,
 * set_round_base = 1) followed by n_draft - 1 chained mtp_draft_step calls,
 * step i taking (d_{i-1}, g_{i-1}).  pend_tokens_dev / pend_hiddens_dev /
 * n_max / n_dev as for mtp_flush_pairs; drafts_dev int32[n_draft] receives
 * d_0..d_{n-1}; hiddens_out_dev [n_draft, hidden] (act dtype, must not overlap
 * the pending hiddens) the g of every draft; draft_logits_dev (nullable) fp32
 * [n_draft, vocab] the draft rows (sampled verification needs them).  The
 * workspace must hold n_max rows.  1 <= n_draft <= MTP_MAX_DRAFT.  A round
 * always has at least one pending pair (the last committed token with its
 * target hidden), so a device count of 0 (like one above n_max) sets state[3] =
 * MTP_DEV_COUNT and every kernel of the call, the chained steps included, is
 * then a no-op. */
int mtp_draft_chain(const mtp_head *head, const mtp_kv *kv, const int32_t *pend_tokens_dev,
                    const void *pend_hiddens_dev, int32_t n_max, const int32_t *n_dev, int32_t n_draft,
                    int32_t *drafts_dev, void *hiddens_out_dev, float *draft_logits_dev, void *ws,
                    size_t ws_bytes, hipStream_t stream);

/* Re-pairing under the keep-accepted rollback policy (the #1174 comment: only
 * the rejected suffix is trimmed), on the device: with k = out_counts_dev[0]
 * from spec_verify and j0 = min(k, n_draft - 1), the next round's pending pairs
 * j = 0..k - j0 are (out_tokens_dev[j0 + j], target hidden row j0 + j) and
 * *pend_count_dev = k + 1 - j0 (1 pair if k < n_draft, 2 if all were
 * accepted).  target_hiddens_dev: [n_draft + 1, hidden] in act_dtype (MTP_F32 or
 * MTP_BF16); pend_hiddens_dev must not overlap it.  Under the roll-back-to-base
 * policy no call is needed: the pending pairs are out_tokens_dev, the target
 * hidden rows and out_counts_dev[1] as they stand. */
int mtp_repair_pending(const int32_t *out_tokens_dev, const int32_t *out_counts_dev,
                       const void *target_hiddens_dev, int32_t hidden, int32_t act_dtype, int32_t n_draft,
                       int32_t *pend_tokens_dev, void *pend_hiddens_dev, int32_t *pend_count_dev,
                       hipStream_t stream);

/* ---- B > 1 independent sessions with ragged acceptance ------------------
 * ("feat(inference): support the qwen3_5_mtp drafter ...": section "Upstream
 * contract to port" advertises ragged batch acceptance, "Implementation plan"
 * and "Acceptance criteria" gate B > 1 behind ragged-acceptance tests, and the
 * #1174 comment trims each row by its own accepted count.)
 * A batch of B sessions (1 <= B <= MTP_MAX_BATCH) shares one draft-KV
 * allocation: mtp_kv.k and .v hold [B, n_kv_heads, capacity, head_dim] (session
 * b's cache starts b * n_kv_heads * capacity * head_dim elements in) and
 * mtp_kv.state holds [B, 4] state words, one {len, round_base, -, err} per
 * session.  Every session keeps its own length, so sessions that accepted
 * different numbers of drafts simply sit at different slots: nothing is padded
 * and no tail needs zeroing (a slot past a session's length is never read).
 * Weights stream once per launch for every session's rows.  Device errors are
 * per session: a set error word makes that session's rows no-ops while the
 * other sessions proceed.  Per-session arrays are session-major. */

/* Workspace bytes for mtp_draft_chain_batch with `batch` sessions of at most
 * max_rows pending pairs each on caches of at most max_capacity slots. */
size_t mtp_batch_workspace_bytes(const mtp_head_config *cfg, int32_t batch, int32_t max_rows,
                                 int32_t max_capacity);

/* mtp_draft_chain for `batch` sessions in one call: one flush of every
 * session's pending pairs (LAST mode, round base recorded per session), then
 * n_draft - 1 chained steps with one row per session.  pend_tokens_dev int32
 * [batch, n_max]; pend_hiddens_dev [batch, n_max, hidden] (act dtype); session
 * b flushes min(n_dev[b * n_dev_stride], n_max) pairs (n_dev nullable: n_max
 * each; a count of 0, below 0 or above n_max sets that session's error word to
 * MTP_DEV_COUNT).  Outputs: drafts_dev int32 [batch, n_draft];
 * hiddens_out_dev [batch, n_draft, hidden]; draft_logits_dev (nullable) fp32
 * [batch, n_draft, vocab].  With the pending pairs taken straight from
 * spec_verify_batch's outputs (tokens [batch, n_draft + 1], target hiddens
 * [batch, n_draft + 1, hidden], n_max = n_draft + 1) the counts are
 * out_counts + 1 with n_dev_stride 2.  Returns MTP_E_UNSUPPORTED for shapes the
 * batched kernels do not take. */
int mtp_draft_chain_batch(const mtp_head *head, const mtp_kv *kv, int32_t batch,
                          const int32_t *pend_tokens_dev, const void *pend_hiddens_dev, int32_t n_max,
                          const int32_t *n_dev, int32_t n_dev_stride, int32_t n_draft, int32_t *drafts_dev,
                          void *hiddens_out_dev, float *draft_logits_dev, void *ws, size_t ws_bytes,
                          hipStream_t stream);

/* spec_verify for `batch` independent sessions in one launch sequence: every
 * array of spec_verify gains a leading [batch] dimension (target logits
 * [batch, n_draft + 1, vocab], draft logits [batch, n_draft, vocab], drafts
 * [batch, n_draft], history [batch, window], history state [batch, 2],
 * uniforms [batch, n_draft + 1], out_tokens [batch, n_draft + 1], out_counts
 * [batch, 2]); each session accepts its own k.  ws_bytes >= batch *
 * spec_verify_workspace_bytes(n_draft, vocab). */
int spec_verify_batch(const spec_sampling *sp, int32_t batch, int32_t n_draft, int32_t vocab,
                      const float *target_logits_dev, const float *draft_logits_dev,
                      const int32_t *draft_tokens_dev, int32_t *history_dev, int32_t *history_state_dev,
                      const float *uniforms_dev, int32_t *out_tokens_dev, int32_t *out_counts_dev, void *ws,
                      size_t ws_bytes, hipStream_t stream);

/* kv_rollback for `batch` sessions: each session's length moves on its own
 * (to_len >= 0 for every session, or MTP_TO_ROUND_BASE to its own round base;
 * with counts_dev = spec_verify_batch's out_counts [batch, 2] each session
 * keeps min(k_b, n_draft - 1) chained entries). */
int kv_rollback_batch(const mtp_kv *kv, int32_t batch, int32_t to_len, const int32_t *counts_dev,
                      int32_t n_draft, hipStream_t stream);

/* mtp_repair_pending for `batch` sessions (out_tokens [batch, n_draft + 1],
 * out_counts [batch, 2], target hiddens [batch, n_draft + 1, hidden]; pending
 * tokens [batch, n_draft + 1], hiddens [batch, n_draft + 1, hidden], counts
 * [batch], so the next mtp_draft_chain_batch takes n_dev_stride 1). */
int mtp_repair_pending_batch(int32_t batch, const int32_t *out_tokens_dev, const int32_t *out_counts_dev,
                             const void *target_hiddens_dev, int32_t hidden, int32_t act_dtype, int32_t n_draft,
                             int32_t *pend_tokens_dev, void *pend_hiddens_dev, int32_t *pend_counts_dev,
                             hipStream_t stream);

/* Workspace bytes for spec_verify with n_draft drafts over vocab logits. */
size_t spec_verify_workspace_bytes(int32_t n_draft, int32_t vocab);

/* Verify n_draft (0..16) drafts against n_draft + 1 target rows ("Facts",
 * Verification; the commit log's rejection sampling, greedy as its point-mass
 * case).  target_logits_dev fp32 [n_draft+1, vocab]; draft_logits_dev fp32
 * [n_draft, vocab] (must be NULL iff temperature == 0); draft_tokens_dev int32
 * [n_draft]; history_dev int32 [window] ring with history_state_dev {head,
 * count} (head = next write slot), updated with the committed tokens;
 * uniforms_dev fp32 [n_draft+1] (u_i for the accept test of draft i, u_N for
 * the residual or bonus draw; may be NULL when greedy).  Outputs:
 * out_tokens_dev int32 [n_draft+1] (first k+1 valid), out_counts_dev int32[2] =
 * {k accepted, k+1 committed}.  Accept d_i iff u_i * q_i(d_i) < p_i(d_i); at the
 * first rejection draw from normalise(max(0, p - q)) (p if that is zero); if all
 * are accepted draw the bonus from p_N.  Sampler order: penalty, temperature,
 * top-k, softmax, top-p, min-p.  Any top_k >= 0 (0 = the whole vocabulary):
 * top_k in 1..256 with ceil(vocab / 4096) * top_k <= 8192 selects per-chunk
 * candidates; other values take the whole-vocabulary path (radix passes over
 * each row's transformed logits, slower). */
int spec_verify(const spec_sampling *sp, int32_t n_draft, int32_t vocab,
                const float *target_logits_dev, const float *draft_logits_dev,
                const int32_t *draft_tokens_dev, int32_t *history_dev,
                int32_t *history_state_dev, const float *uniforms_dev,
                int32_t *out_tokens_dev, int32_t *out_counts_dev, void *ws,
                size_t ws_bytes, hipStream_t stream);

/* Draft-KV rollback (the #1174 comment: trim attention KV by the rejected
 * count): state[0] := to_len (>= 0), or with MTP_TO_ROUND_BASE := state[1]
 * (every chained entry provisional), or := state[1] + min(*n_accepted_dev,
 * n_draft - 1) when n_accepted_dev is given (keep accepted chained entries).
 * O(1): no K/V byte is touched.  A target above the current length sets
 * state[3] = MTP_DEV_ROLLBACK.  to_len > capacity is rejected on the host. */
int kv_rollback(const mtp_kv *kv, int32_t to_len, const int32_t *n_accepted_dev,
                int32_t n_draft, hipStream_t stream);

/* A round's tail in one call: spec_verify (same arguments, same outputs), then
 * in its final kernel the draft-KV rollback kv_rollback(kv, to_len,
 * keep_accepted ? &out_counts_dev[0] : NULL, n_draft) would make (the #1174
 * comment: trim attention KV by the rejected count; keep_accepted 0 or 1, 1
 * only with MTP_TO_ROUND_BASE), with no launch of its own.  report_dev
 * (nullable) receives int32 [6 + n_draft + 1] = {the KV state words after the
 * rollback, k, k + 1, the first k + 1 committed tokens; later entries
 * untouched} through system-scope stores, so it may be host-coherent pinned
 * memory the host reads once the stream has passed this call.  The KV
 * arguments are checked as kv_rollback checks them, before anything is
 * enqueued. */
int spec_verify_rollback(const spec_sampling *sp, int32_t n_draft, int32_t vocab,
                         const float *target_logits_dev, const float *draft_logits_dev,
                         const int32_t *draft_tokens_dev, int32_t *history_dev,
                         int32_t *history_state_dev, const float *uniforms_dev,
                         int32_t *out_tokens_dev, int32_t *out_counts_dev, void *ws,
                         size_t ws_bytes, const mtp_kv *kv, int32_t to_len,
                         int32_t keep_accepted, int32_t *report_dev, hipStream_t stream);

/* Benchmark timing of one kernel class.  After mtp_timing_begin(kind, n) the
 * next n launches of that class (any stream, eager or being captured into a
 * graph) are each bracketed by a pair of HIP events recorded on their stream,
 * in slots 0, 1, 2, ...  mtp_timing_elapsed waits for slots [first, first +
 * count) and returns their summed kernel time (ms); a captured slot holds the
 * timing of the graph's latest replay.  mtp_timing_end returns the sum over all
 * used slots and their count, then releases the events.  Host-side state,
 * process-wide; one class at a time.  Classes:
 *   MTP_TIME_UNEMBED     the unembedding GEMV (lm_head, fused argmax partials)
 *   MTP_TIME_ATTENTION   the attention kernel over the draft KV (not its merge)
 *   MTP_TIME_VERIFY      the verification kernel that reads every logit (the
 *                        per-chunk top-k pass, or the greedy argmax pass)
 *   MTP_TIME_PROJECTION  every projection launch of the head other than the
 *                        unembedding (fc, q/k/v, o, gate/up, down) */
enum { MTP_TIME_UNEMBED = 0, MTP_TIME_ATTENTION = 1, MTP_TIME_VERIFY = 2, MTP_TIME_PROJECTION = 3 };
int mtp_timing_begin(int32_t kind, int32_t max_launches);
/* Suspend (paused != 0) or resume bracketing new launches without releasing
 * the slots, so that only a sample of launches carries the events (each event
 * pair holds the stream for a few microseconds). */
int mtp_timing_pause(int32_t paused);
int mtp_timing_elapsed(int32_t first, int32_t count, float *total_ms);
int mtp_timing_end(float *total_ms, int32_t *launches);

/* Draft-depth controller (host object, no device work).  It chooses how many
 * tokens to draft in each round: argmax over N of committed(N) / cost(N), from
 * live per-position acceptance and a per-depth round cost, N from 0 (plain
 * decode: nothing drafted) up to one past the deepest position drafted so far;
 * every few rounds it drafts one deeper than its choice (a probe: after 4
 * rounds, then 8, 16, ... up to every 512; back to 4 when the choice changes).
 * Its state persists across requests for as long as the object lives.  (The
 * depth-control Facts of "Ollama qwen3_5 MTP loader and SelfDraft path"; the
 * Ollama x/mlxrunner commit choosing the draft length for throughput.)
 *   acceptance of position i: (accepts_i + 1) / (attempts_i + 2)
 *   committed(N) = 1 + sum_{i=1..N} prod_{j<=i} a_j (the round stops at its
 *                  first rejection; the correction or bonus token always commits)
 *   cost: seeded per depth by the caller (any unit, > 0; e.g. the measured round
 *         time at each depth), then cost[d] = 3/4 cost[d] + 1/4 reported time.
 * Ties go to the smaller depth.  fp64, fixed order: decisions are reproducible.
 *
 * mtp_depth_ctl_create: max_depth in [0, MTP_MAX_DRAFT]; cost: HOST double
 *   [max_depth + 1], every entry > 0 (copied).  INVALID_ARG otherwise, *out NULL.
 * mtp_depth_ctl_next: the depth to draft this round (advances the probe
 *   counter); negative status on a NULL controller.
 * mtp_depth_ctl_report: the round drafted `depth`, `accepted` of them were
 *   accepted (0 <= accepted <= depth), and it took `round_cost` (> 0).
 * mtp_depth_ctl_state: the current choice, probe interval and cost table
 *   (HOST double [max_depth + 1]); each output pointer may be NULL.
 * Not thread-safe per controller; distinct controllers are independent. */
typedef struct mtp_depth_ctl mtp_depth_ctl;
int mtp_depth_ctl_create(int32_t max_depth, const double *cost, mtp_depth_ctl **out);
void mtp_depth_ctl_destroy(mtp_depth_ctl *ctl);
int32_t mtp_depth_ctl_next(mtp_depth_ctl *ctl);
int mtp_depth_ctl_report(mtp_depth_ctl *ctl, int32_t depth, int32_t accepted, double round_cost);
int mtp_depth_ctl_state(const mtp_depth_ctl *ctl, int32_t *choice, int32_t *interval, double *cost);

#ifdef __cplusplus
}
#endif
#endif /* MTP_H_ */
