/*
 * dspark_verify.h -- C ABI of the MI355X (gfx950) DSpark verify sampler.
 *
 * One speculative-decoding verify step for B streams, each carrying a block of
 * draft tokens: the drafter's logits get the DSpark Markov-head bias, both sides
 * are softmaxed, and either the token-by-token rule or block verification keeps
 * a prefix of the drafts and emits one token of the target's own.
 *
 * Sources (page titles, with the section each entry point follows):
 *   [P1] "MTP, DSpark and Block Verification, Explained" (al-engr.com)
 *   [P2] "MTP Heads and Confidence Heads" (naphjohn.github.io LLM-blog, ep7)
 *   [P3] "Teaching the Speculator What a Draft Costs" (al-engr.com)
 *
 * Conventions shared by every entry point
 *   - Pointers marked "device" must be device memory of the current HIP device;
 *     "host" pointers are read during the call only.  All tensors are dense,
 *     row-major, with the shapes given.  bf16 values are raw 16-bit patterns.
 *   - The caller owns every buffer, including the workspace.  The library never
 *     allocates, frees or synchronises; all work is enqueued on `stream`
 *     (a hipStream_t; NULL means the default stream) and completes in order.
 *     The one exception is the online cost table, a host object whose create
 *     and destroy calls allocate and free host memory and HIP events.
 *   - Host-checkable errors return a status and enqueue nothing.  A failed
 *     launch returns DSPARK_ERR_HIP.  Device-data preconditions (token ids in
 *     range, temperatures >= 0, num_drafts in [0, k]) are the caller's: the
 *     kernels clamp indices so that no access leaves its buffer, but outputs for
 *     invalid data are unspecified.
 *   - Same inputs, seed and step give bit-identical outputs on every run: no
 *     reduction uses floating-point atomics.
 *   - Random numbers are Philox4x32-10 (Salmon et al., SC'11) with key = seed
 *     and counter = (global stream index, index, purpose, step): purpose 1 gives
 *     the accept uniforms u_{b,j} = ((x >> 8) + 1) 2^-24 (word 0 of counter
 *     (b, j, 1, step)).  The emitted token is drawn by an exponential race over
 *     the vocabulary: Y = argmax_v w_v / E_v with one clock E_v = -ln U_v,
 *     U_v = ((x_v >> 8) + 1/2) 2^-24, per id, x_v = word v mod 4 of counter
 *     (b, v div 4, 3, step); the lowest id wins ties.  Outputs do not depend on
 *     how streams are batched or sharded.
 */
#ifndef DSPARK_VERIFY_H
#define DSPARK_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DSPARK_OK = 0,
  DSPARK_ERR_INVALID_ARG = 1, /* NULL required pointer, non-positive size, k > 32 ... */
  DSPARK_ERR_UNSUPPORTED = 2, /* valid but not implemented: rank R not in {32,64,128,256},
                                 W1/W2t not 16-byte aligned, or B > 4096 */
  DSPARK_ERR_WORKSPACE = 3,   /* workspace NULL, misaligned (256 B) or smaller than required */
  DSPARK_ERR_HIP = 4,         /* a HIP launch or device query failed */
  DSPARK_ERR_NO_MEMORY = 5,   /* a host allocation of the cost table failed */
  DSPARK_ERR_TOO_LARGE = 6    /* dspark_verify_noalloc: the problem's scratch exceeds
                                 DSPARK_NOALLOC_SCRATCH_BYTES */
} dspark_status;

typedef enum { DSPARK_F32 = 0, DSPARK_BF16 = 1 } dspark_dtype;

/*
 * Largest draft block the verify entry points accept.  The drafter the pages describe
 * is trained on blocks of 5 and is run with 3 to 9 drafts [P1 "The number to remember: five", §5, §6]; 32
 * leaves room above that while each stream's candidate rows fit one 32-bit mask and
 * its per-slot values fit fixed arrays in LDS.  Larger k returns DSPARK_ERR_INVALID_ARG.
 */
#define DSPARK_MAX_K 32

/*
 * One verify problem.  Shapes follow the pages' statement of the step: the
 * drafter proposes k tokens with their distributions, the target produces its
 * own distribution at every draft position plus one more, and the sampler keeps
 * a prefix and emits one target token [P1 §1 "One token per step"; P1 §4].
 */
typedef struct {
  int32_t B;                      /* streams, >= 1                                          */
  int32_t k;                      /* draft slots per stream, 1..32                           */
  int32_t V;                      /* vocabulary size, >= 1                                   */
  int32_t dtype;                  /* dspark_dtype of both logit tensors                      */
  const void* target_logits;      /* device [B, k+1, V]; row j is the target at slot j given
                                     x_<j, row gamma_b the bonus position                    */
  const void* draft_logits;       /* device [B, k, V]: raw drafter logits, before the bias   */
  const int32_t* draft_tokens;    /* device [B, k]: x_{b,j} in [0, V)                         */
  const int32_t* num_drafts;      /* device [B]: gamma_b in [0, k] (ragged verify: only rows
                                     0..gamma_b are read); NULL means gamma_b = k            */
  const float* temperature;       /* device [B], >= 0; NULL means 1.  T_b > 0: target logits
                                     and the biased draft logits are both divided by T_b.
                                     T_b = 0: the greedy branch (both entry points), see
                                     dspark_verify_tokenwise                                  */
  const uint16_t* W1;             /* device bf16 [V, R]: Markov factor rows, indexed by the
                                     previous token; NULL switches the bias off              */
  const uint16_t* W2t;            /* device bf16 [V, R]: W2t[v, r] = W2[r, v], the [R, V]
                                     factor stored as a linear layer keeps its weight        */
  const int32_t* anchor_tokens;   /* device [B]: token before slot 0 (the last accepted one);
                                     < 0 leaves slot 0 unbiased; NULL means all < 0         */
  int32_t R;                      /* Markov rank: 32, 64, 128 or 256 (ignored if W1 NULL)    */
  uint32_t step;                  /* Philox counter word: successive calls should differ    */
  uint64_t seed;                  /* Philox key                                             */
} dspark_verify_problem;

typedef struct {
  int32_t* accepted_len;          /* device [B]: drafts kept, s_b in [0, gamma_b]            */
  int32_t* out_tokens;            /* device [B, k+1]: x_0..x_{s-1}, Y, then -1               */
  double* diag;                   /* device [B, k+1, 5] or NULL: per slot j, (log p_j(x_j),
                                     log q_j(x_j), P_j, R_j, h_j); NaN where not computed    */
  void* const* stage_events;      /* NULL, or DSPARK_STAGES + 1 hipEvent_t the call records on
                                     `stream` before its first launch and after each stage
                                     (W1 tile packing, row statistics, scan, residual masses,
                                     sampler); NULL entries are skipped.  When the four
                                     verify stages run as one launch (see
                                     dspark_verify_launches), events 2..5 all follow that
                                     launch.  A timing hook: nothing is allocated           */
} dspark_verify_outputs;

/* Stages per verify call (see stage_events). */
#define DSPARK_STAGES 5

/* Launches a verify call of this problem makes on the current device: 2 (W1 tile
 * packing, then row statistics, scan, residual masses and sampler as phases of one
 * launch whose workgroups are all resident at once) or 5 (one launch per stage).
 * The choice depends on the sizes, the dtype, whether the Markov bias is on, the
 * 16-byte alignment of the two logit pointers, and the device's occupancy; setting
 * DSPARK_VERIFY_LAUNCH=separate in the environment forces 5.  Host only; reads no
 * device memory.  Errors: DSPARK_ERR_INVALID_ARG (invalid sizes, NULL out),
 * DSPARK_ERR_UNSUPPORTED (Markov rank not in {32, 64, 128, 256}), DSPARK_ERR_HIP
 * (device query failed). */
dspark_status dspark_verify_launches(const dspark_verify_problem* p, int32_t* launches);

/* Bytes of workspace the two verify entry points need for this problem (host, pure).
 * Returns 0 if the problem's sizes are invalid. */
size_t dspark_workspace_bytes(const dspark_verify_problem* problem);

/*
 * Streams with temperature 0 take the greedy branch in both verify entry points
 * [P1 §4 "Greedy is a different code path"]: draft j is kept iff it equals the
 * argmax of target row j (the first id among equal maxima); the emitted token is the
 * argmax at the first mismatch, or at the bonus position when every draft is kept.
 * Their diag entries are NaN (no probabilities are formed).
 *
 * Token-by-token verification (Leviathan et al.) [P1 §4 "Token by token"]:
 * draft j is kept iff u_{b,j} <= min(1, p_j(x_j) / q_j(x_j)); at the first
 * rejection t the emitted token is drawn from max(0, p_t - q_t) normalised, and
 * when every draft survives from the bonus position p_gamma.
 * q_j includes the Markov bias W1[prev_j] . W2 [P2 §6; P1 §3 "The Markov fix-up"],
 * prev_0 = anchor, prev_j = x_{j-1}.
 * workspace: device, >= dspark_workspace_bytes(problem), 256-byte aligned; its
 * contents need no initialisation and are scratch after the call.  It holds the
 * call's work counters: calls that may run at the same time (other streams) need
 * workspaces of their own; calls in order on one stream may share one.
 */
dspark_status dspark_verify_tokenwise(const dspark_verify_problem* problem,
                                      const dspark_verify_outputs* out,
                                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * Block verification (Sun et al.) [P1 §4 "Block verification", Figure 3]:
 * P_0 = 1, P_i = min(1, P_{i-1} r_{i-1}); R_i = sum_v max(0, P_i p_i(v) - q_i(v));
 * h_i = R_i / (R_i + 1 - P_i) (1 when P_i = 1), h_gamma = P_gamma; the kept length
 * is tau = the last i with u_{b,i-1} <= h_i (0 if none); the emitted token is drawn
 * from max(0, P_tau p_tau - q_tau) normalised, or from p_gamma when tau = gamma.
 * Same arguments and workspace rules as dspark_verify_tokenwise.
 */
dspark_status dspark_verify_block(const dspark_verify_problem* problem,
                                  const dspark_verify_outputs* out,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * Either verifier with no workspace argument and no allocation, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  method 0 = token-by-token (as
 * dspark_verify_tokenwise), 1 = block (as dspark_verify_block); same problem,
 * outputs, kernels and results.  The scratch is a static buffer of
 * DSPARK_NOALLOC_SCRATCH_BYTES per device, set aside when the library's device
 * code is loaded and held until the process ends; the problem must fit it
 * (dspark_workspace_bytes(problem) <= DSPARK_NOALLOC_SCRATCH_BYTES, else
 * DSPARK_ERR_TOO_LARGE and nothing is enqueued).  Every call on one device uses the
 * same buffer: calls that can overlap on one device (different streams) race and
 * give undefined results; calls in order on one stream are safe.  The buffer keeps
 * the last call's contents; each call clears what it needs cleared with a kernel
 * (no memset).  Calls hipMalloc, hipFree or any allocating routine: never.
 * Errors as dspark_verify_block, plus DSPARK_ERR_INVALID_ARG for another method.
 */
#define DSPARK_NOALLOC_SCRATCH_BYTES (32u << 20)
dspark_status dspark_verify_noalloc(const dspark_verify_problem* problem, const dspark_verify_outputs* out,
                                    int32_t method, void* stream);

/*
 * The drafter's walk with its Markov head [P2 §6 "Why the Markov Head Helps";
 * P1 §3 "The Markov fix-up", Figure 2]: for each stream b and slot j < gamma_b,
 *   x_j ~ softmax((d_j + W1[x_{j-1}] . W2) / T_b),   x_{-1} = anchor_tokens[b]
 * (anchor < 0 or W1 NULL: no bias at that slot), drawn with the exponential race
 * of the verifiers on Philox purpose 16 + j; T_b = 0 takes the largest biased
 * logit (first id among equal ones).  Uses from `problem`: B, k, V, dtype,
 * draft_logits [B, k, V], num_drafts (NULL = k), temperature, W1, W2t, R,
 * anchor_tokens, seed, step; target_logits and draft_tokens are ignored and may be
 * NULL.  tokens_out: device int32 [B, k], -1 past gamma_b; it may be passed as the
 * verify call's draft_tokens.  logq_out: device fp64 [B, k] of log q_j(x_j) (NaN for
 * T_b = 0 and past gamma_b), or NULL.  workspace: as dspark_workspace_bytes(problem);
 * as for the verifiers, calls that may overlap need workspaces of their own.
 * Slot j needs x_{j-1}: when the walk's workgroups (one per 256 ids) can all be
 * resident on the device, one launch runs every slot with grid-wide waits between
 * them and reads W2 once (a small launch first clears its wait words); otherwise 2k
 * launches, two per slot (see dspark_draft_launches).  Both give the same outputs.
 * A wait that expires (possible only if other work holds the device's compute units)
 * marks the slots from there on invalid: tokens -1, log q NaN.
 */
dspark_status dspark_draft_sample(const dspark_verify_problem* problem, int32_t* tokens_out,
                                  double* logq_out, void* workspace, size_t workspace_bytes,
                                  void* stream);

/* Launches dspark_draft_sample makes for this problem on the current device: 2 (wait
 * words cleared, then the one resident launch) or 2k.  The choice depends on V (at
 * most 512 groups of 256 ids on a 256-CU device), the Markov rank, the dtype, the
 * draft logits' 16-byte alignment and the device's occupancy; setting
 * DSPARK_WALK_LAUNCH=separate in the environment forces 2k.  Host only; reads no
 * device memory.  Errors: DSPARK_ERR_INVALID_ARG (invalid sizes, NULL draft logits
 * or out), DSPARK_ERR_UNSUPPORTED (Markov rank or alignment), DSPARK_ERR_HIP (device
 * query failed). */
dspark_status dspark_draft_launches(const dspark_verify_problem* problem, int32_t* launches);

/*
 * Reduced draft vocabulary [P1 §3 "The Markov fix-up": the drafter scores a reduced
 * vocabulary and scatters those logits into target-vocabulary columns]:
 *   out[r, vocab_ids[i]] = reduced[r, i],  out[r, v] = -inf for every other v,
 * so that q = 0 outside the drafter's vocabulary (the verifiers then keep the
 * target's mass there in the residual).  reduced: device [rows, K] of `dtype`;
 * vocab_ids: device int32 [K], distinct ids in [0, V) (others are dropped);
 * out: device [rows, V] of `dtype` (for example the draft_logits of a verify call,
 * rows = B k).  Two launches (fill, scatter).
 */
dspark_status dspark_draft_scatter(const void* reduced, const int32_t* vocab_ids, int32_t rows,
                                   int32_t K, int32_t V, int32_t dtype, void* out, void* stream);

/*
 * Draft count for a batch size [P1 §5: num_speculative_tokens_per_batch_size, a list
 * of (lowest batch, highest batch, drafts) triples]: the drafts of the first triple
 * whose range holds `batch`, else k_default.  Host only, pure; schedule: host
 * int32 [n][3] or NULL.
 */
int32_t dspark_k_for_batch(const int32_t* schedule, int32_t n, int32_t batch, int32_t k_default);

/*
 * DSpark Markov-head bias alone [P2 §6 "Why the Markov Head Helps"]:
 * out[i, v] = logits_in[i, v] + sum_r W1[prev_tokens[i], r] * W2t[v, r]  (fp32).
 * W1, W2t: device bf16 [V, R], R in {32, 64, 128, 256}.  prev_tokens: device
 * [rows]; an id outside [0, V) gives a zero bias row.  logits_in: device
 * [rows, V] of `dtype`, or NULL for zero.  out: device fp32 [rows, V].
 */
dspark_status dspark_markov_bias(const uint16_t* W1, const uint16_t* W2t, int32_t V, int32_t R,
                                 const int32_t* prev_tokens, int32_t rows,
                                 const void* logits_in, int32_t dtype, float* out, void* stream);

/*
 * Confidence head and adaptive verification count [P2 §7-9; P3 "The controller,
 * and the table it reads from"; P1 §6 "The arithmetic you need before tuning k"]:
 *   c_{b,j} = sigmoid(w . hidden[b, j, :] + bias)          (hidden -> Linear -> sigmoid)
 *   a_{b,j} = prod_{i<=j} c_{b,i}                           (prefix survival)
 *   n_b     = argmax_{n in 0..k} (1 + sum_{j<n} a_{b,j}) / verify_ms[n + 1]
 * with the smallest n on ties; verify_ms is indexed by the token count of one
 * stream's verify (n drafts + the target's own position).
 * hidden: device bf16 [B, k, H]; w: device bf16 [H]; verify_ms: HOST float
 * [n_ms], k + 2 <= n_ms <= 256, copied into the launch; n_out: device int32 [B];
 * c_out, a_out: device fp32 [B, k] or NULL.  n_out can be passed as num_drafts
 * of dspark_verify_block for ragged verification without a host round trip.
 */
dspark_status dspark_adaptive_k(const uint16_t* hidden, const uint16_t* w, float bias,
                                int32_t B, int32_t k, int32_t H,
                                const float* verify_ms, int32_t n_ms,
                                int32_t* n_out, float* c_out, float* a_out, void* stream);

/*
 * Batch-level draft scheduler [P2 §9 "Why It Is Called Prefix Survival
 * Probability": candidates are added greedily in descending prefix survival and
 * the low-confidence tail is cut once the expected accepted tokens stop paying;
 * P3 "The controller, and the table it reads from": the cost of a verify pass is
 * a table indexed by its token count].  With a_{b,j} = c_{b,0} ... c_{b,j}, the
 * (b, j) pairs are ranked by descending a, ties by j then b, so every leading part
 * of the ranking holds slots 0..n_b-1 of each stream b.  Taking the first m puts
 * B + m tokens in the verify batch (n_b drafts plus each stream's own target
 * position) and expects E(m) = B + the sum of their a.  The scheduler keeps the m
 * in [0, B k] with the largest E(m) / verify_ms[B + m] (the smallest m on ties) and
 * writes n_b, the count of stream b's slots among the first m.
 * Arithmetic: survivals are fp64 products, then ranked and summed as integer
 * multiples of 2^-40 (order-independent, exact sums), so the result is the fp64
 * definition's except where two survivals at the cut differ by less than 2^-40 (the
 * last draft may go to either stream) or two ratios differ by ~1e-12 relative.
 * c: device fp32 [B, k], values in [0, 1] (for example c_out of dspark_adaptive_k);
 * verify_ms: device fp32 [n_ms], positive, n_ms >= B (k + 1) + 1 (batch token
 * counts B .. B (k + 1) are read); n_out: device int32 [B] (usable as num_drafts
 * of dspark_verify_block); total_out: device int32 [1] = B + m, or NULL;
 * expected_out: device fp64 [1] = E(m), or NULL.  One launch of one workgroup;
 * B k > DSPARK_MAX_SCHEDULE returns DSPARK_ERR_UNSUPPORTED.
 */
#define DSPARK_MAX_SCHEDULE 4096
dspark_status dspark_schedule_batch(const float* c, int32_t B, int32_t k, const float* verify_ms, int32_t n_ms,
                                    int32_t* n_out, int32_t* total_out, double* expected_out, void* stream);

/*
 * Online verify-cost table [P3 "What we changed"].  The caller brackets each real
 * verify step with begin (which records a start event on `stream` and notes the
 * step's token count) and end (a stop event).  Completed pairs are read back
 * later, by poll or the next begin, without ever waiting on the GPU, and filed
 * under their token count; observe files a time measured elsewhere.  After every
 * `rebuild_every` filed observations the served table becomes the boot table
 * with, at each token count that holds at least `min_samples` of its last
 * `window` observations, their median (the mean of the two middle values for an
 * even count, rounded once to fp32).  An observation whose token count lies
 * outside [0, n) is dropped; so is a step begun while DSPARK_COST_EVENTS pairs
 * are still in flight.  Bracket only pure verify steps (drafts present, no
 * prompt prefill in the batch) so that prefill cost stays out of the curve.
 * The table is host state: create copies boot_ms (host fp32 [n], positive and
 * finite; 1 <= min_samples <= window, rebuild_every >= 1); the event pairs are
 * created on the current device at the first begin, and the table belongs to
 * that device.  Not thread-safe.  read copies the first n served entries to host
 * memory (upload them for dspark_schedule_batch or dspark_adaptive_k); stats
 * reports the filed, dropped and in-flight counts; log copies up to `cap` of the
 * first DSPARK_COST_LOG_MAX filed observations, in filing order, and returns how
 * many it copied.
 */
#define DSPARK_COST_EVENTS 64
#define DSPARK_COST_LOG_MAX 65536
typedef struct dspark_cost_table dspark_cost_table;
dspark_status dspark_cost_table_create(const float* boot_ms, int32_t n, int32_t window, int32_t min_samples,
                                       int32_t rebuild_every, dspark_cost_table** out);
void dspark_cost_table_destroy(dspark_cost_table* table);
dspark_status dspark_cost_table_begin(dspark_cost_table* table, int32_t num_tokens, void* stream);
dspark_status dspark_cost_table_end(dspark_cost_table* table, void* stream);
dspark_status dspark_cost_table_poll(dspark_cost_table* table, int32_t* filed);
dspark_status dspark_cost_table_observe(dspark_cost_table* table, int32_t num_tokens, float ms);
dspark_status dspark_cost_table_read(const dspark_cost_table* table, float* out, int32_t n);
dspark_status dspark_cost_table_stats(const dspark_cost_table* table, int64_t* filed, int64_t* dropped,
                                      int32_t* in_flight);
int32_t dspark_cost_table_log(const dspark_cost_table* table, int32_t* tokens, float* ms, int32_t cap);

/*
 * The random words behind a call, for replaying or auditing it (see the conventions
 * above): kind 0 writes word 0 of Philox counter (b, idx0 + i, purpose, step) for
 * i < n (purpose 1: the words of the accept uniforms u_{b,j}, j = idx0 + i); kind 1
 * writes word idx0 + i of the output stream of (b, purpose, step), i.e. word v mod 4
 * of counter (b, v div 4, purpose, step) for v = idx0 + i (purpose 3: the words of
 * the race clocks of the emitted token; 16 + j: slot j of the drafter's walk).
 * out: device uint32 [n].  One launch.
 */
dspark_status dspark_random_words(uint64_t seed, uint32_t b, uint32_t purpose, uint32_t step, uint32_t idx0,
                                  int32_t n, int32_t kind, uint32_t* out, void* stream);

/*
 * The Markov head's second factor in the layout the verify problem takes
 * [P2 §6 "Why the Markov Head Helps": the bias is W1[prev] times W2, W2 of shape
 * rank x vocabulary]: W2t[v, r] = W2[r, v].  W2: device bf16 [R, V] (row r holds
 * the rank-r weights of every id); W2t: device bf16 [V, R], distinct from W2 (no
 * in-place transpose); any R, V >= 1.  One launch; bit-exact (a copy).  Callers
 * whose W2 already sits as a linear layer's weight [V, R] pass it directly.
 * Errors: DSPARK_ERR_INVALID_ARG for NULL pointers, sizes < 1 or overlapping buffers.
 */
dspark_status dspark_w2_transpose(const uint16_t* W2, int32_t R, int32_t V, uint16_t* W2t, void* stream);

/* Static description of a status code. */
const char* dspark_status_string(dspark_status status);

#ifdef __cplusplus
}
#endif

#endif /* DSPARK_VERIFY_H */
