/* sv.h — batched lossless draft verification for speculative decoding on MI355X (gfx950).
 *
 * The operation ("From draft-then-verify to DSpark", section "How speculative decoding works"):
 * for every request b of a batch, the target model has scored k_b + 1 positions and the drafter
 * has proposed k_b tokens x_0..x_{k_b-1}, each drawn from the draft distribution q_i. With p_i
 * and q_i the softmaxes of the target and draft logits over the full vocabulary (both divided by
 * one temperature), draft x_i is kept iff u_i < min(1, p_i(x_i) / q_i(x_i)). The longest run of
 * kept drafts x_0..x_{n-1} is committed; at the first rejected slot n a token y is drawn from
 * max(0, p_n - q_n) renormalised; if all k_b drafts are kept, y is drawn from p_{k_b} (the "+1"
 * of the acceptance length in "Accelerating Large-Model Inference: Engineering Practice from
 * Hidden-State Extraction to DSpark Speculative Decoding", section 1). Greedy mode ("Bringing
 * DSpark to vLLM Metal") keeps drafts while x_i equals the target row's argmax and commits the
 * target argmax at the first mismatch (or at row k_b).
 *
 * Conventions shared by every entry point:
 *  - All array pointers are DEVICE pointers (hipMalloc / torch CUDA tensors on a ROCm build),
 *    owned by the caller. Arrays are row-major and contiguous. Nothing is allocated and nothing
 *    synchronises the host: work is enqueued on `stream` (a hipStream_t; NULL = the default
 *    stream) and outputs are valid once the stream has reached that point.
 *  - Return value: SV_OK, or a negative sv_status. Arguments are validated on the host before
 *    anything is enqueued; on a validation error nothing is launched and no output is written.
 *    SV_ERR_HIP reports a launch failure. sv_last_error() gives a message for the last failing
 *    call on the calling thread.
 *  - Limits: 1 <= B <= 1048576, 1 <= K <= 64, 1 <= V <= 67108864; a batch whose launch would
 *    need 2^24 or more work-groups (B * (2K+1) rows and more) returns SV_ERR_UNSUPPORTED.
 *  - Device-side preconditions are not checked (checking would cost a pass over the data):
 *    draft tokens of verified slots lie in [0, V) and every row that is read has at least one
 *    finite logit; NaN and +inf logits give undefined results. For memory safety a token outside
 *    [0, V) is treated as p(x) = q(x) = 0 (rejected; its target_prob is 0) and num_draft values
 *    are clamped to [0, K].
 *  - Rows a request does not verify (target rows past k_b, draft rows from k_b on) are never
 *    read, and may hold anything.
 *  - The workspace: at least sv_workspace_bytes(B, K, V) bytes, 256-byte aligned, owned by the
 *    caller. Within one call, work-groups hand per-chunk partial results to each other through
 *    it, each value stamped with a number drawn fresh for every call (the call counter, shared
 *    by every entry point of the process), so nothing needs clearing between calls, of any
 *    shape. The library zero-fills a workspace itself, on `stream` before the launch, on the
 *    first call that uses it after the call counter's low 32 bits last wrapped and on the first
 *    call it sees it at all (only the range [workspace, workspace + workspace_bytes) of that
 *    call, and again for a larger range later): a word left from before a wrap could carry a
 *    number that is handed out again. Memory that held other data since the library last used
 *    it as a workspace must be zeroed by the caller (hipMemset or torch.zeros) before it is
 *    passed again. One workspace must not be used by two calls that can run at the same time
 *    (e.g. on two streams). The stamp is fixed when the call is enqueued, so a call captured
 *    into a HIP graph must not be replayed: a replay would take the words of the one before
 *    for its own. sv_verify_batch_noalloc is the entry point whose captured calls replay
 *    correctly.
 *  - A work-group waiting for partials from other work-groups of the same call gives up after a
 *    bounded time (about two seconds) and then stores -2 in that request's accepted_len. This
 *    does not happen in normal operation.
 */
#ifndef SV_H_
#define SV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SV_OK = 0,
  SV_ERR_INVALID_ARG = -1, /* a size, pointer, dtype or temperature is out of range */
  SV_ERR_UNSUPPORTED = -2, /* a valid request the library does not handle */
  SV_ERR_WORKSPACE = -3,   /* workspace missing, misaligned or smaller than required */
  SV_ERR_HIP = -4          /* the HIP runtime refused a launch */
} sv_status;

typedef enum {
  SV_DTYPE_F32 = 0, /* IEEE float32 logits */
  SV_DTYPE_BF16 = 1 /* bfloat16 logits (the upper 16 bits of a float32) */
} sv_dtype;

/* Bytes of device workspace that sv_verify_batch and sv_verify_greedy need for a batch of
 * shape (B, K, V); 0 if the shape is outside the limits. Host-only, no GPU call. */
size_t sv_workspace_bytes(int B, int K, int V);

/* Static text for a status code. */
const char* sv_status_string(int status);

/* Message describing the last failing call made on this thread ("" if none). */
const char* sv_last_error(void);

/* Sampling-mode verification ("From draft-then-verify to DSpark", "How speculative decoding
 * works": the min(1, p/q) acceptance test, the longest accepted prefix, the residual draw from
 * max(0, p - q), and the extra draw from the target when every draft is kept).
 *
 *  target_logits     [B, K+1, V] dtype   target scores of the K+1 positions of each request
 *  draft_logits      [B, K,   V] dtype   the draft logits each draft token was drawn from
 *  dtype             sv_dtype of both logit arrays
 *  temperature       > 0, finite; both p and q are softmax(logits / temperature)
 *  draft_tokens      [B, K] int32        proposals x_i
 *  num_draft         [B] int32 or NULL   k_b, drafts to verify per request (NULL: all K)
 *  uniforms          [B, K] float32      u_i in [0, 1): slot i is kept iff u_i < min(1, p/q)
 *  residual_uniform  [B] float32         r in [0, 1): drives the residual draw or the extra draw
 *                                        (inverse CDF in ascending vocabulary order: the token
 *                                        is the smallest v with sum_{j<=v} w_j > r * sum_j w_j)
 *  accepted_len      [B] int32 out       n = number of kept drafts, 0..k_b
 *  committed         [B, K+1] int32 out  x_0..x_{n-1}, y, then -1 padding
 *  target_prob       [B, K] float32 out  p_i(x_i) for i < k_b, 0 for i >= k_b
 *  draft_prob        [B, K] float32 out or NULL: q_i(x_i) for i < k_b, 0 for i >= k_b
 *  workspace, workspace_bytes            scratch, see above
 *  stream                                hipStream_t
 */
int sv_verify_batch(const void* target_logits, const void* draft_logits, int dtype, int B, int K,
                    int V, float temperature, const int32_t* draft_tokens,
                    const int32_t* num_draft, const float* uniforms,
                    const float* residual_uniform, int32_t* accepted_len, int32_t* committed,
                    float* target_prob, float* draft_prob, void* workspace,
                    size_t workspace_bytes, void* stream);

/* sv_verify_batch without a workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc). The
 * arguments and outputs are those of sv_verify_batch, run by the same kernels; the scratch memory
 * is a 16 MiB array the library holds on each GPU it runs on (from the first call on that GPU until
 * the process ends), whose device address it looks up once per device. Nothing is allocated: no
 * hipMalloc, hipFree or allocating library routine is called. The call runs on the current device
 * (`stream` must belong to it). Every call on one GPU shares that GPU's array, which keeps the last
 * call's words: calls that can overlap on one GPU (two streams, two host threads) race and give
 * undefined results; serialise them. Each call first zero-fills the part of the array it uses (a
 * kernel on `stream`, no memset) and its work-groups hand values to each other under one fixed
 * tag, so nothing depends on host state that changes from call to call: a call captured into a
 * HIP graph gives correct results on every replay (replays, like calls, must not overlap).
 * Returns what sv_verify_batch returns, or SV_ERR_UNSUPPORTED (nothing launched) when the batch
 * needs more than 16 MiB of scratch (sv_workspace_bytes(B, K, V) > 16777216), or SV_ERR_HIP when
 * the array's address cannot be obtained. */
int sv_verify_batch_noalloc(const void* target_logits, const void* draft_logits, int dtype, int B,
                            int K, int V, float temperature, const int32_t* draft_tokens,
                            const int32_t* num_draft, const float* uniforms,
                            const float* residual_uniform, int32_t* accepted_len,
                            int32_t* committed, float* target_prob, float* draft_prob,
                            void* stream);

/* Greedy-mode verification ("Bringing DSpark to vLLM Metal": greedy serving whose output ids
 * equal target-only greedy decoding). g_i = argmax_v target_logits[b, i, v] compared on the
 * stored values, lowest index on ties. n = first i < k_b with x_i != g_i, else k_b.
 *
 *  target_logits  [B, K+1, V] dtype;  draft_tokens [B, K] int32;  num_draft [B] int32 or NULL
 *  accepted_len   [B] int32 out: n;   committed [B, K+1] int32 out: x_0..x_{n-1}, g_n, -1...
 *  Draft logits are not needed: the proposals already are the drafter's greedy choices.
 */
int sv_verify_greedy(const void* target_logits, int dtype, int B, int K, int V,
                     const int32_t* draft_tokens, const int32_t* num_draft,
                     int32_t* accepted_len, int32_t* committed, void* workspace,
                     size_t workspace_bytes, void* stream);

/* Flattened, mixed-mode verification. The per-request verify lengths of one batch packed
 * without padding, each request's rows found through its start index ("flatten every token and
 * track its request ID", DSpark paper review 4.2.2), and greedy and sampling requests in one
 * launch, each sampling request at its own temperature (the vLLM Metal article serves greedy
 * requests only and lists sampled verification as in flight).
 *
 * Request b (0 <= b < B) verifies k_b = num_draft[b] drafts with
 *   target rows  target_logits[target_row_start[b] + i], i = 0..k_b         (k_b + 1 rows)
 *   draft rows   draft_logits[draft_row_start[b] + i],   i = 0..k_b - 1     (k_b rows)
 * temperature[b] == 0: a greedy request, exactly as sv_verify_greedy on its target rows (its
 *   draft rows, uniforms and residual uniform are not read; its probabilities are written 0);
 * temperature[b] >= log2(e) / 2^21 and finite: a sampling request, exactly as sv_verify_batch
 *   with that temperature on its rows.
 * A request is invalid when k_b is outside [0, K], its temperature is negative, not finite or
 * in (0, log2(e)/2^21), its target rows leave [0, n_target_rows), or (sampling, k_b > 0) its
 * draft rows leave [0, n_draft_rows). Nothing of an invalid request is read; it reports
 * accepted_len -3, committed all -1 and probabilities 0. The others are unaffected.
 *
 *  target_logits     [n_target_rows, V] dtype, device       draft_logits [n_draft_rows, V] dtype,
 *                    (NULL allowed when n_draft_rows == 0)
 *  target_row_start, draft_row_start, num_draft  [B] int32, device
 *  temperature       [B] float, device
 *  draft_tokens [B, K] int32, uniforms [B, K] float, residual_uniform [B] float (device; entries
 *  past k_b unused); outputs as sv_verify_batch (accepted_len [B], committed [B, K+1],
 *  target_prob [B, K], draft_prob [B, K] or NULL). K is the largest k_b the call allows.
 *  workspace  sv_workspace_bytes(B, K, V) bytes, as sv_verify_batch.
 * Rows may appear in any order and need not be contiguous per request beyond each request's own
 * run; rows no request uses are never read.
 * Returns SV_OK, SV_ERR_INVALID_ARG (B, K, V, dtype, a NULL required pointer, n_target_rows < 1,
 * n_draft_rows < 0, or draft_logits NULL with n_draft_rows > 0; nothing launched),
 * SV_ERR_UNSUPPORTED, SV_ERR_WORKSPACE or SV_ERR_HIP, as sv_verify_batch.
 */
int sv_verify_ragged(const void* target_logits, const void* draft_logits, int dtype, int B,
                     int K, int V, int64_t n_target_rows, int64_t n_draft_rows,
                     const int32_t* target_row_start, const int32_t* draft_row_start,
                     const int32_t* num_draft, const float* temperature,
                     const int32_t* draft_tokens, const float* uniforms,
                     const float* residual_uniform, int32_t* accepted_len, int32_t* committed,
                     float* target_prob, float* draft_prob, void* workspace,
                     size_t workspace_bytes, void* stream);

/* Confidence-scheduled prefix selection ("DSpark" paper review, 4.2.1 Confidence Head and
 * 4.2.2 Hardware-Aware Prefix Scheduler): how many draft tokens of each request to verify.
 * Prefix survival s[b][k] = c[b][0] * ... * c[b][k] (confidences clamped to [0, 1], NaN = 0,
 * float32 products left to right).
 *  step_time != NULL (hardware-aware): all B*K draft tokens are ranked by survival (ties: earlier
 *    position, then lower request); N = 0 .. B*K is chosen to maximise
 *    (B + sum of the first N ranked survivals) / step_time[B + N]   (fp64 sums; the smallest N
 *    among equal rates; entries that are not finite and positive are skipped), and request b
 *    verifies its tokens among the first N (always a prefix).
 *  step_time == NULL (threshold): request b verifies its drafts up to the first confidence below
 *    `threshold`.
 *
 *  confidence        [B, K] float, device
 *  step_time         [T] float, device: time of a target step that verifies n tokens, n < T;
 *                    T >= B + B*K + 1. The units are the caller's.
 *  num_draft         [B] int32 out (device): k_b
 *  target_row_start  [B] int32 out or NULL: exclusive sums of k_b + 1 (flattened target rows)
 *  draft_row_start   [B] int32 out or NULL: exclusive sums of k_b (flattened draft rows)
 *  summary           [2] float out or NULL: N chosen, and its expected tokens per unit time
 *                    (0, 0 in threshold mode; -1, 0 if the finishing work-group's bounded wait
 *                    for the ranking work-groups ran out, which leaves every k_b = 0)
 *  workspace         hardware-aware mode: device memory of at least
 *                    sv_schedule_workspace_bytes(B, K) bytes, 8-byte aligned (the ranking
 *                    work-groups' results, tagged words as for the verify calls; reusable
 *                    across calls and shapes on one stream, shared with the verify calls'
 *                    workspaces). Threshold mode: may be NULL.
 *  Limits: 1 <= K <= 64, B*K <= 4096. Hardware-aware mode: ceil(B*K / 8) ranking work-groups
 *  and one finishing work-group, last in the grid (no token order is
 *  materialised: each token's rank and the survival sum before it come from a binary search in
 *  every request's block, whose survivals never increase); threshold mode: one work-group.
 *  Asynchronous on `stream`.
 * Returns SV_OK, SV_ERR_INVALID_ARG or SV_ERR_WORKSPACE (nothing launched) or SV_ERR_HIP.
 */
size_t sv_schedule_workspace_bytes(int B, int K);
int sv_schedule_prefix(const float* confidence, int B, int K, const float* step_time, int T,
                       float threshold, int32_t* num_draft, int32_t* target_row_start,
                       int32_t* draft_row_start, float* summary, void* workspace,
                       size_t workspace_bytes, void* stream);

/* Markov-head correction of a parallel draft block ("Accelerating Large-Model Inference ...",
 * section 3, Markov Head; DSpark paper review 4.1): left to right over positions k = 0..K-1,
 *   corrected[b][k][v] = base[b][k][v] + sum_j L[prev][j] * Rf[v][j],
 *   prev = anchor[b] for k = 0 (no bias when anchor is NULL or outside [0, V)), else the token
 *   chosen at k-1;  token[b][k] = argmax_v corrected[b][k][v] (lowest index on ties).
 * The bias is a dense contraction over the rank on the matrix cores (bf16 factors, fp32
 * accumulation); the corrected logits are the block's draft logits for verification.
 *
 *  base_logits   [B, K, V] dtype (SV_DTYPE_F32 / SV_DTYPE_BF16), device
 *  left_factor   [V, R] bf16 bits (uint16), device, 16-byte aligned: row = previous token
 *  right_factor  [V, R] bf16 bits, device, 16-byte aligned: row = candidate token
 *  R             rank, a multiple of 16 in [16, 1024] (256 in the pages)
 *  anchor        [B] int32 device or NULL
 *  draft_tokens  [B, K] int32 out; draft_logits [B, K, V] dtype out or NULL (bf16 rounds to
 *                nearest even)
 *  workspace     sv_markov_workspace_bytes(B, V) bytes, 256-byte aligned, device, owned by the
 *                caller, no clearing needed between calls of any of the library's functions:
 *                every one-launch call takes 2K + 2 consecutive numbers of the process's call
 *                counter and zero-fills the workspace as described for sv_verify_batch, also
 *                when the per-position form or sv_markov_topk left untagged words in it since.
 * With B <= 64 and R <= 256, and when every vocabulary tile fits the registers of a resident
 * work-group (at most five tiles of 64 entries each; V = 151936 on 256 compute units fits), one
 * cooperative launch does all K positions: each work-group keeps the right-factor rows of its
 * tiles in registers from the first position to the last, a position runs as two stages
 * (requests 0..31, then 32..63) so that one half's token hand-off overlaps the other half's
 * tiles, and the work-groups hand the tokens to each other through tagged words in the
 * workspace. The cooperative launch makes the runtime place every work-group at once or refuse
 * the launch; a refused launch falls back to the per-position form below. Waits are bounded at
 * about 2 s all the same (a token that could not be formed is reported as -2 at that position
 * and after). With 64 < B <= 128 (same conditions otherwise), one such launch per block of 64
 * requests, in turn. Otherwise 2K launches (a bias-and-argmax launch and a finishing launch per
 * position). All on `stream`. Returns SV_OK, SV_ERR_INVALID_ARG, SV_ERR_WORKSPACE,
 * SV_ERR_UNSUPPORTED or SV_ERR_HIP; nothing is launched unless SV_OK.
 */
size_t sv_markov_workspace_bytes(int B, int V);
int sv_markov_draft(const void* base_logits, int dtype, int B, int K, int V,
                    const uint16_t* left_factor, const uint16_t* right_factor, int R,
                    const int32_t* anchor, int32_t* draft_tokens, void* draft_logits,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Sampled Markov-head drafting (DSpark paper review, 4.1 Semi-autoregressive generation: the head
 * samples each position's token and biases the next position with the sample; "Accelerating
 * Large-Model Inference ...", section 3, evaluation at temperature 1.0). The correction is that
 * of sv_markov_draft; the token of position k of request b (tau = temperature[b]):
 *   tau == 0: argmax_v corrected[b][k][v], exactly as sv_markov_draft;
 *   tau >= log2(e) / 2^21 and finite: a draw from softmax(d[b][k] / tau), d = the draft_logits
 *     row as stored (bf16: the rounded values, so the draw follows the q row a verifier reads),
 *     by inverse CDF in ascending vocabulary order with u = uniforms[b][k] clamped to [0, 1]
 *     (NaN as 0): the first v whose running mass passes u * (row mass); entries that are NaN or
 *     -inf have no mass; when the row's largest value is +inf only its +inf entries have mass;
 *     a row without mass gives token 0;
 *   any other tau: token -3 at every position (its later positions then get no bias).
 * The drawn token is prev for position k + 1.
 *
 *  base_logits, left_factor, right_factor, R, anchor, draft_tokens as sv_markov_draft
 *  temperature   [B] float, device
 *  uniforms      [B, K] float, device
 *  draft_logits  [B, K, V] dtype out, device, required (the draws read the stored rows back)
 *  workspace     sv_markov_workspace_bytes(B, V) bytes, as sv_markov_draft
 * Under the one-launch conditions of sv_markov_draft (R <= 256, every vocabulary tile in a
 * resident work-group), one cooperative launch per block of 64 requests, in turn (a refused
 * launch falls back to the per-position form below); within a launch the
 * work-groups also hand off each draw: the request's finishing work-group finds which
 * work-group's share of the distribution holds the target, and that work-group finds the token
 * in the entries it wrote (waits bounded as in sv_markov_draft: token -2 when one gives up).
 * Otherwise 2K launches: sv_markov_draft's per-position tile launch, then a finishing launch
 * that draws each request's token from its stored row. All on `stream`. Returns SV_OK,
 * SV_ERR_INVALID_ARG, SV_ERR_WORKSPACE, SV_ERR_UNSUPPORTED or SV_ERR_HIP; nothing is launched
 * unless SV_OK.
 */
int sv_markov_draft_sampled(const void* base_logits, int dtype, int B, int K, int V,
                            const uint16_t* left_factor, const uint16_t* right_factor, int R,
                            const int32_t* anchor, const float* temperature,
                            const float* uniforms, int32_t* draft_tokens, void* draft_logits,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Top-K Markov drafting ("Bringing DSpark to vLLM Metal", Making the draft cheaper): per draft
 * position the candidates are the kc largest base logits (NaN below every number, ties to the
 * lower index), and the Markov correction of sv_markov_draft is applied to those rows only:
 *   z[b][k][j] = base[b][k][c_j] + L[prev] . Rf[c_j],   c = the position's candidates in
 *   ascending vocabulary order, prev = the anchor at k = 0 (no bias when NULL or outside
 *   [0, V)), else the token chosen at k-1;  token = the c_j with the largest z (lowest index on
 *   ties). With kc = V this is sv_markov_draft restricted to its tokens.
 *
 *  base_logits   [B, K, V] dtype, device; left_factor, right_factor [V, R] bf16, 16-byte aligned
 *  R             a multiple of 16 in [16, 256];  kc  candidates, 1 <= kc <= min(64, V)
 *  anchor        [B] int32 device or NULL
 *  draft_tokens  [B, K] int32 out;  candidates [B, K, kc] int32 out or NULL (ascending index)
 *  cand_logits   [B, K, kc] float out or NULL: the corrected logits z of the candidates
 *  workspace     sv_markov_topk_workspace_bytes(B, K, V) bytes, 256-byte aligned, device; no
 *                clearing needed (left holding intermediate tables, not tagged words; a later
 *                call of another function on the same memory zero-fills it first)
 * Four launches on `stream`. Returns SV_OK, SV_ERR_INVALID_ARG, SV_ERR_UNSUPPORTED (more than
 * 2048 chunk candidates per row: ceil(V / 16384) * kc; 524288 entries at kc = 64),
 * SV_ERR_WORKSPACE or SV_ERR_HIP; nothing is launched unless SV_OK.
 */
size_t sv_markov_topk_workspace_bytes(int B, int K, int V);
int sv_markov_topk(const void* base_logits, int dtype, int B, int K, int V,
                   const uint16_t* left_factor, const uint16_t* right_factor, int R, int kc,
                   const int32_t* anchor, int32_t* draft_tokens, int32_t* candidates,
                   float* cand_logits, void* workspace, size_t workspace_bytes, void* stream);

/* Read probe (a measurement aid, not a step of the method): the plainest stream over a device
 * buffer, so that the row stream can be compared with the read bandwidth this device reaches.
 * `groups` work-groups of 256 threads read every 16-byte word of data[0, bytes) once with
 * non-temporal loads, group g a contiguous 1/groups of the words; group g writes the wrapping
 * 32-bit sum of its words to partial[g].
 *
 *  data     device pointer, 16-byte aligned; bytes a multiple of 16 (0 is allowed)
 *  partial  device pointer, [groups] uint32 out, owned by the caller
 *  groups   1 .. 2^20
 *  stream   hipStream_t (NULL = default stream); the call is asynchronous
 * Returns SV_OK, SV_ERR_INVALID_ARG (nothing launched) or SV_ERR_HIP.
 */
int sv_read_probe(const void* data, size_t bytes, uint32_t* partial, int groups, void* stream);

/* Test aid, not a step of the method: sets the process-wide call counter from which every call
 * draws the numbers that stamp its workspace words (see the workspace convention above), so that
 * a test can cross a wrap of its low 32 bits without 2^32 calls. Not for use while calls are
 * being enqueued on another thread. */
void sv_set_call_counter(uint64_t value);

#ifdef __cplusplus
}
#endif

#endif /* SV_H_ */
