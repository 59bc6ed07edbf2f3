/*
 * specverify: speculative-decoding draft verification on AMD Instinct MI355X
 * (gfx950).  C ABI over caller-owned device buffers.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensor pointers are DEVICE pointers owned by the caller, contiguous and
 *   row-major with the vocabulary innermost: a [B, N, V] tensor holds row
 *   (b, j) at element offset (b * N + j) * V.  Element alignment is required;
 *   16-byte alignment of rows is not (unaligned rows take a slower load path).
 * - B = requests, D = draft tokens per request (0 <= D <= 16), N = D + 1
 *   verified positions, V = vocabulary size (1 <= V < 2^31).
 * - dtype: SPECVERIFY_F32 (float) or SPECVERIFY_BF16 (bfloat16 bit patterns).
 * - req_index: optional device array of n_req batch rows to process; outputs
 *   are written at those rows and other rows are left untouched.  NULL means
 *   every row, and then n_req must equal B.  0 <= n_req <= B.  An index
 *   outside [0, B) is skipped on the device.  Listing a row twice makes two
 *   workgroups write identical values to it.
 * - Per-request parameters (temperature, top_k, top_p, seed, offset) are
 *   device arrays of length B indexed by batch row.
 * - Temperature below 1e-5 (compared in double precision) means greedy: a
 *   one-hot at the lowest-index maximum.  The page "TensorRT-LLM
 *   _torch/speculative/interface.py", _sample_sharded_temperature, keeps rows
 *   below the greedy threshold greedy; the threshold value is not on the
 *   pages, 1e-5 is this library's.
 * - Random numbers: Philox4x32-10 (Salmon et al., SC'11) with key = seed and
 *   counter = (block index lo, hi, subsequence lo, hi); word t of a stream is
 *   lane t % 4 of block t / 4; a word w maps to the uniform
 *   u = (2 * (w >> 9) + 1) * 2^-24.  The per-request offset names the
 *   request's own subsequence ("TensorRT-LLM interface.py",
 *   rejection_sampling_one_model docstring).
 * - stream is a hipStream_t passed as void*; NULL is the default stream.
 *   Calls are asynchronous; nothing is read back to the host.  The library
 *   never synchronises and never allocates device memory: every call uses
 *   only its arguments (chain rejection, greedy verify, Gumbel sampling
 *   and the fused verify take an optional caller-owned workspace; see there).
 * - Host-side validation runs before any HIP call.  Return codes:
 *   SPECVERIFY_OK, SPECVERIFY_INVALID_ARGUMENT (nothing launched),
 *   SPECVERIFY_UNSUPPORTED (current device is not gfx950),
 *   SPECVERIFY_HIP_ERROR (launch failed; see specverify_last_error()).
 * - Outputs are written completely for every processed request, including the
 *   -1 padding, so callers need not pre-fill them.
 * - Non-finite inputs never cause out-of-bounds access or a hang; the tokens
 *   they produce are unspecified except where stated.
 * - A request's outputs depend only on its own inputs and (seed, offset), not
 *   on its batch position, B, req_index order or the stream.
 */
#ifndef SPECVERIFY_H_
#define SPECVERIFY_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPECVERIFY_OK 0
#define SPECVERIFY_INVALID_ARGUMENT 1
#define SPECVERIFY_UNSUPPORTED 2
#define SPECVERIFY_HIP_ERROR 3

#define SPECVERIFY_F32 0
#define SPECVERIFY_BF16 1

#define SPECVERIFY_MAX_DRAFT 16
#define SPECVERIFY_STATIC_SCRATCH_BYTES (4 << 20)
#define SPECVERIFY_RNG_SLOT_SPAN 32
#define SPECVERIFY_VERSION 202

/*
 * Temperature softmax followed by top-k then top-p renormalisation.
 *
 * Passage: "tokenspeed sampling/backends/flashinfer.py",
 * FlashInferSamplingBackend.verify -- softmax(logits, temperature) and then
 * top_k_renorm_prob followed by top_p_renorm_prob (the fused kernel replaces
 * that pair); per-row knobs are shared by a request's N positions.
 *
 * logits      [B, npos, V] dtype          input
 * temperature [B] float                   T; T < 1e-5 gives a one-hot at the argmax
 * top_k       [B] int32 or NULL           0 < k < V keeps every value >= the
 *                                         k-th largest (ties kept); else off
 * top_p       [B] float or NULL           top_p < 1 keeps the smallest set of
 *                                         largest values whose mass reaches
 *                                         top_p times the top-k mass (ties at
 *                                         the threshold kept); else off
 * probs_out   [B, npos, V] float          output: w_v / sum of kept w, 0 elsewhere,
 *                                         w_v = exp((z_v - max z) / T)
 * Selection compares logits, never rounded probabilities.  npos >= 1.
 */
int specverify_softmax_renorm(const void* logits, int dtype, int64_t B, int64_t npos, int64_t V,
                              const float* temperature, const int32_t* top_k, const float* top_p,
                              const int32_t* req_index, int64_t n_req, float* probs_out,
                              void* stream);

/*
 * Chain rejection sampling of a linear draft.
 *
 * Passage: "TensorRT-LLM _torch/speculative/interface.py",
 * rejection_sampling_one_model -- draft probs [batch, D, vocab] float32,
 * draft ids [batch, D] int32, target probs [batch, D+1, vocab] float32,
 * per-request Philox seed/offset; returns the accepted draft tokens, the
 * corrected or bonus token, then -1.
 *
 * draft_probs     [B, D, V] float   q, or NULL: target-only verify (below)
 * draft_ids       [B, D] int32      x (may be NULL when D == 0)
 * target_probs    [B, D+1, V] float p
 * seed, offset    [B] uint64        Philox key and subsequence of each request
 * accepted_tokens [B, D+1] int32    output: x_0..x_{L-1}, y, then -1
 * accept_length   [B] int32         output: L in [0, D] (the request emits L+1 tokens)
 *
 * Rule: u_i = uniform of word i (i < D), u_f = uniform of word D.  For i = 0..D-1,
 * accept x_i iff u_i * q_i(x_i) < p_i(x_i) (exact double product); a draft id
 * outside [0, V) is rejected.  At the first rejection i, y is drawn from
 * r = max(0, p_i - q_i); when all D are accepted, y is drawn from r = p_D.
 * The draw is y = min{ j : sum_{v<=j} r_v > u_f * R }, R = sum r, with
 * double-precision sums in ascending index order; an empty r falls back to
 * the target row, and an all-zero target row to floor(u_f * V).
 *
 * Target-only verify (draft_probs NULL, D > 0): "tokenspeed
 * sampling/backends/flashinfer.py", FlashInferSamplingBackend.verify, passes
 * the chain kernel draft tokens without draft probabilities, with acceptance
 * thresholds; this is the thresholds-of-one case: q_i is the point mass at
 * x_i (the zero row for an id outside [0, V)), so x_i is accepted iff
 * u_i < p_i(x_i), and the correction is drawn from p_i with x_i weighing
 * max(0, p_i(x_i) - 1).
 *
 * workspace, workspace_bytes
 *                 caller-owned device memory, or NULL when
 *                 specverify_chain_workspace_bytes(n_req, V) is 0 (then
 *                 workspace_bytes is ignored).  Small batches split each
 *                 request's row over several workgroups, which hand their
 *                 partial sums over through it: one 32-bit counter per request
 *                 (padded to 256 bytes), then one double per 1024 vocabulary
 *                 entries per request.  8-byte aligned, at least the queried
 *                 size.  It must be all zero when a call starts, and every
 *                 call leaves the bytes it used zero, so zero a new
 *                 workspace once (any fill) and reuse it for any later chain
 *                 call it is large enough for; calls that share a workspace
 *                 must not run concurrently (issue them on one stream).  A missing,
 *                 short or misaligned workspace returns
 *                 SPECVERIFY_INVALID_ARGUMENT with nothing launched.  The
 *                 pages ask for the same: "tokenspeed flashinfer.py",
 *                 FlashInferSamplingBackend.__init__, keeps persistent buffers
 *                 and allocates nothing per step; "TensorRT-LLM interface.py"
 *                 checks its rejection buffers on the host so the step can be
 *                 captured in a graph.
 */
int specverify_chain_reject(const float* draft_probs, const int32_t* draft_ids,
                            const float* target_probs, const uint64_t* seed,
                            const uint64_t* offset, int64_t B, int64_t D, int64_t V,
                            const int32_t* req_index, int64_t n_req, int32_t* accepted_tokens,
                            int32_t* accept_length, void* workspace, int64_t workspace_bytes,
                            void* stream);

/*
 * Chain rejection with no workspace argument and no allocation, for callers
 * that cannot allocate device memory or pass one: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * Arguments, results and errors are those of specverify_chain_reject without
 * workspace / workspace_bytes.  Split launches use the library's static
 * scratch instead: one array of SPECVERIFY_STATIC_SCRATCH_BYTES (4 MiB) per
 * device, held until the process ends.  A call whose workspace size
 * (specverify_chain_workspace_bytes) exceeds it returns
 * SPECVERIFY_INVALID_ARGUMENT with nothing launched; calls that need none
 * (n_req >= 256, V <= 262144) never touch it.  The first call on a device
 * resolves the array's address and clears it with a fill kernel on that
 * call's stream; every call returns the bytes it used to zero.  All calls on
 * a device share its array, so calls that overlap in time on one device
 * (different streams, or different host threads without ordering) race on
 * it and give undefined results: issue them on one stream.  Calls no
 * hipMalloc, hipFree or hipMemset.
 */
int specverify_chain_reject_noalloc(const float* draft_probs, const int32_t* draft_ids,
                                    const float* target_probs, const uint64_t* seed,
                                    const uint64_t* offset, int64_t B, int64_t D, int64_t V,
                                    const int32_t* req_index, int64_t n_req, int32_t* accepted_tokens,
                                    int32_t* accept_length, void* stream);

/*
 * Workspace size of specverify_chain_reject / specverify_chain_reject_ragged.
 *
 * *bytes = the workspace a call with n_req processed requests over V
 * vocabulary entries needs: 0 when every request's row is handled by one
 * workgroup that keeps its chunk sums on chip (n_req >= 256 and
 * V <= 262144), else the size described at specverify_chain_reject.
 * Depends on (n_req, V) only.  Host-only: touches no device.
 * n_req >= 0, 1 <= V < 2^31, bytes non-NULL; else SPECVERIFY_INVALID_ARGUMENT.
 */
int specverify_chain_workspace_bytes(int64_t n_req, int64_t V, int64_t* bytes);

/*
 * Ragged chain rejection: each request verifies its own number of positions.
 *
 * Passage: "TensorRT-LLM _torch/speculative/interface.py", SpecMetadata
 * (verify_lens, qo_indptr: request r owns packed rows [qo_indptr[r],
 * qo_indptr[r+1])) and the ragged branch of the one-model sampler: target rows
 * are scattered to the padded [B, D+1, V] layout, padding rows of target and
 * draft are one-hot at token 0 (missing draft ids are 0), the chain verify
 * runs on the rectangle, and the emitted count is clamped to verify_lens.
 *
 * draft_probs     [B, D, V] float32 or NULL (point-mass drafts, as in
 *                 specverify_chain_reject); rows at positions >= len_b - 1 are
 *                 not read.  With t2d: [B, D, Vd], rows over a smaller draft
 *                 vocabulary
 * t2d, Vd         NULL, or the inverse table of specverify_d2t_inverse [V]
 *                 int32 and the draft vocabulary size: target entry v of a
 *                 draft row is draft_probs[..., t2d[v]] (0 where t2d[v] is
 *                 outside [0, Vd)), exactly the row specverify_d2t_expand
 *                 would write, without writing it; needs draft_probs
 * draft_ids       [B, D] int32; entries at positions >= len_b - 1 are not read
 * target_probs    [n_rows, V] float32, packed rows
 * qo_indptr       [B+1] int32, request b's rows are [qo_indptr[b], qo_indptr[b+1]),
 *                 len_b = their count, 1 <= len_b <= D+1
 * seed, offset, B, D, V, req_index, n_req, stream: as in specverify_chain_reject
 * accepted_tokens [B, D+1] int32    output: x_0..x_{L-1}, y, then -1
 * accept_length   [B] int32         output: L in [0, len_b - 1]
 *
 * With d = len_b - 1, positions i < d verify as in specverify_chain_reject.
 * Position d drafts token 0 as a point mass: if u_d < p_d(0) the request
 * emits x_0..x_{d-1}, 0 (L = d); if it rejects there, y is drawn from p_d with
 * token 0 removed.  Together these sample p_d (the page's argument for its
 * padding).  When len_b = D+1 the request is verified exactly as by
 * specverify_chain_reject.  A request whose length is outside [1, D+1] or
 * whose rows fall outside [0, n_rows) gets accept_length -1 and all tokens
 * -1; nothing of it is read.  workspace, workspace_bytes: as in
 * specverify_chain_reject (sized by specverify_chain_workspace_bytes(n_req, V)).
 */
int specverify_chain_reject_ragged(const float* draft_probs, const int32_t* t2d, int64_t Vd,
                                   const int32_t* draft_ids, const float* target_probs,
                                   const int32_t* qo_indptr, int64_t n_rows, const uint64_t* seed,
                                   const uint64_t* offset, int64_t B, int64_t D, int64_t V,
                                   const int32_t* req_index, int64_t n_req, int32_t* accepted_tokens,
                                   int32_t* accept_length, void* workspace, int64_t workspace_bytes,
                                   void* stream);

/*
 * Draft -> target vocabulary placement of draft distributions.
 *
 * Passage: "TensorRT-LLM _torch/speculative/interface.py", one-model sampler
 * (draft vocabulary smaller than the target's): draft entry s belongs to
 * target entry (s + d2t[s]) mod V, an index list computed once and kept in
 * the speculative metadata, and the draft probabilities are scattered into a
 * zero-filled full-vocabulary row; without a d2t table they fill the first
 * Vd entries.  The result is the draft_probs argument of specverify_chain_reject
 * / specverify_chain_reject_ragged (draft ids are target-vocabulary ids).
 *
 * specverify_d2t_inverse builds, once per table, the inverse map
 *   d2t  [Vd] int64 offsets or NULL; draft entry s belongs to target entry
 *        (s + d2t[s]) mod V, a floor modulus (negative offsets wrap)
 *   t2d  [V] int32 output: the draft entry of each target entry, -1 for none
 * Vd <= V (a larger draft vocabulary cannot map one-to-one; INVALID_ARGUMENT).
 * The page's scatter assumes distinct draft entries land on distinct
 * targets; when several share a target, the highest-numbered draft entry is
 * the one kept (what a scatter in ascending draft order leaves), independent
 * of thread timing.
 *
 * specverify_d2t_expand places the rows (a gather: every output row is
 * written once, in order)
 *   draft_probs      [rows, Vd] float32 (rows = B * D)
 *   t2d              [V] int32 from specverify_d2t_inverse
 *   full_draft_probs [rows, V] float32 output: entry t = draft_probs[t2d[t]],
 *                    0 where t2d[t] is outside [0, Vd)
 * Neither call uses a workspace.
 */
int specverify_d2t_inverse(const int64_t* d2t, int64_t Vd, int64_t V, int32_t* t2d, void* stream);
int specverify_d2t_expand(const float* draft_probs, const int32_t* t2d, int64_t rows, int64_t Vd, int64_t V,
                          float* full_draft_probs, void* stream);

/*
 * Single-step sampling: one token per request from its logits row.
 *
 * Passage: "tokenspeed sampling/backends/flashinfer.py", sample -- all-greedy
 * batches take the row argmax; otherwise softmax(logits, temperature) and
 * top_k_top_p_sampling_from_probs(probs, top_k, top_p, filter_apply_order=
 * "joint", seed, offset, deterministic=True).  Min-p: "TensorRT-LLM
 * _torch/speculative/interface.py" passes per-request min_ps to its fused
 * sampler.
 *
 * logits      [B, V] float32 or bf16 (dtype), V <= 524288
 * temperature [B] float32; below 1e-5 the row takes its lowest-index argmax
 * top_k       [B] int32 or NULL (off); top_p [B] float32 or NULL (1, off);
 * min_p       [B] float32 or NULL (0, off)
 * seed, offset [B] uint64: the request's Philox stream; the draw uses word 0
 * tokens      [B] int32 output
 *
 * Joint filter: top-k keeps every value >= the k-th largest (ties kept; off
 * for k <= 0 or k >= V); top-p keeps the smallest set of largest values whose
 * mass reaches top_p of the WHOLE row's mass (ties kept; active iff
 * top_p < 1); both judge the unfiltered row, and a token is kept when it
 * passes both.  Min-p keeps (z - max z) >= T ln(min(min_p, 1)), compared on
 * logits in double precision (active iff min_p > 0), i.e. p >= min_p * p_max.
 * The token is y = min{ j : sum_{v<=j} p'_v > u * R } over the kept,
 * renormalised probabilities p' (double sums in ascending index order), u
 * the uniform of word 0.  No workspace.
 */
int specverify_sample(const void* logits, int dtype, const float* temperature, const int32_t* top_k,
                      const float* top_p, const float* min_p, const uint64_t* seed, const uint64_t* offset,
                      int64_t B, int64_t V, const int32_t* req_index, int64_t n_req, int32_t* tokens,
                      void* stream);

/*
 * Greedy chain verify.
 *
 * Passage: "tokenspeed sampling/backends/flashinfer.py",
 * FlashInferSamplingBackend.verify, all-greedy branch -- target tokens are the
 * row argmax, then verify_chain_greedy writes predict, accept_index (pre-filled
 * with -1) and the accept length; ties go to the lowest index ("TensorRT-LLM
 * interface.py", the draft sampler's key-exchange comments).
 *
 * target_logits   [B, D+1, V] dtype
 * draft_ids       [B, D] int32 (may be NULL when D == 0)
 * accepted_tokens [B, D+1] int32   output: y_0..y_L then -1
 * accept_length   [B] int32        output: L = leading draft ids equal to y
 * predict         [B, D+1] int32 or NULL   output: y_j for j <= L else -1
 * accept_index    [B, D+1] int32 or NULL   output: b*(D+1)+j for j <= L else -1
 *                                          (flat index into predict)
 * argmax_out      [B, D+1] int32 or NULL   output: y_j for every j; requesting
 *                                          it makes every row be read
 * workspace, workspace_bytes
 *                 caller-owned device memory (8-byte aligned) of at least
 *                 specverify_greedy_verify_workspace_bytes(n_req, D) bytes,
 *                 or NULL.  With it every (request, row) gets a workgroup of
 *                 its own, and a row whose request already failed at an
 *                 earlier row stops reading; without it one workgroup per
 *                 request walks its rows in order.  The results are the same.
 *                 Its contents must be zero before the first call and are
 *                 left zero by every call; calls that share one workspace
 *                 must not overlap in time (same stream, or ordered).
 * Rows after the first mismatch are not needed unless argmax_out is given
 * (then every row is read).  Equal values (including -0 and +0) tie; a NaN
 * counts as the maximum, and the first NaN wins.
 */
int specverify_greedy_verify(const void* target_logits, int dtype, const int32_t* draft_ids,
                             int64_t B, int64_t D, int64_t V, const int32_t* req_index,
                             int64_t n_req, int32_t* accepted_tokens, int32_t* accept_length,
                             int32_t* predict, int32_t* accept_index, int32_t* argmax_out,
                             void* workspace, int64_t workspace_bytes, void* stream);

/*
 * Workspace bytes specverify_greedy_verify can use for n_req requests with D
 * drafts (0: it uses none).  *bytes = 0 when D == 0 or n_req == 0, else
 * 128 * n_req (one 128-byte line per request) rounded up to 256.  Host-only.
 */
int specverify_greedy_verify_workspace_bytes(int64_t n_req, int64_t D, int64_t* bytes);

/*
 * Temperature-only target sampling by Gumbel-max, then strict chain acceptance.
 *
 * Passage: "TensorRT-LLM _torch/speculative/interface.py",
 * _sample_sharded_temperature (Gumbel-max is an exact temperature sample; rows
 * below the greedy threshold stay greedy) and
 * _sample_and_accept_draft_tokens_base (strict acceptance counts the leading
 * draft tokens equal to the target's).
 *
 * target_logits   [B, D+1, V] dtype
 * temperature     [B] float
 * draft_ids       [B, D] int32 (may be NULL when D == 0)
 * seed, offset    [B] uint64
 * accepted_tokens [B, D+1] int32   output: y_0..y_L then -1
 * accept_length   [B] int32        output: L
 * sampled_out     [B, D+1] int32 or NULL   output: y_j for every j (all rows read)
 *
 * Row j of request b: s_v = z_v / T + G_v, G_v = -ln(-ln u_v), u_v the uniform
 * of word v of stream (seed_b, offset_b + 32 j); y_j = lowest-index argmax of
 * s, computed in float.  The stream spacing of 32 per row follows the page's
 * _RNG_SLOT_SPAN.  Rows after the first mismatch are not needed unless
 * sampled_out is given (then every row is read).
 *
 * workspace, workspace_bytes
 *                 as for specverify_greedy_verify, sized by
 *                 specverify_gumbel_sample_workspace_bytes(n_req, D).  Without
 *                 sampled_out, row 0 of every request is sampled first and
 *                 only the requests whose row 0 matched its draft go on, their
 *                 later rows cut into pieces over all compute units; with it,
 *                 every (request, row) gets a workgroup.  The results are the
 *                 same in every form.
 */
int specverify_gumbel_sample(const void* target_logits, int dtype, const float* temperature,
                             const int32_t* draft_ids, const uint64_t* seed,
                             const uint64_t* offset, int64_t B, int64_t D, int64_t V,
                             const int32_t* req_index, int64_t n_req, int32_t* accepted_tokens,
                             int32_t* accept_length, int32_t* sampled_out, void* workspace,
                             int64_t workspace_bytes, void* stream);

/*
 * Workspace bytes specverify_gumbel_sample can use (0: it uses none): 0 when
 * D == 0 or n_req == 0, else 128 * n_req (one line per request) + 256 +
 * 128 * n_req * D (one line per later row, for its pieces), rounded up to
 * 256.  Host-only.
 */
int specverify_gumbel_sample_workspace_bytes(int64_t n_req, int64_t D, int64_t* bytes);

/*
 * Fused verify: target rows from logits, then chain rejection, in one call.
 *
 * Passage: "tokenspeed sampling/backends/flashinfer.py",
 * FlashInferSamplingBackend.verify -- the target probabilities are the
 * temperature softmax followed by top-k and then top-p renormalisation, and
 * the chain verify consumes them; the page's aim of keeping the verify hot
 * path to two kernels and "TensorRT-LLM" fused sampling ops motivate one
 * launch that never writes the probabilities.
 *
 * target_logits   [B, D+1, V] dtype
 * temperature     [B] float; top_k [B] int32 or NULL; top_p [B] float or NULL
 *                 (the meanings of specverify_softmax_renorm)
 * draft_probs     [B, D, V] float (may be NULL when D == 0)
 * draft_ids       [B, D] int32 (may be NULL when D == 0)
 * seed, offset    [B] uint64
 * accepted_tokens [B, D+1] int32   output
 * accept_length   [B] int32        output
 *
 * workspace, workspace_bytes
 *                 caller-owned device memory or NULL.  With it (D > 0) every
 *                 (request, target row) gets a workgroup of its own, rows
 *                 dispatched in row order: when all rows fit on the device's
 *                 compute units at once every row is evaluated, otherwise a
 *                 row after one that already ended its request's chain is
 *                 skipped.  It takes
 *                 specverify_verify_fused_workspace_bytes(n_req, D) bytes
 *                 (one 128-byte line per request where the rows meet;
 *                 8-byte aligned, all zero when a call starts; every call
 *                 leaves it zero, so zero it once and reuse it; calls sharing
 *                 it must not overlap).  With NULL, one workgroup per request
 *                 evaluates its rows in order instead (same results).  A
 *                 short or misaligned workspace returns
 *                 SPECVERIFY_INVALID_ARGUMENT.
 *
 * Equivalent to specverify_softmax_renorm on the logits followed by
 * specverify_chain_reject on its output (same tokens whenever that output
 * buffer is 16-byte aligned, except draws within the double-rounding band of
 * a CDF boundary, whose sums may associate differently).  Requests evaluated
 * row by row read logit rows 0..L only; no probability is stored.
 * V <= 524288.
 */
int specverify_verify_fused(const void* target_logits, int dtype, const float* temperature,
                            const int32_t* top_k, const float* top_p, const float* draft_probs,
                            const int32_t* draft_ids, const uint64_t* seed, const uint64_t* offset,
                            int64_t B, int64_t D, int64_t V, const int32_t* req_index,
                            int64_t n_req, int32_t* accepted_tokens, int32_t* accept_length,
                            void* workspace, int64_t workspace_bytes, void* stream);

/*
 * Workspace size of specverify_verify_fused: 128 bytes per request, rounded
 * up to 256, when D > 0 and n_req > 0; else 0 (no workspace used).
 * Host-only.  n_req >= 0, 0 <= D <= 16, bytes non-NULL; else
 * SPECVERIFY_INVALID_ARGUMENT.
 */
int specverify_verify_fused_workspace_bytes(int64_t n_req, int64_t D, int64_t* bytes);

/* Human-readable name of a status code (static string). */
const char* specverify_status_string(int status);

/* Message describing the last failure on the calling thread ("" if none). */
const char* specverify_last_error(void);

/* SPECVERIFY_VERSION of the built library. */
int specverify_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H_ */
