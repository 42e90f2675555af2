/*
 * spec_verify.h -- C ABI of the MI355X (gfx950) batched speculative-sampling
 * verify step.
 *
 * What one call computes, per sequence b (definitions as on the pages):
 *   - p_j = processed target distribution at position j (0 <= j <= gamma_b),
 *     q_i = processed draft distribution at position i (0 <= i < gamma_b).
 *     "Processed" = temperature, then top-k, then top-p, then normalise: the
 *     sampling adjustments are applied to both models before the test
 *     ("Fast Inference from Transformers via Speculative Decoding", mtandhj.com
 *     summary, "Speculative Sampling: theoretical basis"; the Leviathan review,
 *     "Method / Overview": argmax, top-k, nucleus and temperature are all
 *     standard sampling from an adjusted distribution).  Temperature 0 is
 *     argmax (all mass on the largest logit, lowest id on ties).
 *   - Draft x_i is accepted while u_i < min(1, p_i(x_i)/q_i(x_i)), evaluated
 *     division-free as u_i * q_i(x_i) < p_i(x_i); n = number accepted before
 *     the first rejection (Leviathan review, Algorithm 1, step 3; llm-compass,
 *     section 4, speculative_step).
 *   - If n < gamma_b the extra token is drawn from norm(max(0, p_n - q_n)),
 *     else from p_{gamma_b} (the bonus token) (Algorithm 1, steps 4-5; "the
 *     art of guessing well", section "Speculative sampling", where the draft
 *     distribution after the last draft is taken as zero).  The draw is an
 *     inverse CDF over ascending vocabulary id with the residual/bonus uniform
 *     ("the art of guessing well", section "Sampling with shared noise",
 *     textbook method): token = min{v : C(v) > u * Z}.
 *   - alpha_i = sum_v min(p_i(v), q_i(v)) for every draft position
 *     (mtandhj summary, "How to choose gamma"; "the art of guessing well",
 *     "Speculative sampling").
 *
 * Conventions for every entry point:
 *   - Device pointers are HIP device allocations owned by the caller; the
 *     library keeps no reference after the call returns and allocates no
 *     device memory.  All arrays are dense and row-major.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *     and runs asynchronously: there is no host synchronisation and no
 *     device-to-host copy.  Outputs are valid once the stream reaches them.
 *   - Argument errors are reported synchronously by a negative return code
 *     before anything is enqueued.  Bad *data* (NaN or +inf logits, a row of
 *     only -inf, a draft token outside [0, V), gamma_len outside
 *     [1, gamma_max], a negative or NaN temperature, a NaN top_p, a uniform
 *     outside [0, 1)) is reported per sequence: n_accepted = -1, every token
 *     -1, alpha and pq NaN.
 *   - Calls that share one workspace must be ordered (same stream or
 *     synchronised); distinct workspaces make calls independent.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Logit storage types. */
enum { SV_BF16 = 0, SV_FP32 = 1 };

/* Return codes. */
enum {
  SV_OK = 0,
  SV_ERR_ARG = -1,          /* null pointer, bad size, misaligned base      */
  SV_ERR_UNSUPPORTED = -2,  /* unknown dtype, V or gamma_max beyond limits  */
  SV_ERR_WORKSPACE = -3,    /* workspace missing or smaller than required  */
  SV_ERR_HIP = -4,          /* a HIP call failed (see spec_verify_strerror) */
  SV_ERR_SCRATCH = -5       /* spec_verify_noalloc: the call's workspace exceeds its fixed buffer */
};

/* Limits (checked synchronously). */
#define SV_MAX_GAMMA 64      /* gamma_max <= 64: one wavefront ballot spans all drafts */
#define SV_MAX_VOCAB 1048576 /* V <= 2^20                                            */
#define SV_MAX_CANDIDATES 64 /* K <= 64 candidate sequences (multi-candidate verify)  */

/*
 * Bytes of device workspace that spec_verify needs for these sizes
 * (0 for invalid sizes).  The workspace holds per-row candidate lists,
 * per-row statistics and completion counters.
 */
size_t spec_verify_workspace_bytes(int B, int gamma_max, int V, int dtype);

/*
 * Prepare a workspace for its first use: clears the completion counters
 * (enqueued on `stream`).  Every successful spec_verify call leaves the
 * counters cleared again, so this is needed once per allocation.
 * Returns SV_OK or a negative code.
 */
int spec_verify_workspace_init(void* workspace, size_t workspace_bytes, int B, int gamma_max, int V,
                               int dtype, void* stream);

/*
 * The batched verify step.
 *
 *  p_logits     [B][gamma_max+1][V] target logits (bf16 bit patterns or fp32), 16-byte aligned.
 *  q_logits     [B][gamma_max][V]   draft logits, same dtype, 16-byte aligned.
 *  dtype        SV_BF16 or SV_FP32.
 *  draft_tokens [B][gamma_max] int32: x_1..x_gamma_b; slots beyond gamma_b are ignored.
 *  gamma_len    [B] int32 per-sequence gamma_b in [1, gamma_max], or NULL (all gamma_max).
 *               Target rows beyond gamma_b and draft rows at or beyond gamma_b are never read.
 *  uniforms     [B][gamma_max+1] float in [0, 1): u[b][i] (i < gamma_b) tests draft i;
 *               u[b][gamma_max] drives the residual or bonus draw.
 *  temperature  [B] float, >= 0; 0 selects exact argmax matching (uniforms and filters unused).
 *  top_k        [B] int32 or NULL; k <= 0 or k >= V means no top-k.  Keeps every logit
 *               >= the k-th largest (ties kept).
 *  top_p        [B] float or NULL; top_p >= 1 means no top-p.  Applied after top-k: keeps every
 *               value >= t*, the largest value whose mass at-or-above reaches top_p (ties kept).
 *  B, gamma_max, V  sizes; B >= 0 (B == 0 is a no-op), 1 <= gamma_max <= SV_MAX_GAMMA,
 *               1 <= V <= SV_MAX_VOCAB.
 *  out_tokens   [B][gamma_max+1] int32: x_1..x_n, then the drawn token, then -1 padding.
 *  out_n_accepted [B] int32: n, or -1 for an invalid sequence.
 *  out_alpha    [B][gamma_max] float: alpha_i for i < gamma_b, 0 in padded slots.
 *  out_pq       [B][gamma_max][2] float or NULL: (p_i(x_i), q_i(x_i)) for i < gamma_b, 0 beyond.
 *  workspace    device buffer of at least spec_verify_workspace_bytes(...) bytes, 256-byte
 *               aligned, prepared once with spec_verify_workspace_init.
 *  stream       hipStream_t to enqueue on (NULL = default stream).
 *
 * Returns SV_OK, or a negative code (nothing enqueued).
 */
int spec_verify(const void* p_logits, const void* q_logits, int dtype,
                const int32_t* draft_tokens, const int32_t* gamma_len, const float* uniforms,
                const float* temperature, const int32_t* top_k, const float* top_p,
                int B, int gamma_max, int V,
                int32_t* out_tokens, int32_t* out_n_accepted, float* out_alpha, float* out_pq,
                void* workspace, size_t workspace_bytes, void* stream);

/* Hints for spec_verify_ex (bit flags). */
enum {
  SV_HINT_NO_DENSE = 1,  /* the caller knows that every sequence has T == 0 or 0 < top_k <= 512:
                            the per-(sequence, position) kernel for dense sequences is not
                            launched.  A dense sequence in such a call still gets its exact
                            result, from a slower one-workgroup-per-sequence path.            */
  SV_HINT_ALL_DENSE = 2, /* the caller knows that every sequence is dense (T > 0 and top_k <= 0,
                            top_k >= V or top_k > 512): the top-k selection kernel, whose only
                            work would be listing the (sequence, position) pairs, is not
                            launched, and the pair kernel takes them in a fixed order.  A
                            sequence that is not dense still gets its exact result, from the
                            same slower path.  Ignored where the pair kernel does not apply
                            (rows beyond its size limits).  Combined with SV_HINT_NO_DENSE:
                            SV_ERR_ARG.                                                        */
  SV_HINT_UNFILTERED = 4 /* the caller knows that no sequence has top-k or top-p (top_k <= 0 or
                            >= V, top_p >= 1, or NULL): when rows are longer than 64 KB, 16-byte
                            aligned, and the call has at most 512 (sequence, position) pairs,
                            each dense pair's rows are split into chunks over several
                            workgroups (three launches that exchange per-chunk maxima,
                            normalisers and weight sums through the workspace) instead of one
                            workgroup per pair: the latency of small batches with large
                            vocabularies.  When rows are at most 4 KB and 16-byte aligned, the
                            dense pairs' rows stay in registers with no LDS copy, so more pairs
                            run at once.  A sequence that does have top-k or top-p still gets
                            its exact result, from the slower one-workgroup-per-sequence path. */
};

/*
 * spec_verify with lenience (the Leviathan review, section "Lenience"): the
 * acceptance test multiplies q(x) by l in [0, 1], accept iff u * l * q(x) < p(x).
 * No token is then output with more than 1/l times its target probability;
 * alpha (the acceptance rate) rises as l falls; l = 1 is spec_verify exactly.
 * The residual stays max(0, p - q) (the page changes only the acceptance
 * decision).  out_alpha still reports the overlap sum min(p, q).
 *
 *  lenience     [B] float in [0, 1], or NULL (all 1).  A value outside [0, 1] or NaN
 *               makes that sequence invalid.
 *  hints        0 or SV_HINT_* flags (unknown bits, or SV_HINT_NO_DENSE with
 *               SV_HINT_ALL_DENSE: SV_ERR_ARG).
 * Every other argument, the workspace and the error behaviour are those of
 * spec_verify.
 */
int spec_verify_ex(const void* p_logits, const void* q_logits, int dtype,
                   const int32_t* draft_tokens, const int32_t* gamma_len, const float* uniforms,
                   const float* temperature, const int32_t* top_k, const float* top_p, const float* lenience,
                   int hints, int B, int gamma_max, int V,
                   int32_t* out_tokens, int32_t* out_n_accepted, float* out_alpha, float* out_pq,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * spec_verify_ex for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * It takes no workspace.  Its workspace is a fixed device array of
 * SV_NOALLOC_SCRATCH_BYTES inside the library, one copy per GPU, held from the
 * first call on that GPU until the process ends; the call itself allocates
 * nothing (no hipMalloc, no allocating library routine).
 *
 *  Arguments, outputs and data-error behaviour: those of spec_verify_ex, minus
 *  `workspace` and `workspace_bytes`.  The inputs and outputs are still the
 *  caller's device buffers.
 *  SV_ERR_SCRATCH (nothing enqueued) when spec_verify_workspace_bytes(B,
 *  gamma_max, V, dtype) exceeds SV_NOALLOC_SCRATCH_BYTES; the other codes as
 *  for spec_verify_ex.
 *
 * Every call on one GPU uses that GPU's one array: calls that overlap on one
 * GPU (different streams or host threads without ordering between them) race
 * and give undefined results.  Calls ordered on one stream are safe.  Each
 * call clears the counters it needs with a small fill kernel on `stream`, so
 * no preparation call exists or is needed.
 */
#define SV_NOALLOC_SCRATCH_BYTES (64u << 20) /* 64 MiB per GPU */

int spec_verify_noalloc(const void* p_logits, const void* q_logits, int dtype,
                        const int32_t* draft_tokens, const int32_t* gamma_len, const float* uniforms,
                        const float* temperature, const int32_t* top_k, const float* top_p, const float* lenience,
                        int hints, int B, int gamma_max, int V,
                        int32_t* out_tokens, int32_t* out_n_accepted, float* out_alpha, float* out_pq,
                        void* stream);

/*
 * Sampling one token per row from its processed distribution (the drafter's
 * step before a verify, x ~ q after temperature / top-k / top-p: "Fast
 * Inference from Transformers via Speculative Decoding", mtandhj.com summary,
 * "Speculative Sampling: theoretical basis"), by the inverse CDF over
 * ascending vocabulary id at the row's uniform ("Speculative Decoding: the art
 * of guessing well", "Sampling with shared noise", textbook method):
 * token = min{v : C(v) > u * Z}.  T = 0 is argmax (lowest id on ties).
 *
 *  logits       [R][V] bf16 bit patterns or fp32.
 *  uniforms     [R] float in [0, 1).
 *  temperature, top_k, top_p: [R] as for spec_verify (top_k / top_p may be NULL).
 *  out_tokens   [R] int32: the sampled token, or -1 for an invalid row (NaN / +inf
 *               logits, no finite logit, bad temperature or top_p, bad uniform).
 *  workspace    device buffer of spec_sample_workspace_bytes(R, V, dtype) bytes,
 *               256-byte aligned, prepared once with spec_sample_workspace_init.
 * Asynchronous on `stream`, allocates nothing.  Returns SV_OK or a negative code.
 */
size_t spec_sample_workspace_bytes(int R, int V, int dtype);
int spec_sample_workspace_init(void* workspace, size_t workspace_bytes, int R, int V, int dtype, void* stream);
int spec_sample(const void* logits, int dtype, const float* uniforms, const float* temperature,
                const int32_t* top_k, const float* top_p, int R, int V, int32_t* out_tokens,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * The shared-noise drafter's step ("Speculative Decoding: the art of guessing
 * well", section "Sampling with shared noise"): per row, the Gumbel-max sample
 * argmax_i(log q(i) + g_i) over the processed distribution, scored as
 * fl(z + fl(T * g)) without fused multiply-add, lowest id on ties; T = 0 is
 * argmax of z.  With the drafter's logits and the noise vectors later given to
 * spec_verify_gumbel, these are the drafts that the verify compares against.
 *
 *  logits       [R][V] bf16 or fp32;  noise [R][V] float.
 *  temperature, top_k, top_p: [R] as for spec_verify (top_k / top_p may be NULL).
 *  out_tokens   [R] int32: the sample, or -1 for an invalid row (as for
 *               spec_verify_gumbel).
 *  workspace    spec_verify_gumbel_workspace_bytes(R, 0, V, dtype) bytes, 256-byte
 *               aligned, prepared once with spec_verify_gumbel_workspace_init(.., R, 0, ..).
 * Asynchronous on `stream`.  Returns SV_OK or a negative code.
 */
int spec_sample_gumbel(const void* logits, int dtype, const float* noise, const float* temperature,
                       const int32_t* top_k, const float* top_p, int R, int V, int32_t* out_tokens,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Verify with shared Gumbel noise (Gumbel coupling; "Speculative Decoding: the
 * art of guessing well", section "Sampling with shared noise").  The drafter
 * proposed x_k = argmax_i(log q_k(i) + g_k,i) with the same noise vectors g_k
 * that the target uses here; the target's own sample at position k is
 * t_k = argmax_i(log p_k(i) + g_k,i) over its processed distribution p_k
 * (temperature, top-k, top-p as for spec_verify).  The verify keeps the longest
 * prefix with x_k == t_k and appends t at the first disagreement (t after the
 * last draft when all agree): exact matching, drafter-independent output.
 * The score is formed in float32 as fl(z + fl(T * g)) with no fused
 * multiply-add (the argmax of log p + g, multiplied by T > 0); ties go to the
 * lowest id; T = 0 is argmax of z and the noise is not read.
 *
 *  p_logits     [B][gamma_max+1][V] target logits (bf16 bit patterns or fp32).
 *  noise        [B][gamma_max+1][V] float Gumbel noise, one vector per position
 *               (the same vectors the drafter used).  NaN or infinite noise on the
 *               processed support of a used row (T > 0) makes the sequence invalid.
 *  draft_tokens [B][gamma_max] int32 proposals; slots beyond gamma_b ignored.
 *  gamma_len, temperature, top_k, top_p: as for spec_verify (uniforms are not used).
 *  out_tokens   [B][gamma_max+1] int32: x_1..x_n, then t_n, then -1 padding.
 *  out_n_accepted [B] int32: n, or -1 for an invalid sequence.
 *  out_target   [B][gamma_max+1] int32: t_k for k <= gamma_b, -1 beyond (and for an
 *               invalid sequence).
 *  workspace    spec_verify_gumbel_workspace_bytes(B, gamma_max, V, dtype) bytes,
 *               256-byte aligned, prepared once with spec_verify_gumbel_workspace_init
 *               (every successful call leaves it prepared again).
 * Argmax and top-k (<= 512) sequences are streamed once by the select kernel and
 * the noise is read only at their kept ids; other sequences stream logits and
 * noise.  Only noise on the processed support is used, and only there does a NaN
 * or infinite value make the sequence invalid.
 *
 * Invalid data (as for spec_verify, plus bad noise) is reported per sequence with
 * n = -1 and tokens -1.  Base pointers must be aligned to their element size;
 * 16-byte alignment and V a multiple of 8 (bf16) or 4 (fp32) take the vector
 * path.  Asynchronous on `stream`; allocates nothing.  Returns SV_OK or a
 * negative code (nothing enqueued).
 */
int spec_verify_gumbel(const void* p_logits, int dtype, const float* noise, const int32_t* draft_tokens,
                       const int32_t* gamma_len, const float* temperature, const int32_t* top_k,
                       const float* top_p, int B, int gamma_max, int V, int32_t* out_tokens,
                       int32_t* out_n_accepted, int32_t* out_target, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * spec_verify_gumbel with call hints (same section of the same page).
 *
 *  hints        0, SV_HINT_ALL_DENSE or SV_HINT_NO_DENSE.
 *               SV_HINT_ALL_DENSE: the caller knows that every sequence has T > 0 and
 *               no top-k of at most 512.  The select and list launches, whose only
 *               work is on argmax and small-top-k sequences, are skipped, and the
 *               per-(sequence, position) kernel takes every sequence: one that breaks
 *               the promise still gets its exact result there.
 *               SV_HINT_NO_DENSE: the caller knows that every sequence has T == 0 or
 *               0 < top_k <= 512.  The call is two launches: the list kernel also
 *               finishes every sequence, and takes a sequence that breaks the promise
 *               (or whose lists overflowed) row by row with one workgroup, with the
 *               same exact result.
 *               Both bits, or any other bit: SV_ERR_ARG.
 * Every other argument, the workspace and the error behaviour are those of
 * spec_verify_gumbel.
 */
int spec_verify_gumbel_ex(const void* p_logits, int dtype, const float* noise, const int32_t* draft_tokens,
                          const int32_t* gamma_len, const float* temperature, const int32_t* top_k,
                          const float* top_p, int hints, int B, int gamma_max, int V, int32_t* out_tokens,
                          int32_t* out_n_accepted, int32_t* out_target, void* workspace,
                          size_t workspace_bytes, void* stream);

/* Workspace of spec_verify_gumbel (and, with gamma_max = 0 and B = R rows, of
 * spec_sample_gumbel): its size (0 for invalid sizes) and its one-time
 * preparation on `stream`.  Returns SV_OK or a negative code. */
size_t spec_verify_gumbel_workspace_bytes(int B, int gamma_max, int V, int dtype);
int spec_verify_gumbel_workspace_init(void* workspace, size_t workspace_bytes, int B, int gamma_max, int V,
                                      int dtype, void* stream);

/*
 * Multi-candidate verify: K-SEQ at each depth and the SpecTr walk ("SpecTr:
 * Fast Speculative Decoding via Optimal Transport", mtandhj.com, sections
 * "K-SEQ", "Residual distribution", "SpecTr"; that page calls the draft p and
 * the target q, here p is the target and q the draft).  K candidate sequences
 * of length L were drawn from the drafter (repeats allowed).  At depth j the
 * candidates are the j-th tokens of the sequences that agree with the output
 * so far, k of them; with a(x) = min(1, p(x) / (rho* q(x))), where rho* is the
 * smallest rho in [1, k] with rho beta(rho) >= 1 - (1 - beta(rho))^k and
 * beta(rho) = sum_x min(q(x), p(x) / rho), they are tested in order (accept
 * iff u < a); if all are rejected the output is drawn from the residual
 * max(0, p(x) - (P_A / beta) min(q(x), p(x) / rho*)), P_A = 1 - (1 - beta)^k, by
 * the inverse CDF over ascending id (p itself when beta = 0).  The output
 * follows the target exactly.  The round continues while the output is one of
 * the candidates and ends with a draw from the target after depth L.
 *
 *  p_logits     [B][K][L+1][V] target logits: row j of candidate c is the target
 *               after c's first j tokens (rows of candidates with a common prefix
 *               are read from the lowest-numbered one).
 *  q_logits     [B][K][L][V] draft logits, same layout.
 *  candidates   [B][K][L] int32 candidate tokens.
 *  uniforms     [B][L+1][K+1] float in [0, 1): at depth j < L, u[j][i] tests the
 *               i-th candidate (i < k) and u[j][k] drives the residual draw; u[L][0]
 *               drives the draw after depth L.
 *  temperature, top_k, top_p: [B] as for spec_verify (top_k / top_p may be NULL).
 *  out_tokens   [B][L+1] int32: the outputs, out_tokens[b][0..n] valid, -1 after.
 *  out_n        [B] int32: depths whose output was a candidate (0..L); -1 invalid.
 *  out_node_tokens [B][K][L+1] int32: the output at the node of candidate c's
 *               prefix of length j, for each class's lowest-numbered candidate (-1
 *               elsewhere); a node whose class is a single candidate is computed
 *               only if the walk reaches it (-3 otherwise).  Also the call's
 *               scratch: no workspace (out_n holds each sequence's pending
 *               single-candidate chain between the call's launches).
 * 1 <= K <= SV_MAX_CANDIDATES, 1 <= L <= SV_MAX_GAMMA.  Rows above 64 KB are read
 * from global memory on each pass and may hold at most 65536 16-byte units.
 * Invalid data (NaN / +inf or no finite logit on a visited node, a candidate
 * outside [0, V), a uniform outside [0, 1), bad temperature or top_p) gives
 * n = -1 and tokens -1.  Asynchronous on `stream`, allocates nothing.  Returns
 * SV_OK or a negative code (nothing enqueued).
 */
int spec_verify_spectr(const void* p_logits, const void* q_logits, int dtype, const int32_t* candidates,
                       const float* uniforms, const float* temperature, const int32_t* top_k,
                       const float* top_p, int B, int K, int L, int V, int32_t* out_tokens,
                       int32_t* out_n, int32_t* out_node_tokens, void* stream);

/* Kernels of one call, for spec_verify_set_stage_events. */
enum {
  SV_KERNEL_SELECT = 0,  /* streaming top-k / argmax select over the logit rows      */
                         /* (in a call that runs the mixed kernel: only the listing */
                         /* of the dense pairs)                                     */
  SV_KERNEL_PAIR = 1,    /* per-(sequence, position) pass over dense (unfiltered,   */
                         /* large top-k, top-p) sequences; launched when V allows.  */
                         /* For bf16 rows of 32K-131K values with both kinds of     */
                         /* sequence and no hint, the mixed kernel that also        */
                         /* streams the select's rows                               */
  SV_KERNEL_FINISH = 2,  /* per-sequence acceptance, first rejection and draw       */
  SV_KERNEL_GUMBEL = 3,  /* spec_verify_gumbel: the histogram rows' kernel (with    */
                         /* the select units when a list path runs beside it), or   */
                         /* the per-(sequence, position) kernel                     */
  SV_KERNEL_KSEQ = 4     /* per-(sequence, prefix node) K-SEQ of spec_verify_spectr */
};

/*
 * Measurement hook (for benchmarks and profilers, not needed for normal use).
 * With non-NULL hipEvent_t handles `begin` and `end`, every later spec_verify
 * call made from this host thread records `begin` on its stream just before
 * the chosen kernel (SV_KERNEL_*) and `end` just after it, so that
 * hipEventElapsedTime(begin, end) is that kernel's duration.  If a call does
 * not launch that kernel, nothing is recorded.  The caller owns the events.
 * Passing NULL, NULL stops the recording.  Returns SV_OK, or SV_ERR_ARG for
 * an unknown kernel.
 */
int spec_verify_set_stage_events(int kernel, void* begin, void* end);

/*
 * Throughput analytics (host functions; no GPU, no stream).  From the Leviathan
 * review ("Analysis": expected generated tokens, walltime, operations, optimal
 * gamma) and "Speculative Decoding: the art of guessing well" ("How many tokens
 * do we get?"):
 *   expected tokens per round  (1 - alpha^(gamma+1)) / (1 - alpha)   (gamma+1 at alpha = 1)
 *   speedup                    expected tokens / (gamma c + 1), c = drafter/target cost ratio
 *   operations                 (gamma c_hat + gamma + 1) / expected tokens, relative to plain
 *                              decoding, c_hat = drafter/target operations ratio
 *   optimal gamma              the gamma in [1, gamma_max] with the largest speedup (smallest on ties)
 *   acceptance length tau      1 + sum_{k<=gamma} prod_{i<=k} alpha_i, from per-position rates
 *                              (host array alpha[gamma], e.g. a column mean of spec_verify's out_alpha)
 * alpha must lie in [0, 1]; invalid arguments give NaN (or -1 for the optimal gamma).
 */
double spec_verify_expected_tokens(double alpha, int gamma);
double spec_verify_speedup(double alpha, int gamma, double c);
double spec_verify_operations(double alpha, int gamma, double c_hat);
int spec_verify_optimal_gamma(double alpha, double c, int gamma_max);
double spec_verify_acceptance_length(const double* alpha, int gamma);

/* Static description of a return code (for SV_ERR_HIP, the last HIP error of this thread). */
const char* spec_verify_strerror(int code);

/* ABI version: 11. */
int spec_verify_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
