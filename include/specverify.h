/*
 * specverify.h -- batched speculative-sampling verification on AMD Instinct
 * MI355X (gfx950), as a C ABI.
 *
 * The operation (the pages' shared hot path): a target model scores the
 * gamma draft tokens of every row in one pass and the verifier accepts or
 * rejects them token by token, on the device, without a round trip to the
 * host ("FlashSpec: Adaptive Speculative Decoding with Online Bandit Draft
 * Selection and Triton-Optimised Verification" -- technical summary, problem
 * definition and section 1 "On-device verification kernel"). Temperature is
 * applied to the logits before the log-softmax (same section, numerical
 * stability). At the first rejection the correction token is drawn from the
 * residual max(p - q, 0) ("Speculative Speculative Decoding" -- technical
 * summary, section 2, optimisation 2 "Saguaro sampling"); when every draft is
 * accepted a bonus token is drawn from the target's next distribution
 * ("SpecTr-GBV: Multi-Draft Block Verification Accelerating Speculative
 * Decoding" -- section 2, algorithm procedure, termination step).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers are DEVICE pointers unless marked host. The caller owns every
 *   buffer; the library never allocates, frees or synchronises. All work is
 *   enqueued on `stream` (a hipStream_t; NULL = the null stream) and the call
 *   returns without waiting for it.
 * - Argument errors are detected on the host before anything is enqueued and
 *   return a negative status; no partial work is launched.
 * - Logits are row-major with the vocabulary axis contiguous (stride 1);
 *   other strides are in elements, must be >= 0, and may be 0 (broadcast).
 *   Target and draft logits share one dtype (SV_F32 or SV_BF16). Rows whose
 *   start is 16-byte aligned take 128-bit loads; other rows take element
 *   loads (slower, same results).
 * - Random numbers: a Philox4x32-10 stream (Salmon et al., SC'11) keyed by
 *   (seed mod 2^32, seed >> 32) with counter (c0, position, chain row,
 *   purpose), where chain row r = b*K + k and position = pos0[b] + j
 *   (mod 2^32). The accept uniform of position j is word 0 of block
 *   (0, pos0[b]+j, r, 0); the sampling noise of vocabulary id v is word v&3
 *   of block (v>>2, pos0[b]+n, r, 1). A word w maps to
 *   u = (floor(w / 2^9) + 1/2) * 2^-23, strictly inside (0, 1).
 * - A temperature of exactly 0 marks a greedy row: tokens are accepted iff
 *   they equal the target row's argmax (lowest id on ties), nothing random is
 *   drawn, and draft logits are never read.
 * - Results are bit-deterministic: reductions merge in a fixed order and no
 *   floating-point atomics are used.
 * - `workspace` is device scratch of at least specverify_workspace_size()
 *   bytes, 256-byte aligned, with any contents: each call's first launch
 *   clears what must start at zero (the per-chain counters through which the
 *   sampling workgroups of one launch find the last of a chain's splits), so
 *   one buffer serves any number of calls of any sizes (within its size)
 *   ordered on one stream. Calls that overlap in time on one buffer race.
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Logit storage types. */
#define SV_F32 0
#define SV_BF16 1

/* Return status of every entry point. */
#define SV_OK 0
#define SV_EINVAL (-1)     /* null pointer, size or stride out of range      */
#define SV_EDTYPE (-2)     /* unknown logit dtype                            */
#define SV_EWORKSPACE (-3) /* workspace missing or smaller than required     */
#define SV_EALIGN (-4)     /* workspace not 256-byte aligned                 */
#define SV_EHIP (-5)       /* a kernel launch failed                         */
#define SV_ESCRATCH (-6)   /* specverify_step_noalloc: sizes need more scratch
                              than SV_NOALLOC_SCRATCH_BYTES                  */
#define SV_ENOCHECKS (-7)  /* specverify_check_count: the library was built
                              without device-side index checks               */

/* Device scratch held by specverify_step_noalloc on every GPU it runs on. */
#define SV_NOALLOC_SCRATCH_BYTES (32u << 20)

/* Bits OR-ed into the optional device error word; the chain's accept_len and
 * out_token are set to -1 when any of them applies to it. */
#define SV_ERR_TOKEN 1     /* a draft token outside [0, V)                   */
#define SV_ERR_TEMP 2      /* temperature negative or NaN                    */
#define SV_ERR_ROW 4       /* a needed row whose largest logit is not
                              finite: every entry -inf (all masked), or any
                              +inf or NaN entry                              */

/* Size limits checked on the host. */
#define SV_MAX_GAMMA 32
#define SV_MAX_CHAIN_DECISIONS 64 /* K * gamma per batch row */
#define SV_MAX_FANOUT 64          /* candidates per verification outcome */
#define SV_MAX_ARMS 256           /* draft models of the bandit selector */

/* Bandit policies (specverify_bandit_init). */
#define SV_BANDIT_UCB1 0
#define SV_BANDIT_THOMPSON 1

/*
 * Bytes of workspace that specverify_step / specverify_normalize /
 * specverify_residual_sample need for these sizes (the largest of the three;
 * for specverify_normalize pass K = 0 and gamma = P - 1). Pure host function.
 * Returns 0 for sizes the library rejects.
 */
size_t specverify_workspace_size(int64_t B, int64_t K, int64_t gamma, int64_t V, int dtype);

/*
 * Row normalisers (FlashSpec technical summary, section 1: temperature is
 * applied before the log-softmax; arithmetic in log space).
 *   logits       [B, P, V] rows at logits + b*stride_b + p*stride_p (elements)
 *   temperature  [B] float
 *   lnZ          [B, P] double out: ln sum_v exp(z_v / T_b) for T_b > 0;
 *                max_v z_v for T_b == 0 (the T -> 0 limit of T * ln Z);
 *                NaN for T_b < 0 or NaN. An all -inf row gives -inf; a row
 *                holding a NaN gives NaN, and so does a +inf entry when
 *                T_b > 0 (for T_b == 0 the maximum is +inf).
 *   argmax       [B, P] int32 out, or NULL: lowest id of the row maximum of
 *                the raw logits, for every row (NaN entries are passed by).
 * Status: SV_EINVAL (null logits/temperature/lnZ, B/P/V < 1, V >= 2^31,
 * negative stride, or rows of 2^31 or more 8 KB chunks: over 16 TiB of
 * logits), SV_EDTYPE, SV_EWORKSPACE, SV_EALIGN, SV_EHIP.
 */
int specverify_normalize(const void* logits, int dtype, int64_t B, int64_t P, int64_t V,
                         int64_t stride_b, int64_t stride_p, const float* temperature,
                         double* lnZ, int32_t* argmax, void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * Scalar-only accept test (FlashSpec technical summary, section 1 mechanism:
 * the kernel reads two log-probability scalars per candidate, so no pass over
 * the vocabulary is needed).
 *   logp, logq   [B, K, gamma] float: ln p and ln q at each draft token.
 *                A greedy row is encoded ln p in {0, -inf}, ln q = 0.
 *   pos0         [B] int64 or NULL (all 0)
 *   accept_len   [B, K] int32 out: number of leading accepts, where position
 *                j accepts iff ln u_j < ln p_j - ln q_j (a NaN difference
 *                rejects).
 *   accept_bits  [B, K] uint32 out or NULL: bit j = decision at position j
 *                (every position is decided, also after the first rejection).
 * Status: SV_EINVAL (null pointers, B/K < 1, gamma outside [1, 32]), SV_EHIP.
 */
int specverify_accept(const float* logp, const float* logq, int64_t B, int64_t K, int64_t gamma,
                      uint64_t seed, const int64_t* pos0, int32_t* accept_len,
                      uint32_t* accept_bits, void* stream);

/*
 * The emitted token of every chain given its accept length (Speculative
 * Speculative Decoding, technical summary section 2, optimisation 2: residual
 * r proportional to max(p_target - p_draft, 0); SpecTr-GBV section 2,
 * termination step: residual at a rejection, target sample when the whole
 * block is accepted).
 *   target_logits [B, gamma+1, V], draft_logits [B, K, gamma, V] (strides as named)
 *   temperature   [B] float
 *   lnZ_target    [B, gamma+1] double, lnZ_draft [B, K, gamma] double: the
 *                 normalisers of specverify_normalize
 *   argmax_target [B, gamma+1] int32: used for greedy rows (T == 0)
 *   accept_len    [B, K] int32 in: n in [0, gamma]; chains with n < 0 are skipped
 *   out_token     [B, K] int32 out:
 *                 T > 0, n < gamma : argmax_v ln max(p_n - q_n, 0)(v) + G_v
 *                 T > 0, n = gamma : argmax_v z_t[gamma, v] / T + G_v
 *                 T = 0            : argmax_target[b, n]
 *                 with G_v standard Gumbel noise (ties to the lowest id). If
 *                 the residual support is empty (possible only by rounding)
 *                 the token is drawn from p_n with the same noise.
 * Status: as specverify_step.
 */
int specverify_residual_sample(const void* target_logits, const void* draft_logits, int dtype,
                               int64_t B, int64_t K, int64_t gamma, int64_t V,
                               int64_t t_stride_b, int64_t t_stride_j,
                               int64_t d_stride_b, int64_t d_stride_k, int64_t d_stride_j,
                               const float* temperature, const double* lnZ_target,
                               const double* lnZ_draft, const int32_t* argmax_target,
                               const int32_t* accept_len, uint64_t seed, const int64_t* pos0,
                               int32_t* out_token, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * One fused verification step for B rows x K draft branches (all branches of
 * row b share its target rows; each branch is its own token-level chain).
 *   target_logits  [B, gamma+1, V]; row j verifies draft token j, row gamma
 *                  supplies the bonus token
 *   draft_logits   [B, K, gamma, V]
 *   draft_tokens   [B, K, gamma] int32
 *   temperature    [B] float (T == 0: greedy row)
 *   seed, pos0     random stream key and [B] int64 positions (pos0 may be NULL)
 *   accept_len     [B, K] int32 out: n = number of leading accepted drafts
 *   out_token      [B, K] int32 out: correction (n < gamma) or bonus (n = gamma)
 *                  token; the chain emits draft_tokens[b,k,0:n] then out_token
 *   logp, logq     [B, K, gamma] float out or NULL: ln p, ln q at the draft
 *                  tokens (greedy rows: ln p in {0, -inf}, ln q = 0)
 *   lnZ_target     [B, gamma+1] double out or NULL (as specverify_normalize)
 *   lnZ_draft      [B, K, gamma] double out or NULL (not written for greedy rows)
 *   device_error   one int32 out or NULL: OR of SV_ERR_* bits (only set, never
 *                  cleared: zero it before the call)
 * Status: SV_EINVAL (null required pointer, B/K/V < 1, gamma outside [1, 32],
 * K*gamma > 64, V >= 2^31, negative stride, or rows of 2^31 or more 8 KB
 * chunks: over 16 TiB of logits), SV_EDTYPE, SV_EWORKSPACE, SV_EALIGN,
 * SV_EHIP.
 */
int specverify_step(const void* target_logits, const void* draft_logits, int dtype,
                    const int32_t* draft_tokens, int64_t B, int64_t K, int64_t gamma, int64_t V,
                    int64_t t_stride_b, int64_t t_stride_j,
                    int64_t d_stride_b, int64_t d_stride_k, int64_t d_stride_j,
                    const float* temperature, uint64_t seed, const int64_t* pos0,
                    int32_t* accept_len, int32_t* out_token, float* logp, float* logq,
                    double* lnZ_target, double* lnZ_draft, int32_t* device_error,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * specverify_step for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, outputs and results as specverify_step without the
 * workspace: the step runs in a scratch array that the library holds on each
 * GPU from its load until the process ends (SV_NOALLOC_SCRATCH_BYTES, 32 MiB;
 * enough for B = 512 rows x K = 4 branches at gamma = 8, V = 128256). The call
 * allocates nothing and leaves no state that the next call needs: the step's
 * first launch clears what must start at zero. Every call on one GPU shares
 * that GPU's scratch, so calls that overlap in time on one GPU (on different
 * streams, or from different threads) race; order them on one stream.
 * Status: as specverify_step, plus SV_ESCRATCH when specverify_workspace_size
 * for these sizes exceeds SV_NOALLOC_SCRATCH_BYTES (nothing is enqueued).
 */
int specverify_step_noalloc(const void* target_logits, const void* draft_logits, int dtype,
                            const int32_t* draft_tokens, int64_t B, int64_t K, int64_t gamma,
                            int64_t V, int64_t t_stride_b, int64_t t_stride_j, int64_t d_stride_b,
                            int64_t d_stride_k, int64_t d_stride_j, const float* temperature,
                            uint64_t seed, const int64_t* pos0, int32_t* accept_len,
                            int32_t* out_token, float* logp, float* logq, double* lnZ_target,
                            double* lnZ_draft, int32_t* device_error, void* stream);

/*
 * Bytes of workspace that specverify_accept_prob needs for these sizes. Its
 * chunk sums sit after the counter region of the other entry points, so one
 * buffer of the largest size can serve all of them. Pure host function;
 * returns 0 for sizes the library rejects.
 */
size_t specverify_accept_prob_workspace_size(int64_t B, int64_t K, int64_t gamma, int64_t V,
                                             int dtype);

/*
 * Exact acceptance probability of every draft position, and the law of the
 * accept length (FlashSpec technical summary, section 2 "Online bandit draft
 * selection": the bandit's reward is the accepted fraction of draft tokens;
 * Speculative Speculative Decoding technical summary, section 2,
 * optimisation 1 "geometric fan-out": verified lengths fall off
 * geometrically).
 *   target_logits, draft_logits, strides, temperature: as specverify_step
 *   lnZ_target  [B, gamma+1] double in: the normalisers that specverify_step
 *               or specverify_normalize wrote (rows 0..gamma-1 are read;
 *               not read for greedy rows)
 *   lnZ_draft   [B, K, gamma] double in: likewise
 *   alpha       [B, K, gamma] double out: sum_v min(p_j(v), q_j(v)) with
 *               p_j = softmax(z_t[b, j] / T_b), q_j = softmax(z_d[b, k, j] / T_b),
 *               the probability that position j accepts when its draft token
 *               is drawn from q_j. Greedy rows (T == 0): 1 if the lowest-id
 *               argmaxes of target row j and draft row (k, j) agree, else 0.
 *               T < 0 or NaN: NaN.
 *   law         [B, K, gamma+1] double out or NULL: P(n = m) =
 *               alpha_0 ... alpha_{m-1} (1 - alpha_m) for m < gamma and
 *               P(n = gamma) = alpha_0 ... alpha_{gamma-1}.
 * Reads target rows 0..gamma-1 once and every draft row once (also those of
 * greedy rows, whose argmax it needs). Precision: terms in float32 around a
 * per-lane reference, sums in float64 (|d alpha| ~ 1e-7).
 * Status: SV_EINVAL (null required pointer, sizes as specverify_step,
 * negative stride), SV_EDTYPE, SV_EWORKSPACE, SV_EALIGN, SV_EHIP.
 */
int specverify_accept_prob(const void* target_logits, const void* draft_logits, int dtype,
                           int64_t B, int64_t K, int64_t gamma, int64_t V,
                           int64_t t_stride_b, int64_t t_stride_j,
                           int64_t d_stride_b, int64_t d_stride_k, int64_t d_stride_j,
                           const float* temperature, const double* lnZ_target,
                           const double* lnZ_draft, double* alpha, double* law,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Speculation-cache fan-out (Speculative Speculative Decoding technical
 * summary, section 2, optimisation 1 "geometric fan-out": verified lengths
 * fall off geometrically, so short accept lengths get more candidates).
 * Pure host function. fanout [gamma+1] int32 HOST out: F_j proportional to
 * ratio^j, rounded to integers summing to `total` by largest remainders (ties
 * to the smaller j). Status: SV_EINVAL (null, gamma outside [1, 32], ratio
 * outside (0, 1], total < 0 or an F_j above SV_MAX_FANOUT).
 */
int specverify_geometric_fanout(int64_t gamma, int64_t total, double ratio, int32_t* fanout);

/*
 * The most likely emitted tokens of every verification outcome (Speculative
 * Speculative Decoding technical summary, core mechanism items 2-3: a cache
 * keyed by the outcome -- how many drafts are accepted and which token
 * follows; section 2, optimisation 2: that token is drawn from the residual
 * max(p_target - p_draft, 0)).
 *   target_logits, draft_logits, strides, temperature, lnZ_target,
 *   lnZ_draft: as specverify_accept_prob
 *   fanout      [gamma+1] int32 HOST: F_j candidates for outcome n = j, each
 *               in [0, SV_MAX_FANOUT]
 *   cand        [B, K, sum F] int32 out, outcome-major: for outcome j < gamma
 *               the F_j ids of largest max(p_j - q_j, 0); for j = gamma those of
 *               largest p_gamma; greedy rows (T == 0): those of largest raw
 *               target logit of row j. Best first, ties to the lowest id; ids
 *               of zero weight (-inf logit for greedy rows) are never listed,
 *               so a short support is padded with -1. T < 0 or NaN: all -1.
 *   cand_weight [B, K, sum F] float out or NULL: the candidates' weights
 *               (r_j or p_gamma; raw logits for greedy rows), -inf for padding.
 * Weights are ranked in float32 (relative error ~1e-6), so ids whose weights
 * differ by less than that may swap places. No workspace.
 * Status: SV_EINVAL (null required pointer, sizes as specverify_step, a
 * fan-out entry outside [0, SV_MAX_FANOUT], negative stride), SV_EDTYPE,
 * SV_EHIP.
 */
int specverify_residual_topf(const void* target_logits, const void* draft_logits, int dtype,
                             int64_t B, int64_t K, int64_t gamma, int64_t V,
                             int64_t t_stride_b, int64_t t_stride_j,
                             int64_t d_stride_b, int64_t d_stride_k, int64_t d_stride_j,
                             const float* temperature, const double* lnZ_target,
                             const double* lnZ_draft, const int32_t* fanout, int32_t* cand,
                             float* cand_weight, void* stream);

/*
 * Cache hit test of a step's outcome (same passage, item 3: a hit returns the
 * prepared continuation at once).
 *   cand        [B, K, sum F] int32 from specverify_residual_topf
 *   fanout      [gamma+1] int32 HOST, as given there
 *   accept_len, out_token [B, K] int32 from specverify_step
 *   slot        [B, K] int32 out: index into cand[b, k, :] of out_token among
 *               the candidates of outcome n = accept_len, or -1 (miss, or
 *               n outside [0, gamma], or a negative token).
 * Status: SV_EINVAL (null pointer, B/K < 1, gamma outside [1, 32], a fan-out
 * entry outside [0, SV_MAX_FANOUT]), SV_EHIP.
 */
int specverify_cache_lookup(const int32_t* cand, const int32_t* fanout, int64_t B, int64_t K,
                            int64_t gamma, const int32_t* accept_len, const int32_t* out_token,
                            int32_t* slot, void* stream);

/*
 * Draft selection between decoding steps (FlashSpec technical summary,
 * section 2 "Online bandit draft selection": a K-armed bandit over draft
 * models whose reward is the accepted fraction of draft tokens, with UCB1 or
 * Thompson sampling; the policy sees only past acceptance, so the verified
 * output distribution is unchanged). HOST functions on a HOST state buffer the
 * caller owns; no GPU work, no allocation, not thread-safe per state.
 *
 * specverify_bandit_state_size: bytes of state for `arms` arms (0 if arms is
 *   outside [1, SV_MAX_ARMS]).
 * specverify_bandit_init: policy SV_BANDIT_UCB1 (Auer, Cesa-Bianchi, Fischer
 *   2002: each arm once in index order, then argmax mean_i + sqrt(c ln t / n_i),
 *   t = rewards so far, c = 2 in the paper) or SV_BANDIT_THOMPSON (argmax of
 *   theta_i ~ Beta(1 + S_i, 1 + n_i - S_i), S_i the arm's reward sum; Beta draws
 *   from two Marsaglia-Tsang Gamma variates on uniforms of Philox4x32-10 keyed
 *   by `seed`, counter (draw, arm, (variate << 16) | attempt, 2)). Ties go to the
 *   lowest index. Status: SV_EINVAL (null, arms out of range, unknown policy,
 *   c <= 0 or not finite), SV_EWORKSPACE (state_bytes too small).
 * specverify_bandit_select: writes the arm for the next step.
 * specverify_bandit_update: reward in [0, 1] for the arm just played.
 * specverify_bandit_stats: pulls and reward sum of one arm (either may be NULL).
 * specverify_step_reward: the reward of a step from its accept lengths (HOST
 *   array of `chains` int32): sum(clamp(n, 0, gamma)) / (chains * gamma).
 * Status of the last four: SV_EINVAL for a null or uninitialised state, an arm
 * out of range, a reward outside [0, 1], chains < 1 or gamma outside [1, 32].
 */
size_t specverify_bandit_state_size(int32_t arms);
int specverify_bandit_init(void* state, size_t state_bytes, int32_t arms, int32_t policy,
                           uint64_t seed, double c);
int specverify_bandit_select(void* state, int32_t* arm);
int specverify_bandit_update(void* state, int32_t arm, double reward);
int specverify_bandit_stats(const void* state, int32_t arm, int64_t* pulls, double* reward_sum);
int specverify_step_reward(const int32_t* accept_len, int64_t chains, int64_t gamma,
                           double* reward);

/*
 * Branch pruning before verification (FlexDraft technical summary,
 * methodology component 3 "Flex decoding", selective verification for small
 * batches: the cumulative draft confidence estimates how far each branch will
 * be accepted; low-confidence branches are dropped and only high-confidence
 * prefixes verified). The pages give no rule; the one taken here:
 *   logq        [B, K, gamma] float: ln q at each branch's drafted tokens
 *   conf        [B, K, gamma] double out or NULL: running sums of ln q over
 *               j = 0..gamma-1, in order, in float64
 *   prefix_len  [B, K] int32 out or NULL: positions with conf >= log_tau (a
 *               leading run, since ln q <= 0)
 *   keep_mask   [B, K] int32 out: 1 for the `keep` branches of each row with
 *               the largest prefix_len (ties: larger conf at the prefix's last
 *               position, -inf for an empty prefix; then lower k), else 0.
 * Status: SV_EINVAL (null logq/keep_mask, B/K < 1, gamma outside [1, 32],
 * K * gamma > 64, keep < 0, log_tau NaN), SV_EHIP.
 */
int specverify_branch_prune(const float* logq, int64_t B, int64_t K, int64_t gamma,
                            double log_tau, int64_t keep, int32_t* keep_mask,
                            int32_t* prefix_len, double* conf, void* stream);

/*
 * Measurement hook; results are unaffected. The next call on the calling host
 * thread that launches the streaming kernel (specverify_step,
 * specverify_step_noalloc, specverify_normalize) launches it with hipExtLaunchKernel,
 * which marks `before` with the kernel's start and `after` with its end, so
 * that hipEventElapsedTime(before, after) is the kernel's execution time
 * (a profiler's per-kernel duration, read live). One-shot: that launch clears
 * the hook; a call that fails its checks before launching leaves it set.
 * before, after: hipEvent_t handles the caller created (with timing) on the
 * device of the call and keeps alive until the call's stream has passed them;
 * NULL, NULL clears the hook. Pure host function.
 * Status: SV_EINVAL when exactly one of the two is NULL.
 */
int specverify_time_next_stream_kernel(void* before, void* after);

/*
 * Debugging aid. A library built with device-side index checks
 * (build.py --checked: libspecverify_checked.so, -DSV_DEVICE_CHECKS) has every
 * work unit of every kernel check the indices it derived (batch row, branch,
 * position, chunk, split, accept length) against the sizes it was launched
 * with before touching memory; a failed check is counted on the device and
 * the unit is skipped. This call copies the count of the current device into
 * *count and, when reset is non-zero, sets it to zero. Blocking (a device copy
 * on the null stream): call after the work to be checked has completed.
 * Status: SV_ENOCHECKS in a build without the checks (the product library),
 * SV_EINVAL (count NULL), SV_EHIP.
 */
int specverify_check_count(uint32_t* count, int reset);

/* Static host string describing a status code. */
const char* specverify_status_string(int status);

/* Library version: major * 10000 + minor * 100 + patch. */
int specverify_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H */
