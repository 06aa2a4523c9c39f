/*
 * mtpv.h - C ABI of the vocab-side draft-and-verify step of MTP speculative
 * decoding, built for AMD MI355X (gfx950) with hand-written HIP kernels.
 *
 * What the calls compute. The target model has produced hidden states for the
 * k+1 verify positions of each of B requests, and the MTP drafter has proposed k
 * draft tokens per request. One vocabulary head W_lm [V, H], shared by the main
 * model and the MTP drafter ("The Tiny Draft Model Hidden Inside Qwen", sections
 * "One step deeper than the main model" and "What vLLM and SGLang do with the
 * weights"; "Optimize vLLM speculative decoding with FastMTP heads", section "Key
 * features"), is streamed from HBM once per call to produce the logits of every
 * row; the calls then take a distribution at every position, keep the longest
 * prefix of drafts the target agrees with, and replace the first rejected slot
 * with a draw from the corrected distribution ("The Tiny Draft Model Hidden Inside
 * Qwen", section "How the draft becomes real output"; "Speculative Decoding and
 * MTP: Why Guessing Is Free", sections "Speculative decoding: draft, then verify"
 * and "It's exact, not approximate").
 *
 * Notation. B requests, k drafts per request, H hidden width, V vocabulary size,
 * T temperature. Slot j of request b: p_j = softmax(l(target row j) / T) for
 * j = 0..k, q_j = softmax(l(drafter row j) / T) for j = 0..k-1. Draft
 * draft_tokens[b*k + j] is judged against p_j; p_k only feeds the bonus token.
 *
 * Conventions for every call:
 *  - All array arguments are DEVICE pointers owned by the caller, row-major and
 *    contiguous, 16-byte aligned. The library allocates nothing per call.
 *  - dtype selects the storage of hidden states and W_lm: MTPV_BF16 (bf16) or
 *    MTPV_F32 (fp32). Accumulation is fp32 in both cases; sampling math is fp64.
 *  - H must be a multiple of 8 (whole 16-byte loads per row); V >= 1; B >= 1;
 *    0 <= k <= 64.
 *  - stream is a hipStream_t passed as void* (NULL = the default stream). Calls
 *    are asynchronous and stream ordered; nothing synchronizes the host.
 *  - workspace is caller-owned device memory of at least
 *    mtpv_workspace_bytes(B, k, H, V, dtype, mode) bytes, 256-byte aligned. Its
 *    contents need no initialisation and are scratch between calls; two calls
 *    in flight at once must not share one workspace.
 *  - Errors in sizes, pointers, alignment, dtype or workspace are found on the
 *    host before anything is enqueued and returned as a negative mtpv_status.
 *    A draft id outside [0, V) is not a host error (drafts live on the device):
 *    that draft counts as rejected and the call's device error word gets
 *    MTPV_DEVERR_DRAFT_RANGE (read it with mtpv_get_device_error).
 *  - No exception crosses this boundary.
 */
#ifndef MTPV_H_
#define MTPV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__) || defined(__clang__)
#define MTPV_API __attribute__((visibility("default")))
#else
#define MTPV_API
#endif

typedef enum mtpv_status {
    MTPV_OK = 0,
    MTPV_EINVAL = -1,     /* a size or scalar is out of range (B < 1, k < 0, T <= 0, ...) */
    MTPV_EALIGN = -2,     /* H not a multiple of 8, or a pointer not 16-byte aligned   */
    MTPV_EWORKSPACE = -3, /* workspace NULL, misaligned or smaller than required       */
    MTPV_EDTYPE = -4,     /* dtype is neither MTPV_BF16 nor MTPV_F32                   */
    MTPV_ELAUNCH = -5,    /* a kernel launch failed                                    */
    MTPV_EDEVICE = -6,    /* HIP runtime error (no device, bad stream, copy failed)    */
    MTPV_ENULL = -7,      /* a required pointer is NULL                                */
    MTPV_ESCRATCH = -8    /* spec_verify_greedy_noalloc: shape beyond its scratch      */
} mtpv_status;

typedef enum mtpv_dtype { MTPV_BF16 = 0, MTPV_F32 = 1 } mtpv_dtype;

/* Which call a workspace is sized for. */
typedef enum mtpv_mode { MTPV_MODE_GREEDY = 0, MTPV_MODE_SAMPLE = 1, MTPV_MODE_DRAFT = 2 } mtpv_mode;

/* Bits of the per-call device error word. */
#define MTPV_DEVERR_DRAFT_RANGE 1 /* some draft id was outside [0, V); it was rejected */
#define MTPV_DEVERR_DRAFT_LEN 2   /* some draft_len[b] was outside [0, k]; it was clamped */
#define MTPV_DEVERR_TOKEN_RANGE 4 /* mtp_input_fuse: some token was outside [0, V); zero embedding used */

/*
 * Optional exports for parity tests; pass NULL (or NULL members) in production.
 * Rows are numbered as the head sees them: target row (b, j) is row b*(k+1)+j,
 * drafter row (b, j) is row B*(k+1) + b*k + j (sample mode only; in draft mode
 * drafter row (b, j) is row b*k + j). M_eff is the number of rows.
 *   logits    [M_eff, V] fp32: the head's logits l = x . W^T.
 *   probs     [M_eff, V] fp32: softmax(l / T) as the kernels normalise it.
 *   argmax    [M_eff] int32: argmax of each row, lowest id on ties.
 *   row_stats [M_eff, 2] fp64: {max_v l/T, sum_v exp(l/T - max)} per row.
 *   pd_qd     [B, k, 2] fp64: {p_j(d_j), q_j(d_j)} of every slot (greedy: q = 0;
 *             an out-of-range draft gives {-1, -1}).
 */
typedef struct mtpv_debug {
    float* logits;
    float* probs;
    int32_t* argmax;
    double* row_stats;
    double* pd_qd;
} mtpv_debug;

/* Library version: major*10000 + minor*100 + patch. */
MTPV_API int mtpv_version(void);

/* Text for a status code (static storage; never NULL). */
MTPV_API const char* mtpv_status_string(int status);

/*
 * Workspace bytes a call of the given shape and mode needs (0 if the shape is
 * invalid). mode: MTPV_MODE_GREEDY (0) or MTPV_MODE_SAMPLE (1) for the verify
 * calls, MTPV_MODE_DRAFT (2) for spec_draft_sample. Host only; no GPU needed.
 */
MTPV_API size_t mtpv_workspace_bytes(int B, int k, int H, int V, int dtype, int mode);

/*
 * Host-only argument check shared by every call; returns what the call itself
 * would return before enqueueing anything. Pointers are only checked for NULL
 * and alignment, never dereferenced. For MTPV_MODE_DRAFT, k is the number of
 * drafter rows per request, draft_hidden and draft_tokens (output) are
 * required and target_hidden / accepted_len / out_tokens are ignored.
 */
MTPV_API int mtpv_check_args(int mode, int B, int k, int H, int V, int dtype, double temperature,
                    const void* target_hidden, const void* draft_hidden, const void* W_lm,
                    const int32_t* draft_tokens, const int32_t* accepted_len,
                    const int32_t* out_tokens, const void* workspace, size_t workspace_bytes);

/*
 * Greedy verification.
 * The drafts are kept up to the first one the target's argmax disagrees with,
 * which makes greedy speculative decoding emit the same sequence as plain greedy
 * decoding ("The Tiny Draft Model Hidden Inside Qwen", section "How the draft
 * becomes real output"). For each request b:
 *   g_j = argmax_v l(target row j)  (lowest id on ties), j = 0..k
 *   a   = number of leading slots with draft_tokens[b*k+j] == g_j  (0..k)
 *   accepted_len[b] = a
 *   out_tokens[b*(k+1) + j] = draft j for j < a, g_a for j = a, -1 after.
 * hidden       [B, k+1, H] target hidden states (dtype)
 * W_lm         [V, H] shared vocabulary head (dtype)
 * draft_tokens [B, k] int32
 * accepted_len [B] int32 (output), out_tokens [B, k+1] int32 (output)
 * debug        NULL or exports (temperature 1 is used for probs / row_stats)
 */
MTPV_API int spec_verify_greedy(const void* hidden, const void* W_lm, const int32_t* draft_tokens,
                       int B, int k, int H, int V, int dtype,
                       int32_t* accepted_len, int32_t* out_tokens,
                       void* workspace, size_t workspace_bytes,
                       const mtpv_debug* debug, void* stream);

/*
 * Stochastic verification (exact speculative sampling).
 * The surviving tokens must be distributed exactly as the target alone would
 * produce them ("Speculative Decoding and MTP: Why Guessing Is Free", section
 * "It's exact, not approximate"); the first rejected slot is replaced by a draw
 * from the verifier's corrected distribution ("The Tiny Draft Model Hidden
 * Inside Qwen", section "How the draft becomes real output"); k kept drafts
 * give k+1 tokens ("Speculative Decoding and MTP: Why Guessing Is Free",
 * section "Speculative decoding: draft, then verify"). The rule is the standard
 * speculative-sampling rule (Leviathan, Kalman & Matias 2023; Chen et al. 2023):
 *   u_j  = uniform(word 0 of Philox4x32-10(key = seed; counter = (j, b, offset)))
 *   keep draft d = draft_tokens[b*k+j] iff u_j * q_j(d) < p_j(d)
 *          (probability min(1, p/q)); a = first rejected slot, or k
 *   a < k: out[a] ~ normalize(max(0, p_a - q_a)); a = k: out[k] ~ p_k (bonus);
 *          the draw is the smallest id whose ascending prefix sum exceeds
 *          u' * (total mass), u' = uniform(word 1 of the same Philox block at
 *          slot a); if the residual mass is zero the draw uses p_a.
 * uniform(x) = (x >> 8) * 2^-24. Philox key = (low 32 bits, high 32 bits) of
 * seed; counter = (slot, request, low 32 bits, high 32 bits of offset).
 * target_hidden [B, k+1, H], draft_hidden [B, k, H] (the drafter hidden states
 * the drafts were sampled from), W_lm [V, H], draft_tokens [B, k].
 * temperature > 0 applies to both p and q.
 * Outputs as for spec_verify_greedy.
 */
MTPV_API int spec_verify_sample(const void* target_hidden, const void* draft_hidden, const void* W_lm,
                       const int32_t* draft_tokens, int B, int k, int H, int V, int dtype,
                       double temperature, uint64_t seed, uint64_t offset,
                       int32_t* accepted_len, int32_t* out_tokens,
                       void* workspace, size_t workspace_bytes,
                       const mtpv_debug* debug, void* stream);

/*
 * spec_verify_greedy for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * computation and outputs as spec_verify_greedy, with no workspace argument. Its
 * scratch is a file-scope device array of MTPV_NOALLOC_SCRATCH_BYTES held by each
 * GPU the library runs on until the process ends; the call allocates nothing and
 * records no timing events. A shape whose workspace (mtpv_workspace_bytes(B, k, H,
 * V, dtype, MTPV_MODE_GREEDY)) exceeds that size returns MTPV_ESCRATCH before
 * anything is enqueued. Every call on one GPU shares that GPU's array: calls that
 * overlap in time on one GPU (other streams, other host threads) race and must be
 * ordered by the caller. device_error: NULL, or a device int32 that receives the
 * call's device error word (MTPV_DEVERR_* bits; cleared by the call itself).
 * Other arguments, layouts and errors as for spec_verify_greedy.
 */
#define MTPV_NOALLOC_SCRATCH_BYTES (16u << 20)
MTPV_API int spec_verify_greedy_noalloc(const void* hidden, const void* W_lm, const int32_t* draft_tokens,
                       int B, int k, int H, int V, int dtype,
                       int32_t* accepted_len, int32_t* out_tokens, int32_t* device_error, void* stream);

/*
 * Verification with a draft count per request ("dynamic draft length", named as
 * coming drafter support in "Faster Rollouts with MTP Speculative Decoding",
 * section "What's Next"; the pages give no rule, the reading is this one):
 * request b proposed only its first k_b = draft_len[b] drafts, 0 <= k_b <= k, and
 * is verified exactly as a call with k = k_b would verify it: slots 0..k_b-1 are
 * judged, a <= k_b, after k_b acceptances the bonus comes from target row k_b
 * (p_kb), and out_tokens[b*(k+1) + j] = -1 for j > a. Layouts keep the stride
 * k: hidden / target_hidden [B, k+1, H], draft_hidden [B, k, H], draft_tokens
 * [B, k]; rows and drafts past k_b are not used (drafts there may hold any
 * value). draft_len [B] int32 on the device, or NULL for k_b = k everywhere; a
 * value outside [0, k] is clamped into it and sets MTPV_DEVERR_DRAFT_LEN.
 * Philox uniforms as in spec_verify_sample (slot j, request b). Workspace,
 * debug exports and errors as for spec_verify_greedy / spec_verify_sample.
 */
MTPV_API int spec_verify_greedy_ragged(const void* hidden, const void* W_lm, const int32_t* draft_tokens,
                       const int32_t* draft_len, int B, int k, int H, int V, int dtype,
                       int32_t* accepted_len, int32_t* out_tokens,
                       void* workspace, size_t workspace_bytes,
                       const mtpv_debug* debug, void* stream);
MTPV_API int spec_verify_sample_ragged(const void* target_hidden, const void* draft_hidden, const void* W_lm,
                       const int32_t* draft_tokens, const int32_t* draft_len, int B, int k, int H, int V,
                       int dtype, double temperature, uint64_t seed, uint64_t offset,
                       int32_t* accepted_len, int32_t* out_tokens,
                       void* workspace, size_t workspace_bytes,
                       const mtpv_debug* debug, void* stream);

/*
 * Greedy and stochastic verification of the same drafts from one pass over W_lm
 * (both outcomes for A/B acceptance metrics, "Faster Rollouts with MTP
 * Speculative Decoding", section "Monitoring acceptance"): the head runs once
 * over the target and drafter rows as in spec_verify_sample; then
 * accepted_len_greedy / out_tokens_greedy are exactly what spec_verify_greedy
 * returns for (target_hidden, draft_tokens) and accepted_len_sample /
 * out_tokens_sample exactly what spec_verify_sample returns. draft_len as in
 * spec_verify_sample_ragged (NULL = k everywhere). The four output arrays must
 * not overlap. Workspace: mtpv_workspace_bytes(..., MTPV_MODE_SAMPLE). Debug
 * exports are those of the stochastic pass.
 */
MTPV_API int spec_verify_dual(const void* target_hidden, const void* draft_hidden, const void* W_lm,
                       const int32_t* draft_tokens, const int32_t* draft_len, int B, int k, int H, int V,
                       int dtype, double temperature, uint64_t seed, uint64_t offset,
                       int32_t* accepted_len_greedy, int32_t* out_tokens_greedy,
                       int32_t* accepted_len_sample, int32_t* out_tokens_sample,
                       void* workspace, size_t workspace_bytes,
                       const mtpv_debug* debug, void* stream);

/*
 * Input fusion of the MTP module in front of the drafter ("The Tiny Draft Model
 * Hidden Inside Qwen", section "One step deeper than the main model": the module
 * takes the main model's final hidden state and the embedding of the chosen token,
 * normalizes both, concatenates them and projects back to the hidden width with
 * mtp.fc; the embedding table is the main model's, section "What vLLM and SGLang do
 * with the weights"). The page's formula did not survive; the reading is
 *   n(v)   = v / sqrt(mean(v^2) + eps) * g                 (RMS normalization)
 *   x[b]   = [ n(embed[tokens[b]]; norm_emb) | n(hidden[b]; norm_hidden) ]   (2H)
 *   out[b] = x[b] . W_fc^T                                  (no bias)
 * tokens [B] int32; embed [V, H], hidden [B, H], norm_emb [H], norm_hidden [H],
 * W_fc [H, 2H] (rows = outputs): bf16, row-major, 16-byte aligned, H % 8 == 0;
 * out [B, H] fp32. The fused input is rounded to bf16 (the projection's input
 * type) after fp32 normalization; the product accumulates in fp32. A token outside
 * [0, V) contributes a zero embedding half and sets MTPV_DEVERR_TOKEN_RANGE.
 * eps >= 0 and finite. Workspace: mtpv_fuse_workspace_bytes(B, H).
 */
MTPV_API size_t mtpv_fuse_workspace_bytes(int B, int H);
MTPV_API int mtp_input_fuse(const int32_t* tokens, const void* embed, const void* hidden,
                       const void* norm_emb, const void* norm_hidden, const void* W_fc,
                       int B, int H, int V, double eps, float* out,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Top-k soft cross-entropy draft loss ("Faster Rollouts with MTP Speculative
 * Decoding", SkyRL docs, sections "Overview" and "How does it work?": the MTP head is
 * trained toward the detached policy's next-token distribution with a soft
 * cross-entropy over the policy's top-k tokens; k = 256 in the section "Example").
 * The page prints no formula; the reading is, per row n:
 *   K       = the topk tokens with the largest teacher logits (equal logits: lower
 *             token id first; -0.0 and +0.0 are equal)
 *   pt_j    = softmax over the kept teacher logits (j in K)
 *   loss[n] = logsumexp_v(student[n, v]) - sum_{j in K} pt_j * student[n, j]
 *   grad    = grad_scale * (softmax(student[n]) - pt scattered on K)
 * teacher, student [N, V] fp32 row-major (device); loss [N] fp32 (device, output);
 * topk_index [N, topk] int32 (device, output, may be NULL): the kept ids, largest
 * teacher logit first; grad [N, V] fp32 (device, output, may be NULL: no gradient
 * pass). 1 <= topk <= min(V, MTPV_LOSS_MAX_TOPK); N >= 0 (N = 0 does nothing);
 * V <= 2^30. Logits must not be NaN, and every student row needs a finite logit.
 * Rows whose start is 16-byte aligned (V % 4 == 0, aligned bases) take 16-byte loads.
 * Workspace: mtpv_loss_workspace_bytes(N, topk), 256-byte aligned, caller-owned;
 * its contents are scratch. Errors: MTPV_EINVAL (sizes, non-finite grad_scale),
 * MTPV_ENULL, MTPV_EALIGN (a pointer not 4-byte aligned), MTPV_EWORKSPACE.
 */
#define MTPV_LOSS_MAX_TOPK 512
MTPV_API size_t mtpv_loss_workspace_bytes(int N, int topk);
MTPV_API int mtp_draft_loss_topk(const float* teacher, const float* student, int N, int V, int topk,
                            float grad_scale, float* loss, int32_t* topk_index, float* grad,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * Drafter-side sampling through the same shared head: for each request b and
 * drafter row j (0..kd-1), draft_tokens[b*kd + j] ~ softmax(l(drafter row) / T),
 * drawn by inverse transform with uniform(word 2 of Philox(seed; depth0 + j, b,
 * offset)). The MTP module proposes tokens through the main model's head ("The
 * Tiny Draft Model Hidden Inside Qwen", section "What vLLM and SGLang do with
 * the weights"); a chained drafter calls this once per depth with kd = 1 and
 * depth0 = depth, and the verify call then sees the same Philox stream.
 * draft_hidden [B, kd, H]; draft_tokens [B, kd] int32 (output).
 * Workspace: mtpv_workspace_bytes(B, kd, H, V, dtype, MTPV_MODE_DRAFT).
 */
MTPV_API int spec_draft_sample(const void* draft_hidden, const void* W_lm, int B, int kd, int depth0,
                      int H, int V, int dtype, double temperature, uint64_t seed, uint64_t offset,
                      int32_t* draft_tokens, void* workspace, size_t workspace_bytes,
                      const mtpv_debug* debug, void* stream);

/*
 * Reads the device error word (the sticky MTPV_DEVERR_* bits) of the last call
 * that used this workspace: waits for the stream, then copies the word to *err
 * (0 = no error).
 */
MTPV_API int mtpv_get_device_error(const void* workspace, int32_t* err, void* stream);

/*
 * Measurement hooks. mtpv_timing_enable(every) with every >= 1 makes one call in
 * `every` (the 1st, the every+1-th, ... after enabling or a reset read) record a
 * pair of HIP events on its stream around its dominant kernel: the LM-head kernel
 * (the kernel that streams W_lm), or the selection kernel of mtp_draft_loss_topk.
 * every = 1 times every call; every = 0 turns the hooks off; every < 0 returns
 * MTPV_EINVAL. Each event pair adds a few microseconds to the call that records
 * it, so a loop whose rate is measured at the same time times only a sample of
 * its calls. _read waits for those events and returns the summed kernel time in
 * milliseconds and the number of timed launches, then clears them (and restarts
 * the count of calls) if reset != 0. At most 65536 launches are kept between
 * reads; later ones are not timed.
 */
MTPV_API int mtpv_timing_enable(int every);
MTPV_API int mtpv_timing_read(double* ms_total, int64_t* launches, int reset);

/*
 * Plain device-to-device copy of `bytes` bytes with 16-byte vector loads and
 * stores (bytes and both pointers 16-byte aligned). It is the reference kernel
 * that scales hardware byte counters for traffic measurements.
 */
MTPV_API int mtpv_copy_bytes(void* dst, const void* src, size_t bytes, void* stream);

/*
 * Achievable-rate probes, for reporting the verify kernels against what plain
 * kernels reach on the same part (beside the published peaks). Measurement only:
 * they compute nothing of the method and write nothing the caller reads.
 *
 * mtpv_read_bytes: one read sweep of `bytes` bytes at `src` (device pointer,
 * 16-byte aligned, bytes % 16 == 0; 0 bytes launches nothing) with 16-byte
 * non-temporal loads, each workgroup reading 8 KB blocks spaced by the grid. `sink` is a
 * 4-byte-aligned device word the kernel could write but never does. Errors:
 * MTPV_ENULL, MTPV_EALIGN, MTPV_ELAUNCH.
 *
 * mtpv_mfma_rate: 256 workgroups of 4 waves, each wave issuing `iters` rounds of 16
 * independent v_mfma_f32_16x16x32_bf16 (bf16 operands of magnitude 0.5 to 2 with
 * varied bits, fp32 accumulation in registers); *flops receives the flops of the
 * launch (256 * 4 * iters * 16 * 16384). `sink` as above. iters in [1, 2^24], else
 * MTPV_EINVAL. Time either with events on `stream`.
 */
MTPV_API int mtpv_read_bytes(const void* src, size_t bytes, void* sink, void* stream);
MTPV_API int mtpv_mfma_rate(int iters, void* sink, int64_t* flops, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MTPV_H_ */
