/* spec_verify.h - C ABI of the gfx950 (MI355X) speculative-sampling verify step.
 *
 * The verify step of speculative decoding: given the target model's logits at
 * K+1 positions and the draft model's logits at K positions over the whole
 * vocabulary, together with the K draft tokens, decide how many draft tokens
 * survive and which token ends the round.  Sources, cited by page and section:
 *
 *   [QH] quochung.cyou, "A.I" category page, speculative decoding tutorial:
 *        "Chọn token: greedy vs sampling" (greedy = most likely token;
 *        sampling = draw in proportion), "Một vòng speculative decoding" and
 *        "Draft model kém hơn target..." (greedy verify, left-to-right
 *        comparison, the tail after a mismatch is dropped unchecked),
 *        "Modified rejection sampling" with "Giải pháp" (acceptance
 *        probability min(1, p/q)), "Khi reject thì lấy token từ đâu?"
 *        (correction from the normalised residual max(0, p - q)), "Toàn bộ
 *        thuật toán cho một token" and "Áp dụng thuật toán" (first rejection
 *        ends the round; all K accepted -> one bonus token from the target).
 *   [NL] nalar.dev, "Speculative decoding: memverifikasi token draft secara
 *        paralel": "Sampling eksak memerlukan aturan koreksi" (a(x) and the
 *        residual r(x)), "Penolakan memotong prefix yang diterima" (a
 *        rejection truncates the accepted prefix).
 *   [MC] ml-canon-ru card 57 "Speculative Decoding": "Приёмка и почему
 *        распределение НЕ портится" (alpha, the residual, the exactness
 *        identity) and its sketch of one round (strict u < alpha).
 *
 * Conventions fixed here where the pages leave a step open:
 *   - p = softmax(target_logits / T), q = softmax(draft_logits / T), T > 0.
 *   - Test j (j < K) accepts draft token x_j iff u[b,j] * q_j(x_j) < p_j(x_j),
 *     i.e. u < min(1, p/q) with q(x) = 0 meaning alpha = 1 if p(x) > 0, else 0.
 *   - The one final draw uses u[b,K] by inverse CDF over ascending token
 *     index: the smallest i whose running sum of the weights exceeds u * S.
 *     Weights: max(0, p_n - q_n) after a rejection at n (p_n if that sum
 *     rounds to 0), or p_K for the bonus token.
 *   - Greedy sequences: accept x_j iff it equals the lowest-index argmax of the
 *     raw target logits of row j; the final token is that argmax of row n.
 *     They ignore temperature, uniforms and draft logits.
 *
 * Memory: every array argument is a DEVICE pointer owned by the caller,
 * row-major and contiguous, aligned to its element size (16-byte-aligned rows
 * take the vector path; other rows are still handled).  The library
 * allocates and frees nothing.  All calls are asynchronous on `stream` (a
 * hipStream_t; NULL = the default stream) and return after enqueueing.
 *
 * Errors: 0 = OK.  Negative codes are host-detected and nothing is launched:
 *   SV_EINVAL    shape out of range (B < 0, K not in [0, SV_MAX_K], V < 1),
 *                unknown dtype, temperature not finite and > 0, a required
 *                pointer NULL or misaligned, grid too large.
 *   SV_EWORKSPACE workspace NULL, misaligned (16 B) or smaller than
 *                sv_workspace_bytes().
 *   SV_ELAUNCH   the HIP launch failed.
 *   SV_ESCRATCH  (spec_verify_noalloc only) the shape needs more workspace
 *                than the library's static scratch array holds.
 * Per-sequence input faults are reported on the device: a row the method
 * examines that holds NaN or +Inf or is all -Inf, a token outside [0, V), a
 * uniform outside [0, 1) that the method uses, or a sampling sequence with
 * draft_logits == NULL gives accepted_len[b] = -1 and out_tokens[b,:] = -1;
 * other sequences are unaffected.  -Inf logits are legal (masked tokens).
 * Rows past the first rejection never change the result.
 *
 * Determinism: identical inputs give bitwise-identical outputs.
 * Concurrency: calls that share a workspace must be ordered on one stream.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SV_F32  0   /* fp32 logits */
#define SV_BF16 1   /* bf16 logits (uint16 storage) */

#define SV_OK          0
#define SV_EINVAL     -1
#define SV_EWORKSPACE -2
#define SV_ELAUNCH    -3
#define SV_ESCRATCH   -4

#define SV_GAVE_UP    -2   /* accepted_len of a sequence whose SV_MODE_SEQ wait gave up */

#define SV_MAX_K 63
#define SV_MAX_NGRAM 64

/* Optional diagnostics: a host struct of device pointers, each may be NULL.
 * Entries the method never examines (positions after the first rejection,
 * greedy sequences, invalid sequences) are NaN.                              */
typedef struct sv_diag {
    float* p_tok;     /* [B,K]   p_j(x_j) at tested positions j <= n          */
    float* q_tok;     /* [B,K]   q_j(x_j) at tested positions                 */
    float* lse_p;     /* [B,K+1] ln sum_i exp(l_i/T) for target rows j <= n   */
    float* lse_q;     /* [B,K]   same for draft rows j <= min(n, K-1)         */
    float* res_mass;  /* [B]     S of the final draw in probability units:
                                 sum max(0, p_n - q_n), ~1 for the bonus,
                                 0 for greedy, 0 if the residual fell back    */
} sv_diag;

/* Bytes of device workspace spec_verify needs for this shape (0 for B == 0).
 * No initialisation is needed; calls sharing one workspace must be ordered
 * on one stream.                                                            */
size_t sv_workspace_bytes(int32_t B, int32_t K, int32_t V, int32_t dtype);

/* The whole verify step (steps: row statistics, acceptance tests, first
 * rejection, final draw, emit).
 *   target_logits [B, K+1, V] dtype    draft_logits [B, K, V] dtype (may be
 *   NULL when K == 0 or every sequence is greedy)
 *   draft_tokens  [B, K] int32 (NULL allowed only when K == 0)
 *   uniforms      [B, K+1] fp32 in [0,1): column j < K tests position j,
 *                 column K drives the final draw
 *   temperature   shared by p and q
 *   greedy_flag   [B] uint8, 1 = greedy sequence; NULL = all sampling
 * Outputs:
 *   accepted_len  [B] int32: n in [0, K] accepted draft tokens, -1 = invalid
 *                 input, SV_GAVE_UP (-2) = a SV_MODE_SEQ wait gave up (the
 *                 row is then unspecified)
 *   out_tokens    [B, K+1] int32: x_0..x_{n-1}, then the correction or bonus
 *                 token, then -1 padding.                                    */
int spec_verify(const void* target_logits, const void* draft_logits,
                const int32_t* draft_tokens, const float* uniforms,
                float temperature, const uint8_t* greedy_flag,
                int32_t B, int32_t K, int32_t V, int32_t dtype,
                int32_t* accepted_len, int32_t* out_tokens, const sv_diag* diag,
                void* workspace, size_t workspace_bytes, void* stream);

/* spec_verify with the schedule chosen for this call only (SV_MODE_AUTO:
 * the automatic rule; SV_MODE_EAGER / SV_MODE_LAZY / SV_MODE_SEQ as
 * sv_set_mode describes), whatever the process-wide mode is: e.g. a caller
 * that runs other work on the device at the same time asks for
 * SV_MODE_EAGER, which assumes nothing about which workgroups run together.
 * SV_EINVAL for another mode value; otherwise as spec_verify.             */
int spec_verify_mode(int mode, const void* target_logits, const void* draft_logits,
                     const int32_t* draft_tokens, const float* uniforms,
                     float temperature, const uint8_t* greedy_flag,
                     int32_t B, int32_t K, int32_t V, int32_t dtype,
                     int32_t* accepted_len, int32_t* out_tokens, const sv_diag* diag,
                     void* workspace, size_t workspace_bytes, void* stream);

/* spec_verify with separate storage types for the target and the draft
 * logits (each SV_F32 or SV_BF16), e.g. fp32 target logits straight from an
 * LM head with bf16 draft logits.  Same arguments, outputs and errors.      */
int spec_verify_ex(const void* target_logits, const void* draft_logits,
                   const int32_t* draft_tokens, const float* uniforms,
                   float temperature, const uint8_t* greedy_flag,
                   int32_t B, int32_t K, int32_t V, int32_t target_dtype, int32_t draft_dtype,
                   int32_t* accepted_len, int32_t* out_tokens, const sv_diag* diag,
                   void* workspace, size_t workspace_bytes, void* stream);

/* spec_verify for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, outputs and errors as spec_verify with dtype for both
 * target and draft logits, minus the workspace: the call uses a static
 * device array of sv_noalloc_scratch_bytes() (16 MiB) instead, which each
 * GPU the library runs on holds until the process ends (looked up on the
 * first call on each device).  The call allocates and frees nothing.
 * SV_ESCRATCH (nothing launched) when sv_workspace_bytes(B, K, V, dtype)
 * exceeds that size; SV_ELAUNCH when the array's device address cannot be
 * obtained (sv_last_hip_error() tells why).  Every call on one GPU shares its
 * array, which keeps the last call's contents (nothing in it needs to start
 * at zero): calls that may overlap on one GPU (several streams, several
 * threads) race and give undefined results; order them on one stream.   */
int spec_verify_noalloc(const void* target_logits, const void* draft_logits,
                        const int32_t* draft_tokens, const float* uniforms,
                        float temperature, const uint8_t* greedy_flag,
                        int32_t B, int32_t K, int32_t V, int32_t dtype,
                        int32_t* accepted_len, int32_t* out_tokens, const sv_diag* diag,
                        void* stream);
size_t sv_noalloc_scratch_bytes(void);

/* The same call in two parts, for timing and for checking the parts against
 * the whole: sv_stats streams the target rows, and the draft rows of
 * sampling sequences, once into per-chunk statistics (the HBM-bound part);
 * sv_draw settles n, writes the outputs and makes the final draw of sampling
 * sequences.  sv_draw must follow sv_stats on the same stream with identical
 * arguments and the same schedule (sv_set_mode).  Under SV_MODE_SEQ the
 * whole step runs in sv_stats and sv_draw launches nothing.                 */
int sv_stats(const void* target_logits, const void* draft_logits,
             const int32_t* draft_tokens, const float* uniforms,
             float temperature, const uint8_t* greedy_flag,
             int32_t B, int32_t K, int32_t V, int32_t dtype,
             int32_t* accepted_len, int32_t* out_tokens, const sv_diag* diag,
             void* workspace, size_t workspace_bytes, void* stream);
int sv_draw(const void* target_logits, const void* draft_logits,
            const int32_t* draft_tokens, const float* uniforms,
            float temperature, const uint8_t* greedy_flag,
            int32_t B, int32_t K, int32_t V, int32_t dtype,
            int32_t* accepted_len, int32_t* out_tokens, const sv_diag* diag,
            void* workspace, size_t workspace_bytes, void* stream);

/* ---- fused LM head ------------------------------------------------------
 * The target's last step maps each final hidden vector of d values to one
 * score per vocabulary token ([QH] "Hidden state": the LM head turns the last
 * hidden state into the table over the vocabulary).  The K+1 verify positions
 * of B sequences share the weight:
 *     target_logits[m, v] = sum_k hidden[m, k] * W[k, v]   (m < B*(K+1)),
 * bf16 inputs, fp32 accumulation and output.
 *
 * sv_lmhead_packed_bytes: bytes of the packed weight for W [d, V]:
 *   ceil(V/256) * 8 * ceil(d/16) * 1024; 0 when d < 1 or V < 1.
 * sv_lmhead_pack: one-time repack of the static weight from W [d, V] (bf16,
 *   row-major) into w_packed, the matrix-core operand tiles the GEMM streams:
 *   with KT = ceil(d/16), tile (vt, kt), vt < ceil(V/32), kt < KT, is 1 KB at
 *   offset ((vt/8 * KT + kt) * 8 + vt%8) * 1024 bytes (the 8 tiles of each
 *   256 columns alternate per k-tile); its bf16 element l*8 + e (l < 64,
 *   e < 8) is W[kt*16 + 8*(l/32) + e][vt*32 + l%32], 0 past d or V.  Tiles
 *   past ceil(V/32) in the last group are not written.
 *   Both caller-owned device buffers, w_packed of sv_lmhead_packed_bytes.
 *   EINVAL on d < 1, V < 1, NULL pointers, w_dv not 2-byte or w_packed not
 *   16-byte aligned.
 * sv_lmhead: logits [M, V] fp32 = hidden [M, d] bf16 x W, W given as
 *   w_packed.  d must be a multiple of 8 and hidden / w_packed 16-byte
 *   aligned (EINVAL otherwise); M == 0 is a no-op.
 * spec_lmhead_verify: sv_lmhead on hidden [B, K+1, d] into the caller's
 *   target_logits [B, K+1, V] fp32 buffer, then the verify step of
 *   spec_verify on those logits with draft logits of draft_dtype.  Every
 *   check of both parts runs before anything is launched; outputs, errors
 *   and workspace as spec_verify (size it with dtype SV_F32).
 *   Deviation from a plain w_lm [d, V] argument: the weight is taken packed
 *   (sv_lmhead_pack, once per static weight), because the GEMM streams it in
 *   matrix-core operand order (measured 351 -> 271 us for W [4096, 128256]
 *   against reading rows of W^T directly).                               */
size_t sv_lmhead_packed_bytes(int32_t d, int32_t V);
int sv_lmhead_pack(const void* w_dv, void* w_packed, int32_t d, int32_t V, void* stream);
int sv_lmhead(const void* hidden, const void* w_packed, int32_t M, int32_t d, int32_t V,
              float* logits, void* stream);
int spec_lmhead_verify(const void* hidden, const void* w_packed, int32_t d, float* target_logits,
                       const void* draft_logits, int32_t draft_dtype, const int32_t* draft_tokens,
                       const float* uniforms, float temperature, const uint8_t* greedy_flag,
                       int32_t B, int32_t K, int32_t V, int32_t* accepted_len, int32_t* out_tokens,
                       const sv_diag* diag, void* workspace, size_t workspace_bytes, void* stream);

/* spec_lmhead_verify in two calls, for timing the parts: _gemm launches the
 * LM head, _rest the verify step on its logits.  Same arguments and checks
 * as spec_lmhead_verify; _rest must follow _gemm on the same stream with
 * identical arguments.                                                    */
int sv_lmhead_verify_gemm(const void* hidden, const void* w_packed, int32_t d, float* target_logits,
                          const void* draft_logits, int32_t draft_dtype, const int32_t* draft_tokens,
                          const float* uniforms, float temperature, const uint8_t* greedy_flag,
                          int32_t B, int32_t K, int32_t V, int32_t* accepted_len, int32_t* out_tokens,
                          const sv_diag* diag, void* workspace, size_t workspace_bytes, void* stream);
int sv_lmhead_verify_rest(const void* hidden, const void* w_packed, int32_t d, float* target_logits,
                          const void* draft_logits, int32_t draft_dtype, const int32_t* draft_tokens,
                          const float* uniforms, float temperature, const uint8_t* greedy_flag,
                          int32_t B, int32_t K, int32_t V, int32_t* accepted_len, int32_t* out_tokens,
                          const sv_diag* diag, void* workspace, size_t workspace_bytes, void* stream);

/* ---- draft-side sampling step ---------------------------------------------
 * Each draft pass draws its candidate x ~ q = softmax(d / T) ([QH] "Một vòng":
 * the drafter proposes its candidates one pass at a time; [MC]'s sketch
 * samples from draft.probs).  sv_sample draws one token per row of
 * logits [B, V] (dtype SV_F32 / SV_BF16) with uniforms [B] in [0, 1) by the
 * same inverse CDF as the final draw (ascending token index); greedy rows
 * (greedy_flag[b] = 1; NULL = none) take the lowest-index argmax.  Outputs
 * tokens [B] (-1 for an invalid row: NaN / +Inf / all -Inf logits or a
 * uniform outside [0, 1)) and optionally lse [B] = ln sum_i exp(d_i / T)
 * (NaN for greedy rows).  It is the verify step with K = 0 and shares its
 * kernels; workspace from sv_sample_workspace_bytes.  Errors as spec_verify. */
size_t sv_sample_workspace_bytes(int32_t B, int32_t V, int32_t dtype);
int sv_sample(const void* logits, int32_t dtype, const float* uniforms, float temperature,
              const uint8_t* greedy_flag, int32_t B, int32_t V, int32_t* tokens, float* lse,
              void* workspace, size_t workspace_bytes, void* stream);

/* ---- KV-cache commit ---------------------------------------------------------
 * After verification only the accepted prefix may become committed decoding
 * state ([NL] "Verifikasi mengubah jalur cache": truncation, staged writes or
 * index management).  Caches are P planes (e.g. keys and values of every
 * layer) of B sequences of l_max rows of row_bytes bytes:
 *   cache  [P, B, l_max, row_bytes]    cache_len [B] int32 (in: committed
 *   length before the round; out: after)
 *   staged [P, B, K + offset, row_bytes]: the entries the pass computed for
 *   its inputs; offset = 1 when they start with the previous round's final
 *   token, 0 when they hold the K candidates only.
 * With c_b = accepted_len[b] + offset, rows staged[:, b, 0:c_b] are copied to
 * cache[:, b, len_b : len_b + c_b] and len_b grows by c_b.  staged == NULL
 * means the pass wrote the entries in place at [len_b, len_b + K + offset):
 * committing is then the length update alone.  accepted_len[b] = -1 or a
 * commit that would pass l_max leaves sequence b unchanged; status [B]
 * (optional) gets 0 committed, 1 invalid, 2 would overflow.  Works for the
 * draft model's cache the same way.  EINVAL on P < 1, K out of range, offset
 * not 0/1, l_max < 1, row_bytes < 1, NULL or misaligned (4 B) int arrays. */
int sv_kv_commit(void* cache, int32_t* cache_len, const void* staged, const int32_t* accepted_len,
                 int32_t planes, int32_t B, int32_t K, int32_t offset, int64_t l_max, int64_t row_bytes,
                 int32_t* status, void* stream);

/* ---- prompt lookup ------------------------------------------------------
 * Candidates without a draft model ([QH] "Vấn đề 3: Làm sao khi không muốn
 * train drafter?": the continuation of an earlier occurrence of the text's
 * ending, then target verification).
 *
 * sv_lookup_propose: history [B, Lmax] int32 token ids, row b holding
 *   hist_len[b] tokens (prompt and output so far).  For n = n_max down to
 *   n_min, the first n whose last-n-token ending occurs earlier in the
 *   history with at least one token after the occurrence wins; the earliest
 *   such occurrence is used.  Outputs cand [B, K] int32 (the up to K tokens
 *   after it, clipped at the history's end, then -1) and klen [B] int32 (how
 *   many; 0 without a match; -1 when hist_len[b] is outside [0, Lmax]).
 *   EINVAL on B < 0, Lmax < 0, n_min < 1, n_max < n_min, n_max >
 *   SV_MAX_NGRAM, K outside [0, SV_MAX_K], NULL or misaligned (4 B) arrays.
 * spec_verify_lookup: the verify step on such candidates.  A deterministic
 *   proposal is a one-hot draft distribution (all of q on the proposed
 *   token), so with [MC] "Приёмка и почему распределение НЕ портится" a
 *   sampling sequence accepts x_j iff u[b,j] < p_j(x_j), and after a
 *   rejection draws from p_n without x_n (renormalised); greedy sequences
 *   compare with the argmax.  Sequence b has klen[b] candidates (cand
 *   [B, K], entries past klen[b] never read): after klen[b] acceptances the
 *   bonus token comes from p_{klen[b]}; column K of the uniforms drives the
 *   final draw in every case; target rows past klen[b] are never read.
 *   klen[b] outside [0, K] marks the sequence invalid (accepted_len -1).
 *   Other arguments, outputs, workspace and errors as spec_verify (no draft
 *   logits; q_tok reports 1 and lse_q 0 for tested positions).  Schedule:
 *   SV_MODE_SEQ when the mode asks for it or, under SV_MODE_AUTO, when
 *   position 0's target rows alone are at least 64 MiB (and the vocabulary
 *   fits that schedule's limit); otherwise eager (SV_MODE_LAZY runs eager:
 *   the per-position launches take no one-hot rows).                     */
int sv_lookup_propose(const int32_t* history, const int32_t* hist_len, int32_t B, int32_t Lmax,
                      int32_t n_max, int32_t n_min, int32_t K, int32_t* cand, int32_t* klen, void* stream);
int spec_verify_lookup(const void* target_logits, int32_t dtype, const int32_t* cand, const int32_t* klen,
                       const float* uniforms, float temperature, const uint8_t* greedy_flag,
                       int32_t B, int32_t K, int32_t V, int32_t* accepted_len, int32_t* out_tokens,
                       const sv_diag* diag, void* workspace, size_t workspace_bytes, void* stream);

/* Row-statistics schedule, process-wide (thread-safe; a tuning knob: every
 * schedule meets the same definition, though float sums taken in another
 * order may settle a draw within rounding of a boundary differently):
 *   SV_MODE_AUTO  per call: SV_MODE_SEQ when position 0 alone streams at
 *                 least 64 MiB, or at least 16 MiB with K > 0, B <= 64 and
 *                 bf16 target logits, or for K = 0 with V a multiple of 8
 *                 (and the vocabulary fits its limit), else lazy
 *                 when one eager pass would stream at least 64 MiB of logits
 *                 per position (K+1 launches then pay off), else eager
 *   SV_MODE_EAGER one launch streams every row of every position
 *   SV_MODE_LAZY  one launch per position streams it only for sequences that
 *                 reach it (rows past the first rejection are never read)
 *   SV_MODE_SEQ   one launch, one workgroup per sequence walking its own
 *                 positions up to the first rejection and drawing at the end;
 *                 vocabularies above 2,097,152 entries use SV_MODE_LAZY
 * The environment variable SV_MODE=eager|lazy|seq sets the initial value.
 * sv_set_mode returns SV_EINVAL for other values.                          */
#define SV_MODE_AUTO  0
#define SV_MODE_EAGER 1
#define SV_MODE_LAZY  2
#define SV_MODE_SEQ   3
int sv_set_mode(int mode);
int sv_get_mode(void);

/* The schedule (SV_MODE_EAGER, SV_MODE_LAZY or SV_MODE_SEQ) a verify call of
 * this shape and these storage types would use under the current mode;
 * SV_EINVAL for a shape or type the call would reject.                     */
int sv_schedule(int32_t B, int32_t K, int32_t V, int32_t target_dtype, int32_t draft_dtype);

/* Under SV_MODE_SEQ each sequence gets G workgroups that split every row it
 * reaches and exchange partial statistics through the workspace (tagged
 * words; nothing to initialise), G as large as the device holds all of them
 * at once; with lookahead (below) G stops at the fewest workgroups that
 * cover a row in one pass of their loads (1 KiB x 16 per workgroup for
 * bf16 rows, x 8 when a row is fp32), since every further workgroup only
 * lengthens the exchange; G = 1 is one 1024-thread workgroup per sequence.
 * sv_set_seq_groups caps G (1..64; 0 = no cap, the default; the environment
 * variable SV_SEQ_GROUPS sets the initial cap); SV_EINVAL otherwise.
 * sv_seq_groups: the G a call of this shape would use now (0 when it would
 * not run SV_MODE_SEQ), SV_EINVAL for a shape the call would reject.       */
int sv_set_seq_groups(int groups);
int sv_seq_groups(int32_t B, int32_t K, int32_t V, int32_t target_dtype, int32_t draft_dtype);

/* Lookahead of SV_MODE_SEQ (K > 0, several workgroups per sequence): with 1
 * the workgroups of a sequence stream position j+1 before they settle
 * position j, which hides the exchange's round trip behind a stream at the
 * price of one position read past the first rejection (never used; rows past
 * the rejection still never change the result); with 0 they stream a
 * position only once the previous one is settled; with 2 they run two
 * positions ahead (two rows read past the rejection).  sv_set_seq_lookahead:
 * -1 = by shape (the default: 1 while position 0 alone streams less than
 * 64 MiB, else 0; the environment variable SV_SEQ_LOOKAHEAD=0|1|2 sets an
 * initial override), 0, 1 or 2 to force it; SV_EINVAL otherwise.
 * sv_seq_lookahead: the lookahead a call of this shape would use now (0 when
 * it would not run SV_MODE_SEQ with several workgroups per sequence),
 * SV_EINVAL for a shape the call would reject.                            */
int sv_set_seq_lookahead(int lookahead);
int sv_seq_lookahead(int32_t B, int32_t K, int32_t V, int32_t target_dtype, int32_t draft_dtype);

/* Every wait of the SV_MODE_SEQ exchange is bounded: after this many polls
 * (each one load round trip, about 1 us, so the default bounds a wait
 * at roughly a second) it gives up and the sequence reports accepted_len
 * SV_GAVE_UP (-2) instead of hanging, e.g. when other work
 * keeps some of the call's workgroups from running at the same time: a
 * launch of this schedule assumes the device holds all its workgroups at
 * once, so verify calls in flight together on several streams (or next to
 * other work that fills the device) belong under SV_MODE_EAGER or
 * SV_MODE_LAZY (spec_verify_mode picks one per call), or in one stream's
 * order.  -2 is distinct from -1 (invalid input): the inputs may be fine and
 * the call can be repeated.  Under -2 the row of out_tokens is unspecified
 * (callers discard it).  A sequence one of whose workgroups gave up while
 * the others completed holds whichever length was stored last: -2, or the
 * valid length, which then always stands next to its whole row (the row is
 * written only by the workgroups that complete, the length last).  The
 * default (polls = 0) is 2^20; smaller values are for tests that force the
 * give-up path.  A sampling sequence's valid accepted_len is written by the
 * workgroup that draws, after the drawn token, so a valid length always
 * stands next to a written token.  Words a give-up leaves in the workspace
 * carry that call's tags and never match a later call, except a replay of
 * the same captured launch.  Process-wide; SV_EINVAL for polls outside
 * 0..2^20.                                                                */
int sv_set_wait_limit(int32_t polls);

/* ---- measurement aid: the HBM ceiling ---------------------------------
 * Not part of the verify step.  The pages compare decoding methods by the
 * memory traffic their kernels move ([QH] "Vấn đề thời gian"; [NL] "Tingkat
 * penerimaan tidak sama dengan speedup"); these two plain streaming kernels
 * measure the HBM rate this GPU reaches, the ceiling the verify kernels are
 * judged against.
 *
 * sv_hbm_probe(SV_PROBE_READ, src, dst, bytes, stream): reads bytes from src
 *   (16-byte non-temporal loads, eight 256-thread workgroups per compute
 *   unit, grid-stride) and writes one 32-bit word per wave (an XOR of what it
 *   read) to dst, which must hold sv_hbm_probe_words() words.
 * sv_hbm_probe(SV_PROBE_COPY, src, dst, bytes, stream): copies bytes from
 *   src to dst with the same loads and non-temporal stores.
 * Device pointers, 16-byte aligned; bytes > 0 and a multiple of 16; the copy's
 * ranges must not overlap.  Asynchronous on stream.  Returns SV_OK, SV_EINVAL
 * (kind, pointers, size or overlap; nothing launched) or SV_ELAUNCH.
 * sv_hbm_probe_words: the words the read writes on the current device, -1 if
 * the device cannot be queried.                                           */
#define SV_PROBE_READ 0
#define SV_PROBE_COPY 1
int sv_hbm_probe(int32_t kind, const void* src, void* dst, size_t bytes, void* stream);
int32_t sv_hbm_probe_words(void);

/* The HIP error code (hipError_t) behind this thread's most recent
 * SV_ELAUNCH, 0 if none yet.  Entry points clear an error left by an earlier
 * HIP call of the caller before launching, so SV_ELAUNCH always means one of
 * this library's launches failed.                                          */
int sv_last_hip_error(void);

/* Short text for a return code (static storage). */
const char* sv_strerror(int code);

/* ABI version of this header: 1. */
int sv_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SPEC_VERIFY_H */
