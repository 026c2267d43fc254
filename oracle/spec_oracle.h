/* spec_oracle.h - plain fp64 CPU oracle of the speculative-sampling verify step.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or helper with the HIP library; the two meet only at the
 * seeded input generator.
 *
 * Logit storage codes: 0 = fp32, 1 = bf16 (uint16 bits), 2 = fp64.
 * Every value is widened exactly to double before use.
 */
#ifndef SPEC_ORACLE_H
#define SPEC_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Decision flags reported per sequence. */
#define ORACLE_FLAG_TEST_NEAR  1  /* a taken acceptance test had |u - alpha| < 1e-5            */
#define ORACLE_FLAG_DRAW_NEAR  2  /* the final draw had u*S within 1e-5 of a CDF boundary        */
#define ORACLE_FLAG_FALLBACK   4  /* residual mass was exactly 0 after a reject; drew from p_n   */

#define ORACLE_NEAR 1e-5

typedef struct {
    double*  p_tok;        /* [B,K]   p_j(x_j) for tested j, NaN elsewhere                 */
    double*  q_tok;        /* [B,K]   q_j(x_j) for tested j, NaN elsewhere                 */
    double*  lse_p;        /* [B,K+1] log sum exp(l/T) for examined target rows, NaN else   */
    double*  lse_q;        /* [B,K]   same for examined draft rows                          */
    double*  res_mass;     /* [B]     S of the final draw (1 for the bonus, 0 greedy)       */
    double*  test_margin;  /* [B,K]   |u_j - alpha_j| for tested j                           */
    double*  draw_margin;  /* [B]     distance of u*S from the nearest CDF boundary         */
    int32_t* flags;        /* [B]     ORACLE_FLAG_* bits                                     */
} oracle_diag;

/* softmax(l/T) of one row.  Returns 1 and fills p[V], *lse if the row is
 * valid; returns 0 if it holds NaN or +Inf or is all -Inf. */
int oracle_row_softmax(const void* row, int dtype, int32_t V, double T, double* p, double* lse);

/* Index of the largest logit (lowest index among equals).  Returns 1 and
 * sets *idx if valid, 0 on NaN, +Inf or an all -Inf row. */
int oracle_row_argmax(const void* row, int dtype, int32_t V, int32_t* idx);

/* Inverse-CDF draw from the unnormalised non-negative weights r[V] with the
 * uniform u: smallest i whose running sum (ascending i) exceeds u*S.  Sets
 * *S, *margin (distance of u*S from the nearest boundary of the chosen
 * token's interval, in the units of r).  Returns y, or -1 if S == 0. */
int32_t oracle_draw(const double* r, int32_t V, double u, double* S, double* margin);

/* The whole verify step for B sequences (see spec_oracle.c for the steps).
 * target [B,K+1,V] stored as dtype, draft [B,K,V] stored as ddtype (may be
 * NULL when K == 0 or all greedy),
 * tokens [B,K], uniforms [B,K+1] fp32, greedy [B] (NULL = all sampling).
 * Outputs accepted_len [B] (-1 = invalid input) and out_tokens [B,K+1]
 * (padding -1).  diag may be NULL; each of its pointers may be NULL.
 * nthreads <= 0 uses one thread.  Returns 0, or -1 on bad arguments. */
int oracle_verify(const void* target, int dtype, const void* draft, int ddtype,
                  const int32_t* tokens, const float* uniforms, double T,
                  const uint8_t* greedy, int32_t B, int32_t K, int32_t V,
                  int32_t* accepted_len, int32_t* out_tokens,
                  const oracle_diag* diag, int nthreads);

#ifdef __cplusplus
}
#endif
#endif
