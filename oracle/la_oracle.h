/*
 * la_oracle.h -- fp64 CPU oracle for decayed causal linear attention ("lightning attention").
 *
 * TEST INFRASTRUCTURE ONLY.  This library exists to check the GPU library.  Only the test
 * suite, the smoke check and the benchmark's CPU-baseline leg may load or call it; the
 * product path never does.  It shares no source with the GPU path.
 *
 * What is computed (all in double precision, plain loops):
 *
 *   For every packed sequence sigma (tokens [cu[sigma], cu[sigma+1]) of a [T, H, D] tensor,
 *   local index t = 0 .. n-1) and every head h with decay lambda = decay[h]:
 *
 *     o_t = sum_{s <= t} lambda^(t-s) (q_t . k_s) v_s   (+ lambda^(t+1) q_t S0 if an initial
 *                                                          state S0 is given)
 *     final_state[a][b] = sum_s lambda^(n-1-s) k_s[a] v_s[b]  (+ lambda^n S0[a][b])
 *
 *   Decode: S' = lambda S + k^T v ; o = q S' ; S <- S'.
 *
 * Sources.  The pages describe lightning attention as causal linear attention computed with
 * an intra-block left product and an inter-block right product that together avoid a slow
 * cumulative sum ("MiniMax-01 technical report digest", futurefh.com, section 1 "core
 * innovation"); linear attention rests on the associativity (QK^T)V = Q(K^T V) (nabfollower
 * blog "MiniMax M2.1", section "The Core Tech: Lightning Attention"); and it runs as a scan
 * over a fixed-size hidden state (same blog, "analogy" section).  The pages never state a
 * decay: the constant per-head decay lambda^(t-s) is this library's stated problem, and the
 * readings taken where the pages are silent (decay placement, lambda = 0, no normaliser,
 * layouts) are the ones listed in the design notes of the repository.
 *
 * Layouts: activations [T][H][D] row-major (D fastest); states [S][H][D][D] with the key
 * index a first (state[a][b]); decay [H]; cu_seqlens [S+1], 0 = cu[0] <= ... <= cu[S] = T.
 * cu_seqlens == NULL means a single sequence of length T.
 *
 * Every function returns 0 on success and -1 on an invalid argument (NULL required pointer,
 * non-positive sizes, non-monotone cu_seqlens).  Nothing is allocated that outlives a call.
 */
#ifndef LA_ORACLE_H
#define LA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* O1: quadratic masked form, every row.  out: [T][H][D].  init_state: [S][H][D][D] or NULL. */
int lao_quadratic(const double *q, const double *k, const double *v, const double *decay,
                  const int32_t *cu_seqlens, int32_t S, int64_t T, int32_t H, int32_t D,
                  const double *init_state, double *out);

/* O1 restricted to selected token rows (global token indices rows[0..nrows-1]).
 * out: [nrows][H][D]. */
int lao_quadratic_rows(const double *q, const double *k, const double *v, const double *decay,
                       const int32_t *cu_seqlens, int32_t S, int64_t T, int32_t H, int32_t D,
                       const double *init_state, const int64_t *rows, int64_t nrows,
                       double *out);

/* O2: recurrent form.  out [T][H][D] and/or final_state [S][H][D][D] (either may be NULL). */
int lao_recurrent(const double *q, const double *k, const double *v, const double *decay,
                  const int32_t *cu_seqlens, int32_t S, int64_t T, int32_t H, int32_t D,
                  const double *init_state, double *out, double *final_state);

/* O3: closed form of the state after each sequence.  state: [S][H][D][D]. */
int lao_final_state(const double *k, const double *v, const double *decay,
                    const int32_t *cu_seqlens, int32_t S, int64_t T, int32_t H, int32_t D,
                    const double *init_state, double *state);

/* O4: one recurrent decode step for Bt independent sequences.
 * q, k, v, out: [Bt][H][D]; state: [Bt][H][D][D], updated in place. */
int lao_decode_step(const double *q, const double *k, const double *v, const double *decay,
                    int32_t Bt, int32_t H, int32_t D, double *state, double *out);

/* O5: the two association orders of unmasked linear attention for one head, n x D:
 * left  = (Q K^T) V   (n x n scores first),
 * right = Q (K^T V)   (D x D summary first). */
int lao_unmasked_left(const double *q, const double *k, const double *v, int64_t n, int32_t D,
                      double *out);
int lao_unmasked_right(const double *q, const double *k, const double *v, int64_t n, int32_t D,
                       double *out);

/*
 * Gradients of the prefill.  The pages give no backward pass (they state only that the model
 * trains at up to a million tokens of context, abstract of the MiniMax-01 report, and that the
 * training framework parallelises lightning attention over the sequence, technical-report
 * digest section 2); what follows is the derivative of the definition above.  For a loss L with
 * dL/do_t = do_t and dL/dfinal_state = dSn (per sequence and head, dSn may be absent = 0):
 *
 *   dq_t  = sum_{s<=t} lambda^(t-s) (do_t . v_s) k_s  +  lambda^(t+1) S0 do_t
 *   dk_s  = sum_{t>=s} lambda^(t-s) (do_t . v_s) q_t  +  lambda^(n-1-s) dSn v_s
 *   dv_s  = sum_{t>=s} lambda^(t-s) (q_t . k_s) do_t  +  lambda^(n-1-s) dSn^T k_s
 *   dS0   = sum_t lambda^(t+1) q_t^T do_t  +  lambda^n dSn
 *
 * (S0 do_t is the vector sum_b S0[a][b] do_t[b]; dSn v_s likewise; dSn^T k_s is
 * sum_a dSn[a][b] k_s[a].)  lambda is a constant of the operation; no gradient for it.
 *
 * O6: the sums above, term by term (quadratic in n).  O7: the same through two scans:
 *   forward  S_t = lambda S_{t-1} + k_t^T v_t (S_{-1} = S0),  dq_t = S_t do_t;
 *   backward G_t = lambda G_{t+1} + q_t^T do_t (G_{n-1} = q^T do + dSn),
 *            dk_s = G_s v_s,  dv_s = G_s^T k_s,  dS0 = lambda G_0 (dSn when n = 0).
 * init_state and d_final may be NULL (zeros); d_init may be NULL (not computed).
 * dq, dk, dv: [T][H][D]; d_init: [S][H][D][D].
 */
int lao_backward(const double *q, const double *k, const double *v, const double *decay,
                 const int32_t *cu_seqlens, int32_t S, int64_t T, int32_t H, int32_t D,
                 const double *init_state, const double *d_out, const double *d_final,
                 double *dq, double *dk, double *dv, double *d_init);
int lao_backward_recurrent(const double *q, const double *k, const double *v,
                           const double *decay, const int32_t *cu_seqlens, int32_t S, int64_t T,
                           int32_t H, int32_t D, const double *init_state, const double *d_out,
                           const double *d_final, double *dq, double *dk, double *dv,
                           double *d_init);

/* Number of OpenMP threads a parallel region of this library uses (1 without OpenMP). */
int lao_num_threads(void);

/* Threads later parallel regions use (n >= 1; ignored without OpenMP). */
void lao_set_num_threads(int n);

#ifdef __cplusplus
}
#endif

#endif /* LA_ORACLE_H */
