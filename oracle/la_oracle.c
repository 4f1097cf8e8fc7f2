/*
 * la_oracle.c -- fp64 CPU oracle for decayed causal linear attention.
 *
 * TEST INFRASTRUCTURE ONLY (see la_oracle.h).  Plain, slow, obviously-correct loops in double
 * precision.  Powers of lambda are formed by repeated multiplication, never through exp/log,
 * so that lambda = 0 gives 0^0 = 1 exactly and lambda = 1 gives exactly 1.
 *
 * The method's definition (what the block algorithm must reproduce exactly, up to rounding):
 * causal linear attention in which a query t sees every earlier or equal key s with weight
 * lambda^(t-s).  The pages state causal linear attention and its two association orders
 * ("MiniMax-01 technical report digest", futurefh.com, section 1; nabfollower blog, section
 * "The Core Tech: Lightning Attention") and the fixed-size scan state (nabfollower blog,
 * analogy section); the per-head constant decay is the reading adopted where they are silent.
 */
#include "la_oracle.h"

#include <stddef.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* Element offset of (token t, head h, feature 0) in a [T][H][D] tensor. */
static size_t act_off(int64_t t, int32_t h, int32_t H, int32_t D) {
  return ((size_t)t * (size_t)H + (size_t)h) * (size_t)D;
}

/* Element offset of (sequence s, head h) in a [S][H][D][D] state tensor. */
static size_t state_off(int32_t s, int32_t h, int32_t H, int32_t D) {
  return ((size_t)s * (size_t)H + (size_t)h) * (size_t)D * (size_t)D;
}

static double dot(const double *a, const double *b, int32_t D) {
  double acc = 0.0;
  for (int32_t i = 0; i < D; ++i) acc += a[i] * b[i];
  return acc;
}

/* Sequence bounds: [*beg, *end) of sequence s.  cu == NULL means one sequence [0, T). */
static void seq_bounds(const int32_t *cu, int64_t T, int32_t s, int64_t *beg, int64_t *end) {
  if (cu == NULL) {
    *beg = 0;
    *end = T;
  } else {
    *beg = cu[s];
    *end = cu[s + 1];
  }
}

static int check_common(const double *decay, const int32_t *cu, int32_t S, int64_t T,
                        int32_t H, int32_t D) {
  if (decay == NULL || S < 1 || T < 0 || H < 1 || D < 1) return -1;
  if (cu == NULL) return S == 1 ? 0 : -1;
  if (cu[0] != 0 || cu[S] != T) return -1;
  for (int32_t s = 0; s < S; ++s)
    if (cu[s + 1] < cu[s]) return -1;
  return 0;
}

/* Output row t (global index) of sequence [beg, end) for head h:
 *   o_t = sum_{s=beg..t} lambda^(t-s) (q_t . k_s) v_s  +  lambda^(t-beg+1) q_t S0. */
static void quadratic_row(const double *q, const double *k, const double *v, double lam,
                          int64_t beg, int64_t t, int32_t h, int32_t H, int32_t D,
                          const double *S0, double *o) {
  const double *qt = q + act_off(t, h, H, D);
  for (int32_t b = 0; b < D; ++b) o[b] = 0.0;
  double w = 1.0; /* lambda^(t-s), starting at s = t */
  for (int64_t s = t; s >= beg; --s) {
    const double a = w * dot(qt, k + act_off(s, h, H, D), D);
    const double *vs = v + act_off(s, h, H, D);
    for (int32_t b = 0; b < D; ++b) o[b] += a * vs[b];
    w *= lam;
  }
  if (S0 != NULL) {
    /* w now equals lambda^(t-beg+1). */
    for (int32_t b = 0; b < D; ++b) {
      double acc = 0.0;
      for (int32_t a = 0; a < D; ++a) acc += qt[a] * S0[(size_t)a * D + b];
      o[b] += w * acc;
    }
  }
}

int lao_quadratic(const double *q, const double *k, const double *v, const double *decay,
                  const int32_t *cu_seqlens, int32_t S, int64_t T, int32_t H, int32_t D,
                  const double *init_state, double *out) {
  if (q == NULL || k == NULL || v == NULL || out == NULL) return -1;
  if (check_common(decay, cu_seqlens, S, T, H, D) != 0) return -1;
  for (int32_t s = 0; s < S; ++s) {
    int64_t beg, end;
    seq_bounds(cu_seqlens, T, s, &beg, &end);
    const int64_t n = end - beg;
#pragma omp parallel for collapse(2) schedule(dynamic, 16)
    for (int64_t t = 0; t < n; ++t) {
      for (int32_t h = 0; h < H; ++h) {
        const double *S0 = init_state ? init_state + state_off(s, h, H, D) : NULL;
        quadratic_row(q, k, v, decay[h], beg, beg + t, h, H, D, S0, out + act_off(beg + t, h, H, D));
      }
    }
  }
  return 0;
}

int lao_quadratic_rows(const double *q, const double *k, const double *v, const double *decay,
                       const int32_t *cu_seqlens, int32_t S, int64_t T, int32_t H, int32_t D,
                       const double *init_state, const int64_t *rows, int64_t nrows,
                       double *out) {
  if (q == NULL || k == NULL || v == NULL || out == NULL || rows == NULL || nrows < 0) return -1;
  if (check_common(decay, cu_seqlens, S, T, H, D) != 0) return -1;
  for (int64_t r = 0; r < nrows; ++r)
    if (rows[r] < 0 || rows[r] >= T) return -1;
  int bad = 0;
#pragma omp parallel for collapse(2) schedule(dynamic, 4) reduction(| : bad)
  for (int64_t r = 0; r < nrows; ++r) {
    for (int32_t h = 0; h < H; ++h) {
      const int64_t t = rows[r];
      /* Find the sequence holding token t (linear scan: plain and obviously right). */
      int32_t s = 0;
      int64_t beg = 0, end = T;
      for (s = 0; s < S; ++s) {
        seq_bounds(cu_seqlens, T, s, &beg, &end);
        if (t >= beg && t < end) break;
      }
      if (s == S) {
        bad |= 1;
        continue;
      }
      const double *S0 = init_state ? init_state + state_off(s, h, H, D) : NULL;
      quadratic_row(q, k, v, decay[h], beg, t, h, H, D, S0, out + ((size_t)r * H + h) * D);
    }
  }
  return bad ? -1 : 0;
}

int lao_recurrent(const double *q, const double *k, const double *v, const double *decay,
                  const int32_t *cu_seqlens, int32_t S, int64_t T, int32_t H, int32_t D,
                  const double *init_state, double *out, double *final_state) {
  if (k == NULL || v == NULL) return -1;
  if (out != NULL && q == NULL) return -1;
  if (check_common(decay, cu_seqlens, S, T, H, D) != 0) return -1;
  int bad = 0;
#pragma omp parallel for collapse(2) schedule(dynamic, 1) reduction(| : bad)
  for (int32_t s = 0; s < S; ++s) {
    for (int32_t h = 0; h < H; ++h) {
      double *St = (double *)malloc(sizeof(double) * (size_t)D * D);
      if (St == NULL) {
        bad |= 1;
        continue;
      }
      if (init_state)
        memcpy(St, init_state + state_off(s, h, H, D), sizeof(double) * (size_t)D * D);
      else
        memset(St, 0, sizeof(double) * (size_t)D * D);
      const double lam = decay[h];
      int64_t beg, end;
      seq_bounds(cu_seqlens, T, s, &beg, &end);
      for (int64_t t = beg; t < end; ++t) {
        const double *kt = k + act_off(t, h, H, D);
        const double *vt = v + act_off(t, h, H, D);
        /* S_t = lambda S_{t-1} + k_t^T v_t */
        for (int32_t a = 0; a < D; ++a)
          for (int32_t b = 0; b < D; ++b)
            St[(size_t)a * D + b] = lam * St[(size_t)a * D + b] + kt[a] * vt[b];
        if (out != NULL) {
          /* o_t = q_t S_t */
          const double *qt = q + act_off(t, h, H, D);
          double *ot = out + act_off(t, h, H, D);
          for (int32_t b = 0; b < D; ++b) {
            double acc = 0.0;
            for (int32_t a = 0; a < D; ++a) acc += qt[a] * St[(size_t)a * D + b];
            ot[b] = acc;
          }
        }
      }
      if (final_state != NULL)
        memcpy(final_state + state_off(s, h, H, D), St, sizeof(double) * (size_t)D * D);
      free(St);
    }
  }
  return bad ? -1 : 0;
}

int lao_final_state(const double *k, const double *v, const double *decay,
                    const int32_t *cu_seqlens, int32_t S, int64_t T, int32_t H, int32_t D,
                    const double *init_state, double *state) {
  if (k == NULL || v == NULL || state == NULL) return -1;
  if (check_common(decay, cu_seqlens, S, T, H, D) != 0) return -1;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int32_t s = 0; s < S; ++s) {
    for (int32_t h = 0; h < H; ++h) {
      double *St = state + state_off(s, h, H, D);
      const double lam = decay[h];
      int64_t beg, end;
      seq_bounds(cu_seqlens, T, s, &beg, &end);
      for (size_t e = 0; e < (size_t)D * D; ++e) St[e] = 0.0;
      double w = 1.0; /* lambda^(end-1-t), starting at the last token */
      for (int64_t t = end - 1; t >= beg; --t) {
        const double *kt = k + act_off(t, h, H, D);
        const double *vt = v + act_off(t, h, H, D);
        for (int32_t a = 0; a < D; ++a)
          for (int32_t b = 0; b < D; ++b) St[(size_t)a * D + b] += w * kt[a] * vt[b];
        w *= lam;
      }
      if (init_state != NULL) {
        /* w now equals lambda^n. */
        const double *S0 = init_state + state_off(s, h, H, D);
        for (size_t e = 0; e < (size_t)D * D; ++e) St[e] += w * S0[e];
      }
    }
  }
  return 0;
}

int lao_decode_step(const double *q, const double *k, const double *v, const double *decay,
                    int32_t Bt, int32_t H, int32_t D, double *state, double *out) {
  if (q == NULL || k == NULL || v == NULL || decay == NULL || state == NULL || out == NULL)
    return -1;
  if (Bt < 0 || H < 1 || D < 1) return -1;
#pragma omp parallel for collapse(2) schedule(static)
  for (int32_t b = 0; b < Bt; ++b) {
    for (int32_t h = 0; h < H; ++h) {
      const double lam = decay[h];
      const double *qt = q + act_off(b, h, H, D);
      const double *kt = k + act_off(b, h, H, D);
      const double *vt = v + act_off(b, h, H, D);
      double *St = state + state_off(b, h, H, D);
      double *ot = out + act_off(b, h, H, D);
      for (int32_t a = 0; a < D; ++a)
        for (int32_t c = 0; c < D; ++c)
          St[(size_t)a * D + c] = lam * St[(size_t)a * D + c] + kt[a] * vt[c];
      for (int32_t c = 0; c < D; ++c) {
        double acc = 0.0;
        for (int32_t a = 0; a < D; ++a) acc += qt[a] * St[(size_t)a * D + c];
        ot[c] = acc;
      }
    }
  }
  return 0;
}

int lao_unmasked_left(const double *q, const double *k, const double *v, int64_t n, int32_t D,
                      double *out) {
  if (q == NULL || k == NULL || v == NULL || out == NULL || n < 0 || D < 1) return -1;
  /* A = Q K^T (n x n), then out = A V. */
  double *A = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * (size_t)(n > 0 ? n : 1));
  if (A == NULL) return -1;
  for (int64_t t = 0; t < n; ++t)
    for (int64_t s = 0; s < n; ++s) A[(size_t)t * n + s] = dot(q + (size_t)t * D, k + (size_t)s * D, D);
  for (int64_t t = 0; t < n; ++t)
    for (int32_t b = 0; b < D; ++b) {
      double acc = 0.0;
      for (int64_t s = 0; s < n; ++s) acc += A[(size_t)t * n + s] * v[(size_t)s * D + b];
      out[(size_t)t * D + b] = acc;
    }
  free(A);
  return 0;
}

int lao_unmasked_right(const double *q, const double *k, const double *v, int64_t n, int32_t D,
                       double *out) {
  if (q == NULL || k == NULL || v == NULL || out == NULL || n < 0 || D < 1) return -1;
  /* M = K^T V (D x D), then out = Q M. */
  double *M = (double *)calloc((size_t)D * D, sizeof(double));
  if (M == NULL) return -1;
  for (int64_t s = 0; s < n; ++s)
    for (int32_t a = 0; a < D; ++a)
      for (int32_t b = 0; b < D; ++b) M[(size_t)a * D + b] += k[(size_t)s * D + a] * v[(size_t)s * D + b];
  for (int64_t t = 0; t < n; ++t)
    for (int32_t b = 0; b < D; ++b) {
      double acc = 0.0;
      for (int32_t a = 0; a < D; ++a) acc += q[(size_t)t * D + a] * M[(size_t)a * D + b];
      out[(size_t)t * D + b] = acc;
    }
  free(M);
  return 0;
}

/* O6.  Each gradient row is its own sum over the other time index, written as in the
 * definition: dq_t over s <= t, dk_s and dv_s over t >= s, dS0 over all t. */
int lao_backward(const double *q, const double *k, const double *v, const double *decay,
                 const int32_t *cu_seqlens, int32_t S, int64_t T, int32_t H, int32_t D,
                 const double *init_state, const double *d_out, const double *d_final,
                 double *dq, double *dk, double *dv, double *d_init) {
  if (q == NULL || k == NULL || v == NULL || d_out == NULL || dq == NULL || dk == NULL ||
      dv == NULL)
    return -1;
  if (check_common(decay, cu_seqlens, S, T, H, D) != 0) return -1;
  for (int32_t sq = 0; sq < S; ++sq) {
    int64_t beg, end;
    seq_bounds(cu_seqlens, T, sq, &beg, &end);
    const int64_t n = end - beg;
#pragma omp parallel for collapse(2) schedule(dynamic, 8)
    for (int64_t i = 0; i < n; ++i) {
      for (int32_t h = 0; h < H; ++h) {
        const double lam = decay[h];
        const double *S0 = init_state ? init_state + state_off(sq, h, H, D) : NULL;
        const double *dSn = d_final ? d_final + state_off(sq, h, H, D) : NULL;
        const int64_t t = beg + i; /* this row's token */
        /* dq_t = sum_{s<=t} lambda^(t-s) (do_t . v_s) k_s + lambda^(t+1) S0 do_t */
        {
          const double *dout_t = d_out + act_off(t, h, H, D);
          double *g = dq + act_off(t, h, H, D);
          for (int32_t a = 0; a < D; ++a) g[a] = 0.0;
          double w = 1.0; /* lambda^(t-s) */
          for (int64_t s = t; s >= beg; --s) {
            const double c = w * dot(dout_t, v + act_off(s, h, H, D), D);
            const double *ks = k + act_off(s, h, H, D);
            for (int32_t a = 0; a < D; ++a) g[a] += c * ks[a];
            w *= lam;
          }
          if (S0 != NULL) /* w = lambda^(t-beg+1) */
            for (int32_t a = 0; a < D; ++a) {
              double acc = 0.0;
              for (int32_t b = 0; b < D; ++b) acc += S0[(size_t)a * D + b] * dout_t[b];
              g[a] += w * acc;
            }
        }
        /* dk_t and dv_t (t in the role of s above): sums over t' >= t */
        {
          const double *kt = k + act_off(t, h, H, D);
          const double *vt = v + act_off(t, h, H, D);
          double *gk = dk + act_off(t, h, H, D);
          double *gv = dv + act_off(t, h, H, D);
          for (int32_t a = 0; a < D; ++a) gk[a] = gv[a] = 0.0;
          double w = 1.0; /* lambda^(t'-t) */
          for (int64_t tp = t; tp < end; ++tp) {
            const double *qp = q + act_off(tp, h, H, D);
            const double *dp = d_out + act_off(tp, h, H, D);
            const double ck = w * dot(dp, vt, D);
            const double cv = w * dot(qp, kt, D);
            for (int32_t a = 0; a < D; ++a) {
              gk[a] += ck * qp[a];
              gv[a] += cv * dp[a];
            }
            w *= lam;
          }
          if (dSn != NULL) {
            /* lambda^(end-1-t) = w / lambda would divide by zero at lambda = 0: recompute */
            double wn = 1.0;
            for (int64_t m = t; m < end - 1; ++m) wn *= lam;
            for (int32_t a = 0; a < D; ++a) {
              double acck = 0.0, accv = 0.0;
              for (int32_t b = 0; b < D; ++b) {
                acck += dSn[(size_t)a * D + b] * vt[b];
                accv += dSn[(size_t)b * D + a] * kt[b];
              }
              gk[a] += wn * acck;
              gv[a] += wn * accv;
            }
          }
        }
      }
    }
    if (d_init != NULL) {
      /* dS0 = sum_t lambda^(t+1) q_t^T do_t + lambda^n dSn */
#pragma omp parallel for schedule(dynamic, 1)
      for (int32_t h = 0; h < H; ++h) {
        const double lam = decay[h];
        double *g = d_init + state_off(sq, h, H, D);
        for (size_t e = 0; e < (size_t)D * D; ++e) g[e] = 0.0;
        double w = lam; /* lambda^(t+1) at t = beg */
        for (int64_t t = beg; t < end; ++t) {
          const double *qt = q + act_off(t, h, H, D);
          const double *dt = d_out + act_off(t, h, H, D);
          for (int32_t a = 0; a < D; ++a)
            for (int32_t b = 0; b < D; ++b) g[(size_t)a * D + b] += w * qt[a] * dt[b];
          w *= lam;
        }
        if (d_final != NULL) {
          double wn = 1.0;
          for (int64_t m = 0; m < n; ++m) wn *= lam;
          const double *dSn = d_final + state_off(sq, h, H, D);
          for (size_t e = 0; e < (size_t)D * D; ++e) g[e] += wn * dSn[e];
        }
      }
    }
  }
  return 0;
}

/* O7.  Forward scan for dq, reverse scan for dk, dv and dS0. */
int lao_backward_recurrent(const double *q, const double *k, const double *v,
                           const double *decay, const int32_t *cu_seqlens, int32_t S, int64_t T,
                           int32_t H, int32_t D, const double *init_state, const double *d_out,
                           const double *d_final, double *dq, double *dk, double *dv,
                           double *d_init) {
  if (q == NULL || k == NULL || v == NULL || d_out == NULL || dq == NULL || dk == NULL ||
      dv == NULL)
    return -1;
  if (check_common(decay, cu_seqlens, S, T, H, D) != 0) return -1;
  int bad = 0;
#pragma omp parallel for collapse(2) schedule(dynamic, 1) reduction(| : bad)
  for (int32_t sq = 0; sq < S; ++sq) {
    for (int32_t h = 0; h < H; ++h) {
      const size_t DD = (size_t)D * D;
      double *St = (double *)malloc(sizeof(double) * DD);
      double *G = (double *)malloc(sizeof(double) * DD);
      if (St == NULL || G == NULL) {
        free(St);
        free(G);
        bad |= 1;
        continue;
      }
      const double lam = decay[h];
      int64_t beg, end;
      seq_bounds(cu_seqlens, T, sq, &beg, &end);
      /* forward: S_t = lambda S_{t-1} + k_t^T v_t, dq_t = S_t do_t */
      if (init_state)
        memcpy(St, init_state + state_off(sq, h, H, D), sizeof(double) * DD);
      else
        memset(St, 0, sizeof(double) * DD);
      for (int64_t t = beg; t < end; ++t) {
        const double *kt = k + act_off(t, h, H, D);
        const double *vt = v + act_off(t, h, H, D);
        const double *dt = d_out + act_off(t, h, H, D);
        double *g = dq + act_off(t, h, H, D);
        for (int32_t a = 0; a < D; ++a)
          for (int32_t b = 0; b < D; ++b)
            St[(size_t)a * D + b] = lam * St[(size_t)a * D + b] + kt[a] * vt[b];
        for (int32_t a = 0; a < D; ++a) {
          double acc = 0.0;
          for (int32_t b = 0; b < D; ++b) acc += St[(size_t)a * D + b] * dt[b];
          g[a] = acc;
        }
      }
      /* reverse: G starts as dSn; G_t = lambda G_{t+1} + q_t^T do_t (no decay before the
       * last token's term), dk_t = G_t v_t, dv_t = G_t^T k_t */
      if (d_final)
        memcpy(G, d_final + state_off(sq, h, H, D), sizeof(double) * DD);
      else
        memset(G, 0, sizeof(double) * DD);
      for (int64_t t = end - 1; t >= beg; --t) {
        const double *qt = q + act_off(t, h, H, D);
        const double *kt = k + act_off(t, h, H, D);
        const double *vt = v + act_off(t, h, H, D);
        const double *dt = d_out + act_off(t, h, H, D);
        const double w = t == end - 1 ? 1.0 : lam;
        for (int32_t a = 0; a < D; ++a)
          for (int32_t b = 0; b < D; ++b)
            G[(size_t)a * D + b] = w * G[(size_t)a * D + b] + qt[a] * dt[b];
        double *gk = dk + act_off(t, h, H, D);
        double *gv = dv + act_off(t, h, H, D);
        for (int32_t a = 0; a < D; ++a) {
          double acck = 0.0, accv = 0.0;
          for (int32_t b = 0; b < D; ++b) {
            acck += G[(size_t)a * D + b] * vt[b];
            accv += G[(size_t)b * D + a] * kt[b];
          }
          gk[a] = acck;
          gv[a] = accv;
        }
      }
      if (d_init != NULL) {
        double *g = d_init + state_off(sq, h, H, D);
        const double w = end > beg ? lam : 1.0;
        for (size_t e = 0; e < DD; ++e) g[e] = w * G[e];
      }
      free(St);
      free(G);
    }
  }
  return bad ? -1 : 0;
}

int lao_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void lao_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}
