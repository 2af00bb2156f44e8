/*
 * slay_oracle.c -- plain fp64 CPU oracle for causal SLAY attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the independent checker of the HIP
 * library.  Only the test suite, the smoke check and the CPU-baseline leg of
 * the benchmark may load it.  It shares no code, header, table or constant
 * with the GPU library: the Gauss-Laguerre rule, the feature map and every
 * attention form below are written out here on their own.
 *
 * Everything is fp64 and written as plain loops in the order the method
 * states its steps: no blocking, fusion or reordering beyond what each
 * definition itself says.  Random draws (anchor vectors a, PRF vectors g)
 * are inputs, never generated here.
 *
 * Sources (web pages; section names as printed on each page):
 *   [SLAY-abs]  "SLAY: Geometry-Aware Spherical Linearized Attention with
 *               Yat-Kernel", arXiv 2602.04915, English abstract (paperdance).
 *   [SLAY-rev]  nubint.ai review of the same paper, sections "Motivation and
 *               goals" (연구 동기 및 목표) and "Proposed method" (제안 방법,
 *               six bullets, cited as bullet 1..6).
 *
 * Readings taken where the pages are silent (each marked READING below):
 *   - K(u) = u^2 / (2 - 2u + eps): the E-product (q.k)^2/(|q-k|^2+eps) on
 *     unit vectors, where |q-k|^2 = 2 - 2u.
 *   - Laplace variable t = x/(2+eps), plain Gauss-Laguerre (weight e^{-x}).
 *   - anchor feature (a.xh)^2 with a ~ N(0, I); PRF exp(sqrt(beta) g.xh -
 *     beta/2) with g ~ N(0, I); tensor sketch = elementwise product of the
 *     t-th anchor and t-th PRF feature of one node, scaled by sqrt(alpha/m).
 *   - causal mask includes the diagonal (j <= i); no denominator guard.
 *   - zero rows are normalised as x / max(|x|, 1e-12).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_BAD 1

/* ------------------------------------------------------------------------ */
/* Laguerre polynomials L_n(x) with L_n(0) = 1, by the three-term recurrence
 * (n+1) L_{n+1} = (2n+1-x) L_n - n L_{n-1}.                                  */
static double laguerre(int n, double x) {
  double lm1 = 1.0, l = 1.0 - x;
  if (n == 0) return 1.0;
  for (int k = 1; k < n; ++k) {
    double lp1 = ((2.0 * k + 1.0 - x) * l - k * lm1) / (k + 1.0);
    lm1 = l;
    l = lp1;
  }
  return l;
}

static double bisect_root(int n, double lo, double hi) {
  double flo = laguerre(n, lo);
  for (int it = 0; it < 200; ++it) {
    double mid = 0.5 * (lo + hi);
    if (mid <= lo || mid >= hi) break;
    double fm = laguerre(n, mid);
    if (fm == 0.0) return mid;
    if ((fm > 0) == (flo > 0)) { lo = mid; flo = fm; } else { hi = mid; }
  }
  return 0.5 * (lo + hi);
}

/* R-point Gauss-Laguerre rule for int_0^inf e^{-x} f(x) dx
 * ([SLAY-rev] Proposed method, bullet 4: the Laplace integral is discretised
 * with Gauss-Laguerre quadrature).
 * Nodes: the zeros of L_R.  The zeros of L_{n-1} interlace those of L_n, so
 * the rule is built up from n = 1: each zero of L_n is bracketed between
 * consecutive zeros of L_{n-1} (and 0 / an upper bound 4n+6) and found by
 * bisection.  Weights: w_i = x_i / ((R+1)^2 L_{R+1}(x_i)^2).                 */
int orc_gauss_laguerre(int R, double* x, double* w) {
  if (R < 1 || R > 128 || !x || !w) return ORC_BAD;
  double* prev = (double*)malloc(sizeof(double) * (size_t)R);
  double* cur = (double*)malloc(sizeof(double) * (size_t)R);
  if (!prev || !cur) { free(prev); free(cur); return ORC_BAD; }
  cur[0] = 1.0; /* the zero of L_1 */
  for (int n = 2; n <= R; ++n) {
    memcpy(prev, cur, sizeof(double) * (size_t)(n - 1));
    for (int i = 0; i < n; ++i) {
      double lo = (i == 0) ? 0.0 : prev[i - 1];
      double hi = (i == n - 1) ? 4.0 * n + 6.0 : prev[i];
      cur[i] = bisect_root(n, lo, hi);
    }
  }
  for (int i = 0; i < R; ++i) {
    double lr1 = laguerre(R + 1, cur[i]);
    x[i] = cur[i];
    w[i] = cur[i] / ((R + 1.0) * (R + 1.0) * lr1 * lr1);
  }
  free(prev);
  free(cur);
  return ORC_OK;
}

/* Mixture parameters of node r ([SLAY-rev] Proposed method, bullets 2 and 4):
 * 1/(2+eps-2u) = int_0^inf e^{-s(2+eps)} e^{2su} ds; with s = x/(2+eps) the
 * integral becomes (1/(2+eps)) int e^{-x} e^{(2x/(2+eps)) u} dx, so
 * alpha_r = w_r/(2+eps) and beta_r = 2 x_r/(2+eps).                           */
int orc_node_params(int R, double eps, double* alpha, double* beta) {
  if (!(eps > 0.0)) return ORC_BAD;
  double* x = (double*)malloc(sizeof(double) * (size_t)R);
  double* w = (double*)malloc(sizeof(double) * (size_t)R);
  if (!x || !w) { free(x); free(w); return ORC_BAD; }
  int st = orc_gauss_laguerre(R, x, w);
  if (st == ORC_OK)
    for (int r = 0; r < R; ++r) {
      alpha[r] = w[r] / (2.0 + eps);
      beta[r] = 2.0 * x[r] / (2.0 + eps);
    }
  free(x);
  free(w);
  return st;
}

/* Spherical Yat kernel K(u) = u^2/(2-2u+eps) ([SLAY-abs]; [SLAY-rev]
 * Proposed method, bullet 1).  READING: the formula is not printed on the
 * pages; this is the E-product restricted to the unit sphere.                */
void orc_yat_kernel(int64_t n, const double* u, double eps, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = u[i] * u[i] / (2.0 - 2.0 * u[i] + eps);
}

/* Gauss-Laguerre mixture K_R(u) = sum_r alpha_r u^2 e^{beta_r u}
 * ([SLAY-rev] Proposed method, bullets 2 and 4).                              */
int orc_yat_mixture(int64_t n, const double* u, double eps, int R, double* out) {
  double* alpha = (double*)malloc(sizeof(double) * (size_t)R);
  double* beta = (double*)malloc(sizeof(double) * (size_t)R);
  if (!alpha || !beta) { free(alpha); free(beta); return ORC_BAD; }
  int st = orc_node_params(R, eps, alpha, beta);
  if (st == ORC_OK)
    for (int64_t i = 0; i < n; ++i) {
      double s = 0.0;
      for (int r = 0; r < R; ++r) s += alpha[r] * u[i] * u[i] * exp(beta[r] * u[i]);
      out[i] = s;
    }
  free(alpha);
  free(beta);
  return st;
}

/* ------------------------------------------------------------------------ */
/* SLAY feature map of n rows x[n][d] ([SLAY-abs]; [SLAY-rev] Proposed method,
 * bullets 1, 3 and 5).
 *   xh = x / max(|x|, 1e-12)                                  (unit sphere)
 *   psi_{r,t}  = (a_{r,t} . xh)^2                           (anchor feature)
 *   prf_{r,t}  = exp(sqrt(beta_r) g_{r,t} . xh - beta_r/2)     (positive RF)
 *   phi[r*m+t] = sqrt(alpha_r/m) psi_{r,t} prf_{r,t}          (tensor sketch)
 * a, g: [R*m][d] (row r*m+t).  phi: [n][R*m].                               */
int orc_featmap(int64_t n, int d, int R, int m, double eps, const double* x,
                const double* a, const double* g, double* phi) {
  if (n < 0 || d < 1 || R < 1 || m < 1) return ORC_BAD;
  double* alpha = (double*)malloc(sizeof(double) * (size_t)R);
  double* beta = (double*)malloc(sizeof(double) * (size_t)R);
  if (!alpha || !beta) { free(alpha); free(beta); return ORC_BAD; }
  int st = orc_node_params(R, eps, alpha, beta);
  if (st != ORC_OK) { free(alpha); free(beta); return st; }
  const int F = R * m;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    const double* xi = x + i * d;
    double nrm = 0.0;
    for (int c = 0; c < d; ++c) nrm += xi[c] * xi[c];
    nrm = sqrt(nrm);
    if (nrm < 1e-12) nrm = 1e-12;
    for (int r = 0; r < R; ++r) {
      for (int t = 0; t < m; ++t) {
        const double* ar = a + (size_t)(r * m + t) * d;
        const double* gr = g + (size_t)(r * m + t) * d;
        double pa = 0.0, pg = 0.0;
        for (int c = 0; c < d; ++c) {
          pa += ar[c] * (xi[c] / nrm);
          pg += gr[c] * (xi[c] / nrm);
        }
        double psi = pa * pa;
        double prf = exp(sqrt(beta[r]) * pg - 0.5 * beta[r]);
        phi[i * F + r * m + t] = sqrt(alpha[r] / m) * psi * prf;
      }
    }
  }
  free(alpha);
  free(beta);
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Causal normalised attention on features, one head
 * ([SLAY-rev] Proposed method, bullet 6; [SLAY-abs]):
 *   s_ij = phq_i . phk_j,   o_i = sum_{j<=i} s_ij v_j / sum_{j<=i} s_ij.
 * Three forms, written independently, that must agree to rounding.           */

/* (1) brute force: forms the masked L x L score matrix row by row.
 * An initial state (S0 [F][dv], z0 [F]) adds phq_i.S0 and phq_i.z0. */
void orc_attn_brute(int64_t L, int F, int dv, const double* phq, const double* phk,
                    const double* v, const double* S0, const double* z0, double* o) {
  double* s = (double*)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
  for (int64_t i = 0; i < L; ++i) {
    for (int64_t j = 0; j <= i; ++j) {
      double acc = 0.0;
      for (int f = 0; f < F; ++f) acc += phq[i * F + f] * phk[j * F + f];
      s[j] = acc;
    }
    double den = 0.0;
    for (int64_t j = 0; j <= i; ++j) den += s[j];
    if (z0)
      for (int f = 0; f < F; ++f) den += phq[i * F + f] * z0[f];
    for (int e = 0; e < dv; ++e) {
      double num = 0.0;
      for (int64_t j = 0; j <= i; ++j) num += s[j] * v[j * dv + e];
      if (S0)
        for (int f = 0; f < F; ++f) num += phq[i * F + f] * S0[(size_t)f * dv + e];
      o[i * dv + e] = num / den;
    }
  }
  free(s);
}

/* (2) recurrent: S_i = S_{i-1} + phk_i v_i^T, z_i = z_{i-1} + phk_i, then
 * o_i = phq_i^T S_i / phq_i^T z_i (update first, so S_i includes j = i).
 * S [F][dv], z [F] are in/out (the running state).                          */
void orc_attn_recurrent(int64_t L, int F, int dv, const double* phq, const double* phk,
                        const double* v, double* S, double* z, double* o) {
  for (int64_t i = 0; i < L; ++i) {
    for (int f = 0; f < F; ++f) {
      double kf = phk[i * F + f];
      for (int e = 0; e < dv; ++e) S[(size_t)f * dv + e] += kf * v[i * dv + e];
      z[f] += kf;
    }
    double den = 0.0;
    for (int f = 0; f < F; ++f) den += phq[i * F + f] * z[f];
    for (int e = 0; e < dv; ++e) {
      double num = 0.0;
      for (int f = 0; f < F; ++f) num += phq[i * F + f] * S[(size_t)f * dv + e];
      o[i * dv + e] = num / den;
    }
  }
}

/* (3) chunked: for chunks [c0, c0+C), the masked intra-chunk block
 * A = tril(phq_c phk_c^T) gives A v_c and A 1; the state before the chunk
 * gives phq_c S and phq_c z; then S += phk_c^T v_c, z += phk_c^T 1.
 * S, z in/out as in (2).                                                     */
void orc_attn_chunked(int64_t L, int F, int dv, int C, const double* phq, const double* phk,
                      const double* v, double* S, double* z, double* o) {
  double* A = (double*)malloc(sizeof(double) * (size_t)C * (size_t)C);
  for (int64_t c0 = 0; c0 < L; c0 += C) {
    int64_t n = (L - c0 < C) ? (L - c0) : C;
    for (int64_t i = 0; i < n; ++i)
      for (int64_t j = 0; j < n; ++j) {
        double acc = 0.0;
        if (j <= i)
          for (int f = 0; f < F; ++f) acc += phq[(c0 + i) * F + f] * phk[(c0 + j) * F + f];
        A[i * C + j] = acc;
      }
    for (int64_t i = 0; i < n; ++i) {
      double den = 0.0;
      for (int64_t j = 0; j < n; ++j) den += A[i * C + j];
      for (int f = 0; f < F; ++f) den += phq[(c0 + i) * F + f] * z[f];
      for (int e = 0; e < dv; ++e) {
        double num = 0.0;
        for (int64_t j = 0; j < n; ++j) num += A[i * C + j] * v[(c0 + j) * dv + e];
        for (int f = 0; f < F; ++f) num += phq[(c0 + i) * F + f] * S[(size_t)f * dv + e];
        o[(c0 + i) * dv + e] = num / den;
      }
    }
    for (int64_t j = 0; j < n; ++j)
      for (int f = 0; f < F; ++f) {
        double kf = phk[(c0 + j) * F + f];
        for (int e = 0; e < dv; ++e) S[(size_t)f * dv + e] += kf * v[(c0 + j) * dv + e];
        z[f] += kf;
      }
  }
  free(A);
}

/* ------------------------------------------------------------------------ */
/* Whole causal SLAY forward over nh = B*H heads (parallel over heads):
 * q, k [nh][L][d], v [nh][L][dv] -> o [nh][L][dv]; draws [R*m][d] shared by
 * every head (or, if draw_head_stride > 0, head h uses a + h*stride).
 * form: 0 brute, 1 recurrent, 2 chunked (chunk C).  S0/z0 nullable initial
 * state [nh][F][dv] / [nh][F]; S_out/z_out nullable final state.            */
int orc_slay_causal(int64_t nh, int64_t L, int d, int dv, int R, int m, double eps,
                    const double* q, const double* k, const double* v, const double* a,
                    const double* g, int64_t draw_head_stride, int form, int C,
                    const double* S0, const double* z0, double* o, double* S_out, double* z_out) {
  if (nh < 0 || L < 0 || d < 1 || dv < 1 || R < 1 || m < 1) return ORC_BAD;
  if (form == 2 && C < 1) return ORC_BAD;
  const int F = R * m;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
  for (int64_t h = 0; h < nh; ++h) {
    const double* ah = a + (draw_head_stride > 0 ? h * draw_head_stride : 0);
    const double* gh = g + (draw_head_stride > 0 ? h * draw_head_stride : 0);
    double* phq = (double*)malloc(sizeof(double) * (size_t)(L * F + 1));
    double* phk = (double*)malloc(sizeof(double) * (size_t)(L * F + 1));
    double* S = (double*)calloc((size_t)F * dv, sizeof(double));
    double* z = (double*)calloc((size_t)F, sizeof(double));
    if (!phq || !phk || !S || !z) { bad |= 1; free(phq); free(phk); free(S); free(z); continue; }
    bad |= orc_featmap(L, d, R, m, eps, q + h * L * d, ah, gh, phq);
    bad |= orc_featmap(L, d, R, m, eps, k + h * L * d, ah, gh, phk);
    if (S0) memcpy(S, S0 + h * (int64_t)F * dv, sizeof(double) * (size_t)F * dv);
    if (z0) memcpy(z, z0 + h * (int64_t)F, sizeof(double) * (size_t)F);
    const double* vh = v + h * L * dv;
    double* oh = o + h * L * dv;
    if (form == 0) {
      orc_attn_brute(L, F, dv, phq, phk, vh, S0 ? S : NULL, z0 ? z : NULL, oh);
      /* final state for the brute-force form: the plain sums */
      for (int64_t j = 0; j < L; ++j)
        for (int f = 0; f < F; ++f) {
          for (int e = 0; e < dv; ++e) S[(size_t)f * dv + e] += phk[j * F + f] * vh[j * dv + e];
          z[f] += phk[j * F + f];
        }
    } else if (form == 1) {
      orc_attn_recurrent(L, F, dv, phq, phk, vh, S, z, oh);
    } else {
      orc_attn_chunked(L, F, dv, C, phq, phk, vh, S, z, oh);
    }
    if (S_out) memcpy(S_out + h * (int64_t)F * dv, S, sizeof(double) * (size_t)F * dv);
    if (z_out) memcpy(z_out + h * (int64_t)F, z, sizeof(double) * (size_t)F);
    free(phq);
    free(phk);
    free(S);
    free(z);
  }
  return bad ? ORC_BAD : ORC_OK;
}

/* Exact spherical-Yat causal attention (no features), one pass over nh heads:
 * o_i = sum_{j<=i} K(qh_i.kh_j) v_j / sum_{j<=i} K(qh_i.kh_j)
 * ([SLAY-rev] Main results, bullet 1: the comparison point "full spherical
 * YAT attention").  Reported, not used as a parity target.                  */
int orc_yat_exact_causal(int64_t nh, int64_t L, int d, int dv, double eps, const double* q,
                         const double* k, const double* v, double* o) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t h = 0; h < nh; ++h) {
    const double* qh = q + h * L * d;
    const double* kh = k + h * L * d;
    const double* vh = v + h * L * dv;
    double* oh = o + h * L * dv;
    for (int64_t i = 0; i < L; ++i) {
      double nq = 0.0;
      for (int c = 0; c < d; ++c) nq += qh[i * d + c] * qh[i * d + c];
      nq = fmax(sqrt(nq), 1e-12);
      double den = 0.0;
      for (int e = 0; e < dv; ++e) oh[i * dv + e] = 0.0;
      for (int64_t j = 0; j <= i; ++j) {
        double nk = 0.0, u = 0.0;
        for (int c = 0; c < d; ++c) {
          nk += kh[j * d + c] * kh[j * d + c];
          u += qh[i * d + c] * kh[j * d + c];
        }
        nk = fmax(sqrt(nk), 1e-12);
        u = u / (nq * nk);
        double s = u * u / (2.0 - 2.0 * u + eps);
        den += s;
        for (int e = 0; e < dv; ++e) oh[i * dv + e] += s * vh[j * dv + e];
      }
      for (int e = 0; e < dv; ++e) oh[i * dv + e] /= den;
    }
  }
  return ORC_OK;
}

/* Selected rows i of the causal attention of one head, each computed on its
 * own as sum_{j<=i} s_ij v_j / sum_{j<=i} s_ij (spot checks at sizes where
 * the whole forward is too slow).  phq_rows [n_rows][F] holds the features
 * of the selected queries; phk [L][F], v [L][dv] cover every key j <= i.     */
void orc_attn_rows(int64_t n_rows, const int64_t* rows, int F, int dv, const double* phq_rows,
                   const double* phk, const double* v, double* o_rows) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < n_rows; ++r) {
    const int64_t i = rows[r];
    const double* qf = phq_rows + r * F;
    double den = 0.0;
    double* orow = o_rows + r * dv;
    for (int e = 0; e < dv; ++e) orow[e] = 0.0;
    for (int64_t j = 0; j <= i; ++j) {
      double s = 0.0;
      for (int f = 0; f < F; ++f) s += qf[f] * phk[j * F + f];
      den += s;
      for (int e = 0; e < dv; ++e) orow[e] += s * v[j * dv + e];
    }
    for (int e = 0; e < dv; ++e) orow[e] /= den;
  }
}

/* Non-causal SLAY: every query attends to every key,
 *   o_i = (sum_j s_ij v_j + phq_i^T S0) / (sum_j s_ij + phq_i^T z0),
 *   s_ij = phq_i . phk_j,
 * the standard linear-attention contraction of [SLAY-rev] "Proposed method"
 * bullet 6 taken over all keys (READING: the pages' vision and extreme-
 * classification settings, "Motivation and goals" bullet 5 and "Main
 * results" bullet 4, attend bidirectionally).  Written as the score sums,
 * brute force over (i, j); the initial state (S0, z0), when given, adds to
 * every query.  The final state is S0 + sum_j phk_j v_j^T, z0 + sum_j phk_j.
 * Draws of head h start at a + h * draw_head_stride (0: shared).            */
int orc_slay_noncausal(int64_t nh, int64_t Lq, int64_t Lk, int d, int dv, int R, int m, double eps,
                       const double* q, const double* k, const double* v, const double* a,
                       const double* g, int64_t draw_head_stride, const double* S0, const double* z0,
                       double* o, double* S_out, double* z_out) {
  if (nh < 0 || Lq < 0 || Lk < 0 || d < 1 || dv < 1 || R < 1 || m < 1) return ORC_BAD;
  const int F = R * m;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
  for (int64_t h = 0; h < nh; ++h) {
    const double* ah = a + (draw_head_stride > 0 ? h * draw_head_stride : 0);
    const double* gh = g + (draw_head_stride > 0 ? h * draw_head_stride : 0);
    double* phq = (double*)malloc(sizeof(double) * (size_t)(Lq * F + 1));
    double* phk = (double*)malloc(sizeof(double) * (size_t)(Lk * F + 1));
    if (!phq || !phk) { bad |= 1; free(phq); free(phk); continue; }
    bad |= orc_featmap(Lq, d, R, m, eps, q + h * Lq * d, ah, gh, phq);
    bad |= orc_featmap(Lk, d, R, m, eps, k + h * Lk * d, ah, gh, phk);
    const double* vh = v + h * Lk * dv;
    const double* S0h = S0 ? S0 + h * (int64_t)F * dv : NULL;
    const double* z0h = z0 ? z0 + h * (int64_t)F : NULL;
    for (int64_t i = 0; i < Lq; ++i) {
      const double* qf = phq + i * F;
      double den = 0.0;
      double* orow = o + (h * Lq + i) * dv;
      for (int e = 0; e < dv; ++e) orow[e] = 0.0;
      for (int64_t j = 0; j < Lk; ++j) {
        double s = 0.0;
        for (int f = 0; f < F; ++f) s += qf[f] * phk[j * F + f];
        den += s;
        for (int e = 0; e < dv; ++e) orow[e] += s * vh[j * dv + e];
      }
      if (z0h)
        for (int f = 0; f < F; ++f) den += qf[f] * z0h[f];
      if (S0h)
        for (int e = 0; e < dv; ++e)
          for (int f = 0; f < F; ++f) orow[e] += qf[f] * S0h[(size_t)f * dv + e];
      for (int e = 0; e < dv; ++e) orow[e] /= den;
    }
    if (S_out || z_out) {
      for (int f = 0; f < F; ++f) {
        for (int e = 0; e < dv; ++e) {
          double acc = S0h ? S0h[(size_t)f * dv + e] : 0.0;
          for (int64_t j = 0; j < Lk; ++j) acc += phk[j * F + f] * vh[j * dv + e];
          if (S_out) S_out[(h * F + f) * (int64_t)dv + e] = acc;
        }
        double zacc = z0h ? z0h[f] : 0.0;
        for (int64_t j = 0; j < Lk; ++j) zacc += phk[j * F + f];
        if (z_out) z_out[h * F + f] = zacc;
      }
    }
    free(phq);
    free(phk);
  }
  return bad ? ORC_BAD : ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Backward of the causal forward.  The gradient of a scalar loss whose
 * derivative with respect to o is dout (and, optionally, dS_T / dz_T with
 * respect to the final state) is the chain rule applied to the definitions
 * above; the pages define only the forward ([SLAY-rev] Proposed method,
 * bullets 1-6), so every step below is that forward differentiated.          */

/* Vector-Jacobian product of the feature map: dx = J_phi(x)^T dphi.
 * With y_a = a.xh, y_g = g.xh, e = exp(sqrt(beta) y_g - beta/2) and
 * phi = sqrt(alpha/m) y_a^2 e:
 *   d phi / d xh = sqrt(alpha/m) e (2 y_a a + sqrt(beta) y_a^2 g),
 * and for xh = x / max(|x|, 1e-12):
 *   d xh / d x = (I - xh xh^T) / |x|   if |x| >= 1e-12,   I / 1e-12 otherwise.  */
int orc_featmap_vjp(int64_t n, int d, int R, int m, double eps, const double* x,
                    const double* a, const double* g, const double* dphi, double* dx) {
  if (n < 0 || d < 1 || R < 1 || m < 1) return ORC_BAD;
  double* alpha = (double*)malloc(sizeof(double) * (size_t)R);
  double* beta = (double*)malloc(sizeof(double) * (size_t)R);
  if (!alpha || !beta) { free(alpha); free(beta); return ORC_BAD; }
  int st = orc_node_params(R, eps, alpha, beta);
  if (st != ORC_OK) { free(alpha); free(beta); return st; }
  const int F = R * m;
  int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
  for (int64_t i = 0; i < n; ++i) {
    const double* xi = x + i * d;
    double* dxi = dx + i * d;
    double* xh = (double*)malloc(sizeof(double) * (size_t)d);
    double* dxh = (double*)calloc((size_t)d, sizeof(double));
    if (!xh || !dxh) { bad |= 1; free(xh); free(dxh); continue; }
    double nrm = 0.0;
    for (int c = 0; c < d; ++c) nrm += xi[c] * xi[c];
    nrm = sqrt(nrm);
    const int clamped = nrm < 1e-12;
    const double nu = clamped ? 1e-12 : nrm;
    for (int c = 0; c < d; ++c) xh[c] = xi[c] / nu;
    for (int r = 0; r < R; ++r) {
      for (int t = 0; t < m; ++t) {
        const double* ar = a + (size_t)(r * m + t) * d;
        const double* gr = g + (size_t)(r * m + t) * d;
        double ya = 0.0, yg = 0.0;
        for (int c = 0; c < d; ++c) {
          ya += ar[c] * xh[c];
          yg += gr[c] * xh[c];
        }
        const double scale = sqrt(alpha[r] / m);
        const double e = exp(sqrt(beta[r]) * yg - 0.5 * beta[r]);
        const double df = dphi[i * F + r * m + t];
        for (int c = 0; c < d; ++c)
          dxh[c] += df * scale * e * (2.0 * ya * ar[c] + sqrt(beta[r]) * ya * ya * gr[c]);
      }
    }
    if (clamped) {
      for (int c = 0; c < d; ++c) dxi[c] = dxh[c] / nu;
    } else {
      double proj = 0.0;
      for (int c = 0; c < d; ++c) proj += xh[c] * dxh[c];
      for (int c = 0; c < d; ++c) dxi[c] = (dxh[c] - xh[c] * proj) / nu;
    }
    free(xh);
    free(dxh);
  }
  free(alpha);
  free(beta);
  return bad ? ORC_BAD : ORC_OK;
}

/* Feature-space backward of one head.  Forward: s_ij = phq_i . phk_j,
 * den_i = sum_{j<=i} s_ij + phq_i . z0, num_i = sum_{j<=i} s_ij v_j + S0^T phq_i,
 * o_i = num_i / den_i, and the final state S_T = S0 + sum_j phk_j v_j^T,
 * z_T = z0 + sum_j phk_j.  With g_i = dout_i / den_i and
 * h_i = -(dout_i . o_i) / den_i (the derivatives through num_i and den_i),
 * ds_ij = g_i . v_j + h_i for j <= i, and
 *   dphq_i = sum_{j<=i} ds_ij phk_j + S0 g_i + z0 h_i
 *   dphk_j = sum_{i>=j} ds_ij phq_i + dS_T v_j + dz_T
 *   dv_j   = sum_{i>=j} s_ij g_i + dS_T^T phk_j
 *   dS0    = sum_i phq_i g_i^T + dS_T,   dz0 = sum_i phq_i h_i + dz_T.
 * S0, z0, dS_T, dz_T may be NULL (zero).  Two forms, written independently:
 * (0) brute force over the pairs (i, j); (1) recurrent: a forward sweep with
 * the running (S, z) gives o_i, g_i, h_i and dphq_i = S_i g_i + z_i h_i, and
 * a reverse sweep with U_j = dS_T + sum_{i>=j} phq_i g_i^T,
 * u_j = dz_T + sum_{i>=j} phq_i h_i gives dphk_j = U_j v_j + u_j and
 * dv_j = U_j^T phk_j.                                                        */
static int attn_bwd_head(int form, int64_t L, int F, int dv, const double* phq, const double* phk,
                         const double* v, const double* S0, const double* z0, const double* dout,
                         const double* dST, const double* dzT, double* dphq, double* dphk,
                         double* dvv, double* dS0, double* dz0) {
  double* g = (double*)malloc(sizeof(double) * (size_t)(L * dv + 1));
  double* hh = (double*)malloc(sizeof(double) * (size_t)(L + 1));
  double* S = (double*)calloc((size_t)F * dv, sizeof(double));
  double* z = (double*)calloc((size_t)F, sizeof(double));
  double* o = (double*)malloc(sizeof(double) * (size_t)dv);
  if (!g || !hh || !S || !z || !o) { free(g); free(hh); free(S); free(z); free(o); return ORC_BAD; }
  if (form == 0) {
    for (int64_t i = 0; i < L; ++i) {
      double den = 0.0;
      for (int e = 0; e < dv; ++e) o[e] = 0.0;
      for (int64_t j = 0; j <= i; ++j) {
        double s = 0.0;
        for (int f = 0; f < F; ++f) s += phq[i * F + f] * phk[j * F + f];
        den += s;
        for (int e = 0; e < dv; ++e) o[e] += s * v[j * dv + e];
      }
      for (int f = 0; f < F; ++f) {
        if (z0) den += phq[i * F + f] * z0[f];
        if (S0)
          for (int e = 0; e < dv; ++e) o[e] += phq[i * F + f] * S0[(size_t)f * dv + e];
      }
      double dot = 0.0;
      for (int e = 0; e < dv; ++e) {
        o[e] /= den;
        dot += dout[i * dv + e] * o[e];
        g[i * dv + e] = dout[i * dv + e] / den;
      }
      hh[i] = -dot / den;
    }
    for (int64_t i = 0; i < L; ++i) {
      for (int f = 0; f < F; ++f) {
        double acc = 0.0;
        for (int64_t j = 0; j <= i; ++j) {
          double ds = hh[i];
          for (int e = 0; e < dv; ++e) ds += g[i * dv + e] * v[j * dv + e];
          acc += ds * phk[j * F + f];
        }
        if (S0)
          for (int e = 0; e < dv; ++e) acc += S0[(size_t)f * dv + e] * g[i * dv + e];
        if (z0) acc += z0[f] * hh[i];
        dphq[i * F + f] = acc;
      }
    }
    for (int64_t j = 0; j < L; ++j) {
      for (int f = 0; f < F; ++f) {
        double acc = 0.0;
        for (int64_t i = j; i < L; ++i) {
          double ds = hh[i];
          for (int e = 0; e < dv; ++e) ds += g[i * dv + e] * v[j * dv + e];
          acc += ds * phq[i * F + f];
        }
        if (dST)
          for (int e = 0; e < dv; ++e) acc += dST[(size_t)f * dv + e] * v[j * dv + e];
        if (dzT) acc += dzT[f];
        dphk[j * F + f] = acc;
      }
      for (int e = 0; e < dv; ++e) {
        double acc = 0.0;
        for (int64_t i = j; i < L; ++i) {
          double s = 0.0;
          for (int f = 0; f < F; ++f) s += phq[i * F + f] * phk[j * F + f];
          acc += s * g[i * dv + e];
        }
        if (dST)
          for (int f = 0; f < F; ++f) acc += dST[(size_t)f * dv + e] * phk[j * F + f];
        dvv[j * dv + e] = acc;
      }
    }
    for (int f = 0; f < F; ++f) {
      for (int e = 0; e < dv; ++e) {
        double acc = dST ? dST[(size_t)f * dv + e] : 0.0;
        for (int64_t i = 0; i < L; ++i) acc += phq[i * F + f] * g[i * dv + e];
        if (dS0) dS0[(size_t)f * dv + e] = acc;
      }
      double acc = dzT ? dzT[f] : 0.0;
      for (int64_t i = 0; i < L; ++i) acc += phq[i * F + f] * hh[i];
      if (dz0) dz0[f] = acc;
    }
  } else {
    if (S0) memcpy(S, S0, sizeof(double) * (size_t)F * dv);
    if (z0) memcpy(z, z0, sizeof(double) * (size_t)F);
    for (int64_t i = 0; i < L; ++i) {
      for (int f = 0; f < F; ++f) {
        const double kf = phk[i * F + f];
        for (int e = 0; e < dv; ++e) S[(size_t)f * dv + e] += kf * v[i * dv + e];
        z[f] += kf;
      }
      double den = 0.0;
      for (int f = 0; f < F; ++f) den += phq[i * F + f] * z[f];
      double dot = 0.0;
      for (int e = 0; e < dv; ++e) {
        double num = 0.0;
        for (int f = 0; f < F; ++f) num += phq[i * F + f] * S[(size_t)f * dv + e];
        dot += dout[i * dv + e] * (num / den);
        g[i * dv + e] = dout[i * dv + e] / den;
      }
      hh[i] = -dot / den;
      for (int f = 0; f < F; ++f) {
        double acc = z[f] * hh[i];
        for (int e = 0; e < dv; ++e) acc += S[(size_t)f * dv + e] * g[i * dv + e];
        dphq[i * F + f] = acc;
      }
    }
    /* reverse sweep: S, z now hold U, u */
    for (int f = 0; f < F; ++f) {
      for (int e = 0; e < dv; ++e) S[(size_t)f * dv + e] = dST ? dST[(size_t)f * dv + e] : 0.0;
      z[f] = dzT ? dzT[f] : 0.0;
    }
    for (int64_t j = L - 1; j >= 0; --j) {
      for (int f = 0; f < F; ++f) {
        const double qf = phq[j * F + f];
        for (int e = 0; e < dv; ++e) S[(size_t)f * dv + e] += qf * g[j * dv + e];
        z[f] += qf * hh[j];
      }
      for (int f = 0; f < F; ++f) {
        double acc = z[f];
        for (int e = 0; e < dv; ++e) acc += S[(size_t)f * dv + e] * v[j * dv + e];
        dphk[j * F + f] = acc;
      }
      for (int e = 0; e < dv; ++e) {
        double acc = 0.0;
        for (int f = 0; f < F; ++f) acc += S[(size_t)f * dv + e] * phk[j * F + f];
        dvv[j * dv + e] = acc;
      }
    }
    if (dS0) memcpy(dS0, S, sizeof(double) * (size_t)F * dv);
    if (dz0) memcpy(dz0, z, sizeof(double) * (size_t)F);
  }
  free(g);
  free(hh);
  free(S);
  free(z);
  free(o);
  return ORC_OK;
}

/* Whole causal SLAY backward over nh heads (parallel over heads): given the
 * forward's inputs and dout [nh][L][dv] (and nullable dS_T [nh][F][dv],
 * dz_T [nh][F]), returns dq, dk [nh][L][d], dv [nh][L][dv] and nullable
 * dS0 [nh][F][dv], dz0 [nh][F].  The draws are constants (random features
 * are not trained).  form: 0 brute force, 1 recurrent.                       */
int orc_slay_causal_bwd(int64_t nh, int64_t L, int d, int dv, int R, int m, double eps,
                        const double* q, const double* k, const double* v, const double* a,
                        const double* g, int64_t draw_head_stride, int form, const double* S0,
                        const double* z0, const double* dout, const double* dS_T, const double* dz_T,
                        double* dq, double* dk, double* dvv, double* dS0, double* dz0) {
  if (nh < 0 || L < 0 || d < 1 || dv < 1 || R < 1 || m < 1 || (form != 0 && form != 1)) return ORC_BAD;
  const int F = R * m;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
  for (int64_t h = 0; h < nh; ++h) {
    const double* ah = a + (draw_head_stride > 0 ? h * draw_head_stride : 0);
    const double* gh = g + (draw_head_stride > 0 ? h * draw_head_stride : 0);
    const size_t nf = (size_t)(L * F + 1);
    double* phq = (double*)malloc(sizeof(double) * nf);
    double* phk = (double*)malloc(sizeof(double) * nf);
    double* dphq = (double*)malloc(sizeof(double) * nf);
    double* dphk = (double*)malloc(sizeof(double) * nf);
    if (!phq || !phk || !dphq || !dphk) {
      bad |= 1;
      free(phq); free(phk); free(dphq); free(dphk);
      continue;
    }
    bad |= orc_featmap(L, d, R, m, eps, q + h * L * d, ah, gh, phq);
    bad |= orc_featmap(L, d, R, m, eps, k + h * L * d, ah, gh, phk);
    const int64_t sF = (int64_t)F * dv;
    bad |= attn_bwd_head(form, L, F, dv, phq, phk, v + h * L * dv, S0 ? S0 + h * sF : NULL,
                         z0 ? z0 + h * (int64_t)F : NULL, dout + h * L * dv, dS_T ? dS_T + h * sF : NULL,
                         dz_T ? dz_T + h * (int64_t)F : NULL, dphq, dphk, dvv + h * L * dv,
                         dS0 ? dS0 + h * sF : NULL, dz0 ? dz0 + h * (int64_t)F : NULL);
    bad |= orc_featmap_vjp(L, d, R, m, eps, q + h * L * d, ah, gh, dphq, dq + h * L * d);
    bad |= orc_featmap_vjp(L, d, R, m, eps, k + h * L * d, ah, gh, dphk, dk + h * L * d);
    free(phq);
    free(phk);
    free(dphq);
    free(dphk);
  }
  return bad ? ORC_BAD : ORC_OK;
}

/* Threads the OpenMP loops above use (the CPU baseline reports it). */
int orc_max_threads(void) { return omp_get_max_threads(); }
