// slay_api.cpp -- the C ABI of libslay: host-side argument checking, the
// Gauss-Laguerre mixture constants, and dispatch to the HIP kernels.
//
// Nothing here allocates device memory; every launch goes to the caller's
// stream.  Errors are reported before anything is enqueued whenever the
// cause is visible on the host.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <map>
#include <utility>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "slay.h"
#include "slay_internal.hpp"

namespace {

thread_local std::string g_last_error;

constexpr int32_t kNoncausalChunk = 64;  // token chunk of both non-causal paths

slay_status_t fail(slay_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

slay_status_t ok() {
  g_last_error.clear();
  return SLAY_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ---------------------------------------------------------------------------
// Gauss-Laguerre rule (review "Proposed method" bullet 4), fp64.
// Nodes: eigenvalues of the symmetric tridiagonal Jacobi matrix of the
// Laguerre recurrence (diagonal 2i+1, off-diagonal i+1), by cyclic Jacobi
// rotations, each then polished by Newton steps on L_R.  Weights: the
// Christoffel numbers w = 1 / sum_{k<R} L_k(x)^2 (L_k orthonormal for e^{-x}).
void laguerre_pair(int n, double x, double* ln, double* lnm1) {
  double a = 1.0, b = 1.0 - x;  // L_0, L_1
  if (n == 0) {
    *ln = 1.0;
    *lnm1 = 0.0;
    return;
  }
  for (int k = 1; k < n; ++k) {
    const double c = ((2.0 * k + 1.0 - x) * b - k * a) / (k + 1.0);
    a = b;
    b = c;
  }
  *ln = b;
  *lnm1 = a;
}

bool gauss_laguerre(int R, double* x, double* w) {
  if (R < 1 || R > 64) return false;
  std::vector<double> A((size_t)R * R, 0.0), V((size_t)R * R, 0.0);
  for (int i = 0; i < R; ++i) {
    A[(size_t)i * R + i] = 2.0 * i + 1.0;
    V[(size_t)i * R + i] = 1.0;
    if (i + 1 < R) A[(size_t)i * R + i + 1] = A[(size_t)(i + 1) * R + i] = i + 1.0;
  }
  for (int sweep = 0; sweep < 100; ++sweep) {
    double off = 0.0;
    for (int p = 0; p < R; ++p)
      for (int q = p + 1; q < R; ++q) off += A[(size_t)p * R + q] * A[(size_t)p * R + q];
    if (off < 1e-300) break;
    for (int p = 0; p < R; ++p)
      for (int q = p + 1; q < R; ++q) {
        const double apq = A[(size_t)p * R + q];
        if (std::fabs(apq) < 1e-300) continue;
        const double tau = (A[(size_t)q * R + q] - A[(size_t)p * R + p]) / (2.0 * apq);
        const double t = (tau >= 0 ? 1.0 : -1.0) / (std::fabs(tau) + std::sqrt(1.0 + tau * tau));
        const double c = 1.0 / std::sqrt(1.0 + t * t), s = t * c;
        for (int k = 0; k < R; ++k) {  // A <- A J (columns p, q)
          const double akp = A[(size_t)k * R + p], akq = A[(size_t)k * R + q];
          A[(size_t)k * R + p] = c * akp - s * akq;
          A[(size_t)k * R + q] = s * akp + c * akq;
        }
        for (int k = 0; k < R; ++k) {  // A <- J^T A (rows p, q)
          const double apk = A[(size_t)p * R + k], aqk = A[(size_t)q * R + k];
          A[(size_t)p * R + k] = c * apk - s * aqk;
          A[(size_t)q * R + k] = s * apk + c * aqk;
        }
        for (int k = 0; k < R; ++k) {
          const double vkp = V[(size_t)k * R + p], vkq = V[(size_t)k * R + q];
          V[(size_t)k * R + p] = c * vkp - s * vkq;
          V[(size_t)k * R + q] = s * vkp + c * vkq;
        }
      }
  }
  std::vector<double> nodes(R);
  for (int i = 0; i < R; ++i) nodes[i] = A[(size_t)i * R + i];
  std::sort(nodes.begin(), nodes.end());
  for (int i = 0; i < R; ++i) {
    double xi = nodes[i];
    for (int it = 0; it < 8; ++it) {  // Newton on L_R; L_R' = R (L_R - L_{R-1}) / x
      double ln, lm;
      laguerre_pair(R, xi, &ln, &lm);
      const double d = R * (ln - lm) / xi;
      if (d == 0.0) break;
      const double step = ln / d;
      xi -= step;
      if (std::fabs(step) <= 1e-16 * std::fabs(xi)) break;
    }
    double sum = 0.0, a = 1.0, b = 1.0 - xi;
    sum += a * a;
    if (R > 1) sum += b * b;
    for (int k = 1; k + 1 < R; ++k) {
      const double c = ((2.0 * k + 1.0 - xi) * b - k * a) / (k + 1.0);
      a = b;
      b = c;
      sum += b * b;
    }
    x[i] = xi;
    w[i] = 1.0 / sum;
  }
  return true;
}

bool node_params(int R, double eps, double* alpha, double* beta) {
  std::vector<double> x(R), w(R);
  if (!gauss_laguerre(R, x.data(), w.data())) return false;
  for (int r = 0; r < R; ++r) {
    alpha[r] = w[r] / (2.0 + eps);  // Laplace variable s = x/(2+eps)
    beta[r] = 2.0 * x[r] / (2.0 + eps);
  }
  return true;
}

// fp32 kernel constants: phi = (y_a inv)^2 exp2(y_g inv c1 + c0)
slay::NodeConsts node_consts(int R, int m, double eps) {
  slay::NodeConsts nc{};
  double alpha[slay::kMaxNodes], beta[slay::kMaxNodes];
  node_params(R, eps, alpha, beta);
  const double log2e = 1.4426950408889634;
  for (int r = 0; r < R; ++r) {
    nc.c1[r] = (float)(std::sqrt(beta[r]) * log2e);
    nc.c0[r] = (float)(-0.5 * beta[r] * log2e + 0.5 * std::log2(alpha[r] / m));
  }
  return nc;
}

slay_status_t check_params(const slay_params_t* p) {
  if (!p) return fail(SLAY_E_INVALID, "params is NULL");
  if (p->d != 32 && p->d != 64 && p->d != 128)
    return fail(SLAY_E_UNSUPPORTED, "d = %d not supported (32, 64, 128)", p->d);
  if (p->R < 1 || p->R > slay::kMaxNodes) return fail(SLAY_E_INVALID, "R = %d outside [1, 16]", p->R);
  if (p->m < 16 || p->m % 16 != 0) return fail(SLAY_E_UNSUPPORTED, "m = %d must be a positive multiple of 16", p->m);
  if (!(p->eps > 0.0) || !std::isfinite(p->eps)) return fail(SLAY_E_INVALID, "eps must be finite and > 0");
  if (p->draw_dtype != SLAY_F32 && p->draw_dtype != SLAY_BF16) return fail(SLAY_E_INVALID, "bad draw dtype");
  if (!p->anchors || !p->prf) return fail(SLAY_E_INVALID, "anchors/prf pointer is NULL");
  if (!aligned16(p->anchors) || !aligned16(p->prf)) return fail(SLAY_E_INVALID, "draws must be 16-byte aligned");
  if (p->n_draw_sets < 1) return fail(SLAY_E_INVALID, "n_draw_sets must be >= 1");
  const int64_t per = (int64_t)p->R * p->m * p->d;
  if (p->n_draw_sets > 1 && (p->draw_set_stride < per || p->draw_set_stride % 8 != 0))
    return fail(SLAY_E_INVALID, "draw_set_stride must be >= R*m*d and a multiple of 8");
  if ((int64_t)p->R * p->m > 4096) return fail(SLAY_E_UNSUPPORTED, "R*m > 4096");
  return SLAY_OK;
}

// One block of positive orthogonal random-feature directions (the
// linearized 2-simplicial attention page's summary: positive orthogonal
// random features), fp64.  The d x d Gaussian matrix G is factored G = QR by
// Householder reflections; with the columns of Q multiplied by sign(R_ii) the
// factor is the unique one with a positive diagonal of R, which makes it
// Haar-distributed over the orthogonal group.  Row i of the block is column i
// of that Q times |c_i|, the length of an independent Gaussian vector c_i
// (chi-distributed with d degrees of freedom), so every row is marginally
// N(0, I_d) while the rows of the block are mutually orthogonal.
// g, c: [d][d] row-major; out: rows_out <= d rows of d values.
void orthogonal_block(int d, const double* g, const double* c, int rows_out, float* out) {
  std::vector<double> a(g, g + (size_t)d * d);  // reduced in place to R
  std::vector<double> vs((size_t)d * d, 0.0);   // Householder vectors, v_k in vs[k][k..]
  std::vector<double> rdiag(d);
  for (int k = 0; k < d; ++k) {
    double nrm = 0.0;
    for (int i = k; i < d; ++i) nrm += a[(size_t)i * d + k] * a[(size_t)i * d + k];
    nrm = std::sqrt(nrm);
    const double x0 = a[(size_t)k * d + k];
    const double alpha = x0 >= 0.0 ? -nrm : nrm;  // reflect x onto alpha e_k, away from x0 (no cancellation)
    double* v = &vs[(size_t)k * d];
    for (int i = k; i < d; ++i) v[i] = a[(size_t)i * d + k];
    v[k] -= alpha;
    double vn = 0.0;
    for (int i = k; i < d; ++i) vn += v[i] * v[i];
    if (vn > 0.0) {
      const double inv = 1.0 / std::sqrt(vn);
      for (int i = k; i < d; ++i) v[i] *= inv;
      for (int j = k; j < d; ++j) {  // a[k.., j] -= 2 v (v . a[k.., j])
        double dot = 0.0;
        for (int i = k; i < d; ++i) dot += v[i] * a[(size_t)i * d + j];
        for (int i = k; i < d; ++i) a[(size_t)i * d + j] -= 2.0 * v[i] * dot;
      }
    }
    rdiag[k] = a[(size_t)k * d + k];
  }
  // Q = H_0 H_1 ... H_{d-1}: apply the reflections to the identity, last one first
  std::vector<double> q((size_t)d * d, 0.0);
  for (int i = 0; i < d; ++i) q[(size_t)i * d + i] = 1.0;
  for (int k = d - 1; k >= 0; --k) {
    const double* v = &vs[(size_t)k * d];
    for (int j = 0; j < d; ++j) {
      double dot = 0.0;
      for (int i = k; i < d; ++i) dot += v[i] * q[(size_t)i * d + j];
      for (int i = k; i < d; ++i) q[(size_t)i * d + j] -= 2.0 * v[i] * dot;
    }
  }
  for (int i = 0; i < rows_out; ++i) {  // row i = sign(R_ii) Q[:, i] |c_i|
    double len = 0.0;
    for (int t = 0; t < d; ++t) len += c[(size_t)i * d + t] * c[(size_t)i * d + t];
    const double sc = (rdiag[i] < 0.0 ? -1.0 : 1.0) * std::sqrt(len);
    for (int t = 0; t < d; ++t) out[(size_t)i * d + t] = (float)(q[(size_t)t * d + i] * sc);
  }
}

bool mul_ok(int64_t a, int64_t b) { return a == 0 || b <= INT64_MAX / a; }

slay_status_t device_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(SLAY_E_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

slay::ChunkedArgs chunked_args(const slay_params_t* p, const void* q, const void* k, const void* v,
                               slay_dtype_t dt, int32_t B, int32_t H, int64_t L, int32_t dv, int32_t chunk) {
  slay::ChunkedArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.io_bf16 = dt == SLAY_BF16;
  a.causal = true;
  a.n_heads = (int64_t)B * H;
  a.L = L;
  a.Lq = L;
  a.d = p->d;
  a.dv = dv;
  a.F = p->R * p->m;
  a.m = p->m;
  a.R = p->R;
  a.chunk = chunk;
  a.anchors = p->anchors;
  a.prf = p->prf;
  a.draw_set_stride = p->draw_set_stride;
  a.n_draw_sets = p->n_draw_sets;
  return a;
}

}  // namespace

extern "C" {

slay_status_t slay_featmap(const slay_params_t* params, const void* x, slay_dtype_t x_dtype, int64_t n_rows,
                           int64_t rows_per_head, void* phi, slay_dtype_t phi_dtype, void* stream) {
  slay_status_t st = check_params(params);
  if (st != SLAY_OK) return st;
  if (n_rows < 0) return fail(SLAY_E_INVALID, "n_rows < 0");
  if (x_dtype != params->draw_dtype) return fail(SLAY_E_UNSUPPORTED, "x dtype must equal the draw dtype");
  if (phi_dtype != SLAY_F32 && phi_dtype != SLAY_BF16) return fail(SLAY_E_INVALID, "bad phi dtype");
  if (n_rows == 0) return ok();
  if (!x || !phi) return fail(SLAY_E_INVALID, "x/phi pointer is NULL");
  if (!aligned16(x) || !aligned16(phi)) return fail(SLAY_E_INVALID, "x/phi must be 16-byte aligned");
  const int F = params->R * params->m;
  if (!mul_ok(n_rows, F) || !mul_ok(n_rows, params->d)) return fail(SLAY_E_INVALID, "n_rows too large");
  int64_t rph = n_rows, nh = 1;
  if (params->n_draw_sets > 1) {
    if (rows_per_head <= 0 || n_rows % rows_per_head != 0)
      return fail(SLAY_E_INVALID, "rows_per_head must divide n_rows when draws are per head");
    rph = rows_per_head;
    nh = n_rows / rows_per_head;
  }
  slay::FeatmapArgs a{};
  a.x = x;
  a.rows_per_head = rph;
  a.n_heads = nh;
  a.d = params->d;
  a.F = F;
  a.m = params->m;
  a.x_bf16 = x_dtype == SLAY_BF16;
  a.anchors = params->anchors;
  a.prf = params->prf;
  a.draw_set_stride = params->draw_set_stride;
  a.n_draw_sets = params->n_draw_sets;
  a.nc = node_consts(params->R, params->m, params->eps);
  a.phi = phi;
  a.phi_bf16 = phi_dtype == SLAY_BF16;
  return device_status(slay::launch_featmap(a, static_cast<hipStream_t>(stream)), "slay_featmap launch");
}

size_t slay_attn_chunked_fwd_workspace_size(const slay_params_t* params, int32_t B, int32_t H, int64_t L,
                                            int32_t dv, int32_t chunk, slay_dtype_t io_dtype) {
  if (check_params(params) != SLAY_OK || B < 0 || H < 0 || L < 0 || dv < 1 || chunk < 1) return 0;
  slay::ChunkedArgs a = chunked_args(params, nullptr, nullptr, nullptr, io_dtype, B, H, L, dv, chunk);
  if (a.n_heads == 0 || L == 0) return 0;
  if (slay::fused_supported(a)) return slay::fused_workspace_bytes(a);
  if (slay::wide_supported(a)) return slay::wide_workspace_bytes(a);
  return slay::generic_workspace_bytes(a);
}

slay_status_t slay_attn_chunked_fwd(const slay_params_t* params, const void* q, const void* k, const void* v,
                                    slay_dtype_t io_dtype, int32_t B, int32_t H, int64_t L, int32_t dv,
                                    int32_t chunk, const float* S0, const float* z0, void* o, float* S_out,
                                    float* z_out, void* workspace, size_t workspace_bytes, void* stream) {
  return slay::chunked_fwd_entry(params, q, k, v, io_dtype, B, H, L, dv, chunk, S0, z0, o, S_out, z_out, workspace,
                                 workspace_bytes, stream, nullptr);
}

}  // extern "C"

namespace slay {

slay_status_t chunked_fwd_entry(const slay_params_t* params, const void* q, const void* k, const void* v,
                                slay_dtype_t io_dtype, int32_t B, int32_t H, int64_t L, int32_t dv, int32_t chunk,
                                const float* S0, const float* z0, void* o, float* S_out, float* z_out,
                                void* workspace, size_t workspace_bytes, void* stream, ScratchFn scratch) {
  slay_status_t st = check_params(params);
  if (st != SLAY_OK) return st;
  if (B < 0 || H < 0 || L < 0) return fail(SLAY_E_INVALID, "B, H, L must be >= 0");
  if (dv < 1) return fail(SLAY_E_INVALID, "dv must be >= 1");
  if (chunk < 1 || chunk > 128) return fail(SLAY_E_INVALID, "chunk = %d outside [1, 128]", chunk);
  if (io_dtype != SLAY_F32 && io_dtype != SLAY_BF16) return fail(SLAY_E_INVALID, "bad io dtype");
  if (io_dtype != params->draw_dtype) return fail(SLAY_E_UNSUPPORTED, "io dtype must equal the draw dtype");
  const int64_t nh = (int64_t)B * H;
  const int F = params->R * params->m;
  if (!mul_ok(nh, L) || !mul_ok(nh * L, std::max<int64_t>(params->d, dv)) || !mul_ok(nh * L, F))
    return fail(SLAY_E_INVALID, "problem size overflows");
  const bool tokens = nh > 0 && L > 0;
  if (tokens) {
    if (!q || !k || !v || !o) return fail(SLAY_E_INVALID, "q/k/v/o pointer is NULL");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
      return fail(SLAY_E_INVALID, "q/k/v/o must be 16-byte aligned");
    const int es = io_dtype == SLAY_BF16 ? 2 : 4;
    if ((dv * es) % 16 != 0 || (params->d * es) % 16 != 0)
      return fail(SLAY_E_UNSUPPORTED, "rows of q/k/v must be whole 16-byte vectors (dv = %d)", dv);
  }
  slay::ChunkedArgs a = chunked_args(params, q, k, v, io_dtype, B, H, L, dv, chunk);
  a.nc = node_consts(params->R, params->m, params->eps);
  a.S0 = S0;
  a.z0 = z0;
  a.o = o;
  a.S_out = S_out;
  a.z_out = z_out;
  a.ws = workspace;
  a.ws_bytes = workspace_bytes;
  // kernel family: fused (feature map on chip), wide (feature maps in HBM,
  // state on chip), generic (plain FMA, any accepted shape and dtype)
  const int path = slay::fused_supported(a) ? 0 : (slay::wide_supported(a) ? 1 : 2);
  if (path == 2 && !slay::generic_supported(a))
    return fail(SLAY_E_UNSUPPORTED, "shape not supported (d=%d dv=%d F=%d chunk=%d)", params->d, dv, F, chunk);
  const size_t need = (!tokens) ? 0
                      : path == 0 ? slay::fused_workspace_bytes(a)
                      : path == 1 ? slay::wide_workspace_bytes(a)
                                  : slay::generic_workspace_bytes(a);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (scratch && need > 0) {  // the caller's fixed scratch, looked up only once every argument is checked
    if (need > workspace_bytes)
      return fail(SLAY_E_UNSUPPORTED, "workspace of %zu bytes exceeds the fixed scratch of %zu bytes", need,
                  workspace_bytes);
    const hipError_t e = scratch(s, &workspace);
    if (e != hipSuccess) return device_status(e, "scratch lookup");
    a.ws = workspace;
  }
  if (workspace_bytes < need) return fail(SLAY_E_INVALID, "workspace too small: %zu < %zu", workspace_bytes, need);
  if (need > 0 && !workspace) return fail(SLAY_E_INVALID, "workspace is NULL");
  if (need > 0 && !aligned16(workspace)) return fail(SLAY_E_INVALID, "workspace must be 16-byte aligned");
  if (nh == 0) return ok();
  const hipError_t e = path == 0 ? slay::launch_fused(a, s) : path == 1 ? slay::launch_wide(a, s)
                                                                        : slay::launch_generic(a, s);
  return device_status(e, "slay_attn_chunked_fwd launch");
}

}  // namespace slay

namespace {
slay::BackwardArgs backward_args(const slay_params_t* p, slay_dtype_t dt, int32_t B, int32_t H, int64_t L,
                                 int32_t dv, int32_t chunk) {
  slay::BackwardArgs a{};
  a.io_bf16 = dt == SLAY_BF16;
  a.n_heads = (int64_t)B * H;
  a.L = L;
  a.d = p->d;
  a.dv = dv;
  a.F = p->R * p->m;
  a.m = p->m;
  a.R = p->R;
  a.chunk = chunk;
  a.anchors = p->anchors;
  a.prf = p->prf;
  a.draw_set_stride = p->draw_set_stride;
  a.n_draw_sets = p->n_draw_sets;
  return a;
}
}  // namespace

extern "C" {

size_t slay_attn_chunked_bwd_workspace_size(const slay_params_t* params, int32_t B, int32_t H, int64_t L,
                                            int32_t dv, int32_t chunk, slay_dtype_t io_dtype) {
  if (check_params(params) != SLAY_OK || B < 0 || H < 0 || L < 0 || dv < 1 || chunk < 1) return 0;
  const slay::BackwardArgs a = backward_args(params, io_dtype, B, H, L, dv, chunk);
  return slay::backward_fused_supported(a) ? slay::backward_fused_workspace_bytes(a)
                                           : slay::backward_workspace_bytes(a);
}

slay_status_t slay_attn_chunked_bwd(const slay_params_t* params, const void* q, const void* k, const void* v,
                                    const void* dout, slay_dtype_t io_dtype, int32_t B, int32_t H, int64_t L,
                                    int32_t dv, int32_t chunk, const float* S0, const float* z0, const float* dS_T,
                                    const float* dz_T, void* dq, void* dk, void* dv_out, float* dS0, float* dz0,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  slay_status_t st = check_params(params);
  if (st != SLAY_OK) return st;
  if (B < 0 || H < 0 || L < 0) return fail(SLAY_E_INVALID, "B, H, L must be >= 0");
  if (dv < 1) return fail(SLAY_E_INVALID, "dv must be >= 1");
  if (chunk < 1 || chunk > 128) return fail(SLAY_E_INVALID, "chunk = %d outside [1, 128]", chunk);
  if (io_dtype != SLAY_F32 && io_dtype != SLAY_BF16) return fail(SLAY_E_INVALID, "bad io dtype");
  if (io_dtype != params->draw_dtype) return fail(SLAY_E_UNSUPPORTED, "io dtype must equal the draw dtype");
  const int64_t nh = (int64_t)B * H;
  const int F = params->R * params->m;
  if (!mul_ok(nh, L) || !mul_ok(nh * L, std::max<int64_t>(params->d, dv)) || !mul_ok(nh * L, 4 * F))
    return fail(SLAY_E_INVALID, "problem size overflows");
  const bool tokens = nh > 0 && L > 0;
  if (tokens) {
    if (!q || !k || !v || !dout || !dq || !dk || !dv_out) return fail(SLAY_E_INVALID, "q/k/v/dout/dq/dk/dv pointer is NULL");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dout) || !aligned16(dq) || !aligned16(dk) ||
        !aligned16(dv_out))
      return fail(SLAY_E_INVALID, "q/k/v/dout/dq/dk/dv must be 16-byte aligned");
  }
  slay::BackwardArgs a = backward_args(params, io_dtype, B, H, L, dv, chunk);
  const bool fused = slay::backward_fused_supported(a);
  if (!fused && !slay::backward_supported(a))
    return fail(SLAY_E_UNSUPPORTED, "backward shape not supported (d=%d dv=%d F=%d chunk=%d)", params->d, dv, F,
                chunk);
  a.q = q;
  a.k = k;
  a.v = v;
  a.dout = dout;
  a.nc = node_consts(params->R, params->m, params->eps);
  a.S0 = S0;
  a.z0 = z0;
  a.dS_T = dS_T;
  a.dz_T = dz_T;
  a.dq = dq;
  a.dk = dk;
  a.dv_out = dv_out;
  a.dS0 = dS0;
  a.dz0 = dz0;
  a.ws = workspace;
  a.ws_bytes = workspace_bytes;
  const size_t need = fused ? slay::backward_fused_workspace_bytes(a) : slay::backward_workspace_bytes(a);
  if (workspace_bytes < need) return fail(SLAY_E_INVALID, "workspace too small: %zu < %zu", workspace_bytes, need);
  if (need > 0 && !workspace) return fail(SLAY_E_INVALID, "workspace is NULL");
  if (need > 0 && !aligned16(workspace)) return fail(SLAY_E_INVALID, "workspace must be 16-byte aligned");
  if (nh == 0) return ok();
  hipStream_t s = static_cast<hipStream_t>(stream);
  return device_status(fused ? slay::launch_backward_fused(a, s) : slay::launch_backward(a, s),
                       "slay_attn_chunked_bwd launch");
}

size_t slay_attn_varlen_fwd_workspace_size(const slay_params_t* params, int32_t n_seqs, int32_t H,
                                           int64_t total_tokens, int32_t dv, slay_dtype_t io_dtype) {
  if (check_params(params) != SLAY_OK || n_seqs < 0 || H < 0 || total_tokens < 0 || dv < 1) return 0;
  slay::VarlenArgs a{};
  a.c = chunked_args(params, nullptr, nullptr, nullptr, io_dtype, 1, H, total_tokens, dv, 64);
  a.n_seqs = n_seqs;
  return slay::varlen_supported(a) ? slay::varlen_workspace_bytes(a) : 0;
}

slay_status_t slay_attn_varlen_fwd(const slay_params_t* params, const void* q, const void* k, const void* v,
                                   slay_dtype_t io_dtype, int32_t n_seqs, int32_t H, const int64_t* cu_seqlens,
                                   int64_t total_tokens, int32_t dv, const float* S0, const float* z0, void* o,
                                   float* S_out, float* z_out, void* workspace, size_t workspace_bytes, void* stream) {
  slay_status_t st = check_params(params);
  if (st != SLAY_OK) return st;
  if (n_seqs < 0 || H < 0 || total_tokens < 0) return fail(SLAY_E_INVALID, "n_seqs, H, total_tokens must be >= 0");
  if (dv < 1) return fail(SLAY_E_INVALID, "dv must be >= 1");
  if (io_dtype != SLAY_F32 && io_dtype != SLAY_BF16) return fail(SLAY_E_INVALID, "bad io dtype");
  if (io_dtype != params->draw_dtype) return fail(SLAY_E_UNSUPPORTED, "io dtype must equal the draw dtype");
  const int F = params->R * params->m;
  if (!mul_ok(H, total_tokens) || !mul_ok((int64_t)H * total_tokens, std::max<int64_t>(params->d, dv)))
    return fail(SLAY_E_INVALID, "problem size overflows");
  if (total_tokens > (int64_t)INT32_MAX - 64)  // the work list holds token rows as 32-bit integers
    return fail(SLAY_E_UNSUPPORTED, "total_tokens = %lld exceeds 2^31 - 65", (long long)total_tokens);
  slay::VarlenArgs a{};
  a.c = chunked_args(params, q, k, v, io_dtype, 1, H, total_tokens, dv, 64);
  a.n_seqs = n_seqs;
  a.cu = cu_seqlens;
  if (!slay::varlen_supported(a))
    return fail(SLAY_E_UNSUPPORTED, "variable-length batches need bf16, d = dv = 64 and R*m <= 256 (m a multiple of 32); "
                "got d=%d dv=%d F=%d", params->d, dv, F);
  if (H == 0 || n_seqs == 0) return ok();
  if (!cu_seqlens) return fail(SLAY_E_INVALID, "cu_seqlens is NULL");
  if (total_tokens > 0) {
    if (!q || !k || !v || !o) return fail(SLAY_E_INVALID, "q/k/v/o pointer is NULL");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
      return fail(SLAY_E_INVALID, "q/k/v/o must be 16-byte aligned");
  }
  a.c.nc = node_consts(params->R, params->m, params->eps);
  a.c.S0 = S0;
  a.c.z0 = z0;
  a.c.o = o;
  a.c.S_out = S_out;
  a.c.z_out = z_out;
  a.c.ws = workspace;
  a.c.ws_bytes = workspace_bytes;
  const size_t need = slay::varlen_workspace_bytes(a);
  if (workspace_bytes < need) return fail(SLAY_E_INVALID, "workspace too small: %zu < %zu", workspace_bytes, need);
  if (!workspace || !aligned16(workspace)) return fail(SLAY_E_INVALID, "workspace must be non-NULL and 16-byte aligned");
  return device_status(slay::launch_varlen(a, static_cast<hipStream_t>(stream)), "slay_attn_varlen_fwd launch");
}

size_t slay_attn_noncausal_fwd_workspace_size(const slay_params_t* params, int32_t B, int32_t H, int64_t Lq,
                                               int64_t Lk, int32_t dv, slay_dtype_t io_dtype) {
  if (check_params(params) != SLAY_OK || B < 0 || H < 0 || Lq < 0 || Lk < 0 || dv < 1) return 0;
  slay::ChunkedArgs a = chunked_args(params, nullptr, nullptr, nullptr, io_dtype, B, H, Lk, dv, kNoncausalChunk);
  a.causal = false;
  a.Lq = Lq;
  if (a.n_heads == 0) return 0;
  if (slay::fused_supported(a)) return slay::fused_workspace_bytes(a);
  return slay::generic_workspace_bytes(a);
}

slay_status_t slay_attn_noncausal_fwd(const slay_params_t* params, const void* q, const void* k, const void* v,
                                      slay_dtype_t io_dtype, int32_t B, int32_t H, int64_t Lq, int64_t Lk,
                                      int32_t dv, const float* S0, const float* z0, void* o, float* S_out,
                                      float* z_out, void* workspace, size_t workspace_bytes, void* stream) {
  slay_status_t st = check_params(params);
  if (st != SLAY_OK) return st;
  if (B < 0 || H < 0 || Lq < 0 || Lk < 0) return fail(SLAY_E_INVALID, "B, H, Lq, Lk must be >= 0");
  if (dv < 1) return fail(SLAY_E_INVALID, "dv must be >= 1");
  if (io_dtype != SLAY_F32 && io_dtype != SLAY_BF16) return fail(SLAY_E_INVALID, "bad io dtype");
  if (io_dtype != params->draw_dtype) return fail(SLAY_E_UNSUPPORTED, "io dtype must equal the draw dtype");
  const int64_t nh = (int64_t)B * H;
  const int F = params->R * params->m;
  const int64_t Lmax = std::max(Lq, Lk);
  if (!mul_ok(nh, Lmax) || !mul_ok(nh * Lmax, std::max<int64_t>(params->d, dv)) || !mul_ok(nh * Lmax, F))
    return fail(SLAY_E_INVALID, "problem size overflows");
  if (nh > 0 && Lq > 0 && Lk == 0 && !z0)
    return fail(SLAY_E_INVALID, "no keys and no initial state: every denominator would be zero");
  const int es = io_dtype == SLAY_BF16 ? 2 : 4;
  if (nh > 0 && (Lq > 0 || Lk > 0) && ((dv * es) % 16 != 0 || (params->d * es) % 16 != 0))
    return fail(SLAY_E_UNSUPPORTED, "rows of q/k/v must be whole 16-byte vectors (dv = %d)", dv);
  if (nh > 0 && Lq > 0) {
    if (!q || !o) return fail(SLAY_E_INVALID, "q/o pointer is NULL");
    if (!aligned16(q) || !aligned16(o)) return fail(SLAY_E_INVALID, "q/o must be 16-byte aligned");
  }
  if (nh > 0 && Lk > 0) {
    if (!k || !v) return fail(SLAY_E_INVALID, "k/v pointer is NULL");
    if (!aligned16(k) || !aligned16(v)) return fail(SLAY_E_INVALID, "k/v must be 16-byte aligned");
  }
  slay::ChunkedArgs a = chunked_args(params, q, k, v, io_dtype, B, H, Lk, dv, kNoncausalChunk);
  a.causal = false;
  a.Lq = Lq;
  a.nc = node_consts(params->R, params->m, params->eps);
  a.S0 = S0;
  a.z0 = z0;
  a.o = o;
  a.S_out = S_out;
  a.z_out = z_out;
  a.ws = workspace;
  a.ws_bytes = workspace_bytes;
  const bool fused = slay::fused_supported(a);
  if (!fused && !slay::generic_supported(a))
    return fail(SLAY_E_UNSUPPORTED, "shape not supported (d=%d dv=%d F=%d)", params->d, dv, F);
  const size_t need = nh == 0 ? 0 : (fused ? slay::fused_workspace_bytes(a) : slay::generic_workspace_bytes(a));
  if (workspace_bytes < need) return fail(SLAY_E_INVALID, "workspace too small: %zu < %zu", workspace_bytes, need);
  if (need > 0 && !workspace) return fail(SLAY_E_INVALID, "workspace is NULL");
  if (need > 0 && !aligned16(workspace)) return fail(SLAY_E_INVALID, "workspace must be 16-byte aligned");
  if (nh == 0) return ok();
  hipStream_t s = static_cast<hipStream_t>(stream);
  return device_status(fused ? slay::launch_fused(a, s) : slay::launch_generic(a, s),
                       "slay_attn_noncausal_fwd launch");
}

namespace {
slay::DecodeArgs decode_args(const slay_params_t* params, const void* q, const void* k, const void* v,
                             slay_dtype_t io_dtype, int64_t n_heads, int32_t dv, float* S, float* z, void* o) {
  slay::DecodeArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.io_bf16 = io_dtype == SLAY_BF16;
  a.n_heads = n_heads;
  a.d = params->d;
  a.dv = dv;
  a.F = params->R * params->m;
  a.m = params->m;
  a.anchors = params->anchors;
  a.prf = params->prf;
  a.draws_bf16 = params->draw_dtype == SLAY_BF16;
  a.draw_set_stride = params->draw_set_stride;
  a.n_draw_sets = params->n_draw_sets;
  a.S = S;
  a.z = z;
  a.o = o;
  return a;
}
}  // namespace

size_t slay_attn_recurrent_step_workspace_size(const slay_params_t* params, int64_t n_heads, int32_t dv,
                                               slay_dtype_t io_dtype) {
  if (check_params(params) != SLAY_OK || n_heads < 0 || dv < 1) return 0;
  slay::DecodeArgs a = decode_args(params, nullptr, nullptr, nullptr, io_dtype, n_heads, dv, nullptr, nullptr,
                                   nullptr);
  return slay::decode_workspace_bytes(a);
}

slay_status_t slay_attn_recurrent_step(const slay_params_t* params, const void* q, const void* k, const void* v,
                                       slay_dtype_t io_dtype, int64_t n_heads, int32_t dv, float* S, float* z,
                                       void* o, void* workspace, size_t workspace_bytes, void* stream) {
  slay_status_t st = check_params(params);
  if (st != SLAY_OK) return st;
  if (n_heads < 0) return fail(SLAY_E_INVALID, "n_heads < 0");
  if (dv < 1) return fail(SLAY_E_INVALID, "dv must be >= 1");
  if (io_dtype != SLAY_F32 && io_dtype != SLAY_BF16) return fail(SLAY_E_INVALID, "bad io dtype");
  slay::DecodeArgs a = decode_args(params, q, k, v, io_dtype, n_heads, dv, S, z, o);
  if (!slay::decode_supported(a))
    return fail(SLAY_E_UNSUPPORTED, "decode shape not supported (d=%d dv=%d F=%d, io and draw dtypes equal)", a.d,
                dv, a.F);
  if (n_heads == 0) return ok();
  if (!q || !k || !v || !o || !S || !z) return fail(SLAY_E_INVALID, "q/k/v/o/S/z pointer is NULL");
  if (!aligned16(S) || !aligned16(q) || !aligned16(k)) return fail(SLAY_E_INVALID, "q, k, S must be 16-byte aligned");
  if (!mul_ok(n_heads, (int64_t)a.F * dv)) return fail(SLAY_E_INVALID, "problem size overflows");
  const size_t need = slay::decode_workspace_bytes(a);
  if (workspace_bytes < need) return fail(SLAY_E_INVALID, "workspace too small: %zu < %zu", workspace_bytes, need);
  if (!workspace || !aligned16(workspace)) return fail(SLAY_E_INVALID, "workspace must be non-NULL and 16-byte aligned");
  a.ws = workspace;
  a.nc = node_consts(params->R, params->m, params->eps);
  return device_status(slay::launch_decode(a, static_cast<hipStream_t>(stream)), "slay_attn_recurrent_step launch");
}

slay_status_t slay_gl_table(int32_t R, double eps, double* alpha, double* beta) {
  if (R < 1 || R > slay::kMaxNodes || !alpha || !beta || !(eps > 0.0) || !std::isfinite(eps))
    return fail(SLAY_E_INVALID, "slay_gl_table: R in [1, 16], eps > 0, non-NULL outputs");
  node_params(R, eps, alpha, beta);
  return ok();
}

slay_status_t slay_orthogonal_draws(int32_t n_rows, int32_t d, const double* gauss, const double* chi, float* out) {
  if (n_rows < 0 || d < 1 || d > 4096) return fail(SLAY_E_INVALID, "slay_orthogonal_draws: n_rows >= 0, d in [1, 4096]");
  if (n_rows == 0) return ok();
  if (!gauss || !chi || !out) return fail(SLAY_E_INVALID, "slay_orthogonal_draws: NULL pointer");
  const int32_t n_blocks = (n_rows + d - 1) / d;
  for (int32_t b = 0; b < n_blocks; ++b) {
    const size_t off = (size_t)b * d * d;
    const int rows = std::min<int32_t>(d, n_rows - b * d);
    for (size_t i = 0; i < (size_t)d * d; ++i)
      if (!std::isfinite(gauss[off + i]) || !std::isfinite(chi[off + i]))
        return fail(SLAY_E_INVALID, "slay_orthogonal_draws: non-finite input");
    orthogonal_block(d, gauss + off, chi + off, rows, out + (size_t)b * d * d);
  }
  return ok();
}

const char* slay_status_string(slay_status_t status) {
  switch (status) {
    case SLAY_OK: return "ok";
    case SLAY_E_INVALID: return "invalid argument";
    case SLAY_E_UNSUPPORTED: return "unsupported shape or dtype";
    case SLAY_E_DEVICE: return "device error";
    default: return "unknown status";
  }
}

const char* slay_last_error(void) { return g_last_error.c_str(); }

int32_t slay_version(void) { return 100; }

}  // extern "C"

namespace slay {

hipError_t set_max_lds(const void* kernel, int bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  // the largest limit set so far per (kernel, device): a kernel whose LDS
  // size depends on the shape gets its limit raised when a call needs more
  static std::mutex mu;
  static std::map<std::pair<const void*, int>, int> limit;
  std::lock_guard<std::mutex> lock(mu);
  const auto it = limit.find({kernel, dev});
  if (it != limit.end() && it->second >= bytes) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) limit[{kernel, dev}] = bytes;
  return e;
}

}  // namespace slay
