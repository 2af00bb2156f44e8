// slay_backward.hip -- backward of the causal SLAY forward (general path).
//
// The forward ("SLAY: Geometry-Aware Spherical Linearized Attention with
// Yat-Kernel", abstract; nubint.ai review, "Proposed method" bullets 1-6) is
//   o_i = num_i / den_i,  num_i = phi(q_i)^T S_i,  den_i = phi(q_i)^T z_i,
//   S_i = S0 + sum_{j<=i} phi(k_j) v_j^T,  z_i = z0 + sum_{j<=i} phi(k_j).
// Its gradient, written with the augmented value v'_j = [v_j | 1], the
// augmented state S' = [S | z] and, per query, g'_i = [dout_i / den_i | h_i],
// h_i = -(dout_i . o_i) / den_i (the derivatives through num_i and den_i):
//   dphi(q_i) = S'_i g'_i
//   dphi(k_j) = U_j v'_j,        U_j = [dS_T | dz_T] + sum_{i>=j} phi(q_i) g'_i^T
//   dv_j      = U_j[:, :dv]^T phi(k_j)
//   [dS0 | dz0] = U_0
// and dq, dk follow through the feature map's Jacobian.  Chunk by chunk, the
// prefix state S'_c before chunk c and the suffix U_c after it carry
// everything outside the chunk; inside, the masked C x C blocks
// A = tril(phi(Q) phi(K)^T) and D = tril(G' V'^T) do the rest:
//   dphi(Q_c) = D phi(K_c) + G'_c S'_c^T,  dphi(K_c) = D^T phi(Q_c) + V'_c U_c^T,
//   dV_c = A^T G_c + phi(K_c) U_c[:, :dv].
//
// Launches (one stream): the feature map of q and k (fp32 to the workspace);
// per-chunk states phi(K_c)^T V'_c and their exclusive prefix (the forward's
// kernels); bwd_q (g', dphi(q), and the chunk's phi(Q_c)^T G'_c in place of
// its prefix state); the exclusive suffix of those from [dS_T | dz_T], whose
// total is [dS0 | dz0]; bwd_kv (dphi(k), dv); the feature-map VJP for q and k.
// Plain fp32 FMA throughout: it serves every dtype and shape the ABI accepts.
#include "slay_device.hpp"
#include "slay_internal.hpp"

namespace slay {

namespace {

constexpr int kBThreads = 256;
constexpr float kLn2 = 0.6931471805599453f;

template <typename T>
__device__ __forceinline__ float ld(const T* p);
template <>
__device__ __forceinline__ float ld<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float ld<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }

template <typename T>
__device__ __forceinline__ void st(T* p, float x);
template <>
__device__ __forceinline__ void st<float>(float* p, float x) { *p = x; }
template <>
__device__ __forceinline__ void st<uint16_t>(uint16_t* p, float x) { *p = f32_to_bf16(x); }

// Per (chunk, head): g' of every query of the chunk, dphi(q), and the
// chunk's phi(Q_c)^T G'_c written over its (already consumed) prefix state.
// LDS: sA [C][C] (A, then D), sG [C][dv+1] (num', then g').
template <typename TV>
__global__ __launch_bounds__(kBThreads) void bwd_q_kernel(const float* __restrict__ phiq,
                                                          const float* __restrict__ phik, const TV* __restrict__ v,
                                                          const TV* __restrict__ dout, int64_t L, int F, int dv, int C,
                                                          int64_t n_chunks, float* __restrict__ states,
                                                          float* __restrict__ gh, float* __restrict__ dphiq) {
  extern __shared__ float sm[];
  const int E1 = dv + 1;
  float* sA = sm;
  float* sG = sm + C * C;
  const int64_t h = blockIdx.y, c = blockIdx.x;
  const int64_t i0 = c * C;
  const int n = (int)min<int64_t>(C, L - i0);
  const float* pq = phiq + (h * L + i0) * F;
  const float* pk = phik + (h * L + i0) * F;
  const TV* vv = v + (h * L + i0) * dv;
  const TV* dd = dout + (h * L + i0) * dv;
  float* S = states + (h * n_chunks + c) * (int64_t)F * E1;

  for (int p = threadIdx.x; p < n * n; p += kBThreads) {  // A = tril(phi(Q) phi(K)^T)
    const int i = p / n, j = p - (p / n) * n;
    float acc = 0.f;
    if (j <= i)
      for (int f = 0; f < F; ++f) acc = fmaf(pq[(int64_t)i * F + f], pk[(int64_t)j * F + f], acc);
    sA[i * C + j] = acc;
  }
  __syncthreads();
  for (int p = threadIdx.x; p < n * E1; p += kBThreads) {  // num' = A V' + phi(Q) S'
    const int i = p / E1, e = p - (p / E1) * E1;
    float acc = 0.f;
    for (int j = 0; j <= i; ++j) acc = fmaf(sA[i * C + j], e < dv ? ld(vv + (int64_t)j * dv + e) : 1.f, acc);
    for (int f = 0; f < F; ++f) acc = fmaf(pq[(int64_t)i * F + f], S[(int64_t)f * E1 + e], acc);
    sG[i * E1 + e] = acc;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += kBThreads) {  // g' = [dout / den | -(dout . o) / den]
    const float den = sG[i * E1 + dv];
    const float inv = 1.f / den;
    float dot = 0.f;
    for (int e = 0; e < dv; ++e) {
      const float dn = ld(dd + (int64_t)i * dv + e);
      dot = fmaf(dn, sG[i * E1 + e] * inv, dot);
      sG[i * E1 + e] = dn * inv;
    }
    sG[i * E1 + dv] = -dot * inv;
  }
  __syncthreads();
  float* ghc = gh + (h * L + i0) * E1;
  for (int p = threadIdx.x; p < n * E1; p += kBThreads) ghc[p] = sG[p];
  for (int p = threadIdx.x; p < n * n; p += kBThreads) {  // D = tril(G' V'^T)
    const int i = p / n, j = p - (p / n) * n;
    float acc = 0.f;
    if (j <= i) {
      acc = sG[i * E1 + dv];
      for (int e = 0; e < dv; ++e) acc = fmaf(sG[i * E1 + e], ld(vv + (int64_t)j * dv + e), acc);
    }
    sA[i * C + j] = acc;
  }
  __syncthreads();
  float* dq = dphiq + (h * L + i0) * F;
  for (int p = threadIdx.x; p < n * F; p += kBThreads) {  // dphi(Q) = D phi(K) + G' S'^T
    const int i = p / F, f = p - (p / F) * F;
    float acc = 0.f;
    for (int j = 0; j <= i; ++j) acc = fmaf(sA[i * C + j], pk[(int64_t)j * F + f], acc);
    for (int e = 0; e < E1; ++e) acc = fmaf(sG[i * E1 + e], S[(int64_t)f * E1 + e], acc);
    dq[(int64_t)i * F + f] = acc;
  }
  __syncthreads();  // every read of S' is done: its slot now takes phi(Q_c)^T G'_c
  for (int p = threadIdx.x; p < F * E1; p += kBThreads) {
    const int f = p / E1, e = p - (p / E1) * E1;
    float acc = 0.f;
    for (int i = 0; i < n; ++i) acc = fmaf(pq[(int64_t)i * F + f], sG[i * E1 + e], acc);
    S[p] = acc;
  }
}

// Per (chunk, head), with U_c (the suffix after chunk c) in the chunk's slot:
// dphi(K_c) = D^T phi(Q_c) + V'_c U_c^T and dV_c = A^T G_c + phi(K_c) U_c[:, :dv].
// LDS: sA [C][C] (D, then A), sG [C][dv+1] (g').
template <typename TV>
__global__ __launch_bounds__(kBThreads) void bwd_kv_kernel(const float* __restrict__ phiq,
                                                           const float* __restrict__ phik, const TV* __restrict__ v,
                                                           int64_t L, int F, int dv, int C, int64_t n_chunks,
                                                           const float* __restrict__ states,
                                                           const float* __restrict__ gh, float* __restrict__ dphik,
                                                           TV* __restrict__ dv_out) {
  extern __shared__ float sm[];
  const int E1 = dv + 1;
  float* sA = sm;
  float* sG = sm + C * C;
  const int64_t h = blockIdx.y, c = blockIdx.x;
  const int64_t i0 = c * C;
  const int n = (int)min<int64_t>(C, L - i0);
  const float* pq = phiq + (h * L + i0) * F;
  const float* pk = phik + (h * L + i0) * F;
  const TV* vv = v + (h * L + i0) * dv;
  const float* U = states + (h * n_chunks + c) * (int64_t)F * E1;
  const float* ghc = gh + (h * L + i0) * E1;
  for (int p = threadIdx.x; p < n * E1; p += kBThreads) sG[p] = ghc[p];
  __syncthreads();
  for (int p = threadIdx.x; p < n * n; p += kBThreads) {  // D = tril(G' V'^T)
    const int i = p / n, j = p - (p / n) * n;
    float acc = 0.f;
    if (j <= i) {
      acc = sG[i * E1 + dv];
      for (int e = 0; e < dv; ++e) acc = fmaf(sG[i * E1 + e], ld(vv + (int64_t)j * dv + e), acc);
    }
    sA[i * C + j] = acc;
  }
  __syncthreads();
  float* dk = dphik + (h * L + i0) * F;
  for (int p = threadIdx.x; p < n * F; p += kBThreads) {  // dphi(K) = D^T phi(Q) + V' U^T
    const int j = p / F, f = p - (p / F) * F;
    float acc = U[(int64_t)f * E1 + dv];
    for (int i = j; i < n; ++i) acc = fmaf(sA[i * C + j], pq[(int64_t)i * F + f], acc);
    for (int e = 0; e < dv; ++e) acc = fmaf(ld(vv + (int64_t)j * dv + e), U[(int64_t)f * E1 + e], acc);
    dk[(int64_t)j * F + f] = acc;
  }
  __syncthreads();
  for (int p = threadIdx.x; p < n * n; p += kBThreads) {  // A = tril(phi(Q) phi(K)^T)
    const int i = p / n, j = p - (p / n) * n;
    float acc = 0.f;
    if (j <= i)
      for (int f = 0; f < F; ++f) acc = fmaf(pq[(int64_t)i * F + f], pk[(int64_t)j * F + f], acc);
    sA[i * C + j] = acc;
  }
  __syncthreads();
  TV* dvo = dv_out + (h * L + i0) * dv;
  for (int p = threadIdx.x; p < n * dv; p += kBThreads) {  // dV = A^T G + phi(K) U[:, :dv]
    const int j = p / dv, e = p - (p / dv) * dv;
    float acc = 0.f;
    for (int i = j; i < n; ++i) acc = fmaf(sA[i * C + j], sG[i * E1 + e], acc);
    for (int f = 0; f < F; ++f) acc = fmaf(pk[(int64_t)j * F + f], U[(int64_t)f * E1 + e], acc);
    st<TV>(dvo + (int64_t)j * dv + e, acc);
  }
}

// Feature-map VJP: dx = J_phi(x)^T dphi, TR rows per workgroup.
// With xh = x inv (inv = 1 / max(|x|, 1e-12)), y_a = a.xh, y_g = g.xh and
// E = exp2(y_g c1[r] + c0[r]) (so phi = y_a^2 E):
//   d phi / d xh = 2 y_a E a + phi sqrt(beta_r) g,   sqrt(beta_r) = c1[r] ln 2,
//   dx = (dxh - xh (xh . dxh)) inv   (dx = dxh inv where the norm is clamped).
// LDS: sx [TR][d] (xh), sW [TR][2F] (the weights of a and g rows), sD [TR][d].
template <typename TI>
__global__ __launch_bounds__(kBThreads) void fmvjp_kernel(const TI* __restrict__ x, const float* __restrict__ dphi,
                                                          int64_t rows_per_head, int64_t n_rows, int d, int F, int m,
                                                          const TI* __restrict__ anchors, const TI* __restrict__ prf,
                                                          int64_t draw_set_stride, int n_draw_sets, NodeConsts nc,
                                                          int TR, TI* __restrict__ dx) {
  extern __shared__ float sm[];
  float* sx = sm;
  float* sW = sx + TR * d;
  float* sD = sW + TR * 2 * F;
  __shared__ float sinv[16];
  __shared__ int sclamp[16];
  const int64_t r0 = (int64_t)blockIdx.x * TR;
  const int nr = (int)min<int64_t>(TR, n_rows - r0);
  // one draw set per workgroup: TR divides rows_per_head whenever sets differ per head
  const int64_t set = (r0 / rows_per_head) % n_draw_sets;
  const TI* A = anchors + set * draw_set_stride;
  const TI* G = prf + set * draw_set_stride;
  for (int p = threadIdx.x; p < nr * d; p += kBThreads) sx[p] = ld(x + r0 * d + p);
  __syncthreads();
  for (int r = threadIdx.x; r < nr; r += kBThreads) {
    float ss = 0.f;
    for (int c = 0; c < d; ++c) ss = fmaf(sx[r * d + c], sx[r * d + c], ss);
    const int clamp = ss < 1e-24f;
    sinv[r] = clamp ? 1e12f : 1.f / sqrtf(ss);
    sclamp[r] = clamp;
  }
  __syncthreads();
  for (int p = threadIdx.x; p < nr * d; p += kBThreads) sx[p] *= sinv[p / d];
  __syncthreads();
  for (int p = threadIdx.x; p < nr * F; p += kBThreads) {
    const int r = p / F, f = p - (p / F) * F;
    const int node = f / m;
    float ya = 0.f, yg = 0.f;
    for (int c = 0; c < d; ++c) {
      ya = fmaf(ld(A + (int64_t)f * d + c), sx[r * d + c], ya);
      yg = fmaf(ld(G + (int64_t)f * d + c), sx[r * d + c], yg);
    }
    const float E = exp2f(fmaf(yg, nc.c1[node], nc.c0[node]));
    const float phi = ya * ya * E;
    const float df = dphi[(r0 + r) * F + f];
    sW[r * 2 * F + f] = df * 2.f * ya * E;
    sW[r * 2 * F + F + f] = df * phi * (nc.c1[node] * kLn2);
  }
  __syncthreads();
  for (int p = threadIdx.x; p < nr * d; p += kBThreads) {
    const int r = p / d, c = p - (p / d) * d;
    float acc = 0.f;
    for (int f = 0; f < F; ++f) {
      acc = fmaf(sW[r * 2 * F + f], ld(A + (int64_t)f * d + c), acc);
      acc = fmaf(sW[r * 2 * F + F + f], ld(G + (int64_t)f * d + c), acc);
    }
    sD[p] = acc;
  }
  __syncthreads();
  for (int p = threadIdx.x; p < nr * d; p += kBThreads) {
    const int r = p / d;
    float proj = 0.f;
    if (!sclamp[r])
      for (int c = 0; c < d; ++c) proj = fmaf(sx[r * d + c], sD[r * d + c], proj);
    st<TI>(dx + r0 * d + p, (sD[p] - sx[p] * proj) * sinv[r]);
  }
}

struct WsLayout {
  float *phiq, *phik, *dphiq, *dphik, *gh, *states;
  size_t bytes;
};

WsLayout ws_layout(const BackwardArgs& a, void* base) {
  const int64_t nrow = a.n_heads * a.L;
  const int64_t n_chunks = (a.L + a.chunk - 1) / a.chunk;
  const int64_t E1 = a.dv + 1;
  const int64_t nf = nrow * a.F;
  WsLayout w{};
  float* p = static_cast<float*>(base);
  w.phiq = p;
  w.phik = p + nf;
  w.dphiq = p + 2 * nf;
  w.dphik = p + 3 * nf;
  w.gh = p + 4 * nf;
  w.states = w.gh + nrow * E1;
  w.bytes = sizeof(float) * (size_t)(4 * nf + nrow * E1 + a.n_heads * n_chunks * a.F * E1);
  return w;
}

size_t bwd_lds_bytes(const BackwardArgs& a) { return sizeof(float) * (size_t)(a.chunk * a.chunk + a.chunk * (a.dv + 1)); }

int vjp_rows(const BackwardArgs& a) {
  // rows per workgroup: LDS for 2F weights per row within 64 KiB; a divisor
  // of the per-head length when draw sets differ between heads
  int tr = 16;
  while (tr > 1 && sizeof(float) * (size_t)tr * (2 * a.F + 2 * a.d) > 65536) tr /= 2;
  if (a.n_draw_sets > 1)
    while (tr > 1 && a.L % tr != 0) tr /= 2;
  return tr;
}

template <typename TI>
hipError_t launch_vjp(const BackwardArgs& a, const TI* x, const float* dphi, TI* dx, hipStream_t s) {
  const int tr = vjp_rows(a);
  const int64_t n_rows = a.n_heads * a.L;
  const size_t lds = sizeof(float) * (size_t)tr * (2 * a.F + 2 * a.d);
  hipLaunchKernelGGL(fmvjp_kernel<TI>, dim3((unsigned)((n_rows + tr - 1) / tr)), dim3(kBThreads), lds, s, x, dphi,
                     a.L, n_rows, a.d, a.F, a.m, static_cast<const TI*>(a.anchors), static_cast<const TI*>(a.prf),
                     a.draw_set_stride, a.n_draw_sets, a.nc, tr, dx);
  return hipGetLastError();
}

template <typename TV>
hipError_t launch_backward_t(const BackwardArgs& a, hipStream_t s) {
  const WsLayout w = ws_layout(a, a.ws);
  const int64_t n_chunks = (a.L + a.chunk - 1) / a.chunk;

  FeatmapArgs fa{};
  fa.rows_per_head = a.L;
  fa.n_heads = a.n_heads;
  fa.d = a.d;
  fa.F = a.F;
  fa.m = a.m;
  fa.x_bf16 = a.io_bf16;
  fa.anchors = a.anchors;
  fa.prf = a.prf;
  fa.draw_set_stride = a.draw_set_stride;
  fa.n_draw_sets = a.n_draw_sets;
  fa.nc = a.nc;
  fa.phi_bf16 = false;
  fa.x = a.q;
  fa.phi = w.phiq;
  fa.x2 = a.k;
  fa.phi2 = w.phik;
  hipError_t e = launch_featmap(fa, s);
  if (e != hipSuccess) return e;
  e = launch_chunk_state(w.phik, a.v, a.io_bf16, a.n_heads, a.L, a.F, a.dv, a.chunk, n_chunks, w.states, s);
  if (e != hipSuccess) return e;

  ScanArgs sa{};
  sa.states = w.states;
  sa.n_heads = a.n_heads;
  sa.n_items = n_chunks;
  sa.n_terms = n_chunks;
  sa.F = a.F;
  sa.dv = a.dv;
  sa.layout = 0;
  sa.S0 = a.S0;
  sa.z0 = a.z0;
  e = launch_scan(sa, s);
  if (e != hipSuccess) return e;

  const size_t lds = bwd_lds_bytes(a);
  const dim3 grid((unsigned)n_chunks, (unsigned)a.n_heads);
  e = set_max_lds(reinterpret_cast<const void*>(&bwd_q_kernel<TV>), (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_q_kernel<TV>, grid, dim3(kBThreads), lds, s, w.phiq, w.phik, static_cast<const TV*>(a.v),
                     static_cast<const TV*>(a.dout), a.L, a.F, a.dv, a.chunk, n_chunks, w.states, w.gh, w.dphiq);
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  ScanArgs ra{};
  ra.states = w.states;
  ra.n_heads = a.n_heads;
  ra.n_items = n_chunks;
  ra.n_terms = n_chunks;
  ra.F = a.F;
  ra.dv = a.dv;
  ra.layout = 0;
  ra.S0 = a.dS_T;
  ra.z0 = a.dz_T;
  ra.S_out = a.dS0;
  ra.z_out = a.dz0;
  ra.reverse = true;
  e = launch_scan(ra, s);
  if (e != hipSuccess) return e;

  e = set_max_lds(reinterpret_cast<const void*>(&bwd_kv_kernel<TV>), (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_kv_kernel<TV>, grid, dim3(kBThreads), lds, s, w.phiq, w.phik, static_cast<const TV*>(a.v),
                     a.L, a.F, a.dv, a.chunk, n_chunks, w.states, w.gh, w.dphik, static_cast<TV*>(a.dv_out));
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  e = launch_vjp<TV>(a, static_cast<const TV*>(a.q), w.dphiq, static_cast<TV*>(a.dq), s);
  if (e != hipSuccess) return e;
  return launch_vjp<TV>(a, static_cast<const TV*>(a.k), w.dphik, static_cast<TV*>(a.dk), s);
}

}  // namespace

bool backward_supported(const BackwardArgs& a) {
  return featmap_supported(a.d) && a.F % 16 == 0 && a.m % 16 == 0 && a.chunk >= 1 && a.chunk <= 128 && a.dv >= 1 &&
         a.dv <= 256 && bwd_lds_bytes(a) <= 160 * 1024;
}

size_t backward_workspace_bytes(const BackwardArgs& a) {
  if (a.n_heads == 0 || a.L == 0) return 0;
  return ws_layout(a, nullptr).bytes;
}

hipError_t launch_backward(const BackwardArgs& a, hipStream_t s) {
  if (a.n_heads == 0) return hipSuccess;
  if (a.L == 0) {  // no tokens: the gradient of the initial state is that of the final one
    ScanArgs sa{};
    sa.n_heads = a.n_heads;
    sa.F = a.F;
    sa.dv = a.dv;
    sa.layout = 0;
    sa.S0 = a.dS_T;
    sa.z0 = a.dz_T;
    sa.S_out = a.dS0;
    sa.z_out = a.dz0;
    return (a.dS0 || a.dz0) ? launch_scan(sa, s) : hipSuccess;
  }
  return a.io_bf16 ? launch_backward_t<uint16_t>(a, s) : launch_backward_t<float>(a, s);
}

}  // namespace slay
