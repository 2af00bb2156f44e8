// slay_chunked_generic.hip -- the general causal SLAY forward (any dtype and
// shape the ABI accepts) and the inter-chunk prefix scan of (S, z).
//
// Method ("SLAY: Geometry-Aware Spherical Linearized Attention with
// Yat-Kernel", abstract; nubint.ai review, "Proposed method" bullet 6):
// o_i = phi(q_i)^T S_i / phi(q_i)^T z_i with S_i = sum_{j<=i} phi(k_j) v_j^T,
// z_i = sum_{j<=i} phi(k_j), evaluated chunk by chunk without the L x L
// matrix: a masked C x C block inside each chunk plus the state carried in
// from the chunks before it.
//
// This path is unfused and uses plain fp32 FMA for the contractions:
//   1. the feature-map kernel writes fp32 phi(q), phi(k) to the workspace;
//   2. chunk_state: per (head, chunk) dS_c = phi(k_c)^T [v_c | 1];
//   3. scan: exclusive prefix of dS over chunks (plus S0), total -> S_out;
//   4. chunk_out: per (head, chunk) masked intra block + phi(q) S_c, divide.
// It serves fp32 callers (1e-4 parity) and shapes without a fused MFMA
// variant; the bf16 headline shapes take slay_chunked_fused.hip.
#include "slay_device.hpp"
#include "slay_internal.hpp"

namespace slay {

namespace {

constexpr int kGThreads = 256;

__device__ __forceinline__ void scan_map(int64_t idx, int F, int dv, int layout, int& f, int& e) {
  if (layout == 0) {
    f = (int)(idx / (dv + 1));
    e = (int)(idx - (int64_t)f * (dv + 1));
  } else {
    const int NE = (dv + 16) / 16;
    const int i = (int)(idx & 3);
    const int lane = (int)((idx >> 2) & 63);
    const int64_t tile = idx >> 8;
    const int et = (int)(tile % NE);
    const int fb = (int)(tile / NE);
    f = fb * 16 + 4 * (lane >> 4) + i;
    e = et * 16 + (lane & 15);
  }
}

// In-place exclusive prefix over items: item i <- init + sum_{i' < i} delta_i'
// (or, reversed, the exclusive suffix init + sum_{i' > i} delta_i').
__global__ __launch_bounds__(kGThreads) void scan_kernel(ScanArgs a, int64_t E) {
  const int64_t h = blockIdx.y;
  const int64_t idx = (int64_t)blockIdx.x * kGThreads + threadIdx.x;
  if (idx >= E) return;
  int f, e;
  scan_map(idx, a.F, a.dv, a.layout, f, e);
  // a reverse scan walks the items from the last one: item i at st[(n_items - 1 - i) * step]
  const int64_t step = a.reverse ? -E : E;
  float* st = a.states + h * a.n_items * E + idx + (a.reverse ? (a.n_items - 1) * E : 0);
  if (e > a.dv) {
    // padding column of the fragment layout: zero in every delta item, so every
    // prefix is zero too; only the items no delta was written to are stored
    for (int64_t i = a.n_terms; i < a.n_items; ++i) st[i * step] = 0.f;
    return;
  }
  float run = 0.f;
  if (e < a.dv) {
    if (a.S0) run = a.S0[(h * a.F + f) * a.dv + e];
  } else if (e == a.dv) {
    if (a.z0) run = a.z0[h * a.F + f];
  }
  // loads of a batch of items are issued together, then the running sums stored
  constexpr int kBatch = 16;
  for (int64_t i0 = 0; i0 < a.n_items; i0 += kBatch) {
    float d[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) d[b] = (i0 + b < a.n_terms) ? st[(i0 + b) * step] : 0.f;
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      if (i0 + b < a.n_items && (!a.total_only || i0 + b == a.n_items - 1)) st[(i0 + b) * step] = run;
      run += d[b];
    }
  }
  if (e < a.dv) {
    if (a.S_out) a.S_out[(h * a.F + f) * a.dv + e] = run;
  } else if (e == a.dv) {
    if (a.z_out) a.z_out[h * a.F + f] = run;
  }
}

// Initial value of state elements (f + i, e), i < 4: S0 / z0 of row `sh`, or 0.
__device__ __forceinline__ float4 scan_init4(const float* S0, const float* z0, int64_t sh, int F, int dv, int f,
                                             int e) {
  float r[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (e < dv) {
      if (S0) r[i] = S0[(sh * F + f + i) * dv + e];
    } else if (z0) {
      r[i] = z0[sh * F + f + i];
    }
  }
  return make_float4(r[0], r[1], r[2], r[3]);
}

__device__ __forceinline__ void scan_out4(float* S_out, float* z_out, int64_t sh, int F, int dv, int f, int e,
                                          float4 v) {
  const float r[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (e < dv) {
      if (S_out) S_out[(sh * F + f + i) * dv + e] = r[i];
    } else if (z_out) {
      z_out[sh * F + f + i] = r[i];
    }
  }
}

__device__ __forceinline__ float4 add4(float4 a, float4 b) {
  return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}

// scan_kernel for the fragment layout, one 16-byte vector per thread: the four
// elements of a vector share the column e (features f .. f+3), so a vector is
// either all padding or all state.
__global__ __launch_bounds__(kGThreads) void scan4_kernel(ScanArgs a, int64_t E) {
  const int64_t h = blockIdx.y;
  const int64_t idx = ((int64_t)blockIdx.x * kGThreads + threadIdx.x) * 4;
  if (idx >= E) return;
  int f, e;
  scan_map(idx, a.F, a.dv, 1, f, e);
  const int64_t step = a.reverse ? -E : E;
  float4* st = reinterpret_cast<float4*>(a.states + h * a.n_items * E + idx + (a.reverse ? (a.n_items - 1) * E : 0));
  const int64_t step4 = step / 4;
  if (e > a.dv) {  // padding column: zero prefixes, stored only where no delta was written
    for (int64_t i = a.n_terms; i < a.n_items; ++i) st[i * step4] = make_float4(0.f, 0.f, 0.f, 0.f);
    return;
  }
  float4 run = scan_init4(a.S0, a.z0, h, a.F, a.dv, f, e);
  constexpr int kBatch = 16;
  for (int64_t i0 = 0; i0 < a.n_items; i0 += kBatch) {
    float4 d[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b)
      d[b] = (i0 + b < a.n_terms) ? st[(i0 + b) * step4] : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      if (i0 + b < a.n_items && (!a.total_only || i0 + b == a.n_items - 1)) st[(i0 + b) * step4] = run;
      run = add4(run, d[b]);
    }
  }
  scan_out4(a.S_out, a.z_out, h, a.F, a.dv, f, e, run);
}

// dS_c[f][e] = sum_{j in chunk} phik[j][f] * vx[j][e], with vx = [v | 1].
// Each thread owns a 4 (f) x 4 (e) block of the (F, dv+1) state.
template <typename TV>
__global__ __launch_bounds__(kGThreads) void chunk_state_kernel(const float* __restrict__ phik,
                                                                const TV* __restrict__ v, int64_t L,
                                                                int F, int dv, int C, int64_t n_chunks,
                                                                float* __restrict__ states) {
  const int64_t h = blockIdx.y;
  const int64_t c = blockIdx.x;
  const int64_t j0 = c * C;
  const int nj = (int)min<int64_t>(C, L - j0);
  const int E1 = dv + 1;
  const int nfb = (F + 3) / 4, neb = (E1 + 3) / 4;
  const float* pk = phik + (h * L + j0) * F;
  const TV* vv = v + (h * L + j0) * dv;
  float* out = states + (h * n_chunks + c) * (int64_t)F * E1;
  for (int blk = threadIdx.x; blk < nfb * neb; blk += kGThreads) {
    const int f0 = (blk / neb) * 4, e0 = (blk % neb) * 4;
    float acc[4][4] = {};
    for (int j = 0; j < nj; ++j) {
      float kf[4], ve[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) kf[a] = (f0 + a < F) ? pk[(int64_t)j * F + f0 + a] : 0.f;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int e = e0 + b;
        ve[b] = (e < dv) ? Mma<TV>::to_f32(vv[(int64_t)j * dv + e]) : (e == dv ? 1.f : 0.f);
      }
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = fmaf(kf[a], ve[b], acc[a][b]);
    }
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b)
        if (f0 + a < F && e0 + b < E1) out[(int64_t)(f0 + a) * E1 + e0 + b] = acc[a][b];
  }
}

template <typename TV>
__device__ __forceinline__ void store_out(TV* p, float x);
template <>
__device__ __forceinline__ void store_out<float>(float* p, float x) { *p = x; }
template <>
__device__ __forceinline__ void store_out<uint16_t>(uint16_t* p, float x) { *p = f32_to_bf16(x); }

// o_i = (sum_{j<=i in chunk} A_ij v_j + phiq_i S_c) / (sum_j A_ij + phiq_i z_c),
// A_ij = phiq_i . phik_j.  The masked block A lives in LDS (C <= 128).
template <typename TV>
__global__ __launch_bounds__(kGThreads) void chunk_out_kernel(const float* __restrict__ phiq,
                                                              const float* __restrict__ phik,
                                                              const TV* __restrict__ v, int64_t L, int F,
                                                              int dv, int C, int64_t n_chunks,
                                                              const float* __restrict__ states,
                                                              TV* __restrict__ o) {
  extern __shared__ float sA[];  // [C][C]
  const int64_t h = blockIdx.y;
  const int64_t c = blockIdx.x;
  const int64_t i0 = c * C;
  const int n = (int)min<int64_t>(C, L - i0);
  const int E1 = dv + 1;
  const float* pq = phiq + (h * L + i0) * F;
  const float* pk = phik + (h * L + i0) * F;
  const TV* vv = v + (h * L + i0) * dv;
  const float* S = states + (h * n_chunks + c) * (int64_t)F * E1;
  for (int p = threadIdx.x; p < n * n; p += kGThreads) {
    const int i = p / n, j = p - (p / n) * n;
    float acc = 0.f;
    if (j <= i)
      for (int f = 0; f < F; ++f) acc = fmaf(pq[(int64_t)i * F + f], pk[(int64_t)j * F + f], acc);
    sA[i * C + j] = acc;
  }
  __syncthreads();
  for (int p = threadIdx.x; p < n * dv; p += kGThreads) {
    const int i = p / dv, e = p - (p / dv) * dv;
    float num = 0.f, den = 0.f;
    for (int j = 0; j <= i; ++j) {
      const float a = sA[i * C + j];
      num = fmaf(a, Mma<TV>::to_f32(vv[(int64_t)j * dv + e]), num);
      den += a;
    }
    for (int f = 0; f < F; ++f) {
      const float qf = pq[(int64_t)i * F + f];
      num = fmaf(qf, S[(int64_t)f * E1 + e], num);
      den = fmaf(qf, S[(int64_t)f * E1 + dv], den);
    }
    store_out<TV>(o + (h * L + i0 + i) * dv + e, num / den);
  }
}

template <typename TV>
hipError_t launch_generic_t(const ChunkedArgs& a, hipStream_t s) {
  const int64_t nrow = a.n_heads * a.L;
  const int64_t n_chunks = (a.L + a.chunk - 1) / a.chunk;
  float* phiq = static_cast<float*>(a.ws);
  float* phik = phiq + nrow * a.F;
  float* states = phik + nrow * a.F;

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
  fa.phi = phiq;
  hipError_t e = launch_featmap(fa, s);
  if (e != hipSuccess) return e;
  fa.x = a.k;
  fa.phi = phik;
  e = launch_featmap(fa, s);
  if (e != hipSuccess) return e;

  dim3 grid((unsigned)n_chunks, (unsigned)a.n_heads);
  hipLaunchKernelGGL(chunk_state_kernel<TV>, grid, dim3(kGThreads), 0, s, phik,
                     static_cast<const TV*>(a.v), a.L, a.F, a.dv, a.chunk, n_chunks, states);
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  ScanArgs sa{};
  sa.states = states;
  sa.n_heads = a.n_heads;
  sa.n_items = n_chunks;
  sa.n_terms = n_chunks;
  sa.F = a.F;
  sa.dv = a.dv;
  sa.layout = 0;
  sa.S0 = a.S0;
  sa.z0 = a.z0;
  sa.S_out = a.S_out;
  sa.z_out = a.z_out;
  e = launch_scan(sa, s);
  if (e != hipSuccess) return e;

  const size_t lds = sizeof(float) * (size_t)a.chunk * a.chunk;
  hipLaunchKernelGGL(chunk_out_kernel<TV>, grid, dim3(kGThreads), lds, s, phiq, phik,
                     static_cast<const TV*>(a.v), a.L, a.F, a.dv, a.chunk, n_chunks, states,
                     static_cast<TV*>(a.o));
  return hipGetLastError();
}

// Non-causal output: o_i = phi(q_i)^T S / phi(q_i)^T z with the state of all
// keys (S in columns 0..dv-1, z in column dv of the [F][dv+1] layout).
template <typename TV>
__global__ __launch_bounds__(kGThreads) void nc_out_kernel(const float* __restrict__ phiq, int64_t Lq, int F, int dv,
                                                           const float* __restrict__ S, int64_t state_stride,
                                                           TV* __restrict__ o) {
  const int64_t h = blockIdx.y;
  const int64_t i0 = (int64_t)blockIdx.x * 64;
  const int n = (int)min<int64_t>(64, Lq - i0);
  const int E1 = dv + 1;
  const float* pq = phiq + (h * Lq + i0) * F;
  const float* Sh = S + h * state_stride;
  for (int p = threadIdx.x; p < n * dv; p += kGThreads) {
    const int i = p / dv, e = p - (p / dv) * dv;
    float num = 0.f, den = 0.f;
    for (int f = 0; f < F; ++f) {
      const float qf = pq[(int64_t)i * F + f];
      num = fmaf(qf, Sh[(int64_t)f * E1 + e], num);
      den = fmaf(qf, Sh[(int64_t)f * E1 + dv], den);
    }
    store_out<TV>(o + (h * Lq + i0 + i) * dv + e, num / den);
  }
}

// Non-causal general path: phi(q), phi(k) to the workspace, per-chunk states
// of the keys, scan to the total (item n_chunks, S0/z0 included), readout.
template <typename TV>
hipError_t launch_generic_nc_t(const ChunkedArgs& a, hipStream_t s) {
  const int64_t n_chunks = (a.L + a.chunk - 1) / a.chunk;
  float* phiq = static_cast<float*>(a.ws);
  float* phik = phiq + a.n_heads * a.Lq * a.F;
  float* states = phik + a.n_heads * a.L * a.F;

  FeatmapArgs fa{};
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
  hipError_t e;
  if (a.Lq > 0) {
    fa.rows_per_head = a.Lq;
    fa.x = a.q;
    fa.phi = phiq;
    e = launch_featmap(fa, s);
    if (e != hipSuccess) return e;
  }
  if (a.L > 0) {
    fa.rows_per_head = a.L;
    fa.x = a.k;
    fa.phi = phik;
    e = launch_featmap(fa, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(chunk_state_kernel<TV>, dim3((unsigned)n_chunks, (unsigned)a.n_heads), dim3(kGThreads), 0, s,
                       phik, static_cast<const TV*>(a.v), a.L, a.F, a.dv, a.chunk, n_chunks + 1, states);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  ScanArgs sa{};
  sa.states = states;
  sa.n_heads = a.n_heads;
  sa.n_items = n_chunks + 1;
  sa.n_terms = n_chunks;
  sa.F = a.F;
  sa.dv = a.dv;
  sa.layout = 0;
  sa.S0 = a.S0;
  sa.z0 = a.z0;
  sa.S_out = a.S_out;
  sa.z_out = a.z_out;
  e = launch_scan(sa, s);
  if (e != hipSuccess) return e;
  if (a.Lq == 0) return hipSuccess;
  const int64_t E = (int64_t)a.F * (a.dv + 1);
  hipLaunchKernelGGL(nc_out_kernel<TV>, dim3((unsigned)((a.Lq + 63) / 64), (unsigned)a.n_heads), dim3(kGThreads), 0, s,
                     phiq, a.Lq, a.F, a.dv, states + n_chunks * E, (n_chunks + 1) * E, static_cast<TV*>(a.o));
  return hipGetLastError();
}

}  // namespace

// Variable-length batches: per (sequence s, head h) and state element, the
// exclusive prefixes from S0 of (s, h) over the state slots of the sequence's
// pieces of head h, in order: n_a[s] whole segments from slot first[s] on,
// whose deltas the segment-state pass wrote, then the slot of its last piece
// last[s] (-1 for an empty sequence), which gets its prefix and contributes
// no delta.  The main pass writes the final state of every non-empty
// sequence; here only an empty one's (S0) goes to S_out.  States are fragment
// ordered (layout 1); S0/S_out are [n_seqs][H][F][dv].  One 16-byte vector
// (features f .. f+3 of one column) per thread; the padding columns are zero
// in every delta, and so in every prefix.
__global__ __launch_bounds__(kGThreads) void vl_scan_kernel(float* states, int64_t H, int g_max, const int* first,
                                                            const int* n_a, const int* last, int F, int dv,
                                                            const float* S0, const float* z0, float* S_out,
                                                            float* z_out, int64_t E) {
  const int64_t sh = blockIdx.y;  // s * H + h
  const int64_t h = sh % H, sq = sh / H;
  const int64_t idx = ((int64_t)blockIdx.x * kGThreads + threadIdx.x) * 4;
  if (idx >= E) return;
  int f, e;
  scan_map(idx, F, dv, 1, f, e);
  if (e > dv) return;
  float4 run = scan_init4(S0, z0, sh, F, dv, f, e);
  float4* base = reinterpret_cast<float4*>(states + h * g_max * E + idx);
  const int64_t E4 = E / 4;
  const int n = n_a[sq], i0 = first[sq], t = last[sq];
  if (t < 0) {  // empty sequence: the state passes through
    scan_out4(S_out, z_out, sh, F, dv, f, e, run);
    return;
  }
  // the loads of a batch of deltas are issued together, then the prefixes stored
  constexpr int kBatch = 8;
  for (int j0 = 0; j0 < n; j0 += kBatch) {
    float4 d[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) d[b] = j0 + b < n ? base[(int64_t)(i0 + j0 + b) * E4] : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      if (j0 + b < n) base[(int64_t)(i0 + j0 + b) * E4] = run;
      run = add4(run, d[b]);
    }
  }
  base[(int64_t)t * E4] = run;
}

hipError_t launch_chunk_state(const float* phik, const void* v, bool v_bf16, int64_t n_heads, int64_t L, int F,
                              int dv, int C, int64_t item_stride, float* states, hipStream_t s) {
  const int64_t n_chunks = (L + C - 1) / C;
  if (n_heads == 0 || n_chunks == 0) return hipSuccess;
  const dim3 grid((unsigned)n_chunks, (unsigned)n_heads);
  if (v_bf16)
    hipLaunchKernelGGL(chunk_state_kernel<uint16_t>, grid, dim3(kGThreads), 0, s, phik,
                       static_cast<const uint16_t*>(v), L, F, dv, C, item_stride, states);
  else
    hipLaunchKernelGGL(chunk_state_kernel<float>, grid, dim3(kGThreads), 0, s, phik, static_cast<const float*>(v),
                       L, F, dv, C, item_stride, states);
  return hipGetLastError();
}

hipError_t launch_scan_varlen(float* states, int64_t H, int n_seqs, int g_max, const int* first, const int* n_a,
                              const int* last, int F, int dv, const float* S0, const float* z0, float* S_out,
                              float* z_out, hipStream_t s) {
  const int64_t E = scan_state_elems(F, dv, 1);
  if (H == 0 || n_seqs == 0) return hipSuccess;
  hipLaunchKernelGGL(vl_scan_kernel, dim3((unsigned)((E / 4 + kGThreads - 1) / kGThreads), (unsigned)(H * n_seqs)),
                     dim3(kGThreads), 0, s, states, H, g_max, first, n_a, last, F, dv, S0, z0, S_out, z_out, E);
  return hipGetLastError();
}

int64_t scan_state_elems(int F, int dv, int layout) {
  return layout == 0 ? (int64_t)F * (dv + 1) : (int64_t)F * (dv + 16);
}

hipError_t launch_scan(const ScanArgs& a, hipStream_t s) {
  const int64_t E = scan_state_elems(a.F, a.dv, a.layout);
  if (a.n_heads == 0 || E == 0) return hipSuccess;
  if (a.layout == 1) {  // E = F (dv + 16) is a multiple of 64: whole 16-byte vectors
    dim3 grid((unsigned)((E / 4 + kGThreads - 1) / kGThreads), (unsigned)a.n_heads);
    hipLaunchKernelGGL(scan4_kernel, grid, dim3(kGThreads), 0, s, a, E);
    return hipGetLastError();
  }
  dim3 grid((unsigned)((E + kGThreads - 1) / kGThreads), (unsigned)a.n_heads);
  hipLaunchKernelGGL(scan_kernel, grid, dim3(kGThreads), 0, s, a, E);
  return hipGetLastError();
}

namespace {

// dst[b][r][:] = src[b][r][:] for r < rows_src and 0 for rows_src <= r < rows_dst.
template <typename T>
__global__ __launch_bounds__(256) void pad_rows_kernel(T* __restrict__ dst, const T* __restrict__ src,
                                                       int64_t n_blocks, int64_t rows_src, int64_t rows_dst,
                                                       int64_t row_elems, int64_t src_stride, int64_t dst_stride) {
  const int64_t per = rows_dst * row_elems;
  const int64_t total = n_blocks * per;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t b = i / per, rem = i - b * per, r = rem / row_elems, e = rem - r * row_elems;
    dst[b * dst_stride + r * row_elems + e] = r < rows_src ? src[b * src_stride + r * row_elems + e] : T(0);
  }
}

template <typename T>
hipError_t pad_rows_t(T* dst, const T* src, int64_t n_blocks, int64_t rows_src, int64_t rows_dst, int64_t row_elems,
                      int64_t src_stride, int64_t dst_stride, hipStream_t s) {
  const int64_t total = n_blocks * rows_dst * row_elems;
  if (total == 0) return hipSuccess;
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(pad_rows_kernel<T>, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, s, dst, src,
                     n_blocks, rows_src, rows_dst, row_elems, src_stride, dst_stride);
  return hipGetLastError();
}

}  // namespace

hipError_t pad_rows(uint16_t* dst, const uint16_t* src, int64_t n_blocks, int64_t rows_src, int64_t rows_dst,
                    int64_t row_elems, int64_t src_stride, int64_t dst_stride, hipStream_t s) {
  return pad_rows_t(dst, src, n_blocks, rows_src, rows_dst, row_elems, src_stride, dst_stride, s);
}

hipError_t pad_rows(float* dst, const float* src, int64_t n_blocks, int64_t rows_src, int64_t rows_dst,
                    int64_t row_elems, int64_t src_stride, int64_t dst_stride, hipStream_t s) {
  return pad_rows_t(dst, src, n_blocks, rows_src, rows_dst, row_elems, src_stride, dst_stride, s);
}

bool generic_supported(const ChunkedArgs& a) {
  return featmap_supported(a.d) && a.F % 16 == 0 && a.m % 16 == 0 && a.chunk >= 1 && a.chunk <= 128 &&
         a.dv >= 1 && a.dv <= 1024;
}

size_t generic_workspace_bytes(const ChunkedArgs& a) {
  const int64_t n_chunks = (a.L + a.chunk - 1) / a.chunk;
  if (!a.causal)  // phi(q), phi(k), per-chunk states and their total
    return sizeof(float) * (size_t)((a.n_heads * (a.Lq + a.L)) * a.F +
                                    a.n_heads * (n_chunks + 1) * (int64_t)a.F * (a.dv + 1));
  const int64_t nrow = a.n_heads * a.L;
  return sizeof(float) * (size_t)(2 * nrow * a.F + a.n_heads * n_chunks * (int64_t)a.F * (a.dv + 1));
}

hipError_t launch_generic(const ChunkedArgs& a, hipStream_t s) {
  if (!a.causal) {
    if (a.n_heads == 0) return hipSuccess;
    return a.io_bf16 ? launch_generic_nc_t<uint16_t>(a, s) : launch_generic_nc_t<float>(a, s);
  }
  if (a.n_heads == 0 || a.L == 0) {
    // no tokens: the final state is the initial one
    ScanArgs sa{};
    sa.states = nullptr;
    sa.n_heads = a.n_heads;
    sa.n_items = 0;
    sa.n_terms = 0;
    sa.F = a.F;
    sa.dv = a.dv;
    sa.layout = 0;
    sa.S0 = a.S0;
    sa.z0 = a.z0;
    sa.S_out = a.S_out;
    sa.z_out = a.z_out;
    return (a.S_out || a.z_out) ? launch_scan(sa, s) : hipSuccess;
  }
  return a.io_bf16 ? launch_generic_t<uint16_t>(a, s) : launch_generic_t<float>(a, s);
}

}  // namespace slay
