// slay_decode.hip -- O(1)-per-token recurrent SLAY step (decode).
//
// Method ("SLAY: Geometry-Aware Spherical Linearized Attention with
// Yat-Kernel", abstract; nubint.ai review, "Proposed method" bullets 3, 5, 6):
// for one new token per head, phi(q), phi(k) from the anchor x PRF feature map,
// then S += phi(k) v^T, z += phi(k), o = phi(q)^T S / phi(q)^T z (update
// first, so the new token attends to itself).
//
// The step is bound by HBM traffic on the fp32 state: per head it reads and
// writes S (F x dv) and z (F).  One workgroup of F threads serves a run of
// heads.  Thread f keeps the anchor and PRF rows of feature f in registers
// for the whole launch, so the projections of q and k cost 4d FMAs per thread
// and no draw traffic per head.  The state of a head is streamed with
// contiguous float4 accesses (a wave covers 1 KiB per instruction); its loads
// are issued before the feature map of that head so the FMAs hide their
// latency.  phi(q), phi(k) go through LDS; the readout phi(q)^T S is reduced
// in LDS across the threads that share an output column.
#include "slay_device.hpp"
#include "slay_internal.hpp"

namespace slay {

namespace {

template <typename T>
__device__ __forceinline__ float ld1(const T* p);
template <>
__device__ __forceinline__ float ld1<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float ld1<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }

template <typename T>
__device__ __forceinline__ void st1(T* p, float x);
template <>
__device__ __forceinline__ void st1<float>(float* p, float x) { *p = x; }
template <>
__device__ __forceinline__ void st1<uint16_t>(uint16_t* p, float x) { *p = f32_to_bf16(x); }

template <int D, int DV, typename TIO, typename TD>
__global__ __launch_bounds__(256) void decode_kernel(const TIO* __restrict__ q, const TIO* __restrict__ k,
                                                      const TIO* __restrict__ v, int64_t n_heads,
                                                      int heads_per_block, const TD* __restrict__ anchors,
                                                      const TD* __restrict__ prf, int64_t draw_set_stride,
                                                      int n_draw_sets, int F, int m, NodeConsts nc,
                                                      float* __restrict__ S, float* __restrict__ z,
                                                      TIO* __restrict__ o) {
  constexpr int NV4 = DV / 4;  // float4 columns of a state row
  __shared__ float sq[D], sk[D], sv[DV];
  __shared__ float sphq[256], sphk[256];
  __shared__ float4 sred[256];
  __shared__ float sden[4], snorm[2];

  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6, nwave = blockDim.x >> 6;
  const int f = t;  // feature owned for the feature map
  const int node = f / m;
  const float c1 = nc.c1[node], c0 = nc.c0[node];
  // streaming: F threads cover the F x DV/4 float4 grid of a head's state, so
  // each thread owns NV4 rows r0 + i * rstep of one float4 column e4
  const int e4 = t % NV4;
  const int r0 = t / NV4;
  const int rstep = F / NV4;

  float ar[D], gr[D];
  int cur_set = -1;

  const int64_t h0 = (int64_t)blockIdx.x * heads_per_block;
  const int64_t h1 = min<int64_t>(n_heads, h0 + heads_per_block);
  for (int64_t h = h0; h < h1; ++h) {
    const int set = (int)(h % n_draw_sets);
    if (set != cur_set) {
      cur_set = set;
      const TD* a = anchors + (int64_t)set * draw_set_stride + (int64_t)f * D;
      const TD* g = prf + (int64_t)set * draw_set_stride + (int64_t)f * D;
#pragma unroll
      for (int c = 0; c < D; ++c) {
        ar[c] = ld1<TD>(a + c);
        gr[c] = ld1<TD>(g + c);
      }
    }
    // issue the state loads of this head first
    float* Sh = S + h * (int64_t)F * DV;
    float4 sreg[NV4];
#pragma unroll
    for (int i = 0; i < NV4; ++i)
      sreg[i] = *reinterpret_cast<const float4*>(Sh + (int64_t)(r0 + i * rstep) * DV + 4 * e4);
    const float zf = z[h * F + f];

    // token inputs -> LDS, row norms
    float qq = 0.f, kk = 0.f;
    if (t < D) {
      const float qv = ld1<TIO>(q + h * D + t), kv = ld1<TIO>(k + h * D + t);
      sq[t] = qv;
      sk[t] = kv;
      qq = qv * qv;
      kk = kv * kv;
    }
    if (t < DV) sv[t] = ld1<TIO>(v + h * DV + t);
    if (wave == 0) {
      qq = wave_sum(qq);
      kk = wave_sum(kk);
      if (lane == 0) {
        snorm[0] = 1.0f / fmaxf(sqrtf(qq), 1e-12f);
        snorm[1] = 1.0f / fmaxf(sqrtf(kk), 1e-12f);
      }
    }
    __syncthreads();
    const float invq = snorm[0], invk = snorm[1];
    float yaq = 0.f, ygq = 0.f, yak = 0.f, ygk = 0.f;
#pragma unroll
    for (int c = 0; c < D; ++c) {
      const float qc = sq[c], kc = sk[c];
      yaq = fmaf(ar[c], qc, yaq);
      ygq = fmaf(gr[c], qc, ygq);
      yak = fmaf(ar[c], kc, yak);
      ygk = fmaf(gr[c], kc, ygk);
    }
    const float aq = yaq * invq, ak = yak * invk;
    const float phq = aq * aq * fast_exp2(fmaf(ygq, invq * c1, c0));
    const float phk = ak * ak * fast_exp2(fmaf(ygk, invk * c1, c0));
    sphq[f] = phq;
    sphk[f] = phk;
    const float znew = zf + phk;
    z[h * F + f] = znew;
    float den = wave_sum(phq * znew);
    if (lane == 0) sden[wave] = den;
    __syncthreads();

    // S += phi(k) v^T on the owned rows, readout phi(q)^T S_new
    const float4 v4 = make_float4(sv[4 * e4], sv[4 * e4 + 1], sv[4 * e4 + 2], sv[4 * e4 + 3]);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int i = 0; i < NV4; ++i) {
      const int r = r0 + i * rstep;
      const float kr = sphk[r], qr = sphq[r];
      float4 s = sreg[i];
      s.x = fmaf(kr, v4.x, s.x);
      s.y = fmaf(kr, v4.y, s.y);
      s.z = fmaf(kr, v4.z, s.z);
      s.w = fmaf(kr, v4.w, s.w);
      *reinterpret_cast<float4*>(Sh + (int64_t)r * DV + 4 * e4) = s;
      acc.x = fmaf(qr, s.x, acc.x);
      acc.y = fmaf(qr, s.y, acc.y);
      acc.z = fmaf(qr, s.z, acc.z);
      acc.w = fmaf(qr, s.w, acc.w);
    }
    sred[t] = acc;
    __syncthreads();
    if (t < DV) {
      float num = 0.f;
      const int c4 = t >> 2, cc = t & 3;
      for (int rr = 0; rr < rstep; ++rr) {
        const float4 p = sred[rr * NV4 + c4];
        num += (cc == 0) ? p.x : (cc == 1) ? p.y : (cc == 2) ? p.z : p.w;
      }
      float dsum = 0.f;
      for (int w = 0; w < nwave; ++w) dsum += sden[w];
      st1<TIO>(o + h * DV + t, num / dsum);
    }
    __syncthreads();
  }
}

template <int D, int DV, typename TIO, typename TD>
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t s) {
  const int hpb = 8;
  const int64_t blocks = (a.n_heads + hpb - 1) / hpb;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((decode_kernel<D, DV, TIO, TD>), dim3((unsigned)blocks), dim3(a.F), 0, s,
                     static_cast<const TIO*>(a.q), static_cast<const TIO*>(a.k), static_cast<const TIO*>(a.v),
                     a.n_heads, hpb, static_cast<const TD*>(a.anchors), static_cast<const TD*>(a.prf),
                     a.draw_set_stride, a.n_draw_sets, a.F, a.m, a.nc, a.S, a.z, static_cast<TIO*>(a.o));
  return hipGetLastError();
}

template <int D, int DV>
hipError_t launch_decode_dv(const DecodeArgs& a, hipStream_t s) {
  if (a.io_bf16)
    return a.draws_bf16 ? launch_decode_t<D, DV, uint16_t, uint16_t>(a, s)
                        : launch_decode_t<D, DV, uint16_t, float>(a, s);
  return a.draws_bf16 ? launch_decode_t<D, DV, float, uint16_t>(a, s) : launch_decode_t<D, DV, float, float>(a, s);
}

}  // namespace

bool decode_supported(const DecodeArgs& a) {
  const bool dok = (a.d == 32 || a.d == 64);
  const bool dvok = (a.dv == 32 || a.dv == 64);
  // one thread per feature (F <= 256); the F x dv/4 float4 grid of a state
  // must split into whole rows per thread
  return dok && dvok && a.F >= 64 && a.F <= 256 && a.F % 64 == 0 && a.m >= 1 && (a.F % (a.dv / 4)) == 0;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  if (a.d == 64) return a.dv == 64 ? launch_decode_dv<64, 64>(a, s) : launch_decode_dv<64, 32>(a, s);
  return a.dv == 64 ? launch_decode_dv<32, 64>(a, s) : launch_decode_dv<32, 32>(a, s);
}

}  // namespace slay
