// slay_decode.hip -- O(1)-per-token recurrent SLAY step (decode).
//
// Method ("SLAY: Geometry-Aware Spherical Linearized Attention with
// Yat-Kernel", abstract; nubint.ai review, "Proposed method" bullets 3, 5, 6):
// for one new token per head, phi(q), phi(k) from the anchor x PRF feature map,
// then S += phi(k) v^T, z += phi(k), o = phi(q)^T S / phi(q)^T z (update
// first, so the new token attends to itself).
//
// The step is bound by HBM traffic on the fp32 state: per head it reads and
// writes S (F x dv) and z (F).  It runs as two launches on the caller's
// stream:
//   1. the feature-map kernel (slay_featmap.hip) maps the q rows and the k
//      rows of every head in one launch, fp32 out, into the workspace;
//   2. stream_kernel: one workgroup per head reads its state with contiguous
//      float4 accesses (a wave covers 1 KiB per instruction, all loads of a
//      thread issued before any use), applies the rank-1 update, writes it
//      back and forms the readout, reduced across threads in LDS.
// Keeping the projection out of the streaming kernel leaves that kernel with
// few registers, so many workgroups per CU keep enough loads in flight.
#include "slay_device.hpp"
#include "slay_internal.hpp"

namespace slay {

namespace {

constexpr int kST = 256;  // threads per streaming workgroup

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

// One head per workgroup.  The F x DV state is NV4 = DV/4 float4 columns
// wide; thread t owns column c4 = t % NV4 and rows t / NV4 + i * (kST / NV4).
template <int DV, typename TIO>
__global__ __launch_bounds__(kST) void stream_kernel(const float* __restrict__ phq, const float* __restrict__ phk,
                                                     const TIO* __restrict__ v, float* __restrict__ S,
                                                     float* __restrict__ z, TIO* __restrict__ o, int F) {
  constexpr int NV4 = DV / 4;
  constexpr int RG = kST / NV4;  // row groups (threads sharing a column)
  constexpr int NB = 16;         // float4 per thread per batch
  static_assert(kST % NV4 == 0, "DV/4 must divide the workgroup");
  __shared__ float sphq[1024], sphk[1024];
  __shared__ float4 sred[kST];
  __shared__ float sden[kST / 64];

  const int64_t h = blockIdx.x;
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int c4 = t % NV4, r0 = t / NV4;
  float* Sh = S + h * (int64_t)F * DV;
  const int rows_pt = F / RG;  // rows per thread (F is a multiple of RG)

  // phi(q), phi(k) of this head -> LDS; z update and denominator
  float den = 0.f;
  for (int f = t; f < F; f += kST) {
    const float kf = phk[h * F + f], qf = phq[h * F + f];
    sphk[f] = kf;
    sphq[f] = qf;
    const float zn = z[h * F + f] + kf;
    z[h * F + f] = zn;
    den = fmaf(qf, zn, den);
  }
  den = wave_sum(den);
  if (lane == 0) sden[wave] = den;
  float4 v4;
  v4.x = ld1<TIO>(v + h * DV + 4 * c4);
  v4.y = ld1<TIO>(v + h * DV + 4 * c4 + 1);
  v4.z = ld1<TIO>(v + h * DV + 4 * c4 + 2);
  v4.w = ld1<TIO>(v + h * DV + 4 * c4 + 3);

  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int i0 = 0; i0 < rows_pt; i0 += NB) {
    float4 sr[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i)
      if (i0 + i < rows_pt) sr[i] = *reinterpret_cast<const float4*>(Sh + (int64_t)(r0 + (i0 + i) * RG) * DV + 4 * c4);
    if (i0 == 0) __syncthreads();  // phi in LDS
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      if (i0 + i < rows_pt) {
        const int r = r0 + (i0 + i) * RG;
        const float kr = sphk[r], qr = sphq[r];
        float4 s = sr[i];
        s.x = fmaf(kr, v4.x, s.x);
        s.y = fmaf(kr, v4.y, s.y);
        s.z = fmaf(kr, v4.z, s.z);
        s.w = fmaf(kr, v4.w, s.w);
        *reinterpret_cast<float4*>(Sh + (int64_t)r * DV + 4 * c4) = s;
        acc.x = fmaf(qr, s.x, acc.x);
        acc.y = fmaf(qr, s.y, acc.y);
        acc.z = fmaf(qr, s.z, acc.z);
        acc.w = fmaf(qr, s.w, acc.w);
      }
    }
  }
  if (rows_pt == 0) __syncthreads();
  sred[t] = acc;
  __syncthreads();
  if (t < DV) {
    const int cc4 = t >> 2, cc = t & 3;
    float num = 0.f;
#pragma unroll 4
    for (int rg = 0; rg < RG; ++rg) {
      const float4 p = sred[rg * NV4 + cc4];
      num += (cc == 0) ? p.x : (cc == 1) ? p.y : (cc == 2) ? p.z : p.w;
    }
    float dsum = 0.f;
#pragma unroll
    for (int w = 0; w < kST / 64; ++w) dsum += sden[w];
    st1<TIO>(o + h * DV + t, num / dsum);
  }
}

template <int DV, typename TIO>
hipError_t launch_stream(const DecodeArgs& a, const float* phq, const float* phk, hipStream_t s) {
  hipLaunchKernelGGL((stream_kernel<DV, TIO>), dim3((unsigned)a.n_heads), dim3(kST), 0, s, phq, phk,
                     static_cast<const TIO*>(a.v), a.S, a.z, static_cast<TIO*>(a.o), a.F);
  return hipGetLastError();
}

template <typename TIO>
hipError_t launch_stream_dv(const DecodeArgs& a, const float* phq, const float* phk, hipStream_t s) {
  switch (a.dv) {
    case 16: return launch_stream<16, TIO>(a, phq, phk, s);
    case 32: return launch_stream<32, TIO>(a, phq, phk, s);
    case 64: return launch_stream<64, TIO>(a, phq, phk, s);
    case 128: return launch_stream<128, TIO>(a, phq, phk, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool decode_supported(const DecodeArgs& a) {
  const bool dvok = (a.dv == 16 || a.dv == 32 || a.dv == 64 || a.dv == 128);
  // rows of the state split evenly over the row groups of a workgroup
  const int rg = kST / (a.dv / 4);
  return featmap_supported(a.d) && dvok && a.F % 16 == 0 && a.F <= 1024 && a.F % rg == 0 &&
         a.draws_bf16 == a.io_bf16;
}

size_t decode_workspace_bytes(const DecodeArgs& a) { return sizeof(float) * 2 * (size_t)a.n_heads * a.F; }

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  if (a.n_heads == 0) return hipSuccess;
  float* phq = static_cast<float*>(a.ws);
  float* phk = phq + a.n_heads * (int64_t)a.F;
  FeatmapArgs fa{};
  fa.x = a.q;
  fa.x2 = a.k;
  fa.rows_per_head = 1;
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
  fa.phi = phq;
  fa.phi2 = phk;
  fa.phi_bf16 = false;
  if (a.n_draw_sets == 1) {  // one draw for all heads: map all rows as one block of rows
    fa.rows_per_head = a.n_heads;
    fa.n_heads = 1;
  }
  hipError_t e = launch_featmap(fa, s);
  if (e != hipSuccess) return e;
  return a.io_bf16 ? launch_stream_dv<uint16_t>(a, phq, phk, s) : launch_stream_dv<float>(a, phq, phk, s);
}

}  // namespace slay
