// slay_chunked_fused.hip -- causal SLAY forward with the feature map fused
// into the chunked linear-attention contraction (bf16 in / fp32 accumulate /
// bf16 out) on gfx950 MFMA.
//
// Method ("SLAY: Geometry-Aware Spherical Linearized Attention with
// Yat-Kernel", abstract; nubint.ai review, "Proposed method" bullets 1, 3, 5,
// 6): o_i = phi(q_i)^T S_i / phi(q_i)^T z_i, S_i = sum_{j<=i} phi(k_j) v_j^T,
// z_i = sum_{j<=i} phi(k_j), computed without the L x L matrix.
//
// Work split.  Each head's sequence is cut into n_seg segments of whole
// chunks; one workgroup owns one (head, segment).
//   pass 1 (segments 0..n_seg-2): recompute phi(k) and sum the segment's
//           state delta dS = sum_j phi(k_j) [v_j | 1]^T into the workspace;
//   scan   : exclusive prefix of the deltas per head (plus S0), in place;
//   pass 2 : walk the segment's chunks in order, carrying the state on chip.
// The state is kept as S' = [S | z | 0..0], F x (dv+16): column dv holds z,
// so appending a ones column to v (v' = [v | 1 | 0]) makes every contraction
// with v' produce the numerator and the denominator together.
//
// Inside a workgroup (NW waves): wave w owns FBW blocks of 16 features.  It
// keeps its slice of P = [anchors | prf] in registers as MFMA operands and
// its F-slice of S' as fp32 accumulators for the whole segment.  Per chunk
// of C tokens:
//   stage    q, k tiles -> LDS (padded rows) with 1/|x| per row; v -> v'^T in LDS
//   phase A  (all waves, own features)  phi(k): projection with tokens as the
//            MFMA M dimension, so each lane's accumulator holds 4 consecutive
//            tokens of one feature -- exactly the A-operand of the state
//            update, kept in registers; also written to LDS as phi(k)[j][f].
//            phi(q): projection with features as M, written to LDS as
//            phi(q)[i][f] with 8-byte stores.
//   phase B1 intra(ib): A^T = phi(k) phi(q)^T on the causal 16x16 blocks of
//            query block ib, masked, rounded to bf16 and used in registers as
//            the B-operand of num'^T += v'^T A^T;  inter(ib): num'^T +=
//            S'^T phi(q)^T from the bf16 copy of S'^T in LDS.  Separate waves
//            when there are enough, combined through LDS.
//   phase B2 o = num / den (den is row dv of num'^T), 8-byte stores; each
//            wave adds phi(k)^T v' to its S' slice and refreshes its rows of
//            the bf16 S'^T copy for the next chunk.
// The contraction over tokens uses a fixed permutation of the 32 tokens of
// an MFMA k-step (lane group g holds tokens 4g..4g+3 and 16+4g..16+4g+3) on
// both operands, which leaves the sum unchanged and lets accumulators feed
// the next MFMA without a transpose.
#include "slay_device.hpp"
#include "slay_internal.hpp"

namespace slay {

namespace {

constexpr uint16_t kBf16One = 0x3F80;

template <int D_, int DV_, int C_, int NW_, int FBW_>
struct Cfg {
  static constexpr int D = D_, DV = DV_, C = C_, NW = NW_, FBW = FBW_;
  static constexpr int F = NW * FBW * 16;
  static constexpr int NT = NW * 64;       // threads
  static constexpr int NTB = C / 16;       // 16-token blocks per chunk
  static constexpr int NKS = D / 32;       // projection k-steps
  static constexpr int DVP = DV + 16;      // state columns (v | 1 | pad)
  static constexpr int NE = DVP / 16;      // 16-column tiles of the state
  static constexpr int NFK = F / 32;       // k-steps over features
  static constexpr int NTS = C / 32;       // k-steps over tokens
  static constexpr int LDX = D + 8;        // padded row strides (elements)
  static constexpr int LDV = C + 8;
  static constexpr int LDF = F + 8;
  static constexpr int NINTER = (NW - NTB) < NTB ? (NW - NTB) : NTB;  // inter tasks on their own wave
  static_assert(C % 32 == 0 && D % 32 == 0 && DV % 16 == 0, "tile sizes");
  static_assert(NW >= NTB, "one intra task per wave at most");
  // LDS (bytes)
  static constexpr int kQ = 0;
  static constexpr int kK = kQ + C * LDX * 2;
  static constexpr int kV = kK + C * LDX * 2;
  static constexpr int kPq = kV + DVP * LDV * 2;
  static constexpr int kPk = kPq + C * LDF * 2;
  static constexpr int kSt = kPk + C * LDF * 2;
  static constexpr int kX = kSt + DVP * LDF * 2;
  static constexpr int kInv = kX + (NINTER > 0 ? NINTER : 1) * NE * 64 * 16;
  static constexpr int kLds = kInv + 2 * C * 4;
  static constexpr int kLds1 = kV + DVP * LDV * 2 + 2 * C * 4;  // pass 1 footprint (K and v' only)
  static_assert(kLds <= 160 * 1024, "LDS budget");
};

struct Params {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  int64_t L;
  int64_t seg_len;  // tokens per segment (multiple of C)
  int n_seg;
  int m;
  const uint16_t* anchors;
  const uint16_t* prf;
  int64_t draw_set_stride;
  int n_draw_sets;
  NodeConsts nc;
  float* ws;         // [n_heads][n_seg][F/16][NE][64][4] fragment-ordered states
  const float* S0;   // used when there is a single segment
  const float* z0;
  float* S_out;
  float* z_out;
};

__device__ __forceinline__ uint2 pack4(float a, float b, float c, float d) {
  uint2 r;
  r.x = pack_bf16x2(a, b);
  r.y = pack_bf16x2(c, d);
  return r;
}

// Load this wave's slice of P as MFMA operands and its node constants.
template <class K>
__device__ __forceinline__ void load_p(const Params& p, int set, int wave, int lane, bf16x8 (&pa)[K::FBW][K::NKS],
                                       bf16x8 (&pg)[K::FBW][K::NKS], float (&c1)[K::FBW], float (&c0)[K::FBW]) {
  const int g = lane >> 4, col = lane & 15;
  const uint16_t* a = p.anchors + (int64_t)set * p.draw_set_stride;
  const uint16_t* gg = p.prf + (int64_t)set * p.draw_set_stride;
#pragma unroll
  for (int j = 0; j < K::FBW; ++j) {
    const int fb = wave * K::FBW + j;
    const int64_t off = (int64_t)(fb * 16 + col) * K::D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < K::NKS; ++ks) {
      pa[j][ks] = as_bf16x8(*reinterpret_cast<const uint4*>(a + off + ks * 32));
      pg[j][ks] = as_bf16x8(*reinterpret_cast<const uint4*>(gg + off + ks * 32));
    }
    const int node = (fb * 16) / p.m;
    c1[j] = p.nc.c1[node];
    c0[j] = p.nc.c0[node];
  }
}

// Stage a tile of C rows of x (bf16 [.][D]) into LDS; rows >= n are zero.
// Writes 1/max(|x|, 1e-12) per row to sinv.
template <class K>
__device__ __forceinline__ void stage_x(const uint16_t* __restrict__ x, int n, uint16_t* sx, float* sinv) {
  constexpr int VPR = K::D / 8;  // 16-byte vectors per row
  static_assert((K::NT % VPR) == 0, "rows must not straddle threads groups");
  for (int v = threadIdx.x; v < K::C * VPR; v += K::NT) {
    const int r = v / VPR, c = (v % VPR) * 8;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (r < n) val = *reinterpret_cast<const uint4*>(x + (int64_t)r * K::D + c);
    *reinterpret_cast<uint4*>(sx + r * K::LDX + c) = val;
    const uint32_t w[4] = {val.x, val.y, val.z, val.w};
    float ss = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float lo = __uint_as_float(w[q] << 16), hi = __uint_as_float(w[q] & 0xFFFF0000u);
      ss = fmaf(lo, lo, ss);
      ss = fmaf(hi, hi, ss);
    }
#pragma unroll
    for (int o = 1; o < VPR; o <<= 1) ss += __shfl_xor(ss, o, 64);
    if ((v % VPR) == 0) sinv[r] = 1.0f / fmaxf(sqrtf(ss), 1e-12f);
  }
}

// Stage v (bf16 [.][DV]) transposed into v'^T rows 0..DV-1; tokens >= n are zero.
template <class K>
__device__ __forceinline__ void stage_v(const uint16_t* __restrict__ v, int n, uint16_t* sv) {
  constexpr int VPR = K::DV / 8;
  for (int t = threadIdx.x; t < K::C * VPR; t += K::NT) {
    const int r = t / VPR, c = (t % VPR) * 8;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (r < n) val = *reinterpret_cast<const uint4*>(v + (int64_t)r * K::DV + c);
    const uint32_t w[4] = {val.x, val.y, val.z, val.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      sv[(c + 2 * q) * K::LDV + r] = (uint16_t)(w[q] & 0xFFFF);
      sv[(c + 2 * q + 1) * K::LDV + r] = (uint16_t)(w[q] >> 16);
    }
  }
}

// Constant rows of v'^T: row DV is all ones (the z column), rows DV+1.. zero.
template <class K>
__device__ __forceinline__ void init_vones(uint16_t* sv) {
  for (int t = threadIdx.x; t < 16 * K::LDV; t += K::NT) {
    const int r = t / K::LDV;
    sv[(K::DV + r) * K::LDV + (t % K::LDV)] = (r == 0) ? kBf16One : (uint16_t)0;
  }
}

// v' operand for a token k-step s and state column tile et: lane (e = et*16+col,
// group g) gets tokens 32s+4g..+3 and 32s+16+4g..+3 (the shared permutation).
template <class K>
__device__ __forceinline__ bf16x8 vfrag(const uint16_t* sv, int et, int s, int lane) {
  const int g = lane >> 4, col = lane & 15;
  const uint16_t* row = sv + (et * 16 + col) * K::LDV + 32 * s + 4 * g;
  const uint2 lo = *reinterpret_cast<const uint2*>(row);
  const uint2 hi = *reinterpret_cast<const uint2*>(row + 16);
  return as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
}

// phi(k) of the staged chunk for this wave's features (tokens as M).  Returns
// the bf16 A-operands of the state update in kf[j][s]; if PHI_LDS, also
// stores phi(k)[j][f] into LDS.
template <class K, bool PHI_LDS>
__device__ __forceinline__ void phase_k(const uint16_t* sx, const float* sinv, uint16_t* spk, int wave, int lane,
                                        const bf16x8 (&pa)[K::FBW][K::NKS], const bf16x8 (&pg)[K::FBW][K::NKS],
                                        const float (&c1)[K::FBW], const float (&c0)[K::FBW],
                                        bf16x8 (&kf)[K::FBW][K::NTS]) {
  const int g = lane >> 4, col = lane & 15;
#pragma unroll
  for (int tb = 0; tb < K::NTB; ++tb) {
    bf16x8 xa[K::NKS];
#pragma unroll
    for (int ks = 0; ks < K::NKS; ++ks)
      xa[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(sx + (tb * 16 + col) * K::LDX + ks * 32 + 8 * g));
    const float4 inv4 = *reinterpret_cast<const float4*>(sinv + tb * 16 + 4 * g);
    const float inv[4] = {inv4.x, inv4.y, inv4.z, inv4.w};
#pragma unroll
    for (int j = 0; j < K::FBW; ++j) {
      f32x4 ya = {0.f, 0.f, 0.f, 0.f}, yg = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < K::NKS; ++ks) {
        ya = mfma_bf16(xa[ks], pa[j][ks], ya);
        yg = mfma_bf16(xa[ks], pg[j][ks], yg);
      }
      float ph[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a = ya[i] * inv[i];
        ph[i] = a * a * fast_exp2(fmaf(yg[i], inv[i] * c1[j], c0[j]));
      }
      const uint2 pk = pack4(ph[0], ph[1], ph[2], ph[3]);
      // kf[j][s] = (tokens 32s+4g..+3 | 32s+16+4g..+3)
      uint4 cur = __builtin_bit_cast(uint4, kf[j][tb >> 1]);
      if ((tb & 1) == 0) {
        cur.x = pk.x;
        cur.y = pk.y;
      } else {
        cur.z = pk.x;
        cur.w = pk.y;
      }
      kf[j][tb >> 1] = as_bf16x8(cur);
      if (PHI_LDS) {
        const int f = (wave * K::FBW + j) * 16 + col;
        uint16_t* dst = spk + (tb * 16 + 4 * g) * K::LDF + f;
        dst[0] = (uint16_t)(pk.x & 0xFFFF);
        dst[K::LDF] = (uint16_t)(pk.x >> 16);
        dst[2 * K::LDF] = (uint16_t)(pk.y & 0xFFFF);
        dst[3 * K::LDF] = (uint16_t)(pk.y >> 16);
      }
    }
  }
}

// phi(q) of the staged chunk for this wave's features (features as M), to LDS phi(q)[i][f].
template <class K>
__device__ __forceinline__ void phase_q(const uint16_t* sx, const float* sinv, uint16_t* spq, int wave, int lane,
                                        const bf16x8 (&pa)[K::FBW][K::NKS], const bf16x8 (&pg)[K::FBW][K::NKS],
                                        const float (&c1)[K::FBW], const float (&c0)[K::FBW]) {
  const int g = lane >> 4, col = lane & 15;
#pragma unroll
  for (int tb = 0; tb < K::NTB; ++tb) {
    bf16x8 xb[K::NKS];
#pragma unroll
    for (int ks = 0; ks < K::NKS; ++ks)
      xb[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(sx + (tb * 16 + col) * K::LDX + ks * 32 + 8 * g));
    const float inv = sinv[tb * 16 + col];
#pragma unroll
    for (int j = 0; j < K::FBW; ++j) {
      f32x4 ya = {0.f, 0.f, 0.f, 0.f}, yg = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < K::NKS; ++ks) {
        ya = mfma_bf16(pa[j][ks], xb[ks], ya);
        yg = mfma_bf16(pg[j][ks], xb[ks], yg);
      }
      const float s1 = inv * c1[j];
      float ph[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a = ya[i] * inv;
        ph[i] = a * a * fast_exp2(fmaf(yg[i], s1, c0[j]));
      }
      const int f0 = (wave * K::FBW + j) * 16 + 4 * g;
      *reinterpret_cast<uint2*>(spq + (tb * 16 + col) * K::LDF + f0) = pack4(ph[0], ph[1], ph[2], ph[3]);
    }
  }
}

// State update S'[own features] += phi(k)^T v' (tokens contracted).
template <class K>
__device__ __forceinline__ void state_update(const uint16_t* sv, int lane, const bf16x8 (&kf)[K::FBW][K::NTS],
                                             f32x4 (&st)[K::FBW][K::NE]) {
#pragma unroll
  for (int s = 0; s < K::NTS; ++s)
#pragma unroll
    for (int et = 0; et < K::NE; ++et) {
      const bf16x8 vb = vfrag<K>(sv, et, s, lane);
#pragma unroll
      for (int j = 0; j < K::FBW; ++j) st[j][et] = mfma_bf16(kf[j][s], vb, st[j][et]);
    }
}

// Write this wave's S' slice as bf16 rows of S'^T in LDS.
template <class K>
__device__ __forceinline__ void write_st(uint16_t* sst, int wave, int lane, const f32x4 (&st)[K::FBW][K::NE]) {
  const int g = lane >> 4, col = lane & 15;
#pragma unroll
  for (int j = 0; j < K::FBW; ++j)
#pragma unroll
    for (int et = 0; et < K::NE; ++et) {
      const int f0 = (wave * K::FBW + j) * 16 + 4 * g;
      *reinterpret_cast<uint2*>(sst + (et * 16 + col) * K::LDF + f0) =
          pack4(st[j][et][0], st[j][et][1], st[j][et][2], st[j][et][3]);
    }
}

// Fragment-ordered state index of (feature block fb, column tile et, lane).
template <class K>
__device__ __forceinline__ int64_t frag_off(int fb, int et, int lane) {
  return ((int64_t)(fb * K::NE + et) * 64 + lane) * 4;
}

// ---------------------------------------------------------------------------
template <class K>
__global__ __launch_bounds__(K::NT) void pass1_kernel(Params p) {
  extern __shared__ __align__(16) unsigned char lds[];
  uint16_t* sK = reinterpret_cast<uint16_t*>(lds + K::kK - K::kK);
  uint16_t* sV = reinterpret_cast<uint16_t*>(lds + K::C * K::LDX * 2);
  float* sinv = reinterpret_cast<float*>(lds + K::C * K::LDX * 2 + K::DVP * K::LDV * 2);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nseg1 = p.n_seg - 1;
  const int64_t head = blockIdx.x / nseg1;
  const int seg = (int)(blockIdx.x - head * nseg1);
  const int set = (int)(head % p.n_draw_sets);

  bf16x8 pa[K::FBW][K::NKS], pg[K::FBW][K::NKS];
  float c1[K::FBW], c0[K::FBW];
  load_p<K>(p, set, wave, lane, pa, pg, c1, c0);
  f32x4 st[K::FBW][K::NE];
#pragma unroll
  for (int j = 0; j < K::FBW; ++j)
#pragma unroll
    for (int et = 0; et < K::NE; ++et) st[j][et] = f32x4{0.f, 0.f, 0.f, 0.f};
  bf16x8 kf[K::FBW][K::NTS];
  init_vones<K>(sV);

  const int64_t t0 = (int64_t)seg * p.seg_len;
  const int64_t t1 = min<int64_t>(p.L, t0 + p.seg_len);
  for (int64_t c0t = t0; c0t < t1; c0t += K::C) {
    const int n = (int)min<int64_t>(K::C, t1 - c0t);
    __syncthreads();
    stage_x<K>(p.k + (head * p.L + c0t) * K::D, n, sK, sinv);
    stage_v<K>(p.v + (head * p.L + c0t) * K::DV, n, sV);
    __syncthreads();
    phase_k<K, false>(sK, sinv, nullptr, wave, lane, pa, pg, c1, c0, kf);
    state_update<K>(sV, lane, kf, st);
  }
  float* out = p.ws + (head * p.n_seg + seg) * (int64_t)K::F * K::DVP;
#pragma unroll
  for (int j = 0; j < K::FBW; ++j)
#pragma unroll
    for (int et = 0; et < K::NE; ++et)
      *reinterpret_cast<f32x4*>(out + frag_off<K>(wave * K::FBW + j, et, lane)) = st[j][et];
}

template <class K>
__global__ __launch_bounds__(K::NT) void pass2_kernel(Params p) {
  extern __shared__ __align__(16) unsigned char lds[];
  uint16_t* sQ = reinterpret_cast<uint16_t*>(lds + K::kQ);
  uint16_t* sK = reinterpret_cast<uint16_t*>(lds + K::kK);
  uint16_t* sV = reinterpret_cast<uint16_t*>(lds + K::kV);
  uint16_t* sPq = reinterpret_cast<uint16_t*>(lds + K::kPq);
  uint16_t* sPk = reinterpret_cast<uint16_t*>(lds + K::kPk);
  uint16_t* sSt = reinterpret_cast<uint16_t*>(lds + K::kSt);
  f32x4* sX = reinterpret_cast<f32x4*>(lds + K::kX);
  float* sinvq = reinterpret_cast<float*>(lds + K::kInv);
  float* sinvk = sinvq + K::C;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, col = lane & 15;
  const int64_t head = blockIdx.x / p.n_seg;
  const int seg = (int)(blockIdx.x - head * p.n_seg);
  const int set = (int)(head % p.n_draw_sets);

  bf16x8 pa[K::FBW][K::NKS], pg[K::FBW][K::NKS];
  float c1[K::FBW], c0[K::FBW];
  load_p<K>(p, set, wave, lane, pa, pg, c1, c0);

  // initial state of the segment
  f32x4 st[K::FBW][K::NE];
  if (p.n_seg > 1) {
    const float* in = p.ws + (head * p.n_seg + seg) * (int64_t)K::F * K::DVP;
#pragma unroll
    for (int j = 0; j < K::FBW; ++j)
#pragma unroll
      for (int et = 0; et < K::NE; ++et)
        st[j][et] = *reinterpret_cast<const f32x4*>(in + frag_off<K>(wave * K::FBW + j, et, lane));
  } else {
#pragma unroll
    for (int j = 0; j < K::FBW; ++j)
#pragma unroll
      for (int et = 0; et < K::NE; ++et) {
        const int e = et * 16 + col;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int f = (wave * K::FBW + j) * 16 + 4 * g + i;
          float val = 0.f;
          if (e < K::DV) {
            if (p.S0) val = p.S0[(head * K::F + f) * K::DV + e];
          } else if (e == K::DV) {
            if (p.z0) val = p.z0[head * K::F + f];
          }
          st[j][et][i] = val;
        }
      }
  }
  init_vones<K>(sV);
  write_st<K>(sSt, wave, lane, st);
  bf16x8 kf[K::FBW][K::NTS];

  const bool intra_wave = wave < K::NTB;
  const int ib_intra = wave;
  const bool inter_wave = (wave >= K::NTB) && (wave - K::NTB < K::NINTER);
  const int ib_inter = wave - K::NTB;
  const bool self_inter = intra_wave && (wave >= K::NINTER);  // intra wave also does its inter

  const int64_t t0 = (int64_t)seg * p.seg_len;
  const int64_t t1 = min<int64_t>(p.L, t0 + p.seg_len);
  for (int64_t c0t = t0; c0t < t1; c0t += K::C) {
    const int n = (int)min<int64_t>(K::C, t1 - c0t);
    __syncthreads();  // B0: previous chunk done with every LDS tile
    stage_x<K>(p.q + (head * p.L + c0t) * K::D, n, sQ, sinvq);
    stage_x<K>(p.k + (head * p.L + c0t) * K::D, n, sK, sinvk);
    stage_v<K>(p.v + (head * p.L + c0t) * K::DV, n, sV);
    __syncthreads();  // B1
    phase_k<K, true>(sK, sinvk, sPk, wave, lane, pa, pg, c1, c0, kf);
    phase_q<K>(sQ, sinvq, sPq, wave, lane, pa, pg, c1, c0);
    __syncthreads();  // B2: phi(q), phi(k) complete

    f32x4 acc[K::NE];
#pragma unroll
    for (int et = 0; et < K::NE; ++et) acc[et] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (intra_wave) {
      const int ib = ib_intra;
      // A^T blocks (jb, ib), jb <= ib, contracted over all F features
      f32x4 at[K::NTB];
#pragma unroll
      for (int jb = 0; jb < K::NTB; ++jb) at[jb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kf_ = 0; kf_ < K::NFK; ++kf_) {
        const bf16x8 bq = as_bf16x8(*reinterpret_cast<const uint4*>(sPq + (ib * 16 + col) * K::LDF + kf_ * 32 + 8 * g));
#pragma unroll
        for (int jb = 0; jb < K::NTB; ++jb) {
          if (jb <= ib) {
            const bf16x8 ak =
                as_bf16x8(*reinterpret_cast<const uint4*>(sPk + (jb * 16 + col) * K::LDF + kf_ * 32 + 8 * g));
            at[jb] = mfma_bf16(ak, bq, at[jb]);
          }
        }
      }
      // causal mask on the diagonal block: keep j <= i (row 4g+i, column col)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * g + i > col) at[ib][i] = 0.f;
      // num'^T += v'^T A^T over token k-steps s (blocks 2s, 2s+1)
#pragma unroll
      for (int s = 0; s < K::NTS; ++s) {
        if (2 * s <= ib) {
          const uint2 lo = pack4(at[2 * s][0], at[2 * s][1], at[2 * s][2], at[2 * s][3]);
          uint2 hi = make_uint2(0, 0);
          if (2 * s + 1 <= ib) hi = pack4(at[2 * s + 1][0], at[2 * s + 1][1], at[2 * s + 1][2], at[2 * s + 1][3]);
          const bf16x8 ab = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
#pragma unroll
          for (int et = 0; et < K::NE; ++et) acc[et] = mfma_bf16(vfrag<K>(sV, et, s, lane), ab, acc[et]);
        }
      }
    }
    if (inter_wave || self_inter) {
      const int ib = inter_wave ? ib_inter : ib_intra;
#pragma unroll 2
      for (int kf_ = 0; kf_ < K::NFK; ++kf_) {
        const bf16x8 bq = as_bf16x8(*reinterpret_cast<const uint4*>(sPq + (ib * 16 + col) * K::LDF + kf_ * 32 + 8 * g));
#pragma unroll
        for (int et = 0; et < K::NE; ++et) {
          const bf16x8 as =
              as_bf16x8(*reinterpret_cast<const uint4*>(sSt + (et * 16 + col) * K::LDF + kf_ * 32 + 8 * g));
          acc[et] = mfma_bf16(as, bq, acc[et]);
        }
      }
      if (inter_wave) {
#pragma unroll
        for (int et = 0; et < K::NE; ++et) sX[(ib_inter * K::NE + et) * 64 + lane] = acc[et];
      }
    }
    __syncthreads();  // B3: inter partials published; S'^T copy no longer read

    if (intra_wave) {
      const int ib = ib_intra;
      if (!self_inter) {
#pragma unroll
        for (int et = 0; et < K::NE; ++et) {
          const f32x4 x = sX[(ib * K::NE + et) * 64 + lane];
          acc[et] += x;
        }
      }
      // den of token col = element (row dv, column col): lane col (g = 0), i = 0 of tile NE-1
      const float den = __shfl(acc[K::NE - 1][0], col, 64);
      const float rden = 1.0f / den;
      const int tok = ib * 16 + col;
      if (tok < n) {
        uint16_t* orow = p.o + (head * p.L + c0t + tok) * K::DV;
#pragma unroll
        for (int et = 0; et < K::NE - 1; ++et)
          *reinterpret_cast<uint2*>(orow + et * 16 + 4 * g) =
              pack4(acc[et][0] * rden, acc[et][1] * rden, acc[et][2] * rden, acc[et][3] * rden);
      }
    }
    state_update<K>(sV, lane, kf, st);
    write_st<K>(sSt, wave, lane, st);
  }

  if (seg == p.n_seg - 1 && (p.S_out || p.z_out)) {
#pragma unroll
    for (int j = 0; j < K::FBW; ++j)
#pragma unroll
      for (int et = 0; et < K::NE; ++et) {
        const int e = et * 16 + col;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int f = (wave * K::FBW + j) * 16 + 4 * g + i;
          if (e < K::DV) {
            if (p.S_out) p.S_out[(head * K::F + f) * K::DV + e] = st[j][et][i];
          } else if (e == K::DV) {
            if (p.z_out) p.z_out[head * K::F + f] = st[j][et][i];
          }
        }
      }
  }
}

template <class K>
int pick_segments(const ChunkedArgs& a) {
  const int64_t n_chunks = (a.L + K::C - 1) / K::C;
  int64_t want = (256 + a.n_heads - 1) / a.n_heads;
  if (want > n_chunks) want = n_chunks;
  if (want < 1) want = 1;
  const int64_t cps = (n_chunks + want - 1) / want;  // chunks per segment
  return (int)((n_chunks + cps - 1) / cps);
}

template <class K>
int64_t seg_len_of(const ChunkedArgs& a, int n_seg) {
  const int64_t n_chunks = (a.L + K::C - 1) / K::C;
  return ((n_chunks + n_seg - 1) / n_seg) * K::C;
}

template <class K>
size_t ws_bytes_t(const ChunkedArgs& a) {
  const int n_seg = pick_segments<K>(a);
  return n_seg > 1 ? sizeof(float) * (size_t)a.n_heads * n_seg * K::F * K::DVP : 0;
}

template <class K>
hipError_t launch_t(const ChunkedArgs& a, hipStream_t s) {
  const int n_seg = pick_segments<K>(a);
  Params p{};
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.o = static_cast<uint16_t*>(a.o);
  p.L = a.L;
  p.n_seg = n_seg;
  p.seg_len = seg_len_of<K>(a, n_seg);
  p.m = a.m;
  p.anchors = static_cast<const uint16_t*>(a.anchors);
  p.prf = static_cast<const uint16_t*>(a.prf);
  p.draw_set_stride = a.draw_set_stride;
  p.n_draw_sets = a.n_draw_sets;
  p.nc = a.nc;
  p.ws = static_cast<float*>(a.ws);
  p.S0 = a.S0;
  p.z0 = a.z0;
  p.S_out = a.S_out;
  p.z_out = a.z_out;
  hipError_t e;
  if (n_seg > 1) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&pass1_kernel<K>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, K::kLds1);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(pass1_kernel<K>, dim3((unsigned)(a.n_heads * (n_seg - 1))), dim3(K::NT), K::kLds1, s, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    ScanArgs sa{};
    sa.states = p.ws;
    sa.n_heads = a.n_heads;
    sa.n_items = n_seg;
    sa.n_terms = n_seg - 1;
    sa.F = K::F;
    sa.dv = K::DV;
    sa.layout = 1;
    sa.S0 = a.S0;
    sa.z0 = a.z0;
    sa.S_out = nullptr;
    sa.z_out = nullptr;
    e = launch_scan(sa, s);
    if (e != hipSuccess) return e;
  }
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&pass2_kernel<K>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, K::kLds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(pass2_kernel<K>, dim3((unsigned)(a.n_heads * n_seg)), dim3(K::NT), K::kLds, s, p);
  return hipGetLastError();
}

typedef Cfg<64, 64, 64, 8, 2> CfgF256;
typedef Cfg<64, 64, 64, 8, 1> CfgF128;
typedef Cfg<64, 64, 64, 6, 1> CfgF96;
typedef Cfg<64, 64, 64, 4, 1> CfgF64;

template <typename Fn>
bool dispatch(const ChunkedArgs& a, Fn&& fn) {
  if (!a.io_bf16 || a.d != 64 || a.dv != 64 || a.chunk != 64 || a.m % 16 != 0) return false;
  switch (a.F) {
    case 256: fn(CfgF256()); return true;
    case 128: fn(CfgF128()); return true;
    case 96: fn(CfgF96()); return true;
    case 64: fn(CfgF64()); return true;
    default: return false;
  }
}

}  // namespace

bool fused_supported(const ChunkedArgs& a) {
  return dispatch(a, [](auto) {});
}

size_t fused_workspace_bytes(const ChunkedArgs& a) {
  size_t r = 0;
  dispatch(a, [&](auto k) { r = ws_bytes_t<decltype(k)>(a); });
  return r;
}

hipError_t launch_fused(const ChunkedArgs& a, hipStream_t s) {
  if (a.n_heads == 0) return hipSuccess;
  if (a.L == 0) return launch_generic(a, s);  // only the state passes through
  hipError_t e = hipErrorInvalidValue;
  dispatch(a, [&](auto k) { e = launch_t<decltype(k)>(a, s); });
  return e;
}

}  // namespace slay
