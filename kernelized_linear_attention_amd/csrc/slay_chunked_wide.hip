// slay_chunked_wide.hip -- causal SLAY forward for wide shapes (bf16; F up
// to 512 and dv of 64 or 128, e.g. d = dv = 128 with F = 512) on gfx950 MFMA.
//
// Method ("SLAY: Geometry-Aware Spherical Linearized Attention with
// Yat-Kernel", abstract; nubint.ai review, "Proposed method" bullet 6):
// o_i = phi(q_i)^T S_i / phi(q_i)^T z_i with S_i = sum_{j<=i} phi(k_j) v_j^T,
// z_i = sum_{j<=i} phi(k_j), evaluated chunk by chunk without the L x L
// matrix.
//
// Why a path of its own.  The fused kernels keep one head's whole state
// (F x (dv+16) fp32) in accumulators next to the projection matrix
// P = [anchors; prf] (2F x d bf16) in registers.  At F = 512, d = dv = 128
// these are 295 KB and 256 KB: more than one CU holds.  Here the feature
// maps are written to HBM once in bf16 and the contraction kernels keep only
// the state on chip:
//   1. featmap : phi(q), phi(k) -> workspace, [rows][F] bf16 (one launch);
//   2. wstate  : per (head, segment) the segment's deltas dS = phi(K)^T V and
//                dz = phi(K)^T 1, stored fragment-ordered (segments but the last);
//   3. scan    : exclusive prefix over the segments of each head, plus S0, z0;
//   4. wout    : per (head, segment), 32-token chunks from the prefix state:
//                A = tril(phi(Q) phi(K)^T) on the chunk,
//                o = (phi(Q) S + A V) / (phi(Q) z + A 1), then S += phi(K)^T V,
//                z += phi(K)^T 1; the last segment writes the final state.
//
// Wave layout (8 waves per workgroup).  The dv columns form NCG groups of 32
// (two 16-column MFMA tiles) and the F features NFS = 8 / NCG slices; wave
// (cg, fs) keeps S[slice fs][group cg] as fp32 accumulators for the whole
// segment (128 registers at F = 512, dv = 128).  Per chunk it computes its
// partial num^T = S^T phi(Q)^T over its features, with the accumulators
// themselves as the MFMA A operand (two 16-feature tiles give a lane the 8
// features 4g..4g+3 and 16+4g..16+4g+3 of one column; phi(q) is read in the
// same feature order), then the state update with phi(K)^T and V^T staged
// token-contiguous in LDS.  The partials of a token tile meet in LDS and the
// wave (cg, it) finishes tile it: num^T += V^T A^T, divide, store.  z is
// summed in fp32 on the VALU: wave w owns features [w F/8, (w+1) F/8) of z,
// adds phi(k) over the chunk (bf16 dot products with ones) and forms its part
// of phi(q) . z for every token from a bf16 copy of z (as S enters the
// readout in bf16).
// The three causal 16x16 tiles of A^T are formed by waves 0..2, rounded to
// bf16 (the same values feed A V and A 1) and shared through LDS.
#include "slay_device.hpp"
#include "slay_internal.hpp"

namespace slay {

namespace {

template <int F_, int DV_>
struct WCfg {
  static constexpr int F = F_, DV = DV_;
  static constexpr int C = 32;             // tokens per chunk
  static constexpr int NW = 8, NT = NW * 64;
  static constexpr int NCG = DV / 32;      // column groups of 32
  static constexpr int NFS = NW / NCG;     // feature slices
  static constexpr int FS = F / NFS;       // features per slice
  static constexpr int NFT = FS / 16;      // 16-feature accumulator tiles per column tile
  static constexpr int NKS = FS / 32;      // readout k-steps
  static constexpr int NE = DV / 16 + 1;   // column tiles of a stored state (z in column dv)
  static constexpr int ZPW = F / NW;       // z features per wave
  static constexpr int QPT = F / 128;      // 16-byte phi(q) row pieces per thread and chunk
  static constexpr int LQ = F + 8;         // phi rows in LDS (elements): 16 lanes of a column hit distinct banks
  static constexpr int LT = C + 8;         // token-contiguous rows (phi(k)^T, v^T)
  static constexpr int LA = C + 8;         // rows of A
  static constexpr int LD = 12;            // denominator parts per token: 8 waves, 2 row-sum tiles, 2 zero
  static constexpr int NSLOT = NFS - 1;    // partials one output wave receives
  // output pass LDS (bytes)
  static constexpr int oQ = 0;
  static constexpr int oK = oQ + C * LQ * 2;
  static constexpr int oKt = oK + C * LQ * 2;
  static constexpr int oVt = oKt + F * LT * 2;
  static constexpr int oA = oVt + DV * LT * 2;
  static constexpr int oP = oA + C * LA * 2;
  static constexpr int oDen = oP + NCG * 2 * NSLOT * 2 * 1024;
  static constexpr int oZ = oDen + C * LD * 4;
  static constexpr int LO = DV + 8;        // staged output rows
  static constexpr int oO = oZ + F * 4;
  static constexpr int kLds = oO + C * LO * 2;
  // state pass LDS: phi(k)^T and v^T double-buffered
  static constexpr int bKt = F * LT * 2, bVt = DV * LT * 2;
  static constexpr int oZ1 = 2 * (bKt + bVt);
  static constexpr int kLds1 = oZ1 + F * 4;
  static_assert(DV % 32 == 0 && NW % NCG == 0 && NFS >= 2, "column groups");
  static_assert(F % 128 == 0 && F <= NT && FS % 32 == 0 && ZPW <= 64 && ZPW % 16 == 0, "feature slices");
  static_assert(4 * DV <= NT, "one v block per thread");
  static_assert(kLds <= 160 * 1024 && kLds1 <= 160 * 1024, "LDS budget");
};

struct WParams {
  const uint16_t* phiq;  // [n_heads * L][F]
  const uint16_t* phik;
  const uint16_t* v;     // [n_heads * L][dv]
  uint16_t* o;
  float* states;         // [n_heads][n_seg][F/16][NE][64][4]
  int64_t L;
  int64_t seg_len;       // multiple of 32
  int n_seg;
  float* S_out;          // nullable [n_heads][F][dv]
  float* z_out;          // nullable [n_heads][F]
};

__device__ __forceinline__ float lo_f(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_f(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ bf16x8 ld8w(const uint16_t* p) { return as_bf16x8(*reinterpret_cast<const uint4*>(p)); }
__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

// Registers holding one chunk's loads until they are written to LDS.
template <class K>
struct WPref {
  uint4 q[K::QPT];  // phi(q) row pieces
  uint4 k[4];       // phi(k): 4 tokens x 8 features
  uint32_t v[4];    // v: 4 tokens x 2 columns
};

// Issue the loads of chunk rows [0, 32) starting at packed row `row0`; rows
// at or beyond `n` read as zero (the ragged tail of a sequence).
template <class K, bool WANT_Q>
__device__ __forceinline__ void w_load(const WParams& p, int64_t row0, int n, int tid, WPref<K>& pf) {
  // Each address is a wave-uniform row base plus one 32-bit lane offset in
  // bytes (the same offset for the four rows of a thread), so the loads take
  // the scalar-base form and few registers hold addresses.
  const uint4 z4 = {0u, 0u, 0u, 0u};
  if constexpr (WANT_Q) {
    // piece u of thread tid is 8 elements at row-major offset 8 (tid + u NT)
    const char* base = reinterpret_cast<const char*>(p.phiq + row0 * K::F);
    const uint32_t off = 16u * (uint32_t)tid;
#pragma unroll
    for (int u = 0; u < K::QPT; ++u) {
      const int r = (tid + u * K::NT) / (K::F / 8);
      pf.q[u] = z4;
      if (r < n) pf.q[u] = *reinterpret_cast<const uint4*>(base + (size_t)u * K::NT * 16 + off);
    }
  }
  if (tid < K::F) {
    const int r4 = tid % 8, c8 = tid / 8;
    const uint32_t off = 2u * (uint32_t)(4 * r4 * K::F + 8 * c8);
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const char* base = reinterpret_cast<const char*>(p.phik + (row0 + x) * K::F);
      pf.k[x] = z4;
      if (4 * r4 + x < n) pf.k[x] = *reinterpret_cast<const uint4*>(base + off);
    }
  }
  if (tid < 4 * K::DV) {
    const int r4 = tid / (K::DV / 2), c2 = tid % (K::DV / 2);
    const uint32_t off = 2u * (uint32_t)(4 * r4 * K::DV + 2 * c2);
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const char* base = reinterpret_cast<const char*>(p.v + (row0 + x) * K::DV);
      pf.v[x] = 0u;
      if (4 * r4 + x < n) pf.v[x] = *reinterpret_cast<const uint32_t*>(base + off);
    }
  }

}

// Write a chunk to LDS: phi(q), phi(k) as rows (when ROWS), phi(k)^T and v^T
// token-contiguous (a 4-token block is transposed in registers with byte
// permutes and written as 8-byte column pieces).
template <class K, bool ROWS>
__device__ __forceinline__ void w_store(uint16_t* sQ, uint16_t* sK, uint16_t* sKt, uint16_t* sVt, int tid,
                                        const WPref<K>& pf) {
  if constexpr (ROWS) {
#pragma unroll
    for (int u = 0; u < K::QPT; ++u) {
      const int piece = tid + u * K::NT;
      const int r = piece / (K::F / 8), c8 = piece % (K::F / 8);
      *reinterpret_cast<uint4*>(sQ + r * K::LQ + 8 * c8) = pf.q[u];
    }
  }
  if (tid < K::F) {
    const int r4 = tid % 8, c8 = tid / 8;
    if constexpr (ROWS) {
#pragma unroll
      for (int x = 0; x < 4; ++x) *reinterpret_cast<uint4*>(sK + (4 * r4 + x) * K::LQ + 8 * c8) = pf.k[x];
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t a = word(pf.k[0], w), b = word(pf.k[1], w), c = word(pf.k[2], w), d = word(pf.k[3], w);
      *reinterpret_cast<uint2*>(sKt + (8 * c8 + 2 * w) * K::LT + 4 * r4) = make_uint2(lo16_pair(a, b), lo16_pair(c, d));
      *reinterpret_cast<uint2*>(sKt + (8 * c8 + 2 * w + 1) * K::LT + 4 * r4) =
          make_uint2(hi16_pair(a, b), hi16_pair(c, d));
    }
  }
  if (tid < 4 * K::DV) {
    const int r4 = tid / (K::DV / 2), c2 = tid % (K::DV / 2);
    *reinterpret_cast<uint2*>(sVt + (2 * c2) * K::LT + 4 * r4) =
        make_uint2(lo16_pair(pf.v[0], pf.v[1]), lo16_pair(pf.v[2], pf.v[3]));
    *reinterpret_cast<uint2*>(sVt + (2 * c2 + 1) * K::LT + 4 * r4) =
        make_uint2(hi16_pair(pf.v[0], pf.v[1]), hi16_pair(pf.v[2], pf.v[3]));
  }
}

// S[slice fs][group cg] += phi(K)^T V over one staged chunk; returns the
// wave's V^T operands (they are also the A operands of V^T A^T).
template <class K>
__device__ __forceinline__ void w_update(const uint16_t* sKt, const uint16_t* sVt, int cg, int fs, int lane,
                                         f32x4 (&acc)[K::NFT][2], uint4 (&bv)[2]) {
  const int g = lane >> 4, col = lane & 15;
#pragma unroll
  for (int et = 0; et < 2; ++et)
    bv[et] = *reinterpret_cast<const uint4*>(sVt + (32 * cg + 16 * et + col) * K::LT + 8 * g);
#pragma unroll
  for (int ft = 0; ft < K::NFT; ++ft) {
    const bf16x8 ak = ld8w(sKt + (fs * K::FS + 16 * ft + col) * K::LT + 8 * g);
#pragma unroll
    for (int et = 0; et < 2; ++et) acc[ft][et] = mfma_bf16(ak, as_bf16x8(bv[et]), acc[ft][et]);
  }
}

// z[f] += sum over the chunk's tokens of phi(k)[f] for the wave's features
// (lane f - w*ZPW), accumulated in fp32 (bf16 dot products with ones); a bf16
// copy of z goes to sZb for the denominators when sZb is set.
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

template <class K>
__device__ __forceinline__ void w_zupdate(const uint16_t* sKt, uint16_t* sZb, int zf, int lane, float& zreg) {
  constexpr uint32_t kOnes = 0x3F803F80u;  // bf16 pair (1, 1)
  if (lane < K::ZPW) {
    const uint16_t* kr = sKt + zf * K::LT;
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int x = 0; x < K::C / 8; ++x) {
      const uint4 kv = *reinterpret_cast<const uint4*>(kr + 8 * x);
      s0 = dot2(kv.x, kOnes, s0);
      s1 = dot2(kv.y, kOnes, s1);
      s0 = dot2(kv.z, kOnes, s0);
      s1 = dot2(kv.w, kOnes, s1);
    }
    zreg += s0 + s1;
    if (sZb) sZb[zf] = f32_to_bf16(zreg);
  }
}

template <class K>
__global__ __launch_bounds__(K::NT) void wstate_kernel(WParams p) {
  extern __shared__ __align__(16) unsigned char lds[];
  float* sZ = reinterpret_cast<float*>(lds + K::oZ1);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int cg = wave % K::NCG, fs = wave / K::NCG;
  const int64_t h = blockIdx.x / (p.n_seg - 1);
  const int seg = (int)(blockIdx.x - h * (p.n_seg - 1));
  const int64_t row0 = h * p.L + (int64_t)seg * p.seg_len;  // segments before the last are full
  const int n_chunks = (int)(p.seg_len / K::C);
  const int zf = wave * K::ZPW + lane;

  f32x4 acc[K::NFT][2];
#pragma unroll
  for (int ft = 0; ft < K::NFT; ++ft)
#pragma unroll
    for (int et = 0; et < 2; ++et) acc[ft][et] = f32x4{0.f, 0.f, 0.f, 0.f};
  float zreg = 0.f;

  WPref<K> pf;
  w_load<K, false>(p, row0, K::C, tid, pf);
  w_store<K, false>(nullptr, nullptr, reinterpret_cast<uint16_t*>(lds), reinterpret_cast<uint16_t*>(lds + 2 * K::bKt),
                    tid, pf);
  __syncthreads();
  for (int c = 0; c < n_chunks; ++c) {
    const int b = c & 1;
    const uint16_t* sKt = reinterpret_cast<const uint16_t*>(lds + b * K::bKt);
    const uint16_t* sVt = reinterpret_cast<const uint16_t*>(lds + 2 * K::bKt + b * K::bVt);
    const bool more = c + 1 < n_chunks;
    if (more) w_load<K, false>(p, row0 + (int64_t)(c + 1) * K::C, K::C, tid, pf);
    uint4 bv[2];
    w_update<K>(sKt, sVt, cg, fs, lane, acc, bv);
    w_zupdate<K>(sKt, nullptr, zf, lane, zreg);
    if (more)
      w_store<K, false>(nullptr, nullptr, reinterpret_cast<uint16_t*>(lds + (b ^ 1) * K::bKt),
                        reinterpret_cast<uint16_t*>(lds + 2 * K::bKt + (b ^ 1) * K::bVt), tid, pf);
    __syncthreads();
  }
  // deltas of this segment -> item (h, seg), fragment order
  float* st = p.states + (h * p.n_seg + seg) * (int64_t)(K::F / 16) * K::NE * 256;
#pragma unroll
  for (int ft = 0; ft < K::NFT; ++ft)
#pragma unroll
    for (int et = 0; et < 2; ++et)
      *reinterpret_cast<f32x4*>(st + ((fs * K::NFT + ft) * K::NE + 2 * cg + et) * 256 + lane * 4) = acc[ft][et];
  if (lane < K::ZPW) sZ[zf] = zreg;
  __syncthreads();
  // z tile: column dv of the state, i.e. lanes 0, 16, 32, 48 of tile NE-1
  for (int x = tid; x < (K::F / 16) * 64; x += K::NT) {
    const int ft = x >> 6, L = x & 63;
    f32x4 val = {0.f, 0.f, 0.f, 0.f};
    if ((L & 15) == 0) val = *reinterpret_cast<const f32x4*>(sZ + 16 * ft + 4 * (L >> 4));
    *reinterpret_cast<f32x4*>(st + (ft * K::NE + K::NE - 1) * 256 + L * 4) = val;
  }
}

// Token tile IT of the chunk (by the waves with fs == IT): add the other
// slices' partials of num^T, then V^T A^T, divide by the denominator and
// stage the bf16 rows in LDS.
template <class K, int IT>
__device__ __forceinline__ void w_finish(const float* sP, const uint16_t* sA, const float* sDen, uint16_t* sO,
                                         int cg, int fs, int lane, const f32x4 (&num)[2], const uint4 (&bv)[2]) {
  const int g = lane >> 4, col = lane & 15;
  f32x4 r[2] = {num[0], num[1]};
#pragma unroll
  for (int slot = 0; slot < K::NSLOT; ++slot)
#pragma unroll
    for (int et = 0; et < 2; ++et)
      r[et] += *reinterpret_cast<const f32x4*>(sP + ((((cg * 2 + IT) * K::NSLOT + slot) * 2 + et) * 64 + lane) * 4);
  const bf16x8 av = ld8w(sA + (16 * IT + col) * K::LA + 8 * g);
#pragma unroll
  for (int et = 0; et < 2; ++et) r[et] = mfma_bf16(as_bf16x8(bv[et]), av, r[et]);
  const float* dr = sDen + (16 * IT + col) * K::LD;
  const f32x4 d0 = *reinterpret_cast<const f32x4*>(dr), d1 = *reinterpret_cast<const f32x4*>(dr + 4),
              d2 = *reinterpret_cast<const f32x4*>(dr + 8);
  const float den = ((d0[0] + d0[1]) + (d0[2] + d0[3])) + ((d1[0] + d1[1]) + (d1[2] + d1[3])) +
                    ((d2[0] + d2[1]) + (d2[2] + d2[3]));
  const float rd = __builtin_amdgcn_rcpf(den);
  // staged in LDS: a lane's four columns are 8 bytes of one row, so direct
  // stores would leave every lane its own partial-line write
  uint16_t* orow = sO + (16 * IT + col) * K::LO + 32 * cg + 4 * g;
#pragma unroll
  for (int et = 0; et < 2; ++et)
    *reinterpret_cast<uint2*>(orow + 16 * et) =
        make_uint2(pack_bf16x2(r[et][0] * rd, r[et][1] * rd), pack_bf16x2(r[et][2] * rd, r[et][3] * rd));
  (void)fs;
}

template <class K>
__global__ __launch_bounds__(K::NT) void wout_kernel(WParams p) {
  extern __shared__ __align__(16) unsigned char lds[];
  uint16_t* sQ = reinterpret_cast<uint16_t*>(lds + K::oQ);
  uint16_t* sK = reinterpret_cast<uint16_t*>(lds + K::oK);
  uint16_t* sKt = reinterpret_cast<uint16_t*>(lds + K::oKt);
  uint16_t* sVt = reinterpret_cast<uint16_t*>(lds + K::oVt);
  uint16_t* sA = reinterpret_cast<uint16_t*>(lds + K::oA);
  float* sP = reinterpret_cast<float*>(lds + K::oP);
  float* sDen = reinterpret_cast<float*>(lds + K::oDen);
  uint16_t* sZb = reinterpret_cast<uint16_t*>(lds + K::oZ);  // bf16 copy of z (denominators)
  uint16_t* sO = reinterpret_cast<uint16_t*>(lds + K::oO);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, col = lane & 15;
  const int cg = wave % K::NCG, fs = wave / K::NCG;
  const int64_t item = blockIdx.x;
  const int64_t h = item / p.n_seg;
  const int seg = (int)(item - h * p.n_seg);
  const int64_t t0 = (int64_t)seg * p.seg_len;
  const int64_t t1 = (t0 + p.seg_len < p.L) ? t0 + p.seg_len : p.L;
  const int n_chunks = (int)((t1 - t0 + K::C - 1) / K::C);
  const int64_t hrow = h * p.L;
  const int zf = wave * K::ZPW + lane;

  // the segment's prefix state
  const float* st = p.states + item * (int64_t)(K::F / 16) * K::NE * 256;
  f32x4 acc[K::NFT][2];
#pragma unroll
  for (int ft = 0; ft < K::NFT; ++ft)
#pragma unroll
    for (int et = 0; et < 2; ++et)
      acc[ft][et] = *reinterpret_cast<const f32x4*>(st + ((fs * K::NFT + ft) * K::NE + 2 * cg + et) * 256 + lane * 4);
  float zreg = 0.f;
  if (lane < K::ZPW) {
    zreg = st[((zf >> 4) * K::NE + K::NE - 1) * 256 + 64 * ((zf & 15) >> 2) + (zf & 3)];
    sZb[zf] = f32_to_bf16(zreg);
  }
  for (int x = tid; x < K::C * K::LA / 2; x += K::NT) reinterpret_cast<uint32_t*>(sA)[x] = 0u;
  for (int x = tid; x < K::C * K::LD; x += K::NT) sDen[x] = 0.f;

  WPref<K> pf;
  w_load<K, true>(p, hrow + t0, (int)((t1 - t0) < K::C ? (t1 - t0) : K::C), tid, pf);
  w_store<K, true>(sQ, sK, sKt, sVt, tid, pf);
  __syncthreads();

  for (int c = 0; c < n_chunks; ++c) {
    const int64_t r0 = t0 + (int64_t)c * K::C;
    const bool more = c + 1 < n_chunks;
    if (more) {
      const int64_t left = t1 - r0 - K::C;
      w_load<K, true>(p, hrow + r0 + K::C, (int)(left < K::C ? left : K::C), tid, pf);
    }

    // ---- phase 1: everything that reads the staged chunk ----
    if (wave < 3) {  // causal tiles of A^T: (jt, it) = (0,0), (0,1), (1,1)
      const int jt = wave == 2 ? 1 : 0, it = wave == 0 ? 0 : 1;
      const uint16_t* ak = sK + (16 * jt + col) * K::LQ + 8 * g;
      const uint16_t* bq = sQ + (16 * it + col) * K::LQ + 8 * g;
      f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < K::F / 32; ++ks) t = mfma_bf16(ld8w(ak + 32 * ks), ld8w(bq + 32 * ks), t);
      // lane holds A^T[j = 16jt + 4g + ii][i = 16it + col]; mask j > i, round to bf16
      float a[4];
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) a[ii] = (jt == it && 4 * g + ii > col) ? 0.f : t[ii];
      const uint32_t w01 = pack_bf16x2(a[0], a[1]), w23 = pack_bf16x2(a[2], a[3]);
      *reinterpret_cast<uint2*>(sA + (16 * it + col) * K::LA + 16 * jt + 4 * g) = make_uint2(w01, w23);
      float rs = (lo_f(w01) + hi_f(w01)) + (lo_f(w23) + hi_f(w23));
      rs += __shfl_xor(rs, 16, 64);
      rs += __shfl_xor(rs, 32, 64);
      if (g == 0) sDen[(16 * it + col) * K::LD + 8 + jt] = rs;
    }
    {  // this wave's part of phi(q_i) . z for all 32 tokens (z before the chunk)
      const int i = lane & 31, hf = lane >> 5;
      const int f0 = wave * K::ZPW + hf * (K::ZPW / 2);
      const uint16_t* qr = sQ + i * K::LQ + f0;
      float d0 = 0.f, d1 = 0.f;
#pragma unroll
      for (int x = 0; x < K::ZPW / 2; x += 8) {
        const uint4 qv = *reinterpret_cast<const uint4*>(qr + x);
        const uint4 zv = *reinterpret_cast<const uint4*>(sZb + f0 + x);
        d0 = dot2(qv.x, zv.x, d0);
        d1 = dot2(qv.y, zv.y, d1);
        d0 = dot2(qv.z, zv.z, d0);
        d1 = dot2(qv.w, zv.w, d1);
      }
      float d = d0 + d1;
      d += __shfl_xor(d, 32, 64);
      if (hf == 0) sDen[i * K::LD + wave] = d;
    }
    w_zupdate<K>(sKt, sZb, zf, lane, zreg);

    // partial num^T = S^T phi(Q)^T over the wave's features
    f32x4 num[2][2];
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
      for (int et = 0; et < 2; ++et) num[it][et] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < K::NKS; ++ks) {
      bf16x8 aop[2];
#pragma unroll
      for (int et = 0; et < 2; ++et) {
        const f32x4 u = acc[2 * ks][et], w = acc[2 * ks + 1][et];
        aop[et] = as_bf16x8(make_uint4(pack_bf16x2(u[0], u[1]), pack_bf16x2(u[2], u[3]), pack_bf16x2(w[0], w[1]),
                                       pack_bf16x2(w[2], w[3])));
      }
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        const uint16_t* qr = sQ + (16 * it + col) * K::LQ + fs * K::FS + 32 * ks + 4 * g;
        const uint2 lo = *reinterpret_cast<const uint2*>(qr);
        const uint2 hi = *reinterpret_cast<const uint2*>(qr + 16);
        const bf16x8 bq = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
#pragma unroll
        for (int et = 0; et < 2; ++et) num[it][et] = mfma_bf16(aop[et], bq, num[it][et]);
      }
    }
    uint4 bv[2];
    w_update<K>(sKt, sVt, cg, fs, lane, acc, bv);
    // hand the other token tiles' partials to their output waves
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      if (it == fs) continue;
      const int slot = fs < it ? fs : fs - 1;
#pragma unroll
      for (int et = 0; et < 2; ++et)
        *reinterpret_cast<f32x4*>(sP + ((((cg * 2 + it) * K::NSLOT + slot) * 2 + et) * 64 + lane) * 4) = num[it][et];
    }
    __syncthreads();

    // ---- phase 2: finish token tile fs (waves with fs < 2), stage the next chunk ----
    // (a branch per tile keeps num[] in registers: indexing it with the
    // runtime fs would move it to scratch memory)
    if (fs == 0)
      w_finish<K, 0>(sP, sA, sDen, sO, cg, fs, lane, num[0], bv);
    else if (fs == 1)
      w_finish<K, 1>(sP, sA, sDen, sO, cg, fs, lane, num[1], bv);
    if (more) w_store<K, true>(sQ, sK, sKt, sVt, tid, pf);
    // Loads and stores retire in issue order and share one counter: with the
    // prefetch known complete here, the next chunk's prefetch does not wait
    // for the output stores below.
    wait_vmem();
    __syncthreads();
    // whole output rows of the chunk, 16 bytes per thread (read before the
    // next chunk's phase 2 writes the staging rows again)
    if (tid < K::C * K::DV / 8) {
      const int rr = tid / (K::DV / 8), pc = tid % (K::DV / 8);
      if (r0 + rr < t1)
        *reinterpret_cast<uint4*>(p.o + (hrow + r0 + rr) * K::DV + 8 * pc) =
            *reinterpret_cast<const uint4*>(sO + rr * K::LO + 8 * pc);
    }
  }

  if (seg == p.n_seg - 1) {  // final state of the head
    if (p.S_out) {
#pragma unroll
      for (int ft = 0; ft < K::NFT; ++ft)
#pragma unroll
        for (int et = 0; et < 2; ++et)
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            const int f = fs * K::FS + 16 * ft + 4 * g + ii, e = 32 * cg + 16 * et + col;
            p.S_out[(h * K::F + f) * K::DV + e] = acc[ft][et][ii];
          }
    }
    if (p.z_out && lane < K::ZPW) p.z_out[h * K::F + zf] = zreg;
  }
}

// Segments: about one workgroup per CU over the whole batch (the output and
// state passes hold one workgroup per CU), whole chunks each.
int64_t w_seg_len(int64_t n_heads, int64_t L) {
  constexpr int64_t kTargetGroups = 256;
  int64_t s = (n_heads * L + kTargetGroups - 1) / kTargetGroups;
  s = (s + 31) / 32 * 32;
  return s < 32 ? 32 : s;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

template <class K>
size_t w_ws_bytes(const ChunkedArgs& a) {
  if (a.L == 0 || a.n_heads == 0) return 0;
  const int64_t seg = w_seg_len(a.n_heads, a.L);
  const int64_t n_seg = (a.L + seg - 1) / seg;
  const size_t phi = align256((size_t)a.n_heads * a.L * K::F * 2);
  return 2 * phi + sizeof(float) * (size_t)a.n_heads * n_seg * K::F * K::NE * 16;
}

template <class K>
hipError_t w_launch(const ChunkedArgs& a, hipStream_t s) {
  const int64_t seg = w_seg_len(a.n_heads, a.L);
  const int64_t n_seg = (a.L + seg - 1) / seg;
  const size_t phi = align256((size_t)a.n_heads * a.L * K::F * 2);
  uint16_t* phiq = static_cast<uint16_t*>(a.ws);
  uint16_t* phik = reinterpret_cast<uint16_t*>(static_cast<unsigned char*>(a.ws) + phi);
  float* states = reinterpret_cast<float*>(static_cast<unsigned char*>(a.ws) + 2 * phi);

  FeatmapArgs fa{};
  fa.x = a.q;
  fa.x2 = a.k;
  fa.rows_per_head = a.L;
  fa.n_heads = a.n_heads;
  fa.d = a.d;
  fa.F = a.F;
  fa.m = a.m;
  fa.x_bf16 = true;
  fa.anchors = a.anchors;
  fa.prf = a.prf;
  fa.draw_set_stride = a.draw_set_stride;
  fa.n_draw_sets = a.n_draw_sets;
  fa.nc = a.nc;
  fa.phi = phiq;
  fa.phi2 = phik;
  fa.phi_bf16 = true;
  hipError_t e = launch_featmap(fa, s);
  if (e != hipSuccess) return e;

  WParams p{};
  p.phiq = phiq;
  p.phik = phik;
  p.v = static_cast<const uint16_t*>(a.v);
  p.o = static_cast<uint16_t*>(a.o);
  p.states = states;
  p.L = a.L;
  p.seg_len = seg;
  p.n_seg = (int)n_seg;
  p.S_out = a.S_out;
  p.z_out = a.z_out;
  if (n_seg > 1) {
    e = set_max_lds(reinterpret_cast<const void*>(&wstate_kernel<K>), K::kLds1);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(wstate_kernel<K>, dim3((unsigned)(a.n_heads * (n_seg - 1))), dim3(K::NT), K::kLds1, s, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  ScanArgs sa{};
  sa.states = states;
  sa.n_heads = a.n_heads;
  sa.n_items = n_seg;
  sa.n_terms = n_seg - 1;
  sa.F = K::F;
  sa.dv = K::DV;
  sa.layout = 1;
  sa.S0 = a.S0;
  sa.z0 = a.z0;
  e = launch_scan(sa, s);
  if (e != hipSuccess) return e;
  e = set_max_lds(reinterpret_cast<const void*>(&wout_kernel<K>), K::kLds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(wout_kernel<K>, dim3((unsigned)(a.n_heads * n_seg)), dim3(K::NT), K::kLds, s, p);
  return hipGetLastError();
}

template <typename Fn>
bool w_dispatch(const ChunkedArgs& a, Fn&& fn) {
  if (!a.causal || !a.io_bf16 || !featmap_supported(a.d) || a.m % 16 != 0) return false;
  if (a.chunk % 32 != 0 || a.chunk > 128) return false;
  if (a.dv == 128) {
    switch (a.F) {
      case 128: fn(WCfg<128, 128>()); return true;
      case 256: fn(WCfg<256, 128>()); return true;
      case 384: fn(WCfg<384, 128>()); return true;
      case 512: fn(WCfg<512, 128>()); return true;
      default: return false;
    }
  }
  if (a.dv == 64) {
    switch (a.F) {
      case 128: fn(WCfg<128, 64>()); return true;
      case 256: fn(WCfg<256, 64>()); return true;
      case 384: fn(WCfg<384, 64>()); return true;
      case 512: fn(WCfg<512, 64>()); return true;
      default: return false;
    }
  }
  return false;
}

}  // namespace

bool wide_supported(const ChunkedArgs& a) {
  return w_dispatch(a, [](auto) {});
}

size_t wide_workspace_bytes(const ChunkedArgs& a) {
  size_t r = 0;
  w_dispatch(a, [&](auto k) { r = w_ws_bytes<decltype(k)>(a); });
  return r;
}

hipError_t launch_wide(const ChunkedArgs& a, hipStream_t s) {
  if (a.n_heads == 0 || a.L == 0) return launch_generic(a, s);  // only the state passes through
  hipError_t e = hipErrorInvalidValue;
  w_dispatch(a, [&](auto k) { e = w_launch<decltype(k)>(a, s); });
  return e;
}

}  // namespace slay
