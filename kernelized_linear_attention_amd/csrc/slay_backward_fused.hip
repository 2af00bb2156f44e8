// slay_backward_fused.hip -- MFMA backward of the causal SLAY forward (bf16,
// d = dv = 64, F = 256).
//
// The forward ("SLAY: Geometry-Aware Spherical Linearized Attention with
// Yat-Kernel", abstract; nubint.ai review, "Proposed method" bullets 1-6)
// differentiated, with v'_j = [v_j | 1 | 0..], S' = [S | z | 0..] (80 columns)
// and g'_i = [dout_i / den_i | h_i | 0..], h_i = -(dout_i . o_i) / den_i:
//   dphi(q_i) = S'_i g'_i,  dphi(k_j) = U_j v'_j,  dv_j = U_j[:, :dv]^T phi(k_j),
//   U_j = [dS_T | dz_T] + sum_{i>=j} phi(q_i) g'_i^T,  [dS0 | dz0] = U_0,
// then dq, dk through the feature map's Jacobian.
//
// Launches (one stream):
//   1. the feature map writes phi(q), phi(k) to the workspace in bf16;
//   2. the forward's segment-state pass and scan give S' before every segment;
//   3. bwd_q_kernel, one workgroup per (head, segment), walks the segment's
//      32-token chunks forward with S'^T in MFMA accumulators (each wave two
//      16-feature blocks) and a bf16 copy in LDS: the masked block
//      A = tril(phi(Q) phi(K)^T), num' = A V' + phi(Q) S', g', the masked block
//      D = tril(G' V'^T), dphi(Q) = D phi(K) + G' S'^T, the segment's
//      sum phi(Q)^T G' (written over its prefix state) and the state update;
//   4. the reverse scan of those sums from [dS_T | dz_T] gives U after every
//      segment, and its total [dS0 | dz0];
//   5. bwd_kv_kernel walks each segment's chunks backward with U^T in
//      accumulators: dphi(K) = D^T phi(Q) + V' U^T, dV = A^T G + phi(K) U,
//      then U += phi(Q)^T G';
//   6. vjp_kernel maps dphi back to dq and dk: y = P x (MFMA), the weights
//      w_a = dphi 2 y_a E / |x|, w_g = dphi phi sqrt(beta) from the epilogue,
//      dxh = P^T w (MFMA, the weights straight from the accumulators), then
//      dx = (dxh - xh (xh . dxh)) / |x|.
// Every MFMA operand comes from LDS tiles with rows padded to an odd multiple
// of 16 bytes, or from accumulators of an earlier MFMA: a 16x16 accumulator
// tile gives each lane four consecutive rows of one column, so two tiles
// side by side are the eight consecutive k-values one lane feeds a 16x16x32
// MFMA, provided the other operand is read with the same k order.  All
// contractions use the one 16x16x32 bf16 shape, the 80-column ones as two full
// steps plus a tail step whose second half is zero.  (An earlier tail step in
// the 16x16x16 shape gave wrong results for a reason never established --
// possibly an operand-layout mistake in that code; the one shape whose lane
// layout is checked is used instead.)
#include "slay_device.hpp"
#include "slay_internal.hpp"

namespace slay {

namespace {

__device__ __forceinline__ bf16x8 ld8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}
// four values then four zeros: the 16-column tail block (columns 64..79) of
// an 80-column contraction as one 16x16x32 step whose other half is zero
__device__ __forceinline__ bf16x8 ld4z(const uint16_t* p) {
  const uint2 a = *reinterpret_cast<const uint2*>(p);
  return __builtin_bit_cast(bf16x8, make_uint4(a.x, a.y, 0u, 0u));
}
__device__ __forceinline__ bf16x8 ld4x2(const uint16_t* p0, const uint16_t* p1) {
  const uint2 a = *reinterpret_cast<const uint2*>(p0);
  const uint2 b = *reinterpret_cast<const uint2*>(p1);
  return __builtin_bit_cast(bf16x8, make_uint4(a.x, a.y, b.x, b.y));
}
__device__ __forceinline__ uint2 pk4(const f32x4& a) {
  return make_uint2(pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]));
}
// two accumulator tiles as one 8-wide operand: the first tile's four values, then the second's
__device__ __forceinline__ bf16x8 pk_pair(const f32x4& a, const f32x4& b) {
  const uint2 x = pk4(a), y = pk4(b);
  return __builtin_bit_cast(bf16x8, make_uint4(x.x, x.y, y.x, y.y));
}

constexpr f32x4 kZero4 = {0.f, 0.f, 0.f, 0.f};
constexpr uint16_t kOneBf16 = 0x3F80;

template <int NF_>
struct BwdK {
  static constexpr int NF = NF_;          // 16-feature blocks
  static constexpr int F = NF * 16;
  static constexpr int C = 32;            // tokens per chunk step
  static constexpr int NI = C / 16;       // 16-token blocks per chunk
  static constexpr int DV = 64;
  static constexpr int E = 80;            // [v | 1 | 0 ...] columns
  static constexpr int NE = E / 16;
  static constexpr int NA = NI * (NI + 1) / 2;  // causal 16x16 blocks of a C x C block
  static constexpr int NW = NF / 2;       // waves: two feature blocks each
  static constexpr int NT = NW * 64;
  // LDS row strides in elements (odd multiples of 16 bytes)
  static constexpr int LQ = F + 8, LT = C + 8, LV = E + 8, LS = F + 8, LA = C + 8, LN = E + 4;
  static constexpr int oQ = 0;                    // phi(Q) [C][LQ]
  static constexpr int oQT = oQ + C * LQ * 2;     // phi(Q)^T [F][LT]
  static constexpr int oK = oQT + F * LT * 2;     // phi(K) [C][LQ]
  static constexpr int oKT = oK + C * LQ * 2;     // phi(K)^T [F][LT]
  static constexpr int oV = oKT + F * LT * 2;     // V' [C][LV]
  static constexpr int oVT = oV + C * LV * 2;     // V'^T [E][LT]
  static constexpr int oS = oVT + E * LT * 2;     // bf16 S'^T or U^T [E][LS]
  static constexpr int oG = oS + E * LS * 2;      // G' [C][LV]
  static constexpr int oGT = oG + C * LV * 2;     // G'^T [E][LT]
  static constexpr int oA = oGT + E * LT * 2;     // masked A [C][LA] (bwd_q: A[i][j]; bwd_kv: A^T[j][i])
  static constexpr int oD = oA + C * LA * 2;      // masked D (bwd_q: D[i][j]; bwd_kv: D^T[j][i])
  static constexpr int oN = oD + C * LA * 2;      // fp32 [C][LN]: num' (bwd_q) or dV partials (bwd_kv)
  static constexpr int kLds = oN + C * LN * 4;
  static_assert(kLds <= 160 * 1024, "LDS budget");
  static_assert(NF % 2 == 0, "two feature blocks per wave");
  static_assert(NT == 512 && F == 256 && C == 32, "the staging maps 512 threads onto 32 x 256 tiles");
};

struct BwdParams {
  const uint16_t* phiq;  // [n_heads * L][F] bf16
  const uint16_t* phik;
  const uint16_t* v;     // [n_heads * L][64]
  const uint16_t* dout;  // [n_heads * L][64]
  int64_t L, seg_len;
  int n_seg;
  float* states;         // [n_heads][n_seg][F/16][NE][64][4]
  uint16_t* g;           // [n_heads * L][80]: [dout/den | h | 0 ...]
  uint16_t* dphiq;       // [n_heads * L][F]
  uint16_t* dphik;
  uint16_t* dv;          // [n_heads * L][64]
};

struct Lds {
  uint16_t *Q, *QT, *K, *KT, *V, *VT, *S, *G, *GT, *A, *D;
  float* N;
};

template <class K>
__device__ __forceinline__ Lds lds_of(char* base) {
  Lds l;
  l.Q = reinterpret_cast<uint16_t*>(base + K::oQ);
  l.QT = reinterpret_cast<uint16_t*>(base + K::oQT);
  l.K = reinterpret_cast<uint16_t*>(base + K::oK);
  l.KT = reinterpret_cast<uint16_t*>(base + K::oKT);
  l.V = reinterpret_cast<uint16_t*>(base + K::oV);
  l.VT = reinterpret_cast<uint16_t*>(base + K::oVT);
  l.S = reinterpret_cast<uint16_t*>(base + K::oS);
  l.G = reinterpret_cast<uint16_t*>(base + K::oG);
  l.GT = reinterpret_cast<uint16_t*>(base + K::oGT);
  l.A = reinterpret_cast<uint16_t*>(base + K::oA);
  l.D = reinterpret_cast<uint16_t*>(base + K::oD);
  l.N = reinterpret_cast<float*>(base + K::oN);
  return l;
}

// 8 bf16 of a uint4 written down a column of a transposed tile
__device__ __forceinline__ void scatter8(uint16_t* col, int stride, const uint4& x) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    col[(2 * t) * stride] = (uint16_t)(w[t] & 0xFFFFu);
    col[(2 * t + 1) * stride] = (uint16_t)(w[t] >> 16);
  }
}

// Regions no chunk writes stay zero: columns 65..79 of V', G' (rows of their
// transposes) and the blocks of the masked tiles above the diagonal.
template <class K>
__device__ void zero_constant_regions(const Lds& s, int tid) {
  for (int idx = tid; idx < K::C * 15; idx += K::NT) {
    const int r = idx / 15, e = 65 + idx % 15;
    s.V[r * K::LV + e] = 0;
    s.G[r * K::LV + e] = 0;
    s.VT[e * K::LT + r] = 0;
    s.GT[e * K::LT + r] = 0;
  }
  for (int idx = tid; idx < K::C * K::LA; idx += K::NT) {
    s.A[idx] = 0;
    s.D[idx] = 0;
  }
}

// Chunk staging, software-pipelined: the global loads of chunk c+1 are issued
// into registers right after chunk c is written to LDS, so they are in flight
// while chunk c is computed.  A thread moves one 4-row x 8-column block of a
// feature tile: four 16-byte row pieces, written as rows and, transposed in
// registers (v_perm), as eight 8-byte column pieces of the transposed tile.
__device__ __forceinline__ void transpose4x8(const uint4 (&in)[4], uint2 (&out)[8]) {
  const uint32_t w[4][4] = {{in[0].x, in[0].y, in[0].z, in[0].w},
                            {in[1].x, in[1].y, in[1].z, in[1].w},
                            {in[2].x, in[2].y, in[2].z, in[2].w},
                            {in[3].x, in[3].y, in[3].z, in[3].w}};
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    out[2 * u] = make_uint2(lo16_pair(w[0][u], w[1][u]), lo16_pair(w[2][u], w[3][u]));
    out[2 * u + 1] = make_uint2(hi16_pair(w[0][u], w[1][u]), hi16_pair(w[2][u], w[3][u]));
  }
}

__device__ __forceinline__ uint4 ld_row(const uint16_t* p, bool ok) {
  return ok ? *reinterpret_cast<const uint4*>(p) : make_uint4(0, 0, 0, 0);
}

// block u of a [C][width] tile: rows 4(u % 8) .. +3, columns 8(u / 8) .. +7
template <class K>
__device__ __forceinline__ void load_block(const uint16_t* src, int width, int64_t row0, int n, int u,
                                           uint4 (&blk)[4]) {
  const int r = 4 * (u & 7), c = 8 * (u >> 3);
#pragma unroll
  for (int t = 0; t < 4; ++t) blk[t] = ld_row(src + (row0 + r + t) * width + c, r + t < n);
}

template <class K>
__device__ __forceinline__ void store_block(uint16_t* rows, int ld_rows, uint16_t* cols, int u, const uint4 (&blk)[4]) {
  const int r = 4 * (u & 7), c = 8 * (u >> 3);
#pragma unroll
  for (int t = 0; t < 4; ++t) *reinterpret_cast<uint4*>(rows + (r + t) * ld_rows + c) = blk[t];
  uint2 tr[8];
  transpose4x8(blk, tr);
#pragma unroll
  for (int t = 0; t < 8; ++t) *reinterpret_cast<uint2*>(cols + (c + t) * K::LT + r) = tr[t];
}

// the ones column of V' (and V'^T) counts the chunk's valid rows only
template <class K, bool TV>
__device__ __forceinline__ void store_ones(const Lds& s, int n, int tid) {
  for (int r = tid; r < K::C; r += K::NT) {
    const uint16_t one = r < n ? kOneBf16 : (uint16_t)0;
    s.V[r * K::LV + K::DV] = one;
    if (TV) s.VT[K::DV * K::LT + r] = one;
  }
}

// bwd_q: threads < 256 move a phi(Q) block, the others a phi(K) block; threads
// < 256 also one 16-byte piece of v (row t/8, columns 8(t%8)..) and of dout.
struct PrefQ {
  uint4 blk[4];
  uint4 v, dout;
};

template <class K>
__device__ __forceinline__ void load_q(const BwdParams& p, int64_t row0, int n, int tid, PrefQ& pf) {
  load_block<K>(tid < 256 ? p.phiq : p.phik, K::F, row0, n, tid & 255, pf.blk);
  const int r = (tid & 255) >> 3, c = 8 * (tid & 7);
  pf.v = ld_row(p.v + (row0 + r) * K::DV + c, tid < 256 && r < n);
  pf.dout = ld_row(p.dout + (row0 + r) * K::DV + c, tid < 256 && r < n);
}

template <class K>
__device__ __forceinline__ void store_q(const Lds& s, const PrefQ& pf, int n, int tid) {
  store_block<K>(tid < 256 ? s.Q : s.K, K::LQ, tid < 256 ? s.QT : s.KT, tid & 255, pf.blk);
  if (tid < 256) {
    const int r = tid >> 3, c = 8 * (tid & 7);
    *reinterpret_cast<uint4*>(s.V + r * K::LV + c) = pf.v;
    scatter8(s.VT + c * K::LT + r, K::LT, pf.v);
  }
  store_ones<K, true>(s, n, tid);
}

// bwd_kv: threads < 256 move a phi(Q) block (rows and transposed) and one
// piece of v; the others four row pieces of phi(K) and, for the first 80, a
// block of g' (rows and transposed).
struct PrefKV {
  uint4 blk[4];
  uint4 gb[4];
  uint4 v;
};

template <class K>
__device__ __forceinline__ void load_kv(const BwdParams& p, int64_t row0, int n, int tid, PrefKV& pf) {
  const int u = tid & 255;
  const bool lo = tid < 256;
  if (lo) {
    load_block<K>(p.phiq, K::F, row0, n, u, pf.blk);
  } else {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int idx = u + 256 * t, r = idx >> 5, c = 8 * (idx & 31);
      pf.blk[t] = ld_row(p.phik + (row0 + r) * K::F + c, r < n);
    }
  }
  const int r = u >> 3, c = 8 * (u & 7);
  pf.v = ld_row(p.v + (row0 + r) * K::DV + c, lo && r < n);
  // g' blocks on threads 256 .. 335 (80 blocks of 4 rows x 8 columns); the rest load nothing
  const bool gok = !lo && u < 8 * (K::E / 8);
  load_block<K>(p.g, K::E, row0, gok ? n : 0, gok ? u : 0, pf.gb);
}

template <class K>
__device__ __forceinline__ void store_kv(const Lds& s, const PrefKV& pf, int n, int tid) {
  if (tid < 256) {
    store_block<K>(s.Q, K::LQ, s.QT, tid, pf.blk);
    const int r = tid >> 3, c = 8 * (tid & 7);
    *reinterpret_cast<uint4*>(s.V + r * K::LV + c) = pf.v;
  } else {
    const int u = tid - 256;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int idx = u + 256 * t, r = idx >> 5, c = 8 * (idx & 31);
      *reinterpret_cast<uint4*>(s.K + r * K::LQ + c) = pf.blk[t];
    }
    if (u < 8 * (K::E / 8)) store_block<K>(s.G, K::LV, s.GT, u, pf.gb);
  }
  store_ones<K, false>(s, n, tid);
}

// Fragment-ordered state item: element (f, e) of tile (f/16, e/16) sits at
// lane (e%16) + 16((f%16)/4), slot f%4.  The transposed accumulator
// T[eb][j] (C[m = e][n = f], f in feature block fb = 2 wave + j) of this lane
// holds (f = fb*16 + l%16, e = eb*16 + 4(l/16) + r).
template <class K>
__device__ __forceinline__ int item_index(int fb, int eb, int g, int c16, int r) {
  return ((fb * K::NE + eb) * 64 + (4 * g + r) + 16 * (c16 >> 2)) * 4 + (c16 & 3);
}

// bf16 copy of the state, [e][f] rows.  Lanes l, l^1 hold features f, f+1
// of rows e..e+3: the even lane writes the (f, f+1) words of rows e, e+1, the
// odd lane those of e+2, e+3 (one 4-byte store per row instead of two 2-byte
// ones); v_perm takes bytes 0-3 from this lane's word, 4-7 from the neighbour's.
template <class K>
__device__ __forceinline__ void write_state_copy(const Lds& s, const f32x4 (&T)[K::NE][2], int wave, int g, int c16) {
  const bool odd = c16 & 1;
  const uint32_t sel0 = odd ? 0x01000504u : 0x05040100u;
  const uint32_t sel1 = odd ? 0x03020706u : 0x07060302u;
#pragma unroll
  for (int eb = 0; eb < K::NE; ++eb)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int fb = 2 * wave + j;
      const uint2 pk = pk4(T[eb][j]);
      const uint32_t mine = odd ? pk.y : pk.x;
      const uint32_t recv = swap_lane_pair(odd ? pk.x : pk.y);
      uint32_t* dst = reinterpret_cast<uint32_t*>(s.S + (eb * 16 + 4 * g + (odd ? 2 : 0)) * K::LS + fb * 16 + (c16 & ~1));
      dst[0] = __builtin_amdgcn_perm(recv, mine, sel0);
      dst[K::LS / 2] = __builtin_amdgcn_perm(recv, mine, sel1);
    }
}

// the causal 16x16 blocks (ib, jb), jb <= ib, in order (0,0), (1,0), (1,1), ...
__device__ __forceinline__ void causal_block(int it, int& ib, int& jb) {
  ib = 0;
  while ((ib + 1) * (ib + 2) / 2 <= it) ++ib;
  jb = it - ib * (ib + 1) / 2;
}

template <class K>
__global__ __launch_bounds__(K::NT) void bwd_q_kernel(BwdParams p) {
  extern __shared__ __align__(16) char lds_raw[];
  const Lds s = lds_of<K>(lds_raw);
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, c16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t h = blockIdx.x / p.n_seg;
  const int seg = (int)(blockIdx.x - h * p.n_seg);
  const int64_t t_begin = seg * p.seg_len;
  const int64_t t_end = min<int64_t>(p.L, t_begin + p.seg_len);
  float* item = p.states + (h * p.n_seg + seg) * (int64_t)(K::F * K::E);

  zero_constant_regions<K>(s, tid);
  f32x4 ST[K::NE][2], UT[K::NE][2];
#pragma unroll
  for (int eb = 0; eb < K::NE; ++eb)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int r = 0; r < 4; ++r) ST[eb][j][r] = item[item_index<K>(2 * wave + j, eb, g, c16, r)];
      UT[eb][j] = kZero4;
    }

  PrefQ pf;
  load_q<K>(p, h * p.L + t_begin, (int)min<int64_t>(K::C, t_end - t_begin), tid, pf);
  // Vector loads and stores retire in issue order and share one counter.  The
  // step loop starts with no load in flight and waits for its prefetch once,
  // before its own stores; a wait for the prefetch issued later would also
  // wait for the previous step's stores.
  wait_vmem();
  for (int64_t t0 = t_begin; t0 < t_end; t0 += K::C) {
    const int n = (int)min<int64_t>(K::C, t_end - t0);
    const int64_t row0 = h * p.L + t0;
    __syncthreads();
    // the state before this chunk, as the bf16 copy [1] reads (written here, a
    // phase after the update, so the update's MFMAs are done by now)
    write_state_copy<K>(s, ST, wave, g, c16);
    store_q<K>(s, pf, n, tid);
    const uint4 dcur = pf.dout;
    if (t0 + K::C < t_end) load_q<K>(p, row0 + K::C, (int)min<int64_t>(K::C, t_end - t0 - K::C), tid, pf);
    __syncthreads();
    // [1] A^T blocks (masked, to s.A as A[i][j]) and phi(Q) S' (to s.N as num'[i][e])
    for (int it = wave; it < K::NA + K::NI * K::NE; it += K::NW) {
      f32x4 acc = kZero4;
      if (it < K::NA) {
        int ib, jb;
        causal_block(it, ib, jb);
#pragma unroll
        for (int kk = 0; kk < K::F; kk += 32)
          acc = mfma_bf16(ld8(s.K + (jb * 16 + c16) * K::LQ + kk + 8 * g), ld8(s.Q + (ib * 16 + c16) * K::LQ + kk + 8 * g),
                          acc);
        const int i = ib * 16 + c16;
        f32x4 m;
#pragma unroll
        for (int r = 0; r < 4; ++r) m[r] = (jb * 16 + 4 * g + r <= i) ? acc[r] : 0.f;
        *reinterpret_cast<uint2*>(s.A + i * K::LA + jb * 16 + 4 * g) = pk4(m);
      } else {
        const int ib = (it - K::NA) / K::NE, eb = (it - K::NA) - ((it - K::NA) / K::NE) * K::NE;
#pragma unroll
        for (int kk = 0; kk < K::F; kk += 32)
          acc = mfma_bf16(ld8(s.S + (eb * 16 + c16) * K::LS + kk + 8 * g), ld8(s.Q + (ib * 16 + c16) * K::LQ + kk + 8 * g),
                          acc);
        *reinterpret_cast<f32x4*>(s.N + (ib * 16 + c16) * K::LN + eb * 16 + 4 * g) = acc;
      }
    }
    __syncthreads();
    // [2] num'^T += V'^T A^T over the chunk's keys
    for (int it = wave; it < K::NI * K::NE; it += K::NW) {
      const int ib = it / K::NE, eb = it - (it / K::NE) * K::NE;
      f32x4* pn = reinterpret_cast<f32x4*>(s.N + (ib * 16 + c16) * K::LN + eb * 16 + 4 * g);
      *pn = mfma_bf16(ld8(s.VT + (eb * 16 + c16) * K::LT + 8 * g), ld8(s.A + (ib * 16 + c16) * K::LA + 8 * g), *pn);
    }
    __syncthreads();
    wait_vmem();  // the next chunk's prefetch, before this step's stores
    // [3] g' = [dout / den | -(dout . num) / den^2 | 0]: eight threads per token
    static_assert(K::NT >= K::C * 8, "one pass: thread t holds the dout piece of token t/8");
    if (tid < K::C * 8) {
      const int idx = tid;
      const int r = idx >> 3, e0 = (idx & 7) * 8;
      const uint4 dr = dcur;  // this thread's piece of dout, staged with the chunk
      const uint32_t dw[4] = {dr.x, dr.y, dr.z, dr.w};
      float dn[8];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        dn[2 * t] = __uint_as_float(dw[t] << 16);
        dn[2 * t + 1] = __uint_as_float(dw[t] & 0xFFFF0000u);
      }
      const float* nr = s.N + r * K::LN;
      float dot = 0.f;
#pragma unroll
      for (int t = 0; t < 8; ++t) dot = fmaf(dn[t], nr[e0 + t], dot);
      dot += __shfl_xor(dot, 1, 64);
      dot += __shfl_xor(dot, 2, 64);
      dot += __shfl_xor(dot, 4, 64);
      const float inv = r < n ? 1.f / nr[K::DV] : 0.f;
      uint4 gv;
      gv.x = pack_bf16x2(dn[0] * inv, dn[1] * inv);
      gv.y = pack_bf16x2(dn[2] * inv, dn[3] * inv);
      gv.z = pack_bf16x2(dn[4] * inv, dn[5] * inv);
      gv.w = pack_bf16x2(dn[6] * inv, dn[7] * inv);
      *reinterpret_cast<uint4*>(s.G + r * K::LV + e0) = gv;
      scatter8(s.GT + e0 * K::LT + r, K::LT, gv);
      if (r < n) *reinterpret_cast<uint4*>(p.g + (row0 + r) * K::E + e0) = gv;
      if ((idx & 7) == 0) {
        const uint16_t hb = f32_to_bf16(-dot * inv * inv);
        s.G[r * K::LV + K::DV] = hb;
        s.GT[K::DV * K::LT + r] = hb;
        if (r < n) {
          *reinterpret_cast<uint4*>(p.g + (row0 + r) * K::E + K::DV) = make_uint4(hb, 0, 0, 0);
          *reinterpret_cast<uint4*>(p.g + (row0 + r) * K::E + K::DV + 8) = make_uint4(0, 0, 0, 0);
        }
      }
    }
    __syncthreads();
    // [4] D (masked, to s.D as D[i][j]); dphi(Q)^T = S' G'^T; sum phi(Q)^T G'; S' += phi(K)^T V'
    for (int it = wave; it < K::NA; it += K::NW) {
      int ib, jb;
      causal_block(it, ib, jb);
      const uint16_t* vr = s.V + (jb * 16 + c16) * K::LV;
      const uint16_t* gr = s.G + (ib * 16 + c16) * K::LV;
      f32x4 acc = mfma_bf16(ld8(vr + 8 * g), ld8(gr + 8 * g), kZero4);
      acc = mfma_bf16(ld8(vr + 32 + 8 * g), ld8(gr + 32 + 8 * g), acc);
      acc = mfma_bf16(ld4z(vr + 64 + 4 * g), ld4z(gr + 64 + 4 * g), acc);
      const int i = ib * 16 + c16;
      f32x4 m;
#pragma unroll
      for (int r = 0; r < 4; ++r) m[r] = (jb * 16 + 4 * g + r <= i) ? acc[r] : 0.f;
      *reinterpret_cast<uint2*>(s.D + i * K::LA + jb * 16 + 4 * g) = pk4(m);
    }
    f32x4 DQ[2][K::NI];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const bf16x8 a01 = pk_pair(ST[0][j], ST[1][j]);
      const bf16x8 a23 = pk_pair(ST[2][j], ST[3][j]);
      const bf16x8 a4 = pk_pair(ST[4][j], kZero4);
#pragma unroll
      for (int ib = 0; ib < K::NI; ++ib) {
        const uint16_t* gr = s.G + (ib * 16 + c16) * K::LV + 4 * g;
        f32x4 acc = mfma_bf16(a01, ld4x2(gr, gr + 16), kZero4);
        acc = mfma_bf16(a23, ld4x2(gr + 32, gr + 48), acc);
        DQ[j][ib] = mfma_bf16(a4, ld4z(gr + 64), acc);
      }
    }
#pragma unroll
    for (int eb = 0; eb < K::NE; ++eb) {
      const bf16x8 gt = ld8(s.GT + (eb * 16 + c16) * K::LT + 8 * g);
      const bf16x8 vt = ld8(s.VT + (eb * 16 + c16) * K::LT + 8 * g);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int fb = 2 * wave + j;
        UT[eb][j] = mfma_bf16(gt, ld8(s.QT + (fb * 16 + c16) * K::LT + 8 * g), UT[eb][j]);
        ST[eb][j] = mfma_bf16(vt, ld8(s.KT + (fb * 16 + c16) * K::LT + 8 * g), ST[eb][j]);
      }
    }
    __syncthreads();
    // [5] dphi(Q)^T += phi(K)^T D^T; write dphi(Q)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int fb = 2 * wave + j;
      const bf16x8 kt = ld8(s.KT + (fb * 16 + c16) * K::LT + 8 * g);
#pragma unroll
      for (int ib = 0; ib < K::NI; ++ib) {
        const f32x4 acc = mfma_bf16(kt, ld8(s.D + (ib * 16 + c16) * K::LA + 8 * g), DQ[j][ib]);
        const int i = ib * 16 + c16;
        if (i < n) *reinterpret_cast<uint2*>(p.dphiq + (row0 + i) * K::F + fb * 16 + 4 * g) = pk4(acc);
      }
    }
  }
  // the segment's sum of phi(Q)^T G' replaces its (consumed) prefix state
#pragma unroll
  for (int eb = 0; eb < K::NE; ++eb)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) item[item_index<K>(2 * wave + j, eb, g, c16, r)] = UT[eb][j][r];
}

template <class K>
__global__ __launch_bounds__(K::NT) void bwd_kv_kernel(BwdParams p) {
  extern __shared__ __align__(16) char lds_raw[];
  const Lds s = lds_of<K>(lds_raw);
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, c16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t h = blockIdx.x / p.n_seg;
  const int seg = (int)(blockIdx.x - h * p.n_seg);
  const int64_t t_begin = seg * p.seg_len;
  const int64_t t_end = min<int64_t>(p.L, t_begin + p.seg_len);
  const float* item = p.states + (h * p.n_seg + seg) * (int64_t)(K::F * K::E);

  zero_constant_regions<K>(s, tid);
  f32x4 UT[K::NE][2];
#pragma unroll
  for (int eb = 0; eb < K::NE; ++eb)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) UT[eb][j][r] = item[item_index<K>(2 * wave + j, eb, g, c16, r)];

  const int n_steps = (int)((t_end - t_begin + K::C - 1) / K::C);
  auto rows_of = [&](int cs) { return (int)min<int64_t>(K::C, t_end - (t_begin + (int64_t)cs * K::C)); };
  PrefKV pf;
  load_kv<K>(p, h * p.L + t_begin + (int64_t)(n_steps - 1) * K::C, rows_of(n_steps - 1), tid, pf);
  wait_vmem();  // as in bwd_q_kernel: no load in flight when the step loop starts
  for (int cs = n_steps - 1; cs >= 0; --cs) {
    const int64_t t0 = t_begin + (int64_t)cs * K::C;
    const int n = rows_of(cs);
    const int64_t row0 = h * p.L + t0;
    __syncthreads();
    write_state_copy<K>(s, UT, wave, g, c16);  // U after this chunk, as the bf16 copy [1] reads
    store_kv<K>(s, pf, n, tid);
    if (cs > 0) load_kv<K>(p, row0 - K::C, K::C, tid, pf);
    __syncthreads();
    // [1] A^T and D^T (masked, as [j][i]); dV^T = U^T phi(K)^T (to s.N as [j][e])
    for (int it = wave; it < 2 * K::NA + (K::DV / 16) * K::NI; it += K::NW) {
      if (it < 2 * K::NA) {
        int ib, jb;
        causal_block(it % K::NA, ib, jb);
        f32x4 acc = kZero4;
        if (it < K::NA) {  // A[i][j] = phi(Q_i) . phi(K_j)
#pragma unroll
          for (int kk = 0; kk < K::F; kk += 32)
            acc = mfma_bf16(ld8(s.Q + (ib * 16 + c16) * K::LQ + kk + 8 * g),
                            ld8(s.K + (jb * 16 + c16) * K::LQ + kk + 8 * g), acc);
        } else {  // D[i][j] = g'_i . v'_j
          const uint16_t* gr = s.G + (ib * 16 + c16) * K::LV;
          const uint16_t* vr = s.V + (jb * 16 + c16) * K::LV;
          acc = mfma_bf16(ld8(gr + 8 * g), ld8(vr + 8 * g), acc);
          acc = mfma_bf16(ld8(gr + 32 + 8 * g), ld8(vr + 32 + 8 * g), acc);
          acc = mfma_bf16(ld4z(gr + 64 + 4 * g), ld4z(vr + 64 + 4 * g), acc);
        }
        // acc[r] = X[i = ib*16 + 4g + r][j = jb*16 + l%16] -> [j][i], masked i >= j
        const int j = jb * 16 + c16;
        f32x4 m;
#pragma unroll
        for (int r = 0; r < 4; ++r) m[r] = (ib * 16 + 4 * g + r >= j) ? acc[r] : 0.f;
        uint16_t* dst = it < K::NA ? s.A : s.D;
        *reinterpret_cast<uint2*>(dst + j * K::LA + ib * 16 + 4 * g) = pk4(m);
      } else {
        const int k2 = it - 2 * K::NA;
        const int eb = k2 / K::NI, jb = k2 - (k2 / K::NI) * K::NI;
        f32x4 acc = kZero4;
#pragma unroll
        for (int kk = 0; kk < K::F; kk += 32)
          acc = mfma_bf16(ld8(s.S + (eb * 16 + c16) * K::LS + kk + 8 * g), ld8(s.K + (jb * 16 + c16) * K::LQ + kk + 8 * g),
                          acc);
        *reinterpret_cast<f32x4*>(s.N + (jb * 16 + c16) * K::LN + eb * 16 + 4 * g) = acc;
      }
    }
    // dphi(K)^T = U V'^T for own feature blocks
    f32x4 DK[2][K::NI];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const bf16x8 a01 = pk_pair(UT[0][j], UT[1][j]);
      const bf16x8 a23 = pk_pair(UT[2][j], UT[3][j]);
      const bf16x8 a4 = pk_pair(UT[4][j], kZero4);
#pragma unroll
      for (int jb = 0; jb < K::NI; ++jb) {
        const uint16_t* vr = s.V + (jb * 16 + c16) * K::LV + 4 * g;
        f32x4 acc = mfma_bf16(a01, ld4x2(vr, vr + 16), kZero4);
        acc = mfma_bf16(a23, ld4x2(vr + 32, vr + 48), acc);
        DK[j][jb] = mfma_bf16(a4, ld4z(vr + 64), acc);
      }
    }
    __syncthreads();
    wait_vmem();  // the next chunk's prefetch, before this step's stores
    // [2] dphi(K)^T += phi(Q)^T D; dV^T += G^T A; U^T += G'^T phi(Q)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int fb = 2 * wave + j;
      const bf16x8 qt = ld8(s.QT + (fb * 16 + c16) * K::LT + 8 * g);
#pragma unroll
      for (int jb = 0; jb < K::NI; ++jb) {
        const f32x4 acc = mfma_bf16(qt, ld8(s.D + (jb * 16 + c16) * K::LA + 8 * g), DK[j][jb]);
        const int jj = jb * 16 + c16;
        if (jj < n) *reinterpret_cast<uint2*>(p.dphik + (row0 + jj) * K::F + fb * 16 + 4 * g) = pk4(acc);
      }
    }
    for (int it = wave; it < (K::DV / 16) * K::NI; it += K::NW) {
      const int eb = it / K::NI, jb = it - (it / K::NI) * K::NI;
      const f32x4 part = *reinterpret_cast<const f32x4*>(s.N + (jb * 16 + c16) * K::LN + eb * 16 + 4 * g);
      const f32x4 acc = mfma_bf16(ld8(s.GT + (eb * 16 + c16) * K::LT + 8 * g), ld8(s.A + (jb * 16 + c16) * K::LA + 8 * g),
                                  part);
      const int jj = jb * 16 + c16;
      if (jj < n) *reinterpret_cast<uint2*>(p.dv + (row0 + jj) * K::DV + eb * 16 + 4 * g) = pk4(acc);
    }
#pragma unroll
    for (int eb = 0; eb < K::NE; ++eb) {
      const bf16x8 gt = ld8(s.GT + (eb * 16 + c16) * K::LT + 8 * g);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        UT[eb][j] = mfma_bf16(gt, ld8(s.QT + ((2 * wave + j) * 16 + c16) * K::LT + 8 * g), UT[eb][j]);
    }
  }
}

// ---------------------------------------------------------------------------
// Feature-map VJP on MFMA.  Each wave owns two 16-feature blocks and keeps
// their rows of P = [anchors; prf] in registers, both as the A-operand of
// y^T = P x^T (rows f, 8 consecutive d per lane) and, transposed, as the
// A-operand of dxh^T = P^T w (rows d, the k order of the two accumulator tiles
// that hold w).  Per 32-row tile: x staged in LDS; every wave forms its
// features' y, the weights w and its partial dxh over those features into its
// own fp32 LDS tile; then, summing the waves' partials, the projection
// dx = (dxh - xh (xh . dxh)) / |x|, 16 lanes per row.  x and dphi of the
// next three tiles are in flight while the current one is computed.
template <int NF_>
struct VjpK {
  static constexpr int NF = NF_, F = NF * 16, D = 64;
  static constexpr int NW = NF / 2, NT = NW * 64;
  static constexpr int RT = 32, NRB = RT / 16;  // rows per tile
  static constexpr int LX = D + 8, LR = D + 4;
  // x tile, per-wave partials, 1/|x| per row (negative where |x| is clamped)
  static constexpr int oX = 0, oR = RT * LX * 2, oI = oR + NW * RT * LR * 4, kLds = oI + RT * 4;
  static_assert(NT >= RT * 8 && NT >= RT * 16, "one x piece and one output piece per thread");
};

struct VjpParams {
  const uint16_t* x[2];     // q, k [n_rows][64]
  const uint16_t* dphi[2];  // [n_rows][F]
  uint16_t* dx[2];
  int64_t n_rows, rows_per_head;
  int m, n_draw_sets;
  const uint16_t* anchors;
  const uint16_t* prf;
  int64_t draw_set_stride;
  NodeConsts nc;
};

template <class K>
struct VjpPref {
  uint4 x;                  // threads < 8 RT: row t/8, columns 8(t%8) ..
  uint2 dp[K::NRB][2];      // dphi of row 16 rb + l%16, features 16 fb_j + 4(l/16) ..
};

template <class K>
__device__ __forceinline__ void vjp_load(const uint16_t* __restrict__ x, const uint16_t* __restrict__ dphi,
                                         int64_t n_rows, int64_t r0, int tid, int wave, int g, int c16,
                                         VjpPref<K>& pf) {
  const int64_t xr = r0 + (tid >> 3);
  pf.x = (tid < K::RT * 8 && xr < n_rows) ? *reinterpret_cast<const uint4*>(x + xr * K::D + 8 * (tid & 7))
                                          : make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int rb = 0; rb < K::NRB; ++rb) {
    const int64_t row = r0 + rb * 16 + c16;
#pragma unroll
    for (int j = 0; j < 2; ++j)
      pf.dp[rb][j] = row < n_rows
                         ? *reinterpret_cast<const uint2*>(dphi + row * K::F + (2 * wave + j) * 16 + 4 * g)
                         : make_uint2(0, 0);
  }
}

template <class K>
__global__ __launch_bounds__(K::NT) void vjp_kernel(VjpParams p) {
  extern __shared__ __align__(16) char lds_raw[];
  uint16_t* sX = reinterpret_cast<uint16_t*>(lds_raw + K::oX);
  float* sR = reinterpret_cast<float*>(lds_raw + K::oR);
  float* sI = reinterpret_cast<float*>(lds_raw + K::oI);
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, c16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int side = blockIdx.y;
  const uint16_t* __restrict__ x = p.x[side];
  const uint16_t* __restrict__ dphi = p.dphi[side];
  uint16_t* __restrict__ dx = p.dx[side];
  const int64_t n_tiles = (p.n_rows + K::RT - 1) / K::RT;

  bf16x8 pa[2][2], pg[2][2], pt[2][K::D / 16];
  float c1[2], c0[2], sb[2];
  int set = -1;
  // The next tile's rows are loaded while this one is computed.  Vector loads
  // and stores retire in issue order and share one counter, so the loop
  // starts with no load in flight and waits for the prefetch once, before
  // the tile's stores: a deeper prefetch (or one rotated through registers)
  // would make each wait for it also wait for the stores issued since.
  VjpPref<K> pf;
  const int64_t gs = gridDim.x;
  auto load_tile = [&](int64_t t, VjpPref<K>& dst) {
    if (t < n_tiles) vjp_load<K>(x, dphi, p.n_rows, t * K::RT, tid, wave, g, c16, dst);
  };
  load_tile(blockIdx.x, pf);
  wait_vmem();
  for (int64_t tile = blockIdx.x; tile < n_tiles; tile += gs) {
    const int64_t r0 = tile * K::RT;
    const int tset = (int)((r0 / p.rows_per_head) % p.n_draw_sets);  // a tile never spans two draw sets
    if (tset != set) {  // this wave's rows of P, as both operands
      set = tset;
      const uint16_t* A = p.anchors + set * p.draw_set_stride;
      const uint16_t* G = p.prf + set * p.draw_set_stride;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int fb = 2 * wave + j;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          pa[j][kk] = ld8(A + (fb * 16 + c16) * K::D + kk * 32 + 8 * g);
          pg[j][kk] = ld8(G + (fb * 16 + c16) * K::D + kk * 32 + 8 * g);
        }
#pragma unroll
        for (int cb = 0; cb < K::D / 16; ++cb) {
          uint16_t e[8];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            e[i] = A[(fb * 16 + 4 * g + i) * K::D + cb * 16 + c16];
            e[4 + i] = G[(fb * 16 + 4 * g + i) * K::D + cb * 16 + c16];
          }
          pt[j][cb] = __builtin_bit_cast(bf16x8, make_uint4(e[0] | ((uint32_t)e[1] << 16), e[2] | ((uint32_t)e[3] << 16),
                                                            e[4] | ((uint32_t)e[5] << 16), e[6] | ((uint32_t)e[7] << 16)));
        }
        const int node = (fb * 16) / p.m;
        c1[j] = p.nc.c1[node];
        c0[j] = p.nc.c0[node];
        sb[j] = c1[j] * 0.6931471805599453f;  // sqrt(beta_r)
      }
      wait_vmem();  // here, where the reload is rare, rather than at the first use
    }
    __syncthreads();  // the previous tile's readers of sX and sR are done
    const VjpPref<K> cur = pf;
    load_tile(tile + gs, pf);
    if (tid < K::RT * 8) {  // x rows, and 1/|x| once per row (eight threads per row)
      *reinterpret_cast<uint4*>(sX + (tid >> 3) * K::LX + 8 * (tid & 7)) = cur.x;
      const uint32_t wds[4] = {cur.x.x, cur.x.y, cur.x.z, cur.x.w};
      float ss = 0.f;  // bf16 products are exact in fp32
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const bf16x2 h2 = __builtin_bit_cast(bf16x2, wds[t]);
        ss = __builtin_amdgcn_fdot2_f32_bf16(h2, h2, ss, false);
      }
      ss += __shfl_xor(ss, 1, 64);
      ss += __shfl_xor(ss, 2, 64);
      ss += __shfl_xor(ss, 4, 64);
      if ((tid & 7) == 0) sI[tid >> 3] = ss < 1e-24f ? -1e12f : __builtin_amdgcn_rsqf(ss);
    }
    __syncthreads();
#pragma unroll
    for (int rb = 0; rb < K::NRB; ++rb) {
      const bf16x8 xb0 = ld8(sX + (rb * 16 + c16) * K::LX + 8 * g);
      const bf16x8 xb1 = ld8(sX + (rb * 16 + c16) * K::LX + 32 + 8 * g);
      const float inv = fabsf(sI[rb * 16 + c16]);
      f32x4 dX[K::D / 16];
#pragma unroll
      for (int cb = 0; cb < K::D / 16; ++cb) dX[cb] = kZero4;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        // y[f = 16 fb + 4g + r][row 16 rb + l%16] for the anchors and the prf of the same four features
        f32x4 ya = mfma_bf16(pa[j][0], xb0, kZero4);
        ya = mfma_bf16(pa[j][1], xb1, ya);
        f32x4 yg = mfma_bf16(pg[j][0], xb0, kZero4);
        yg = mfma_bf16(pg[j][1], xb1, yg);
        const uint2 dr = cur.dp[rb][j];
        const float dp[4] = {__uint_as_float(dr.x << 16), __uint_as_float(dr.x & 0xFFFF0000u),
                             __uint_as_float(dr.y << 16), __uint_as_float(dr.y & 0xFFFF0000u)};
        // u = dphi * a * e: w_a = 2u, w_g = u a sqrt(beta)
        const float s1 = inv * c1[j];
        f32x4 wa, wg;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float a = ya[r] * inv;
          const float e = fast_exp2(fmaf(yg[r], s1, c0[j]));
          const float u = dp[r] * (a * e);
          wa[r] = u + u;
          wg[r] = (u * a) * sb[j];
        }
        const bf16x8 w = pk_pair(wa, wg);
#pragma unroll
        for (int cb = 0; cb < K::D / 16; ++cb) dX[cb] = mfma_bf16(pt[j][cb], w, dX[cb]);
      }
      // dX[cb][r] = this wave's part of dxh[row 16 rb + l%16][c = 16 cb + 4g + r]
#pragma unroll
      for (int cb = 0; cb < K::D / 16; ++cb)
        *reinterpret_cast<f32x4*>(sR + (wave * K::RT + rb * 16 + c16) * K::LR + cb * 16 + 4 * g) = dX[cb];
    }
    __syncthreads();
    wait_vmem();  // the next tile's prefetch, before this tile's stores
    if (tid < K::RT * 16) {  // 16 lanes per row, four columns each
      const int rr = tid >> 4, c = 4 * (tid & 15);
      const int64_t row = r0 + rr;
      const uint2 xr = *reinterpret_cast<const uint2*>(sX + rr * K::LX + c);
      const float xv[4] = {__uint_as_float(xr.x << 16), __uint_as_float(xr.x & 0xFFFF0000u),
                           __uint_as_float(xr.y << 16), __uint_as_float(xr.y & 0xFFFF0000u)};
      f32x4 dh = kZero4;
#pragma unroll
      for (int w = 0; w < K::NW; ++w) dh += *reinterpret_cast<const f32x4*>(sR + (w * K::RT + rr) * K::LR + c);
      float pr = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) pr = fmaf(xv[r], dh[r], pr);
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) pr += __shfl_xor(pr, o, 64);
      const float si = sI[rr];
      const bool clamp = si < 0.f;
      const float inv = fabsf(si);
      const float proj = clamp ? 0.f : pr * inv;  // xh . dxh
      f32x4 o;
#pragma unroll
      for (int r = 0; r < 4; ++r) o[r] = (dh[r] - xv[r] * inv * proj) * inv;
      if (row < p.n_rows) *reinterpret_cast<uint2*>(dx + row * K::D + c) = pk4(o);
    }
  }
}

// ---------------------------------------------------------------------------
using K256 = BwdK<16>;
using V256 = VjpK<16>;

struct FusedWs {
  uint16_t *phiq, *phik, *dphiq, *dphik, *g;
  float* states;
  size_t bytes;
};

FusedWs fused_ws(const BackwardArgs& a, int n_seg, void* base) {
  const int64_t rows = a.n_heads * a.L;
  const size_t nphi = (size_t)rows * a.F * 2;
  FusedWs w{};
  char* p = static_cast<char*>(base);
  size_t off = 0;
  auto take = [&](size_t b) {
    char* q = p ? p + off : nullptr;
    off += (b + 255) & ~(size_t)255;
    return q;
  };
  w.states = reinterpret_cast<float*>(take(sizeof(float) * (size_t)a.n_heads * n_seg * K256::F * K256::E));
  w.phiq = reinterpret_cast<uint16_t*>(take(nphi));
  w.phik = reinterpret_cast<uint16_t*>(take(nphi));
  w.dphiq = reinterpret_cast<uint16_t*>(take(nphi));
  w.dphik = reinterpret_cast<uint16_t*>(take(nphi));
  w.g = reinterpret_cast<uint16_t*>(take((size_t)rows * K256::E * 2));
  w.bytes = off;
  return w;
}

ChunkedArgs forward_args(const BackwardArgs& a) {
  ChunkedArgs c{};
  c.q = a.q;
  c.k = a.k;
  c.v = a.v;
  c.io_bf16 = a.io_bf16;
  c.causal = true;
  c.n_heads = a.n_heads;
  c.L = a.L;
  c.Lq = a.L;
  c.d = a.d;
  c.dv = a.dv;
  c.F = a.F;
  c.m = a.m;
  c.R = a.R;
  c.chunk = a.chunk;
  c.anchors = a.anchors;
  c.prf = a.prf;
  c.draw_set_stride = a.draw_set_stride;
  c.n_draw_sets = a.n_draw_sets;
  c.nc = a.nc;
  c.S0 = a.S0;
  c.z0 = a.z0;
  return c;
}

// Feature counts below 256 run the F = 256 kernels on zero-padded features:
// the draws get zero rows f >= F (so phi_f = 0 and every contraction with it
// vanishes, and the node constants beyond R are zero, so the feature map and
// its VJP stay finite there), the states and their gradients zero rows.
// Workspace of the padded call after the F = 256 one: padded draws and states.
struct PadWs {
  uint16_t *anchors, *prf;
  float *S0, *z0, *dS_T, *dz_T, *dS0, *dz0;
  size_t bytes;
};

PadWs pad_ws(const BackwardArgs& a, char* base) {
  PadWs w{};
  size_t off = 0;
  auto take = [&](size_t b) {
    char* q = base ? base + off : nullptr;
    off += (b + 255) & ~(size_t)255;
    return q;
  };
  const size_t nd = (size_t)a.n_draw_sets * K256::F * a.d * 2;
  const size_t ns = (size_t)a.n_heads * K256::F * a.dv * 4, nz = (size_t)a.n_heads * K256::F * 4;
  w.anchors = reinterpret_cast<uint16_t*>(take(nd));
  w.prf = reinterpret_cast<uint16_t*>(take(nd));
  w.S0 = reinterpret_cast<float*>(take(ns));
  w.z0 = reinterpret_cast<float*>(take(nz));
  w.dS_T = reinterpret_cast<float*>(take(ns));
  w.dz_T = reinterpret_cast<float*>(take(nz));
  w.dS0 = reinterpret_cast<float*>(take(ns));
  w.dz0 = reinterpret_cast<float*>(take(nz));
  w.bytes = off;
  return w;
}

BackwardArgs padded_args(const BackwardArgs& a) {
  BackwardArgs p = a;
  p.F = K256::F;
  return p;
}

}  // namespace

bool backward_fused_supported(const BackwardArgs& a) {
  if (a.n_heads == 0 || a.L == 0) return false;  // nothing for the MFMA kernels: the general launcher handles it
  // F < 256 runs on zero-padded features (a multiple of 32, as the m % 32 rule gives)
  if (!a.io_bf16 || a.d != 64 || a.dv != 64 || a.F > K256::F || a.F % 32 != 0 || a.chunk != 64 || a.m % 32 != 0)
    return false;
  if (a.n_draw_sets > 1 && a.L % V256::RT != 0) return false;  // a VJP tile must not span two draw sets
  int64_t seg_len = 0;
  return fused_segment_count(forward_args(padded_args(a)), &seg_len) > 0 && seg_len % K256::C == 0;
}

size_t backward_fused_workspace_bytes(const BackwardArgs& a) {
  if (a.n_heads == 0 || a.L == 0) return 0;
  const BackwardArgs ap = padded_args(a);
  int64_t seg_len = 0;
  const int n_seg = fused_segment_count(forward_args(ap), &seg_len);
  const size_t base = fused_ws(ap, n_seg, nullptr).bytes;
  return a.F == K256::F ? base : base + pad_ws(a, nullptr).bytes;
}

namespace {

hipError_t launch_backward_fused_256(const BackwardArgs& a, hipStream_t s) {
  const ChunkedArgs fa = forward_args(a);
  int64_t seg_len = 0;
  const int n_seg = fused_segment_count(fa, &seg_len);
  const FusedWs w = fused_ws(a, n_seg, a.ws);

  FeatmapArgs fm{};
  fm.x = a.q;
  fm.x2 = a.k;
  fm.rows_per_head = a.L;
  fm.n_heads = a.n_heads;
  fm.d = a.d;
  fm.F = a.F;
  fm.m = a.m;
  fm.x_bf16 = true;
  fm.anchors = a.anchors;
  fm.prf = a.prf;
  fm.draw_set_stride = a.draw_set_stride;
  fm.n_draw_sets = a.n_draw_sets;
  fm.nc = a.nc;
  fm.phi = w.phiq;
  fm.phi2 = w.phik;
  fm.phi_bf16 = true;
  hipError_t e = launch_featmap(fm, s);
  if (e != hipSuccess) return e;
  e = launch_segment_prefix(fa, w.states, s);
  if (e != hipSuccess) return e;

  BwdParams p{};
  p.phiq = w.phiq;
  p.phik = w.phik;
  p.v = static_cast<const uint16_t*>(a.v);
  p.dout = static_cast<const uint16_t*>(a.dout);
  p.L = a.L;
  p.seg_len = seg_len;
  p.n_seg = n_seg;
  p.states = w.states;
  p.g = w.g;
  p.dphiq = w.dphiq;
  p.dphik = w.dphik;
  p.dv = static_cast<uint16_t*>(a.dv_out);
  const dim3 grid((unsigned)(a.n_heads * n_seg));
  e = set_max_lds(reinterpret_cast<const void*>(&bwd_q_kernel<K256>), K256::kLds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_q_kernel<K256>, grid, dim3(K256::NT), K256::kLds, s, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  ScanArgs ra{};
  ra.states = w.states;
  ra.n_heads = a.n_heads;
  ra.n_items = n_seg;
  ra.n_terms = n_seg;
  ra.F = a.F;
  ra.dv = a.dv;
  ra.layout = 1;
  ra.S0 = a.dS_T;
  ra.z0 = a.dz_T;
  ra.S_out = a.dS0;
  ra.z_out = a.dz0;
  ra.reverse = true;
  e = launch_scan(ra, s);
  if (e != hipSuccess) return e;

  e = set_max_lds(reinterpret_cast<const void*>(&bwd_kv_kernel<K256>), K256::kLds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_kv_kernel<K256>, grid, dim3(K256::NT), K256::kLds, s, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  VjpParams vp{};
  vp.x[0] = static_cast<const uint16_t*>(a.q);
  vp.x[1] = static_cast<const uint16_t*>(a.k);
  vp.dphi[0] = w.dphiq;
  vp.dphi[1] = w.dphik;
  vp.dx[0] = static_cast<uint16_t*>(a.dq);
  vp.dx[1] = static_cast<uint16_t*>(a.dk);
  vp.n_rows = a.n_heads * a.L;
  vp.rows_per_head = a.L;
  vp.m = a.m;
  vp.n_draw_sets = a.n_draw_sets;
  vp.anchors = static_cast<const uint16_t*>(a.anchors);
  vp.prf = static_cast<const uint16_t*>(a.prf);
  vp.draw_set_stride = a.draw_set_stride;
  vp.nc = a.nc;
  e = set_max_lds(reinterpret_cast<const void*>(&vjp_kernel<V256>), V256::kLds);
  if (e != hipSuccess) return e;
  const int64_t n_tiles = (vp.n_rows + V256::RT - 1) / V256::RT;
  const unsigned gx = (unsigned)(n_tiles < 128 ? n_tiles : 128);  // one workgroup per CU over both sides
  hipLaunchKernelGGL(vjp_kernel<V256>, dim3(gx, 2), dim3(V256::NT), V256::kLds, s, vp);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_backward_fused(const BackwardArgs& a, hipStream_t s) {
  if (a.n_heads == 0 || a.L == 0) return launch_backward(a, s);  // only the state gradient passes through
  if (a.F == K256::F) return launch_backward_fused_256(a, s);
  BackwardArgs ap = padded_args(a);
  int64_t seg_len = 0;
  const int n_seg = fused_segment_count(forward_args(ap), &seg_len);
  const PadWs w = pad_ws(a, static_cast<char*>(a.ws) + fused_ws(ap, n_seg, nullptr).bytes);
  const int64_t nh = a.n_heads, F = a.F, P = K256::F, d = a.d, dv = a.dv;
  hipError_t e = pad_rows(w.anchors, static_cast<const uint16_t*>(a.anchors), a.n_draw_sets, F, P, d,
                                    a.draw_set_stride, P * d, s);
  if (e == hipSuccess)
    e = pad_rows(w.prf, static_cast<const uint16_t*>(a.prf), a.n_draw_sets, F, P, d, a.draw_set_stride,
                           P * d, s);
  if (e != hipSuccess) return e;
  ap.anchors = w.anchors;
  ap.prf = w.prf;
  ap.draw_set_stride = P * d;
  // padded inputs (read before anything is written: a gradient output may alias its input)
  struct In {
    const float* src;
    float* dst;
    int64_t row_elems;
    const float** slot;
  } ins[4] = {{a.S0, w.S0, dv, &ap.S0}, {a.z0, w.z0, 1, &ap.z0}, {a.dS_T, w.dS_T, dv, &ap.dS_T}, {a.dz_T, w.dz_T, 1, &ap.dz_T}};
  for (const In& in : ins) {
    if (!in.src) continue;
    e = pad_rows(in.dst, in.src, nh, F, P, in.row_elems, F * in.row_elems, P * in.row_elems, s);
    if (e != hipSuccess) return e;
    *in.slot = in.dst;
  }
  ap.dS0 = a.dS0 ? w.dS0 : nullptr;
  ap.dz0 = a.dz0 ? w.dz0 : nullptr;
  e = launch_backward_fused_256(ap, s);
  if (e != hipSuccess) return e;
  if (a.dS0) e = pad_rows(a.dS0, w.dS0, nh, F, F, dv, P * dv, F * dv, s);
  if (e == hipSuccess && a.dz0) e = pad_rows(a.dz0, w.dz0, nh, F, F, 1, P, F, s);
  return e;
}

}  // namespace slay
