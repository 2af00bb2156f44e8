// slay_backward_fused.hip -- MFMA backward of the causal SLAY forward (bf16
// inputs and gradients, d = dv = 64, F = 256; smaller F on zero-padded
// features).
//
// The forward ("SLAY: Geometry-Aware Spherical Linearized Attention with
// Yat-Kernel", abstract; nubint.ai review, "Proposed method" bullets 1-6)
// differentiated, with v'_j = [v_j | 1 | 0..], S' = [S | z | 0..] (80 columns)
// and g'_i = [dout_i / den_i | h_i | 0..], h_i = -(dout_i . o_i) / den_i:
//   dphi(q_i) = S'_i g'_i,  dphi(k_j) = U_j v'_j,  dv_j = U_j[:, :dv]^T phi(k_j),
//   U_j = [dS_T | dz_T] + sum_{i>=j} phi(q_i) g'_i^T,  [dS0 | dz0] = U_0,
// then dq, dk through the feature map's Jacobian.
//
// Precision.  The gradient with respect to q is a small difference of large
// terms: o_i depends on q_i only through how the scores of the i keys
// before it change, so dq_i shrinks roughly like 1/sqrt(i) next to the
// products S'_i g'_i it is formed from.  With bf16 operands (8 mantissa bits)
// in those products the per-row error of dq grows to tens of percent at
// L = 16384.  Every product that touches a state, g', phi or U therefore
// runs on split operands: x = x_hi + x_lo, both bf16, so the pair carries 16
// mantissa bits, and a product of two split values is taken as
// x_hi y_hi + x_lo y_hi + x_hi y_lo (fp32 accumulation).  phi(q), phi(k) are
// recomputed on chip in fp32 wherever a kernel needs them (the projection
// P x on MFMA, exact bf16 products), the states and U live in fp32 MFMA
// accumulators, g' is formed and stored in fp32, and the masked
// intra-chunk blocks A = tril(phi(Q) phi(K)^T) and D = tril(G' V'^T) are split
// too where they feed the numerators and dphi (A only in bf16 for dV, whose
// terms are all positive-weighted).  dphi leaves in bf16: its rounding does
// not meet the cancellation.
//
// Token contractions run 16 tokens per step on the 16x16x32 bf16 MFMA: a
// lane's eight k-slots hold four tokens' hi parts and the same four tokens'
// lo parts, against the other operand's value for those tokens twice, so one
// instruction applies a split operand exactly.  (The lane layouts of that
// shape, checked on gfx950, are in slay_device.hpp.)
//
// Launches (one stream), one workgroup of 8 waves per (head, segment), wave
// w owning features [32w, 32w + 32) and keeping their rows of the projection
// P = [anchors; prf] in registers, from which it forms phi of its features for
// each 16-token step:
//   1. pb_state_kernel sums each segment's phi(K)^T V' (all but the last);
//      the prefix scan turns them into S' before every segment (plus S0, z0);
//   2. pb_g_kernel walks each segment with S' in accumulators, forms the
//      numerators and denominators (per-wave partials over the wave's
//      features, summed through LDS) and writes g' in fp32;
//   3. pb_dq_kernel walks each segment again: dphi(Q) = D phi(K) + G' S'^T,
//      and the segment's sum phi(Q)^T G' (written over its prefix state);
//   4. the reverse scan gives U after every segment (plus dS_T, dz_T) and
//      [dS0 | dz0];
//   5. pb_dk_kernel walks each segment backward with U in accumulators:
//      dphi(K) = D^T phi(Q) + V' U^T, dV = A^T G + phi(K) U (per-wave partials
//      summed through LDS), then U += phi(Q)^T G';
//   6. vjp_kernel maps dphi back to dq and dk.
#include <algorithm>
#include <type_traits>

#include "slay_device.hpp"
#include "slay_internal.hpp"

namespace slay {

namespace {

__device__ __forceinline__ bf16x8 ld8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
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
constexpr uint2 kZero2 = {0u, 0u};

__device__ __forceinline__ bf16x8 cat(const uint2& a, const uint2& b) {
  return __builtin_bit_cast(bf16x8, make_uint4(a.x, a.y, b.x, b.y));
}
__device__ __forceinline__ f32x4 unpk4(const uint2& h) {
  f32x4 r;
  r[0] = __uint_as_float(h.x << 16);
  r[1] = __uint_as_float(h.x & 0xFFFF0000u);
  r[2] = __uint_as_float(h.y << 16);
  r[3] = __uint_as_float(h.y & 0xFFFF0000u);
  return r;
}
// x = hi + lo: hi the bf16 rounding of x, lo the bf16 rounding of the (exact) remainder
__device__ __forceinline__ void split4(const f32x4& x, uint2& hi, uint2& lo) {
  hi = pk4(x);
  lo = pk4(x - unpk4(hi));
}
// a split value as one operand: k-slots 0-3 the hi parts, 4-7 the lo parts
__device__ __forceinline__ bf16x8 hilo(const f32x4& x) {
  uint2 h, l;
  split4(x, h, l);
  return cat(h, l);
}

// ---------------------------------------------------------------------------
// Precise segment kernels.
constexpr int kT = 16;             // tokens per step
constexpr int kF = 256;            // features
constexpr int kE = 80;             // columns of v' and g' (dv + 1, padded to 16)
constexpr int kNE = kE / 16;
constexpr int kDV = 64;
constexpr int kW = 8, kNT = kW * 64;  // waves; wave w owns feature blocks 2w, 2w + 1
// LDS row strides in elements (odd multiples of 16 bytes)
// [e][t] tiles hold each group of four tokens twice (v', g' hi) or once and then four zeros (g' lo), so that
// one 16-byte read gives a lane its whole operand: four tokens against the split other side's hi and lo parts
// (or, with the zeros, against its hi parts alone).  80-byte rows: at 96 bytes (which keeps the 16-byte
// reads apart in banks) the staging stores, whose rows lie 8 apart, collide, and the backward measured
// 843 against 831 us; 64-byte rows 888 us, 112- and 144-byte rows no better than 80.
constexpr int kLD = 40;
// [t][e] tiles ("row tiles") keep each token's 80 columns as 16-byte chunks that pair the two 16-column
// blocks one 16x16x32 step contracts together: chunk 4p + g holds columns 32p + 4g .. +3 and
// 32p + 16 + 4g .. +3 (p = 0, 1), chunk 8 + g columns 64 + 4g .. +3 and four zeros, so a lane's operand
// is one 16-byte read.  224-byte rows keep those reads apart in banks.
constexpr int kLR = 112;
constexpr int kLP = kE + 8;        // fp32 partials [w][t][e] (row stride 32 mod 64 bytes: 16-byte accesses in one pass)
constexpr int kLPV = kDV + 8;

struct PbParams {
  const uint16_t* q;     // [n_heads * L][64]
  const uint16_t* k;
  const uint16_t* anchors;  // [n_draw_sets][F][64] (draw set of head h: h % n_draw_sets)
  const uint16_t* prf;
  int64_t draw_set_stride;
  int n_draw_sets, m;
  NodeConsts nc;
  const uint16_t* v;     // [n_heads * L][64]
  const uint16_t* dout;  // [n_heads * L][64]
  int64_t L, seg_len;
  int n_seg;
  float* states;         // [n_heads][n_seg][F / 16][kNE][64][4]: element (f, e) at lane e%16 + 16 ((f%16)/4), slot f%4
  float* g;              // [n_heads * L][80] fp32: [dout/den | h | 0 ...]
  uint16_t* dphiq;       // [n_heads * L][F] bf16
  uint16_t* dphik;
  uint16_t* dv;          // [n_heads * L][64]
};

// The feature map of the step's tokens for this wave's features, on chip:
// y = P x (bf16 products, fp32 accumulation) for the anchor and PRF rows of
// the wave's two feature blocks, then phi = (y_a / |x|)^2 exp2(y_g c1 / |x| + c0)
// in fp32 (c1 = sqrt(beta_r) log2 e, c0 = -beta_r/2 log2 e + log2 sqrt(alpha_r/m)),
// with |x| clamped at 1e-12.  The same registers serve both operand orders.
struct Proj {
  bf16x8 a[2][2], p[2][2];  // [feature block j][k-step]: rows 16 fb + c, columns 32 kk + 8g ..
  float c1[2], c0[2];
};

__device__ __forceinline__ void load_proj(Proj& P, const PbParams& p, int64_t h, int w, int g, int c) {
  const int64_t set = h % p.n_draw_sets;
  const uint16_t* A = p.anchors + set * p.draw_set_stride;
  const uint16_t* G = p.prf + set * p.draw_set_stride;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int fb = 2 * w + j;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      P.a[j][kk] = ld8(A + (16 * fb + c) * kDV + 32 * kk + 8 * g);
      P.p[j][kk] = ld8(G + (16 * fb + c) * kDV + 32 * kk + 8 * g);
    }
    const int node = (16 * fb) / p.m;
    P.c1[j] = p.nc.c1[node];
    P.c0[j] = p.nc.c0[node];
  }
}

// rows t0 + c of x (zero past n), with 1/|x| and log2(1/|x|^2) of that row
struct XRows {
  bf16x8 x0, x1;
  float inv, lg;
};

// Global inputs of one 16-token step, all issued one step ahead of their
// use into the registers the step has just consumed: its q, k rows (read by
// the feature map) and the v and g' pieces (staged in LDS at the top of the
// step, before the next step's loads reuse their registers).  dout is
// loaded at the top of its own step: it is read only after the step's two
// barriers.  Rows past the step's n read its last row (an unconditional
// load: a select between addresses would go through a private zero copy)
// and are zeroed where used.
struct StepIn {
  uint4 qa, qb, ka, kb;  // rows t0 + c of q and k: columns 8g .. and 32 + 8g ..
  uint4 v;               // threads < 128: v row t0 + tid/8, columns 8 (tid % 8) ..
  f32x4 gp;              // staging thread u = (tid + 256) % 512 < 320: the g' piece of g_piece(u)
};

// g' pieces: staging thread u < 320 holds row t = 2 (u / 40) + u % 2, columns 4 ((u % 40) / 2) ..,
// so that lanes u and u^1 hold the same columns of a token pair
__device__ __forceinline__ void g_piece(int u, int& t, int& e0) {
  t = 2 * (u / (kE / 2)) + (u & 1);
  e0 = 4 * ((u % (kE / 2)) >> 1);
}

// Global accesses of a step: a wave-uniform row base (scalar registers) plus a 32-bit lane offset in
// elements, so no lane holds a 64-bit address.
template <class T, class E>
__device__ __forceinline__ T& at_row(E* base, int64_t row0, int row_elems, uint32_t off) {
  using B = typename std::conditional<std::is_const<E>::value, const char, char>::type;
  B* b = reinterpret_cast<B*>(base + row0 * row_elems);
  return *reinterpret_cast<T*>(b + off * (uint32_t)sizeof(E));
}

template <bool Q, bool K, bool V, bool G>
__device__ __forceinline__ void load_step(StepIn& s, const PbParams& p, int64_t row0, int n, int g, int c, int tid) {
  const uint32_t rx = (uint32_t)min(c, n - 1) * kDV;
  if (Q) {
    s.qa = at_row<const uint4>(p.q, row0, kDV, rx + 8 * g);
    s.qb = at_row<const uint4>(p.q, row0, kDV, rx + 32 + 8 * g);
  }
  if (K) {
    s.ka = at_row<const uint4>(p.k, row0, kDV, rx + 8 * g);
    s.kb = at_row<const uint4>(p.k, row0, kDV, rx + 32 + 8 * g);
  }
  if (V && tid < kT * 8)
    s.v = at_row<const uint4>(p.v, row0, kDV, (uint32_t)min(tid >> 3, n - 1) * kDV + 8 * (tid & 7));
  if (G) {
    const int u = (tid + 256) & (kNT - 1);
    if (u < kT * (kE / 4)) {
      int t, e0;
      g_piece(u, t, e0);
      s.gp = at_row<const f32x4>(p.g, row0, kE, (uint32_t)min(t, n - 1) * kE + e0);
    }
  }
}

// every thread: dout row t0 + tid/32, columns 2(tid%32), 2(tid%32) + 1
__device__ __forceinline__ uint32_t load_dout(const PbParams& p, int64_t row0, int n, int tid) {
  return at_row<const uint32_t>(p.dout, row0, kDV, (uint32_t)min(tid >> 5, n - 1) * kDV + 2 * (tid & 31));
}

__device__ __forceinline__ XRows finish_x(uint4 a, uint4 b, bool valid) {
  if (!valid) a = b = make_uint4(0, 0, 0, 0);
  XRows X;
  X.x0 = __builtin_bit_cast(bf16x8, a);
  X.x1 = __builtin_bit_cast(bf16x8, b);
  const uint32_t wd[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  float ss = 0.f;  // bf16 products are exact in fp32
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const bf16x2 h2 = __builtin_bit_cast(bf16x2, wd[t]);
    ss = __builtin_amdgcn_fdot2_f32_bf16(h2, h2, ss, false);
  }
  ss += __shfl_xor(ss, 16, 64);
  ss += __shfl_xor(ss, 32, 64);
  X.inv = __builtin_amdgcn_rsqf(fmaxf(ss, 1e-24f));  // 1 / max(|x|, 1e-12), within 1 ulp
  X.lg = 2.0f * __builtin_amdgcn_logf(X.inv);  // log2(inv^2)
  return X;
}

// phi[t0 + c][16 fb + 4g + r] (r < 4): a lane's k-slots over the wave's features, tokens on lanes
__device__ __forceinline__ f32x4 phi_feat(const Proj& P, const XRows& X, int j) {
  f32x4 ya = mfma_bf16(P.a[j][0], X.x0, kZero4);
  ya = mfma_bf16(P.a[j][1], X.x1, ya);
  f32x4 yg = mfma_bf16(P.p[j][0], X.x0, kZero4);
  yg = mfma_bf16(P.p[j][1], X.x1, yg);
  const float s1 = X.inv * P.c1[j], c0 = P.c0[j] + X.lg;
  f32x4 o;
#pragma unroll
  for (int r = 0; r < 4; ++r) o[r] = ya[r] * ya[r] * fast_exp2(fmaf(yg[r], s1, c0));
  return o;
}

// phi[t0 + 4g + r][16 fb + c] (r < 4): four tokens per lane, features on lanes
__device__ __forceinline__ f32x4 phi_tok(const Proj& P, const XRows& X, int j, int g) {
  f32x4 ya = mfma_bf16(X.x0, P.a[j][0], kZero4);
  ya = mfma_bf16(X.x1, P.a[j][1], ya);
  f32x4 yg = mfma_bf16(X.x0, P.p[j][0], kZero4);
  yg = mfma_bf16(X.x1, P.p[j][1], yg);
  f32x4 o;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float inv = __shfl(X.inv, 4 * g + r, 64), lg = __shfl(X.lg, 4 * g + r, 64);
    o[r] = ya[r] * ya[r] * fast_exp2(fmaf(yg[r], inv * P.c1[j], P.c0[j] + lg));
  }
  return o;
}

// position of column e (a multiple of 4: four columns together) in a row of a row tile
__device__ __forceinline__ int rcol(int e) {
  const int b = e >> 4, g = (e >> 2) & 3;
  return b < 4 ? 8 * (4 * (b >> 1) + g) + 4 * (b & 1) : 8 * (8 + g);
}

// position of token t in a row of an [e][t] tile (the first of its two places)
__device__ __forceinline__ int tok_at(int t) { return 8 * (t >> 2) + (t & 3); }

// Zero n bytes of LDS (a multiple of 16), every thread taking part: the [e][t] tiles' parts
// that never change (the zero columns of V', the zero halves of the g' lo tiles) are set once.
__device__ __forceinline__ void zero_lds(void* p, int n, int tid) {
  for (int i = tid; i < n / 16; i += kNT) static_cast<uint4*>(p)[i] = make_uint4(0, 0, 0, 0);
}

// A 16 x 16 fp32 tile in the MFMA result order (lane (g, c): rows 4g .. 4g+3 of column c) moved to
// the transposed order through the wave's own LDS tile: tr_put stores it, tr_get returns rows
// 4g .. 4g+3 of column c of the transpose.  phi of one operand order becomes the other's this way
// rather than by a second projection and epilogue.  The wave's LDS accesses run in order, so no
// barrier separates the two.
constexpr int kLTR = 24;  // 96-byte rows: the 16-byte reads stay apart in banks
__device__ __forceinline__ void tr_put(float* T, const f32x4& v, int g, int c) {
#pragma unroll
  for (int r = 0; r < 4; ++r) T[(4 * g + r) * kLTR + c] = v[r];
}
__device__ __forceinline__ f32x4 tr_get(const float* T, int g, int c) {
  return *reinterpret_cast<const f32x4*>(T + c * kLTR + 4 * g);
}

// V' = [v | 1 | 0] of the step's tokens (zero rows past n) as [t][e] rows and [e][t] columns
// (either may be null; the zero columns of the latter are set once, before the walk).
// The columns are written as token pairs: lanes t and t^1 (lane ^ 8) trade their
// eight values, and the even token's lane writes four columns, the odd one's the
// other four, 4-byte stores into both places of the pair.
__device__ __forceinline__ void stage_v(uint4 x, int n, uint16_t* VR, uint16_t* VT, int tid) {
  if (tid < kT * 8) {
    const int t = tid >> 3, e0 = 8 * (tid & 7);
    if (t >= n) x = make_uint4(0, 0, 0, 0);
    if (VR) {
      *reinterpret_cast<uint2*>(VR + t * kLR + rcol(e0)) = make_uint2(x.x, x.y);
      *reinterpret_cast<uint2*>(VR + t * kLR + rcol(e0 + 4)) = make_uint2(x.z, x.w);
    }
    if (!VT) return;
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};  // columns (e0 + 2i, e0 + 2i + 1) of token t
    uint32_t o[4];                                // the same of token t ^ 1
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = (uint32_t)__shfl_xor((int)w[i], 8, 64);
    const bool odd = t & 1;
#pragma unroll
    for (int r = 0; r < 4; ++r) {  // columns e0 + 4 odd + r
      const int i = 2 * (odd ? 1 : 0) + (r >> 1);
      const int sh = 16 * (r & 1);
      const uint32_t mine = (w[i] >> sh) & 0xFFFFu, other = (o[i] >> sh) & 0xFFFFu;
      const uint32_t pair = odd ? (other | (mine << 16)) : (mine | (other << 16));  // even token in the low half
      uint32_t* d = reinterpret_cast<uint32_t*>(VT + (e0 + 4 * (odd ? 1 : 0) + r) * kLD + tok_at(t & ~1));
      d[0] = pair;
      d[2] = pair;
    }
  } else if (tid < kT * 8 + kT / 2) {  // the ones column, a token pair per thread
    const int t = 2 * (tid - kT * 8);
    const uint32_t one = (t < n ? 0x3F80u : 0u) | (t + 1 < n ? 0x3F800000u : 0u);
    if (VR) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        // chunks 8 .. 11: column 64 (ones) and zeros
        static_assert(8 * 8 == kDV, "the last block's chunks follow the first 64 columns");
        *reinterpret_cast<uint4*>(VR + (t + u) * kLR + kDV) = make_uint4((one >> (16 * u)) & 0xFFFFu, 0, 0, 0);
#pragma unroll
        for (int q = 1; q < 4; ++q) *reinterpret_cast<uint4*>(VR + (t + u) * kLR + kDV + 8 * q) = make_uint4(0, 0, 0, 0);
      }
    }
    if (VT) {
      uint32_t* d = reinterpret_cast<uint32_t*>(VT + kDV * kLD + tok_at(t));
      d[0] = one;
      d[2] = one;
    }
  }
}

// g' of the step's tokens split into hi and lo bf16, as [t][e] rows and [e][t] columns (the
// zero halves of the lo columns are set once, before the walk).  Like V', the columns are
// written as token pairs: lanes u and u^1 hold tokens t and t^1 of the same four columns,
// trade them, and the even token's lane writes two columns, the odd one's the other two.
__device__ __forceinline__ void stage_g(f32x4 x, int n, uint16_t* GRh, uint16_t* GRl, uint16_t* GTh, uint16_t* GTl,
                                        int tid) {
  const int u = (tid + 256) & (kNT - 1);
  if (u < kT * (kE / 4)) {
    int t, e0;
    g_piece(u, t, e0);
    if (t >= n) x = kZero4;
    uint2 h, l;
    split4(x, h, l);
    *reinterpret_cast<uint2*>(GRh + t * kLR + rcol(e0)) = h;  // the last block's zero halves are set once
    *reinterpret_cast<uint2*>(GRl + t * kLR + rcol(e0)) = l;
    if (!GTh) return;
    const bool odd = t & 1;
    const uint32_t mh = odd ? h.y : h.x, ml = odd ? l.y : l.x;  // columns e0 + 2 odd, e0 + 2 odd + 1 of token t
    const uint32_t oh = (uint32_t)__shfl_xor((int)(odd ? h.x : h.y), 1, 64);  // the same columns of token t ^ 1
    const uint32_t ol = (uint32_t)__shfl_xor((int)(odd ? l.x : l.y), 1, 64);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int sh = 16 * k;
      const uint32_t ah = (mh >> sh) & 0xFFFFu, bh = (oh >> sh) & 0xFFFFu;
      const uint32_t al = (ml >> sh) & 0xFFFFu, bl = (ol >> sh) & 0xFFFFu;
      const uint32_t ph = odd ? (bh | (ah << 16)) : (ah | (bh << 16));  // even token in the low half
      const uint32_t pl = odd ? (bl | (al << 16)) : (al | (bl << 16));
      const int at = (e0 + 2 * (odd ? 1 : 0) + k) * kLD + tok_at(t & ~1);
      uint32_t* dh = reinterpret_cast<uint32_t*>(GTh + at);
      dh[0] = ph;
      dh[2] = ph;
      *reinterpret_cast<uint32_t*>(GTl + at) = pl;
    }
  }
}

// the lane's operand from row e of an [e][t] tile: tokens 4g .. 4g+3, then the same again (or zeros)
__device__ __forceinline__ bf16x8 col8(const uint16_t* T, int e, int g) {
  return ld8(T + e * kLD + 8 * g);
}
// chunk q of row r of a row tile: for q = 2 e0 + g, columns 16 e0 + 4g .. +3 and 16 (e0 + 1) + 4g .. +3
// (e0 even; for the last block, zeros in place of the second four)
__device__ __forceinline__ bf16x8 rchunk(const uint16_t* R, int r, int q) { return ld8(R + r * kLR + 8 * q); }

// state item of (head, seg) and its accumulator tiles: element (f = 16 fb + 4g + r, e = 16 eb + c) of the
// tile (fb, eb) in lane 16 g + c, slot r ("C[f][e]" order: one 16-byte access per lane)
__device__ __forceinline__ float* item_ptr(const PbParams& p, int64_t h, int seg) {
  return p.states + (h * p.n_seg + seg) * (int64_t)(kF * kE);
}
__device__ __forceinline__ f32x4 load_fe(const float* item, int fb, int eb, int lane) {
  return *reinterpret_cast<const f32x4*>(item + ((fb * kNE + eb) * 64 + lane) * 4);
}
__device__ __forceinline__ void store_fe(float* item, int fb, int eb, int lane, const f32x4& x) {
  *reinterpret_cast<f32x4*>(item + ((fb * kNE + eb) * 64 + lane) * 4) = x;
}
// the transposed tile order ("C[e][f]"): element (e = 16 eb + 4g + r, f = 16 fb + c) in lane 16 g + c, slot r
__device__ __forceinline__ f32x4 load_ef(const float* item, int fb, int eb, int g, int c) {
  f32x4 x;
#pragma unroll
  for (int r = 0; r < 4; ++r) x[r] = item[((fb * kNE + eb) * 64 + (4 * g + r) + 16 * (c >> 2)) * 4 + (c & 3)];
  return x;
}

// A segment's steps.  The body takes the step's q, k rows (issued during the
// previous step), its token range, the step's index (its parity picks the
// LDS buffers of the double-buffered tiles) and a callback that issues the
// next step's rows into the same registers once the body has consumed them.
template <bool REV, class LOAD, class BODY>
__device__ __forceinline__ void walk_steps(int64_t t_begin, int64_t t_end, LOAD load, BODY body) {
  const int n_steps = (int)((t_end - t_begin + kT - 1) / kT);
  auto geom = [&](int i, int64_t& t0, int& n) {
    const int st = REV ? n_steps - 1 - i : i;
    t0 = t_begin + (int64_t)st * kT;
    n = (int)min<int64_t>(kT, t_end - t0);
  };
  StepIn in;
  int64_t t0;
  int n;
  geom(0, t0, n);
  load(in, t0, n);
  for (int i = 0; i < n_steps; ++i) {
    int64_t tc;
    int nc;
    geom(i, tc, nc);
    auto prefetch = [&]() {
      if (i + 1 < n_steps) {
        int64_t tn;
        int nn;
        geom(i + 1, tn, nn);
        load(in, tn, nn);
      }
    };
    body(in, tc, nc, i, prefetch);
  }
}

// (1) sum over each segment's keys (all segments but the last) of phi(k) v'^T, in the item order
__global__ __launch_bounds__(kNT) void pb_state_kernel(PbParams p) {
  __shared__ __align__(16) uint16_t VT2[2][kE * kLD];
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, c = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  zero_lds(VT2, sizeof(VT2), tid);
  __syncthreads();
  const int n_items = p.n_seg - 1;
  const int64_t h = blockIdx.x / n_items;
  const int seg = (int)(blockIdx.x - h * n_items);
  const int64_t t_begin = seg * p.seg_len;
  const int64_t t_end = min<int64_t>(p.L, t_begin + p.seg_len);
  Proj P;
  load_proj(P, p, h, w, g, c);
  f32x4 S[2][kNE];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int eb = 0; eb < kNE; ++eb) S[j][eb] = kZero4;
  walk_steps<false>(
      t_begin, t_end,
      [&](StepIn& in, int64_t t0, int n) { load_step<false, true, true, false>(in, p, h * p.L + t0, n, g, c, tid); },
      [&](StepIn& in, int64_t t0, int n, int step, auto prefetch) {
        const XRows xk = finish_x(in.ka, in.kb, c < n);
        // double-buffered VT: the previous step's readers use the other buffer, and a
        // buffer is written again only after every wave has passed the next step's barrier
        uint16_t* VT = VT2[step & 1];
        stage_v(in.v, n, nullptr, VT, tid);
        prefetch();
        f32x4 kt[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) kt[j] = phi_tok(P, xk, j, g);
        __syncthreads();
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const bf16x8 a = hilo(kt[j]);
#pragma unroll
          for (int eb = 0; eb < kNE; ++eb) S[j][eb] = mfma_bf16(a, col8(VT, 16 * eb + c, g), S[j][eb]);
        }
      });
  float* item = item_ptr(p, h, seg);
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int eb = 0; eb < kNE; ++eb) store_fe(item, 2 * w + j, eb, lane, S[j][eb]);
}

// (2) numerators, denominators and g' of every token, with S' (the item: the state before the segment) in
// accumulators
__global__ __launch_bounds__(kNT) void pb_g_kernel(PbParams p) {
  __shared__ __align__(16) uint16_t VT2[2][kE * kLD];
  __shared__ __align__(16) float P2[2][kW * kT * kLP];
  __shared__ __align__(16) float TR[kW][2][kT * kLTR];  // each wave's phi(k) transposes
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, c = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  zero_lds(VT2, sizeof(VT2), tid);
  __syncthreads();
  const int64_t h = blockIdx.x / p.n_seg;
  const int seg = (int)(blockIdx.x - h * p.n_seg);
  const int64_t t_begin = seg * p.seg_len;
  const int64_t t_end = min<int64_t>(p.L, t_begin + p.seg_len);
  const float* item = item_ptr(p, h, seg);
  Proj Pj;
  load_proj(Pj, p, h, w, g, c);
  f32x4 S[2][kNE];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int eb = 0; eb < kNE; ++eb) S[j][eb] = load_fe(item, 2 * w + j, eb, lane);
  walk_steps<false>(
      t_begin, t_end,
      [&](StepIn& in, int64_t t0, int n) { load_step<true, true, true, false>(in, p, h * p.L + t0, n, g, c, tid); },
      [&](StepIn& in, int64_t t0, int n, int step, auto prefetch) {
        const int64_t row0 = h * p.L + t0;
        const uint32_t dout2 = load_dout(p, row0, n, tid);
        const XRows xq = finish_x(in.qa, in.qb, c < n), xk = finish_x(in.ka, in.kb, c < n);
        // double-buffered VT and P: the previous step's readers use the other buffers, and a
        // buffer is written again only after every wave has passed the next step's barriers
        uint16_t* VT = VT2[step & 1];
        float* P = P2[step & 1];
        stage_v(in.v, n, nullptr, VT, tid);
        prefetch();
        const f32x4 qa = phi_feat(Pj, xq, 0), qb = phi_feat(Pj, xq, 1);
        const f32x4 ka = phi_feat(Pj, xk, 0), kb = phi_feat(Pj, xk, 1);
        tr_put(TR[w][0], ka, g, c);  // phi(k) with tokens in k-slots, for the state update
        tr_put(TR[w][1], kb, g, c);
        __syncthreads();
        // this wave's part of A^T[j][i] = sum_f phi(K_j)_f phi(Q_i)_f over its features (split phi), masked j <= i
        uint2 qh0, ql0, qh1, ql1, kh0, kl0, kh1, kl1;
        split4(qa, qh0, ql0);
        split4(qb, qh1, ql1);
        split4(ka, kh0, kl0);
        split4(kb, kh1, kl1);
        const bf16x8 qh = cat(qh0, qh1), ql = cat(ql0, ql1), kh = cat(kh0, kh1);
        f32x4 at = mfma_bf16(kh, qh, kZero4);  // lane: j = 4g + r, i = c
        at = mfma_bf16(cat(kl0, kl1), qh, at);
        at = mfma_bf16(kh, ql, at);
#pragma unroll
        for (int r = 0; r < 4; ++r) at[r] = (4 * g + r <= c && c < n) ? at[r] : 0.f;
        const bf16x8 atb = hilo(at);  // A^T split: slots 0-3 hi, 4-7 lo of the same four keys
        // num'^T[e][i] partial = V'^T A^T (this wave's A part) + S'^T phi(Q)^T over this wave's features
#pragma unroll
        for (int eb = 0; eb < kNE; ++eb) {
          f32x4 acc = mfma_bf16(col8(VT, 16 * eb + c, g), atb, kZero4);
          uint2 s0h, s0l, s1h, s1l;
          split4(S[0][eb], s0h, s0l);
          split4(S[1][eb], s1h, s1l);
          const bf16x8 sh = cat(s0h, s1h), sl = cat(s0l, s1l);
          acc = mfma_bf16(sh, qh, acc);
          acc = mfma_bf16(sl, qh, acc);
          acc = mfma_bf16(sh, ql, acc);
          *reinterpret_cast<f32x4*>(P + (w * kT + c) * kLP + 16 * eb + 4 * g) = acc;  // lane: e = 16 eb + 4g + r, i = c
        }
        // S' += phi(K)^T V' for this wave's features (after its use: S' is the state before the chunk)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const bf16x8 a = hilo(tr_get(TR[w][j], g, c));
#pragma unroll
          for (int eb = 0; eb < kNE; ++eb) S[j][eb] = mfma_bf16(a, col8(VT, 16 * eb + c, g), S[j][eb]);
        }
        __syncthreads();
        // g' = [dout / den | -(dout . num) / den^2 | 0]: 32 threads per token (every wave), two columns each
        {
          static_assert(kNT == kT * 32 && kDV == 64, "32 threads per token, two columns each");
          const int i = tid >> 5, e0 = 2 * (tid & 31);
          float n0 = 0.f, n1 = 0.f, den = 0.f;
#pragma unroll
          for (int ww = 0; ww < kW; ++ww) {
            const float* pr = P + (ww * kT + i) * kLP;
            const float2 x = *reinterpret_cast<const float2*>(pr + e0);
            n0 += x.x;
            n1 += x.y;
            den += pr[kDV];
          }
          const uint32_t dw = i < n ? dout2 : 0u;
          const float d0 = __uint_as_float(dw << 16), d1 = __uint_as_float(dw & 0xFFFF0000u);
          float dot = sum_lanes16(fmaf(d0, n0, d1 * n1));
          dot += __shfl_xor(dot, 16, 64);  // the token's other 16 lanes
          if (i < n) {
            const float inv = __builtin_amdgcn_rcpf(den);  // v_rcp_f32, within 1 ulp
            float* gr = &at_row<float>(p.g, row0, kE, (uint32_t)i * kE);
            *reinterpret_cast<float2*>(gr + e0) = make_float2(d0 * inv, d1 * inv);
            const int q = tid & 31;
            if (q < (kE - kDV) / 4) {  // h and the zero columns, 16 bytes per thread
              f32x4 hz = kZero4;
              if (q == 0) hz[0] = -dot * inv * inv;
              *reinterpret_cast<f32x4*>(gr + kDV + 4 * q) = hz;
            }
          }
        }
      });
}

// (3) dphi(Q) = D phi(K) + G' S'^T for this wave's features, and the segment's sum phi(Q)^T G' (written over
// the item once the walk is done)
__global__ __launch_bounds__(kNT) void pb_dq_kernel(PbParams p) {
  __shared__ __align__(16) uint16_t VT2[2][kE * kLD];
  __shared__ __align__(16) uint16_t VR2[2][kT * kLR];
  __shared__ __align__(16) uint16_t GRh2[2][kT * kLR];
  __shared__ __align__(16) uint16_t GRl2[2][kT * kLR];
  __shared__ __align__(16) uint16_t GTh2[2][kE * kLD];
  __shared__ __align__(16) uint16_t GTl2[2][kE * kLD];
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, c = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  zero_lds(VT2, sizeof(VT2), tid);
  zero_lds(GTl2, sizeof(GTl2), tid);
  zero_lds(GRh2, sizeof(GRh2), tid);
  zero_lds(GRl2, sizeof(GRl2), tid);
  __syncthreads();
  const int64_t h = blockIdx.x / p.n_seg;
  const int seg = (int)(blockIdx.x - h * p.n_seg);
  const int64_t t_begin = seg * p.seg_len;
  const int64_t t_end = min<int64_t>(p.L, t_begin + p.seg_len);
  float* item = item_ptr(p, h, seg);
  Proj P;
  load_proj(P, p, h, w, g, c);
  f32x4 S[kNE][2], U[2][kNE];  // S' as C[e][f] (contractions over e), U as C[f][e]
#pragma unroll
  for (int eb = 0; eb < kNE; ++eb)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      S[eb][j] = load_ef(item, 2 * w + j, eb, g, c);
      U[j][eb] = kZero4;
    }
  walk_steps<false>(
      t_begin, t_end,
      [&](StepIn& in, int64_t t0, int n) { load_step<true, true, true, true>(in, p, h * p.L + t0, n, g, c, tid); },
      [&](StepIn& in, int64_t t0, int n, int step, auto prefetch) {
        const int64_t row0 = h * p.L + t0;
        const XRows xq = finish_x(in.qa, in.qb, c < n), xk = finish_x(in.ka, in.kb, c < n);
        // double-buffered tiles: the previous step's readers use the other buffers, and a
        // buffer is written again only after every wave has passed the next step's barrier
        const int sb = step & 1;
        uint16_t *VT = VT2[sb], *VR = VR2[sb], *GRh = GRh2[sb], *GRl = GRl2[sb], *GTh = GTh2[sb], *GTl = GTl2[sb];
        stage_v(in.v, n, VR, VT, tid);
        stage_g(in.gp, n, GRh, GRl, GTh, GTl, tid);
        prefetch();
        bf16x8 qt[2], kt[2];  // split phi of the step's tokens, four per lane
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          qt[j] = hilo(phi_tok(P, xq, j, g));
          kt[j] = hilo(phi_tok(P, xk, j, g));
        }
        __syncthreads();
        // D^T[j][i] = v'_j . g'_i (split g'), masked j <= i < n; every wave forms it (lane: j = 4g + r, i = c)
        f32x4 dt = kZero4;
#pragma unroll
        for (int e0 = 0; e0 < kNE; e0 += 2) {
          const bf16x8 vr = rchunk(VR, c, 2 * e0 + g);
          dt = mfma_bf16(vr, rchunk(GRh, c, 2 * e0 + g), dt);
          dt = mfma_bf16(vr, rchunk(GRl, c, 2 * e0 + g), dt);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) dt[r] = (4 * g + r <= c && c < n) ? dt[r] : 0.f;
        uint2 d4, d4l;
        split4(dt, d4, d4l);
        // dphi(Q)^T[f][i] for this wave's features (both blocks per chunk of g', so each chunk is read once
        // and its registers are free before the next)
        f32x4 acc[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          acc[j] = mfma_bf16(kt[j], cat(d4, d4), kZero4);
          acc[j] = mfma_bf16(kt[j], cat(d4l, kZero2), acc[j]);  // lo parts against zeros
        }
#pragma unroll
        for (int e0 = 0; e0 < kNE; e0 += 2) {
          const int e1 = e0 + 1 < kNE ? e0 + 1 : -1;
          const bf16x8 gh = rchunk(GRh, c, 2 * e0 + g), gl = rchunk(GRl, c, 2 * e0 + g);
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            uint2 a0h, a0l, a1h = kZero2, a1l = kZero2;
            split4(S[e0][j], a0h, a0l);
            if (e1 >= 0) split4(S[e1][j], a1h, a1l);
            const bf16x8 sh = cat(a0h, a1h), sl = cat(a0l, a1l);
            acc[j] = mfma_bf16(sh, gh, acc[j]);
            acc[j] = mfma_bf16(sl, gh, acc[j]);
            acc[j] = mfma_bf16(sh, gl, acc[j]);
          }
        }
#pragma unroll
        for (int j = 0; j < 2; ++j)
          if (c < n) at_row<uint2>(p.dphiq, row0, kF, (uint32_t)c * kF + 16 * (2 * w + j) + 4 * g) = pk4(acc[j]);
        // U += phi(Q)^T G' and S' += V'^T phi(K) for this wave's features
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
          for (int eb = 0; eb < kNE; ++eb) {
            U[j][eb] = mfma_bf16(qt[j], col8(GTh, 16 * eb + c, g), U[j][eb]);
            U[j][eb] = mfma_bf16(qt[j], col8(GTl, 16 * eb + c, g), U[j][eb]);  // g' lo against phi hi (lo: zeros)
            S[eb][j] = mfma_bf16(col8(VT, 16 * eb + c, g), kt[j], S[eb][j]);
          }
        }
      });
  // every wave read only its own feature blocks of the item, at the start
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int eb = 0; eb < kNE; ++eb) store_fe(item, 2 * w + j, eb, lane, U[j][eb]);
}

// (5) dphi(K) = D^T phi(Q) + V' U^T for this wave's features, dV = A^T G + phi(K) U[:, :dv] (per-wave partials
// summed through LDS), walking the segment backward with U (the item: U after the segment) in accumulators
__global__ __launch_bounds__(kNT) void pb_dk_kernel(PbParams p) {
  __shared__ __align__(16) uint16_t VR2[2][kT * kLR];
  __shared__ __align__(16) uint16_t GRh2[2][kT * kLR];
  __shared__ __align__(16) uint16_t GRl2[2][kT * kLR];
  __shared__ __align__(16) uint16_t GTh2[2][kE * kLD];
  __shared__ __align__(16) uint16_t GTl2[2][kE * kLD];
  __shared__ __align__(16) float P2[2][kW * kT * kLPV];
  __shared__ __align__(16) float TR[kW][2][kT * kLTR];  // each wave's phi(q) transposes
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, c = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  zero_lds(GTl2, sizeof(GTl2), tid);
  zero_lds(GRh2, sizeof(GRh2), tid);
  zero_lds(GRl2, sizeof(GRl2), tid);
  __syncthreads();
  const int64_t h = blockIdx.x / p.n_seg;
  const int seg = (int)(blockIdx.x - h * p.n_seg);
  const int64_t t_begin = seg * p.seg_len;
  const int64_t t_end = min<int64_t>(p.L, t_begin + p.seg_len);
  const float* item = item_ptr(p, h, seg);
  Proj Pj;
  load_proj(Pj, p, h, w, g, c);
  // U as C[e][f] (contraction over e: dphi(K)) and, for its dv columns, as C[f][e] (over f: dV).  dV
  // rounds its copy to single bf16, so that copy takes g' hi alone.
  constexpr int kNEA = kDV / 16;
  f32x4 UA[2][kNEA], UB[kNE][2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int eb = 0; eb < kNE; ++eb) {
      if (eb < kNEA) UA[j][eb] = load_fe(item, 2 * w + j, eb, lane);
      UB[eb][j] = load_ef(item, 2 * w + j, eb, g, c);
    }
  walk_steps<true>(
      t_begin, t_end,
      [&](StepIn& in, int64_t t0, int n) { load_step<true, true, true, true>(in, p, h * p.L + t0, n, g, c, tid); },
      [&](StepIn& in, int64_t t0, int n, int step, auto prefetch) {
        const int64_t row0 = h * p.L + t0;
        const XRows xq = finish_x(in.qa, in.qb, c < n), xk = finish_x(in.ka, in.kb, c < n);
        // double-buffered tiles and partials: the previous step's readers use the other
        // buffers, and a buffer is written again only after every wave has passed the next
        // step's barriers
        const int sb = step & 1;
        uint16_t *VR = VR2[sb], *GRh = GRh2[sb], *GRl = GRl2[sb], *GTh = GTh2[sb], *GTl = GTl2[sb];
        float* P = P2[sb];
        stage_v(in.v, n, VR, nullptr, tid);
        stage_g(in.gp, n, GRh, GRl, GTh, GTl, tid);
        prefetch();
        const f32x4 qa = phi_feat(Pj, xq, 0), qb = phi_feat(Pj, xq, 1);
        const f32x4 ka = phi_feat(Pj, xk, 0), kb = phi_feat(Pj, xk, 1);
        tr_put(TR[w][0], qa, g, c);  // phi(q) with tokens in k-slots, for dphi(K) and U
        tr_put(TR[w][1], qb, g, c);
        __syncthreads();
        bf16x8 qt[2];  // split phi(q) of the step's tokens, four per lane
#pragma unroll
        for (int j = 0; j < 2; ++j) qt[j] = hilo(tr_get(TR[w][j], g, c));
        // this wave's part of A[i][j] over its features, masked i >= j (lane: i = 4g + r, j = c)
        f32x4 aw = mfma_bf16(pk_pair(qa, qb), pk_pair(ka, kb), kZero4);
#pragma unroll
        for (int r = 0; r < 4; ++r) aw[r] = (4 * g + r >= c && 4 * g + r < n) ? aw[r] : 0.f;
        const bf16x8 awb = cat(pk4(aw), kZero2);
        // D[i][j] = g'_i . v'_j (split g'), masked i >= j (lane: i = 4g + r, j = c)
        f32x4 dm = kZero4;
#pragma unroll
        for (int e0 = 0; e0 < kNE; e0 += 2) {
          const bf16x8 vr = rchunk(VR, c, 2 * e0 + g);
          dm = mfma_bf16(rchunk(GRh, c, 2 * e0 + g), vr, dm);
          dm = mfma_bf16(rchunk(GRl, c, 2 * e0 + g), vr, dm);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) dm[r] = (4 * g + r >= c && 4 * g + r < n) ? dm[r] : 0.f;
        uint2 d4, d4l;
        split4(dm, d4, d4l);
        // dphi(K)^T[f][j] for this wave's features (both blocks per chunk of v', as for dphi(Q))
        f32x4 acc[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          acc[j] = mfma_bf16(qt[j], cat(d4, d4), kZero4);
          acc[j] = mfma_bf16(qt[j], cat(d4l, kZero2), acc[j]);  // lo parts against zeros
        }
#pragma unroll
        for (int e0 = 0; e0 < kNE; e0 += 2) {
          const int e1 = e0 + 1 < kNE ? e0 + 1 : -1;
          const bf16x8 vr = rchunk(VR, c, 2 * e0 + g);
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            uint2 a0h, a0l, a1h = kZero2, a1l = kZero2;
            split4(UB[e0][j], a0h, a0l);
            if (e1 >= 0) split4(UB[e1][j], a1h, a1l);
            acc[j] = mfma_bf16(cat(a0h, a1h), vr, acc[j]);
            acc[j] = mfma_bf16(cat(a0l, a1l), vr, acc[j]);
          }
        }
#pragma unroll
        for (int j = 0; j < 2; ++j)
          if (c < n) at_row<uint2>(p.dphik, row0, kF, (uint32_t)c * kF + 16 * (2 * w + j) + 4 * g) = pk4(acc[j]);
        // dV^T[e][j] partial (e < dv): G^T A over this wave's A part, and U^T phi(K)^T over its features
#pragma unroll
        for (int eb = 0; eb < kDV / 16; ++eb) {
          f32x4 acc = mfma_bf16(col8(GTh, 16 * eb + c, g), awb, kZero4);  // second copy against zeros
          acc = mfma_bf16(pk_pair(UA[0][eb], UA[1][eb]), pk_pair(ka, kb), acc);
          *reinterpret_cast<f32x4*>(P + (w * kT + c) * kLPV + 16 * eb + 4 * g) = acc;  // lane: e = 16 eb + 4g + r, j = c
        }
        // U += phi(Q)^T G' (both orders) for the earlier chunks
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
          for (int eb = 0; eb < kNE; ++eb) {
            const bf16x8 gh = col8(GTh, 16 * eb + c, g), gl = col8(GTl, 16 * eb + c, g);
            if (eb < kNEA) UA[j][eb] = mfma_bf16(qt[j], gh, UA[j][eb]);
            UB[eb][j] = mfma_bf16(gh, qt[j], UB[eb][j]);
            UB[eb][j] = mfma_bf16(gl, qt[j], UB[eb][j]);
          }
        }
        __syncthreads();
        if (tid < kT * 8) {  // dV rows: sum of the waves' partials, eight columns per thread
          const int jj = tid >> 3, e0 = 8 * (tid & 7);
          f32x4 a0 = kZero4, a1 = kZero4;
#pragma unroll
          for (int ww = 0; ww < kW; ++ww) {
            const float* pr = P + (ww * kT + jj) * kLPV + e0;
            a0 += *reinterpret_cast<const f32x4*>(pr);
            a1 += *reinterpret_cast<const f32x4*>(pr + 4);
          }
          if (jj < n) {
            const uint2 lo = pk4(a0), hi = pk4(a1);
            at_row<uint4>(p.dv, row0, kDV, (uint32_t)jj * kDV + e0) = make_uint4(lo.x, lo.y, hi.x, hi.y);
          }
        }
      });
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
// next tiles are in flight while the current one is computed.
template <int NF_>
struct VjpK {
  static constexpr int NF = NF_, F = NF * 16, D = 64;
  static constexpr int NW = NF / 2, NT = NW * 64;
  static constexpr int RT = 32, NRB = RT / 16;  // rows per tile
  static constexpr int LX = D + 8, LR = D + 4;
  // x tiles and 1/|x| per row (negative where |x| is clamped), both double-buffered by tile
  // parity; per-wave partials
  static constexpr int oX = 0, oR = 2 * RT * LX * 2, oI = oR + NW * RT * LR * 4;
  static constexpr int kLds = oI + 2 * RT * 4;
  static_assert(NT >= RT * 8 && NT == RT * 16, "one x piece per thread (some idle), one output piece per thread");
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

typedef unsigned int u32x2v __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));

// Buffer resource over rows [r0, min(r0 + rt, n_rows)) of a row-major array:
// accesses past those rows (or past the end, for a tile past the last) read
// zeros and write nothing, so every thread issues the same memory
// instructions for every tile.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* base, int64_t r0, int64_t n_rows, int rt,
                                                           int row_bytes) {
  const int64_t nr = max<int64_t>(0, min<int64_t>(rt, n_rows - r0));
  char* b = const_cast<char*>(static_cast<const char*>(base)) + (nr > 0 ? r0 : 0) * row_bytes;
  return __builtin_amdgcn_make_buffer_rsrc(b, (short)0, (int)(nr * row_bytes), 0x00020000);
}
constexpr int kOutOfRange = 0x7FFFFFF0;

template <class K>
__device__ __forceinline__ void vjp_load(const uint16_t* __restrict__ x, const uint16_t* __restrict__ dphi,
                                         int64_t n_rows, int64_t r0, int tid, int wave, int g, int c16,
                                         VjpPref<K>& pf) {
  const __amdgpu_buffer_rsrc_t rx = tile_rsrc(x, r0, n_rows, K::RT, K::D * 2);
  const int xo = tid < K::RT * 8 ? (tid >> 3) * (K::D * 2) + 16 * (tid & 7) : kOutOfRange;
  pf.x = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, xo, 0, 0));
  const __amdgpu_buffer_rsrc_t rd = tile_rsrc(dphi, r0, n_rows, K::RT, K::F * 2);
#pragma unroll
  for (int rb = 0; rb < K::NRB; ++rb)
#pragma unroll
    for (int j = 0; j < 2; ++j)
      pf.dp[rb][j] = __builtin_bit_cast(
          uint2, __builtin_amdgcn_raw_buffer_load_b64(rd, (rb * 16 + c16) * (K::F * 2) + ((2 * wave + j) * 16 + 4 * g) * 2,
                                                      0, 0));
}

// 2x of a bf16 value, exactly (through fp32)
__device__ __forceinline__ uint16_t twice_bf16(uint16_t b) {
  return (uint16_t)(__float_as_uint(2.0f * __uint_as_float((uint32_t)b << 16)) >> 16);
}

template <class K>
__global__ __launch_bounds__(K::NT) void vjp_kernel(VjpParams p) {
  extern __shared__ __align__(16) char lds_raw[];
  float* sR = reinterpret_cast<float*>(lds_raw + K::oR);
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
  // Tiles are loaded two ahead, into two register sets that alternate (the
  // loop body is taken twice per iteration, once per set).  A tile's x rows
  // move to LDS at its start; its dphi pieces are read from the registers by
  // the thread that loaded them, and the set is reloaded (for the tile two
  // ahead) once they have been used, so no loaded value is copied between
  // registers and dphi needs no trip through LDS.  Vector loads
  // and stores retire in issue order and share one counter; every load and
  // store here is a bounded buffer access issued by every thread for every
  // tile (a tile past the last one reads zeros and writes nothing), so the
  // compiler can count what is in flight and a tile's staging waits only for
  // its own rows, not for the stores issued since.
  const int64_t gs = gridDim.x;
  auto load_tile = [&](int64_t t, VjpPref<K>& dst) {
    vjp_load<K>(x, dphi, p.n_rows, t * K::RT, tid, wave, g, c16, dst);
  };
  auto tile_body = [&](int64_t tile, VjpPref<K>& pf, int buf) {
    // sX and sI of this tile's parity: their last readers (the tile before the previous one)
    // are done once every thread has passed the previous tile's staging barrier, which it
    // reaches after its own reads of them; sR is written only after this tile's staging
    // barrier
    uint16_t* sX = reinterpret_cast<uint16_t*>(lds_raw + K::oX) + buf * K::RT * K::LX;
    float* sI = reinterpret_cast<float*>(lds_raw + K::oI) + buf * K::RT;
    const int64_t r0 = tile * K::RT;
    // a tile never spans two draw sets; one set skips the 64-bit division on the scalar unit
    const int tset = p.n_draw_sets == 1 ? 0 : (int)((r0 / p.rows_per_head) % p.n_draw_sets);
    if (tset != set && r0 < p.n_rows) {  // this wave's rows of P, as both operands
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
            e[i] = twice_bf16(A[(fb * 16 + 4 * g + i) * K::D + cb * 16 + c16]);  // the anchor weight's factor 2
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
    if (tid < K::RT * 8) {  // x rows, and 1/|x| once per row (eight threads per row)
      *reinterpret_cast<uint4*>(sX + (tid >> 3) * K::LX + 8 * (tid & 7)) = pf.x;
      const uint32_t wds[4] = {pf.x.x, pf.x.y, pf.x.z, pf.x.w};
      float ss = 0.f;  // bf16 products are exact in fp32
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const bf16x2 h2 = __builtin_bit_cast(bf16x2, wds[t]);
        ss = __builtin_amdgcn_fdot2_f32_bf16(h2, h2, ss, false);
      }
      ss = sum_lanes8(ss);
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
        const uint2 dr = pf.dp[rb][j];
        const float dp[4] = {__uint_as_float(dr.x << 16), __uint_as_float(dr.x & 0xFFFF0000u),
                             __uint_as_float(dr.y << 16), __uint_as_float(dr.y & 0xFFFF0000u)};
        // u = dphi * a * e: w_a = 2u (the 2 is in the transposed anchor rows), w_g = u a sqrt(beta)
        const float s1 = inv * c1[j];
        f32x4 wa, wg;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float a = ya[r] * inv;
          const float e = fast_exp2(fmaf(yg[r], s1, c0[j]));
          const float u = dp[r] * (a * e);
          wa[r] = u;
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
    load_tile(tile + 2 * gs, pf);
    __syncthreads();
    const __amdgpu_buffer_rsrc_t ro = tile_rsrc(dx, r0, p.n_rows, K::RT, K::D * 2);
    {  // 16 lanes per row, four columns each
      const int rr = tid >> 4, c = 4 * (tid & 15);
      const uint2 xr = *reinterpret_cast<const uint2*>(sX + rr * K::LX + c);
      const float xv[4] = {__uint_as_float(xr.x << 16), __uint_as_float(xr.x & 0xFFFF0000u),
                           __uint_as_float(xr.y << 16), __uint_as_float(xr.y & 0xFFFF0000u)};
      f32x4 dh = kZero4;
#pragma unroll
      for (int w = 0; w < K::NW; ++w) dh += *reinterpret_cast<const f32x4*>(sR + (w * K::RT + rr) * K::LR + c);
      float pr = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) pr = fmaf(xv[r], dh[r], pr);
      pr = sum_lanes16(pr);
      const float si = sI[rr];
      const bool clamp = si < 0.f;
      const float inv = fabsf(si);
      const float proj = clamp ? 0.f : pr * inv;  // xh . dxh
      f32x4 o;
#pragma unroll
      for (int r = 0; r < 4; ++r) o[r] = (dh[r] - xv[r] * inv * proj) * inv;
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2v, pk4(o)), ro, rr * (K::D * 2) + c * 2, 0, 0);
    }
  };
  VjpPref<K> pf0, pf1;
  load_tile(blockIdx.x, pf0);
  load_tile(blockIdx.x + gs, pf1);
  for (int64_t tile = blockIdx.x; tile < n_tiles; tile += 2 * gs) {
    tile_body(tile, pf0, 0);
    tile_body(tile + gs, pf1, 1);  // past the last tile: zeros in, nothing out
  }
}

// ---------------------------------------------------------------------------
using V256 = VjpK<16>;

// Segments of the precise kernels: about PB_WG workgroups over all heads, whole
// 16-token steps, at least 64 tokens each.
#ifndef PB_WG
#define PB_WG 256
#endif
int64_t pb_seg_len(int64_t n_heads, int64_t L) {
  const int64_t want = (L * n_heads + PB_WG - 1) / PB_WG;
  return std::max<int64_t>(64, (want + kT - 1) / kT * kT);
}

struct PbWs {
  float *states, *g;
  uint16_t *dphiq, *dphik;
  size_t bytes;
};

PbWs pb_ws(const BackwardArgs& a, int n_seg, void* base) {
  const int64_t rows = a.n_heads * a.L;
  PbWs w{};
  char* p = static_cast<char*>(base);
  size_t off = 0;
  auto take = [&](size_t b) {
    char* q = p ? p + off : nullptr;
    off += (b + 255) & ~(size_t)255;
    return q;
  };
  w.states = reinterpret_cast<float*>(take(sizeof(float) * (size_t)a.n_heads * n_seg * kF * kE));
  w.g = reinterpret_cast<float*>(take(sizeof(float) * (size_t)rows * kE));
  w.dphiq = reinterpret_cast<uint16_t*>(take(2 * (size_t)rows * kF));
  w.dphik = reinterpret_cast<uint16_t*>(take(2 * (size_t)rows * kF));
  w.bytes = off;
  return w;
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
  const size_t nd = (size_t)a.n_draw_sets * kF * a.d * 2;
  const size_t ns = (size_t)a.n_heads * kF * a.dv * 4, nz = (size_t)a.n_heads * kF * 4;
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
  p.F = kF;
  return p;
}

}  // namespace

bool backward_fused_supported(const BackwardArgs& a) {
  if (a.n_heads == 0 || a.L == 0) return false;  // nothing for the MFMA kernels: the general launcher handles it
  // F < 256 runs on zero-padded features (a multiple of 32, as the m % 32 rule gives)
  if (!a.io_bf16 || a.d != 64 || a.dv != 64 || a.F > kF || a.F % 32 != 0 || a.chunk != 64 || a.m % 32 != 0)
    return false;
  if (a.n_draw_sets > 1 && a.L % V256::RT != 0) return false;  // a VJP tile must not span two draw sets
  return true;
}

size_t backward_fused_workspace_bytes(const BackwardArgs& a) {
  if (a.n_heads == 0 || a.L == 0) return 0;
  const BackwardArgs ap = padded_args(a);
  const int64_t seg_len = pb_seg_len(a.n_heads, a.L);
  const int n_seg = (int)((a.L + seg_len - 1) / seg_len);
  const size_t base = pb_ws(ap, n_seg, nullptr).bytes;
  return a.F == kF ? base : base + pad_ws(a, nullptr).bytes;
}

namespace {

hipError_t launch_backward_fused_256(const BackwardArgs& a, hipStream_t s) {
  const int64_t seg_len = pb_seg_len(a.n_heads, a.L);
  const int n_seg = (int)((a.L + seg_len - 1) / seg_len);
  const PbWs w = pb_ws(a, n_seg, a.ws);

  PbParams p{};
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.anchors = static_cast<const uint16_t*>(a.anchors);
  p.prf = static_cast<const uint16_t*>(a.prf);
  p.draw_set_stride = a.draw_set_stride;
  p.n_draw_sets = a.n_draw_sets;
  p.m = a.m;
  p.nc = a.nc;
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
  hipError_t e = hipSuccess;
  if (n_seg > 1) {
    hipLaunchKernelGGL(pb_state_kernel, dim3((unsigned)(a.n_heads * (n_seg - 1))), dim3(kNT), 0, s, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  ScanArgs fa{};  // S' before every segment: S0 + the earlier segments' sums
  fa.states = w.states;
  fa.n_heads = a.n_heads;
  fa.n_items = n_seg;
  fa.n_terms = n_seg - 1;
  fa.F = kF;
  fa.dv = a.dv;
  fa.layout = 1;
  fa.S0 = a.S0;
  fa.z0 = a.z0;
  if ((e = launch_scan(fa, s)) != hipSuccess) return e;
  const dim3 grid((unsigned)(a.n_heads * n_seg));
  hipLaunchKernelGGL(pb_g_kernel, grid, dim3(kNT), 0, s, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(pb_dq_kernel, grid, dim3(kNT), 0, s, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  ScanArgs ra{};  // U after every segment: [dS_T | dz_T] + the later segments' sums; the total is [dS0 | dz0]
  ra.states = w.states;
  ra.n_heads = a.n_heads;
  ra.n_items = n_seg;
  ra.n_terms = n_seg;
  ra.F = kF;
  ra.dv = a.dv;
  ra.layout = 1;
  ra.S0 = a.dS_T;
  ra.z0 = a.dz_T;
  ra.S_out = a.dS0;
  ra.z_out = a.dz0;
  ra.reverse = true;
  if ((e = launch_scan(ra, s)) != hipSuccess) return e;
  hipLaunchKernelGGL(pb_dk_kernel, grid, dim3(kNT), 0, s, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;

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
  if (a.F == kF) return launch_backward_fused_256(a, s);
  BackwardArgs ap = padded_args(a);
  const int64_t seg_len = pb_seg_len(a.n_heads, a.L);
  const int n_seg = (int)((a.L + seg_len - 1) / seg_len);
  const PadWs w = pad_ws(a, static_cast<char*>(a.ws) + pb_ws(ap, n_seg, nullptr).bytes);
  const int64_t nh = a.n_heads, F = a.F, P = kF, d = a.d, dv = a.dv;
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
