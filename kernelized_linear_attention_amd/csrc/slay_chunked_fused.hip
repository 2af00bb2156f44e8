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
// Feature waves: wave w owns FBW blocks of 16 features.  It keeps its slice
// of P = [anchors | prf] in registers as MFMA operands and its F-slice of S'
// as fp32 accumulators for the whole segment.  phi(k) is projected with
// tokens as the MFMA M dimension, so each lane's accumulator holds 4
// consecutive tokens of one feature -- exactly the A-operand of the state
// update, kept in registers (and, in pass 2, also written to LDS as
// phi(k)[j][f]); phi(q) is projected with features as M and written to LDS as
// phi(q)[i][f].  Pass 2 adds four consumer waves that run the contractions of
// chunk c (the causal blocks A^T = phi(k) phi(q)^T, masked and rounded to
// bf16, then v'^T A^T; and S'^T phi(q)^T from a bf16 copy of S'^T in LDS)
// while the feature waves map chunk c+1 (see pass2s_kernel).
// The contraction over tokens uses a fixed permutation of the 32 tokens of
// an MFMA k-step (lane group g holds tokens 4g..4g+3 and 16+4g..16+4g+3) on
// both operands, which leaves the sum unchanged and lets accumulators feed
// the next MFMA without a transpose.
#include <type_traits>

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
  // Rows of v'^T and of the bf16 copy of S'^T kept in LDS: the DV value
  // rows, row DV (ones / z) and one zero row that stands for rows DV+1..DV+15.
  static constexpr int VROWS = DV + 2;
  static constexpr int LDX = D + 8;        // padded row strides (elements)
  static constexpr int LDV = C + 4;        // 34 dwords: 16 lanes x 8 bytes hit 32 distinct banks
  static constexpr int LDF = F + 8;
  static_assert(C % 32 == 0 && D % 32 == 0 && DV % 16 == 0, "tile sizes");
  static constexpr int kVbuf = VROWS * LDV * 2;  // one v'^T buffer (bytes)
  // pass 1 LDS: k tile with its row scales (two buffers), v'^T (three buffers)
  static constexpr int kKbuf1 = C * LDX * 2 + 2 * C * 4;
  static constexpr int kLds1 = 2 * kKbuf1 + 3 * kVbuf;
  // pass 1 splits the features over FS1 workgroups of NW / FS1 waves
  static constexpr int FS1 = 1;
  // phi projections of block tb+1 issued before the epilogue of block tb
  static constexpr bool PIPE = true;
  // pass 1 with dedicated stager waves (pass1s_kernel); at 6 feature waves
  // (F = 96) that measured 3% faster over the whole forward than pass1_kernel
  static constexpr bool STAGERS1 = (NW >= 6);
};

struct Params {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  int64_t L;
  int64_t seg_len;  // tokens per segment (multiple of C)
  int n_seg;
  int sub;          // pass-1 sub-segments per segment (seg_len / sub is a multiple of C)
  int m;
  const uint16_t* anchors;
  const uint16_t* prf;
  int64_t draw_set_stride;
  int n_draw_sets;
  NodeConsts nc;
  float* ws;         // [n_heads][p1_items][F/16][NE][64][4] fragment-ordered states:
                     // after the scan, item s * sub is the prefix of segment s and
                     // item p1_segs the total
  int p1_segs;       // segments the segment-state pass covers per head (of the keys)
  int p1_items;      // p1_segs + 1
  int64_t Lq;        // queries per head (non-causal; the causal path has Lq = L)
  int64_t qseg_len;  // queries per workgroup of the non-causal output pass
  int n_qseg;
  const float* S0;   // used when there is a single segment
  const float* z0;
  float* S_out;
  float* z_out;
  // Variable-length batches: the packed token axis of each head holds
  // sequences s at tokens cu[s] .. cu[s+1] (T tokens per head).  Workgroup w
  // takes work item g = w / n_heads of head w % n_heads (so the heads' items
  // of one g run side by side).  The main pass has vl_count[0] items, the
  // segment-state pass the first vl_count[1] of them: the whole segments that
  // another segment of their sequence follows.  vl_item[g] = (chunks of 32
  // tokens, chunks of 64, a, b): a whole segment (b < 0) of sequence -1 - b
  // starting at row a of the head's packed axis, owning state slot g (the
  // last piece of its sequence when g >= vl_count[1]); or a pack of sequence
  // tails walked one after another (b >= 0) whose chunk descriptors start at
  // vl_list32[a]: (row of the chunk's first token in the packed axis, tokens,
  // state slot, kFirst | kLast | kSeqEnd | sequence << 3).  A pack walks at
  // most vl_cap chunks.
  const int* vl_count;
  const int4* vl_item;
  const int4* vl_list32;
  int vl_cap;
  const int64_t* cu;
  int64_t T;
  int g_max;         // work items per head
  int64_t n_heads;
};

// Where a dense workgroup's tokens lie: the packed row of the head's token 0,
// its token range and its state item.
struct Geo {
  int64_t head;
  int64_t row0;
  int64_t t0, t1;
  int64_t item;
  int seg;
};

// per_head: work items per head; items_per_head: state items per head in the
// workspace.
__device__ __forceinline__ Geo geo_of(const Params& p, int per_head, int64_t seg_len, int64_t items_per_head) {
  Geo g;
  const int64_t w = blockIdx.x;
  g.head = w / per_head;
  g.seg = (int)(w - g.head * per_head);
  g.row0 = g.head * p.L;
  g.t0 = (int64_t)g.seg * seg_len;
  g.t1 = min<int64_t>(p.L, g.t0 + seg_len);
  g.item = g.head * items_per_head + g.seg;
  return g;
}

// chunk flags: first / last chunk of its piece; the piece ends its sequence
constexpr int kFirst = 1, kLast = 2, kSeqEnd = 4;

// One chunk of a workgroup's walk.
struct ChunkRef {
  int64_t row;   // packed row of the chunk's first token
  int n;         // tokens in the chunk (1 .. C)
  int64_t item;  // state item of the chunk's piece
  int flags;     // kFirst, kLast, kSeqEnd
  int seq;       // variable-length: the piece's sequence
};

// The chunks a workgroup walks.  Dense (VL false): the whole chunks of one
// (head, segment), a single piece.  Variable-length: a whole segment of one
// sequence (one piece, whole chunks), or (main pass only) a pack of sequence
// tails, one piece each, whose chunk descriptors every thread of the
// workgroup copies to LDS before the workgroup's first barrier.
template <class K, bool VL>
struct Chunks {
  int64_t head;
  int nch;
  bool valid;
  Geo geo;            // dense, and a variable-length whole segment (row0, item)
  bool pack;          // VL: a pack of tails
  bool seq_end;       // VL whole segment: the last piece of its sequence
  int seq;            // VL whole segment: its sequence
  const int4* list;   // VL pack: descriptors in LDS
  int64_t head_row, head_item;
  __device__ __forceinline__ ChunkRef at(int c) const {
    if (VL && pack) {  // the same descriptor in every lane: kept in scalar registers
      const int4 e = list[c];
      const int w = __builtin_amdgcn_readfirstlane(e.w);
      return {head_row + __builtin_amdgcn_readfirstlane(e.x), __builtin_amdgcn_readfirstlane(e.y),
              head_item + __builtin_amdgcn_readfirstlane(e.z), w & 7, w >> 3};
    }
    const int64_t c0 = geo.t0 + (int64_t)c * K::C;
    const bool last = c == nch - 1;
    return {geo.row0 + c0, (int)min<int64_t>(K::C, geo.t1 - c0), geo.item,
            (c == 0 ? kFirst : 0) | (last ? kLast : 0) | (last && seq_end ? kSeqEnd : 0), seq};
  }
};

// per_head, seg_len, items_per_head as for geo_of (dense only); sl: LDS room
// for vl_cap chunk descriptors (VL only); nt: threads of the workgroup.
template <class K, bool VL>
__device__ __forceinline__ Chunks<K, VL> chunks_of(const Params& p, int per_head, int64_t seg_len,
                                                   int64_t items_per_head, int4* sl, int nt) {
  Chunks<K, VL> c{};
  if constexpr (VL) {
    const int64_t nh = p.n_heads;
    const int gi = (int)(blockIdx.x / nh);
    c.head = blockIdx.x - (int64_t)gi * nh;
    const int n_pass1 = p.vl_count[1];
    c.valid = gi < (K::C == 64 ? n_pass1 : p.vl_count[0]);
    if (!c.valid) return c;
    const int4 info = p.vl_item[gi];
    c.nch = K::C == 64 ? info.y : info.x;
    c.head_row = c.head * p.T;
    c.head_item = c.head * p.g_max;
    c.pack = K::C != 64 && info.w >= 0;  // the segment-state pass sees whole segments only
    if (c.pack) {
      const int4* src = p.vl_list32 + info.z;
      for (int t = threadIdx.x; t < c.nch; t += nt) sl[t] = src[t];
      c.list = sl;
    } else {
      c.geo.row0 = c.head_row + info.z;
      c.geo.t0 = 0;
      c.geo.t1 = p.seg_len;
      c.geo.item = c.head_item + gi;
      c.seq = -1 - info.w;
      c.seq_end = gi >= n_pass1;
    }
  } else {
    c.geo = geo_of(p, per_head, seg_len, items_per_head);
    c.head = c.geo.head;
    c.valid = true;
    c.nch = (int)((c.geo.t1 - c.geo.t0 + K::C - 1) / K::C);
  }
  return c;
}

__device__ __forceinline__ uint2 pack4(float a, float b, float c, float d) {
  uint2 r;
  r.x = pack_bf16x2(a, b);
  r.y = pack_bf16x2(c, d);
  return r;
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of N consecutive lanes (N = 4, 8 or 16), in DPP.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  v += dpp<0xB1>(v);                     // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);                     // quad_perm [2,3,0,1]
  if (N >= 8) v += dpp<0x141>(v);        // row_half_mirror
  if (N >= 16) v += dpp<0x140>(v);       // row_mirror
  return v;
}

// LDS row that holds state column e = et*16 + col: the value rows, row DV for
// column DV (z / ones), and the shared zero row for the padding columns.
template <class K>
__device__ __forceinline__ int vrow(int et, int col) {
  return et < K::NE - 1 ? et * 16 + col : (col == 0 ? K::DV : K::DV + 1);
}

// Per-lane LDS element offsets of the rows that hold state-column tile et,
// for a buffer with row stride LD.
template <class K, int LD>
struct RowOff {
  int off[K::NE];
  __device__ __forceinline__ explicit RowOff(int col) {
#pragma unroll
    for (int et = 0; et < K::NE; ++et) off[et] = vrow<K>(et, col) * LD;
  }
};

// Load this wave's slice of P as MFMA operands and its node constants.
// fb0: first 16-feature block of this wave.
template <class K>
__device__ __forceinline__ void load_p(const Params& p, int set, int fb0, int lane, bf16x8 (&pa)[K::FBW][K::NKS],
                                       bf16x8 (&pg)[K::FBW][K::NKS], float (&c1)[K::FBW], float (&c0)[K::FBW]) {
  const int g = lane >> 4, col = lane & 15;
  const uint16_t* a = p.anchors + (int64_t)set * p.draw_set_stride;
  const uint16_t* gg = p.prf + (int64_t)set * p.draw_set_stride;
#pragma unroll
  for (int j = 0; j < K::FBW; ++j) {
    const int fb = fb0 + j;
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

// Chunk inputs in flight: q, k rows as 16-byte vectors, v as 8-byte pieces
// of two consecutive tokens.  Loaded one chunk ahead into registers and
// written to LDS one step later.
template <class K, int NT = K::NT>
struct Prefetch {
  static constexpr int XV = (K::C * (K::D / 8) + NT - 1) / NT;          // q/k vectors per thread
  static constexpr int VV = ((K::C / 2) * (K::DV / 4) + NT - 1) / NT;   // v pieces per thread
  uint4 q[XV], k[XV];
  uint2 v0[VV], v1[VV];
};

template <class K, int NT = K::NT>
__device__ __forceinline__ void load_x(int tid, const uint16_t* __restrict__ x, int n,
                                       uint4 (&r)[Prefetch<K, NT>::XV]) {
  constexpr int VPR = K::D / 8;
#pragma unroll
  for (int i = 0; i < Prefetch<K, NT>::XV; ++i) {
    const int vec = tid + i * NT;
    const int row = vec / VPR, c = (vec % VPR) * 8;
    r[i] = make_uint4(0, 0, 0, 0);
    if (vec < K::C * VPR && row < n) r[i] = *reinterpret_cast<const uint4*>(x + (int64_t)row * K::D + c);
  }
}

template <class K, int NT = K::NT>
__device__ __forceinline__ void load_v(int tid, const uint16_t* __restrict__ v, int n, uint2 (&r0)[Prefetch<K, NT>::VV],
                                       uint2 (&r1)[Prefetch<K, NT>::VV]) {
  constexpr int HP = K::C / 2;  // token pairs
#pragma unroll
  for (int i = 0; i < Prefetch<K, NT>::VV; ++i) {
    const int item = tid + i * NT;
    const int rp = item % HP, e4 = item / HP;
    r0[i] = make_uint2(0, 0);
    r1[i] = make_uint2(0, 0);
    if (item < HP * (K::DV / 4)) {
      if (2 * rp < n) r0[i] = *reinterpret_cast<const uint2*>(v + (int64_t)(2 * rp) * K::DV + 4 * e4);
      if (2 * rp + 1 < n) r1[i] = *reinterpret_cast<const uint2*>(v + (int64_t)(2 * rp + 1) * K::DV + 4 * e4);
    }
  }
}

template <class K, int NT = K::NT>
// row0: packed row of token 0 of the sequence; c0t: the chunk's first token in it
__device__ __forceinline__ void issue_loads(int tid, const Params& p, int64_t row0, int64_t c0t, int n, bool want_q,
                                            Prefetch<K, NT>& pf) {
  if (want_q) load_x<K, NT>(tid, p.q + (row0 + c0t) * K::D, n, pf.q);
  load_x<K, NT>(tid, p.k + (row0 + c0t) * K::D, n, pf.k);
  load_v<K, NT>(tid, p.v + (row0 + c0t) * K::DV, n, pf.v0, pf.v1);
}

// Write staged q or k vectors to LDS (padded rows) with, per row,
// inv = 1/max(|x|, 1e-12) and lg = log2(inv^2).  The squares are summed with
// the bf16 dot instruction (products of bf16 values are exact in fp32) and
// inv comes from the hardware reciprocal square root (about 1 ulp).
template <class K, int NT = K::NT>
__device__ __forceinline__ void store_x(int tid, const uint4 (&r)[Prefetch<K, NT>::XV], uint16_t* sx, float* sinv,
                                        float* slg) {
  constexpr int VPR = K::D / 8;  // 16-byte vectors per row, consecutive threads
  static_assert((NT % VPR) == 0 && (VPR == 4 || VPR == 8 || VPR == 16), "rows must not straddle lane groups");
#pragma unroll
  for (int i = 0; i < Prefetch<K, NT>::XV; ++i) {
    const int vec = tid + i * NT;
    if (vec >= K::C * VPR) break;  // uniform over whole waves
    const int row = vec / VPR, c = (vec % VPR) * 8;
    *reinterpret_cast<uint4*>(sx + row * K::LDX + c) = r[i];
    const uint32_t w[4] = {r[i].x, r[i].y, r[i].z, r[i].w};
    float ss = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bf16x2 h = __builtin_bit_cast(bf16x2, w[q]);
      ss = __builtin_amdgcn_fdot2_f32_bf16(h, h, ss, false);
    }
    ss = group_sum<VPR>(ss);
    if ((vec % VPR) == 0) {
      const float inv = __builtin_amdgcn_rsqf(fmaxf(ss, 1e-24f));
      sinv[row] = inv;
      slg[row] = 2.0f * __builtin_amdgcn_logf(inv);  // v_log_f32 is log2
    }
  }
}

// Write staged v transposed into v'^T rows 0..DV-1: each thread packs the
// same 4 columns of two consecutive tokens into four 32-bit words.
template <class K, int NT = K::NT>
__device__ __forceinline__ void store_v(int tid, const uint2 (&r0)[Prefetch<K, NT>::VV],
                                        const uint2 (&r1)[Prefetch<K, NT>::VV], uint16_t* sv) {
  constexpr int HP = K::C / 2;
#pragma unroll
  for (int i = 0; i < Prefetch<K, NT>::VV; ++i) {
    const int item = tid + i * NT;
    if (item >= HP * (K::DV / 4)) break;
    const int rp = item % HP, e4 = item / HP;
    uint32_t* dst = reinterpret_cast<uint32_t*>(sv + (4 * e4) * K::LDV + 2 * rp);
    dst[0] = lo16_pair(r0[i].x, r1[i].x);
    dst[K::LDV / 2] = hi16_pair(r0[i].x, r1[i].x);
    dst[K::LDV] = lo16_pair(r0[i].y, r1[i].y);
    dst[3 * K::LDV / 2] = hi16_pair(r0[i].y, r1[i].y);
  }
}

// Constant rows of a v'^T buffer: row DV all ones (the z column), row DV+1 zero.
template <class K, int NT = K::NT>
__device__ __forceinline__ void init_vconst(int tid, uint16_t* sv) {
  for (int t = tid; t < 2 * K::LDV; t += NT)
    sv[K::DV * K::LDV + t] = (t < K::LDV) ? kBf16One : (uint16_t)0;
}

// v' operand for a token k-step s and state column tile et: lane (e = et*16+col,
// group g) gets tokens 32s+4g..+3 and 32s+16+4g..+3 (the shared permutation).
template <class K>
__device__ __forceinline__ bf16x8 vfrag(const uint16_t* sv, const RowOff<K, K::LDV>& vo, int et, int s, int lane) {
  const int g = lane >> 4;
  const uint16_t* row = sv + vo.off[et] + 32 * s + 4 * g;
  const uint2 lo = *reinterpret_cast<const uint2*>(row);
  const uint2 hi = *reinterpret_cast<const uint2*>(row + 16);
  return as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
}

// Scheduling hint for the preceding straight-line code: alternate one MFMA
// with NV VALU instructions, NM times, so the matrix pipe works while the
// wave issues its VALU epilogue (the scheduler keeps dependencies).
template <int NM, int NV>
__device__ __forceinline__ void mfma_valu_interleave() {
#pragma unroll
  for (int i = 0; i < NM; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);  // VALU
  }
}

// Projection accumulators of one 16-token block: y_a (anchor) and y_g (PRF)
// for each of the wave's FBW feature blocks.
template <class K>
struct Proj {
  f32x4 a[K::FBW], g[K::FBW];
};

// Projection of token block tb with tokens as M: each lane's accumulator
// holds tokens 4g..4g+3 of feature col of each block.
template <class K>
__device__ __forceinline__ void proj_tok(const uint16_t* sx, int tb, int lane, const bf16x8 (&pa)[K::FBW][K::NKS],
                                         const bf16x8 (&pg)[K::FBW][K::NKS], Proj<K>& y) {
  const int g = lane >> 4, col = lane & 15;
  bf16x8 xa[K::NKS];
#pragma unroll
  for (int ks = 0; ks < K::NKS; ++ks)
    xa[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(sx + (tb * 16 + col) * K::LDX + ks * 32 + 8 * g));
#pragma unroll
  for (int j = 0; j < K::FBW; ++j) {
    f32x4 ya = mfma_bf16(xa[0], pa[j][0], f32x4{0.f, 0.f, 0.f, 0.f});
    f32x4 yg = mfma_bf16(xa[0], pg[j][0], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
    for (int ks = 1; ks < K::NKS; ++ks) {
      ya = mfma_bf16(xa[ks], pa[j][ks], ya);
      yg = mfma_bf16(xa[ks], pg[j][ks], yg);
    }
    y.a[j] = ya;
    y.g[j] = yg;
  }
}

// Projection of token block tb with features as M: each lane's accumulator
// holds features 4g..4g+3 of each block for token col.
template <class K>
__device__ __forceinline__ void proj_feat(const uint16_t* sx, int tb, int lane, const bf16x8 (&pa)[K::FBW][K::NKS],
                                          const bf16x8 (&pg)[K::FBW][K::NKS], Proj<K>& y) {
  const int g = lane >> 4, col = lane & 15;
  bf16x8 xb[K::NKS];
#pragma unroll
  for (int ks = 0; ks < K::NKS; ++ks)
    xb[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(sx + (tb * 16 + col) * K::LDX + ks * 32 + 8 * g));
#pragma unroll
  for (int j = 0; j < K::FBW; ++j) {
    f32x4 ya = mfma_bf16(pa[j][0], xb[0], f32x4{0.f, 0.f, 0.f, 0.f});
    f32x4 yg = mfma_bf16(pg[j][0], xb[0], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
    for (int ks = 1; ks < K::NKS; ++ks) {
      ya = mfma_bf16(pa[j][ks], xb[ks], ya);
      yg = mfma_bf16(pg[j][ks], xb[ks], yg);
    }
    y.a[j] = ya;
    y.g[j] = yg;
  }
}

// State update slice for token k-step s: S'[own features] += phi(k)^T v'
// over tokens 32s..32s+31.
template <class K>
__device__ __forceinline__ void state_update_step(const uint16_t* sv, const RowOff<K, K::LDV>& vo, int lane, int s,
                                                  const bf16x8 (&kf)[K::FBW][K::NTS], f32x4 (&st)[K::FBW][K::NE]) {
#pragma unroll
  for (int et = 0; et < K::NE; ++et) {
    const bf16x8 vb = vfrag<K>(sv, vo, et, s, lane);
#pragma unroll
    for (int j = 0; j < K::FBW; ++j) st[j][et] = mfma_bf16(kf[j][s], vb, st[j][et]);
  }
}

// phi epilogue of a token block projected with tokens as M:
// phi = (y_a inv)^2 exp2(y_g inv c1 + c0) = y_a^2 exp2(y_g (inv c1) + (c0 + log2 inv^2)).
// Each lane holds 4 tokens of one feature; s1 = inv c1 and c0' = c0 + log2
// inv^2 are formed per token.  The wave's FBW feature blocks belong to one
// Gauss-Laguerre node (the dispatcher requires m % (16 FBW) == 0), so they
// are formed once per token for all blocks.  Results go to kf (the A operand
// of the state update) and, with PHI_LDS, to LDS as phi(k)[j][f].
template <class K, bool PHI_LDS>
__device__ __forceinline__ void epi_tok(const float* sinv, const float* slg, uint16_t* spk, int fb0, int tb, int lane,
                                        const float (&c1)[K::FBW], const float (&c0)[K::FBW], const Proj<K>& y,
                                        bf16x8 (&kf)[K::FBW][K::NTS]) {
  const int g = lane >> 4, col = lane & 15;
  const float4 inv4 = *reinterpret_cast<const float4*>(sinv + tb * 16 + 4 * g);
  const float4 lg4 = *reinterpret_cast<const float4*>(slg + tb * 16 + 4 * g);
  const float s1[4] = {inv4.x * c1[0], inv4.y * c1[0], inv4.z * c1[0], inv4.w * c1[0]};
  const float c0p[4] = {c0[0] + lg4.x, c0[0] + lg4.y, c0[0] + lg4.z, c0[0] + lg4.w};
#pragma unroll
  for (int j = 0; j < K::FBW; ++j) {
    {
      float ph[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ph[i] = y.a[j][i] * y.a[j][i] * fast_exp2(fmaf(y.g[j][i], s1[i], c0p[i]));
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
        // lanes col, col^1 hold features f, f+1 of tokens t..t+3: the even lane
        // writes the (f, f+1) words of tokens t, t+1, the odd lane those of
        // t+2, t+3.  Bytes 0-3 of the v_perm source are this lane's word,
        // 4-7 the neighbour's; the selector puts feature f in the low half.
        const bool odd = col & 1;
        const uint32_t mine = odd ? pk.y : pk.x;
        const uint32_t recv = swap_lane_pair(odd ? pk.x : pk.y);
        const uint32_t sel0 = odd ? 0x01000504u : 0x05040100u;
        const uint32_t sel1 = odd ? 0x03020706u : 0x07060302u;
        const int f = (fb0 + j) * 16 + (col & ~1);
        uint32_t* dst = reinterpret_cast<uint32_t*>(spk + (tb * 16 + 4 * g + (odd ? 2 : 0)) * K::LDF + f);
        dst[0] = __builtin_amdgcn_perm(recv, mine, sel0);
        dst[K::LDF / 2] = __builtin_amdgcn_perm(recv, mine, sel1);
      }
    }
  }
}

// phi epilogue of a token block projected with features as M, to LDS
// phi(q)[i][f] with one 8-byte store per lane and block.
template <class K>
__device__ __forceinline__ void epi_feat(const float* sinv, const float* slg, uint16_t* spq, int wave, int tb,
                                         int lane, const float (&c1)[K::FBW], const float (&c0)[K::FBW],
                                         const Proj<K>& y) {
  const int g = lane >> 4, col = lane & 15;
  const float inv = sinv[tb * 16 + col], lg = slg[tb * 16 + col];
  const float s1 = inv * c1[0], c0p = c0[0] + lg;  // one node per wave, as in epi_tok
#pragma unroll
  for (int j = 0; j < K::FBW; ++j) {
    float ph[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) ph[i] = y.a[j][i] * y.a[j][i] * fast_exp2(fmaf(y.g[j][i], s1, c0p));
    const int f0 = (wave * K::FBW + j) * 16 + 4 * g;
    *reinterpret_cast<uint2*>(spq + (tb * 16 + col) * K::LDF + f0) = pack4(ph[0], ph[1], ph[2], ph[3]);
  }
}

// phi(k) of a staged chunk for this wave's features (tokens as M), software
// pipelined: the projection MFMAs of block tb+1 are issued before the VALU
// epilogue of block tb, so the two overlap.  With SU the state update of the
// previous chunk (from kf_prev and v'^T in sv_prev) is spread over the first
// NTS steps; it reads kf_prev[.][s] before step s rewrites kf (kf_prev may be
// the same array as kf).
template <class K, bool PHI_LDS, bool SU>
__device__ __forceinline__ void phase_k(const uint16_t* sx, const float* sinv, const float* slg, uint16_t* spk,
                                        int fb0, int lane, const bf16x8 (&pa)[K::FBW][K::NKS],
                                        const bf16x8 (&pg)[K::FBW][K::NKS], const float (&c1)[K::FBW],
                                        const float (&c0)[K::FBW], bf16x8 (&kf)[K::FBW][K::NTS],
                                        const uint16_t* sv_prev, const RowOff<K, K::LDV>& vo,
                                        const bf16x8 (&kf_prev)[K::FBW][K::NTS], f32x4 (&st)[K::FBW][K::NE]) {
  if constexpr (K::PIPE) {
    Proj<K> y[2];
    proj_tok<K>(sx, 0, lane, pa, pg, y[0]);
#pragma unroll
    for (int tb = 0; tb < K::NTB; ++tb) {
      if (tb + 1 < K::NTB) proj_tok<K>(sx, tb + 1, lane, pa, pg, y[(tb + 1) & 1]);
      if (SU && tb < K::NTS) state_update_step<K>(sv_prev, vo, lane, tb, kf_prev, st);
      epi_tok<K, PHI_LDS>(sinv, slg, spk, fb0, tb, lane, c1, c0, y[tb & 1], kf);
    }
  } else {  // one block at a time (fewer live registers)
#pragma unroll
    for (int tb = 0; tb < K::NTB; ++tb) {
      Proj<K> y;
      proj_tok<K>(sx, tb, lane, pa, pg, y);
      if (SU && tb < K::NTS) state_update_step<K>(sv_prev, vo, lane, tb, kf_prev, st);
      epi_tok<K, PHI_LDS>(sinv, slg, spk, fb0, tb, lane, c1, c0, y, kf);
    }
  }
}

// phi(q) of the staged chunk for this wave's features (features as M), to
// LDS phi(q)[i][f]; pipelined like phase_k.
template <class K>
__device__ __forceinline__ void phase_q(const uint16_t* sx, const float* sinv, const float* slg, uint16_t* spq,
                                        int wave, int lane, const bf16x8 (&pa)[K::FBW][K::NKS],
                                        const bf16x8 (&pg)[K::FBW][K::NKS], const float (&c1)[K::FBW],
                                        const float (&c0)[K::FBW]) {
  if constexpr (K::PIPE) {
    Proj<K> y[2];
    proj_feat<K>(sx, 0, lane, pa, pg, y[0]);
#pragma unroll
    for (int tb = 0; tb < K::NTB; ++tb) {
      if (tb + 1 < K::NTB) proj_feat<K>(sx, tb + 1, lane, pa, pg, y[(tb + 1) & 1]);
      epi_feat<K>(sinv, slg, spq, wave, tb, lane, c1, c0, y[tb & 1]);
    }
  } else {
#pragma unroll
    for (int tb = 0; tb < K::NTB; ++tb) {
      Proj<K> y;
      proj_feat<K>(sx, tb, lane, pa, pg, y);
      epi_feat<K>(sinv, slg, spq, wave, tb, lane, c1, c0, y);
    }
  }
}

// Write this wave's S' slice as bf16 rows of S'^T in LDS (value rows and the z row).
template <class K>
__device__ __forceinline__ void write_st(uint16_t* sst, const RowOff<K, K::LDF>& so, int wave, int lane,
                                         const f32x4 (&st)[K::FBW][K::NE]) {
  const int g = lane >> 4, col = lane & 15;
#pragma unroll
  for (int j = 0; j < K::FBW; ++j)
#pragma unroll
    for (int et = 0; et < K::NE; ++et) {
      if (et == K::NE - 1 && col != 0) continue;  // padding columns are not stored
      const int f0 = (wave * K::FBW + j) * 16 + 4 * g;
      *reinterpret_cast<uint2*>(sst + so.off[et] + f0) =
          pack4(st[j][et][0], st[j][et][1], st[j][et][2], st[j][et][3]);
    }
}

// Fragment-ordered state index of (feature block fb, column tile et, lane).
template <class K>
__device__ __forceinline__ int64_t frag_off(int fb, int et, int lane) {
  return ((int64_t)(fb * K::NE + et) * 64 + lane) * 4;
}

// State for the wave's feature blocks fb0..fb0+FBW-1: workspace state item
// `item` (absolute index) when from_ws, else S0/z0 of the head (zero when absent).
template <class K>
__device__ __forceinline__ void load_state_item(const Params& p, int64_t head, bool from_ws, int64_t item, int fb0,
                                                int lane, f32x4 (&st)[K::FBW][K::NE]) {
  const int g = lane >> 4, col = lane & 15;
  if (from_ws) {  // a wave-uniform base plus one 32-bit lane offset
    const float* in = p.ws + item * (int64_t)K::F * K::DVP + frag_off<K>(fb0, 0, 0);
    const uint32_t off = (uint32_t)lane * 4;
#pragma unroll
    for (int j = 0; j < K::FBW; ++j)
#pragma unroll
      for (int et = 0; et < K::NE; ++et)
        st[j][et] = *reinterpret_cast<const f32x4*>(in + (j * K::NE + et) * 256 + off);
  } else {
#pragma unroll
    for (int j = 0; j < K::FBW; ++j)
#pragma unroll
      for (int et = 0; et < K::NE; ++et) {
        const int e = et * 16 + col;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int f = (fb0 + j) * 16 + 4 * g + i;
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
}

// Initial state of causal segment seg: the scanned prefix from the workspace,
// or S0/z0 when the head is one segment.
template <class K>
__device__ __forceinline__ void load_state(const Params& p, int64_t head, int seg, int fb0, int lane,
                                           f32x4 (&st)[K::FBW][K::NE]) {
  load_state_item<K>(p, head, p.n_seg > 1, head * p.p1_items + (int64_t)seg * p.sub, fb0, lane, st);
}

// Final state of state row `head` (a head; for a variable-length batch,
// sequence * n_heads + head) for the wave's feature blocks.
template <class K>
// Addresses are a wave-uniform base plus one 32-bit lane offset, so the
// stores add few live registers where they sit inside a chunk loop.
__device__ __forceinline__ void store_state_out(const Params& p, int64_t head, int fb0, int lane,
                                                const f32x4 (&st)[K::FBW][K::NE]) {
  const int g = lane >> 4, col = lane & 15;
  const int64_t row0 = head * K::F + fb0 * 16;  // first feature row of the wave
  if (p.S_out) {
    float* base = p.S_out + row0 * K::DV;
    const uint32_t off = (uint32_t)(4 * g * K::DV + col);
#pragma unroll
    for (int j = 0; j < K::FBW; ++j)
#pragma unroll
      for (int et = 0; et < K::NE - 1; ++et)  // tile NE-1 holds z and padding
#pragma unroll
        for (int i = 0; i < 4; ++i) base[(j * 16 + i) * K::DV + et * 16 + off] = st[j][et][i];
  }
  if (p.z_out && col == 0) {
    float* base = p.z_out + row0;
    const uint32_t off = (uint32_t)(4 * g);
#pragma unroll
    for (int j = 0; j < K::FBW; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) base[j * 16 + i + off] = st[j][K::NE - 1][i];
  }
}

// ---------------------------------------------------------------------------
// pass 1: per-segment state deltas.  Every workgroup stages the whole chunk;
// the F features are split over FS workgroups of NW/FS waves.  One barrier
// per chunk, software pipelined over chunks: step c stages chunk c+1 (loaded
// one step earlier) and computes phi(k) of chunk c while the state update of
// chunk c-1 runs beside it, so MFMA and VALU work of two chunks overlap.
// k tiles are double-buffered, v'^T triple-buffered (chunk c-1 is still read
// while chunk c+1 is staged), and phi(k) alternates between two register sets.
// At least 2 waves per SIMD are asked for (the 4-wave shape would otherwise
// keep MFMA results in accumulator registers, each copied out by a VALU op).
template <class K, int FS>
__global__ __launch_bounds__(K::NT / FS, 2) void pass1_kernel(Params p) {
  constexpr int NT1 = K::NT / FS;
  extern __shared__ __align__(16) unsigned char lds[];
  auto sK = [&](int b) { return reinterpret_cast<uint16_t*>(lds + b * K::kKbuf1); };
  auto sInv = [&](int b) { return reinterpret_cast<float*>(lds + b * K::kKbuf1 + K::C * K::LDX * 2); };
  auto sV = [&](int b) { return reinterpret_cast<uint16_t*>(lds + 2 * K::kKbuf1 + b * K::kVbuf); };

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nsub = p.p1_segs;  // sub-segments covered by pass 1
  const int n_items = p.p1_items;
  const int fs = (int)(blockIdx.x % FS);
  const int64_t hs = blockIdx.x / FS;
  const int64_t head = hs / nsub;
  const int seg = (int)(hs - head * nsub);  // sub-segment index
  const int set = (int)(head % p.n_draw_sets);
  const int fb0 = (fs * (K::NW / FS) + wave) * K::FBW;

  bf16x8 pa[K::FBW][K::NKS], pg[K::FBW][K::NKS];
  float c1[K::FBW], c0[K::FBW];
  load_p<K>(p, set, fb0, lane, pa, pg, c1, c0);
  f32x4 st[K::FBW][K::NE];
#pragma unroll
  for (int j = 0; j < K::FBW; ++j)
#pragma unroll
    for (int et = 0; et < K::NE; ++et) st[j][et] = f32x4{0.f, 0.f, 0.f, 0.f};
  // phi(k) of the current and the previous chunk; the "previous" of chunk 0
  // is zero and meets the zeroed value rows of v'^T buffer 2
  bf16x8 kfa[K::FBW][K::NTS] = {}, kfb[K::FBW][K::NTS] = {};
  const RowOff<K, K::LDV> vo(lane & 15);
  for (int t = threadIdx.x; t < K::DV * K::LDV / 2; t += NT1) reinterpret_cast<uint32_t*>(sV(2))[t] = 0u;
  init_vconst<K, NT1>(threadIdx.x, sV(0));
  init_vconst<K, NT1>(threadIdx.x, sV(1));
  init_vconst<K, NT1>(threadIdx.x, sV(2));

  const int64_t sub_len = p.seg_len / p.sub;
  const int64_t t0 = (int64_t)seg * sub_len;
  const int64_t t1 = min<int64_t>(p.L, t0 + sub_len);
  const int nch = (int)((t1 - t0 + K::C - 1) / K::C);
  Prefetch<K, NT1> pf;
  auto load_chunk = [&](int cc) {  // chunk min(cc, nch-1): the last one again past the end
    const int64_t c2 = t0 + (int64_t)min(cc, nch - 1) * K::C;
    issue_loads<K, NT1>(threadIdx.x, p, head * p.L, c2, (int)min<int64_t>(K::C, t1 - c2), false, pf);
  };
  load_chunk(0);
  store_x<K, NT1>(threadIdx.x, pf.k, sK(0), sInv(0), sInv(0) + K::C);
  store_v<K, NT1>(threadIdx.x, pf.v0, pf.v1, sV(0));
  load_chunk(1);
  __syncthreads();
  // step c: chunk c's phi(k) into kf_cur, chunk c-1's state update from kf_prev
  auto step = [&](int c, bf16x8(&kf_cur)[K::FBW][K::NTS], const bf16x8(&kf_prev)[K::FBW][K::NTS]) {
    const int bn = (c + 1) & 1, vn = (c + 1) % 3;
    store_x<K, NT1>(threadIdx.x, pf.k, sK(bn), sInv(bn), sInv(bn) + K::C);
    store_v<K, NT1>(threadIdx.x, pf.v0, pf.v1, sV(vn));
    load_chunk(c + 2);
    const int b = c & 1;
    phase_k<K, false, true>(sK(b), sInv(b), sInv(b) + K::C, nullptr, fb0, lane, pa, pg, c1, c0, kf_cur,
                            sV((c + 2) % 3), vo, kf_prev, st);
    __syncthreads();
  };
  for (int c = 0; c < nch; c += 2) {
    step(c, kfa, kfb);
    if (c + 1 < nch) step(c + 1, kfb, kfa);
  }
  // state update of the last chunk
  const uint16_t* sv_last = sV((nch - 1) % 3);
  if (nch & 1) {
#pragma unroll
    for (int s_ = 0; s_ < K::NTS; ++s_) state_update_step<K>(sv_last, vo, lane, s_, kfa, st);
  } else {
#pragma unroll
    for (int s_ = 0; s_ < K::NTS; ++s_) state_update_step<K>(sv_last, vo, lane, s_, kfb, st);
  }
  float* out = p.ws + (head * n_items + seg) * (int64_t)K::F * K::DVP;
#pragma unroll
  for (int j = 0; j < K::FBW; ++j)
#pragma unroll
    for (int et = 0; et < K::NE; ++et)
      *reinterpret_cast<f32x4*>(out + frag_off<K>(fb0 + j, et, lane)) = st[j][et];
}

// Pass 1 with 4 stager waves beside the NW feature waves: the stagers load
// and stage k and v'^T (and the row scales of k); the feature waves only run
// phi(k) and the state update.  Same buffers and one barrier per chunk as
// pass1_kernel: in the interval of chunk c the stagers write chunk c+1 and
// load chunk c+2 while the feature waves process chunk c.
template <class K, bool VL>
__global__ __launch_bounds__(K::NT + 256) void pass1s_kernel(Params p) {
  constexpr int NS = 256;  // stager threads
  extern __shared__ __align__(16) unsigned char lds[];
  auto sK = [&](int b) { return reinterpret_cast<uint16_t*>(lds + b * K::kKbuf1); };
  auto sInv = [&](int b) { return reinterpret_cast<float*>(lds + b * K::kKbuf1 + K::C * K::LDX * 2); };
  auto sV = [&](int b) { return reinterpret_cast<uint16_t*>(lds + 2 * K::kKbuf1 + b * K::kVbuf); };

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const Chunks<K, VL> ch = chunks_of<K, VL>(p, p.p1_segs, p.seg_len / p.sub, p.p1_items,
                                            reinterpret_cast<int4*>(lds + K::kLds1), K::NT + NS);
  if (!ch.valid) return;  // a variable-length launch's spare work item (whole workgroup)
  if constexpr (VL) __syncthreads();  // chunk list in LDS
  const int64_t head = ch.head;
  const int set = (int)(head % p.n_draw_sets);
  const int nch = ch.nch;

  for (int t = threadIdx.x; t < K::DV * K::LDV / 2; t += K::NT + NS) reinterpret_cast<uint32_t*>(sV(2))[t] = 0u;
  for (int b = 0; b < 3; ++b) init_vconst<K, K::NT + NS>(threadIdx.x, sV(b));

  if (wave < K::NW) {  // feature waves
    const int fb0 = wave * K::FBW;
    bf16x8 pa[K::FBW][K::NKS], pg[K::FBW][K::NKS];
    float c1[K::FBW], c0[K::FBW];
    load_p<K>(p, set, fb0, lane, pa, pg, c1, c0);
    f32x4 st[K::FBW][K::NE];
#pragma unroll
    for (int j = 0; j < K::FBW; ++j)
#pragma unroll
      for (int et = 0; et < K::NE; ++et) st[j][et] = f32x4{0.f, 0.f, 0.f, 0.f};
    // phi(k) of the current and the previous chunk; the "previous" of chunk 0
    // is zero and meets the zeroed value rows of v'^T buffer 2
    bf16x8 kfa[K::FBW][K::NTS] = {}, kfb[K::FBW][K::NTS] = {};
    const RowOff<K, K::LDV> vo(lane & 15);
    __syncthreads();  // chunk 0 staged
    auto step = [&](int c, bf16x8(&kf_cur)[K::FBW][K::NTS], const bf16x8(&kf_prev)[K::FBW][K::NTS]) {
      const int b = c & 1;
      phase_k<K, false, true>(sK(b), sInv(b), sInv(b) + K::C, nullptr, fb0, lane, pa, pg, c1, c0, kf_cur,
                              sV((c + 2) % 3), vo, kf_prev, st);
      mfma_valu_interleave<K::NTB * K::FBW * K::NKS * 2 + K::NTS * K::NE * K::FBW, 3>();
      __syncthreads();
    };
    for (int c = 0; c < nch; c += 2) {
      step(c, kfa, kfb);
      if (c + 1 < nch) step(c + 1, kfb, kfa);
    }
    const uint16_t* sv_last = sV((nch - 1) % 3);
    if (nch & 1) {
#pragma unroll
      for (int s_ = 0; s_ < K::NTS; ++s_) state_update_step<K>(sv_last, vo, lane, s_, kfa, st);
    } else {
#pragma unroll
      for (int s_ = 0; s_ < K::NTS; ++s_) state_update_step<K>(sv_last, vo, lane, s_, kfb, st);
    }
    // one piece per workgroup (variable-length packs never come here)
    float* out = p.ws + ch.at(0).item * (int64_t)K::F * K::DVP;
#pragma unroll
    for (int j = 0; j < K::FBW; ++j)
#pragma unroll
      for (int et = 0; et < K::NE; ++et)
        *reinterpret_cast<f32x4*>(out + frag_off<K>(fb0 + j, et, lane)) = st[j][et];
  } else {  // stagers
    const int stid = threadIdx.x - K::NT;
    Prefetch<K, NS> pf;
    auto load_chunk = [&](int cc) {  // chunk min(cc, nch-1): the last one again past the end
      const ChunkRef r = ch.at(min(cc, nch - 1));
      issue_loads<K, NS>(stid, p, r.row, 0, r.n, false, pf);
    };
    load_chunk(0);
    store_x<K, NS>(stid, pf.k, sK(0), sInv(0), sInv(0) + K::C);
    store_v<K, NS>(stid, pf.v0, pf.v1, sV(0));
    load_chunk(1);
    __syncthreads();  // chunk 0 staged
    for (int c = 0; c < nch; ++c) {
      const int bn = (c + 1) & 1;
      // chunk c+1 (a repeat of the last past the end; never read then)
      store_x<K, NS>(stid, pf.k, sK(bn), sInv(bn), sInv(bn) + K::C);
      store_v<K, NS>(stid, pf.v0, pf.v1, sV((c + 1) % 3));
      load_chunk(c + 2);
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------------------
// Warp-specialized main pass.  NP producer waves own the features (their
// slice of P and of the state S' in registers) and NC = 4 consumer waves own
// the contractions, so the feature map (VALU) of chunk c+1 runs beside the
// contractions (MFMA and LDS) of chunk c.  phi(q), phi(k) are double-buffered
// in LDS, the staged q, k tiles double- and v'^T triple-buffered.  Per chunk:
//   [A] consumers: intra + inter of chunk c for their (token block, column
//       half), staging of chunk c+2, loads of chunk c+3; producers: phi(k),
//       phi(q) of chunk c+1 with the state update by chunk c spread through
//       the phi(k) pipeline;
//   [B] producers refresh the bf16 S'^T copy; consumers of the first column
//       half write their outputs (the denominator comes from the other half).
template <int D_, int DV_, int NP_, int FBW_>
struct CfgS : Cfg<D_, DV_, 32, NP_, FBW_> {
  using B = Cfg<D_, DV_, 32, NP_, FBW_>;
  static constexpr int NP = NP_, NC = 4;
  static constexpr bool PIPE = false;  // consumers run beside the producers; keep registers low
  static constexpr int NTW = (NP + NC) * 64;           // threads
  static constexpr int ESPLIT = (B::NE + 1) / 2;       // column tiles [0, ESPLIT) | [ESPLIT, NE)
  static constexpr int kXt = B::C * B::LDX * 2;        // one staged x tile (bytes)
  static constexpr int kPt = B::C * B::LDF * 2;        // one phi tile
  static constexpr int kSQ = 0;                        // sQ[2]
  static constexpr int kSK = kSQ + 2 * kXt;            // sK[2]
  static constexpr int kSV = kSK + 2 * kXt;            // v'^T [3]
  static constexpr int kSPq = kSV + 3 * B::kVbuf;      // phi(q) [2]
  static constexpr int kSPk = kSPq + 2 * kPt;          // phi(k) [2]
  static constexpr int kSSt = kSPk + 2 * kPt;          // bf16 S'^T
  static constexpr int kSInv = kSSt + B::VROWS * B::LDF * 2;  // [2][inv q, lg q, inv k, lg k][C]
  static constexpr int kSDen = kSInv + 2 * 4 * B::C * 4;      // [NTB][16] denominators
  static constexpr int kLdsS = kSDen + B::NTB * 16 * 4;
  static_assert(B::NTB == 2 && B::NTS == 1, "one consumer per (token block, column half)");
  static_assert(kLdsS <= 160 * 1024, "LDS budget");
};

// Consumer task: columns [E0, E1) of num'^T for token block IB of the staged
// chunk = intra (A^T of the causal blocks, then v'^T A^T) + inter (S'^T phi(q)^T).
template <class K, int IB, int E0, int E1>
__device__ __forceinline__ void consumer_task(const uint16_t* sPq, const uint16_t* sPk, const uint16_t* sVc,
                                              const uint16_t* sSt, const RowOff<K, K::LDV>& vo,
                                              const RowOff<K, K::LDF>& so, int lane, f32x4 (&acc)[E1 - E0]) {
  const int g = lane >> 4, col = lane & 15;
  f32x4 at[IB + 1];
#pragma unroll
  for (int kf_ = 0; kf_ < K::NFK; ++kf_) {
    const bf16x8 bq = as_bf16x8(*reinterpret_cast<const uint4*>(sPq + (IB * 16 + col) * K::LDF + kf_ * 32 + 8 * g));
#pragma unroll
    for (int jb = 0; jb <= IB; ++jb) {
      const bf16x8 ak = as_bf16x8(*reinterpret_cast<const uint4*>(sPk + (jb * 16 + col) * K::LDF + kf_ * 32 + 8 * g));
      at[jb] = mfma_bf16(ak, bq, kf_ == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : at[jb]);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (4 * g + i > col) at[IB][i] = 0.f;  // causal mask, diagonal block: keep j <= i
  const uint2 lo = pack4(at[0][0], at[0][1], at[0][2], at[0][3]);
  uint2 hi = make_uint2(0, 0);
  if constexpr (IB == 1) hi = pack4(at[IB][0], at[IB][1], at[IB][2], at[IB][3]);
  const bf16x8 ab = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
#pragma unroll
  for (int et = E0; et < E1; ++et) acc[et - E0] = mfma_bf16(vfrag<K>(sVc, vo, et, 0, lane), ab, f32x4{0.f, 0.f, 0.f, 0.f});
  const uint16_t* q0 = sPq + (IB * 16 + col) * K::LDF + 8 * g;
#pragma unroll
  for (int kf_ = 0; kf_ < K::NFK; ++kf_) {
    const bf16x8 bq = as_bf16x8(*reinterpret_cast<const uint4*>(q0 + kf_ * 32));
#pragma unroll
    for (int et = E0; et < E1; ++et) {
      const bf16x8 as = as_bf16x8(*reinterpret_cast<const uint4*>(sSt + so.off[et] + kf_ * 32 + 8 * g));
      acc[et - E0] = mfma_bf16(as, bq, acc[et - E0]);
    }
  }
}

// o = num / den for columns [E0, E1) of token block IB (den of token col in rden).
template <class K, int IB, int E0, int E1>
__device__ __forceinline__ void consumer_out(const Params& p, int64_t row0, int n, int lane, float rden,
                                             const f32x4 (&acc)[E1 - E0]) {
  const int g = lane >> 4, col = lane & 15;
  const int tok = IB * 16 + col;
  if (tok < n) {
    uint16_t* orow = p.o + (row0 + tok) * K::DV;
#pragma unroll
    for (int et = E0; et < E1; ++et) {
      if (et * 16 >= K::DV) continue;  // the z / padding tile
      *reinterpret_cast<uint2*>(orow + et * 16 + 4 * g) =
          pack4(acc[et - E0][0] * rden, acc[et - E0][1] * rden, acc[et - E0][2] * rden, acc[et - E0][3] * rden);
    }
  }
}

template <class K, int IB, int H>
__device__ __forceinline__ void consumer_step(const Params& p, int64_t row0, int n, const uint16_t* sPq,
                                              const uint16_t* sPk, const uint16_t* sVc, const uint16_t* sSt,
                                              float* sDen, const RowOff<K, K::LDV>& vo, const RowOff<K, K::LDF>& so,
                                              int lane, f32x4 (&acc0)[K::ESPLIT]) {
  if constexpr (H == 0) {
    consumer_task<K, IB, 0, K::ESPLIT>(sPq, sPk, sVc, sSt, vo, so, lane, acc0);
  } else {
    f32x4 acc1[K::NE - K::ESPLIT];
    consumer_task<K, IB, K::ESPLIT, K::NE>(sPq, sPk, sVc, sSt, vo, so, lane, acc1);
    // den of token col: element (row DV, column col) of the last tile
    const int col = lane & 15;
    const float den = __shfl(acc1[K::NE - 1 - K::ESPLIT][0], col, 64);
    if (lane < 16) sDen[IB * 16 + lane] = den;
    consumer_out<K, IB, K::ESPLIT, K::NE>(p, row0, n, lane, __builtin_amdgcn_rcpf(den), acc1);
  }
}

template <class K, bool VL>
__global__ __launch_bounds__(K::NTW) void pass2s_kernel(Params p) {
  extern __shared__ __align__(16) unsigned char lds[];
  auto sQ = [&](int b) { return reinterpret_cast<uint16_t*>(lds + K::kSQ + b * K::kXt); };
  auto sK = [&](int b) { return reinterpret_cast<uint16_t*>(lds + K::kSK + b * K::kXt); };
  auto sV = [&](int b) { return reinterpret_cast<uint16_t*>(lds + K::kSV + b * K::kVbuf); };
  auto sPq = [&](int b) { return reinterpret_cast<uint16_t*>(lds + K::kSPq + b * K::kPt); };
  auto sPk = [&](int b) { return reinterpret_cast<uint16_t*>(lds + K::kSPk + b * K::kPt); };
  auto sInv = [&](int b, int w) { return reinterpret_cast<float*>(lds + K::kSInv) + (b * 4 + w) * K::C; };
  uint16_t* sSt = reinterpret_cast<uint16_t*>(lds + K::kSSt);
  float* sDen = reinterpret_cast<float*>(lds + K::kSDen);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15;
  const bool producer = wave < K::NP;
  const int cw = wave - K::NP;           // consumer index: token block cw >> 1, column half cw & 1
  const int ctid = threadIdx.x - K::NP * 64;  // thread index among the consumers
  const Chunks<K, VL> ch = chunks_of<K, VL>(p, p.n_seg, p.seg_len, p.p1_items,
                                            reinterpret_cast<int4*>(lds + K::kLdsS), K::NTW);
  if (!ch.valid) return;  // a variable-length launch's spare work item (whole workgroup)
  if constexpr (VL) __syncthreads();  // chunk list in LDS
  const int64_t head = ch.head;
  const int set = (int)(head % p.n_draw_sets);
  const int fb0 = (producer ? wave : 0) * K::FBW;

  const RowOff<K, K::LDV> vo(col);
  const RowOff<K, K::LDF> so(col);
  for (int b = 0; b < 3; ++b) init_vconst<K, K::NTW>(threadIdx.x, sV(b));
  for (int t = threadIdx.x; t < K::LDF; t += K::NTW) sSt[(K::DV + 1) * K::LDF + t] = 0;
  const int nch = ch.nch;

  // Producers and consumers run separate code (so each keeps only its own
  // registers live); both execute the same barriers: two in the prologue and
  // two per chunk.
  if (producer) {
    bf16x8 pa[K::FBW][K::NKS], pg[K::FBW][K::NKS];
    float c1[K::FBW], c0[K::FBW];
    f32x4 st[K::FBW][K::NE];
    bf16x8 kf[K::FBW][K::NTS] = {};
    load_p<K>(p, set, fb0, lane, pa, pg, c1, c0);
    load_state_item<K>(p, head, VL || p.n_seg > 1, ch.at(0).item, fb0, lane, st);
    write_st<K>(sSt, so, wave, lane, st);
    __syncthreads();  // chunks 0 and 1 staged
    phase_k<K, true, false>(sK(0), sInv(0, 2), sInv(0, 3), sPk(0), fb0, lane, pa, pg, c1, c0, kf, nullptr, vo, kf, st);
    phase_q<K>(sQ(0), sInv(0, 0), sInv(0, 1), sPq(0), wave, lane, pa, pg, c1, c0);
    __syncthreads();  // phi of chunk 0 in LDS
    // ---- [B] S'^T copy of the state before chunk c+1: the state after
    // chunk c, or (variable-length) a new piece's initial state from the scan ----
    auto interval_b = [&](int c) {
      __syncthreads();  // B
      if constexpr (VL) {
        const ChunkRef r = ch.at(c);  // the state after a sequence's last chunk is its final state
        if ((r.flags & kSeqEnd) && (p.S_out || p.z_out))
          store_state_out<K>(p, (int64_t)r.seq * p.n_heads + head, fb0, lane, st);
        if (c + 1 < nch) {
          const ChunkRef r1 = ch.at(c + 1);
          if (r1.flags & kFirst) load_state_item<K>(p, head, true, r1.item, fb0, lane, st);
        }
      }
      write_st<K>(sSt, so, wave, lane, st);
      __syncthreads();  // A
    };
    // the last chunk is peeled off, so the loop body holds no branch that
    // writes the state accumulators two ways
    for (int c = 0; c < nch - 1; ++c) {
      const int bn = (c & 1) ^ 1;
      // ---- [A] phi of chunk c+1, state update by chunk c ----
      phase_k<K, true, true>(sK(bn), sInv(bn, 2), sInv(bn, 3), sPk(bn), fb0, lane, pa, pg, c1, c0, kf, sV(c % 3), vo,
                             kf, st);
      phase_q<K>(sQ(bn), sInv(bn, 0), sInv(bn, 1), sPq(bn), wave, lane, pa, pg, c1, c0);
      mfma_valu_interleave<K::NTB * K::FBW * K::NKS * 4 + K::NTS * K::NE * K::FBW, 3>();
      interval_b(c);
    }
    {  // [A] of the last chunk: its state update only
      const uint16_t* sVc = sV((nch - 1) % 3);
#pragma unroll
      for (int s_ = 0; s_ < K::NTS; ++s_) state_update_step<K>(sVc, vo, lane, s_, kf, st);
      interval_b(nch - 1);
    }
    if (!VL && ch.geo.seg == p.n_seg - 1 && (p.S_out || p.z_out)) store_state_out<K>(p, head, fb0, lane, st);
  } else {
    // The SIMD issues from the highest-priority ready wave first: consumers
    // (MFMA and LDS, little VALU) go ahead of the VALU-heavy producers, which
    // fill the issue slots the consumers leave while they wait on LDS.
    __builtin_amdgcn_s_setprio(2);
    Prefetch<K, K::NC * 64> pf;
    auto load_chunk = [&](int cc) {  // chunk min(cc, nch-1): the last one again past the end
      const ChunkRef r = ch.at(min(cc, nch - 1));
      issue_loads<K, K::NC * 64>(ctid, p, r.row, 0, r.n, true, pf);
    };
    auto stage = [&](int bx, int bv) {
      store_x<K, K::NC * 64>(ctid, pf.q, sQ(bx), sInv(bx, 0), sInv(bx, 1));
      store_x<K, K::NC * 64>(ctid, pf.k, sK(bx), sInv(bx, 2), sInv(bx, 3));
      store_v<K, K::NC * 64>(ctid, pf.v0, pf.v1, sV(bv));
    };
    // prologue: chunks 0 and 1 staged, chunk 2 in flight
    load_chunk(0);
    stage(0, 0);
    load_chunk(1);
    stage(1, 1);
    load_chunk(2);
    __syncthreads();
    __syncthreads();
    // one loop per consumer role, so each keeps only its own addresses live
    auto consumer_loop = [&](auto ib_c, auto h_c) {
      constexpr int IB = decltype(ib_c)::value, H = decltype(h_c)::value;
      for (int c = 0; c < nch; ++c) {
        const int b = c & 1;
        const ChunkRef r = ch.at(c);
        const int64_t row0 = r.row;
        const int n = r.n;
        f32x4 acc0[K::ESPLIT];
        // ---- [A] contractions of chunk c; staging of chunk c+2 ----
        consumer_step<K, IB, H>(p, row0, n, sPq(b), sPk(b), sV(c % 3), sSt, sDen, vo, so, lane, acc0);
        stage(b, (c + 2) % 3);  // chunk c+2 (a repeat of the last past the end; never read then)
        load_chunk(c + 3);
        __syncthreads();  // B
        // ---- [B] first column half: outputs with the other half's denominators ----
        if constexpr (H == 0) {
          const float rden = __builtin_amdgcn_rcpf(sDen[IB * 16 + col]);
          consumer_out<K, IB, 0, K::ESPLIT>(p, row0, n, lane, rden, acc0);
        }
        __syncthreads();  // A
      }
    };
    switch (cw) {  // wave-uniform
      case 0: consumer_loop(std::integral_constant<int, 0>(), std::integral_constant<int, 0>()); break;
      case 1: consumer_loop(std::integral_constant<int, 0>(), std::integral_constant<int, 1>()); break;
      case 2: consumer_loop(std::integral_constant<int, 1>(), std::integral_constant<int, 0>()); break;
      default: consumer_loop(std::integral_constant<int, 1>(), std::integral_constant<int, 1>()); break;
    }
  }
}

// ---------------------------------------------------------------------------
// Non-causal output pass: o = phi(q)^T S' / phi(q)^T z over the state of all
// keys (the total from the workspace, or S0/z0 when there are no keys).  One
// workgroup per (head, query segment); each wave keeps its feature slice of P
// in registers and writes its slice of the bf16 S'^T copy once.  Per chunk c
// of 64 queries, one barrier: the inter tasks of chunk c (one per (16-query
// block, column half)) beside phi(q) of chunk c+1 and the staging of c+2.

// Inter task for query block IB, column half H of num'^T = S'^T phi(q)^T,
// then o = num / den for that half; each half also computes the denominator
// tile (the z row), so the halves need no exchange.
template <class K, int H>
__device__ __forceinline__ void nc_task(const Params& p, int64_t row0, int n, int ib, const uint16_t* sPq,
                                        const uint16_t* sSt, const RowOff<K, K::LDF>& so, int lane) {
  constexpr int NV = K::NE - 1;         // value tiles
  constexpr int NH = NV / 2 + 1;        // tiles of this half, the last one the denominator tile
  const int g = lane >> 4, col = lane & 15;
  auto tile = [](int i) { return i < NH - 1 ? H * (NV / 2) + i : K::NE - 1; };
  f32x4 acc[NH];
  const uint16_t* q0 = sPq + (ib * 16 + col) * K::LDF + 8 * g;
#pragma unroll
  for (int kf_ = 0; kf_ < K::NFK; ++kf_) {
    const bf16x8 bq = as_bf16x8(*reinterpret_cast<const uint4*>(q0 + kf_ * 32));
#pragma unroll
    for (int i = 0; i < NH; ++i) {
      const bf16x8 as = as_bf16x8(*reinterpret_cast<const uint4*>(sSt + so.off[tile(i)] + kf_ * 32 + 8 * g));
      acc[i] = mfma_bf16(as, bq, kf_ == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[i]);
    }
  }
  const float rden = __builtin_amdgcn_rcpf(__shfl(acc[NH - 1][0], col, 64));
  const int tok = ib * 16 + col;
  if (tok < n) {
    uint16_t* orow = p.o + (row0 + tok) * K::DV;
#pragma unroll
    for (int i = 0; i < NH - 1; ++i)
      *reinterpret_cast<uint2*>(orow + tile(i) * 16 + 4 * g) =
          pack4(acc[i][0] * rden, acc[i][1] * rden, acc[i][2] * rden, acc[i][3] * rden);
  }
}

// (at least 2 waves per SIMD, for the reason given at pass1_kernel)
template <class K>
__global__ __launch_bounds__(K::NT, 2) void ncout_kernel(Params p) {
  constexpr int kXt = K::C * K::LDX * 2, kPt = K::C * K::LDF * 2;
  extern __shared__ __align__(16) unsigned char lds[];
  auto sQ = [&](int b) { return reinterpret_cast<uint16_t*>(lds + b * kXt); };
  auto sInv = [&](int b) { return reinterpret_cast<float*>(lds + 2 * kXt) + b * 2 * K::C; };
  auto sPq = [&](int b) { return reinterpret_cast<uint16_t*>(lds + 2 * kXt + 4 * K::C * 4 + b * kPt); };
  uint16_t* sSt = reinterpret_cast<uint16_t*>(lds + 2 * kXt + 4 * K::C * 4 + 2 * kPt);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15;
  const int64_t head = blockIdx.x / p.n_qseg;
  const int qs = (int)(blockIdx.x - head * p.n_qseg);
  const int set = (int)(head % p.n_draw_sets);
  const int fb0 = wave * K::FBW;

  bf16x8 pa[K::FBW][K::NKS], pg[K::FBW][K::NKS];
  float c1[K::FBW], c0[K::FBW];
  load_p<K>(p, set, fb0, lane, pa, pg, c1, c0);
  const RowOff<K, K::LDF> so(col);
  {
    f32x4 st[K::FBW][K::NE];
    load_state_item<K>(p, head, p.L > 0, head * p.p1_items + p.p1_items - 1, fb0, lane, st);
    write_st<K>(sSt, so, wave, lane, st);
  }
  for (int t = threadIdx.x; t < K::LDF; t += K::NT) sSt[(K::DV + 1) * K::LDF + t] = 0;

  const int64_t t0 = (int64_t)qs * p.qseg_len;
  const int64_t t1 = min<int64_t>(p.Lq, t0 + p.qseg_len);
  const int nch = (int)((t1 - t0 + K::C - 1) / K::C);
  Prefetch<K> pf;
  auto load_chunk = [&](int cc) {  // chunk min(cc, nch-1): the last one again past the end
    const int64_t c2 = t0 + (int64_t)min(cc, nch - 1) * K::C;
    load_x<K>(threadIdx.x, p.q + (head * p.Lq + c2) * K::D, (int)min<int64_t>(K::C, t1 - c2), pf.q);
  };
  load_chunk(0);
  store_x<K>(threadIdx.x, pf.q, sQ(0), sInv(0), sInv(0) + K::C);
  load_chunk(1);
  __syncthreads();
  phase_q<K>(sQ(0), sInv(0), sInv(0) + K::C, sPq(0), wave, lane, pa, pg, c1, c0);
  store_x<K>(threadIdx.x, pf.q, sQ(1), sInv(1), sInv(1) + K::C);
  load_chunk(2);
  __syncthreads();
  for (int c = 0; c < nch; ++c) {
    const int b = c & 1;
    const int64_t row0 = head * p.Lq + t0 + (int64_t)c * K::C;
    const int n = (int)min<int64_t>(K::C, t1 - (t0 + (int64_t)c * K::C));
    // Vector loads and stores retire in issue order and share one counter:
    // the rows of chunk c+2 (loaded before the previous chunk's feature map)
    // are waited for here, before this chunk's output stores, so that their
    // staging below does not also wait for those stores.
    wait_vmem();
    for (int t = wave; t < 2 * K::NTB; t += K::NW) {  // wave-uniform task loop
      if (t & 1) nc_task<K, 1>(p, row0, n, t >> 1, sPq(b), sSt, so, lane);
      else nc_task<K, 0>(p, row0, n, t >> 1, sPq(b), sSt, so, lane);
    }
    // chunk c+2 into the x buffer chunk c used (phase_q below reads the other)
    store_x<K>(threadIdx.x, pf.q, sQ(b), sInv(b), sInv(b) + K::C);  // a repeat past the end
    load_chunk(c + 3);
    if (c + 1 < nch) phase_q<K>(sQ(b ^ 1), sInv(b ^ 1), sInv(b ^ 1) + K::C, sPq(b ^ 1), wave, lane, pa, pg, c1, c0);
    __syncthreads();
  }
}

// The non-causal output pass reads phi(q) and the bf16 S'^T copy only as
// 16-byte MFMA operands (16 rows per access), which run without bank
// conflicts at a row stride of 32 (mod 64) bytes: F + 16 elements.  The
// causal passes keep F + 8, with which their mix of accesses measured faster.
template <class K>
struct NcCfg : K {
  static constexpr int LDF = K::F + 16;
};

template <class K>
constexpr int ncout_lds() {
  return 2 * K::C * K::LDX * 2 + 4 * K::C * 4 + 2 * K::C * K::LDF * 2 + K::VROWS * K::LDF * 2;
}

typedef Cfg<64, 64, 64, 8, 2> CfgF256;
typedef Cfg<64, 64, 64, 8, 1> CfgF128;
typedef Cfg<64, 64, 64, 6, 1> CfgF96;
typedef Cfg<64, 64, 64, 4, 1> CfgF64;

// Main-pass configuration for a segment-pass configuration: the same feature
// waves as producers, 32-token chunks; both use the same segments and the
// same fragment-ordered workspace.
template <class K>
struct MainPass {
  using type = CfgS<K::D, K::DV, K::NW, K::FBW>;
};

// Segments per head for n_heads heads of L tokens: enough workgroups to fill
// the chip (about 256), each an even number of chunks.
template <class K>
int pick_segments(int64_t n_heads, int64_t L) {
  const int64_t n_chunks = (L + K::C - 1) / K::C;
  int64_t want = (256 + n_heads - 1) / n_heads;
  if (want > n_chunks) want = n_chunks;
  if (want < 1) want = 1;
  const int64_t cps = (n_chunks + want - 1) / want;  // chunks per segment
  return (int)((n_chunks + cps - 1) / cps);
}

template <class K>
int64_t seg_len_of(int64_t L, int n_seg) {
  const int64_t n_chunks = (L + K::C - 1) / K::C;
  const int64_t cps = (n_chunks + n_seg - 1) / n_seg;
  return ((cps + 1) / 2) * 2 * K::C;  // an even number of chunks
}

template <class K>
int64_t seg_len_for(int64_t n_heads, int64_t L) {
  return seg_len_of<K>(L, pick_segments<K>(n_heads, L));
}

template <class K>
int segments_of(int64_t n_heads, int64_t L) {
  const int64_t seg_len = seg_len_for<K>(n_heads, L);
  return (int)((L + seg_len - 1) / seg_len);
}

template <class K>
int segments_of(const ChunkedArgs& a) {
  return segments_of<K>(a.n_heads, a.L);
}

constexpr int kSub = 1;  // pass-1 sub-segments per segment

template <class K>
size_t ws_bytes_t(const ChunkedArgs& a) {
  const int n_seg = segments_of<K>(a);
  return n_seg > 1 ? sizeof(float) * (size_t)a.n_heads * ((n_seg - 1) * kSub + 1) * K::F * K::DVP : 0;
}

template <class K>
hipError_t launch_t(const ChunkedArgs& a, hipStream_t s) {
  const int n_seg = segments_of<K>(a);
  Params p{};
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.o = static_cast<uint16_t*>(a.o);
  p.L = a.L;
  p.n_seg = n_seg;
  p.seg_len = seg_len_for<K>(a.n_heads, a.L);
  p.sub = kSub;
  p.p1_segs = (n_seg - 1) * kSub;
  p.p1_items = p.p1_segs + 1;
  p.Lq = a.L;
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
    if constexpr (K::STAGERS1) {
      e = set_max_lds(reinterpret_cast<const void*>(&pass1s_kernel<K, false>), K::kLds1);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL((pass1s_kernel<K, false>), dim3((unsigned)(a.n_heads * (n_seg - 1) * kSub)), dim3(K::NT + 256),
                         K::kLds1, s, p);
    } else {
      constexpr int FS = K::FS1;
      e = set_max_lds(reinterpret_cast<const void*>(&pass1_kernel<K, FS>), K::kLds1);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL((pass1_kernel<K, FS>), dim3((unsigned)(a.n_heads * (n_seg - 1) * kSub * FS)),
                         dim3(K::NT / FS), K::kLds1, s, p);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    ScanArgs sa{};
    sa.states = p.ws;
    sa.n_heads = a.n_heads;
    sa.n_items = (n_seg - 1) * kSub + 1;
    sa.n_terms = (n_seg - 1) * kSub;
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
  using KS = typename MainPass<K>::type;
  e = set_max_lds(reinterpret_cast<const void*>(&pass2s_kernel<KS, false>), KS::kLdsS);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((pass2s_kernel<KS, false>), dim3((unsigned)(a.n_heads * n_seg)), dim3(KS::NTW), KS::kLdsS, s,
                     p);
  return hipGetLastError();
}

template <typename Fn>
bool dispatch(const ChunkedArgs& a, Fn&& fn) {
  if (!a.io_bf16 || a.d != 64 || a.dv != 64 || a.chunk != 64 || a.m % 16 != 0) return false;
  switch (a.F) {
    case 256:
      if (a.m % 32 != 0) return false;  // a wave's two feature blocks must share a node
      fn(CfgF256());
      return true;
    case 128: fn(CfgF128()); return true;
    case 96: fn(CfgF96()); return true;
    case 64: fn(CfgF64()); return true;
    default: return false;
  }
}

// Non-causal: segment-state pass over every key segment, scan to the total
// (item p1_segs), then the output pass over query segments.
template <class K>
size_t ws_bytes_nc_t(const ChunkedArgs& a) {
  if (a.L == 0) return 0;
  const int n_seg = segments_of<K>(a);
  return sizeof(float) * (size_t)a.n_heads * (n_seg * kSub + 1) * K::F * K::DVP;
}

template <class K>
hipError_t launch_nc_t(const ChunkedArgs& a, hipStream_t s) {
  Params p{};
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.o = static_cast<uint16_t*>(a.o);
  p.L = a.L;
  p.Lq = a.Lq;
  p.sub = kSub;
  p.m = a.m;
  p.anchors = static_cast<const uint16_t*>(a.anchors);
  p.prf = static_cast<const uint16_t*>(a.prf);
  p.draw_set_stride = a.draw_set_stride;
  p.n_draw_sets = a.n_draw_sets;
  p.nc = a.nc;
  p.ws = static_cast<float*>(a.ws);
  p.S0 = a.S0;
  p.z0 = a.z0;
  hipError_t e;
  ScanArgs sa{};
  sa.n_heads = a.n_heads;
  sa.F = K::F;
  sa.dv = K::DV;
  sa.S0 = a.S0;
  sa.z0 = a.z0;
  sa.S_out = a.S_out;
  sa.z_out = a.z_out;
  if (a.L > 0) {
    const int n_seg = segments_of<K>(a);
    p.n_seg = n_seg;
    p.seg_len = seg_len_for<K>(a.n_heads, a.L);
    p.p1_segs = n_seg * kSub;
    p.p1_items = p.p1_segs + 1;
    if constexpr (K::STAGERS1) {
      e = set_max_lds(reinterpret_cast<const void*>(&pass1s_kernel<K, false>), K::kLds1);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL((pass1s_kernel<K, false>), dim3((unsigned)(a.n_heads * p.p1_segs)), dim3(K::NT + 256), K::kLds1, s,
                         p);
    } else {
      e = set_max_lds(reinterpret_cast<const void*>(&pass1_kernel<K, 1>), K::kLds1);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL((pass1_kernel<K, 1>), dim3((unsigned)(a.n_heads * p.p1_segs)), dim3(K::NT), K::kLds1, s, p);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    sa.states = p.ws;
    sa.n_items = p.p1_items;
    sa.n_terms = p.p1_segs;
    sa.layout = 1;
    sa.total_only = true;  // the output pass reads only the total (the last item)
  } else {  // no keys: the state is S0/z0 (the output pass reads them directly)
    p.p1_items = 1;
    sa.states = nullptr;
    sa.n_items = 0;
    sa.n_terms = 0;
    sa.layout = 0;
  }
  if (sa.n_items > 0 || sa.S_out || sa.z_out) {
    e = launch_scan(sa, s);
    if (e != hipSuccess) return e;
  }
  if (a.Lq == 0) return hipSuccess;
  p.n_qseg = segments_of<K>(a.n_heads, a.Lq);
  p.qseg_len = seg_len_for<K>(a.n_heads, a.Lq);
  using KN = NcCfg<K>;
  constexpr int lds = ncout_lds<KN>();
  static_assert(lds <= 160 * 1024, "LDS budget");
  e = set_max_lds(reinterpret_cast<const void*>(&ncout_kernel<KN>), lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(ncout_kernel<KN>, dim3((unsigned)(a.n_heads * p.n_qseg)), dim3(KN::NT), lds, s, p);
  return hipGetLastError();
}

// Prefix states of every key segment, the input of the fused backward: the
// segment-state pass over segments 0..n_seg-2 and the scan, after which item s
// of ws (fragment order, [n_heads][n_seg][F/16][NE][64][4]) holds S0 plus the
// states of all keys before segment s.
template <class K>
hipError_t segment_prefix_t(const ChunkedArgs& a, float* ws, hipStream_t s) {
  const int n_seg = segments_of<K>(a);
  Params p{};
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.L = a.L;
  p.Lq = a.L;
  p.sub = kSub;
  p.m = a.m;
  p.anchors = static_cast<const uint16_t*>(a.anchors);
  p.prf = static_cast<const uint16_t*>(a.prf);
  p.draw_set_stride = a.draw_set_stride;
  p.n_draw_sets = a.n_draw_sets;
  p.nc = a.nc;
  p.ws = ws;
  p.n_seg = n_seg;
  p.seg_len = seg_len_for<K>(a.n_heads, a.L);
  p.p1_segs = (n_seg - 1) * kSub;
  p.p1_items = p.p1_segs + 1;
  hipError_t e;
  if (n_seg > 1) {
    if constexpr (K::STAGERS1) {
      e = set_max_lds(reinterpret_cast<const void*>(&pass1s_kernel<K, false>), K::kLds1);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL((pass1s_kernel<K, false>), dim3((unsigned)(a.n_heads * p.p1_segs)), dim3(K::NT + 256), K::kLds1, s,
                         p);
    } else {
      e = set_max_lds(reinterpret_cast<const void*>(&pass1_kernel<K, 1>), K::kLds1);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL((pass1_kernel<K, 1>), dim3((unsigned)(a.n_heads * p.p1_segs)), dim3(K::NT), K::kLds1, s, p);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  ScanArgs sa{};
  sa.states = ws;
  sa.n_heads = a.n_heads;
  sa.n_items = p.p1_items;
  sa.n_terms = p.p1_segs;
  sa.F = K::F;
  sa.dv = K::DV;
  sa.layout = 1;
  sa.S0 = a.S0;
  sa.z0 = a.z0;
  return launch_scan(sa, s);
}

}  // namespace

// ---------------------------------------------------------------------------
// Variable-length batches (F = 256 configuration).
namespace {

// Work list (one workgroup of 256 threads).  A sequence of len tokens is cut
// into len / seg_len whole segments and a shorter tail; its last piece (the
// tail, or else its last whole segment) needs no segment state, because no
// later piece of the sequence starts from it: the main pass ends that piece
// with the sequence's final state.  State slots, in order: the whole segments
// that another piece follows (A: the segment-state pass covers them), the
// whole segments that end their sequence (B), the tails (C).  Main-pass work
// items: one per whole segment (item g owns slot g), then packs of
// consecutive tails whose lengths rounded up to 32 tokens sum to at most
// seg_len, walked one after another by one workgroup, so the tails of short
// sequences do not each take a compute unit.  Threads own blocks of at least
// 4 consecutive sequences and pack within their block.  Outputs: per
// sequence its first A slot, its A count and the slot of its last piece (-1
// if it is empty), for the scan; per item the descriptor of Params::vl_item;
// the packs' chunk descriptors; the item counts of both passes.  Offsets
// that do not rise from 0 to T without decreasing give no items.
__global__ __launch_bounds__(256) void vl_setup_kernel(const int64_t* __restrict__ cu, int n_seqs, int64_t T,
                                                       int64_t seg_len, int g_max, int* __restrict__ first,
                                                       int* __restrict__ n_a, int* __restrict__ last,
                                                       int* __restrict__ count, int4* __restrict__ item,
                                                       int4* __restrict__ list32) {
  constexpr int NV = 5;  // per-thread counts: slots A, B, C, packs, pack chunks
  constexpr int kStage = 2048;  // offsets and tails of up to this many sequences are staged in LDS
  __shared__ int part[4][NV];
  __shared__ int bad;
  __shared__ int64_t scu[kStage + 1];
  __shared__ int4 stail[kStage];  // per tail: first descriptor, row, slot, sequence
  const int tid = threadIdx.x;
  const uint32_t sl = (uint32_t)seg_len;  // <= 8192
  const int per = max(4, (n_seqs + 255) / 256);  // sequences per thread: the serial depth of the walk
  const int s0 = min(n_seqs, tid * per), s1 = min(n_seqs, s0 + per);
  // The threads walk their sequences one after another; with the offsets in
  // LDS (read by all threads together in one round trip) each step costs no
  // memory round trip, and the tails' chunk descriptors are written after the
  // walk by all threads together.  Larger batches read the offsets from
  // memory and write the descriptors during the walk.
  const bool staged = n_seqs <= kStage;
  if (staged)
    for (int i = tid; i <= n_seqs; i += 256) scu[i] = cu[i];
  if (tid == 0) bad = 0;
  __syncthreads();
  // the rest of the kernel, with the offsets read from LDS or from memory
  // (one or the other at compile time: a pointer that may be either would
  // make every read a flat access that waits for all stores in flight)
  auto run = [&](auto staged_c) {
    constexpr bool ST = decltype(staged_c)::value;
    auto ofs_at = [&](int i) -> int64_t { return ST ? scu[i] : cu[i]; };
    const bool ends_bad = tid == 0 && (ofs_at(0) != 0 || ofs_at(n_seqs) != T);
    int v[NV] = {0, 0, 0, 0, 0};
    int lbad = ends_bad ? 1 : 0;
    {
      int fill = -1;  // tokens in this thread's open pack (-1: none)
      for (int sq = s0; sq < s1; ++sq) {
        const int64_t len = ofs_at(sq + 1) - ofs_at(sq);
        lbad |= len < 0;
        const uint32_t l = (uint32_t)max<int64_t>(len, 0);  // T < 2^31: 32-bit arithmetic
        const int nf = (int)(l / sl);
        const int r = (int)(l - nf * sl);
        if (r) {
          v[0] += nf;
          const int pl = (r + 31) / 32 * 32;
          if (fill < 0 || fill + pl > (int)sl) {
            ++v[3];
            fill = 0;
          }
          fill += pl;
          ++v[2];
          v[4] += (r + 31) / 32;
        } else if (nf > 0) {
          v[0] += nf - 1;
          ++v[1];
        }
      }
    }
    if (lbad) atomicOr(&bad, 1);
    // exclusive prefix of the per-thread counts: inclusive scan within each wave
    // (shuffles), then the four wave totals
    const int lane = tid & 63, wv = tid >> 6;
    int inc[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) inc[i] = v[i];
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int u = __shfl_up(inc[i], o, 64);
        if (lane >= o) inc[i] += u;
      }
    }
    if (lane == 63)
#pragma unroll
      for (int i = 0; i < NV; ++i) part[wv][i] = inc[i];
    __syncthreads();
    int base[NV], tot[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      base[i] = inc[i] - v[i];
      tot[i] = 0;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        if (w < wv) base[i] += part[w][i];
        tot[i] += part[w][i];
      }
    }
    const int ra = tot[0], rb = tot[1], rc = tot[2], rp = tot[3];
    if (tid == 0 && ra + rb + rc > g_max) atomicOr(&bad, 1);
    __syncthreads();  // every wave has read the wave totals; bad is final
    const bool ok = bad == 0;
    if (tid == 0) {
      count[0] = ok ? ra + rb + rp : 0;
      count[1] = ok ? ra : 0;
    }
    if (!ok) {  // no pieces: the scan passes every sequence's initial state through
      for (int sq = s0; sq < s1; ++sq) {
        first[sq] = 0;
        n_a[sq] = 0;
        last[sq] = -1;
      }
      return;
    }
    const int S32 = (int)(sl / 32), S64 = (int)(sl / 64);
    int slot_a = base[0], slot_b = ra + base[1], slot_c = ra + rb + base[2], pk = ra + rb + base[3];
    int pos = base[4];
    int open = -1, open0 = 0;  // this thread's open pack: item, first descriptor
    int fill = 0;
    auto close = [&]() {
      if (open >= 0) item[open] = make_int4(pos - open0, 0, open0, open0);
    };
    for (int sq = s0; sq < s1; ++sq) {
      const int c0 = (int)ofs_at(sq);
      const uint32_t len = (uint32_t)(ofs_at(sq + 1) - c0);
      const int nf = (int)(len / sl);
      const int r = (int)(len - nf * sl);
      const int na = r ? nf : max(nf - 1, 0);
      first[sq] = slot_a;
      n_a[sq] = na;
      for (int j = 0; j < na; ++j) item[slot_a + j] = make_int4(S32, S64, c0 + j * (int)sl, -1 - sq);
      slot_a += na;
      if (r) {
        last[sq] = slot_c;
        const int pl = (r + 31) / 32 * 32;
        if (open < 0 || fill + pl > (int)sl) {
          close();
          open = pk++;
          open0 = pos;
          fill = 0;
        }
        fill += pl;
        const int row = c0 + nf * (int)sl;
        const int n32 = (r + 31) / 32;
        if constexpr (ST) {
          stail[slot_c - ra - rb] = make_int4(pos, row, slot_c, sq);
        } else {
          for (int i = 0; i < n32; ++i)
            list32[pos + i] = make_int4(row + 32 * i, min(32, r - 32 * i), slot_c,
                                        (i == 0 ? kFirst : 0) | (i == n32 - 1 ? kLast | kSeqEnd : 0) | (sq << 3));
        }
        pos += n32;
        ++slot_c;
      } else if (nf > 0) {
        last[sq] = slot_b;
        item[slot_b] = make_int4(S32, S64, c0 + na * (int)sl, -1 - sq);
        ++slot_b;
      } else {
        last[sq] = -1;
      }
    }
    close();
    if constexpr (!ST) return;
    __syncthreads();  // every tail recorded
    // one wave per tail, one lane per chunk
    for (int t = tid >> 6; t < rc; t += 4) {
      const int4 ti = stail[t];
      const int r = (int)((uint32_t)(scu[ti.w + 1] - scu[ti.w]) % sl);
      const int n32 = (r + 31) / 32;
      for (int i = lane; i < n32; i += 64)
        list32[ti.x + i] = make_int4(ti.y + 32 * i, min(32, r - 32 * i), ti.z,
                                     (i == 0 ? kFirst : 0) | (i == n32 - 1 ? kLast | kSeqEnd : 0) | (ti.w << 3));
    }
  };
  if (staged)
    run(std::true_type());
  else
    run(std::false_type());
}

// Tokens per work item: about 256 work items over the chip, a multiple of two
// chunks, at most 8192 (so a pack's chunk descriptors take at most 4 KiB of LDS).
int64_t vl_seg_len(int64_t H, int64_t T) {
  const int64_t want = (H * T + 255) / 256;
  const int64_t sl = ((want + 127) / 128) * 128;
  return sl < 128 ? 128 : (sl > 8192 ? 8192 : sl);
}

// Work items per head: every sequence adds at most one partial segment.
int vl_g_max(int64_t T, int n_seqs, int64_t seg_len) { return (int)(T / seg_len + n_seqs); }

struct VlWs {
  int *first, *n_a, *last, *count;
  int4 *item, *list32;
  float* states;
  size_t bytes;
};

VlWs vl_ws(const VarlenArgs& a, int g_max, void* base) {
  VlWs w{};
  char* p = static_cast<char*>(base);
  size_t off = 0;
  auto take = [&](size_t b) {
    char* q = p ? p + off : nullptr;
    off += (b + 255) & ~(size_t)255;
    return q;
  };
  w.states = reinterpret_cast<float*>(take(sizeof(float) * (size_t)a.c.n_heads * g_max * CfgF256::F * CfgF256::DVP));
  w.item = reinterpret_cast<int4*>(take(sizeof(int4) * (size_t)g_max));
  // pack descriptors: every tail r takes ceil(r / 32) <= r / 32 + 1 of them
  w.list32 = reinterpret_cast<int4*>(take(sizeof(int4) * (size_t)(a.c.L / 32 + a.n_seqs)));
  w.first = reinterpret_cast<int*>(take(sizeof(int) * (size_t)a.n_seqs));
  w.n_a = reinterpret_cast<int*>(take(sizeof(int) * (size_t)a.n_seqs));
  w.last = reinterpret_cast<int*>(take(sizeof(int) * (size_t)a.n_seqs));
  w.count = reinterpret_cast<int*>(take(2 * sizeof(int)));
  w.bytes = off;
  return w;
}

}  // namespace

// Feature counts the fused kernels are not built for run a built count's
// kernels on zero-padded features: the draws get zero rows f >= F (phi_f = 0,
// and the node constants beyond R are zero, so the exponent stays finite),
// the initial states zero rows, and the first F rows of the final states are
// copied out.  No result changes; the padded work is the cost.
namespace {

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// F itself when kernels are built for it, else the smallest built count it
// can be padded to; 0 when there is none.
int fused_target_F(const ChunkedArgs& a) {
  if (!a.io_bf16 || a.d != 64 || a.dv != 64 || a.chunk != 64 || a.m % 16 != 0) return 0;
  for (const int Fb : {CfgF64::F, CfgF96::F, CfgF128::F, CfgF256::F}) {
    if (Fb < a.F) continue;
    if (Fb == CfgF256::F && a.m % 32 != 0) continue;  // a wave's two feature blocks must share a node
    if ((Fb - 1) / a.m >= kMaxNodes) continue;        // node of every padded feature in the table
    return Fb;
  }
  return 0;
}

// Padded copies: draws [n_sets][Fp][d], states [n_state][Fp][dv] and [n_state][Fp].
struct FPad {
  uint16_t *anchors, *prf;
  float *S0, *z0, *S_out, *z_out;
  size_t bytes;
};

FPad fpad_ws(const ChunkedArgs& a, int Fp, int64_t n_state, char* base) {
  FPad w{};
  size_t off = 0;
  auto take = [&](size_t b) {
    char* q = base ? base + off : nullptr;
    off += align256(b);
    return q;
  };
  const size_t nd = (size_t)a.n_draw_sets * Fp * a.d * 2;
  const size_t ns = (size_t)n_state * Fp * a.dv * 4, nz = (size_t)n_state * Fp * 4;
  w.anchors = reinterpret_cast<uint16_t*>(take(nd));
  w.prf = reinterpret_cast<uint16_t*>(take(nd));
  w.S0 = reinterpret_cast<float*>(take(ns));
  w.z0 = reinterpret_cast<float*>(take(nz));
  w.S_out = reinterpret_cast<float*>(take(ns));
  w.z_out = reinterpret_cast<float*>(take(nz));
  w.bytes = off;
  return w;
}

// Fill the padded inputs and point ap (a copy of a with F = Fp) at them.  The
// inputs are copied before anything is written: S_out may alias S0.
hipError_t pad_inputs(const ChunkedArgs& a, int Fp, int64_t n_state, const FPad& w, ChunkedArgs& ap, hipStream_t s) {
  const int64_t F = a.F, d = a.d, dv = a.dv;
  hipError_t e = pad_rows(w.anchors, static_cast<const uint16_t*>(a.anchors), a.n_draw_sets, F, Fp, d,
                          a.draw_set_stride, (int64_t)Fp * d, s);
  if (e == hipSuccess)
    e = pad_rows(w.prf, static_cast<const uint16_t*>(a.prf), a.n_draw_sets, F, Fp, d, a.draw_set_stride,
                 (int64_t)Fp * d, s);
  if (e == hipSuccess && a.S0) e = pad_rows(w.S0, a.S0, n_state, F, Fp, dv, F * dv, (int64_t)Fp * dv, s);
  if (e == hipSuccess && a.z0) e = pad_rows(w.z0, a.z0, n_state, F, Fp, 1, F, Fp, s);
  if (e != hipSuccess) return e;
  ap = a;
  ap.F = Fp;
  ap.anchors = w.anchors;
  ap.prf = w.prf;
  ap.draw_set_stride = (int64_t)Fp * d;
  ap.S0 = a.S0 ? w.S0 : nullptr;
  ap.z0 = a.z0 ? w.z0 : nullptr;
  ap.S_out = a.S_out ? w.S_out : nullptr;
  ap.z_out = a.z_out ? w.z_out : nullptr;
  return hipSuccess;
}

hipError_t pad_outputs(const ChunkedArgs& a, int Fp, int64_t n_state, const FPad& w, hipStream_t s) {
  const int64_t F = a.F, dv = a.dv;
  hipError_t e = hipSuccess;
  if (a.S_out) e = pad_rows(a.S_out, w.S_out, n_state, F, F, dv, (int64_t)Fp * dv, F * dv, s);
  if (e == hipSuccess && a.z_out) e = pad_rows(a.z_out, w.z_out, n_state, F, F, 1, Fp, F, s);
  return e;
}

size_t varlen_bytes_exact(const VarlenArgs& a) {
  return vl_ws(a, vl_g_max(a.c.L, a.n_seqs, vl_seg_len(a.c.n_heads, a.c.L)), nullptr).bytes;
}

hipError_t launch_varlen_exact(const VarlenArgs& a, hipStream_t s);

}  // namespace

bool varlen_supported(const VarlenArgs& a) {
  // F <= 256 (below 256 on zero-padded features); m % 32 == 0 keeps a wave's two feature blocks on one node
  return a.c.io_bf16 && a.c.d == 64 && a.c.dv == 64 && a.c.F <= CfgF256::F && a.c.m % 32 == 0;
}

size_t varlen_workspace_bytes(const VarlenArgs& a) {
  if (a.c.n_heads == 0 || a.n_seqs == 0) return 0;
  if (a.c.F == CfgF256::F) return varlen_bytes_exact(a);
  VarlenArgs ap = a;
  ap.c.F = CfgF256::F;
  return align256(varlen_bytes_exact(ap)) + fpad_ws(a.c, CfgF256::F, (int64_t)a.n_seqs * a.c.n_heads, nullptr).bytes;
}

hipError_t launch_varlen(const VarlenArgs& a, hipStream_t s) {
  if (a.c.F == CfgF256::F || a.c.n_heads == 0 || a.n_seqs == 0) return launch_varlen_exact(a, s);
  VarlenArgs ap = a;
  ap.c.F = CfgF256::F;
  const int64_t n_state = (int64_t)a.n_seqs * a.c.n_heads;
  const FPad w = fpad_ws(a.c, CfgF256::F, n_state, static_cast<char*>(a.c.ws) + align256(varlen_bytes_exact(ap)));
  hipError_t e = pad_inputs(a.c, CfgF256::F, n_state, w, ap.c, s);
  if (e != hipSuccess) return e;
  e = launch_varlen_exact(ap, s);
  if (e != hipSuccess) return e;
  return pad_outputs(a.c, CfgF256::F, n_state, w, s);
}

namespace {

hipError_t launch_varlen_exact(const VarlenArgs& a, hipStream_t s) {
  using K = CfgF256;
  using KS = typename MainPass<K>::type;
  const int64_t H = a.c.n_heads, T = a.c.L;
  if (H == 0 || a.n_seqs == 0) return hipSuccess;
  const int64_t seg_len = vl_seg_len(H, T);
  const int g_max = vl_g_max(T, a.n_seqs, seg_len);
  const VlWs w = vl_ws(a, g_max, a.c.ws);
  hipLaunchKernelGGL(vl_setup_kernel, dim3(1), dim3(256), 0, s, a.cu, a.n_seqs, T, seg_len, g_max, w.first,
                     w.n_a, w.last, w.count, w.item, w.list32);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  Params p{};
  p.q = static_cast<const uint16_t*>(a.c.q);
  p.k = static_cast<const uint16_t*>(a.c.k);
  p.v = static_cast<const uint16_t*>(a.c.v);
  p.o = static_cast<uint16_t*>(a.c.o);
  p.L = T;
  p.Lq = T;
  p.seg_len = seg_len;
  p.n_seg = g_max;
  p.sub = kSub;
  p.p1_segs = g_max;
  p.p1_items = g_max;
  p.m = a.c.m;
  p.anchors = static_cast<const uint16_t*>(a.c.anchors);
  p.prf = static_cast<const uint16_t*>(a.c.prf);
  p.draw_set_stride = a.c.draw_set_stride;
  p.n_draw_sets = a.c.n_draw_sets;
  p.nc = a.c.nc;
  p.ws = w.states;
  p.vl_count = w.count;
  p.vl_item = w.item;
  p.vl_list32 = w.list32;
  p.vl_cap = (int)(seg_len / 32);
  p.cu = a.cu;
  p.T = T;
  p.g_max = g_max;
  p.n_heads = H;
  const unsigned grid = (unsigned)(H * g_max);
  p.S_out = a.c.S_out;  // the main pass writes the final state of every non-empty sequence
  p.z_out = a.c.z_out;
  const int lds_list = (int)sizeof(int4) * p.vl_cap;  // a pack's chunk descriptors (main pass)
  if (T > 0) {  // the states of the whole segments another piece follows
    e = set_max_lds(reinterpret_cast<const void*>(&pass1s_kernel<K, true>), K::kLds1);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((pass1s_kernel<K, true>), dim3(grid), dim3(K::NT + 256), K::kLds1, s, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  e = launch_scan_varlen(w.states, H, a.n_seqs, g_max, w.first, w.n_a, w.last, K::F, K::DV, a.c.S0, a.c.z0,
                         a.c.S_out, a.c.z_out, s);
  if (e != hipSuccess || T == 0) return e;
  e = set_max_lds(reinterpret_cast<const void*>(&pass2s_kernel<KS, true>), KS::kLdsS + lds_list);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((pass2s_kernel<KS, true>), dim3(grid), dim3(KS::NTW), KS::kLdsS + lds_list, s, p);
  return hipGetLastError();
}

}  // namespace

int fused_segment_count(const ChunkedArgs& a, int64_t* seg_len) {
  int n = 0;
  dispatch(a, [&](auto k) {
    using K = decltype(k);
    n = segments_of<K>(a);
    *seg_len = seg_len_for<K>(a.n_heads, a.L);
  });
  return n;
}

hipError_t launch_segment_prefix(const ChunkedArgs& a, float* ws, hipStream_t s) {
  hipError_t e = hipErrorInvalidValue;
  dispatch(a, [&](auto k) { e = segment_prefix_t<decltype(k)>(a, ws, s); });
  return e;
}

bool fused_supported(const ChunkedArgs& a) { return fused_target_F(a) != 0; }

namespace {

size_t fused_bytes_exact(const ChunkedArgs& a) {
  size_t r = 0;
  dispatch(a, [&](auto k) { r = a.causal ? ws_bytes_t<decltype(k)>(a) : ws_bytes_nc_t<decltype(k)>(a); });
  return r;
}

}  // namespace

size_t fused_workspace_bytes(const ChunkedArgs& a) {
  const int Fp = fused_target_F(a);
  if (Fp == 0) return 0;
  if (Fp == a.F) return fused_bytes_exact(a);
  ChunkedArgs ap = a;
  ap.F = Fp;
  return align256(fused_bytes_exact(ap)) + fpad_ws(a, Fp, a.n_heads, nullptr).bytes;
}

hipError_t launch_fused(const ChunkedArgs& a, hipStream_t s) {
  if (a.n_heads == 0) return hipSuccess;
  const int Fp = fused_target_F(a);
  if (Fp != a.F) {  // zero-padded features
    if (a.causal && a.L == 0) return launch_generic(a, s);  // only the state passes through
    ChunkedArgs ap = a;
    ap.F = Fp;
    const FPad w = fpad_ws(a, Fp, a.n_heads, static_cast<char*>(a.ws) + align256(fused_bytes_exact(ap)));
    hipError_t e = pad_inputs(a, Fp, a.n_heads, w, ap, s);
    if (e != hipSuccess) return e;
    e = launch_fused(ap, s);
    if (e != hipSuccess) return e;
    return pad_outputs(a, Fp, a.n_heads, w, s);
  }
  hipError_t e = hipErrorInvalidValue;
  if (!a.causal) {
    dispatch(a, [&](auto k) { e = launch_nc_t<decltype(k)>(a, s); });
    return e;
  }
  if (a.L == 0) return launch_generic(a, s);  // only the state passes through
  dispatch(a, [&](auto k) { e = launch_t<decltype(k)>(a, s); });
  return e;
}

}  // namespace slay
