// slay_featmap.hip -- the SLAY feature map phi(x) on MFMA (gfx950).
//
// Method ("SLAY: Geometry-Aware Spherical Linearized Attention with
// Yat-Kernel", abstract; nubint.ai review, "Proposed method" bullets 1, 3, 5):
// rows are projected onto the unit sphere, node r of the Gauss-Laguerre
// mixture contributes m features, each the product of an anchor feature
// (a.xh)^2 and a positive random feature exp(sqrt(beta_r) g.xh - beta_r/2),
// scaled by sqrt(alpha_r/m):  phi[r*m+t] = sqrt(alpha_r/m) (a_rt.xh)^2 prf_rt(xh).
//
// Kernel shape: a 256-thread workgroup owns a slice of 64*FBW features for
// the whole launch and keeps that slice of the projection matrix
// P = [anchors | prf] in registers as MFMA A-operands.  It walks row tiles
// of x (64 rows; 16 or 32 for small launches such as a decode step's one
// row per head): stages the tile in LDS (padded rows, so the per-lane
// 16-byte reads are bank-conflict free), computes 1/|x| per row, then per
// 16-token block runs Y^T = P_slice x^T on 16x16 MFMA tiles and applies the
// square / exp2 / scale epilogue straight from the accumulators.  The 1/|x|
// scale is applied to the fp32 accumulator, (x/|x|).P = (x.P)/|x|, so bf16
// inputs are never rounded twice.  The tile's features are written back from
// an LDS staging copy with coalesced 16-byte non-temporal buffer stores that
// stay in flight while the next tile is computed.
#include "slay_device.hpp"
#include "slay_internal.hpp"

namespace slay {

namespace {

constexpr int kTileRows = 64;  // rows per tile of large launches
constexpr int kThreads = 256;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <typename TI>
struct XStage {
  static constexpr int kPad = 16 / sizeof(TI);  // one 16-byte slot per row
};

template <typename TO>
__device__ __forceinline__ void store4(TO* p, float a, float b, float c, float d);

template <>
__device__ __forceinline__ void store4<float>(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}

template <>
__device__ __forceinline__ void store4<uint16_t>(uint16_t* p, float a, float b, float c, float d) {
  uint2 v;
  v.x = pack_bf16x2(a, b);
  v.y = pack_bf16x2(c, d);
  *reinterpret_cast<uint2*>(p) = v;
}

// Every variant asks for at least 2 waves per SIMD: with 1 the compiler may
// keep the MFMA results in accumulator registers and copy each one out with
// a VALU instruction.  The d = 128 bf16 variant is held to 3: it otherwise
// takes 164 registers and runs 2 waves per SIMD, with its memory latency
// exposed.
template <typename TI, typename TO, int D, int FBW, int TR>
__global__ __launch_bounds__(kThreads, (sizeof(TI) == 2 && D == 128) ? 3 : 2) void featmap_kernel(
    const TI* __restrict__ x_a, const TI* __restrict__ x_b, int64_t rows_per_head, int64_t n_heads,
    const TI* __restrict__ anchors, const TI* __restrict__ prf, int64_t draw_set_stride, int n_draw_sets, int F,
    int m, NodeConsts nc, TO* __restrict__ phi_a, TO* __restrict__ phi_b, int gx) {
  // blockIdx.z selects the input: z = 1 maps the second input in the same launch
  const TI* __restrict__ x = blockIdx.z ? x_b : x_a;
  TO* __restrict__ phi = blockIdx.z ? phi_b : phi_a;
  using M = Mma<TI>;
  constexpr int KS = D / M::K;               // MFMA k-steps over d
  constexpr int LDX = D + XStage<TI>::kPad;  // padded LDS row stride (elements)
  constexpr int VEC = 16 / sizeof(TI);       // elements per 16-byte vector
  constexpr int VPR = D / VEC;               // 16-byte vectors per row
  static_assert(D % M::K == 0, "d must be a multiple of the MFMA k-step");
  static_assert((TR * VPR) % kThreads == 0 && TR % 16 == 0, "tile staging must divide evenly");

  constexpr int FWS = 4 * FBW * 16;              // features per workgroup slice
  constexpr int LDO = FWS + 16 / sizeof(TO);      // padded output staging stride
  __shared__ __align__(16) TI sx[TR * LDX];
  __shared__ __align__(16) TO so[TR * LDO];
  __shared__ float sinv[TR], slg[TR];

  const int lane = threadIdx.x & 63;
  // wave-uniform, so the node constants below are scalar loads and no vector
  // load of them is left for the tile loop to wait on
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;
  const int col = lane & 15;
  const int n_fblk = F / 16;
  // Workgroup id -> (row-tile walker bx, feature slice by): the gy slices of
  // the same walker get ids that are equal modulo 8, so they run on one XCD
  // and start together, and the later slices read each x tile from that
  // XCD's L2 rather than from HBM.
  const int gy = (F + FWS - 1) / FWS;
  const int grp = (int)blockIdx.x / (8 * gy), rem = (int)blockIdx.x - grp * 8 * gy;
  const int by = rem >> 3, bx = grp * 8 + (rem & 7);
  if (bx >= gx) return;
  const int fblk0 = by * (4 * FBW) + wave * FBW;

  const int tiles_per_head = (int)((rows_per_head + TR - 1) / TR);
  const int n_tiles = tiles_per_head * (int)n_heads;

  typename M::frag pa[FBW][KS], pg[FBW][KS];
  int cur_set = -1;

  // x tile vectors of the next tile are loaded into registers while the
  // current tile is computed (one tile of prefetch)
  constexpr int PER_T = TR * VPR / kThreads;
  constexpr int TPR = kThreads / TR;  // threads per row; a thread's vectors lie in one row
  uint4 xr[PER_T];
  auto load_tile = [&](int tt) {
    const int hh = tt / tiles_per_head;
    const int64_t r0 = (int64_t)(tt - hh * tiles_per_head) * TR;
    const int64_t nr = min<int64_t>(TR, rows_per_head - r0);
    const TI* src = x + ((int64_t)hh * rows_per_head + r0) * D;
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int v = threadIdx.x * PER_T + i;
      const int r = v / VPR;
      const int c = (v - r * VPR) * VEC;
      // unconditional load of a row inside the tile (rows past its end repeat
      // its last row; their features are never stored): a conditional load
      // lets the compiler move work on the loaded value next to the load,
      // which then waits on it at once
      const int64_t rc = r < nr ? r : nr - 1;
      xr[i] = *reinterpret_cast<const uint4*>(src + rc * D + c);
    }
  };
  if (bx < n_tiles) load_tile(bx);
  // the tile loop below then starts with no load in flight, so its staging
  // needs no wait on the counter that the stores also use
  wait_vmem();

  for (int t = bx; t < n_tiles; t += gx) {
    const int h = t / tiles_per_head;
    const int64_t row0 = (int64_t)(t - h * tiles_per_head) * TR;  // row within head
    const int64_t nrow = min<int64_t>(TR, rows_per_head - row0);
    TO* pt = phi + ((int64_t)h * rows_per_head + row0) * (int64_t)F;

    // (re)load this wave's slice of P when the draw set changes
    const int set = (int)(h % n_draw_sets);
    if (set != cur_set) {
      cur_set = set;
      const TI* a = anchors + (int64_t)set * draw_set_stride;
      const TI* gg = prf + (int64_t)set * draw_set_stride;
#pragma unroll
      for (int j = 0; j < FBW; ++j) {
        const int fb = min(fblk0 + j, n_fblk - 1);
        const int64_t rowoff = (int64_t)(fb * 16 + col) * D;
        if constexpr (sizeof(TI) == 4) {
          // fp32: lane group g owns d in [g D/4, (g+1) D/4), k-step ks its
          // ks-th element (the x operand below uses the same order, so the
          // sum over d is unchanged); one lane's operands are contiguous
#pragma unroll
          for (int q = 0; q < KS / 4; ++q) {
            const float4 va = *reinterpret_cast<const float4*>(a + rowoff + g * KS + 4 * q);
            const float4 vg = *reinterpret_cast<const float4*>(gg + rowoff + g * KS + 4 * q);
            pa[j][4 * q] = va.x, pa[j][4 * q + 1] = va.y, pa[j][4 * q + 2] = va.z, pa[j][4 * q + 3] = va.w;
            pg[j][4 * q] = vg.x, pg[j][4 * q + 1] = vg.y, pg[j][4 * q + 2] = vg.z, pg[j][4 * q + 3] = vg.w;
          }
        } else {
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            pa[j][ks] = M::load(a + rowoff + ks * M::K + M::KL * g);
            pg[j][ks] = M::load(gg + rowoff + ks * M::K + M::KL * g);
          }
        }
      }
      // wait here, where the reload is rare, so that the first MFMA of the
      // tile does not wait for every load in flight (the next tile's prefetch
      // included) to learn that P has arrived
      wait_vmem();
    }

    // stage the x tile in LDS and compute 1/max(|x|, 1e-12) per row
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int v = threadIdx.x * PER_T + i;
      const int r = v / VPR;
      const int c = (v - r * VPR) * VEC;
      *reinterpret_cast<uint4*>(&sx[r * LDX + c]) = xr[i];
      const TI* e = reinterpret_cast<const TI*>(&xr[i]);
#pragma unroll
      for (int q = 0; q < VEC; ++q) {
        const float f = M::to_f32(e[q]);
        ss += f * f;
      }
    }
    ss = sum_lanes<TPR>(ss);
    if ((threadIdx.x % TPR) == 0) {
      const float inv = 1.0f / fmaxf(sqrtf(ss), 1e-12f);
      sinv[threadIdx.x / TPR] = inv;
      slg[threadIdx.x / TPR] = 2.0f * __builtin_amdgcn_logf(inv);  // log2(inv^2)
    }
    __syncthreads();
    if (t + gx < n_tiles) load_tile(t + gx);

#pragma unroll
    for (int tb = 0; tb < TR / 16; ++tb) {
      f32x4 ya[FBW], yg[FBW];
#pragma unroll
      for (int j = 0; j < FBW; ++j) {
        ya[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        yg[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      typename M::frag b[KS];
      if constexpr (sizeof(TI) == 4) {  // the permuted fp32 order of the P operands
#pragma unroll
        for (int q = 0; q < KS / 4; ++q) {
          const float4 v = *reinterpret_cast<const float4*>(&sx[(tb * 16 + col) * LDX + g * KS + 4 * q]);
          b[4 * q] = v.x, b[4 * q + 1] = v.y, b[4 * q + 2] = v.z, b[4 * q + 3] = v.w;
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) b[ks] = M::load(&sx[(tb * 16 + col) * LDX + ks * M::K + M::KL * g]);
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int j = 0; j < FBW; ++j) {
          ya[j] = M::mma(pa[j][ks], b[ks], ya[j]);
          yg[j] = M::mma(pg[j][ks], b[ks], yg[j]);
        }
      }
      const int r = tb * 16 + col;  // token of this lane's C column
      const float inv = sinv[r], lg = slg[r];
#pragma unroll
      for (int j = 0; j < FBW; ++j) {
        const int fbl = wave * FBW + j;  // feature block within the workgroup slice
        const int node = (min(fblk0 + j, n_fblk - 1) * 16) / m;
        // (y_a inv)^2 exp2(y_g inv c1 + c0) = y_a^2 exp2(y_g (inv c1) + (c0 + log2 inv^2))
        const float s1 = inv * nc.c1[node];
        const float c0 = nc.c0[node] + lg;
        float o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = ya[j][i] * ya[j][i] * fast_exp2(fmaf(yg[j][i], s1, c0));
        store4<TO>(so + r * LDO + fbl * 16 + 4 * g, o[0], o[1], o[2], o[3]);
      }
    }
    __syncthreads();
    // coalesced write-out of the tile's feature slice: 16-byte pieces of each
    // row as buffer stores bounded by the tile's rows (pieces past its last row
    // or past F are dropped by the bounds check), so every thread issues the
    // same number of stores and the next tile's staging waits only for the
    // prefetched rows, not for these stores
    {
      constexpr int PPR = FWS * (int)sizeof(TO) / 16;  // 16-byte pieces per row of the slice
      constexpr int NPC = (TR * PPR + kThreads - 1) / kThreads;  // pieces per thread
      const int fcols = min(FWS, F - by * FWS);
      const int ppr = fcols * (int)sizeof(TO) / 16;
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          pt, (short)0, (int)(nrow * F * (int64_t)sizeof(TO)), 0x00020000);
      u32x4 val[NPC];
#pragma unroll
      for (int i = 0; i < NPC; ++i) {
        const int pc = min(threadIdx.x + i * kThreads, TR * PPR - 1);
        const int rr = pc / PPR, q = pc - rr * PPR;
        val[i] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(so + rr * LDO) + q * 16);
      }
#pragma unroll
      for (int i = 0; i < NPC; ++i) {
        const int pc = threadIdx.x + i * kThreads;
        const int rr = pc / PPR, q = pc - rr * PPR;
        const bool ok = pc < TR * PPR && q < ppr;
        const int off = ok ? rr * F * (int)sizeof(TO) + by * FWS * (int)sizeof(TO) + q * 16 : 0x7FFFFFF0;
        // non-temporal (cache policy 2): phi is written once and not read
        // back here; even a decode step, whose next kernel reads phi at once,
        // measured slower with cached stores
        __builtin_amdgcn_raw_buffer_store_b128(val[i], rs, off, 0, 2);
      }
    }
    // No barrier here: the next tile's staging writes sx, sinv and slg, whose
    // last readers (this tile's projection) all finished before the barrier
    // above, and its epilogue writes so only after the next staging barrier,
    // which every thread reaches after reading its pieces of so.
  }
}

template <typename TI, typename TO, int D, int FBW, int TR>
hipError_t launch_t(const FeatmapArgs& a, hipStream_t s) {
  const int FW = 4 * FBW * 16;
  const int gy = (a.F + FW - 1) / FW;
  const int64_t tiles = ((a.rows_per_head + TR - 1) / TR) * a.n_heads;
  // 1024 workgroups in all, one per (walker, slice): four per CU at the
  // headline shape's occupancy, so every walker starts at once
  int64_t gx = 1024 / gy;
  if (gx < 1) gx = 1;
  if (gx > tiles) gx = tiles;
  if (tiles == 0) return hipSuccess;
  const int gz = a.x2 ? 2 : 1;
  const unsigned n_groups = (unsigned)((gx + 7) / 8);  // walkers in groups of 8, one id per (walker, slice)
  hipLaunchKernelGGL((featmap_kernel<TI, TO, D, FBW, TR>), dim3(n_groups * 8 * gy, 1, gz), dim3(kThreads), 0, s,
                     static_cast<const TI*>(a.x), static_cast<const TI*>(a.x2), a.rows_per_head, a.n_heads,
                     static_cast<const TI*>(a.anchors), static_cast<const TI*>(a.prf), a.draw_set_stride,
                     a.n_draw_sets, a.F, a.m, a.nc, static_cast<TO*>(a.phi), static_cast<TO*>(a.phi2), (int)gx);
  return hipGetLastError();
}

// Row tile of small launches: the smallest of (kSmallRows, 32, 64) whose
// staging divides evenly over the workgroup.
constexpr int kSmallRows = 64;
template <typename TI, int D>
constexpr int small_tile_rows() {
  constexpr int vpr = D / (16 / (int)sizeof(TI));
  return (kSmallRows <= 16 && (16 * vpr) % kThreads == 0)   ? 16
         : (kSmallRows <= 32 && (32 * vpr) % kThreads == 0) ? 32
                                                            : 64;
}

template <typename TI, typename TO>
hipError_t launch_d(const FeatmapArgs& a, hipStream_t s) {
  constexpr bool bf = sizeof(TI) == 2;
  // Few rows (e.g. one decode token per head): one feature block per wave and
  // short row tiles give many small workgroups, so the dependent MFMA chains
  // of different tiles run side by side.
  const int64_t rows = a.rows_per_head * a.n_heads * (a.x2 ? 2 : 1);
  const bool small = ((rows + kTileRows - 1) / kTileRows) * ((a.F + 127) / 128) < 1024;
  switch (a.d) {
    case 32:
      return small ? launch_t<TI, TO, 32, 1, small_tile_rows<TI, 32>()>(a, s) : launch_t<TI, TO, 32, 4, kTileRows>(a, s);
    case 64:
      return small ? launch_t<TI, TO, 64, 1, small_tile_rows<TI, 64>()>(a, s) : launch_t<TI, TO, 64, 2, kTileRows>(a, s);
    case 128:
      return small ? launch_t<TI, TO, 128, 1, small_tile_rows<TI, 128>()>(a, s)
                   : launch_t<TI, TO, 128, bf ? 2 : 1, kTileRows>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool featmap_supported(int d) { return d == 32 || d == 64 || d == 128; }

hipError_t launch_featmap(const FeatmapArgs& a, hipStream_t s) {
  if (a.x_bf16) {
    return a.phi_bf16 ? launch_d<uint16_t, uint16_t>(a, s) : launch_d<uint16_t, float>(a, s);
  }
  return a.phi_bf16 ? launch_d<float, uint16_t>(a, s) : launch_d<float, float>(a, s);
}

}  // namespace slay
