// slay_device.hpp -- device-side building blocks shared by the SLAY kernels
// (gfx950 / CDNA4, wave64).
//
// MFMA operand layouts used throughout (checked on gfx950 with a one-wave
// in-bounds probe), lane l, g = l / 16:
//   v_mfma_f32_16x16x32_bf16  A[l%16][8g+i], B[8g+i][l%16] (i < 8);  C[4g+i][l%16] (i < 4)
//   v_mfma_f32_16x16x4_f32    A[l%16][g],    B[g][l%16];             C[4g+i][l%16]
// So a 16x16 C tile gives each lane four consecutive rows of one column.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace slay {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kMaxNodes = 16;

// Per-node constants of the feature map, in fp32, computed on the host from
// the fp64 Gauss-Laguerre rule:
//   phi = (y_a * inv)^2 * exp2(y_g * inv * c1[r] + c0[r])
//   c1 = sqrt(beta_r) * log2(e),  c0 = (-beta_r / 2) * log2(e) + log2(sqrt(alpha_r / m))
// with y_a = a.x, y_g = g.x and inv = 1 / max(|x|, 1e-12).
struct NodeConsts {
  float c1[kMaxNodes];
  float c0[kMaxNodes];
};

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}

// fp32 -> bf16 with round to nearest even: gfx950's v_cvt_pk_bf16_f32
// converts two values per instruction.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return (uint16_t)(pack_bf16x2(f, 0.f) & 0xFFFFu); }

// Exchange a 32-bit value with the neighbouring lane (l ^ 1) through DPP.
__device__ __forceinline__ uint32_t swap_lane_pair(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);  // quad_perm [1,0,3,2]
}

// Byte permute (v_perm_b32): low 16 bits of lo | low 16 bits of hi << 16, and the high halves.
__device__ __forceinline__ uint32_t lo16_pair(uint32_t lo, uint32_t hi) { return __builtin_amdgcn_perm(hi, lo, 0x05040100u); }
__device__ __forceinline__ uint32_t hi16_pair(uint32_t lo, uint32_t hi) { return __builtin_amdgcn_perm(hi, lo, 0x07060302u); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// s_waitcnt vmcnt(0) with the other counters left alone (gfx9 encoding: vmcnt
// in bits 3:0 and 15:14, expcnt in 6:4, lgkmcnt in 11:8).  Vector loads and
// stores retire in issue order and share this counter.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Sums over groups of 4, 8 or 16 consecutive lanes by DPP moves, with no LDS
// round trip: quad_perm [1,0,3,2] and [2,3,0,1] pair lanes inside each quad,
// row_half_mirror lane i with 7-i and row_mirror lane i with 15-i of each
// 16-lane row.  Each step adds two partial sums that the paired lanes hold in
// swapped order, so every lane of a group ends with the same bits.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float sum_lanes4(float x) {
  x += dpp_mov<0xB1>(x);
  return x + dpp_mov<0x4E>(x);
}
__device__ __forceinline__ float sum_lanes8(float x) { x = sum_lanes4(x); return x + dpp_mov<0x141>(x); }
__device__ __forceinline__ float sum_lanes16(float x) { x = sum_lanes8(x); return x + dpp_mov<0x140>(x); }
template <int N>
__device__ __forceinline__ float sum_lanes(float x) {
  static_assert(N == 1 || N == 4 || N == 8 || N == 16, "DPP sums cover groups of 4, 8 or 16 lanes");
  if constexpr (N == 4) return sum_lanes4(x);
  if constexpr (N == 8) return sum_lanes8(x);
  if constexpr (N == 16) return sum_lanes16(x);
  return x;
}

__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& v) {
  return __builtin_bit_cast(bf16x8, v);
}

// Element type traits for the 16x16 MFMA step: K contraction elements per
// instruction, KL consecutive k-elements per lane.
template <typename T>
struct Mma;

template <>
struct Mma<uint16_t> {  // bf16 stored as raw 16-bit
  static constexpr int K = 32;
  static constexpr int KL = 8;
  typedef bf16x8 frag;
  __device__ __forceinline__ static frag load(const uint16_t* p) {
    return as_bf16x8(*reinterpret_cast<const uint4*>(p));
  }
  __device__ __forceinline__ static f32x4 mma(const frag& a, const frag& b, const f32x4& c) {
    return mfma_bf16(a, b, c);
  }
  __device__ __forceinline__ static float to_f32(uint16_t v) { return bf16_to_f32(v); }
};

template <>
struct Mma<float> {
  static constexpr int K = 4;
  static constexpr int KL = 1;
  typedef float frag;
  __device__ __forceinline__ static frag load(const float* p) { return *p; }
  __device__ __forceinline__ static f32x4 mma(const frag& a, const frag& b, const f32x4& c) {
    return mfma_f32(a, b, c);
  }
  __device__ __forceinline__ static float to_f32(float v) { return v; }
};

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace slay
