// slay_internal.hpp -- host-side launch interface between the C ABI layer
// (slay_api.cpp) and the HIP kernels.  Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "slay.h"
#include "slay_device.hpp"

namespace slay {

// slay_attn_chunked_fwd's checks and launch.  With `scratch` set, the call
// uses a fixed device scratch of workspace_bytes bytes instead of `workspace`:
// once every argument has passed its checks, scratch(stream, &ptr) supplies
// its device address, and a shape whose workspace exceeds the scratch is
// refused (SLAY_E_UNSUPPORTED).
typedef hipError_t (*ScratchFn)(hipStream_t stream, void** ptr);
slay_status_t chunked_fwd_entry(const slay_params_t* params, const void* q, const void* k, const void* v,
                                slay_dtype_t io_dtype, int32_t B, int32_t H, int64_t L, int32_t dv, int32_t chunk,
                                const float* S0, const float* z0, void* o, float* S_out, float* z_out,
                                void* workspace, size_t workspace_bytes, void* stream, ScratchFn scratch);

// Raise a kernel's dynamic-LDS limit once per (kernel, device): the setting
// persists on the device, so later launches make no call besides the launch
// itself (they may be under stream capture).
hipError_t set_max_lds(const void* kernel, int bytes);

struct FeatmapArgs {
  const void* x;          // [n_heads * rows_per_head][d]
  const void* x2;         // nullable: a second input of the same shape (phi2 <- phi(x2)), same launch
  int64_t rows_per_head;  // rows sharing one draw set
  int64_t n_heads;
  int d, F, m;
  bool x_bf16;            // x and draws: bf16 if true, else fp32
  const void* anchors;    // [n_draw_sets][F][d]
  const void* prf;
  int64_t draw_set_stride;  // elements between draw sets
  int n_draw_sets;          // head h uses set h % n_draw_sets
  NodeConsts nc;
  void* phi;              // [rows][F]
  void* phi2;             // used when x2 is set
  bool phi_bf16;
};

bool featmap_supported(int d);
hipError_t launch_featmap(const FeatmapArgs& a, hipStream_t s);

// Chunked forward over n_heads = B*H heads: causal (Lq == L) or non-causal
// (every query attends to all L keys; Lq queries per head).
struct ChunkedArgs {
  const void* q;  // [n_heads][Lq][d]
  const void* k;  // [n_heads][L][d]
  const void* v;  // [n_heads][L][dv]
  bool io_bf16;
  bool causal;
  int64_t n_heads, L, Lq;
  int d, dv, F, m, R, chunk;
  const void* anchors;
  const void* prf;
  int64_t draw_set_stride;
  int n_draw_sets;
  NodeConsts nc;
  const float* S0;  // nullable [n_heads][F][dv]
  const float* z0;  // nullable [n_heads][F]
  void* o;          // [n_heads][Lq][dv]
  float* S_out;     // nullable
  float* z_out;     // nullable
  void* ws;
  size_t ws_bytes;
};

// Fused MFMA path (bf16): returns true if the shape has a compiled variant.
bool fused_supported(const ChunkedArgs& a);
size_t fused_workspace_bytes(const ChunkedArgs& a);
hipError_t launch_fused(const ChunkedArgs& a, hipStream_t s);

// Segment geometry of the fused path (0 segments if the shape has no fused
// variant) and the prefix states of every key segment in its fragment-ordered
// layout [n_heads][n_seg][F/16][(dv+16)/16][64][4] (the backward's input).
int fused_segment_count(const ChunkedArgs& a, int64_t* seg_len);
hipError_t launch_segment_prefix(const ChunkedArgs& a, float* ws, hipStream_t s);

// Wide MFMA path (bf16, causal, F in {128, 256, 384, 512}, dv in {64, 128}):
// feature maps materialised in bf16, the state kept on chip per segment.
bool wide_supported(const ChunkedArgs& a);
size_t wide_workspace_bytes(const ChunkedArgs& a);
hipError_t launch_wide(const ChunkedArgs& a, hipStream_t s);

// Generic path (any supported dtype/shape; unfused, plain FMA).
bool generic_supported(const ChunkedArgs& a);
size_t generic_workspace_bytes(const ChunkedArgs& a);
hipError_t launch_generic(const ChunkedArgs& a, hipStream_t s);

// Zero-padded copies of row blocks on the stream: dst[b][r][:] = src[b][r][:]
// for r < rows_src, 0 for rows_src <= r < rows_dst (row_elems elements per
// row; strides in elements).  Feature counts the MFMA kernels are not built
// for run a larger count's kernels on zero-padded draws and states.
hipError_t pad_rows(uint16_t* dst, const uint16_t* src, int64_t n_blocks, int64_t rows_src, int64_t rows_dst,
                    int64_t row_elems, int64_t src_stride, int64_t dst_stride, hipStream_t s);
hipError_t pad_rows(float* dst, const float* src, int64_t n_blocks, int64_t rows_src, int64_t rows_dst,
                    int64_t row_elems, int64_t src_stride, int64_t dst_stride, hipStream_t s);

// Prefix scan of per-item states (shared by both paths).
// layout 0: plain [F][dv+1] (z in column dv); layout 1: MFMA fragment order
// with dv+16 columns (z in column dv), see slay_chunked_fused.hip.
struct ScanArgs {
  float* states;      // [n_heads][n_items][E], in place: item i <- init + sum_{i'<i} item i'
  int64_t n_heads;
  int64_t n_items;    // number of prefix entries written
  int64_t n_terms;    // number of delta items read (n_items or n_items - 1)
  int F, dv, layout;
  const float* S0;    // nullable init
  const float* z0;
  float* S_out;       // nullable: init + sum of all n_terms items
  float* z_out;
  bool reverse;       // suffix instead of prefix: item i <- init + sum_{i' > i} item i' (n_terms == n_items)
  bool total_only;    // write only the last item (the total), not the prefixes before it
};
int64_t scan_state_elems(int F, int dv, int layout);
hipError_t launch_scan(const ScanArgs& a, hipStream_t s);
hipError_t launch_scan_varlen(float* states, int64_t H, int n_seqs, int g_max, const int* first, const int* n_a,
                              const int* last, int F, int dv, const float* S0, const float* z0, float* S_out,
                              float* z_out, hipStream_t s);

// Variable-length batch of the causal forward: n_seqs sequences packed along
// the token axis of each of H heads (q, k [H][T][d], v, o [H][T][dv]),
// sequence s at tokens cu[s] .. cu[s+1] (device int64, n_seqs + 1 entries);
// states [n_seqs][H][F][dv].
struct VarlenArgs {
  ChunkedArgs c;  // q, k, v, o, dtypes, d, dv, F, m, R, draws, nc, S0, z0, S_out, z_out, ws (n_heads = H, L = T)
  int n_seqs;
  const int64_t* cu;
};
bool varlen_supported(const VarlenArgs& a);
size_t varlen_workspace_bytes(const VarlenArgs& a);
hipError_t launch_varlen(const VarlenArgs& a, hipStream_t s);

// Per-chunk states dS_c = phi(k_c)^T [v_c | 1] of the general path, fp32
// [n_heads][item_stride][F][dv+1] (chunk c at item c).
hipError_t launch_chunk_state(const float* phik, const void* v, bool v_bf16, int64_t n_heads, int64_t L, int F,
                              int dv, int C, int64_t item_stride, float* states, hipStream_t s);

// Backward of the causal chunked forward.
struct BackwardArgs {
  const void* q;     // [n_heads][L][d]
  const void* k;
  const void* v;     // [n_heads][L][dv]
  const void* dout;  // [n_heads][L][dv]
  bool io_bf16;
  int64_t n_heads, L;
  int d, dv, F, m, R, chunk;
  const void* anchors;
  const void* prf;
  int64_t draw_set_stride;
  int n_draw_sets;
  NodeConsts nc;
  const float* S0;    // nullable [n_heads][F][dv]
  const float* z0;    // nullable [n_heads][F]
  const float* dS_T;  // nullable gradient of the final state
  const float* dz_T;
  void* dq;           // [n_heads][L][d]
  void* dk;
  void* dv_out;       // [n_heads][L][dv]
  float* dS0;         // nullable [n_heads][F][dv]
  float* dz0;         // nullable [n_heads][F]
  void* ws;
  size_t ws_bytes;
};
bool backward_supported(const BackwardArgs& a);
// MFMA path of the backward (bf16, d = dv = 64, chunk 64, F <= 256 a multiple
// of 32; F below 256 on zero-padded features).
bool backward_fused_supported(const BackwardArgs& a);
size_t backward_fused_workspace_bytes(const BackwardArgs& a);
hipError_t launch_backward_fused(const BackwardArgs& a, hipStream_t s);
size_t backward_workspace_bytes(const BackwardArgs& a);
hipError_t launch_backward(const BackwardArgs& a, hipStream_t s);

// Recurrent decode step.
struct DecodeArgs {
  const void* q;  // [n_heads][d]
  const void* k;
  const void* v;  // [n_heads][dv]
  bool io_bf16;
  int64_t n_heads;
  int d, dv, F, m;
  const void* anchors;  // fp32 draws
  const void* prf;
  bool draws_bf16;
  int64_t draw_set_stride;
  int n_draw_sets;
  NodeConsts nc;
  float* S;  // [n_heads][F][dv]
  float* z;  // [n_heads][F]
  void* o;   // [n_heads][dv]
  void* ws;  // phi(q), phi(k): 2 * n_heads * F fp32
};
bool decode_supported(const DecodeArgs& a);
size_t decode_workspace_bytes(const DecodeArgs& a);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);

}  // namespace slay
