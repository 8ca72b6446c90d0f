// Host-side launch parameters and launchers of the gfx950 kernels.  The public
// C entry points (api.hip) validate their arguments, fill these structs and
// call the launchers; nothing here checks arguments again.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ea {

struct SegArg {
  int s0, l0, s1, n;  // rows [0,l0) at s0+i, rows [l0,n) at s1+(i-l0)
};

struct FwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  void* o;
  float* lse;
  int B, H, D, Sq, Sk;
  int64_t q_batch_rows, k_batch_rows;
  SegArg qs, ks;
  int causal;
  int o_bf16;
  int merge;  // 1: merge into (o, lse) as an fp32 accumulator instead of overwriting
  float scale;
  int rope;             // 1: q rows are turned by their rotary angles in registers before use
  uint16_t* q_rot;      // when rope: the turned q rows are also written here (may be null)
  double inv_freq[64];  // when rope: theta^(-2k/D), k < D/2
};

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const void* o;
  const uint16_t* dout;
  const float* lse;
  float* delta;
  float* dq;
  float* dk;
  float* dv;
  int B, H, D, Sq, Sk;
  int Hs;  // heads per token row (the row stride); H of them, from the pointers on, are processed
  int64_t q_batch_rows, k_batch_rows;
  SegArg qs, ks;
  int causal;
  int o_bf16;
  float scale;
  int rope;             // 1: q, k are rotated rows; dq, dk contributions are turned back before they are added
  double inv_freq[64];  // when rope: theta^(-2k/D), k < D/2
};

struct MergeArgs {
  float* o_acc;
  float* lse_acc;
  const void* o_part;
  const float* lse_part;
  int part_bf16;
  int B, H, D, Sq;
  int64_t q_batch_rows;
};

struct XentArgs {
  void* logits;  // [rows, V] with row_stride, overwritten by the gradient
  const int64_t* labels;
  float* loss;
  float* lse;
  long rows, row_stride;
  int V;
  long ignore_index;
  float grad_scale;
  int bf16;
};

struct RopeArgs {
  const void* x;  // [B, S, H, D] with batch stride batch_rows * H * D
  void* y;        // same layout; may equal x
  int B, H, S, D;
  int64_t batch_rows;
  SegArg seg;
  int inverse;
  int bf16;
  double inv_freq[64];  // theta^(-2k/D), k < D/2
};

// Workgroup shapes of the elementwise launches (the host bounds their grids).
constexpr int kXentBlock = 512;        // threads per workgroup, one workgroup per logits row
constexpr int kRopeBlock = 256;        // threads per workgroup
constexpr int kRopeRowsPerBlock = 4;   // token rows per workgroup

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_delta(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_dkdv(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t stream);
hipError_t launch_merge(const MergeArgs& a, hipStream_t stream);
hipError_t launch_xent(const XentArgs& a, hipStream_t stream);
hipError_t launch_rope(const RopeArgs& a, hipStream_t stream);

}  // namespace ea
