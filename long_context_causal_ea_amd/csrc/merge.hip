// LSE merge of a ring step's partial (O, LSE) into the running accumulator.
// Ring attention visits one rank's key/value share per step (EasyContext
// core-technology page, hotelren.com, section 1), so each query row ends up
// with one partial result per step; over disjoint key sets the exact
// combination is a log-sum-exp of the LSEs and an LSE-weighted sum of the Os.
// Elementwise and HBM-bound: D/8 lanes per (row, head), 16-byte accesses.
#include "ea_device.h"
#include "ea_launch.h"

namespace ea {

template <int D>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a, long rows_per_batch, long total_rows) {
  constexpr int LPR = D / 8;
  const long gt = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long row = gt / LPR;
  const int part = (int)(gt % LPR);
  if (row >= total_rows) return;
  const long b = row / rows_per_batch, rem = row % rows_per_batch;
  const long srow = b * a.q_batch_rows * a.H + rem;
  const long off = srow * D + part * 8;

  constexpr float NEG_INF = -__builtin_inff();
  const float l1 = a.lse_acc[srow], l2 = a.lse_part[srow];
  const float mx = fmaxf(l1, l2), mn = fminf(l1, l2);
  const float L = (mx == NEG_INF) ? NEG_INF : mx + log1pf(expf(mn - mx));
  const float w1 = (L == NEG_INF) ? 0.f : expf(l1 - L);
  const float w2 = (L == NEG_INF) ? 0.f : expf(l2 - L);

  float pv[8];
  if (a.part_bf16) {
    const u32x4 u = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.o_part) + off);
#pragma unroll
    for (int e = 0; e < 8; ++e) pv[e] = bf16_to_f32((uint16_t)((u[e >> 1] >> ((e & 1) * 16)) & 0xffffu));
  } else {
    const f32x4* pp = reinterpret_cast<const f32x4*>(static_cast<const float*>(a.o_part) + off);
    const f32x4 x = pp[0], y = pp[1];
    pv[0] = x[0]; pv[1] = x[1]; pv[2] = x[2]; pv[3] = x[3];
    pv[4] = y[0]; pv[5] = y[1]; pv[6] = y[2]; pv[7] = y[3];
  }
  f32x4* ap = reinterpret_cast<f32x4*>(a.o_acc + off);
  f32x4 x = ap[0], y = ap[1];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[e] = w1 * x[e] + w2 * pv[e];
    y[e] = w1 * y[e] + w2 * pv[4 + e];
  }
  ap[0] = x;
  ap[1] = y;
  if (part == 0) a.lse_acc[srow] = L;
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream) {
  const long rows_per_batch = (long)a.Sq * a.H;
  const long total = rows_per_batch * a.B;
  if (total == 0) return hipSuccess;
  const long threads = total * (a.D / 8);
  dim3 grid((unsigned)((threads + 255) / 256)), block(256);
  if (a.D == 64)
    hipLaunchKernelGGL(merge_kernel<64>, grid, block, 0, stream, a, rows_per_batch, total);
  else
    hipLaunchKernelGGL(merge_kernel<128>, grid, block, 0, stream, a, rows_per_batch, total);
  return hipGetLastError();
}

}  // namespace ea
