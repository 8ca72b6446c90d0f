// Rotary position embedding of query/key rows by their global positions, and
// its transpose for gradients (the rotary base the pages raise for long
// contexts: EasyContext core-technology page, hotelren.com, further
// optimisations; kwkr.cn ZeRO-3 offload page, training script rope-theta and
// advanced optimisation item 2; cn486.com page, training strategy).
//
// Llama "rotate-half" convention, per row of head dimension D at position p and
// k = 0 .. D/2-1:  phi_k = p * theta^(-2k/D),
//   y_k = x_k cos phi_k - x_{k+D/2} sin phi_k,  y_{k+D/2} = x_{k+D/2} cos phi_k + x_k sin phi_k
// (inverse: phi_k -> -phi_k).
//
// HBM-bound elementwise pass.  A workgroup takes kRopeRows token rows (all H
// heads of each).  The D/2 angles of a row are shared by its heads: they are
// formed once per row (rope_cos_sin: fp64 angle from frequencies computed on
// the host in fp64, fp32 cosine and sine) and kept in LDS.  The rotation
// (rope_turn) is fp32 with one rounding to the output type; the attention
// kernels that rotate query rows in registers use the same two functions.  Each
// thread handles the two 16-byte chunks that hold x_k .. and x_{k+D/2} .. of
// one head.
#include "ea_device.h"
#include "ea_launch.h"

namespace ea {

constexpr int kRopeThreads = kRopeBlock;
constexpr int kRopeRows = kRopeRowsPerBlock;

struct RopeParams {
  const void* x;
  void* y;
  int64_t batch_stride;  // elements between batches (batch_rows * H * D)
  int S, H, rows;        // rows = B * S
  Seg seg;
  int inverse;
  double f[64];          // theta^(-2k/D), k < D/2
};

template <bool BF16>
struct RopeIO {
  static constexpr int EPC = BF16 ? 8 : 4;
  __device__ static void load(const void* p, float* v) {
    const u32x4 u = __builtin_nontemporal_load(static_cast<const u32x4*>(p));
    if constexpr (BF16) {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = __uint_as_float((e & 1) ? (u[e >> 1] & 0xffff0000u) : (u[e >> 1] << 16));
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = __uint_as_float(u[e]);
    }
  }
  __device__ static void store(void* p, const float* v) {
    u32x4 u;
    if constexpr (BF16) {
#pragma unroll
      for (int q = 0; q < 4; ++q) u[q] = pack_bf16x2(v[2 * q], v[2 * q + 1]);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) u[q] = __float_as_uint(v[q]);
    }
    __builtin_nontemporal_store(u, static_cast<u32x4*>(p));
  }
};

template <bool BF16, int D>
__global__ __launch_bounds__(kRopeThreads) void rope_kernel(RopeParams p) {
  using IO = RopeIO<BF16>;
  constexpr int HALF = D / 2, EPC = IO::EPC, CPH = HALF / EPC;  // chunks per half row
  constexpr int ESZ = BF16 ? 2 : 4;
  // (cos, sin) of angle k at slot k + k / EPC: the chunks a wave reads together
  // (one per lane group) then fall on distinct LDS banks
  constexpr int SLOTS = HALF + HALF / EPC;
  __shared__ float2 cs[kRopeRows][SLOTS];

  const int tid = threadIdx.x;
  const int row0 = blockIdx.x * kRopeRows;

  // ---- angles of the workgroup's rows
  for (int idx = tid; idx < kRopeRows * HALF; idx += kRopeThreads) {
    const int r = idx / HALF, k = idx % HALF, gr = row0 + r;
    if (gr >= p.rows) continue;
    float2 t = rope_cos_sin(seg_pos(p.seg, gr % p.S), p.f[k]);
    if (p.inverse) t.y = -t.y;  // the transpose: turn by minus the angle
    cs[r][k + k / EPC] = t;
  }
  __syncthreads();

  // ---- rotate: item = (row, head, chunk of the first half)
  const int items_per_row = p.H * CPH;
  for (int idx = tid; idx < kRopeRows * items_per_row; idx += kRopeThreads) {
    const int r = idx / items_per_row, rem = idx % items_per_row, gr = row0 + r;
    if (gr >= p.rows) break;  // rows are taken in order, so every later item is past the end too
    const int h = rem / CPH, c = rem % CPH;
    const int b = gr / p.S, i = gr % p.S;
    const int64_t off = (int64_t)b * p.batch_stride + ((int64_t)i * p.H + h) * D + c * EPC;
    const char* src = static_cast<const char*>(p.x) + off * ESZ;
    char* dst = static_cast<char*>(p.y) + off * ESZ;
    float lo[EPC], hi[EPC];
    IO::load(src, lo);
    IO::load(src + HALF * ESZ, hi);
#pragma unroll
    for (int e = 0; e < EPC; ++e) rope_turn(lo[e], hi[e], cs[r][c * (EPC + 1) + e], false);
    IO::store(dst, lo);
    IO::store(dst + HALF * ESZ, hi);
  }
}

template <bool BF16>
static hipError_t launch_rope_t(const RopeParams& p, int D, hipStream_t stream) {
  dim3 grid((unsigned)((p.rows + kRopeRows - 1) / kRopeRows)), block(kRopeThreads);
  if (D == 128)
    hipLaunchKernelGGL((rope_kernel<BF16, 128>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((rope_kernel<BF16, 64>), grid, block, 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_rope(const RopeArgs& a, hipStream_t stream) {
  if (a.B == 0 || a.S == 0) return hipSuccess;
  RopeParams p;
  p.x = a.x;
  p.y = a.y;
  p.batch_stride = a.batch_rows * a.H * a.D;
  p.S = a.S;
  p.H = a.H;
  p.rows = a.B * a.S;
  p.seg = Seg{a.seg.s0, a.seg.l0, a.seg.s1, a.seg.n};
  p.inverse = a.inverse;
  for (int k = 0; k < 64; ++k) p.f[k] = k < a.D / 2 ? a.inv_freq[k] : 0.0;
  return a.bf16 ? launch_rope_t<true>(p, a.D, stream) : launch_rope_t<false>(p, a.D, stream);
}

}  // namespace ea
