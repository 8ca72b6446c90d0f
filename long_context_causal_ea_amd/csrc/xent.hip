// Fused cross-entropy forward + backward over vocabulary logits, gradient
// written in place (the fused cross-entropy kernel with in-place backward that
// the training step uses: EasyContext ZeRO-3 offload page, kwkr.cn, section
// on advanced optimisation combined with other techniques, item 1; cn486.com
// page, summary of the training script's technology stack).
//
// Per row i of x [N, V] with label y_i and upstream gradient scale g:
//   LSE_i = ln sum_j exp(x_ij),   loss_i = LSE_i - x_{i,y_i},
//   x_ij <- g * (exp(x_ij - LSE_i) - [j == y_i])
// (0 loss and 0 gradient where y_i == ignore_index).
//
// HBM-bound: one workgroup per row reads the row once (non-temporal 16-byte
// loads, consecutive lanes on consecutive chunks) into registers, takes each
// thread's maximum m_t and sum of exp(x - m_t), reduces (max, sum) over the
// workgroup and writes g * exp(x - LSE) back over the row with non-temporal
// stores.  bf16 rows are held packed and exponentiated twice (registers, not
// ALU, limit how many rows are in flight); fp32 rows are held as exp(x - m_t)
// and scaled by exp(m_t - LSE).  Rows longer than the register budget (65536
// elements at 512 threads) are streamed twice instead.
#include "ea_device.h"
#include "ea_launch.h"

namespace ea {

struct XentParams {
  void* x;
  const int64_t* labels;
  float* loss;
  float* lse;
  long row_stride;  // elements between rows
  int V;
  long ignore_index;
  float g;
};

constexpr int kXentThreads = kXentBlock;

// (m, s) stands for s * exp(m): merge another such pair into it
__device__ __forceinline__ void combine(float& m, float& s, float m2, float s2) {
  const float mn = fmaxf(m, m2);
  const float a = (m == -__builtin_inff()) ? 0.f : s * fast_exp2((m - mn) * kLog2e);
  const float b = (m2 == -__builtin_inff()) ? 0.f : s2 * fast_exp2((m2 - mn) * kLog2e);
  m = mn;
  s = a + b;
}

template <bool BF16>
struct XentIO {
  static constexpr int EPC = BF16 ? 8 : 4;  // elements per 16-byte chunk
  // 16-byte chunk c; non-temporal, as every byte of the row is read once and written once
  __device__ static u32x4 load_raw(const void* base, int c) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base) + c);
  }
  // element e of a 16-byte chunk of bf16 values, as fp32
  __device__ static float unpack(const u32x4& u, int e) {
    return __uint_as_float((e & 1) ? (u[e >> 1] & 0xffff0000u) : (u[e >> 1] << 16));
  }
  __device__ static void load(const void* base, int c, float* v) {
    const u32x4 u = load_raw(base, c);
    if constexpr (BF16) {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = unpack(u, e);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = __uint_as_float(u[e]);
    }
  }
  __device__ static void store(void* base, int c, const float* v) {
    if constexpr (BF16) {
      u32x4 o;
#pragma unroll
      for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(v[2 * q], v[2 * q + 1]);
      __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(base) + c);
    } else {
      __builtin_nontemporal_store((f32x4{v[0], v[1], v[2], v[3]}), reinterpret_cast<f32x4*>(base) + c);
    }
  }
  __device__ static float load1(const void* base, long j) {
    if constexpr (BF16) return bf16_to_f32(reinterpret_cast<const uint16_t*>(base)[j]);
    else return reinterpret_cast<const float*>(base)[j];
  }
  __device__ static void store1(void* base, long j, float y) {
    if constexpr (BF16) {
      reinterpret_cast<uint16_t*>(base)[j] = (uint16_t)(pack_bf16x2(y, 0.f) & 0xffffu);
    } else {
      reinterpret_cast<float*>(base)[j] = y;
    }
  }
};

// CPT: 16-byte chunks per thread held in registers (0: stream the row twice)
template <bool BF16, int CPT>
__global__ __launch_bounds__(kXentThreads) void xent_kernel(XentParams p) {
  using IO = XentIO<BF16>;
  constexpr int EPC = IO::EPC, NT = kXentThreads;
  constexpr float NEG_INF = -__builtin_inff();
  // bf16 rows stay packed in registers (half the registers, so more rows in
  // flight per CU) at the price of a second exponential per element; fp32 rows
  // keep exp(x - m) from pass 1
  constexpr bool PK = BF16;
  __shared__ float red_m[NT / 64], red_s[NT / 64], lbl_x;

  const long row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  constexpr int ESZ = BF16 ? 2 : 4;
  void* base = static_cast<char*>(p.x) + row * p.row_stride * ESZ;
  // Rows need not start on 16 bytes: up to EPC-1 head elements before the first
  // aligned chunk and up to EPC-1 tail elements after the last one are taken
  // one per lane.
  const int mis = (int)((reinterpret_cast<uintptr_t>(base) & 15) / ESZ);
  const int head = mis ? min(EPC - mis, p.V) : 0;
  void* body = static_cast<char*>(base) + head * ESZ;
  const int nchunk = (p.V - head) / EPC, tail0 = head + nchunk * EPC;
  const long label = p.labels[row];
  const bool ignored = label == p.ignore_index;
  const bool bad = !ignored && (label < 0 || label >= p.V);
  const bool head_lane = tid < head, tail_lane = tail0 + tid < p.V;
  if (tid == 0) lbl_x = (ignored || bad) ? 0.f : IO::load1(base, label);  // read before any write to the row

  // ---- pass 1: this thread's maximum m and sum s of exp(x - m)
  float m = NEG_INF, s = 0.f;
  float xv[CPT > 0 && !PK ? CPT * EPC : 1];
  u32x4 raw[CPT > 0 && PK ? CPT : 1];
  float xh = head_lane ? IO::load1(base, tid) : NEG_INF;
  float xt = tail_lane ? IO::load1(base, tail0 + tid) : NEG_INF;
  if constexpr (CPT > 0 && PK) {
#pragma unroll
    for (int k = 0; k < CPT; ++k)
      raw[k] = (tid + NT * k < nchunk) ? IO::load_raw(body, tid + NT * k) : u32x4{0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u};
#pragma unroll
    for (int k = 0; k < CPT; ++k)
#pragma unroll
      for (int e = 0; e < EPC; ++e) m = fmaxf(m, IO::unpack(raw[k], e));
    // keep the compiler from holding the unpacked fp32 copies live across the passes
#pragma unroll
    for (int k = 0; k < CPT; ++k) asm volatile("" : "+v"(raw[k]));
    m = fmaxf(m, fmaxf(xh, xt));
    if (m != NEG_INF) {
      const float ml = m * kLog2e;
#pragma unroll
      for (int k = 0; k < CPT; ++k)
#pragma unroll
        for (int e = 0; e < EPC; ++e) s += fast_exp2(__builtin_fmaf(IO::unpack(raw[k], e), kLog2e, -ml));
#pragma unroll
      for (int k = 0; k < CPT; ++k) asm volatile("" : "+v"(raw[k]));
      xh = fast_exp2(__builtin_fmaf(xh, kLog2e, -ml));
      xt = fast_exp2(__builtin_fmaf(xt, kLog2e, -ml));
      s += xh + xt;
    }
  } else if constexpr (CPT > 0) {
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      if (tid + NT * k < nchunk)
        IO::load(body, tid + NT * k, &xv[k * EPC]);
      else
#pragma unroll
        for (int e = 0; e < EPC; ++e) xv[k * EPC + e] = NEG_INF;
    }
#pragma unroll
    for (int i = 0; i < CPT * EPC; ++i) m = fmaxf(m, xv[i]);
    m = fmaxf(m, fmaxf(xh, xt));
    if (m != NEG_INF) {
      const float ml = m * kLog2e;
#pragma unroll
      for (int i = 0; i < CPT * EPC; ++i) {
        xv[i] = fast_exp2(__builtin_fmaf(xv[i], kLog2e, -ml));  // exp(x - m); 0 for the padding
        s += xv[i];
      }
      xh = fast_exp2(__builtin_fmaf(xh, kLog2e, -ml));
      xt = fast_exp2(__builtin_fmaf(xt, kLog2e, -ml));
      s += xh + xt;
    }
  } else {
    for (int c = tid; c < nchunk; c += NT) {
      float v[EPC];
      IO::load(body, c, v);
      float cm = NEG_INF;
#pragma unroll
      for (int e = 0; e < EPC; ++e) cm = fmaxf(cm, v[e]);
      float cs = 0.f;
      if (cm != NEG_INF)
#pragma unroll
        for (int e = 0; e < EPC; ++e) cs += fast_exp2((v[e] - cm) * kLog2e);
      combine(m, s, cm, cs);
    }
    if (head_lane) combine(m, s, xh, 1.f);
    if (tail_lane) combine(m, s, xt, 1.f);
  }

  // ---- workgroup reduction of (max, sum)
  float wm = m, ws = s;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) combine(wm, ws, __shfl_xor(wm, o), __shfl_xor(ws, o));
  if (lane == 0) {
    red_m[w] = wm;
    red_s[w] = ws;
  }
  __syncthreads();  // also orders the label read above before the writes below
  float rm = red_m[0], rs = red_s[0];
#pragma unroll
  for (int i = 1; i < NT / 64; ++i) combine(rm, rs, red_m[i], red_s[i]);
  const float lse = rm + logf(rs);

  // ---- pass 2: gradient over the row
  const float g = ignored ? 0.f : (bad ? __builtin_nanf("") : p.g);
  const long lrel = (ignored || bad) ? -1 : label - head;  // label within the aligned body
  const long lc = (lrel >= 0 && lrel < (long)nchunk * EPC) ? lrel / EPC : -1;  // its chunk (-1: none)
  const int le = (int)(lrel - lc * EPC);
  if constexpr (CPT > 0) {
    // exp(x - LSE) = exp(x - m) * exp(m - LSE)
    const float f = g * ((m == NEG_INF) ? 0.f : fast_exp2((m - lse) * kLog2e));
    const float ll = lse * kLog2e;
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      const int c = tid + NT * k;
      if (c >= nchunk) continue;
      float y[EPC];
      if constexpr (PK) {
#pragma unroll
        for (int e = 0; e < EPC; ++e) y[e] = g * fast_exp2(__builtin_fmaf(IO::unpack(raw[k], e), kLog2e, -ll));
      } else {
#pragma unroll
        for (int e = 0; e < EPC; ++e) y[e] = xv[k * EPC + e] * f;
      }
      if (c == lc)
#pragma unroll
        for (int e = 0; e < EPC; ++e) y[e] -= (e == le) ? g : 0.f;
      IO::store(body, c, y);
    }
    if (head_lane) IO::store1(base, tid, xh * f - (tid == label ? g : 0.f));
    if (tail_lane) {
      const long j = tail0 + tid;
      IO::store1(base, j, xt * f - (j == label ? g : 0.f));
    }
  } else {
    for (int c = tid; c < nchunk; c += NT) {
      float v[EPC];
      IO::load(body, c, v);
#pragma unroll
      for (int e = 0; e < EPC; ++e) v[e] = g * fast_exp2((v[e] - lse) * kLog2e);
      if (c == lc)
#pragma unroll
        for (int e = 0; e < EPC; ++e) v[e] -= (e == le) ? g : 0.f;
      IO::store(body, c, v);
    }
    if (head_lane) IO::store1(base, tid, g * fast_exp2((xh - lse) * kLog2e) - (tid == label ? g : 0.f));
    if (tail_lane) {
      const long j = tail0 + tid;
      IO::store1(base, j, g * fast_exp2((xt - lse) * kLog2e) - (j == label ? g : 0.f));
    }
  }
  if (tid == 0) {
    p.lse[row] = lse;
    p.loss[row] = ignored ? 0.f : (bad ? __builtin_nanf("") : lse - lbl_x);
  }
}

template <bool BF16>
static hipError_t launch_xent_t(const XentParams& p, long rows, hipStream_t stream) {
  constexpr int EPC = XentIO<BF16>::EPC;
  const long per = (p.V / EPC + kXentThreads - 1) / kXentThreads;  // chunks per thread
  const long elems = per * EPC;                                    // elements per thread
  dim3 grid((unsigned)rows), block(kXentThreads);
  if (per <= 4)
    hipLaunchKernelGGL((xent_kernel<BF16, 4>), grid, block, 0, stream, p);
  else if (per * EPC <= 64)
    hipLaunchKernelGGL((xent_kernel<BF16, 64 / EPC>), grid, block, 0, stream, p);
  else if (elems <= 128)
    hipLaunchKernelGGL((xent_kernel<BF16, 128 / EPC>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((xent_kernel<BF16, 0>), grid, block, 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_xent(const XentArgs& a, hipStream_t stream) {
  if (a.rows == 0) return hipSuccess;
  XentParams p;
  p.x = a.logits;
  p.labels = a.labels;
  p.loss = a.loss;
  p.lse = a.lse;
  p.row_stride = a.row_stride;
  p.V = a.V;
  p.ignore_index = a.ignore_index;
  p.g = a.grad_scale;
  return a.bf16 ? launch_xent_t<true>(p, a.rows, stream) : launch_xent_t<false>(p, a.rows, stream);
}

}  // namespace ea
