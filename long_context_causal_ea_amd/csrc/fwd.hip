// Forward kernel: tiled attention with online softmax and LSE output
// (EasyContext core-technology page, hotelren.com, section 2 "Flash Attention
// optimisation": the attention matrix is never stored; key/value tiles are
// staged on chip and the softmax is accumulated tile by tile).
//
// gfx950 mapping
//  - One workgroup = 4 waves = 128 query rows of one (batch, head); each wave
//    owns 32 rows.  Key/value tiles of 64 rows stream through LDS, double
//    buffered, with the next tile's global loads in flight during compute.
//  - Scores are computed transposed, S^T = K Q^T, with the 32x32x16 bf16 MFMA:
//    every lane then holds 32 scores of ONE query row, so the row max and row
//    sum are in-lane reductions plus one exchange with lane l^32.
//  - P^T (bf16, round-to-nearest-even) feeds O^T += V^T P^T directly from
//    registers.  K and V tiles are stored row-major in LDS with an XOR swizzle
//    of 16-byte chunks; the V^T operand is read with the gfx950 LDS transpose
//    read, so no transposed copy is ever written.
//  - exp is computed as exp2 with scale*log2(e) folded into one FMA.
//  - Tiles are classified per wave from global positions: SKIP (no allowed
//    pair), FULL (all allowed, no mask work) or PARTIAL (element mask; also
//    ragged key tails).  Tiles no query of the workgroup may see are never
//    loaded.
#include <type_traits>

#include "ea_device.h"
#include "ea_launch.h"

namespace ea {

struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  void* o;
  float* lse;
  long q_bstride, k_bstride, lse_bstride;  // elements between batches
  long rs;                                 // row stride (H*D elements)
  int H, Sq, Sk, nqb;
  Seg qs, ks;
  int causal, o_bf16;
  float scale, c;  // c = scale * log2(e)
};

#ifndef EA_FWD_BK
#define EA_FWD_BK 64
#endif
#ifndef EA_FWD_MIN_WG
#define EA_FWD_MIN_WG 2  // workgroups per CU the register budget is sized for
#endif

template <int D>
struct FwdCfg {
  static constexpr int BQ = 128, BK = EA_FWD_BK, NT = 256;
  static constexpr int NMB = BK / 32, NKB = BK / 16;  // 32-key MFMA blocks, 16-key reduction steps
  static constexpr int CPR = D / 8;  // 16-byte chunks per row
  static constexpr int NKL = BK * CPR / NT;  // chunks per thread per tile (each of K and V)
  static constexpr int LDS_T = BK * D;
  static_assert(BK % 32 == 0 && NKL * NT == BK * CPR, "unsupported key tile");
};

template <int D>
__global__ __launch_bounds__(256, EA_FWD_MIN_WG) void fwd_kernel(FwdParams p) {
  using Cfg = FwdCfg<D>;
  constexpr int BQ = Cfg::BQ, BK = Cfg::BK, CPR = Cfg::CPR;
  constexpr int NKS = D / 16, NDB = D / 32, NMB = Cfg::NMB, NKB = Cfg::NKB;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][Cfg::LDS_T];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][Cfg::LDS_T];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int ln = lane & 31, g = lane >> 5;

  // ---- work item: (batch*head) major, longest query blocks first
  const int work = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = work / p.nqb;
  const int qb = p.nqb - 1 - work % p.nqb;
  const int b = bh / p.H, h = bh % p.H;
  const int D_ = D;

  const uint16_t* qp = p.q + b * p.q_bstride + (long)h * D_;
  const uint16_t* kp = p.k + b * p.k_bstride + (long)h * D_;
  const uint16_t* vp = p.v + b * p.k_bstride + (long)h * D_;

  const int i0 = qb * BQ;
  const int qrow = i0 + w * 32 + ln;
  const bool row_ok = qrow < p.Sq;

  // ---- this lane's query row in MFMA B-operand form (8 dims per k-step)
  bf16x8 qf[NKS];
  {
    const u32x4* src = reinterpret_cast<const u32x4*>(qp + (long)(row_ok ? qrow : 0) * p.rs + 8 * g);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      u32x4 u = row_ok ? src[2 * ks] : u32x4{0u, 0u, 0u, 0u};
      qf[ks] = as_bf16x8(u);
    }
  }
  const int qpos = seg_pos(p.qs, row_ok ? qrow : (p.Sq - 1));
  const KeyWindow kwin = key_window(p.ks, qpos, p.causal);

  // ---- position ranges of the workgroup's and this wave's valid rows
  const int wg_end = min(i0 + BQ, p.Sq);
  int qmin_wg, qmax_wg;
  seg_range(p.qs, i0, wg_end, qmin_wg, qmax_wg);
  const int w0 = i0 + w * 32, w1 = min(w0 + 32, p.Sq);
  const bool wave_live = w0 < w1;
  int qmin_w = 0, qmax_w = -1;
  if (wave_live) seg_range(p.qs, w0, w1, qmin_w, qmax_w);

  // ---- key tiles to visit: up to two contiguous runs
  int e0 = p.Sk, b1 = p.Sk, e1 = p.Sk;
  if (p.causal) causal_key_ranges(p.ks, qmax_wg, e0, b1, e1);
  const int nA = (e0 + BK - 1) / BK;
  int tB0 = b1 / BK, tB1 = (e1 + BK - 1) / BK;
  if (e1 <= b1) tB1 = tB0;
  if (tB0 < nA) tB0 = nA;
  const int nB = tB1 > tB0 ? tB1 - tB0 : 0;
  const int nt = nA + nB;

  // ---- running statistics (raw-score units for the max)
  constexpr float NEG_INF = -__builtin_inff();
  float m_run = NEG_INF, l_run = 0.f;
  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};

  u32x4 kreg[Cfg::NKL], vreg[Cfg::NKL];

  auto tile_of = [&](int t) { return t < nA ? t : tB0 + (t - nA); };

  // global -> registers: consecutive threads take consecutive 16-byte chunks of a row
  auto load_tile = [&](int jt) {
    const int j0 = jt * BK;
#pragma unroll
    for (int it = 0; it < Cfg::NKL; ++it) {
      const int c = tid + Cfg::NT * it;
      const int row = c / CPR, col = c % CPR;
      const int j = j0 + row;
      const long off = (long)j * p.rs + col * 8;
      kreg[it] = j < p.Sk ? *reinterpret_cast<const u32x4*>(kp + off) : u32x4{0u, 0u, 0u, 0u};
      vreg[it] = j < p.Sk ? *reinterpret_cast<const u32x4*>(vp + off) : u32x4{0u, 0u, 0u, 0u};
    }
  };

  // registers -> LDS, swizzled row-major
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int it = 0; it < Cfg::NKL; ++it) {
      const int c = tid + Cfg::NT * it;
      const int row = c / CPR, col = c % CPR;
      const int o = tile_off<D>(row, col);
      *reinterpret_cast<u32x4*>(&Ks[buf][o]) = kreg[it];
      *reinterpret_cast<u32x4*>(&Vs[buf][o]) = vreg[it];
    }
  };

  // per-lane LDS offsets (elements), fixed for the whole kernel: with the tile
  // buffer, the 32-key block and the 16-key step folded in as immediates, no
  // address arithmetic is left in the loop
  int kofs[NKS];  // K operand: row ln, chunk 2*ks+g
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) kofs[ks] = ln * D + (((2 * ks + g) ^ swz<D>(ln)) << 3);
  int vofs[2][NDB];  // V^T transpose read: rows 8*half + trow (+16 per step), 32 dims per block
  {
    const int trow = 4 * g + ((lane & 15) >> 2);
    const int tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int col = 32 * db + tcol;
        vofs[half][db] = tile_off<D>(8 * half + trow, col >> 3) + (col & 7);
      }
  }

  // one key tile: classify, scores, online softmax, P V.  BUF is a compile-time
  // buffer index so that every LDS offset is an immediate.
  auto tile_step = [&](auto BUF, int t) {
    constexpr int buf = decltype(BUF)::value;
    const int jt = tile_of(t);
    const int j0 = jt * BK;
    store_tile(buf);
    __syncthreads();
    if (t + 1 < nt) load_tile(tile_of(t + 1));

    // wave-level tile class
    int cls = kSkip;
    if (wave_live) {
      const int jend = min(j0 + BK, p.Sk);
      int kmn, kmx;
      seg_range(p.ks, j0, jend, kmn, kmx);
      const bool tail = j0 + BK > p.Sk;
      if (!p.causal) cls = tail ? kPartial : kFull;
      else if (kmn > qmax_w) cls = kSkip;
      else if (kmx <= qmin_w && !tail) cls = kFull;
      else cls = kPartial;
    }
    if (cls == kSkip) return;

    // S^T = K Q^T, one 32-key MFMA block at a time
    f32x16 st[NMB];
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
      st[mb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(&Ks[buf][kofs[ks] + mb * 32 * D]);
        st[mb] = mfma32(as_bf16x8(a), qf[ks], st[mb]);
      }
    }

    if (cls == kPartial) {
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = j0 + mb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
          st[mb][r] = in_window(kwin, j) ? st[mb][r] : NEG_INF;
        }
      }
    }

    // online softmax: tile max, conditional rescale, exponentials, partial sums
    float mx = NEG_INF;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[mb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mnew = fmaxf(m_run, mx);
    if (__any(mnew > m_run)) {
      const float alpha = (m_run == NEG_INF) ? 0.f : fast_exp2((m_run - mnew) * p.c);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
      m_run = mnew;
    }
    const float msub = (m_run == NEG_INF) ? 0.f : m_run * p.c;
    bf16x8 pb[NKB];
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = fast_exp2(__builtin_fmaf(st[mb][r], p.c, -msub));
        st[mb][r] = e;
        l_run += e;
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int o = 8 * kk;
        pb[2 * mb + kk] = pack_bf16x8(st[mb][o + 0], st[mb][o + 1], st[mb][o + 2], st[mb][o + 3], st[mb][o + 4],
                                      st[mb][o + 5], st[mb][o + 6], st[mb][o + 7]);
      }
    }

    // O^T += V^T P^T; V^T read transposed from the row-major V tile
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const u32x2 lo = ds_read_tr16(&Vs[buf][vofs[0][db] + kb * 16 * D]);
        const u32x2 hi = ds_read_tr16(&Vs[buf][vofs[1][db] + kb * 16 * D]);
        const u32x4 a = {lo[0], lo[1], hi[0], hi[1]};
        oacc[db] = mfma32(as_bf16x8(a), pb[kb], oacc[db]);
      }
    }
  };

  if (nt > 0) load_tile(tile_of(0));
  for (int t = 0; t < nt; t += 2) {
    tile_step(std::integral_constant<int, 0>{}, t);
    if (t + 1 < nt) tile_step(std::integral_constant<int, 1>{}, t + 1);
  }

  // ---- epilogue: normalise, write O and LSE
  const float lt = l_run + __shfl_xor(l_run, 32);
  if (!row_ok) return;
  const bool has = lt > 0.f;
  const float inv = has ? 1.f / lt : 0.f;
  if (p.o_bf16) {
    uint16_t* op = static_cast<uint16_t*>(p.o) + b * p.q_bstride + (long)h * D_ + (long)qrow * p.rs;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = db * 32 + 8 * q4 + 4 * g;
        u32x2 val;
        val[0] = pack_bf16x2(oacc[db][4 * q4 + 0] * inv, oacc[db][4 * q4 + 1] * inv);
        val[1] = pack_bf16x2(oacc[db][4 * q4 + 2] * inv, oacc[db][4 * q4 + 3] * inv);
        *reinterpret_cast<u32x2*>(op + d0) = val;
      }
  } else {
    float* op = static_cast<float*>(p.o) + b * p.q_bstride + (long)h * D_ + (long)qrow * p.rs;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = db * 32 + 8 * q4 + 4 * g;
        f32x4 val = {oacc[db][4 * q4 + 0] * inv, oacc[db][4 * q4 + 1] * inv, oacc[db][4 * q4 + 2] * inv,
                     oacc[db][4 * q4 + 3] * inv};
        *reinterpret_cast<f32x4*>(op + d0) = val;
      }
  }
  if (g == 0) {
    const float lse = has ? (m_run * p.scale + logf(lt)) : NEG_INF;
    p.lse[b * p.lse_bstride + (long)qrow * p.H + h] = lse;
  }
}

static Seg to_seg(const SegArg& s) { return Seg{s.s0, s.l0, s.s1, s.n}; }

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
  FwdParams p;
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.o = a.o;
  p.lse = a.lse;
  p.rs = (long)a.H * a.D;
  p.q_bstride = (long)a.q_batch_rows * p.rs;
  p.k_bstride = (long)a.k_batch_rows * p.rs;
  p.lse_bstride = (long)a.q_batch_rows * a.H;
  p.H = a.H;
  p.Sq = a.Sq;
  p.Sk = a.Sk;
  p.qs = to_seg(a.qs);
  p.ks = to_seg(a.ks);
  p.causal = a.causal;
  p.o_bf16 = a.o_bf16;
  p.scale = a.scale;
  p.c = a.scale * kLog2e;
  const int BQ = FwdCfg<128>::BQ;
  p.nqb = (a.Sq + BQ - 1) / BQ;
  const long nwg = (long)a.B * a.H * p.nqb;
  if (nwg == 0) return hipSuccess;
  dim3 grid((unsigned)nwg), block(256);
  if (a.D == 64)
    hipLaunchKernelGGL(fwd_kernel<64>, grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL(fwd_kernel<128>, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace ea
