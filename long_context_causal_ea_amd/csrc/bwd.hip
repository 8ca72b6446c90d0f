// Backward kernels: recompute-from-LSE gradient of tiled attention
// (EasyContext core-technology page, hotelren.com, section 2 "Flash Attention
// optimisation": recomputation replaces the stored attention matrix).
//
// Three launches on one stream:
//  1. delta:  Delta_i = <dO_i, O_i>, one pass over O and dO (HBM-bound).
//  2. dkdv:   one workgroup per block of 16*NW keys (NW waves x 16 keys).  Each
//             wave keeps its keys' K and V rows in registers and its dK^T, dV^T
//             accumulators in fp32 registers, and streams query tiles (Q, dO,
//             LSE, Delta) through double-buffered LDS.  Scores are computed
//             with the key on the MFMA column (lane) axis of the 16x16x32 MFMA,
//             so P and dS come out of the MFMA already in the B-operand form
//             that dV^T += dO^T P and dK^T += Q^T dS need; the dO^T and Q^T
//             operands are read from the row-major tiles with the LDS
//             transpose read.
//  3. dq:     one workgroup per 128-query block, streaming key tiles like the
//             forward; recomputes S^T and dP^T with the query on the lane axis
//             and accumulates dQ^T += K^T dS^T in registers (K^T by transpose
//             read of the row-major K tile).
// All LDS tiles are row-major with the XOR chunk swizzle of ea_device.h.
// The dq pass recomputes the two score products instead of exchanging dS
// through atomics: every output element is then written by exactly one
// workgroup, without atomics, and results are bitwise reproducible.
#include "ea_device.h"
#include "ea_launch.h"

// Tile and occupancy choices (workgroups per CU the register budget is sized for).
#ifndef EA_DQ_BK
#define EA_DQ_BK 32
#endif
#ifndef EA_DQ_MIN_WG
#define EA_DQ_MIN_WG 2
#endif
#ifndef EA_DKDV_WAVES
#define EA_DKDV_WAVES 8  // waves per dK/dV workgroup (16 keys each); 4 or 8
#endif
#ifndef EA_DKDV_BQ
#define EA_DKDV_BQ 64  // query rows per dK/dV tile; 32 or 64
#endif

namespace ea {

struct BwdParams {
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
  long q_bstride, k_bstride, row_bstride;  // elements between batches (tokens*H*D, tokens*H*D, tokens*H)
  long rs;                                 // H*D
  int H, Sq, Sk, nblk;
  Seg qs, ks;
  int causal, o_bf16;
  float scale, c;
};

// ------------------------------------------------------------------ Delta
template <int D>
__global__ __launch_bounds__(256) void delta_kernel(BwdParams p, long rows_per_batch, long total_rows) {
  constexpr int LPR = D / 8;  // lanes per row
  const long gt = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long row = gt / LPR;
  const int part = (int)(gt % LPR);
  float acc = 0.f;
  if (row < total_rows) {
    const long b = row / rows_per_batch, rem = row % rows_per_batch;
    const long off = b * p.q_bstride + rem * D + part * 8;
    const u32x4 du = *reinterpret_cast<const u32x4*>(p.dout + off);
    float ov[8];
    if (p.o_bf16) {
      const u32x4 ou = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(p.o) + off);
#pragma unroll
      for (int e = 0; e < 8; ++e) ov[e] = bf16_to_f32((uint16_t)((ou[e >> 1] >> ((e & 1) * 16)) & 0xffffu));
    } else {
      const f32x4* op = reinterpret_cast<const f32x4*>(static_cast<const float*>(p.o) + off);
      const f32x4 a = op[0], bb = op[1];
      ov[0] = a[0]; ov[1] = a[1]; ov[2] = a[2]; ov[3] = a[3];
      ov[4] = bb[0]; ov[5] = bb[1]; ov[6] = bb[2]; ov[7] = bb[3];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += bf16_to_f32((uint16_t)((du[e >> 1] >> ((e & 1) * 16)) & 0xffffu)) * ov[e];
  }
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
  if (row < total_rows && part == 0) {
    const long b = row / rows_per_batch, rem = row % rows_per_batch;
    p.delta[b * p.row_bstride + rem] = acc;
  }
}

// lse (natural log) -> base-2 units; rows without any allowed key (-inf) get
// +inf so that their recomputed probabilities are exactly 0.
__device__ __forceinline__ float lse_to_log2(float l) {
  return l == -__builtin_inff() ? __builtin_inff() : l * kLog2e;
}

// ------------------------------------------------------------------ dK, dV
// One workgroup per block of NW*16 keys; each wave owns 16 keys.  The 16x16x32
// MFMA puts the wave's 16 keys on the lane axis, so P and dS leave the score
// products as B operands of dV^T += dO^T P and dK^T += Q^T dS, and the dK^T /
// dV^T accumulators of 16 keys x D dims take D/2 registers each: two waves fit
// per SIMD.
template <int D>
struct DkdvCfg {
  static constexpr int NW = EA_DKDV_WAVES, NT = 64 * NW, BKV = 16 * NW, BQ = EA_DKDV_BQ;
  static constexpr int NQB = BQ / 16, NKK = BQ / 32;  // 16-query score blocks, 32-query reduction steps
  static constexpr int CPR = D / 8;
  static constexpr int NL = 2 * BQ * CPR / NT;  // 16-byte chunks per thread per tile (Q and dO together)
  static constexpr int LDS_T = BQ * D;
  static_assert(NL * NT == 2 * BQ * CPR && NL >= 1 && BQ % 32 == 0 && 2 * BQ <= NT, "unsupported query tile");
};

template <int D>
__global__ __launch_bounds__(64 * EA_DKDV_WAVES, 8 / EA_DKDV_WAVES) void dkdv_kernel(BwdParams p) {
  using Cfg = DkdvCfg<D>;
  constexpr int BKV = Cfg::BKV, BQ = Cfg::BQ, CPR = Cfg::CPR, NT = Cfg::NT;
  constexpr int NKS = D / 32, NDB = D / 16, NQB = Cfg::NQB, NKK = Cfg::NKK;
  __shared__ __attribute__((aligned(16))) uint16_t Qs[2][Cfg::LDS_T];
  __shared__ __attribute__((aligned(16))) uint16_t Os[2][Cfg::LDS_T];   // dO
  __shared__ __attribute__((aligned(16))) float Ls[2][BQ];
  __shared__ __attribute__((aligned(16))) float Ds[2][BQ];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform (scalar)
  const int l16 = lane & 15, g4 = lane >> 4;

  const int work = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = work / p.nblk;
  const int kb = work % p.nblk;  // lowest keys first: under the causal rule they see the most queries
  const int b = bh / p.H, h = bh % p.H;
  const int D_ = D;

  const uint16_t* qp = p.q + b * p.q_bstride + (long)h * D_;
  const uint16_t* op = p.dout + b * p.q_bstride + (long)h * D_;
  const uint16_t* kp = p.k + b * p.k_bstride + (long)h * D_;
  const uint16_t* vp = p.v + b * p.k_bstride + (long)h * D_;
  const float* lsep = p.lse + b * p.row_bstride + h;
  const float* delp = p.delta + b * p.row_bstride + h;

  const int j0 = kb * BKV;
  const int kw0 = j0 + 16 * w;
  const int krow = kw0 + l16;
  const bool key_ok = krow < p.Sk;

  // this lane's key row in MFMA B-operand form (8 dims per lane per 32-dim step)
  bf16x8 kf[NKS], vf[NKS];
  {
    const long off = (long)(key_ok ? krow : 0) * p.rs + 8 * g4;
    const u32x4* ksrc = reinterpret_cast<const u32x4*>(kp + off);
    const u32x4* vsrc = reinterpret_cast<const u32x4*>(vp + off);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      kf[ks] = as_bf16x8(key_ok ? ksrc[4 * ks] : u32x4{0u, 0u, 0u, 0u});
      vf[ks] = as_bf16x8(key_ok ? vsrc[4 * ks] : u32x4{0u, 0u, 0u, 0u});
    }
  }
  const int kpos = seg_pos(p.ks, key_ok ? krow : (p.Sk - 1));
  QueryWindow qwin = query_window(p.qs, kpos, p.causal);
  if (!key_ok) qwin = QueryWindow{0, 0, 0, 0};

  // key position ranges (workgroup and wave)
  const int wg_end = min(j0 + BKV, p.Sk);
  int kmin_wg, kmax_wg;
  seg_range(p.ks, j0, wg_end, kmin_wg, kmax_wg);
  const int kw1 = min(kw0 + 16, p.Sk);
  const bool wave_live = kw0 < kw1;
  int kmin_w = 0x7fffffff, kmax_w = 0;
  if (wave_live) seg_range(p.ks, kw0, kw1, kmin_w, kmax_w);

  // query tiles that may see this key block: per query segment, a suffix
  int a0 = 0, a1 = p.Sq, c0 = p.Sq, c1 = p.Sq;
  if (p.causal) {
    const int l0 = p.qs.l0, len1 = p.qs.n - p.qs.l0;
    long f0 = (long)kmin_wg - p.qs.s0;
    f0 = f0 < 0 ? 0 : (f0 > l0 ? l0 : f0);
    long f1 = (long)kmin_wg - p.qs.s1;
    f1 = f1 < 0 ? 0 : (f1 > len1 ? len1 : f1);
    a0 = (int)f0;
    a1 = l0;
    c0 = l0 + (int)f1;
    c1 = p.qs.n;
  }
  int tA0 = a0 / BQ, tA1 = (a1 + BQ - 1) / BQ;
  if (a1 <= a0) tA1 = tA0;
  int tC0 = c0 / BQ, tC1 = (c1 + BQ - 1) / BQ;
  if (c1 <= c0) tC1 = tC0;
  if (tC0 < tA1 && tA1 > tA0) tC0 = tA1;
  const int nA = tA1 - tA0;
  const int nC = tC1 > tC0 ? tC1 - tC0 : 0;
  const int nt = nA + nC;
  auto tile_of = [&](int t) { return t < nA ? tA0 + t : tC0 + (t - nA); };

  f32x4 dka[NDB], dva[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dka[db] = f32x4{};
    dva[db] = f32x4{};
  }

  // staging: chunk c of the tile pair (Q rows then dO rows); consecutive threads
  // take consecutive 16-byte chunks of a row
  u32x4 sreg[Cfg::NL];
  float lreg = 0.f;

  auto load_tile = [&](int it) {
    const int i0 = it * BQ;
#pragma unroll
    for (int k = 0; k < Cfg::NL; ++k) {
      const int c = tid + NT * k;
      const int tns = c / (BQ * CPR), within = c % (BQ * CPR);
      const int row = within / CPR, col = within % CPR;
      const int i = i0 + row;
      const uint16_t* src = tns ? op : qp;
      sreg[k] = i < p.Sq ? *reinterpret_cast<const u32x4*>(src + (long)i * p.rs + col * 8) : u32x4{0u, 0u, 0u, 0u};
    }
    if (tid < 2 * BQ) {
      const int i = i0 + (tid % BQ);
      if (tid < BQ)
        lreg = i < p.Sq ? lse_to_log2(lsep[(long)i * p.H]) : __builtin_inff();
      else
        lreg = i < p.Sq ? delp[(long)i * p.H] : 0.f;
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int k = 0; k < Cfg::NL; ++k) {
      const int c = tid + NT * k;
      const int tns = c / (BQ * CPR), within = c % (BQ * CPR);
      uint16_t* dst = tns ? Os[buf] : Qs[buf];
      *reinterpret_cast<u32x4*>(&dst[tile_off<D>(within / CPR, within % CPR)]) = sreg[k];
    }
    if (tid < BQ)
      Ls[buf][tid] = lreg;
    else if (tid < 2 * BQ)
      Ds[buf][tid - BQ] = lreg;
  };

  const int swq = swz<D>(l16);                 // Q/dO operand rows are 16*mb + l16
  const int trow = 4 * g4 + (l16 >> 2);        // transpose read: query row (+16 for the second half)
  const int tcol = 4 * (l16 & 3);              // transpose read: dim column within 16

  if (nt > 0) load_tile(tile_of(0));

  for (int t = 0; t < nt; ++t) {
    const int buf = t & 1;
    const int it = tile_of(t);
    const int i0 = it * BQ;
    store_tile(buf);
    __syncthreads();
    if (t + 1 < nt) load_tile(tile_of(t + 1));

    int cls = kSkip;
    if (wave_live) {
      const int iend = min(i0 + BQ, p.Sq);
      int qmn, qmx;
      seg_range(p.qs, i0, iend, qmn, qmx);
      const bool tail = (i0 + BQ > p.Sq) || (kw0 + 16 > p.Sk);
      if (!p.causal) cls = tail ? kPartial : kFull;
      else if (kmin_w > qmx) cls = kSkip;
      else if (kmax_w <= qmn && !tail) cls = kFull;
      else cls = kPartial;
    }
    if (cls == kSkip) continue;

    // S = Q K^T and dP = dO V^T for 16-query blocks; lane = key,
    // register e of block mb = query 16*mb + 4*g4 + e
    f32x4 s[NQB], dp[NQB];
#pragma unroll
    for (int mb = 0; mb < NQB; ++mb) {
      s[mb] = f32x4{};
      dp[mb] = f32x4{};
      const uint16_t* qrow = &Qs[buf][(16 * mb + l16) * D];
      const uint16_t* orow = &Os[buf][(16 * mb + l16) * D];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int o = ((4 * ks + g4) ^ swq) << 3;
        const u32x4 aq = *reinterpret_cast<const u32x4*>(qrow + o);
        s[mb] = mfma16(as_bf16x8(aq), kf[ks], s[mb]);
        const u32x4 ao = *reinterpret_cast<const u32x4*>(orow + o);
        dp[mb] = mfma16(as_bf16x8(ao), vf[ks], dp[mb]);
      }
    }

    float pv[NQB][4], dsv[NQB][4];
#pragma unroll
    for (int mb = 0; mb < NQB; ++mb) {
      const int qi = 16 * mb + 4 * g4;
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(&Ls[buf][qi]);
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(&Ds[buf][qi]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float x = fast_exp2(__builtin_fmaf(s[mb][e], p.c, -l4[e]));
        if (cls == kPartial) x = in_window(qwin, i0 + qi + e) ? x : 0.f;
        pv[mb][e] = x;
        dsv[mb][e] = x * (dp[mb][e] - d4[e]);
      }
    }

    // dV^T += dO^T P ; dK^T += Q^T dS  (reduction over 32 queries per step:
    // query blocks 2*kk and 2*kk+1; dO^T and Q^T read transposed from the
    // row-major tiles)
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const int m0 = 2 * kk, m1 = 2 * kk + 1;
      const bf16x8 pb = pack_bf16x8(pv[m0][0], pv[m0][1], pv[m0][2], pv[m0][3], pv[m1][0], pv[m1][1], pv[m1][2],
                                    pv[m1][3]);
      const bf16x8 sb = pack_bf16x8(dsv[m0][0], dsv[m0][1], dsv[m0][2], dsv[m0][3], dsv[m1][0], dsv[m1][1],
                                    dsv[m1][2], dsv[m1][3]);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int col = 16 * db + tcol;
        const int o0 = tile_off<D>(32 * kk + trow, col >> 3) + (col & 7);
        const int o1 = tile_off<D>(32 * kk + 16 + trow, col >> 3) + (col & 7);
        const u32x2 olo = ds_read_tr16(&Os[buf][o0]);
        const u32x2 ohi = ds_read_tr16(&Os[buf][o1]);
        const u32x4 ao = {olo[0], olo[1], ohi[0], ohi[1]};
        dva[db] = mfma16(as_bf16x8(ao), pb, dva[db]);
        const u32x2 qlo = ds_read_tr16(&Qs[buf][o0]);
        const u32x2 qhi = ds_read_tr16(&Qs[buf][o1]);
        const u32x4 aq = {qlo[0], qlo[1], qhi[0], qhi[1]};
        dka[db] = mfma16(as_bf16x8(aq), sb, dka[db]);
      }
    }
  }

  if (!key_ok || nt == 0) return;
  float* dkp = p.dk + b * p.k_bstride + (long)h * D_ + (long)krow * p.rs;
  float* dvp = p.dv + b * p.k_bstride + (long)h * D_ + (long)krow * p.rs;
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int d0 = 16 * db + 4 * g4;
    f32x4 k4 = *reinterpret_cast<f32x4*>(dkp + d0);
    f32x4 v4 = *reinterpret_cast<f32x4*>(dvp + d0);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      k4[e] += p.scale * dka[db][e];
      v4[e] += dva[db][e];
    }
    *reinterpret_cast<f32x4*>(dkp + d0) = k4;
    *reinterpret_cast<f32x4*>(dvp + d0) = v4;
  }
}

// ------------------------------------------------------------------ dQ
template <int D>
struct DqCfg {
  static constexpr int BQ = 128, BK = EA_DQ_BK, NT = 256;
  static constexpr int NMB = BK / 32, NKB = BK / 16;
  static constexpr int CPR = D / 8;
  static constexpr int NKL = BK * CPR / NT;  // 16-byte chunks per thread per tile (each of K and V)
  static constexpr int LDS_T = BK * D;
  static_assert(BK % 32 == 0 && NKL * NT == BK * CPR, "unsupported key tile");
};

template <int D>
__global__ __launch_bounds__(256, EA_DQ_MIN_WG) void dq_kernel(BwdParams p) {
  using Cfg = DqCfg<D>;
  constexpr int BQ = Cfg::BQ, BK = Cfg::BK, CPR = Cfg::CPR;
  constexpr int NKS = D / 16, NDB = D / 32, NMB = Cfg::NMB, NKB = Cfg::NKB;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][Cfg::LDS_T];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][Cfg::LDS_T];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform (scalar)
  const int ln = lane & 31, g = lane >> 5;

  const int work = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = work / p.nblk;
  const int qb = p.nblk - 1 - work % p.nblk;
  const int b = bh / p.H, h = bh % p.H;
  const int D_ = D;

  const uint16_t* qp = p.q + b * p.q_bstride + (long)h * D_;
  const uint16_t* op = p.dout + b * p.q_bstride + (long)h * D_;
  const uint16_t* kp = p.k + b * p.k_bstride + (long)h * D_;
  const uint16_t* vp = p.v + b * p.k_bstride + (long)h * D_;

  const int i0 = qb * BQ;
  const int qrow = i0 + 32 * w + ln;
  const bool row_ok = qrow < p.Sq;

  bf16x8 qf[NKS], of[NKS];
  {
    const long off = (long)(row_ok ? qrow : 0) * p.rs + 8 * g;
    const u32x4* qsrc = reinterpret_cast<const u32x4*>(qp + off);
    const u32x4* osrc = reinterpret_cast<const u32x4*>(op + off);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      qf[ks] = as_bf16x8(row_ok ? qsrc[2 * ks] : u32x4{0u, 0u, 0u, 0u});
      of[ks] = as_bf16x8(row_ok ? osrc[2 * ks] : u32x4{0u, 0u, 0u, 0u});
    }
  }
  const long srow = b * p.row_bstride + (long)(row_ok ? qrow : 0) * p.H + h;
  const float lse2 = row_ok ? lse_to_log2(p.lse[srow]) : __builtin_inff();
  const float dlt = row_ok ? p.delta[srow] : 0.f;
  const int qpos = seg_pos(p.qs, row_ok ? qrow : (p.Sq - 1));
  const KeyWindow kwin = key_window(p.ks, qpos, p.causal);

  const int wg_end = min(i0 + BQ, p.Sq);
  int qmin_wg, qmax_wg;
  seg_range(p.qs, i0, wg_end, qmin_wg, qmax_wg);
  const int w0 = i0 + 32 * w, w1 = min(w0 + 32, p.Sq);
  const bool wave_live = w0 < w1;
  int qmin_w = 0, qmax_w = -1;
  if (wave_live) seg_range(p.qs, w0, w1, qmin_w, qmax_w);

  int e0 = p.Sk, b1 = p.Sk, e1 = p.Sk;
  if (p.causal) causal_key_ranges(p.ks, qmax_wg, e0, b1, e1);
  const int nA = (e0 + BK - 1) / BK;
  int tB0 = b1 / BK, tB1 = (e1 + BK - 1) / BK;
  if (e1 <= b1) tB1 = tB0;
  if (tB0 < nA) tB0 = nA;
  const int nB = tB1 > tB0 ? tB1 - tB0 : 0;
  const int nt = nA + nB;
  auto tile_of = [&](int t) { return t < nA ? t : tB0 + (t - nA); };

  f32x16 dqa[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dqa[db] = f32x16{};

  // staging: consecutive threads take consecutive 16-byte chunks of a row
  u32x4 kreg[Cfg::NKL], vreg[Cfg::NKL];

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
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int it = 0; it < Cfg::NKL; ++it) {
      const int c = tid + Cfg::NT * it;
      const int o = tile_off<D>(c / CPR, c % CPR);
      *reinterpret_cast<u32x4*>(&Ks[buf][o]) = kreg[it];
      *reinterpret_cast<u32x4*>(&Vs[buf][o]) = vreg[it];
    }
  };

  const int swk = swz<D>(ln);                                  // K/V operand rows are mb*32 + ln
  const int trow = 4 * g + ((lane & 15) >> 2);                 // transpose read: row within a 16-key step
  const int tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);    // transpose read: column within 32 dims

  if (nt > 0) load_tile(tile_of(0));

  for (int t = 0; t < nt; ++t) {
    const int buf = t & 1;
    const int jt = tile_of(t);
    const int j0 = jt * BK;
    store_tile(buf);
    __syncthreads();
    if (t + 1 < nt) load_tile(tile_of(t + 1));

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
    if (cls == kSkip) continue;

    f32x16 st[NMB], dpt[NMB];
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
      st[mb] = f32x16{};
      dpt[mb] = f32x16{};
      const uint16_t* krow = &Ks[buf][(mb * 32 + ln) * D];
      const uint16_t* vrow = &Vs[buf][(mb * 32 + ln) * D];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int o = ((2 * ks + g) ^ swk) << 3;
        const u32x4 a = *reinterpret_cast<const u32x4*>(krow + o);
        st[mb] = mfma32(as_bf16x8(a), qf[ks], st[mb]);
        const u32x4 b = *reinterpret_cast<const u32x4*>(vrow + o);
        dpt[mb] = mfma32(as_bf16x8(b), of[ks], dpt[mb]);
      }
    }

    bf16x8 sb[NKB];
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float pv = fast_exp2(__builtin_fmaf(st[mb][r], p.c, -lse2));
        if (cls == kPartial) pv = in_window(kwin, j0 + mb * 32 + 8 * (r >> 2) + 4 * g + (r & 3)) ? pv : 0.f;
        st[mb][r] = pv * (dpt[mb][r] - dlt);
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int o = 8 * kk;
        sb[2 * mb + kk] = pack_bf16x8(st[mb][o], st[mb][o + 1], st[mb][o + 2], st[mb][o + 3], st[mb][o + 4],
                                      st[mb][o + 5], st[mb][o + 6], st[mb][o + 7]);
      }
    }

    // dQ^T += K^T dS^T; K^T read transposed from the row-major K tile
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int col = db * 32 + tcol;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const u32x2 lo = ds_read_tr16(&Ks[buf][tile_off<D>(kb * 16 + trow, col >> 3) + (col & 7)]);
        const u32x2 hi = ds_read_tr16(&Ks[buf][tile_off<D>(kb * 16 + 8 + trow, col >> 3) + (col & 7)]);
        const u32x4 a = {lo[0], lo[1], hi[0], hi[1]};
        dqa[db] = mfma32(as_bf16x8(a), sb[kb], dqa[db]);
      }
    }
  }

  if (!row_ok || nt == 0) return;
  float* dqp = p.dq + b * p.q_bstride + (long)h * D_ + (long)qrow * p.rs;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d0 = db * 32 + 8 * q4 + 4 * g;
      f32x4 v4 = *reinterpret_cast<f32x4*>(dqp + d0);
#pragma unroll
      for (int e = 0; e < 4; ++e) v4[e] += p.scale * dqa[db][4 * q4 + e];
      *reinterpret_cast<f32x4*>(dqp + d0) = v4;
    }
}

// ------------------------------------------------------------------ launchers
static Seg to_seg(const SegArg& s) { return Seg{s.s0, s.l0, s.s1, s.n}; }

static BwdParams make_params(const BwdArgs& a) {
  BwdParams p;
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.o = a.o;
  p.dout = a.dout;
  p.lse = a.lse;
  p.delta = a.delta;
  p.dq = a.dq;
  p.dk = a.dk;
  p.dv = a.dv;
  p.rs = (long)a.H * a.D;
  p.q_bstride = (long)a.q_batch_rows * p.rs;
  p.k_bstride = (long)a.k_batch_rows * p.rs;
  p.row_bstride = (long)a.q_batch_rows * a.H;
  p.H = a.H;
  p.Sq = a.Sq;
  p.Sk = a.Sk;
  p.qs = to_seg(a.qs);
  p.ks = to_seg(a.ks);
  p.causal = a.causal;
  p.o_bf16 = a.o_bf16;
  p.scale = a.scale;
  p.c = a.scale * kLog2e;
  p.nblk = 0;
  return p;
}

hipError_t launch_bwd_delta(const BwdArgs& a, hipStream_t stream) {
  BwdParams p = make_params(a);
  const long rows_per_batch = (long)a.Sq * a.H;
  const long total = rows_per_batch * a.B;
  if (total == 0) return hipSuccess;
  const int lpr = a.D / 8;
  const long threads = total * lpr;
  dim3 grid((unsigned)((threads + 255) / 256)), block(256);
  if (a.D == 64)
    hipLaunchKernelGGL(delta_kernel<64>, grid, block, 0, stream, p, rows_per_batch, total);
  else
    hipLaunchKernelGGL(delta_kernel<128>, grid, block, 0, stream, p, rows_per_batch, total);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv(const BwdArgs& a, hipStream_t stream) {
  BwdParams p = make_params(a);
  const int bkv = DkdvCfg<128>::BKV;
  p.nblk = (a.Sk + bkv - 1) / bkv;
  const long nwg = (long)a.B * a.H * p.nblk;
  if (nwg == 0 || a.Sq == 0) return hipSuccess;
  dim3 grid((unsigned)nwg), block(DkdvCfg<128>::NT);
  if (a.D == 64)
    hipLaunchKernelGGL(dkdv_kernel<64>, grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL(dkdv_kernel<128>, grid, block, 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t stream) {
  BwdParams p = make_params(a);
  p.nblk = (a.Sq + 127) / 128;
  const long nwg = (long)a.B * a.H * p.nblk;
  if (nwg == 0 || a.Sk == 0) return hipSuccess;
  dim3 grid((unsigned)nwg), block(256);
  if (a.D == 64)
    hipLaunchKernelGGL(dq_kernel<64>, grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL(dq_kernel<128>, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace ea
