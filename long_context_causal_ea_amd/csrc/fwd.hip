// Forward kernel: tiled attention with online softmax and LSE output
// (EasyContext core-technology page, hotelren.com, section 2 "Flash Attention
// optimisation": the attention matrix is never stored; key/value tiles are
// staged on chip and the softmax is accumulated tile by tile).
//
// gfx950 mapping
//  - One workgroup = 8 waves = 256 query rows of one (batch, head), one
//    workgroup (two waves per SIMD) per CU; each wave owns 32 rows.  Key/value
//    tiles of 64 rows (two 32-key blocks) stream through a ring of LDS stages
//    filled by direct global->LDS loads, three tiles in flight, so one barrier
//    covers 32 matrix-core products per wave.
//  - The loop is software-pipelined: each step first issues the scores of tile
//    t+1 to the matrix cores, then runs the softmax of tile t (row maximum,
//    rescale, exponentials) on the vector ALUs while they execute.
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
//  - With a rotary base, each lane turns its query row in registers right
//    after loading it (dims k and k + D/2 are in the same lane) and can write
//    the turned row out for the backward; keys arrive already turned.
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
  int causal, o_bf16, merge;
  float scale, c;  // c = scale * log2(e)
  int rope;        // 1: turn the q rows by their rotary angles after loading them
  uint16_t* q_rot; // when rope: the turned rows are also written here (may be null)
  double f[64];    // rotary frequencies theta^(-2k/D), k < D/2
};

#ifndef EA_FWD_NW
#define EA_FWD_NW 8  // waves per workgroup (32 query rows each)
#endif
#ifndef EA_FWD_NMB
#define EA_FWD_NMB 2  // 32-key blocks per key/value tile
#endif
#ifndef EA_FWD_NST
#define EA_FWD_NST 4  // LDS stages of the key/value ring (tiles in flight: NST - 1)
#endif

template <int D>
struct FwdCfg {
  static constexpr int NW = EA_FWD_NW, NMB = EA_FWD_NMB, BQ = 32 * NW, BK = 32 * NMB, NT = 64 * NW;
  static constexpr int NST = EA_FWD_NST;
  static constexpr int CPR = D / 8;                   // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;                // rows one wave covers per direct-to-LDS load
  static constexpr int NLT = BK / RPI;                // direct-to-LDS loads per tile (each of K and V)
  static constexpr int NKL = (NLT + NW - 1) / NW;     // per wave (waves w + NW*i < NLT take part)
  static constexpr int LDS_T = BK * D;
  static constexpr int MIN_WG = NW >= 8 ? 1 : 2;      // workgroups per CU (two waves per SIMD)
  static_assert(NLT * RPI == BK && (NLT % NW == 0 || NLT < NW), "unsupported key tile");
};

// Rows of a key/value tile that lie past the end of the keys load the last key
// row instead (so every address is valid); the score mask removes them.
template <int D>
__global__ __launch_bounds__(64 * EA_FWD_NW, FwdCfg<128>::MIN_WG) void fwd_kernel(FwdParams p) {
  using Cfg = FwdCfg<D>;
  constexpr int BQ = Cfg::BQ, BK = Cfg::BK, CPR = Cfg::CPR, NST = Cfg::NST, RPI = Cfg::RPI, NMB = Cfg::NMB;
  constexpr int NKS = D / 16, NDB = D / 32;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[NST][Cfg::LDS_T];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[NST][Cfg::LDS_T];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform (scalar)
  const int ln = lane & 31, g = lane >> 5;

  // ---- work item: (batch*head) major, longest query blocks first
  const int work = xcd_remap(blockIdx.x, gridDim.x, p.nqb);
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
    // land the Q rows before the direct-to-LDS ring starts: the compiler cannot
    // see those loads and would otherwise wait for all of them at each use of Q
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) asm volatile("" : "+v"(qf[ks]));
  }
  const int qpos = seg_pos(p.qs, row_ok ? qrow : (p.Sq - 1));
  if (p.rope) {
    // rotary embedding of the row in registers: qf[ks] holds dims 16*ks + 8*g + e, and dims k and k + D/2
    // are packs ks and ks + NKS/2 of the same lane
#pragma unroll
    for (int ks = 0; ks < NKS / 2; ++ks) {
      const u32x4 ul = __builtin_bit_cast(u32x4, qf[ks]), uh = __builtin_bit_cast(u32x4, qf[ks + NKS / 2]);
      float lo[8], hi[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        lo[e] = __uint_as_float((e & 1) ? (ul[e >> 1] & 0xffff0000u) : (ul[e >> 1] << 16));
        hi[e] = __uint_as_float((e & 1) ? (uh[e >> 1] & 0xffff0000u) : (uh[e >> 1] << 16));
        rope_turn(lo[e], hi[e], rope_cos_sin(qpos, p.f[16 * ks + 8 * g + e]), false);
      }
      qf[ks] = pack_bf16x8(lo[0], lo[1], lo[2], lo[3], lo[4], lo[5], lo[6], lo[7]);
      qf[ks + NKS / 2] = pack_bf16x8(hi[0], hi[1], hi[2], hi[3], hi[4], hi[5], hi[6], hi[7]);
    }
    if (p.q_rot != nullptr && row_ok) {  // the turned rows for the backward
      u32x4* dst = reinterpret_cast<u32x4*>(p.q_rot + b * p.q_bstride + (long)h * D_ + (long)qrow * p.rs + 8 * g);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) dst[2 * ks] = __builtin_bit_cast(u32x4, qf[ks]);
    }
  }
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
  auto tile_of = [&](int t) { return t < nA ? t : tB0 + (t - nA); };

  // ---- running statistics (raw-score units for the max)
  constexpr float NEG_INF = -__builtin_inff();
  // The running maximum is raised only when a tile's maximum exceeds it by more
  // than 8 (in log2 units): probabilities then stay below 2^8, exactly
  // representable in the accumulation, and the rescale of O is rare.
  const float raise_thr = 8.f / p.c;
  float m_run = NEG_INF, l_run = 0.f;
  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};

  // ---- direct global -> LDS loads: one instruction moves 16 bytes per lane into
  // 64 consecutive 16-byte LDS slots (RPI rows); lane i fills slot i % CPR of row
  // i / CPR, i.e. chunk (slot ^ swz(row)) of that row in the swizzled layout.
  const int dma_row = lane / CPR, dma_slot = lane % CPR;
  long dma_off[Cfg::NKL];  // element offset of this lane's 16 bytes within a tile whose first row is 0
#pragma unroll
  for (int it = 0; it < Cfg::NKL; ++it) {
    const int row = RPI * (w + Cfg::NW * it) + dma_row;
    dma_off[it] = (long)row * p.rs + ((dma_slot ^ swz<D>(row)) << 3);
  }
  auto issue_tile = [&](auto STAGE, int t) {
    constexpr int stage = decltype(STAGE)::value;
    const int tt = t < nt ? t : nt - 1;  // past the end: reload the last tile into a stage nobody reads
    const int j0 = tile_of(tt) * BK;
    const bool whole = j0 + BK <= p.Sk;
#pragma unroll
    for (int it = 0; it < Cfg::NKL; ++it) {
      if (Cfg::NLT < Cfg::NW && w >= Cfg::NLT) break;  // this wave loads nothing (its vmcnt waits pass at once)
      const int row0 = RPI * (w + Cfg::NW * it);
      long off = (long)j0 * p.rs + dma_off[it];
      if (!whole) {
        const int row = row0 + dma_row;
        const int j = min(j0 + row, p.Sk - 1);
        off = (long)j * p.rs + ((dma_slot ^ swz<D>(row)) << 3);
      }
      dma16(kp + off, &Ks[stage][row0 * D]);
      dma16(vp + off, &Vs[stage][row0 * D]);
    }
  };
  constexpr int LOADS_PER_TILE = 2 * Cfg::NKL;

  // per-lane LDS offsets (elements), fixed for the whole kernel
  // K operand: row ln (+32 per key block), chunk 2*ks+g, i.e. slot (2*ks+g) ^ swz(ln) = 2*(ks ^ kx) + kg
  const int kx = swz<D>(ln) >> 1, kbase = ln * D + ((g ^ (swz<D>(ln) & 1)) << 3);
  int vofs[2][NDB];  // V^T transpose read: rows 8*half + trow (+16 per k-step), 32 dims per block
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

  // wave-level class of tile t: FULL (no mask needed) or PARTIAL (element mask).
  // A tile with no allowed pair for this wave is computed as PARTIAL (all of it
  // masked): that keeps the loop one straight pipeline, and such tiles are the
  // few past each wave's diagonal.
  auto classify = [&](int t) {
    const int j0 = tile_of(t) * BK;
    if (!wave_live || j0 + BK > p.Sk) return (int)kPartial;
    if (!p.causal) return (int)kFull;
    int kmn, kmx;
    seg_range(p.ks, j0, j0 + BK, kmn, kmx);
    return kmx <= qmin_w ? (int)kFull : (int)kPartial;
  };

  // S^T = K Q^T of the tile in stage STAGE, one 32-key block per output;
  // register r of block mb holds key 32*mb + 8*(r/4) + 4*g + r%4 of query ln
  auto scores = [&](auto STAGE, f32x16 (&st)[NMB]) {
    constexpr int stage = decltype(STAGE)::value;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
      st[mb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(&Ks[stage][mb * 32 * D + kbase + ((ks ^ kx) << 4)]);
        st[mb] = mfma32(as_bf16x8(a), qf[ks], st[mb]);
      }
    }
  };

  using I0 = std::integral_constant<int, 0>;

  // one pipeline step: the scores of tile t+1 (into st_next, stage STAGE+1), then
  // the softmax and P V of tile t (scores in st_cur, stage STAGE)
  auto step = [&](auto STAGE, int t, f32x16 (&st_cur)[NMB], int& cls_cur, f32x16 (&st_next)[NMB], int& cls_next) {
    constexpr int stage = decltype(STAGE)::value;
    constexpr int nstage = (stage + 1) % NST, fstage = (stage + NST - 1) % NST;
    // tile t+1 resident for every wave; everyone is done with stage (t-1) % NST
    lds_ring_sync<(NST - 3) * LOADS_PER_TILE>();
    issue_tile(std::integral_constant<int, fstage>{}, t + NST - 1);
    const int j0 = tile_of(t) * BK;
    const bool has_next = t + 1 < nt;
    cls_next = has_next ? classify(t + 1) : (int)kFull;

    if (cls_cur == kPartial) {
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = j0 + 32 * mb + 8 * (r >> 2) + 4 * g + (r & 3);
          st_cur[mb][r] = in_window(kwin, j) ? st_cur[mb][r] : NEG_INF;
        }
    }
    // The scores of tile t+1 go to the matrix cores first: they do not depend on
    // the softmax of tile t, so its maximum, rescale and exponentials (vector
    // ALUs) run while they execute.  On the last tile the scores of a dummy tile
    // are computed and dropped.
    scores(std::integral_constant<int, nstage>{}, st_next);
    float mx = NEG_INF;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st_cur[mb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    if (__any(mx > m_run + raise_thr)) {
      const float mnew = fmaxf(m_run, mx);
      const float alpha = (m_run == NEG_INF) ? 0.f : fast_exp2((m_run - mnew) * p.c);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
      m_run = mnew;
    }

    const float msub = (m_run == NEG_INF) ? 0.f : m_run * p.c;
    bf16x8 pb[2 * NMB];  // P^T as B operands, one per 16-key k-step
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
      float e[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        e[r] = fast_exp2(__builtin_fmaf(st_cur[mb][r], p.c, -msub));
        l_run += e[r];
      }
      pb[2 * mb] = pack_bf16x8(e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]);
      pb[2 * mb + 1] = pack_bf16x8(e[8], e[9], e[10], e[11], e[12], e[13], e[14], e[15]);
    }
    // O^T += V^T P^T; V^T read transposed from the row-major V tile.  Key steps outermost, so the first
    // products need only the first packs of P (each accumulator still adds the key steps in order)
#pragma unroll
    for (int kk = 0; kk < 2 * NMB; ++kk)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const u32x2 lo = ds_read_tr16(&Vs[stage][vofs[0][db] + 16 * kk * D]);
        const u32x2 hi = ds_read_tr16(&Vs[stage][vofs[1][db] + 16 * kk * D]);
        const u32x4 a = {lo[0], lo[1], hi[0], hi[1]};
        oacc[db] = mfma32(as_bf16x8(a), pb[kk], oacc[db]);
      }
  };

  if (nt > 0) {
    // prologue: NST-1 tiles in flight, scores of tile 0
    static_assert(NST == 4, "the loop below is unrolled for a ring of 4 stages");
    issue_tile(std::integral_constant<int, 0>{}, 0);
    issue_tile(std::integral_constant<int, 1>{}, 1);
    issue_tile(std::integral_constant<int, 2>{}, 2);
    lds_ring_sync<(NST - 2) * LOADS_PER_TILE>();
    int cls_a = classify(0), cls_b = kFull;
    f32x16 st_a[NMB], st_b[NMB];
    scores(I0{}, st_a);

    // unrolled by the ring size so that every stage index is a constant and the
    // two score buffers alternate without copies
    for (int t = 0; t < nt; t += 4) {
      step(std::integral_constant<int, 0>{}, t, st_a, cls_a, st_b, cls_b);
      if (t + 1 >= nt) break;
      step(std::integral_constant<int, 1>{}, t + 1, st_b, cls_b, st_a, cls_a);
      if (t + 2 >= nt) break;
      step(std::integral_constant<int, 2>{}, t + 2, st_a, cls_a, st_b, cls_b);
      if (t + 3 >= nt) break;
      step(std::integral_constant<int, 3>{}, t + 3, st_b, cls_b, st_a, cls_a);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // retire the trailing (unused) loads
  }

  // ---- epilogue: normalise, write O and LSE
  const float lt = l_run + __shfl_xor(l_run, 32);
  if (!row_ok) return;
  const bool has = lt > 0.f;
  const float inv = has ? 1.f / lt : 0.f;
  const long lse_at = b * p.lse_bstride + (long)qrow * p.H + h;
  if (p.merge) {
    // merge this partial (O = oacc / lt, LSE) into the fp32 accumulator (o, lse):
    // the log-sum-exp of the two LSEs and the LSE-weighted sum of the two Os,
    // a side at -inf contributing nothing (the same arithmetic as merge_kernel)
    float* op = static_cast<float*>(p.o) + b * p.q_bstride + (long)h * D_ + (long)qrow * p.rs;
    const float l1 = p.lse[lse_at];
    const float l2 = has ? (m_run * p.scale + logf(lt)) : NEG_INF;
    const float mx = fmaxf(l1, l2), mn = fminf(l1, l2);
    const float L = (mx == NEG_INF) ? NEG_INF : mx + log1pf(expf(mn - mx));
    const float w1 = (L == NEG_INF) ? 0.f : expf(l1 - L);
    const float w2 = (L == NEG_INF) ? 0.f : expf(l2 - L);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = db * 32 + 8 * q4 + 4 * g;
        f32x4 acc = *reinterpret_cast<const f32x4*>(op + d0);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = w1 * acc[e] + w2 * (oacc[db][4 * q4 + e] * inv);
        *reinterpret_cast<f32x4*>(op + d0) = acc;
      }
    if (g == 0) p.lse[lse_at] = L;
    return;
  }
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
    p.lse[lse_at] = lse;
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
  p.merge = a.merge;
  p.scale = a.scale;
  p.c = a.scale * kLog2e;
  p.rope = a.rope;
  p.q_rot = a.rope ? a.q_rot : nullptr;
  for (int k = 0; k < 64; ++k) p.f[k] = a.rope && k < a.D / 2 ? a.inv_freq[k] : 0.0;
  const int BQ = FwdCfg<128>::BQ;
  p.nqb = (a.Sq + BQ - 1) / BQ;
  const long nwg = (long)a.B * a.H * p.nqb;
  if (nwg == 0) return hipSuccess;
  dim3 grid((unsigned)nwg), block(FwdCfg<128>::NT);
  if (a.D == 64)
    hipLaunchKernelGGL(fwd_kernel<64>, grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL(fwd_kernel<128>, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace ea
