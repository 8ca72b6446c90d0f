// Forward kernel: tiled attention with online softmax and LSE output
// (EasyContext core-technology page, hotelren.com, section 2 "Flash Attention
// optimisation": the attention matrix is never stored; key/value tiles are
// staged on chip and the softmax is accumulated tile by tile).
//
// gfx950 mapping
//  - One workgroup = 8 waves = 256 query rows of one (batch, head), one
//    workgroup (two waves per SIMD) per CU; each wave owns 32 rows.  Key/value
//    tiles of 64 rows (two 32-key blocks) stream through a ring of 4 LDS stages
//    filled by direct global->LDS loads, issued two tiles ahead.
//  - Ping-pong between the two waves of each SIMD (waves w and w + 4): each
//    tile takes a product phase (the scores of tile t and O += P V of tile t-1
//    on the matrix cores) and a softmax phase (rescale, exponentials) on the
//    vector ALU.  Between two workgroup barriers (one per tile) the first-half
//    wave runs product phase then softmax phase, the second-half wave softmax
//    phase then product phase, so each tends to issue products while the other
//    runs vector work.  A wave that issues products and vector work in turn
//    stalls its vector work behind every product that waits for the matrix
//    core; in the ping-pong one wave feeds the matrix core while the other
//    keeps the vector ALU busy.  The product phase also takes the row sums of
//    the previous tile and the row maximum of the new scores, so the softmax
//    phase is no longer than the product phase.
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

  // ---- running statistics, in base-2 units: each score s becomes
  // z = s*c - moff, moff being the row's running offset (the running maximum of
  // s*c, up to rounding), and P = exp2(z).  The offset is raised only when a
  // tile's z exceeds 8: probabilities then stay below 2^8, exactly representable
  // in the accumulation, and the rescale of O is rare.  -inf: no score yet.
  constexpr float NEG_INF = -__builtin_inff();
  constexpr float kLn2 = 0.693147180559945309f;
  // The row sum is kept as four partial sums (summed at the end) and the row
  // maximum of a tile is formed by four independent chains: each phase runs
  // alone on its SIMD's vector ALU, so its dependency chains are not hidden
  // behind another wave's work.
  float moff = NEG_INF, l_run[4] = {0.f, 0.f, 0.f, 0.f};
  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};

  // ---- direct global -> LDS loads: one instruction moves 16 bytes per lane into
  // 64 consecutive 16-byte LDS slots (RPI rows); lane i fills slot i % CPR of row
  // i / CPR, i.e. chunk (slot ^ swz(row)) of that row in the swizzled layout.
  const int dma_row = lane / CPR, dma_slot = lane % CPR;
  // byte offset of this lane's 16 bytes from the first row of a tile (a tile spans
  // BK rows of H*D elements, so it fits in 32 bits); the tile's first row is a
  // scalar base
  uint32_t dma_off[Cfg::NKL];
#pragma unroll
  for (int it = 0; it < Cfg::NKL; ++it) {
    const int row = RPI * (w + Cfg::NW * it) + dma_row;
    dma_off[it] = (uint32_t)(((long)row * p.rs + ((dma_slot ^ swz<D>(row)) << 3)) * 2);
  }
  auto load_kv = [&](auto STAGE, const uint16_t* kb, const uint16_t* vb) {
    constexpr int stage = decltype(STAGE)::value;
#pragma unroll
    for (int it = 0; it < Cfg::NKL; ++it) {
      if (Cfg::NLT < Cfg::NW && w >= Cfg::NLT) break;  // this wave loads nothing (its vmcnt waits pass at once)
      const int row0 = RPI * (w + Cfg::NW * it);
      dma16_s(kb, dma_off[it], &Ks[stage][row0 * D]);
      dma16_s(vb, dma_off[it], &Vs[stage][row0 * D]);
    }
  };
  // Any tile t (prologue, and a ragged last tile): t past the last tile reloads
  // it into a stage nobody reads; rows past the end of the keys load the last
  // key row (the element mask removes them).  Only the last tile visited, the
  // highest, can be ragged.
  auto issue_any = [&](auto STAGE, int t) {
    constexpr int stage = decltype(STAGE)::value;
    const int tt = t < nt ? t : nt - 1;
    const int j0 = __builtin_amdgcn_readfirstlane(tile_of(tt) * BK);
    const uint16_t* kb = kp + (long)j0 * p.rs;
    const uint16_t* vb = vp + (long)j0 * p.rs;
    if (j0 + BK <= p.Sk) {
      load_kv(STAGE, kb, vb);
      return;
    }
#pragma unroll
    for (int it = 0; it < Cfg::NKL; ++it) {
      if (Cfg::NLT < Cfg::NW && w >= Cfg::NLT) break;
      const int row0 = RPI * (w + Cfg::NW * it), row = row0 + dma_row;
      const int jj = min(row, p.Sk - 1 - j0);
      const uint32_t off = (uint32_t)(((long)jj * p.rs + ((dma_slot ^ swz<D>(row)) << 3)) * 2);
      dma16_s(kb, off, &Ks[stage][row0 * D]);
      dma16_s(vb, off, &Vs[stage][row0 * D]);
    }
  };
  // Tiles 2 .. nfast-1 (whole): scalar pointers to the first row of the next
  // tile, stepped up one tile per load, except once, from the last tile of the
  // first run over the causally skipped tiles to the first tile of the second.
  const int nfast = nt > 0 && tile_of(nt - 1) * BK + BK > p.Sk ? nt - 1 : nt;
  const long kstep = (long)BK * p.rs, kjump = (long)(tB0 - nA + 1) * BK * p.rs;
  const uint16_t* nk = kp;
  const uint16_t* nv = vp;
  {
    const int r2 = __builtin_amdgcn_readfirstlane(tile_of(2 < nt ? 2 : 0) * BK);
    nk += (long)r2 * p.rs;
    nv += (long)r2 * p.rs;
  }
  auto issue_next = [&](auto STAGE, int m) {  // loads tile m + 2 (>= 2, < nfast), then points at tile m + 3
    load_kv(STAGE, nk, nv);
    const long st = m + 3 == nA ? kjump : kstep;
    nk += st;
    nv += st;
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

  // The compiler may move pure arithmetic across a barrier (it moved exponentials
  // of a softmax phase into the next product phase, where their results are
  // used); an empty asm statement that takes a phase's results as in-out
  // operands keeps their computation before the phase's closing barrier.
  auto pin_phase_outputs = [](f32x16 (&s16)[NMB], f32x16 (&o16)[NDB]) {
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) asm volatile("" : "+v"(s16[mb]));
#pragma unroll
    for (int db = 0; db < NDB; ++db) asm volatile("" : "+v"(o16[db]));
  };
  f32x16 st[NMB];         // S^T of the tile between its product phase and its softmax phase
  bf16x8 pb[2 * NMB];     // P^T as B operands, one per 16-key k-step, until the next product phase
  float ep[16 * NMB];     // the same probabilities in fp32, added to the row sums in the next product phase
  float mx_t = NEG_INF;   // row maximum of the tile's z, formed in its product phase
#pragma unroll
  for (int kk = 0; kk < 2 * NMB; ++kk) pb[kk] = bf16x8{};
#pragma unroll
  for (int r = 0; r < 16 * NMB; ++r) ep[r] = 0.f;

  // row maximum of st (both halves of the wave): four independent chains, then
  // the lane swap
  auto row_max = [&]() {
    float m4[4] = {NEG_INF, NEG_INF, NEG_INF, NEG_INF};
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) m4[(r >> 1) & 3] = fmaxf(fmaxf(m4[(r >> 1) & 3], st[mb][r]), st[mb][r + 1]);
    return xor32_max(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])));
  };

  // Product phase of tile t: S^T(t) = K(t) Q^T from stage KSTAGE, then
  // O^T += V^T(t-1) P^T(t-1) from stage VSTAGE (V^T read transposed from the
  // row-major V tile).  No product waits for vector-ALU work.  The first phase
  // (t = 0) adds P = 0 times the resident tile 0; the last (t = nt) computes the
  // scores of a stage holding no new tile and drops them, so every phase is the same
  // straight run of products.  Their operands go through a register ring PF
  // products deep, pinned by scheduling groups (left to itself the compiler read
  // each K operand right before its product and waited for it).  Between the
  // products the wave adds the previous tile's probabilities to its row sums and,
  // once the scores have landed, turns them into z = s*c - moff and forms their
  // row maximum: vector work that would otherwise lengthen the softmax phase,
  // which runs alone on its vector ALU.
  auto m_phase = [&](auto KSTAGE, auto VSTAGE) {
    constexpr int kstage = decltype(KSTAGE)::value, vstage = decltype(VSTAGE)::value;
    constexpr int NS = NKS * NMB, NPV = 2 * NMB * NDB, N = NS + NPV, PF = 3;
    __builtin_amdgcn_s_setprio(2);  // the products win the issue port from the other wave's vector work
    constexpr int ADD_PER = (16 * NMB + NS - 1) / NS;     // row-sum adds per score product
    constexpr int MAX_PER = (56 + NPV - 3) / (NPV - 2);  // z and row-maximum work per O product (after the first two)
    static_assert(PF <= NS, "the ring starts inside the score products");
    auto rd = [&](int i) {
      if (i < NS) {  // K operand of score product i (k-step major)
        const int ks = i / NMB, mb = i % NMB;
        return *reinterpret_cast<const u32x4*>(&Ks[kstage][mb * 32 * D + kbase + ((ks ^ kx) << 4)]);
      }
      const int kk = (i - NS) / NDB, db = (i - NS) % NDB;  // V^T operand of O product i - NS
      const u32x2 lo = ds_read_tr16(&Vs[vstage][vofs[0][db] + 16 * kk * D]);
      const u32x2 hi = ds_read_tr16(&Vs[vstage][vofs[1][db] + 16 * kk * D]);
      return u32x4{lo[0], lo[1], hi[0], hi[1]};
    };
    u32x4 fr[N];
#pragma unroll
    for (int i = 0; i < PF; ++i) fr[i] = rd(i);
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) st[mb] = f32x16{};
#pragma unroll
    for (int i = 0; i < N; ++i) {
      if (i + PF < N) fr[i + PF] = rd(i + PF);
      if (i < NS) {
        st[i % NMB] = mfma32(as_bf16x8(fr[i]), qf[i / NMB], st[i % NMB]);
      } else {
        const int j = i - NS;
        oacc[j % NDB] = mfma32(as_bf16x8(fr[i]), pb[j / NDB], oacc[j % NDB]);
      }
    }
#pragma unroll
    for (int r = 0; r < 16 * NMB; ++r) l_run[r & 3] += ep[r];
    const float msub = moff == NEG_INF ? 0.f : moff;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) st[mb][r] = __builtin_fmaf(st[mb][r], p.c, -msub);
    mx_t = row_max();
    __builtin_amdgcn_sched_group_barrier(0x100, PF, 0);  // operands of the first PF products
#pragma unroll
    for (int i = 0; i < N; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // product i
      if (i + PF < NS) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // the read of score product i + PF
      } else if (i + PF < N) {
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // the two reads of O product i + PF - NS
      }
      if (i < NS) {
        __builtin_amdgcn_sched_group_barrier(0x002, ADD_PER, 0);  // row-sum adds
      } else if (i >= NS + 2) {
        __builtin_amdgcn_sched_group_barrier(0x002, MAX_PER, 0);  // z and row maximum of the new scores
      }
    }
    pin_phase_outputs(st, oacc);
    asm volatile("" : "+v"(mx_t), "+v"(l_run[0]), "+v"(l_run[1]), "+v"(l_run[2]), "+v"(l_run[3]));
    __builtin_amdgcn_s_setprio(0);
  };

  // Softmax phase of tile t: mask (the maximum is then formed again), raise of
  // the offset (rare), exponentials, P^T packed to bf16.
  auto v_phase = [&](int t) {
    const int j0 = tile_of(t) * BK;
    float mx = mx_t;
    if (classify(t) == kPartial) {
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = j0 + 32 * mb + 8 * (r >> 2) + 4 * g + (r & 3);
          st[mb][r] = in_window(kwin, j) ? st[mb][r] : NEG_INF;
        }
      mx = row_max();
    }
    // raise when some z exceeds 8, or on a row's first finite scores (its z are
    // then s*c, unshifted); every row of the wave takes the larger of its offset
    // and its maximum
    if (__any(mx > (moff == NEG_INF ? NEG_INF : 8.f))) {
      const float shift = moff == NEG_INF ? (mx == NEG_INF ? 0.f : mx) : fmaxf(mx, 0.f);
      const float alpha = moff == NEG_INF ? 0.f : fast_exp2(-shift);
#pragma unroll
      for (int i = 0; i < 4; ++i) l_run[i] *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) st[mb] -= shift;
      moff = moff == NEG_INF ? (mx == NEG_INF ? NEG_INF : mx) : moff + shift;
    }
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
      float* e = ep + 16 * mb;
#pragma unroll
      for (int r = 0; r < 16; ++r) e[r] = fast_exp2(st[mb][r]);
      pb[2 * mb] = pack_bf16x8(e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]);
      pb[2 * mb + 1] = pack_bf16x8(e[8], e[9], e[10], e[11], e[12], e[13], e[14], e[15]);
    }
#pragma unroll
    for (int kk = 0; kk < 2 * NMB; ++kk) asm volatile("" : "+v"(pb[kk]));
#pragma unroll
    for (int r = 0; r < 16 * NMB; ++r) asm volatile("" : "+v"(ep[r]));
    asm volatile("" : "+v"(l_run[0]), "+v"(l_run[1]), "+v"(l_run[2]), "+v"(l_run[3]), "+v"(moff));
    pin_phase_outputs(st, oacc);
  };

  // Step boundaries.  Step m starts once tile m is resident for every wave (each
  // wave waits for its own loads of it, then the barrier), after which the load
  // of tile m+2 goes out into the stage tile m-2 held: its last readers (the O
  // products of tile m-2) ran in step m-1.  The scheduling walls keep every
  // instruction in its phase.
  // Near the end (and before a ragged last tile) the wave waits for all of its loads.
  auto sync_even = [&](auto STAGE2, int m) {
    __builtin_amdgcn_sched_barrier(0);
    if (m + 2 < nfast) {
      lds_ring_sync<LOADS_PER_TILE>();
      issue_next(STAGE2, m);
    } else {
      lds_ring_sync<0>();
      if (m + 2 < nt) issue_any(STAGE2, m + 2);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  if (nt > 0) {
    static_assert(NST == 4, "the phase schedule below is written for a ring of 4 stages");
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    using S3 = std::integral_constant<int, 3>;
    issue_any(S0{}, 0);
    issue_any(S1{}, 1);
    sync_even(S2{}, 0);
    // Ping-pong: waves w and w + NW/2 share a SIMD.  In step t the first half
    // runs the product phase of tile t, then its softmax; the second half runs
    // the softmax of tile t-1, then the product phase of tile t.  So one wave of
    // each SIMD tends to issue products while the other runs vector work, and the
    // product phase's issue priority keeps the matrix core fed where they
    // overlap.  (A second barrier per tile that forced the phases apart cost
    // more in waiting than it gained.)  Both halves pass the same nt + 1
    // barriers.
    if (w < Cfg::NW / 2) {
      __builtin_amdgcn_sched_barrier(0);
      m_phase(S0{}, S0{});
      for (int t0 = 0;; t0 += 4) {
        v_phase(t0);
        __builtin_amdgcn_sched_barrier(0);
        sync_even(S3{}, t0 + 1);
        __builtin_amdgcn_sched_barrier(0);
        m_phase(S1{}, S0{});
        if (t0 + 1 == nt) break;
        v_phase(t0 + 1);
        __builtin_amdgcn_sched_barrier(0);
        sync_even(S0{}, t0 + 2);
        __builtin_amdgcn_sched_barrier(0);
        m_phase(S2{}, S1{});
        if (t0 + 2 == nt) break;
        v_phase(t0 + 2);
        __builtin_amdgcn_sched_barrier(0);
        sync_even(S1{}, t0 + 3);
        __builtin_amdgcn_sched_barrier(0);
        m_phase(S3{}, S2{});
        if (t0 + 3 == nt) break;
        v_phase(t0 + 3);
        __builtin_amdgcn_sched_barrier(0);
        sync_even(S2{}, t0 + 4);
        __builtin_amdgcn_sched_barrier(0);
        m_phase(S0{}, S3{});
        if (t0 + 4 == nt) break;
      }
    } else {
      __builtin_amdgcn_sched_barrier(0);
      m_phase(S0{}, S0{});
      for (int t0 = 0;; t0 += 4) {
        sync_even(S3{}, t0 + 1);
        v_phase(t0);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_sched_barrier(0);
        m_phase(S1{}, S0{});
        if (t0 + 1 == nt) break;
        sync_even(S0{}, t0 + 2);
        v_phase(t0 + 1);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_sched_barrier(0);
        m_phase(S2{}, S1{});
        if (t0 + 2 == nt) break;
        sync_even(S1{}, t0 + 3);
        v_phase(t0 + 2);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_sched_barrier(0);
        m_phase(S3{}, S2{});
        if (t0 + 3 == nt) break;
        sync_even(S2{}, t0 + 4);
        v_phase(t0 + 3);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_sched_barrier(0);
        m_phase(S0{}, S3{});
        if (t0 + 4 == nt) break;
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // retire the trailing (unused) loads
  }

  // ---- epilogue: normalise, write O and LSE
  const float l1 = (l_run[0] + l_run[1]) + (l_run[2] + l_run[3]);
  const float lt = l1 + __shfl_xor(l1, 32);
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
    const float l2 = has ? (moff * kLn2 + logf(lt)) : NEG_INF;
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
    const float lse = has ? (moff * kLn2 + logf(lt)) : NEG_INF;
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
