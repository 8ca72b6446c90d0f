// Backward kernels: recompute-from-LSE gradient of tiled attention
// (EasyContext core-technology page, hotelren.com, section 2 "Flash Attention
// optimisation": recomputation replaces the stored attention matrix).
//
// Three launches on one stream:
//  1. delta:  Delta_i = <dO_i, O_i>, one pass over O and dO (HBM-bound).
//  2. dkdv:   one workgroup per 128-key block: 8 waves, two per SIMD, in pairs
//             sharing 32 keys (one wave holds K and produces P and dV, the
//             other holds V and produces dS and dK; P crosses over in LDS);
//             the pair alternates product and vector phases (ping-pong).
//             32-row query tiles (Q, dO, LSE, Delta) stream through a
//             direct-to-LDS ring.  Scores are computed with the key on the MFMA
//             column (lane) axis, so P and dS come out of the MFMA already in
//             the B-operand form that dV^T += dO^T P and dK^T += Q^T dS need;
//             the dO^T and Q^T operands are read from the row-major tiles with
//             the LDS transpose read.
//  3. dq:     one workgroup (8 waves, two per SIMD) per 256-query block, streaming key/value tiles
//             through a direct-to-LDS ring like the forward; recomputes S^T and
//             dP^T with the query on the lane axis and accumulates
//             dQ^T += K^T dS^T in registers (K^T by transpose read of the
//             row-major K tile).  Like the forward it runs a ping-pong between
//             the two waves of each SIMD: product and arithmetic phases in
//             opposite orders between the workgroup barriers.
// All LDS tiles are row-major with the XOR chunk swizzle of ea_device.h.
// The dq pass recomputes the two score products instead of exchanging dS
// through atomics (fp32 atomic adds into L2 were measured at about 1.4 TB/s on
// MI355X, far too slow for the hundreds of GB of partial dQ a fused pass would
// add): every output element is then written by exactly one workgroup and
// results are bitwise reproducible.
#include <type_traits>

#include "ea_device.h"
#include "ea_launch.h"

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
  long rs;                                 // Hs*D
  int H, Hs, Sq, Sk, nblk;                 // heads in this launch, heads per token row
  Seg qs, ks;
  int causal, o_bf16;
  float scale, c;
  int rope;       // 1: q and k are rotated rows; dq and dk are turned back before they are added
  double f[64];   // rotary frequencies theta^(-2k/D), k < D/2 (when rope)
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

// Turn an MFMA accumulator over dims (acc[db] holds dims 32*db + 8*(r/4) +
// 4*g + r%4 of one row, the row being the lane's query or key at position pos)
// back by the rotary angle of that position: dims k and k + D/2 sit in blocks
// db and db + NDB/2 of the same lane and register.
template <int NDB>
__device__ __forceinline__ void rope_back(f32x16 (&acc)[NDB], int pos, const double* f, int g) {
#pragma unroll
  for (int db = 0; db < NDB / 2; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int k = 32 * db + 8 * (r >> 2) + 4 * g + (r & 3);
      float lo = acc[db][r], hi = acc[db + NDB / 2][r];
      rope_turn(lo, hi, rope_cos_sin(pos, f[k]), true);
      acc[db][r] = lo;
      acc[db + NDB / 2][r] = hi;
    }
}

// ------------------------------------------------------------------ dK, dV
// One workgroup = 8 waves = 128 keys of one (batch, head), two waves per SIMD.
// The 32 keys of key group kw (0..3) are shared by a pair of waves:
//   wave kw     (role A) holds the keys' K rows, computes S = Q K^T, the
//               probabilities P = exp2(S*c - LSE*log2 e) (element mask on
//               partial tiles) and dV^T += dO^T P;
//   wave 4 + kw (role B) holds the V rows, computes dP = dO V^T, takes P of the
//               same keys from A through LDS, forms dS = P (dP - Delta) and
//               accumulates dK^T += Q^T dS.
// Each wave thus needs one operand tensor and one accumulator (32 keys x D fp32)
// in registers, which leaves room for two waves per SIMD.  Scores use the
// 32x32x16 MFMA with the key on the lane axis, so P and dS leave the MFMA in
// the B-operand form of the dV / dK products; dO^T and Q^T are read from the
// row-major tiles by the LDS transpose read.
//
// P crosses from A to B through LDS as fp16 pairs (round to nearest even):
// half the bytes of an fp32 hand-over.  Over long key ranges P is tiny (about
// 1e-6 for a near-uniform row over 700K keys), below fp16's smallest normal
// value, where only a few significant bits would survive; so both roles work
// with P * 2^kPScaleLog2 (the exponent offset is folded into the base-2 LSE,
// no extra arithmetic), which keeps every P >= 3.7e-9 normal in fp16 with 11
// significant bits, and the epilogue multiplies the accumulators by the exact
// inverse power of two.
//
// 32-row query tiles (Q, dO, LSE, Delta) stream through a 6-stage LDS ring of
// direct global->LDS loads, issued four tiles ahead.  The two waves of a SIMD
// (A and B of one key group) run a ping-pong: in step t A issues the products
// of tile t (S(t), dV += dO(t-1)^T P(t-1)), then turns S(t) into P(t) and hands
// it to B; B forms dS(t-1), then issues its products (dP(t),
// dK += Q(t-1)^T dS(t-1)).  One workgroup barrier per step orders both the ring
// and the hand-over.  Each role runs its own copy of the loop so that its
// accumulator stays in the same registers.
// The dK/dV pass works with P * 2^kPScaleLog2 (see the fp16 hand-over below).
constexpr int kPScaleLog2 = 14;

template <int D>
struct DkdvCfg {
  static constexpr int NW = 8, NT = 512, BKV = 128, BQ = 32, NST = 6;
  static constexpr int CPR = D / 8;                  // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;               // rows one direct-to-LDS load covers
  static constexpr int NI = 2 * BQ / RPI;            // loads per tile (Q and dO)
  static constexpr int NIW = NI / NW;                // loads per wave per tile
  static constexpr int LDS_T = BQ * D;
  static_assert(NIW >= 1 && NIW * NW == NI, "unsupported query tile");
};

template <int D>
__global__ __launch_bounds__(512, 1) void dkdv_kernel(BwdParams p) {
  using Cfg = DkdvCfg<D>;
  constexpr int BKV = Cfg::BKV, BQ = Cfg::BQ, CPR = Cfg::CPR, NST = Cfg::NST, RPI = Cfg::RPI;
  constexpr int NKS = D / 16, NDB = D / 32;
  constexpr int OT = Cfg::LDS_T;
  // stage s: Q tile at QO[s][0], dO tile at QO[s][OT]
  __shared__ __attribute__((aligned(16))) uint16_t QO[NST][2 * OT];
  // LSE of the rows, then Delta.  The largest alignment places it first in LDS,
  // so its accesses take the 16-bit immediate offset of the LDS instructions
  // (behind the 112 KB of tiles each access needed an address add: 0.6 ms of
  // the pass at 64K tokens)
  __shared__ __attribute__((aligned(1024))) float Ss[NST][2 * BQ];
  // P of the last two tiles per key group, fp16 pairs: [slot][group][half of the 16 values][lane][pair]
  __shared__ __attribute__((aligned(16))) uint32_t Ps[2][4][2][64][4];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform (scalar)
  const int role = w >> 2, kw = w & 3;
  const int ln = lane & 31, g = lane >> 5;

  const int work = xcd_remap(blockIdx.x, gridDim.x, p.nblk);
  const int bh = work / p.nblk;
  const int kb = work % p.nblk;  // lowest keys first: under the causal rule they see the most queries
  const int b = bh / p.H, h = bh % p.H;
  const int D_ = D;

  const uint16_t* qp = p.q + b * p.q_bstride + (long)h * D_;
  const uint16_t* op = p.dout + b * p.q_bstride + (long)h * D_;
  const float* lsep = p.lse + b * p.row_bstride + h;
  const float* delp = p.delta + b * p.row_bstride + h;

  const int j0 = kb * BKV;
  const int kw0 = j0 + 32 * kw;
  const int krow = kw0 + ln;
  const bool key_ok = krow < p.Sk;

  // this lane's key row of K (role A) or V (role B) as MFMA B operand: dims 16*ks + 8*g .. +7
  bf16x8 kvf[NKS];
  {
    const uint16_t* kv = (role == 0 ? p.k : p.v) + b * p.k_bstride + (long)h * D_;
    const u32x4* src = reinterpret_cast<const u32x4*>(kv + (long)(key_ok ? krow : 0) * p.rs + 8 * g);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) kvf[ks] = as_bf16x8(key_ok ? src[2 * ks] : u32x4{0u, 0u, 0u, 0u});
    // land these before the direct-to-LDS ring starts (see the forward kernel)
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) asm volatile("" : "+v"(kvf[ks]));
  }
  const int kpos = seg_pos(p.ks, key_ok ? krow : (p.Sk - 1));
  QueryWindow qwin = query_window(p.qs, kpos, p.causal);
  if (!key_ok) qwin = QueryWindow{0, 0, 0, 0};

  // key position ranges (workgroup and key group)
  const int wg_end = min(j0 + BKV, p.Sk);
  int kmin_wg, kmax_wg;
  seg_range(p.ks, j0, wg_end, kmin_wg, kmax_wg);
  const int kw1 = min(kw0 + 32, p.Sk);
  const bool group_live = kw0 < kw1;
  int kmin_w = 0x7fffffff, kmax_w = 0;
  if (group_live) seg_range(p.ks, kw0, kw1, kmin_w, kmax_w);

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
  // last query tile first: the workgroups an XCD starts together (neighbouring
  // key blocks) then begin at the same query tile instead of 4 tiles apart per
  // key block, so more of their reads hit the XCD's L2 (20 % fewer L2 misses at
  // 64K tokens, same time)
  auto tile_of = [&](int t) {
    const int u = nt - 1 - t;
    return u < nA ? tA0 + u : tC0 + (u - nA);
  };

  f32x16 acc[NDB];  // dV^T (role A) or dK^T (role B): rows = dims, columns = keys
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};

  // ---- direct global -> LDS loads: load k of a tile (k = w + NW*i) moves rows
  // [RPI*(k % (NI/2)), +RPI) of Q (k < NI/2) or dO; lane i fills 16-byte slot
  // i % CPR of row i / CPR, i.e. chunk slot ^ swz(row).  Wave 0 also moves the
  // tile's 32 LSE and 32 Delta values (4 bytes per lane, lane i to word i).
  // (Spreading that load over the eight waves, eight lanes each, so that every
  // wave waits for the same count, cost 2.6 ms at 64K tokens: each wave then
  // waits for a scattered load of its own.)
  const int dma_row = lane / CPR, dma_slot = lane % CPR;
  uint32_t dma_off[Cfg::NIW];
#pragma unroll
  for (int i = 0; i < Cfg::NIW; ++i) {
    const int k = w + Cfg::NW * i, part = k % (Cfg::NI / 2);
    const int row = RPI * part + dma_row;
    dma_off[i] = (uint32_t)(((long)row * p.rs + ((dma_slot ^ swz<D>(row)) << 3)) * 2);
  }
  const float* stat_src = g == 0 ? lsep : delp;  // lanes 0..31: LSE, 32..63: Delta
  const float* stat_lane = stat_src + (long)ln * p.Hs;
  const bool stat_mine = w == 0;  // uniform per wave
  auto load_rows = [&](int stage, const uint16_t* qt, const uint16_t* ot, const float* st) {
#pragma unroll
    for (int i = 0; i < Cfg::NIW; ++i) {
      const int k = w + Cfg::NW * i, tns = k / (Cfg::NI / 2), part = k % (Cfg::NI / 2);
      dma16_s(tns ? ot : qt, dma_off[i], &QO[stage][tns * OT + RPI * part * D]);
    }
    if (stat_mine) dma4(st, &Ss[stage][0]);
  };
  // Any tile t (prologue): t past the last tile reloads the last one into a
  // stage nobody reads; rows past the end of the queries load the last row
  // (the element mask removes them).  Only the first tile visited can be such
  // a ragged tile: it is the highest tile of the last segment visited first.
  auto issue_any = [&](int stage, int t) {
    const int tt = t < nt ? t : nt - 1;
    const int i0 = __builtin_amdgcn_readfirstlane(tile_of(tt) * BQ);
    const uint16_t* qt = qp + (long)i0 * p.rs;
    const uint16_t* ot = op + (long)i0 * p.rs;
    if (i0 + BQ <= p.Sq) {
      load_rows(stage, qt, ot, stat_lane + (long)i0 * p.Hs);
      return;
    }
#pragma unroll
    for (int i = 0; i < Cfg::NIW; ++i) {
      const int k = w + Cfg::NW * i, tns = k / (Cfg::NI / 2), part = k % (Cfg::NI / 2);
      const int row0 = RPI * part, row = row0 + dma_row;
      const int ii = min(row, p.Sq - 1 - i0);
      const uint32_t off = (uint32_t)(((long)ii * p.rs + ((dma_slot ^ swz<D>(row)) << 3)) * 2);
      dma16_s(tns ? ot : qt, off, &QO[stage][tns * OT + row0 * D]);
    }
    if (stat_mine) dma4(stat_src + (long)min(i0 + ln, p.Sq - 1) * p.Hs, &Ss[stage][0]);
  };
  // Tiles 5, 6, ... (whole, before the last): scalar pointers to the first row
  // of the next tile, stepped down one tile per load, except once, from the
  // lowest tile of the segment visited first over the causally skipped tiles
  // to the highest tile of the other (a longer step).
  const long tstep = (long)BQ * p.rs;
  const long jstep = (long)(tC0 - tA1 + 1) * BQ * p.rs;
  const int sstep = BQ * p.Hs, sjump = (tC0 - tA1 + 1) * BQ * p.Hs;
  const uint16_t* nq = qp;
  const uint16_t* no = op;
  int ns = 0;  // statistics: first row times Hs (Sq*Hs < 2^29: the Delta launch's grid check bounds it)
  {
    const int r5 = __builtin_amdgcn_readfirstlane(tile_of(5 < nt ? 5 : 0) * BQ);
    nq += (long)r5 * p.rs;
    no += (long)r5 * p.rs;
    ns = r5 * p.Hs;
  }
  auto issue_next = [&](int stage, int m) {  // loads tile m + 4 (>= 5, < nt), then points at tile m + 5
    load_rows(stage, nq, no, stat_lane + ns);
    const bool jump = m + 5 == nC;
    const long st = jump ? jstep : tstep;
    nq -= st;
    no -= st;
    ns -= jump ? sjump : sstep;
  };
  constexpr int LOADS = Cfg::NIW;  // per tile and wave (wave 0: one more)
  // this wave's loads of all but the last N tiles it issued have landed
  auto wait_loads = [&](auto N) {
    constexpr int n = decltype(N)::value;
    if (w == 0)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(n * (LOADS + 1)) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(n * LOADS) : "memory");
  };

  // per-lane LDS offsets (elements)
  // operand of the score products: row ln, chunk 2*ks+g = slot 2*(ks ^ qx) + (g ^ (swz & 1))
  const int qx = swz<D>(ln) >> 1, qbase = ln * D + ((g ^ (swz<D>(ln) & 1)) << 3);
  int tofs[2][NDB];  // dO^T / Q^T transpose read: rows 8*half + trow (+16 per k-step), 32 dims per block
  {
    const int trow = 4 * g + ((lane & 15) >> 2);
    const int tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int col = 32 * db + tcol;
        tofs[half][db] = tile_off<D>(8 * half + trow, col >> 3) + (col & 7);
      }
  }

  // class of tile t for this key group: FULL (no mask) or PARTIAL (element mask).
  auto classify = [&](int t) {
    const int i0 = tile_of(t) * BQ;
    if (!group_live || i0 + BQ > p.Sq || kw0 + 32 > p.Sk) return (int)kPartial;
    if (!p.causal) return (int)kFull;
    int qmn, qmx;
    seg_range(p.qs, i0, i0 + BQ, qmn, qmx);
    return kmax_w <= qmn ? (int)kFull : (int)kPartial;
  };

  using RoleA = std::integral_constant<int, 0>;
  using RoleB = std::integral_constant<int, 1>;
  const float c = p.c;
  constexpr float NEG_INF = -__builtin_inff();

  // Ping-pong between the two waves of each SIMD (A = wave kw, B = wave 4 + kw,
  // same keys).  In step t (between two workgroup barriers) A runs its product
  // phase of query tile t (S(t), then dV^T += dO(t-1)^T P(t-1)), then turns S(t)
  // into P(t) and hands it to B through LDS; B forms dS(t-1) = P(t-1) (dP(t-1) -
  // Delta), then runs its product phase (dP(t), then dK^T += Q(t-1)^T dS(t-1)).
  // So one wave of each SIMD tends to feed the matrix core while the other runs
  // vector work.  (A second barrier per step that forced the phases apart cost
  // more in waiting than it gained.)
  f32x4 lsepf[4];  // A: base-2 LSE of the tile's rows, read in the product phase; B: -Delta of the next tile's
                   // rows, read in the vector phase, the start of the next dP accumulation
  f32x16 sx;                             // A: S of the current tile; B: dP
  bf16x8 pk[2] = {bf16x8{}, bf16x8{}};   // A: P of the previous tile; B: dS of the previous tile (bf16)

  // operand i of a score-like product: 16 bytes of row ln of the Q (A) or dO (B)
  // tile in stage cst
  constexpr int PF = 3;  // depth of the product phases' operand ring
  auto score_op = [&](auto ROLE, auto CST, int i) {
    constexpr int R = decltype(ROLE)::value, cst = decltype(CST)::value;
    return *reinterpret_cast<const u32x4*>(&QO[cst][qbase + ((i ^ qx) << 4) + R * OT]);
  };

  // product phase: the score-like product of tile (stage cst) with this wave's
  // K or V rows, then acc += (tile^T operand of stage pst) x pk, the transposed
  // operand being dO (A: dV) or Q (B: dK).  Operands through a register ring PF
  // products deep, pinned by scheduling groups (left to itself the compiler read
  // each operand right before its product and waited for it).  The first PF
  // operands (`pre`) are read by the caller: in the loop during the wave's
  // vector phase before (the tile has been resident since the barrier before
  // it), so the first products need not wait for LDS after the barrier
  // (-0.4 ms at 64K tokens for the K side, -0.1 more for the V side).
  auto m_phase = [&](auto ROLE, auto CST, auto PST, const u32x4 (&pre)[PF], auto&& hook) {
    constexpr int R = decltype(ROLE)::value, cst = decltype(CST)::value, pst = decltype(PST)::value;
    // The K side's product and vector phases are the critical chain of the pair:
    // its products win the issue port while the V side's overlap them (the V
    // side's vector phase is the shorter one).  Priority for the V side's
    // products instead starved the K side (+7.6 ms at 64K tokens).
    if constexpr (R == 0) __builtin_amdgcn_s_setprio(2);
    constexpr int NSC = NKS, NAC = 2 * NDB, N = NSC + NAC;
    static_assert(PF <= NSC, "the ring starts inside the score products");
    auto rd = [&](int i) {
      if (i < NSC) return score_op(ROLE, CST, i);
      const int kk = (i - NSC) / NDB, db = (i - NSC) % NDB;
      constexpr int base = R == 0 ? OT : 0;
      const u32x2 lo = ds_read_tr16(&QO[pst][base + tofs[0][db] + 16 * kk * D]);
      const u32x2 hi = ds_read_tr16(&QO[pst][base + tofs[1][db] + 16 * kk * D]);
      return u32x4{lo[0], lo[1], hi[0], hi[1]};
    };
    u32x4 fr[N];
#pragma unroll
    for (int i = 0; i < PF; ++i) fr[i] = pre[i];
    if constexpr (R == 0) {  // the new tile's LSE (converted in the previous step) for the vector phase
      const f32x4* lsrc = reinterpret_cast<const f32x4*>(&Ss[cst][4 * g]);
#pragma unroll
      for (int m = 0; m < 4; ++m) lsepf[m] = lsrc[2 * m];
    }
    hook();  // the tile loads, while the first reads are under way
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      if (i + PF < N) fr[i + PF] = rd(i + PF);
      if (i < NSC) {
        f32x16 c0 = f32x16{};  // B: dP - Delta comes out of the products (register r holds row 8(r/4)+4g+r%4)
        if constexpr (R == 1) {
#pragma unroll
          for (int r = 0; r < 16; ++r) c0[r] = lsepf[r >> 2][r & 3];
        }
        sx = mfma32(as_bf16x8(fr[i]), kvf[i], i == 0 ? c0 : sx);
      } else {
        const int j = i - NSC;
        acc[j % NDB] = mfma32(as_bf16x8(fr[i]), pk[j / NDB], acc[j % NDB]);
      }
    }
#pragma unroll
    for (int i = 0; i < N; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // product i
      if (i + PF < NSC) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // the read of score product i + PF
      } else if (i + PF < N) {
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // the two reads of product i + PF
      }
    }
    asm volatile("" : "+v"(sx));
    if constexpr (R == 0) {
#pragma unroll
      for (int m = 0; m < 4; ++m) asm volatile("" : "+v"(lsepf[m]));
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db) asm volatile("" : "+v"(acc[db]));
    if constexpr (R == 0) __builtin_amdgcn_s_setprio(0);
  };

  // bf16 packs of a lane's 16 values: pk[kk] holds values 8*kk .. 8*kk+7
  auto pack16 = [&](const float* v) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int o = 8 * kk;
      pk[kk] = pack_bf16x8(v[o], v[o + 1], v[o + 2], v[o + 3], v[o + 4], v[o + 5], v[o + 6], v[o + 7]);
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) asm volatile("" : "+v"(pk[kk]));
  };

  // A's vector phase for tile t: mask, P = exp2(S c - LSE2) (the LSE
  // of the tile's rows, already in base-2 units (see to_log2), was read in the
  // product phase of the same step), published to
  // B as fp16 pairs, kept as bf16 packs for dV.  A barrier does not wait for
  // memory, so A waits for its LDS writes before the barrier that publishes them.
  auto a_v = [&](int t, auto SN, u32x4 (&pre)[PF]) {
#pragma unroll
    for (int i = 0; i < PF; ++i) pre[i] = score_op(RoleA{}, SN, i);  // for the next product phase
    if (classify(t) == kPartial) {
      const int i0 = tile_of(t) * BQ;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = i0 + 8 * (r >> 2) + 4 * g + (r & 3);
        sx[r] = in_window(qwin, i) ? sx[r] : NEG_INF;
      }
    }
    float pv[16];
    uint32_t* pdst = &Ps[t & 1][kw][0][lane][0];
#pragma unroll
    for (int j = 0; j < 2; ++j) {  // each half is written as soon as it is formed (the wall keeps it so), so
                                   // the first write's latency passes under the second half's exponentials
#pragma unroll
      for (int r = 8 * j; r < 8 * j + 8; ++r) pv[r] = fast_exp2(__builtin_fmaf(sx[r], c, -lsepf[r >> 2][r & 3]));
      u32x4 hv;
#pragma unroll
      for (int e = 0; e < 4; ++e) hv[e] = pack_f16x2(pv[8 * j + 2 * e], pv[8 * j + 2 * e + 1]);
      *reinterpret_cast<u32x4*>(pdst + j * 256) = hv;
      __builtin_amdgcn_sched_barrier(0);
    }
    pack16(pv);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  };

  // Wave 4 (a V-side wave) rewrites the row statistics of tile t+1 during step
  // t, after its vector phase: lanes 0..31 the LSE in base-2 units less
  // kPScaleLog2, so that exp2 gives 2^kPScaleLog2 P (-inf, a row without any
  // allowed key, becomes +inf so that its recomputed probabilities are exactly
  // 0), lanes 32..63 Delta negated (the start of the dP accumulations); the next
  // barrier publishes the converted values before they are read in step t+1
  // (wave 4 waits for its write first: a barrier does not wait for memory).
  auto stat_conv = [&](float l) {
    return g == 1 ? -l : (l == -__builtin_inff() ? __builtin_inff() : l * kLog2e - kPScaleLog2);
  };
  auto to_log2 = [&](auto ST) {
    constexpr int stage = decltype(ST)::value;
    if (w == 4) {
      const float l = Ss[stage][lane];
      Ss[stage][lane] = stat_conv(l);
    }
    if (w == 4) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  };
  // the same in two parts around B's vector phase, so that the read's latency hides under it (B's
  // vector phase issues the read)
  auto lse_read = [&](auto ST) {
    constexpr int stage = decltype(ST)::value;
    return w == 4 ? Ss[stage][lane] : 0.f;
  };
  auto lse_write = [&](auto ST, float l) {
    constexpr int stage = decltype(ST)::value;
    if (w == 4) Ss[stage][lane] = stat_conv(l);
    if (w == 4) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  };

  // B's vector phase for tile t: dS = P (dP - Delta) from A's P(t) (its product
  // phase started the dP accumulation from -Delta).  It reads P(t) first, then
  // -Delta of tile t+1 (stage SN, negated one step earlier) for the next
  // product phase and, on wave 4, the raw statistic of tile t+2 (stage SNN)
  // that it converts afterwards (returned); the reads return in that order.
  auto b_v = [&](auto SN, auto SNN, int t, u32x4 (&pre)[PF], auto&& hook) {
    const u32x4* psrc8 = reinterpret_cast<const u32x4*>(&Ps[t & 1][kw][0][lane][0]);
    u32x4 ph[2];
    ph[0] = psrc8[0];
    ph[1] = psrc8[64];
    {
      const f32x4* dsrc = reinterpret_cast<const f32x4*>(&Ss[decltype(SN)::value][BQ + 4 * g]);
#pragma unroll
      for (int m = 0; m < 4; ++m) lsepf[m] = dsrc[2 * m];
    }
    const float lraw = lse_read(SNN);
#pragma unroll
    for (int i = 0; i < PF; ++i) pre[i] = score_op(RoleB{}, SN, i);  // for the next product phase
    __builtin_amdgcn_sched_group_barrier(0x100, 7 + PF, 0);  // the reads in program order
    __builtin_amdgcn_sched_barrier(0);
    hook();  // the tile loads, while the reads are under way
    __builtin_amdgcn_sched_barrier(0);
    float dsv[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) dsv[r] = mul_f16_f32(ph[r >> 3][(r & 7) >> 1], r & 1, sx[r]);
    pack16(dsv);
    asm volatile("" : "+v"(sx));
    return lraw;
  };

  // Step m starts once tiles m and m+1 are resident for every wave (tile m+1
  // for the LSE conversion); then the loads of tile m+4 go into the stage tile
  // m-2 held (its last readers, the dV and dK products of tile m-2, ran in step
  // m-1).  Each wave issues those loads right after the first LDS reads of the
  // phase that follows the barrier (`hook`), so that their address work passes
  // under the reads' latency.
  constexpr int AHEAD = 2;  // tiles in flight beyond the two needed
  static_assert(NST == 6, "loads run four tiles ahead in a ring of six stages");
  // Near the end no tile is loaded and the wave waits for all of its loads.
  auto sync_wait = [&](int m) {  // returns whether tile m + 4 is to be loaded
    __builtin_amdgcn_sched_barrier(0);
    const bool more = m + 4 < nt;
    if (more) {
      wait_loads(std::integral_constant<int, AHEAD>{});
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    }
    __builtin_amdgcn_sched_barrier(0);
    return more;
  };
  auto sync_plain = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  using S0 = std::integral_constant<int, 0>;
  // step t of each role with every stage index a constant (t = 6 i + U): tile
  // t in stage U, tile t+1 in stage U+1, loads of tile t+5 into stage U+5
  auto a_step = [&](auto U, int t) {
    constexpr int u = decltype(U)::value;
    using ST = std::integral_constant<int, u % NST>;
    using SN = std::integral_constant<int, (u + 1) % NST>;
    using SL = std::integral_constant<int, (u + 5) % NST>;
    __builtin_amdgcn_sched_barrier(0);
    u32x4 pre[PF];
    a_v(t, SN{}, pre);
    const bool more = sync_wait(t + 1);
    m_phase(RoleA{}, SN{}, ST{}, pre, [&]() { if (more) issue_next(SL::value, t + 1); });
    return t + 1 < nt;
  };
  auto b_step = [&](auto U, int t) {
    constexpr int u = decltype(U)::value;
    using ST = std::integral_constant<int, u % NST>;
    using SN = std::integral_constant<int, (u + 1) % NST>;
    using SL = std::integral_constant<int, (u + 5) % NST>;
    using SNN = std::integral_constant<int, (u + 2) % NST>;
    const bool more = sync_wait(t + 1);
    u32x4 pre[PF];
    const float lraw = b_v(SN{}, SNN{}, t, pre, [&]() { if (more) issue_next(SL::value, t + 1); });
    lse_write(SNN{}, lraw);
    __builtin_amdgcn_sched_barrier(0);
    m_phase(RoleB{}, SN{}, ST{}, pre, [] {});
    return t + 1 < nt;
  };

  if (nt > 0) {
    for (int i = 0; i < 4; ++i) issue_any(i, i);
    wait_loads(std::integral_constant<int, AHEAD>{});
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    issue_any(4, 4);
    // Both roles pass the same nt + 2 barriers (one extra after the first step,
    // which publishes the LSE of tiles 0 and 1).  The first product phase of
    // each role adds zeros times the resident tile 0, the last one computes the
    // score-like product of a stage that holds no new tile (an older or a
    // reloaded one) and drops it, so every product phase is the same straight
    // run of products.
    if (role == 0) {
      u32x4 pre[PF];
#pragma unroll
      for (int i = 0; i < PF; ++i) pre[i] = score_op(RoleA{}, S0{}, i);
      m_phase(RoleA{}, S0{}, S0{}, pre, [] {});
      sync_plain();
      {  // tile 0's LSE is converted before this barrier, after the first product phase read it
        const f32x4* lsrc = reinterpret_cast<const f32x4*>(&Ss[0][4 * g]);
#pragma unroll
        for (int m = 0; m < 4; ++m) lsepf[m] = lsrc[2 * m];
      }
      for (int t = 0;; t += 6) {
        if (!a_step(std::integral_constant<int, 0>{}, t)) break;
        if (!a_step(std::integral_constant<int, 1>{}, t + 1)) break;
        if (!a_step(std::integral_constant<int, 2>{}, t + 2)) break;
        if (!a_step(std::integral_constant<int, 3>{}, t + 3)) break;
        if (!a_step(std::integral_constant<int, 4>{}, t + 4)) break;
        if (!a_step(std::integral_constant<int, 5>{}, t + 5)) break;
      }
    } else {
      to_log2(S0{});
      to_log2(std::integral_constant<int, 1>{});
      sync_plain();
      {
        const f32x4* dsrc = reinterpret_cast<const f32x4*>(&Ss[0][BQ + 4 * g]);
#pragma unroll
        for (int m = 0; m < 4; ++m) lsepf[m] = dsrc[2 * m];
      }
      u32x4 pre[PF];
#pragma unroll
      for (int i = 0; i < PF; ++i) pre[i] = score_op(RoleB{}, S0{}, i);
      m_phase(RoleB{}, S0{}, S0{}, pre, [] {});
      for (int t = 0;; t += 6) {
        if (!b_step(std::integral_constant<int, 0>{}, t)) break;
        if (!b_step(std::integral_constant<int, 1>{}, t + 1)) break;
        if (!b_step(std::integral_constant<int, 2>{}, t + 2)) break;
        if (!b_step(std::integral_constant<int, 3>{}, t + 3)) break;
        if (!b_step(std::integral_constant<int, 4>{}, t + 4)) break;
        if (!b_step(std::integral_constant<int, 5>{}, t + 5)) break;
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // retire the trailing (unused) loads
  }

  if (!key_ok || nt == 0) return;
  // dK of rotated keys turned back by the key's position: the gradient with respect to the unrotated row
  // (the rotation is linear, so turning each call's contribution before it is added is exact)
  if (role == 1 && p.rope) rope_back(acc, kpos, p.f, g);
  float* dst = (role == 0 ? p.dv : p.dk) + b * p.k_bstride + (long)h * D_ + (long)krow * p.rs;
  constexpr float kPUnscale = 1.f / (float)(1 << kPScaleLog2);  // exact: the accumulators hold 2^kPScaleLog2 P
  const float mul = role == 0 ? kPUnscale : p.scale * kPUnscale;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d0 = 32 * db + 8 * q4 + 4 * g;
      f32x4 v4 = *reinterpret_cast<f32x4*>(dst + d0);
#pragma unroll
      for (int e = 0; e < 4; ++e) v4[e] += mul * acc[db][4 * q4 + e];
      *reinterpret_cast<f32x4*>(dst + d0) = v4;
    }
}

// ------------------------------------------------------------------ dQ
// One workgroup = 8 waves = 256 query rows of one (batch, head), two waves per
// SIMD, so each key/value tile in LDS serves eight waves; each wave owns
// 32 rows and keeps their Q and dO rows as MFMA B operands and its dQ^T
// accumulator in registers.  Key/value tiles of 32 rows stream through a
// 4-stage direct-to-LDS ring (K and V of a stage side by side), loaded two
// tiles ahead, exactly like the forward.  Per tile: S^T = K Q^T and
// dP^T = V dO^T (query on the lane axis, so each lane's LSE and Delta are one
// value), P and dS = P (dP - Delta), then dQ^T += K^T dS^T with K^T read by the
// LDS transpose read.  The products of tile t and the dQ product of tile t-1
// form one phase, the P / dS arithmetic of tile t another, and the two waves
// of a SIMD run them in opposite orders between the barriers (the forward's
// ping-pong).
template <int D>
struct DqCfg {
  static constexpr int NW = 8, BQ = 32 * NW, BK = 32, NT = 64 * NW, NST = 4;
  static constexpr int CPR = D / 8;                // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;             // rows one direct-to-LDS load covers
  static constexpr int NLT = BK / RPI;             // loads per tile (each of K and V)
  static constexpr int NKL = (NLT + NW - 1) / NW;  // per wave (waves w + NW*i < NLT take part)
  static constexpr int LDS_T = BK * D;
  static_assert(NLT * RPI == BK && (NLT % NW == 0 || NLT < NW), "unsupported key tile");
};

template <int D>
__global__ __launch_bounds__(64 * DqCfg<128>::NW, 1) void dq_kernel(BwdParams p) {
  using Cfg = DqCfg<D>;
  constexpr int BQ = Cfg::BQ, BK = Cfg::BK, CPR = Cfg::CPR, NST = Cfg::NST, RPI = Cfg::RPI;
  constexpr int NKS = D / 16, NDB = D / 32, KT = Cfg::LDS_T;
  // stage s: K tile at KV[s][0], V tile at KV[s][KT]
  __shared__ __attribute__((aligned(16))) uint16_t KV[NST][2 * KT];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform (scalar)
  const int ln = lane & 31, g = lane >> 5;

  const int work = xcd_remap(blockIdx.x, gridDim.x, p.nblk);
  const int bh = work / p.nblk;
  const int qb = p.nblk - 1 - work % p.nblk;  // longest query blocks first
  const int b = bh / p.H, h = bh % p.H;
  const int D_ = D;

  const uint16_t* qp = p.q + b * p.q_bstride + (long)h * D_;
  const uint16_t* op = p.dout + b * p.q_bstride + (long)h * D_;
  const uint16_t* kp = p.k + b * p.k_bstride + (long)h * D_;
  const uint16_t* vp = p.v + b * p.k_bstride + (long)h * D_;

  const int i0 = qb * BQ;
  const int qrow = i0 + 32 * w + ln;
  const bool row_ok = qrow < p.Sq;

  // this lane's Q and dO rows as MFMA B operands: dims 16*ks + 8*g .. +7
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
  const long srow = b * p.row_bstride + (long)(row_ok ? qrow : 0) * p.Hs + h;
  const float lse2 = row_ok ? lse_to_log2(p.lse[srow]) : __builtin_inff();
  const float dlt = row_ok ? p.delta[srow] : 0.f;
  // land these before the direct-to-LDS ring starts (see the forward kernel)
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) asm volatile("" : "+v"(qf[ks]), "+v"(of[ks]));
  float l2 = lse2, dl = dlt;
  asm volatile("" : "+v"(l2), "+v"(dl));
  f32x16 negd;  // -Delta of the lane's row: the start of every dP^T accumulation, so dP^T - Delta comes out of it
#pragma unroll
  for (int r = 0; r < 16; ++r) negd[r] = -dl;
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

  // ---- direct global -> LDS loads (as in the forward); rows past the end of
  // the keys load the last key row, and the element mask removes them
  const int dma_row = lane / CPR, dma_slot = lane % CPR;
  uint32_t dma_off[Cfg::NKL];  // byte offset from the tile's first row (a scalar base)
#pragma unroll
  for (int it = 0; it < Cfg::NKL; ++it) {
    const int row = RPI * (w + Cfg::NW * it) + dma_row;
    dma_off[it] = (uint32_t)(((long)row * p.rs + ((dma_slot ^ swz<D>(row)) << 3)) * 2);
  }
  auto load_kv = [&](auto STAGE, const uint16_t* kb, const uint16_t* vb) {
    constexpr int stage = decltype(STAGE)::value;
#pragma unroll
    for (int it = 0; it < Cfg::NKL; ++it) {
      if (Cfg::NLT < Cfg::NW && w >= Cfg::NLT) break;  // this wave loads nothing
      const int row0 = RPI * (w + Cfg::NW * it);
      dma16_s(kb, dma_off[it], &KV[stage][row0 * D]);
      dma16_s(vb, dma_off[it], &KV[stage][KT + row0 * D]);
    }
  };
  // Any tile t (prologue, and a ragged last tile): t past the last tile reloads
  // it into a stage nobody reads.  Only the last tile visited, the highest, can
  // be ragged.
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
      dma16_s(kb, off, &KV[stage][row0 * D]);
      dma16_s(vb, off, &KV[stage][KT + row0 * D]);
    }
  };
  // Tiles 2 .. nfast-1 (whole): scalar pointers stepped up one tile per load,
  // except once, over the causally skipped tiles between the two runs.
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

  // per-lane LDS offsets: K / V operand row ln, chunk 2*ks+g = slot 2*(ks ^ kx) + (g ^ (swz & 1))
  const int kx = swz<D>(ln) >> 1, kbase = ln * D + ((g ^ (swz<D>(ln) & 1)) << 3);
  int tofs[2][NDB];  // K^T transpose read: rows 8*half + trow (+16 per k-step), 32 dims per block
  {
    const int trow = 4 * g + ((lane & 15) >> 2);
    const int tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int col = 32 * db + tcol;
        tofs[half][db] = tile_off<D>(8 * half + trow, col >> 3) + (col & 7);
      }
  }

  // wave-level class of tile t: FULL or PARTIAL (a tile without any allowed pair
  // is computed fully masked, keeping the loop one straight pipeline)
  auto classify = [&](int t) {
    const int j0 = tile_of(t) * BK;
    if (!wave_live || j0 + BK > p.Sk) return (int)kPartial;
    if (!p.causal) return (int)kFull;
    int kmn, kmx;
    seg_range(p.ks, j0, j0 + BK, kmn, kmx);
    return kmx <= qmin_w ? (int)kFull : (int)kPartial;
  };

  constexpr float NEG_INF = -__builtin_inff();
  const float c = p.c;

  f32x16 sc, dpv;  // S^T and dP^T - Delta of a tile between its product phase and its arithmetic phase;
                   // register r of lane l holds key 8*(r/4) + 4*g + r%4 of query ln
  bf16x8 sb[2] = {bf16x8{}, bf16x8{}};  // dS^T of the previous tile, keys 0-15 and 16-31, as B operands

  // Product phase of tile t: S^T(t) = K Q^T and dP^T(t) = V dO^T from stage
  // CSTAGE (k-step major; the dP^T accumulation starts from -Delta), then
  // dQ^T += K^T(t-1) dS^T(t-1) with K^T read transposed from stage PSTAGE.  The
  // first phase (t = 0) adds dS = 0 times the resident tile 0; the last (t = nt)
  // computes the products of a stage holding no new tile and drops them.
  // Operands go through a register ring PF products deep, pinned by scheduling
  // groups (as in the forward).
  auto m_phase = [&](auto CSTAGE, auto PSTAGE) {
    constexpr int cst = decltype(CSTAGE)::value, pst = decltype(PSTAGE)::value;
    constexpr int NSD = 2 * NKS, NDQ = 2 * NDB, N = NSD + NDQ, PF = 3;
    __builtin_amdgcn_s_setprio(2);  // the products win the issue port from the other wave's vector work
    static_assert(PF <= NSD, "the ring starts inside the score products");
    auto rd = [&](int i) {
      if (i < NSD) {  // K (even i) or V (odd i) operand of k-step i / 2
        const int o = kbase + (((i >> 1) ^ kx) << 4) + ((i & 1) ? KT : 0);
        return *reinterpret_cast<const u32x4*>(&KV[cst][o]);
      }
      const int kk = (i - NSD) / NDB, db = (i - NSD) % NDB;  // K^T operand of dQ product i - NSD
      const u32x2 lo = ds_read_tr16(&KV[pst][tofs[0][db] + 16 * kk * D]);
      const u32x2 hi = ds_read_tr16(&KV[pst][tofs[1][db] + 16 * kk * D]);
      return u32x4{lo[0], lo[1], hi[0], hi[1]};
    };
    u32x4 fr[N];
#pragma unroll
    for (int i = 0; i < PF; ++i) fr[i] = rd(i);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      if (i + PF < N) fr[i + PF] = rd(i + PF);
      if (i < NSD) {
        const int ks = i >> 1;
        if (i & 1)
          dpv = mfma32(as_bf16x8(fr[i]), of[ks], ks == 0 ? negd : dpv);
        else
          sc = mfma32(as_bf16x8(fr[i]), qf[ks], ks == 0 ? f32x16{} : sc);
      } else {
        const int j = i - NSD;
        dqa[j % NDB] = mfma32(as_bf16x8(fr[i]), sb[j / NDB], dqa[j % NDB]);
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x100, PF, 0);  // operands of the first PF products
#pragma unroll
    for (int i = 0; i < N; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // product i
      if (i + PF < NSD) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // the read of score product i + PF
      } else if (i + PF < N) {
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // the two reads of dQ product i + PF - NSD
      }
    }
    asm volatile("" : "+v"(sc), "+v"(dpv));
#pragma unroll
    for (int db = 0; db < NDB; ++db) asm volatile("" : "+v"(dqa[db]));
    __builtin_amdgcn_s_setprio(0);
  };

  // Arithmetic phase of tile t: mask, P = exp2(S c - LSE2), dS = P (dP - Delta)
  // (lse2 = +inf for a row without any allowed key, so its P is exactly 0),
  // packed to bf16.
  auto v_phase = [&](int t) {
    if (classify(t) == kPartial) {
      const int j0 = tile_of(t) * BK;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = j0 + 8 * (r >> 2) + 4 * g + (r & 3);
        sc[r] = in_window(kwin, j) ? sc[r] : NEG_INF;
      }
    }
    float dsv[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) dsv[r] = fast_exp2(__builtin_fmaf(sc[r], c, -l2)) * dpv[r];
    sb[0] = pack_bf16x8(dsv[0], dsv[1], dsv[2], dsv[3], dsv[4], dsv[5], dsv[6], dsv[7]);
    sb[1] = pack_bf16x8(dsv[8], dsv[9], dsv[10], dsv[11], dsv[12], dsv[13], dsv[14], dsv[15]);
    asm volatile("" : "+v"(sb[0]), "+v"(sb[1]));
    asm volatile("" : "+v"(sc), "+v"(dpv));
#pragma unroll
    for (int db = 0; db < NDB; ++db) asm volatile("" : "+v"(dqa[db]));
  };

  // Step boundaries, as in the forward: step m starts once tile m is resident
  // for every wave, and then the load of tile m+2 goes into the stage tile m-2
  // held (its last readers, the dQ products of tile m-2, ran in step m-1).
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
    // Ping-pong between the two waves of each SIMD (waves w and w + NW/2), as in
    // the forward: in step t the first half runs the product phase of tile t,
    // then its arithmetic; the second half the arithmetic of tile t-1, then the
    // product phase of tile t; both pass the same nt + 1 barriers.
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

  if (!row_ok || nt == 0) return;
  if (p.rope) rope_back(dqa, qpos, p.f, g);  // gradient with respect to the unrotated query row
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
  p.rs = (long)a.Hs * a.D;
  p.q_bstride = (long)a.q_batch_rows * p.rs;
  p.k_bstride = (long)a.k_batch_rows * p.rs;
  p.row_bstride = (long)a.q_batch_rows * a.Hs;
  p.H = a.H;
  p.Hs = a.Hs;
  p.rope = a.rope;
  for (int k = 0; k < 64; ++k) p.f[k] = a.rope && k < a.D / 2 ? a.inv_freq[k] : 0.0;
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
  p.nblk = (a.Sq + DqCfg<128>::BQ - 1) / DqCfg<128>::BQ;
  const long nwg = (long)a.B * a.H * p.nblk;
  if (nwg == 0 || a.Sk == 0) return hipSuccess;
  dim3 grid((unsigned)nwg), block(DqCfg<128>::NT);
  if (a.D == 64)
    hipLaunchKernelGGL(dq_kernel<64>, grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL(dq_kernel<128>, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace ea
