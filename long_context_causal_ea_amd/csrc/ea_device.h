// Device-side building blocks shared by the gfx950 attention kernels:
// vector types, the bf16 MFMA wrappers, global-position segments and the
// XCD-aware work mapping.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ea {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kNumXcd = 8;  // MI355X: 8 accelerator complex dies, 32 CUs each

// D(32x32, fp32) += A(32x16, bf16) * B(16x32, bf16).
// Lane l supplies row (l % 32) of A and column (l % 32) of B, each holding the
// 8 reduction indices 8*(l/32) .. 8*(l/32)+7 of the 16.  Output register r of
// lane l holds D[8*(r/4) + 4*(l/32) + r%4][l % 32].
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// D(16x16, fp32) += A(16x32, bf16) * B(32x16, bf16).
// Lane l supplies row (l % 16) of A and column (l % 16) of B, each holding the
// 8 reduction indices 8*(l/16) .. 8*(l/16)+7 of the 32.  Output register r of
// lane l holds D[4*(l/16) + r][l % 16].
__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& u) { return __builtin_bit_cast(bf16x8, u); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Round-to-nearest-even fp32 -> bf16 of two values, packed low/high (one
// v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Round-to-nearest-even fp32 -> fp16 of two values, packed low/high.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}

// Half `hi` (0: low, 1: high) of a packed fp16 pair, widened to fp32 (exact),
// times b, in one instruction: the mixed-precision FMA takes the fp16 half as
// it is and adds -0, which leaves every product, the sign of a zero one
// included, as the fp32 multiply rounds it.  (The compiler does not form it
// from a conversion and a multiply.)
__device__ __forceinline__ float mul_f16_f32(uint32_t u, int hi, float b) {
  float y;
  if (hi)
    asm("v_fma_mix_f32 %0, %1, %2, -%3 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(y) : "v"(u), "v"(b), "v"(0.0f));
  else
    asm("v_fma_mix_f32 %0, %1, %2, -%3 op_sel:[0,0,0] op_sel_hi:[1,0,0]" : "=v"(y) : "v"(u), "v"(b), "v"(0.0f));
  return y;
}

__device__ __forceinline__ bf16x8 pack_bf16x8(float x0, float x1, float x2, float x3, float x4, float x5,
                                              float x6, float x7) {
  u32x4 u;
  u[0] = pack_bf16x2(x0, x1);
  u[1] = pack_bf16x2(x2, x3);
  u[2] = pack_bf16x2(x4, x5);
  u[3] = pack_bf16x2(x6, x7);
  return as_bf16x8(u);
}

// ---- LDS tiles: row-major [rows][D] bf16, 16-byte chunks XOR-swizzled per row.
// Chunk c of row r is stored at chunk slot c ^ swz(r).  The swizzle keeps the
// access patterns of the kernels free of bank conflicts on 64 banks x 4 bytes.
// Measured on gfx950: a 16-byte read is served in four passes, each taking
// lanes 8j..8j+7 together with lanes 32+8j..32+8j+7; a transpose read in two
// passes of 32 consecutive lanes; a 16-byte write in passes of 16 consecutive
// lanes.  The patterns are
//  (a) 32x32x16 operands: lanes l and l+32 read chunks 2k and 2k+1 of row l%32,
//  (b) 16x16x32 operands: lanes l, l+16, l+32, l+48 read chunks 4k..4k+3 of
//      row l%16, so one pass holds chunks 4k and 4k+2 of 8 consecutive rows,
//  (c) transpose reads of 4 consecutive rows x 64 bytes (32x32 operands) or of
//      8 consecutive rows x 32 bytes (16x16 operands) per 32 lanes,
//  (d) row-wise tile writes.
// For 16 chunks per row they are all conflict-free when, over every aligned 8
// rows, bits {1,2,3} and bits {0,2,3} of swz(r) both take 8 distinct values,
// and over every aligned 4 rows bits {2,3} take 4 distinct values:
// swz(r) = (r mod 4) * 4 + (3 if bit 2 of r else 0) ^ (bit 3 of r).
template <int D>
__device__ __forceinline__ int swz(int r);
template <>
__device__ __forceinline__ int swz<128>(int r) {  // 16 chunks per row
  return ((r & 3) << 2) | ((((r >> 2) & 1) * 3) ^ ((r >> 3) & 1));
}
template <>
__device__ __forceinline__ int swz<64>(int r) {  // 8 chunks per row, two rows per 256 bytes
  return ((r >> 1) & 1) | (((r >> 2) & 1) << 1) | ((((r >> 1) ^ (r >> 3)) & 1) << 2);
}
template <int D>
__device__ __forceinline__ int tile_off(int r, int chunk) {
  return r * D + ((chunk ^ swz<D>(r)) << 3);
}

// LDS transpose read (gfx950 ds_read_b64_tr_b16).  Within each group of 16
// lanes, if lane i addresses the 4 elements T[r0 + i/4][c0 + 4*(i%4) .. +3] of a
// row-major tile, lane j receives T[r0 + e][c0 + j] for e = 0..3: a 4 x 16 block
// read transposed, i.e. 4 consecutive rows of one column per lane.
typedef short short4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 ds_read_tr16(const uint16_t* p) {
  short4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4_t*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// Direct global -> LDS load of 16 bytes per lane (gfx950 global_load_lds_dwordx4):
// lane i's 16 bytes land at LDS byte address lds_base + 16*i (lds_base must be
// the same for the whole wave).  Issued as inline assembly on purpose: the
// compiler would otherwise wait for every such load in flight before any later
// LDS read, which defeats a multi-stage ring.  Callers therefore own the
// ordering: "s_waitcnt vmcnt(n)" for their own loads, then a workgroup barrier,
// then a compiler memory fence (lds_ring_sync below) before reading the data.
__device__ __forceinline__ void dma16(const void* gptr, const void* lds_base) {
  const uint32_t m0 = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const char*)lds_base);
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(gptr), "{m0}"(m0) : "memory");
}

// The same with a uniform 64-bit base held in scalar registers and a 32-bit
// per-lane byte offset (one vector register per address instead of two).
__device__ __forceinline__ void dma16_s(const void* sbase, uint32_t voff, const void* lds_base) {
  const uint32_t m0 = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const char*)lds_base);
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(m0) : "memory");
}

// Direct global -> LDS load of 4 bytes per lane (global_load_lds_dword): lane
// i's value lands at LDS byte address lds_base + 4*i.  Same ordering rules as
// dma16.
__device__ __forceinline__ void dma4(const void* gptr, const void* lds_base) {
  const uint32_t m0 = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const char*)lds_base);
  asm volatile("global_load_lds_dword %0, off" ::"v"(gptr), "{m0}"(m0) : "memory");
}

// Wait until at most N direct-to-LDS loads of this wave are in flight, then
// synchronise the workgroup; afterwards every wave sees the completed loads.
template <int N>
__device__ __forceinline__ void lds_ring_sync() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// max(x of this lane, x of lane l ^ 32): gfx950's lane swap between the two
// halves of a wave (a vector-ALU instruction, no LDS round trip).  Whichever
// half each output holds, the larger of the two outputs is the pair's maximum.
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Exponent base 2 on the hardware transcendental unit.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Global positions of the rows of one tensor: rows [0, l0) sit at s0 + i, rows
// [l0, n) at s1 + (i - l0).  A single-segment tensor has l0 = n.
struct Seg {
  int s0, l0, s1, n;
};

__device__ __forceinline__ int seg_pos(const Seg& g, int i) { return i < g.l0 ? g.s0 + i : g.s1 + (i - g.l0); }

// Smallest and largest position among rows [a, b) (a < b <= n).
__host__ __device__ __forceinline__ void seg_range(const Seg& g, int a, int b, int& mn, int& mx) {
  mn = 0x7fffffff;
  mx = -1;
  if (a < g.l0) {
    int e = b < g.l0 ? b : g.l0;
    mn = g.s0 + a;
    mx = g.s0 + e - 1;
  }
  if (b > g.l0) {
    int st = a > g.l0 ? a : g.l0;
    int p0 = g.s1 + (st - g.l0), p1 = g.s1 + (b - 1 - g.l0);
    mn = p0 < mn ? p0 : mn;
    mx = p1 > mx ? p1 : mx;
  }
}

// Key rows that any query with position <= qmax may see under the causal rule,
// as up to two row ranges [0, e0) and [b1, e1) of the key tensor.
__host__ __device__ __forceinline__ void causal_key_ranges(const Seg& k, int qmax, int& e0, int& b1, int& e1) {
  long n0 = (long)qmax - k.s0 + 1;
  n0 = n0 < 0 ? 0 : (n0 > k.l0 ? k.l0 : n0);
  e0 = (int)n0;
  long len1 = k.n - k.l0;
  long n1 = (long)qmax - k.s1 + 1;
  n1 = n1 < 0 ? 0 : (n1 > len1 ? len1 : n1);
  b1 = k.l0;
  e1 = k.l0 + (int)n1;
}

// ---- rotary position embedding (Llama "rotate-half"): dims k and k + D/2 of a
// row at position p turn by phi = p * f_k, f_k = theta^(-2k/D).  The angle is
// formed in fp64 (positions reach 2^31, where an fp32 angle is off by a large
// fraction of a radian) and its cosine and sine are rounded to fp32; the
// rotation itself is fp32 with one rounding to the output type.  Every kernel
// that rotates uses these functions, so a row rotated in any of them has the
// same bits.
//
// cos and sin in fp64 for a >= 0: Cody-Waite reduction a = n pi/2 + r with a
// two-part pi/2 (|r| <= pi/4; the product n * hi is exact to the last place of
// r by fma), then the Taylor series of sin r to r^15 and of cos r to r^16 (the
// first omitted terms are below 1e-16 relative on |r| <= pi/4), and the
// quadrant n mod 4 swaps and negates them.  Short and register-light, unlike
// a general sincos that must also handle huge arguments.
__device__ __forceinline__ float2 rope_cos_sin(int pos, double f) {
  const double a = (double)pos * f;
  constexpr double kPio2Hi = 1.5707963267948966;      // pi/2 rounded to double
  constexpr double kPio2Lo = 6.123233995736766e-17;   // pi/2 - kPio2Hi
  constexpr double k2OverPi = 0.6366197723675814;
  const double n = __builtin_rint(a * k2OverPi);
  double r = __builtin_fma(-n, kPio2Hi, a);
  r = __builtin_fma(-n, kPio2Lo, r);
  const double z = r * r;
  // 1/k! for the odd (sin) and even (cos) terms
  double sp = 7.647163731819816e-13;                  // 1/15!
  sp = __builtin_fma(sp, -z, 1.6059043836821613e-10); // 1/13!
  sp = __builtin_fma(sp, -z, 2.505210838544172e-08);  // 1/11!
  sp = __builtin_fma(sp, -z, 2.7557319223985893e-06); // 1/9!
  sp = __builtin_fma(sp, -z, 0.0001984126984126984);  // 1/7!
  sp = __builtin_fma(sp, -z, 0.008333333333333333);  // 1/5!
  sp = __builtin_fma(sp, -z, 0.16666666666666666); // 1/3!
  const double sn = __builtin_fma(-r * z, sp, r);
  double cp = 4.779477332387385e-14;                  // 1/16!
  cp = __builtin_fma(cp, -z, 1.1470745597729725e-11); // 1/14!
  cp = __builtin_fma(cp, -z, 2.08767569878681e-09);   // 1/12!
  cp = __builtin_fma(cp, -z, 2.755731922398589e-07);  // 1/10!
  cp = __builtin_fma(cp, -z, 2.48015873015873e-05);   // 1/8!
  cp = __builtin_fma(cp, -z, 0.001388888888888889);  // 1/6!
  cp = __builtin_fma(cp, -z, 0.041666666666666664); // 1/4!
  cp = __builtin_fma(cp, -z, 0.5);                    // 1/2!
  const double cs = __builtin_fma(-z, cp, 1.0);
  const int quad = (int)((long long)n & 3);
  const double c = (quad & 1) ? sn : cs, s = (quad & 1) ? cs : sn;
  return make_float2((float)((quad == 1 || quad == 2) ? -c : c), (float)((quad >= 2) ? -s : s));
}

// (lo, hi) = dims (k, k + D/2) turned by the angle whose (cos, sin) is cs;
// inverse turns by minus that angle (the transpose, for gradients).
__device__ __forceinline__ void rope_turn(float& lo, float& hi, float2 cs, bool inverse) {
  const float sn = inverse ? -cs.y : cs.y;
  const float l = lo, h = hi;
  lo = __builtin_fmaf(l, cs.x, -h * sn);
  hi = __builtin_fmaf(h, cs.x, l * sn);
}

// Key rows a query at position qpos may see, as [0, lim0) U [l0, lim1) of the
// key tensor (under the full mask: [0, n)).  Computed once per query row, so
// that the element mask of a partial tile is a few integer compares.
struct KeyWindow {
  int lim0, l0, lim1;
};

__device__ __forceinline__ KeyWindow key_window(const Seg& k, int qpos, bool causal) {
  if (!causal) return KeyWindow{k.n, k.n, k.n};
  long a = (long)qpos - k.s0 + 1;
  a = a < 0 ? 0 : (a > k.l0 ? k.l0 : a);
  long c = (long)k.l0 + ((long)qpos - k.s1 + 1);
  c = c < k.l0 ? k.l0 : (c > k.n ? k.n : c);
  return KeyWindow{(int)a, k.l0, (int)c};
}

__device__ __forceinline__ bool in_window(const KeyWindow& w, int j) {
  return (j < w.lim0) | ((j >= w.l0) & (j < w.lim1));
}

// Query rows that may see a key at position kpos, as [lo0, hi0) U [lo1, n).
struct QueryWindow {
  int lo0, hi0, lo1, n;
};

__device__ __forceinline__ QueryWindow query_window(const Seg& q, int kpos, bool causal) {
  if (!causal) return QueryWindow{0, q.n, q.n, q.n};
  long a = (long)kpos - q.s0;
  a = a < 0 ? 0 : (a > q.l0 ? q.l0 : a);
  long c = (long)q.l0 + ((long)kpos - q.s1);
  c = c < q.l0 ? q.l0 : (c > q.n ? q.n : c);
  return QueryWindow{(int)a, q.l0, (int)c, q.n};
}

__device__ __forceinline__ bool in_window(const QueryWindow& w, int i) {
  return ((i >= w.lo0) & (i < w.hi0)) | ((i >= w.lo1) & (i < w.n));
}

enum TileClass { kSkip = 0, kFull = 1, kPartial = 2 };

// Hardware places workgroup `bid` on XCD bid % 8 and each XCD runs its share in
// dispatch order, so the work an XCD receives is fixed at launch.  The work list
// is (batch*head) major with `per_bh` items per head, longest first within a
// head.  When every XCD's contiguous slice of the list holds whole heads, the
// slices carry equal work and one head's tiles stay in one XCD's L2: use them.
// Otherwise (say 4 heads over 8 XCDs, where contiguous slices would give half the
// XCDs the long end of a causal triangle and 1.5x the mean work) deal the list in
// rounds of kXcdChunk consecutive items per XCD, the order of the XCDs reversed on
// every other round: neighbouring items still run side by side on one XCD, and
// the alternation evens out the items' decreasing sizes.  Both are bijections on
// [0, nwg).
constexpr int kXcdChunk = 32;  // workgroups resident on one XCD (32 CUs, one each)

__device__ __forceinline__ int xcd_remap(int bid, int nwg, int per_bh) {
  const int x = bid % kNumXcd, s = bid / kNumXcd;
  const int per = nwg / kNumXcd, rem = nwg % kNumXcd;
  if (nwg % (kNumXcd * per_bh) == 0) return x * per + s;
  const int rfull = per / kXcdChunk, r = s / kXcdChunk;
  if (r < rfull) {
    const int chunk = (r & 1) ? (kNumXcd - 1 - x) : x;
    return (r * kNumXcd + chunk) * kXcdChunk + s % kXcdChunk;
  }
  // last, partial round: contiguous slices of what is left
  const int per2 = per - rfull * kXcdChunk;
  return rfull * kNumXcd * kXcdChunk + x * per2 + (x < rem ? x : rem) + (s - rfull * kXcdChunk);
}

}  // namespace ea
