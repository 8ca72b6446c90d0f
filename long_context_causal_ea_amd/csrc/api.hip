// Public C entry points (declared in include/ea_attn.h): argument validation on
// the host, before any HIP call, then kernel launches on the caller's stream.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "../../include/ea_attn.h"
#include "ea_launch.h"

namespace {

using ea::SegArg;

constexpr int64_t kPosLimit = (int64_t)1 << 31;  // every position and length < 2^31

thread_local char g_hip_msg[256] = "no HIP error";

int hip_fail(hipError_t e) {
  const char* s = hipGetErrorString(e);
  strncpy(g_hip_msg, s ? s : "unknown HIP error", sizeof(g_hip_msg) - 1);
  g_hip_msg[sizeof(g_hip_msg) - 1] = 0;
  return EA_ERR_HIP;
}

// ---- optional per-kernel event timing
struct ProfRec {
  int kernel;
  hipEvent_t a, b;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfRec> g_prof_recs;
std::vector<hipEvent_t> g_prof_pool;

hipEvent_t prof_event() {
  if (!g_prof_pool.empty()) {
    hipEvent_t e = g_prof_pool.back();
    g_prof_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Launch through `fn`, bracketing it with events on `s` while profiling is on.
template <class F>
hipError_t timed_launch(int kernel, hipStream_t s, F fn) {
  std::unique_lock<std::mutex> lk(g_prof_mu);
  if (!g_prof_on) {
    lk.unlock();
    return fn();
  }
  hipEvent_t a = prof_event(), b = prof_event();
  if (a) (void)hipEventRecord(a, s);
  const hipError_t e = fn();
  if (b) (void)hipEventRecord(b, s);
  if (a && b)
    g_prof_recs.push_back(ProfRec{kernel, a, b});
  else {
    if (a) g_prof_pool.push_back(a);
    if (b) g_prof_pool.push_back(b);
  }
  return e;
}

int check_segs(const int64_t* seg, int n, int64_t S, SegArg* out) {
  if (!seg) return EA_ERR_NULL;
  if (n != 1 && n != 2) return EA_ERR_POSITIONS;
  int64_t total = 0;
  for (int s = 0; s < n; ++s) {
    const int64_t st = seg[2 * s], len = seg[2 * s + 1];
    if (st < 0 || len < 0 || st >= kPosLimit || len > kPosLimit - st) return EA_ERR_POSITIONS;
    total += len;
  }
  if (total != S) return EA_ERR_POSITIONS;
  out->s0 = (int)seg[0];
  out->l0 = (int)seg[1];
  out->s1 = n == 2 ? (int)seg[2] : 0;
  out->n = (int)S;
  return EA_OK;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

struct Span {
  uintptr_t lo, hi;  // [lo, hi) bytes; empty if lo == hi
};

Span span_of(const void* p, int B, int64_t batch_rows, int64_t S, int64_t row_elems, int64_t elem_bytes) {
  if (!p || S == 0) return Span{0, 0};
  const int64_t elems = ((int64_t)(B - 1) * batch_rows + S) * row_elems;
  return Span{(uintptr_t)p, (uintptr_t)p + (uintptr_t)(elems * elem_bytes)};
}

bool overlap(const Span& a, const Span& b) {
  if (a.lo == a.hi || b.lo == b.hi) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

// A HIP launch takes at most 2^32 - 1 threads in one grid dimension; every
// launcher here uses one dimension.  Rounded up to whole workgroups.
bool grid_fits(int64_t threads, int64_t block) {
  const int64_t wgs = (threads + block - 1) / block;
  return wgs * block <= (((int64_t)1 << 32) - 1);
}

int check_common(int B, int H, int64_t Sq, int64_t Sk, int D, int64_t qbr, int64_t kbr, int mask_mode,
                 float scale) {
  if (B < 1 || H < 1 || Sq < 0 || Sk < 0 || Sq >= kPosLimit || Sk >= kPosLimit) return EA_ERR_SHAPE;
  if (qbr < Sq || kbr < Sk) return EA_ERR_SHAPE;
  if (qbr >= kPosLimit || kbr >= kPosLimit) return EA_ERR_SHAPE;
  if (D != 64 && D != 128) return EA_ERR_UNSUPPORTED;
  if (mask_mode != EA_MASK_FULL && mask_mode != EA_MASK_CAUSAL) return EA_ERR_UNSUPPORTED;
  if (!(scale > 0.f) || !isfinite(scale)) return EA_ERR_UNSUPPORTED;
  // grids: forward and dq one 512-thread workgroup per 256 query rows per (batch, head), dk/dv one per 128
  // keys, Delta D/8 threads per (row, head)
  const int64_t bh = (int64_t)B * H;
  if (!grid_fits(bh * ((Sq + 255) / 256) * 512, 512) || !grid_fits(bh * ((Sk + 127) / 128) * 512, 512))
    return EA_ERR_SHAPE;
  if (!grid_fits(bh * Sq * (D / 8), 256)) return EA_ERR_SHAPE;
  return EA_OK;
}

bool theta_ok(double theta) { return theta > 0.0 && isfinite(theta); }

void rope_freqs(double theta, int D, double* f) {
  for (int k = 0; k < 64; ++k) f[k] = k < D / 2 ? pow(theta, -2.0 * k / D) : 0.0;
}

}  // namespace

extern "C" {

int ea_version(void) { return 200; }  // 0.2.0

const char* ea_strerror(int status) {
  switch (status) {
    case EA_OK: return "ok";
    case EA_ERR_NULL: return "a required pointer is NULL";
    case EA_ERR_SHAPE: return "B, H, sequence length or batch row stride out of range";
    case EA_ERR_UNSUPPORTED: return "unsupported head dimension, dtype, mask mode, scale or other parameter";
    case EA_ERR_POSITIONS: return "bad position segments (count, lengths, starts, or a position >= 2^31)";
    case EA_ERR_ALIGN: return "pointer misaligned (the alignment each call documents in ea_attn.h)";
    case EA_ERR_ALIAS: return "an output buffer overlaps an input buffer";
    case EA_ERR_HIP: return "a HIP launch failed (see ea_last_hip_error)";
    default: return "unknown status";
  }
}

const char* ea_last_hip_error(void) { return g_hip_msg; }

int ea_profile_begin(void) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (const ProfRec& r : g_prof_recs) {
    g_prof_pool.push_back(r.a);
    g_prof_pool.push_back(r.b);
  }
  g_prof_recs.clear();
  g_prof_on = true;
  return EA_OK;
}

int ea_profile_end(void) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_on = false;
  return EA_OK;
}

int ea_profile_query(int kernel, double* total_ms, int64_t* launches) {
  if (kernel < 0 || kernel >= EA_KERNEL_COUNT) return EA_ERR_UNSUPPORTED;
  if (!total_ms || !launches) return EA_ERR_NULL;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  double sum = 0.0;
  int64_t n = 0;
  for (const ProfRec& r : g_prof_recs) {
    if (r.kernel != kernel) continue;
    hipError_t e = hipEventSynchronize(r.b);
    if (e != hipSuccess) return hip_fail(e);
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, r.a, r.b);
    if (e != hipSuccess) return hip_fail(e);
    sum += ms;
    ++n;
  }
  *total_ms = sum;
  *launches = n;
  return EA_OK;
}

const char* ea_kernel_name(int kernel) {
  switch (kernel) {
    case EA_KERNEL_FWD: return "fwd";
    case EA_KERNEL_BWD_DELTA: return "bwd_delta";
    case EA_KERNEL_BWD_DKDV: return "bwd_dkdv";
    case EA_KERNEL_BWD_DQ: return "bwd_dq";
    case EA_KERNEL_LSE_MERGE: return "lse_merge";
    case EA_KERNEL_XENT: return "xent";
    case EA_KERNEL_ROPE: return "rope";
    default: return "unknown";
  }
}

int ea_ring_source(int rank, int step, int world) {
  if (world < 1 || rank < 0 || rank >= world || step < 0) return -1;
  return (int)(((int64_t)rank - step % world + world) % world);
}

int ea_zigzag_segments(int64_t s_total, int world, int rank, int64_t* seg_out) {
  if (!seg_out) return EA_ERR_NULL;
  if (world < 1 || rank < 0 || rank >= world || s_total <= 0) return EA_ERR_POSITIONS;
  if (s_total % (2 * (int64_t)world) != 0 || s_total > kPosLimit) return EA_ERR_POSITIONS;
  const int64_t C = s_total / (2 * (int64_t)world);
  seg_out[0] = (int64_t)rank * C;
  seg_out[1] = C;
  seg_out[2] = (int64_t)(2 * world - 1 - rank) * C;
  seg_out[3] = C;
  return EA_OK;
}

// rope: 0 none; 1 turn q by the rotary angles of its positions (theta), writing
// the turned rows to q_rot when it is not NULL.
static int attn_fwd(const void* q, const void* k, const void* v, void* o, int o_dtype, float* lse, int B, int H,
                    int64_t Sq, int64_t Sk, int D, int64_t q_batch_rows, int64_t k_batch_rows, const int64_t* q_seg,
                    int n_qseg, const int64_t* k_seg, int n_kseg, int mask_mode, float scale, int merge,
                    int rope, double theta, void* q_rot, void* stream) {
  int st = check_common(B, H, Sq, Sk, D, q_batch_rows, k_batch_rows, mask_mode, scale);
  if (st) return st;
  if (o_dtype != EA_F32 && o_dtype != EA_BF16) return EA_ERR_UNSUPPORTED;
  if (merge != 0 && merge != 1) return EA_ERR_UNSUPPORTED;
  if (merge && o_dtype != EA_F32) return EA_ERR_UNSUPPORTED;
  if (rope && !theta_ok(theta)) return EA_ERR_UNSUPPORTED;
  ea::FwdArgs a;
  if ((st = check_segs(q_seg, n_qseg, Sq, &a.qs))) return st;
  if ((st = check_segs(k_seg, n_kseg, Sk, &a.ks))) return st;
  if (Sq == 0) return EA_OK;
  if (!q || !o || !lse) return EA_ERR_NULL;
  if (Sk > 0 && (!k || !v)) return EA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(o, 16) || !aligned(lse, 4)) return EA_ERR_ALIGN;
  if (Sk > 0 && (!aligned(k, 16) || !aligned(v, 16))) return EA_ERR_ALIGN;
  const int64_t row = (int64_t)H * D;
  const int osz = o_dtype == EA_F32 ? 4 : 2;
  const Span sq = span_of(q, B, q_batch_rows, Sq, row, 2), sk = span_of(k, B, k_batch_rows, Sk, row, 2),
             sv = span_of(v, B, k_batch_rows, Sk, row, 2);
  const Span so = span_of(o, B, q_batch_rows, Sq, row, osz), sl = span_of(lse, B, q_batch_rows, Sq, H, 4);
  for (const Span& out : {so, sl})
    for (const Span& in : {sq, sk, sv})
      if (overlap(out, in)) return EA_ERR_ALIAS;
  if (overlap(so, sl)) return EA_ERR_ALIAS;
  if (rope && q_rot) {
    if (!aligned(q_rot, 16)) return EA_ERR_ALIGN;
    const Span sr = span_of(q_rot, B, q_batch_rows, Sq, row, 2);
    for (const Span& x : {sq, sk, sv, so, sl})
      if (overlap(sr, x)) return EA_ERR_ALIAS;
  }

  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = o;
  a.lse = lse;
  a.B = B;
  a.H = H;
  a.D = D;
  a.Sq = (int)Sq;
  a.Sk = (int)Sk;
  a.q_batch_rows = q_batch_rows;
  a.k_batch_rows = k_batch_rows;
  a.causal = mask_mode == EA_MASK_CAUSAL;
  a.o_bf16 = o_dtype == EA_BF16;
  a.merge = merge;
  a.scale = scale;
  a.rope = rope;
  a.q_rot = rope ? static_cast<uint16_t*>(q_rot) : nullptr;
  rope_freqs(rope ? theta : 1.0, D, a.inv_freq);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = timed_launch(EA_KERNEL_FWD, s, [&] { return ea::launch_fwd(a, s); });
  return e == hipSuccess ? EA_OK : hip_fail(e);
}

int ea_attn_fwd(const void* q, const void* k, const void* v, void* o, int o_dtype, float* lse, int B, int H,
                int64_t Sq, int64_t Sk, int D, int64_t q_batch_rows, int64_t k_batch_rows, const int64_t* q_seg,
                int n_qseg, const int64_t* k_seg, int n_kseg, int mask_mode, float scale, void* stream) {
  return attn_fwd(q, k, v, o, o_dtype, lse, B, H, Sq, Sk, D, q_batch_rows, k_batch_rows, q_seg, n_qseg, k_seg,
                  n_kseg, mask_mode, scale, 0, 0, 0.0, nullptr, stream);
}

int ea_attn_fwd_merge(const void* q, const void* k, const void* v, float* o_acc, float* lse_acc, int B, int H,
                      int64_t Sq, int64_t Sk, int D, int64_t q_batch_rows, int64_t k_batch_rows,
                      const int64_t* q_seg, int n_qseg, const int64_t* k_seg, int n_kseg, int mask_mode,
                      float scale, void* stream) {
  return attn_fwd(q, k, v, o_acc, EA_F32, lse_acc, B, H, Sq, Sk, D, q_batch_rows, k_batch_rows, q_seg, n_qseg,
                  k_seg, n_kseg, mask_mode, scale, 1, 0, 0.0, nullptr, stream);
}

int ea_attn_fwd_rope(const void* q, const void* k, const void* v, void* o, int o_dtype, float* lse, void* q_rot,
                     int merge, int B, int H, int64_t Sq, int64_t Sk, int D, int64_t q_batch_rows,
                     int64_t k_batch_rows, const int64_t* q_seg, int n_qseg, const int64_t* k_seg, int n_kseg,
                     int mask_mode, float scale, double theta, void* stream) {
  return attn_fwd(q, k, v, o, o_dtype, lse, B, H, Sq, Sk, D, q_batch_rows, k_batch_rows, q_seg, n_qseg, k_seg,
                  n_kseg, mask_mode, scale, merge, 1, theta, q_rot, stream);
}

}  // extern "C"

namespace {

// rope: 0 none; 1 q and k are rows turned by their rotary angles (theta), and the
// dq, dk contributions are turned back before they are added.
int attn_bwd(const void* q, const void* k, const void* v, const void* o, int o_dtype, const void* dout,
             const float* lse, float* delta, int delta_ready, float* dq, float* dk, float* dv, int B, int H,
             int64_t Sq, int64_t Sk, int D, int64_t q_batch_rows, int64_t k_batch_rows, const int64_t* q_seg,
             int n_qseg, const int64_t* k_seg, int n_kseg, int mask_mode, float scale, int rope, double theta,
             void* stream) {
  int st = check_common(B, H, Sq, Sk, D, q_batch_rows, k_batch_rows, mask_mode, scale);
  if (st) return st;
  if (o_dtype != EA_F32 && o_dtype != EA_BF16) return EA_ERR_UNSUPPORTED;
  if (rope && !theta_ok(theta)) return EA_ERR_UNSUPPORTED;
  ea::BwdArgs a;
  if ((st = check_segs(q_seg, n_qseg, Sq, &a.qs))) return st;
  if ((st = check_segs(k_seg, n_kseg, Sk, &a.ks))) return st;
  if (Sq == 0) return EA_OK;
  if (!q || !dout || !lse || !delta || !dq) return EA_ERR_NULL;
  if (!delta_ready && !o) return EA_ERR_NULL;
  if (Sk > 0 && (!k || !v || !dk || !dv)) return EA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(dout, 16) || !aligned(dq, 16) || !aligned(lse, 4) || !aligned(delta, 4))
    return EA_ERR_ALIGN;
  if (!delta_ready && !aligned(o, 16)) return EA_ERR_ALIGN;
  if (Sk > 0 && (!aligned(k, 16) || !aligned(v, 16) || !aligned(dk, 16) || !aligned(dv, 16)))
    return EA_ERR_ALIGN;
  const int64_t row = (int64_t)H * D;
  const int osz = o_dtype == EA_F32 ? 4 : 2;
  const Span sq = span_of(q, B, q_batch_rows, Sq, row, 2), sk = span_of(k, B, k_batch_rows, Sk, row, 2),
             sv = span_of(v, B, k_batch_rows, Sk, row, 2), sdo = span_of(dout, B, q_batch_rows, Sq, row, 2),
             sl = span_of(lse, B, q_batch_rows, Sq, H, 4),
             so = delta_ready ? Span{0, 0} : span_of(o, B, q_batch_rows, Sq, row, osz);
  const Span sdl = span_of(delta, B, q_batch_rows, Sq, H, 4), sdq = span_of(dq, B, q_batch_rows, Sq, row, 4),
             sdk = span_of(dk, B, k_batch_rows, Sk, row, 4), sdv = span_of(dv, B, k_batch_rows, Sk, row, 4);
  for (const Span& out : {sdl, sdq, sdk, sdv})
    for (const Span& in : {sq, sk, sv, sdo, sl, so})
      if (overlap(out, in)) return EA_ERR_ALIAS;
  if (overlap(sdq, sdk) || overlap(sdq, sdv) || overlap(sdk, sdv) || overlap(sdl, sdq) || overlap(sdl, sdk) ||
      overlap(sdl, sdv))
    return EA_ERR_ALIAS;

  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = o;
  a.dout = static_cast<const uint16_t*>(dout);
  a.lse = lse;
  a.delta = delta;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.B = B;
  a.H = H;
  a.D = D;
  a.Sq = (int)Sq;
  a.Sk = (int)Sk;
  a.q_batch_rows = q_batch_rows;
  a.k_batch_rows = k_batch_rows;
  a.causal = mask_mode == EA_MASK_CAUSAL;
  a.o_bf16 = o_dtype == EA_BF16;
  a.scale = scale;
  a.Hs = H;
  a.rope = rope;
  rope_freqs(rope ? theta : 1.0, D, a.inv_freq);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (!delta_ready) e = timed_launch(EA_KERNEL_BWD_DELTA, s, [&] { return ea::launch_bwd_delta(a, s); });
  if (e != hipSuccess) return hip_fail(e);
  if (Sk == 0) return EA_OK;
  e = timed_launch(EA_KERNEL_BWD_DKDV, s, [&] { return ea::launch_bwd_dkdv(a, s); });
  if (e != hipSuccess) return hip_fail(e);
  e = timed_launch(EA_KERNEL_BWD_DQ, s, [&] { return ea::launch_bwd_dq(a, s); });
  return e == hipSuccess ? EA_OK : hip_fail(e);
}

}  // namespace

extern "C" {

int ea_attn_bwd(const void* q, const void* k, const void* v, const void* o, int o_dtype, const void* dout,
                const float* lse, float* delta, int delta_ready, float* dq, float* dk, float* dv, int B, int H,
                int64_t Sq, int64_t Sk, int D, int64_t q_batch_rows, int64_t k_batch_rows, const int64_t* q_seg,
                int n_qseg, const int64_t* k_seg, int n_kseg, int mask_mode, float scale, void* stream) {
  return attn_bwd(q, k, v, o, o_dtype, dout, lse, delta, delta_ready, dq, dk, dv, B, H, Sq, Sk, D, q_batch_rows,
                  k_batch_rows, q_seg, n_qseg, k_seg, n_kseg, mask_mode, scale, 0, 0.0, stream);
}

int ea_attn_bwd_rope(const void* q, const void* k, const void* v, const void* o, int o_dtype, const void* dout,
                     const float* lse, float* delta, int delta_ready, float* dq, float* dk, float* dv, int B, int H,
                     int64_t Sq, int64_t Sk, int D, int64_t q_batch_rows, int64_t k_batch_rows,
                     const int64_t* q_seg, int n_qseg, const int64_t* k_seg, int n_kseg, int mask_mode, float scale,
                     double theta, void* stream) {
  return attn_bwd(q, k, v, o, o_dtype, dout, lse, delta, delta_ready, dq, dk, dv, B, H, Sq, Sk, D, q_batch_rows,
                  k_batch_rows, q_seg, n_qseg, k_seg, n_kseg, mask_mode, scale, 1, theta, stream);
}

int ea_lse_merge(float* o_acc, float* lse_acc, const void* o_part, int part_dtype, const float* lse_part, int B,
                 int H, int64_t Sq, int D, int64_t q_batch_rows, void* stream) {
  if (B < 1 || H < 1 || Sq < 0 || Sq >= kPosLimit || q_batch_rows < Sq || q_batch_rows >= kPosLimit)
    return EA_ERR_SHAPE;
  if (D != 64 && D != 128) return EA_ERR_UNSUPPORTED;
  if (part_dtype != EA_F32 && part_dtype != EA_BF16) return EA_ERR_UNSUPPORTED;
  if (!grid_fits((int64_t)B * H * Sq * (D / 8), 256)) return EA_ERR_SHAPE;
  if (Sq == 0) return EA_OK;
  if (!o_acc || !lse_acc || !o_part || !lse_part) return EA_ERR_NULL;
  if (!aligned(o_acc, 16) || !aligned(o_part, 16) || !aligned(lse_acc, 4) || !aligned(lse_part, 4))
    return EA_ERR_ALIGN;
  const int64_t row = (int64_t)H * D;
  const Span sa = span_of(o_acc, B, q_batch_rows, Sq, row, 4), sla = span_of(lse_acc, B, q_batch_rows, Sq, H, 4);
  const Span sp = span_of(o_part, B, q_batch_rows, Sq, row, part_dtype == EA_F32 ? 4 : 2),
             slp = span_of(lse_part, B, q_batch_rows, Sq, H, 4);
  if (overlap(sa, sp) || overlap(sa, slp) || overlap(sla, sp) || overlap(sla, slp) || overlap(sa, sla))
    return EA_ERR_ALIAS;
  ea::MergeArgs a;
  a.o_acc = o_acc;
  a.lse_acc = lse_acc;
  a.o_part = o_part;
  a.lse_part = lse_part;
  a.part_bf16 = part_dtype == EA_BF16;
  a.B = B;
  a.H = H;
  a.D = D;
  a.Sq = (int)Sq;
  a.q_batch_rows = q_batch_rows;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = timed_launch(EA_KERNEL_LSE_MERGE, s, [&] { return ea::launch_merge(a, s); });
  return e == hipSuccess ? EA_OK : hip_fail(e);
}

int ea_xent_fwd_bwd(void* logits, int dtype, const int64_t* labels, float* loss, float* lse, int64_t rows,
                    int64_t vocab, int64_t row_stride, int64_t ignore_index, float grad_scale, void* stream) {
  if (rows < 0 || rows >= kPosLimit || vocab < 1 || vocab >= kPosLimit || row_stride < vocab) return EA_ERR_SHAPE;
  if (!grid_fits(rows * ea::kXentBlock, ea::kXentBlock)) return EA_ERR_SHAPE;  // one workgroup per row
  if (dtype != EA_F32 && dtype != EA_BF16) return EA_ERR_UNSUPPORTED;
  if (!isfinite(grad_scale)) return EA_ERR_UNSUPPORTED;
  if (rows == 0) return EA_OK;
  if (!logits || !labels || !loss || !lse) return EA_ERR_NULL;
  const int esz = dtype == EA_F32 ? 4 : 2;
  if (!aligned(logits, esz) || !aligned(labels, 8) || !aligned(loss, 4) || !aligned(lse, 4))
    return EA_ERR_ALIGN;
  const Span sx = Span{(uintptr_t)logits, (uintptr_t)logits + (uintptr_t)(((rows - 1) * row_stride + vocab) * esz)};
  const Span sy = Span{(uintptr_t)labels, (uintptr_t)labels + (uintptr_t)(rows * 8)};
  const Span sl = Span{(uintptr_t)loss, (uintptr_t)loss + (uintptr_t)(rows * 4)};
  const Span se = Span{(uintptr_t)lse, (uintptr_t)lse + (uintptr_t)(rows * 4)};
  if (overlap(sx, sy) || overlap(sx, sl) || overlap(sx, se) || overlap(sy, sl) || overlap(sy, se) || overlap(sl, se))
    return EA_ERR_ALIAS;
  ea::XentArgs a;
  a.logits = logits;
  a.labels = labels;
  a.loss = loss;
  a.lse = lse;
  a.rows = (long)rows;
  a.row_stride = (long)row_stride;
  a.V = (int)vocab;
  a.ignore_index = (long)ignore_index;
  a.grad_scale = grad_scale;
  a.bf16 = dtype == EA_BF16;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = timed_launch(EA_KERNEL_XENT, s, [&] { return ea::launch_xent(a, s); });
  return e == hipSuccess ? EA_OK : hip_fail(e);
}

int ea_rope(const void* x, void* y, int dtype, int B, int H, int64_t S, int D, int64_t batch_rows,
            const int64_t* seg, int n_seg, double theta, int inverse, void* stream) {
  if (B < 1 || H < 1 || S < 0 || S >= kPosLimit || batch_rows < S || batch_rows >= kPosLimit) return EA_ERR_SHAPE;
  if ((int64_t)B * S >= kPosLimit) return EA_ERR_SHAPE;
  if (!grid_fits((int64_t)B * S * (ea::kRopeBlock / ea::kRopeRowsPerBlock), ea::kRopeBlock)) return EA_ERR_SHAPE;
  if (D != 64 && D != 128) return EA_ERR_UNSUPPORTED;
  if (dtype != EA_F32 && dtype != EA_BF16) return EA_ERR_UNSUPPORTED;
  if (!theta_ok(theta)) return EA_ERR_UNSUPPORTED;
  if (inverse != 0 && inverse != 1) return EA_ERR_UNSUPPORTED;
  ea::RopeArgs a;
  int st = check_segs(seg, n_seg, S, &a.seg);
  if (st) return st;
  if (S == 0) return EA_OK;
  if (!x || !y) return EA_ERR_NULL;
  if (!aligned(x, 16) || !aligned(y, 16)) return EA_ERR_ALIGN;
  const int esz = dtype == EA_F32 ? 4 : 2;
  const Span sx = span_of(x, B, batch_rows, S, (int64_t)H * D, esz), sy = span_of(y, B, batch_rows, S, (int64_t)H * D, esz);
  if (x != y && overlap(sx, sy)) return EA_ERR_ALIAS;
  a.x = x;
  a.y = y;
  a.B = B;
  a.H = H;
  a.S = (int)S;
  a.D = D;
  a.batch_rows = batch_rows;
  a.inverse = inverse;
  a.bf16 = dtype == EA_BF16;
  rope_freqs(theta, D, a.inv_freq);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = timed_launch(EA_KERNEL_ROPE, s, [&] { return ea::launch_rope(a, s); });
  return e == hipSuccess ? EA_OK : hip_fail(e);
}

}  // extern "C"
