/*
 * ea_attn: blockwise causal attention (forward, backward, LSE merge) for one
 * sequence-parallel rank's share of a long sequence, on AMD MI355X (gfx950),
 * with the rotary position embedding and the fused cross-entropy of the same
 * training step (ea_rope, ea_xent_fwd_bwd, declared further below).
 *
 * The operations follow the EasyContext pages:
 *  - ring attention cuts one sequence over GPUs; each rank attends its local
 *    queries to one rank's key/value share per ring step and combines the
 *    partial results (EasyContext core-technology page, hotelren.com,
 *    section 1 "sequence parallelism");
 *  - the zigzag ring mode interleaves tokens across ranks (EasyContext
 *    training-script walkthrough, mlqm.cn, section on model preparation and
 *    parallel strategies);
 *  - each rank's shard carries its global position ids (EasyContext
 *    "1M tokens with minimal resources" page, cn486.com, usage code);
 *  - the per-block attention is the tiled Flash Attention forward and its
 *    recompute-based backward (hotelren.com page, section 2 "Flash Attention
 *    optimisation").
 * No formula is printed on the pages; the definitions used are stated with
 * each call below.
 *
 * Conventions shared by every call
 * --------------------------------
 *  Layout.  Per-token tensors are [B, S, H, D] row-major with D contiguous:
 *    element (b, i, h, d) lives at ((b * batch_rows + i) * H + h) * D + d,
 *    where batch_rows (>= S) is the row stride between batches, so a
 *    contiguous row sub-range of a larger buffer is passed as a pointer offset
 *    with the parent's batch_rows.  Per-row statistics (LSE, Delta) are
 *    [B, S, H] fp32 at ((b * batch_rows + i) * H + h).
 *  Types.  q, k, v, dout are bf16 (stored as uint16_t).  o is fp32 or bf16
 *    (o_dtype / part_dtype: EA_F32 or EA_BF16).  lse, delta, dq, dk, dv are fp32.
 *  Positions.  Token i of a tensor has a global integer position given by at
 *    most two segments: seg = {start0, len0, start1, len1} (n_seg = 2) or
 *    {start0, len0} (n_seg = 1); rows [0, len0) have positions start0 + i, rows
 *    [len0, len0 + len1) have positions start1 + (i - len0).  The lengths must
 *    sum to the tensor's row count, starts must be >= 0 and every position
 *    < 2^31.  Segment arrays are host memory, read during the call only.
 *  Mask.  EA_MASK_FULL allows every (query, key) pair; EA_MASK_CAUSAL allows
 *    key j for query i iff pos_k(j) <= pos_q(i) (the diagonal is kept).
 *  Scale.  scale multiplies <q_i, k_j>; it must be finite and > 0.
 *  Sizes.  B, H >= 1; D in {64, 128}; S >= 0 and < 2^31.  Each launch is one
 *    grid dimension of at most 2^32 - 1 threads; shapes that would need more
 *    are EA_ERR_SHAPE (attention: B*H*ceil(S/256)*512 threads for queries,
 *    B*H*ceil(Sk/128)*512 for keys, B*H*Sq*D/8 for Delta and the merge).
 *  Alignment.  q, k, v, o, dout and o_part must be 16-byte aligned; fp32
 *    arrays 4-byte aligned.
 *  Ownership.  The caller owns every buffer (device memory, except the
 *    segment arrays).  The library allocates nothing and keeps no state on the
 *    device.  Inputs are read-only; outputs may not overlap inputs (except the
 *    in-place accumulators of ea_lse_merge).
 *  Streams.  `stream` is a hipStream_t (NULL = the default stream).  All work
 *    is enqueued on it and the call returns without synchronising; buffers
 *    must stay alive until the stream passes the call.  Calls that write the
 *    same buffers must be ordered on one stream.
 *  Errors.  Every call returns EA_OK (0) or a positive code.  Argument errors
 *    (EA_ERR_NULL ... EA_ERR_ALIAS) are found on the host before any HIP call
 *    is made, and nothing is enqueued.  EA_ERR_HIP means a launch failed; the
 *    HIP message is then available from ea_last_hip_error() (per thread).  No
 *    call aborts, throws or synchronises the device.
 */
#ifndef EA_ATTN_H
#define EA_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum ea_status {
  EA_OK = 0,
  EA_ERR_NULL = 1,         /* a required pointer is NULL */
  EA_ERR_SHAPE = 2,        /* B, H, S, batch_rows out of range */
  EA_ERR_UNSUPPORTED = 3,  /* D, dtype, mask mode, scale or another parameter not supported */
  EA_ERR_POSITIONS = 4,    /* bad segment count, lengths, starts or positions >= 2^31 */
  EA_ERR_ALIGN = 5,        /* pointer misaligned */
  EA_ERR_ALIAS = 6,        /* an output overlaps an input */
  EA_ERR_HIP = 7           /* a HIP launch failed */
};

enum ea_mask { EA_MASK_FULL = 0, EA_MASK_CAUSAL = 1 };
enum ea_dtype { EA_F32 = 0, EA_BF16 = 1 };

/*
 * Forward.  For every (b, query row i, head h):
 *   S_ij  = scale * <q_i, k_j> for allowed pairs,
 *   LSE_i = ln sum_j exp(S_ij)            (natural log; -inf if no key is allowed),
 *   O_i   = sum_j exp(S_ij - LSE_i) v_j    (0 if no key is allowed).
 * q [B,Sq,H,D], k and v [B,Sk,H,D] (bf16); writes o [B,Sq,H,D] in o_dtype and
 * lse [B,Sq,H] (fp32).  Sq == 0 does nothing; Sk == 0 writes O = 0, LSE = -inf.
 * This is one ring step's partial result when k/v hold one rank's share.
 */
int ea_attn_fwd(const void* q, const void* k, const void* v, void* o, int o_dtype, float* lse,
                int B, int H, int64_t Sq, int64_t Sk, int D,
                int64_t q_batch_rows, int64_t k_batch_rows,
                const int64_t* q_seg, int n_qseg, const int64_t* k_seg, int n_kseg,
                int mask_mode, float scale, void* stream);

/*
 * Forward merged into an accumulator: the partial result of this call (O_part,
 * LSE_part as ea_attn_fwd defines them) is combined into the fp32 accumulator
 * (o_acc, lse_acc) exactly as ea_lse_merge combines a stored partial, in the
 * same launch, so a ring step's partial never goes through memory (the ring
 * combines one partial per visited share: hotelren.com page, section 1).
 * o_acc [B,Sq,H,D] and lse_acc [B,Sq,H] are fp32, read and written in place
 * (same layout and row stride q_batch_rows as q); every other argument is as
 * for ea_attn_fwd.  A row with no allowed key in this call leaves its
 * accumulator unchanged (both -inf gives (0, -inf)), so Sk == 0 changes
 * nothing but such rows.  o_acc and lse_acc must not overlap q, k, v or each
 * other.  Results equal ea_attn_fwd into a separate fp32 partial followed by
 * ea_lse_merge, up to the order of rounding.
 */
int ea_attn_fwd_merge(const void* q, const void* k, const void* v, float* o_acc, float* lse_acc,
                      int B, int H, int64_t Sq, int64_t Sk, int D,
                      int64_t q_batch_rows, int64_t k_batch_rows,
                      const int64_t* q_seg, int n_qseg, const int64_t* k_seg, int n_kseg,
                      int mask_mode, float scale, void* stream);

/*
 * Backward by recomputation from the saved statistics (the recompute-and-tile
 * gradient of the hotelren.com page, section 2).  With P_ij =
 * exp(scale*<q_i,k_j> - LSE_i) on allowed pairs (0 elsewhere):
 *   Delta_i = <dout_i, o_i>
 *   dS_ij   = P_ij (<dout_i, v_j> - Delta_i)
 *   dq_i   += scale * sum_j dS_ij k_j
 *   dk_j   += scale * sum_i dS_ij q_i
 *   dv_j   += sum_i P_ij dout_i
 * dq [B,Sq,H,D], dk and dv [B,Sk,H,D] are fp32 and ACCUMULATED (+=): zero them
 * before the first call.  lse and o must be the FINAL statistics of the query
 * rows over all keys they attend to (for a ring: the merged result), so that
 * the per-step calls sum to the gradient of the whole attention.
 * delta [B,Sq,H] fp32: if delta_ready == 0 the call first computes Delta from
 * o and dout into it; otherwise it is read as given (compute it once per ring,
 * then pass delta_ready = 1).  Rows whose lse is -inf contribute nothing.
 * Sq == 0 or Sk == 0 leaves the accumulators unchanged (Delta is still
 * written when Sq > 0 and delta_ready == 0).
 */
int ea_attn_bwd(const void* q, const void* k, const void* v, const void* o, int o_dtype,
                const void* dout, const float* lse, float* delta, int delta_ready,
                float* dq, float* dk, float* dv,
                int B, int H, int64_t Sq, int64_t Sk, int D,
                int64_t q_batch_rows, int64_t k_batch_rows,
                const int64_t* q_seg, int n_qseg, const int64_t* k_seg, int n_kseg,
                int mask_mode, float scale, void* stream);

/*
 * Forward and backward with the rotary position embedding fused in (the
 * rotary base that the pages raise for long contexts: hotelren.com page,
 * further optimisations; kwkr.cn ZeRO-3 offload page, training script
 * rope-theta and advanced optimisation item 2; cn486.com page, training
 * strategy).  The rotation is the one ea_rope applies (declared below): dims k
 * and k + D/2 of a row at position p turn by p * theta^(-2k/D), fp64 angles,
 * fp32 arithmetic, one rounding to bf16.  0 < theta finite, else
 * EA_ERR_UNSUPPORTED.
 *
 * ea_attn_fwd_rope: q is the UNROTATED query [B,Sq,H,D] bf16; each row is
 * turned by the angles of its position (from q_seg) in registers, right after
 * it is loaded, and the turned rows are used for the scores.  k must already
 * be rotated by its own positions (ea_rope with k_seg).  q_rot (optional, NULL
 * for none): [B,Sq,H,D] bf16 with q's layout and q_batch_rows, 16-byte aligned,
 * overlapping no other argument; receives the turned query rows, bit for bit
 * what ea_rope would write, for the backward.  merge = 0 writes o (o_dtype) and
 * lse like ea_attn_fwd; merge = 1 merges into the fp32 accumulator (o, lse) like
 * ea_attn_fwd_merge (o_dtype must then be EA_F32).  Other arguments, results
 * and errors as for those calls.
 */
int ea_attn_fwd_rope(const void* q, const void* k, const void* v, void* o, int o_dtype, float* lse, void* q_rot,
                     int merge, int B, int H, int64_t Sq, int64_t Sk, int D,
                     int64_t q_batch_rows, int64_t k_batch_rows,
                     const int64_t* q_seg, int n_qseg, const int64_t* k_seg, int n_kseg,
                     int mask_mode, float scale, double theta, void* stream);

/*
 * ea_attn_bwd_rope: the backward of attention over rotated rows, returning the
 * gradients with respect to the UNROTATED q and k.  q and k are the ROTATED
 * rows the forward used (q_rot of ea_attn_fwd_rope, k rotated by ea_rope).
 * The call computes dQ and dK of the rotated rows exactly as ea_attn_bwd does,
 * then turns each row's contribution back by minus its angle (queries by
 * q_seg, keys by k_seg) before adding it into dq and dk; dv and delta are as
 * for ea_attn_bwd.  The rotation is linear, so contributions accumulated over
 * several calls (a ring's steps) sum to the gradient of the unrotated inputs.
 * Other arguments, results and errors as for ea_attn_bwd.
 */
int ea_attn_bwd_rope(const void* q, const void* k, const void* v, const void* o, int o_dtype,
                     const void* dout, const float* lse, float* delta, int delta_ready,
                     float* dq, float* dk, float* dv,
                     int B, int H, int64_t Sq, int64_t Sk, int D,
                     int64_t q_batch_rows, int64_t k_batch_rows,
                     const int64_t* q_seg, int n_qseg, const int64_t* k_seg, int n_kseg,
                     int mask_mode, float scale, double theta, void* stream);

/*
 * In-place LSE merge of a partial result over a disjoint key set into an
 * accumulator (ring attention combines one step's partial per rank visited;
 * hotelren.com page, section 1 "sequence parallelism"):
 *   L   = ln(exp(lse_acc) + exp(lse_part))
 *   o_acc = exp(lse_acc - L) * o_acc + exp(lse_part - L) * o_part,  lse_acc = L.
 * A side whose LSE is -inf contributes nothing; both -inf gives (0, -inf).
 * o_acc [B,Sq,H,D] fp32, lse_acc [B,Sq,H]; o_part in part_dtype, lse_part fp32;
 * all with row stride q_batch_rows between batches.
 */
int ea_lse_merge(float* o_acc, float* lse_acc, const void* o_part, int part_dtype,
                 const float* lse_part, int B, int H, int64_t Sq, int D,
                 int64_t q_batch_rows, void* stream);

/*
 * Fused cross-entropy over vocabulary logits, forward and backward, with the
 * gradient written in place over the logits (the fused cross-entropy kernel
 * with in-place backward of the training step: kwkr.cn ZeRO-3 offload page,
 * section on advanced optimisation combined with other techniques, item 1;
 * cn486.com page, summary of the training script's technology stack).  For every row i of logits [rows, vocab] (row i starts at
 * element i * row_stride) with label y_i:
 *   lse_i  = ln sum_j exp(x_ij)                         (fp32 [rows])
 *   loss_i = lse_i - x_{i,y_i}                          (fp32 [rows])
 *   x_ij  <- grad_scale * (exp(x_ij - lse_i) - [j == y_i])
 * Rows with y_i == ignore_index get loss 0 and gradient 0 (lse is still
 * written).  Any other label outside [0, vocab) gives loss NaN and a NaN
 * gradient row.  logits are bf16 or fp32 (dtype EA_BF16 / EA_F32; the gradient
 * is rounded to nearest even into bf16); labels are int64 on the device.  For a
 * mean over the rows that are not ignored pass grad_scale = 1 / that count.
 * Alignment: logits to their element size (any row_stride; rows that start
 * on 16 bytes are read and written in 16-byte pieces only), labels 8, loss and
 * lse 4.  Sizes: 0 <= rows < 2^23 (one 512-thread workgroup per row),
 * 1 <= vocab <= row_stride, vocab < 2^31.  loss, lse and labels must not overlap the logits or each
 * other.  rows == 0 does nothing.  Enqueued on `stream` like the calls above.
 */
int ea_xent_fwd_bwd(void* logits, int dtype, const int64_t* labels, float* loss, float* lse, int64_t rows,
                    int64_t vocab, int64_t row_stride, int64_t ignore_index, float grad_scale, void* stream);

/*
 * Rotary position embedding by global position (the rotary base that the
 * pages raise for long contexts: hotelren.com page, further optimisations;
 * kwkr.cn ZeRO-3 offload page, training script rope-theta and advanced
 * optimisation item 2; cn486.com page, training strategy).  Llama
 * "rotate-half" convention: for each row of x [B, S, H, D] at position p (from
 * seg, as for ea_attn_fwd) and k = 0 .. D/2-1, with phi = p * theta^(-2k/D),
 *   y_k       = x_k cos(phi) - x_{k+D/2} sin(phi)
 *   y_{k+D/2} = x_{k+D/2} cos(phi) + x_k sin(phi)
 * inverse = 1 applies the transpose (phi -> -phi): it turns the gradient with
 * respect to rotated rows into the gradient with respect to the unrotated ones
 * (dQ, dK of ea_attn_bwd on rotated Q, K).  Angles are formed in fp64 (exact
 * for positions up to 2^31), the rotation in fp32, one rounding to the output.
 * x and y: dtype EA_BF16 or EA_F32 (both), same layout and batch stride
 * batch_rows * H * D elements, 16-byte aligned; y == x rotates in place,
 * otherwise they must not overlap.  D in {64, 128}; 0 < theta finite;
 * B * S < 2^26 (64 threads per token row).  S == 0 does nothing.  Enqueued on `stream` like the calls above.
 */
int ea_rope(const void* x, void* y, int dtype, int B, int H, int64_t S, int D, int64_t batch_rows,
            const int64_t* seg, int n_seg, double theta, int inverse, void* stream);

/*
 * Host-only helper (no HIP call): position segments of one rank's share in a
 * zigzag ring.  The sequence of s_total tokens is cut into 2*world equal
 * chunks of C tokens; rank r holds chunk r followed by chunk 2*world-1-r
 * (reading of the mlqm.cn walkthrough's zigzag mode: interleaving an early and
 * a late chunk balances causal work across ranks).  Writes
 * seg_out[4] = {r*C, C, (2*world-1-r)*C, C}.  Returns EA_ERR_POSITIONS if
 * s_total is not a positive multiple of 2*world, rank is out of range, or a
 * position would reach 2^31; EA_ERR_NULL for a NULL seg_out.
 */
int ea_zigzag_segments(int64_t s_total, int world, int rank, int64_t* seg_out);

/* Host-only helper: the rank whose key/value share rank `rank` holds at ring
 * step `step` of `world` ranks: (rank - step) mod world.  Returns -1 for
 * out-of-range arguments. */
int ea_ring_source(int rank, int step, int world);

/*
 * Per-kernel timing (diagnostics).  Between ea_profile_begin() and
 * ea_profile_end() every kernel the library launches (on any stream) is
 * bracketed by a pair of HIP events recorded on its stream.  Recording adds
 * two event records per launch and no synchronisation.  ea_profile_query()
 * waits for the recorded events of one kernel kind and returns the summed
 * device time in milliseconds and the number of launches since the last
 * ea_profile_begin().  Kernel kinds are the EA_KERNEL_* values;
 * ea_kernel_name() gives their names.  Returns EA_OK, EA_ERR_UNSUPPORTED for a
 * bad kind, EA_ERR_NULL for NULL outputs, or EA_ERR_HIP.  Profiling state is
 * process-wide and guarded by a lock.
 */
enum ea_kernel {
  EA_KERNEL_FWD = 0,
  EA_KERNEL_BWD_DELTA = 1,
  EA_KERNEL_BWD_DKDV = 2,
  EA_KERNEL_BWD_DQ = 3,
  EA_KERNEL_LSE_MERGE = 4,
  EA_KERNEL_XENT = 5,
  EA_KERNEL_ROPE = 6,
  EA_KERNEL_COUNT = 7
};
int ea_profile_begin(void);
int ea_profile_end(void);
int ea_profile_query(int kernel, double* total_ms, int64_t* launches);
const char* ea_kernel_name(int kernel);

const char* ea_strerror(int status);
/* Text of the last HIP error seen by an EA_ERR_HIP return on this thread. */
const char* ea_last_hip_error(void);
/* Library version, major * 10000 + minor * 100 + patch. */
int ea_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EA_ATTN_H */
