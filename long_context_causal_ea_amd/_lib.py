"""ctypes binding of libea_attn.so (argument marshalling only).

Every entry point of include/ea_attn.h is exposed under its C name.  The
wrappers take torch tensors laid out [B, S, H, D] (D contiguous; any row
sub-range view of a larger buffer is fine), read their pointers, shapes and
batch row strides, and pass them through.  All computation happens in the HIP
library; if it is missing the first call raises.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("EA_LIB", os.path.join(HERE, "libea_attn.so"))

EA_OK = 0
EA_MASK_FULL, EA_MASK_CAUSAL = 0, 1
EA_F32, EA_BF16 = 0, 1

_lib = None


class EaError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str = ""):
        self.status = status
        msg = f"{where}: {strerror(status)} (status {status})"
        if detail:
            msg += f": {detail}"
        super().__init__(msg)


def lib():
    """Load the HIP library once.  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"HIP library not found at {LIB_PATH}; build it with `python -m long_context_causal_ea_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
    pi64 = ctypes.POINTER(ctypes.c_int64)
    L.ea_attn_fwd.argtypes = [vp, vp, vp, vp, i32, vp, i32, i32, i64, i64, i32, i64, i64,
                              pi64, i32, pi64, i32, i32, f32, vp]
    L.ea_attn_fwd.restype = i32
    L.ea_attn_fwd_merge.argtypes = [vp, vp, vp, vp, vp, i32, i32, i64, i64, i32, i64, i64,
                                    pi64, i32, pi64, i32, i32, f32, vp]
    L.ea_attn_fwd_merge.restype = i32
    L.ea_attn_bwd.argtypes = [vp, vp, vp, vp, i32, vp, vp, vp, i32, vp, vp, vp, i32, i32, i64, i64, i32,
                              i64, i64, pi64, i32, pi64, i32, i32, f32, vp]
    L.ea_attn_bwd.restype = i32
    L.ea_attn_bwd_ws.argtypes = [vp, vp, vp, vp, i32, vp, vp, vp, i32, vp, vp, vp, i32, i32, i64, i64, i32,
                                 i64, i64, pi64, i32, pi64, i32, i32, f32, vp, i64, vp]
    L.ea_attn_bwd_ws.restype = i32
    L.ea_attn_bwd_ws_bytes.argtypes = [i64, i64, pi64, i32, pi64, i32, i32, pi64]
    L.ea_attn_bwd_ws_bytes.restype = i32
    L.ea_lse_merge.argtypes = [vp, vp, vp, i32, vp, i32, i32, i64, i32, i64, vp]
    L.ea_lse_merge.restype = i32
    L.ea_xent_fwd_bwd.argtypes = [vp, i32, vp, vp, vp, i64, i64, i64, i64, f32, vp]
    L.ea_xent_fwd_bwd.restype = i32
    L.ea_rope.argtypes = [vp, vp, i32, i32, i32, i64, i32, i64, pi64, i32, ctypes.c_double, i32, vp]
    L.ea_rope.restype = i32
    L.ea_zigzag_segments.argtypes = [i64, i32, i32, pi64]
    L.ea_zigzag_segments.restype = i32
    L.ea_ring_source.argtypes = [i32, i32, i32]
    L.ea_ring_source.restype = i32
    L.ea_strerror.argtypes = [i32]
    L.ea_strerror.restype = ctypes.c_char_p
    L.ea_last_hip_error.argtypes = []
    L.ea_last_hip_error.restype = ctypes.c_char_p
    L.ea_version.argtypes = []
    L.ea_version.restype = i32
    L.ea_profile_begin.argtypes = []
    L.ea_profile_begin.restype = i32
    L.ea_profile_end.argtypes = []
    L.ea_profile_end.restype = i32
    L.ea_profile_query.argtypes = [i32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
    L.ea_profile_query.restype = i32
    L.ea_kernel_name.argtypes = [i32]
    L.ea_kernel_name.restype = ctypes.c_char_p
    _lib = L
    return L


EXPORTS = ("ea_attn_fwd", "ea_attn_fwd_merge", "ea_attn_bwd", "ea_attn_bwd_ws", "ea_attn_bwd_ws_bytes", "ea_lse_merge", "ea_xent_fwd_bwd", "ea_rope", "ea_zigzag_segments",
           "ea_ring_source",
           "ea_strerror", "ea_last_hip_error", "ea_version", "ea_profile_begin", "ea_profile_end",
           "ea_profile_query", "ea_kernel_name")

KERNELS = ("fwd", "bwd_delta", "bwd_dkdv", "bwd_dq", "lse_merge", "xent", "rope", "bwd_dq_panel")


def strerror(status: int) -> str:
    return lib().ea_strerror(int(status)).decode()


def ea_version() -> int:
    return int(lib().ea_version())


def _check(status: int, where: str):
    if status != EA_OK:
        detail = lib().ea_last_hip_error().decode() if status == 7 else ""
        raise EaError(status, where, detail)


def _segs(seg):
    seg = [int(x) for x in seg]
    if len(seg) not in (2, 4):
        raise ValueError("segments are (start, len) or (start0, len0, start1, len1)")
    arr = (ctypes.c_int64 * len(seg))(*seg)
    return arr, len(seg) // 2


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _rows(t, H, D):
    """Batch row stride of a [B, S, H, D] view (rows must be H*D elements apart)."""
    if t.dim() != 4 or t.shape[2] != H or t.shape[3] != D:
        raise ValueError(f"expected [B, S, {H}, {D}], got {tuple(t.shape)}")
    if t.stride(3) != 1 or t.stride(2) != D or (t.shape[1] > 1 and t.stride(1) != H * D):
        raise ValueError("rows of a [B, S, H, D] tensor must be contiguous")
    if t.shape[0] > 1 and t.stride(0) % (H * D) != 0:
        raise ValueError("batch stride must be a whole number of rows")
    return t.stride(0) // (H * D) if t.shape[0] > 1 else t.shape[1]


def _stat_rows(t, H):
    if t.dim() != 3 or t.shape[2] != H or t.stride(2) != 1 or (t.shape[1] > 1 and t.stride(1) != H):
        raise ValueError("statistics must be [B, S, H] with contiguous rows")
    return t.stride(0) // H if t.shape[0] > 1 else t.shape[1]


def _dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return EA_F32
    if t.dtype == torch.bfloat16:
        return EA_BF16
    raise ValueError(f"unsupported dtype {t.dtype}")


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _require_bf16(*ts):
    import torch
    for t in ts:
        if t is not None and t.dtype != torch.bfloat16:
            raise ValueError("q, k, v and dout must be bfloat16")


def ea_attn_fwd(q, k, v, o, lse, q_seg, k_seg, causal=True, scale=None, stream=None):
    """O and LSE of q against k/v.  Shapes [B,Sq,H,D], [B,Sk,H,D]; o [B,Sq,H,D]; lse [B,Sq,H]."""
    _require_bf16(q, k, v)
    B, sq, H, D = q.shape
    sk = k.shape[1]
    qbr, kbr = _rows(q, H, D), _rows(k, H, D)
    if _rows(v, H, D) != kbr or _rows(o, H, D) != qbr or _stat_rows(lse, H) != qbr or v.shape[1] != sk:
        raise ValueError("q/o/lse and k/v must share shapes and batch row strides")
    scale = D ** -0.5 if scale is None else float(scale)
    qs, nq = _segs(q_seg)
    ks, nk = _segs(k_seg)
    st = lib().ea_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _dtype_code(o), _ptr(lse), B, H, sq, sk, D,
                           qbr, kbr, qs, nq, ks, nk, EA_MASK_CAUSAL if causal else EA_MASK_FULL, scale,
                           _stream(stream))
    _check(st, "ea_attn_fwd")


def ea_attn_fwd_merge(q, k, v, o_acc, lse_acc, q_seg, k_seg, causal=True, scale=None, stream=None):
    """Forward of q against k/v merged in place into the fp32 accumulator (o_acc [B,Sq,H,D], lse_acc [B,Sq,H])."""
    import torch
    _require_bf16(q, k, v)
    if o_acc.dtype != torch.float32 or lse_acc.dtype != torch.float32:
        raise TypeError("o_acc and lse_acc must be float32")
    B, sq, H, D = q.shape
    sk = k.shape[1]
    qbr, kbr = _rows(q, H, D), _rows(k, H, D)
    if _rows(v, H, D) != kbr or _rows(o_acc, H, D) != qbr or _stat_rows(lse_acc, H) != qbr or v.shape[1] != sk:
        raise ValueError("q/o_acc/lse_acc and k/v must share shapes and batch row strides")
    scale = D ** -0.5 if scale is None else float(scale)
    qs, nq = _segs(q_seg)
    ks, nk = _segs(k_seg)
    st = lib().ea_attn_fwd_merge(_ptr(q), _ptr(k), _ptr(v), _ptr(o_acc), _ptr(lse_acc), B, H, sq, sk, D,
                                 qbr, kbr, qs, nq, ks, nk, EA_MASK_CAUSAL if causal else EA_MASK_FULL, scale,
                                 _stream(stream))
    _check(st, "ea_attn_fwd_merge")


def ea_attn_bwd(q, k, v, o, dout, lse, delta, dq, dk, dv, q_seg, k_seg, causal=True, scale=None,
                delta_ready=False, stream=None, workspace=None):
    """Accumulates dq, dk, dv (fp32) for the final (o, lse); writes delta unless delta_ready.

    workspace: None recomputes the scores for dq (``ea_attn_bwd``); a device tensor (any dtype, contiguous)
    keeps the bf16 dS panel there and computes dq from it (``ea_attn_bwd_ws``; size per (batch, head) from
    ``ea_attn_bwd_ws_bytes``)."""
    _require_bf16(q, k, v, dout)
    B, sq, H, D = q.shape
    sk = k.shape[1]
    qbr, kbr = _rows(q, H, D), _rows(k, H, D)
    for t, r in ((dout, qbr), (dq, qbr), (v, kbr), (dk, kbr), (dv, kbr)):
        if _rows(t, H, D) != r:
            raise ValueError("inconsistent batch row strides")
    if o is not None and _rows(o, H, D) != qbr:
        raise ValueError("inconsistent batch row strides")
    if _stat_rows(lse, H) != qbr or _stat_rows(delta, H) != qbr:
        raise ValueError("inconsistent statistics row strides")
    scale = D ** -0.5 if scale is None else float(scale)
    qs, nq = _segs(q_seg)
    ks, nk = _segs(k_seg)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _dtype_code(o) if o is not None else EA_F32,
            _ptr(dout), _ptr(lse), _ptr(delta), 1 if delta_ready else 0, _ptr(dq), _ptr(dk),
            _ptr(dv), B, H, sq, sk, D, qbr, kbr, qs, nq, ks, nk,
            EA_MASK_CAUSAL if causal else EA_MASK_FULL, scale)
    if workspace is None:
        _check(lib().ea_attn_bwd(*args, _stream(stream)), "ea_attn_bwd")
        return
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib().ea_attn_bwd_ws(*args, _ptr(workspace), nbytes, _stream(stream)), "ea_attn_bwd_ws")


def ea_attn_bwd_ws_bytes(sq: int, sk: int, q_seg, k_seg, causal=True) -> int:
    """Bytes of dS panel one (batch, head) of ``ea_attn_bwd_ws`` needs."""
    qs, nq = _segs(q_seg)
    ks, nk = _segs(k_seg)
    out = ctypes.c_int64(0)
    st = lib().ea_attn_bwd_ws_bytes(int(sq), int(sk), qs, nq, ks, nk, EA_MASK_CAUSAL if causal else EA_MASK_FULL,
                                    ctypes.byref(out))
    _check(st, "ea_attn_bwd_ws_bytes")
    return int(out.value)


def ea_lse_merge(o_acc, lse_acc, o_part, lse_part, stream=None):
    B, sq, H, D = o_acc.shape
    qbr = _rows(o_acc, H, D)
    if _rows(o_part, H, D) != qbr or _stat_rows(lse_acc, H) != qbr or _stat_rows(lse_part, H) != qbr:
        raise ValueError("inconsistent batch row strides")
    st = lib().ea_lse_merge(_ptr(o_acc), _ptr(lse_acc), _ptr(o_part), _dtype_code(o_part), _ptr(lse_part),
                            B, H, sq, D, qbr, _stream(stream))
    _check(st, "ea_lse_merge")


def ea_xent_fwd_bwd(logits, labels, loss, lse, grad_scale=1.0, ignore_index=-100, stream=None):
    """Cross-entropy of each row of logits [rows, vocab] (bf16 or fp32, rows contiguous) against int64
    labels [rows]; writes loss and lse (fp32 [rows]) and overwrites logits with the gradient."""
    import torch
    if logits.dim() != 2 or logits.stride(1) != 1:
        raise ValueError("logits must be [rows, vocab] with contiguous rows")
    rows, vocab = logits.shape
    row_stride = logits.stride(0) if rows > 1 else vocab
    for t, dt, name in ((labels, torch.int64, "labels"), (loss, torch.float32, "loss"), (lse, torch.float32, "lse")):
        if t.dtype != dt or t.dim() != 1 or t.shape[0] != rows or (rows > 1 and t.stride(0) != 1):
            raise ValueError(f"{name} must be a contiguous {dt} vector of {rows} rows")
    st = lib().ea_xent_fwd_bwd(_ptr(logits), _dtype_code(logits), _ptr(labels), _ptr(loss), _ptr(lse), rows,
                               vocab, row_stride, int(ignore_index), float(grad_scale), _stream(stream))
    _check(st, "ea_xent_fwd_bwd")


def ea_rope(x, y, seg, theta, inverse=False, stream=None):
    """Rotary embedding of x [B, S, H, D] (bf16 or fp32) by the positions of seg into y (same shape, dtype and
    batch stride; y may be x).  inverse=True applies the transpose (for gradients)."""
    if x.dim() != 4 or y.shape != x.shape or y.dtype != x.dtype:
        raise ValueError("x and y must be [B, S, H, D] tensors of one shape and dtype")
    B, S, H, D = x.shape
    rows = _rows(x, H, D)
    if _rows(y, H, D) != rows:
        raise ValueError("x and y must have the same batch stride")
    sg, ns = _segs(seg)
    st = lib().ea_rope(_ptr(x), _ptr(y), _dtype_code(x), B, H, S, D, rows, sg, ns, float(theta), int(bool(inverse)),
                       _stream(stream))
    _check(st, "ea_rope")


def ea_zigzag_segments(s_total: int, world: int, rank: int):
    out = (ctypes.c_int64 * 4)()
    _check(lib().ea_zigzag_segments(int(s_total), int(world), int(rank), out), "ea_zigzag_segments")
    return [int(x) for x in out]


def ea_ring_source(rank: int, step: int, world: int) -> int:
    r = int(lib().ea_ring_source(int(rank), int(step), int(world)))
    if r < 0:
        raise ValueError("bad ring arguments")
    return r


def ea_profile_begin():
    _check(lib().ea_profile_begin(), "ea_profile_begin")


def ea_profile_end():
    _check(lib().ea_profile_end(), "ea_profile_end")


def ea_profile_query(kernel):
    """(total device ms, launches) of one kernel kind since ea_profile_begin(); waits for its events."""
    kid = KERNELS.index(kernel) if isinstance(kernel, str) else int(kernel)
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    _check(lib().ea_profile_query(kid, ctypes.byref(ms), ctypes.byref(n)), "ea_profile_query")
    return float(ms.value), int(n.value)


def ea_kernel_name(kernel: int) -> str:
    return lib().ea_kernel_name(int(kernel)).decode()
