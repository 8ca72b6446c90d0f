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
    vp, i32, i64, f32, f64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_double
    pi64 = ctypes.POINTER(ctypes.c_int64)
    L.ea_attn_fwd.argtypes = [vp, vp, vp, vp, i32, vp, i32, i32, i64, i64, i32, i64, i64,
                              pi64, i32, pi64, i32, i32, f32, vp]
    L.ea_attn_fwd.restype = i32
    L.ea_attn_fwd_merge.argtypes = [vp, vp, vp, vp, vp, i32, i32, i64, i64, i32, i64, i64,
                                    pi64, i32, pi64, i32, i32, f32, vp]
    L.ea_attn_fwd_merge.restype = i32
    L.ea_attn_fwd_rope.argtypes = [vp, vp, vp, vp, i32, vp, vp, i32, i32, i32, i64, i64, i32, i64, i64,
                                   pi64, i32, pi64, i32, i32, f32, f64, vp]
    L.ea_attn_fwd_rope.restype = i32
    L.ea_attn_bwd.argtypes = [vp, vp, vp, vp, i32, vp, vp, vp, i32, vp, vp, vp, i32, i32, i64, i64, i32,
                              i64, i64, pi64, i32, pi64, i32, i32, f32, vp]
    L.ea_attn_bwd.restype = i32
    L.ea_attn_bwd_rope.argtypes = [vp, vp, vp, vp, i32, vp, vp, vp, i32, vp, vp, vp, i32, i32, i64, i64, i32,
                                   i64, i64, pi64, i32, pi64, i32, i32, f32, f64, vp]
    L.ea_attn_bwd_rope.restype = i32
    L.ea_lse_merge.argtypes = [vp, vp, vp, i32, vp, i32, i32, i64, i32, i64, vp]
    L.ea_lse_merge.restype = i32
    L.ea_xent_fwd_bwd.argtypes = [vp, i32, vp, vp, vp, i64, i64, i64, i64, f32, vp]
    L.ea_xent_fwd_bwd.restype = i32
    L.ea_rope.argtypes = [vp, vp, i32, i32, i32, i64, i32, i64, pi64, i32, f64, i32, vp]
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


EXPORTS = ("ea_attn_fwd", "ea_attn_fwd_merge", "ea_attn_fwd_rope", "ea_attn_bwd", "ea_attn_bwd_rope",
           "ea_lse_merge", "ea_xent_fwd_bwd", "ea_rope", "ea_zigzag_segments", "ea_ring_source",
           "ea_strerror", "ea_last_hip_error", "ea_version", "ea_profile_begin", "ea_profile_end",
           "ea_profile_query", "ea_kernel_name")

KERNELS = ("fwd", "bwd_delta", "bwd_dkdv", "bwd_dq", "lse_merge", "xent", "rope")


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


def _dtype_is(name, t, *dtypes):
    if t.dtype not in dtypes:
        raise ValueError(f"{name} must be {' or '.join(str(d) for d in dtypes)}, got {t.dtype}")


def _on_device(ref, tensors):
    """Every tensor must live on ref's GPU (the kernels dereference these pointers on the device)."""
    for name, t in tensors.items():
        if t is None:
            continue
        if t.device.type != "cuda" or t.device != ref.device:
            raise ValueError(f"{name} is on {t.device}; every tensor of the call must be on one CUDA device "
                             f"({ref.device if ref.device.type == 'cuda' else 'a CUDA device'})")


def _attn_layout(q, k, q_side, k_side, stats):
    """Shapes and row strides of one attention call, checked before anything reaches the library.

    q [B, Sq, H, D] and k [B, Sk, H, D]; every tensor in q_side must have q's shape and batch row stride, every
    one in k_side k's, every one in stats the shape [B, Sq, H] with q's batch row stride.  Returns
    (B, Sq, H, D, Sk, q_batch_rows, k_batch_rows)."""
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be [B, S, H, D]")
    B, sq, H, D = q.shape
    sk = k.shape[1]
    if tuple(k.shape) != (B, sk, H, D):
        raise ValueError(f"k must be [B={B}, Sk, H={H}, D={D}], got {tuple(k.shape)}")
    qbr, kbr = _rows(q, H, D), _rows(k, H, D)
    for side, shape, br in ((q_side, (B, sq, H, D), qbr), (k_side, (B, sk, H, D), kbr)):
        for name, t in side.items():
            if t is None:
                continue
            if tuple(t.shape) != shape:
                raise ValueError(f"{name} must have shape {shape}, got {tuple(t.shape)}")
            if _rows(t, H, D) != br:
                raise ValueError(f"{name} must have the batch row stride of {'q' if br is qbr else 'k'}")
    for name, t in stats.items():
        if tuple(t.shape) != (B, sq, H):
            raise ValueError(f"{name} must have shape {(B, sq, H)}, got {tuple(t.shape)}")
        if _stat_rows(t, H) != qbr:
            raise ValueError(f"{name} must have the batch row stride of q")
    return B, sq, H, D, sk, qbr, kbr


def _fwd_checks(q, k, v, o, lse, o_dtypes, q_rot=None):
    import torch
    bf = torch.bfloat16
    for name, t in (("q", q), ("k", k), ("v", v)):
        _dtype_is(name, t, bf)
    _dtype_is("o", o, *o_dtypes)
    _dtype_is("lse", lse, torch.float32)
    if q_rot is not None:
        _dtype_is("q_rot", q_rot, bf)
    dims = _attn_layout(q, k, {"o": o, "q_rot": q_rot}, {"v": v}, {"lse": lse})
    _on_device(q, {"q": q, "k": k, "v": v, "o": o, "lse": lse, "q_rot": q_rot})
    return dims


def ea_attn_fwd(q, k, v, o, lse, q_seg, k_seg, causal=True, scale=None, stream=None):
    """O and LSE of q against k/v.  Shapes [B,Sq,H,D], [B,Sk,H,D]; o [B,Sq,H,D] (fp32 or bf16); lse [B,Sq,H] fp32."""
    import torch
    B, sq, H, D, sk, qbr, kbr = _fwd_checks(q, k, v, o, lse, (torch.float32, torch.bfloat16))
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
    B, sq, H, D, sk, qbr, kbr = _fwd_checks(q, k, v, o_acc, lse_acc, (torch.float32,))
    scale = D ** -0.5 if scale is None else float(scale)
    qs, nq = _segs(q_seg)
    ks, nk = _segs(k_seg)
    st = lib().ea_attn_fwd_merge(_ptr(q), _ptr(k), _ptr(v), _ptr(o_acc), _ptr(lse_acc), B, H, sq, sk, D,
                                 qbr, kbr, qs, nq, ks, nk, EA_MASK_CAUSAL if causal else EA_MASK_FULL, scale,
                                 _stream(stream))
    _check(st, "ea_attn_fwd_merge")


def ea_attn_fwd_rope(q, k, v, o, lse, q_seg, k_seg, theta, q_rot=None, merge=False, causal=True, scale=None,
                     stream=None):
    """Forward with q UNROTATED (turned by its positions in the kernel) and k already rotated (ea_rope).

    q_rot: optional bf16 [B,Sq,H,D] that receives the turned q for the backward.  merge=True merges into the fp32
    accumulator (o, lse) like ea_attn_fwd_merge; otherwise o (fp32 or bf16) and lse are written."""
    import torch
    dts = (torch.float32,) if merge else (torch.float32, torch.bfloat16)
    B, sq, H, D, sk, qbr, kbr = _fwd_checks(q, k, v, o, lse, dts, q_rot)
    scale = D ** -0.5 if scale is None else float(scale)
    qs, nq = _segs(q_seg)
    ks, nk = _segs(k_seg)
    st = lib().ea_attn_fwd_rope(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _dtype_code(o), _ptr(lse), _ptr(q_rot),
                                1 if merge else 0, B, H, sq, sk, D, qbr, kbr, qs, nq, ks, nk,
                                EA_MASK_CAUSAL if causal else EA_MASK_FULL, scale, float(theta), _stream(stream))
    _check(st, "ea_attn_fwd_rope")


def _bwd_args(q, k, v, o, dout, lse, delta, dq, dk, dv, q_seg, k_seg, causal, scale, delta_ready):
    import torch
    bf, f32 = torch.bfloat16, torch.float32
    for name, t in (("q", q), ("k", k), ("v", v), ("dout", dout)):
        _dtype_is(name, t, bf)
    if o is not None:
        _dtype_is("o", o, f32, bf)
    elif not delta_ready:
        raise ValueError("o is needed unless delta_ready")
    for name, t in (("lse", lse), ("delta", delta), ("dq", dq), ("dk", dk), ("dv", dv)):
        _dtype_is(name, t, f32)
    B, sq, H, D, sk, qbr, kbr = _attn_layout(q, k, {"o": o, "dout": dout, "dq": dq}, {"v": v, "dk": dk, "dv": dv},
                                             {"lse": lse, "delta": delta})
    _on_device(q, {"q": q, "k": k, "v": v, "o": o, "dout": dout, "lse": lse, "delta": delta, "dq": dq, "dk": dk,
                   "dv": dv})
    scale = D ** -0.5 if scale is None else float(scale)
    qs, nq = _segs(q_seg)
    ks, nk = _segs(k_seg)
    return (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _dtype_code(o) if o is not None else EA_F32,
            _ptr(dout), _ptr(lse), _ptr(delta), 1 if delta_ready else 0, _ptr(dq), _ptr(dk),
            _ptr(dv), B, H, sq, sk, D, qbr, kbr, qs, nq, ks, nk,
            EA_MASK_CAUSAL if causal else EA_MASK_FULL, scale)


def ea_attn_bwd(q, k, v, o, dout, lse, delta, dq, dk, dv, q_seg, k_seg, causal=True, scale=None,
                delta_ready=False, stream=None):
    """Accumulates dq, dk, dv (fp32) for the final (o, lse); writes delta unless delta_ready."""
    args = _bwd_args(q, k, v, o, dout, lse, delta, dq, dk, dv, q_seg, k_seg, causal, scale, delta_ready)
    _check(lib().ea_attn_bwd(*args, _stream(stream)), "ea_attn_bwd")


def ea_attn_bwd_rope(q, k, v, o, dout, lse, delta, dq, dk, dv, q_seg, k_seg, theta, causal=True, scale=None,
                     delta_ready=False, stream=None):
    """ea_attn_bwd on ROTATED q, k (q_rot of ea_attn_fwd_rope, k from ea_rope); dq and dk accumulate the
    gradients with respect to the unrotated rows."""
    args = _bwd_args(q, k, v, o, dout, lse, delta, dq, dk, dv, q_seg, k_seg, causal, scale, delta_ready)
    _check(lib().ea_attn_bwd_rope(*args, float(theta), _stream(stream)), "ea_attn_bwd_rope")


def ea_lse_merge(o_acc, lse_acc, o_part, lse_part, stream=None):
    """In place: (o_acc, lse_acc) <- merge with (o_part, lse_part).  o_acc fp32 [B,Sq,H,D], o_part fp32 or bf16
    of the same shape, lse_acc and lse_part fp32 [B,Sq,H]."""
    import torch
    _dtype_is("o_acc", o_acc, torch.float32)
    _dtype_is("o_part", o_part, torch.float32, torch.bfloat16)
    _dtype_is("lse_acc", lse_acc, torch.float32)
    _dtype_is("lse_part", lse_part, torch.float32)
    if o_acc.dim() != 4:
        raise ValueError("o_acc must be [B, S, H, D]")
    B, sq, H, D = o_acc.shape
    _attn_layout(o_acc, o_acc, {"o_part": o_part}, {}, {"lse_acc": lse_acc, "lse_part": lse_part})
    _on_device(o_acc, {"o_acc": o_acc, "lse_acc": lse_acc, "o_part": o_part, "lse_part": lse_part})
    qbr = _rows(o_acc, H, D)
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
    _dtype_is("logits", logits, torch.float32, torch.bfloat16)
    for t, dt, name in ((labels, torch.int64, "labels"), (loss, torch.float32, "loss"), (lse, torch.float32, "lse")):
        if t.dtype != dt or t.dim() != 1 or t.shape[0] != rows or (rows > 1 and t.stride(0) != 1):
            raise ValueError(f"{name} must be a contiguous {dt} vector of {rows} rows")
    _on_device(logits, {"logits": logits, "labels": labels, "loss": loss, "lse": lse})
    st = lib().ea_xent_fwd_bwd(_ptr(logits), _dtype_code(logits), _ptr(labels), _ptr(loss), _ptr(lse), rows,
                               vocab, row_stride, int(ignore_index), float(grad_scale), _stream(stream))
    _check(st, "ea_xent_fwd_bwd")


def ea_rope(x, y, seg, theta, inverse=False, stream=None):
    """Rotary embedding of x [B, S, H, D] (bf16 or fp32) by the positions of seg into y (same shape, dtype and
    batch stride; y may be x).  inverse=True applies the transpose (for gradients)."""
    import torch
    if x.dim() != 4 or y.shape != x.shape or y.dtype != x.dtype:
        raise ValueError("x and y must be [B, S, H, D] tensors of one shape and dtype")
    _dtype_is("x", x, torch.float32, torch.bfloat16)
    B, S, H, D = x.shape
    rows = _rows(x, H, D)
    if _rows(y, H, D) != rows:
        raise ValueError("x and y must have the same batch stride")
    _on_device(x, {"x": x, "y": y})
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
