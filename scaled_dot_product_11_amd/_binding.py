"""ctypes binding of the gfx950 SDPA library: argument marshalling only.

Every step of the forward runs in the HIP library; PyTorch provides device memory and the
current stream.  There is no fallback of any kind: if the library is missing, or the
tensors are not on a GPU, the call raises.
"""
import ctypes
import math
import os

import torch  # must precede loading the library: it binds to torch's HIP runtime

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsdpa_gfx950.so")

SDPA_F32, SDPA_BF16, SDPA_F16 = 0, 1, 2
SDPA_CAUSAL_NONE, SDPA_CAUSAL_TOP_LEFT, SDPA_CAUSAL_BOTTOM_RIGHT = 0, 1, 2
_DTYPES = {torch.float32: SDPA_F32, torch.bfloat16: SDPA_BF16, torch.float16: SDPA_F16}

STATUS_NAMES = {
    0: "SDPA_OK", 1: "SDPA_ERR_NULL", 2: "SDPA_ERR_RANK", 3: "SDPA_ERR_SHAPE",
    4: "SDPA_ERR_HEAD_DIM", 5: "SDPA_ERR_DTYPE", 6: "SDPA_ERR_STRIDE", 7: "SDPA_ERR_ALIGN",
    8: "SDPA_ERR_SCALE", 9: "SDPA_ERR_DEVICE", 10: "SDPA_ERR_CAUSAL", 11: "SDPA_ERR_WORKSPACE",
    12: "SDPA_ERR_STATIC_WORKSPACE",
}
SDPA_STATIC_WORKSPACE_BYTES = 16 << 20

EXPORTS = ("sdpa_fwd", "sdpa_check", "sdpa_fwd_bias", "sdpa_fwd_bias_check", "sdpa_fwd_splitkv", "sdpa_fwd_splitkv_check",
           "sdpa_fwd_splitkv_workspace", "sdpa_fwd_splitkv_noalloc", "sdpa_fwd_varlen", "sdpa_fwd_varlen_check", "sdpa_bwd",
           "sdpa_bwd_check", "sdpa_bwd_bias", "sdpa_bwd_bias_check", "sdpa_bwd_varlen",
           "sdpa_bwd_varlen_check", "sdpa_strerror", "sdpa_plan", "sdpa_plan_item")


class SdpaError(RuntimeError):
    """A nonzero status from the library (status code in .status)."""

    def __init__(self, status, msg):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


class SdpaPlan(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in
                ("block_m", "block_n", "threads", "q_tiles", "bh", "items", "lds_bytes",
                 "is_causal")]


_lib = None


def load_library():
    """Load libsdpa_gfx950.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m scaled_dot_product_11_amd.build` (or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    common = [vp, vp, vp, vp, vp, ctypes.c_int, i64, i64, i64, i64, i64,
              ctypes.POINTER(i64), ctypes.c_float, ctypes.c_int, vp, ctypes.c_int]
    lib.sdpa_fwd.argtypes = common + [vp]
    lib.sdpa_fwd.restype = ctypes.c_int
    lib.sdpa_check.argtypes = common
    lib.sdpa_check.restype = ctypes.c_int
    bwd_common = [vp] * 10 + [ctypes.c_int, i64, i64, i64, i64, i64, ctypes.POINTER(i64),
                              ctypes.c_float, ctypes.c_int, vp, ctypes.c_int]
    lib.sdpa_bwd.argtypes = bwd_common + [vp]
    lib.sdpa_bwd.restype = ctypes.c_int
    lib.sdpa_bwd_check.argtypes = bwd_common
    lib.sdpa_bwd_check.restype = ctypes.c_int
    lib.sdpa_bwd_bias.argtypes = bwd_common + [vp]  # the bias takes the mask's place
    lib.sdpa_bwd_bias.restype = ctypes.c_int
    lib.sdpa_bwd_bias_check.argtypes = bwd_common
    lib.sdpa_bwd_bias_check.restype = ctypes.c_int
    bwd_varlen_common = [vp] * 12 + [i64] * 7 + [ctypes.POINTER(i64), ctypes.c_float,
                                                 ctypes.c_int, ctypes.c_int]
    lib.sdpa_bwd_varlen.argtypes = bwd_varlen_common + [vp]
    lib.sdpa_bwd_varlen.restype = ctypes.c_int
    lib.sdpa_bwd_varlen_check.argtypes = bwd_varlen_common
    lib.sdpa_bwd_varlen_check.restype = ctypes.c_int
    varlen_common = [vp] * 7 + [i64] * 6 + [ctypes.POINTER(i64), ctypes.c_float, ctypes.c_int,
                                        ctypes.c_int]
    lib.sdpa_fwd_varlen.argtypes = varlen_common + [vp]
    lib.sdpa_fwd_varlen.restype = ctypes.c_int
    lib.sdpa_fwd_varlen_check.argtypes = varlen_common
    lib.sdpa_fwd_varlen_check.restype = ctypes.c_int
    lib.sdpa_fwd_bias.argtypes = common + [vp]  # the bias takes the mask's place
    lib.sdpa_fwd_bias.restype = ctypes.c_int
    lib.sdpa_fwd_bias_check.argtypes = common
    lib.sdpa_fwd_bias_check.restype = ctypes.c_int
    split_common = [vp] * 5 + [ctypes.c_int, i64, i64, i64, i64, i64, ctypes.POINTER(i64),
                               ctypes.c_float, ctypes.c_int, i64, vp, i64, ctypes.c_int]
    lib.sdpa_fwd_splitkv.argtypes = split_common + [vp]
    lib.sdpa_fwd_splitkv.restype = ctypes.c_int
    lib.sdpa_fwd_splitkv_check.argtypes = split_common
    lib.sdpa_fwd_splitkv_check.restype = ctypes.c_int
    lib.sdpa_fwd_splitkv_noalloc.argtypes = [vp] * 5 + [ctypes.c_int, i64, i64, i64, i64, i64,
                                                        ctypes.POINTER(i64), ctypes.c_float,
                                                        ctypes.c_int, i64, ctypes.c_int, vp]
    lib.sdpa_fwd_splitkv_noalloc.restype = ctypes.c_int
    lib.sdpa_fwd_splitkv_workspace.argtypes = [i64] * 6 + [ctypes.c_int]
    lib.sdpa_fwd_splitkv_workspace.restype = i64
    lib.sdpa_strerror.argtypes = [ctypes.c_int]
    lib.sdpa_strerror.restype = ctypes.c_char_p
    lib.sdpa_plan.argtypes = [ctypes.c_int, i64, i64, i64, i64, i64, ctypes.c_int, ctypes.c_int,
                              ctypes.POINTER(SdpaPlan)]
    lib.sdpa_plan.restype = ctypes.c_int
    lib.sdpa_plan_item.argtypes = [ctypes.POINTER(SdpaPlan), i64, ctypes.POINTER(i64),
                                   ctypes.POINTER(i64)]
    lib.sdpa_plan_item.restype = ctypes.c_int
    _lib = lib
    return lib


def sdpa_strerror(status: int) -> str:
    return load_library().sdpa_strerror(int(status)).decode()


def _raise_on(status):
    if status != 0:
        raise SdpaError(status, sdpa_strerror(status))


def causal_mode(is_causal):
    """The C ABI causal mode for a bool (True = top-left) or an int 0 / 1 / 2."""
    if isinstance(is_causal, bool):
        return SDPA_CAUSAL_TOP_LEFT if is_causal else SDPA_CAUSAL_NONE
    return int(is_causal)


def _stream_handle(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _sizes(q, k):
    if q.dim() == 3:
        return 1, q.shape[0], q.shape[1], k.shape[1], q.shape[2]
    if q.dim() == 4:
        return q.shape[0], q.shape[1], q.shape[2], k.shape[2], q.shape[3]
    return 0, 0, 0, 0, q.shape[-1] if q.dim() else 0


def _marshal(q, k, v, out, lse, mask, scale, is_causal):
    rank = q.dim()
    B, H, Lq, Lk, D = _sizes(q, k)
    dtype = _DTYPES.get(q.dtype, -1)
    strides = [*q.stride(), *k.stride(), *v.stride(), *out.stride()]
    mask_ptr, mask_keep = None, None
    if mask is not None:
        m = _mask_view(mask, q.shape[:-1], Lk)
        strides += list(m.stride())
        mask_ptr, mask_keep = m.data_ptr(), m
    else:
        strides += [0] * rank
    arr = (ctypes.c_int64 * len(strides))(*strides)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    args = [q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
            None if lse is None else lse.data_ptr(), rank, B, H, Lq, Lk, D, arr,
            float(scale), causal_mode(is_causal), mask_ptr, dtype]
    return args, mask_keep


def _check_shapes(q, k, v, out, lse, mask):
    rank = q.dim()
    if k.dim() != rank or v.dim() != rank:
        raise ValueError("q, k and v must have the same rank")
    if rank in (3, 4):
        qs, ks = q.shape, k.shape
        if ks != v.shape:
            raise ValueError("k and v must have the same shape")
        if ks[:-2] != qs[:-2] or ks[-1] != qs[-1]:
            raise ValueError("k must match q in the leading dims and the head dim")
        if out is not None and out.shape != qs:
            raise ValueError("out must have q's shape")
        if lse is not None and (lse.shape != qs[:-1] or lse.dtype != torch.float32 or
                                not lse.is_contiguous()):
            raise ValueError("lse must be a contiguous float32 tensor of shape q.shape[:-1]")
    dt = q.dtype
    if k.dtype != dt or v.dtype != dt or (out is not None and out.dtype != dt):
        raise ValueError("q, k, v and out must share one dtype")
    tensors = (q, k, v, out, lse, mask)
    for t in tensors:
        if t is not None and not t.is_cuda:
            raise ValueError("sdpa_fwd runs on the GPU only: every tensor must be on a cuda device")
    dev = q.device
    for t in tensors:
        if t is not None and t.device != dev:
            raise ValueError("all tensors must be on the same device")


def _on_device(device, fn, *args):
    """fn(*args) with `device` current; the current device is switched (and restored) only
    when it is another one."""
    if device.index is None or device.index == torch.cuda.current_device():
        return fn(*args)
    with torch.cuda.device(device):
        return fn(*args)


def sdpa_fwd(q, k, v, out=None, lse=None, *, scale=None, is_causal=False, mask=None,
             stream=None, return_lse=True):
    """Fused SDPA forward through the C ABI `sdpa_fwd`.

    q: [N,Lq,D] or [B,H,Lq,D]; k, v: [N,Lk,D] or [B,H,Lk,D]; bf16, fp16 or fp32 cuda tensors with
    unit innermost stride (any other strides).  mask: optional bool/uint8 tensor
    broadcastable to q.shape[:-1] + (Lk,), True/nonzero = visible.  is_causal: False/True
    (top-left) or a mode 0 / 1 / 2 (2 = bottom-right).  scale defaults to 1/sqrt(D).  out/lse are allocated when not given (out contiguous, lse float32
    [..., Lq]).  Returns (out, lse) -- lse is None when return_lse is False and no lse
    tensor was passed.  The kernel is enqueued on `stream` (default: torch's current
    stream of q's device); nothing is synchronised.
    """
    _check_shapes(q, k, v, out, lse, mask)
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
    args, _keep = _marshal(q, k, v, out, lse, mask, scale, is_causal)
    handle = _stream_handle(stream, q.device)
    status = _on_device(q.device, load_library().sdpa_fwd, *args, handle)
    _raise_on(status)
    return out, lse


def _mask_view(mask, lead_shape, Lk):
    m = mask.expand(*lead_shape, Lk)
    if m.dtype == torch.bool:
        m = m.view(torch.uint8)
    if m.dtype != torch.uint8:
        raise TypeError("mask must be a bool or uint8 tensor")
    return m


def sdpa_bwd(q, k, v, out, dout, lse, dq=None, dk=None, dv=None, delta=None, *, scale=None,
             is_causal=False, mask=None, stream=None):
    """Gradients of the fused SDPA through the C ABI `sdpa_bwd` (bf16 or fp16).

    q, k, v, mask, scale, is_causal: as passed to sdpa_fwd; out and lse: what sdpa_fwd
    returned for them; dout: the upstream gradient, shaped like out.  dq/dk/dv (shaped and
    typed like q/k/v) and delta (float32 scratch shaped like lse, receives rowsum(dout *
    out)) are allocated when not given.  Returns (dq, dk, dv); two kernels are enqueued on
    `stream` (default: torch's current stream of q's device), nothing is synchronised.
    """
    _check_shapes(q, k, v, out, lse, mask)
    return _bwd_call("sdpa_bwd", q, k, v, out, dout, lse, dq, dk, dv, delta, scale, is_causal,
                     None if mask is None else _mask_view(mask, q.shape[:-1], k.shape[-2]),
                     stream)


def sdpa_bwd_bias(q, k, v, out, dout, lse, bias, dq=None, dk=None, dv=None, delta=None, *,
                  scale=None, is_causal=False, stream=None):
    """Gradients of sdpa_fwd_bias through the C ABI `sdpa_bwd_bias`, the bias held constant.

    bias: the float32 tensor passed to sdpa_fwd_bias (broadcastable to q.shape[:-1] +
    (Lk,)); out and lse: what sdpa_fwd_bias returned.  Otherwise as sdpa_bwd.  Returns
    (dq, dk, dv)."""
    if bias is None or bias.dtype != torch.float32:
        raise TypeError("bias must be a float32 tensor")
    _check_shapes(q, k, v, out, lse, bias)
    return _bwd_call("sdpa_bwd_bias", q, k, v, out, dout, lse, dq, dk, dv, delta, scale,
                     is_causal, bias.expand(*q.shape[:-1], k.shape[-2]), stream)


def _bwd_call(entry, q, k, v, out, dout, lse, dq, dk, dv, delta, scale, is_causal, extra,
              stream):
    """Marshal the dense backward's arguments for `entry` (sdpa_bwd with the boolean mask
    view `extra`, or sdpa_bwd_bias with the expanded bias `extra`; None for neither)."""
    for name, t, like in (("dout", dout, q), ("dq", dq, q), ("dk", dk, k), ("dv", dv, k)):
        if t is not None and (tuple(t.shape) != tuple(like.shape) or t.dtype != q.dtype or
                              t.device != q.device):
            raise ValueError(f"{name} must match {'q' if like is q else 'k'} in shape, dtype "
                             "and device")
    if dout is None or lse is None:
        raise ValueError("dout and the forward's lse are required")
    if delta is not None and (tuple(delta.shape) != tuple(lse.shape) or
                              delta.dtype != torch.float32 or not delta.is_contiguous() or
                              delta.device != q.device):
        raise ValueError("delta must be a contiguous float32 tensor shaped like lse")
    dq = torch.empty(q.shape, dtype=q.dtype, device=q.device) if dq is None else dq
    dk = torch.empty(k.shape, dtype=k.dtype, device=k.device) if dk is None else dk
    dv = torch.empty(v.shape, dtype=v.dtype, device=v.device) if dv is None else dv
    delta = torch.empty(lse.shape, dtype=torch.float32, device=q.device) if delta is None else delta
    rank = q.dim()
    B, H, Lq, Lk, D = _sizes(q, k)
    strides = [*q.stride(), *k.stride(), *v.stride(), *out.stride(), *dout.stride(),
               *dq.stride(), *dk.stride(), *dv.stride()]
    strides += [0] * rank if extra is None else list(extra.stride())
    arr = (ctypes.c_int64 * len(strides))(*strides)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    handle = _stream_handle(stream, q.device)
    status = _on_device(q.device, getattr(load_library(), entry),
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(),
        lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(),
        rank, B, H, Lq, Lk, D, arr, float(scale), causal_mode(is_causal),
        None if extra is None else extra.data_ptr(), _DTYPES.get(q.dtype, -1), handle)
    _raise_on(status)
    return dq, dk, dv


def sdpa_bwd_varlen(q, k, v, out, dout, lse, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                    max_seqlen_k, dq=None, dk=None, dv=None, delta=None, *, scale=None,
                    is_causal=False, stream=None):
    """Gradients of sdpa_fwd_varlen through the C ABI `sdpa_bwd_varlen` (bf16 or fp16).

    q, k, v, cu_seqlens_q, cu_seqlens_k, scale, is_causal: as passed to sdpa_fwd_varlen;
    out, lse: what it returned; dout shaped like out; max_seqlen_q / max_seqlen_k: int
    bounds of the query and key lengths.  dq/dk/dv and delta ([H, total_q] float32
    scratch) are allocated when not given.  Returns (dq, dk, dv)."""
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k and v must be [tokens, H, D]")
    if tuple(k.shape) != tuple(v.shape) or k.shape[1:] != q.shape[1:]:
        raise ValueError("k and v must be [total_k, H, D] with q's H and D")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k and v must share one dtype")
    for name, t in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        if t.dtype != torch.int32 or t.dim() != 1 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 1-D int32 tensor")
    if cu_seqlens_q.numel() != cu_seqlens_k.numel() or cu_seqlens_q.numel() < 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k need the same nseq + 1 >= 1 entries")
    if out is None or dout is None or lse is None:
        raise ValueError("out, dout and the forward's lse are required")
    total_q, H, D = q.shape
    total_k = k.shape[0]
    for name, t, like in (("out", out, q), ("dout", dout, q), ("dq", dq, q), ("dk", dk, k),
                          ("dv", dv, k)):
        if t is not None and (tuple(t.shape) != tuple(like.shape) or t.dtype != q.dtype):
            raise ValueError(f"{name} must match {'q' if like is q else 'k'} in shape and dtype")
    for name, t in (("lse", lse), ("delta", delta)):
        if t is not None and (tuple(t.shape) != (H, total_q) or t.dtype != torch.float32 or
                              not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous float32 tensor [H, total_q]")
    ts = (q, k, v, out, dout, lse, cu_seqlens_q, cu_seqlens_k, dq, dk, dv, delta)
    if any(t is not None and t.device.type != "cuda" for t in ts):
        raise ValueError("sdpa_bwd_varlen runs on the GPU only: every tensor must be on a cuda device")
    if len({t.device for t in ts if t is not None}) != 1:
        raise ValueError("all tensors must be on the same device")
    dq = torch.empty(q.shape, dtype=q.dtype, device=q.device) if dq is None else dq
    dk = torch.empty(k.shape, dtype=k.dtype, device=k.device) if dk is None else dk
    dv = torch.empty(v.shape, dtype=v.dtype, device=v.device) if dv is None else dv
    if delta is None:
        delta = torch.empty((H, total_q), dtype=torch.float32, device=q.device)
    strides = [*q.stride(), *k.stride(), *v.stride(), *out.stride(), *dout.stride(),
               *dq.stride(), *dk.stride(), *dv.stride()]
    arr = (ctypes.c_int64 * 24)(*strides)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    handle = _stream_handle(stream, q.device)
    status = _on_device(q.device, load_library().sdpa_bwd_varlen,
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(),
        lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(),
        cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), cu_seqlens_q.numel() - 1,
        int(max_seqlen_q), int(max_seqlen_k), total_q, total_k, H, D, arr, float(scale),
        causal_mode(is_causal), _DTYPES.get(q.dtype, -1), handle)
    _raise_on(status)
    return dq, dk, dv


def sdpa_fwd_bias(q, k, v, bias, out=None, lse=None, *, scale=None, is_causal=False,
                  stream=None, return_lse=True):
    """SDPA forward with an additive float mask (C ABI `sdpa_fwd_bias`): bias is a float32
    cuda tensor broadcastable to q.shape[:-1] + (Lk,), added to the scaled scores (-inf
    hides a key).  Otherwise as sdpa_fwd.  Returns (out, lse)."""
    _check_shapes(q, k, v, out, lse, bias)
    if bias.dtype != torch.float32:
        raise TypeError("bias must be a float32 tensor")
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
    B, H, Lq, Lk, D = _sizes(q, k)
    b = bias.expand(*q.shape[:-1], Lk)
    strides = [*q.stride(), *k.stride(), *v.stride(), *out.stride(), *b.stride()]
    arr = (ctypes.c_int64 * len(strides))(*strides)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    handle = _stream_handle(stream, q.device)
    status = _on_device(q.device, load_library().sdpa_fwd_bias,
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
        None if lse is None else lse.data_ptr(), q.dim(), B, H, Lq, Lk, D, arr,
        float(scale), causal_mode(is_causal), b.data_ptr(), _DTYPES.get(q.dtype, -1), handle)
    _raise_on(status)
    return out, lse


def sdpa_fwd_bias_check(q_ptr, k_ptr, v_ptr, out_ptr, lse_ptr, rank, B, H, Lq, Lk, D, strides,
                        scale, is_causal, bias_ptr, dtype) -> int:
    """The C ABI `sdpa_fwd_bias_check` on raw integers (as sdpa_check, with the bias pointer
    in the mask's place).  Host-only."""
    arr = (ctypes.c_int64 * len(strides))(*strides) if strides is not None else None
    return load_library().sdpa_fwd_bias_check(q_ptr, k_ptr, v_ptr, out_ptr, lse_ptr, rank, B, H,
                                              Lq, Lk, D, arr, float(scale), int(is_causal),
                                              bias_ptr, int(dtype))


def sdpa_fwd_splitkv_workspace(B, H, Lq, Lk, D, num_splits=0, dtype=SDPA_BF16) -> int:
    """The C ABI `sdpa_fwd_splitkv_workspace`: workspace bytes (host-only)."""
    n = load_library().sdpa_fwd_splitkv_workspace(B, H, Lq, Lk, D, int(num_splits), int(dtype))
    if n < 0:
        _raise_on(-n)
    return n


def sdpa_fwd_splitkv(q, k, v, out=None, lse=None, *, scale=None, is_causal=False, num_splits=0,
                     workspace=None, stream=None, return_lse=True):
    """sdpa_fwd with the keys split across workgroups (C ABI `sdpa_fwd_splitkv`), for few
    query rows against many keys.  Same tensors as sdpa_fwd, no mask.  num_splits: 0 lets
    the library choose.  workspace: a cuda tensor of at least sdpa_fwd_splitkv_workspace()
    bytes (allocated with torch when not given).  Returns (out, lse)."""
    _check_shapes(q, k, v, out, lse, None)
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
    rank = q.dim()
    B, H, Lq, Lk, D = _sizes(q, k)
    dtype = _DTYPES.get(q.dtype, -1)
    need = sdpa_fwd_splitkv_workspace(B, H, Lq, Lk, D, num_splits, dtype) if dtype >= 0 else 0
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    if workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on q's device")
    strides = [*q.stride(), *k.stride(), *v.stride(), *out.stride()]
    arr = (ctypes.c_int64 * len(strides))(*strides)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    handle = _stream_handle(stream, q.device)
    status = _on_device(q.device, load_library().sdpa_fwd_splitkv,
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
        None if lse is None else lse.data_ptr(), rank, B, H, Lq, Lk, D, arr, float(scale),
        causal_mode(is_causal), int(num_splits), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), dtype, handle)
    _raise_on(status)
    return out, lse


def sdpa_fwd_splitkv_noalloc(q, k, v, out, lse=None, *, scale=None, is_causal=False,
                             num_splits=0, stream=None):
    """sdpa_fwd_splitkv without a workspace argument (C ABI `sdpa_fwd_splitkv_noalloc`): the
    partial results go to the library's static per-device workspace of
    SDPA_STATIC_WORKSPACE_BYTES, for callers that cannot allocate.  out (and lse, if wanted)
    must be given: this call allocates nothing.  Calls that overlap in time on one device
    share the workspace.  Returns (out, lse)."""
    _check_shapes(q, k, v, out, lse, None)
    if out is None:
        raise ValueError("sdpa_fwd_splitkv_noalloc allocates nothing: pass out (and lse)")
    rank = q.dim()
    B, H, Lq, Lk, D = _sizes(q, k)
    strides = [*q.stride(), *k.stride(), *v.stride(), *out.stride()]
    arr = (ctypes.c_int64 * len(strides))(*strides)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    handle = _stream_handle(stream, q.device)
    status = _on_device(q.device, load_library().sdpa_fwd_splitkv_noalloc,
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
        None if lse is None else lse.data_ptr(), rank, B, H, Lq, Lk, D, arr, float(scale),
        causal_mode(is_causal), int(num_splits), _DTYPES.get(q.dtype, -1), handle)
    _raise_on(status)
    return out, lse


def sdpa_fwd_splitkv_check(ptrs, rank, B, H, Lq, Lk, D, strides, scale, causal, num_splits,
                           workspace_ptr, workspace_bytes, dtype) -> int:
    """The C ABI `sdpa_fwd_splitkv_check` on raw integers: ptrs = (q, k, v, out, lse),
    strides a list of 4*rank ints.  Host-only."""
    arr = (ctypes.c_int64 * len(strides))(*strides) if strides is not None else None
    return load_library().sdpa_fwd_splitkv_check(*ptrs, rank, B, H, Lq, Lk, D, arr, float(scale),
                                                 int(causal), int(num_splits), workspace_ptr,
                                                 int(workspace_bytes), int(dtype))


def sdpa_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, out=None, lse=None, *,
                    scale=None, is_causal=False, stream=None, return_lse=True):
    """Fused forward over packed variable-length sequences through the C ABI
    `sdpa_fwd_varlen`.

    q: [total_q, H, D], k, v: [total_k, H, D] (bf16, fp16 or fp32 cuda tensors, unit dim stride);
    cu_seqlens_q / cu_seqlens_k: int32 cuda tensors of nseq + 1 offsets; max_seqlen_q: an
    int bound of the query lengths (it sizes the launch).  is_causal: False/True (top-left)
    or a mode 0 / 1 / 2, applied per sequence.  out ([total_q, H, D]) and lse ([H, total_q]
    float32) are allocated when not given.  Returns (out, lse).
    """
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k and v must be [tokens, H, D]")
    if tuple(k.shape) != tuple(v.shape) or k.shape[1:] != q.shape[1:]:
        raise ValueError("k and v must be [total_k, H, D] with q's H and D")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k and v must share one dtype")
    for name, t in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        if t.dtype != torch.int32 or t.dim() != 1 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 1-D int32 tensor")
    if cu_seqlens_q.numel() != cu_seqlens_k.numel() or cu_seqlens_q.numel() < 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k need the same nseq + 1 >= 1 entries")
    ts = (q, k, v, cu_seqlens_q, cu_seqlens_k, out, lse)
    if any(t is not None and t.device.type != "cuda" for t in ts):
        raise ValueError("sdpa_fwd_varlen runs on the GPU only: every tensor must be on a cuda device")
    if len({t.device for t in ts if t is not None}) != 1:
        raise ValueError("all tensors must be on the same device")
    total_q, H, D = q.shape
    total_k = k.shape[0]
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    elif tuple(out.shape) != tuple(q.shape) or out.dtype != q.dtype:
        raise ValueError("out must have q's shape and dtype")
    if lse is None and return_lse:
        lse = torch.empty((H, total_q), dtype=torch.float32, device=q.device)
    elif lse is not None and (tuple(lse.shape) != (H, total_q) or lse.dtype != torch.float32 or
                              not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 tensor [H, total_q]")
    strides = [*q.stride(), *k.stride(), *v.stride(), *out.stride()]
    arr = (ctypes.c_int64 * 12)(*strides)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    handle = _stream_handle(stream, q.device)
    status = _on_device(q.device, load_library().sdpa_fwd_varlen,
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
        None if lse is None else lse.data_ptr(), cu_seqlens_q.data_ptr(),
        cu_seqlens_k.data_ptr(), cu_seqlens_q.numel() - 1, int(max_seqlen_q), total_q,
        total_k, H, D, arr, float(scale), causal_mode(is_causal), _DTYPES.get(q.dtype, -1),
        handle)
    _raise_on(status)
    return out, lse


def sdpa_fwd_varlen_check(ptrs, nseq, max_seqlen_q, total_q, total_k, H, D, strides, scale,
                          causal, dtype) -> int:
    """The C ABI `sdpa_fwd_varlen_check` on raw integers: ptrs = the 7 pointers (q, k, v,
    out, lse, cu_seqlens_q, cu_seqlens_k) as ints, strides a list of 12 ints.  Host-only."""
    arr = (ctypes.c_int64 * len(strides))(*strides) if strides is not None else None
    return load_library().sdpa_fwd_varlen_check(*ptrs, nseq, max_seqlen_q, total_q, total_k, H,
                                                D, arr, float(scale), int(causal), int(dtype))


def sdpa_bwd_check(ptrs, rank, B, H, Lq, Lk, D, strides, scale, is_causal, mask_ptr,
                   dtype) -> int:
    """The C ABI `sdpa_bwd_check` on raw integers: ptrs = the 10 pointers (q, k, v, out,
    dout, lse, dq, dk, dv, delta) as ints, strides a list of 9*rank ints.  Host-only."""
    arr = (ctypes.c_int64 * len(strides))(*strides) if strides is not None else None
    return load_library().sdpa_bwd_check(*ptrs, rank, B, H, Lq, Lk, D, arr, float(scale),
                                         int(is_causal), mask_ptr, int(dtype))


def sdpa_bwd_bias_check(ptrs, rank, B, H, Lq, Lk, D, strides, scale, is_causal, bias_ptr,
                        dtype) -> int:
    """The C ABI `sdpa_bwd_bias_check` on raw integers (as sdpa_bwd_check, with the bias
    pointer in the mask's place).  Host-only."""
    arr = (ctypes.c_int64 * len(strides))(*strides) if strides is not None else None
    return load_library().sdpa_bwd_bias_check(*ptrs, rank, B, H, Lq, Lk, D, arr, float(scale),
                                              int(is_causal), bias_ptr, int(dtype))


def sdpa_bwd_varlen_check(ptrs, nseq, max_seqlen_q, max_seqlen_k, total_q, total_k, H, D,
                          strides, scale, causal, dtype) -> int:
    """The C ABI `sdpa_bwd_varlen_check` on raw integers: ptrs = the 12 pointers (q, k, v,
    out, dout, lse, dq, dk, dv, delta, cu_seqlens_q, cu_seqlens_k) as ints, strides a list
    of 24 ints.  Host-only."""
    arr = (ctypes.c_int64 * len(strides))(*strides) if strides is not None else None
    return load_library().sdpa_bwd_varlen_check(*ptrs, nseq, max_seqlen_q, max_seqlen_k, total_q,
                                                total_k, H, D, arr, float(scale), int(causal),
                                                int(dtype))


def sdpa_check(q_ptr, k_ptr, v_ptr, out_ptr, lse_ptr, rank, B, H, Lq, Lk, D, strides, scale,
               is_causal, mask_ptr, dtype) -> int:
    """The C ABI `sdpa_check` on raw integers (pointers as ints, strides as a list of
    5*rank ints).  Host-only: needs no GPU.  Returns the status code."""
    arr = (ctypes.c_int64 * len(strides))(*strides) if strides is not None else None
    return load_library().sdpa_check(q_ptr, k_ptr, v_ptr, out_ptr, lse_ptr, rank, B, H, Lq, Lk, D,
                                     arr, float(scale), int(is_causal), mask_ptr, int(dtype))


def sdpa_plan(rank, B, H, Lq, Lk, D, is_causal, dtype) -> SdpaPlan:
    """The C ABI `sdpa_plan`: launch plan of the tile scheduler (host-only)."""
    plan = SdpaPlan()
    _raise_on(load_library().sdpa_plan(rank, B, H, Lq, Lk, D, int(is_causal), int(dtype),
                                       ctypes.byref(plan)))
    return plan


def sdpa_plan_item(plan: SdpaPlan, block: int):
    """The C ABI `sdpa_plan_item`: (bh, q_tile) run by workgroup `block` (host-only)."""
    bh, qt = ctypes.c_int64(), ctypes.c_int64()
    _raise_on(load_library().sdpa_plan_item(ctypes.byref(plan), int(block), ctypes.byref(bh),
                                            ctypes.byref(qt)))
    return bh.value, qt.value
