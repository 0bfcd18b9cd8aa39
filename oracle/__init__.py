"""fp64 CPU oracle for the scaled-dot-product-attention forward.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the CPU-baseline leg of the
benchmark may import this package; the product path never does.  It shares no code with
the HIP library and does not import it.

The arithmetic lives in oracle.c (plain fp64 loops, one output row at a time); this module
only marshals torch CPU tensors (or numpy arrays) into pointers and strides.

What is computed, per "Profiling in PyTorch (part 3): attention" (naive causal attention
section: the five primitive steps and the default scale 1/sqrt(head_dim); SDPA math
backend section: the safe softmax that keeps fully masked rows free of NaN):

    out[b,h,i,:] = sum_j softmax_j(scale * q[b,h,i,:].k[b,h,j,:] over visible j) v[b,h,j,:]
    lse[b,h,i]   = log sum_{visible j} exp(scale * q.k)         (natural log)

with visible j = (not causal or j <= i) and (no mask or mask[b,h,i,j] != 0); a row with
no visible key returns zeros and lse = -inf.  A rank-3 [N,L,D] input is read as the
rank-4 input [1,N,L,D], following the PyTorch 2.14 note on rank-3 SDPA inputs (a folded
or missing batch dimension is the same computation).
"""
import ctypes
import math
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# ORACLE_LIB points the wrapper at another build of oracle.c (the mutation test uses it to
# check that the pins reject deliberately broken copies).
_LIB_PATH = os.environ.get("ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

_DTYPE_CODE = {torch.float32: 0, torch.bfloat16: 1, torch.float64: 2, torch.float16: 3}


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _build
            _build.build()
        lib = ctypes.CDLL(_LIB_PATH)
        i64p = ctypes.POINTER(ctypes.c_int64)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.oracle_sdpa_fwd.restype = ctypes.c_int
        lib.oracle_sdpa_fwd.argtypes = [
            ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_int64,
            ctypes.c_void_p, i64p, ctypes.c_void_p, i64p, ctypes.c_void_p, i64p,
            ctypes.c_void_p, i64p,
            ctypes.c_int, ctypes.c_double, i64p, ctypes.c_int64, dp, dp, ctypes.c_int]
        lib.oracle_sdpa_fwd_bias.restype = ctypes.c_int
        lib.oracle_sdpa_fwd_bias.argtypes = [
            ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_int64,
            ctypes.c_void_p, i64p, ctypes.c_void_p, i64p, ctypes.c_void_p, i64p,
            ctypes.c_void_p, i64p, dp, i64p,
            ctypes.c_int, ctypes.c_double, i64p, ctypes.c_int64, dp, dp, ctypes.c_int]
        lib.oracle_sdpa_bwd.restype = ctypes.c_int
        lib.oracle_sdpa_bwd.argtypes = [
            ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_int64,
            ctypes.c_void_p, i64p, ctypes.c_void_p, i64p, ctypes.c_void_p, i64p,
            ctypes.c_void_p, i64p, ctypes.c_void_p, i64p,
            ctypes.c_int, ctypes.c_double, dp, dp, dp, ctypes.c_int]
        lib.oracle_sdpa_bwd_bias.restype = ctypes.c_int
        lib.oracle_sdpa_bwd_bias.argtypes = [
            ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_int64,
            ctypes.c_void_p, i64p, ctypes.c_void_p, i64p, ctypes.c_void_p, i64p,
            ctypes.c_void_p, i64p, ctypes.c_void_p, i64p, dp, i64p,
            ctypes.c_int, ctypes.c_double, dp, dp, dp, ctypes.c_int]
        lib.oracle_default_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def default_threads() -> int:
    """OpenMP threads the oracle uses when nthreads <= 0."""
    return int(_load().oracle_default_threads())


def _as_tensor(x):
    if isinstance(x, np.ndarray):
        return torch.from_numpy(x)
    return x


def _strides4(t):
    """(b, h, row, d) element strides of a rank-3 or rank-4 tensor (rank 3 -> B = 1)."""
    s = t.stride()
    return (0,) + tuple(s) if t.dim() == 3 else tuple(s)


def _check_qkv(q, k, v):
    for t in (q, k, v):
        if t.device.type != "cpu":
            raise ValueError("the oracle reads host memory; move tensors to the CPU first")
    if not (q.dim() == k.dim() == v.dim() and q.dim() in (3, 4)):
        raise ValueError("q, k, v must all be rank 3 or all rank 4")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in _DTYPE_CODE:
        raise ValueError("q, k, v must share one dtype among float32, bfloat16, float16, float64")
    if q.dim() == 3:
        B, H, Lq, D = 1, q.shape[0], q.shape[1], q.shape[2]
        Lk = k.shape[1]
    else:
        B, H, Lq, D = q.shape
        Lk = k.shape[2]
    if tuple(k.shape) != tuple(q.shape[:-2]) + (Lk, D) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v must have q's leading dims, the same length Lk and head dim")
    return B, H, Lq, Lk, D


def _mask_args(mask, q, Lk):
    """(pointer, strides array, keep-alive tensor) of a bool/uint8 mask expanded to q's rows."""
    if mask is None:
        return None, None, None
    mask_t = _as_tensor(mask).expand(tuple(q.shape[:-1]) + (Lk,))
    if mask_t.dtype == torch.bool:
        mask_t = mask_t.view(torch.uint8)
    if mask_t.dtype != torch.uint8:
        raise ValueError("mask must be bool or uint8")
    return ctypes.c_void_p(mask_t.data_ptr()), (ctypes.c_int64 * 4)(*_strides4(mask_t)), mask_t


def _bias_args(bias, q, Lk):
    """(pointer, strides array, keep-alive tensor) of a float bias expanded to q's rows,
    read exactly as float64."""
    if bias is None:
        return None, None, None
    # converted in its own (unbroadcast) shape, then broadcast with zero strides
    bias_t = _as_tensor(bias).to(torch.float64).expand(tuple(q.shape[:-1]) + (Lk,))
    bptr = ctypes.cast(ctypes.c_void_p(bias_t.data_ptr()), ctypes.POINTER(ctypes.c_double))
    return bptr, (ctypes.c_int64 * 4)(*_strides4(bias_t)), bias_t


def sdpa_bwd_oracle(q, k, v, dout, *, mask=None, is_causal=False, scale=None, nthreads=0,
                    bias=None):
    """Gradients (dq, dk, dv) of out = sdpa(q, k, v) for the upstream gradient dout, in fp64.

    Same tensor conventions as sdpa_oracle (mask, bias, is_causal, scale); dout has q's shape
    and dtype.  The bias is a constant: it shifts the scores, and no gradient is returned for
    it.  Returns float64 numpy arrays shaped like q, k and v.  Fully masked query rows
    contribute nothing.
    """
    q, k, v, dout = _as_tensor(q), _as_tensor(k), _as_tensor(v), _as_tensor(dout)
    B, H, Lq, Lk, D = _check_qkv(q, k, v)
    if tuple(dout.shape) != tuple(q.shape) or dout.dtype != q.dtype or dout.device.type != "cpu":
        raise ValueError("dout must be a CPU tensor with q's shape and dtype")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    mptr, ms_arr, _keep = _mask_args(mask, q, Lk)
    bptr, bs_arr, _keep_b = _bias_args(bias, q, Lk)
    dq = np.zeros((B * H * Lq, D), dtype=np.float64)
    dk = np.zeros((B * H * Lk, D), dtype=np.float64)
    dv = np.zeros((B * H * Lk, D), dtype=np.float64)
    st = _load().oracle_sdpa_bwd_bias(
        _DTYPE_CODE[q.dtype], B, H, Lq, Lk, D,
        ctypes.c_void_p(q.data_ptr()), (ctypes.c_int64 * 4)(*_strides4(q)),
        ctypes.c_void_p(k.data_ptr()), (ctypes.c_int64 * 4)(*_strides4(k)),
        ctypes.c_void_p(v.data_ptr()), (ctypes.c_int64 * 4)(*_strides4(v)),
        ctypes.c_void_p(dout.data_ptr()), (ctypes.c_int64 * 4)(*_strides4(dout)),
        mptr, ms_arr, bptr, bs_arr, 1 if is_causal else 0, float(scale),
        dq.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
        dk.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
        dv.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), int(nthreads))
    if st != 0:
        raise RuntimeError(f"oracle_sdpa_bwd_bias failed with status {st}")
    return dq.reshape(tuple(q.shape)), dk.reshape(tuple(k.shape)), dv.reshape(tuple(v.shape))


def sdpa_oracle(q, k, v, *, mask=None, is_causal=False, scale=None, rows=None, nthreads=0,
                bias=None):
    """Evaluate the plain definition in fp64.

    q: [N,Lq,D] or [B,H,Lq,D]; k, v: same rank with Lk rows; CPU tensors (or numpy) of one
    dtype among float32 / bfloat16 / float16 / float64, any strides.  mask: optional bool or uint8
    tensor broadcastable to [B,H,Lq,Lk] (rank 4) or [N,Lq,Lk] (rank 3); nonzero = visible.
    bias: optional float tensor of the same broadcast shapes, added to the scaled scores
    (-inf hides a key), read exactly in fp64.
    rows: optional int64 flat row ids (b*H + h)*Lq + i.

    Returns (out, lse) as float64 numpy arrays: shaped like q and q.shape[:-1] when rows is
    None, else [len(rows), D] and [len(rows)].
    """
    q, k, v = _as_tensor(q), _as_tensor(k), _as_tensor(v)
    for t in (q, k, v):
        if t.device.type != "cpu":
            raise ValueError("the oracle reads host memory; move tensors to the CPU first")
    if not (q.dim() == k.dim() == v.dim() and q.dim() in (3, 4)):
        raise ValueError("q, k, v must all be rank 3 or all rank 4")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in _DTYPE_CODE:
        raise ValueError("q, k, v must share one dtype among float32, bfloat16, float16, float64")
    rank = q.dim()
    if rank == 3:
        B, H, Lq, D = 1, q.shape[0], q.shape[1], q.shape[2]
        Lk = k.shape[1]
    else:
        B, H, Lq, D = q.shape
        Lk = k.shape[2]
    if tuple(k.shape) != tuple(q.shape[:-2]) + (Lk, D) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v must have q's leading dims, the same length Lk and head dim")
    if scale is None:
        scale = 1.0 / math.sqrt(D)

    mptr, ms_arr, mask_t = None, None, None
    if mask is not None:
        mask_t = _as_tensor(mask)
        full = tuple(q.shape[:-1]) + (Lk,)
        mask_t = mask_t.expand(full)
        if mask_t.dtype == torch.bool:
            mask_t = mask_t.view(torch.uint8)
        if mask_t.dtype != torch.uint8:
            raise ValueError("mask must be bool or uint8")
        ms = _strides4(mask_t)
        ms_arr = (ctypes.c_int64 * 4)(*ms)
        mptr = ctypes.c_void_p(mask_t.data_ptr())

    bptr, bs_arr, bias_t = None, None, None
    if bias is not None:
        # converted in its own (unbroadcast) shape, then broadcast with zero strides
        bias_t = _as_tensor(bias).to(torch.float64).expand(tuple(q.shape[:-1]) + (Lk,))
        bs_arr = (ctypes.c_int64 * 4)(*_strides4(bias_t))
        bptr = ctypes.cast(ctypes.c_void_p(bias_t.data_ptr()), ctypes.POINTER(ctypes.c_double))

    if rows is None:
        n = B * H * Lq
        rows_arr, rows_ptr = None, None
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        n = rows_arr.shape[0]
        rows_ptr = rows_arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))

    out = np.zeros((n, D), dtype=np.float64)
    lse = np.zeros((n,), dtype=np.float64)
    qs = (ctypes.c_int64 * 4)(*_strides4(q))
    ks = (ctypes.c_int64 * 4)(*_strides4(k))
    vs = (ctypes.c_int64 * 4)(*_strides4(v))
    lib = _load()
    st = lib.oracle_sdpa_fwd_bias(
        _DTYPE_CODE[q.dtype], B, H, Lq, Lk, D,
        ctypes.c_void_p(q.data_ptr()), qs, ctypes.c_void_p(k.data_ptr()), ks,
        ctypes.c_void_p(v.data_ptr()), vs, mptr, ms_arr, bptr, bs_arr,
        1 if is_causal else 0, float(scale), rows_ptr, n,
        out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
        lse.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), int(nthreads))
    if st != 0:
        raise RuntimeError(f"oracle_sdpa_fwd failed with status {st}")
    if rows is None:
        out = out.reshape(tuple(q.shape))
        lse = lse.reshape(tuple(q.shape[:-1]))
    return out, lse
