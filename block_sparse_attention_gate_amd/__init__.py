"""Python binding of libmoba.so, the MI355X (gfx950) MoBA forward library.

Argument marshalling only: every step of the forward runs in the HIP kernels
behind the C ABI declared in ``include/moba.h``.  PyTorch supplies device
memory (tensors, the workspace) and the current HIP stream.  There is no
fallback: if ``libmoba.so`` has not been built, importing this package fails.

Layouts (contiguous, head_dim innermost):
  prefill  q, out [L, H, D]        k, v [L, Hkv, D]
  general  q, out [S, Lq, H, D]    k, v [S, L, Hkv, D]
"""

from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoba.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")

_lib = ctypes.CDLL(LIB_PATH)

MOBA_DTYPE_F32 = 0
MOBA_DTYPE_BF16 = 1
MOBA_OK = 0
MOBA_ERR_INVALID_ARGUMENT = 1
MOBA_ERR_UNSUPPORTED = 2
MOBA_ERR_OUT_OF_MEMORY = 3
MOBA_ERR_HIP = 4


class MobaArgs(ctypes.Structure):
    """Mirror of ``moba_args`` in include/moba.h."""

    _fields_ = [
        ("struct_size", ctypes.c_size_t),
        ("q", ctypes.c_void_p),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("out", ctypes.c_void_p),
        ("k_block_mean", ctypes.c_void_p),
        ("sel_out", ctypes.c_void_p),
        ("batch", ctypes.c_int32),
        ("n_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("topk", ctypes.c_int32),
        ("q_len", ctypes.c_int64),
        ("kv_len", ctypes.c_int64),
        ("dtype", ctypes.c_int),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("stream", ctypes.c_void_p),
        ("lse_out", ctypes.c_void_p),
        ("kv_lens", ctypes.c_void_p),
        ("routed_bytes_limit", ctypes.c_size_t),
    ]


class MobaBwdArgs(ctypes.Structure):
    """Mirror of ``moba_bwd_args`` in include/moba.h."""

    _fields_ = [
        ("struct_size", ctypes.c_size_t),
        ("q", ctypes.c_void_p),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("out", ctypes.c_void_p),
        ("dout", ctypes.c_void_p),
        ("lse", ctypes.c_void_p),
        ("sel", ctypes.c_void_p),
        ("dq", ctypes.c_void_p),
        ("dk", ctypes.c_void_p),
        ("dv", ctypes.c_void_p),
        ("batch", ctypes.c_int32),
        ("n_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("topk", ctypes.c_int32),
        ("q_len", ctypes.c_int64),
        ("kv_len", ctypes.c_int64),
        ("dtype", ctypes.c_int),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("stream", ctypes.c_void_p),
    ]


class MobaVarlenArgs(ctypes.Structure):
    """Mirror of ``moba_varlen_args`` in include/moba.h."""

    _fields_ = [
        ("struct_size", ctypes.c_size_t),
        ("q", ctypes.c_void_p),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("out", ctypes.c_void_p),
        ("dout", ctypes.c_void_p),
        ("dq", ctypes.c_void_p),
        ("dk", ctypes.c_void_p),
        ("dv", ctypes.c_void_p),
        ("cu_seqlens_q", ctypes.c_void_p),
        ("cu_seqlens_k", ctypes.c_void_p),
        ("sel", ctypes.c_void_p),
        ("lse", ctypes.c_void_p),
        ("batch", ctypes.c_int32),
        ("n_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("topk", ctypes.c_int32),
        ("dtype", ctypes.c_int),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("stream", ctypes.c_void_p),
    ]


_P = ctypes.c_void_p
_I32, _I64 = ctypes.c_int32, ctypes.c_int64
_ST = ctypes.c_int

_SIGNATURES = {
    "moba_forward": (_ST, [_P, _P, _P, _I64, _I32, _I32, _I32, _I32, _I32, _P, ctypes.c_int, _P]),
    "moba_full_attention": (_ST, [_P, _P, _P, _I64, _I32, _I32, _I32, _P, ctypes.c_int, _P]),
    "moba_forward_ex": (_ST, [ctypes.POINTER(MobaArgs)]),
    "moba_forward_noalloc": (_ST, [ctypes.POINTER(MobaArgs)]),
    "moba_full_attention_ex": (_ST, [ctypes.POINTER(MobaArgs)]),
    "moba_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(MobaArgs)]),
    "moba_full_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(MobaArgs)]),
    "moba_naive_ex": (_ST, [ctypes.POINTER(MobaArgs)]),
    "moba_naive_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(MobaArgs)]),
    "moba_backward_ex": (_ST, [ctypes.POINTER(MobaBwdArgs)]),
    "moba_forward_varlen": (_ST, [ctypes.POINTER(MobaVarlenArgs)]),
    "moba_backward_varlen": (_ST, [ctypes.POINTER(MobaVarlenArgs)]),
    "moba_varlen_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(MobaVarlenArgs), _I32]),
    "moba_backward_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(MobaBwdArgs)]),
    "moba_block_mean": (_ST, [_P, _I32, _I64, _I32, _I32, _I32, _P, ctypes.c_int, _P]),
    "moba_block_mean_update": (_ST, [_P, _I32, _I64, _I32, _I32, _I32, _I32, _P, ctypes.c_int,
                                     _P]),
    "moba_route": (_ST, [_P, _I32, _I32, _I32, _I64, _I64, _I32, _I32, _P, _P, _P,
                         ctypes.c_size_t, _P]),
    "moba_route_workspace_size": (ctypes.c_size_t, [_I32, _I32, _I32, _I64, _I64, _I32, _I32]),
    "moba_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "moba_last_error": (ctypes.c_char_p, []),
    "moba_abi_version": (_I32, []),
    "moba_profile_enable": (_ST, [_I32]),
    "moba_profile_reset": (_ST, []),
    "moba_profile_read": (_ST, [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double),
                                ctypes.POINTER(ctypes.c_int64)]),
}
for _name, (_res, _args) in _SIGNATURES.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args

EXPORTED = tuple(_SIGNATURES)


class MobaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


def _check(status: int, what: str):
    if status == MOBA_OK:
        return
    msg = f"{what}: {_lib.moba_status_string(status).decode()}: {_lib.moba_last_error().decode()}"
    if status in (MOBA_ERR_INVALID_ARGUMENT, MOBA_ERR_UNSUPPORTED):
        err = ValueError(msg)
        err.status = status
        raise err
    if status == MOBA_ERR_OUT_OF_MEMORY:
        raise MemoryError(msg)
    raise MobaError(status, msg)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MOBA_DTYPE_BF16
    if t.dtype == torch.float32:
        return MOBA_DTYPE_F32
    raise ValueError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _dev_tensor(t, name, dtype=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _stream_ptr(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _shape4(q, k, v):
    """Return (S, Lq, H, D, L, Hkv) for prefill (3-D) or general (4-D) tensors."""
    if q.dim() == 3:
        if k.dim() != 3 or v.dim() != 3:
            raise ValueError("q, k, v must all be 3-D (prefill) or 4-D (batched)")
        L, H, D = q.shape
        Lk, Hkv, Dk = k.shape
        if Lk != L:
            raise ValueError("3-D form needs q_len == kv_len")
        S, Lq = 1, L
    elif q.dim() == 4:
        S, Lq, H, D = q.shape
        Sk, Lk, Hkv, Dk = k.shape
        if Sk != S:
            raise ValueError("batch of q and k differ")
    else:
        raise ValueError("q must be 3-D or 4-D")
    if tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v shapes differ")
    if Dk != D:
        raise ValueError("head_dim of q and k differ")
    return S, Lq, H, D, Lk, Hkv


def _args(q, k, v, out, block_size=64, topk=1, k_block_mean=None, sel_out=None) -> MobaArgs:
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        _dev_tensor(t, name, q.dtype)
    S, Lq, H, D, L, Hkv = _shape4(q, k, v)
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must have the shape of q")
    a = MobaArgs()
    a.struct_size = ctypes.sizeof(MobaArgs)
    a.q, a.k, a.v, a.out = q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr()
    if k_block_mean is not None:
        _dev_tensor(k_block_mean, "k_block_mean", torch.float32)
        nb = -(-L // int(block_size)) if block_size > 0 else 0
        if tuple(k_block_mean.shape) != (S, Hkv, nb, D):
            raise ValueError(f"k_block_mean must be float32 [{S}, {Hkv}, {nb}, {D}]")
        a.k_block_mean = k_block_mean.data_ptr()
    if sel_out is not None:
        _dev_tensor(sel_out, "sel_out", torch.int32)
        if tuple(sel_out.shape) != (S, H, Lq, topk):
            raise ValueError(f"sel_out must be int32 [{S}, {H}, {Lq}, {topk}]")
        a.sel_out = sel_out.data_ptr()
    a.batch, a.n_heads, a.n_kv_heads, a.head_dim = S, H, Hkv, D
    a.block_size, a.topk = int(block_size), int(topk)
    a.q_len, a.kv_len = Lq, L
    a.dtype = _dtype_code(q)
    a.stream = _stream_ptr(q.device)
    return a


def moba_forward(q, k, v, block_size, topk, out=None):
    """MoBA prefill forward (C ``moba_forward``; the library allocates its
    workspace stream-ordered).  q [L, H, D], k, v [L, Hkv, D]."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        _dev_tensor(t, name, q.dtype)
    if q.dim() != 3:
        raise ValueError("moba_forward takes 3-D prefill tensors; use moba_forward_ex")
    S, Lq, H, D, L, Hkv = _shape4(q, k, v)
    out = torch.empty_like(q) if out is None else _dev_tensor(out, "out", q.dtype)
    st = _lib.moba_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(), L, H, Hkv, D,
                           int(block_size), int(topk), out.data_ptr(), _dtype_code(q),
                           _stream_ptr(q.device))
    _check(st, "moba_forward")
    return out


def moba_full_attention(q, k, v, out=None):
    """Full causal attention (C ``moba_full_attention``), prefill layout."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        _dev_tensor(t, name, q.dtype)
    if q.dim() != 3:
        raise ValueError("moba_full_attention takes 3-D prefill tensors; use the _ex form")
    S, Lq, H, D, L, Hkv = _shape4(q, k, v)
    out = torch.empty_like(q) if out is None else _dev_tensor(out, "out", q.dtype)
    st = _lib.moba_full_attention(q.data_ptr(), k.data_ptr(), v.data_ptr(), L, H, Hkv, D,
                                  out.data_ptr(), _dtype_code(q), _stream_ptr(q.device))
    _check(st, "moba_full_attention")
    return out


def moba_workspace_size(q, k, v, block_size, topk, k_block_mean=None, sel_out=None,
                        routed_bytes_limit=0) -> int:
    """Workspace bytes moba_forward_ex needs (C ``moba_workspace_size``)."""
    a = _args(q, k, v, q, block_size, topk, k_block_mean, sel_out)
    a.routed_bytes_limit = int(routed_bytes_limit)
    n = int(_lib.moba_workspace_size(ctypes.byref(a)))
    if n == 0 and _lib.moba_last_error():
        raise ValueError(f"moba_workspace_size: {_lib.moba_last_error().decode()}")
    return n


def moba_full_workspace_size(q, k, v) -> int:
    """Workspace bytes moba_full_attention_ex needs (C ``moba_full_workspace_size``)."""
    a = _args(q, k, v, q)
    n = int(_lib.moba_full_workspace_size(ctypes.byref(a)))
    if n == 0 and _lib.moba_last_error():
        raise ValueError(f"moba_full_workspace_size: {_lib.moba_last_error().decode()}")
    return n


def _workspace_tensor(nbytes: int, device, workspace):
    if nbytes == 0:
        return None
    if workspace is not None:
        # the library checks the size and rejects a short workspace
        return _dev_tensor(workspace, "workspace")
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _kv_lens_ptr(kv_lens, S):
    if kv_lens is None:
        return None
    _dev_tensor(kv_lens, "kv_lens", torch.int32)
    if kv_lens.numel() != S:
        raise ValueError(f"kv_lens must be int32 [{S}] (one cache length per sequence)")
    return kv_lens.data_ptr()


def moba_forward_ex(q, k, v, block_size, topk, *, out=None, k_block_mean=None, sel_out=None,
                    return_selection=False, workspace=None, lse_out=None, return_lse=False,
                    kv_lens=None, routed_bytes_limit=0):
    """General MoBA forward (C ``moba_forward_ex``): batches, q_len <= kv_len,
    optional precomputed block means, optional selection and log-sum-exp
    outputs (what moba_backward_ex needs).  The workspace is a torch
    allocation (or the given uint8 tensor).  Returns ``out``, then the
    selection ``[S, H, Lq, topk]`` if asked, then the log-sum-exp
    ``[S, H, Lq]`` if asked (``[H, ...]`` without the batch axis for 3-D q).
    ``kv_lens`` (int32 ``[S]`` on the device, decode batches with q_len 1):
    the cache length of each sequence; ``k``/``v`` then hold ``kv_len`` rows
    per sequence of which sequence s uses the first ``kv_lens[s]``.
    ``routed_bytes_limit`` (bytes, 0 = the library's 12 GiB): above it large
    bf16 problems route a few KV heads of one sequence at a time, which
    bounds the workspace; the output is the same bits."""
    out = torch.empty_like(q) if out is None else out
    S, Lq, H, D, L, Hkv = _shape4(q, k, v)
    if return_selection and sel_out is None:
        sel_out = torch.empty((S, H, Lq, int(topk)), dtype=torch.int32, device=q.device)
    if return_lse and lse_out is None:
        lse_out = torch.empty((S, H, Lq), dtype=torch.float32, device=q.device)
    if lse_out is not None:
        _dev_tensor(lse_out, "lse_out", torch.float32)
        if lse_out.numel() != S * H * Lq:
            raise ValueError(f"lse_out must be float32 [{S}, {H}, {Lq}]")
    a = _args(q, k, v, out, block_size, topk, k_block_mean, sel_out)
    if lse_out is not None:
        a.lse_out = lse_out.data_ptr()
    a.kv_lens = _kv_lens_ptr(kv_lens, S)
    a.routed_bytes_limit = int(routed_bytes_limit)
    need = int(_lib.moba_workspace_size(ctypes.byref(a)))
    if need == 0 and _lib.moba_last_error():
        _check(_lib.moba_forward_ex(ctypes.byref(a)), "moba_forward_ex")  # raises the error
    ws = _workspace_tensor(need, q.device, workspace)
    if ws is not None:
        a.workspace = ws.data_ptr()
        a.workspace_bytes = ws.numel() * ws.element_size()
    _check(_lib.moba_forward_ex(ctypes.byref(a)), "moba_forward_ex")
    res = [out]
    if return_selection:
        res.append(sel_out[0] if q.dim() == 3 else sel_out)
    if return_lse:
        res.append(lse_out.view(S, H, Lq)[0] if q.dim() == 3 else lse_out.view(S, H, Lq))
    return res[0] if len(res) == 1 else tuple(res)


def moba_forward_noalloc(q, k, v, block_size, topk, *, out=None, k_block_mean=None,
                         sel_out=None, lse_out=None, kv_lens=None):
    """moba_forward_ex without any device allocation (C ``moba_forward_noalloc``):
    the library's static per-GPU scratch array (64 MiB) is the workspace;
    larger problems raise ValueError.  ``out``, ``sel_out`` and ``lse_out``
    are written when given (allocate them beforehand to stay allocation-free);
    returns ``out``."""
    if out is None:
        out = torch.empty_like(q)
    S, Lq, H, D, L, Hkv = _shape4(q, k, v)
    a = _args(q, k, v, out, block_size, topk, k_block_mean, sel_out)
    if lse_out is not None:
        _dev_tensor(lse_out, "lse_out", torch.float32)
        if lse_out.numel() != S * H * Lq:
            raise ValueError(f"lse_out must be float32 [{S}, {H}, {Lq}]")
        a.lse_out = lse_out.data_ptr()
    a.kv_lens = _kv_lens_ptr(kv_lens, S)
    _check(_lib.moba_forward_noalloc(ctypes.byref(a)), "moba_forward_noalloc")
    return out


def moba_route_workspace_size(batch, n_heads, n_kv_heads, q_len, kv_len, block_size,
                              topk) -> int:
    """Workspace bytes of moba_route (C ``moba_route_workspace_size``)."""
    n = int(_lib.moba_route_workspace_size(int(batch), int(n_heads), int(n_kv_heads),
                                           int(q_len), int(kv_len), int(block_size), int(topk)))
    if n == 0:
        raise ValueError(f"moba_route_workspace_size: {_lib.moba_last_error().decode()}")
    return n


def moba_route(sel, n_kv_heads, kv_len, block_size, *, workspace=None):
    """The query -> block dispatch alone (C ``moba_route``): from a selection
    ``sel`` int32 [S, H, Lq, topk] (or [H, Lq, topk]) on the GPU, returns
    ``(bucket_off, list)``: uint32-valued int32 tensors, bucket_off
    [S * Hkv * nb + 1] (entry offsets per (sequence, KV head, block) bucket)
    and the slot ids of the routed entries bucket by bucket, ascending inside
    each bucket (list holds bucket_off[-1] entries)."""
    _dev_tensor(sel, "sel", torch.int32)
    if sel.dim() == 3:
        sel = sel.unsqueeze(0)
    if sel.dim() != 4:
        raise ValueError("sel must be [S, H, Lq, topk] or [H, Lq, topk]")
    S, H, Lq, topk = (int(x) for x in sel.shape)
    nb = -(-int(kv_len) // int(block_size))
    args = (S, H, int(n_kv_heads), Lq, int(kv_len), int(block_size), topk)
    need = int(_lib.moba_route_workspace_size(*args))
    if need == 0:
        raise ValueError(f"moba_route: {_lib.moba_last_error().decode()}")
    ws = _workspace_tensor(need, sel.device, workspace)
    boff = torch.empty(S * int(n_kv_heads) * nb + 1, dtype=torch.int32, device=sel.device)
    lst = torch.empty(max(S * H * Lq * (topk - 1), 1), dtype=torch.int32, device=sel.device)
    st = _lib.moba_route(sel.data_ptr(), *args, boff.data_ptr(), lst.data_ptr(),
                         None if ws is None else ws.data_ptr(),
                         0 if ws is None else ws.numel() * ws.element_size(),
                         _stream_ptr(sel.device))
    _check(st, "moba_route")
    n = int(boff[-1].item())
    return boff, lst[:n]


def _bwd_args(q, k, v, out, dout, lse, sel, dq, dk, dv, block_size, topk) -> MobaBwdArgs:
    for name, t in (("q", q), ("out", out), ("dout", dout), ("dq", dq)):
        _dev_tensor(t, name, q.dtype)
        if tuple(t.shape) != tuple(q.shape):
            raise ValueError(f"{name} must have the shape of q")
    for name, t in (("k", k), ("v", v), ("dk", dk), ("dv", dv)):
        _dev_tensor(t, name, q.dtype)
        if tuple(t.shape) != tuple(k.shape):
            raise ValueError(f"{name} must have the shape of k")
    S, Lq, H, D, L, Hkv = _shape4(q, k, v)
    _dev_tensor(lse, "lse", torch.float32)
    if lse.numel() != S * H * Lq:
        raise ValueError(f"lse must be float32 [{S}, {H}, {Lq}]")
    _dev_tensor(sel, "sel", torch.int32)
    if sel.numel() != S * H * Lq * int(topk):
        raise ValueError(f"sel must be int32 [{S}, {H}, {Lq}, {topk}]")
    a = MobaBwdArgs()
    a.struct_size = ctypes.sizeof(MobaBwdArgs)
    a.q, a.k, a.v, a.out, a.dout = (t.data_ptr() for t in (q, k, v, out, dout))
    a.lse, a.sel = lse.data_ptr(), sel.data_ptr()
    a.dq, a.dk, a.dv = dq.data_ptr(), dk.data_ptr(), dv.data_ptr()
    a.batch, a.n_heads, a.n_kv_heads, a.head_dim = S, H, Hkv, D
    a.block_size, a.topk = int(block_size), int(topk)
    a.q_len, a.kv_len = Lq, L
    a.dtype = _dtype_code(q)
    a.stream = _stream_ptr(q.device)
    return a


def moba_backward_ex(q, k, v, out, dout, lse, sel, block_size, topk, *, dq=None, dk=None,
                     dv=None, workspace=None):
    """Gradients ``(dq, dk, dv)`` of ``sum(out * dout)`` for a MoBA forward (bf16 or fp32)
    (C ``moba_backward_ex``); ``lse`` and ``sel`` are the forward's
    ``return_lse`` / ``return_selection`` outputs for the same q, k, v."""
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    a = _bwd_args(q, k, v, out, dout, lse, sel, dq, dk, dv, block_size, topk)
    need = int(_lib.moba_backward_workspace_size(ctypes.byref(a)))
    if need == 0 and _lib.moba_last_error():
        _check(_lib.moba_backward_ex(ctypes.byref(a)), "moba_backward_ex")  # raises the error
    ws = _workspace_tensor(need, q.device, workspace)
    if ws is not None:
        a.workspace = ws.data_ptr()
        a.workspace_bytes = ws.numel() * ws.element_size()
    _check(_lib.moba_backward_ex(ctypes.byref(a)), "moba_backward_ex")
    return dq, dk, dv


def moba_backward_workspace_size(q, k, v, block_size, topk) -> int:
    """Workspace bytes moba_backward_ex needs for these shapes (0 and
    moba_last_error() for an invalid set)."""
    S, Lq, H, D, L, Hkv = _shape4(q, k, v)
    a = MobaBwdArgs()
    a.struct_size = ctypes.sizeof(MobaBwdArgs)
    fake = 1 << 40   # only checked for NULL and alignment, never dereferenced
    a.q = a.k = a.v = a.out = a.dout = a.lse = a.sel = a.dq = a.dk = a.dv = fake
    a.batch, a.n_heads, a.n_kv_heads, a.head_dim = S, H, Hkv, D
    a.block_size, a.topk = int(block_size), int(topk)
    a.q_len, a.kv_len = Lq, L
    a.dtype = _dtype_code(q)
    return int(_lib.moba_backward_workspace_size(ctypes.byref(a)))


def _cu_array(cu, batch=None):
    a = np.ascontiguousarray(np.asarray(cu.cpu() if hasattr(cu, "cpu") else cu, dtype=np.int64))
    if a.ndim != 1 or a.size < 2 or (batch is not None and a.size != batch + 1):
        raise ValueError("cu_seqlens must be a 1-D sequence of batch + 1 offsets")
    return a


def _varlen_args(q, k, v, out, cu_q, cu_k, block_size, topk, sel=None, lse=None):
    for name, t, ref in (("q", q, q), ("out", out, q)):
        _dev_tensor(t, name, q.dtype)
        if t.dim() != 3 or tuple(t.shape) != tuple(ref.shape):
            raise ValueError(f"{name} must be [total_q, n_heads, head_dim]")
    for name, t in (("k", k), ("v", v)):
        _dev_tensor(t, name, q.dtype)
        if t.dim() != 3 or tuple(t.shape) != tuple(k.shape):
            raise ValueError(f"{name} must be [total_k, n_kv_heads, head_dim]")
    Tq, H, D = q.shape
    Tk, Hkv, _ = k.shape
    if cu_q[-1] != Tq or cu_k[-1] != Tk or cu_q.size != cu_k.size:
        raise ValueError("cu_seqlens must end at the packed lengths and have equal sizes")
    a = MobaVarlenArgs()
    a.struct_size = ctypes.sizeof(MobaVarlenArgs)
    a.q, a.k, a.v, a.out = q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr()
    a.cu_seqlens_q = cu_q.ctypes.data
    a.cu_seqlens_k = cu_k.ctypes.data
    if sel is not None:
        _dev_tensor(sel, "sel", torch.int32)
        if sel.numel() != H * Tq * int(topk):
            raise ValueError(f"sel must hold n_heads * total_q * topk = {H * Tq * int(topk)} int32")
        a.sel = sel.data_ptr()
    if lse is not None:
        _dev_tensor(lse, "lse", torch.float32)
        if lse.numel() != H * Tq:
            raise ValueError(f"lse must hold n_heads * total_q = {H * Tq} float32")
        a.lse = lse.data_ptr()
    a.batch = cu_q.size - 1
    a.n_heads, a.n_kv_heads, a.head_dim = H, Hkv, D
    a.block_size, a.topk = int(block_size), int(topk)
    a.dtype = _dtype_code(q)
    a.stream = _stream_ptr(q.device)
    return a


def _varlen_run(fn, a, backward, device, workspace, what):
    need = int(_lib.moba_varlen_workspace_size(ctypes.byref(a), int(backward)))
    if need == 0 and _lib.moba_last_error():
        _check(fn(ctypes.byref(a)), what)  # raises the error
    ws = _workspace_tensor(need, device, workspace)
    if ws is not None:
        a.workspace = ws.data_ptr()
        a.workspace_bytes = ws.numel() * ws.element_size()
    _check(fn(ctypes.byref(a)), what)


def moba_forward_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, block_size, topk, *, out=None,
                        return_selection=False, return_lse=False, workspace=None):
    """Packed variable-length MoBA forward (C ``moba_forward_varlen``): q
    [total_q, H, D], k and v [total_k, Hkv, D], sequence s at rows
    cu_seqlens_q[s]:cu_seqlens_q[s+1] of q and cu_seqlens_k[s]:... of k (host
    offsets).  The selection (flat, per sequence an [H, q_len_s, topk] block)
    and log-sum-exp (per sequence [H, q_len_s]) come back flat when asked."""
    cu_q = _cu_array(cu_seqlens_q)
    cu_k = _cu_array(cu_seqlens_k, cu_q.size - 1)
    out = torch.empty_like(q) if out is None else out
    H = q.shape[1]
    sel = (torch.empty(H * q.shape[0] * int(topk), dtype=torch.int32, device=q.device)
           if return_selection else None)
    lse = (torch.empty(H * q.shape[0], dtype=torch.float32, device=q.device)
           if return_lse else None)
    a = _varlen_args(q, k, v, out, cu_q, cu_k, block_size, topk, sel, lse)
    _varlen_run(_lib.moba_forward_varlen, a, False, q.device, workspace, "moba_forward_varlen")
    res = [out] + ([sel] if return_selection else []) + ([lse] if return_lse else [])
    return res[0] if len(res) == 1 else tuple(res)


def moba_backward_varlen(q, k, v, out, dout, lse, sel, cu_seqlens_q, cu_seqlens_k, block_size,
                         topk, *, workspace=None):
    """Packed variable-length backward (C ``moba_backward_varlen``): the
    forward's flat selection and log-sum-exp in, (dq, dk, dv) out."""
    cu_q = _cu_array(cu_seqlens_q)
    cu_k = _cu_array(cu_seqlens_k, cu_q.size - 1)
    _dev_tensor(dout, "dout", q.dtype)
    if tuple(dout.shape) != tuple(q.shape):
        raise ValueError("dout must have the shape of q")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    a = _varlen_args(q, k, v, out, cu_q, cu_k, block_size, topk, sel, lse)
    a.dout, a.dq, a.dk, a.dv = dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr()
    _varlen_run(_lib.moba_backward_varlen, a, True, q.device, workspace, "moba_backward_varlen")
    return dq, dk, dv


def moba_varlen_workspace_size(q, k, v, cu_seqlens_q, cu_seqlens_k, block_size, topk,
                               backward=False) -> int:
    """Workspace bytes of moba_forward_varlen (or moba_backward_varlen)."""
    cu_q = _cu_array(cu_seqlens_q)
    cu_k = _cu_array(cu_seqlens_k, cu_q.size - 1)
    a = _varlen_args(q, k, v, q, cu_q, cu_k, block_size, topk)
    if backward:
        fake = 1 << 40   # only checked for NULL, never dereferenced by a size query
        a.dout = a.dq = a.dk = a.dv = a.sel = a.lse = fake
    return int(_lib.moba_varlen_workspace_size(ctypes.byref(a), int(bool(backward))))


def moba_full_attention_ex(q, k, v, *, out=None, workspace=None, kv_lens=None):
    """Full causal attention in the general form (C ``moba_full_attention_ex``);
    ``kv_lens`` as for moba_forward_ex."""
    out = torch.empty_like(q) if out is None else out
    a = _args(q, k, v, out)
    a.kv_lens = _kv_lens_ptr(kv_lens, _shape4(q, k, v)[0])
    need = int(_lib.moba_full_workspace_size(ctypes.byref(a)))
    if need == 0 and _lib.moba_last_error():
        _check(_lib.moba_full_attention_ex(ctypes.byref(a)), "moba_full_attention_ex")
    ws = _workspace_tensor(need, q.device, workspace)
    if ws is not None:
        a.workspace = ws.data_ptr()
        a.workspace_bytes = ws.numel() * ws.element_size()
    _check(_lib.moba_full_attention_ex(ctypes.byref(a)), "moba_full_attention_ex")
    return out


def moba_naive_workspace_size(q, k, v, block_size, topk, k_block_mean=None, sel_out=None) -> int:
    """Workspace bytes moba_naive_ex needs (C ``moba_naive_workspace_size``)."""
    a = _args(q, k, v, q, block_size, topk, k_block_mean, sel_out)
    n = int(_lib.moba_naive_workspace_size(ctypes.byref(a)))
    if n == 0 and _lib.moba_last_error():
        raise ValueError(f"moba_naive_workspace_size: {_lib.moba_last_error().decode()}")
    return n


def moba_naive_ex(q, k, v, block_size, topk, *, out=None, k_block_mean=None, sel_out=None,
                  return_selection=False, workspace=None):
    """Mask-based MoBA (C ``moba_naive_ex``): the same gate and selection as
    moba_forward_ex, then dense scores for every (query, key) pair, the block
    mask, row softmax and P V.  A comparison baseline; bf16 only.  Returns
    ``out`` (and the selection ``[S, H, Lq, topk]`` if asked)."""
    out = torch.empty_like(q) if out is None else out
    S, Lq, H, D, L, Hkv = _shape4(q, k, v)
    if return_selection and sel_out is None:
        sel_out = torch.empty((S, H, Lq, int(topk)), dtype=torch.int32, device=q.device)
    a = _args(q, k, v, out, block_size, topk, k_block_mean, sel_out)
    need = int(_lib.moba_naive_workspace_size(ctypes.byref(a)))
    if need == 0 and _lib.moba_last_error():
        _check(_lib.moba_naive_ex(ctypes.byref(a)), "moba_naive_ex")  # raises the error
    ws = _workspace_tensor(need, q.device, workspace)
    if ws is not None:
        a.workspace = ws.data_ptr()
        a.workspace_bytes = ws.numel() * ws.element_size()
    _check(_lib.moba_naive_ex(ctypes.byref(a)), "moba_naive_ex")
    if return_selection:
        return out, (sel_out[0] if q.dim() == 3 else sel_out)
    return out


def moba_block_mean(k, block_size, out=None, first_block=0):
    """Block-mean keys: k [S, L, Hkv, D] (or [L, Hkv, D]) -> fp32 [S, Hkv, nb, D],
    nb = ceil(L / block_size); a partial last block is the mean of the keys it holds.

    first_block > 0 recomputes only blocks first_block..nb-1 of ``out`` (which
    must then be given) and leaves the others as they are: the incremental
    update of a growing cache (moba_block_mean_update)."""
    _dev_tensor(k, "k")
    k4 = k if k.dim() == 4 else k.unsqueeze(0)
    S, L, Hkv, D = k4.shape
    nb = -(-L // int(block_size)) if block_size > 0 else 0
    if out is None:
        if first_block:
            raise ValueError("first_block > 0 updates an existing out tensor")
        out = torch.empty((S, Hkv, max(nb, 1), D), dtype=torch.float32, device=k.device)
    else:
        _dev_tensor(out, "out", torch.float32)
        if tuple(out.shape) not in ((S, Hkv, nb, D), (Hkv, nb, D) if S == 1 else ()):
            raise ValueError(f"out must be float32 [{S}, {Hkv}, {nb}, {D}]")
    if first_block:
        st = _lib.moba_block_mean_update(k4.data_ptr(), S, L, Hkv, D, int(block_size),
                                         int(first_block), out.data_ptr(), _dtype_code(k4),
                                         _stream_ptr(k.device))
    else:
        st = _lib.moba_block_mean(k4.data_ptr(), S, L, Hkv, D, int(block_size), out.data_ptr(),
                                  _dtype_code(k4), _stream_ptr(k.device))
    _check(st, "moba_block_mean_update" if first_block else "moba_block_mean")
    return out


def moba_block_mean_update(k, block_size, first_block, out):
    """Recompute blocks first_block..nb-1 of the block means ``out`` in place
    (a cache that grew); blocks before first_block are left as they are."""
    return moba_block_mean(k, block_size, out=out, first_block=int(first_block))


def moba_status_string(status: int) -> str:
    return _lib.moba_status_string(int(status)).decode()


def moba_last_error() -> str:
    return _lib.moba_last_error().decode()


def moba_abi_version() -> int:
    return int(_lib.moba_abi_version())


def moba_profile_enable(on: bool = True):
    _check(_lib.moba_profile_enable(1 if on else 0), "moba_profile_enable")


def moba_profile_reset():
    _check(_lib.moba_profile_reset(), "moba_profile_reset")


def moba_profile_read(name: str):
    """Return (total_ms, launches) recorded for kernel `name` since the last reset."""
    ms = ctypes.c_double(0.0)
    n = ctypes.c_int64(0)
    _check(_lib.moba_profile_read(name.encode(), ctypes.byref(ms), ctypes.byref(n)),
           "moba_profile_read")
    return ms.value, n.value


KERNEL_NAMES = ("block_mean", "transpose_v", "gate_topk", "route_count", "route_scan_rows",
                "route_scan_buckets", "route_scatter", "attn_routed", "attn_own_merge",
                "attn_full", "decode_plan", "decode_attn", "decode_merge", "merge_partials",
                "pool_transpose", "block_mean_finalize", "route_scan_small", "bwd_dot",
                "bwd_tail", "bwd_dq_routed", "bwd_dq_own", "bwd_dkdv", "naive_scores",
                "naive_softmax", "naive_pv", "bwd_entries")
