"""ctypes binding of libfa.so: the same entry points as include/fa.h.

Argument marshalling only: tensors are turned into device pointers and
sizes, the stream into its HIP handle, and a non-OK status into an
exception. Every step of the computation runs in the library's HIP kernels;
there is no fallback of any kind, and a missing library is an error.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

from .build import LIB

FA_F32, FA_F16, FA_BF16 = 0, 1, 2
FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_WORKSPACE, FA_ERR_HIP = 0, -1, -2, -3, -4
FA_ERR_TOO_LARGE = -5
FA_NOALLOC_MAX_ROWS = 1 << 22  # fa_bwd_noalloc's built-in scratch, in query rows

EXPORTS = ("fa_fwd", "fa_bwd", "fa_bwd_workspace_bytes", "fa_bwd_noalloc", "fa_bwd_dsum", "fa_bwd_dkdv",
           "fa_bwd_dq", "fa_fwd_partial", "fa_merge", "fa_fwd_split_workspace_bytes",
           "fa_fwd_split", "fa_fwd_gqa", "fa_bwd_gqa_workspace_bytes", "fa_bwd_gqa",
           "fa_fwd_sparse", "fa_bwd_sparse", "fa_sparse_plan",
           "fa_fwd_sparse_planned_workspace_bytes", "fa_fwd_sparse_planned",
           "fa_bwd_sparse_planned_workspace_bytes", "fa_bwd_sparse_planned", "fa_fp8_quantize", "fa_fwd_fp8",
           "fa_fwd_fp8_workspace_bytes", "fa_fwd_fp8_incoherent", "fa_strerror")

_DTYPE = {torch.float32: FA_F32, torch.float16: FA_F16, torch.bfloat16: FA_BF16}
_lib: Optional[ctypes.CDLL] = None


class FaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status}: {fa_strerror(status)}")


def lib() -> ctypes.CDLL:
    """Load libfa.so from the package directory (raises if it is not built).
    FA_LIBRARY in the environment names another build of the same sources
    to load instead (the host-sanitized one, for the tests)."""
    global _lib
    if _lib is not None:
        return _lib
    path = os.environ.get("FA_LIBRARY", LIB)
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m exact_io_aware_07_amd.build`")
    _lib = bind(ctypes.CDLL(path))
    return _lib


def bind(L: ctypes.CDLL) -> ctypes.CDLL:
    """Set the argument and result types of every entry point on a loaded
    copy of the library (libfa.so, or a variant built from the same
    sources)."""
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, vp, i, i]
    L.fa_fwd.restype = i
    L.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, vp, sz, vp, i, i]
    L.fa_bwd.restype = i
    L.fa_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, vp, i, i]
    L.fa_bwd_noalloc.restype = i
    L.fa_bwd_workspace_bytes.argtypes = [i, i, i, i]
    L.fa_bwd_workspace_bytes.restype = sz
    L.fa_bwd_dsum.argtypes = [vp, vp, vp, i, i, i, i, vp, i, i]
    L.fa_bwd_dsum.restype = i
    L.fa_bwd_dkdv.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, vp, i]
    L.fa_bwd_dkdv.restype = i
    L.fa_bwd_dq.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, vp, i, i]
    L.fa_bwd_dq.restype = i
    L.fa_fwd_partial.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, i, vp, vp, i]
    L.fa_fwd_partial.restype = i
    L.fa_merge.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_longlong, i, vp, i]
    L.fa_merge.restype = i
    L.fa_fwd_split_workspace_bytes.argtypes = [i, i, i, i, i]
    L.fa_fwd_split_workspace_bytes.restype = sz
    L.fa_fwd_split.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, i, vp, sz, vp, i, i]
    L.fa_fwd_split.restype = i
    L.fa_fwd_gqa.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, vp, i, i]
    L.fa_fwd_gqa.restype = i
    L.fa_bwd_gqa_workspace_bytes.argtypes = [i, i, i, i, i]
    L.fa_bwd_gqa_workspace_bytes.restype = sz
    L.fa_bwd_gqa.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, vp, sz,
                             vp, i, i]
    L.fa_bwd_gqa.restype = i
    ll = ctypes.c_longlong
    L.fa_fwd_sparse.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, vp, ll, ll, vp, i, i]
    L.fa_fwd_sparse.restype = i
    L.fa_bwd_sparse.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, vp, ll,
                                ll, vp, sz, vp, i, i]
    L.fa_bwd_sparse.restype = i
    L.fa_sparse_plan.argtypes = [vp, ll, ll, i, i, i, i, vp, ll, vp]
    L.fa_sparse_plan.restype = i
    L.fa_fwd_sparse_planned_workspace_bytes.argtypes = [i, i, i, i, vp]
    L.fa_fwd_sparse_planned_workspace_bytes.restype = sz
    L.fa_fwd_sparse_planned.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, vp, ll, ll, vp, vp,
                                        vp, sz, vp, i, i]
    L.fa_fwd_sparse_planned.restype = i
    L.fa_bwd_sparse_planned_workspace_bytes.argtypes = [i, i, i, i, vp]
    L.fa_bwd_sparse_planned_workspace_bytes.restype = sz
    L.fa_bwd_sparse_planned.argtypes = ([vp] * 9 + [i, i, i, i, f, i, vp, vp, ll, ll, vp, vp, vp, sz,
                                                     vp, i, i])
    L.fa_bwd_sparse_planned.restype = i
    L.fa_fp8_quantize.argtypes = [vp] * 11 + [i, i, i, i, vp, i]
    L.fa_fp8_quantize.restype = i
    L.fa_fwd_fp8.argtypes = [vp] * 6 + [i, vp, vp, i, i, i, i, f, i, vp, vp, i]
    L.fa_fwd_fp8.restype = i
    L.fa_fwd_fp8_workspace_bytes.argtypes = [i, i, i, i]
    L.fa_fwd_fp8_workspace_bytes.restype = sz
    L.fa_fwd_fp8_incoherent.argtypes = [vp] * 6 + [i, i, i, i, f, i, vp, vp, sz, vp, i, i]
    L.fa_fwd_fp8_incoherent.restype = i
    L.fa_strerror.argtypes = [i]
    L.fa_strerror.restype = ctypes.c_char_p
    return L


def fa_strerror(status: int) -> str:
    return lib().fa_strerror(int(status)).decode()


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream, device) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _torch_stream(stream, device):
    """The torch stream object of ``stream`` (None: torch's current stream;
    a raw HIP handle is wrapped)."""
    if stream is None:
        return torch.cuda.current_stream(device)
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream), device=device)


def _temp(nbytes: int, device, stream) -> torch.Tensor:
    """A device byte buffer the library's kernels use on ``stream``.

    torch's caching allocator hands a freed block to the next allocation of
    the stream it was allocated on, without waiting for work on other
    streams. The buffer is therefore allocated on ``stream`` itself, so that
    once it is dropped it is reused only behind the kernels already enqueued
    there."""
    with torch.cuda.stream(_torch_stream(stream, device)):
        return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


def _check_tensor(name: str, t: torch.Tensor, shape, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")


def _check_o(o: torch.Tensor, q: torch.Tensor) -> int:
    """O for a backward: q's shape, in q's dtype or fp32 (the forward's fp32
    output); returns its dtype code."""
    _check_tensor("o", o, q.shape)
    if o.dtype not in (q.dtype, torch.float32):
        raise ValueError(f"o has dtype {o.dtype}, expected {q.dtype} or torch.float32")
    return _DTYPE[o.dtype]


def _kv(kv_len: Optional[torch.Tensor], B: int) -> Optional[int]:
    if kv_len is None:
        return None
    _check_tensor("kv_len", kv_len, (B,), torch.int32)
    return kv_len.data_ptr()


def fa_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
           scale: float, causal: bool = False, kv_len: Optional[torch.Tensor] = None,
           stream=None) -> None:
    """Enqueue the forward on ``stream`` (default: torch's current stream).

    q, k, v: [B, H, N, d] device tensors of one dtype; o: [B, H, N, d] in that
    dtype or fp32; lse: [B, H, N] fp32; kv_len: int32 [B] or None.
    """
    B, H, N, d = q.shape
    for name, t in (("k", k), ("v", v)):
        _check_tensor(name, t, q.shape, q.dtype)
    _check_tensor("q", q, q.shape)
    _check_tensor("o", o, q.shape)
    _check_tensor("lse", lse, (B, H, N), torch.float32)
    st = lib().fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, float(scale),
                      int(bool(causal)), _kv(kv_len, B), _stream(stream, q.device),
                      _DTYPE.get(q.dtype, -99), _DTYPE.get(o.dtype, -99))
    if st != FA_OK:
        raise FaError(st, "fa_fwd")


def fa_bwd_workspace_bytes(B: int, H: int, N: int, d: int) -> int:
    return int(lib().fa_bwd_workspace_bytes(B, H, N, d))


def fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, scale: float, causal: bool = False,
           kv_len: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
           stream=None) -> None:
    """Enqueue the backward; writes dq, dk, dv ([B, H, N, d], input dtype).

    ``workspace`` is a device tensor of at least fa_bwd_workspace_bytes()
    bytes (allocated here when None).
    """
    B, H, N, d = q.shape
    for name, t in (("k", k), ("v", v), ("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv)):
        _check_tensor(name, t, q.shape, q.dtype)
    _check_tensor("q", q, q.shape)
    o_dt = _check_o(o, q)
    _check_tensor("lse", lse, (B, H, N), torch.float32)
    need = fa_bwd_workspace_bytes(B, H, N, d)
    if workspace is None:
        workspace = _temp(need, q.device, stream)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib().fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
                      _ptr(dk), _ptr(dv), B, H, N, d, float(scale), int(bool(causal)),
                      _kv(kv_len, B), _ptr(workspace), ws_bytes, _stream(stream, q.device),
                      _DTYPE.get(q.dtype, -99), o_dt)
    if st != FA_OK:
        raise FaError(st, "fa_bwd")


def fa_bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, scale: float, causal: bool = False,
                   kv_len: Optional[torch.Tensor] = None, stream=None) -> None:
    """fa_bwd with its workspace in the library's own device array (at most
    FA_NOALLOC_MAX_ROWS = B * H * N rows); allocates nothing."""
    B, H, N, d = q.shape
    for name, t in (("k", k), ("v", v), ("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv)):
        _check_tensor(name, t, q.shape, q.dtype)
    _check_tensor("q", q, q.shape)
    o_dt = _check_o(o, q)
    _check_tensor("lse", lse, (B, H, N), torch.float32)
    st = lib().fa_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
                              _ptr(dk), _ptr(dv), B, H, N, d, float(scale), int(bool(causal)),
                              _kv(kv_len, B), _stream(stream, q.device), _DTYPE.get(q.dtype, -99), o_dt)
    if st != FA_OK:
        raise FaError(st, "fa_bwd_noalloc")


def fa_bwd_dsum(o, dout, dsum, stream=None) -> None:
    """D_i alone: dsum[b, h, i] = sum_c dout * o (fp32 [B, H, N]); o in
    dout's dtype or fp32."""
    B, H, N, d = o.shape
    _check_tensor("dout", dout, o.shape)
    o_dt = _check_o(o, dout)
    _check_tensor("dsum", dsum, (B, H, N), torch.float32)
    st = lib().fa_bwd_dsum(_ptr(o), _ptr(dout), _ptr(dsum), B, H, N, d, _stream(stream, o.device),
                           _DTYPE.get(dout.dtype, -99), o_dt)
    if st != FA_OK:
        raise FaError(st, "fa_bwd_dsum")


def fa_bwd_dkdv(q, k, v, dout, lse, dsum, dk, dv, scale: float, causal: bool = False,
                kv_len: Optional[torch.Tensor] = None, stream=None) -> None:
    """Backward stage after fa_bwd_dq (or fa_bwd_dsum): writes dk, dv."""
    B, H, N, d = q.shape
    for name, t in (("k", k), ("v", v), ("dout", dout), ("dk", dk), ("dv", dv)):
        _check_tensor(name, t, q.shape, q.dtype)
    _check_tensor("q", q, q.shape)
    _check_tensor("lse", lse, (B, H, N), torch.float32)
    _check_tensor("dsum", dsum, (B, H, N), torch.float32)
    st = lib().fa_bwd_dkdv(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(lse), _ptr(dsum), _ptr(dk),
                           _ptr(dv), B, H, N, d, float(scale), int(bool(causal)), _kv(kv_len, B),
                           _stream(stream, q.device), _DTYPE.get(q.dtype, -99))
    if st != FA_OK:
        raise FaError(st, "fa_bwd_dkdv")


def fa_bwd_dq(q, k, v, o, dout, lse, dsum, dq, scale: float, causal: bool = False,
              kv_len: Optional[torch.Tensor] = None, stream=None) -> None:
    """Backward stage: writes dq and dsum (D_i = rowsum(dout * o), fp32 [B, H, N])."""
    B, H, N, d = q.shape
    for name, t in (("k", k), ("v", v), ("dout", dout), ("dq", dq)):
        _check_tensor(name, t, q.shape, q.dtype)
    _check_tensor("q", q, q.shape)
    o_dt = _check_o(o, q)
    _check_tensor("lse", lse, (B, H, N), torch.float32)
    _check_tensor("dsum", dsum, (B, H, N), torch.float32)
    st = lib().fa_bwd_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dsum),
                         _ptr(dq), B, H, N, d, float(scale), int(bool(causal)), _kv(kv_len, B),
                         _stream(stream, q.device), _DTYPE.get(q.dtype, -99), o_dt)
    if st != FA_OK:
        raise FaError(st, "fa_bwd_dq")


def fa_fwd_partial(q, k, v, o_part, lse_part, scale: float, causal: bool = False,
                   q_pos0: int = 0, k_pos0: int = 0, kv_len=None, stream=None) -> None:
    """Enqueue attention of q [B, H, Nq, d] (positions q_pos0 + i) over k, v
    [B, H, Nk, d] (positions k_pos0 + j): o_part fp32 [B, H, Nq, d], lse_part
    fp32 [B, H, Nq]."""
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    _check_tensor("q", q, q.shape)
    for name, t in (("k", k), ("v", v)):
        _check_tensor(name, t, (B, H, Nk, d), q.dtype)
    _check_tensor("o_part", o_part, (B, H, Nq, d), torch.float32)
    _check_tensor("lse_part", lse_part, (B, H, Nq), torch.float32)
    st = lib().fa_fwd_partial(_ptr(q), _ptr(k), _ptr(v), _ptr(o_part), _ptr(lse_part), B, H, Nq,
                              Nk, d, float(scale), int(bool(causal)), int(q_pos0), int(k_pos0),
                              _kv(kv_len, B), _stream(stream, q.device), _DTYPE.get(q.dtype, -99))
    if st != FA_OK:
        raise FaError(st, "fa_fwd_partial")


def fa_merge(o_a, lse_a, o_b, lse_b, o, lse, stream=None) -> None:
    """Enqueue (o, lse) = merge((o_a, lse_a), (o_b, lse_b)): o_a, o_b fp32
    [..., d]; lse_a, lse_b, lse fp32 [...]; o [..., d] fp32/fp16/bf16 (may be
    o_a, with lse = lse_a, when fp32)."""
    d = o_a.shape[-1]
    rows = lse_a.numel()
    for name, t in (("o_a", o_a), ("o_b", o_b)):
        _check_tensor(name, t, o_a.shape, torch.float32)
    for name, t in (("lse_a", lse_a), ("lse_b", lse_b), ("lse", lse)):
        _check_tensor(name, t, lse_a.shape, torch.float32)
    _check_tensor("o", o, o_a.shape)
    if tuple(o_a.shape[:-1]) != tuple(lse_a.shape):
        raise ValueError("o_a and lse_a disagree on the row shape")
    st = lib().fa_merge(_ptr(o_a), _ptr(lse_a), _ptr(o_b), _ptr(lse_b), _ptr(o), _ptr(lse), rows,
                        d, _stream(stream, o_a.device), _DTYPE.get(o.dtype, -99))
    if st != FA_OK:
        raise FaError(st, "fa_merge")


def fa_fwd_split_workspace_bytes(B: int, H: int, N: int, d: int, num_splits: int) -> int:
    return int(lib().fa_fwd_split_workspace_bytes(B, H, N, d, num_splits))


def fa_fwd_split(q, k, v, o, lse, scale: float, causal: bool = False, kv_len=None,
                 num_splits: int = 2, workspace=None, stream=None) -> None:
    """Enqueue the key-split forward (same results as fa_fwd). ``workspace``
    is a device tensor of at least fa_fwd_split_workspace_bytes() bytes, or
    None to let torch allocate one here (plumbing only)."""
    B, H, N, d = q.shape
    for name, t in (("k", k), ("v", v)):
        _check_tensor(name, t, q.shape, q.dtype)
    _check_tensor("q", q, q.shape)
    _check_tensor("o", o, q.shape)
    _check_tensor("lse", lse, (B, H, N), torch.float32)
    need = fa_fwd_split_workspace_bytes(B, H, N, d, num_splits)
    if workspace is None and need:
        workspace = _temp(need, q.device, stream)
    if workspace is not None and not workspace.is_cuda:
        raise ValueError("workspace must be a device tensor")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().fa_fwd_split(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d,
                            float(scale), int(bool(causal)), _kv(kv_len, B), int(num_splits),
                            _ptr(workspace), ws_bytes, _stream(stream, q.device),
                            _DTYPE.get(q.dtype, -99), _DTYPE.get(o.dtype, -99))
    if st != FA_OK:
        raise FaError(st, "fa_fwd_split")


def _gqa_shapes(q, k):
    B, H, N, d = q.shape
    if k.dim() != 4 or k.shape[0] != B or k.shape[2] != N or k.shape[3] != d:
        raise ValueError(f"k has shape {tuple(k.shape)}, expected [{B}, Hkv, {N}, {d}]")
    return B, H, int(k.shape[1]), N, d


def fa_fwd_gqa(q, k, v, o, lse, scale: float, causal: bool = False, kv_len=None,
               stream=None) -> None:
    """Enqueue grouped-query attention: q, o [B, H, N, d]; k, v [B, Hkv, N, d]
    with H % Hkv == 0 (query head h uses K/V head h // (H // Hkv)); lse fp32
    [B, H, N]."""
    B, H, Hkv, N, d = _gqa_shapes(q, k)
    _check_tensor("q", q, q.shape)
    for name, t in (("k", k), ("v", v)):
        _check_tensor(name, t, (B, Hkv, N, d), q.dtype)
    _check_tensor("o", o, q.shape)
    _check_tensor("lse", lse, (B, H, N), torch.float32)
    st = lib().fa_fwd_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Hkv, N, d,
                          float(scale), int(bool(causal)), _kv(kv_len, B),
                          _stream(stream, q.device), _DTYPE.get(q.dtype, -99),
                          _DTYPE.get(o.dtype, -99))
    if st != FA_OK:
        raise FaError(st, "fa_fwd_gqa")


def fa_bwd_gqa_workspace_bytes(B: int, H: int, Hkv: int, N: int, d: int) -> int:
    return int(lib().fa_bwd_gqa_workspace_bytes(B, H, Hkv, N, d))


def fa_bwd_gqa(q, k, v, o, dout, lse, dq, dk, dv, scale: float, causal: bool = False,
               kv_len=None, workspace=None, stream=None) -> None:
    """Enqueue the grouped-query backward: dq [B, H, N, d]; dk, dv
    [B, Hkv, N, d], each the sum over the K/V head's query heads."""
    B, H, Hkv, N, d = _gqa_shapes(q, k)
    for name, t in (("dout", dout), ("dq", dq)):
        _check_tensor(name, t, q.shape, q.dtype)
    o_dt = _check_o(o, q)
    for name, t in (("k", k), ("v", v), ("dk", dk), ("dv", dv)):
        _check_tensor(name, t, (B, Hkv, N, d), q.dtype)
    _check_tensor("q", q, q.shape)
    _check_tensor("lse", lse, (B, H, N), torch.float32)
    need = fa_bwd_gqa_workspace_bytes(B, H, Hkv, N, d)
    if workspace is None:
        workspace = _temp(need, q.device, stream)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib().fa_bwd_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
                          _ptr(dk), _ptr(dv), B, H, Hkv, N, d, float(scale), int(bool(causal)),
                          _kv(kv_len, B), _ptr(workspace), ws_bytes, _stream(stream, q.device),
                          _DTYPE.get(q.dtype, -99), o_dt)
    if st != FA_OK:
        raise FaError(st, "fa_bwd_gqa")


def _mask_strides(block_mask, B: int, H: int, N: int, device_ok: bool = True):
    """Element strides (batch, head) of a uint8 block mask shaped [nb, nb],
    [H, nb, nb] or [B, H, nb, nb] (nb = ceil(N / 128)); a missing leading
    axis, or one of extent 1, is shared (stride 0). ``device_ok``: the mask
    must be a device tensor (else a CPU one)."""
    nb = (N + 127) // 128
    if block_mask.dtype != torch.uint8:
        raise ValueError("block_mask must be uint8")
    if block_mask.is_cuda != device_ok or not block_mask.is_contiguous():
        raise ValueError("block_mask must be a contiguous " + ("device" if device_ok else "CPU") + " tensor")
    shp = tuple(block_mask.shape)
    if len(shp) < 2 or shp[-2:] != (nb, nb):
        raise ValueError(f"block_mask has shape {shp}, expected [..., {nb}, {nb}]")
    lead = (1,) * (4 - len(shp)) + shp[:-2]
    if len(lead) != 2 or lead[0] not in (1, B) or lead[1] not in (1, H):
        raise ValueError(f"block_mask has shape {shp}, expected [B or 1, H or 1, {nb}, {nb}]")
    sh = nb * nb if lead[1] == H and H > 1 else 0
    sb = lead[1] * nb * nb if lead[0] == B and B > 1 else 0
    return sb, sh


def fa_fwd_sparse(q, k, v, o, lse, block_mask, scale: float, causal: bool = False, kv_len=None,
                  stream=None) -> None:
    """Enqueue block-sparse attention: like fa_fwd, restricted to the 128x128
    (query block, key block) pairs ``block_mask`` (uint8, nonzero keeps)
    keeps; see _mask_strides for its accepted shapes."""
    B, H, N, d = q.shape
    for name, t in (("k", k), ("v", v)):
        _check_tensor(name, t, q.shape, q.dtype)
    _check_tensor("q", q, q.shape)
    _check_tensor("o", o, q.shape)
    _check_tensor("lse", lse, (B, H, N), torch.float32)
    sb, sh = _mask_strides(block_mask, B, H, N)
    st = lib().fa_fwd_sparse(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d,
                             float(scale), int(bool(causal)), _kv(kv_len, B), _ptr(block_mask),
                             sb, sh, _stream(stream, q.device), _DTYPE.get(q.dtype, -99),
                             _DTYPE.get(o.dtype, -99))
    if st != FA_OK:
        raise FaError(st, "fa_fwd_sparse")


def fa_bwd_sparse(q, k, v, o, dout, lse, dq, dk, dv, block_mask, scale: float,
                  causal: bool = False, kv_len=None, workspace=None, stream=None) -> None:
    """Enqueue the block-sparse backward (gradients of fa_fwd_sparse's output)."""
    B, H, N, d = q.shape
    for name, t in (("k", k), ("v", v), ("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv)):
        _check_tensor(name, t, q.shape, q.dtype)
    _check_tensor("q", q, q.shape)
    o_dt = _check_o(o, q)
    _check_tensor("lse", lse, (B, H, N), torch.float32)
    sb, sh = _mask_strides(block_mask, B, H, N)
    need = fa_bwd_workspace_bytes(B, H, N, d)
    if workspace is None:
        workspace = _temp(need, q.device, stream)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib().fa_bwd_sparse(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
                             _ptr(dk), _ptr(dv), B, H, N, d, float(scale), int(bool(causal)),
                             _kv(kv_len, B), _ptr(block_mask), sb, sh, _ptr(workspace), ws_bytes,
                             _stream(stream, q.device), _DTYPE.get(q.dtype, -99), o_dt)
    if st != FA_OK:
        raise FaError(st, "fa_bwd_sparse")


def fa_sparse_plan(block_mask, B: int, H: int, N: int, causal: bool = False) -> dict:
    """Host-side plan of the planned block-sparse entry points (see
    include/fa.h) from a CPU uint8 block mask of the shapes fa_fwd_sparse
    accepts. Returns, on the CPU, {"plan": int32 flat array, "counts": int32
    [8]} and views of the plan's four parts as [n, 4] arrays: "col_items",
    "cols", "row_items", "rows"."""
    if block_mask.is_cuda or block_mask.dtype != torch.uint8:
        raise ValueError("the plan reads a CPU uint8 copy of the mask")
    m = block_mask.contiguous()
    sb, sh = _mask_strides(m, B, H, N, device_ok=False)
    counts = torch.zeros(8, dtype=torch.int32)
    L = lib()
    st = L.fa_sparse_plan(_ptr(m), sb, sh, B, H, N, int(bool(causal)), None, 0, _ptr(counts))
    if st != FA_OK:
        raise FaError(st, "fa_sparse_plan")
    c = [int(x) for x in counts]
    n = 4 * (c[0] + c[1] + c[3] + c[4])
    plan = torch.zeros(max(n, 4), dtype=torch.int32)
    st = L.fa_sparse_plan(_ptr(m), sb, sh, B, H, N, int(bool(causal)), _ptr(plan), plan.numel(),
                          _ptr(counts))
    if st != FA_OK:
        raise FaError(st, "fa_sparse_plan")
    out = {"plan": plan, "counts": counts}
    o = 0
    for name, k in (("col_items", c[0]), ("cols", c[1]), ("row_items", c[3]), ("rows", c[4])):
        out[name] = plan[o:o + 4 * k].view(k, 4)
        o += 4 * k
    return out


def fa_fwd_sparse_planned_workspace_bytes(B: int, H: int, N: int, d: int, counts) -> int:
    c = torch.as_tensor(counts, dtype=torch.int32).contiguous()
    return int(lib().fa_fwd_sparse_planned_workspace_bytes(B, H, N, d, _ptr(c)))


def fa_bwd_sparse_planned_workspace_bytes(B: int, H: int, N: int, d: int, counts) -> int:
    c = torch.as_tensor(counts, dtype=torch.int32).contiguous()
    return int(lib().fa_bwd_sparse_planned_workspace_bytes(B, H, N, d, _ptr(c)))


def _plan_args(plan: dict, device, stream=None):
    """(device plan, CPU counts) of a plan from fa_sparse_plan. A plan whose
    "plan" tensor is already on the device is used in place; a host one is
    copied on every call (a copy that graph capture cannot record), on the
    stream the kernels run on, into memory allocated there (see _temp)."""
    counts = torch.as_tensor(plan["counts"], dtype=torch.int32).contiguous()
    if counts.is_cuda or counts.numel() != 8:
        raise ValueError("plan['counts'] must be the 8 host counts of fa_sparse_plan")
    with torch.cuda.stream(_torch_stream(stream, device)):
        return plan["plan"].to(device=device, dtype=torch.int32).contiguous(), counts


def fa_fwd_sparse_planned(q, k, v, o, lse, block_mask, plan: dict, scale: float, causal: bool = False,
                          kv_len=None, workspace=None, stream=None) -> None:
    """fa_fwd_sparse with the plan of fa_sparse_plan (long mask rows cut into
    pieces whose partial O and LSE are merged)."""
    B, H, N, d = q.shape
    for name, t in (("k", k), ("v", v)):
        _check_tensor(name, t, q.shape, q.dtype)
    _check_tensor("q", q, q.shape)
    _check_tensor("o", o, q.shape)
    _check_tensor("lse", lse, (B, H, N), torch.float32)
    sb, sh = _mask_strides(block_mask, B, H, N)
    dplan, counts = _plan_args(plan, q.device, stream)
    need = fa_fwd_sparse_planned_workspace_bytes(B, H, N, d, counts)
    if workspace is None:
        workspace = _temp(need, q.device, stream)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib().fa_fwd_sparse_planned(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d,
                                     float(scale), int(bool(causal)), _kv(kv_len, B), _ptr(block_mask),
                                     sb, sh, _ptr(dplan), _ptr(counts), _ptr(workspace), ws_bytes,
                                     _stream(stream, q.device), _DTYPE.get(q.dtype, -99),
                                     _DTYPE.get(o.dtype, -99))
    if st != FA_OK:
        raise FaError(st, "fa_fwd_sparse_planned")


def fa_bwd_sparse_planned(q, k, v, o, dout, lse, dq, dk, dv, block_mask, plan: dict, scale: float,
                          causal: bool = False, kv_len=None, workspace=None, stream=None) -> None:
    """fa_bwd_sparse with the plan of fa_sparse_plan (long mask columns and
    rows cut into pieces whose fp32 partials are added in order)."""
    B, H, N, d = q.shape
    for name, t in (("k", k), ("v", v), ("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv)):
        _check_tensor(name, t, q.shape, q.dtype)
    _check_tensor("q", q, q.shape)
    o_dt = _check_o(o, q)
    _check_tensor("lse", lse, (B, H, N), torch.float32)
    sb, sh = _mask_strides(block_mask, B, H, N)
    dplan, counts = _plan_args(plan, q.device, stream)
    need = fa_bwd_sparse_planned_workspace_bytes(B, H, N, d, counts)
    if workspace is None:
        workspace = _temp(need, q.device, stream)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib().fa_bwd_sparse_planned(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                                     _ptr(dq), _ptr(dk), _ptr(dv), B, H, N, d, float(scale),
                                     int(bool(causal)), _kv(kv_len, B), _ptr(block_mask), sb, sh,
                                     _ptr(dplan), _ptr(counts), _ptr(workspace), ws_bytes,
                                     _stream(stream, q.device), _DTYPE.get(q.dtype, -99), o_dt)
    if st != FA_OK:
        raise FaError(st, "fa_bwd_sparse_planned")


def fp8_buffers(B: int, H: int, N: int, d: int, device="cuda") -> dict:
    """Device buffers for fa_fp8_quantize / fa_fwd_fp8 (allocated with torch)."""
    np_ = (N + 63) // 64 * 64
    u8, f32 = torch.uint8, torch.float32
    return {"q8": torch.empty((B, H, N, d), dtype=u8, device=device),
            "k8": torch.empty((B, H, N, d), dtype=u8, device=device),
            "vt8": torch.empty((B, H, d, np_), dtype=u8, device=device),
            "q_scale": torch.empty((B, H, (N + 127) // 128), dtype=f32, device=device),
            "k_scale": torch.empty((B, H, (N + 63) // 64), dtype=f32, device=device),
            "v_scale": torch.empty((B, H), dtype=f32, device=device),
            "v_amax": torch.empty((B, H, (N + 63) // 64), dtype=f32, device=device)}


def _signs(signs, d):
    if signs is None:
        return None
    _check_tensor("signs", signs, (d,), torch.int8)
    return signs.data_ptr()


def fa_fp8_quantize(q, k, v, signs, bufs: dict, stream=None) -> None:
    """Enqueue the rotation (signs: int8 [d] of +-1, or None) and e4m3
    quantisation of q, k, v [B, H, N, d] into ``bufs`` (see fp8_buffers)."""
    B, H, N, d = q.shape
    for name, t in (("k", k), ("v", v)):
        _check_tensor(name, t, q.shape, q.dtype)
    _check_tensor("q", q, q.shape)
    ref = fp8_buffers(B, H, N, d, device="meta")
    for name, t in bufs.items():
        _check_tensor(name, t, ref[name].shape, ref[name].dtype)
    st = lib().fa_fp8_quantize(_ptr(q), _ptr(k), _ptr(v), _signs(signs, d), _ptr(bufs["q8"]),
                               _ptr(bufs["k8"]), _ptr(bufs["vt8"]), _ptr(bufs["q_scale"]),
                               _ptr(bufs["k_scale"]), _ptr(bufs["v_scale"]), _ptr(bufs["v_amax"]),
                               B, H, N, d, _stream(stream, q.device), _DTYPE.get(q.dtype, -99))
    if st != FA_OK:
        raise FaError(st, "fa_fp8_quantize")


def fa_fwd_fp8(bufs: dict, rotated: bool, o, lse, scale: float, causal: bool = False,
               kv_len=None, stream=None) -> None:
    """Enqueue attention on the codes in ``bufs``: o [B, H, N, d] (fp32, fp16
    or bf16), lse fp32 [B, H, N]."""
    B, H, N, d = bufs["q8"].shape
    _check_tensor("o", o, (B, H, N, d))
    _check_tensor("lse", lse, (B, H, N), torch.float32)
    st = lib().fa_fwd_fp8(_ptr(bufs["q8"]), _ptr(bufs["k8"]), _ptr(bufs["vt8"]),
                          _ptr(bufs["q_scale"]), _ptr(bufs["k_scale"]), _ptr(bufs["v_scale"]),
                          int(bool(rotated)), _ptr(o), _ptr(lse), B, H, N, d, float(scale),
                          int(bool(causal)), _kv(kv_len, B), _stream(stream, o.device),
                          _DTYPE.get(o.dtype, -99))
    if st != FA_OK:
        raise FaError(st, "fa_fwd_fp8")


def fa_fwd_fp8_workspace_bytes(B: int, H: int, N: int, d: int) -> int:
    return int(lib().fa_fwd_fp8_workspace_bytes(B, H, N, d))


def fa_fwd_fp8_incoherent(q, k, v, signs, o, lse, scale: float, causal: bool = False,
                          kv_len=None, workspace=None, stream=None) -> None:
    """Enqueue both FP8 steps (workspace allocated here when None)."""
    B, H, N, d = q.shape
    for name, t in (("k", k), ("v", v)):
        _check_tensor(name, t, q.shape, q.dtype)
    _check_tensor("q", q, q.shape)
    _check_tensor("o", o, q.shape)
    _check_tensor("lse", lse, (B, H, N), torch.float32)
    need = fa_fwd_fp8_workspace_bytes(B, H, N, d)
    if workspace is None:
        workspace = _temp(need, q.device, stream)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib().fa_fwd_fp8_incoherent(_ptr(q), _ptr(k), _ptr(v), _signs(signs, d), _ptr(o),
                                     _ptr(lse), B, H, N, d, float(scale), int(bool(causal)),
                                     _kv(kv_len, B), _ptr(workspace), ws_bytes,
                                     _stream(stream, q.device), _DTYPE.get(q.dtype, -99),
                                     _DTYPE.get(o.dtype, -99))
    if st != FA_OK:
        raise FaError(st, "fa_fwd_fp8_incoherent")


# Convenience wrappers that allocate the outputs with torch (plumbing only).

# K and V with fewer heads than Q go to the grouped-query entry points.

def attention_forward(q, k, v, causal: bool = False, kv_len=None, scale: Optional[float] = None,
                      out_dtype: Optional[torch.dtype] = None, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    B, H, N, d = q.shape
    scale = d ** -0.5 if scale is None else scale
    if not q.is_cuda:
        raise ValueError("q must be a device tensor")
    # outputs are allocated on the stream that writes them (see _temp)
    with torch.cuda.stream(_torch_stream(stream, q.device)):
        o = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if k.dim() == 4 and k.shape[1] != H:
        fa_fwd_gqa(q, k, v, o, lse, scale, causal, kv_len, stream)
    else:
        fa_fwd(q, k, v, o, lse, scale, causal, kv_len, stream)
    return o, lse


def attention_backward(q, k, v, o, dout, lse, causal: bool = False, kv_len=None,
                       scale: Optional[float] = None, stream=None):
    d = q.shape[-1]
    scale = d ** -0.5 if scale is None else scale
    if not q.is_cuda:
        raise ValueError("q must be a device tensor")
    with torch.cuda.stream(_torch_stream(stream, q.device)):
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    if k.dim() == 4 and k.shape[1] != q.shape[1]:
        fa_bwd_gqa(q, k, v, o, dout, lse, dq, dk, dv, scale, causal, kv_len, None, stream)
    else:
        fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, scale, causal, kv_len, None, stream)
    return dq, dk, dv


class _Attention(torch.autograd.Function):
    """Autograd glue: the forward keeps O and LSE, the backward recomputes
    from them through the library (no N x N tensor is ever formed)."""

    @staticmethod
    def forward(ctx, q, k, v, causal: bool, scale: float, kv_len):
        o, lse = attention_forward(q, k, v, causal=causal, kv_len=kv_len, scale=scale)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.kv_len, ctx.causal, ctx.scale = kv_len, causal, scale
        return o

    @staticmethod
    def backward(ctx, dout):
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv = attention_backward(q, k, v, o, dout.contiguous(), lse, causal=ctx.causal,
                                        kv_len=ctx.kv_len, scale=ctx.scale)
        return dq, dk, dv, None, None, None


def scaled_dot_product_attention(q, k, v, is_causal: bool = False, scale: Optional[float] = None,
                                 kv_len=None) -> torch.Tensor:
    """softmax(scale * Q K^T) V with autograd, in the shape convention of
    torch's scaled_dot_product_attention (q [B, H, N, d]; k, v [B, H or H_kv,
    N, d]; top-left causal mask; scale defaults to 1 / sqrt(d)), plus per-batch
    key lengths kv_len (int32 [B] on the device, or None). Inputs must be
    contiguous fp16 / bf16 / fp32 device tensors of head dim 64 or 128; no
    dropout and no arbitrary mask. Forward and backward run the library's
    kernels (fa_fwd / fa_bwd, or the grouped-query entry points)."""
    d = q.shape[-1]
    return _Attention.apply(q, k, v, bool(is_causal), d ** -0.5 if scale is None else float(scale),
                            kv_len)
