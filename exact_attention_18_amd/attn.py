"""Thin ctypes binding over libattn.so (argument marshalling only).

Every step of the forward runs in the HIP kernels of libattn.so; this module
checks tensor dtypes, devices, shapes and contiguity, allocates the outputs
with PyTorch when the caller does not pass them, and forwards raw device
pointers and torch's current HIP stream to the C ABI declared in
``include/attn.h``.  There is no fallback: if the library is missing or a call
returns an error, a ``RuntimeError`` is raised.
"""

from __future__ import annotations

import contextlib
import ctypes
import math
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libattn.so")
# The race-check build: the same kernels with conservative synchronisation
# (compiled with ATTN_FORCE_SAFE=1); used only to check that the tuned build
# has no missing wait or barrier.
SAFE_LIB_PATH = os.path.join(_PKG, "libattn_safe.so")
# The software-exp2 build: 8 of every 32 exponentials of the d = 128 softmax
# as a polynomial on the FMA pipe (compiled with ATTN_EXP2_POLY=8).
EXP2POLY_LIB_PATH = os.path.join(_PKG, "libattn_exp2poly.so")

# attn_status codes (include/attn.h)
ATTN_OK = 0
ATTN_ERR_NULL = -1
ATTN_ERR_HEAD_DIM = -2
ATTN_ERR_HEADS = -3
ATTN_ERR_SIZE = -4
ATTN_ERR_LAUNCH = -5
ATTN_ERR_ALIGN = -6
ATTN_ERR_TOO_LARGE = -7
ATTN_ERR_SCRATCH = -8

EXPORTS = ("attn_fwd", "attn_fwd_dims", "attn_fwd_blocksparse", "attn_fwd_varlen",
           "attn_fwd_varlen_ordered", "attn_varlen_plan", "attn_bwd", "attn_bwd_noalloc",
           "attn_bwd_varlen",
           "attn_bwd_varlen_ordered", "attn_bwd_workspace_size",
           "attn_probe_mfma", "attn_probe_softmax_issue", "attn_probe_xcd", "attn_strerror",
           "attn_last_hip_error",
           "attn_version")

_lib = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Open libattn.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(p)
    vp, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, i32, vp, vp]
    lib.attn_fwd.restype = i32
    lib.attn_fwd_dims.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, i32, vp,
                                  vp]
    lib.attn_fwd_dims.restype = i32
    lib.attn_fwd_blocksparse.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, i32,
                                         vp, vp, i32, vp]
    lib.attn_fwd_blocksparse.restype = i32
    lib.attn_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32,
                                    i32, vp]
    lib.attn_fwd_varlen.restype = i32
    lib.attn_fwd_varlen_ordered.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                            f32, i32, vp, vp]
    lib.attn_fwd_varlen_ordered.restype = i32
    lib.attn_varlen_plan.argtypes = [vp, vp, i32, i32, i32, i32, vp, vp]
    lib.attn_varlen_plan.restype = i32
    lib.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                             f32, i32, vp, vp]
    lib.attn_bwd.restype = i32
    lib.attn_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                     i32, f32, i32, vp, vp]
    lib.attn_bwd_noalloc.restype = i32
    lib.attn_bwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32,
                                    i32, i32, i32, i32, f32, i32, vp]
    lib.attn_bwd_varlen.restype = i32
    lib.attn_bwd_varlen_ordered.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32,
                                            i32, i32, i32, i32, i32, f32, i32, vp, vp]
    lib.attn_bwd_varlen_ordered.restype = i32
    lib.attn_bwd_workspace_size.argtypes = [i32, i32, i32]
    lib.attn_bwd_workspace_size.restype = ctypes.c_size_t
    lib.attn_probe_mfma.argtypes = [vp, i32, i32, i32, vp, vp, vp]
    lib.attn_probe_mfma.restype = i32
    lib.attn_probe_softmax_issue.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp]
    lib.attn_probe_softmax_issue.restype = i32
    lib.attn_probe_xcd.argtypes = [i32, vp, vp]
    lib.attn_probe_xcd.restype = i32
    lib.attn_strerror.argtypes = [i32]
    lib.attn_strerror.restype = ctypes.c_char_p
    lib.attn_last_hip_error.argtypes = []
    lib.attn_last_hip_error.restype = i32
    lib.attn_version.argtypes = []
    lib.attn_version.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


@contextlib.contextmanager
def using_library(path: str):
    """Route the calls of this module through another build of the library (e.g. SAFE_LIB_PATH)."""
    global _lib
    saved = load_library()
    _lib = load_library(path)
    try:
        yield _lib
    finally:
        _lib = saved


def strerror(code: int) -> str:
    return load_library().attn_strerror(int(code)).decode()


def _check(rc: int, what: str):
    if rc != ATTN_OK:
        lib = load_library()
        msg = f"{what}: {strerror(rc)} (status {rc})"
        if rc == ATTN_ERR_LAUNCH:
            msg += f", hipError {lib.attn_last_hip_error()}"
        raise RuntimeError(msg)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_handle(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: Optional[float] = None,
             causal: bool = False, seqlens_k: Optional[torch.Tensor] = None,
             out: Optional[torch.Tensor] = None,
             lse: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """O, LSE = attention forward of bf16 q [B,Nq,Hq,d], k [B,Nk,Hkv,d], v [B,Nk,Hkv,dv].

    Returns O bf16 [B,Nq,Hq,dv] and LSE fp32 [B,Hq,Nq] (natural log).  dv == d,
    or (d, dv) = (192, 128).  Launches on torch's current stream of q's device
    and does not synchronise.
    """
    lib = load_library()
    _need(q, "q", torch.bfloat16)
    dev = q.device
    _need(k, "k", torch.bfloat16, dev)
    _need(v, "v", torch.bfloat16, dev)
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4 or v.shape[:3] != k.shape[:3]:
        raise ValueError("expected q [B,Nq,Hq,d], k [B,Nk,Hkv,d] and v [B,Nk,Hkv,dv]")
    B, Nq, Hq, d = q.shape
    Bk, Nk, Hkv, dk = k.shape
    dv = v.shape[3]
    if Bk != B or dk != d:
        raise ValueError("q and k disagree on batch or head dim")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if seqlens_k is not None:
        _need(seqlens_k, "seqlens_k", torch.int32, dev)
        if seqlens_k.shape != (B,):
            raise ValueError("seqlens_k must have shape [B]")
    if out is None:
        out = torch.empty((B, Nq, Hq, dv), dtype=torch.bfloat16, device=dev)
    else:
        _need(out, "out", torch.bfloat16, dev)
        if out.shape != (B, Nq, Hq, dv):
            raise ValueError("out must have shape [B,Nq,Hq,dv]")
    if lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=dev)
    else:
        _need(lse, "lse", torch.float32, dev)
        if lse.shape != (B, Hq, Nq):
            raise ValueError("lse must have shape [B,Hq,Nq]")
    if dv == d:
        rc = lib.attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, Nq, Nk, d,
                          float(scale), int(bool(causal)), _ptr(seqlens_k), _stream_handle(dev))
    else:
        rc = lib.attn_fwd_dims(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, Nq, Nk,
                               d, dv, float(scale), int(bool(causal)), _ptr(seqlens_k),
                               _stream_handle(dev))
    _check(rc, "attn_fwd")
    return out, lse


def attn_fwd_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens_q: torch.Tensor,
                    cu_seqlens_k: torch.Tensor, max_seqlen_q: int, max_seqlen_k: int,
                    scale: Optional[float] = None, causal: bool = False,
                    out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                    seq_order: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Packed forward: q [Tq,Hq,d], k/v [Tk,Hkv,d], cu_seqlens int32 [S+1] on the GPU.

    Returns O bf16 [Tq,Hq,d] and LSE fp32 [Hq,Tq].  Rows of a freshly allocated
    O / LSE that belong to no sequence are left as zero.  seq_order (int32 [S],
    from attn_varlen_plan) sets the order in which sequences are scheduled
    (attn_fwd_varlen_ordered); without it the sequences run in index order
    (attn_fwd_varlen).
    """
    lib = load_library()
    _need(q, "q", torch.bfloat16)
    dev = q.device
    _need(k, "k", torch.bfloat16, dev)
    _need(v, "v", torch.bfloat16, dev)
    _need(cu_seqlens_q, "cu_seqlens_q", torch.int32, dev)
    _need(cu_seqlens_k, "cu_seqlens_k", torch.int32, dev)
    if q.dim() != 3 or k.dim() != 3 or v.shape != k.shape:
        raise ValueError("expected q [Tq,Hq,d] and k, v [Tk,Hkv,d] of equal shape")
    Tq, Hq, d = q.shape
    _, Hkv, dk = k.shape
    if dk != d:
        raise ValueError("q and k disagree on head dim")
    if cu_seqlens_q.dim() != 1 or cu_seqlens_k.shape != cu_seqlens_q.shape:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must be 1-D of equal length")
    num_seqs = cu_seqlens_q.numel() - 1
    if seq_order is not None:
        _need(seq_order, "seq_order", torch.int32, dev)
        if seq_order.shape != (num_seqs,):
            raise ValueError("seq_order must have shape [num_seqs]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.zeros_like(q)
    else:
        _need(out, "out", torch.bfloat16, dev)
        if out.shape != q.shape:
            raise ValueError("out must have q's shape")
    if lse is None:
        lse = torch.zeros((Hq, Tq), dtype=torch.float32, device=dev)
    else:
        _need(lse, "lse", torch.float32, dev)
        if lse.shape != (Hq, Tq):
            raise ValueError("lse must have shape [Hq,Tq]")
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
            num_seqs, Hq, Hkv, int(max_seqlen_q), int(max_seqlen_k), d, float(scale),
            int(bool(causal)))
    if seq_order is None:
        rc = lib.attn_fwd_varlen(*args, _stream_handle(dev))
        _check(rc, "attn_fwd_varlen")
    else:
        rc = lib.attn_fwd_varlen_ordered(*args, _ptr(seq_order), _stream_handle(dev))
        _check(rc, "attn_fwd_varlen_ordered")
    return out, lse


def attn_varlen_plan(cu_seqlens_q: torch.Tensor, cu_seqlens_k: torch.Tensor, max_seqlen_q: int,
                     max_seqlen_k: int, causal: bool = False,
                     out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Longest-first sequence order (int32 [S]) for attn_fwd_varlen's seq_order."""
    lib = load_library()
    _need(cu_seqlens_q, "cu_seqlens_q", torch.int32)
    dev = cu_seqlens_q.device
    _need(cu_seqlens_k, "cu_seqlens_k", torch.int32, dev)
    if cu_seqlens_q.dim() != 1 or cu_seqlens_k.shape != cu_seqlens_q.shape:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must be 1-D of equal length")
    num_seqs = cu_seqlens_q.numel() - 1
    if out is None:
        out = torch.empty((num_seqs,), dtype=torch.int32, device=dev)
    else:
        _need(out, "out", torch.int32, dev)
        if out.shape != (num_seqs,):
            raise ValueError("out must have shape [num_seqs]")
    rc = lib.attn_varlen_plan(_ptr(cu_seqlens_q), _ptr(cu_seqlens_k), num_seqs, int(max_seqlen_q),
                              int(max_seqlen_k), int(bool(causal)), _ptr(out), _stream_handle(dev))
    _check(rc, "attn_varlen_plan")
    return out


def attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
             dout: torch.Tensor, scale: Optional[float] = None, causal: bool = False,
             seqlens_k: Optional[torch.Tensor] = None,
             workspace: Optional[torch.Tensor] = None,
             out: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None
             ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """dQ, dK, dV (bf16) of the batched forward from its O and LSE and the upstream dO.

    Layouts as in attn_fwd; d is 64 or 128.  The workspace (uint8, at least
    attn_bwd_workspace_size bytes) is allocated here when not given.
    """
    lib = load_library()
    _need(q, "q", torch.bfloat16)
    dev = q.device
    for t, n in ((k, "k"), (v, "v"), (o, "o"), (dout, "dout")):
        _need(t, n, torch.bfloat16, dev)
    _need(lse, "lse", torch.float32, dev)
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape or o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("expected q, o, dout [B,Nq,Hq,d] and k, v [B,Nk,Hkv,d]")
    B, Nq, Hq, d = q.shape
    Bk, Nk, Hkv, dk_ = k.shape
    if Bk != B or dk_ != d:
        raise ValueError("q and k disagree on batch or head dim")
    if lse.shape != (B, Hq, Nq):
        raise ValueError("lse must have shape [B,Hq,Nq]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if seqlens_k is not None:
        _need(seqlens_k, "seqlens_k", torch.int32, dev)
        if seqlens_k.shape != (B,):
            raise ValueError("seqlens_k must have shape [B]")
    need = int(lib.attn_bwd_workspace_size(B, Hq, Nq))
    if workspace is None:
        workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=dev)
    else:
        _need(workspace, "workspace", torch.uint8, dev)
        if workspace.numel() < need:
            raise ValueError(f"workspace needs {need} bytes")
    if out is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    else:
        dq, dk, dv = out
        _need(dq, "dq", torch.bfloat16, dev)
        _need(dk, "dk", torch.bfloat16, dev)
        _need(dv, "dv", torch.bfloat16, dev)
        if dq.shape != q.shape or dk.shape != k.shape or dv.shape != k.shape:
            raise ValueError("dq, dk, dv must have the shapes of q, k, v")
    rc = lib.attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
                      _ptr(dv), _ptr(workspace), B, Hq, Hkv, Nq, Nk, d, float(scale),
                      int(bool(causal)), _ptr(seqlens_k), _stream_handle(dev))
    _check(rc, "attn_bwd")
    return dq, dk, dv


def attn_bwd_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                    lse: torch.Tensor, dout: torch.Tensor, cu_seqlens_q: torch.Tensor,
                    cu_seqlens_k: torch.Tensor, max_seqlen_q: int, max_seqlen_k: int,
                    scale: Optional[float] = None, causal: bool = False,
                    seq_order: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None,
                    out: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None
                    ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """dQ, dK, dV (bf16) of the packed forward (attn_fwd_varlen) from its O and LSE.

    q, o, dout [Tq,Hq,d]; k, v [Tk,Hkv,d]; lse [Hq,Tq] as attn_fwd_varlen
    returns it; d is 64 or 128.  Rows and keys that belong to no sequence are
    not written (zero when dq, dk, dv are allocated here).
    """
    lib = load_library()
    _need(q, "q", torch.bfloat16)
    dev = q.device
    for t, n in ((k, "k"), (v, "v"), (o, "o"), (dout, "dout")):
        _need(t, n, torch.bfloat16, dev)
    _need(lse, "lse", torch.float32, dev)
    _need(cu_seqlens_q, "cu_seqlens_q", torch.int32, dev)
    _need(cu_seqlens_k, "cu_seqlens_k", torch.int32, dev)
    if q.dim() != 3 or k.dim() != 3 or v.shape != k.shape or o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("expected q, o, dout [Tq,Hq,d] and k, v [Tk,Hkv,d]")
    Tq, Hq, d = q.shape
    _, Hkv, dk_ = k.shape
    if dk_ != d:
        raise ValueError("q and k disagree on head dim")
    if lse.shape != (Hq, Tq):
        raise ValueError("lse must have shape [Hq,Tq]")
    if cu_seqlens_q.dim() != 1 or cu_seqlens_k.shape != cu_seqlens_q.shape:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must be 1-D of equal length")
    num_seqs = cu_seqlens_q.numel() - 1
    if seq_order is not None:
        _need(seq_order, "seq_order", torch.int32, dev)
        if seq_order.shape != (num_seqs,):
            raise ValueError("seq_order must have shape [num_seqs]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = int(lib.attn_bwd_workspace_size(1, Hq, Tq))
    if workspace is None:
        workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=dev)
    else:
        _need(workspace, "workspace", torch.uint8, dev)
        if workspace.numel() < need:
            raise ValueError(f"workspace needs {need} bytes")
    if out is None:
        dq, dk, dv = torch.zeros_like(q), torch.zeros_like(k), torch.zeros_like(v)
    else:
        dq, dk, dv = out
        _need(dq, "dq", torch.bfloat16, dev)
        _need(dk, "dk", torch.bfloat16, dev)
        _need(dv, "dv", torch.bfloat16, dev)
        if dq.shape != q.shape or dk.shape != k.shape or dv.shape != k.shape:
            raise ValueError("dq, dk, dv must have the shapes of q, k, v")
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
            _ptr(dv), _ptr(workspace), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), num_seqs, Tq, Hq,
            Hkv, int(max_seqlen_q), int(max_seqlen_k), d, float(scale), int(bool(causal)))
    if seq_order is None:
        rc = lib.attn_bwd_varlen(*args, _stream_handle(dev))
        _check(rc, "attn_bwd_varlen")
    else:
        rc = lib.attn_bwd_varlen_ordered(*args, _ptr(seq_order), _stream_handle(dev))
        _check(rc, "attn_bwd_varlen_ordered")
    return dq, dk, dv


SPARSE_BLOCK = 128  # block-sparse mask granularity (query rows and keys)


def attn_fwd_blocksparse(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, block_mask: torch.Tensor,
                         scale: Optional[float] = None, causal: bool = False,
                         seqlens_k: Optional[torch.Tensor] = None,
                         out: Optional[torch.Tensor] = None,
                         lse: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Block-sparse forward; block_mask uint8 [1 or Hq, ceil(Nq/128), ceil(Nk/128)] on the GPU."""
    lib = load_library()
    _need(q, "q", torch.bfloat16)
    dev = q.device
    _need(k, "k", torch.bfloat16, dev)
    _need(v, "v", torch.bfloat16, dev)
    _need(block_mask, "block_mask", torch.uint8, dev)
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("expected q [B,Nq,Hq,d] and k, v [B,Nk,Hkv,d] of equal shape")
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    nbq, nbk = -(-Nq // SPARSE_BLOCK), -(-Nk // SPARSE_BLOCK)
    if block_mask.dim() != 3 or block_mask.shape[1:] != (nbq, nbk):
        raise ValueError(f"block_mask must have shape [1 or Hq, {nbq}, {nbk}]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if seqlens_k is not None:
        _need(seqlens_k, "seqlens_k", torch.int32, dev)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=dev)
    rc = lib.attn_fwd_blocksparse(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, Nq,
                                  Nk, d, float(scale), int(bool(causal)), _ptr(seqlens_k),
                                  _ptr(block_mask), int(block_mask.shape[0]), _stream_handle(dev))
    _check(rc, "attn_fwd_blocksparse")
    return out, lse


PROBE_WAVES = 8  # waves per probe workgroup (include/attn.h, attn_probe_mfma)
PROBE_FLOP_PER_ITER = 16 * 2 * 32 * 32 * 16  # per wave, either shape


def attn_probe_mfma(operands: torch.Tensor, iters: int, workgroups: int,
                    sink: Optional[torch.Tensor] = None,
                    clocks: Optional[torch.Tensor] = None,
                    shape: int = 32) -> Tuple[torch.Tensor, torch.Tensor]:
    """Launch the matrix-core rate probe; returns (sink, clocks) on the device.

    operands: bf16 [8, 64, 8] (4 A then 4 B operands, per lane).  shape: 32
    (32x32x16 MFMA: the d = 64 and (192, 128) kernels) or 16 (16x16x32: the
    d = 128 kernel).  FLOP per launch is
    workgroups * 8 * iters * 16 * 32768 for either shape (probe_flop()).
    clocks[w] = (shader-clock ticks, 100 MHz real-time ticks) of wave w's loop.
    """
    _need(operands, "operands", torch.bfloat16)
    if tuple(operands.shape) != (8, 64, 8):
        raise ValueError(f"operands must be [8, 64, 8], got {tuple(operands.shape)}")
    dev = operands.device
    n = workgroups * 64 * PROBE_WAVES
    if sink is None:
        sink = torch.empty(n, dtype=torch.float32, device=dev)
    if clocks is None:
        clocks = torch.empty((workgroups * PROBE_WAVES, 2), dtype=torch.int64, device=dev)
    _need(sink, "sink", torch.float32, dev)
    _need(clocks, "clocks", torch.int64, dev)
    if sink.numel() < n or clocks.numel() < 2 * workgroups * PROBE_WAVES:
        raise ValueError("sink or clocks too small for the grid")
    rc = load_library().attn_probe_mfma(_ptr(operands), int(shape), int(iters), int(workgroups),
                                        _ptr(sink), _ptr(clocks), _stream_handle(dev))
    _check(rc, "attn_probe_mfma")
    return sink, clocks


def probe_flop(iters: int, workgroups: int) -> float:
    return float(workgroups) * PROBE_WAVES * iters * PROBE_FLOP_PER_ITER


def attn_probe_xcd(workgroups: int, device=None) -> torch.Tensor:
    """Placement of a grid of 512-thread workgroups: int32 [workgroups, 2] on the device.

    Row w holds the XCD workgroup w ran on and the raw HW_ID register of its
    first wave (attn_probe_xcd in include/attn.h).
    """
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else device
    ids = torch.empty((workgroups, 2), dtype=torch.int32, device=dev)
    rc = load_library().attn_probe_xcd(int(workgroups), _ptr(ids), _stream_handle(dev))
    _check(rc, "attn_probe_xcd")
    return ids


def attn_probe_softmax_issue(operands: torch.Tensor, mfma_on: bool, exp_kind: int, budget_us: int,
                             workgroups: int) -> Tuple[torch.Tensor, torch.Tensor]:
    """Launch the softmax issue probe; returns (values fp32 [64, 32], stats int64 [wg * 8, 4]).

    exp_kind: 0 none, 1 v_exp_f32, 2 polynomial exp2, 3 polynomial on 8 of 32
    elements.  stats[w] = (iterations, shader ticks, 100 MHz ticks, checksum
    bits) of wave w (attn_probe_softmax_issue in include/attn.h).
    """
    _need(operands, "operands", torch.bfloat16)
    if tuple(operands.shape) != (8, 64, 8):
        raise ValueError(f"operands must be [8, 64, 8], got {tuple(operands.shape)}")
    dev = operands.device
    values = torch.zeros((64, 32), dtype=torch.float32, device=dev)
    stats = torch.empty((workgroups * PROBE_WAVES, 4), dtype=torch.int64, device=dev)
    rc = load_library().attn_probe_softmax_issue(_ptr(operands), int(bool(mfma_on)), int(exp_kind),
                                                 int(budget_us), int(workgroups), _ptr(values),
                                                 _ptr(stats), _stream_handle(dev))
    _check(rc, "attn_probe_softmax_issue")
    return values, stats
