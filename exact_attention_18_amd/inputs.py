"""Seeded synthetic inputs and the workload registry.

This module is shared by the tests, the benchmark and the oracle's callers.  It
holds no attention arithmetic: it only draws random tensors and names shapes.

Recipe (the same for every workload): one ``torch.Generator`` per workload,
seeded with the workload's seed; Q, K, V are drawn in that order as float32
i.i.d. N(0, 1) in the layouts below, Q is multiplied by ``q_mult`` where the
workload asks for peaky softmax rows, and each tensor is rounded once to
bfloat16 (round-to-nearest-even).  The GPU and the oracle consume these very
bf16 tensors (the oracle upcasts them exactly to fp64).  Key-padding lengths
and packed sequence lengths are integers drawn uniformly from an inclusive
range with a second seed.

Layouts: q, o [B, Nq, Hq, d]; k, v [B, Nk, Hkv, d]; lse [B, Hq, Nq] (fp32).
Packed (varlen): q, o [Tq, Hq, d]; k, v [Tk, Hkv, d]; lse [Hq, Tq];
cu_seqlens int32 [num_seqs + 1] starting at 0.

Workload shapes follow the pages' workloads: the FlashAttention-1 kernel
analysis shape (sequence 1024, head dim 64, 16 heads, batch 64; "059 ·
FlashAttention" (wq-win), section 4 table) and the FlashAttention-4 sweep shape
(hidden 2048 = 16 x 128, sequence 1k-32k, head dim 128, causal;
FlashAttention-4 (papercache summary), experimental setup).  Dropout, which the
FlashAttention-1 kernel analysis included, is not part of any workload.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    N: int  # Nq == Nk in every workload
    d: int
    causal: bool
    seed: int
    q_mult: float = 1.0
    pad_seed: Optional[int] = None  # key padding: lengths ~ U{pad_lo..N}
    pad_lo: int = 0
    varlen_seed: Optional[int] = None  # packed: num_seqs lengths ~ U{lo..hi}
    varlen_seqs: int = 0
    varlen_lo: int = 0
    varlen_hi: int = 0
    dv: int = 0  # value / output head dimension when it differs from d
    sparse_window: int = -1  # block-sparse: key blocks within this distance of the query block ...
    sparse_global: int = 0   # ... plus the first sparse_global key blocks (128 x 128 blocks)

    @property
    def d_v(self) -> int:
        return self.dv or self.d

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def sparse(self) -> bool:
        return self.sparse_window >= 0

    @property
    def varlen(self) -> bool:
        return self.varlen_seed is not None


WORKLOADS = {
    # Single head, the small case the oracle finishes in well under a second.
    "single_head_n256_d64": Workload("single_head_n256_d64", 1, 1, 1, 256, 64, False, 1001),
    # FlashAttention-1 kernel-analysis shape, non-causal and with key padding.
    "batch64_h16_n1024_d64": Workload("batch64_h16_n1024_d64", 64, 16, 16, 1024, 64, False, 2001),
    "batch64_h16_n1024_d64_keypad": Workload("batch64_h16_n1024_d64_keypad", 64, 16, 16, 1024, 64,
                                             False, 2001, pad_seed=2002, pad_lo=512),
    # Causal training shape.
    "causal_b16_h16_n4096_d128": Workload("causal_b16_h16_n4096_d128", 16, 16, 16, 4096, 128, True,
                                          3001),
    # Grouped-query causal, Q x3 for peaky rows: the headline workload.
    "gqa_causal_b4_hq32_hkv8_n8192_d128": Workload("gqa_causal_b4_hq32_hkv8_n8192_d128", 4, 32, 8,
                                                   8192, 128, True, 4001, q_mult=3.0),
    # Long context, and its packed ragged variant.
    "long_causal_b1_h32_n32768_d128": Workload("long_causal_b1_h32_n32768_d128", 1, 32, 32, 32768,
                                               128, True, 5001),
    "varlen_causal_8seq_h32_d128": Workload("varlen_causal_8seq_h32_d128", 1, 32, 32, 16384, 128,
                                            True, 5001, varlen_seed=5002, varlen_seqs=8,
                                            varlen_lo=2048, varlen_hi=16384),
    # Asymmetric head dimensions: scores at d = 192, values at d = 128, 16 heads,
    # batch 4 x 8192 tokens (the (192, 128) shape of the FlashAttention-4 sweep).
    "asym_causal_b4_h16_n8192_dqk192_dv128": Workload("asym_causal_b4_h16_n8192_dqk192_dv128", 4,
                                                      16, 16, 8192, 192, True, 6001, dv=128),
    # Block-sparse: sliding window of +-8 blocks of 128 plus one global key block,
    # on the headline's grouped-query shape (non-causal).
    "blocksparse_window_b4_hq32_hkv8_n8192_d128": Workload(
        "blocksparse_window_b4_hq32_hkv8_n8192_d128", 4, 32, 8, 8192, 128, False, 7001,
        sparse_window=8, sparse_global=1),
}

SPARSE_BLOCK = 128


def window_block_mask(nbq, nbk, window, n_global):
    """uint8 [1, nbq, nbk]: block (i, j) set iff |i - j| <= window or j < n_global."""
    i = torch.arange(nbq)[:, None]
    j = torch.arange(nbk)[None, :]
    return (((i - j).abs() <= window) | (j < n_global)).to(torch.uint8)[None]

HEADLINE = "gqa_causal_b4_hq32_hkv8_n8192_d128"


def make_qkv(B, Nq, Nk, Hq, Hkv, d, seed, q_mult=1.0, d_v=None):
    """Q [B,Nq,Hq,d], K [B,Nk,Hkv,d], V [B,Nk,Hkv,d_v] (d_v defaults to d) as bf16 CPU tensors."""
    g = torch.Generator().manual_seed(int(seed))
    q = torch.randn((B, Nq, Hq, d), generator=g, dtype=torch.float32)
    k = torch.randn((B, Nk, Hkv, d), generator=g, dtype=torch.float32)
    v = torch.randn((B, Nk, Hkv, d if d_v is None else d_v), generator=g, dtype=torch.float32)
    if q_mult != 1.0:
        q.mul_(q_mult)
    return q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)


def make_qkv_on(device, B, Nq, Nk, Hq, Hkv, d, seed):
    """As make_qkv (Q, K, V i.i.d. N(0, 1), rounded once to bf16), drawn on `device`.

    For inputs of several GiB, which the host would take long to draw: a
    seeded generator of that device fills them there, and a checker reads the
    very tensors back.
    """
    g = torch.Generator(device=device).manual_seed(int(seed))
    out = []
    for shape in ((B, Nq, Hq, d), (B, Nk, Hkv, d), (B, Nk, Hkv, d)):
        out.append(torch.randn(shape, generator=g, device=device, dtype=torch.float32)
                   .to(torch.bfloat16))
    return tuple(out)


def make_trend_qkv(B, N, Hq, Hkv, d, seed, scale, step, jump_at=None, jump=0.0, d_v=None):
    """Q, K, V whose scores climb (or fall) along the keys, as bf16 CPU tensors.

    Drawn as make_qkv (Q, K, V i.i.d. N(0, 1)), then dimension 0 is replaced:
    every query row of an even query head holds +8 there and of an odd head
    -8, and key j holds j * step / (8 |scale|), plus jump / (8 |scale|) at key
    jump_at.  So scale * q_i . k_j is +-(j * step (+ jump)) up to the sign of
    scale, plus the N(0, 1)-scale contribution of the other d - 1 dimensions:
    rows of one parity find a larger maximum in every later key tile (and,
    past jump_at, one key far above all earlier ones), rows of the other
    parity keep their maximum in the first keys.  Shapes as make_qkv with
    Nq = Nk = N.
    """
    q, k, v = make_qkv(B, N, N, Hq, Hkv, d, seed, d_v=d_v)
    q, k = q.float(), k.float()
    sign = torch.tensor([1.0 if h % 2 == 0 else -1.0 for h in range(Hq)])
    q[..., 0] = 8.0 * sign
    t = torch.arange(N, dtype=torch.float32) * float(step)
    if jump_at is not None:
        t[jump_at] += float(jump)
    k[..., 0] = (t / (8.0 * abs(scale)))[None, :, None]
    return q.to(torch.bfloat16), k.to(torch.bfloat16), v


def make_dout(shape, seed):
    """Upstream gradient dO of the given shape: i.i.d. N(0,1) rounded once to bf16."""
    g = torch.Generator().manual_seed(int(seed))
    return torch.randn(tuple(shape), generator=g, dtype=torch.float32).to(torch.bfloat16)


def make_packed_qkv(total_q, total_k, Hq, Hkv, d, seed, q_mult=1.0):
    """Packed Q [Tq,Hq,d], K [Tk,Hkv,d], V [Tk,Hkv,d] as bf16 CPU tensors."""
    g = torch.Generator().manual_seed(int(seed))
    q = torch.randn((total_q, Hq, d), generator=g, dtype=torch.float32)
    k = torch.randn((total_k, Hkv, d), generator=g, dtype=torch.float32)
    v = torch.randn((total_k, Hkv, d), generator=g, dtype=torch.float32)
    if q_mult != 1.0:
        q.mul_(q_mult)
    return q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)


def make_seqlens(n, lo, hi, seed):
    """n int32 lengths drawn uniformly from {lo, ..., hi}."""
    g = torch.Generator().manual_seed(int(seed))
    return torch.randint(int(lo), int(hi) + 1, (n,), generator=g, dtype=torch.int64).to(torch.int32)


def cu_from_lengths(lengths):
    """int32 offsets [0, l0, l0+l1, ...] of a packed batch."""
    lengths = torch.as_tensor(lengths, dtype=torch.int64)
    cu = torch.zeros(lengths.numel() + 1, dtype=torch.int64)
    cu[1:] = torch.cumsum(lengths, 0)
    return cu.to(torch.int32)


def workload_inputs(w: Workload):
    """All inputs of a workload as CPU tensors, in a dict.

    Padded workloads: q, k, v, seqlens_k (or None), and block_mask for the
    block-sparse ones.  Packed workloads: q, k, v, cu_seqlens_q, cu_seqlens_k,
    lengths, max_seqlen.
    """
    if w.varlen:
        lengths = make_seqlens(w.varlen_seqs, w.varlen_lo, w.varlen_hi, w.varlen_seed)
        cu = cu_from_lengths(lengths)
        total = int(cu[-1])
        q, k, v = make_packed_qkv(total, total, w.Hq, w.Hkv, w.d, w.seed, w.q_mult)
        return dict(q=q, k=k, v=v, cu_seqlens_q=cu, cu_seqlens_k=cu.clone(), lengths=lengths,
                    max_seqlen=int(lengths.max()))
    q, k, v = make_qkv(w.B, w.N, w.N, w.Hq, w.Hkv, w.d, w.seed, w.q_mult, d_v=w.d_v)
    seqlens = None
    if w.pad_seed is not None:
        seqlens = make_seqlens(w.B, w.pad_lo, w.N, w.pad_seed)
    out = dict(q=q, k=k, v=v, seqlens_k=seqlens)
    if w.sparse:
        nb = -(-w.N // SPARSE_BLOCK)
        out["block_mask"] = window_block_mask(nb, nb, w.sparse_window, w.sparse_global)
    return out

