"""Plain fp64 CPU definition of the exact-attention backward pass.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module, and this module imports nothing from the product path.

What is computed, with the passages it follows
----------------------------------------------
For one head, with S = scale * Q K^T (masked entries -inf), P = softmax(S)
row-wise and O = P V, and an upstream gradient dO of O
(FlashAttention-4 (papercache summary), section 2.1, the displayed backward
equations):

    dV = P^T dO,        dP = dO V^T,
    dS = dsoftmax(dP),  row-wise ds = (diag(p) - p p^T) dp,
    dQ = scale * dS K,  dK = scale * dS^T Q.

Row-wise, (diag(p) - p p^T) dp = p * (dp - <p, dp>), so
dS_ij = P_ij (dP_ij - D_i) with D_i = sum_j P_ij dP_ij; and because O = P V,
D_i = <dO_i, O_i> (the row statistic the blockwise backward reads instead of
P).  The forward's saved LSE gives P back as exp(S - LSE) ("059 ·
FlashAttention" (wq-win), section 3: the backward recomputes the needed
probability blocks on chip from the inputs and the saved row statistics;
FlashAttention notes (xwysyy), "Recomputation").

Grouped-query heads: query head h reads key/value head h // G, so the
gradient of a key/value head is the sum over the G query heads that read it
(the chain rule through the shared operand).

``attention_backward*`` form P and dS in full (the plain definition).
``blockwise_backward_head`` runs the recompute form block by block -- outer
loop over key/value blocks, inner loop over query blocks, P rebuilt from the
saved LSE and dS from D = <dO, O> -- so the tests can show in fp64 that it
reaches the one-shot result.
"""

from __future__ import annotations

import numpy as np

from .attention import _run_jobs, attention_probs

__all__ = [
    "attention_backward_head",
    "attention_backward",
    "attention_backward_varlen",
    "blockwise_backward_head",
    "softmax_backward_delta",
]


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def attention_backward_head(q, k, v, do, scale, causal=False, nk_valid=None, return_ds=False):
    """dQ, dK, dV of one head from the definition (P and dS materialised).

    q: [Nq, d], k: [Nk, d], v: [Nk, dv], do: [Nq, dv].  Masked keys get P = 0
    and therefore dS = 0; a row with no visible key contributes nothing.
    With return_ds, also returns (P, dS).
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    _, p, _ = attention_probs(q, k, scale, causal, nk_valid)
    dv = p.T @ do                                   # dV = P^T dO
    dp = do @ v.T                                   # dP = dO V^T
    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))  # (diag(p) - p p^T) dp, row-wise
    dq = scale * (ds @ k)                           # dQ = scale dS K
    dk = scale * (ds.T @ q)                         # dK = scale dS^T Q
    if return_ds:
        return dq, dk, dv, p, ds
    return dq, dk, dv


def softmax_backward_delta(o, do):
    """D_i = <dO_i, O_i> per row (equal to sum_j P_ij dP_ij since O = P V)."""
    return (_f64(o) * _f64(do)).sum(axis=-1)


def attention_backward(q, k, v, do, scale, causal=False, seqlens_k=None, workers=None):
    """Batched, grouped-query backward in the [B, N, H, d] layout.

    q, do: [B, Nq, Hq, d]; k, v: [B, Nk, Hkv, d]; seqlens_k: optional [B]
    valid key counts.  Returns dQ [B, Nq, Hq, d], dK and dV [B, Nk, Hkv, d]
    in fp64; the key/value gradients sum over each KV head's query heads.
    """
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    dq = np.zeros((B, Nq, Hq, d))
    dk = np.zeros((B, Nk, Hkv, k.shape[3]))
    dv = np.zeros((B, Nk, Hkv, v.shape[3]))
    jobs = [(b, h) for b in range(B) for h in range(Hq)]

    def one(bh):
        b, h = bh
        nk_valid = None if seqlens_k is None else int(seqlens_k[b])
        return attention_backward_head(q[b, :, h], k[b, :, h // G], v[b, :, h // G],
                                       do[b, :, h], scale, causal, nk_valid)

    for (b, h), (dq_, dk_, dv_) in zip(jobs, _run_jobs(one, jobs, workers)):
        dq[b, :, h] = dq_
        dk[b, :, h // G] += dk_
        dv[b, :, h // G] += dv_
    return dq, dk, dv


def attention_backward_varlen(q, k, v, do, cu_seqlens_q, cu_seqlens_k, scale, causal=False,
                              workers=None):
    """Packed variable-length backward (layouts of attention_forward_varlen).

    q, do: [Tq, Hq, d]; k, v: [Tk, Hkv, d].  Returns dQ [Tq, Hq, d], dK and
    dV [Tk, Hkv, d]; rows and keys that belong to no sequence stay zero.
    """
    Tq, Hq, d = q.shape
    Tk, Hkv = k.shape[0], k.shape[1]
    G = Hq // Hkv
    cq = [int(x) for x in cu_seqlens_q]
    ck = [int(x) for x in cu_seqlens_k]
    dq = np.zeros((Tq, Hq, d))
    dk = np.zeros((Tk, Hkv, k.shape[2]))
    dv = np.zeros((Tk, Hkv, v.shape[2]))
    jobs = [(z, h) for z in range(len(cq) - 1) for h in range(Hq)]

    def one(zh):
        z, h = zh
        return attention_backward_head(q[cq[z]:cq[z + 1], h], k[ck[z]:ck[z + 1], h // G],
                                       v[ck[z]:ck[z + 1], h // G], do[cq[z]:cq[z + 1], h],
                                       scale, causal)

    for (z, h), (dq_, dk_, dv_) in zip(jobs, _run_jobs(one, jobs, workers)):
        dq[cq[z]:cq[z + 1], h] = dq_
        dk[ck[z]:ck[z + 1], h // G] += dk_
        dv[ck[z]:ck[z + 1], h // G] += dv_
    return dq, dk, dv


def blockwise_backward_head(q, k, v, o, do, lse, scale, causal=False, nk_valid=None,
                            block_rows=16, block_cols=16):
    """The recompute backward for one head, block by block, in fp64.

    Inputs are those a fused backward reads: Q, K, V, the forward's O and LSE
    (natural log) and dO.  D = <dO, O> per row is formed first.  Then for each
    key/value block (outer loop) and each query block (inner loop):
        P  = exp(S - LSE)              (S masked to -inf; rows with LSE = -inf give 0)
        dV_block += P^T dO_block
        dP = dO_block V_block^T
        dS = P * (dP - D_block)
        dQ_block += scale dS K_block,  dK_block += scale dS^T Q_block
    Returns dQ, dK, dV.
    """
    q, k, v, o, do, lse = (_f64(x) for x in (q, k, v, o, do, lse))
    nq, nk = q.shape[0], k.shape[0]
    if nk_valid is None:
        nk_valid = nk
    dmat = softmax_backward_delta(o, do)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for c0 in range(0, nk, block_cols):
        cols = np.arange(c0, min(c0 + block_cols, nk))
        for r0 in range(0, nq, block_rows):
            rows = np.arange(r0, min(r0 + block_rows, nq))
            s = scale * (q[rows] @ k[cols].T)
            vis = cols[None, :] < nk_valid
            if causal:
                vis = vis & (cols[None, :] <= rows[:, None])
            s = np.where(vis, s, -np.inf)
            has = np.isfinite(lse[rows])
            p = np.where(has[:, None], np.exp(s - np.where(has, lse[rows], 0.0)[:, None]), 0.0)
            dv[cols] += p.T @ do[rows]
            dp = do[rows] @ v[cols].T
            ds = p * (dp - dmat[rows][:, None])
            dq[rows] += scale * (ds @ k[cols])
            dk[cols] += scale * (ds.T @ q[rows])
    return dq, dk, dv
