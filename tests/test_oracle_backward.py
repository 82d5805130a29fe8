"""Pins of the fp64 backward oracle to facts fixed by the pages and by the mathematics.

The backward oracle is checked against: the gradient teaching example printed
on the pages (golden file), central finite differences of the forward
definition, torch autograd of the plain definition in float64 on the CPU,
invariants of the softmax gradient (rows of dS sum to zero, so the key
gradients sum to zero; the value gradients sum to the upstream gradient; a
common shift of every key changes no gradient), GQA as repeated-head MHA,
packed sequences as separate heads, and the blockwise recompute form.  The
planted-mistake tests show the finite-difference pin rejects the plausible
wrong variants (a dropped row term, a flipped sign, a missing scale, a
transposed contraction).
"""

import math
import os

import numpy as np
import pytest
import torch

from oracle import (
    attention_backward,
    attention_backward_head,
    attention_backward_varlen,
    attention_forward,
    attention_head,
    attention_probs,
    blockwise_backward_head,
    softmax_backward_delta,
)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_gradient.txt")


def _golden():
    vals = {}
    for line in open(GOLDEN, encoding="utf-8"):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        key, expr = [t.strip() for t in line.split("=", 1)]
        if "*ln" in expr:
            a, b = expr.split("*ln")
            vals[key] = float(a) * math.log(float(b))
        else:
            vals[key] = float(expr)
    return vals


G = _golden()


def _worked():
    # d = 1, scale = 1, q = 1: the scores are the keys, 0 and ln 3 (weights 1/4, 3/4).
    q = np.array([[1.0]])
    k = np.array([[0.0], [math.log(3.0)]])
    v = np.array([[G["value_0"]], [G["value_1"]]])
    do = np.array([[G["upstream"]]])
    return q, k, v, do


def test_worked_gradient_example():
    q, k, v, do = _worked()
    dq, dk, dv, p, ds = attention_backward_head(q, k, v, do, 1.0, return_ds=True)
    o, _ = attention_head(q, k, v, 1.0)
    assert np.allclose(p[0], [G["weight_0"], G["weight_1"]], atol=1e-15)
    assert abs(o[0, 0] - G["output"]) < 1e-13
    assert np.allclose(ds[0], [G["dscore_0"], G["dscore_1"]], atol=1e-13)
    assert abs(ds.sum() - G["dscore_sum"]) < 1e-13
    assert np.allclose(dv[:, 0], [G["dv_0"], G["dv_1"]], atol=1e-13)
    assert np.allclose(dk[:, 0], [G["dk_0"], G["dk_1"]], atol=1e-13)
    assert abs(dq[0, 0] - G["dq"]) < 1e-13


def test_worked_gradient_blockwise_reproduces_the_two_numbers():
    """One key per block: the blockwise recompute reaches -1.5 and +1.5 (via dK = dS^T q)."""
    q, k, v, do = _worked()
    o, lse = attention_head(q, k, v, 1.0)
    dq, dk, dv = blockwise_backward_head(q, k, v, o, do, lse, 1.0, block_rows=1, block_cols=1)
    assert np.allclose(dk[:, 0], [G["dscore_0"], G["dscore_1"]], atol=1e-13)  # q = 1
    assert np.allclose(dv[:, 0], [G["dv_0"], G["dv_1"]], atol=1e-13)
    assert abs(dq[0, 0] - G["dq"]) < 1e-13


# ---------------------------------------------------------------- finite differences

def _loss(q, k, v, do, scale, causal, nk_valid):
    o, _ = attention_head(q, k, v, scale, causal, nk_valid)
    return float((o * do).sum())


def _fd_grads(q, k, v, do, scale, causal, nk_valid, h=1e-6):
    """Central differences of L = sum(O * dO) with respect to every input entry."""
    out = []
    for which in range(3):
        arrs = [q.copy(), k.copy(), v.copy()]
        g = np.zeros_like(arrs[which])
        for idx in np.ndindex(g.shape):
            plus = [a.copy() for a in arrs]
            minus = [a.copy() for a in arrs]
            plus[which][idx] += h
            minus[which][idx] -= h
            g[idx] = (_loss(*plus, do, scale, causal, nk_valid)
                      - _loss(*minus, do, scale, causal, nk_valid)) / (2 * h)
        out.append(g)
    return out


FD_CASES = [
    # nq, nk, d, causal, nk_valid
    (4, 6, 3, False, None),
    (6, 6, 2, True, None),
    (5, 7, 3, False, 4),
    (7, 5, 2, True, 3),
]


@pytest.mark.parametrize("nq,nk,d,causal,nk_valid", FD_CASES)
def test_backward_matches_finite_differences(nq, nk, d, causal, nk_valid):
    rng = np.random.default_rng(100 + nq * 10 + nk + d + int(causal))
    q, k, v, do = (rng.standard_normal(s) for s in [(nq, d), (nk, d), (nk, d), (nq, d)])
    scale = 0.7
    dq, dk, dv = attention_backward_head(q, k, v, do, scale, causal, nk_valid)
    fq, fk, fv = _fd_grads(q, k, v, do, scale, causal, nk_valid)
    for got, ref in ((dq, fq), (dk, fk), (dv, fv)):
        assert np.abs(got - ref).max() <= 1e-7 * max(1.0, np.abs(ref).max())


def _buggy(kind, q, k, v, do, scale, causal, nk_valid):
    """Plausible mistakes, planted in a copy of the oracle's steps."""
    _, p, _ = attention_probs(q, k, scale, causal, nk_valid)
    dp = do @ v.T
    dmat = (p * dp).sum(axis=1, keepdims=True)
    ds = p * (dp - dmat)
    if kind == "no_row_term":
        ds = p * dp
    elif kind == "sign":
        ds = p * (dmat - dp)
    dq = (1.0 if kind == "no_scale" else scale) * (ds @ k)
    dk = scale * (ds.T @ q)
    dv = p.T @ do
    if kind == "dv_uses_dp":
        dv = p.T @ (do - do.mean(axis=0))
    return dq, dk, dv


@pytest.mark.parametrize("kind", ["no_row_term", "sign", "no_scale", "dv_uses_dp"])
def test_finite_differences_reject_planted_mistakes(kind):
    rng = np.random.default_rng(7)
    q, k, v, do = (rng.standard_normal(s) for s in [(4, 3), (5, 3), (5, 3), (4, 3)])
    scale = 0.7
    got = _buggy(kind, q, k, v, do, scale, False, None)
    ref = _fd_grads(q, k, v, do, scale, False, None)
    worst = max(np.abs(a - b).max() for a, b in zip(got, ref))
    assert worst > 1e-3, kind


# ---------------------------------------------------------------- autograd cross-check

def _torch_reference(q, k, v, do, scale, causal, nk_valid):
    """Softmax attention written with torch ops, differentiated by autograd (float64)."""
    qt, kt, vt = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    s = scale * qt @ kt.T
    nq, nk = s.shape
    mask = torch.zeros(nq, nk, dtype=torch.bool)
    if nk_valid is not None:
        mask |= torch.arange(nk)[None, :] >= nk_valid
    if causal:
        mask |= torch.arange(nk)[None, :] > torch.arange(nq)[:, None]
    s = s.masked_fill(mask, float("-inf"))
    p = torch.softmax(s, dim=1)
    p = torch.nan_to_num(p, nan=0.0)  # rows without a visible key
    o = p @ vt
    (o * torch.tensor(do)).sum().backward()
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


@pytest.mark.parametrize("nq,nk,d,causal,nk_valid", FD_CASES + [(33, 40, 8, True, None), (20, 31, 16, False, 17)])
def test_backward_matches_torch_autograd(nq, nk, d, causal, nk_valid):
    rng = np.random.default_rng(200 + nq + nk + d)
    q, k, v, do = (rng.standard_normal(s) for s in [(nq, d), (nk, d), (nk, d), (nq, d)])
    scale = 1.0 / math.sqrt(d)
    got = attention_backward_head(q, k, v, do, scale, causal, nk_valid)
    ref = _torch_reference(q, k, v, do, scale, causal, nk_valid)
    for a, b in zip(got, ref):
        assert np.abs(a - b).max() <= 1e-12 * max(1.0, np.abs(b).max())


# ---------------------------------------------------------------- invariants

def test_softmax_gradient_invariants():
    rng = np.random.default_rng(11)
    nq, nk, d = 12, 17, 6
    q, k, v, do = (rng.standard_normal(s) for s in [(nq, d), (nk, d), (nk, d), (nq, d)])
    scale = 0.4
    dq, dk, dv, p, ds = attention_backward_head(q, k, v, do, scale, True, return_ds=True)
    assert np.abs(ds.sum(axis=1)).max() < 1e-13                 # rows of dS sum to zero
    assert np.abs(dk.sum(axis=0)).max() < 1e-12                 # hence sum_j dK_j = 0
    assert np.abs(dv.sum(axis=0) - do.sum(axis=0)).max() < 1e-12  # P rows sum to one
    o, _ = attention_head(q, k, v, scale, True)
    assert np.abs(softmax_backward_delta(o, do) - (p * (do @ v.T)).sum(axis=1)).max() < 1e-12
    # A common shift of every key leaves P, hence every gradient, unchanged.
    w = rng.standard_normal(d)
    dq2, dk2, dv2 = attention_backward_head(q, k + w, v, do, scale, True)
    for a, b in ((dq, dq2), (dk, dk2), (dv, dv2)):
        assert np.abs(a - b).max() < 1e-10


def test_row_without_visible_key_has_zero_gradient():
    rng = np.random.default_rng(12)
    q, k, v, do = (rng.standard_normal(s) for s in [(3, 4), (5, 4), (5, 4), (3, 4)])
    dq, dk, dv = attention_backward_head(q, k, v, do, 0.5, False, nk_valid=0)
    assert not dq.any() and not dk.any() and not dv.any()


# ---------------------------------------------------------------- blockwise, GQA, varlen

@pytest.mark.parametrize("br,bc", [(1, 1), (4, 3), (16, 16), (7, 64)])
@pytest.mark.parametrize("causal,nk_valid", [(False, None), (True, None), (False, 19), (True, 0)])
def test_blockwise_backward_equals_one_shot(br, bc, causal, nk_valid):
    rng = np.random.default_rng(300 + br + bc)
    nq, nk, d = 23, 29, 5
    q, k, v, do = (rng.standard_normal(s) for s in [(nq, d), (nk, d), (nk, d), (nq, d)])
    scale = 0.6
    o, lse = attention_head(q, k, v, scale, causal, nk_valid)
    ref = attention_backward_head(q, k, v, do, scale, causal, nk_valid)
    got = blockwise_backward_head(q, k, v, o, do, lse, scale, causal, nk_valid, br, bc)
    for a, b in zip(got, ref):
        assert np.abs(a - b).max() <= 1e-12 * max(1.0, np.abs(b).max())


def test_gqa_backward_is_repeated_head_mha_summed():
    rng = np.random.default_rng(13)
    B, Nq, Nk, Hq, Hkv, d = 2, 9, 11, 6, 2, 4
    q = rng.standard_normal((B, Nq, Hq, d))
    k = rng.standard_normal((B, Nk, Hkv, d))
    v = rng.standard_normal((B, Nk, Hkv, d))
    do = rng.standard_normal((B, Nq, Hq, d))
    sl = np.array([11, 5])
    dq, dk, dv = attention_backward(q, k, v, do, 0.5, True, sl)
    G = Hq // Hkv
    kr, vr = np.repeat(k, G, axis=2), np.repeat(v, G, axis=2)
    dq2, dkr, dvr = attention_backward(q, kr, vr, do, 0.5, True, sl)
    assert np.abs(dq - dq2).max() < 1e-13
    assert np.abs(dk - dkr.reshape(B, Nk, Hkv, G, d).sum(axis=3)).max() < 1e-13
    assert np.abs(dv - dvr.reshape(B, Nk, Hkv, G, d).sum(axis=3)).max() < 1e-13
    # padded keys get no gradient
    assert not dk[1, 5:].any() and not dv[1, 5:].any()


def test_varlen_backward_is_per_sequence():
    rng = np.random.default_rng(14)
    lq, lk = [3, 0, 7, 5], [4, 2, 7, 1]
    cq, ck = np.concatenate([[0], np.cumsum(lq)]), np.concatenate([[0], np.cumsum(lk)])
    Hq, Hkv, d = 4, 2, 3
    q = rng.standard_normal((cq[-1], Hq, d))
    k = rng.standard_normal((ck[-1], Hkv, d))
    v = rng.standard_normal((ck[-1], Hkv, d))
    do = rng.standard_normal((cq[-1], Hq, d))
    dq, dk, dv = attention_backward_varlen(q, k, v, do, cq, ck, 0.5, True)
    for z in range(len(lq)):
        if lq[z] == 0:
            continue
        a, b, c, e = cq[z], cq[z + 1], ck[z], ck[z + 1]
        dq1, dk1, dv1 = attention_backward(q[None, a:b], k[None, c:e], v[None, c:e],
                                           do[None, a:b], 0.5, True)
        assert np.abs(dq[a:b] - dq1[0]).max() < 1e-13
        assert np.abs(dk[c:e] - dk1[0]).max() < 1e-13
        assert np.abs(dv[c:e] - dv1[0]).max() < 1e-13
    assert not dk[ck[1]:ck[2]].any()  # the sequence with no queries leaves its keys untouched
