"""Pins of the block-sparse oracle to facts fixed by the definition.

The operator (FlashAttention notes (xwysyy), "Block-Sparse FlashAttention"):
S = scale Q K^T with the positions of zero blocks of the block mask set to
-inf, P = softmax(S), O = P V.  Checked against: the dense oracle for an
all-ones mask, dense attention over a sliced key range for masks with one
block per row, brute force in pure Python (with causal and padding masks),
empty rows, per-head masks; a transposed block mask (a plausible mistake) is
shown to fail the brute-force pin.
"""

import math

import numpy as np
import pytest

from oracle import (attention_forward, attention_forward_blocksparse, attention_head,
                    block_mask_to_elements)


def _inputs(seed, B, Nq, Nk, Hq, Hkv, d):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, Nq, Hq, d)), rng.standard_normal((B, Nk, Hkv, d)),
            rng.standard_normal((B, Nk, Hkv, d)))


def test_all_ones_mask_is_dense():
    q, k, v = _inputs(1, 2, 37, 45, 4, 2, 8)
    bm = np.ones((1, 5, 6), dtype=np.uint8)
    for causal in (False, True):
        o1, l1 = attention_forward_blocksparse(q, k, v, 0.3, bm, bq=8, bk=8, causal=causal)
        o2, l2 = attention_forward(q, k, v, 0.3, causal)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_one_block_per_row_is_attention_over_that_key_block():
    q, k, v = _inputs(2, 1, 32, 40, 2, 2, 4)
    bq, bk = 8, 10
    cols = [3, 0, 2, 1]  # query block r sees key block cols[r] only
    bm = np.zeros((1, 4, 4), dtype=np.uint8)
    for r, c in enumerate(cols):
        bm[0, r, c] = 1
    o, lse = attention_forward_blocksparse(q, k, v, 0.5, bm, bq=bq, bk=bk)
    for h in range(2):
        for r, c in enumerate(cols):
            rows = slice(r * bq, (r + 1) * bq)
            ks = slice(c * bk, (c + 1) * bk)
            o_ref, l_ref = attention_head(q[0, rows, h], k[0, ks, h], v[0, ks, h], 0.5)
            assert np.abs(o[0, rows, h] - o_ref).max() < 1e-12
            assert np.abs(lse[0, h, rows] - l_ref).max() < 1e-12


def _brute(q, k, v, scale, allowed, causal, nk_valid):
    nq, nk = q.shape[0], k.shape[0]
    o = np.zeros((nq, v.shape[1]))
    lse = np.zeros(nq)
    for i in range(nq):
        ws, vis = [], []
        for j in range(nk):
            if allowed[i][j] and j < nk_valid and (not causal or j <= i):
                vis.append(j)
                ws.append(scale * sum(q[i, t] * k[j, t] for t in range(q.shape[1])))
        if not vis:
            lse[i] = -math.inf
            continue
        m = max(ws)
        e = [math.exp(w - m) for w in ws]
        tot = sum(e)
        lse[i] = m + math.log(tot)
        for w, j in zip(e, vis):
            o[i] += (w / tot) * v[j]
    return o, lse


@pytest.mark.parametrize("causal,nk_valid", [(False, 19), (True, 23), (True, 7)])
def test_brute_force_with_causal_and_padding(causal, nk_valid):
    rng = np.random.default_rng(3)
    q, k, v = _inputs(4, 1, 17, 23, 1, 1, 3)
    bq, bk = 4, 5
    bm = rng.integers(0, 2, size=(1, 5, 5)).astype(np.uint8)
    bm[0, 1] = 0  # an empty block row
    o, lse = attention_forward_blocksparse(q, k, v, 0.7, bm, bq=bq, bk=bk, causal=causal,
                                           seqlens_k=np.array([nk_valid]))
    allowed = block_mask_to_elements(bm[0], 17, 23, bq, bk)
    ob, lb = _brute(q[0, :, 0], k[0, :, 0], v[0, :, 0], 0.7, allowed, causal, nk_valid)
    assert np.abs(o[0, :, 0] - ob).max() < 1e-12
    fin = np.isfinite(lb)
    assert np.array_equal(np.isfinite(lse[0, 0]), fin)
    assert np.abs(lse[0, 0][fin] - lb[fin]).max() < 1e-12
    assert (o[0, 4:8, 0] == 0).all() and np.isneginf(lse[0, 0, 4:8]).all()


def test_transposed_block_mask_fails_the_brute_force_pin():
    rng = np.random.default_rng(5)
    q, k, v = _inputs(6, 1, 16, 16, 1, 1, 3)
    bm = rng.integers(0, 2, size=(1, 4, 4)).astype(np.uint8)
    bm[0, 0, 3] = 1
    bm[0, 3, 0] = 0
    wrong = bm.transpose(0, 2, 1)
    o, _ = attention_forward_blocksparse(q, k, v, 0.7, wrong, bq=4, bk=4)
    ob, _ = _brute(q[0, :, 0], k[0, :, 0], v[0, :, 0], 0.7,
                   block_mask_to_elements(bm[0], 16, 16, 4, 4), False, 16)
    assert np.abs(o[0, :, 0] - ob).max() > 1e-3


def test_per_head_masks():
    rng = np.random.default_rng(7)
    q, k, v = _inputs(8, 2, 20, 24, 4, 2, 4)
    bm = rng.integers(0, 2, size=(4, 3, 3)).astype(np.uint8)
    o, lse = attention_forward_blocksparse(q, k, v, 0.4, bm, bq=8, bk=8, causal=True)
    for h in range(4):
        o1, l1 = attention_forward_blocksparse(q[:, :, h:h + 1], k[:, :, h // 2:h // 2 + 1],
                                               v[:, :, h // 2:h // 2 + 1], 0.4, bm[h:h + 1], bq=8,
                                               bk=8, causal=True)
        assert np.array_equal(o[:, :, h], o1[:, :, 0])
        assert np.array_equal(lse[:, h], l1[:, 0])
