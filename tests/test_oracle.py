"""Pins of the fp64 CPU oracle to facts fixed by the pages and by the mathematics.

Each test checks the oracle against something other than itself: the worked
example printed on the pages (golden file), closed forms, invariants of the
definition, a library routine with the same definition (torch's
scaled_dot_product_attention in float64 on the CPU), and brute force in pure
Python on tiny inputs.  The planted-mistake tests show that the pins reject
the plausible wrong variants (naive block averaging, a denominator-only merge,
a missing scale, a transposed operand, a mirrored causal mask, a wrong GQA
head map, the wrong logarithm base).
"""

import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import (
    attention_forward,
    attention_forward_varlen,
    attention_head,
    attention_probs,
    attention_rows,
    online_softmax_head,
)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.txt")


def _golden():
    vals = {}
    for line in open(GOLDEN, encoding="utf-8"):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        key, expr = [t.strip() for t in line.split("=", 1)]
        if expr.startswith("ln"):
            vals[key] = math.log(float(expr[2:]))
        else:
            vals[key] = float(Fraction(expr))
    return vals


G = _golden()


def _worked_inputs():
    # d = 1, scale = 1: score_j = q * k_j.
    q = np.array([[1.0]])
    k = np.array([[G["score_0"]], [G["score_1"]]])
    v = np.array([[G["value_0"]], [G["value_1"]]])
    return q, k, v


# ---------------------------------------------------------------- worked example

def test_worked_example_output_and_lse():
    q, k, v = _worked_inputs()
    o, lse = attention_head(q, k, v, scale=1.0)
    assert abs(o[0, 0] - G["output"]) <= 1e-12
    assert abs(lse[0] - G["lse"]) <= 1e-12


def test_worked_example_weights():
    q, k, _ = _worked_inputs()
    _, p, _ = attention_probs(q, k, scale=1.0)
    np.testing.assert_allclose(p[0], [G["weight_0"], G["weight_1"]], rtol=0, atol=1e-15)


@pytest.mark.parametrize("normalize_each_step", [False, True])
def test_worked_example_blockwise_one_key_per_block(normalize_each_step):
    q, k, v = _worked_inputs()
    o, lse = online_softmax_head(q, k, v, 1.0, block_rows=1, block_cols=1,
                                 normalize_each_step=normalize_each_step)
    assert abs(o[0, 0] - G["output"]) <= 1e-12
    assert abs(lse[0] - G["lse"]) <= 1e-12


def test_worked_example_merge_states():
    """After block 0: m=0, l=1, u=2; after block 1 both l and u were scaled by 1/3."""
    q, k, v = _worked_inputs()
    _, _, trace = online_softmax_head(q, k, v, 1.0, block_rows=1, block_cols=1, trace_row=0)
    (m0, l0, u0), (m1, l1, u1) = trace
    assert (m0, l0, u0[0]) == pytest.approx((G["state_after_block0_m"], G["state_after_block0_l"],
                                             G["state_after_block0_u"]), abs=1e-12)
    assert (m1, l1, u1[0]) == pytest.approx((G["state_after_block1_m"], G["state_after_block1_l"],
                                             G["state_after_block1_u"]), abs=1e-12)
    # The factor applied to the old statistics is exactly 1/3 = e^(0 - ln 3).
    assert math.exp(m0 - m1) == pytest.approx(G["merge_factor"], abs=1e-15)


def test_worked_example_rejects_wrong_merges():
    """The wrong variants the page warns about give 6 and 9, not the oracle's 8."""
    q, k, v = _worked_inputs()
    o, _ = attention_head(q, k, v, scale=1.0)
    s = [G["score_0"], G["score_1"]]
    vals = [G["value_0"], G["value_1"]]
    # Averaging per-block softmax outputs: each single-key block has softmax 1.
    naive = sum(vals) / 2
    assert naive == G["naive_block_average"]
    # Rescaling only the denominator: u keeps block 0's value at its old base.
    m_new = max(s)
    l_bad = 1.0 * math.exp(s[0] - m_new) + math.exp(s[1] - m_new)
    u_bad = vals[0] + math.exp(s[1] - m_new) * vals[1]
    assert u_bad / l_bad == pytest.approx(G["denominator_only_merge"], abs=1e-12)
    assert abs(o[0, 0] - naive) > 1 and abs(o[0, 0] - u_bad / l_bad) > 0.5


# ---------------------------------------------------------------- invariants

def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("causal,nk_valid", [(False, None), (True, None), (False, 13), (True, 9)])
def test_probability_rows_sum_to_one(causal, nk_valid):
    q, k = _rand((17, 8), 1), _rand((21, 8), 2)
    _, p, _ = attention_probs(q, k, 0.35, causal, nk_valid)
    assert (p >= 0).all()
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    nk = nk_valid if nk_valid is not None else 21
    assert (p[:, nk:] == 0).all()
    if causal:
        assert (np.triu(p, 1) == 0).all()


def test_constant_values_give_constant_output():
    q, k = _rand((19, 16), 3), _rand((23, 16), 4)
    c = _rand((1, 5), 5)
    v = np.repeat(c, 23, axis=0)
    for causal, nkv in [(False, None), (True, None), (False, 7)]:
        o, _ = attention_head(q, k, v, 0.25, causal, nkv)
        np.testing.assert_allclose(o, np.repeat(c, 19, axis=0), rtol=0, atol=1e-12)


def test_shift_invariance_of_keys():
    """Adding w to every key row shifts row i's scores by scale*q_i.w."""
    q, k, v = _rand((11, 6), 6), _rand((14, 6), 7), _rand((14, 6), 8)
    w = _rand((6,), 9)
    scale = 0.4
    o1, l1 = attention_head(q, k, v, scale)
    o2, l2 = attention_head(q, k + w, v, scale)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-10)
    np.testing.assert_allclose(l2 - l1, scale * (q @ w), rtol=0, atol=1e-10)


def test_joint_permutation_of_keys_and_values():
    q, k, v = _rand((9, 5), 10), _rand((15, 5), 11), _rand((15, 7), 12)
    perm = np.random.default_rng(13).permutation(15)
    o1, l1 = attention_head(q, k, v, 0.5)
    o2, l2 = attention_head(q, k[perm], v[perm], 0.5)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-12)
    # With key padding, permuting within the visible set changes nothing either.
    p_in = np.concatenate([np.random.default_rng(14).permutation(10), np.arange(10, 15)])
    o3, l3 = attention_head(q, k, v, 0.5, nk_valid=10)
    o4, l4 = attention_head(q, k[p_in], v[p_in], 0.5, nk_valid=10)
    np.testing.assert_allclose(o4, o3, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l4, l3, rtol=0, atol=1e-12)


def test_masked_keys_do_not_matter():
    """Keys past the valid length, and future keys under the causal mask, are ignored."""
    q, k, v = _rand((12, 4), 15), _rand((12, 4), 16), _rand((12, 4), 17)
    o1, l1 = attention_head(q, k, v, 0.5, nk_valid=8)
    k2, v2 = k.copy(), v.copy()
    k2[8:] += 100.0
    v2[8:] -= 50.0
    o2, l2 = attention_head(q, k2, v2, 0.5, nk_valid=8)
    np.testing.assert_allclose(o2, o1, atol=0, rtol=0)
    np.testing.assert_allclose(l2, l1, atol=0, rtol=0)
    oc, lc = attention_head(q, k, v, 0.5, causal=True)
    for i in range(12):
        k3, v3 = k.copy(), v.copy()
        k3[i + 1:] = 7.0
        v3[i + 1:] = -3.0
        o3, l3 = attention_head(q, k3, v3, 0.5, causal=True, rows=[i])
        np.testing.assert_allclose(o3[0], oc[i], atol=1e-14, rtol=0)
        assert l3[0] == pytest.approx(lc[i], abs=1e-14)


# ---------------------------------------------------------------- closed forms

def test_single_key_closed_form():
    q, k, v = _rand((7, 3), 18), _rand((1, 3), 19), _rand((1, 4), 20)
    o, lse = attention_head(q, k, v, 0.7)
    np.testing.assert_allclose(o, np.repeat(v, 7, axis=0), rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, 0.7 * (q @ k[0]), rtol=0, atol=1e-14)


def test_zero_query_closed_form():
    """q = 0: uniform weights over visible keys, LSE = ln(#visible) (natural log)."""
    n = 10
    q = np.zeros((n, 4))
    k, v = _rand((n, 4), 21), _rand((n, 3), 22)
    o, lse = attention_head(q, k, v, 1.3, causal=True)
    for i in range(n):
        np.testing.assert_allclose(o[i], v[: i + 1].mean(axis=0), rtol=0, atol=1e-13)
        assert lse[i] == pytest.approx(math.log(i + 1), abs=1e-14)
    o, lse = attention_head(q, k, v, 1.3, nk_valid=6)
    np.testing.assert_allclose(o, np.repeat(v[:6].mean(axis=0, keepdims=True), n, 0), atol=1e-13)
    np.testing.assert_allclose(lse, math.log(6), atol=1e-14)


def test_causal_first_row_closed_form():
    q, k, v = _rand((5, 3), 23), _rand((5, 3), 24), _rand((5, 2), 25)
    o, lse = attention_head(q, k, v, 0.9, causal=True)
    np.testing.assert_allclose(o[0], v[0], rtol=0, atol=1e-15)
    assert lse[0] == pytest.approx(0.9 * q[0] @ k[0], abs=1e-15)


def test_row_without_visible_key():
    q, k, v = _rand((3, 2), 26), _rand((4, 2), 27), _rand((4, 2), 28)
    o, lse = attention_head(q, k, v, 1.0, nk_valid=0)
    assert (o == 0).all() and np.isneginf(lse).all()
    o, lse = online_softmax_head(q, k, v, 1.0, nk_valid=0, block_rows=2, block_cols=3)
    assert (o == 0).all() and np.isneginf(lse).all()


# ---------------------------------------------------------------- brute force and library

def _brute(q, k, v, scale, causal, nk_valid):
    """Pure-Python loops over tiny inputs."""
    out, lses = [], []
    for i in range(len(q)):
        terms = []
        for j in range(len(k)):
            if j >= nk_valid or (causal and j > i):
                continue
            s = scale * sum(q[i][t] * k[j][t] for t in range(len(q[i])))
            terms.append((s, j))
        top = max(s for s, _ in terms)
        den = sum(math.exp(s - top) for s, _ in terms)
        row = [sum(math.exp(s - top) * v[j][c] for s, j in terms) / den for c in range(len(v[0]))]
        out.append(row)
        lses.append(top + math.log(den))
    return np.array(out), np.array(lses)


@pytest.mark.parametrize("causal,nk_valid", [(False, 5), (True, 5), (False, 3), (True, 4)])
def test_brute_force_tiny(causal, nk_valid):
    q, k, v = _rand((4, 3), 29), _rand((5, 3), 30), _rand((5, 2), 31)
    o, lse = attention_head(q, k, v, 0.6, causal, nk_valid)
    ob, lb = _brute(q.tolist(), k.tolist(), v.tolist(), 0.6, causal, nk_valid)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lb, rtol=0, atol=1e-13)


def _sdpa(q, k, v, scale, mask):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v),
                                                         attn_mask=torch.from_numpy(mask)[None, None],
                                                         scale=scale)
    s = scale * torch.from_numpy(q) @ torch.from_numpy(k).T
    s = s.masked_fill(~torch.from_numpy(mask), -math.inf)
    return o[0, 0].numpy(), torch.logsumexp(s, dim=1).numpy()


@pytest.mark.parametrize("nq,nk,d,dv,causal,nk_valid", [
    (33, 47, 16, 24, False, None),
    (40, 40, 64, 64, True, None),
    (31, 50, 8, 8, False, 29),
    (45, 45, 32, 16, True, 30),
])
def test_against_library_sdpa_float64(nq, nk, d, dv, causal, nk_valid):
    q, k, v = _rand((nq, d), 32) * 2.0, _rand((nk, d), 33), _rand((nk, dv), 34)
    scale = 1.0 / math.sqrt(d) * 1.7
    i = np.arange(nq)[:, None]
    j = np.arange(nk)[None, :]
    mask = j < (nk if nk_valid is None else nk_valid)
    if causal:
        mask = mask & (j <= i)
    o, lse = attention_head(q, k, v, scale, causal, nk_valid)
    o_ref, lse_ref = _sdpa(q, k, v, scale, mask)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-10)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-10)


def test_pins_reject_planted_mistakes():
    """Plausible oracle mistakes, planted in copies on the CPU, fail the pins above."""
    q, k, v = _rand((6, 4), 35), _rand((8, 4), 36), _rand((8, 3), 37)
    scale = 0.45
    good, good_lse = _brute(q.tolist(), k.tolist(), v.tolist(), scale, True, 8)
    # (a) scale dropped
    o_a, _ = attention_head(q, k, v, 1.0, True)
    # (b) mirrored causal mask (j >= i)
    o_b, _ = attention_head(q[::-1], k[::-1], v[::-1], scale, True)
    # (c) LSE in log2 instead of natural log
    lse_c = good_lse / math.log(2.0)
    for bad in (o_a, o_b[::-1]):
        assert np.abs(bad - good).max() > 1e-3
    assert np.abs(lse_c - good_lse).max() > 1e-3
    o, lse = attention_head(q, k, v, scale, True)
    np.testing.assert_allclose(o, good, atol=1e-13)
    np.testing.assert_allclose(lse, good_lse, atol=1e-13)


# ---------------------------------------------------------------- blockwise == one-shot

@pytest.mark.parametrize("d", [1, 4, 64])
def test_blockwise_recurrence_matches_definition(d):
    rng = np.random.default_rng(100 + d)
    for nq, nk in [(67, 67), (13, 41), (64, 64)]:
        q = rng.standard_normal((nq, d)) * 3.0
        k = rng.standard_normal((nk, d))
        v = rng.standard_normal((nk, d + 1))
        scale = 1.0 / math.sqrt(d)
        for causal, nkv in [(False, None), (True, None), (False, nk - 5), (True, nk // 2)]:
            ref_o, ref_l = attention_head(q, k, v, scale, causal, nkv)
            for br in (1, 3, 16, 64):
                for bc in (1, 5, 16, 64):
                    for tau, norm in [(None, False), (8.0, False), (None, True)]:
                        o, l = online_softmax_head(q, k, v, scale, causal, nkv, br, bc, tau, norm)
                        np.testing.assert_allclose(o, ref_o, rtol=0, atol=1e-12)
                        np.testing.assert_allclose(l, ref_l, rtol=0, atol=1e-12)


def test_conditional_rescale_keeps_stale_max():
    """With tau = 8 (log2 units) some max increases are skipped, and the result is still exact."""
    rng = np.random.default_rng(7)
    n, d = 64, 8
    q = rng.standard_normal((n, d)) * 2.0
    k = rng.standard_normal((n, d))
    v = rng.standard_normal((n, d))
    _, _, tr_plain = online_softmax_head(q, k, v, 0.5, block_rows=64, block_cols=4, trace_row=5)
    o_tau, l_tau, tr_tau = online_softmax_head(q, k, v, 0.5, block_rows=64, block_cols=4, tau=8.0,
                                               trace_row=5)
    m_plain = [t[0] for t in tr_plain]
    m_tau = [t[0] for t in tr_tau]
    assert any(a < b for a, b in zip(m_tau, m_plain)), "tau never skipped a rescale"
    # The stale max is never more than tau (in log2 units) below the true max.
    assert all((b - a) / math.log(2.0) <= 8.0 + 1e-12 for a, b in zip(m_tau, m_plain))
    ref_o, ref_l = attention_head(q, k, v, 0.5)
    np.testing.assert_allclose(o_tau, ref_o, atol=1e-12)
    np.testing.assert_allclose(l_tau, ref_l, atol=1e-12)


# ---------------------------------------------------------------- batched layouts

def test_gqa_equals_mha_with_repeated_heads():
    rng = np.random.default_rng(40)
    B, N, Hq, Hkv, d = 2, 19, 8, 2, 8
    q = rng.standard_normal((B, N, Hq, d))
    k = rng.standard_normal((B, N, Hkv, d))
    v = rng.standard_normal((B, N, Hkv, d))
    seq = [19, 11]
    o, lse = attention_forward(q, k, v, 0.3, causal=True, seqlens_k=seq)
    kr = torch.from_numpy(k).repeat_interleave(Hq // Hkv, dim=2).numpy()
    vr = torch.from_numpy(v).repeat_interleave(Hq // Hkv, dim=2).numpy()
    o2, lse2 = attention_forward(q, kr, vr, 0.3, causal=True, seqlens_k=seq, workers=3)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)
    # And each head against the library routine.
    for b in range(B):
        for h in range(Hq):
            mask = (np.arange(N)[None, :] <= np.arange(N)[:, None]) & (np.arange(N)[None, :] < seq[b])
            o_ref, l_ref = _sdpa(q[b, :, h], kr[b, :, h], vr[b, :, h], 0.3, mask)
            np.testing.assert_allclose(o[b, :, h], o_ref, atol=1e-10)
            np.testing.assert_allclose(lse[b, h], l_ref, atol=1e-10)
    # A wrong head map (h % Hkv instead of h // G) changes the answer.
    o_wrong_h1, _ = attention_head(q[0, :, 1], k[0, :, 1], v[0, :, 1], 0.3, True)
    assert np.abs(o_wrong_h1 - o[0, :, 1]).max() > 1e-3


def test_varlen_matches_library_per_sequence():
    rng = np.random.default_rng(41)
    lens = [5, 17, 1, 9]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T, Hq, Hkv, d = int(cu[-1]), 4, 2, 8
    q = rng.standard_normal((T, Hq, d))
    k = rng.standard_normal((T, Hkv, d))
    v = rng.standard_normal((T, Hkv, d))
    o, lse = attention_forward_varlen(q, k, v, cu, cu, 0.4, causal=True, workers=2)
    for z, L in enumerate(lens):
        a, b = cu[z], cu[z + 1]
        mask = np.arange(L)[None, :] <= np.arange(L)[:, None]
        for h in range(Hq):
            o_ref, l_ref = _sdpa(q[a:b, h], k[a:b, h // 2], v[a:b, h // 2], 0.4, mask)
            np.testing.assert_allclose(o[a:b, h], o_ref, atol=1e-10)
            np.testing.assert_allclose(lse[h, a:b], l_ref, atol=1e-10)


def test_sampled_rows_match_full_forward():
    rng = np.random.default_rng(42)
    B, N, Hq, Hkv, d = 2, 33, 4, 1, 16
    q = rng.standard_normal((B, N, Hq, d))
    k = rng.standard_normal((B, N, Hkv, d))
    v = rng.standard_normal((B, N, Hkv, d))
    o, lse = attention_forward(q, k, v, 0.25, causal=True, seqlens_k=[33, 20])
    samples = [(0, 0, 0), (1, 3, 32), (1, 2, 19), (0, 1, 17)]
    os_, ls_ = attention_rows(q, k, v, 0.25, True, samples, seqlens_k=[33, 20])
    for n, (b, h, i) in enumerate(samples):
        np.testing.assert_allclose(os_[n], o[b, i, h], atol=1e-14)
        assert ls_[n] == pytest.approx(lse[b, h, i], abs=1e-14)


def test_partial_head_selection_leaves_rest_unset():
    rng = np.random.default_rng(43)
    q = rng.standard_normal((1, 8, 2, 4))
    k = rng.standard_normal((1, 8, 2, 4))
    o, lse = attention_forward(q, k, k, 0.5, heads=[(0, 1)])
    assert np.isnan(o[0, :, 0]).all() and np.isfinite(o[0, :, 1]).all()
    assert np.isnan(lse[0, 0]).all() and np.isfinite(lse[0, 1]).all()
