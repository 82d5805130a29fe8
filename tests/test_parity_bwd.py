"""GPU parity of the backward pass against the fp64 CPU oracle.

The backward consumes the GPU forward's own O and LSE (as in training), and a
seeded upstream gradient dO.  Small shapes are compared on every element of
dQ, dK and dV; they span several key and query tiles, ragged tails,
Nq != Nk, GQA groups and key padding, at head dimensions 128 and 64.  At the
headline benchmark's size and at the d = 64 batch workload's, one whole
(batch, KV head) slice -- its query heads' dQ and the KV head's dK, dV -- is
compared element by element.  The packed (varlen) entry point is checked on
small ragged batches in full (with a zero-length sequence, lq != lk, GQA and
both masks) and, at the ragged benchmark's size, on its shortest sequence.
Tolerances are derived in parity_util (and, for a dQ column that is a small
difference of large terms, in the climbing-score test).
"""

import math

import numpy as np
import pytest
import torch

import oracle
from exact_attention_18_amd import attn, inputs
from parity_util import assert_grad_parity, grad_errors, to_np64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

SMALL = [
    # B, Nq, Nk, Hq, Hkv, causal, padded
    (1, 64, 64, 1, 1, False, False),
    (2, 200, 200, 4, 2, True, False),
    (1, 130, 517, 2, 1, False, False),
    (1, 517, 130, 2, 2, True, False),
    (2, 333, 333, 8, 2, True, True),
    (3, 257, 257, 2, 2, False, True),
    (1, 1, 1, 1, 1, True, False),
    (1, 300, 45, 4, 1, True, False),
    # dQ workgroups pack 8 query heads (G = 8, 16) and several groups per unit (G = 6, 16)
    (1, 300, 300, 16, 2, True, True),
    (2, 257, 257, 6, 1, True, False),
    (1, 200, 333, 16, 1, False, False),
    (1, 390, 390, 12, 1, True, True),
]


def _fwd_bwd(q, k, v, do, scale, causal, seqlens):
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    sl = None if seqlens is None else seqlens.to(DEV)
    o, lse = attn.attn_fwd(qd, kd, vd, scale, causal, sl)
    dq, dk, dv = attn.attn_bwd(qd, kd, vd, o, lse, dod, scale, causal, sl)
    torch.cuda.synchronize()
    return dq, dk, dv


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("B,Nq,Nk,Hq,Hkv,causal,padded", SMALL)
def test_backward_small_shapes_full_oracle(B, Nq, Nk, Hq, Hkv, causal, padded, d):
    seed = 9000 + B * 31 + Nq * 7 + Nk + Hq * 3 + int(causal) + d
    q, k, v = inputs.make_qkv(B, Nq, Nk, Hq, Hkv, d, seed, q_mult=2.0)
    do = inputs.make_dout(q.shape, seed + 1)
    seqlens = None
    if padded:
        seqlens = inputs.make_seqlens(B, 0, Nk, seed + 2)
        seqlens[0] = 0
        if B > 1:
            seqlens[1] = Nk
    scale = 1.0 / math.sqrt(d)
    print(f"[parity-bwd] B={B} Nq={Nq} Nk={Nk} Hq={Hq} Hkv={Hkv} d={d} causal={causal} "
          f"padded={padded}", flush=True)
    dq, dk, dv = _fwd_bwd(q, k, v, do, scale, causal, seqlens)
    rq, rk, rv = oracle.attention_backward(to_np64(q), to_np64(k), to_np64(v), to_np64(do), scale,
                                           causal, None if seqlens is None else seqlens.numpy(),
                                           workers=8)
    floors = {"dq": 0.0, "dk": 0.0, "dv": 0.0}
    if Nk == 1:
        # One key: P = 1 in every row, so dS = dP - D vanishes in exact
        # arithmetic and dQ, dK are rounding residues of dP and D = <dO, O>;
        # they are measured against the size of those cancelled terms.
        o1 = np.repeat(to_np64(v), Hq // Hkv, axis=2)  # with one key, O = V exactly
        o1 = np.broadcast_to(o1, do.shape)
        dmax = float(np.abs(oracle.softmax_backward_delta(o1, to_np64(do))).max())
        floors["dq"] = scale * dmax * float(np.abs(to_np64(k)).max())
        floors["dk"] = scale * dmax * float(np.abs(to_np64(q)).max())
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        assert_grad_parity(grad_errors(to_np64(got), ref, floors[name]), name)
    if padded:  # keys past a batch element's length get exactly zero gradient
        sl = seqlens.numpy()
        for b in range(B):
            assert (dk[b, sl[b]:] == 0).all() and (dv[b, sl[b]:] == 0).all()


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("B,N,Hq,Hkv,causal,padded", [
    (2, 700, 8, 2, True, False),     # 4 heads per dQ workgroup
    (1, 333, 16, 2, True, True),     # 8 heads per dQ workgroup, key padding
    (2, 517, 6, 1, True, False),     # 2 heads per dQ workgroup, 3 workgroups per row block
    (1, 300, 16, 1, False, False),   # 8 heads, 2 workgroups per row block, non-causal
])
def test_backward_grouped_heads_dq_equals_repeated_kv_heads_bitwise(B, N, Hq, Hkv, causal, padded,
                                                                   d):
    """dQ of a GQA call equals dQ of the MHA call with K and V repeated G times, bit for bit.

    The dQ kernel packs up to 8 query heads of a KV group into a workgroup
    (256 / heads rows each) while the MHA call takes one head per workgroup.
    A row's arithmetic does not depend on that: keys past a row's causal
    limit add exact zeros, and D and the LSE come from forwards that are
    themselves bitwise equal.
    """
    G = Hq // Hkv
    q, k, v = inputs.make_qkv(B, N, N, Hq, Hkv, d, 9050 + Hq + N + d, q_mult=3.0)
    do = inputs.make_dout(q.shape, 9051 + N)
    seqlens = inputs.make_seqlens(B, N // 2, N, 9052 + N) if padded else None
    kr = k.repeat_interleave(G, dim=2).contiguous()
    vr = v.repeat_interleave(G, dim=2).contiguous()
    print(f"[parity-bwd] gqa dq bitwise B={B} N={N} Hq={Hq} Hkv={Hkv} d={d} causal={causal}",
          flush=True)
    dq1, _, _ = _fwd_bwd(q, k, v, do, 0.088, causal, seqlens)
    dq2, _, _ = _fwd_bwd(q, kr, vr, do, 0.088, causal, seqlens)
    assert torch.equal(dq1, dq2)


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("scale_mult", [-1.0, 0.0])
def test_backward_any_finite_scale_full_oracle(d, scale_mult):
    """Negative and zero scales through the forward and the backward."""
    B, N, Hq, Hkv = 2, 300, 4, 2
    seed = 9070 + d + int(scale_mult)
    q, k, v = inputs.make_qkv(B, N, N, Hq, Hkv, d, seed, q_mult=2.0)
    do = inputs.make_dout(q.shape, seed + 1)
    seqlens = inputs.make_seqlens(B, 1, N, seed + 2)
    scale = scale_mult / math.sqrt(d)
    for causal in (True, False):
        print(f"[parity-bwd] scale={scale:.4f} d={d} causal={causal}", flush=True)
        dq, dk, dv = _fwd_bwd(q, k, v, do, scale, causal, seqlens)
        rq, rk, rv = oracle.attention_backward(to_np64(q), to_np64(k), to_np64(v), to_np64(do),
                                               scale, causal, seqlens.numpy(), workers=8)
        for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
            if scale == 0.0 and name != "dv":
                # scores do not depend on Q or K: their gradients are exactly zero
                assert (got == 0).all(), name
                assert np.abs(ref).max() == 0.0, name
                continue
            assert_grad_parity(grad_errors(to_np64(got), ref), name)


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("causal", [True, False])
def test_backward_climbing_scores_full_oracle(d, causal):
    """Scores that climb along the keys (a new row maximum in every key tile, one
    key 100 above the trend) or fall (later tiles' P underflows): the forward
    rescales at every tile, and the backward rebuilds P from an LSE near 200.

    The trend lives in dimension 0 of the keys (up to ~300 there, against
    N(0, 1) elsewhere).  Since sum_j dS_ij = 0, dQ_i0 = scale sum_j dS_ij K_j0
    is the small difference of terms as large as scale sum_j |dS_ij| |K_j0|:
    rounding dS to bf16 (<= 2^-9 relative) and D = <dO, O> taken from the
    bf16 O (<= 2^-9 sum_d |dO_id O_id|) move it by up to 2^-9 scale
    sum_j (|dS_ij| + P_ij sum_d |dO_id O_id|) |K_j0|, whatever the kernel
    (a CPU model of those two roundings alone reaches 0.55 of this).  That
    column is held to twice this bound plus its own bf16 rounding; every
    other column of dQ, and dK and dV, to the usual bars.
    """
    B, N, Hq, Hkv = 1, 600, 4, 2
    scale = 1.0 / math.sqrt(d)
    q, k, v = inputs.make_trend_qkv(B, N, Hq, Hkv, d, 9420 + d, scale, step=0.25, jump_at=400,
                                    jump=100.0)
    do = inputs.make_dout(q.shape, 9421 + d)
    print(f"[parity-bwd] climbing scores d={d} causal={causal}", flush=True)
    dq, dk, dv = _fwd_bwd(q, k, v, do, scale, causal, None)
    qn, kn, vn, don = (to_np64(t) for t in (q, k, v, do))
    rq, rk, rv = oracle.attention_backward(qn, kn, vn, don, scale, causal, None, workers=8)
    dqn = to_np64(dq)
    for name, got, ref in (("dq[..., 1:]", dqn[..., 1:], rq[..., 1:]), ("dk", to_np64(dk), rk),
                           ("dv", to_np64(dv), rv)):
        errs = grad_errors(got, ref)
        print(f"[parity-bwd]   {name}: {errs}", flush=True)
        assert_grad_parity(errs, name)
    worst = 0.0
    for h in range(Hq):
        kh = kn[0, :, h // (Hq // Hkv)]
        _, _, _, p, ds = oracle.attention_backward_head(qn[0, :, h], kh, vn[0, :, h // (Hq // Hkv)],
                                                        don[0, :, h], scale, causal,
                                                        return_ds=True)
        o_bf = (p @ vn[0, :, h // (Hq // Hkv)]).astype(np.float32)
        o_bf = torch.from_numpy(o_bf).to(torch.bfloat16).double().numpy()
        d_err = np.abs(o_bf * don[0, :, h]).sum(axis=1, keepdims=True)
        bound = 2.0 ** -9 * scale * ((np.abs(ds) + p * d_err) @ np.abs(kh[:, 0]))
        err = np.abs(dqn[0, :, h, 0] - rq[0, :, h, 0])
        allowed = np.maximum(2 * bound + 2.0 ** -8 * np.abs(rq[0, :, h, 0]), 1e-30)
        worst = max(worst, float((err / allowed).max()))
    print(f"[parity-bwd]   dq[..., 0]: error / bound {worst:.3f}", flush=True)
    assert worst <= 1.0


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_constant_values_give_zero_score_gradients(d, causal):
    """With V equal to a constant c_h in every row of KV head h, O = c_h for any
    scores, so dQ = dK = 0 exactly: dP_ij = c_h sum_d dO_id equals D_i = <dO_i,
    O_i> and dS = P (dP - D) vanishes.  The GPU forms D from its bf16 O, so
    dS_ij is P_ij times at most |sum_d dO_id (O_id - c_h)| plus fp32 rounding,
    which bounds dQ_i by scale e_i max|K| and dK_j by scale sum_i P_ij e_i |Q_i|
    (e_i that residue, P_ij <= 1).  dV = P^T dO is compared with the oracle."""
    B, N, Hq, Hkv = 1, 333, 4, 2
    q, k, _ = inputs.make_qkv(B, N, N, Hq, Hkv, d, 9700 + d + int(causal), q_mult=3.0)
    consts = torch.tensor([1.5, -0.375], dtype=torch.bfloat16)
    v = consts.view(1, 1, Hkv, 1).expand(B, N, Hkv, d).contiguous()
    do = inputs.make_dout(q.shape, 9701 + d)
    scale = 1.0 / math.sqrt(d)
    print(f"[parity-bwd] constant V d={d} causal={causal}", flush=True)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = attn.attn_fwd(qd, kd, vd, scale, causal)
    dq, dk, dv = attn.attn_bwd(qd, kd, vd, o, lse, dod, scale, causal)
    torch.cuda.synchronize()
    qn, kn, don, on = to_np64(q), to_np64(k), to_np64(do), to_np64(o)
    c = np.repeat(consts.double().numpy(), Hq // Hkv)                   # per query head
    absdo = np.abs(don).sum(axis=-1)                                    # [B, N, Hq]
    e = np.abs((don * (on - c[None, None, :, None])).sum(axis=-1)) + 2.0 ** -20 * np.abs(c) * absdo
    dq_bound = 2 * scale * e * np.abs(kn).max() + 1e-30
    assert (np.abs(to_np64(dq)).max(axis=-1) <= dq_bound).all()
    G = Hq // Hkv
    dkn = to_np64(dk)
    for g in range(Hkv):  # a KV head's dK sums its G query heads
        dk_bound = 2 * scale * e[:, :, g * G:(g + 1) * G].sum() * np.abs(qn).max() + 1e-30
        assert np.abs(dkn[:, :, g]).max() <= dk_bound
    _, _, rv = oracle.attention_backward(qn, kn, to_np64(v), don, scale, causal, None, workers=8)
    assert_grad_parity(grad_errors(to_np64(dv), rv), "dv")


@pytest.mark.parametrize("d", [128, 64])
def test_backward_key_rows_past_2gib(d):
    """The backward over K and V of 2^18 + 77 rows of 8 KiB (4096 / d KV heads):
    rows past 2 GiB into each array.  dQ, dK and dV of heads 0 and the last
    against the oracle in full."""
    B, Nq, Nk = 1, 100, (1 << 18) + 77
    H = 8192 // (2 * d)
    q, k, v = inputs.make_qkv_on(DEV, B, Nq, Nk, H, H, d, 9510 + d)
    do = inputs.make_dout(q.shape, 9511 + d).to(DEV)
    assert k[0, -1].data_ptr() - k.data_ptr() > 2 ** 31
    scale = 1.0 / math.sqrt(d)
    print(f"[parity-bwd] key rows past 2 GiB d={d} H={H} Nk={Nk}", flush=True)
    o, lse = attn.attn_fwd(q, k, v, scale, False)
    dq, dk, dv = attn.attn_bwd(q, k, v, o, lse, do, scale, False)
    torch.cuda.synchronize()
    for h in (0, H - 1):
        rq, rk, rv = oracle.attention_backward_head(to_np64(q[0, :, h]), to_np64(k[0, :, h]),
                                                    to_np64(v[0, :, h]), to_np64(do[0, :, h]),
                                                    scale, False)
        for name, got, ref in (("dq", dq[0, :, h], rq), ("dk", dk[0, :, h], rk),
                               ("dv", dv[0, :, h], rv)):
            assert_grad_parity(grad_errors(to_np64(got), ref), f"{name} head {h}")
    del q, k, v, do, o, lse, dq, dk, dv
    torch.cuda.empty_cache()


@pytest.mark.parametrize("d", [128, 64])
def test_backward_is_deterministic(d):
    q, k, v = inputs.make_qkv(2, 700, 700, 8, 2, d, 9100, q_mult=3.0)
    do = inputs.make_dout(q.shape, 9101)
    a = _fwd_bwd(q, k, v, do, 0.088, True, None)
    b = _fwd_bwd(q, k, v, do, 0.088, True, None)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("wname", [inputs.HEADLINE, "batch64_h16_n1024_d64"])
def test_backward_full_size_slice(wname):
    """A benchmark workload at full size; one (batch, KV head) slice compared in full."""
    w = inputs.WORKLOADS[wname]
    x = inputs.workload_inputs(w)
    do = inputs.make_dout(x["q"].shape, w.seed + 77)
    print(f"[parity-bwd] full size {w.name}", flush=True)
    dq, dk, dv = _fwd_bwd(x["q"], x["k"], x["v"], do, w.scale, w.causal, None)
    assert torch.isfinite(dq).all() and torch.isfinite(dk).all() and torch.isfinite(dv).all()
    G = w.Hq // w.Hkv
    b, hkv = min(1, w.B - 1), min(3, w.Hkv - 1)
    hs = slice(hkv * G, (hkv + 1) * G)
    q = to_np64(x["q"][b:b + 1, :, hs])
    k = to_np64(x["k"][b:b + 1, :, hkv:hkv + 1])
    v = to_np64(x["v"][b:b + 1, :, hkv:hkv + 1])
    rq, rk, rv = oracle.attention_backward(q, k, v, to_np64(do[b:b + 1, :, hs]), w.scale, w.causal,
                                           workers=4)
    for name, got, ref in (("dq", dq[b:b + 1, :, hs], rq), ("dk", dk[b:b + 1, :, hkv:hkv + 1], rk),
                           ("dv", dv[b:b + 1, :, hkv:hkv + 1], rv)):
        errs = grad_errors(to_np64(got), ref)
        print(f"[parity-bwd] {w.name} {name}: {errs}", flush=True)
        assert_grad_parity(errs, name)


def _fwd_bwd_varlen(q, k, v, do, cq, ck, mq, mk, scale, causal, order=None):
    qd, kd, vd, dod, cqd, ckd = (t.to(DEV) for t in (q, k, v, do, cq, ck))
    od = None if order is None else order.to(DEV)
    o, lse = attn.attn_fwd_varlen(qd, kd, vd, cqd, ckd, mq, mk, scale, causal, seq_order=od)
    dq, dk, dv = attn.attn_bwd_varlen(qd, kd, vd, o, lse, dod, cqd, ckd, mq, mk, scale, causal,
                                      seq_order=od)
    torch.cuda.synchronize()
    return dq, dk, dv


VARLEN = [
    # query lengths, key lengths (None: the same), Hq, Hkv, causal
    ([1, 130, 257, 0, 64, 200], None, 4, 2, True),
    ([1, 130, 257, 0, 64, 200], None, 16, 2, True),
    ([300, 7, 129], None, 6, 1, False),
    ([1, 130, 257, 0, 64, 200], None, 4, 4, False),
    ([64, 129, 5], [300, 17, 128], 2, 1, False),
    ([64, 129, 5, 0], [300, 17, 128, 40], 4, 1, True),
]


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("lq,lk,Hq,Hkv,causal", VARLEN)
def test_backward_varlen_small_full_oracle(lq, lk, Hq, Hkv, causal, d):
    lq = torch.tensor(lq, dtype=torch.int32)
    lk = lq.clone() if lk is None else torch.tensor(lk, dtype=torch.int32)
    cq, ck = inputs.cu_from_lengths(lq), inputs.cu_from_lengths(lk)
    Tq, Tk = int(cq[-1]), int(ck[-1])
    seed = 9300 + Tq + 3 * Tk + Hq + int(causal) + d
    q, _, _ = inputs.make_packed_qkv(Tq, 1, Hq, Hkv, d, seed, q_mult=2.0)
    _, k, v = inputs.make_packed_qkv(1, Tk, Hq, Hkv, d, seed + 1)
    do = inputs.make_dout(q.shape, seed + 2)
    scale = 1.0 / math.sqrt(d)
    print(f"[parity-bwd] varlen lq={lq.tolist()} lk={lk.tolist()} Hq={Hq} Hkv={Hkv} d={d} "
          f"causal={causal}", flush=True)
    dq, dk, dv = _fwd_bwd_varlen(q, k, v, do, cq, ck, int(lq.max()), int(lk.max()), scale, causal)
    rq, rk, rv = oracle.attention_backward_varlen(to_np64(q), to_np64(k), to_np64(v), to_np64(do),
                                                  cq.numpy(), ck.numpy(), scale, causal, workers=8)
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        assert_grad_parity(grad_errors(to_np64(got), ref), name)
    # keys of a sequence with no query rows get exactly zero gradient
    for z in range(len(lq)):
        if int(lq[z]) == 0:
            assert (dk[int(ck[z]):int(ck[z + 1])] == 0).all()
            assert (dv[int(ck[z]):int(ck[z + 1])] == 0).all()


def test_backward_varlen_plan_order_changes_nothing():
    lq = torch.tensor([40, 700, 3, 260], dtype=torch.int32)
    cq = inputs.cu_from_lengths(lq)
    T = int(cq[-1])
    q, k, v = inputs.make_packed_qkv(T, T, 4, 2, 128, 9400, q_mult=2.0)
    do = inputs.make_dout(q.shape, 9401)
    mx = int(lq.max())
    order = attn.attn_varlen_plan(cq.to(DEV), cq.to(DEV), mx, mx, True).cpu()
    a = _fwd_bwd_varlen(q, k, v, do, cq, cq, mx, mx, 0.088, True)
    b = _fwd_bwd_varlen(q, k, v, do, cq, cq, mx, mx, 0.088, True, order)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_backward_varlen_full_size_shortest_sequence():
    """The ragged benchmark workload; its shortest sequence compared in full for two heads."""
    w = inputs.WORKLOADS["varlen_causal_8seq_h32_d128"]
    x = inputs.workload_inputs(w)
    do = inputs.make_dout(x["q"].shape, w.seed + 77)
    cu, mx = x["cu_seqlens_q"], x["max_seqlen"]
    print(f"[parity-bwd] full size {w.name}", flush=True)
    dq, dk, dv = _fwd_bwd_varlen(x["q"], x["k"], x["v"], do, cu, cu, mx, mx, w.scale, w.causal)
    assert torch.isfinite(dq).all() and torch.isfinite(dk).all() and torch.isfinite(dv).all()
    z = int(torch.argmin(x["lengths"]))
    r0, r1 = int(cu[z]), int(cu[z + 1])
    G = w.Hq // w.Hkv
    for h in (0, w.Hq - 1):
        hk = h // G
        rq, rk, rv = oracle.attention_backward_head(
            to_np64(x["q"][r0:r1, h]), to_np64(x["k"][r0:r1, hk]), to_np64(x["v"][r0:r1, hk]),
            to_np64(do[r0:r1, h]), w.scale, w.causal)
        errs = grad_errors(to_np64(dq[r0:r1, h]), rq)
        print(f"[parity-bwd] {w.name} seq {z} (len {r1 - r0}) head {h} dq: {errs}", flush=True)
        assert_grad_parity(errs, "dq")
        if G == 1:  # with one query head per KV head, dK and dV of the head compare directly
            assert_grad_parity(grad_errors(to_np64(dk[r0:r1, hk]), rk), "dk")
            assert_grad_parity(grad_errors(to_np64(dv[r0:r1, hk]), rv), "dv")
