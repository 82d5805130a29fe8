"""GPU parity: the HIP forward against the fp64 CPU oracle on the same seeded bf16 inputs.

Small shapes are compared element by element over every output; they span
several query and key tiles, ragged tails, Nq != Nk, every GQA group size of
the workloads, key padding (including empty and full rows) and packed
sequences; inputs whose scores climb along the keys drive the conditional
rescale at every key tile and overflow exponentials taken against a stale
maximum.  The full-size workloads are launched exactly as the benchmark
launches them, into outputs prefilled with NaN, and compared with the oracle
on every element, plus properties that hold at any size (the GPU's own LSE
normalises its row, reruns are bitwise identical, nothing outside the outputs
is written).
"""

import math

import numpy as np
import pytest
import torch

import oracle
from exact_attention_18_amd import attn, inputs
from parity_util import assert_parity, errors, sample_rows, to_np64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _run(q, k, v, scale, causal, seqlens=None):
    o, lse = attn.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), scale, causal,
                           None if seqlens is None else seqlens.to(DEV))
    torch.cuda.synchronize()
    return o, lse


SMALL = [
    # B, Nq, Nk, Hq, Hkv, d, causal, padded
    (1, 256, 256, 1, 1, 64, False, False),
    (2, 200, 200, 4, 4, 64, False, False),
    (2, 333, 333, 8, 2, 128, True, False),
    (1, 130, 517, 2, 1, 128, False, False),
    (1, 517, 130, 2, 2, 64, True, False),
    (1, 130, 517, 2, 2, 128, True, False),
    (3, 300, 300, 8, 1, 64, True, True),
    (4, 257, 257, 2, 2, 128, False, True),
    (2, 391, 391, 4, 4, 128, True, True),
    (1, 1, 1, 1, 1, 64, False, False),
    (1, 1, 1, 1, 1, 128, True, False),
    (1, 64, 0, 1, 1, 128, False, False),
    (1, 96, 0, 2, 1, 64, True, False),
    # d = 128 with more query rows than keys under the causal mask (rows past
    # Nk see every key), grouped heads, and key padding with it
    (1, 517, 130, 4, 2, 128, True, False),
    (2, 300, 200, 8, 4, 128, True, True),
]


@pytest.mark.parametrize("B,Nq,Nk,Hq,Hkv,d,causal,padded", SMALL)
def test_small_shapes_full_oracle(B, Nq, Nk, Hq, Hkv, d, causal, padded):
    seed = 7000 + B * 31 + Nq * 7 + Nk + Hq * 3 + d + int(causal)
    q, k, v = inputs.make_qkv(B, Nq, Nk, Hq, Hkv, d, seed, q_mult=2.0)
    seqlens = None
    if padded:
        seqlens = inputs.make_seqlens(B, 0, Nk, seed + 1)
        seqlens[0] = 0
        if B > 1:
            seqlens[1] = Nk
    scale = 1.0 / math.sqrt(d)
    print(f"[parity] B={B} Nq={Nq} Nk={Nk} Hq={Hq} Hkv={Hkv} d={d} causal={causal}", flush=True)
    o, lse = _run(q, k, v, scale, causal, seqlens)
    o_ref, lse_ref = oracle.attention_forward(to_np64(q), to_np64(k), to_np64(v), scale, causal,
                                              None if seqlens is None else seqlens.numpy(),
                                              workers=8)
    errs = errors(to_np64(o), to_np64(lse), o_ref, lse_ref)
    assert_parity(errs, "small")
    # Rows without any visible key: exactly zero output and -inf LSE.
    empty = np.isneginf(lse_ref)
    if empty.any():
        lse_np = to_np64(lse)
        assert np.isneginf(lse_np[empty]).all()
        o_np = to_np64(o).transpose(0, 2, 1, 3)  # [B,Hq,Nq,d]
        assert (o_np[empty] == 0).all()


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n_tiles", [1, 2, 3, 4, 5, 6])
@pytest.mark.parametrize("tail", [0, 17])
def test_key_tile_counts_full_oracle(d, causal, n_tiles, tail):
    """Every key-tile count from one to six, whole and ragged.

    A 64-key tile count of n puts the last tile at either parity of the
    double-buffered loop, and one or two tiles leave no steady-state
    iteration; a ragged tail masks the last tile.  Nq = 130 adds a query
    block whose waves hold no rows.
    """
    Nk = 64 * (n_tiles - 1) + (tail if tail else 64)
    Nq = 130
    seed = 7300 + 17 * n_tiles + tail + d + int(causal)
    q, k, v = inputs.make_qkv(2, Nq, Nk, 2, 1, d, seed, q_mult=2.0)
    scale = 1.0 / math.sqrt(d)
    print(f"[parity] tile counts Nq={Nq} Nk={Nk} d={d} causal={causal}", flush=True)
    o, lse = _run(q, k, v, scale, causal)
    o_ref, lse_ref = oracle.attention_forward(to_np64(q), to_np64(k), to_np64(v), scale, causal,
                                              None, workers=8)
    assert_parity(errors(to_np64(o), to_np64(lse), o_ref, lse_ref), "small")


ASYM = [
    # B, Nq, Nk, Hq, Hkv, causal, padded  (d_qk = 192, d_v = 128)
    (1, 300, 300, 4, 4, True, False),
    (2, 130, 517, 2, 1, False, False),
    (3, 257, 257, 4, 2, True, True),
    (1, 1, 1, 1, 1, False, False),
    (1, 64, 0, 2, 1, True, False),
]


@pytest.mark.parametrize("B,Nq,Nk,Hq,Hkv,causal,padded", ASYM)
def test_asymmetric_head_dims_full_oracle(B, Nq, Nk, Hq, Hkv, causal, padded):
    seed = 7500 + B * 31 + Nq * 7 + Nk + Hq * 3 + int(causal)
    q, k, v = inputs.make_qkv(B, Nq, Nk, Hq, Hkv, 192, seed, q_mult=2.0, d_v=128)
    seqlens = None
    if padded:
        seqlens = inputs.make_seqlens(B, 0, Nk, seed + 1)
        seqlens[0] = 0
    scale = 1.0 / math.sqrt(192)
    print(f"[parity] (192,128) B={B} Nq={Nq} Nk={Nk} Hq={Hq} Hkv={Hkv} causal={causal}", flush=True)
    o, lse = _run(q, k, v, scale, causal, seqlens)
    assert o.shape == (B, Nq, Hq, 128)
    o_ref, lse_ref = oracle.attention_forward(to_np64(q), to_np64(k), to_np64(v), scale, causal,
                                              None if seqlens is None else seqlens.numpy(),
                                              workers=8)
    assert_parity(errors(to_np64(o), to_np64(lse), o_ref, lse_ref), "(192,128)")


SPARSE = [
    # B, Nq, Nk, Hq, Hkv, causal, padded, mask_heads, density
    (1, 300, 300, 4, 4, False, False, 1, 0.5),
    (2, 517, 390, 4, 2, True, False, 4, 0.5),
    (2, 257, 700, 8, 2, False, True, 8, 0.3),
    (1, 1000, 1000, 2, 1, True, False, 1, 0.2),
    (1, 64, 64, 1, 1, False, False, 1, 0.0),
]


@pytest.mark.parametrize("B,Nq,Nk,Hq,Hkv,causal,padded,mh,density", SPARSE)
def test_blocksparse_full_oracle(B, Nq, Nk, Hq, Hkv, causal, padded, mh, density):
    seed = 7700 + B * 31 + Nq * 7 + Nk + Hq * 3 + int(causal)
    q, k, v = inputs.make_qkv(B, Nq, Nk, Hq, Hkv, 128, seed, q_mult=2.0)
    nbq, nbk = -(-Nq // 128), -(-Nk // 128)
    g = torch.Generator().manual_seed(seed + 3)
    bm = (torch.rand((mh, nbq, nbk), generator=g) < density).to(torch.uint8)
    if nbq > 1:
        bm[:, 1, :] = 0  # a query block with no visible key
    seqlens = None
    if padded:
        seqlens = inputs.make_seqlens(B, 0, Nk, seed + 1)
    scale = 1.0 / math.sqrt(128)
    print(f"[parity] block-sparse B={B} Nq={Nq} Nk={Nk} Hq={Hq} causal={causal} heads={mh}",
          flush=True)
    o, lse = attn.attn_fwd_blocksparse(q.to(DEV), k.to(DEV), v.to(DEV), bm.to(DEV), scale, causal,
                                       None if seqlens is None else seqlens.to(DEV))
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_forward_blocksparse(
        to_np64(q), to_np64(k), to_np64(v), scale, bm.numpy(), 128, 128, causal,
        None if seqlens is None else seqlens.numpy(), workers=8)
    errs = errors(to_np64(o), to_np64(lse), o_ref, lse_ref)
    assert_parity(errs, "block-sparse")
    empty = np.isneginf(lse_ref)
    assert np.isneginf(to_np64(lse)[empty]).all()


def test_blocksparse_longest_key_range():
    """Block-sparse at its largest key range, Nk = 262144 (4096 key tiles of 64):
    one query block visits every tile (its work list full), the other a random
    half of the blocks; all rows against the oracle."""
    Nq, Nk = 256, 262144
    q, k, v = inputs.make_qkv(1, Nq, Nk, 1, 1, 128, 7900, q_mult=2.0)
    nbk = Nk // 128
    g = torch.Generator().manual_seed(7901)
    bm = torch.zeros((1, Nq // 128, nbk), dtype=torch.uint8)
    bm[0, 0] = 1
    bm[0, 1] = (torch.rand(nbk, generator=g) < 0.5).to(torch.uint8)
    scale = 1.0 / math.sqrt(128)
    print(f"[parity] block-sparse Nk={Nk}", flush=True)
    o, lse = attn.attn_fwd_blocksparse(q.to(DEV), k.to(DEV), v.to(DEV), bm.to(DEV), scale, False)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_forward_blocksparse(
        to_np64(q), to_np64(k), to_np64(v), scale, bm.numpy(), 128, 128, False, workers=8)
    assert_parity(errors(to_np64(o), to_np64(lse), o_ref, lse_ref), "block-sparse Nk=262144")


def test_blocksparse_all_ones_is_the_dense_kernel_bitwise():
    """With every block set, the block-sparse kernel visits every key tile in order, as the dense one.

    Both run the same steps on the same MFMA shape, so the outputs are equal
    bit for bit; a missing, repeated or misordered tile would show.
    """
    q, k, v = inputs.make_qkv(2, 600, 600, 8, 2, 128, 7800, q_mult=3.0)
    bm = torch.ones((1, 5, 5), dtype=torch.uint8, device=DEV)
    for causal in (False, True):
        o1, l1 = attn.attn_fwd_blocksparse(q.to(DEV), k.to(DEV), v.to(DEV), bm, 0.088, causal)
        o2, l2 = attn.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), 0.088, causal)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_varlen_small_full_oracle():
    lengths = torch.tensor([1, 130, 257, 0, 64, 200], dtype=torch.int32)
    cu = inputs.cu_from_lengths(lengths)
    T = int(cu[-1])
    for causal, d, (Hq, Hkv) in [(True, 128, (4, 2)), (False, 64, (4, 4)), (True, 64, (8, 1))]:
        q, k, v = inputs.make_packed_qkv(T, T, Hq, Hkv, d, 8100 + d + int(causal))
        scale = 1.0 / math.sqrt(d)
        print(f"[parity] varlen causal={causal} d={d} Hq={Hq} Hkv={Hkv}", flush=True)
        o, lse = attn.attn_fwd_varlen(q.to(DEV), k.to(DEV), v.to(DEV), cu.to(DEV), cu.to(DEV),
                                      int(lengths.max()), int(lengths.max()), scale, causal)
        torch.cuda.synchronize()
        o_ref, lse_ref = oracle.attention_forward_varlen(to_np64(q), to_np64(k), to_np64(v),
                                                         cu.numpy(), cu.numpy(), scale, causal)
        assert_parity(errors(to_np64(o), to_np64(lse), o_ref, lse_ref), "varlen small")


def test_varlen_separate_key_lengths():
    """Packed sequences whose key lengths differ from their query lengths."""
    lq = torch.tensor([64, 129, 5], dtype=torch.int32)
    lk = torch.tensor([300, 17, 128], dtype=torch.int32)
    cq, ck = inputs.cu_from_lengths(lq), inputs.cu_from_lengths(lk)
    q, _, _ = inputs.make_packed_qkv(int(cq[-1]), 1, 2, 1, 128, 8200)
    _, k, v = inputs.make_packed_qkv(1, int(ck[-1]), 2, 1, 128, 8201)
    scale = 1.0 / math.sqrt(128)
    for causal in (False, True):
        o, lse = attn.attn_fwd_varlen(q.to(DEV), k.to(DEV), v.to(DEV), cq.to(DEV), ck.to(DEV),
                                      int(lq.max()), int(lk.max()), scale, causal)
        torch.cuda.synchronize()
        o_ref, lse_ref = oracle.attention_forward_varlen(to_np64(q), to_np64(k), to_np64(v),
                                                         cq.numpy(), ck.numpy(), scale, causal)
        assert_parity(errors(to_np64(o), to_np64(lse), o_ref, lse_ref), "varlen lq != lk")


def _plan_keys(lq, lk, mq, mk, causal):
    """Sort key of the LPT plan, from its definition: key tiles of the longest work tile."""
    lq = np.minimum(np.maximum(lq, 0), mq)
    lk = np.minimum(np.maximum(lk, 0), mk)
    w = np.minimum(lq, lk) if causal else lk
    return np.minimum((w + 63) // 64, 8191)


@pytest.mark.parametrize("case", ["mixed", "many", "equal"])
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_plan_orders_sequences_longest_first(case, causal):
    rng = np.random.default_rng(8600 + len(case) + int(causal))
    if case == "mixed":
        lq = np.array([1, 130, 257, 0, 64, 200, 5000, 63, 64, 65], dtype=np.int64)
        lk = np.array([300, 17, 257, 9, 0, 4096, 70, 63, 64, 700], dtype=np.int64)
    elif case == "many":
        lq = rng.integers(0, 2000, size=3000)
        lk = rng.integers(0, 2000, size=3000)
    else:
        lq = np.full(1500, 777)
        lk = np.full(1500, 777)
    mq, mk = int(lq.max()), int(lk.max())
    cq = inputs.cu_from_lengths(torch.tensor(lq, dtype=torch.int32)).to(DEV)
    ck = inputs.cu_from_lengths(torch.tensor(lk, dtype=torch.int32)).to(DEV)
    print(f"[parity] varlen plan {case} causal={causal} n={len(lq)}", flush=True)
    order = attn.attn_varlen_plan(cq, ck, mq, mk, causal).cpu().numpy()
    assert sorted(order.tolist()) == list(range(len(lq))), "not a permutation"
    keys = _plan_keys(lq, lk, mq, mk, causal)[order]
    assert (np.diff(keys) <= 0).all(), "keys increase somewhere"


def test_varlen_plan_changes_no_output():
    lengths = torch.tensor([1, 130, 257, 0, 64, 200, 700, 3], dtype=torch.int32)
    cu = inputs.cu_from_lengths(lengths).to(DEV)
    T, ms = int(lengths.sum()), int(lengths.max())
    for causal, d, (Hq, Hkv) in [(True, 128, (4, 2)), (False, 64, (4, 4))]:
        q, k, v = inputs.make_packed_qkv(T, T, Hq, Hkv, d, 8700 + d)
        qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
        scale = 1.0 / math.sqrt(d)
        plan = attn.attn_varlen_plan(cu, cu, ms, ms, causal)
        o1, l1 = attn.attn_fwd_varlen(qd, kd, vd, cu, cu, ms, ms, scale, causal)
        o2, l2 = attn.attn_fwd_varlen(qd, kd, vd, cu, cu, ms, ms, scale, causal, seq_order=plan)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        o_ref, lse_ref = oracle.attention_forward_varlen(to_np64(q), to_np64(k), to_np64(v),
                                                         cu.cpu().numpy(), cu.cpu().numpy(), scale,
                                                         causal)
        assert_parity(errors(to_np64(o2), to_np64(l2), o_ref, lse_ref), "varlen with plan")


def test_outputs_are_not_overrun():
    """O and LSE written inside their buffers only (sentinels around both)."""
    B, N, Hq, Hkv, d = 2, 333, 4, 2, 128
    q, k, v = inputs.make_qkv(B, N, N, Hq, Hkv, d, 8300)
    pad = 64
    n_o, n_l = B * N * Hq * d, B * Hq * N
    obuf = torch.full((n_o + 2 * pad,), 7.0, dtype=torch.bfloat16, device=DEV)
    lbuf = torch.full((n_l + 2 * pad,), 7.0, dtype=torch.float32, device=DEV)
    out = obuf[pad:pad + n_o].view(B, N, Hq, d)
    lse = lbuf[pad:pad + n_l].view(B, Hq, N)
    attn.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), 0.088, True, out=out, lse=lse)
    torch.cuda.synchronize()
    assert (obuf[:pad] == 7).all() and (obuf[-pad:] == 7).all()
    assert (lbuf[:pad] == 7).all() and (lbuf[-pad:] == 7).all()
    o_ref, lse_ref = oracle.attention_forward(to_np64(q), to_np64(k), to_np64(v), 0.088, True)
    assert_parity(errors(to_np64(out), to_np64(lse), o_ref, lse_ref), "sentinel")


def test_reruns_are_bitwise_identical():
    q, k, v = inputs.make_qkv(2, 1000, 1000, 8, 2, 128, 8400, q_mult=3.0)
    o1, l1 = _run(q, k, v, 0.088, True)
    o2, l2 = _run(q, k, v, 0.088, True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("B,N,Hq,Hkv,causal,padded", [
    (2, 1000, 8, 2, True, False),    # 4 heads per workgroup
    (1, 700, 16, 2, True, True),     # 8 heads per workgroup, key padding
    (2, 517, 6, 3, True, False),     # 2 heads per workgroup
    (1, 300, 12, 4, False, False),   # 1 head per workgroup (G = 3), non-causal
    (1, 600, 12, 2, True, False),    # G = 6: 2 heads per workgroup, 3 workgroups per row block
    (1, 520, 12, 1, True, True),     # G = 12: 4 heads per workgroup, 3 per row block, padding
    (1, 777, 16, 1, False, False),   # G = 16: 8 heads per workgroup, 2 per row block
])
def test_grouped_heads_equal_repeated_kv_heads_bitwise(B, N, Hq, Hkv, causal, padded):
    """GQA (h_kv = h_q // G) is MHA with each K/V head repeated G times.

    The d = 128 kernel packs up to 8 query heads of a KV group into one
    workgroup (256 / heads rows each) while the MHA call takes one head per
    workgroup; a row's arithmetic does not depend on that, so the outputs are
    bitwise equal.
    """
    G = Hq // Hkv
    q, k, v = inputs.make_qkv(B, N, N, Hq, Hkv, 128, 8600 + Hq + N, q_mult=3.0)
    seqlens = inputs.make_seqlens(B, N // 2, N, 8700 + N) if padded else None
    kr = k.repeat_interleave(G, dim=2).contiguous()
    vr = v.repeat_interleave(G, dim=2).contiguous()
    print(f"[parity] gqa bitwise B={B} N={N} Hq={Hq} Hkv={Hkv} causal={causal} padded={padded}",
          flush=True)
    o1, l1 = _run(q, k, v, 0.088, causal, seqlens)
    o2, l2 = _run(q, kr, vr, 0.088, causal, seqlens)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_grouped_heads_equal_repeated_kv_heads_bitwise_varlen():
    lengths = torch.tensor([300, 1, 517, 0, 256], dtype=torch.int32)
    cu = inputs.cu_from_lengths(lengths)
    T = int(cu[-1])
    q, k, v = inputs.make_packed_qkv(T, T, 8, 2, 128, 8800, q_mult=3.0)
    mx = int(lengths.max())
    outs = []
    for kk, vv in ((k, v), (k.repeat_interleave(4, dim=1).contiguous(),
                            v.repeat_interleave(4, dim=1).contiguous())):
        o, lse = attn.attn_fwd_varlen(q.to(DEV), kk.to(DEV), vv.to(DEV), cu.to(DEV), cu.to(DEV),
                                      mx, mx, 0.088, True)
        torch.cuda.synchronize()
        outs.append((o.cpu(), lse.cpu()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("d_qk,d_v", [(64, 64), (128, 128), (192, 128)])
@pytest.mark.parametrize("causal", [False, True])
def test_constant_values_give_constant_output(d_qk, d_v, causal):
    """V equal to a constant c_h in every row of KV head h: every row with a
    visible key gets O = c_h exactly in real arithmetic (its weights sum to
    one), whatever the scores.  On peaky rows (Q x 3) the GPU's O differs from
    c_h only by the bf16 rounding of P against the fp32 row sum (at most 2^-9
    relative) and of O itself (one bf16 step at 1.5 is 2^-7)."""
    B, N, Hq, Hkv = 2, 333, 4, 2
    q, k, _ = inputs.make_qkv(B, N, N, Hq, Hkv, d_qk, 9600 + d_qk + int(causal), q_mult=3.0)
    consts = torch.tensor([1.5, -0.375], dtype=torch.bfloat16)  # exact in bf16
    v = consts.view(1, 1, Hkv, 1).expand(B, N, Hkv, d_v).contiguous()
    scale = 1.0 / math.sqrt(d_qk)
    print(f"[parity] constant V d=({d_qk},{d_v}) causal={causal}", flush=True)
    o, lse = _run(q, k, v, scale, causal)
    want = consts.float().repeat_interleave(Hq // Hkv).view(1, 1, Hq, 1).double().numpy()
    err = np.abs(to_np64(o) - want)
    assert err.max() <= 2.0 ** -7 + 2.0 ** -9 * 1.5, err.max()
    _, lse_ref = oracle.attention_forward(to_np64(q), to_np64(k), to_np64(v), scale, causal,
                                          workers=8)
    assert np.abs(to_np64(lse) - lse_ref).max() <= 1e-3


def test_side_streams_and_concurrent_calls():
    """Calls on two non-default streams at once (each call runs on the stream
    current when it is made, shares no state with other calls and allocates
    nothing) give the default-stream results bit for bit, forward and
    backward."""
    cases = []
    for B, N, Hq, Hkv, d, causal, seed in ((2, 1000, 8, 2, 128, True, 9800),
                                           (3, 700, 4, 4, 64, False, 9801)):
        q, k, v = inputs.make_qkv(B, N, N, Hq, Hkv, d, seed, q_mult=2.0)
        do = inputs.make_dout(q.shape, seed + 1)
        cases.append(tuple(t.to(DEV) for t in (q, k, v, do)) + (causal,))

    def run(qd, kd, vd, dod, causal):
        o, lse = attn.attn_fwd(qd, kd, vd, 0.09, causal)
        return (o, lse) + tuple(attn.attn_bwd(qd, kd, vd, o, lse, dod, 0.09, causal))

    ref = [run(*c) for c in cases]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]  # default priority
    got = []
    for st, c in zip(streams, cases):
        with torch.cuda.stream(st):
            got.append(run(*c))
    torch.cuda.synchronize()
    print("[parity] two side streams", flush=True)
    for r, g in zip(ref, got):
        for x, y in zip(r, g):
            assert torch.equal(x, y)


def test_key_shift_moves_lse_by_the_query_dot_shift():
    """softmax(x) = softmax(x - c): adding w to every key moves LSE_i by scale*q_i.w."""
    B, N, H, d = 1, 300, 2, 64
    q, k, v = inputs.make_qkv(B, N, N, H, H, d, 8500)
    w = torch.zeros(d)
    w[::7] = 0.5
    k2 = (k.float() + w).to(torch.bfloat16)
    scale = 0.125
    o1, l1 = _run(q, k2, v, scale, False)
    o_ref, l_ref = oracle.attention_forward(to_np64(q), to_np64(k2), to_np64(v), scale, False)
    assert_parity(errors(to_np64(o1), to_np64(l1), o_ref, l_ref), "shifted keys")


# ------------------------------------------------------------------ any finite scale

@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("scale_mult", [-1.0, 0.0, -3.0])
@pytest.mark.parametrize("causal,padded", [(True, False), (False, True)])
def test_any_finite_scale_full_oracle(d, scale_mult, causal, padded):
    """Negative and zero scales (the boundary accepts every finite scale).

    |scale| up to 3/sqrt(d) on N(0, 1) queries: rows as peaky as the
    headline's (Q x 3 at 1/sqrt(d)), for which the tolerance is stated.
    """
    B, N, Hq, Hkv = 3, 333, 4, 2
    seed = 8900 + d + int(causal) + int(10 * abs(scale_mult))
    q, k, v = inputs.make_qkv(B, N, N, Hq, Hkv, d, seed)
    seqlens = None
    if padded:
        seqlens = inputs.make_seqlens(B, 0, N, seed + 1)
        seqlens[0] = 0  # rows with no visible key
    scale = scale_mult / math.sqrt(d)
    print(f"[parity] scale={scale:.4f} d={d} causal={causal} padded={padded}", flush=True)
    o, lse = _run(q, k, v, scale, causal, seqlens)
    o_ref, lse_ref = oracle.attention_forward(to_np64(q), to_np64(k), to_np64(v), scale, causal,
                                              None if seqlens is None else seqlens.numpy(),
                                              workers=8)
    assert_parity(errors(to_np64(o), to_np64(lse), o_ref, lse_ref), f"scale {scale}")


@pytest.mark.parametrize("d", [64, 128])
def test_negative_scale_is_the_positive_scale_on_negated_queries_bitwise(d):
    q, k, v = inputs.make_qkv(2, 400, 400, 8, 2, d, 8950 + d, q_mult=3.0)
    for causal in (False, True):
        o1, l1 = _run(q, k, v, -0.1, causal)
        o2, l2 = _run(-q, k, v, 0.1, causal)
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_any_finite_scale_other_entry_points():
    """Negative and zero scales through the packed, (192, 128) and block-sparse entry points."""
    lengths = torch.tensor([1, 130, 257, 0, 64], dtype=torch.int32)
    cu = inputs.cu_from_lengths(lengths)
    T, mx = int(cu[-1]), int(lengths.max())
    for scale in (-0.2, 0.0):
        q, k, v = inputs.make_packed_qkv(T, T, 4, 2, 128, 8960, q_mult=2.0)
        o, lse = attn.attn_fwd_varlen(q.to(DEV), k.to(DEV), v.to(DEV), cu.to(DEV), cu.to(DEV), mx,
                                      mx, scale, True)
        torch.cuda.synchronize()
        o_ref, lse_ref = oracle.attention_forward_varlen(to_np64(q), to_np64(k), to_np64(v),
                                                         cu.numpy(), cu.numpy(), scale, True)
        assert_parity(errors(to_np64(o), to_np64(lse), o_ref, lse_ref), f"varlen scale {scale}")

        q, k, v = inputs.make_qkv(2, 300, 300, 4, 2, 192, 8961, q_mult=2.0, d_v=128)
        o, lse = _run(q, k, v, scale, True)
        o_ref, lse_ref = oracle.attention_forward(to_np64(q), to_np64(k), to_np64(v), scale, True)
        assert_parity(errors(to_np64(o), to_np64(lse), o_ref, lse_ref), f"(192,128) scale {scale}")

        q, k, v = inputs.make_qkv(1, 517, 517, 4, 2, 128, 8962, q_mult=2.0)
        g = torch.Generator().manual_seed(8963)
        bm = (torch.rand((1, 5, 5), generator=g) < 0.5).to(torch.uint8)
        o, lse = attn.attn_fwd_blocksparse(q.to(DEV), k.to(DEV), v.to(DEV), bm.to(DEV), scale, False)
        torch.cuda.synchronize()
        o_ref, lse_ref = oracle.attention_forward_blocksparse(to_np64(q), to_np64(k), to_np64(v),
                                                              scale, bm.numpy(), 128, 128, False)
        assert_parity(errors(to_np64(o), to_np64(lse), o_ref, lse_ref), f"sparse scale {scale}")


# ------------------------------------------------------------------ scores that climb along the keys

# Score step 0.25 per key (23 log2 units per 64-key tile) and, at key 400, one
# key 100 above the trend (144 log2 units): rows of even query heads find a
# maximum more than tau = 8 log2 units above their running one in every key
# tile up to the jump, and exponentials taken against their stale maximum
# overflow to +inf there; rows of odd heads keep their first tile's maximum
# and the later tiles' exponentials underflow to 0.  LSE reaches ~200.
TREND = dict(step=0.25, jump_at=400, jump=100.0)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_climbing_scores_rescale_every_tile(d, causal, sign):
    """The conditional rescale at every key tile, and a stale maximum that overflows exp2."""
    B, N, Hq, Hkv = 2, 600, 4, 2
    scale = sign / math.sqrt(d)
    q, k, v = inputs.make_trend_qkv(B, N, Hq, Hkv, d, 9400 + d, scale, **TREND)
    print(f"[parity] climbing scores d={d} causal={causal} scale={scale:.4f}", flush=True)
    o, lse = _run(q, k, v, scale, causal)
    o_ref, lse_ref = oracle.attention_forward(to_np64(q), to_np64(k), to_np64(v), scale, causal,
                                              workers=8)
    assert_parity(errors(to_np64(o), to_np64(lse), o_ref, lse_ref), "climbing scores")


def test_climbing_scores_other_entry_points():
    """The same inputs through the (192, 128), block-sparse and packed entry points."""
    scale = 1.0 / math.sqrt(192)
    q, k, v = inputs.make_trend_qkv(2, 600, 4, 2, 192, 9410, scale, d_v=128, **TREND)
    print("[parity] climbing scores (192, 128)", flush=True)
    for causal in (False, True):
        o, lse = _run(q, k, v, scale, causal)
        o_ref, lse_ref = oracle.attention_forward(to_np64(q), to_np64(k), to_np64(v), scale,
                                                  causal, workers=8)
        assert_parity(errors(to_np64(o), to_np64(lse), o_ref, lse_ref), "(192,128) climbing")

    scale = 1.0 / math.sqrt(128)
    q, k, v = inputs.make_trend_qkv(1, 600, 4, 2, 128, 9411, scale, **TREND)
    g = torch.Generator().manual_seed(9412)
    bm = (torch.rand((1, 5, 5), generator=g) < 0.6).to(torch.uint8)
    bm[0, :, 3] = 1  # the block holding the jump
    print("[parity] climbing scores block-sparse", flush=True)
    o, lse = attn.attn_fwd_blocksparse(q.to(DEV), k.to(DEV), v.to(DEV), bm.to(DEV), scale, False)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_forward_blocksparse(to_np64(q), to_np64(k), to_np64(v), scale,
                                                          bm.numpy(), 128, 128, False)
    assert_parity(errors(to_np64(o), to_np64(lse), o_ref, lse_ref), "sparse climbing")

    # one packed sequence of 600 rows beside a short one
    q2, k2, v2 = inputs.make_trend_qkv(1, 130, 4, 2, 128, 9413, scale, step=0.25)
    qp, kp, vp = (torch.cat([a[0], b[0]]) for a, b in ((q, q2), (k, k2), (v, v2)))
    cu = inputs.cu_from_lengths([600, 130])
    print("[parity] climbing scores packed", flush=True)
    o, lse = attn.attn_fwd_varlen(qp.to(DEV), kp.to(DEV), vp.to(DEV), cu.to(DEV), cu.to(DEV), 600,
                                  600, scale, True)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_forward_varlen(to_np64(qp), to_np64(kp), to_np64(vp),
                                                     cu.numpy(), cu.numpy(), scale, True)
    assert_parity(errors(to_np64(o), to_np64(lse), o_ref, lse_ref), "packed climbing")


# ------------------------------------------------------------------ key rows past 2 GiB

@pytest.mark.parametrize("d,padded", [(128, False), (64, True)])
def test_key_rows_past_2gib(d, padded):
    """K and V of 2^18 + 77 rows of 8 KiB (4096 / d KV heads): rows past 2 GiB
    into each array, so every key address needs more than 31 bits.  Short
    query blocks see every key (non-causal); the first and the last head are
    compared with the oracle on every row."""
    B, Nq, Nk = 1, 100, (1 << 18) + 77
    H = 8192 // (2 * d)
    q, k, v = inputs.make_qkv_on(DEV, B, Nq, Nk, H, H, d, 9500 + d)
    assert k[0, -1].data_ptr() - k.data_ptr() > 2 ** 31
    seqlens = torch.tensor([Nk - 5], dtype=torch.int32) if padded else None
    scale = 1.0 / math.sqrt(d)
    print(f"[parity] key rows past 2 GiB d={d} H={H} Nk={Nk} padded={padded}", flush=True)
    o, lse = _run(q, k, v, scale, False, seqlens)
    nk = Nk - 5 if padded else Nk
    for h in (0, H - 1):
        o_ref, lse_ref = oracle.attention_forward(
            to_np64(q[:, :, h:h + 1]), to_np64(k[:, :nk, h:h + 1]), to_np64(v[:, :nk, h:h + 1]),
            scale, False)
        assert_parity(errors(to_np64(o[:, :, h:h + 1]), to_np64(lse[:, h:h + 1]), o_ref, lse_ref),
                      f"head {h}")
    del q, k, v, o, lse
    torch.cuda.empty_cache()


# ------------------------------------------------------------------ full-size workloads

FULL = [name for name in inputs.WORKLOADS if name != "single_head_n256_d64"]


def _oracle_workers():
    """Host threads for the oracle: the process's CPU share, at most 16."""
    from oracle.attention import default_workers

    return max(1, min(16, default_workers()))


def _launch_workload(w, x, out, lse):
    """The workload's forward exactly as the benchmark's step launches it, into out / lse."""
    qd, kd, vd = x["q"].to(DEV), x["k"].to(DEV), x["v"].to(DEV)
    if w.varlen:
        cu = x["cu_seqlens_q"].to(DEV)
        ms = x["max_seqlen"]
        plan = attn.attn_varlen_plan(cu, cu, ms, ms, w.causal)  # longest-first order
        attn.attn_fwd_varlen(qd, kd, vd, cu, cu, ms, ms, w.scale, w.causal, out=out, lse=lse,
                             seq_order=plan)
    elif w.sparse:
        attn.attn_fwd_blocksparse(qd, kd, vd, x["block_mask"].to(DEV), w.scale, w.causal, out=out,
                                  lse=lse)
    else:
        sl = None if x["seqlens_k"] is None else x["seqlens_k"].to(DEV)
        attn.attn_fwd(qd, kd, vd, w.scale, w.causal, sl, out=out, lse=lse)
    torch.cuda.synchronize()


def _nan_outputs(w, x):
    q = x["q"]
    out = torch.full(q.shape[:-1] + (w.d_v,), float("nan"), dtype=torch.bfloat16, device=DEV)
    if w.varlen:
        lse = torch.full((w.Hq, q.shape[0]), float("nan"), dtype=torch.float32, device=DEV)
    else:
        lse = torch.full((w.B, w.Hq, w.N), float("nan"), dtype=torch.float32, device=DEV)
    return out, lse


@pytest.mark.parametrize("name", FULL)
def test_full_workload_whole_output(name):
    """Every element of a full-size workload against the oracle.

    The outputs start as NaN, so a row block that no workgroup writes (a
    mis-decoded grid item, the second item of a pair, a padding item) fails.
    The launch is the benchmark's; a second launch must be bitwise identical.
    """
    w = inputs.WORKLOADS[name]
    print(f"[parity] full workload {name}: launching", flush=True)
    x = inputs.workload_inputs(w)
    o, lse = _nan_outputs(w, x)
    _launch_workload(w, x, o, lse)
    assert not torch.isnan(o).any(), "output elements left unwritten"
    assert not torch.isnan(lse).any(), "LSE entries left unwritten"
    o2, lse2 = _nan_outputs(w, x)
    _launch_workload(w, x, o2, lse2)
    assert torch.equal(o, o2) and torch.equal(lse, lse2), "reruns differ"
    del o2, lse2
    torch.cuda.empty_cache()
    q32, k32, v32 = (x[n].float().numpy() for n in ("q", "k", "v"))
    o_np = o.float().cpu().numpy().astype(np.float64)
    lse_np = lse.cpu().numpy().astype(np.float64)
    del o, lse
    workers = _oracle_workers()
    print(f"[parity] full workload {name}: oracle on {workers} threads", flush=True)
    if w.varlen:
        cu = x["cu_seqlens_q"].numpy()
        o_ref, lse_ref = oracle.attention_forward_varlen(q32, k32, v32, cu, cu, w.scale, w.causal,
                                                         workers=workers)
    elif w.sparse:
        o_ref, lse_ref = oracle.attention_forward_blocksparse(
            q32, k32, v32, w.scale, x["block_mask"].numpy(), inputs.SPARSE_BLOCK,
            inputs.SPARSE_BLOCK, w.causal, workers=workers)
    else:
        sl = None if x["seqlens_k"] is None else x["seqlens_k"].numpy()
        o_ref, lse_ref = oracle.attention_forward(q32, k32, v32, w.scale, w.causal, sl,
                                                  workers=workers)
    errs = errors(o_np, lse_np, o_ref, lse_ref)
    errs["elements"] = int(o_np.size)
    print(f"[parity] {name}: {errs}", flush=True)
    assert_parity(errs, name)
    if not w.varlen and not w.sparse:
        # The GPU's own LSE normalises its rows: sum_j exp(s_ij - LSE_i) = 1.
        G = w.Hq // w.Hkv
        sl = None if x["seqlens_k"] is None else x["seqlens_k"].numpy()
        rng = np.random.default_rng(w.seed)
        for b, h, i in sample_rows(rng, w.B, w.Hq, w.N, 16):
            nk = w.N if sl is None else int(sl[b])
            hi = min(nk, i + 1) if w.causal else nk
            s = w.scale * (k32[b, :hi, h // G].astype(np.float64) @ q32[b, i, h].astype(np.float64))
            assert abs(np.exp(s - lse_np[b, h, i]).sum() - 1.0) <= 1e-3
