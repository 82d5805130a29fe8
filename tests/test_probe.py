"""GPU: the matrix-core rate probe (attn_probe_mfma) does all the work it counts.

With every operand element 1.0, each 32x32x16 MFMA adds 16 to every
accumulator element; a wave runs 2 MFMAs per accumulator per loop iteration,
so each of its 8 x 16 accumulator registers ends at 32 * iters and every lane's
sink value is 8 * 16 * 32 * iters, exactly representable in fp32 here.  The
16x16x32 shape adds 32 per MFMA into 16 x 4 registers, 2 MFMAs each per
iteration: the same 4096 * iters.  Zero operands give zero.  The clocks record positive tick counts whose ratio is a
plausible shader clock.
"""

import pytest
import torch

from exact_attention_18_amd import attn

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.mark.parametrize("shape", [32, 16])
@pytest.mark.parametrize("value", [1.0, 0.0])
def test_probe_does_every_mfma_it_counts(value, shape):
    iters, wg = 64, torch.cuda.get_device_properties(0).multi_processor_count
    ops = torch.full((8, 64, 8), value, dtype=torch.bfloat16, device=DEV)
    sink, clocks = attn.attn_probe_mfma(ops, iters, wg, shape=shape)
    torch.cuda.synchronize()
    expect = 4096 * iters * value
    assert sink.numel() == wg * 512
    assert torch.equal(sink.cpu(), torch.full((wg * 512,), expect, dtype=torch.float32))
    c = clocks.cpu().to(torch.float64)
    assert (c > 0).all()
    ghz = c[:, 0] / c[:, 1] * 0.1
    assert ((ghz > 0.3) & (ghz < 3.0)).all(), (ghz.min().item(), ghz.max().item())


def test_workgroups_are_dealt_round_robin_to_the_xcds():
    """The forward's grid order assumes workgroup w runs on XCD w % (number of XCDs).

    The probe records the XCD of every workgroup of a grid several times the
    CU count.  In single-partition mode all 8 XCDs appear and the mapping is
    w % 8; a device partitioned to one XCD shows only XCD ids of one value.
    """
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    n = 4 * cus + 5
    ids = attn.attn_probe_xcd(n).cpu()
    xcc = ids[:, 0]
    seen = sorted(set(xcc.tolist()))
    print(f"[probe] {n} workgroups, XCDs seen {seen}, CUs {cus}", flush=True)
    assert ((xcc >= 0) & (xcc < 8)).all()
    if len(seen) > 1:
        assert len(seen) == 8
        assert torch.equal(xcc, torch.arange(n, dtype=torch.int32) % 8)


@pytest.mark.parametrize("kind", [1, 2, 3])
def test_softmax_issue_probe_computes_exp2_and_counts(kind):
    """The probe's exponentials are exp2 (v_exp_f32, or the polynomial within its
    8.6e-5 minimax bound plus fp32 rounding), and every wave reports work and ticks."""
    import numpy as np
    wg = torch.cuda.get_device_properties(0).multi_processor_count
    ops = torch.full((8, 64, 8), 1.0, dtype=torch.bfloat16, device=DEV)
    values, stats = attn.attn_probe_softmax_issue(ops, True, kind, 200, wg)
    torch.cuda.synchronize()
    x = ((np.arange(64)[:, None] + 64 * np.arange(32)[None, :]) / 256.0 - 8.0).astype(np.float32)
    ref = np.exp2(x.astype(np.float64))
    rel = np.abs(values.cpu().numpy().astype(np.float64) - ref) / ref
    poly = np.zeros((64, 32), dtype=bool)
    if kind == 2:
        poly[:] = True
    elif kind == 3:
        poly[:, (np.arange(32) % 8) < 2] = True
    assert rel[~poly].max(initial=0.0) <= 2e-6
    assert rel[poly].max(initial=0.0) <= 1e-4
    st = stats.cpu()
    assert (st[:, 0] > 0).all() and (st[:, 1] > 0).all() and (st[:, 2] > 0).all()
