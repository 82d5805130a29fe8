"""GPU parity of the software-exp2 build (libattn_exp2poly.so) against the oracle.

The build evaluates 8 of every 32 exponentials of the d = 128 softmax as a
degree-3 polynomial on the FMA pipe instead of v_exp_f32 (the partial
exponential emulation of FlashAttention-4 (papercache summary), section
3.1.3).  Its relative error (8.6e-5) is far below the bf16 rounding of P, so
it must meet the same tolerance as the default build, on small shapes with
masks, key padding and empty rows and on the headline workload in full; a
masked score must still contribute exactly nothing.
"""

import math
import os

import numpy as np
import pytest
import torch

import oracle
from exact_attention_18_amd import attn, inputs
from parity_util import assert_parity, errors, to_np64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def poly_lib():
    if not os.path.exists(attn.EXP2POLY_LIB_PATH):
        pytest.fail("libattn_exp2poly.so is not built (build() compiles it)")
    return attn.EXP2POLY_LIB_PATH


@pytest.mark.parametrize("B,N,Hq,Hkv,causal,padded", [
    (2, 333, 8, 2, True, False),
    (3, 300, 4, 4, False, True),
    (1, 517, 4, 1, True, True),
])
def test_exp2_poly_build_small_shapes(poly_lib, B, N, Hq, Hkv, causal, padded):
    q, k, v = inputs.make_qkv(B, N, N, Hq, Hkv, 128, 9900 + N, q_mult=3.0)
    sl = None
    if padded:
        sl = inputs.make_seqlens(B, 0, N, 9901)
        sl[0] = 0  # rows with no visible key
    with attn.using_library(poly_lib):
        o, lse = attn.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), 1 / math.sqrt(128), causal,
                               None if sl is None else sl.to(DEV))
        torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_forward(to_np64(q), to_np64(k), to_np64(v), 1 / math.sqrt(128),
                                              causal, None if sl is None else sl.numpy(), workers=8)
    assert_parity(errors(to_np64(o), to_np64(lse), o_ref, lse_ref), "exp2 poly")
    if padded:
        assert (o[0] == 0).all() and torch.isneginf(lse[0]).all()


def test_exp2_poly_build_headline_whole_output(poly_lib):
    w = inputs.WORKLOADS[inputs.HEADLINE]
    x = inputs.workload_inputs(w)
    print(f"[parity] exp2 poly build, {w.name}", flush=True)
    with attn.using_library(poly_lib):
        o, lse = attn.attn_fwd(x["q"].to(DEV), x["k"].to(DEV), x["v"].to(DEV), w.scale, w.causal)
        torch.cuda.synchronize()
    o_np = o.float().cpu().numpy().astype(np.float64)
    lse_np = lse.cpu().numpy().astype(np.float64)
    del o, lse
    from oracle.attention import default_workers
    o_ref, lse_ref = oracle.attention_forward(x["q"].float().numpy(), x["k"].float().numpy(),
                                              x["v"].float().numpy(), w.scale, w.causal,
                                              workers=max(1, min(16, default_workers())))
    errs = errors(o_np, lse_np, o_ref, lse_ref)
    print(f"[parity] exp2 poly build {w.name}: {errs}", flush=True)
    assert_parity(errs, "exp2 poly headline")
