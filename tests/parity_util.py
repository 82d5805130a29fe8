"""Shared helpers of the GPU parity tests: conversions, error metrics, tolerances.

Tolerances for bf16 inputs with fp32 accumulation, against the fp64 oracle on
the same bf16 tensors: max |O - O_ref| <= 2e-2, mean |O - O_ref| <= 2e-3,
max |LSE - LSE_ref| <= 1e-3.  Error budget: rounding O to bf16 alone costs up
to 2^-9 |O| (|O| reaches about 4.5 on the peaky Q x3 rows, i.e. ~9e-3), and
rounding P to bf16 before the P V contraction adds a random-sign term of the
same order per element; the LSE error is dominated by fp32 exp2/log2 (~1e-6
relative), far inside 1e-3.
"""

import numpy as np
import torch

O_MAX_ABS = 2e-2
O_MEAN_ABS = 2e-3
LSE_MAX_ABS = 1e-3


def to_np64(t: torch.Tensor) -> np.ndarray:
    """Exact upcast of a (bf16/fp32) tensor to a float64 numpy array."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def lse_error(lse_gpu, lse_ref):
    """Max |difference|, counting matching -inf entries as exact."""
    lse_gpu = np.asarray(lse_gpu, dtype=np.float64)
    lse_ref = np.asarray(lse_ref, dtype=np.float64)
    both_inf = np.isneginf(lse_gpu) & np.isneginf(lse_ref)
    if (np.isneginf(lse_gpu) != np.isneginf(lse_ref)).any():
        return float("inf")
    d = np.abs(np.where(both_inf, 0.0, lse_gpu - np.where(both_inf, 0.0, lse_ref)))
    return float(d.max()) if d.size else 0.0


def errors(o_gpu, lse_gpu, o_ref, lse_ref):
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    o_ref = np.asarray(o_ref, dtype=np.float64)
    e = np.abs(o_gpu - o_ref)
    return dict(o_max=float(e.max()) if e.size else 0.0,
                o_mean=float(e.mean()) if e.size else 0.0,
                lse_max=lse_error(lse_gpu, lse_ref))


def assert_parity(errs, what=""):
    assert np.isfinite(errs["o_max"]), f"{what}: non-finite output {errs}"
    assert errs["o_max"] <= O_MAX_ABS, f"{what}: {errs}"
    assert errs["o_mean"] <= O_MEAN_ABS, f"{what}: {errs}"
    assert errs["lse_max"] <= LSE_MAX_ABS, f"{what}: {errs}"


def sample_rows(rng, B, H, N, n, block=128):
    """(b, h, i) samples: first/last rows, block edges, and random rows."""
    special = [0, 1, N - 1, N - 2] + [x for m in range(block, N, block * 7) for x in (m - 1, m)]
    special = [i for i in special if 0 <= i < N]
    out = []
    for t in range(n):
        b = int(rng.integers(B))
        h = int(rng.integers(H))
        i = special[t] if t < len(special) else int(rng.integers(N))
        out.append((b, h, i))
    return out


# Backward tolerance, derived from the arithmetic (no value is stated for the
# backward): every product in a gradient has one operand rounded to bf16 (P or
# dS, relative error <= 2^-9) and every gradient is rounded to bf16 on output
# (<= 2^-9 relative), so the expected relative Frobenius error is about
# sqrt(2) * 2^-9 = 2.8e-3; the bars below leave a factor ~3.5 (Frobenius) and
# one bf16 ulp at the largest magnitude plus accumulation (max abs).
GRAD_REL_FRO = 1e-2
GRAD_MAX_REL = 2e-2


def grad_errors(got, ref, floor=0.0):
    """Relative Frobenius and max errors of a gradient.

    floor bounds the reference scale from below: a gradient that vanishes in
    exact arithmetic (a softmax over one key is constant, so dQ and dK are 0)
    is the difference of two roundings of terms of that size, and is measured
    against them instead of against its own near-zero reference.
    """
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    scale = max(np.abs(ref).max(), floor, 1e-30)
    norm = max(np.linalg.norm(ref), floor * np.sqrt(ref.size), 1e-30)
    return {"rel_fro": float(np.linalg.norm(got - ref) / norm),
            "max_rel": float(np.abs(got - ref).max() / scale)}


def assert_grad_parity(errs, what):
    assert errs["rel_fro"] <= GRAD_REL_FRO, f"{what}: {errs}"
    assert errs["max_rel"] <= GRAD_MAX_REL, f"{what}: {errs}"
