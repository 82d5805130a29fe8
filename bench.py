#!/usr/bin/env python3
"""Benchmark of the fused exact-attention forward on one MI355X.

One step = one launch of the whole forward (attn_fwd: scores, online softmax,
output contraction, epilogue) over the workload's seeded synthetic inputs,
already resident in HBM.  W warm-up steps, then K timed steps on torch's
current stream, bracketed by torch.cuda.synchronize().  Prints ONE JSON line.

value       : algorithmic TFLOP/s of the step, FLOPs counted as the pages count
              them: 4 * Nq * Nk * d per head (2 * Nq * Nk * (d_qk + d_v) when the
              score and value head dimensions differ), halved under the causal mask
              (FlashAttention-4 (papercache summary), experimental setup).
roofline    : the forward kernel against the dense bf16 MFMA peak of MI355X
              (2516.6 TFLOP/s = 256 CUs x 2.4 GHz x 4096 FLOP/clk/CU); its
              duration is the mean of per-launch HIP events recorded on the
              launch stream inside the timed region.
mfma_sustained: what the matrix cores sustain on this device with one MFMA
              shape and nothing else (attn_probe_mfma), for random and for
              zero operands, with the shader clock each ran at; the chip lowers
              its clock under matrix-core load, so the published peak is not
              reachable with random data.  The top level holds 32x32x16,
              shape_16x16x32 the 16x16x32 MFMA (a higher clock);
              forward_frac_of_random relates the forward to the random-operand
              rate of the shape it runs on (forward_mfma_shape).
cpu_baseline: the CPU oracle as it stands, timed on this host on a bounded
              sample of heads of the same workload (heads are independent and
              equal in cost, so the rate is the workload's rate).
parity_sample: the heads that sample computed, compared element by element
              with the timed launches' own O and LSE: max and mean |O - O_oracle|
              and max |LSE - LSE_oracle| (the parity tests' bars are 2e-2, 2e-3
              and 1e-3).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np
import torch

from exact_attention_18_amd import attn, inputs

PEAK_BF16_TFLOPS = 2516.6
METRIC = "attn fwd TFLOP/s bf16 hd128 causal N=8192 + % of MFMA bf16 peak"
ROOT = os.path.dirname(os.path.abspath(__file__))
# Sources the forward kernels are built from (their hash keys the committed traffic figure).
KERNEL_SRCS = [os.path.join(ROOT, "exact_attention_18_amd", "csrc", n) for n in ("attn_fwd.hip", "cdna4.h")]


def _code_tokens(text: str) -> str:
    """C++ source with comments removed and whitespace runs collapsed to one space."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":  # string or character literal, copied whole
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_sha256() -> str:
    """sha256 of the forward's code (attn_fwd.hip, then cdna4.h), comments and layout ignored."""
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        h.update(_code_tokens(open(path, encoding="utf-8").read()).encode())
        h.update(b"\0")
    return h.hexdigest()


def measured_traffic(workload: str, profiles_dir: str = os.path.join(ROOT, "profiles")):
    """HBM bytes per launch from the committed rocprofv3 summary of this workload.

    The summary records FETCH_SIZE / WRITE_SIZE of the forward scaled by a
    plain-copy calibration, and the sha256 of the forward's code (attn_fwd.hip,
    then cdna4.h, comments and whitespace ignored) it was taken on; a summary
    of other code gives None.
    """
    path = os.path.join(profiles_dir, f"attn_fwd_{workload}.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith(("|", "-", "#", "`")):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    sha = kernel_source_sha256()
    if fields.get("kernel_source_sha256") != sha or "traffic_bytes_per_launch" not in fields:
        return None
    return float(fields["traffic_bytes_per_launch"])


def algorithmic_flops(w: inputs.Workload, x) -> float:
    if w.varlen:
        lens = x["lengths"].to(torch.float64)
        per = (2.0 * lens * lens * (w.d + w.d_v)).sum().item()
        f = per * w.Hq
    elif w.sparse:  # the (row, key) pairs inside nonzero blocks, within N x N
        bm = x["block_mask"][0].to(torch.float64)
        sizes = torch.full((bm.shape[0],), float(inputs.SPARSE_BLOCK), dtype=torch.float64)
        sizes[-1] = w.N - inputs.SPARSE_BLOCK * (bm.shape[0] - 1)
        pairs = (sizes[:, None] * bm * sizes[None, :]).sum().item()
        f = 2.0 * pairs * (w.d + w.d_v) * w.B * w.Hq
    else:
        nk = (torch.full((w.B,), float(w.N), dtype=torch.float64) if x["seqlens_k"] is None
              else x["seqlens_k"].to(torch.float64))
        f = (2.0 * w.N * nk * (w.d + w.d_v)).sum().item() * w.Hq
    return f / 2.0 if w.causal else f


def make_step(w, x, dev):
    q, k, v = x["q"].to(dev), x["k"].to(dev), x["v"].to(dev)
    out = torch.empty(q.shape[:-1] + (w.d_v,), dtype=torch.bfloat16, device=dev)
    if w.varlen:
        cu = x["cu_seqlens_q"].to(dev)
        ms = x["max_seqlen"]
        lse = torch.empty((w.Hq, q.shape[0]), dtype=torch.float32, device=dev)

        plan = torch.empty((cu.numel() - 1,), dtype=torch.int32, device=dev)

        def step():  # LPT plan (FlashAttention-4 summary, section 3.3), then the forward
            attn.attn_varlen_plan(cu, cu, ms, ms, w.causal, out=plan)
            attn.attn_fwd_varlen(q, k, v, cu, cu, ms, ms, w.scale, w.causal, out=out, lse=lse,
                                 seq_order=plan)
            return out, lse
    elif w.sparse:
        bm = x["block_mask"].to(dev)
        lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device=dev)

        def step():
            attn.attn_fwd_blocksparse(q, k, v, bm, w.scale, w.causal, out=out, lse=lse)
            return out, lse
    else:
        sl = None if x["seqlens_k"] is None else x["seqlens_k"].to(dev)
        lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device=dev)

        def step():
            attn.attn_fwd(q, k, v, w.scale, w.causal, sl, out=out, lse=lse)
            return out, lse
    return step


def cpu_baseline(w, x, target_s: float, got=None):
    """Time the oracle on whole heads until about target_s seconds have passed.

    A head is a (batch, query head) pair, or a (sequence, query head) pair of a
    packed batch; each is the oracle's plain fp64 computation of that head
    (attention_head, with the block mask's element pattern for the
    block-sparse workload).  Heads are visited in a seeded random order and
    run `workers` at a time; the rate is the visited heads' algorithmic FLOPs
    over the wall time.

    got: the GPU's (O, LSE) of the workload as float NumPy arrays, or None.
    Each visited head's oracle result is then compared with its slice of
    them; returns (baseline, parity) with parity None when got is None.
    """
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    from oracle.attention import default_workers

    workers = default_workers()
    q = x["q"].float().numpy()
    k = x["k"].float().numpy()
    v = x["v"].float().numpy()
    G = w.Hq // w.Hkv
    rng = np.random.default_rng(w.seed)

    def diff(o_ref, l_ref, o_got, l_got):
        """max and sum of |O - O_ref|, element count, max |LSE - LSE_ref| of one head."""
        if got is None:
            return None
        e = np.abs(o_got - o_ref)
        both_inf = np.isneginf(l_got) & np.isneginf(l_ref)
        de = np.where(both_inf, 0.0, np.abs(l_got - np.where(both_inf, 0.0, l_ref)))
        return (float(e.max()) if e.size else 0.0, float(e.sum()), e.size,
                float(de.max()) if de.size else 0.0)

    if w.varlen:
        cu = x["cu_seqlens_q"].numpy()
        heads = [(z, h) for z in range(len(cu) - 1) for h in range(w.Hq)]

        def one(zh):
            z, h = zh
            a, e = int(cu[z]), int(cu[z + 1])
            o_ref, l_ref = oracle.attention_head(q[a:e, h], k[a:e, h // G], v[a:e, h // G],
                                                 w.scale, w.causal)
            L = e - a
            f = 2.0 * L * L * (w.d + w.d_v)
            cmp = None if got is None else diff(o_ref, l_ref, got[0][a:e, h], got[1][h, a:e])
            return (f / 2.0 if w.causal else f), cmp
    else:
        sl = None if x.get("seqlens_k") is None else x["seqlens_k"].numpy()
        allowed = None
        if w.sparse:
            allowed = oracle.block_mask_to_elements(x["block_mask"][0].numpy(), w.N, w.N,
                                                    inputs.SPARSE_BLOCK, inputs.SPARSE_BLOCK)
        heads = [(b, h) for b in range(w.B) for h in range(w.Hq)]
        per_head = algorithmic_flops(w, x) / (w.B * w.Hq)

        def one(bh):
            b, h = bh
            nk = None if sl is None else int(sl[b])
            o_ref, l_ref = oracle.attention_head(q[b, :, h], k[b, :, h // G], v[b, :, h // G],
                                                 w.scale, w.causal, nk, allowed=allowed)
            cmp = None if got is None else diff(o_ref, l_ref, got[0][b, :, h], got[1][b, h])
            return per_head, cmp
    rng.shuffle(heads)
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover - threadpoolctl is present in this image
        threadpool_limits = None
    done, flop, t_total, pos = 0, 0.0, 0.0, 0
    cmps = []
    with ThreadPoolExecutor(max_workers=workers) as ex:
        while pos < len(heads) and t_total < target_s:
            chunk = heads[pos:pos + workers]
            t0 = time.perf_counter()
            if threadpool_limits is not None:
                with threadpool_limits(limits=1):
                    res = list(ex.map(one, chunk))
            else:
                res = list(ex.map(one, chunk))
            t_total += time.perf_counter() - t0
            flop += sum(r[0] for r in res)
            cmps += [r[1] for r in res if r[1] is not None]
            done += len(chunk)
            pos += len(chunk)
    kind = "(sequence, head)" if w.varlen else "(batch, head)"
    base = {"value": flop / t_total / 1e12, "unit": "TFLOP/s", "cores": workers, "kind": "oracle",
            "sample": f"{done} of {len(heads)} {kind} pairs of {w.name}, fp64 NumPy with S and P "
                      f"materialised, {workers} threads, {t_total:.1f} s wall"}
    parity = None
    if got is not None:
        n = sum(c[2] for c in cmps)
        parity = {"heads": len(cmps), "o_max_abs": max((c[0] for c in cmps), default=0.0),
                  "o_mean_abs": sum(c[1] for c in cmps) / n if n else 0.0,
                  "lse_max_abs": max((c[3] for c in cmps), default=0.0)}
    return base, parity


def mfma_sustained(dev, iters: int = 8192, reps: int = 3, seed: int = 7):
    """Sustained bf16 matrix-core rate of this device, with and without operand bits.

    attn_probe_mfma streams one MFMA shape over a full grid laid out as the
    forward's (one 8-wave workgroup per CU) with no other work: 32x32x16 (the
    "random" and "zeros" entries; the d = 64 and (192, 128) kernels) and
    16x16x32 (the "shape_16x16x32" entry; the d = 128 kernel).  Random operands (uniform in [-1, 1), as
    bf16) give the rate the forward's data allows; zeros give the power-light
    bound.  The shader clock is the mean over waves of s_memtime ticks /
    s_memrealtime ticks x 100 MHz.
    """
    wg = torch.cuda.get_device_properties(dev).multi_processor_count
    g = torch.Generator().manual_seed(seed)
    cases = (("random", torch.rand((8, 64, 8), generator=g) * 2 - 1),
             ("zeros", torch.zeros((8, 64, 8))))
    flop = attn.probe_flop(iters, wg)

    def measure(shape):
        res = {}
        for name, ops in cases:
            ops = ops.to(torch.bfloat16).to(dev)
            sink, clocks = attn.attn_probe_mfma(ops, iters, wg, shape=shape)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                attn.attn_probe_mfma(ops, iters, wg, sink=sink, clocks=clocks, shape=shape)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            c = clocks.cpu().to(torch.float64)
            ghz = float((c[:, 0] / c[:, 1]).mean()) * 0.1
            res[name] = {"tflops": round(flop / (ms * 1e-3) / 1e12, 1),
                         "shader_clock_ghz": round(ghz, 3), "ms": round(ms, 4)}
        return res

    out = measure(32)
    out["shape_16x16x32"] = measure(16)
    out["workgroups"] = wg
    out["iters"] = iters
    return out


def softmax_issue(dev, budget_us: int = 20000, seed: int = 7):
    """Issue cost of the softmax's exponential beside the matrix core (attn_probe_softmax_issue).

    For each (MFMA wave on/off, exponential kind) the probe runs a full grid,
    one 8-wave workgroup per CU, for budget_us of real time.  Reported per
    case, as means over the waves of all CUs: shader cycles per MFMA of the
    MFMA waves, shader cycles per softmax element of the softmax waves (one
    element = one score's FMA, exp2, running-sum add, half a v_max3 and half
    a bf16 pack, as in the forward), and the shader clock.
    """
    wg = torch.cuda.get_device_properties(dev).multi_processor_count
    g = torch.Generator().manual_seed(seed)
    ops = (torch.rand((8, 64, 8), generator=g) * 2 - 1).to(torch.bfloat16).to(dev)
    kinds = {0: "none", 1: "v_exp_f32", 2: "polynomial", 3: "polynomial_on_8_of_32"}
    out = {"budget_us": budget_us, "workgroups": wg}
    for mfma_on in (1, 0):
        for kind in (0, 1, 2, 3):
            if not mfma_on and kind == 0:
                continue
            _, st = attn.attn_probe_softmax_issue(ops, bool(mfma_on), kind, budget_us, wg)
            torch.cuda.synchronize()
            st = st.cpu().to(torch.float64).view(wg, 8, 4)
            case = {}
            if mfma_on:
                m = st[:, :4]
                case["mfma_cycles_per_mfma"] = round(float((m[..., 1] / (m[..., 0] * 16)).mean()), 2)
                case["clock_ghz"] = round(float((m[..., 1] / m[..., 2]).mean()) * 0.1, 3)
            if kind:
                v = st[:, 4:]
                case["softmax_cycles_per_element"] = round(float((v[..., 1] / (v[..., 0] * 32)).mean()), 3)
                case.setdefault("clock_ghz", round(float((v[..., 1] / v[..., 2]).mean()) * 0.1, 3))
            out[("mfma+" if mfma_on else "") + kinds[kind]] = case
    return out


def compare_builds(w, x, dev, libs, steps: int, rounds: int, which: str = "fwd"):
    """TFLOP/s of the workload's step under each library build, in interleaved rounds in one process.

    Each round times `steps` steps under every build in turn (after 3 untimed
    steps), so clock and temperature drift affect every build alike.  Returns
    per build the mean, min and max over the rounds, the change of the mean
    against the first build, and whether its outputs equal the first build's
    bit for bit.  which = "bwd" times the backward (FLOPs 2.5x the forward's).
    """
    flops = algorithmic_flops(w, x) * (2.5 if which == "bwd" else 1.0)
    res = {lib: [] for lib in libs}
    outs = {}
    for rnd in range(rounds):
        for lib in libs:
            with attn.using_library(os.path.abspath(lib)):
                step = make_bwd_step(w, x, dev) if which == "bwd" else make_step(w, x, dev)
                if rnd == 0:
                    outs[lib] = [t.clone() for t in step()]
                for _ in range(3):
                    step()
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(steps):
                    step()
                e1.record()
                torch.cuda.synchronize()
                res[lib].append(flops / (e0.elapsed_time(e1) / steps * 1e-3) / 1e12)
        print(f"[bench] compare round {rnd}: " +
              " ".join(f"{os.path.basename(l)}={res[l][-1]:.1f}" for l in libs), file=sys.stderr,
              flush=True)
    base = float(np.mean(res[libs[0]]))
    return {os.path.basename(l): {"tflops_mean": round(float(np.mean(r)), 1),
                                  "min": round(float(np.min(r)), 1),
                                  "max": round(float(np.max(r)), 1),
                                  "vs_first_pct": round((float(np.mean(r)) / base - 1) * 100, 2),
                                  "bitwise_equal_first": all(
                                      torch.equal(a, b) for a, b in zip(outs[l], outs[libs[0]]))}
            for l, r in res.items()}


def warm_up(step, n):
    """Runs n untimed warm-up steps; returns the first one's time in ms (cold caches), or None."""
    if n <= 0:
        return None
    f_s, f_e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    f_s.record()
    step()
    f_e.record()
    for _ in range(n - 1):
        step()
    torch.cuda.synchronize()
    return round(f_s.elapsed_time(f_e), 5)


def bench_backward(args, w, x, dev, fwd_flops):
    """Times attn_bwd on the workload (FLOPs: 2.5x the forward, as the pages count them)."""
    if w.sparse or w.d not in (64, 128) or w.d_v != w.d:
        print("the backward covers the dense workloads with d = 64 or 128", file=sys.stderr)
        sys.exit(2)
    step = make_bwd_step(w, x, dev)
    first_ms = warm_up(step, args.warmup)
    K = args.steps
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(K):
        step()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / K
    flops = 2.5 * fwd_flops
    value = flops / (ms * 1e-3) / 1e12
    # MFMA work actually issued: 5 contractions in the dK/dV kernel's four plus the
    # dQ kernel's three (S and dP are formed in both), i.e. 3.5x the forward's two.
    issued = 3.5 * fwd_flops / (ms * 1e-3) / 1e12
    line = {
        "metric": f"attn bwd TFLOP/s bf16 hd{w.d} (2.5x forward FLOPs)",
        "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "first_run_ms": first_ms,
        "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded i.i.d. N(0,1) bf16; dO seeded likewise)",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "N": w.N, "d": w.d,
                   "causal": w.causal, "algorithmic_flop": flops, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(value, 3), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(value / PEAK_BF16_TFLOPS, 4),
                     "traffic": None, "mfma_issued_tflops": round(issued, 3)},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def make_bwd_step(w, x, dev):
    """One backward call (attn_bwd, or the LPT plan and attn_bwd_varlen) on the workload.

    The forward's O and LSE are computed once here; the step returns the
    (dq, dk, dv) output tensors it writes.
    """
    q, k, v = x["q"].to(dev), x["k"].to(dev), x["v"].to(dev)
    do = inputs.make_dout(x["q"].shape, w.seed + 77).to(dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    lib = attn.load_library()
    if w.varlen:
        # packed: the LPT plan and the backward, as the forward's step runs plan + forward
        cq, ck, mx = x["cu_seqlens_q"].to(dev), x["cu_seqlens_k"].to(dev), x["max_seqlen"]
        order = torch.empty((cq.numel() - 1,), dtype=torch.int32, device=dev)
        attn.attn_varlen_plan(cq, ck, mx, mx, w.causal, out=order)
        o, lse = attn.attn_fwd_varlen(q, k, v, cq, ck, mx, mx, w.scale, w.causal, seq_order=order)
        ws = torch.empty((lib.attn_bwd_workspace_size(1, w.Hq, q.shape[0]),), dtype=torch.uint8,
                         device=dev)

        def step():
            attn.attn_varlen_plan(cq, ck, mx, mx, w.causal, out=order)
            attn.attn_bwd_varlen(q, k, v, o, lse, do, cq, ck, mx, mx, w.scale, w.causal,
                                 seq_order=order, workspace=ws, out=(dq, dk, dv))
            return dq, dk, dv
    else:
        sl = None if x["seqlens_k"] is None else x["seqlens_k"].to(dev)
        o, lse = attn.attn_fwd(q, k, v, w.scale, w.causal, sl)
        ws = torch.empty((lib.attn_bwd_workspace_size(w.B, w.Hq, w.N),), dtype=torch.uint8,
                         device=dev)

        def step():
            attn.attn_bwd(q, k, v, o, lse, do, w.scale, w.causal, sl, workspace=ws,
                          out=(dq, dk, dv))
            return dq, dk, dv
    return step


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=inputs.HEADLINE, choices=sorted(inputs.WORKLOADS))
    ap.add_argument("--pass", dest="which", default="fwd", choices=("fwd", "bwd"),
                    help="fwd (default): the forward; bwd: the backward (attn_bwd) of the same "
                         "workload, from the forward's O and LSE and a seeded dO")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="CPU-oracle sample budget (0 disables the cpu_baseline leg)")
    ap.add_argument("--no-mfma-probe", action="store_true",
                    help="skip the sustained matrix-core rate measurement (attn_probe_mfma)")
    ap.add_argument("--library", default=None, metavar="PATH",
                    help="time another build of the library (e.g. "
                         "exact_attention_18_amd/libattn_exp2poly.so) instead of libattn.so")
    ap.add_argument("--compare", nargs="+", default=None, metavar="LIB",
                    help="only compare library builds: the workload's TFLOP/s under each, in "
                         "interleaved rounds in one process (one JSON line)")
    ap.add_argument("--rounds", type=int, default=4, help="rounds of --compare")
    ap.add_argument("--softmax-issue", action="store_true",
                    help="only measure the issue cost of the softmax's exp2 (hardware or polynomial) "
                         "beside a wave streaming MFMAs (attn_probe_softmax_issue), one JSON line")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run plain device-to-device copies of BYTES bytes (to scale the "
                         "FETCH_SIZE / WRITE_SIZE counters of the forward to bytes)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the forward "
              f"shards over (batch, KV head) with no communication; see the design notes)",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.softmax_issue:
        print(json.dumps({"softmax_issue": softmax_issue(dev)}), flush=True)
        return
    if args.copy_calibration:
        n = args.copy_calibration // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n * 4, "copies": args.steps}), flush=True)
        return
    if args.library:
        lib_ctx = attn.using_library(os.path.abspath(args.library))
        lib_ctx.__enter__()
    w = inputs.WORKLOADS[args.workload]
    print(f"[bench] workload {w.name}: generating inputs", file=sys.stderr, flush=True)
    x = inputs.workload_inputs(w)
    flops = algorithmic_flops(w, x)
    attn.load_library()
    if args.compare:
        cmp_ = compare_builds(w, x, dev, args.compare, args.steps, args.rounds, args.which)
        print(json.dumps({"compare": cmp_, "workload": w.name, "pass": args.which,
                          "steps": args.steps, "rounds": args.rounds}), flush=True)
        return
    if args.which == "bwd":
        return bench_backward(args, w, x, dev, flops)
    step = make_step(w, x, dev)

    first_ms = warm_up(step, args.warmup)
    K = args.steps
    ev_s = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    ev_e = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for i in range(K):
        ev_s[i].record()
        step_out = step()
        ev_e[i].record()
    t_end.record()
    torch.cuda.synchronize()
    ms_total = t_start.elapsed_time(t_end)
    ms_step = ms_total / K
    per_step = [a.elapsed_time(b) for a, b in zip(ev_s, ev_e)]
    kernel_ms = float(np.mean(per_step))
    median_ms = float(np.median(per_step))
    print(f"[bench] {K} steps, {ms_step:.4f} ms/step, kernel {kernel_ms:.4f} ms", file=sys.stderr,
          flush=True)

    value = flops / (ms_step * 1e-3) / 1e12
    achieved = flops / (kernel_ms * 1e-3) / 1e12
    probe = None
    if not args.no_mfma_probe:
        print("[bench] sustained matrix-core rate (attn_probe_mfma)", file=sys.stderr, flush=True)
        probe = mfma_sustained(dev)
        # the d = 128 forward runs on 16x16x32 MFMAs; the others on 32x32x16
        shape16 = w.d == 128 and w.d_v == 128
        probe["forward_mfma_shape"] = "16x16x32" if shape16 else "32x32x16"
        ref = probe["shape_16x16x32"]["random"] if shape16 else probe["random"]
        probe["forward_frac_of_random"] = round(achieved / ref["tflops"], 4)
    cpu = parity = None
    if args.cpu_seconds > 0:
        # the timed launches' own outputs, for the heads the oracle sample computes
        got = tuple(t.float().cpu().numpy() for t in step_out)
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        cpu, parity = cpu_baseline(w, x, args.cpu_seconds, got)
    cfg = {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "N": w.N, "d": w.d, "d_v": w.d_v,
           "causal": w.causal, "q_mult": w.q_mult, "algorithmic_flop": flops,
           "parallelism": "single GPU"}
    if args.library:
        cfg["library"] = os.path.basename(args.library)
    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "ms_per_step_median": round(median_ms, 5),
        "first_run_ms": first_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded i.i.d. N(0,1) bf16)",
        "config": cfg,
        "pct_of_mfma_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": None if args.library else measured_traffic(w.name),
                     "kernel_ms": round(kernel_ms, 5)},
        "mfma_sustained": probe,
        "cpu_baseline": cpu,
        "parity_sample": parity,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
