"""Plain fp64 CPU definition of exact attention, and the blockwise online recurrence.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module, and this module imports nothing from the product path.

What is computed, with the passages it follows
----------------------------------------------
* ``O = softmax(scale * Q K^T) V`` with softmax taken row-wise, ``scale = 1/sqrt(d)``
  in every workload (FlashAttention-4 (papercache summary), section 2.1
  "multi-head attention"; "059 · FlashAttention" (wq-win), section 2, the
  displayed definition; FlashAttention V1 到 V4 (chengxuchu), section 2).
  The FlashAttention notes (xwysyy) drop the scale in their "attention formula
  recap"; here the scale is an explicit argument.
* Safe softmax: subtract the row maximum ``m``, exponentiate, divide by the sum
  ``l`` (FlashAttention notes (xwysyy), "Safe Softmax").  The output also carries
  the per-row log-sum-exp ``LSE = m + ln l`` (natural log), the normaliser that
  the forward saves for the backward (FlashAttention notes (xwysyy),
  "Recomputation" and the code-structure overview of ``softmax_lse``).
* Masks (FlashAttention notes (xwysyy), "attention formula recap", masking on S;
  "059 · FlashAttention", section 3, causal / padding masks):
    - causal: key ``j`` visible to query ``i`` iff ``j <= i`` (top-left aligned);
    - key padding: key ``j`` visible iff ``j < nk_valid`` of that batch element;
    - varlen: indices local to each packed sequence.
  A row with no visible key yields ``O = 0`` and ``LSE = -inf``.
* Grouped-query heads: query head ``h`` reads key/value head ``h // G`` with
  ``G = Hq / Hkv`` (FlashAttention notes (xwysyy), "core observation": GQA stays
  exact; FlashAttention-4 (papercache summary), section 3.3, KV head shared by
  its group of query heads).

The one-shot functions materialise S and P in fp64 (a chunk of query rows at a
time, which is still the plain definition).  ``online_softmax_head`` runs the
blockwise recurrence itself; it exists so that the tests can show, in fp64,
that the recurrence reaches the one-shot result (Theorem 1 of the original
paper, as restated in "059 · FlashAttention", section 2).
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

__all__ = [
    "attention_probs",
    "attention_head",
    "attention_forward",
    "attention_forward_varlen",
    "attention_rows",
    "online_softmax_head",
    "block_mask_to_elements",
    "attention_forward_blocksparse",
]


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _visible(rows, nk, causal, nk_valid):
    """Boolean [len(rows), nk]: which keys each query row may attend to."""
    rows = np.asarray(rows)
    cols = np.arange(nk)
    vis = np.broadcast_to(cols[None, :] < nk_valid, (rows.shape[0], nk))
    if causal:
        vis = vis & (cols[None, :] <= rows[:, None])
    return vis


def attention_probs(q, k, scale, causal=False, nk_valid=None, rows=None, allowed=None):
    """Materialised scores, probabilities and LSE for one head.

    q: [Nq, d], k: [Nk, d].  Returns (S, P, LSE) for the requested query rows
    (all rows by default), where masked scores are -inf, every row of P with a
    visible key sums to 1, and LSE = m + ln(l) per row.

    Follows the safe softmax of FlashAttention notes (xwysyy), "Safe Softmax":
    m(x) = max_i x_i, f(x) = exp(x - m(x)), l(x) = sum f(x), softmax = f / l.
    """
    q = _f64(q)
    k = _f64(k)
    nq, nk = q.shape[0], k.shape[0]
    if nk_valid is None:
        nk_valid = nk
    rows = np.arange(nq) if rows is None else np.asarray(rows)
    s = scale * (q[rows] @ k.T)
    vis = _visible(rows, nk, causal, nk_valid)
    if allowed is not None:  # extra visibility mask [Nq, Nk] (block-sparse)
        vis = vis & np.asarray(allowed, dtype=bool)[rows]
    s = np.where(vis, s, -np.inf)
    m = s.max(axis=1) if nk > 0 else np.full(rows.shape[0], -np.inf)
    has_key = np.isfinite(m)
    m_safe = np.where(has_key, m, 0.0)
    e = np.exp(s - m_safe[:, None])  # exp(-inf) = 0 for masked keys
    l = e.sum(axis=1)
    p = np.where(has_key[:, None], e / np.where(has_key, l, 1.0)[:, None], 0.0)
    with np.errstate(divide="ignore"):
        lse = np.where(has_key, m_safe + np.log(np.where(has_key, l, 1.0)), -np.inf)
    return s, p, lse


def attention_head(q, k, v, scale, causal=False, nk_valid=None, rows=None, chunk=256,
                   allowed=None):
    """O = P V and LSE for one head, P materialised a chunk of rows at a time.

    q: [Nq, d], k: [Nk, d], v: [Nk, dv].  Returns (O [R, dv], LSE [R]) for the
    requested rows R (all rows by default).  The standard, unfused computation
    (FlashAttention notes (xwysyy), "Algorithm 0": S = Q K^T, P = softmax(S),
    O = P V), done in fp64.
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    out = np.zeros((rows.shape[0], v.shape[1]))
    lse = np.zeros(rows.shape[0])
    for r0 in range(0, rows.shape[0], chunk):
        rr = rows[r0 : r0 + chunk]
        _, p, l_ = attention_probs(q, k, scale, causal, nk_valid, rows=rr, allowed=allowed)
        out[r0 : r0 + rr.shape[0]] = p @ v
        lse[r0 : r0 + rr.shape[0]] = l_
    return out, lse


def _run_jobs(fn, jobs, workers):
    """Run independent per-head jobs, optionally on a thread pool.

    Heads are independent, so the order of evaluation does not change any
    value.  BLAS is limited to one thread per worker while the pool runs.
    """
    if workers is None or workers <= 1 or len(jobs) <= 1:
        return [fn(j) for j in jobs]
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover - threadpoolctl is present in this image
        threadpool_limits = None
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            with ThreadPoolExecutor(max_workers=workers) as ex:
                return list(ex.map(fn, jobs))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        return list(ex.map(fn, jobs))


def attention_forward(q, k, v, scale, causal=False, seqlens_k=None, workers=None, heads=None):
    """Batched, grouped-query forward in the [B, N, H, d] layout.

    q: [B, Nq, Hq, d], k: [B, Nk, Hkv, d], v: [B, Nk, Hkv, dv] (any real dtype;
    upcast to fp64).  seqlens_k: optional [B] ints, keys j >= seqlens_k[b] are
    masked.  Returns O [B, Nq, Hq, dv] and LSE [B, Hq, Nq] in fp64.

    ``heads``: optional list of (b, h) pairs; only those heads are computed and
    the rest of O / LSE is left as NaN (used to time a bounded sample).
    """
    B, Nq, Hq, _ = q.shape
    Hkv = k.shape[2]
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    dv = v.shape[3]
    out = np.full((B, Nq, Hq, dv), np.nan)
    lse = np.full((B, Hq, Nq), np.nan)
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(Hq)]

    def one(bh):
        b, h = bh
        nk_valid = None if seqlens_k is None else int(seqlens_k[b])
        return attention_head(q[b, :, h, :], k[b, :, h // G, :], v[b, :, h // G, :],
                              scale, causal, nk_valid)

    res = _run_jobs(one, heads, workers)
    for (b, h), (o_bh, l_bh) in zip(heads, res):
        out[b, :, h, :] = o_bh
        lse[b, h, :] = l_bh
    return out, lse


def attention_forward_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, scale, causal=False,
                             workers=None):
    """Packed variable-length forward.

    q: [Tq, Hq, d], k: [Tk, Hkv, d], v: [Tk, Hkv, dv]; sequence z owns query
    rows cu_seqlens_q[z] .. cu_seqlens_q[z+1]-1 and keys cu_seqlens_k[z] ..
    cu_seqlens_k[z+1]-1, with indices local to the sequence for the causal
    rule.  Returns O [Tq, Hq, dv] and LSE [Hq, Tq] in fp64.  Query rows that
    belong to no sequence are left as NaN.
    """
    Tq, Hq, _ = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    out = np.full((Tq, Hq, v.shape[2]), np.nan)
    lse = np.full((Hq, Tq), np.nan)
    cq = [int(x) for x in cu_seqlens_q]
    ck = [int(x) for x in cu_seqlens_k]
    jobs = [(z, h) for z in range(len(cq) - 1) for h in range(Hq)]

    def one(zh):
        z, h = zh
        return attention_head(q[cq[z]:cq[z + 1], h, :], k[ck[z]:ck[z + 1], h // G, :],
                              v[ck[z]:ck[z + 1], h // G, :], scale, causal)

    res = _run_jobs(one, jobs, workers)
    for (z, h), (o_zh, l_zh) in zip(jobs, res):
        out[cq[z]:cq[z + 1], h, :] = o_zh
        lse[h, cq[z]:cq[z + 1]] = l_zh
    return out, lse


def attention_rows(q, k, v, scale, causal, samples, seqlens_k=None):
    """Selected output rows of the batched forward, each by the plain definition.

    samples: iterable of (b, h, i).  Returns O [n, dv] and LSE [n].  Used to
    check full-size launches on rows the oracle can afford one by one.
    """
    Hq = q.shape[2]
    G = Hq // k.shape[2]
    samples = list(samples)
    out = np.zeros((len(samples), v.shape[3]))
    lse = np.zeros(len(samples))
    for n, (b, h, i) in enumerate(samples):
        nk_valid = None if seqlens_k is None else int(seqlens_k[b])
        o_, l_ = attention_head(q[b, :, h, :], k[b, :, h // G, :], v[b, :, h // G, :],
                                scale, causal, nk_valid, rows=[i])
        out[n] = o_[0]
        lse[n] = l_[0]
    return out, lse


def block_mask_to_elements(block_mask, nq, nk, bq, bk):
    """Element visibility [nq, nk] of a block mask: (i, j) allowed iff block_mask[i//bq, j//bk]."""
    bm = np.asarray(block_mask, dtype=bool)
    return bm[np.arange(nq)[:, None] // bq, np.arange(nk)[None, :] // bk]


def attention_forward_blocksparse(q, k, v, scale, block_mask, bq=128, bk=128, causal=False,
                                  seqlens_k=None, workers=None):
    """Block-sparse forward: S masked to -inf outside the nonzero blocks, then softmax, P V.

    The operator of block-sparse FlashAttention (FlashAttention notes
    (xwysyy), "Block-Sparse FlashAttention": P = softmax(S with the positions
    of zero blocks of the block mask set to -inf), O = P V), on top of the
    causal / padding masks.  block_mask: [Hm, ceil(Nq/bq), ceil(Nk/bk)] with
    Hm = 1 (shared by every head) or Hq; shared by the batch.  Layouts as in
    attention_forward.  Returns O [B, Nq, Hq, dv] and LSE [B, Hq, Nq].
    """
    B, Nq, Hq, _ = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    bm = np.asarray(block_mask)
    out = np.zeros((B, Nq, Hq, v.shape[3]))
    lse = np.zeros((B, Hq, Nq))
    allowed = [block_mask_to_elements(bm[h], Nq, Nk, bq, bk) for h in range(bm.shape[0])]
    jobs = [(b, h) for b in range(B) for h in range(Hq)]

    def one(bh):
        b, h = bh
        nk_valid = None if seqlens_k is None else int(seqlens_k[b])
        return attention_head(q[b, :, h], k[b, :, h // G], v[b, :, h // G], scale, causal, nk_valid,
                              allowed=allowed[h if len(allowed) > 1 else 0])

    for (b, h), (o_bh, l_bh) in zip(jobs, _run_jobs(one, jobs, workers)):
        out[b, :, h] = o_bh
        lse[b, h] = l_bh
    return out, lse


def online_softmax_head(q, k, v, scale, causal=False, nk_valid=None, block_rows=16,
                        block_cols=16, tau=None, normalize_each_step=False, trace_row=None):
    """The blockwise online-softmax recurrence for one head, in fp64.

    Query rows are taken block_rows at a time; for each query block the keys
    are visited block_cols at a time, keeping per row the running maximum m,
    the running sum l and the output accumulator.

    Unnormalised form (default), as in FlashAttention V1 到 V4 (chengxuchu),
    section 3.4.1, and "059 · FlashAttention" (wq-win), section 2:
        m' = max(m, max s),  l' = e^(m - m') l + sum_j e^(s_j - m'),
        u' = e^(m - m') u + sum_j e^(s_j - m') v_j,  O = u / l at the end.

    ``normalize_each_step=True`` keeps O normalised after every block instead,
    with the block-local max m~, P~ = e^(S - m~) and l~ = rowsum P~, as in the
    forward-pass algorithm of FlashAttention notes (xwysyy), "Algorithm 1":
        l' = e^(m - m') l + e^(m~ - m') l~,
        O' = (l e^(m - m') O + e^(m~ - m') P~ V) / l'.

    ``tau`` (only with the unnormalised form) applies the conditional rescaling
    of FlashAttention-4 (papercache summary), section 3.1.4: the running max is
    raised (and l, u rescaled) only when it would grow by more than tau, where
    tau is measured in log2 units (tau = 8 means a factor of 256); otherwise
    the stale max is kept and the block is accumulated with e^(s - m_old).
    The final u / l is exact either way.

    ``trace_row``: if set, also return the list of (m, l, u) of that row after
    each key block.

    Returns (O [Nq, dv], LSE [Nq]) or (O, LSE, trace).
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    nq, nk = q.shape[0], k.shape[0]
    dv = v.shape[1]
    if nk_valid is None:
        nk_valid = nk
    if tau is not None and normalize_each_step:
        raise ValueError("tau applies to the unnormalised form only")
    out = np.zeros((nq, dv))
    lse = np.full(nq, -np.inf)
    trace = []
    for i0 in range(0, nq, block_rows):
        rows = np.arange(i0, min(i0 + block_rows, nq))
        m = np.full(rows.shape[0], -np.inf)
        l = np.zeros(rows.shape[0])
        acc = np.zeros((rows.shape[0], dv))
        for j0 in range(0, nk, block_cols):
            cols = np.arange(j0, min(j0 + block_cols, nk))
            s = scale * (q[rows] @ k[cols].T)
            vis = _visible(rows, nk, causal, nk_valid)[:, cols]
            s = np.where(vis, s, -np.inf)
            m_blk = s.max(axis=1)
            if normalize_each_step:
                blk_has = np.isfinite(m_blk)
                m_blk_safe = np.where(blk_has, m_blk, 0.0)
                p_t = np.exp(s - m_blk_safe[:, None])
                l_t = p_t.sum(axis=1)
                m_new = np.maximum(m, m_blk)
                live = np.isfinite(m_new)
                m_new_safe = np.where(live, m_new, 0.0)
                a_old = np.where(np.isfinite(m), np.exp(m - m_new_safe), 0.0)
                a_blk = np.where(blk_has, np.exp(m_blk_safe - m_new_safe), 0.0)
                l_new = a_old * l + a_blk * l_t
                num = (l * a_old)[:, None] * acc + a_blk[:, None] * (p_t @ v[cols])
                acc = np.where(live[:, None], num / np.where(l_new > 0, l_new, 1.0)[:, None], 0.0)
                m, l = m_new, l_new
            else:
                m_cand = np.maximum(m, m_blk)
                if tau is None:
                    grow = np.ones(rows.shape[0], dtype=bool)
                else:
                    # First visible block always raises m (m = -inf before it).
                    with np.errstate(invalid="ignore"):
                        grow = ~np.isfinite(m) | ((m_cand - m) / math.log(2.0) > tau)
                m_new = np.where(grow, m_cand, m)
                live = np.isfinite(m_new)
                m_new_safe = np.where(live, m_new, 0.0)
                alpha = np.where(np.isfinite(m), np.exp(m - m_new_safe), 0.0)
                p = np.exp(s - m_new_safe[:, None])
                p = np.where(live[:, None], p, 0.0)
                l = alpha * l + p.sum(axis=1)
                acc = alpha[:, None] * acc + p @ v[cols]
                m = m_new
            if trace_row is not None and i0 <= trace_row < i0 + rows.shape[0]:
                r = trace_row - i0
                trace.append((float(m[r]), float(l[r]), acc[r].copy()))
        has = l > 0
        if normalize_each_step:
            out[rows] = np.where(has[:, None], acc, 0.0)
        else:
            out[rows] = np.where(has[:, None], acc / np.where(has, l, 1.0)[:, None], 0.0)
        with np.errstate(divide="ignore"):
            lse[rows] = np.where(has, np.where(np.isfinite(m), m, 0.0) + np.log(np.where(has, l, 1.0)),
                                 -np.inf)
    if trace_row is not None:
        return out, lse, trace
    return out, lse


def default_workers():
    """Host threads the oracle may use (the process's CPU affinity)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1
