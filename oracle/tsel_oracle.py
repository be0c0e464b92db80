"""CPU oracle for attention-score visual-token selection (fp64, numpy).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this module;
only the test suite, the smoke check and the benchmark's CPU-baseline leg do.
It shares no code with the HIP library: it reads the same stored Q/K bits
that the seeded generator produced and computes every step from its plain
definition, in float64, with no blocking beyond row blocks for memory.

What it computes, and where the pages define it:

* ``attention_stats`` -- per row the natural-log softmax normaliser
  ``LSE[h, i] = log sum_{j visible(i)} exp(scale * q_{i,h} . k_{j,g(h)})``
  over every visible key, text keys included (the REDtech article, section
  3.2, reuses FlashAttention's softmax LSE, which is this quantity; the
  LiteVLM review's formula section fixes the 1/sqrt(d) scale), and the column
  mass ``mass[c] = sum_h sum_{i sees c} exp(s_{i,c,h} - LSE[h, i])`` of each
  vision candidate (the score of a vision token is the attention it receives:
  LiteVLM review, formula section; averaged over heads and rows: REDtech
  article, section 3.2).
* ``scores`` -- ``mass / (Hq * n_b)``, the average over heads and over all
  rows of the request (constant divisor; masked pairs contribute zero).
* ``budget_k`` -- ``k = floor(r * N + 1e-6)`` clamped to ``[0, N]``: the
  LiteVLM main-results table's token counts (858, 948, 2292, 1063) all follow
  floor(r * vision) + text; the 1e-6 absorbs decimal ratios that are
  just below an integer product in binary64.
* ``topk`` -- one global pool per request across all of its images
  (REDtech article, section 3.1 and 3.2), keeping the k largest scores; equal
  scores go to the lower candidate index; a non-finite score ranks as -inf.
* ``mass_budget`` -- an input-dependent budget (a reading; the pages give
  no algorithm): per pool the fewest top-ranked candidates whose score mass
  reaches a fraction tau of the pool's total, clamped to [r_min, r_max] of
  the pool, counted in integer mass units of 2^-32 so that k is exact.
* ``compact`` / ``compact_loop`` -- stable compaction of each request: text
  tokens always stay, candidates stay iff kept; emits original packed token
  index, (image, row, col), new cu_seqlens and per-image kept counts, and the
  gathered embedding rows (REDtech article, section 3.2: new multimodal
  lengths, image boundaries and original spatial indices).

Readings of points the pages leave open are listed in the design notes; the
numeric pins live in ``tests/test_oracle.py``.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional, Sequence

import numpy as np

ROW_BLOCK = 256


def fp8_e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    """Decode OCP FP8 E4M3 byte codes to float64, exactly: sign bit, 4
    exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds
    subnormals m * 2^-9; no infinities; exponent and mantissa all ones is
    NaN (the format the LiteVLM review's FP8 deployment refers to)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 0xF) & (m == 0x7), np.nan, mag)
    return sign * mag


def to_f64(t) -> np.ndarray:
    """Exact widening of stored fp32/f16/bf16/fp8 values to float64."""
    try:
        import torch
        if isinstance(t, torch.Tensor):
            t = t.detach().to("cpu")
            if t.dtype == torch.float8_e4m3fn:
                return fp8_e4m3_to_f64(t.view(torch.uint8).numpy())
            return t.to(torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(t, dtype=np.float64)


def problem_scale(prob, d: int) -> float:
    """The problem's softmax scale: its own (fp8 inputs carry dequantisation
    factors) or 1/sqrt(d)."""
    s = getattr(prob, "softmax_scale", None)
    return default_scale(d) if s is None else float(s)


def default_scale(d: int) -> float:
    """1/sqrt(d) softmax temperature (LiteVLM review, formula section)."""
    return 1.0 / math.sqrt(d)


def attention_segments(prob):
    """Attention segments: requests for full/causal masks, images for the
    block-diagonal (per-image ViT) mask.  Each entry is
    ``(tok_lo, tok_hi, request, cand_local_positions, cand_global_indices)``."""
    segs = []
    cu, cui, st, hw, cc = (prob.cu_seqlens, prob.cu_images, prob.img_start, prob.img_hw,
                           prob.cu_cands)
    if prob.mask == "blockdiag":
        for b in range(prob.B):
            for s in range(cui[b], cui[b + 1]):
                n = int(hw[s, 0] * hw[s, 1])
                lo = int(st[s])
                segs.append((lo, lo + n, b, np.arange(n), np.arange(cc[s], cc[s] + n)))
    else:
        for b in range(prob.B):
            lo, hi = int(cu[b]), int(cu[b + 1])
            loc, glob = [], []
            for s in range(cui[b], cui[b + 1]):
                n = int(hw[s, 0] * hw[s, 1])
                loc.append(np.arange(st[s] - lo, st[s] - lo + n))
                glob.append(np.arange(cc[s], cc[s] + n))
            loc = np.concatenate(loc) if loc else np.zeros(0, np.int64)
            glob = np.concatenate(glob) if glob else np.zeros(0, np.int64)
            segs.append((lo, hi, b, loc, glob))
    return segs


def _segment_head(q64, k64, seg, h, g, scale, causal, lse_given):
    """One (segment, head): full-row logits, LSE (or the supplied one), and the
    column mass of the segment's candidates.  Plain definition, row blocks of
    256 rows only to bound memory."""
    lo, hi, _b, loc, _glob = seg
    n = hi - lo
    Qs = q64[lo:hi, h, :]
    Ks = k64[lo:hi, g, :]
    lse_out = np.empty(n)
    mass = np.zeros(len(loc))
    for r0 in range(0, n, ROW_BLOCK):
        r1 = min(n, r0 + ROW_BLOCK)
        # Causal rows r0..r1-1 see keys 0..r1-1 only; keys past r1 would be
        # masked to -inf, so they are left out of the logits.
        kend = r1 if causal else n
        S = scale * (Qs[r0:r1] @ Ks[:kend].T)
        if causal:
            rows = np.arange(r0, r1)[:, None]
            seen = np.arange(kend)[None, :] <= rows
            S = np.where(seen, S, -np.inf)
        if lse_given is None:
            m = S.max(axis=1)
            lse_rows = m + np.log(np.exp(S - m[:, None]).sum(axis=1))
        else:
            lse_rows = lse_given[lo + r0: lo + r1]
        lse_out[r0:r1] = lse_rows
        vis = loc < kend
        if vis.any():
            with np.errstate(invalid="ignore"):  # -inf - (-inf) at masked pairs, zeroed below
                P = np.exp(S[:, loc[vis]] - lse_rows[:, None])
            if causal:
                # A masked pair adds nothing to the mass, whatever the row's
                # (supplied) LSE: exp(-inf - LSE) is 0 for every LSE but -inf.
                P = np.where(seen[:, loc[vis]], P, 0.0)
            mass[vis] += P.sum(axis=0)
    return lse_out, mass


def attention_stats(prob, lse_in: Optional[np.ndarray] = None, scale: Optional[float] = None,
                    heads: Optional[Sequence[int]] = None, workers: int = 1,
                    segments: Optional[Sequence[int]] = None):
    """Return ``(lse [Hq, T] float64, mass [N] float64)``.

    ``lse_in`` (``[Hq, T]``) switches to the supplied-LSE path: the rows'
    normaliser is taken from it instead of being computed.  ``heads``
    restricts the work to a subset of query heads (their LSE rows and their
    share of the mass); ``segments`` to a subset of attention segments
    (requests, or images under the block-diagonal mask).  Entries outside the
    subset are NaN (LSE) or 0 (mass).  ``workers`` > 1 runs (segment, head)
    tasks on threads; numpy's BLAS and ufuncs release the GIL, and the
    per-task results are summed in a fixed order, so the answer does not
    depend on it.
    """
    q64, k64 = to_f64(prob.q), to_f64(prob.k)
    hq, hkv, d = q64.shape[1], k64.shape[1], q64.shape[2]
    assert hq % hkv == 0
    rep = hq // hkv
    scale = problem_scale(prob, d) if scale is None else scale
    causal = prob.mask == "causal"
    segs = attention_segments(prob)
    heads = list(range(hq)) if heads is None else list(heads)
    seg_ids = range(len(segs)) if segments is None else list(segments)
    tasks = [(si, h) for h in heads for si in seg_ids]
    lse_in64 = None if lse_in is None else np.asarray(lse_in, np.float64)

    def run(task):
        si, h = task
        given = None if lse_in64 is None else lse_in64[h]
        return _segment_head(q64, k64, segs[si], h, h // rep, scale, causal, given)

    if workers > 1:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(1), ThreadPoolExecutor(workers) as ex:
            results = list(ex.map(run, tasks))
    else:
        results = [run(t) for t in tasks]
    lse = np.full((hq, prob.T), np.nan)
    mass = np.zeros(prob.N)
    for (si, h), (lse_rows, m) in zip(tasks, results):
        lo, hi, _b, _loc, glob = segs[si]
        lse[h, lo:hi] = lse_rows
        mass[glob] += m
    return lse, mass


def attention_forward(prob, v=None, scale: Optional[float] = None, workers: int = 1,
                      heads: Optional[Sequence[int]] = None):
    """The attention layer's forward pass whose softmax normaliser the
    selection reuses (REDtech article, section 3.2): ``O = softmax(S) V`` per
    head and row, S the scaled, masked logits over the row's visible keys,
    plus the LSE.  Returns ``(o [T, Hq, d], lse [Hq, T])`` in float64; rows
    or heads outside ``heads`` are NaN."""
    q64, k64 = to_f64(prob.q), to_f64(prob.k)
    v64 = to_f64(prob.v if v is None else v)
    hq, hkv, d = q64.shape[1], k64.shape[1], q64.shape[2]
    dv = v64.shape[2]
    rep = hq // hkv
    scale = problem_scale(prob, d) if scale is None else scale
    causal = prob.mask == "causal"
    segs = attention_segments(prob)
    heads = list(range(hq)) if heads is None else list(heads)
    tasks = [(si, h) for h in heads for si in range(len(segs))]

    def run_one(task):
        si, h = task
        lo, hi = segs[si][0], segs[si][1]
        g = h // rep
        n = hi - lo
        o = np.empty((n, dv))
        lse = np.empty(n)
        for r0 in range(0, n, ROW_BLOCK):
            r1 = min(n, r0 + ROW_BLOCK)
            kend = r1 if causal else n
            S = scale * (q64[lo + r0:lo + r1, h, :] @ k64[lo:lo + kend, g, :].T)
            if causal:
                S = np.where(np.arange(kend)[None, :] <= np.arange(r0, r1)[:, None], S, -np.inf)
            m = S.max(axis=1)
            lse[r0:r1] = m + np.log(np.exp(S - m[:, None]).sum(axis=1))
            P = np.exp(S - lse[r0:r1, None])
            o[r0:r1] = P @ v64[lo:lo + kend, g, :]
        return o, lse

    if workers > 1:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(1), ThreadPoolExecutor(workers) as ex:
            results = list(ex.map(run_one, tasks))
    else:
        results = [run_one(t) for t in tasks]
    o_all = np.full((prob.T, hq, dv), np.nan)
    lse_all = np.full((hq, prob.T), np.nan)
    for (si, h), (o, lse) in zip(tasks, results):
        lo, hi = segs[si][0], segs[si][1]
        o_all[lo:hi, h, :] = o
        lse_all[h, lo:hi] = lse
    return o_all, lse_all


def lse_rows(prob, tokens: Sequence[int], scale: Optional[float] = None) -> np.ndarray:
    """LSE of selected rows, every query head: ``[Hq, len(tokens)]`` float64.
    Each row is the log-sum-exp of its visible logits, one row at a time."""
    q64, k64 = to_f64(prob.q), to_f64(prob.k)
    hq, hkv, d = q64.shape[1], k64.shape[1], q64.shape[2]
    rep = hq // hkv
    scale = problem_scale(prob, d) if scale is None else scale
    segs = attention_segments(prob)
    out = np.full((hq, len(tokens)), np.nan)
    for col, t in enumerate(tokens):
        for lo, hi, _b, _loc, _glob in segs:
            if lo <= t < hi:
                kend = t + 1 if prob.mask == "causal" else hi
                for h in range(hq):
                    z = scale * (k64[lo:kend, h // rep, :] @ q64[t, h, :])
                    m = z.max()
                    out[h, col] = m + np.log(np.exp(z - m).sum())
    return out


def forward_rows(prob, tokens: Sequence[int], v=None, scale: Optional[float] = None) -> np.ndarray:
    """Attention-forward output of selected rows, every query head:
    ``[len(tokens), Hq, dv]`` float64, one row at a time (softmax of the
    row's visible logits times the values)."""
    q64, k64 = to_f64(prob.q), to_f64(prob.k)
    v64 = to_f64(prob.v if v is None else v)
    hq, hkv, d = q64.shape[1], k64.shape[1], q64.shape[2]
    rep = hq // hkv
    scale = problem_scale(prob, d) if scale is None else scale
    segs = attention_segments(prob)
    out = np.full((len(tokens), hq, v64.shape[2]), np.nan)
    for row, t in enumerate(tokens):
        for lo, hi, _b, _loc, _glob in segs:
            if lo <= t < hi:
                kend = t + 1 if prob.mask == "causal" else hi
                for h in range(hq):
                    z = scale * (k64[lo:kend, h // rep, :] @ q64[t, h, :])
                    p = np.exp(z - z.max())
                    out[row, h] = (p / p.sum()) @ v64[lo:kend, h // rep, :]
    return out


def request_of_candidate(prob) -> np.ndarray:
    """Request index of every candidate."""
    out = np.empty(prob.N, np.int64)
    for b in range(prob.B):
        s0, s1 = prob.cu_images[b], prob.cu_images[b + 1]
        out[prob.cu_cands[s0]:prob.cu_cands[s1]] = b
    return out


def scores(prob, mass: np.ndarray) -> np.ndarray:
    """Average attention received: mass / (Hq * n_b) (constant divisor over
    all rows of the request)."""
    n_b = np.diff(prob.cu_seqlens).astype(np.float64)
    return mass / (prob.hq * n_b[request_of_candidate(prob)])


def budget_k(ratio: float, n: int) -> int:
    """k = floor(r * N + 1e-6), r clamped to [0, 1]; NaN is an error."""
    if math.isnan(ratio):
        raise ValueError("keep ratio is NaN")
    r = min(max(float(ratio), 0.0), 1.0)
    return int(min(max(math.floor(r * n + 1e-6), 0), n))


def pool_bounds(prob):
    """Candidate range [lo, hi) of each request's pool."""
    return [(int(prob.cu_cands[prob.cu_images[b]]), int(prob.cu_cands[prob.cu_images[b + 1]]))
            for b in range(prob.B)]


def topk(prob, score: np.ndarray, ratios=None):
    """Keep flags (uint8 [N]) and k per pool.  Largest scores first, equal
    scores by lower candidate index, non-finite scores rank as -inf."""
    ratios = prob.keep_ratio if ratios is None else ratios
    keep = np.zeros(prob.N, np.uint8)
    ks = []
    for b, (lo, hi) in enumerate(pool_bounds(prob)):
        n = hi - lo
        k = budget_k(ratios[b], n)
        ks.append(k)
        if k == 0:
            continue
        key = np.asarray(score[lo:hi], np.float64)
        key = np.where(np.isfinite(key), key, -np.inf)
        order = np.lexsort((np.arange(n), -key))
        keep[lo + order[:k]] = 1
    return keep, np.asarray(ks, np.int64)


def _ranked(score_pool) -> np.ndarray:
    """Candidate order of one pool: largest score first, equal scores by lower
    index, non-finite scores as -inf (the top-k order)."""
    key = np.asarray(score_pool, np.float64)
    key = np.where(np.isfinite(key), key, -np.inf)
    return np.lexsort((np.arange(len(key)), -key))


MASS_UNIT = 2.0 ** 32


def mass_units(score_pool) -> np.ndarray:
    """Score mass of each candidate in integer units of 2^-32:
    floor(min(s, 1) * 2^32) for a finite s > 0, else 0.  (Scores are averages
    of probabilities, so they lie in [0, 1]; integer units make the budget an
    exact computation whatever the summation order.)"""
    s = np.asarray(score_pool, np.float64)
    ok = np.isfinite(s) & (s > 0)
    return np.floor(np.minimum(np.where(ok, s, 0.0), 1.0) * MASS_UNIT).astype(np.uint64)


def mass_budget_k(score_pool, tau: float, r_min: float, r_max: float) -> int:
    """Input-dependent budget of one pool (a reading: the REDtech article,
    section 6.2, lists choosing the compression rate from the input as future
    work, and section 5.2 prunes less on detail-dense inputs; VisionZip's
    observation, section 3.1, is that a few dominant tokens carry most of the
    attention).  k* is the fewest top-ranked candidates whose mass reaches
    target = min(M, ceil((tau * M) * (1 - 1e-12))) of the pool's total M (in
    the units of ``mass_units``; products in binary64, the factor absorbing
    the binary error of decimal fractions such as 0.9), then
    k = clamp(k*, floor(r_min*N + 1e-6), floor(r_max*N + 1e-6))."""
    for v in (tau, r_min, r_max):
        if math.isnan(v):
            raise ValueError("tau / r_min / r_max must not be NaN")
    if r_min > r_max:
        raise ValueError("r_min > r_max")
    n = len(score_pool)
    m = mass_units(score_pool)
    total = int(m.sum(dtype=np.uint64))
    t = min(max(float(tau), 0.0), 1.0)
    target = min(total, int(math.ceil((t * float(total)) * (1.0 - 1e-12))))
    if target == 0:
        kstar = 0
    else:
        pref = np.cumsum(m[_ranked(score_pool)], dtype=np.uint64)
        kstar = int(np.searchsorted(pref, np.uint64(target), side="left")) + 1
    return min(max(kstar, budget_k(r_min, n)), budget_k(r_max, n))


def mass_budget(prob, score: np.ndarray, tau, r_min, r_max):
    """Keep flags (uint8 [N]) and k per pool under the input-dependent budget
    (per-pool tau, r_min, r_max); the kept set is the top-k of ``topk``."""
    keep = np.zeros(prob.N, np.uint8)
    ks = []
    for b, (lo, hi) in enumerate(pool_bounds(prob)):
        k = mass_budget_k(score[lo:hi], tau[b], r_min[b], r_max[b])
        ks.append(k)
        keep[lo + _ranked(score[lo:hi])[:k]] = 1
    return keep, np.asarray(ks, np.int64)


def _token_tables(prob):
    T = prob.T
    cand = np.full(T, -1, np.int64)
    img = np.full(T, -1, np.int64)
    for s in range(prob.S):
        n = int(prob.img_hw[s, 0] * prob.img_hw[s, 1])
        t0 = int(prob.img_start[s])
        cand[t0:t0 + n] = np.arange(prob.cu_cands[s], prob.cu_cands[s] + n)
        img[t0:t0 + n] = s
    return cand, img


def compact(prob, keep: np.ndarray, emb=None, with_positions: bool = True):
    """Stable compaction (numpy).  Returns a dict with ``token_idx`` [T_out],
    ``spatial`` [T_out, 3] ((img, row, col), -1 for text), ``cu_seqlens``
    [B+1], ``img_counts`` [S], the rotary ``positions`` [T_out, 3] of the
    kept tokens (unless ``with_positions`` is false: a token-by-token loop,
    slow for millions of tokens) and, when ``emb`` is given, ``emb``
    [T_out, D] (a row copy, bit-exact)."""
    cand, img = _token_tables(prob)
    if prob.N == 0:
        keep_tok = np.ones(prob.T, bool)
    else:
        keep_tok = np.where(cand >= 0, np.asarray(keep)[np.maximum(cand, 0)] != 0, True)
    token_idx = np.nonzero(keep_tok)[0]
    spatial = np.full((len(token_idx), 3), -1, np.int64)
    s = img[token_idx]
    is_img = s >= 0
    off = token_idx[is_img] - prob.img_start[s[is_img]]
    w = prob.img_hw[s[is_img], 1]
    spatial[is_img, 0] = s[is_img]
    spatial[is_img, 1] = off // w
    spatial[is_img, 2] = off % w
    csum = np.concatenate([[0], np.cumsum(keep_tok)])
    cu_out = csum[prob.cu_seqlens]
    img_counts = np.array([int(keep[prob.cu_cands[t]:prob.cu_cands[t + 1]].sum())
                           for t in range(prob.S)], np.int64)
    out = dict(token_idx=token_idx.astype(np.int64), spatial=spatial,
               cu_seqlens=cu_out.astype(np.int64), img_counts=img_counts)
    if emb is not None:
        out["emb"] = emb[token_idx]
    if with_positions:
        out["positions"] = rope_positions(prob)[token_idx]
    return out


def rope_positions(prob) -> np.ndarray:
    """Rotary (t, h, w) position of every token of the full layout, [T, 3].

    The REDtech article (section 3.2) updates the mRoPE positions of the
    compressed sequence without stating a rule; the reading taken is that a
    kept token keeps its position in the full request under the Qwen-VL
    multimodal scheme: walking a request in token order with an index i from
    0, a text token takes (i, i, i) and moves i on by 1; an image of rows x
    cols takes, for its token (row, col), (i, i + row, i + col), and moves i
    on by max(rows, cols)."""
    pos = np.full((prob.T, 3), -1, np.int64)
    for b in range(prob.B):
        lo, hi = int(prob.cu_seqlens[b]), int(prob.cu_seqlens[b + 1])
        starts = {int(prob.img_start[s]): s for s in range(prob.cu_images[b], prob.cu_images[b + 1])}
        t, i = lo, 0
        while t < hi:
            if t in starts:
                s = starts[t]
                rows, cols = int(prob.img_hw[s, 0]), int(prob.img_hw[s, 1])
                for r in range(rows):
                    for c in range(cols):
                        pos[t + r * cols + c] = (i, i + r, i + c)
                t += rows * cols
                i += max(rows, cols)
            else:
                pos[t] = (i, i, i)
                t += 1
                i += 1
    return pos


def compact_loop(prob, keep):
    """The same compaction as a token-by-token Python loop (cross-check)."""
    token_idx, spatial, cu_out = [], [], [0]
    img_counts = [0] * prob.S
    s_ptr = 0
    for b in range(prob.B):
        for t in range(int(prob.cu_seqlens[b]), int(prob.cu_seqlens[b + 1])):
            while s_ptr < prob.S and prob.img_start[s_ptr] + prob.img_hw[s_ptr, 0] * prob.img_hw[s_ptr, 1] <= t:
                s_ptr += 1
            in_img = s_ptr < prob.S and prob.img_start[s_ptr] <= t
            if in_img:
                o = t - int(prob.img_start[s_ptr])
                c = int(prob.cu_cands[s_ptr]) + o
                if keep[c]:
                    w = int(prob.img_hw[s_ptr, 1])
                    token_idx.append(t)
                    spatial.append((s_ptr, o // w, o % w))
                    img_counts[s_ptr] += 1
            else:
                token_idx.append(t)
                spatial.append((-1, -1, -1))
        cu_out.append(len(token_idx))
    return dict(token_idx=np.asarray(token_idx, np.int64),
                spatial=np.asarray(spatial, np.int64).reshape(-1, 3),
                cu_seqlens=np.asarray(cu_out, np.int64),
                img_counts=np.asarray(img_counts, np.int64))


def run(prob, lse_in: Optional[np.ndarray] = None, workers: int = 1, with_emb: bool = True):
    """Every step on one problem: LSE (or the supplied one), mass, score, keep
    flags, k per pool and the compaction."""
    lse, mass = attention_stats(prob, lse_in=lse_in, workers=workers)
    sc = scores(prob, mass)
    keep, ks = topk(prob, sc)
    comp = compact(prob, keep, prob.emb if with_emb else None)
    return dict(lse=lse, mass=mass, score=sc, keep=keep, k=ks, compact=comp)


def default_workers() -> int:
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:  # pragma: no cover
        return max(1, min(16, os.cpu_count() or 1))
