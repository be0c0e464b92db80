"""Comparison helpers for the GPU parity tests.

Tolerances (written here, used by every GPU test):

* scores: |gpu - oracle| <= max(rtol * |oracle|, 1e-6), rtol = 2e-3 for
  bf16/f16/fp8 inputs and 1e-4 for fp32 inputs (fp8 inputs are the same
  stored bits on both sides and their products are exact in the fp32
  accumulator, so the fp32 pipeline after the dot product sets the error,
  as for bf16); the same rule is applied to the
  column mass (score * Hq * n_b), whose magnitude is O(1), so the 1e-6 floor
  does not hide relative errors of tiny scores.
* LSE: |gpu - oracle| <= 1e-4 (bf16/f16/fp8) or 1e-5 (fp32), absolute,
  natural log units.
* kept sets: exact, except inside the tie band of a pool.  With oracle
  masses m sorted descending, m_(k) the k-th and m_(k+1) the (k+1)-th, let
  tau = max(rtol * m_(k) / (1 - 2 rtol), 1e-6).  A GPU mass g_j passes the
  mass test when |g_j - m_j| <= t_j = max(rtol * m_j, 1e-6), and t_j <= tau
  for every m_j <= m_(k) + 2 tau.  Then
    - m_j > m_(k+1) + 2 tau: g_j > m_(k+1) + tau >= g_i for each of the
      n - k candidates i with m_i <= m_(k+1), so j is kept by any such GPU;
    - m_j < m_(k) - 2 tau: g_j < m_(k) - tau <= g_i for each of the k
      candidates i with m_i >= m_(k), so j is dropped by any such GPU.
  Only candidates with m_(k) - 2 tau <= m_j <= m_(k+1) + 2 tau may be chosen
  freely (the count must still be k); that band holds candidates only when
  m_(k) - m_(k+1) <= 2 tau, the widest gap the score tolerance can explain.
  Everything outside it must match the oracle's kept set exactly.
* compaction, gather and rotary positions: bit-exact against the oracle's
  compaction of the oracle's flags whenever the kept sets agree; otherwise
  checked for validity against the GPU's own flags (order, bounds, spatial
  indices, counts, rows, each token's full-layout position).
"""
from __future__ import annotations

import numpy as np
import torch

import attention_score_selection_amd as tsel
import oracle


def rtol_of(prob) -> float:
    return 1e-4 if prob.dtype == "f32" else 2e-3


def lse_tol_of(prob) -> float:
    return 1e-5 if prob.dtype == "f32" else 1e-4


def run_gpu(prob, dev, lse=None, with_emb=True, emb=None):
    """Whole path on the GPU; returns numpy arrays."""
    lay = tsel.Layout.from_problem(prob, dev)
    q, k = prob.q.to(dev), prob.k.to(dev)
    e = None
    if with_emb:
        e = (prob.emb if emb is None else emb).to(dev)
    lse_t = None if lse is None else torch.as_tensor(lse, dtype=torch.float32).contiguous().to(dev)
    scale = prob.softmax_scale if prob.softmax_scale is not None else 0.0
    out = tsel.select(q, k, lay, prob.mask, prob.keep_ratio, emb=e, lse=lse_t, softmax_scale=scale)
    torch.cuda.synchronize(dev)
    comp = {key: v.cpu() for key, v in out["compact"].items()}
    return dict(lse=out["lse"].cpu().double().numpy(), score=out["score"].cpu().double().numpy(),
                keep=out["keep"].cpu().numpy(), k=np.asarray(out["k"]), compact=comp)


def mass_of(prob, score):
    n_b = np.diff(prob.cu_seqlens).astype(np.float64)
    return np.asarray(score, np.float64) * prob.hq * n_b[oracle.request_of_candidate(prob)]


def check_scores(prob, gpu_score, ref_mass, cands=None):
    """Score and mass tolerance on all (or the listed) candidates."""
    rtol = rtol_of(prob)
    idx = np.arange(prob.N) if cands is None else np.asarray(cands)
    ref_score = oracle.scores(prob, ref_mass)[idx]
    g = gpu_score[idx]
    bad = np.abs(g - ref_score) > np.maximum(rtol * np.abs(ref_score), 1e-6)
    assert not bad.any(), (f"{prob.name}: {bad.sum()} scores out of tolerance, e.g. c={idx[bad][:5]} "
                           f"gpu={g[bad][:5]} ref={ref_score[bad][:5]}")
    gm = mass_of(prob, gpu_score)[idx]
    rm = ref_mass[idx]
    bad = np.abs(gm - rm) > np.maximum(rtol * np.abs(rm), 1e-6)
    assert not bad.any(), (f"{prob.name}: {bad.sum()} masses out of tolerance, e.g. c={idx[bad][:5]} "
                           f"gpu={gm[bad][:5]} ref={rm[bad][:5]}")


def check_lse(prob, gpu_lse, ref_lse):
    tol = lse_tol_of(prob)
    ok = np.isfinite(ref_lse)
    err = np.abs(gpu_lse[ok] - ref_lse[ok])
    assert err.max(initial=0.0) <= tol, f"{prob.name}: LSE error {err.max()} > {tol}"


def check_keep(prob, gpu_keep, ref_mass, ks, pools=None):
    """Kept sets per pool, exact outside the tie band.  Returns True when the
    GPU's flags equal the oracle's everywhere checked."""
    rtol = rtol_of(prob)
    exact = True
    bounds = oracle.pool_bounds(prob)
    for b in (range(prob.B) if pools is None else pools):
        lo, hi = bounds[b]
        n, k = hi - lo, int(ks[b])
        g = gpu_keep[lo:hi].astype(bool)
        assert g.sum() == k, f"{prob.name}: pool {b} keeps {g.sum()} != k={k}"
        if n == 0 or k == 0 or k == n:
            continue
        m = np.where(np.isfinite(ref_mass[lo:hi]), ref_mass[lo:hi], -np.inf)
        ref_keep = np.zeros(n, bool)
        ref_keep[np.lexsort((np.arange(n), -m))[:k]] = True
        band = tie_band(m, k, rtol)
        if band.any():
            print(f"[tie band] {prob.name} pool {b}: {int(band.sum())} of {n} candidates free "
                  f"(k = {k})", flush=True)
            assert np.array_equal(g[~band], ref_keep[~band]), f"{prob.name}: pool {b} differs outside band"
            exact = exact and np.array_equal(g, ref_keep)
        else:
            assert np.array_equal(g, ref_keep), (f"{prob.name}: pool {b} kept set differs "
                                                 f"({np.sum(g != ref_keep)} positions)")
    return exact


def tie_band(m, k, rtol):
    """Candidates of one pool (oracle masses m, -inf for non-finite) whose
    membership in the top k is not fixed by the mass tolerance: those with
    m_(k) - 2 tau <= m <= m_(k+1) + 2 tau (see the module docstring)."""
    n = len(m)
    if k == 0 or k == n:
        return np.zeros(n, bool)
    srt = np.sort(m)[::-1]
    mk, mk1 = srt[k - 1], srt[k]
    if not (np.isfinite(mk) and np.isfinite(mk1)):
        return np.zeros(n, bool)
    tau = max(rtol * abs(mk) / (1.0 - 2.0 * rtol), 1e-6)
    return (m >= mk - 2 * tau) & (m <= mk1 + 2 * tau)


def check_compaction_valid(prob, keep, comp, emb=None):
    """Properties the compaction of `keep` must have (no oracle involved)."""
    tok = comp["token_idx"].numpy().astype(np.int64)
    sp = comp["spatial"].numpy().astype(np.int64)
    cu = comp["cu_seqlens"].numpy().astype(np.int64)
    cnt = comp["img_counts"].numpy().astype(np.int64)[: prob.S]
    cand_of = np.full(prob.T, -1, np.int64)
    img_of = np.full(prob.T, -1, np.int64)
    for s in range(prob.S):
        n = int(prob.img_hw[s, 0] * prob.img_hw[s, 1])
        t0 = int(prob.img_start[s])
        cand_of[t0:t0 + n] = np.arange(prob.cu_cands[s], prob.cu_cands[s] + n)
        img_of[t0:t0 + n] = s
    stays = np.where(cand_of >= 0, keep[np.maximum(cand_of, 0)] != 0 if prob.N else True, True)
    assert len(tok) == int(stays.sum())
    assert np.all(stays[tok]) and len(np.unique(tok)) == len(tok)
    assert np.all(np.diff(tok) > 0)  # requests are packed in order, so globally increasing
    assert cu[0] == 0 and cu[-1] == len(tok)
    for b in range(prob.B):
        seg = tok[cu[b]:cu[b + 1]]
        assert np.all((seg >= prob.cu_seqlens[b]) & (seg < prob.cu_seqlens[b + 1]))
    s = img_of[tok]
    assert np.array_equal(sp[:, 0], np.where(s >= 0, s, -1))
    is_img = s >= 0
    off = tok[is_img] - prob.img_start[s[is_img]]
    w = prob.img_hw[s[is_img], 1]
    assert np.array_equal(sp[is_img, 1], off // w) and np.array_equal(sp[is_img, 2], off % w)
    assert np.all(sp[~is_img] == -1)
    for si in range(prob.S):
        assert cnt[si] == int(keep[prob.cu_cands[si]:prob.cu_cands[si + 1]].sum())
    if emb is not None:
        assert torch.equal(comp["emb"].view(torch.uint8) if comp["emb"].dtype != torch.uint8 else comp["emb"],
                           emb[torch.from_numpy(tok)].view(torch.uint8))
    if "positions" in comp:
        # Each kept token keeps its full-layout rotary position.
        assert np.array_equal(comp["positions"].numpy(), oracle.rope_positions(prob)[tok])


def check_compaction_exact(prob, comp, ref_comp, emb=None):
    assert np.array_equal(comp["token_idx"].numpy(), ref_comp["token_idx"])
    assert np.array_equal(comp["spatial"].numpy(), ref_comp["spatial"])
    assert np.array_equal(comp["cu_seqlens"].numpy(), ref_comp["cu_seqlens"])
    assert np.array_equal(comp["img_counts"].numpy()[: prob.S], ref_comp["img_counts"])
    if emb is not None:
        want = emb[torch.from_numpy(ref_comp["token_idx"])]
        assert torch.equal(comp["emb"].view(torch.uint8), want.view(torch.uint8))
    if "positions" in comp:
        assert np.array_equal(comp["positions"].numpy(), ref_comp["positions"])


def full_check(prob, got, ref, emb=None):
    """Scores, LSE, kept sets and compaction against a full oracle run."""
    check_lse(prob, got["lse"], ref["lse"])
    check_scores(prob, got["score"], ref["mass"])
    assert np.array_equal(got["k"], ref["k"])
    exact = check_keep(prob, got["keep"], ref["mass"], ref["k"])
    check_compaction_valid(prob, got["keep"], got["compact"], emb)
    if exact:
        ref_comp = oracle.compact(prob, ref["keep"])
        check_compaction_exact(prob, got["compact"], ref_comp, emb)
    return exact
