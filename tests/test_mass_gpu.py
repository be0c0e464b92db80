"""GPU parity of the input-dependent budget (tsel_budget_mass) against the oracle.

The budget is integer arithmetic on integer mass units plus one binary64
product per pool, so k and the keep flags must match the oracle exactly on
the same fp32 scores.  Scores are drawn here (not by the GPU path), or come
from the GPU column score and are handed to both sides unchanged.
"""
import numpy as np
import pytest
import torch

import attention_score_selection_amd as tsel
import oracle
from workloads import make_config, make_problem, random_medium

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    tsel.lib()
    return torch.device("cuda:0")


def announce(name, extra=""):
    print(f"\n[case] mass budget {name} {extra}", flush=True)


def run_both(prob, score, tau, rmin, rmax, dev):
    lay = tsel.Layout.from_problem(prob, dev)
    keep, k = tsel.tsel_budget_mass(lay, torch.from_numpy(score).to(dev), tau, rmin, rmax)
    torch.cuda.synchronize(dev)
    ref_keep, ref_k = oracle.mass_budget(prob, score.astype(np.float64), tau, rmin, rmax)
    got_k = k.cpu().numpy()
    assert np.array_equal(got_k, ref_k), (got_k, ref_k)
    assert np.array_equal(keep.cpu().numpy(), ref_keep)
    return got_k


def pools_problem(sizes, name, seed):
    reqs = []
    for n in sizes:
        side = int(np.ceil(np.sqrt(n)))
        while n % side:
            side -= 1
        reqs.append((n + 3, [(2, n // side, side)]))
    return make_problem(name, reqs, 1, 1, 64, "bf16", "causal", 1.0, seed, ratio_range=(0.1, 0.9), emb_dim=4)


@pytest.mark.parametrize("pattern", ["diffuse", "peaked", "ties", "nonfinite", "above_one"])
def test_budget_mass_synthetic_pools(dev, pattern):
    """Pools on both sides of every register-run size of the top-k admission
    (1024, 4096, 16384 and 32768 candidates) and past the last."""
    sizes = [5, 1000, 1023, 1025, 4096, 4097, 16385, 32768, 32769, 50000]
    prob = pools_problem(sizes, "mass_pools_" + pattern, 41)
    rng = np.random.default_rng(42)
    parts = []
    for b, (lo, hi) in enumerate(oracle.pool_bounds(prob)):
        n = hi - lo
        w = rng.gamma(0.3 if pattern == "peaked" else 3.0, size=n)
        if pattern == "peaked":
            w[rng.choice(n, size=max(1, n // 100), replace=False)] *= 200.0
        parts.append(w / w.sum())
    score = np.concatenate(parts).astype(np.float32)
    if pattern == "ties":
        score = (np.round(score * prob.N / 4.0) * 4.0 / prob.N).astype(np.float32)
    if pattern == "nonfinite":
        idx = rng.choice(prob.N, size=prob.N // 50, replace=False)
        score[idx[0::4]] = np.nan
        score[idx[1::4]] = np.inf
        score[idx[2::4]] = -np.inf
        score[idx[3::4]] = -1e-3
    if pattern == "above_one":
        score[rng.choice(prob.N, size=7, replace=False)] = np.float32(3.5)
    announce(prob.name, f"pools={sizes}")
    B = prob.B
    for tau in (0.0, 0.3, 0.5, 0.9, 0.99, 1.0):
        run_both(prob, score, [tau] * B, [0.0] * B, [1.0] * B, dev)
    tau = list(rng.random(B))
    rmin = list(rng.random(B) * 0.3)
    rmax = [m + 0.6 for m in rmin]
    run_both(prob, score, tau, rmin, rmax, dev)


def test_budget_mass_uniform_pools_exact(dev):
    """Equal scores: k = tau * n exactly for tau on the grid 1/n (the 1e-12
    slack of the target absorbs the binary error of the decimal fraction)."""
    sizes = [10, 100, 40000]
    prob = pools_problem(sizes, "mass_uniform", 43)
    score = np.concatenate([np.full(n, 1.0 / n) for n in sizes]).astype(np.float32)
    announce(prob.name)
    for tau in (0.1, 0.5, 0.9):
        k = run_both(prob, score, [tau] * prob.B, [0.0] * prob.B, [1.0] * prob.B, dev)
        assert list(k) == [round(tau * n) for n in sizes]


def test_budget_mass_empty_and_zero_pools(dev):
    reqs = [(0, []), (37, [(5, 4, 6)]), (20, []), (41, [(0, 3, 3), (12, 5, 5)]), (9, [(1, 2, 2)])]
    prob = make_problem("mass_empties", reqs, 2, 1, 64, "bf16", "causal", 1.0, 44, ratio_range=(0.3, 0.8),
                        emb_dim=4)
    score = np.zeros(prob.N, np.float32)
    score[24:] = np.linspace(0.01, 0.2, prob.N - 24).astype(np.float32)  # first image: all zero
    announce(prob.name)
    k = run_both(prob, score, [0.7] * prob.B, [0.25] * prob.B, [0.9] * prob.B, dev)
    assert k[0] == 0 and k[2] == 0  # no candidates
    assert k[1] == oracle.budget_k(0.25, 24)  # zero mass: the lower bound


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_budget_mass_on_column_scores(dev, cfg):
    """The GPU column score of a named workload (one pool of 3072, 30720 or
    15000 candidates, or the varlen batch's eight pools), handed unchanged to
    both sides."""
    prob = make_config(cfg)
    announce(prob.name)
    lay = tsel.Layout.from_problem(prob, dev)
    q, k = prob.q.to(dev), prob.k.to(dev)
    scale = prob.softmax_scale or 0.0
    lse = tsel.tsel_lse(q, k, lay, prob.mask, scale)
    score = tsel.tsel_colscore(q, k, lay, prob.mask, lse, scale).cpu().numpy()
    for tau in (0.5, 0.8, 0.95):
        got = run_both(prob, score, [tau] * prob.B, [0.1] * prob.B, [0.9] * prob.B, dev)
        print(f"[check] tau={tau} k={list(got)} of N={prob.N}", flush=True)


def test_budget_mass_varlen_batch_per_request(dev):
    """Eight pools of the varlen batch with per-request tau and bounds."""
    prob = random_medium(45, "causal", dtype="f16", hq=4, hkv=4, d=64, n_req=8)
    announce(prob.name, f"B={prob.B} N={prob.N}")
    rng = np.random.default_rng(46)
    w = rng.gamma(0.5, size=prob.N)
    score = (w / w.sum()).astype(np.float32)
    run_both(prob, score, list(rng.random(prob.B)), [0.05] * prob.B, [0.95] * prob.B, dev)


def test_select_with_mass_budget(dev):
    """select(..., mass=...) runs the input-dependent budget inside the whole
    path; the kept set and compaction match the oracle's mass budget on the
    same GPU scores."""
    prob = random_medium(47, "causal", dtype="bf16", hq=8, hkv=2, d=128, n_req=3)
    announce(prob.name)
    lay = tsel.Layout.from_problem(prob, dev)
    q, k, emb = prob.q.to(dev), prob.k.to(dev), prob.emb.to(dev)
    tau, lo, hi = [0.7, 0.9, 0.5], [0.1, 0.2, 0.0], [0.9, 0.95, 1.0]
    out = tsel.select(q, k, lay, "causal", None, emb=emb, mass=(tau, lo, hi))
    torch.cuda.synchronize(dev)
    score = out["score"].cpu().numpy()
    ref_keep, ref_k = oracle.mass_budget(prob, score.astype(np.float64), tau, lo, hi)
    assert np.array_equal(np.asarray(out["k"]), ref_k)
    assert np.array_equal(out["keep"].cpu().numpy(), ref_keep)
    comp = oracle.compact(prob, ref_keep)
    assert np.array_equal(out["compact"]["token_idx"].cpu().numpy(), comp["token_idx"])
    assert np.array_equal(out["compact"]["positions"].cpu().numpy(), comp["positions"])
    assert torch.equal(out["compact"]["emb"].cpu(), prob.emb[torch.from_numpy(comp["token_idx"])])
