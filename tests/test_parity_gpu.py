"""GPU parity: the HIP path through the C-ABI against the CPU oracle.

Small and medium randomized layouts and the three smaller named workloads
are compared element by element with a live oracle run.  The two large
workloads are checked at full size: the 16384-token GQA decoder layer
against oracle scores stored by ``tests/golden/make_oracle_cache.py`` plus
live per-row LSE samples, and the varlen batch with the oracle's own LSE
supplied and live oracle masses for sampled requests.  Tolerances are
documented in ``tests/parity.py``.
"""
import os
import sys

import numpy as np
import pytest
import torch

import attention_score_selection_amd as tsel
import oracle
from workloads import make_config, make_problem, random_medium, random_small

sys.path.insert(0, os.path.dirname(__file__))
import parity as P  # noqa: E402

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    tsel.lib()  # raises if the library is not built
    return torch.device("cuda:0")


def announce(prob):
    print(f"\n[case] {prob.name} T={prob.T} N={prob.N} Hq={prob.hq} Hkv={prob.hkv} d={prob.d} "
          f"{prob.dtype} {prob.mask}", flush=True)


SMALL = [(s, m, dt, hq, hkv, d) for s, (m, dt, hq, hkv, d) in enumerate([
    ("full", "f32", 4, 4, 64), ("causal", "f32", 4, 2, 64), ("blockdiag", "f32", 2, 1, 128),
    ("full", "bf16", 8, 2, 128), ("causal", "bf16", 4, 1, 80), ("blockdiag", "bf16", 6, 2, 96),
    ("full", "f16", 3, 3, 96), ("causal", "f16", 16, 1, 64), ("blockdiag", "f16", 4, 4, 80),
    ("causal", "bf16", 12, 4, 128), ("full", "bf16", 32, 2, 64), ("causal", "f32", 2, 2, 96),
    ("full", "bf16", 4, 4, 72), ("blockdiag", "f16", 4, 2, 72), ("causal", "f32", 2, 1, 72),
])]


@pytest.mark.parametrize("seed,mask,dtype,hq,hkv,d", SMALL)
def test_small_random(dev, seed, mask, dtype, hq, hkv, d):
    prob = random_small(100 + seed, mask, dtype=dtype, hq=hq, hkv=hkv, d=d, n_req=3)
    announce(prob)
    got = P.run_gpu(prob, dev)
    P.full_check(prob, got, oracle.run(prob, with_emb=False), prob.emb)


MEDIUM = [("causal", "bf16", 8, 1, 128), ("full", "f16", 16, 4, 80), ("blockdiag", "bf16", 4, 4, 64),
          ("causal", "f32", 4, 2, 64), ("causal", "f16", 64, 8, 128), ("full", "bf16", 2, 2, 96),
          ("blockdiag", "bf16", 16, 16, 72)]


@pytest.mark.parametrize("i", range(len(MEDIUM)))
def test_medium_random(dev, i):
    mask, dtype, hq, hkv, d = MEDIUM[i]
    prob = random_medium(200 + i, mask, dtype=dtype, hq=hq, hkv=hkv, d=d, n_req=2 + i % 2)
    announce(prob)
    got = P.run_gpu(prob, dev)
    P.full_check(prob, got, oracle.run(prob, workers=oracle.default_workers(), with_emb=False),
                 prob.emb)


# One request longer than a row chunk (512 tokens at 16 folded heads) in a
# launch with enough jobs for full-size chunks, so the column score cuts the
# range after its last whole chunk (400 tokens) into pieces of 128; a short
# second request stays one chunk and makes the launch reorder its jobs.
LONG_SEGMENT = [(4496, [(100, 32, 32), (1161, 32, 32), (2185, 32, 32), (3259, 32, 32)]),
                (300, [(10, 12, 12)])]


@pytest.mark.parametrize("mask", ["causal", "full"])
def test_long_segment_last_chunk_pieces(dev, mask):
    prob = make_problem(f"long_segment_pieces_{mask}_f32_h32x2_d128", LONG_SEGMENT, 32, 2, 128, "f32",
                        mask, 1.0, 61, ratio_range=(0.3, 0.9), emb_dim=16)
    announce(prob)
    lay = tsel.Layout.from_problem(prob, dev)
    # 2 head blocks x 12 chunks (8 whole + 4 pieces) x N candidates of fp32.
    op = tsel.binding.TSEL_OP_COLSCORE
    assert tsel.tsel_workspace_size(op, lay, prob.q, prob.k, mask) == 2 * 12 * prob.N * 4
    got = P.run_gpu(prob, dev)
    P.full_check(prob, got, oracle.run(prob, workers=oracle.default_workers(), with_emb=False), prob.emb)


def layout_only(seed, t_target, n_req=3):
    """A layout of about t_target tokens (images of 64-128 rows and columns
    with text between them), without Q/K: for the compaction alone."""
    rng = np.random.default_rng(seed)
    seqlens, starts, hw = [0], [], []
    per = t_target // n_req
    for _ in range(n_req):
        t = seqlens[-1] + 37
        while t < seqlens[-1] + per:
            h, w = (int(x) for x in rng.integers(64, 129, size=2))
            starts.append(t)
            hw.append((h, w))
            t += h * w + int(rng.integers(0, 51))
        seqlens.append(t + 11)
    cu_images = [0]
    for b in range(n_req):
        cu_images.append(sum(1 for x in starts if x < seqlens[b + 1]))
    hw = np.array(hw, np.int64)
    cu_cands = np.concatenate([[0], np.cumsum(hw[:, 0] * hw[:, 1])])
    from types import SimpleNamespace
    return SimpleNamespace(T=seqlens[-1], B=n_req, S=len(starts), N=int(cu_cands[-1]),
                           cu_seqlens=np.array(seqlens, np.int64), cu_images=np.array(cu_images, np.int64),
                           img_start=np.array(starts, np.int64), img_hw=hw, cu_cands=cu_cands)


@pytest.mark.parametrize("t_target", [300_000, 4_300_000])
def test_compaction_alone_at_block_count_limits(dev, t_target):
    """tsel_compact alone on random keep flags: ~300 token blocks of 1024
    (the scatter pass forms its own block offsets and image counts) and over
    4096 blocks (a one-block scan between count and scatter forms them)."""
    lay_np = layout_only(70 + t_target % 7, t_target)
    print(f"\n[case] compaction alone T={lay_np.T} S={lay_np.S} N={lay_np.N}", flush=True)
    keep = (np.random.default_rng(71).random(lay_np.N) < 0.6).astype(np.uint8)
    lay = tsel.Layout(lay_np.cu_seqlens, lay_np.cu_images, lay_np.img_start, lay_np.img_hw, lay_np.cu_cands, dev)
    kb = [int(keep[lay_np.cu_cands[lay_np.cu_images[b]]:lay_np.cu_cands[lay_np.cu_images[b + 1]]].sum())
          for b in range(lay_np.B)]
    out = tsel.tsel_compact(lay, torch.from_numpy(keep).to(dev), kb)
    torch.cuda.synchronize(dev)
    ref = oracle.compact(lay_np, keep, with_positions=False)
    assert np.array_equal(out["token_idx"].cpu().numpy(), ref["token_idx"])
    assert np.array_equal(out["spatial"].cpu().numpy(), ref["spatial"])
    assert np.array_equal(out["cu_seqlens"].cpu().numpy(), ref["cu_seqlens"])
    assert np.array_equal(out["img_counts"].cpu().numpy()[: lay_np.S], ref["img_counts"])


SMALL_FP8 = [("full", 4, 4, 64), ("causal", 8, 2, 128), ("blockdiag", 4, 2, 64), ("causal", 16, 1, 128)]


@pytest.mark.parametrize("i", range(len(SMALL_FP8)))
def test_small_random_fp8(dev, i):
    """OCP E4M3 inputs with per-tensor factors folded into the softmax scale."""
    mask, hq, hkv, d = SMALL_FP8[i]
    prob = random_small(150 + i, mask, dtype="fp8", hq=hq, hkv=hkv, d=d, n_req=3)
    announce(prob)
    got = P.run_gpu(prob, dev)
    P.full_check(prob, got, oracle.run(prob, with_emb=False), prob.emb)


@pytest.mark.parametrize("mask,hq,hkv,d,std", [("causal", 8, 2, 128, 1.0), ("full", 16, 4, 64, 1.0),
                                               ("causal", 64, 8, 128, 0.0884)])
def test_medium_random_fp8(dev, mask, hq, hkv, d, std):
    prob = random_medium(250 + hq, mask, dtype="fp8", hq=hq, hkv=hkv, d=d, n_req=2, std=std)
    announce(prob)
    got = P.run_gpu(prob, dev)
    P.full_check(prob, got, oracle.run(prob, workers=oracle.default_workers(), with_emb=False),
                 prob.emb)


def test_litevlm_workload_fp8(dev):
    prob = make_config(2, dtype="fp8")
    announce(prob)
    got = P.run_gpu(prob, dev)
    P.full_check(prob, got, oracle.run(prob, workers=oracle.default_workers(), with_emb=False),
                 prob.emb)


@pytest.mark.parametrize("cfg,std", [(1, None), (2, None), (2, 1.0), (3, None)])
def test_named_workload_live_oracle(dev, cfg, std):
    prob = make_config(cfg, seed=cfg if std is None else cfg + 100, std=std)
    announce(prob)
    got = P.run_gpu(prob, dev)
    ref = oracle.run(prob, workers=oracle.default_workers(), with_emb=False)
    P.full_check(prob, got, ref, prob.emb)


def test_decoder_16384_gqa_full_size(dev):
    """Full-size GQA decoder layer: every score against the stored oracle
    masses, the kept set, the compaction, and live LSE samples."""
    cache = np.load(os.path.join(GOLDEN, "oracle_c4.npz"))
    prob = make_config(4)
    announce(prob)
    assert input_digest(prob) == str(cache["digest"]), "regenerated inputs differ from the stored oracle's"
    got = P.run_gpu(prob, dev)
    ref_mass = cache["mass"]
    P.check_scores(prob, got["score"], ref_mass)
    ref_keep, ref_k = oracle.topk(prob, oracle.scores(prob, ref_mass))
    assert np.array_equal(got["k"], ref_k)
    exact = P.check_keep(prob, got["keep"], ref_mass, ref_k)
    P.check_compaction_valid(prob, got["keep"], got["compact"], prob.emb)
    if exact:
        P.check_compaction_exact(prob, got["compact"], oracle.compact(prob, ref_keep), prob.emb)
    rows = np.linspace(0, prob.T - 1, 24).astype(int)
    ref_lse = oracle.lse_rows(prob, rows)
    P.check_lse(prob, got["lse"][:, rows], ref_lse)


def test_decoder_16384_gqa_fp8_full_size(dev):
    """The same layer with fp8 Q/K (the configuration the fp8 benchmark line
    times): every score against stored oracle masses, kept set, compaction,
    live LSE samples."""
    cache = np.load(os.path.join(GOLDEN, "oracle_c4_fp8.npz"))
    prob = make_config(4, dtype="fp8")
    announce(prob)
    assert input_digest(prob) == str(cache["digest"]), "regenerated inputs differ from the stored oracle's"
    assert float(cache["scale"]) == prob.softmax_scale
    got = P.run_gpu(prob, dev)
    ref_mass = cache["mass"]
    P.check_scores(prob, got["score"], ref_mass)
    ref_keep, ref_k = oracle.topk(prob, oracle.scores(prob, ref_mass))
    assert np.array_equal(got["k"], ref_k)
    exact = P.check_keep(prob, got["keep"], ref_mass, ref_k)
    P.check_compaction_valid(prob, got["keep"], got["compact"], prob.emb)
    if exact:
        P.check_compaction_exact(prob, got["compact"], oracle.compact(prob, ref_keep), prob.emb)
    rows = np.linspace(0, prob.T - 1, 24).astype(int)
    P.check_lse(prob, got["lse"][:, rows], oracle.lse_rows(prob, rows))


def input_digest(prob):
    import hashlib
    h = hashlib.sha256()
    for t in (prob.q, prob.k):
        h.update(t.contiguous().view(torch.uint8).numpy().tobytes())
    return h.hexdigest()


def test_varlen_supplied_lse_full_size(dev):
    """Varlen batch with the LSE supplied (the oracle's, rounded to fp32, as a
    FlashAttention forward would hand it over): every score of all eight
    requests against the live oracle masses computed from that same fp32
    LSE, every pool's kept set, and the compaction bit-exact when the kept
    sets agree."""
    prob = make_config(5)
    announce(prob)
    workers = oracle.default_workers()
    lse64, _ = oracle.attention_stats(prob, workers=workers)
    lse32 = lse64.astype(np.float32)
    got = P.run_gpu(prob, dev, lse=lse32)
    _, ref_mass = oracle.attention_stats(prob, lse_in=lse32, workers=workers)
    P.check_scores(prob, got["score"], ref_mass)
    ref_keep, ref_k = oracle.topk(prob, oracle.scores(prob, ref_mass))
    assert np.array_equal(got["k"], ref_k)
    exact = P.check_keep(prob, got["keep"], ref_mass, ref_k)
    P.check_compaction_valid(prob, got["keep"], got["compact"], prob.emb)
    if exact:
        P.check_compaction_exact(prob, got["compact"], oracle.compact(prob, ref_keep), prob.emb)
    print(f"[check] {prob.B} pools, {prob.N} candidates compared; kept sets exact: {exact}", flush=True)


@pytest.mark.parametrize("mask,dtype,hq,hkv,d", [("causal", "bf16", 16, 16, 128), ("full", "f16", 4, 2, 64),
                                                  ("blockdiag", "bf16", 8, 8, 80), ("causal", "f32", 2, 1, 96)])
def test_lse_key_split_matches_oracle(dev, mask, dtype, hq, hkv, d):
    """Grids too small to fill the GPU split every row block's keys into
    ranges whose partial log-sum-exps a merge pass combines; the split must
    be in use here (nonzero LSE workspace) and every LSE, score and kept set
    must match the oracle."""
    if mask == "blockdiag":
        reqs = [(3000, [(0, 30, 40), (1200, 25, 36), (2100, 30, 30)])]
    else:
        reqs = [(3214, [(256 * i, 16, 16) for i in range(12)]), (700, [(40, 20, 20)])]
    prob = make_problem(f"lse_split_{mask}_{dtype}_h{hq}x{hkv}_d{d}", reqs, hq, hkv, d, dtype, mask,
                        1.0 if mask != "causal" else 0.5, 63, ratio_range=(0.4, 0.9), emb_dim=32)
    announce(prob)
    lay = tsel.Layout.from_problem(prob, dev)
    need = tsel.tsel_workspace_size(tsel.binding.TSEL_OP_LSE, lay, prob.q, prob.k, mask)
    print(f"[check] LSE workspace {need} bytes = {need // (4 * hq * prob.T)} key splits", flush=True)
    assert need > 0 and need % (4 * hq * prob.T) == 0
    got = P.run_gpu(prob, dev)
    P.full_check(prob, got, oracle.run(prob, workers=oracle.default_workers(), with_emb=False), prob.emb)


# Logit offsets (natural log) of a planted large-norm key above the ordinary
# logits.  The LSE kernel sums exp2(c1*s - m) against m = (largest logit of
# the first key tile) + 32 in log2 units, and redoes a workgroup exactly (max
# pass, then sum pass) when any row sum leaves [2^-100, 2^100], i.e. when a
# later key's logit exceeds the first tile's largest by more than 132 log2
# units = 91.5 nats.  50 nats stays on the one-pass path with terms up to
# 2^40; 150 nats forces the exact path.
@pytest.mark.parametrize("nats", [50.0, 150.0])
@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("f16", 128)])
def test_lse_large_logit_range_one_pass_and_exact_fallback(dev, nats, dtype, d):
    """Q rows share a direction u; two keys, one at token 40 of the first
    request (past the first 32-key tile, first row block) and one at token
    300 of the second request (a later row block: 256 tokens per row block
    at d = 64, 2 query heads per KV head), are set to alpha * u so that every
    row after them sees a logit about `nats` above the others.  LSE, scores,
    kept sets and compaction against the live oracle."""
    reqs = [(420, [(8, 12, 16), (220, 10, 12)]), (520, [(30, 16, 16), (320, 12, 14)])]
    prob = make_problem(f"large_logit_{int(nats)}nats_{dtype}_d{d}", reqs, 4, 2, d, dtype, "causal",
                        0.5, 41, ratios=0.5, emb_dim=16)
    rng = np.random.default_rng(42)
    u = torch.from_numpy(rng.choice([-1.0, 1.0], size=d).astype(np.float32))
    q = prob.q.float()
    q = 0.5 * u + 0.5 * q  # shared direction plus noise of std 0.25
    # alpha: scale * (0.5 u) . (alpha u) = alpha * 0.5 * d / sqrt(d) = nats.
    alpha = nats / (0.5 * d ** 0.5)
    k = prob.k.float()
    t0 = int(prob.cu_seqlens[1])
    for t in (40, t0 + 300):
        k[t, :, :] = alpha * u
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    prob.q, prob.k = q.to(tdt), k.to(tdt)
    announce(prob)
    got = P.run_gpu(prob, dev)
    ref = oracle.run(prob, with_emb=False)
    # The planted keys do sit far above the first key tile of the rows after them.
    assert np.median(ref["lse"][:, 45:int(prob.cu_seqlens[1])]) > nats - 5
    P.full_check(prob, got, ref, prob.emb)


@pytest.mark.parametrize("cfg", [4, 5])
def test_large_shapes_value_sensitive(dev, cfg):
    """The decoder shapes at std 1 (peaked attention), reduced to 3 requests
    / 4096 tokens so the live oracle stays fast."""
    if cfg == 4:
        imgs = [(i * 750, 25, 30) for i in range(4)]
        prob = make_problem("decoder_4096_gqa64x8_std1", [(4096, imgs)], 64, 8, 128, "bf16",
                            "causal", 1.0, 104, ratios=0.6, emb_dim=512)
    else:
        reqs = [(1500, [(0, 20, 30), (600, 16, 20)]), (900, [(0, 17, 23)]), (2100, [(0, 32, 32)])]
        prob = make_problem("varlen_3req_h32_std1", reqs, 32, 32, 128, "f16", "causal", 1.0, 105,
                            ratio_range=(0.5, 0.9), emb_dim=256)
    announce(prob)
    ref = oracle.run(prob, workers=oracle.default_workers(), with_emb=False)
    got = P.run_gpu(prob, dev)
    P.full_check(prob, got, ref, prob.emb)


def test_long_sequence_properties(dev):
    """One 98304-token request (96 images of 32x32, so every token is a
    candidate), causal, 2/1 heads, d = 64: many row chunks and key blocks per
    head block.  Checks the LSE of sampled rows against the row-at-a-time
    oracle and, at full size, the identity sum_c mass_c = Hq * T (each row's
    probabilities sum to one and every key is a candidate) to 1e-4, plus the
    kept count and compacted length."""
    T = 98304
    imgs = [(i * 1024, 32, 32) for i in range(96)]
    prob = make_problem("long_98304_h2_d64_causal", [(T, imgs)], 2, 1, 64, "bf16", "causal", 1.0, 106,
                        ratios=0.5, emb_dim=16)
    announce(prob)
    lay = tsel.Layout.from_problem(prob, dev)
    q, k = prob.q.to(dev), prob.k.to(dev)
    out = tsel.select(q, k, lay, "causal", prob.keep_ratio)
    torch.cuda.synchronize(dev)
    mass_total = float(out["score"].double().sum()) * prob.hq * T
    print(f"[check] sum of column masses {mass_total:.6f} vs Hq*T = {prob.hq * T}", flush=True)
    assert abs(mass_total - prob.hq * T) <= 1e-4 * prob.hq * T
    rows = np.linspace(0, T - 1, 16).astype(int)
    ref = oracle.lse_rows(prob, rows)
    got = out["lse"].cpu().double().numpy()[:, rows]
    assert np.max(np.abs(got - ref)) <= 1e-4
    kept = int(out["keep"].sum())
    assert kept == int(out["k"][0]) == oracle.budget_k(0.5, T)
    assert int(out["compact"]["cu_seqlens"][-1]) == kept
    # The 98304-candidate pool takes the many-block top-k: its kept set is
    # exactly the oracle's top-k of the same (GPU) scores.
    ref_keep, _ = oracle.topk(prob, out["score"].cpu().double().numpy())
    assert np.array_equal(out["keep"].cpu().numpy(), ref_keep)


# ---------------------------------------------------------------------------
# Edge cases.
# ---------------------------------------------------------------------------

def test_many_requests_multi_launch_budgets(dev):
    """300 requests (more than one 256-pool top-k launch and several 64-pool
    mass-budget launches), each a short text run around one small image, and
    a few imageless requests: the whole path against the oracle, plus the
    mass budget on the GPU scores."""
    rng = np.random.default_rng(110)
    reqs = []
    for b in range(300):
        if b % 37 == 5:
            reqs.append((int(rng.integers(1, 9)), []))
            continue
        h, w = int(rng.integers(1, 4)), int(rng.integers(1, 5))
        pre = int(rng.integers(0, 4))
        reqs.append((pre + h * w + int(rng.integers(0, 4)), [(pre, h, w)]))
    prob = make_problem("many_300req_h4x2_d64", reqs, 4, 2, 64, "bf16", "causal", 1.0, 111,
                        ratio_range=(0.2, 0.9), emb_dim=16)
    announce(prob)
    got = P.run_gpu(prob, dev)
    P.full_check(prob, got, oracle.run(prob, with_emb=False), prob.emb)
    lay = tsel.Layout.from_problem(prob, dev)
    score = got["score"].astype(np.float32)
    tau = list(rng.random(prob.B))
    keep, k = tsel.tsel_budget_mass(lay, torch.from_numpy(score).to(dev), tau, [0.1] * prob.B, [0.9] * prob.B)
    torch.cuda.synchronize(dev)
    ref_keep, ref_k = oracle.mass_budget(prob, score.astype(np.float64), tau, [0.1] * prob.B, [0.9] * prob.B)
    assert np.array_equal(k.cpu().numpy(), ref_k)
    assert np.array_equal(keep.cpu().numpy(), ref_keep)


def test_debug_mode_checks_device_mirrors(dev, monkeypatch):
    """TSEL_DEBUG=1: a call first compares the device layout arrays with their
    host mirrors.  Consistent arrays pass and give the usual result; a device
    array that differs is rejected before any kernel runs (the layout is never
    used without the check while it is inconsistent)."""
    prob = random_small(61, "causal", dtype="bf16", hq=4, hkv=2, d=64, n_req=3)
    announce(prob)
    lay = tsel.Layout.from_problem(prob, dev)
    q, k = prob.q.to(dev), prob.k.to(dev)
    ref = tsel.tsel_lse(q, k, lay, "causal")
    monkeypatch.setenv("TSEL_DEBUG", "1")
    got = tsel.tsel_lse(q, k, lay, "causal")
    torch.cuda.synchronize(dev)
    assert torch.equal(got, ref)
    lay.d["cu_cands"][1] += 1
    torch.cuda.synchronize(dev)
    with pytest.raises(tsel.TselError, match="TSEL_DEBUG: device cu_cands"):
        tsel.tsel_lse(q, k, lay, "causal")
    with pytest.raises(tsel.TselError, match="TSEL_DEBUG"):
        tsel.tsel_colscore(q, k, lay, "causal", ref)
    lay.d["cu_cands"][1] -= 1
    torch.cuda.synchronize(dev)
    assert torch.equal(tsel.tsel_lse(q, k, lay, "causal"), ref)


def test_keep_nothing_and_everything(dev):
    prob = random_small(31, "causal", dtype="bf16", hq=4, hkv=2, d=64, n_req=3)
    prob.keep_ratio = np.array([0.0, 1.0, 0.5])
    announce(prob)
    got = P.run_gpu(prob, dev)
    P.full_check(prob, got, oracle.run(prob, with_emb=False), prob.emb)
    lo, hi = oracle.pool_bounds(prob)[0]
    assert got["keep"][lo:hi].sum() == 0
    lo, hi = oracle.pool_bounds(prob)[1]
    assert got["keep"][lo:hi].all()


def test_exact_ties_keep_lowest_indices(dev):
    """Zero keys under a full mask: every score is exactly 1/n; the budget
    keeps the first k candidates of each pool."""
    prob = random_small(32, "full", dtype="bf16", hq=4, hkv=2, d=64, n_req=2)
    prob.k = torch.zeros_like(prob.k)
    announce(prob)
    got = P.run_gpu(prob, dev)
    for b, (lo, hi) in enumerate(oracle.pool_bounds(prob)):
        n_b = prob.cu_seqlens[b + 1] - prob.cu_seqlens[b]
        assert np.all(got["score"][lo:hi] == got["score"][lo])
        assert abs(got["score"][lo] - 1.0 / n_b) <= 2e-3 / n_b
        k = got["k"][b]
        assert got["keep"][lo:lo + k].all() and not got["keep"][lo + k:hi].any()
    P.full_check(prob, got, oracle.run(prob, with_emb=False), prob.emb)


def test_empty_requests_and_imageless_requests(dev):
    reqs = [(0, []), (37, [(5, 4, 6)]), (0, []), (20, []), (41, [(0, 3, 3), (12, 5, 5)]), (0, [])]
    prob = make_problem("empties", reqs, 4, 2, 64, "bf16", "causal", 1.0, 33,
                        ratio_range=(0.3, 0.8), emb_dim=24)
    announce(prob)
    got = P.run_gpu(prob, dev)
    P.full_check(prob, got, oracle.run(prob, with_emb=False), prob.emb)


def test_tiny_images_blockdiag(dev):
    reqs = [(1 + 4 + 2 + 9, [(0, 1, 1), (1, 2, 2), (5, 1, 2), (7, 3, 3)])]
    prob = make_problem("tiny_images", reqs, 2, 1, 64, "f16", "blockdiag", 1.0, 34, ratios=0.5,
                        emb_dim=8)
    announce(prob)
    got = P.run_gpu(prob, dev)
    P.full_check(prob, got, oracle.run(prob, with_emb=False), prob.emb)


@pytest.mark.parametrize("n_img", [64, 65, 90])
def test_many_images_in_one_request(dev, n_img):
    """One causal request holding n_img small images (2x3, 1x4, ...) between
    text runs: the column score maps candidates to tokens through a per-lane
    image table when a segment has at most 64 images and through a search of
    the layout beyond that; both against the oracle, with GQA and a second
    request after the first."""
    rng = np.random.default_rng(200 + n_img)
    imgs, t = [], 0
    for i in range(n_img):
        t += int(rng.integers(0, 3))
        h, w = int(rng.integers(1, 4)), int(rng.integers(1, 5))
        imgs.append((t, h, w))
        t += h * w
    n0 = t + 5
    reqs = [(n0, imgs), (40, [(3, 4, 4)])]
    prob = make_problem(f"many_images_{n_img}", reqs, 8, 2, 64, "bf16", "causal", 1.0, 300 + n_img,
                        ratios=0.5, emb_dim=16)
    announce(prob)
    got = P.run_gpu(prob, dev)
    P.full_check(prob, got, oracle.run(prob, with_emb=False), prob.emb)


# Images whose candidate counts leave every kind of last key block: with
# four resident 32-key groups per wave a key block holds 512 candidates, and
# a block of 1, 31, 33, 96, 97, 129, 300 or 511 leaves waves with no group,
# with one partly filled group, or with fewer groups than the others.
RAGGED_IMAGES = [(27, 19), (1, 31), (5, 109), (1, 97), (3, 43), (19, 32), (31, 33), (28, 29), (1, 1), (7, 73)]


@pytest.mark.parametrize("mask,dtype,hq,hkv,d", [("causal", "bf16", 16, 16, 64), ("causal", "f16", 32, 4, 128),
                                                 ("full", "bf16", 16, 16, 64), ("causal", "fp8", 16, 16, 128)])
def test_ragged_key_block_tails(dev, mask, dtype, hq, hkv, d):
    """One image per request, each a different candidate count; text before
    and after it.  Sized so that the column score keeps its widest key
    blocks (at least 512 jobs once row chunks are cut to 64 tokens); every
    score, kept set and compaction against the oracle."""
    reqs = [(7 + h * w + 40, [(7, h, w)]) for h, w in RAGGED_IMAGES]
    F = 1
    while F < 16 and (hq // hkv) % (2 * F) == 0:
        F *= 2
    jobs_at_64 = (hq // F) * sum(((h * w + 511) // 512) * ((n + 63) // 64) for n, ((_, h, w),) in reqs)
    assert jobs_at_64 >= 512, jobs_at_64
    prob = make_problem(f"ragged_tails_{mask}_{dtype}_{hq}x{hkv}_d{d}", reqs, hq, hkv, d, dtype, mask,
                        1.0, 400 + d + hq, ratio_range=(0.3, 0.8), emb_dim=16)
    announce(prob)
    got = P.run_gpu(prob, dev)
    P.full_check(prob, got, oracle.run(prob, with_emb=False), prob.emb)


def test_nonfinite_inputs_rank_last(dev):
    """A NaN in one query row poisons the LSE of that row and the scores of
    every candidate the row sees; those rank as -inf, identically on both sides."""
    prob = random_small(35, "causal", dtype="bf16", hq=2, hkv=1, d=64, n_req=2)
    q = prob.q.clone()
    t_bad = int(prob.cu_seqlens[1]) - 3  # late row of request 0
    q[t_bad, 1, 5] = float("nan")
    prob.q = q
    announce(prob)
    got = P.run_gpu(prob, dev)
    ref = oracle.run(prob, with_emb=False)
    assert np.array_equal(np.isnan(got["score"]), np.isnan(ref["score"]))
    assert np.isnan(ref["score"]).any()
    fin = np.isfinite(ref["score"])
    rtol = P.rtol_of(prob)
    assert np.all(np.abs(got["score"][fin] - ref["score"][fin]) <=
                  np.maximum(rtol * np.abs(ref["score"][fin]), 1e-6))
    assert np.array_equal(got["keep"], ref["keep"])


@pytest.mark.filterwarnings("ignore:invalid value encountered:RuntimeWarning")  # the oracle's inf - inf
@pytest.mark.parametrize("bad", [float("nan"), float("inf")])
def test_nonfinite_key_poisons_the_rows_that_see_it(dev, bad):
    """A NaN or +inf in one key of one KV head: every row of that head group
    that sees the key has a NaN LSE (for +inf: the logit is +-inf and the
    row's normaliser inf - inf), and the scores those rows reach are NaN; the
    same pattern, the remaining scores and the kept sets as the oracle."""
    prob = random_small(41, "causal", dtype="bf16", hq=4, hkv=2, d=64, n_req=2)
    k = prob.k.clone()
    t_bad = int(prob.cu_seqlens[1]) + 5  # an early token of request 1
    k[t_bad, 1, 7] = bad
    prob.k = k
    announce(prob)
    got = P.run_gpu(prob, dev)
    ref = oracle.run(prob, with_emb=False)
    assert np.array_equal(np.isnan(got["lse"]), np.isnan(ref["lse"]))
    assert np.isnan(ref["lse"]).any()
    fin_l = np.isfinite(ref["lse"])
    assert np.max(np.abs(got["lse"][fin_l] - ref["lse"][fin_l])) <= P.lse_tol_of(prob)
    assert np.array_equal(np.isnan(got["score"]), np.isnan(ref["score"]))
    fin = np.isfinite(ref["score"])
    rtol = P.rtol_of(prob)
    assert np.all(np.abs(got["score"][fin] - ref["score"][fin]) <=
                  np.maximum(rtol * np.abs(ref["score"][fin]), 1e-6))
    assert np.array_equal(got["k"], ref["k"])
    P.check_keep(prob, got["keep"], ref["mass"], ref["k"])


def test_strided_qk_from_fused_projection(dev):
    """Q and K as views into one fused [T, Hq + 2*Hkv, d] projection."""
    prob = random_medium(36, "causal", dtype="bf16", hq=8, hkv=2, d=128, n_req=2)
    announce(prob)
    T = prob.T
    qkv = torch.empty((T, 8 + 2 * 2, 128), dtype=torch.bfloat16)
    qkv[:, :8] = prob.q
    qkv[:, 8:10] = prob.k
    qkv[:, 10:] = 0
    lay = tsel.Layout.from_problem(prob, dev)
    g = qkv.to(dev)
    q, k = g[:, :8], g[:, 8:10]
    lse = tsel.tsel_lse(q, k, lay, "causal")
    score = tsel.tsel_colscore(q, k, lay, "causal", lse)
    torch.cuda.synchronize()
    ref = oracle.run(prob, with_emb=False)
    P.check_lse(prob, lse.cpu().double().numpy(), ref["lse"])
    P.check_scores(prob, score.cpu().double().numpy(), ref["mass"])


def test_supplied_lse_shift_identity(dev):
    """Supplying LSE + delta scales every score by exp(-delta) (reuse path)."""
    prob = random_medium(37, "causal", dtype="f16", hq=4, hkv=4, d=128, n_req=2)
    announce(prob)
    lay = tsel.Layout.from_problem(prob, dev)
    q, k = prob.q.to(dev), prob.k.to(dev)
    lse = tsel.tsel_lse(q, k, lay, "causal")
    s0 = tsel.tsel_colscore(q, k, lay, "causal", lse).double()
    s1 = tsel.tsel_colscore(q, k, lay, "causal", (lse + 0.75).contiguous()).double()
    torch.cuda.synchronize()
    ratio = (s1 / s0).cpu().numpy()
    assert np.allclose(ratio, np.exp(-0.75), rtol=1e-5)


def test_supplied_lse_nonfinite_rows(dev):
    """A supplied LSE holding +inf (the row contributes nothing), -inf (every
    score the row reaches becomes +inf) and NaN rows: the column score starts
    its accumulation chains from -LSE/scale, so these reach the chains
    directly; scores, their non-finite pattern and the kept sets against the
    oracle with the same LSE."""
    prob = random_medium(39, "causal", dtype="f16", hq=4, hkv=2, d=128, n_req=2)
    announce(prob)
    lse64, _ = oracle.attention_stats(prob)
    lse32 = lse64.astype(np.float32)
    rng = np.random.default_rng(39)
    t0, t1 = int(prob.cu_seqlens[1]), int(prob.cu_seqlens[2])
    for val in (np.inf, -np.inf, np.nan):
        h = int(rng.integers(0, prob.hq))
        t = int(rng.integers(t0 + (t1 - t0) // 2, t1))  # a late row of request 1
        lse32[h, t] = val
    ref = oracle.run(prob, lse_in=lse32.astype(np.float64), with_emb=False)
    got = P.run_gpu(prob, dev, lse=lse32)
    assert np.array_equal(np.isnan(got["score"]), np.isnan(ref["score"]))
    assert np.array_equal(np.isposinf(got["score"]), np.isposinf(ref["score"]))
    assert np.isnan(ref["score"]).any() and np.isposinf(ref["score"]).any()
    fin = np.isfinite(ref["score"])
    rtol = P.rtol_of(prob)
    assert np.all(np.abs(got["score"][fin] - ref["score"][fin]) <=
                  np.maximum(rtol * np.abs(ref["score"][fin]), 1e-6))
    assert np.array_equal(got["k"], ref["k"])
    P.check_keep(prob, got["keep"], np.where(np.isfinite(ref["mass"]), ref["mass"], -np.inf), ref["k"])


def test_deterministic_repeat(dev):
    prob = random_medium(38, "causal", dtype="bf16", hq=16, hkv=4, d=128, n_req=3)
    announce(prob)
    a = P.run_gpu(prob, dev)
    b = P.run_gpu(prob, dev)
    assert np.array_equal(a["lse"], b["lse"], equal_nan=True)
    assert np.array_equal(a["score"], b["score"])
    assert np.array_equal(a["keep"], b["keep"])
    for key in a["compact"]:
        assert torch.equal(a["compact"][key], b["compact"][key])


@pytest.mark.parametrize("pattern", ["distinct", "ties", "nonfinite"])
def test_budget_topk_synthetic_scores_all_pool_sizes(dev, pattern):
    """tsel_budget_topk alone on synthetic fp32 scores (drawn here, not by the
    GPU path), pools on both sides of every register-run size (1, 4, 16 and 32
    keys per thread: pool limits 1024, 4096, 16384, 32768) and past the last
    into the streaming path, against the oracle's rank rule exactly."""
    sizes = [5, 1000, 1023, 1024, 1025, 3000, 4096, 4097, 9000, 16384, 16385, 32768, 32769, 50000]
    reqs, off = [], 0
    for n in sizes:
        side = int(np.ceil(np.sqrt(n)))
        while n % side:
            side -= 1
        reqs.append((n + 3, [(2, n // side, side)]))
    prob = make_problem("topk_pools_" + pattern, reqs, 1, 1, 64, "bf16", "causal", 1.0, 37,
                        ratio_range=(0.1, 0.9), emb_dim=4)
    rng = np.random.default_rng(38)
    score = (rng.random(prob.N) * 1e-4 + 3e-5).astype(np.float32)
    if pattern == "ties":
        score = np.round(score * 2e5).astype(np.float32) / np.float32(2e5)  # ~20 distinct values
    if pattern == "nonfinite":
        idx = rng.choice(prob.N, size=prob.N // 50, replace=False)
        score[idx[0::3]] = np.nan
        score[idx[1::3]] = np.inf
        score[idx[2::3]] = -np.inf
    announce(prob)
    lay = tsel.Layout.from_problem(prob, dev)
    keep, ks = tsel.tsel_budget_topk(lay, torch.from_numpy(score).to(dev), prob.keep_ratio)
    torch.cuda.synchronize(dev)
    ref_keep, ref_k = oracle.topk(prob, score.astype(np.float64))
    assert np.array_equal(ks, ref_k)
    assert np.array_equal(keep.cpu().numpy(), ref_keep)


@pytest.mark.parametrize("pattern", ["distinct", "ties", "nonfinite"])
def test_budget_topk_many_large_pools(dev, pattern):
    """70 pools of 32769..40000 candidates (two launches of the many-block
    top-k, 64 pools each at most) and one pool of 10^6, plus small pools in
    between, on synthetic fp32 scores, against the oracle's rank rule
    exactly; k from 0 to N."""
    rng = np.random.default_rng(39)
    reqs = []
    for i in range(70):
        n = int(rng.integers(32769, 40001))
        side = 1
        for f in range(int(np.sqrt(n)), 0, -1):
            if n % f == 0:
                side = f
                break
        reqs.append((n + 2, [(1, n // side, side)]))
        if i % 10 == 3:
            reqs.append((50, [(3, 5, 7)]))
    reqs.append((1_000_000 + 5, [(5, 1000, 1000)]))
    prob = make_problem("topk_many_large_" + pattern, reqs, 1, 1, 64, "bf16", "causal", 1.0, 40,
                        ratio_range=(0.05, 0.95), emb_dim=4)
    prob.keep_ratio[0], prob.keep_ratio[1], prob.keep_ratio[-1] = 0.0, 1.0, 0.37
    score = (rng.random(prob.N) * 1e-4 + 3e-5).astype(np.float32)
    if pattern == "ties":
        score = np.round(score * 1e5).astype(np.float32) / np.float32(1e5)  # ~10 distinct values
    if pattern == "nonfinite":
        idx = rng.choice(prob.N, size=prob.N // 40, replace=False)
        score[idx[0::3]] = np.nan
        score[idx[1::3]] = np.inf
        score[idx[2::3]] = -np.inf
    announce(prob)
    lay = tsel.Layout.from_problem(prob, dev)
    assert tsel.tsel_workspace_size(tsel.binding.TSEL_OP_TOPK, lay) > 0
    keep, ks = tsel.tsel_budget_topk(lay, torch.from_numpy(score).to(dev), prob.keep_ratio)
    torch.cuda.synchronize(dev)
    ref_keep, ref_k = oracle.topk(prob, score.astype(np.float64))
    assert np.array_equal(ks, ref_k)
    assert np.array_equal(keep.cpu().numpy(), ref_keep)
