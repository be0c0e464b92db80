"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Every check here uses a value fixed by the pages or by mathematics:
high-precision brute force on tiny inputs, closed forms (two keys, zero
keys under each mask, a single dominant key), invariants (mass conservation,
GQA = repeated MHA, permutation equivariance, the supplied-LSE identity),
library routines for the special cases they cover, brute-force rank
counting for the budget, the token counts printed in the LiteVLM review's
main-results table for the budget rule, and a token-by-token loop for the
compaction.  The last group plants mistakes in a copy of the oracle's
arithmetic and checks that the pins catch them.
"""
import math
import os

import mpmath
import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle import tsel_oracle as O
from workloads import Problem, layout_arrays, make_config, make_problem, random_small

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def handmade(requests, q, k, mask, ratios=1.0, emb_dim=4):
    """Problem from explicit fp64-representable Q/K values (stored as fp32)."""
    cu, cui, st, hw, cc = layout_arrays(requests)
    T = int(cu[-1])
    q = torch.as_tensor(np.asarray(q, np.float32))
    k = torch.as_tensor(np.asarray(k, np.float32))
    assert q.shape[0] == T and k.shape[0] == T
    B = len(cu) - 1
    p = Problem(name="hand", q=q, k=k, mask=mask, cu_seqlens=cu, cu_images=cui,
                img_start=st, img_hw=hw, cu_cands=cc,
                keep_ratio=np.broadcast_to(np.float64(ratios), (B,)).copy(),
                emb_dim=emb_dim, emb_dtype="f32", dtype="f32")
    p.emb = torch.arange(T * emb_dim, dtype=torch.float32).reshape(T, emb_dim)
    return p


def visible(prob, i, j):
    """Visibility straight from the mask's wording, token by token."""
    cu = prob.cu_seqlens
    bi = np.searchsorted(cu, i, side="right") - 1
    bj = np.searchsorted(cu, j, side="right") - 1
    if bi != bj:
        return False
    if prob.mask == "causal":
        return j <= i
    if prob.mask == "blockdiag":
        def img(t):
            for s in range(prob.S):
                n = prob.img_hw[s, 0] * prob.img_hw[s, 1]
                if prob.img_start[s] <= t < prob.img_start[s] + n:
                    return s
            return -1
        return img(i) == img(j) and img(i) >= 0
    return True


def mp_reference(prob, scale=None):
    """50-digit brute force: LSE per (h, i) and mass per candidate.  Inputs are
    widened by torch (its own fp8 decode included), not by the oracle."""
    mpmath.mp.dps = 50
    q = prob.q.to(torch.float64).numpy()
    k = prob.k.to(torch.float64).numpy()
    T, hq, d = q.shape
    rep = hq // k.shape[1]
    scale = 1 / mpmath.sqrt(d) if scale is None else mpmath.mpf(scale)
    cand_tok = []
    for s in range(prob.S):
        n = int(prob.img_hw[s, 0] * prob.img_hw[s, 1])
        cand_tok += list(range(int(prob.img_start[s]), int(prob.img_start[s]) + n))
    lse = [[None] * T for _ in range(hq)]
    mass = [mpmath.mpf(0)] * len(cand_tok)
    for h in range(hq):
        g = h // rep
        for i in range(T):
            logits = {}
            for j in range(T):
                if visible(prob, i, j):
                    logits[j] = scale * mpmath.fsum(mpmath.mpf(float(q[i, h, t])) *
                                                    mpmath.mpf(float(k[j, g, t])) for t in range(d))
            if not logits:
                continue
            L = mpmath.log(mpmath.fsum(mpmath.exp(v) for v in logits.values()))
            lse[h][i] = L
            for c, j in enumerate(cand_tok):
                if j in logits:
                    mass[c] += mpmath.exp(logits[j] - L)
    return lse, mass


@pytest.mark.parametrize("mask", ["full", "causal", "blockdiag"])
def test_mpmath_bruteforce_tiny(mask):
    rng = np.random.default_rng(11)
    if mask == "blockdiag":
        reqs = [(7, [(0, 1, 3), (3, 2, 2)])]
    else:
        reqs = [(5, [(1, 1, 3)]), (3, [(0, 1, 2)])]
    T = sum(r[0] for r in reqs)
    q = rng.standard_normal((T, 2, 4)) * 1.5
    k = rng.standard_normal((T, 1, 4)) * 1.5
    prob = handmade(reqs, q, k, mask)
    lse, mass = oracle.attention_stats(prob)
    ref_lse, ref_mass = mp_reference(prob)
    for h in range(2):
        for i in range(T):
            if ref_lse[h][i] is not None:
                assert abs(lse[h, i] - float(ref_lse[h][i])) <= 1e-12 * max(1, abs(lse[h, i]))
    for c in range(prob.N):
        assert abs(mass[c] - float(ref_mass[c])) <= 1e-12 * max(1.0, float(ref_mass[c]))


# ---------------------------------------------------------------------------
# The row-at-a-time LSE (``lse_rows``), the checker of the GPU LSE at sizes
# where the full oracle is too slow: pinned to brute force, to the zero-key
# closed form and to planted mistakes of its own, independently of
# ``attention_stats``.
# ---------------------------------------------------------------------------

LSE_ROWS_LAYOUTS = {
    # two requests, a text prefix, text between images and after them
    "full": [(9, [(1, 1, 3), (5, 1, 2)]), (5, [(0, 2, 2)])],
    "causal": [(9, [(1, 1, 3), (5, 1, 2)]), (5, [(0, 2, 2)])],
    # every token inside an image; images of unequal sizes in two requests
    "blockdiag": [(7, [(0, 1, 3), (3, 2, 2)]), (6, [(0, 2, 3)])],
}


@pytest.mark.parametrize("mask", ["full", "causal", "blockdiag"])
def test_lse_rows_mpmath_bruteforce_gqa(mask):
    """Every row of a two-request layout with GQA (6 query heads on 2 KV
    heads, so a wrong head mapping reads the other KV head) against the
    50-digit brute force, whose visibility comes from the mask's wording."""
    rng = np.random.default_rng(12)
    reqs = LSE_ROWS_LAYOUTS[mask]
    T = sum(r[0] for r in reqs)
    q = rng.standard_normal((T, 6, 4)) * 1.5
    k = rng.standard_normal((T, 2, 4)) * 1.5
    prob = handmade(reqs, q, k, mask)
    got = oracle.lse_rows(prob, list(range(T)))
    ref_lse, _ = mp_reference(prob)
    for h in range(6):
        for i in range(T):
            assert ref_lse[h][i] is not None
            assert abs(got[h, i] - float(ref_lse[h][i])) <= 1e-12 * max(1.0, abs(got[h, i])), (h, i)


@pytest.mark.parametrize("mask", ["full", "causal", "blockdiag"])
def test_lse_rows_zero_keys_count_visible(mask):
    """Zero keys make every visible logit 0, so LSE_i = log(number of keys row
    i sees): the request length (full), the position in the request plus one
    (causal) or the image size (block-diagonal).  A wrong key range under any
    mask changes the count."""
    reqs = {"full": [(40, [(3, 4, 5)]), (23, [(2, 3, 3)]), (7, [])],
            "causal": [(40, [(3, 4, 5)]), (23, [(2, 3, 3)]), (7, [])],
            "blockdiag": [(20, [(0, 4, 5)]), (9, [(0, 3, 3)]), (30, [(0, 2, 3), (6, 4, 6)])]}[mask]
    prob = make_problem("zero_k_" + mask, reqs, 4, 2, 64, "f32", mask, 1.0, 13, ratios=0.5)
    prob.k = torch.zeros_like(prob.k)
    T = prob.T
    got = oracle.lse_rows(prob, list(range(T)))
    want = np.empty(T)
    for b in range(prob.B):
        lo, hi = int(prob.cu_seqlens[b]), int(prob.cu_seqlens[b + 1])
        for t in range(lo, hi):
            want[t] = (hi - lo) if mask == "full" else (t - lo + 1)
    if mask == "blockdiag":
        for s in range(prob.S):
            n = int(prob.img_hw[s, 0] * prob.img_hw[s, 1])
            want[prob.img_start[s]:prob.img_start[s] + n] = n
    np.testing.assert_allclose(got, np.broadcast_to(np.log(want), got.shape), rtol=0, atol=1e-13)


def test_lse_rows_sampled_rows_and_repeated_heads():
    """Sampled rows of a GQA problem equal the same rows of the problem with
    its K heads repeated (MHA), and a row's value does not depend on which
    other rows are asked for."""
    prob = random_small(14, "causal", dtype="bf16", hq=8, hkv=2, d=64, n_req=3)
    rows = [0, 5, prob.T // 2, prob.T - 1]
    a = oracle.lse_rows(prob, rows)
    mha = random_small(14, "causal", dtype="bf16", hq=8, hkv=2, d=64, n_req=3)
    mha.k = prob.k.repeat_interleave(4, dim=1)
    b = oracle.lse_rows(mha, rows)
    np.testing.assert_array_equal(a, b)
    c = oracle.lse_rows(prob, rows[::-1])[:, ::-1]
    np.testing.assert_array_equal(a, c)


def _lse_rows_variant(kind):
    """A copy of the row-at-a-time LSE with one planted mistake."""
    def f(prob, tokens, scale=None):
        q64, k64 = O.to_f64(prob.q), O.to_f64(prob.k)
        hq, hkv, d = q64.shape[1], k64.shape[1], q64.shape[2]
        rep = hq // hkv
        scale = O.problem_scale(prob, d) if scale is None else scale
        segs = O.attention_segments(prob)
        if kind == "blockdiag_as_request":
            segs = [(int(prob.cu_seqlens[b]), int(prob.cu_seqlens[b + 1])) + s[2:]
                    for b in range(prob.B) for s in segs[:1]]
        out = np.full((hq, len(tokens)), np.nan)
        for col, t in enumerate(tokens):
            for lo, hi, *_ in segs:
                if lo <= t < hi:
                    kend = (t if kind == "causal_off_by_one" else t + 1) if prob.mask == "causal" else hi
                    kend = max(kend, lo + 1)
                    for h in range(hq):
                        g = h % hkv if kind == "gqa_modulo" else h // rep
                        z = scale * (k64[lo:kend, g, :] @ q64[t, h, :])
                        m = z.max()
                        out[h, col] = m + np.log(np.exp(z - m).sum())
        return out
    return f


@pytest.mark.parametrize("kind", ["causal_off_by_one", "gqa_modulo", "blockdiag_as_request"])
def test_lse_rows_planted_mistakes_are_caught(kind, monkeypatch):
    monkeypatch.setattr(oracle, "lse_rows", _lse_rows_variant(kind))
    caught = 0
    for check in ([lambda m=m: test_lse_rows_mpmath_bruteforce_gqa(m) for m in ("full", "causal", "blockdiag")] +
                  [lambda m=m: test_lse_rows_zero_keys_count_visible(m) for m in ("causal", "blockdiag")]):
        try:
            check()
        except AssertionError:
            caught += 1
    assert caught >= 1, kind


def test_fp8_decoder_matches_format():
    """OCP E4M3: every byte code against torch's float8_e4m3fn widening, and
    the format's landmarks (largest finite 448, smallest normal 2^-6, smallest
    subnormal 2^-9, NaN codes, signed zero)."""
    codes = np.arange(256, dtype=np.uint8)
    mine = O.fp8_e4m3_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    assert np.array_equal(mine[~np.isnan(mine)], ref[~np.isnan(ref)])
    assert mine[0x7E] == 448.0 and mine[0xFE] == -448.0
    assert mine[0x08] == 2.0 ** -6 and mine[0x01] == 2.0 ** -9 and mine[0x07] == 7 * 2.0 ** -9
    assert np.isnan(mine[0x7F]) and np.isnan(mine[0xFF]) and np.isnan(mine).sum() == 2
    assert mine[0x80] == 0.0 and math.copysign(1.0, mine[0x80]) == -1.0
    assert mine[0x38] == 1.0 and mine[0x3C] == 1.5


def test_rope_positions_hand_example():
    """The rotary-position reading worked by hand: request A = 3 text tokens,
    a 2x3 image, 2 text tokens; request B = a 1x4 image, 1 text token."""
    prob = handmade([(11, [(3, 2, 3)]), (5, [(0, 1, 4)])], np.zeros((16, 1, 4)), np.zeros((16, 1, 4)),
                    "causal")
    want = [(0, 0, 0), (1, 1, 1), (2, 2, 2),
            (3, 3, 3), (3, 3, 4), (3, 3, 5), (3, 4, 3), (3, 4, 4), (3, 4, 5),
            (6, 6, 6), (7, 7, 7),
            (0, 0, 0), (0, 0, 1), (0, 0, 2), (0, 0, 3), (4, 4, 4)]
    assert np.array_equal(O.rope_positions(prob), np.array(want))
    keep = np.array([1, 0, 1, 1, 0, 1, 0, 1, 1, 0], np.uint8)
    comp = O.compact(prob, keep)
    assert np.array_equal(comp["positions"], np.array(want)[comp["token_idx"]])
    assert [tuple(x) for x in comp["positions"][3:7]] == [(3, 3, 3), (3, 3, 5), (3, 4, 3), (3, 4, 5)]


def test_rope_positions_structure_random_layouts():
    """Every image: one t for all its tokens, h - t = row, w - t = col; the
    next token after an image sits max(rows, cols) past the image's t; text
    tokens step by one."""
    for seed in range(4):
        p = random_small(300 + seed, "causal", dtype="f32", n_req=3)
        pos = O.rope_positions(p)
        assert np.all(pos >= 0)
        img_of = np.full(p.T, -1)
        for s in range(p.S):
            rows, cols = p.img_hw[s]
            t0 = p.img_start[s]
            blk = pos[t0:t0 + rows * cols]
            assert np.all(blk[:, 0] == blk[0, 0])
            r, c = np.divmod(np.arange(rows * cols), cols)
            assert np.array_equal(blk[:, 1] - blk[:, 0], r) and np.array_equal(blk[:, 2] - blk[:, 0], c)
            img_of[t0:t0 + rows * cols] = s
            nxt = t0 + rows * cols
            b = np.searchsorted(p.cu_seqlens, t0, side="right") - 1
            if nxt < p.cu_seqlens[b + 1]:
                assert pos[nxt, 0] == blk[0, 0] + max(rows, cols)
        for b in range(p.B):
            lo = p.cu_seqlens[b]
            if lo < p.cu_seqlens[b + 1]:
                assert pos[lo, 0] == 0
            for t in range(lo + 1, p.cu_seqlens[b + 1]):
                if img_of[t] < 0 and img_of[t - 1] < 0:
                    assert tuple(pos[t]) == (pos[t - 1, 0] + 1,) * 3


@pytest.mark.parametrize("mask", ["full", "causal"])
def test_fp8_problem_against_bruteforce(mask):
    """An fp8 problem from the generator (per-tensor factors folded into its
    softmax scale): the oracle's LSE and mass against 50-digit brute force
    with that scale."""
    reqs = [(6, [(1, 1, 3)]), (4, [(0, 2, 1)])]
    prob = make_problem("fp8_tiny", reqs, 2, 1, 4, "fp8", mask, 1.0, 21, ratios=0.5, emb_dim=4)
    assert prob.q.dtype == torch.float8_e4m3fn and prob.softmax_scale is not None
    assert float(prob.q.to(torch.float32).abs().max()) == 448.0
    lse, mass = oracle.attention_stats(prob)
    ref_lse, ref_mass = mp_reference(prob, scale=prob.softmax_scale)
    for h in range(2):
        for i in range(prob.T):
            if ref_lse[h][i] is not None:
                assert abs(lse[h, i] - float(ref_lse[h][i])) <= 1e-12 * max(1, abs(lse[h, i]))
    for c in range(prob.N):
        assert abs(mass[c] - float(ref_mass[c])) <= 1e-12 * max(1.0, float(ref_mass[c]))


@pytest.mark.parametrize("mask", ["full", "causal"])
def test_attention_forward_matches_torch_sdpa(mask):
    """One request: the forward pass equals torch's scaled_dot_product_attention
    in float64 (GQA heads expanded), and its LSE equals attention_stats'."""
    p = make_problem("fwd", [(90, [(10, 6, 9)])], 4, 2, 32, "f32", mask, 1.0, 41, ratios=0.5)
    o, lse = oracle.attention_forward(p)
    q = torch.from_numpy(O.to_f64(p.q)).permute(1, 0, 2)
    k = torch.from_numpy(O.to_f64(p.k)).repeat_interleave(2, dim=1).permute(1, 0, 2)
    v = torch.from_numpy(O.to_f64(p.v)).repeat_interleave(2, dim=1).permute(1, 0, 2)
    want = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=(mask == "causal"))
    np.testing.assert_allclose(o, want.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-13)
    lse2, _ = oracle.attention_stats(p)
    np.testing.assert_allclose(lse, lse2, rtol=1e-14)


def test_forward_rows_equal_attention_forward():
    """The row-at-a-time forward agrees with the blocked one (two code paths)."""
    for mask in ("full", "causal", "blockdiag"):
        p = random_small(43, mask, dtype="bf16", hq=4, hkv=2, d=64, n_req=2)
        o, _ = oracle.attention_forward(p)
        rows = np.arange(0, p.T, 7)
        np.testing.assert_allclose(oracle.forward_rows(p, rows), o[rows], rtol=1e-12, atol=1e-14)


def test_attention_forward_invariants():
    """Rows of P sum to one (V = 1 gives O = 1), and with V the identity on
    the keys O is P itself, whose candidate columns summed over rows and heads
    give attention_stats' mass (two separate code paths)."""
    p = random_small(42, "causal", dtype="f32", hq=2, hkv=1, d=64, n_req=1)
    T = p.T
    ones = torch.ones((T, 1, 64), dtype=torch.float32)
    o, _ = oracle.attention_forward(p, v=ones)
    np.testing.assert_allclose(o, 1.0, rtol=1e-13)
    eye = torch.zeros((T, 1, T), dtype=torch.float32)
    eye[torch.arange(T), 0, torch.arange(T)] = 1.0
    pq = make_problem("fwd_eye", [(T, [(int(p.img_start[s]), int(p.img_hw[s, 0]), int(p.img_hw[s, 1]))
                                       for s in range(p.S)])], 2, 1, 64, "f32", "causal", 1.0, 42,
                      ratios=0.5)
    pq.q, pq.k = p.q, p.k
    o, _ = oracle.attention_forward(pq, v=eye, scale=1 / math.sqrt(64))
    _, mass = oracle.attention_stats(pq)
    cand_tok = np.concatenate([np.arange(pq.img_start[s], pq.img_start[s] + pq.img_hw[s, 0] * pq.img_hw[s, 1])
                               for s in range(pq.S)])
    np.testing.assert_allclose(o.sum(axis=(0, 1))[cand_tok], mass, rtol=1e-12)


def test_two_keys_logistic_closed_form():
    """Full mask, two tokens: P(i -> key 0) = sigmoid(s_i0 - s_i1)."""
    rng = np.random.default_rng(3)
    d = 8
    q = rng.standard_normal((2, 3, d))
    k = rng.standard_normal((2, 3, d))
    prob = handmade([(2, [(0, 1, 2)])], q, k, "full")
    q64, k64 = O.to_f64(prob.q), O.to_f64(prob.k)
    _, mass = oracle.attention_stats(prob)
    want = np.zeros(2)
    for h in range(3):
        for i in range(2):
            s0 = q64[i, h] @ k64[0, h] / math.sqrt(d)
            s1 = q64[i, h] @ k64[1, h] / math.sqrt(d)
            p0 = 1.0 / (1.0 + math.exp(-(s0 - s1)))
            want += [p0, 1.0 - p0]
    np.testing.assert_allclose(mass, want, rtol=1e-13)


def harmonic(m):
    return sum(1.0 / i for i in range(1, m + 1))


def test_zero_keys_full_is_uniform():
    n, hq = 37, 3
    q = np.random.default_rng(0).standard_normal((n, hq, 16))
    prob = handmade([(n, [(0, 1, n)])], q, np.zeros((n, 1, 16)), "full")
    _, mass = oracle.attention_stats(prob)
    np.testing.assert_allclose(mass, hq, rtol=1e-13)
    np.testing.assert_allclose(oracle.scores(prob, mass), 1.0 / n, rtol=1e-13)


def test_zero_keys_causal_harmonic():
    """Row i sees i+1 keys uniformly: mass_j = Hq * (H_n - H_j), j 0-based."""
    n, hq = 41, 2
    q = np.random.default_rng(1).standard_normal((n, hq, 16))
    prob = handmade([(n, [(0, 1, n)])], q, np.zeros((n, 2, 16)), "causal")
    _, mass = oracle.attention_stats(prob)
    want = [hq * (harmonic(n) - harmonic(j)) for j in range(n)]
    np.testing.assert_allclose(mass, want, rtol=1e-13)


def test_zero_keys_causal_text_prefix_scale_zero():
    """scale = 0 is the same as zero keys; with a text prefix of p tokens the
    candidate at token t gets Hq * (H_n - H_t)."""
    n, p, hq = 30, 7, 2
    rng = np.random.default_rng(2)
    q = rng.standard_normal((n, hq, 8))
    k = rng.standard_normal((n, 1, 8))
    prob = handmade([(n, [(p, 2, 9)])], q, k, "causal")
    _, mass = oracle.attention_stats(prob, scale=0.0)
    want = [hq * (harmonic(n) - harmonic(t)) for t in range(p, p + 18)]
    np.testing.assert_allclose(mass, want, rtol=1e-13)


def test_zero_keys_blockdiag_unequal_images():
    sizes = [(2, 3), (5, 7), (1, 4)]
    imgs, off = [], 0
    for h, w in sizes:
        imgs.append((off, h, w))
        off += h * w
    hq = 4
    q = np.random.default_rng(4).standard_normal((off, hq, 8))
    prob = handmade([(off, imgs)], q, np.zeros((off, 4, 8)), "blockdiag")
    _, mass = oracle.attention_stats(prob)
    np.testing.assert_allclose(mass, hq, rtol=1e-13)


@pytest.mark.parametrize("mask", ["full", "causal", "blockdiag"])
def test_mass_conservation_all_candidates(mask):
    """Every token a candidate and the LSE computed: sum_c mass = Hq * n_b."""
    rng = np.random.default_rng(5)
    if mask == "blockdiag":
        reqs = [(60, [(0, 5, 6), (30, 3, 10)])]
    else:
        reqs = [(48, [(0, 6, 8)]), (35, [(0, 5, 7)])]
    T = sum(r[0] for r in reqs)
    prob = handmade(reqs, rng.standard_normal((T, 4, 16)) * 2,
                    rng.standard_normal((T, 2, 16)) * 2, mask)
    _, mass = oracle.attention_stats(prob)
    for b, (lo, hi) in enumerate(oracle.pool_bounds(prob)):
        n_b = prob.cu_seqlens[b + 1] - prob.cu_seqlens[b]
        assert abs(mass[lo:hi].sum() - 4 * n_b) <= 1e-11 * n_b
    sc = oracle.scores(prob, mass)
    for lo, hi in oracle.pool_bounds(prob):
        assert abs(sc[lo:hi].sum() - 1.0) < 1e-12


def test_single_dominant_key():
    """k* = alpha * u with q_i . u > 0 for all rows: it is the top-1 key, each
    row's probability obeys 1/(1 + (n-1) e^{-delta_i}) <= P, and for a large
    alpha the mass tends to Hq * (rows that see k*)."""
    rng = np.random.default_rng(6)
    n, hq, d, j = 50, 2, 16, 20
    u = np.zeros(d)
    u[0] = 1.0
    q = rng.standard_normal((n, hq, d)) * 0.3
    q[:, :, 0] = np.abs(q[:, :, 0]) + 1.0
    k = rng.standard_normal((n, 1, d)) * 0.3
    for alpha, check_limit in ((20.0, False), (4000.0, True)):
        kk = k.copy()
        kk[j, 0] = alpha * u
        prob = handmade([(n, [(0, 5, 10)])], q, kk, "causal")
        lse, mass = oracle.attention_stats(prob)
        sc = oracle.scores(prob, mass)
        assert int(np.argmax(sc)) == j
        q64, k64 = O.to_f64(prob.q), O.to_f64(prob.k)
        for h in range(hq):
            for i in range(j, n):
                s = q64[i, h] @ k64[: i + 1, 0].T / math.sqrt(d)
                delta = s[j] - np.max(np.delete(s, j))
                p = math.exp(s[j] - lse[h, i])
                assert p >= 1.0 / (1.0 + i * math.exp(-delta)) - 1e-12
        if check_limit:
            assert abs(mass[j] - hq * (n - j)) < 1e-9


def test_gqa_equals_repeated_mha():
    p = make_problem("g", [(90, [(10, 5, 12)])], 8, 2, 32, "f32", "causal", 1.0, 7, ratios=0.5)
    _, mass_g = oracle.attention_stats(p)
    k_rep = p.k.repeat_interleave(4, dim=1)
    p2 = make_problem("m", [(90, [(10, 5, 12)])], 8, 8, 32, "f32", "causal", 1.0, 7, ratios=0.5)
    p2.q, p2.k = p.q, k_rep
    _, mass_m = oracle.attention_stats(p2)
    np.testing.assert_allclose(mass_g, mass_m, rtol=1e-12)


def test_permutation_equivariance_full_mask():
    p = make_problem("p", [(64, [(0, 8, 8)])], 3, 3, 16, "f32", "full", 1.0, 8, ratios=0.5)
    _, mass = oracle.attention_stats(p)
    perm = np.random.default_rng(9).permutation(64)
    p.q, p.k = p.q[perm], p.k[perm]
    _, mass_p = oracle.attention_stats(p)
    np.testing.assert_allclose(mass_p, mass[perm], rtol=1e-12)


def test_supplied_lse_identity_and_shift():
    """Supplied LSE equal to the computed one gives the same mass; LSE + delta
    scales every mass by exp(-delta)."""
    p = random_small(12, "causal", dtype="f32")
    lse, mass = oracle.attention_stats(p)
    _, mass_same = oracle.attention_stats(p, lse_in=lse)
    np.testing.assert_array_equal(mass_same, mass)
    delta = 0.37
    _, mass_shift = oracle.attention_stats(p, lse_in=lse + delta)
    np.testing.assert_allclose(mass_shift, mass * math.exp(-delta), rtol=1e-13)


def test_supplied_lse_nonfinite_row_reaches_only_visible_pairs():
    """A supplied LSE of -inf for one row makes every mass that row reaches
    +inf and leaves the masses of the candidates it cannot see (causal: later
    tokens, or other requests) exactly as with that row contributing nothing
    (LSE = +inf): masked pairs add zero whatever the row's LSE."""
    p = random_small(15, "causal", dtype="f32", n_req=2)
    lse, _ = oracle.attention_stats(p)
    b = 0
    lo, hi = int(p.cu_seqlens[b]), int(p.cu_seqlens[b + 1])
    t = lo + (hi - lo) // 2
    h = 1 % p.hq
    neg, pos = lse.copy(), lse.copy()
    neg[h, t], pos[h, t] = -np.inf, np.inf
    _, m_neg = oracle.attention_stats(p, lse_in=neg)
    _, m_pos = oracle.attention_stats(p, lse_in=pos)
    # token of every candidate
    tok = np.concatenate([np.arange(p.img_start[s], p.img_start[s] + p.img_hw[s, 0] * p.img_hw[s, 1])
                          for s in range(p.S)])
    seen = (tok <= t) & (tok >= lo)
    assert seen.any() and (~seen).any()
    assert np.all(np.isposinf(m_neg[seen]))
    np.testing.assert_array_equal(m_neg[~seen], m_pos[~seen])
    assert np.all(np.isfinite(m_pos))


def test_lse_and_softmax_match_library_routines():
    """Full mask, one request: the LSE is scipy's logsumexp of the logits and
    the mass is the column sum of torch's float64 softmax."""
    p = make_problem("l", [(70, [(0, 7, 10)])], 2, 2, 24, "f32", "full", 1.5, 10, ratios=0.5)
    lse, mass = oracle.attention_stats(p)
    q64 = torch.from_numpy(O.to_f64(p.q))
    k64 = torch.from_numpy(O.to_f64(p.k))
    want_mass = np.zeros(70)
    for h in range(2):
        logits = (q64[:, h] @ k64[:, h].T / math.sqrt(24)).numpy()
        np.testing.assert_allclose(lse[h], scipy.special.logsumexp(logits, axis=1), rtol=1e-13)
        want_mass += torch.softmax(torch.from_numpy(logits), dim=1).sum(0).numpy()
    np.testing.assert_allclose(mass, want_mass, rtol=1e-12)


def test_named_workloads_shapes():
    """Sizes of the five workloads (cheap: no scoring)."""
    p1 = make_config(1)
    assert (p1.T, p1.hq, p1.d, p1.N, len(p1.dominant)) == (256, 4, 64, 256, 8)
    p3 = make_config(3)
    assert (p3.T, p3.S, p3.N, p3.d) == (30720, 30, 30720, 80)
    assert 15 * 10 <= len(p3.dominant) <= 15 * 20
    p4 = make_config(4)
    assert (p4.T, p4.hq, p4.hkv, p4.N) == (16384, 64, 8, 15000)
    p5 = make_config(5)
    assert p5.B == 8 and all(2048 <= n <= 8192 for n in np.diff(p5.cu_seqlens))
    for b in range(8):
        lo, hi = oracle.pool_bounds(p5)[b]
        assert hi - lo <= p5.cu_seqlens[b + 1] - p5.cu_seqlens[b] - 1
        assert 0.5 <= p5.keep_ratio[b] < 0.9


# ---------------------------------------------------------------------------
# Budget and top-k.
# ---------------------------------------------------------------------------

def read_golden_counts():
    rows = []
    with open(os.path.join(GOLDEN, "p1_token_counts.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                name, vis, text, r, printed = line.split()
                rows.append((name, int(vis), int(text), float(r), int(printed)))
    return rows


def test_budget_rule_reproduces_litevlm_table():
    rows = read_golden_counts()
    assert len(rows) == 5
    for name, vis, text, r, printed in rows:
        assert oracle.budget_k(r, vis) + text == printed, name


def test_budget_rule_named_workloads_and_edges():
    assert oracle.budget_k(0.4, 256) == 102
    assert oracle.budget_k(0.8, 3072) == 2457
    assert oracle.budget_k(0.6, 30720) == 18432
    assert oracle.budget_k(0.6, 15000) == 9000
    assert oracle.budget_k(0.57, 100) == 57      # 0.57 * 100 = 56.999... in binary64
    assert oracle.budget_k(0.29, 100) == 29
    assert oracle.budget_k(0.0, 10) == 0 and oracle.budget_k(1.0, 10) == 10
    assert oracle.budget_k(-3.0, 10) == 0 and oracle.budget_k(7.0, 10) == 10
    with pytest.raises(ValueError):
        oracle.budget_k(float("nan"), 10)


def brute_keep(score, k):
    s = np.where(np.isfinite(score), score, -np.inf)
    n = len(s)
    keep = np.zeros(n, np.uint8)
    for j in range(n):
        rank = sum(1 for l in range(n) if s[l] > s[j] or (s[l] == s[j] and l < j))
        keep[j] = rank < k
    return keep


def test_topk_matches_brute_force_rank():
    rng = np.random.default_rng(13)
    p = random_small(13, "full", dtype="f32", n_req=3)
    for trial in range(5):
        sc = rng.integers(0, 12, size=p.N).astype(np.float64) / 7.0  # many exact ties
        if trial == 3:
            sc[::5] = np.nan
            sc[1] = np.inf
            sc[2] = -np.inf
        keep, ks = oracle.topk(p, sc)
        for b, (lo, hi) in enumerate(oracle.pool_bounds(p)):
            np.testing.assert_array_equal(keep[lo:hi], brute_keep(sc[lo:hi], ks[b]))
            assert keep[lo:hi].sum() == ks[b]


def test_topk_k_zero_and_all_and_ties():
    p = random_small(14, "full", dtype="f32", n_req=1)
    n = p.N
    sc = np.ones(n)
    keep, _ = oracle.topk(p, sc, ratios=[0.0])
    assert keep.sum() == 0
    keep, _ = oracle.topk(p, sc, ratios=[1.0])
    assert keep.sum() == n
    keep, ks = oracle.topk(p, sc, ratios=[0.5])
    assert keep[: ks[0]].all() and not keep[ks[0]:].any()


# ---------------------------------------------------------------------------
# Input-dependent (mass) budget.
# ---------------------------------------------------------------------------

def test_mass_units_hand_values():
    sc = np.array([0.25, 1.0, 2.0, -1.0, np.nan, np.inf, 1e-12, 0.0, -0.0, 0.5 + 2.0 ** -40], np.float32)
    m = oracle.mass_units(sc)
    assert m.dtype == np.uint64
    # 0.25 -> 2^30; 1 and 2 (clamped) -> 2^32; negative, NaN, inf, zeros -> 0;
    # 1e-12 * 2^32 = 0.0043 -> 0; fp32 rounds 0.5 + 2^-40 to 0.5 -> 2^31.
    assert list(m) == [2 ** 30, 2 ** 32, 2 ** 32, 0, 0, 0, 0, 0, 0, 2 ** 31]


def _brute_kstar(sc, tau):
    """Fewest candidates of ANY subset whose integer mass reaches the target
    (the top-ranked subset of that size is the heaviest, so this equals k*)."""
    m = [int(x) for x in oracle.mass_units(sc)]
    total = sum(m)
    target = min(total, math.ceil((tau * float(total)) * (1.0 - 1e-12)))
    if target == 0:
        return 0
    n = len(m)
    for size in range(1, n + 1):
        for mask in range(1 << n):
            if bin(mask).count("1") == size and sum(m[i] for i in range(n) if mask >> i & 1) >= target:
                return size
    raise AssertionError("target above total")


def test_mass_budget_matches_subset_brute_force():
    rng = np.random.default_rng(21)
    for trial in range(60):
        n = int(rng.integers(1, 9))
        sc = (rng.integers(0, 6, size=n) / rng.integers(5, 40)).astype(np.float32)
        if trial % 7 == 3:
            sc[rng.integers(0, n)] = np.nan
        if trial % 11 == 5:
            sc[rng.integers(0, n)] = -0.5
        tau = float(rng.choice([0.0, 0.1, 0.25, 0.5, 0.6, 0.9, 0.999, 1.0, rng.random()]))
        k = oracle.mass_budget_k(sc, tau, 0.0, 1.0)
        assert k == _brute_kstar(sc, tau), (sc, tau)


def test_mass_budget_uniform_closed_form():
    # n equal scores: k* = tau * n exactly for decimal tau on the grid 1/n.
    for n in (4, 10, 20, 100):
        sc = np.full(n, 1.0 / n, np.float32)
        for i in range(n + 1):
            assert oracle.mass_budget_k(sc, i / n, 0.0, 1.0) == i, (n, i)


def test_mass_budget_dominant_and_edges():
    sc = np.array([0.01] * 5 + [0.9] + [0.01] * 5, np.float32)
    assert oracle.mass_budget_k(sc, 0.5, 0.0, 1.0) == 1  # the dominant token alone
    assert oracle.mass_budget_k(sc, 0.0, 0.0, 1.0) == 0
    assert oracle.mass_budget_k(sc, 1.0, 0.0, 1.0) == 11  # every positive-mass candidate
    assert oracle.mass_budget_k(sc, 0.5, 0.4, 1.0) == 4  # floor(0.4 * 11) lower bound
    assert oracle.mass_budget_k(sc, 1.0, 0.0, 0.5) == 5  # floor(0.5 * 11) upper bound
    zero = np.zeros(7, np.float32)
    assert oracle.mass_budget_k(zero, 0.9, 0.0, 1.0) == 0  # no mass: nothing needed
    assert oracle.mass_budget_k(zero, 0.9, 0.3, 1.0) == 2
    assert oracle.mass_budget_k(np.zeros(0, np.float32), 0.5, 0.0, 1.0) == 0
    with_zero = np.array([0.5, 0.0, 0.25, 0.0], np.float32)
    assert oracle.mass_budget_k(with_zero, 1.0, 0.0, 1.0) == 2  # zero-mass candidates never needed
    for bad in [(float("nan"), 0.0, 1.0), (0.5, float("nan"), 1.0), (0.5, 0.6, 0.5)]:
        with pytest.raises(ValueError):
            oracle.mass_budget_k(sc, *bad)


def test_mass_budget_monotone_and_keeps_top_k():
    rng = np.random.default_rng(22)
    p = random_small(22, "full", dtype="f32", n_req=3)
    sc = rng.gamma(0.5, size=p.N) / p.N
    sc[::9] = sc[1::9]  # some exact ties
    prev = None
    for tau in np.linspace(0.0, 1.0, 21):
        keep, ks = oracle.mass_budget(p, sc, [tau] * p.B, [0.1] * p.B, [0.95] * p.B)
        for b, (lo, hi) in enumerate(oracle.pool_bounds(p)):
            n = hi - lo
            assert oracle.budget_k(0.1, n) <= ks[b] <= oracle.budget_k(0.95, n)
            np.testing.assert_array_equal(keep[lo:hi], brute_keep(sc[lo:hi], ks[b]))
        if prev is not None:
            assert (ks >= prev).all()
        prev = ks


# ---------------------------------------------------------------------------
# Compaction.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("mask", ["full", "causal", "blockdiag"])
def test_compaction_numpy_equals_loop_and_invariants(mask):
    p = random_small(21, mask, dtype="f32", n_req=3)
    rng = np.random.default_rng(0)
    keep = (rng.random(p.N) < 0.6).astype(np.uint8)
    a = oracle.compact(p, keep, p.emb.numpy())
    b = oracle.compact_loop(p, keep)
    for key in ("token_idx", "spatial", "cu_seqlens", "img_counts"):
        np.testing.assert_array_equal(a[key], b[key])
    text = p.T - p.N
    assert len(a["token_idx"]) == text + keep.sum()
    for r in range(p.B):
        seg = a["token_idx"][a["cu_seqlens"][r]:a["cu_seqlens"][r + 1]]
        assert np.all(np.diff(seg) > 0)
        assert np.all((seg >= p.cu_seqlens[r]) & (seg < p.cu_seqlens[r + 1]))
    np.testing.assert_array_equal(a["emb"], p.emb.numpy()[a["token_idx"]])
    for s in range(p.S):
        rows = a["spatial"][a["spatial"][:, 0] == s]
        h, w = p.img_hw[s]
        assert len(rows) == a["img_counts"][s]
        assert np.all((rows[:, 1] < h) & (rows[:, 2] < w))


# ---------------------------------------------------------------------------
# Planted mistakes: each variant breaks one step of the arithmetic on the CPU
# and at least one pin above must notice.
# ---------------------------------------------------------------------------

def _variant_segment_head(kind):
    def f(q64, k64, seg, h, g, scale, causal, lse_given):
        lo, hi, _b, loc, _glob = seg
        n = hi - lo
        Qs, Ks = q64[lo:hi, h, :], k64[lo:hi, g, :]
        S = (1.0 if kind == "no_scale" else scale) * (Qs @ Ks.T)
        if causal:
            tri = np.arange(n)[None, :] <= np.arange(n)[:, None]
            if kind == "causal_transposed":
                tri = tri.T
            S = np.where(tri, S, -np.inf)
        m = S.max(axis=1)
        lse_rows = m + np.log(np.exp(S - m[:, None]).sum(axis=1))
        if lse_given is not None:
            lse_rows = lse_given[lo:hi]
        P = np.exp(S - lse_rows[:, None])
        mass = (P.sum(axis=1) if kind == "row_sums" else P.sum(axis=0))[loc]
        return lse_rows, mass
    return f


@pytest.mark.parametrize("kind", ["no_scale", "causal_transposed", "row_sums"])
def test_planted_mistakes_are_caught(kind, monkeypatch):
    monkeypatch.setattr(O, "_segment_head", _variant_segment_head(kind))
    caught = 0
    for check in (test_two_keys_logistic_closed_form, test_zero_keys_causal_harmonic,
                  lambda: test_mass_conservation_all_candidates("causal"),
                  lambda: test_single_dominant_key(),
                  lambda: test_mpmath_bruteforce_tiny("causal")):
        try:
            check()
        except AssertionError:
            caught += 1
    assert caught >= 1, kind
