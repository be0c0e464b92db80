"""GPU parity of the attention forward (tsel_attention_fwd) against the oracle.

Tolerances (written here):

* LSE: |gpu - oracle| <= 1e-4 (natural log units), as for tsel_lse.
* O: |gpu - oracle| <= eps * (max|V| + |oracle|) with eps = 2^-8 (bf16) or
  2^-10 (f16).  The kernel feeds the probabilities to the matrix unit in the
  input type (relative rounding 2^-9 for bf16, 2^-11 for f16 per term) while
  their sum stays fp32, so each output value is off by at most that rounding
  times sum_j p_j |v_j| <= max|V|; the output itself is rounded to the input
  type (the |oracle| term).  eps is twice the per-term rounding.
"""
import numpy as np
import pytest
import torch

import attention_score_selection_amd as tsel
import oracle
from workloads import make_config, make_problem, random_medium, random_small

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    tsel.lib()
    return torch.device("cuda:0")


def announce(prob, extra=""):
    print(f"\n[case] forward {prob.name} T={prob.T} Hq={prob.hq} Hkv={prob.hkv} d={prob.d} "
          f"{prob.dtype} {prob.mask} {extra}", flush=True)


def run_fwd(prob, dev, v=None):
    lay = tsel.Layout.from_problem(prob, dev)
    q, k = prob.q.to(dev), prob.k.to(dev)
    vv = (prob.v if v is None else v).to(dev)
    scale = prob.softmax_scale if prob.softmax_scale is not None else 0.0
    out, lse = tsel.tsel_attention_fwd(q, k, vv, lay, prob.mask, scale)
    torch.cuda.synchronize(dev)
    return out.cpu().double().numpy(), lse.cpu().double().numpy()


def check(prob, out, lse, ref_o, ref_lse, v=None, rows=None):
    eps = 2.0 ** -8 if prob.dtype == "bf16" else 2.0 ** -10
    vmax = float((prob.v if v is None else v).double().abs().max())
    o = out if rows is None else out[rows]
    bad = np.abs(o - ref_o) > eps * (vmax + np.abs(ref_o))
    print(f"[check] worst |err| / bound = {np.max(np.abs(o - ref_o) / (eps * (vmax + np.abs(ref_o)))):.3g}, "
          f"LSE max err {np.nanmax(np.abs((lse if rows is None else lse[:, rows]) - ref_lse)):.3g}", flush=True)
    assert not bad.any(), (f"{prob.name}: {bad.sum()} output values off, worst "
                           f"{np.max(np.abs(o - ref_o) - eps * (vmax + np.abs(ref_o))):.3g}")
    l = lse if rows is None else lse[:, rows]
    assert np.nanmax(np.abs(l - ref_lse)) <= 1e-4, f"{prob.name}: LSE off"


SMALL = [("full", "bf16", 4, 4, 64), ("causal", "bf16", 8, 2, 128), ("blockdiag", "bf16", 6, 2, 96),
         ("causal", "f16", 16, 1, 80), ("full", "f16", 3, 3, 96), ("causal", "bf16", 12, 4, 80),
         ("blockdiag", "f16", 4, 4, 128), ("causal", "f16", 32, 2, 64), ("blockdiag", "bf16", 4, 4, 72),
         ("causal", "f16", 8, 2, 72)]


@pytest.mark.parametrize("i", range(len(SMALL)))
def test_forward_small(dev, i):
    mask, dtype, hq, hkv, d = SMALL[i]
    prob = random_small(400 + i, mask, dtype=dtype, hq=hq, hkv=hkv, d=d, n_req=3)
    announce(prob)
    out, lse = run_fwd(prob, dev)
    ref_o, ref_lse = oracle.attention_forward(prob)
    check(prob, out, lse, ref_o, ref_lse)


@pytest.mark.parametrize("mask,dtype,hq,hkv,d,std", [("causal", "bf16", 8, 2, 128, 1.0),
                                                     ("full", "f16", 16, 4, 80, 1.0),
                                                     ("blockdiag", "bf16", 4, 4, 64, 1.0),
                                                     ("causal", "bf16", 8, 8, 128, 2.5),
                                                     ("causal", "f16", 16, 2, 128, 2.5)])
def test_forward_medium(dev, mask, dtype, hq, hkv, d, std):
    """Includes peaked logits (std 2.5: logit spreads of tens) so the running
    maximum moves many times."""
    prob = random_medium(450 + hq + d, mask, dtype=dtype, hq=hq, hkv=hkv, d=d, n_req=2, std=std)
    announce(prob, f"std={std}")
    out, lse = run_fwd(prob, dev)
    ref_o, ref_lse = oracle.attention_forward(prob, workers=oracle.default_workers())
    check(prob, out, lse, ref_o, ref_lse)


def test_forward_lse_matches_oracle_and_identity_values(dev):
    """V = 1 gives O = 1 (rows of P sum to one), within the output rounding."""
    prob = random_small(460, "causal", dtype="bf16", hq=4, hkv=2, d=128, n_req=2)
    ones = torch.ones_like(prob.v)
    announce(prob, "v=1")
    out, lse = run_fwd(prob, dev, v=ones)
    assert np.max(np.abs(out - 1.0)) <= 2.0 ** -8
    _, ref_lse = oracle.attention_forward(prob, v=ones)
    assert np.nanmax(np.abs(lse - ref_lse)) <= 1e-4


@pytest.mark.parametrize("mask,dtype,d", [("causal", "bf16", 80), ("blockdiag", "f16", 128)])
def test_forward_fused_qkv_projection(dev, mask, dtype, d):
    """Q, K and V as views into one fused [T, Hq + 2*Hkv, d] projection, so
    the key and value tiles are copied from rows (Hq + 2*Hkv)*d elements
    apart; d = 80 also has a padded last column group."""
    hq, hkv = 8, 2
    prob = random_medium(463 + d, mask, dtype=dtype, hq=hq, hkv=hkv, d=d, n_req=2)
    announce(prob, "fused qkv")
    qkv = torch.empty((prob.T, hq + 2 * hkv, d), dtype=prob.q.dtype)
    qkv[:, :hq] = prob.q
    qkv[:, hq:hq + hkv] = prob.k
    qkv[:, hq + hkv:] = prob.v
    g = qkv.to(dev)
    q, k, v = g[:, :hq], g[:, hq:hq + hkv], g[:, hq + hkv:]
    lay = tsel.Layout.from_problem(prob, dev)
    scale = prob.softmax_scale if prob.softmax_scale is not None else 0.0
    out, lse = tsel.tsel_attention_fwd(q, k, v, lay, prob.mask, scale)
    torch.cuda.synchronize(dev)
    ref_o, ref_lse = oracle.attention_forward(prob, workers=oracle.default_workers())
    check(prob, out.cpu().double().numpy(), lse.cpu().double().numpy(), ref_o, ref_lse)


@pytest.mark.parametrize("mask,dtype,hq,hkv,d", [("causal", "bf16", 8, 2, 128), ("full", "f16", 4, 4, 80),
                                                 ("blockdiag", "bf16", 6, 3, 72)])
def test_forward_head_major_kv(dev, mask, dtype, hq, hkv, d):
    """K and V stored head-major ([Hkv, T, d]) and passed as [T, Hkv, d] views:
    the token stride is exactly head_dim, so a key or value row ends where the
    next begins, and a ragged last tile's valid rows reach the very end of the
    range its copy may read."""
    prob = random_medium(471 + d, mask, dtype=dtype, hq=hq, hkv=hkv, d=d, n_req=2)
    announce(prob, "head-major k/v")
    k = prob.k.permute(1, 0, 2).contiguous().to(dev).permute(1, 0, 2)
    v = prob.v.permute(1, 0, 2).contiguous().to(dev).permute(1, 0, 2)
    assert k.stride(0) == d and v.stride(0) == d
    lay = tsel.Layout.from_problem(prob, dev)
    scale = prob.softmax_scale if prob.softmax_scale is not None else 0.0
    out, lse = tsel.tsel_attention_fwd(prob.q.to(dev), k, v, lay, prob.mask, scale)
    torch.cuda.synchronize(dev)
    ref_o, ref_lse = oracle.attention_forward(prob, workers=oracle.default_workers())
    check(prob, out.cpu().double().numpy(), lse.cpu().double().numpy(), ref_o, ref_lse)


def test_forward_empty_and_imageless_requests(dev):
    reqs = [(0, []), (37, [(5, 4, 6)]), (0, []), (20, []), (41, [(0, 3, 3), (12, 5, 5)])]
    prob = make_problem("fwd_empties", reqs, 4, 2, 64, "bf16", "causal", 1.0, 461,
                        ratio_range=(0.3, 0.8), emb_dim=8)
    announce(prob)
    out, lse = run_fwd(prob, dev)
    ref_o, ref_lse = oracle.attention_forward(prob)
    check(prob, out, lse, ref_o, ref_lse)


@pytest.mark.parametrize("cfg", [4, 5, 3])
def test_forward_named_workload_sampled_rows(dev, cfg):
    """A named workload at full size (the 16384-token GQA decoder layer, the
    varlen batch in f16, the 30-image block-diagonal workload at d = 80): 24
    sampled rows of every head against the row-at-a-time oracle."""
    prob = make_config(cfg)
    announce(prob)
    out, lse = run_fwd(prob, dev)
    rows = np.linspace(0, prob.T - 1, 24).astype(int)
    ref_o = oracle.forward_rows(prob, rows)
    ref_lse = oracle.lse_rows(prob, rows)
    check(prob, out, lse, ref_o, ref_lse, rows=rows)
