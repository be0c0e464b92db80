"""The whole path captured in a HIP graph and replayed.

No call of the library allocates, copies, sets memory or synchronises: each
enqueues kernels only, and the host computes every size from the layout's
host mirrors, so the path can be captured once and replayed.  Each replay
here follows eager work that changes the inputs in place, and every replay is
compared with an eager run on the same inputs: the kernels are deterministic,
so the results must be identical bit for bit.
"""
import numpy as np
import pytest
import torch

import attention_score_selection_amd as tsel
from workloads import random_medium

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    tsel.lib()
    return torch.device("cuda:0")


def flat(out):
    d = {"lse": out["lse"], "score": out["score"], "keep": out["keep"]}
    d.update({"c_" + k: v for k, v in out["compact"].items()})
    return d


@pytest.mark.parametrize("mask,dtype,hq,hkv,d", [("causal", "bf16", 16, 4, 128), ("blockdiag", "f16", 8, 8, 80)])
def test_graph_replays_match_eager(dev, mask, dtype, hq, hkv, d):
    prob = random_medium(480 + hq, mask, dtype=dtype, hq=hq, hkv=hkv, d=d, n_req=2)
    print(f"\n[case] graph {prob.name} T={prob.T} N={prob.N} {dtype} {mask}", flush=True)
    lay = tsel.Layout.from_problem(prob, dev)
    q, k, emb = prob.q.to(dev), prob.k.to(dev), prob.emb.to(dev)
    ratios = prob.keep_ratio
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):  # warm-up outside the capture
        tsel.select(q, k, lay, mask, ratios, emb=emb)
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize(dev)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        captured = flat(tsel.select(q, k, lay, mask, ratios, emb=emb))
    gen = torch.Generator(device="cpu").manual_seed(481)
    for rep in range(3):
        # Eager work between replays: new inputs in place (same sizes, so the
        # kept counts per pool, fixed by the ratios, do not change).
        q.copy_((torch.randn(q.shape, generator=gen) * prob.std).to(q.dtype))
        k.copy_((torch.randn(k.shape, generator=gen) * prob.std).to(k.dtype))
        torch.cuda.synchronize(dev)
        g.replay()
        torch.cuda.synchronize(dev)
        eager = flat(tsel.select(q, k, lay, mask, ratios, emb=emb))
        torch.cuda.synchronize(dev)
        for key, ref in eager.items():
            got = captured[key]
            assert got.shape == ref.shape, key
            assert torch.equal(got.view(torch.uint8), ref.view(torch.uint8)), f"replay {rep}: {key} differs"
        print(f"[check] replay {rep}: all outputs identical to eager", flush=True)
        assert np.isfinite(eager["score"].cpu().numpy()).all()
