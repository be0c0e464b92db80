"""The entry point that allocates nothing (tsel_colscore_noalloc) against the
workspace entry point it varies (tsel_colscore), through the C ABI.

Both run the same kernels; only where the column-score partials live
differs (the library's static device buffer, or a caller workspace), so the
scores must be identical bit for bit.  Two calls in a row, the second on a
smaller problem, show that the buffer's leftover contents from the first call
do not leak into the second.
"""
import ctypes

import pytest
import torch

import attention_score_selection_amd as tsel
from attention_score_selection_amd import binding as B
from workloads import make_config, random_medium

pytestmark = pytest.mark.gpu


def noalloc_scores(prob, lay, q, k, lse, dev):
    attn = B.make_attn(q, k, prob.mask, prob.softmax_scale or 0.0)
    out = torch.full((prob.N,), float("nan"), dtype=torch.float32, device=dev)
    rc = tsel.lib().tsel_colscore_noalloc(ctypes.byref(attn), ctypes.byref(lay.c), lse.data_ptr(),
                                          out.data_ptr(), torch.cuda.current_stream(dev).cuda_stream)
    assert rc == B.TSEL_OK, tsel.lib().tsel_last_error().decode()
    return out


def test_noalloc_equals_workspace_entry_point_two_calls():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    dev = torch.device("cuda:0")
    big = make_config(4)  # 16384-token GQA layer: ~9.1 MB of partials
    small = random_medium(301, "causal", dtype="f16", hq=8, hkv=2, d=128, n_req=3)
    for prob in (big, small):
        print(f"\n[case] noalloc vs workspace: {prob.name} T={prob.T} N={prob.N}", flush=True)
        lay = tsel.Layout.from_problem(prob, dev)
        q, k = prob.q.to(dev), prob.k.to(dev)
        scale = prob.softmax_scale or 0.0
        need = tsel.tsel_workspace_size(B.TSEL_OP_COLSCORE, lay, q, k, prob.mask, scale)
        assert 0 < need <= 16 << 20
        lse = tsel.tsel_lse(q, k, lay, prob.mask, scale)
        ref = tsel.tsel_colscore(q, k, lay, prob.mask, lse, scale)
        got = noalloc_scores(prob, lay, q, k, lse, dev)
        torch.cuda.synchronize(dev)
        assert torch.equal(got, ref), f"{prob.name}: {int((got != ref).sum())} scores differ"
        # The binding's wrapper reaches the same entry point.
        again = tsel.tsel_colscore_noalloc(q, k, lay, prob.mask, lse, scale)
        torch.cuda.synchronize(dev)
        assert torch.equal(again, ref)
