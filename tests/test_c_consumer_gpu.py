"""The whole selection path driven from a plain C99 program through the C ABI
(tests/c_consumer/tsel_consumer.c: include/tsel.h and the HIP runtime's C API,
no torch), checked against the oracle with the same bars as the Python-driven
parity tests.  The inputs are the seeded workloads, written to a file here."""
import os
import struct
import subprocess
import sys

import numpy as np
import pytest
import torch

import oracle
from workloads import random_small

sys.path.insert(0, os.path.dirname(__file__))
import parity as P  # noqa: E402

pytestmark = pytest.mark.gpu
EXE = os.path.join(os.path.dirname(__file__), "c_consumer", "tsel_consumer")
DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2}
MASK_CODE = {"full": 0, "causal": 1, "blockdiag": 2}


def write_input(prob, path):
    emb = prob.emb.contiguous()
    row_bytes = emb.shape[1] * emb.element_size()
    with open(path, "wb") as f:
        f.write(struct.pack("<10i", 0x31435354, prob.T, prob.B, prob.S, prob.hq, prob.hkv, prob.d,
                            DTYPE_CODE[prob.dtype], MASK_CODE[prob.mask], row_bytes))
        for a in (prob.cu_seqlens, prob.cu_images, prob.img_start, prob.img_hw, prob.cu_cands):
            f.write(np.ascontiguousarray(np.asarray(a, np.int32).reshape(-1)).tobytes())
        f.write(np.ascontiguousarray(np.asarray(prob.keep_ratio, np.float64)).tobytes())
        for t in (prob.q, prob.k, emb):
            f.write(t.contiguous().view(torch.uint8).numpy().tobytes())
    return row_bytes


def read_output(prob, path, row_bytes):
    buf = open(path, "rb").read()
    off = 0

    def take(dtype, n):
        nonlocal off
        a = np.frombuffer(buf, dtype=dtype, count=n, offset=off)
        off += a.nbytes
        return a.copy()

    lse = take(np.float32, prob.hq * prob.T).reshape(prob.hq, prob.T).astype(np.float64)
    score = take(np.float32, prob.N).astype(np.float64)
    k = take(np.int32, prob.B)
    keep = take(np.uint8, prob.N)
    t_out = int(take(np.int32, 1)[0])
    comp = {"token_idx": torch.from_numpy(take(np.int32, t_out)),
            "spatial": torch.from_numpy(take(np.int32, 3 * t_out).reshape(t_out, 3)),
            "cu_seqlens": torch.from_numpy(take(np.int32, prob.B + 1)),
            "img_counts": torch.from_numpy(take(np.int32, prob.S)),
            "positions": torch.from_numpy(take(np.int32, 3 * t_out).reshape(t_out, 3))}
    comp["emb"] = torch.from_numpy(take(np.uint8, t_out * row_bytes).reshape(t_out, row_bytes))
    assert off == len(buf)
    return dict(lse=lse, score=score, keep=keep, k=k.astype(np.int64), compact=comp)


CASES = [("causal", "bf16", 8, 2, 128), ("full", "f32", 4, 4, 64), ("blockdiag", "f16", 4, 2, 72),
         ("causal", "f16", 16, 4, 80)]


@pytest.mark.parametrize("i", range(len(CASES)))
def test_c_program_drives_the_path(tmp_path, i):
    if not os.path.exists(EXE):  # normally built by __graft_entry__.build(); plain gcc, no HIP compile
        sys.path.insert(0, os.path.join(os.path.dirname(__file__), "c_consumer"))
        import build_consumer
        build_consumer.build()
    mask, dtype, hq, hkv, d = CASES[i]
    prob = random_small(700 + i, mask, dtype=dtype, hq=hq, hkv=hkv, d=d, n_req=3)
    print(f"\n[case] C consumer {prob.name} T={prob.T} N={prob.N} {dtype} {mask} d={d}", flush=True)
    row_bytes = write_input(prob, tmp_path / "in.bin")
    r = subprocess.run([EXE, "run", str(tmp_path / "in.bin"), str(tmp_path / "out.bin")],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    got = read_output(prob, tmp_path / "out.bin", row_bytes)
    emb_bytes = prob.emb.contiguous().view(torch.uint8).reshape(prob.T, row_bytes)
    P.full_check(prob, got, oracle.run(prob, with_emb=False), emb_bytes)
