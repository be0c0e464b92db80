"""Write the stored oracle masses of the 16384-token GQA decoder workload.

The oracle on that workload takes minutes of CPU time, too long for a GPU
test, so its column masses are computed once here, by ``oracle/`` only, and
stored with a digest of the regenerated Q/K bytes (and the problem's softmax
scale).  Run from the repository root:
    python tests/golden/make_oracle_cache.py          # bf16 inputs -> oracle_c4.npz
    python tests/golden/make_oracle_cache.py fp8      # fp8 inputs  -> oracle_c4_fp8.npz
"""
import hashlib
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from workloads import make_config  # noqa: E402


def digest(prob) -> str:
    h = hashlib.sha256()
    for t in (prob.q, prob.k):
        h.update(t.contiguous().view(torch.uint8).numpy().tobytes())
    return h.hexdigest()


def main():
    dtype = sys.argv[1] if len(sys.argv) > 1 else "bf16"
    prob = make_config(4) if dtype == "bf16" else make_config(4, dtype=dtype)
    t0 = time.time()
    _, mass = oracle.attention_stats(prob, workers=oracle.default_workers())
    fname = "oracle_c4.npz" if dtype == "bf16" else f"oracle_c4_{dtype}.npz"
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), fname)
    scale = np.nan if prob.softmax_scale is None else prob.softmax_scale
    np.savez_compressed(out, mass=mass, digest=np.array(digest(prob)), name=np.array(prob.name),
                        scale=np.array(scale))
    print(f"wrote {out} in {time.time() - t0:.1f}s")


if __name__ == "__main__":
    main()
