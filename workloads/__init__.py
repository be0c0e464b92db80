"""Seeded synthetic workloads for attention-score visual-token selection.

This module only draws inputs: token layouts (requests, images, text), the
per-head Q and K of one attention layer, keep ratios and the embedding rows
that get gathered.  It contains none of the selection method's arithmetic
(no softmax, no scoring, no budget rule, no compaction); both the CPU oracle
in ``oracle/`` and the GPU path consume what it returns.

Recipe (numpy ``default_rng(seed)``, PCG64), in draw order:

1. layout (only the varlen batch draws it),
2. Q as standard normals in fp32, times ``std``,
3. K the same way,
4. dominant keys (tokens whose K is multiplied by 4 in every KV head),
5. keep ratios (only the varlen batch draws them).

Embedding rows (standard normals) come from their own stream,
``default_rng([seed, 1])``, drawn on first use: a gather copies bytes, so
the rows are only needed by the compaction checks and the benchmark.  The
values V of the layer's attention (standard normals, [T, Hkv, d], in the
Q/K storage type; bf16 for fp8 problems), used only by the attention
forward, come from ``default_rng([seed, 2])``, also drawn on first use.

Q/K/emb are generated in fp32 and then rounded to the storage dtype with
round-to-nearest-even (torch ``.to``), so every consumer reads the same
stored bits.  For fp8 (OCP E4M3) Q and K are first divided by a per-tensor
factor (largest magnitude / 448, rounded to fp32) so that they span the
format's range, and the problem's ``softmax_scale`` becomes
``fp32(sq * sk / sqrt(d))``: the quantised logits then equal the original
ones up to the fp8 rounding.  Embeddings of an fp8 problem are bf16.

The five named workloads follow the problem statements of the pages: one
ViT-layer image (LiteVLM / VisionZip single image), a LiteVLM-style
first-decoder-layer selection over 12 tiles of 256 tokens plus 142 text
tokens (LiteVLM, section 5 main-results table), a VisionZip-style 30-image
block-diagonal pool (REDtech article, section 3.2), a large GQA decoder
layer with Qwen3-VL-32B head shapes (REDtech article, section 3.3), and a
varlen batch of 8 requests with a supplied LSE (REDtech article, section 3.2:
reuse of the FlashAttention LSE).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import numpy as np
import torch

MASKS = ("full", "causal", "blockdiag")
DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16,
          "fp8": torch.float8_e4m3fn}
FP8_MAX = 448.0


@dataclass
class Problem:
    """One batch of selection work.  Arrays are CPU-resident.

    Token layout: requests are packed back to back (``cu_seqlens``); images
    are disjoint token ranges ``[img_start[s], img_start[s] + h*w)`` sorted by
    start; request ``b`` owns images ``cu_images[b] .. cu_images[b+1]-1``;
    candidate index ``c`` enumerates image tokens in token order and
    ``cu_cands[s]`` is the first candidate of image ``s``.
    """

    name: str
    q: torch.Tensor            # [T, Hq, d] storage dtype
    k: torch.Tensor            # [T, Hkv, d] storage dtype
    mask: str                  # "full" | "causal" | "blockdiag"
    cu_seqlens: np.ndarray     # int32 [B+1]
    cu_images: np.ndarray      # int32 [B+1]
    img_start: np.ndarray      # int32 [S]
    img_hw: np.ndarray         # int32 [S, 2]  (rows, cols)
    cu_cands: np.ndarray       # int32 [S+1]
    keep_ratio: np.ndarray     # float64 [B]
    emb_dim: int = 64
    emb_dtype: str = "bf16"
    lse_supplied: bool = False
    seed: int = 0
    dtype: str = "bf16"
    std: float = 1.0
    dominant: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int64))
    softmax_scale: Optional[float] = None   # None: 1/sqrt(d)
    _emb: Optional[torch.Tensor] = None
    _v: Optional[torch.Tensor] = None

    @property
    def v(self) -> torch.Tensor:
        """Attention values [T, Hkv, d] (drawn on first use)."""
        if self._v is None:
            rng = np.random.default_rng([self.seed, 2])
            x = rng.standard_normal((self.T, self.hkv, self.d), dtype=np.float32)
            self._v = _round(x, "bf16" if self.dtype == "fp8" else self.dtype)
        return self._v

    @v.setter
    def v(self, value: torch.Tensor):
        self._v = value

    @property
    def emb(self) -> torch.Tensor:
        """Embedding rows [T, emb_dim] in ``emb_dtype`` (drawn on first use)."""
        if self._emb is None:
            rng = np.random.default_rng([self.seed, 1])
            x = rng.standard_normal((self.T, self.emb_dim), dtype=np.float32)
            self._emb = _round(x, self.emb_dtype)
        return self._emb

    @emb.setter
    def emb(self, value: torch.Tensor):
        self._emb = value

    @property
    def T(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def B(self) -> int:
        return len(self.cu_seqlens) - 1

    @property
    def S(self) -> int:
        return len(self.img_start)

    @property
    def N(self) -> int:
        return int(self.cu_cands[-1])

    @property
    def hq(self) -> int:
        return self.q.shape[1]

    @property
    def hkv(self) -> int:
        return self.k.shape[1]

    @property
    def d(self) -> int:
        return self.q.shape[2]


def layout_arrays(requests: Sequence[Tuple[int, Sequence[Tuple[int, int, int]]]]):
    """Build packed layout arrays.

    ``requests`` is a list of ``(length, images)``, where each image is
    ``(offset_in_request, rows, cols)``.  Images of a request must be sorted,
    disjoint and inside the request.
    """
    cu_seqlens = [0]
    cu_images = [0]
    img_start: List[int] = []
    img_hw: List[Tuple[int, int]] = []
    for length, images in requests:
        base = cu_seqlens[-1]
        prev_end = 0
        for off, h, w in images:
            if off < prev_end or off + h * w > length or h <= 0 or w <= 0:
                raise ValueError("images must be sorted, disjoint and inside the request")
            img_start.append(base + off)
            img_hw.append((h, w))
            prev_end = off + h * w
        cu_seqlens.append(base + length)
        cu_images.append(len(img_start))
    cu_cands = [0]
    for h, w in img_hw:
        cu_cands.append(cu_cands[-1] + h * w)
    return (np.asarray(cu_seqlens, np.int32), np.asarray(cu_images, np.int32),
            np.asarray(img_start, np.int32).reshape(-1),
            np.asarray(img_hw, np.int32).reshape(-1, 2), np.asarray(cu_cands, np.int32))


def _round(x: np.ndarray, dtype: str) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DTYPES[dtype])


def _quantize_fp8(x: np.ndarray):
    """fp8 E4M3 copy of ``x`` divided by its per-tensor factor; returns
    (tensor, factor)."""
    amax = float(np.max(np.abs(x))) if x.size else 0.0
    f = np.float32(amax / FP8_MAX) if amax > 0 else np.float32(1.0)
    return _round(x / f, "fp8"), float(f)


def make_problem(name: str, requests, hq: int, hkv: int, d: int, dtype: str, mask: str,
                 std: float, seed: int, ratios=None, ratio_range=None, emb_dim: int = 64,
                 emb_dtype: Optional[str] = None, dominant_spec=None,
                 lse_supplied: bool = False, rng: Optional[np.random.Generator] = None) -> Problem:
    """Draw Q, K, dominant keys, ratios and embeddings for a given layout.

    ``dominant_spec``: ``None``; ``("count", n)`` picks ``n`` tokens of the
    whole batch without replacement; ``("images", n_img, lo, hi)`` picks
    ``n_img`` images by permutation and, in each, ``U{lo..hi}`` tokens
    without replacement.  Their K rows are multiplied by 4 in every KV head.
    """
    assert mask in MASKS and dtype in DTYPES
    if rng is None:
        rng = np.random.default_rng(seed)
    cu_seqlens, cu_images, img_start, img_hw, cu_cands = layout_arrays(requests)
    T = int(cu_seqlens[-1])
    qf = rng.standard_normal((T, hq, d), dtype=np.float32) * np.float32(std)
    kf = rng.standard_normal((T, hkv, d), dtype=np.float32) * np.float32(std)
    dom = np.zeros(0, np.int64)
    if dominant_spec is not None:
        if dominant_spec[0] == "count":
            dom = np.sort(rng.choice(T, size=dominant_spec[1], replace=False))
        elif dominant_spec[0] == "images":
            _, n_img, lo, hi = dominant_spec
            picked = rng.permutation(len(img_start))[:n_img]
            toks = []
            for s in np.sort(picked):
                size = int(img_hw[s, 0] * img_hw[s, 1])
                n_dom = int(rng.integers(lo, hi + 1))
                toks.append(int(img_start[s]) + rng.choice(size, size=n_dom, replace=False))
            dom = np.sort(np.concatenate(toks)) if toks else dom
        else:
            raise ValueError(dominant_spec)
        kf[dom] *= np.float32(4.0)
    B = len(cu_seqlens) - 1
    if ratios is not None:
        keep_ratio = np.broadcast_to(np.asarray(ratios, np.float64), (B,)).copy()
    else:
        lo, hi = ratio_range
        keep_ratio = rng.uniform(lo, hi, size=B)
    softmax_scale = None
    if dtype == "fp8":
        q, fq = _quantize_fp8(qf)
        k, fk = _quantize_fp8(kf)
        softmax_scale = float(np.float32(fq * fk / np.sqrt(d)))
        emb_dtype = emb_dtype or "bf16"
    else:
        q, k = _round(qf, dtype), _round(kf, dtype)
    return Problem(name=name, q=q, k=k, mask=mask,
                   cu_seqlens=cu_seqlens, cu_images=cu_images, img_start=img_start,
                   img_hw=img_hw, cu_cands=cu_cands, keep_ratio=keep_ratio, emb_dim=emb_dim,
                   emb_dtype=emb_dtype or dtype, lse_supplied=lse_supplied, seed=seed,
                   dtype=dtype, std=std, dominant=dom, softmax_scale=softmax_scale)


# ----------------------------------------------------------------------------
# The five named workloads.
# ----------------------------------------------------------------------------

CONFIG_NAMES = {
    1: "vit_image_16x16_h4_d64_f32_full",
    2: "litevlm_12x256_plus142_h16_d128_bf16_causal",
    3: "visionzip_30x1024_h16_d80_bf16_blockdiag",
    4: "decoder_16384_gqa64x8_d128_bf16_causal",
    5: "varlen_8req_h32_d128_f16_causal_lse_supplied",
}


def varlen_layout(rng: np.random.Generator, n_req: int = 8, lmin: int = 2048, lmax: int = 8192,
                  img_max: int = 12, side_min: int = 16, side_max: int = 32):
    """Varlen batch layout: per request L ~ U{lmin..lmax}, n_img ~ U{1..img_max},
    each image h, w ~ U{side_min..side_max}; trailing images are dropped while
    the image tokens exceed L-1 (at least one text token stays); images come
    first in the request, text after them."""
    reqs = []
    for _ in range(n_req):
        L = int(rng.integers(lmin, lmax + 1))
        n_img = int(rng.integers(1, img_max + 1))
        hw = rng.integers(side_min, side_max + 1, size=(n_img, 2))
        sizes = hw[:, 0] * hw[:, 1]
        while n_img > 0 and int(sizes[:n_img].sum()) > L - 1:
            n_img -= 1
        images, off = [], 0
        for i in range(n_img):
            h, w = int(hw[i, 0]), int(hw[i, 1])
            images.append((off, h, w))
            off += h * w
        reqs.append((L, images))
    return reqs


def make_config(cfg: int, seed: Optional[int] = None, std: Optional[float] = None,
                dtype: Optional[str] = None) -> Problem:
    """Named workload ``cfg`` in 1..5 (seed defaults to ``cfg``).  ``std``
    overrides the Q/K standard deviation (used for the value-sensitive
    variants of the near-uniform decoder workloads).  ``dtype`` overrides the
    Q/K storage type of the decoder workloads (2 and 4), e.g. "fp8" for the
    low-precision scoring LiteVLM deploys; the name then says so."""
    seed = cfg if seed is None else seed
    name = CONFIG_NAMES[cfg]
    if dtype is not None:
        if cfg not in (2, 4):
            raise ValueError("dtype override is defined for workloads 2 and 4")
        name = name.replace("_bf16_", f"_{dtype}_")
    if cfg == 1:
        return make_problem(name, [(256, [(0, 16, 16)])], 4, 4, 64, "f32", "full",
                            1.0 if std is None else std, seed, ratios=0.4, emb_dim=256,
                            dominant_spec=("count", 8))
    if cfg == 2:
        d = 128
        imgs = [(i * 256, 16, 16) for i in range(12)]
        return make_problem(name, [(12 * 256 + 142, imgs)], 16, 16, d, dtype or "bf16", "causal",
                            1.0 / np.sqrt(d) if std is None else std, seed, ratios=0.8,
                            emb_dim=2048, emb_dtype="bf16")
    if cfg == 3:
        imgs = [(i * 1024, 32, 32) for i in range(30)]
        return make_problem(name, [(30 * 1024, imgs)], 16, 16, 80, "bf16", "blockdiag",
                            1.0 if std is None else std, seed, ratios=0.6, emb_dim=1280,
                            dominant_spec=("images", 15, 10, 20))
    if cfg == 4:
        d = 128
        imgs = [(i * 750, 25, 30) for i in range(20)]
        return make_problem(name, [(16384, imgs)], 64, 8, d, dtype or "bf16", "causal",
                            1.0 / np.sqrt(d) if std is None else std, seed, ratios=0.6,
                            emb_dim=5120, emb_dtype="bf16")
    if cfg == 5:
        d = 128
        rng = np.random.default_rng(seed)
        reqs = varlen_layout(rng)
        return make_problem(name, reqs, 32, 32, d, "f16", "causal",
                            1.0 / np.sqrt(d) if std is None else std, seed,
                            ratio_range=(0.5, 0.9), emb_dim=4096, lse_supplied=True, rng=rng)
    raise KeyError(cfg)


def random_small(seed: int, mask: str, dtype: str = "bf16", hq: int = 4, hkv: int = 2,
                 d: int = 64, n_req: int = 2, text_prefix: bool = True,
                 interleave: bool = True, std: float = 1.0, emb_dim: int = 40) -> Problem:
    """Small randomized layout for parity sweeps: requests of a few hundred
    tokens, 1-3 images each of h, w in 3..13, an optional text prefix, and
    optional text between images; ragged everywhere."""
    rng = np.random.default_rng(seed)
    reqs = []
    for _ in range(n_req):
        n_img = int(rng.integers(1, 4))
        images, off = [], 0
        if text_prefix or mask == "blockdiag":
            off = 0 if mask == "blockdiag" else int(rng.integers(0, 40))
        for _ in range(n_img):
            h, w = int(rng.integers(3, 14)), int(rng.integers(3, 14))
            images.append((off, h, w))
            off += h * w
            if interleave and mask != "blockdiag":
                off += int(rng.integers(0, 30))
        length = off if mask == "blockdiag" else off + int(rng.integers(1, 50))
        reqs.append((length, images))
    return make_problem(f"small_{mask}_{dtype}_s{seed}", reqs, hq, hkv, d, dtype, mask, std,
                        seed, ratio_range=(0.2, 0.95), emb_dim=emb_dim, rng=rng)


def random_medium(seed: int, mask: str, dtype: str = "bf16", hq: int = 8, hkv: int = 2,
                  d: int = 128, n_req: int = 2, std: float = 1.0, emb_dim: int = 200,
                  side=(8, 40), max_images: int = 4) -> Problem:
    """Medium randomized layout (a few thousand tokens): several row blocks,
    row chunks and key blocks of the GPU kernels, text prefixes, text between
    images (except under the block-diagonal mask), ragged tails."""
    rng = np.random.default_rng(seed)
    reqs = []
    for _ in range(n_req):
        n_img = int(rng.integers(1, max_images + 1))
        images, off = [], 0 if mask == "blockdiag" else int(rng.integers(0, 100))
        for _ in range(n_img):
            h, w = (int(x) for x in rng.integers(side[0], side[1] + 1, size=2))
            images.append((off, h, w))
            off += h * w
            if mask != "blockdiag":
                off += int(rng.integers(0, 120))
        length = off if mask == "blockdiag" else off + int(rng.integers(1, 300))
        reqs.append((length, images))
    return make_problem(f"medium_{mask}_{dtype}_h{hq}x{hkv}_d{d}_s{seed}", reqs, hq, hkv, d, dtype,
                        mask, std, seed, ratio_range=(0.3, 0.9), emb_dim=emb_dim, rng=rng)
