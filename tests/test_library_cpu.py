"""Host-side checks of the C-ABI library that need no GPU.

The library must load and export every function ``include/tsel.h``
declares, and its argument validation must reject bad input with the
documented codes before it touches the HIP runtime.  Every call below fails
validation, so no kernel is launched.
"""
import ctypes
import os
import re
import subprocess
import sys

import numpy as np
import pytest

from attention_score_selection_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tsel.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from attention_score_selection_amd import build
        build.build()
    return B.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tsel_[a-z_]+)\s*\(", text)))


def test_header_declares_the_path(lib):
    names = declared_functions()
    for n in ("tsel_lse", "tsel_colscore", "tsel_budget_topk", "tsel_compact", "tsel_attention_fwd",
              "tsel_mrope_positions", "tsel_budget_mass"):
        assert n in names
    assert set(names) == set(B.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version(lib):
    header = open(HEADER).read()
    want = int(re.search(r"#define TSEL_VERSION (\d+)", header).group(1))
    assert lib.tsel_version() == want == 4


FAKE = 4096  # non-null device address that validation never dereferences


class HostLayout:
    """A tsel_layout_t whose device fields hold placeholder addresses."""

    def __init__(self, cu_seqlens, cu_images, img_start, img_hw, cu_cands):
        self.h = [np.ascontiguousarray(np.asarray(a, np.int32).reshape(-1))
                  for a in (cu_seqlens, cu_images, img_start, img_hw, cu_cands)]
        c = B.CLayout()
        c.num_reqs = len(self.h[0]) - 1
        c.num_images = len(self.h[2])
        c.total_tokens = int(self.h[0][-1])
        for name, arr in zip(("cu_seqlens", "cu_images", "img_start", "img_hw", "cu_cands"), self.h):
            setattr(c, name + "_h", arr.ctypes.data if arr.size else None)
            setattr(c, name, FAKE if arr.size else None)
        self.c = c


def good_layout():
    # two requests: [img 4x4 @0, text 3] and [text 2, img 2x3 @2, text 1]
    return HostLayout([0, 19, 28], [0, 1, 2], [0, 21], [[4, 4], [2, 3]], [0, 16, 22])


def attn(dtype=B.TSEL_BF16, hq=8, hkv=2, d=128, mask=1, q=FAKE, k=FAKE, st=None):
    a = B.CAttn()
    a.dtype, a.num_heads_q, a.num_heads_kv, a.head_dim = dtype, hq, hkv, d
    a.q, a.k = q, k
    a.q_stride_tok, a.q_stride_head = (st or (hq * d, d))
    a.k_stride_tok, a.k_stride_head = hkv * d, d
    a.mask, a.softmax_scale = mask, 0.0
    return a


def last_error(lib):
    return lib.tsel_last_error().decode()


def call_lse(lib, a, lay, out=FAKE, ws=None, ws_bytes=0):
    return lib.tsel_lse(ctypes.byref(a), ctypes.byref(lay.c), out, ws, ws_bytes, None)


def test_attn_validation_codes(lib):
    lay = good_layout()
    assert call_lse(lib, attn(d=112), lay) == B.TSEL_EUNSUPPORTED
    assert "head_dim" in last_error(lib)
    assert call_lse(lib, attn(dtype=7), lay) == B.TSEL_EUNSUPPORTED
    assert call_lse(lib, attn(hq=6, hkv=4), lay) == B.TSEL_EINVAL
    assert call_lse(lib, attn(q=FAKE + 8), lay) == B.TSEL_EINVAL
    assert "aligned" in last_error(lib)
    assert call_lse(lib, attn(st=(8 * 128 + 4, 128)), lay) == B.TSEL_EINVAL
    assert call_lse(lib, attn(mask=5), lay) == B.TSEL_EINVAL
    a = attn()
    a.softmax_scale = float("nan")
    assert call_lse(lib, a, lay) == B.TSEL_EINVAL
    # BLOCKDIAG needs every token inside an image.
    assert call_lse(lib, attn(mask=2), lay) == B.TSEL_EINVAL
    assert "BLOCKDIAG" in last_error(lib)
    assert lib.tsel_lse(None, ctypes.byref(lay.c), FAKE, None, 0, None) == B.TSEL_EINVAL
    # fp8 inputs take whole 64-wide k chunks only.
    assert call_lse(lib, attn(dtype=B.TSEL_FP8_E4M3, d=96), lay) == B.TSEL_EUNSUPPORTED
    assert "fp8" in last_error(lib)
    assert call_lse(lib, attn(dtype=B.TSEL_FP8_E4M3, d=72), lay) == B.TSEL_EUNSUPPORTED
    # A 32-row tile must span less than 2 GiB of the buffers it is read from.
    assert call_lse(lib, attn(st=(1 << 28, 128)), lay) == B.TSEL_EUNSUPPORTED
    assert "2 GiB" in last_error(lib)


@pytest.mark.parametrize("bad", ["cu_end", "overlap", "outside", "cands", "empty_grid", "no_reqs"])
def test_layout_validation(lib, bad):
    args = dict(cu_seqlens=[0, 19, 28], cu_images=[0, 1, 2], img_start=[0, 21],
                img_hw=[[4, 4], [2, 3]], cu_cands=[0, 16, 22])
    if bad == "cu_end":
        pass
    elif bad == "overlap":
        args.update(cu_images=[0, 2, 2], img_start=[0, 10], cu_seqlens=[0, 40, 49])
    elif bad == "outside":
        args["img_start"] = [0, 25]
    elif bad == "cands":
        args["cu_cands"] = [0, 16, 21]
    elif bad == "empty_grid":
        args["img_hw"] = [[4, 4], [0, 3]]
    elif bad == "no_reqs":
        args.update(cu_seqlens=[0], cu_images=[0], img_start=[], img_hw=[], cu_cands=[0])
    lay = HostLayout(**args)
    if bad == "cu_end":
        lay.c.total_tokens = 30  # cu_seqlens must end at total_tokens
    assert call_lse(lib, attn(), lay) == B.TSEL_EINVAL
    assert last_error(lib)


def test_topk_rejects_nan_ratio(lib):
    lay = good_layout()
    ratios = np.array([0.5, np.nan])
    k_h = np.zeros(2, np.int32)
    rc = lib.tsel_budget_topk(ctypes.byref(lay.c), FAKE, ratios.ctypes.data, k_h.ctypes.data, FAKE, None, 0, None)
    assert rc == B.TSEL_EINVAL and "NaN" in last_error(lib)


def test_layout_max_seqlen_checked_when_given(lib):
    lay = good_layout()
    lay.c.max_seqlen = 19  # the longest of the two requests (19 and 9 tokens)
    assert lib.tsel_workspace_size(B.TSEL_OP_COMPACT, None, ctypes.byref(lay.c)) != ctypes.c_size_t(-1).value
    lay.c.max_seqlen = 20
    assert lib.tsel_workspace_size(B.TSEL_OP_COMPACT, None, ctypes.byref(lay.c)) == ctypes.c_size_t(-1).value
    assert "max_seqlen" in last_error(lib)
    lay.c.max_seqlen = 0  # not given
    assert lib.tsel_workspace_size(B.TSEL_OP_COMPACT, None, ctypes.byref(lay.c)) != ctypes.c_size_t(-1).value


def test_lse_key_split_workspace(lib):
    """A small causal grid (one 3214-token request, 16 heads) splits its keys:
    the LSE then needs Hq * T * (splits of the request) floats of workspace,
    and a shortfall is refused before any launch.  A grid that fills the GPU
    (the 16384-token layer, 64/8 heads) needs none."""
    lay = HostLayout([0, 3214], [0, 12], [256 * i for i in range(12)], [[16, 16]] * 12,
                     [256 * i for i in range(13)])
    a = attn(hq=16, hkv=16, d=128)
    need = lib.tsel_workspace_size(B.TSEL_OP_LSE, ctypes.byref(a), ctypes.byref(lay.c))
    assert need > 0 and need % (16 * 3214 * 4) == 0
    splits = need // (16 * 3214 * 4)
    assert 2 <= splits <= 13
    assert call_lse(lib, a, lay, ws=FAKE, ws_bytes=need - 4) == B.TSEL_EWORKSPACE
    assert "workspace" in last_error(lib)
    big = HostLayout([0, 16384], [0, 20], [750 * i for i in range(20)], [[25, 30]] * 20,
                     [750 * i for i in range(21)])
    assert lib.tsel_workspace_size(B.TSEL_OP_LSE, ctypes.byref(attn(hq=64, hkv=8, d=128)),
                                   ctypes.byref(big.c)) == 0


def test_topk_workspace_for_large_pools(lib):
    """Pools above 32768 candidates are spread over blocks of 16384 and need
    workspace (state and histograms of up to 64 such pools, plus one count
    per block); pools that fit one workgroup need none."""
    small = good_layout()
    assert lib.tsel_workspace_size(B.TSEL_OP_TOPK, None, ctypes.byref(small.c)) == 0
    lay = HostLayout([0, 40000, 140010], [0, 1, 2], [0, 40010], [[200, 200], [250, 400]],
                     [0, 40000, 140000])
    need = lib.tsel_workspace_size(B.TSEL_OP_TOPK, None, ctypes.byref(lay.c))
    blocks = 3 + 7  # ceil(40000 / 16384) + ceil(100000 / 16384)
    assert need == (64 * 4 + 64 * 256 + blocks) * 4
    ratios = np.array([0.5, 0.5])
    k_h = np.zeros(2, np.int32)
    rc = lib.tsel_budget_topk(ctypes.byref(lay.c), FAKE, ratios.ctypes.data, k_h.ctypes.data, FAKE, FAKE,
                              need - 4, None)
    assert rc == B.TSEL_EWORKSPACE and "workspace" in last_error(lib)


@pytest.mark.parametrize("tau,rmin,rmax,msg", [((0.5, np.nan), (0.0, 0.0), (1.0, 1.0), "NaN"),
                                                ((0.5, 0.5), (0.0, np.nan), (1.0, 1.0), "NaN"),
                                                ((0.5, 0.5), (0.0, 0.7), (1.0, 0.6), "r_min > r_max")])
def test_budget_mass_validation(lib, tau, rmin, rmax, msg):
    """Bad host arguments fail before any launch (no GPU needed)."""
    lay = good_layout()
    arrs = [np.asarray(x, np.float64) for x in (tau, rmin, rmax)]
    rc = lib.tsel_budget_mass(ctypes.byref(lay.c), FAKE, arrs[0].ctypes.data, arrs[1].ctypes.data,
                              arrs[2].ctypes.data, FAKE, FAKE, None)
    assert rc == B.TSEL_EINVAL and msg in last_error(lib)
    rc = lib.tsel_budget_mass(ctypes.byref(lay.c), FAKE, arrs[0].ctypes.data, arrs[1].ctypes.data,
                              None, FAKE, FAKE, None)
    assert rc == B.TSEL_EINVAL


def test_workspace_sizes_and_shortfall(lib):
    lay = good_layout()
    a = attn()
    need = lib.tsel_workspace_size(B.TSEL_OP_COLSCORE, ctypes.byref(a), ctypes.byref(lay.c))
    assert 0 < need < 1 << 30
    assert need % 4 == 0
    assert lib.tsel_workspace_size(B.TSEL_OP_LSE, ctypes.byref(a), ctypes.byref(lay.c)) == 0
    assert lib.tsel_workspace_size(B.TSEL_OP_TOPK, None, ctypes.byref(lay.c)) == 0
    comp = lib.tsel_workspace_size(B.TSEL_OP_COMPACT, None, ctypes.byref(lay.c))
    assert comp >= 3 * 4
    assert lib.tsel_workspace_size(9, None, ctypes.byref(lay.c)) == ctypes.c_size_t(-1).value
    rc = lib.tsel_colscore(ctypes.byref(a), ctypes.byref(lay.c), FAKE, FAKE, FAKE, need - 4, None)
    assert rc == B.TSEL_EWORKSPACE
    rc = lib.tsel_compact(ctypes.byref(lay.c), FAKE, None, 0, 0, 10, None, 0, FAKE, None, None, None,
                          FAKE, comp - 4, None)
    assert rc == B.TSEL_EWORKSPACE


def test_colscore_noalloc_rejects_problems_over_its_static_scratch(lib):
    """tsel_colscore_noalloc keeps its partials in a 16 MiB static device
    buffer: a problem needing more is refused before any HIP call."""
    # One 32768-token request, 30000 candidates (30 images of 25 x 40), 64/8 heads:
    # 8 head blocks x 35 row chunks x 30000 candidates x 4 bytes = 33.6 MB.
    starts = [100 + 1000 * i for i in range(30)]
    lay = HostLayout([0, 32768], [0, 30], starts, [[25, 40]] * 30,
                     [1000 * i for i in range(31)])
    a = attn(hq=64, hkv=8, d=128)
    need = lib.tsel_workspace_size(B.TSEL_OP_COLSCORE, ctypes.byref(a), ctypes.byref(lay.c))
    assert need > 16 << 20
    rc = lib.tsel_colscore_noalloc(ctypes.byref(a), ctypes.byref(lay.c), FAKE, FAKE, None)
    assert rc == B.TSEL_EWORKSPACE
    assert "16777216" in last_error(lib) and str(need) in last_error(lib)
    # Validation errors come first, as in tsel_colscore.
    assert lib.tsel_colscore_noalloc(ctypes.byref(attn(d=112)), ctypes.byref(lay.c), FAKE, FAKE,
                                     None) == B.TSEL_EUNSUPPORTED


def test_colscore_cuts_the_last_chunk_of_long_segments(lib):
    """Row chunks of 8192 query rows (512 tokens at 16 folded heads); a
    segment longer than one chunk, in a launch with at least 512 jobs, has
    the range after its last whole chunk cut into pieces of a quarter chunk,
    each with its own partial row in the workspace."""
    # Request 0: 4496 tokens, four 32x32 images; request 1: 300 tokens, one 12x12 image.
    lay = HostLayout([0, 4496, 4796], [0, 4, 5], [100, 1161, 2185, 3259, 4506],
                     [[32, 32]] * 4 + [[12, 12]], [0, 1024, 2048, 3072, 4096, 4240])
    a = attn(dtype=B.TSEL_F32, hq=32, hkv=2, d=128)
    need = lib.tsel_workspace_size(B.TSEL_OP_COLSCORE, ctypes.byref(a), ctypes.byref(lay.c))
    # 2 head blocks x (8 whole chunks + 400 tokens in 4 pieces of 128) x 4240 candidates.
    assert need == 2 * 12 * 4240 * 4
    # A short layout halves its chunks instead and is never cut.
    a = attn(dtype=B.TSEL_F32, hq=32, hkv=2, d=128)
    need = lib.tsel_workspace_size(B.TSEL_OP_COLSCORE, ctypes.byref(a), ctypes.byref(good_layout().c))
    assert need == 2 * 1 * 22 * 4


def test_attention_fwd_validation(lib):
    lay = good_layout()
    f = lib.tsel_attention_fwd
    a = attn(dtype=B.TSEL_F32)
    assert f(ctypes.byref(a), ctypes.byref(lay.c), FAKE, 256, 128, FAKE, 1024, 128, FAKE, None) == \
        B.TSEL_EUNSUPPORTED
    assert "bf16 or f16" in last_error(lib)
    a = attn()
    assert f(ctypes.byref(a), ctypes.byref(lay.c), None, 256, 128, FAKE, 1024, 128, FAKE, None) == B.TSEL_EINVAL
    assert f(ctypes.byref(a), ctypes.byref(lay.c), FAKE + 8, 256, 128, FAKE, 1024, 128, FAKE, None) == \
        B.TSEL_EINVAL
    assert f(ctypes.byref(a), ctypes.byref(lay.c), FAKE, 256, 128, FAKE + 2, 1024, 128, FAKE, None) == \
        B.TSEL_EINVAL
    assert f(ctypes.byref(a), ctypes.byref(lay.c), FAKE, 250, 128, FAKE, 1024, 128, FAKE, None) == B.TSEL_EINVAL
    assert f(ctypes.byref(a), ctypes.byref(lay.c), FAKE, 256, 128, FAKE, 1023, 128, FAKE, None) == B.TSEL_EINVAL
    # Token strides below head_dim (rows overlapping in memory) are refused for k and for v.
    assert f(ctypes.byref(a), ctypes.byref(lay.c), FAKE, 64, 128, FAKE, 1024, 128, FAKE, None) == \
        B.TSEL_EUNSUPPORTED
    assert "token strides" in last_error(lib)
    a.k_stride_tok = 64
    assert f(ctypes.byref(a), ctypes.byref(lay.c), FAKE, 256, 128, FAKE, 1024, 128, FAKE, None) == \
        B.TSEL_EUNSUPPORTED


def test_mrope_validation(lib):
    lay = good_layout()
    f = lib.tsel_mrope_positions
    assert f(ctypes.byref(lay.c), FAKE, FAKE, -1, FAKE, FAKE, 64, None) == B.TSEL_EINVAL
    assert f(ctypes.byref(lay.c), None, FAKE, 4, FAKE, FAKE, 64, None) == B.TSEL_EINVAL
    need = lib.tsel_workspace_size(B.TSEL_OP_MROPE, None, ctypes.byref(lay.c))
    assert need == 4 * 2
    assert f(ctypes.byref(lay.c), FAKE, FAKE, 4, FAKE, FAKE, need - 1, None) == B.TSEL_EWORKSPACE


def test_compact_rejects_inconsistent_embedding_args(lib):
    lay = good_layout()
    comp = lib.tsel_workspace_size(B.TSEL_OP_COMPACT, None, ctypes.byref(lay.c))
    rc = lib.tsel_compact(ctypes.byref(lay.c), FAKE, FAKE, 64, 128, 10, FAKE, 128, FAKE, None, None,
                          None, FAKE, comp, None)
    assert rc == B.TSEL_EINVAL


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        B.lib()


# ---------------------------------------------------------------------------
# The C ABI from C: the header alone compiles as strict C99 and as C++11, and
# a plain-C program (tests/c_consumer) links the library and sees its
# validation contract.  No GPU is touched.
# ---------------------------------------------------------------------------

def test_header_is_plain_c_and_cpp(tmp_path):
    src = tmp_path / "hdr.c"
    src.write_text('#include "tsel.h"\nint main(void) { return tsel_version() == TSEL_VERSION ? 0 : 1; }\n')
    inc = os.path.dirname(HEADER)
    for cmd in (["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-fsyntax-only"],
                ["g++", "-std=c++11", "-Wall", "-Wextra", "-pedantic", "-Werror", "-fsyntax-only", "-x", "c++"]):
        r = subprocess.run(cmd + ["-I", inc, str(src)], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr


def test_c_consumer_host_checks(lib):
    sys.path.insert(0, os.path.join(os.path.dirname(__file__), "c_consumer"))
    import build_consumer
    exe = build_consumer.BIN if os.path.exists(build_consumer.BIN) else build_consumer.build()
    r = subprocess.run([exe, "check"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "check ok" in r.stdout
