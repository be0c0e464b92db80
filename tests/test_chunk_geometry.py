"""Host check of the column score's row-chunk geometry (the split of a long
segment's last chunk into pieces), compiled from the library's own header
with hipcc's host pass; no GPU needed."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def hipcc():
    path = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    return path if os.path.exists(path) else shutil.which("hipcc")


@pytest.mark.skipif(hipcc() is None, reason="hipcc is not installed")
def test_chunks_tile_every_segment(tmp_path):
    exe = str(tmp_path / "chunk_geometry")
    subprocess.run([hipcc(), "-O1", "-std=c++17", "-I", os.path.join(ROOT, "include"),
                    "-I", os.path.join(ROOT, "attention_score_selection_amd", "csrc"),
                    os.path.join(HERE, "host", "chunk_geometry.cpp"), "-o", exe],
                   check=True, capture_output=True, timeout=300)
    out = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0, out.stdout + out.stderr
    assert out.stdout.startswith("ok"), out.stdout


@pytest.mark.skipif(hipcc() is None, reason="hipcc is not installed")
def test_value_tile_transposing_reads(tmp_path):
    """The attention forward's value-fragment reads: each lane gets its keys
    and column, reads stay in the tile, no LDS bank is shared (host
    simulation of the transposing read's measured lane rule)."""
    exe = str(tmp_path / "vtile_geometry")
    r = subprocess.run([hipcc(), "-O1", "-std=c++17", "-x", "hip", "--offload-arch=gfx950",
                        "-I", os.path.join(ROOT, "include"),
                        "-I", os.path.join(ROOT, "attention_score_selection_amd", "csrc"),
                        os.path.join(HERE, "host", "vtile_geometry.cpp"), "-o", exe],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    out = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0, out.stdout + out.stderr
    assert out.stdout.startswith("ok"), out.stdout
