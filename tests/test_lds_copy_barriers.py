"""The streamed tiles reach LDS through LDS-direct buffer loads, which each wave
issues for its own share of a tile and which complete only when that wave's
vector-memory counter drains.  A tile is read by every wave of the workgroup,
so each wave must wait for its copies before the barrier that precedes the
reads: a barrier reached while a copy may still be in flight lets another wave
read a half-written tile.  Likewise every LDS read of a stage must have
returned before the barrier after which a copy into that stage may start.  The
kernels leave both waits to the compiler (the workgroup fence of
__syncthreads() drains both counters; the reads of one stage are not made to
wait for a copy into the other).  This test compiles the kernel sources for
gfx950 with the library's flags and checks the emitted code: along every
control-flow path of every kernel, no s_barrier is reached after an LDS-direct
load without an s_waitcnt vmcnt(0) in between, nor after an LDS read without an
s_waitcnt lgkmcnt(0) in between.  Planted snippets pin the checker itself.
CPU only (cross-compiles; nothing runs on a GPU)."""
import os
import re
import subprocess

import pytest

from attention_score_selection_amd import build

CSRC = build.CSRC


def _functions(lines):
    name, body = None, []
    for ln in lines:
        m = re.match(r"^(_Z\S+):", ln)
        if m:
            if name:
                yield name, body
            name, body = m.group(1), []
            continue
        if name is None:
            continue
        if ".Lfunc_end" in ln:
            yield name, body
            name = None
            continue
        body.append(ln)
    if name:
        yield name, body


def _blocks(body):
    """Basic blocks (a new one at every label and after every branch) and
    their successors."""
    blocks, cur = [], {"label": None, "ins": []}
    for ln in body:
        m = re.match(r"^(\.LBB\w+):", ln.strip())
        if m:
            blocks.append(cur)
            cur = {"label": m.group(1), "ins": []}
            continue
        t = ln.split(";")[0].strip()
        if not t or t.startswith("."):
            continue
        cur["ins"].append(t)
        if re.match(r"^s_c?branch", t):
            blocks.append(cur)
            cur = {"label": None, "ins": []}
    blocks.append(cur)
    where = {b["label"]: i for i, b in enumerate(blocks) if b["label"]}
    succ = []
    for i, b in enumerate(blocks):
        s, falls = [], True
        for t in b["ins"]:
            m = re.match(r"^s_(c?branch\w*)\s+(\.LBB\w+)", t)
            if m:
                s.append(where[m.group(2)])
                falls = falls and m.group(1) != "branch"
            if t.startswith("s_endpgm") or t.startswith("s_setpc"):
                falls = False
        if falls and i + 1 < len(blocks):
            s.append(i + 1)
        succ.append(s)
    return blocks, succ


LDS_COPY = (r"^buffer_load_\w+\s.*\blds\b", "vmcnt(0)")   # LDS-direct load, drained by vmcnt(0)
LDS_READ = (r"^ds_(read|load)", "lgkmcnt(0)")                # LDS read, drained by lgkmcnt(0)


def _step(ins, pending, kind, found=None):
    for t in ins:
        if re.match(kind[0], t):
            pending = True
        elif t.startswith("s_waitcnt") and kind[1] in t:
            pending = False
        elif t.startswith("s_barrier") and pending and found is not None:
            found.append(t)
    return pending


def unsafe_barriers(asm_text, kind=LDS_COPY):
    """(kernel, barriers, LDS-direct loads, barriers reachable with an access
    of `kind` in flight) per kernel of an assembly listing: a forward
    may-analysis, the in-flight flag joined by OR where paths meet."""
    out = []
    for name, body in _functions(asm_text.splitlines()):
        blocks, succ = _blocks(body)
        state_in = [False] * len(blocks)
        changed = True
        while changed:
            changed = False
            for i, b in enumerate(blocks):
                if _step(b["ins"], state_in[i], kind):
                    for j in succ[i]:
                        if not state_in[j]:
                            state_in[j] = changed = True
        bad = []
        for i, b in enumerate(blocks):
            _step(b["ins"], state_in[i], kind, bad)
        nbar = sum(t.startswith("s_barrier") for b in blocks for t in b["ins"])
        ndma = sum(bool(re.match(r"^buffer_load_\w+\s.*\blds\b", t)) for b in blocks for t in b["ins"])
        out.append((name, nbar, ndma, len(bad)))
    return out


PLANTED_BAD = """_Zbad:
\tbuffer_load_dwordx4 v2, s[4:7], 0 offen lds
\ts_cbranch_scc1 .LBB0_2
\ts_waitcnt vmcnt(0)
.LBB0_2:
\ts_barrier
\ts_endpgm
.Lfunc_end0:
"""
PLANTED_LOOP = """_Zloop:
.LBB1_1:
\ts_barrier
\tbuffer_load_dwordx4 v2, s[4:7], 0 offen lds
\ts_cbranch_scc1 .LBB1_1
\ts_waitcnt vmcnt(0)
\ts_endpgm
.Lfunc_end1:
"""
PLANTED_GOOD = """_Zgood:
\tbuffer_load_dwordx4 v2, s[4:7], 0 offen lds
\ts_cbranch_scc1 .LBB2_2
\tv_mov_b32 v1, 0
.LBB2_2:
\ts_waitcnt vmcnt(0) lgkmcnt(0)
\ts_barrier
\ts_endpgm
.Lfunc_end2:
"""


def test_checker_catches_planted_races():
    # A branch around the wait, and a loop whose back edge carries a copy to
    # the barrier, are both flagged; a wait on every path is not.
    assert unsafe_barriers(PLANTED_BAD)[0][3] == 1
    assert unsafe_barriers(PLANTED_LOOP)[0][3] == 1
    assert unsafe_barriers(PLANTED_GOOD)[0][3] == 0
    read = "_Zread:\n\tds_read_b128 v[0:3], v4\n\ts_waitcnt vmcnt(0)\n\ts_barrier\n\ts_endpgm\n.Lfunc_end3:\n"
    assert unsafe_barriers(read, LDS_READ)[0][3] == 1
    assert unsafe_barriers(read.replace("vmcnt(0)", "lgkmcnt(0)"), LDS_READ)[0][3] == 0


@pytest.mark.parametrize("src", ["attn.hip", "fwd.hip"])
def test_no_barrier_with_lds_copy_in_flight(tmp_path, src):
    asm = tmp_path / (src + ".s")
    cmd = [build.hipcc(), *build.compile_flags(), "-x", "hip", "--offload-device-only", "-S",
           os.path.join(CSRC, src), "-o", str(asm)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    res = unsafe_barriers(asm.read_text())
    streamed = [x for x in res if x[2] > 0]
    assert streamed, "no kernel with LDS-direct loads found"
    print(f"{src}: {len(streamed)} kernels with LDS-direct loads, "
          f"{sum(x[1] for x in streamed)} barriers, {sum(x[2] for x in streamed)} loads")
    bad = [(n[:80], k) for n, _, _, k in res if k]
    assert not bad, f"barriers reachable with an LDS-direct load in flight: {bad}"
    bad = [(n[:80], k) for n, _, _, k in unsafe_barriers(asm.read_text(), LDS_READ) if k]
    assert not bad, f"barriers reachable with an LDS read in flight: {bad}"
