"""The GEMM kernels' machine code, checked on the host (hipcc cross-compiles for gfx950):

* no kernel uses scratch memory or spills a vector register: a spilled vector register
  goes through scratch loads and stores, which the vector-memory counter counts too, so
  a spill would silently break the hand-counted waits of the tile and strip kernels
  (scalar registers spill into lanes of vector registers, without memory, and are
  allowed);
* in every main loop of the tile kernel the wait before each barrier allows exactly the
  loads of the two steps issued since the stage it publishes, i.e. twice the loads the
  loop issues per step: every load the waits count is one the code actually emits.
"""
import os
import re
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "weight_activation_quantized_amd", "csrc", "mixllm_gemm.hip")


def _hipcc():
    for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    pytest.skip("hipcc not found")


@pytest.fixture(scope="module", params=["", "MIXLLM_FOLD_BIAS=1"])
def asm(request, tmp_path_factory):
    out = tmp_path_factory.mktemp("asm") / "gemm.s"
    cmd = [_hipcc(), "-x", "hip", "-std=c++17", "-O3", "-ffp-contract=off", "-fno-fast-math",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{os.path.dirname(SRC)}", "--offload-arch=gfx950",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "--offload-device-only", "-S",
           SRC, "-o", str(out)]
    if request.param:
        cmd.insert(4, "-D" + request.param)
    subprocess.run(cmd, check=True, capture_output=True, timeout=600)
    return out.read_text().split("\n")


def _kernel_meta(lines):
    text = "\n".join(lines)
    out = {}
    for block in text.split("  - .agpr_count:")[1:]:
        name = re.search(r"\.name:\s+(\S+)", block).group(1)
        out[name] = {k: int(re.search(rf"\.{k}:\s+(\d+)", block).group(1))
                     for k in ("private_segment_fixed_size", "vgpr_spill_count", "sgpr_spill_count")}
    return out


def test_no_kernel_uses_scratch(asm):
    meta = _kernel_meta(asm)
    assert any("gemm_tile_kernel" in n for n in meta)
    for name, m in meta.items():
        assert m["private_segment_fixed_size"] == 0 and m["vgpr_spill_count"] == 0, (name, m)


def _tile_loops(lines):
    """(kernel, [(loads, wait before the barrier) per barrier segment], loads after the
    last barrier) of each loop inside a tile kernel's body."""
    cur, out = None, []
    for i, line in enumerate(lines):
        m = re.match(r"^(_ZN\S*gemm_tile_kernel\S*):", line)
        if m:
            cur = m.group(1)
        elif re.match(r"^_ZN\S*:", line) or line.startswith(".Lfunc_end"):
            cur = None
        if cur and "Loop Header" in line:
            j, segs, loads, waits = i + 1, [], 0, []
            while not re.search(r"s_cbranch_scc[01] \.LBB", lines[j]):
                t = lines[j].strip()
                if t.startswith(("buffer_load", "global_load")):
                    loads += 1
                m2 = re.search(r"vmcnt\((\d+)\)", t)
                if m2:
                    waits.append(int(m2.group(1)))
                if t.startswith("s_barrier"):
                    segs.append((loads, waits[-1] if waits else None))
                    loads = 0
                j += 1
            if segs:
                out.append((cur, segs, loads))
    return out


def test_tile_waits_match_the_loads(asm):
    loops = _tile_loops(asm)
    assert len(loops) >= 12
    for name, segs, tail in loops:
        # the loop is rotated: the loads after its last barrier belong to the first step
        per_step = [tail] + [n for n, _ in segs[1:]]
        waits = [w for _, w in segs]
        assert len(set(per_step)) == 1 and per_step[0] > 0, (name, segs, tail)
        assert waits == [2 * per_step[0]] * len(waits), (name, segs, tail)
