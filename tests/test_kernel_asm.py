"""The GEMM kernels' machine code, checked on the host (hipcc cross-compiles for gfx950):

* no kernel uses scratch memory or spills a vector register: a spilled vector register
  goes through scratch loads and stores, which the vector-memory counter counts too, so
  a spill would silently break the hand-counted waits of the tile and strip kernels
  (scalar registers spill into lanes of vector registers, without memory, and are
  allowed);
* in every main loop of the tile kernel the wait before each barrier allows exactly the
  loads issued since the stage it publishes: with LD direct-to-LDS loads (the stages) and
  LW register loads (the weights) per step, 2 LD + 3 LW where the weights go out a step
  early (the folding waves), 2 (LD + LW) otherwise: every load the waits count is one the
  code actually emits.
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
    """(kernel, loads per step as (direct-to-LDS, register) counts, [wait before each
    barrier]) of each loop inside a tile kernel's body that has barriers."""
    cur, out = None, []
    for i, line in enumerate(lines):
        m = re.match(r"^(_ZN\S*gemm_tile_kernel\S*):", line)
        if m:
            cur = m.group(1)
        elif re.match(r"^_ZN\S*:", line) or line.startswith(".Lfunc_end"):
            cur = None
        if cur and "Loop Header" in line:
            j, nb, ld, lw, waits, last = i + 1, 0, 0, 0, [], None
            while not re.search(r"s_cbranch_scc[01] \.LBB", lines[j]):
                t = lines[j].strip()
                if t.startswith(("buffer_load", "global_load")):
                    if re.search(r"\blds\b", t):
                        ld += 1
                    else:
                        lw += 1
                m2 = re.search(r"vmcnt\((\d+)\)", t)
                if m2:
                    last = int(m2.group(1))
                if t.startswith("s_barrier"):
                    nb += 1
                    waits.append(last)
                j += 1
            if nb:
                assert ld % nb == 0 and lw % nb == 0, (cur, ld, lw, nb)
                out.append((cur, (ld // nb, lw // nb), waits))
    return out


def test_tile_waits_match_the_loads(asm):
    loops = _tile_loops(asm)
    assert len(loops) >= 12
    for name, (ld, lw), waits in loops:
        assert ld > 0, name
        expect = 2 * ld + 3 * lw if lw and "Lb0" in name else 2 * (ld + lw)
        assert waits == [expect] * len(waits), (name, ld, lw, waits)
