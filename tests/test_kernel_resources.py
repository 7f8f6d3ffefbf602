"""Build-time guard of the main pass's copy pipeline (CPU only; compiles the
kernels for gfx950 with hipcc, no GPU).

The key/value-stationary pass copies the Q / dO tiles of pair i + 2 straight
into LDS and, before the barrier that publishes them, waits with an explicit
vector-memory count that assumes exactly which memory operations were issued
after those copies (the lse / Delta loads and the previous pair's 8 dQ
atomics).  A register spill inside that loop would add scratch loads or
stores to the count and let the barrier publish a tile that has not landed.
This test compiles bwd.hip to assembly and requires that no scratch
instruction sits in any loop that issues direct-to-LDS copies, for every
instantiation; it also bounds the spills the compiler reports per kernel
(bwd_kernel: at most two VGPRs, spilled before and reloaded after its loop
in some D = 128 variants; the forward and the dQ pass wait for all their
copies with a zero count, so their spills cannot break a count)."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "atomics_bwd_preprocess_amd", "csrc")

HIPCC = shutil.which("hipcc") or ("/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc")
                                  else None)
pytestmark = pytest.mark.skipif(HIPCC is None, reason="hipcc not available")


def _compile_asm(src: str, tmp_path) -> tuple:
    out = os.path.join(str(tmp_path), os.path.basename(src) + ".s")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "--cuda-device-only", "-S", src, "-o", out, "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=CSRC)
    assert r.returncode == 0, r.stderr[-4000:]
    return open(out).read(), r.stderr


def _functions(asm: str) -> dict:
    """Kernel name -> its assembly lines (from its label to its end marker)."""
    out = {}
    for m in re.finditer(r"^(_ZN4attn\S*_kernel\S*):\s*(?:;.*)?$", asm, flags=re.M):
        name = m.group(1)
        end = asm.find(f".Lfunc_end", m.end())
        out[name] = asm[m.end():end].split("\n")
    return out


def _loops(lines: list) -> dict:
    """Top-level loop header -> the lines of every block inside that loop
    (the compiler annotates each block with the loop it belongs to)."""
    blocks, cur = [], None
    for ln in lines:
        if re.match(r"^(\.LBB\S+:|; %bb\.\d+:)", ln):
            cur = [ln]
            blocks.append(cur)
        elif cur is not None:
            cur.append(ln)
    loops = {}
    for b in blocks:
        head = b[0]
        m = re.match(r"^\.L(BB\d+_\d+):.*Loop Header: Depth=1", head)
        if m:
            loops.setdefault(m.group(1), []).extend(b)
            continue
        m = re.search(r"(?:in Loop: Header|Parent Loop) (BB\d+_\d+) Depth=1", head) or \
            re.search(r"in Loop: Header=(BB\d+_\d+) Depth=1", head)
        if m:
            loops.setdefault(m.group(1), []).extend(b)
    return loops


def _remarks(stderr: str) -> dict:
    """Kernel name -> {'vgpr_spill': n, 'scratch': bytes} from the
    kernel-resource-usage remarks."""
    out, name = {}, None
    for ln in stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", ln)
        if m:
            name = m.group(1)
            out[name] = {}
            continue
        m = re.search(r"VGPRs Spill: (\d+)", ln)
        if m and name:
            out[name]["vgpr_spill"] = int(m.group(1))
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", ln)
        if m and name:
            out[name]["scratch"] = int(m.group(1))
    return out


def test_no_scratch_in_the_copy_pipelined_loops(tmp_path):
    asm, err = _compile_asm(os.path.join(CSRC, "bwd.hip"), tmp_path)
    funcs = {n: f for n, f in _functions(asm).items() if "bwd_kernel" in n}
    assert len(funcs) >= 20, sorted(funcs)
    pipelined, bad = 0, []
    for name, lines in funcs.items():
        for head, body in _loops(lines).items():
            text = "\n".join(body)
            if re.search(r"buffer_load_dword\S*\s.*\blds\b", text):
                pipelined += 1
                bad += [(name, head, ln.strip()) for ln in body if "scratch_" in ln]
    assert not bad, f"scratch access in a copy loop: {bad[:4]}"
    assert pipelined >= len(funcs)  # every instantiation has its pair loop
    rem = _remarks(err)
    for name in funcs:
        assert rem[name]["vgpr_spill"] <= 2 and rem[name]["scratch"] <= 16, (name, rem[name])


@pytest.mark.parametrize("src,kernel,max_spill", [("dq.hip", "dq_kernel", 1),
                                                  ("fwd.hip", "fwd_kernel", 0)])
def test_other_passes_wait_for_all_copies(src, kernel, max_spill, tmp_path):
    # Only the main pass waits with a nonzero count; the others wait for
    # every outstanding copy, which a spill cannot break.
    text = open(os.path.join(CSRC, src)).read()
    assert "kVmcnt0 +" not in text and "kVmcnt0+" not in text
    _, err = _compile_asm(os.path.join(CSRC, src), tmp_path)
    rem = {n: r for n, r in _remarks(err).items() if kernel in n}
    assert rem
    for name, r in rem.items():
        assert r["vgpr_spill"] <= max_spill, (name, r)
