"""Properties of the gfx950 code the compiler makes from the kernel sources
(CPU only: hipcc cross-compiles to assembly, nothing runs).

- Every DPP lane move (v_mov_b32_dpp) runs with the full execution mask: a DPP
  move reads its source lane whether or not that lane is active, and reading
  an inactive lane gives no defined value.  The kernels combine rotated values
  with bit masks and keep loop control uniform so that no move lands inside a
  region where part of the wavefront is switched off.
- No kernel spills scalar or vector registers and none uses scratch memory.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "lora_adapter_pool_amd", "csrc")


def _hipcc():
    cand = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    return cand if os.path.exists(cand) else shutil.which("hipcc")


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    cc = _hipcc()
    if not cc:
        pytest.skip("hipcc not available")
    text = []
    for src in sorted(f for f in os.listdir(CSRC) if f.endswith(".hip")):
        out = tmp_path_factory.mktemp("isa") / (src + ".s")
        cmd = [cc, "-O3", "-std=c++17", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", "-x",
               "hip", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
               "-packed-fp32-ops", "--cuda-device-only", "-S", "-o", str(out),
               os.path.join(CSRC, src)]
        subprocess.run(cmd, check=True, capture_output=True, text=True)
        text.append(out.read_text())
    return "\n".join(text)


def _kernels(text):
    """(name, body lines) of every function in the assembly."""
    cur, body = None, []
    for line in text.split("\n"):
        m = re.match(r"^(_Z\w+):", line)
        if m:
            if cur:
                yield cur, body
            cur, body = m.group(1), []
        elif cur:
            body.append(line.strip())
            if line.startswith(".Lfunc_end"):
                yield cur, body
                cur, body = None, []


def test_dpp_moves_run_with_full_exec(asm):
    narrowing = re.compile(r"s_(and|andn2|or|xor)_saveexec_b64|s_(mov|and|andn2|xor)_b64 exec,")
    restore = re.compile(r"s_or_b64 exec, exec,")
    moves, bad = 0, []
    for name, body in _kernels(asm):
        depth = 0
        for ins in body:
            if narrowing.match(ins):
                depth += 1
            elif restore.match(ins):
                depth = 0
            if "_dpp" in ins:
                moves += 1
                if depth:
                    bad.append(name)
                    break
    assert moves > 0, "the decode kernels use DPP row rotates"
    assert not bad, f"DPP moves inside an exec-narrowed region: {bad[:3]}"


def test_no_spills_or_scratch(asm):
    sizes = re.findall(r"\.amdhsa_private_segment_fixed_size (\d+)", asm)
    assert sizes and all(int(v) == 0 for v in sizes), "a kernel uses scratch memory"
    for key in ("sgpr_spill_count", "vgpr_spill_count"):
        counts = re.findall(rf"\.{key}:\s+(\d+)", asm)
        assert counts and all(int(c) == 0 for c in counts), f"a kernel has {key} > 0"
