"""Machine-code checks of the split kernel (no GPU needed): hipcc compiles the
kernels for gfx950 and the assembly is checked for MFMA result hazards the
compiler cannot see through inline asm, and for scratch traffic in the tile
loop (each scratch reload there waits for every tile load in flight)."""
import os
import re
import shutil
import subprocess

import pytest

from tests import asm_hazards

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "deepseek_mla_decode_amd", "csrc", "mla_kernels.hip")


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    from deepseek_mla_decode_amd import build
    out = tmp_path_factory.mktemp("asm") / "k.s"
    flags = [f for f in build.FLAGS if f not in ("-fPIC", "-shared")]
    subprocess.run([hipcc, *flags, "--cuda-device-only", "-S", "-o", str(out), SRC], check=True,
                   capture_output=True)
    return out.read_text()


def test_split_kernels_have_no_mfma_result_hazards(asm):
    found = asm_hazards.kernel_hazards(asm, "split_kernel")
    assert len(found) == 16, sorted(found)
    bad = {k: v[:5] for k, v in found.items() if v}
    assert not bad, bad


def test_checker_flags_a_planted_early_read(asm):
    """Plant a read of an MFMA accumulator right behind the MFMA."""
    lines = asm.split("\n")
    for n, x in enumerate(lines):
        m = re.search(r"v_mfma_f32_32x32x16_\w+ a\[(\d+):\d+\]", x)
        if m:
            lines.insert(n + 1, f"\tv_accvgpr_read_b32 v0, a{m.group(1)}")
            break
    found = asm_hazards.kernel_hazards("\n".join(lines), "split_kernel")
    assert any(p[0] == "R1" for v in found.values() for p in v)


def _loop_bodies(asm, kernel):
    """Lines of each innermost loop of `kernel`: its header block and every
    block the compiler's comments place in it (wherever the layout puts them)."""
    lines = asm.split("\n")
    start = next(i for i, l in enumerate(lines) if l.startswith(kernel + ":"))
    end = next((i for i in range(start + 1, len(lines)) if re.match(r"^_Z\w+:", lines[i])), len(lines))
    body = lines[start:end]
    blocks = []   # (label, comment text, lines)
    for i, x in enumerate(body):
        if re.match(r"^\.LBB\w+:", x):
            comment = x + (body[i + 1] if i + 1 < len(body) and body[i + 1].lstrip().startswith(";") else "")
            blocks.append((x.split(":")[0], comment, [x]))
        elif blocks:
            blocks[-1][2].append(x)
    for label, comment, blines in blocks:
        if "Inner Loop Header" in comment:
            tag = "Header=" + label.replace(".LBB", "BB")
            yield blines + [y for lab, com, bl in blocks if tag in com.split(";", 1)[-1] and lab != label for y in bl]


def test_tile_loops_do_not_touch_scratch(asm):
    kernels = sorted(set(re.findall(r"^(_ZN3mla12split_kernel\w+):", asm, flags=re.M)))
    assert len(kernels) == 16
    for k in kernels:
        loops = [b for b in _loop_bodies(asm, k) if sum("v_mfma" in y for y in b) >= 64]
        assert loops, f"{k}: tile loop not found"
        for b in loops:
            sc = [y.strip() for y in b if "scratch_" in y]
            assert not sc, f"{k}: scratch access in the tile loop: {sc[:3]}"
