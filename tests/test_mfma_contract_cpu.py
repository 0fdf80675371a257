"""The hazard contract of the 256-tile kernel's inline-asm MFMAs, checked on
the compiled gfx950 code (no GPU needed).

The accumulating MFMA is inline asm with a tied accumulator operand, so the
compiler treats it as finishing at once, while the hardware writes the result
over its later passes.  The kernel is correct only if nothing but MFMAs
touches an accumulator between the first and the last MFMA (no register
copies of accumulators, no other value placed in an accumulator register):
a copy there would read a half-written result.  The compiler may insert such
copies under register pressure, so every gemm256_kernel instance is compiled
to assembly with the library's own flags and checked:
  * its MFMAs use exactly FM·FN·4 = 128 accumulator registers, VGPRs or
    AGPRs (each accumulator in one place for the whole k-loop);
  * between its first and last MFMA no other instruction reads or writes one
    of them (VALU, VMEM address operands, LDS read destinations).
"""
import concurrent.futures
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from muon_newton_schulz_06_amd import build  # noqa: E402

SOURCES = ["gemm_syrk", "gemm_sq", "gemm_axpy", "gemm_final"]
REG = re.compile(r"\b([va])\[(\d+):(\d+)\]|\b([va])(\d+)\b")


def vregs(text):
    """Vector registers named in text, as (file, index): file 'v' or 'a'."""
    out = set()
    for m in REG.finditer(text):
        if m.group(1):
            out |= {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
        else:
            out.add((m.group(4), int(m.group(5))))
    return out


def assembly(src):
    cmd = [build.hipcc(), *build.flags(), "-S", "--cuda-device-only", "-o", "-",
           os.path.join(build.CSRC, src + ".hip")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr[-2000:]}")
    return r.stdout


def violations(asm):
    """(kernel, MFMA count, accumulator registers, offending lines) per gemm256_kernel."""
    out = []
    for kern in re.findall(r"^(_ZN4muon14gemm256_kernel\w+):", asm, re.M):
        body = asm.split(kern + ":", 1)[1].split("s_endpgm", 1)[0].splitlines()
        mf = [i for i, line in enumerate(body) if "v_mfma" in line]
        accs = set()
        for i in mf:
            accs |= vregs(body[i].split("v_mfma", 1)[1].split(None, 1)[1].split(",")[0])
        bad = []
        for line in body[mf[0]:mf[-1] + 1] if mf else []:
            t = line.strip()
            if not t or t.startswith((";", ".")) or "v_mfma" in t:
                continue
            parts = t.split(None, 1)
            ins, ops = parts[0], parts[1] if len(parts) > 1 else ""
            if ins.startswith("s_"):
                continue  # scalar code: no VGPR operands
            if vregs(ops.split(";")[0]) & accs:
                bad.append(t)
        out.append((kern, len(mf), len(accs), bad))
    return out


@pytest.fixture(scope="module")
def compiled():
    try:
        build.hipcc()
    except RuntimeError as e:
        pytest.skip(str(e))
    with concurrent.futures.ThreadPoolExecutor(len(SOURCES)) as ex:
        return dict(zip(SOURCES, ex.map(assembly, SOURCES)))


def test_accumulators_are_touched_only_by_mfmas(compiled):
    seen = 0
    for src, asm in compiled.items():
        for kern, n_mfma, n_acc, bad in violations(asm):
            seen += 1
            assert n_mfma > 0, (src, kern)
            assert n_acc == 128, (src, kern, n_acc, "accumulators moved between registers")
            assert not bad, (src, kern, bad[:5])
    assert seen >= 9  # SYRK, A², a·Y + B·Y, and the final product's 6 variants


def test_checker_flags_a_copied_accumulator():
    """The checker itself: an accumulator copied between MFMAs is flagged."""
    asm = "\n".join([
        "_ZN4muon14gemm256_kernelILi0ELi0EEEvNS_10GemmLaunchE:",
        "\tv_mfma_f32_16x16x32_f16 v[0:3], v[200:203], v[204:207], v[0:3]",
        "\tv_mov_b32_e32 v250, v1",
        "\tglobal_load_lds_dwordx4 v[2:3], off",
        "\tds_read_b128 v[4:7], v240",
        "\tv_mfma_f32_16x16x32_f16 v[4:7], v[200:203], v[204:207], v[4:7]",
        "\ts_endpgm",
    ])
    ((kern, n_mfma, n_acc, bad),) = violations(asm)
    assert n_mfma == 2 and n_acc == 8
    assert len(bad) == 3


def test_checker_flags_a_copied_agpr_accumulator():
    """The same for accumulators held in AGPRs: a read-out between MFMAs is
    flagged, and v0 is not confused with a0."""
    asm = "\n".join([
        "_ZN4muon14gemm256_kernelILi1ELi0EEEvNS_10GemmLaunchE:",
        "\tv_mfma_f32_16x16x32_f16 a[0:3], v[0:3], v[4:7], a[0:3]",
        "\tv_add_f32_e32 v8, v0, v1",
        "\tv_accvgpr_read_b32 v9, a2",
        "\tv_mfma_f32_16x16x32_f16 a[4:7], v[0:3], v[4:7], a[4:7]",
        "\ts_endpgm",
    ])
    ((kern, n_mfma, n_acc, bad),) = violations(asm)
    assert n_mfma == 2 and n_acc == 8
    assert bad == ["v_accvgpr_read_b32 v9, a2"]
