"""Static checks of the grouped GEMM's gfx950 assembly (hipcc, no GPU).

* No transposing LDS read (`ds_read_b64_tr_b16`) may directly follow an
  `s_waitcnt vmcnt(0)`: the compiler puts one there when it sees a direct
  global->LDS load in flight, which makes every reduction step wait for the
  loads it has just issued for a later step.  The stage loads are issued by
  inline assembly for that reason; this test fails if the wait comes back.
* Every assembly block that issues direct global->LDS loads opens with
  `s_nop 4` (a vector-memory read of an SGPR needs five wait states after a
  vector instruction wrote it, which the compiler does not insert before
  assembly) and sets M0 one wait state before each load.
* The large kernels spill no vector registers.
"""
import os
import re
import shutil
import subprocess

import pytest

from scale_only_quantization_amd import build as B

HIPCC = B.HIPCC


@pytest.fixture(scope="module")
def gemm_asm(tmp_path_factory):
    if not (os.path.exists(HIPCC) or shutil.which(HIPCC)):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("isa") / "fq_gemm.s"
    cmd = [HIPCC, *B.FLAGS, "--cuda-device-only", "-S", os.path.join(B.CSRC, "fq_gemm.hip"), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text().split("\n")


def _instructions(lines):
    """(index, text) of the instructions: no labels, comments or directives."""
    for i, l in enumerate(lines):
        t = l.strip()
        if not t or t.startswith((";", ".")) or t.endswith(":"):
            continue
        yield i, t


def test_no_load_wait_before_transposing_reads(gemm_asm):
    prev = None
    bad = []
    n_tr = 0
    for i, t in _instructions(gemm_asm):
        if t.startswith("ds_read_b64_tr_b16"):
            n_tr += 1
            if prev is not None and re.match(r"s_waitcnt\s+vmcnt\(0\)\s*$", prev[1]):
                bad.append(prev[0])
        prev = (i, t)
    assert n_tr > 100, "no transposing reads found: the kernel changed shape"
    assert not bad, f"s_waitcnt vmcnt(0) right before a transposing LDS read at lines {bad[:10]}"


def test_assembly_stage_loads_keep_their_wait_states(gemm_asm):
    blocks = 0
    i = 0
    L = gemm_asm
    while i < len(L):
        if "ASMSTART" in L[i]:
            j = i + 1
            body = []
            while j < len(L) and "ASMEND" not in L[j]:
                t = L[j].strip()
                if t and not t.startswith(";"):
                    body.append(t)
                j += 1
            if any(b.startswith("buffer_load") and b.endswith("lds") for b in body):
                blocks += 1
                assert re.match(r"s_nop\s+([4-9]|1[0-5])\b", body[0]), f"line {i}: {body[:2]}"
                for k, b in enumerate(body):
                    if b.startswith("buffer_load"):
                        assert k >= 2 and body[k - 1].startswith("s_nop") and "m0" in body[k - 2], f"line {i}"
            i = j
        i += 1
    assert blocks >= 10


def test_large_kernels_do_not_spill(gemm_asm):
    text = "\n".join(gemm_asm)
    spills = {}
    for blk in text.split("- .agpr_count:")[1:]:
        name = re.search(r"\.name:\s+(\S+)", blk).group(1)
        if "k_gemm" not in name:
            continue
        spills[name] = int(re.search(r"\.vgpr_spill_count:\s+(\d+)", blk).group(1))
    assert spills, "no k_gemm kernels in the metadata"
    assert all(v == 0 for v in spills.values()), spills
