"""Guard against a code-generation fault of the installed HIP compiler (CPU only).

The post-register-allocation run of the AMDGPU instruction-shrinking pass
deletes `vcc = S_AND_B64 vcc, exec` (the exec mask applied to a compare result
that feeds a uniform branch) as redundant for VCC, even when a later scalar
instruction (for example S_CSELECT) still reads the SCC bit that the AND set.
The reader then sees a stale SCC and the kernel computes a wrong value with no
error.  A Top-K kernel selected its radix prefix this way and lost ties.

This test compiles every library source for gfx950 with the library's own
flags, dumps the machine IR right before each run of that pass and fails if
any such AND still has an SCC reader, so a source change that reintroduces
the pattern is caught before it reaches a GPU.
"""
import os
import re
import subprocess
import tempfile

import pytest

from fp4_sparse_attention_amd import build as B

_AND = re.compile(r"\$vcc = S_AND_B64 (killed )?(renamable )?\$(vcc|exec), (killed )?(renamable )?\$(vcc|exec), "
                  r"implicit-def \$scc\s*$")
_READ = re.compile(r"implicit (killed )?\$scc")


def _live_scc_reads(mir: str):
    lines = mir.split("\n")
    hits = []
    for i, line in enumerate(lines):
        if not _AND.search(line):
            continue
        for j in range(i + 1, min(i + 60, len(lines))):
            nxt = lines[j]
            if _READ.search(nxt):
                hits.append((i + 1, line.strip(), nxt.strip()))
                break
            if "implicit-def $scc" in nxt or "implicit-def dead $scc" in nxt or nxt.strip().startswith("bb."):
                break
    return hits


@pytest.mark.skipif(not os.path.exists(B.HIPCC), reason="hipcc not installed")
@pytest.mark.parametrize("src", B.SOURCES)
def test_no_scc_reader_after_vcc_exec_and(src):
    with tempfile.TemporaryDirectory() as tmp:
        cmd = [B.HIPCC, *B.CFLAGS, "--cuda-device-only", "-c", os.path.join(B.CSRC, src),
               "-o", os.path.join(tmp, "dev.o"), "-mllvm", "-print-before=si-shrink-instructions"]
        p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
    assert p.returncode == 0, p.stderr[-2000:]
    if "__global__" in open(os.path.join(B.CSRC, src)).read():
        assert "S_ENDPGM" in p.stderr, "no machine IR was dumped"
    hits = _live_scc_reads(p.stderr)
    assert not hits, "\n".join(f"MIR line {n}: {a}\n    then {b}" for n, a, b in hits[:5])


def test_detector_finds_the_pattern():
    # a hand-written MIR fragment with the faulty shape, and one without it
    bad = ("  renamable $vcc = V_CMP_EQ_U32_e64 killed $vgpr2, $vgpr11, implicit $exec\n"
           "  renamable $vcc = S_AND_B64 killed renamable $vcc, $exec, implicit-def $scc\n"
           "  renamable $sgpr3 = S_CSELECT_B32 -1, killed renamable $sgpr3, implicit $scc\n")
    good = bad.replace("implicit-def $scc\n", "implicit-def dead $scc\n")
    assert len(_live_scc_reads(bad)) == 1
    assert _live_scc_reads(good) == []
