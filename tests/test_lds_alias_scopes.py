"""The prefill GEMM's stage loads are the compiler's buffer->LDS builtin, so
the compiler's wait analysis sees them.  It tells the ring stages apart only
through the alias scope of each LDS access (every stage is a __shared__
array of its own): an LDS read without one would make the compiler wait for
every stage load in flight before it, draining the ring once per K block
(this happened to the MX weight-scale byte reads, 11-17 % slower).  Checks,
on the machine code before wait insertion, that every LDS read of the six
prefill kernel instances carries an alias scope, and, on the final assembly,
that the compiler's full waits for every load stay few (CPU only: hipcc
cross-compiles for gfx950)."""
import os
import re
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from sparse_moe_layer_fp32_amd import build as b  # noqa: E402

KERNELS = [f"_ZN3moe12_GLOBAL__N_124grouped_gemm_wide_kernelILb{g}ELb{m}ELb{f}EEEvNS_8GemmArgsE"
           for g in (0, 1) for m, f in ((0, 0), (1, 0), (1, 1))]


@pytest.mark.skipif(not os.path.exists(b.HIPCC) and shutil.which("hipcc") is None, reason="no hipcc")
def test_prefill_lds_reads_carry_alias_scopes(tmp_path):
    src = os.path.join(b.CSRC, "gemm.hip")
    cmd = [b.HIPCC, *b.FLAGS, *b.EXTRA["gemm.hip"], "--cuda-device-only", "-c", src,
           "-o", str(tmp_path / "gemm.o"), "-mllvm", "-print-before=si-insert-waitcnts",
           "-mllvm", "-filter-print-funcs=" + ",".join(KERNELS)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    text = r.stdout + r.stderr
    # one machine function dump per kernel instance
    parts = re.split(r"# Machine code for function ", text)[1:]
    seen = {}
    for part in parts:
        name = part.split(":", 1)[0].strip()
        reads = [ln for ln in part.splitlines() if re.search(r"= DS_READ", ln)]
        seen[name] = reads
    assert set(seen) == set(KERNELS), sorted(seen)
    for name, reads in seen.items():
        assert len(reads) > 100, (name, len(reads))
        bare = [ln.strip()[:160] for ln in reads if "alias.scope" not in ln]
        assert not bare, (name, bare[:3])


@pytest.mark.skipif(not os.path.exists(b.HIPCC) and shutil.which("hipcc") is None, reason="no hipcc")
def test_prefill_kernels_do_not_drain_the_ring(tmp_path):
    """The ring waits are explicit counts, chosen per path by the number of
    operations a wave has in flight.  Where the compiler cannot follow which
    count a path carries, it waits for every load before the LDS reads that
    may alias a stage in flight: a full drain, once per step.  A branch that
    left a wave's epilogue issuing 12 or 18 stores made it do so (229 drains
    per kernel instead of 16-17, the prologue, the end and the one-block
    paths).  Bounds the drains of every prefill kernel instance (CPU only)."""
    src = os.path.join(b.CSRC, "gemm.hip")
    out = tmp_path / "gemm.s"
    cmd = [b.HIPCC, *b.FLAGS, *b.EXTRA["gemm.hip"], "--cuda-device-only", "-S", src, "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    asm = out.read_text()
    for name in KERNELS:
        a = asm.index("\n" + name + ":")
        body = asm[a:asm.index(".Lfunc_end", a)]
        drains = len(re.findall(r"s_waitcnt vmcnt\(0\)", body))
        waits = len(re.findall(r"s_waitcnt vmcnt", body))
        assert drains <= 24 and waits <= 80, (name, drains, waits)
