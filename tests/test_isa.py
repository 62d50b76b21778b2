"""Checks on the library's compiled gfx950 code (CPU: hipcc cross-compiles).

The LDS transfers (buffer_load_dwordx4 ... lds, issued through inline asm)
set M0 to their LDS address and leave it there.  That is sound only while no
other instruction in the library reads M0: the compiler treats M0 as its own
and could otherwise rely on a value the transfers overwrite.  This test
compiles the kernels to assembly and checks that every instruction naming M0
is one of the transfers' own M0 writes, and that every LDS transfer follows
such a write.
"""
import os
import re
import shutil
import subprocess

import pytest

from normalization_gemm_amd import build as ngbuild

HIPCC = next((c for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc"))
              if c and os.path.exists(c)), None)


@pytest.fixture(scope="module")
def device_asm(tmp_path_factory):
    if HIPCC is None:
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("isa") / "ng_api.s"
    flags = [f for f in ngbuild.HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    src = os.path.join(ngbuild.CSRC, "ng_api.hip")
    res = subprocess.run([HIPCC, *flags, "--cuda-device-only", "-S", "-o", str(out), src],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return out.read_text()


# a transfer's M0 write: from a scalar register (the compiler may pick VCC's
# halves for the asm operand)
OWN_WRITE = r"^s_mov_b32 m0, (s\d+|vcc_lo|vcc_hi)$"


def _instructions(text):
    for line in text.splitlines():
        line = line.split(";")[0].strip()
        if line and not line.startswith(".") and not line.endswith(":"):
            yield line


def test_m0_is_written_only_by_the_lds_transfers(device_asm):
    own_write = re.compile(OWN_WRITE)
    naming_m0 = [i for i in _instructions(device_asm) if re.search(r"\bm0\b", i)]
    assert naming_m0, "no LDS transfer found in the compiled code"
    others = [i for i in naming_m0 if not own_write.match(i)]
    assert not others, others[:10]
    # instructions that read M0 implicitly
    implicit = re.compile(r"^(s_movrel|v_movrel|s_sendmsg|ds_gws|ds_\w*addtid|ds_append|"
                          r"ds_consume|s_set_gpr_idx|v_interp|v_readlane_b32 \S+, \S+, m0)")
    assert not [i for i in _instructions(device_asm) if implicit.match(i)]


def test_every_lds_transfer_follows_its_m0_write(device_asm):
    ins = list(_instructions(device_asm))
    n = 0
    for k, i in enumerate(ins):
        if re.match(r"^(buffer|global)_load\w* .*\blds$", i):
            n += 1
            assert ins[k - 1] == "s_nop 0" and re.match(OWN_WRITE, ins[k - 2]), \
                ins[k - 3:k + 1]
    assert n > 0
