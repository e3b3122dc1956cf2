"""Properties of the compiled device code that the kernels' speed relies on
(no GPU needed: hipcc cross-compiles for gfx950 here).

* The fp8 decode kernel keeps its whole working set in registers: any scratch
  use puts spill traffic next to the gather stream (a spill inside the tile
  loop costs several per cent).  The bf16 kernel may keep a few per-piece
  values in scratch, never more than a small bound.
* Packed-fp32 VALU instructions are disabled for device code by a build flag;
  none may appear in the output.
"""

import os
import re
import subprocess

import pytest

from mla_latent_attention_amd import build

SRC = os.path.join(build.CSRC, "mla_decode.hip")


@pytest.fixture(scope="module")
def compiled(tmp_path_factory):
    out = tmp_path_factory.mktemp("asm") / "mla_decode.s"
    flags = [f for f in build.FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [build.hipcc(), *flags, "--cuda-device-only", "-S", SRC, "-o", str(out),
           "-Rpass-analysis=kernel-resource-usage"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    usage, name = {}, None
    for line in res.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name:
            usage[name] = int(m.group(1))
    return out.read_text(), usage


def _scratch(usage, needle):
    hits = [v for k, v in usage.items() if needle in k]
    assert hits, f"kernel {needle} not found in {list(usage)}"
    return hits[0]


def test_fp8_decode_kernel_uses_no_scratch(compiled):
    _, usage = compiled
    assert _scratch(usage, "mla_decode_fp8_kernel") == 0


def test_bf16_decode_kernel_scratch_is_small(compiled):
    _, usage = compiled
    assert _scratch(usage, "mla_decode_bf16_kernel") <= 64


def test_no_packed_fp32_valu(compiled):
    asm, _ = compiled
    assert not re.search(r"\bv_pk_(add|mul|fma)_f32\b", asm)
