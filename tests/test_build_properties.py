"""Properties of the compiled device code that the kernels' speed relies on
(no GPU needed: hipcc cross-compiles for gfx950 here).

* The fp8 decode kernel keeps its whole working set in registers: any scratch
  use puts spill traffic next to the gather stream (a spill inside the tile
  loop costs several per cent).  The bf16 kernel may keep a few per-piece
  values in scratch, never more than a small bound.
* The group-mode kernel holds 256 accumulators per lane besides q; some
  per-piece values may sit in scratch (a bounded amount), but its tile loop
  (the blocks that hold the MFMA steps) touches no scratch.  It writes m0, which its inline-asm LDS DMA reads
  as the LDS destination, only in the instruction right before each DMA: the
  compiler itself then never sees a stale m0.
* No MFMA accumulates onto the result of an MFMA of another kind: gfx950
  returns garbage when a 16x16x32 fp8 MFMA reads the result of a 16x16x128
  f8f6f4 MFMA as its accumulator right behind it (or the other way round),
  and the compiler does not keep them apart, so accumulator chains stay
  within one instruction.
* Packed-fp32 VALU instructions are disabled for device code by a build flag;
  none may appear in the output.
* No register spill is stored while a divergent branch's narrowed exec mask
  is still in force at the branch's join (a scratch store right before the
  exec restore): only the branch's lanes would save the value, and the other
  lanes would reload stale data.  One kernel build showed exactly that (its
  partial-slot index was saved for one lane), so every build is scanned.
"""

import os
import re
import subprocess

import pytest

from mla_latent_attention_amd import build


def _compile(tmp_path_factory, name):
    out = tmp_path_factory.mktemp("asm") / (name + ".s")
    flags = [f for f in build.FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [build.hipcc(), *flags, "--cuda-device-only", "-S", os.path.join(build.CSRC, name),
           "-o", str(out), "-Rpass-analysis=kernel-resource-usage"]
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


@pytest.fixture(scope="module")
def compiled(tmp_path_factory):
    return _compile(tmp_path_factory, "mla_decode.hip")


@pytest.fixture(scope="module")
def compiled_groups(tmp_path_factory):
    return _compile(tmp_path_factory, "mla_decode_groups.hip")


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


def test_group_decode_kernel_scratch_is_small(compiled_groups):
    _, usage = compiled_groups
    assert _scratch(usage, "mla_decode_groups_fp8_kernel") <= 368


def test_group_tile_loop_touches_no_scratch(compiled_groups):
    """Every basic block holding P.V steps (the builtin MFMAs of the tile loop,
    16 or more per block) is free of scratch loads and stores."""
    asm, _ = compiled_groups
    blocks, cur = [], []
    for line in asm.splitlines():
        t = line.strip()
        if re.match(r"^\.LBB\d+_\d+:", t) or t.startswith(".Lfunc_end"):
            blocks.append(cur)
            cur = []
        elif t and not t.startswith((";", ".")):
            cur.append(t)
    blocks.append(cur)
    loops = [b for b in blocks if sum(1 for t in b if t.startswith("v_mfma")) >= 16]
    assert len(loops) >= 3  # one per kernel build at least
    for b in loops:
        bad = [t for t in b if t.startswith("scratch_")]
        assert not bad, bad[:4]


def test_group_kernel_m0_written_only_for_its_dma(compiled_groups):
    asm, _ = compiled_groups
    lines = [l.strip() for l in asm.splitlines()]
    code = [l for l in lines if l and not l.startswith((";", "."))]
    writes = [i for i, l in enumerate(code) if re.match(r"s_\w+\s+m0\b", l)]
    dmas = [i for i, l in enumerate(code) if l.startswith("global_load_lds_dwordx4")]
    assert dmas and len(writes) == len(dmas)
    assert all(code[i + 1].startswith("global_load_lds_dwordx4") for i in writes)
    # nothing else names m0 (reads included)
    others = [l for i, l in enumerate(code) if re.search(r"\bm0\b", l) and i not in writes]
    assert not others, others[:5]


def _regs(tok):
    m = re.match(r"([va])\[(\d+):(\d+)\]", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([va])(\d+)$", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


def mixed_mfma_chains(asm):
    """(line, mfma, previous writer) wherever an MFMA's accumulator registers
    were last written by an MFMA of another kind (straight-line order within a
    function; any other write in between ends the chain)."""
    last, bad = {}, []
    for ln, line in enumerate(asm.splitlines(), 1):
        t = line.strip()
        if "-- Begin function" in t:
            last = {}
        if not t or t.startswith((";", ".")) or t.endswith(":"):
            continue
        parts = re.split(r"[\s,]+", t)
        op = parts[0]
        if op.startswith("v_mfma") and len(parts) > 4:
            prev = {last.get(r) for r in _regs(parts[4])}
            if any(p and p.startswith("v_mfma") and p != op for p in prev):
                bad.append((ln, op, sorted(p for p in prev if p)))
        if len(parts) > 1 and op.startswith(("v_", "ds_read", "global_load", "buffer_load",
                                             "scratch_load", "flat_load")):
            for r in _regs(parts[1]):
                last[r] = op
    return bad


@pytest.mark.parametrize("which", ["compiled", "compiled_groups"])
def test_mfma_accumulator_chains_do_not_mix_kinds(which, request):
    asm, _ = request.getfixturevalue(which)
    assert "v_mfma" in asm
    bad = mixed_mfma_chains(asm)
    assert not bad, bad[:5]


def test_mixed_chain_detector_flags_a_mixed_chain():
    asm = "\n".join([
        "v_mfma_scale_f32_16x16x128_f8f6f4 v[0:3], v[4:11], v[12:19], 0, v1, v1",
        "v_mfma_f32_16x16x32_fp8_fp8 v[0:3], v[20:21], v[22:23], v[0:3]",
        "v_mov_b32 v0, 0",
        "v_mfma_f32_16x16x32_fp8_fp8 v[30:33], v[20:21], v[22:23], v[30:33]",
    ])
    assert [b[0] for b in mixed_mfma_chains(asm)] == [2]


@pytest.mark.parametrize("which", ["compiled", "compiled_groups"])
def test_no_packed_fp32_valu(which, request):
    asm, _ = request.getfixturevalue(which)
    assert not re.search(r"\bv_pk_(add|mul|fma)_f32\b", asm)


def _spill_before_exec_restore(asm):
    """(line, text) of scratch stores directly followed by an exec restore."""
    hits, prev = [], None
    for n, line in enumerate(asm.splitlines()):
        t = line.strip()
        if prev is not None and t.startswith("s_or_b64 exec, exec"):
            hits.append(prev)
        prev = (n, t) if t.startswith("scratch_store") else None
    return hits


def test_no_spill_store_under_a_narrowed_exec_mask(compiled, compiled_groups):
    for asm, _ in (compiled, compiled_groups):
        assert _spill_before_exec_restore(asm) == []


def test_spill_scanner_flags_the_pattern():
    asm = "\n".join(["  v_add_u32_e32 v10, s4, v3", "  s_and_saveexec_b64 s[12:13], s[16:17]",
                      ".LBB0_1:", "  scratch_store_dword off, v10, off", "  s_or_b64 exec, exec, s[12:13]"])
    assert len(_spill_before_exec_restore(asm)) == 1
    assert _spill_before_exec_restore(asm.replace("scratch_store_dword", "v_mov_b32")) == []
