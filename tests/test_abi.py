"""The C-ABI library loads, exports every symbol include/mla.h declares, and
rejects bad arguments on the host before touching HIP (no GPU needed)."""

import ctypes as C
import os
import re

import pytest

from mla_latent_attention_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(mla_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("mla_decode", "mla_merge_partials", "mla_decode_workspace_bytes",
                     "mla_status_string"):
        assert required in names


@pytest.mark.parametrize("which", ["release", "debug"])
def test_library_exports_every_declared_symbol(which):
    L = _lib.lib() if which == "release" else _lib.debug_lib()
    for name in declared_functions():
        assert hasattr(L, name), f"{name} declared in mla.h but not exported"
        assert name in _lib.SIGNATURES, f"binding has no signature for {name}"


def test_status_strings():
    L = _lib.lib()
    for code, name in _lib.STATUS.items():
        assert L.mla_status_string(code).decode().startswith(name)
    assert L.mla_status_string(99).decode() == "MLA_ERR_UNKNOWN"


def test_check_bits_match_the_header():
    text = open(HEADER).read()
    bits = {int(v): k for k, v in re.findall(r"#define (MLA_CHECK_\w+) (\d+)", text)}
    assert bits == _lib.CHECK_BITS
    assert re.search(r"MLA_ERR_BAD_INPUT = 8", text)


def test_workspace_size_is_pure_and_bounded():
    L = _lib.lib()
    ws = L.mla_decode_workspace_bytes_ex(16, 16, 16, 1, 256)
    assert ws >= 2 * 256 * 16 * (512 + 1) * 4 + 16 * 16  # partials + one descriptor per unit
    assert ws % 256 == 0
    assert L.mla_decode_workspace_bytes_ex(0, 16, 16, 1, 256) == 0
    assert L.mla_decode_workspace_bytes_ex(16, 16, 16, 0, 256) == 0
    assert L.mla_decode_workspace_bytes_ex(16, 16, 16, 1, 0) == 0
    assert L.mla_decode_workspace_bytes_ex(2, 9, 16, 4, 8) == 0  # more tokens than 2 * 4


FAKE = C.c_void_p(0x1000)  # never dereferenced: validation fails first


def _decode(**over):
    args = dict(
        q=FAKE, q_dtype=0, kv=FAKE, kv_dtype=0, pool=256, o=FAKE, qo=FAKE, kvp=FAKE, idx=FAKE,
        idx_len=164, lpl=None, batch=2, T=2, H=16, qmax=1, sm=0.072, qs=None, ks=None, rl=0,
        lse=None, ws=FAKE, ws_len=1 << 30, nw=8, stream=None,
    )
    args.update(over)
    return _lib.lib().mla_decode_ex(*args.values())


@pytest.mark.parametrize(
    "over,status",
    [
        (dict(q=None), 1),
        (dict(kv=None), 1),
        (dict(o=None), 1),
        (dict(idx=None), 1),
        (dict(rl=1, lse=None), 1),
        (dict(q_dtype=1, kv_dtype=0), 3),
        (dict(q_dtype=2, kv_dtype=2), 3),
        (dict(H=12), 4),
        (dict(H=0), 4),
        (dict(batch=0), 2),
        (dict(qmax=0), 2),
        (dict(qmax=65), 2),
        (dict(T=3, qmax=1), 2),
        (dict(pool=0), 2),
        (dict(nw=-1), 2),
        (dict(ws=None), 5),
        (dict(ws_len=1024), 5),
    ],
)
def test_decode_rejects_bad_arguments_before_any_launch(over, status):
    assert _decode(**over) == status


@pytest.mark.parametrize(
    "args,status",
    [
        ((None, 2, FAKE, 8, 32, 96, FAKE, FAKE, None), 1),
        ((FAKE, 0, FAKE, 8, 32, 96, FAKE, FAKE, None), 3),
        ((FAKE, 2, FAKE, 0, 32, 96, FAKE, FAKE, None), 2),
        ((FAKE, 2, None, 8, 32, 96, FAKE, FAKE, None), 1),
    ],
)
def test_merge_rejects_bad_arguments(args, status):
    assert _lib.lib().mla_merge_partials(*args) == status


def _decode_dcp(**over):
    args = dict(
        q=FAKE, q_dtype=0, kv=FAKE, kv_dtype=0, pool=256, o=FAKE, qo=FAKE, kvp=FAKE, idx=FAKE,
        idx_len=164, lpl=None, batch=2, T=2, H=16, qmax=1, sm=0.072, qs=None, ks=None, rl=0,
        lse=None, gkv=FAKE, cps=8, cpr=3, odt=1, ws=FAKE, ws_len=1 << 30, stream=None,
    )
    args.update(over)
    return _lib.lib().mla_decode_dcp(*args.values())


@pytest.mark.parametrize(
    "over,status",
    [
        (dict(gkv=None), 1),
        (dict(cps=0), 2),
        (dict(cps=1025), 2),
        (dict(cpr=8), 2),
        (dict(cpr=-1), 2),
        (dict(q=None), 1),
        (dict(H=24), 4),
        (dict(qmax=65), 2),
        (dict(ws=None), 5),
        (dict(odt=0), 3),
        (dict(odt=7), 3),
    ],
)
def test_decode_dcp_rejects_bad_arguments_before_any_launch(over, status):
    assert _decode_dcp(**over) == status


def _decode_paged(**over):
    args = dict(
        q=FAKE, q_dtype=0, kv=FAKE, kv_dtype=0, pool=1024, o=FAKE, qo=FAKE, kvp=FAKE, idx=FAKE,
        idx_len=8, lpl=FAKE, page=128, batch=2, T=2, H=16, qmax=1, sm=0.072, qs=None, ks=None,
        rl=0, lse=None, ws=FAKE, ws_len=1 << 30, stream=None,
    )
    args.update(over)
    return _lib.lib().mla_decode_paged(*args.values())


@pytest.mark.parametrize(
    "over,status",
    [
        (dict(page=0), 2),
        (dict(page=3), 2),
        (dict(page=8192), 2),
        (dict(lpl=None), 1),
        (dict(pool=1000), 2),
        (dict(pool=1 << 31), 2),
        (dict(q=None), 1),
        (dict(H=24), 4),
        (dict(ws=None), 5),
    ],
)
def test_decode_paged_rejects_bad_arguments_before_any_launch(over, status):
    assert _decode_paged(**over) == status


def _rope(**over):
    args = dict(ql=FAKE, qp=FAKE, kl=FAKE, kp=FAKE, pos=FAKE, cs=FAKE, max_pos=100, style=0,
                q_out=FAKE, T=16, H=12, Hp=16, pool=FAKE, n=1024, slots=FAKE, qs=None, ks=None,
                stream=None)
    args.update(over)
    return _lib.lib().mla_rope_quant_cache(*args.values())


@pytest.mark.parametrize(
    "over,status",
    [(dict(ql=None), 1), (dict(slots=None), 1), (dict(pool=None), 1), (dict(style=2), 2),
     (dict(Hp=8), 2), (dict(T=0), 2), (dict(max_pos=0), 2), (dict(n=0), 2)],
)
def test_rope_quant_cache_rejects_bad_arguments(over, status):
    assert _rope(**over) == status


@pytest.mark.parametrize(
    "args,status",
    [((None, FAKE, FAKE, 16, 12, 16, None), 1), ((FAKE, FAKE, None, 16, 12, 16, None), 1),
     ((FAKE, FAKE, FAKE, 16, 12, 8, None), 2), ((FAKE, FAKE, FAKE, 0, 12, 16, None), 2),
     ((FAKE, FAKE, FAKE, 16, 70000, 70000, None), 2)],
)
def test_latent_to_v_rejects_bad_arguments(args, status):
    assert _lib.lib().mla_latent_to_v(*args) == status


def _step(**over):
    args = dict(ql=FAKE, qp=FAKE, kl=FAKE, kp=FAKE, pos=FAKE, cs=FAKE, max_pos=100, style=0,
                slots=FAKE, pool=FAKE, n=1 << 20, qo=FAKE, kvp=FAKE, kvi=FAKE, kvi_len=1000,
                B=16, T=16, H=12, Hp=16, mq=1, sm=0.07, qs=None, ks=None, w=FAKE, o=FAKE,
                out=FAKE, ret_lse=0, lse=None, ws=FAKE, ws_len=1 << 30, stream=None)
    args.update(over)
    return _lib.lib().mla_decode_step(*args.values())


@pytest.mark.parametrize(
    "over,status",
    [(dict(ql=None), 1), (dict(slots=None), 1), (dict(w=None), 1), (dict(out=None), 1),
     (dict(o=None), 1), (dict(ret_lse=1), 1), (dict(Hp=24), 4), (dict(Hp=0), 4),
     (dict(H=20), 2), (dict(H=0), 2), (dict(style=2), 2), (dict(max_pos=0), 2), (dict(T=0), 2),
     (dict(mq=65), 2), (dict(n=0), 2), (dict(kvi_len=-1), 2)],
)
def test_decode_step_rejects_bad_arguments_before_any_launch(over, status):
    assert _step(**over) == status


def test_decode_step_workspace_size_rejects_bad_shapes():
    L = _lib.lib()
    assert L.mla_decode_step_workspace_bytes(16, 16, 24, 1) == 0
    assert L.mla_decode_step_workspace_bytes(16, 0, 16, 1) == 0


def _check(**over):
    args = dict(qo=FAKE, kvp=FAKE, kvi=FAKE, kvi_len=1000, lpl=None, page=1, pool=1 << 20, B=16,
                T=16, mq=1, g=None, cp=1, rank=0, status=FAKE, stream=None)
    args.update(over)
    return _lib.lib().mla_check_inputs(*args.values())


@pytest.mark.parametrize(
    "over,status",
    [(dict(qo=None), 1), (dict(kvp=None), 1), (dict(status=None), 1), (dict(kvi=None), 1),
     (dict(page=0), 2), (dict(page=3), 2), (dict(page=8192), 2), (dict(B=0), 2),
     (dict(T=-1), 2), (dict(mq=0), 2), (dict(kvi_len=-1), 2), (dict(pool=0), 2),
     (dict(g=FAKE, cp=0), 2), (dict(g=FAKE, cp=4, rank=4), 2), (dict(g=FAKE, cp=4, rank=-1), 2)],
)
def test_check_inputs_rejects_bad_arguments_before_any_launch(over, status):
    assert _check(**over) == status


def test_check_inputs_allows_an_empty_index_list_without_a_pointer():
    # kv_indices may be NULL when the list is empty; the call then gets as far
    # as the launch, which needs a GPU, so only the argument checks are run
    # here: a NULL status still fails first.
    assert _check(kvi=None, kvi_len=0, status=None) == 1


def test_header_and_plain_c_caller_compile_as_c11():
    """include/mla.h is a C header: the plain-C caller the GPU tests run
    compiles with gcc in C11 mode, warnings as errors."""
    import shutil
    import subprocess

    from mla_latent_attention_amd import build

    gcc = shutil.which("gcc")
    if gcc is None or not os.path.exists(os.path.join(build.ROCM, "include", "hip")):
        pytest.skip("gcc or the ROCm headers are not installed")
    res = subprocess.run([gcc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-fsyntax-only",
                          "-D__HIP_PLATFORM_AMD__", f"-I{build.ROCM}/include",
                          f"-I{os.path.join(build.ROOT, 'include')}", build.C_DRIVER_SRC],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
