"""The C ABI on the host, without a GPU: the library loads, exports every
function include/moe_decode.h declares, the ctypes mirror of the config struct
matches the C layout, and argument errors are reported before any device work.
"""

import ctypes
import os
import subprocess
import tempfile

import pytest

import fp8_block_scaled_moe_amd as pkg
from fp8_block_scaled_moe_amd import _capi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_capi.LIB_PATH):
        from fp8_block_scaled_moe_amd import build
        build.build()
    return pkg.lib()


def test_exports_every_declared_function(L):
    names = pkg.header_functions()
    assert {"moe_decode_create", "moe_decode_run", "moe_decode_destroy"} <= set(names)
    for n in names:
        assert hasattr(L, n), f"{n} declared in include/moe_decode.h but not exported"


def test_config_layout_matches_c(tmp_path):
    src = tmp_path / "layout.c"
    fields = [f for f, _ in _capi.MoeDecodeConfig._fields_]
    body = "\n".join(f'  printf("%zu\\n", offsetof(moe_decode_config, {f}));' for f in fields)
    src.write_text(
        "#include <stdio.h>\n#include <stddef.h>\n#include \"moe_decode.h\"\n"
        f"int main(void) {{\n  printf(\"%zu\\n\", sizeof(moe_decode_config));\n{body}\n  return 0;\n}}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                    str(src), "-o", str(exe)], check=True)
    out = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True,
                                          check=True).stdout.split()]
    assert out[0] == ctypes.sizeof(_capi.MoeDecodeConfig)
    for f, off in zip(fields, out[1:]):
        assert getattr(_capi.MoeDecodeConfig, f).offset == off, f


def _cfg(**kw):
    c = _capi.MoeDecodeConfig()
    c.hidden, c.inter, c.experts, c.top_k, c.max_tokens = 256, 128, 8, 2, 4
    c.limit, c.routed_scale = 7.0, 2.5
    c.w13 = c.w13_scale = c.w2 = c.w2_scale = 4096  # never dereferenced on the error paths
    for k, v in kw.items():
        setattr(c, k, v)
    return c


_SHARED = dict(sw13=8192, sw13_scale=8192, sw2=8192, sw2_scale=8192, shared_limit=7.0)


@pytest.mark.parametrize("kw,code", [
    (dict(hidden=200), _capi.ERR_UNSUPPORTED),
    (dict(inter=100), _capi.ERR_UNSUPPORTED),
    (dict(top_k=9), _capi.ERR_UNSUPPORTED),
    (dict(top_k=0), _capi.ERR_INVALID_ARG),
    (dict(experts=2000, top_k=4), _capi.ERR_UNSUPPORTED),
    (dict(experts=64, top_k=33), _capi.ERR_UNSUPPORTED),
    (dict(max_tokens=0), _capi.ERR_INVALID_ARG),
    (dict(max_tokens=257), _capi.ERR_UNSUPPORTED),
    # each limit alone is allowed; together the routing kernel's LDS (token
    # masks of 1024 experts x 4 words, 8192 routes) exceeds 64 KiB
    (dict(max_tokens=256, experts=1024, top_k=32), _capi.ERR_UNSUPPORTED),
    (dict(logits_dtype=7), _capi.ERR_UNSUPPORTED),
    (dict(limit=0.0), _capi.ERR_INVALID_ARG),
    (dict(w13=None), _capi.ERR_INVALID_ARG),
    (dict(w2_scale=4100), _capi.ERR_INVALID_ARG),   # misaligned
    (dict(gemm_path=5), _capi.ERR_UNSUPPORTED),
    (dict(launch_mode=5), _capi.ERR_UNSUPPORTED),
    (dict(launch_mode=-1), _capi.ERR_UNSUPPORTED),
    (dict(splits1=-1), _capi.ERR_INVALID_ARG),
    # shared expert
    (dict(shared_inter=-128), _capi.ERR_INVALID_ARG),
    (dict(shared_inter=128), _capi.ERR_INVALID_ARG),                  # no shared weights
    (dict(shared_inter=100, **_SHARED), _capi.ERR_UNSUPPORTED),
    (dict(shared_inter=128, shared_scale_format=2, **_SHARED), _capi.ERR_UNSUPPORTED),
    (dict(dict(_SHARED, shared_limit=0.0), shared_inter=128), _capi.ERR_INVALID_ARG),
    (dict(dict(_SHARED, sw2=4104), shared_inter=128), _capi.ERR_INVALID_ARG),  # misaligned
    # weight format and local experts
    (dict(weight_format=5), _capi.ERR_UNSUPPORTED),
    (dict(local_begin=4, local_experts=5), _capi.ERR_INVALID_ARG),   # 4 + 5 > 8 experts
    (dict(local_begin=-1), _capi.ERR_INVALID_ARG),
    (dict(local_experts=-2), _capi.ERR_INVALID_ARG),
    (dict(weight_format=1, hidden=384), _capi.ERR_UNSUPPORTED),      # FP4 needs multiples of 256
    (dict(weight_format=1, inter=128), _capi.ERR_UNSUPPORTED),
    (dict(weight_format=1, inter=256, ue8m0_act=1), _capi.ERR_UNSUPPORTED),
    (dict(weight_format=1, inter=256, gemm_path=3), _capi.ERR_UNSUPPORTED),
    (dict(dict(_SHARED, shared_inter=128), weight_format=1, inter=256), _capi.ERR_UNSUPPORTED),
])
def test_create_rejects_bad_config(L, kw, code):
    h = ctypes.c_void_p(1234)
    assert L.moe_decode_create(ctypes.byref(_cfg(**kw)), ctypes.byref(h)) == code
    assert h.value is None


def test_null_arguments(L):
    h = ctypes.c_void_p()
    assert L.moe_decode_create(None, ctypes.byref(h)) == _capi.ERR_INVALID_ARG
    assert L.moe_decode_create(ctypes.byref(_cfg()), None) == _capi.ERR_INVALID_ARG
    assert L.moe_decode_run(None, 1, *([None] * 9)) == _capi.ERR_INVALID_ARG
    L.moe_decode_destroy(None)
    assert L.moe_decode_plan(None, 1, None, 9) == _capi.ERR_INVALID_ARG
    assert L.moe_decode_debug_stage(None, 0, None, 0, None) == _capi.ERR_INVALID_ARG
    assert L.moe_decode_set_timing(None, 1) == _capi.ERR_INVALID_ARG
    assert L.moe_decode_debug_codec(None, None, None, 4, None) == _capi.ERR_INVALID_ARG


def test_error_strings(L):
    for code in (0, -1, -2, -3, -4, -5):
        assert pkg.error_string(code) and pkg.error_string(code) != "unknown error"
    assert pkg.error_string(-99) == "unknown error"


def test_missing_library_fails_loudly(monkeypatch):
    monkeypatch.setattr(_capi, "_lib", None)
    monkeypatch.setattr(_capi, "LIB_PATH", os.path.join(tempfile.gettempdir(), "no_such_lib.so"))
    with pytest.raises(RuntimeError, match="missing"):
        _capi.lib()


def test_boundary_header_compiles_as_c(tmp_path):
    src = tmp_path / "b.c"
    src.write_text("#include \"moe_boundary.h\"\nint main(void) { return MOE_BOUNDARY_MAX_D > 0 ? 0 : 1; }\n")
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                    str(src), "-o", str(tmp_path / "b")], check=True)


def test_boundary_argument_errors(L):
    """Argument checks of the boundary calls return before any device work."""
    fake = ctypes.c_void_p(0x1000)   # never dereferenced: every case fails validation first
    odd = ctypes.c_void_p(0x1008)
    # MXFP8: negative T, null or misaligned pointers, D not a multiple of 32 or too long
    assert L.moe_mxfp8_quantize(fake, -1, 64, fake, fake, None) == _capi.ERR_INVALID_ARG
    assert L.moe_mxfp8_quantize(None, 1, 64, fake, fake, None) == _capi.ERR_INVALID_ARG
    assert L.moe_mxfp8_quantize(odd, 1, 64, fake, fake, None) == _capi.ERR_INVALID_ARG
    assert L.moe_mxfp8_quantize(fake, 1, 48, fake, fake, None) == _capi.ERR_UNSUPPORTED
    assert L.moe_mxfp8_quantize(fake, 1, 0, fake, fake, None) == _capi.ERR_UNSUPPORTED
    assert L.moe_mxfp8_quantize(fake, 1, 16384 + 32, fake, fake, None) == _capi.ERR_UNSUPPORTED
    assert L.moe_mxfp8_quantize(fake, 0, 64, fake, fake, None) == _capi.OK   # empty call
    # reduce + RMSNorm
    args = lambda T, N, D, eps=1e-5, lat=fake: (fake, T, N, D, fake, eps, lat, fake, None)  # noqa: E731
    assert L.moe_reduce_rmsnorm(*args(-1, 1, 64)) == _capi.ERR_INVALID_ARG
    assert L.moe_reduce_rmsnorm(*args(1, 1, 64, eps=-1.0)) == _capi.ERR_INVALID_ARG
    assert L.moe_reduce_rmsnorm(*args(1, 1, 64, eps=float("nan"))) == _capi.ERR_INVALID_ARG
    assert L.moe_reduce_rmsnorm(*args(1, 1, 64, lat=odd)) == _capi.ERR_INVALID_ARG
    assert L.moe_reduce_rmsnorm(*args(1, 0, 64)) == _capi.ERR_UNSUPPORTED
    assert L.moe_reduce_rmsnorm(*args(1, 65, 64)) == _capi.ERR_UNSUPPORTED
    assert L.moe_reduce_rmsnorm(*args(1, 1, 12)) == _capi.ERR_UNSUPPORTED
    assert L.moe_reduce_rmsnorm(*args(0, 1, 64)) == _capi.OK
