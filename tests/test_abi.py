"""The C ABI on a host without a GPU: the library loads, exports exactly what
include/fa.h declares, and rejects invalid arguments before any HIP call."""

import ctypes
import os
import re
import subprocess

import pytest

from exact_tiled_attention_prefill_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

needs_lib = pytest.mark.skipif(not os.path.exists(binding.library_path()),
                               reason="libfa.so not built (run __graft_entry__.build())")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("fa_prefill", "fa_decode", "fa_prefill_f32", "fa_decode_f32", "fa_decode_ws",
              "fa_decode_f32_ws", "fa_decode_workspace_bytes", "fa_decode_paged",
              "fa_decode_paged_workspace_bytes", "fa_prefill_varlen", "fa_strerror", "fa_version"):
        assert n in names
    assert set(names) == set(binding.SIGNATURES)


@needs_lib
def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(binding.library_path())
    for n in declared_functions():
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", binding.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (fa_[a-z0-9_]+)$", out, flags=re.M))
    assert exported == set(declared_functions())


@needs_lib
def test_strerror_and_version():
    lib = binding.load_library()
    for code in range(6):
        assert lib.fa_strerror(code).decode().startswith("FA_")
    assert b"unknown" in lib.fa_strerror(99)
    assert lib.fa_version() >= 100


P = ctypes.c_void_p(0x10000)  # never dereferenced: every case fails validation first
P_MIS = ctypes.c_void_p(0x10002)


def prefill_call(fn, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=None, B=1, Hq=4, Hkv=2, N=16, d=128, causal=1, scale=0.1)
    a.update(kw)
    return fn(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["N"], a["d"],
              a["causal"], ctypes.c_float(a["scale"]), None)


@needs_lib
@pytest.mark.parametrize("name", ["fa_prefill", "fa_prefill_f32"])
@pytest.mark.parametrize("kw,code", [
    (dict(q=None), binding.FA_ERR_INVALID_ARG),
    (dict(k=None), binding.FA_ERR_INVALID_ARG),
    (dict(v=None), binding.FA_ERR_INVALID_ARG),
    (dict(o=None), binding.FA_ERR_INVALID_ARG),
    (dict(B=0), binding.FA_ERR_INVALID_ARG),
    (dict(N=0), binding.FA_ERR_INVALID_ARG),
    (dict(N=-5), binding.FA_ERR_INVALID_ARG),
    (dict(Hq=0), binding.FA_ERR_INVALID_ARG),
    (dict(Hkv=0), binding.FA_ERR_INVALID_ARG),
    (dict(Hq=6, Hkv=4), binding.FA_ERR_INVALID_ARG),
    (dict(causal=2), binding.FA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), binding.FA_ERR_INVALID_ARG),
    (dict(scale=3e38), binding.FA_ERR_INVALID_ARG),    # |scale| log2(e) overflows fp32
    (dict(scale=-3e38), binding.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), binding.FA_ERR_INVALID_ARG),
    (dict(q=P_MIS), binding.FA_ERR_INVALID_ARG),
    (dict(o=P_MIS), binding.FA_ERR_INVALID_ARG),
    (dict(lse=ctypes.c_void_p(0x10001)), binding.FA_ERR_INVALID_ARG),
    (dict(d=96), binding.FA_ERR_UNSUPPORTED),
    (dict(d=256), binding.FA_ERR_UNSUPPORTED),
    (dict(d=32), binding.FA_ERR_UNSUPPORTED),
])
def test_prefill_rejects_invalid_arguments(name, kw, code):
    fn = getattr(binding.load_library(), name)
    assert prefill_call(fn, **kw) == code


@needs_lib
def test_prefill_grid_limit_follows_each_kernels_tile():
    # every call here fails validation (no device call): 2^20 heads x
    # ceil(2^15 / 16) = 2^31 workgroups of the fp32 kernel's 16-row tiles;
    # 2^24 heads x ceil(2^14 / 128) = 2^31 of the bf16 kernels' 128-row tiles
    lib = binding.load_library()
    assert prefill_call(lib.fa_prefill_f32, Hq=1 << 20, Hkv=1, N=1 << 15) == binding.FA_ERR_INVALID_ARG
    assert prefill_call(lib.fa_prefill, Hq=1 << 24, Hkv=1, N=1 << 14) == binding.FA_ERR_INVALID_ARG


def decode_call(fn, ws=False, **kw):
    a = dict(q=P, k=P, v=P, sl=P, o=P, B=2, Hq=8, Hkv=2, maxlen=1024, d=128, scale=0.1,
             w=P, wb=1 << 30)
    a.update(kw)
    args = [a["q"], a["k"], a["v"], a["sl"], a["o"], a["B"], a["Hq"], a["Hkv"], a["maxlen"], a["d"],
            ctypes.c_float(a["scale"])]
    if ws:
        args += [a["w"], a["wb"]]
    return fn(*args, None)


@needs_lib
@pytest.mark.parametrize("name", ["fa_decode", "fa_decode_f32", "fa_decode_ws", "fa_decode_f32_ws"])
@pytest.mark.parametrize("kw,code", [
    (dict(q=None), binding.FA_ERR_INVALID_ARG),
    (dict(k=None), binding.FA_ERR_INVALID_ARG),
    (dict(v=None), binding.FA_ERR_INVALID_ARG),
    (dict(sl=None), binding.FA_ERR_INVALID_ARG),
    (dict(o=None), binding.FA_ERR_INVALID_ARG),
    (dict(B=0), binding.FA_ERR_INVALID_ARG),
    (dict(maxlen=0), binding.FA_ERR_INVALID_ARG),
    (dict(Hq=8, Hkv=3), binding.FA_ERR_INVALID_ARG),
    (dict(scale=float("-inf")), binding.FA_ERR_INVALID_ARG),
    (dict(scale=2.5e38), binding.FA_ERR_INVALID_ARG),  # |scale| log2(e) overflows fp32
    (dict(k=P_MIS), binding.FA_ERR_INVALID_ARG),
    (dict(sl=ctypes.c_void_p(0x10001)), binding.FA_ERR_INVALID_ARG),
    (dict(B=70000), binding.FA_ERR_INVALID_ARG),
    (dict(d=80), binding.FA_ERR_UNSUPPORTED),
])
def test_decode_rejects_invalid_arguments(name, kw, code):
    fn = getattr(binding.load_library(), name)
    assert decode_call(fn, ws=name.endswith("_ws"), **kw) == code


@needs_lib
@pytest.mark.parametrize("name", ["fa_decode_ws", "fa_decode_f32_ws"])
def test_decode_ws_rejects_small_or_missing_workspace(name):
    lib = binding.load_library()
    fn = getattr(lib, name)
    need = lib.fa_decode_workspace_bytes(2, 8, 2, 1024, 128)
    assert need > 0
    assert decode_call(fn, ws=True, w=None) == binding.FA_ERR_INVALID_ARG
    assert decode_call(fn, ws=True, wb=need - 1) == binding.FA_ERR_INVALID_ARG
    assert decode_call(fn, ws=True, w=ctypes.c_void_p(0x10010)) == binding.FA_ERR_INVALID_ARG


@needs_lib
def test_workspace_bytes():
    lib = binding.load_library()
    # the fp32 path's partials, the larger of the two paths' here: [B,Hq,nsplit,d]
    # fp32 outputs and [B,Hq,nsplit] fp64 log-sum-exps, each padded to 256 bytes
    nsplit = (32768 + 511) // 512
    po = 64 * 32 * nsplit * 128 * 4
    pl = 64 * 32 * nsplit * 8
    rnd = lambda x: (x + 255) // 256 * 256
    assert lib.fa_decode_workspace_bytes(64, 32, 8, 32768, 128) == rnd(po) + rnd(pl)
    assert lib.fa_decode_workspace_bytes(0, 32, 8, 32768, 128) == 0
    assert lib.fa_decode_workspace_bytes(64, 32, 5, 32768, 128) == 0
    assert lib.fa_decode_workspace_bytes(64, 32, 8, 32768, 96) == 0


def varlen_call(fn, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=None, cq=P, ck=P, B=2, Hq=8, Hkv=2, tq=100, tk=300, mq=60, d=128,
             causal=1, w=-1, scale=0.1)
    a.update(kw)
    return fn(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cq"], a["ck"], a["B"], a["Hq"], a["Hkv"], a["tq"],
              a["tk"], a["mq"], a["d"], a["causal"], a["w"], ctypes.c_float(a["scale"]), None)


@needs_lib
@pytest.mark.parametrize("kw,code", [
    (dict(q=None), binding.FA_ERR_INVALID_ARG),
    (dict(k=None), binding.FA_ERR_INVALID_ARG),
    (dict(o=None), binding.FA_ERR_INVALID_ARG),
    (dict(cq=None), binding.FA_ERR_INVALID_ARG),
    (dict(ck=None), binding.FA_ERR_INVALID_ARG),
    (dict(cq=ctypes.c_void_p(0x10002)), binding.FA_ERR_INVALID_ARG),
    (dict(B=0), binding.FA_ERR_INVALID_ARG),
    (dict(tq=0), binding.FA_ERR_INVALID_ARG),
    (dict(tk=0), binding.FA_ERR_INVALID_ARG),
    (dict(mq=0), binding.FA_ERR_INVALID_ARG),
    (dict(mq=101), binding.FA_ERR_INVALID_ARG),
    (dict(w=-2), binding.FA_ERR_INVALID_ARG),
    (dict(causal=3), binding.FA_ERR_INVALID_ARG),
    (dict(Hq=8, Hkv=3), binding.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), binding.FA_ERR_INVALID_ARG),
    (dict(v=P_MIS), binding.FA_ERR_INVALID_ARG),
    (dict(lse=ctypes.c_void_p(0x10001)), binding.FA_ERR_INVALID_ARG),
    (dict(d=48), binding.FA_ERR_UNSUPPORTED),
])
def test_prefill_varlen_rejects_invalid_arguments(kw, code):
    assert varlen_call(binding.load_library().fa_prefill_varlen, **kw) == code


def paged_call(fn, **kw):
    a = dict(q=P, kp=P, vp=P, bt=P, sl=P, o=P, B=2, Hq=8, Hkv=2, num_pages=64, page=32, max_pages=32, d=128,
             scale=0.1, w=None, wb=0)
    a.update(kw)
    return fn(a["q"], a["kp"], a["vp"], a["bt"], a["sl"], a["o"], a["B"], a["Hq"], a["Hkv"], a["num_pages"],
              a["page"], a["max_pages"], a["d"], ctypes.c_float(a["scale"]), a["w"], a["wb"], None)


@needs_lib
@pytest.mark.parametrize("kw,code", [
    (dict(q=None), binding.FA_ERR_INVALID_ARG),
    (dict(kp=None), binding.FA_ERR_INVALID_ARG),
    (dict(vp=None), binding.FA_ERR_INVALID_ARG),
    (dict(bt=None), binding.FA_ERR_INVALID_ARG),
    (dict(bt=ctypes.c_void_p(0x10002)), binding.FA_ERR_INVALID_ARG),
    (dict(sl=None), binding.FA_ERR_INVALID_ARG),
    (dict(o=None), binding.FA_ERR_INVALID_ARG),
    (dict(page=24), binding.FA_ERR_INVALID_ARG),
    (dict(page=8), binding.FA_ERR_INVALID_ARG),
    (dict(page=0), binding.FA_ERR_INVALID_ARG),
    (dict(page=1 << 21), binding.FA_ERR_INVALID_ARG),
    (dict(num_pages=0), binding.FA_ERR_INVALID_ARG),
    (dict(max_pages=0), binding.FA_ERR_INVALID_ARG),
    (dict(max_pages=1 << 27, page=64), binding.FA_ERR_INVALID_ARG),
    (dict(Hq=8, Hkv=3), binding.FA_ERR_INVALID_ARG),
    (dict(kp=P_MIS), binding.FA_ERR_INVALID_ARG),
    (dict(w=P, wb=16), binding.FA_ERR_INVALID_ARG),
    (dict(d=96), binding.FA_ERR_UNSUPPORTED),
])
def test_decode_paged_rejects_invalid_arguments(kw, code):
    assert paged_call(binding.load_library().fa_decode_paged, **kw) == code


@needs_lib
def test_paged_workspace_bytes():
    lib = binding.load_library()
    for page, pages in ((16, 2048), (64, 512), (1024, 32)):
        assert lib.fa_decode_paged_workspace_bytes(64, 32, 8, page, pages, 128) == \
            lib.fa_decode_workspace_bytes(64, 32, 8, page * pages, 128)
    assert lib.fa_decode_paged_workspace_bytes(64, 32, 8, 24, 100, 128) == 0
    assert lib.fa_decode_paged_workspace_bytes(64, 32, 8, 64, 0, 128) == 0
    assert lib.fa_decode_paged_workspace_bytes(64, 32, 5, 64, 10, 128) == 0


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setenv("FA_LIBRARY", str(tmp_path / "missing.so"))
    monkeypatch.setattr(binding, "_lib", None)
    with pytest.raises(binding.FaError):
        binding.load_library()


@needs_lib
@pytest.mark.parametrize("kw,code", [
    (dict(q=None), binding.FA_ERR_INVALID_ARG),
    (dict(sl=None), binding.FA_ERR_INVALID_ARG),
    (dict(Hq=8, Hkv=3), binding.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), binding.FA_ERR_INVALID_ARG),
    (dict(d=80), binding.FA_ERR_UNSUPPORTED),
    (dict(B=4096, Hq=64, Hkv=8, maxlen=65536), binding.FA_ERR_TOO_LARGE),
    (dict(B=60000, Hq=32, Hkv=8, maxlen=1 << 20), binding.FA_ERR_TOO_LARGE),
])
def test_decode_noalloc_rejects_before_any_hip_call(kw, code):
    """fa_decode_noalloc: invalid arguments, and sizes whose partials exceed
    its fixed array, are refused on the host (no device here)."""
    assert decode_call(binding.load_library().fa_decode_noalloc, **kw) == code
