"""The C-ABI library loads, exports every declared entry point, and rejects
bad arguments on the host (no device is touched, so this runs without a GPU)."""
import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

from exact_io_aware_56_amd import _lib  # noqa: E402

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="libfa.so not built")


def declared_functions():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fa_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(_lib.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_status_strings():
    lib = _lib.load()
    assert lib.fa_abi_version() == 8
    assert _lib.status_name(0) == "FA_OK"
    assert _lib.status_name(-1) == "FA_ERR_INVALID_ARG"
    assert _lib.status_name(-2) == "FA_ERR_UNSUPPORTED"
    assert _lib.status_name(-3) == "FA_ERR_HIP"
    assert _lib.status_name(12345) == "FA_UNKNOWN_STATUS"


# Fake, aligned, never-dereferenced addresses: validation must reject before use.
P = 1 << 20


def call(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=1, N=16, d=64, scale=0.125, causal=0,
             key_len=None, dtype=2, stream=None)
    a.update(kw)
    return _lib.fa_fwd_raw(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"],
                           a["d"], a["scale"], a["causal"], a["key_len"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(k=None), -1), (dict(v=None), -1), (dict(o=None), -1),
    (dict(lse=None), -1), (dict(B=0), -1), (dict(H=-1), -1), (dict(N=0), -1), (dict(d=0), -1),
    (dict(dtype=4), -1), (dict(dtype=-1), -1), (dict(scale=0.0), -1), (dict(scale=-1.0), -1),
    (dict(scale=math.inf), -1), (dict(scale=math.nan), -1), (dict(q=P + 8), -1),
    (dict(o=P + 4), -1), (dict(lse=P + 2), -1), (dict(key_len=P + 1), -1),
    (dict(B=1 << 30, H=1 << 30, N=1 << 30), -1), (dict(d=96), -2), (dict(d=512), -2),
    (dict(d=32, dtype=0), -2), (dict(d=256, dtype=0), -2), (dict(d=256, dtype=3), -2),
    # head dimension 256 keeps one head under 1 GiB too: 2^21 rows x 256 x bf16
    (dict(N=1 << 21, d=256), -2),
    # one head's N x d tensor must stay under 1 GiB: 2^22 rows x 128 x bf16 is exactly 1 GiB
    (dict(N=1 << 22, d=128), -2), (dict(N=(1 << 21) + 1, d=128, dtype=0), -2),
])
def test_invalid_arguments_are_rejected_on_host(kw, status):
    assert call(**kw) == status
    assert _lib.load().fa_last_error().decode() != ""


@pytest.mark.parametrize("entry", ["fa_fwd_fp8_raw", "fa_fwd_fp8_p8_raw"])
def test_fp8_descales_are_validated(entry):
    f = getattr(_lib, entry)
    for bad in (0.0, -2.0, math.inf, math.nan):
        assert f(P, P, P, P, P, 1, 1, 16, 128, 0.1, 1, None, bad, 1.0, 1.0, None) == -1
        assert f(P, P, P, P, P, 1, 1, 16, 128, 0.1, 1, None, 1.0, 1.0, bad, None) == -1
    # scale * q_descale * k_descale must stay finite
    assert f(P, P, P, P, P, 1, 1, 16, 128, 3e38, 1, None, 1e10, 1.0, 1.0, None) == -1


@pytest.mark.parametrize("args,status", [
    (dict(d=256), -2), (dict(d=96), -2), (dict(d=32), -2), (dict(q=None), -1), (dict(N=0), -1),
    (dict(o=P + 4), -1), (dict(scale=math.nan), -1),
])
def test_fp8_p8_entry_point_rejects_bad_arguments(args, status):
    a = dict(q=P, N=16, d=128, scale=0.1, o=P)
    a.update(args)
    st = _lib.fa_fwd_fp8_p8_raw(a["q"], P, P, a["o"], P, 1, 1, a["N"], a["d"], a["scale"], 1, None,
                                1.0, 1.0, 1.0, None)
    assert st == status


def gqa_call(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=8, H_kv=2, N=16, d=64, scale=0.125, causal=0,
             key_len=None, dtype=2, qd=1.0, kd=1.0, vd=1.0, stream=None)
    a.update(kw)
    return _lib.fa_fwd_gqa_raw(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"],
                               a["H_kv"], a["N"], a["d"], a["scale"], a["causal"], a["key_len"],
                               a["dtype"], a["qd"], a["kd"], a["vd"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(H_kv=0), -1), (dict(H_kv=-2), -1), (dict(H_kv=3), -1), (dict(H_kv=16), -1),
    (dict(H=6, H_kv=4), -1), (dict(k=None), -1), (dict(v=P + 8), -1), (dict(qd=0.0), -1),
    (dict(vd=math.nan), -1), (dict(dtype=5), -1), (dict(d=512), -2), (dict(d=96, H_kv=1), -2),
    (dict(d=256, dtype=0), -2),
])
def test_grouped_entry_point_rejects_bad_arguments(kw, status):
    assert gqa_call(**kw) == status
    assert _lib.load().fa_last_error().decode() != ""


def decode_call(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=2, H=8, H_kv=2, Nq=1, Nk=4096, d=128, scale=0.1,
             causal=1, key_len=None, dtype=2, ws=P, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return _lib.fa_fwd_decode_raw(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"],
                                  a["H_kv"], a["Nq"], a["Nk"], a["d"], a["scale"], a["causal"],
                                  a["key_len"], a["dtype"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(ws=None), -1), (dict(ws=P + 8), -1), (dict(ws_bytes=1024), -1), (dict(q=None), -1),
    (dict(Nq=0), -1), (dict(Nk=0), -1), (dict(H_kv=3), -1), (dict(H_kv=0), -1),
    (dict(scale=math.nan), -1), (dict(dtype=7), -1), (dict(lse=P + 1), -1),
    (dict(dtype=0), -2), (dict(dtype=3), -2), (dict(d=256), -2), (dict(Nk=1 << 22), -2),
])
def test_decode_entry_point_rejects_bad_arguments(kw, status):
    assert decode_call(**kw) == status
    assert _lib.load().fa_last_error().decode() != ""


def noalloc_call(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=2, H=8, H_kv=2, Nq=1, Nk=4096, d=128, scale=0.1,
             causal=1, key_len=None, dtype=2, stream=None)
    a.update(kw)
    return _lib.fa_fwd_decode_noalloc_raw(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"],
                                          a["H"], a["H_kv"], a["Nq"], a["Nk"], a["d"], a["scale"],
                                          a["causal"], a["key_len"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(Nq=0), -1), (dict(H_kv=3), -1), (dict(scale=math.nan), -1),
    (dict(o=P + 8), -1), (dict(dtype=0), -2), (dict(d=256), -2),
    # partial results beyond the library's scratch: 64*32*64 rows x (128+1) floats
    (dict(B=64, H=32, H_kv=8, Nq=64, Nk=8192), -2),
])
def test_noalloc_decode_rejects_bad_arguments(kw, status):
    assert noalloc_call(**kw) == status
    assert _lib.load().fa_last_error().decode() != ""


def test_noalloc_decode_limit_is_the_workspace_size():
    limit = 8 << 20
    header = open(HEADER).read()
    assert re.search(r"#define FA_DECODE_NOALLOC_MAX_BYTES \(8u << 20\)", header)
    assert _lib.decode_workspace_bytes(64, 32, 8, 64, 8192, 128) > limit
    assert noalloc_call(B=64, H=32, H_kv=8, Nq=64, Nk=8192) == -2
    assert "FA_DECODE_NOALLOC_MAX_BYTES" in _lib.load().fa_last_error().decode()
    # the decode workload of the benchmark fits
    assert _lib.decode_workspace_bytes(16, 32, 8, 1, 16384, 128) <= limit


def test_decode_workspace_size():
    ws = _lib.decode_workspace_bytes
    n = ws(2, 8, 2, 1, 4096, 128)
    assert n > 0 and n % 4 == 0
    # exactly too small is rejected before anything is enqueued
    assert decode_call(ws_bytes=n - 1) == -1
    assert ws(2, 8, 3, 1, 4096, 128) == 0 and ws(0, 8, 2, 1, 64, 64) == 0
    assert ws(1, 1, 1, 1, 1, 64) > 0
    # covers one partial O row and LSE per (query row, chunk)
    rows = 2 * 8 * 1
    assert n >= rows * 4 * (128 + 1)


def window_call(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=4, H_kv=2, N=64, d=64, scale=0.125, causal=1,
             wl=16, wr=-1, key_len=None, dtype=2, qd=1.0, kd=1.0, vd=1.0, stream=None)
    a.update(kw)
    return _lib.fa_fwd_window_raw(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"],
                                  a["H_kv"], a["N"], a["d"], a["scale"], a["causal"], a["wl"],
                                  a["wr"], a["key_len"], a["dtype"], a["qd"], a["kd"], a["vd"],
                                  a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=0), -2), (dict(dtype=3), -2), (dict(d=256), -2), (dict(H_kv=3), -1),
    (dict(q=None), -1), (dict(scale=0.0), -1), (dict(wr=5, d=96), -2),
])
def test_window_entry_point_rejects_bad_arguments(kw, status):
    assert window_call(**kw) == status
    assert _lib.load().fa_last_error().decode() != ""


def varlen_call(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, cu=P, B=3, H=4, H_kv=2, total=100, max_seqlen=50, d=64,
             scale=0.125, causal=1, dtype=2, stream=None)
    a.update(kw)
    return _lib.fa_fwd_varlen_raw(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cu"], a["B"],
                                  a["H"], a["H_kv"], a["total"], a["max_seqlen"], a["d"],
                                  a["scale"], a["causal"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(cu=None), -1), (dict(q=None), -1), (dict(lse=None), -1), (dict(B=0), -1),
    (dict(H=0), -1), (dict(total=0), -1), (dict(max_seqlen=0), -1), (dict(H_kv=3), -1),
    (dict(dtype=7), -1), (dict(scale=math.nan), -1), (dict(k=P + 8), -1), (dict(cu=P + 2), -1),
    (dict(dtype=0), -2), (dict(dtype=3), -2), (dict(d=256), -2), (dict(d=96), -2),
    (dict(total=1 << 23, max_seqlen=1 << 23), -2),
    (dict(B=1 << 30, H=8, max_seqlen=1000, total=100000), -1),
])
def test_varlen_entry_point_rejects_bad_arguments(kw, status):
    assert varlen_call(**kw) == status
    assert _lib.load().fa_last_error().decode() != ""


def sig_default(fn, name):
    import inspect
    return inspect.signature(fn).parameters[name].default


def test_python_binding_names_the_entry_points():
    import inspect

    import exact_io_aware_56_amd as fa

    assert callable(fa.fa_fwd) and callable(fa.fa_fwd_fp8) and callable(fa.fa_fwd_gqa)
    assert callable(fa.fa_fwd_fp8_p8) and sig_default(fa.fwd, "p8") is False
    sig = inspect.signature(fa.fwd)
    assert list(sig.parameters)[:3] == ["q", "k", "v"]
    for name in ("scale", "causal", "key_len"):
        assert sig.parameters[name].kind is inspect.Parameter.KEYWORD_ONLY, name
    assert sig.parameters["causal"].default is False
    assert sig.parameters["key_len"].default is None
