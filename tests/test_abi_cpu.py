"""The C-ABI library loads, exports every declared symbol and rejects bad arguments
before touching a GPU (no compute calls here)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(csa_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from certified_sparse_attention_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from certified_sparse_attention_amd import _build
        _build.build()
    return _lib.load()


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert len(names) >= 10
    for name in names:
        assert hasattr(lib, name), name


def test_binding_covers_every_declared_symbol():
    from certified_sparse_attention_amd import _lib
    assert set(_declared()) == set(_lib.SYMBOLS)


def test_status_strings(lib):
    assert lib.csa_status_string(0) == b"CSA_OK"
    assert lib.csa_status_string(-1) == b"CSA_ERR_INVALID_ARGUMENT"
    assert lib.csa_status_string(-2) == b"CSA_ERR_UNSUPPORTED"
    assert lib.csa_status_string(-3) == b"CSA_ERR_WORKSPACE"
    assert lib.csa_status_string(-4) == b"CSA_ERR_HIP"


def _shape(H=8, G=4, d=128, n_cap=4096):
    from certified_sparse_attention_amd import _lib
    return _lib.Shape(H, G, d, n_cap)


def _params(**kw):
    from certified_sparse_attention_amd import _lib
    p = dict(eps=0.05, delta=0.01, r=2, J=30, window=64, measure=2, seed=1, step=0, layer=0, cand_budget=0)
    p.update(kw)
    return _lib.Params(**p)


def test_workspace_bytes_validates(lib):
    ok = lib.csa_workspace_bytes(ctypes.byref(_shape()), ctypes.byref(_params()), 4096)
    assert ok > 0
    assert lib.csa_workspace_bytes(ctypes.byref(_shape(d=64)), ctypes.byref(_params()), 4096) == 0
    assert lib.csa_workspace_bytes(ctypes.byref(_shape(G=8)), ctypes.byref(_params()), 4096) == 0
    assert lib.csa_workspace_bytes(ctypes.byref(_shape()), ctypes.byref(_params(J=61)), 4096) == 0
    assert lib.csa_workspace_bytes(ctypes.byref(_shape()), ctypes.byref(_params(delta=1.0)), 4096) == 0
    assert lib.csa_workspace_bytes(ctypes.byref(_shape()), ctypes.byref(_params(window=16)), 4096) == 0
    assert lib.csa_workspace_bytes(ctypes.byref(_shape()), ctypes.byref(_params(window=1025)), 4096) == 0
    assert lib.csa_workspace_bytes(ctypes.byref(_shape()), ctypes.byref(_params(window=1024)), 4096) > 0
    assert lib.csa_workspace_bytes(ctypes.byref(_shape(n_cap=100)), ctypes.byref(_params()), 64) == 0
    # grows with n and J
    a = lib.csa_workspace_bytes(ctypes.byref(_shape()), ctypes.byref(_params()), 2048)
    b = lib.csa_workspace_bytes(ctypes.byref(_shape()), ctypes.byref(_params(J=48)), 4096)
    assert a < ok < b


@pytest.mark.parametrize("bad", [
    dict(shape=None), dict(d=96), dict(G=0), dict(G=8), dict(eps=0.0), dict(eps=-1.0),
    dict(delta=0.0), dict(r=0), dict(J=-1), dict(J=70), dict(window=8), dict(window=2048), dict(measure=5),
    dict(n=0), dict(n=5000), dict(null_q=True), dict(ws_small=True),
])
def test_certified_call_rejects_bad_arguments(lib, bad):
    from certified_sparse_attention_amd import _lib
    sh = None if "shape" in bad else _shape(d=bad.get("d", 128), G=bad.get("G", 4))
    pr = _params(**{k: v for k, v in bad.items() if k in ("eps", "delta", "r", "J", "window", "measure")})
    fake = ctypes.c_void_p(0x1000)      # never dereferenced: validation fails first
    pk = _lib.Packed(fake, fake, fake, fake, fake, fake)
    n = bad.get("n", 1024)
    rc = lib.csa_certified_decode_attention(
        ctypes.byref(sh) if sh is not None else None, ctypes.byref(pr),
        None if bad.get("null_q") else fake, fake, fake, ctypes.byref(pk), n,
        fake, 16 if bad.get("ws_small") else 1 << 40, fake, fake, fake, fake, None, None)
    assert rc in (-1, -2, -3), rc
    assert len(lib.csa_last_error()) > 0


def test_pack_rejects_bad_block_range(lib):
    from certified_sparse_attention_amd import _lib
    fake = ctypes.c_void_p(0x1000)
    pk = _lib.Packed(fake, fake, fake, fake, fake, fake)
    sh = _shape(n_cap=4096)
    assert lib.csa_pack_kv_4bit(ctypes.byref(sh), fake, fake, 0, 129, ctypes.byref(pk), None) == -1
    assert lib.csa_pack_kv_4bit(ctypes.byref(sh), fake, fake, 5, 4, ctypes.byref(pk), None) == -1
    pk2 = _lib.Packed(fake, None, fake, fake, fake, fake)
    assert lib.csa_pack_kv_4bit(ctypes.byref(sh), fake, fake, 0, 1, ctypes.byref(pk2), None) == -1


def test_dense_rejects_bad_arguments(lib):
    fake = ctypes.c_void_p(0x1000)
    sh = _shape()
    assert lib.csa_dense_decode_attention(ctypes.byref(sh), fake, fake, fake, 0, fake, 1 << 30, fake, None) == -1
    assert lib.csa_dense_decode_attention(ctypes.byref(sh), fake, fake, fake, 64, fake, 4, fake, None) == -3
    assert lib.csa_dense_workspace_bytes(ctypes.byref(sh), 4096) > 0


def test_stream_read_rejects_bad_arguments(lib):
    fake = ctypes.c_void_p(0x1000)
    assert lib.csa_stream_read(None, 1024, 4, fake, None, None, None) == -1            # null buffer
    assert lib.csa_stream_read(fake, 1000, 4, fake, None, None, None) == -1            # not a multiple of 16
    assert lib.csa_stream_read(ctypes.c_void_p(0x1004), 1024, 4, fake, None, None, None) == -1   # misaligned
    assert lib.csa_stream_read(fake, 1024, 0, fake, None, None, None) == -1            # no workgroups
    assert lib.csa_stream_read(fake, 1024, 70000, fake, None, None, None) == -1        # too many


def test_workspace_bytes_batch_validates(lib):
    one = lib.csa_workspace_bytes(ctypes.byref(_shape()), ctypes.byref(_params()), 4096)
    b1 = lib.csa_workspace_bytes_batch(ctypes.byref(_shape()), ctypes.byref(_params()), 1, 4096)
    b16 = lib.csa_workspace_bytes_batch(ctypes.byref(_shape()), ctypes.byref(_params()), 16, 4096)
    assert b1 == one and b16 > 8 * one
    assert lib.csa_workspace_bytes_batch(ctypes.byref(_shape()), ctypes.byref(_params()), 0, 4096) == 0
    assert lib.csa_workspace_bytes_batch(ctypes.byref(_shape()), ctypes.byref(_params()), 65, 4096) == 0
    assert lib.csa_workspace_bytes_batch(ctypes.byref(_shape()), ctypes.byref(_params()), 64, 4096) > 0


@pytest.mark.parametrize("bad", [
    dict(num_items=0), dict(num_items=65), dict(num_slots=0), dict(slot=2), dict(slot=-1), dict(n=0),
    dict(n=5000), dict(eps=0.0), dict(eps=float("nan")), dict(null_items=True), dict(null_q=True),
    dict(ws_small=True), dict(J=61),
])
def test_batch_call_rejects_bad_arguments(lib, bad):
    from certified_sparse_attention_amd import _lib
    sh = _shape(n_cap=4096)
    pr = _params(**{k: v for k, v in bad.items() if k in ("J",)})
    fake = ctypes.c_void_p(0x1000)      # never dereferenced: validation fails first
    pk = _lib.Packed(*([fake] * 9))
    nitems = bad.get("num_items", 3)
    arr = (_lib.Item * max(nitems, 1))()
    for i in range(max(nitems, 1)):
        arr[i] = _lib.Item(1000 + i, i % 2, 0, 0.05, 1, 0)
    arr[0] = _lib.Item(bad.get("n", 1000), bad.get("slot", 0), 0, bad.get("eps", 0.05), 1, 0)
    rc = lib.csa_certified_decode_attention_batch(
        ctypes.byref(sh), ctypes.byref(pr), bad.get("num_slots", 2), nitems, None if bad.get("null_items") else arr,
        None if bad.get("null_q") else fake, fake, fake, ctypes.byref(pk), fake,
        16 if bad.get("ws_small") else 1 << 40, fake, fake, fake, fake, None)
    assert rc in (-1, -2, -3), rc
    assert len(lib.csa_last_error()) > 0
