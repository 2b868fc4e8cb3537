"""The C-ABI library builds for gfx950, loads, exports every symbol the
header declares, and rejects bad arguments on the host before touching a
device.  No kernel is launched here."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    from linear_attention_state_anchor_amd import _lib, build
    if not os.path.exists(_lib.LIB_PATH):
        build.build()
    return _lib.load()


def declared_symbols():
    names = set()
    inc = os.path.join(ROOT, "include")
    for f in os.listdir(inc):
        if f.endswith(".h"):
            text = open(os.path.join(inc, f)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(sr_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_every_declared_symbol_is_exported(lib):
    from linear_attention_state_anchor_amd import _lib
    syms = declared_symbols()
    assert "sr_gdn_replay_state" in syms and "sr_replay_group" in syms
    for s in syms:
        assert hasattr(lib, s), s
        assert s in _lib.SIGNATURES, f"binding lacks {s}"


def test_version_and_status_strings(lib):
    assert b"gfx950" in lib.sr_version()
    for code in range(7):
        assert lib.sr_status_str(code)
    assert lib.sr_status_str(99) == b"unknown status"


def _desc(**kw):
    from linear_attention_state_anchor_amd import _lib
    base = dict(n_seqs=1, total_tokens=4, h_k=1, h_v=1, d_k=64, d_v=64,
                dtype_qkv=_lib.SR_BF16, dtype_o=_lib.SR_BF16, erase=1,
                alpha_is_log=0, scale=1.0)
    base.update(kw)
    return _lib.GdnDesc(**base)


def test_gdn_argument_validation(lib):
    from linear_attention_state_anchor_amd import _lib
    io = _lib.GdnIO()
    call = lambda d, i=io: lib.sr_gdn_replay_state(ctypes.byref(d), ctypes.byref(i), None)
    assert lib.sr_gdn_replay_state(None, None, None) == _lib.SR_EINVAL
    assert call(_desc(n_seqs=-1)) == _lib.SR_ESHAPE
    assert call(_desc(h_k=3, h_v=4)) == _lib.SR_ESHAPE
    assert call(_desc(d_k=0)) == _lib.SR_ESHAPE
    assert call(_desc(dtype_qkv=7)) == _lib.SR_EDTYPE
    assert call(_desc(dtype_o=-1)) == _lib.SR_EDTYPE
    assert call(_desc(erase=2)) == _lib.SR_EINVAL
    assert call(_desc()) == _lib.SR_EINVAL            # null pointers
    assert call(_desc(n_seqs=0)) == _lib.SR_OK        # nothing to do
    # misaligned q/k/v for the chunked kernel
    fake = ctypes.c_void_p(0x1008)
    io2 = _lib.GdnIO(fake, fake, fake, fake, None, fake, None, fake, None)
    assert call(_desc(), io2) == _lib.SR_EINVAL
    # unsupported head size on every kernel
    io3 = _lib.GdnIO(None, ctypes.c_void_p(0x1000), ctypes.c_void_p(0x1000),
                     ctypes.c_void_p(0x1000), None, ctypes.c_void_p(0x1000), None,
                     ctypes.c_void_p(0x1000), None)
    assert call(_desc(d_k=48, d_v=48), io3) == _lib.SR_ESHAPE


def test_gather_argument_validation(lib):
    from linear_attention_state_anchor_amd import _lib
    P = ctypes.c_void_p(0x1000)
    g = lambda **kw: lib.sr_gather_suffix(
        kw.get("pool", P), kw.get("hidden", 64), kw.get("eb", 2), kw.get("np_", 1),
        kw.get("pt", P), kw.get("pts", 4), P, P, kw.get("n", 1), kw.get("T", 3),
        kw.get("out", P), kw.get("cu", P), None)
    assert g(eb=3) == _lib.SR_EDTYPE
    assert g(hidden=3) == _lib.SR_ESHAPE              # row not a multiple of 16 B
    assert g(n=-1) == _lib.SR_ESHAPE
    assert g(cu=None) == _lib.SR_EINVAL
    assert g(pool=None) == _lib.SR_EINVAL
    assert g(pool=ctypes.c_void_p(0x1004)) == _lib.SR_EINVAL
    assert g(n=0) == _lib.SR_ESHAPE                   # rows but no requests
