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
    for code in range(8):
        assert lib.sr_status_str(code) != b"unknown status"
    assert lib.sr_status_str(99) == b"unknown status"


def test_gdn_workspace_bytes(lib):
    ws = lambda **kw: lib.sr_gdn_workspace_bytes(ctypes.byref(_desc(**kw)))
    bad = ctypes.c_size_t(-1).value
    assert ws() == 0
    assert ws(d_k=128, d_v=128, h_k=16, h_v=32) == 0
    assert ws(dtype_qkv=2, d_k=32, d_v=128) == 0        # token-serial fp32 kernel
    assert ws(h_k=3, h_v=4) == bad
    assert ws(d_k=48, d_v=48) == bad
    assert lib.sr_gdn_workspace_bytes(None) == bad


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
    call = lambda d, i=io: lib.sr_gdn_replay_state(ctypes.byref(d), ctypes.byref(i), None, 0,
                                                   None)
    assert lib.sr_gdn_replay_state(None, None, None, 0, None) == _lib.SR_EINVAL
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


def test_anchor_gather_argument_validation(lib):
    from linear_attention_state_anchor_amd import _lib
    P = ctypes.c_void_p(0x1000)
    offs = (ctypes.c_int32 * 4)(60, 61, 62, 63)
    g = lambda a=4, o=offs, **kw: lib.sr_gather_anchors(
        P, 64, 2, 1, a, o, P, 4, P, P, kw.get("n", 1), kw.get("T", 3), P, P, None, None)
    assert g(o=None) == _lib.SR_EINVAL
    assert g(a=0) == _lib.SR_ESHAPE
    assert g(a=65) == _lib.SR_ESHAPE
    bad = (ctypes.c_int32 * 4)(60, 62, 61, 63)         # not increasing
    assert g(o=bad) == _lib.SR_ESHAPE
    out = (ctypes.c_int32 * 4)(0, 1, 2, 64)            # past the page
    assert g(o=out) == _lib.SR_ESHAPE
    assert g(n=0) == _lib.SR_ESHAPE


def test_replay_budget_host_function(lib):
    from linear_attention_state_anchor_amd import replay_budget
    assert replay_budget([0, 1, 20, 21, 100, 20480, 32768], 0.05, 0) == [0, 1, 1, 2, 5, 1024,
                                                                         1639]
    assert replay_budget([20480, 32768, 8192], 0.05, 512) == [512, 512, 410]
    assert replay_budget([32768, 2048], 0.05, 256) == [256, 103]
    assert replay_budget([100], 0.07, 0) == [7]         # 0.07 * 100 is 7.000000000000001 in binary
    assert replay_budget([3276 * 10], 0.10, 0) == [3276]
    import pytest as _pt
    with _pt.raises(ValueError):
        replay_budget([10], 0.0, 0)
    with _pt.raises(ValueError):
        replay_budget([-1], 0.05, 0)


def test_binding_rejects_bad_buffers_before_the_library():
    """Python-side checks: caller-supplied buffers with the wrong shape,
    dtype or device raise ValueError/TypeError before any pointer reaches
    the library (checked on CPU tensors, which fail the device test first,
    and on shape mismatches the checks see before the device test)."""
    import pytest as _pt
    import torch
    import linear_attention_state_anchor_amd as sr
    with _pt.raises(ValueError):
        sr.gdn_replay_state(None, torch.zeros(4, 1, 64), torch.zeros(4, 1, 64),
                            torch.zeros(4, 1), want_o=False)   # host tensors
    with _pt.raises(TypeError):
        sr.gdn_replay_state(None, [0.0], None, None, want_o=False)
    with _pt.raises(ValueError):
        sr.replay_budget([5], 1.5)
