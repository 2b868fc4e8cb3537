"""ctypes declarations of the C ABI in include/sr_replay.h.

Argument marshalling only: no arithmetic of the method happens here.  Loading
fails loudly when libsr_replay.so has not been built; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsr_replay.so")

SR_OK, SR_EINVAL, SR_ESHAPE, SR_EDTYPE, SR_EWORKSPACE, SR_ELAUNCH, SR_EDEVICE, SR_EDATA = range(8)
# statuses that mean "the arguments (or the device data they point to) are
# outside the contract", raised as ValueError
ARGUMENT_STATUSES = (SR_EINVAL, SR_ESHAPE, SR_EDTYPE, SR_EWORKSPACE, SR_EDATA)
SR_BF16, SR_F16, SR_F32 = 0, 1, 2
SR_LAYER_GDN, SR_LAYER_FA = 0, 1

c_i32 = ctypes.c_int32
c_p = ctypes.c_void_p


class GdnDesc(ctypes.Structure):
    _fields_ = [("n_seqs", c_i32), ("total_tokens", c_i32), ("h_k", c_i32),
                ("h_v", c_i32), ("d_k", c_i32), ("d_v", c_i32),
                ("dtype_qkv", c_i32), ("dtype_o", c_i32), ("erase", c_i32),
                ("alpha_is_log", c_i32), ("scale", ctypes.c_float)]


class GdnIO(ctypes.Structure):
    _fields_ = [("q", c_p), ("k", c_p), ("v", c_p), ("alpha", c_p), ("beta", c_p),
                ("cu_seqlens", c_p), ("initial_state", c_p), ("final_state", c_p),
                ("o", c_p)]


class GroupDesc(ctypes.Structure):
    _fields_ = [("n_layers", c_i32), ("layer_kind", ctypes.POINTER(c_i32)),
                ("hidden", c_i32), ("h_k", c_i32), ("h_v", c_i32), ("d", c_i32),
                ("conv_width", c_i32), ("rms_eps", ctypes.c_float),
                ("l2_eps", ctypes.c_float), ("n_seqs", c_i32),
                ("total_tokens", c_i32), ("max_seqlen", c_i32),
                ("layer_events", ctypes.POINTER(c_p)), ("ffn_dim", c_i32)]


class LayerWeights(ctypes.Structure):
    _fields_ = [("packed", c_p), ("ffn", c_p)]


# every symbol the header declares, with (restype, argtypes)
SIGNATURES = {
    "sr_version": (ctypes.c_char_p, []),
    "sr_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "sr_gdn_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(GdnDesc)]),
    "sr_gdn_replay_state": (ctypes.c_int, [ctypes.POINTER(GdnDesc), ctypes.POINTER(GdnIO), c_p,
                                           ctypes.c_size_t, c_p]),
    "sr_check_replay_inputs": (ctypes.c_int, [ctypes.POINTER(GdnDesc), ctypes.POINTER(GdnIO),
                                              c_p]),
    "sr_gdn_decode_step": (ctypes.c_int, [ctypes.POINTER(GdnDesc), ctypes.POINTER(GdnIO), c_p]),
    "sr_gather_suffix": (ctypes.c_int, [c_p, c_i32, c_i32, ctypes.c_int64, c_p, c_i32, c_p,
                                        c_p, c_i32, c_i32, c_p, c_p, c_p]),
    "sr_gather_anchors": (ctypes.c_int, [c_p, c_i32, c_i32, ctypes.c_int64, c_i32,
                                         ctypes.POINTER(c_i32), c_p, c_i32, c_p, c_p, c_i32,
                                         c_i32, c_p, c_p, c_p, c_p]),
    "sr_check_gather_inputs": (ctypes.c_int, [ctypes.c_int64, c_i32, ctypes.POINTER(c_i32), c_p,
                                              c_i32, c_p, c_p, c_i32, c_i32, c_p]),
    "sr_replay_budget": (ctypes.c_int64, [ctypes.POINTER(c_i32), c_i32, ctypes.c_double, c_i32,
                                          ctypes.POINTER(c_i32)]),
    "sr_packed_layer_bytes": (ctypes.c_size_t, [c_i32, c_i32, c_i32, c_i32, c_i32]),
    "sr_pack_gdn_layer": (ctypes.c_int, [c_p, c_p, c_p, c_i32, c_i32, c_i32, c_i32, c_i32,
                                         c_p, c_p]),
    "sr_packed_ffn_bytes": (ctypes.c_size_t, [c_i32, c_i32]),
    "sr_pack_ffn": (ctypes.c_int, [c_p, c_p, c_p, c_i32, c_i32, c_p, c_p]),
    "sr_replay_group_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(GroupDesc)]),
    "sr_replay_group": (ctypes.c_int, [ctypes.POINTER(GroupDesc), ctypes.POINTER(LayerWeights),
                                       c_p, c_p, c_p, c_p, c_p, ctypes.c_size_t, c_p]),
    "sr_extend_group": (ctypes.c_int, [ctypes.POINTER(GroupDesc), ctypes.POINTER(LayerWeights),
                                       c_p, c_p, c_p, c_p, c_p, c_p, c_p, c_p, ctypes.c_size_t,
                                       c_p]),
    "sr_replay_group_noalloc_max_bytes": (ctypes.c_size_t, []),
    "sr_replay_group_noalloc": (ctypes.c_int, [ctypes.POINTER(GroupDesc),
                                               ctypes.POINTER(LayerWeights), c_p, c_p, c_p, c_p,
                                               c_p]),
}

_lib = None
_lock = threading.Lock()


class ReplayError(RuntimeError):
    """A nonzero status from the C ABI (launch or device failures)."""

    def __init__(self, fn, status):
        self.status = status
        msg = load().sr_status_str(status).decode()
        super().__init__(f"{fn} failed: status {status} ({msg})")


class ReplayArgumentError(ReplayError, ValueError):
    """A status that rejects the arguments (or the device data they point to):
    SR_EINVAL, SR_ESHAPE, SR_EDTYPE, SR_EWORKSPACE, SR_EDATA."""


def load():
    """Load libsr_replay.so (raises if it is missing: no fallback path)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m linear_attention_state_anchor_amd.build` (hipcc, gfx950)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
        return lib


def check(fn, status):
    if status != SR_OK:
        if status in ARGUMENT_STATUSES:
            raise ReplayArgumentError(fn, status)
        raise ReplayError(fn, status)
