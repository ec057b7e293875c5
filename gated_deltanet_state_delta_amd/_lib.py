"""ctypes view of libgdn.so: the structs and prototypes of include/libgdn.h.

Loading is lazy; a missing library raises at first use (there is no other
implementation to fall back to).
"""
from __future__ import annotations

import ctypes
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libgdn.so")

GDN_OK = 0
GDN_F32, GDN_BF16 = 0, 1
GDN_DECAY_LOG, GDN_DECAY_GAMMA = 0, 1

STATUS_NAMES = {0: "GDN_OK", 1: "GDN_ERR_NULL", 2: "GDN_ERR_SHAPE", 3: "GDN_ERR_DTYPE",
                4: "GDN_ERR_LAYOUT", 5: "GDN_ERR_UNSUPPORTED", 6: "GDN_ERR_HIP"}

# every extern "C" symbol include/libgdn.h declares
EXPORTED = ("gdn_last_error", "gdn_version", "gdn_gate", "gdn_prefill", "gdn_prefill_workspace_size",
            "gdn_prefill_noalloc", "gdn_decode", "gdn_conv1d", "gdn_wait_timeouts")
NOALLOC_SCRATCH_BYTES = 32 << 20  # GDN_NOALLOC_SCRATCH_BYTES

_i32, _i64, _f32, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p


class PrefillArgs(ctypes.Structure):
    _fields_ = [
        ("n_seqs", _i32), ("seq_len", _i32), ("total_tokens", _i64),
        ("hq", _i32), ("hv", _i32), ("dk", _i32), ("dv", _i32),
        ("io_dtype", _i32), ("decay_kind", _i32), ("chunk_size", _i32), ("scale", _f32),
        ("q", _vp), ("q_stride_token", _i64), ("q_stride_head", _i64),
        ("k", _vp), ("k_stride_token", _i64), ("k_stride_head", _i64),
        ("v", _vp), ("v_stride_token", _i64), ("v_stride_head", _i64),
        ("out", _vp), ("out_stride_token", _i64), ("out_stride_head", _i64),
        ("decay", _vp), ("beta", _vp), ("cu_seqlens", _vp),
        ("initial_state", _vp), ("final_state", _vp),
        ("qk_l2norm", _i32), ("qk_l2norm_eps", _f32),
        ("A_log", _vp), ("dt_bias", _vp), ("gate_a", _vp), ("gate_b", _vp),
        ("update_rule", _i32),
        ("state_pool", _vp), ("pool_size", _i32),
        ("pool_slot_stride", _i64), ("pool_head_stride", _i64),
        ("read_slot", _vp), ("write_slot", _vp),
        ("workspace", _vp), ("workspace_bytes", ctypes.c_size_t),
        ("decay_per_key", _i32),
    ]


class DecodeArgs(ctypes.Structure):
    _fields_ = [
        ("batch", _i32), ("T", _i32), ("n_householder", _i32),
        ("hq", _i32), ("hv", _i32), ("dk", _i32), ("dv", _i32),
        ("io_dtype", _i32), ("disable_state_update", _i32), ("scale", _f32),
        ("q", _vp), ("k", _vp), ("v", _vp), ("A_log", _vp), ("dt_bias", _vp),
        ("a", _vp), ("b", _vp),
        ("pool", _vp), ("pool_size", _i32),
        ("pool_slot_stride", _i64), ("pool_head_stride", _i64),
        ("read_idx", _vp), ("write_idx", _vp), ("scatter_idx", _vp),
        ("out", _vp),
        ("qk_l2norm", _i32), ("qk_l2norm_eps", _f32),
        ("decay_per_key", _vp),
    ]


class Conv1dArgs(ctypes.Structure):
    _fields_ = [
        ("total_tokens", _i64), ("conv_dim", _i32), ("kernel_size", _i32),
        ("n_seqs", _i32), ("io_dtype", _i32), ("write_state", _i32), ("max_slots", _i32),
        ("x", _vp), ("x_stride_token", _i64),
        ("weight", _vp), ("conv_state", _vp),
        ("slot_idx", _vp), ("row_offsets", _vp),
        ("out", _vp), ("out_stride_token", _i64),
    ]


_lock = threading.Lock()
_lib = None


def load(path: str | None = None):
    """Load libgdn.so (once) and declare its prototypes."""
    global _lib
    with _lock:
        if _lib is not None and path is None:
            return _lib
        p = path or LIB_PATH
        if not os.path.exists(p):
            raise RuntimeError("libgdn.so is not built (%s); run "
                               "`python -m gated_deltanet_state_delta_amd.build`" % p)
        lib = ctypes.CDLL(p)
        lib.gdn_last_error.restype = ctypes.c_char_p
        lib.gdn_last_error.argtypes = []
        lib.gdn_version.restype = ctypes.c_char_p
        lib.gdn_version.argtypes = []
        lib.gdn_gate.restype = ctypes.c_int
        lib.gdn_gate.argtypes = [_vp, _vp, _vp, _vp, _i32, _i64, _i32, _vp, _vp, _vp, _vp]
        lib.gdn_prefill_workspace_size.restype = ctypes.c_size_t
        lib.gdn_prefill_workspace_size.argtypes = [ctypes.POINTER(PrefillArgs)]
        lib.gdn_prefill.restype = ctypes.c_int
        lib.gdn_prefill.argtypes = [ctypes.POINTER(PrefillArgs), _vp]
        lib.gdn_prefill_noalloc.restype = ctypes.c_int
        lib.gdn_prefill_noalloc.argtypes = [ctypes.POINTER(PrefillArgs), _vp]
        lib.gdn_decode.restype = ctypes.c_int
        lib.gdn_decode.argtypes = [ctypes.POINTER(DecodeArgs), _vp]
        lib.gdn_wait_timeouts.restype = ctypes.c_int
        lib.gdn_wait_timeouts.argtypes = [ctypes.POINTER(ctypes.c_uint32), _i32]
        lib.gdn_conv1d.restype = ctypes.c_int
        lib.gdn_conv1d.argtypes = [ctypes.POINTER(Conv1dArgs), _vp]
        if path is None:
            _lib = lib
        return lib


class GdnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("%s: %s" % (STATUS_NAMES.get(status, str(status)), msg))
        self.status = status


def check(status: int):
    if status != GDN_OK:
        raise GdnError(status, load().gdn_last_error().decode(errors="replace"))
