"""ctypes mirror of ``include/swa_sdpa.h`` and loader of ``libswa_sdpa.so``.

Argument marshalling only: every step of the attention runs in the HIP
library.  Loading fails loudly when the library has not been built; there is
no fallback path.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libswa_sdpa.so")

(SDPA_OK, SDPA_ERR_INVALID_ARG, SDPA_ERR_UNSUPPORTED, SDPA_ERR_WORKSPACE, SDPA_ERR_HIP,
 SDPA_ERR_RELAY_TIMEOUT) = range(6)
SDPA_BF16, SDPA_F16 = 0, 1
SDPA_LAYOUT_BHSD, SDPA_LAYOUT_THD = 0, 1

_i32, _i64, _f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float
_vp = ctypes.c_void_p


class AttnDesc(ctypes.Structure):
    _fields_ = [
        ("dtype", _i32), ("layout", _i32), ("batch", _i32), ("heads_q", _i32),
        ("heads_kv", _i32), ("head_dim", _i32), ("seq_q", _i32), ("seq_kv", _i32),
        ("total_q", _i64), ("total_kv", _i64), ("causal", _i32), ("bottom_right", _i32),
        ("window_left", _i32), ("window_right", _i32), ("scale", _f32), ("deterministic", _i32), ("has_sink", _i32),
        ("has_seq_lens", _i32), ("q_run_tiles", _i32), ("engine", _i32),
        ("stride_q", _i64 * 3), ("stride_k", _i64 * 3), ("stride_v", _i64 * 3),
        ("stride_o", _i64 * 3), ("stride_do", _i64 * 3), ("stride_dq", _i64 * 3),
        ("stride_dk", _i64 * 3), ("stride_dv", _i64 * 3),
    ]


class FwdTensors(ctypes.Structure):
    _fields_ = [("q", _vp), ("k", _vp), ("v", _vp), ("sink", _vp), ("cu_seqlens_q", _vp),
                ("cu_seqlens_kv", _vp), ("seq_lens_q", _vp), ("seq_lens_kv", _vp),
                ("o", _vp), ("lse", _vp)]


class BwdTensors(ctypes.Structure):
    _fields_ = [("q", _vp), ("k", _vp), ("v", _vp), ("o", _vp), ("dO", _vp), ("lse", _vp),
                ("sink", _vp), ("cu_seqlens_q", _vp), ("cu_seqlens_kv", _vp),
                ("seq_lens_q", _vp), ("seq_lens_kv", _vp), ("dq", _vp), ("dk", _vp),
                ("dv", _vp), ("dsink", _vp)]


EXPORTS = [
    "sdpa_bwd_plan", "sdpa_bwd_run", "sdpa_bwd_run_events", "sdpa_bwd_plan_destroy",
    "sdpa_fwd_plan", "sdpa_fwd_run", "sdpa_fwd_plan_destroy", "sdpa_bwd_schedule",
    "sdpa_bwd_relay_expiries", "sdpa_bwd_plan_set_relay_watchdog", "sdpa_status_string", "sdpa_last_error",
    "sdpa_bwd_run_noalloc",
]

_lib = None


def load(path: str = LIB_PATH):
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} not found: build it first (python -m sliding_window_attention_flash_amd.build "
            "or __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    PP = ctypes.POINTER(_vp)
    sz = ctypes.POINTER(ctypes.c_size_t)
    lib.sdpa_bwd_plan.argtypes = [ctypes.POINTER(AttnDesc), PP, sz]
    lib.sdpa_bwd_run.argtypes = [_vp, ctypes.POINTER(BwdTensors), _vp, ctypes.c_size_t, _vp]
    lib.sdpa_bwd_run_events.argtypes = [_vp, ctypes.POINTER(BwdTensors), _vp, ctypes.c_size_t,
                                        _vp, _vp, _vp]
    lib.sdpa_bwd_run_noalloc.argtypes = [_vp, ctypes.POINTER(BwdTensors), _vp]
    lib.sdpa_bwd_run_noalloc.restype = ctypes.c_int
    lib.sdpa_bwd_plan_destroy.argtypes = [_vp]
    lib.sdpa_bwd_plan_destroy.restype = None
    lib.sdpa_fwd_plan.argtypes = [ctypes.POINTER(AttnDesc), PP, sz]
    lib.sdpa_fwd_run.argtypes = [_vp, ctypes.POINTER(FwdTensors), _vp, ctypes.c_size_t, _vp]
    lib.sdpa_fwd_plan_destroy.argtypes = [_vp]
    lib.sdpa_fwd_plan_destroy.restype = None
    ip = ctypes.POINTER(_i32)
    lib.sdpa_bwd_schedule.argtypes = [_vp, _i32, _i32, ip, ip, ip, ip, _i32, ip, ip, _i32, ip, ip]
    lib.sdpa_bwd_relay_expiries.argtypes = [_vp, _vp, _vp, ip]
    lib.sdpa_bwd_relay_expiries.restype = ctypes.c_int
    lib.sdpa_bwd_plan_set_relay_watchdog.argtypes = [_vp, _i32, _i32]
    lib.sdpa_bwd_plan_set_relay_watchdog.restype = ctypes.c_int
    lib.sdpa_status_string.argtypes = [ctypes.c_int]
    lib.sdpa_status_string.restype = ctypes.c_char_p
    lib.sdpa_last_error.argtypes = []
    lib.sdpa_last_error.restype = ctypes.c_char_p
    for name in ("sdpa_bwd_plan", "sdpa_bwd_run", "sdpa_bwd_run_events", "sdpa_fwd_plan",
                 "sdpa_fwd_run", "sdpa_bwd_schedule"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


class SdpaError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = load()
        msg = lib.sdpa_last_error().decode(errors="replace")
        name = lib.sdpa_status_string(status).decode()
        super().__init__(f"{where}: {name}: {msg}")
        self.status = status


def check(status: int, where: str) -> None:
    if status != SDPA_OK:
        raise SdpaError(status, where)
