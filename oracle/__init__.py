"""fp64 CPU oracle for sliding-window attention forward and backward.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this package.  The GPU
library and its Python binding never do; the two share no code.

The arithmetic lives in ``swa_oracle.c`` (plain C, fp64, OpenMP over
independent (sequence, head) units).  This module compiles it with gcc and
marshals torch CPU tensors into it; it performs no attention arithmetic of
its own.

Every function here states the layout it expects.  Two layouts are built in:

* dense ``[B, H, S, D]`` (``Problem.dense``), with optional per-batch valid
  lengths (padding mask);
* packed ``[T, H, D]`` (``Problem.packed``) with ``cu_seqlens`` giving each
  sequence's first row and per-sequence valid lengths (THD).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "swa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libswa_oracle.so")

BF16, F16, F64 = 0, 1, 2
_DT = {torch.bfloat16: BF16, torch.float16: F16, torch.float64: F64}


class _Problem(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int),
        ("batch", ctypes.c_int),
        ("heads_q", ctypes.c_int),
        ("heads_kv", ctypes.c_int),
        ("head_dim", ctypes.c_int),
        ("causal", ctypes.c_int),
        ("bottom_right", ctypes.c_int),
        ("window_left", ctypes.c_int),
        ("window_right", ctypes.c_int),
        ("dense", ctypes.c_int),
        ("has_sink", ctypes.c_int),
        ("scale", ctypes.c_double),
        ("len_q", ctypes.c_void_p),
        ("len_kv", ctypes.c_void_p),
        ("row0_q", ctypes.c_void_p),
        ("row0_kv", ctypes.c_void_p),
        ("q_stride_h", ctypes.c_int64),
        ("q_stride_r", ctypes.c_int64),
        ("kv_stride_h", ctypes.c_int64),
        ("kv_stride_r", ctypes.c_int64),
        ("stat_ld", ctypes.c_int64),
    ]


def build(out_path: str = _LIB_PATH, mutant: int = 0) -> str:
    """Compile the oracle with gcc (``mutant`` > 0 plants a known mistake,
    used only by the test that checks the pins catch mistakes)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11", "-o", out_path, _SRC, "-lm", "-lpthread"]
    if mutant:
        cmd.insert(1, f"-DORACLE_MUTANT={int(mutant)}")
    subprocess.run(cmd, check=True)
    return out_path


_lib_cache: dict = {}


def load(path: str = _LIB_PATH):
    """Load (building first if absent) the oracle shared library."""
    if path in _lib_cache:
        return _lib_cache[path]
    if not os.path.exists(path):
        build(path)
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(_Problem)
    vp, i32 = ctypes.c_void_p, ctypes.c_int
    lib.oracle_forward.argtypes = [P, vp, vp, vp, vp, vp, vp]
    lib.oracle_backward.argtypes = [P] + [vp] * 12
    lib.oracle_dq_rows.argtypes = [P, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp]
    lib.oracle_dkdv_rows.argtypes = [P, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp]
    lib.oracle_attended_pairs.argtypes = [P]
    lib.oracle_attended_pairs.restype = ctypes.c_int64
    lib.oracle_num_threads.restype = ctypes.c_int
    for name in ("oracle_forward", "oracle_backward", "oracle_dq_rows", "oracle_dkdv_rows"):
        getattr(lib, name).restype = ctypes.c_int
    _lib_cache[path] = lib
    return lib


def num_threads() -> int:
    return int(load().oracle_num_threads())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


@dataclass
class Problem:
    """Shape and mask of one attention problem, plus the row addressing of
    the tensors handed to the oracle (see ``swa_oracle.h``)."""

    batch: int
    heads_q: int
    heads_kv: int
    head_dim: int
    len_q: torch.Tensor  # int32 [batch]
    len_kv: torch.Tensor  # int32 [batch]
    row0_q: torch.Tensor  # int64 [batch]
    row0_kv: torch.Tensor  # int64 [batch]
    q_stride_h: int
    q_stride_r: int
    kv_stride_h: int
    kv_stride_r: int
    stat_ld: int
    causal: bool = True
    bottom_right: bool = False
    window_left: int = -1
    scale: float = 1.0
    has_sink: bool = False
    dense_scan: bool = False
    q_numel: int = 0
    kv_numel: int = 0
    window_right: int = 0  # causal only: inclusive right band (0: plain causal)
    _keep: list = field(default_factory=list, repr=False)

    @staticmethod
    def dense(B, Hq, Hkv, Sq, Skv, D, *, causal=True, bottom_right=False, window_left=-1,
              window_right=0, scale=None, has_sink=False, len_q=None, len_kv=None) -> "Problem":
        """Contiguous ``[B, H, S, D]`` tensors; ``len_q`` / ``len_kv`` (int
        sequences or tensors of length B) give valid lengths, default S."""
        lq = torch.full((B,), Sq, dtype=torch.int32) if len_q is None else torch.as_tensor(len_q, dtype=torch.int32).clone()
        lk = torch.full((B,), Skv, dtype=torch.int32) if len_kv is None else torch.as_tensor(len_kv, dtype=torch.int32).clone()
        return Problem(B, Hq, Hkv, D, lq, lk,
                       torch.arange(B, dtype=torch.int64) * (Hq * Sq),
                       torch.arange(B, dtype=torch.int64) * (Hkv * Skv),
                       Sq * D, D, Skv * D, D, Sq, causal, bottom_right, window_left,
                       (D ** -0.5) if scale is None else float(scale), has_sink,
                       q_numel=B * Hq * Sq * D, kv_numel=B * Hkv * Skv * D, window_right=window_right)

    @staticmethod
    def packed(Hq, Hkv, D, cu_q, cu_kv, len_q, len_kv, total_q, total_kv, *, causal=True,
               bottom_right=False, window_left=-1, window_right=0, scale=None,
               has_sink=False) -> "Problem":
        """Contiguous ``[T, H, D]`` tensors; sequence b starts at row
        ``cu_q[b]`` and has ``len_q[b]`` valid rows (similarly for kv)."""
        cu_q = torch.as_tensor(cu_q, dtype=torch.int64)
        cu_kv = torch.as_tensor(cu_kv, dtype=torch.int64)
        B = int(cu_q.numel()) - 1
        lq = torch.as_tensor(len_q, dtype=torch.int32).clone()
        lk = torch.as_tensor(len_kv, dtype=torch.int32).clone()
        stat_ld = int(lq.max()) if B else 1
        return Problem(B, Hq, Hkv, D, lq, lk, cu_q[:B].clone(), cu_kv[:B].clone(),
                       D, Hq * D, D, Hkv * D, max(stat_ld, 1), causal, bottom_right,
                       window_left, (D ** -0.5) if scale is None else float(scale), has_sink,
                       q_numel=int(total_q) * Hq * D, kv_numel=int(total_kv) * Hkv * D,
                       window_right=window_right)

    @staticmethod
    def for_workload(w) -> "Problem":
        """The problem of a synthetic workload description: any object with
        the fields of ``sliding_window_attention_flash_amd.synth.Workload``
        (batch, heads, head_dim, lengths, mask, scale, sink, layout and the
        packed slot capacities)."""
        kw = dict(causal=w.causal, bottom_right=w.bottom_right, window_left=w.window_left,
                  window_right=w.window_right, scale=w.softmax_scale, has_sink=w.sink)
        if w.layout == "thd":
            cu_q, cu_kv = [0], [0]
            for c in w.cap_q:
                cu_q.append(cu_q[-1] + c)
            for c in w.cap_kv:
                cu_kv.append(cu_kv[-1] + c)
            return Problem.packed(w.heads_q, w.heads_kv, w.head_dim, cu_q, cu_kv, w.valid_len_q(),
                                  w.valid_len_kv(), w.total_q, w.total_kv, **kw)
        return Problem.dense(w.batch, w.heads_q, w.heads_kv, w.seq_q, w.seq_kv, w.head_dim,
                             len_q=w.valid_len_q(), len_kv=w.valid_len_kv(), **kw)

    def _c(self, dtype_code: int) -> _Problem:
        self._keep = [self.len_q.contiguous(), self.len_kv.contiguous(),
                      self.row0_q.contiguous(), self.row0_kv.contiguous()]
        lq, lk, rq, rk = self._keep
        return _Problem(dtype_code, self.batch, self.heads_q, self.heads_kv, self.head_dim,
                        int(self.causal), int(self.bottom_right), int(self.window_left),
                        int(self.window_right), int(self.dense_scan), int(self.has_sink), float(self.scale),
                        lq.data_ptr(), lk.data_ptr(), rq.data_ptr(), rk.data_ptr(),
                        self.q_stride_h, self.q_stride_r, self.kv_stride_h, self.kv_stride_r,
                        self.stat_ld)


def _prep(t: torch.Tensor) -> torch.Tensor:
    if t.device.type != "cpu":
        raise ValueError("oracle inputs must be CPU tensors")
    if t.dtype not in _DT:
        raise ValueError(f"oracle input dtype {t.dtype} not supported")
    return t.contiguous()


def _common(q, k, v, dO=None):
    ts = [_prep(t) for t in (q, k, v) + ((dO,) if dO is not None else ())]
    dt = {t.dtype for t in ts}
    if len(dt) != 1:
        raise ValueError("q, k, v, dO must share one dtype")
    return ts, _DT[ts[0].dtype]


def _sink(p: Problem, sink):
    if not p.has_sink:
        return None
    if sink is None:
        raise ValueError("problem has a sink but no sink tensor given")
    if sink.device.type != "cpu":
        raise ValueError("oracle inputs must be CPU tensors")
    return sink.to(torch.float64).contiguous()


def forward(p: Problem, q, k, v, sink=None, lib=None):
    """Returns (O fp64 shaped like q, LSE fp64 [B, Hq, stat_ld])."""
    lib = lib or load()
    (q, k, v), dt = _common(q, k, v)
    sk = _sink(p, sink)
    o = torch.zeros(q.shape, dtype=torch.float64)
    lse = torch.full((p.batch, p.heads_q, p.stat_ld), float("-inf"), dtype=torch.float64)
    cp = p._c(dt)
    rc = lib.oracle_forward(ctypes.byref(cp), _ptr(q), _ptr(k), _ptr(v), _ptr(sk), _ptr(o), _ptr(lse))
    if rc:
        raise RuntimeError("oracle_forward rejected the problem")
    return o, lse


def backward(p: Problem, q, k, v, dO, sink=None, lib=None):
    """Returns dict with dq, dk, dv (fp64, shaped like q / k / v), dsink
    (fp64 [Hq] or None), o, lse, delta."""
    lib = lib or load()
    (q, k, v, dO), dt = _common(q, k, v, dO)
    sk = _sink(p, sink)
    dq = torch.zeros(q.shape, dtype=torch.float64)
    dk = torch.zeros(k.shape, dtype=torch.float64)
    dv = torch.zeros(v.shape, dtype=torch.float64)
    o = torch.zeros(q.shape, dtype=torch.float64)
    lse = torch.full((p.batch, p.heads_q, p.stat_ld), float("-inf"), dtype=torch.float64)
    delta = torch.zeros((p.batch, p.heads_q, p.stat_ld), dtype=torch.float64)
    dsink = torch.zeros(p.heads_q, dtype=torch.float64) if p.has_sink else None
    cp = p._c(dt)
    rc = lib.oracle_backward(ctypes.byref(cp), _ptr(q), _ptr(k), _ptr(v), _ptr(dO), _ptr(sk),
                             _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dsink), _ptr(o), _ptr(lse),
                             _ptr(delta))
    if rc:
        raise RuntimeError("oracle_backward rejected the problem")
    return dict(dq=dq, dk=dk, dv=dv, dsink=dsink, o=o, lse=lse, delta=delta)


def dq_rows(p: Problem, q, k, v, dO, b, h, i, sink=None, lib=None) -> torch.Tensor:
    """dQ rows for samples (b[s], h[s], i[s]) -> fp64 [n, D]."""
    lib = lib or load()
    (q, k, v, dO), dt = _common(q, k, v, dO)
    sk = _sink(p, sink)
    b, h, i = (torch.as_tensor(x, dtype=torch.int32).contiguous() for x in (b, h, i))
    n = int(b.numel())
    out = torch.zeros((n, p.head_dim), dtype=torch.float64)
    cp = p._c(dt)
    rc = lib.oracle_dq_rows(ctypes.byref(cp), _ptr(q), _ptr(k), _ptr(v), _ptr(dO), _ptr(sk), n,
                            _ptr(b), _ptr(h), _ptr(i), _ptr(out))
    if rc:
        raise RuntimeError("oracle_dq_rows rejected the problem")
    return out


def dkdv_rows(p: Problem, q, k, v, dO, b, hk, j, sink=None, lib=None):
    """dK and dV rows for samples (b[s], hk[s], j[s]) -> two fp64 [n, D]."""
    lib = lib or load()
    (q, k, v, dO), dt = _common(q, k, v, dO)
    sk = _sink(p, sink)
    b, hk, j = (torch.as_tensor(x, dtype=torch.int32).contiguous() for x in (b, hk, j))
    n = int(b.numel())
    dk = torch.zeros((n, p.head_dim), dtype=torch.float64)
    dv = torch.zeros((n, p.head_dim), dtype=torch.float64)
    cp = p._c(dt)
    rc = lib.oracle_dkdv_rows(ctypes.byref(cp), _ptr(q), _ptr(k), _ptr(v), _ptr(dO), _ptr(sk), n,
                              _ptr(b), _ptr(hk), _ptr(j), _ptr(dk), _ptr(dv))
    if rc:
        raise RuntimeError("oracle_dkdv_rows rejected the problem")
    return dk, dv


def attended_pairs(p: Problem) -> int:
    """Attended (query, key) pairs for one query head, summed over sequences."""
    cp = p._c(F64)
    return int(load().oracle_attended_pairs(ctypes.byref(cp)))
