"""Python binding of the swa_sdpa C ABI (``include/swa_sdpa.h``).

The functions named like the C entry points (``sdpa_bwd_plan``,
``sdpa_bwd_run``, ...) marshal arguments and call the library; ``forward``
and ``backward`` are conveniences that describe torch tensors, allocate the
outputs and the workspace with torch, and call those entry points.  No
attention arithmetic happens in Python.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib
from ._lib import AttnDesc, BwdTensors, FwdTensors, check

_DT = {torch.bfloat16: _lib.SDPA_BF16, torch.float16: _lib.SDPA_F16}


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(int(stream.cuda_stream))


class BwdPlan:
    def __init__(self, handle: ctypes.c_void_p, ws_bytes: int, desc: AttnDesc):
        self.handle, self.workspace_bytes, self.desc = handle, ws_bytes, desc
        self._destroy = _lib.load().sdpa_bwd_plan_destroy

    def __del__(self):
        if getattr(self, "handle", None):
            self._destroy(self.handle)
            self.handle = None


class FwdPlan:
    def __init__(self, handle: ctypes.c_void_p, ws_bytes: int, desc: AttnDesc):
        self.handle, self.workspace_bytes, self.desc = handle, ws_bytes, desc
        self._destroy = _lib.load().sdpa_fwd_plan_destroy

    def __del__(self):
        if getattr(self, "handle", None):
            self._destroy(self.handle)
            self.handle = None


def sdpa_bwd_plan(desc: AttnDesc) -> BwdPlan:
    lib = _lib.load()
    h, n = ctypes.c_void_p(), ctypes.c_size_t()
    check(lib.sdpa_bwd_plan(ctypes.byref(desc), ctypes.byref(h), ctypes.byref(n)), "sdpa_bwd_plan")
    return BwdPlan(h, int(n.value), desc)


def sdpa_bwd_run(plan: BwdPlan, tensors: BwdTensors, workspace: Optional[torch.Tensor],
                 stream=None) -> None:
    ws = _p(workspace)
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    check(_lib.load().sdpa_bwd_run(plan.handle, ctypes.byref(tensors), ws, nbytes, _stream(stream)),
          "sdpa_bwd_run")


def sdpa_bwd_run_noalloc(plan: BwdPlan, tensors: BwdTensors, stream=None) -> None:
    """The backward on the library's own scratch workspace (no allocation)."""
    check(_lib.load().sdpa_bwd_run_noalloc(plan.handle, ctypes.byref(tensors), _stream(stream)),
          "sdpa_bwd_run_noalloc")


def sdpa_bwd_run_events(plan: BwdPlan, tensors: BwdTensors, workspace, stream, start_event,
                        stop_event) -> None:
    """``start_event`` / ``stop_event`` are raw hipEvent_t handles (ints)."""
    ws = _p(workspace)
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    check(_lib.load().sdpa_bwd_run_events(plan.handle, ctypes.byref(tensors), ws, nbytes,
                                          _stream(stream), ctypes.c_void_p(start_event),
                                          ctypes.c_void_p(stop_event)), "sdpa_bwd_run_events")


def sdpa_bwd_relay_expiries(plan: BwdPlan, workspace: torch.Tensor, stream=None,
                            raise_on_timeout: bool = False) -> int:
    """Relay waits of the last run that hit the watchdog (synchronizes).  The
    library returns SDPA_ERR_RELAY_TIMEOUT when the count is > 0; that raises
    here only with ``raise_on_timeout``, otherwise the count says it."""
    n = ctypes.c_int32()
    st = _lib.load().sdpa_bwd_relay_expiries(plan.handle, _p(workspace), _stream(stream), ctypes.byref(n))
    if st != _lib.SDPA_ERR_RELAY_TIMEOUT or raise_on_timeout:
        check(st, "sdpa_bwd_relay_expiries")
    return int(n.value)


def sdpa_bwd_plan_set_relay_watchdog(plan: BwdPlan, spin_limit: int, unreachable: bool) -> None:
    """Test hook: spins before a relay wait gives up, and whether every wait
    targets a turn no visitor releases (a host-forced timeout)."""
    check(_lib.load().sdpa_bwd_plan_set_relay_watchdog(plan.handle, int(spin_limit), int(bool(unreachable))),
          "sdpa_bwd_plan_set_relay_watchdog")


def sdpa_fwd_plan(desc: AttnDesc) -> FwdPlan:
    lib = _lib.load()
    h, n = ctypes.c_void_p(), ctypes.c_size_t()
    check(lib.sdpa_fwd_plan(ctypes.byref(desc), ctypes.byref(h), ctypes.byref(n)), "sdpa_fwd_plan")
    return FwdPlan(h, int(n.value), desc)


def sdpa_fwd_run(plan: FwdPlan, tensors: FwdTensors, workspace: Optional[torch.Tensor],
                 stream=None) -> None:
    ws = _p(workspace)
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    check(_lib.load().sdpa_fwd_run(plan.handle, ctypes.byref(tensors), ws, nbytes, _stream(stream)),
          "sdpa_fwd_run")


def sdpa_bwd_schedule(plan: BwdPlan, len_q: int, len_kv: int) -> dict:
    """Tile schedule of one sequence: tile sizes, per-kv-tile [q_lo, q_hi)
    and per-q-tile relay visitor range [kv_first, kv_last]."""
    lib = _lib.load()
    tq, tk, nq, nk = (ctypes.c_int32() for _ in range(4))
    check(lib.sdpa_bwd_schedule(plan.handle, len_q, len_kv, ctypes.byref(tq), ctypes.byref(tk),
                                ctypes.byref(nq), ctypes.byref(nk), 0, None, None, 0, None, None),
          "sdpa_bwd_schedule")
    nq_, nk_ = nq.value, nk.value
    qlo, qhi = (ctypes.c_int32 * max(nk_, 1))(), (ctypes.c_int32 * max(nk_, 1))()
    kf, kl = (ctypes.c_int32 * max(nq_, 1))(), (ctypes.c_int32 * max(nq_, 1))()
    check(lib.sdpa_bwd_schedule(plan.handle, len_q, len_kv, None, None, None, None, nk_, qlo, qhi,
                                nq_, kf, kl), "sdpa_bwd_schedule")
    return dict(tile_q=tq.value, tile_kv=tk.value, n_q=nq_, n_kv=nk_,
                q_lo=list(qlo)[:nk_], q_hi=list(qhi)[:nk_],
                kv_first=list(kf)[:nq_], kv_last=list(kl)[:nq_])


# ---------------------------------------------------------------------------
# conveniences on torch tensors


def _strides(t: torch.Tensor, packed: bool):
    if t is None:
        return (0, 0, 0)
    if t.stride(-1) != 1:
        raise ValueError("the head_dim axis must be contiguous")
    if packed:
        return (0, t.stride(1), t.stride(0))
    return (t.stride(0), t.stride(1), t.stride(2))


@dataclass
class Geometry:
    """Shapes and mask of a problem, inferred from the tensors."""
    layout: int
    batch: int
    heads_q: int
    heads_kv: int
    head_dim: int
    seq_q: int
    seq_kv: int
    total_q: int
    total_kv: int


def geometry(q, k, cu_seqlens_q=None, max_seqlen_q=None, max_seqlen_kv=None) -> Geometry:
    if q.dim() == 4:
        B, Hq, Sq, D = q.shape
        _, Hkv, Skv, _ = k.shape
        return Geometry(_lib.SDPA_LAYOUT_BHSD, B, Hq, Hkv, D, Sq, Skv, B * Sq, B * Skv)
    if q.dim() == 3:
        if cu_seqlens_q is None or max_seqlen_q is None or max_seqlen_kv is None:
            raise ValueError("packed [T, H, D] tensors need cu_seqlens and max_seqlen_q / max_seqlen_kv")
        T, Hq, D = q.shape
        Tk, Hkv, _ = k.shape
        return Geometry(_lib.SDPA_LAYOUT_THD, cu_seqlens_q.numel() - 1, Hq, Hkv, D,
                        int(max_seqlen_q), int(max_seqlen_kv), T, Tk)
    raise ValueError("q must be [B, H, S, D] or [T, H, D]")


def make_desc(g: Geometry, dtype, *, causal=True, bottom_right=False, window_left=-1,
              window_right=0, q_run_tiles=0, engine=0, scale=None, deterministic=False, has_sink=False,
              has_seq_lens=False, q=None, k=None, v=None, o=None, dO=None, dq=None, dk=None, dv=None) -> AttnDesc:
    if dtype not in _DT:
        raise ValueError(f"dtype {dtype} not supported (bf16 / f16)")
    packed = g.layout == _lib.SDPA_LAYOUT_THD
    d = AttnDesc()
    d.dtype, d.layout, d.batch = _DT[dtype], g.layout, g.batch
    d.heads_q, d.heads_kv, d.head_dim = g.heads_q, g.heads_kv, g.head_dim
    d.seq_q, d.seq_kv, d.total_q, d.total_kv = g.seq_q, g.seq_kv, g.total_q, g.total_kv
    d.causal, d.bottom_right, d.window_left = int(causal), int(bottom_right), int(window_left)
    d.window_right, d.q_run_tiles, d.engine = int(window_right), int(q_run_tiles), int(engine)
    d.scale = float(scale) if scale is not None else g.head_dim ** -0.5
    d.deterministic, d.has_sink, d.has_seq_lens = int(deterministic), int(has_sink), int(has_seq_lens)
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", dO), ("dq", dq), ("dk", dk), ("dv", dv)):
        getattr(d, "stride_" + name)[:] = _strides(t, packed)
    return d


def lse_shape(g: Geometry):
    if g.layout == _lib.SDPA_LAYOUT_THD:
        return (g.heads_q, g.total_q)
    return (g.batch, g.heads_q, g.seq_q)


class Forward:
    """A planned forward bound to fixed tensors (O and LSE are allocated
    here unless given)."""

    def __init__(self, q, k, v, *, causal=True, bottom_right=False, window_left=-1, window_right=0,
                 q_run_tiles=0, engine=0, scale=None, sink=None, cu_seqlens_q=None, cu_seqlens_kv=None,
                 seq_lens_q=None, seq_lens_kv=None, max_seqlen_q=None, max_seqlen_kv=None, o=None,
                 lse=None):
        g = geometry(q, k, cu_seqlens_q, max_seqlen_q, max_seqlen_kv)
        self.o = torch.empty_like(q) if o is None else o
        self.lse = torch.empty(lse_shape(g), dtype=torch.float32, device=q.device) if lse is None else lse
        desc = make_desc(g, q.dtype, causal=causal, bottom_right=bottom_right, window_left=window_left,
                         window_right=window_right, q_run_tiles=q_run_tiles, engine=engine, scale=scale,
                         has_sink=sink is not None, has_seq_lens=seq_lens_q is not None,
                         q=q, k=k, v=v, o=self.o)
        self.plan = sdpa_fwd_plan(desc)
        self._keep = (q, k, v, sink, cu_seqlens_q, cu_seqlens_kv, seq_lens_q, seq_lens_kv)
        self.tensors = FwdTensors(q=_p(q), k=_p(k), v=_p(v), sink=_p(sink), cu_seqlens_q=_p(cu_seqlens_q),
                                  cu_seqlens_kv=_p(cu_seqlens_kv), seq_lens_q=_p(seq_lens_q),
                                  seq_lens_kv=_p(seq_lens_kv), o=_p(self.o), lse=_p(self.lse))

    def run(self, stream=None):
        sdpa_fwd_run(self.plan, self.tensors, None, stream)
        return self.o, self.lse


def forward(q, k, v, *, stream=None, **kw):
    """Window-trimmed forward: returns (O like q, LSE fp32).  Keywords as
    for ``Forward``."""
    return Forward(q, k, v, **kw).run(stream)


class Backward:
    """A planned backward bound to fixed tensors (used by the benchmark and
    the tests to rerun the same launch)."""

    def __init__(self, q, k, v, o, dO, lse, *, causal=True, bottom_right=False, window_left=-1,
                 window_right=0, q_run_tiles=0, engine=0, scale=None, deterministic=False, sink=None,
                 cu_seqlens_q=None, cu_seqlens_kv=None, seq_lens_q=None, seq_lens_kv=None, max_seqlen_q=None,
                 max_seqlen_kv=None, dq=None, dk=None, dv=None, dsink=None, workspace=None):
        g = geometry(q, k, cu_seqlens_q, max_seqlen_q, max_seqlen_kv)
        self.dq = torch.empty_like(q) if dq is None else dq
        self.dk = torch.empty_like(k) if dk is None else dk
        self.dv = torch.empty_like(v) if dv is None else dv
        self.dsink = None
        if sink is not None:
            self.dsink = torch.empty(g.heads_q, dtype=torch.float32, device=q.device) if dsink is None else dsink
        desc = make_desc(g, q.dtype, causal=causal, bottom_right=bottom_right,
                         window_left=window_left, window_right=window_right,
                         q_run_tiles=q_run_tiles, engine=engine, scale=scale, deterministic=deterministic,
                         has_sink=sink is not None, has_seq_lens=seq_lens_q is not None,
                         q=q, k=k, v=v, o=o, dO=dO, dq=self.dq, dk=self.dk, dv=self.dv)
        self.plan = sdpa_bwd_plan(desc)
        nbytes = self.plan.workspace_bytes
        if workspace is None:
            workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=q.device)
        self.workspace = workspace
        self._keep = (q, k, v, o, dO, lse, sink, cu_seqlens_q, cu_seqlens_kv, seq_lens_q, seq_lens_kv)
        self.tensors = BwdTensors(q=_p(q), k=_p(k), v=_p(v), o=_p(o), dO=_p(dO), lse=_p(lse),
                                  sink=_p(sink), cu_seqlens_q=_p(cu_seqlens_q),
                                  cu_seqlens_kv=_p(cu_seqlens_kv), seq_lens_q=_p(seq_lens_q),
                                  seq_lens_kv=_p(seq_lens_kv), dq=_p(self.dq), dk=_p(self.dk),
                                  dv=_p(self.dv), dsink=_p(self.dsink))

    def run(self, stream=None):
        sdpa_bwd_run(self.plan, self.tensors, self.workspace, stream)
        return self.dq, self.dk, self.dv, self.dsink

    def relay_expiries(self, stream=None) -> int:
        return sdpa_bwd_relay_expiries(self.plan, self.workspace, stream)

    def run_events(self, start_event: int, stop_event: int, stream=None):
        sdpa_bwd_run_events(self.plan, self.tensors, self.workspace, stream, start_event, stop_event)
        return self.dq, self.dk, self.dv, self.dsink


def backward(q, k, v, o, dO, lse, **kw):
    """Window-bounded backward: returns (dQ, dK, dV, dSink or None)."""
    return Backward(q, k, v, o, dO, lse, **kw).run(kw.get("stream"))
