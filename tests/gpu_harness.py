"""Helpers for GPU parity tests: run the HIP path on a workload, build the
matching oracle problem, and compare with the tolerance of the target:
per gradient, relative Frobenius error <= 1e-2 and max-abs error
<= 3e-2 * max|ref| over the valid rows; padding rows must be exactly zero
and nothing may be NaN.
"""
from __future__ import annotations

import sys
import time

import torch

import oracle
from sliding_window_attention_flash_amd import api
from sliding_window_attention_flash_amd.synth import Workload, make_inputs

REL_FRO = 1e-2
MAX_ABS = 3e-2


def say(msg: str) -> None:
    sys.stdout.write(f"[{time.strftime('%H:%M:%S')}] {msg}\n")
    sys.stdout.flush()


def mask_kw(w: Workload) -> dict:
    return dict(causal=w.causal, bottom_right=w.bottom_right, window_left=w.window_left,
                window_right=w.window_right, scale=w.softmax_scale)


def seq_kw(w: Workload, inp: dict) -> dict:
    kw = dict(cu_seqlens_q=inp["cu_seqlens_q"], cu_seqlens_kv=inp["cu_seqlens_kv"],
              seq_lens_q=inp["seq_lens_q"], seq_lens_kv=inp["seq_lens_kv"])
    if w.layout == "thd":
        kw.update(max_seqlen_q=w.seq_q, max_seqlen_kv=w.seq_kv)
    return kw


def gpu_forward(w: Workload, inp: dict):
    return api.forward(inp["q"], inp["k"], inp["v"], sink=inp["sink"], **mask_kw(w), **seq_kw(w, inp))


def stream_eligible(w: Workload) -> bool:
    """Shapes the streaming kernel applies to (its engines 1 and 2)."""
    return (w.heads_q == w.heads_kv and w.causal and w.window_right == 0 and 0 <= w.window_left <= 128
            and w.head_dim == 64)


def stream_engine(w: Workload, det: int) -> int:
    """The engine that runs the streaming kernel in dQ mode ``det`` (fp32
    atomics, chunk relay; the per-kv-tile relay for 2) where it applies,
    else 0 (the plan's choice): small shapes would otherwise take the
    per-tile kernels by the measured table."""
    if not stream_eligible(w):
        return 0
    return {0: 1, 1: 2, 2: 4}[int(det)]


def gpu_backward(w: Workload, inp: dict, o, lse, deterministic=None, nan_fill=True, engine=None):
    det = w.deterministic if deterministic is None else deterministic
    engine = w.engine if engine is None else engine
    q, k, v = inp["q"], inp["k"], inp["v"]
    fill = float("nan") if nan_fill else 0.0
    dq, dk, dv = (torch.full_like(t, fill) for t in (q, k, v))
    dsink = None
    if inp["sink"] is not None:
        dsink = torch.full((w.heads_q,), fill, dtype=torch.float32, device=q.device)
    bw = api.Backward(q, k, v, o, inp["dO"], lse, deterministic=det, sink=inp["sink"], engine=engine,
                      dq=dq, dk=dk, dv=dv, dsink=dsink, **mask_kw(w), **seq_kw(w, inp))
    return bw


def oracle_problem(w: Workload) -> oracle.Problem:
    return oracle.Problem.for_workload(w)


def row_masks(w: Workload, device="cpu"):
    """Boolean masks of valid rows and of padding rows, broadcastable to the
    q-side and kv-side tensors."""
    lq, lk = w.valid_len_q(), w.valid_len_kv()
    if w.layout == "thd":
        vq = torch.zeros(w.total_q, dtype=torch.bool)
        vk = torch.zeros(w.total_kv, dtype=torch.bool)
        pq = torch.zeros_like(vq)
        pk = torch.zeros_like(vk)
        r = 0
        for b in range(w.batch):
            vq[r:r + lq[b]] = True
            pq[r + lq[b]:r + w.cap_q[b]] = True
            r += w.cap_q[b]
        r = 0
        for b in range(w.batch):
            vk[r:r + lk[b]] = True
            pk[r + lk[b]:r + w.cap_kv[b]] = True
            r += w.cap_kv[b]
        return vq.view(-1, 1, 1), pq.view(-1, 1, 1), vk.view(-1, 1, 1), pk.view(-1, 1, 1)
    ar_q, ar_k = torch.arange(w.seq_q), torch.arange(w.seq_kv)
    vq = torch.stack([ar_q < n for n in lq]).view(w.batch, 1, w.seq_q, 1)
    vk = torch.stack([ar_k < n for n in lk]).view(w.batch, 1, w.seq_kv, 1)
    return vq, ~vq, vk, ~vk


def errors(gpu: torch.Tensor, ref: torch.Tensor):
    g, r = gpu.double().reshape(-1), ref.double().reshape(-1)
    diff = (g - r)
    rn = float(r.norm())
    rmax = float(r.abs().max()) if r.numel() else 0.0
    rel = float(diff.norm()) / rn if rn > 0 else float(g.abs().max() if g.numel() else 0.0)
    mab = float(diff.abs().max()) / rmax if rmax > 0 else float(g.abs().max() if g.numel() else 0.0)
    return rel, mab


def assert_close(name: str, gpu: torch.Tensor, ref: torch.Tensor, rel_tol=REL_FRO, max_tol=MAX_ABS):
    assert not torch.isnan(gpu).any(), f"{name}: NaN in the GPU result (unwritten element?)"
    rel, mab = errors(gpu, ref)
    say(f"    {name:6s} rel_fro={rel:.2e} max_abs/max|ref|={mab:.2e}")
    assert rel <= rel_tol, f"{name}: relative Frobenius error {rel:.3e} > {rel_tol}"
    assert mab <= max_tol, f"{name}: max-abs error {mab:.3e} > {max_tol} * max|ref|"


def oracle_full(w: Workload, inp_cpu: dict) -> dict:
    """The full fp64 oracle backward (with its forward) on the inputs."""
    p = oracle_problem(w)
    t0 = time.time()
    ref = oracle.backward(p, inp_cpu["q"], inp_cpu["k"], inp_cpu["v"], inp_cpu["dO"],
                          inp_cpu["sink"])
    say(f"    oracle backward {time.time() - t0:.1f}s ({oracle.num_threads()} threads)")
    return ref


def compare_full(w: Workload, inp_cpu: dict, gpu: dict, check_fwd=True, ref=None):
    """Element-by-element comparison against the full fp64 oracle (computed
    here unless ``ref``, an earlier oracle_full result on the same inputs,
    is given)."""
    if ref is None:
        ref = oracle_full(w, inp_cpu)
    vq, pq, vk, pk = row_masks(w)
    if check_fwd:
        o = gpu["o"].cpu()
        assert_close("O", torch.where(vq, o.double(), 0), torch.where(vq, ref["o"], 0))
        lse_g = gpu["lse"].cpu().double()
        lse_r = _lse_to_gpu_layout(w, ref["lse"])
        valid = torch.isfinite(lse_r)
        assert torch.equal(torch.isfinite(lse_g), valid), "LSE: -inf pattern differs"
        err = float((lse_g[valid] - lse_r[valid]).abs().max()) if valid.any() else 0.0
        say(f"    LSE    max_abs={err:.2e}")
        assert err <= 1e-3, f"LSE max-abs error {err}"
        if pq.any():
            assert torch.count_nonzero(torch.where(pq, o, 0)) == 0, "O padding rows not zero"
    for name, g, r, valid, pad in (("dQ", gpu["dq"], ref["dq"], vq, pq),
                                   ("dK", gpu["dk"], ref["dk"], vk, pk),
                                   ("dV", gpu["dv"], ref["dv"], vk, pk)):
        g = g.cpu()
        assert not torch.isnan(g).any(), f"{name}: NaN (unwritten element?)"
        assert_close(name, torch.where(valid, g.double(), 0), torch.where(valid, r, 0))
        if pad.any():
            assert torch.count_nonzero(torch.where(pad, g, 0)) == 0, f"{name}: padding rows not zero"
    if w.sink:
        assert_close("dSink", gpu["dsink"].cpu(), ref["dsink"])
    return ref


def _lse_to_gpu_layout(w: Workload, lse_ref: torch.Tensor) -> torch.Tensor:
    """Oracle LSE [B, Hq, stat_ld] -> the library's LSE layout."""
    if w.layout == "thd":
        out = torch.full((w.heads_q, w.total_q), float("-inf"), dtype=torch.float64)
        r = 0
        for b in range(w.batch):
            n = w.valid_len_q()[b]
            out[:, r:r + n] = lse_ref[b, :, :n]
            r += w.cap_q[b]
        return out
    out = torch.full((w.batch, w.heads_q, w.seq_q), float("-inf"), dtype=torch.float64)
    for b in range(w.batch):
        n = w.valid_len_q()[b]
        out[b, :, :n] = lse_ref[b, :, :n]
    return out


def batch_entries(w: Workload, inp_cpu: dict, gpu: dict, idx):
    """A dense workload restricted to the batch entries ``idx``: the
    workload, its CPU inputs and its GPU outputs (so the full oracle can
    check whole entries of a workload too large to check at once)."""
    assert w.layout == "bhsd"
    sel = torch.tensor(idx)
    pads = {}
    if w.pad_len_q:
        pads["pad_len_q"] = tuple(w.pad_len_q[i] for i in idx)
    if w.pad_len_kv:
        pads["pad_len_kv"] = tuple(w.pad_len_kv[i] for i in idx)
    ws = w.with_(name=f"{w.name}_b{'_'.join(map(str, idx))}", batch=len(idx), **pads)
    inp = {k: (v[sel] if isinstance(v, torch.Tensor) and k in ("q", "k", "v", "dO") else v)
           for k, v in inp_cpu.items()}
    gsel = sel.to(gpu["dq"].device)
    out = {k: (v[gsel] if isinstance(v, torch.Tensor) and k in ("o", "lse", "dq", "dk", "dv") else v)
           for k, v in gpu.items()}
    return ws, inp, out


def run_gpu(w: Workload, seed=0, deterministic=None, runs=1, engine=None):
    """Inputs on the GPU, forward, then the backward (engine: the workload's
    unless given; 0 is the plan's choice); returns CPU copies of the inputs
    and the GPU outputs (a list when runs > 1)."""
    inp = make_inputs(w, device="cuda", seed=seed)
    o, lse = gpu_forward(w, inp)
    bw = gpu_backward(w, inp, o, lse, deterministic=deterministic, engine=engine)
    outs = []
    for _ in range(runs):
        dq, dk, dv, dsink = bw.run()
        torch.cuda.synchronize()
        outs.append(dict(o=o, lse=lse, dq=dq.clone(), dk=dk.clone(), dv=dv.clone(),
                         dsink=None if dsink is None else dsink.clone(),
                         expiries=bw.relay_expiries() if (w.deterministic if deterministic is None else deterministic) else 0))
    inp_cpu = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    return inp_cpu, (outs[0] if runs == 1 else outs), inp


def sample_rows(w: Workload, n: int, seed: int, kv_side: bool):
    """(b, head, row) samples over valid rows: random ones plus the first and
    last rows of each sequence and rows at tile boundaries."""
    g = torch.Generator().manual_seed(seed)
    heads = w.heads_kv if kv_side else w.heads_q
    lens = w.valid_len_kv() if kv_side else w.valid_len_q()
    bs, hs, rs = [], [], []
    for b in range(w.batch):
        L = lens[b]
        if L == 0:
            continue
        for r in {0, L - 1, min(63, L - 1), min(64, L - 1), L // 2}:
            bs.append(b)
            hs.append(int(torch.randint(0, heads, (1,), generator=g)))
            rs.append(r)
    while len(bs) < n:
        b = int(torch.randint(0, w.batch, (1,), generator=g))
        if lens[b] == 0:
            continue
        bs.append(b)
        hs.append(int(torch.randint(0, heads, (1,), generator=g)))
        rs.append(int(torch.randint(0, lens[b], (1,), generator=g)))
    return bs, hs, rs


def gather_rows(w: Workload, t: torch.Tensor, bs, hs, rs, kv_side: bool) -> torch.Tensor:
    if w.layout == "thd":
        caps = w.cap_kv if kv_side else w.cap_q
        starts = [0]
        for c in caps:
            starts.append(starts[-1] + c)
        idx = torch.tensor([starts[b] + r for b, r in zip(bs, rs)])
        return t[idx, torch.tensor(hs)]
    return t[torch.tensor(bs), torch.tensor(hs), torch.tensor(rs)]


def compare_sampled(w: Workload, inp_cpu: dict, gpu: dict, n_q=256, n_kv=128, seed=7):
    """Sampled comparison for sizes where the full oracle is too slow: dQ
    rows and dK / dV rows computed one at a time by the oracle."""
    p = oracle_problem(w)
    bs, hs, rs = sample_rows(w, n_q, seed, kv_side=False)
    t0 = time.time()
    ref_dq = oracle.dq_rows(p, inp_cpu["q"], inp_cpu["k"], inp_cpu["v"], inp_cpu["dO"], bs, hs, rs,
                            inp_cpu["sink"])
    g_dq = gather_rows(w, gpu["dq"].cpu(), bs, hs, rs, kv_side=False)
    bk, hk, jk = sample_rows(w, n_kv, seed + 1, kv_side=True)
    ref_dk, ref_dv = oracle.dkdv_rows(p, inp_cpu["q"], inp_cpu["k"], inp_cpu["v"], inp_cpu["dO"],
                                      bk, hk, jk, inp_cpu["sink"])
    say(f"    oracle sampled rows {time.time() - t0:.1f}s ({len(bs)} dQ, {len(bk)} dK/dV rows)")
    g_dk = gather_rows(w, gpu["dk"].cpu(), bk, hk, jk, kv_side=True)
    g_dv = gather_rows(w, gpu["dv"].cpu(), bk, hk, jk, kv_side=True)
    assert_close("dQ[s]", g_dq, ref_dq)
    assert_close("dK[s]", g_dk, ref_dk)
    assert_close("dV[s]", g_dv, ref_dv)
    # properties over the whole output
    for name, t in (("dQ", gpu["dq"]), ("dK", gpu["dk"]), ("dV", gpu["dv"])):
        assert not torch.isnan(t).any(), f"{name}: NaN somewhere in the full output"
