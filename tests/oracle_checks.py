"""Checks that pin the fp64 oracle to facts other than itself.

Each ``check_*`` function raises AssertionError on failure and takes an
optional ``lib`` (a loaded oracle library), so the same battery can be run
against deliberately broken builds of the oracle (see
``test_oracle_pins.py::test_pins_catch_planted_mistakes``).

What pins what:
* finite differences of L = sum(dO * O): the backward is the gradient of the
  forward (dQ, dK, dV, dSink);
* torch fp64 autograd on an explicit boolean mask, and torch's own
  ``scaled_dot_product_attention(is_causal=True)``: the forward softmax
  arithmetic and the causal mask;
* closed forms: window 0 keeps only the diagonal key, constant V gives zero
  dQ / dK, zero Q gives a uniform average (also over a right band);
* invariants: dS rows sum to zero (dQ unchanged by shifting every key by one
  vector; dK sums to zero over keys), window >= S equals plain causal,
  bottom-right equals the matching rows of a square top-left problem, a
  top-left right band R equals the bottom-right mask with s_kv - s_q = R,
  a right band wider than the keys equals the window-only mask, GQA
  equals the group sum of the head-expanded MHA problem, keys outside every
  window get zero dK / dV, padding and packed sequences equal independent
  dense problems.
"""
from __future__ import annotations

import math

import torch

import oracle
from oracle import Problem

F64 = torch.float64


def rnd(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=F64) * scale


def dense_case(B, Hq, Hkv, Sq, Skv, D, seed, **kw):
    p = Problem.dense(B, Hq, Hkv, Sq, Skv, D, **kw)
    q = rnd((B, Hq, Sq, D), seed)
    k = rnd((B, Hkv, Skv, D), seed + 1)
    v = rnd((B, Hkv, Skv, D), seed + 2)
    dO = rnd((B, Hq, Sq, D), seed + 3)
    sink = rnd((Hq,), seed + 4) if kw.get("has_sink") else None
    return p, q, k, v, dO, sink


def packed_case(Hq, Hkv, D, len_q, len_kv, cap_q, cap_kv, seed, **kw):
    cu_q = [0]
    for c in cap_q:
        cu_q.append(cu_q[-1] + c)
    cu_kv = [0]
    for c in cap_kv:
        cu_kv.append(cu_kv[-1] + c)
    p = Problem.packed(Hq, Hkv, D, cu_q, cu_kv, len_q, len_kv, cu_q[-1], cu_kv[-1], **kw)
    q = rnd((cu_q[-1], Hq, D), seed)
    k = rnd((cu_kv[-1], Hkv, D), seed + 1)
    v = rnd((cu_kv[-1], Hkv, D), seed + 2)
    dO = rnd((cu_q[-1], Hq, D), seed + 3)
    sink = rnd((Hq,), seed + 4) if kw.get("has_sink") else None
    return p, q, k, v, dO, sink, cu_q, cu_kv


# Small problems used by the finite-difference and torch checks.  Together
# they cover MHA / GQA / MQA, top-left / bottom-right, windows 0 / 3 / none,
# a window-only (non-causal) mask, sinks, a fully masked row, padding and a
# packed batch.
FD_CASES = [
    dict(B=2, Hq=4, Hkv=4, Sq=7, Skv=7, D=8, causal=True, bottom_right=False, window_left=3, has_sink=False),
    dict(B=2, Hq=4, Hkv=2, Sq=13, Skv=19, D=8, causal=True, bottom_right=True, window_left=3, has_sink=True),
    dict(B=1, Hq=4, Hkv=1, Sq=13, Skv=19, D=8, causal=True, bottom_right=True, window_left=-1, has_sink=False),
    dict(B=2, Hq=4, Hkv=2, Sq=13, Skv=7, D=8, causal=True, bottom_right=False, window_left=3, has_sink=True),
    dict(B=1, Hq=4, Hkv=4, Sq=7, Skv=7, D=8, causal=True, bottom_right=False, window_left=0, has_sink=False),
    dict(B=1, Hq=2, Hkv=1, Sq=7, Skv=19, D=8, causal=False, bottom_right=True, window_left=3, has_sink=True),
    dict(B=2, Hq=2, Hkv=1, Sq=9, Skv=9, D=8, causal=True, bottom_right=False, window_left=2, has_sink=False,
         len_q=[9, 5], len_kv=[9, 6]),
    # right-band widening: keys up to anchor + R
    dict(B=1, Hq=4, Hkv=2, Sq=9, Skv=13, D=8, causal=True, bottom_right=True, window_left=3, window_right=2,
         has_sink=True),
    dict(B=1, Hq=2, Hkv=2, Sq=11, Skv=8, D=8, causal=True, bottom_right=False, window_left=-1, window_right=3,
         has_sink=False),
]


def make_fd_case(c, seed):
    c = dict(c)
    B, Hq, Hkv, Sq, Skv, D = (c.pop(x) for x in ("B", "Hq", "Hkv", "Sq", "Skv", "D"))
    return dense_case(B, Hq, Hkv, Sq, Skv, D, seed, scale=0.7, **c)


PACKED_FD = dict(Hq=4, Hkv=2, D=8, len_q=[5, 8, 3], len_kv=[9, 4, 10], cap_q=[8, 8, 4],
                 cap_kv=[9, 6, 12], causal=True, bottom_right=True, window_left=3, has_sink=True)


def make_packed_fd(seed):
    c = dict(PACKED_FD)
    args = [c.pop(x) for x in ("Hq", "Hkv", "D", "len_q", "len_kv", "cap_q", "cap_kv")]
    p, q, k, v, dO, sink, _, _ = packed_case(*args, seed, scale=0.7, **c)
    return p, q, k, v, dO, sink


def _loss(p, q, k, v, dO, sink, lib):
    o, _ = oracle.forward(p, q, k, v, sink, lib=lib)
    return float((o * dO).sum())


def fd_grad(p, q, k, v, dO, sink, which, lib, h=1e-5):
    """Central differences of L = sum(dO * O) for every element of one input."""
    tensors = dict(q=q, k=k, v=v, sink=sink)
    x = tensors[which]
    g = torch.zeros_like(x)
    flat, gflat = x.view(-1), g.view(-1)
    for n in range(flat.numel()):
        old = float(flat[n])
        flat[n] = old + h
        lp = _loss(p, tensors["q"], tensors["k"], tensors["v"], dO, tensors["sink"], lib)
        flat[n] = old - h
        lm = _loss(p, tensors["q"], tensors["k"], tensors["v"], dO, tensors["sink"], lib)
        flat[n] = old
        gflat[n] = (lp - lm) / (2 * h)
    return g


def _close(a, b, tol, what):
    err = float((a - b).abs().max()) if a.numel() else 0.0
    ref = max(1.0, float(b.abs().max()) if b.numel() else 0.0)
    assert err <= tol * ref, f"{what}: max|diff| {err:.3e} > {tol:.1e} * {ref:.3g}"


def check_finite_differences(lib=None, cases=None):
    cases = cases if cases is not None else [make_fd_case(c, 11 + 7 * n) for n, c in enumerate(FD_CASES)]
    cases = list(cases) + [make_packed_fd(500)]
    for n, (p, q, k, v, dO, sink) in enumerate(cases):
        r = oracle.backward(p, q, k, v, dO, sink, lib=lib)
        for which, an in (("q", r["dq"]), ("k", r["dk"]), ("v", r["dv"])):
            _close(fd_grad(p, q, k, v, dO, sink, which, lib), an, 1e-7, f"case {n} d{which}")
        if p.has_sink:
            _close(fd_grad(p, q, k, v, dO, sink, "sink", lib), r["dsink"], 1e-7, f"case {n} dsink")


def explicit_mask(lq, lk, causal, bottom_right, window_left, window_right=0):
    i = torch.arange(lq)[:, None]
    j = torch.arange(lk)[None, :]
    a = i + (lk - lq if bottom_right else 0)
    m = torch.ones(lq, lk, dtype=torch.bool)
    if causal:
        m &= j <= a + window_right
    if window_left >= 0:
        m &= (a - j) <= window_left
    return m


def torch_reference(p: Problem, q, k, v, dO, sink, layout="dense"):
    """fp64 autograd through torch.softmax on an explicit mask; returns
    (O, dq, dk, dv, dsink) in the input layouts."""
    q = q.clone().requires_grad_(True)
    k = k.clone().requires_grad_(True)
    v = v.clone().requires_grad_(True)
    s_t = sink.clone().requires_grad_(True) if sink is not None else None
    G = p.heads_q // p.heads_kv
    outs = torch.zeros_like(q)
    loss = 0.0
    for b in range(p.batch):
        lq, lk = int(p.len_q[b]), int(p.len_kv[b])
        m = explicit_mask(lq, lk, p.causal, p.bottom_right, p.window_left, p.window_right)
        for h in range(p.heads_q):
            if layout == "dense":
                qb, kb, vb, dob = q[b, h, :lq], k[b, h // G, :lk], v[b, h // G, :lk], dO[b, h, :lq]
            else:
                r0q, r0k = int(p.row0_q[b]), int(p.row0_kv[b])
                qb, kb, vb = q[r0q:r0q + lq, h], k[r0k:r0k + lk, h // G], v[r0k:r0k + lk, h // G]
                dob = dO[r0q:r0q + lq, h]
            s = (qb @ kb.T) * p.scale
            s = s.masked_fill(~m, float("-inf"))
            if s_t is not None:
                s = torch.cat([s, s_t[h].expand(lq, 1)], dim=1)
            ok = torch.isfinite(s).any(dim=1, keepdim=True)
            s = torch.where(ok, s, torch.zeros_like(s))
            P = torch.softmax(s, dim=1) * ok
            o = P[:, :lk] @ vb
            loss = loss + (o * dob).sum()
            if layout == "dense":
                outs[b, h, :lq] = o.detach()
            else:
                outs[r0q:r0q + lq, h] = o.detach()
    loss.backward()
    return (outs, q.grad, k.grad, v.grad, s_t.grad if s_t is not None else None)


def check_torch_autograd(lib=None):
    cases = [make_fd_case(c, 101 + 3 * n) for n, c in enumerate(FD_CASES)]
    cases.append(dense_case(2, 4, 2, 37, 53, 16, 900, scale=0.3, causal=True, bottom_right=True,
                            window_left=11, has_sink=True))
    cases.append(dense_case(1, 2, 2, 64, 64, 16, 901, scale=0.25, causal=True, window_left=1))
    for n, (p, q, k, v, dO, sink) in enumerate(cases):
        r = oracle.backward(p, q, k, v, dO, sink, lib=lib)
        o_t, dq_t, dk_t, dv_t, ds_t = torch_reference(p, q, k, v, dO, sink)
        _close(r["o"], o_t, 1e-12, f"torch case {n} O")
        _close(r["dq"], dq_t, 1e-12, f"torch case {n} dQ")
        _close(r["dk"], dk_t, 1e-12, f"torch case {n} dK")
        _close(r["dv"], dv_t, 1e-12, f"torch case {n} dV")
        if ds_t is not None:
            _close(r["dsink"], ds_t, 1e-12, f"torch case {n} dSink")
    p, q, k, v, dO, sink = make_packed_fd(77)
    r = oracle.backward(p, q, k, v, dO, sink, lib=lib)
    o_t, dq_t, dk_t, dv_t, ds_t = torch_reference(p, q, k, v, dO, sink, layout="packed")
    for name, a, b in (("O", r["o"], o_t), ("dQ", r["dq"], dq_t), ("dK", r["dk"], dk_t),
                       ("dV", r["dv"], dv_t), ("dSink", r["dsink"], ds_t)):
        _close(a, b, 1e-12, f"torch packed {name}")


def check_torch_sdpa_causal(lib=None):
    """torch's own causal SDPA (top-left, no window) -- an independent mask."""
    p, q, k, v, dO, _ = dense_case(2, 3, 3, 29, 29, 16, 321, scale=0.4, causal=True, window_left=-1)
    qq, kk, vv = (t.clone().requires_grad_(True) for t in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, is_causal=True, scale=0.4)
    (o * dO).sum().backward()
    r = oracle.backward(p, q, k, v, dO, None, lib=lib)
    _close(r["o"], o.detach(), 1e-12, "sdpa O")
    _close(r["dq"], qq.grad, 1e-12, "sdpa dQ")
    _close(r["dk"], kk.grad, 1e-12, "sdpa dK")
    _close(r["dv"], vv.grad, 1e-12, "sdpa dV")
    # a window at least as long as the sequence is plain causal
    pw = Problem.dense(2, 3, 3, 29, 29, 16, scale=0.4, causal=True, window_left=29)
    rw = oracle.backward(pw, q, k, v, dO, None, lib=lib)
    for key in ("o", "dq", "dk", "dv"):
        assert torch.equal(rw[key], r[key]), f"window >= S differs from causal in {key}"
    # a right band reaching past every key is the window-only (non-causal) mask
    for wl in (-1, 5):
        pn = Problem.dense(2, 3, 3, 29, 29, 16, scale=0.4, causal=False, window_left=wl)
        pr = Problem.dense(2, 3, 3, 29, 29, 16, scale=0.4, causal=True, window_left=wl, window_right=28)
        rn = oracle.backward(pn, q, k, v, dO, None, lib=lib)
        rr = oracle.backward(pr, q, k, v, dO, None, lib=lib)
        for key in ("o", "dq", "dk", "dv"):
            assert torch.equal(rr[key], rn[key]), f"right band >= S differs from window-only in {key}"
        if wl < 0:  # no window, no causal bound: torch's unmasked SDPA
            qq, kk, vv = (t.clone().requires_grad_(True) for t in (q, k, v))
            o = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, scale=0.4)
            (o * dO).sum().backward()
            _close(rr["o"], o.detach(), 1e-12, "unmasked sdpa O")
            _close(rr["dq"], qq.grad, 1e-12, "unmasked sdpa dQ")
            _close(rr["dk"], kk.grad, 1e-12, "unmasked sdpa dK")


def check_closed_forms(lib=None):
    # window 0 (inclusive): only the anchor key is visible, P = 1.
    for br in (False, True):
        p, q, k, v, dO, _ = dense_case(2, 2, 1, 9, 12, 8, 41, scale=0.5, causal=True,
                                       bottom_right=br, window_left=0)
        r = oracle.backward(p, q, k, v, dO, None, lib=lib)
        diag = 12 - 9 if br else 0
        exp_o = torch.zeros_like(q)
        exp_dv = torch.zeros_like(v)
        for b in range(2):
            for h in range(2):
                for i in range(9):
                    a = i + diag
                    if a < 12:
                        exp_o[b, h, i] = v[b, 0, a]
                        exp_dv[b, 0, a] += dO[b, h, i]
        _close(r["o"], exp_o, 1e-14, f"W=0 O (br={br})")
        _close(r["dv"], exp_dv, 1e-14, f"W=0 dV (br={br})")
        assert float(r["dq"].abs().max()) < 1e-14 and float(r["dk"].abs().max()) < 1e-14, "W=0 dQ/dK"
    # every V row equal, no sink: O = that row, dS = 0 so dQ = dK = 0.
    p, q, k, v, dO, _ = dense_case(1, 2, 2, 11, 11, 8, 42, scale=0.5, causal=True, window_left=4)
    v = v[:, :, :1].expand_as(v).contiguous()
    r = oracle.backward(p, q, k, v, dO, None, lib=lib)
    _close(r["o"], v[:, :, :1].expand(1, 2, 11, 8), 1e-13, "constant V: O")
    assert float(r["dq"].abs().max()) < 1e-12 and float(r["dk"].abs().max()) < 1e-12, "constant V: dQ/dK"
    # Q = 0, no sink: uniform weights over the visible keys.
    p, q, k, v, dO, _ = dense_case(1, 1, 1, 10, 10, 8, 43, scale=0.5, causal=True, window_left=3)
    q = torch.zeros_like(q)
    o, lse = oracle.forward(p, q, k, v, None, lib=lib)
    for i in range(10):
        lo = max(0, i - 3)
        _close(o[0, 0, i], v[0, 0, lo:i + 1].mean(0), 1e-14, f"Q=0 row {i}")
        assert abs(float(lse[0, 0, i]) - math.log(i + 1 - lo)) < 1e-14, f"Q=0 LSE row {i}"
    # Q = 0 with a right band R and left window W: row i averages keys
    # [i - W, i + R] clipped to the sequence (R + W + 1 keys inside it).
    for W, R in ((0, 2), (1, 3)):
        p, q, k, v, dO, _ = dense_case(1, 1, 1, 10, 12, 8, 44, scale=0.5, causal=True, window_left=W,
                                       window_right=R)
        q = torch.zeros_like(q)
        o, lse = oracle.forward(p, q, k, v, None, lib=lib)
        for i in range(10):
            lo, hi = max(0, i - W), min(11, i + R)
            _close(o[0, 0, i], v[0, 0, lo:hi + 1].mean(0), 1e-14, f"Q=0 band W={W} R={R} row {i}")
            assert abs(float(lse[0, 0, i]) - math.log(hi + 1 - lo)) < 1e-14, f"Q=0 band LSE row {i}"


def check_invariants(lib=None):
    # dS rows sum to 0 (no sink): shifting every key by one vector leaves
    # O and dQ unchanged, and dK sums to zero over the keys of each kv head.
    p, q, k, v, dO, _ = dense_case(2, 4, 2, 15, 15, 8, 51, scale=0.6, causal=True, window_left=5)
    r = oracle.backward(p, q, k, v, dO, None, lib=lib)
    c = rnd((1, 1, 1, 8), 52)
    r2 = oracle.backward(p, q, k + c, v, dO, None, lib=lib)
    _close(r2["o"], r["o"], 1e-12, "key shift: O")
    _close(r2["dq"], r["dq"], 1e-12, "key shift: dQ")
    _close(r["dk"].sum(dim=2), torch.zeros(2, 2, 8, dtype=F64), 1e-12, "sum_j dK_j")
    # with a sink: row sums of dS equal exp(sink - LSE) * delta, the negated
    # per-row dSink term.
    p, q, k, v, dO, sink = dense_case(2, 4, 2, 15, 15, 8, 53, scale=0.6, causal=True,
                                      window_left=5, has_sink=True)
    r = oracle.backward(p, q, k, v, dO, sink, lib=lib)
    t = torch.exp(sink.view(1, 4, 1) - r["lse"]) * r["delta"]  # [B, Hq, S]
    assert abs(float(r["dsink"].sum() + t.sum())) < 1e-12 * max(1.0, float(t.abs().sum()))
    _close(r["dsink"], -t.sum(dim=(0, 2)), 1e-12, "dSink from row terms")
    want = p.scale * (q * t[..., None]).view(2, 2, 2, 15, 8).sum(dim=(2, 3))
    _close(r["dk"].sum(dim=2), want, 1e-12, "sum_j dK_j with sink")
    # GQA equals the group sum of the head-expanded MHA problem.
    p, q, k, v, dO, sink = dense_case(2, 6, 2, 14, 17, 8, 54, scale=0.6, causal=True,
                                      bottom_right=True, window_left=4, has_sink=True)
    r = oracle.backward(p, q, k, v, dO, sink, lib=lib)
    ke, ve = k.repeat_interleave(3, dim=1), v.repeat_interleave(3, dim=1)
    pm = Problem.dense(2, 6, 6, 14, 17, 8, scale=0.6, causal=True, bottom_right=True,
                       window_left=4, has_sink=True)
    rm = oracle.backward(pm, q, ke, ve, dO, sink, lib=lib)
    _close(r["dq"], rm["dq"], 1e-13, "GQA dQ vs expanded")
    _close(r["dk"], rm["dk"].view(2, 2, 3, 17, 8).sum(2), 1e-13, "GQA dK vs group sum")
    _close(r["dv"], rm["dv"].view(2, 2, 3, 17, 8).sum(2), 1e-13, "GQA dV vs group sum")
    _close(r["dsink"], rm["dsink"], 1e-13, "GQA dSink")
    # bottom-right rows equal the last rows of a square top-left problem
    # over the same keys (anchor shift by s_kv - s_q).
    p, q, k, v, dO, _ = dense_case(1, 2, 2, 6, 15, 8, 55, scale=0.6, causal=True,
                                   bottom_right=True, window_left=4)
    ro, lse = oracle.forward(p, q, k, v, None, lib=lib)
    pt = Problem.dense(1, 2, 2, 15, 15, 8, scale=0.6, causal=True, window_left=4)
    qt = torch.zeros(1, 2, 15, 8, dtype=F64)
    qt[:, :, 9:] = q
    ot, lset = oracle.forward(pt, qt, k, v, None, lib=lib)
    _close(ro, ot[:, :, 9:], 1e-14, "BR vs shifted TL: O")
    _close(lse, lset[:, :, 9:], 1e-14, "BR vs shifted TL: LSE")
    # a top-left right band R is the bottom-right mask of a problem with
    # s_kv - s_q = R (anchor i + R), its left window moved by R as well.
    p, q, k, v, dO, sink = dense_case(2, 4, 2, 9, 14, 8, 59, scale=0.6, causal=True, window_left=2,
                                      window_right=5, has_sink=True)
    r = oracle.backward(p, q, k, v, dO, sink, lib=lib)
    pb = Problem.dense(2, 4, 2, 9, 14, 8, scale=0.6, causal=True, bottom_right=True, window_left=7,
                       has_sink=True)
    rb = oracle.backward(pb, q, k, v, dO, sink, lib=lib)
    for key in ("o", "lse", "dq", "dk", "dv", "dsink"):
        _close(r[key], rb[key], 1e-14, f"TL right band vs BR: {key}")
    # keys outside every window (BR, s_q < s_kv - W): exact zero dK / dV.
    p, q, k, v, dO, _ = dense_case(1, 2, 1, 5, 20, 8, 56, scale=0.6, causal=True,
                                   bottom_right=True, window_left=3)
    r = oracle.backward(p, q, k, v, dO, None, lib=lib)
    first = 20 - 5 - 3  # smallest key any row sees
    assert torch.count_nonzero(r["dk"][:, :, :first]) == 0 and torch.count_nonzero(r["dv"][:, :, :first]) == 0
    assert torch.count_nonzero(r["dv"][:, :, first:]) > 0
    # padding: valid rows equal the unpadded problem; padded rows are zero.
    p, q, k, v, dO, _ = dense_case(2, 2, 2, 12, 12, 8, 57, scale=0.6, causal=True,
                                   window_left=3, len_q=[12, 7], len_kv=[12, 9])
    r = oracle.backward(p, q, k, v, dO, None, lib=lib)
    ps = Problem.dense(1, 2, 2, 7, 9, 8, scale=0.6, causal=True, window_left=3)
    rs = oracle.backward(ps, q[1:, :, :7].contiguous(), k[1:, :, :9].contiguous(),
                         v[1:, :, :9].contiguous(), dO[1:, :, :7].contiguous(), None, lib=lib)
    _close(r["dq"][1:, :, :7], rs["dq"], 0, "padded dQ")
    _close(r["dk"][1:, :, :9], rs["dk"], 0, "padded dK")
    assert torch.count_nonzero(r["dq"][1, :, 7:]) == 0 and torch.count_nonzero(r["dk"][1, :, 9:]) == 0
    # packed sequences equal independent dense problems.
    p, q, k, v, dO, sink, cu_q, cu_kv = packed_case(
        4, 2, 8, [5, 8, 3], [9, 4, 10], [8, 8, 4], [9, 6, 12], 58, scale=0.6, causal=True,
        bottom_right=True, window_left=3, has_sink=True)
    r = oracle.backward(p, q, k, v, dO, sink, lib=lib)
    dsink = torch.zeros(4, dtype=F64)
    for b, (lq, lk) in enumerate(zip([5, 8, 3], [9, 4, 10])):
        pd = Problem.dense(1, 4, 2, lq, lk, 8, scale=0.6, causal=True, bottom_right=True,
                           window_left=3, has_sink=True)
        sl = lambda t, c, L: t[c[b]:c[b] + L].permute(1, 0, 2).unsqueeze(0).contiguous()
        rd = oracle.backward(pd, sl(q, cu_q, lq), sl(k, cu_kv, lk), sl(v, cu_kv, lk),
                             sl(dO, cu_q, lq), sink, lib=lib)
        _close(sl(r["dq"], cu_q, lq), rd["dq"], 1e-15, f"packed seq {b} dQ")
        _close(sl(r["dk"], cu_kv, lk), rd["dk"], 1e-15, f"packed seq {b} dK")
        _close(sl(r["dv"], cu_kv, lk), rd["dv"], 1e-15, f"packed seq {b} dV")
        dsink += rd["dsink"]
        assert torch.count_nonzero(r["dq"][cu_q[b] + lq:cu_q[b + 1]]) == 0
        assert torch.count_nonzero(r["dk"][cu_kv[b] + lk:cu_kv[b + 1]]) == 0
    _close(r["dsink"], dsink, 1e-13, "packed dSink")


def check_dense_scan(lib=None):
    """The key-interval loops visit exactly the keys the mask keeps."""
    for n, c in enumerate(FD_CASES):
        p, q, k, v, dO, sink = make_fd_case(c, 200 + n)
        r = oracle.backward(p, q, k, v, dO, sink, lib=lib)
        p.dense_scan = True
        rd = oracle.backward(p, q, k, v, dO, sink, lib=lib)
        for key in ("o", "lse", "dq", "dk", "dv"):
            assert torch.equal(r[key], rd[key]), f"dense scan differs in {key} (case {n})"


def check_sampled_rows(lib=None):
    """Row-at-a-time gradients equal the full backward."""
    p, q, k, v, dO, sink = dense_case(2, 4, 2, 21, 26, 8, 61, scale=0.6, causal=True,
                                      bottom_right=True, window_left=6, has_sink=True)
    r = oracle.backward(p, q, k, v, dO, sink, lib=lib)
    bs, hs, is_ = [0, 1, 1, 0], [0, 3, 2, 1], [0, 20, 7, 13]
    dq = oracle.dq_rows(p, q, k, v, dO, bs, hs, is_, sink, lib=lib)
    for s in range(4):
        _close(dq[s], r["dq"][bs[s], hs[s], is_[s]], 1e-14, "dq row")
    bk, hk, js = [0, 1, 1, 0], [0, 1, 0, 1], [0, 25, 11, 4]
    dk, dv = oracle.dkdv_rows(p, q, k, v, dO, bk, hk, js, sink, lib=lib)
    for s in range(4):
        _close(dk[s], r["dk"][bk[s], hk[s], js[s]], 1e-14, "dk row")
        _close(dv[s], r["dv"][bk[s], hk[s], js[s]], 1e-14, "dv row")


def finite_bit_patterns(dtype):
    """Every finite value of a 16-bit float type, as a 1-D tensor of that
    type: all 65536 bit patterns except the all-ones exponent (inf / NaN).
    Covers both zeros, every subnormal and the largest finite values."""
    bits = torch.arange(1 << 16, dtype=torch.int32)
    exp_mask = 0x7F80 if dtype == torch.bfloat16 else 0x7C00
    keep = (bits & exp_mask) != exp_mask
    return bits[keep].to(torch.int16).view(dtype)


def _as_rows(vals, D, fill=0.0):
    """Pads a 1-D tensor to a multiple of D and shapes it [1, 1, rows, D]."""
    n = -(-vals.numel() // D)
    out = torch.full((n * D,), fill, dtype=vals.dtype)
    out[:vals.numel()] = vals
    return out.view(1, 1, n, D)


def check_widening(lib=None):
    """The oracle's exact widening of bf16 / f16 storage to fp64, pinned to
    torch's own conversion (an independent routine) through closed forms of
    the window-0 mask, where each row sees only its anchor key, so P = 1:
      * O_i = V_i and dV_j = dO_j exactly, with V and dO holding every finite
        bit pattern of the type (both zeros, all subnormals, the extremes);
      * LSE_i = scale * <Q_i, K_i> = Q_i0 when K_i = e_0 and scale = 1, and
        K_i0 when Q_i = e_0: every finite pattern through Q and through K.
    Then the problems of the torch cross-check, stored as 16-bit values, give
    bitwise the results of the same values stored as fp64."""
    for dt in (torch.bfloat16, torch.float16):
        pat = finite_bit_patterns(dt)
        v = _as_rows(pat, 8)
        dO = _as_rows(pat.flip(0), 8)
        n = v.shape[2]
        p = Problem.dense(1, 1, 1, n, n, 8, causal=True, window_left=0, scale=1.0)
        zero = torch.zeros_like(v)
        r = oracle.backward(p, zero, zero, v, dO, None, lib=lib)
        assert torch.equal(r["o"], v.to(F64)), f"{dt}: O != V widened by torch"
        assert torch.equal(r["dv"], dO.to(F64)), f"{dt}: dV != dO widened by torch"
        # every pattern in column 0 of Q (then of K), the other operand e_0
        col = torch.zeros(pat.numel(), 8, dtype=dt)
        col[:, 0] = pat
        e0 = torch.zeros(pat.numel(), 8, dtype=dt)
        e0[:, 0] = 1.0
        col, e0 = col.view(1, 1, -1, 8), e0.view(1, 1, -1, 8)
        m = col.shape[2]
        pm = Problem.dense(1, 1, 1, m, m, 8, causal=True, window_left=0, scale=1.0)
        want = pat.to(F64).view(1, 1, m)
        for name, qq, kk in (("Q", col, e0), ("K", e0, col)):
            _, lse = oracle.forward(pm, qq, kk, e0, None, lib=lib)
            assert torch.equal(lse, want), f"{dt}: LSE != {name} widened by torch"
    # 16-bit storage against fp64 storage of the same values: bitwise equal
    for n, c in enumerate(FD_CASES[:4]):
        p, q, k, v, dO, sink = make_fd_case(c, 300 + n)
        for dt in (torch.bfloat16, torch.float16):
            q16, k16, v16, dO16 = (t.to(dt) for t in (q, k, v, dO))
            r16 = oracle.backward(p, q16, k16, v16, dO16, sink, lib=lib)
            r64 = oracle.backward(p, *(t.to(F64) for t in (q16, k16, v16, dO16)), sink, lib=lib)
            for key in ("o", "lse", "dq", "dk", "dv"):
                assert torch.equal(r16[key], r64[key]), f"{dt} storage differs from fp64 in {key} (case {n})"


ALL_CHECKS = [check_finite_differences, check_torch_autograd, check_torch_sdpa_causal,
              check_closed_forms, check_invariants, check_dense_scan, check_sampled_rows,
              check_widening]
