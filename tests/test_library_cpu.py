"""Host-side checks of the HIP library (no GPU needed): exported symbols,
descriptor validation, the window-bounded tile schedule against brute force,
and a host simulation of the ordered dQ relay."""
import ctypes
import os
import re
import threading
import time

import pytest
import torch

import oracle_checks as oc
from sliding_window_attention_flash_amd import _lib, api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_library_exports_every_declared_symbol(lib):
    header = open(os.path.join(ROOT, "include", "swa_sdpa.h")).read()
    declared = set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(sdpa_\w+)\s*\(", header, re.M))
    assert {"sdpa_bwd_plan", "sdpa_bwd_run", "sdpa_fwd_plan", "sdpa_fwd_run"} <= declared
    missing = [s for s in sorted(declared) if not hasattr(lib, s)]
    assert not missing, f"declared but not exported: {missing}"
    assert set(_lib.EXPORTS) == declared


def _desc(**kw):
    g = api.Geometry(kw.pop("layout", 0), kw.pop("B", 2), kw.pop("Hq", 4), kw.pop("Hkv", 2),
                     kw.pop("D", 64), kw.pop("Sq", 300), kw.pop("Skv", 300), 600, 600)
    q = torch.empty(g.batch, g.heads_q, g.seq_q, g.head_dim, dtype=torch.bfloat16)
    k = torch.empty(g.batch, g.heads_kv, g.seq_kv, g.head_dim, dtype=torch.bfloat16)
    d = api.make_desc(g, torch.bfloat16, q=q, k=k, v=k, o=q, dO=q, dq=q, dk=k, dv=k,
                      window_left=kw.pop("window_left", 64), window_right=kw.pop("window_right", 0),
                      bottom_right=kw.pop("bottom_right", False))
    for key, val in kw.items():
        setattr(d, key, val)
    return d


@pytest.mark.parametrize("field,value,status,needle", [
    ("head_dim", 96, _lib.SDPA_ERR_UNSUPPORTED, "head_dim"),
    ("heads_q", 5, _lib.SDPA_ERR_INVALID_ARG, "multiple"),
    ("dtype", 7, _lib.SDPA_ERR_INVALID_ARG, "dtype"),
    ("window_left", -2, _lib.SDPA_ERR_INVALID_ARG, "window_left"),
    ("scale", 0.0, _lib.SDPA_ERR_INVALID_ARG, "scale"),
    ("batch", 0, _lib.SDPA_ERR_INVALID_ARG, "batch"),
    ("deterministic", 3, _lib.SDPA_ERR_INVALID_ARG, "deterministic"),
    ("window_right", -1, _lib.SDPA_ERR_INVALID_ARG, "window_right"),
    ("q_run_tiles", 17, _lib.SDPA_ERR_INVALID_ARG, "q_run_tiles"),
])
def test_plan_rejects_bad_descriptors(lib, field, value, status, needle):
    d = _desc(**{field: value})
    with pytest.raises(_lib.SdpaError) as e:
        api.sdpa_bwd_plan(d)
    assert e.value.status == status and needle in str(e.value)


def test_plan_rejects_right_band_without_causal(lib):
    d = _desc(window_right=8)
    d.causal = 0
    with pytest.raises(_lib.SdpaError, match="needs causal"):
        api.sdpa_bwd_plan(d)


def test_plan_rejects_bottom_right_with_more_queries_than_keys(lib):
    d = _desc(Sq=400, Skv=300, bottom_right=True)
    with pytest.raises(_lib.SdpaError) as e:
        api.sdpa_bwd_plan(d)
    assert e.value.status == _lib.SDPA_ERR_UNSUPPORTED


def test_plan_rejects_unaligned_strides_and_thd_without_lengths(lib):
    d = _desc()
    d.stride_q[2] = 60
    with pytest.raises(_lib.SdpaError, match="stride_q"):
        api.sdpa_bwd_plan(d)
    d = _desc(layout=1)
    d.stride_q[:] = (0, 64, 256)
    with pytest.raises(_lib.SdpaError, match="seq_lens"):
        api.sdpa_bwd_plan(d)


def test_plan_rejects_row_strides_beyond_32_bits(lib):
    d = _desc()
    d.stride_k[2] = 1 << 32
    with pytest.raises(_lib.SdpaError) as e:
        api.sdpa_bwd_plan(d)
    assert e.value.status == _lib.SDPA_ERR_UNSUPPORTED and "stride_k" in str(e.value)


def test_run_validates_workspace_and_tensors_before_touching_a_device(lib):
    plan = api.sdpa_bwd_plan(_desc())
    t = _lib.BwdTensors()
    rc = lib.sdpa_bwd_run(plan.handle, ctypes.byref(t), None, plan.workspace_bytes - 1, None)
    assert rc == _lib.SDPA_ERR_WORKSPACE
    assert b"smaller than the planned" in lib.sdpa_last_error()
    rc = lib.sdpa_bwd_run(plan.handle, ctypes.byref(t), ctypes.c_void_p(1000), plan.workspace_bytes, None)
    assert rc == _lib.SDPA_ERR_WORKSPACE  # misaligned workspace
    assert b"256-byte" in lib.sdpa_last_error()


@pytest.mark.parametrize("det", [0, 1, 2])
def test_workspace_size_formula(lib, det):
    # delta, fp32 dQ partials (the per-kv-tile relay only: otherwise this
    # GQA shape computes dQ in the q-major pass), relay counters, control
    # words, dSink partials
    plan = api.sdpa_bwd_plan(_desc(B=2, Hq=4, Hkv=2, D=64, Sq=300, Skv=300, deterministic=det))
    rows = 2 * 4 * 300
    ntq = 5
    expect = 0
    for nbytes in (4 * rows, 4 * rows * 64 if det == 2 else 0, 4 * 2 * 4 * ntq, 16, 4 * 4 * 2 * ntq):
        expect = (expect + nbytes + 255) // 256 * 256
    assert plan.workspace_bytes == expect


def _sections(*nbytes):
    total = 0
    for n in nbytes:
        total = (total + n + 255) // 256 * 256
    return total


@pytest.mark.parametrize("det", [0, 1])
def test_streaming_workspace_size(lib, det):
    # multi-head, causal, window <= 128, head_dim 64: the streaming kernel.
    # Unordered: one 64-row fp32 slot per (batch, head, q-tile) for the
    # boundary partials; ordered: the partial rows plus the relay stash.
    B, H, S, D = 2, 4, 300, 64
    plan = api.sdpa_bwd_plan(_desc(B=B, Hq=H, Hkv=H, D=D, Sq=S, Skv=S, window_left=128, deterministic=det,
                                   engine=1 if det == 0 else 2))
    rows, ntq = B * H * S, 5
    acc = 4 * B * H * ntq * 64 * D if det == 0 else 4 * rows * D
    stash = 4 * rows * D if det == 1 else 0
    assert plan.workspace_bytes == _sections(4 * rows, acc, stash, 4 * B * H * ntq, 16, 4 * H * B * ntq)


def test_streaming_workspace_packed_scales_with_rows_not_batch_times_longest(lib):
    # packed layout, 200 short sequences and one long one: the unordered
    # mode's partial-sum slots follow the packed rows (per head at most
    # total_q / 64 + B + 1 slots), not batch x the longest sequence's tiles
    B, H, D, S = 201, 4, 64, 32768
    T = 200 * 64 + S
    g = api.Geometry(_lib.SDPA_LAYOUT_THD, B, H, H, D, S, S, T, T)
    q = torch.empty(T, H, D, dtype=torch.bfloat16)
    d = api.make_desc(g, torch.bfloat16, q=q, k=q, v=q, o=q, dO=q, dq=q, dk=q, dv=q, window_left=128,
                      has_seq_lens=True, engine=1)
    plan = api.sdpa_bwd_plan(d)
    rows, ntq = H * T, S // 64
    slots = H * ((T >> 6) + B + 1)
    acc = 4 * max(rows * D, slots * 64 * D)
    assert plan.workspace_bytes == _sections(4 * rows, acc, 4 * B * H * ntq, 16, 4 * H * B * ntq)
    assert plan.workspace_bytes < 3 * 4 * rows * D


# ---- the window-bounded schedule, brute force ------------------------------------


def _schedule_cases():
    g = torch.Generator().manual_seed(17)
    cases = [(256, 256, 64, False, True, 0), (32768 // 64, 32768 // 64, 128, False, True, 0),
             (100, 1000, 50, True, True, 0), (260, 130, 40, False, True, 0), (190, 190, -1, False, True, 0),
             (100, 250, 50, True, False, 0), (150, 170, -1, False, False, 0),
             (16484 % 997, 16484 % 997, 96, True, True, 0), (1, 1, 0, False, True, 0), (0, 5, 3, False, True, 0),
             (5, 0, 3, True, True, 0), (300, 300, 64, False, True, 70), (200, 333, 100, True, True, 1),
             (190, 190, -1, False, True, 64), (128, 128, 0, False, True, 1000)]
    for _ in range(60):
        lq, lk = (int(x) for x in torch.randint(0, 400, (2,), generator=g))
        w = int(torch.randint(-1, 300, (1,), generator=g))
        br = bool(torch.randint(0, 2, (1,), generator=g))
        causal = bool(torch.randint(0, 3, (1,), generator=g))  # mostly causal
        wr = int(torch.randint(0, 150, (1,), generator=g)) if causal and torch.rand(1, generator=g) < 0.3 else 0
        cases.append((lq, lk, w, br, causal, wr))
    return cases


@pytest.mark.parametrize("mha", [False, True], ids=["gqa_tiles", "mha"])
@pytest.mark.parametrize("lq,lk,w,br,causal,wr", _schedule_cases())
def test_schedule_covers_the_mask_exactly(lib, lq, lk, w, br, causal, wr, mha):
    # multi-head causal plans with a window <= 128 (and no right band) run
    # the streaming kernel's 128-key kv-steps (forced: this small shape
    # would take the per-tile kernels by the plan's table)
    stream = mha and causal and wr == 0 and 0 <= w <= 128
    d = _desc(window_left=w, window_right=wr, bottom_right=br, Hkv=4 if mha else 2, engine=2 if stream else 0)
    d.causal = int(causal)
    plan = api.sdpa_bwd_plan(d)
    s = api.sdpa_bwd_schedule(plan, lq, lk)
    Tq, Tk = s["tile_q"], s["tile_kv"]
    m = oc.explicit_mask(lq, lk, causal, br, w, wr) if lq and lk else torch.zeros(lq, lk, dtype=torch.bool)
    nq, nk = s["n_q"], s["n_kv"]
    assert nq == -(-lq // Tq) and nk == -(-lk // Tk)
    # tile-level visibility from brute force
    vis = torch.zeros(nq, nk, dtype=torch.bool)
    for i in range(nq):
        for j in range(nk):
            vis[i, j] = bool(m[i * Tq:(i + 1) * Tq, j * Tk:(j + 1) * Tk].any())
    visited = torch.zeros(nq, nk, dtype=torch.bool)
    for j in range(nk):
        lo, hi = s["q_lo"][j], s["q_hi"][j]
        for i in range(max(lo, 0), min(hi, nq)):
            visited[i, j] = True
        if hi <= lo:
            assert not vis[:, j].any(), f"kv-tile {j} stores zeros but has a visible pair"
    # every visible pair is visited (the bound never cuts real work)
    assert not (vis & ~visited).any()
    # the bounds are tight up to tile rounding: for a full kv-tile whose
    # bounding rows exist, q_lo and q_hi - 1 both touch the mask (a partial
    # last tile keeps the formula's kv_base + tile_kv, so it may run long)
    diag = (lk - lq) if br else 0
    for j in range(nk):
        lo, hi = s["q_lo"][j], s["q_hi"][j]
        if hi > lo and vis[:, j].any():
            first = int(torch.nonzero(vis[:, j])[0])
            last = int(torch.nonzero(vis[:, j])[-1])
            r_lo = j * Tk - diag - wr
            if causal and 0 <= r_lo < lq:
                assert lo == first
            r_hi = j * Tk + Tk - 1 + w - diag
            if w >= 0 and (j + 1) * Tk <= lk and 0 <= r_hi < lq:
                assert hi - 1 == last
    # relay visitor ranges equal the visited set, contiguous
    for i in range(nq):
        vs = torch.nonzero(visited[i]).view(-1).tolist()
        if vs:
            assert vs == list(range(vs[0], vs[-1] + 1)), "visitors not contiguous"
            assert s["kv_first"][i] == vs[0] and s["kv_last"][i] == vs[-1]
        else:
            assert s["kv_first"][i] > s["kv_last"][i] or s["kv_last"][i] < 0


# ---- host simulation of the ordered relay ----------------------------------------


def simulate_relay(s, kv_first=None, timeout_s=2.0):
    """One thread per kv-tile visits its q-tiles in descending order; each
    visit waits for its turn (j - kv_first(i)), logs itself, adds its
    partial (here the value 2^j) into the q-tile's running sum, and passes
    the turn on.  A wait past the watchdog gives up and adds NaN instead, as
    the kernels do.  Returns (log per q-tile, expired waits, sums)."""
    kv_first = kv_first or s["kv_first"]
    nq, nk = s["n_q"], s["n_kv"]
    sem = [0] * nq
    log = [[] for _ in range(nq)]
    sums = [0.0] * nq
    expired = []
    lock = threading.Lock()

    def visitor(j):
        for i in range(s["q_hi"][j] - 1, s["q_lo"][j] - 1, -1):
            turn = j - kv_first[i]
            t0 = time.time()
            gave_up = False
            while True:
                with lock:
                    if sem[i] == turn:
                        break
                if time.time() - t0 > timeout_s:
                    with lock:
                        expired.append((i, j))
                    gave_up = True
                    break
                time.sleep(0.0005)
            with lock:
                log[i].append(j)
                sums[i] += float("nan") if gave_up else float(2 ** j)
                sem[i] = turn + 1

    ts = [threading.Thread(target=visitor, args=(j,)) for j in range(nk)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    return log, expired, sums


@pytest.mark.parametrize("mha", [False, True])
@pytest.mark.parametrize("lq,lk,w,br,wr", [(640, 640, 128, False, 0), (300, 700, 100, True, 0),
                                           (500, 500, 0, False, 0), (500, 500, 40, False, 90),
                                           (300, 700, 100, True, 33)])
def test_relay_simulation_orders_every_q_tile(lib, lq, lk, w, br, wr, mha):
    stream = mha and wr == 0 and 0 <= w <= 128
    plan = api.sdpa_bwd_plan(_desc(window_left=w, window_right=wr, bottom_right=br, Hkv=4 if mha else 2,
                                   engine=2 if stream else 0))
    s = api.sdpa_bwd_schedule(plan, lq, lk)
    log, expired, sums = simulate_relay(s)
    assert not expired
    for i in range(s["n_q"]):
        assert log[i] == list(range(s["kv_first"][i], s["kv_last"][i] + 1))
        assert sums[i] == sum(2.0 ** j for j in log[i])


def test_relay_simulation_with_wrong_first_visitor_times_out(lib):
    # Counting turns from kv-tile 0 (the pre-window rule) instead of kv_first
    # leaves every q-tile past the first window waiting for a turn that no
    # visitor takes: the watchdog, not a hang, ends the run.
    plan = api.sdpa_bwd_plan(_desc(window_left=64))
    s = api.sdpa_bwd_schedule(plan, 512, 512)
    log, expired, sums = simulate_relay(s, kv_first=[0] * s["n_q"], timeout_s=0.3)
    assert expired
    # a q-tile whose wait gave up ends poisoned (NaN), never with a plausible
    # sum; the others keep the ordered sum
    bad = {i for i, _ in expired}
    for i in range(s["n_q"]):
        if i in bad:
            assert sums[i] != sums[i]
        else:
            assert sums[i] == sum(2.0 ** j for j in log[i])


def test_relay_watchdog_hook_validates_and_status_names(lib):
    plan = api.sdpa_bwd_plan(_desc(deterministic=2))
    assert lib.sdpa_bwd_plan_set_relay_watchdog(plan.handle, -1, 0) == _lib.SDPA_ERR_INVALID_ARG
    assert b"spin_limit" in lib.sdpa_last_error()
    assert lib.sdpa_bwd_plan_set_relay_watchdog(plan.handle, 16, 2) == _lib.SDPA_ERR_INVALID_ARG
    assert lib.sdpa_bwd_plan_set_relay_watchdog(None, 16, 1) == _lib.SDPA_ERR_INVALID_ARG
    assert lib.sdpa_bwd_plan_set_relay_watchdog(plan.handle, 16, 1) == _lib.SDPA_OK
    assert lib.sdpa_bwd_plan_set_relay_watchdog(plan.handle, 0, 0) == _lib.SDPA_OK
    assert lib.sdpa_status_string(_lib.SDPA_ERR_RELAY_TIMEOUT) == b"SDPA_ERR_RELAY_TIMEOUT"


# ---- the streaming kernel's shift-form schedule, brute force (C++) --------------


def test_stream_schedule_shift_forms_brute_force(tmp_path):
    """StreamSched (the schedule the streaming kernel evaluates) against the
    mask's definition and SeqSched: bounds, retirement, bands and dQ rounds
    (tests/host/stream_sched_check.cpp)."""
    import shutil
    import subprocess
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path / "stream_sched_check")
    csrc = os.path.join(ROOT, "sliding_window_attention_flash_amd", "csrc")
    subprocess.run(["g++", "-std=c++17", "-O2", "-fsanitize=undefined", "-fno-sanitize-recover=all",
                    "-I" + csrc, os.path.join(ROOT, "tests", "host", "stream_sched_check.cpp"), "-o", exe],
                   check=True, capture_output=True, text=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and "stream sched: ok" in r.stdout, r.stdout + r.stderr


def test_noalloc_rejects_a_workspace_beyond_its_scratch(lib):
    # batch 2, 16 heads, S = 32768, window 128, ordered: ~0.5 GB of workspace,
    # more than the 64 MiB scratch; rejected before any device call
    d = _desc(B=2, Hq=16, Hkv=16, D=64, Sq=32768, Skv=32768, window_left=128, deterministic=1)
    plan = api.sdpa_bwd_plan(d)
    assert plan.workspace_bytes > 64 << 20
    t = _lib.BwdTensors()
    rc = lib.sdpa_bwd_run_noalloc(plan.handle, ctypes.byref(t), None)
    assert rc == _lib.SDPA_ERR_WORKSPACE
    msg = lib.sdpa_last_error()
    assert b"scratch" in msg and str(plan.workspace_bytes).encode() in msg
    assert lib.sdpa_bwd_run_noalloc(None, ctypes.byref(t), None) == _lib.SDPA_ERR_INVALID_ARG


# ---- engine choice -----------------------------------------------------------------


@pytest.mark.parametrize("kw,status,needle", [
    (dict(engine=6), _lib.SDPA_ERR_INVALID_ARG, "engine 6"),
    (dict(engine=5), _lib.SDPA_ERR_UNSUPPORTED, "q-major streaming kernel"),
    (dict(engine=5, D=128, window_left=100), _lib.SDPA_ERR_UNSUPPORTED, "q-major streaming kernel"),
    (dict(engine=5, D=128, window_right=3), _lib.SDPA_ERR_UNSUPPORTED, "q-major streaming kernel"),
    (dict(engine=5, D=128, bottom_right=True, Skv=316), _lib.SDPA_ERR_UNSUPPORTED, "q-major streaming kernel"),
    (dict(engine=5, D=128, deterministic=2), _lib.SDPA_ERR_INVALID_ARG, "per-kv-tile relay"),
    (dict(engine=5, D=128, Hq=130, Hkv=1, has_sink=1), _lib.SDPA_ERR_UNSUPPORTED, "q-major streaming kernel"),
    (dict(engine=1, Hkv=2), _lib.SDPA_ERR_UNSUPPORTED, "streaming kernel"),
    (dict(engine=2, Hkv=4, window_left=200), _lib.SDPA_ERR_UNSUPPORTED, "streaming kernel"),
    (dict(engine=2, Hkv=4, D=128), _lib.SDPA_ERR_UNSUPPORTED, "streaming kernel"),
    (dict(engine=1, Hkv=4, deterministic=1), _lib.SDPA_ERR_INVALID_ARG, "not repeatable"),
    (dict(engine=3, Hkv=4, deterministic=2), _lib.SDPA_ERR_INVALID_ARG, "per-kv-tile relay"),
])
def test_plan_rejects_engines_that_do_not_apply(lib, kw, status, needle):
    with pytest.raises(_lib.SdpaError) as e:
        api.sdpa_bwd_plan(_desc(**kw))
    assert e.value.status == status and needle in str(e.value)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(engine=6, D=128, Hq=8, Hkv=1), _lib.SDPA_ERR_INVALID_ARG, "engine 6"),
    (dict(engine=-1), _lib.SDPA_ERR_INVALID_ARG, "engine -1"),
    (dict(engine=5, D=128, Hq=4, Hkv=2), _lib.SDPA_ERR_UNSUPPORTED, "q-major forward"),  # groups of 2
    (dict(engine=5, D=64, Hq=8, Hkv=1), _lib.SDPA_ERR_UNSUPPORTED, "q-major forward"),
    (dict(engine=5, D=128, Hq=8, Hkv=1, window_left=100), _lib.SDPA_ERR_UNSUPPORTED, "q-major forward"),
    (dict(engine=5, D=128, Hq=8, Hkv=1, window_right=3), _lib.SDPA_ERR_UNSUPPORTED, "q-major forward"),
    (dict(engine=5, D=128, Hq=8, Hkv=1, bottom_right=True, Skv=316), _lib.SDPA_ERR_UNSUPPORTED, "q-major forward"),
])
def test_forward_plan_rejects_engines_that_do_not_apply(lib, kw, status, needle):
    with pytest.raises(_lib.SdpaError) as e:
        api.sdpa_fwd_plan(_desc(**kw))
    assert e.value.status == status and needle in str(e.value)


@pytest.mark.parametrize("kw", [dict(engine=5, D=128, Hq=8, Hkv=1), dict(engine=5, D=128, Hq=16, Hkv=1, window_left=0),
                                dict(engine=5, D=128, Hq=8, Hkv=1, bottom_right=True, Skv=332, window_left=96),
                                dict(engine=3, D=128, Hq=8, Hkv=1), dict(engine=0, D=128, Hq=4, Hkv=2),
                                dict(engine=2, D=64, Hq=4, Hkv=4)])
def test_forward_plan_accepts_engines_that_apply(lib, kw):
    # the q-major forward where forced on its shapes; any other engine (or
    # the default, on shapes it does not take) plans the per-tile forward
    plan = api.sdpa_fwd_plan(_desc(**kw))
    assert plan.workspace_bytes == 0


@pytest.mark.parametrize("engine,det,tile_kv", [(1, 0, 128), (2, 0, 128), (2, 1, 128), (3, 0, 64), (3, 1, 64),
                                                (4, 0, 64), (4, 2, 64)])
def test_forced_engine_sets_the_schedule_and_workspace(lib, engine, det, tile_kv):
    # multi-head, causal, window 128, head_dim 64: every engine applies
    B, H, S, D = 2, 4, 300, 64
    plan = api.sdpa_bwd_plan(_desc(B=B, Hq=H, Hkv=H, D=D, Sq=S, Skv=S, window_left=128, engine=engine,
                                   deterministic=det))
    s = api.sdpa_bwd_schedule(plan, S, S)
    assert s["tile_kv"] == tile_kv
    rows, ntq = B * H * S, 5
    acc = {1: 4 * B * H * ntq * 64 * D, 2: 4 * rows * D, 3: 0, 4: 4 * rows * D}[engine]
    stash = 4 * rows * D if engine == 2 else 0
    assert plan.workspace_bytes == _sections(4 * rows, acc, stash, 4 * B * H * ntq, 16, 4 * H * B * ntq)


def _qstream_chunks(B, Hkv, G, S):
    # the plan's chunking for the q-major streaming kernel, restated: r
    # rounds of 256 blocks, chunks of ceil(nqt / floor(256 r / (B Hkv)))
    # 32-row steps (at least 3), least r (C G + 6), fewer rounds on a tie
    bh, nqt = B * Hkv, (S + 31) // 32
    n_cap = max(1, nqt // 3)
    best_c, best_cost = nqt, None
    for r in range(1, 65):
        n0 = min(max(256 * r // bh, 1), n_cap)
        c = -(-nqt // n0)
        n = -(-nqt // c)
        cost = -(-bh * n // 256) * (c * G + 6)
        if best_cost is None or cost < best_cost:
            best_c, best_cost = c, cost
        if n0 == n_cap:
            break
    return -(-nqt // best_c)


@pytest.mark.parametrize("B,Hq,Hkv,Sq,Skv", [(2, 8, 2, 1000, 1064), (1, 2, 2, 300, 300), (12, 48, 6, 16484, 16484),
                                           (1, 8, 1, 16384, 16384)])
def test_forced_engine_5_schedule_and_workspace(lib, B, Hq, Hkv, Sq, Skv):
    # q-major streaming kernel: 32-row q-steps and 32-key tiles; workspace:
    # no delta rows (formed in LDS), the fp32 dK / dV partials of the three
    # kv-tiles at each chunk boundary (both sides), then the common sections
    D = 128
    plan = api.sdpa_bwd_plan(_desc(B=B, Hq=Hq, Hkv=Hkv, D=D, Sq=Sq, Skv=Skv, window_left=96, bottom_right=True,
                                   engine=5, deterministic=1))
    s = api.sdpa_bwd_schedule(plan, Sq, Skv)
    assert (s["tile_q"], s["tile_kv"]) == (32, 32)
    nch = _qstream_chunks(B, Hkv, Hq // Hkv, Sq)
    ntq, nqs = -(-Sq // 64), -(-Sq // 32)
    part = 4 * B * Hkv * nch * 6 * 32 * 2 * D
    # (the dSink partials, one per 32-row q-step and query head)
    assert plan.workspace_bytes == _sections(0, part, 0, 4 * B * Hq * ntq, 16, 4 * Hq * B * nqs)


@pytest.mark.parametrize("B,Hq,Hkv,S,W,det,qstream", [
    (1, 8, 1, 1024, 96, 0, True),     # window of 64 keys or more: the q-major streaming kernel, any grid
    (2, 16, 2, 4096, 64, 1, True),    # repeatable, so deterministic 1 too
    (2, 16, 2, 4096, 32, 0, False),   # 32-key window, 512 q-steps: the per-tile kernels
    (2, 16, 2, 8160, 32, 0, False),   # 1020 q-steps
    (2, 16, 2, 8192, 32, 0, True),    # 1024 q-steps
    (1, 2, 2, 1024, 32, 0, True),     # multi-head: any window, any grid
    (2, 16, 2, 4096, 100, 0, False),  # window beyond 96: not eligible
    (2, 16, 2, 4096, 96, 2, False),   # deterministic 2: the per-kv-tile relay
])
def test_default_engine_d128_follows_the_measured_table(lib, B, Hq, Hkv, S, W, det, qstream):
    plan = api.sdpa_bwd_plan(_desc(B=B, Hq=Hq, Hkv=Hkv, D=128, Sq=S, Skv=S, window_left=W, deterministic=det))
    assert (api.sdpa_bwd_schedule(plan, S, S)["tile_q"] == 32) == qstream


@pytest.mark.parametrize("S,qstream", [(4096, True), (4064, False)])
def test_default_engine_d128_with_sink_from_512_q_steps(lib, S, qstream):
    # groups of 8, a 32-key window and sink logits: the q-major streaming
    # kernel from 512 q-steps (the per-tile path also runs bwd_dot then)
    plan = api.sdpa_bwd_plan(_desc(B=2, Hq=16, Hkv=2, D=128, Sq=S, Skv=S, window_left=32, has_sink=1))
    assert (api.sdpa_bwd_schedule(plan, S, S)["tile_q"] == 32) == qstream


@pytest.mark.parametrize("B,H,S,det,stream", [
    (2, 16, 32768, 1, True),    # 2^20 query rows: the streaming kernel (chunk relay)
    (2, 16, 32768, 0, True),    # unordered too: the chunk relay ties or beats the atomics
    (2, 16, 2048, 0, True),     # exactly 2^16 rows
    (2, 16, 1024, 0, False),    # 2^15 rows: the per-tile kernels
    (1, 2, 16384, 1, False),
    (2, 16, 32768, 2, False),   # deterministic 2: the per-kv-tile relay
])
def test_default_engine_follows_the_measured_table(lib, B, H, S, det, stream):
    plan = api.sdpa_bwd_plan(_desc(B=B, Hq=H, Hkv=H, D=64, Sq=S, Skv=S, window_left=128, deterministic=det))
    assert (api.sdpa_bwd_schedule(plan, S, S)["tile_kv"] == 128) == stream
