"""CPU tests of the host side: the state machine in schedule.hpp (built with g++
through a test shim) against the oracle's schedules, and the C-ABI library's
exports and pure-host calls (no device work)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
from conftest import ROOT

CSRC = os.path.join(ROOT, "bounded_kv_block_amd", "csrc")
SHIM_SRC = os.path.join(ROOT, "tests", "csrc", "schedule_shim.cpp")


@pytest.fixture(scope="module")
def shim(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("shim") / "libschedshim.so")
    subprocess.run(["g++", "-std=c++17", "-O1", "-shared", "-fPIC", f"-I{CSRC}", SHIM_SRC, "-o", out],
                   check=True)
    L = ctypes.CDLL(out)
    L.sched_new.restype = ctypes.c_void_p
    L.sched_new.argtypes = [ctypes.c_int] * 10
    L.sched_new_ref.restype = ctypes.c_void_p
    L.sched_new_ref.argtypes = [ctypes.c_int] * 9
    for n in ("sched_free",):
        getattr(L, n).argtypes = [ctypes.c_void_p]
    for n in ("sched_n_slots", "sched_open", "sched_cur_slot", "sched_memory_count", "sched_n_dynamic"):
        getattr(L, n).argtypes = [ctypes.c_void_p]
        getattr(L, n).restype = ctypes.c_int
    L.sched_mark.argtypes = [ctypes.c_void_p, ctypes.c_int]
    L.sched_last_evicted.argtypes = [ctypes.c_void_p]
    L.sched_last_evicted.restype = ctypes.c_int64
    L.sched_commit.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int),
                               ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
    L.sched_segments.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64), ctypes.c_int]
    L.sched_bank.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int),
                             ctypes.c_int]
    L.sched_commit_displace.argtypes = [ctypes.c_void_p, ctypes.c_int]
    L.sched_pending.argtypes = [ctypes.c_void_p]
    L.sched_pending.restype = ctypes.c_int64
    L.sched_bank_full.argtypes = [ctypes.c_void_p]
    L.sched_new_pose.restype = ctypes.c_void_p
    L.sched_new_pose.argtypes = [ctypes.c_int] * 8
    L.sched_resolve.argtypes = [ctypes.c_void_p, ctypes.c_int64]
    for n in ("sched_bank_count", "sched_free_slots"):
        getattr(L, n).argtypes = [ctypes.c_void_p]
        getattr(L, n).restype = ctypes.c_int
    return L


class Sched:
    def __init__(self, L, **kw):
        self.L = L
        self.layers = kw.get("layers", 1)
        if kw.get("ref_frames") or kw.get("relative"):
            self.p = L.sched_new_ref(self.layers, kw["frames"], kw["tpf"], kw["window"], kw.get("statics", 0),
                                     kw.get("k", 0), kw.get("bank", 0), kw.get("ref_frames", 0),
                                     int(kw.get("relative", 0)))
            return
        args = [kw.get("convkv", 0), self.layers, kw["frames"], kw["tpf"], kw["window"], kw.get("statics", 0),
                kw.get("k", 0), kw.get("bank", 0), kw.get("kernel", 1), kw.get("memory_frames", 0)]
        self.p = L.sched_new(*args)

    def __del__(self):
        self.L.sched_free(self.p)

    def segments(self):
        buf = (ctypes.c_int64 * (7 * 32))()
        n = self.L.sched_segments(self.p, buf, 32)
        return [tuple(buf[7 * i:7 * i + 7]) for i in range(n)]

    def bank(self):
        ids = (ctypes.c_int64 * 300)()
        slots = (ctypes.c_int * 300)()
        n = self.L.sched_bank(self.p, ids, slots, 300)
        return [int(ids[i]) for i in range(n)], [int(slots[i]) for i in range(n)]

    def commit(self):
        ts = (ctypes.c_int * 64)()
        tf = (ctypes.c_int * 64)()
        n = ctypes.c_int(0)
        ok = self.L.sched_commit(self.p, ts, tf, 64, ctypes.byref(n))
        return ok, [(ts[i], tf[i]) for i in range(n.value)]


STATIC, DYNAMIC, WINDOW, CURRENT, MEMORY, REFERENCE = range(6)


@pytest.mark.parametrize("W,B,S,k", [(3, 8, 1, 1), (3, 56, 1, 2), (3, 16, 1, 2), (3, 64, 1, 2), (3, 0, 0, 0),
                                     (2, 3, 1, 3), (1, 1, 0, 1), (4, 5, 1, 0)])
def test_prsink_state_machine_matches_oracle(shim, W, B, S, k):
    F, tpf = 3, 4
    T = F * tpf
    s = Sched(shim, frames=F, tpf=tpf, window=W, statics=S, k=k, bank=B)
    n_slots = shim.sched_n_slots(s.p)
    assert n_slots == S + W + 1 + B
    slot_of = {}
    for m in range(90):
        assert shim.sched_open(s.p) == 1
        assert shim.sched_open(s.p) == 0                     # already open
        want = oracle.prsink_schedule(m, W, B, S)
        segs = s.segments()
        kinds = [g[0] for g in segs]
        nd = min(k, len(want["bank"]))
        assert kinds == [STATIC] * len(want["static"]) + [DYNAMIC] * nd + [WINDOW] * len(want["window"]) + [CURRENT]
        assert [g[1] for g in segs if g[0] == STATIC] == want["static"]
        assert [g[1] for g in segs if g[0] == WINDOW] == want["window"]
        assert [g[5] for g in segs if g[0] == DYNAMIC] == list(range(nd))
        assert all(g[2] == T for g in segs)
        for g in segs:
            if g[0] != DYNAMIC:
                assert g[3] == g[1] * F                      # absolute temporal position
        bank_ids, bank_slots = s.bank()
        assert bank_ids == want["bank"]
        cur = shim.sched_cur_slot(s.p)
        slot_of[m] = cur
        # every block in the cache owns its slot; slots are never shared
        live = [g[4] for g in segs if g[0] != DYNAMIC] + bank_slots
        assert len(set(live)) == len(live) and all(0 <= x < n_slots for x in live)
        for g in segs:
            if g[0] in (STATIC, WINDOW):
                assert g[4] == slot_of[g[1]]                 # a block keeps its slot
        for b, sl in zip(bank_ids, bank_slots):
            assert sl == slot_of[b]
        ok, taps = s.commit()
        assert ok == 0                                       # not every layer attended
        shim.sched_mark(s.p, 0)
        ok, taps = s.commit()
        assert ok == 1 and taps == []
        ev = shim.sched_last_evicted(s.p)
        assert ev == (-1 if want["evicted"] is None else want["evicted"])


@pytest.mark.parametrize("R", [1, 3])
def test_prsink_reference_segment(shim, R):
    """Reference frames: one permanent first segment of R * tokens-per-frame
    keys at t0 = 0 (no slot); every block's t0 moves to R + id * frames; slots
    and the rest of the context are as without it."""
    F, tpf, W, B, S, k = 3, 4, 3, 8, 1, 2
    s = Sched(shim, frames=F, tpf=tpf, window=W, statics=S, k=k, bank=B, ref_frames=R)
    s0 = Sched(shim, frames=F, tpf=tpf, window=W, statics=S, k=k, bank=B)
    assert shim.sched_n_slots(s.p) == shim.sched_n_slots(s0.p) == S + W + 1 + B
    for m in range(30):
        assert shim.sched_open(s.p) == 1 and shim.sched_open(s0.p) == 1
        segs, segs0 = s.segments(), s0.segments()
        assert segs[0] == (REFERENCE, -1, R * tpf, 0, -1, -1, 0)
        assert len(segs) == len(segs0) + 1
        for g, g0 in zip(segs[1:], segs0):
            assert g[:3] == g0[:3] and g[4:] == g0[4:]
            assert g[3] == (-1 if g[0] == DYNAMIC else R + g[1] * F)
        for x in (s, s0):
            shim.sched_mark(x.p, 0)
            assert x.commit()[0] == 1


@pytest.mark.parametrize("W,B,S", [(3, 4, 1), (1, 2, 1), (2, 1, 0)])
def test_prsink_pose_bank_state_machine(shim, W, B, S):
    """Pose-aware replacement in the host state machine: the pending
    eviction and bank-full flags, and commits with the displaced bank
    position the oracle's exact ranking picks, reproduce the oracle's bank
    on every block; slots stay distinct and a block keeps its slot."""
    rng = np.random.default_rng(7)
    P = rng.standard_normal((60, 5)).astype(np.float32)
    sim = oracle.simulate_prsink_pose_bank(60, lambda b: P[b], W, B, S)
    s = Sched(shim, frames=2, tpf=4, window=W, statics=S, k=1, bank=B)
    n_slots = shim.sched_n_slots(s.p)
    slot_of = {}
    for m in range(59):
        assert shim.sched_open(s.p) == 1
        bank_ids, bank_slots = s.bank()
        assert bank_ids == sim[m]["bank"], m
        slot_of[m] = shim.sched_cur_slot(s.p)
        for b, sl in zip(bank_ids, bank_slots):
            assert sl == slot_of[b]
        live = [g[4] for g in s.segments() if g[0] != DYNAMIC] + bank_slots
        assert len(set(live)) == len(live) and all(0 <= x < n_slots for x in live)
        ev = shim.sched_pending(s.p)
        assert ev == (-1 if sim[m]["evicted"] is None else sim[m]["evicted"])
        full = shim.sched_bank_full(s.p) == 1
        assert full == (len(bank_ids) == B)
        displace = -1
        if ev >= 0 and full:
            victim = oracle.retrieve(P[ev], [(b, P[b]) for b in bank_ids], 1)[0]
            displace = bank_ids.index(victim)
        shim.sched_mark(s.p, 0)
        assert shim.sched_commit_displace(s.p, displace) == 1


@pytest.mark.parametrize("W,B,lag", [(3, 4, 2), (1, 2, 1), (2, 3, 0)])
def test_prsink_pose_bank_deferred_displacement(shim, W, B, lag):
    """Pose-aware replacement decided on the device: a commit into a full
    bank displaces a member the host learns of later (resolved `lag` blocks
    late, as a readback would land), using the spare slots meanwhile.  After
    each resolution the host's bank equals the oracle's; the bank count is
    right at every block; slots stay distinct; a block can always open."""
    rng = np.random.default_rng(3)
    P = rng.standard_normal((50, 4)).astype(np.float32)
    sim = oracle.simulate_prsink_pose_bank(50, lambda b: P[b], W, B, 1)
    p = shim.sched_new_pose(1, 2, 4, W, 1, 1, B, 2)
    deferred = shim.sched_deferred_code()
    pending = []                                   # (resolve at block, victim id)
    for m in range(49):
        for due, vid in [x for x in pending if x[0] <= m or shim.sched_free_slots(p) == 0]:
            assert shim.sched_resolve(p, vid) == 1
            pending.remove((due, vid))
        assert shim.sched_open(p) == 1, m
        assert shim.sched_bank_count(p) == len(sim[m]["bank"]), m
        if not pending:
            ids = (ctypes.c_int64 * 512)()
            slots = (ctypes.c_int * 512)()
            n = shim.sched_bank(p, ids, slots, 512)
            assert sorted(ids[:n]) == sorted(sim[m]["bank"]), m
            assert len(set(slots[:n])) == n and shim.sched_cur_slot(p) not in slots[:n]
        ev = shim.sched_pending(p)
        displace = -1
        if ev >= 0 and shim.sched_bank_full(p) == 1:
            victim = oracle.retrieve(P[ev], [(b, P[b]) for b in sim[m]["bank"]], 1)[0]
            pending.append((m + 1 + lag, victim))
            displace = deferred
        shim.sched_mark(p, 0)
        assert shim.sched_commit_displace(p, displace) == 1
    shim.sched_free(p)


@pytest.mark.parametrize("R,k", [(0, 2), (2, 3), (1, 0)])
def test_prsink_relative_segments(shim, R, k):
    """Context-relative PR-Sink: the same blocks, slots and order as with
    absolute positions; block segments take consecutive frames after the
    reference (the retrieved run's first position on each retrieved segment:
    the device adds frames x rank by id) and contiguous context-K rows."""
    F, tpf, W, B, S = 3, 4, 3, 8, 1
    T = F * tpf
    s = Sched(shim, frames=F, tpf=tpf, window=W, statics=S, k=k, bank=B, ref_frames=R, relative=1)
    s0 = Sched(shim, frames=F, tpf=tpf, window=W, statics=S, k=k, bank=B, ref_frames=R)
    for m in range(30):
        assert shim.sched_open(s.p) == 1 and shim.sched_open(s0.p) == 1
        segs, segs0 = s.segments(), s0.segments()
        assert [g[:3] + g[4:6] for g in segs] == [g[:3] + g[4:6] for g in segs0]
        blocks = [g for g in segs if g[0] != REFERENCE]
        nd = sum(g[0] == DYNAMIC for g in blocks)
        t, want_t = R, []
        for g in blocks:
            want_t.append(t if g[0] != DYNAMIC else R + S * F)
            t += F
        assert [g[3] for g in blocks] == want_t
        assert [g[6] for g in blocks] == [i * T for i in range(len(blocks))]
        assert blocks[-1][3] == R + (len(blocks) - 1) * F and nd <= k
        for x in (s, s0):
            shim.sched_mark(x.p, 0)
            assert x.commit()[0] == 1


@pytest.mark.parametrize("F,tpf,W,K,M", [(3, 4, 3, 5, 1), (2, 3, 3, 5, 1), (1, 5, 2, 3, 2), (4, 2, 3, 5, 2),
                                         (3, 1024, 3, 5, 1)])
def test_convkv_state_machine_matches_oracle(shim, F, tpf, W, K, M):
    T = F * tpf
    s = Sched(shim, convkv=1, frames=F, tpf=tpf, window=W, kernel=K, memory_frames=M, layers=2)
    n_slots = shim.sched_n_slots(s.p)
    staged = -(-K * M // F)
    assert n_slots == W + 1 + staged
    slot_of = {}
    for m in range(40):
        assert shim.sched_open(s.p) == 1
        want = oracle.convkv_schedule(m, F, W, K, M)
        segs = s.segments()
        n_mem = len(want["memory"])
        assert shim.sched_memory_count(s.p) == n_mem
        assert [g[0] for g in segs] == [MEMORY] * n_mem + [WINDOW] * len(want["window"]) + [CURRENT]
        assert [g[1] for g in segs if g[0] == WINDOW] == want["window"]
        assert [g[3] for g in segs if g[0] == WINDOW] == want["t0"]["window"]
        assert segs[-1][3] == want["t0"]["current"]
        assert [g[3] for g in segs if g[0] == MEMORY] == list(range(n_mem))
        offs = np.cumsum([0] + [g[2] for g in segs])[:-1]
        assert [g[6] for g in segs] == list(offs)             # contiguous context-K rows
        assert [g[2] for g in segs] == [tpf] * n_mem + [T] * (len(segs) - n_mem)
        slot_of[m] = shim.sched_cur_slot(s.p)
        shim.sched_mark(s.p, 0)
        ok, _ = s.commit()
        assert ok == 0                                       # layer 1 not attended
        shim.sched_mark(s.p, 1)
        ok, taps = s.commit()
        assert ok == 1
        nxt = oracle.convkv_schedule(m + 1, F, W, K, M)
        want_taps = [(slot_of[e // F], e % F) for grp in nxt["memory"] for e in grp]
        if m - W >= 0:                                       # something was evicted: memory rebuilt
            assert taps == want_taps, m
        else:
            assert taps == []
        # taps only read blocks that are no longer in the window (staged slots)
        win_slots = {slot_of[b] for b in nxt["window"]}
        assert not (set(t[0] for t in taps) & win_slots)


# ------------------------------------------------------------------ C-ABI exports
def _declared():
    with open(os.path.join(ROOT, "include", "bkv.h")) as fh:
        text = fh.read()
    return sorted(set(re.findall(r"^\s*(?:bkv_status|const char\*)\s+(bkv_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    from bounded_kv_block_amd import bkv
    declared = _declared()
    assert set(declared) == set(bkv.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", bkv.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (bkv_\w+)", out))
    assert set(declared) <= exported, set(declared) - exported
    L = bkv.lib()
    for name in declared:
        assert hasattr(L, name)


def test_workspace_size_and_validation():
    from bounded_kv_block_amd import bkv, synth
    c2 = bkv.config_from_workload(synth.workload("prsink_512"))
    n = bkv.workspace_size(c2)
    slot = 2 * 40 * 3072 * 128 * 2
    # 480 (head, 256-query) units > 256 workgroups: the workspace holds 256
    # fp32 split slots (O, m, l of 256 rows), one per key part of a cut unit
    split = 256 * (8 * 64 * 64 * 4 + 8 * 2 * 64 * 4)
    qs = 3072 * 40 * 128 * 2                 # bf16 q scratch of the fused projection path
    assert 61 * slot + split + qs <= n < 61 * slot + split + qs + (1 << 20)   # 61 slots of 62.9 MB
    n8 = bkv.workspace_size(bkv.config_from_workload(synth.workload("prsink_512", heads=8)))
    assert (61 * slot + qs) // 5 <= n8 < (61 * slot + qs) // 5 + (1 << 20)    # 96 units: no split slots
    c3 = bkv.config_from_workload(synth.workload("prsink_720x416"))
    assert bkv.workspace_size(c3) >= 40 * 21 * 2 * 40 * 3520 * 128 * 2
    c5 = bkv.config_from_workload(synth.workload("convkv_512"))
    n5 = bkv.workspace_size(c5)
    ctx = 13312 * 40 * 128 * 2                               # rotated context K
    mem = 2 * 1024 * 40 * 128 * 2                            # memory frame K + V
    assert 6 * slot + ctx + mem + split + qs <= n5 < 6 * slot + ctx + mem + split + qs + (1 << 20)
    c1 = bkv.config_from_workload(synth.workload("tiny_fp32"))
    assert bkv.workspace_size(c1) > 13 * 2 * 2 * 128 * 64 * 4
    bad = [dict(rope=(44, 42, 40)), dict(rope=(43, 43, 42)), dict(window=0), dict(dynamic_k=9),
           dict(bank=257), dict(head_dim=64), dict(layers=0)]
    for b in bad:
        with pytest.raises(bkv.BkvError) as ei:
            bkv.workspace_size(bkv.config_from_workload(synth.workload("prsink_512", **b)))
        assert ei.value.status in (bkv.BKV_ERR_ARG, bkv.BKV_ERR_UNSUPPORTED), b
    c = bkv.config_from_workload(synth.workload("prsink_512"))
    c.struct_size = 12
    with pytest.raises(bkv.BkvError):
        bkv.workspace_size(c)
    bad5 = bkv.config_from_workload(synth.workload("convkv_512", conv_stride=4))
    with pytest.raises(bkv.BkvError):
        bkv.workspace_size(bad5)
    assert bkv.lib().bkv_status_str(bkv.BKV_ERR_STATE) == b"BKV_ERR_STATE"


def test_fp8_key_cache_workspace_and_validation():
    """FP8 key cache: a PR-Sink slot holds E4M3 K (1 byte per value), one
    int32 exponent per (head, 64-token tile) and the bf16 V^T; ConvKV keeps
    bf16 slots and an E4M3 context buffer with one exponent per (head, tile
    of a segment); head_dim 128 only."""
    from bounded_kv_block_amd import bkv, synth
    n16 = bkv.workspace_size(bkv.config_from_workload(synth.workload("prsink_512")))
    n8 = bkv.workspace_size(bkv.config_from_workload(synth.workload("prsink_512_fp8k")))
    H, Tp, D = 40, 3072, 128
    kx = -(-(4 * H * Tp // 64) // 256) * 256          # exponents, 256-byte aligned
    slot8 = H * Tp * D + kx + H * Tp * D * 2
    slot16 = 2 * H * Tp * D * 2
    assert n16 - n8 == 61 * (slot16 - slot8)            # same 61 slots, tables, split slots, q scratch
    with pytest.raises(bkv.BkvError) as ei:
        bkv.workspace_size(bkv.config_from_workload(synth.workload("prsink_512_fp8k", head_dim=64)))
    assert ei.value.status == bkv.BKV_ERR_UNSUPPORTED
    c16 = bkv.workspace_size(bkv.config_from_workload(synth.workload("convkv_512")))
    c8 = bkv.workspace_size(bkv.config_from_workload(synth.workload("convkv_512", dtype="bf16_fp8k")))
    al = lambda n: -(-n // 256) * 256
    rows = 13312 + 64                                   # largest context + one key tile
    xt = 1024 // 64 + 4 * (3072 // 64)                  # tiles: the memory frame, 3 windows + current
    ctx16 = al(H * rows * D * 2)
    ctx8 = al(al(H * rows * D) + 4 * H * xt)
    assert c16 - c8 == ctx16 - ctx8                     # same bf16 slots, memory and q scratch
    c = bkv.config_from_workload(synth.workload("prsink_512"))
    c.dtype = 4
    with pytest.raises(bkv.BkvError) as ei:
        bkv.workspace_size(c)
    assert ei.value.status == bkv.BKV_ERR_ARG


def test_fp8_kv_cache_workspace():
    """FP8 KV cache: a PR-Sink slot holds E4M3 K and E4M3 V^T (1 byte per
    value each) with one int32 exponent per (head, 64-token tile) for each,
    so K+V bytes per slot are half the bf16 slot's plus the exponents; a
    ConvKV slot keeps its raw bf16 K and V^T (the conv and the rotation read
    them) and adds the E4M3 V^T; its memory adds E4M3 V^T and exponents."""
    from bounded_kv_block_amd import bkv, synth
    al = lambda n: -(-n // 256) * 256
    H, Tp, D = 40, 3072, 128
    kx = 4 * H * Tp // 64
    n16 = bkv.workspace_size(bkv.config_from_workload(synth.workload("prsink_512")))
    n88 = bkv.workspace_size(bkv.config_from_workload(synth.workload("prsink_512_fp8kv")))
    slot16 = 2 * H * Tp * D * 2
    slot88 = al(al(H * Tp * D + kx) + H * Tp * D + kx)
    assert 2 * (slot88 - 2 * kx) <= slot16 and n16 - n88 == 61 * (slot16 - slot88)
    c16 = bkv.workspace_size(bkv.config_from_workload(synth.workload("convkv_512")))
    c88 = bkv.workspace_size(bkv.config_from_workload(synth.workload("convkv_512_fp8kv")))
    c8 = bkv.workspace_size(bkv.config_from_workload(synth.workload("convkv_512_fp8k")))
    slot_c = 2 * H * Tp * D * 2
    slot_c88 = al(2 * H * Tp * D * 2 + H * Tp * D + kx)
    mem_extra = al(al(2 * H * 1024 * D * 2) + H * 1024 * D + 4 * H * 1024 // 64) - al(2 * H * 1024 * D * 2)
    assert c88 - c8 == 6 * (slot_c88 - slot_c) + mem_extra and c8 < c16
    with pytest.raises(bkv.BkvError) as ei:
        bkv.workspace_size(bkv.config_from_workload(synth.workload("prsink_512_fp8kv", head_dim=64)))
    assert ei.value.status == bkv.BKV_ERR_UNSUPPORTED


def test_workspace_is_constant_in_stream_length():
    """Cache bytes do not depend on how long the stream runs: no config field
    names a stream length, and the 1080-block workload needs the same bytes as
    a 60-block one with the same bank."""
    from bounded_kv_block_amd import bkv, synth
    a = bkv.workspace_size(bkv.config_from_workload(synth.workload("prsink_long")))
    b = bkv.workspace_size(bkv.config_from_workload(synth.workload("prsink_long", blocks=60)))
    assert a == b


def test_reference_frames_workspace_and_validation():
    """Reference frames: one slot-shaped region per layer of R * grid_h * grid_w
    keys padded to a 64-key tile, plus an R-row temporal RoPE table; PR-Sink
    only, 0..8 frames; the largest context (reference, static, 8 dynamic, a
    window of 8, current) fits the segment limit."""
    from bounded_kv_block_amd import bkv, synth
    n0 = bkv.workspace_size(bkv.config_from_workload(synth.workload("prsink_512")))
    n1 = bkv.workspace_size(bkv.config_from_workload(synth.workload("prsink_512_ref")))
    H, D = 40, 128
    assert n1 - n0 == 2 * H * 1024 * D * 2 + 256        # K + V^T of 1024 tokens, 1-row table (one 256 B block)
    n8 = bkv.workspace_size(bkv.config_from_workload(synth.workload("prsink_512_fp8k")))
    n8r = bkv.workspace_size(bkv.config_from_workload(synth.workload("prsink_512_fp8k", reference_frames=2)))
    kx = -(-(4 * H * 2048 // 64) // 256) * 256
    assert n8r - n8 == H * 2048 * D + kx + H * 2048 * D * 2 + 512   # 2 x 23 (cos, sin) pairs -> 512 B
    nodd = bkv.workspace_size(bkv.config_from_workload(synth.workload("tiny_fp32", grid_h=3, grid_w=5,
                                                                      reference_frames=1)))
    n0dd = bkv.workspace_size(bkv.config_from_workload(synth.workload("tiny_fp32", grid_h=3, grid_w=5)))
    assert nodd - n0dd >= 2 * 2 * 64 * 64 * 4            # 15 keys padded to one 64-key tile
    big = synth.workload("prsink_512", reference_frames=8, window=8, dynamic_k=8, bank=64)
    assert bkv.workspace_size(bkv.config_from_workload(big)) > 0
    for b, st in ((dict(reference_frames=9), bkv.BKV_ERR_ARG), (dict(reference_frames=-1), bkv.BKV_ERR_ARG)):
        with pytest.raises(bkv.BkvError) as ei:
            bkv.workspace_size(bkv.config_from_workload(synth.workload("prsink_512", **b)))
        assert ei.value.status == st, b
    with pytest.raises(bkv.BkvError) as ei:
        bkv.workspace_size(bkv.config_from_workload(synth.workload("convkv_512", reference_frames=1)))
    assert ei.value.status == bkv.BKV_ERR_UNSUPPORTED


def test_relative_positions_workspace_and_validation():
    """Context-relative PR-Sink adds a context-K buffer of the largest context
    (less the reference) plus one key tile, per layer, and a temporal table
    of its frames (with the FP8 key cache: E4M3 rows and tile exponents, and
    bf16 slots).  ConvKV's memory-only reset needs no extra bytes; an
    unknown positions value is rejected."""
    from bounded_kv_block_amd import bkv, synth
    n0 = bkv.workspace_size(bkv.config_from_workload(synth.workload("prsink_512")))
    n1 = bkv.workspace_size(bkv.config_from_workload(synth.workload("prsink_512_rel")))
    ctx = (21504 + 64) * 40 * 128 * 2
    al = lambda n: -(-n // 256) * 256
    tt = al(8 * 21 * 23) - al(8 * 3 * 23)                # 21 t rows of 23 (cos, sin) pairs instead of 3
    assert n1 - n0 == ctx + tt
    r8 = bkv.workspace_size(bkv.config_from_workload(synth.workload("prsink_512_fp8k", positions="relative")))
    ctx8 = al(al((21504 + 64) * 40 * 128) + 4 * 40 * 7 * 48)
    assert n1 - r8 == ctx - ctx8                        # bf16 slots and a q scratch in both
    assert (bkv.workspace_size(bkv.config_from_workload(synth.workload("convkv_512_abs")))
            == bkv.workspace_size(bkv.config_from_workload(synth.workload("convkv_512"))))
    c = bkv.config_from_workload(synth.workload("convkv_512"))
    c.rope_positions = 3
    with pytest.raises(bkv.BkvError) as ei:
        bkv.workspace_size(c)
    assert ei.value.status == bkv.BKV_ERR_ARG


def test_pose_bank_validation():
    """Pose-aware replacement needs poses and a bank; ConvKV has no bank; an
    unknown policy is rejected.  It adds two spare slots (blocks open while a
    displaced member is being read back), their pose rows, and the device's
    bank table (ids and slots of 256 members) with four readback pairs."""
    from bounded_kv_block_amd import bkv, synth
    al = lambda n: -(-n // 256) * 256
    n0 = bkv.workspace_size(bkv.config_from_workload(synth.workload("prsink_512", bank=8)))
    n1 = bkv.workspace_size(bkv.config_from_workload(synth.workload("prsink_512_posebank")))
    slot = 2 * 40 * 3072 * 128 * 2
    poses = al(4 * 15 * 128) - al(4 * 13 * 128)
    table = al(4 * (2 * 256 + 2 * 4))
    assert n1 - n0 == 2 * slot + poses + table
    for w in (synth.workload("prsink_512_posebank", bank=0), synth.workload("prsink_512_posebank", pose_dim=0,
                                                                          dynamic_k=0)):
        with pytest.raises(bkv.BkvError) as ei:
            bkv.workspace_size(bkv.config_from_workload(w))
        assert ei.value.status == bkv.BKV_ERR_ARG
    c = bkv.config_from_workload(synth.workload("convkv_512"))
    c.bank_policy = 1
    with pytest.raises(bkv.BkvError) as ei:
        bkv.workspace_size(c)
    assert ei.value.status == bkv.BKV_ERR_ARG
    c = bkv.config_from_workload(synth.workload("prsink_512"))
    c.bank_policy = 2
    with pytest.raises(bkv.BkvError) as ei:
        bkv.workspace_size(c)
    assert ei.value.status == bkv.BKV_ERR_ARG


def test_schedule_stress_under_address_and_ub_sanitizers(tmp_path):
    """The host state machine under AddressSanitizer and
    UndefinedBehaviorSanitizer (a g++ build of schedule.hpp with a stand-alone
    driver): hundreds of random configurations of each mode, long streams,
    late-resolved bank displacements, slot and count invariants after every
    call; any sanitizer finding aborts the run."""
    exe = str(tmp_path / "schedule_stress")
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", f"-I{CSRC}",
                    os.path.join(ROOT, "tests", "csrc", "schedule_stress.cpp"), "-o", exe], check=True)
    r = subprocess.run([exe, "300"], capture_output=True, text=True, timeout=240,
                       env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1"))
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "no violation" in r.stdout
