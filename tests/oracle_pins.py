"""Checks that pin the oracle to facts outside itself.

Each check takes the oracle function(s) it pins as arguments, so the same
check runs against the real oracle (tests/test_oracle.py) and against copies
with a planted mistake (tests/test_oracle_mutations.py), which must fail it.
Every check raises AssertionError on a mismatch.
"""
from __future__ import annotations

import numpy as np

from conftest import ids, read_table


# ---------------------------------------------------------------- schedules
def check_prsink_golden(prsink_schedule):
    """Hand-derived table (tests/golden) for window 3, bank 8, one static block."""
    for row in read_table("prsink_schedule_w3_b8_s1.txt"):
        m = int(row[0])
        s = prsink_schedule(m, 3, 8, 1)
        assert s["static"] == ids(row[1]), (m, s)
        assert s["bank"] == ids(row[2]), (m, s)
        assert s["window"] == ids(row[3]), (m, s)
        ev = None if row[4] == "-" else int(row[4])
        assert s["evicted"] == ev, (m, s)


def check_prsink_closed_vs_sim(prsink_schedule, simulate_prsink):
    for W in (1, 2, 3, 4):
        for B in (0, 1, 2, 5, 8):
            for S in (0, 1, 2):
                sim = simulate_prsink(30, W, B, S)
                for m in range(30):
                    assert prsink_schedule(m, W, B, S) == sim[m], (W, B, S, m)


def check_convkv_golden(convkv_schedule):
    for row in read_table("convkv_schedule_f3_w3_k5_m1.txt"):
        m = int(row[0])
        s = convkv_schedule(m, 3, 3, 5, 1)
        assert s["window"] == ids(row[1]), (m, s)
        assert s["evicted_frames"] == int(row[2]), (m, s)
        assert s["memory"] == ([] if row[3] == "-" else [ids(row[3])]), (m, s)
        assert s["t0"]["window"] == ids(row[4]), (m, s)
        assert s["t0"]["current"] == int(row[5]), (m, s)
        assert s["evicted"] == (None if row[6] == "-" else int(row[6])), (m, s)


def check_convkv_closed_vs_sim(convkv_schedule, simulate_convkv):
    for F in (1, 2, 3, 4):
        for W in (1, 2, 3):
            for K in (2, 3, 5):
                for M in (1, 2, 3):
                    sim = simulate_convkv(25, F, W, K, M)
                    for m in range(25):
                        assert convkv_schedule(m, F, W, K, M) == sim[m], (F, W, K, M, m)


# ---------------------------------------------------------------- retrieval
def check_retrieval_hand(retrieve):
    """2-D poses whose cosines are known by hand: 1, 1/sqrt2, 0, -1."""
    q = np.array([1, 0], np.float32)
    bank = [(10, np.array([1, 1], np.float32)), (11, np.array([3, 0], np.float32)),
            (12, np.array([0, 2], np.float32)), (13, np.array([-1, 0], np.float32))]
    assert retrieve(q, bank, 4) == [11, 10, 12, 13]
    assert retrieve(q, bank, 2) == [11, 10]
    assert retrieve(q, bank, 9) == [11, 10, 12, 13]          # fewer candidates than k
    assert retrieve(q, [], 3) == []


def check_retrieval_ties(retrieve, rng):
    """Exact ties (bitwise duplicate; a copy scaled by 2) go to the lower stream id."""
    P = 32
    for trial in range(20):
        base = rng.standard_normal(P).astype(np.float32)
        q = (base + 0.3 * rng.standard_normal(P)).astype(np.float32)
        others = [rng.standard_normal(P).astype(np.float32) for _ in range(5)]
        dup = base.copy()
        twice = (base * np.float32(2)).astype(np.float32)
        for a, b in ((base, dup), (base, twice), (twice, base)):
            lo, hi = 3 + trial, 40 + trial
            bank = [(hi, b), (7, others[0]), (lo, a), (90, others[1])]
            got = retrieve(q, bank, 2)
            # base is by construction the closest: it and its tie take the top 2, low id first
            assert got == [lo, hi], (trial, got)
    # zero-norm poses score 0: ranked above negative cosines, below positive ones
    q = np.array([1, 0, 0], np.float32)
    bank = [(5, np.zeros(3, np.float32)), (2, np.array([-1, 0, 0], np.float32)),
            (9, np.array([1, 1, 0], np.float32)), (3, np.zeros(3, np.float32))]
    assert retrieve(q, bank, 4) == [9, 3, 5, 2]
    assert retrieve(np.zeros(3, np.float32), bank, 4) == [2, 3, 5, 9]   # zero query: all tie


def check_retrieval_vs_fp64(retrieve, rng):
    """On tie-free random data the exact ranking equals an fp64 numpy argsort."""
    from oracle.retrieval import fp64_cosines
    for trial in range(30):
        P = int(rng.integers(2, 130))
        n = int(rng.integers(1, 70))
        q = rng.standard_normal(P).astype(np.float32)
        poses = rng.standard_normal((n, P)).astype(np.float32)
        id_list = list(rng.permutation(1000)[:n])
        bank = list(zip(id_list, poses))
        k = int(rng.integers(1, 6))
        c = fp64_cosines(q, poses)
        order = np.argsort(-c, kind="stable")
        assert retrieve(q, bank, k) == [id_list[i] for i in order[:k]], trial


def check_repeat_pose(retrieve_stream):
    """Tiny fp32 stream: blocks 7 and 11 copy an earlier pose (+0.01 noise) and must
    retrieve exactly that block (LiveAnimate page, 方法: the dynamic sink restores
    the context of a recurring pose)."""
    from bounded_kv_block_amd import synth
    cfg = synth.workload("tiny_fp32")
    src = synth.repeat_sources(cfg)
    assert set(src) == {3, 7, 11} and src[3] == 0
    for m in (7, 11):
        assert retrieve_stream(cfg, m) == [src[m]], (m, src)


# ---------------------------------------------------------------- rope
def check_rope_frequencies(rope_frequencies):
    w = rope_frequencies(4, 10000.0)
    assert np.allclose(w, [1.0, 0.01], rtol=0, atol=1e-15)
    w = rope_frequencies(44, 10000.0)
    assert len(w) == 22 and w[0] == 1.0
    assert np.isclose(w[21], 10000.0 ** (-42.0 / 44.0), rtol=1e-14)


def check_rope_properties(apply_rope, rng):
    N, H, D = 7, 3, 24
    split = (8, 8, 8)
    x = rng.standard_normal((N, H, D))
    zero = np.zeros(N)
    assert np.array_equal(apply_rope(x, zero, zero, zero, split), x)          # identity at 0
    pt, ph, pw = rng.integers(0, 50, (3, N)).astype(np.float64)
    y = apply_rope(x, pt, ph, pw, split)
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    # hand value: one pair, position 1 -> rotation by 1 radian
    e = np.zeros((1, 1, 2))
    e[0, 0, 0] = 1.0
    r = apply_rope(e, np.ones(1), np.zeros(1), np.zeros(1), (2, 0, 0))
    assert np.allclose(r[0, 0], [np.cos(1.0), np.sin(1.0)], atol=1e-15)
    # complex-multiplication formulation, per axis
    out = np.empty_like(x)
    off = 0
    for size, pos in zip(split, (pt, ph, pw)):
        i = np.arange(size // 2)
        z = x[:, :, off:off + size:2] + 1j * x[:, :, off + 1:off + size:2]
        z = z * np.exp(1j * pos[:, None, None] * (10000.0 ** (-2.0 * i / size))[None, None, :])
        out[:, :, off:off + size:2] = z.real
        out[:, :, off + 1:off + size:2] = z.imag
        off += size
    assert np.allclose(y, out, atol=1e-12)
    # relative positions: shifting every t (or y, x) by a constant keeps q.k
    q = rng.standard_normal((N, H, D))
    k = rng.standard_normal((N, H, D))
    qt, kt = rng.integers(0, 40, (2, N)).astype(np.float64)
    a = np.einsum("nhd,mhd->hnm", apply_rope(q, qt, ph, pw, split), apply_rope(k, kt, ph, pw, split))
    b = np.einsum("nhd,mhd->hnm", apply_rope(q, qt + 17, ph + 3, pw, split),
                  apply_rope(k, kt + 17, ph + 3, pw, split))
    assert np.allclose(a, b, atol=1e-10)
    # an axis only touches its own channels
    y2 = apply_rope(x, pt, zero, zero, split)
    assert np.array_equal(y2[:, :, 8:], x[:, :, 8:])


# ---------------------------------------------------------------- attention
def check_attention_vs_torch(attention, rng):
    import torch
    for (Nq, Nk, H, D) in ((5, 9, 2, 8), (33, 70, 3, 16), (64, 1, 1, 4)):
        q = rng.standard_normal((Nq, H, D))
        k = rng.standard_normal((Nk, H, D))
        v = rng.standard_normal((Nk, H, D))
        got = attention(q, k, v)
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a.transpose(1, 0, 2)))[None]
        ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v))[0]
        assert np.allclose(got, ref.numpy().transpose(1, 0, 2), atol=1e-12), (Nq, Nk)


def check_attention_closed_forms(attention, softmax_weights, rng):
    H, D = 2, 8
    k = rng.standard_normal((11, H, D))
    v = rng.standard_normal((11, H, D))
    o = attention(np.zeros((4, H, D)), k, v)                      # Q = 0 -> mean of V
    assert np.allclose(o, np.broadcast_to(v.mean(axis=0), o.shape), atol=1e-14)
    o1 = attention(rng.standard_normal((3, H, D)), k[:1], v[:1])  # one key -> that value
    assert np.allclose(o1, np.broadcast_to(v[0], o1.shape), atol=1e-14)
    p = softmax_weights(rng.standard_normal((6, D)), k[:, 0], 0.5)
    assert np.all(p >= 0) and np.allclose(p.sum(axis=1), 1.0, atol=1e-12)
    # two keys, closed form: p0 = 1 / (1 + exp(s*(q.k1 - q.k0)))
    q1 = rng.standard_normal((1, 1, D))
    kk = rng.standard_normal((2, 1, D))
    vv = np.zeros((2, 1, D))
    vv[1, 0, 0] = 1.0
    s = 1 / np.sqrt(D)
    z = s * (kk[:, 0] @ q1[0, 0])
    want = 1 / (1 + np.exp(z[0] - z[1]))
    assert np.isclose(attention(q1, kk, vv)[0, 0, 0], want, rtol=1e-13)
    # key/value order does not matter
    q = rng.standard_normal((5, H, D))
    perm = rng.permutation(11)
    assert np.allclose(attention(q, k, v), attention(q, k[perm], v[perm]), atol=1e-13)


# ---------------------------------------------------------------- convkv
def check_conv_memory(conv_memory, rng):
    n, H, S, D, K = 5, 2, 6, 4, 5
    fr = rng.standard_normal((n, H, S, D))
    onehot = np.zeros((H, D, K))
    onehot[:, :, K - 1] = 1.0
    assert np.array_equal(conv_memory(fr, onehot)[0], fr[-1])          # tap 4 -> newest frame
    mean = np.full((H, D, K), 1.0 / K)
    assert np.allclose(conv_memory(fr, mean)[0], fr.mean(axis=0), atol=1e-14)
    w = rng.standard_normal((H, D, K))
    got = conv_memory(fr, w)[0]
    for h in range(H):
        for c in range(D):
            for s in range(S):
                ref = np.correlate(fr[:, h, s, c], w[h, c, :], mode="valid")
                assert np.isclose(got[h, s, c], ref[0], rtol=1e-13, atol=1e-14)
    fr2 = rng.standard_normal((n, H, S, D))
    assert np.allclose(conv_memory(2 * fr - 3 * fr2, w), 2 * conv_memory(fr, w) - 3 * conv_memory(fr2, w),
                       atol=1e-12)
    two = rng.standard_normal((2 * K, H, S, D))                       # two output frames, stride K
    out = conv_memory(two, w)
    assert out.shape[0] == 2 and np.allclose(out[1], conv_memory(two[K:], w)[0], atol=1e-14)


# -- FP8 (E4M3) quantisation ----------------------------------------------------
def _e4m3_sweep():
    """Every bf16 magnitude in [2^-12, 448], the midpoints between neighbours,
    the subnormal grid and its midpoints, both signs, and zero."""
    mags = [np.ldexp(1.0 + m / 128.0, e) for e in range(-12, 9) for m in range(128)]
    mags += [np.ldexp(1.0 + (m + 0.5) / 128.0, e) for e in range(-12, 9) for m in range(128)]
    mags += [j * 2.0 ** -10 for j in range(0, 16)]
    x = np.array(mags, np.float64)
    x = x[x <= 448.0]
    return np.concatenate([x, -x, [0.0]])


def check_e4m3_vs_torch(e4m3_round):
    """Library pin: torch's float8_e4m3fn conversion (OCP E4M3, nearest-even)."""
    import torch
    x = _e4m3_sweep()
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = e4m3_round(x)
    assert np.array_equal(got, want), np.nonzero(got != want)[0][:5]


def check_e4m3_hand(e4m3_round):
    """Values worked by hand from the format (3 mantissa bits, bias 7, max 448)."""
    cases = [(1.0, 1.0), (1.0625, 1.0), (1.1875, 1.25), (-1.0625, -1.0), (448.0, 448.0),
             (440.0, 448.0), (424.0, 416.0), (2.0 ** -6, 2.0 ** -6), (1.5 * 2.0 ** -9, 2.0 ** -8),
             (0.5 * 2.0 ** -9, 0.0), (0.75 * 2.0 ** -9, 2.0 ** -9), (3.0 * 2.0 ** -10, 2.0 ** -8)]
    for x, want in cases:
        assert e4m3_round(np.array([x]))[0] == want, (x, want)


def check_pow2_exponent(pow2_exponents, rng):
    """The smallest e with amax * 2^-e <= 448: hand values and the defining
    inequalities on random magnitudes."""
    hand = [(448.0, 0), (449.0, 1), (224.0, -1), (224.5, 0), (1.0, -8), (0.0, 0), (3.5, -7)]
    for a, e in hand:
        assert pow2_exponents(np.array([a]))[0] == e, (a, e)
    a = np.exp(rng.uniform(-20, 20, 2000))
    e = pow2_exponents(a)
    assert np.all(a * 2.0 ** -e.astype(float) <= 448.0)
    assert np.all(a * 2.0 ** -(e - 1).astype(float) > 448.0)


def check_fp8_groups(quantize_keys, quantize_queries, rng):
    """Group structure: K has one scale per (64-token tile, head), Q one per
    (token, head); values representable at the group's scale are kept exactly;
    relative rounding error of normal values is at most 2^-4."""
    T, H, D = 150, 3, 16
    k = rng.standard_normal((T, H, D))
    qk = quantize_keys(k)
    # a tile's values depend only on that tile: scaling tile 1 of head 2 by 2^10
    k2 = k.copy()
    k2[64:128, 2] *= 2.0 ** 10
    qk2 = quantize_keys(k2)
    assert np.array_equal(np.delete(qk2, np.s_[64:128], axis=0), np.delete(qk, np.s_[64:128], axis=0))
    assert np.array_equal(qk2[64:128, :2], qk[64:128, :2])
    assert np.array_equal(qk2[64:128, 2], qk[64:128, 2] * 2.0 ** 10)
    big = np.abs(k) > np.abs(k).max() * 2.0 ** -6
    assert np.all(np.abs(qk - k)[big] <= 2.0 ** -4 * np.abs(k)[big] + 1e-300)
    # a row of E4M3 values whose largest magnitude is 448 is unchanged
    q = rng.integers(-8, 9, (4, 2, D)).astype(np.float64)
    q[:, :, 0] = 448.0
    assert np.array_equal(quantize_queries(q), q)
    # per-row scales: one row's magnitude does not affect another row
    q3 = rng.standard_normal((5, 2, D))
    q4 = q3.copy()
    q4[2] *= 1e4
    assert np.array_equal(np.delete(quantize_queries(q4), 2, axis=0), np.delete(quantize_queries(q3), 2, axis=0))


# ---------------------------------------------------------------- QKV projection
def check_projection_brute_force(qkv_projection, rng):
    """Every output element against an explicit sum over the hidden channels
    on a tiny case (loops, not a matmul)."""
    T, C, H, D = 3, 5, 2, 4
    x, w, b = rng.normal(size=(T, C)), rng.normal(size=(3 * H * D, C)), rng.normal(size=3 * H * D)
    q, k, v = qkv_projection(x, w, b, H, D)
    for which, out in enumerate((q, k, v)):
        for t in range(T):
            for h in range(H):
                for d in range(D):
                    o = which * H * D + h * D + d
                    want = b[o]
                    for c in range(C):
                        want += x[t, c] * w[o, c]
                    assert abs(out[t, h, d] - want) <= 1e-12 * (1 + abs(want)), (which, t, h, d)


def check_projection_layout(qkv_projection):
    """A one-hot hidden state picks one column of W: row o = which*H*D + h*D + d
    of W lands in q/k/v[which][., h, d]; a zero state returns the bias."""
    C, H, D = 6, 3, 4
    w = np.arange(3 * H * D * C, dtype=np.float64).reshape(3 * H * D, C)
    for c in range(C):
        x = np.zeros((1, C))
        x[0, c] = 1.0
        q, k, v = qkv_projection(x, w, None, H, D)
        for which, out in enumerate((q, k, v)):
            for h in range(H):
                for d in range(D):
                    assert out[0, h, d] == w[which * H * D + h * D + d, c], (c, which, h, d)
    b = np.arange(3 * H * D, dtype=np.float64) + 0.5
    q, k, v = qkv_projection(np.zeros((2, C)), w, b, H, D)
    assert np.array_equal(np.concatenate([a.reshape(2, -1) for a in (q, k, v)], axis=1), np.tile(b, (2, 1)))


# ---------------------------------------------------------- reference sink
def check_prsink_reference(Ref, token_positions, apply_rope, masked_attention, make_cfg, make_provider):
    """PR-Sink with R reference frames: block m's output equals dense attention
    over [the R reference frames at t = 0..R-1, then every block 0..m with
    frame f of block b at t = R + b * frames + f], masked to the reference
    (always), the hand-derived static and window blocks, the retrieved blocks
    and block m itself; the query sits at t = R + m * frames + f."""
    golden = {int(r[0]): r for r in read_table("prsink_schedule_w3_b8_s1.txt")}
    for R in (1, 2):
        cfg = make_cfg(R)
        prov = make_provider(cfg)
        ref = Ref(cfg, prov)
        F, gh, gw = cfg["frames"], cfg["grid_h"], cfg["grid_w"]
        f, y, x = token_positions(F, gh, gw)
        fr, yr, xr = token_positions(R, gh, gw)
        k_ref, v_ref = prov.reference(0)
        assert k_ref.shape[0] == R * gh * gw
        last = cfg["steps"] - 1
        for m in range(cfg["blocks"]):
            sel = ref.selection(m)
            allowed = set(ids(golden[m][1])) | set(sel) | set(ids(golden[m][3])) | {m}
            ks = [apply_rope(k_ref, fr.astype(np.float64), yr, xr, cfg["rope"])]
            vs = [np.asarray(v_ref, np.float64)]
            keep = [np.ones(k_ref.shape[0], bool)]
            for b in range(m + 1):
                _, k, v = prov.qkv(0, b, last if b < m else 0)
                ks.append(apply_rope(k, R + b * F + f, y, x, cfg["rope"]))
                vs.append(np.asarray(v, np.float64))
                keep.append(np.full(k.shape[0], b in allowed))
            q, _, _ = prov.qkv(0, m, 0)
            qr = apply_rope(q, R + m * F + f, y, x, cfg["rope"])
            keep = np.concatenate(keep)
            mask = np.broadcast_to(keep[None, :], (q.shape[0], keep.size))
            want = masked_attention(qr, np.concatenate(ks), np.concatenate(vs), mask)
            got = ref.attend(m, 0, 0)
            assert np.allclose(got, want, atol=1e-12, rtol=0), (R, m)


# ------------------------------------------------- context-relative positions
def check_prsink_relative(Ref, token_positions, apply_rope, make_cfg, make_provider):
    """PR-Sink with context-relative positions: block m's output equals torch
    SDPA (fp64) over one clip made of the context's frames -- the reference
    frames, then the frames of every context block in stream-id order (the
    hand-derived static and window blocks, the retrieved ones, block m) --
    rotated by plain 3D RoPE at the clip's own frame indices, with the
    queries at the clip's last frames.  The stream must retrieve out of id
    order at least once, so that the order is pinned."""
    import torch
    golden = {int(r[0]): r for r in read_table("prsink_schedule_w3_b8_s1.txt")}
    for R in (0, 1):
        cfg = make_cfg(R)
        prov = make_provider(cfg)
        ref = Ref(cfg, prov)
        F, gh, gw = cfg["frames"], cfg["grid_h"], cfg["grid_w"]
        last = cfg["steps"] - 1
        unordered = 0
        for m in range(cfg["blocks"]):
            sel = ref.selection(m)
            unordered += sel != sorted(sel)
            blocks = sorted(set(ids(golden[m][1])) | set(sel) | set(ids(golden[m][3])) | {m})
            ks, vs = [], []
            if R:
                k_ref, v_ref = prov.reference(0)
                ks.append(np.asarray(k_ref, np.float64))
                vs.append(np.asarray(v_ref, np.float64))
            for b in blocks:
                _, k, v = prov.qkv(0, b, last if b < m else 0)
                ks.append(np.asarray(k, np.float64))
                vs.append(np.asarray(v, np.float64))
            k_clip, v_clip = np.concatenate(ks), np.concatenate(vs)
            n_frames = R + len(blocks) * F
            f, y, x = token_positions(n_frames, gh, gw)
            assert f.size == k_clip.shape[0]
            kr = apply_rope(k_clip, f.astype(np.float64), y, x, cfg["rope"])
            q, _, _ = prov.qkv(0, m, 0)
            nq = q.shape[0]
            qr = apply_rope(np.asarray(q, np.float64), f[-nq:].astype(np.float64), y[-nq:], x[-nq:], cfg["rope"])
            t = lambda a: torch.from_numpy(np.ascontiguousarray(a.transpose(1, 0, 2)))[None]
            want = torch.nn.functional.scaled_dot_product_attention(t(qr), t(kr), t(v_clip))[0].numpy()
            got = ref.attend(m, 0, 0)
            assert np.allclose(got, want.transpose(1, 0, 2), atol=1e-12, rtol=0), (R, m)
        assert unordered > 0


# ------------------------------------------- ConvKV, memory-only position reset
def check_convkv_absolute(Ref, token_positions, apply_rope, make_cfg, make_provider):
    """ConvKV with only the memory's positions restarted.  With one-hot weights
    on the newest tap the memory frame is the newest evicted frame (frame
    3(m-3)-1 overall, for 3-frame blocks and a window of 3), so block m's
    output equals torch SDPA (fp64) over [that raw frame rotated at t = 0,
    the hand-derived window blocks and block m rotated at their absolute
    frame indices b*3 + f], with the queries at m*3 + f.  Before any memory
    exists the output equals the context-relative reading's (the positions
    differ by one shift at most, which RoPE logits do not see)."""
    import torch
    golden = {int(r[0]): r for r in read_table("convkv_schedule_f3_w3_k5_m1.txt")}
    cfg = make_cfg("absolute")
    F, gh, gw, K = cfg["frames"], cfg["grid_h"], cfg["grid_w"], cfg["conv_kernel"]
    assert F == 3 and cfg["window"] == 3 and K == 5 and cfg["memory_frames"] == 1
    Tf = gh * gw
    prov = make_provider(cfg)
    w = np.zeros((cfg["heads"], cfg["head_dim"], K), np.float32)
    w[:, :, K - 1] = 1.0
    prov._w[0] = (w, w)
    ref = Ref(cfg, prov)
    last = cfg["steps"] - 1
    f, y, x = token_positions(F, gh, gw)
    f1, y1, x1 = token_positions(1, gh, gw)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(np.asarray(a, np.float64).transpose(1, 0, 2)))[None]
    for m in range(cfg["blocks"]):
        ks, vs = [], []
        if golden[m][3] != "-":
            newest = ids(golden[m][3])[-1]
            assert newest == 3 * (m - 3) - 1
            b, fr = divmod(newest, F)
            _, k, v = prov.qkv(0, b, last)
            sl = slice(fr * Tf, (fr + 1) * Tf)
            ks.append(apply_rope(np.asarray(k[sl], np.float64), np.zeros(Tf), y1, x1, cfg["rope"]))
            vs.append(np.asarray(v[sl], np.float64))
        for b in ids(golden[m][1]) + [m]:
            _, k, v = prov.qkv(0, b, last if b < m else 0)
            ks.append(apply_rope(np.asarray(k, np.float64), b * F + f, y, x, cfg["rope"]))
            vs.append(np.asarray(v, np.float64))
        q, _, _ = prov.qkv(0, m, 0)
        qr = apply_rope(np.asarray(q, np.float64), m * F + f, y, x, cfg["rope"])
        want = torch.nn.functional.scaled_dot_product_attention(t(qr), t(np.concatenate(ks)),
                                                                t(np.concatenate(vs)))[0].numpy()
        got = ref.attend(m, 0, 0)
        assert np.allclose(got, want.transpose(1, 0, 2), atol=1e-12, rtol=0), m
    cfg_d = make_cfg("default")
    prov_d = make_provider(cfg_d)
    prov_d._w[0] = (w, w)
    ref_d = Ref(cfg_d, prov_d)
    for m in range(5):        # blocks 0-3: the same positions; block 4: all shifted by one block
        assert np.allclose(ref.attend(m, 0, 0), ref_d.attend(m, 0, 0), atol=1e-12, rtol=0), m
    assert not np.allclose(ref.attend(8, 0, 0), ref_d.attend(8, 0, 0), atol=1e-6)


# --------------------------------------------------- pose-aware bank replacement
def check_pose_bank_golden(simulate_pose_bank):
    """Hand-derived table (tests/golden/prsink_pose_bank_w1_b2_s1.txt): window
    1, bank 2, one static block, 2-D poses with exact ties, a zero pose and
    replacements of the newer member."""
    rows = read_table("prsink_pose_bank_w1_b2_s1.txt")
    poses = {int(r[0]): np.array([float(r[1]), float(r[2])], np.float32) for r in rows}
    sim = simulate_pose_bank(len(rows), lambda b: poses[b], 1, 2, 1)
    for r in rows:
        m = int(r[0])
        s = sim[m]
        assert s["static"] == ids(r[3]), (m, s)
        assert s["bank"] == ids(r[4]), (m, s)
        assert s["window"] == ids(r[5]), (m, s)
        assert s["evicted"] == (None if r[6] == "-" else int(r[6])), (m, s)


def check_pose_bank_properties(simulate_pose_bank, prsink_schedule, rng):
    """Random poses: static and window as the FIFO schedule; the bank equals
    the FIFO bank while it has never been full; afterwards it holds exactly B
    distinct blocks that left the window, always including the newest one;
    each replacement removes a member whose cosine to the entering block's
    pose is the largest (fp64 on tie-free data)."""
    for W, B, S in ((3, 4, 1), (1, 1, 0), (2, 5, 1), (3, 2, 1)):
        n = 40
        P = rng.standard_normal((n, 6)).astype(np.float32)
        sim = simulate_pose_bank(n, lambda b: P[b], W, B, S)
        full = False
        for m in range(n):
            s, f = sim[m], prsink_schedule(m, W, B, S)
            assert s["static"] == f["static"] and s["window"] == f["window"] and s["evicted"] == f["evicted"]
            if not full:
                assert s["bank"] == f["bank"], (W, B, S, m)
            full = full or len(s["bank"]) == B
            if full:
                assert len(s["bank"]) == B == len(set(s["bank"]))
                assert all(b < (m - W) for b in s["bank"]) and max(s["bank"]) == m - W - 1
            if m + 1 < n and s["evicted"] is not None and len(s["bank"]) == B:
                gone = set(s["bank"]) - set(sim[m + 1]["bank"])
                assert len(gone) == 1
                e = s["evicted"]
                cos = {b: float(P[b].astype(np.float64) @ P[e] / (np.linalg.norm(P[b].astype(np.float64))
                                                                  * np.linalg.norm(P[e].astype(np.float64))))
                       for b in s["bank"]}
                assert gone.pop() == max(cos, key=cos.get), (W, B, S, m)


# ------------------------------------------------ FP8 keys at stream level
def check_fp8_pow2_invariance(Ref, cfgs, make_provider):
    """FP8 key cache, either policy: multiplying every K by 2^a and every Q by
    2^-a moves each tile's and each row's power-of-two scale but no E4M3 code
    (the conv memory is linear in K), so every output is bit-identical; with
    a = 0 the FP8 output differs from the bf16 reading's (the codes round)."""
    for cfg in cfgs:
        base = make_provider(cfg)

        class Scaled:
            def __init__(self, a):
                self.a = a

            def qkv(self, layer, block, step):
                q, k, v = base.qkv(layer, block, step)
                return (np.asarray(q, np.float64) * 2.0 ** -self.a, np.asarray(k, np.float64) * 2.0 ** self.a,
                        v)

            def pose(self, b):
                return base.pose(b)

            def conv_weights(self, layer):
                return base.conv_weights(layer)

            def reference(self, layer):
                k, v = base.reference(layer)
                return np.asarray(k, np.float64) * 2.0 ** self.a, v

        outs = {}
        for a in (0, 5, -7):
            ref = Ref(cfg, Scaled(a))
            outs[a] = [ref.attend(m, 0, 0) for m in (0, cfg["blocks"] - 1)]
        for a in (5, -7):
            for x, y in zip(outs[0], outs[a]):
                assert np.array_equal(x, y), (cfg["name"], a)
        plain = Ref(dict(cfg, dtype="bf16"), Scaled(0)).attend(cfg["blocks"] - 1, 0, 0)
        assert not np.array_equal(plain, outs[0][1])


# ------------------------------------------------ FP8 attention, hand-worked
def fp8_golden_cfg(dtype):
    """The two-segment stream of golden/fp8_attend_two_segments.txt."""
    from bounded_kv_block_amd import synth
    return synth.workload("prsink_512", dtype=dtype, heads=1, head_dim=4, frames=1, grid_h=1, grid_w=1,
                          window=1, static=1, dynamic_k=0, bank=0, pose_dim=0, rope=(0, 0, 0),
                          softmax_scale=1.0, blocks=2, pose_kind="none")


class Fp8GoldenProvider:
    """Inputs of golden/fp8_attend_two_segments.txt, [1 token, 1 head, 4]."""
    QKV = {0: ((0.0, 0.0, 0.0, 0.0), (0.0, 0.0, 40960.0, 0.0), (0.0, 1.09375, 0.0, 0.0)),
           1: ((1.0, 0.0, 0.0, 0.0), (1.09375, 0.0, 0.0, 0.0), (1.0, 0.0, 0.0, 40960.0))}

    def qkv(self, layer, block, step):
        return tuple(np.array(x, np.float64).reshape(1, 1, 4) for x in self.QKV[block])

    def pose(self, b):
        return np.zeros(0, np.float32)


def check_fp8_attend_golden(Ref):
    """Block 1 of the hand-worked two-segment stream, for the plain bf16
    reading, the FP8 key cache and the FP8 KV cache, equals the hand-derived
    values to 1e-13 (relative)."""
    rows = {r[0]: [float(x) for x in r[1:]] for r in read_table("fp8_attend_two_segments.txt")}
    for dtype in ("bf16", "bf16_fp8k", "bf16_fp8kv"):
        ref = Ref(fp8_golden_cfg(dtype), Fp8GoldenProvider())
        got = ref.attend(1, 0, 0)[0, 0]
        want = np.array(rows[dtype])
        assert np.allclose(got, want, rtol=1e-13, atol=1e-13), (dtype, got, want)


# ------------------------------------------------ token layout
def check_token_positions(token_positions):
    """(frame, y, x) of each token of a 2-frame 2x3 block against the hand table."""
    rows = read_table("token_positions_f2_h2_w3.txt")
    f, y, x = token_positions(2, 2, 3)
    assert len(f) == len(rows)
    for tok, ff, yy, xx in rows:
        t = int(tok)
        assert (int(f[t]), int(y[t]), int(x[t])) == (int(ff), int(yy), int(xx)), tok


# ------------------------------------------------ bf16 rounding of the projection
def check_bf16_round(bf16_round, rng):
    """Nearest bf16, ties to even: hand values (ties at 1 + 2^-8 and 1 + 3*2^-8,
    negative ties, a carry into the next binade, small and large magnitudes)
    and torch's float32 -> bfloat16 conversion on random fp32 values (exact
    in fp64, so no double rounding)."""
    import torch
    hand = [(1 + 2.0 ** -8, 1.0), (1 + 3 * 2.0 ** -8, 1 + 2.0 ** -6), (-(1 + 2.0 ** -8), -1.0),
            (1 + 2.0 ** -8 + 2.0 ** -30, 1 + 2.0 ** -7), (2 - 2.0 ** -9, 2.0), (3.0 * 2.0 ** -100, 3.0 * 2.0 ** -100),
            (1.0 + 2.0 ** -7, 1.0 + 2.0 ** -7), (0.0, 0.0), (255.5, 256.0), (-1000.1, -1000.0)]
    for x, want in hand:
        assert float(bf16_round(np.array([x]))[0]) == want, (x, want)
    x = (rng.standard_normal(50000) * np.exp(rng.uniform(-20, 20, 50000))).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    assert np.array_equal(bf16_round(x.astype(np.float64)), want)


def check_fp8_pv_row_scale(attention_fp8_pv):
    """P of one query row with base-2 logits 0, -7.5, -12 against keys whose
    values are the unit vectors: P = 1, 2^-7.5 = 0.0055243, 2^-12.  The row's
    scale is 2^-8 (largest P = 1): 256 P = 256 (exact), 1.41421 (binade
    [1, 2), quantum 1/8: 11.31 -> 11 -> 1.375), 2^-4 (exact, a normal
    value).  So o = (1, 1.375/256, 0.0625/256) / (1 + 2^-7.5 + 2^-12).
    (At unit scale 2^-7.5 would be a subnormal, 3 * 2^-9, and 2^-12 would
    round to 0.)"""
    q = np.ones((1, 1, 1))
    k = np.array([0.0, -7.5, -12.0]).reshape(3, 1, 1)
    v = np.eye(3).reshape(3, 1, 3)
    l = 1.0 + 2.0 ** -7.5 + 2.0 ** -12
    want = np.array([1.0, 1.375 / 256.0, 0.0625 / 256.0]) / l
    got = attention_fp8_pv(q, k, v)[0, 0]
    assert np.allclose(got, want, rtol=1e-14, atol=0), (got, want)


def check_convkv_memory_cached_dtype(Ref, conv_memory, bf16_round, make_cfg, make_provider):
    """The ConvKV memory frame as the cache holds it: for a bf16 cache, the
    exact conv output (``conv_memory`` of the evicted raw frames, assembled
    here by hand from the provider) rounded to bf16 -- values that bf16
    represents and that differ from the exact output; for the fp32 cache, the
    exact output itself."""
    for dtype in ("bf16", "f32"):
        cfg = make_cfg(dtype)
        prov = make_provider(cfg)
        ref = Ref(cfg, prov)
        m = cfg["blocks"] - 1
        mk, mv = ref.memory(m, 0, [0, 1])
        F, Tf = cfg["frames"], cfg["grid_h"] * cfg["grid_w"]
        frames = ref.schedule(m)["memory"][0]
        wk, wv = (np.asarray(w, np.float64)[[0, 1]] for w in prov.conv_weights(0))
        fk = np.stack([np.asarray(prov.qkv(0, e // F, cfg["steps"] - 1)[1], np.float64)[(e % F) * Tf:(e % F + 1) * Tf][:, [0, 1]]
                       for e in frames]).transpose(0, 2, 1, 3)
        exact = conv_memory(fk, wk)[0].transpose(1, 0, 2)
        if dtype == "bf16":
            assert np.array_equal(mk[0], bf16_round(exact)) and not np.array_equal(mk[0], exact)
            assert np.array_equal(bf16_round(mv[0]), mv[0])
        else:
            assert np.array_equal(mk[0], exact)


def check_fp8_pv_slack(slack_fn, pv_fn):
    """How far an FP8-KV output may move where the FP8 product's rounding
    decides a P code (``slack_fn(q, k, v, rel) -> (o, slack)``), worked by
    hand.

    One query row, base-2 logits z = (8, log2 248, 4) through q = (1), value
    rows the unit vectors.  The largest P is 256, so the row's scale is 2^0
    and p = (256, 248, 16).  256 and 16 are codes, their neighbouring rounding
    boundaries 248/272 and 15.5/17 at least 1.5% away; 248 is itself the
    boundary between the codes 240 and 256 (fp64's 2^log2(248) may land a
    hair either side).  With any rel > 0 the middle key's P has both codes,
    one step of 16 apart, so slack = (0, 16, 0) / (256 + p1 + 16) and o is
    (256, 240 or 256, 16) / l; with rel = 0 every slack is zero and o is
    ``pv_fn``'s.

    The bound grows with sum_i |q_i k_i|, not with |z|: q = (1, 1) and
    k = (z + 10, -10) give the same z = log2(1.01 * 248) (P 1% above the
    boundary, 250.48, which rounds to 256) but sum |q k| = |z| + 20.  The
    other code needs a bound of log2(1.01) = 0.01436 in z: rel = 7e-4 gives
    7e-4 (7.97 + 20) = 0.0196 (slack), while 7e-4 |z| = 0.0056 would not.

    Channels weigh |v|: a value row (-1, 2) gives slack step * (1, 2) / l."""
    q = np.ones((1, 1, 1))
    z = np.array([8.0, np.log2(248.0), 4.0])
    k = z.reshape(3, 1, 1)
    v = np.eye(3).reshape(3, 1, 3)
    p1 = float(np.exp2(z[1]))
    assert abs(p1 - 248.0) < 1e-12
    l = 256.0 + p1 + 16.0
    o, s = slack_fn(q, k, v, 2.0 ** -14)
    assert np.allclose(s[0, 0], [0.0, 16.0 / l, 0.0], rtol=1e-14, atol=0), s
    assert np.isclose(o[0, 0, 0], 256.0 / l, rtol=1e-14) and np.isclose(o[0, 0, 2], 16.0 / l, rtol=1e-14), o
    assert min(abs(o[0, 0, 1] - 240.0 / l), abs(o[0, 0, 1] - 256.0 / l)) < 1e-15, o
    o0, s0 = slack_fn(q, k, v, 0.0)
    assert np.all(s0 == 0.0) and np.allclose(o0, pv_fn(q, k, v), rtol=1e-15, atol=0)

    zt = float(np.log2(1.01 * 248.0))
    q2 = np.ones((1, 1, 2))
    k2 = np.array([[zt + 10.0, -10.0], [0.0, 0.0]]).reshape(2, 1, 2)     # second key: z = 0, P = 1
    v2 = np.array([[-1.0, 2.0], [0.0, 0.0]]).reshape(2, 1, 2)
    P = np.array([2.0 ** zt, 1.0])
    l2 = P.sum()                                                      # scale 2^0: p = P
    _, s_small = slack_fn(q2, k2, v2, 1e-4)                           # 1e-4 * 27.97 = 0.0028 < 0.01436
    assert np.all(s_small == 0.0), s_small
    _, s_mid = slack_fn(q2, k2, v2, 7e-4)
    assert np.allclose(s_mid[0, 0], np.array([1.0, 2.0]) * 16.0 / l2, rtol=1e-12, atol=0), s_mid
