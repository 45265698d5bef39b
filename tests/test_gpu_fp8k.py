"""GPU parity of the FP8 key cache (PR-Sink, dtype "bf16_fp8k") through the
C-ABI against the CPU oracle.

Retrieval indices exact; the stored keys equal the oracle's E4M3
quantisation (value codes and per-tile scales) except where the rotated key
lies on a rounding tie within the fp32-vs-fp64 rotation error; attention
outputs within max-abs 2e-2 of the fp64 oracle (which quantises Q and K the
same way); power-of-two rescalings of Q and K that cancel leave the output
bit-identical."""
import numpy as np
import pytest

import oracle
from bounded_kv_block_amd import synth
from gpu_helpers import TOL, Run, max_err

pytestmark = pytest.mark.gpu


def _stream(cfg, run=None, check=None, heads=None, rows=None, host_inputs=True):
    run = run or Run(cfg, host_inputs)
    ref = oracle.PRSinkReference(cfg, run)
    outs = []
    for m in range(cfg["blocks"]):
        run.open(m)
        sel = ref.selection(m)
        assert run.cache.selection() == sel, m
        out = run.attend(m, 0, 0)
        if check is None or m in check:
            want = ref.attend(m, 0, 0, heads=heads, rows=rows, selection=sel)
            err = max_err(out, want, heads, rows)
            print(f"block {m}: max|err| {err:.3e}", flush=True)
            assert err <= TOL["bf16_fp8k"], (m, err)
        outs.append(out)
        run.cache.commit()
        if not host_inputs:
            run.drop(set(range(m - 70, m + 2)))
    return run, outs


def test_fp8k_small_ragged():
    """3 heads, 3 frames of 6x10 = 180 tokens (two full 64-key tiles and a
    52-key tail per segment, a ragged query tile), RoPE 44/42/42, top-2 over
    a bank of 4, 14 blocks: every output of every block."""
    cfg = synth.workload("prsink_512_fp8k", heads=3, grid_h=6, grid_w=10, bank=4, blocks=14,
                         pose_dim=16, keyframes=5)
    _stream(cfg)


def test_fp8k_single_token_blocks():
    """Degenerate blocks of one token: one key per segment, one query."""
    cfg = synth.workload("prsink_512_fp8k", heads=2, frames=1, grid_h=1, grid_w=1, bank=3, blocks=10,
                         pose_dim=8, keyframes=3)
    _stream(cfg)


def test_fp8k_multistep_multilayer():
    """2 layers x 3 steps per block; the cache keeps each layer's last-step K."""
    cfg = synth.workload("prsink_512_fp8k", heads=2, grid_h=4, grid_w=10, bank=3, blocks=8, pose_dim=16,
                         keyframes=4, layers=2, steps=3)
    run = Run(cfg)
    ref = oracle.PRSinkReference(cfg, run)
    for m in range(cfg["blocks"]):
        run.open(m)
        sel = ref.selection(m)
        assert run.cache.selection() == sel
        for s in range(3):
            for l in range(2):
                out = run.attend(m, l, s)
                err = max_err(out, ref.attend(m, l, s, selection=sel))
                assert err <= TOL["bf16_fp8k"], (m, l, s, err)
        run.cache.commit()


def _e4m3_quantum(y):
    a = np.abs(y)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a >= 2.0 ** -6, 2.0 ** (e - 3), 2.0 ** -9)


def test_fp8k_stored_keys_match_oracle_quantisation():
    """Every context segment's stored K, dequantised (E4M3 code x 2^e, exact
    in bf16), against the oracle's quantisation of the fp64-rotated keys.  An
    element may differ only by one E4M3 step, and only where the scaled
    rotated key sits within 1e-4 of a quantum of a rounding tie (the kernel
    rotates in fp32).  V is stored exactly."""
    cfg = synth.workload("prsink_512_fp8k", heads=2, grid_h=6, grid_w=10, bank=4, blocks=9, pose_dim=16,
                         keyframes=4)
    run = Run(cfg)
    ref = oracle.PRSinkReference(cfg, run)
    n_total = n_tie = 0
    for m in range(cfg["blocks"]):
        run.open(m)
        run.attend(m, 0, 0)
        kv = ref.context_kv(m, 0, 0, [0, 1], ref.selection(m))
        for i, (_, _, kr, v) in enumerate(kv):
            gk, gv = run.cache.export_segment(0, i)
            got = gk.float().cpu().numpy().astype(np.float64)
            want = oracle.fp8.quantize_keys(kr)
            T = kr.shape[0]
            nt = (T + 63) // 64
            pad = np.zeros((nt * 64,) + kr.shape[1:])
            pad[:T] = kr
            amax = np.abs(pad).reshape(nt, 64, *kr.shape[1:]).max(axis=(1, 3))
            sc = np.repeat(np.ldexp(1.0, oracle.fp8.pow2_exponents(amax)), 64, axis=0)[:T][:, :, None]
            y = kr / sc
            q = _e4m3_quantum(y)
            frac = np.abs(y) / q - np.floor(np.abs(y) / q)
            near_tie = np.abs(frac - 0.5) < 1e-4
            diff = got != want
            assert np.all(near_tie[diff]), (m, i, int(diff.sum()))
            assert np.all(np.abs(got - want)[diff] <= (q * sc * (1 + 1e-12))[diff]), (m, i)
            n_total += diff.size
            n_tie += int(diff.sum())
            assert np.array_equal(gv.float().cpu().numpy(), v), (m, i)
        run.cache.commit()
    assert n_tie <= 1e-3 * n_total


class _Rescaled(Run):
    """Inputs of the stream with Q x 2^-s and K x 2^s (exact in bf16); block
    `zero_k` gets K = 0 and its first 5 query rows Q = 0 when given."""

    def __init__(self, cfg, s, zero_k=None):
        super().__init__(cfg, host_inputs=True)
        self.s, self.zero_k = s, zero_k

    def qkv(self, layer, block, step):
        q, k, v = super().qkv(layer, block, step)
        q = q * np.float32(2.0 ** -self.s)
        k = k * np.float32(2.0 ** self.s)
        if block == self.zero_k:
            q = q.copy()
            q[:5] = 0
            k = np.zeros_like(k)
        return q, k, v

    def qkv_dev(self, layer, block, step):
        key = (layer, block, step)
        if key not in self._dev:
            self._dev[key] = tuple(self.torch.from_numpy(np.ascontiguousarray(a)).to(self.device).to(self.dt)
                                   for a in self.qkv(layer, block, step))
        return self._dev[key]


def test_fp8k_power_of_two_rescaling_and_zero_keys():
    """Scales far from 1 on both operands (K x 2^25, Q x 2^-25 and K x 2^-40,
    Q x 2^40) move every tile and row exponent but no E4M3 code, so the
    outputs equal the unscaled stream's bit for bit; a block whose K is all
    zero (exponent 0, every code 0) and whose first query rows are zero is
    checked against the oracle on every block."""
    cfg = synth.workload("prsink_512_fp8k", heads=2, grid_h=6, grid_w=10, bank=4, blocks=8, pose_dim=16,
                         keyframes=4)
    _, base = _stream(cfg, run=_Rescaled(cfg, 0), check={0, 7})
    for s in (25, -40):
        _, outs = _stream(cfg, run=_Rescaled(cfg, s), check={7})
        for m, (a, b) in enumerate(zip(base, outs)):
            assert bool((a == b).all()), (s, m)
    _stream(cfg, run=_Rescaled(cfg, 0, zero_k=3))


def test_fp8k_prsink_512_full_shape_sampled():
    """512x512 shapes at full size (40 x 128, 3072 queries, 21504 keys once
    warm) with the FP8 key cache: indices on every block, outputs sampled (2
    heads, 160 query rows incl. the last) on blocks 0, 4, 6, 9."""
    cfg = synth.workload("prsink_512_fp8k", blocks=10)
    run, _ = _stream(cfg, host_inputs=False, check={0, 4, 6, 9}, heads=[0, 39],
                     rows=np.r_[0:64, 1500:1532, 3008:3072])
    assert run.cache.stats()["split_attends"] == 0


def test_fp8k_split_launch_key_parts():
    """1800-query blocks, 40 heads: the split launch (one full round, then the
    64 remainder units cut into 4 key parts) with the FP8 key cache."""
    cfg = synth.workload("prsink_512_fp8k", frames=2, grid_h=30, grid_w=30, blocks=8)
    run, _ = _stream(cfg, host_inputs=False, check={0, 4, 7}, heads=[0, 33, 39],
                     rows=np.r_[0:64, 900:964, 1736:1800])
    assert run.cache.stats()["split_attends"] == cfg["blocks"]


# ---- FP8 keys in a context gathered per block (ConvKV, context-relative PR-Sink)
def _check_stored_keys(run, kv, layer=0):
    """Every segment's stored K (E4M3 x 2^e, exact in bf16) against the
    oracle's quantisation of its rotated K, one E4M3 step apart at most and
    only at rounding ties within the fp32-vs-fp64 rotation error (for memory
    frames, whose raw K the oracle holds bf16-rounded as the cache does, within a
    bf16 step of the fp32-vs-fp64 conv sum: 2^-4 of an E4M3 step); V exact
    up to bf16 storage of the conv memory."""
    n_total = n_tie = 0
    for i, (kind, _, kr, v) in enumerate(kv):
        gk, gv = run.cache.export_segment(layer, i)
        got = gk.float().cpu().numpy().astype(np.float64)
        want = oracle.fp8.quantize_keys(kr)
        T = kr.shape[0]
        nt = (T + 63) // 64
        pad = np.zeros((nt * 64,) + kr.shape[1:])
        pad[:T] = kr
        amax = np.abs(pad).reshape(nt, 64, *kr.shape[1:]).max(axis=(1, 3))
        sc = np.repeat(np.ldexp(1.0, oracle.fp8.pow2_exponents(amax)), 64, axis=0)[:T][:, :, None]
        y = kr / sc
        q = _e4m3_quantum(y)
        frac = np.abs(y) / q - np.floor(np.abs(y) / q)
        near_tie = np.abs(frac - 0.5) < (2.0 ** -4 if kind == "memory" else 1e-4)
        diff = got != want
        assert np.all(near_tie[diff]), (i, kind, int(diff.sum()))
        assert np.all(np.abs(got - want)[diff] <= (q * sc * (1 + 1e-12))[diff]), (i, kind)
        n_total += diff.size
        n_tie += int(diff.sum())
        gv = gv.float().cpu().numpy().astype(np.float64)
        if kind == "memory":
            assert np.max(np.abs(gv - v)) <= 2.0 ** -7 * np.max(np.abs(v)) + 1e-6, (i, kind)
        else:
            assert np.array_equal(gv, v), (i, kind)
    return n_total, n_tie


def _convkv_stream(cfg, check=None, heads=None, rows=None, host_inputs=True, keys=False):
    run = Run(cfg, host_inputs)
    ref = oracle.ConvKVReference(cfg, run)
    n_total = n_tie = 0
    for m in range(cfg["blocks"]):
        run.open(m)
        assert run.cache.context() == ref.context(m), m
        out = run.attend(m, 0, 0)
        if check is None or m in check:
            err = max_err(out, ref.attend(m, 0, 0, heads=heads, rows=rows), heads, rows)
            print(f"block {m}: max|err| {err:.3e}", flush=True)
            assert err <= TOL["bf16_fp8k"], (m, err)
        if keys:
            a, b = _check_stored_keys(run, ref.context_kv(m, 0, 0, list(range(cfg["heads"]))))
            n_total += a
            n_tie += b
        run.cache.commit()
        if not host_inputs:
            run.drop(set(range(m - 8, m + 2)))
    assert n_tie <= 1e-3 * max(n_total, 1)
    return run


def test_fp8k_convkv_small_ragged_with_keys():
    """ConvKV with the FP8 key cache: 2 heads, 3 frames of 4x6 (a 24-token
    memory frame and 72-token blocks: a partial tile in every segment), 12
    blocks; every output, and every segment's stored E4M3 keys and V."""
    cfg = synth.workload("convkv_512", dtype="bf16_fp8k", heads=2, grid_h=4, grid_w=6, blocks=12)
    run = _convkv_stream(cfg, keys=True)
    assert run.cache.stats()["memory_count"] == 1


def test_fp8k_convkv_memory_only_reset_two_memory_frames():
    """The memory-only position reset (window and current absolute) with two
    memory frames of 6x10 tokens and FP8 keys, 16 blocks."""
    cfg = synth.workload("convkv_512_abs", dtype="bf16_fp8k", heads=2, grid_h=6, grid_w=10, frames=2,
                         memory_frames=2, blocks=16)
    _convkv_stream(cfg, keys=True)


def test_fp8k_relative_prsink_with_keys():
    """Context-relative PR-Sink with FP8 keys and one reference frame: the
    gather quantises the re-rotated context per segment, retrieved blocks
    included; indices, positions, outputs and stored keys on 14 blocks."""
    cfg = synth.workload("prsink_512_fp8k", heads=2, grid_h=6, grid_w=10, bank=4, blocks=14, pose_dim=16,
                         keyframes=5, positions="relative", reference_frames=1)
    run = Run(cfg)
    ref = oracle.PRSinkReference(cfg, run)
    for m in range(cfg["blocks"]):
        run.open(m)
        sel = ref.selection(m)
        assert run.cache.selection() == sel, m
        assert run.cache.context() == ref.context(m, sel), m
        out = run.attend(m, 0, 0)
        err = max_err(out, ref.attend(m, 0, 0, selection=sel))
        assert err <= TOL["bf16_fp8k"], (m, err)
        _check_stored_keys(run, ref.context_kv(m, 0, 0, [0, 1], sel))
        run.cache.commit()


def test_fp8k_convkv_512_full_shape_sampled():
    """ConvKV 512x512 at full size with FP8 keys (13312 keys once warm, the
    1024-token memory frame quantised in 16 tiles): outputs of 2 heads on
    sampled rows of blocks 0, 4, 5 and 11."""
    cfg = synth.workload("convkv_512", dtype="bf16_fp8k", blocks=12)
    _convkv_stream(cfg, host_inputs=False, check={0, 4, 5, 11}, heads=[0, 21],
                   rows=np.r_[0:64, 1500:1532, 3008:3072])
