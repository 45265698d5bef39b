"""GPU parity of the fused QKV projection path (bkv_attend_qkv) against the
CPU oracle: q, k, v are the oracle's fp64 projection x W^T + b of the same
bf16 hidden states and weights, rounded to bf16 where the unfused path
receives its bf16 inputs, fed to the same stream references.  Outputs
within max-abs 2e-2; the stored K (rotated) and V within bf16 rounding of
the oracle's."""
import numpy as np
import pytest

import oracle
from bounded_kv_block_amd import synth
from gpu_helpers import TOL, Run, max_err, oracle_err

pytestmark = pytest.mark.gpu


class QkvRun(Run):
    """A stream driven through bkv_attend_qkv.  The oracle provider's qkv() is
    the oracle's projection of the same hidden states (only `heads` filled,
    the rest zero: the references read only the heads they are asked for)."""

    def __init__(self, cfg, host_inputs=True, heads=None, bias=True):
        super().__init__(cfg, host_inputs)
        torch = self.torch
        H, D = cfg["heads"], cfg["head_dim"]
        self.heads = list(range(H)) if heads is None else list(heads)
        self._x_dev, self._x_host = {}, {}
        self._pw = {}
        for l in range(cfg["layers"]):
            if host_inputs:
                w, b = synth.qkv_weights(cfg, l)
                wd = torch.from_numpy(w).to(self.device).to(torch.bfloat16)
                bd = torch.from_numpy(b).to(self.device).to(torch.bfloat16)
            else:
                wd, bd = synth.qkv_weights_device(cfg, l, self.device)
            w64 = wd.float().cpu().numpy().astype(np.float64)
            b64 = bd.float().cpu().numpy().astype(np.float64)
            rows = np.concatenate([np.arange(i * H * D + h * D, i * H * D + (h + 1) * D)
                                   for i in range(3) for h in self.heads])
            self._pw[l] = (wd, bd if bias else None, w64[rows], b64[rows] if bias else None)

    def x_dev(self, layer, block, step):
        key = (layer, block, step)
        if key not in self._x_dev:
            if self.host_inputs:
                x = synth.hidden(self.cfg, layer, block, step)
                self._x_dev[key] = self.torch.from_numpy(x).to(self.device).to(self.torch.bfloat16)
            else:
                self._x_dev[key] = synth.hidden_device(self.cfg, layer, block, step, self.device)
        return self._x_dev[key]

    def qkv(self, layer, block, step):
        key = (layer, block, step)
        if key not in self._host:
            H, D = self.cfg["heads"], self.cfg["head_dim"]
            x = self.x_dev(layer, block, step).float().cpu().numpy()
            _, _, wsel, bsel = self._pw[layer]
            # q, k and v leave the projection in bf16, where the unfused path
            # receives its bf16 inputs
            parts = oracle.qkv_projection(x, wsel, bsel, len(self.heads), D, round_bf16=True)
            full = []
            for i, p in enumerate(parts):
                a = np.zeros((x.shape[0], H, D))
                a[:, self.heads, :] = p
                full.append(a)
            self._host[key] = tuple(full)
        return self._host[key]

    def attend(self, m, layer, step):
        wd, bd, _, _ = self._pw[layer]
        return self.cache.attend_qkv(layer, self.x_dev(layer, m, step), wd, bd)

    def drop(self, keep_blocks):
        for key in list(self._x_dev):
            if key[1] not in keep_blocks:
                del self._x_dev[key]


def _stream(cfg, run, check=None, heads=None, rows=None, export=False):
    Ref = oracle.ConvKVReference if cfg["mode"] == "convkv" else oracle.PRSinkReference
    ref = Ref(cfg, run)
    worst = 0.0
    for m in range(cfg["blocks"]):
        run.open(m)
        if cfg["mode"] == "convkv":
            out = run.attend(m, 0, 0)
            want = (lambda **kw: ref.attend(m, 0, 0, heads=heads, **kw)) if check is None or m in check else None
        else:
            sel = ref.selection(m)
            assert run.cache.selection() == sel, m
            out = run.attend(m, 0, 0)
            want = ((lambda **kw: ref.attend(m, 0, 0, heads=heads, selection=sel, **kw))
                    if check is None or m in check else None)
        if want is not None:
            err = oracle_err(out, want, heads, rows, TOL["bf16"])
            worst = max(worst, err)
            print(f"block {m}: max|err| {err:.3e}", flush=True)
            assert err <= TOL["bf16"], (m, err)
        if export and cfg["mode"] != "convkv":
            kv = ref.context_kv(m, 0, 0, run.heads, ref.selection(m))
            for i, (_, _, kr, v) in enumerate(kv):
                gk, gv = run.cache.export_segment(0, i)
                gk = gk.float().cpu().numpy()[:, run.heads]
                gv = gv.float().cpu().numpy()[:, run.heads]
                # Half an ulp of the stored rotated value (2^-8 |K~|), plus the
                # projection's own bf16 rounding: where the fp32 and fp64 sums
                # straddle a rounding boundary, each input of a RoPE pair may
                # differ by one ulp (up to 2^-7 of it), which the orthonormal
                # rotation carries over as at most sqrt(2) 2^-7 of the pair's
                # norm; such straddles are rare.
                pn = np.sqrt(kr ** 2 + kr.reshape(*kr.shape[:-1], -1, 2)[..., ::-1].reshape(kr.shape) ** 2)
                d = np.abs(gk - kr)
                assert np.all(d <= 2.0 ** -8 * np.abs(kr) + np.sqrt(2.0) * 2.0 ** -7 * pn + 1e-3), (m, i)
                assert np.mean(d > 2.0 ** -8 * np.abs(kr) + 1e-3) < 1e-2, (m, i)
                # V: both sides round the projection to bf16; where the fp32
                # and fp64 sums straddle a boundary they differ by one ulp
                assert np.all(np.abs(gv - v) <= 2.0 ** -7 * np.abs(v) + 1e-3), (m, i)
                assert np.mean(gv != v) < 1e-2, (m, i)
        run.cache.commit()
        if not run.host_inputs:
            run.drop(set(range(m - 70, m + 2)))
            run._host.clear()                 # oracle projections are recomputed when needed
    return worst


def test_qkv_small_ragged_with_export():
    """3 heads (3*3*128 = 1152 projected features: 4.5 feature tiles of 256),
    3 frames of 6x10 = 180 tokens (one partial token tile), model_dim 256,
    bias, RoPE 44/42/42, top-2 over a bank of 4, 12 blocks: every output, and
    the stored K and V of every context segment."""
    cfg = synth.workload("prsink_512_qkv", heads=3, grid_h=6, grid_w=10, bank=4, blocks=12, pose_dim=16,
                         keyframes=5, model_dim=256)
    _stream(cfg, QkvRun(cfg), export=True)


def test_qkv_odd_width_no_bias_single_token():
    """model_dim 96 (three 32-channel steps, fewer than the pipeline depth),
    no bias, one-token blocks."""
    cfg = synth.workload("prsink_512_qkv", heads=2, frames=1, grid_h=1, grid_w=1, bank=3, blocks=9,
                         pose_dim=8, keyframes=3, model_dim=96)
    _stream(cfg, QkvRun(cfg, bias=False))
    cfg = synth.workload("prsink_512_qkv", heads=2, grid_h=4, grid_w=10, bank=3, blocks=8,
                         pose_dim=16, keyframes=4, model_dim=32)
    _stream(cfg, QkvRun(cfg, bias=False))


def test_qkv_convkv_small():
    """ConvKV through the fused path: the epilogue writes raw K to the slot and
    K rotated at context positions into the context buffer; 8 blocks (the
    memory frame appears at block 5)."""
    cfg = synth.workload("convkv_512", heads=2, grid_h=4, grid_w=6, blocks=8, model_dim=128)
    run = QkvRun(cfg)
    _stream(cfg, run)
    assert run.cache.stats()["memory_count"] == 1


def test_qkv_prsink_512_full_shape_sampled():
    """512x512 shapes at full size with model_dim 5120 (x [3072, 5120], W
    [15360, 5120]): indices on every block, outputs of heads 0 and 39 on
    sampled rows of blocks 0 and 7."""
    cfg = synth.workload("prsink_512_qkv", blocks=8)
    heads = [0, 39]
    run = QkvRun(cfg, host_inputs=False, heads=heads)
    _stream(cfg, run, check={0, 7}, heads=heads, rows=np.r_[0:64, 1500:1532, 3008:3072])


# ---- the fused path with the FP8 key cache (K quantised in the epilogue)
def test_qkv_fp8k_small_ragged():
    """FP8 keys from the projection's epilogue: 3 heads, 180-token blocks (a
    ragged last token tile, whose clamped rows must not enter the tile's
    scale), model_dim 256, bias, 12 blocks: every output."""
    cfg = synth.workload("prsink_512_qkv", dtype="bf16_fp8k", heads=3, grid_h=6, grid_w=10, bank=4, blocks=12,
                         pose_dim=16, keyframes=5, model_dim=256)
    _stream_fp8(cfg, QkvRun(cfg))


def test_qkv_fp8k_convkv_small():
    """ConvKV with FP8 keys through the fused path: raw K to the slot, E4M3
    K~ into the context buffer; 8 blocks (memory from block 5)."""
    cfg = synth.workload("convkv_512", dtype="bf16_fp8k", heads=2, grid_h=4, grid_w=6, blocks=8, model_dim=128)
    _stream_fp8(cfg, QkvRun(cfg))


def test_qkv_fp8k_prsink_512_full_shape_sampled():
    cfg = synth.workload("prsink_512_qkv", dtype="bf16_fp8k", blocks=8)
    heads = [0, 39]
    _stream_fp8(cfg, QkvRun(cfg, host_inputs=False, heads=heads), check={0, 7}, heads=heads,
                rows=np.r_[0:64, 1500:1532, 3008:3072])


def _stream_fp8(cfg, run, check=None, heads=None, rows=None):
    Ref = oracle.ConvKVReference if cfg["mode"] == "convkv" else oracle.PRSinkReference
    ref = Ref(cfg, run)
    for m in range(cfg["blocks"]):
        run.open(m)
        sel = None if cfg["mode"] == "convkv" else ref.selection(m)
        if sel is not None:
            assert run.cache.selection() == sel, m
        out = run.attend(m, 0, 0)
        if check is None or m in check:
            want = ((lambda **kw: ref.attend(m, 0, 0, heads=heads, **kw)) if sel is None
                    else (lambda **kw: ref.attend(m, 0, 0, heads=heads, selection=sel, **kw)))
            err = oracle_err(out, want, heads, rows, TOL["bf16_fp8k"])
            print(f"block {m}: max|err| {err:.3e}", flush=True)
            assert err <= TOL["bf16_fp8k"], (m, err)
        run.cache.commit()
        if not run.host_inputs:
            run.drop(set(range(m - 70, m + 2)))
            run._host.clear()


# ---- the fused path with the FP8 KV cache (K and V quantised in the epilogue)
def test_qkv_fp8kv_small_ragged():
    """FP8 K and V from the projection's epilogue: 3 heads, 180-token blocks
    (a ragged last token tile, whose clamped rows must not enter either tile
    scale), model_dim 256, bias, 12 blocks: every output."""
    cfg = synth.workload("prsink_512_qkv", dtype="bf16_fp8kv", heads=3, grid_h=6, grid_w=10, bank=4, blocks=12,
                         pose_dim=16, keyframes=5, model_dim=256)
    _stream_fp8(cfg, QkvRun(cfg))


def test_qkv_fp8kv_convkv_small():
    """ConvKV with the FP8 KV cache through the fused path: raw K and V^T to
    the slot (the conv reads them), E4M3 V^T beside them, E4M3 K~ into the
    context buffer; 8 blocks (memory from block 5)."""
    cfg = synth.workload("convkv_512", dtype="bf16_fp8kv", heads=2, grid_h=4, grid_w=6, blocks=8, model_dim=128)
    _stream_fp8(cfg, QkvRun(cfg))


# ---- tile edges of the projection: 256 tokens x 256 features per workgroup,
# 32 channels per step, four steps in flight
@pytest.mark.parametrize("dtype,mode,heads,tokens,model_dim,bias", [
    ("bf16", "pr_sink", 1, (1, 1, 257), 160, True),        # 1.5 feature tiles; a 1-row token tile; 5 steps
    ("bf16_fp8k", "pr_sink", 5, (1, 16, 16), 288, False),  # 7.5 feature tiles; exactly one token tile; 9 steps
    ("bf16_fp8kv", "pr_sink", 1, (1, 5, 13), 64, True),    # 65 tokens; 2 steps
    ("bf16", "convkv", 5, (1, 1, 257), 96, False),
    ("bf16_fp8k", "convkv", 1, (2, 8, 8), 160, True),
    ("bf16_fp8kv", "convkv", 3, (1, 16, 16), 288, True),
], ids=["bf16-prsink-H1-T257-C160", "fp8k-prsink-H5-T256-C288", "fp8kv-prsink-H1-T65-C64",
        "bf16-convkv-H5-T257-C96", "fp8k-convkv-H1-T128-C160", "fp8kv-convkv-H3-T256-C288"])
def test_qkv_tile_edges(dtype, mode, heads, tokens, model_dim, bias):
    """Every output of every block, on shapes at the projection's tile edges."""
    frames, gh, gw = tokens
    if mode == "pr_sink":
        cfg = synth.workload("prsink_512_qkv", dtype=dtype, heads=heads, frames=frames, grid_h=gh, grid_w=gw,
                             bank=3, blocks=9, pose_dim=8, keyframes=3, model_dim=model_dim)
    else:
        cfg = synth.workload("convkv_512", dtype=dtype, heads=heads, frames=frames, grid_h=gh, grid_w=gw,
                             blocks=10, model_dim=model_dim)
    run = QkvRun(cfg, bias=bias)
    if dtype == "bf16":
        worst = _stream(cfg, run)
    else:
        _stream_fp8(cfg, run)
        worst = None
    if mode == "convkv":
        assert run.cache.stats()["memory_count"] >= 1
    print("worst", worst, flush=True)
