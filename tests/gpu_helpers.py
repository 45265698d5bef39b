"""Helpers for the GPU tests: drive a bkv.Cache over a seeded workload and hand
the very same inputs to the oracle."""
from __future__ import annotations

import numpy as np

from bounded_kv_block_amd import bkv, synth

TOL = {"f32": 1e-5, "bf16": 2e-2, "bf16_fp8k": 2e-2, "bf16_fp8kv": 2e-2}


class Run:
    """A stream on the GPU plus an oracle provider over the same inputs.

    host_inputs=True draws Q/K/V with the numpy generator and copies them to
    the device; otherwise they are drawn on the device (large shapes) and
    copied back for the oracle on demand.
    """

    def __init__(self, cfg: dict, host_inputs: bool = True, device="cuda"):
        import torch
        self.torch = torch
        self.cfg = cfg
        self.host_inputs = host_inputs
        self.device = torch.device(device)
        self.cache = bkv.Cache(cfg, self.device)
        self._poses_np = synth.poses(cfg, max(cfg["blocks"], 1))
        self._dev = {}
        self._host = {}
        self._w = {}
        self.dt = torch.float32 if cfg["dtype"] == "f32" else torch.bfloat16
        if cfg["mode"] == "convkv":
            for l in range(cfg["layers"]):
                wk, wv = synth.conv_weights(cfg, l)
                self._w[l] = (wk, wv)
                self.cache.set_conv_weights(l, torch.from_numpy(wk).to(self.device),
                                            torch.from_numpy(wv).to(self.device))
        self._ref = {}
        if cfg.get("reference_frames"):
            for l in range(cfg["layers"]):
                self._ref[l] = synth.reference(cfg, l)
                self.set_reference(l)

    def set_reference(self, layer):
        k, v = (self.torch.from_numpy(a).to(self.device).to(self.dt) for a in self._ref[layer])
        self.cache.set_reference(layer, k, v)

    # ---- inputs
    def qkv_dev(self, layer, block, step):
        key = (layer, block, step)
        if key not in self._dev:
            if self.host_inputs:
                arrs = synth.qkv(self.cfg, layer, block, step)
                self._dev[key] = tuple(self.torch.from_numpy(a).to(self.device).to(self.dt) for a in arrs)
            else:
                self._dev[key] = synth.qkv_device(self.cfg, layer, block, step, self.device)
        return self._dev[key]

    def drop(self, keep_blocks):
        """Forget device inputs of blocks not in keep_blocks (bounds memory)."""
        for key in list(self._dev):
            if key[1] not in keep_blocks:
                del self._dev[key]

    def pose_dev(self, block):
        if self.cfg["pose_dim"] == 0:
            return None
        return self.torch.from_numpy(self._poses_np[block]).to(self.device)

    # ---- oracle provider interface
    def qkv(self, layer, block, step):
        key = (layer, block, step)
        if key not in self._host:
            if self.host_inputs:
                self._host[key] = synth.qkv(self.cfg, layer, block, step)
            else:
                self._host[key] = tuple(t.float().cpu().numpy() for t in
                                        synth.qkv_device(self.cfg, layer, block, step, self.device))
        return self._host[key]

    def pose(self, block):
        return self._poses_np[block]

    def conv_weights(self, layer):
        return self._w[layer]

    def reference(self, layer):
        return self._ref[layer]

    # ---- driving
    def open(self, m):
        assert self.cache.stats()["block"] == m
        self.cache.retrieve(self.pose_dev(m))

    def attend(self, m, layer, step):
        q, k, v = self.qkv_dev(layer, m, step)
        return self.cache.attend(layer, q, k, v)


def max_err(got, want, heads=None, rows=None):
    """Largest |got - want|.  ``want`` may be the oracle's (output, slack)
    pair (``attend(..., with_slack=True)``): then the largest amount by which
    |got - want| exceeds the slack, i.e. the error left once every P code that
    the FP8 product's rounding may decide either way has been allowed its other
    value.  Where the slack is zero this is the plain error."""
    slack = None
    if isinstance(want, tuple):
        want, slack = want
    g = got.float().cpu().numpy().astype(np.float64)
    if heads is not None:
        g = g[:, heads, :]
    if rows is not None:
        g = g[rows]
        want = want[rows]
        slack = None if slack is None else slack[rows]
    if not g.size:
        return 0.0
    d = np.abs(g - want)
    return float(np.max(d if slack is None else d - slack))


def oracle_err(got, attend, heads=None, rows=None, tol=None):
    """max_err of ``got`` against the oracle's ``attend(rows=...)`` (a callable
    taking the reference's ``rows`` and ``with_slack`` keywords).  Rows whose
    error exceeds ``tol`` are compared again beyond the oracle's slack
    (``attend(rows=those, with_slack=True)``; zero slack, and so the same
    error, for the dtypes without an FP8 P): the slack is computed only where
    it is needed."""
    want = attend(rows=rows)
    g = got.float().cpu().numpy().astype(np.float64)
    if heads is not None:
        g = g[:, heads, :]
    rs = np.arange(g.shape[0]) if rows is None else np.asarray(rows)
    if not rs.size:
        return 0.0
    row_err = np.max(np.abs(g[rs] - want[rs]), axis=tuple(range(1, g.ndim)))
    err = float(np.max(row_err))
    if tol is None or err <= tol:
        return err
    bad = rs[row_err > tol]
    want2, slack = attend(rows=bad, with_slack=True)
    excess = float(np.max(np.abs(g[bad] - want2[bad]) - slack[bad]))
    good = row_err[row_err <= tol]
    return max(excess, float(np.max(good)) if good.size else 0.0)

