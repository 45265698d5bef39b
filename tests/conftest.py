import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def read_table(name):
    """Rows of a whitespace table under tests/golden ('#' comments, '-' = empty)."""
    rows = []
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


def ids(field):
    return [] if field == "-" else [int(x) for x in field.split(",")]


class SynthProvider:
    """Oracle input provider backed by the seeded host generators (cached)."""

    def __init__(self, cfg):
        from bounded_kv_block_amd import synth
        self.cfg = cfg
        self._synth = synth
        self._qkv = {}
        self._poses = synth.poses(cfg, max(cfg["blocks"], 1))
        self._w = {}

    def qkv(self, layer, block, step):
        key = (layer, block, step)
        if key not in self._qkv:
            self._qkv[key] = self._synth.qkv(self.cfg, layer, block, step)
        return self._qkv[key]

    def pose(self, block):
        return self._poses[block]

    def conv_weights(self, layer):
        if layer not in self._w:
            self._w[layer] = self._synth.conv_weights(self.cfg, layer)
        return self._w[layer]

    def reference(self, layer):
        return self._synth.reference(self.cfg, layer)


@pytest.fixture
def rng():
    return np.random.default_rng(1234)
