"""Full-output parity at full size: on one steady block of each workload,
every head and every query of the attention output against the CPU oracle
(max-abs 2e-2), through the same C-ABI calls and launch configuration the
benchmark times -- the 512x512 PR-Sink block (3072 queries over 21504 keys),
one layer of the 720x416 block at its third sampling step (3510 queries over
24570 keys, split launch), the ConvKV block (3072 queries over 13312 keys,
the 1024-token memory frame present), and the 512x512, 720x416 and ConvKV
blocks with the FP8 key cache and with the FP8 KV cache (whose 720x416 split
launch also carries the zeroed query rows past the block's end)."""
import numpy as np
import pytest

import oracle
from bounded_kv_block_amd import synth
from gpu_helpers import TOL, Run, max_err, oracle_err

pytestmark = pytest.mark.gpu


def _prsink(cfg, block, layer=0, step=0):
    run = Run(cfg, host_inputs=False)
    ref = oracle.PRSinkReference(cfg, run)
    L, S = cfg["layers"], cfg["steps"]
    for m in range(block + 1):
        run.open(m)
        sel = ref.selection(m)
        assert run.cache.selection() == sel, m
        for s in range(S):
            for l in range(L):
                out = run.attend(m, l, s)
                if m == block and (l, s) == (layer, step):
                    assert run.cache.stats()["n_keys"] == 7 * synth.tokens_per_block(cfg)
                    err = oracle_err(out, lambda **kw: ref.attend(m, l, s, selection=sel, **kw), tol=TOL[cfg["dtype"]])
                    print(f"{cfg['name']} block {m} layer {l} step {s}: all {cfg['heads']} heads x "
                          f"{out.shape[0]} queries, max|err| {err:.3e}", flush=True)
                    assert err <= TOL[cfg["dtype"]], err
                run._dev.clear()
        run.cache.commit()
        run._host.clear()
    return run


def test_prsink_512_every_output_of_a_steady_block():
    _prsink(synth.workload("prsink_512", blocks=7), 6)


def test_prsink_720x416_every_output_of_one_layer():
    run = _prsink(synth.workload("prsink_720x416", blocks=7), 6, layer=21, step=2)
    assert run.cache.stats()["split_attends"] == 7 * 40 * 3


def test_prsink_512_fp8k_every_output_of_a_steady_block():
    _prsink(synth.workload("prsink_512_fp8k", blocks=7), 6)


def test_prsink_512_fp8kv_every_output_of_a_steady_block():
    _prsink(synth.workload("prsink_512_fp8kv", blocks=7), 6)


def test_prsink_720x416_fp8kv_every_output_of_one_layer():
    run = _prsink(synth.workload("prsink_720x416_fp8kv", blocks=7), 6, layer=33, step=2)
    assert run.cache.stats()["split_attends"] == 7 * 40 * 3


@pytest.mark.parametrize("name", ["convkv_512", "convkv_512_fp8kv"])
def test_convkv_512_every_output_of_a_steady_block(name):
    cfg = synth.workload(name, blocks=7)
    run = Run(cfg, host_inputs=False)
    ref = oracle.ConvKVReference(cfg, run)
    for m in range(cfg["blocks"]):
        run.open(m)
        assert run.cache.context() == list(ref.context(m)), m
        out = run.attend(m, 0, 0)
        if m == 6:
            assert run.cache.stats()["n_keys"] == 1024 + 4 * 3072
            err = oracle_err(out, lambda **kw: ref.attend(m, 0, 0, **kw), tol=TOL[cfg["dtype"]])
            print(f"{name} block {m}: all 40 heads x 3072 queries, max|err| {err:.3e}", flush=True)
            assert err <= TOL[cfg["dtype"]], err
        run.cache.commit()
        run.drop(set(range(m - 8, m + 2)))
        run._host.clear()
