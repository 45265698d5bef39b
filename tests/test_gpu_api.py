"""C-ABI contract on the GPU: call-order errors leave the handle unchanged,
reset + replay reproduces indices and outputs bit for bit, and device memory
stays flat over a stream."""
import numpy as np
import pytest

from bounded_kv_block_amd import bkv, synth
from gpu_helpers import Run

pytestmark = pytest.mark.gpu


def _small(**kw):
    base = dict(heads=2, grid_h=4, grid_w=6, bank=4, blocks=12, pose_dim=16, keyframes=4)
    base.update(kw)
    return synth.workload("prsink_512", **base)


def test_call_order_errors():
    import torch
    cfg = _small(layers=2)
    run = Run(cfg)
    c = run.cache
    q, k, v = run.qkv_dev(0, 0, 0)
    with pytest.raises(bkv.BkvError) as e:
        c.attend(0, q, k, v)
    assert e.value.status == bkv.BKV_ERR_STATE                 # attend before retrieve
    with pytest.raises(bkv.BkvError) as e:
        c.commit()
    assert e.value.status == bkv.BKV_ERR_STATE                 # commit with nothing open
    run.open(0)
    with pytest.raises(bkv.BkvError) as e:
        c.retrieve(run.pose_dev(0))
    assert e.value.status == bkv.BKV_ERR_STATE                 # retrieve while open
    with pytest.raises(bkv.BkvError) as e:
        c.attend(2, q, k, v)
    assert e.value.status == bkv.BKV_ERR_ARG                   # layer out of range
    c.attend(0, q, k, v)
    with pytest.raises(bkv.BkvError) as e:
        c.commit()
    assert e.value.status == bkv.BKV_ERR_STATE                 # layer 1 not attended
    assert c.stats()["open"] == 1 and c.stats()["block"] == 0  # state unchanged
    with pytest.raises(ValueError):
        c.attend(1, q[:-1], k, v)                              # shape checked by the binding
    with pytest.raises(bkv.BkvError) as e:
        bkv._check(bkv.lib().bkv_attend(c._h, 1, None, None, None, None, c._s()), "bkv_attend")
    assert e.value.status == bkv.BKV_ERR_ARG
    q1, k1, v1 = run.qkv_dev(1, 0, 0)
    c.attend(1, q1, k1, v1)
    c.commit()
    assert c.stats()["block"] == 1 and c.stats()["open"] == 0
    with pytest.raises(bkv.BkvError) as e:
        c.set_conv_weights(0, torch.zeros(2, 128, 5, device=run.device), torch.zeros(2, 128, 5, device=run.device))
    assert e.value.status == bkv.BKV_ERR_UNSUPPORTED
    cv = synth.workload("convkv_512", heads=2, grid_h=4, grid_w=6, blocks=3)
    cc = bkv.Cache(cv, run.device)
    with pytest.raises(bkv.BkvError) as e:
        cc.retrieve(None)                                      # conv weights not set
    assert e.value.status == bkv.BKV_ERR_STATE


def test_workspace_too_small_is_refused():
    import ctypes
    import torch
    cfg = bkv.config_from_workload(_small())
    need = bkv.workspace_size(cfg)
    ws = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    h = ctypes.c_void_p()
    st = bkv.lib().bkv_create(ctypes.byref(cfg), ctypes.c_void_p(ws.data_ptr()), need - 256,
                              ctypes.c_void_p(torch.cuda.current_stream().cuda_stream), ctypes.byref(h))
    assert st == bkv.BKV_ERR_WORKSPACE and not h.value


def _drive(run, n):
    sels, outs = [], []
    for m in range(n):
        run.open(m)
        sels.append(run.cache.selection())
        outs.append(run.attend(m, 0, 0).clone())
        run.cache.commit()
    return sels, outs


def test_reset_replay_is_bitwise_identical():
    cfg = _small()
    run = Run(cfg)
    s1, o1 = _drive(run, 12)
    run.cache.reset()
    assert run.cache.stats()["block"] == 0
    s2, o2 = _drive(run, 12)
    assert s1 == s2
    for a, b in zip(o1, o2):
        assert bool((a == b).all())


def test_memory_is_flat_over_the_stream():
    import gc
    import torch
    gc.collect()                     # objects of earlier tests must not be freed mid-loop
    gc.disable()
    try:
        _memory_flat(torch)
    finally:
        gc.enable()


def _memory_flat(torch):
    cfg = _small(blocks=40)
    run = Run(cfg)
    q, k, v = run.qkv_dev(0, 0, 0)
    out = torch.empty_like(q)
    ws = run.cache.stats()["workspace_bytes"]
    seen = set()
    for m in range(40):
        run.cache.retrieve(run.pose_dev(m))
        run.cache.attend(0, q, k, v, out)
        run.cache.commit()
        torch.cuda.synchronize()
        seen.add(torch.cuda.memory_allocated())
        assert run.cache.stats()["workspace_bytes"] == ws
    assert len(seen) == 1


def test_mfma_probe_rate():
    """The sustained-rate probe reports a plausible bf16 MFMA rate (between a
    tenth of and just above the 2.5 PFLOP/s nominal peak), and bad arguments
    are refused."""
    from bounded_kv_block_amd import bkv
    t = bkv.probe_mfma(512, 2000)
    assert 250.0 < t < 2600.0, t
    with pytest.raises(bkv.BkvError) as ei:
        bkv.probe_mfma(0, 10)
    assert ei.value.status == bkv.BKV_ERR_ARG
