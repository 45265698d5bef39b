#!/usr/bin/env python3
"""Throughput of bounded-KV block attention on one MI355X.

One step = one streaming block through the whole path: bkv_retrieve (pose
top-k, block open), bkv_attend for every (sampling step, layer) -- K/V append
with fused 3D RoPE and the flash-attention kernel over the bounded context --
and bkv_commit (window/bank bookkeeping; ConvKV: memory rebuild).  Inputs
(Q/K/V pools, poses) are resident in HBM before timing starts.

Prints one JSON line: query tokens/s of the whole step (value), attention
TFLOP/s and % of the bf16 MFMA peak, per-kernel event timings, the roofline
of the dominant kernel, per-block latency percentiles and the CPU oracle
timed on a bounded sample of the same workload.

The default workload is the 720x416-shaped stream (3510 queries per block,
24570 keys of context, 40 layers x 3 sampling steps per block): one step is
one block of 120 attends.  `--workload prsink_long` runs its whole 1080-block
stream (unless --steps is given) and reports the per-block latency
distribution over it: p50, p99, the least-squares slope over block index and
whether the workspace and torch's device allocation stayed constant.  It runs
the stream once untimed first and resets the cache: on a fresh GPU the clock
settles over the first second or so of sustained load, which moves per-block
latency by a percent or two with time, not with the stream's length.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "query tokens/s & TFLOP/s of bounded-KV block attention (% bf16 MFMA peak)"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA
PEAK_FP32_TFLOPS = 157.3       # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed blocks (default 20; prsink_long: the rest of its 1080-block stream)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="prsink_720x416",
                    choices=["prsink_512", "prsink_512_fp8k", "prsink_512_fp8kv", "prsink_512_qkv", "prsink_512_ref",
                             "prsink_512_rel", "prsink_512_posebank", "prsink_512_qkv_fp8k", "prsink_720x416",
                             "prsink_720x416_fp8kv", "prsink_long", "convkv_512", "convkv_512_abs", "convkv_512_fp8k",
                             "convkv_512_fp8kv", "tiny_fp32"])
    ap.add_argument("--pool", type=int, default=4, help="distinct resident input blocks cycled through")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU-oracle sample time")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (a known-size reference "
                         "for the HBM byte counters) and exit")
    return ap.parse_args()


def calibrate_copy(mib):
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    dst.copy_(src)
    ev[0].record()
    for _ in range(5):
        dst.copy_(src)
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / 5
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "avg_ms": ms,
                      "gbs": 2 * n / (ms * 1e-3) / 1e9}), flush=True)


def measured_traffic(workload):
    """HBM bytes per attention launch from the committed rocprofv3 byte-counter
    summary of this workload (FETCH_SIZE and WRITE_SIZE, each scaled by what
    the counter reads for a plain copy of known size), or None when there is
    no summary or the kernel source has changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"attention_{workload}_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for ln in open(path):
        parts = ln.split()
        if len(parts) == 2 and parts[0] in ("traffic_bytes", "kernels_hip_sha256"):
            kv[parts[0]] = parts[1]
    src = os.path.join(ROOT, "bounded_kv_block_amd", "csrc", "kernels.hip")
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if kv.get("kernels_hip_sha256") != sha or "traffic_bytes" not in kv:
        return None
    return float(kv["traffic_bytes"])


def attention_launches(T, H):
    """Launches of one split attention call: whole rounds of 256 units, the
    remainder units cut into 256 // remainder key parts, and the merge of the
    parts when there is more than one."""
    units = -(-T // 256) * H
    rem = units % 256
    return 2 + (1 if 256 // rem > 1 else 0)


def steady_block(cfg):
    """First block whose context has its final size."""
    if cfg["mode"] == "convkv":
        return cfg["window"] + 2
    return cfg["static"] + cfg["window"] + cfg["dynamic_k"]


def cpu_baseline(cfg, run_inputs, poses, m, target_s, weights=None):
    """The oracle, as it stands, on block m of the same stream: retrieval plus
    attention of whole heads (all queries) until about target_s seconds.  With
    `weights` (the fused-projection workload), run_inputs gives hidden states
    and the oracle also projects each head's q, k, v inside the timed region."""
    import numpy as np
    import oracle

    H, D = cfg["heads"], cfg["head_dim"]

    class Prov:
        def __init__(self):
            self.cache = {}
            self.head = 0
            if weights is not None:
                self.w = weights[0].float().cpu().numpy().astype(np.float64)
                self.b = weights[1].float().cpu().numpy().astype(np.float64)

        def hidden(self, layer, block, step):
            key = ("x", layer, block, step)
            if key not in self.cache:
                self.cache[key] = run_inputs(layer, block, step).float().cpu().numpy()
            return self.cache[key]

        def qkv(self, layer, block, step):
            if weights is not None:       # this head's projection (timed: it is the oracle's work)
                h = self.head
                x = self.hidden(layer, block, step)
                rows = np.concatenate([np.arange(i * H * D + h * D, i * H * D + (h + 1) * D) for i in range(3)])
                parts = oracle.qkv_projection(x, self.w[rows], self.b[rows], 1, D, round_bf16=True)
                out = []
                for part in parts:
                    a = np.zeros((x.shape[0], H, D))
                    a[:, h:h + 1, :] = part
                    out.append(a)
                return tuple(out)
            key = (layer, block, step)
            if key not in self.cache:
                self.cache[key] = tuple(t.float().cpu().numpy() for t in run_inputs(layer, block, step))
            return self.cache[key]

        def pose(self, b):
            return poses[b]

        def conv_weights(self, layer):
            from bounded_kv_block_amd import synth
            return synth.conv_weights(cfg, layer)

        def reference(self, layer):
            key = ("ref", layer)
            if key not in self.cache:
                from bounded_kv_block_amd import synth
                self.cache[key] = synth.reference(cfg, layer)
            return self.cache[key]

    prov = Prov()
    ref = (oracle.ConvKVReference if cfg["mode"] == "convkv" else oracle.PRSinkReference)(cfg, prov)
    # fetch the inputs first (not part of the oracle's work)
    fetch = prov.hidden if weights is not None else prov.qkv
    for kind, b, _, _ in (ref.context(m) if cfg["mode"] == "convkv" else ref.context(m, ref.selection(m))):
        if kind != "memory":
            fetch(0, b, cfg["steps"] - 1)
    if cfg["mode"] == "convkv":
        for grp in ref.schedule(m)["memory"]:
            for e in grp:
                fetch(0, e // cfg["frames"], cfg["steps"] - 1)
    fetch(0, m, 0)
    if cfg.get("reference_frames"):
        prov.reference(0)
    t0 = time.perf_counter()
    sel = ref.selection(m) if cfg["mode"] != "convkv" else None
    done = 0
    while done < H:
        prov.head = done
        if cfg["mode"] == "convkv":
            ref.attend(m, 0, 0, heads=[done])
        else:
            ref.attend(m, 0, 0, heads=[done], selection=sel)
        done += 1
        if time.perf_counter() - t0 >= target_s:
            break
    dt = time.perf_counter() - t0
    T = cfg["frames"] * cfg["grid_h"] * cfg["grid_w"]
    attends = cfg["layers"] * cfg["steps"]
    try:
        from threadpoolctl import threadpool_info
        blas = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        blas = 1
    res = {"value": T * done / H / dt / attends, "unit": "query tokens/s", "cores": int(blas),
           "host_cpus": len(os.sched_getaffinity(0)), "kind": "oracle",
           "sample": f"block {m} of the {cfg['name']} stream, layer 0, step 0: retrieval + "
                     f"{'fp64 QKV projection + ' if weights is not None else ''}fp64 attention of {done}/{H} heads "
                     f"x all {T} queries over the block's bounded context, "
                     f"{dt:.1f} s; value scaled to the whole block (x{H}/{done} heads"
                     f"{f', x{attends} attends per block' if attends > 1 else ''})"}
    res["fp32_numpy"] = cpu_fp32(cfg, ref, m, sel, target_s / 2, attends)
    return res


def cpu_fp32(cfg, ref, m, sel, target_s, attends):
    """CPU throughput line: the attention step (softmax(scale q k^T) v per
    head over the block's bounded context, the O(T * N_k * D) part of the
    path) as plain fp32 numpy matrix products, on the same block's rotated
    q, k and v (rotation and retrieval done beforehand, untimed)."""
    import numpy as np
    H, D = cfg["heads"], cfg["head_dim"]
    s = cfg.get("softmax_scale", 0.0) or 1.0 / np.sqrt(D)
    done, dt = 0, 0.0
    while done < H and dt < target_s:
        heads = [done]
        ref.p.head = done                  # the fused workload's provider projects this head
        if cfg["mode"] == "convkv":
            kv = ref.context_kv(m, 0, 0, heads)
            t0 = ref.positions(m)[1]
        else:
            kv = ref.context_kv(m, 0, 0, heads, sel)
            t0 = ref.context(m, sel)[-1][3]
        q, _, _ = ref.p.qkv(0, m, 0)
        q = ref._rot(q, lambda f: t0 + f, heads)[:, 0, :].astype(np.float32)
        k = np.concatenate([x[2][:, 0, :] for x in kv]).astype(np.float32)
        v = np.concatenate([x[3][:, 0, :] for x in kv]).astype(np.float32)
        c0 = time.perf_counter()
        for r in range(0, q.shape[0], 256):
            z = (q[r:r + 256] @ k.T) * np.float32(s)
            z -= z.max(axis=1, keepdims=True)
            np.exp(z, out=z)
            z /= z.sum(axis=1, keepdims=True)
            _ = z @ v
        dt += time.perf_counter() - c0
        done += 1
    T = q.shape[0]
    return {"value": T * done / H / dt / attends, "unit": "query tokens/s",
            "sample": f"{done}/{H} heads of the same block, fp32 numpy, {dt:.1f} s; "
                      f"value scaled to the whole block"}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): "
              "the bounded-KV path shards by heads across GPUs (one cache per GPU); this benchmark "
              "measures the one-GPU share.",
              file=sys.stderr)
        sys.exit(2)

    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return

    import numpy as np
    import torch
    from bounded_kv_block_amd import bkv, synth

    cfg = synth.workload(args.workload)
    long_stream = args.workload == "prsink_long"
    if args.steps is None:
        args.steps = cfg["blocks"] - steady_block(cfg) - args.warmup if long_stream else 20
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    T = synth.tokens_per_block(cfg)
    H, D, L, S = cfg["heads"], cfg["head_dim"], cfg["layers"], cfg["steps"]
    cache = bkv.Cache(cfg, dev)
    if cfg["mode"] == "convkv":
        for l in range(L):
            wk, wv = synth.conv_weights(cfg, l)
            cache.set_conv_weights(l, torch.from_numpy(wk).to(dev), torch.from_numpy(wv).to(dev))
    if cfg.get("reference_frames"):
        dt_in = torch.float32 if cfg["dtype"] == "f32" else torch.bfloat16
        for l in range(L):
            cache.set_reference(l, *(torch.from_numpy(a).to(dev).to(dt_in) for a in synth.reference(cfg, l)))

    # resident inputs: a pool of blocks per (layer, step), cycled by block id
    # (q, k, v; or hidden states and per-layer projection weights)
    fused = bool(cfg.get("qkv"))
    pool = max(1, args.pool if L * S == 1 else 1)
    inputs = {}
    for b in range(pool):
        for l in range(L):
            for s in range(S):
                inputs[(l, b, s)] = (synth.hidden_device(cfg, l, b, s, dev) if fused
                                     else synth.qkv_device(cfg, l, b, s, dev))
    weights = {l: synth.qkv_weights_device(cfg, l, dev) for l in range(L)} if fused else {}

    def block_inputs(layer, block, step):
        return inputs[(layer, block % pool, step)]

    prefix = steady_block(cfg)
    n_blocks = prefix + args.warmup + args.steps
    poses_np = synth.poses(cfg, n_blocks)
    poses = torch.from_numpy(poses_np).to(dev) if cfg["pose_dim"] else None
    out = torch.empty((T, H, D), dtype=torch.float32 if cfg["dtype"] == "f32" else torch.bfloat16, device=dev)

    def attend(l, m, s):
        if fused:
            w, b = weights[l]
            cache.attend_qkv(l, block_inputs(l, m, s), w, b, out)
        else:
            q, k, v = block_inputs(l, m, s)
            cache.attend(l, q, k, v, out)

    def step(m):
        cache.retrieve(poses[m] if poses is not None else None)
        for s in range(S):
            for l in range(L):
                attend(l, m, s)
        cache.commit()

    m = 0
    if long_stream:                                # settling pass, then back to block 0
        for mm in range(n_blocks):
            step(mm)
        torch.cuda.synchronize()
        cache.reset()
    for _ in range(prefix + args.warmup):          # fill the cache, then warm up
        step(m)
        m += 1
    torch.cuda.synchronize()
    alloc0 = torch.cuda.memory_allocated(dev)
    ws_bytes = set()
    n_keys = []
    launches = args.steps * (3 + 2 * L * S + L) + 16
    cache.profile_start(launches)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i].record()
        cache.retrieve(poses[m] if poses is not None else None)
        st = cache.stats()
        n_keys.append(st["n_keys"])
        ws_bytes.add(int(st["workspace_bytes"]))
        for s in range(S):
            for l in range(L):
                attend(l, m, s)
        cache.commit()
        m += 1
    ev[-1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kt = cache.profile_stop()
    alloc1 = torch.cuda.memory_allocated(dev)
    wall = t1 - t0
    per_block = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)])
    # least-squares slope of the per-block latency over the block index
    xb = np.arange(args.steps, dtype=np.float64)
    slope = float(np.polyfit(xb, per_block, 1)[0]) if args.steps > 1 else 0.0

    bf16 = cfg["dtype"] != "f32"
    fp8k = cfg["dtype"] in ("bf16_fp8k", "bf16_fp8kv")
    fp8v = cfg["dtype"] == "bf16_fp8kv"
    Nk = int(np.median(n_keys))
    flop_attend = 4.0 * H * T * Nk * D
    attn_n, attn_ms, _ = kt["attention"]
    attn_avg_ms = attn_ms / attn_n
    attn_tflops = flop_attend / (attn_avg_ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if bf16 else PEAK_FP32_TFLOPS
    if fp8v:
        peak = PEAK_FP8_TFLOPS                              # both products on fp8 MFMA
    elif fp8k:
        # half the flops (Q K^T) on fp8 MFMA, half (P V) on bf16: the peak of
        # that mix is the harmonic mean of the two
        peak = 1.0 / (0.5 / PEAK_FP8_TFLOPS + 0.5 / PEAK_BF16_TFLOPS)
    esz = 2 if bf16 else 4
    kesz = 1 if fp8k else esz                               # bytes per cached K value
    vesz = 1 if fp8v else esz                               # bytes per cached V value
    kernels = {}
    for name, (n, tot, mx) in kt.items():
        kernels[name] = {"launches": int(n), "avg_us": 1e3 * tot / n, "max_us": 1e3 * mx}
    # algorithmic bytes of the HBM-bound kernels, per launch
    # K, V read token-major; rotated K and V^T written (a context gathered per
    # block -- ConvKV, relative positions -- also keeps the raw K in the slot)
    ctx_mode = cfg["mode"] == "convkv" or cfg.get("positions") == "relative"
    app_bytes = (2.0 * T * H * D * esz + T * H * D * (kesz + vesz) + (T * H * D * esz if ctx_mode else 0)
                 + (T * H * D * esz if fp8v and cfg["mode"] == "convkv" else 0))
    if "append" in kernels:
        kernels["append"]["gbs"] = app_bytes / (kernels["append"]["avg_us"] * 1e-6) / 1e9
    if "qkv" in kernels:
        g_flop = 2.0 * T * cfg["model_dim"] * 3 * H * D
        kernels["qkv"]["tflops"] = g_flop / (kernels["qkv"]["avg_us"] * 1e-6) / 1e12
        kernels["qkv"]["pct_peak"] = 100.0 * kernels["qkv"]["tflops"] / PEAK_BF16_TFLOPS
        kernels["qkv"]["flop_per_launch"] = g_flop
    if "gather" in kernels:         # re-rotated rows: the context less the current block and the reference
        ctx_rows = Nk - T - cfg.get("reference_frames", 0) * cfg["grid_h"] * cfg["grid_w"]
        g_bytes = ctx_rows * H * D * (esz + kesz)      # raw K read, rotated K written (E4M3 with FP8 keys)
        kernels["gather"]["gbs"] = g_bytes / (kernels["gather"]["avg_us"] * 1e-6) / 1e9
    if "conv" in kernels:
        Tf = cfg["grid_h"] * cfg["grid_w"]
        c_bytes = (2 * cfg["conv_kernel"] + 2) * cfg["memory_frames"] * Tf * H * D * esz
        kernels["conv"]["gbs"] = c_bytes / (kernels["conv"]["avg_us"] * 1e-6) / 1e9

    attends_per_step = L * S
    # algorithmic bytes of one attention launch: Q and the output once, K and V
    # of the whole bounded context once
    attn_bytes = 2.0 * T * H * D * esz + Nk * H * D * (kesz + vesz)
    value = args.steps * T / wall
    res = {
        "metric": METRIC,
        "value": value,
        "unit": "query tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": 1e3 * wall / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": (("fp8_e4m3 QK^T + fp8_e4m3 PV" if fp8v else "fp8_e4m3 QK^T + bf16 PV") if fp8k else "bf16")
                 if bf16 else "f32",
        "data": "synthetic",
        "config": {"workload": cfg["name"], "mode": cfg["mode"], "heads": H, "head_dim": D,
                   "queries_per_block": T, "keys_per_block": Nk, "layers": L, "steps_per_block": S,
                   "attends_per_block": attends_per_step, "window": cfg["window"],
                   "dynamic_k": cfg["dynamic_k"], "bank": cfg["bank"], "rope": list(cfg["rope"]),
                   "timed_blocks": [m - args.steps, m - 1],
                   **({"model_dim": cfg["model_dim"], "qkv_projection": "fused (bkv_attend_qkv)"} if fused else {}),
                   **({"reference_frames": cfg["reference_frames"]} if cfg.get("reference_frames") else {}),
                   **({"positions": cfg["positions"]} if cfg.get("positions", "default") != "default" else {}),
                   **({"bank_policy": cfg["bank_policy"]} if cfg.get("bank_policy", "fifo") != "fifo" else {})},
        "attention_tflops": attn_tflops,
        "attention_pct_peak": 100.0 * attn_tflops / peak,
        "attention_peak_tflops": peak,
        "step_tflops": flop_attend * attends_per_step * args.steps / wall / 1e12,
        "latency_ms": {"p50": float(np.percentile(per_block, 50)), "p99": float(np.percentile(per_block, 99)),
                       "max": float(per_block.max()), "blocks": int(args.steps),
                       "slope_ms_per_1000_blocks": 1000.0 * slope,
                       "slope_pct_of_p50_per_1000_blocks": 100.0 * 1000.0 * slope / float(np.percentile(per_block, 50)),
                       # the fitted change from the first timed block to the last: the
                       # per-1000-block figure extrapolates short runs far past their span
                       "drift_pct_of_p50_over_run": 100.0 * slope * (args.steps - 1) / float(np.percentile(per_block, 50))},
        "memory": {"workspace_bytes_constant": len(ws_bytes) == 1,
                   "torch_allocated_constant": alloc0 == alloc1,
                   "torch_allocated_bytes": int(alloc1)},
        "kernels": kernels,
        "roofline": {"kernel": "attention", "bound": "mfma" if bf16 else "alu", "achieved": attn_tflops,
                     "peak": peak, "unit": "TFLOP/s", "frac": attn_tflops / peak, "traffic": measured_traffic(cfg["name"]),
                     "traffic_unit": "HBM bytes per launch", "algorithmic_bytes": attn_bytes,
                     "flop_per_launch": flop_attend, "avg_launch_us": 1e3 * attn_avg_ms,
                     # an attention call whose last round of units is split runs
                     # the whole rounds, then the remainder units cut into key
                     # parts, then (more than one part per unit) the merge of the
                     # parts: the times and flops above are per call, all launches
                     "launches_per_call": attention_launches(T, H) if cache.stats()["split_attends"] else 1},
        "workspace_bytes": int(cache.stats()["workspace_bytes"]),
    }
    # what the device sustains right after the timed region: the bf16 MFMA
    # rate of an MFMA-only loop (same instruction, 2 waves per SIMD) and a
    # 1 GiB device copy
    mfma_s = bkv.probe_mfma(1024, 40000, dev)
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    cev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    cev[0].record()
    for _ in range(5):
        dst.copy_(src)
    cev[1].record()
    torch.cuda.synchronize()
    copy_gbs = 2 * (1 << 30) * 5 / (cev[0].elapsed_time(cev[1]) * 1e-3) / 1e9
    del src, dst
    res["sustained"] = {"mfma_bf16_tflops": mfma_s, "copy_gbs": copy_gbs,
                        "how": "bkv_probe_mfma(1024 workgroups x 8 waves, 40000 rounds of 8 independent "
                               "v_mfma_f32_32x32x16_bf16 on pseudo-random full-mantissa operands) and 5 "
                               "device-to-device copies of 1 GiB, event-timed after the timed region"}
    if bf16 and not fp8k:
        res["roofline"]["frac_sustained"] = attn_tflops / mfma_s
    for name in ("append", "gather", "conv"):
        if name in kernels and "gbs" in kernels[name]:
            kernels[name]["frac_hbm_peak"] = kernels[name]["gbs"] / PEAK_HBM_GBS
            kernels[name]["frac_copy"] = kernels[name]["gbs"] / copy_gbs
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfg, block_inputs, poses_np, m - 1, args.cpu_seconds,
                                           weights[0] if fused else None)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
