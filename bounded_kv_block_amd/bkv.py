"""Thin ctypes binding over libbkv.so (include/bkv.h): argument marshalling only.

Every step of the path -- retrieval, RoPE, append, attention, compression --
runs in the library's HIP kernels.  PyTorch supplies device memory (the
workspace and the caller's tensors) and the current stream.  There is no
fallback: if libbkv.so is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbkv.so")

BKV_OK, BKV_ERR_ARG, BKV_ERR_STATE, BKV_ERR_WORKSPACE, BKV_ERR_DEVICE, BKV_ERR_UNSUPPORTED = range(6)
PR_SINK, CONVKV = 0, 1
F32, BF16, BF16_FP8K, BF16_FP8KV = 0, 1, 2, 3
DTYPES = {"f32": F32, "bf16": BF16, "bf16_fp8k": BF16_FP8K, "bf16_fp8kv": BF16_FP8KV}
POSITIONS = {"default": 0, "relative": 1, "absolute": 2}     # bkv_positions
BANK_POLICIES = {"fifo": 0, "pose": 1}                        # bkv_bank_policy
SEG_KINDS = {0: "static", 1: "dynamic", 2: "window", 3: "current", 4: "memory", 5: "reference"}

# every symbol include/bkv.h declares
EXPORTS = ("bkv_workspace_size", "bkv_create", "bkv_destroy", "bkv_reset", "bkv_set_conv_weights",
           "bkv_set_reference",
           "bkv_profile_start", "bkv_profile_stop",
           "bkv_retrieve", "bkv_attend", "bkv_attend_static_scratch", "bkv_attend_qkv", "bkv_commit", "bkv_selection",
           "bkv_context", "bkv_stats",
           "bkv_export_segment", "bkv_status_str", "bkv_last_error", "bkv_probe_mfma")


class Config(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("mode", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("layers", ctypes.c_int32), ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("frames_per_block", ctypes.c_int32), ("grid_h", ctypes.c_int32), ("grid_w", ctypes.c_int32),
                ("window_blocks", ctypes.c_int32), ("static_blocks", ctypes.c_int32),
                ("dynamic_k", ctypes.c_int32), ("bank_blocks", ctypes.c_int32), ("pose_dim", ctypes.c_int32),
                ("rope_t", ctypes.c_int32), ("rope_h", ctypes.c_int32), ("rope_w", ctypes.c_int32),
                ("rope_theta", ctypes.c_double), ("conv_kernel", ctypes.c_int32),
                ("conv_stride", ctypes.c_int32), ("memory_frames", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("reference_frames", ctypes.c_int32),
                ("rope_positions", ctypes.c_int32), ("bank_policy", ctypes.c_int32)]


class Segment(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("id", ctypes.c_int32), ("tokens", ctypes.c_int32),
                ("t0", ctypes.c_int32)]


class Stats(ctypes.Structure):
    _fields_ = [("block", ctypes.c_int64), ("open", ctypes.c_int32), ("n_segments", ctypes.c_int32),
                ("n_keys", ctypes.c_int64), ("last_evicted", ctypes.c_int64),
                ("bank_count", ctypes.c_int32), ("memory_count", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_size_t), ("split_attends", ctypes.c_int64)]


class KernelTime(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_char * 24), ("launches", ctypes.c_int64), ("total_ms", ctypes.c_double),
                ("max_ms", ctypes.c_double)]


class BkvError(RuntimeError):
    def __init__(self, status: int, call: str, msg: str):
        super().__init__(f"{call}: {_status_name(status)}: {msg}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Open libbkv.so once (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run bounded_kv_block_amd/build.py first")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        sig = {
            "bkv_workspace_size": [ctypes.POINTER(Config), ctypes.POINTER(sz)],
            "bkv_create": [ctypes.POINTER(Config), vp, sz, vp, ctypes.POINTER(vp)],
            "bkv_destroy": [vp],
            "bkv_reset": [vp],
            "bkv_set_conv_weights": [vp, i32, vp, vp, vp],
            "bkv_set_reference": [vp, i32, vp, vp, vp],
            "bkv_retrieve": [vp, vp, vp],
            "bkv_attend": [vp, i32, vp, vp, vp, vp, vp],
            "bkv_attend_static_scratch": [vp, i32, vp, vp, vp, vp, vp],
            "bkv_attend_qkv": [vp, i32, vp, vp, vp, i32, vp, vp],
            "bkv_commit": [vp, vp],
            "bkv_selection": [vp, ctypes.POINTER(i32), i32, ctypes.POINTER(i32), vp],
            "bkv_context": [vp, ctypes.POINTER(Segment), i32, ctypes.POINTER(i32), vp],
            "bkv_stats": [vp, ctypes.POINTER(Stats)],
            "bkv_export_segment": [vp, i32, i32, vp, vp, vp],
            "bkv_profile_start": [vp, i32],
            "bkv_profile_stop": [vp, ctypes.POINTER(KernelTime), i32, ctypes.POINTER(i32)],
            "bkv_probe_mfma": [i32, i32, ctypes.POINTER(ctypes.c_double), vp],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        L.bkv_status_str.argtypes = [ctypes.c_int]
        L.bkv_status_str.restype = ctypes.c_char_p
        L.bkv_last_error.argtypes = []
        L.bkv_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _status_name(s: int) -> str:
    try:
        return lib().bkv_status_str(s).decode()
    except Exception:
        return str(s)


def _check(status: int, call: str):
    if status != BKV_OK:
        raise BkvError(status, call, lib().bkv_last_error().decode(errors="replace"))


def config_from_workload(w: dict) -> Config:
    """ABI config from a workload dict (keys as in bounded_kv_block_amd.synth)."""
    c = Config()
    c.struct_size = ctypes.sizeof(Config)
    c.mode = CONVKV if w["mode"] == "convkv" else PR_SINK
    c.dtype = DTYPES[w["dtype"]]
    c.layers, c.heads, c.head_dim = w["layers"], w["heads"], w["head_dim"]
    c.frames_per_block, c.grid_h, c.grid_w = w["frames"], w["grid_h"], w["grid_w"]
    c.window_blocks, c.static_blocks = w["window"], w["static"]
    c.dynamic_k, c.bank_blocks, c.pose_dim = w["dynamic_k"], w["bank"], w["pose_dim"]
    c.rope_t, c.rope_h, c.rope_w = w["rope"]
    c.rope_theta = float(w.get("theta", 10000.0))
    c.conv_kernel, c.conv_stride, c.memory_frames = w["conv_kernel"], w["conv_stride"], w["memory_frames"]
    c.softmax_scale = float(w.get("softmax_scale", 0.0))
    c.reference_frames = int(w.get("reference_frames", 0) or 0)
    c.rope_positions = POSITIONS[w.get("positions", "default")]
    c.bank_policy = BANK_POLICIES[w.get("bank_policy", "fifo")]
    return c


def workspace_size(cfg: Config) -> int:
    n = ctypes.c_size_t()
    _check(lib().bkv_workspace_size(ctypes.byref(cfg), ctypes.byref(n)), "bkv_workspace_size")
    return n.value


def _stream(torch, device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


class Cache:
    """One bounded cache over a workspace tensor on ``device``.

    Calls run on torch's current stream of that device.
    """

    def __init__(self, cfg, device="cuda"):
        import torch
        self._torch = torch
        self.config = cfg if isinstance(cfg, Config) else config_from_workload(cfg)
        self.device = torch.device(device)
        if self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        c = self.config
        self.T = c.frames_per_block * c.grid_h * c.grid_w
        # Q/K/V/out are bf16 also with the FP8 key cache
        self.dtype = torch.float32 if c.dtype == F32 else torch.bfloat16
        nbytes = workspace_size(c)
        # 256-byte alignment: torch's allocator hands out 512-byte aligned blocks
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        assert self.workspace.data_ptr() % 256 == 0
        self._h = ctypes.c_void_p()
        with torch.cuda.device(self.device):
            _check(lib().bkv_create(ctypes.byref(c), ctypes.c_void_p(self.workspace.data_ptr()),
                                    nbytes, _stream(torch, self.device), ctypes.byref(self._h)),
                   "bkv_create")

    # -- helpers ----------------------------------------------------------
    def _s(self):
        return _stream(self._torch, self.device)

    def _tensor(self, x, name, shape=None, dtype=None):
        if not isinstance(x, self._torch.Tensor):
            raise TypeError(f"{name} must be a torch tensor")
        if x.device != self.device:
            raise ValueError(f"{name} is on {x.device}, cache is on {self.device}")
        if dtype is not None and x.dtype != dtype:
            raise ValueError(f"{name} has dtype {x.dtype}, expected {dtype}")
        if shape is not None and tuple(x.shape) != tuple(shape):
            raise ValueError(f"{name} has shape {tuple(x.shape)}, expected {tuple(shape)}")
        if not x.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        return ctypes.c_void_p(x.data_ptr())

    @property
    def qkv_shape(self):
        c = self.config
        return (self.T, c.heads, c.head_dim)

    # -- the path -----------------------------------------------------------
    def set_conv_weights(self, layer: int, wk, wv):
        c = self.config
        shp = (c.heads, c.head_dim, c.conv_kernel)
        _check(lib().bkv_set_conv_weights(self._h, layer,
                                          self._tensor(wk, "wk", shp, self._torch.float32),
                                          self._tensor(wv, "wv", shp, self._torch.float32), self._s()),
               "bkv_set_conv_weights")

    @property
    def reference_shape(self):
        c = self.config
        return (c.reference_frames * c.grid_h * c.grid_w, c.heads, c.head_dim)

    def set_reference(self, layer: int, k, v):
        shp = self.reference_shape
        _check(lib().bkv_set_reference(self._h, layer, self._tensor(k, "k", shp, self.dtype),
                                       self._tensor(v, "v", shp, self.dtype), self._s()), "bkv_set_reference")

    def retrieve(self, pose=None):
        p = None if pose is None else self._tensor(pose, "pose", (self.config.pose_dim,), self._torch.float32)
        _check(lib().bkv_retrieve(self._h, p, self._s()), "bkv_retrieve")

    def attend(self, layer: int, q, k, v, out=None):
        shp = self.qkv_shape
        if out is None:
            out = self._torch.empty(shp, dtype=self.dtype, device=self.device)
        _check(lib().bkv_attend(self._h, layer, self._tensor(q, "q", shp, self.dtype),
                                self._tensor(k, "k", shp, self.dtype), self._tensor(v, "v", shp, self.dtype),
                                self._tensor(out, "out", shp, self.dtype), self._s()), "bkv_attend")
        return out

    def attend_static_scratch(self, layer: int, q, k, v, out=None):
        """bkv_attend with the split launch's part states in the library's
        static device array (the allocation-free entry point)."""
        shp = self.qkv_shape
        if out is None:
            out = self._torch.empty(shp, dtype=self.dtype, device=self.device)
        _check(lib().bkv_attend_static_scratch(self._h, layer, self._tensor(q, "q", shp, self.dtype),
                                               self._tensor(k, "k", shp, self.dtype),
                                               self._tensor(v, "v", shp, self.dtype),
                                               self._tensor(out, "out", shp, self.dtype), self._s()),
               "bkv_attend_static_scratch")
        return out

    def attend_qkv(self, layer: int, x, w, b=None, out=None):
        """Fused projection + attention: q|k|v = x w^T + b inside the library.
        x [T, model_dim], w [3*H*D, model_dim], b [3*H*D] or None, all bf16."""
        c = self.config
        bf = self._torch.bfloat16
        if not isinstance(x, self._torch.Tensor) or x.dim() != 2:
            raise ValueError("x must be a 2-D tensor [T, model_dim]")
        C = int(x.shape[1])
        n = 3 * c.heads * c.head_dim
        shp = self.qkv_shape
        if out is None:
            out = self._torch.empty(shp, dtype=self.dtype, device=self.device)
        bp = None if b is None else self._tensor(b, "b", (n,), bf)
        _check(lib().bkv_attend_qkv(self._h, layer, self._tensor(x, "x", (self.T, C), bf),
                                    self._tensor(w, "w", (n, C), bf), bp, C,
                                    self._tensor(out, "out", shp, self.dtype), self._s()), "bkv_attend_qkv")
        return out

    def commit(self):
        _check(lib().bkv_commit(self._h, self._s()), "bkv_commit")

    # -- inspection -----------------------------------------------------------
    def selection(self) -> list:
        buf = (ctypes.c_int32 * 16)()
        n = ctypes.c_int32()
        _check(lib().bkv_selection(self._h, buf, 16, ctypes.byref(n), self._s()), "bkv_selection")
        return [int(buf[i]) for i in range(n.value)]

    def context(self) -> list:
        buf = (Segment * 32)()
        n = ctypes.c_int32()
        _check(lib().bkv_context(self._h, buf, 32, ctypes.byref(n), self._s()), "bkv_context")
        return [(SEG_KINDS[buf[i].kind], buf[i].id, buf[i].tokens, buf[i].t0) for i in range(n.value)]

    def stats(self) -> dict:
        s = Stats()
        _check(lib().bkv_stats(self._h, ctypes.byref(s)), "bkv_stats")
        return {f: getattr(s, f) for f, _ in Stats._fields_}

    def export_segment(self, layer: int, seg: int):
        """(K as attended, V) of context segment ``seg``: each [tokens, H, D]."""
        ctx = self.context()
        n = ctx[seg][2] if 0 <= seg < len(ctx) else 0
        c = self.config
        k = self._torch.empty((n, c.heads, c.head_dim), dtype=self.dtype, device=self.device)
        v = self._torch.empty_like(k)
        _check(lib().bkv_export_segment(self._h, layer, seg, ctypes.c_void_p(k.data_ptr()),
                                        ctypes.c_void_p(v.data_ptr()), self._s()), "bkv_export_segment")
        return k, v

    def profile_start(self, max_launches: int):
        """Record HIP events around each kernel the cache launches (on its stream)."""
        _check(lib().bkv_profile_start(self._h, max_launches), "bkv_profile_start")

    def profile_stop(self) -> dict:
        """{kernel: (launches, total_ms, max_ms)}; waits for the recorded events."""
        buf = (KernelTime * 16)()
        n = ctypes.c_int32()
        _check(lib().bkv_profile_stop(self._h, buf, 16, ctypes.byref(n)), "bkv_profile_stop")
        return {buf[i].kernel.decode(): (buf[i].launches, buf[i].total_ms, buf[i].max_ms) for i in range(n.value)}

    def reset(self):
        _check(lib().bkv_reset(self._h), "bkv_reset")

    def close(self):
        if getattr(self, "_h", None) and self._h.value:
            lib().bkv_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def probe_mfma(workgroups: int = 1024, iters: int = 4000, device="cuda") -> float:
    """Sustained bf16 MFMA rate in TFLOP/s (bkv_probe_mfma) on ``device``."""
    import torch
    dev = torch.device(device)
    with torch.cuda.device(dev):
        t = ctypes.c_double()
        _check(lib().bkv_probe_mfma(workgroups, iters, ctypes.byref(t), _stream(torch, dev)), "bkv_probe_mfma")
    return t.value
