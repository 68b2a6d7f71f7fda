"""ctypes binding of libmoe's C ABI (include/moe.h): argument marshalling only.

Every step of the layer runs in the HIP library; this module turns torch tensors into device
pointers and the current HIP stream into a handle, and raises ``MoeError`` on a non-zero
status. There is no fallback: if ``libmoe.so`` is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")
ABI_VERSION = 8  # MOE_ABI_VERSION of include/moe.h that this binding marshals for

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_WORKSPACE = -3
MOE_ERR_HIP = -4
MOE_ERR_TIMEOUT = -5

MOE_SCHED_EXPERT_WAVE = 0
MOE_SCHED_INTERLEAVED = 1
MOE_SCHED_AUTO = 2
MOE_FLAG_FORCE_WAIT_TIMEOUT = 0x1
MOE_FLAG_NO_WIDE_TAILS = 0x2
MOE_FLAG_WIDE_TAILS = 0x4
MOE_FLAG_PLAN_ONE_LAUNCH = 0x8
MOE_FLAG_TEST_ABSENT_GROUP = 0x10
MOE_STATIC_WORKSPACE_BYTES = 8 << 20  # workspace array of moe_layer_noalloc
ATTN_TILE_QUERIES = 128  # include/attn.h
ATTN_WORKGROUPS_PER_CU = 2


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {strerror(status)} ({status})")


class CConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "T", "H", "I", "E", "k", "experts_per_wave", "schedule", "lead_waves", "num_workgroups",
        "tile_m", "spin_limit", "flags")] + [(n, ctypes.c_float) for n in (
            "xs_issue_us", "xs_drain_gbps", "xs_capacity_mib")] + [("reserved", ctypes.c_int32), ("trace", ctypes.c_void_p)]


class CRouting(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("topk_ids", "topk_w", "counts", "offsets", "perm", "pos")]


class CLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in (
        "total_bytes", "header", "chunk_counts", "mblk_expert", "mblk_row0", "mblk_rows", "mblk_ready",
        "tasks", "unit_start", "group_units", "group_tasks", "wave_table", "layer_sync", "defer_slots")] + [(n, ctypes.c_int32) for n in (
            "chunks", "chunk_tokens", "max_mblk", "max_tasks", "max_slots", "tile_m", "tile_n1", "tile_n2", "n1_tiles",
            "n2_tiles")]


class CTraceRec(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("task", "workgroup", "xcc", "hw_id")] + [
        (n, ctypes.c_int64) for n in ("t_claim", "t_claimed", "t_start", "t_epilogue", "t_end", "t_release")]


# numpy view of a trace buffer (moe_trace_rec, 64 bytes per record)
TRACE_DTYPE = [("task", "<i4"), ("workgroup", "<i4"), ("xcc", "<i4"), ("hw_id", "<i4"), ("t_claim", "<i8"),
               ("t_claimed", "<i8"), ("t_start", "<i8"), ("t_epilogue", "<i8"), ("t_end", "<i8"),
               ("t_release", "<i8")]


class CAttnConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("B", "heads", "M", "d", "num_workgroups")] + [
        ("reserved", ctypes.c_int32 * 3)]


class CBurstCfg(ctypes.Structure):
    _fields_ = [("producers", ctypes.c_int32), ("bytes", ctypes.c_int32), ("periods", ctypes.c_int32),
                ("reserved0", ctypes.c_int32), ("gap_ticks", ctypes.c_int64)]


@dataclass
class MoeConfig:
    """Python mirror of ``moe_config``."""

    T: int
    H: int
    I: int
    E: int
    k: int
    experts_per_wave: int = 1
    schedule: int = MOE_SCHED_EXPERT_WAVE
    lead_waves: int = 0
    num_workgroups: int = 0
    tile_m: int = 0
    spin_limit: int = 0
    flags: int = 0
    xs_issue_us: float = 0.0      # X-Stage calibration for MOE_SCHED_AUTO (0 = this GPU's memory)
    xs_drain_gbps: float = 0.0
    xs_capacity_mib: float = 0.0
    reserved: int = 0
    trace: object = None  # device buffer of moe_trace_rec (a torch tensor or an address), or None

    def to_c(self) -> CConfig:
        c = CConfig()
        for n in ("T", "H", "I", "E", "k", "experts_per_wave", "schedule", "lead_waves", "num_workgroups",
                  "tile_m", "spin_limit", "flags"):
            setattr(c, n, int(getattr(self, n)))
        for n in ("xs_issue_us", "xs_drain_gbps", "xs_capacity_mib"):
            setattr(c, n, float(getattr(self, n)))
        c.reserved = int(self.reserved)
        c.trace = _ptr(self.trace)
        return c


_lib = None


def load(path: str | None = None) -> ctypes.CDLL:
    """Load libmoe.so (built in-tree by ``mixture_experts_ffn_dispatch_amd.build``). A different
    build of the same ABI may be named by ``path`` on the first call."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m mixture_experts_ffn_dispatch_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    vp = ctypes.c_void_p
    sig = {
        "moe_abi_version": (ctypes.c_int32, []),
        "moe_strerror": (ctypes.c_char_p, [ctypes.c_int32]),
        "moe_workspace_size": (ctypes.c_int32, [P(CConfig), P(ctypes.c_size_t)]),
        "moe_workspace_layout": (ctypes.c_int32, [P(CConfig), P(CLayout)]),
        "moe_plan": (ctypes.c_int32, [P(CConfig), vp, P(CRouting), vp, ctypes.c_size_t, vp]),
        "moe_dispatch": (ctypes.c_int32, [P(CConfig), P(CRouting), vp, vp, vp]),
        "moe_forward": (ctypes.c_int32, [P(CConfig), vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]),
        "moe_forward_gather": (ctypes.c_int32, [P(CConfig), P(CRouting), vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                                                vp]),
        "moe_combine": (ctypes.c_int32, [P(CConfig), P(CRouting), vp, vp, vp]),
        "moe_status_read": (ctypes.c_int32, [vp, ctypes.c_size_t, vp]),
        "moe_layer": (ctypes.c_int32, [P(CConfig), vp, P(CRouting), vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]),
        "moe_layer_noalloc": (ctypes.c_int32, [P(CConfig), vp, P(CRouting), vp, vp, vp, vp, vp, vp, vp, vp]),
        "moe_burst_gap": (ctypes.c_int32, [P(CBurstCfg), vp, ctypes.c_size_t, vp, vp]),
        "attn_forward": (ctypes.c_int32, [P(CAttnConfig), vp, vp, vp, vp, vp, vp]),
        "moe_burst_clock_hz": (ctypes.c_int32, [P(ctypes.c_int64)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.moe_abi_version() != ABI_VERSION:  # the structures below would be misread
        raise ImportError(f"{path} has ABI version {lib.moe_abi_version()}, this binding needs {ABI_VERSION}: "
                          "rebuild it")
    _lib = lib
    return lib


def strerror(status: int) -> str:
    return load().moe_strerror(int(status)).decode()


def abi_version() -> int:
    return int(load().moe_abi_version())


def _check(status: int, where: str) -> None:
    if status != MOE_OK:
        raise MoeError(status, where)


def _ptr(t) -> int | None:
    """Device pointer of a torch tensor (or an int address / None)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _cfg(cfg) -> CConfig:
    return cfg if isinstance(cfg, CConfig) else cfg.to_c()


def _routing(rt) -> CRouting:
    r = CRouting()
    for n in ("topk_ids", "topk_w", "counts", "offsets", "perm", "pos"):
        setattr(r, n, _ptr(rt[n]) if rt.get(n) is not None else None)
    return r


def moe_workspace_size(cfg) -> int:
    n = ctypes.c_size_t(0)
    _check(load().moe_workspace_size(ctypes.byref(_cfg(cfg)), ctypes.byref(n)), "moe_workspace_size")
    return int(n.value)


def moe_workspace_layout(cfg) -> dict:
    L = CLayout()
    _check(load().moe_workspace_layout(ctypes.byref(_cfg(cfg)), ctypes.byref(L)), "moe_workspace_layout")
    return {n: int(getattr(L, n)) for n, _ in CLayout._fields_}


def moe_plan(cfg, logits, rt: dict, ws, stream=None) -> None:
    c = _cfg(cfg)
    _check(load().moe_plan(ctypes.byref(c), _ptr(logits), ctypes.byref(_routing(rt)), _ptr(ws),
                           ws.numel() * ws.element_size(), _stream(stream)), "moe_plan")


def moe_dispatch(cfg, rt: dict, x, xd, stream=None) -> None:
    _check(load().moe_dispatch(ctypes.byref(_cfg(cfg)), ctypes.byref(_routing(rt)), _ptr(x), _ptr(xd),
                               _stream(stream)), "moe_dispatch")


def moe_forward(cfg, xd, w1, w2, act, yd, ws, stream=None) -> None:
    _check(load().moe_forward(ctypes.byref(_cfg(cfg)), _ptr(xd), _ptr(w1), _ptr(w2), _ptr(act), _ptr(yd),
                              _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)), "moe_forward")


def moe_forward_gather(cfg, rt: dict, x, w1, w2, act, yd, ws, stream=None) -> None:
    _check(load().moe_forward_gather(ctypes.byref(_cfg(cfg)), ctypes.byref(_routing(rt)), _ptr(x), _ptr(w1), _ptr(w2),
                                     _ptr(act), _ptr(yd), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "moe_forward_gather")


def moe_combine(cfg, rt: dict, yd, out, stream=None) -> None:
    _check(load().moe_combine(ctypes.byref(_cfg(cfg)), ctypes.byref(_routing(rt)), _ptr(yd), _ptr(out),
                              _stream(stream)), "moe_combine")


def moe_layer(cfg, logits, rt: dict, x, w1, w2, act, yd, out, ws, stream=None) -> None:
    """The whole layer in one kernel launch (ws must be zero-filled before its first use)."""
    _check(load().moe_layer(ctypes.byref(_cfg(cfg)), _ptr(logits), ctypes.byref(_routing(rt)), _ptr(x), _ptr(w1),
                            _ptr(w2), _ptr(act), _ptr(yd), _ptr(out), _ptr(ws), ws.numel() * ws.element_size(),
                            _stream(stream)), "moe_layer")


def moe_layer_noalloc(cfg, logits, rt: dict, x, w1, w2, act, yd, out, status=None, stream=None) -> None:
    """The whole layer (plan, forward with the gather, combine) with the library's static
    workspace array; ``status`` (a device int32 tensor or None) receives the device-side error
    word."""
    _check(load().moe_layer_noalloc(ctypes.byref(_cfg(cfg)), _ptr(logits), ctypes.byref(_routing(rt)), _ptr(x),
                                    _ptr(w1), _ptr(w2), _ptr(act), _ptr(yd), _ptr(out), _ptr(status),
                                    _stream(stream)), "moe_layer_noalloc")


def attn_forward(B: int, heads: int, M: int, q, k, v, o, lse=None, d: int = 128, num_workgroups: int = 0,
                 stream=None) -> None:
    """Attention forward (include/attn.h): q, k, v, o [B, heads, M, d] bf16; lse float32 or None."""
    c = CAttnConfig(B=B, heads=heads, M=M, d=d, num_workgroups=num_workgroups)
    _check(load().attn_forward(ctypes.byref(c), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _stream(stream)),
           "attn_forward")


def moe_burst_gap(producers: int, nbytes: int, periods: int, gap_ticks: int, buf, times, stream=None) -> None:
    c = CBurstCfg(producers=producers, bytes=nbytes, periods=periods, reserved0=0, gap_ticks=gap_ticks)
    _check(load().moe_burst_gap(ctypes.byref(c), _ptr(buf), buf.numel() * buf.element_size(), _ptr(times),
                                _stream(stream)), "moe_burst_gap")


def moe_burst_clock_hz() -> int:
    hz = ctypes.c_int64(0)
    _check(load().moe_burst_clock_hz(ctypes.byref(hz)), "moe_burst_clock_hz")
    return int(hz.value)


def moe_status_read(ws, stream=None) -> int:
    """Synchronises the stream and returns the device-side status code (0 = OK)."""
    return int(load().moe_status_read(_ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))
