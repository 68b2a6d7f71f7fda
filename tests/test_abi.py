"""The C ABI without a GPU: the library loads, exports every declared entry point, and the
host-only calls (layout, validation) behave as the header says. No kernel is launched."""
import ctypes
import os
import re

import pytest

import mixture_experts_ffn_dispatch_amd as moe
from mixture_experts_ffn_dispatch_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")
ATTN_HEADER = os.path.join(ROOT, "include", "attn.h")


def declared_functions():
    names = set()
    for h in (HEADER, ATTN_HEADER):
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b((?:moe|attn)_[a-z_]+)\s*\(", text))
    return sorted(names)


def test_headers_compile_as_c_and_cpp(tmp_path):
    # both headers are plain C: the host compilers accept them on their own
    import shutil
    import subprocess

    src = tmp_path / "h.c"
    src.write_text('#include "moe.h"\n#include "attn.h"\nint main(void) { return (int)sizeof(moe_config); }\n')
    for cc, extra in (("gcc", ["-std=c99"]), ("g++", ["-x", "c++", "-std=c++17"])):
        if shutil.which(cc):
            r = subprocess.run([cc, *extra, "-fsyntax-only", "-Wall", "-Werror", f"-I{os.path.dirname(HEADER)}", str(src)],
                               capture_output=True, text=True)
            assert r.returncode == 0, r.stderr


def test_library_exports_every_declared_symbol():
    lib = moe.load()
    names = declared_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), n
    assert moe.abi_version() == 8



def test_binding_matches_header():
    """The ctypes structures list the header's fields in order, and both name one ABI version."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    assert int(re.search(r"#define MOE_ABI_VERSION (\d+)", text).group(1)) == _lib.ABI_VERSION
    for struct, cls in (("moe_config", _lib.CConfig), ("moe_routing", _lib.CRouting),
                        ("moe_ws_layout", _lib.CLayout), ("moe_burst_cfg", _lib.CBurstCfg),
                        ("moe_trace_rec", _lib.CTraceRec), ("attn_config", _lib.CAttnConfig)):
        src = text if struct != "attn_config" else re.sub(r"/\*.*?\*/", "", open(ATTN_HEADER).read(), flags=re.S)
        body = re.search(r"typedef struct " + struct + r" \{(.*?)\} " + struct + ";", src, flags=re.S).group(1)
        assert re.findall(r"(\w+)(?:\[\d+\])?;", body) == [n for n, _ in cls._fields_], struct


def test_struct_sizes():
    # moe_config: 12 ints, the three X-Stage calibration floats, a reserved word, then the
    # trace pointer at byte 64; a trace record is 64 bytes, matching the numpy view the tests
    # read traces with
    import numpy as np

    assert ctypes.sizeof(_lib.CConfig) == 72 and _lib.CConfig.trace.offset == 64
    assert ctypes.sizeof(_lib.CTraceRec) == 64 == np.dtype(_lib.TRACE_DTYPE).itemsize


def test_strerror():
    for code in (0, -1, -2, -3, -4, -5, 7):
        assert isinstance(moe.strerror(code), str) and moe.strerror(code)


def _cfg(**kw):
    base = dict(T=4096, H=7168, I=2048, E=32, k=8, experts_per_wave=4)
    base.update(kw)
    return moe.MoeConfig(**base)


def test_layout_is_consistent():
    L = moe.moe_workspace_layout(_cfg())
    assert L["tile_m"] == 256 and L["n1_tiles"] == 16 and L["n2_tiles"] == 28
    assert L["chunk_tokens"] == 16 and L["chunks"] == 256
    # max m-blocks: every row of every active expert fills tiles, plus one partial per expert
    assert L["max_mblk"] == (4096 * 8 + 32 * 255) // 256
    assert L["max_tasks"] == L["max_mblk"] * (16 + 28)
    offs = [L[n] for n in ("header", "chunk_counts", "mblk_expert", "mblk_row0", "mblk_rows", "mblk_ready", "tasks")]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    assert L["total_bytes"] >= L["tasks"] + 4 * L["max_tasks"]
    assert moe.moe_workspace_size(_cfg()) == L["total_bytes"]


@pytest.mark.parametrize("T,k,E,tile", [(4096, 8, 32, 256), (8192, 8, 128, 256), (512, 6, 64, 128),
                                         (65536, 2, 16, 256), (256, 2, 8, 128), (8, 1, 64, 32),
                                         (1200, 6, 64, 256), (1194, 6, 64, 128), (256, 5, 64, 128),
                                         (256, 4, 64, 32)])
def test_auto_tile_height(T, k, E, tile):
    assert moe.moe_workspace_layout(_cfg(T=T, k=k, E=E))["tile_m"] == tile


@pytest.mark.parametrize("kw,code", [
    (dict(T=0), moe.MOE_ERR_INVALID_ARG),
    (dict(k=0), moe.MOE_ERR_INVALID_ARG),
    (dict(k=33, E=64), moe.MOE_ERR_UNSUPPORTED),
    (dict(k=9, E=8), moe.MOE_ERR_INVALID_ARG),
    (dict(E=1025, k=2), moe.MOE_ERR_UNSUPPORTED),
    (dict(H=100), moe.MOE_ERR_UNSUPPORTED),
    (dict(I=96), moe.MOE_ERR_UNSUPPORTED),
    (dict(experts_per_wave=0), moe.MOE_ERR_INVALID_ARG),
    (dict(lead_waves=-1), moe.MOE_ERR_INVALID_ARG),
    (dict(tile_m=48), moe.MOE_ERR_UNSUPPORTED),
    (dict(flags=32), moe.MOE_ERR_INVALID_ARG),
    (dict(flags=6), moe.MOE_ERR_INVALID_ARG),  # wide last m-blocks forced both on and off
    (dict(reserved=1), moe.MOE_ERR_INVALID_ARG),
    (dict(schedule=3), moe.MOE_ERR_INVALID_ARG),
    (dict(schedule=2, lead_waves=2), moe.MOE_ERR_INVALID_ARG),  # the automatic order picks the lead
    (dict(xs_drain_gbps=-1.0), moe.MOE_ERR_INVALID_ARG),
    (dict(xs_issue_us=float("nan")), moe.MOE_ERR_INVALID_ARG),
    (dict(xs_capacity_mib=float("inf")), moe.MOE_ERR_INVALID_ARG),
    (dict(T=1 << 20, H=8192, k=8, E=64), moe.MOE_ERR_UNSUPPORTED),  # row buffers past 4 GiB
    # 2^24 rows in 32-row tiles: m-block 0x7FFFF would exist, which the sentinel task words
    # (no task, no-op slot, flush) rely on being out of range
    (dict(T=1 << 22, k=4, E=64, H=64, I=64, tile_m=32), moe.MOE_ERR_UNSUPPORTED),
])
def test_invalid_configs_rejected(kw, code):
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_workspace_size(_cfg(**kw))
    assert ei.value.status == code


def test_mblock_limit_alone_rejects():
    # 4193800 * 4 rows in 32-row tiles over 64 experts: at most (16775200 + 64 * 31) / 32 =
    # 524287 = 0x7FFFF m-blocks, the sentinel task words' m-block, while the tile list
    # (2 * 524287 = 1048574 tiles) stays below its own limit of 2^20: only the m-block check
    # can reject this plan
    kw = dict(T=4193800, k=4, E=64, H=64, I=64, tile_m=32)
    R = kw["T"] * kw["k"]
    max_mblk = (R + kw["E"] * (kw["tile_m"] - 1)) // kw["tile_m"]
    assert max_mblk == 0x7FFFF and 2 * max_mblk <= 1 << 20
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_workspace_size(_cfg(**kw))
    assert ei.value.status == moe.MOE_ERR_UNSUPPORTED
    # one m-block fewer is accepted
    L = moe.moe_workspace_layout(_cfg(**dict(kw, T=4193800 - 8)))
    assert L["max_mblk"] == 0x7FFFF - 1


def test_large_plan_below_the_limits_accepted():
    # 2^22 rows in 32-row tiles: 131134 m-blocks at most, 262268 tiles, below both limits
    L = moe.moe_workspace_layout(_cfg(T=1 << 20, k=4, E=64, H=64, I=64, tile_m=32))
    assert L["max_mblk"] == ((1 << 22) + 64 * 31) // 32 < (1 << 19) - 1
    assert L["max_tasks"] == 2 * L["max_mblk"] <= 1 << 20


def test_null_pointers_rejected_before_any_launch():
    lib = moe.load()
    c = _cfg().to_c()
    rt = _lib.CRouting()
    # a valid config with missing pointers must fail on the host, touching no device
    assert lib.moe_plan(ctypes.byref(c), None, ctypes.byref(rt), None, 0, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_dispatch(ctypes.byref(c), ctypes.byref(rt), None, None, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_forward(ctypes.byref(c), None, None, None, None, None, None, 0, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_combine(ctypes.byref(c), ctypes.byref(rt), None, None, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_forward_gather(ctypes.byref(c), ctypes.byref(rt), None, None, None, None, None, None, 0,
                                  None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_forward_gather(ctypes.byref(c), None, 1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20,
                                  1 << 30, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_status_read(None, 0, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_burst_gap(None, None, 0, None, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_burst_clock_hz(None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_workspace_size(None, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_workspace_size(ctypes.byref(c), None) == moe.MOE_ERR_INVALID_ARG


def test_undersized_workspace_rejected():
    lib = moe.load()
    c = _cfg().to_c()
    need = moe.moe_workspace_size(_cfg())
    rt = _lib.CRouting(*([1 << 20] * 6))  # non-null dummies: the size check comes first
    dummy = 1 << 20
    assert lib.moe_plan(ctypes.byref(c), dummy, ctypes.byref(rt), dummy, need - 1, None) == moe.MOE_ERR_WORKSPACE
    assert lib.moe_forward(ctypes.byref(c), dummy, dummy, dummy, dummy, dummy, dummy, need - 1, None) == \
        moe.MOE_ERR_WORKSPACE
    assert lib.moe_forward_gather(ctypes.byref(c), ctypes.byref(rt), dummy, dummy, dummy, dummy, dummy, dummy,
                                  need - 1, None) == moe.MOE_ERR_WORKSPACE


def test_attention_rejects_invalid_configs_on_the_host():
    lib = moe.load()
    dummy = 1 << 20

    def call(**kw):
        base = dict(B=1, heads=1, M=64, d=128, num_workgroups=0)
        base.update(kw)
        c = _lib.CAttnConfig(**base)
        return lib.attn_forward(ctypes.byref(c), dummy, dummy, dummy, dummy, None, None)

    assert call(M=0) == moe.MOE_ERR_INVALID_ARG
    assert call(B=0) == moe.MOE_ERR_INVALID_ARG
    assert call(heads=-1) == moe.MOE_ERR_INVALID_ARG
    assert call(d=64) == moe.MOE_ERR_UNSUPPORTED
    assert call(M=1 << 23) == moe.MOE_ERR_UNSUPPORTED  # a head of 2 GiB
    c = _lib.CAttnConfig(B=1, heads=1, M=64, d=128)
    assert lib.attn_forward(ctypes.byref(c), None, dummy, dummy, dummy, None, None) == moe.MOE_ERR_INVALID_ARG
    c.reserved[1] = 1
    assert lib.attn_forward(ctypes.byref(c), dummy, dummy, dummy, dummy, None, None) == moe.MOE_ERR_INVALID_ARG
