"""Host-side checks of the C ABI (no GPU needed, no kernel is launched).

The library must load, export every function that include/vs.h declares,
size its workspaces, and reject invalid arguments with a status code before
anything would be enqueued.
"""
import ctypes
import os
import re

import pytest

import vertical_slash_sparse_amd as vsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "vs.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vs_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_binding_names():
    assert _declared_functions() == sorted(vsa.exported_symbols())


def test_library_exports_every_declared_symbol():
    L = vsa.lib()
    for name in _declared_functions():
        assert hasattr(L, name), name
    # the dynamic symbol table, read with ctypes
    raw = ctypes.CDLL(vsa.LIB_PATH)
    for name in _declared_functions():
        assert ctypes.cast(getattr(raw, name), ctypes.c_void_p).value


def test_status_strings():
    assert vsa.status_str(vsa.VS_OK) == "ok"
    assert "workspace" in vsa.status_str(vsa.VS_ERR_WORKSPACE)
    assert vsa.status_str(99) == "unknown status"


def test_workspace_sizes():
    # per row: each chunk's largest key and counts, the decision state and one
    # (count, mass) histogram of 2048 bins per digit pass -- no per-candidate arrays
    per_row = vsa.vs_select_workspace_bytes(1, 131072)
    assert 3 * 2048 * 12 < per_row < 128 * 1024
    assert vsa.vs_select_workspace_bytes(8, 131072) >= 8 * 3 * 2048 * 12
    assert vsa.vs_select_workspace_bytes(0, 10) == 0
    a = vsa.vs_attn_workspace_bytes(8, 131072, 4096, 8192)
    b = vsa.vs_attn_workspace_bytes(8, 262144, 262144, 262144)
    assert 0 < a < b
    assert vsa.vs_attn_workspace_bytes(8, 0, 1, 1) == 0
    # a packed batch holds every sequence's rows plus the sequence table
    one = vsa.vs_attn_varlen_workspace_bytes(8, 1, 4096, 64, 128)
    many = vsa.vs_attn_varlen_workspace_bytes(8, 16, 4096, 64, 128)
    assert many >= vsa.vs_attn_workspace_bytes(8 * 16, 4096, 64, 128) > one > 0
    assert vsa.vs_attn_varlen_workspace_bytes(8, 16, 4096, 64, 128) > vsa.vs_attn_workspace_bytes(8, 4096, 64, 128)
    assert vsa.vs_attn_varlen_workspace_bytes(8, 0, 4096, 64, 128) == 0
    assert vsa.vs_attn_varlen_workspace_bytes(0, 4, 4096, 64, 128) == 0
    assert vsa.vs_attn_varlen_workspace_bytes(8, 4, 4096, 0, 128) == 0


def _fake(addr=0x1000):
    return ctypes.c_void_p(addr)


def test_invalid_arguments_are_rejected_before_launch():
    L = vsa.lib()
    p = _fake()
    # vs_select: null pointers, bad mass, bad cap, small workspace
    assert L.vs_select(None, 1, 10, 0, 0.5, 5, p, p, p, 1 << 20, None) == vsa.VS_ERR_INVALID
    assert L.vs_select(p, 1, 10, 0, 0.0, 5, p, p, p, 1 << 20, None) == vsa.VS_ERR_INVALID
    assert L.vs_select(p, 1, 10, 0, 1.5, 5, p, p, p, 1 << 20, None) == vsa.VS_ERR_INVALID
    assert L.vs_select(p, 1, 10, 0, 0.5, 11, p, p, p, 1 << 20, None) == vsa.VS_ERR_INVALID
    assert L.vs_select(p, 1, 10, 0, 0.5, 0, p, p, p, 1 << 20, None) == vsa.VS_ERR_INVALID
    assert L.vs_select(p, 1, 10, 7, 0.5, 5, p, p, p, 1 << 20, None) == vsa.VS_ERR_INVALID
    assert L.vs_select(p, 1, 10, 0, 0.5, 5, p, p, p, 8, None) == vsa.VS_ERR_WORKSPACE
    # vs_select_threshold: alpha in (0, 1], same other checks
    assert L.vs_select_threshold(p, 1, 10, 0, 0.0, 5, p, p, p, 1 << 20, None) == vsa.VS_ERR_INVALID
    assert L.vs_select_threshold(p, 1, 10, 0, 1.01, 5, p, p, p, 1 << 20, None) == vsa.VS_ERR_INVALID
    assert L.vs_select_threshold(None, 1, 10, 0, 0.5, 5, p, p, p, 1 << 20, None) == vsa.VS_ERR_INVALID
    assert L.vs_select_threshold(p, 1, 10, 0, 0.5, 11, p, p, p, 1 << 20, None) == vsa.VS_ERR_INVALID
    assert L.vs_select_threshold(p, 1, 10, 0, 0.5, 5, p, p, p, 8, None) == vsa.VS_ERR_WORKSPACE
    # vs_select_both: pointers, heads, mass, both caps, workspace
    both = lambda **kw: L.vs_select_both(*[kw.get(k, dv) for k, dv in (
        ("vlog", p), ("slog", p), ("heads", 2), ("n", 10), ("mass", 0.5), ("cap_v", 5), ("cap_s", 5),
        ("v_idx", p), ("v_cnt", p), ("s_off", p), ("s_cnt", p), ("ws", p), ("ws_bytes", 1 << 20),
        ("stream", None))])
    for name in ("vlog", "slog", "v_idx", "v_cnt", "s_off", "s_cnt", "ws"):
        assert both(**{name: None}) == vsa.VS_ERR_INVALID, name
    assert both(heads=0) == vsa.VS_ERR_INVALID
    assert both(heads=32768) == vsa.VS_ERR_INVALID
    assert both(n=0) == vsa.VS_ERR_INVALID
    assert both(mass=0.0) == vsa.VS_ERR_INVALID
    assert both(mass=1.5) == vsa.VS_ERR_INVALID
    assert both(cap_v=0) == vsa.VS_ERR_INVALID
    assert both(cap_s=11) == vsa.VS_ERR_INVALID
    assert both(ws_bytes=8) == vsa.VS_ERR_WORKSPACE
    assert L.vs_select_both_workspace_bytes(3, 1000) == L.vs_select_workspace_bytes(6, 1000)
    assert L.vs_select_both_workspace_bytes(0, 1000) == 0
    # vs_attn_aggregate: pointers, shapes, workspace
    agg = lambda **kw: L.vs_attn_aggregate(*[kw.get(k, dv) for k, dv in (
        ("q", p), ("k", p), ("v", p), ("h_q", 8), ("h_kv", 2), ("n", 256), ("d", 128),
        ("scale", ctypes.c_float(0.088)), ("out", p), ("lse", p), ("a_v", p), ("a_s", p), ("ws", p),
        ("ws_bytes", 1 << 30), ("stream", None))])
    assert agg(lse=None) == vsa.VS_ERR_INVALID
    assert agg(a_s=None) == vsa.VS_ERR_INVALID
    assert agg(h_q=6) == vsa.VS_ERR_UNSUPPORTED
    assert agg(d=96) == vsa.VS_ERR_UNSUPPORTED
    assert agg(ws_bytes=16) == vsa.VS_ERR_WORKSPACE
    assert L.vs_aggregate_workspace_bytes(2, 256) > L.vs_attn_workspace_bytes(2, 256, 1, 256)
    # vs_index: shapes (d in {64, 128}; hidden a multiple of 32 up to 256)
    assert L.vs_index(p, p, 8, 100, 96, 128, p, p, p, p, None) == vsa.VS_ERR_UNSUPPORTED
    assert L.vs_index(p, p, 8, 100, 128, 48, p, p, p, p, None) == vsa.VS_ERR_UNSUPPORTED
    assert L.vs_index(p, p, 8, 100, 128, 288, p, p, p, p, None) == vsa.VS_ERR_UNSUPPORTED
    assert L.vs_index(p, p, 8, 100, 64, 0, p, p, p, p, None) == vsa.VS_ERR_INVALID
    assert L.vs_index(p, p, 0, 100, 128, 128, p, p, p, p, None) == vsa.VS_ERR_INVALID
    assert L.vs_index(None, p, 8, 100, 128, 128, p, p, p, p, None) == vsa.VS_ERR_INVALID
    # one KV-head tensor must fit a 32-bit byte range (8 x 2^21 x 128 x 2 B = 4 GiB)
    assert L.vs_index(p, p, 8, 1 << 21, 128, 128, p, p, p, p, None) == vsa.VS_ERR_UNSUPPORTED

    def attn(**kw):
        a = dict(q=p, k=p, v=p, dt=0, h_q=32, h_kv=8, n=1024, d=128, scale=0.088, vi=p, vc=p,
                 cap_v=16, so=p, sc=p, cap_s=16, out=p, lse=None, ws=p, ws_bytes=1 << 30)
        a.update(kw)
        return L.vs_sparse_attn_prefill(a["q"], a["k"], a["v"], a["dt"], a["h_q"], a["h_kv"], a["n"],
                                        a["d"], a["scale"], a["vi"], a["vc"], a["cap_v"], a["so"],
                                        a["sc"], a["cap_s"], a["out"], a["lse"], a["ws"],
                                        a["ws_bytes"], None)

    assert attn(q=None) == vsa.VS_ERR_INVALID
    assert attn(h_q=30) == vsa.VS_ERR_INVALID          # h_q % h_kv != 0
    assert attn(h_q=24) == vsa.VS_ERR_UNSUPPORTED      # group 3
    assert attn(d=96) == vsa.VS_ERR_UNSUPPORTED
    assert attn(dt=5) == vsa.VS_ERR_INVALID
    assert attn(scale=float("nan")) == vsa.VS_ERR_INVALID
    assert attn(scale=float("-inf")) == vsa.VS_ERR_INVALID
    # any finite scale passes the checks (the workspace check comes later)
    for sc in (-1.0, 0.0, -0.0, 1e-30, 12.5):
        assert attn(scale=sc, ws_bytes=16) == vsa.VS_ERR_WORKSPACE, sc
    assert attn(cap_v=0) == vsa.VS_ERR_INVALID
    assert attn(n=0) == vsa.VS_ERR_INVALID
    assert attn(ws_bytes=16) == vsa.VS_ERR_WORKSPACE
    # vs_block_discover: pointers, alpha, skel, group x skel, words, workspace
    def disc(**kw):
        a = dict(q=p, k=p, h_q=8, h_kv=2, n=1000, d=128, scale=ctypes.c_float(0.088), skel=8,
                 alpha=ctypes.c_float(0.5), mask=p, wpr=1, score=None, ws=p, ws_bytes=1 << 30)
        a.update(kw)
        return L.vs_block_discover(a["q"], a["k"], a["h_q"], a["h_kv"], a["n"], a["d"], a["scale"],
                                   a["skel"], a["alpha"], a["mask"], a["wpr"], a["score"], a["ws"],
                                   a["ws_bytes"], None)

    assert disc(mask=None) == vsa.VS_ERR_INVALID
    assert disc(alpha=ctypes.c_float(0.0)) == vsa.VS_ERR_INVALID
    assert disc(alpha=ctypes.c_float(1.5)) == vsa.VS_ERR_INVALID
    assert disc(skel=3) == vsa.VS_ERR_INVALID            # must divide 64
    assert disc(skel=16) == vsa.VS_ERR_UNSUPPORTED       # G * skel = 64 > 32
    assert disc(wpr=0) == vsa.VS_ERR_INVALID             # 16 blocks need one word
    assert disc(d=96) == vsa.VS_ERR_UNSUPPORTED
    assert disc(h_q=6) == vsa.VS_ERR_UNSUPPORTED
    assert disc(n=16384 * 64 + 1, wpr=513) == vsa.VS_ERR_UNSUPPORTED   # more than 16384 blocks
    assert disc(ws_bytes=16) == vsa.VS_ERR_WORKSPACE
    # block means (bf16 hi and lo) and the fp32 block scores of every pair
    assert L.vs_block_workspace_bytes(2, 1000, 128) == 2 * 2 * 16 * 128 * 2 + 256 * ((2 * 16 * 16 * 4 + 255) // 256)
    # vs_block_attn_prefill
    def battn(**kw):
        a = dict(q=p, k=p, v=p, dt=0, h_q=8, h_kv=2, n=1000, d=128, scale=ctypes.c_float(0.088),
                 mask=p, wpr=1, out=p, lse=None, ws=p, ws_bytes=256)
        a.update(kw)
        return L.vs_block_attn_prefill(a["q"], a["k"], a["v"], a["dt"], a["h_q"], a["h_kv"], a["n"],
                                       a["d"], a["scale"], a["mask"], a["wpr"], a["out"], a["lse"],
                                       a["ws"], a["ws_bytes"], None)

    assert battn(mask=None) == vsa.VS_ERR_INVALID
    assert battn(wpr=0) == vsa.VS_ERR_INVALID
    assert battn(dt=3) == vsa.VS_ERR_INVALID
    assert battn(h_q=24) == vsa.VS_ERR_UNSUPPORTED
    assert battn(d=80) == vsa.VS_ERR_UNSUPPORTED
    assert battn(scale=ctypes.c_float(float("inf"))) == vsa.VS_ERR_INVALID
    assert battn(ws_bytes=8) == vsa.VS_ERR_WORKSPACE
    assert L.vs_block_attn_workspace_bytes() >= 32
    # per-query-head sets and packed batches
    assert L.vs_sparse_attn_prefill_qh(p, p, p, 0, 8, 2, 100, 128, ctypes.c_float(0.1), None, p, 4,
                                       p, p, 4, p, None, p, 1 << 30, None) == vsa.VS_ERR_INVALID
    assert L.vs_sparse_attn_prefill_qh(p, p, p, 0, 8, 2, 100, 128, ctypes.c_float(0.1), p, p, 4,
                                       p, p, 4, p, None, p, 16, None) == vsa.VS_ERR_WORKSPACE
    cu = (ctypes.c_int32 * 3)(0, 50, 120)
    bad = (ctypes.c_int32 * 3)(0, 60, 50)
    cup = ctypes.cast(cu, ctypes.c_void_p)

    def varlen(cu_p=cup, total=120, nseq=2, ws_bytes=1 << 30, h_q=8):
        return L.vs_sparse_attn_prefill_varlen(p, p, p, 0, h_q, 2, total, 128, ctypes.c_float(0.1),
                                               cu_p, nseq, 0, p, p, 4, p, p, 4, p, None, p,
                                               ws_bytes, None)

    assert varlen(cu_p=None) == vsa.VS_ERR_INVALID
    assert varlen(total=121) == vsa.VS_ERR_INVALID          # cu[nseq] must equal total
    assert varlen(cu_p=ctypes.cast(bad, ctypes.c_void_p), total=50) == vsa.VS_ERR_INVALID
    assert varlen(nseq=0) == vsa.VS_ERR_INVALID
    assert varlen(h_q=24) == vsa.VS_ERR_UNSUPPORTED
    assert varlen(ws_bytes=16) == vsa.VS_ERR_WORKSPACE
    t = (ctypes.c_int64 * 4)()
    assert L.vs_attn_tile_counts(None, 8, 1024, 16, 16, 32, ctypes.cast(t, ctypes.c_void_p), None) == vsa.VS_ERR_INVALID
    assert L.vs_attn_tile_counts(p, 8, 1024, 16, 16, 24, ctypes.cast(t, ctypes.c_void_p), None) == vsa.VS_ERR_UNSUPPORTED


def test_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros(2, 8, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        vsa.vs_index(x, x, torch.zeros(128, 256, dtype=torch.bfloat16), torch.zeros(2, 128, dtype=torch.bfloat16))


def test_noalloc_checks_before_launch():
    """The allocation-free attention entry point: null pointers, and shapes
    whose workspace exceeds its static array, are rejected before anything
    touches a device."""
    L = vsa.lib()
    p = _fake()
    n = 1 << 20
    assert vsa.vs_attn_workspace_bytes(8, n, n, n) > vsa.NOALLOC_SCRATCH_BYTES
    assert L.vs_sparse_attn_prefill_noalloc(p, p, p, 0, 32, 8, n, 128, ctypes.c_float(0.1), p, p, n,
                                            p, p, n, p, None, None) == vsa.VS_ERR_WORKSPACE
    assert L.vs_sparse_attn_prefill_noalloc(None, p, p, 0, 32, 8, 1024, 128, ctypes.c_float(0.1), p, p, 4,
                                            p, p, 4, p, None, None) == vsa.VS_ERR_INVALID
    assert L.vs_sparse_attn_prefill_noalloc(p, p, p, 0, 32, 8, 1024, 128, ctypes.c_float(0.1), p, p, 0,
                                            p, p, 4, p, None, None) == vsa.VS_ERR_INVALID


def test_grid_limits_are_rejected_before_launch():
    """Shapes whose launches would not fit 2^32 work-items along one grid
    dimension return VS_ERR_UNSUPPORTED; the largest shapes that fit pass on
    to the workspace check."""
    L = vsa.lib()
    p = _fake()

    def attn(h_q, h_kv, n, d=64, ws_bytes=16):
        return L.vs_sparse_attn_prefill(p, p, p, 0, h_q, h_kv, n, d, ctypes.c_float(0.1), p, p, 4,
                                        p, p, 4, p, None, p, ws_bytes, None)

    # the tile builder: one 1024-thread workgroup per index-set row
    assert attn(1 << 22, 1 << 22, 1) == vsa.VS_ERR_UNSUPPORTED
    assert attn((1 << 22) - 1, (1 << 22) - 1, 1) == vsa.VS_ERR_WORKSPACE
    # the attention grid: 512 threads per (row, 64-position block) at G = 4
    n = (1 << 23) - 1
    assert attn(256, 64, n) == vsa.VS_ERR_UNSUPPORTED
    assert attn(252, 63, n) == vsa.VS_ERR_WORKSPACE
    # per-query-head sets: one set per query head, 256 positions per workgroup
    assert L.vs_sparse_attn_prefill_qh(p, p, p, 0, 1 << 22, 1 << 22, 1, 64, ctypes.c_float(0.1), p, p, 4,
                                       p, p, 4, p, None, p, 16, None) == vsa.VS_ERR_UNSUPPORTED
    # packed batches: nseq * sets index-set rows
    nseq = (1 << 22) // 8
    cu = (ctypes.c_int32 * (nseq + 1))(*([0] * nseq + [1]))
    assert L.vs_sparse_attn_prefill_varlen(p, p, p, 0, 32, 8, 1, 64, ctypes.c_float(0.1),
                                           ctypes.cast(cu, ctypes.c_void_p), nseq, 0, p, p, 4, p, p, 4,
                                           p, None, p, 1 << 40, None) == vsa.VS_ERR_UNSUPPORTED
    nseq -= 1
    cu = (ctypes.c_int32 * (nseq + 1))(*([0] * nseq + [1]))
    assert L.vs_sparse_attn_prefill_varlen(p, p, p, 0, 32, 8, 1, 64, ctypes.c_float(0.1),
                                           ctypes.cast(cu, ctypes.c_void_p), nseq, 0, p, p, 4, p, p, 4,
                                           p, None, p, 16, None) == vsa.VS_ERR_WORKSPACE
    # list capacities have no grid limit (the bit-setting pass strides over them)
    assert L.vs_sparse_attn_prefill(p, p, p, 0, 32, 8, 1024, 128, ctypes.c_float(0.1), p, p, 1 << 26,
                                    p, p, 1 << 26, p, None, p, 16, None) == vsa.VS_ERR_WORKSPACE
    # aggregation and discovery launch h_kv along a 65535-limited dimension
    assert L.vs_attn_aggregate(p, p, p, 65536, 65536, 16, 64, ctypes.c_float(0.1), p, p, p, p, p,
                               1 << 40, None) == vsa.VS_ERR_UNSUPPORTED
    assert L.vs_block_discover(p, p, 65536, 65536, 16, 64, ctypes.c_float(0.1), 8, ctypes.c_float(0.5),
                               p, 1, None, p, 1 << 40, None) == vsa.VS_ERR_UNSUPPORTED
