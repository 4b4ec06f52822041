"""Python binding of libvs: vertical-slash sparse prefill on MI355X (gfx950).

Thin ctypes marshalling over the C ABI in ``include/vs.h``; the functions
keep the C names.  Every step of the computation runs in the HIP kernels of
``libvs.so``; PyTorch only provides device memory and the current stream.
There is no fallback: if the library is missing or cannot be loaded the
calls raise.

    vs_index(k_rope, v, w1, w2)                    -> (vlog, slog)
    vs_select(logit, kind, mass, cap)              -> (idx, count)
    vs_select_threshold(logit, kind, alpha, cap)   -> (idx, count)
    vs_select_both(vlog, slog, mass, cap_v, cap_s) -> (v_idx, v_cnt, s_off, s_cnt)
    vs_attn_aggregate(q, k, v)                     -> (out, lse, a_v, a_s)
    vs_block_discover(q, k, skel, alpha)           -> mask (, score)
    vs_block_attn_prefill(q, k, v, mask)           -> (out, lse)
    vs_sparse_attn_prefill(q, k, v, v_idx, v_cnt, s_off, s_cnt, scale=None)
                                                   -> (out, lse)
    vs_sparse_attn_prefill_qh(...)                 per-query-head lists [h_q, cap]
    vs_sparse_attn_prefill_varlen(q, k, v, cu_seqlens, v_idx, v_cnt, s_off, s_cnt)
                                                   packed batch of sequences
    vs_prefill(q, k, v, w1, w2, mass)              -> (out, lse, (v_idx, v_cnt, s_off, s_cnt))
                                                   index -> select x2 -> attention
"""
from __future__ import annotations

import ctypes
import functools
import inspect
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# VS_SANITIZE=1 loads the build whose host code is instrumented with
# AddressSanitizer and UndefinedBehaviorSanitizer (python -m
# vertical_slash_sparse_amd.build --sanitize; clang's ASan runtime preloaded)
LIB_PATH = os.path.join(_HERE, "libvs_san.so" if os.environ.get("VS_SANITIZE") == "1" else "libvs.so")

VS_OK, VS_ERR_INVALID, VS_ERR_UNSUPPORTED, VS_ERR_WORKSPACE, VS_ERR_HIP = range(5)
VS_BF16, VS_F32 = 0, 1
VS_VERTICAL, VS_SLASH = 0, 1

_SYMBOLS = ("vs_index", "vs_select_workspace_bytes", "vs_select", "vs_select_threshold",
            "vs_select_both_workspace_bytes", "vs_select_both",
            "vs_attn_workspace_bytes", "vs_attn_varlen_workspace_bytes",
            "vs_aggregate_workspace_bytes", "vs_attn_aggregate",
            "vs_sparse_attn_prefill", "vs_sparse_attn_prefill_noalloc", "vs_sparse_attn_prefill_qh",
            "vs_sparse_attn_prefill_varlen",
            "vs_attn_tile_counts", "vs_block_workspace_bytes",
            "vs_block_discover", "vs_block_attn_workspace_bytes", "vs_block_attn_prefill",
            "vs_status_str")


class VSError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status_str(status)} ({status})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libvs.so (built by ``vertical_slash_sparse_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run `python -m vertical_slash_sparse_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, f64, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_double, ctypes.c_float, ctypes.c_size_t
        L.vs_index.argtypes = [P, P, i32, i32, i32, i32, P, P, P, P, P]
        L.vs_index.restype = i32
        L.vs_select_workspace_bytes.argtypes = [i32, i32]
        L.vs_select_workspace_bytes.restype = sz
        L.vs_select.argtypes = [P, i32, i32, i32, f64, i32, P, P, P, sz, P]
        L.vs_select.restype = i32
        L.vs_select_threshold.argtypes = [P, i32, i32, i32, f64, i32, P, P, P, sz, P]
        L.vs_select_threshold.restype = i32
        L.vs_select_both_workspace_bytes.argtypes = [i32, i32]
        L.vs_select_both_workspace_bytes.restype = sz
        L.vs_select_both.argtypes = [P, P, i32, i32, f64, i32, i32, P, P, P, P, P, sz, P]
        L.vs_select_both.restype = i32
        L.vs_aggregate_workspace_bytes.argtypes = [i32, i32]
        L.vs_aggregate_workspace_bytes.restype = sz
        L.vs_attn_aggregate.argtypes = [P, P, P, i32, i32, i32, i32, f32, P, P, P, P, P, sz, P]
        L.vs_attn_aggregate.restype = i32
        L.vs_attn_workspace_bytes.argtypes = [i32, i32, i32, i32]
        L.vs_attn_workspace_bytes.restype = sz
        L.vs_attn_varlen_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
        L.vs_attn_varlen_workspace_bytes.restype = sz
        L.vs_sparse_attn_prefill.argtypes = [P, P, P, i32, i32, i32, i32, i32, f32, P, P, i32, P, P,
                                             i32, P, P, P, sz, P]
        L.vs_sparse_attn_prefill.restype = i32
        L.vs_sparse_attn_prefill_noalloc.argtypes = [P, P, P, i32, i32, i32, i32, i32, f32, P, P, i32,
                                                     P, P, i32, P, P, P]
        L.vs_sparse_attn_prefill_noalloc.restype = i32
        L.vs_sparse_attn_prefill_qh.argtypes = [P, P, P, i32, i32, i32, i32, i32, f32, P, P, i32, P,
                                                P, i32, P, P, P, sz, P]
        L.vs_sparse_attn_prefill_qh.restype = i32
        L.vs_sparse_attn_prefill_varlen.argtypes = [P, P, P, i32, i32, i32, i32, i32, f32, P, i32, i32,
                                                    P, P, i32, P, P, i32, P, P, P, sz, P]
        L.vs_sparse_attn_prefill_varlen.restype = i32
        L.vs_attn_tile_counts.argtypes = [P, i32, i32, i32, i32, i32, P, P]
        L.vs_attn_tile_counts.restype = i32
        L.vs_block_workspace_bytes.argtypes = [i32, i32, i32]
        L.vs_block_workspace_bytes.restype = sz
        L.vs_block_discover.argtypes = [P, P, i32, i32, i32, i32, f32, i32, f32, P, i32, P, P, sz, P]
        L.vs_block_discover.restype = i32
        L.vs_block_attn_workspace_bytes.argtypes = []
        L.vs_block_attn_workspace_bytes.restype = sz
        L.vs_block_attn_prefill.argtypes = [P, P, P, i32, i32, i32, i32, i32, f32, P, i32, P, P, P,
                                            sz, P]
        L.vs_block_attn_prefill.restype = i32
        L.vs_status_str.argtypes = [i32]
        L.vs_status_str.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().vs_status_str(int(status)).decode()


vs_status_str = status_str


def _check(fn: str, status: int):
    if status != VS_OK:
        raise VSError(fn, status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor, stream=None):
    s = torch.cuda.current_stream(t.device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _on_stream(fn):
    """Run a wrapper with `stream` (when given) as torch's current stream, so
    that every tensor it allocates -- outputs, workspaces, temporaries -- comes
    from that stream's pool.  A temporary freed on return then cannot be handed
    to work on another stream while the kernels enqueued on `stream` still
    read or write it."""
    sig = inspect.signature(fn)

    @functools.wraps(fn)
    def wrapper(*args, **kwargs):
        stream = sig.bind(*args, **kwargs).arguments.get("stream")
        if stream is None:
            return fn(*args, **kwargs)
        with torch.cuda.stream(stream):
            return fn(*args, **kwargs)
    return wrapper


def _need(t: torch.Tensor, name: str, dtype, ndim: int, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


@_on_stream
def vs_index(k_rope: torch.Tensor, v: torch.Tensor, w1: torch.Tensor, w2: torch.Tensor,
             vlog: torch.Tensor | None = None, slog: torch.Tensor | None = None, stream=None):
    """VSIndexer logits.  k_rope, v: bf16 [h_kv, n, d]; w1: bf16 [hidden, 2d];
    w2: bf16 [2, hidden].  Returns fp32 (vlog, slog) [h_kv, n]."""
    _need(k_rope, "k_rope", torch.bfloat16, 3)
    dev = k_rope.device
    _need(v, "v", torch.bfloat16, 3, dev)
    _need(w1, "w1", torch.bfloat16, 2, dev)
    _need(w2, "w2", torch.bfloat16, 2, dev)
    h_kv, n, d = k_rope.shape
    if v.shape != k_rope.shape or w1.shape[1] != 2 * d or w2.shape != (2, w1.shape[0]):
        raise ValueError("vs_index: inconsistent shapes")
    vlog = torch.empty((h_kv, n), dtype=torch.float32, device=dev) if vlog is None else vlog
    slog = torch.empty((h_kv, n), dtype=torch.float32, device=dev) if slog is None else slog
    for t, nm in ((vlog, "vlog"), (slog, "slog")):
        _need(t, nm, torch.float32, 2, dev)
        if t.shape != (h_kv, n):
            raise ValueError(f"{nm} must be [h_kv, n]")
    st = lib().vs_index(_ptr(k_rope), _ptr(v), h_kv, n, d, w1.shape[0], _ptr(w1), _ptr(w2),
                        _ptr(vlog), _ptr(slog), _stream(k_rope, stream))
    _check("vs_index", st)
    return vlog, slog


def vs_select_workspace_bytes(heads: int, n: int) -> int:
    return int(lib().vs_select_workspace_bytes(heads, n))


def _select_outputs(fn, logit, cap, idx, count, workspace):
    _need(logit, "logit", torch.float32, 2)
    dev = logit.device
    heads, n = logit.shape
    idx = torch.empty((heads, cap), dtype=torch.int32, device=dev) if idx is None else idx
    count = torch.empty((heads,), dtype=torch.int32, device=dev) if count is None else count
    _need(idx, "idx", torch.int32, 2, dev)
    _need(count, "count", torch.int32, 1, dev)
    if idx.shape != (heads, cap) or count.shape != (heads,):
        raise ValueError(f"{fn}: idx must be [heads, cap] and count [heads]")
    need = vs_select_workspace_bytes(heads, n)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, 1, dev)
    return heads, n, idx, count, workspace


@_on_stream
def vs_select_threshold(logit: torch.Tensor, kind: int, alpha: float, cap: int,
                        idx: torch.Tensor | None = None, count: torch.Tensor | None = None,
                        workspace: torch.Tensor | None = None, stream=None):
    """Max-based dynamic threshold: per head the candidates whose softmax score
    is at least alpha times the largest, at most cap of them.  logit: fp32
    [heads, n].  Returns int32 (idx [heads, cap] ascending then -1, count [heads])."""
    heads, n, idx, count, workspace = _select_outputs("vs_select_threshold", logit, cap, idx, count,
                                                      workspace)
    st = lib().vs_select_threshold(_ptr(logit), heads, n, int(kind), float(alpha), int(cap), _ptr(idx),
                                   _ptr(count), _ptr(workspace), workspace.numel(),
                                   _stream(logit, stream))
    _check("vs_select_threshold", st)
    return idx, count


@_on_stream
def vs_select(logit: torch.Tensor, kind: int, mass: float, cap: int, idx: torch.Tensor | None = None,
              count: torch.Tensor | None = None, workspace: torch.Tensor | None = None, stream=None):
    """Cumulative-mass selection.  logit: fp32 [heads, n].  kind: VS_VERTICAL
    or VS_SLASH.  Returns int32 (idx [heads, cap] ascending then -1, count [heads])."""
    _need(logit, "logit", torch.float32, 2)
    dev = logit.device
    heads, n = logit.shape
    idx = torch.empty((heads, cap), dtype=torch.int32, device=dev) if idx is None else idx
    count = torch.empty((heads,), dtype=torch.int32, device=dev) if count is None else count
    _need(idx, "idx", torch.int32, 2, dev)
    _need(count, "count", torch.int32, 1, dev)
    if idx.shape != (heads, cap) or count.shape != (heads,):
        raise ValueError("vs_select: idx must be [heads, cap] and count [heads]")
    need = vs_select_workspace_bytes(heads, n)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, 1, dev)
    st = lib().vs_select(_ptr(logit), heads, n, int(kind), float(mass), int(cap), _ptr(idx),
                         _ptr(count), _ptr(workspace), workspace.numel(), _stream(logit, stream))
    _check("vs_select", st)
    return idx, count


def vs_attn_workspace_bytes(h_kv: int, n: int, cap_v: int, cap_s: int) -> int:
    return int(lib().vs_attn_workspace_bytes(h_kv, n, cap_v, cap_s))


def vs_attn_varlen_workspace_bytes(sets: int, nseq: int, max_len: int, cap_v: int, cap_s: int) -> int:
    """Workspace bytes of a packed batch: nseq sequences of at most max_len
    positions, `sets` index-set rows each."""
    return int(lib().vs_attn_varlen_workspace_bytes(sets, nseq, max_len, cap_v, cap_s))


def vs_select_both_workspace_bytes(heads: int, n: int) -> int:
    return int(lib().vs_select_both_workspace_bytes(heads, n))


@_on_stream
def vs_select_both(vlog: torch.Tensor, slog: torch.Tensor, mass: float, cap_v: int, cap_s: int,
                   v_idx: torch.Tensor | None = None, v_cnt: torch.Tensor | None = None,
                   s_off: torch.Tensor | None = None, s_cnt: torch.Tensor | None = None,
                   workspace: torch.Tensor | None = None, stream=None):
    """Both cumulative-mass selections of a layer in one launch chain:
    vlog as VERTICAL (cap_v), slog as SLASH (cap_s), fp32 [heads, n] each.
    Returns int32 (v_idx [heads, cap_v], v_cnt [heads], s_off [heads, cap_s],
    s_cnt [heads]), bit-identical to two vs_select calls."""
    _need(vlog, "vlog", torch.float32, 2)
    dev = vlog.device
    _need(slog, "slog", torch.float32, 2, dev)
    if slog.shape != vlog.shape:
        raise ValueError("vs_select_both: vlog and slog must have the same shape")
    heads, n = vlog.shape
    v_idx = torch.empty((heads, cap_v), dtype=torch.int32, device=dev) if v_idx is None else v_idx
    s_off = torch.empty((heads, cap_s), dtype=torch.int32, device=dev) if s_off is None else s_off
    v_cnt = torch.empty((heads,), dtype=torch.int32, device=dev) if v_cnt is None else v_cnt
    s_cnt = torch.empty((heads,), dtype=torch.int32, device=dev) if s_cnt is None else s_cnt
    for t, nm, shape in ((v_idx, "v_idx", (heads, cap_v)), (s_off, "s_off", (heads, cap_s)),
                         (v_cnt, "v_cnt", (heads,)), (s_cnt, "s_cnt", (heads,))):
        _need(t, nm, torch.int32, len(shape), dev)
        if t.shape != shape:
            raise ValueError(f"vs_select_both: {nm} must be {list(shape)}")
    need = vs_select_both_workspace_bytes(heads, n)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, 1, dev)
    st = lib().vs_select_both(_ptr(vlog), _ptr(slog), heads, n, float(mass), int(cap_v), int(cap_s),
                              _ptr(v_idx), _ptr(v_cnt), _ptr(s_off), _ptr(s_cnt), _ptr(workspace),
                              workspace.numel(), _stream(vlog, stream))
    _check("vs_select_both", st)
    return v_idx, v_cnt, s_off, s_cnt


@_on_stream
def vs_sparse_attn_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                           v_idx: torch.Tensor, v_cnt: torch.Tensor, s_off: torch.Tensor,
                           s_cnt: torch.Tensor, scale: float | None = None,
                           out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                           want_lse: bool = True, workspace: torch.Tensor | None = None,
                           stream=None):
    """Vertical-slash sparse causal prefill.  q [h_q, n, d], k/v [h_kv, n, d]
    (bf16 or fp32, all the same); index lists int32 [h_kv, cap] with counts
    int32 [h_kv].  Returns (out [h_q, n, d] in the input dtype, lse fp32 [h_q, n])."""
    if q.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("q must be bf16 or fp32")
    dt = VS_BF16 if q.dtype == torch.bfloat16 else VS_F32
    _need(q, "q", q.dtype, 3)
    dev = q.device
    _need(k, "k", q.dtype, 3, dev)
    _need(v, "v", q.dtype, 3, dev)
    for t, nm in ((v_idx, "v_idx"), (s_off, "s_off")):
        _need(t, nm, torch.int32, 2, dev)
    for t, nm in ((v_cnt, "v_cnt"), (s_cnt, "s_cnt")):
        _need(t, nm, torch.int32, 1, dev)
    h_q, n, d = q.shape
    h_kv = k.shape[0]
    if k.shape != (h_kv, n, d) or v.shape != k.shape:
        raise ValueError("vs_sparse_attn_prefill: k and v must be [h_kv, n, d]")
    if v_idx.shape[0] != h_kv or s_off.shape[0] != h_kv or v_cnt.shape != (h_kv,) or s_cnt.shape != (h_kv,):
        raise ValueError("vs_sparse_attn_prefill: index lists must have h_kv rows")
    cap_v, cap_s = v_idx.shape[1], s_off.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out = torch.empty_like(q) if out is None else out
    _need(out, "out", q.dtype, 3, dev)
    if out.shape != q.shape:
        raise ValueError("out must match q")
    if want_lse and lse is None:
        lse = torch.empty((h_q, n), dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, 2, dev)
        if lse.shape != (h_q, n):
            raise ValueError("lse must be [h_q, n]")
    need = vs_attn_workspace_bytes(h_kv, n, cap_v, cap_s)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, 1, dev)
    st = lib().vs_sparse_attn_prefill(_ptr(q), _ptr(k), _ptr(v), dt, h_q, h_kv, n, d, scale,
                                      _ptr(v_idx), _ptr(v_cnt), cap_v, _ptr(s_off), _ptr(s_cnt),
                                      cap_s, _ptr(out), _ptr(lse), _ptr(workspace),
                                      workspace.numel(), _stream(q, stream))
    _check("vs_sparse_attn_prefill", st)
    return out, lse


NOALLOC_SCRATCH_BYTES = 64 << 20  # the static workspace of vs_sparse_attn_prefill_noalloc, per GPU


@_on_stream
def vs_sparse_attn_prefill_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                                   v_idx: torch.Tensor, v_cnt: torch.Tensor, s_off: torch.Tensor,
                                   s_cnt: torch.Tensor, out: torch.Tensor, lse: torch.Tensor | None,
                                   scale: float | None = None, stream=None):
    """vs_sparse_attn_prefill with the library's static workspace, for callers
    that cannot allocate: the caller passes every output (out, and lse or
    None) and nothing is allocated here or in the library.  Calls that overlap
    on one GPU share that workspace and race."""
    if out is None:
        raise ValueError("vs_sparse_attn_prefill_noalloc: the caller passes `out` (nothing is allocated)")
    dt, dev, h_q, h_kv, n, d, out, lse = _attn_common(q, k, v, out, lse, False, None)
    for t, nm in ((v_idx, "v_idx"), (s_off, "s_off")):
        _need(t, nm, torch.int32, 2, dev)
    for t, nm in ((v_cnt, "v_cnt"), (s_cnt, "s_cnt")):
        _need(t, nm, torch.int32, 1, dev)
    if v_idx.shape[0] != h_kv or s_off.shape[0] != h_kv or v_cnt.shape != (h_kv,) or s_cnt.shape != (h_kv,):
        raise ValueError("vs_sparse_attn_prefill_noalloc: index lists must have h_kv rows")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = lib().vs_sparse_attn_prefill_noalloc(_ptr(q), _ptr(k), _ptr(v), dt, h_q, h_kv, n, d, scale,
                                              _ptr(v_idx), _ptr(v_cnt), v_idx.shape[1], _ptr(s_off),
                                              _ptr(s_cnt), s_off.shape[1], _ptr(out), _ptr(lse),
                                              _stream(q, stream))
    _check("vs_sparse_attn_prefill_noalloc", st)
    return out, lse


def _attn_common(q, k, v, out, lse, want_lse, rows):
    if q.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("q must be bf16 or fp32")
    dt = VS_BF16 if q.dtype == torch.bfloat16 else VS_F32
    _need(q, "q", q.dtype, 3)
    dev = q.device
    _need(k, "k", q.dtype, 3, dev)
    _need(v, "v", q.dtype, 3, dev)
    h_q, n, d = q.shape
    h_kv = k.shape[0]
    if k.shape != (h_kv, n, d) or v.shape != k.shape:
        raise ValueError("k and v must be [h_kv, rows, d] like q")
    out = torch.empty_like(q) if out is None else out
    _need(out, "out", q.dtype, 3, dev)
    if out.shape != q.shape:
        raise ValueError("out must match q")
    if want_lse and lse is None:
        lse = torch.empty((h_q, n), dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, 2, dev)
        if lse.shape != (h_q, n):
            raise ValueError("lse must be [h_q, rows]")
    return dt, dev, h_q, h_kv, n, d, out, lse


@_on_stream
def vs_sparse_attn_prefill_qh(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                              v_idx: torch.Tensor, v_cnt: torch.Tensor, s_off: torch.Tensor,
                              s_cnt: torch.Tensor, scale: float | None = None,
                              out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                              want_lse: bool = True, workspace: torch.Tensor | None = None,
                              stream=None):
    """Vertical-slash prefill with one index set per query head: lists int32
    [h_q, cap] and counts [h_q]; query head h reads K/V head h // (h_q/h_kv)."""
    dt, dev, h_q, h_kv, n, d, out, lse = _attn_common(q, k, v, out, lse, want_lse, None)
    for t, nm in ((v_idx, "v_idx"), (s_off, "s_off")):
        _need(t, nm, torch.int32, 2, dev)
    for t, nm in ((v_cnt, "v_cnt"), (s_cnt, "s_cnt")):
        _need(t, nm, torch.int32, 1, dev)
    if v_idx.shape[0] != h_q or s_off.shape[0] != h_q or v_cnt.shape != (h_q,) or s_cnt.shape != (h_q,):
        raise ValueError("vs_sparse_attn_prefill_qh: index lists must have h_q rows")
    cap_v, cap_s = v_idx.shape[1], s_off.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    need = vs_attn_workspace_bytes(h_q, n, cap_v, cap_s)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, 1, dev)
    st = lib().vs_sparse_attn_prefill_qh(_ptr(q), _ptr(k), _ptr(v), dt, h_q, h_kv, n, d, scale,
                                         _ptr(v_idx), _ptr(v_cnt), cap_v, _ptr(s_off), _ptr(s_cnt),
                                         cap_s, _ptr(out), _ptr(lse), _ptr(workspace),
                                         workspace.numel(), _stream(q, stream))
    _check("vs_sparse_attn_prefill_qh", st)
    return out, lse


@_on_stream
def vs_sparse_attn_prefill_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens,
                                  v_idx: torch.Tensor, v_cnt: torch.Tensor, s_off: torch.Tensor,
                                  s_cnt: torch.Tensor, per_query_head: bool = False,
                                  scale: float | None = None, out: torch.Tensor | None = None,
                                  lse: torch.Tensor | None = None, want_lse: bool = True,
                                  workspace: torch.Tensor | None = None, stream=None):
    """Packed batch of causal sequences: q [h_q, total, d], k/v [h_kv, total, d];
    cu_seqlens (host sequence of nseq+1 ints from 0 to total); lists int32
    [nseq, S, cap] and counts [nseq, S] with S = h_kv (or h_q when
    per_query_head), positions relative to each sequence's first row."""
    dt, dev, h_q, h_kv, n, d, out, lse = _attn_common(q, k, v, out, lse, want_lse, None)
    cu = (ctypes.c_int32 * len(cu_seqlens))(*[int(x) for x in cu_seqlens])
    nseq = len(cu_seqlens) - 1
    sets = h_q if per_query_head else h_kv
    for t, nm in ((v_idx, "v_idx"), (s_off, "s_off")):
        _need(t, nm, torch.int32, 3, dev)
    for t, nm in ((v_cnt, "v_cnt"), (s_cnt, "s_cnt")):
        _need(t, nm, torch.int32, 2, dev)
    if v_idx.shape[:2] != (nseq, sets) or s_off.shape[:2] != (nseq, sets) or \
            v_cnt.shape != (nseq, sets) or s_cnt.shape != (nseq, sets):
        raise ValueError("vs_sparse_attn_prefill_varlen: lists must be [nseq, sets, cap]")
    cap_v, cap_s = v_idx.shape[2], s_off.shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    max_len = max([int(cu_seqlens[i + 1]) - int(cu_seqlens[i]) for i in range(nseq)] + [1])
    need = vs_attn_varlen_workspace_bytes(sets, max(nseq, 1), max_len, cap_v, cap_s)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, 1, dev)
    st = lib().vs_sparse_attn_prefill_varlen(_ptr(q), _ptr(k), _ptr(v), dt, h_q, h_kv, n, d, scale,
                                             ctypes.cast(cu, ctypes.c_void_p), nseq,
                                             1 if per_query_head else 0, _ptr(v_idx), _ptr(v_cnt),
                                             cap_v, _ptr(s_off), _ptr(s_cnt), cap_s, _ptr(out),
                                             _ptr(lse), _ptr(workspace), workspace.numel(),
                                             _stream(q, stream))
    _check("vs_sparse_attn_prefill_varlen", st)
    return out, lse


def vs_aggregate_workspace_bytes(h_kv: int, n: int) -> int:
    return int(lib().vs_aggregate_workspace_bytes(h_kv, n))


@_on_stream
def vs_attn_aggregate(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: float | None = None,
                      out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                      a_v: torch.Tensor | None = None, a_s: torch.Tensor | None = None,
                      workspace: torch.Tensor | None = None, stream=None):
    """Dense causal attention plus its weights summed per KV head along key
    columns (a_v) and diagonals (a_s).  q [h_q, n, d], k/v [h_kv, n, d] bf16.
    Returns (out, lse, a_v [h_kv, n], a_s [h_kv, n])."""
    _need(q, "q", torch.bfloat16, 3)
    dev = q.device
    _need(k, "k", torch.bfloat16, 3, dev)
    _need(v, "v", torch.bfloat16, 3, dev)
    h_q, n, d = q.shape
    h_kv = k.shape[0]
    if k.shape != (h_kv, n, d) or v.shape != (h_kv, n, d):
        raise ValueError("vs_attn_aggregate: k and v must be [h_kv, n, d] like q")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((h_q, n), dtype=torch.float32, device=dev) if lse is None else lse
    a_v = torch.empty((h_kv, n), dtype=torch.float32, device=dev) if a_v is None else a_v
    a_s = torch.empty((h_kv, n), dtype=torch.float32, device=dev) if a_s is None else a_s
    _need(out, "out", torch.bfloat16, 3, dev)
    _need(lse, "lse", torch.float32, 2, dev)
    _need(a_v, "a_v", torch.float32, 2, dev)
    _need(a_s, "a_s", torch.float32, 2, dev)
    need = vs_aggregate_workspace_bytes(h_kv, n)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, 1, dev)
    st = lib().vs_attn_aggregate(_ptr(q), _ptr(k), _ptr(v), h_q, h_kv, n, d, scale, _ptr(out), _ptr(lse),
                                 _ptr(a_v), _ptr(a_s), _ptr(workspace), workspace.numel(),
                                 _stream(q, stream))
    _check("vs_attn_aggregate", st)
    return out, lse, a_v, a_s


def vs_attn_tile_counts(workspace: torch.Tensor, h_kv: int, n: int, cap_v: int, cap_s: int,
                        h_q: int, stream=None):
    """(contiguous tiles, gathered tiles, query rows per tile, keys per tile)
    of the last vs_sparse_attn_prefill that used ``workspace`` (synchronous)."""
    tiles = (ctypes.c_int64 * 4)()
    st = lib().vs_attn_tile_counts(_ptr(workspace), h_kv, n, cap_v, cap_s, h_q,
                                   ctypes.cast(tiles, ctypes.c_void_p), _stream(workspace, stream))
    _check("vs_attn_tile_counts", st)
    return tuple(int(x) for x in tiles)


BLOCK = 64  # query and key block size of the block-sparse mode


def vs_block_workspace_bytes(h_kv: int, n: int, d: int) -> int:
    return int(lib().vs_block_workspace_bytes(h_kv, n, d))


def block_words_per_row(n: int) -> int:
    return ((n + BLOCK - 1) // BLOCK + 31) // 32


@_on_stream
def vs_block_discover(q: torch.Tensor, k: torch.Tensor, skel: int, alpha: float,
                      scale: float | None = None, mask: torch.Tensor | None = None,
                      want_score: bool = False, workspace: torch.Tensor | None = None,
                      stream=None):
    """FlashPrefill block discovery: per (KV head, query block of 64) the key
    blocks whose skeleton-probe score is at least alpha times the best, and
    the diagonal block.  q [h_q, n, d], k [h_kv, n, d] bf16.  Returns mask
    int32 [h_kv, nb, words] (bit b of word w <-> key block 32 w + b; the words
    are unsigned), plus score fp32 [h_kv, nb, nb] when want_score."""
    _need(q, "q", torch.bfloat16, 3)
    dev = q.device
    _need(k, "k", torch.bfloat16, 3, dev)
    h_q, n, d = q.shape
    h_kv = k.shape[0]
    if k.shape != (h_kv, n, d):
        raise ValueError("vs_block_discover: k must be [h_kv, n, d] like q")
    nb = (n + BLOCK - 1) // BLOCK
    wpr = block_words_per_row(n)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    mask = torch.empty((h_kv, nb, wpr), dtype=torch.int32, device=dev) if mask is None else mask
    _need(mask, "mask", torch.int32, 3, dev)
    if mask.shape[:2] != (h_kv, nb):
        raise ValueError("vs_block_discover: mask must be [h_kv, nb, words]")
    score = torch.empty((h_kv, nb, nb), dtype=torch.float32, device=dev) if want_score else None
    need = vs_block_workspace_bytes(h_kv, n, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, 1, dev)
    st = lib().vs_block_discover(_ptr(q), _ptr(k), h_q, h_kv, n, d, scale, int(skel), float(alpha),
                                 _ptr(mask), mask.shape[2], _ptr(score), _ptr(workspace),
                                 workspace.numel(), _stream(q, stream))
    _check("vs_block_discover", st)
    return (mask, score) if want_score else mask


@_on_stream
def vs_block_attn_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, mask: torch.Tensor,
                          scale: float | None = None, out: torch.Tensor | None = None,
                          lse: torch.Tensor | None = None, want_lse: bool = True,
                          workspace: torch.Tensor | None = None, stream=None):
    """Block-sparse causal prefill: row i of a query head of KV head g attends
    to keys j <= i whose block j // 64 is set in mask[g, i // 64].  q [h_q, n,
    d], k/v [h_kv, n, d] (bf16 or fp32); mask int32 [h_kv, nb, words].
    Returns (out, lse fp32 [h_q, n])."""
    if q.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("q must be bf16 or fp32")
    dt = VS_BF16 if q.dtype == torch.bfloat16 else VS_F32
    _need(q, "q", q.dtype, 3)
    dev = q.device
    _need(k, "k", q.dtype, 3, dev)
    _need(v, "v", q.dtype, 3, dev)
    _need(mask, "mask", torch.int32, 3, dev)
    h_q, n, d = q.shape
    h_kv = k.shape[0]
    if k.shape != (h_kv, n, d) or v.shape != k.shape:
        raise ValueError("vs_block_attn_prefill: k and v must be [h_kv, n, d]")
    if mask.shape[:2] != (h_kv, (n + BLOCK - 1) // BLOCK):
        raise ValueError("vs_block_attn_prefill: mask must be [h_kv, nb, words]")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out = torch.empty_like(q) if out is None else out
    _need(out, "out", q.dtype, 3, dev)
    if out.shape != q.shape:
        raise ValueError("out must match q")
    if want_lse and lse is None:
        lse = torch.empty((h_q, n), dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, 2, dev)
        if lse.shape != (h_q, n):
            raise ValueError("lse must be [h_q, n]")
    if workspace is None:
        workspace = torch.empty(int(lib().vs_block_attn_workspace_bytes()), dtype=torch.uint8,
                                device=dev)
    _need(workspace, "workspace", torch.uint8, 1, dev)
    st = lib().vs_block_attn_prefill(_ptr(q), _ptr(k), _ptr(v), dt, h_q, h_kv, n, d, scale,
                                     _ptr(mask), mask.shape[2], _ptr(out), _ptr(lse),
                                     _ptr(workspace), workspace.numel(), _stream(q, stream))
    _check("vs_block_attn_prefill", st)
    return out, lse


def exported_symbols():
    return _SYMBOLS


@_on_stream
def vs_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, w1: torch.Tensor, w2: torch.Tensor,
               mass: float = 0.95, cap_v: int | None = None, cap_s: int | None = None,
               scale: float | None = None, stream=None):
    """One vertical-slash sparse prefill layer the way VSPrefill's inference
    pipeline runs it (VSPrefill, English page, section 3 "Adaptive Inference
    Pipeline"): the indexer scores every position from [K_rope | V]
    (vs_index), the cumulative-mass budget picks each KV head's columns and
    slash offsets (vs_select, twice), and sparse attention runs over their
    union (vs_sparse_attn_prefill; the two selections run as one chain,
    vs_select_both).  q bf16 [h_q, n, d]; k (already rotated)
    and v bf16 [h_kv, n, d]; w1 bf16 [hidden, 2d]; w2 bf16 [2, hidden].
    cap_v / cap_s bound the budgets (default n, i.e. uncapped).  Every launch
    goes on one stream; nothing is synchronised.  Returns (out, lse,
    (v_idx, v_cnt, s_off, s_cnt))."""
    h_kv, n, _ = k.shape
    cap_v = n if cap_v is None else int(cap_v)
    cap_s = n if cap_s is None else int(cap_s)
    vlog, slog = vs_index(k, v, w1, w2, stream=stream)
    ws = torch.empty(max(vs_select_both_workspace_bytes(h_kv, n), 1), dtype=torch.uint8, device=k.device)
    v_idx, v_cnt, s_off, s_cnt = vs_select_both(vlog, slog, mass, cap_v, cap_s, workspace=ws, stream=stream)
    out, lse = vs_sparse_attn_prefill(q, k, v, v_idx, v_cnt, s_off, s_cnt, scale=scale, stream=stream)
    return out, lse, (v_idx, v_cnt, s_off, s_cnt)
