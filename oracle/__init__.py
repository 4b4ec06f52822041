"""fp64 CPU oracle for vertical-slash sparse prefill -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It is independent of the HIP path: it
shares no kernels, headers, helpers or constants with
``vertical_slash_sparse_amd`` and neither imports the other.  The arithmetic
lives in ``vs_oracle.c`` (plain C, fp64, OpenMP over rows); this module only
builds that file with gcc and marshals numpy arrays to it.

Every function here is pinned by ``tests/test_oracle.py`` (vertical-slash
path, selection, indexer, aggregation) and ``tests/test_oracle_blocks.py``
(FlashPrefill block discovery and block-sparse attention) against brute
force, closed forms, library routines or hand-derived values.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "vs_oracle.c")
# VS_SANITIZE=1 selects a build instrumented with AddressSanitizer and
# UndefinedBehaviorSanitizer (clang's runtime, which the process must preload;
# see the sanitizer test in tests/)
SANITIZE = os.environ.get("VS_SANITIZE") == "1"
_LIB = os.path.join(_HERE, "libvs_oracle_san.so" if SANITIZE else "libvs_oracle.so")
_CLANG = "/opt/rocm/llvm/bin/clang"
_CLANG_LIB = "/opt/rocm/llvm/lib"

BF16, F32, F64 = 0, 1, 2
VERTICAL, SLASH = 0, 1


def build(force: bool = True, sanitize: bool | None = None) -> str:
    """Compile vs_oracle.c with gcc (fp64, no FMA contraction, OpenMP); with
    ``sanitize`` (default: VS_SANITIZE=1), with clang and -fsanitize=address,
    undefined into libvs_oracle_san.so instead."""
    sanitize = SANITIZE if sanitize is None else sanitize
    lib_path = os.path.join(_HERE, "libvs_oracle_san.so" if sanitize else "libvs_oracle.so")
    if force or not os.path.exists(lib_path) or os.path.getmtime(lib_path) < os.path.getmtime(_SRC):
        tmp = lib_path + ".tmp"
        if sanitize:
            cmd = [_CLANG, "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                   "-ffp-contract=off", "-fno-fast-math", "-fsanitize=address,undefined",
                   "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", _SRC, "-o", tmp,
                   "-L" + _CLANG_LIB, "-Wl,-rpath," + _CLANG_LIB, "-lm"]
        else:
            cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                   "-fno-fast-math", _SRC, "-o", tmp, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, lib_path)
    return lib_path


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_double
        L.vso_attn_rows.argtypes = [P, P, P, i32, i32, i32, i32, i32, f64, P, P, i32, P, P, i32,
                                    P, P, i64, P, P, i32]
        L.vso_attn_rows.restype = i32
        L.vso_index.argtypes = [P, P, i32, i32, i32, i32, i32, P, P, i32, P, P, i32]
        L.vso_index.restype = i32
        L.vso_select.argtypes = [P, i32, i32, i32, f64, i32, P, P, P, P]
        L.vso_select.restype = i32
        L.vso_select_threshold.argtypes = [P, i32, i32, i32, f64, i32, P, P, P]
        L.vso_select_threshold.restype = i32
        L.vso_aggregate.argtypes = [P, P, i32, i32, i32, i32, i32, f64, P, P, i32]
        L.vso_aggregate.restype = i32
        L.vso_exp_spec.argtypes = [ctypes.c_float]
        L.vso_exp_spec.restype = ctypes.c_float
        L.vso_mass_u.argtypes = [ctypes.c_float]
        L.vso_mass_u.restype = ctypes.c_uint64
        L.vso_row_set.argtypes = [P, P, i32, P, P, i32, i32, i32, P]
        L.vso_row_set.restype = i32
        L.vso_pair_count.argtypes = [P, P, i32, P, P, i32, i32, i32]
        L.vso_pair_count.restype = i64
        L.vso_block_means.argtypes = [P, i32, i32, i32, i32, i32, P]
        L.vso_block_means.restype = i32
        L.vso_block_scores.argtypes = [P, i32, i32, i32, i32, i32, f64, i32, i32, P, P, P, i64, P,
                                       i32]
        L.vso_block_scores.restype = i32
        L.vso_block_select.argtypes = [P, i32, i32, ctypes.c_float, P, i32]
        L.vso_block_select.restype = i32
        L.vso_block_attn_rows.argtypes = [P, P, P, i32, i32, i32, i32, i32, f64, i32, P, i32, P,
                                          P, i64, P, P, i32]
        L.vso_block_attn_rows.restype = i32
        L.vso_num_threads.restype = i32
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.float64:
        return F64
    raise TypeError(f"unsupported oracle input dtype {a.dtype}")


def _c(a, dtype=None):
    return np.ascontiguousarray(a if dtype is None else np.asarray(a, dtype=dtype))


def num_threads() -> int:
    return int(lib().vso_num_threads())


def attn(q, k, v, vidx, vcnt, soff, scnt, scale=None, rows=None, nthreads=0):
    """Sparse causal attention over the vertical-slash index sets.

    q [hq,n,d], k/v [hkv,n,d] as bf16 bits (uint16), fp32 or fp64; index lists
    int32 [hkv, cap] ascending with counts [hkv].  ``rows`` is None (every row)
    or an int array [m, 2] of (head, row).  Returns (out [m, d], lse [m]) in
    fp64, or ([hq, n, d], [hq, n]) when ``rows`` is None."""
    q, k, v = _c(q), _c(k), _c(v)
    hq, n, d = q.shape
    hkv = k.shape[0]
    assert k.shape == v.shape == (hkv, n, d) and q.dtype == k.dtype == v.dtype
    vidx, vcnt, soff, scnt = (_c(x, np.int32) for x in (vidx, vcnt, soff, scnt))
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    full = rows is None
    if full:
        hh, ii = np.meshgrid(np.arange(hq), np.arange(n), indexing="ij")
        rows = np.stack([hh.ravel(), ii.ravel()], axis=1)
    rows = _c(rows, np.int32).reshape(-1, 2)
    rh, ri = _c(rows[:, 0]), _c(rows[:, 1])
    m = rows.shape[0]
    out = np.empty((m, d), dtype=np.float64)
    lse = np.empty(m, dtype=np.float64)
    rc = lib().vso_attn_rows(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), hq, hkv, n, d, scale,
                             _ptr(vidx), _ptr(vcnt), vidx.shape[1], _ptr(soff), _ptr(scnt),
                             soff.shape[1], _ptr(rh), _ptr(ri), m, _ptr(out), _ptr(lse),
                             int(nthreads))
    if rc:
        raise ValueError("oracle attn: invalid arguments")
    if full:
        return out.reshape(hq, n, d), lse.reshape(hq, n)
    return out, lse


def attn_qh(q, k, v, vidx, vcnt, soff, scnt, scale=None, rows=None, nthreads=0):
    """Like attn() with one index set per QUERY head (lists [hq, cap]): the
    same definition with every query head's K/V head repeated, so that the
    set of head h is the set of "KV head" h."""
    q = _c(q)
    hq = q.shape[0]
    group = hq // k.shape[0]
    k = np.repeat(_c(k), group, axis=0)
    v = np.repeat(_c(v), group, axis=0)
    return attn(q, k, v, vidx, vcnt, soff, scnt, scale=scale, rows=rows, nthreads=nthreads)


def attn_varlen(q, k, v, cu_seqlens, vidx, vcnt, soff, scnt, per_query_head=False, scale=None,
                rows=None, nthreads=0):
    """Packed batch: sequence s is rows cu[s]..cu[s+1]-1 of every head and
    attends only within itself, with its own lists vidx[s] ... (positions
    relative to its first row).  Returns (out [hq, total, d], lse [hq, total]),
    or with ``rows`` (int [m, 2] of (head, packed row)) (out [m, d], lse [m])."""
    q, k, v = _c(q), _c(k), _c(v)
    hq, total, d = q.shape
    fn = attn_qh if per_query_head else attn
    cu = [int(x) for x in cu_seqlens]
    if rows is not None:
        rows = _c(rows, np.int32).reshape(-1, 2)
        out = np.zeros((rows.shape[0], d), dtype=np.float64)
        lse = np.zeros(rows.shape[0], dtype=np.float64)
        seq = np.searchsorted(np.array(cu), rows[:, 1], side="right") - 1
        for s in range(len(cu) - 1):
            sel = np.nonzero(seq == s)[0]
            if len(sel) == 0:
                continue
            a, b = cu[s], cu[s + 1]
            local = np.stack([rows[sel, 0], rows[sel, 1] - a], axis=1)
            o, l = fn(q[:, a:b], k[:, a:b], v[:, a:b], vidx[s], vcnt[s], soff[s], scnt[s],
                      scale=scale, rows=local, nthreads=nthreads)
            out[sel] = o
            lse[sel] = l
        return out, lse
    out = np.zeros((hq, total, d), dtype=np.float64)
    lse = np.zeros((hq, total), dtype=np.float64)
    for s in range(len(cu) - 1):
        a, b = cu[s], cu[s + 1]
        if b == a:
            continue
        o, l = fn(q[:, a:b], k[:, a:b], v[:, a:b], vidx[s], vcnt[s], soff[s], scnt[s],
                  scale=scale, nthreads=nthreads)
        out[:, a:b] = o
        lse[:, a:b] = l
    return out, lse


def index(k, v, w1, w2, nthreads=0):
    """VSIndexer logits (vlog, slog) [hkv, n] fp64 from k/v [hkv,n,d]."""
    k, v, w1, w2 = _c(k), _c(v), _c(w1), _c(w2)
    hkv, n, d = k.shape
    hidden = w1.shape[0]
    assert w1.shape == (hidden, 2 * d) and w2.shape == (2, hidden)
    vlog = np.empty((hkv, n), dtype=np.float64)
    slog = np.empty((hkv, n), dtype=np.float64)
    rc = lib().vso_index(_ptr(k), _ptr(v), _dtype_code(k), hkv, n, d, hidden, _ptr(w1), _ptr(w2),
                         _dtype_code(w1), _ptr(vlog), _ptr(slog), int(nthreads))
    if rc:
        raise ValueError("oracle index: invalid arguments")
    return vlog, slog


def select(logit, kind, mass, cap, return_ut=False):
    """Cumulative-mass selection per head.  logit fp32 [heads, n].
    Returns (idx int32 [heads, cap], count int32 [heads])."""
    logit = _c(logit, np.float32)
    heads, n = logit.shape
    idx = np.empty((heads, cap), dtype=np.int32)
    cnt = np.empty(heads, dtype=np.int32)
    U = np.empty(heads, dtype=np.uint64)
    T = np.empty(heads, dtype=np.uint64)
    rc = lib().vso_select(_ptr(logit), heads, n, int(kind), float(mass), int(cap), _ptr(idx),
                          _ptr(cnt), _ptr(U), _ptr(T))
    if rc:
        raise ValueError("oracle select: invalid arguments")
    return (idx, cnt, U, T) if return_ut else (idx, cnt)


def aggregate(q, k, scale=None, nthreads=0):
    """Full causal attention weights of every query head summed per KV head
    along key columns (a_v [hkv, n]) and along diagonals i-j (a_s [hkv, n]),
    fp64, unnormalised."""
    q, k = _c(q), _c(k)
    hq, n, d = q.shape
    hkv = k.shape[0]
    assert k.shape == (hkv, n, d) and q.dtype == k.dtype
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    a_v = np.empty((hkv, n), dtype=np.float64)
    a_s = np.empty((hkv, n), dtype=np.float64)
    rc = lib().vso_aggregate(_ptr(q), _ptr(k), _dtype_code(q), hq, hkv, n, d, scale, _ptr(a_v),
                             _ptr(a_s), int(nthreads))
    if rc:
        raise ValueError("oracle aggregate: invalid arguments")
    return a_v, a_s


def select_threshold(logit, kind, alpha, cap, return_a=False):
    """Max-based dynamic threshold per head: candidates whose softmax score
    is at least alpha times the largest, decided on the quantised masses
    (u >= ceil(alpha * 2^32)), at most cap of them in (score desc, index asc)
    order.  Returns (idx int32 [heads, cap], count int32 [heads])."""
    logit = _c(logit, np.float32)
    heads, n = logit.shape
    idx = np.empty((heads, cap), dtype=np.int32)
    cnt = np.empty(heads, dtype=np.int32)
    A = np.zeros(1, dtype=np.uint64)
    rc = lib().vso_select_threshold(_ptr(logit), heads, n, int(kind), float(alpha), int(cap),
                                    _ptr(idx), _ptr(cnt), _ptr(A))
    if rc:
        raise ValueError("oracle select_threshold: invalid arguments")
    return (idx, cnt, int(A[0])) if return_a else (idx, cnt)


def exp_spec(x) -> np.ndarray:
    f = lib().vso_exp_spec
    return np.array([f(float(t)) for t in np.asarray(x, dtype=np.float32).ravel()],
                    dtype=np.float32).reshape(np.shape(x))


def mass_u(x) -> np.ndarray:
    f = lib().vso_mass_u
    return np.array([f(float(t)) for t in np.asarray(x, dtype=np.float32).ravel()],
                    dtype=np.uint64).reshape(np.shape(x))


def row_set(vidx, vcnt, soff, scnt, g, i):
    vidx, vcnt, soff, scnt = (_c(x, np.int32) for x in (vidx, vcnt, soff, scnt))
    buf = np.empty(i + 1, dtype=np.int32)
    m = lib().vso_row_set(_ptr(vidx), _ptr(vcnt), vidx.shape[1], _ptr(soff), _ptr(scnt),
                          soff.shape[1], int(g), int(i), _ptr(buf))
    return buf[:m].copy()


def pair_count(vidx, vcnt, soff, scnt, g, n) -> int:
    vidx, vcnt, soff, scnt = (_c(x, np.int32) for x in (vidx, vcnt, soff, scnt))
    return int(lib().vso_pair_count(_ptr(vidx), _ptr(vcnt), vidx.shape[1], _ptr(soff),
                                    _ptr(scnt), soff.shape[1], int(g), int(n)))


# ---------------------------------------------------------------- FlashPrefill blocks

BLOCK = 64  # query and key block size of the block-sparse mode


def block_means(k, bs=BLOCK):
    """Mean key of every block of bs positions, fp64 [hkv, nb, d] (the last
    block averages the keys it has)."""
    k = _c(k)
    hkv, n, d = k.shape
    nb = (n + bs - 1) // bs
    kbar = np.empty((hkv, nb, d), dtype=np.float64)
    if lib().vso_block_means(_ptr(k), _dtype_code(k), hkv, n, d, bs, _ptr(kbar)):
        raise ValueError("oracle block_means: invalid arguments")
    return kbar


def block_scores(q, k, skel, scale=None, bs=BLOCK, rows=None, nthreads=0):
    """Block scores [hkv, nb, nb] fp64: for query block I and candidate J < I,
    the softmax probability of J under scale * q . kbar_J averaged over the
    skeleton probes (rows bs*I + m*(bs/skel) < n of every query head of the
    group); zero for J >= I.  With ``rows`` (int [m, 2] of (g, I)) only those
    query blocks, as [m, nb]."""
    q = _c(q)
    hq, n, d = q.shape
    hkv = k.shape[0]
    assert k.shape == (hkv, n, d) and q.dtype == _c(k).dtype
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    kbar = block_means(k, bs)
    nb = kbar.shape[1]
    if rows is None:
        score = np.empty((hkv, nb, nb), dtype=np.float64)
        rg = ri = None
        m = 0
    else:
        rows = _c(rows, np.int32).reshape(-1, 2)
        rg, ri = _c(rows[:, 0]), _c(rows[:, 1])
        m = rows.shape[0]
        score = np.empty((m, nb), dtype=np.float64)
    if lib().vso_block_scores(_ptr(q), _dtype_code(q), hq, hkv, n, d, scale, bs, int(skel),
                              _ptr(kbar), None if rg is None else _ptr(rg),
                              None if ri is None else _ptr(ri), m, _ptr(score), int(nthreads)):
        raise ValueError("oracle block_scores: invalid arguments")
    return score


def words_per_row(nb):
    return (nb + 31) // 32


def block_select(score, alpha):
    """Max-based threshold on fp32 scores [hkv, nb, nb], decided in fp32:
    keep J < I when score >= alpha * max (one fp32 product), and J = I.
    Returns the mask uint32 [hkv, nb, words_per_row(nb)]."""
    score = _c(score, np.float32)
    hkv, nb, nb2 = score.shape
    assert nb == nb2
    wpr = words_per_row(nb)
    mask = np.empty((hkv, nb, wpr), dtype=np.uint32)
    if lib().vso_block_select(_ptr(score), hkv, nb, float(np.float32(alpha)), _ptr(mask), wpr):
        raise ValueError("oracle block_select: invalid arguments")
    return mask


def mask_to_dense(mask, nb):
    """Block mask words -> bool [hkv, nb, nb]."""
    bits = np.unpackbits(mask.view(np.uint8), axis=-1, bitorder="little")
    return bits[..., :nb].astype(bool)


def block_attn(q, k, v, mask, scale=None, bs=BLOCK, rows=None, nthreads=0):
    """Causal attention of every query head over S_i = {j <= i : block j/bs
    kept for query block i/bs of its KV head}.  Same conventions as attn()."""
    q, k, v = _c(q), _c(k), _c(v)
    hq, n, d = q.shape
    hkv = k.shape[0]
    assert k.shape == v.shape == (hkv, n, d) and q.dtype == k.dtype == v.dtype
    mask = _c(mask, np.uint32)
    nb = (n + bs - 1) // bs
    assert mask.shape[:2] == (hkv, nb)
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    full = rows is None
    if full:
        hh, ii = np.meshgrid(np.arange(hq), np.arange(n), indexing="ij")
        rows = np.stack([hh.ravel(), ii.ravel()], axis=1)
    rows = _c(rows, np.int32).reshape(-1, 2)
    rh, ri = _c(rows[:, 0]), _c(rows[:, 1])
    m = rows.shape[0]
    out = np.empty((m, d), dtype=np.float64)
    lse = np.empty(m, dtype=np.float64)
    if lib().vso_block_attn_rows(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), hq, hkv, n, d, scale,
                                 bs, _ptr(mask), mask.shape[2], _ptr(rh), _ptr(ri), m, _ptr(out),
                                 _ptr(lse), int(nthreads)):
        raise ValueError("oracle block_attn: invalid arguments")
    if full:
        return out.reshape(hq, n, d), lse.reshape(hq, n)
    return out, lse
