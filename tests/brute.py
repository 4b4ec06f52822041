"""Brute-force checkers for tiny inputs (numpy, fp64).

Deliberately written differently from the oracle: the pattern is an explicit
n x n boolean mask filled cell by cell from the definition, attention is a
dense masked softmax over that mask, and selection is an exhaustive search
over subsets.  Used only to pin the oracle on small cases.
"""
from __future__ import annotations

import itertools

import numpy as np


def explicit_mask(n: int, cols, offs) -> np.ndarray:
    """mask[i, j] = (j <= i) and (j is a selected column or i - j is a selected offset)."""
    cset, oset = set(int(c) for c in cols), set(int(o) for o in offs)
    m = np.zeros((n, n), dtype=bool)
    for i in range(n):
        for j in range(i + 1):
            m[i, j] = (j in cset) or ((i - j) in oset)
    return m


def masked_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, mask: np.ndarray, scale: float):
    """Single head: q, k, v [n, d] fp64; dense scores, masked softmax per row."""
    s = (q @ k.T) * scale
    n, d = q.shape
    out = np.zeros((n, d))
    lse = np.full(n, -np.inf)
    for i in range(n):
        sel = mask[i]
        if not sel.any():
            continue
        row = s[i, sel]
        mx = row.max()
        w = np.exp(row - mx)
        out[i] = (w[:, None] * v[sel]).sum(0) / w.sum()
        lse[i] = mx + np.log(w.sum())
    return out, lse


def min_subset_size(u, T) -> int:
    """Smallest number of items whose masses sum to at least T (exhaustive)."""
    u = [int(x) for x in u]
    for size in range(1, len(u) + 1):
        for comb in itertools.combinations(range(len(u)), size):
            if sum(u[c] for c in comb) >= T:
                return size
    return len(u)
