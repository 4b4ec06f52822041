"""Shared helpers for the GPU tests: moving seeded numpy inputs to the device
and comparing against the oracle with the stated tolerances."""
from __future__ import annotations

import numpy as np
import torch

import workloads

# attention output vs the fp64 oracle (bf16 inputs, fp32 accumulation)
ATOL_MAX = 2e-2
ATOL_MEAN = 2e-3
# indexer logits vs the fp64 oracle (bf16 inputs, fp32 accumulation)
INDEX_ATOL = 1e-3


def to_dev(a: np.ndarray, device="cuda") -> torch.Tensor:
    """uint16 arrays are bf16 bit patterns; everything else keeps its dtype."""
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def bits_f64(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return workloads.bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def assert_attn_close(out_gpu: np.ndarray, lse_gpu: np.ndarray, out_ref: np.ndarray,
                      lse_ref: np.ndarray, what: str = ""):
    """max-abs <= 2e-2 and mean-abs <= 2e-3 on O and on finite lse; -inf lse
    (empty rows) must match exactly with O == 0 there."""
    assert out_gpu.shape == out_ref.shape
    assert np.isfinite(out_gpu).all(), f"{what}: non-finite output"
    err = np.abs(out_gpu - out_ref)
    assert err.max() <= ATOL_MAX, f"{what}: O max-abs {err.max():.3e}"
    assert err.mean() <= ATOL_MEAN, f"{what}: O mean-abs {err.mean():.3e}"
    empty_ref = np.isneginf(lse_ref)
    assert (np.isneginf(lse_gpu) == empty_ref).all(), f"{what}: empty-row pattern differs"
    assert (out_gpu[empty_ref] == 0).all(), f"{what}: empty rows must be zero"
    fin = ~empty_ref
    if fin.any():
        le = np.abs(lse_gpu[fin] - lse_ref[fin])
        assert le.max() <= ATOL_MAX, f"{what}: lse max-abs {le.max():.3e}"
        assert le.mean() <= ATOL_MEAN, f"{what}: lse mean-abs {le.mean():.3e}"


def _edge_rows(n: int, block: int) -> list:
    return sorted({0, 1, block - 1, block, n - block, n - 2, n - 1} & set(range(n)))


def sample_rows(rng, hq: int, n: int, per_head: int, block: int = 64) -> np.ndarray:
    """(head, row) pairs: first and last rows, both ends of the first and last
    query blocks, and on top of those `per_head` random rows, for every head."""
    fixed = _edge_rows(n, block)
    rows = []
    for h in range(hq):
        extra = rng.choice(n, size=min(per_head, n), replace=False)
        for i in sorted(set(fixed) | set(int(x) for x in extra)):
            rows.append((h, i))
    return np.array(rows, dtype=np.int32)


def stratified_rows(rng, hq: int, n: int, strata: int = 64, per_block: int = 2,
                    whole_blocks: int = 2, block: int = 64) -> np.ndarray:
    """(head, row) pairs spread over the whole sequence, for full-size parity:
    - the edge rows of sample_rows, for every head;
    - per head, the query blocks are cut into `strata` equal runs and one
      block is drawn from each run, `per_block` random rows of it;
    - `whole_blocks` interior query blocks (neither the first nor the last)
      drawn once, every row of them for every head.
    Rows are unique and sorted by (head, row)."""
    nb = (n + block - 1) // block
    fixed = _edge_rows(n, block)
    edges = np.linspace(0, nb, min(strata, nb) + 1).astype(np.int64)
    rows = set()
    for h in range(hq):
        rows.update((h, i) for i in fixed)
        for s in range(len(edges) - 1):
            if edges[s + 1] <= edges[s]:
                continue
            b = int(rng.integers(edges[s], edges[s + 1]))
            r0, r1 = b * block, min(n, (b + 1) * block)
            take = rng.choice(np.arange(r0, r1), size=min(per_block, r1 - r0), replace=False)
            rows.update((h, int(i)) for i in take)
    if nb > 2 and whole_blocks > 0:
        for b in rng.choice(np.arange(1, nb - 1), size=min(whole_blocks, nb - 2), replace=False):
            r0, r1 = int(b) * block, min(n, (int(b) + 1) * block)
            rows.update((h, i) for h in range(hq) for i in range(r0, r1))
    return np.array(sorted(rows), dtype=np.int32)
