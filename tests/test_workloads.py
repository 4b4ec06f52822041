"""The seeded input generators: bf16 rounding of fp64 values is a single
round-to-nearest-even (the rotary embedding is applied in fp64 and rounded
once), checked against integer arithmetic on the fp64 bits."""
import numpy as np

import workloads


def _bf16_exact(x: np.ndarray) -> np.ndarray:
    """Round normal fp64 values to bf16 bits, nearest-even, by integer arithmetic."""
    out = np.zeros(x.shape, np.uint16)
    for i, v in enumerate(x):
        b = int(np.float64(v).view(np.uint64))
        sign, e, m = b >> 63, (b >> 52) & 0x7FF, b & ((1 << 52) - 1)
        if v == 0:
            out[i] = sign << 15
            continue
        full = m | (1 << 52)
        keep, rem, halfway = full >> 45, full & ((1 << 45) - 1), 1 << 44
        if rem > halfway or (rem == halfway and keep & 1):
            keep += 1
        ee = e - 1023 + 127
        if keep >> 8:
            keep >>= 1
            ee += 1
        out[i] = (sign << 15) | (ee << 7) | (keep & 0x7F)
    return out


def test_bf16_single_rounding_with_halfway_cases():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(4000)
    base = workloads.bf16_bits_to_f32(workloads.to_bf16_bits(x[:1000].astype(np.float32))).astype(np.float64)
    half_ulp = np.abs(base) * 2.0 ** -8
    # exact ties, and values a hair either side of a tie (double rounding
    # through plain fp32 gets the latter wrong)
    y = np.concatenate([x, base + np.sign(base) * half_ulp,
                        base + np.sign(base) * half_ulp * (1 + 2.0 ** -30),
                        base + np.sign(base) * half_ulp * (1 - 2.0 ** -30)])
    y = y[np.abs(y) > 1e-30]
    assert np.array_equal(workloads.to_bf16_bits(y), _bf16_exact(y))


def test_bf16_from_fp32_unchanged():
    z = np.random.default_rng(1).standard_normal(2000).astype(np.float32)
    assert np.array_equal(workloads.to_bf16_bits(z), _bf16_exact(z.astype(np.float64)))


def test_banded_zipf_logits_are_a_permuted_zipf_with_runs():
    """The clustered recipe keeps the Zipf pmf (its ranks are a permutation of
    1..n) and puts the best ranks next to its centres: the top 400 indices of
    each head form at most `centers` contiguous runs (one per centre, the one
    at 0 cut in half)."""
    rng = np.random.default_rng(11)
    n, s, centers = 5000, 1.1, 4
    lg = workloads.banded_zipf_logits(rng, 3, n, s, centers)
    for h in range(3):
        ranks = np.rint(np.exp(-lg[h].astype(np.float64) / s)).astype(np.int64)
        assert np.array_equal(np.sort(ranks), np.arange(1, n + 1))
        top = np.sort(np.argsort(ranks)[:400])
        assert top[0] == 0
        assert (np.diff(top) > 1).sum() + 1 <= centers


def test_clustered_scores_slash_vector_is_position_indexed():
    """Offset o's slash score sits at position n-1-o.  The centres (distance
    0) hold the best ranks, and offset 0 is a centre, so position n-1 is among
    the top s_centers slash logits; column 0 is among the top v_centers."""
    w = workloads.WORKLOADS["clustered128k"]
    v, sl = workloads.clustered_scores("clustered128k", n=4096)
    assert v.shape == sl.shape == (8, 4096)
    for h in range(8):
        assert 0 in np.argsort(-v[h])[:w["v_centers"]]
        assert 4095 in np.argsort(-sl[h])[:w["s_centers"]]
