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
