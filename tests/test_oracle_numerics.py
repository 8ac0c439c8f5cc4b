"""Pins of the oracle's storage rounding to float32 (``oracle.round_f32``).

Every fp32 parity check compares against ``round_f32`` of the float64 oracle, so
the rounding itself is pinned here against hand-worked cases of the IEEE 754
rule (round to nearest, ties to even), against an integer re-derivation of that
rule from the float64 bit pattern, and against torch's own float64 -> float32
conversion (a different library).
"""
import numpy as np
import pytest

import oracle


def test_ties_go_to_even():
    one = 1.0
    u = 2.0 ** -23                                              # float32 spacing at 1
    assert oracle.round_f32(one + 2.0 ** -24) == one            # halfway 1 / 1 + u: even is 1
    assert oracle.round_f32(one + 3 * 2.0 ** -24) == one + 2 * u  # halfway 1 + u / 1 + 2u: even is 1 + 2u
    assert oracle.round_f32(one + 2.0 ** -24 + 2.0 ** -50) == one + u  # just above the tie
    assert oracle.round_f32(one + 2.0 ** -24 - 2.0 ** -50) == one      # just below the tie
    assert oracle.round_f32(-(one + 3 * 2.0 ** -24)) == -(one + 2 * u)
    assert oracle.round_f32(0.1) == 0.100000001490116119384765625     # the float32 nearest to 0.1


def test_subnormals_overflow_and_specials():
    tiny = 2.0 ** -149                                          # smallest float32 subnormal
    assert oracle.round_f32(tiny) == tiny
    assert oracle.round_f32(2.0 ** -150) == 0.0                 # halfway 0 / tiny: even is 0
    assert oracle.round_f32(3 * 2.0 ** -150) == 2 * tiny        # halfway tiny / 2 tiny: even is 2 tiny
    assert oracle.round_f32(2.0 ** -150 + 2.0 ** -200) == tiny
    big = (2.0 - 2.0 ** -23) * 2.0 ** 127                       # largest finite float32
    assert oracle.round_f32(big) == big
    assert oracle.round_f32(big + 2.0 ** 103) == np.inf         # halfway to 2^128: even overflows
    assert oracle.round_f32(big + 2.0 ** 103 - 2.0 ** 80) == big
    assert oracle.round_f32(-np.inf) == -np.inf
    assert np.isnan(oracle.round_f32(np.nan))
    assert oracle.round_f32(0.0) == 0.0


def _round_f32_from_bits(x):
    """The same rule re-derived on the float64 bit pattern with integer arithmetic:
    keep the top 24 significant bits (fewer below 2^-126), ties to even."""
    out = np.empty_like(x)
    for i, v in enumerate(x):
        m, e = np.frexp(abs(v))              # |v| = m 2^e, m in [0.5, 1)
        m, e = float(m), int(e)
        keep = 24 if e - 1 >= -126 else 24 - (-126 - (e - 1))  # significant bits float32 holds here
        scaled = int(np.ldexp(m, 53))        # the 53-bit significand as an integer
        if keep < 1:                          # below half the smallest subnormal
            out[i] = np.copysign(0.0, v) if keep < 0 or scaled <= 1 << 52 else np.copysign(2.0 ** -149, v)
            continue
        drop = 53 - keep
        q, r = divmod(scaled, 1 << drop)
        half = 1 << (drop - 1)
        if r > half or (r == half and (q & 1)):
            q += 1
        out[i] = np.copysign(np.ldexp(float(q), e - 53 + drop), v)
    return out


@pytest.mark.parametrize("seed", [0, 1])
def test_against_integer_rederivation(seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(4000) * np.exp2(rng.integers(-140, 120, size=4000))
    # include exact ties at random exponents: a float32 value plus half a float32 step
    base = rng.standard_normal(500).astype(np.float32).astype(np.float64)
    _, e = np.frexp(base)
    ties = base + np.copysign(np.ldexp(1.0, e - 25), base)
    x = np.concatenate([x, ties])
    assert np.array_equal(oracle.round_f32(x), _round_f32_from_bits(x))


def test_against_torch_conversion():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(7)
    x = rng.standard_normal(20000) * np.exp2(rng.integers(-150, 127, size=20000))
    ref = torch.from_numpy(x).to(torch.float32).to(torch.float64).numpy()
    assert np.array_equal(oracle.round_f32(x), ref)
