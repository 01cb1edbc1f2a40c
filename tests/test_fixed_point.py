"""Host-side check of the fixed-point term the lookup-table GEMVs add across workgroups.

Each workgroup adds its row sum v (fp32) to a 64-bit word as round-half-even(v * 2^24), saturated at
+-(2^47 - 1), plus a bias of 2^47.  The kernels compute that integer in fp32 and 32-bit integers only:
    a = |v| * 2^24                       (exact: a power-of-two scale)
    h = floor(a * 2^-32)                 (exact)
    r = fma(h, -2^32, a)                 (claimed exact: a multiple of ulp(a) below 2^32)
    n = h * 2^32 + rint(r)               (rint: round half to even)
    term = 2^47 - n if v < 0 else 2^47 + n
This test replays those steps in float32 with numpy, emulating the single-rounding fma by computing
the exact value in float64 and rounding it once to float32, and compares the result with an exact
integer reference over edge cases and random values.
"""
import numpy as np

BIAS = 1 << 47
SCALE = np.float32(2.0 ** 24)


def reference(v: np.ndarray) -> np.ndarray:
    """round-half-even(v * 2^24) clamped to +-(2^47 - 1), plus 2^47, as Python integers."""
    out = []
    for x in v.astype(np.float64):
        d = x * 2.0 ** 24                                # exact in float64
        n = int(np.rint(d))                              # round half to even, exact for |d| < 2^53
        n = max(-(BIAS - 1), min(BIAS - 1, n))
        out.append(BIAS + n)
    return np.array(out, dtype=object)


def kernel_steps(v: np.ndarray) -> np.ndarray:
    v = v.astype(np.float32)
    a = (np.abs(v) * SCALE).astype(np.float32)
    out = []
    for vi, ai in zip(v, a):
        n = BIAS - 1                                      # saturated magnitude
        if ai < np.float32(BIAS):
            h = np.floor(np.float32(ai * np.float32(2.0 ** -32)))
            exact = float(h) * -(2.0 ** 32) + float(ai)   # the fma before its one rounding
            r = np.float32(exact)
            assert float(r) == exact, (vi, ai, exact)     # the claim: no rounding happens here
            n = int(h) * (1 << 32) + int(np.rint(r))
        out.append(BIAS - n if vi < 0 else BIAS + n)
    return np.array(out, dtype=object)


def _cases() -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(2024))
    edge = [0.0, -0.0, 1.0, -1.0, 2.0 ** -24, -(2.0 ** -24), 1.5 * 2.0 ** -24, 2.5 * 2.0 ** -24,
            -2.5 * 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -149, -(2.0 ** -149),
            2.0 ** 8 - 2.0 ** -16, 2.0 ** 8, 2.0 ** 22, 2.0 ** 23 - 0.5, -(2.0 ** 23 - 0.5), 2.0 ** 23,
            -(2.0 ** 23), 2.0 ** 30, -(2.0 ** 40)]
    ties = (g.integers(-2 ** 20, 2 ** 20, 2000) + 0.5) * 2.0 ** -24      # exact halves of the last unit
    spread = [g.standard_normal(2000) * 10.0 ** e for e in range(-8, 8)]
    return np.concatenate([np.array(edge), ties, *spread]).astype(np.float32)


def test_fixed_point_term_matches_exact_rounding():
    v = _cases()
    assert list(kernel_steps(v)) == list(reference(v))


def test_fixed_point_sums_are_order_independent_and_exact():
    # the words add as integers: any order gives the same total, equal to the sum of the rounded terms
    g = np.random.Generator(np.random.PCG64(7))
    v = (g.standard_normal(255) * 3.0).astype(np.float32)
    terms = kernel_steps(v)
    total = sum(terms) - len(v) * BIAS
    assert total == sum(int(np.rint(float(x) * 2.0 ** 24)) for x in v)
    perm = g.permutation(len(v))
    assert sum(terms[perm]) == sum(terms)
    # 255 terms below 2^48 each leave the 56-bit field without a carry into the count byte
    assert max(terms) < 1 << 48 and sum(terms) < 1 << 56
