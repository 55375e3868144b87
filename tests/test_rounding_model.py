"""Host model of the rotation's fp64 -> fp16 rounding (no GPU).

The device helper (f64_to_f32_odd, then one RNE conversion to fp16) rounds
to odd into fp32 by clearing the 29 mantissa bits an fp32 drops and setting
the lowest kept bit when any of them was set; this file restates those
integer steps with numpy and checks them against numpy's direct,
correctly rounded float64 -> float16 conversion on values chosen to break a
wrong rounding: every fp16 midpoint and its fp64 neighbours, offsets around
them, the subnormal and overflow boundaries, zeros, infinities and random
values over many decades.
"""
import numpy as np


def _odd_f32(d):
    u = d.view(np.uint64)
    lo = (u & np.uint64(0xFFFFFFFF)).astype(np.uint32)
    hi = u & np.uint64(0xFFFFFFFF00000000)
    sticky = ((lo & np.uint32(0x1FFFFFFF)) + np.uint32(0x1FFFFFFF)) & np.uint32(0x20000000)
    lo2 = (lo & np.uint32(0xE0000000)) | sticky
    return (hi | lo2.astype(np.uint64)).view(np.float64).astype(np.float32)


def _model(d):
    with np.errstate(over="ignore", invalid="ignore"):
        return _odd_f32(d).astype(np.float16)


def _values():
    h = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = (h[:-1] + h[1:]) / 2  # exact in fp64
    mids = np.concatenate([mids, [65504.0 + 8.0]])  # the overflow midpoint
    offs = np.array([1, 2, 3, 1 << 10, 1 << 20, 1 << 28, 1 << 29, (1 << 29) + 1, 1 << 30],
                    dtype=np.int64)
    base = mids.view(np.int64)
    near = [mids]
    for o in offs:
        near += [(base + o).view(np.float64), (base - o).view(np.float64)]
    rng = np.random.default_rng(5)
    rand = rng.standard_normal(400_000) * 10.0 ** rng.uniform(-9, 6, 400_000)
    special = np.array([0.0, 2.0 ** -24, 2.0 ** -25, 2.0 ** -25 * (1 + 2.0 ** -52),
                        2.0 ** -14, 65504.0, 65519.999, 65520.0, 1e300, np.inf,
                        1e-40, 1e-310])
    v = np.concatenate(near + [rand, special])
    return np.concatenate([v, -v])


def test_round_to_odd_then_nearest_is_correctly_rounded():
    d = _values()
    assert d.size > 2_000_000
    with np.errstate(over="ignore"):
        want = d.astype(np.float16)
    got = _model(d)
    assert np.array_equal(got.view(np.uint16), want.view(np.uint16))


def test_plain_double_rounding_would_fail_here():
    """The values above do catch a double rounding through fp32 without the
    sticky bit (so the check has teeth)."""
    d = _values()
    with np.errstate(over="ignore"):
        naive = d.astype(np.float32).astype(np.float16)
        want = d.astype(np.float16)
    assert not np.array_equal(naive.view(np.uint16), want.view(np.uint16))


def test_nan_stays_nan():
    d = np.array([np.nan, -np.nan, np.uint64(0x7FF0000000000001).view(np.float64)])
    assert np.all(np.isnan(_model(d)))
