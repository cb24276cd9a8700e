"""The quantizer takes |v| / scale as RN32(RN64(|v| * RN64(1 / scale))) instead
of an fp32 division, for ratios of at least 2^-100 (smaller ones take the
division). This checks on the CPU that the route gives the correctly rounded
fp32 quotient: on random pairs, on pairs built to sit close to rounding
boundaries, and across the whole exponent range."""
import numpy as np

TINY = np.float32(2.0 ** -100)


def route(a, b):
    rs = 1.0 / b.astype(np.float64)
    return (a.astype(np.float64) * rs).astype(np.float32)


def check(a, b):
    a = np.abs(a.astype(np.float32))
    b = np.abs(b.astype(np.float32))
    a, b = np.minimum(a, b), np.maximum(a, b)  # a bucket's scale is its largest magnitude
    keep = b > 0
    a, b = a[keep], b[keep]
    with np.errstate(all="ignore"):
        want = a / b  # IEEE fp32 division, correctly rounded
        got = route(a, b)
    sel = got >= TINY
    bad = np.nonzero(got[sel].view(np.uint32) != want[sel].view(np.uint32))[0]
    assert bad.size == 0, (a[sel][bad[:5]], b[sel][bad[:5]], got[sel][bad[:5]], want[sel][bad[:5]])
    return int(sel.sum())


def test_random_pairs():
    rng = np.random.default_rng(1)
    n = 0
    for _ in range(8):
        n += check(rng.standard_normal(1 << 20), rng.standard_normal(1 << 20))
        n += check(rng.random(1 << 20), rng.random(1 << 20))
    assert n > 10_000_000


def test_random_bit_patterns_over_all_exponents():
    rng = np.random.default_rng(2)
    for _ in range(8):
        a = rng.integers(0, 0x7F800000, 1 << 20, dtype=np.uint32).view(np.float32)
        b = rng.integers(0, 0x7F800000, 1 << 20, dtype=np.uint32).view(np.float32)
        check(a, b)


def test_near_rounding_boundaries():
    """a = RN(b * q) for random q: quotients land within an ulp of q, and with
    b's significand all ones or a random odd number the exact quotient falls
    as close to a midpoint as 24-bit operands allow."""
    rng = np.random.default_rng(3)
    for sig in (0xFFFFFF, None):
        m = np.full(1 << 20, sig, np.uint32) if sig else (rng.integers(1 << 22, 1 << 23, 1 << 20,
                                                                        dtype=np.uint32) * 2 + 1)
        e = rng.integers(-60, 60, 1 << 20)
        b = np.ldexp(m.astype(np.float64), e - 23).astype(np.float32)
        q = rng.random(1 << 20).astype(np.float32)
        for d in (-2, -1, 0, 1, 2):  # neighbours of RN(b * q)
            a = (b.astype(np.float64) * q.astype(np.float64)).astype(np.float32)
            a = np.nextafter(a, np.float32(np.inf) if d > 0 else np.float32(0), dtype=np.float32) if d else a
            if abs(d) == 2:
                a = np.nextafter(a, np.float32(np.inf) if d > 0 else np.float32(0), dtype=np.float32)
            check(a, b)


def test_level_boundaries_of_the_quantizer():
    """Values at, just below and just above l / s * scale for every level l
    of s = 1, 7, 127 and many scales."""
    rng = np.random.default_rng(4)
    scales = np.abs(rng.standard_normal(4096)).astype(np.float32) * np.float32(1e-3)
    for s in (1, 7, 127):
        for lvl in range(s + 1):
            a = (scales.astype(np.float64) * lvl / s).astype(np.float32)
            for a2 in (a, np.nextafter(a, np.float32(0)), np.nextafter(a, np.float32(np.inf))):
                check(a2, scales)
