"""Host model of the quantiser's reciprocal fast path (no GPU).

The HIP quantiser decides each NF4 index from v' = w * r, r a reciprocal of
the block maximum a within 2 ulp of 1/a, instead of the correctly rounded
v = w / a that defines the index; a lane whose v' lies within a relative
2^-20 of the threshold of its bucket (the 64 buckets of width 1/32 over
[-1, 1]) redoes its elements with the division.  This test models that
decision in numpy (fp32 arithmetic emulated exactly) and checks the claim
it rests on: every (w, a) whose two indices differ is flagged.  The
reference index here is the nearest-codepoint rule written out directly
(count of midpoints strictly below v, midpoints rounded down to fp32).
"""
import numpy as np
import pytest

CB = np.array([-1.0, -0.696, -0.525, -0.395, -0.284, -0.185, -0.091, 0.0, 0.080, 0.161, 0.246,
               0.338, 0.441, 0.563, 0.723, 1.0], dtype=np.float32)


def _thresholds():
    t = []
    for i in range(15):
        mid = (float(CB[i]) + float(CB[i + 1])) / 2
        v = np.float32(mid)
        if float(v) > mid:
            v = np.nextafter(v, np.float32(-np.inf))
        t.append(v)
    return np.array(t, dtype=np.float32)


T = _thresholds()


def _buckets():
    c = np.zeros(65, np.int64)
    tin = np.full(65, np.inf, np.float32)
    for k in range(65):
        lo = np.float32(-1.0 + k * 0.03125)
        hi = np.float32(lo + np.float32(0.03125))
        c[k] = np.sum(T < lo)
        inside = T[(T >= lo) & (T < hi)]
        assert inside.size <= 1
        if inside.size:
            tin[k] = inside[0]
            assert min(inside[0] - lo, hi - inside[0]) >= 1.9e-3  # thresholds clear of bucket edges
    g = np.where(np.isfinite(tin), np.abs(tin) * np.float32(2.0 ** -20), 0).astype(np.float32)
    return c, tin, g


C, TIN, G = _buckets()


def _unflagged_mismatches(w, a, ulps):
    """Pairs the fast path would decide wrongly without a flag.  Block
    maxima outside [2^-125, 2^125] always take the division and are left
    out."""
    w = w.astype(np.float32)
    a = a.astype(np.float32)
    fast_ok = (a >= np.float32(2.0 ** -125)) & (a <= np.float32(2.0 ** 125))
    w, a = w[fast_ok], a[fast_ok]
    v = (w / a).astype(np.float32)                       # correctly rounded quotient
    r = (np.float32(1) / a).astype(np.float32)
    for _ in range(abs(ulps)):
        r = np.nextafter(r, np.float32(np.inf) if ulps > 0 else np.float32(0)).astype(np.float32)
    vp = (w * r).astype(np.float32)
    # bucket key trunc(fma(v', 32, 32)): the fma is exact in fp64, then rounded once
    key = np.trunc((vp.astype(np.float64) * 32 + 32).astype(np.float32)).astype(np.int64)
    assert key.min() >= 0 and key.max() <= 64           # no clamp needed when |w| <= a
    near = np.abs((vp - TIN[key]).astype(np.float32)) < G[key]
    fast = C[key] + (vp > TIN[key])
    exact = np.sum(v[:, None] > T[None, :], axis=1)
    return int(((fast != exact) & ~near).sum()), int(near.sum())


@pytest.mark.parametrize("ulps", [-2, 0, 2])
def test_guard_covers_every_bf16_ratio_class(ulps):
    bits = np.arange(0, 0x7F80, dtype=np.uint32)
    vals = (bits << 16).view(np.float32)
    bad = 0
    for e in (0, -120, 120):
        for m in range(0, 128, 16):
            a = np.float32((1 + m / 128) * 2.0 ** e)
            ws = vals[vals <= a]
            ws = np.concatenate([ws, -ws])
            bad += _unflagged_mismatches(ws, np.full(ws.size, a), ulps)[0]
    assert bad == 0


@pytest.mark.parametrize("ulps", [-2, 0, 2])
def test_guard_covers_fp32_pairs_and_planted_thresholds(ulps):
    rng = np.random.default_rng(ulps + 10)
    n = 400_000
    a = (np.abs(rng.standard_normal(n)) + 1e-3).astype(np.float32)
    a *= np.float32(2.0) ** rng.integers(-118, 118, n).astype(np.float32)
    w = (rng.uniform(-1, 1, n).astype(np.float32) * a).astype(np.float32)
    k = rng.integers(0, 15, n // 4)
    w[: n // 4] = (T[k] * a[: n // 4]).astype(np.float32)           # on a threshold times a
    w[n // 4: n // 2] = np.nextafter(w[: n // 4], np.float32(np.inf))
    a = np.maximum(a, np.abs(w))
    bad, flagged = _unflagged_mismatches(w, a, ulps)
    assert bad == 0
    assert flagged < n // 2 + n // 100  # only the planted neighbourhoods, not everything
