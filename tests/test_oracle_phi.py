"""Pins for the oracle's offset maps (oracle/phi.py).

The log-bucket map (DeBERTa reading) is pinned by hand-derived rows
(tests/golden/log_bucket_points.txt), by a second exact evaluation through
60-digit decimal thresholds, and by structure (exact region equal to the
truncated DeBERTa map, sign symmetry, monotonicity, every row reached).

The T5 map is pinned three ways that do not share the oracle's float-log code:
the integer closed form f(n) = min(15, 1 + bitlen(n^2)) for n >= 8 (exact, from
8 + floor(2 log2(n/8)) = 2 + floor(log2 n^2)), the hand-derived bucket starts
in tests/golden/t5_bucket_starts.txt, and structural properties (exact region,
sign split, monotonicity, range).
"""

import os

import numpy as np
import pytest

from oracle import log_bucket, phi_rows, num_rows, t5_bucket

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _closed_form_lower(n):
    n = np.asarray(n, dtype=object)
    out = []
    for x in n.tolist():
        x = int(x)
        out.append(x if x < 8 else min(15, 1 + (x * x).bit_length()))
    return np.array(out, dtype=np.int64)


def test_t5_closed_form_exhaustive():
    n = np.arange(0, 20000, dtype=np.int64)
    want = _closed_form_lower(n)
    assert np.array_equal(t5_bucket(-n, 32, 128, True, 8), want)
    pos = n[1:]
    assert np.array_equal(t5_bucket(pos, 32, 128, True, 8), 16 + want[1:])


def test_t5_golden_bucket_starts():
    rows = [l.split() for l in open(os.path.join(GOLD, "t5_bucket_starts.txt"))
            if l.strip() and not l.startswith("#")]
    for n, lo, hi in ((int(a), int(b), int(c)) for a, b, c in rows):
        assert int(t5_bucket(-n, 32, 128, True, 8)) == lo, n
        if n > 0:
            assert int(t5_bucket(n, 32, 128, True, 8)) == hi, n


def test_t5_default_max_exact_is_half_of_half():
    o = np.arange(-300, 301)
    assert np.array_equal(t5_bucket(o, 32, 128, True, None), t5_bucket(o, 32, 128, True, 8))


def test_t5_structure():
    o = np.arange(-5000, 5001)
    bk = t5_bucket(o, 32, 128, True, 8)
    assert bk.min() == 0 and bk.max() == 31
    # exact region |o| < 8
    for x in range(0, 8):
        assert t5_bucket(-x, 32, 128, True, 8) == x
    for x in range(1, 8):
        assert t5_bucket(x, 32, 128, True, 8) == 16 + x
    # monotone in |o| within each half, saturation from 91 on
    neg = t5_bucket(-np.arange(0, 5000), 32, 128, True, 8)
    assert np.all(np.diff(neg) >= 0)
    assert np.all(neg[91:] == 15) and neg[90] == 14


def test_t5_unidirectional():
    o = np.arange(-400, 401)
    bk = t5_bucket(o, 32, 128, False, None)
    assert np.all(bk[o >= 0] == 0)
    n = -o[o < 0]
    # 32 buckets, max_exact 16: exact below 16, clamp at 31
    assert np.array_equal(bk[o < 0][n < 16], n[n < 16])
    assert bk.max() == 31


def test_truncated_and_identity_rows():
    N = 50
    r = phi_rows({"kind": "truncated", "lo": -3, "hi": 5}, N)
    o = np.arange(-(N - 1), N)
    assert num_rows({"kind": "truncated", "lo": -3, "hi": 5}, N) == 9
    assert np.all(r[o <= -3] == 0) and np.all(r[o >= 5] == 8)
    inner = (o > -3) & (o < 5)
    assert np.array_equal(r[inner], o[inner] + 3)
    ri = phi_rows({"kind": "identity"}, N)
    assert num_rows({"kind": "identity"}, N) == 2 * N - 1
    assert np.array_equal(ri, np.arange(2 * N - 1))
    # a truncation wider than every reachable offset is the identity map shifted
    rw = phi_rows({"kind": "truncated", "lo": -(N - 1), "hi": N - 1}, N)
    assert np.array_equal(rw, ri)


def test_z_bytes_closed_forms():
    # Relation projection bytes for the 8K Shaw shape: B*H*N*R*4 = 101,056,512 B;
    # grouped window overhead (G-1)/N = 127/8192 ~ 1.6 % (grouped-range section).
    assert 1 * 12 * 8192 * num_rows({"kind": "truncated", "lo": -128, "hi": 128}, 8192) * 4 == 101056512
    assert abs(127 / 8192 - 0.0155) < 1e-4
    # explicit fp32 score matrix n^2 * 4 B (attention primer): 1/4/16/64 MiB
    for n, mib in ((512, 1), (1024, 4), (2048, 16), (4096, 64)):
        assert n * n * 4 == mib * 2 ** 20


@pytest.mark.parametrize("N", [1, 2, 7])
def test_small_n_rows(N):
    for phi in ({"kind": "truncated", "lo": -2, "hi": 2}, {"kind": "identity"},
                {"kind": "t5", "num_buckets": 32, "max_distance": 128, "bidirectional": True}):
        r = phi_rows(phi, N)
        assert r.shape == (2 * N - 1,)
        assert r.min() >= 0 and r.max() < num_rows(phi, N)


def test_log_bucket_golden_points():
    rows = [l.split() for l in open(os.path.join(GOLD, "log_bucket_points.txt"))
            if l.strip() and not l.startswith("#")]
    for o, r in ((int(a), int(b)) for a, b in rows):
        assert int(log_bucket(o, 256, 512)) == r, o


def _decimal_buckets(n_max, k, m):
    """Buckets (before the row clamp) of offsets 0..n_max by thresholds: for
    n > mid the step t is the least t with mid * ((m-1)/mid)^(t/(mid-1)) >= n,
    the thresholds taken at 60 significant digits (an evaluation independent
    of the oracle's)."""
    from decimal import Decimal, getcontext
    getcontext().prec = 60
    mid = k // 2
    c = (Decimal(m - 1) / Decimal(mid)).ln()
    thr = []
    t = 0
    while True:
        u = Decimal(mid) * (c * Decimal(t) / Decimal(mid - 1)).exp()
        thr.append(u)
        if u >= n_max or t > 4 * k:
            break
        t += 1
    out = []
    j = 0
    for n in range(n_max + 1):
        if n <= mid:
            out.append(n)
            continue
        while thr[j] < n:
            j += 1
        out.append(mid + j)
    return np.array(out, dtype=np.int64)


@pytest.mark.parametrize("k,m", [(256, 512), (64, 300), (32, 40)])
def test_log_bucket_matches_decimal_thresholds(k, m):
    n = np.arange(0, 6000)
    bucket = _decimal_buckets(5999, k, m)
    assert np.array_equal(log_bucket(n, k, m), np.minimum(bucket + k, 2 * k - 1))
    # negative offsets take the negated bucket
    assert np.array_equal(log_bucket(-n, k, m), np.maximum(k - bucket, 0))


def test_log_bucket_structure():
    k, m = 256, 512
    o = np.arange(-20000, 20001)
    r = log_bucket(o, k, m)
    assert r.min() == 0 and r.max() == 2 * k - 1
    assert np.all(np.diff(r) >= 0)
    assert set(r.tolist()) == set(range(2 * k))
    near = np.abs(o) <= k // 2
    # inside the exact range the map equals the truncated DeBERTa map
    assert np.array_equal(r[near], np.clip(o[near], -256, 255) + 256)
    inner = np.abs(o) <= m - 1
    assert np.array_equal(r[inner][::-1], 2 * k - r[inner])
    assert num_rows({"kind": "log", "num_buckets": k, "max_distance": m}, 8192) == 2 * k


def test_log_bucket_float64_has_no_near_ties():
    """The direct float64 evaluation of the ceiling equals the exact one for
    every offset below 20000 at these parameters, so a float64 evaluation
    (the HIP path's) can be bit-exact."""
    import math
    for k, m in ((256, 512), (64, 300), (32, 40)):
        mid = k // 2
        n = np.arange(mid + 1, 20000)
        f = np.array([mid + math.ceil(math.log(x / mid) / math.log((m - 1) / mid) * (mid - 1))
                      for x in n.tolist()])
        want = np.minimum(f + k, 2 * k - 1)
        assert np.array_equal(log_bucket(n, k, m), want), (k, m)
