"""Offset maps phi(i, j) -> relation row, written from their definitions.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The score of Eq. (1) on the nanless.github.io digest of "Fast and Exact
Relative-Position Attention via Structure-Aware Kernels" indexes its relation
tables by a row r = phi(i, j) that depends only on the offset o = j - i (the
page's sections on the grouped reachable range and on constant tiles speak of
"offsets"; reading adopted: o = j - i, key index minus query index).  The
setup section lists the maps per mechanism:

* truncated (Shaw; DeBERTa as configured here): r = clip(o, lo, hi) - lo,
  R = hi - lo + 1 rows.  Beyond the thresholds it saturates to the first or
  last row (section on constant tiles and the saturated region).
* identity (Transformer-XL): r = o + N - 1, R = 2N - 1 rows.
* T5 buckets: 32 bidirectional buckets up to distance 128.  The page does not
  print the bucket function; the reading adopted is the standard T5 relative
  position bucket (Raffel et al., 2020), evaluated in float64:
  half the buckets per sign when bidirectional (keys after the query take the
  upper half), exact buckets for n < max_exact, logarithmic buckets from
  max_exact up to max_distance, clamped to the last bucket.

* log buckets (DeBERTa): the setup section names "256 log buckets to 512
  distance" for DeBERTa without printing the function; the reading adopted
  is DeBERTa's published log-bucket position scheme (He et al., 2021), with
  num_buckets = k, max_distance = m, mid = k / 2 and o = j - i: offsets with
  |o| <= mid keep their own bucket o; beyond, the bucket is
  sign(o) * (mid + ceil((mid - 1) * ln(|o| / mid) / ln((m - 1) / mid)));
  the row is the bucket plus k, clamped to [0, 2k - 1] (R = 2k rows).  The
  ceiling is taken exactly (integer arithmetic, no rounding of logarithms).

A phi descriptor is a dict:
  {"kind": "truncated", "lo": int, "hi": int}
  {"kind": "identity"}
  {"kind": "t5", "num_buckets": int, "max_distance": int,
   "bidirectional": bool, "max_exact": int or None}
  {"kind": "log", "num_buckets": int, "max_distance": int}
"""

import math

import numpy as np


def t5_bucket(o, num_buckets=32, max_distance=128, bidirectional=True, max_exact=None):
    """T5 relative-position bucket of offset(s) ``o`` (= key - query).

    Float64 evaluation of the standard definition:
      bidirectional: nb = num_buckets // 2, base = nb if o > 0 else 0, n = |o|
      otherwise:     nb = num_buckets,      base = 0,                n = max(-o, 0)
      me = max_exact (default nb // 2)
      bucket = base + n                                         if n < me
             = base + min(nb - 1, me + int(ln(n/me)/ln(max_distance/me) * (nb - me)))  otherwise
    """
    o = np.asarray(o, dtype=np.int64)
    if bidirectional:
        nb = num_buckets // 2
        base = np.where(o > 0, nb, 0).astype(np.int64)
        n = np.abs(o)
    else:
        nb = num_buckets
        base = np.zeros_like(o)
        n = np.maximum(-o, 0)
    me = nb // 2 if max_exact is None else int(max_exact)
    out = np.empty_like(o)
    small = n < me
    out[small] = n[small]
    big = ~small
    if np.any(big):
        nf = n[big].astype(np.float64)
        val = np.log(nf / me) / math.log(max_distance / me) * (nb - me)
        out[big] = np.minimum(nb - 1, me + val.astype(np.int64))
    return base + out


def _log_step(n, mid, m):
    """ceil((mid - 1) * ln(n / mid) / ln((m - 1) / mid)) for integers n > mid,
    m - 1 > mid, exactly.

    With c = (m - 1) / mid > 1, the value is the least integer t with
    t >= (mid - 1) * ln(n / mid) / ln(c), i.e. with c**t >= (n / mid)**(mid - 1),
    i.e. (m - 1)**t * mid**(mid - 1) >= n**(mid - 1) * mid**t (positive
    integers, compared exactly).  A float64 estimate gives the start; the
    exact test moves it to the least such t.
    """
    def ok(t):
        return (m - 1) ** t * mid ** (mid - 1) >= n ** (mid - 1) * mid ** t
    t = max(0, math.ceil((mid - 1) * math.log(n / mid) / math.log((m - 1) / mid)))
    while t > 0 and ok(t - 1):
        t -= 1
    while not ok(t):
        t += 1
    return t


def log_bucket(o, num_buckets=256, max_distance=512):
    """Row (in [0, 2 * num_buckets)) of the log-bucket map for offset(s) o = key - query:
      n = |o|, mid = num_buckets // 2
      bucket = o                                         if n <= mid
             = sign(o) * (mid + _log_step(n, mid, m))      otherwise
      row = clip(bucket + num_buckets, 0, 2 * num_buckets - 1)
    """
    o = np.asarray(o, dtype=np.int64)
    k, m = int(num_buckets), int(max_distance)
    mid = k // 2
    steps = {}
    out = np.empty(o.shape, dtype=np.int64)
    flat = o.reshape(-1)
    res = out.reshape(-1)
    for idx in range(flat.size):
        oo = int(flat[idx])
        n = abs(oo)
        if n <= mid:
            b = oo
        else:
            if n not in steps:
                steps[n] = _log_step(n, mid, m)
            b = (mid + steps[n]) * (1 if oo > 0 else -1)
        res[idx] = min(max(b + k, 0), 2 * k - 1)
    return out


def num_rows(phi, N):
    """Number of relation-table rows R that the map indexes."""
    kind = phi["kind"]
    if kind == "truncated":
        return int(phi["hi"]) - int(phi["lo"]) + 1
    if kind == "identity":
        return 2 * int(N) - 1
    if kind == "t5":
        return int(phi["num_buckets"])
    if kind == "log":
        return 2 * int(phi["num_buckets"])
    raise ValueError(f"unknown phi kind {kind!r}")


def phi_of_offset(phi, o, N):
    """Row index for offset array ``o`` (= j - i)."""
    o = np.asarray(o, dtype=np.int64)
    kind = phi["kind"]
    if kind == "truncated":
        lo, hi = int(phi["lo"]), int(phi["hi"])
        return np.clip(o, lo, hi) - lo
    if kind == "identity":
        return o + (int(N) - 1)
    if kind == "t5":
        return t5_bucket(o, phi["num_buckets"], phi["max_distance"],
                         phi.get("bidirectional", True), phi.get("max_exact"))
    if kind == "log":
        return log_bucket(o, phi["num_buckets"], phi["max_distance"])
    raise ValueError(f"unknown phi kind {kind!r}")


def phi_rows(phi, N):
    """Row index of every offset o = -(N-1) .. N-1, as int64[2N-1] (entry o + N - 1)."""
    o = np.arange(-(int(N) - 1), int(N), dtype=np.int64)
    return phi_of_offset(phi, o, N)
