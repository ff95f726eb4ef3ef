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

A phi descriptor is a dict:
  {"kind": "truncated", "lo": int, "hi": int}
  {"kind": "identity"}
  {"kind": "t5", "num_buckets": int, "max_distance": int,
   "bidirectional": bool, "max_exact": int or None}
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


def num_rows(phi, N):
    """Number of relation-table rows R that the map indexes."""
    kind = phi["kind"]
    if kind == "truncated":
        return int(phi["hi"]) - int(phi["lo"]) + 1
    if kind == "identity":
        return 2 * int(N) - 1
    if kind == "t5":
        return int(phi["num_buckets"])
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
    raise ValueError(f"unknown phi kind {kind!r}")


def phi_rows(phi, N):
    """Row index of every offset o = -(N-1) .. N-1, as int64[2N-1] (entry o + N - 1)."""
    o = np.arange(-(int(N) - 1), int(N), dtype=np.int64)
    return phi_of_offset(phi, o, N)
