"""Shared helpers of the parity tests: run the HIP path and the oracle on the
same seeded inputs and compare them (test infrastructure only)."""

import json
import os

import numpy as np
import torch

import oracle
from relpos_synth import as_f64, make_inputs  # noqa: F401

# Tolerances, max |x - ref| / max |ref| per tensor.
#  fp16: 2e-3 on O and 1e-2 on every gradient (fp16 inputs, fp32 accumulation).
#  bf16: O to 2 * 2^-8 (two bf16 unit roundoffs: O is stored in bf16, up to
#        2^-9 |O|, and P is rounded to bf16 before P V, up to 2^-9 per term);
#        gradients keep 1e-2.
#  fp32: 1e-4 on everything (no 16-bit rounding anywhere on the path).
# LSE is fp32 in every case: absolute 2e-3.
# A reference that is identically zero in exact arithmetic (max |ref| below
# 1e-12, e.g. table gradients when every offset maps to one row) is checked
# absolutely: max |x| <= ZERO_ABS.
TOL = {"f16": (2e-3, 1e-2), "bf16": (2.0 ** -7, 1e-2), "f32": (1e-4, 1e-4)}
TOL_O, TOL_G = TOL["f16"]
TOL_LSE_ABS = 2e-3
ZERO_ABS = 1e-4
ALL_OUTPUTS = ("O", "lse", "dq", "dk", "dv", "daq", "dak", "db")


def require_gpu():
    assert torch.cuda.is_available(), "GPU test run without a visible GPU"
    import exact_relative_position_amd._binding as b
    b.lib()  # raises if the HIP library is missing
    return torch.device("cuda:0")


def gpu_dropout(w):
    """The library's (p, seed, offset) for a workload's (t, seed, offset)."""
    return None if w.dropout is None else (w.dropout[0] / 256.0, w.dropout[1], w.dropout[2])


def gpu_run(w, x, dev, keep_z=True, backward=True):
    import exact_relative_position_amd as rp
    t = {k: (None if v is None else v.to(dev)) for k, v in x.items()}
    drop = gpu_dropout(w)
    O, lse, zs = rp.forward(t["q"], t["k"], t["v"], t["aq"], t["ak"], t["b"], phi=w.phi,
                            tau=w.tau, causal=w.causal, key_len=t["key_len"], keep_z=keep_z,
                            dropout=drop, zchunk=w.zchunk, relation=w.relation)
    out = {"O": O, "lse": lse}
    if backward:
        dq, dk, dv, daq, dak, db = rp.backward(t["q"], t["k"], t["v"], t["aq"], t["ak"], t["b"],
                                               O, lse, t["do"], zs, phi=w.phi, tau=w.tau,
                                               causal=w.causal, key_len=t["key_len"],
                                               dropout=drop, zchunk=w.zchunk,
                                               relation=w.relation)
        out.update(dq=dq, dk=dk, dv=dv, daq=daq, dak=dak, db=db)
    torch.cuda.synchronize(dev)
    return {k: (None if v is None else v.detach().cpu().double().numpy()) for k, v in out.items()}


def oracle_run(w, x, bh=None, query_rows=None, backward=True):
    f = {k: as_f64(v) for k, v in x.items() if k != "key_len"}
    kl = None if x["key_len"] is None else x["key_len"].numpy()
    O, L = oracle.forward(f["q"], f["k"], f["v"], f["aq"], f["ak"], f["b"], phi=w.phi, tau=w.tau,
                          causal=w.causal, key_len=kl, bh=bh, query_rows=query_rows,
                          dropout=w.dropout)
    out = {"O": O, "lse": L}
    if backward:
        g = oracle.backward(f["q"], f["k"], f["v"], f["aq"], f["ak"], f["b"], dO=f["do"],
                            phi=w.phi, tau=w.tau, causal=w.causal, key_len=kl, bh=bh,
                            query_rows=query_rows, dropout=w.dropout)
        out.update(g)
    return out


def rel_err(x, ref):
    """max |x - ref| / max |ref|; absolute max |x| when ref is identically zero."""
    x, ref = np.asarray(x), np.asarray(ref)
    fin = np.isfinite(ref)
    assert np.array_equal(fin, np.isfinite(x)), "non-finite entries differ"
    if not fin.any():
        return 0.0
    assert np.array_equal(x[~fin], ref[~fin])
    scale = np.abs(ref[fin]).max()
    diff = np.abs(x[fin] - ref[fin]).max()
    if scale < 1e-12:
        return float(np.abs(x[fin]).max())
    return float(diff / scale)


def tolerances(dtype):
    return TOL[dtype]


# Elementwise check of 16-bit outputs.  O is stored in the input type, and the
# weights P are rounded to it before P V, with the normaliser summing the
# rounded weights; the rounding of P perturbs every output of a row by at
# most 2^-(p+1) (p = 8 bf16 / 11 fp16 significant bits) times the spread of
# V around O under P, which is bounded by the row's scale, and storing O adds
# half an ulp of the element.  A float64 model of exactly this arithmetic
# (P rounded, fp32 sums) stays within 1.15 ulps of the row's largest
# |O| on the bf16 and fp16 workloads, so every element is required to lie
# within ULP_ROW = 2 units in the last place of the 16-bit type, taken at
# the largest |O| of its row.
ULP_ROW = 2.0
_MANT = {"f16": 10, "bf16": 7}
_MIN_EXP = {"f16": -14, "bf16": -126}


def ulp16(a, dtype):
    """Spacing of the 16-bit type at |a| (subnormal spacing below the normals)."""
    a = np.abs(np.asarray(a, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** _MIN_EXP[dtype])))
    return 2.0 ** (e - _MANT[dtype])


def check_rows_ulp(got, ref, dtype, label="", k=ULP_ROW):
    """Every element of a 16-bit O within k ulps of its row's largest |ref|;
    returns the largest error in those units and the fraction of elements
    equal to the oracle value rounded to the 16-bit type."""
    if dtype not in _MANT:
        return None
    got, ref = np.asarray(got), np.asarray(ref)
    scale = ulp16(np.abs(ref).max(axis=-1, keepdims=True), dtype)
    units = np.abs(got - ref) / scale
    worst = float(units.max()) if units.size else 0.0
    assert worst <= k, f"{label} O: {worst:.2f} ulps of the row scale > {k}"
    t = torch.float16 if dtype == "f16" else torch.bfloat16
    r16 = torch.from_numpy(np.ascontiguousarray(ref)).to(t).double().numpy()
    exact = float((got == r16).mean()) if got.size else 1.0
    return {"ulps_row_max": worst, "frac_equal_rounded": exact}


def elementwise_stats(x, ref):
    """Distribution of the elementwise error of a tensor against its
    reference, relative to the reference's largest magnitude: the median,
    99th percentile and maximum of |x - ref| / max|ref|, the rms error over
    the rms of the reference, and the number of elements."""
    x, ref = np.asarray(x, dtype=np.float64), np.asarray(ref, dtype=np.float64)
    fin = np.isfinite(ref)
    d = np.abs(x[fin] - ref[fin])
    r = ref[fin]
    if d.size == 0:
        return {"n": 0}
    scale = max(float(np.abs(r).max()), 1e-300)
    rel = d / scale
    rms_ref = float(np.sqrt(np.mean(r * r)))
    return {"n": int(d.size), "p50": float(np.percentile(rel, 50)),
            "p99": float(np.percentile(rel, 99)), "max": float(rel.max()),
            "rms_rel": float(np.sqrt(np.mean(d * d)) / rms_ref) if rms_ref > 0 else 0.0}


def record(label, report, stats):
    """Append one parity record (max-normalised errors and elementwise
    statistics) as a JSON line to the file named by RELPOS_PARITY_REPORT."""
    path = os.environ.get("RELPOS_PARITY_REPORT")
    if not path:
        return
    with open(path, "a") as fh:
        fh.write(json.dumps({"case": label, "err": report, "stats": stats}) + "\n")


def compare(got, ref, names, sel=None, tol_o=TOL_O, tol_g=TOL_G, label="", dtype=None):
    """Assert the tolerances on the named outputs; ``sel`` indexes a subset.
    With a 16-bit ``dtype`` the output O is also checked element by element
    (check_rows_ulp).  Returns the max-normalised errors; the elementwise
    statistics go to the parity record."""
    report = {}
    stats = {}
    for n in names:
        if ref.get(n) is None:
            assert got.get(n) is None, n
            continue
        a, r = got[n], ref[n]
        if sel is not None:
            a, r = a[sel], r[sel]
        if n == "lse":
            fin = np.isfinite(r)
            assert np.array_equal(fin, np.isfinite(a)), f"{label} lse: -inf rows differ"
            err = float(np.abs(a[fin] - r[fin]).max()) if fin.any() else 0.0
            report[n] = err
            assert err <= TOL_LSE_ABS, f"{label} lse abs err {err:.3e}"
            continue
        err = rel_err(a, r)
        report[n] = err
        stats[n] = elementwise_stats(a, r)
        tol = tol_o if n == "O" else tol_g
        if np.abs(r[np.isfinite(r)]).max(initial=0.0) < 1e-12:
            tol = ZERO_ABS
        assert err <= tol, f"{label} {n}: err {err:.3e} > {tol:.1e}"
        if n == "O" and dtype is not None:
            u = check_rows_ulp(a, r, dtype, label)
            if u is not None:
                stats[n].update(u)
    record(label, report, stats)
    return report
