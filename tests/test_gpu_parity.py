"""GPU parity: the HIP path against the fp64 oracle on the same seeded inputs.

Small shapes (oracle over everything) span several 128-row blocks and 64-key
tiles with a ragged tail, every map, every term, both masks, shared tables
and degenerate sizes.  Full shapes (the 8K layer-benchmark workloads, run in
the launch configuration the benchmark times) compare every output of one
head completely and O/LSE on sampled rows of the other heads.
"""

import math
import sys

import numpy as np
import pytest
import torch

from parity_util import compare, gpu_run, make_inputs, oracle_run, rel_err, require_gpu, \
    tolerances
from relpos_synth import DEBERTA256, DEBERTA_LOG, IDENTITY, SHAW16, T5_32_128, WORKLOADS, \
    Workload, sweep_workloads

pytestmark = pytest.mark.gpu

ALL = ("O", "lse", "dq", "dk", "dv", "daq", "dak", "db")

SMALL = [
    Workload("shaw_ragged_f16", 2, 2, 333, 64, "f16", SHAW16, 1 / 8, has_aq=True),
    Workload("shaw_n256_f32", 1, 1, 256, 64, "f32", SHAW16, 1 / 8, has_aq=True),
    Workload("deberta_f16", 1, 3, 600, 64, "f16", {"kind": "truncated", "lo": -40, "hi": 31},
             1 / math.sqrt(192), has_aq=True, has_ak=True),
    Workload("deberta_full_range_f16", 1, 2, 640, 64, "f16", DEBERTA256, 1 / math.sqrt(192),
             has_aq=True, has_ak=True),
    Workload("t5_keypad_bf16", 2, 2, 500, 64, "bf16", T5_32_128, 1.0, has_b=True,
             key_padding=True, pad_frac=0.3),
    Workload("txl_causal_bf16", 2, 2, 300, 64, "bf16", IDENTITY, 1 / 8, has_aq=True, has_b=True,
             causal=True, b_std=0.02),
    Workload("txl_all_terms_f16", 1, 2, 300, 64, "f16", IDENTITY, 1 / 8, has_aq=True,
             has_ak=True, has_b=True, b_std=0.1),
    Workload("trunc_all_masks_f32", 2, 2, 200, 64, "f32", {"kind": "truncated", "lo": -20,
                                                             "hi": 9},
             0.2, has_aq=True, has_ak=True, has_b=True, causal=True, key_padding=True),
    Workload("t5_vector_tables_f16", 1, 2, 400, 64, "f16", T5_32_128, 1 / 8, has_aq=True,
             has_ak=True, has_b=True),
    Workload("t5_unidirectional_bf16", 1, 2, 260, 64, "bf16",
             {"kind": "t5", "num_buckets": 32, "max_distance": 128, "bidirectional": False},
             1 / 8, has_aq=True, has_b=True, causal=True),
    Workload("shared_tables_f16", 2, 3, 270, 64, "f16", {"kind": "truncated", "lo": -64,
                                                           "hi": 64},
             1 / 8, has_aq=True, has_ak=True, has_b=True, shared_tables=True),
    Workload("grouped_truncation_f16", 1, 2, 200, 64, "f16", {"kind": "truncated", "lo": -250,
                                                                "hi": 150},
             1 / 8, has_aq=True, has_ak=True, has_b=True),
    Workload("no_tables_causal_bf16", 1, 2, 190, 64, "bf16", {"kind": "truncated", "lo": -1,
                                                                "hi": 1}, 1 / 8, causal=True),
    Workload("one_row_table_f16", 1, 1, 150, 64, "f16", {"kind": "truncated", "lo": 3, "hi": 3},
             1 / 8, has_aq=True, has_ak=True, has_b=True),
    Workload("n5_f16", 1, 1, 5, 64, "f16", SHAW16, 1 / 8, has_aq=True, has_ak=True, has_b=True),
    Workload("n1_bf16", 1, 1, 1, 64, "bf16", IDENTITY, 1 / 8, has_aq=True, has_b=True),
    Workload("n129_causal_f16", 1, 1, 129, 64, "f16", IDENTITY, 1 / 8, has_aq=True, has_b=True,
             causal=True, b_std=0.02),
    # wide bands (windows of >= 1024 columns, as here, or no shorter than the
    # sequence, as in the tiny cases above): Z^Q rows staged in LDS by the
    # forward and the query pass, band stores staged, rows of dZ^Q shifted;
    # causal: grouped query / key passes
    Workload("wide_band_causal_bf16", 1, 2, 1000, 64, "bf16", IDENTITY, 1 / 8, has_aq=True,
             has_b=True, causal=True, b_std=0.02),
    Workload("wide_band_all_terms_f16", 1, 1, 1100, 64, "f16", IDENTITY, 1 / 8, has_aq=True,
             has_ak=True, has_b=True, b_std=0.1),
    # wide windows without a query-side table: the query pass stages its band
    # stores but has no Z^Q rows to stage; b is looked up per band score
    Workload("wide_band_key_and_bias_f16", 1, 2, 1100, 64, "f16", IDENTITY, 1 / 8, has_aq=False,
             has_ak=True, has_b=True, b_std=0.1),
    Workload("wide_band_bias_only_bf16", 1, 2, 1060, 64, "bf16", IDENTITY, 1 / 8, has_aq=False,
             has_b=True, causal=True, b_std=0.1),
    Workload("wide_band_causal_keypad_f16", 2, 1, 1050, 64, "f16",
             {"kind": "truncated", "lo": -1040, "hi": 1030}, 1 / 8, has_aq=True, has_ak=True,
             causal=True, key_padding=True, pad_frac=0.2),
    # log buckets: unfolded to [-300, 279] (580 columns: staged key-pass band
    # stores), every term, copied columns folded back
    Workload("log_buckets_f16", 1, 2, 900, 64, "f16",
             {"kind": "log", "num_buckets": 64, "max_distance": 300}, 1 / 8, has_aq=True,
             has_ak=True, has_b=True),
    Workload("log_buckets_keypad_bf16", 2, 2, 420, 64, "bf16",
             {"kind": "log", "num_buckets": 32, "max_distance": 40}, 1 / 8, has_aq=True,
             has_b=True, key_padding=True, pad_frac=0.3),
    # attention dropout (t / 256), with every kernel variant it reaches:
    # plain, key-side term, staged rows, grouped causal blocks, padding
    Workload("dropout_shaw_ragged_f16", 2, 2, 333, 64, "f16", SHAW16, 1 / 8, has_aq=True,
             dropout=(26, 0x9E3779B97F4A7C15, 3)),
    Workload("dropout_all_terms_keypad_bf16", 2, 2, 600, 64, "bf16",
             {"kind": "truncated", "lo": -40, "hi": 31}, 1 / math.sqrt(192), has_aq=True,
             has_ak=True, has_b=True, key_padding=True, pad_frac=0.3,
             dropout=(64, 12345, 0)),
    Workload("dropout_wide_band_causal_f16", 1, 2, 1000, 64, "f16", IDENTITY, 1 / 8,
             has_aq=True, has_b=True, causal=True, b_std=0.02, dropout=(128, 7, 0xFFFFFFFF)),
    Workload("dropout_t5_keypad_bf16", 2, 2, 500, 64, "bf16", T5_32_128, 1.0, has_b=True,
             key_padding=True, pad_frac=0.3, dropout=(200, 2 ** 63 + 11, 5)),
    Workload("dropout_shared_tables_f16", 2, 3, 270, 64, "f16",
             {"kind": "truncated", "lo": -64, "hi": 64}, 1 / 8, has_aq=True, has_ak=True,
             has_b=True, shared_tables=True, dropout=(13, 99, 1)),
    Workload("dropout_nearly_all_n5_f16", 1, 1, 5, 64, "f16", SHAW16, 1 / 8, has_aq=True,
             has_ak=True, has_b=True, dropout=(255, 3, 0)),
    # bucketed maps shorter than their saturation offset: the unfolded map is
    # clipped to the offsets that exist (+-(N - 1)), and bucket rows no
    # offset reaches get zero gradients
    Workload("t5_shorter_than_saturation_f16", 2, 2, 50, 64, "f16", T5_32_128, 1 / 8,
             has_aq=True, has_ak=True, has_b=True, key_padding=True, pad_frac=0.3),
    Workload("log_huge_max_distance_bf16", 1, 2, 300, 64, "bf16",
             {"kind": "log", "num_buckets": 256, "max_distance": 1 << 20}, 1 / 8, has_aq=True,
             has_ak=True, has_b=True, causal=True),
    Workload("t5_huge_max_distance_f32", 1, 2, 200, 64, "f32",
             {"kind": "t5", "num_buckets": 32, "max_distance": 1 << 24, "bidirectional": True},
             1.0, has_b=True),
]


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_small_parity(w):
    dev = require_gpu()
    x = make_inputs(w)
    _say(f"[gpu] small parity {w.name} B{w.B} H{w.H} N{w.N} {w.dtype}")
    got = gpu_run(w, x, dev)
    ref = oracle_run(w, x)
    to, tg = tolerances(w.dtype)
    rep = compare(got, ref, ALL, tol_o=to, tol_g=tg, label=w.name, dtype=w.dtype)
    _say(f"  {w.name}: " + " ".join(f"{k}={v:.2e}" for k, v in rep.items()))


def _random_workloads(n, seed=7):
    """Seeded random small configurations: map kind and parameters, terms,
    masks, dtype, shared tables, a ragged N and, for 16-bit inputs, attention
    dropout half of the time (fixed by the seed, so every run checks the same
    cases)."""
    rng = np.random.default_rng(seed)
    rng_drop = np.random.default_rng(seed + 1)  # its own stream: the other draws stay put
    out = []
    for c in range(n):
        N = int(rng.integers(1, 700))
        kind = ["truncated", "t5", "identity", "log"][c % 4]
        if kind == "truncated":
            lo = int(rng.integers(-300, 1))
            phi = {"kind": kind, "lo": lo, "hi": int(rng.integers(lo, 300))}
        elif kind == "t5":
            nb = int(rng.choice([8, 16, 32, 64]))
            bi = bool(rng.integers(0, 2))
            per = nb // 2 if bi else nb
            phi = {"kind": kind, "num_buckets": nb, "bidirectional": bi,
                   "max_distance": int(rng.integers(per // 2 + 1, 400))}
        elif kind == "identity":
            phi = {"kind": kind}
        else:
            k = int(rng.choice([4, 16, 64, 128]))
            phi = {"kind": kind, "num_buckets": k,
                   "max_distance": int(rng.integers(k // 2 + 2, 3 * k))}
        terms = rng.integers(0, 2, size=3).astype(bool)
        dtype = ["f16", "bf16", "f32"][int(rng.integers(0, 3))]
        drop = (int(rng_drop.integers(1, 256)), int(rng_drop.integers(0, 2 ** 63)),
                int(rng_drop.integers(0, 2 ** 32)))
        if dtype == "f32" or rng_drop.random() < 0.5:
            drop = None
        tag = "" if drop is None else f"_drop{drop[0]}"
        out.append(Workload(f"random{c}_{kind}_{dtype}{tag}", int(rng.integers(1, 3)),
                            int(rng.integers(1, 4)), N, 64, dtype, phi,
                            float(rng.choice([1 / 8, 0.3, 1.0])), has_aq=bool(terms[0]),
                            has_ak=bool(terms[1]), has_b=bool(terms[2]),
                            causal=bool(rng.integers(0, 2)),
                            key_padding=bool(rng.integers(0, 2)), pad_frac=0.4,
                            shared_tables=bool(rng.integers(0, 2)), b_std=0.3,
                            seed=100 + c, dropout=drop))
    return out


# In-block relation (RELPOS_REL_INBLOCK): the forward computes the query-side
# term inside each block from Q and the tables, with no stored projection.
# Narrow and wide bands, saturated tiles on both sides, ragged tails, every
# mask, b, bucketed maps through the fold table, shared tables, dropout and
# degenerate sizes; "stored_" cases pin the stored path on shapes that the
# automatic choice sends in-block (the identity map, short sequences).
INBLOCK = [
    Workload("ib_shaw_ragged_f16", 2, 2, 333, 64, "f16", SHAW16, 1 / 8, has_aq=True, relation=2),
    Workload("ib_trunc_bias_bf16", 1, 3, 700, 64, "bf16", {"kind": "truncated", "lo": -100,
                                                            "hi": 60},
             1 / 8, has_aq=True, has_b=True, relation=2),
    Workload("ib_txl_causal_bf16", 2, 2, 300, 64, "bf16", IDENTITY, 1 / 8, has_aq=True,
             has_b=True, causal=True, b_std=0.02, relation=2),
    Workload("ib_keypad_causal_f16", 2, 2, 450, 64, "f16", {"kind": "truncated", "lo": -64,
                                                             "hi": 64},
             1 / 8, has_aq=True, has_b=True, causal=True, key_padding=True, pad_frac=0.3,
             relation=2),
    Workload("ib_log_buckets_keypad_bf16", 2, 2, 420, 64, "bf16",
             {"kind": "log", "num_buckets": 32, "max_distance": 40}, 1 / 8, has_aq=True,
             has_b=True, key_padding=True, pad_frac=0.3, relation=2),
    Workload("ib_t5_vector_f16", 1, 2, 400, 64, "f16", T5_32_128, 1 / 8, has_aq=True,
             has_b=True, relation=2),
    Workload("ib_shared_tables_f16", 2, 3, 270, 64, "f16", {"kind": "truncated", "lo": -64,
                                                             "hi": 64},
             1 / 8, has_aq=True, has_b=True, shared_tables=True, relation=2),
    Workload("ib_one_row_table_bf16", 1, 1, 150, 64, "bf16", {"kind": "truncated", "lo": 3,
                                                               "hi": 3},
             1 / 8, has_aq=True, has_b=True, relation=2),
    Workload("ib_n5_f16", 1, 1, 5, 64, "f16", SHAW16, 1 / 8, has_aq=True, has_b=True, relation=2),
    Workload("ib_n1_bf16", 1, 1, 1, 64, "bf16", IDENTITY, 1 / 8, has_aq=True, has_b=True,
             relation=2),
    Workload("ib_wide_causal_f16", 1, 2, 1000, 64, "f16", IDENTITY, 1 / 8, has_aq=True,
             has_b=True, causal=True, b_std=0.02, relation=2),
    Workload("ib_dropout_shaw_f16", 2, 2, 333, 64, "f16", SHAW16, 1 / 8, has_aq=True,
             has_b=True, dropout=(26, 0x9E3779B97F4A7C15, 3), relation=2),
    Workload("ib_dropout_txl_bf16", 1, 2, 520, 64, "bf16", IDENTITY, 1 / 8, has_aq=True,
             has_b=True, causal=True, b_std=0.02, dropout=(64, 12345, 0), relation=2),
    Workload("stored_txl_causal_bf16", 2, 2, 300, 64, "bf16", IDENTITY, 1 / 8, has_aq=True,
             has_b=True, causal=True, b_std=0.02, relation=1),
    Workload("stored_wide_band_causal_bf16", 1, 2, 1000, 64, "bf16", IDENTITY, 1 / 8,
             has_aq=True, has_b=True, causal=True, b_std=0.02, relation=1),
    Workload("stored_short_shaw_f16", 4, 2, 200, 64, "f16", {"kind": "truncated", "lo": -128,
                                                              "hi": 128},
             1 / 8, has_aq=True, has_b=True, relation=1),
]


@pytest.mark.parametrize("w", INBLOCK, ids=[w.name for w in INBLOCK])
def test_inblock_parity(w):
    """Every output against the oracle (the backward projects Z^Q itself)."""
    test_small_parity(w)


def test_inblock_matches_stored_forward():
    """The in-block forward against the stored one on the same inputs: the
    same mathematics in fp32, summed in a different order, so O agrees to
    well within one 16-bit unit and LSE closely; both are deterministic."""
    dev = require_gpu()
    w = Workload("ib_vs_stored_f16", 2, 3, 777, 64, "f16", {"kind": "truncated", "lo": -200,
                                                             "hi": 100},
                 1 / 8, has_aq=True, has_b=True, causal=True)
    x = make_inputs(w)
    _say("[gpu] in-block vs stored forward")
    a = gpu_run(w.with_(relation=2), x, dev, backward=False)
    a2 = gpu_run(w.with_(relation=2), x, dev, backward=False)
    s = gpu_run(w.with_(relation=1), x, dev, backward=False)
    assert np.array_equal(a["O"], a2["O"]) and np.array_equal(a["lse"], a2["lse"])
    assert rel_err(a["O"], s["O"]) < 1e-3
    assert np.abs(a["lse"] - s["lse"]).max() < 1e-4


@pytest.mark.parametrize("w", _random_workloads(24), ids=lambda w: w.name)
def test_random_small_parity(w):
    """Seeded random configurations, every output against the oracle."""
    test_small_parity(w)


@pytest.mark.parametrize("table", ["aq", "ak", "b"])
def test_present_all_zero_table(table):
    """A table passed as all zeros is not the same call as an absent one (the
    kernels add its lookups and return its gradient), but it must give the
    absent case's O and dQ/dK/dV, and a gradient equal to the oracle's, which
    is non-zero: daQ = (dZ^Q)^T Q, daK = (dZ^K)^T K, db = column sums of dZ^Q."""
    dev = require_gpu()
    w = Workload(f"zero_{table}_f16", 1, 2, 333, 64, "f16",
                 {"kind": "truncated", "lo": -40, "hi": 31}, 1 / 8,
                 **{"has_" + table: True})
    x = make_inputs(w)
    x[table] = torch.zeros_like(x[table])
    _say(f"[gpu] present all-zero table {table}")
    got = gpu_run(w, x, dev)
    ref = oracle_run(w, x)
    to, tg = tolerances(w.dtype)
    compare(got, ref, ALL, tol_o=to, tol_g=tg, label=w.name, dtype=w.dtype)
    g = {"aq": "daq", "ak": "dak", "b": "db"}[table]
    assert np.abs(ref[g]).max() > 1e-3 and np.abs(got[g]).max() > 1e-3, g
    absent = w.with_(has_aq=False, has_ak=False, has_b=False, name=f"absent_{table}")
    y = dict(x)
    y[table] = None
    got0 = gpu_run(absent, y, dev)
    compare({k: got[k] for k in ("O", "lse", "dq", "dk", "dv")},
            {k: got0[k] for k in ("O", "lse", "dq", "dk", "dv")},
            ("O", "lse", "dq", "dk", "dv"), tol_o=to, tol_g=tg, label=f"zero vs absent {table}")


@pytest.mark.parametrize("B,N,relation", [(1, 0, 0), (0, 100, 0), (2, 0, 2), (0, 0, 1)])
def test_empty_inputs(B, N, relation):
    """No token (N = 0) or no batch entry (B = 0): empty outputs, and the
    table gradients exist and are zero (no pair reaches any row)."""
    import exact_relative_position_amd as rp
    dev = require_gpu()
    H, R = 2, 33
    f16 = dict(dtype=torch.float16, device=dev)
    q = torch.zeros(B, H, N, 64, **f16)
    aq = torch.randn(H, R, 64, **f16)
    bt = torch.randn(H, R, **f16)
    phi = SHAW16
    _say(f"[gpu] empty inputs B{B} N{N} relation {relation}")
    O, lse, zs = rp.forward(q, q, q, aq, None, bt, phi=phi, tau=0.125, relation=relation)
    assert O.shape == q.shape and lse.shape == (B, H, N)
    dq, dk, dv, daq, dak, db = rp.backward(q, q, q, aq, None, bt, O, lse, q, zs, phi=phi,
                                           tau=0.125, relation=relation)
    torch.cuda.synchronize(dev)
    assert dq.shape == q.shape and dk.shape == q.shape and dv.shape == q.shape and dak is None
    assert daq.shape == (H, R, 64) and db.shape == (H, R)
    assert torch.count_nonzero(daq).item() == 0 and torch.count_nonzero(db).item() == 0


def test_fully_masked_batch():
    dev = require_gpu()
    w = Workload("dead_rows_f16", 2, 2, 200, 64, "f16", SHAW16, 1 / 8, has_aq=True, has_b=True,
                 key_padding=True)
    x = make_inputs(w)
    x["key_len"][0] = 0
    _say(f"[gpu] fully masked batch {w.name}")
    got = gpu_run(w, x, dev)
    ref = oracle_run(w, x)
    compare(got, ref, ALL, tol_o=tolerances(w.dtype)[0], tol_g=tolerances(w.dtype)[1],
            label=w.name)
    assert np.all(got["O"][0] == 0) and np.all(np.isneginf(got["lse"][0]))
    for n in ("dq", "dk", "dv"):
        assert np.all(got[n][0] == 0), n


def test_padded_keys_have_exact_zero_grads():
    dev = require_gpu()
    w = WORKLOADS["t5_n8192_f16"].with_(N=777, H=2, name="t5_pad_zero")
    x = make_inputs(w)
    x["key_len"][0] = 500
    _say("[gpu] padded keys zero grads")
    got = gpu_run(w, x, dev)
    assert np.all(got["dk"][0, :, 500:] == 0) and np.all(got["dv"][0, :, 500:] == 0)


@pytest.mark.parametrize("dropout", [None, (26, 77, 1)])
def test_recompute_projection_matches_saved(dropout):
    dev = require_gpu()
    w = SMALL[2].with_(dropout=dropout)
    x = make_inputs(w)
    _say("[gpu] zsave vs recompute")
    a = gpu_run(w, x, dev, keep_z=True)
    b = gpu_run(w, x, dev, keep_z=False)
    for n in ALL:
        if a[n] is not None:
            np.testing.assert_array_equal(a[n], b[n], err_msg=n)


def test_bitwise_deterministic():
    dev = require_gpu()
    w = WORKLOADS["deberta_n8192_f16"].with_(N=2048, H=4, name="det")
    x = make_inputs(w)
    _say("[gpu] determinism")
    a = gpu_run(w, x, dev)
    b = gpu_run(w, x, dev)
    for n in ALL:
        if a[n] is not None:
            np.testing.assert_array_equal(a[n], b[n], err_msg=n)


@pytest.mark.parametrize("dropout", [None, (26, 77, 1)])
@pytest.mark.parametrize("inblock", [False, True])
def test_strided_layout_bnhd(dropout, inblock):
    """Q, K, V given as [B, N, H, d] memory viewed as [B, H, N, d] (with the
    relation stored, or computed in the block from Q read through the
    strides)."""
    dev = require_gpu()
    if inblock:
        w = Workload("strided_inblock_bf16", 2, 3, 300, 64, "bf16", IDENTITY, 1 / 8,
                     has_aq=True, has_b=True, causal=True, b_std=0.02, dropout=dropout,
                     relation=2)
    else:
        w = Workload("strided_f16", 2, 3, 257, 64, "f16", SHAW16, 1 / 8, has_aq=True,
                     has_ak=True, dropout=dropout)
    x = make_inputs(w)
    _say("[gpu] strided layout")
    ref = gpu_run(w, x, dev)
    y = dict(x)
    for n in ("q", "k", "v", "do"):
        y[n] = x[n].transpose(1, 2).contiguous().transpose(1, 2)
    got = gpu_run(w, y, dev)
    for n in ALL:
        if ref[n] is not None:
            np.testing.assert_array_equal(got[n], ref[n], err_msg=n)


@pytest.mark.parametrize("causal", [False, True])
def test_fused_passes_match_separate_launches(causal):
    """The query and key passes in one launch (causal: dealt rank by rank)
    give bit for bit the outputs of one launch per pass; the shape has more
    blocks per pass than the device holds at once, so the causal launch is
    not split between wave groups."""
    import exact_relative_position_amd._binding as B_
    dev = require_gpu()
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    N = 1536
    nblk = N // 128
    H = (2 * cus) // nblk + 1
    w = Workload("fused_passes", 1, H, N, 64, "f16", {"kind": "truncated", "lo": -300, "hi": 300},
                 1 / 8, has_aq=True, has_ak=True, has_b=True, causal=causal)
    x = make_inputs(w)
    t = {k: (None if v is None else v.to(dev)) for k, v in x.items()}
    _say(f"[gpu] fused vs separate passes causal={causal} H={H}")
    run = B_.Prepared(t["q"], t["k"], t["v"], t["aq"], t["ak"], t["b"], t["do"], phi=w.phi,
                      tau=w.tau, causal=causal, key_len=t["key_len"], keep_z=True)
    outs = ("dq", "dk", "dv", "daq", "dak", "db")
    got = []
    for passes in ((B_.BWD_QUERY_PASS | B_.BWD_KEY_PASS,), (B_.BWD_QUERY_PASS, B_.BWD_KEY_PASS)):
        for n in outs:
            getattr(run, n).fill_(float("nan"))
        run.fwd()
        run.bwd(B_.BWD_PREPARE)
        for p in passes:
            run.bwd(p)
        run.bwd(B_.BWD_CONTRACT)
        torch.cuda.synchronize(dev)
        got.append({n: getattr(run, n).cpu().clone() for n in outs})
    for n in outs:
        assert torch.isfinite(got[0][n]).all(), n
        assert torch.equal(got[0][n], got[1][n]), n


FULL = ["shaw_n256_f32", "shaw_n8192_f16", "deberta_n8192_f16", "deberta_log_n8192_f16",
        "t5_n8192_f16", "txl_n4096_bf16", "txl_n8192_f16"]


@pytest.mark.parametrize("name", FULL)
def test_full_shape_parity(name):
    """Every output of head 0 (all batches) in full, O/LSE on sampled rows elsewhere."""
    _full_parity(WORKLOADS[name])


@pytest.mark.parametrize("name", ["shaw_n8192_f16", "deberta_n8192_f16", "txl_n4096_bf16",
                                  "txl_n8192_f16"])
def test_full_shape_dropout_parity(name):
    """Full-size workloads with attention dropout p = 26/256 (about 0.1): the
    fused launch, the two-group split (Transformer-XL 4K) and the causal
    rank-by-rank launch (Transformer-XL 8K)."""
    w = WORKLOADS[name]
    _full_parity(w.with_(name=name + "_dropout", dropout=(26, 2024, 0)))


def test_dropout_zero_is_bitwise_no_dropout():
    dev = require_gpu()
    w = SMALL[0]
    x = make_inputs(w)
    a = gpu_run(w, x, dev)
    b = gpu_run(w.with_(dropout=(0, 5, 5)), x, dev)
    for n in ALL:
        if a[n] is not None:
            assert np.array_equal(a[n], b[n]), n


def test_dropout_offset_changes_the_mask_and_is_deterministic():
    dev = require_gpu()
    w = next(v for v in SMALL if v.name == "dropout_shaw_ragged_f16")
    x = make_inputs(w)
    a = gpu_run(w, x, dev)
    a2 = gpu_run(w, x, dev)
    c = gpu_run(w.with_(dropout=(w.dropout[0], w.dropout[1], w.dropout[2] + 1)), x, dev)
    for n in ALL:
        if a[n] is not None:
            assert np.array_equal(a[n], a2[n]), n
    assert not np.array_equal(a["O"], c["O"])
    assert np.array_equal(a["lse"], c["lse"])  # the LSE is that of the undropped softmax


def test_autograd_wrapper_with_dropout():
    """relpos_attention keeps the dropout descriptor for its backward: its
    gradients are the binding-level backward's, bit for bit, and match the
    oracle."""
    dev = require_gpu()
    import exact_relative_position_amd as rp
    from parity_util import gpu_dropout
    w = next(v for v in SMALL if v.name == "dropout_all_terms_keypad_bf16")
    x = make_inputs(w)
    got = gpu_run(w, x, dev)
    t = {k: (None if v is None else v.to(dev)) for k, v in x.items()}
    leaves = {n: t[n].clone().requires_grad_(True) for n in ("q", "k", "v", "aq", "ak", "b")}
    O = rp.relpos_attention(leaves["q"], leaves["k"], leaves["v"], leaves["aq"], leaves["ak"],
                            leaves["b"], phi=w.phi, tau=w.tau, causal=w.causal,
                            key_len=t["key_len"], dropout=gpu_dropout(w))
    O.backward(t["do"])
    torch.cuda.synchronize(dev)
    f64 = lambda z: z.detach().cpu().double().numpy()  # noqa: E731
    assert np.array_equal(f64(O), got["O"])
    for n, g in (("q", "dq"), ("k", "dk"), ("v", "dv")):
        assert np.array_equal(f64(leaves[n].grad), got[g]), n
    # table gradients come back in the table dtype (bf16 here)
    for n, g in (("aq", "daq"), ("ak", "dak"), ("b", "db")):
        np.testing.assert_array_equal(f64(leaves[n].grad),
                                      torch.from_numpy(got[g]).to(torch.bfloat16).double().numpy(),
                                      err_msg=n)


def test_dropout_fp32_is_rejected():
    dev = require_gpu()
    import exact_relative_position_amd as rp
    w = next(v for v in SMALL if v.dtype == "f32")
    x = {k: (None if v is None else v.to(dev)) for k, v in make_inputs(w).items()}
    with pytest.raises(rp.RelposError, match="UNSUPPORTED"):
        rp.forward(x["q"], x["k"], x["v"], x["aq"], None, None, phi=w.phi, tau=w.tau,
                   dropout=(0.1, 1, 0))


def test_shaw_n16384_parity():
    """The largest point of the memory-scaling run (Shaw, 1 x 12 x 16384)."""
    from relpos_synth import memory_scaling_workloads
    _full_parity(memory_scaling_workloads()["shaw_n16384_f16"], n_others=2)


@pytest.mark.parametrize("name", list(sweep_workloads()))
def test_sweep_parity(name):
    """The layer sweep's points (N = 128 .. 8192 at 16384 tokens, each
    mechanism): head 0 over every batch in full, O/LSE on sampled rows of a
    few other heads."""
    _full_parity(sweep_workloads()[name], n_others=2)


def full_heads(H):
    """Heads whose every output is checked at full size: the first, a middle
    and the last.  Equal-work launches place one head's blocks on one XCD
    (head mod 8) and causal launches deal blocks rank by rank over all
    heads, so these three reach different XCDs, the start, middle and end of
    the dispatch order, and both ends of the causal interleave."""
    return sorted({0, H // 2, H - 1})


def test_inblock_attend_stage_builds_its_tables():
    """With the relation in the block, the attention stage alone (no
    projection stage before it) builds the fold table of a bucketed map
    itself and gives the oracle's O and LSE."""
    import exact_relative_position_amd._binding as B_
    dev = require_gpu()
    w = Workload("ib_attend_stage_log_f16", 1, 2, 500, 64, "f16",
                 {"kind": "log", "num_buckets": 32, "max_distance": 60}, 1 / 8, has_aq=True,
                 has_b=True, relation=2)
    x = make_inputs(w)
    t = {k: (None if v is None else v.to(dev)) for k, v in x.items()}
    _say("[gpu] in-block attend stage alone")
    run = B_.Prepared(t["q"], t["k"], t["v"], t["aq"], t["ak"], t["b"], t["do"], phi=w.phi,
                      tau=w.tau, relation=2)
    run.fwd(B_.FWD_ATTEND)
    torch.cuda.synchronize(dev)
    got = {"O": run.O.cpu().double().numpy(), "lse": run.lse.cpu().double().numpy()}
    ref = oracle_run(w, x, backward=False)
    to, tg = tolerances(w.dtype)
    compare(got, ref, ("O", "lse"), tol_o=to, tol_g=tg, label=w.name, dtype=w.dtype)


@pytest.mark.parametrize("name,relation", [("txl_n4096_bf16", 1), ("txl_n4096_bf16", 2),
                                           ("shaw_n8192_f16", 2)])
def test_full_shape_relation_modes(name, relation):
    """A full-size workload with the relation forced stored (1) or in the
    block (2), whichever the automatic choice would not take."""
    w = WORKLOADS[name]
    _full_parity(w.with_(name=f"{name}_rel{relation}", relation=relation))


def _full_parity(w, n_others=6):
    dev = require_gpu()
    name = w.name
    x = make_inputs(w)
    _say(f"[gpu] full-shape parity {name} B{w.B} H{w.H} N{w.N} {w.dtype}")
    got = gpu_run(w, x, dev)
    to, tg = tolerances(w.dtype)
    heads = full_heads(w.H)
    rep = {}
    for h in heads:
        # every output of head h over the whole batch, table gradients
        # included (per-head tables: the sum over the batch of head h only)
        pairs = [(b, h) for b in range(w.B)]
        ref = oracle_run(w, x, bh=pairs)
        r = compare(got, {k: v for k, v in ref.items() if k in ("O", "lse", "dq", "dk", "dv")},
                    ("O", "lse", "dq", "dk", "dv"), sel=(slice(None), h), tol_o=to, tol_g=tg,
                    label=f"{name} h{h}", dtype=w.dtype)
        tabs = {n: ref[n][h] for n in ("daq", "dak", "db") if ref[n] is not None}
        r.update(compare({n: got[n][h] for n in tabs}, tabs, tuple(tabs), tol_o=to, tol_g=tg,
                         label=f"{name} h{h} tables"))
        for k, v in r.items():
            rep[k] = max(rep.get(k, 0.0), v)
    rng = np.random.default_rng(1)
    rows = np.sort(rng.choice(w.N, size=min(w.N, 48), replace=False))
    others = [(b, h) for b in range(w.B) for h in range(w.H) if h not in heads][:n_others]
    if others:
        refo = oracle_run(w, x, bh=others, query_rows=rows, backward=False)
        for (b, h) in others:
            compare({"O": got["O"][b, h, rows], "lse": got["lse"][b, h, rows]},
                    {"O": refo["O"][b, h, rows], "lse": refo["lse"][b, h, rows]},
                    ("O", "lse"), tol_o=to, tol_g=tg, label=f"{name} b{b} h{h}",
                    dtype=w.dtype)
    _say(f"  {name} heads {heads}: " + " ".join(f"{k}={v:.2e}" for k, v in rep.items()))


def test_phi_tables_bit_exact():
    dev = require_gpu()
    import exact_relative_position_amd as rp
    from oracle import phi_rows as oracle_rows
    cases = [(SHAW16, 256), ({"kind": "truncated", "lo": -128, "hi": 128}, 8192),
             (DEBERTA256, 8192), (T5_32_128, 8192), (IDENTITY, 4096),
             ({"kind": "t5", "num_buckets": 32, "max_distance": 128, "bidirectional": False},
              5000),
             ({"kind": "t5", "num_buckets": 64, "max_distance": 1000, "bidirectional": True},
              20000),
             (DEBERTA_LOG, 8192),
             ({"kind": "log", "num_buckets": 64, "max_distance": 300}, 2000),
             ({"kind": "log", "num_buckets": 32, "max_distance": 40}, 20000)]
    for phi, N in cases:
        _say(f"[gpu] phi rows {phi['kind']} N{N}")
        rows, fold = rp.phi_rows(phi, N, device=dev)
        torch.cuda.synchronize()
        want = oracle_rows(phi, N)
        np.testing.assert_array_equal(rows.cpu().numpy(), want)
        R, lo, hi = rp.phi_info(phi, N)
        o = np.arange(lo, hi + 1)
        np.testing.assert_array_equal(fold.cpu().numpy(), oracle_rows(phi, max(N, hi + 1))[
            o + max(N, hi + 1) - 1])


# Chunked query-side projection (zchunk): the forward and the backward
# recompute Z^Q and dZ^Q one chunk of queries at a time, so the memory is
# linear in N for the identity map.  Every output against the oracle, on
# shapes with several chunks and a ragged last one.
CHUNKED = [
    Workload("chunk_txl_causal_bf16", 2, 2, 1000, 64, "bf16", IDENTITY, 1 / 8, has_aq=True,
             has_b=True, causal=True, b_std=0.02, zchunk=256),
    Workload("chunk_txl_f16", 1, 3, 700, 64, "f16", IDENTITY, 1 / 8, has_aq=True, has_b=True,
             b_std=0.1, zchunk=128),
    Workload("chunk_txl_f32", 1, 2, 400, 64, "f32", IDENTITY, 1 / 8, has_aq=True, zchunk=128),
    Workload("chunk_trunc_keypad_f16", 2, 2, 900, 64, "f16",
             {"kind": "truncated", "lo": -300, "hi": 200}, 1 / 8, has_aq=True, has_b=True,
             key_padding=True, pad_frac=0.3, zchunk=256),
    Workload("chunk_t5_bias_bf16", 1, 2, 777, 64, "bf16", T5_32_128, 1.0, has_b=True,
             key_padding=True, zchunk=384),
    Workload("chunk_log_causal_f16", 1, 2, 640, 64, "f16",
             {"kind": "log", "num_buckets": 64, "max_distance": 300}, 1 / 8, has_aq=True,
             has_b=True, causal=True, zchunk=128),
    Workload("chunk_dropout_txl_f16", 1, 2, 600, 64, "f16", IDENTITY, 1 / 8, has_aq=True,
             has_b=True, causal=True, b_std=0.02, dropout=(26, 11, 2), zchunk=256),
    Workload("chunk_shared_tables_f16", 2, 3, 500, 64, "f16",
             {"kind": "truncated", "lo": -64, "hi": 64}, 1 / 8, has_aq=True, has_b=True,
             shared_tables=True, zchunk=128),
]


@pytest.mark.parametrize("w", CHUNKED, ids=[w.name for w in CHUNKED])
def test_chunked_projection_parity(w):
    """Every output against the oracle, with the automatic relation choice
    (the identity map's forward in-block, its backward chunked) and with the
    projection stored and chunked in both passes; stored, the forward's O
    and LSE and the dQ of the chunked run are the unchunked stored run's bit
    for bit (each query block does the same arithmetic on the same
    projection values), and the chunk-summed outputs (dK, dV, daQ, db) are
    deterministic."""
    test_small_parity(w)
    ws = w.with_(name=w.name + "_stored", relation=1)
    test_small_parity(ws)
    dev = require_gpu()
    x = make_inputs(w)
    got = gpu_run(ws, x, dev)
    again = gpu_run(ws, x, dev)
    whole = gpu_run(ws.with_(zchunk=0), x, dev, keep_z=False)
    for n in ALL:
        if got[n] is not None:
            np.testing.assert_array_equal(got[n], again[n], err_msg=n)
    for n in ("O", "lse", "dq"):
        np.testing.assert_array_equal(got[n], whole[n], err_msg=n)


@pytest.mark.parametrize("name", ["txl_n4096_bf16", "txl_n8192_f16"])
def test_full_shape_chunked_projection(name):
    """The Transformer-XL workloads with the projection computed 1024 queries
    at a time: every output of three heads against the oracle."""
    w = WORKLOADS[name]
    _full_parity(w.with_(name=name + "_chunk1024", zchunk=1024))
