"""Pins for the oracle's forward and backward (oracle/attention.py).

Each check reaches the oracle from outside its own code:
* hand-derived worked examples (tests/golden/worked_examples.json);
* brute force: pure-Python loops with explicit dot products (N <= 16, d <= 8);
* reduction to a library routine: with no relation tables the oracle equals
  torch's scaled_dot_product_attention (CPU, float64) and its autograd grads;
* autograd of a dense gather formulation written in torch (all gradients,
  tables included);
* central finite differences of sum(O * dO) for every input;
* invariants of softmax (shifts of b or of every aQ row change nothing,
  sum_r db_r = 0, sum_r daQ_r = 0), causal row 0, key padding zeros.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import phi_rows, num_rows

GOLD = os.path.join(os.path.dirname(__file__), "golden")

PHIS = {
    "shaw": {"kind": "truncated", "lo": -3, "hi": 2},
    "identity": {"kind": "identity"},
    "t5": {"kind": "t5", "num_buckets": 32, "max_distance": 128, "bidirectional": True,
           "max_exact": 8},
    "t5uni": {"kind": "t5", "num_buckets": 16, "max_distance": 32, "bidirectional": False},
}


def _rand(rng, B, H, N, d, phi, aq=True, ak=True, b=True, shared=False, scale=0.7):
    R = num_rows(phi, N)
    tH = () if shared else (H,)
    x = dict(
        q=rng.standard_normal((B, H, N, d)) * scale,
        k=rng.standard_normal((B, H, N, d)) * scale,
        v=rng.standard_normal((B, H, N, d)),
        aQ=rng.standard_normal(tH + (R, d)) * 0.5 if aq else None,
        aK=rng.standard_normal(tH + (R, d)) * 0.5 if ak else None,
        b=rng.standard_normal(tH + (R,)) if b else None,
        dO=rng.standard_normal((B, H, N, d)),
    )
    return x


def _num(v):
    if isinstance(v, str):
        mult = 1.0
        if v[0].isdigit():
            mult, v = float(v[0]), v[1:]
        return mult * math.log(float(v[2:]))
    return float(v)


def _arr(x):
    if x is None:
        return None
    return np.vectorize(_num, otypes=[np.float64])(np.array(x, dtype=object))


# ---------------------------------------------------------------- worked examples
def test_worked_examples():
    ex = json.load(open(os.path.join(GOLD, "worked_examples.json")))["examples"]
    for e in ex:
        q, k, v = (_arr(e[n])[None, None] for n in ("q", "k", "v"))
        aq, ak, b = _arr(e["aq"]), _arr(e["ak"]), _arr(e["b"])
        kl = None if e["key_len"] is None else np.array(e["key_len"])
        O, L = oracle.forward(q, k, v, aq, ak, b, phi=e["phi"], tau=e["tau"],
                              causal=e["causal"], key_len=kl)
        np.testing.assert_allclose(O[0, 0], _arr(e["O"]), rtol=0, atol=1e-12, err_msg=e["name"])
        np.testing.assert_allclose(L[0, 0], _arr(e["LSE"]), rtol=0, atol=1e-12, err_msg=e["name"])
        if "do" in e:
            g = oracle.backward(q, k, v, aq, ak, b, dO=_arr(e["do"])[None, None], phi=e["phi"],
                                tau=e["tau"], causal=e["causal"], key_len=kl)
            for name in ("dq", "dk", "dv"):
                np.testing.assert_allclose(g[name][0, 0], _arr(e[name]), atol=1e-12, err_msg=name)
            np.testing.assert_allclose(g["db"], _arr(e["db"]), atol=1e-12)


# ---------------------------------------------------------------- brute force
def _brute_forward(q, k, v, aQ, aK, b, phi, tau, causal, key_len):
    """Pure-Python loops: one score at a time, explicit dot products."""
    B, H, N, d = q.shape
    rows = phi_rows(phi, N)
    O = np.zeros((B, H, N, d))
    L = np.zeros((B, H, N))

    def dot(x, y):
        s = 0.0
        for t in range(len(x)):
            s += float(x[t]) * float(y[t])
        return s

    for bb in range(B):
        for h in range(H):
            tq = None if aQ is None else (aQ if aQ.ndim == 2 else aQ[h])
            tk = None if aK is None else (aK if aK.ndim == 2 else aK[h])
            tb = None if b is None else (b if b.ndim == 1 else b[h])
            for i in range(N):
                sc = []
                for j in range(N):
                    if (causal and j > i) or (key_len is not None and j >= key_len[bb]):
                        sc.append(None)
                        continue
                    r = int(rows[(j - i) + N - 1])
                    s = dot(q[bb, h, i], k[bb, h, j])
                    if tq is not None:
                        s += dot(q[bb, h, i], tq[r])
                    if tk is not None:
                        s += dot(k[bb, h, j], tk[r])
                    if tb is not None:
                        s += float(tb[r])
                    sc.append(tau * s)
                live = [s for s in sc if s is not None]
                if not live:
                    L[bb, h, i] = -math.inf
                    continue
                m = max(live)
                w = [0.0 if s is None else math.exp(s - m) for s in sc]
                tot = sum(w)
                L[bb, h, i] = m + math.log(tot)
                for t in range(d):
                    O[bb, h, i, t] = sum(w[j] * float(v[bb, h, j, t]) for j in range(N)) / tot
    return O, L


@pytest.mark.parametrize("phiname", list(PHIS))
@pytest.mark.parametrize("causal,padded", [(False, False), (True, False), (False, True)])
def test_brute_force(phiname, causal, padded):
    rng = np.random.default_rng([list(PHIS).index(phiname), int(causal), int(padded)])
    phi = PHIS[phiname]
    B, H, N, d = 2, 2, 13, 5
    x = _rand(rng, B, H, N, d, phi)
    kl = np.array([N - 4, N]) if padded else None
    O, L = oracle.forward(x["q"], x["k"], x["v"], x["aQ"], x["aK"], x["b"], phi=phi, tau=0.6,
                          causal=causal, key_len=kl, row_block=4)
    Ob, Lb = _brute_forward(x["q"], x["k"], x["v"], x["aQ"], x["aK"], x["b"], phi, 0.6, causal, kl)
    np.testing.assert_allclose(O, Ob, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(L, Lb, rtol=1e-12, atol=1e-12)


def test_brute_force_shared_tables_and_dead_rows():
    rng = np.random.default_rng(7)
    phi = PHIS["shaw"]
    x = _rand(rng, 2, 3, 9, 4, phi, shared=True)
    kl = np.array([0, 5])   # batch 0 has every key masked
    O, L = oracle.forward(x["q"], x["k"], x["v"], x["aQ"], x["aK"], x["b"], phi=phi, tau=1.1,
                          key_len=kl)
    Ob, Lb = _brute_forward(x["q"], x["k"], x["v"], x["aQ"], x["aK"], x["b"], phi, 1.1, False, kl)
    np.testing.assert_allclose(O, Ob, atol=1e-12)
    assert np.all(O[0] == 0) and np.all(np.isneginf(L[0]))
    np.testing.assert_allclose(L[1], Lb[1], atol=1e-12)
    g = oracle.backward(x["q"], x["k"], x["v"], x["aQ"], x["aK"], x["b"], dO=x["dO"], phi=phi,
                        tau=1.1, key_len=kl)
    for n in ("dq", "dk", "dv"):
        assert np.all(g[n][0] == 0)


# ---------------------------------------------------------------- SDPA reduction
@pytest.mark.parametrize("causal", [False, True])
def test_reduces_to_sdpa(causal):
    rng = np.random.default_rng(3)
    B, H, N, d = 2, 3, 70, 16
    x = _rand(rng, B, H, N, d, PHIS["shaw"], aq=False, ak=False, b=False)
    kl = np.array([N, 51])
    tau = 0.3
    O, L = oracle.forward(x["q"], x["k"], x["v"], phi=PHIS["shaw"], tau=tau, causal=causal,
                          key_len=kl, row_block=16)
    g = oracle.backward(x["q"], x["k"], x["v"], dO=x["dO"], phi=PHIS["shaw"], tau=tau,
                        causal=causal, key_len=kl, row_block=16)
    tq, tk, tv = (torch.tensor(x[n], requires_grad=True) for n in ("q", "k", "v"))
    allowed = torch.ones(B, 1, N, N, dtype=torch.bool)
    jj = torch.arange(N)
    for bb in range(B):
        allowed[bb, :, :, jj >= int(kl[bb])] = False
    if causal:
        allowed &= torch.ones(N, N, dtype=torch.bool).tril()
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=allowed, scale=tau)
    ref.backward(torch.tensor(x["dO"]))
    np.testing.assert_allclose(O, ref.detach().numpy(), atol=1e-12)
    for n, t in (("dq", tq), ("dk", tk), ("dv", tv)):
        np.testing.assert_allclose(g[n], t.grad.numpy(), atol=1e-11)


# ---------------------------------------------------------------- torch autograd (gather form)
def _torch_dense(q, k, v, aQ, aK, b, rows_nn, tau, allowed):
    raw = q @ k.transpose(-1, -2)
    H = q.shape[1]
    idx = rows_nn.expand(q.shape[0], H, -1, -1)
    if aQ is not None:
        tq = aQ if aQ.dim() == 3 else aQ.expand(H, -1, -1)
        raw = raw + torch.gather(q @ tq.transpose(-1, -2), 3, idx)
    if aK is not None:
        tk = aK if aK.dim() == 3 else aK.expand(H, -1, -1)
        ZK = k @ tk.transpose(-1, -2)                       # [B,H,N(j),R]
        raw = raw + torch.gather(ZK, 3, idx.transpose(-1, -2)).transpose(-1, -2)
    if b is not None:
        tb = b if b.dim() == 2 else b.expand(H, -1)
        raw = raw + tb[:, rows_nn[0, 0]][None]
    S = (tau * raw).masked_fill(~allowed, -math.inf)
    return torch.softmax(S, dim=-1) @ v


@pytest.mark.parametrize("phiname", ["shaw", "identity", "t5"])
@pytest.mark.parametrize("shared", [False, True])
def test_autograd_gather_formulation(phiname, shared):
    rng = np.random.default_rng(11)
    phi = PHIS[phiname]
    B, H, N, d = 2, 2, 150, 8
    x = _rand(rng, B, H, N, d, phi, shared=shared)
    tau = 0.4
    kl = np.array([N, 120])
    causal = phiname == "identity"
    g = oracle.backward(x["q"], x["k"], x["v"], x["aQ"], x["aK"], x["b"], dO=x["dO"], phi=phi,
                        tau=tau, causal=causal, key_len=kl, row_block=64)
    O, _ = oracle.forward(x["q"], x["k"], x["v"], x["aQ"], x["aK"], x["b"], phi=phi, tau=tau,
                          causal=causal, key_len=kl, row_block=64)
    rows = phi_rows(phi, N)
    ii = np.arange(N)[:, None]
    jj = np.arange(N)[None, :]
    rows_nn = torch.tensor(rows[jj - ii + N - 1])[None, None]
    allowed = torch.ones(B, 1, N, N, dtype=torch.bool)
    for bb in range(B):
        allowed[bb, :, :, int(kl[bb]):] = False
    if causal:
        allowed &= torch.ones(N, N, dtype=torch.bool).tril()
    T = {n: torch.tensor(x[n], requires_grad=True) for n in ("q", "k", "v", "aQ", "aK", "b")}
    out = _torch_dense(T["q"], T["k"], T["v"], T["aQ"], T["aK"], T["b"], rows_nn, tau, allowed)
    out.backward(torch.tensor(x["dO"]))
    np.testing.assert_allclose(O, out.detach().numpy(), atol=1e-12)
    for n, t in (("dq", "q"), ("dk", "k"), ("dv", "v"), ("daq", "aQ"), ("dak", "aK"), ("db", "b")):
        np.testing.assert_allclose(g[n], T[t].grad.numpy(), atol=1e-11, err_msg=n)


# ---------------------------------------------------------------- finite differences
@pytest.mark.parametrize("phiname,causal", [("shaw", False), ("t5", False), ("identity", True)])
def test_finite_differences(phiname, causal):
    rng = np.random.default_rng(5)
    phi = PHIS[phiname]
    B, H, N, d = 1, 2, 9, 3
    x = _rand(rng, B, H, N, d, phi)
    tau = 0.8
    kl = np.array([7])

    def loss(y):
        O, _ = oracle.forward(y["q"], y["k"], y["v"], y["aQ"], y["aK"], y["b"], phi=phi, tau=tau,
                              causal=causal, key_len=kl)
        return float(np.sum(O * x["dO"]))

    g = oracle.backward(x["q"], x["k"], x["v"], x["aQ"], x["aK"], x["b"], dO=x["dO"], phi=phi,
                        tau=tau, causal=causal, key_len=kl)
    h = 1e-6
    for name, gname in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("aQ", "daq"), ("aK", "dak"),
                        ("b", "db")):
        num = np.zeros_like(x[name])
        it = np.nditer(x[name], flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            y = {kk: (vv.copy() if isinstance(vv, np.ndarray) else vv) for kk, vv in x.items()}
            y[name][idx] += h
            fp = loss(y)
            y[name][idx] -= 2 * h
            fm = loss(y)
            num[idx] = (fp - fm) / (2 * h)
        np.testing.assert_allclose(g[gname], num, atol=2e-7, rtol=1e-6, err_msg=name)


# ---------------------------------------------------------------- invariants
def test_softmax_shift_invariants():
    rng = np.random.default_rng(9)
    phi = PHIS["shaw"]
    B, H, N, d = 1, 2, 40, 6
    x = _rand(rng, B, H, N, d, phi)
    args = dict(phi=phi, tau=0.7)
    O, _ = oracle.forward(x["q"], x["k"], x["v"], x["aQ"], x["aK"], x["b"], **args)
    g = oracle.backward(x["q"], x["k"], x["v"], x["aQ"], x["aK"], x["b"], dO=x["dO"], **args)
    b2 = x["b"] + 3.25
    aq2 = x["aQ"] + rng.standard_normal((H, 1, d))
    O2, _ = oracle.forward(x["q"], x["k"], x["v"], aq2, x["aK"], b2, **args)
    g2 = oracle.backward(x["q"], x["k"], x["v"], aq2, x["aK"], b2, dO=x["dO"], **args)
    np.testing.assert_allclose(O2, O, atol=1e-12)
    for n in ("dq", "dk", "dv", "db", "dak"):
        np.testing.assert_allclose(g2[n], g[n], atol=1e-11, err_msg=n)
    # rows of G sum to zero
    np.testing.assert_allclose(g["db"].sum(axis=-1), 0, atol=1e-12)
    np.testing.assert_allclose(g["daq"].sum(axis=1), 0, atol=1e-12)


def test_wide_truncation_equals_identity():
    rng = np.random.default_rng(4)
    N = 20
    x = _rand(rng, 1, 1, N, 4, PHIS["identity"])
    wide = {"kind": "truncated", "lo": -(N - 1), "hi": N - 1}
    a = oracle.forward(x["q"], x["k"], x["v"], x["aQ"], x["aK"], x["b"], phi=wide, tau=1.0)
    c = oracle.forward(x["q"], x["k"], x["v"], x["aQ"], x["aK"], x["b"], phi=PHIS["identity"],
                       tau=1.0)
    np.testing.assert_array_equal(a[0], c[0])


def test_causal_row_zero_and_padding_zeros():
    rng = np.random.default_rng(2)
    phi = PHIS["t5"]
    N = 30
    x = _rand(rng, 2, 2, N, 4, phi)
    kl = np.array([22, 30])
    O, _ = oracle.forward(x["q"], x["k"], x["v"], x["aQ"], x["aK"], x["b"], phi=phi, tau=1.0,
                          causal=True, key_len=kl)
    np.testing.assert_allclose(O[:, :, 0], x["v"][:, :, 0], atol=1e-14)
    g = oracle.backward(x["q"], x["k"], x["v"], x["aQ"], x["aK"], x["b"], dO=x["dO"], phi=phi,
                        tau=1.0, causal=True, key_len=kl)
    assert np.all(g["dq"][:, :, 0] == 0)
    assert np.all(g["dk"][0, :, 22:] == 0) and np.all(g["dv"][0, :, 22:] == 0)


def test_row_and_pair_sampling_match_full():
    rng = np.random.default_rng(8)
    phi = PHIS["shaw"]
    x = _rand(rng, 2, 2, 50, 4, phi)
    full = oracle.forward(x["q"], x["k"], x["v"], x["aQ"], x["aK"], x["b"], phi=phi, tau=0.5,
                          row_block=16)
    rows = np.array([0, 3, 17, 49])
    part = oracle.forward(x["q"], x["k"], x["v"], x["aQ"], x["aK"], x["b"], phi=phi, tau=0.5,
                          row_block=16, bh=[(1, 0)], query_rows=rows)
    np.testing.assert_allclose(part[0][1, 0, rows], full[0][1, 0, rows], atol=1e-14)
    gf = oracle.backward(x["q"], x["k"], x["v"], x["aQ"], x["aK"], x["b"], dO=x["dO"], phi=phi,
                         tau=0.5, row_block=16)
    gp = oracle.backward(x["q"], x["k"], x["v"], x["aQ"], x["aK"], x["b"], dO=x["dO"], phi=phi,
                         tau=0.5, row_block=16, bh=[(0, 1)], query_rows=rows)
    np.testing.assert_allclose(gp["dq"][0, 1, rows], gf["dq"][0, 1, rows], atol=1e-13)
