"""Pins for the oracle's attention dropout (oracle/dropout.py and the
``dropout`` argument of oracle.forward / oracle.backward).

* the generator against the published Philox4x32-10 known-answer vectors
  (tests/golden/philox4x32_10_kat.txt);
* the counter layout and byte choice against a per-score statement of the
  reading (pure-Python scalar generator, one score at a time);
* keep rates within binomial bounds; t = 0 keeps every score and reproduces
  the no-dropout results exactly;
* brute force of the dropped forward (pure-Python loops);
* torch autograd of a dense formulation with an explicit keep mask, and
  central finite differences of sum(O * dO) with the mask held fixed;
* unbiasedness: averaged over many generator offsets, the dropped output
  approaches the undropped one.
"""

import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import phi_rows
from oracle.dropout import keep_mask, philox4x32_10, random_bytes

GOLD = os.path.join(os.path.dirname(__file__), "golden")
SHAW = {"kind": "truncated", "lo": -3, "hi": 2}


def _kat():
    rows = []
    with open(os.path.join(GOLD, "philox4x32_10_kat.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                w = [int(x, 16) for x in line.split()]
                rows.append((w[0:4], w[4:6], w[6:10]))
    return rows


def test_philox_known_answers():
    kat = _kat()
    assert len(kat) == 3
    for ctr, key, want in kat:
        got = philox4x32_10(np.array(ctr, dtype=np.uint64), key)
        assert [int(x) for x in got] == want


def _philox_scalar(c, k):
    # one call, Python integers (the round function as the SC 2011 paper states it)
    m0, m1, w0, w1, msk = 0xD2511F53, 0xCD9E8D57, 0x9E3779B9, 0xBB67AE85, 0xFFFFFFFF
    c = [int(v) for v in c]
    k0, k1 = (int(v) for v in k)
    for _ in range(10):
        a, b = m0 * c[0], m1 * c[2]
        c = [(b >> 32) ^ c[1] ^ k0, b & msk, (a >> 32) ^ c[3] ^ k1, a & msk]
        k0, k1 = (k0 + w0) & msk, (k1 + w1) & msk
    return c


def test_random_bytes_per_score():
    seed, offset, bh, N = 0x0123456789ABCDEF, 7, 5, 23
    rows = np.array([0, 1, 2, 3, 4, 9, 22])
    u = random_bytes(seed, offset, bh, rows, N)
    assert u.shape == (len(rows), N)
    for a, i in enumerate(rows):
        for j in range(N):
            x = _philox_scalar((j // 4, i // 4, bh, offset), (seed & 0xFFFFFFFF, seed >> 32))
            assert u[a, j] == (x[i % 4] >> (8 * (j % 4))) & 0xFF, (i, j)


@pytest.mark.parametrize("t", [0, 1, 26, 128, 255])
def test_keep_rate(t):
    N = 1024
    K = keep_mask((t, 42, 0, ), 3, np.arange(N), N)
    n = K.size
    p_keep = 1 - t / 256
    if t == 0:
        assert K.all()
        return
    sd = math.sqrt(n * p_keep * (1 - p_keep))
    assert abs(K.sum() - n * p_keep) < 6 * sd
    # different (batch, head) pairs and offsets draw different masks
    assert (K != keep_mask((t, 42, 0), 4, np.arange(N), N)).any()
    assert (K != keep_mask((t, 42, 1), 3, np.arange(N), N)).any()


def _rand(rng, B, H, N, d, R):
    return dict(q=rng.standard_normal((B, H, N, d)) * 0.7, k=rng.standard_normal((B, H, N, d)) * 0.7,
                v=rng.standard_normal((B, H, N, d)), aQ=rng.standard_normal((H, R, d)) * 0.5,
                aK=rng.standard_normal((H, R, d)) * 0.5, b=rng.standard_normal((H, R)),
                dO=rng.standard_normal((B, H, N, d)))


def test_threshold_zero_is_no_dropout():
    rng = np.random.default_rng(1)
    B, H, N, d = 2, 2, 37, 8
    x = _rand(rng, B, H, N, d, 6)
    kw = dict(phi=SHAW, tau=0.5, causal=True)
    args = (x["q"], x["k"], x["v"], x["aQ"], x["aK"], x["b"])
    O0, L0 = oracle.forward(*args, **kw)
    O1, L1 = oracle.forward(*args, **kw, dropout=(0, 99, 3))
    assert np.array_equal(O0, O1) and np.array_equal(L0, L1)
    g0 = oracle.backward(*args, dO=x["dO"], **kw)
    g1 = oracle.backward(*args, dO=x["dO"], **kw, dropout=(0, 99, 3))
    for n in g0:
        assert np.array_equal(g0[n], g1[n]), n


def test_brute_force_dropped_forward():
    rng = np.random.default_rng(2)
    B, H, N, d = 1, 2, 11, 4
    x = _rand(rng, B, H, N, d, 6)
    tau, drop = 0.6, (77, 2024, 5)
    O, L = oracle.forward(x["q"], x["k"], x["v"], x["aQ"], x["aK"], x["b"], phi=SHAW, tau=tau,
                          causal=True, dropout=drop)
    rows = phi_rows(SHAW, N)
    scale = 256.0 / (256 - drop[0])
    for h in range(H):
        for i in range(N):
            sc = []
            for j in range(i + 1):
                r = int(rows[j - i + N - 1])
                s = sum(x["q"][0, h, i, t] * (x["k"][0, h, j, t] + x["aQ"][h, r, t]) +
                        x["k"][0, h, j, t] * x["aK"][h, r, t] for t in range(d))
                sc.append(tau * (s + x["b"][h, r]))
            m = max(sc)
            w = [math.exp(s - m) for s in sc]
            tot = sum(w)
            assert L[0, h, i] == pytest.approx(m + math.log(tot), abs=1e-12)
            for t in range(d):
                acc = 0.0
                for j in range(i + 1):
                    xw = _philox_scalar((j // 4, i // 4, h, drop[2]), (drop[1], 0))
                    if (xw[i % 4] >> (8 * (j % 4))) & 0xFF >= drop[0]:
                        acc += w[j] / tot * scale * x["v"][0, h, j, t]
                assert O[0, h, i, t] == pytest.approx(acc, abs=1e-12)


def test_autograd_with_explicit_mask():
    rng = np.random.default_rng(3)
    B, H, N, d = 2, 2, 70, 8
    x = _rand(rng, B, H, N, d, 6)
    tau, drop = 0.45, (51, 7, 11)
    kl = np.array([N, 61])
    args = (x["q"], x["k"], x["v"], x["aQ"], x["aK"], x["b"])
    O, _ = oracle.forward(*args, phi=SHAW, tau=tau, key_len=kl, dropout=drop, row_block=32)
    g = oracle.backward(*args, dO=x["dO"], phi=SHAW, tau=tau, key_len=kl, dropout=drop,
                        row_block=32)
    rows = phi_rows(SHAW, N)
    ii, jj = np.arange(N)[:, None], np.arange(N)[None, :]
    r = torch.tensor(rows[jj - ii + N - 1])
    T = {n: torch.tensor(x[n], requires_grad=True) for n in ("q", "k", "v", "aQ", "aK", "b")}
    out = torch.zeros(B, H, N, d, dtype=torch.float64)
    outs = []
    for bb in range(B):
        for h in range(H):
            q, k = T["q"][bb, h], T["k"][bb, h]
            raw = q @ k.T + torch.gather(q @ T["aQ"][h].T, 1, r) + \
                torch.gather(k @ T["aK"][h].T, 1, r.T).T + T["b"][h][r]
            S = (tau * raw).masked_fill(torch.tensor(jj >= kl[bb]), -math.inf)
            K = torch.tensor(keep_mask(drop, bb * H + h, np.arange(N), N), dtype=torch.float64)
            outs.append((torch.softmax(S, -1) * K * (256 / (256 - drop[0]))) @ T["v"][bb, h])
    out = torch.stack(outs).reshape(B, H, N, d)
    out.backward(torch.tensor(x["dO"]))
    np.testing.assert_allclose(O, out.detach().numpy(), atol=1e-12)
    for n, t in (("dq", "q"), ("dk", "k"), ("dv", "v"), ("daq", "aQ"), ("dak", "aK"), ("db", "b")):
        np.testing.assert_allclose(g[n], T[t].grad.numpy(), atol=1e-11, err_msg=n)


def test_finite_differences_with_dropout():
    rng = np.random.default_rng(4)
    B, H, N, d = 1, 1, 10, 3
    x = _rand(rng, B, H, N, d, 6)
    tau, drop = 0.8, (90, 31337, 0)
    names = ("q", "k", "v", "aQ", "aK", "b")

    def loss(y):
        O, _ = oracle.forward(*(y[n] for n in names), phi=SHAW, tau=tau, dropout=drop)
        return float(np.sum(O * x["dO"]))

    g = oracle.backward(*(x[n] for n in names), dO=x["dO"], phi=SHAW, tau=tau, dropout=drop)
    h = 1e-6
    for name, gname in zip(names, ("dq", "dk", "dv", "daq", "dak", "db")):
        num = np.zeros_like(x[name])
        it = np.nditer(x[name], flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            y = {kk: vv.copy() for kk, vv in x.items()}
            y[name][idx] += h
            fp = loss(y)
            y[name][idx] -= 2 * h
            num[idx] = (fp - loss(y)) / (2 * h)
        np.testing.assert_allclose(g[gname], num, atol=2e-7, rtol=1e-6, err_msg=name)


def test_dropped_output_is_unbiased():
    rng = np.random.default_rng(5)
    B, H, N, d = 1, 1, 16, 4
    x = _rand(rng, B, H, N, d, 6)
    args = (x["q"], x["k"], x["v"], x["aQ"], None, None)
    O, _ = oracle.forward(*args, phi=SHAW, tau=0.7)
    n = 4000
    acc = np.zeros_like(O)
    for off in range(n):
        acc += oracle.forward(*args, phi=SHAW, tau=0.7, dropout=(64, 12345, off))[0]
    mean = acc / n
    # per entry: var(O_drop) <= (p / (1-p)) * sum_j P_ij^2 v_j^2 <= (1/3) max v^2
    bound = 6 * math.sqrt(np.max(x["v"] ** 2) / 3 / n)
    assert np.max(np.abs(mean - O)) < bound
    # a wrong keep scale (1 instead of 1/(1-p)) would sit far outside the bound
    assert np.max(np.abs(0.75 * mean - O)) > bound
