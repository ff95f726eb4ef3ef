"""Host-side checks of the C ABI (no GPU needed, nothing is launched).

* the library loads and exports every function include/relpos_attn.h declares;
* descriptor validation returns the documented status before any launch;
* host-side map facts (R, unfolded thresholds) and buffer sizes match their
  closed forms.
"""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "relpos_attn.h")

b = pytest.importorskip("exact_relative_position_amd._binding")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(b.LIB_PATH):
        pytest.fail("librelpos_attn.so is not built; run __graft_entry__.build()")
    return b.lib()


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"\b(relpos_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert set(names) == set(b.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for code, name in b.STATUS.items():
        assert L.relpos_status_string(code).decode() == name


def _prob(B=1, H=2, N=256, d=64, dtype=1, tau=0.125):
    p = b.Problem()
    p.B, p.H, p.N, p.d, p.dtype, p.tau = B, H, N, d, dtype, tau
    for role in range(8):
        p.strides[role][0] = H * N * d
        p.strides[role][1] = N * d
        p.strides[role][2] = d
    p.aq_head_stride = 0
    p.ak_head_stride = 0
    p.b_head_stride = 0
    return p


def _ws(L, p, phi, mask=None, terms=1, pass_=0, zs=0):
    n = ctypes.c_size_t()
    m = mask or b.Mask()
    st = L.relpos_attn_workspace_size(ctypes.byref(p), ctypes.byref(phi), ctypes.byref(m), terms,
                                      pass_, zs, ctypes.byref(n))
    return st, n.value


def test_phi_info_closed_forms():
    assert b.phi_info({"kind": "truncated", "lo": -128, "hi": 128}, 8192) == (257, -128, 128)
    assert b.phi_info({"kind": "truncated", "lo": -256, "hi": 255}, 8192) == (512, -256, 255)
    assert b.phi_info({"kind": "identity"}, 4096) == (8191, -4095, 4095)
    # T5, 32 bidirectional buckets to 128: the last bucket starts at |o| = 91
    assert b.phi_info({"kind": "t5", "num_buckets": 32, "max_distance": 128,
                       "bidirectional": True}, 8192) == (32, -91, 91)
    R, lo, hi = b.phi_info({"kind": "t5", "num_buckets": 32, "max_distance": 128,
                            "bidirectional": False}, 100)
    assert (R, hi) == (32, 0) and lo < 0
    # log buckets 256 to 512 (hand-derived in tests/golden/log_bucket_points.txt):
    # 2 * 256 rows, the last row from o = 506 on, the first from o = -512 down
    assert b.phi_info({"kind": "log", "num_buckets": 256, "max_distance": 512}, 8192) == \
        (512, -512, 506)


@pytest.mark.parametrize("k,m", [(256, 512), (64, 300), (32, 40), (4, 5)])
def test_phi_info_log_matches_oracle(k, m):
    """The unfolded thresholds are where the oracle's rows reach their two
    constant runs."""
    import numpy as np
    from oracle import log_bucket
    n = np.arange(0, 2 * m + 2)
    pos = log_bucket(n, k, m)
    neg = log_bucket(-n, k, m)
    hi = int(np.argmax(pos == 2 * k - 1))
    lo = -int(np.argmax(neg == 0))
    assert b.phi_info({"kind": "log", "num_buckets": k, "max_distance": m}, 4096) == \
        (2 * k, lo, hi)


def test_zsave_size_closed_form(L):
    # Shaw 8K: B*H*N*Wp*4 bytes, window W = R = 257 (single group since
    # R <= N + 127), rows padded to Wp = 288 floats (a multiple of 128 bytes)
    p = _prob(B=1, H=12, N=8192)
    phi = b.phi_struct({"kind": "truncated", "lo": -128, "hi": 128})
    n = ctypes.c_size_t()
    assert L.relpos_attn_zsave_size(ctypes.byref(p), ctypes.byref(phi), 1, ctypes.byref(n)) == 0
    assert n.value == 12 * 8192 * 288 * 4
    # identity map: the window is N + G - 1 = N + 127 = 4223 columns per row,
    # padded to 4224
    p = _prob(B=2, H=8, N=4096, dtype=2)
    phi = b.phi_struct({"kind": "identity"})
    assert L.relpos_attn_zsave_size(ctypes.byref(p), ctypes.byref(phi), 1, ctypes.byref(n)) == 0
    assert n.value == 2 * 8 * 4096 * 4224 * 4
    # no vector table: nothing to keep
    assert L.relpos_attn_zsave_size(ctypes.byref(p), ctypes.byref(phi), 4, ctypes.byref(n)) == 0
    assert n.value == 0


def test_workspace_is_linear_in_n(L):
    phi = b.phi_struct({"kind": "truncated", "lo": -128, "hi": 128})
    sizes = []
    for N in (1024, 2048, 4096, 8192):
        st, n = _ws(L, _prob(H=12, N=N), phi, terms=1, pass_=1)
        assert st == 0
        sizes.append(n)
    for a, c in zip(sizes, sizes[1:]):
        assert 1.9 < c / a < 2.1


@pytest.mark.parametrize("field,value,code", [
    ("d", 128, -2), ("tau", 0.0, -1), ("tau", float("nan"), -1), ("dtype", 7, -1),
    ("N", -1, -1), ("N", (1 << 20) + 1, -2),
])
def test_bad_problem(L, field, value, code):
    p = _prob()
    setattr(p, field, value)
    phi = b.phi_struct({"kind": "truncated", "lo": -4, "hi": 4})
    st, _ = _ws(L, p, phi)
    assert st == code
    assert L.relpos_last_error().decode() != ""


@pytest.mark.parametrize("dtype,p,code", [
    (1, -0.1, -1), (1, 1.0, -1), (2, float("nan"), -1),
    (1, 0.999, -1),      # rounds to t = 256 of 256
    (0, 0.1, -2),        # dropout is implemented for 16-bit inputs only
    (0, 0.001, 0),       # rounds to t = 0: no dropout, fine for fp32
    (2, 0.1, 0), (1, 255 / 256, 0),
])
def test_dropout_probability(L, dtype, p, code):
    pr = _prob(dtype=dtype)
    pr.dropout_p = p
    pr.dropout_seed = 0xFFFFFFFFFFFFFFFF
    pr.dropout_offset = 0xFFFFFFFF
    phi = b.phi_struct({"kind": "truncated", "lo": -4, "hi": 4})
    assert _ws(L, pr, phi)[0] == code


def test_problem_struct_layout():
    # the dropout fields follow the table strides, 8-byte aligned seed last
    assert b.Problem.dropout_p.offset == b.Problem.b_head_stride.offset + 8
    assert b.Problem.dropout_offset.offset == b.Problem.dropout_p.offset + 4
    assert b.Problem.dropout_seed.offset == b.Problem.dropout_offset.offset + 4
    assert ctypes.sizeof(b.Problem) == b.Problem.dropout_seed.offset + 8


@pytest.mark.parametrize("phi", [
    {"kind": "truncated", "lo": 5, "hi": 4},
    {"kind": "t5", "num_buckets": 31, "max_distance": 128, "bidirectional": True},
    {"kind": "t5", "num_buckets": 32, "max_distance": 4, "bidirectional": True},
    {"kind": "t5", "num_buckets": 32, "max_distance": 128, "bidirectional": True,
     "max_exact": 16},
    {"kind": "log", "num_buckets": 255, "max_distance": 512},
    {"kind": "log", "num_buckets": 2, "max_distance": 512},
    {"kind": "log", "num_buckets": 256, "max_distance": 129},
])
def test_bad_phi(L, phi):
    st, _ = _ws(L, _prob(), b.phi_struct(phi))
    assert st == -1


def test_bad_phi_kind(L):
    phi = b.Phi()
    phi.kind = 9
    assert _ws(L, _prob(), phi)[0] == -1


def test_mask_validation(L):
    phi = b.phi_struct({"kind": "truncated", "lo": -4, "hi": 4})
    m = b.Mask()
    m.flags = 2  # key padding without key_len
    assert _ws(L, _prob(), phi, mask=m)[0] == -1
    m.flags = 8
    assert _ws(L, _prob(), phi, mask=m)[0] == -1


FAKE = 1 << 20  # aligned, never dereferenced: every call below fails validation first


def _fwd(L, p, phi, ptrs, ws=None, ws_bytes=0, zs=None, mask=None):
    m = mask or b.Mask()
    args = [ctypes.c_void_p(x) if x else None for x in ptrs]
    return L.relpos_attn_fwd(ctypes.byref(p), ctypes.byref(phi), ctypes.byref(m), *args,
                             ctypes.c_void_p(zs) if zs else None,
                             ctypes.c_void_p(ws) if ws else None, ws_bytes, None)


def test_fwd_validation_before_launch(L):
    phi = b.phi_struct({"kind": "truncated", "lo": -4, "hi": 4})
    p = _prob()
    good = [FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE]  # Q K V aQ aK b O lse
    bad_q = list(good)
    bad_q[0] = None
    assert _fwd(L, p, phi, bad_q) == -1
    mis = list(good)
    mis[1] = FAKE + 2
    assert _fwd(L, p, phi, mis) == -1
    assert "misaligned" in L.relpos_last_error().decode()
    # the projection needs workspace when no zsave buffer is given
    assert _fwd(L, p, phi, good) == -3
    p2 = _prob()
    p2.strides[0][2] = 60  # row stride not a multiple of 16 bytes
    assert _fwd(L, p2, phi, good) == -1
    p3 = _prob()
    p3.aq_head_stride = 3
    assert _fwd(L, p3, phi, good) == -1


def test_bwd_grad_presence_must_match(L):
    phi = b.phi_struct({"kind": "truncated", "lo": -4, "hi": 4})
    p = _prob()
    m = b.Mask()
    P = ctypes.c_void_p
    # aQ given, daQ missing
    st = L.relpos_attn_bwd(ctypes.byref(p), ctypes.byref(phi), ctypes.byref(m),
                           P(FAKE), P(FAKE), P(FAKE), P(FAKE), None, None, P(FAKE), P(FAKE),
                           P(FAKE), None, P(FAKE), P(FAKE), P(FAKE), None, None, None, None, 0,
                           None)
    assert st == -1
    # db given without b
    st = L.relpos_attn_bwd(ctypes.byref(p), ctypes.byref(phi), ctypes.byref(m),
                           P(FAKE), P(FAKE), P(FAKE), None, None, None, P(FAKE), P(FAKE),
                           P(FAKE), None, P(FAKE), P(FAKE), P(FAKE), None, None, P(FAKE), None,
                           0, None)
    assert st == -1
    # valid pointers but no workspace
    st = L.relpos_attn_bwd(ctypes.byref(p), ctypes.byref(phi), ctypes.byref(m),
                           P(FAKE), P(FAKE), P(FAKE), None, None, None, P(FAKE), P(FAKE),
                           P(FAKE), None, P(FAKE), P(FAKE), P(FAKE), None, None, None, None, 0,
                           None)
    assert st == -3


def test_python_descriptor_marshalling():
    import torch
    q = torch.empty(2, 10, 3, 64, dtype=torch.float16).transpose(1, 2)  # [B,H,N,d] view
    p = b.problem(q, 0.5, {b.T_Q: q})
    assert tuple(p.strides[0]) == (10 * 3 * 64, 64, 3 * 64)
    assert p.dtype == 1 and abs(p.tau - 0.5) < 1e-7
    s = b.phi_struct({"kind": "t5", "num_buckets": 32, "max_distance": 128,
                      "bidirectional": True})
    assert (s.kind, s.num_buckets, s.max_distance, s.bidirectional, s.max_exact) == \
        (1, 32, 128, 1, 0)
    aq = torch.empty(3, 9, 64, dtype=torch.float16)
    assert b._table_hs(aq, True) == 9 * 64
    assert b._table_hs(aq[0], True) == 0
