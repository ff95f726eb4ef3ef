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
    # padded to 4224, plus 32 floats of slack for the shifted rows of dZ^Q
    # (windows of 1024 columns or more)
    # (with the stored relation; the automatic choice computes the identity
    # map's relation in the block and keeps nothing)
    p = _prob(B=2, H=8, N=4096, dtype=2)
    phi = b.phi_struct({"kind": "identity"})
    assert L.relpos_attn_zsave_size(ctypes.byref(p), ctypes.byref(phi), 1, ctypes.byref(n)) == 0
    assert n.value == 0
    p.relation = 1
    assert L.relpos_attn_zsave_size(ctypes.byref(p), ctypes.byref(phi), 1, ctypes.byref(n)) == 0
    assert n.value == 2 * 8 * 4096 * 4256 * 4
    # no vector table: nothing to keep
    assert L.relpos_attn_zsave_size(ctypes.byref(p), ctypes.byref(phi), 4, ctypes.byref(n)) == 0
    assert n.value == 0


@pytest.mark.parametrize("phi,N,want", [
    # T5 saturates at |o| = 91: below N = 92 the unfolded map is every offset
    ({"kind": "t5", "num_buckets": 32, "max_distance": 128, "bidirectional": True}, 50,
     (32, -49, 49)),
    ({"kind": "t5", "num_buckets": 32, "max_distance": 128, "bidirectional": True}, 92,
     (32, -91, 91)),
    ({"kind": "t5", "num_buckets": 32, "max_distance": 1 << 24, "bidirectional": True}, 512,
     (32, -511, 511)),
    ({"kind": "t5", "num_buckets": 32, "max_distance": 128, "bidirectional": False}, 10,
     (32, -9, 0)),
    ({"kind": "log", "num_buckets": 256, "max_distance": 1 << 20}, 512, (512, -511, 511)),
    ({"kind": "log", "num_buckets": 256, "max_distance": 512}, 1, (512, 0, 0)),
])
def test_bucketed_unfold_is_clipped_to_reachable_offsets(phi, N, want):
    assert b.phi_info(phi, N) == want


def test_bucketed_workspace_grows_with_n_not_max_distance(L):
    """The unfolded tables, dZ and the contraction partials of a bucketed map
    are sized by the offsets that exist at this N: a huge max_distance costs
    nothing at N = 512."""
    p = _prob(B=1, H=12, N=512)
    sizes = []
    for m in (600, 1 << 20, 1 << 24):
        phi = b.phi_struct({"kind": "log", "num_buckets": 256, "max_distance": m})
        st, n = _ws(L, p, phi, terms=7, pass_=1)
        assert st == 0
        sizes.append(n)
    assert sizes[0] == sizes[1] == sizes[2]
    phi = b.phi_struct({"kind": "t5", "num_buckets": 32, "max_distance": 1 << 24,
                        "bidirectional": True})
    st, n = _ws(L, p, phi, terms=4, pass_=1)
    assert st == 0 and n < 64 << 20


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
    (1, 0.001, -1),      # rounds to t = 0: refused rather than silently no dropout
    (0, 1 / 512 - 1e-6, -1),
    (1, 1 / 512 + 1e-6, 0),  # rounds to t = 1
    (0, 0.0, 0),         # exactly 0: no dropout, fine for fp32
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
    assert b.Problem.zchunk.offset == b.Problem.dropout_seed.offset + 8
    assert b.Problem.relation.offset == b.Problem.zchunk.offset + 8
    assert ctypes.sizeof(b.Problem) == b.Problem.relation.offset + 8  # padded to 8 bytes


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


# Python-side validation: every tensor argument is checked before anything
# reaches the library (so a wrong dtype, shape or device can never hand the
# kernels a pointer they would misread).  CPU tensors with device_type="cpu"
# stand in for device tensors here.

def _inputs(B=2, H=3, N=40, dtype=None, phi=None):
    import torch
    dtype = dtype or torch.float16
    phi = phi or {"kind": "truncated", "lo": -4, "hi": 4}
    R = b.phi_info(phi, N)[0]
    t = lambda *s: torch.zeros(*s, dtype=dtype)  # noqa: E731
    return dict(q=t(B, H, N, 64), k=t(B, H, N, 64), v=t(B, H, N, 64), aq=t(H, R, 64),
                ak=t(R, 64), b=t(H, R), phi=phi, key_len=torch.full((B,), N, dtype=torch.int32))


def _check(x, **kw):
    b.check_inputs(x["q"], x["k"], x["v"], x["aq"], x["ak"], x["b"], phi=x["phi"],
                   key_len=x["key_len"], device_type="cpu", **kw)


def test_check_inputs_accepts_a_consistent_problem():
    _check(_inputs())
    x = _inputs(phi={"kind": "identity"})
    _check(x)
    x = _inputs(phi={"kind": "t5", "num_buckets": 32, "max_distance": 128,
                     "bidirectional": True})
    assert x["aq"].shape[1] == 32
    _check(x)


@pytest.mark.parametrize("mutate,match", [
    (lambda x, T: x.update(aq=x["aq"].float()), "aq has dtype"),        # fp32 table, fp16 q
    (lambda x, T: x.update(b=x["b"].to(T.bfloat16)), "b has dtype"),
    (lambda x, T: x.update(k=x["k"][:, :, :-1]), "k has shape"),
    (lambda x, T: x.update(v=x["v"].float()), "v has dtype"),
    (lambda x, T: x.update(aq=x["aq"][:, :-1]), "aq has 8 rows"),        # too few rows
    (lambda x, T: x.update(ak=T.zeros(17, 64, dtype=T.float16)), "ak has 17 rows"),
    (lambda x, T: x.update(aq=T.zeros(2, 9, 64, dtype=T.float16)), "aq must be"),  # H mismatch
    (lambda x, T: x.update(aq=T.zeros(3, 9, 32, dtype=T.float16)), "aq must be"),  # d mismatch
    (lambda x, T: x.update(b=T.zeros(3, 9, 1, dtype=T.float16)), "b must be"),
    (lambda x, T: x.update(key_len=x["key_len"].long()), "int32"),
    (lambda x, T: x.update(key_len=x["key_len"][:1]), "key_len must be a contiguous"),
    (lambda x, T: x.update(q=x["q"][0]), r"q must be a \[B, H, N, d\]"),
    (lambda x, T: x.update(q=x["q"].double(), k=x["k"].double(), v=x["v"].double()),
     "unsupported dtype"),
])
def test_check_inputs_rejects(mutate, match):
    import torch
    x = _inputs()
    mutate(x, torch)
    with pytest.raises((ValueError, TypeError), match=match):
        _check(x)


def test_identity_table_for_another_n_is_rejected():
    # an identity-map table built for N = 40 (79 rows) used at N = 41
    import torch
    x = _inputs(phi={"kind": "identity"})
    x["q"] = x["k"] = x["v"] = torch.zeros(2, 3, 41, 64, dtype=torch.float16)
    with pytest.raises(ValueError, match="aq has 79 rows"):
        _check(x)


def test_host_tensors_are_rejected_before_the_library():
    """The public entry points refuse host tensors: a host pointer handed to a
    kernel would fault the GPU."""
    import torch
    x = _inputs()
    with pytest.raises(ValueError, match="needs cuda tensors"):
        b.forward(x["q"], x["k"], x["v"], x["aq"], None, None, phi=x["phi"], tau=0.125)
    o = torch.zeros_like(x["q"])
    lse = torch.zeros(2, 3, 40)
    with pytest.raises(ValueError, match="needs cuda tensors"):
        b.backward(x["q"], x["k"], x["v"], None, None, None, o, lse, o, phi=x["phi"], tau=0.125)


def test_backward_checks_lse_and_saved_projections():
    import torch
    x = _inputs()
    lse = torch.zeros(2, 3, 40)
    with pytest.raises(ValueError, match="lse must be"):
        b._check_lse(lse.double(), x["q"])
    with pytest.raises(ValueError, match="lse must be"):
        b._check_lse(lse[:, :, :-1], x["q"])
    b._check_lse(lse, x["q"])
    with pytest.raises(ValueError, match="zsave must be"):
        b._check_zsave(torch.zeros(10, dtype=torch.uint8), x["q"], 11)
    b._check_zsave(torch.zeros(11, dtype=torch.uint8), x["q"], 11)


def test_noalloc_forward_validates_before_touching_the_device(L):
    """The allocation-free forward checks every argument, and that the
    forward fits its static scratch, before it looks up the scratch or
    launches anything (so these calls need no GPU)."""
    phi = b.phi_struct({"kind": "truncated", "lo": -128, "hi": 128})
    m = b.Mask()
    P = ctypes.c_void_p

    def call(p, q=FAKE, zs=None):
        return L.relpos_attn_fwd_noalloc(ctypes.byref(p), ctypes.byref(phi), ctypes.byref(m),
                                         P(q) if q else None, P(FAKE), P(FAKE), P(FAKE), None,
                                         None, P(FAKE), P(FAKE), P(zs) if zs else None, None)
    assert call(_prob(), q=None) == -1
    assert call(_prob(), q=FAKE + 4) == -1
    # 12 x 16384 rows of a 288-float window: 226 MB of projections, above the
    # 128 MiB scratch unless a zsave buffer takes them
    big = _prob(B=1, H=12, N=16384)
    assert call(big) == -3
    err = L.relpos_last_error().decode()
    assert "allocation-free limit" in err and str(b.NOALLOC_SCRATCH_BYTES) in err
    ws = ctypes.c_size_t()
    assert L.relpos_attn_workspace_size(ctypes.byref(big), ctypes.byref(phi), ctypes.byref(m), 1,
                                        0, 0, ctypes.byref(ws)) == 0
    assert ws.value > b.NOALLOC_SCRATCH_BYTES


# Chunked query-side projection (zchunk): validation and the memory model.

@pytest.mark.parametrize("zchunk,terms,code", [
    (100, 1, -1), (-128, 1, -1), (128, 3, -2),   # aK cannot be chunked
    (128, 1, 0), (128, 5, 0), (4096, 3, 0),       # zchunk >= N: no chunking, aK fine
])
def test_zchunk_validation(L, zchunk, terms, code):
    p = _prob(N=1000)
    p.zchunk = zchunk
    phi = b.phi_struct({"kind": "identity"})
    assert _ws(L, p, phi, terms=terms, pass_=1)[0] == code


def test_chunked_projection_is_never_kept(L):
    p = _prob(N=1000)
    p.zchunk = 256
    phi = b.phi_struct({"kind": "identity"})
    n = ctypes.c_size_t()
    assert L.relpos_attn_zsave_size(ctypes.byref(p), ctypes.byref(phi), 1, ctypes.byref(n)) == 0
    assert n.value == 0


def test_chunked_identity_workspace_is_linear_in_n(L):
    """With the identity map the projection window is N + 127 columns per
    query: unchunked, the backward workspace grows about 4x per doubling of
    N; with 1024-query chunks about 2x (the chunk's Z^Q and dZ^Q grow with
    the window only, the rest with N)."""
    phi = b.phi_struct({"kind": "identity"})
    sizes = {0: [], 1024: []}
    for zc in sizes:
        for N in (2048, 4096, 8192, 16384):
            p = _prob(H=12, N=N)
            p.zchunk = zc
            st, n = _ws(L, p, phi, terms=5, pass_=1)
            assert st == 0
            sizes[zc].append(n)
    for a, c in zip(sizes[0], sizes[0][1:]):
        assert 3.5 < c / a < 4.5
    for a, c in zip(sizes[1024], sizes[1024][1:]):
        assert 1.8 < c / a < 2.2
    # forward: only the chunk's Z^Q (rows of N + 127 columns padded to 128
    # bytes, plus 32 floats of row-shift slack)
    p = _prob(H=12, N=16384)
    p.zchunk = 1024
    st, n = _ws(L, p, phi, terms=5, pass_=0)
    assert st == 0 and n < 12 * 1024 * (16384 + 160) * 4 + (1 << 20)


# Relation mode (stored projection or in-block recompute): validation, the
# length rule of the automatic choice, and the memory it saves.

SHAW = {"kind": "truncated", "lo": -128, "hi": 128}


def _zsave(L, p, phi, terms):
    n = ctypes.c_size_t()
    st = L.relpos_attn_zsave_size(ctypes.byref(p), ctypes.byref(phi), terms, ctypes.byref(n))
    return st, n.value


@pytest.mark.parametrize("dtype,terms,zchunk,relation,code", [
    (1, 1, 0, 3, -1), (1, 1, 0, -1, -1),          # unknown modes
    (0, 1, 0, 2, -2),                             # fp32: not in the block
    (1, 3, 0, 2, -2),                             # aK present
    (1, 1, 128, 2, 0),                            # the backward is chunked, not the forward
    (1, 4, 0, 2, 0), (0, 4, 0, 2, 0),             # no aQ: nothing to compute, accepted
    (1, 5, 0, 2, 0), (2, 1, 0, 2, 0), (0, 1, 0, 1, 0), (0, 3, 0, 0, 0),
])
def test_relation_mode_validation(L, dtype, terms, zchunk, relation, code):
    p = _prob(N=1000, dtype=dtype)
    p.zchunk = zchunk
    p.relation = relation
    assert _ws(L, p, b.phi_struct(SHAW), terms=terms, pass_=0)[0] == code


@pytest.mark.parametrize("N,relation,inblock", [
    (128, 0, True), (257, 0, True), (258, 0, False), (8192, 0, False),  # 257 table rows
    (128, 1, False), (8192, 2, True),
])
def test_relation_mode_keeps_no_projection_in_block(L, N, relation, inblock):
    """In the block (chosen, or picked automatically where the relation window
    min(R, N + 127) is no narrower than the sequence, i.e. N <= R) the
    forward holds no projection: nothing to keep, and its workspace has no
    Z^Q.  The backward still projects Z^Q into its own workspace."""
    phi = b.phi_struct(SHAW)
    p = _prob(H=12, N=N)
    p.relation = relation
    st, nz = _zsave(L, p, phi, 1)
    assert st == 0
    st, nf = _ws(L, p, phi, terms=1, pass_=0)
    assert st == 0
    p.relation = 1
    _, nz_stored = _zsave(L, p, phi, 1)
    _, nf_stored = _ws(L, p, phi, terms=1, pass_=0)
    _, nb_stored = _ws(L, p, phi, terms=1, pass_=1)
    p.relation = relation
    _, nb = _ws(L, p, phi, terms=1, pass_=1)
    assert nb == nb_stored  # the backward is the same either way
    if inblock:
        assert nz == 0 and nf == 0
        assert nz_stored >= 12 * N * min(257, N + 127) * 4
    else:
        assert nz == nz_stored and nf == nf_stored


# Empty inputs: no token, or no batch entry, is a no-op that succeeds before
# any device call (null tensors are fine then); the backward with no table
# gradient to clear needs no device either.

@pytest.mark.parametrize("B,N", [(1, 0), (0, 256), (0, 0)])
def test_empty_problem_is_a_no_op(L, B, N):
    p = _prob(B=B, N=N)
    phi = b.phi_struct({"kind": "truncated", "lo": -16, "hi": 16})
    m = b.Mask()
    for relation in (0, 1, 2):
        p.relation = relation
        st, n = _ws(L, p, phi, terms=5, pass_=0)
        assert st == 0
        assert L.relpos_attn_fwd(ctypes.byref(p), ctypes.byref(phi), ctypes.byref(m), None,
                                 None, None, None, None, None, None, None, None, None, 0,
                                 None) == 0
    # backward without the contraction stage and without tables: nothing to do
    assert L.relpos_attn_bwd_stages(ctypes.byref(p), ctypes.byref(phi), ctypes.byref(m), None,
                                    None, None, None, None, None, None, None, None, None, None,
                                    None, None, None, None, None, None, 0, None,
                                    b.BWD_ALL & ~b.BWD_CONTRACT) == 0
