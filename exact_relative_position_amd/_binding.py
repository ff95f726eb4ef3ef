"""ctypes binding of librelpos_attn.so (declared in include/relpos_attn.h).

Argument marshalling only: every step of the computation runs in the HIP
library.  PyTorch supplies device memory (outputs, workspace, the saved
projections) and the current stream.  If the library is missing or fails to
load, every entry point raises; there is no fallback path.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librelpos_attn.so")

RELPOS_OK = 0
STATUS = {0: "RELPOS_OK", -1: "RELPOS_ERR_INVALID_ARG", -2: "RELPOS_ERR_UNSUPPORTED",
          -3: "RELPOS_ERR_WORKSPACE", -4: "RELPOS_ERR_HIP"}
DTYPE = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
PHI_KIND = {"truncated": 0, "t5": 1, "identity": 2, "log": 3}
MASK_CAUSAL, MASK_KEY_PADDING = 1, 2
TERM_AQ, TERM_AK, TERM_B = 1, 2, 4
PASS_FWD, PASS_BWD = 0, 1
REL_AUTO, REL_STORED, REL_INBLOCK = 0, 1, 2
T_Q, T_K, T_V, T_O, T_DO, T_DQ, T_DK, T_DV = range(8)

EXPORTS = ("relpos_attn_workspace_size", "relpos_attn_zsave_size", "relpos_attn_fwd",
           "relpos_attn_bwd", "relpos_attn_fwd_stages", "relpos_attn_bwd_stages",
           "relpos_attn_fwd_noalloc", "relpos_phi_info", "relpos_phi_rows",
           "relpos_status_string", "relpos_last_error")
NOALLOC_SCRATCH_BYTES = 128 << 20
FWD_PROJECT, FWD_ATTEND, FWD_ALL = 1, 2, 3
BWD_PREPARE, BWD_QUERY_PASS, BWD_KEY_PASS, BWD_CONTRACT, BWD_ALL = 1, 2, 4, 8, 15


class Phi(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("lo", ctypes.c_int32), ("hi", ctypes.c_int32),
                ("num_buckets", ctypes.c_int32), ("max_exact", ctypes.c_int32),
                ("max_distance", ctypes.c_int32), ("bidirectional", ctypes.c_int32)]


class Mask(ctypes.Structure):
    _fields_ = [("flags", ctypes.c_int32), ("key_len", ctypes.c_void_p)]


class Problem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("H", ctypes.c_int64), ("N", ctypes.c_int64),
                ("d", ctypes.c_int64), ("dtype", ctypes.c_int32), ("tau", ctypes.c_float),
                ("strides", (ctypes.c_int64 * 3) * 8), ("aq_head_stride", ctypes.c_int64),
                ("ak_head_stride", ctypes.c_int64), ("b_head_stride", ctypes.c_int64),
                ("dropout_p", ctypes.c_float), ("dropout_offset", ctypes.c_uint32),
                ("dropout_seed", ctypes.c_uint64), ("zchunk", ctypes.c_int64),
                ("relation", ctypes.c_int32)]


class RelposError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


_lib = None


def lib():
    """Load the library once; raise if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built (run __graft_entry__.build() or "
                               "python exact_relative_position_amd/build.py)")
        L = ctypes.CDLL(LIB_PATH)
        P, V, I32, I64, SZ = (ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                              ctypes.c_size_t)
        pp, pphi, pm = ctypes.POINTER(Problem), ctypes.POINTER(Phi), ctypes.POINTER(Mask)
        L.relpos_attn_workspace_size.argtypes = [pp, pphi, pm, I32, I32, I32,
                                                 ctypes.POINTER(SZ)]
        L.relpos_attn_zsave_size.argtypes = [pp, pphi, I32, ctypes.POINTER(SZ)]
        L.relpos_attn_fwd.argtypes = [pp, pphi, pm, P, P, P, P, P, P, P, P, P, P, SZ, V]
        L.relpos_attn_bwd.argtypes = [pp, pphi, pm, P, P, P, P, P, P, P, P, P, P,
                                      P, P, P, P, P, P, P, SZ, V]
        L.relpos_attn_fwd_stages.argtypes = L.relpos_attn_fwd.argtypes + [I32]
        L.relpos_attn_bwd_stages.argtypes = L.relpos_attn_bwd.argtypes + [I32]
        L.relpos_attn_fwd_noalloc.argtypes = [pp, pphi, pm, P, P, P, P, P, P, P, P, P, V]
        L.relpos_phi_info.argtypes = [pphi, I64, ctypes.POINTER(I64), ctypes.POINTER(I64),
                                      ctypes.POINTER(I64)]
        L.relpos_phi_rows.argtypes = [pphi, I64, P, P, V]
        for fn in ("relpos_attn_workspace_size", "relpos_attn_zsave_size", "relpos_attn_fwd",
                   "relpos_attn_bwd", "relpos_attn_fwd_stages", "relpos_attn_bwd_stages",
                   "relpos_attn_fwd_noalloc", "relpos_phi_info", "relpos_phi_rows"):
            getattr(L, fn).restype = I32
        L.relpos_status_string.argtypes = [I32]
        L.relpos_status_string.restype = ctypes.c_char_p
        L.relpos_last_error.argtypes = []
        L.relpos_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(status):
    if status != RELPOS_OK:
        raise RelposError(status, lib().relpos_last_error().decode())


def phi_struct(phi):
    """C descriptor of a phi dict ({"kind": "truncated"|"t5"|"identity"|"log", ...})."""
    kind = phi["kind"]
    s = Phi()
    s.kind = PHI_KIND[kind]
    if kind == "truncated":
        s.lo, s.hi = int(phi["lo"]), int(phi["hi"])
    elif kind == "t5":
        s.num_buckets = int(phi["num_buckets"])
        s.max_exact = int(phi.get("max_exact") or 0)
        s.max_distance = int(phi["max_distance"])
        s.bidirectional = 1 if phi.get("bidirectional", True) else 0
    elif kind == "log":
        s.num_buckets = int(phi["num_buckets"])
        s.max_distance = int(phi["max_distance"])
    return s


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _strides(t):
    if t.stride(-1) != 1:
        raise ValueError("the head dimension must be contiguous")
    return (t.stride(0), t.stride(1), t.stride(2))


def _table_hs(t, vec):
    if t is None:
        return 0
    shared = t.dim() == (2 if vec else 1)
    if vec and t.stride(-1) != 1 or (vec and t.stride(-2) != t.shape[-1]):
        raise ValueError("table rows must be contiguous")
    if not vec and t.stride(-1) != 1:
        raise ValueError("bias table must be contiguous along rows")
    return 0 if shared else t.stride(0)


def _same(t, q, name, shape=None):
    """``t`` on q's device with q's dtype and ``shape`` (q's shape by default)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device != q.device:
        raise ValueError(f"{name} is on {t.device}, q on {q.device}")
    if t.dtype != q.dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, q has {q.dtype} (tables and tensors "
                         "share one element type)")
    want = tuple(q.shape) if shape is None else tuple(shape)
    if tuple(t.shape) != want:
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {want}")


def check_inputs(q, k, v, aq, ak, b, *, phi, key_len=None, tensors=(), device_type="cuda"):
    """Validate every tensor argument before anything reaches the library.

    q, k, v (and the extra [B, H, N, d] ``tensors``, as (name, tensor) pairs)
    must share q's device, dtype and shape; q must be on a ``device_type``
    device with a dtype the library knows.  A vector table is [H, R, d] or,
    shared by all heads, [R, d]; the bias is [H, R] or [R]; R is the row count
    of ``phi`` at this N.  ``key_len`` is an int32 [B] tensor on q's device.
    Raises TypeError / ValueError naming the offending argument."""
    if not isinstance(q, torch.Tensor) or q.dim() != 4:
        raise ValueError("q must be a [B, H, N, d] tensor")
    if q.device.type != device_type:
        raise ValueError(f"q is on {q.device}; the library needs {device_type} tensors")
    if q.dtype not in DTYPE:
        raise ValueError(f"unsupported dtype {q.dtype} (float32, float16 or bfloat16)")
    B, H, N, d = q.shape
    for name, t in (("k", k), ("v", v)) + tuple(tensors):
        _same(t, q, name)
    R = phi_info(phi, N)[0] if N > 0 else None
    for name, t, vec in (("aq", aq, True), ("ak", ak, True), ("b", b, False)):
        if t is None:
            continue
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a tensor or None")
        full, shared = (3, 2) if vec else (2, 1)
        if t.dim() not in (full, shared) or (vec and t.shape[-1] != d) or \
                (t.dim() == full and t.shape[0] != H):
            raise ValueError(f"{name} must be [H, R{', d' if vec else ''}] or "
                             f"[R{', d' if vec else ''}] with H = {H}, d = {d}; "
                             f"got {tuple(t.shape)}")
        _same(t, q, name, t.shape)
        rows = t.shape[-2] if vec else t.shape[-1]
        if R is not None and rows != R:
            raise ValueError(f"{name} has {rows} rows; the map {phi.get('kind')} has R = {R} "
                             f"at N = {N}")
    if key_len is not None:
        if not isinstance(key_len, torch.Tensor):
            raise TypeError("key_len must be a tensor or None")
        if key_len.device != q.device:
            raise ValueError(f"key_len is on {key_len.device}, q on {q.device}")
        if key_len.dtype != torch.int32:
            raise ValueError(f"key_len must be int32, got {key_len.dtype}")
        if tuple(key_len.shape) != (B,) or not key_len.is_contiguous():
            raise ValueError(f"key_len must be a contiguous [B] = [{B}] tensor, "
                             f"got {tuple(key_len.shape)}")


def _check_lse(lse, q):
    B, H, N, _ = q.shape
    if not isinstance(lse, torch.Tensor) or lse.device != q.device or \
            lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, N) or \
            not lse.is_contiguous():
        raise ValueError(f"lse must be a contiguous float32 [B, H, N] = [{B}, {H}, {N}] tensor "
                         f"on {q.device}")


def _check_zsave(zsave, q, nbytes):
    if zsave is None:
        return
    if not isinstance(zsave, torch.Tensor) or zsave.device != q.device or \
            not zsave.is_contiguous() or zsave.numel() * zsave.element_size() < nbytes:
        raise ValueError(f"zsave must be a contiguous tensor on {q.device} of at least "
                         f"{nbytes} bytes (the forward's saved projections)")


def problem(q, tau, tensors, aq=None, ak=None, b=None, dropout=None, zchunk=0, relation=0):
    """Problem descriptor; ``tensors`` maps a role index to its [B,H,N,d] tensor;
    ``dropout`` = (p, seed, offset) or None; ``zchunk`` = query rows per chunk
    of the projection (0: the whole sequence); ``relation`` = REL_AUTO,
    REL_STORED or REL_INBLOCK (how the forward gets the query-side term)."""
    B, H, N, d = q.shape
    p = Problem()
    p.B, p.H, p.N, p.d = B, H, N, d
    p.dtype = DTYPE[q.dtype]
    p.tau = float(tau)
    for role, t in tensors.items():
        for i, s in enumerate(_strides(t)):
            p.strides[role][i] = s
    p.aq_head_stride = _table_hs(aq, True)
    p.ak_head_stride = _table_hs(ak, True)
    p.b_head_stride = _table_hs(b, False)
    if dropout is not None:
        p.dropout_p = float(dropout[0])
        p.dropout_seed = int(dropout[1]) & 0xFFFFFFFFFFFFFFFF
        p.dropout_offset = int(dropout[2]) & 0xFFFFFFFF
    p.zchunk = int(zchunk)
    p.relation = int(relation)
    return p


def mask_struct(causal, key_len):
    m = Mask()
    m.flags = (MASK_CAUSAL if causal else 0) | (MASK_KEY_PADDING if key_len is not None else 0)
    m.key_len = None if key_len is None else key_len.data_ptr()
    return m


def _terms(aq, ak, b):
    return (TERM_AQ if aq is not None else 0) | (TERM_AK if ak is not None else 0) | \
           (TERM_B if b is not None else 0)


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _workspace(nbytes, dev):
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=dev)


def zsave_size(prob, phi_s, terms):
    n = ctypes.c_size_t()
    _check(lib().relpos_attn_zsave_size(ctypes.byref(prob), ctypes.byref(phi_s), terms,
                                        ctypes.byref(n)))
    return n.value


def workspace_size(prob, phi_s, mask_s, terms, pass_, zsave_given):
    n = ctypes.c_size_t()
    _check(lib().relpos_attn_workspace_size(ctypes.byref(prob), ctypes.byref(phi_s),
                                            ctypes.byref(mask_s), terms, pass_,
                                            1 if zsave_given else 0, ctypes.byref(n)))
    return n.value


def phi_info(phi, N):
    R, lo, hi = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    s = phi_struct(phi)
    _check(lib().relpos_phi_info(ctypes.byref(s), int(N), ctypes.byref(R), ctypes.byref(lo),
                                 ctypes.byref(hi)))
    return R.value, lo.value, hi.value


def phi_rows(phi, N, device="cuda"):
    """Device-computed row table (int32[2N-1]) and unfold table (int32[R_unf])."""
    R, lo, hi = phi_info(phi, N)
    rows = torch.empty(2 * N - 1, dtype=torch.int32, device=device)
    fold = torch.empty(hi - lo + 1, dtype=torch.int32, device=device)
    s = phi_struct(phi)
    _check(lib().relpos_phi_rows(ctypes.byref(s), int(N), _ptr(rows), _ptr(fold),
                                 _stream(rows.device)))
    return rows, fold


def forward(q, k, v, aq=None, ak=None, b=None, *, phi, tau, causal=False, key_len=None,
            keep_z=True, out=None, dropout=None, zchunk=0, relation=REL_AUTO):
    """O, LSE (and the saved projections, or None) of the relative-position
    attention; ``dropout`` = (p, seed, offset) or None; ``zchunk`` > 0 computes
    the projection one chunk of queries at a time (nothing is kept)."""
    check_inputs(q, k, v, aq, ak, b, phi=phi, key_len=key_len,
                 tensors=(() if out is None else (("out", out),)))
    dev = q.device
    O = torch.empty_like(q) if out is None else out
    B, H, N, _ = q.shape
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    prob = problem(q, tau, {T_Q: q, T_K: k, T_V: v, T_O: O}, aq, ak, b, dropout, zchunk, relation)
    phi_s = phi_struct(phi)
    mask_s = mask_struct(causal, key_len)
    terms = _terms(aq, ak, b)
    zs = None
    if keep_z and (aq is not None or ak is not None):
        nz = zsave_size(prob, phi_s, terms)
        zs = _workspace(nz, dev) if nz > 0 else None
    ws = _workspace(workspace_size(prob, phi_s, mask_s, terms, PASS_FWD, zs is not None), dev)
    _check(lib().relpos_attn_fwd(ctypes.byref(prob), ctypes.byref(phi_s), ctypes.byref(mask_s),
                                 _ptr(q), _ptr(k), _ptr(v), _ptr(aq), _ptr(ak), _ptr(b),
                                 _ptr(O), _ptr(lse), _ptr(zs), _ptr(ws), ws.numel(),
                                 _stream(dev)))
    return O, lse, zs


def forward_noalloc(q, k, v, aq=None, ak=None, b=None, *, phi, tau, O, lse, zsave=None,
                    causal=False, key_len=None, dropout=None, zchunk=0, relation=REL_AUTO):
    """relpos_attn_fwd_noalloc: the forward into caller-given O and LSE (and
    zsave, or None), with the library's static scratch instead of a
    workspace; allocates nothing."""
    check_inputs(q, k, v, aq, ak, b, phi=phi, key_len=key_len, tensors=(("O", O),))
    _check_lse(lse, q)
    prob = problem(q, tau, {T_Q: q, T_K: k, T_V: v, T_O: O}, aq, ak, b, dropout, zchunk, relation)
    phi_s = phi_struct(phi)
    mask_s = mask_struct(causal, key_len)
    _check_zsave(zsave, q, zsave_size(prob, phi_s, _terms(aq, ak, b)))
    _check(lib().relpos_attn_fwd_noalloc(ctypes.byref(prob), ctypes.byref(phi_s),
                                         ctypes.byref(mask_s), _ptr(q), _ptr(k), _ptr(v),
                                         _ptr(aq), _ptr(ak), _ptr(b), _ptr(O), _ptr(lse),
                                         _ptr(zsave), _stream(q.device)))


def backward(q, k, v, aq, ak, b, o, lse, do, zsave=None, *, phi, tau, causal=False,
             key_len=None, dropout=None, zchunk=0, relation=REL_AUTO):
    """dQ, dK, dV (input dtype) and daQ, daK, db (fp32, shape of their table, or None)."""
    check_inputs(q, k, v, aq, ak, b, phi=phi, key_len=key_len, tensors=(("o", o), ("do", do)))
    _check_lse(lse, q)
    dev = q.device
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    daq = None if aq is None else torch.empty(aq.shape, dtype=torch.float32, device=dev)
    dak = None if ak is None else torch.empty(ak.shape, dtype=torch.float32, device=dev)
    db = None if b is None else torch.empty(b.shape, dtype=torch.float32, device=dev)
    prob = problem(q, tau, {T_Q: q, T_K: k, T_V: v, T_O: o, T_DO: do, T_DQ: dq, T_DK: dk,
                            T_DV: dv}, aq, ak, b, dropout, zchunk, relation)
    phi_s = phi_struct(phi)
    mask_s = mask_struct(causal, key_len)
    terms = _terms(aq, ak, b)
    _check_zsave(zsave, q, zsave_size(prob, phi_s, terms))
    ws = _workspace(workspace_size(prob, phi_s, mask_s, terms, PASS_BWD, zsave is not None), dev)
    _check(lib().relpos_attn_bwd(ctypes.byref(prob), ctypes.byref(phi_s), ctypes.byref(mask_s),
                                 _ptr(q), _ptr(k), _ptr(v), _ptr(aq), _ptr(ak), _ptr(b),
                                 _ptr(o), _ptr(lse), _ptr(do), _ptr(zsave),
                                 _ptr(dq), _ptr(dk), _ptr(dv), _ptr(daq), _ptr(dak), _ptr(db),
                                 _ptr(ws), ws.numel(), _stream(dev)))
    return dq, dk, dv, daq, dak, db


class Prepared:
    """One problem with every output, the saved projections and both
    workspaces allocated up front, so that ``fwd()``/``bwd()`` only enqueue
    library calls (nothing is allocated in between)."""

    def __init__(self, q, k, v, aq, ak, b, do, *, phi, tau, causal=False, key_len=None,
                 keep_z=True, dropout=None, zchunk=0, relation=REL_AUTO):
        check_inputs(q, k, v, aq, ak, b, phi=phi, key_len=key_len, tensors=(("do", do),))
        dev = q.device
        self.dev = dev
        self.q, self.k, self.v, self.aq, self.ak, self.b, self.do = q, k, v, aq, ak, b, do
        self.key_len = key_len
        B, H, N, _ = q.shape
        self.O = torch.empty_like(q)
        self.lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
        self.dq, self.dk, self.dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        f32 = dict(dtype=torch.float32, device=dev)
        self.daq = None if aq is None else torch.empty(aq.shape, **f32)
        self.dak = None if ak is None else torch.empty(ak.shape, **f32)
        self.db = None if b is None else torch.empty(b.shape, **f32)
        self.prob = problem(q, tau, {T_Q: q, T_K: k, T_V: v, T_O: self.O, T_DO: do, T_DQ: self.dq,
                                     T_DK: self.dk, T_DV: self.dv}, aq, ak, b, dropout, zchunk, relation)
        self.phi_s = phi_struct(phi)
        self.mask_s = mask_struct(causal, key_len)
        terms = _terms(aq, ak, b)
        self.zs = None
        if keep_z and (aq is not None or ak is not None):
            nz = zsave_size(self.prob, self.phi_s, terms)
            self.zs = _workspace(nz, dev) if nz > 0 else None
        zg = self.zs is not None
        self.ws_f = _workspace(workspace_size(self.prob, self.phi_s, self.mask_s, terms,
                                              PASS_FWD, zg), dev)
        self.ws_b = _workspace(workspace_size(self.prob, self.phi_s, self.mask_s, terms,
                                              PASS_BWD, zg), dev)
        self.stream = _stream(dev)
        P = _ptr
        self._fargs = (ctypes.byref(self.prob), ctypes.byref(self.phi_s),
                       ctypes.byref(self.mask_s), P(q), P(k), P(v), P(aq), P(ak), P(b),
                       P(self.O), P(self.lse), P(self.zs), P(self.ws_f), self.ws_f.numel(),
                       self.stream)
        self._bargs = (ctypes.byref(self.prob), ctypes.byref(self.phi_s),
                       ctypes.byref(self.mask_s), P(q), P(k), P(v), P(aq), P(ak), P(b),
                       P(self.O), P(self.lse), P(do), P(self.zs), P(self.dq), P(self.dk),
                       P(self.dv), P(self.daq), P(self.dak), P(self.db), P(self.ws_b),
                       self.ws_b.numel(), self.stream)

    def fwd(self, stages=FWD_ALL):
        _check(lib().relpos_attn_fwd_stages(*self._fargs, stages))

    def bwd(self, stages=BWD_ALL):
        _check(lib().relpos_attn_bwd_stages(*self._bargs, stages))

    def extra_bytes(self):
        """Device bytes this call owns beyond its inputs and outputs."""
        n = self.ws_f.numel() + self.ws_b.numel()
        return n + (0 if self.zs is None else self.zs.numel())
