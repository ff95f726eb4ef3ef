"""Seeded synthetic inputs for relative-position attention.

This module holds no arithmetic of the method: it only draws random numbers,
rounds them to a storage dtype and names the workloads.  Both the CPU oracle
(via the tests) and the HIP path take their inputs from here.

Draw order (one ``numpy.random.default_rng(seed)`` stream, float64 standard
normals, each scaled by its standard deviation): Q, K, V, aQ, aK, b (each only
if present), then U (one uniform per batch, key padding only), then dO.
Every tensor is then rounded to the workload dtype with torch ``.to(dtype)``
(round to nearest even); the rounded tensors are the exact inputs both sides
see.

Workloads are the layer-benchmark shapes (12 heads, head dim 64, 8K tokens,
FP16) of the setup section of "Fast and Exact Relative-Position Attention via
Structure-Aware Kernels" (nanless.github.io digest), one per mechanism, plus
small parity shapes.  The pages use no dataset for this benchmark; these
seeded inputs are the whole input.
"""

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str                  # "f32" | "f16" | "bf16"
    phi: dict                   # oracle/ABI-neutral phi descriptor (see oracle.phi)
    tau: float
    has_aq: bool = False
    has_ak: bool = False
    has_b: bool = False
    causal: bool = False
    key_padding: bool = False   # key_len[b] = N - floor(U * pad_frac * N)
    pad_frac: float = 0.1
    qkv_std: Optional[float] = None   # default 1/sqrt(d)
    aq_std: float = 0.1
    ak_std: float = 0.1
    b_std: float = 1.0
    do_std: float = 1.0
    shared_tables: bool = False       # one table for all heads
    seed: int = 0
    # attention dropout: (t, generator seed, generator offset), drop
    # probability t / 256; None = no dropout
    dropout: Optional[tuple] = None
    # query rows per chunk of the query-side projection (0: the whole
    # sequence); a run setting, not an input
    zchunk: int = 0
    # how the forward gets the query-side relation: 0 by sequence length,
    # 1 stored projection, 2 in the block; a run setting, not an input
    relation: int = 0

    def with_(self, **kw):
        return dataclasses.replace(self, **kw)


def rows_for(phi, N):
    """Number of table rows R (plain data bookkeeping; identical to the map's row count)."""
    kind = phi["kind"]
    if kind == "truncated":
        return phi["hi"] - phi["lo"] + 1
    if kind == "identity":
        return 2 * N - 1
    if kind == "t5":
        return phi["num_buckets"]
    if kind == "log":
        return 2 * phi["num_buckets"]
    raise ValueError(kind)


SHAW16 = {"kind": "truncated", "lo": -16, "hi": 16}
SHAW128 = {"kind": "truncated", "lo": -128, "hi": 128}
DEBERTA256 = {"kind": "truncated", "lo": -256, "hi": 255}
T5_32_128 = {"kind": "t5", "num_buckets": 32, "max_distance": 128, "bidirectional": True,
             "max_exact": 8}
IDENTITY = {"kind": "identity"}
# DeBERTa's own map on the pages: 256 log buckets to distance 512 (2 * 256 rows)
DEBERTA_LOG = {"kind": "log", "num_buckets": 256, "max_distance": 512}

WORKLOADS = {
    # Shaw truncation +-16, 1x1x256x64, fp32, aQ only, seed 0.
    "shaw_n256_f32": Workload("shaw_n256_f32", 1, 1, 256, 64, "f32", SHAW16, 1 / 8, has_aq=True),
    # Shaw truncation +-128, 1x12x8192x64, fp16, aQ only.
    "shaw_n8192_f16": Workload("shaw_n8192_f16", 1, 12, 8192, 64, "f16", SHAW128, 1 / 8,
                               has_aq=True),
    # DeBERTa-style content-to-position and position-to-content, clip(-256, 255).
    "deberta_n8192_f16": Workload("deberta_n8192_f16", 1, 12, 8192, 64, "f16", DEBERTA256,
                                  1 / math.sqrt(192), has_aq=True, has_ak=True),
    # The same with DeBERTa's log-bucket map (256 buckets to distance 512).
    "deberta_log_n8192_f16": Workload("deberta_log_n8192_f16", 1, 12, 8192, 64, "f16",
                                      DEBERTA_LOG, 1 / math.sqrt(192), has_aq=True,
                                      has_ak=True),
    # T5 32 bidirectional buckets to distance 128, scalar bias, key padding.
    "t5_n8192_f16": Workload("t5_n8192_f16", 1, 12, 8192, 64, "f16", T5_32_128, 1.0,
                             has_b=True, key_padding=True, b_std=1.0),
    # Transformer-XL identity map, speech-encoder shape, bf16, causal.
    "txl_n4096_bf16": Workload("txl_n4096_bf16", 2, 8, 4096, 64, "bf16", IDENTITY, 1 / 8,
                               has_aq=True, has_b=True, causal=True, b_std=0.02),
    # Transformer-XL identity map at the 8K layer-benchmark shape (parity only).
    "txl_n8192_f16": Workload("txl_n8192_f16", 1, 12, 8192, 64, "f16", IDENTITY, 1 / 8,
                              has_aq=True, has_b=True, causal=True, b_std=0.02),
}


# The layer benchmark's length sweep (same setup section): a budget of 16384
# tokens per batch, N from 128 to 8192 (B = 16384 / N), 12 heads, head dim
# 64, FP16, bidirectional attention; each mechanism with its map and terms
# as in the workloads above, without masks, and DeBERTa with the pages'
# log-bucket map.
SWEEP_NS = (128, 256, 512, 1024, 2048, 4096, 8192)
SWEEP_TOKENS = 16384


def sweep_workloads():
    """Name -> Workload for every (mechanism, N) point of the sweep."""
    mechs = {
        "shaw": dict(phi=SHAW128, tau=1 / 8, has_aq=True),
        "txl": dict(phi=IDENTITY, tau=1 / 8, has_aq=True, has_b=True, b_std=0.02),
        "deberta": dict(phi=DEBERTA_LOG, tau=1 / math.sqrt(192), has_aq=True, has_ak=True),
        "t5": dict(phi=T5_32_128, tau=1.0, has_b=True, b_std=1.0),
    }
    out = {}
    for m, kw in mechs.items():
        for N in SWEEP_NS:
            name = f"{m}_sweep_n{N}"
            out[name] = Workload(name, SWEEP_TOKENS // N, 12, N, 64, "f16", **kw)
    return out


# Memory scaling in N at a fixed batch (the Shaw workload, 1 x 12 x N, fp16):
# the method keeps O(N d + N R) bytes per sequence, so the extra memory should
# about double per doubling of N.
MEMORY_NS = (1024, 2048, 4096, 8192, 16384)


def memory_scaling_workloads(mechanism="shaw"):
    """Name -> Workload at each N of MEMORY_NS: the Shaw workload (1 x 12 x N,
    fp16), or the Transformer-XL identity map at the same shape (fp16,
    causal, aQ + b) with its projection computed 1024 queries at a time."""
    if mechanism == "txl":
        base = WORKLOADS["txl_n8192_f16"].with_(zchunk=1024)
        return {f"txl_n{N}_f16_chunk1024": base.with_(name=f"txl_n{N}_f16_chunk1024", N=N)
                for N in MEMORY_NS}
    base = WORKLOADS["shaw_n8192_f16"]
    return {f"shaw_n{N}_f16": base.with_(name=f"shaw_n{N}_f16", N=N) for N in MEMORY_NS}


def make_inputs(w: Workload):
    """Return a dict of CPU torch tensors in the workload dtype (tables too).

    Keys: q, k, v, do, aq, ak, b (None when absent), key_len (int32 [B] or None).
    """
    rng = np.random.default_rng(w.seed)
    dt = DTYPES[w.dtype]
    B, H, N, d = w.B, w.H, w.N, w.d
    R = rows_for(w.phi, N)
    std = (1.0 / math.sqrt(d)) if w.qkv_std is None else w.qkv_std
    tH = () if w.shared_tables else (H,)

    def draw(shape, s):
        return torch.from_numpy(rng.standard_normal(shape) * s).to(dt)

    out = {}
    out["q"] = draw((B, H, N, d), std)
    out["k"] = draw((B, H, N, d), std)
    out["v"] = draw((B, H, N, d), std)
    out["aq"] = draw(tH + (R, d), w.aq_std) if w.has_aq else None
    out["ak"] = draw(tH + (R, d), w.ak_std) if w.has_ak else None
    out["b"] = draw(tH + (R,), w.b_std) if w.has_b else None
    if w.key_padding:
        U = rng.random(B)
        kl = N - np.floor(U * w.pad_frac * N).astype(np.int64)
        out["key_len"] = torch.from_numpy(kl.astype(np.int32))
    else:
        out["key_len"] = None
    out["do"] = draw((B, H, N, d), w.do_std)
    return out


def as_f64(t):
    """Exact float64 numpy copy of a (rounded) tensor, or None."""
    return None if t is None else t.to(torch.float64).numpy()
