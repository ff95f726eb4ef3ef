"""Exact relative-position attention on MI355X (gfx950).

``relpos_attention`` is a drop-in attention with additive relative-position
terms (Eq. 1 of "Fast and Exact Relative-Position Attention via
Structure-Aware Kernels", nanless.github.io digest):

    S_ij = tau * (q_i.k_j + q_i.aQ[phi(i,j)] + k_j.aK[phi(i,j)] + b[phi(i,j)]) + M_ij
    O    = softmax(S) V

with phi a truncated (Shaw, DeBERTa), bucketed (T5 buckets, DeBERTa log
buckets) or identity (Transformer-XL) offset map.  Forward and backward run in the HIP library
``librelpos_attn.so`` (C ABI in include/relpos_attn.h); this package only
marshals arguments and lets PyTorch own device memory and streams.

phi is a dict: {"kind": "truncated", "lo": lo, "hi": hi},
{"kind": "t5", "num_buckets": 32, "max_distance": 128, "bidirectional": True},
{"kind": "log", "num_buckets": 256, "max_distance": 512} (2 * num_buckets
table rows), or {"kind": "identity"}.

Attention dropout (fp16 / bf16): ``dropout=(p, seed, offset)`` drops each
weight of P with probability p (rounded to a multiple of 1/256) and scales the
kept ones by 1 / (1 - p); the keep mask is a function of (seed, offset, batch,
head, query, key) only, recomputed by the backward.
"""

import torch

from . import _binding
from ._binding import RelposError, phi_info, phi_rows  # noqa: F401

__all__ = ["relpos_attention", "RelPosAttention", "forward", "backward", "phi_rows",
           "phi_info", "RelposError"]

forward = _binding.forward
backward = _binding.backward


class RelPosAttention(torch.autograd.Function):
    """Autograd wrapper: the forward keeps O, LSE and the relation projections."""

    @staticmethod
    def forward(ctx, q, k, v, aq, ak, b, phi, tau, causal, key_len, dropout=None, zchunk=0,
                relation=0):
        O, lse, zs = _binding.forward(q, k, v, aq, ak, b, phi=phi, tau=tau, causal=causal,
                                      key_len=key_len, keep_z=True, dropout=dropout,
                                      zchunk=zchunk, relation=relation)
        ctx.save_for_backward(q, k, v, aq, ak, b, O, lse, zs, key_len)
        ctx.cfg = (phi, tau, causal, dropout, zchunk, relation)
        return O

    @staticmethod
    def backward(ctx, dO):
        q, k, v, aq, ak, b, O, lse, zs, key_len = ctx.saved_tensors
        phi, tau, causal, dropout, zchunk, relation = ctx.cfg
        dq, dk, dv, daq, dak, db = _binding.backward(
            q, k, v, aq, ak, b, O, lse, dO.contiguous(), zs, phi=phi, tau=tau, causal=causal,
            key_len=key_len, dropout=dropout, zchunk=zchunk, relation=relation)
        cast = lambda g, t: None if g is None else g.to(t.dtype)  # noqa: E731
        return (dq, dk, dv, cast(daq, aq), cast(dak, ak), cast(db, b), None, None, None, None,
                None, None, None)


def relpos_attention(q, k, v, aq=None, ak=None, b=None, *, phi, tau, causal=False,
                     key_len=None, dropout=None, zchunk=0, relation=0):
    """Differentiable relative-position attention; q, k, v are [B, H, N, 64] on the GPU;
    ``dropout`` = (p, seed, offset) or None; ``zchunk`` > 0 (a multiple of 128)
    recomputes the query-side projection one chunk of queries at a time in both
    passes, so that memory stays linear in N for the identity map; ``relation``
    (0 auto, 1 stored, 2 in-block) says how the forward gets the query-side
    relation term (in-block: recomputed inside each attention block, nothing
    stored; the backward projects it)."""
    return RelPosAttention.apply(q, k, v, aq, ak, b, phi, tau, causal, key_len, dropout, zchunk,
                                 relation)
