"""The allocation-free forward (relpos_attn_fwd_noalloc) against the
workspace forward (relpos_attn_fwd), through the C ABI: the same O and LSE
bit for bit, on two calls in a row whose second problem is smaller (the
static scratch keeps the first call's contents, which must not leak into
the second)."""

import math
import sys

import pytest
import torch

from parity_util import make_inputs, require_gpu
from relpos_synth import T5_32_128, Workload

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _both(w, keep_z):
    import exact_relative_position_amd._binding as B_
    dev = require_gpu()
    x = make_inputs(w)
    t = {k: (None if v is None else v.to(dev)) for k, v in x.items()}
    args = (t["q"], t["k"], t["v"], t["aq"], t["ak"], t["b"])
    kw = dict(phi=w.phi, tau=w.tau, causal=w.causal, key_len=t["key_len"])
    O_ref, lse_ref, zs_ref = B_.forward(*args, keep_z=keep_z, **kw)
    O = torch.full_like(t["q"], float("nan"))
    lse = torch.full(lse_ref.shape, float("nan"), dtype=torch.float32, device=dev)
    zs = None if zs_ref is None else torch.zeros_like(zs_ref)
    B_.forward_noalloc(*args, O=O, lse=lse, zsave=zs, **kw)
    torch.cuda.synchronize(dev)
    assert torch.equal(O, O_ref), "O"
    assert torch.equal(lse, lse_ref), "lse"
    if zs is not None:
        # the kept projections serve the backward exactly as the workspace
        # forward's do
        g_ref = B_.backward(*args, O_ref, lse_ref, t["do"], zs_ref, **kw)
        g = B_.backward(*args, O, lse, t["do"], zs, **kw)
        torch.cuda.synchronize(dev)
        for a, r in zip(g, g_ref):
            assert (a is None) == (r is None)
            if a is not None:
                assert torch.equal(a, r)
    return O.float().abs().max().item()


CASES = [
    # projections in the scratch (no zsave), then a smaller problem
    (Workload("noalloc_shaw_f16", 1, 4, 2048, 64, "f16", {"kind": "truncated", "lo": -128,
                                                          "hi": 128}, 1 / 8, has_aq=True),
     Workload("noalloc_shaw_small_f16", 1, 2, 1000, 64, "f16",
              {"kind": "truncated", "lo": -40, "hi": 31}, 1 / 8, has_aq=True, has_ak=True)),
    # bucketed map: fold table and unfolded bias in the scratch
    (Workload("noalloc_t5_bf16", 2, 3, 1500, 64, "bf16", T5_32_128, 1.0, has_b=True,
              key_padding=True),
     Workload("noalloc_t5_small_bf16", 1, 1, 300, 64, "bf16", T5_32_128, 1.0, has_b=True)),
    # identity map, causal, projections in the scratch
    (Workload("noalloc_txl_f16", 1, 2, 1024, 64, "f16", {"kind": "identity"}, 1 / 8,
              has_aq=True, has_b=True, causal=True, b_std=0.02),
     Workload("noalloc_txl_small_f16", 1, 1, 200, 64, "f16", {"kind": "identity"}, 1 / 8,
              has_aq=True, has_b=True, causal=True, b_std=0.02)),
]


@pytest.mark.parametrize("pair", CASES, ids=[c[0].name for c in CASES])
@pytest.mark.parametrize("keep_z", [False, True])
def test_noalloc_forward_matches_workspace_forward(pair, keep_z):
    for w in pair:
        _say(f"[gpu] noalloc {w.name} keep_z={keep_z}")
        assert math.isfinite(_both(w, keep_z))


def test_noalloc_rejects_a_forward_above_the_scratch():
    import exact_relative_position_amd._binding as B_
    dev = require_gpu()
    q = torch.zeros(1, 12, 16384, 64, dtype=torch.float16, device=dev)
    aq = torch.zeros(12, 257, 64, dtype=torch.float16, device=dev)
    O = torch.empty_like(q)
    lse = torch.empty(1, 12, 16384, dtype=torch.float32, device=dev)
    with pytest.raises(B_.RelposError, match="allocation-free limit"):
        B_.forward_noalloc(q, q, q, aq, phi={"kind": "truncated", "lo": -128, "hi": 128},
                           tau=0.125, O=O, lse=lse)
