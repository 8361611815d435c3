"""The allocation-free forward (edge_moe_forward_noalloc): its output equals
edge_moe_forward's with a caller workspace, bitwise, on two calls in a row
(the second with a smaller batch, so that stale contents of the shared scratch
would show), and it rejects dims whose workspace exceeds the scratch."""
import ctypes

import numpy as np
import pytest
import torch

import shared_matrix_expert_amd as em
import synth
from gpu_helpers import Layer, bits_to_dev, f32_to_dev, say

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)


def _noalloc(D, x, idx, w, W, y):
    lib = em.load()
    cw = em.cweights(W)
    return lib.edge_moe_forward_noalloc(ctypes.byref(em.cdims(D)), em._ptr(x), em._ptr(idx), em._ptr(w),
                                        ctypes.byref(cw), em._ptr(y), em._stream(None))


@pytest.mark.parametrize("cfg", [2, 0])
def test_noalloc_matches_forward_twice(cfg):
    base = synth.config(cfg).dims
    W = synth.make_weights(cfg, 1, device="cuda")
    for T in (base.T, max(1, base.T // 4)):
        say(f"case: no-alloc forward cfg={cfg} T={T}")
        D = base.with_T(T)
        x = synth.make_activations(cfg, 1, T=T)
        wr, bias = synth.make_router(cfg, 1)
        lay = Layer(D, W)
        xd = bits_to_dev(x)
        idx, w, _ = lay.route(xd, bits_to_dev(wr), f32_to_dev(bias if T == base.T else None))
        y_ref, _ = lay.forward(xd, idx, w)
        y = torch.full((D.T, D.d), float("nan"), dtype=torch.float32, device="cuda")
        st = _noalloc(D, xd, idx, w, lay.W, y)
        assert st == em.EDGE_MOE_OK, em.status_string(st)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), "no-alloc output differs from edge_moe_forward"


def test_noalloc_rejects_large_workspace():
    D = synth.config(3).dims                    # 16K tokens: far beyond the scratch
    st = em.load().edge_moe_forward_noalloc(ctypes.byref(em.cdims(D)), 0x10000, 0x20000, 0x30000,
                                            ctypes.byref(em.CWeights(*([0x50000] * 20))), 0x40000, None)
    assert st == em.EDGE_MOE_EWORKSPACE
