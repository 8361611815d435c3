"""The next-layer prefetch (edge_moe_prefetch) is a pure performance hint:
layers run with it on a second stream give bitwise the outputs they give
without it, whatever the predicted groups (right, wrong, out of range)."""
import numpy as np
import pytest
import torch

import shared_matrix_expert_amd as em
import synth
from gpu_helpers import DEV, Layer, bits_to_dev, f32_to_dev, say

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)


def test_prefetch_leaves_results_unchanged():
    say("case: two full-size layers with and without the next-layer prefetch")
    D = synth.config(2).dims
    x = synth.make_activations(2, 0)
    layers = []
    for layer in (0, 1):
        wr, bias = synth.make_router(2, 0, layer)
        layers.append((Layer(D, synth.make_weights(2, 0, layer, device=DEV)), bits_to_dev(wr), f32_to_dev(bias)))
    side = torch.cuda.Stream()
    pws = torch.empty(em.edge_moe_prefetch_ws_bytes(), dtype=torch.uint8, device=DEV)
    G = D.n_experts // D.experts_per_group
    cases = {"none": None,
             "right": torch.arange(G, dtype=torch.int32, device=DEV),
             "wrong and out of range": torch.tensor([3, -1, G, 7, 7, 1000], dtype=torch.int32, device=DEV)}
    outs = {}
    for name, groups in cases.items():
        xd = bits_to_dev(x)
        ys = []
        for li, (lay, wr, bias) in enumerate(layers):
            if groups is not None and li == 0:
                ev = torch.cuda.Event()
                ev.record(torch.cuda.current_stream())
                side.wait_event(ev)
                em.edge_moe_prefetch(D, layers[1][0].W, groups, 3, pws, side)
            idx, w, _ = lay.route(xd, wr, bias, want_logits=False)
            y, _ = lay.forward(xd, idx, w)
            ys.append(y)
            nxt = torch.empty_like(xd)
            em.edge_moe_residual(xd, y, nxt)
            xd = nxt
        torch.cuda.synchronize()
        outs[name] = [y.cpu().numpy() for y in ys]
    for name in cases:
        for a, b in zip(outs[name], outs["none"]):
            assert np.array_equal(a, b), name
