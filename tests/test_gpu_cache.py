"""Expert streaming from host memory (edge_moe_cache_*): a layer whose expert
tensors live in pinned host memory and reach HBM through an LRU of S slots per
group gives bitwise the output of the same layer with all E experts resident
(the persistent launch: the same up to the order of fp32 additions, for the
reason given at its case).

Each case runs a sequence of batches (different tokens, so different routing)
through one cache: route with the full layer, rename the experts to slots,
run the slot layer (G groups of S experts, the slot tensors in place of the
expert tensors), and compare y bit for bit with the resident layer.  S is
chosen from the batches so that every batch fits and experts are evicted
between batches; the eviction count is checked."""
import numpy as np
import pytest
import torch

import shared_matrix_expert_amd as em
import synth
from gpu_helpers import DEV, Layer, bits_to_dev, f32_to_dev, say

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)


def _slots_needed(idx_list, P):
    need = 1
    for idx in idx_list:
        ids = np.unique(idx.cpu().numpy())
        need = max(need, int(np.bincount(ids // P).max()))
    return need


def _run(cfg, T, batches, tiled, persistent=False, slack=0, predict=False, pinned=True):
    D = synth.config(cfg).dims.with_T(T)
    G, P = D.n_experts // D.experts_per_group, D.experts_per_group
    say(f"case: expert cache cfg {cfg} T={T} tiled={tiled} persistent={persistent} pinned={pinned}")
    wr, bias = synth.make_router(cfg, 0)
    lay = Layer(D, synth.make_weights(cfg, 0, device=DEV), tiled=tiled)
    wr, bias = bits_to_dev(wr), f32_to_dev(bias)
    routed = []
    for b in range(batches):
        xd = bits_to_dev(synth.make_activations(cfg, 100 + b, T=T))
        idx, w, _ = lay.route(xd, wr, bias, want_logits=False)
        routed.append((xd, idx, w))
    S = min(P, _slots_needed([r[1] for r in routed], P) + slack)
    say(f"  {S} slots per group of {P}")
    keys = [k for k in em.EXPERT_TENSOR_KEYS if lay.W.get(k) is not None]
    # pinned host memory takes the gather kernel, pageable memory hipMemcpyAsync
    host = {k: lay.W[k].cpu().pin_memory() if pinned else lay.W[k].cpu() for k in keys}
    slots = {k: torch.empty((G * S,) + tuple(lay.W[k].shape[1:]), dtype=lay.W[k].dtype, device=DEV)
             for k in keys}
    cache = em.ExpertCache(D, S, host, slots)
    SD = em.slot_dims(D, S)
    SW = em.slot_weights(lay.W, slots)
    ws = torch.empty(em.edge_moe_workspace_bytes(SD), dtype=torch.uint8, device=DEV)
    fwd = em.edge_moe_forward_persistent if persistent else em.edge_moe_forward
    side = torch.cuda.Stream()
    ready = torch.cuda.Event()
    rng = np.random.default_rng(3)
    for b, (xd, idx, w) in enumerate(routed):
        if persistent:
            y_ref = torch.empty(T, D.d, dtype=torch.float32, device=DEV)
            em.edge_moe_forward_persistent(D, xd, idx, w, lay.W, y_ref, lay.ws)
        else:
            y_ref, _ = lay.forward(xd, idx, w)
        idx_h = idx.cpu()
        slot_h = torch.empty_like(idx_h)
        torch.cuda.current_stream().wait_event(ready)      # a prediction's copies land first
        st = cache.map(idx_h, slot_h)
        sidx = slot_h.to(DEV)
        y = torch.empty(T, D.d, dtype=torch.float32, device=DEV)
        fwd(SD, xd, sidx, w, SW, y, ws)
        torch.cuda.synchronize()
        same = torch.equal(y.view(torch.int32), y_ref.view(torch.int32))
        dy = (y.double() - y_ref.double()).abs()
        ratio = float((dy / (1e-5 * (y_ref.double().abs() + y_ref.double().abs().max()))).max())
        say(f"  batch {b}: hits {st['hits']} misses {st['misses']} evictions {st['evictions']} "
            f"bitwise equal {same}, worst |dy| / fp32-order bound {ratio:.3g}")
        if persistent:
            # the persistent launch splits a 32-row pass's distinct experts over
            # two K halves by their rank in the pass, so the expert numbering
            # sets which fp32 partial a row's delta term joins: equal up to the
            # order of fp32 additions
            assert ratio <= 1.0, f"batch {b} differs from the resident layer beyond fp32 reordering"
        else:
            assert same, f"batch {b} differs from the resident layer"
        if predict and b + 1 < len(routed):
            # half of the next batch's experts and as many it does not use, copied
            # on a second stream after this batch's kernels
            nxt = np.unique(routed[b + 1][1].cpu().numpy())
            wrong = rng.choice(np.setdiff1d(np.arange(D.n_experts), nxt), size=len(nxt) // 2, replace=False)
            guess = torch.from_numpy(np.concatenate([nxt[::2], wrong]).astype(np.int32))
            ev = torch.cuda.Event()
            ev.record()
            side.wait_event(ev)
            cache.prefetch(guess, side)
            ready.record(side)
    tot = cache.totals()
    cache.close()
    return tot


def test_cache_verify_full_size_tiled():
    tot = _run(2, 8, batches=6, tiled=True)
    assert tot["evictions"] > 0


def test_cache_verify_full_size_with_predicted_copies():
    tot = _run(2, 8, batches=5, tiled=True, slack=8, predict=True)
    assert tot["evictions"] > 0 and tot["hits"] > 0


def test_cache_verify_full_size_persistent():
    tot = _run(2, 8, batches=4, tiled=True, persistent=True)
    assert tot["evictions"] > 0


def test_cache_decode_t1_row_major():
    tot = _run(1, 1, batches=8, tiled=False)
    assert tot["evictions"] > 0


def test_cache_decode_t1_pageable_host_memory():
    tot = _run(1, 1, batches=6, tiled=True, pinned=False)
    assert tot["evictions"] > 0


@pytest.mark.parametrize("T", [37, 72])
def test_cache_large_batch_full_size(T):
    # batches above the decode kernels' range: the permutation and tiled GEMM path
    tot = _run(1, T, batches=4, tiled=False)
    assert tot["misses"] > 0


def test_streamed_stack_equals_resident():
    # the benchmark's streamed decode stack (two full-size layers with the
    # residual between them, 8 slots per group, a new token per step): every
    # token's output, with and without next-layer prediction, bitwise equal to
    # the same stack with every expert resident
    import bench
    say("case: streamed two-layer decode stack against the resident stack")
    ss = bench.StreamStack(2, 8, n_tokens=16)
    assert ss.check(n_tokens=6)
    tot = [L["cache"].totals() for L in ss.layers]
    assert all(t["misses"] > 0 for t in tot)
    assert sum(t["evictions"] for t in tot) > 0
