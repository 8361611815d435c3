"""GPU parity: the HIP library (through its C-ABI) against the float64 oracle.

Gates: expert indices and their order bit-exact; routing weights |dw| <= 1e-6;
logits bitwise (both sides round the exact dot product once); layer output
|dy| <= 2e-3 + 2e-3 |y_ref| on every element; repeated runs bitwise equal.
"""
import numpy as np
import pytest
import torch

import shared_matrix_expert_amd as em
import synth
from oracle.layer import moe_forward, residual, route
from gpu_helpers import (DEV, Layer, bits_to_dev, expected_permutation, f32_to_dev, say, tile_cover_sample,
                         y_within_tolerance)

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

GPU_TINY = synth.Dims(T=5, d=128, h=256, n_experts=16, experts_per_group=4, top_k=3,
                      delta_rank=8, lora_rank=2, quant_group=32)


def _inputs(cfg, seed, layer=0, T=None):
    x = synth.make_activations(cfg, seed, T=T, layer=layer)
    wr, bias = synth.make_router(cfg, seed, layer)
    return x, wr, bias


def _check_route(D, x, wr, bias, lay, sample=None):
    idx, w, lg = lay.route(bits_to_dev(x), bits_to_dev(wr), f32_to_dev(bias))
    torch.cuda.synchronize()
    rows = np.arange(D.T) if sample is None else sample
    ref = route(x[rows], wr, bias, D.top_k)
    g_idx = idx.cpu().numpy()[rows]
    g_w = w.cpu().numpy()[rows]
    g_lg = lg.cpu().numpy()[rows]
    assert np.array_equal(g_lg.astype(np.float64), ref["logits"]), "logits differ"
    assert np.array_equal(g_idx, ref["idx"]), "expert indices differ"
    assert np.max(np.abs(g_w - ref["w"])) <= 1e-6
    return idx, w, ref


def _run_parity(D, x, wr, bias, Wdev, sample=None, keep=False, tiled=None, persistent=False):
    lay = Layer(D, Wdev, tiled=tiled, persistent=persistent)
    idx, w, ref = _check_route(D, x, wr, bias, lay, sample)
    y, tr = lay.forward(bits_to_dev(x), idx, w, trace=keep)
    torch.cuda.synchronize()
    rows = np.arange(D.T) if sample is None else sample
    Wh = synth.weights_to_numpy(Wdev)
    fw = moe_forward(x[rows], ref["idx"], ref["w"], Wh, D.experts_per_group, keep=keep)
    ok, ratio = y_within_tolerance(y.cpu().numpy()[rows], fw["y"])
    say(f"  worst |dy| / bound = {ratio:.3g}")
    assert ok, f"y outside tolerance (worst ratio {ratio:.3g})"
    return lay, idx, w, y, tr, fw


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tiny_layer(seed):
    say(f"case: tiny C0 seed={seed}")
    D = synth.config(0).dims
    x, wr, bias = _inputs(0, seed)
    W = synth.make_weights(0, seed, device="cuda")
    _run_parity(D, x, wr, bias, W)


def test_tiny_multi_group_layer():
    say("case: tiny multi-group")
    D = GPU_TINY
    rng = np.random.default_rng(11)
    x = synth.bf16_bits_from_f32(rng.standard_normal((D.T, D.d), dtype=np.float32))
    wr = synth.bf16_bits_from_f32(rng.standard_normal((D.n_experts, D.d), dtype=np.float32) * np.float32(0.1))
    from helpers import random_weights
    Wh = random_weights(D, 3)
    Wdev = {k: torch.from_numpy(v.view(np.int16) if v.dtype == np.uint16 else v).to("cuda")
            for k, v in Wh.items()}
    _run_parity(D, x, wr, None, Wdev)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_decode_layer(seed):
    say(f"case: decode C1 seed={seed}")
    D = synth.config(1).dims
    x, wr, bias = _inputs(1, seed)
    _run_parity(D, x, wr, bias, synth.make_weights(1, seed, device="cuda"))


def _check_trace(D, idx, tr, fw):
    # permutation bit-exact against a numpy lexsort
    offs, rt, rs = expected_permutation(idx.cpu().numpy(), D.n_experts)
    assert np.array_equal(tr["expert_offsets"].cpu().numpy(), offs)
    assert np.array_equal(tr["row_token"].cpu().numpy(), rt)
    assert np.array_equal(tr["row_slot"].cpu().numpy(), rs)
    # activations: a bf16 value differs from the oracle's where the fp32 pre-activation
    # landed on the other side of a rounding midpoint (one bf16 step, 2^-7 |a|) or
    # where a low-rank input (R1 / R2) rounded the other way, which shifts that
    # row's pre-activations by at most |B_up| * one bf16 step of z (~2e-3); both
    # are rare
    act = tr["act"].cpu().numpy().view(np.uint16)               # slot order
    a_gpu = (act.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ref_a = fw["a"].reshape(-1, D.h)
    dev = np.abs(a_gpu - ref_a)
    assert np.all(dev <= 2.0 ** -7 * np.abs(ref_a) + 4e-3), float(np.max(dev))
    assert np.mean(a_gpu != ref_a) < 5e-3, float(np.mean(a_gpu != ref_a))
    # expert outputs per slot: a sanity bound (the gate is on y, where the k slots
    # are averaged); a low-rank input rounded the other way moves a slot's o by ~1e-3
    o_gpu = tr["expert_out"].cpu().numpy().astype(np.float64)
    o_ref = fw["o"].reshape(-1, D.d)
    assert np.all(np.abs(o_gpu - o_ref) <= 1e-2 + 1e-2 * np.abs(o_ref)), float(np.max(np.abs(o_gpu - o_ref)))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_verify_skewed_layer(seed):
    say(f"case: verify C2 seed={seed}")
    D = synth.config(2).dims
    x, wr, bias = _inputs(2, seed)
    lay, idx, w, y, tr, fw = _run_parity(D, x, wr, bias, synth.make_weights(2, seed, device="cuda"),
                                         keep=True)
    _check_trace(D, idx, tr, fw)
    # determinism
    y2, _ = lay.forward(bits_to_dev(x), idx, w)
    assert torch.equal(y, y2)


@pytest.mark.parametrize("cfg,seed", [(1, 0), (1, 2), (2, 0), (2, 2)])
def test_persistent_layer(cfg, seed):
    """The single persistent launch (edge_moe_forward_persistent) on the decode
    and verify batches, traced: permutation, activations and expert outputs
    per slot, y, and bitwise equal repeats."""
    say(f"case: persistent layer cfg={cfg} seed={seed}")
    D = synth.config(cfg).dims
    x, wr, bias = _inputs(cfg, seed)
    lay, idx, w, y, tr, fw = _run_parity(D, x, wr, bias, synth.make_weights(cfg, seed, device="cuda"),
                                         keep=True, persistent=True)
    _check_trace(D, idx, tr, fw)
    y2, _ = lay.forward(bits_to_dev(x), idx, w)
    assert torch.equal(y, y2)


@pytest.mark.parametrize("T", [2, 5])
def test_persistent_ragged(T):
    say(f"case: persistent layer, ragged T={T}")
    D = synth.config(1).dims.with_T(T)
    x = synth.make_activations(1, 6, T=T)
    wr, _ = synth.make_router(1, 6)
    _run_parity(D, x, wr, None, synth.make_weights(1, 6, device="cuda"), persistent=True)


def test_persistent_unsupported_shapes():
    """Shapes outside the persistent launch's limits are refused before anything runs."""
    D = synth.config(2).dims.with_T(12)                       # more than 8 tokens
    lay = Layer(D, synth.make_weights(2, 0, device="cuda"), persistent=True)
    x = bits_to_dev(synth.make_activations(2, 0, T=12))
    idx = torch.zeros(D.T, D.top_k, dtype=torch.int32, device=DEV)
    w = torch.zeros(D.T, D.top_k, dtype=torch.float32, device=DEV)
    with pytest.raises(em.EdgeMoeError) as ei:
        lay.forward(x, idx, w)
    assert ei.value.status == em.EDGE_MOE_EUNSUPPORTED
    D8 = synth.config(2).dims
    lay = Layer(D8, synth.make_weights(2, 0, device="cuda"), tiled=False, persistent=True)
    x = bits_to_dev(synth.make_activations(2, 0))
    with pytest.raises(em.EdgeMoeError) as ei:                 # no stored copies
        lay.forward(x, idx[:8], w[:8])
    assert ei.value.status == em.EDGE_MOE_EUNSUPPORTED


def test_verify_row_major_weights():
    """The verify batch with the row-major shared matrices only (no tiled copies)."""
    say("case: verify C2 seed=1, row-major shared matrices")
    D = synth.config(2).dims
    x, wr, bias = _inputs(2, 1)
    lay, idx, w, y, tr, fw = _run_parity(D, x, wr, bias, synth.make_weights(2, 1, device="cuda"),
                                         keep=True, tiled=False)
    _check_trace(D, idx, tr, fw)


def _tiled_reference(q: np.ndarray):
    """The decode-tiled layout written out from its definition: q [M][N][K/2]
    bytes -> the tiled bytes."""
    M, N, KB = q.shape
    K = 2 * KB
    out = np.empty(M * N * KB, dtype=np.uint8)
    for g in range(M):
        for n in range(N // 128):
            for b in range(K // 256):
                for t in range(8):
                    for c in range(2):
                        for l in range(64):
                            i, j = l % 16, l // 16
                            row = 128 * n + 16 * t + i
                            src = q[g, row, (2 * b + c) * 64 + 16 * j:(2 * b + c) * 64 + 16 * j + 16]
                            off = g * N * KB + n * 64 * K + b * 16384 + t * 2048 + c * 1024 + l * 16
                            out[off:off + 16] = src
    return out


def test_tile_shared_layout():
    """edge_moe_tile_shared against its definition, byte for byte, on random codes
    (the shared up and down and A_up sets)."""
    say("case: decode-tiled layout")
    D = synth.Dims(T=1, d=1024, h=1024, n_experts=16, experts_per_group=8, top_k=4,
                   delta_rank=128, lora_rank=4, quant_group=128)
    rng = np.random.default_rng(11)
    G = D.n_experts // D.experts_per_group
    for which, (M, N, K) in ((0, (G, D.h, D.d)), (1, (G, D.d, D.h)), (2, (D.n_experts, D.delta_rank, D.d))):
        q = rng.integers(0, 256, (M, N, K // 2), dtype=np.uint8)
        qd = torch.from_numpy(q).to("cuda")
        dq = torch.empty_like(qd)
        em.edge_moe_tile_shared(D, which, qd, dq)
        torch.cuda.synchronize()
        assert np.array_equal(dq.cpu().numpy().reshape(-1), _tiled_reference(q))


def test_colblock_layout():
    """The column-blocked A_dn copy (edge_moe_tile_shared kind 3) against its
    definition, byte for byte, on random codes: for expert e and block cb of
    128 columns, the rows' 64-byte segments in row order."""
    say("case: column-blocked a_dn layout")
    D = synth.Dims(T=1, d=1024, h=1024, n_experts=4, experts_per_group=4, top_k=2,
                   delta_rank=128, lora_rank=4, quant_group=128)
    rng = np.random.default_rng(12)
    q = rng.integers(0, 256, (D.n_experts, D.delta_rank, D.h // 2), dtype=np.uint8)
    qd = torch.from_numpy(q).to("cuda")
    dq = torch.empty_like(qd)
    em.edge_moe_tile_shared(D, 3, qd, dq)
    torch.cuda.synchronize()
    ref = q.reshape(D.n_experts, D.delta_rank, D.h // 128, 64).transpose(0, 2, 1, 3).reshape(-1)
    assert np.array_equal(dq.cpu().numpy().reshape(-1), ref)


def test_prefill_layer_tile_cover():
    """The 16K-token prefill at full size: the whole permutation (163,840 slots)
    against a numpy lexsort, and logits, indices and y against the oracle on
    >= 1024 tokens chosen so that every 128-row tile of every prefill GEMM
    (shared up, shared down, the rank-128 inputs of every expert) holds a
    checked row."""
    say("case: prefill C3 seed=0, tile-covering token sample")
    D = synth.config(3).dims
    x, wr, bias = _inputs(3, 0)
    Wdev = synth.make_weights(3, 0, device="cuda")
    lay = Layer(D, Wdev)
    xd = bits_to_dev(x)
    idx, w, lg = lay.route(xd, bits_to_dev(wr), f32_to_dev(bias))
    R = D.T * D.top_k
    tr = {"expert_offsets": torch.empty(D.n_experts + 1, dtype=torch.int32, device=DEV),
          "row_token": torch.empty(R, dtype=torch.int32, device=DEV),
          "row_slot": torch.empty(R, dtype=torch.int32, device=DEV)}
    y = torch.empty(D.T, D.d, dtype=torch.float32, device=DEV)
    em.edge_moe_forward(D, xd, idx, w, lay.W, y, lay.ws, trace=tr)
    torch.cuda.synchronize()
    idx_h = idx.cpu().numpy()
    offs, rt, rs = expected_permutation(idx_h, D.n_experts)
    assert np.array_equal(tr["expert_offsets"].cpu().numpy(), offs), "expert offsets differ"
    assert np.array_equal(tr["row_token"].cpu().numpy(), rt), "row tokens differ"
    assert np.array_equal(tr["row_slot"].cpu().numpy(), rs), "row slots differ"
    sample, n_cover, n_tiles = tile_cover_sample(offs, rt, D.experts_per_group, D.n_groups, D.T, 1024)
    say(f"  {n_cover} tokens cover {n_tiles} row tiles; {sample.size} tokens checked")
    ref = route(x[sample], wr, bias, D.top_k)
    assert np.array_equal(lg.cpu().numpy()[sample].astype(np.float64), ref["logits"]), "logits differ"
    assert np.array_equal(idx_h[sample], ref["idx"]), "expert indices differ"
    assert np.max(np.abs(w.cpu().numpy()[sample] - ref["w"])) <= 1e-6
    fw = moe_forward(x[sample], ref["idx"], ref["w"], synth.weights_to_numpy(Wdev), D.experts_per_group)
    ok, ratio = y_within_tolerance(y.cpu().numpy()[sample], fw["y"])
    say(f"  worst |dy| / bound = {ratio:.3g}")
    assert ok, f"y outside tolerance (worst ratio {ratio:.3g})"
    y2, _ = lay.forward(xd, idx, w)
    assert torch.equal(y, y2)


def test_general_fallback_traced():
    """A batch above the decode limit at shapes the LDS-tiled prefill GEMMs do
    not take (quant groups of 32, r = 8): every stage on the general GEMM, with
    the permutation, activations and expert outputs checked."""
    say("case: general fallback GEMMs, C0 shapes at T=100, traced")
    D = synth.config(0).dims.with_T(100)
    x = synth.make_activations(0, 4, T=100)
    wr, _ = synth.make_router(0, 4)
    lay, idx, w, y, tr, fw = _run_parity(D, x, wr, None, synth.make_weights(0, 4, device="cuda"), keep=True)
    _check_trace(D, idx, tr, fw)
    y2, _ = lay.forward(bits_to_dev(x), idx, w)
    assert torch.equal(y, y2)


def test_verify_delta_handoff():
    """A verify batch routed by hand so that two groups carry 32 and 24 rows
    (the 32- and 24-row staged passes) and the six others 1-8 rows each: the
    hot groups hand their delta down to three light groups' workgroups each,
    and the combine adds it back (the trace's expert outputs include it)."""
    say("case: verify T=8, hand-built routing with 32- and 24-row groups")
    D = synth.config(2).dims
    T, k, P = D.T, D.top_k, D.experts_per_group
    idx = np.zeros((T, k), dtype=np.int32)
    for t in range(T):
        if t < 4:
            hot = [(3 * t + j) % 20 for j in range(8)]                 # group 0: 32 rows
        else:
            hot = [P + (2 * t + j) % 15 for j in range(6)]             # group 1: 24 rows
        light = [(2 + (t + m) % 6) * P + (5 * t + m) % P for m in range(k - len(hot))]
        idx[t] = hot + light
    counts = np.bincount(idx.ravel() // P, minlength=D.n_experts // P)
    assert counts[0] == 32 and counts[1] == 24 and all(1 <= c <= 8 for c in counts[2:]), counts
    rng = np.random.default_rng(7)
    w = rng.uniform(0.1, 1.0, size=(T, k)).astype(np.float32)
    w /= w.sum(axis=1, keepdims=True)
    x = synth.make_activations(2, 3)
    Wdev = synth.make_weights(2, 3, device="cuda")
    lay = Layer(D, Wdev)
    idx_d = torch.from_numpy(idx).to("cuda")
    w_d = torch.from_numpy(w).to("cuda")
    y, tr = lay.forward(bits_to_dev(x), idx_d, w_d, trace=True)
    torch.cuda.synchronize()
    fw = moe_forward(x, idx, w.astype(np.float64), synth.weights_to_numpy(Wdev), P, keep=True)
    ok, ratio = y_within_tolerance(y.cpu().numpy(), fw["y"])
    say(f"  worst |dy| / bound = {ratio:.3g}")
    assert ok, f"y outside tolerance (worst ratio {ratio:.3g})"
    _check_trace(D, idx_d, tr, fw)
    y2, _ = lay.forward(bits_to_dev(x), idx_d, w_d)
    assert torch.equal(y, y2)
    # the same batch through the persistent launch (32-row passes of the down tasks)
    lay.persistent = True
    y3, tr3 = lay.forward(bits_to_dev(x), idx_d, w_d, trace=True)
    torch.cuda.synchronize()
    ok, ratio = y_within_tolerance(y3.cpu().numpy(), fw["y"])
    say(f"  persistent: worst |dy| / bound = {ratio:.3g}")
    assert ok, f"persistent y outside tolerance (worst ratio {ratio:.3g})"
    _check_trace(D, idx_d, tr3, fw)


@pytest.mark.parametrize("spread", ["one_group", "random"])
def test_decode_traced(spread):
    """One decode token, traced (permutation, activations, per-slot outputs):
    the routed case, and a hand-routed one with all ten experts in one group
    (the shared down's 10-row pass takes the 16-row staged instance, and the
    other seven groups' workgroups have no rows)."""
    say(f"case: decode T=1 traced, {spread}")
    D = synth.config(1).dims
    Wdev = synth.make_weights(1, 4, device="cuda")
    x, wr, bias = _inputs(1, 4)
    if spread == "random":
        _run_parity(D, x, wr, bias, Wdev, keep=True)
        return
    idx = np.array([[3, 17, 22, 41, 5, 63, 0, 58, 30, 9]], dtype=np.int32)   # group 0 only
    w = np.random.default_rng(8).uniform(0.1, 1.0, size=(1, D.top_k)).astype(np.float32)
    w /= w.sum(axis=1, keepdims=True)
    lay = Layer(D, Wdev)
    idx_d = torch.from_numpy(idx).to("cuda")
    w_d = torch.from_numpy(w).to("cuda")
    y, tr = lay.forward(bits_to_dev(x), idx_d, w_d, trace=True)
    torch.cuda.synchronize()
    fw = moe_forward(x, idx, w.astype(np.float64), synth.weights_to_numpy(Wdev), D.experts_per_group, keep=True)
    ok, ratio = y_within_tolerance(y.cpu().numpy(), fw["y"])
    say(f"  worst |dy| / bound = {ratio:.3g}")
    assert ok, f"y outside tolerance (worst ratio {ratio:.3g})"
    _check_trace(D, idx_d, tr, fw)
    y2, _ = lay.forward(bits_to_dev(x), idx_d, w_d)
    assert torch.equal(y, y2)


def test_graph_replay_two_layers():
    """Two full-size layers (route, forward, residual each) captured as one HIP
    graph: every replay, with eager work on the same workspaces and a
    synchronisation between replays, equals the eager pass bitwise."""
    say("case: HIP graph of two C2 layers, 4 replays")
    D = synth.config(2).dims
    layers = []
    for li in range(2):
        wr, bias = synth.make_router(2, li)
        layers.append((Layer(D, synth.make_weights(2, li, device="cuda")), bits_to_dev(wr), f32_to_dev(bias)))
    x0 = bits_to_dev(synth.make_activations(2, 0))
    x_other = bits_to_dev(synth.make_activations(2, 9))
    bufs = [torch.empty_like(x0) for _ in range(2)]
    idx = torch.empty(D.T, D.top_k, dtype=torch.int32, device="cuda")
    w = torch.empty(D.T, D.top_k, dtype=torch.float32, device="cuda")
    y = torch.empty(D.T, D.d, dtype=torch.float32, device="cuda")

    def run(x):
        for li, (lay, wr, bias) in enumerate(layers):
            em.edge_moe_route(D, x, wr, bias, idx, w, None, lay.ws)
            em.edge_moe_forward(D, x, idx, w, lay.W, y, lay.ws)
            em.edge_moe_residual(x, y, bufs[li])
            x = bufs[li]

    run(x0)
    torch.cuda.synchronize()
    ref = [bufs[0].clone(), bufs[1].clone(), y.clone(), idx.clone(), w.clone()]
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            run(x0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(4):
        # eager work between replays: another batch through the same layers and
        # workspaces, then the outputs cleared
        run(x_other)
        for t in (bufs[0], bufs[1], y, idx, w):
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [bufs[0], bufs[1], y, idx, w]
        assert all(torch.equal(a, b) for a, b in zip(got, ref)), f"replay {rep} differs from the eager pass"


_NS2_FAULT = pytest.mark.skip(reason="faulted the GPU (memory aperture violation) under the two-subtile "
                                     "decode kernels for 17-32 tokens; that instance is no longer built "
                                     "(17-32 tokens take the four-subtile kernels) and the case stays off "
                                     "the GPU until the fault's cause is shown")


@pytest.mark.parametrize("T", [2, 13, 16, pytest.param(24, marks=_NS2_FAULT), pytest.param(32, marks=_NS2_FAULT),
                               37, 200])
def test_ragged_batches(T):
    """Token counts that leave partial tiles and cross the router's small/large
    paths; 13 and 16 put more than 8 tokens into a group, so the shared up
    stages x as 16 rows x 1024 elements instead of 8 x 2048; 24 and 32 would
    run the four-subtile kernels and are skipped for the reason given."""
    say(f"case: ragged T={T}")
    D = synth.config(1).dims.with_T(T)
    x = synth.make_activations(1, 5, T=T)
    wr, _ = synth.make_router(1, 5)
    sample = np.unique(np.linspace(0, T - 1, min(T, 12)).astype(int))
    _run_parity(D, x, wr, None, synth.make_weights(1, 5, device="cuda"), sample=sample)


def test_general_path_traced():
    """A batch above the decode limit (T=72, full shapes): permutation kernels,
    the LDS-tiled shared-matrix GEMMs over partial row tiles, every slot's
    activation and expert output against the oracle."""
    say("case: general path T=72 traced")
    D = synth.config(1).dims.with_T(72)
    x = synth.make_activations(1, 3, T=72)
    wr, _ = synth.make_router(1, 3)
    lay, idx, w, y, tr, fw = _run_parity(D, x, wr, None, synth.make_weights(1, 3, device="cuda"), keep=True)
    _check_trace(D, idx, tr, fw)
    y2, _ = lay.forward(bits_to_dev(x), idx, w)
    assert torch.equal(y, y2)


def test_zero_delta_zero_lora():
    """Zero deltas and LoRA: every expert of a group is the same FFN (on the GPU too)."""
    say("case: zero delta / LoRA, verify shapes")
    D = synth.config(2).dims
    x, wr, bias = _inputs(2, 0)
    W = synth.make_weights(2, 0, device="cuda", zero_delta=True, zero_lora=True)
    _run_parity(D, x, wr, bias, W)


@pytest.mark.parametrize("pattern", ["2", "3", "4", "6", "8", "5+3"])
def test_repeated_token_batches(pattern):
    """Batches made of repeated tokens, so that selected experts carry several
    rows: "n" is one token n times (every selected expert has n rows), "5+3"
    one token five times beside three distinct ones.  The sampled verify
    routings give one or two rows per expert; these cases fill the decode
    kernels' 16-row tiles further and put up to 8 rows into one expert's
    range.  Traced: permutation, activations and expert outputs too."""
    say(f"case: repeated-token batch {pattern}")
    if "+" in pattern:
        n, m = (int(p) for p in pattern.split("+"))
        base = synth.make_activations(1, 9, T=1 + m)
        x = np.concatenate([np.repeat(base[:1], n, axis=0), base[1:]])
    else:
        n = int(pattern)
        x = np.repeat(synth.make_activations(1, 9, T=1), n, axis=0)
    D = synth.config(1).dims.with_T(x.shape[0])
    wr, _ = synth.make_router(1, 9)
    lay, idx, w, y, tr, fw = _run_parity(D, x, wr, None, synth.make_weights(1, 9, device="cuda"), keep=True)
    _check_trace(D, idx, tr, fw)
    counts = np.bincount(idx.cpu().numpy().ravel(), minlength=D.n_experts)
    assert counts.max() == n


def test_top1_routing():
    say("case: top-1")
    D = synth.Dims(**{**synth.config(2).dims.__dict__, "top_k": 1})
    x, wr, _ = _inputs(2, 1)
    lay = Layer(D, synth.make_weights(2, 1, device="cuda"))
    idx, w, _ = _check_route(D, x, wr, None, lay)
    assert torch.all(w == 1.0)


@pytest.mark.parametrize("E,T,d", [(64, 8, 256), (512, 8, 256), (1024, 8, 256), (512, 40, 256), (512, 8, 4096)])
def test_route_ties(E, T, d):
    """Many equal logits (experts share one of 5 weight rows, every 13th row is
    zero): the order must be descending logit, equal logits by lower index.
    Covers both top-k register layouts (E <= 512 and E <= 1024) and the three
    logits kernels (T <= 16; larger batches; the K-split one at d = 4096)."""
    say(f"case: route ties E={E} T={T} d={d}")
    D = synth.Dims(T=T, d=d, h=256, n_experts=E, experts_per_group=max(E // 16, 4), top_k=10,
                   delta_rank=8, lora_rank=2, quant_group=32)
    rng = np.random.default_rng(E + T)
    x = synth.bf16_bits_from_f32(rng.standard_normal((T, D.d), dtype=np.float32))
    base = rng.standard_normal((5, D.d), dtype=np.float32) * np.float32(0.05)
    w = base[(np.arange(E) * 7919) % 5].copy()
    w[::13] = 0.0
    wr = synth.bf16_bits_from_f32(w)
    lay = Layer(D, {})
    _check_route(D, x, wr, None, lay)
    bias = np.zeros(E, dtype=np.float32)
    bias[::3] = np.float32(0.25)
    _check_route(D, x, wr, bias, lay)


def test_residual_bit_exact():
    say("case: residual")
    rng = np.random.default_rng(4)
    x = synth.bf16_bits_from_f32(rng.standard_normal((8, 4096), dtype=np.float32))
    y = (rng.standard_normal((8, 4096)) * 0.5).astype(np.float32)
    y[0, :4] = [2.0 ** -8, 3 * 2.0 ** -8, 0.0, -1.0]
    x[0, :4] = synth.bf16_bits_from_f32(np.array([1.0, 1.0, 0.0, 1.0], dtype=np.float32))
    xd = bits_to_dev(x)
    out = torch.empty_like(xd)
    em.edge_moe_residual(xd, f32_to_dev(y), out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint16), residual(x, y))


def test_workspace_too_small_is_rejected():
    D = synth.config(2).dims
    x, wr, bias = _inputs(2, 0)
    lay = Layer(D, synth.make_weights(2, 0, device="cuda"))
    idx, w, _ = lay.route(bits_to_dev(x), bits_to_dev(wr), f32_to_dev(bias))
    y = torch.empty(D.T, D.d, dtype=torch.float32, device="cuda")
    with pytest.raises(em.EdgeMoeError) as ei:
        em.edge_moe_forward(D, bits_to_dev(x), idx, w, lay.W, y, lay.ws[:1024])
    assert ei.value.status == em.EDGE_MOE_EWORKSPACE


def _kernel_names(fn):
    """Names of the library kernels that fn() enqueues (from the library's
    kernel timing table)."""
    em.edge_moe_prof_reset()
    em.edge_moe_prof_enable(True)
    try:
        fn()
        torch.cuda.synchronize()
    finally:
        em.edge_moe_prof_enable(False)
    names = set(em.edge_moe_prof_read())
    em.edge_moe_prof_reset()
    return names


def test_stack_48_teacher_forced():
    """The 48-layer stack (T=8, independent routers, residual between layers):
    the chain runs on the GPU; on sampled layers the oracle recomputes the layer
    from the GPU's own input x_l (teacher forcing: an untethered chain may
    legitimately take another route at a near tie) and the residual is checked
    bitwise.

    The stack has no normalisation, so activations grow about 2x per layer
    (|x| ~ 3e3 at layer 12, ~1e14 at layer 47).  A rounding point (R1-R5) that
    lands on the other side of a bf16 midpoint moves the outputs by an amount
    proportional to the row's magnitude (a z2 value one bf16 step apart moves o
    by ~1e-4 of the row), and outputs that cancel to far below the row's
    magnitude carry fp32 accumulation error at the row's scale.  So the
    element-wise gate applies to the first layers (|x| ~ 1-5) and deeper
    layers are gated relative to each token's row: |dy| <= 2e-3 max|y_row|."""
    say("case: 48-layer stack, teacher-forced on sampled layers")
    cfg = synth.config(4)
    D = cfg.dims
    elementwise = (0, 1)
    row_scaled = (12, 24, cfg.layers - 1)
    lay = None
    x = bits_to_dev(synth.make_activations(4, 0))
    # the kernels a verify batch with decode-tiled weights runs (the benchmark's
    # stack takes the same path): every layer below must run exactly these
    x2 = bits_to_dev(synth.make_activations(2, 0))
    ref_lay = Layer(D, synth.make_weights(2, 0, device="cuda"))
    ridx, rw, _ = ref_lay.route(x2, bits_to_dev(synth.make_router(2, 0)[0]), None)
    ref_names = _kernel_names(lambda: ref_lay.forward(x2, ridx, rw))
    del ref_lay
    for layer in range(cfg.layers):
        wr, _ = synth.make_router(4, 0, layer)
        W = synth.make_weights(4, 0, layer, device="cuda")
        if lay is None:
            lay = Layer(D, W)                       # decode-tiled copies, as in the benchmark
        else:
            lay.W = em.tile_weights(D, W)
        idx, w, _ = lay.route(x, bits_to_dev(wr), None)
        names = _kernel_names(lambda: lay.forward(x, idx, w))
        assert names == ref_names, f"layer {layer}: kernels {names} differ from the verify path's {ref_names}"
        y, _ = lay.forward(x, idx, w)
        x_next = torch.empty_like(x)
        em.edge_moe_residual(x, y, x_next)
        torch.cuda.synchronize()
        if layer in elementwise + row_scaled:
            xb = x.cpu().numpy().view(np.uint16)
            ref = route(xb, wr, None, D.top_k)
            assert np.array_equal(idx.cpu().numpy(), ref["idx"]), f"layer {layer}: expert indices differ"
            fw = moe_forward(xb, ref["idx"], ref["w"], synth.weights_to_numpy(W), D.experts_per_group)
            yg = y.cpu().numpy()
            if layer in elementwise:
                ok, ratio = y_within_tolerance(yg, fw["y"])
            else:
                dev = np.abs(yg.astype(np.float64) - fw["y"])
                ratio = float(np.max(dev / (2e-3 * np.max(np.abs(fw["y"]), axis=1, keepdims=True))))
                ok = ratio <= 1.0
            say(f"  layer {layer}: worst |dy| / bound = {ratio:.3g}")
            assert ok, f"layer {layer}: y outside tolerance"
            assert np.array_equal(x_next.cpu().numpy().view(np.uint16), residual(xb, yg))
        del W
        x = x_next
