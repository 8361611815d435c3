"""GPU parity of the MX variant (edge_moe_forward_mx, MXFP4 shared and delta
matrices on the scaled FP4 x FP8 matrix cores) against the oracle's MX mode.

Routing is the int4 layer's (same router call, checked bitwise there); the
permutation is compared bit for bit; y element-wise against the oracle.

Gate on y (D24): |dy| <= 4e-3 + 4e-3 |y_ref| (twice the int4 layer's bound)
on at least 99.99 % of elements and within three times that on every element,
and at least 99.7 % of elements within the int4 layer's own 2e-3 + 2e-3 |y_ref|.
Why the variant needs more: the activation rows are requantised to E4M3 before
S_dn and A_dn, so an activation whose bf16 rounding lands on the other side of
a midpoint (as in the int4 layer) moves that term by a whole E4M3 step, 16 bf16
steps, whenever the two bf16 values straddle an E4M3 rounding boundary (about
one flip in 16); the scaled FP4 x FP8 matrix cores sum each instruction's 128
products to about 2^-13.5 of their magnitude sum (measured on gfx950), not
fp32, which doubles the share of activations that round the other way (about
0.8 % against 0.4 %); and an R1 input that rounds the other way shifts a whole
row's pre-activations, so a few tokens carry tens of E4M3 changes at once.  At
the full 16K prefill (4.2 M checked elements) those tokens put a few elements
per hundred thousand past the 1x bound (worst 2.1x), which small samples never
reach.
"""
import numpy as np
import pytest
import torch

import shared_matrix_expert_amd as em
import synth
from oracle import mx
from oracle.layer import route
from gpu_helpers import DEV, bits_to_dev, expected_permutation, f32_to_dev, say, tile_cover_sample

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)


def mx_gate(y, y_ref):
    """D24: (ok, summary) for GPU outputs y against the oracle's y_ref."""
    err = np.abs(np.asarray(y, dtype=np.float64) - y_ref)
    ratio = err / (4e-3 + 4e-3 * np.abs(y_ref))
    within_mx = float(np.mean(ratio <= 1.0))
    within_int4 = float(np.mean(err <= 2e-3 + 2e-3 * np.abs(y_ref)))
    worst = float(ratio.max())
    ok = worst <= 3.0 and within_mx >= 0.9999 and within_int4 >= 0.997
    return ok, (f"worst |dy| / bound = {worst:.3g}, within the bound {within_mx:.6f}, "
                f"within the int4 gate {within_int4:.5f}, max |dy| = {err.max():.3g}")


def _run_mx(cfg, seed, T=None, trace=True, sample=None):
    D = synth.config(cfg).dims if T is None else synth.config(cfg).dims.with_T(T)
    x = synth.make_activations(cfg, seed, T=D.T)
    wr, bias = synth.make_router(cfg, seed)
    W = synth.make_weights_mx(cfg, seed, device=DEV)
    ws = torch.empty(max(em.edge_moe_workspace_bytes(D), em.edge_moe_workspace_bytes_mx(D)),
                     dtype=torch.uint8, device=DEV)
    xd = bits_to_dev(x)
    idx = torch.empty(D.T, D.top_k, dtype=torch.int32, device=DEV)
    w = torch.empty(D.T, D.top_k, dtype=torch.float32, device=DEV)
    em.edge_moe_route(D, xd, bits_to_dev(wr), f32_to_dev(bias), idx, w, None, ws)
    y = torch.empty(D.T, D.d, dtype=torch.float32, device=DEV)
    R = D.T * D.top_k
    tr = None
    if trace:
        tr = {"expert_offsets": torch.empty(D.n_experts + 1, dtype=torch.int32, device=DEV),
              "row_token": torch.empty(R, dtype=torch.int32, device=DEV),
              "row_slot": torch.empty(R, dtype=torch.int32, device=DEV),
              "act": torch.empty(R, D.h, dtype=torch.int16, device=DEV),
              "expert_out": torch.empty(R, D.d, dtype=torch.float32, device=DEV)}
    em.edge_moe_forward_mx(D, xd, idx, w, W, y, ws, trace=tr)
    torch.cuda.synchronize()
    rows = np.arange(D.T) if sample is None else np.asarray(sample)
    ref = route(x[rows], wr, bias, D.top_k)
    assert np.array_equal(idx.cpu().numpy()[rows], ref["idx"]), "expert indices differ"
    Wh = synth.weights_to_numpy(W)
    fw = mx.moe_forward_mx(x[rows], ref["idx"], ref["w"], Wh, D.experts_per_group, keep=trace)
    yg = y.cpu().numpy()[rows]
    ok, msg = mx_gate(yg, fw["y"])
    say(f"  MX {D.T} tokens: {msg}, max |y| = {np.abs(fw['y']).max():.3g}")
    if trace:
        offs, rt, rs = expected_permutation(idx.cpu().numpy(), D.n_experts)
        assert np.array_equal(tr["expert_offsets"].cpu().numpy(), offs)
        assert np.array_equal(tr["row_token"].cpu().numpy(), rt)
        assert np.array_equal(tr["row_slot"].cpu().numpy(), rs)
        act = tr["act"].cpu().numpy().view(np.uint16)
        a_gpu = (act.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        ref_a = fw["a"].reshape(-1, D.h)
        say(f"  activations differing: {np.mean(a_gpu != ref_a):.4f}, "
            f"max |da| = {np.max(np.abs(a_gpu - ref_a)):.3g}")
    assert ok, f"y outside tolerance: {msg}"
    return D, y, fw


@pytest.mark.parametrize("seed", [0, 1])
def test_mx_small_layer(seed):
    say(f"case: MX small (cfg 5) seed={seed}")
    _run_mx(5, seed)


@pytest.mark.parametrize("T", [1, 8, 37])
def test_mx_small_ragged(T):
    say(f"case: MX small (cfg 5) T={T}")
    _run_mx(5, 0, T=T)


@pytest.mark.parametrize("seed", [0, 1])
def test_mx_verify_full_size(seed):
    say(f"case: MX verify T=8 at full size (cfg 2 shapes) seed={seed}")
    _run_mx(2, seed)


@pytest.mark.parametrize("seed", [0, 1])
def test_mx_prefill_tile_cover(seed):
    """The MX variant at the full 16K-token prefill, the launch the benchmark's
    MX line times: the whole 163,840-slot permutation against a lexsort, and y
    against the oracle's MX mode on >= 1024 tokens chosen so that every
    128-row tile of every MX GEMM (distinct token rows of each group for the
    shared up, each group's rows for the shared down, each expert's rows for
    its rank-128 inputs) holds a checked row.  Routing is checked bitwise on
    the same tokens."""
    say(f"case: MX prefill C3 seed={seed}, tile-covering token sample")
    D = synth.config(3).dims
    x = synth.make_activations(3, seed)
    wr, bias = synth.make_router(3, seed)
    W = synth.make_weights_mx(3, seed, device=DEV)
    ws = torch.empty(max(em.edge_moe_workspace_bytes(D), em.edge_moe_workspace_bytes_mx(D)),
                     dtype=torch.uint8, device=DEV)
    xd = bits_to_dev(x)
    idx = torch.empty(D.T, D.top_k, dtype=torch.int32, device=DEV)
    w = torch.empty(D.T, D.top_k, dtype=torch.float32, device=DEV)
    em.edge_moe_route(D, xd, bits_to_dev(wr), f32_to_dev(bias), idx, w, None, ws)
    R = D.T * D.top_k
    tr = {"expert_offsets": torch.empty(D.n_experts + 1, dtype=torch.int32, device=DEV),
          "row_token": torch.empty(R, dtype=torch.int32, device=DEV),
          "row_slot": torch.empty(R, dtype=torch.int32, device=DEV)}
    y = torch.empty(D.T, D.d, dtype=torch.float32, device=DEV)
    em.edge_moe_forward_mx(D, xd, idx, w, W, y, ws, trace=tr)
    torch.cuda.synchronize()
    say("  forward done")
    idx_h = idx.cpu().numpy()
    offs, rt, rs = expected_permutation(idx_h, D.n_experts)
    assert np.array_equal(tr["expert_offsets"].cpu().numpy(), offs), "expert offsets differ"
    assert np.array_equal(tr["row_token"].cpu().numpy(), rt), "row tokens differ"
    assert np.array_equal(tr["row_slot"].cpu().numpy(), rs), "row slots differ"
    sample, n_cover, n_tiles = tile_cover_sample(offs, rt, D.experts_per_group, D.n_groups, D.T, 1024)
    say(f"  {n_cover} tokens cover {n_tiles} row tiles; {sample.size} tokens checked")
    ref = route(x[sample], wr, bias, D.top_k)
    assert np.array_equal(idx_h[sample], ref["idx"]), "expert indices differ"
    assert np.max(np.abs(w.cpu().numpy()[sample] - ref["w"])) <= 1e-6
    say("  oracle routing done")
    fw = mx.moe_forward_mx(x[sample], ref["idx"], ref["w"], synth.weights_to_numpy(W), D.experts_per_group)
    ok, msg = mx_gate(y.cpu().numpy()[sample], fw["y"])
    say(f"  MX prefill: {msg}")
    assert ok, f"y outside tolerance: {msg}"
