"""Pins of the oracle's expert layer.

* exact mode against the plain dense definition with W_e materialised;
* hand-built layers whose contract-mode output has a closed form that depends
  on each bf16 rounding point R1..R5;
* zero deltas and zero LoRA: every expert of a group is the same FFN;
* token-permutation equivariance and expert relabelling within a group;
* V = 0 removes the LoRA branch;
* a per-element loop implementation on a tiny layer.
"""
import math

import numpy as np
import pytest

import synth
from oracle import codecs
from oracle.layer import moe_forward, residual, route
from helpers import TINY, bf16_from, random_router, random_weights, random_x, set_int4, zero_weights


def _dense_layer(x_bits, idx, w, W, P):
    """y = sum_j w_j W_dn_e silu(W_up_e x) with W_e = S_g + B_e A_e + V_g U_g materialised."""
    X = codecs.bf16_to_f64(x_bits)
    T, d = X.shape
    h = W["s_up"].shape[1]
    r = W["a_up"].shape[1]
    y = np.zeros((T, d))
    for t in range(T):
        for j in range(idx.shape[1]):
            e = int(idx[t, j])
            g = e // P
            Wup = (codecs.dequant(W["s_up"][g], W["s_up_scale"][g], d)
                   + codecs.dequant(W["b_up"][e], W["b_up_scale"][e], r)
                   @ codecs.dequant(W["a_up"][e], W["a_up_scale"][e], d)
                   + codecs.bf16_to_f64(W["lora_up_v"][g]) @ codecs.bf16_to_f64(W["lora_up_u"][g]))
            Wdn = (codecs.dequant(W["s_dn"][g], W["s_dn_scale"][g], h)
                   + codecs.dequant(W["b_dn"][e], W["b_dn_scale"][e], r)
                   @ codecs.dequant(W["a_dn"][e], W["a_dn_scale"][e], h)
                   + codecs.bf16_to_f64(W["lora_dn_v"][g]) @ codecs.bf16_to_f64(W["lora_dn_u"][g]))
            y[t] += w[t, j] * (Wdn @ codecs.silu(Wup @ X[t]))
    return y


@pytest.mark.parametrize("D,seed", [(TINY, 0), (TINY, 1), (synth.config(0).dims, 2)])
def test_exact_mode_equals_materialised_dense(D, seed):
    W = random_weights(D, seed)
    x = random_x(D.T, D.d, seed)
    wr = random_router(D.n_experts, D.d, seed)
    rt = route(x, wr, None, D.top_k)
    got = moe_forward(x, rt["idx"], rt["w"], W, D.experts_per_group, mode="exact")["y"]
    ref = _dense_layer(x, rt["idx"], rt["w"], W, D.experts_per_group)
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))
    # every group is exercised on the multi-group layer
    if D.n_groups > 1:
        assert len(set((rt["idx"] // D.experts_per_group).ravel().tolist())) == D.n_groups


# ---- closed forms that isolate each rounding point ---------------------------------

D8 = synth.Dims(T=1, d=8, h=8, n_experts=4, experts_per_group=4, top_k=1,
                delta_rank=2, lora_rank=2, quant_group=8)
SILU1_BF16 = 0.73046875            # bf16(SiLU(1)) = bf16(0.7310585786...)


def _onehot(n, k, i, j, v=1.0):
    m = np.zeros((n, k))
    m[i, j] = v
    return m


def _x(vals):
    v = np.zeros((1, 8), dtype=np.float32)
    v[0, :len(vals)] = vals
    return bf16_from(v)


def _run(W, x, mode="contract"):
    return moe_forward(x, np.array([[0]], dtype=np.int32), np.array([[1.0]]), W, 4, mode=mode)["y"][0]


def test_closed_form_R1_delta_input():
    W = zero_weights(D8)
    a = np.zeros((2, 8)); a[0, 0] = a[0, 1] = 1.0
    set_int4(W, D8, "a_up", 0, a)                         # z1_0 = x0 + x1 = 1 + 2^-8
    set_int4(W, D8, "b_up", 0, _onehot(8, 2, 0, 0))       # h_0 = z1_0
    set_int4(W, D8, "s_dn", 0, _onehot(8, 8, 0, 0))       # o_0 = a_0
    x = _x([1.0, 2.0 ** -8])
    assert _run(W, x)[0] == SILU1_BF16                    # R1 ties 1 + 2^-8 down to 1
    assert _run(W, x, "exact")[0] == pytest.approx(codecs.silu(np.array([1 + 2.0 ** -8]))[0], rel=1e-15)


def test_closed_form_R2_lora_up_input():
    W = zero_weights(D8)
    u = np.zeros((2, 8), dtype=np.float32); u[0, 0] = u[0, 1] = 1.0
    W["lora_up_u"][0] = bf16_from(u)
    W["lora_up_v"][0] = bf16_from(_onehot(8, 2, 0, 0))
    set_int4(W, D8, "s_dn", 0, _onehot(8, 8, 0, 0))
    x = _x([1.0, 2.0 ** -8])
    assert _run(W, x)[0] == SILU1_BF16


def test_closed_form_R3_activation():
    W = zero_weights(D8)
    set_int4(W, D8, "s_up", 0, _onehot(8, 8, 0, 0))
    set_int4(W, D8, "s_dn", 0, _onehot(8, 8, 3, 0, 2.0))   # o_3 = 2 a_0
    y = _run(W, _x([1.0]))
    assert y[3] == 2 * SILU1_BF16 and np.count_nonzero(y) == 1
    assert _run(W, _x([1.0]), "exact")[3] == pytest.approx(2 / (1 + math.exp(-1)), rel=1e-15)


def _two_activations(W):
    """h_0 = 8 -> a_0 = bf16(SiLU(8)) = 8;  h_1 = 1/16 -> a_1 = 0.0322265625."""
    s = np.zeros((8, 8)); s[0, 0] = 8.0; s[1, 0] = 0.0625
    set_int4(W, D8, "s_up", 0, s)


def test_two_activation_values():
    assert codecs.rn_bf16(codecs.silu(np.array([8.0])))[0] == 8.0
    assert codecs.rn_bf16(codecs.silu(np.array([0.0625])))[0] == 0.0322265625


def test_closed_form_R4_delta_down_input():
    W = zero_weights(D8)
    _two_activations(W)
    a = np.zeros((2, 8)); a[0, 0] = a[0, 1] = 1.0
    set_int4(W, D8, "a_dn", 0, a)                         # z2_0 = a_0 + a_1 = 8.0322265625
    set_int4(W, D8, "b_dn", 0, _onehot(8, 2, 5, 0))       # o_5 = z2_0
    y = _run(W, _x([1.0]))
    assert y[5] == 8.0625 and np.count_nonzero(y) == 1    # R4: nearest bf16 above


def test_closed_form_R5_lora_down_input():
    W = zero_weights(D8)
    _two_activations(W)
    u = np.zeros((2, 8), dtype=np.float32); u[1, 0] = u[1, 1] = 1.0
    W["lora_dn_u"][0] = bf16_from(u)
    W["lora_dn_v"][0] = bf16_from(_onehot(8, 2, 6, 1))
    y = _run(W, _x([1.0]))
    assert y[6] == 8.0625 and np.count_nonzero(y) == 1


def test_closed_form_combine_weights_and_groups():
    """Two groups, two slots: y = w0 * o(expert in group 0) + w1 * o(expert in group 1)."""
    D = synth.Dims(T=1, d=8, h=8, n_experts=4, experts_per_group=2, top_k=2,
                   delta_rank=2, lora_rank=2, quant_group=8)
    W = zero_weights(D)
    set_int4(W, D, "s_up", 0, _onehot(8, 8, 0, 0))
    set_int4(W, D, "s_up", 1, _onehot(8, 8, 0, 0))
    set_int4(W, D, "s_dn", 0, _onehot(8, 8, 1, 0))        # group 0 writes y_1
    set_int4(W, D, "s_dn", 1, _onehot(8, 8, 2, 0, 4.0))   # group 1 writes y_2
    y = moe_forward(_x([1.0]), np.array([[3, 0]], dtype=np.int32), np.array([[0.75, 0.25]]),
                    W, 2)["y"][0]
    assert y[1] == 0.25 * SILU1_BF16 and y[2] == 0.75 * 4 * SILU1_BF16


# ---- structural identities ---------------------------------------------------------

def test_zero_delta_zero_lora_group_identity_single_group():
    D = synth.config(0).dims
    W = random_weights(D, 5, zero_delta=True, zero_lora=True)
    x = random_x(D.T, D.d, 5)
    X = codecs.bf16_to_f64(x)
    Sup = codecs.dequant(W["s_up"][0], W["s_up_scale"][0], D.d)
    Sdn = codecs.dequant(W["s_dn"][0], W["s_dn_scale"][0], D.h)
    ffn = codecs.silu(X @ Sup.T) @ Sdn.T
    rng = np.random.default_rng(0)
    for _ in range(3):
        idx = np.stack([rng.permutation(D.n_experts)[:D.top_k] for _ in range(D.T)]).astype(np.int32)
        w = rng.dirichlet(np.ones(D.top_k), size=D.T)
        y = moe_forward(x, idx, w, W, D.experts_per_group, mode="exact")["y"]
        np.testing.assert_allclose(y, ffn, rtol=1e-12, atol=1e-12)


def test_zero_delta_zero_lora_group_identity_multi_group():
    D = TINY
    W = random_weights(D, 6, zero_delta=True, zero_lora=True)
    x = random_x(D.T, D.d, 6)
    X = codecs.bf16_to_f64(x)
    wr = random_router(D.n_experts, D.d, 6)
    rt = route(x, wr, None, D.top_k)
    y = moe_forward(x, rt["idx"], rt["w"], W, D.experts_per_group, mode="exact")["y"]
    ref = np.zeros_like(y)
    for g in range(D.n_groups):
        Sup = codecs.dequant(W["s_up"][g], W["s_up_scale"][g], D.d)
        Sdn = codecs.dequant(W["s_dn"][g], W["s_dn_scale"][g], D.h)
        Wg = np.where(rt["idx"] // D.experts_per_group == g, rt["w"], 0.0).sum(1)
        ref += Wg[:, None] * (codecs.silu(X @ Sup.T) @ Sdn.T)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("mode", ["exact", "contract"])
def test_token_permutation_equivariance(mode):
    D = TINY
    W = random_weights(D, 7)
    x = random_x(D.T, D.d, 7)
    rt = route(x, random_router(D.n_experts, D.d, 7), None, D.top_k)
    y = moe_forward(x, rt["idx"], rt["w"], W, D.experts_per_group, mode=mode)["y"]
    perm = np.random.default_rng(1).permutation(D.T)
    yp = moe_forward(x[perm], rt["idx"][perm], rt["w"][perm], W, D.experts_per_group, mode=mode)["y"]
    np.testing.assert_allclose(yp, y[perm], rtol=1e-12, atol=1e-14)


def test_expert_relabel_within_group():
    D = TINY
    W = random_weights(D, 8)
    x = random_x(D.T, D.d, 8)
    rt = route(x, random_router(D.n_experts, D.d, 8), None, D.top_k)
    y = moe_forward(x, rt["idx"], rt["w"], W, D.experts_per_group, mode="exact")["y"]
    P = D.experts_per_group
    pi = np.concatenate([g * P + np.random.default_rng(g).permutation(P) for g in range(D.n_groups)])
    W2 = dict(W)
    for n in ("a_up", "b_up", "a_dn", "b_dn"):
        for suf in ("", "_scale"):
            arr = np.empty_like(W[n + suf])
            arr[pi] = W[n + suf]                       # expert e's delta now lives at pi[e]
            W2[n + suf] = arr
    y2 = moe_forward(x, pi[rt["idx"]].astype(np.int32), rt["w"], W2, P, mode="exact")["y"]
    np.testing.assert_allclose(y2, y, rtol=1e-12, atol=1e-14)


def test_lora_v_zero_removes_branch():
    D = TINY
    W = random_weights(D, 9)
    W["lora_up_v"][:] = 0
    W["lora_dn_v"][:] = 0
    x = random_x(D.T, D.d, 9)
    rt = route(x, random_router(D.n_experts, D.d, 9), None, D.top_k)
    y = moe_forward(x, rt["idx"], rt["w"], W, D.experts_per_group)["y"]
    W["lora_up_u"] = random_weights(D, 10)["lora_up_u"]
    W["lora_dn_u"] = random_weights(D, 11)["lora_dn_u"]
    y2 = moe_forward(x, rt["idx"], rt["w"], W, D.experts_per_group)["y"]
    assert np.array_equal(y, y2)


def test_contract_close_to_exact():
    D = synth.config(0).dims
    W = random_weights(D, 12)
    x = synth.make_activations(0, 0)
    wr, _ = synth.make_router(0, 0)
    rt = route(x, wr, None, D.top_k)
    yc = moe_forward(x, rt["idx"], rt["w"], W, D.experts_per_group, mode="contract")["y"]
    ye = moe_forward(x, rt["idx"], rt["w"], W, D.experts_per_group, mode="exact")["y"]
    rel = np.sqrt(np.mean((yc - ye) ** 2)) / np.sqrt(np.mean(ye ** 2))
    assert 1e-5 < rel < 2e-2


# ---- per-element loops on a tiny layer ---------------------------------------------

def _bf16_round_scalar(v):
    if v == 0.0:
        return 0.0
    m, e = math.frexp(v)
    return math.ldexp(round(m * 256.0) / 256.0, e)      # Python round is half-to-even


def test_per_element_loops_contract_mode():
    D = TINY
    W = random_weights(D, 13)
    x = random_x(D.T, D.d, 13)
    rt = route(x, random_router(D.n_experts, D.d, 13), None, D.top_k)
    got = moe_forward(x, rt["idx"], rt["w"], W, D.experts_per_group)["y"]
    X = codecs.bf16_to_f64(x).tolist()

    def mat(name, i, K):
        return codecs.dequant(W[name][i], W[name + "_scale"][i], K).tolist()

    def bmat(name, i):
        return codecs.bf16_to_f64(W[name][i]).tolist()

    def mv(M, v):
        return [math.fsum(a * b for a, b in zip(row, v)) for row in M]

    P, d, h, r = D.experts_per_group, D.d, D.h, D.delta_rank
    for t in range(D.T):
        yt = [0.0] * d
        for j in range(D.top_k):
            e = int(rt["idx"][t, j]); g = e // P
            z1 = [_bf16_round_scalar(v) for v in mv(mat("a_up", e, d), X[t])]
            zl = [_bf16_round_scalar(v) for v in mv(bmat("lora_up_u", g), X[t])]
            s1, d1, l1 = mv(mat("s_up", g, d), X[t]), mv(mat("b_up", e, r), z1), mv(bmat("lora_up_v", g), zl)
            a = [_bf16_round_scalar(hh / (1 + math.exp(-hh))) for hh in
                 (math.fsum((p, q, s)) for p, q, s in zip(s1, d1, l1))]
            z2 = [_bf16_round_scalar(v) for v in mv(mat("a_dn", e, h), a)]
            zl2 = [_bf16_round_scalar(v) for v in mv(bmat("lora_dn_u", g), a)]
            o = [math.fsum(v) for v in zip(mv(mat("s_dn", g, h), a), mv(mat("b_dn", e, r), z2),
                                           mv(bmat("lora_dn_v", g), zl2))]
            for n in range(d):
                yt[n] += rt["w"][t, j] * o[n]
        np.testing.assert_allclose(got[t], yt, rtol=1e-12, atol=1e-14)


def test_residual_closed_forms():
    x = bf16_from(np.array([[1.0, 1.0, -1.0, 0.0, 3.0, 2.0 ** -20]], dtype=np.float32))
    y = np.array([[2.0 ** -8, 3 * 2.0 ** -8, -(2.0 ** -8 + 2.0 ** -30), 0.1, -3.0, 1.0]],
                 dtype=np.float32)
    out = codecs.bf16_to_f64(residual(x, y))[0]
    assert out[0] == 1.0                          # 1 + 2^-8: tie, to even
    assert out[1] == 1.0 + 2.0 ** -6              # 1 + 3 * 2^-8: tie, to even (up)
    assert out[2] == -(1.0 + 2.0 ** -7)           # just past the midpoint
    assert out[3] == 0.10009765625                # bf16(fp32(0.1)) = 205 / 2048
    assert out[4] == 0.0
    assert out[5] == 1.0
