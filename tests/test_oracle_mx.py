"""Pins of the oracle's MX (MXFP4 weights, MXFP8 product inputs) mode.

Each check compares against something other than the oracle's own formula:
the element tables the OCP Microscaling specification prints, a brute-force
nearest-value search over every code, structural properties of the grids,
closed forms on constructed inputs, and the int4 layer (itself pinned in
tests/test_oracle_layer.py) when the MX quantiser is switched off.
"""
import numpy as np
import pytest

from oracle import codecs, layer, mx
import synth
from helpers import TINY, bf16_from, set_int4, zero_weights


# ---------------------------------------------------------------- element codecs --

def test_e2m1_table():
    """The 16 E2M1 values as the specification tabulates them."""
    want = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    got = mx.e2m1_to_f64(np.arange(16))
    assert got[:8].tolist() == want
    assert (-got[8:]).tolist() == want
    assert np.signbit(got[8])                       # code 8 is -0


def test_e4m3_known_codes():
    table = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0, 0x3F: 1.875,
             0x40: 2.0, 0x7E: 448.0, 0x80: -0.0, 0xB8: -1.0, 0xFE: -448.0}
    for c, v in table.items():
        got = float(mx.e4m3_to_f64(np.array([c]))[0])
        assert got == v and np.signbit(got) == np.signbit(v), hex(c)
    assert np.isnan(mx.e4m3_to_f64(np.array([0x7F, 0xFF]))).all()


def test_e4m3_grid_structure():
    """Codes 0x00..0x7E are strictly increasing; the spacing is 2^-9 through the
    subnormals and the first binade, then doubles at every power of two."""
    v = mx.e4m3_to_f64(np.arange(0x7F))
    dv = np.diff(v)
    assert np.all(dv > 0)
    for i, step in enumerate(dv):
        lo = v[i]
        want = 2.0 ** -9 if lo < 2.0 ** -5 else 2.0 ** (np.floor(np.log2(lo)) - 3)
        assert step == want, (i, lo, step)


def _brute_e4m3(x):
    """Nearest finite E4M3 magnitude to |x| by search over all codes, ties to
    the even code, then saturate at 448; sign from x."""
    grid = mx.e4m3_to_f64(np.arange(0x7F))
    a = min(abs(x), 448.0)
    d = np.abs(grid - a)
    best = np.flatnonzero(d == d.min())
    c = int(best[0]) if len(best) == 1 else int([b for b in best if b % 2 == 0][0])
    return c | (0x80 if np.signbit(x) else 0)


def test_e4m3_encode_brute_force():
    rng = np.random.default_rng(7)
    grid = mx.e4m3_to_f64(np.arange(0x7F))
    mids = (grid[:-1] + grid[1:]) / 2                           # every tie
    vals = np.concatenate([grid, mids, mids * (1 + 1e-12), mids * (1 - 1e-12),
                           rng.uniform(0, 512, 2000), np.exp2(rng.uniform(-14, 9, 2000)),
                           [448, 449, 463.99, 464, 464.01, 500, 1e6, 2.0 ** -10, 2.0 ** -10 * 1.0000001,
                            3 * 2.0 ** -11, 0.0]])
    vals = np.concatenate([vals, -vals])
    got = mx.e4m3_encode(vals)
    for x, c in zip(vals, got):
        assert int(c) == _brute_e4m3(float(x)), (x, hex(int(c)), hex(_brute_e4m3(float(x))))


def test_e4m3_decode_encode_roundtrip():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    assert np.array_equal(mx.e4m3_encode(mx.e4m3_to_f64(codes)), codes.astype(np.uint8))


# ---------------------------------------------------------------- blocks ----------

def test_unpack_fp4_nibble_order():
    b = np.array([[0x21, 0xF7]], dtype=np.uint8)          # elements 1, 2, 7, 15
    assert mx.unpack_fp4(b).tolist() == [[1, 2, 7, 15]]


def test_dequant_mxfp4_every_code_and_scale():
    codes = np.arange(128) % 16                            # all 16 codes in every block
    packed = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)[None, :]
    table = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6] * 8)
    for X in (0, 100, 127, 130, 254):
        got = mx.dequant_mxfp4(packed, np.full((1, 1, 4), X), 128)[0]
        assert np.array_equal(got, table * 2.0 ** (X - 127))


def test_scale_layout_k_step_major():
    """Stored [K/128][N][4]: row n's block b scale sits at [b // 4][n][b % 4]."""
    N, K = 3, 256
    sc = np.zeros((K // 128, N, 4), dtype=np.int64)
    for n in range(N):
        for b in range(K // 32):
            sc[b // 4, n, b % 4] = 100 + 10 * n + b
    rows = mx.scales_by_row(sc)
    assert rows.tolist() == [[100 + 10 * n + b for b in range(K // 32)] for n in range(N)]
    packed = np.full((N, K // 2), 0x22, dtype=np.uint8)          # every element 1.0
    w = mx.dequant_mxfp4(packed, sc, K)
    for n in range(N):
        for b in range(K // 32):
            assert np.all(w[n, 32 * b:32 * b + 32] == 2.0 ** (100 + 10 * n + b - 127))


def test_block_scale_range():
    rng = np.random.default_rng(3)
    amax = np.exp2(rng.uniform(-100, 100, 5000))
    X = mx.block_scale_exp(amax)
    r = amax / np.exp2(X - 127.0)
    assert np.all((r >= 256) & (r < 512))
    assert mx.block_scale_exp(np.array([0.0]))[0] == 0
    assert mx.block_scale_exp(np.array([2.0 ** -140]))[0] == 0           # limited below
    assert mx.block_scale_exp(np.array([2.0 ** 200]))[0] == 254          # limited above
    assert mx.block_scale_exp(np.array([1.0, 1.999, 2.0]))[0:3].tolist() == [119, 119, 120]


def _blocks(rng, n=64, K=128):
    mag = np.exp2(rng.uniform(-6, 6, (n, K // 32, 1)))
    v = rng.standard_normal((n, K // 32, 32)) * mag
    return v.reshape(n, K)


def test_quant_error_bound_and_saturation():
    """Each element within half an E4M3 quantum of its scaled value, except the
    block maxima that saturate (scaled magnitude >= 464), which become 448."""
    rng = np.random.default_rng(5)
    v = _blocks(rng)
    codes, X = mx.quant_mxfp8(v)
    s = np.repeat(np.exp2(X - 127.0), 32, axis=-1)
    a = np.abs(v) / s
    q = np.abs(mx.e4m3_to_f64(codes))
    e = np.floor(np.log2(np.where(a > 0, a, 1)))
    half = np.exp2(np.maximum(e, -6) - 4)
    ok = np.where(a >= 464, q == 448, np.abs(q - a) <= half)
    assert ok.all()
    assert np.array_equal(np.signbit(mx.e4m3_to_f64(codes)), np.signbit(v))


def test_quant_idempotent_and_scale_equivariant():
    rng = np.random.default_rng(11)
    v = _blocks(rng)
    q = mx.q_mxfp8(v)
    assert np.array_equal(mx.q_mxfp8(q), q)
    for k in (-20, -3, 5, 30):
        assert np.array_equal(mx.q_mxfp8(v * 2.0 ** k), q * 2.0 ** k)


def test_quant_blocks_are_independent_and_along_k():
    """Changing one block's values leaves the other blocks' results alone, and
    the scale follows the block's own maximum."""
    rng = np.random.default_rng(13)
    v = _blocks(rng, n=4)
    w = v.copy()
    w[:, 32:64] *= 1000.0
    qv, qw = mx.q_mxfp8(v), mx.q_mxfp8(w)
    assert np.array_equal(np.delete(qv, np.s_[32:64], axis=1), np.delete(qw, np.s_[32:64], axis=1))
    _, X = mx.quant_mxfp8(w)
    _, X0 = mx.quant_mxfp8(v)
    assert np.all(X[:, 1] > X0[:, 1]) and np.array_equal(X[:, [0, 2, 3]], X0[:, [0, 2, 3]])


# ---------------------------------------------------------------- the layer -------

def _int4_layer_inputs(seed):
    rng = np.random.default_rng(seed)
    D = synth.Dims(T=6, d=64, h=64, n_experts=8, experts_per_group=4, top_k=3, delta_rank=32,
                   lora_rank=4, quant_group=32)
    W = zero_weights(D)
    for name, lead, N, K in (("s_up", D.n_groups, D.h, D.d), ("s_dn", D.n_groups, D.d, D.h),
                             ("a_up", D.n_experts, D.delta_rank, D.d), ("b_up", D.n_experts, D.h, D.delta_rank),
                             ("a_dn", D.n_experts, D.delta_rank, D.h), ("b_dn", D.n_experts, D.d, D.delta_rank)):
        for i in range(lead):
            q = rng.integers(-4, 5, (N, K))
            q[:, ::D.gq(K)] = 4                      # every group's max is 4: power-of-two scale 2^-6
            set_int4(W, D, name, i, q * 2.0 ** -6)
    for name, shape in (("lora_up_u", (D.n_groups, D.lora_rank, D.d)), ("lora_up_v", (D.n_groups, D.h, D.lora_rank)),
                        ("lora_dn_u", (D.n_groups, D.lora_rank, D.h)), ("lora_dn_v", (D.n_groups, D.d, D.lora_rank))):
        W[name] = bf16_from(rng.standard_normal(shape) * 0.05)
    x = bf16_from(rng.standard_normal((D.T, D.d)))
    idx = np.array([rng.permutation(D.n_experts)[:D.top_k] for _ in range(D.T)])
    w = rng.dirichlet(np.ones(D.top_k), D.T)
    return D, W, x, idx, w


def test_mx_layer_without_quantiser_is_the_int4_layer():
    """With the int4 decoder and the quantiser switched off, the MX layer is the
    int4 layer's definition exactly (same rounding points, same order)."""
    for seed in (0, 1):
        D, W, x, idx, w = _int4_layer_inputs(seed)
        ref = layer.moe_forward(x, idx, w, W, D.experts_per_group, keep=True)
        got = mx.moe_forward_mx(x, idx, w, W, D.experts_per_group, keep=True, quantise=False,
                                dequant=codecs.dequant)
        for k in ("y", "o", "z1", "zl", "h", "a", "z2", "zl2"):
            assert np.array_equal(got[k], ref[k]), k


def test_mx_quantiser_changes_the_layer():
    D, W, x, idx, w = _int4_layer_inputs(2)
    a = mx.moe_forward_mx(x, idx, w, W, D.experts_per_group, quantise=False, dequant=codecs.dequant)["y"]
    b = mx.moe_forward_mx(x, idx, w, W, D.experts_per_group, quantise=True, dequant=codecs.dequant)["y"]
    assert not np.array_equal(a, b)
    assert np.max(np.abs(a - b)) < 0.1 * np.max(np.abs(a))


def _mx_diag_weights(n, diag):
    """One group of one expert, d = h = r = n: MXFP4 matrices with E2M1 code
    diag[name] on the diagonal (scale 2^0) for the names given, zero elsewhere;
    zero LoRA."""
    W = {}
    for name in ("s_up", "s_dn", "a_up", "b_up", "a_dn", "b_dn"):
        codes = np.zeros((n, n), dtype=np.uint8)
        if name in diag:
            codes[np.arange(n), np.arange(n)] = diag[name]
        W[name] = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)[None]
        W[name + "_scale"] = np.full((1, n // 128, n, 4), 127, dtype=np.int64)
    for name in ("lora_up_u", "lora_up_v", "lora_dn_u", "lora_dn_v"):
        W[name] = np.zeros((1, n, 8) if name.endswith("_v") else (1, 8, n), dtype=np.uint16)
    return W


def test_mx_quantiser_points_shared_path():
    """S_up = S_dn = I, no delta, no LoRA: h = Q(x), o = Q(R3(SiLU(Q(x))))."""
    rng = np.random.default_rng(17)
    n, T = 128, 3
    W = _mx_diag_weights(n, {"s_up": 2, "s_dn": 2})
    x = bf16_from(rng.standard_normal((T, n)) * 3)
    idx = np.zeros((T, 1), dtype=np.int64)
    out = mx.moe_forward_mx(x, idx, np.ones((T, 1)), W, 1, keep=True)
    X = codecs.bf16_to_f64(x)
    assert np.array_equal(out["h"][:, 0], mx.q_mxfp8(X))
    assert not np.array_equal(mx.q_mxfp8(X), X)
    assert np.array_equal(out["o"][:, 0], mx.q_mxfp8(codecs.rn_bf16(codecs.silu(mx.q_mxfp8(X)))))


def test_mx_quantiser_points_delta_path():
    """S = 0, A_up = A_dn = 1.5 I (code 3), B_up = B_dn = I: z1 = R1(1.5 Q(x))
    = 1.5 Q(x) exactly, h = z1 (z1 meets B_up unquantised, although Q(z1) != z1),
    a = R3(SiLU(h)), z2 = R4(1.5 Q(a)) = 1.5 Q(a), o = z2."""
    rng = np.random.default_rng(19)
    n, T = 128, 3
    W = _mx_diag_weights(n, {"a_up": 3, "b_up": 2, "a_dn": 3, "b_dn": 2})
    x = bf16_from(rng.standard_normal((T, n)) * 3)
    idx = np.zeros((T, 1), dtype=np.int64)
    out = mx.moe_forward_mx(x, idx, np.ones((T, 1)), W, 1, keep=True)
    X = codecs.bf16_to_f64(x)
    z1 = 1.5 * mx.q_mxfp8(X)
    assert np.array_equal(out["z1"][:, 0], z1)
    assert np.array_equal(out["h"][:, 0], z1)
    assert not np.array_equal(mx.q_mxfp8(z1), z1)
    a = codecs.rn_bf16(codecs.silu(z1))
    assert np.array_equal(out["a"][:, 0], a)
    z2 = 1.5 * mx.q_mxfp8(a)
    assert not np.array_equal(mx.q_mxfp8(a), a)
    assert np.array_equal(out["z2"][:, 0], z2)
    assert np.array_equal(out["o"][:, 0], z2)


def test_mx_lora_takes_unquantised_inputs():
    """S = 0, no delta; U_up, V_up, U_dn, V_dn pick / place the first 8
    coordinates (bf16 identity blocks): zl = x[:8], h[:8] = x[:8],
    zl2 = a[:8], o[:8] = a[:8]: the LoRA branch sees x and a, not Q(x), Q(a)."""
    rng = np.random.default_rng(23)
    n, T, rL = 128, 3, 8
    W = _mx_diag_weights(n, {})
    eye_u = np.zeros((1, rL, n), dtype=np.float32)
    eye_u[0, np.arange(rL), np.arange(rL)] = 1.0
    eye_v = np.transpose(eye_u, (0, 2, 1)).copy()
    W["lora_up_u"], W["lora_dn_u"] = bf16_from(eye_u), bf16_from(eye_u)
    W["lora_up_v"], W["lora_dn_v"] = bf16_from(eye_v), bf16_from(eye_v)
    x = bf16_from(rng.standard_normal((T, n)) * 3)
    idx = np.zeros((T, 1), dtype=np.int64)
    out = mx.moe_forward_mx(x, idx, np.ones((T, 1)), W, 1, keep=True)
    X = codecs.bf16_to_f64(x)
    assert not np.array_equal(mx.q_mxfp8(X)[:, :rL], X[:, :rL])
    assert np.array_equal(out["zl"][:, 0], X[:, :rL])
    assert np.array_equal(out["h"][:, 0, :rL], X[:, :rL])
    a = codecs.rn_bf16(codecs.silu(X[:, :rL]))
    assert np.array_equal(out["zl2"][:, 0], a)
    assert np.array_equal(out["o"][:, 0, :rL], a)


def test_synth_mxfp4_rounding_is_nearest():
    """The synthetic weights' storage rounding: each decoded weight is the
    nearest point of its block's MXFP4 grid (brute force over the 8 E2M1
    magnitudes, saturating at 6), and the block scale follows its maximum."""
    import torch
    w = torch.randn(4, 256, generator=torch.Generator().manual_seed(3)) * 0.02
    w[0, :32] = 0.0                                          # an all-zero block
    w[1, :32] = 0.001
    w[1, 6] = 0.012                                          # block max: X = floor(log2 .012) - 2 + 127 = 118
    w[1, 5] = 2.5 * 2.0 ** -9                                # then w / 2^-9 = 2.5, a tie between 2 and 3
    q, X = synth.quantize_mxfp4_torch(w)
    vals = mx.dequant_mxfp4(q.numpy(), synth.mx_scales_by_step(X).numpy(), 256)
    wn = w.double().numpy()
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    for n in range(4):
        for b in range(8):
            blk = wn[n, 32 * b:32 * b + 32]
            amax = np.abs(blk).max()
            x = int(X[n, b])
            if amax == 0:
                assert x == 0 and np.all(vals[n, 32 * b:32 * b + 32] == 0)
                continue
            assert 4 <= amax / 2.0 ** (x - 127) < 8
            for i, v in enumerate(blk):
                a = min(abs(v) / 2.0 ** (x - 127), 6.0)
                dd = np.abs(grid - a)
                cand = np.flatnonzero(dd == dd.min())
                j = cand[0] if len(cand) == 1 else [c for c in cand if c % 2 == 0][0]
                assert abs(vals[n, 32 * b + i]) == grid[j] * 2.0 ** (x - 127), (n, b, i)
    assert int(X[1, 0]) == 118 and vals[1, 5] == 2.0 * 2.0 ** -9
