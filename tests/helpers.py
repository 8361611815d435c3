"""Test helpers: hand-built weight sets in the documented byte layouts."""
import numpy as np

from oracle import codecs
import synth

TINY = synth.Dims(T=6, d=16, h=32, n_experts=8, experts_per_group=4, top_k=3,
                  delta_rank=4, lora_rank=2, quant_group=8)


def int4_from(q, s, gq):
    """q int array [..., N, K], s float array [..., N, K/gq] -> packed, fp16 bits."""
    q = np.asarray(q, dtype=np.int8)
    s = np.asarray(s, dtype=np.float16)
    assert s.shape[-1] * gq == q.shape[-1]
    return codecs.pack_int4(q), s.view(np.uint16)


def bf16_from(v):
    return synth.bf16_bits_from_f32(np.asarray(v, dtype=np.float32))


def zero_weights(D):
    """All-zero weight set with the right shapes (host numpy)."""
    G, E, d, h, r, rL = D.n_groups, D.n_experts, D.d, D.h, D.delta_rank, D.lora_rank
    W = {}
    for name, lead, N, K in (("s_up", G, h, d), ("s_dn", G, d, h), ("a_up", E, r, d),
                             ("b_up", E, h, r), ("a_dn", E, r, h), ("b_dn", E, d, r)):
        W[name] = np.zeros((lead, N, K // 2), dtype=np.uint8)
        W[name + "_scale"] = np.zeros((lead, N, K // D.gq(K)), dtype=np.uint16)
    W["lora_up_u"] = np.zeros((G, rL, d), dtype=np.uint16)
    W["lora_up_v"] = np.zeros((G, h, rL), dtype=np.uint16)
    W["lora_dn_u"] = np.zeros((G, rL, h), dtype=np.uint16)
    W["lora_dn_v"] = np.zeros((G, d, rL), dtype=np.uint16)
    return W


def set_int4(W, D, name, index, dense):
    """Store an exactly representable dense float matrix [N][K] as int4 with one
    power-of-two scale per group (the group's max |value| / 4 rounded up to 2^k)."""
    dense = np.asarray(dense, dtype=np.float64)
    N, K = dense.shape
    gq = D.gq(K)
    g = dense.reshape(N, K // gq, gq)
    amax = np.abs(g).max(-1)
    s = np.where(amax > 0, 2.0 ** np.ceil(np.log2(np.maximum(amax, 1e-30) / 4)), 1.0)
    q = g / s[..., None]
    assert np.all(q == np.rint(q)) and np.all(np.abs(q) <= 7), "not representable"
    p, sb = int4_from(q.reshape(N, K).astype(np.int8), s, gq)
    W[name][index] = p
    W[name + "_scale"][index] = sb


def random_weights(D, seed, zero_delta=False, zero_lora=False):
    """Random weights through the input generator on the CPU, as host arrays."""
    import torch as _t
    out = {}
    G, E, d, h, r, rL = D.n_groups, D.n_experts, D.d, D.h, D.delta_rank, D.lora_rank
    tg = _t.Generator().manual_seed(int(np.random.default_rng(seed).integers(1 << 62)))
    for name, lead, N, K, zero in (("s_up", G, h, d, False), ("s_dn", G, d, h, False),
                                   ("a_up", E, r, d, zero_delta), ("b_up", E, h, r, zero_delta),
                                   ("a_dn", E, r, h, zero_delta), ("b_dn", E, d, r, zero_delta)):
        w = _t.randn(lead, N, K, generator=tg) * synth.WEIGHT_STD
        if zero:
            w.zero_()
        p, s = synth.quantize_int4_torch(w, D.gq(K))
        out[name] = p.numpy()
        out[name + "_scale"] = s.numpy().view(np.uint16)
    for name, shape in (("lora_up_u", (G, rL, d)), ("lora_up_v", (G, h, rL)),
                        ("lora_dn_u", (G, rL, h)), ("lora_dn_v", (G, d, rL))):
        w = _t.randn(*shape, generator=tg) * synth.WEIGHT_STD
        if zero_lora:
            w.zero_()
        out[name] = w.to(_t.bfloat16).view(_t.int16).numpy().view(np.uint16)
    return out


def random_x(T, d, seed):
    rng = np.random.default_rng(seed)
    return synth.bf16_bits_from_f32(rng.standard_normal((T, d), dtype=np.float32))


def random_router(E, d, seed, std=0.3):
    rng = np.random.default_rng(seed + 1000)
    return synth.bf16_bits_from_f32(rng.standard_normal((E, d), dtype=np.float32) * np.float32(std))
