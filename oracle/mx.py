"""Microscaling (MX) variant of the expert layer, plain float64 (oracle; test
infrastructure only).

The pages ship 4-bit builds of the model for their hardware (byteiota
"Edge0-145B: Run a 145B Open-Source Model on Your Laptop", What You Need to Run
It: an NVFP4 file and a 3-bit file).  The MI355X-native 4-bit floating format
is MXFP4 as defined by the Open Compute Project's Microscaling Formats (MX)
specification v1.0, whose definitions this module follows:

* a block of 32 consecutive elements shares one E8M0 scale, the power of two
  2^(X - 127) for the byte X (X = 255 is NaN and never produced here);
* E2M1 (FP4) elements: sign bit 3, exponent bits 2..1 with bias 1, mantissa bit
  0; exponent 0 is subnormal (0 or 0.5); magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6;
* E4M3 (FP8) elements: sign bit 7, exponent bits 6..3 with bias 7, mantissa
  bits 2..0; exponent 0 is subnormal (m/8 * 2^-6); no infinities, S.1111.111
  is NaN, so the largest magnitude is 448.

Readings (each listed in the design notes, "MX variant"):

* Weights (S_up, S_dn, A_up, B_up, A_dn, B_dn) are stored as MXFP4 along K
  (two codes per byte, element 2i in the low nibble of byte i); the E8M0
  scales of an N x K matrix are stored K-step-major, [K/128][N][4]: for each
  128-element step of K, the four block scales of every row in turn (the
  layout the library's tiled products load one step at a time).  LoRA
  factors stay bf16.
* The inputs of the large MXFP4 products are quantised to MXFP8 (E4M3) along
  K first: the token rows x (for S_up and A_up) and the activation rows a (for
  S_dn and A_dn), where the matrix cores multiply FP4 by FP8.  The rank-r
  inputs z1 and z2 (already rounded to bf16 by R1 and R4) meet B_up and B_dn
  unquantised: a second rounding there, to 3-bit mantissas, would make every
  delta jump with the last bit of z1 or z2, and those products are a few
  percent of the work.  The LoRA products take the unquantised x and a, as in
  the int4 layer.
* The block scale is the specification's: X = floor(log2(amax)) - 8 + 127
  (8 = the exponent of E4M3's largest normal), limited to 0..254, X = 0 for an
  all-zero block; each element is v / 2^(X - 127) rounded to the nearest E4M3
  value, ties to the even code, and magnitudes above 448 saturate to 448 (the
  specification leaves the overflow behaviour to the implementation).
* The rest of the layer is the int4 layer's definition (oracle/layer.py):
  roundings R1..R5 to bf16 at the same points, SiLU, fp64 elsewhere, y in slot
  order.

Pins (tests/test_oracle_mx.py): both element codecs exhaustively against
their bit-field definitions and against each other's grids; the E4M3 encoder
against a brute-force nearest-value search; the block scale's range property;
quantisation error bounds and scale equivariance; the layer against the int4
oracle on inputs for which every quantiser is the identity (so the MX mode
reduces to a layer the int4 pins already fix), against the same layer with
the quantiser disabled (which must then differ), and identity-structured
weights that show where the quantiser sits and where it does not.
"""
from __future__ import annotations

from typing import Dict

import numpy as np

from .codecs import bf16_to_f64, rn_bf16, silu

MX_BLOCK = 32
E4M3_MAX = 448.0
E2M1_MAX = 6.0


# ------------------------------------------------------------------ element codecs --

def e2m1_to_f64(codes: np.ndarray) -> np.ndarray:
    """4-bit E2M1 codes -> float64 (bit fields: s | ee | m, exponent bias 1)."""
    c = np.asarray(codes).astype(np.int64) & 0xF
    s = np.where(c & 0x8, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = (c & 0x1).astype(np.float64)
    mag = np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * np.exp2(e.astype(np.float64) - 1.0))
    return s * mag


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    """8-bit E4M3 codes -> float64 (s | eeee | mmm, bias 7; S.1111.111 -> NaN)."""
    c = np.asarray(codes).astype(np.int64) & 0xFF
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return s * mag


def e8m0_to_f64(x: np.ndarray) -> np.ndarray:
    """E8M0 scale bytes -> 2^(X - 127) (255 -> NaN)."""
    xi = np.asarray(x).astype(np.int64)
    return np.where(xi == 255, np.nan, np.exp2(xi.astype(np.float64) - 127.0))


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """float64 values -> E4M3 codes: nearest representable magnitude, ties to
    the even code (the even mantissa), |v| above 448 saturated to 448; the
    sign bit is the sign of v (so -0.0 and negatives that round to zero give
    0x80).  Inputs must be finite."""
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("non-finite input")
    a = np.abs(v)
    sign = np.where(np.signbit(v), 0x80, 0x00)
    # the quantum of the binade: 2^(e - 3) for normals (e >= -6), 2^-9 below
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    # guard floor(log2) against rounding at exact powers of two
    e = np.where(np.exp2(e) > a, e - 1, e)
    e = np.where(np.exp2(e + 1) <= a, e + 1, e)
    quantum = np.exp2(np.maximum(e, -6.0) - 3.0)
    n = np.rint(a / quantum)                      # round half to even on the quantum grid
    q = np.minimum(n * quantum, E4M3_MAX)
    q = np.where(a > 0, q, 0.0)
    # encode the (exactly representable) magnitude q
    sub = q < 2.0 ** -6
    code_sub = np.rint(q / 2.0 ** -9).astype(np.int64)
    eq = np.floor(np.log2(np.where(q > 0, q, 1.0)))
    eq = np.where(np.exp2(eq) > q, eq - 1, eq)
    man = np.rint((q / np.exp2(eq) - 1.0) * 8.0).astype(np.int64)
    code_norm = ((eq.astype(np.int64) + 7) << 3) | man
    code = np.where(sub, code_sub, code_norm)
    return (code | sign).astype(np.uint8)


# ------------------------------------------------------------------ MX blocks ------

def unpack_fp4(packed: np.ndarray) -> np.ndarray:
    """Packed bytes [..., K/2] -> E2M1 codes [..., K] (element 2i in the low nibble)."""
    p = np.asarray(packed).astype(np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def scales_by_row(scales: np.ndarray) -> np.ndarray:
    """E8M0 scales stored [K/128][N][4] -> [N][K/32] (row n's block scales in K order)."""
    s = np.asarray(scales)
    steps, N, four = s.shape
    assert four == 4
    return np.transpose(s, (1, 0, 2)).reshape(N, 4 * steps)


def dequant_mxfp4(packed: np.ndarray, scales: np.ndarray, K: int) -> np.ndarray:
    """MXFP4 matrix [N][K/2] codes + E8M0 scales [K/128][N][4] -> float64
    [N][K], exactly (every E2M1 value times a power of two is a float64)."""
    c = unpack_fp4(packed)
    assert c.shape[-1] == K and K % 128 == 0
    vals = e2m1_to_f64(c)
    sc = e8m0_to_f64(scales_by_row(scales))
    return vals * np.repeat(sc, MX_BLOCK, axis=-1)


def block_scale_exp(amax: np.ndarray) -> np.ndarray:
    """E8M0 byte of an MXFP8 block with largest magnitude amax:
    floor(log2(amax)) - 8 + 127 limited to 0..254; 0 for amax = 0."""
    a = np.asarray(amax, dtype=np.float64)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.where(np.exp2(e) > a, e - 1, e)
    e = np.where(np.exp2(e + 1) <= a, e + 1, e)
    x = np.clip(e - 8 + 127, 0, 254)
    return np.where(a > 0, x, 0).astype(np.int64)


def quant_mxfp8(v: np.ndarray):
    """Quantise rows [..., K] (K a multiple of 32) to MXFP8 along the last axis.
    Returns (E4M3 codes [..., K] uint8, E8M0 bytes [..., K/32] int64)."""
    v = np.asarray(v, dtype=np.float64)
    K = v.shape[-1]
    assert K % MX_BLOCK == 0
    blocks = v.reshape(v.shape[:-1] + (K // MX_BLOCK, MX_BLOCK))
    x = block_scale_exp(np.abs(blocks).max(axis=-1))
    scaled = blocks / np.exp2(x.astype(np.float64) - 127.0)[..., None]
    codes = e4m3_encode(scaled).reshape(v.shape)
    return codes, x


def q_mxfp8(v: np.ndarray) -> np.ndarray:
    """The value an MXFP8 round trip gives: decode(quant_mxfp8(v))."""
    codes, x = quant_mxfp8(v)
    K = codes.shape[-1]
    return e4m3_to_f64(codes) * np.repeat(np.exp2(x.astype(np.float64) - 127.0), MX_BLOCK, axis=-1)[..., :K]


# ------------------------------------------------------------------ the layer ------

def moe_forward_mx(x_bits: np.ndarray, idx: np.ndarray, w: np.ndarray, W: dict,
                   experts_per_group: int, keep: bool = False, quantise: bool = True,
                   dequant=None) -> Dict[str, np.ndarray]:
    """Expert layer with MXFP4 shared and delta matrices.

    For token t and slot j with expert e in group g:
        x~ = Q(x)                                    (MXFP8 of the token row)
        h  = S_up_g x~ + B_up_e R1(A_up_e x~) + V_up_g R2(U_up_g x)
        a  = R3(SiLU(h));  a~ = Q(a)
        o  = S_dn_g a~ + B_dn_e R4(A_dn_e a~) + V_dn_g R5(U_dn_g a)
        y_t = sum_{j=0..k-1} w_tj o_tj                (slot order)
    with every weight its exact MXFP4 value and Q the MXFP8 round trip along
    the product's K.  ``quantise=False`` replaces Q by the identity (used by
    the pins only).  ``dequant`` overrides the weight decoder (pins only: the
    int4 decoder turns this function into the int4 layer's definition).
    Rows are batched per group and per expert for speed only.
    """
    Q = q_mxfp8 if quantise else (lambda v: v)
    dq = dequant_mxfp4 if dequant is None else dequant
    X = bf16_to_f64(x_bits)
    T, d = X.shape
    k = idx.shape[1]
    P = experts_per_group
    h = W["s_up"].shape[1]
    r = W["a_up"].shape[1]
    rL = W["lora_up_u"].shape[1]
    n_groups = W["s_up"].shape[0]
    idx = np.asarray(idx)
    if idx.min(initial=0) < 0 or idx.max(initial=0) >= n_groups * P:
        raise ValueError("expert index out of range")
    for t in range(T):
        if len(set(idx[t].tolist())) != k:
            raise ValueError("duplicate expert in a token's selection")
    Xq = Q(X)
    O = np.zeros((T, k, d))
    inter = {}
    if keep:
        inter = {n: np.zeros((T, k, s)) for n, s in
                 (("z1", r), ("zl", rL), ("h", h), ("a", h), ("z2", r), ("zl2", rL))}
    grp = idx // P
    for g in range(n_groups):
        tt, jj = np.nonzero(grp == g)
        if tt.size == 0:
            continue
        Sup = dq(W["s_up"][g], W["s_up_scale"][g], d)
        Sdn = dq(W["s_dn"][g], W["s_dn_scale"][g], h)
        Uup = bf16_to_f64(W["lora_up_u"][g])
        Vup = bf16_to_f64(W["lora_up_v"][g])
        Udn = bf16_to_f64(W["lora_dn_u"][g])
        Vdn = bf16_to_f64(W["lora_dn_v"][g])
        Xg, Xgq = X[tt], Xq[tt]
        zl = rn_bf16(Xg @ Uup.T)                                    # R2 (unquantised x)
        H = Xgq @ Sup.T + zl @ Vup.T
        ee = idx[tt, jj]
        z1_all = np.zeros((tt.size, r))
        for e in np.unique(ee):
            m = ee == e
            Aup = dq(W["a_up"][e], W["a_up_scale"][e], d)
            Bup = dq(W["b_up"][e], W["b_up_scale"][e], r)
            z1 = rn_bf16(Xgq[m] @ Aup.T)                            # R1
            z1_all[m] = z1
            H[m] += z1 @ Bup.T
        A = rn_bf16(silu(H))                                        # R3
        Aq = Q(A)
        zl2 = rn_bf16(A @ Udn.T)                                    # R5 (unquantised a)
        Og = Aq @ Sdn.T + zl2 @ Vdn.T
        z2_all = np.zeros((tt.size, r))
        for e in np.unique(ee):
            m = ee == e
            Adn = dq(W["a_dn"][e], W["a_dn_scale"][e], h)
            Bdn = dq(W["b_dn"][e], W["b_dn_scale"][e], r)
            z2 = rn_bf16(Aq[m] @ Adn.T)                             # R4
            z2_all[m] = z2
            Og[m] += z2 @ Bdn.T
        O[tt, jj] = Og
        if keep:
            inter["z1"][tt, jj] = z1_all
            inter["zl"][tt, jj] = zl
            inter["h"][tt, jj] = H
            inter["a"][tt, jj] = A
            inter["z2"][tt, jj] = z2_all
            inter["zl2"][tt, jj] = zl2
    wf = np.asarray(w, dtype=np.float64)
    y = np.zeros((T, d))
    for j in range(k):
        y += wf[:, j:j + 1] * O[:, j, :]
    out = {"y": y, "o": O}
    out.update(inter)
    return out
