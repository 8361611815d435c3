"""Router and expert layer, plain float64 (oracle; test infrastructure only).

What the pages fix
------------------
* Each token activates 10 of 512 experts (the Chinese commentary page, section
  "145B 为什么不用同时装进显存"; byteiota "Edge0-145B: Run a 145B Open-Source
  Model on Your Laptop", Not Compression - Architecture).
* Each group of 64 experts shares two large matrices; each expert keeps only a
  small set of its own parameters that capture its differences (launch post
  "Edge0-145B: Frontier AI Capabilities on Your Own Computer", Under the Hood,
  Architecture paragraph; HN digest page, Overcoming the Memory Wall; Portuguese
  page, "Como 145 bilhões de parâmetros cabem em 29 GB").
* The base is 4-bit and a LoRA branch runs in parallel with it (byteiota, The
  Three Pillars, Recover-LoRA paragraph).

Readings where the pages are silent (each listed in the design notes)
---------------------------------------------------------------------
* The two shared matrices are the up (d->h) and down (h->d) projections of a
  non-gated SiLU FFN; the expert difference is a rank-r additive delta on both,
  W_e = S_g + B_e A_e in N x K storage; the LoRA pair (U, V) is per group and per
  shared matrix, scale 1; expert e belongs to group e // 64.
* Router: linear, fp32 logits that are the correctly rounded value of the exact
  dot product (bf16 x bf16 products are exact; the sum is certified exact in
  f64 or rounded from the exact rational sum), plus an optional fp32 bias
  added in fp32.
  Top-k on the logits, descending, ties to the lower index; weights are the
  softmax renormalised over the k selected.
* Contract mode rounds to bf16 (RNE) at exactly five points, the inputs of the
  two low-rank products and of the two LoRA products (R1, R2, R4, R5) and the
  activation (R3); every other quantity stays float64.  Exact mode drops all
  five and equals the plain dense definition with W_e materialised.
* The output y is float (no rounding); y_t = sum_j w_tj o_tj in slot order.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np

from .codecs import bf16_to_f64, dequant, rn_bf16, rn_f32, silu


def _bf16_quantum_exp(v: np.ndarray) -> np.ndarray:
    """Exponent of a power of two that divides every bf16 value (its last
    significand bit): floor(log2|v|) - 7; +inf for zeros."""
    a = np.abs(v)
    out = np.full(a.shape, np.inf)
    nz = a > 0
    _, e = np.frexp(a[nz])           # a = m * 2**e, m in [0.5, 1)
    out[nz] = (e - 1) - 7
    return out


def _rn32_of_exact_sum(prods) -> float:
    """float32 value nearest to the exact sum of float64 terms (ties to even),
    computed with rationals; used only where the float64 certificate fails."""
    from fractions import Fraction
    S = sum((Fraction(p) for p in prods), Fraction(0))
    c = np.float32(float(S))
    lo = np.nextafter(c, np.float32(-np.inf))
    hi = np.nextafter(c, np.float32(np.inf))
    best = min((abs(Fraction(float(v)) - S), int(np.float32(v).view(np.uint32)) & 1, float(v))
               for v in (lo, c, hi))
    return best[2]


def _logits_rn32(X: np.ndarray, W: np.ndarray) -> np.ndarray:
    """RN32 of the exact sums L[t, e] = sum_j X[t, j] * W[e, j] (bf16 operands).

    Each product is exact in float64 (8-bit x 8-bit significands).  If every
    product of a dot is a multiple of 2**Q and sum_j |p_j| < 2**(53+Q), every
    partial sum in any order is an exactly representable float64, so the BLAS
    value is the exact sum and one float32 conversion rounds it correctly.
    Entries that fail this certificate are rounded from the exact rational sum.
    """
    L = X @ W.T
    M = np.abs(X) @ np.abs(W).T
    qx = _bf16_quantum_exp(X)
    qw = _bf16_quantum_exp(W)
    T = X.shape[0]
    Q = np.empty(L.shape)
    step = max(1, (1 << 22) // max(1, W.size))
    for t0 in range(0, T, step):
        Q[t0:t0 + step] = np.min(qx[t0:t0 + step, None, :] + qw[None, :, :], axis=2)
    ok = np.ones(L.shape, dtype=bool)          # Q = +inf: all products zero, L = 0
    fin = np.isfinite(Q)
    ok[fin] = M[fin] * (1.0 + 1e-9) < np.ldexp(1.0, (Q[fin] + 53).astype(np.int64))
    out = rn_f32(L)
    for t, e in np.argwhere(~ok):
        out[t, e] = _rn32_of_exact_sum((X[t] * W[e]).tolist())
    return out


def route(x_bits: np.ndarray, wr_bits: np.ndarray, bias: Optional[np.ndarray],
          k: int) -> Dict[str, np.ndarray]:
    """Router logits, top-k selection and renormalised softmax weights.

    x_bits [T][d] and wr_bits [E][d] are bf16 bit patterns; bias [E] float32 or
    None.  Returns logits [T][E] (float32 values as float64), idx [T][k] int32 in
    selection order, w [T][k] float64.
    """
    X = bf16_to_f64(x_bits)
    W = bf16_to_f64(wr_bits)
    logits = _logits_rn32(X, W)
    if bias is not None:
        logits = rn_f32(logits + np.asarray(bias, dtype=np.float32).astype(np.float64)[None, :])
    idx, w = select_topk(logits, k)
    return {"logits": logits, "idx": idx, "w": w}


def select_topk(logits: np.ndarray, k: int):
    """Top-k by logit, descending, ties (including +0 / -0) to the lower index,
    and the softmax renormalised over the selected k (float64)."""
    # a stable sort of -logit keeps equal keys in index order
    order = np.argsort(-logits, axis=1, kind="stable")
    idx = order[:, :k].astype(np.int32)
    sel = np.take_along_axis(logits, idx, axis=1)
    u = np.exp(sel - sel[:, :1])
    w = u / u.sum(axis=1, keepdims=True)
    return idx, w


def _group_tensors(W: dict, g: int, d: int, h: int):
    Sup = dequant(W["s_up"][g], W["s_up_scale"][g], d)          # [h][d]
    Sdn = dequant(W["s_dn"][g], W["s_dn_scale"][g], h)          # [d][h]
    Uup = bf16_to_f64(W["lora_up_u"][g])                        # [rL][d]
    Vup = bf16_to_f64(W["lora_up_v"][g])                        # [h][rL]
    Udn = bf16_to_f64(W["lora_dn_u"][g])                        # [rL][h]
    Vdn = bf16_to_f64(W["lora_dn_v"][g])                        # [d][rL]
    return Sup, Sdn, Uup, Vup, Udn, Vdn


def _expert_tensors(W: dict, e: int, d: int, h: int, r: int):
    Aup = dequant(W["a_up"][e], W["a_up_scale"][e], d)          # [r][d]
    Bup = dequant(W["b_up"][e], W["b_up_scale"][e], r)          # [h][r]
    Adn = dequant(W["a_dn"][e], W["a_dn_scale"][e], h)          # [r][h]
    Bdn = dequant(W["b_dn"][e], W["b_dn_scale"][e], r)          # [d][r]
    return Aup, Bup, Adn, Bdn


def moe_forward(x_bits: np.ndarray, idx: np.ndarray, w: np.ndarray, W: dict,
                experts_per_group: int, mode: str = "contract",
                keep: bool = False) -> Dict[str, np.ndarray]:
    """Expert layer output y [T][d] (float64) for routed tokens.

    For token t and selected slot j with expert e in group g (contract mode):
        h  = S_up_g x + B_up_e R1(A_up_e x) + V_up_g R2(U_up_g x)
        a  = R3(SiLU(h))
        o  = S_dn_g a + B_dn_e R4(A_dn_e a) + V_dn_g R5(U_dn_g a)
        y_t = sum_{j=0..k-1} w_tj o_tj
    where every weight is its exact dequantised value and R = round to bf16.
    ``mode="exact"`` drops R1..R5.  Rows are batched per group and per expert
    for speed only; each row's arithmetic is the per-row definition above.

    W holds host arrays in the documented layouts (uint8 packed int4, uint16
    fp16-scale bits, uint16 bf16 bits).  With keep=True the per-slot
    intermediates are returned too (z1, zl, h, a, z2, zl2, o: [T][k][...]).
    """
    if mode not in ("contract", "exact"):
        raise ValueError(mode)
    R = rn_bf16 if mode == "contract" else (lambda v: v)
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

    O = np.zeros((T, k, d))
    inter = {}
    if keep:
        inter = {n: np.zeros((T, k, s)) for n, s in
                 (("z1", r), ("zl", rL), ("h", h), ("a", h), ("z2", r), ("zl2", rL))}

    grp = idx // P
    for g in range(n_groups):
        tt, jj = np.nonzero(grp == g)          # rows of group g, in (t, j) order
        if tt.size == 0:
            continue
        Sup, Sdn, Uup, Vup, Udn, Vdn = _group_tensors(W, g, d, h)
        Xg = X[tt]
        zl = R(Xg @ Uup.T)                                     # R2
        H = Xg @ Sup.T + zl @ Vup.T
        ee = idx[tt, jj]
        z1_all = np.zeros((tt.size, r))
        for e in np.unique(ee):
            m = ee == e
            Aup, Bup, _, _ = _expert_tensors(W, int(e), d, h, r)
            z1 = R(Xg[m] @ Aup.T)                              # R1
            z1_all[m] = z1
            H[m] += z1 @ Bup.T
        A = R(silu(H))                                         # R3
        zl2 = R(A @ Udn.T)                                     # R5
        Og = A @ Sdn.T + zl2 @ Vdn.T
        z2_all = np.zeros((tt.size, r))
        for e in np.unique(ee):
            m = ee == e
            _, _, Adn, Bdn = _expert_tensors(W, int(e), d, h, r)
            z2 = R(A[m] @ Adn.T)                               # R4
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
    for j in range(k):                                        # slot order
        y += wf[:, j:j + 1] * O[:, j, :]
    out = {"y": y, "o": O}
    out.update(inter)
    return out


def residual(x_bits: np.ndarray, y: np.ndarray) -> np.ndarray:
    """Residual between stacked layers: x' = RN_bf16(x + y), returned as bf16 bits.

    The layers are stacked 48 deep (byteiota "Edge0-145B: Run a 145B Open-Source
    Model on Your Laptop", Not Compression - Architecture); the residual form is
    a stated reading.  x (bf16) + y (float32 values) is exact in float64 for the
    layer's value ranges, so one bf16 rounding of it is the definition.
    """
    v = rn_bf16(bf16_to_f64(x_bits) + np.asarray(y, dtype=np.float64))
    return (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def layer_forward(x_bits, wr_bits, bias, W, experts_per_group, k, mode="contract", keep=False):
    """route() followed by moe_forward() on the routed experts."""
    rt = route(x_bits, wr_bits, bias, k)
    fw = moe_forward(x_bits, rt["idx"], rt["w"], W, experts_per_group, mode=mode, keep=keep)
    fw.update(rt)
    return fw
