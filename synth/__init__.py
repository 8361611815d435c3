"""Seeded synthetic inputs for the shared-matrix MoE layer.

This module is shared by the CPU oracle (tests only) and by the GPU path's tests
and benchmark.  It holds no arithmetic of the layer itself: it draws activations,
router weights and expert weights, rounds them to the storage formats (bf16
activations, int4 + fp16-scale weights, bf16 LoRA factors) and packs them in the
byte layout that the C-ABI documents.  Nothing here routes, dequantises or
multiplies.

Shapes follow the workloads the pages describe: 512 experts per layer with 10
active per token and groups of 64 experts sharing two large matrices
("Edge0-145B: Frontier AI Capabilities on Your Own Computer", Under the Hood,
Architecture paragraph; byteiota "Edge0-145B: Run a 145B Open-Source Model on
Your Laptop", Not Compression - Architecture), 48 layers (same byteiota section),
a 4-bit base with a parallel bf16 Recover-LoRA branch (byteiota, The Three
Pillars, Recover-LoRA paragraph), speculative verification of several tokens
per weight read (launch post, Under the Hood, Scheduling paragraph) and a 16K
prefill (byteiota, Benchmark Numbers).

Random streams
--------------
* activations x, router weights W_r: numpy PCG64 seeded from
  ``SeedSequence([cfg_id, layer, tensor_id, seed])`` - always drawn on the host,
  so routing inputs are the same whichever device the weights live on;
* int4 / bf16 expert tensors: ``torch.Generator(device)`` seeded from the same
  kind of SeedSequence.  The values depend on the device's generator (CPU and
  GPU streams differ) but are deterministic for a device; parity always feeds
  the identical bytes to both sides.
"""
from __future__ import annotations

import dataclasses
import json
import os
from typing import Dict, Optional

import numpy as np

__all__ = [
    "Dims", "CONFIGS", "config", "make_activations", "make_router",
    "make_weights", "quantize_int4_torch", "bf16_bits_from_f32",
    "skew_bias_table", "WEIGHT_STD", "make_weights_mx", "quantize_mxfp4_torch",
]

WEIGHT_STD = 0.02  # std of every expert weight before quantisation


@dataclasses.dataclass(frozen=True)
class Dims:
    """Layer shape.  Weights are stored N x K (out x in); K is packed for int4."""
    T: int
    d: int
    h: int
    n_experts: int
    experts_per_group: int
    top_k: int
    delta_rank: int
    lora_rank: int
    quant_group: int

    @property
    def n_groups(self) -> int:
        return self.n_experts // self.experts_per_group

    def gq(self, K: int) -> int:
        """Effective quantisation group along K: min(quant_group, K)."""
        return min(self.quant_group, K)

    def with_T(self, T: int) -> "Dims":
        return dataclasses.replace(self, T=T)


@dataclasses.dataclass(frozen=True)
class Config:
    cfg_id: int
    name: str
    dims: Dims
    router_std: float
    skew: bool = False      # bias groups 0-1 so that 48 of 80 picks land there
    layers: int = 1


_FULL = dict(d=4096, h=8192, n_experts=512, experts_per_group=64, top_k=10,
             delta_rank=128, lora_rank=16, quant_group=128)

CONFIGS: Dict[int, Config] = {
    0: Config(0, "tiny T=4", Dims(T=4, d=256, h=512, n_experts=64, experts_per_group=64,
                                   top_k=4, delta_rank=8, lora_rank=4, quant_group=32),
              router_std=0.02),
    1: Config(1, "decode T=1", Dims(T=1, **_FULL), router_std=0.02),
    2: Config(2, "verify T=8 skewed", Dims(T=8, **_FULL), router_std=0.02, skew=True),
    3: Config(3, "prefill T=16384", Dims(T=16384, **_FULL), router_std=1.0 / 64.0),
    4: Config(4, "48-layer stack T=8", Dims(T=8, **_FULL), router_std=0.02, layers=48),
    # small shapes for the MXFP4 variant (rank 128, several groups, T past the decode range)
    5: Config(5, "mx small T=96", Dims(T=96, d=512, h=1024, n_experts=64, experts_per_group=8,
                                       top_k=4, delta_rank=128, lora_rank=16, quant_group=32),
              router_std=0.02),
}


def config(cfg_id: int) -> Config:
    return CONFIGS[cfg_id]


# tensor ids for the seed sequences
_TID = {
    "x": 1, "w_router": 2,
    "s_up": 10, "s_dn": 11, "a_up": 12, "b_up": 13, "a_dn": 14, "b_dn": 15,
    "lora_up_u": 20, "lora_up_v": 21, "lora_dn_u": 22, "lora_dn_v": 23,
}


def _seedseq(cfg_id: int, layer: int, name: str, seed: int) -> np.random.SeedSequence:
    return np.random.SeedSequence([cfg_id, layer, _TID[name], seed])


def _torch_seed(cfg_id: int, layer: int, name: str, seed: int) -> int:
    st = _seedseq(cfg_id, layer, name, seed).generate_state(2, np.uint32)
    return int((int(st[0]) << 31) ^ int(st[1])) & ((1 << 63) - 1)


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round-to-nearest-even) and return the bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    if np.any((u & 0x7F800000) == 0x7F800000):
        raise ValueError("non-finite input")
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def make_activations(cfg_id: int, seed: int, T: Optional[int] = None, layer: int = 0) -> np.ndarray:
    """x ~ N(0, 1) rounded to bf16: uint16 bits [T][d]."""
    cfg = CONFIGS[cfg_id]
    T = cfg.dims.T if T is None else T
    rng = np.random.Generator(np.random.PCG64(_seedseq(cfg_id, layer, "x", seed)))
    x = rng.standard_normal((T, cfg.dims.d), dtype=np.float32)
    return bf16_bits_from_f32(x)


def make_router(cfg_id: int, seed: int, layer: int = 0, with_skew: bool = True):
    """Router weights W_r [E][d] as bf16 bits and the optional fp32 bias [E].

    The bias is only used by the skewed verify workload: a constant beta added to
    every expert of groups 0 and 1, calibrated per (seed, layer) by a committed
    script so that exactly 48 of the 80 top-10 picks of the T=8 batch fall in those
    two groups (60 %).
    """
    cfg = CONFIGS[cfg_id]
    D = cfg.dims
    rng = np.random.Generator(np.random.PCG64(_seedseq(cfg_id, layer, "w_router", seed)))
    w = rng.standard_normal((D.n_experts, D.d), dtype=np.float32) * np.float32(cfg.router_std)
    bits = bf16_bits_from_f32(w)
    bias = None
    if cfg.skew and with_skew:
        beta = skew_bias_table().get((seed, layer))
        if beta is None:
            raise KeyError(f"no calibrated skew bias for seed={seed} layer={layer}; "
                           "run tests/golden/make_skew_bias.py")
        bias = np.zeros(D.n_experts, dtype=np.float32)
        bias[: 2 * D.experts_per_group] = np.float32(beta)
    return bits, bias


_SKEW_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                          "tests", "golden", "c2_skew_bias.json")


def skew_bias_table() -> Dict[tuple, float]:
    if not os.path.exists(_SKEW_PATH):
        return {}
    with open(_SKEW_PATH) as f:
        data = json.load(f)
    return {(int(e["seed"]), int(e["layer"])): float(e["beta"]) for e in data["entries"]}


# ----------------------------------------------------------------------------------
# expert weights (torch, on the requested device)
# ----------------------------------------------------------------------------------

def quantize_int4_torch(w, gq: int):
    """Symmetric int4 quantisation along the last axis in groups of ``gq``.

    s = fp16(absmax / 7) per group, q = clamp(round_half_even(w / s), -8, 7)
    (q = 0 where s = 0).  Returns (packed uint8 [..., K/2], fp16 scale bits as
    int16 [..., K/gq]).  Byte i of a row holds element 2i in its low nibble and
    element 2i+1 in its high nibble, both two's complement.
    """
    import torch
    K = w.shape[-1]
    assert K % gq == 0 and K % 2 == 0
    lead = w.shape[:-1]
    wg = w.reshape(*lead, K // gq, gq)
    s16 = (wg.abs().amax(dim=-1) / 7.0).to(torch.float16)
    sf = s16.to(torch.float32).unsqueeze(-1)
    q = torch.where(sf > 0, torch.round(wg / torch.where(sf > 0, sf, torch.ones_like(sf))),
                    torch.zeros_like(wg))
    q = q.clamp_(-8, 7).to(torch.int16).reshape(*lead, K)
    nib = (q & 0xF).to(torch.uint8)
    packed = nib[..., 0::2] | (nib[..., 1::2] << 4)
    return packed.contiguous(), s16.view(torch.int16).contiguous()


def _int4_tensor(name, shape, gq, cfg_id, layer, seed, device, zero=False):
    import torch
    if zero:
        K = shape[-1]
        return (torch.zeros(*shape[:-1], K // 2, dtype=torch.uint8, device=device),
                torch.zeros(*shape[:-1], K // gq, dtype=torch.int16, device=device))
    g = torch.Generator(device=device)
    g.manual_seed(_torch_seed(cfg_id, layer, name, seed))
    # draw and quantise one leading slice at a time to bound temporary memory
    qs, ss = [], []
    for i in range(shape[0]):
        w = torch.randn(*shape[1:], generator=g, device=device, dtype=torch.float32) * WEIGHT_STD
        q, s = quantize_int4_torch(w, gq)
        qs.append(q)
        ss.append(s)
    return torch.stack(qs).contiguous(), torch.stack(ss).contiguous()


def _bf16_tensor(name, shape, cfg_id, layer, seed, device, zero=False):
    import torch
    if zero:
        return torch.zeros(*shape, dtype=torch.int16, device=device)
    g = torch.Generator(device=device)
    g.manual_seed(_torch_seed(cfg_id, layer, name, seed))
    w = torch.randn(*shape, generator=g, device=device, dtype=torch.float32) * WEIGHT_STD
    return w.to(torch.bfloat16).view(torch.int16).contiguous()


def make_weights(cfg_id: int, seed: int, layer: int = 0, device="cpu",
                 zero_delta: bool = False, zero_lora: bool = False) -> dict:
    """All int4 / bf16 tensors of one layer as torch tensors on ``device``.

    Layouts (N x K, K packed two per byte for int4, scales [N][K/Gq_eff]):
      s_up [G][h][d/2]   s_up_scale [G][h][d/Gq]     shared up   (per group)
      s_dn [G][d][h/2]   s_dn_scale [G][d][h/Gq]     shared down (per group)
      a_up [E][r][d/2]   b_up [E][h][r/2]            delta up    (per expert)
      a_dn [E][r][h/2]   b_dn [E][d][r/2]            delta down  (per expert)
      lora_up_u [G][rL][d]  lora_up_v [G][h][rL]     bf16 bits   (per group)
      lora_dn_u [G][rL][h]  lora_dn_v [G][d][rL]
    """
    D = CONFIGS[cfg_id].dims
    G, E, d, h, r, rL = D.n_groups, D.n_experts, D.d, D.h, D.delta_rank, D.lora_rank
    out = {}
    args = (cfg_id, layer, seed, device)
    out["s_up"], out["s_up_scale"] = _int4_tensor("s_up", (G, h, d), D.gq(d), *args)
    out["s_dn"], out["s_dn_scale"] = _int4_tensor("s_dn", (G, d, h), D.gq(h), *args)
    out["a_up"], out["a_up_scale"] = _int4_tensor("a_up", (E, r, d), D.gq(d), *args, zero=zero_delta)
    out["b_up"], out["b_up_scale"] = _int4_tensor("b_up", (E, h, r), D.gq(r), *args, zero=zero_delta)
    out["a_dn"], out["a_dn_scale"] = _int4_tensor("a_dn", (E, r, h), D.gq(h), *args, zero=zero_delta)
    out["b_dn"], out["b_dn_scale"] = _int4_tensor("b_dn", (E, d, r), D.gq(r), *args, zero=zero_delta)
    out["lora_up_u"] = _bf16_tensor("lora_up_u", (G, rL, d), *args, zero=zero_lora)
    out["lora_up_v"] = _bf16_tensor("lora_up_v", (G, h, rL), *args, zero=zero_lora)
    out["lora_dn_u"] = _bf16_tensor("lora_dn_u", (G, rL, h), *args, zero=zero_lora)
    out["lora_dn_v"] = _bf16_tensor("lora_dn_v", (G, d, rL), *args, zero=zero_lora)
    return out


# ----------------------------------------------------------------------------------
# MXFP4 expert weights (the microscaling variant of the layer)
# ----------------------------------------------------------------------------------

MX_BLOCK = 32
_E2M1_GRID = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def quantize_mxfp4_torch(w):
    """Round float32 weights to MXFP4 along the last axis (OCP Microscaling
    Formats v1.0): per block of 32, E8M0 byte X = floor(log2(amax)) - 2 + 127
    (2 = the exponent of E2M1's largest value), limited to 0..254 (0 for an
    all-zero block); each element is the E2M1 value nearest to w / 2^(X-127),
    ties to the even code, saturated at 6.  Returns (codes packed two per byte,
    element 2i in the low nibble: uint8 [..., K/2]; E8M0 bytes uint8 [..., K/32]).
    This is the storage rounding of the synthetic weights, not a step of the layer."""
    import torch
    K = w.shape[-1]
    assert K % MX_BLOCK == 0
    lead = w.shape[:-1]
    b = w.reshape(*lead, K // MX_BLOCK, MX_BLOCK).to(torch.float32)
    amax = b.abs().amax(dim=-1)
    _, ex = torch.frexp(amax)                        # amax = m * 2^ex, m in [0.5, 1)
    X = torch.where(amax > 0, (ex - 1 - 2 + 127).clamp(0, 254), torch.zeros_like(ex))
    scale = torch.pow(torch.tensor(2.0, device=w.device), (X - 127).to(torch.float32))
    a = (b.abs() / scale.unsqueeze(-1)).clamp(max=6.0)
    grid = torch.tensor(_E2M1_GRID, device=w.device)
    mids = (grid[:-1] + grid[1:]) / 2
    idx = (a.unsqueeze(-1) > mids).sum(-1)           # nearest, the lower one at a tie
    tie = (a.unsqueeze(-1) == mids).any(-1)
    idx = torch.where(tie & (idx % 2 == 1), idx + 1, idx)
    code = (idx | torch.where(b < 0, 8, 0)).to(torch.uint8).reshape(*lead, K)
    packed = code[..., 0::2] | (code[..., 1::2] << 4)
    return packed.contiguous(), X.to(torch.uint8).contiguous()


def mx_scales_by_step(X):
    """E8M0 bytes [..., N, K/32] -> the stored K-step-major layout [..., K/128, N, 4]."""
    lead, N, nb = X.shape[:-2], X.shape[-2], X.shape[-1]
    assert nb % 4 == 0
    return X.reshape(*lead, N, nb // 4, 4).transpose(-3, -2).contiguous()


def _mxfp4_tensor(name, shape, cfg_id, layer, seed, device, zero=False):
    import torch
    if zero:
        K = shape[-1]
        return (torch.zeros(*shape[:-1], K // 2, dtype=torch.uint8, device=device),
                torch.zeros(shape[0], K // 128, shape[1], 4, dtype=torch.uint8, device=device))
    g = torch.Generator(device=device)
    g.manual_seed(_torch_seed(cfg_id, layer, name, seed))
    qs, ss = [], []
    for i in range(shape[0]):
        w = torch.randn(*shape[1:], generator=g, device=device, dtype=torch.float32) * WEIGHT_STD
        q, s = quantize_mxfp4_torch(w)
        qs.append(q)
        ss.append(mx_scales_by_step(s))
    return torch.stack(qs).contiguous(), torch.stack(ss).contiguous()


def make_weights_mx(cfg_id: int, seed: int, layer: int = 0, device="cpu",
                    zero_delta: bool = False, zero_lora: bool = False) -> dict:
    """The MXFP4 variant of make_weights: the same draws (same streams, same
    N(0, 0.02^2)), rounded to MXFP4 instead of int4.  Layouts: codes as the
    int4 ones ([N][K/2], two per byte), E8M0 scales uint8 stored K-step-major
    [K/128][N][4] under the same "_scale" names; LoRA factors bf16 as in
    make_weights."""
    D = CONFIGS[cfg_id].dims
    G, E, d, h, r, rL = D.n_groups, D.n_experts, D.d, D.h, D.delta_rank, D.lora_rank
    out = {}
    args = (cfg_id, layer, seed, device)
    out["s_up"], out["s_up_scale"] = _mxfp4_tensor("s_up", (G, h, d), *args)
    out["s_dn"], out["s_dn_scale"] = _mxfp4_tensor("s_dn", (G, d, h), *args)
    out["a_up"], out["a_up_scale"] = _mxfp4_tensor("a_up", (E, r, d), *args, zero=zero_delta)
    out["b_up"], out["b_up_scale"] = _mxfp4_tensor("b_up", (E, h, r), *args, zero=zero_delta)
    out["a_dn"], out["a_dn_scale"] = _mxfp4_tensor("a_dn", (E, r, h), *args, zero=zero_delta)
    out["b_dn"], out["b_dn_scale"] = _mxfp4_tensor("b_dn", (E, d, r), *args, zero=zero_delta)
    out["lora_up_u"] = _bf16_tensor("lora_up_u", (G, rL, d), *args, zero=zero_lora)
    out["lora_up_v"] = _bf16_tensor("lora_up_v", (G, h, rL), *args, zero=zero_lora)
    out["lora_dn_u"] = _bf16_tensor("lora_dn_u", (G, rL, h), *args, zero=zero_lora)
    out["lora_dn_v"] = _bf16_tensor("lora_dn_v", (G, d, rL), *args, zero=zero_lora)
    return out


WEIGHT_NAMES = ("s_up", "s_up_scale", "s_dn", "s_dn_scale", "a_up", "a_up_scale",
                "b_up", "b_up_scale", "a_dn", "a_dn_scale", "b_dn", "b_dn_scale",
                "lora_up_u", "lora_up_v", "lora_dn_u", "lora_dn_v")


def weights_to_numpy(wts: dict) -> dict:
    """Host copies with the unsigned views the oracle decodes (uint8 / uint16)."""
    out = {}
    for k, v in wts.items():
        a = v.detach().cpu().numpy()
        if a.dtype == np.int16:
            a = a.view(np.uint16)
        out[k] = a
    return out
