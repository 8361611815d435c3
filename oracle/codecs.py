"""Exact decoders and rounding helpers (oracle; test infrastructure only).

The pages state that the base model is stored as 4-bit integers ("Edge0-145B:
Run a 145B Open-Source Model on Your Laptop", The Three Pillars: SSD expert
streaming and Recover-LoRA paragraphs; the Chinese commentary page, section
"145B 为什么不用同时装进显存", calls it native 4-bit).  They give no encoding,
so the library fixes one (a stated reading): signed two's-complement nibbles,
element 2i in the low nibble of byte i and 2i+1 in the high nibble, one fp16
scale per group of ``Gq_eff = min(Gq, K)`` consecutive elements along K.  The
dequantised weight is q*s exactly (both factors are small enough that the f64
product is exact).

Pins (tests/test_oracle_codecs.py): exhaustive nibble tables, library
conversions for bf16/fp16, constructed RNE ties.
"""
from __future__ import annotations

import numpy as np

BF16_MAX = float.fromhex("0x1.fep127")
F32_MIN_NORMAL = 2.0 ** -126


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly (bf16 is the top half of fp32)."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def fp16_to_f64(bits: np.ndarray) -> np.ndarray:
    """IEEE binary16 bit patterns (uint16) -> float64, exactly."""
    return np.asarray(bits).astype(np.uint16).view(np.float16).astype(np.float64)


def unpack_int4(packed: np.ndarray) -> np.ndarray:
    """Packed bytes [..., K/2] -> signed int8 values [..., K] in -8..7.

    Byte i carries element 2i in bits 0-3 and element 2i+1 in bits 4-7; a
    nibble v >= 8 stands for v - 16 (two's complement).
    """
    p = np.asarray(packed).astype(np.uint8)
    lo = (p & 0x0F).astype(np.int16)
    hi = (p >> 4).astype(np.int16)
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def pack_int4(q: np.ndarray) -> np.ndarray:
    """Inverse of unpack_int4 for values in -8..7 (used by the codec pins)."""
    q = np.asarray(q).astype(np.int16)
    if q.min(initial=0) < -8 or q.max(initial=0) > 7:
        raise ValueError("int4 out of range")
    n = (q & 0xF).astype(np.uint8)
    return (n[..., 0::2] | (n[..., 1::2] << 4)).astype(np.uint8)


def dequant(packed: np.ndarray, scale_bits: np.ndarray, K: int) -> np.ndarray:
    """W_hat[n, k] = q[n, k] * s[n, k // Gq_eff] in float64 (exact).

    ``scale_bits`` has shape [..., N, K/Gq_eff]; the group size is inferred as
    K / scale_bits.shape[-1].
    """
    q = unpack_int4(packed).astype(np.float64)
    assert q.shape[-1] == K, (q.shape, K)
    s = fp16_to_f64(scale_bits)
    ng = s.shape[-1]
    assert K % ng == 0
    gq = K // ng
    return q * np.repeat(s, gq, axis=-1)


def rn_bf16(v: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 value, ties to even.

    bf16 keeps 8 significant bits and fp32's exponent range, subnormals
    included.  With v = m * 2**e, m in [0.5, 1), a normal result is
    rint(m * 256) / 256 * 2**e (rint is half-to-even); below 2**-126 the grid
    is the fixed spacing 2**-133, so the result is rint(v * 2**133) * 2**-133.
    Deep stacks of layers reach that range (SiLU of a large negative
    pre-activation).  Overflow is asserted rather than handled.
    """
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("non-finite value at a bf16 rounding point")
    a = np.abs(v)
    if np.any(a >= BF16_MAX):
        raise ValueError("value outside the bf16 range")
    m, e = np.frexp(v)
    normal = np.ldexp(np.rint(m * 256.0) / 256.0, e)
    sub = np.ldexp(np.rint(np.ldexp(v, 133)), -133)
    return np.where(a < F32_MIN_NORMAL, sub, normal)


def rn_f32(v: np.ndarray) -> np.ndarray:
    """Round float64 to the nearest float32 (IEEE RNE), returned as float64."""
    return np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)


def silu(v: np.ndarray) -> np.ndarray:
    """SiLU(v) = v / (1 + exp(-v)) in float64 (the expert activation)."""
    v = np.asarray(v, dtype=np.float64)
    with np.errstate(over="ignore"):
        return v / (1.0 + np.exp(-v))
