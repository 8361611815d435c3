"""Host-side checks of the C-ABI library (no GPU needed).

The library must load and export every function that include/edge_moe.h
declares; validation that happens before any device call (dims, null or
misaligned pointers, workspace size) is exercised with fake addresses that the
library never dereferences.
"""
import ctypes
import dataclasses
import os
import re

import pytest

import shared_matrix_expert_amd as em
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "edge_moe.h")


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(edge_moe_[a-z_]+)\s*\(", src)))


def test_header_declares_the_binding_set():
    assert set(header_functions()) == set(em.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = em.load()
    for name in header_functions():
        assert hasattr(lib, name), name
        ctypes.cast(getattr(lib, name), ctypes.c_void_p)


def test_abi_version_and_status_strings():
    assert em.edge_moe_abi_version() == 5
    for st in (0, -1, -2, -3, -4):
        assert em.status_string(st)
    assert em.status_string(7) == "unknown status"


def test_workspace_bytes_valid_and_invalid():
    for cfg in (0, 1, 2, 3):
        D = synth.config(cfg).dims
        n = em.edge_moe_workspace_bytes(D)
        assert n > 0 and n % 256 == 0
    D = synth.config(1).dims
    assert em.edge_moe_workspace_bytes(D.with_T(2)) > em.edge_moe_workspace_bytes(D.with_T(1))
    bad = [D.with_T(0), synth.Dims(**{**D.__dict__, "n_experts": 500}),
           synth.Dims(**{**D.__dict__, "top_k": 600}),
           synth.Dims(**{**D.__dict__, "d": 4000}),
           synth.Dims(**{**D.__dict__, "quant_group": 48}),
           synth.Dims(**{**D.__dict__, "lora_rank": 3})]
    for b in bad:
        assert em.edge_moe_workspace_bytes(b) == 0, b


class _Fake:
    """Stand-in for a device tensor: an address that is never dereferenced."""
    def __init__(self, addr, nbytes=1 << 40):
        self.addr, self.nbytes = addr, nbytes


def _call_forward(D, x=0x10000, idx=0x20000, w=0x30000, y=0x40000, ws=0x100000, ws_bytes=None,
                  wptr=0x50000):
    lib = em.load()
    cw = em.CWeights(*([wptr] * len(em._WEIGHT_FIELDS)))
    if ws_bytes is None:
        ws_bytes = em.edge_moe_workspace_bytes(D)
    return lib.edge_moe_forward(ctypes.byref(em.cdims(D)), x, idx, w, ctypes.byref(cw), y, ws,
                                ws_bytes, None)


def test_forward_validation_before_device():
    D = synth.config(2).dims
    assert _call_forward(D, x=None) == em.EDGE_MOE_EINVAL
    assert _call_forward(D, x=0x10008) == em.EDGE_MOE_EINVAL          # not 16-byte aligned
    assert _call_forward(D, y=0x40004) == em.EDGE_MOE_EINVAL
    assert _call_forward(D, wptr=None) == em.EDGE_MOE_EINVAL
    assert _call_forward(D, ws=None) == em.EDGE_MOE_EWORKSPACE
    assert _call_forward(D, ws=0x100010) == em.EDGE_MOE_EINVAL        # not 256-byte aligned
    assert _call_forward(D, ws_bytes=1024) == em.EDGE_MOE_EWORKSPACE
    assert _call_forward(D.with_T(0)) == em.EDGE_MOE_EINVAL
    assert _call_forward(synth.Dims(**{**D.__dict__, "delta_rank": 12})) == em.EDGE_MOE_EUNSUPPORTED
    assert _call_forward(synth.Dims(**{**D.__dict__, "top_k": 40})) == em.EDGE_MOE_EUNSUPPORTED
    lib = em.load()
    assert lib.edge_moe_forward(None, 0x10000, 0x20000, 0x30000, None, 0x40000, 0x100000, 1 << 30,
                                None) == em.EDGE_MOE_EINVAL


def test_route_validation_before_device():
    lib = em.load()
    D = synth.config(2).dims
    cd = ctypes.byref(em.cdims(D))
    ok = dict(x=0x10000, wr=0x20000, b=None, idx=0x30000, w=0x40000, lg=None, ws=0x100000,
              nb=em.edge_moe_workspace_bytes(D))

    def call(**kw):
        a = {**ok, **kw}
        return lib.edge_moe_route(cd, a["x"], a["wr"], a["b"], a["idx"], a["w"], a["lg"], a["ws"],
                                  a["nb"], None)
    assert call(x=None) == em.EDGE_MOE_EINVAL
    assert call(wr=0x20002) == em.EDGE_MOE_EINVAL
    assert call(idx=0x30002) == em.EDGE_MOE_EINVAL
    assert call(b=0x50001) == em.EDGE_MOE_EINVAL
    assert call(ws=None) == em.EDGE_MOE_EWORKSPACE
    assert call(nb=16) == em.EDGE_MOE_EWORKSPACE


def test_binding_requires_the_library(tmp_path):
    em_mod = em
    saved = em_mod._lib
    try:
        em_mod._lib = None
        with pytest.raises(RuntimeError):
            em_mod.load(str(tmp_path / "missing.so"))
    finally:
        em_mod._lib = saved


def test_copy_validation_before_any_device_call():
    lib = em.load()
    base = 1 << 40                          # never dereferenced: rejected first
    cases = [(base + 8, base + 4096, 64),   # misaligned dst
             (base, base + 4096 + 8, 64),   # misaligned src
             (base, base + 4096, 24),       # not a multiple of 16
             (base, base + 32, 64),         # overlapping
             (0, base, 64)]                 # null
    for dst, src, n in cases:
        assert lib.edge_moe_copy(ctypes.c_void_p(dst), ctypes.c_void_p(src), n, None) == em.EDGE_MOE_EINVAL


def test_mfma_peak_validation_before_any_device_call():
    lib = em.load()
    base = 1 << 40                          # never dereferenced: rejected first
    for out, blocks, iters in [(0, 1, 1), (base + 2, 1, 1), (base, 0, 1), (base, 1, 0), (base, -4, 8)]:
        assert lib.edge_moe_mfma_peak(ctypes.c_void_p(out), blocks, iters, None) == em.EDGE_MOE_EINVAL


def test_tiled_weights_all_or_none():
    """The decode-tiled codes are optional: s_up's and s_dn's both or neither,
    a_up's on its own; aligned; only for shapes the layout takes."""
    lib = em.load()
    D = synth.config(2).dims

    def fwd(dims, ptrs):
        cw = em.CWeights(*ptrs)
        return lib.edge_moe_forward(ctypes.byref(em.cdims(dims)), 0x10000, 0x20000, 0x30000, ctypes.byref(cw),
                                    0x40000, 0x100000, em.edge_moe_workspace_bytes(dims), None)
    assert fwd(D, [0x50000] * 16 + [0x60000, None, None, None]) == em.EDGE_MOE_EINVAL      # s_up without s_dn
    assert fwd(D, [0x50000] * 16 + [0x60008, 0x70000, None, None]) == em.EDGE_MOE_EINVAL   # not 16-byte aligned
    assert fwd(D, [0x50000] * 16 + [None, None, 0x80008, None]) == em.EDGE_MOE_EINVAL      # a_up not aligned
    assert fwd(D, [0x50000] * 16 + [None, None, None, 0x90008]) == em.EDGE_MOE_EINVAL      # a_dn not aligned
    T0 = synth.config(0).dims                                                              # quant groups of 32
    assert fwd(T0, [0x50000] * 20) == em.EDGE_MOE_EUNSUPPORTED
    D64 = synth.Dims(**{**D.__dict__, "delta_rank": 64})                                  # a_dn needs r = 128
    assert fwd(D64, [0x50000] * 16 + [None, None, None, 0x90000]) == em.EDGE_MOE_EUNSUPPORTED


def test_tile_shared_validation_before_device():
    lib = em.load()
    D = synth.config(2).dims
    cd = ctypes.byref(em.cdims(D))
    base = 1 << 40
    big = 1 << 34                                       # beyond any matrix of these dims
    ok = dict(which=0, sq=base, dq=base + big)

    def call(**kw):
        a = {**ok, **kw}
        return lib.edge_moe_tile_shared(cd, a["which"], ctypes.c_void_p(a["sq"]), ctypes.c_void_p(a["dq"]), None)
    assert call(which=4) == em.EDGE_MOE_EINVAL
    assert call(which=-1) == em.EDGE_MOE_EINVAL
    assert call(sq=base + 8) == em.EDGE_MOE_EINVAL                 # not 16-byte aligned
    assert call(dq=base + 64) == em.EDGE_MOE_EINVAL                # overlaps the source
    assert call(sq=0) == em.EDGE_MOE_EINVAL
    T0 = synth.config(0).dims                                      # quant groups of 32
    assert lib.edge_moe_tile_shared(ctypes.byref(em.cdims(T0)), 0, ctypes.c_void_p(base),
                                    ctypes.c_void_p(base + big), None) == em.EDGE_MOE_EUNSUPPORTED
    D8 = synth.Dims(**{**D.__dict__, "delta_rank": 64})            # a_up rank not a multiple of 128
    assert lib.edge_moe_tile_shared(ctypes.byref(em.cdims(D8)), 2, ctypes.c_void_p(base),
                                    ctypes.c_void_p(base + big), None) == em.EDGE_MOE_EUNSUPPORTED
    assert lib.edge_moe_tile_shared(ctypes.byref(em.cdims(D8)), 3, ctypes.c_void_p(base),
                                    ctypes.c_void_p(base + big), None) == em.EDGE_MOE_EUNSUPPORTED


def test_mx_shapes_and_validation_before_any_device_call():
    """The MX variant takes rank 128, d and h multiples of 256, lora rank 8..32
    (multiple of 8); other shapes get no workspace size and EUNSUPPORTED."""
    D = synth.config(5).dims
    assert em.edge_moe_workspace_bytes_mx(D) > em.edge_moe_workspace_bytes(D) > 0
    for bad in (dict(delta_rank=64), dict(d=384), dict(h=640), dict(lora_rank=4), dict(lora_rank=40)):
        Db = dataclasses.replace(D, **bad)
        assert em.edge_moe_workspace_bytes_mx(Db) == 0, bad
    lib = em.load()
    base = 1 << 40
    W = em.CWeightsMX(*([base] * 16))
    dims = em.cdims(dataclasses.replace(D, delta_rank=64))
    st = lib.edge_moe_forward_mx(ctypes.byref(dims), base, base, base, ctypes.byref(W), base, base,
                                 1 << 40, None, None)
    assert st == em.EDGE_MOE_EUNSUPPORTED
    W2 = em.CWeightsMX(*([base] * 15 + [base + 8]))       # misaligned LoRA factor
    st = lib.edge_moe_forward_mx(ctypes.byref(em.cdims(D)), base, base, base, ctypes.byref(W2), base, base,
                                 1 << 40, None, None)
    assert st == em.EDGE_MOE_EINVAL
    st = lib.edge_moe_forward_mx(ctypes.byref(em.cdims(D)), base, base, base, ctypes.byref(W), base, base,
                                 16, None, None)
    assert st == em.EDGE_MOE_EWORKSPACE


def test_prefetch_validation_before_any_device_call():
    D = synth.config(2).dims
    lib = em.load()
    base = 1 << 40
    W = em.CWeights(*([base] * 16 + [None] * 4))
    ws_n = em.edge_moe_prefetch_ws_bytes()
    assert ws_n >= 64 * 1024
    dims = ctypes.byref(em.cdims(D))
    call = lambda groups, n, parts, ws, nbytes: lib.edge_moe_prefetch(dims, ctypes.byref(W), groups, n, parts,  # noqa: E731
                                                                      ws, nbytes, None)
    assert call(base, 4, 0, base, ws_n) == em.EDGE_MOE_EINVAL          # no part
    assert call(base, 4, 4, base, ws_n) == em.EDGE_MOE_EINVAL          # unknown part
    assert call(base, -1, 1, base, ws_n) == em.EDGE_MOE_EINVAL         # negative count
    assert call(base, 33, 1, base, ws_n) == em.EDGE_MOE_EINVAL         # more than 4 G entries
    assert call(base + 2, 4, 1, base, ws_n) == em.EDGE_MOE_EINVAL      # misaligned list
    assert call(base, 4, 1, base, ws_n - 4) == em.EDGE_MOE_EWORKSPACE  # scratch too small
    assert call(base, 4, 1, None, ws_n) == em.EDGE_MOE_EWORKSPACE
    assert call(None, 0, 1, base, ws_n) == em.EDGE_MOE_OK              # nothing to read: no device call


def test_cache_validation_before_any_device_call():
    lib = em.load()
    st = em.CCacheStats()
    assert lib.edge_moe_cache_map(None, 1, None, None, None, ctypes.byref(st)) == em.EDGE_MOE_EINVAL
    assert lib.edge_moe_cache_prefetch(None, 1, None, None, None) == em.EDGE_MOE_EINVAL
    assert lib.edge_moe_cache_totals(None, ctypes.byref(st)) == em.EDGE_MOE_EINVAL
    assert lib.edge_moe_cache_slot_of(None, 0) == -2
    lib.edge_moe_cache_destroy(None)
    D = synth.config(1).dims
    fake = em.CExpertTensors(*([0x1000] * 8 + [None, None]))
    c = lib.edge_moe_cache_create(ctypes.byref(em.cdims(D)), 8, ctypes.byref(fake), None)   # plans only
    assert c
    lib.edge_moe_cache_destroy(c)
    assert not lib.edge_moe_cache_create(ctypes.byref(em.cdims(D)), 8, ctypes.byref(em.CExpertTensors()), None)
    assert not lib.edge_moe_cache_create(ctypes.byref(em.cdims(D)), 0, ctypes.byref(fake), None)
    assert not lib.edge_moe_cache_create(ctypes.byref(em.cdims(D)), 65, ctypes.byref(fake), None)
    for bad in (dict(d=100), dict(quant_group=48), dict(delta_rank=12), dict(n_experts=500)):
        Db = dataclasses.replace(D, **bad)
        assert not lib.edge_moe_cache_create(ctypes.byref(em.cdims(Db)), 8, ctypes.byref(fake), None), bad
