"""Python binding of libedge_moe.so (the shared-matrix sparse-MoE expert layer).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  Functions carry the C names and take torch tensors that live on the
GPU (PyTorch provides device memory and streams here, nothing else); the
library is required - calls raise if it is not built.

    import shared_matrix_expert_amd as em
    ws = torch.empty(em.edge_moe_workspace_bytes(dims), dtype=torch.uint8, device="cuda")
    em.edge_moe_route(dims, x, w_router, bias, idx, w, None, ws)
    em.edge_moe_forward(dims, x, idx, w, weights, y, ws)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libedge_moe.so")

EDGE_MOE_OK = 0
EDGE_MOE_EINVAL = -1
EDGE_MOE_EUNSUPPORTED = -2
EDGE_MOE_EWORKSPACE = -3
EDGE_MOE_EHIP = -4

EXPORTED = ("edge_moe_workspace_bytes", "edge_moe_route", "edge_moe_forward",
            "edge_moe_forward_traced", "edge_moe_residual", "edge_moe_status_string",
            "edge_moe_abi_version", "edge_moe_copy", "edge_moe_tile_shared",
            "edge_moe_prof_enable", "edge_moe_prof_read", "edge_moe_prof_reset")


class CDims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("T", "d", "h", "n_experts", "experts_per_group", "top_k",
                 "delta_rank", "lora_rank", "quant_group")]


_WEIGHT_FIELDS = ("s_up_q", "s_up_scale", "s_dn_q", "s_dn_scale", "a_up_q", "a_up_scale",
                  "b_up_q", "b_up_scale", "a_dn_q", "a_dn_scale", "b_dn_q", "b_dn_scale",
                  "lora_up_u", "lora_up_v", "lora_dn_u", "lora_dn_v",
                  "s_up_t", "s_dn_t", "a_up_t")
# keys of the weight dicts made by the input generator -> struct fields (the
# last three, the decode-tiled codes, are optional)
_WEIGHT_KEYS = ("s_up", "s_up_scale", "s_dn", "s_dn_scale", "a_up", "a_up_scale",
                "b_up", "b_up_scale", "a_dn", "a_dn_scale", "b_dn", "b_dn_scale",
                "lora_up_u", "lora_up_v", "lora_dn_u", "lora_dn_v",
                "s_up_t", "s_dn_t", "a_up_t")
_OPTIONAL_KEYS = ("s_up_t", "s_dn_t", "a_up_t")


class CWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in _WEIGHT_FIELDS]


class CTrace(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("expert_offsets", "row_token", "row_slot", "act", "expert_out")]


class EdgeMoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: status {status} ({status_string(status)})")
        self.status = status


_lib: Optional[ctypes.CDLL] = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the shared library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m shared_matrix_expert_amd.build`")
    # PyTorch-ROCm ships its own HIP runtime; load it first so that the library
    # binds to the same runtime instance as the streams and memory it is given.
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    lib.edge_moe_workspace_bytes.argtypes = [ctypes.POINTER(CDims)]
    lib.edge_moe_workspace_bytes.restype = sz
    lib.edge_moe_route.argtypes = [ctypes.POINTER(CDims), vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.edge_moe_route.restype = i32
    lib.edge_moe_forward.argtypes = [ctypes.POINTER(CDims), vp, vp, vp, ctypes.POINTER(CWeights),
                                     vp, vp, sz, vp]
    lib.edge_moe_forward.restype = i32
    lib.edge_moe_forward_traced.argtypes = [ctypes.POINTER(CDims), vp, vp, vp,
                                            ctypes.POINTER(CWeights), vp, vp, sz, vp,
                                            ctypes.POINTER(CTrace)]
    lib.edge_moe_forward_traced.restype = i32
    lib.edge_moe_residual.argtypes = [ctypes.c_int32, ctypes.c_int32, vp, vp, vp, vp]
    lib.edge_moe_residual.restype = i32
    lib.edge_moe_copy.argtypes = [vp, vp, sz, vp]
    lib.edge_moe_copy.restype = i32
    lib.edge_moe_tile_shared.argtypes = [ctypes.POINTER(CDims), ctypes.c_int32, vp, vp, vp]
    lib.edge_moe_tile_shared.restype = i32
    lib.edge_moe_status_string.argtypes = [i32]
    lib.edge_moe_status_string.restype = ctypes.c_char_p
    lib.edge_moe_abi_version.argtypes = []
    lib.edge_moe_abi_version.restype = i32
    lib.edge_moe_prof_enable.argtypes = [i32]
    lib.edge_moe_prof_enable.restype = i32
    lib.edge_moe_prof_read.argtypes = [vp, vp, vp, i32]
    lib.edge_moe_prof_read.restype = i32
    lib.edge_moe_prof_reset.argtypes = []
    lib.edge_moe_prof_reset.restype = None
    _lib = lib
    return lib


def cdims(dims) -> CDims:
    return CDims(*(int(getattr(dims, f)) for f, _ in CDims._fields_))


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors passed to the library must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def cweights(weights: dict) -> CWeights:
    return CWeights(*(_ptr(weights.get(k) if k in _OPTIONAL_KEYS else weights[k]) for k in _WEIGHT_KEYS))


def edge_moe_tile_shared(dims, which, src_q, dst_q, stream=None) -> None:
    """Decode-tiled copy of the codes of s_up (which=0), s_dn (1) or a_up (2)."""
    st = load().edge_moe_tile_shared(ctypes.byref(cdims(dims)), int(which), _ptr(src_q), _ptr(dst_q),
                                     _stream(stream))
    if st != EDGE_MOE_OK:
        raise EdgeMoeError("edge_moe_tile_shared", st)


def tile_weights(dims, weights: dict, stream=None) -> dict:
    """A copy of the weight dict with the decode-tiled codes added (new device
    tensors of the sizes of s_up / s_dn / a_up; a_up only when its rank is a
    multiple of 128)."""
    import torch
    out = dict(weights)
    for which, key in ((0, "s_up"), (1, "s_dn"), (2, "a_up")):
        if which == 2 and dims.delta_rank % 128:
            continue
        q = torch.empty_like(weights[key])
        edge_moe_tile_shared(dims, which, weights[key], q, stream)
        out[key + "_t"] = q
    return out


def status_string(status: int) -> str:
    return load().edge_moe_status_string(int(status)).decode()


def edge_moe_copy(dst, src, stream=None) -> None:
    """Plain device copy of src into dst (same byte size), one library kernel."""
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != n:
        raise ValueError("edge_moe_copy: dst and src differ in size")
    st = load().edge_moe_copy(_ptr(dst), _ptr(src), n, _stream(stream))
    if st != EDGE_MOE_OK:
        raise EdgeMoeError("edge_moe_copy", st)


def edge_moe_abi_version() -> int:
    return int(load().edge_moe_abi_version())


def edge_moe_workspace_bytes(dims) -> int:
    return int(load().edge_moe_workspace_bytes(ctypes.byref(cdims(dims))))


def edge_moe_route(dims, x, w_router, bias, topk_idx, topk_w, logits_out, ws, stream=None) -> None:
    lib = load()
    st = lib.edge_moe_route(ctypes.byref(cdims(dims)), _ptr(x), _ptr(w_router), _ptr(bias),
                            _ptr(topk_idx), _ptr(topk_w), _ptr(logits_out), _ptr(ws),
                            ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream))
    if st != EDGE_MOE_OK:
        raise EdgeMoeError("edge_moe_route", st)


def edge_moe_forward(dims, x, topk_idx, topk_w, weights, y, ws, stream=None, trace=None) -> None:
    lib = load()
    cw = cweights(weights) if isinstance(weights, dict) else weights
    args = (ctypes.byref(cdims(dims)), _ptr(x), _ptr(topk_idx), _ptr(topk_w), ctypes.byref(cw),
            _ptr(y), _ptr(ws), ws.numel() * ws.element_size() if ws is not None else 0,
            _stream(stream))
    if trace is None:
        st = lib.edge_moe_forward(*args)
    else:
        tr = CTrace(*(_ptr(trace.get(n)) for n, _ in CTrace._fields_))
        st = lib.edge_moe_forward_traced(*args, ctypes.byref(tr))
    if st != EDGE_MOE_OK:
        raise EdgeMoeError("edge_moe_forward", st)


def edge_moe_residual(x, y, x_out, stream=None) -> None:
    T, d = x.shape
    st = load().edge_moe_residual(int(T), int(d), _ptr(x), _ptr(y), _ptr(x_out), _stream(stream))
    if st != EDGE_MOE_OK:
        raise EdgeMoeError("edge_moe_residual", st)


def edge_moe_prof_enable(on: bool) -> bool:
    return bool(load().edge_moe_prof_enable(1 if on else 0))


def edge_moe_prof_reset() -> None:
    load().edge_moe_prof_reset()


def edge_moe_prof_read() -> dict:
    """{kernel name: (launches, total ms)} accumulated since the last reset."""
    lib = load()
    n = lib.edge_moe_prof_read(None, None, None, 0)
    names = (ctypes.c_char * 64 * max(n, 1))()
    launches = (ctypes.c_int64 * max(n, 1))()
    total = (ctypes.c_double * max(n, 1))()
    n = lib.edge_moe_prof_read(ctypes.cast(names, ctypes.c_void_p), ctypes.cast(launches, ctypes.c_void_p),
                               ctypes.cast(total, ctypes.c_void_p), n)
    return {names[i].value.decode(): (int(launches[i]), float(total[i])) for i in range(n)}
