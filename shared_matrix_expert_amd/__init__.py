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
            "edge_moe_prof_enable", "edge_moe_prof_read", "edge_moe_prof_reset",
            "edge_moe_forward_noalloc", "edge_moe_forward_persistent", "edge_moe_mfma_peak",
            "edge_moe_workspace_bytes_mx", "edge_moe_forward_mx", "edge_moe_prefetch_ws_bytes",
            "edge_moe_prefetch", "edge_moe_cache_create", "edge_moe_cache_destroy", "edge_moe_cache_map",
            "edge_moe_cache_prefetch", "edge_moe_cache_totals", "edge_moe_cache_slot_of")


class CDims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("T", "d", "h", "n_experts", "experts_per_group", "top_k",
                 "delta_rank", "lora_rank", "quant_group")]


_WEIGHT_FIELDS = ("s_up_q", "s_up_scale", "s_dn_q", "s_dn_scale", "a_up_q", "a_up_scale",
                  "b_up_q", "b_up_scale", "a_dn_q", "a_dn_scale", "b_dn_q", "b_dn_scale",
                  "lora_up_u", "lora_up_v", "lora_dn_u", "lora_dn_v",
                  "s_up_t", "s_dn_t", "a_up_t", "a_dn_t")
# keys of the weight dicts made by the input generator -> struct fields (the
# last four, the decode-tiled and column-blocked codes, are optional)
_WEIGHT_KEYS = ("s_up", "s_up_scale", "s_dn", "s_dn_scale", "a_up", "a_up_scale",
                "b_up", "b_up_scale", "a_dn", "a_dn_scale", "b_dn", "b_dn_scale",
                "lora_up_u", "lora_up_v", "lora_dn_u", "lora_dn_v",
                "s_up_t", "s_dn_t", "a_up_t", "a_dn_t")
_OPTIONAL_KEYS = ("s_up_t", "s_dn_t", "a_up_t", "a_dn_t")


class CWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in _WEIGHT_FIELDS]


# the MX variant: E8M0 scale bytes in place of the fp16 scales, no tiled copies
_WEIGHT_FIELDS_MX = ("s_up_q", "s_up_e", "s_dn_q", "s_dn_e", "a_up_q", "a_up_e",
                     "b_up_q", "b_up_e", "a_dn_q", "a_dn_e", "b_dn_q", "b_dn_e",
                     "lora_up_u", "lora_up_v", "lora_dn_u", "lora_dn_v")


class CWeightsMX(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in _WEIGHT_FIELDS_MX]


# per-expert tensors that an expert cache streams (weight-dict keys, struct order)
EXPERT_TENSOR_KEYS = ("a_up", "a_up_scale", "b_up", "b_up_scale", "a_dn", "a_dn_scale",
                      "b_dn", "b_dn_scale", "a_up_t", "a_dn_t")


class CExpertTensors(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("a_up_q", "a_up_scale", "b_up_q", "b_up_scale", "a_dn_q", "a_dn_scale",
                 "b_dn_q", "b_dn_scale", "a_up_t", "a_dn_t")]


class CCacheStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("hits", "misses", "evictions", "bytes_copied")]


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
    lib.edge_moe_forward_persistent.argtypes = [ctypes.POINTER(CDims), vp, vp, vp, ctypes.POINTER(CWeights),
                                                vp, vp, sz, vp, ctypes.POINTER(CTrace)]
    lib.edge_moe_forward_persistent.restype = i32
    lib.edge_moe_prefetch_ws_bytes.argtypes = []
    lib.edge_moe_prefetch_ws_bytes.restype = sz
    lib.edge_moe_prefetch.argtypes = [ctypes.POINTER(CDims), ctypes.POINTER(CWeights), vp, i32, i32, vp, sz, vp]
    lib.edge_moe_prefetch.restype = i32
    lib.edge_moe_workspace_bytes_mx.argtypes = [ctypes.POINTER(CDims)]
    lib.edge_moe_workspace_bytes_mx.restype = sz
    lib.edge_moe_forward_mx.argtypes = [ctypes.POINTER(CDims), vp, vp, vp, ctypes.POINTER(CWeightsMX),
                                        vp, vp, sz, vp, ctypes.POINTER(CTrace)]
    lib.edge_moe_forward_mx.restype = i32
    lib.edge_moe_mfma_peak.argtypes = [vp, ctypes.c_int32, ctypes.c_int32, vp]
    lib.edge_moe_mfma_peak.restype = i32
    lib.edge_moe_forward_noalloc.argtypes = [ctypes.POINTER(CDims), vp, vp, vp, ctypes.POINTER(CWeights), vp, vp]
    lib.edge_moe_forward_noalloc.restype = i32
    lib.edge_moe_cache_create.argtypes = [ctypes.POINTER(CDims), i32, ctypes.POINTER(CExpertTensors),
                                          ctypes.POINTER(CExpertTensors)]
    lib.edge_moe_cache_create.restype = vp
    lib.edge_moe_cache_destroy.argtypes = [vp]
    lib.edge_moe_cache_destroy.restype = None
    lib.edge_moe_cache_map.argtypes = [vp, i32, vp, vp, vp, ctypes.POINTER(CCacheStats)]
    lib.edge_moe_cache_map.restype = i32
    lib.edge_moe_cache_prefetch.argtypes = [vp, i32, vp, vp, ctypes.POINTER(CCacheStats)]
    lib.edge_moe_cache_prefetch.restype = i32
    lib.edge_moe_cache_totals.argtypes = [vp, ctypes.POINTER(CCacheStats)]
    lib.edge_moe_cache_totals.restype = i32
    lib.edge_moe_cache_slot_of.argtypes = [vp, i32]
    lib.edge_moe_cache_slot_of.restype = i32
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


def cweights_mx(weights: dict) -> CWeightsMX:
    """Struct of an MX weight dict (keys as the int4 ones: codes under the
    matrix name, E8M0 bytes under "<name>_scale")."""
    return CWeightsMX(*(_ptr(weights[k]) for k in _WEIGHT_KEYS[:16]))


def edge_moe_prefetch_ws_bytes() -> int:
    return int(load().edge_moe_prefetch_ws_bytes())


def edge_moe_prefetch(dims, weights, groups, parts, ws, stream=None) -> None:
    """Read the listed groups' shared matrices (parts: 1 S_up, 2 S_dn, 3 both)
    so that a later layer call finds them in the memory-side cache."""
    n = 0 if groups is None else int(groups.numel())
    st = load().edge_moe_prefetch(ctypes.byref(cdims(dims)), ctypes.byref(cweights(weights)),
                                  _ptr(groups) if n else None, n, int(parts), _ptr(ws),
                                  ws.numel() * ws.element_size(), _stream(stream))
    if st != EDGE_MOE_OK:
        raise EdgeMoeError("edge_moe_prefetch", st)


def edge_moe_workspace_bytes_mx(dims) -> int:
    return int(load().edge_moe_workspace_bytes_mx(ctypes.byref(cdims(dims))))


def edge_moe_forward_mx(dims, x, topk_idx, topk_w, weights, y, ws, stream=None, trace=None) -> None:
    """The expert layer with MXFP4 shared and delta matrices."""
    tr = None if trace is None else ctypes.byref(CTrace(*(_ptr(trace.get(n)) for n, _ in CTrace._fields_)))
    st = load().edge_moe_forward_mx(ctypes.byref(cdims(dims)), _ptr(x), _ptr(topk_idx), _ptr(topk_w),
                                    ctypes.byref(cweights_mx(weights)), _ptr(y), _ptr(ws),
                                    ws.numel() * ws.element_size(), _stream(stream), tr)
    if st != EDGE_MOE_OK:
        raise EdgeMoeError("edge_moe_forward_mx", st)


def edge_moe_tile_shared(dims, which, src_q, dst_q, stream=None) -> None:
    """Decode-tiled copy of the codes of s_up (which=0), s_dn (1) or a_up (2),
    or the column-blocked copy of a_dn (3)."""
    st = load().edge_moe_tile_shared(ctypes.byref(cdims(dims)), int(which), _ptr(src_q), _ptr(dst_q),
                                     _stream(stream))
    if st != EDGE_MOE_OK:
        raise EdgeMoeError("edge_moe_tile_shared", st)


def tile_weights(dims, weights: dict, stream=None) -> dict:
    """A copy of the weight dict with the decode-tiled codes added (new device
    tensors of the sizes of s_up / s_dn / a_up / a_dn; a_up only when its rank
    is a multiple of 128, a_dn only when its rank is 128)."""
    import torch
    out = dict(weights)
    for which, key in ((0, "s_up"), (1, "s_dn"), (2, "a_up"), (3, "a_dn")):
        if which == 2 and dims.delta_rank % 128:
            continue
        if which == 3 and dims.delta_rank != 128:
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


def edge_moe_forward_persistent(dims, x, topk_idx, topk_w, weights, y, ws, stream=None, trace=None) -> None:
    """The decode / verify layer as one persistent launch (T <= 8, stored copies
    of kinds 0-3 in `weights`); trace as edge_moe_forward's."""
    tr = None if trace is None else CTrace(*(_ptr(trace.get(n)) for n, _ in CTrace._fields_))
    st = load().edge_moe_forward_persistent(ctypes.byref(cdims(dims)), _ptr(x), _ptr(topk_idx), _ptr(topk_w),
                                            ctypes.byref(cweights(weights)), _ptr(y), _ptr(ws), ws.numel() * ws.element_size(),
                                            _stream(stream), None if tr is None else ctypes.byref(tr))
    if st != EDGE_MOE_OK:
        raise EdgeMoeError("edge_moe_forward_persistent", st)


def edge_moe_mfma_peak(out, blocks, iters, stream=None) -> None:
    """Matrix-core calibration launch (blocks * 4 * iters * 8 * 16384 flops)."""
    st = load().edge_moe_mfma_peak(_ptr(out), int(blocks), int(iters), _stream(stream))
    if st != EDGE_MOE_OK:
        raise EdgeMoeError("edge_moe_mfma_peak", st)


def edge_moe_forward_noalloc(dims, x, topk_idx, topk_w, weights, y, stream=None) -> None:
    """edge_moe_forward with the library's own per-device scratch as workspace
    (no allocation; calls that overlap on one GPU race)."""
    st = load().edge_moe_forward_noalloc(ctypes.byref(cdims(dims)), _ptr(x), _ptr(topk_idx), _ptr(topk_w),
                                         ctypes.byref(cweights(weights)), _ptr(y), _stream(stream))
    if st != EDGE_MOE_OK:
        raise EdgeMoeError("edge_moe_forward_noalloc", st)


def edge_moe_residual(x, y, x_out, stream=None) -> None:
    T, d = x.shape
    st = load().edge_moe_residual(int(T), int(d), _ptr(x), _ptr(y), _ptr(x_out), _stream(stream))
    if st != EDGE_MOE_OK:
        raise EdgeMoeError("edge_moe_residual", st)


def _host_ptr(t) -> Optional[int]:
    if t is None:
        return None
    if t.is_cuda:
        raise ValueError("this argument must be in host memory")
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    return t.data_ptr()


def _stats(c: CCacheStats) -> dict:
    return {n: int(getattr(c, n)) for n, _ in CCacheStats._fields_}


class ExpertCache:
    """edge_moe_cache_*: an LRU of `slots_per_group` HBM slots per group for one
    layer's expert tensors, filled from host memory.

    host:  dict with EXPERT_TENSOR_KEYS (the last two optional) of host tensors
           holding the layer's E experts (pin them for the copies to overlap);
    slots: dict of device tensors with G * S experts each, the same keys set,
           or None for a cache that only plans.
    map() renames a batch's expert ids to slots and issues the copies of the
    misses; the layer then runs on slot_dims() with the slot tensors in place
    of the expert tensors (slot_weights())."""

    def __init__(self, dims, slots_per_group: int, host: dict, slots: Optional[dict] = None):
        self._lib = load()
        self.S = int(slots_per_group)
        self._keep = (host, slots)
        # the library trusts the buffers to hold E experts (host) and G * S
        # slots (device) of the per-expert sizes its dims imply: check them here
        per = expert_tensor_bytes(dims)
        G = dims.n_experts // dims.experts_per_group
        for k in EXPERT_TENSOR_KEYS:
            for side, tensors, count in (("host", host, dims.n_experts), ("slot", slots, G * self.S)):
                t = None if tensors is None else tensors.get(k)
                if t is not None and t.numel() * t.element_size() != count * per[k]:
                    raise ValueError(f"{side} tensor {k}: {t.numel() * t.element_size()} bytes, "
                                     f"expected {count} x {per[k]}")
        ch = CExpertTensors(*(_host_ptr(host.get(k)) for k in EXPERT_TENSOR_KEYS))
        cs = None if slots is None else CExpertTensors(*(_ptr(slots.get(k)) for k in EXPERT_TENSOR_KEYS))
        self._h = self._lib.edge_moe_cache_create(ctypes.byref(cdims(dims)), self.S, ctypes.byref(ch),
                                                  None if cs is None else ctypes.byref(cs))
        if not self._h:
            raise ValueError("edge_moe_cache_create rejected its arguments")

    def map(self, topk_idx, slot_idx, stream=None) -> dict:
        """topk_idx, slot_idx: host int32 [T][k] tensors; returns this call's counts."""
        T = topk_idx.shape[0] if topk_idx.dim() else 0
        st = CCacheStats()
        r = self._lib.edge_moe_cache_map(self._h, int(T), _host_ptr(topk_idx), _host_ptr(slot_idx),
                                         _stream(stream) if self._keep[1] is not None else None, ctypes.byref(st))
        if r != EDGE_MOE_OK:
            raise EdgeMoeError("edge_moe_cache_map", r)
        return _stats(st)

    def prefetch(self, experts, stream=None) -> dict:
        st = CCacheStats()
        r = self._lib.edge_moe_cache_prefetch(self._h, int(experts.numel()), _host_ptr(experts),
                                              _stream(stream) if self._keep[1] is not None else None,
                                              ctypes.byref(st))
        if r != EDGE_MOE_OK:
            raise EdgeMoeError("edge_moe_cache_prefetch", r)
        return _stats(st)

    def totals(self) -> dict:
        st = CCacheStats()
        r = self._lib.edge_moe_cache_totals(self._h, ctypes.byref(st))
        if r != EDGE_MOE_OK:
            raise EdgeMoeError("edge_moe_cache_totals", r)
        return _stats(st)

    def slot_of(self, expert: int) -> int:
        return int(self._lib.edge_moe_cache_slot_of(self._h, int(expert)))

    def close(self) -> None:
        if self._h:
            self._lib.edge_moe_cache_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def expert_tensor_bytes(dims) -> dict:
    """Bytes of one expert's tensor of each EXPERT_TENSOR_KEYS key (packed int4
    codes, fp16 scales per min(quant_group, K) elements; the decode copies are
    the size of the codes they copy)."""
    r, d, h, q = dims.delta_rank, dims.d, dims.h, dims.quant_group
    sc = lambda n, k: n * (k // min(q, k)) * 2  # noqa: E731
    out = {"a_up": r * d // 2, "a_up_scale": sc(r, d), "b_up": h * r // 2, "b_up_scale": sc(h, r),
           "a_dn": r * h // 2, "a_dn_scale": sc(r, h), "b_dn": d * r // 2, "b_dn_scale": sc(d, r)}
    out["a_up_t"], out["a_dn_t"] = out["a_up"], out["a_dn"]
    return out


class _SlotDims:
    def __init__(self, dims, S: int):
        for f, _ in CDims._fields_:
            setattr(self, f, int(getattr(dims, f)))
        self.n_experts = (self.n_experts // self.experts_per_group) * S
        self.experts_per_group = S


def slot_dims(dims, slots_per_group: int):
    """The dims of the slot layer: G groups of S experts."""
    return _SlotDims(dims, slots_per_group)


def slot_weights(weights: dict, slots: dict) -> dict:
    """The resident layer's weights with the slot tensors in place of the
    per-expert tensors (missing optional slot tensors drop the key)."""
    out = {k: v for k, v in weights.items() if k not in EXPERT_TENSOR_KEYS}
    out.update({k: v for k, v in slots.items() if v is not None})
    return out


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
