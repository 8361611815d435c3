"""Benchmark of the shared-matrix MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one pass of the whole layer (router, permutation, shared / delta /
LoRA products, activation, combine) over one batch already resident in HBM.
The headline line measures the T=8 speculative-verify batch with skewed
routing (the launch post's Scheduling paragraph verifies several draft tokens
per weight read); each step uses the next of 4 layer instances so that the
~400 MB a step touches cannot be served from the 256 MB Infinity Cache.  The
same JSON line carries the 16K-token prefill measurement (byteiota page,
Benchmark Numbers: 16K prefill).

Printed: ONE JSON line on stdout.  Per-kernel times go to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
MFMA_FP8_PEAK_TFLOPS = 5000.0  # MI355X dense fp8
PCIE_PEAK_GBS = 64.0            # host link, PCIe 5.0 x16, one direction
METRIC = "MoE-layer tokens/s at T=8 verify & 16K prefill; % peak HBM GB/s / % MFMA"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------- algorithmic work ---

def weight_bytes(D):
    """Bytes of each weight unit: per group (shared pair + LoRA), per expert (deltas)."""
    d, h, r, rL = D.d, D.h, D.delta_rank, D.lora_rank
    gs = lambda K: min(D.quant_group, K)  # noqa: E731
    i4 = lambda N, K: N * K // 2 + N * (K // gs(K)) * 2  # noqa: E731
    per = {
        "s_up": i4(h, d), "s_dn": i4(d, h),
        "lu_u": rL * d * 2, "lu_v": h * rL * 2, "ld_u": rL * h * 2, "ld_v": d * rL * 2,
        "a_up": i4(r, d), "b_up": i4(h, r), "a_dn": i4(r, h), "b_dn": i4(d, r),
        "w_router": D.n_experts * D.d * 2,
    }
    return per


def kernel_bytes(D, idx: np.ndarray):
    """Algorithmic HBM bytes per launch of each kernel for one routed batch:
    the weight bytes it must stream (each touched group / distinct expert once)
    plus the activations it must read and write once."""
    per = weight_bytes(D)
    T, k = idx.shape
    G = len(np.unique(idx // D.experts_per_group))
    X = len(np.unique(idx))
    R = T * k
    U = sum(len(np.unique(np.nonzero((idx // D.experts_per_group) == g)[0]))
            for g in range(D.n_experts // D.experts_per_group))
    d, h, r, rL, E = D.d, D.h, D.delta_rank, D.lora_rank, D.n_experts
    x_b = T * d * 2                       # the batch, bf16
    logits_b = T * E * 4
    split = T <= 8 and d == 4096 and E % 8 == 0 and E <= 512
    split_b = 8 * T * E * 8
    gw_up = per["s_up"] + per["lu_u"] + per["lu_v"]
    gw_dn = per["s_dn"] + per["ld_u"] + per["ld_v"]
    return {
        # router: the one-pass logits kernels write fp32 logits that the top-k
        # reads; the K-split one (up to 8 tokens, d = 4096) writes 8 fp64 slice
        # sums per logit, which the top-k reads instead
        "router_logits_small": per["w_router"] + x_b + logits_b,
        "router_logits_tiled": per["w_router"] + x_b + logits_b,
        "router_logits_split": per["w_router"] + x_b + split_b,
        "router_topk": (split_b if split else logits_b) + R * 8,
        # decode / verify path: each touched group's and expert's weights once,
        # the kernel's inputs read once and its outputs written once
        "dec_up": G * (per["s_up"] + per["lu_u"]) + X * per["a_up"] + x_b
                  + U * h * 4 + R * r * 4 + U * rL * 4,
        # the work-list shared up (decode-tiled codes) moves the same bytes
        "dec_up_ws": G * (per["s_up"] + per["lu_u"]) + X * per["a_up"] + x_b
                     + U * h * 4 + R * r * 4 + U * rL * 4,
        "dec_act": X * (per["b_up"] + per["a_dn"]) + G * (per["lu_v"] + per["ld_u"])
                   + U * h * 4 + R * r * 4 + U * rL * 4 + R * h * 2 + R * (r + rL) * 2,
        "dec_down": G * (per["s_dn"] + per["ld_v"]) + X * per["b_dn"] + R * h * 2
                    + R * (r + rL) * 2 + R * 4 + T * d * 4,
        # the wave-streamed down kernels (row-major, decode-tiled shared matrix)
        # move the same algorithmic bytes
        "dec_down_ws": G * (per["s_dn"] + per["ld_v"]) + X * per["b_dn"] + R * h * 2
                       + R * (r + rL) * 2 + R * 4 + T * d * 4,
        "dec_down_wst": G * (per["s_dn"] + per["ld_v"]) + X * per["b_dn"] + R * h * 2
                        + R * (r + rL) * 2 + R * 4 + T * d * 4,
        # the persistent decode layer: every touched group's and distinct
        # expert's weights once, the batch read once and y written once (its
        # intermediates stay in the workspace and the caches)
        "dec_layer": G * (per["s_up"] + per["s_dn"] + per["lu_u"] + per["lu_v"] + per["ld_u"] + per["ld_v"])
                     + X * (per["a_up"] + per["b_up"] + per["a_dn"] + per["b_dn"]) + x_b + T * d * 4,
        "pl_clear": 1536 * 4,
        # general (prefill) path
        "gemm_z1": X * per["a_up"] + R * d * 2 + R * r * 2,
        "lora_in_up": G * per["lu_u"] + U * d * 2,
        "gemm_shared_up": G * (per["s_up"] + per["lu_v"]) + U * d * 2 + U * h * 4,
        "gemm_delta_up_act": X * per["b_up"] + R * r * 2 + R * h * 4 + R * h * 2,
        "gemm_z2": X * per["a_dn"] + R * h * 2,
        "lora_in_down": G * per["ld_u"] + R * h * 2,
        "gemm_down": G * (per["s_dn"] + per["ld_v"]) + X * per["b_dn"] + R * h * 2 + R * d * 4,
        "combine": R * d * 4 + T * d * 4,
        "pf_gather_x": 2 * U * d * 2,
        "pf_shared_up": G * (per["s_up"] + per["lu_v"]) + U * d * 2 + U * h * 4,
        "pf_delta_up_act": X * per["b_up"] + R * r * 2 + R * h * 4 + R * h * 2,
        "pf_down": G * (per["s_dn"] + per["ld_v"]) + X * per["b_dn"] + R * h * 2 + R * d * 4,
    }, {"groups": G, "experts": X, "rows": R, "unique": U, "gw_up": gw_up, "gw_dn": gw_dn}


def step_bytes(D, idx):
    """Whole-step algorithmic bytes: touched weights once + router weights."""
    per = weight_bytes(D)
    G = len(np.unique(idx // D.experts_per_group))
    X = len(np.unique(idx))
    g_b = per["s_up"] + per["s_dn"] + per["lu_u"] + per["lu_v"] + per["ld_u"] + per["ld_v"]
    e_b = per["a_up"] + per["b_up"] + per["a_dn"] + per["b_dn"]
    return per["w_router"] + G * g_b + X * e_b


def step_flops(D, idx):
    """Algorithmic MFMA flops of one layer step: every stage once (the pf_* and
    gemm_* names of kernel_flops are two implementations of the same stages)."""
    return sum(v for k, v in kernel_flops(D, idx).items() if not k.startswith(("pf_", "mx_")))


def kernel_flops(D, idx):
    """Algorithmic MFMA flops per launch (shared up once per (token, group))."""
    T, k = idx.shape
    R = T * k
    U = sum(len(np.unique(np.nonzero((idx // D.experts_per_group) == g)[0]))
            for g in range(D.n_experts // D.experts_per_group))
    d, h, r, rL = D.d, D.h, D.delta_rank, D.lora_rank
    return {
        "gemm_z1": 2 * R * r * d,
        "lora_in_up": 2 * U * rL * d,
        "gemm_shared_up": 2 * U * h * d + 2 * U * h * rL,
        "gemm_delta_up_act": 2 * R * h * r,
        "gemm_z2": 2 * R * r * h,
        "lora_in_down": 2 * R * rL * h,
        "gemm_down": 2 * R * d * h + 2 * R * d * r + 2 * R * d * rL,
        "pf_z1": 2 * R * r * d,
        "pf_z2": 2 * R * r * h,
        "pf_shared_up": 2 * U * h * d + 2 * U * h * rL,
        "pf_delta_up_act": 2 * R * h * r,
        "pf_down": 2 * R * d * h + 2 * R * d * r + 2 * R * d * rL,
        # the MX variant's kernels (same products)
        "mx_z1": 2 * R * r * d,
        "mx_shared_up": 2 * U * h * d + 2 * U * h * rL,
        "mx_z2": 2 * R * r * h,
        "mx_down": 2 * R * d * h + 2 * R * d * r + 2 * R * d * rL,
    }


# ---------------------------------------------------------------- device workload ----

class Workload:
    def __init__(self, cfg_id, layers, seed=0, host_init=False, mx=False):
        import torch
        import shared_matrix_expert_amd as em
        import synth
        self.torch, self.em = torch, em
        c = synth.config(cfg_id)
        self.D = c.dims
        self.cfg_id = cfg_id
        self.mx = mx
        self.layers = []
        x = synth.make_activations(cfg_id, seed)
        self.x_host = x
        self.x = torch.from_numpy(x.view(np.int16)).cuda()
        for layer in range(layers):
            wr, bias = synth.make_router(cfg_id, seed, layer)
            self.layers.append({
                "wr_host": wr, "bias_host": bias,
                "wr": torch.from_numpy(wr.view(np.int16)).cuda(),
                "bias": None if bias is None else torch.from_numpy(bias).cuda(),
                "W": (self._weights_mx(synth, cfg_id, seed, layer, host_init) if mx else
                      self._weights(synth, cfg_id, seed, layer, host_init, em, self.D)),
            })
        D = self.D
        ws_bytes = em.edge_moe_workspace_bytes(D)
        if mx:
            ws_bytes = max(ws_bytes, em.edge_moe_workspace_bytes_mx(D))
        self.ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
        self.idx = torch.empty(D.T, D.top_k, dtype=torch.int32, device="cuda")
        self.w = torch.empty(D.T, D.top_k, dtype=torch.float32, device="cuda")
        self.y = torch.empty(D.T, D.d, dtype=torch.float32, device="cuda")
        self.stream = torch.cuda.current_stream()

    @staticmethod
    def _weights(synth, cfg_id, seed, layer, host_init, em, D):
        """Weights made on the device, or (host_init) on the host and copied over,
        so that no kernel but the library's runs in the process (counter runs).
        Decode batches also get the decode-tiled copies of the shared matrices,
        written once here by the library (a stored format, outside any step)."""
        if not host_init:
            W = synth.make_weights(cfg_id, seed, layer, device="cuda")
        else:
            W = {k: v.cuda() for k, v in synth.make_weights(cfg_id, seed, layer, device="cpu").items()}
        if D.T <= 16 and D.quant_group == 128 and D.d % 1024 == 0 and D.h % 1024 == 0:
            W = em.tile_weights(D, W)          # kinds 0-3: the decode kernels and the persistent launch
        return W

    @staticmethod
    def _weights_mx(synth, cfg_id, seed, layer, host_init):
        if not host_init:
            return synth.make_weights_mx(cfg_id, seed, layer, device="cuda")
        return {k: v.cuda() for k, v in synth.make_weights_mx(cfg_id, seed, layer, device="cpu").items()}

    persistent = False   # the layer through edge_moe_forward_persistent (one persistent launch)

    def step(self, i):
        L = self.layers[i % len(self.layers)]
        em, D = self.em, self.D
        em.edge_moe_route(D, self.x, L["wr"], L["bias"], self.idx, self.w, None, self.ws, self.stream)
        if self.mx:
            em.edge_moe_forward_mx(D, self.x, self.idx, self.w, L["W"], self.y, self.ws, self.stream)
        elif self.persistent:
            em.edge_moe_forward_persistent(D, self.x, self.idx, self.w, L["W"], self.y, self.ws, self.stream)
        else:
            em.edge_moe_forward(D, self.x, self.idx, self.w, L["W"], self.y, self.ws, self.stream)

    def routed_indices(self):
        """Expert indices of every layer instance (from one step each)."""
        out = []
        for i in range(len(self.layers)):
            self.step(i)
            self.torch.cuda.synchronize()
            out.append(self.idx.cpu().numpy().copy())
        return out

    def time_steps(self, steps, warmup):
        torch = self.torch
        for i in range(warmup):
            self.step(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            self.step(i)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps

    def kernel_times(self, steps):
        """Average per-launch ms of every kernel, from HIP events recorded by the
        library on the stream it launches on (a separate pass of `steps` steps)."""
        em, torch = self.em, self.torch
        em.edge_moe_prof_reset()
        em.edge_moe_prof_enable(True)
        for i in range(steps):
            self.step(i)
        torch.cuda.synchronize()
        em.edge_moe_prof_enable(False)
        tab = em.edge_moe_prof_read()
        em.edge_moe_prof_reset()
        return {k: (n, ms / max(n, 1)) for k, (n, ms) in tab.items()}


def roofline_hbm(D, idxs, ktimes):
    """Dominant kernel by total time; achieved = its algorithmic bytes / its avg time."""
    name = max(ktimes, key=lambda k: ktimes[k][0] * ktimes[k][1])
    bytes_per = np.mean([kernel_bytes(D, ix)[0].get(name, 0) for ix in idxs])
    avg_ms = ktimes[name][1]
    gbs = bytes_per / (avg_ms * 1e-3) / 1e9
    return name, {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                  "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                  "kernel": name, "avg_ms": round(avg_ms, 5), "bytes_per_launch": int(bytes_per)}


def stored_traffic(kernel: str, workload_tag: str):
    """HBM bytes per launch of `kernel` from the counter summary under profiles/,
    or None when there is none or it was taken with other kernel sources."""
    from shared_matrix_expert_amd.build import sources_digest
    from shared_matrix_expert_amd.profsum import read_traffic
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload_tag}_traffic.txt")
    if not os.path.exists(path):
        return None
    t = read_traffic(path)
    if t.get("sources_sha256") != sources_digest(kernel):
        return None
    return int(float(t["traffic_bytes_per_dispatch"]))


# Library kernel names (the per-kernel event table) and their names in a
# rocprofv3 kernel trace, for the kernels that can be a roofline's dominant one.
TRACE_NAMES = {"mx_down": "mx_gemm<1>", "mx_shared_up": "mx_gemm<0>", "dec_down_wst": "dec_down_ws<true>", "dec_down_ws": "dec_down_ws<false>", "dec_act": "dec_act<1>",
               "dec_up_ws": "dec_up_ws", "dec_layer": "dec_layer<16>", "router_topk": "router_topk_split",
               "router_logits_split": "router_logits_split", "pf_down": "pf_gemm<1>",
               "pf_shared_up": "pf_gemm<0>", "pf_z1": "pf_gemm<2>", "pf_z2": "pf_gemm<3>",
               "pf_delta_up_act": "pf_act"}


def rocprof_avg_ms(kernel: str, workload_tag: str):
    """Average launch time of `kernel` in the committed rocprofv3 kernel
    statistics of the workload (profiles/<tag>_kernels.md), or None."""
    path = os.path.join(ROOT, "profiles", f"{workload_tag}_kernels.md")
    want = TRACE_NAMES.get(kernel, kernel)
    if not os.path.exists(path):
        return None
    for line in open(path):
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) >= 4 and cells[0] == want:
            return float(cells[3]) / 1e3
    return None


def add_rocprof(roof, workload_tag):
    """Beside the live event time that `frac` uses: the same kernel's rocprofv3
    average from profiles/ and the fraction it gives."""
    ms = rocprof_avg_ms(roof["kernel"], workload_tag)
    roof["avg_ms_rocprof"] = round(ms, 5) if ms else None
    if ms:
        if roof["unit"] == "GB/s":
            roof["frac_rocprof"] = round(roof["bytes_per_launch"] / (ms * 1e-3) / 1e9 / roof["peak"], 4)
        else:
            roof["frac_rocprof"] = round(roof["flops_per_launch"] / (ms * 1e-3) / 1e12 / roof["peak"], 4)
    roof["time_source"] = "frac: HIP events around each launch in this run; frac_rocprof: profiles/%s_kernels.md" % workload_tag
    return roof


def kernel_table(D, idxs, ktimes):
    """Per-kernel average time, algorithmic bytes and the HBM rate they imply."""
    out = {}
    for k, (n, ms) in sorted(ktimes.items(), key=lambda kv: -kv[1][0] * kv[1][1]):
        b = float(np.mean([kernel_bytes(D, ix)[0].get(k, 0) for ix in idxs]))
        out[k] = {"avg_us": round(ms * 1e3, 2), "bytes": int(b),
                  "GBs": round(b / (ms * 1e-3) / 1e9, 1) if b else None}
    return out


def roofline_mfma(D, idxs, ktimes, peak=MFMA_BF16_PEAK_TFLOPS):
    fl = {k: np.mean([kernel_flops(D, ix).get(k, 0) for ix in idxs]) for k in ktimes}
    cand = {k: v for k, v in ktimes.items() if fl.get(k, 0) > 0}
    name = max(cand, key=lambda k: cand[k][0] * cand[k][1])
    avg_ms = ktimes[name][1]
    tf = fl[name] / (avg_ms * 1e-3) / 1e12
    return name, {"bound": "mfma", "achieved": round(tf, 2), "peak": peak,
                  "unit": "TFLOP/s", "frac": round(tf / peak, 4), "traffic": None,
                  "kernel": name, "avg_ms": round(avg_ms, 4), "flops_per_launch": int(fl[name])}


class Stack:
    """The 48-layer stack of full-size layers (T=8), every layer's weights and
    router resident in HBM at once; one step is route + layer + residual through
    all layers in sequence."""

    def __init__(self, seed=0, host_init=False):
        import torch
        import shared_matrix_expert_amd as em
        import synth
        self.torch, self.em = torch, em
        c = synth.config(4)
        self.D = c.dims
        self.n_layers = c.layers
        self.x0 = torch.from_numpy(synth.make_activations(4, seed).view(np.int16)).cuda()
        self.layers = []
        for layer in range(self.n_layers):
            wr, _ = synth.make_router(4, seed, layer)
            self.layers.append({"wr": torch.from_numpy(wr.view(np.int16)).cuda(),
                                "W": Workload._weights(synth, 4, seed, layer, host_init, em, self.D)})
        D = self.D
        self.ws = torch.empty(em.edge_moe_workspace_bytes(D), dtype=torch.uint8, device="cuda")
        self.idx = torch.empty(D.T, D.top_k, dtype=torch.int32, device="cuda")
        self.w = torch.empty(D.T, D.top_k, dtype=torch.float32, device="cuda")
        self.y = torch.empty(D.T, D.d, dtype=torch.float32, device="cuda")
        self.xa = torch.empty_like(self.x0)
        self.xb = torch.empty_like(self.x0)
        self.stream = torch.cuda.current_stream()
        self.idxs = []
        self.pf_stream = None
        self.pf_ws = None

    def predictions(self, hit_rate, seed=0):
        """A synthetic stand-in for the prerouter head: for each layer, the groups
        its recorded routing touched, each kept with probability hit_rate and
        otherwise replaced by a group it did not touch (device int32 lists)."""
        rng = np.random.default_rng(seed)
        G = self.D.n_experts // self.D.experts_per_group
        out = []
        for ix in self.idxs:
            true = sorted(set((ix // self.D.experts_per_group).ravel().tolist()))
            other = [g for g in range(G) if g not in true]
            pred = []
            for g in true:
                if rng.random() < hit_rate or not other:
                    pred.append(g)
                else:
                    pred.append(other.pop(int(rng.integers(len(other)))))
            out.append(self.torch.tensor(pred, dtype=self.torch.int32, device="cuda"))
        return out

    def step(self, record=False, prefetch=None, parts=1):
        """One pass.  With prefetch (a device group list per layer), layer l+1's
        predicted groups are read on a second stream, starting with layer l."""
        em, D, torch = self.em, self.D, self.torch
        x = self.x0
        for li, L in enumerate(self.layers):
            if prefetch is not None and li + 1 < self.n_layers:
                ev = torch.cuda.Event()
                ev.record(self.stream)
                self.pf_stream.wait_event(ev)
                em.edge_moe_prefetch(D, self.layers[li + 1]["W"], prefetch[li + 1], parts, self.pf_ws,
                                     self.pf_stream)
            em.edge_moe_route(D, x, L["wr"], None, self.idx, self.w, None, self.ws, self.stream)
            em.edge_moe_forward(D, x, self.idx, self.w, L["W"], self.y, self.ws, self.stream)
            if record:
                self.torch.cuda.synchronize()
                self.idxs.append(self.idx.cpu().numpy().copy())
            out = self.xa if li % 2 == 0 else self.xb
            em.edge_moe_residual(x, self.y, out, self.stream)
            x = out

    def time_steps(self, steps, warmup):
        torch = self.torch
        self.step(record=True)
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            self.step()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps

    def final_x(self):
        return self.xa if (self.n_layers - 1) % 2 == 0 else self.xb

    def time_prefetch(self, steps, hit_rate, parts=1):
        """Passes with the next layer's predicted shared matrices read ahead on
        a second stream (default priority); returns (seconds per pass, whether
        the output equals the plain pass bitwise)."""
        torch = self.torch
        if self.pf_stream is None:
            self.pf_stream = torch.cuda.Stream()
            self.pf_ws = torch.empty(self.em.edge_moe_prefetch_ws_bytes(), dtype=torch.uint8, device="cuda")
        pred = self.predictions(hit_rate)
        self.step()
        torch.cuda.synchronize()
        ref = self.final_x().clone()
        self.step(prefetch=pred, parts=parts)
        torch.cuda.synchronize()
        same = bool(torch.equal(ref, self.final_x()))
        t0 = time.perf_counter()
        for _ in range(steps):
            self.step(prefetch=pred, parts=parts)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps, same

    def time_graph(self, steps):
        """The same pass captured once as a HIP graph (48 x (route, layer,
        residual) launches) and replayed; returns (seconds per replay, whether
        the first replay's output equals the eager pass bitwise)."""
        torch = self.torch
        self.step()
        torch.cuda.synchronize()
        ref = (self.xa if (self.n_layers - 1) % 2 == 0 else self.xb).clone()
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        eager_stream = self.stream
        with torch.cuda.stream(side):
            self.stream = side
            with torch.cuda.graph(g, stream=side):
                self.step()
        self.stream = eager_stream
        torch.cuda.current_stream().wait_stream(side)
        self.xa.zero_()
        self.xb.zero_()
        g.replay()
        torch.cuda.synchronize()
        same = bool(torch.equal(ref, self.xa if (self.n_layers - 1) % 2 == 0 else self.xb))
        t0 = time.perf_counter()
        for _ in range(steps):
            g.replay()
        torch.cuda.synchronize()
        sec = (time.perf_counter() - t0) / steps
        del g
        return sec, same


class StreamStack:
    """Decode (T=1) through a stack of full-size layers whose per-expert tensors
    live in pinned host memory and reach HBM through an LRU of S slots per group
    and layer (edge_moe_cache_*); the shared matrices (with their decode-tiled
    copies), the LoRA factors and the routers stay resident.  One step decodes a
    new synthetic token through every layer: route, read the routed experts back
    to the host, rename them to slots (the misses' copies go on the compute
    stream), run the slot layer, add the residual.

    With predict=True, layer l+1's experts are guessed while layer l runs, by
    routing layer l's input through layer l+1's router (the next layer's own
    router standing in for the pages' light prerouter head), and the guesses'
    copies go on a second stream (default priority) so that they overlap layer
    l's kernels; layer l+1 waits for them before its kernels start."""

    def __init__(self, n_layers, slots_per_group, seed=0, n_tokens=512, host_init=False):
        import torch
        import shared_matrix_expert_amd as em
        import synth
        self.torch, self.em = torch, em
        self.D = D = synth.config(1).dims
        self.S = slots_per_group
        self.n_layers = n_layers
        self.xs = torch.from_numpy(synth.make_activations(1, seed + 7, T=n_tokens).view(np.int16)).cuda()
        G = D.n_experts // D.experts_per_group
        self.SD = em.slot_dims(D, self.S)
        self.layers = []
        keys = em.EXPERT_TENSOR_KEYS[:8]
        for layer in range(n_layers):
            wr, bias = synth.make_router(1, seed, layer)
            W = Workload._weights(synth, 1, seed, layer, host_init, em, D)
            W.pop("a_up_t", None)
            W.pop("a_dn_t", None)
            host = {k: W[k].cpu().pin_memory() for k in keys}
            slots = {k: torch.empty((G * self.S,) + tuple(W[k].shape[1:]), dtype=W[k].dtype, device="cuda")
                     for k in keys}
            resident = W
            self.layers.append({"wr": torch.from_numpy(wr.view(np.int16)).cuda(),
                                "bias": None if bias is None else torch.from_numpy(bias).cuda(),
                                "W": resident, "SW": em.slot_weights(W, slots),
                                "cache": em.ExpertCache(D, self.S, host, slots), "slots": slots,
                                "ready": torch.cuda.Event()})
        self.expert_bytes_resident = sum(W[k].numel() * W[k].element_size() for k in keys)
        self.slot_bytes = sum(v.numel() * v.element_size() for v in self.layers[0]["slots"].values())
        self.ws = torch.empty(max(em.edge_moe_workspace_bytes(D), em.edge_moe_workspace_bytes(self.SD)),
                              dtype=torch.uint8, device="cuda")
        self.idx = torch.empty(1, D.top_k, dtype=torch.int32, device="cuda")
        self.pidx = torch.empty(1, D.top_k, dtype=torch.int32, device="cuda")
        self.w = torch.empty(1, D.top_k, dtype=torch.float32, device="cuda")
        self.pw = torch.empty_like(self.w)
        self.sidx = torch.empty_like(self.idx)
        self.idx_h = torch.empty(2, D.top_k, dtype=torch.int32).pin_memory()
        self.slot_h = torch.empty(1, D.top_k, dtype=torch.int32).pin_memory()
        self.y = torch.empty(1, D.d, dtype=torch.float32, device="cuda")
        self.xa = torch.empty(1, D.d, dtype=torch.int16, device="cuda")
        self.xb = torch.empty_like(self.xa)
        self.stream = torch.cuda.current_stream()
        self.copy_stream = torch.cuda.Stream()
        self.tok = 0

    def drop_resident_experts(self):
        """Free the resident copies of the expert tensors (kept until the
        streamed pass has been checked against them)."""
        for L in self.layers:
            for k in self.em.EXPERT_TENSOR_KEYS[:8]:
                L["W"].pop(k, None)
        self.torch.cuda.empty_cache()

    def step(self, predict=False, resident=False, stats=None):
        em, D, torch = self.em, self.D, self.torch
        x = self.xs[self.tok % self.xs.shape[0]:self.tok % self.xs.shape[0] + 1]
        self.tok += 1
        for li, L in enumerate(self.layers):
            em.edge_moe_route(D, x, L["wr"], L["bias"], self.idx, self.w, None, self.ws, self.stream)
            out = self.xa if li % 2 == 0 else self.xb
            if resident:
                em.edge_moe_forward(D, x, self.idx, self.w, L["W"], self.y, self.ws, self.stream)
                em.edge_moe_residual(x, self.y, out, self.stream)
                x = out
                continue
            nxt = self.layers[li + 1] if predict and li + 1 < self.n_layers else None
            if nxt is not None:
                em.edge_moe_route(D, x, nxt["wr"], nxt["bias"], self.pidx, self.pw, None, self.ws, self.stream)
                self.idx_h[1].copy_(self.pidx[0], non_blocking=True)
            self.idx_h[0].copy_(self.idx[0])                     # waits for the stream: routing is on the host now
            # this layer's predicted copies land before any copy of the batch's
            # misses (which may reuse a slot a prediction is still filling) and
            # before its kernels
            self.stream.wait_event(L["ready"])
            st = L["cache"].map(self.idx_h[:1], self.slot_h, self.stream)
            if stats is not None:
                for k in st:
                    stats[k] = stats.get(k, 0) + st[k]
            self.sidx.copy_(self.slot_h, non_blocking=True)
            em.edge_moe_forward(self.SD, x, self.sidx, self.w, L["SW"], self.y, self.ws, self.stream)
            if nxt is not None:
                # layer l+1's slots: the last kernels reading them (its previous
                # token) precede everything enqueued since on this stream
                ev = torch.cuda.Event()
                ev.record(self.stream)
                self.copy_stream.wait_event(ev)
                guess = torch.unique(self.idx_h[1]).to(torch.int32)
                pst = nxt["cache"].prefetch(guess, self.copy_stream)
                nxt["ready"].record(self.copy_stream)
                if stats is not None:
                    stats["prefetched"] = stats.get("prefetched", 0) + pst["misses"]
                    stats["prefetch_bytes"] = stats.get("prefetch_bytes", 0) + pst["bytes_copied"]
            em.edge_moe_residual(x, self.y, out, self.stream)
            x = out
        return x

    def check(self, n_tokens=2):
        """The streamed pass against the resident one, bitwise, on a few tokens."""
        torch = self.torch
        ok = True
        for predict in (False, True):
            for i in range(n_tokens):
                t = self.tok
                ref = self.step(resident=True).clone()
                self.tok = t
                got = self.step(predict=predict)
                torch.cuda.synchronize()
                ok = ok and bool(torch.equal(ref, got))
        return ok

    def time_steps(self, steps, warmup, predict=False, resident=False):
        torch = self.torch
        for _ in range(warmup):
            self.step(predict=predict, resident=resident)
        torch.cuda.synchronize()
        stats = {}
        t0 = time.perf_counter()
        for _ in range(steps):
            self.step(predict=predict, resident=resident, stats=stats)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps, stats


def h2d_rate(torch, mib=256, reps=5):
    """Measured host -> HBM copy rate from pinned memory (GB/s)."""
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8).pin_memory()
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst.copy_(src, non_blocking=True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src, non_blocking=True)
    e1.record()
    torch.cuda.synchronize()
    return n * reps / (e0.elapsed_time(e1) / 1e3) / 1e9


def stream_line(args):
    """Decode with the experts streamed from host memory (edge_moe_cache_*):
    tokens/s through a stack of full-size layers, for a few slot counts, with
    and without next-layer prediction; the all-resident pass through the same
    loop beside it."""
    import torch
    log("building the host-streamed decode stack ...")
    rate = h2d_rate(torch)
    out = {"unit": "tokens/s", "h2d_pinned_GBs": round(rate, 1), "layers": args.stream_layers,
           "workload": "decode T=1, a new synthetic token every step through %d full-size layers; per-expert "
                       "int4 tensors (A_up, B_up, A_dn, B_dn with scales, %.2f MB per expert) in pinned host "
                       "memory, S slots per group and layer in HBM" % (args.stream_layers, 0.0)}
    first = True
    for S in args.stream_slots:
        ss = StreamStack(args.stream_layers, S, host_init=args.host_init)
        per_expert = ss.expert_bytes_resident / ss.D.n_experts
        if first:
            out["workload"] = out["workload"].replace("0.00 MB", "%.2f MB" % (per_expert / 1e6))
            rsec, _ = ss.time_steps(args.stream_steps, 3, resident=True)
            out["resident"] = {"value": round(1 / rsec, 1), "ms_per_step": round(rsec * 1e3, 4),
                               "what": "the same loop with every expert resident (no host round trip)"}
            log(f"  resident: {rsec * 1e3:.3f} ms per token")
            first = False
        same = ss.check()
        ss.drop_resident_experts()
        for predict in (False, True):
            sec, st = ss.time_steps(args.stream_steps, 3, predict=predict)
            em = ss.em
            em.edge_moe_prof_reset()
            em.edge_moe_prof_enable(True)
            _, pst = ss.time_steps(max(10, args.stream_steps // 4), 0, predict=predict)
            torch.cuda.synchronize()
            em.edge_moe_prof_enable(False)
            tab = em.edge_moe_prof_read()
            em.edge_moe_prof_reset()
            g_n, g_ms = tab.get("cache_gather", (0, 0.0))
            g_bytes = pst.get("bytes_copied", 0) + pst.get("prefetch_bytes", 0)
            n = args.stream_steps * args.stream_layers
            hits, misses = st.get("hits", 0), st.get("misses", 0)
            copied = st.get("bytes_copied", 0) + st.get("prefetch_bytes", 0)
            key = f"S{S}" + ("_predict" if predict else "")
            out[key] = {
                "value": round(1 / sec, 1), "ms_per_step": round(sec * 1e3, 4), "slots_per_group": S,
                "hbm_expert_bytes_per_layer": ss.slot_bytes,
                "host_expert_bytes_per_layer": ss.expert_bytes_resident,
                "hit_rate": round(hits / max(hits + misses, 1), 4),
                "experts_copied_per_layer": round((misses + st.get("prefetched", 0)) / n, 2),
                "h2d_bytes_per_token": int(copied / args.stream_steps),
                "h2d_GBs": round(copied / args.stream_steps / sec / 1e9, 2),
                "link_busy_frac": round(copied / args.stream_steps / (rate * 1e9) / sec, 4),
                "equals_resident": same}
            if g_n:
                # the gather kernel against the host link: bytes it moved over its
                # launches' summed time (HIP events around each launch)
                ach = g_bytes / (g_ms * 1e-3) / 1e9
                out[key]["roofline"] = {"bound": "host link", "kernel": "cache_gather", "launches": g_n,
                                        "avg_ms": round(g_ms / g_n, 5),
                                        "bytes_per_launch": int(g_bytes / g_n),
                                        "achieved": round(ach, 1), "peak": PCIE_PEAK_GBS, "unit": "GB/s",
                                        "frac": round(ach / PCIE_PEAK_GBS, 4),
                                        "frac_of_measured_dma": round(ach / rate, 4)}
            log(f"  stream {key}: {sec * 1e3:.3f} ms per token, hit rate {out[key]['hit_rate']}, "
                f"{out[key]['h2d_GBs']} GB/s host->HBM, equal to resident: {same}")
        del ss
        torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------- CPU baseline -------

def cpu_baseline(wl: Workload, budget_s: float = 30.0):
    """The oracle (float64 numpy) on the host cores, on a bounded sample: route +
    expert layer for the first layer instance's batch, repeated while time allows."""
    import synth
    from oracle.layer import moe_forward, route
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        blas_threads = 1
    L = wl.layers[0]
    Wh = synth.weights_to_numpy(L["W"])
    D = wl.D
    T = D.T
    tokens = 0
    t0 = time.perf_counter()
    reps = 0
    while True:
        rt = route(wl.x_host, L["wr_host"], L["bias_host"], D.top_k)
        moe_forward(wl.x_host, rt["idx"], rt["w"], Wh, D.experts_per_group)
        tokens += T
        reps += 1
        if time.perf_counter() - t0 > budget_s / 3 or reps >= 3:
            break
    el = time.perf_counter() - t0
    cores = min(len(os.sched_getaffinity(0)), blas_threads)
    return {"value": round(tokens / el, 3), "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{reps} x (route + expert layer) on the T={T} batch of layer instance 0, "
                      f"float64 numpy, {el:.1f} s"}


def cpu_baseline_prefill(wl: Workload, n_tokens: int = 16):
    import synth
    from oracle.layer import moe_forward, route
    L = wl.layers[0]
    Wh = synth.weights_to_numpy(L["W"])
    D = wl.D
    x = wl.x_host[:n_tokens]
    t0 = time.perf_counter()
    rt = route(x, L["wr_host"], L["bias_host"], D.top_k)
    moe_forward(x, rt["idx"], rt["w"], Wh, D.experts_per_group)
    el = time.perf_counter() - t0
    return {"value": round(n_tokens / el, 3), "unit": "tokens/s",
            "cores": int(len(os.sched_getaffinity(0))), "kind": "oracle",
            "sample": f"first {n_tokens} of the 16384 prefill tokens, float64 numpy, {el:.1f} s"}


# ---------------------------------------------------------------- main ---------------

def persistent_line(wl, steps, warmup, tag):
    """The same workload through the persistent launch: tokens/s, per-kernel
    event times, and the layer kernel's HBM roofline."""
    wl.persistent = True
    idxs = wl.routed_indices()
    sec = wl.time_steps(steps, warmup)
    kt = wl.kernel_times(max(20, steps // 4))
    name, roof = roofline_hbm(wl.D, idxs, kt)
    roof["traffic"] = stored_traffic(name, tag)
    add_rocprof(roof, tag)
    sb = float(np.mean([step_bytes(wl.D, ix) for ix in idxs]))
    wl.persistent = False
    log(f"  persistent launch ({tag}): {sec * 1e6:.1f} us per step")
    return {"value": round(wl.D.T / sec, 1), "unit": "tokens/s", "steps": steps, "ms_per_step": round(sec * 1e3, 5),
            "what": "route, then the layer as one persistent launch (edge_moe_forward_persistent)",
            "roofline": roof, "kernels": kernel_table(wl.D, idxs, kt),
            "step_hbm": {"bytes_per_step": int(sb), "achieved_GBs": round(sb / sec / 1e9, 1),
                         "frac": round(sb / sec / 1e9 / HBM_PEAK_GBS, 4)}}


def calibrate(em, torch):
    """Measured peaks on this GPU, beside the published ones: a plain device
    copy of 1 GiB (read + write bytes over time) and the matrix-core
    calibration launch (the faster of two and four workgroups of four waves
    per compute unit)."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(2):
        em.edge_moe_copy(b, a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 10
    e0.record()
    for _ in range(reps):
        em.edge_moe_copy(b, a)
    e1.record()
    torch.cuda.synchronize()
    copy_s = e0.elapsed_time(e1) / 1e3 / reps
    del a, b
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    iters, best = 20000, (0.0, "")
    for per_cu in (2, 4):                      # two and four waves per SIMD
        blocks = per_cu * cus
        out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
        em.edge_moe_mfma_peak(out, blocks, 100)
        e0.record()
        em.edge_moe_mfma_peak(out, blocks, iters)
        e1.record()
        torch.cuda.synchronize()
        rate = blocks * 4 * iters * 8 * 16384 / (e0.elapsed_time(e1) / 1e3) / 1e12
        if rate > best[0]:
            best = (rate, f"{blocks} x 256 threads, {iters} rounds")
    return {"copy_GBs": round(2 * n / copy_s / 1e9, 1), "copy_bytes": n,
            "mfma_bf16_TFLOPs": round(best[0], 1), "mfma_launch": best[1],
            "published": {"hbm_GBs": HBM_PEAK_GBS, "mfma_bf16_TFLOPs": MFMA_BF16_PEAK_TFLOPS}}


def mx_prefill_line(args):
    """The same 16K prefill through the MX variant (MXFP4 shared and delta
    matrices, MXFP8 activations on the scaled FP4 x FP8 matrix cores): tokens/s
    and the dominant kernel against the dense FP8 peak (its large products run
    at the FP8 rate)."""
    import torch
    log("building MX prefill workload ...")
    wp = Workload(3, 1, host_init=args.host_init, mx=True)
    pidx = wp.routed_indices()
    psec = wp.time_steps(args.prefill_steps, 2)
    pk = wp.kernel_times(args.prefill_steps)
    for k, (n, ms) in sorted(pk.items(), key=lambda kv: -kv[1][0] * kv[1][1]):
        log(f"  MX prefill kernel {k:20s} launches {n:5d} avg {ms:9.3f} ms")
    name, roof = roofline_mfma(wp.D, pidx, pk, peak=MFMA_FP8_PEAK_TFLOPS)
    roof["dtype"] = "fp8 x fp4 (E4M3 activations, E2M1 weights, E8M0 block scales)"
    roof["traffic"] = stored_traffic(name, "prefill_16k_mx")
    add_rocprof(roof, "prefill_16k_mx")
    total_fl = float(np.mean([step_flops(wp.D, ix) for ix in pidx]))
    out = {"value": round(wp.D.T / psec, 1), "unit": "tokens/s", "steps": args.prefill_steps,
           "ms_per_step": round(psec * 1e3, 3),
           "workload": "prefill T=16384, one layer, MXFP4 weights (same draws as the int4 layer), "
                       "router logits ~ N(0,1)",
           "roofline": roof,
           "step_mfma": {"flops_per_step": int(total_fl),
                         "achieved_TFLOPs": round(total_fl / psec / 1e12, 2),
                         "frac_of_fp8_peak": round(total_fl / psec / 1e12 / MFMA_FP8_PEAK_TFLOPS, 4)}}
    del wp
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--prefill-steps", type=int, default=5)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-stack", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--stack-steps", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-verify", action="store_true", help="skip the verify T=8 workload (profiling runs)")
    ap.add_argument("--no-calibrate", action="store_true")
    ap.add_argument("--no-mx", action="store_true", help="skip the MX-variant prefill line")
    ap.add_argument("--layers", type=int, default=4)
    ap.add_argument("--no-stream", action="store_true", help="skip the host-streamed decode line (also skipped by --no-decode)")
    ap.add_argument("--stream-layers", type=int, default=4)
    ap.add_argument("--stream-steps", type=int, default=100)
    ap.add_argument("--stream-slots", type=int, nargs="+", default=[16, 32])
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--host-init", action="store_true",
                    help="make the weights on the host (no kernel but the library's runs)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(the layer shards by tokens or by expert group; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import shared_matrix_expert_amd as em
    em.load()
    torch.cuda.init()

    if args.calib_copy_mib:
        n = args.calib_copy_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        em.edge_moe_copy(b, a)
        torch.cuda.synchronize()
        log(f"calibration copy of {n} bytes done")

    line = {"metric": METRIC, "note": "verify workload skipped (--no-verify)"}
    if not args.no_verify:
        # ---- verify T=8, skewed routing, rotating layer instances
        log("building verify workload ...")
        wl = Workload(2, args.layers, host_init=args.host_init)
        D = wl.D
        idxs = wl.routed_indices()
        sec = wl.time_steps(args.steps, args.warmup)
        ktimes = wl.kernel_times(max(20, args.steps // 4))
        for k, (n, ms) in sorted(ktimes.items(), key=lambda kv: -kv[1][0] * kv[1][1]):
            log(f"  verify kernel {k:22s} launches {n:5d} avg {ms * 1e3:8.2f} us")
        kname, roof = roofline_hbm(D, idxs, ktimes)
        roof["traffic"] = stored_traffic(kname, "verify_t8")
        add_rocprof(roof, "verify_t8")
        sb = float(np.mean([step_bytes(D, ix) for ix in idxs]))
        line = {
            "metric": METRIC,
            "value": round(D.T / sec, 1),
            "unit": "tokens/s",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": args.warmup,
            "ms_per_step": round(sec * 1e3, 5),
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": "bf16",
            "data": "synthetic",
            "config": {"workload": "speculative-verify batch T=8, skewed routing (48 of 80 top-10 picks "
                                   "in 2 of 8 groups), one layer: d=4096 h=8192 E=512 (8 groups of 64) "
                                   "top-10, int4 shared/delta (Gq=128, fp16 scales), r=128, bf16 LoRA "
                                   "rL=16; steps rotate over %d layer instances" % args.layers,
                       "T": D.T, "layers_rotated": args.layers},
            "roofline": roof,
            "kernels": kernel_table(D, idxs, ktimes),
            "step_hbm": {"bytes_per_step": int(sb), "achieved_GBs": round(sb / sec / 1e9, 1),
                         "frac": round(sb / sec / 1e9 / HBM_PEAK_GBS, 4)},
        }
        line["persistent"] = persistent_line(wl, args.steps, args.warmup, "verify_t8")
        if not args.no_cpu_baseline:
            log("timing the oracle on the host ...")
            line["cpu_baseline"] = cpu_baseline(wl)
        del wl
        torch.cuda.empty_cache()

    if not args.no_decode:
        log("building decode workload (T=1) ...")
        wd = Workload(1, args.layers, host_init=args.host_init)
        didx = wd.routed_indices()
        dsec = wd.time_steps(args.steps, args.warmup)
        dkt = wd.kernel_times(max(20, args.steps // 4))
        dname, droof = roofline_hbm(wd.D, didx, dkt)
        droof["traffic"] = stored_traffic(dname, "decode_t1")
        add_rocprof(droof, "decode_t1")
        dsb = float(np.mean([step_bytes(wd.D, ix) for ix in didx]))
        line["decode_t1"] = {
            "value": round(wd.D.T / dsec, 1), "unit": "tokens/s", "steps": args.steps,
            "ms_per_step": round(dsec * 1e3, 5),
            "workload": "decode T=1, one layer, %d rotating layer instances" % args.layers,
            "roofline": droof, "kernels": kernel_table(wd.D, didx, dkt),
            "step_hbm": {"bytes_per_step": int(dsb), "achieved_GBs": round(dsb / dsec / 1e9, 1),
                         "frac": round(dsb / dsec / 1e9 / HBM_PEAK_GBS, 4)},
        }
        log(f"  decode: {dsec * 1e6:.1f} us per step")
        line["decode_t1"]["persistent"] = persistent_line(wd, args.steps, args.warmup, "decode_t1")
        del wd
        torch.cuda.empty_cache()

    if not args.no_decode and not args.no_stream:
        line["decode_t1_streamed"] = stream_line(args)

    if not args.no_stack:
        log("building the 48-layer stack ...")
        st = Stack(host_init=args.host_init)
        ssec = st.time_steps(args.stack_steps, 2)
        sb = float(sum(step_bytes(st.D, ix) + 2 * st.D.T * st.D.d * 2 for ix in st.idxs))
        line["stack_48"] = {
            "value": round(st.D.T / ssec, 1), "unit": "tokens/s", "steps": args.stack_steps,
            "ms_per_step": round(ssec * 1e3, 4),
            "workload": "T=8 batch through 48 full-size layers in sequence (independent routers, "
                        "residual between layers), all weights resident",
            "hbm": {"bytes_per_step": int(sb), "achieved_GBs": round(sb / ssec / 1e9, 1),
                    "frac": round(sb / ssec / 1e9 / HBM_PEAK_GBS, 4)},
        }
        log(f"  stack: {ssec * 1e3:.3f} ms per pass, {st.D.T / ssec:.1f} tokens/s")
        gsec, gsame = st.time_graph(args.stack_steps)
        line["stack_48"]["graph"] = {"value": round(st.D.T / gsec, 1), "unit": "tokens/s",
                                     "ms_per_step": round(gsec * 1e3, 4), "equals_eager": gsame,
                                     "what": "the same pass captured once as a HIP graph and replayed"}
        log(f"  stack, HIP graph: {gsec * 1e3:.3f} ms per replay, equal to eager: {gsame}")
        pf = {}
        for hit, parts in ((1.0, 1), (0.5, 1), (1.0, 3)):
            psec, psame = st.time_prefetch(args.stack_steps, hit, parts)
            key = f"hit{hit:.1f}_{'s_up' if parts == 1 else 's_up+s_dn'}"
            pf[key] = {"value": round(st.D.T / psec, 1), "ms_per_step": round(psec * 1e3, 4), "equals_plain": psame}
            log(f"  stack, prefetch {key}: {psec * 1e3:.3f} ms per pass, equal to plain: {psame}")
        line["stack_48"]["prefetch"] = dict(pf, what="layer l+1's predicted groups' shared matrices read on a "
                                                    "second stream while layer l runs (synthetic predictor with "
                                                    "the stated hit rate)")
        del st
        torch.cuda.empty_cache()

    if not args.no_prefill:
        log("building prefill workload ...")
        wp = Workload(3, 1, host_init=args.host_init)
        pidx = wp.routed_indices()
        psec = wp.time_steps(args.prefill_steps, 2)
        pk = wp.kernel_times(args.prefill_steps)
        for k, (n, ms) in sorted(pk.items(), key=lambda kv: -kv[1][0] * kv[1][1]):
            log(f"  prefill kernel {k:22s} launches {n:5d} avg {ms:9.3f} ms")
        pname, proof = roofline_mfma(wp.D, pidx, pk)
        proof["traffic"] = stored_traffic(pname, "prefill_16k")
        add_rocprof(proof, "prefill_16k")
        total_fl = float(np.mean([step_flops(wp.D, ix) for ix in pidx]))
        line["prefill_16k"] = {
            "value": round(wp.D.T / psec, 1), "unit": "tokens/s", "steps": args.prefill_steps,
            "ms_per_step": round(psec * 1e3, 3),
            "workload": "prefill T=16384, one layer, router logits ~ N(0,1) (near-uniform load)",
            "roofline": proof,
            "step_mfma": {"flops_per_step": int(total_fl),
                          "achieved_TFLOPs": round(total_fl / psec / 1e12, 2),
                          "frac": round(total_fl / psec / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)},
        }
        if not args.no_cpu_baseline:
            line["prefill_16k"]["cpu_baseline"] = cpu_baseline_prefill(wp)
        del wp
        torch.cuda.empty_cache()
        if not args.no_mx:
            line["prefill_16k_mx"] = mx_prefill_line(args)
    if not args.no_calibrate:
        line["calibration"] = calibrate(em, torch)
        log(f"  calibration: {line['calibration']}")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
