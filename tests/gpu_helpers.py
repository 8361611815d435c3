"""Shared pieces of the GPU tests: run the library on device tensors, compare with the oracle."""
import sys

import numpy as np
import torch

import shared_matrix_expert_amd as em
import synth

DEV = "cuda"


def say(*a):
    print(*a, flush=True, file=sys.stderr)


def bits_to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV)


def f32_to_dev(a) -> torch.Tensor:
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def tile_ok(D) -> bool:
    """Shapes the decode-tiled codes take (quant groups of 128, d and h multiples
    of 1024)."""
    return D.quant_group == 128 and D.d % 1024 == 0 and D.h % 1024 == 0


class Layer:
    """Device buffers for one layer and the two library calls.  By default the
    shared matrices also get their decode-tiled copies where the shape allows
    (as in the benchmark); tiled=False keeps the row-major ones only."""

    def __init__(self, D, weights: dict, tiled=None, persistent=False):
        self.D = D
        self.persistent = persistent
        if tiled is None:
            tiled = bool(weights) and tile_ok(D)
        self.W = em.tile_weights(D, weights) if tiled else weights
        self.ws = torch.empty(em.edge_moe_workspace_bytes(D), dtype=torch.uint8, device=DEV)

    def route(self, x, wr, bias, want_logits=True):
        D = self.D
        idx = torch.empty(D.T, D.top_k, dtype=torch.int32, device=DEV)
        w = torch.empty(D.T, D.top_k, dtype=torch.float32, device=DEV)
        lg = torch.empty(D.T, D.n_experts, dtype=torch.float32, device=DEV) if want_logits else None
        em.edge_moe_route(D, x, wr, bias, idx, w, lg, self.ws)
        return idx, w, lg

    def forward(self, x, idx, w, trace=False):
        D = self.D
        y = torch.empty(D.T, D.d, dtype=torch.float32, device=DEV)
        tr = None
        if trace:
            R = D.T * D.top_k
            tr = {"expert_offsets": torch.empty(D.n_experts + 1, dtype=torch.int32, device=DEV),
                  "row_token": torch.empty(R, dtype=torch.int32, device=DEV),
                  "row_slot": torch.empty(R, dtype=torch.int32, device=DEV),
                  "act": torch.empty(R, D.h, dtype=torch.int16, device=DEV),
                  "expert_out": torch.empty(R, D.d, dtype=torch.float32, device=DEV)}
        if self.persistent:
            em.edge_moe_forward_persistent(D, x, idx, w, self.W, y, self.ws, trace=tr)
        else:
            em.edge_moe_forward(D, x, idx, w, self.W, y, self.ws, trace=tr)
        return y, tr


def y_within_tolerance(y_gpu: np.ndarray, y_ref: np.ndarray):
    """|dy| <= 2e-3 + 2e-3 |y_ref| on every element; returns (ok, worst err/bound)."""
    err = np.abs(y_gpu.astype(np.float64) - y_ref)
    bound = 2e-3 + 2e-3 * np.abs(y_ref)
    ratio = float(np.max(err / bound)) if err.size else 0.0
    return bool(np.all(err <= bound)), ratio


def expected_permutation(idx: np.ndarray, E: int):
    """Rows sorted by (expert, token): offsets, row tokens and slots (numpy lexsort)."""
    T, k = idx.shape
    t = np.repeat(np.arange(T), k)
    j = np.tile(np.arange(k), T)
    e = idx.ravel()
    order = np.lexsort((t, e))
    offs = np.concatenate([[0], np.cumsum(np.bincount(e, minlength=E))])
    return offs.astype(np.int32), t[order].astype(np.int32), j[order].astype(np.int32)


def tile_cover_sample(offs, row_tok, P, G, T, target, seed=0, tile=128):
    """Tokens chosen so that every 128-row tile of the prefill GEMMs holds at
    least one of them: the shared-up rows (distinct tokens of each group, by
    token), the shared-down rows (each group's rows, by expert then token) and
    the rank-128 input rows (each expert's rows, by token).  Greedy over the
    tiles in order, then random tokens up to `target`."""
    rng = np.random.default_rng(seed)
    tiles = []                                   # arrays of the tokens in each tile
    for g in range(G):
        rows = row_tok[offs[g * P]:offs[(g + 1) * P]]
        for t0 in range(0, rows.size, tile):
            tiles.append(rows[t0:t0 + tile])
        u = np.unique(rows)
        for t0 in range(0, u.size, tile):
            tiles.append(u[t0:t0 + tile])
    for e in range(G * P):
        rows = row_tok[offs[e]:offs[e + 1]]
        for t0 in range(0, rows.size, tile):
            tiles.append(rows[t0:t0 + tile])
    chosen = set()
    for tl in tiles:
        if not chosen.intersection(tl.tolist()):
            chosen.add(int(rng.choice(tl)))
    n_cover = len(chosen)
    while len(chosen) < max(target, n_cover):
        chosen.add(int(rng.integers(T)))
    return np.array(sorted(chosen)), n_cover, len(tiles)
