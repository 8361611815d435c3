"""Host-side checks of the expert cache (edge_moe_cache_*), no GPU needed.

A cache created without slot tensors plans exactly as a real one (the same
placement, the same counts) and issues no copy, so its replacement policy is
checked here against:
  - hand-worked least-recently-used sequences (the textbook policy: on a miss
    with no free slot, the entry unused for the longest time leaves);
  - a separate model of the stated rule written in the test (resident experts
    of the batch refreshed first; a miss takes the group's first free slot,
    else its least recently used slot that the batch does not use, the lowest
    slot among equals), on random batch sequences;
  - invariants: every batch expert resident afterwards in a slot of its own
    group, distinct experts in distinct slots, hits + misses = distinct experts,
    bytes = misses x the per-expert bytes of the host tensors.
"""
import random

import numpy as np
import pytest
import torch

import shared_matrix_expert_amd as em
import synth


def _dims(G=4, P=8, k=3, d=256, h=512, r=8, gq=32):
    return synth.Dims(T=1, d=d, h=h, n_experts=G * P, experts_per_group=P, top_k=k,
                      delta_rank=r, lora_rank=4, quant_group=gq)


def _host(D, tiled=False):
    E, r, d, h = D.n_experts, D.delta_rank, D.d, D.h
    u8 = dict(dtype=torch.uint8)
    t = {"a_up": torch.zeros(E, r, d // 2, **u8), "a_up_scale": torch.zeros(E, r, d // D.gq(d), dtype=torch.int16),
         "b_up": torch.zeros(E, h, r // 2, **u8), "b_up_scale": torch.zeros(E, h, r // D.gq(r), dtype=torch.int16),
         "a_dn": torch.zeros(E, r, h // 2, **u8), "a_dn_scale": torch.zeros(E, r, h // D.gq(h), dtype=torch.int16),
         "b_dn": torch.zeros(E, d, r // 2, **u8), "b_dn_scale": torch.zeros(E, d, r // D.gq(r), dtype=torch.int16)}
    if tiled:
        t["a_up_t"] = torch.zeros_like(t["a_up"])
        t["a_dn_t"] = torch.zeros_like(t["a_dn"])
    return t


def _per_expert_bytes(host, E):
    return sum(v.numel() * v.element_size() for v in host.values()) // E


def _map(c, ids, k):
    idx = torch.tensor(ids, dtype=torch.int32).reshape(-1, k)
    out = torch.full_like(idx, -7)
    st = c.map(idx, out)
    return out.reshape(-1).tolist(), st


class Model:
    """The placement rule, written out independently of the library."""

    def __init__(self, G, P, S):
        self.P, self.S = P, S
        self.slot_exp = [-1] * (G * S)
        self.stamp = [0] * (G * S)
        self.tick = 0

    def where(self, e):
        return self.slot_exp.index(e) if e in self.slot_exp else -1

    def _place(self, e, st):
        i = self.where(e)
        if i >= 0:
            self.stamp[i] = self.tick
            st["hits"] += 1
            return
        g = e // self.P
        rng = range(g * self.S, (g + 1) * self.S)
        free = [j for j in rng if self.slot_exp[j] < 0]
        if free:
            j = free[0]
        else:
            cand = [j for j in rng if self.stamp[j] < self.tick]
            if not cand:
                return
            j = min(cand, key=lambda j: (self.stamp[j], j))
            st["evictions"] += 1
        self.slot_exp[j] = e
        self.stamp[j] = self.tick
        st["misses"] += 1

    def map(self, ids):
        distinct = list(dict.fromkeys(ids))
        per_group = {}
        for e in distinct:
            per_group[e // self.P] = per_group.get(e // self.P, 0) + 1
        if max(per_group.values()) > self.S:
            return None
        self.tick += 1
        for e in distinct:
            if self.where(e) >= 0:
                self.stamp[self.where(e)] = self.tick
        st = {"hits": 0, "misses": 0, "evictions": 0}
        for e in distinct:
            self._place(e, st)
        return [self.where(e) for e in ids], st

    def prefetch(self, ids):
        self.tick += 1
        st = {"hits": 0, "misses": 0, "evictions": 0}
        for e in ids:
            self._place(e, st)
        return st


def test_textbook_lru_sequence_one_group():
    # capacity 2, accesses A B A C B: miss miss hit miss(evicts B) miss(evicts A)
    D = _dims(G=1, P=8, k=1)
    host = _host(D)
    c = em.ExpertCache(D, 2, host)
    A, B, C = 3, 5, 6
    seen = []
    for e in (A, B, A, C, B):
        _, st = _map(c, [e], 1)
        seen.append((st["hits"], st["misses"], st["evictions"]))
    assert seen == [(0, 1, 0), (0, 1, 0), (1, 0, 0), (0, 1, 1), (0, 1, 1)]
    assert c.slot_of(A) == -1 and c.slot_of(B) >= 0 and c.slot_of(C) >= 0
    tot = c.totals()
    assert (tot["hits"], tot["misses"], tot["evictions"]) == (1, 4, 2)
    assert tot["bytes_copied"] == 4 * _per_expert_bytes(host, D.n_experts)


def test_textbook_lru_capacity_three():
    # capacity 3: 1 2 3 1 4 (evicts 2) 2 (evicts 3) 5 (evicts 1) 1 (evicts 4)
    D = _dims(G=1, P=8, k=1)
    c = em.ExpertCache(D, 3, _host(D))
    res = []
    for e in (1, 2, 3, 1, 4, 2, 5, 1):
        _, st = _map(c, [e], 1)
        res.append("h" if st["hits"] else "m")
    assert "".join(res) == "mmmhmmmm"
    assert sorted(e for e in range(8) if c.slot_of(e) >= 0) == [1, 2, 5]


def test_batch_experts_are_never_evicted_by_the_same_batch():
    # group of 3 slots holding 0 1 2 (2 least recent); batch {2, 3}: 3 must not evict 2
    D = _dims(G=1, P=8, k=2)
    c = em.ExpertCache(D, 3, _host(D))
    _map(c, [2, 0], 2)
    _map(c, [1, 0], 2)
    slots, st = _map(c, [2, 3], 2)
    assert st["hits"] == 1 and st["misses"] == 1 and st["evictions"] == 1
    assert c.slot_of(2) == slots[0] and c.slot_of(3) == slots[1] and c.slot_of(0) == -1
    assert c.slot_of(1) >= 0


def test_slots_stay_in_their_group_and_repeats_count_once():
    D = _dims(G=4, P=8, k=3)
    host = _host(D, tiled=True)
    S = 3
    c = em.ExpertCache(D, S, host)
    ids = [9, 9, 17, 9, 30, 17]            # two tokens, repeated experts
    slots, st = _map(c, ids, 3)
    assert st["misses"] == 3 and st["hits"] == 0
    for e, s in zip(ids, slots):
        assert (e // D.experts_per_group) * S <= s < (e // D.experts_per_group + 1) * S
    assert slots[0] == slots[1] == slots[3] and slots[2] == slots[5]
    assert len({slots[0], slots[2], slots[4]}) == 3
    assert st["bytes_copied"] == 3 * _per_expert_bytes(host, D.n_experts)


def test_group_over_capacity_is_rejected_and_changes_nothing():
    D = _dims(G=2, P=8, k=3)
    c = em.ExpertCache(D, 2, _host(D))
    _map(c, [0, 1, 8], 3)
    before = (c.totals(), [c.slot_of(e) for e in range(D.n_experts)])
    idx = torch.tensor([[2, 3, 4]], dtype=torch.int32)       # three distinct experts of group 0
    with pytest.raises(em.EdgeMoeError) as ei:
        c.map(idx, torch.empty_like(idx))
    assert ei.value.status == em.EDGE_MOE_EUNSUPPORTED
    assert (c.totals(), [c.slot_of(e) for e in range(D.n_experts)]) == before


def test_prefetch_then_map_hits_and_skips_past_capacity():
    D = _dims(G=2, P=8, k=2)
    c = em.ExpertCache(D, 2, _host(D))
    st = c.prefetch(torch.tensor([1, 2, 3, 9], dtype=torch.int32))   # 3 is past group 0's two slots
    assert st["misses"] == 3 and c.slot_of(3) == -1
    _, st = _map(c, [1, 9, 2, 9], 2)
    assert st["hits"] == 3 and st["misses"] == 0


def test_random_sequences_follow_the_stated_rule():
    rnd = random.Random(5)
    for G, P, S, k in ((4, 8, 3, 3), (2, 16, 5, 4), (1, 8, 8, 2), (3, 8, 1, 1)):
        D = _dims(G=G, P=P, k=k)
        host = _host(D)
        eb = _per_expert_bytes(host, D.n_experts)
        c = em.ExpertCache(D, S, host)
        m = Model(G, P, S)
        for step in range(300):
            if rnd.random() < 0.2:
                ids = [rnd.randrange(G * P) for _ in range(rnd.randint(0, 6))]
                st = c.prefetch(torch.tensor(ids, dtype=torch.int32))
                want = m.prefetch(ids)
                assert {x: st[x] for x in want} == want
                continue
            T = rnd.randint(1, 3)
            ids = [rnd.randrange(G * P) for _ in range(T * k)]
            want = m.map(ids)
            if want is None:
                with pytest.raises(em.EdgeMoeError):
                    _map(c, ids, k)
                continue
            slots, st = _map(c, ids, k)
            assert slots == want[0], (G, P, S, k, step)
            assert {x: st[x] for x in want[1]} == want[1]
            assert st["bytes_copied"] == st["misses"] * eb
            assert st["hits"] + st["misses"] == len(set(ids))
        assert [c.slot_of(e) for e in range(G * P)] == [m.where(e) for e in range(G * P)]


def test_create_and_map_validation():
    D = _dims(G=2, P=8, k=2)
    host = _host(D)
    for S in (0, 9, -1):
        with pytest.raises(ValueError):
            em.ExpertCache(D, S, host)
    partial = dict(host)
    del partial["b_dn"]
    with pytest.raises(ValueError):
        em.ExpertCache(D, 2, partial)
    c = em.ExpertCache(D, 2, host)
    for bad in ([[0, 16]], [[-1, 0]]):
        idx = torch.tensor(bad, dtype=torch.int32)
        with pytest.raises(em.EdgeMoeError) as ei:
            c.map(idx, torch.empty_like(idx))
        assert ei.value.status == em.EDGE_MOE_EINVAL
    with pytest.raises(em.EdgeMoeError):
        c.prefetch(torch.tensor([16], dtype=torch.int32))
    assert c.slot_of(16) == -2 and c.slot_of(0) == -1
    # an empty batch is valid and changes nothing
    assert _map(c, [], 2)[1]["misses"] == 0
    c.close()


def test_binding_checks_buffer_sizes():
    D = _dims(G=2, P=8, k=2)
    host = _host(D)
    short = dict(host)
    short["b_up_scale"] = host["b_up_scale"][:-1]
    with pytest.raises(ValueError, match="b_up_scale"):
        em.ExpertCache(D, 2, short)
    per = em.expert_tensor_bytes(D)
    for k, v in host.items():
        assert v.numel() * v.element_size() == D.n_experts * per[k]


def test_slot_dims_and_weights():
    D = synth.config(2).dims
    SD = em.slot_dims(D, 16)
    assert (SD.n_experts, SD.experts_per_group, SD.T, SD.d) == (8 * 16, 16, D.T, D.d)
    W = {"s_up": 1, "a_up": 2, "a_up_t": 3, "lora_up_u": 4}
    out = em.slot_weights(W, {"a_up": 20, "a_up_t": None})
    assert out == {"s_up": 1, "a_up": 20, "lora_up_u": 4}
    assert np.all(np.array(list(em.EXPERT_TENSOR_KEYS)) == np.array(
        ["a_up", "a_up_scale", "b_up", "b_up_scale", "a_dn", "a_dn_scale", "b_dn", "b_dn_scale",
         "a_up_t", "a_dn_t"]))
