"""Expert slot bank host logic (CPU, no GPU work): the plan against a plain model of the policy
("Hy4-preview Flash-MoE STQ1_0", slot-bank mode: experts streamed into a fixed set of slots on
demand): hits keep their slot, a miss takes an empty slot, else the least recently used slot no
expert of the step holds (lowest slot on ties); a step with more distinct experts than slots is
refused and changes nothing."""
import numpy as np
import pytest

import bit_quantized_moe_softmax_amd as M


class ModelBank:
    def __init__(self, E, S):
        self.E, self.S = E, S
        self.slot_of = [-1] * E
        self.expert_in = [-1] * S
        self.last = [0] * S
        self.step = 0

    def plan(self, ids):
        distinct = list(dict.fromkeys(int(e) for e in ids))
        if len(distinct) > self.S:
            return None
        self.step += 1
        for e in distinct:
            if self.slot_of[e] >= 0:
                self.last[self.slot_of[e]] = self.step
        copies = 0
        for e in distinct:
            if self.slot_of[e] >= 0:
                continue
            empty = [s for s in range(self.S) if self.expert_in[s] < 0]
            if empty:
                v = empty[0]
            else:
                cands = [s for s in range(self.S) if self.last[s] < self.step]
                v = min(cands, key=lambda s: (self.last[s], s))
            if self.expert_in[v] >= 0:
                self.slot_of[self.expert_in[v]] = -1
            self.expert_in[v] = e
            self.slot_of[e] = v
            self.last[v] = self.step
            copies += 1
        return list(self.slot_of), copies


@pytest.mark.parametrize("E,S", [(16, 8), (8, 8), (32, 5)])
def test_slot_bank_plan_matches_model(E, S):
    g = np.random.default_rng(E * 100 + S)
    bank = M.SlotBank(E, S, [100, 4, 100, 4, 100, 4])
    model = ModelBank(E, S)
    hits = misses = 0
    for step in range(200):
        n = int(g.integers(1, 2 * S + 2))
        # skewed ids, so experts come back and hits happen
        ids = np.minimum(g.zipf(1.5, n) - 1, E - 1).astype(np.int32)
        want = model.plan(ids)
        if want is None:
            with pytest.raises(M.MoeError):
                bank.plan(ids)
            continue
        slot_of, n_copies = bank.plan(ids)
        assert list(slot_of) == want[0] and n_copies == want[1]
        assert all(slot_of[e] >= 0 for e in ids)
        d = len(set(ids.tolist()))
        misses += want[1]
        hits += d - want[1]
    assert bank.stats() == (hits, misses) and hits > 0 and misses > 0


def test_slot_bank_argument_checks():
    with pytest.raises(M.MoeError):
        M.SlotBank(8, 9, [1] * 6)            # more slots than experts
    bank = M.SlotBank(8, 4, [1] * 6)
    with pytest.raises(M.MoeError):
        bank.plan(np.array([8], dtype=np.int32))   # expert id out of range
    slot_of, n = bank.plan(np.array([], dtype=np.int32))
    assert n == 0 and (slot_of == -1).all()


def test_slot_bank_plan_again_before_fetch_is_all_hits():
    """A step planned twice before its fetch: the second plan finds every expert resident,
    makes no copy of its own and keeps the slots (the first plan's copies stay pending)."""
    bank = M.SlotBank(16, 8, [100, 4, 100, 4, 100, 4])
    ids = np.array([3, 9, 3, 12], dtype=np.int32)
    slot_of, n = bank.plan(ids)
    again, n2 = bank.plan(ids)
    assert n == 3 and n2 == 0 and (again == slot_of).all()
    assert bank.stats() == (3, 3)
