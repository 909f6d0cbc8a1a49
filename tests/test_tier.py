"""Host-side checks of the off-HBM expert tier (no GPU): buffer sizes,
argument validation, and the slot plan against a plain least-recently-used
model written here (an ordered list of slots, most recent first)."""
import numpy as np
import pytest

import bit_dequant_expert_moe_amd as moe

D = moe.Dims(hidden=4096, inter=1024, n_experts=64, top_k=4, bits=4)
BLOB = moe.moe_expert_bytes(D)
A = 0x7f0000000000  # fake, aligned addresses: the host-only calls never touch them


def _tier(n_slots=8, t_max=1, n_layers=3, **kw):
    args = dict(d=D, host_ptrs=[A + l * (1 << 32) for l in range(n_layers)], host_stride=BLOB,
                slots=A + (1 << 40), slot_stride=BLOB, n_slots=n_slots,
                staging=A + (1 << 41), dev_scratch=A + (1 << 42), t_max=t_max)
    args.update(kw)
    return moe.Tier(**args)


class LRUModel:
    """Slots ordered most recent first; a miss takes the least recent slot
    that the current call has not used."""

    def __init__(self, n_slots, E):
        self.order = list(range(n_slots))
        self.key = [None] * n_slots
        self.where = {}
        self.E = E
        self.hits = self.misses = self.evictions = 0

    def call(self, layer, ids):
        used, slots, copies = set(), [], []
        for e in ids:
            if e < 0 or e >= self.E:
                slots.append(-1)
                copies.append(-1)
                continue
            k = (layer, e)
            if k in self.where:
                s = self.where[k]
                if s not in used:
                    self.hits += 1
                copies.append(-1)
            else:
                s = next(x for x in reversed(self.order) if x not in used)
                if self.key[s] is not None:
                    del self.where[self.key[s]]
                    self.evictions += 1
                self.key[s] = k
                self.where[k] = s
                self.misses += 1
                copies.append(e)
            self.order.remove(s)
            self.order.insert(0, s)
            used.add(s)
            slots.append(s)
        return slots, copies


def test_buffer_sizes():
    assert moe.moe_tier_staging_bytes(D, 1) == 2 * 256
    assert moe.moe_tier_device_bytes(D, 1) == 3 * 256
    assert moe.moe_tier_staging_bytes(D, 256) == 2 * 4096
    assert moe.moe_tier_staging_bytes(D, 0) == 0
    assert moe.moe_tier_device_bytes(D, 4097) == 0
    big = moe.moe_tier_workspace_bytes(D, 1024, 4)
    assert big >= moe.moe_workspace_bytes(D, 4)
    assert big >= moe.moe_workspace_bytes(moe.Dims(hidden=4096, inter=1024, n_experts=1024,
                                                   top_k=4, bits=4), 4)
    assert moe.moe_tier_workspace_bytes(D, 1025, 1) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(n_slots=3), -2),                 # fewer slots than one call's experts
    (dict(n_slots=7, t_max=2), -2),
    (dict(n_slots=1025), -2),
    (dict(t_max=0), -2),
    (dict(t_max=300, n_slots=1024), -2),   # t_max K > n_slots
    (dict(host_stride=BLOB - 16), -2),
    (dict(slot_stride=BLOB + 16), -4),
    (dict(slots=A + (1 << 40) + 64), -4),
    (dict(dev_scratch=A + 8), -4),
    (dict(staging=A + 8), -4),
    (dict(slots=None), -1),
    (dict(staging=None), -1),
    (dict(host_ptrs=[A, 0, A]), -1),
    (dict(n_layers=0, host_ptrs=[]), -2),
])
def test_create_validation(kw, status):
    n_layers = kw.pop("n_layers", 3)
    if "host_ptrs" not in kw:
        kw["host_ptrs"] = [A + l * (1 << 32) for l in range(n_layers)]
    with pytest.raises(moe.MoeError) as ei:
        _tier(**kw)
    assert ei.value.status == status


def test_plan_matches_lru_model():
    rng = np.random.default_rng(5)
    for n_slots, t_max in [(8, 1), (13, 2), (64, 3)]:
        tier = _tier(n_slots=n_slots, t_max=t_max)
        model = LRUModel(n_slots, D.n_experts)
        prev = {}
        for call in range(400):
            layer = int(rng.integers(0, 3))
            T = int(rng.integers(1, t_max + 1))
            # tokens reuse recent experts of the layer often, as decode does
            ids = []
            for t in range(T):
                row = []
                while len(row) < 4:
                    if prev.get(layer) and rng.random() < 0.6:
                        e = int(rng.choice(prev[layer]))
                    else:
                        e = int(rng.integers(0, D.n_experts))
                    if e not in row:
                        row.append(e)
                ids.append(row)
            if call % 37 == 0:
                ids[0][3] = -1  # an invalid id maps to no slot
            prev[layer] = [e for r in ids for e in r if e >= 0]
            flat = np.array(ids, dtype=np.int32).reshape(-1)
            slots, copies = tier.plan(layer, flat, T)
            ms, mc = model.call(layer, flat.tolist())
            assert slots.tolist() == ms, (call, flat, slots, ms)
            assert copies.tolist() == mc
        st = tier.stats()
        assert (st["hits"], st["misses"], st["evictions"]) == (model.hits, model.misses,
                                                                 model.evictions)
        assert st["bytes"] == model.misses * BLOB
        tier.close()


def test_plan_hand_worked():
    # 8 empty slots, most recent first 0..7: misses fill from slot 7 down.
    tier = _tier(n_slots=8, t_max=2)
    # call 1, two tokens: the repeats (4 in token 0 and 1, 1 in both tokens)
    # take one slot and one copy each
    slots, copies = tier.plan(0, np.array([1, 2, 3, 4, 4, 5, 1, 6], np.int32), 2)
    assert slots.tolist() == [7, 6, 5, 4, 4, 3, 7, 2]
    assert copies.tolist() == [1, 2, 3, 4, -1, 5, -1, 6]
    # now, most recent first: 2(6) 7(1) 3(5) 4(4) 5(3) 6(2) 0(-) 1(-)
    # call 2: 1 hits; 7 and 8 take the empty slots 1 and 0; 9 evicts expert 2
    # (least recent), so 2 misses in turn and evicts 3, and so on
    slots2, copies2 = tier.plan(0, np.array([1, 7, 8, 9, 2, 3, 10, 11], np.int32), 2)
    assert slots2.tolist() == [7, 1, 0, 6, 5, 4, 3, 2]
    assert copies2.tolist() == [-1, 7, 8, 9, 2, 3, 10, 11]
    st = tier.stats()
    assert (st["hits"], st["misses"], st["evictions"]) == (1, 13, 5)
    # the same expert id of another layer is another blob
    s3, c3 = tier.plan(1, np.array([1, 2, 3, 4], np.int32), 1)
    assert c3.tolist() == [1, 2, 3, 4]
    with pytest.raises(moe.MoeError):
        tier.plan(3, np.array([1, 2, 3, 4], np.int32), 1)   # no such layer
    with pytest.raises(moe.MoeError):
        tier.plan(0, np.array([1, 2, 3, 4] * 3, np.int32), 3)  # T above t_max
    tier.close()
