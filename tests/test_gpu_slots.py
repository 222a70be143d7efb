"""Adapter slots on the GPU: batches named by user adapter ids, run back to
back while slots are loaded on a side stream and reused; every batch matches
the oracle for the adapters it named, and the resident slots hold exactly the
oracle's expected pool contents."""
import dataclasses

import numpy as np
import pytest

import lora_adapter_pool_amd as L
import oracle
import workloads as W
from gpu_helpers import check_rows, to_dev
from lora_adapter_pool_amd.slots import AdapterSlots, SlotError

pytestmark = pytest.mark.gpu


def test_slots_back_to_back_batches():
    import torch
    K, outs, R = 520, (264, 136), 16
    user_ids = [11, 22, 33, 44, 55]
    rng = np.random.default_rng(21)
    ranks = {a: int(rng.choice([8, 16])) for a in user_ids}
    alphas = {a: 2.0 * ranks[a] for a in user_ids}
    adapters = W._draw_slots(rng, "bf16", K, list(outs), ranks, alphas, rslora=False)
    pool = L.LoraPool("bf16", 3, R, K, list(outs))
    slots = AdapterSlots(pool, max_cpu_loras=5)
    for a in user_ids:
        ad = adapters[a]
        slots.register(a, f"adapter-{a}", ad.A, ad.B, ad.rank, ad.alpha)

    batches = []
    for i in range(10):
        T = int(rng.integers(20, 60))
        use = list(rng.choice(user_ids, size=int(rng.integers(1, 4)), replace=False))
        ids = [int(rng.choice(use)) if rng.random() > 0.15 else None for _ in range(T)]
        pre = (rng.random(T) < 0.5).astype(np.uint8)
        x = W.to_dtype_values(rng.standard_normal((T, K)), "bf16")
        y = W.to_dtype_values(rng.standard_normal((T, sum(outs))), "bf16")
        batches.append((ids, pre, x, y))
    outs_dev = []
    for ids, pre, x, y in batches:          # back to back, no synchronisation
        xd, yd = to_dev(x, "bf16"), to_dev(y, "bf16")
        slots.apply(xd, yd, ids, pre)
        outs_dev.append(yd)
    torch.cuda.synchronize()
    for i, ((ids, pre, x, y), yd) in enumerate(zip(batches, outs_dev)):
        wl = W.Workload("slots", "bf16", K, list(outs), 3, R, adapters,
                        np.array([-1 if a is None else a for a in ids], np.int32), pre, x, y)
        check_rows(wl, yd, label=f"slots batch {i}")

    # the resident slots hold the oracle's padded, folded adapters, bit for bit
    exp_wl = W.Workload("slots", "bf16", K, list(outs), 3, R, adapters,
                        np.zeros(1, np.int32), np.zeros(1, np.uint8),
                        np.zeros((1, K), np.float32), np.zeros((1, sum(outs)), np.float32))
    exp = oracle.expected_pool(exp_wl)
    Av = pool.A_view().float().cpu().numpy()
    Bv = pool.B_view().float().cpu().numpy()
    assert len(slots.table.gpu) == 3
    for a, slot in slots.table.gpu.items():
        for s in range(len(outs)):
            assert np.array_equal(Av[slot, s].view(np.uint32), exp[a]["A"][s].view(np.uint32))
        Bexp = np.concatenate([exp[a]["B"][s] for s in range(len(outs))], axis=0)
        assert np.array_equal(Bv[slot].view(np.uint32), Bexp.view(np.uint32))

    # a sixth adapter pushes the least recently used non-resident one out of the
    # host cache; naming it again is an error
    ad = adapters[11]
    resident = set(slots.table.gpu)
    gone = next(a for a in slots.table.cpu if a not in resident)
    slots.register(66, "adapter-66", ad.A, ad.B, ad.rank, ad.alpha)
    with pytest.raises(SlotError):
        slots.apply(to_dev(batches[0][2][:1], "bf16"), to_dev(batches[0][3][:1], "bf16"), [gone])


def test_slots_ragged_equals_padded():
    """Slots loaded and reused between batches, applied with each slot's true
    rank: bit for bit the padded result, batch by batch (batches large enough
    that the plan goes through device records, which carry the rank)."""
    import torch
    K, outs, R = 520, (264,), 32
    user_ids = [1, 2, 3, 4]
    rng = np.random.default_rng(22)
    ranks = {a: int(rng.choice([8, 16])) for a in user_ids}
    adapters = W._draw_slots(rng, "bf16", K, list(outs), ranks,
                             {a: 2.0 * ranks[a] for a in user_ids}, rslora=False)
    pools = [L.LoraPool("bf16", 2, R, K, list(outs)) for _ in range(2)]
    runs = [AdapterSlots(p, max_cpu_loras=4) for p in pools]
    for sl in runs:
        for a in user_ids:
            ad = adapters[a]
            sl.register(a, f"adapter-{a}", ad.A, ad.B, ad.rank, ad.alpha)
    for i in range(5):
        T = int(rng.integers(600, 800))
        use = list(rng.choice(user_ids, size=2, replace=False))
        ids = [int(rng.choice(use)) if rng.random() > 0.1 else None for _ in range(T)]
        x = to_dev(W.to_dtype_values(rng.standard_normal((T, K)), "bf16"), "bf16")
        y = to_dev(W.to_dtype_values(rng.standard_normal((T, sum(outs))), "bf16"), "bf16")
        ys = [y.clone(), y.clone()]
        runs[0].apply(x, ys[0], ids)
        runs[1].apply(x, ys[1], ids, ragged=True)
        torch.cuda.synchronize()
        assert torch.equal(ys[0].view(torch.int16), ys[1].view(torch.int16)), f"batch {i}"
        assert pools[1].slot_ranks().tolist() == [
            ranks[a] for a in sorted(runs[1].table.gpu, key=lambda a: runs[1].table.gpu[a])]
