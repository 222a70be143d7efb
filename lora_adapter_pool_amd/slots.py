"""Adapter slots: user adapter ids -> GPU pool slots, with a host cache.

The vLLM multi-LoRA article (LoRARequest rules; step 2; "限制与边界") fixes the
rules this follows:
  - an adapter is named by an integer id that is unique across adapters (the
    same id always means the same adapter);
  - max_loras is the number of distinct adapters one batch can use at once
    (pre-allocated GPU slots), not the number of adapters that can be loaded;
  - max_cpu_loras sizes a host-side cache of adapters;
  - max_lora_rank must cover every adapter's rank, else it cannot be loaded.
A request without adapter (None) runs the base model: its rows get slot -1.

Readings where the article is silent: both levels evict the least recently
used adapter (a GPU slot is only taken from an adapter the current batch does
not use; a host entry only from an adapter that is not resident on the GPU),
free slots are taken in increasing order, and a batch that needs more than
max_loras distinct adapters is an error (the caller's scheduler splits it).

SlotTable is the policy alone (pure Python, no GPU).  AdapterSlots drives a
LoraPool with it: host copies in pinned memory, loads into a slot on a side
stream (host-to-device copy, then lora_pool_load's pad-and-fold kernel), the
compute stream waiting on the load, and a slot overwritten only after the
compute stream has passed the last batch that read it.
"""
from __future__ import annotations

from collections import OrderedDict
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np

from . import _lib as L


class SlotError(L.LoraError):
    pass


@dataclass
class BatchSlots:
    """Slots of one batch: slot per row (-1 = no adapter), and the adapters
    that must be loaded before the batch runs as (adapter id, slot, evicted
    adapter id or None)."""
    ids: np.ndarray
    loads: List[tuple] = field(default_factory=list)


class SlotTable:
    """LRU policy of GPU slots (max_loras) and host cache (max_cpu_loras)."""

    def __init__(self, max_loras: int, max_cpu_loras: int, max_lora_rank: int):
        if max_loras < 1 or max_cpu_loras < max_loras:
            raise SlotError(L.LORA_E_SHAPE, "need 1 <= max_loras <= max_cpu_loras")
        self.max_loras, self.max_cpu_loras, self.max_lora_rank = (
            int(max_loras), int(max_cpu_loras), int(max_lora_rank))
        self.names: Dict[int, str] = {}          # every id ever registered -> name
        self.cpu: "OrderedDict[int, int]" = OrderedDict()   # cached id -> rank (LRU first)
        self.gpu: "OrderedDict[int, int]" = OrderedDict()   # resident id -> slot (LRU first)
        self.evicted_cpu: List[int] = []

    def register(self, adapter_id: int, name: str, rank: int) -> Optional[int]:
        """Add an adapter to the host cache; returns the id evicted from the
        cache to make room, or None."""
        adapter_id = int(adapter_id)
        if adapter_id < 0:
            raise SlotError(L.LORA_E_ID, f"adapter id must be >= 0, got {adapter_id}")
        if adapter_id in self.names and self.names[adapter_id] != name:
            raise SlotError(L.LORA_E_ID, f"adapter id {adapter_id} already names "
                                         f"'{self.names[adapter_id]}', not '{name}'")
        if adapter_id in self.cpu:
            raise SlotError(L.LORA_E_ID, f"adapter id {adapter_id} is already registered")
        if rank < 1 or rank > self.max_lora_rank:
            raise SlotError(L.LORA_E_RANK, f"adapter rank {rank} must be in "
                                           f"[1, max_lora_rank = {self.max_lora_rank}]")
        evicted = None
        if len(self.cpu) >= self.max_cpu_loras:
            evicted = next((a for a in self.cpu if a not in self.gpu), None)
            if evicted is None:
                raise SlotError(L.LORA_E_WORKSPACE, "host cache full of resident adapters")
            del self.cpu[evicted]
            self.evicted_cpu.append(evicted)
        self.names[adapter_id] = name
        self.cpu[adapter_id] = int(rank)
        return evicted

    def plan_batch(self, adapter_ids: Sequence[Optional[int]]) -> BatchSlots:
        """Slot of every row, and the loads the batch needs (LRU updates)."""
        wanted = []
        for a in adapter_ids:
            if a is None or a == -1:
                continue
            a = int(a)
            if a not in self.cpu:
                raise SlotError(L.LORA_E_ID, f"adapter id {a} is not registered "
                                             f"(or was evicted from the host cache)")
            if a not in wanted:
                wanted.append(a)
        if len(wanted) > self.max_loras:
            raise SlotError(L.LORA_E_SHAPE, f"batch uses {len(wanted)} adapters, "
                                            f"max_loras = {self.max_loras}")
        loads = []
        for a in wanted:
            if a in self.gpu:
                continue
            used = set(self.gpu.values())
            free = [s for s in range(self.max_loras) if s not in used]
            if free:
                slot, victim = free[0], None
            else:
                victim = next(b for b in self.gpu if b not in wanted)
                slot = self.gpu.pop(victim)
            self.gpu[a] = slot
            loads.append((a, slot, victim))
        for a in wanted:  # most recently used last, in order of first use
            self.gpu.move_to_end(a)
            self.cpu.move_to_end(a)
        ids = np.array([-1 if (a is None or a == -1) else self.gpu[int(a)] for a in adapter_ids],
                       dtype=np.int32)
        return BatchSlots(ids, loads)


class AdapterSlots:
    """A LoraPool whose slots hold adapters named by user ids."""

    def __init__(self, pool, max_cpu_loras: int, side_stream=None):
        import torch
        self.torch = torch
        self.pool = pool
        self.table = SlotTable(pool.max_loras, max_cpu_loras, pool.R)
        self.host: Dict[int, dict] = {}
        self.side = side_stream or torch.cuda.Stream()
        self.slot_free_ev: Dict[int, object] = {}   # slot -> event after its last read
        self.loaded_ev: Dict[int, object] = {}      # slot -> event after its last load

    def register(self, adapter_id: int, name: str, A: Sequence, B: Sequence, rank: int,
                 alpha: float, use_rslora: bool = False) -> None:
        """A[s] [rank, in_features], B[s] [out_s, rank] per slice, host arrays
        in the pool dtype's values; kept in pinned memory."""
        torch = self.torch
        S = len(self.pool.out_features)
        if len(A) != S or len(B) != S:
            raise SlotError(L.LORA_E_SHAPE, f"need {S} slices of A and B")
        for s in range(S):
            if tuple(A[s].shape) != (rank, self.pool.K) or \
                    tuple(B[s].shape) != (self.pool.out_features[s], rank):
                raise SlotError(L.LORA_E_SHAPE, f"slice {s}: A {tuple(A[s].shape)}, "
                                                f"B {tuple(B[s].shape)} for rank {rank}")
        evicted = self.table.register(adapter_id, name, rank)
        if evicted is not None:
            self.host.pop(evicted, None)

        def pinned(a):
            t = torch.as_tensor(np.ascontiguousarray(a, dtype=np.float32)).to(self.pool.tdtype)
            return t.pin_memory()
        self.host[int(adapter_id)] = {"A": [pinned(a) for a in A], "B": [pinned(b) for b in B],
                                      "rank": int(rank), "alpha": float(alpha),
                                      "rslora": bool(use_rslora)}

    def _load(self, adapter_id: int, slot: int, compute) -> None:
        torch = self.torch
        h = self.host[adapter_id]
        with torch.cuda.stream(self.side):
            ev = self.slot_free_ev.get(slot)
            if ev is not None:
                self.side.wait_event(ev)  # the slot's last reader has run
            dev = {k: [t.to("cuda", non_blocking=True) for t in h[k]] for k in ("A", "B")}
            for s in range(len(h["A"])):
                self.pool.load(slot, s, dev["A"][s], dev["B"][s], h["rank"], h["alpha"],
                               h["rslora"], stream=self.side)
            for k in ("A", "B"):  # staging tensors stay valid until the loads ran
                for t in dev[k]:
                    t.record_stream(self.side)
            done = torch.cuda.Event()
            done.record(self.side)
        self.loaded_ev[slot] = done

    def prepare(self, adapter_ids: Sequence[Optional[int]], stream=None) -> np.ndarray:
        """Slots for a batch's rows; loads what is missing on the side stream
        and makes `stream` (default: current) wait for it."""
        torch = self.torch
        compute = stream or torch.cuda.current_stream()
        bs = self.table.plan_batch(adapter_ids)
        for a, slot, _victim in bs.loads:
            self._load(a, slot, compute)
        for slot in set(int(s) for s in bs.ids if s >= 0):
            ev = self.loaded_ev.get(slot)
            if ev is not None:
                compute.wait_event(ev)
        return bs.ids

    def apply(self, x, y, adapter_ids: Sequence[Optional[int]], prefill=None,
              stream=None, ragged: bool = False) -> np.ndarray:
        """y += the LoRA delta of each row's adapter (None = base model).
        ragged: skip each slot's padded ranks (LoraPool.apply; same result)."""
        torch = self.torch
        compute = stream or torch.cuda.current_stream()
        ids = self.prepare(adapter_ids, compute)
        self.pool.apply(x, y, ids, prefill, stream=compute, ragged=ragged)
        done = torch.cuda.Event()
        done.record(compute)
        for slot in set(int(s) for s in ids if s >= 0):
            self.slot_free_ev[slot] = done
        return ids
