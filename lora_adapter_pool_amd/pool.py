"""A rank-padded adapter pool in HBM plus the per-call workspace of lora_apply.

Thin owner of device memory (torch tensors) around the C ABI: it allocates the
pool once ([vLLM] step 2 of the vLLM offline multi-LoRA article: max_loras
slots pre-allocated at max_lora_rank), loads adapters through lora_pool_load and
calls lora_apply with a device workspace and a small ring of pinned host
staging buffers (a buffer is reused only after the stream has passed the call
that last read it).  It records the rank loaded into each slot and slice, so
apply(..., ragged=True) can pass each slot's true rank to lora_apply_ranked.
"""
from __future__ import annotations

from typing import List, Optional, Sequence

import numpy as np

from . import _lib as L


class LoraPool:
    def __init__(self, dtype: str, max_loras: int, max_lora_rank: int, in_features: int,
                 out_features: Sequence[int], device: str = "cuda", staging_slots: int = 3):
        import torch

        self.torch = torch
        self.dtype = "bf16" if dtype in ("bf16", "bfloat16") else "f32"
        self.tdtype = torch.bfloat16 if self.dtype == "bf16" else torch.float32
        self.desc = L.make_desc(self.dtype, max_loras, max_lora_rank, in_features, out_features)
        L.lora_pool_validate(self.desc)
        eb = 2 if self.dtype == "bf16" else 4
        self.max_loras = int(max_loras)
        self.R = int(max_lora_rank)
        self.K = int(in_features)
        self.out_features = [int(o) for o in out_features]
        self.O = sum(self.out_features)
        self.device = device
        self.A = torch.zeros(L.lora_pool_bytes_A(self.desc) // eb, dtype=self.tdtype, device=device)
        self.B = torch.zeros(L.lora_pool_bytes_B(self.desc) // eb, dtype=self.tdtype, device=device)
        # rank last loaded into each (slot, slice); 0 = nothing loaded (zeros)
        self.loaded_ranks = np.zeros((self.max_loras, len(self.out_features)), np.int32)
        self._ws = None
        self._staging: List[list] = [[None, None] for _ in range(max(1, staging_slots))]
        self._next = 0

    # views in the documented layouts
    def A_view(self):
        return self.A.view(self.max_loras, len(self.out_features), self.R, self.K)

    def B_view(self):
        return self.B.view(self.max_loras, self.O, self.R)

    def load(self, slot: int, slice_: int, A_src, B_src, rank: int, alpha: float,
             use_rslora: bool = False, stream=None) -> None:
        L.lora_pool_load(self.desc, self.A, self.B, slot, slice_, A_src, B_src, rank, alpha,
                         use_rslora, stream=stream)
        self.loaded_ranks[slot, slice_] = rank

    def clear(self, slot: int, stream=None) -> None:
        L.lora_pool_clear(self.desc, self.A, self.B, slot, stream=stream)
        self.loaded_ranks[slot, :] = 0

    def merge(self, slot: int, slice_: int, W, W_out=None, stream=None):
        """Merged-weight mode: W_out (default: a new tensor) = W + s B A of the
        adapter in `slot`, for the base weight W [out_s, in] of slice `slice_`."""
        if W.dtype != self.tdtype or not W.is_contiguous():
            raise L.LoraError(L.LORA_E_DTYPE, "W must be a contiguous tensor of the pool dtype")
        if tuple(W.shape) != (self.out_features[slice_], self.K):
            raise L.LoraError(L.LORA_E_SHAPE, f"W must be [{self.out_features[slice_]}, {self.K}]")
        out = self.torch.empty_like(W) if W_out is None else W_out
        if out.dtype != W.dtype or out.shape != W.shape or not out.is_contiguous():
            raise L.LoraError(L.LORA_E_SHAPE, "W_out must match W")
        st = self.torch.cuda.current_stream() if stream is None else stream
        L.lora_merge_weights(self.desc, self.A, self.B, slot, slice_, W, out, stream=st)
        return out

    def slot_ranks(self) -> np.ndarray:
        """int32[max_loras]: the largest rank loaded into each slot; a slot with
        nothing loaded holds zeros and reports 1 (any rank gives a zero delta)."""
        return np.maximum(self.loaded_ranks.max(axis=1), 1).astype(np.int32)

    def workspace(self, T: int):
        need = L.lora_apply_workspace_bytes(self.desc, T)
        if self._ws is None or self._ws.numel() < need:
            self._ws = self.torch.empty(max(need, 256), dtype=self.torch.uint8, device=self.device)
        return self._ws

    def _staging_buffer(self, T: int, stream):
        need = L.lora_apply_host_meta_bytes(self.desc, T)
        slot = self._staging[self._next]
        self._next = (self._next + 1) % len(self._staging)
        buf, ev = slot
        if ev is not None:
            ev.synchronize()  # the stream has passed the call that last read this buffer
        if buf is None or buf.numel() < need:
            buf = self.torch.empty(max(need, 64), dtype=self.torch.uint8, pin_memory=True)
            slot[0] = buf
        return slot, buf, need

    def apply(self, x, y, ids, prefill=None, bgmv_max_rank: int = 0, stream=None,
              ragged: bool = False) -> None:
        """y (in place) += per-row LoRA delta for x; ids int32 per row (-1 = none).
        ragged: skip each slot's padded ranks (same result)."""
        torch = self.torch
        T = int(x.shape[0])
        ids = np.ascontiguousarray(np.asarray(ids, dtype=np.int32))
        pre = None if prefill is None else np.ascontiguousarray(np.asarray(prefill, dtype=np.uint8))
        if ids.shape[0] != T or (pre is not None and pre.shape[0] != T):
            raise L.LoraError(L.LORA_E_SHAPE, "ids / prefill length must equal the token count")
        ws = self.workspace(T)
        slot, buf, need = self._staging_buffer(T, stream)
        st = torch.cuda.current_stream() if stream is None else stream
        if ragged:
            L.lora_apply_ranked(self.desc, self.A, self.B, x, y, T, ids, pre, bgmv_max_rank,
                                self.slot_ranks(), ws, ws.numel(), buf, buf.numel(), stream=st)
        else:
            L.lora_apply(self.desc, self.A, self.B, x, y, T, ids, pre, bgmv_max_rank, ws,
                         ws.numel(), buf, buf.numel(), stream=st)
        ev = slot[1] or torch.cuda.Event()
        ev.record(st)
        slot[1] = ev
