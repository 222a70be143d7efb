"""Helpers of the GPU parity tests: load a workload's adapters into a pool,
run the HIP path through the C ABI, compare with the fp64 oracle."""
from __future__ import annotations

import sys

import numpy as np

import lora_adapter_pool_amd as L
import oracle

TOL = {"f32": 1e-5, "bf16": 1e-2}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def torch_dtype(dtype):
    import torch
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def to_dev(a, dtype):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch_dtype(dtype)).cuda()


def make_pool(wl, R=None, host_source=False):
    pool = L.LoraPool(wl.dtype, wl.max_loras, R or wl.max_lora_rank, wl.in_features,
                      wl.out_features)
    for a, ad in sorted(wl.slots.items()):
        for s in range(wl.num_slices):
            if host_source:
                import torch
                A = torch.from_numpy(np.ascontiguousarray(ad.A[s])).to(torch_dtype(wl.dtype))
                B = torch.from_numpy(np.ascontiguousarray(ad.B[s])).to(torch_dtype(wl.dtype))
                pool.load(a, s, A.contiguous(), B.contiguous(), ad.rank, ad.alpha, ad.use_rslora)
            else:
                pool.load(a, s, to_dev(ad.A[s], wl.dtype), to_dev(ad.B[s], wl.dtype), ad.rank,
                          ad.alpha, ad.use_rslora)
    return pool


def y_to_np(y):
    import torch
    return y.to(torch.float32).cpu().numpy().astype(np.float64)


def run_apply(wl, pool=None, bgmv_max_rank=0, x=None, ids=None, prefill=None, y=None):
    import torch
    pool = pool or make_pool(wl)
    xd = to_dev(wl.x if x is None else x, wl.dtype)
    yd = to_dev(wl.y_in, wl.dtype) if y is None else y
    pool.apply(xd, yd, wl.ids if ids is None else ids, wl.prefill if prefill is None else prefill,
               bgmv_max_rank=bgmv_max_rank)
    torch.cuda.synchronize()
    return yd


def run_entry_points(wl, pool, mode, bgmv_max_rank=0):
    """Drive the four grouped entry points directly with device metadata from
    the library's host builder; returns (y, v_sgmv, v_bgmv, meta)."""
    import torch
    m = L.lora_build_meta(wl.ids, wl.prefill, wl.max_loras, pool.R, bgmv_max_rank)
    xd = to_dev(wl.x, wl.dtype)
    yd = to_dev(wl.y_in, wl.dtype)
    dev = {k: torch.from_numpy(np.ascontiguousarray(v.astype(np.int32))).cuda() if v.size else
           torch.zeros(1, dtype=torch.int32, device="cuda") for k, v in m.items()}
    S, R, T = wl.num_slices, pool.R, wl.T
    ns, nb = int(m["sgmv_perm"].size), int(m["bgmv_tok"].size)
    vs = torch.full((max(ns, 1), S * R), float("nan"), dtype=torch.float32, device="cuda")
    vb = torch.full((max(nb, 1), S * R), float("nan"), dtype=torch.float32, device="cuda")
    nseg = int(m["seg_ids"].size)
    if mode in ("both", "sgmv"):
        L.lora_sgmv_shrink(pool.desc, xd, pool.A, vs, dev["sgmv_perm"], dev["seg_starts"],
                           dev["seg_lens"], dev["seg_ids"], nseg, ns, T)
    if mode in ("both", "bgmv"):
        L.lora_bgmv_shrink(pool.desc, xd, pool.A, vb, dev["bgmv_tok"], dev["bgmv_ids"], nb, T)
    if mode in ("both", "sgmv"):
        L.lora_sgmv_expand(pool.desc, vs, pool.B, yd, dev["sgmv_perm"], dev["seg_starts"],
                           dev["seg_lens"], dev["seg_ids"], nseg, ns, T)
    if mode in ("both", "bgmv"):
        L.lora_bgmv_expand(pool.desc, vb, pool.B, yd, dev["bgmv_tok"], dev["bgmv_ids"], nb, T)
    torch.cuda.synchronize()
    return yd, vs, vb, m


def plan_v(plan, S, R, fill=0.0):
    """fp32 v for a plan's stages: every K-split partial of every row."""
    import torch
    rows = plan["num_sgmv_rows"] + plan["num_bgmv_rows"]
    parts = max(plan["ksplit"], plan["ksplit_wave"])
    return torch.full((parts * max(rows, 1), S * R), fill, dtype=torch.float32, device="cuda")


_ORACLE_CACHE = {}


def _digest(wl):
    import hashlib
    h = hashlib.blake2b(digest_size=16)
    for a in (wl.ids, wl.x, wl.y_in):
        h.update(np.ascontiguousarray(a).tobytes())
    for a in sorted(wl.slots):
        ad = wl.slots[a]
        h.update(repr((a, ad.rank, ad.alpha, ad.use_rslora)).encode())
        for m in list(ad.A) + list(ad.B):
            h.update(np.ascontiguousarray(m).tobytes())
    return (wl.dtype, tuple(wl.out_features), h.hexdigest())


def oracle_rows(wl, rows):
    """The fp64 oracle on `rows`; the result for a whole workload is kept, so
    tests that check the same batch (the same inputs) compute it once."""
    key = _digest(wl)
    full = _ORACLE_CACHE.get(key)
    if full is None and len(rows) == wl.T:
        full = oracle.lora_forward_rows(wl)
        _ORACLE_CACHE.clear()       # one full-size batch at a time (memory)
        _ORACLE_CACHE[key] = full
    if full is not None:
        return full[np.asarray(rows, np.int64)]
    return oracle.lora_forward_rows(wl, rows)


def zero_y(wl):
    """The same batch with y_in = 0: y_out is then the delta alone, rounded once
    to the dtype, so the tolerance measures the delta itself."""
    import dataclasses
    return dataclasses.replace(wl, y_in=np.zeros_like(wl.y_in), name=wl.name + "_y0")


# Delta-only bar for bf16 outputs with y_in = 0: the one rounding of the
# output is at most 2^-9 of each element, and the fp32 sums (and the hi + lo
# bf16 pair that carries v into the MFMA expands, about 2^-17 of v) add far
# less, so 2^-8 leaves a factor two over the rounding alone.
DELTA_TOL_BF16 = 2.0 ** -8


def check_rows(wl, y_gpu, rows=None, tol=None, label=""):
    """Active rows within tolerance of the oracle; none rows bit-identical."""
    import torch
    rows = list(range(wl.T)) if rows is None else list(rows)
    idx = torch.as_tensor(rows, dtype=torch.long, device=y_gpu.device)
    yg = y_to_np(y_gpu.index_select(0, idx))
    ref = oracle_rows(wl, rows)
    act = np.asarray([wl.ids[r] >= 0 for r in rows])
    tol = TOL[wl.dtype] if tol is None else tol
    err = oracle.rel_err_rows(yg[act], ref[act]) if act.any() else 0.0
    if (~act).any():
        y_in_bits = torch.from_numpy(np.ascontiguousarray(wl.y_in[np.asarray(rows)[~act]])).to(
            torch_dtype(wl.dtype))
        got_bits = y_gpu.index_select(0, idx[torch.as_tensor(~act, device=y_gpu.device)]).cpu()
        assert torch.equal(got_bits.view(torch.int16) if wl.dtype == "bf16" else
                           got_bits.view(torch.int32),
                           y_in_bits.view(torch.int16) if wl.dtype == "bf16" else
                           y_in_bits.view(torch.int32)), f"{label}: a row without adapter changed"
    say(f"  {label}: rows={len(rows)} active={int(act.sum())} rel_err={err:.3e} tol={tol:.0e}")
    assert err <= tol, f"{label}: rel err {err} > {tol}"
    return err
