"""Benchmark of the multi-LoRA delta path on one MI355X.

A step is one lora_apply call (host metadata build, metadata copy, shrink and
expand kernels) over one synthetic batch.  Default workload: decode batch of
64 single-token rows, in = out = 3072, 8 adapters of rank 16 (bf16, 10% rows
without adapter).  The adapter pool, x and y are replicated enough times
(>= 1 GiB in total) that every step reads cold HBM; steps rotate replicas.

Prints one JSON line.  Besides the headline numbers it reports:
  roofline      the dominant kernel's algorithmic bytes / its average launch time
                (HIP events around back-to-back launches on the launch stream)
  secondary     the same measurement for the long-prefill SGMV workload
                (in = out = 4096, 16 sequences of 64..1024 tokens, ranks padded to 64)
  cpu_baseline  the fp64 oracle timed on the host for a bounded sample
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
KERNEL_SRC = os.path.join(ROOT, "lora_adapter_pool_amd", "csrc", "lora_kernels.hip")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=400)
    p.add_argument("--warmup", type=int, default=40)
    p.add_argument("--workload", default="bgmv_decode",
                   choices=["bgmv_decode", "sgmv_prefill", "qkv_decode", "mlp_mixed"])
    p.add_argument("--replica-mib", type=float, default=1024.0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-secondary", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="seconds of oracle time per CPU leg (all cores, then one thread)")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--sweep", action="store_true",
                   help="also sweep BGMV decode over batch size, adapter count and rank")
    p.add_argument("--record-traffic", metavar="PMC_DIR", default=None,
                   help="write profiles/traffic.json from rocprofv3 counter runs and exit")
    return p.parse_args()


# ---------------------------------------------------------------- workloads

def make_workloads(name, seed):
    import workloads as W
    if name == "bgmv_decode":
        return [W.config_bgmv_decode(seed=seed)]
    if name == "sgmv_prefill":
        return [W.config_sgmv_prefill(seed=seed)]
    if name == "qkv_decode":
        return [W.config_qkv_decode(seed=seed)]
    gu, dn = W.config_mlp_mixed(seed=seed)
    return [gu, dn]


WORKLOAD_DESC = {
    "bgmv_decode": "BGMV decode bf16: in=out=3072, 64 single-token rows, 8 adapters rank 16 "
                   "alpha 32, 10% rows without adapter",
    "sgmv_prefill": "SGMV prefill bf16: in=out=4096, 16 sequences of 64..1024 tokens, 16 adapters "
                    "ranks {8,16,32,64} padded to 64",
    "qkv_decode": "fused QKV decode bf16: in=4096, q/k/v=4096/1024/1024, 256 tokens, 64 adapters "
                  "rank 16 Zipf(1.1), rsLoRA",
    "mlp_mixed": "mixed MLP bf16: gate_up 4096->2x14336 and down 14336->4096, 8 prefill sequences "
                 "+ 256 decode tokens, 32 adapters",
}


def algorithmic(wl):
    """Bytes and flops the method must move / do for one call (each active
    adapter's padded A and B once, x once per active row, v written and read in
    fp32, y read and written per active row), split by kernel stage."""
    e = 2 if wl.dtype == "bf16" else 4
    act = wl.ids >= 0
    Ta = int(act.sum())
    nact = len(set(wl.ids[act].tolist()))
    K, R, S, O = wl.in_features, wl.max_lora_rank, wl.num_slices, wl.O
    shrink = Ta * K * e + nact * S * R * K * e + Ta * S * R * 4
    expand = nact * R * O * e + Ta * S * R * 4 + 2 * Ta * O * e
    flops = 2 * Ta * R * (S * K + O)
    return {"Ta": Ta, "n_act": nact, "shrink_bytes": shrink, "expand_bytes": expand,
            "bytes": shrink + expand, "flops": flops, "shrink_flops": 2 * Ta * R * S * K,
            "expand_flops": 2 * Ta * R * O, "apply_bytes": shrink + expand, "apply_flops": flops}


class Setup:
    """Replicated pool / x / y for one workload, plus prebuilt device metadata."""

    def __init__(self, wl, replica_bytes, ragged=False):
        import torch
        import lora_adapter_pool_amd as L
        self.wl = wl
        self.L = L
        tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(tdt).cuda()  # noqa: E731
        pool = L.LoraPool(wl.dtype, wl.max_loras, wl.max_lora_rank, wl.in_features,
                          wl.out_features)
        for a, ad in sorted(wl.slots.items()):
            for s in range(wl.num_slices):
                pool.load(a, s, dev(ad.A[s]), dev(ad.B[s]), ad.rank, ad.alpha, ad.use_rslora)
        self.desc = pool.desc
        # ragged: each slot's true rank goes to lora_apply_ranked
        self.slot_ranks = pool.slot_ranks() if ragged else None
        x0, y0 = dev(wl.x), dev(wl.y_in)
        per = (pool.A.numel() + pool.B.numel() + x0.numel() + y0.numel()) * x0.element_size()
        self.nrep = max(1, min(4096, int(np.ceil(replica_bytes / per))))
        self.A = [pool.A] + [pool.A.clone() for _ in range(self.nrep - 1)]
        self.B = [pool.B] + [pool.B.clone() for _ in range(self.nrep - 1)]
        self.x = [x0] + [x0.clone() for _ in range(self.nrep - 1)]
        self.y = [y0] + [y0.clone() for _ in range(self.nrep - 1)]
        self.pA = [t.data_ptr() for t in self.A]
        self.pB = [t.data_ptr() for t in self.B]
        self.px = [t.data_ptr() for t in self.x]
        self.py = [t.data_ptr() for t in self.y]
        self.T = wl.T
        self.ids = np.ascontiguousarray(wl.ids.astype(np.int32))
        self.pre = np.ascontiguousarray(wl.prefill.astype(np.uint8))
        self.ws_bytes = L.lora_apply_workspace_bytes(self.desc, self.T)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device="cuda")
        self.mh_bytes = L.lora_apply_host_meta_bytes(self.desc, self.T)
        self.nstage = 8
        self.stage = [torch.empty(self.mh_bytes, dtype=torch.uint8, pin_memory=True)
                      for _ in range(self.nstage)]
        self.stage_ev = [None] * self.nstage
        # the batch's tile plan, copied once, for the kernel-only loops (the same
        # launches lora_apply makes after its own plan copy)
        self.plan_d, img, _ = L.lora_apply_plan(self.desc, self.ids, self.pre,
                                                slot_ranks=self.slot_ranks)
        self.plan = L.plan_struct(self.plan_d)
        # lora_apply skips the plan copy for plans of at most 48 wavefront tiles
        self.small_plan = self.plan_d["mfma_tiles"] == 0 and self.plan_d["wave_tiles"] <= 48
        self.image = torch.from_numpy(img if img.size else np.zeros(4, np.int32)).cuda()
        # host copy: a small plan then travels in the kernel arguments, as in lora_apply
        self.image_host = np.ascontiguousarray(img if img.size else np.zeros(4, np.int32))
        rows = self.plan_d["num_sgmv_rows"] + self.plan_d["num_bgmv_rows"]
        S, R = wl.num_slices, wl.max_lora_rank
        parts = max(self.plan_d["ksplit"], self.plan_d["ksplit_wave"])
        self.v = torch.zeros((parts * max(rows, 1), S * R), dtype=torch.float32,
                             device="cuda")
        self.bytes_per_rep = per
        # the arguments of every call, converted once: a step is one call of
        # the library's CPython binding, as a caller's serving loop would make
        # it (numpy's `.ctypes` and torch's data_ptr() build objects on every
        # access, and ctypes converts 14 arguments in about 1.6 us)
        self._desc_ref = ctypes.byref(self.desc)
        self._desc_a = ctypes.addressof(self.desc)
        from lora_adapter_pool_amd import _lib as LL
        self._pc = LL.pycall()
        self._fa = LL.entry_address("lora_apply")
        self._fr = LL.entry_address("lora_apply_ranked")
        self._ids_p = self.ids.ctypes.data
        self._pre_p = self.pre.ctypes.data
        self._ranks_p = self.slot_ranks.ctypes.data if self.slot_ranks is not None else None
        self._ws_p = self.ws.data_ptr()
        self._stage_p = [t.data_ptr() for t in self.stage]
        self._plan_ref = ctypes.byref(self.plan)
        self._image_p = self.image.data_ptr()
        self._image_host_p = self.image_host.ctypes.data
        self._v_p = self.v.data_ptr()
        self._lib = L.lib()
        torch.cuda.synchronize()

    def _apply(self, r, stage_ptr, stream_ptr):
        if self._ranks_p is None:
            return self._pc.apply(self._fa, self._desc_a, self.pA[r], self.pB[r], self.px[r],
                                  self.py[r], self.T, self._ids_p, self._pre_p, 0, self._ws_p,
                                  self.ws_bytes, stage_ptr, self.mh_bytes, stream_ptr)
        return self._pc.apply_ranked(self._fr, self._desc_a, self.pA[r], self.pB[r], self.px[r],
                                     self.py[r], self.T, self._ids_p, self._pre_p, 0,
                                     self._ranks_p, self._ws_p, self.ws_bytes, stage_ptr,
                                     self.mh_bytes, stream_ptr)

    def apply_step(self, i, stream_ptr):
        import torch
        L = self.L
        r = i % self.nrep
        if self.small_plan:
            # the plan travels in the kernel arguments: the GPU never reads the
            # staging buffer, so one buffer serves every call without events
            st = self._apply(r, self._stage_p[0], stream_ptr)
            if st != 0:
                raise RuntimeError(f"lora_apply failed: {L.last_error()}")
            return
        j = i % self.nstage
        if self.stage_ev[j] is not None:
            self.stage_ev[j].synchronize()
        st = self._apply(r, self._stage_p[j], stream_ptr)
        if st != 0:
            raise RuntimeError(f"lora_apply failed: {L.last_error()}")
        ev = self.stage_ev[j] or torch.cuda.Event()
        ev.record()
        self.stage_ev[j] = ev

    def kernel_launch(self, which, i, stream_ptr):
        """One launch group of the plan (replica i): 'shrink', 'expand', or
        'apply' (both stages in the one launch lora_apply makes for a small
        decode plan)."""
        lib = self._lib
        r = i % self.nrep
        d = self._desc_ref
        if which == "apply":
            st = lib.lora_plan_apply(d, self.px[r], self.pA[r], self.pB[r], self.py[r], self.T,
                                     self._plan_ref, self._image_p, self._image_host_p,
                                     self._ws_p, self.ws_bytes, stream_ptr)
        elif which == "shrink":
            st = lib.lora_plan_shrink(d, self.px[r], self.pA[r], self._v_p, self.T,
                                      self._plan_ref, self._image_p, self._image_host_p,
                                      stream_ptr)
        else:
            st = lib.lora_plan_expand(d, self._v_p, self.pB[r], self.py[r], self.T,
                                      self._plan_ref, self._image_p, self._image_host_p,
                                      stream_ptr)
        if st != 0:
            raise RuntimeError(f"{which} failed: {self.L.last_error()}")

    def kernels(self):
        """Names of the kernels each launch group runs for this batch."""
        return stage_kernels(self.wl)


def time_kernel(setups, which, launches, warm, stream_ptr):
    """Average duration of one launch group ('shrink' / 'expand') over
    back-to-back launches, from HIP events recorded on the launch stream (the
    stream torch's events use) around the loop."""
    import torch
    for i in range(warm):
        for s in setups:
            s.kernel_launch(which, i, stream_ptr)
    n = 0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(launches):
        for s in setups:
            s.kernel_launch(which, warm + i, stream_ptr)
            n += 1
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / max(n, 1)  # us per launch group


def measure(setups, steps, warmup, stream_ptr):
    """Whole steps (every call of the workload) timed between two synchronizes."""
    import torch
    for i in range(warmup):
        for s in setups:
            s.apply_step(i, stream_ptr)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        for s in setups:
            s.apply_step(warmup + i, stream_ptr)
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def mfma_cap_tflops(a):
    """The MFMA rate a kernel group would need to run at the HBM roof: its
    arithmetic intensity (algorithmic flops per algorithmic byte) times 8 TB/s."""
    return a["flops"] / a["bytes"] * HBM_PEAK_GBS / 1e3


def workload_leg(name, seed, steps, stream_ptr, replica_bytes):
    """One named workload measured like the headline: whole lora_apply steps
    (wall clock between two synchronizes) and each launch group on its own
    (HIP events around back-to-back launches), with the algorithmic rate, its
    fraction of 8 TB/s, the HBM traffic rocprofv3 counted for that group (when
    recorded for the current kernel source) and the MFMA rate against both the
    bf16 peak and the rate the workload's arithmetic intensity allows at the HBM
    roof.  Returns (object, setups)."""
    wls = make_workloads(name, seed)
    setups = [Setup(w, replica_bytes / len(wls)) for w in wls]
    el = measure(setups, steps, min(10, steps), stream_ptr)
    st = el / steps
    algs = [algorithmic(s.wl) for s in setups]
    tot = {k: sum(a[k] for a in algs) for k in ("Ta", "bytes", "flops")}
    dom, pk = kernel_roofline(setups, stream_ptr, 50)
    kus = sum(r["step_us"] for r in pk.values())
    cap = mfma_cap_tflops(tot)
    tf = tot["flops"] / (kus * 1e-6) / 1e12
    per = {}
    for k, r in pk.items():
        traffic = load_traffic(k, name)
        per[k] = {"us": round(r["us"], 2), "GBs": round(r["GBs"], 1),
                  "frac": round(r["GBs"] / HBM_PEAK_GBS, 3),
                  "TFLOPs": round(r["TFLOPs"], 1),
                  "traffic": traffic,
                  "traffic_over_algorithmic": (round(traffic / r["bytes"], 3)
                                               if traffic else None),
                  "kernels": r["kernels"]}
    obj = {
        "workload": WORKLOAD_DESC[name],
        "calls_per_step": len(setups),
        "active_tokens": tot["Ta"],
        "tokens_per_s": tot["Ta"] / st, "ms_per_step": st * 1e3,
        "algorithmic_bytes_per_step": tot["bytes"],
        "achieved_GBs_step": tot["bytes"] / st / 1e9,
        "kernel_us_per_step": kus,
        "achieved_GBs_kernels": tot["bytes"] / (kus * 1e-6) / 1e9,
        "frac_hbm_peak_kernels": tot["bytes"] / (kus * 1e-6) / 1e9 / HBM_PEAK_GBS,
        "arithmetic_intensity": tot["flops"] / tot["bytes"],
        "mfma_tflops_kernels": tf,
        "mfma_util_of_peak": tf / MFMA_BF16_PEAK_TFLOPS,
        "mfma_cap_tflops": cap,
        "mfma_util_of_cap": tf / cap,
        "per_kernel": per,
        "dominant_kernel": dom,
    }
    for k, r in pk.items():
        log(f"[bench] {name} {k}: {r['us']:.2f} us/launch, {r['GBs']:.0f} GB/s, "
            f"{r['TFLOPs']:.1f} TFLOP/s")
    log(f"[bench] {name}: {st * 1e6:.1f} us/step, kernels {kus:.1f} us, "
        f"{obj['achieved_GBs_kernels']:.0f} GB/s ({obj['frac_hbm_peak_kernels']:.3f} of peak), "
        f"MFMA {tf:.0f} TFLOP/s = {tf / cap:.2f} of the intensity cap")
    return obj, setups


def ragged_decode_leg(seed, steps, stream_ptr, replica_bytes):
    """Decode batch whose adapters (rank 16) sit in a pool sized for rank 64:
    lora_apply with the padded slots against lora_apply_ranked with each slot's
    true rank; the padded ranks are most of the weight bytes here."""
    import dataclasses
    import torch
    import workloads as W
    wl = W.config_bgmv_decode(seed=seed, T=256, K=4096, O=4096, n_adapters=64, rank=16)
    wl = dataclasses.replace(wl, max_lora_rank=64)
    res = {"workload": "BGMV decode bf16: in=out=4096, 256 tokens, 64 adapters rank 16 in a "
                       "pool of rank 64, 10% rows without adapter"}
    for ragged in (False, True):
        st = [Setup(wl, replica_bytes, ragged=ragged)]
        t = measure(st, steps, 10, stream_ptr) / steps
        _, pk = kernel_roofline(st, stream_ptr, 50)
        # algorithmic bytes: the padded path must move rank-64 weights and v,
        # the ragged path only the adapters' rank 16
        alg = algorithmic(dataclasses.replace(wl, max_lora_rank=16) if ragged else wl)
        res["ragged" if ragged else "padded"] = {
            "us_per_step": round(t * 1e6, 2),
            "per_kernel_us": {k: round(r["us"], 2) for k, r in pk.items()},
            "per_kernel_GBs": {k: round(alg[f"{k}_bytes"] / (r["us"] * 1e3), 1)
                               for k, r in pk.items()}}
        del st
        torch.cuda.empty_cache()
    res["speedup"] = res["padded"]["us_per_step"] / res["ragged"]["us_per_step"]
    return res


def merge_leg(seed, stream_ptr, cpu=True):
    """Merged-weight mode: lora_merge_weights on one projection's weight (rank
    64 pool), timed with HIP events over back-to-back launches, against the
    bytes it must move (W read and written, the slot's A and B read once); and
    a single-adapter prefill batch run both ways: base GEMM then lora_apply, or
    the base GEMM on the merged weight alone (torch's GEMM for the base)."""
    import torch
    import lora_adapter_pool_amd as L
    import workloads as W
    res = {}
    for name, out_s, K in (("4096x4096", 4096, 4096), ("14336x4096", 14336, 4096)):
        pool = L.LoraPool("bf16", 2, 64, K, [out_s])
        rng = np.random.default_rng(seed)
        A = torch.from_numpy(rng.standard_normal((64, K), np.float32) / np.sqrt(K)).to(
            torch.bfloat16).cuda()
        B = torch.from_numpy(rng.standard_normal((out_s, 64), np.float32) * 0.02).to(
            torch.bfloat16).cuda()
        pool.load(0, 0, A, B, 64, 128.0)
        W0 = torch.from_numpy(W.draw_base_weight(seed, out_s, K, "bf16")).to(torch.bfloat16).cuda()
        # enough replicas of (W, W_out) that no launch finds its weights in a cache
        nrep = max(2, int(np.ceil(2 ** 30 / (2 * W0.numel() * 2))))
        Ws = [W0] + [W0.clone() for _ in range(nrep - 1)]
        Wos = [torch.empty_like(W0) for _ in range(nrep)]
        for i in range(5):
            L.lora_merge_weights(pool.desc, pool.A, pool.B, 0, 0, Ws[i % nrep], Wos[i % nrep],
                                 stream=stream_ptr)
        n = 50
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(n):
            L.lora_merge_weights(pool.desc, pool.A, pool.B, 0, 0, Ws[i % nrep], Wos[i % nrep],
                                 stream=stream_ptr)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / n
        nbytes = 2 * out_s * K * 2 + 64 * K * 2 + out_s * 64 * 2
        res[name] = {"us": round(us, 2), "GBs": round(nbytes / us / 1e3, 1),
                     "frac_hbm_peak": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 3),
                     "kernel": "merge_rows_kernel<2>"}  # (ranks <= 128; rank 64 here)
        del pool, A, B, W0, Ws, Wos
        torch.cuda.empty_cache()
    # one adapter for the whole batch: 16 sequences of 64..1024 tokens, in = out = 4096
    wl = W.config_sgmv_prefill(seed=seed, n_adapters=1, rank_choices=(16,), max_lora_rank=16)
    pool = L.LoraPool("bf16", 1, 16, 4096, [4096])
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).cuda()  # noqa
    ad = wl.slots[0]
    pool.load(0, 0, dev(ad.A[0]), dev(ad.B[0]), ad.rank, ad.alpha)
    Wb = dev(W.draw_base_weight(seed, 4096, 4096, "bf16"))
    Wt = Wb.t().contiguous()
    Wmt = pool.merge(0, 0, Wb).t().contiguous()
    x = dev(wl.x)

    def runtime():
        y = x @ Wt
        pool.apply(x, y, wl.ids, wl.prefill)
        return y

    def merged():
        return x @ Wmt

    out = {}
    for label, fn in (("base_gemm_plus_delta", runtime), ("merged_gemm", merged)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(20):
            fn()
        torch.cuda.synchronize()
        out[label] = round((time.perf_counter() - t0) / 20 * 1e6, 1)
    res["single_adapter_prefill_us"] = dict(out, tokens=int(wl.T))
    if cpu:
        # the oracle's merge (fp64 product, one rounding) on a 1024-row sample
        # of the 4096 x 4096 rank-64 case, scaled to the whole weight
        import oracle
        rng = np.random.default_rng(seed)
        slot = {"A": [rng.standard_normal((64, 4096)) / 64.0],
                "B": [rng.standard_normal((1024, 64)) * 0.02]}
        Ws = W.draw_base_weight(seed, 1024, 4096, "bf16")
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            oracle.merged_weight(Ws, slot, 0, "bf16")
            el = time.perf_counter() - t0
        res["cpu_oracle"] = {"us_4096x4096": round(el * 4 * 1e6, 1), "kind": "oracle",
                             "sample": "1024 of 4096 rows, scaled x4; one BLAS thread",
                             "cores": 1}
    return res


def device_meta_leg(s, steps, stream_ptr):
    """The delta path driven from device metadata: lora_build_meta_device, then
    the four grouped entry points with upper-bound sizes (num_segs = max_loras,
    rows = T), no host work per step and graph-capturable.  Reports the
    builder's own time (HIP events over back-to-back launches) and whole steps
    over the rotating replicas (wall clock between two synchronizes)."""
    import torch
    L = s.L
    lib = L.lib()
    wl, T, ML, R = s.wl, s.T, s.wl.max_loras, s.wl.max_lora_rank
    rows = {"sgmv_perm": T, "bgmv_tok": T, "bgmv_ids": T}
    meta = {k: torch.zeros(max(rows.get(k, ML), 1), dtype=torch.int32, device="cuda")
            for k in ("sgmv_perm", "seg_starts", "seg_lens", "seg_ids", "bgmv_tok", "bgmv_ids")}
    m = L._lib.lora_meta()
    for k, t in meta.items():
        setattr(m, k, ctypes.cast(t.data_ptr(), ctypes.POINTER(ctypes.c_int32)))
    counts = torch.zeros(4, dtype=torch.int32, device="cuda")
    ids_d = torch.from_numpy(s.ids).cuda()
    pre_d = torch.from_numpy(s.pre).cuda()
    SR = wl.num_slices * R
    v_s = torch.zeros((max(T, 1), SR), dtype=torch.float32, device="cuda")
    v_b = torch.zeros((max(T, 1), SR), dtype=torch.float32, device="cuda")
    d = ctypes.byref(s.desc)
    P = {k: t.data_ptr() for k, t in meta.items()}

    def build():
        return lib.lora_build_meta_device(ids_d.data_ptr(), pre_d.data_ptr(), T, ML, R, 0,
                                          ctypes.byref(m), counts.data_ptr(), stream_ptr)

    def step(i):
        r = i % s.nrep
        sts = [build(),
               lib.lora_sgmv_shrink(d, s.px[r], s.pA[r], v_s.data_ptr(), P["sgmv_perm"],
                                    P["seg_starts"], P["seg_lens"], P["seg_ids"], ML, T, T,
                                    stream_ptr),
               lib.lora_bgmv_shrink(d, s.px[r], s.pA[r], v_b.data_ptr(), P["bgmv_tok"],
                                    P["bgmv_ids"], T, T, stream_ptr),
               lib.lora_sgmv_expand(d, v_s.data_ptr(), s.pB[r], s.py[r], P["sgmv_perm"],
                                    P["seg_starts"], P["seg_lens"], P["seg_ids"], ML, T, T,
                                    stream_ptr),
               lib.lora_bgmv_expand(d, v_b.data_ptr(), s.pB[r], s.py[r], P["bgmv_tok"],
                                    P["bgmv_ids"], T, T, stream_ptr)]
        if any(sts):
            raise RuntimeError(f"device-metadata step failed: {L.last_error()}")

    for _ in range(10):
        build()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(100):
        build()
    e1.record()
    torch.cuda.synchronize()
    builder_us = e0.elapsed_time(e1) * 1e3 / 100
    for i in range(10):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(10 + i)
    torch.cuda.synchronize()
    step_us = (time.perf_counter() - t0) / steps * 1e6
    # lora_apply_device: the same device metadata, then a device-built plan of
    # 8-row tiles and the tile kernels (4 launches, no host work per batch)
    nws = L.lora_apply_device_workspace_bytes(s.desc, T)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")

    def plan_step(i):
        r = i % s.nrep
        if lib.lora_apply_device(d, s.pA[r], s.pB[r], s.px[r], s.py[r], T, ids_d.data_ptr(),
                                 pre_d.data_ptr(), 0, ws.data_ptr(), nws, stream_ptr):
            raise RuntimeError(f"lora_apply_device failed: {L.last_error()}")

    for i in range(10):
        plan_step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        plan_step(10 + i)
    torch.cuda.synchronize()
    plan_us = (time.perf_counter() - t0) / steps * 1e6
    # the same calls captured in a graph (20 calls over 20 replicas), replayed
    ncap = min(20, s.nrep)
    gs = torch.cuda.Stream()
    gs.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(gs):
        with torch.cuda.graph(graph, stream=gs):
            cap_ptr = torch.cuda.current_stream().cuda_stream
            for r in range(ncap):
                if lib.lora_apply_device(d, s.pA[r], s.pB[r], s.px[r], s.py[r], T,
                                         ids_d.data_ptr(), pre_d.data_ptr(), 0, ws.data_ptr(),
                                         nws, cap_ptr):
                    raise RuntimeError(f"lora_apply_device failed: {L.last_error()}")
    torch.cuda.current_stream().wait_stream(gs)
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    reps = max(5, steps // ncap)
    t0 = time.perf_counter()
    for _ in range(reps):
        graph.replay()
    torch.cuda.synchronize()
    graph_us = (time.perf_counter() - t0) / (reps * ncap) * 1e6
    a = algorithmic(wl)
    return {"builder_us": round(builder_us, 2), "step_us": round(step_us, 2),
            "tokens_per_s": a["Ta"] / (step_us * 1e-6), "launches_per_step": 5,
            "device_plan_step_us": round(plan_us, 2),
            "device_plan_tokens_per_s": a["Ta"] / (plan_us * 1e-6),
            "device_plan_graph_step_us": round(graph_us, 2),
            "counts": counts.cpu().tolist()[:3]}


def device_plan_leg(s, steps, stream_ptr):
    """lora_apply_device on a setup's batch: device ids -> device metadata and
    plan -> tile kernels, whole steps over the rotating replicas."""
    import torch
    L = s.L
    lib = L.lib()
    d = ctypes.byref(s.desc)
    ids_d = torch.from_numpy(s.ids).cuda()
    pre_d = torch.from_numpy(s.pre).cuda()
    nws = L.lora_apply_device_workspace_bytes(s.desc, s.T)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")

    ids_p, pre_p, ws_p = ids_d.data_ptr(), pre_d.data_ptr(), ws.data_ptr()

    def step(i):
        r = i % s.nrep
        if lib.lora_apply_device(d, s.pA[r], s.pB[r], s.px[r], s.py[r], s.T, ids_p, pre_p, 0,
                                 ws_p, nws, stream_ptr):
            raise RuntimeError(f"lora_apply_device failed: {L.last_error()}")

    for i in range(5):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(5 + i)
    torch.cuda.synchronize()
    step_us = (time.perf_counter() - t0) / steps * 1e6
    # the metadata builder alone on the same batch (HIP events)
    T, ML = s.T, s.wl.max_loras
    meta = {k: torch.zeros(max(T if k in ("sgmv_perm", "bgmv_tok", "bgmv_ids") else ML, 1),
                           dtype=torch.int32, device="cuda")
            for k in ("sgmv_perm", "seg_starts", "seg_lens", "seg_ids", "bgmv_tok", "bgmv_ids")}
    m = L._lib.lora_meta()
    for k, t in meta.items():
        setattr(m, k, ctypes.cast(t.data_ptr(), ctypes.POINTER(ctypes.c_int32)))
    counts = torch.zeros(4, dtype=torch.int32, device="cuda")

    def build():
        if lib.lora_build_meta_device(ids_d.data_ptr(), pre_d.data_ptr(), T, ML,
                                      s.wl.max_lora_rank, 0, ctypes.byref(m), counts.data_ptr(),
                                      stream_ptr):
            raise RuntimeError(f"lora_build_meta_device failed: {L.last_error()}")

    for _ in range(3):
        build()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(20):
        build()
    e1.record()
    torch.cuda.synchronize()
    return step_us, e0.elapsed_time(e1) * 1e3 / 20


def slot_load_leg(seed):
    """Adapter slots: time to make an adapter resident (pinned host copy ->
    device on the side stream, then the pad-and-fold kernel), cycling four
    adapters through two slots so every batch loads one; for a q_proj-like
    adapter (3072 -> 3072, rank 16) and a gate_up-like one (4096 -> 2 x 14336,
    rank 64)."""
    import torch
    import workloads as W
    from lora_adapter_pool_amd.slots import AdapterSlots
    import lora_adapter_pool_amd as L
    res = {}
    for name, K, outs, r in (("q_proj 3072x3072 r16", 3072, [3072], 16),
                             ("gate_up 4096x2x14336 r64", 4096, [14336, 14336], 64)):
        rng = np.random.default_rng(seed)
        ids = [1, 2, 3, 4]
        ads = W._draw_slots(rng, "bf16", K, outs, {a: r for a in ids},
                            {a: 2.0 * r for a in ids}, rslora=False)
        pool = L.LoraPool("bf16", 2, r, K, outs)
        sl = AdapterSlots(pool, max_cpu_loras=4)
        for a in ids:
            sl.register(a, f"a{a}", ads[a].A, ads[a].B, r, 2.0 * r)
        host_bytes = 2 * r * (K * len(outs) + sum(outs))
        for i in range(4):
            sl.prepare([ids[i % 4]])
        torch.cuda.synchronize()
        n = 40
        t0 = time.perf_counter()
        for i in range(n):
            sl.prepare([ids[i % 4]])
            torch.cuda.synchronize()
        us = (time.perf_counter() - t0) / n * 1e6
        res[name] = {"load_us": round(us, 1), "adapter_bytes": host_bytes,
                     "GBs": round(host_bytes / (us * 1e-6) / 1e9, 2)}
        del sl, pool
        torch.cuda.empty_cache()
    return res


def copy_bandwidth():
    import torch
    n = 1 << 28  # 256 Mi bf16 = 512 MiB per buffer
    a = torch.empty(n, dtype=torch.bfloat16, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    reps = 10
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) / 1e3 / reps
    del a, b
    return 2 * n * 2 / sec / 1e9, 2 * n * 2


def kernel_roofline(setups, stream_ptr, launches):
    """Per launch group (shrink, expand): average time and algorithmic-bytes
    rate; returns the dominant group (larger time per step)."""
    res = {}
    for which in setups[0].kernels():
        us = time_kernel(setups, which, launches, 10, stream_ptr)
        by = fl = 0
        names = []
        for s in setups:
            a = algorithmic(s.wl)
            by += a[f"{which}_bytes"]
            fl += a[f"{which}_flops"]
            names += s.kernels()[which]
        n = len(setups)
        res[which] = {"us": us, "bytes": by / n, "flops": fl / n,
                      "GBs": by / n / (us * 1e-6) / 1e9, "TFLOPs": fl / n / (us * 1e-6) / 1e12,
                      "step_us": us * n, "kernels": sorted(set(names))}
    dom = max(res, key=lambda k: res[k]["step_us"])
    return dom, res


TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")
COPY_BYTES = 2 * (1 << 28)  # the device-copy measurement moves 512 MiB each way


def kernel_source_sha():
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]


def load_traffic(stage, workload):
    """HBM bytes per launch group from committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE counters, valid only while the kernel source is unchanged."""
    if not os.path.exists(TRAFFIC_JSON):
        return None
    try:
        with open(TRAFFIC_JSON) as f:
            ent = json.load(f).get(f"{workload}:{stage}")
        if not ent or ent.get("kernel_source_sha") != kernel_source_sha():
            return None
        return float(ent["hbm_bytes_per_launch"])
    except (OSError, ValueError, KeyError):
        return None


def one_launch(wl, p):
    """Whether lora_apply runs this batch's plan as one launch: no MFMA tiles,
    at most 12 wavefront tiles, a bf16 pool and max_lora_rank <= 32."""
    if os.environ.get("LORA_ONEPASS_DECODE", "1").startswith("0"):
        return False
    return (wl.dtype == "bf16" and not p["mfma_tiles"] and 0 < p["wave_tiles"] <= 12
            and wl.max_loras <= 2 ** 28 and wl.max_lora_rank <= 32 and wl.T < 65536)


def stage_kernels(wl):
    """Kernel names of each launch group for a workload's batch (host-side
    plan only, no GPU)."""
    import lora_adapter_pool_amd as L
    d = L.make_desc(wl.dtype, wl.max_loras, wl.max_lora_rank, wl.in_features, wl.out_features)
    p, _, _ = L.lora_apply_plan(d, wl.ids, wl.prefill)
    tag = "unsigned short" if wl.dtype == "bf16" else "float"
    kb = 16 if wl.max_lora_rank <= 16 else 64
    if one_launch(wl, p):
        nt = 1 if wl.max_lora_rank <= 16 else 2
        share = -(-(-(-wl.in_features // 32)) // 8)
        cb = min(-(-share // 4) * 4, 16 if nt == 1 else 8)
        return {"apply": [f"decode_onepass_kernel<{nt}, {cb}, 5>"]}
    out = {"shrink": [], "expand": []}
    if p["mfma_tiles"]:
        # whole 64-wide K steps up to K = 8192: tiles staged by direct loads to LDS
        dma = wl.in_features % 64 == 0 and wl.in_features <= 8192
        # four LDS stages when the launch has at most one workgroup per compute
        # unit
        grid = p["mfma_tiles"] * len(wl.out_features) * p["ksplit"] * -(-wl.max_lora_rank // 64)
        stages = os.environ.get("LORA_DMA_STAGES")
        nst = (4 if stages.startswith("4") else 3) if stages else 4 if grid <= 256 else 3
        out["shrink"].append(f"shrink_mfma_dma_kernel<2, {nst}>" if dma else "shrink_mfma_kernel<2>")
        rows = wl.max_lora_rank <= 64 and wl.T * wl.O * 2 < 2 ** 31
        kp = 8 if p["ksplit"] > 4 else 4
        out["expand"].append(f"expand_mfma_rows_kernel<2, {kp}>" if rows else "expand_mfma_kernel<2>")
    if p["wave_tiles"]:
        # modes 3 / 4: records in the kernel arguments (up to 12 / 48 tiles),
        # 2: device image
        small = not p["mfma_tiles"]
        mode = (3 if p["wave_tiles"] <= 12 else 4 if p["wave_tiles"] <= 48 else 2) if small else 2
        R = wl.max_lora_rank
        if wl.dtype == "bf16" and R <= 64 and os.environ.get("LORA_TILE_MFMA_SHRINK", "1") != "0":
            # MFMA tiles of 8 rows: rank tiles of 16 and K chunks per batch,
            # partials of v summed by the expand (loaded in powers of two)
            nt = 1 if R <= 16 else 2 if R <= 32 else 4
            cb = {1: 8, 2: 6, 4: 4}[nt]
            kp = p["ksplit_wave"]
            kp2 = 1 if kp == 1 else 2 if kp == 2 else 4 if kp <= 4 else 8
            out["shrink"].append(f"shrink_tile_mfma_kernel<{nt}, {cb}, {mode}>")
            if os.environ.get("LORA_TILE_MFMA_EXPAND", "1") != "0" and wl.T * wl.O * 2 < 2 ** 31:
                out["expand"].append(f"expand_tile_mfma_kernel<{1 if R <= 32 else 2}, {kp2}, {mode}>")
            else:
                out["expand"].append(f"expand_wave_kernel<{tag}, 8, {kb}, {kp2}, {mode}>")
        else:
            out["shrink"].append(f"shrink_wave_kernel<{tag}, 8, 4, {mode}>")
            out["expand"].append(f"expand_wave_kernel<{tag}, 8, {kb}, 1, {mode}>")
    return out


def record_traffic(pmc_dir, workload, seed):
    """Write profiles/traffic.json entries for `workload` from two rocprofv3
    counter runs of this script: <pmc_dir>/fetch (--pmc FETCH_SIZE) and
    <pmc_dir>/write (--pmc WRITE_SIZE).  Both counters are scaled by what they
    read for the device-to-device copy of known size that every run makes."""
    import csv
    import glob

    def per_kernel(sub, counter):
        vals = {}
        for f in glob.glob(os.path.join(pmc_dir, sub, "*_counter_collection.csv")):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] != counter:
                    continue
                name = r["Kernel_Name"].split("(")[0].replace("void ", "").replace("lora::", "")
                vals.setdefault(name, []).append(float(r["Counter_Value"]) * 1024.0)
        return vals

    fetch, write = per_kernel("fetch", "FETCH_SIZE"), per_kernel("write", "WRITE_SIZE")
    # the copies of the bandwidth measurement are the largest copyBuffer dispatches
    cf = COPY_BYTES / max(fetch["__amd_rocclr_copyBuffer"])
    cw = COPY_BYTES / max(write["__amd_rocclr_copyBuffer"])
    data = {}
    if os.path.exists(TRAFFIC_JSON):
        data = json.load(open(TRAFFIC_JSON))
    sha = kernel_source_sha()
    wls = make_workloads(workload, seed)
    kern = {}
    for wl in wls:
        for k, v in stage_kernels(wl).items():
            kern.setdefault(k, set()).update(v)
    # calls of the workload whose launch group uses each kernel
    users = {}
    for wl in wls:
        for k, v in stage_kernels(wl).items():
            for n in v:
                users[(k, n)] = users.get((k, n), 0) + 1
    for stage, names in kern.items():
        # one launch group = one dispatch of each of its kernels; averaged over
        # the workload's calls like the algorithmic bytes (a kernel that only
        # some calls use counts for those)
        tot = 0.0
        for n in names:
            f, w = fetch.get(n), write.get(n)
            if not f or not w:
                raise SystemExit(f"no counters for {n} in {pmc_dir}")
            tot += ((sum(f) / len(f)) * cf + (sum(w) / len(w)) * cw) * users[(stage, n)] / len(wls)
        data[f"{workload}:{stage}"] = {
            "hbm_bytes_per_launch": tot, "kernels": sorted(names),
            "fetch_scale": cf, "write_scale": cw, "kernel_source_sha": sha}
    with open(TRAFFIC_JSON, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
    print(json.dumps({k: v for k, v in data.items() if k.startswith(workload + ":")}, indent=1))


def _oracle_rate(wl, rows, seconds):
    """The fp64 oracle on `rows` of `wl`, over and over on one BLAS thread,
    until `seconds` have passed: (active rows done, seconds)."""
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover
        threadpool_limits = None
    import oracle
    ctx = threadpool_limits(limits=1) if threadpool_limits else None
    try:
        act = int(sum(1 for t in rows if wl.ids[t] >= 0))
        t0 = time.perf_counter()
        n = 0
        while True:
            oracle.lora_forward_rows(wl, rows)
            n += 1
            if time.perf_counter() - t0 >= seconds:
                break
        el = time.perf_counter() - t0
    finally:
        if ctx is not None:
            ctx.__exit__(None, None, None)
    return n * act, el


def _oracle_worker(job):
    """One process of the all-core oracle run: the workload is drawn again from
    its seed (the same values), then the oracle runs on this process's rows."""
    name, seed, lo, hi, seconds = job
    wl = make_workloads(name, seed)[0]
    return _oracle_rate(wl, list(range(lo, hi)), seconds)


def cpu_baseline(wl, seconds, name, seed):
    """The fp64 oracle as it stands, timed on this host for about `seconds`:
    once in one process per visible core (at most 16), each on a contiguous
    share of the batch's rows (rows are independent), which is the baseline
    reported; and once in this process on one thread."""
    import multiprocessing as mp
    ncores = min(16, len(os.sched_getaffinity(0)))
    cpu = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    nproc = max(1, min(ncores, wl.T))
    bounds = [(wl.T * k // nproc, wl.T * (k + 1) // nproc) for k in range(nproc)]
    # spawn: the workers start fresh interpreters and never touch the GPU
    try:
        with mp.get_context("spawn").Pool(nproc) as pool:
            res = pool.map_async(_oracle_worker,
                                 [(name, seed, lo, hi, seconds) for lo, hi in bounds]).get(
                                     timeout=3 * seconds + 120)
    except Exception as e:  # the workers did not finish: report the one-thread run only
        res = None
        log(f"[bench] all-core oracle run failed ({e!r}); reporting one thread")
    n_one, el_one = _oracle_rate(wl, list(range(wl.T)), seconds)
    one = {"value": n_one / el_one, "unit": "LoRA-delta tokens/s", "cores": 1,
           "sample": f"{n_one} active rows (whole batches) in {el_one:.1f} s in one process on "
                     f"one BLAS thread"}
    if res is None:
        return dict(one, kind="oracle", sample=one["sample"] + f"; host CPU: {cpu}")
    v_all = sum(n / el for n, el in res)
    done = sum(n for n, _ in res)
    return {"value": v_all, "unit": "LoRA-delta tokens/s", "cores": nproc, "kind": "oracle",
            "sample": f"the per-token fp64 oracle in {nproc} processes (one per visible core, "
                      f"one BLAS thread each), each repeating its share of the rows of the same "
                      f"workload for {seconds:.0f} s: {done} active rows in all; host CPU: {cpu}",
            "single_thread": one}


def bgmv_sweep(seed, stream_ptr):
    """BGMV decode at in = out = 4096 over batch size T, adapters in the batch
    and rank: per launch group, average time and algorithmic GB/s, to show
    where the decode kernels leave the launch-latency regime."""
    import torch
    import workloads as W
    rows = []
    for rank, n_adapters in ((16, 8), (16, 64), (64, 8)):
        for T in (64, 256, 1024, 4096):
            wl = W.config_bgmv_decode(seed=seed, T=T, K=4096, O=4096, n_adapters=n_adapters,
                                      rank=rank, alpha=2.0 * rank, p_none=0.0)
            s = Setup(wl, 1024 * 2 ** 20)
            el = measure([s], 50, 5, stream_ptr)
            dom, res = kernel_roofline([s], stream_ptr, 50)
            a = algorithmic(wl)
            row = {"T": T, "adapters": n_adapters, "rank": rank, "step_us": el / 50 * 1e6,
                   "bytes_per_step": a["bytes"],
                   "stages": {k: {"us": round(r["us"], 2), "GBs": round(r["GBs"], 1),
                                  "frac": round(r["GBs"] / HBM_PEAK_GBS, 3), "kernels": r["kernels"]}
                              for k, r in res.items()}}
            rows.append(row)
            log(f"[bench] sweep T={T} adapters={n_adapters} R={rank}: step {row['step_us']:.1f} us, "
                + ", ".join(f"{k} {v['us']:.1f} us {v['GBs']:.0f} GB/s" for k, v in row["stages"].items()))
            del s
            torch.cuda.empty_cache()
    return rows


def main():
    args = parse()
    if args.record_traffic:
        record_traffic(args.record_traffic, args.workload, args.seed)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1 "
                                   "(token rows are independent, so data parallelism needs no "
                                   "exchange; see the sharding notes in the design document)"}))
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    stream_ptr = torch.cuda.current_stream().cuda_stream
    t_start = time.perf_counter()

    wls = make_workloads(args.workload, args.seed)
    log(f"[bench] workload {args.workload}: T={wls[0].T} dtype={wls[0].dtype}")
    rep_bytes = args.replica_mib * 2 ** 20 / len(wls)
    setups = [Setup(wl, rep_bytes) for wl in wls]
    log(f"[bench] replicas {[s.nrep for s in setups]} ({sum(s.nrep * s.bytes_per_rep for s in setups) / 2**20:.0f} MiB)")

    el = measure(setups, args.steps, args.warmup, stream_ptr)
    algs = [algorithmic(s.wl) for s in setups]
    Ta = sum(a["Ta"] for a in algs)
    step_s = el / args.steps
    value = Ta / step_s
    log(f"[bench] {args.steps} steps in {el:.3f} s: {step_s * 1e6:.1f} us/step")

    launches = max(50, min(400, args.steps))
    dom, per_kernel = kernel_roofline(setups, stream_ptr, launches)
    for k, r in per_kernel.items():
        log(f"[bench] {k}: {r['us']:.2f} us/launch, {r['GBs']:.0f} GB/s algorithmic, "
            f"{r['TFLOPs']:.1f} TFLOP/s")
    d = per_kernel[dom]
    traffic = load_traffic(dom, args.workload)
    copy_gbs, _ = copy_bandwidth()
    log(f"[bench] device copy bandwidth {copy_gbs:.0f} GB/s")
    kernel_us_step = sum(r["step_us"] for r in per_kernel.values())
    total_bytes = sum(a["bytes"] for a in algs)

    out = {
        "metric": "LoRA-delta tokens/s + achieved HBM GB/s (% peak), BGMV decode and SGMV prefill",
        "value": value,
        "unit": "LoRA-delta tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_s * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wls[0].dtype,
        "data": "synthetic",
        "config": {
            "workload": WORKLOAD_DESC[args.workload],
            "tokens": wls[0].T, "active_tokens": Ta, "adapters_active": algs[0]["n_act"],
            "replicas": setups[0].nrep, "seed": args.seed,
        },
        "achieved_GBs_step": total_bytes / step_s / 1e9,
        "frac_hbm_peak_step": total_bytes / step_s / 1e9 / HBM_PEAK_GBS,
        "kernel_us_per_step": kernel_us_step,
        "achieved_GBs_kernels": total_bytes / (kernel_us_step * 1e-6) / 1e9,
        "copy_GBs_measured": copy_gbs,
        "per_kernel": {k: {"us": round(r["us"], 3), "GBs": round(r["GBs"], 1),
                           "TFLOPs": round(r["TFLOPs"], 2), "kernels": r["kernels"]}
                       for k, r in per_kernel.items()},
        "roofline": {"bound": "hbm", "kernel": " + ".join(d["kernels"]), "stage": dom,
                     "achieved": d["GBs"], "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": d["GBs"] / HBM_PEAK_GBS,
                     "traffic": traffic, "algorithmic_bytes_per_launch": d["bytes"],
                     "avg_launch_us": d["us"]},
    }
    out["slot_load"] = slot_load_leg(args.seed)
    log(f"[bench] slot loads: {out['slot_load']}")
    dm = device_meta_leg(setups[0], max(20, args.steps // 4), stream_ptr)
    out["device_meta"] = dict(dm, workload=setups[0].wl.name)
    log(f"[bench] device metadata: builder {dm['builder_us']:.2f} us, step {dm['step_us']:.2f} us "
        f"(5 launches); device plan (lora_apply_device) {dm['device_plan_step_us']:.2f} us, "
        f"replayed in a graph {dm['device_plan_graph_step_us']:.2f} us")
    del setups
    torch.cuda.empty_cache()
    if not args.no_secondary:
        out["ragged_decode"] = ragged_decode_leg(args.seed, max(50, args.steps // 4), stream_ptr,
                                                 args.replica_mib * 2 ** 20)
        log(f"[bench] ragged decode: {out['ragged_decode']}")
        out["merge"] = merge_leg(args.seed, stream_ptr, cpu=not args.no_cpu_baseline)
        log(f"[bench] merged weights: {out['merge']}")
        torch.cuda.empty_cache()

    if not args.no_secondary and args.workload != "sgmv_prefill":
        wl2 = make_workloads("sgmv_prefill", args.seed)
        out["secondary"], s2 = workload_leg("sgmv_prefill", args.seed, max(20, args.steps // 10),
                                            stream_ptr, args.replica_mib * 2 ** 20)
        st2 = out["secondary"]["ms_per_step"] * 1e-3
        a2 = algorithmic(wl2[0])
        dp, db = device_plan_leg(s2[0], max(20, args.steps // 10), stream_ptr)
        out["secondary"]["device_plan_step_us"] = round(dp, 2)
        out["secondary"]["device_builder_us"] = round(db, 2)
        log(f"[bench] prefill from device ids (lora_apply_device): {dp:.1f} us/step, "
            f"builder alone {db:.1f} us")
        del s2
        torch.cuda.empty_cache()
        # the same batch with each slot's true rank (lora_apply_ranked): the
        # padded ranks' weights are neither read nor multiplied
        s3 = [Setup(w, args.replica_mib * 2 ** 20, ragged=True) for w in wl2]
        el3 = measure(s3, max(20, args.steps // 10), 5, stream_ptr)
        st3 = el3 / max(20, args.steps // 10)
        _, pk3 = kernel_roofline(s3, stream_ptr, 50)
        out["secondary"]["ragged"] = {
            "slot_ranks": s3[0].slot_ranks.tolist(),
            "tokens_per_s": a2["Ta"] / st3, "ms_per_step": st3 * 1e3,
            "speedup_vs_padded": st2 / st3,
            "per_kernel": {k: {"us": round(r["us"], 2)} for k, r in pk3.items()},
        }
        log(f"[bench] prefill ragged ranks: {st3 * 1e6:.1f} us/step vs padded {st2 * 1e6:.1f} "
            + ", ".join(f"{k} {r['us']:.2f} us" for k, r in pk3.items()))
        del s3
        torch.cuda.empty_cache()

    if not args.no_secondary:
        # the other two named workloads, each measured the same way
        for name in ("qkv_decode", "mlp_mixed"):
            if name == args.workload:
                continue
            steps_w = max(20, args.steps // (10 if name == "qkv_decode" else 40))
            out[name], sw = workload_leg(name, args.seed, steps_w, stream_ptr,
                                         args.replica_mib * 2 ** 20)
            del sw
            torch.cuda.empty_cache()

    if args.sweep:
        out["bgmv_sweep"] = bgmv_sweep(args.seed, stream_ptr)

    if not args.no_cpu_baseline:
        log(f"[bench] timing the oracle on the host for ~{args.cpu_seconds:.0f} s")
        out["cpu_baseline"] = cpu_baseline(wls[0], args.cpu_seconds, args.workload, args.seed)
    else:
        out["cpu_baseline"] = None
    out["wall_s"] = time.perf_counter() - t_start
    out["host"] = platform.node()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
