"""Device-side metadata builder (lora_build_meta_device) against the host
builder and the oracle's builder, and the whole delta path driven from device
metadata with upper-bound sizes, eagerly and captured in a graph."""
import dataclasses

import numpy as np
import pytest

import lora_adapter_pool_amd as L
import oracle
import workloads as W
from gpu_helpers import check_rows, make_pool, say, to_dev

pytestmark = pytest.mark.gpu
KEYS = ("sgmv_perm", "seg_starts", "seg_lens", "seg_ids", "bgmv_tok", "bgmv_ids")


def _device_meta(ids, prefill, max_loras, R, bgmv_max_rank=0):
    import torch
    T = int(ids.size)
    cap = {"sgmv_perm": T, "bgmv_tok": T, "bgmv_ids": T, "seg_starts": max_loras,
           "seg_lens": max_loras, "seg_ids": max_loras}
    arrays = {k: torch.full((max(n, 1),), 12345, dtype=torch.int32, device="cuda")
              for k, n in cap.items()}
    counts = torch.full((4,), -7, dtype=torch.int32, device="cuda")
    ids_d = torch.from_numpy(np.ascontiguousarray(ids, np.int32)).cuda() if T else \
        torch.zeros(1, dtype=torch.int32, device="cuda")
    pre_d = None if prefill is None else torch.from_numpy(
        np.ascontiguousarray(prefill, np.uint8)).cuda()
    L.lora_build_meta_device(ids_d, pre_d, T, max_loras, R, bgmv_max_rank, arrays, counts)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy()[:cap[k]] for k, v in arrays.items()}, counts.cpu().numpy()


def _check_against_host(ids, prefill, max_loras, R, bgmv_max_rank=0):
    got, counts = _device_meta(ids, prefill, max_loras, R, bgmv_max_rank)
    valid = np.where((ids >= -1) & (ids < max_loras), ids, -1).astype(np.int32)
    ref = L.lora_build_meta(valid, prefill, max_loras, R, bgmv_max_rank)
    lim = bgmv_max_rank if bgmv_max_rank > 0 else 64
    pre_list = [0] * ids.size if prefill is None else prefill.tolist()
    orc = oracle.build_meta(valid.tolist(), pre_list, R, lim)
    ns, nseg, nb = ref["sgmv_perm"].size, ref["seg_ids"].size, ref["bgmv_tok"].size
    assert counts.tolist() == [ns, nseg, nb, int(np.sum(ids != valid))]
    for k in KEYS:
        n = ref[k].size
        assert got[k][:n].tolist() == ref[k].tolist() == list(orc[k]), k
    # padding behind the counts
    T = ids.size
    assert np.all(got["seg_lens"][nseg:] == 0) and np.all(got["seg_starts"][nseg:] == ns)
    assert np.all(got["bgmv_ids"][nb:T] == -1) and np.all(got["bgmv_tok"][nb:T] == 0)
    assert np.all(got["sgmv_perm"][ns:T] == 0)
    return counts


@pytest.mark.parametrize("T,max_loras,sorted_ids,pre_kind,R", [
    (0, 4, False, "none", 16), (1, 1, False, "rand", 16), (63, 7, False, "rand", 16),
    (64, 8, False, "zero", 16), (65, 8, True, "rand", 16), (300, 64, False, "rand", 128),
    (1000, 1000, False, "rand", 16), (8772, 16, True, "one", 64), (4096, 8192, False, "rand", 16),
    (3000, 33, True, "runs", 32), (5000, 200, False, "rand", 16), (2049, 256, False, "rand", 64),
    (70000, 100, False, "rand", 16)])
def test_device_builder_matches_host(T, max_loras, sorted_ids, pre_kind, R):
    rng = np.random.default_rng(T + max_loras)
    ids = rng.integers(-1, max_loras, size=T).astype(np.int32)
    if sorted_ids:
        ids = np.sort(ids)
    pre = {"none": None, "zero": np.zeros(T, np.uint8), "one": np.ones(T, np.uint8),
           "rand": rng.integers(0, 2, size=T).astype(np.uint8),
           "runs": np.repeat(rng.integers(0, 2, size=T // 50 + 1), 50)[:T].astype(np.uint8)}[pre_kind]
    counts = _check_against_host(ids, pre, max_loras, R)
    say(f"  T={T} max_loras={max_loras}: rows {counts[0]} segs {counts[1]} bgmv {counts[2]}")


def test_device_builder_rank_limit_and_bad_ids():
    """bgmv_max_rank sends every row to SGMV when the pool rank exceeds it; ids
    outside [-1, max_loras) are counted and left out."""
    rng = np.random.default_rng(3)
    ids = rng.integers(-1, 12, size=500).astype(np.int32)
    pre = rng.integers(0, 2, size=500).astype(np.uint8)
    _check_against_host(ids, pre, 12, 64, bgmv_max_rank=32)
    bad = ids.copy()
    bad[[5, 77, 400]] = [-2, 12, 1 << 30]
    counts = _check_against_host(bad, pre, 12, 16)
    assert counts[3] == 3


def _pipeline(pool, wl, xd, yd, ids_d, pre_d, meta, counts, v_s, v_b):
    """Device builder then the four grouped entry points with upper-bound sizes."""
    T = wl.T
    L.lora_build_meta_device(ids_d, pre_d, T, wl.max_loras, pool.R, 0, meta, counts)
    L.lora_sgmv_shrink(pool.desc, xd, pool.A, v_s, meta["sgmv_perm"], meta["seg_starts"],
                       meta["seg_lens"], meta["seg_ids"], wl.max_loras, T, T)
    L.lora_bgmv_shrink(pool.desc, xd, pool.A, v_b, meta["bgmv_tok"], meta["bgmv_ids"], T, T)
    L.lora_sgmv_expand(pool.desc, v_s, pool.B, yd, meta["sgmv_perm"], meta["seg_starts"],
                       meta["seg_lens"], meta["seg_ids"], wl.max_loras, T, T)
    L.lora_bgmv_expand(pool.desc, v_b, pool.B, yd, meta["bgmv_tok"], meta["bgmv_ids"], T, T)


def _buffers(wl, pool):
    import torch
    T = wl.T
    meta = {k: torch.zeros(max(T if k in ("sgmv_perm", "bgmv_tok", "bgmv_ids") else wl.max_loras,
                               1), dtype=torch.int32, device="cuda") for k in KEYS}
    counts = torch.zeros(4, dtype=torch.int32, device="cuda")
    SR = wl.num_slices * pool.R
    v_s = torch.zeros((T, SR), dtype=torch.float32, device="cuda")
    v_b = torch.zeros((T, SR), dtype=torch.float32, device="cuda")
    return meta, counts, v_s, v_b


def test_device_metadata_pipeline_matches_oracle():
    """Mixed prefill + decode batch (short and long segments, BGMV rows) driven
    entirely from device metadata: within tolerance of the oracle, rows without
    adapter untouched."""
    import torch
    wl, _ = W.config_mlp_mixed(seed=6, n_prefill=3, len_lo=5, len_hi=90, n_decode=40,
                               hidden=520, inter=264, n_adapters=5)
    pool = make_pool(wl)
    meta, counts, v_s, v_b = _buffers(wl, pool)
    xd, yd = to_dev(wl.x, wl.dtype), to_dev(wl.y_in, wl.dtype)
    ids_d = torch.from_numpy(wl.ids.astype(np.int32)).cuda()
    pre_d = torch.from_numpy(wl.prefill.astype(np.uint8)).cuda()
    _pipeline(pool, wl, xd, yd, ids_d, pre_d, meta, counts, v_s, v_b)
    torch.cuda.synchronize()
    check_rows(wl, yd, label="device metadata pipeline")


def test_device_metadata_pipeline_graph_replays():
    """The same path captured in one graph; between replays new ids (and
    prefill flags) are written into the device buffers the graph reads, and
    every replay matches the exact result for the ids it saw."""
    import torch
    wl = W.config_integer(seed=31, T=160, K=520, outs=(264, 136), max_loras=6, max_lora_rank=16,
                          ranks=(16, 8), dtype="bf16")
    pool = make_pool(wl)
    meta, counts, v_s, v_b = _buffers(wl, pool)
    xd = to_dev(wl.x, wl.dtype)
    y0 = to_dev(wl.y_in, wl.dtype)
    yd = y0.clone()
    ids_d = torch.zeros(wl.T, dtype=torch.int32, device="cuda")
    pre_d = torch.zeros(wl.T, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _pipeline(pool, wl, xd, yd, ids_d, pre_d, meta, counts, v_s, v_b)
    rng = np.random.default_rng(5)
    for rep in range(4):
        ids = rng.integers(-1, 6, size=wl.T).astype(np.int32)
        pre = (rng.random(wl.T) < [0.0, 0.5, 1.0, 0.3][rep]).astype(np.uint8)
        if rep == 3:
            order = np.argsort(ids, kind="stable")
            ids, pre = ids[order], np.ones(wl.T, np.uint8)  # long sorted prefill segments
        ids_d.copy_(torch.from_numpy(ids))
        pre_d.copy_(torch.from_numpy(pre))
        yd.copy_(y0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        case = dataclasses.replace(wl, ids=ids, prefill=pre)
        exp = oracle.round_exact_to_dtype(oracle.lora_forward_rows(case), wl.dtype)
        bad = np.argwhere(yd.float().cpu().numpy() != exp)
        assert bad.size == 0, f"replay {rep}: {len(bad)} mismatches, first {bad[:3]}"
