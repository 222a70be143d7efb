"""lora_apply_device: the delta path from device ids, through the device
metadata builder, a device-built plan of 8-row tiles and the tile kernels,
against the fp64 oracle (named workloads, exact integer inputs, fp32 pools,
pool ranks above 64 and above the BGMV limit, ids outside the slot range,
a workspace reused by batches of different sizes), and captured in a graph
replayed with new ids."""
import dataclasses

import numpy as np
import pytest

import lora_adapter_pool_amd as L
import oracle
import workloads as W
from gpu_helpers import check_rows, make_pool, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    say(f"[gpu] {request.node.name}")
    yield


def _ws(pool, T):
    import torch
    n = L.lora_apply_device_workspace_bytes(pool.desc, T)
    return torch.empty(n, dtype=torch.uint8, device="cuda"), n


def _run(wl, pool=None, ids=None, prefill=None, ws=None, bgmv_max_rank=0):
    import torch
    pool = pool or make_pool(wl)
    ids = wl.ids if ids is None else ids
    prefill = wl.prefill if prefill is None else prefill
    xd, yd = to_dev(wl.x, wl.dtype), to_dev(wl.y_in, wl.dtype)
    ids_d = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).cuda()
    pre_d = torch.from_numpy(np.ascontiguousarray(prefill, dtype=np.uint8)).cuda()
    buf, n = ws if ws is not None else _ws(pool, wl.T)
    L.lora_apply_device(pool.desc, pool.A, pool.B, xd, yd, wl.T, ids_d, pre_d, bgmv_max_rank,
                        buf, n)
    torch.cuda.synchronize()
    return yd


def test_device_plan_bgmv_decode_full():
    wl = W.config_bgmv_decode(seed=0)
    check_rows(wl, _run(wl), label="bgmv decode, device plan")


def test_device_plan_qkv_decode_full():
    wl = W.config_qkv_decode(seed=0)
    check_rows(wl, _run(wl), label="fused qkv decode, device plan")


def test_device_plan_prefill_full():
    wl = W.config_sgmv_prefill(seed=0)
    check_rows(wl, _run(wl), label="sgmv prefill, device plan (all rows)")


def test_device_plan_mlp_mixed_full():
    gu, dn = W.config_mlp_mixed(seed=0)
    for wl in (gu, dn):
        check_rows(wl, _run(wl), label=f"{wl.name}, device plan (all rows)")


def test_device_plan_mixed_small():
    gu, dn = W.config_mlp_mixed(seed=1, n_prefill=3, len_lo=5, len_hi=70, n_decode=37,
                                hidden=264, inter=520, n_adapters=8)
    for wl in (gu, dn):
        check_rows(wl, _run(wl), label=f"{wl.name}, device plan")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_device_plan_exact_integer(dtype):
    wl = W.config_integer(seed=21, T=300, K=520, outs=(264, 136), max_loras=6,
                          max_lora_rank=64, dtype=dtype)
    exp = oracle.round_exact_to_dtype(oracle.lora_forward_rows(wl), dtype)
    bad = np.argwhere(_run(wl).float().cpu().numpy() != exp)
    assert bad.size == 0, f"{len(bad)} mismatches, first {bad[:3]}"


@pytest.mark.parametrize("R", [80, 128])
def test_device_plan_large_ranks(R):
    # 80: the VALU kernels (R > 64); 128: above the BGMV limit, every row SGMV
    wl = W.config_mlp_mixed(seed=2, n_prefill=2, len_lo=20, len_hi=60, n_decode=11, hidden=136,
                            inter=264, n_adapters=4, rank_choices=(8, 16), max_lora_rank=R)[0]
    check_rows(wl, _run(wl), label=f"device plan R={R}")


def test_device_plan_skips_out_of_range_ids():
    wl = W.config_integer(seed=22, T=120, K=264, outs=(136,), max_loras=4, max_lora_rank=16,
                          ranks=(16, 8, 16, 8), dtype="bf16")
    ids = wl.ids.copy()
    ids[::7] = 9      # outside [-1, max_loras): skipped like -1
    ids[3::11] = -5
    pool = make_pool(wl)
    ws = _ws(pool, wl.T)
    y = _run(wl, pool=pool, ids=ids, ws=ws)
    case = dataclasses.replace(wl, ids=np.where((ids < -1) | (ids >= 4), -1, ids).astype(np.int32))
    exp = oracle.round_exact_to_dtype(oracle.lora_forward_rows(case), "bf16")
    assert np.array_equal(y.float().cpu().numpy(), exp)
    # the workspace's first four words report the batch: SGMV rows, segments,
    # BGMV rows and the rows whose id was out of range (skipped)
    import torch
    counts = ws[0][:16].view(torch.int32).cpu().numpy()
    bad = int(((ids < -1) | (ids >= 4)).sum())
    m = oracle.build_meta(case.ids.tolist(), case.prefill.tolist(), 16)
    assert counts.tolist() == [len(m["sgmv_perm"]), len(m["seg_ids"]), len(m["bgmv_tok"]), bad]


def test_device_plan_workspace_reused_across_batches():
    """A large batch then a small one on the same workspace: the small batch's
    plan must not pick up the large batch's tile records."""
    big = W.config_integer(seed=23, T=400, K=264, outs=(136,), max_loras=6, max_lora_rank=16,
                           ranks=(16, 8, 16, 8, 16, 8), dtype="bf16")
    pool = make_pool(big)
    ws = _ws(pool, big.T)
    for T in (400, 37, 5, 400):
        wl = W.config_integer(seed=23 + T, T=T, K=264, outs=(136,), max_loras=6,
                              max_lora_rank=16, ranks=(16, 8, 16, 8, 16, 8), dtype="bf16")
        wl = dataclasses.replace(wl, slots=big.slots)
        exp = oracle.round_exact_to_dtype(oracle.lora_forward_rows(wl), "bf16")
        y = _run(wl, pool=pool, ws=ws)
        bad = np.argwhere(y.float().cpu().numpy() != exp)
        assert bad.size == 0, f"T={T}: {len(bad)} mismatches"


def test_device_plan_graph_replays():
    """lora_apply_device captured in one graph; new ids and prefill flags are
    written into its input buffers between replays; every replay is exact."""
    import torch
    wl = W.config_integer(seed=24, T=200, K=520, outs=(264, 136), max_loras=6, max_lora_rank=16,
                          ranks=(16, 8), dtype="bf16")
    pool = make_pool(wl)
    buf, n = _ws(pool, wl.T)
    xd = to_dev(wl.x, wl.dtype)
    y0 = to_dev(wl.y_in, wl.dtype)
    yd = y0.clone()
    ids_d = torch.zeros(wl.T, dtype=torch.int32, device="cuda")
    pre_d = torch.zeros(wl.T, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        L.lora_apply_device(pool.desc, pool.A, pool.B, xd, yd, wl.T, ids_d, pre_d, 0, buf, n)
    rng = np.random.default_rng(6)
    for rep in range(4):
        ids = rng.integers(-1, 6, size=wl.T).astype(np.int32)
        pre = (rng.random(wl.T) < [0.0, 0.5, 1.0, 0.2][rep]).astype(np.uint8)
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


@pytest.mark.parametrize("R,T,n", [(16, 40, 4), (32, 64, 4), (16, 9, 8), (32, 1, 3)])
def test_device_plan_one_launch_exact(R, T, n):
    """Small bf16 plans (at most 24 records, R <= 32) run as the one-launch
    decode kernel reading the device-built records: exact on integer inputs."""
    ranks = tuple(8 if a % 2 else R for a in range(n))
    wl = W.config_integer(seed=40 + R + T, T=T, K=1032, outs=(520, 264), max_loras=n,
                          max_lora_rank=R, ranks=ranks, dtype="bf16")
    assert -(-T // 8) + 2 * min(n, T) <= 24
    exp = oracle.round_exact_to_dtype(oracle.lora_forward_rows(wl), "bf16")
    bad = np.argwhere(_run(wl).float().cpu().numpy() != exp)
    assert bad.size == 0, f"{len(bad)} mismatches, first {bad[:3]}"


def test_device_plan_one_launch_graph_replays():
    import torch
    wl = W.config_integer(seed=25, T=48, K=520, outs=(264, 136), max_loras=4, max_lora_rank=16,
                          ranks=(16, 8, 16, 8), dtype="bf16")
    pool = make_pool(wl)
    buf, n = _ws(pool, wl.T)
    xd = to_dev(wl.x, wl.dtype)
    y0 = to_dev(wl.y_in, wl.dtype)
    yd = y0.clone()
    ids_d = torch.zeros(wl.T, dtype=torch.int32, device="cuda")
    pre_d = torch.zeros(wl.T, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        L.lora_apply_device(pool.desc, pool.A, pool.B, xd, yd, wl.T, ids_d, pre_d, 0, buf, n)
    rng = np.random.default_rng(7)
    for rep in range(4):
        ids = rng.integers(-1, 4, size=wl.T).astype(np.int32)
        pre = (rng.random(wl.T) < [0.0, 0.5, 1.0, 0.2][rep]).astype(np.uint8)
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


def test_device_plan_large_decode_mfma_runs():
    """A large decode batch over few adapters: the device plan puts the long
    runs on 64-row MFMA tiles, as the host plan does; exact on integer inputs
    and within tolerance of the oracle on real-valued ones."""
    wl = W.config_integer(seed=26, T=2600, K=520, outs=(264, 136), max_loras=4,
                          max_lora_rank=64, ranks=(64, 16, 32, 8), prefill_frac=0.0,
                          p_none=0.05, dtype="bf16")
    p, _, _ = L.lora_apply_plan(make_pool(wl).desc, wl.ids, wl.prefill)
    assert p["mfma_tiles"] > 0  # the host plan's rule sends these runs to MFMA tiles
    exp = oracle.round_exact_to_dtype(oracle.lora_forward_rows(wl), "bf16")
    bad = np.argwhere(_run(wl).float().cpu().numpy() != exp)
    assert bad.size == 0, f"{len(bad)} mismatches, first {bad[:3]}"
    real = W.config_bgmv_decode(seed=6, T=2304, K=1032, O=776, n_adapters=6, rank=16)
    check_rows(real, _run(real), label="large decode, device plan")


def _device_ranked_vs_plain(wl, ranks, R=None, label=""):
    import torch
    pool = make_pool(wl, R=R)
    buf, n = _ws(pool, wl.T)
    xd = to_dev(wl.x, wl.dtype)
    ids_d = torch.from_numpy(np.ascontiguousarray(wl.ids, dtype=np.int32)).cuda()
    pre_d = torch.from_numpy(np.ascontiguousarray(wl.prefill, dtype=np.uint8)).cuda()
    ranks_d = torch.from_numpy(np.ascontiguousarray(ranks, dtype=np.int32)).cuda()
    ys = []
    for ranked in (False, True):
        y = to_dev(wl.y_in, wl.dtype)
        if ranked:
            L.lora_apply_device_ranked(pool.desc, pool.A, pool.B, xd, y, wl.T, ids_d, pre_d, 0,
                                       ranks_d, buf, n)
        else:
            L.lora_apply_device(pool.desc, pool.A, pool.B, xd, y, wl.T, ids_d, pre_d, 0, buf, n)
        torch.cuda.synchronize()
        ys.append(y)
    diff = int((ys[0].view(torch.int16) != ys[1].view(torch.int16)).sum().item())
    say(f"  {label}: ranks {list(ranks)[:8]}, elements differing: {diff}")
    assert diff == 0
    check_rows(wl, ys[1], label=f"{label} ranked")


def test_device_plan_ranked_equals_plain():
    gu, dn = W.config_mlp_mixed(seed=5, n_prefill=4, len_lo=5, len_hi=90, n_decode=650,
                                hidden=264, inter=520, n_adapters=8, rank_choices=(8, 16, 40, 64),
                                max_lora_rank=64)
    for wl in (gu, dn):
        ranks = [wl.slots[a].rank if a in wl.slots else 0 for a in range(wl.max_loras)]
        _device_ranked_vs_plain(wl, ranks, label=f"{wl.name}, device plan")
    big = W.config_bgmv_decode(seed=6, T=2304, K=1032, O=776, n_adapters=6, rank=16)
    _device_ranked_vs_plain(big, [16] * 6, R=64, label="large decode rank 16 in pool rank 64")
    # values outside [0, max_lora_rank] act as the pool's rank
    _device_ranked_vs_plain(big, [999, -3, 16, 0, 64, 16], R=64, label="out-of-range ranks")


COMBO_CASES = {
    # K not a multiple of 64: the register-staged 64-row shrink; ranks 8 / 16
    "r16_regk": lambda: W.config_mlp_mixed(seed=8, n_prefill=3, len_lo=40, len_hi=200,
                                           n_decode=300, hidden=264, inter=520, n_adapters=8,
                                           rank_choices=(8, 16), max_lora_rank=16),
    # K a multiple of 64: the DMA-staged 64-row shrink; ranks up to 32
    "r32_dma": lambda: W.config_mlp_mixed(seed=9, n_prefill=3, len_lo=40, len_hi=200,
                                          n_decode=300, hidden=512, inter=1024, n_adapters=8,
                                          rank_choices=(16, 32), max_lora_rank=32),
    # ranks up to 64 (two 32-rank chunks in the 8-row expand)
    "r64_dma": lambda: W.config_mlp_mixed(seed=10, n_prefill=3, len_lo=40, len_hi=200,
                                          n_decode=300, hidden=512, inter=1024, n_adapters=8,
                                          rank_choices=(16, 64), max_lora_rank=64),
    # a small batch: the 8-row tiles' shrink splits K (the expand then launches apart)
    "r64_small": lambda: W.config_mlp_mixed(seed=11, n_prefill=1, len_lo=20, len_hi=60,
                                            n_decode=24, hidden=512, inter=1024, n_adapters=4,
                                            rank_choices=(16, 64), max_lora_rank=64),
}


@pytest.mark.parametrize("case", sorted(COMBO_CASES))
def test_device_plan_combined_launch_matches_separate(case, monkeypatch):
    """A device-built plan runs each stage's 64-row and 8-row tiles in one
    launch; with LORA_COMBINED_LAUNCH=0 it launches them apart.  Both forms run
    the same arithmetic on the same records: equal bit for bit, and within
    tolerance of the oracle."""
    import torch
    for wl in COMBO_CASES[case]():
        pool = make_pool(wl)
        ws = _ws(pool, wl.T)
        monkeypatch.delenv("LORA_COMBINED_LAUNCH", raising=False)
        y1 = _run(wl, pool=pool, ws=ws)
        monkeypatch.setenv("LORA_COMBINED_LAUNCH", "0")
        y0 = _run(wl, pool=pool, ws=ws)
        monkeypatch.delenv("LORA_COMBINED_LAUNCH", raising=False)
        diff = int((y1.view(torch.int16) != y0.view(torch.int16)).sum().item())
        say(f"  {case} {wl.name}: T={wl.T} K={wl.in_features} R={wl.max_lora_rank} "
            f"elements differing between one and two launches per stage: {diff}")
        assert diff == 0
        check_rows(wl, y1, label=f"{case} {wl.name}, one launch per stage")
