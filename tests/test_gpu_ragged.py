"""Ragged ranks (lora_apply_ranked): pools whose slots hold adapters of lower
rank than the slot rank.  The kernels skip the padded ranks, whose weights are
zero, so the result must equal the padded path's bit for bit and the oracle's
within tolerance, on plans that reach every kernel that reads the record rank:
wavefront tiles from the device plan (more than 48 of them), 64-row MFMA tiles
for prefill segments and for long decode runs, and ranks above 64."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_helpers import check_rows, make_pool, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    say(f"[gpu] {request.node.name}")
    yield


def _bits(t):
    import torch
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _ranked_vs_padded(wl, R=None, label=""):
    import torch
    pool = make_pool(wl, R=R)
    x = to_dev(wl.x, wl.dtype)
    ys = []
    for ragged in (False, True):
        y = to_dev(wl.y_in, wl.dtype)
        pool.apply(x, y, wl.ids, wl.prefill, ragged=ragged)
        torch.cuda.synchronize()
        ys.append(y)
    diff = int((_bits(ys[0]) != _bits(ys[1])).sum().item())
    say(f"  {label}: slot ranks {pool.slot_ranks().tolist()[:12]} pool rank {pool.R}, "
        f"elements differing from the padded path: {diff}")
    assert diff == 0
    check_rows(wl, ys[1], label=f"{label} ragged")


def test_ragged_mixed_wave_tiles():
    # ~650 decode rows over 8 adapters plus short prefill segments: more than 48
    # wavefront tiles, so they run from the device plan and read the record rank
    gu, dn = W.config_mlp_mixed(seed=5, n_prefill=4, len_lo=5, len_hi=90, n_decode=650,
                                hidden=264, inter=520, n_adapters=8, rank_choices=(8, 16, 40, 64),
                                max_lora_rank=64)
    for wl in (gu, dn):
        _ranked_vs_padded(wl, label=wl.name)


@pytest.mark.parametrize("rank,R", [(16, 64), (8, 32), (24, 64)])
def test_ragged_decode_mfma_runs(rank, R):
    # a large decode batch over few adapters: long runs take 64-row MFMA tiles
    wl = W.config_bgmv_decode(seed=6, T=2304, K=1032, O=776, n_adapters=6, rank=rank)
    _ranked_vs_padded(wl, R=R, label=f"decode rank {rank} in pool rank {R}")


def test_ragged_prefill_segments():
    wl = W.config_sgmv_prefill(seed=7, n_seqs=10, len_lo=1, len_hi=150, K=1032, O=520,
                               n_adapters=10, rank_choices=(8, 16, 32, 48), max_lora_rank=64)
    _ranked_vs_padded(wl, label="prefill")


def test_ragged_large_pool_rank():
    # pool rank 128 (> 64): the shrink skips padded ranks, the expand reads all
    wl = W.config_sgmv_prefill(seed=8, n_seqs=6, len_lo=20, len_hi=130, K=520, O=264,
                               n_adapters=6, rank_choices=(8, 16, 72), max_lora_rank=128)
    _ranked_vs_padded(wl, label="prefill, pool rank 128")


def test_ragged_fp32_pool():
    gu, _ = W.config_mlp_mixed(seed=9, n_prefill=2, len_lo=5, len_hi=40, n_decode=420,
                               hidden=136, inter=264, n_adapters=6, rank_choices=(8, 16),
                               max_lora_rank=32, dtype="f32")
    _ranked_vs_padded(gu, label="fp32 pool")


def test_ragged_integer_exact():
    # exact arithmetic: the ragged path equals the oracle's result exactly
    import torch
    wl = W.config_integer(seed=3, T=700, max_loras=6)
    pool = make_pool(wl)
    y = to_dev(wl.y_in, wl.dtype)
    pool.apply(to_dev(wl.x, wl.dtype), y, wl.ids, wl.prefill, ragged=True)
    torch.cuda.synchronize()
    exp = oracle.round_exact_to_dtype(oracle.lora_forward_rows(wl), wl.dtype)
    bad = np.argwhere(y.float().cpu().numpy() != exp)
    assert bad.size == 0, f"{len(bad)} mismatches, first {bad[:3]}"


@pytest.mark.parametrize("T,n", [(64, 8), (200, 6)])
def test_ragged_small_plans_by_value(T, n):
    # plans of at most 48 wavefront tiles travel in the kernel arguments (the
    # one-launch decode kernel for at most 12): the rank field is not carried
    # and the result is the padded path's
    wl = W.config_bgmv_decode(seed=T, T=T, K=1032, O=776, n_adapters=n, rank=8)
    import lora_adapter_pool_amd as L
    d = L.make_desc(wl.dtype, wl.max_loras, 32, wl.in_features, wl.out_features)
    p, _, _ = L.lora_apply_plan(d, wl.ids, wl.prefill)
    assert p["mfma_tiles"] == 0 and p["wave_tiles"] <= 48
    _ranked_vs_padded(wl, R=32, label=f"by-value plan T={T}")
