"""Seeded random shapes and batches through both plans of the delta path:
lora_apply (host-built plan) and lora_apply_device (device-built plan), every
row against the fp64 oracle.  Each case draws its dtype, in_features and one
to three slice widths (multiples of 8, most not of 64), slot count, padded
rank and each slot's own rank, alpha, rsLoRA, the BGMV rank limit, and a
batch of sorted prefill segments and decode rows (uniform or Zipf ids) with
rows without adapter, in a random order (workloads.config_random)."""
import numpy as np
import pytest

import lora_adapter_pool_amd as L
import workloads as W
from gpu_helpers import check_rows, make_pool, run_apply, say, to_dev

pytestmark = pytest.mark.gpu

# 64 batches of up to 900 rows, and 8 of up to 6 000 (decode runs long enough
# for 64-row MFMA tiles, deeper K splits)
CASES = [(seed, 900) for seed in range(64)] + [(seed, 6000) for seed in range(100, 108)]


@pytest.fixture(autouse=True)
def _announce(request):
    say(f"[gpu] {request.node.name}")
    yield


def _run_device(wl, pool, bgmv_max_rank):
    import torch
    xd, yd = to_dev(wl.x, wl.dtype), to_dev(wl.y_in, wl.dtype)
    ids_d = torch.from_numpy(np.ascontiguousarray(wl.ids, dtype=np.int32)).cuda()
    pre_d = torch.from_numpy(np.ascontiguousarray(wl.prefill, dtype=np.uint8)).cuda()
    n = L.lora_apply_device_workspace_bytes(pool.desc, wl.T)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    L.lora_apply_device(pool.desc, pool.A, pool.B, xd, yd, wl.T, ids_d, pre_d, bgmv_max_rank,
                        ws, n)
    torch.cuda.synchronize()
    return yd


@pytest.mark.parametrize("seed,max_T", CASES)
def test_random_shapes_both_plans(seed, max_T):
    wl = W.config_random(seed, max_T)
    lim = wl.info["bgmv_max_rank"]
    say(f"  {wl.name}: {wl.dtype} K={wl.in_features} outs={wl.out_features} "
        f"max_loras={wl.max_loras} R={wl.max_lora_rank} T={wl.T} "
        f"active={wl.active_tokens} prefill={int(wl.prefill.sum())} bgmv_max_rank={lim}")
    pool = make_pool(wl)
    check_rows(wl, run_apply(wl, pool=pool, bgmv_max_rank=lim), label=f"{wl.name} host plan")
    check_rows(wl, _run_device(wl, pool, lim), label=f"{wl.name} device plan")
