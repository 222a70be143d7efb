"""lora_apply_device_noalloc (the entry point for callers that cannot allocate:
its workspace is the library's per-GPU scratch array) against
lora_apply_device with a workspace of the caller's, on two calls in a row, the
second with a smaller batch: equal bit for bit (the same kernels, plan and K
splits), and within tolerance of the fp64 oracle.  The one-launch decode form,
the two-stage 8-row tile form, 64-row MFMA prefill tiles and an fp32 pool are
each covered, and twelve pairs of random shapes and batches; free device
memory does not change across the second call."""
import numpy as np
import pytest

import lora_adapter_pool_amd as L
import workloads as W
from gpu_helpers import check_rows, make_pool, say, to_dev

pytestmark = pytest.mark.gpu


def _dev_ids(wl):
    import torch
    ids = torch.from_numpy(np.ascontiguousarray(wl.ids, dtype=np.int32)).cuda()
    pre = torch.from_numpy(np.ascontiguousarray(wl.prefill, dtype=np.uint8)).cuda()
    return ids, pre


def _both(wl, pool):
    """y from lora_apply_device (caller's workspace) and from the no-alloc form."""
    import torch
    ids, pre = _dev_ids(wl)
    xd = to_dev(wl.x, wl.dtype)
    y_ref = to_dev(wl.y_in, wl.dtype)
    n = L.lora_apply_device_workspace_bytes(pool.desc, wl.T)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    L.lora_apply_device(pool.desc, pool.A, pool.B, xd, y_ref, wl.T, ids, pre, 0, ws, n)
    y_na = to_dev(wl.y_in, wl.dtype)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    L.lora_apply_device_noalloc(pool.desc, pool.A, pool.B, xd, y_na, wl.T, ids, pre, 0)
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    return y_ref, y_na, free0, free1


def _bits(t):
    import torch
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


CASES = {
    # one-launch decode form (small bf16 plan, R <= 32), then a smaller batch
    "decode_onepass": lambda: (W.config_bgmv_decode(seed=0),
                               W.config_bgmv_decode(seed=1, T=23)),
    # two-stage 8-row MFMA tiles (three slices), then a smaller batch
    "qkv_tiles": lambda: (W.config_qkv_decode(seed=3, T=300, K=520, outs=(264, 72, 72),
                                              n_adapters=24, rank=16),
                          W.config_qkv_decode(seed=4, T=61, K=520, outs=(264, 72, 72),
                                              n_adapters=24, rank=16)),
    # long prefill segments on 64-row MFMA tiles, then a smaller batch
    "prefill_mfma": lambda: (W.config_sgmv_prefill(seed=5, n_seqs=6, len_lo=40, len_hi=300,
                                                   K=1032, O=520, n_adapters=6,
                                                   rank_choices=(8, 16, 32, 64),
                                                   max_lora_rank=64),
                             W.config_sgmv_prefill(seed=6, n_seqs=3, len_lo=20, len_hi=90,
                                                   K=1032, O=520, n_adapters=6,
                                                   rank_choices=(8, 16, 32, 64),
                                                   max_lora_rank=64)),
    # fp32 pool (VALU kernels), two slices
    "fp32": lambda: (W.config_qkv_decode(seed=7, T=90, K=264, outs=(136, 72), n_adapters=5,
                                         rank=16, dtype="f32"),
                     W.config_qkv_decode(seed=8, T=33, K=264, outs=(136, 72), n_adapters=5,
                                         rank=16, dtype="f32")),
}


def _check_pair(case, first, second):
    import torch
    assert second.T < first.T
    for k, wl in enumerate((first, second)):
        pool = make_pool(wl)
        y_ref, y_na, free0, free1 = _both(wl, pool)
        same = torch.equal(_bits(y_ref.cpu()), _bits(y_na.cpu()))
        say(f"  call {k + 1}: T={wl.T} bit-identical to lora_apply_device: {same}; "
            f"free device memory {free0} -> {free1}")
        assert same, f"{case} call {k + 1}: differs from lora_apply_device"
        if k == 1:
            # (the first call on a device may make the HIP runtime load the
            # code object that holds the scratch array; later calls must not
            # change device memory at all)
            assert free1 == free0, "the no-alloc entry point changed free device memory"
        check_rows(wl, y_na, label=f"{case} call {k + 1} (no-alloc) vs oracle")
        del pool, y_ref, y_na


@pytest.mark.parametrize("case", sorted(CASES))
def test_noalloc_equals_device_path_twice(case):
    say(f"[gpu] no-alloc entry point: {case}")
    _check_pair(case, *CASES[case]())


def _random_pair(seed):
    """A random shape and batch (workloads.config_random), then a smaller one
    of another random shape."""
    first = W.config_random(seed, 900)
    return first, W.config_random(seed + 500, max(1, first.T - 1))


RANDOM_SEEDS = list(range(12))  # (each first batch has more than one row)


@pytest.mark.parametrize("seed", RANDOM_SEEDS)
def test_noalloc_random_shapes_twice(seed):
    say(f"[gpu] no-alloc entry point: random shapes, seed {seed}")
    _check_pair(f"random {seed}", *_random_pair(seed))
