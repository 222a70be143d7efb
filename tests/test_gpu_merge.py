"""Merged-weight mode (lora_merge_weights) against the fp64 oracle: every
element of W + s B A, the bf16 result within one bf16 step of the oracle's
single rounding plus the error of the kernel's fp32 sum (more than one step
only where W and the delta cancel), and exact on integer inputs; shapes with ragged tails in both dimensions, pool ranks that
are not multiples of 32, in-place merges, fp32 pools, and the full-size
projection; and the merged weight used in a base product against the runtime
delta."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_helpers import make_pool, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    say(f"[gpu] {request.node.name}")
    yield


def _ulps_bf16(got, want):
    """Distance in bfloat16 steps between two arrays of bfloat16 values."""
    def key(a):
        b = (np.asarray(a, np.float32).view(np.uint32) >> 16).astype(np.int64)
        return np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)
    return np.abs(key(got) - key(want))


def _merge_and_check(wl, seeds=(0,), integer=False, in_place=False, label=""):
    import torch
    pool = make_pool(wl)
    ref_pool = oracle.expected_pool(wl)
    worst = 0
    for a in sorted(wl.slots):
        for sl, width in enumerate(wl.out_features):
            Wb = W.draw_base_weight(100 * a + sl + seeds[0], width, wl.in_features, wl.dtype,
                                    integer_values=integer)
            Wd = to_dev(Wb, wl.dtype)
            out = pool.merge(a, sl, Wd, Wd if in_place else None)
            torch.cuda.synchronize()
            got = out.float().cpu().numpy()
            want = oracle.merged_weight(Wb, ref_pool[a], sl, wl.dtype)
            if integer:
                bad = np.argwhere(got != want)
                assert bad.size == 0, f"{label} slot {a} slice {sl}: {len(bad)} mismatches"
            elif wl.dtype == "bf16":
                # the kernel sums R exact products and W in fp32, then rounds
                # once: within one bf16 step of the oracle's single rounding
                # plus the fp32 sum's error, (R + 2) 2^-24 (|W| + |B| |A|);
                # more than one step only where W and the delta cancel
                u = _ulps_bf16(got, want.astype(np.float32))
                worst = max(worst, int(u.max()))
                terms = np.abs(Wb) + (np.abs(ref_pool[a]["B"][sl]).astype(np.float64)
                                      @ np.abs(ref_pool[a]["A"][sl]).astype(np.float64))
                step = np.spacing(np.abs(want).astype(np.float32)).astype(np.float64) * 65536
                bound = step + (wl.max_lora_rank + 2) * 2.0 ** -24 * terms
                over = np.abs(got - want) > bound
                assert not over.any(), f"{label} slot {a} slice {sl}: {int(over.sum())} outside"
                assert (u > 1).mean() <= 1e-4, f"{label}: {(u > 1).mean()} beyond one step"
            else:
                scale = np.abs(Wb) + np.abs(ref_pool[a]["B"][sl]) @ np.abs(ref_pool[a]["A"][sl])
                err = np.max(np.abs(got - want) / (scale + 1e-30))
                assert err <= 2e-6, f"{label} slot {a} slice {sl}: rel err {err}"
    say(f"  {label}: slots {sorted(wl.slots)} slices {wl.out_features} K {wl.in_features} "
        f"R {wl.max_lora_rank}: worst {worst} ulp")


@pytest.mark.parametrize("R", [16, 24, 64, 96, 128, 256])
def test_merge_bf16_ragged_tiles(R):
    # 520 x 1032 and 1032 x 520 weights: partial 128-row and 64-column tiles;
    # adapters of mixed ranks in a pool of rank R
    gu, dn = W.config_mlp_mixed(seed=R, n_prefill=1, len_lo=1, len_hi=2, n_decode=2,
                                hidden=1032, inter=520, n_adapters=3,
                                rank_choices=(8, min(R, 16), R), max_lora_rank=R)
    for wl in (gu, dn):
        _merge_and_check(wl, label=f"{wl.name} bf16 R={R}")


@pytest.mark.parametrize("nblk", ["1", "3", "8"])
def test_merge_row_blocks_exact(nblk, monkeypatch):
    # ranks <= 128: a workgroup walks several 64-row blocks of W over its 256
    # columns; 1032 rows (17 blocks) and 2056 x 1032 leave the last workgroup a
    # partial block and blocks past the end; exact on integer inputs
    monkeypatch.setenv("LORA_MERGE_NBLK", nblk)
    for K, out, R in ((520, 1032, 64), (1032, 2056, 128), (264, 520, 32)):
        wl = W.config_integer(seed=K + out + R, T=4, K=K, outs=(out,), max_loras=2,
                              max_lora_rank=R, ranks=(R, 8))
        _merge_and_check(wl, integer=True, label=f"row blocks {nblk}: K={K} out={out} R={R}")


def test_merge_exact_integer():
    wl = W.config_integer(seed=11, T=8, K=520, outs=(264, 136), max_loras=6, max_lora_rank=64)
    _merge_and_check(wl, integer=True, label="integer")


def test_merge_in_place():
    wl = W.config_integer(seed=12, T=8, K=264, outs=(136,), max_loras=2, max_lora_rank=32,
                          ranks=(8, 32))
    _merge_and_check(wl, integer=True, in_place=True, label="integer in place")


def test_merge_fp32_pool():
    wl = W.config_qkv_decode(seed=13, T=8, K=264, outs=(136, 72), n_adapters=3, rank=16,
                             dtype="f32")
    _merge_and_check(wl, label="fp32")


def test_merge_full_projection():
    # in = out = 4096, rank 64, as one prefill projection's weight
    wl = W.config_sgmv_prefill(seed=14, n_seqs=2, len_lo=1, len_hi=2, K=4096, O=4096,
                               n_adapters=2, rank_choices=(16, 64), max_lora_rank=64)
    _merge_and_check(wl, label="4096 x 4096")


def test_merged_base_product_matches_runtime_delta():
    """One adapter for the whole batch: x W'^T equals x W^T followed by the
    runtime delta, within bf16 rounding of the two routes."""
    import torch
    wl = W.config_sgmv_prefill(seed=15, n_seqs=1, len_lo=200, len_hi=200, K=1032, O=520,
                               n_adapters=1, rank_choices=(16,), max_lora_rank=32)
    pool = make_pool(wl)
    Wb = W.draw_base_weight(3, 520, 1032, "bf16")
    Wd = to_dev(Wb, "bf16")
    Wm = pool.merge(0, 0, Wd)
    x = to_dev(wl.x, "bf16")
    y_base = (x.float() @ Wd.float().t()).to(torch.bfloat16)
    pool.apply(x, y_base, wl.ids, wl.prefill)
    y_merged = (x.float() @ Wm.float().t()).to(torch.bfloat16)
    torch.cuda.synchronize()
    a, b = y_base.float().cpu().numpy(), y_merged.float().cpu().numpy()
    err = float(np.max(np.abs(a - b) / (np.max(np.abs(b), axis=1, keepdims=True) + 1e-30)))
    say(f"  merged vs runtime: max row-relative difference {err:.2e}")
    assert err < 2e-2


@pytest.mark.parametrize("K,out,R", [(8, 8, 8), (24, 16, 16)])
def test_merge_smallest_shapes(K, out, R):
    # one partial tile in both dimensions; exact on integer inputs
    wl = W.config_integer(seed=K + out, T=4, K=K, outs=(out,), max_loras=2, max_lora_rank=R,
                          ranks=(R, 8))
    _merge_and_check(wl, integer=True, label=f"smallest K={K} out={out} R={R}")
