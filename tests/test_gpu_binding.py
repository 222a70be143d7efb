"""The CPython binding (_lora_call) against ctypes on the GPU: LoraPool.apply
through each route gives bit-identical y (one-launch decode, 8-row MFMA tiles
over three slices, 64-row MFMA prefill tiles, ragged ranks, an fp32 pool), and
the result is within tolerance of the fp64 oracle."""
import ctypes

import numpy as np
import pytest

import lora_adapter_pool_amd as L
from lora_adapter_pool_amd import _lib
import workloads as W
from gpu_helpers import check_rows, make_pool, say, to_dev

pytestmark = pytest.mark.gpu


class _CtypesRoute:
    """Stands in for the binding module: the same calls through ctypes."""

    def __init__(self):
        self.lib = _lib.lib()
        self.dp = ctypes.POINTER(_lib.lora_pool_desc)

    def apply(self, fn, desc, *a):
        assert fn == _lib.entry_address("lora_apply")
        return self.lib.lora_apply(ctypes.cast(desc, self.dp), *a)

    def apply_ranked(self, fn, desc, *a):
        assert fn == _lib.entry_address("lora_apply_ranked")
        return self.lib.lora_apply_ranked(ctypes.cast(desc, self.dp), *a)


CASES = {
    "decode_onepass": lambda: W.config_bgmv_decode(seed=0),
    "qkv_tiles": lambda: W.config_qkv_decode(seed=3, T=300, K=520, outs=(264, 72, 72),
                                             n_adapters=24, rank=16),
    "prefill_mfma": lambda: W.config_sgmv_prefill(seed=5, n_seqs=6, len_lo=40, len_hi=300,
                                                  K=1024, O=520, n_adapters=6,
                                                  rank_choices=(8, 16, 32, 64),
                                                  max_lora_rank=64),
    "fp32": lambda: W.config_qkv_decode(seed=7, T=90, K=264, outs=(136, 72), n_adapters=5,
                                        rank=16, dtype="f32"),
}


def _bits(t):
    import torch
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("ragged", [False, True])
@pytest.mark.parametrize("case", sorted(CASES))
def test_binding_equals_ctypes(case, ragged, monkeypatch):
    import torch
    if ragged and case == "fp32":
        pytest.skip("ragged ranks change nothing for fp32 pools")
    say(f"[gpu] binding vs ctypes: {case}, ragged={ragged}")
    wl = CASES[case]()
    pool = make_pool(wl)
    xd = to_dev(wl.x, wl.dtype)
    y_bind = to_dev(wl.y_in, wl.dtype)
    pool.apply(xd, y_bind, wl.ids, wl.prefill, ragged=ragged)
    torch.cuda.synchronize()
    y_ct = to_dev(wl.y_in, wl.dtype)
    monkeypatch.setattr(_lib, "_pycall", _CtypesRoute())
    pool.apply(xd, y_ct, wl.ids, wl.prefill, ragged=ragged)
    torch.cuda.synchronize()
    monkeypatch.undo()
    assert torch.equal(_bits(y_bind.cpu()), _bits(y_ct.cpu())), f"{case}: routes differ"
    check_rows(wl, y_bind, label=f"{case} (binding) vs oracle")
