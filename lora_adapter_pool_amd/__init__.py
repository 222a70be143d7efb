"""MI355X (gfx950) multi-LoRA delta path: SGMV / BGMV shrink and expand behind a
C ABI (include/lora_pool.h), with a thin ctypes binding.

    y[t] += s_a * B_a (A_a x_t)  for each row t with adapter slot a = ids[t] >= 0
"""
from ._lib import (  # noqa: F401
    LORA_BF16, LORA_F32, LoraError, lib, make_desc, lora_apply, lora_apply_host_meta_bytes,
    lora_apply_device, lora_apply_device_noalloc, lora_apply_device_ranked,
    lora_apply_device_workspace_bytes, NOALLOC_SCRATCH_BYTES,
    lora_apply_plan, lora_apply_ranked,
    lora_merge_weights, lora_plan_apply, lora_plan_expand, lora_plan_shrink, plan_struct,
    lora_apply_workspace_bytes, lora_bgmv_expand, lora_bgmv_shrink, lora_build_meta,
    lora_build_meta_device,
    lora_pool_bytes_A, lora_pool_bytes_B, lora_pool_clear, lora_pool_load, lora_pool_validate,
    lora_scaling, lora_sgmv_expand, lora_sgmv_shrink, last_error,
)
from .pool import LoraPool  # noqa: F401
