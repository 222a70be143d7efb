"""Seeded synthetic workloads for the multi-LoRA delta path.

This module only draws inputs: batch structure (which token uses which adapter,
prefill or decode), adapter ranks and alphas, unpadded/unfolded adapter
matrices A (r x in) and B (out x r), activations x and base outputs y.  It holds
none of the method's arithmetic (no scaling, no padding, no folding, no delta),
so both the fp64 oracle and the HIP library can consume what it returns.

Values are drawn in fp64 with ``numpy.random.default_rng(seed)``, rounded to
fp32 (round-to-nearest-even), and, for bf16 workloads, rounded once more to
bf16 (round-to-nearest-even, via torch's CPU cast).  Arrays are returned as
float32 holding exactly the dtype-representable values the GPU receives.

Draw order (fixed): batch structure -> ranks -> A, B per slot (slot order,
slice order) -> x -> y_in.

Distributions: x ~ N(0, 1); A ~ N(0, 1/in); B ~ N(0, 0.02^2); y_in ~ N(0, 1).

The five named workloads mirror the sizes the multi-LoRA serving pages talk
about (q_proj-sized decode, long prefill, fused QKV with GQA slices, and a
gate_up/down MLP pair with mixed prefill and decode rows); their exact recipes
are in the ``config_*`` functions below.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence

import numpy as np

DTYPES = ("f32", "bf16")


@dataclasses.dataclass
class AdapterSpec:
    """One pool slot: the adapter's own rank and alpha, and per-slice matrices."""

    rank: int
    alpha: float
    use_rslora: bool
    A: List[np.ndarray]  # per slice, [rank, in_features], float32 (dtype-exact)
    B: List[np.ndarray]  # per slice, [out_s, rank], float32 (dtype-exact)


@dataclasses.dataclass
class Workload:
    name: str
    dtype: str                 # "f32" or "bf16"
    in_features: int           # K
    out_features: List[int]    # out_s per slice
    max_loras: int
    max_lora_rank: int         # R (padded slot rank)
    slots: Dict[int, AdapterSpec]
    ids: np.ndarray            # int32 [T], -1 = no adapter
    prefill: np.ndarray        # uint8 [T]
    x: np.ndarray              # float32 [T, K]
    y_in: np.ndarray           # float32 [T, O]
    info: dict = dataclasses.field(default_factory=dict)

    @property
    def T(self) -> int:
        return int(self.ids.shape[0])

    @property
    def O(self) -> int:
        return int(sum(self.out_features))

    @property
    def num_slices(self) -> int:
        return len(self.out_features)

    @property
    def active_tokens(self) -> int:
        return int((self.ids >= 0).sum())


# ----------------------------------------------------------------------------
# dtype rounding of drawn values (input preparation, not the method)
# ----------------------------------------------------------------------------

def to_dtype_values(a: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp64 draws to the workload dtype; return float32 holding them."""
    a32 = np.asarray(a, dtype=np.float64).astype(np.float32)
    if dtype == "f32":
        return a32
    if dtype != "bf16":
        raise ValueError(f"unknown dtype {dtype}")
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def _normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float64) * std


def _draw_slots(rng, dtype, K, outs, ranks: Dict[int, int], alphas: Dict[int, float],
                rslora: bool, a_std: Optional[float] = None, b_std: float = 0.02,
                integer_values: bool = False) -> Dict[int, AdapterSpec]:
    slots: Dict[int, AdapterSpec] = {}
    if a_std is None:
        a_std = 1.0 / math.sqrt(K)
    for slot in sorted(ranks):
        r = ranks[slot]
        As, Bs = [], []
        for out_s in outs:
            if integer_values:
                A = rng.integers(-1, 2, size=(r, K)).astype(np.float64)
                B = rng.integers(-1, 2, size=(out_s, r)).astype(np.float64)
            else:
                A = _normal(rng, (r, K), a_std)
                B = _normal(rng, (out_s, r), b_std)
            As.append(to_dtype_values(A, dtype))
            Bs.append(to_dtype_values(B, dtype))
        slots[slot] = AdapterSpec(rank=r, alpha=float(alphas[slot]), use_rslora=rslora,
                                  A=As, B=Bs)
    return slots


def _draw_xy(rng, dtype, T, K, O, integer_values=False):
    if integer_values:
        x = rng.integers(-1, 2, size=(T, K)).astype(np.float64)
        y = rng.integers(-8, 9, size=(T, O)).astype(np.float64)
    else:
        x = rng.standard_normal(size=(T, K), dtype=np.float64)
        y = rng.standard_normal(size=(T, O), dtype=np.float64)
    return to_dtype_values(x, dtype), to_dtype_values(y, dtype)


# ----------------------------------------------------------------------------
# Named workloads
# ----------------------------------------------------------------------------

def config_tiny_fp32(seed: int = 0, max_lora_rank: int = 8, prefill: bool = True,
                     dtype: str = "f32") -> Workload:
    """in=out=256, 4 adapters of rank 8 with alpha 16, 32 tokens in 4 contiguous
    runs of 8 using adapters [0, 1, none, 3]."""
    rng = np.random.default_rng(seed)
    K, outs = 256, [256]
    ids = np.repeat(np.array([0, 1, -1, 3], dtype=np.int32), 8)
    pre = np.full(ids.shape, 1 if prefill else 0, dtype=np.uint8)
    ranks = {a: 8 for a in range(4)}
    alphas = {a: 16.0 for a in range(4)}
    slots = _draw_slots(rng, dtype, K, outs, ranks, alphas, rslora=False)
    x, y = _draw_xy(rng, dtype, ids.shape[0], K, sum(outs))
    return Workload("tiny_fp32", dtype, K, outs, 4, max_lora_rank, slots, ids, pre, x, y,
                    info={"seq_lens": [8, 8, 8, 8]})


def config_bgmv_decode(seed: int = 0, T: int = 64, K: int = 3072, O: int = 3072,
                       n_adapters: int = 8, rank: int = 16, alpha: float = 32.0,
                       p_none: float = 0.1, dtype: str = "bf16") -> Workload:
    """Decode batch of single-token rows; per-token adapter uniform over the
    adapters, each token independently without adapter with probability p_none."""
    rng = np.random.default_rng(seed)
    none = rng.random(T) < p_none
    ids = rng.integers(0, n_adapters, size=T).astype(np.int32)
    ids[none] = -1
    pre = np.zeros(T, dtype=np.uint8)
    ranks = {a: rank for a in range(n_adapters)}
    alphas = {a: alpha for a in range(n_adapters)}
    slots = _draw_slots(rng, dtype, K, [O], ranks, alphas, rslora=False)
    x, y = _draw_xy(rng, dtype, T, K, O)
    return Workload("bgmv_decode", dtype, K, [O], n_adapters, rank, slots, ids, pre, x, y)


def config_sgmv_prefill(seed: int = 0, n_seqs: int = 16, len_lo: int = 64, len_hi: int = 1024,
                        K: int = 4096, O: int = 4096, n_adapters: int = 16,
                        rank_choices: Sequence[int] = (8, 16, 32, 64), max_lora_rank: int = 64,
                        random_assignment: bool = False, dtype: str = "bf16",
                        integer_values: bool = False, alpha_per_rank: float = 2.0) -> Workload:
    """Prefill batch: sequences with lengths uniform in [len_lo, len_hi]; sequence i
    uses adapter i (or a uniformly drawn adapter with random_assignment), tokens laid
    out by ascending adapter id; adapter ranks drawn from rank_choices, alpha = 2r."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(len_lo, len_hi + 1, size=n_seqs)
    if random_assignment:
        seq_ids = rng.integers(0, n_adapters, size=n_seqs)
    else:
        seq_ids = np.arange(n_seqs) % n_adapters
    order = np.argsort(seq_ids, kind="stable")
    lens, seq_ids = lens[order], seq_ids[order]
    ids = np.repeat(seq_ids.astype(np.int32), lens)
    pre = np.ones(ids.shape[0], dtype=np.uint8)
    ranks = {a: int(rng.choice(np.asarray(rank_choices))) for a in range(n_adapters)}
    alphas = {a: alpha_per_rank * ranks[a] for a in range(n_adapters)}
    slots = _draw_slots(rng, dtype, K, [O], ranks, alphas, rslora=False,
                        integer_values=integer_values)
    x, y = _draw_xy(rng, dtype, ids.shape[0], K, O, integer_values=integer_values)
    return Workload("sgmv_prefill", dtype, K, [O], n_adapters, max_lora_rank, slots, ids, pre,
                    x, y, info={"seq_lens": lens.tolist(), "seq_ids": seq_ids.tolist()})


def zipf_probs(n: int, s: float) -> np.ndarray:
    w = (np.arange(n, dtype=np.float64) + 1.0) ** (-s)
    return w / w.sum()


def config_qkv_decode(seed: int = 0, T: int = 256, K: int = 4096,
                      outs: Sequence[int] = (4096, 1024, 1024), n_adapters: int = 64,
                      rank: int = 16, alpha: float = 16.0, zipf_s: float = 1.1,
                      dtype: str = "bf16") -> Workload:
    """Fused q/k/v decode with uneven (GQA) slices, each slice with its own A/B;
    adapter popularity follows a truncated Zipf law; rsLoRA scaling."""
    rng = np.random.default_rng(seed)
    ids = rng.choice(n_adapters, size=T, p=zipf_probs(n_adapters, zipf_s)).astype(np.int32)
    pre = np.zeros(T, dtype=np.uint8)
    ranks = {a: rank for a in range(n_adapters)}
    alphas = {a: alpha for a in range(n_adapters)}
    slots = _draw_slots(rng, dtype, K, list(outs), ranks, alphas, rslora=True)
    x, y = _draw_xy(rng, dtype, T, K, sum(outs))
    return Workload("qkv_decode", dtype, K, list(outs), n_adapters, rank, slots, ids, pre, x, y)


def mixed_batch_structure(rng, n_prefill: int, len_lo: int, len_hi: int, n_decode: int,
                          n_adapters: int, p_none: float):
    """Requests = prefill sequences (whole sequence shares one adapter or none)
    followed by single-token decode requests (each its own adapter or none)."""
    lens = rng.integers(len_lo, len_hi + 1, size=n_prefill)
    req_ids = rng.integers(0, n_adapters, size=n_prefill + n_decode).astype(np.int32)
    none = rng.random(n_prefill + n_decode) < p_none
    req_ids[none] = -1
    ids = np.concatenate([np.repeat(req_ids[:n_prefill], lens), req_ids[n_prefill:]])
    pre = np.concatenate([np.ones(int(lens.sum()), np.uint8), np.zeros(n_decode, np.uint8)])
    return ids.astype(np.int32), pre, lens


def config_mlp_mixed(seed: int = 0, n_prefill: int = 8, len_lo: int = 128, len_hi: int = 2048,
                     n_decode: int = 256, hidden: int = 4096, inter: int = 14336,
                     n_adapters: int = 32, rank_choices: Sequence[int] = (16, 64),
                     max_lora_rank: int = 64, p_none: float = 0.05,
                     dtype: str = "bf16"):
    """gate_up (hidden -> 2 x inter, two slices) and down (inter -> hidden) over one
    mixed batch of prefill sequences plus decode tokens; returns (gate_up, down)."""
    rng = np.random.default_rng(seed)
    ids, pre, lens = mixed_batch_structure(rng, n_prefill, len_lo, len_hi, n_decode,
                                           n_adapters, p_none)
    ranks = {a: int(rng.choice(np.asarray(rank_choices))) for a in range(n_adapters)}
    alphas = {a: 2.0 * ranks[a] for a in range(n_adapters)}
    T = ids.shape[0]
    slots_gu = _draw_slots(rng, dtype, hidden, [inter, inter], ranks, alphas, rslora=False)
    slots_dn = _draw_slots(rng, dtype, inter, [hidden], ranks, alphas, rslora=False)
    x_gu, y_gu = _draw_xy(rng, dtype, T, hidden, 2 * inter)
    x_dn, y_dn = _draw_xy(rng, dtype, T, inter, hidden)
    info = {"seq_lens": lens.tolist(), "n_decode": n_decode}
    gu = Workload("mlp_gate_up", dtype, hidden, [inter, inter], n_adapters, max_lora_rank,
                  slots_gu, ids, pre, x_gu, y_gu, info=dict(info))
    dn = Workload("mlp_down", dtype, inter, [hidden], n_adapters, max_lora_rank, slots_dn,
                  ids.copy(), pre.copy(), x_dn, y_dn, info=dict(info))
    return gu, dn


def config_random(seed: int, max_T: int = 900) -> Workload:
    """A seeded random shape and batch, for fuzzing the dispatch: dtype;
    in_features and one to three slice widths (multiples of 8, most not of
    64); slot count, padded rank and each slot's own rank; alpha and rsLoRA;
    and a batch of sorted prefill segments and decode rows (uniform or Zipf
    ids), with rows without adapter, in a random order of blocks."""
    rng = np.random.default_rng(10_000 + seed)
    dtype = "bf16" if rng.random() < 0.75 else "f32"
    K = 8 * int(rng.integers(1, 513))
    S = int(rng.integers(1, 4))
    outs = [8 * int(rng.integers(1, 257)) for _ in range(S)]
    R = int(rng.choice([8, 16, 24, 32, 40, 64, 72, 128]))
    ML = int(rng.integers(1, 48))
    rslora = bool(rng.random() < 0.3)
    used = sorted(rng.choice(ML, size=int(rng.integers(1, ML + 1)), replace=False).tolist())
    ranks = {a: int(rng.integers(1, R + 1)) for a in used}
    alphas = {a: float(rng.choice([1.0, 8.0, 16.0, 2.0 * ranks[a]])) for a in used}
    slots = _draw_slots(rng, dtype, K, outs, ranks, alphas, rslora)
    p_none = float(rng.choice([0.0, 0.1, 0.5]))
    probs = zipf_probs(len(used), 1.1) if rng.random() < 0.5 else np.full(len(used), 1.0 / len(used))
    blocks = []  # (ids, flags)
    budget = int(rng.integers(1, max_T + 1))
    while budget > 0:
        n = int(min(budget, rng.integers(1, 400)))
        if rng.random() < 0.5:  # a prefill segment of one adapter (or none)
            a = -1 if rng.random() < p_none else int(rng.choice(used))
            blocks.append((np.full(n, a, np.int32), np.ones(n, np.uint8)))
        else:  # decode rows
            ids = rng.choice(np.asarray(used, np.int32), size=n, p=probs).astype(np.int32)
            ids[rng.random(n) < p_none] = -1
            blocks.append((ids, np.zeros(n, np.uint8)))
        budget -= n
    order = rng.permutation(len(blocks))
    ids = np.concatenate([blocks[i][0] for i in order])
    flags = np.concatenate([blocks[i][1] for i in order])
    x, y = _draw_xy(rng, dtype, ids.size, K, sum(outs))
    return Workload(name=f"random{seed}", dtype=dtype, in_features=K, out_features=outs,
                    max_loras=ML, max_lora_rank=R, slots=slots, ids=ids, prefill=flags, x=x,
                    y_in=y, info={"seed": seed, "bgmv_max_rank": int(rng.choice([0, 8, 16, 64, 128]))})


def config_integer(seed: int = 0, T: int = 96, K: int = 520, outs: Sequence[int] = (264, 136),
                   max_loras: int = 6, max_lora_rank: int = 64,
                   ranks: Sequence[int] = (8, 16, 64, 32, 48, 64), prefill_frac: float = 0.5,
                   p_none: float = 0.1, dtype: str = "bf16", rslora: bool = False) -> Workload:
    """Exact-arithmetic workload: x, A, B in {-1, 0, 1}, y_in integers in [-8, 8],
    alpha chosen so every scale is a power of two (alpha = 2r, or alpha = 4 sqrt(r)
    with rsLoRA for square ranks).  Every product and partial sum is then an
    integer far below 2^24, so any summation order gives the same fp32 value."""
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, max_loras, size=T).astype(np.int32)
    ids[rng.random(T) < p_none] = -1
    pre = (rng.random(T) < prefill_frac).astype(np.uint8)
    rk = {a: int(ranks[a % len(ranks)]) for a in range(max_loras)}
    if rslora:
        al = {a: 4.0 * math.sqrt(rk[a]) for a in range(max_loras)}
    else:
        al = {a: 2.0 * rk[a] for a in range(max_loras)}
    slots = _draw_slots(rng, dtype, K, list(outs), rk, al, rslora=rslora, integer_values=True)
    x, y = _draw_xy(rng, dtype, T, K, sum(outs), integer_values=True)
    return Workload("integer", dtype, K, list(outs), max_loras, max_lora_rank, slots, ids, pre,
                    x, y)


def with_zero_B(wl: Workload) -> Workload:
    """Same workload with every B matrix replaced by zeros."""
    slots = {a: AdapterSpec(s.rank, s.alpha, s.use_rslora, list(s.A),
                            [np.zeros_like(b) for b in s.B]) for a, s in wl.slots.items()}
    return dataclasses.replace(wl, slots=slots, name=wl.name + "_zeroB")


NAMED = {
    "tiny_fp32": config_tiny_fp32,
    "bgmv_decode": config_bgmv_decode,
    "sgmv_prefill": config_sgmv_prefill,
    "qkv_decode": config_qkv_decode,
    "mlp_mixed": config_mlp_mixed,
}


def draw_base_weight(seed: int, out_features: int, K: int, dtype: str = "bf16",
                     integer_values: bool = False) -> np.ndarray:
    """A base projection weight [out_features, K] for the merged-weight mode:
    entries N(0, 1/K) (the usual scale of a linear layer's weight), or integers
    in [-8, 8] for exact-arithmetic checks; rounded to the dtype."""
    rng = np.random.default_rng(seed)
    if integer_values:
        w = rng.integers(-8, 9, size=(out_features, K)).astype(np.float64)
    else:
        w = rng.standard_normal(size=(out_features, K)) / np.sqrt(K)
    return to_dtype_values(w, dtype)
