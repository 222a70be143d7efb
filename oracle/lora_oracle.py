"""fp64 CPU oracle for the multi-LoRA delta path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: it is used by ``tests/``, by ``__graft_entry__.smoke()``
and by the ``cpu_baseline`` leg of ``bench.py``.  It shares no code with the
HIP library (no kernels, helpers, tables or pre/post-processing); the only
thing both sides share is the seeded input generator in ``workloads.py``,
which draws inputs and holds none of the method's arithmetic.

Pages cited (by title and section):

* [TGI] "Text Generation Inference 多 LoRA 适配器服务实战: LORA_ADAPTERS 配置与
  SGMV/BGMV 内核加速原理" (nxmr.cn).  Sections used: "什么是 LoRA" (what LoRA
  is); implementation step 3 "权重预处理: 缩放因子与 rank 对齐" (weight
  preparation: scaling factor folded into lora_B, rank padding); step 4
  "推理时计算: SGMV 与 BGMV" (prefill segments -> SGMV, decode tokens -> BGMV,
  choice by prefill flag and rank limit); step 5 (uneven q/k/v slices).
* [vLLM] "vLLM 怎么在离线推理中为单次请求挂载不同 LoRA 适配器" (lmnt.cn).
  Sections used: the LoRARequest binding rules (a None entry runs the base
  model), step 2 on max_loras / max_lora_rank, and "限制与边界" (limits: the
  slot rank must cover every adapter's rank).
* [QA] "Multi-LoRA serving: 一基座, 多 adapter" (inference-learning-path).
  Sections used: "直接答案" (delta W = B A with B in R^{d x r}, A in R^{r x k};
  one shared base GEMM Wx per batch plus a per-row B(Ax) grouped by adapter
  id) and the follow-up on merging an adapter into the base weights.

Every function below is a plain definition written out; there is no blocking,
fusion or reordering beyond the definition.  Parity status of each function is
listed in ``PINS`` at the bottom of the file.
"""
from __future__ import annotations

import math
from typing import Dict, Iterable, List, Optional, Sequence

import numpy as np

BGMV_MAX_RANK_DEFAULT = 64


# ----------------------------------------------------------------------------
# Scaling (TGI, step 3: standard scale alpha / r, rsLoRA scale alpha / sqrt(r))
# ----------------------------------------------------------------------------

def scaling(rank: int, alpha: float, use_rslora: bool) -> float:
    """LoRA scale for an adapter of its own rank ``rank`` (never the padded slot
    rank: padding adds zero rows and must not change the result).
    [TGI] step 3: alpha / r, or alpha / r**0.5 when rsLoRA is enabled."""
    if rank <= 0:
        raise ValueError("rank must be positive")
    if use_rslora:
        return float(alpha) / math.sqrt(float(rank))
    return float(alpha) / float(rank)


# ----------------------------------------------------------------------------
# The delta path itself, per token, in fp64
# ----------------------------------------------------------------------------

def slice_offsets(out_features: Sequence[int]) -> List[int]:
    """Column offset of each output slice inside the fused output row
    ([TGI] step 5: q/k/v or gate/up slices of different widths sit side by side)."""
    offs, acc = [], 0
    for o in out_features:
        offs.append(acc)
        acc += int(o)
    return offs


def lora_forward_rows(wl, rows: Optional[Iterable[int]] = None, y_in=None) -> np.ndarray:
    """Per-token fp64 loop: for token t with adapter a = ids[t] >= 0 and every
    slice s, y[t, off_s:off_s+out_s] = y_in[...] + s_a * B_{a,s} (A_{a,s} x_t);
    tokens with id -1 keep y_in.

    [QA] direct answer: the base output Wx is shared by the batch and each row
    adds B(Ax) of its own adapter.  [TGI] step 3 gives s_a.  [vLLM] LoRARequest
    rules: a row without adapter is served by the base model unchanged.

    Uses the unpadded, unfolded adapter matrices; returns fp64 rows.
    """
    if rows is None:
        rows = range(wl.T)
    rows = list(rows)
    src = wl.y_in if y_in is None else y_in
    offs = slice_offsets(wl.out_features)
    out = np.empty((len(rows), sum(wl.out_features)), dtype=np.float64)
    for i, t in enumerate(rows):
        y = np.array(src[t], dtype=np.float64)
        a = int(wl.ids[t])
        if a >= 0:
            ad = wl.slots[a]
            s_a = scaling(ad.rank, ad.alpha, ad.use_rslora)
            xt = np.asarray(wl.x[t], dtype=np.float64)
            for sl, (off, width) in enumerate(zip(offs, wl.out_features)):
                A = np.asarray(ad.A[sl], dtype=np.float64)   # [r, K]
                B = np.asarray(ad.B[sl], dtype=np.float64)   # [out_s, r]
                v = A @ xt                                   # shrink: x -> r
                y[off:off + width] += s_a * (B @ v)          # expand: r -> out
        out[i] = y
    return out


def lora_shrink_rows(wl, rows: Iterable[int]) -> np.ndarray:
    """The intermediate v_t = A_{a,s} x_t for each slice, concatenated in slice
    order and zero-extended to the padded rank R: [len(rows), S * R] fp64.
    Rows without adapter give zeros.  ([QA] direct answer: the A x stage.)"""
    rows = list(rows)
    R, S = wl.max_lora_rank, wl.num_slices
    out = np.zeros((len(rows), S * R), dtype=np.float64)
    for i, t in enumerate(rows):
        a = int(wl.ids[t])
        if a < 0:
            continue
        ad = wl.slots[a]
        xt = np.asarray(wl.x[t], dtype=np.float64)
        for sl in range(S):
            v = np.asarray(ad.A[sl], dtype=np.float64) @ xt
            out[i, sl * R: sl * R + ad.rank] = v
    return out


def brute_force_rows(wl, rows: Iterable[int]) -> List[List[float]]:
    """Pure-Python triple loop of the same definition (tiny inputs only):
    y[j] += s * sum_k B[j][k] * sum_i A[k][i] * x[i]."""
    offs = slice_offsets(wl.out_features)
    res = []
    for t in rows:
        y = [float(v) for v in wl.y_in[t]]
        a = int(wl.ids[t])
        if a >= 0:
            ad = wl.slots[a]
            s_a = scaling(ad.rank, ad.alpha, ad.use_rslora)
            xt = [float(v) for v in wl.x[t]]
            for sl, off in enumerate(offs):
                A = ad.A[sl]
                B = ad.B[sl]
                v = []
                for k in range(ad.rank):
                    acc = 0.0
                    row = A[k]
                    for i in range(len(xt)):
                        acc += float(row[i]) * xt[i]
                    v.append(acc)
                for j in range(B.shape[0]):
                    acc = 0.0
                    for k in range(ad.rank):
                        acc += float(B[j][k]) * v[k]
                    y[off + j] += s_a * acc
        res.append(y)
    return res


def merged_weight_rows(W: np.ndarray, wl, rows: Iterable[int]) -> np.ndarray:
    """Closed form from merging the adapter into the base weight ([QA] follow-up
    on merging; delta W = B A): y_t = (W + s_a B_a A_a) x_t, computed by forming
    the merged matrix first.  W is [O, K] fp64; rows without adapter use W."""
    offs = slice_offsets(wl.out_features)
    out = []
    for t in rows:
        xt = np.asarray(wl.x[t], dtype=np.float64)
        a = int(wl.ids[t])
        Wm = np.array(W, dtype=np.float64)
        if a >= 0:
            ad = wl.slots[a]
            s_a = scaling(ad.rank, ad.alpha, ad.use_rslora)
            for sl, (off, width) in enumerate(zip(offs, wl.out_features)):
                dW = np.asarray(ad.B[sl], np.float64) @ np.asarray(ad.A[sl], np.float64)
                Wm[off:off + width] += s_a * dW
        out.append(Wm @ xt)
    return np.asarray(out)


# ----------------------------------------------------------------------------
# Rounding helpers (the oracle's own; used only to state what a dtype holds)
# ----------------------------------------------------------------------------

def f32_to_bf16_rne(a) -> np.ndarray:
    """Round float32 values to the nearest bfloat16, ties to even; NaN stays NaN.
    Returns float32 holding the rounded values."""
    a32 = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = a32.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    out = (r & np.uint64(0xFFFFFFFF)).astype(np.uint32).view(np.float32).copy()
    out[np.isnan(a32)] = np.nan
    return out


def f64_to_bf16_rne(a) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 in one step, ties to even
    (finite inputs).  Rounding through float32 first is not the same: a value
    just above a bfloat16 midpoint can land on the midpoint in float32 and
    then tie to even.  Method: take the float32-then-bfloat16 candidate and its
    two bfloat16 neighbours, keep the one nearest in float64, ties to the even
    bit pattern.  Returns float64 holding the rounded values."""
    v = np.asarray(a, dtype=np.float64)
    c = f32_to_bf16_rne(v.astype(np.float32)).view(np.uint32) >> np.uint32(16)
    best = None
    best_err = None
    for d in (0, -1, 1):  # the float32-route candidate first: it is always finite
        bits = (c.astype(np.int64) + d).astype(np.uint32)
        val = (bits << np.uint32(16)).astype(np.uint32).view(np.float32).astype(np.float64)
        err = np.abs(val - v)
        if best is None:
            best, best_err, best_bits = val, err, bits
            continue
        take = (err < best_err) | ((err == best_err) & ((bits & 1) == 0) & ((best_bits & 1) == 1))
        best = np.where(take, val, best)
        best_bits = np.where(take, bits, best_bits)
        best_err = np.where(take, err, best_err)
    return best


def round_exact_to_dtype(values_fp64, dtype: str) -> np.ndarray:
    """Single rounding of values that are exactly representable in fp32 (e.g.
    integers below 2^24) to the storage dtype."""
    v32 = np.asarray(values_fp64, dtype=np.float64).astype(np.float32)
    if not np.array_equal(v32.astype(np.float64), np.asarray(values_fp64, np.float64)):
        raise ValueError("values are not exactly representable in fp32")
    return v32 if dtype == "f32" else f32_to_bf16_rne(v32)


# ----------------------------------------------------------------------------
# Adapter pool contents (TGI step 3; vLLM step 2 and limits)
# ----------------------------------------------------------------------------

def expected_pool(wl) -> Dict[int, dict]:
    """What a rank-padded pool slot must hold after loading an adapter.

    [TGI] step 3: the scale is multiplied into lora_B once at load time
    (associativity), and ranks are padded so every adapter fits the kernels'
    vector width.  [vLLM] step 2 and limits: each slot is pre-sized to
    max_lora_rank, which must cover the adapter's rank.

    For slot a, slice s (R = max_lora_rank, r = adapter rank):
      A_pad[s] = [A_s ; zeros(R - r, K)]                      shape [R, K]
      B_fold[s] = [round_dtype(fp32(B_s) * fp32(s_a)) , 0]    shape [out_s, R]
    The fold multiplies in fp32 and rounds once to the pool dtype, so it is a
    rounding decision both sides take in the same precision.
    """
    R = wl.max_lora_rank
    out = {}
    for a, ad in wl.slots.items():
        if ad.rank > R:
            raise ValueError("adapter rank exceeds the slot rank")
        s32 = np.float32(scaling(ad.rank, ad.alpha, ad.use_rslora))
        A_pad, B_fold = [], []
        for sl in range(wl.num_slices):
            A = np.asarray(ad.A[sl], np.float32)
            B = np.asarray(ad.B[sl], np.float32)
            Ap = np.zeros((R, wl.in_features), np.float32)
            Ap[:ad.rank] = A
            prod = (B * s32).astype(np.float32)
            if wl.dtype == "bf16":
                prod = f32_to_bf16_rne(prod)
            Bp = np.zeros((B.shape[0], R), np.float32)
            Bp[:, :ad.rank] = prod
            A_pad.append(Ap)
            B_fold.append(Bp)
        out[a] = {"A": A_pad, "B": B_fold, "scale_f32": float(s32)}
    return out


def forward_from_pool_rows(wl, pool: Dict[int, dict], rows: Iterable[int]) -> np.ndarray:
    """The same delta evaluated from padded, folded pool slots in fp64:
    y = y_in + B_fold (A_pad x).  Differs from ``lora_forward_rows`` only by the
    fold's rounding; identical when every scale is a power of two."""
    offs = slice_offsets(wl.out_features)
    rows = list(rows)
    out = np.empty((len(rows), sum(wl.out_features)), dtype=np.float64)
    for i, t in enumerate(rows):
        y = np.array(wl.y_in[t], dtype=np.float64)
        a = int(wl.ids[t])
        if a >= 0:
            xt = np.asarray(wl.x[t], np.float64)
            for sl, (off, width) in enumerate(zip(offs, wl.out_features)):
                v = pool[a]["A"][sl].astype(np.float64) @ xt
                y[off:off + width] += pool[a]["B"][sl].astype(np.float64) @ v
        out[i] = y
    return out


def merged_weight(W, pool_slot: dict, sl: int, dtype: str) -> np.ndarray:
    """Merged-weight mode ([QA] follow-up on merging an adapter into the base):
    W' = W + B_fold A_pad for one slice of one pool slot (B_fold holds the
    scale, so this is W + s_a B A), formed in fp64 and rounded once to the
    dtype, nearest with ties to even.  W is [out_s, K]."""
    Wm = np.asarray(W, np.float64) + (np.asarray(pool_slot["B"][sl], np.float64)
                                      @ np.asarray(pool_slot["A"][sl], np.float64))
    if dtype == "bf16":
        return f64_to_bf16_rne(Wm)
    return Wm.astype(np.float32).astype(np.float64)


def pool_bytes(max_loras: int, num_slices: int, R: int, K: int, out_total: int,
               elem_bytes: int):
    """Pool footprint: every slot reserves R rows of A per slice and R columns of
    B per output column ([vLLM] step 2: each slot is a pre-allocated tensor, so
    memory grows with max_loras and max_lora_rank).  Returns (A bytes, B bytes)."""
    return (max_loras * num_slices * R * K * elem_bytes, max_loras * R * out_total * elem_bytes)


# ----------------------------------------------------------------------------
# Segment / index metadata (TGI step 4)
# ----------------------------------------------------------------------------

def build_meta(ids: Sequence[int], prefill: Sequence[int], max_lora_rank: int,
               bgmv_max_rank: int = BGMV_MAX_RANK_DEFAULT) -> dict:
    """Split the batch's rows between the two grouped kernels and group them.

    [TGI] step 4: prefill rows go to SGMV (segments of contiguous tokens that
    share an adapter), decode rows to BGMV (per-token adapter gather); SGMV is
    also used whenever the rank exceeds the BGMV limit.  Rows without adapter
    (id -1, [vLLM] None request) are in neither set.

    SGMV: token indices sorted by (id, index) -> perm; each maximal run of equal
    id in perm is one segment (start offset into perm, length, id).
    BGMV: token indices sorted by (id, index) -> bgmv_tok, with their ids.
    """
    T = len(ids)
    use_sgmv_all = max_lora_rank > bgmv_max_rank
    sg = [t for t in range(T) if ids[t] >= 0 and (bool(prefill[t]) or use_sgmv_all)]
    bg = [t for t in range(T) if ids[t] >= 0 and not (bool(prefill[t]) or use_sgmv_all)]
    perm = sorted(sg, key=lambda t: (int(ids[t]), t))
    seg_starts, seg_lens, seg_ids = [], [], []
    for pos, t in enumerate(perm):
        a = int(ids[t])
        if seg_ids and seg_ids[-1] == a:
            seg_lens[-1] += 1
        else:
            seg_starts.append(pos)
            seg_lens.append(1)
            seg_ids.append(a)
    bgmv_tok = sorted(bg, key=lambda t: (int(ids[t]), t))
    bgmv_ids = [int(ids[t]) for t in bgmv_tok]
    return {
        "sgmv_perm": perm,
        "seg_starts": seg_starts,
        "seg_lens": seg_lens,
        "seg_ids": seg_ids,
        "bgmv_tok": bgmv_tok,
        "bgmv_ids": bgmv_ids,
    }


# ----------------------------------------------------------------------------
# Error metric
# ----------------------------------------------------------------------------

def rel_err_rows(y_test, y_ref) -> float:
    """max over rows of ||y_test[t] - y_ref[t]||_inf / ||y_ref[t]||_inf."""
    yt = np.asarray(y_test, np.float64)
    yr = np.asarray(y_ref, np.float64)
    if yt.size == 0:
        return 0.0
    num = np.max(np.abs(yt - yr), axis=1)
    den = np.maximum(np.max(np.abs(yr), axis=1), np.finfo(np.float64).tiny)
    return float(np.max(num / den))


# ----------------------------------------------------------------------------
# Adapter slots ([vLLM] LoRARequest rules, step 2, limits)
# ----------------------------------------------------------------------------

def slot_residency(batches: Sequence[Sequence[Optional[int]]], max_loras: int) -> List[tuple]:
    """(adapters resident in the GPU slots after the batch, least recently used
    first; adapters the batch had to load, in load order) for each batch,
    under the reading that a batch of at most max_loras distinct adapters
    makes each of them resident, in order of first use in the batch, evicting
    the least recently used adapter the batch does not use when no slot is
    free; every adapter of the batch then becomes most recently used, in order
    of first use.  ([vLLM] step 2: max_loras is the number of distinct
    adapters one batch can use; the article does not fix the eviction order,
    least recently used is the reading.)"""
    resident: List[int] = []          # LRU first
    out = []
    for batch in batches:
        wanted: List[int] = []
        for a in batch:
            if a is not None and a != -1 and a not in wanted:
                wanted.append(int(a))
        assert len(wanted) <= max_loras
        loaded = []
        for a in wanted:
            if a in resident:
                continue
            if len(resident) == max_loras:
                victim = [b for b in resident if b not in wanted][0]
                resident.remove(victim)
            resident.append(a)
            loaded.append(a)
        for a in wanted:
            resident.remove(a)
            resident.append(a)
        out.append((list(resident), loaded))
    return out


# What pins each function (tests/test_oracle_pins.py):
PINS = {
    "scaling": "closed-form values (alpha/r, alpha/sqrt(r)); rsLoRA vs standard ratio",
    "slice_offsets": "hand-worked three-slice example of widths 2, 1, 3 "
                     "(tests/golden/delta_slices_hand.json)",
    "lora_forward_rows": "brute force; merged-weight closed form; hand worked examples "
                         "(one slice; three slices of different widths); B=0 and id=-1 "
                         "invariants; linearity; permutation equivariance",
    "lora_shrink_rows": "equals A x by brute force; zero beyond the adapter rank; "
                        "slice-by-slice layout from the three-slice hand example",
    "brute_force_rows": "hand worked example (tests/golden/delta_hand.json)",
    "merged_weight_rows": "hand worked example; agrees with lora_forward_rows",
    "f32_to_bf16_rne": "torch's float32 -> bfloat16 cast (a library routine), ties",
    "f64_to_bf16_rne": "equals f32_to_bf16_rne on float32 values; hand double-rounding "
                       "cases; brute-force nearest over all bfloat16 values near 1",
    "merged_weight": "merged weight times x equals the runtime delta (forward_from_pool); "
                     "hand 2x2 example; exact on integer inputs",
    "expected_pool": "padding inert (forward_from_pool == forward for power-of-two "
                     "scales); fold rounding bounded by 2^-8",
    "build_meta": "worked example (tests/golden/builder_tiny.json); numpy stable "
                  "argsort; property checks",
    "pool_bytes": "r(d+k) parameter count per matrix",
    "rel_err_rows": "hand values",
    "slot_residency": "hand-worked sequence (tests/test_oracle_pins.py); capacity and "
                      "membership invariants on random sequences",
}
