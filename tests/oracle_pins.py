"""Pins of the fp64 oracle against facts fixed outside the oracle itself.

Each ``pin_*`` takes the oracle module (so a planted mistake can be injected by
patching it) and raises AssertionError when the oracle disagrees with:
hand-worked values (tests/golden), closed forms, invariants, a library routine
(torch's bfloat16 cast, numpy's stable argsort) or a pure-Python brute force.
"""
from __future__ import annotations

import json
import math
import os
import types

import numpy as np

import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def hand_workload(rslora_slot1=True):
    g = _load("delta_hand.json")
    slots = {}
    for k, s in g["slots"].items():
        slots[int(k)] = W.AdapterSpec(
            rank=s["rank"], alpha=s["alpha"],
            use_rslora=(s["use_rslora"] if int(k) != 1 else rslora_slot1),
            A=[np.asarray(s["A"], np.float32)], B=[np.asarray(s["B"], np.float32)])
    return W.Workload("hand", "f32", g["in_features"], g["out_features"], 2, 4, slots,
                      np.asarray(g["ids"], np.int32), np.zeros(3, np.uint8),
                      np.asarray(g["x"], np.float32), np.asarray(g["y_in"], np.float32)), g


# --- delta definition -------------------------------------------------------

def pin_hand_example(O):
    wl, g = hand_workload()
    got = O.lora_forward_rows(wl)
    assert np.array_equal(got, np.asarray(g["y_out"], np.float64)), got
    wl2, _ = hand_workload(rslora_slot1=False)
    got2 = O.lora_forward_rows(wl2, rows=[2])
    assert np.array_equal(got2[0], np.asarray(g["y_out_slot1_without_rslora"])), got2
    bf = O.brute_force_rows(wl, range(3))
    assert np.array_equal(np.asarray(bf), np.asarray(g["y_out"], np.float64)), bf
    m = O.merged_weight_rows(np.asarray(g["merged_W"], np.float64), wl, [0])
    assert np.array_equal(m[0], np.asarray(g["merged_t0"], np.float64)), m


def slices_hand_workload(rslora_slot1=True, R=4):
    g = _load("delta_slices_hand.json")
    slots = {}
    for k, s in g["slots"].items():
        slots[int(k)] = W.AdapterSpec(
            rank=s["rank"], alpha=s["alpha"],
            use_rslora=(s["use_rslora"] if int(k) != 1 else rslora_slot1),
            A=[np.asarray(a, np.float32) for a in s["A"]],
            B=[np.asarray(b, np.float32) for b in s["B"]])
    T = len(g["ids"])
    return W.Workload("hand_slices", "f32", g["in_features"], g["out_features"], 2, R, slots,
                      np.asarray(g["ids"], np.int32), np.zeros(T, np.uint8),
                      np.asarray(g["x"], np.float32), np.asarray(g["y_in"], np.float32)), g


def pin_slices_hand_example(O):
    """Three output slices of widths 2, 1, 3, each with its own A and B: the
    placement of every slice's delta in the fused output row is fixed by the
    hand-worked values, so a reversed, shifted or collapsed slice layout, or
    one slice's A used for another, fails here."""
    wl, g = slices_hand_workload()
    assert list(O.slice_offsets(wl.out_features)) == g["slice_offsets"]
    want = np.asarray(g["y_out"], np.float64)
    assert np.array_equal(O.lora_forward_rows(wl), want)
    assert np.array_equal(np.asarray(O.brute_force_rows(wl, range(wl.T))), want)
    wl2, _ = slices_hand_workload(rslora_slot1=False)
    assert np.array_equal(O.lora_forward_rows(wl2, rows=[2])[0],
                          np.asarray(g["y_out_t2_without_rslora"], np.float64))
    # the padded, folded pool gives the same rows (scales 2 and 1 fold exactly)
    pool = O.expected_pool(wl)
    assert np.array_equal(O.forward_from_pool_rows(wl, pool, range(wl.T)), want)
    # merging into a zero base weight leaves exactly the delta
    d = O.merged_weight_rows(np.zeros((wl.O, wl.in_features)), wl, [0, 2, 3])
    assert np.array_equal(d, want[[0, 2, 3]] - wl.y_in[[0, 2, 3]].astype(np.float64))
    # the rank-space intermediate is laid out slice by slice, R values each:
    # t0 (slot 0, rank 2): A_s x = [1, 2], [3, -1], [2, 2]
    v = O.lora_shrink_rows(wl, [0, 1])
    assert np.array_equal(v[0], [1, 2, 0, 0, 3, -1, 0, 0, 2, 2, 0, 0]) and not np.any(v[1])


def pin_scaling(O):
    # alpha / r and alpha / sqrt(r); the values used by the named workloads
    assert O.scaling(8, 16.0, False) == 2.0
    assert O.scaling(16, 32.0, False) == 2.0
    assert O.scaling(16, 16.0, True) == 4.0
    assert O.scaling(64, 128.0, False) == 2.0
    assert O.scaling(4, 8.0, True) == 4.0 and O.scaling(4, 8.0, False) == 2.0
    assert abs(O.scaling(2, 4.0, True) - 2.0 * math.sqrt(2.0)) < 1e-15
    assert O.scaling(3, 1.5, False) == 0.5


def pin_brute_force_tiny(O):
    wl = W.config_tiny_fp32(seed=3)
    rows = list(range(wl.T))
    ref = O.lora_forward_rows(wl, rows)
    bf = np.asarray(O.brute_force_rows(wl, rows))
    assert O.rel_err_rows(ref, bf) < 1e-12


def pin_merged_closed_form(O):
    for wl in (W.config_tiny_fp32(seed=5),
               W.config_qkv_decode(seed=1, T=12, K=64, outs=(64, 16, 16), n_adapters=4,
                                   rank=16, dtype="f32")):
        rng = np.random.default_rng(11)
        Wb = rng.standard_normal((wl.O, wl.in_features))
        y_base = wl.x.astype(np.float64) @ Wb.T
        rows = list(range(wl.T))
        got = O.lora_forward_rows(wl, rows, y_in=y_base)
        ref = O.merged_weight_rows(Wb, wl, rows)
        assert O.rel_err_rows(got, ref) < 1e-12


def pin_zero_B_and_none_rows(O):
    wl = W.with_zero_B(W.config_tiny_fp32(seed=2))
    got = O.lora_forward_rows(wl)
    assert np.array_equal(got, wl.y_in.astype(np.float64))
    wl = W.config_tiny_fp32(seed=2)
    got = O.lora_forward_rows(wl)
    none = np.where(wl.ids < 0)[0]
    assert none.size > 0
    assert np.array_equal(got[none], wl.y_in[none].astype(np.float64))
    act = np.where(wl.ids >= 0)[0]
    assert np.all(np.any(got[act] != wl.y_in[act], axis=1))


def pin_linearity(O):
    wl = W.config_tiny_fp32(seed=4)
    zero = np.zeros_like(wl.y_in)
    d1 = O.lora_forward_rows(wl, y_in=zero)
    wl2 = W.Workload(**{**wl.__dict__, "x": wl.x * 2.0})
    d2 = O.lora_forward_rows(wl2, y_in=zero)
    assert np.array_equal(d2, 2.0 * d1)


def pin_permutation(O):
    wl = W.config_qkv_decode(seed=2, T=20, K=64, outs=(32, 16), n_adapters=5, rank=8,
                             dtype="f32")
    ref = O.lora_forward_rows(wl)
    p = np.random.default_rng(0).permutation(wl.T)
    wlp = W.Workload(**{**wl.__dict__, "ids": wl.ids[p], "x": wl.x[p], "y_in": wl.y_in[p],
                        "prefill": wl.prefill[p]})
    got = O.lora_forward_rows(wlp)
    assert np.array_equal(got, ref[p])


def pin_shrink(O):
    wl = W.config_tiny_fp32(seed=6, max_lora_rank=16)
    rows = list(range(wl.T))
    v = O.lora_shrink_rows(wl, rows)
    for i in (0, 9, 17, 30):
        a = int(wl.ids[i])
        if a < 0:
            assert not np.any(v[i])
            continue
        ad = wl.slots[a]
        for k in range(16):
            if k >= ad.rank:
                assert v[i, k] == 0.0
            else:
                bf = sum(float(ad.A[0][k][j]) * float(wl.x[i][j]) for j in range(wl.in_features))
                assert abs(v[i, k] - bf) <= 1e-12 * max(1.0, abs(bf))


# --- pool -------------------------------------------------------------------

def pin_padding_inert(O):
    for R in (8, 16, 64):
        wl = W.config_tiny_fp32(seed=7, max_lora_rank=R)
        pool = O.expected_pool(wl)
        for a, p in pool.items():
            r = wl.slots[a].rank
            assert not np.any(p["A"][0][r:]) and not np.any(p["B"][0][:, r:])
            assert p["A"][0].shape == (R, wl.in_features) and p["B"][0].shape == (256, R)
        got = O.forward_from_pool_rows(wl, pool, range(wl.T))
        ref = O.lora_forward_rows(wl)
        assert np.array_equal(got, ref)     # s = 2: the fold is exact


def pin_fold_rounding(O):
    # non-power-of-two scale (alpha 3, r 8 -> 0.375 * bf16 B is inexact in bf16)
    wl = W.config_sgmv_prefill(seed=1, n_seqs=3, len_lo=4, len_hi=6, K=64, O=48,
                               n_adapters=3, rank_choices=(8,), max_lora_rank=16,
                               alpha_per_rank=3.0 / 8.0)
    pool = O.expected_pool(wl)
    rows = list(range(wl.T))
    got = O.forward_from_pool_rows(wl, pool, rows)
    ref = O.lora_forward_rows(wl, rows)
    d_ref = ref - wl.y_in.astype(np.float64)
    d_got = got - wl.y_in.astype(np.float64)
    # each folded entry is within 2^-8 relative of s*B, so the delta is within
    # 2^-8 of sum_k |s B_jk v_k| (bounded here by the norm of the terms)
    for i, t in enumerate(rows):
        ad = wl.slots[int(wl.ids[t])]
        s = O.scaling(ad.rank, ad.alpha, ad.use_rslora)
        v = ad.A[0].astype(np.float64) @ wl.x[t].astype(np.float64)
        bound = (2.0 ** -8) * (np.abs(s * ad.B[0].astype(np.float64)) @ np.abs(v)) + 1e-12
        assert np.all(np.abs(d_got[i] - d_ref[i]) <= bound)
    assert not np.array_equal(got, ref)  # the fold really rounds here


def pin_pool_bytes(O):
    # one matrix, one slot, rank r: r (d + k) parameters
    r, d, k = 16, 4096, 3072
    a, b = O.pool_bytes(1, 1, r, k, d, 1)
    assert a + b == r * (d + k)
    assert d * k / (r * (d + k)) > 100  # the "about 100x fewer" order of magnitude
    a, b = O.pool_bytes(64, 3, 16, 4096, 6144, 2)
    assert a == 64 * 3 * 16 * 4096 * 2 and b == 64 * 16 * 6144 * 2


def pin_bf16_rne(O):
    import torch
    rng = np.random.default_rng(0)
    a = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(3.0),
        (rng.standard_normal(2000) * 1e-38).astype(np.float32),
        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 1.0 + 2 ** -8 + 2 ** -20,
                  -1.00390625, 65504.0, 3.3895314e38, np.inf, -np.inf], np.float32),
    ])
    # exact ties: low 16 bits == 0x8000
    ties = (rng.integers(0, 2 ** 31, 500, dtype=np.uint64).astype(np.uint32) & 0x7FFF0000) | 0x8000
    a = np.concatenate([a, ties.view(np.float32)[np.isfinite(ties.view(np.float32))]])
    ref = torch.from_numpy(a.copy()).to(torch.bfloat16).to(torch.float32).numpy()
    got = O.f32_to_bf16_rne(a)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    assert np.isnan(O.f32_to_bf16_rne(np.array([np.nan], np.float32))[0])


def pin_f64_to_bf16_rne(O):
    import torch
    # float32 inputs: one rounding, so torch's float32 -> bfloat16 cast decides
    rng = np.random.default_rng(1)
    a = np.concatenate([rng.standard_normal(5000).astype(np.float32) * np.float32(7.0),
                        np.array([1.00390625, 1.01171875, -1.00390625, 3.0], np.float32)])
    ref = torch.from_numpy(a.copy()).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.f64_to_bf16_rne(a.astype(np.float64)), ref)
    # hand cases where rounding through float32 first goes wrong: just above,
    # just below and exactly on the midpoint between 1 and 1 + 2^-7
    got = O.f64_to_bf16_rne(np.array([1 + 2 ** -8 + 2 ** -30, 1 + 2 ** -8 - 2 ** -30, 1 + 2 ** -8,
                                      -(1 + 2 ** -8 + 2 ** -30), 1 + 3 * 2 ** -8]))
    assert list(got) == [1 + 2 ** -7, 1.0, 1.0, -(1 + 2 ** -7), 1 + 2 ** -6]
    # brute force: nearest of the 129 bfloat16 values in [1, 2], ties to even
    grid = 1.0 + np.arange(129) / 128.0
    v = 1.0 + rng.random(3000)
    v[:200] = 1.0 + (rng.integers(0, 128, 200) + 0.5) / 128.0  # exact midpoints
    d = np.abs(v[:, None] - grid[None, :])
    best = d.min(axis=1, keepdims=True)
    want = []
    for i in range(v.size):
        cand = np.nonzero(d[i] == best[i, 0])[0]
        want.append(grid[cand[0]] if cand.size == 1 else grid[[c for c in cand if c % 2 == 0][0]])
    assert np.array_equal(O.f64_to_bf16_rne(v), np.asarray(want))


def pin_merged_weight(O):
    # hand 2 x 2: W + B A with B = [[2], [0.5]], A = [[1, -1]] (rank 1 padded to 2)
    slot = {"A": [np.array([[1.0, -1.0], [0.0, 0.0]])], "B": [np.array([[2.0, 0.0], [0.5, 0.0]])]}
    W0 = np.array([[1.0, 2.0], [3.0, 4.0]])
    for dt in ("f32", "bf16"):
        assert np.array_equal(O.merged_weight(W0, slot, 0, dt), [[3.0, 0.0], [3.5, 3.5]])
    # exact integer inputs: the merged weight applied to x equals the base
    # product plus the runtime delta from the same pool, slice by slice
    wl = W.config_integer(seed=5, T=24, K=72, outs=(40, 24), max_loras=4, max_lora_rank=16,
                          ranks=(8, 16, 8, 16), dtype="bf16")
    pool = O.expected_pool(wl)
    offs = O.slice_offsets(wl.out_features)
    rows = [t for t in range(wl.T) if wl.ids[t] >= 0]
    delta = O.forward_from_pool_rows(wl, pool, rows) - wl.y_in[rows].astype(np.float64)
    for sl, (off, width) in enumerate(zip(offs, wl.out_features)):
        Wb = W.draw_base_weight(9 + sl, width, wl.in_features, "bf16", integer_values=True)
        for i, t in enumerate(rows):
            Wm = O.merged_weight(Wb, pool[int(wl.ids[t])], sl, "bf16")
            x = wl.x[t].astype(np.float64)
            assert np.array_equal(Wm @ x, Wb.astype(np.float64) @ x + delta[i, off:off + width])


# --- builder ----------------------------------------------------------------

META_KEYS = ("sgmv_perm", "seg_starts", "seg_lens", "seg_ids", "bgmv_tok", "bgmv_ids")


def pin_builder_golden(O):
    for case in _load("builder_tiny.json")["cases"]:
        m = O.build_meta(case["ids"], case["prefill"], case["max_lora_rank"], 64)
        for k in META_KEYS:
            assert list(m[k]) == case[k], (case["name"], k, m[k])


def check_meta_properties(ids, prefill, R, m, bgmv_max_rank=64):
    ids = np.asarray(ids)
    pre = np.asarray(prefill).astype(bool)
    T = ids.shape[0]
    sg_mask = (ids >= 0) & (pre | (R > bgmv_max_rank))
    bg_mask = (ids >= 0) & ~(pre | (R > bgmv_max_rank))
    perm = np.asarray(m["sgmv_perm"], np.int64)
    # library routine: numpy's stable argsort over the id key
    sg = np.where(sg_mask)[0]
    assert np.array_equal(perm, sg[np.argsort(ids[sg], kind="stable")])
    bg = np.where(bg_mask)[0]
    assert np.array_equal(np.asarray(m["bgmv_tok"], np.int64), bg[np.argsort(ids[bg], kind="stable")])
    assert np.array_equal(np.asarray(m["bgmv_ids"]), ids[np.asarray(m["bgmv_tok"], np.int64)])
    st, ln, sid = (np.asarray(m[k], np.int64) for k in ("seg_starts", "seg_lens", "seg_ids"))
    assert ln.sum() == perm.size and np.all(ln > 0)
    assert np.all(np.diff(sid) > 0) if sid.size > 1 else True
    if st.size:
        assert st[0] == 0 and np.array_equal(st[1:], np.cumsum(ln)[:-1])
    for s, l, a in zip(st, ln, sid):
        assert np.all(ids[perm[s:s + l]] == a)
    assert len(set(sid.tolist())) == sid.size == len(set(ids[sg].tolist()))
    assert perm.size + len(m["bgmv_tok"]) == int((ids >= 0).sum()) <= T


def pin_builder_properties(O):
    rng = np.random.default_rng(123)
    for trial in range(60):
        T = int(rng.integers(0, 300))
        n = int(rng.integers(1, 40))
        ids = rng.integers(-1, n, size=T)
        if trial % 3 == 0:
            ids = np.sort(ids)
        pre = rng.integers(0, 2, size=T)
        R = int(rng.choice([8, 16, 64, 72, 128]))
        m = O.build_meta(ids.tolist(), pre.tolist(), R, 64)
        check_meta_properties(ids, pre, R, m)


def pin_rel_err(O):
    assert O.rel_err_rows([[1.0, 2.0]], [[1.0, 2.0]]) == 0.0
    assert O.rel_err_rows([[1.0, 2.5], [1.0, -3.5]], [[1.0, 2.0], [1.0, -4.0]]) == 0.25
    assert O.rel_err_rows(np.zeros((0, 3)), np.zeros((0, 3))) == 0.0


def pin_slot_residency(O):
    """Hand-worked: max_loras = 2.  [1] loads 1; [2] loads 2 -> {1, 2}; [3]
    evicts 1 (least recently used) -> {2, 3}; [None, 2] loads nothing, touches
    2 -> {3, 2}; [1, 2] evicts 3 (not in the batch) -> {1, 2}, 2 most recent
    (order of first use); [2, 2, None] -> {1, 2}; [4, 1] evicts 2, the one not
    in the batch, and leaves 1 most recent -> {4, 1}; [3, 4] evicts 1 and
    keeps 4, which the batch uses, though 4 is the least recently used."""
    got = O.slot_residency([[1], [2], [3], [None, 2], [1, 2], [2, 2, None], [4, 1], [3, 4]], 2)
    assert got == [([1], [1]), ([1, 2], [2]), ([2, 3], [3]), ([3, 2], []), ([1, 2], [1]),
                   ([1, 2], []), ([4, 1], [4]), ([3, 4], [3])]
    # max_loras = 1 serialises adapters: each new adapter replaces the last
    assert O.slot_residency([[5], [6], [6], [5]], 1) == [([5], [5]), ([6], [6]), ([6], []),
                                                          ([5], [5])]
    # invariants on random sequences: capacity; every adapter of a batch
    # resident after it; loads are exactly the adapters that were not resident
    rng = np.random.default_rng(4)
    for _ in range(50):
        m = int(rng.integers(1, 5))
        batches = [list(rng.choice(np.arange(8), size=int(rng.integers(0, m + 1)),
                                   replace=False)) for _ in range(20)]
        prev = []
        for b, (res, loaded) in zip(batches, O.slot_residency(batches, m)):
            assert len(res) <= m and len(set(res)) == len(res)
            assert set(int(a) for a in b) <= set(res)
            assert sorted(loaded) == sorted(set(int(a) for a in b) - set(prev))
            prev = res


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")
            and isinstance(v, types.FunctionType)]
