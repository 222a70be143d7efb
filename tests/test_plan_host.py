"""lora_apply's host tile plan (CPU only): every SGMV and BGMV row of the batch
is covered exactly once by the shrink tiles and once by the expand tiles, each
tile holds consecutive rows of one adapter, and the records carry the tokens
the metadata builder assigns to those rows."""
from fractions import Fraction

import numpy as np
import pytest

import lora_adapter_pool_amd as L
from lora_adapter_pool_amd import _lib
import workloads as W

WAVE_ROWS, MFMA_ROWS, MFMA_MIN_ROWS, MAX_KSPLIT, MAX_KSPLIT_MFMA = 8, 64, 16, 8, 8
MAX_KSPLIT_MFMA_WIDE = 4   # pools of rank > 32
BGMV_MFMA_MIN_ROWS = 48


def bgmv_mfma_min_total(R):
    """Rows in long runs a decode batch needs before those runs take 64-row
    MFMA tiles: 2048 for pools of rank <= 16, else 1024."""
    return 2048 if R <= 16 else 1024

INT32_MAX = np.iinfo(np.int32).max


def _bgmv_runs(b):
    """(start, length) of each run of equal ids among the BGMV rows."""
    runs, i = [], 0
    while i < b.size:
        j = i
        while j < b.size and b[j] == b[i]:
            j += 1
        runs.append((i, j - i))
        i = j
    return runs


def record_rank(desc, slot_ranks, slot):
    """Rank a tile record carries: the slot's rank rounded up to 8, or 0 (the
    pool rank) without slot ranks, for rank 0 or when the rounding reaches it."""
    if slot_ranks is None or slot_ranks[slot] <= 0:
        return 0
    r8 = -(-int(slot_ranks[slot]) // 8) * 8
    return r8 if r8 < desc.max_lora_rank else 0


def _check_plan(desc, ids, prefill, bgmv_max_rank=0, slot_ranks=None):
    ids = np.asarray(ids, np.int32)
    R = desc.max_lora_rank
    p, img, v = L.lora_apply_plan(desc, ids, prefill, bgmv_max_rank, slot_ranks=slot_ranks)
    m = L.lora_build_meta(ids, prefill, desc.max_loras, R, bgmv_max_rank)
    ns, nb = m["sgmv_perm"].size, m["bgmv_tok"].size
    assert (p["num_sgmv_rows"], p["num_bgmv_rows"], p["num_segs"]) == (ns, nb, m["seg_ids"].size)
    assert p["image_offset"] % 16 == 0 and p["off_wave"] % 4 == 0
    # token and adapter of every v row, in the builder's order
    row_tok = np.concatenate([m["sgmv_perm"], m["bgmv_tok"]]).astype(np.int64)
    np.testing.assert_array_equal(v["perm"], row_tok)
    row_ids = ids[row_tok] if row_tok.size else np.zeros(0, np.int32)
    seg_len_of_row = np.zeros(ns, np.int64)
    for st, ln in zip(m["seg_starts"], m["seg_lens"]):
        seg_len_of_row[st:st + ln] = ln
    bf16 = desc.dtype == L.LORA_BF16
    thr = MFMA_MIN_ROWS if bf16 else INT32_MAX
    assert p["mfma_min_rows"] == thr
    # BGMV runs take MFMA tiles only in bf16 batches whose long runs hold many rows
    runs = _bgmv_runs(m["bgmv_ids"])
    long_rows = sum(ln for _, ln in runs if ln >= BGMV_MFMA_MIN_ROWS)
    bthr = (BGMV_MFMA_MIN_ROWS if bf16 and long_rows >= bgmv_mfma_min_total(desc.max_lora_rank)
            else INT32_MAX)
    assert p["bgmv_mfma_min_rows"] == bthr
    run_len_of_row = np.zeros(nb, np.int64)
    for st, ln in runs:
        run_len_of_row[st:st + ln] = ln
    # length of the run (segment or BGMV run) each v row belongs to, and whether
    # that run goes to MFMA tiles
    run_len = np.concatenate([seg_len_of_row, run_len_of_row])
    is_mfma = np.concatenate([seg_len_of_row >= thr, run_len_of_row >= bthr])

    shrink_cover = np.zeros(ns + nb, np.int64)
    for rec in v["wave"]:
        slot, rows, first, rank = (int(x) for x in rec[:4])
        assert 1 <= rows <= WAVE_ROWS and 0 <= slot < desc.max_loras
        assert rank == record_rank(desc, slot_ranks, slot)
        assert 0 <= first and first + rows <= ns + nb
        np.testing.assert_array_equal(rec[4:4 + rows], row_tok[first:first + rows])
        assert np.all(rec[4 + rows:] == -1)
        assert np.all(row_ids[first:first + rows] == slot)
        if first < ns:  # SGMV tiles stay inside the SGMV rows
            assert first + rows <= ns
        assert not np.any(is_mfma[first:first + rows])
        shrink_cover[first:first + rows] += 1
    for rec in v["mfma"]:
        slot, rows_rank, first, tok0 = (int(x) for x in rec)
        rows = rows_rank & 0xffff  # rows | rank << 16
        assert rows_rank >> 16 == record_rank(desc, slot_ranks, slot)
        assert bf16 and 1 <= rows <= MFMA_ROWS and first + rows <= ns + nb
        # word 3: first token when the tile's tokens are consecutive, else -1
        toks = v["perm"][first:first + rows]
        consecutive = bool(np.all(toks == toks[0] + np.arange(rows)))
        assert tok0 == (int(toks[0]) if consecutive else -1)
        assert first >= ns or first + rows <= ns  # never across the SGMV / BGMV boundary
        assert np.all(row_ids[first:first + rows] == slot)
        assert np.all(is_mfma[first:first + rows])
        shrink_cover[first:first + rows] += 1
    np.testing.assert_array_equal(shrink_cover, np.ones(ns + nb, np.int64))
    # tile counts: each segment / BGMV run cut into ceil(len / tile rows) pieces
    want_wave = want_mfma = 0
    for ln in m["seg_lens"]:
        if ln >= thr:
            want_mfma += -(-int(ln) // MFMA_ROWS)
        else:
            want_wave += -(-int(ln) // WAVE_ROWS)
    for _, ln in runs:
        if ln >= bthr:
            want_mfma += -(-ln // MFMA_ROWS)
        else:
            want_wave += -(-ln // WAVE_ROWS)
    assert (p["wave_tiles"], p["mfma_tiles"]) == (want_wave, want_mfma)
    assert p["image_bytes"] == 4 * (p["off_mfma"] + 4 * p["mfma_tiles"])
    # K split of the MFMA shrink: of the splits k up to 8 (rank <= 32, else 4)
    # with wgs (k - 1) < 512 and >= 4 steps of 64 per part, the one with the
    # least work on the busiest of 256 compute units, ceil(wgs k / 256) / k,
    # the most parts on a tie
    want_split = 1
    if p["mfma_tiles"]:
        wgs = p["mfma_tiles"] * desc.num_slices * -(-R // 64)
        ksteps = -(-desc.in_features // 64)
        top = MAX_KSPLIT_MFMA if R <= 32 else MAX_KSPLIT_MFMA_WIDE
        best = None
        loads = {}
        for k in range(1, top + 1):
            if k > 1 and (wgs * (k - 1) >= 512 or ksteps // k < 4):
                break
            load = loads[k] = Fraction(-(-wgs * k // 256), k)
            if best is None or load <= best:
                best, want_split = load, k
        # with the DMA-staged shrink (K a multiple of 64 up to 8192), a tie at
        # most two workgroups per compute unit goes to the most parts of the
        # tie at one workgroup per unit (that shrink then runs four stages)
        K = desc.in_features
        lone = [k for k, v in loads.items() if v == best and wgs * k <= 256]
        if K % 64 == 0 and K <= 8192 and lone and wgs * want_split <= 512:
            want_split = max(lone)
    assert p["ksplit"] == want_split
    # K split of the wavefront tiles (bf16, R <= 64): of the splits k <= 8 that
    # keep <= 1024 workgroups and one load batch per part (4 waves x CB chunks
    # of 32; CB = 8, 6, 4 for R <= 16, 32, 64), the one with the least work on
    # the busiest of 256 compute units, ceil(wgs k / 256) / k (fewest parts on
    # a tie)
    want_wave = 1
    if desc.dtype == _lib.LORA_BF16 and p["wave_tiles"] and R <= 64:
        cb = 8 if R <= 16 else 6 if R <= 32 else 4
        nk = -(-desc.in_features // 32)
        wgs = p["wave_tiles"] * desc.num_slices
        best = None
        for k in range(1, MAX_KSPLIT + 1):
            if k > 1 and (wgs * k > 1024 or nk // k < 4 * cb):
                break
            load = Fraction(-(-wgs * k // 256), k)
            if best is None or load < best:
                best, want_wave = load, k
    assert p["ksplit_wave"] == want_wave and p["reserved"] == 0
    assert p["image_bytes"] + p["image_offset"] <= L.lora_apply_host_meta_bytes(desc, ids.size)
    return p


@pytest.mark.parametrize("prefill", [True, False])
def test_plan_tiny(prefill):
    wl = W.config_tiny_fp32(seed=0, prefill=prefill)
    d = L.make_desc(wl.dtype, wl.max_loras, wl.max_lora_rank, wl.in_features, wl.out_features)
    p = _check_plan(d, wl.ids, wl.prefill)
    # three adapters with 8 rows each: three full wavefront tiles either way
    assert p["wave_tiles"] == 3 and p["mfma_tiles"] == 0


def test_plan_named_workloads():
    cases = [W.config_bgmv_decode(seed=0), W.config_sgmv_prefill(seed=0),
             W.config_qkv_decode(seed=0)] + list(W.config_mlp_mixed(seed=0))
    for wl in cases:
        d = L.make_desc(wl.dtype, wl.max_loras, wl.max_lora_rank, wl.in_features,
                        wl.out_features)
        _check_plan(d, wl.ids, wl.prefill)


def test_plan_fuzz():
    rng = np.random.default_rng(7)
    for it in range(300):
        ml = int(rng.integers(1, 70))
        T = int(rng.integers(0, 400))
        if it % 10 == 0:  # large decode batches: long BGMV runs may take MFMA tiles
            ml = int(rng.integers(1, 24))
            T = int(rng.integers(1000, 3000))
        R = int(rng.choice([8, 16, 64, 80]))
        dtype = "bf16" if it % 3 else "f32"
        d = L.make_desc(dtype, ml, R, 64, [64, 32])
        ids = rng.integers(-1, ml, size=T).astype(np.int32)
        if it % 4 == 0:  # long runs of one adapter
            ids = np.sort(ids)
        pre = (rng.random(T) < rng.random()).astype(np.uint8)
        _check_plan(d, ids, pre if it % 5 else None, bgmv_max_rank=int(rng.choice([0, 8, 128])))


def test_plan_ragged_ranks():
    """With slot ranks the plan is the padded plan with each record's rank
    field set: same tiles, rows, tokens and K splits."""
    rng = np.random.default_rng(11)
    for it in range(120):
        ml = int(rng.integers(1, 40))
        R = int(rng.choice([8, 16, 32, 64, 128]))
        T = int(rng.integers(0, 600)) if it % 6 else int(rng.integers(1500, 2600))
        d = L.make_desc("bf16" if it % 4 else "f32", ml, R, 128, [64, 96])
        ids = rng.integers(-1, ml, size=T).astype(np.int32)
        if it % 3 == 0:
            ids = np.sort(ids)
        pre = (rng.random(T) < 0.5).astype(np.uint8) if it % 2 else None
        ranks = rng.integers(0, R + 1, size=ml).astype(np.int32)
        p0, img0, v0 = L.lora_apply_plan(d, ids, pre)
        p1 = _check_plan(d, ids, pre, slot_ranks=ranks)
        _, img1, v1 = L.lora_apply_plan(d, ids, pre, slot_ranks=ranks)
        assert p0 == p1
        np.testing.assert_array_equal(v0["perm"], v1["perm"])
        w0, w1 = v0["wave"].copy(), v1["wave"].copy()
        w0[:, 3] = w1[:, 3] = 0
        np.testing.assert_array_equal(w0, w1)
        np.testing.assert_array_equal(v0["mfma"][:, 1], v1["mfma"][:, 1] & 0xffff)
        np.testing.assert_array_equal(np.delete(v0["mfma"], 1, axis=1),
                                      np.delete(v1["mfma"], 1, axis=1))


def test_plan_ragged_rank_errors():
    d = L.make_desc("bf16", 4, 16, 64, [64])
    ids = np.array([0, 1, 2, 3], np.int32)
    for bad in ([0, 0, 0, 17], [-1, 0, 0, 0]):
        with pytest.raises(L.LoraError) as e:
            L.lora_apply_plan(d, ids, slot_ranks=np.array(bad, np.int32))
        assert e.value.status == _lib.LORA_E_RANK
    with pytest.raises(ValueError):
        L.lora_apply_plan(d, ids, slot_ranks=np.zeros(3, np.int32))
    # a full rank, or a rank that rounds up to the pool's, reads as 0
    _, _, v = L.lora_apply_plan(d, ids, slot_ranks=np.array([16, 9, 8, 1], np.int32))
    assert list(v["wave"][:, 3]) == [0, 0, 8, 8]


@pytest.mark.parametrize("T,n,rank,want_mfma", [(64, 8, 16, False), (512, 4, 16, False),
                                                (1024, 8, 16, False), (2048, 8, 16, True),
                                                (1024, 8, 64, True), (1024, 64, 64, False),
                                                (4096, 64, 16, True)])
def test_plan_bgmv_runs_on_mfma(T, n, rank, want_mfma):
    """Decode batches: sorted runs of one adapter go to MFMA tiles only when
    the batch is large (sooner for a higher pool rank) and its runs are long."""
    wl = W.config_bgmv_decode(seed=1, T=T, K=256, O=256, n_adapters=n, rank=rank, p_none=0.0)
    d = L.make_desc(wl.dtype, wl.max_loras, wl.max_lora_rank, wl.in_features, wl.out_features)
    p = _check_plan(d, wl.ids, wl.prefill)
    assert (p["mfma_tiles"] > 0) == want_mfma
    assert (p["bgmv_mfma_min_rows"] != INT32_MAX) == want_mfma
    # an fp32 pool never uses MFMA tiles
    d32 = L.make_desc("f32", wl.max_loras, wl.max_lora_rank, wl.in_features, wl.out_features)
    p32 = _check_plan(d32, wl.ids, wl.prefill)
    assert p32["mfma_tiles"] == 0


def test_plan_errors():
    d = L.make_desc("bf16", 4, 16, 64, [64])
    with pytest.raises(L.LoraError) as e:
        L.lora_apply_plan(d, np.array([0, 4], np.int32))
    assert e.value.status == -6
    p, _, _ = L.lora_apply_plan(d, np.zeros(0, np.int32))
    assert p["wave_tiles"] == p["mfma_tiles"] == 0 and p["image_bytes"] == 0


def test_plan_entry_validation_before_hip():
    """Malformed plans are rejected on the host, before any GPU call."""
    import lora_adapter_pool_amd._lib as _lib
    FAKE = 1 << 20
    d = L.make_desc("bf16", 4, 16, 64, [64])
    ids = np.array([0, 0, 1, 3, -1, 2], np.int32)
    p, _, _ = L.lora_apply_plan(d, ids, np.ones(6, np.uint8))

    def status(fn, plan, image=FAKE, T=6, desc=d):
        try:
            fn(desc, FAKE, FAKE, FAKE, T, plan, image, None, 0)
            return 0
        except L.LoraError as e:
            return e.status

    for fn in (L.lora_plan_shrink, L.lora_plan_expand):
        for key, val in (("wave_tiles", -1), ("off_wave", -4), ("num_bgmv_rows", -2), ("ksplit", 0),
                         ("ksplit", MAX_KSPLIT_MFMA + 1), ("ksplit_wave", 0),
                         ("ksplit_wave", MAX_KSPLIT + 1)):
            assert status(fn, dict(p, **{key: val})) == _lib.LORA_E_ARG
        assert status(fn, dict(p, image_bytes=p["image_bytes"] - 4)) == _lib.LORA_E_ARG
        assert status(fn, p, image=FAKE + 4) == _lib.LORA_E_ALIGN
        assert status(fn, dict(p, off_wave=p["off_wave"] + 1)) == _lib.LORA_E_ALIGN
        assert status(fn, p, image=0) == _lib.LORA_E_ARG
        assert status(fn, p, T=0) == 0  # no rows: no-op, nothing launched
        empty = dict(p, wave_tiles=0, mfma_tiles=0)
        assert status(fn, empty) == 0
    # more than four partials of the MFMA shrink only for pools of rank <= 32
    d64 = L.make_desc("bf16", 4, 64, 64, [64])
    p64, _, _ = L.lora_apply_plan(d64, ids, np.ones(6, np.uint8))
    for fn in (L.lora_plan_shrink, L.lora_plan_expand):
        assert status(fn, dict(p64, ksplit=MAX_KSPLIT_MFMA_WIDE + 1), desc=d64) == _lib.LORA_E_ARG
    # MFMA tiles need a bf16 pool
    d32 = L.make_desc("f32", 4, 16, 64, [64])
    pm, _, _ = L.lora_apply_plan(d, np.zeros(40, np.int32), np.ones(40, np.uint8))
    assert pm["mfma_tiles"] > 0
    assert status(L.lora_plan_shrink, pm, desc=d32, T=40) == _lib.LORA_E_DTYPE


def _device_plan_counts(ids, prefill, max_loras, R, mfma_min, bgmv_min, bgmv_total,
                        bgmv_max_rank=64):
    """Records a device-built plan writes (lora_apply_device's rules): per slot,
    SGMV rows on 64-row tiles when there are at least mfma_min of them, BGMV
    rows when there are at least bgmv_min of them and such runs hold at least
    bgmv_total rows of the batch; the rest on 8-row tiles."""
    m = L.lora_build_meta(ids, prefill, max_loras, R, bgmv_max_rank)
    sc = np.zeros(max_loras, np.int64)
    for a, ln in zip(m["seg_ids"], m["seg_lens"]):
        sc[a] += ln
    bc = np.bincount(m["bgmv_ids"], minlength=max_loras) if m["bgmv_ids"].size else \
        np.zeros(max_loras, np.int64)
    ms = sc >= mfma_min
    mb = (bc >= bgmv_min) & (bc[bc >= bgmv_min].sum() >= bgmv_total)
    wave = int(np.sum(np.where(ms, 0, -(-sc // 8)) + np.where(mb, 0, -(-bc // 8))))
    mfma = int(np.sum(np.where(ms, -(-sc // 64), 0) + np.where(mb, -(-bc // 64), 0)))
    return wave, mfma


def _mfma_cap(T, ml, sgmv, mfma_min, bmin, btot):
    """The device plan's 64-row record capacity as documented: ceil(T/64) plus
    the runs that can take MFMA tiles (at most min(ml, T // mfma_min) SGMV
    runs when the batch can hold SGMV rows; in batches of at least btot rows,
    at most min(ml, T // bmin) BGMV runs), and never more than the per-slot
    bound ceil(T/64) + 2 min(ml, T)."""
    runs = (min(ml, T // mfma_min) if sgmv else 0) + (min(ml, T // bmin) if T >= btot else 0)
    if runs == 0:
        return 0
    return min(-(-T // 64) + 2 * min(ml, T), -(-T // 64) + runs)


def test_device_plan_capacity_bounds():
    """The device plan's record capacities, ceil(T/8) + 2 min(max_loras, T)
    8-row records and the 64-row capacity above, cover every batch: random
    mixes, one row per slot in each set, long runs, and batches built to reach
    the 64-row bound (every slot with exactly the SGMV threshold's rows, BGMV
    runs of exactly the run threshold in batches at the total threshold)."""
    rng = np.random.default_rng(3)
    cases = []
    for _ in range(300):
        ml = int(rng.integers(1, 80))
        T = int(rng.integers(1, 700))
        ids = rng.integers(-1, ml, size=T).astype(np.int32)
        if rng.random() < 0.3:
            ids = np.sort(ids)
        cases.append((ml, ids, (rng.random(T) < rng.random()).astype(np.uint8)))
    for ml in (1, 7, 64):  # every slot with one SGMV row and one BGMV row
        ids = np.repeat(np.arange(ml, dtype=np.int32), 2)
        cases.append((ml, ids, np.tile(np.array([1, 0], np.uint8), ml)))
    for ml in (3, 40, 130):  # every slot at the SGMV threshold, then BGMV runs of 48
        sg = np.repeat(np.arange(ml, dtype=np.int32), 16)
        bg = np.repeat(np.arange(ml, dtype=np.int32), 48)
        extra = np.zeros(max(0, 2048 - sg.size - bg.size), np.int32)  # reach the total threshold
        ids = np.concatenate([sg, bg, extra])
        pre = np.concatenate([np.ones(sg.size, np.uint8), np.zeros(bg.size + extra.size, np.uint8)])
        cases.append((ml, ids, pre))
        cases.append((ml, np.concatenate([bg, extra]), np.zeros(bg.size + extra.size, np.uint8)))
    for ml, ids, pre in cases:
        T = ids.size
        for mfma_min, bmin, btot in ((16, 48, 1024), (16, 48, 2048), (1, 1, 0),
                                     (2 ** 31 - 1,) * 3):
            wave, mfma = _device_plan_counts(ids, pre, ml, 16, mfma_min, bmin, btot)
            assert wave <= -(-T // 8) + 2 * min(ml, T)
            assert mfma <= _mfma_cap(T, ml, True, mfma_min, bmin, btot), (ml, T, mfma_min)
            if not pre.any():  # no SGMV row: the bound without flags holds too
                assert mfma <= _mfma_cap(T, ml, False, mfma_min, bmin, btot), (ml, T, mfma_min)
