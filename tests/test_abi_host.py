"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, the host metadata builder is bit-exact against the oracle's,
and every validation error is returned before any HIP call."""
import ctypes
import math

import numpy as np
import pytest

import lora_adapter_pool_amd as L
from lora_adapter_pool_amd import _lib
import oracle
from oracle_pins import META_KEYS, _load, check_meta_properties


@pytest.fixture(scope="module")
def lib():
    return L.lib()


def test_library_exports_every_header_function(lib):
    names = _lib.header_functions()
    assert len(names) >= 16
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib._SIGNATURES), "binding and header disagree"
    assert lib.lora_abi_version() == 3


def test_pool_geometry_and_bytes():
    d = L.make_desc("bf16", 64, 16, 4096, [4096, 1024, 1024])
    assert L.lora_pool_bytes_A(d) == 64 * 3 * 16 * 4096 * 2
    assert L.lora_pool_bytes_B(d) == 64 * 16 * 6144 * 2
    a, b = oracle.pool_bytes(64, 3, 16, 4096, 6144, 2)
    assert (a, b) == (L.lora_pool_bytes_A(d), L.lora_pool_bytes_B(d))
    d = L.make_desc("f32", 4, 8, 256, [256])
    assert L.lora_pool_bytes_A(d) == 4 * 8 * 256 * 4


@pytest.mark.parametrize("r,alpha,rs", [(8, 16.0, 0), (16, 32.0, 0), (16, 16.0, 1), (64, 128.0, 0),
                                        (4, 8.0, 1), (3, 1.0, 0), (7, 5.0, 1), (2, 4.0, 1)])
def test_scaling_matches_oracle(r, alpha, rs):
    got = L.lora_scaling(r, alpha, rs)
    assert got == np.float32(oracle.scaling(r, alpha, bool(rs)))
    assert math.isnan(L.lora_scaling(0, 1.0, 0))


def test_builder_golden_cases():
    for case in _load("builder_tiny.json")["cases"]:
        m = L.lora_build_meta(case["ids"], case["prefill"], 8, case["max_lora_rank"], 64)
        for k in META_KEYS:
            assert m[k].tolist() == case[k], (case["name"], k)


def test_builder_bit_exact_vs_oracle_fuzz():
    rng = np.random.default_rng(7)
    for trial in range(200):
        T = int(rng.integers(0, 700))
        n = int(rng.integers(1, 70))
        ids = rng.integers(-1, n, size=T).astype(np.int32)
        if trial % 4 == 0:
            ids = np.sort(ids)
        pre = rng.integers(0, 2, size=T).astype(np.uint8)
        if trial % 5 == 0:
            pre[:] = 1
        R = int(rng.choice([8, 16, 32, 64, 72, 128]))
        lim = int(rng.choice([0, 16, 64, 100]))
        got = L.lora_build_meta(ids, pre, n, R, lim)
        ref = oracle.build_meta(ids.tolist(), pre.tolist(), R, lim if lim > 0 else 64)
        for k in META_KEYS:
            assert got[k].tolist() == list(ref[k]), (trial, k)
        check_meta_properties(ids, pre, R, got, lim if lim > 0 else 64)


def test_builder_long_runs_vs_oracle_fuzz():
    """Long runs of one adapter and one prefill flag (the builder scans them 16
    rows at a time), flags other than 0 / 1, and flips inside runs at every
    offset of a 16-row block."""
    rng = np.random.default_rng(8)
    for trial in range(150):
        n = int(rng.integers(1, 20))
        lens = rng.integers(1, 90, size=int(rng.integers(1, 12)))
        ids = np.concatenate([np.full(ln, rng.integers(-1, n), np.int32) for ln in lens])
        flags = rng.choice(np.array([0, 1, 7, 255], np.uint8), size=len(lens))
        pre = np.concatenate([np.full(ln, f, np.uint8) for ln, f in zip(lens, flags)])
        for _ in range(int(rng.integers(0, 3))):
            if ids.size:
                pre[int(rng.integers(0, ids.size))] ^= np.uint8(rng.choice([1, 128]))
        R = int(rng.choice([16, 64, 128]))
        got = L.lora_build_meta(ids, pre, n, R, 0)
        ref = oracle.build_meta(ids.tolist(), [int(v != 0) for v in pre], R, 64)
        for k in META_KEYS:
            assert got[k].tolist() == list(ref[k]), (trial, k)
        check_meta_properties(ids, (pre != 0).astype(np.uint8), R, got, 64)


def test_builder_walk_choice_vs_oracle():
    """The builder walks a batch by runs or row by row depending on its first
    512 rows; batches whose head misleads that choice (a sorted head over a
    mixed tail, a mixed head over long runs, runs crossing the 512-row mark)
    still sort exactly as the oracle's builder does."""
    rng = np.random.default_rng(9)
    for trial in range(60):
        n = int(rng.integers(1, 40))
        head = int(rng.integers(400, 700))
        tail = int(rng.integers(0, 3000))
        sorted_ids = np.sort(rng.integers(-1, n, size=head)).astype(np.int32)
        mixed_ids = rng.integers(-1, n, size=tail).astype(np.int32)
        if trial % 2:
            ids = np.concatenate([mixed_ids[: head], np.sort(rng.integers(-1, n, size=tail))])
        else:
            ids = np.concatenate([sorted_ids, mixed_ids])
        ids = ids.astype(np.int32)
        pre = (rng.random(ids.size) < (0.5 if trial % 3 else 0.0)).astype(np.uint8)
        if trial % 3 == 1:  # flags in runs too
            pre = np.repeat(rng.integers(0, 2, size=-(-ids.size // 64)), 64)[: ids.size].astype(np.uint8)
        R = int(rng.choice([16, 64, 128]))
        got = L.lora_build_meta(ids, pre, n, R, 0)
        ref = oracle.build_meta(ids.tolist(), pre.tolist(), R, 64)
        for k in META_KEYS:
            assert got[k].tolist() == list(ref[k]), (trial, k)
        check_meta_properties(ids, pre, R, got, 64)


def test_device_builder_validates_before_hip():
    """lora_build_meta_device rejects bad arguments before any HIP call."""
    import ctypes
    lib = _lib.lib()
    FAKE = 1 << 20
    good = {k: FAKE for k in ("sgmv_perm", "seg_starts", "seg_lens", "seg_ids", "bgmv_tok",
                              "bgmv_ids")}

    def status(T=8, max_loras=4, ids=FAKE, counts=FAKE, drop=None, out=True):
        m = _lib.lora_meta()
        for k, p in good.items():
            setattr(m, k, ctypes.cast(None if k == drop else p, ctypes.POINTER(ctypes.c_int32)))
        return lib.lora_build_meta_device(ids, None, T, max_loras, 16, 0,
                                          ctypes.byref(m) if out else None, counts, None)

    assert status(out=False) == _lib.LORA_E_ARG
    assert status(counts=None) == _lib.LORA_E_ARG
    assert status(T=-1) == _lib.LORA_E_ARG
    assert status(max_loras=0) == _lib.LORA_E_SHAPE
    assert status(max_loras=_lib.META_DEVICE_MAX_LORAS + 1) == _lib.LORA_E_SHAPE
    assert status(drop="seg_lens") == _lib.LORA_E_ARG
    assert status(drop="bgmv_ids") == _lib.LORA_E_ARG
    assert status(ids=None) == _lib.LORA_E_ARG


def test_builder_named_workload_shapes():
    import workloads as W
    wl = W.config_sgmv_prefill(seed=0, K=64, O=64)
    m = L.lora_build_meta(wl.ids, wl.prefill, wl.max_loras, wl.max_lora_rank)
    assert m["sgmv_perm"].tolist() == list(range(wl.T))   # laid out by adapter already
    assert m["seg_ids"].tolist() == list(range(16)) and m["bgmv_tok"].size == 0
    gu, _ = W.config_mlp_mixed(seed=0, hidden=64, inter=64)
    m = L.lora_build_meta(gu.ids, gu.prefill, gu.max_loras, gu.max_lora_rank)
    ref = oracle.build_meta(gu.ids.tolist(), gu.prefill.tolist(), gu.max_lora_rank)
    for k in META_KEYS:
        assert m[k].tolist() == list(ref[k])
    assert m["bgmv_tok"].size == int(((gu.ids >= 0) & (gu.prefill == 0)).sum())


def test_builder_null_prefill_means_decode():
    m = L.lora_build_meta([1, 0, 1], None, 2, 16)
    assert m["bgmv_tok"].tolist() == [1, 0, 2] and m["sgmv_perm"].size == 0


def test_builder_rejects_bad_ids():
    with pytest.raises(L.LoraError) as e:
        L.lora_build_meta([0, 5], [0, 0], 4, 16)
    assert e.value.status == _lib.LORA_E_ID and "ids[1]" in str(e.value)
    with pytest.raises(L.LoraError) as e:
        L.lora_build_meta([-2], [0], 4, 16)
    assert e.value.status == _lib.LORA_E_ID


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=7), _lib.LORA_E_DTYPE),
    (dict(max_loras=0), _lib.LORA_E_SHAPE),
    (dict(max_lora_rank=12), _lib.LORA_E_ALIGN),
    (dict(max_lora_rank=0), _lib.LORA_E_RANK),
    (dict(in_features=100), _lib.LORA_E_ALIGN),
    (dict(in_features=0), _lib.LORA_E_SHAPE),
    (dict(num_slices=0), _lib.LORA_E_SHAPE),
    (dict(num_slices=9), _lib.LORA_E_SHAPE),
    (dict(out0=20), _lib.LORA_E_ALIGN),
])
def test_descriptor_validation(kw, status):
    d = L.make_desc("bf16", 4, 16, 256, [256])
    for k, v in kw.items():
        if k == "out0":
            d.out_features[0] = v
        else:
            setattr(d, k, v)
    with pytest.raises(L.LoraError) as e:
        L.lora_pool_validate(d)
    assert e.value.status == status


FAKE = 1 << 20  # non-null, 16-byte aligned; never dereferenced (validation fails first)


def _status(fn, *a):
    try:
        fn(*a)
        return 0
    except L.LoraError as e:
        return e.status


def test_pool_load_errors_before_hip():
    d = L.make_desc("bf16", 4, 16, 256, [256])
    args = lambda **k: [d, k.get("A", FAKE), k.get("B", FAKE), k.get("slot", 0),
                        k.get("sl", 0), FAKE, FAKE, k.get("r", 8), 16.0, False]
    assert _status(L.lora_pool_load, *args(r=17), True, 0) == _lib.LORA_E_RANK
    assert _status(L.lora_pool_load, *args(r=0), True, 0) == _lib.LORA_E_RANK
    assert _status(L.lora_pool_load, *args(slot=4), True, 0) == _lib.LORA_E_ID
    assert _status(L.lora_pool_load, *args(slot=-1), True, 0) == _lib.LORA_E_ID
    assert _status(L.lora_pool_load, *args(sl=1), True, 0) == _lib.LORA_E_ID
    assert _status(L.lora_pool_load, *args(A=FAKE + 8), True, 0) == _lib.LORA_E_ALIGN
    assert _status(L.lora_pool_load, *args(A=0), True, 0) == _lib.LORA_E_ARG
    assert _status(L.lora_pool_clear, d, FAKE, FAKE, 9, 0) == _lib.LORA_E_ID


def test_kernel_entry_points_validate_before_hip():
    d = L.make_desc("bf16", 4, 16, 256, [256])
    # zero rows: a no-op that touches nothing
    assert _status(L.lora_bgmv_shrink, d, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 5, 0) == 0
    assert _status(L.lora_sgmv_expand, d, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 0, 5, 0) == 0
    assert _status(L.lora_bgmv_shrink, d, FAKE, FAKE, FAKE, FAKE, FAKE, -1, 5, 0) == _lib.LORA_E_ARG
    assert _status(L.lora_bgmv_expand, d, FAKE, FAKE, FAKE + 4, FAKE, FAKE, 3, 5, 0) == _lib.LORA_E_ALIGN
    assert _status(L.lora_bgmv_expand, d, FAKE, FAKE, FAKE, 0, FAKE, 3, 5, 0) == _lib.LORA_E_ARG
    assert _status(L.lora_sgmv_shrink, d, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, -2, 4, 5,
                   0) == _lib.LORA_E_ARG
    assert _status(L.lora_sgmv_shrink, d, FAKE, FAKE, FAKE, 0, FAKE, FAKE, FAKE, 1, 4, 5,
                   0) == _lib.LORA_E_ARG
    bad = L.make_desc("bf16", 4, 20, 256, [256])
    assert _status(L.lora_bgmv_shrink, bad, FAKE, FAKE, FAKE, FAKE, FAKE, 3, 5, 0) == _lib.LORA_E_ALIGN


def _aligned_i32(n):
    raw = np.zeros(n + 16, np.int32)
    off = (-raw.ctypes.data % 64) // 4
    return raw[off:off + n]


def test_apply_validation_before_hip():
    d = L.make_desc("bf16", 4, 16, 256, [256])
    T = 6
    ws_need = L.lora_apply_workspace_bytes(d, T)
    mh_need = L.lora_apply_host_meta_bytes(d, T)
    # staging: builder arrays (3T + 3 max_loras words, padded to 4), then the
    # plan image: perm (T, padded to 4), <= ceil(T/8) + 2 max_loras wave tiles
    # of 16 words, <= ceil(T/64) + 2 max_loras MFMA tiles of 4 words (each
    # segment and each BGMV run adds at most one partial tile)
    up4 = lambda n: (n + 3) // 4 * 4  # noqa: E731
    image = up4(T) + 16 * (-(-T // 8) + 2 * 4) + 4 * (-(-T // 64) + 2 * 4)
    assert mh_need == 4 * (up4(3 * T + 3 * 4) + image)
    # workspace: the plan image (padded to 256 bytes), then v (up to 8 K-split
    # partials of T rows x S x R fp32)
    assert ws_need == ((4 * image + 255) // 256) * 256 + 8 * T * 16 * 4
    ids = np.array([0, 1, -1, 3, 2, 0], np.int32)
    meta = _aligned_i32(mh_need // 4)
    ok = [d, FAKE, FAKE, FAKE, FAKE + 64, T, ids, None, 0, FAKE, ws_need, meta, mh_need, 0]

    def with_(i, v):
        a = list(ok)
        a[i] = v
        return a
    assert _status(L.lora_apply, *with_(9, FAKE)[:10], ws_need - 1, meta, mh_need, 0) == _lib.LORA_E_WORKSPACE
    assert _status(L.lora_apply, *ok[:12], mh_need - 4, 0) == _lib.LORA_E_WORKSPACE
    bad_ids = ids.copy()
    bad_ids[3] = 4
    assert _status(L.lora_apply, *with_(6, bad_ids)) == _lib.LORA_E_ID
    assert _status(L.lora_apply, *with_(3, FAKE + 2)) == _lib.LORA_E_ALIGN
    assert _status(L.lora_apply, *with_(5, -1)) == _lib.LORA_E_ARG
    assert _status(L.lora_apply, *with_(5, 0)) == 0          # T = 0: no-op
    assert _status(L.lora_apply, *with_(6, None)) == _lib.LORA_E_ARG
    # last_error carries a message for the most recent failure
    _status(L.lora_apply, *with_(6, bad_ids))
    assert "ids[3]" in L.last_error()


def test_apply_ranked_validation_before_hip():
    """lora_apply_ranked checks slot_ranks (and everything lora_apply checks)
    on the host before any GPU call."""
    d = L.make_desc("bf16", 4, 16, 256, [256])
    T = 6
    ws_need = L.lora_apply_workspace_bytes(d, T)
    mh_need = L.lora_apply_host_meta_bytes(d, T)
    ids = np.array([0, 1, -1, 3, 2, 0], np.int32)
    meta = _aligned_i32(mh_need // 4)
    ranks = np.array([8, 16, 0, 4], np.int32)
    ok = [d, FAKE, FAKE, FAKE, FAKE + 64, T, ids, None, 0, ranks, FAKE, ws_need, meta, mh_need, 0]

    def with_(i, v):
        a = list(ok)
        a[i] = v
        return a
    for bad in ([8, 16, 17, 4], [8, -2, 0, 4]):
        assert _status(L.lora_apply_ranked, *with_(9, np.array(bad, np.int32))) == _lib.LORA_E_RANK
    assert "slot_ranks" in L.last_error()
    bad_ids = ids.copy()
    bad_ids[3] = 4
    assert _status(L.lora_apply_ranked, *with_(6, bad_ids)) == _lib.LORA_E_ID
    assert _status(L.lora_apply_ranked, *with_(11, ws_need - 1)) == _lib.LORA_E_WORKSPACE
    assert _status(L.lora_apply_ranked, *with_(5, 0)) == 0  # T = 0: no-op


def test_pycall_binding_matches_ctypes_before_hip():
    """The CPython binding (_lora_call) of lora_apply, lora_apply_ranked and
    lora_apply_device hands the same arguments to the same entry points as
    ctypes: equal statuses and messages on every host-checked error; its own
    argument errors raise before any call."""
    lib = L.lib()
    pc = _lib.pycall()
    d = L.make_desc("bf16", 4, 16, 256, [256])
    da = ctypes.addressof(d)
    T = 6
    ws_need = L.lora_apply_workspace_bytes(d, T)
    mh_need = L.lora_apply_host_meta_bytes(d, T)
    dws = L.lora_apply_device_workspace_bytes(d, T)
    ids = np.array([0, 1, -1, 3, 2, 0], np.int32)
    bad_ids = ids.copy()
    bad_ids[3] = 4
    ranks = np.array([8, 16, 0, 4], np.int32)
    bad_ranks = np.array([8, 16, 17, 4], np.int32)
    meta = _aligned_i32(mh_need // 4)
    P = lambda a: None if a is None else a.ctypes.data  # noqa: E731
    # (T, ids, ranks, ws_bytes, meta_bytes, x): each fails on the host, before
    # any GPU call, in every entry point it is passed to (the pointers are
    # fake); the last one only in lora_apply_ranked
    cases = [(-1, ids, ranks, ws_need, mh_need, FAKE), (T, bad_ids, ranks, ws_need, mh_need, FAKE),
             (T, ids, ranks, ws_need - 1, mh_need, FAKE), (T, ids, ranks, ws_need, mh_need - 4, FAKE),
             (T, ids, ranks, ws_need, mh_need, FAKE + 2), (T, None, ranks, ws_need, mh_need, FAKE),
             (T, ids, bad_ranks, ws_need, mh_need, FAKE)]
    for k, (t, i, r, wb, mb, x) in enumerate(cases):
        args = (FAKE, FAKE, x, FAKE + 64, t, P(i), None, 0)
        tail = (FAKE, wb, P(meta), mb, 0)
        if k < len(cases) - 1:
            want = lib.lora_apply(ctypes.byref(d), *args, *tail)
            msg = L.last_error()
            assert pc.apply(_lib.entry_address("lora_apply"), da, *args, *tail) == want < 0
            assert L.last_error() == msg
        want = lib.lora_apply_ranked(ctypes.byref(d), *args, P(r), *tail)
        msg = L.last_error()
        assert pc.apply_ranked(_lib.entry_address("lora_apply_ranked"), da, *args, P(r),
                               *tail) == want < 0
        assert L.last_error() == msg
        # (the device path reads ids on the GPU: a workspace one byte short
        # keeps every case on the host)
        dargs = (FAKE, FAKE, x, FAKE + 64, t, P(i), None, 0, FAKE, dws - 1)
        want = lib.lora_apply_device(ctypes.byref(d), *dargs, 0)
        msg = L.last_error()
        got = pc.apply_device(_lib.entry_address("lora_apply_device"), da, *dargs, 0)
        assert got == want < 0 and L.last_error() == msg
    # T = 0 is a no-op through both
    assert pc.apply(_lib.entry_address("lora_apply"), da, FAKE, FAKE, FAKE, FAKE + 64, 0, None,
                    None, 0, FAKE, ws_need, P(meta), mh_need, 0) == 0
    # a NULL descriptor (None or 0) reaches the entry point as NULL
    assert pc.apply(_lib.entry_address("lora_apply"), None, FAKE, FAKE, FAKE, FAKE, T, P(ids),
                    None, 0, FAKE, ws_need, P(meta), mh_need, 0) == _lib.LORA_E_ARG
    assert "NULL" in L.last_error()
    # the binding's own checks: argument count, int32 range, entry address
    with pytest.raises(TypeError):
        pc.apply(_lib.entry_address("lora_apply"), da, FAKE)
    with pytest.raises(OverflowError):
        pc.apply(_lib.entry_address("lora_apply"), da, FAKE, FAKE, FAKE, FAKE, 1 << 31, P(ids),
                 None, 0, FAKE, ws_need, P(meta), mh_need, 0)
    with pytest.raises(ValueError):
        pc.apply(0, da, FAKE, FAKE, FAKE, FAKE, T, P(ids), None, 0, FAKE, ws_need, P(meta),
                 mh_need, 0)


def test_merge_validation_before_hip():
    """lora_merge_weights rejects bad slots, slices, ranks, alignment and
    overlapping buffers on the host, before any GPU call."""
    d = L.make_desc("bf16", 4, 16, 64, [64, 32])
    nbytes = 64 * 64 * 2

    def st(*a):
        try:
            L.lora_merge_weights(*a, stream=0)
            return 0
        except L.LoraError as e:
            return e.status
    assert st(d, FAKE, FAKE, 4, 0, FAKE, FAKE + nbytes) == _lib.LORA_E_ID
    assert st(d, FAKE, FAKE, -1, 0, FAKE, FAKE + nbytes) == _lib.LORA_E_ID
    assert st(d, FAKE, FAKE, 0, 2, FAKE, FAKE + nbytes) == _lib.LORA_E_ID
    assert st(d, FAKE, FAKE, 0, 0, FAKE + 2, FAKE + nbytes) == _lib.LORA_E_ALIGN
    assert st(d, FAKE, FAKE, 0, 0, FAKE, FAKE + 1024) == _lib.LORA_E_ARG   # partial overlap
    assert st(d, None, FAKE, 0, 0, FAKE, FAKE) == _lib.LORA_E_ARG
    big = L.make_desc("bf16", 2, 520, 64, [64])
    assert st(big, FAKE, FAKE, 0, 0, FAKE, FAKE) == _lib.LORA_E_RANK
    assert "max_lora_rank" in L.last_error()


def _device_ws_bytes(T, ML, R, S):
    """lora_apply_device's workspace, written out from its documented layout:
    count words, metadata, v-row map, 8-row records (one partial tile per slot
    and row set), 64-row records (pieces of the runs that take MFMA tiles: SGMV
    runs of >= 16 rows, and BGMV runs of >= 48 rows in batches of >= 2048 rows
    for R <= 16, >= 1024 rows above), then 8 partials of v."""
    up = lambda n, a: (n + a - 1) // a * a  # noqa: E731
    meta = up(16, 256)
    meta = up(meta + 4 * T, 16)
    meta = up(meta + 4 * T, 16)
    meta = up(meta + 4 * T, 16)
    meta = up(meta + 4 * ML, 16)
    meta = up(meta + 4 * ML, 16)
    meta = up(meta + 4 * ML, 16)
    perm = up(meta + 4 * T, 256)                 # v row -> token
    cap = -(-T // 8) + 2 * min(ML, T)
    tiles = up(perm + cap * 16 * 4, 256)         # 8-row records
    runs = min(ML, T // 16) + (min(ML, T // 48) if T >= (2048 if R <= 16 else 1024) else 0)
    mcap = min(-(-T // 64) + 2 * min(ML, T), -(-T // 64) + runs)
    mtiles = up(tiles + mcap * 4 * 4, 256)       # 64-row records
    return mtiles + 8 * T * S * R * 4            # v: up to 8 partials of T x S x R fp32


def test_device_workspace_bytes():
    """The device workspace follows its documented layout, including the MFMA
    record capacity at sizes where its two bounds differ."""
    for ML, R, outs, T in ((6, 16, [256, 128], 100), (64, 16, [512], 256), (64, 16, [512], 5000),
                           (4, 64, [256], 3000), (300, 32, [256, 256, 64], 700)):
        d = L.make_desc("bf16", ML, R, 256, outs)
        assert L.lora_apply_device_workspace_bytes(d, T) == _device_ws_bytes(T, ML, R, len(outs)), \
            (ML, R, T)


def test_apply_device_validation_before_hip():
    """lora_apply_device: workspace size and every argument check on the host,
    before any GPU call."""
    d = L.make_desc("bf16", 6, 16, 256, [256, 128])
    T = 100
    need = L.lora_apply_device_workspace_bytes(d, T)
    assert need == _device_ws_bytes(T, 6, 16, 2)
    ok = [d, FAKE, FAKE, FAKE, FAKE + 4096, T, FAKE, None, 0, FAKE, need]

    def with_(i, v):
        a = list(ok)
        a[i] = v
        return a

    def st(*a):
        try:
            L.lora_apply_device(*a, stream=0)
            return 0
        except L.LoraError as e:
            return e.status
    assert st(*with_(10, need - 1)) == _lib.LORA_E_WORKSPACE
    assert st(*with_(9, FAKE + 16)) == _lib.LORA_E_ALIGN      # ws must be 256-byte aligned
    assert st(*with_(3, FAKE + 2)) == _lib.LORA_E_ALIGN
    assert st(*with_(6, None)) == _lib.LORA_E_ARG
    assert st(*with_(5, -1)) == _lib.LORA_E_ARG
    assert st(*with_(5, 0)) == 0                               # T = 0: no-op
    big = L.make_desc("bf16", 8193, 16, 256, [256])
    assert st(*([big] + ok[1:])) == _lib.LORA_E_SHAPE
    with pytest.raises(L.LoraError):
        L.lora_apply_device_workspace_bytes(big, 10)

    # the ranked form runs the same checks (its rank table is device memory)
    def st_r(*a):
        try:
            L.lora_apply_device_ranked(*a[:9], FAKE, *a[9:], stream=0)
            return 0
        except L.LoraError as e:
            return e.status
    assert st_r(*with_(10, need - 1)) == _lib.LORA_E_WORKSPACE
    assert st_r(*with_(6, None)) == _lib.LORA_E_ARG
    assert st_r(*with_(5, 0)) == 0


def test_apply_device_noalloc_validation_before_hip():
    """lora_apply_device_noalloc: a batch whose workspace exceeds the library's
    scratch is rejected, and every argument is checked, before any GPU call."""
    d = L.make_desc("bf16", 32, 64, 4096, [14336, 14336])      # S * R = 128
    ok = [d, FAKE, FAKE, FAKE, FAKE + 4096, 100, FAKE, None, 0]

    def st(*a):
        try:
            L.lora_apply_device_noalloc(*a, stream=0)
            return 0
        except L.LoraError as e:
            return e.status
    # the largest T that fits the scratch, found from the documented size
    lo, hi = 1, 1 << 20
    while lo < hi:
        mid = (lo + hi + 1) // 2
        if L.lora_apply_device_workspace_bytes(d, mid) <= L.NOALLOC_SCRATCH_BYTES:
            lo = mid
        else:
            hi = mid - 1
    assert 15000 < lo < 17000                     # about 16 000 rows at S * R = 128
    big = list(ok)
    big[5] = lo + 1
    assert st(*big) == _lib.LORA_E_WORKSPACE
    assert "scratch" in L.last_error()
    for i, v in ((6, None), (1, None), (3, FAKE + 2), (5, -1)):
        a = list(ok)
        a[i] = v
        assert st(*a) in (_lib.LORA_E_ARG, _lib.LORA_E_ALIGN)
    a = list(ok)
    a[5] = 0
    assert st(*a) == 0                           # T = 0: no-op
    big_pool = L.make_desc("bf16", 8193, 16, 256, [256])
    assert st(*([big_pool] + ok[1:])) == _lib.LORA_E_SHAPE
