"""Plant plausible mistakes in the oracle (on the CPU, by patching it) and
check that at least one pin catches each of them."""
import math

import numpy as np
import pytest

import oracle.lora_oracle as O
from oracle_pins import ALL_PINS


def _caught(monkeypatch_ctx):
    failures = 0
    for pin in ALL_PINS:
        try:
            pin(O)
        except Exception:
            failures += 1
    return failures


def _orig(name):
    return getattr(O, name)


def mut_scale_padded_rank(wl_rank, alpha, rs):
    # uses a fixed padded rank instead of the adapter's own rank
    return alpha / (math.sqrt(64) if rs else 64)


def mut_scale_no_sqrt(rank, alpha, rs):
    return alpha / rank


def mut_scale_inverted(rank, alpha, rs):
    return (math.sqrt(rank) if rs else rank) / alpha


def _forward_factory(kind):
    base = O.lora_forward_rows

    def fwd(wl, rows=None, y_in=None):
        if rows is None:
            rows = range(wl.T)
        rows = list(rows)
        src = wl.y_in if y_in is None else y_in
        out = base(wl, rows, y_in=y_in)
        d = out - np.asarray(src, np.float64)[rows]
        if kind == "sign":
            return np.asarray(src, np.float64)[rows] - d
        if kind == "drop_delta_for_last_slice":
            off = sum(wl.out_features[:-1])
            out[:, off:] = np.asarray(src, np.float64)[rows][:, off:]
            return out
        if kind == "off_by_one_id":
            wl2 = type(wl)(**{**wl.__dict__, "ids": np.where(wl.ids >= 0,
                            (wl.ids + 1) % max(1, len(wl.slots)), wl.ids).astype(np.int32)})
            return base(wl2, rows, y_in=y_in)
        if kind == "none_rows_zeroed":
            out[np.asarray(wl.ids)[rows] < 0] = 0.0
            return out
        raise AssertionError(kind)
    return fwd


def _meta_factory(kind):
    base = O.build_meta

    def bm(ids, prefill, R, bgmv_max_rank=64):
        m = base(ids, prefill, R, bgmv_max_rank)
        if kind == "unstable":
            m["sgmv_perm"] = list(reversed(m["sgmv_perm"]))
        elif kind == "rank_rule_ignored":
            m = base(ids, prefill, 0, bgmv_max_rank)
        elif kind == "prefill_ignored":
            m = base(ids, [0] * len(ids), R, bgmv_max_rank)
        elif kind == "seg_start_by_len":
            m["seg_starts"] = list(m["seg_lens"])
        return m
    return bm


def _pool_factory(kind):
    base = O.expected_pool

    def ep(wl):
        p = base(wl)
        for a in p:
            if kind == "no_padding_zero":
                r = wl.slots[a].rank
                p[a]["A"][0][r:] = 1.0
            elif kind == "unfolded":
                p[a]["B"] = [b / p[a]["scale_f32"] for b in p[a]["B"]]
        return p
    return ep


def _rne_trunc(a):
    a32 = np.ascontiguousarray(np.asarray(a, np.float32))
    return (a32.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)


def _offsets_reversed(out_features):
    # slices laid out last to first (the last slice's delta in the first columns)
    outs = [int(o) for o in out_features]
    offs, acc = [0] * len(outs), 0
    for i in reversed(range(len(outs))):
        offs[i] = acc
        acc += outs[i]
    return offs


def _offsets_all_zero(out_features):
    return [0] * len(list(out_features))


def _offsets_inclusive(out_features):
    # each slice starts after its own width (an off-by-one in the prefix sum),
    # clamped so the last slice still fits the row
    outs = [int(o) for o in out_features]
    total = sum(outs)
    offs, acc = [], 0
    for o in outs:
        acc += o
        offs.append(min(acc, total - o))
    return offs


def _forward_slice_A_rotated(wl, rows=None, y_in=None):
    # each slice uses the next slice's A (shapes agree: [rank, in_features])
    slots = {a: type(ad)(**{**ad.__dict__, "A": ad.A[1:] + ad.A[:1]}) for a, ad in wl.slots.items()}
    wl2 = type(wl)(**{**wl.__dict__, "slots": slots})
    return _ORIG_FORWARD(wl2, rows, y_in=y_in)


def _shrink_rank_major(wl, rows):
    # v laid out rank by rank (k * S + s) instead of slice by slice (s * R + k)
    v = _ORIG_SHRINK(wl, rows)
    R, S = wl.max_lora_rank, wl.num_slices
    return v.reshape(v.shape[0], S, R).transpose(0, 2, 1).reshape(v.shape[0], S * R)


_ORIG_FORWARD = O.lora_forward_rows
_ORIG_SHRINK = O.lora_shrink_rows


MUTATIONS = {
    "scale_padded_rank": ("scaling", mut_scale_padded_rank),
    "scale_no_sqrt": ("scaling", mut_scale_no_sqrt),
    "scale_inverted": ("scaling", mut_scale_inverted),
    "delta_sign": ("lora_forward_rows", _forward_factory("sign")),
    "delta_dropped_last_slice": ("lora_forward_rows", _forward_factory("drop_delta_for_last_slice")),
    "delta_wrong_adapter": ("lora_forward_rows", _forward_factory("off_by_one_id")),
    "none_rows_zeroed": ("lora_forward_rows", _forward_factory("none_rows_zeroed")),
    "builder_unstable": ("build_meta", _meta_factory("unstable")),
    "builder_rank_rule_ignored": ("build_meta", _meta_factory("rank_rule_ignored")),
    "builder_prefill_ignored": ("build_meta", _meta_factory("prefill_ignored")),
    "builder_seg_starts": ("build_meta", _meta_factory("seg_start_by_len")),
    "pool_padding_not_zero": ("expected_pool", _pool_factory("no_padding_zero")),
    "pool_unfolded": ("expected_pool", _pool_factory("unfolded")),
    "bf16_truncation": ("f32_to_bf16_rne", _rne_trunc),
    "bf16_double_rounding": ("f64_to_bf16_rne",
                             lambda a: O.f32_to_bf16_rne(np.asarray(a, np.float32)).astype(np.float64)),
    "slices_reversed": ("slice_offsets", _offsets_reversed),
    "slices_all_at_column_0": ("slice_offsets", _offsets_all_zero),
    "slices_offset_by_own_width": ("slice_offsets", _offsets_inclusive),
    "slice_A_rotated": ("lora_forward_rows", _forward_slice_A_rotated),
    "shrink_rank_major_layout": ("lora_shrink_rows", _shrink_rank_major),
    "merge_sign": ("merged_weight",
                   lambda W, ps, sl, dt: np.asarray(W, np.float64) - ps["B"][sl] @ ps["A"][sl]),
    "merge_wrong_slice": ("merged_weight",
                          lambda W, ps, sl, dt: np.asarray(W, np.float64)
                          + ps["B"][sl] @ ps["A"][(sl + 1) % len(ps["A"])]
                          if ps["A"][(sl + 1) % len(ps["A"])].shape == ps["A"][sl].shape
                          else np.asarray(W, np.float64)),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(O, attr, fn)
    assert _caught(monkeypatch) > 0, f"no pin caught mutation {name}"


def test_slot_residency_mutations_are_caught(monkeypatch):
    """Plausible slips in the residency model: evicting the most recently used
    adapter, or evicting one the batch itself uses."""
    def mru(batches, max_loras):
        resident, out = [], []
        for batch in batches:
            wanted = []
            for a in batch:
                if a is not None and a != -1 and a not in wanted:
                    wanted.append(int(a))
            loaded = []
            for a in wanted:
                if a not in resident:
                    if len(resident) == max_loras:
                        resident.remove([b for b in resident if b not in wanted][-1])
                    resident.append(a)
                    loaded.append(a)
            for a in wanted:
                resident.remove(a)
                resident.append(a)
            out.append((list(resident), loaded))
        return out

    def any_victim(batches, max_loras):
        resident, out = [], []
        for batch in batches:
            loaded = []
            for a in batch:
                if a is None or a == -1:
                    continue
                if a in resident:
                    resident.remove(a)
                else:
                    if len(resident) == max_loras:
                        resident.pop(0)
                    loaded.append(int(a))
                resident.append(int(a))
            out.append((list(resident), loaded))
        return out

    for bad in (mru, any_victim):
        monkeypatch.setattr(O, "slot_residency", bad)
        with pytest.raises(AssertionError):
            from oracle_pins import pin_slot_residency
            pin_slot_residency(O)
