"""ctypes binding of liblora_pool.so (include/lora_pool.h).

Argument marshalling only: tensors become ``data_ptr()`` values, the HIP stream
is torch's current stream, status codes become ``LoraError``.  Every step of the
delta path runs in the library's HIP kernels; there is no fallback.  Importing
the compute functions without a built library raises immediately.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Dict, Optional, Sequence

import numpy as np

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "liblora_pool.so")
HEADER = os.path.join(os.path.dirname(PKG_DIR), "include", "lora_pool.h")

LORA_OK = 0
LORA_E_ARG = -1
LORA_E_DTYPE = -2
LORA_E_SHAPE = -3
LORA_E_ALIGN = -4
LORA_E_RANK = -5
LORA_E_ID = -6
LORA_E_WORKSPACE = -7
LORA_E_HIP = -8
STATUS_NAMES = {0: "LORA_OK", -1: "LORA_E_ARG", -2: "LORA_E_DTYPE", -3: "LORA_E_SHAPE",
                -4: "LORA_E_ALIGN", -5: "LORA_E_RANK", -6: "LORA_E_ID",
                -7: "LORA_E_WORKSPACE", -8: "LORA_E_HIP"}

LORA_F32 = 0
LORA_BF16 = 1
LORA_MAX_SLICES = 8
LORA_BGMV_MAX_RANK_DEFAULT = 64


class LoraError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class lora_pool_desc(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("max_loras", ctypes.c_int32),
                ("max_lora_rank", ctypes.c_int32), ("in_features", ctypes.c_int32),
                ("num_slices", ctypes.c_int32),
                ("out_features", ctypes.c_int32 * LORA_MAX_SLICES)]


class lora_meta(ctypes.Structure):
    _fields_ = [("num_sgmv_rows", ctypes.c_int32), ("num_segs", ctypes.c_int32),
                ("num_bgmv_rows", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("sgmv_perm", ctypes.POINTER(ctypes.c_int32)),
                ("seg_starts", ctypes.POINTER(ctypes.c_int32)),
                ("seg_lens", ctypes.POINTER(ctypes.c_int32)),
                ("seg_ids", ctypes.POINTER(ctypes.c_int32)),
                ("bgmv_tok", ctypes.POINTER(ctypes.c_int32)),
                ("bgmv_ids", ctypes.POINTER(ctypes.c_int32))]


class lora_plan(ctypes.Structure):
    _fields_ = [("num_sgmv_rows", ctypes.c_int32), ("num_bgmv_rows", ctypes.c_int32),
                ("num_segs", ctypes.c_int32), ("wave_tiles", ctypes.c_int32),
                ("mfma_tiles", ctypes.c_int32), ("mfma_min_rows", ctypes.c_int32),
                ("ksplit", ctypes.c_int32), ("bgmv_mfma_min_rows", ctypes.c_int32),
                ("ksplit_wave", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("image_offset", ctypes.c_int64), ("image_bytes", ctypes.c_int64),
                ("off_perm", ctypes.c_int64), ("off_wave", ctypes.c_int64),
                ("off_mfma", ctypes.c_int64)]


PLAN_WAVE_ROWS = 8
PLAN_MFMA_ROWS = 64
PLAN_MAX_KSPLIT = 8        # partials of v (wavefront tiles)
PLAN_MAX_KSPLIT_MFMA = 8   # partials of v (MFMA tiles, pools of rank <= 32)
PLAN_MAX_KSPLIT_MFMA_WIDE = 4   # ... pools of rank > 32
PLAN_WAVE_WORDS = 16
PLAN_MFMA_WORDS = 4

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_DP = ctypes.POINTER(lora_pool_desc)

_SIGNATURES = {
    "lora_last_error": (ctypes.c_char_p, []),
    "lora_abi_version": (_I32, []),
    "lora_pool_validate": (_I32, [_DP]),
    "lora_pool_bytes_A": (_I64, [_DP]),
    "lora_pool_bytes_B": (_I64, [_DP]),
    "lora_scaling": (ctypes.c_float, [_I32, ctypes.c_float, _I32]),
    "lora_pool_load": (_I32, [_DP, _P, _P, _I32, _I32, _P, _P, _I32, ctypes.c_float, _I32, _I32,
                              _P]),
    "lora_pool_clear": (_I32, [_DP, _P, _P, _I32, _P]),
    "lora_build_meta": (_I32, [_P, _P, _I32, _I32, _I32, _I32, ctypes.POINTER(lora_meta)]),
    "lora_build_meta_device": (_I32, [_P, _P, _I32, _I32, _I32, _I32, ctypes.POINTER(lora_meta),
                                      _P, _P]),
    "lora_sgmv_shrink": (_I32, [_DP, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _P]),
    "lora_sgmv_expand": (_I32, [_DP, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _P]),
    "lora_bgmv_shrink": (_I32, [_DP, _P, _P, _P, _P, _P, _I32, _I32, _P]),
    "lora_bgmv_expand": (_I32, [_DP, _P, _P, _P, _P, _P, _I32, _I32, _P]),
    "lora_apply_workspace_bytes": (_I64, [_DP, _I32]),
    "lora_apply_host_meta_bytes": (_I64, [_DP, _I32]),
    "lora_apply_plan": (_I32, [_DP, _I32, _P, _P, _I32, _P, _I64, ctypes.POINTER(lora_plan)]),
    "lora_apply_plan_ranked": (_I32, [_DP, _I32, _P, _P, _I32, _P, _P, _I64,
                                      ctypes.POINTER(lora_plan)]),
    "lora_plan_shrink": (_I32, [_DP, _P, _P, _P, _I32, ctypes.POINTER(lora_plan), _P, _P, _P]),
    "lora_plan_expand": (_I32, [_DP, _P, _P, _P, _I32, ctypes.POINTER(lora_plan), _P, _P, _P]),
    "lora_plan_apply": (_I32, [_DP, _P, _P, _P, _P, _I32, ctypes.POINTER(lora_plan), _P, _P, _P,
                               _I64, _P]),
    "lora_apply": (_I32, [_DP, _P, _P, _P, _P, _I32, _P, _P, _I32, _P, _I64, _P, _I64, _P]),
    "lora_apply_device_workspace_bytes": (_I64, [_DP, _I32]),
    "lora_apply_device": (_I32, [_DP, _P, _P, _P, _P, _I32, _P, _P, _I32, _P, _I64, _P]),
    "lora_apply_device_ranked": (_I32, [_DP, _P, _P, _P, _P, _I32, _P, _P, _I32, _P, _P, _I64,
                                        _P]),
    "lora_apply_device_noalloc": (_I32, [_DP, _P, _P, _P, _P, _I32, _P, _P, _I32, _P]),
    "lora_merge_weights": (_I32, [_DP, _P, _P, _I32, _I32, _P, _P, _P]),
    "lora_apply_ranked": (_I32, [_DP, _P, _P, _P, _P, _I32, _P, _P, _I32, _P, _P, _I64, _P, _I64,
                                 _P]),
}

_lib: Optional[ctypes.CDLL] = None


def header_functions() -> list:
    """Names of the functions include/lora_pool.h declares."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s*(lora_[a-z0-9_A-Z]+)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


def lib() -> ctypes.CDLL:
    """Load liblora_pool.so; raise if it was not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m lora_adapter_pool_amd.build` "
            "(there is no fallback implementation)")
    h = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(h, name)
        fn.restype = res
        fn.argtypes = args
    _lib = h
    return h


_pycall = None


def pycall():
    """The CPython binding of the per-call entry points (module _lora_call:
    apply, apply_ranked, apply_device), built beside the library; raise if it
    was not built.  Each function takes the entry point's address (see
    entry_address) and then that entry point's arguments as Python ints."""
    global _pycall
    if _pycall is None:
        try:
            from . import _lora_call
        except ImportError as e:
            raise RuntimeError(
                "the _lora_call binding is missing: build it with "
                "`python -m lora_adapter_pool_amd.build`") from e
        _pycall = _lora_call
    return _pycall


_addresses: dict = {}


def entry_address(name: str) -> int:
    """Address of an entry point of the loaded library (for pycall())."""
    a = _addresses.get(name)
    if a is None:
        a = _addresses[name] = ctypes.cast(getattr(lib(), name), ctypes.c_void_p).value
    return a


def last_error() -> str:
    return lib().lora_last_error().decode("utf-8", "replace")


def _check(status: int) -> int:
    if status < 0:
        raise LoraError(int(status), last_error())
    return status


def make_desc(dtype: str, max_loras: int, max_lora_rank: int, in_features: int,
              out_features: Sequence[int]) -> lora_pool_desc:
    d = lora_pool_desc()
    d.dtype = {"f32": LORA_F32, "fp32": LORA_F32, "float32": LORA_F32,
               "bf16": LORA_BF16, "bfloat16": LORA_BF16}[dtype]
    d.max_loras = int(max_loras)
    d.max_lora_rank = int(max_lora_rank)
    d.in_features = int(in_features)
    d.num_slices = len(out_features)
    for i, o in enumerate(out_features[:LORA_MAX_SLICES]):
        d.out_features[i] = int(o)
    return d


def _ptr(t) -> Optional[int]:
    """data_ptr of a torch tensor / address of a numpy array / int / None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# --------------------------------------------------------------------- pool

def lora_pool_validate(desc) -> int:
    return _check(lib().lora_pool_validate(ctypes.byref(desc)))


def lora_pool_bytes_A(desc) -> int:
    return _check(lib().lora_pool_bytes_A(ctypes.byref(desc)))


def lora_pool_bytes_B(desc) -> int:
    return _check(lib().lora_pool_bytes_B(ctypes.byref(desc)))


def lora_scaling(r: int, alpha: float, use_rslora: bool) -> float:
    return float(lib().lora_scaling(int(r), float(alpha), int(bool(use_rslora))))


def lora_pool_load(desc, A_pool, B_pool, slot, slice_, A_src, B_src, r, alpha, use_rslora,
                   src_on_device: Optional[bool] = None, stream=None) -> None:
    if src_on_device is None:
        src_on_device = not isinstance(A_src, np.ndarray) and bool(getattr(A_src, "is_cuda", False))
    _check(lib().lora_pool_load(ctypes.byref(desc), _ptr(A_pool), _ptr(B_pool), int(slot),
                                int(slice_), _ptr(A_src), _ptr(B_src), int(r), float(alpha),
                                int(bool(use_rslora)), int(bool(src_on_device)), _stream(stream)))


def lora_pool_clear(desc, A_pool, B_pool, slot, stream=None) -> None:
    _check(lib().lora_pool_clear(ctypes.byref(desc), _ptr(A_pool), _ptr(B_pool), int(slot),
                                 _stream(stream)))


# ----------------------------------------------------------------- metadata

def lora_build_meta(ids, prefill, max_loras: int, max_lora_rank: int,
                    bgmv_max_rank: int = 0) -> Dict[str, np.ndarray]:
    ids = np.ascontiguousarray(np.asarray(ids, dtype=np.int32))
    T = int(ids.shape[0])
    pre = None if prefill is None else np.ascontiguousarray(np.asarray(prefill, dtype=np.uint8))
    cap_rows, cap_segs = max(T, 1), max(int(max_loras), 1)
    bufs = {k: np.zeros(cap_rows, np.int32) for k in ("sgmv_perm", "bgmv_tok", "bgmv_ids")}
    bufs.update({k: np.zeros(cap_segs, np.int32) for k in ("seg_starts", "seg_lens", "seg_ids")})
    m = lora_meta()
    for k, a in bufs.items():
        setattr(m, k, a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)))
    _check(lib().lora_build_meta(ids.ctypes.data if T else None,
                                 None if pre is None else pre.ctypes.data, T, int(max_loras),
                                 int(max_lora_rank), int(bgmv_max_rank), ctypes.byref(m)))
    return {
        "sgmv_perm": bufs["sgmv_perm"][:m.num_sgmv_rows].copy(),
        "seg_starts": bufs["seg_starts"][:m.num_segs].copy(),
        "seg_lens": bufs["seg_lens"][:m.num_segs].copy(),
        "seg_ids": bufs["seg_ids"][:m.num_segs].copy(),
        "bgmv_tok": bufs["bgmv_tok"][:m.num_bgmv_rows].copy(),
        "bgmv_ids": bufs["bgmv_ids"][:m.num_bgmv_rows].copy(),
    }


# ------------------------------------------------------------ grouped kernels

def lora_sgmv_shrink(desc, x, A_pool, v, perm, seg_starts, seg_lens, seg_ids, num_segs,
                     num_rows, T, stream=None) -> None:
    _check(lib().lora_sgmv_shrink(ctypes.byref(desc), _ptr(x), _ptr(A_pool), _ptr(v), _ptr(perm),
                                  _ptr(seg_starts), _ptr(seg_lens), _ptr(seg_ids), int(num_segs),
                                  int(num_rows), int(T), _stream(stream)))


def lora_sgmv_expand(desc, v, B_pool, y, perm, seg_starts, seg_lens, seg_ids, num_segs,
                     num_rows, T, stream=None) -> None:
    _check(lib().lora_sgmv_expand(ctypes.byref(desc), _ptr(v), _ptr(B_pool), _ptr(y), _ptr(perm),
                                  _ptr(seg_starts), _ptr(seg_lens), _ptr(seg_ids), int(num_segs),
                                  int(num_rows), int(T), _stream(stream)))


META_DEVICE_MAX_LORAS = 8192


def lora_build_meta_device(ids, prefill, T, max_loras, max_lora_rank, bgmv_max_rank, arrays,
                           counts, stream=None) -> None:
    """Device-side builder: `arrays` maps the lora_meta array names (sgmv_perm,
    seg_starts, seg_lens, seg_ids, bgmv_tok, bgmv_ids) to device int32 tensors;
    `counts` is a device int32[4] (rows, segments, BGMV rows, rejected ids)."""
    m = lora_meta()
    for k in ("sgmv_perm", "seg_starts", "seg_lens", "seg_ids", "bgmv_tok", "bgmv_ids"):
        setattr(m, k, ctypes.cast(_ptr(arrays.get(k)), ctypes.POINTER(ctypes.c_int32)))
    _check(lib().lora_build_meta_device(_ptr(ids), _ptr(prefill), int(T), int(max_loras),
                                        int(max_lora_rank), int(bgmv_max_rank), ctypes.byref(m),
                                        _ptr(counts), _stream(stream)))


def lora_bgmv_shrink(desc, x, A_pool, v, tok, ids, n, T, stream=None) -> None:
    _check(lib().lora_bgmv_shrink(ctypes.byref(desc), _ptr(x), _ptr(A_pool), _ptr(v), _ptr(tok),
                                  _ptr(ids), int(n), int(T), _stream(stream)))


def lora_bgmv_expand(desc, v, B_pool, y, tok, ids, n, T, stream=None) -> None:
    _check(lib().lora_bgmv_expand(ctypes.byref(desc), _ptr(v), _ptr(B_pool), _ptr(y), _ptr(tok),
                                  _ptr(ids), int(n), int(T), _stream(stream)))


# --------------------------------------------------------------- dispatcher

def lora_apply_workspace_bytes(desc, T: int) -> int:
    return _check(lib().lora_apply_workspace_bytes(ctypes.byref(desc), int(T)))


def lora_apply_host_meta_bytes(desc, T: int) -> int:
    return _check(lib().lora_apply_host_meta_bytes(ctypes.byref(desc), int(T)))


def lora_apply_plan(desc, ids, prefill=None, bgmv_max_rank: int = 0, slot_ranks=None):
    """Host tile plan of one batch: (plan fields as a dict, device image as an
    int32 array with 'perm', 'wave' [n, 16] and 'mfma' [n, 4] views).  With
    slot_ranks (int32[max_loras], 0 = max_lora_rank) the tile records carry each
    slot's rank (lora_apply_plan_ranked)."""
    ids = np.ascontiguousarray(np.asarray(ids, dtype=np.int32))
    T = int(ids.shape[0])
    pre = None if prefill is None else np.ascontiguousarray(np.asarray(prefill, dtype=np.uint8))
    nbytes = lora_apply_host_meta_bytes(desc, T)
    raw = np.zeros(nbytes // 4 + 16, np.int32)
    off = (-raw.ctypes.data % 64) // 4
    stage = raw[off:off + nbytes // 4]
    p = lora_plan()
    if slot_ranks is None:
        _check(lib().lora_apply_plan(ctypes.byref(desc), T, ids.ctypes.data if T else None,
                                     None if pre is None else pre.ctypes.data,
                                     int(bgmv_max_rank), stage.ctypes.data, nbytes,
                                     ctypes.byref(p)))
    else:
        sr = np.ascontiguousarray(np.asarray(slot_ranks, dtype=np.int32))
        if sr.shape != (desc.max_loras,):
            raise ValueError(f"slot_ranks has shape {sr.shape}, needs ({desc.max_loras},)")
        _check(lib().lora_apply_plan_ranked(ctypes.byref(desc), T,
                                            ids.ctypes.data if T else None,
                                            None if pre is None else pre.ctypes.data,
                                            int(bgmv_max_rank), sr.ctypes.data,
                                            stage.ctypes.data, nbytes, ctypes.byref(p)))
    d = {k: getattr(p, k) for k, _ in lora_plan._fields_}
    img = stage[p.image_offset // 4: (p.image_offset + p.image_bytes) // 4].copy()
    views = {
        "perm": img[p.off_perm:p.off_perm + p.num_sgmv_rows + p.num_bgmv_rows],
        "wave": img[p.off_wave:p.off_wave + PLAN_WAVE_WORDS * p.wave_tiles].reshape(-1, PLAN_WAVE_WORDS),
        "mfma": img[p.off_mfma:p.off_mfma + PLAN_MFMA_WORDS * p.mfma_tiles].reshape(-1, PLAN_MFMA_WORDS),
    }
    return d, img, views


def plan_struct(d: dict) -> "lora_plan":
    """lora_plan from the dict lora_apply_plan returns."""
    p = lora_plan()
    for k, _ in lora_plan._fields_:
        setattr(p, k, int(d[k]))
    return p


def lora_plan_shrink(desc, x, A_pool, v, T, plan, image, image_host=None, stream=None) -> None:
    p = plan if isinstance(plan, lora_plan) else plan_struct(plan)
    _check(lib().lora_plan_shrink(ctypes.byref(desc), _ptr(x), _ptr(A_pool), _ptr(v), int(T),
                                  ctypes.byref(p), _ptr(image), _ptr(image_host),
                                  _stream(stream)))


def lora_plan_expand(desc, v, B_pool, y, T, plan, image, image_host=None, stream=None) -> None:
    p = plan if isinstance(plan, lora_plan) else plan_struct(plan)
    _check(lib().lora_plan_expand(ctypes.byref(desc), _ptr(v), _ptr(B_pool), _ptr(y), int(T),
                                  ctypes.byref(p), _ptr(image), _ptr(image_host),
                                  _stream(stream)))


def lora_plan_apply(desc, x, A_pool, B_pool, y, T, plan, image, image_host=None, ws=None,
                    ws_bytes=0, stream=None) -> None:
    """Both stages of a plan (one launch for small plans); ws as for lora_apply."""
    p = plan if isinstance(plan, lora_plan) else plan_struct(plan)
    _check(lib().lora_plan_apply(ctypes.byref(desc), _ptr(x), _ptr(A_pool), _ptr(B_pool), _ptr(y),
                                 int(T), ctypes.byref(p), _ptr(image), _ptr(image_host), _ptr(ws),
                                 int(ws_bytes), _stream(stream)))


def lora_apply(desc, A_pool, B_pool, x, y, T, ids_host, prefill_host, bgmv_max_rank, ws,
               ws_bytes, meta_host, meta_host_bytes, stream=None) -> None:
    _check(pycall().apply(entry_address("lora_apply"), ctypes.addressof(desc), _ptr(A_pool),
                          _ptr(B_pool), _ptr(x), _ptr(y), int(T), _ptr(ids_host),
                          _ptr(prefill_host), int(bgmv_max_rank), _ptr(ws), int(ws_bytes),
                          _ptr(meta_host), int(meta_host_bytes), _stream(stream)))


def lora_apply_ranked(desc, A_pool, B_pool, x, y, T, ids_host, prefill_host, bgmv_max_rank,
                      slot_ranks_host, ws, ws_bytes, meta_host, meta_host_bytes,
                      stream=None) -> None:
    """lora_apply with each slot's true rank (host int32[max_loras], 0 = max_lora_rank)."""
    _check(pycall().apply_ranked(entry_address("lora_apply_ranked"), ctypes.addressof(desc),
                                 _ptr(A_pool), _ptr(B_pool), _ptr(x), _ptr(y), int(T),
                                 _ptr(ids_host), _ptr(prefill_host), int(bgmv_max_rank),
                                 _ptr(slot_ranks_host), _ptr(ws), int(ws_bytes), _ptr(meta_host),
                                 int(meta_host_bytes), _stream(stream)))


def lora_merge_weights(desc, A_pool, B_pool, slot, slice_, W, W_out, stream=None) -> None:
    """W_out = round(W + B_fold A) for one slot and slice (W, W_out [out_s, K]
    device tensors of the pool dtype; W_out may be W)."""
    _check(lib().lora_merge_weights(ctypes.byref(desc), _ptr(A_pool), _ptr(B_pool), int(slot),
                                    int(slice_), _ptr(W), _ptr(W_out), _stream(stream)))


def lora_apply_device_workspace_bytes(desc, T: int) -> int:
    return _check(lib().lora_apply_device_workspace_bytes(ctypes.byref(desc), int(T)))


def lora_apply_device(desc, A_pool, B_pool, x, y, T, ids, prefill, bgmv_max_rank, ws, ws_bytes,
                      stream=None) -> None:
    """The delta path from device ids / prefill flags (device metadata and a
    device-built tile plan; graph-capturable)."""
    _check(pycall().apply_device(entry_address("lora_apply_device"), ctypes.addressof(desc),
                                 _ptr(A_pool), _ptr(B_pool), _ptr(x), _ptr(y), int(T), _ptr(ids),
                                 _ptr(prefill), int(bgmv_max_rank), _ptr(ws), int(ws_bytes),
                                 _stream(stream)))


NOALLOC_SCRATCH_BYTES = 64 << 20   # LORA_NOALLOC_SCRATCH_BYTES


def lora_apply_device_noalloc(desc, A_pool, B_pool, x, y, T, ids, prefill, bgmv_max_rank,
                              stream=None):
    """lora_apply_device with the library's own per-GPU scratch as workspace:
    allocates nothing; batches needing more than NOALLOC_SCRATCH_BYTES are
    rejected.  Calls that overlap on one GPU race on the scratch."""
    _check(lib().lora_apply_device_noalloc(ctypes.byref(desc), _ptr(A_pool), _ptr(B_pool),
                                           _ptr(x), _ptr(y), int(T), _ptr(ids), _ptr(prefill),
                                           int(bgmv_max_rank), _stream(stream)))


def lora_apply_device_ranked(desc, A_pool, B_pool, x, y, T, ids, prefill, bgmv_max_rank,
                             slot_ranks, ws, ws_bytes, stream=None) -> None:
    """lora_apply_device with each slot's true rank (device int32[max_loras])."""
    _check(lib().lora_apply_device_ranked(ctypes.byref(desc), _ptr(A_pool), _ptr(B_pool),
                                          _ptr(x), _ptr(y), int(T), _ptr(ids), _ptr(prefill),
                                          int(bgmv_max_rank), _ptr(slot_ranks), _ptr(ws),
                                          int(ws_bytes), _stream(stream)))
