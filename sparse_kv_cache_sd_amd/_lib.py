"""ctypes binding of libsdkv.so (include/sd.h): argument marshalling only.

Every function below takes torch tensors, checks that each one lives on the
GPU with the dtype, shape and contiguity the C ABI expects (so that no kernel
is ever handed a host pointer or a short buffer), and calls the entry point
of the same name.  All arithmetic happens in the HIP kernels.  A missing
library raises at once; there is no fallback.
"""

from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsdkv.so")

SD_F32, SD_BF16 = 0, 1
UNIT_TOKEN, UNIT_PAGE = 0, 1
_UNITS = {"token": UNIT_TOKEN, "page": UNIT_PAGE}
_STATUS = {0: "SD_OK", 1: "SD_E_NULL", 2: "SD_E_SHAPE", 3: "SD_E_DTYPE", 4: "SD_E_RATIO",
           5: "SD_E_WORKSPACE", 6: "SD_E_UNSUPPORTED", 7: "SD_E_DEVICE"}
WS_ALIGN = 256


class SdError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


class SdShape(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
        ("max_seq_len", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("num_pages", ctypes.c_int64),
        ("softmax_scale", ctypes.c_float),
    ]


class SdSelection(ctypes.Structure):
    _fields_ = [
        ("kind", ctypes.c_int32),
        ("init_units", ctypes.c_int32),
        ("local_units", ctypes.c_int32),
        ("scorer", ctypes.c_int32),
        ("r_kv", ctypes.c_double),
        ("max_dropped", ctypes.c_double),
    ]


SEL_TOPK, SEL_WINDOW, SEL_INIT_LOCAL_TOPK, SEL_MASS_BUDGET = 0, 1, 2, 3
_SEL_KINDS = {"topk": SEL_TOPK, "window": SEL_WINDOW, "init_local_topk": SEL_INIT_LOCAL_TOPK,
              "mass_budget": SEL_MASS_BUDGET}
_SCORERS = {"bounds": 0, "compressed": 1}

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_SELP = ctypes.POINTER(SdSelection)
_SIGS = {
    "sd_keep_count": (ctypes.c_int32, [ctypes.c_double, _I32]),
    "sd_workspace_bytes": (ctypes.c_int, [ctypes.POINTER(SdShape), _I32, ctypes.c_double,
                                          ctypes.POINTER(ctypes.c_size_t)]),
    "sd_update_page_bounds": (ctypes.c_int, [ctypes.POINTER(SdShape), _P, _P, _P, _P, _I32, _P,
                                             _P]),
    "sd_append_page_bounds": (ctypes.c_int, [ctypes.POINTER(SdShape), _P, _P, _P, _P, _I32, _P,
                                             _P]),
    "sd_score_pages": (ctypes.c_int, [ctypes.POINTER(SdShape), _P, _P, _P, _P, _P, _I32, _P,
                                      _P, _P]),
    "sd_select_topk": (ctypes.c_int, [ctypes.POINTER(SdShape), _I32, _P, _P, ctypes.c_double,
                                      _P, _P, _P, ctypes.c_size_t, _P]),
    "sd_attend_splitk": (ctypes.c_int, [ctypes.POINTER(SdShape), _P, _P, _P, _P, _P, _I32, _P,
                                        _P, _I32, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "sd_decode_step": (ctypes.c_int, [ctypes.POINTER(SdShape), _P, _P, _P, _P, _P, _P, _I32,
                                      ctypes.c_double, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "sd_select_attend": (ctypes.c_int, [ctypes.POINTER(SdShape), _P, _P, _P, _P, _P, _P,
                                        ctypes.c_double, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "sd_attend_partials": (ctypes.c_int, [ctypes.POINTER(SdShape), _P, _P, _P, _P, _P, _I32, _P,
                                          _P, _I32, _P, _P, ctypes.c_double, _P, _P, _P,
                                          ctypes.c_size_t, _P]),
    "sd_merge_splits": (ctypes.c_int, [ctypes.POINTER(SdShape), _P, _P, _P, ctypes.c_size_t, _P]),
    "sd_selection_capacity": (ctypes.c_int32, [_SELP, _I32]),
    "sd_workspace_bytes_sel": (ctypes.c_int, [ctypes.POINTER(SdShape), _I32, _SELP,
                                              ctypes.POINTER(ctypes.c_size_t)]),
    "sd_select_units": (ctypes.c_int, [ctypes.POINTER(SdShape), _I32, _P, _P, _P, _SELP, _P, _P,
                                       _P, ctypes.c_size_t, _P]),
    "sd_decode_step_sel": (ctypes.c_int, [ctypes.POINTER(SdShape), _P, _P, _P, _P, _P, _P, _I32,
                                          _SELP, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "sd_update_compressed_keys": (ctypes.c_int, [ctypes.POINTER(SdShape), _P, _P, _P, _P, _P]),
    "sd_score_compressed": (ctypes.c_int, [ctypes.POINTER(SdShape), _P, _P, _P, _P, _P]),
    "sd_workspace_bytes_entmax": (ctypes.c_int, [ctypes.POINTER(SdShape), _I32, _SELP,
                                                 ctypes.POINTER(ctypes.c_size_t)]),
    "sd_decode_step_entmax": (ctypes.c_int, [ctypes.POINTER(SdShape), _P, _P, _P, _P, _P, _P,
                                             _I32, _SELP, ctypes.c_double, _P, _P, _P, _P, _P,
                                             ctypes.c_size_t, _P]),
    "sd_dropped_mass": (ctypes.c_int, [ctypes.POINTER(SdShape), _P, _P, _P, _P, _P, _I32, _P,
                                       _P]),
    "sd_decode_step_noalloc": (ctypes.c_int, [ctypes.POINTER(SdShape), _P, _P, _P, _P, _P, _P,
                                              _I32, ctypes.c_double, _P, _P, _P, _P, _P]),
    "sd_last_error": (ctypes.c_char_p, []),
}
EXPORTS = tuple(_SIGS)

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m sparse_kv_cache_sd_amd.build`")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(h, name)
            f.restype = res
            f.argtypes = args
        _lib = h
    return _lib


def _check(status: int) -> None:
    if status != 0:
        raise SdError(status, lib().sd_last_error().decode())


# ----------------------------------------------------------------------------
# shape
# ----------------------------------------------------------------------------

@dataclass(frozen=True)
class Shape:
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    max_pages_per_seq: int
    max_seq_len: int
    dtype: str             # "f32" | "bf16"
    num_pages: int
    softmax_scale: float = 0.0

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def units_max(self, unit: str) -> int:
        return self.max_pages_per_seq if unit == "page" else self.max_seq_len

    def c(self) -> SdShape:
        return SdShape(self.batch, self.num_q_heads, self.num_kv_heads, self.head_dim,
                       self.page_size, self.max_pages_per_seq, self.max_seq_len,
                       SD_F32 if self.dtype == "f32" else SD_BF16, self.num_pages,
                       self.softmax_scale)


def _unit(unit) -> int:
    if isinstance(unit, str):
        return _UNITS[unit]
    return int(unit)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(t, name, dtype, shape=None, optional=False):
    """Device pointer of a contiguous GPU tensor of the given dtype and shape."""
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _ws(ws, need):
    if need == 0 and ws is None:
        return None, 0
    p = _dev(ws, "ws", torch.uint8)
    if ws.data_ptr() % WS_ALIGN:
        raise ValueError(f"ws must be {WS_ALIGN}-byte aligned")
    return p, ws.numel()


# ----------------------------------------------------------------------------
# entry points
# ----------------------------------------------------------------------------

def keep_count(r_kv: float, num_units: int) -> int:
    k = lib().sd_keep_count(float(r_kv), int(num_units))
    if k < 0:
        raise ValueError("r_kv must be finite and > 0, num_units >= 1")
    return k


def workspace_bytes(shape: Shape, unit, r_kv: float) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().sd_workspace_bytes(ctypes.byref(shape.c()), _unit(unit), float(r_kv),
                                    ctypes.byref(out)))
    return int(out.value)


def alloc_workspace(shape: Shape, unit, r_kv: float, device="cuda") -> torch.Tensor:
    """A workspace for calls with this shape, unit and keep ratio."""
    n = max(1, workspace_bytes(shape, unit, r_kv))
    return torch.empty(n, dtype=torch.uint8, device=device)


def _kv_shape(s: Shape):
    return (s.num_pages, s.num_kv_heads, s.page_size, s.head_dim)


def _bounds_shape(s: Shape):
    return (s.batch, s.num_kv_heads, s.max_pages_per_seq, 2, s.head_dim)


def bounds_shape(shape: Shape):
    """Shape of the page-statistics tensor: [B, H_kv, max_pages_per_seq, 2, d]."""
    return _bounds_shape(shape)


def update_page_bounds(shape: Shape, k_pages, block_table, seq_lens, page_bounds, pages=None,
                       stream=None):
    """Page bounds of every page, or of the listed (sequence, logical page)
    pairs only (``pages``: int32 [n, 2] on the device)."""
    s = shape
    n = 0
    if pages is not None:
        if pages.dim() != 2 or pages.shape[1] != 2:
            raise ValueError("pages must have shape (n, 2)")
        n = int(pages.shape[0])
        if n == 0:
            return  # nothing to update (an empty tensor has no device address to pass)
    _check(lib().sd_update_page_bounds(
        ctypes.byref(s.c()),
        _dev(k_pages, "k_pages", s.torch_dtype, _kv_shape(s)),
        _dev(block_table, "block_table", torch.int32, (s.batch, s.max_pages_per_seq)),
        _dev(seq_lens, "seq_lens", torch.int32, (s.batch,)),
        _dev(pages, "pages", torch.int32, optional=True), n,
        _dev(page_bounds, "page_bounds", s.torch_dtype,
             _bounds_shape(s)),
        _stream(stream)))


def append_page_bounds(shape: Shape, k_pages, block_table, seq_lens, appended, max_appended,
                       page_bounds, stream=None):
    """Fold the tokens each sequence gained (``appended``: int32 [B] on the
    device, each at most ``max_appended``) into their pages' bounds."""
    s = shape
    _check(lib().sd_append_page_bounds(
        ctypes.byref(s.c()),
        _dev(k_pages, "k_pages", s.torch_dtype, _kv_shape(s)),
        _dev(block_table, "block_table", torch.int32, (s.batch, s.max_pages_per_seq)),
        _dev(seq_lens, "seq_lens", torch.int32, (s.batch,)),
        _dev(appended, "appended", torch.int32, (s.batch,)), int(max_appended),
        _dev(page_bounds, "page_bounds", s.torch_dtype, _bounds_shape(s)),
        _stream(stream)))


def score_pages(shape: Shape, q, k_pages, page_bounds, block_table, seq_lens, unit,
                unit_scores, token_logits=None, stream=None):
    s, u = shape, _unit(unit)
    umax = s.max_pages_per_seq if u == UNIT_PAGE else s.max_seq_len
    _check(lib().sd_score_pages(
        ctypes.byref(s.c()),
        _dev(q, "q", s.torch_dtype, (s.batch, s.num_q_heads, s.head_dim)),
        _dev(k_pages, "k_pages", s.torch_dtype, _kv_shape(s), optional=u == UNIT_PAGE),
        _dev(page_bounds, "page_bounds", s.torch_dtype,
             _bounds_shape(s), optional=u == UNIT_TOKEN),
        _dev(block_table, "block_table", torch.int32, (s.batch, s.max_pages_per_seq)),
        _dev(seq_lens, "seq_lens", torch.int32, (s.batch,)),
        u,
        _dev(unit_scores, "unit_scores", torch.float32, (s.batch, s.num_kv_heads, umax)),
        _dev(token_logits, "token_logits", torch.float32,
             (s.batch, s.num_q_heads, s.max_seq_len), optional=u == UNIT_PAGE),
        _stream(stream)))


def select_topk(shape: Shape, unit, seq_lens, unit_scores, r_kv, sel_idx, sel_count,
                ws=None, stream=None):
    s, u = shape, _unit(unit)
    umax = s.max_pages_per_seq if u == UNIT_PAGE else s.max_seq_len
    k_max = keep_count(r_kv, umax)
    wp, wn = _ws(ws, 0)
    _check(lib().sd_select_topk(
        ctypes.byref(s.c()), u,
        _dev(seq_lens, "seq_lens", torch.int32, (s.batch,)),
        _dev(unit_scores, "unit_scores", torch.float32, (s.batch, s.num_kv_heads, umax)),
        float(r_kv),
        _dev(sel_idx, "sel_idx", torch.int32, (s.batch, s.num_kv_heads, k_max)),
        _dev(sel_count, "sel_count", torch.int32, (s.batch, s.num_kv_heads)),
        wp, wn, _stream(stream)))


def attend_splitk(shape: Shape, q, k_pages, v_pages, block_table, seq_lens, unit, sel_idx,
                  sel_count, out, lse, ws, token_logits=None, stream=None):
    s, u = shape, _unit(unit)
    k_max = 0
    if sel_idx is not None:
        if sel_idx.dim() != 3 or tuple(sel_idx.shape[:2]) != (s.batch, s.num_kv_heads):
            raise ValueError("sel_idx must have shape (B, H_kv, k_max)")
        k_max = int(sel_idx.shape[2])
    wp, wn = _ws(ws, 1)
    _check(lib().sd_attend_splitk(
        ctypes.byref(s.c()),
        _dev(q, "q", s.torch_dtype, (s.batch, s.num_q_heads, s.head_dim)),
        _dev(k_pages, "k_pages", s.torch_dtype, _kv_shape(s), optional=token_logits is not None),
        _dev(v_pages, "v_pages", s.torch_dtype, _kv_shape(s)),
        _dev(block_table, "block_table", torch.int32, (s.batch, s.max_pages_per_seq)),
        _dev(seq_lens, "seq_lens", torch.int32, (s.batch,)),
        u,
        _dev(sel_idx, "sel_idx", torch.int32, optional=True),
        _dev(sel_count, "sel_count", torch.int32, (s.batch, s.num_kv_heads),
             optional=sel_idx is None),
        k_max,
        _dev(token_logits, "token_logits", torch.float32,
             (s.batch, s.num_q_heads, s.max_seq_len), optional=True),
        _dev(out, "out", torch.float32, (s.batch, s.num_q_heads, s.head_dim)),
        _dev(lse, "lse", torch.float32, (s.batch, s.num_q_heads)),
        wp, wn, _stream(stream)))


def decode_step(shape: Shape, q, k_pages, v_pages, page_bounds, block_table, seq_lens, unit,
                r_kv, out, lse, ws, sel_idx=None, sel_count=None, stream=None):
    s, u = shape, _unit(unit)
    umax = s.max_pages_per_seq if u == UNIT_PAGE else s.max_seq_len
    dense = r_kv >= 1.0
    wp, wn = _ws(ws, 1)
    k_max = keep_count(r_kv, umax) if not (math.isnan(r_kv) or r_kv <= 0) else 0
    _check(lib().sd_decode_step(
        ctypes.byref(s.c()),
        _dev(q, "q", s.torch_dtype, (s.batch, s.num_q_heads, s.head_dim)),
        _dev(k_pages, "k_pages", s.torch_dtype, _kv_shape(s)),
        _dev(v_pages, "v_pages", s.torch_dtype, _kv_shape(s)),
        _dev(page_bounds, "page_bounds", s.torch_dtype,
             _bounds_shape(s), optional=dense or u == UNIT_TOKEN),
        _dev(block_table, "block_table", torch.int32, (s.batch, s.max_pages_per_seq)),
        _dev(seq_lens, "seq_lens", torch.int32, (s.batch,)),
        u, float(r_kv),
        _dev(out, "out", torch.float32, (s.batch, s.num_q_heads, s.head_dim)),
        _dev(lse, "lse", torch.float32, (s.batch, s.num_q_heads)),
        _dev(sel_idx, "sel_idx", torch.int32, (s.batch, s.num_kv_heads, k_max), optional=True),
        _dev(sel_count, "sel_count", torch.int32, (s.batch, s.num_kv_heads), optional=True),
        wp, wn, _stream(stream)))


def decode_step_noalloc(shape: Shape, q, k_pages, v_pages, page_bounds, block_table, seq_lens,
                        unit, r_kv, out, lse, sel_idx=None, sel_count=None, stream=None):
    """decode_step with the library's static device scratch instead of a
    workspace (no allocation; calls on one device must not overlap)."""
    s, u = shape, _unit(unit)
    umax = s.max_pages_per_seq if u == UNIT_PAGE else s.max_seq_len
    dense = r_kv >= 1.0
    k_max = keep_count(r_kv, umax) if not (math.isnan(r_kv) or r_kv <= 0) else 0
    _check(lib().sd_decode_step_noalloc(
        ctypes.byref(s.c()),
        _dev(q, "q", s.torch_dtype, (s.batch, s.num_q_heads, s.head_dim)),
        _dev(k_pages, "k_pages", s.torch_dtype, _kv_shape(s)),
        _dev(v_pages, "v_pages", s.torch_dtype, _kv_shape(s)),
        _dev(page_bounds, "page_bounds", s.torch_dtype,
             _bounds_shape(s), optional=dense or u == UNIT_TOKEN),
        _dev(block_table, "block_table", torch.int32, (s.batch, s.max_pages_per_seq)),
        _dev(seq_lens, "seq_lens", torch.int32, (s.batch,)),
        u, float(r_kv),
        _dev(out, "out", torch.float32, (s.batch, s.num_q_heads, s.head_dim)),
        _dev(lse, "lse", torch.float32, (s.batch, s.num_q_heads)),
        _dev(sel_idx, "sel_idx", torch.int32, (s.batch, s.num_kv_heads, k_max), optional=True),
        _dev(sel_count, "sel_count", torch.int32, (s.batch, s.num_kv_heads), optional=True),
        _stream(stream)))


def select_attend(shape: Shape, q, k_pages, v_pages, block_table, seq_lens, unit_scores, r_kv,
                  out, lse, ws, sel_idx=None, sel_count=None, stream=None):
    s = shape
    k_max = keep_count(r_kv, s.max_pages_per_seq)
    wp, wn = _ws(ws, 1)
    _check(lib().sd_select_attend(
        ctypes.byref(s.c()),
        _dev(q, "q", s.torch_dtype, (s.batch, s.num_q_heads, s.head_dim)),
        _dev(k_pages, "k_pages", s.torch_dtype, _kv_shape(s)),
        _dev(v_pages, "v_pages", s.torch_dtype, _kv_shape(s)),
        _dev(block_table, "block_table", torch.int32, (s.batch, s.max_pages_per_seq)),
        _dev(seq_lens, "seq_lens", torch.int32, (s.batch,)),
        _dev(unit_scores, "unit_scores", torch.float32,
             (s.batch, s.num_kv_heads, s.max_pages_per_seq)),
        float(r_kv),
        _dev(out, "out", torch.float32, (s.batch, s.num_q_heads, s.head_dim)),
        _dev(lse, "lse", torch.float32, (s.batch, s.num_q_heads)),
        _dev(sel_idx, "sel_idx", torch.int32, (s.batch, s.num_kv_heads, k_max), optional=True),
        _dev(sel_count, "sel_count", torch.int32, (s.batch, s.num_kv_heads), optional=True),
        wp, wn, _stream(stream)))


def attend_partials(shape: Shape, q, k_pages, v_pages, block_table, seq_lens, unit, ws,
                    sel_idx=None, sel_count=None, token_logits=None, unit_scores=None,
                    r_kv=1.0, sel_out=None, sel_count_out=None, stream=None):
    s, u = shape, _unit(unit)
    k_max = 0
    if sel_idx is not None:
        if sel_idx.dim() != 3 or tuple(sel_idx.shape[:2]) != (s.batch, s.num_kv_heads):
            raise ValueError("sel_idx must have shape (B, H_kv, k_max)")
        k_max = int(sel_idx.shape[2])
    km_sel = keep_count(r_kv, s.max_pages_per_seq) if unit_scores is not None else 0
    wp, wn = _ws(ws, 1)
    _check(lib().sd_attend_partials(
        ctypes.byref(s.c()),
        _dev(q, "q", s.torch_dtype, (s.batch, s.num_q_heads, s.head_dim)),
        _dev(k_pages, "k_pages", s.torch_dtype, _kv_shape(s), optional=token_logits is not None),
        _dev(v_pages, "v_pages", s.torch_dtype, _kv_shape(s)),
        _dev(block_table, "block_table", torch.int32, (s.batch, s.max_pages_per_seq)),
        _dev(seq_lens, "seq_lens", torch.int32, (s.batch,)),
        u,
        _dev(sel_idx, "sel_idx", torch.int32, optional=True),
        _dev(sel_count, "sel_count", torch.int32, (s.batch, s.num_kv_heads),
             optional=sel_idx is None),
        k_max,
        _dev(token_logits, "token_logits", torch.float32,
             (s.batch, s.num_q_heads, s.max_seq_len), optional=True),
        _dev(unit_scores, "unit_scores", torch.float32,
             (s.batch, s.num_kv_heads, s.max_pages_per_seq), optional=True),
        float(r_kv),
        _dev(sel_out, "sel_out", torch.int32, (s.batch, s.num_kv_heads, km_sel), optional=True),
        _dev(sel_count_out, "sel_count_out", torch.int32, (s.batch, s.num_kv_heads),
             optional=True),
        wp, wn, _stream(stream)))


def merge_splits(shape: Shape, out, lse, ws, stream=None):
    s = shape
    wp, wn = _ws(ws, 1)
    _check(lib().sd_merge_splits(
        ctypes.byref(s.c()),
        _dev(out, "out", torch.float32, (s.batch, s.num_q_heads, s.head_dim)),
        _dev(lse, "lse", torch.float32, (s.batch, s.num_q_heads)),
        wp, wn, _stream(stream)))


# ----------------------------------------------------------------------------
# structured index sets
# ----------------------------------------------------------------------------

@dataclass(frozen=True)
class Selection:
    """Which units a decode step keeps: kind "topk", "window",
    "init_local_topk" or "mass_budget" (include/sd.h, sd_selection)."""
    kind: str = "topk"
    r_kv: float = 0.3
    init_units: int = 0
    local_units: int = 0
    max_dropped: float = 0.0
    scorer: str = "bounds"   # page unit: "bounds" or "compressed"

    def c(self) -> SdSelection:
        if self.kind not in _SEL_KINDS:
            raise ValueError(f"unknown selection kind {self.kind!r}")
        if self.scorer not in _SCORERS:
            raise ValueError(f"unknown scorer {self.scorer!r}")
        return SdSelection(_SEL_KINDS[self.kind], int(self.init_units), int(self.local_units),
                           _SCORERS[self.scorer], float(self.r_kv), float(self.max_dropped))


def selection_capacity(sel: Selection, num_units: int) -> int:
    c = lib().sd_selection_capacity(ctypes.byref(sel.c()), int(num_units))
    if c < 0:
        raise ValueError("invalid selection or num_units < 1")
    return c


def workspace_bytes_sel(shape: Shape, unit, sel: Selection) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().sd_workspace_bytes_sel(ctypes.byref(shape.c()), _unit(unit),
                                        ctypes.byref(sel.c()), ctypes.byref(out)))
    return int(out.value)


def alloc_workspace_sel(shape: Shape, unit, sel: Selection, device="cuda") -> torch.Tensor:
    n = max(1, workspace_bytes_sel(shape, unit, sel))
    return torch.empty(n, dtype=torch.uint8, device=device)


def select_units(shape: Shape, unit, seq_lens, unit_scores, sel: Selection, sel_idx, sel_count,
                 ws=None, token_logits=None, stream=None):
    s, u = shape, _unit(unit)
    umax = s.max_pages_per_seq if u == UNIT_PAGE else s.max_seq_len
    cap = selection_capacity(sel, umax)
    wp, wn = _ws(ws, 0)
    _check(lib().sd_select_units(
        ctypes.byref(s.c()), u,
        _dev(seq_lens, "seq_lens", torch.int32, (s.batch,)),
        _dev(unit_scores, "unit_scores", torch.float32, (s.batch, s.num_kv_heads, umax),
             optional=sel.kind == "window"),
        _dev(token_logits, "token_logits", torch.float32,
             (s.batch, s.num_q_heads, s.max_seq_len), optional=sel.kind != "mass_budget"),
        ctypes.byref(sel.c()),
        _dev(sel_idx, "sel_idx", torch.int32, (s.batch, s.num_kv_heads, cap)),
        _dev(sel_count, "sel_count", torch.int32, (s.batch, s.num_kv_heads)),
        wp, wn, _stream(stream)))


def compressed_keys_shape(shape: Shape):
    """Shape of the compressed-key tensor (fp32): [B, H_kv, ceil(max_seq_len / 16), d]."""
    return (shape.batch, shape.num_kv_heads, -(-shape.max_seq_len // 16), shape.head_dim)


def update_compressed_keys(shape: Shape, k_pages, block_table, seq_lens, compressed_keys,
                           stream=None):
    s = shape
    _check(lib().sd_update_compressed_keys(
        ctypes.byref(s.c()),
        _dev(k_pages, "k_pages", s.torch_dtype, _kv_shape(s)),
        _dev(block_table, "block_table", torch.int32, (s.batch, s.max_pages_per_seq)),
        _dev(seq_lens, "seq_lens", torch.int32, (s.batch,)),
        _dev(compressed_keys, "compressed_keys", torch.float32, compressed_keys_shape(s)),
        _stream(stream)))


def score_compressed(shape: Shape, q, compressed_keys, seq_lens, unit_scores, stream=None):
    s = shape
    _check(lib().sd_score_compressed(
        ctypes.byref(s.c()),
        _dev(q, "q", s.torch_dtype, (s.batch, s.num_q_heads, s.head_dim)),
        _dev(compressed_keys, "compressed_keys", torch.float32, compressed_keys_shape(s)),
        _dev(seq_lens, "seq_lens", torch.int32, (s.batch,)),
        _dev(unit_scores, "unit_scores", torch.float32,
             (s.batch, s.num_kv_heads, s.max_pages_per_seq)),
        _stream(stream)))


def decode_step_sel(shape: Shape, q, k_pages, v_pages, page_bounds, block_table, seq_lens, unit,
                    sel: Selection, out, lse, ws, sel_idx=None, sel_count=None, stream=None):
    """page_bounds: the page bounds, or with sel.scorer == "compressed" the
    compressed keys."""
    s, u = shape, _unit(unit)
    umax = s.max_pages_per_seq if u == UNIT_PAGE else s.max_seq_len
    cap = selection_capacity(sel, umax)
    wp, wn = _ws(ws, 1)
    stats = (_dev(page_bounds, "compressed_keys", torch.float32, compressed_keys_shape(s),
                  optional=True)
             if sel.scorer == "compressed" else
             _dev(page_bounds, "page_bounds", s.torch_dtype, _bounds_shape(s), optional=True))
    _check(lib().sd_decode_step_sel(
        ctypes.byref(s.c()),
        _dev(q, "q", s.torch_dtype, (s.batch, s.num_q_heads, s.head_dim)),
        _dev(k_pages, "k_pages", s.torch_dtype, _kv_shape(s)),
        _dev(v_pages, "v_pages", s.torch_dtype, _kv_shape(s)),
        stats,
        _dev(block_table, "block_table", torch.int32, (s.batch, s.max_pages_per_seq)),
        _dev(seq_lens, "seq_lens", torch.int32, (s.batch,)),
        u, ctypes.byref(sel.c()),
        _dev(out, "out", torch.float32, (s.batch, s.num_q_heads, s.head_dim)),
        _dev(lse, "lse", torch.float32, (s.batch, s.num_q_heads)),
        _dev(sel_idx, "sel_idx", torch.int32, (s.batch, s.num_kv_heads, cap), optional=True),
        _dev(sel_count, "sel_count", torch.int32, (s.batch, s.num_kv_heads), optional=True),
        wp, wn, _stream(stream)))


# ----------------------------------------------------------------------------
# alpha-entmax attention over the kept set
# ----------------------------------------------------------------------------

def workspace_bytes_entmax(shape: Shape, unit, sel: Selection) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().sd_workspace_bytes_entmax(ctypes.byref(shape.c()), _unit(unit),
                                           ctypes.byref(sel.c()), ctypes.byref(out)))
    return int(out.value)


def alloc_workspace_entmax(shape: Shape, unit, sel: Selection, device="cuda") -> torch.Tensor:
    n = max(1, workspace_bytes_entmax(shape, unit, sel))
    return torch.empty(n, dtype=torch.uint8, device=device)


def decode_step_entmax(shape: Shape, q, k_pages, v_pages, page_stats, block_table, seq_lens, unit,
                       sel: Selection, alpha: float, out, ws, tau=None, sel_idx=None,
                       sel_count=None, stream=None):
    """page_stats: the page bounds, or with sel.scorer == "compressed" the
    compressed keys (may be None where they are not read)."""
    s, u = shape, _unit(unit)
    umax = s.max_pages_per_seq if u == UNIT_PAGE else s.max_seq_len
    cap = selection_capacity(sel, umax)
    wp, wn = _ws(ws, 1)
    stats = (_dev(page_stats, "compressed_keys", torch.float32, compressed_keys_shape(s),
                  optional=True)
             if sel.scorer == "compressed" else
             _dev(page_stats, "page_bounds", s.torch_dtype, _bounds_shape(s), optional=True))
    _check(lib().sd_decode_step_entmax(
        ctypes.byref(s.c()),
        _dev(q, "q", s.torch_dtype, (s.batch, s.num_q_heads, s.head_dim)),
        _dev(k_pages, "k_pages", s.torch_dtype, _kv_shape(s)),
        _dev(v_pages, "v_pages", s.torch_dtype, _kv_shape(s)),
        stats,
        _dev(block_table, "block_table", torch.int32, (s.batch, s.max_pages_per_seq)),
        _dev(seq_lens, "seq_lens", torch.int32, (s.batch,)),
        u, ctypes.byref(sel.c()), float(alpha),
        _dev(out, "out", torch.float32, (s.batch, s.num_q_heads, s.head_dim)),
        _dev(tau, "tau", torch.float32, (s.batch, s.num_q_heads), optional=True),
        _dev(sel_idx, "sel_idx", torch.int32, (s.batch, s.num_kv_heads, cap), optional=True),
        _dev(sel_count, "sel_count", torch.int32, (s.batch, s.num_kv_heads), optional=True),
        wp, wn, _stream(stream)))


# ----------------------------------------------------------------------------
# dropped mass on the device (token unit)
# ----------------------------------------------------------------------------

def dropped_mass(shape: Shape, seq_lens, block_table, token_logits, sel_idx, sel_count, delta,
                 stream=None):
    """delta [B, H_q] fp32 from the stored token logits and a kept token list
    (sel_idx [B, H_kv, k_max], sel_count [B, H_kv])."""
    s = shape
    if sel_idx.dim() != 3:
        raise ValueError("sel_idx must be [B, H_kv, k_max]")
    k_max = int(sel_idx.shape[2])
    _check(lib().sd_dropped_mass(
        ctypes.byref(s.c()),
        _dev(seq_lens, "seq_lens", torch.int32, (s.batch,)),
        _dev(block_table, "block_table", torch.int32, (s.batch, s.max_pages_per_seq)),
        _dev(token_logits, "token_logits", torch.float32, (s.batch, s.num_q_heads, s.max_seq_len)),
        _dev(sel_idx, "sel_idx", torch.int32, (s.batch, s.num_kv_heads, k_max)),
        _dev(sel_count, "sel_count", torch.int32, (s.batch, s.num_kv_heads)),
        k_max,
        _dev(delta, "delta", torch.float32, (s.batch, s.num_q_heads)),
        _stream(stream)))
