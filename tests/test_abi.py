"""The C ABI without a GPU: the library loads, exports every entry point
include/sd.h declares, and rejects bad host-visible arguments with the
documented status before touching the device."""

import ctypes
import os
import re

import pytest

import sparse_kv_cache_sd_amd as sd
from sparse_kv_cache_sd_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "sd.h")


def declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"SD_API\s+[\w\s\*]+?\b(sd_\w+)\s*\(", text)))


def test_header_and_binding_agree():
    names = declared()
    assert len(names) >= 10
    assert sorted(_lib.EXPORTS) == names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(sd.LIB_PATH)
    for name in declared():
        assert hasattr(lib, name), name


@pytest.mark.parametrize("r,U,k", [(0.3, 2048, 615), (0.07, 100, 7), (0.05, 16384, 820),
                                   (1.0, 9, 9), (2.0, 9, 9), (1e-9, 50, 1)])
def test_keep_count_matches_rule(r, U, k):
    assert sd.keep_count(r, U) == k


def test_keep_count_rejects():
    assert sd.lib().sd_keep_count(0.0, 10) == -1
    assert sd.lib().sd_keep_count(float("nan"), 10) == -1
    assert sd.lib().sd_keep_count(0.5, 0) == -1


def _shape(**kw):
    base = dict(batch=1, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16,
                max_pages_per_seq=2048, max_seq_len=32768, dtype="bf16", num_pages=2048)
    base.update(kw)
    return sd.Shape(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), 6), (dict(page_size=32), 6), (dict(num_q_heads=48), 6),
    (dict(num_q_heads=30), 2), (dict(max_seq_len=40000), 2), (dict(batch=0), 2),
    (dict(num_pages=0), 2),
])
def test_shape_validation(kw, status):
    with pytest.raises(sd.SdError) as e:
        sd.workspace_bytes(_shape(**kw), "page", 0.3)
    assert e.value.status == status


def test_ratio_and_unit_validation():
    with pytest.raises(sd.SdError) as e:
        sd.workspace_bytes(_shape(), "page", 0.0)
    assert e.value.status == 4
    n = ctypes.c_size_t()
    st = sd.lib().sd_workspace_bytes(ctypes.byref(_shape().c()), 7, 0.3, ctypes.byref(n))
    assert st == 2


def test_workspace_grows_with_selection_buffers():
    s = _shape()
    page = sd.workspace_bytes(s, "page", 0.3)
    tok = sd.workspace_bytes(s, "token", 0.3)
    assert tok > page > 0


def test_null_pointers_rejected_before_any_launch():
    lib = sd.lib()
    sh = ctypes.byref(_shape().c())
    st = lib.sd_decode_step(sh, None, None, None, None, None, None, 1, 0.3, None, None, None,
                            None, None, 0, None)
    assert st == 1 and b"required" in lib.sd_last_error()
    st = lib.sd_attend_splitk(sh, None, None, None, None, None, 1, None, None, 0, None, None,
                              None, None, 0, None)
    assert st == 1
    st = lib.sd_select_topk(sh, 1, None, None, 0.3, None, None, None, 0, None)
    assert st == 1
    st = lib.sd_merge_splits(sh, None, None, None, 0, None)
    assert st == 1


def test_workspace_size_and_alignment_checked():
    lib = sd.lib()
    sh = ctypes.byref(_shape().c())
    fake = ctypes.c_void_p(0x10000)       # never dereferenced: validation fails first
    st = lib.sd_merge_splits(sh, fake, fake, ctypes.c_void_p(0x10010), 1 << 30, None)
    assert st == 5 and b"aligned" in lib.sd_last_error()
    st = lib.sd_merge_splits(sh, fake, fake, ctypes.c_void_p(0x10000), 16, None)
    assert st == 5 and b"smaller" in lib.sd_last_error()


def test_entmax_validation_before_any_launch():
    lib = sd.lib()
    sh = ctypes.byref(_shape().c())
    sel = ctypes.byref(sd.Selection("topk", 0.3).c())
    for bad in (1.0, 0.5, 2.01, float("nan"), float("inf")):
        st = lib.sd_decode_step_entmax(sh, None, None, None, None, None, None, 1, sel, bad, None,
                                       None, None, None, None, 0, None)
        assert st == 4 and b"alpha" in lib.sd_last_error()
    st = lib.sd_decode_step_entmax(sh, None, None, None, None, None, None, 1, sel, 1.5, None,
                                   None, None, None, None, 0, None)
    assert st == 1 and b"required" in lib.sd_last_error()
    fake = ctypes.c_void_p(0x10000)       # never dereferenced: validation fails first
    st = lib.sd_decode_step_entmax(sh, fake, fake, fake, fake, fake, fake, 1, sel, 1.5, fake,
                                   None, None, None, ctypes.c_void_p(0x10000), 16, None)
    assert st == 5 and b"smaller" in lib.sd_last_error()


@pytest.mark.parametrize("n", [8192, 8193, 131072, 1 << 20])
def test_budget_workspace_past_one_block(n):
    # every length is accepted; past 8192 tokens the budget's many-block
    # scratch (per-slice partials and the pass histograms: at least
    # (1 + G) * 256 u64 per (b, g) and pass) is added to the top-k's
    s = _shape(max_pages_per_seq=n // 16 + 1, max_seq_len=n, num_pages=n // 16 + 1)
    top = sd.workspace_bytes_sel(s, "token", sd.Selection("topk", 0.5))
    bud = sd.workspace_bytes_sel(s, "token", sd.Selection("mass_budget", 0.5, max_dropped=0.1))
    hist = 4 * 8 * (1 + 4) * 256 * 8
    if n <= 8192:
        assert bud == top
    else:
        assert bud >= top + hist


def test_entmax_kept_slots_limit():
    # the thresholds take at most 1024 chunks of 16384 kept slots per head
    def shp(n):
        return sd.Shape(batch=1, num_q_heads=8, num_kv_heads=8, head_dim=64, page_size=64,
                        max_pages_per_seq=n // 64 + 1, max_seq_len=n, dtype="bf16",
                        num_pages=n // 64 + 1)
    dense = sd.Selection("topk", 1.0)
    assert sd.workspace_bytes_entmax(shp(1024 * 16384), "token", dense) > 0
    with pytest.raises(sd.SdError) as e:
        sd.workspace_bytes_entmax(shp(1024 * 16384 + 1), "token", dense)
    assert "UNSUPPORTED" in str(e.value)


def test_entmax_workspace_holds_logits_and_thresholds():
    s = _shape()
    for unit in ("page", "token"):
        sel = sd.Selection("topk", 0.3)
        ent = sd.workspace_bytes_entmax(s, unit, sel)
        soft = sd.workspace_bytes_sel(s, unit, sel)
        extra = 2 * 4 * s.batch * s.num_q_heads       # thresholds and lse
        if unit == "page":
            extra += 4 * s.batch * s.num_q_heads * s.max_seq_len   # logits of kept tokens
        assert ent >= soft + extra


def test_dropped_mass_validation_before_any_launch():
    lib = sd.lib()
    sh = ctypes.byref(_shape().c())
    fake = ctypes.c_void_p(0x10000)       # never dereferenced: validation fails first
    st = lib.sd_dropped_mass(sh, None, fake, fake, fake, fake, 4, fake, None)
    assert st == 1 and b"required" in lib.sd_last_error()
    st = lib.sd_dropped_mass(sh, fake, fake, fake, fake, fake, 0, fake, None)
    assert st == 2
    big = ctypes.byref(_shape(max_pages_per_seq=32768, max_seq_len=300000, num_pages=32768).c())
    st = lib.sd_dropped_mass(big, fake, fake, fake, fake, fake, 4, fake, None)
    assert st == 6


def test_page_bounds_list_arguments():
    """An empty page list is accepted and enqueues nothing; a negative count
    is refused; the append form needs max_appended in [1, max_seq_len]."""
    s = _shape()
    p = ctypes.c_void_p(16)     # never dereferenced: nothing is enqueued
    f = sd.lib().sd_update_page_bounds
    assert f(ctypes.byref(s.c()), p, p, p, p, 0, p, None) == 0
    assert f(ctypes.byref(s.c()), p, p, p, p, -1, p, None) == 2
    g = sd.lib().sd_append_page_bounds
    assert g(ctypes.byref(s.c()), p, p, p, p, 0, p, None) == 2
    assert g(ctypes.byref(s.c()), p, p, p, p, 32769, p, None) == 2
    assert g(ctypes.byref(s.c()), p, p, p, None, 1, p, None) == 1


def test_noalloc_refuses_shapes_past_the_static_scratch():
    """The allocation-free step refuses, before touching the device, a shape
    whose scratch exceeds its static 32 MiB (1M tokens in token unit)."""
    s = _shape(num_q_heads=64, max_pages_per_seq=16384, max_seq_len=1 << 20, num_pages=16384,
               page_size=64)
    assert sd.workspace_bytes(s, "token", 0.05) > 32 << 20
    p = ctypes.c_void_p(16)     # never dereferenced: the call is refused on the host
    st = sd.lib().sd_decode_step_noalloc(ctypes.byref(s.c()), p, p, p, None, p, p, 0,
                                         ctypes.c_double(0.05), p, p, None, None, None)
    assert st == 5
    assert b"static scratch" in sd.lib().sd_last_error()
