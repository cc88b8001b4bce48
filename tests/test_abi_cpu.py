"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments on the host before anything is launched (no GPU needed)."""
import ctypes
import os
import re

import pytest

from retention_scored_decode_amd import trimkv as tk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared():
    src = open(os.path.join(ROOT, "include", "trimkv.h")).read()
    return sorted(set(re.findall(r"^\S.*?\b(trimkv_\w+)\(", src, re.M)))


def test_exports_every_declared_symbol():
    names = declared()
    assert len(names) == 22
    L = tk.lib()
    for n in names:
        assert hasattr(L, n), n
    assert sorted(tk.EXPORTS) == names


def fake_cache(n_heads=4, head_dim=128, dtype=tk.BF16, n_pages=64, page_size=16, nulls=()):
    f = dict(k=0x1000, v=0x2000, meta=0x3000, page_off=0x5000, page_ids=0x6000, len=0x7000)
    for n in nulls:
        f[n] = None
    return tk.CacheStruct(n_heads, head_dim, page_size, dtype, n_pages, f["k"], f["v"], f["meta"],
                          f["page_off"], f["page_ids"], f["len"])


P = ctypes.c_void_p
X = P(0x8000)


def test_strerror():
    assert tk.strerror(0) == "ok"
    assert "workspace" in tk.strerror(tk.EWORKSPACE)


def test_unsupported_shapes():
    L = tk.lib()
    for kw in (dict(page_size=8), dict(head_dim=96), dict(dtype=7)):
        c = fake_cache(**kw)
        assert L.trimkv_score(ctypes.byref(c), 1, X, X, X, None) == tk.EUNSUPPORTED
    c = fake_cache()
    assert L.trimkv_decode_attn(ctypes.byref(c), None, None, X, 17, ctypes.c_float(1.0), X, X, None, X, 1 << 30,
                                None) == tk.EUNSUPPORTED
    assert L.trimkv_decode_attn(ctypes.byref(c), None, None, X, 0, ctypes.c_float(1.0), X, X, None, X, 1 << 30,
                                None) == tk.EUNSUPPORTED


def test_null_and_inconsistent_arguments():
    L = tk.lib()
    c = fake_cache()
    assert L.trimkv_score(None, 1, X, X, X, None) == tk.EINVAL
    assert L.trimkv_score(ctypes.byref(c), 0, X, X, X, None) == tk.EINVAL
    assert L.trimkv_score(ctypes.byref(c), 1, None, X, X, None) == tk.EINVAL
    assert L.trimkv_log_beta(None, None, 5, 16, None) == tk.EINVAL
    assert L.trimkv_log_beta(X, X, -1, 16, None) == tk.EINVAL
    assert L.trimkv_log_beta(X, X, 5, 8, None) == tk.EINVAL
    # keep and lse_ref together
    assert L.trimkv_decode_attn(ctypes.byref(c), X, X, X, 4, ctypes.c_float(1.0), X, X, None, X, 1 << 30,
                                None) == tk.EINVAL
    assert L.trimkv_select_global(ctypes.byref(c), X, 5, X, X, X, X, None, None, X, 1 << 30, None) == tk.EINVAL
    bad = fake_cache(nulls=("page_off",))
    assert L.trimkv_select_global(ctypes.byref(bad), X, 1, X, X, X, X, None, None, X, 1 << 30, None) == tk.EINVAL
    assert L.trimkv_allocate(X, X, 0, 10, None, X, None) == tk.EINVAL
    assert L.trimkv_allocate(X, X, 4, -1, None, X, None) == tk.EINVAL
    assert L.trimkv_append(ctypes.byref(c), None, X, X, X, None, None) == tk.EINVAL


def test_decode_err_argument_checks():
    """trimkv_decode_attn_err: mask mode only (keep and err required), bf16
    caches only, its own workspace (the decode workspace plus a second set of
    partial outputs)."""
    L = tk.lib()
    c = fake_cache()
    F = ctypes.c_float(1.0)
    need = L.trimkv_workspace_size(tk.OP_DECODE_ERR, ctypes.byref(c), 0, 4)
    assert need > L.trimkv_workspace_size(tk.OP_DECODE_ATTN, ctypes.byref(c), 0, 4)
    assert L.trimkv_decode_attn_err(ctypes.byref(c), None, X, 4, F, X, X, None, X, X, need, None) == tk.EINVAL
    assert L.trimkv_decode_attn_err(ctypes.byref(c), X, X, 4, F, X, X, None, None, X, need, None) == tk.EINVAL
    assert L.trimkv_decode_attn_err(ctypes.byref(c), X, X, 4, F, X, X, None, X, X, need - 1, None) == tk.EWORKSPACE
    assert L.trimkv_decode_attn_err(ctypes.byref(c), X, X, 17, F, X, X, None, X, X, need, None) == tk.EUNSUPPORTED
    f32 = fake_cache(dtype=tk.F32, head_dim=64)
    assert L.trimkv_decode_attn_err(ctypes.byref(f32), X, X, 4, F, X, X, None, X, X, 1 << 30, None) == \
        tk.EUNSUPPORTED
    odd = ctypes.c_void_p(0x10008)
    assert L.trimkv_decode_attn_err(ctypes.byref(c), odd, X, 4, F, X, X, None, X, X, need, None) == tk.EINVAL


def test_gated_argument_checks():
    """trimkv_decode_attn_gated: segment list and t required (as
    trimkv_score), bf16 caches only, the decode workspace."""
    L = tk.lib()
    c = fake_cache()
    F = ctypes.c_float(1.0)
    need = L.trimkv_workspace_size(tk.OP_DECODE_ATTN, ctypes.byref(c), 0, 4)
    g = L.trimkv_decode_attn_gated
    assert g(ctypes.byref(c), 1, X, X, None, X, 4, F, X, X, None, X, need - 1, None) == tk.EWORKSPACE
    assert g(ctypes.byref(c), 0, X, X, None, X, 4, F, X, X, None, X, need, None) == tk.EINVAL
    assert g(ctypes.byref(c), 5, X, X, None, X, 4, F, X, X, None, X, need, None) == tk.EINVAL
    assert g(ctypes.byref(c), 1, None, X, None, X, 4, F, X, X, None, X, need, None) == tk.EINVAL
    assert g(ctypes.byref(c), 1, X, None, None, X, 4, F, X, X, None, X, need, None) == tk.EINVAL
    assert g(ctypes.byref(c), 1, X, X, None, X, 4, F, X, None, None, X, need, None) == tk.EINVAL
    assert g(ctypes.byref(c), 1, X, X, ctypes.c_void_p(0x10008), X, 4, F, X, X, None, X, need, None) == tk.EINVAL
    assert g(ctypes.byref(c), 1, X, X, None, X, 17, F, X, X, None, X, need, None) == tk.EUNSUPPORTED
    f32 = fake_cache(dtype=tk.F32, head_dim=64)
    assert g(ctypes.byref(f32), 1, X, X, None, X, 4, F, X, X, None, X, 1 << 30, None) == tk.EUNSUPPORTED


def test_append_score_select_argument_checks():
    """trimkv_append_score_select: the append's inputs (as trimkv_append) and
    the fused selection's (as trimkv_score_select), the selection workspace."""
    L = tk.lib()
    c = fake_cache()
    need = L.trimkv_workspace_size(tk.OP_SELECT, ctypes.byref(c), 1, 0)
    f = L.trimkv_append_score_select
    args = [X, X, X, 1, X, X, X, X, X, X, None, None, None, X]
    for i in (0, 1, 2, 4, 5, 6, 7, 8, 9):   # every required pointer
        bad = list(args)
        bad[i] = None
        assert f(ctypes.byref(c), *bad, need, None) == tk.EINVAL, i
    for n_seg in (0, 5):
        bad = list(args)
        bad[3] = n_seg
        assert f(ctypes.byref(c), *bad, need, None) == tk.EINVAL, n_seg
    for i in (7, 8):   # score and keep: 16-byte aligned
        bad = list(args)
        bad[i] = ctypes.c_void_p(0x10008)
        assert f(ctypes.byref(c), *bad, need, None) == tk.EINVAL, i
    assert f(ctypes.byref(c), *args, need - 1, None) == tk.EWORKSPACE
    assert f(ctypes.byref(fake_cache(head_dim=96)), *args, 1 << 30, None) == tk.EUNSUPPORTED
    assert f(ctypes.byref(fake_cache(nulls=("k",))), *args, 1 << 30, None) == tk.EINVAL


def test_decode_attn_evict_tailfill_argument_checks():
    """trimkv_decode_attn_evict_tailfill: mask mode (keep and kept required),
    the eviction's table rules, its own workspace (the decode workspace plus
    the hole lists)."""
    L = tk.lib()
    c = fake_cache()
    F = ctypes.c_float(1.0)
    need = L.trimkv_workspace_size(tk.OP_DECODE_EVICT, ctypes.byref(c), 0, 4)
    assert need > L.trimkv_workspace_size(tk.OP_DECODE_ATTN, ctypes.byref(c), 0, 4)
    f = L.trimkv_decode_attn_evict_tailfill
    A, B, C, D = (ctypes.c_void_p(x) for x in (0x21000, 0x22000, 0x23000, 0x24000))
    args = [X, X, X, 4, F, X, X, 1, A, B, C, D, X]
    assert f(ctypes.byref(c), *args[:12], X, need - 1, None) == tk.EWORKSPACE
    for i in (0, 1, 2, 5, 6, 8, 9, 10, 11):
        bad = list(args)
        bad[i] = None
        assert f(ctypes.byref(c), *bad, need, None) == tk.EINVAL, i
    bad = list(args)
    bad[7] = -1
    assert f(ctypes.byref(c), *bad, need, None) == tk.EINVAL
    for i, alias in ((10, 0x5000), (11, 0x6000), (10, 0x21000), (11, 0x22000)):   # the new table aliases
        bad = list(args)
        bad[i] = ctypes.c_void_p(alias)
        assert f(ctypes.byref(c), *bad, need, None) == tk.EINVAL, (i, alias)
    bad = list(args)
    bad[0] = ctypes.c_void_p(0x10008)   # keep: 16-byte aligned
    assert f(ctypes.byref(c), *bad, need, None) == tk.EINVAL
    bad = list(args)
    bad[3] = 17
    assert f(ctypes.byref(c), *bad, need, None) == tk.EUNSUPPORTED
    huge = fake_cache(n_pages=1 << 28)
    assert f(ctypes.byref(huge), *args, 1 << 40, None) == tk.EUNSUPPORTED


def test_compact_inplace_argument_checks():
    """trimkv_compact_inplace: the new table must not alias the current or
    the home table; keep aligned; slots in 32 bits; its own small workspace."""
    L = tk.lib()
    c = fake_cache()
    need = L.trimkv_workspace_size(tk.OP_COMPACT_INPLACE, ctypes.byref(c), 0, 0)
    assert need >= 4 * 4
    f = L.trimkv_compact_inplace
    A, B, C, D = (ctypes.c_void_p(x) for x in (0x21000, 0x22000, 0x23000, 0x24000))
    assert f(ctypes.byref(c), X, None, 1, A, B, C, D, X, need - 1, None) == tk.EWORKSPACE
    assert f(ctypes.byref(c), X, None, -1, A, B, C, D, X, need, None) == tk.EINVAL
    assert f(ctypes.byref(c), None, None, 1, A, B, C, D, X, need, None) == tk.EINVAL
    assert f(ctypes.byref(c), X, None, 1, None, B, C, D, X, need, None) == tk.EINVAL
    assert f(ctypes.byref(c), X, None, 1, A, B, None, D, X, need, None) == tk.EINVAL
    assert f(ctypes.byref(c), X, None, 1, A, B, ctypes.c_void_p(0x5000), D, X, need, None) == tk.EINVAL  # page_off
    assert f(ctypes.byref(c), X, None, 1, A, B, C, ctypes.c_void_p(0x6000), X, need, None) == tk.EINVAL  # page_ids
    assert f(ctypes.byref(c), X, None, 1, A, B, A, D, X, need, None) == tk.EINVAL
    assert f(ctypes.byref(c), ctypes.c_void_p(0x10008), None, 1, A, B, C, D, X, need, None) == tk.EINVAL
    huge = fake_cache(n_pages=1 << 28)
    assert f(ctypes.byref(huge), X, None, 1, A, B, C, D, X, 1 << 20, None) == tk.EUNSUPPORTED


def test_recency_floor_argument_checks():
    L = tk.lib()
    assert L.trimkv_allocate_floor(X, X, 4, 10, -1, None, X, None) == tk.EINVAL
    assert L.trimkv_allocate_floor(X, X, 0, 10, 4, None, X, None) == tk.EINVAL
    assert L.trimkv_allocate_floor(X, X, 4, -1, 4, None, X, None) == tk.EINVAL
    assert L.trimkv_allocate_floor(X, X, 4, 10, 4, None, None, None) == tk.EINVAL
    c = fake_cache()
    assert L.trimkv_mark_recent(ctypes.byref(c), -1, X, None) == tk.EINVAL
    assert L.trimkv_mark_recent(ctypes.byref(c), 4, None, None) == tk.EINVAL
    assert L.trimkv_mark_recent(ctypes.byref(fake_cache(page_size=8)), 4, X, None) == tk.EUNSUPPORTED


def test_workspace_checks():
    L = tk.lib()
    c = fake_cache()
    need = L.trimkv_workspace_size(tk.OP_SELECT, ctypes.byref(c), 1, 0)
    assert need > 0
    assert L.trimkv_select_global(ctypes.byref(c), X, 1, X, X, X, X, None, None, X, need - 1, None) == tk.EWORKSPACE
    assert L.trimkv_select_global(ctypes.byref(c), X, 1, X, X, X, X, None, None, None, need, None) == tk.EWORKSPACE
    need = L.trimkv_workspace_size(tk.OP_DECODE_ATTN, ctypes.byref(c), 0, 4)
    assert L.trimkv_decode_attn(ctypes.byref(c), None, None, X, 4, ctypes.c_float(1.0), X, X, None, X, need - 1,
                                None) == tk.EWORKSPACE
    # bf16 decode workspace: partials of a bounded number of waves (+ heads), growing with heads and group;
    # fp32 work lists and the mass logits grow with the pool
    big = fake_cache(n_pages=1 << 16)
    assert L.trimkv_workspace_size(tk.OP_DECODE_ATTN, ctypes.byref(big), 0, 4) == need
    assert L.trimkv_workspace_size(tk.OP_DECODE_ATTN, ctypes.byref(fake_cache(n_heads=512)), 0, 4) > need
    assert L.trimkv_workspace_size(tk.OP_DECODE_ATTN, ctypes.byref(c), 0, 8) > need
    f32 = fake_cache(dtype=tk.F32, head_dim=64)
    f32big = fake_cache(dtype=tk.F32, head_dim=64, n_pages=1 << 16)
    assert L.trimkv_workspace_size(tk.OP_DECODE_ATTN, ctypes.byref(f32big), 0, 4) > \
        L.trimkv_workspace_size(tk.OP_DECODE_ATTN, ctypes.byref(f32), 0, 4)
    assert L.trimkv_workspace_size(tk.OP_ATTN_MASS, ctypes.byref(big), 0, 4) > \
        L.trimkv_workspace_size(tk.OP_ATTN_MASS, ctypes.byref(c), 0, 4)
    assert L.trimkv_workspace_size(99, ctypes.byref(c), 0, 0) == 0


def test_compact_capacity_and_compatibility():
    L = tk.lib()
    src = fake_cache(n_heads=4, n_pages=64)
    ws = L.trimkv_workspace_size(tk.OP_COMPACT, ctypes.byref(src), 0, 0)
    # need ceil((100 + 4*1)/16) + 4 = 11 pages
    small = tk.CacheStruct(4, 128, 16, tk.BF16, 10, 0x11000, 0x12000, 0x13000, 0x15000, 0x16000, 0x17000)
    ok = tk.CacheStruct(4, 128, 16, tk.BF16, 11, 0x11000, 0x12000, 0x13000, 0x15000, 0x16000, 0x17000)
    assert L.trimkv_compact(ctypes.byref(src), X, None, 1, 100, ctypes.byref(small), X, X, ws, None) == tk.ECAPACITY
    other = tk.CacheStruct(4, 64, 16, tk.BF16, 11, 0x11000, 0x12000, 0x13000, 0x15000, 0x16000, 0x17000)
    assert L.trimkv_compact(ctypes.byref(src), X, None, 1, 100, ctypes.byref(other), X, X, ws, None) == tk.EINVAL
    assert L.trimkv_compact(ctypes.byref(src), X, None, -1, 100, ctypes.byref(ok), X, X, ws, None) == tk.EINVAL
    assert L.trimkv_compact(ctypes.byref(src), X, None, 1, 100, ctypes.byref(ok), X, X, ws - 1, None) == tk.EWORKSPACE
    # aliasing source and destination pools
    assert L.trimkv_compact(ctypes.byref(src), X, None, 1, 100, ctypes.byref(src), X, X, ws, None) in (tk.EINVAL,
                                                                                                   tk.ECAPACITY)


def test_keep_plane_alignment_and_slot_width():
    L = tk.lib()
    src = fake_cache(n_heads=4, n_pages=64)
    ok = tk.CacheStruct(4, 128, 16, tk.BF16, 11, 0x11000, 0x12000, 0x13000, 0x15000, 0x16000, 0x17000)
    ws = L.trimkv_workspace_size(tk.OP_COMPACT, ctypes.byref(src), 0, 0)
    odd = ctypes.c_void_p(0x1008)   # keep planes start on 16-byte boundaries
    assert L.trimkv_compact(ctypes.byref(src), odd, None, 1, 100, ctypes.byref(ok), X, X, ws, None) == tk.EINVAL
    need = L.trimkv_workspace_size(tk.OP_DECODE_ATTN, ctypes.byref(src), 0, 4)
    assert L.trimkv_decode_attn(ctypes.byref(src), odd, None, X, 4, ctypes.c_float(1.0), X, X, None, X, need,
                                None) == tk.EINVAL
    need = L.trimkv_workspace_size(tk.OP_SELECT, ctypes.byref(src), 1, 0)
    assert L.trimkv_select_global(ctypes.byref(src), X, 1, X, X, odd, X, None, None, X, need, None) == tk.EINVAL
    # compaction carries slots in 32 bits
    huge = fake_cache(n_heads=4, n_pages=1 << 28)
    big_ws = L.trimkv_workspace_size(tk.OP_COMPACT, ctypes.byref(huge), 0, 0)
    dst = tk.CacheStruct(4, 128, 16, tk.BF16, 11, 0x11000, 0x12000, 0x13000, 0x15000, 0x16000, 0x17000)
    assert L.trimkv_compact(ctypes.byref(huge), X, None, 1, 100, ctypes.byref(dst), X, X, big_ws,
                            None) == tk.EUNSUPPORTED


def test_profile_hook_arguments():
    L = tk.lib()
    assert L.trimkv_profile_next(None, None) == tk.OK
    assert L.trimkv_profile_next(X, None) == tk.EINVAL
    assert L.trimkv_profile_next(None, X) == tk.EINVAL


def test_build_rejects_kernels_with_scratch():
    from retention_scored_decode_amd.build import scratch_users
    rep = "\n".join([
        "x.hip:9:1: remark: Function Name: k_a [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:9:1: remark:     VGPRs: 64 [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:9:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:20:1: remark: Function Name: k_b [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:20:1: remark:     ScratchSize [bytes/lane]: 60 [-Rpass-analysis=kernel-resource-usage]",
    ])
    assert scratch_users(rep) == [("k_b", 60)]
    assert scratch_users(rep.replace(": 60 ", ": 0 ")) == []


def test_noalloc_decode_rejects_calls_beyond_its_scratch():
    """The allocation-free decode refuses, before any device call, a cache
    whose partials cannot fit the static scratch, and checks its arguments
    as the workspace variant does."""
    L = tk.lib()
    big = fake_cache(n_heads=1 << 20, n_pages=1 << 22)
    f = lambda c, g=4, keep=None, lse=None, q=X: L.trimkv_decode_attn_noalloc(
        ctypes.byref(c), keep, lse, q, g, ctypes.c_float(0.1), X, X, None, None)
    assert f(big) == tk.EWORKSPACE
    c = fake_cache()
    assert f(c, g=17) == tk.EUNSUPPORTED
    assert f(c, q=None) == tk.EINVAL
    assert f(c, keep=X, lse=X) == tk.EINVAL
    assert f(fake_cache(head_dim=96)) == tk.EUNSUPPORTED
