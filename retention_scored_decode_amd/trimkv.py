"""ctypes binding of libtrimkv.so: same names as the C ABI, argument
marshalling only.  Tensors are passed as device pointers (``data_ptr()``),
the stream is torch's current HIP stream unless one is given.  Every step of
the path runs in the library's HIP kernels; there is no Python or CPU
fallback: if the library is missing or the device is not a GPU, calls fail.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtrimkv.so")

PAGE = 16
F32, BF16 = 0, 1
OK, EINVAL, EUNSUPPORTED, EWORKSPACE, ECAPACITY, EHIP, EINVARIANT = 0, -1, -2, -3, -4, -5, -6
(OP_SCORE, OP_SELECT, OP_COMPACT, OP_DECODE_ATTN, OP_ATTN_MASS, OP_VALIDATE, OP_DECODE_ERR, OP_COMPACT_INPLACE,
 OP_EVICT_TAILFILL, OP_DECODE_EVICT) = range(10)

EXPORTS = ["trimkv_log_beta", "trimkv_score", "trimkv_select_global", "trimkv_compact",
           "trimkv_decode_attn", "trimkv_decode_attn_gated", "trimkv_decode_attn_err", "trimkv_attn_mass",
           "trimkv_decode_attn_noalloc", "trimkv_score_select", "trimkv_append_score_select", "trimkv_evict_tailfill",
           "trimkv_decode_attn_evict_tailfill",
           "trimkv_allocate", "trimkv_compact_inplace",
           "trimkv_allocate_floor", "trimkv_mark_recent", "trimkv_append",
           "trimkv_workspace_size", "trimkv_validate_cache", "trimkv_strerror", "trimkv_profile_next"]


class TrimkvError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__("%s failed: %s (%d)" % (what, strerror(status), status))
        self.status = status


class CacheStruct(ctypes.Structure):
    _fields_ = [("n_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("n_pages", ctypes.c_int64),
                ("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("meta", ctypes.c_void_p),
                ("page_off", ctypes.c_void_p), ("page_ids", ctypes.c_void_p), ("len", ctypes.c_void_p)]


_lib = None


def lib():
    """Load libtrimkv.so (built in place by retention_scored_decode_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libtrimkv.so is not built: run `python -m retention_scored_decode_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        cp = ctypes.POINTER(CacheStruct)
        sig = {
            "trimkv_log_beta": [vp, vp, i64, i32, vp],
            "trimkv_score": [cp, i32, vp, vp, vp, vp],
            "trimkv_select_global": [cp, vp, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp],
            "trimkv_compact": [cp, vp, vp, i32, i64, cp, vp, vp, sz, vp],
            "trimkv_score_select": [cp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
            "trimkv_append_score_select": [cp, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
            "trimkv_compact_inplace": [cp, vp, vp, i32, vp, vp, vp, vp, vp, sz, vp],
            "trimkv_evict_tailfill": [cp, vp, vp, i32, vp, vp, vp, vp, vp, sz, vp],
            "trimkv_decode_attn_evict_tailfill": [cp, vp, vp, vp, i32, ctypes.c_float, vp, vp, i32, vp, vp, vp, vp,
                                                  vp, sz, vp],
            "trimkv_decode_attn": [cp, vp, vp, vp, i32, ctypes.c_float, vp, vp, vp, vp, sz, vp],
            "trimkv_decode_attn_noalloc": [cp, vp, vp, vp, i32, ctypes.c_float, vp, vp, vp, vp],
            "trimkv_decode_attn_err": [cp, vp, vp, i32, ctypes.c_float, vp, vp, vp, vp, vp, sz, vp],
            "trimkv_decode_attn_gated": [cp, i32, vp, vp, vp, vp, i32, ctypes.c_float, vp, vp, vp, vp, sz, vp],
            "trimkv_attn_mass": [cp, vp, i32, ctypes.c_float, vp, vp, vp, sz, vp],
            "trimkv_allocate": [vp, vp, i32, i64, vp, vp, vp],
            "trimkv_allocate_floor": [vp, vp, i32, i64, i32, vp, vp, vp],
            "trimkv_mark_recent": [cp, i32, vp, vp],
            "trimkv_append": [cp, vp, vp, vp, vp, vp, vp],
            "trimkv_workspace_size": [ctypes.c_int, cp, i32, i32],
            "trimkv_validate_cache": [cp, vp, vp, sz, vp],
            "trimkv_strerror": [ctypes.c_int],
            "trimkv_profile_next": [vp, vp],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        L.trimkv_workspace_size.restype = ctypes.c_size_t
        L.trimkv_strerror.restype = ctypes.c_char_p
        _lib = L
    return _lib


def strerror(status: int) -> str:
    return lib().trimkv_strerror(int(status)).decode()


def _p(t: Optional[torch.Tensor]):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _check(rc: int, what: str):
    if rc != OK:
        raise TrimkvError(rc, what)


class Cache:
    """A paged KV pool plus its page table, as device tensors.

    k, v [n_pages, 16, D] (torch.bfloat16 or float32); meta [n_pages, 2, 16]
    int32 (row 0: ln beta as fp32 bits, row 1: positions); page_off
    [n_heads + 1] i32, page_ids [n_pages] i32, length [n_heads] i32.
    """

    def __init__(self, k, v, meta, page_off, page_ids, length):
        self.k, self.v, self.meta = k, v, meta
        self.page_off, self.page_ids, self.length = page_off, page_ids, length
        self._s = None

    @classmethod
    def empty(cls, n_heads: int, n_pages: int, head_dim: int, dtype: torch.dtype, device="cuda"):
        return cls(torch.empty((n_pages, PAGE, head_dim), dtype=dtype, device=device),
                   torch.empty((n_pages, PAGE, head_dim), dtype=dtype, device=device),
                   torch.empty((n_pages, 2, PAGE), dtype=torch.int32, device=device),
                   torch.zeros(n_heads + 1, dtype=torch.int32, device=device),
                   torch.empty(n_pages, dtype=torch.int32, device=device),
                   torch.zeros(n_heads, dtype=torch.int32, device=device))

    @property
    def lnb(self) -> torch.Tensor:
        """[n_pages, 16] float32 view of the ln(beta) half of meta."""
        return self.meta[:, 0, :].view(torch.float32)

    @property
    def pos(self) -> torch.Tensor:
        """[n_pages, 16] int32 view of the positions half of meta."""
        return self.meta[:, 1, :]

    @property
    def n_heads(self) -> int:
        return int(self.length.shape[0])

    @property
    def n_pages(self) -> int:
        return int(self.k.shape[0])

    @property
    def head_dim(self) -> int:
        return int(self.k.shape[2])

    @property
    def dtype_code(self) -> int:
        return BF16 if self.k.dtype == torch.bfloat16 else F32

    def struct(self) -> CacheStruct:
        s = CacheStruct(self.n_heads, self.head_dim, PAGE, self.dtype_code, self.n_pages,
                        self.k.data_ptr(), self.v.data_ptr(), self.meta.data_ptr(),
                        self.page_off.data_ptr(), self.page_ids.data_ptr(), self.length.data_ptr())
        self._s = s
        return s


def workspace_size(op: int, cache: Cache, n_seg: int = 0, group: int = 0) -> int:
    return int(lib().trimkv_workspace_size(op, ctypes.byref(cache.struct()), n_seg, group))


def workspace(op: int, cache: Cache, n_seg: int = 0, group: int = 0) -> torch.Tensor:
    n = workspace_size(op, cache, n_seg, group)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=cache.k.device)


def log_beta(beta: torch.Tensor, lnb: torch.Tensor, out_page_stride: int = PAGE, stream=None):
    """lnb[(i // 16) * out_page_stride + i % 16] = ln(beta[i]); pass a cache's
    meta (and out_page_stride=32) to fill its ln(beta) half."""
    _check(lib().trimkv_log_beta(_p(beta), _p(lnb), beta.numel(), int(out_page_stride), _stream(stream)),
           "trimkv_log_beta")


def score(cache: Cache, seg_head_begin: torch.Tensor, t: torch.Tensor, out: torch.Tensor, stream=None):
    n_seg = seg_head_begin.numel() - 1
    _check(lib().trimkv_score(ctypes.byref(cache.struct()), n_seg, _p(seg_head_begin), _p(t), _p(out),
                              _stream(stream)), "trimkv_score")


def select_global(cache: Cache, score: torch.Tensor, seg_head_begin: torch.Tensor, budget: torch.Tensor,
                  keep: torch.Tensor, kept: torch.Tensor, keptsum: Optional[torch.Tensor] = None,
                  ws: Optional[torch.Tensor] = None, stream=None, status: Optional[torch.Tensor] = None):
    """status: optional int32 [1] device counter, incremented by timed-out waits."""
    n_seg = seg_head_begin.numel() - 1
    if ws is None:
        ws = workspace(OP_SELECT, cache, n_seg)
    _check(lib().trimkv_select_global(ctypes.byref(cache.struct()), _p(score), n_seg, _p(seg_head_begin),
                                      _p(budget), _p(keep), _p(kept), _p(keptsum), _p(status), _p(ws),
                                      ws.numel(), _stream(stream)), "trimkv_select_global")


def score_select(cache: Cache, seg_head_begin: torch.Tensor, t: torch.Tensor, budget: torch.Tensor,
                 score: torch.Tensor, keep: torch.Tensor, kept: torch.Tensor, keptsum: Optional[torch.Tensor] = None,
                 ws: Optional[torch.Tensor] = None, stream=None, status: Optional[torch.Tensor] = None):
    """score() and select_global() in one call (scores formed in the first pass)."""
    n_seg = seg_head_begin.numel() - 1
    if ws is None:
        ws = workspace(OP_SELECT, cache, n_seg)
    _check(lib().trimkv_score_select(ctypes.byref(cache.struct()), n_seg, _p(seg_head_begin), _p(t), _p(budget),
                                     _p(score), _p(keep), _p(kept), _p(keptsum), _p(status), _p(ws), ws.numel(),
                                     _stream(stream)), "trimkv_score_select")


def append_score_select(cache: Cache, k_new: torch.Tensor, v_new: torch.Tensor, beta_new: torch.Tensor,
                        seg_head_begin: torch.Tensor, t: torch.Tensor, budget: torch.Tensor, score: torch.Tensor,
                        keep: torch.Tensor, kept: torch.Tensor, keptsum: Optional[torch.Tensor] = None,
                        ws: Optional[torch.Tensor] = None, stream=None, append_status: Optional[torch.Tensor] = None,
                        select_status: Optional[torch.Tensor] = None):
    """append() then score_select() in one call (the new entries are written
    by the selection's first kernel)."""
    n_seg = seg_head_begin.numel() - 1
    if ws is None:
        ws = workspace(OP_SELECT, cache, n_seg)
    _check(lib().trimkv_append_score_select(ctypes.byref(cache.struct()), _p(k_new), _p(v_new), _p(beta_new), n_seg,
                                            _p(seg_head_begin), _p(t), _p(budget), _p(score), _p(keep), _p(kept),
                                            _p(keptsum), _p(append_status), _p(select_status), _p(ws), ws.numel(),
                                            _stream(stream)), "trimkv_append_score_select")


def compact(src: Cache, keep: torch.Tensor, reserve: int, max_kept_total: int, dst: Cache,
            pages_used: torch.Tensor, ws: Optional[torch.Tensor] = None, stream=None,
            kept: Optional[torch.Tensor] = None):
    if ws is None:
        ws = workspace(OP_COMPACT, src)
    _check(lib().trimkv_compact(ctypes.byref(src.struct()), _p(keep), _p(kept), int(reserve), int(max_kept_total),
                                ctypes.byref(dst.struct()), _p(pages_used), _p(ws), ws.numel(),
                                _stream(stream)), "trimkv_compact")


def compact_inplace(cache: Cache, keep: torch.Tensor, reserve: int, home_off: torch.Tensor,
                    home_ids: torch.Tensor, new_page_off: torch.Tensor, new_page_ids: torch.Tensor,
                    kept: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None, stream=None) -> Cache:
    """Evict in place; returns the new view (same pools and length tensor,
    the new page table)."""
    if ws is None:
        ws = workspace(OP_COMPACT_INPLACE, cache)
    _check(lib().trimkv_compact_inplace(ctypes.byref(cache.struct()), _p(keep), _p(kept), int(reserve),
                                        _p(home_off), _p(home_ids), _p(new_page_off), _p(new_page_ids),
                                        _p(ws), ws.numel(), _stream(stream)), "trimkv_compact_inplace")
    return Cache(cache.k, cache.v, cache.meta, new_page_off, new_page_ids, cache.length)


def evict_tailfill(cache: Cache, keep: torch.Tensor, reserve: int, home_off: torch.Tensor, home_ids: torch.Tensor,
                   new_page_off: torch.Tensor, new_page_ids: torch.Tensor, kept: Optional[torch.Tensor] = None,
                   ws: Optional[torch.Tensor] = None, stream=None) -> Cache:
    """Evict in place, moving only the kept entries that fill holes; returns
    the new view (same pools and length tensor, the new page table)."""
    if ws is None:
        ws = workspace(OP_EVICT_TAILFILL, cache)
    _check(lib().trimkv_evict_tailfill(ctypes.byref(cache.struct()), _p(keep), _p(kept), int(reserve),
                                       _p(home_off), _p(home_ids), _p(new_page_off), _p(new_page_ids),
                                       _p(ws), ws.numel(), _stream(stream)), "trimkv_evict_tailfill")
    return Cache(cache.k, cache.v, cache.meta, new_page_off, new_page_ids, cache.length)


def decode_attn_evict_tailfill(cache: Cache, keep: torch.Tensor, kept: torch.Tensor, q: torch.Tensor, group: int,
                               scale: float, out: torch.Tensor, dropped: torch.Tensor, reserve: int,
                               home_off: torch.Tensor, home_ids: torch.Tensor, new_page_off: torch.Tensor,
                               new_page_ids: torch.Tensor, ws: Optional[torch.Tensor] = None, stream=None) -> Cache:
    """Mask-mode decode_attn(), then evict_tailfill() of the same keep plane,
    the merge and the eviction in one launch; returns the new view."""
    if ws is None:
        ws = workspace(OP_DECODE_EVICT, cache, 0, group)
    _check(lib().trimkv_decode_attn_evict_tailfill(ctypes.byref(cache.struct()), _p(keep), _p(kept), _p(q), int(group),
                                                   ctypes.c_float(scale), _p(out), _p(dropped), int(reserve),
                                                   _p(home_off), _p(home_ids), _p(new_page_off), _p(new_page_ids),
                                                   _p(ws), ws.numel(), _stream(stream)),
           "trimkv_decode_attn_evict_tailfill")
    return Cache(cache.k, cache.v, cache.meta, new_page_off, new_page_ids, cache.length)


def decode_attn(cache: Cache, q: torch.Tensor, group: int, scale: float, out: torch.Tensor,
                dropped: torch.Tensor, keep: Optional[torch.Tensor] = None,
                lse_ref: Optional[torch.Tensor] = None, lse_out: Optional[torch.Tensor] = None,
                ws: Optional[torch.Tensor] = None, stream=None):
    if ws is None:
        ws = workspace(OP_DECODE_ATTN, cache, 0, group)
    _check(lib().trimkv_decode_attn(ctypes.byref(cache.struct()), _p(keep), _p(lse_ref), _p(q), int(group),
                                    float(scale), _p(out), _p(dropped), _p(lse_out), _p(ws), ws.numel(),
                                    _stream(stream)), "trimkv_decode_attn")


def decode_attn_noalloc(cache: Cache, q: torch.Tensor, group: int, scale: float, out: torch.Tensor,
                        dropped: torch.Tensor, keep: Optional[torch.Tensor] = None,
                        lse_ref: Optional[torch.Tensor] = None, lse_out: Optional[torch.Tensor] = None, stream=None):
    """decode_attn without a workspace (the library's static per-GPU scratch)."""
    _check(lib().trimkv_decode_attn_noalloc(ctypes.byref(cache.struct()), _p(keep), _p(lse_ref), _p(q), int(group),
                                            float(scale), _p(out), _p(dropped), _p(lse_out), _stream(stream)),
           "trimkv_decode_attn_noalloc")


def decode_attn_gated(cache: Cache, seg: torch.Tensor, t: torch.Tensor, q: torch.Tensor, group: int, scale: float,
                      out: torch.Tensor, dropped: torch.Tensor, keep: Optional[torch.Tensor] = None,
                      lse_out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None, stream=None):
    if ws is None:
        ws = workspace(OP_DECODE_ATTN, cache, 0, group)
    _check(lib().trimkv_decode_attn_gated(ctypes.byref(cache.struct()), int(seg.numel()) - 1, _p(seg), _p(t),
                                          _p(keep), _p(q), int(group), float(scale), _p(out), _p(dropped),
                                          _p(lse_out), _p(ws), ws.numel(), _stream(stream)),
           "trimkv_decode_attn_gated")


def decode_attn_err(cache: Cache, q: torch.Tensor, group: int, scale: float, keep: torch.Tensor,
                    out: torch.Tensor, dropped: torch.Tensor, err: torch.Tensor, mu: Optional[torch.Tensor] = None,
                    ws: Optional[torch.Tensor] = None, stream=None):
    if ws is None:
        ws = workspace(OP_DECODE_ERR, cache, 0, group)
    _check(lib().trimkv_decode_attn_err(ctypes.byref(cache.struct()), _p(keep), _p(q), int(group), float(scale),
                                        _p(out), _p(dropped), _p(mu), _p(err), _p(ws), ws.numel(),
                                        _stream(stream)), "trimkv_decode_attn_err")


def attn_mass(cache: Cache, q: torch.Tensor, group: int, scale: float, mass: torch.Tensor,
              lse_full: torch.Tensor, ws: Optional[torch.Tensor] = None, stream=None):
    if ws is None:
        ws = workspace(OP_ATTN_MASS, cache, 0, group)
    _check(lib().trimkv_attn_mass(ctypes.byref(cache.struct()), _p(q), int(group), float(scale), _p(mass),
                                  _p(lse_full), _p(ws), ws.numel(), _stream(stream)), "trimkv_attn_mass")


def allocate(keptsum: torch.Tensor, length: torch.Tensor, total_budget: int, budget_out: torch.Tensor,
             mbar_out: Optional[torch.Tensor] = None, stream=None):
    _check(lib().trimkv_allocate(_p(keptsum), _p(length), int(keptsum.numel()), int(total_budget),
                                 _p(mbar_out), _p(budget_out), _stream(stream)), "trimkv_allocate")


def allocate_floor(keptsum: torch.Tensor, length: torch.Tensor, total_budget: int, floor: int,
                   budget_out: torch.Tensor, mbar_out: Optional[torch.Tensor] = None, stream=None):
    _check(lib().trimkv_allocate_floor(_p(keptsum), _p(length), int(keptsum.numel()), int(total_budget), int(floor),
                                       _p(mbar_out), _p(budget_out), _stream(stream)), "trimkv_allocate_floor")


def mark_recent(cache: Cache, floor: int, plane: torch.Tensor, stream=None):
    _check(lib().trimkv_mark_recent(ctypes.byref(cache.struct()), int(floor), _p(plane), _stream(stream)),
           "trimkv_mark_recent")


def append(cache: Cache, k_new: torch.Tensor, v_new: torch.Tensor, beta_new: torch.Tensor, t: torch.Tensor,
           stream=None, status: Optional[torch.Tensor] = None):
    """status: optional int32 [1] device counter, incremented by the number
    of heads that had no free slot."""
    _check(lib().trimkv_append(ctypes.byref(cache.struct()), _p(k_new), _p(v_new), _p(beta_new), _p(t),
                               _p(status), _stream(stream)), "trimkv_append")


def profile_next(start, stop):
    """Arm the measurement hook: the next call's main kernel(s) are bracketed
    by the two torch.cuda.Event objects (already recorded once, so their
    handles exist), on that call's stream."""
    h = lambda e: None if e is None else ctypes.c_void_p(e.cuda_event)
    _check(lib().trimkv_profile_next(h(start), h(stop)), "trimkv_profile_next")


def validate_cache(cache: Cache, t: torch.Tensor, ws: Optional[torch.Tensor] = None, stream=None) -> int:
    if ws is None:
        ws = workspace(OP_VALIDATE, cache)
    return int(lib().trimkv_validate_cache(ctypes.byref(cache.struct()), _p(t), _p(ws), ws.numel(),
                                           _stream(stream)))
