"""Helpers shared by the GPU parity tests: upload seeded synthetic caches,
run the HIP path through the C ABI, and build the oracle's per-head view of
the same bytes.  Nothing here computes a step of the method."""
from __future__ import annotations

import math

import numpy as np
import torch

import synth
from oracle import reference as ref
from retention_scored_decode_amd import trimkv as tk

OUT_TOL = 2e-3       # max-abs error of attention outputs vs the float64 oracle
DROP_TOL = 1e-5      # absolute error of the dropped mass


def cuda(a, dtype=None):
    a = np.ascontiguousarray(a)
    return torch.from_numpy(a).to("cuda") if dtype is None else torch.from_numpy(a.astype(dtype)).to("cuda")


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda").view(torch.bfloat16)


def kv_dev(a: np.ndarray, dtype: str) -> torch.Tensor:
    return bf16_dev(a) if dtype == "bf16" else cuda(a, np.float32)


def kv_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    return (synth.bf16_bits_to_f32(a) if dtype == "bf16" else a).astype(np.float64)


def upload(pc: synth.PagedCache) -> tk.Cache:
    """Device copy of a host cache; ln(beta) computed on the GPU (a0) straight
    into the cache's metadata blocks."""
    meta = torch.zeros((pc.n_pages, 2, 16), dtype=torch.int32, device="cuda")
    meta[:, 1, :] = cuda(pc.pos, np.int32)
    tk.log_beta(cuda(pc.beta, np.float32), meta, out_page_stride=32)
    return tk.Cache(kv_dev(pc.k, pc.dtype), kv_dev(pc.v, pc.dtype), meta, cuda(pc.page_off, np.int32),
                    cuda(pc.page_ids, np.int32), cuda(pc.length, np.int32))


class OracleView:
    """Per-head, slot-ordered arrays of a host cache, as the oracle sees it."""

    def __init__(self, pc: synth.PagedCache):
        po, pi, ln = pc.page_off, pc.page_ids, pc.length
        self.pc = pc
        self.lnb = [ref.ln_beta(b) for b in ref.gather_heads(pc.beta, po, pi, ln)]
        self.pos = ref.gather_heads(pc.pos, po, pi, ln)
        self.k_raw = ref.gather_heads(pc.k, po, pi, ln)
        self.v_raw = ref.gather_heads(pc.v, po, pi, ln)
        self.k = [kv_f64(x, pc.dtype) for x in self.k_raw]
        self.v = [kv_f64(x, pc.dtype) for x in self.v_raw]

    def scores(self, t_of_head):
        return [ref.score_f32(self.lnb[h], t_of_head[h], self.pos[h]) for h in range(len(self.pos))]


def plane_from_heads(per_head, page_off, length, n_pages, fill=np.nan, dtype=np.float32):
    plane = np.full(n_pages * synth.PAGE, fill, dtype=dtype)
    for h, x in enumerate(per_head):
        plane[ref.head_csr_slots(page_off, length, h)] = x
    return plane


def heads_from_plane(plane, page_off, length):
    return ref.csr_plane_to_heads(np.asarray(plane).reshape(-1), page_off, length)


def seg_t(seg_head_begin, t_per_seg, n_heads):
    t = np.zeros(n_heads, np.int64)
    for s in range(len(seg_head_begin) - 1):
        t[seg_head_begin[s]:seg_head_begin[s + 1]] = t_per_seg[s]
    return t


def dst_capacity(n_heads, max_kept, reserve):
    return -(-(max_kept + n_heads * reserve) // synth.PAGE) + n_heads


def download_cache(c: tk.Cache):
    """Host copies of a device cache: (page_off, page_ids, len, k, v, lnb, pos)."""
    f = lambda t: t.cpu().numpy()
    k = c.k.view(torch.int16).cpu().numpy().view(np.uint16) if c.k.dtype == torch.bfloat16 else f(c.k)
    v = c.v.view(torch.int16).cpu().numpy().view(np.uint16) if c.v.dtype == torch.bfloat16 else f(c.v)
    meta = f(c.meta)
    lnb = np.ascontiguousarray(meta[:, 0, :]).view(np.float32)
    pos = np.ascontiguousarray(meta[:, 1, :])
    return f(c.page_off), f(c.page_ids), f(c.length), k, v, lnb, pos


def f32_bits(a):
    return np.asarray(a, np.float32).view(np.uint32)


def scale_of(d):
    return 1.0 / math.sqrt(d)


def decode_by_heads(kv_of, q64, group, scale, dtype, heads, keep_of=None, lse_ref=None, gate_of=None, batch=32):
    """The float64 oracle's decode attention over many heads, a batch of heads
    at a time so that only one batch's float64 K and V are held.  kv_of(h)
    gives head h's raw K and V rows (cache dtype), keep_of(h) its keep mask
    (None: every row); lse_ref is indexed by query row; gate_of(h), if given,
    head h's ln r per row (retention-gated attention).  Returns out, dropped
    and LSE for the query rows of `heads`, in order."""
    outs, drops, lses = [], [], []
    for i in range(0, len(heads), batch):
        hs = heads[i:i + batch]
        K, V = [], []
        for h in hs:
            k, v = kv_of(h)
            K.append(kv_f64(k, dtype))
            V.append(kv_f64(v, dtype))
        rows = np.concatenate([np.arange(h * group, (h + 1) * group) for h in hs])
        keep = None if keep_of is None else [keep_of(h) for h in hs]
        if gate_of is not None:
            o, d, l = ref.decode_attn_gated(K, V, q64[rows], group, scale, [gate_of(h) for h in hs], keep=keep)
        else:
            o, d, l = ref.decode_attn(K, V, q64[rows], group, scale, keep=keep,
                                      lse_ref=None if lse_ref is None else lse_ref[rows])
        outs.append(o)
        drops.append(d)
        lses.append(l)
    return np.concatenate(outs), np.concatenate(drops), np.concatenate(lses)
