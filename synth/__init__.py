"""Seeded synthetic inputs for retention-scored KV eviction and decode.

This module only draws random inputs and lays them out in the paged pool
format; it computes nothing the method computes (no logarithm of beta, no
score, no selection, no attention).  Both the HIP path (through the tests and
the benchmark) and the CPU oracle consume the exact bytes it produces.

Recipe (one per workload; all draws in float64, rounded to float32 with
round-to-nearest-even, then to bfloat16 with round-to-nearest-even for bf16
workloads):

* every random stream is a numpy ``Generator(PCG64(SeedSequence(seed,
  spawn_key=(stream, index))))`` so that any single head, query block or
  decode step can be regenerated on its own;
* beta per entry from the workload's distribution (a mixture picks its
  component per entry with one uniform draw);
* K and V ~ N(0, 1) per entry and channel; in the 8B/32K workload each
  (layer, KV head, channel) of K, and independently of V, is an outlier
  channel with probability 0.01 and is scaled by 8 before rounding;
* one query per Q head ~ N(0, 1) (scaled by 2 in the 128K workload);
* the physical page of every logical page is a seeded random permutation of
  the pool, so the page table is exercised.

The workloads follow the 7-8B-model, tens-of-thousands-token settings of the
pages: DBTrimKV (global budget, paged per-head layout), TRIM-KV (32K decode
throughput, 128K LongMemEval at 25% KV), ContourKV (dropped-mass allocation)
and IndexMem (RULER-16K at 90% eviction, 8B models).  They stand in for the
pages' benchmark suites, which are neither available nor reproduced.
"""
from __future__ import annotations

import dataclasses
import math
from fractions import Fraction
from typing import Optional

import numpy as np

PAGE = 16

# stream ids for SeedSequence spawn keys
S_BETA, S_K, S_V, S_Q, S_OUTLIER, S_PERM, S_STEP = range(7)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int            # independent sequences
    layers: int
    kv_heads: int         # KV heads per layer
    group: int            # Q heads per KV head
    head_dim: int
    ctx: int              # cached tokens per head before eviction
    dtype: str            # "f32" or "bf16"
    seed: int
    beta: tuple = ("beta", 5.0, 1.0)   # ("beta", a, b) | ("mix", w, (a1,b1), (a2,b2)) | None
    beta_block: Optional[tuple] = None  # (lo, hi, dist) positions [lo,hi) drawn from dist
    budget_frac: Optional[Fraction] = None   # per-segment budget as a fraction of entries
    budget_abs: Optional[int] = None         # per-segment absolute budget
    per_seq_segments: bool = False           # one segment per sequence
    outlier_p: float = 0.0
    outlier_scale: float = 1.0
    q_scale: float = 1.0
    reserve: int = 0                         # spare slots per head in the prefill pool
    steps: int = 0                           # streaming decode steps
    mass_topk: int = 0                       # per-head top-mass size (dropped-mass workload)

    @property
    def n_heads(self) -> int:
        return self.batch * self.layers * self.kv_heads

    @property
    def n_qheads(self) -> int:
        return self.n_heads * self.group

    @property
    def pages_per_head(self) -> int:
        return -(-(self.ctx + self.reserve) // PAGE)

    @property
    def n_pages(self) -> int:
        return self.n_heads * self.pages_per_head

    @property
    def t(self) -> int:
        """Decode step at which the prefill cache is scored (positions 0..t-1)."""
        return self.ctx

    @property
    def n_seg(self) -> int:
        return self.batch if self.per_seq_segments else 1

    def heads_per_seg(self) -> int:
        return self.n_heads // self.n_seg

    def seg_head_begin(self) -> np.ndarray:
        hps = self.heads_per_seg()
        return (np.arange(self.n_seg + 1, dtype=np.int64) * hps).astype(np.int32)

    def budget(self) -> int:
        """Per-segment budget.  Rounding: floor(p*N + 1/2) in exact rationals."""
        n = self.heads_per_seg() * self.ctx
        if self.budget_abs is not None:
            return int(self.budget_abs)
        if self.budget_frac is None:
            return n
        return int(math.floor(Fraction(self.budget_frac) * n + Fraction(1, 2)))

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


MIX_8B = ("mix", 0.7, (2.0, 2.0), (50.0, 1.0))

WORKLOADS = {
    # 2 layers x 2 KV heads x 2 Q heads, D 64, 512 tokens, fp32, budget 256
    "tiny": Workload("tiny", 1, 2, 2, 1, 64, 512, "f32", seed=1,
                     beta=("beta", 5.0, 1.0), budget_abs=256),
    # Llama-3.1-8B shape, one sequence, 32K tokens per head, 10% global budget
    "llama8b_32k": Workload("llama8b_32k", 1, 32, 8, 4, 128, 32768, "bf16", seed=2,
                            beta=MIX_8B, budget_frac=Fraction(1, 10),
                            outlier_p=0.01, outlier_scale=8.0),
    # 16 sequences of the Llama-3.1-8B shape, 16K tokens, 12.5% per-sequence budget
    "batched16_16k": Workload("batched16_16k", 16, 32, 8, 4, 128, 16384, "bf16", seed=3,
                              beta=MIX_8B, budget_frac=Fraction(1, 8),
                              per_seq_segments=True),
    # Qwen3-8B shape, 128K tokens, query x2, per-head top-1024 mass, 5% global budget
    "qwen8b_128k": Workload("qwen8b_128k", 1, 36, 8, 4, 128, 131072, "bf16", seed=4,
                            beta=None, budget_frac=Fraction(1, 20), q_scale=2.0,
                            mass_topk=1024),
    # 28 layers x 4 KV heads (GQA 7), 64K prefill, 8192 streaming steps,
    # fixed budget 4096 x 28 x 4; positions [24576, 40960) bimodal beta
    "stream_gqa7": Workload("stream_gqa7", 1, 28, 4, 7, 128, 65536, "bf16", seed=5,
                            beta=("beta", 5.0, 1.0),
                            beta_block=(24576, 40960, ("mix", 0.5, (1.0, 20.0), (40.0, 1.0))),
                            budget_abs=4096 * 28 * 4, reserve=1, steps=8192),
}


def _rng(seed: int, stream: int, index: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(stream, index))))


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float64 -> float32 (RNE) -> bfloat16 (RNE); returns uint16 bit patterns."""
    # finite inputs only: the rounding increment cannot carry out of 32 bits
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def _draw_beta(rng: np.random.Generator, dist, n: int) -> np.ndarray:
    if dist[0] == "beta":
        return rng.beta(dist[1], dist[2], n)
    if dist[0] == "const":   # the same retention for every entry (closed-form cases)
        return np.full(n, float(dist[1]))
    if dist[0] == "mix":
        w, (a1, b1), (a2, b2) = dist[1], dist[2], dist[3]
        u = rng.random(n)
        c1 = rng.beta(a1, b1, n)
        c2 = rng.beta(a2, b2, n)
        return np.where(u < w, c1, c2)
    raise ValueError(dist)


def head_beta(w: Workload, h: int) -> np.ndarray:
    """beta (float32) of positions 0..ctx-1 of flat KV head h."""
    rng = _rng(w.seed, S_BETA, h)
    if w.beta is None:
        return np.ones(w.ctx, dtype=np.float32)
    b = _draw_beta(rng, w.beta, w.ctx)
    if w.beta_block is not None:
        lo, hi, dist = w.beta_block
        lo, hi = min(lo, w.ctx), min(hi, w.ctx)
        b[lo:hi] = _draw_beta(rng, dist, hi - lo)
    return b.astype(np.float32)


def head_kv(w: Workload, h: int):
    """(K, V) of flat KV head h, [ctx, D]; uint16 bf16 bits or float32."""
    out = []
    for stream in (S_K, S_V):
        rng = _rng(w.seed, stream, h)
        x = rng.standard_normal((w.ctx, w.head_dim))
        if w.outlier_p > 0.0:
            m = _rng(w.seed, S_OUTLIER, 2 * h + (stream == S_V)).random(w.head_dim) < w.outlier_p
            x[:, m] *= w.outlier_scale
        out.append(f64_to_bf16_bits(x) if w.dtype == "bf16" else x.astype(np.float32))
    return out[0], out[1]


def queries(w: Workload, index: int = 0) -> np.ndarray:
    """One query per Q head, [n_qheads, D] (bf16 bits or float32)."""
    rng = _rng(w.seed, S_Q, index)
    x = rng.standard_normal((w.n_qheads, w.head_dim)) * w.q_scale
    return f64_to_bf16_bits(x) if w.dtype == "bf16" else x.astype(np.float32)


def page_perm(w: Workload, n_pages: Optional[int] = None) -> np.ndarray:
    n = w.n_pages if n_pages is None else n_pages
    return _rng(w.seed, S_PERM).permutation(n).astype(np.int32)


def stream_step(w: Workload, s: int):
    """Inputs drawn at streaming step s (1-based): beta, K, V of one new entry
    per KV head and one query per Q head, in that order."""
    rng = _rng(w.seed, S_STEP, s)
    beta = rng.beta(5.0, 1.0, w.n_heads).astype(np.float32)
    k = rng.standard_normal((w.n_heads, w.head_dim))
    v = rng.standard_normal((w.n_heads, w.head_dim))
    q = rng.standard_normal((w.n_qheads, w.head_dim)) * w.q_scale
    conv = (f64_to_bf16_bits if w.dtype == "bf16" else (lambda a: a.astype(np.float32)))
    return beta, conv(k), conv(v), conv(q)


@dataclasses.dataclass
class PagedCache:
    """Host copy of a paged KV pool.

    k, v     [n_pages, 16, D]   uint16 (bf16 bits) or float32
    beta     [n_pages, 16]      float32 (raw retention; its log is the method's job)
    pos      [n_pages, 16]      int32
    page_off [n_heads + 1]      int32  CSR offsets into page_ids
    page_ids [n_pages]          int32  physical page of each logical page
    length   [n_heads]          int32  valid entries per head
    """
    k: np.ndarray
    v: np.ndarray
    beta: np.ndarray
    pos: np.ndarray
    page_off: np.ndarray
    page_ids: np.ndarray
    length: np.ndarray
    head_dim: int
    dtype: str

    @property
    def n_heads(self) -> int:
        return int(self.length.shape[0])

    @property
    def n_pages(self) -> int:
        return int(self.k.shape[0])


def empty_pool(n_pages: int, d: int, dtype: str):
    kd = np.uint16 if dtype == "bf16" else np.float32
    return (np.zeros((n_pages, PAGE, d), kd), np.zeros((n_pages, PAGE, d), kd),
            np.zeros((n_pages, PAGE), np.float32), np.zeros((n_pages, PAGE), np.int32))


def build_cache(w: Workload, heads: Optional[list] = None, lengths: Optional[np.ndarray] = None,
                perm: Optional[np.ndarray] = None, extra_pages: int = 0, workers: int = 1) -> PagedCache:
    """Prefill pool for workload w.

    Every head holds positions 0..len-1 in slot order (len = ctx unless
    ``lengths`` gives ragged per-head lengths, each <= ctx) in
    ceil((len + reserve)/16) logical pages; logical page c of the CSR lives in
    physical page perm[c].
    """
    H, D = w.n_heads, w.head_dim
    if lengths is None:
        lengths = np.full(H, w.ctx, dtype=np.int32)
    lengths = np.asarray(lengths, dtype=np.int32)
    pages = -(-(lengths.astype(np.int64) + w.reserve) // PAGE)
    page_off = np.zeros(H + 1, dtype=np.int64)
    np.cumsum(pages, out=page_off[1:])
    n_used = int(page_off[-1])
    n_pages = n_used + extra_pages
    if perm is None:
        perm = _rng(w.seed, S_PERM).permutation(n_pages).astype(np.int32)
    k, v, beta, pos = empty_pool(n_pages, D, w.dtype)

    def fill(h):
        n = int(lengths[h])
        if n == 0:
            return
        bh = head_beta(w, h)[:n]
        kh, vh = head_kv(w, h)
        kh, vh = kh[:n], vh[:n]
        phys = perm[page_off[h]:page_off[h + 1]]
        slots = phys[np.arange(n) // PAGE].astype(np.int64) * PAGE + np.arange(n) % PAGE
        k.reshape(-1, D)[slots] = kh
        v.reshape(-1, D)[slots] = vh
        beta.reshape(-1)[slots] = bh
        pos.reshape(-1)[slots] = np.arange(n, dtype=np.int32)

    # heads write disjoint slots, so threads may fill them concurrently
    if workers > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(fill, range(H)))
    else:
        for h in range(H):
            fill(h)
    return PagedCache(k, v, beta, pos, page_off.astype(np.int32), perm.astype(np.int32),
                      lengths.copy(), D, w.dtype)


def random_ragged_cache(seed: int, n_heads: int, d: int, dtype: str, max_len: int,
                        reserve: int = 0, min_len: int = 0, t: Optional[int] = None,
                        beta_dist=("beta", 5.0, 1.0)) -> PagedCache:
    """A cache with ragged per-head lengths and strictly increasing but gappy
    positions (as after evictions), used for kernel edge cases."""
    rng = _rng(seed, 100)
    lengths = rng.integers(min_len, max_len + 1, n_heads).astype(np.int32)
    pages = -(-(lengths.astype(np.int64) + reserve) // PAGE)
    page_off = np.zeros(n_heads + 1, dtype=np.int64)
    np.cumsum(pages, out=page_off[1:])
    n_pages = int(page_off[-1]) + 3
    perm = rng.permutation(n_pages).astype(np.int32)
    k, v, beta, pos = empty_pool(n_pages, d, dtype)
    t = t if t is not None else 4 * max_len + 8
    for h in range(n_heads):
        n = int(lengths[h])
        if n == 0:
            continue
        p = np.sort(rng.choice(t, size=n, replace=False)).astype(np.int32)
        kh = rng.standard_normal((n, d))
        vh = rng.standard_normal((n, d))
        bh = _draw_beta(rng, beta_dist, n).astype(np.float32)
        phys = perm[page_off[h]:page_off[h + 1]]
        slots = phys[np.arange(n) // PAGE].astype(np.int64) * PAGE + np.arange(n) % PAGE
        conv = f64_to_bf16_bits if dtype == "bf16" else (lambda a: a.astype(np.float32))
        k.reshape(-1, d)[slots] = conv(kh)
        v.reshape(-1, d)[slots] = conv(vh)
        beta.reshape(-1)[slots] = bh
        pos.reshape(-1)[slots] = p
    return PagedCache(k, v, beta, pos, page_off.astype(np.int32), perm, lengths, d, dtype)
