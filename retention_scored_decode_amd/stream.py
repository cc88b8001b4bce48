"""The streaming decode loop: generated steps as a fixed sequence of C-ABI
calls, launched eagerly or replayed from captured HIP graphs.

A step (TRIM-KV page, section 2: a new entry per head with its retention;
the lowest current scores are evicted once the budget is exceeded) appends
one entry per KV head, scores every entry at the step's t, selects the
global top M, runs mask-mode decode attention with the step's queries
(renormalised output and dropped mass), and evicts, keeping one spare slot
per head for the next append.  With tail fill the step is, by default, two
fused calls: the append written by the selection's first kernel, and the
attention's merge beside the eviction in one launch.  Eviction is either out of place, into the
other of two pools, or in place by tail fill: the cache stays in its home
pages and only the kept entries that fill holes below a head's new length
move, the new page table going to the other of two table buffers.

Every per-step quantity is read from device memory (t included), so a run
of steps can be captured once and replayed: capture() records the next n
steps, in graphs of `chunk` steps each, with each step's inputs taken from
its own entry of device-resident banks.  The library enqueues no memory
sets, host synchronisations or allocations inside a step, so the graphs
hold only its kernels.  This module only orders calls; every step of the
method runs in the library's kernels.
"""
from __future__ import annotations

from typing import List

import torch

from . import trimkv as tk


class StreamLoop:
    """Streaming steps.

    pools:  out of place, two Cache objects of equal capacity, at least
            ceil((M + n_heads) / 16) + n_heads pages each; the current cache
            is pools[0].  Tail fill, one Cache: the current cache, whose page
            table is the home list of every head (room for M entries plus one
            spare slot per head and step to come).
    banks:  device tensors of per-step inputs, step entry first:
            k [S, H, D], v [S, H, D] (cache dtype), beta [S, H] float32,
            q [S, H * group, D] (cache dtype), t [S, 1] int32 (the decode
            step; entry s is appended at position t[s] - 1);
    first:  the bank entry of the next step;
    evict:  "out_of_place" or "tail_fill";
    fused:  tail fill only: a step is two calls, trimkv_append_score_select
            and trimkv_decode_attn_evict_tailfill (the same results as the
            four separate calls, with two launches fewer).
    """

    def __init__(self, pools: List[tk.Cache], budget: int, group: int, scale: float, banks: dict, first: int = 0,
                 evict: str = "out_of_place", fused: bool = True):
        assert evict in ("out_of_place", "tail_fill")
        self.tail_fill = evict == "tail_fill"
        self.fused = fused and self.tail_fill
        if self.tail_fill:
            assert len(pools) == 1
        else:
            assert len(pools) == 2 and pools[0].n_pages == pools[1].n_pages
        base = pools[0]
        dev = base.k.device
        H, D = base.n_heads, base.head_dim
        self.pools, self.M, self.G, self.scale = pools, int(budget), int(group), float(scale)
        self.banks = banks
        self.next = int(first)
        n = base.n_pages * tk.PAGE
        self.score = torch.empty(n, dtype=torch.float32, device=dev)
        self.keep = torch.empty(n, dtype=torch.uint8, device=dev)
        self.kept = torch.empty(H, dtype=torch.int32, device=dev)
        self.used = torch.zeros(1, dtype=torch.int64, device=dev)
        self.out = torch.empty((H * group, D), dtype=torch.float32, device=dev)
        self.dropped = torch.empty(H * group, dtype=torch.float32, device=dev)
        self.seg = torch.tensor([0, H], dtype=torch.int32, device=dev)
        self.bud = torch.tensor([self.M], dtype=torch.int64, device=dev)
        self.ws_sel = tk.workspace(tk.OP_SELECT, base, 1)
        self.ws_att = tk.workspace(tk.OP_DECODE_ATTN, base, 0, group)
        if self.tail_fill:
            self.home_off, self.home_ids = base.page_off.clone(), base.page_ids.clone()
            self.tables = [(torch.empty_like(base.page_off), torch.empty_like(base.page_ids)) for _ in range(2)]
            self.ws_ev = tk.workspace(tk.OP_EVICT_TAILFILL, base)
            if self.fused:
                self.ws_att = tk.workspace(tk.OP_DECODE_EVICT, base, 0, group)
        else:
            self.ws_ev = tk.workspace(tk.OP_COMPACT, base)
        # failure counters (append: heads without a free slot; select: timed-out waits)
        self.status = torch.zeros(2, dtype=torch.int32, device=dev)
        self.view = base      # the current cache
        self.graphs: list = []

    def _step(self, i: int, src: tk.Cache) -> tk.Cache:
        """Step of bank entry i on cache src; returns the cache after eviction."""
        b = self.banks
        if self.fused:
            tk.append_score_select(src, b["k"][i], b["v"][i], b["beta"][i], self.seg, b["t"][i], self.bud, self.score,
                                   self.keep, self.kept, ws=self.ws_sel, append_status=self.status[0:1],
                                   select_status=self.status[1:2])
            off, ids = self.tables[i % 2]
            return tk.decode_attn_evict_tailfill(src, self.keep, self.kept, b["q"][i], self.G, self.scale, self.out,
                                                 self.dropped, 1, self.home_off, self.home_ids, off, ids,
                                                 ws=self.ws_att)
        tk.append(src, b["k"][i], b["v"][i], b["beta"][i], b["t"][i], status=self.status[0:1])
        tk.score_select(src, self.seg, b["t"][i], self.bud, self.score, self.keep, self.kept, ws=self.ws_sel,
                        status=self.status[1:2])
        tk.decode_attn(src, b["q"][i], self.G, self.scale, self.out, self.dropped, keep=self.keep, ws=self.ws_att)
        if self.tail_fill:
            off, ids = self.tables[i % 2]
            return tk.evict_tailfill(src, self.keep, 1, self.home_off, self.home_ids, off, ids, kept=self.kept,
                                     ws=self.ws_ev)
        dst = self.pools[1] if src.k.data_ptr() == self.pools[0].k.data_ptr() else self.pools[0]
        tk.compact(src, self.keep, 1, self.M, dst, self.used, ws=self.ws_ev, kept=self.kept)
        return dst

    def run(self, n: int = 1):
        """The next n steps, launched eagerly."""
        for _ in range(n):
            self.view = self._step(self.next, self.view)
            self.next += 1

    def capture(self, n: int, chunk: int = 64):
        """Record the next n steps (graphs of `chunk` steps) without running
        them; replay() then runs them.  The library's one-time host set-up
        must have run (an eager step in this process first)."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        graphs, i, view = [], self.next, self.view
        with torch.cuda.stream(side):
            while i < self.next + n:
                g = torch.cuda.CUDAGraph()
                m = min(chunk, self.next + n - i)
                with torch.cuda.graph(g, stream=side):
                    for _ in range(m):
                        view = self._step(i, view)
                        i += 1
                graphs.append((g, m, view))
        torch.cuda.current_stream().wait_stream(side)
        self.graphs = graphs

    def replay(self, graphs: int = -1):
        """Run the captured steps: the next `graphs` graphs (all by default)."""
        k = len(self.graphs) if graphs < 0 else min(graphs, len(self.graphs))
        for g, m, view in self.graphs[:k]:
            g.replay()
            self.view = view
            self.next += m
        self.graphs = self.graphs[k:]

    @property
    def cache(self) -> tk.Cache:
        """The current cache (the one the last step evicted into)."""
        return self.view
