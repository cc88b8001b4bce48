"""The streaming decode loop: generated steps as a fixed sequence of C-ABI
calls, launched eagerly or replayed from captured HIP graphs.

A step (TRIM-KV page, section 2: a new entry per head with its retention;
the lowest current scores are evicted once the budget is exceeded) appends
one entry per KV head, scores every entry at the step's t, selects the
global top M, runs mask-mode decode attention with the step's queries
(renormalised output and dropped mass), and evicts into the other of two
pools (one spare slot per head for the next append).

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
    """Streaming steps over two ping-pong pools.

    pools:  two Cache objects of equal capacity, at least
            ceil((M + n_heads) / 16) + n_heads pages each;
    banks:  device tensors of per-step inputs, step entry first:
            k [S, H, D], v [S, H, D] (cache dtype), beta [S, H] float32,
            q [S, H * group, D] (cache dtype), t [S, 1] int32 (the decode
            step; entry s is appended at position t[s] - 1);
    first:  the bank entry of the next step; the current cache is pools[0].
    """

    def __init__(self, pools: List[tk.Cache], budget: int, group: int, scale: float, banks: dict, first: int = 0):
        assert len(pools) == 2 and pools[0].n_pages == pools[1].n_pages
        dev = pools[0].k.device
        H, D = pools[0].n_heads, pools[0].head_dim
        self.pools, self.M, self.G, self.scale = pools, int(budget), int(group), float(scale)
        self.banks = banks
        self.next = int(first)
        n = pools[0].n_pages * tk.PAGE
        self.score = torch.empty(n, dtype=torch.float32, device=dev)
        self.keep = torch.empty(n, dtype=torch.uint8, device=dev)
        self.kept = torch.empty(H, dtype=torch.int32, device=dev)
        self.used = torch.zeros(1, dtype=torch.int64, device=dev)
        self.out = torch.empty((H * group, D), dtype=torch.float32, device=dev)
        self.dropped = torch.empty(H * group, dtype=torch.float32, device=dev)
        self.seg = torch.tensor([0, H], dtype=torch.int32, device=dev)
        self.bud = torch.tensor([self.M], dtype=torch.int64, device=dev)
        self.ws_sel = tk.workspace(tk.OP_SELECT, pools[0], 1)
        self.ws_att = tk.workspace(tk.OP_DECODE_ATTN, pools[0], 0, group)
        self.ws_cmp = tk.workspace(tk.OP_COMPACT, pools[0])
        # failure counters (append: heads without a free slot; select: timed-out waits)
        self.status = torch.zeros(2, dtype=torch.int32, device=dev)
        self.cur = 0          # index of the pool holding the current cache
        self.graphs: list = []

    def _step(self, i: int, src: tk.Cache, dst: tk.Cache):
        b = self.banks
        tk.append(src, b["k"][i], b["v"][i], b["beta"][i], b["t"][i], status=self.status[0:1])
        tk.score_select(src, self.seg, b["t"][i], self.bud, self.score, self.keep, self.kept, ws=self.ws_sel,
                        status=self.status[1:2])
        tk.decode_attn(src, b["q"][i], self.G, self.scale, self.out, self.dropped, keep=self.keep, ws=self.ws_att)
        tk.compact(src, self.keep, 1, self.M, dst, self.used, ws=self.ws_cmp, kept=self.kept)

    def run(self, n: int = 1):
        """The next n steps, launched eagerly."""
        for _ in range(n):
            self._step(self.next, self.pools[self.cur], self.pools[1 - self.cur])
            self.cur = 1 - self.cur
            self.next += 1

    def capture(self, n: int, chunk: int = 64):
        """Record the next n steps (graphs of `chunk` steps) without running
        them; replay() then runs them.  The library's one-time host set-up
        must have run (an eager step in this process first)."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        graphs, i, cur = [], self.next, self.cur
        with torch.cuda.stream(side):
            while i < self.next + n:
                g = torch.cuda.CUDAGraph()
                m = min(chunk, self.next + n - i)
                with torch.cuda.graph(g, stream=side):
                    for _ in range(m):
                        self._step(i, self.pools[cur], self.pools[1 - cur])
                        cur = 1 - cur
                        i += 1
                graphs.append((g, m))
        torch.cuda.current_stream().wait_stream(side)
        self.graphs = graphs

    def replay(self, graphs: int = -1):
        """Run the captured steps: the next `graphs` graphs (all by default)."""
        k = len(self.graphs) if graphs < 0 else min(graphs, len(self.graphs))
        for g, m in self.graphs[:k]:
            g.replay()
            self.cur = (self.cur + m) % 2
            self.next += m
        self.graphs = self.graphs[k:]

    @property
    def cache(self) -> tk.Cache:
        """The current cache (the pool the last step evicted into)."""
        return self.pools[self.cur]
