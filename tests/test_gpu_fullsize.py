"""Parity at the full size of the 8B-shape, 32K-context workload, in the launch
configuration the benchmark times (score -> select -> mask-mode attention ->
compaction -> plain decode on the compacted cache).

Selection and the compacted page table are checked for every head; scores,
compacted rows and both attention modes on a sample of heads spread over the
layers (the float64 oracle gathers only those heads).  Well under a minute,
most of it generating the 4 GB synthetic cache and the oracle's selection."""
import math
import os
import time

import numpy as np
import pytest
import torch

import synth
from oracle import reference as ref
from retention_scored_decode_amd import trimkv as tk
from gpu_helpers import DROP_TOL, OUT_TOL, cuda, download_cache, f32_bits, heads_from_plane, kv_f64, upload

pytestmark = pytest.mark.gpu


def say(*a):
    print("[fullsize]", *a, flush=True)


@pytest.fixture(scope="module")
def full_c2():
    w = synth.WORKLOADS["llama8b_32k"]
    t0 = time.time()
    pc = synth.build_cache(w, workers=min(16, os.cpu_count() or 1))
    say("generated", w.name, "in %.1f s" % (time.time() - t0))
    return w, pc


def test_full_size_pipeline(full_c2):
    w, pc = full_c2
    H, G, D = pc.n_heads, w.group, w.head_dim
    M = w.budget()
    c = upload(pc)
    seg = cuda(w.seg_head_begin(), np.int32)
    score = torch.empty(pc.n_pages * 16, dtype=torch.float32, device="cuda")
    tk.score(c, seg, cuda(np.full(w.n_seg, w.t, np.int32)), score)
    keep = torch.empty(pc.n_pages * 16, dtype=torch.uint8, device="cuda")
    kept = torch.empty(H, dtype=torch.int32, device="cuda")
    tk.select_global(c, score, seg, cuda(np.full(w.n_seg, M, np.int64)), keep, kept)
    q_bits = synth.queries(w)
    q_dev = torch.from_numpy(np.ascontiguousarray(q_bits).view(np.int16)).to("cuda").view(torch.bfloat16)
    q64 = synth.bf16_bits_to_f32(q_bits).astype(np.float64)
    scale = 1.0 / math.sqrt(D)
    nq = H * G
    out_m = torch.empty((nq, D), dtype=torch.float32, device="cuda")
    drop_m = torch.empty(nq, dtype=torch.float32, device="cuda")
    tk.decode_attn(c, q_dev, G, scale, out_m, drop_m, keep=keep)
    cap = -(-M // 16) + H
    dst = tk.Cache.empty(H, cap, D, torch.bfloat16)
    used = torch.zeros(1, dtype=torch.int64, device="cuda")
    tk.compact(c, keep, 0, M, dst, used, kept=kept)
    out_p = torch.empty((nq, D), dtype=torch.float32, device="cuda")
    drop_p = torch.empty(nq, dtype=torch.float32, device="cuda")
    lse_p = torch.empty(nq, dtype=torch.float32, device="cuda")
    tk.decode_attn(dst, q_dev, G, scale, out_p, drop_p, lse_out=lse_p)
    torch.cuda.synchronize()
    say("GPU pipeline done")

    # ---- scores and selection, every head ----
    po, pi, ln = pc.page_off, pc.page_ids, pc.length
    lnb = [ref.ln_beta(b) for b in ref.gather_heads(pc.beta, po, pi, ln)]
    pos = ref.gather_heads(pc.pos, po, pi, ln)
    want_scores = [ref.score_f32(lnb[h], w.t, pos[h]) for h in range(H)]
    got_scores = heads_from_plane(score.cpu().numpy(), po, ln)
    for h in range(H):
        assert np.array_equal(f32_bits(got_scores[h]), f32_bits(want_scores[h])), ("score", h)
    say("scores bit-exact")
    want_keep, want_kept = ref.select_global(want_scores, w.seg_head_begin(), [M])
    got_keep = heads_from_plane(keep.cpu().numpy(), po, ln)
    for h in range(H):
        assert np.array_equal(got_keep[h].astype(bool), want_keep[h]), ("keep", h)
    assert np.array_equal(kept.cpu().numpy(), want_kept)
    assert int(want_kept.sum()) == M
    say("selection bit-exact")

    # ---- compaction: page table for every head, rows for a sample ----
    dpo, dpi, dln, dk, dv, dlnb, dpos = download_cache(dst)
    wpo, _, wln = ref.compact_layout(want_kept, 0)
    assert np.array_equal(dpo, wpo) and np.array_equal(dln, wln)
    assert int(used.item()) == int(wpo[-1])
    assert np.array_equal(dpi[:int(wpo[-1])], np.arange(int(wpo[-1]), dtype=np.int32))
    sample = list(range(0, H, 17)) + [H - 1]
    flat_k, flat_v = pc.k.reshape(-1, D), pc.v.reshape(-1, D)
    for h in sample:
        src = ref.head_phys_slots(po, pi, ln, h)[want_keep[h]]
        assert np.array_equal(ref.gather_heads(dk, dpo, dpi, dln)[h], flat_k[src]), ("k rows", h)
        assert np.array_equal(ref.gather_heads(dv, dpo, dpi, dln)[h], flat_v[src]), ("v rows", h)
        assert np.array_equal(f32_bits(ref.gather_heads(dlnb, dpo, dpi, dln)[h]), f32_bits(lnb[h][want_keep[h]]))
        assert np.array_equal(ref.gather_heads(dpos, dpo, dpi, dln)[h], pos[h][want_keep[h]])
    say("compaction checked")

    # ---- attention on the sampled heads, both modes ----
    om, dm, op, dp, lp = (x.cpu().numpy() for x in (out_m, drop_m, out_p, drop_p, lse_p))
    K = [kv_f64(flat_k[ref.head_phys_slots(po, pi, ln, h)], pc.dtype) for h in sample]
    V = [kv_f64(flat_v[ref.head_phys_slots(po, pi, ln, h)], pc.dtype) for h in sample]
    qs = np.concatenate([q64[h * G:(h + 1) * G] for h in sample])
    rows = np.concatenate([np.arange(h * G, (h + 1) * G) for h in sample])
    kp = [want_keep[h] for h in sample]
    wout, wdrop, _ = ref.decode_attn(K, V, qs, G, scale, keep=kp)
    assert np.max(np.abs(om[rows] - wout)) <= OUT_TOL
    assert np.max(np.abs(dm[rows] - wdrop)) <= DROP_TOL
    wout2, _, wlse2 = ref.decode_attn([k[m] for k, m in zip(K, kp)], [v[m] for v, m in zip(V, kp)], qs, G, scale)
    assert np.max(np.abs(op[rows] - wout2)) <= OUT_TOL
    assert np.all(dp[rows] == 0.0)
    assert np.all(np.abs(lp[rows] - wlse2) <= 1e-4 * np.maximum(1, np.abs(wlse2)))
    # properties at every head: finite outputs, dropped mass in [0, 1], both modes agree on the kept set
    assert np.all(np.isfinite(om)) and np.all(np.isfinite(op))
    assert np.all((dm >= 0) & (dm <= 1))
    assert np.max(np.abs(op - om)) <= OUT_TOL
    say("attention checked on", len(sample), "heads; modes agree on all", H)
