"""The allocation-free decode entry point (trimkv_decode_attn_noalloc)
against the workspace entry point (trimkv_decode_attn) through the C ABI:
bit-identical outputs, dropped mass and log-sum-exp, and both within the
float64 oracle's tolerances; two calls in a row on one GPU, the second with
a smaller input, so that nothing of the first call's scratch leaks into the
second."""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import reference as ref
from retention_scored_decode_amd import trimkv as tk
from gpu_helpers import DROP_TOL, OUT_TOL, OracleView, cuda, kv_dev, plane_from_heads, upload

pytestmark = pytest.mark.gpu


def _call(fn, c, q, G, keep):
    """One decode call of either entry point into NaN-filled outputs."""
    nq = c.n_heads * G
    out = torch.full((nq, c.head_dim), np.nan, dtype=torch.float32, device="cuda")
    dropped = torch.full((nq,), np.nan, dtype=torch.float32, device="cuda")
    lse = torch.full((nq,), np.nan, dtype=torch.float32, device="cuda")
    fn(c, q, G, 1.0 / math.sqrt(c.head_dim), out, dropped, keep=keep, lse_out=lse)
    torch.cuda.synchronize()
    return out.cpu().numpy(), dropped.cpu().numpy(), lse.cpu().numpy()


def _check(pc, G, seed):
    rng = np.random.default_rng(seed)
    c = upload(pc)
    ov = OracleView(pc)
    H, D = pc.n_heads, pc.head_dim
    qx = rng.standard_normal((H * G, D))
    q_bits = synth.f64_to_bf16_bits(qx) if pc.dtype == "bf16" else qx.astype(np.float32)
    q64 = (synth.bf16_bits_to_f32(q_bits) if pc.dtype == "bf16" else q_bits).astype(np.float64)
    q = kv_dev(q_bits, pc.dtype)
    keep_h = [rng.random(int(n)) < 0.3 for n in pc.length]
    keep = cuda(plane_from_heads([k.astype(np.uint8) for k in keep_h], pc.page_off, pc.length, pc.n_pages, 0,
                                 np.uint8))
    for kp, kh in ((None, None), (keep, keep_h)):
        a = _call(tk.decode_attn, c, q, G, kp)
        b = _call(tk.decode_attn_noalloc, c, q, G, kp)
        for x, y in zip(a, b):
            assert np.array_equal(x.view(np.uint32), y.view(np.uint32)), "differs from the workspace entry point"
        wout, wdrop, wlse = ref.decode_attn(ov.k, ov.v, q64, G, 1.0 / math.sqrt(D), keep=kh)
        assert np.max(np.abs(b[0] - wout)) <= OUT_TOL
        assert np.max(np.abs(b[1] - wdrop)) <= DROP_TOL
        fin = np.isfinite(wlse)
        assert np.array_equal(fin, np.isfinite(b[2]))
        assert np.all(np.abs(b[2][fin] - wlse[fin]) <= 1e-4 * np.maximum(1, np.abs(wlse[fin])))


def test_noalloc_decode_two_calls_second_smaller():
    big = synth.WORKLOADS["llama8b_32k"].scaled(layers=4, ctx=4001)
    small = synth.WORKLOADS["stream_gqa7"].scaled(layers=1, kv_heads=3, ctx=333)
    _check(synth.build_cache(big), big.group, 1)
    _check(synth.build_cache(small), small.group, 2)


def test_noalloc_decode_ragged_and_fp32():
    pc = synth.random_ragged_cache(611, n_heads=37, d=64, dtype="bf16", max_len=3000)
    _check(pc, 3, 3)
    pc = synth.random_ragged_cache(612, n_heads=5, d=128, dtype="f32", max_len=700)
    _check(pc, 2, 4)
