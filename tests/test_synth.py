"""The seeded generator: determinism, shapes and the page-table layout."""
import numpy as np

import synth


def test_same_seed_same_bytes():
    w = synth.WORKLOADS["llama8b_32k"].scaled(layers=1, kv_heads=2, ctx=100)
    a = synth.build_cache(w)
    b = synth.build_cache(w)
    for f in ("k", "v", "beta", "pos", "page_off", "page_ids", "length"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    assert np.array_equal(synth.queries(w), synth.queries(w))


def test_layout_positions_through_page_table():
    w = synth.WORKLOADS["stream_gqa7"].scaled(layers=1, ctx=70)
    c = synth.build_cache(w)
    assert sorted(c.page_ids.tolist()) == list(range(c.n_pages))
    for h in range(c.n_heads):
        n = int(c.length[h])
        i = np.arange(n)
        phys = c.page_ids[c.page_off[h] + i // 16]
        assert np.array_equal(c.pos[phys, i % 16], i)
        # one spare slot per head (reserve)
        assert (c.page_off[h + 1] - c.page_off[h]) * 16 >= n + 1


def test_bf16_rounding_is_rne():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -9, -2.5, 3.0e-3])
    b = synth.f64_to_bf16_bits(x)
    back = synth.bf16_bits_to_f32(b)
    assert back[0] == 1.0 and back[1] == 1.0          # tie to even
    assert back[2] == 1.0 + 2 ** -7                   # tie to even (up)
    assert back[3] == -2.5


def test_outlier_channels_scaled():
    w = synth.WORKLOADS["llama8b_32k"].scaled(layers=4, ctx=64)
    n_out = 0
    for h in range(w.n_heads):
        k, _ = synth.head_kv(w, h)
        sd = synth.bf16_bits_to_f32(k).std(axis=0)
        n_out += int((sd > 4).sum())
    # about 1% of 32 heads x 128 channels
    assert 10 <= n_out <= 80
