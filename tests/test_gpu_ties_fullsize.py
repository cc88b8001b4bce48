"""Tie ranking of the global selection at the full size of the 8B-shape,
32K-context workload: 256 heads x 32,768 entries in a pool of 524,288 pages
placed at random, with each head's positions shuffled over its slots (slot
order is not position order, as after tail-filled eviction), and a budget of
10 % of the entries (838,861).

Scores tie heavily (DBTrimKV page, Method 3: one global ranking; the ties
rank by head ascending, then position descending):
  - beta = 1 everywhere: every score is 0; the heads fill in order and the
    head that straddles the budget keeps its most recent entries (a
    selection over its positions);
  - beta = 1/2 everywhere: entries of equal age tie across all heads;
  - beta drawn from {1/2, 0.9, 1}: a third of each head ties at score 0,
    far more than the budget.
Both paths -- score then select, and the fused score + select -- are
compared bit for bit with each other and with the oracle's selection over
the flat entries (a partial sort under the same total order), and the
first two cases also with their closed forms."""
import numpy as np
import pytest
import torch

from oracle import reference as ref
from retention_scored_decode_amd import trimkv as tk
from gpu_helpers import f32_bits

pytestmark = pytest.mark.gpu

H, L, PAGE, D = 256, 32768, 16, 128
M = 838861


def say(*a):
    print("[ties-fullsize]", *a, flush=True)


@pytest.fixture(scope="module")
def pool():
    rng = np.random.default_rng(2024)
    per_head = L // PAGE
    n_pages = H * per_head
    page_off = np.arange(H + 1, dtype=np.int32) * per_head
    page_ids = rng.permutation(n_pages).astype(np.int32)
    pos = np.empty((H, L), np.int32)   # CSR slot order: head h, entry i
    for h in range(H):
        pos[h] = rng.permutation(L)
    dev = {
        "k": torch.empty((n_pages, PAGE, D), dtype=torch.bfloat16, device="cuda"),   # never read here
        "v": torch.empty((n_pages, PAGE, D), dtype=torch.bfloat16, device="cuda"),
        "off": torch.from_numpy(page_off).cuda(),
        "ids": torch.from_numpy(page_ids).cuda(),
        "len": torch.full((H,), L, dtype=torch.int32, device="cuda"),
    }
    return rng, n_pages, page_ids, pos, dev


def run_case(pool, beta_csr):
    """beta_csr: [H, L] float32 in CSR slot order.  Returns the GPU keep
    plane (CSR order, as bool [H, L]) and kept counts, after checking that
    both paths agree bit for bit."""
    _, n_pages, page_ids, pos, dev = pool
    # metadata blocks in physical page order: ln beta from the GPU's own
    # kernel (a0), positions as generated
    beta_phys = np.empty((n_pages, PAGE), np.float32)
    beta_phys[page_ids] = beta_csr.reshape(n_pages, PAGE)
    pos_phys = np.empty((n_pages, PAGE), np.int32)
    pos_phys[page_ids] = pos.reshape(n_pages, PAGE)
    meta = torch.zeros((n_pages, 2, PAGE), dtype=torch.int32, device="cuda")
    meta[:, 1, :] = torch.from_numpy(pos_phys).cuda()
    tk.log_beta(torch.from_numpy(beta_phys).cuda(), meta, out_page_stride=2 * PAGE)
    c = tk.Cache(dev["k"], dev["v"], meta, dev["off"], dev["ids"], dev["len"])
    seg = torch.tensor([0, H], dtype=torch.int32, device="cuda")
    t = torch.tensor([L], dtype=torch.int32, device="cuda")
    bud = torch.tensor([M], dtype=torch.int64, device="cuda")
    n = n_pages * PAGE
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    s1 = torch.empty(n, dtype=torch.float32, device="cuda")
    k1 = torch.empty(n, dtype=torch.uint8, device="cuda")
    kept1 = torch.empty(H, dtype=torch.int32, device="cuda")
    tk.score(c, seg, t, s1)
    tk.select_global(c, s1, seg, bud, k1, kept1, status=status)
    s2 = torch.empty(n, dtype=torch.float32, device="cuda")
    k2 = torch.empty(n, dtype=torch.uint8, device="cuda")
    kept2 = torch.empty(H, dtype=torch.int32, device="cuda")
    tk.score_select(c, seg, t, bud, s2, k2, kept2, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0, "a tie-rank wait timed out"
    assert np.array_equal(f32_bits(s1.cpu().numpy()), f32_bits(s2.cpu().numpy()))
    keep = k1.cpu().numpy()
    assert np.array_equal(keep, k2.cpu().numpy())
    kept = kept1.cpu().numpy()
    assert np.array_equal(kept, kept2.cpu().numpy())
    assert np.all((keep == 0) | (keep == 1))
    keep = keep.astype(bool).reshape(H, L)
    assert np.array_equal(keep.sum(axis=1), kept)
    return keep, kept


def oracle_keep(pool, beta_csr):
    _, _, _, pos, _ = pool
    lnb = ref.ln_beta(beta_csr.reshape(-1))
    sc = ref.score_f32(lnb, L, pos.reshape(-1))
    head = np.repeat(np.arange(H, dtype=np.int64), L)
    return ref.select_flat(sc, head, pos.reshape(-1), M).reshape(H, L)


def test_ties_beta_one(pool):
    beta = np.ones((H, L), np.float32)
    keep, kept = run_case(pool, beta)
    pos = pool[3]
    full = M // L                      # heads kept whole, in head order
    rest = M - full * L
    want_kept = np.zeros(H, np.int64)
    want_kept[:full] = L
    want_kept[full] = rest
    assert np.array_equal(kept, want_kept)
    assert np.array_equal(keep[full], pos[full] >= L - rest)   # the straddling head: its most recent
    assert keep[:full].all() and not keep[full + 1:].any()
    assert np.array_equal(keep, oracle_keep(pool, beta))
    say("beta = 1: heads 0..%d whole, head %d keeps its %d most recent" % (full - 1, full, rest))


def test_ties_beta_half(pool):
    beta = np.full((H, L), 0.5, np.float32)
    keep, kept = run_case(pool, beta)
    pos = pool[3]
    ages = M // H                      # every head keeps ages 1..ages
    extra = M - ages * H               # the first `extra` heads also keep age ages + 1
    age = L - pos
    want = age <= ages
    want[:extra] |= age[:extra] == ages + 1
    assert np.array_equal(keep, want)
    assert np.array_equal(keep, oracle_keep(pool, beta))
    say("beta = 1/2: ages 1..%d everywhere, age %d in heads 0..%d" % (ages, ages + 1, extra - 1))


def test_ties_beta_three_values(pool):
    rng = pool[0]
    beta = rng.choice(np.array([0.5, 0.9, 1.0], np.float32), size=(H, L))
    keep, kept = run_case(pool, beta)
    want = oracle_keep(pool, beta)
    assert np.array_equal(keep, want)
    straddle = int(np.flatnonzero(kept > 0)[-1])
    say("beta in {1/2, 0.9, 1}: heads up to %d keep entries; head %d keeps %d of its %d ties at 0"
        % (straddle, straddle, int(kept[straddle]), int((beta[straddle] == 1.0).sum())))
