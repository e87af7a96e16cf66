"""GPU parity of top-k on long rows, bit-exact against the oracle (rank
order of "Module glm5next_dsa_ref", topk_pools: higher score first, then the
smaller index; INVALID past the visible keys).

Rows of 16385 .. 262144 keys take the shared-threshold path: every block of
4096 columns reports (key, count) pairs, the largest pair key that the
pairs guarantee k keys above becomes the row's threshold, the keys at or
above it are compacted, and a segmented merge ranks them.  The score
distributions below are chosen so that each part of it is exercised: value
buckets (normal, quantised, relu-like with many exact zeros), all-equal rows
(column order), monotone rows (one block holds every winner), one outlier
per block (the order-key buckets take over from the value buckets), two
narrow clusters far apart (the threshold keeps more candidates than the
workspace holds, so the raw row is ranked in one block), infinities.
Longer rows take the chunked path (chunk winners, then a segmented, cached
or streaming merge), covered at 300000 keys."""
import numpy as np
import pytest
import torch

import oracle
from tests.parity import cpu, note

pytestmark = pytest.mark.gpu

POISON_I32 = 0x7EADBEEF


@pytest.fixture(scope="module")
def dsa():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    from sparse_attention_scores_amd import binding
    binding.load()
    return binding


def _row(kind, n, rng):
    i = np.arange(n)
    if kind == "normal":
        return rng.standard_normal(n) * 5
    if kind == "quantised":
        return np.round(rng.standard_normal(n) * 20) / 4
    if kind == "all_equal":
        return np.full(n, 1.5)
    if kind == "increasing":
        return i * 1e-3
    if kind == "decreasing":
        return -i * 1e-3
    if kind == "one_outlier":
        return np.where(i == 5, 1e30, rng.random(n))
    if kind == "outlier_per_block":
        return np.where(i % 4096 == 7, 1e6, rng.random(n) * 1e-3)
    if kind == "two_clusters":
        return np.where(i % 2 == 0, 1000 + rng.random(n), rng.random(n))
    if kind == "relu_like":
        return np.maximum(rng.standard_normal(n), 0) * 3
    if kind == "with_inf":
        return np.where(i % 9000 == 1, np.inf, rng.standard_normal(n))
    raise ValueError(kind)


KINDS = ["normal", "quantised", "all_equal", "increasing", "decreasing", "one_outlier",
         "outlier_per_block", "two_clusters", "relu_like", "with_inf"]


def _check(dsa, S, lo, hi, k, n_sink=0, noalloc=False):
    rows = S.shape[0]
    St = torch.tensor(S, device="cuda")
    lo_t = torch.tensor(lo, dtype=torch.int32, device="cuda")
    hi_t = torch.tensor(hi, dtype=torch.int32, device="cuda")
    idx = torch.full((rows, k), POISON_I32, dtype=torch.int32, device="cuda")
    dsa.topk(St, lo_t, hi_t, k, out=idx, n_sink=n_sink)
    torch.cuda.synchronize()
    # the oracle's visible range is [pad, q_pos + 1): pad = lo, q_pos = hi - 1
    ref = oracle.topk(S, np.asarray(hi) - 1, np.asarray(lo), k, n_sink=n_sink)
    got = cpu(idx).numpy()
    bad = np.nonzero((got != ref).any(1))[0]
    assert bad.size == 0, (f"rows differ: {bad[:10]}; first {got[bad[0], :8]} vs "
                           f"{ref[bad[0], :8]}")
    if noalloc:
        idx2 = torch.full_like(idx, POISON_I32)
        dsa.topk_noalloc(St, lo_t, hi_t, k, idx2, n_sink=n_sink)
        torch.cuda.synchronize()
        assert torch.equal(idx2, idx)


@pytest.mark.parametrize("n,k", [(131072, 2048), (131072, 5), (40000, 777)])
def test_topk_long_distributions(dsa, n, k):
    """One row per distribution, full visibility, in one launch."""
    note(f"topk long rows, every distribution, n={n} k={k}")
    rng = np.random.default_rng(n + k)
    S = np.stack([_row(kind, n, rng) for kind in KINDS]).astype(np.float32)
    _check(dsa, S, [0] * len(KINDS), [n] * len(KINDS), k)


def test_topk_long_visibility_and_sinks(dsa):
    """Visible ranges that start and end inside blocks, cover fewer keys than
    k, sit inside one block, or are empty; with and without sinks; and the
    allocation-free entry point."""
    note("topk long rows, visibility windows and sinks")
    n, k = 131072, 2048
    rng = np.random.default_rng(7)
    kinds = ["normal", "quantised", "relu_like", "outlier_per_block", "all_equal", "increasing",
             "normal", "normal"]
    S = np.stack([_row(kd, n, rng) for kd in kinds]).astype(np.float32)
    lo = [300, 4095, 0, 77, 5000, 130000, 9000, 12345]
    hi = [n, 100000, 1500, 4100, 9000, n, 9000, 12346]   # 1500 < k; an empty row; one key
    for n_sink in (0, 1, 3):
        _check(dsa, S, lo, hi, k, n_sink=n_sink, noalloc=True)


@pytest.mark.parametrize("n", [16385, 262144])
def test_topk_long_path_limits(dsa, n):
    """The shortest and the longest rows the shared-threshold path takes."""
    note(f"topk long rows at the path's limits, n={n}")
    rng = np.random.default_rng(n)
    kinds = ["normal", "quantised", "outlier_per_block", "two_clusters"]
    S = np.stack([_row(kd, n, rng) for kd in kinds]).astype(np.float32)
    _check(dsa, S, [0, 11, 0, 3], [n, n - 5, n, n], 2048, noalloc=True)


def test_topk_long_many_rows(dsa):
    """300 rows of 20000 keys (1500 blocks per launch), ties on every third
    row, windows on every fourth."""
    note("topk long rows, 300 x 20000")
    rows, n, k = 300, 20000, 2048
    rng = np.random.default_rng(3)
    S = rng.standard_normal((rows, n)).astype(np.float32)
    S[::3] = np.round(S[::3] * 20.0) / 20.0
    lo = np.zeros(rows, np.int64)
    hi = np.full(rows, n)
    lo[1::4] = 1000
    hi[1::4] = n - 333
    _check(dsa, S, lo, hi, k)


@pytest.mark.parametrize("rows,k", [(4, 800), (2, 100), (2, 2048)])
def test_topk_chunked_beyond_the_threshold_path(dsa, rows, k):
    """300000-key rows take the chunked path: a segmented merge over cached
    chunk winners (4 rows, k 800), one cached merge block per row (k 100) and
    the streaming merge (k 2048: 19 chunks of winners exceed the cache)."""
    note(f"topk chunked path rows={rows} k={k}")
    n = 300000
    rng = np.random.default_rng(rows * k)
    S = rng.standard_normal((rows, n)).astype(np.float32)
    S[0, 200000:210000] += 30.0           # every winner of row 0 in one chunk
    S[1] = np.round(S[1] * 8) / 8
    lo = [0, 17] + [5] * (rows - 2)
    hi = [n, n - 1000] + [n] * (rows - 2)
    _check(dsa, S, lo, hi, k)
