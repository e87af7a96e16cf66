"""The allocation-free top-k (dsa_topk_noalloc) against dsa_topk with a
caller workspace, through the C ABI: bit-exact, on two calls in a row (the
second smaller, so the scratch holds the first call's winners when it
starts), and on rows short enough to need no scratch at all."""
import pytest
import torch

from tests.parity import cpu, note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    from sparse_attention_scores_amd import binding
    binding.load()
    return binding


def _rows(rows, n, seed, window=False):
    gen = torch.Generator(device="cuda").manual_seed(seed)
    S = torch.randn(rows, n, generator=gen, device="cuda")
    S[::2] = torch.round(S[::2] * 16.0) / 16.0   # exact ties in every other row
    lo = torch.zeros(rows, dtype=torch.int32, device="cuda")
    hi = torch.full((rows,), n, dtype=torch.int32, device="cuda")
    if window:
        lo[1::3] = 777
        hi[1::3] = n - 4321
    return S, lo, hi


def _both(dsa, S, lo, hi, k):
    ws = torch.empty(max(dsa.topk_workspace_size(S.shape[0], S.shape[1], k), 1),
                     dtype=torch.uint8, device="cuda")
    ref = dsa.topk(S, lo, hi, k, workspace=ws)
    got = torch.full_like(ref, 0x7EADBEEF)
    dsa.topk_noalloc(S, lo, hi, k, got)
    torch.cuda.synchronize()
    return cpu(got), cpu(ref)


def test_noalloc_topk_matches_workspace_topk_twice(dsa):
    # the long-context decode shape: 8 rows of 131072 keys, k 2048 (1 MiB of scratch)
    note("no-alloc top-k: 8 x 131072, k 2048")
    S, lo, hi = _rows(8, 131072, 1, window=True)
    got, ref = _both(dsa, S, lo, hi, 2048)
    assert torch.equal(got, ref)
    # a second, smaller call right after: fewer rows, fewer chunks, smaller k
    note("no-alloc top-k: 3 x 40000, k 700 (second call)")
    S2, lo2, hi2 = _rows(3, 40000, 2)
    got2, ref2 = _both(dsa, S2, lo2, hi2, 700)
    assert torch.equal(got2, ref2)


def test_noalloc_topk_near_its_limit_then_short_rows(dsa):
    # 60 rows x 8 chunks x 2048 x 8 bytes = 7.5 MiB of scratch, one merge block per row
    note("no-alloc top-k: 60 x 131072, k 2048")
    S, lo, hi = _rows(60, 131072, 3, window=True)
    got, ref = _both(dsa, S, lo, hi, 2048)
    assert torch.equal(got, ref)
    # rows of at most 16384 keys use no scratch
    note("no-alloc top-k: 32 x 8192, k 2048 (no scratch)")
    S2, lo2, hi2 = _rows(32, 8192, 4)
    got2, ref2 = _both(dsa, S2, lo2, hi2, 2048)
    assert torch.equal(got2, ref2)
