"""GPU parity of the Walsh-Hadamard rotation and the indexer-key cache write
("Another DSA attempt": the decode indexer-K cache commit -- keys rotated and
written to the cache at kv_head, queries rotated the same way -- and the
serving-correctness commit -- the Sylvester construction) against the oracle:
bit-exact rotated values, fp8 codes, row scales and untouched rows; then the
decode step as write-then-score."""
import numpy as np
import pytest
import torch

import oracle
from sparse_attention_scores_amd import workloads as W
from tests.parity import check_scores, cpu, note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    from sparse_attention_scores_amd import binding
    binding.load()
    return binding


def _bf16_bits(t):
    return cpu(t).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("d", [32, 64, 128, 256])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_rotation_bit_exact(dsa, d, dtype):
    note(f"hadamard rotate d={d} {dtype}")
    gen = torch.Generator(device="cuda").manual_seed(d)
    x = (torch.randn(37, d, generator=gen, device="cuda") * 3).to(dtype)
    y32 = dsa.hadamard_rotate(x, out_dtype=torch.float32)
    y16 = dsa.hadamard_rotate(x, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref = oracle.hadamard_rows(cpu(x))
    assert np.array_equal(cpu(y32).numpy(), ref)
    assert np.array_equal(_bf16_bits(y16), _bf16_bits(torch.from_numpy(ref).bfloat16()))
    # in place
    z = x.clone()
    dsa.hadamard_rotate(z, out=z)
    torch.cuda.synchronize()
    assert torch.equal(cpu(z), torch.from_numpy(ref).to(dtype))


def _cache_case(dsa, B, n_new, n_cache, d, heads, k_new, fp8=True, seed=0):
    gen = torch.Generator(device="cuda").manual_seed(seed)
    if fp8:
        cache = torch.randint(0, 256, (B, n_cache, d), generator=gen, device="cuda",
                              dtype=torch.uint8)
        cache[cache == 0x7F] = 0   # no NaN codes in the untouched rows
        cache[cache == 0xFF] = 0
        scales = torch.rand(B, n_cache, generator=gen, device="cuda")
        c0, s0 = cpu(cache).numpy().copy(), cpu(scales).numpy().copy()
        kv = torch.tensor(heads, dtype=torch.int32, device="cuda")
        dsa.index_cache_write(k_new, kv, cache.view(torch.float8_e4m3fn), scales)
        torch.cuda.synchronize()
        rc, rs = oracle.index_cache_write(cpu(k_new), heads, c0, s0)
        assert np.array_equal(cpu(cache).numpy(), rc), "fp8 codes differ"
        assert np.array_equal(cpu(scales).numpy(), rs), "row scales differ"
    else:
        cache = torch.randn(B, n_cache, d, generator=gen, device="cuda").bfloat16()
        c0 = _bf16_bits(cache).copy()
        kv = torch.tensor(heads, dtype=torch.int32, device="cuda")
        dsa.index_cache_write(k_new, kv, cache)
        torch.cuda.synchronize()
        rc, _ = oracle.index_cache_write(cpu(k_new), heads, c0)
        assert np.array_equal(_bf16_bits(cache), rc), "bf16 rows differ"


@pytest.mark.parametrize("d", [32, 64, 128, 256])
def test_cache_write_fp8_and_bf16(dsa, d):
    """Random rows (bf16 and f32 inputs), an all-zero row, a row of widely
    spread magnitudes; kv_head at the start, in the middle, one row short of
    the end (the overflowing row is dropped) and negative (dropped)."""
    note(f"index cache write d={d}")
    B, n_new, n_cache = 4, 3, 23
    gen = torch.Generator(device="cuda").manual_seed(100 + d)
    k = torch.randn(B, n_new, d, generator=gen, device="cuda")
    k[1, 1] = 0.0
    k[2, 0] = torch.logspace(-8, 8, d, device="cuda") * torch.sign(torch.randn(d, generator=gen, device="cuda"))
    heads = [0, 9, n_cache - 2, -1]
    for kd in (k, k.bfloat16()):
        _cache_case(dsa, B, n_new, n_cache, d, heads, kd, fp8=True, seed=d)
        _cache_case(dsa, B, n_new, n_cache, d, heads, kd, fp8=False, seed=d)


def test_cache_write_fp8_rounding_ties(dsa):
    """Rows built so that the rotated values land exactly on e4m3 rounding
    midpoints (and a hair either side) with a power-of-two row scale: d = 64
    (sqrt(d) = 8), x = H y / 8 is exact in f32 for dyadic y, so the kernel's
    rotation reproduces y exactly and the codes test the ties-to-even rule."""
    note("index cache write: e4m3 ties")
    import scipy.linalg
    d = 64
    H = scipy.linalg.hadamard(d).astype(np.float64)
    vals = np.array([oracle.e4m3_value(c) for c in range(127)])
    mids = (vals[:-1] + vals[1:]) / 2
    rows = []
    rng = np.random.default_rng(1)
    for scale_pow in (0, -6):
        sel = mids[(mids >= 2.0 ** -4) & (mids < 400)]
        for start in range(0, len(sel), d - 1):
            y = np.zeros(d)
            chunk = sel[start:start + d - 1]
            y[:len(chunk)] = chunk * rng.choice([-1, 1], len(chunk))
            y[d - 1] = 448.0                       # the row maximum: scale 2^scale_pow
            rows.append(y * 2.0 ** scale_pow)
    y = np.stack(rows)
    x = (y @ H) / 8.0                               # H symmetric: H y / sqrt(d) inverts the rotation
    x32 = x.astype(np.float32)
    k_new = torch.tensor(x32.reshape(len(rows), 1, d), device="cuda")
    _cache_case(dsa, len(rows), 1, 2, d, [1] * len(rows), k_new, fp8=True, seed=7)
    # the construction is exact, so the rotated values are the intended midpoints
    assert np.array_equal(oracle.hadamard_rows(x32), y.astype(np.float32))


def test_decode_write_then_score(dsa):
    """Long-decode shape, reduced: the keys of the context go into an fp8
    cache through the cache write (rotated, quantised per row), the new
    token's key is appended at kv_head, the queries are rotated, and the
    indexer scores the rotated queries against the cache.  Parity on the
    GPU's own cache and rotated queries; against the unrotated f64 scores the
    difference is the fp8 quantisation alone."""
    note("decode: cache write then score")
    inp = W.make(4, device="cuda", B=2, Tk=3000)
    B, Tk, d, Hi = inp["B"], inp["Tk"], inp["d"], inp["Hi"]
    gen = torch.Generator(device="cuda").manual_seed(5)
    kf = torch.randn(B, Tk, d, generator=gen, device="cuda") / d ** 0.5
    cache = torch.zeros(B, Tk, d, dtype=torch.uint8, device="cuda").view(torch.float8_e4m3fn)
    scales = torch.zeros(B, Tk, device="cuda")
    zero = torch.zeros(B, dtype=torch.int32, device="cuda")
    dsa.index_cache_write(kf[:, :Tk - 1].contiguous(), zero, cache, scales)
    last = torch.full((B,), Tk - 1, dtype=torch.int32, device="cuda")
    dsa.index_cache_write(kf[:, Tk - 1:].contiguous(), last, cache, scales)
    q_rot = dsa.hadamard_rotate(inp["q_idx"])
    lo, hi = dsa.visibility_ranges(inp["pad"], inp["q_pos"])
    S = dsa.index_scores(q_rot, cache, inp["w"], lo, hi, inp["scale_idx"], k_scale=scales)
    torch.cuda.synchronize()
    ref, A = oracle.index_scores(cpu(q_rot), cpu(cache), cpu(inp["w"]), inp["scale_idx"],
                                 cpu(inp["q_pos"]), cpu(inp["pad"]), k_scale=cpu(scales),
                                 want_mag=True)
    check_scores(cpu(S).numpy().reshape(ref.shape), ref, A, 1e-3, "write then score",
                 d=d, heads=Hi)
    # the cache holds exactly the oracle's rotated, quantised rows
    rc, rs = oracle.index_cache_write(cpu(kf), np.zeros(B, np.int32),
                                      np.zeros((B, Tk, d), np.uint8), np.zeros((B, Tk), np.float32))
    assert np.array_equal(cpu(cache.view(torch.uint8)).numpy(), rc)
    assert np.array_equal(cpu(scales).numpy(), rs)
    # against the unrotated exact scores: within the fp8 quantisation error
    exact = oracle.index_scores(cpu(inp["q_idx"]), cpu(kf).numpy().astype(np.float64),
                                cpu(inp["w"]), inp["scale_idx"], cpu(inp["q_pos"]),
                                cpu(inp["pad"]))
    vis = exact > -3e38
    rel = np.abs(ref[vis].astype(np.float64) - exact[vis]) / (A[vis] + 1e-30)
    assert float(rel.max()) < 0.1, float(rel.max())
