"""Pins of the oracle's indexer-key cache write: the Sylvester Hadamard
rotation, the OCP e4m3 encoder and the per-row fp8 quantisation
("Another DSA attempt": the decode indexer-K cache commit -- rotated keys
written to the per-layer cache at kv_head, the rotation score-preserving --
and the serving-correctness commit -- the Sylvester construction, H
symmetric and orthonormal).  Each pin checks the oracle against something
other than itself: scipy's Hadamard matrix, the index-score definition,
torch's float8_e4m3fn conversion, closed forms."""
import numpy as np
import pytest
import scipy.linalg
import torch

import oracle


@pytest.mark.parametrize("d", [2, 8, 32, 64, 128, 256])
def test_rotation_is_scipy_sylvester_hadamard_over_sqrt_d(d):
    _, R = oracle.hadamard_rows(np.eye(d), want_f64=True)   # row i = H e_i / sqrt(d)
    H = scipy.linalg.hadamard(d).astype(np.float64) / np.sqrt(d)
    assert np.allclose(R, H.T, rtol=0, atol=1e-15)
    assert np.allclose(R, R.T, rtol=0, atol=1e-15)            # symmetric
    assert np.allclose(R @ R.T, np.eye(d), rtol=0, atol=1e-12)  # orthonormal: H H = I


def test_rotation_closed_forms():
    d = 128
    ones = np.ones((1, d))
    _, y = oracle.hadamard_rows(ones, want_f64=True)
    expect = np.zeros((1, d))
    expect[0, 0] = np.sqrt(d)                  # H 1 = d e_0, over sqrt(d)
    assert np.allclose(y, expect, atol=1e-12)
    e0 = np.zeros((1, d))
    e0[0, 0] = 1.0
    _, y = oracle.hadamard_rows(e0, want_f64=True)
    assert np.allclose(y, np.full((1, d), 1 / np.sqrt(d)), atol=1e-15)
    with pytest.raises(ValueError):
        oracle.hadamard_rows(np.ones((1, 48)))


def test_rotation_leaves_index_scores_unchanged():
    """The rotation is score-preserving: index scores of (Hq, Hk) equal those
    of (q, k) -- the same orthonormal H on the queries and on the keys."""
    rng = np.random.default_rng(3)
    B, Tq, Tk, Hh, d = 2, 3, 40, 4, 64
    q = rng.standard_normal((B, Tq, Hh, d))
    k = rng.standard_normal((B, Tk, d))
    w = rng.uniform(size=(B, Tq, Hh)).astype(np.float32)
    q_pos = np.full((B, Tq), Tk - 1, np.int32)
    pad = np.zeros(B, np.int32)
    _, hq = oracle.hadamard_rows(q, want_f64=True)
    _, hk = oracle.hadamard_rows(k, want_f64=True)
    S0, A0 = oracle.index_scores(q, k, w, 0.125, q_pos, pad, want_mag=True)
    S1 = oracle.index_scores(hq, hk, w, 0.125, q_pos, pad)
    # both rounded once to f32 from f64 values that differ by f64 rounding
    assert np.all(np.abs(S1.astype(np.float64) - S0) <= 1e-6 * np.abs(S0) + 1e-12 * A0)


def test_e4m3_encoder_matches_torch_rounding():
    """Every representable value, every midpoint between neighbours (ties
    to even) and values a hair either side of the midpoints, across the
    subnormal and normal ranges up to 448."""
    vals = np.array([oracle.e4m3_value(c) for c in range(127)])   # 0 .. 448
    mids = (vals[:-1] + vals[1:]) / 2
    probes = np.concatenate([vals, mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
                             np.linspace(0, 448, 4001)]).astype(np.float32)
    probes = np.concatenate([probes, -probes])
    ours = oracle.e4m3_encode(probes)
    ref = torch.from_numpy(probes).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_encoder_round_trips_codes_and_saturates():
    for c in range(127):
        v = np.float32(oracle.e4m3_value(c))
        assert oracle.e4m3_encode(v) == c
        assert oracle.e4m3_encode(-v) == c | 0x80
    # beyond the largest finite value: saturation (reading), never NaN (0x7f)
    assert oracle.e4m3_encode(np.float32(449.0)) == 0x7E
    assert oracle.e4m3_encode(np.float32(1e6)) == 0x7E
    assert oracle.e4m3_encode(np.float32(-3e38)) == 0xFE


def test_row_quantisation_scale_and_error_bound():
    rng = np.random.default_rng(5)
    y = rng.standard_normal((50, 128)).astype(np.float32) * rng.uniform(1e-3, 1e3, (50, 1)).astype(np.float32)
    y[7] = 0.0
    codes, sc = oracle.quantize_e4m3_rows(y)
    assert sc[7] == 1.0 and np.all(codes[7] == 0)
    for r in range(50):
        if r == 7:
            continue
        mx = np.abs(y[r]).max()
        assert sc[r] == np.float32(mx) / np.float32(448.0)
        imax = int(np.argmax(np.abs(y[r])))
        assert codes[r, imax] & 0x7F == 0x7E                  # the largest maps to 448
        deq = np.array([oracle.e4m3_value(int(c)) for c in codes[r]]) * np.float64(sc[r])
        # e4m3 has 4 significant bits: half an ulp is 2^-4 relative in the
        # normal range; below it (|y/s| < 2^-6) the spacing is 2^-9 absolute
        err = np.abs(deq - y[r].astype(np.float64))
        bound = np.maximum(np.abs(y[r]) * 2.0 ** -4, 2.0 ** -10 * sc[r]) * (1 + 1e-6)
        assert np.all(err <= bound)


def test_cache_write_rows_and_untouched_rows():
    rng = np.random.default_rng(9)
    B, n_new, d, n_cache = 3, 2, 32, 10
    k_new = rng.standard_normal((B, n_new, d)).astype(np.float32)
    cache = rng.integers(0, 256, (B, n_cache, d)).astype(np.uint8)
    scales = rng.uniform(size=(B, n_cache)).astype(np.float32)
    heads = np.array([0, 8, 9], np.int32)                      # the last one overflows by one
    c2, s2 = oracle.index_cache_write(k_new, heads, cache, scales)
    y = oracle.hadamard_rows(k_new)
    codes, sc = oracle.quantize_e4m3_rows(y)
    for b in range(B):
        for r in range(n_cache):
            i = r - heads[b]
            if 0 <= i < n_new:
                assert np.array_equal(c2[b, r], codes[b, i]) and s2[b, r] == sc[b, i]
            else:
                assert np.array_equal(c2[b, r], cache[b, r]) and s2[b, r] == scales[b, r]
    # bf16 cache: the rotated rows rounded to bf16
    cb = np.zeros((B, n_cache, d), np.uint16)
    c3, s3 = oracle.index_cache_write(k_new, heads, cb)
    assert s3 is None
    got = torch.from_numpy(c3.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(got[0, 0:2], torch.from_numpy(y[0]).bfloat16().float().numpy())
    assert np.all(c3[0, 2:] == 0)
