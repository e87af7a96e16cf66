"""Pins of the oracle's storage decoders and index scores (CPU only).

Index score (page "Module glm5next_dsa_ref", index_scores; page "GLM-5.2: the
DSA sparse attention moves onto the pure fak kernel", section "The selection
stays host-side BY DESIGN"): score[q,s] = sum_h w[q,h] * relu(scale * q_h . k_s)
over visible keys (page "Module glm5next_dsa_ref", visible: causal and not
padding)."""
import math

import numpy as np
import pytest
import torch

import oracle

FLT_MAX = np.finfo(np.float32).max


# ---------------------------------------------------------------- decoders

def test_bf16_decoder_all_codes_match_torch():
    codes = np.arange(65536, dtype=np.uint16)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = np.array([oracle.bf16_value(int(c)) for c in codes[::7]])
    r = ref[::7]
    both_nan = np.isnan(got) & np.isnan(r)
    assert np.all((got == r) | both_nan)


def test_e4m3_decoder_all_codes_match_torch_and_spec():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    got = np.array([oracle.e4m3_value(int(c)) for c in codes])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # values fixed by the OCP e4m3fn definition
    assert oracle.e4m3_value(0x38) == 1.0
    assert oracle.e4m3_value(0x7E) == 448.0
    assert oracle.e4m3_value(0xFE) == -448.0
    assert oracle.e4m3_value(0x01) == 2.0 ** -9
    assert oracle.e4m3_value(0x08) == 2.0 ** -6
    assert math.isnan(oracle.e4m3_value(0x7F)) and math.isnan(oracle.e4m3_value(0xFF))
    assert oracle.e4m3_value(0x80) == 0.0


# ---------------------------------------------------------------- helpers

def _dense_ref(q, k, w, scale, q_pos, pad):
    """Straight numpy statement of the definition (f64)."""
    B, Tq, H, d = q.shape
    Tk = k.shape[1]
    logits = np.einsum("bthc,bsc->bths", q, k) * scale
    S = np.einsum("bth,bths->bts", w, np.maximum(logits, 0.0))
    s = np.arange(Tk)
    vis = (s[None, None, :] >= pad[:, None, None]) & (s[None, None, :] <= q_pos[:, :, None])
    return np.where(vis, S, -np.inf), vis


def _rand(shape, rng):
    return rng.standard_normal(shape)


# ---------------------------------------------------------------- index scores

def test_index_single_head_unit_weight_is_relu_gemm():
    rng = np.random.default_rng(1)
    B, T, d = 2, 33, 16
    q = _rand((B, T, 1, d), rng)
    k = _rand((B, T, d), rng)
    w = np.ones((B, T, 1))
    q_pos = np.full((B, T), T - 1)  # every key visible
    pad = np.zeros(B)
    S = oracle.index_scores(q, k, w, 0.3, q_pos, pad)
    ref = np.maximum(0.3 * np.matmul(q[:, :, 0, :], np.swapaxes(k, 1, 2)), 0.0)
    np.testing.assert_allclose(S.reshape(B, T, T), ref, rtol=1e-7, atol=1e-30)


def test_index_brute_force_heads_weights_negative_scale():
    rng = np.random.default_rng(2)
    B, Tq, Tk, H, d = 2, 5, 9, 3, 8
    q = _rand((B, Tq, H, d), rng)
    k = _rand((B, Tk, d), rng)
    w = rng.uniform(-1, 1, (B, Tq, H))
    q_pos = np.array([[0, 3, 4, 7, 8], [2, 2, 5, 6, 8]])
    pad = np.array([0, 2])
    for scale in (0.7, -0.45):
        S = oracle.index_scores(q, k, w, scale, q_pos, pad).reshape(B, Tq, Tk)
        ref, vis = _dense_ref(q, k, w, scale, q_pos, pad)
        np.testing.assert_allclose(S[vis], ref[vis], rtol=2e-7, atol=1e-12)
        assert np.all(S[~vis] == -FLT_MAX)


def test_index_visibility_is_causal_inclusive_and_skips_padding():
    rng = np.random.default_rng(3)
    B, T, H, d = 1, 8, 2, 4
    q = np.abs(_rand((B, T, H, d), rng))
    k = np.abs(_rand((B, T, d), rng))  # positive dots: every visible score > 0
    w = np.ones((B, T, H))
    q_pos = np.arange(T)[None, :]
    pad = np.array([3])
    S = oracle.index_scores(q, k, w, 1.0, q_pos, pad).reshape(T, T)
    for t in range(T):
        for s in range(T):
            visible = 3 <= s <= t
            assert (S[t, s] > 0) == visible, (t, s)
            assert (S[t, s] == -FLT_MAX) == (not visible)


def test_index_zero_weights_give_zero():
    rng = np.random.default_rng(4)
    q = _rand((1, 4, 3, 8), rng)
    k = _rand((1, 4, 8), rng)
    S = oracle.index_scores(q, k, np.zeros((1, 4, 3)), 1.0, np.full((1, 4), 3), [0])
    assert np.all(S == 0.0)


def _sylvester(n):
    h = np.array([[1.0]])
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h / math.sqrt(n)


@pytest.mark.parametrize("d", [32, 128])
def test_index_hadamard_rotation_leaves_scores_unchanged(d):
    rng = np.random.default_rng(5)
    B, T, H = 1, 16, 4
    q = _rand((B, T, H, d), rng)
    k = _rand((B, T, d), rng)
    w = rng.uniform(0, 1, (B, T, H))
    q_pos = np.arange(T)[None, :]
    pad = [0]
    Hm = _sylvester(d)
    assert np.allclose(Hm @ Hm.T, np.eye(d))
    S0 = oracle.index_scores(q, k, w, 1 / math.sqrt(d), q_pos, pad)
    S1 = oracle.index_scores(q @ Hm.T, k @ Hm.T, w, 1 / math.sqrt(d), q_pos, pad)
    vis = S0 != -FLT_MAX
    np.testing.assert_allclose(S1[vis], S0[vis], rtol=1e-6, atol=1e-12)
    assert np.array_equal(S0 == -FLT_MAX, S1 == -FLT_MAX)


def test_index_bf16_and_fp8_inputs_decode_exactly():
    rng = np.random.default_rng(6)
    B, T, H, d = 1, 6, 2, 16
    qf = torch.from_numpy(_rand((B, T, H, d), rng)).float()
    kf = torch.from_numpy(_rand((B, T, d), rng)).float()
    qb = qf.to(torch.bfloat16)
    k8 = (kf * 20).clamp(-448, 448).to(torch.float8_e4m3fn)
    ks = torch.full((B, T), 0.05)
    w = np.ones((B, T, H))
    q_pos = np.full((B, T), T - 1)
    S = oracle.index_scores(qb, k8, w, 0.5, q_pos, [0], k_scale=ks)
    qd = qb.double().numpy()
    kd = k8.double().numpy() * 0.05
    ref, vis = _dense_ref(qd, kd, w, 0.5, q_pos, np.array([0]))
    np.testing.assert_allclose(S.reshape(B, T, T), ref, rtol=2e-7, atol=1e-12)


def test_index_magnitude_bounds_score():
    rng = np.random.default_rng(7)
    q = _rand((1, 5, 3, 8), rng)
    k = _rand((1, 5, 8), rng)
    w = rng.uniform(-1, 1, (1, 5, 3))
    S, A = oracle.index_scores(q, k, w, 0.9, np.full((1, 5), 4), [0], want_mag=True)
    assert np.all(np.abs(S) <= A * (1 + 1e-6))


def test_index_pooled_visibility():
    # pool i (tokens pad + i*kpool .. pad + i*kpool + kpool - 1) is a candidate
    # for query qpos iff qpos >= pad and its last token is <= qpos
    pad, kpool = 2, 4
    assert not oracle.pool_visible(pad, kpool, 1, 0)   # padded query
    assert not oracle.pool_visible(pad, kpool, 4, 0)   # pool 0 = tokens 2..5
    assert oracle.pool_visible(pad, kpool, 5, 0)
    assert not oracle.pool_visible(pad, kpool, 8, 1)   # pool 1 = tokens 6..9
    assert oracle.pool_visible(pad, kpool, 9, 1)
    rng = np.random.default_rng(8)
    L, d, H = 14, 4, 2
    NP = L // kpool
    q = np.abs(_rand((1, L, H, d), rng))
    pk = np.abs(_rand((1, NP, d), rng))
    S = oracle.index_scores(q, pk, np.ones((1, L, H)), 1.0, np.arange(L)[None], [pad],
                            kpool=kpool).reshape(L, NP)
    for t in range(L):
        n_full = (t - pad + 1) // kpool if t >= pad else 0
        for i in range(NP):
            assert (S[t, i] != -FLT_MAX) == (i < n_full), (t, i)


def test_index_batch_invariance():
    rng = np.random.default_rng(9)
    B, T, H, d = 3, 7, 2, 8
    q = _rand((B, T, H, d), rng)
    k = _rand((B, T, d), rng)
    w = rng.uniform(0, 1, (B, T, H))
    q_pos = np.tile(np.arange(T), (B, 1))
    pad = np.array([0, 1, 3])
    S = oracle.index_scores(q, k, w, 0.4, q_pos, pad).reshape(B, T, T)
    for b in range(B):
        Sb = oracle.index_scores(q[b:b + 1], k[b:b + 1], w[b:b + 1], 0.4, q_pos[b:b + 1],
                                 pad[b:b + 1]).reshape(T, T)
        assert np.array_equal(S[b], Sb)


def test_index_rows_subset_matches_full():
    rng = np.random.default_rng(10)
    q = _rand((2, 6, 2, 4), rng)
    k = _rand((2, 6, 4), rng)
    w = rng.uniform(0, 1, (2, 6, 2))
    q_pos = np.tile(np.arange(6), (2, 1))
    full = oracle.index_scores(q, k, w, 1.0, q_pos, [0, 0])
    rows = [11, 0, 7]
    sub = oracle.index_scores(q, k, w, 1.0, q_pos, [0, 0], rows=rows)
    assert np.array_equal(sub, full[rows])
