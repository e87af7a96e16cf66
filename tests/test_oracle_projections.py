"""Pins of the oracle's dense projections ahead of the path: linear,
LayerNorm with bias, NEOX rotary embedding, the indexer front-end and
expand_kv ("Module glm5next_dsa_ref": linear, layer_norm, expand_kv and the
k_norm / NoPE invariants; "Another DSA attempt": the batch-local indexer
commit's front-end, the CPU crash-fix commit and the review on the k_norm
eps).  Each pin checks the oracle against something other than itself:
explicit loops, torch's float64 LayerNorm, the complex-number form of the
rotation, closed forms and invariants."""
import numpy as np
import pytest
import torch

import oracle


def test_linear_is_x_times_w_transposed():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 5))
    w = rng.standard_normal((4, 5))
    y = oracle.linear(x, w)
    for i in range(3):
        for j in range(4):
            assert abs(y[i, j] - sum(x[i, t] * w[j, t] for t in range(5))) < 1e-12
    # bf16 operands are decoded exactly from their bits
    xb = torch.tensor(x, dtype=torch.float32).bfloat16()
    assert np.array_equal(oracle.linear(xb, np.eye(5)), xb.double().numpy())


def test_layer_norm_against_torch_and_closed_forms():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((6, 128)) * 3 + 1.5
    w = rng.standard_normal(128)
    b = rng.standard_normal(128)
    for eps in (1e-6, 1e-5):
        ref = torch.nn.functional.layer_norm(torch.tensor(x), (128,), torch.tensor(w),
                                             torch.tensor(b), eps).numpy()
        assert np.allclose(oracle.layer_norm(x, w, b, eps), ref, rtol=0, atol=1e-12)
    # a constant row normalises to zero: the output is the bias
    assert np.allclose(oracle.layer_norm(np.full((1, 8), 7.0), np.ones(8), b[:8], 1e-6), b[:8])
    # the mean is subtracted (LayerNorm, not RMSNorm): a shifted row gives the same output
    assert np.allclose(oracle.layer_norm(x + 100.0, w, b, 1e-6), oracle.layer_norm(x, w, b, 1e-6),
                       atol=1e-9)
    # eps enters inside the root: a row of +-1 has variance 1
    y = oracle.layer_norm(np.array([[1.0, -1.0, 1.0, -1.0]]), np.ones(4), np.zeros(4), 0.25)
    assert np.allclose(y, np.array([[1, -1, 1, -1]]) / np.sqrt(1.25))


def test_rope_neox_against_the_complex_form():
    rng = np.random.default_rng(3)
    T, H, D, R, theta = 5, 3, 16, 8, 10000.0
    x = rng.standard_normal((T, H, D))
    pos = np.array([0, 1, 7, 100, 16383])
    y = oracle.rope_neox(x, pos, R, theta)
    h = R // 2
    for t in range(T):
        for i in range(h):
            z = (x[t, :, i] + 1j * x[t, :, i + h]) * np.exp(1j * pos[t] * theta ** (-2 * i / R))
            assert np.allclose(y[t, :, i], z.real, atol=1e-12)
            assert np.allclose(y[t, :, i + h], z.imag, atol=1e-12)
    assert np.array_equal(y[..., R:], x[..., R:])          # the nope part passes through
    assert np.allclose(y[0], x[0], atol=0)                  # position 0: identity


def test_rope_pairs_i_with_i_plus_half():
    """NEOX pairing (i, i + R/2), not adjacent entries (2i, 2i + 1)."""
    x = np.zeros((1, 8))
    x[0, 1] = 1.0
    y = oracle.rope_neox(x, [3], 8, 10000.0)
    nz = set(np.nonzero(np.abs(y[0]) > 1e-15)[0])
    assert nz == {1, 5}


def test_rope_scores_depend_on_relative_position_only():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((1, 64))
    k = rng.standard_normal((1, 64))
    for m, n in ((10, 3), (5000, 4993), (16383, 16376)):
        a = (oracle.rope_neox(q, [m], 64, 10000.0) @ oracle.rope_neox(k, [n], 64, 10000.0).T)[0, 0]
        b = (oracle.rope_neox(q, [m - n], 64, 10000.0) @ k.T)[0, 0]
        assert abs(a - b) < 1e-9 * (np.abs(q).sum() * np.abs(k).sum())


def test_indexer_frontend_composition_and_shift_invariance():
    """The front-end's pieces in the pages' order, and index scores over its
    outputs unchanged when every position moves by the same offset (the
    rotation only sees relative positions; q and k rotate alike)."""
    rng = np.random.default_rng(5)
    T, Hi, d, R, r_q, hid = 6, 4, 32, 16, 24, 40
    ql = rng.standard_normal((T, r_q))
    x = rng.standard_normal((T, hid))
    wq = rng.standard_normal((Hi * d, r_q)) / 5
    wk = rng.standard_normal((d, hid)) / 6
    g, bta = rng.standard_normal(d), rng.standard_normal(d)
    wp = rng.standard_normal((Hi, hid))
    pos = np.arange(T) + 11
    q, k, w = oracle.indexer_frontend(ql, x, pos, wq, wk, g, bta, wp, Hi, R, 10000.0, 1e-6)
    q0 = oracle.rope_neox((ql @ wq.T).reshape(T, Hi, d), pos, R, 10000.0)
    kk = x @ wk.T
    kn = (kk - kk.mean(1, keepdims=True)) / np.sqrt(kk.var(1, keepdims=True) + 1e-6) * g + bta
    assert np.allclose(q, q0, atol=1e-12)
    assert np.allclose(k, oracle.rope_neox(kn, pos, R, 10000.0), atol=1e-12)
    assert np.allclose(w, x @ wp.T, atol=1e-12)
    q2, k2, _ = oracle.indexer_frontend(ql, x, pos + 1000, wq, wk, g, bta, wp, Hi, R, 10000.0,
                                        1e-6)
    S1 = np.einsum("thd,sd->ths", q, k)
    S2 = np.einsum("thd,sd->ths", q2, k2)
    assert np.allclose(S1, S2, atol=1e-9)


def test_expand_kv_splits_each_head_key_then_value():
    rng = np.random.default_rng(6)
    T, r, H, kd, vd = 3, 10, 4, 6, 5
    lat = rng.standard_normal((T, r))
    w = rng.standard_normal((H * (kd + vd), r))
    K, V = oracle.expand_kv(lat, w, H, kd, vd)
    assert K.shape == (T, H, kd) and V.shape == (T, H, vd)
    for h in range(H):
        rows = w[h * (kd + vd):(h + 1) * (kd + vd)]
        assert np.allclose(K[:, h], lat @ rows[:kd].T, atol=1e-12)
        assert np.allclose(V[:, h], lat @ rows[kd:].T, atol=1e-12)
    # an identity block reproduces the latent in head 0's keys
    w2 = np.zeros((H * (kd + vd), r))
    w2[:kd, :kd] = np.eye(kd)
    K2, _ = oracle.expand_kv(lat, w2, H, kd, vd)
    assert np.array_equal(K2[:, 0], lat[:, :kd])
