"""Pins of the oracle's sparse attention (CPU only).

Definition (page "GLM-5.2: the DSA sparse attention moves onto the pure fak
kernel", table under "What changed": per-head softmax(scale*q*k) then the
in-order sum of w*V over the selected keys, key width kd = qk_nope + qk_rope
different from value width vd; page "Module glm5next_dsa_ref",
mla_masked_attention over a per-query selected set, topk_to_mask: duplicates
collapse, out-of-range and INVALID entries are dropped)."""
import math

import numpy as np
import pytest
import torch

import oracle

INV = oracle.INVALID


def _rand(shape, rng):
    return rng.standard_normal(shape)


def _masked_dense(q, K, V, mask, scale):
    """Brute force in the pages' mask form (ik_llama.cpp batch-local indexer
    commit): full scores, -inf outside the selected set, softmax, matmul."""
    Tq, H, _ = q.shape
    out = np.zeros((Tq, H, V.shape[-1]))
    for t in range(Tq):
        for h in range(H):
            s = K[:, h, :] @ q[t, h] * scale
            s = np.where(mask[t], s, -np.inf)
            if not mask[t].any():
                continue
            p = np.exp(s - s.max())
            out[t, h] = (p / p.sum()) @ V[:, h, :]
    return out


def test_topk_ge_n_keys_is_dense_causal_attention():
    """top_k >= n_keys makes the selection a no-op: the result is dense causal
    attention (checked against torch's scaled_dot_product_attention in f64)."""
    rng = np.random.default_rng(20)
    B, T, H, kd, vd = 2, 12, 3, 10, 6
    q = _rand((B, T, H, kd), rng)
    K = _rand((B, T, H, kd), rng)
    V = _rand((B, T, H, vd), rng)
    q_pos = np.tile(np.arange(T), (B, 1))
    idx = np.tile(np.arange(T, dtype=np.int32), (B, T, 1))  # every key listed
    scale = 1 / math.sqrt(kd)
    out, lse = oracle.sparse_attend(q, K, V, idx, scale, kv_heads=H, q_pos=q_pos,
                                    pad=np.zeros(B))
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(K).permute(0, 2, 1, 3)
    tv = torch.from_numpy(V).permute(0, 2, 1, 3)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True,
                                                           scale=scale)
    ref = ref.permute(0, 2, 1, 3).reshape(B * T, H, vd).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)
    # lse against the log-sum-exp of the causal logits
    logits = np.einsum("bthc,bshc->bths", q, K) * scale
    causal = np.tril(np.ones((T, T), bool))
    lref = np.log(np.where(causal[None, :, None, :], np.exp(logits), 0).sum(-1))
    np.testing.assert_allclose(lse, lref.reshape(B * T, H), rtol=1e-12)


def test_matches_masked_dense_brute_force():
    rng = np.random.default_rng(21)
    Tq, Tk, H, kd, vd, n_sel = 6, 15, 2, 8, 5, 7
    q = _rand((1, Tq, H, kd), rng)
    K = _rand((1, Tk, H, kd), rng)
    V = _rand((1, Tk, H, vd), rng)
    idx = rng.integers(-2, Tk + 3, (1, Tq, n_sel)).astype(np.int32)
    idx[0, 0, :] = INV                                           # empty row
    out, lse = oracle.sparse_attend(q, K, V, idx, 0.3, kv_heads=H)
    mask = np.zeros((Tq, Tk), bool)
    for t in range(Tq):
        for j in idx[0, t]:
            if 0 <= j < Tk:
                mask[t, j] = True
    ref = _masked_dense(q[0], K[0], V[0], mask, 0.3)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-14)
    assert np.all(out[0] == 0.0) and np.all(lse[0] == -np.inf)


def test_set_semantics_duplicates_invalid_out_of_range_permutation():
    rng = np.random.default_rng(22)
    Tk, H, kd, vd = 20, 2, 6, 4
    q = _rand((1, 1, H, kd), rng)
    K = _rand((1, Tk, H, kd), rng)
    V = _rand((1, Tk, H, vd), rng)
    base = np.array([[[3, 7, 11, 19]]], np.int32)
    noisy = np.array([[[11, INV, 3, 3, 25, 7, -5, 19, 11, 20]]], np.int32)
    perm = np.array([[[19, 3, 11, 7]]], np.int32)
    o0, l0 = oracle.sparse_attend(q, K, V, base, 0.5, kv_heads=H)
    o1, l1 = oracle.sparse_attend(q, K, V, noisy, 0.5, kv_heads=H)
    o2, l2 = oracle.sparse_attend(q, K, V, perm, 0.5, kv_heads=H)
    assert np.array_equal(o0, o1) and np.array_equal(o0, o2)
    assert np.array_equal(l0, l1) and np.array_equal(l0, l2)


def test_single_selected_key_returns_its_value_row():
    rng = np.random.default_rng(23)
    q = _rand((1, 1, 3, 5), rng)
    K = _rand((1, 9, 3, 5), rng)
    V = _rand((1, 9, 3, 4), rng)
    out, lse = oracle.sparse_attend(q, K, V, np.array([[[6]]], np.int32), 0.7, kv_heads=3)
    assert np.array_equal(out[0], V[0, 6])
    np.testing.assert_allclose(lse[0], 0.7 * np.einsum("hc,hc->h", q[0, 0], K[0, 6]),
                               rtol=1e-15)


def test_visibility_filter_drops_invisible_entries():
    rng = np.random.default_rng(24)
    T, H, kd, vd = 10, 2, 4, 3
    q = _rand((1, T, H, kd), rng)
    K = _rand((1, T, H, kd), rng)
    V = _rand((1, T, H, vd), rng)
    idx = np.tile(np.arange(T, dtype=np.int32), (1, T, 1))
    q_pos = np.arange(T)[None]
    out, _ = oracle.sparse_attend(q, K, V, idx, 0.5, kv_heads=H, q_pos=q_pos, pad=[2])
    for t in range(T):
        sel = np.array([[[j for j in range(2, t + 1)] or [INV]]], np.int32)
        o, _ = oracle.sparse_attend(q[:, t:t + 1], K, V, sel, 0.5, kv_heads=H)
        assert np.array_equal(out[t], o[0])


def test_shared_kv_head_equals_replicated_heads_and_absorbed_alias():
    rng = np.random.default_rng(25)
    Tk, H, kd, vd = 11, 4, 9, 6
    q = _rand((1, 2, H, kd), rng)
    lat = _rand((1, Tk, kd), rng)                     # one latent row per key
    idx = np.array([[[1, 4, 9, 2], [0, 10, 3, INV]]], np.int32)
    # absorbed: K = latent row, V = its first vd columns, one kv head
    o_abs, l_abs = oracle.sparse_attend(q, lat, None, idx, 0.3, kv_heads=1,
                                        k_row_stride=kd, vd=vd)
    # the same with explicit, replicated per-head K and V
    Kr = np.repeat(lat[:, :, None, :], H, axis=2)
    Vr = np.repeat(lat[:, :, None, :vd], H, axis=2)
    o_rep, l_rep = oracle.sparse_attend(q, Kr, Vr, idx, 0.3, kv_heads=H)
    np.testing.assert_allclose(o_abs, o_rep, rtol=1e-15)
    np.testing.assert_allclose(l_abs, l_rep, rtol=1e-15)


def test_batch_invariance():
    rng = np.random.default_rng(26)
    B, T, H, kd, vd = 3, 8, 2, 4, 3
    q = _rand((B, T, H, kd), rng)
    K = _rand((B, T, 1, kd), rng)
    V = _rand((B, T, 1, vd), rng)
    idx = rng.integers(0, T, (B, T, 5)).astype(np.int32)
    out, _ = oracle.sparse_attend(q, K, V, idx, 0.5, kv_heads=1)
    for b in range(B):
        ob, _ = oracle.sparse_attend(q[b:b + 1], K[b:b + 1], V[b:b + 1], idx[b:b + 1], 0.5,
                                     kv_heads=1)
        assert np.array_equal(out[b * T:(b + 1) * T], ob)


def test_topk_to_mask_rules():
    m = oracle.topk_to_mask([3, 3, INV, 9, -4, 12, 0], 10)
    assert np.flatnonzero(m).tolist() == [0, 3, 9]
    m = oracle.topk_to_mask([3, 3, INV, 9, -4, 12, 0], 10, pad=1, qpos=8)
    assert np.flatnonzero(m).tolist() == [3]
