"""Pins of the oracle's top-k, pool keys and pool select (CPU only).

Rules (page "Module glm5next_dsa_ref"): topk_pools orders by higher score then
smaller index; pool_states pools from the first valid token with a per-channel
softmax over the slot axis, and a trailing partial pool is not a pool;
expand_selection writes every row for its full out_width with INVALID padding,
appends the visible tail, and leaves a padded query row all INVALID.  The
ik_llama.cpp batch-local indexer commit (PR #2063 thread) takes
top_k(min(top_k, n_tokens)) of the visible keys."""
import json
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")
INV = oracle.INVALID


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _brute_topk(row, lo, hi, k):
    cand = sorted(range(lo, hi), key=lambda s: (-float(row[s]), s))
    out = cand[:k]
    return out + [INV] * (k - len(out))


# ---------------------------------------------------------------- top-k

def test_topk_golden_tie_order():
    g = _gold("topk_tie_order.json")
    S = np.array([g["scores"]], np.float32)
    n = S.shape[1]
    got = oracle.topk(S, [n - 1], [0], g["k"])
    assert got[0].tolist() == g["expected"]
    got = oracle.topk(S, [n - 1], [0], g["k_all"])
    assert got[0].tolist() == g["expected_all"]


def test_topk_brute_force_random_rows_with_ties():
    rng = np.random.default_rng(11)
    for trial in range(40):
        n = int(rng.integers(1, 40))
        S = rng.integers(-3, 4, (6, n)).astype(np.float32) * 0.5
        qpos = rng.integers(0, n, 6)
        pad = rng.integers(0, 3, 6)
        k = int(rng.integers(1, 12))
        got = oracle.topk(S, qpos, pad, k)
        for r in range(6):
            assert got[r].tolist() == _brute_topk(S[r], pad[r], qpos[r] + 1, k)


def test_topk_all_equal_scores_give_ascending_indices():
    S = np.full((1, 20), 0.25, np.float32)
    assert oracle.topk(S, [19], [4], 5)[0].tolist() == [4, 5, 6, 7, 8]


def test_topk_k_at_least_visible_returns_all_visible_ranked():
    S = np.array([[3.0, 1.0, 2.0, 9.0, 9.0]], np.float32)
    got = oracle.topk(S, [3], [1], 6)[0].tolist()
    assert got == [3, 2, 1, INV, INV, INV]  # key 4 is in the future


def test_topk_signed_zero_ties_go_to_smaller_index():
    S = np.array([[-0.0, 0.0, -0.0, 0.0]], np.float32)
    assert oracle.topk(S, [3], [0], 4)[0].tolist() == [0, 1, 2, 3]


def test_topk_nan_is_rejected():
    S = np.array([[1.0, np.nan]], np.float32)
    with pytest.raises(ValueError):
        oracle.topk(S, [1], [0], 1)


def test_topk_pool_mode_candidates():
    # pooled visibility: pad 1, kpool 2 -> query 4 sees pools 0 (1,2) and 1 (3,4)
    S = np.array([[0.1, 0.9, 5.0, 0.2]], np.float32)
    assert oracle.topk(S, [4], [1], 3, kpool=2)[0].tolist() == [1, 0, INV]


# ---------------------------------------------------------------- pool keys

def test_pool_keys_golden_first_valid_token():
    g = _gold("pool_first_valid_token.json")
    L, d, kp = len(g["tokens"]), 3, g["kpool"]
    k = np.arange(L * d, dtype=np.float64).reshape(1, L, d)
    gate = np.zeros((1, L, d))
    pk, npools = oracle.pool_keys(k, gate, [g["pad"]], kp)
    assert npools[0] == g["expected_n_pools"]
    toks = g["expected_pool_tokens"][0]
    np.testing.assert_allclose(pk[0, 0], k[0, toks].mean(0), rtol=1e-15)


def test_pool_keys_golden_trailing_partial_pool():
    g = _gold("pool_trailing_partial.json")
    L, d, kp = g["seq"], 2, g["kpool"]
    k = np.arange(L * d, dtype=np.float64).reshape(1, L, d)
    pk, npools = oracle.pool_keys(k, np.zeros((1, L, d)), [g["pad"]], kp)
    assert npools[0] == g["expected_n_pools"]
    np.testing.assert_allclose(pk[0, 0], k[0, g["expected_pool_tokens"][0]].mean(0))


def test_pool_keys_dominant_slot_and_unused_rows_zero():
    rng = np.random.default_rng(12)
    B, L, d, kp = 1, 13, 4, 4      # pad 2: 11 valid tokens -> 2 pools of 3 rows
    k = rng.standard_normal((B, L, d))
    gate = np.zeros((B, L, d))
    gate[0, 3, :] = 60.0     # slot 1 of pool 0 (pad 2: pool 0 = tokens 2..5)
    pk, npools = oracle.pool_keys(k, gate, [2], kp)
    assert npools[0] == 2
    np.testing.assert_allclose(pk[0, 0], k[0, 3], rtol=1e-20, atol=1e-24)
    assert np.all(pk[0, 2] == 0.0)


def test_pool_keys_softmax_runs_per_channel_over_slots():
    rng = np.random.default_rng(13)
    B, L, d, kp = 2, 13, 5, 4
    k = rng.standard_normal((B, L, d))
    gate = rng.standard_normal((B, L, d)) * 3
    pads = np.array([0, 3])
    pk, npools = oracle.pool_keys(k, gate, pads, kp)
    for b in range(B):
        n = (L - pads[b]) // kp
        assert npools[b] == n
        for i in range(n):
            t = pads[b] + i * kp + np.arange(kp)
            g = gate[b, t, :]                       # [slot, channel]
            p = np.exp(g - g.max(0)) / np.exp(g - g.max(0)).sum(0)
            np.testing.assert_allclose(pk[b, i], (p * k[b, t, :]).sum(0), rtol=1e-12)
    # a gate that differs only across channels (same for every slot) gives the mean
    gate2 = np.tile(rng.standard_normal((1, 1, d)), (B, L, 1))
    pk2, _ = oracle.pool_keys(k, gate2, pads, kp)
    np.testing.assert_allclose(pk2[0, 0], k[0, 0:4].mean(0), rtol=1e-12)


# ---------------------------------------------------------------- pool select

def _brute_pool_select(row, pad, qpos, kp, select_k, width):
    tok = [INV] * width
    if qpos < pad:
        return tok
    n_full = (qpos - pad + 1) // kp
    order = sorted(range(n_full), key=lambda i: (-float(row[i]), i))[:select_k]
    out = []
    for i in order:
        out += [pad + i * kp + j for j in range(kp)]
    out += list(range(pad + n_full * kp, qpos + 1))
    return out + [INV] * (width - len(out))


def test_pool_select_brute_force_and_invariants():
    rng = np.random.default_rng(14)
    L, kp, sk = 23, 4, 3
    width = sk * kp + kp - 1
    NP = L // kp
    for pad in (0, 2, 5):
        S = rng.integers(-2, 3, (L, NP)).astype(np.float32)
        qpos = np.arange(L)
        tok, pools = oracle.pool_select(S, qpos, np.full(L, pad), kp, sk, width,
                                        want_pools=True)
        for t in range(L):
            row = tok[t].tolist()
            assert row == _brute_pool_select(S[t], pad, t, kp, sk, width), (pad, t)
            assert len(row) == width
            valid = [x for x in row if x != INV]
            assert all(pad <= x <= t for x in valid)        # no pad, no future token
            assert row[len(valid):] == [INV] * (width - len(valid))
            if t < pad:
                assert valid == []
            n_full = (t - pad + 1) // kp if t >= pad else 0
            if sk >= n_full and t >= pad:
                assert sorted(valid) == list(range(pad, t + 1))
            np_taken = sum(1 for x in pools[t] if x != INV)
            assert np_taken == min(sk, n_full)


def test_pool_select_golden_tail():
    g = _gold("pool_trailing_partial.json")
    L, kp = g["seq"], g["kpool"]
    S = np.zeros((L, L // kp), np.float32)
    tok = oracle.pool_select(S, np.arange(L), np.zeros(L), kp, 1, 8)
    assert tok[L - 1].tolist()[:7] == g["expected_pool_tokens"][0] + g["expected_tail_at_last_position"]


def test_pool_select_out_width_too_small_is_an_error():
    S = np.zeros((8, 2), np.float32)
    with pytest.raises(ValueError):
        oracle.pool_select(S, np.arange(8), np.zeros(8), 4, 2, 5)
