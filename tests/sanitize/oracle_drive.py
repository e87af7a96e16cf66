"""Every oracle entry point on small seeded inputs and on its edge cases
(empty selections, ragged and fully padded rows, duplicates and INVALID
entries, k larger than the row, a trailing partial pool, an all-zero
cache row, rows written outside the cache).

Run by tests/test_sanitizers.py in a child process whose oracle library is
built with AddressSanitizer and UndefinedBehaviorSanitizer (DSA_ORACLE_LIB);
any out-of-bounds access or undefined operation in dsa_oracle.c aborts the
child.  torch is kept out of the process (the sanitizer runtime is
preloaded, and the oracle only needs numpy here)."""
import os
import sys

sys.modules["torch"] = None  # the oracle's optional torch paths fall back to numpy
ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402


def bf16_bits(x):
    """float32 -> bf16 bits, round to nearest even (finite inputs)."""
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def main():
    rng = np.random.default_rng(11)
    for c in range(256):
        oracle.e4m3_value(c)
    for b in (0, 0x3F80, 0x7F7F, 0x8001, 0xFFFF):
        oracle.bf16_value(b)

    # index scores: bf16, f32 and fp8 keys, pooled visibility, row subsets
    B, Tq, Tk, H, d = 3, 5, 37, 4, 32
    q = rng.standard_normal((B, Tq, H, d)).astype(np.float32)
    k = rng.standard_normal((B, Tk, d)).astype(np.float32)
    w = rng.uniform(size=(B, Tq, H)).astype(np.float32)
    pad = np.array([0, 3, Tk], np.int32)                    # the last row fully padded
    q_pos = np.tile(np.array([0, 2, 9, 30, Tk - 1], np.int32), (B, 1))
    S, A = oracle.index_scores(q, k, w, 0.17, q_pos, pad, want_mag=True)
    oracle.index_scores(bf16_bits(q), bf16_bits(k), w, 0.17, q_pos, pad, rows=[0, 7, 14])
    codes, sc = oracle.quantize_e4m3_rows(k / 4)
    oracle.index_scores(bf16_bits(q), codes, w, 0.17, q_pos, pad, k_scale=sc)
    oracle.index_scores(q, k[:, :9], w, 0.17, q_pos, pad, kpool=4)

    # top-k: k above the row length, ties, padded rows, pooled visibility
    rows_qpos = q_pos.reshape(-1)
    rows_pad = np.repeat(pad, Tq)
    oracle.topk(S, rows_qpos, rows_pad, 8)
    oracle.topk(S, rows_qpos, rows_pad, 64)
    oracle.topk(np.zeros_like(S), rows_qpos, rows_pad, 5)
    oracle.topk(S[:, :9], rows_qpos, rows_pad, 3, kpool=4)

    # pool keys (a trailing partial pool; a fully padded sequence) and select
    L, kp = 23, 4
    kk = rng.standard_normal((B, L, d)).astype(np.float32)
    gate = rng.standard_normal((B, L, d)).astype(np.float32)
    ppad = np.array([0, 2, L], np.int32)
    pk, npools, mag = oracle.pool_keys(kk, gate, ppad, kp, want_mag=True)
    oracle.pool_keys(bf16_bits(kk), bf16_bits(gate), ppad, kp)
    qp = np.tile(np.arange(L, dtype=np.int32), (B, 1))
    PS = rng.standard_normal((B * L, L // kp)).astype(np.float32)
    oracle.pool_select(PS, qp.reshape(-1), np.repeat(ppad, L), kp, 2, 2 * kp + kp - 1,
                       want_pools=True)
    oracle.pool_select(PS, qp.reshape(-1), np.repeat(ppad, L), kp, 8, 8 * kp + kp - 1)
    try:
        oracle.pool_select(PS, qp.reshape(-1), np.repeat(ppad, L), kp, 2, 2 * kp)
        raise AssertionError("a too narrow out_width was accepted")
    except ValueError:
        pass

    # topk_to_mask and attention: duplicates, INVALID, out of range, empty rows
    idx = rng.integers(-1, Tk + 3, (B, Tq, 12)).astype(np.int32)
    idx[0, 0] = -1                                          # empty selection
    idx[1, 1, :4] = 5                                       # duplicates
    for row in idx.reshape(-1, 12)[:4]:
        oracle.topk_to_mask(row, Tk)
        oracle.topk_to_mask(row, Tk, pad=2, qpos=20)
    kd, vd, kvh = 24, 16, 2
    qa = rng.standard_normal((B, Tq, H, kd)).astype(np.float32)
    K = rng.standard_normal((B, Tk, kvh, kd)).astype(np.float32)
    V = rng.standard_normal((B, Tk, kvh, vd)).astype(np.float32)
    oracle.sparse_attend(qa, K, V, idx, 0.2, kvh, q_pos=q_pos, pad=pad)
    oracle.sparse_attend(qa, K, V, idx, 0.2, kvh, rows=[1, 2, 13])
    Kabs = rng.standard_normal((B, Tk, 1, kd)).astype(np.float32)
    oracle.sparse_attend(qa, Kabs, None, idx, 0.2, 1, vd=vd)       # V = K's first vd columns
    oracle.sparse_attend(bf16_bits(qa), bf16_bits(K), bf16_bits(V), idx, 0.2, kvh)
    try:
        oracle.sparse_attend(qa, K, V, idx, 0.2, 3)
        raise AssertionError("kv_heads that does not divide the heads was accepted")
    except ValueError:
        pass

    # the cache write: rotation, e4m3, per-row quantisation, rows outside
    for dd in (2, 32, 64, 128, 256):
        oracle.hadamard_rows(rng.standard_normal((3, dd)).astype(np.float32), want_f64=True)
    oracle.hadamard_rows(bf16_bits(rng.standard_normal((2, 64))))
    try:
        oracle.hadamard_rows(np.ones((1, 48), np.float32))
        raise AssertionError("a width that is not a power of two was accepted")
    except ValueError:
        pass
    oracle.e4m3_encode(np.array([0.0, -0.0, 1e-9, 448.0, 449.0, 3e38, -3e38], np.float32))
    y = rng.standard_normal((4, 64)).astype(np.float32)
    y[2] = 0.0
    oracle.quantize_e4m3_rows(y)
    cache = rng.integers(0, 256, (3, 9, 64)).astype(np.uint8)
    scales = rng.uniform(size=(3, 9)).astype(np.float32)
    oracle.index_cache_write(rng.standard_normal((3, 2, 64)).astype(np.float32),
                             np.array([0, 8, -1], np.int32), cache, scales)
    print("oracle drive: done", flush=True)


if __name__ == "__main__":
    main()
