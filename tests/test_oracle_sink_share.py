"""Pins of the oracle's selection rules around top-k ("Another DSA attempt"):

- attention-sink force-inclusion: the decode indexer-K cache commit boosts
  the first key(s) by 1e20 so the sink survives top-k; the per-sequence sink
  commit adds the boost only for the query's own sequence; the
  serving-correctness commit anchors it on the sequence's first present
  position (a fresh sequence from position 0 is unchanged);
- IndexShare: the commit message and review comments -- 21 "full" layers
  (0, 1, 2, then every 4th up to 74) of GLM-5.2's 78 compute their own
  top-k, the other 57 reuse the most recent full layer's; full iff
  il <= 1 or il % 4 == 2.

Each pin checks the oracle against something other than itself: the pages'
enumeration and counts, and a brute-force sorted() selection."""
import numpy as np
import pytest

import oracle


def _brute(row, cols, k, sinks):
    """Sinks first in column order, then the other visible columns by
    (higher score, smaller column), INVALID-padded: the selection the 1e20
    boost produces whenever every score is far below 1e20."""
    rest = sorted((c for c in cols if c not in sinks), key=lambda c: (-float(row[c]), c))
    sel = list(sinks) + rest
    return (sel + [-1] * k)[:k]


@pytest.mark.parametrize("n_sink", [1, 2, 4])
def test_sink_survives_topk_per_sequence(n_sink):
    rng = np.random.default_rng(n_sink)
    Tk, k = 300, 16
    pads = np.array([0, 5, 37, 120], np.int32)
    rows_pad, rows_q, S = [], [], []
    for p in pads:
        for qp in (p, p + 1, p + 3, p + 50, Tk - 1):
            row = rng.standard_normal(Tk).astype(np.float32) * 10
            row[p:p + n_sink] = -1e6       # the sinks' own scores are the row's lowest
            S.append(row)
            rows_pad.append(p)
            rows_q.append(qp)
    S = np.stack(S)
    got = oracle.topk(S, rows_q, rows_pad, k, n_sink=n_sink)
    for r in range(len(S)):
        p, qp = rows_pad[r], rows_q[r]
        cols = list(range(p, qp + 1))
        sinks = [c for c in range(p, p + n_sink) if c <= qp]   # causal mask still applies
        assert list(got[r]) == _brute(S[r], cols, k, sinks), (r, p, qp)
        # anchored on the row's own first present position, not column 0
        assert got[r][0] == p


def test_fresh_sequence_sink_is_leading_cells():
    """pad 0: the sink cells are 0 .. n_sink - 1, the pre-fix behaviour."""
    rng = np.random.default_rng(3)
    S = rng.standard_normal((6, 64)).astype(np.float32)
    got = oracle.topk(S, np.full(6, 63, np.int32), np.zeros(6, np.int32), 8, n_sink=3)
    assert np.all(got[:, :3] == np.array([0, 1, 2]))
    plain = oracle.topk(S, np.full(6, 63, np.int32), np.zeros(6, np.int32), 8)
    for r in range(6):
        rest = [c for c in plain[r] if c not in (0, 1, 2)]
        assert list(got[r, 3:]) == rest[:5]


def test_sink_is_an_f32_boost_of_1e20():
    """The boost is added to the f32 score: a key scoring above 1e20 still
    outranks the sink, and sinks with scores large enough to survive the
    f32 addition are ordered by their boosted values."""
    S = np.zeros((2, 10), np.float32)
    S[0, 6] = 3e20                     # above the boosted sink
    S[1, 0] = -1e13                    # two sinks whose boosted values differ
    S[1, 1] = 1e13
    got = oracle.topk(S, [9, 9], [0, 0], 3, n_sink=2)
    assert list(got[0]) == [6, 0, 1]
    b0 = np.float32(np.float32(-1e13) + np.float32(1e20))
    b1 = np.float32(np.float32(1e13) + np.float32(1e20))
    assert b1 > b0                     # the premise: the f32 sums differ
    assert list(got[1]) == [1, 0, 2]


def test_sink_with_few_visible_keys_and_pools():
    S = np.arange(40, dtype=np.float32).reshape(2, 20)
    # query at its sequence's first present position: one visible key, the sink
    got = oracle.topk(S, [4, 4], [4, 4], 5, n_sink=3)
    assert list(got[0]) == [4, -1, -1, -1, -1]
    # pooled keys (kpool 4): the sinks are the first visible pools
    got = oracle.topk(S[:, :5], [19, 19], [0, 0], 3, kpool=4, n_sink=1)
    assert list(got[0]) == [0, 4, 3]


def test_index_share_matches_the_pages_enumeration():
    full = [il for il in range(78) if oracle.index_share_source(il) == il]
    assert full == [0, 1, 2] + list(range(6, 75, 4))
    assert len(full) == 21 and 78 - len(full) == 57
    for il in range(78):
        src = oracle.index_share_source(il)
        assert src in full and src <= il
        # the most recent full layer: none between it and il
        assert not any(src < f <= il for f in full)
    assert oracle.index_share_source(-1) == -1
