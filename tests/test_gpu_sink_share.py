"""GPU parity of the selection rules around top-k ("Another DSA attempt"):
attention-sink force-inclusion (the decode indexer-K cache commit, the
per-sequence sink commit, the serving-correctness commit's first-present
anchor) through every top-k kernel path, and IndexShare (the IndexShare
commit: shared layers reuse the most recent full layer's selection) in a
small layer loop.  Selections are compared bit for bit with the oracle,
which adds the pages' f32 boost of 1e20 to the sink scores; every score
here is far below 2^42 in magnitude, where that boost and the path's
sinks-first order agree."""
import numpy as np
import pytest
import torch

import oracle
from sparse_attention_scores_amd import workloads as W
from tests.parity import check_attend, cpu, note

pytestmark = pytest.mark.gpu

POISON_I32 = 0x7EADBEEF


@pytest.fixture(scope="module")
def dsa():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    from sparse_attention_scores_amd import binding
    binding.load()
    return binding


def _rows(rows, n, seed):
    """Scores with the sinks' own values at the bottom of the row, quantised
    ties on every third row, left pads (first present positions) from 0 to
    300, and query positions at, just after and far from the first present
    position."""
    gen = torch.Generator(device="cuda").manual_seed(seed)
    S = torch.randn(rows, n, generator=gen, device="cuda") * 5
    S[::3] = torch.round(S[::3] * 4.0) / 4.0
    pad = torch.tensor([(r * 37) % 301 for r in range(rows)], dtype=torch.int32, device="cuda")
    qpos = torch.full((rows,), n - 1, dtype=torch.int32, device="cuda")
    qpos[1::5] = pad[1::5]                  # only the sink visible
    qpos[2::5] = pad[2::5] + 2
    qpos[3::5] = torch.clamp(pad[3::5] + 5000, max=n - 1)
    ar = torch.arange(n, device="cuda")
    S[(ar[None, :] >= pad[:, None]) & (ar[None, :] < pad[:, None] + 4)] = -1e4
    return S, pad, qpos


@pytest.mark.parametrize("rows,n,k,n_sink", [
    (32, 8192, 2048, 1),      # decode shape: segmented kernel, 8 blocks per row
    (512, 4096, 2048, 2),     # prefill shape: 512-thread segmented kernel
    (8, 131072, 2048, 1),     # long decode: chunks + segmented merge
    (256, 20000, 2048, 4),    # chunks + one-block merge
    (16, 3000, 100, 3),
    (4, 1000, 5, 8),          # more sinks than top_k: the first k visible keys
])
def test_topk_sinks_every_path(dsa, rows, n, k, n_sink):
    note(f"topk sinks rows={rows} n={n} k={k} n_sink={n_sink}")
    S, pad, qpos = _rows(rows, n, rows + n + k)
    lo, hi = pad, qpos + 1
    idx = torch.full((rows, k), POISON_I32, dtype=torch.int32, device="cuda")
    dsa.topk(S, lo, hi, k, out=idx, n_sink=n_sink)
    torch.cuda.synchronize()
    ref = oracle.topk(cpu(S).numpy(), cpu(qpos).numpy(), cpu(pad).numpy(), k, n_sink=n_sink)
    got = cpu(idx).numpy()
    bad = np.nonzero((got != ref).any(1))[0]
    assert bad.size == 0, f"rows differ: {bad[:10]}; first {got[bad[0], :8]} vs {ref[bad[0], :8]}"
    # the sinks lead each row at its own first present position
    p = cpu(pad).numpy()
    vis = cpu(qpos).numpy() - p + 1
    for r in range(rows):
        m = min(n_sink, k, vis[r])
        assert np.array_equal(got[r, :m], p[r] + np.arange(m))
    # the allocation-free entry point agrees
    if dsa.topk_workspace_size(rows, n, k) <= (16 << 20):
        idx2 = torch.full_like(idx, POISON_I32)
        dsa.topk_noalloc(S, lo, hi, k, idx2, n_sink=n_sink)
        torch.cuda.synchronize()
        assert torch.equal(idx2, idx)


def test_decode_step_with_sink(dsa):
    """The decode workload's scores (index_scores on its own inputs) with one
    sink per sequence; left pads give each sequence a different anchor."""
    note("decode step with a sink")
    inp = W.make(2, device="cuda", B=6, Tk=9000)
    pad = torch.tensor([0, 1, 17, 300, 2048, 5000], dtype=torch.int32, device="cuda")
    lo, hi = dsa.visibility_ranges(pad, inp["q_pos"])
    S = dsa.index_scores(inp["q_idx"], inp["k_idx"], inp["w"], lo, hi, inp["scale_idx"])
    idx = dsa.topk(S.view(6, -1), lo, hi, 2048, n_sink=1)
    torch.cuda.synchronize()
    ref = oracle.topk(cpu(S).numpy().reshape(6, -1), cpu(inp["q_pos"]).numpy().reshape(-1),
                      cpu(pad).numpy(), 2048, n_sink=1)
    assert np.array_equal(cpu(idx).numpy(), ref)
    assert np.array_equal(cpu(idx).numpy()[:, 0], cpu(pad).numpy())


def test_index_share_layer_loop(dsa):
    """Six layers of decode over per-layer inputs: full layers (0, 1, 2)
    score and select, shared layers (3, 4, 5) attend with layer 2's rows.
    Each layer's output matches the oracle's attention over the selection
    the oracle computes for that layer's source."""
    note("IndexShare layer loop")
    B, Tk, k = 2, 3000, 512
    full_rows = {}
    outs = []
    layers = list(range(6))
    assert [dsa.index_share_source(il) for il in layers] == [0, 1, 2, 2, 2, 2]
    per_layer = [W.make(2, device="cuda", B=B, Tk=Tk, seed=500 + il) for il in layers]
    lo, hi = dsa.visibility_ranges(per_layer[0]["pad"], per_layer[0]["q_pos"])
    for il in layers:
        inp = per_layer[il]
        src = dsa.index_share_source(il)
        if src == il:
            S = dsa.index_scores(inp["q_idx"], inp["k_idx"], inp["w"], lo, hi, inp["scale_idx"])
            full_rows[il] = (S, dsa.topk(S.view(B, -1), lo, hi, k, n_sink=1).view(B, 1, k))
        idx = full_rows[src][1]
        out, lse = dsa.sparse_attend(inp["q"], inp["KV"], None, idx, inp["scale_attn"], 1,
                                     vd=inp["vd"], vis_lo=lo, vis_hi=hi)
        outs.append((out, lse))
    torch.cuda.synchronize()
    for il in layers:
        inp = per_layer[il]
        src = oracle.index_share_source(il)
        S_src = cpu(full_rows[src][0]).numpy().reshape(B, -1)
        sel = oracle.topk(S_src, cpu(inp["q_pos"]).numpy().reshape(-1),
                          cpu(inp["pad"]).numpy(), k, n_sink=1)
        assert np.array_equal(cpu(full_rows[src][1]).numpy().reshape(B, -1), sel)
        ref, lref = oracle.sparse_attend(cpu(inp["q"]), cpu(inp["KV"]), None,
                                         sel.reshape(B, 1, k), inp["scale_attn"], 1,
                                         q_pos=cpu(inp["q_pos"]), pad=cpu(inp["pad"]),
                                         k_row_stride=inp["KV"].shape[-1], vd=inp["vd"])
        out, lse = outs[il]
        check_attend(cpu(out).numpy().reshape(ref.shape), ref,
                     cpu(lse).numpy().reshape(lref.shape), lref, bf16=True,
                     what=f"layer {il} (selection of layer {src})")
