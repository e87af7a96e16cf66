"""GPU parity at the full sizes of each configuration, in the launch
configuration bench.py times (the tests drive bench.py's own step objects).

The oracle recomputes a seeded sample of rows one by one: scores on sampled
query rows, top-k / pool select on every row (cheap), attention on sampled
rows fed the selection the GPU produced -- which equals the oracle's own
top-k of the GPU scores, checked bit for bit first.  Sample sizes: every
row of the decode configurations; 512 score rows and 256 attention rows
per sequence for the prefill and pooled ones, always with the first valid
row, the last, and the rows around where the selection starts to bite."""
import numpy as np
import pytest
import torch

import bench
import oracle
from sparse_attention_scores_amd import workloads as W
from tests.parity import check_attend, check_scores, cpu, note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    from sparse_attention_scores_amd import binding
    binding.load()
    return binding


def _sample(n_rows, n, seed, must=()):
    rng = np.random.default_rng(seed)
    pick = set(int(x) for x in must if 0 <= x < n_rows)
    pick |= set(int(x) for x in rng.choice(n_rows, size=min(n, n_rows), replace=False))
    return np.array(sorted(pick), np.int64)


@pytest.mark.parametrize("cfg,score_rows,attend_rows", [(2, 32, 32), (3, 512, 256), (4, 8, 8)])
def test_fullsize_absorbed_step(dsa, cfg, score_rows, attend_rows):
    note(f"full-size step, config {cfg}")
    inp = W.make(cfg, device="cuda")
    step = bench.Step(dsa, inp)
    if step.cached:
        k_before = cpu(inp["k_idx"]).view(torch.uint8).numpy().copy()
        s_before = cpu(inp["k_scale"]).numpy().copy()
    for name in step.stages:
        getattr(step, name)()
    torch.cuda.synchronize()
    if step.cached:
        # write-then-score: the cache holds the new token's rotated fp8 row,
        # every other row is untouched, and the queries were rotated
        B, Tk = inp["B"], inp["Tk"]
        rc, rs = oracle.index_cache_write(cpu(inp["k_new"]), np.full(B, Tk - 1, np.int32),
                                          k_before, s_before)
        assert np.array_equal(cpu(inp["k_idx"]).view(torch.uint8).numpy(), rc)
        assert np.array_equal(cpu(inp["k_scale"]).numpy(), rs)
        qr = oracle.hadamard_rows(cpu(inp["q_idx"]))
        assert torch.equal(cpu(step.q_used), torch.from_numpy(qr).bfloat16())
    B, Tq, Tk, k = inp["B"], inp["Tq"], inp["Tk"], inp["top_k"]
    n_rows = B * Tq
    qp = cpu(inp["q_pos"]).numpy().reshape(-1)
    pd = np.repeat(cpu(inp["pad"]).numpy(), Tq)
    # -- scores on sampled rows (first row, last row, where selection starts to bite)
    must = [0, n_rows - 1, min(k, n_rows - 1), min(k + 1, n_rows - 1)]
    rows = _sample(n_rows, score_rows, 100 + cfg, must)
    note(f"  oracle scores on {len(rows)} rows")
    kq = cpu(inp["k_idx"])
    ks = None if inp["k_scale"] is None else cpu(inp["k_scale"])
    ref, A = oracle.index_scores(cpu(step.q_used), kq, cpu(inp["w"]), inp["scale_idx"],
                                 cpu(inp["q_pos"]), cpu(inp["pad"]), k_scale=ks, rows=rows,
                                 want_mag=True)
    S_rows = cpu(step.S.reshape(n_rows, Tk)[torch.tensor(rows, device="cuda")]).numpy()
    check_scores(S_rows, ref, A, 1e-3, f"config {cfg} scores")
    # -- top-k: every row, bit-exact on the GPU's scores
    note("  oracle top-k on every row")
    S_all = cpu(step.S).numpy().reshape(n_rows, Tk)
    ref_idx = oracle.topk(S_all, qp, pd, k)
    got_idx = cpu(step.idx).numpy().reshape(n_rows, k)
    bad = np.nonzero((got_idx != ref_idx).any(1))[0]
    assert bad.size == 0, f"config {cfg}: top-k rows differ: {bad[:8]}"
    del S_all
    # -- attention on sampled rows with that selection
    rows = _sample(n_rows, attend_rows, 200 + cfg, must)
    note(f"  oracle attention on {len(rows)} rows")
    out_ref, lse_ref = oracle.sparse_attend(cpu(inp["q"]), cpu(inp["KV"]), None,
                                            ref_idx.reshape(B, Tq, k), inp["scale_attn"], 1,
                                            q_pos=cpu(inp["q_pos"]), pad=cpu(inp["pad"]),
                                            rows=rows, k_row_stride=inp["kd"], vd=inp["vd"])
    r_t = torch.tensor(rows, device="cuda")
    out_g = cpu(step.out.reshape(n_rows, inp["H"], inp["vd"])[r_t]).numpy()
    lse_g = cpu(step.lse.reshape(n_rows, inp["H"])[r_t]).numpy()
    check_attend(out_g, out_ref, lse_g, lse_ref, bf16=True, what=f"config {cfg} attend")


def test_fullsize_pooled_step(dsa):
    note("full-size pooled step, config 5")
    inp = W.make(5, device="cuda")
    step = bench.PooledStep(dsa, inp)
    for f in (step.pool_keys, step.index, step.pool_select, step.attend):
        f()
    torch.cuda.synchronize()
    B, L, kp, d = inp["B"], inp["L"], inp["kpool"], inp["d"]
    NP = L // kp
    n_rows = B * L
    pads = cpu(inp["pad"]).numpy()
    # -- pool keys: every pool, within one bf16 ulp of the f64 value
    note("  oracle pool keys")
    pk_ref, np_ref, mag = oracle.pool_keys(cpu(inp["k_idx"]), cpu(inp["gate"]), pads, kp,
                                           want_mag=True)
    assert cpu(step.npools).tolist() == np_ref.tolist()
    from tests.parity import bf16_ulp_ok
    bf16_ulp_ok(cpu(step.pk), pk_ref, mag, "config 5 pool keys")
    # -- pooled scores on sampled rows (the GPU's pooled keys as the input)
    must = [0, L - 1, 2 * L + 36, 2 * L + 37, 3 * L + 63, 3 * L + 64, 4 * L - 1]
    rows = _sample(n_rows, 512 * B, 105, must)
    note(f"  oracle pooled scores on {len(rows)} rows")
    ref, A = oracle.index_scores(cpu(inp["q_idx"]), cpu(step.pk), cpu(inp["w"]),
                                 inp["scale_idx"], cpu(inp["q_pos"]), pads, kpool=kp, rows=rows,
                                 want_mag=True)
    S_rows = cpu(step.S.reshape(n_rows, NP)[torch.tensor(rows, device="cuda")]).numpy()
    check_scores(S_rows, ref, A, 1e-3, "config 5 pooled scores")
    # -- pool select: every row, bit-exact on the GPU's scores
    note("  oracle pool select on every row")
    qp = cpu(inp["q_pos"]).numpy().reshape(-1)
    pd = np.repeat(pads, L)
    S_all = cpu(step.S).numpy().reshape(n_rows, NP)
    tok_ref = oracle.pool_select(S_all, qp, pd, kp, inp["select_k"], inp["out_width"])
    del S_all
    tok = cpu(step.tok).numpy().reshape(n_rows, -1)
    bad = np.nonzero((tok != tok_ref).any(1))[0]
    assert bad.size == 0, f"pool select rows differ: {bad[:8]}"
    # -- per-head attention on sampled rows of every sequence: the first
    # rows, the first valid one, both sides of a 256-query block boundary,
    # where the selection starts to bite, and the last row
    for b in range(B):
        p = int(pads[b])
        bite = p + kp * inp["select_k"]  # the first position with more pools than select_k
        must_b = [0, p, p + 1, 255, 256, bite - 1, bite + kp - 1, L - 1]
        rows_b = _sample(L, 256, 300 + b, must_b)
        note(f"  oracle attention, sequence {b}, {len(rows_b)} rows")
        sl = slice(b, b + 1)
        out_ref, lse_ref = oracle.sparse_attend(
            cpu(inp["q"][sl]), cpu(inp["K"][sl]), cpu(inp["V"][sl]),
            tok_ref.reshape(B, L, -1)[sl], inp["scale_attn"], inp["H"],
            q_pos=cpu(inp["q_pos"][sl]), pad=pads[sl], rows=rows_b)
        r_t = torch.tensor(rows_b, device="cuda")
        out_g = cpu(step.out[b][r_t]).numpy()
        lse_g = cpu(step.lse[b][r_t]).numpy()
        check_attend(out_g, out_ref, lse_g, lse_ref, bf16=True, what=f"config 5 attend seq {b}")
