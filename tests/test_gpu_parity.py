"""GPU parity: every stage of the libdsa path against the CPU oracle.

Stage-wise, as the correctness criteria are stated: scores on identical
inputs; top-k as the oracle's top-k applied to the GPU's own scores
(bit-exact); attention fed the oracle's selection.  Sizes span several tiles
and a ragged tail.  All calls go through the C ABI (binding -> libdsa.so)."""
import numpy as np
import pytest
import torch

import oracle
from sparse_attention_scores_amd import workloads as W
from tests.parity import FLT_MAX, bf16_ulp_ok, check_attend, check_scores, cpu, note

pytestmark = pytest.mark.gpu

INV = -1


@pytest.fixture(scope="module")
def dsa():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    from sparse_attention_scores_amd import binding
    binding.load()
    return binding


def _ranges(dsa, inp, kpool=0):
    return dsa.visibility_ranges(inp["pad"], inp["q_pos"], kpool)


def _rows_qpos_pad(inp):
    B, Tq = inp["q_pos"].shape
    qp = cpu(inp["q_pos"]).numpy().reshape(-1)
    pd = np.repeat(cpu(inp["pad"]).numpy(), Tq)
    return qp, pd


# ---------------------------------------------------------------- visibility

def test_visibility_ranges_match_definition(dsa):
    note("visibility ranges")
    pad = torch.tensor([0, 3, 7], dtype=torch.int32, device="cuda")
    q_pos = torch.arange(12, dtype=torch.int32, device="cuda").repeat(3, 1)
    lo, hi = dsa.visibility_ranges(pad, q_pos, 0)
    plo, phi = dsa.visibility_ranges(pad, q_pos, 4)
    torch.cuda.synchronize()
    lo, hi, plo, phi = (cpu(x).numpy() for x in (lo, hi, plo, phi))
    for b, p in enumerate([0, 3, 7]):
        for t in range(12):
            vis = [s for s in range(12) if oracle.token_visible(p, t, s)]
            got = list(range(lo[b, t], hi[b, t]))
            assert got == vis, (b, t)
            pools = [i for i in range(3) if oracle.pool_visible(p, 4, t, i)]
            assert list(range(plo[b, t], phi[b, t])) == pools, (b, t)


# ---------------------------------------------------------------- index scores

INDEX_CASES = [
    # (config, overrides, variant)
    (1, {}, None),
    (2, dict(B=2, Tk=1000), None),
    (2, dict(B=3, Tk=517), "tie"),
    (3, dict(Tq=300, Tk=300), None),
    # odd row length: score rows start off 16-byte boundaries, so the
    # vector fill of the masked keys needs its scalar head and tail
    (3, dict(Tq=211, Tk=211), None),
    (4, dict(B=2, Tk=4133), None),
]


def _index_case(dsa, cfg, over, variant, seed=None):
    inp = W.make(cfg, device="cuda", variant=variant, seed=seed, **over)
    lo, hi = _ranges(dsa, inp)
    S = dsa.index_scores(inp["q_idx"], inp["k_idx"], inp["w"], lo, hi, inp["scale_idx"],
                         k_scale=inp["k_scale"])
    torch.cuda.synchronize()
    return inp, lo, hi, S


@pytest.mark.parametrize("cfg,over,variant", INDEX_CASES)
def test_index_scores_parity(dsa, cfg, over, variant):
    note(f"index scores config {cfg} {over} {variant}")
    inp, lo, hi, S = _index_case(dsa, cfg, over, variant)
    ref, A = oracle.index_scores(cpu(inp["q_idx"]), cpu(inp["k_idx"]), cpu(inp["w"]),
                                 inp["scale_idx"], cpu(inp["q_pos"]), cpu(inp["pad"]),
                                 k_scale=None if inp["k_scale"] is None else cpu(inp["k_scale"]),
                                 want_mag=True)
    rtol = 1e-5 if inp["dtype"] == "f32" else 1e-3
    check_scores(cpu(S).numpy().reshape(ref.shape), ref, A, rtol, f"config {cfg}")


@pytest.mark.parametrize("cfg,over", [(3, dict(Tq=200, Tk=200)), (2, dict(B=2, Tk=1000)),
                                      (4, dict(B=1, Tk=2000))])
def test_index_scores_negative_scale_and_weights(dsa, cfg, over):
    """A negative scale and weights of both signs (prefill, decode, fp8 keys)."""
    note(f"index scores negative scale config {cfg} {over}")
    inp = W.make(cfg, device="cuda", **over)
    scale = -abs(inp["scale_idx"])
    w = inp["w"] - 0.5
    lo, hi = _ranges(dsa, inp)
    S = dsa.index_scores(inp["q_idx"], inp["k_idx"], w, lo, hi, scale, k_scale=inp["k_scale"])
    torch.cuda.synchronize()
    ref, A = oracle.index_scores(cpu(inp["q_idx"]), cpu(inp["k_idx"]), cpu(w), scale,
                                 cpu(inp["q_pos"]), cpu(inp["pad"]),
                                 k_scale=None if inp["k_scale"] is None else cpu(inp["k_scale"]),
                                 want_mag=True)
    check_scores(cpu(S).numpy().reshape(ref.shape), ref, A, 1e-3, f"config {cfg} negative scale")


def test_index_scores_padding_and_pooled_ranges(dsa):
    note("index scores: left padding + pooled visibility")
    B, L, H, d, kp = 3, 70, 32, 128, 4
    gen = torch.Generator(device="cuda").manual_seed(7)
    q = (torch.randn(B, L, H, d, generator=gen, device="cuda") / d ** 0.5).bfloat16()
    k = (torch.randn(B, L // kp, d, generator=gen, device="cuda") / d ** 0.5).bfloat16()
    w = torch.rand(B, L, H, generator=gen, device="cuda")
    pad = torch.tensor([0, 5, 66], dtype=torch.int32, device="cuda")
    q_pos = torch.arange(L, dtype=torch.int32, device="cuda").repeat(B, 1)
    lo, hi = dsa.visibility_ranges(pad, q_pos, kp)
    S = dsa.index_scores(q, k, w, lo, hi, 0.088)
    torch.cuda.synchronize()
    ref, A = oracle.index_scores(cpu(q), cpu(k), cpu(w), 0.088, cpu(q_pos), cpu(pad), kpool=kp,
                                 want_mag=True)
    check_scores(cpu(S).numpy().reshape(ref.shape), ref, A, 1e-3, "pooled ranges")


@pytest.mark.parametrize("fp8", [False, True])
def test_index_scores_decode_padding(dsa, fp8):
    """Decode rows (one and three queries per sequence) with left padding,
    one sequence wholly padded, and query positions short of the end: the
    decode kernel's visible tiles, its partial tiles and its -FLT_MAX rows."""
    note(f"index scores decode padding fp8={fp8}")
    B, H, d, Tk = 4, 32, 128, 1000
    gen = torch.Generator(device="cuda").manual_seed(11)
    for n_q in (1, 3):
        q = (torch.randn(B, n_q, H, d, generator=gen, device="cuda") / d ** 0.5).bfloat16()
        kf = torch.randn(B, Tk, d, generator=gen, device="cuda") / d ** 0.5
        k, k_scale = W.quantize_fp8_rows(kf) if fp8 else (kf.bfloat16(), None)
        w = torch.rand(B, n_q, H, generator=gen, device="cuda")
        pad = torch.tensor([0, 37, 999, 1000], dtype=torch.int32, device="cuda")
        last = torch.tensor([999, 999, 999, 700], dtype=torch.int32, device="cuda")
        q_pos = (last[:, None] - torch.arange(n_q - 1, -1, -1, dtype=torch.int32,
                                              device="cuda")[None, :] * 333).contiguous()
        lo, hi = dsa.visibility_ranges(pad, q_pos)
        S = dsa.index_scores(q, k, w, lo, hi, 0.088, k_scale=k_scale)
        torch.cuda.synchronize()
        ref, A = oracle.index_scores(cpu(q), cpu(k), cpu(w), 0.088, cpu(q_pos), cpu(pad),
                                     k_scale=None if k_scale is None else cpu(k_scale),
                                     want_mag=True)
        check_scores(cpu(S).numpy().reshape(ref.shape), ref, A, 1e-3, f"decode n_q={n_q}")


# ---------------------------------------------------------------- top-k

TOPK_CASES = [
    (1, {}, None, 8),
    (2, dict(B=4, Tk=8192), None, 2048),     # bench row length, one block per row
    (2, dict(B=3, Tk=517), "tie", 64),       # massive exact ties
    (2, dict(B=2, Tk=3000), None, 2048),     # k > visible for none, small-block path
    (2, dict(B=300, Tk=6000), None, 2048),   # many rows of 6000 keys: one block per row
    (3, dict(Tq=300, Tk=300), None, 100),    # causal: k >= visible on early rows
    (3, dict(Tq=2600, Tk=2600), None, 2048), # short rows, k = 2048: the last bucket spills past k
    (4, dict(B=2, Tk=40000), None, 2048),    # > one block's cache: threshold path
    (4, dict(B=1, Tk=40000), "tie", 2048),   # threshold path with ties
    (4, dict(B=1, Tk=150000), None, 2048),   # threshold path, a partial last block
]


@pytest.mark.parametrize("cfg,over,variant,k", TOPK_CASES)
def test_topk_bit_exact_on_gpu_scores(dsa, cfg, over, variant, k):
    note(f"topk config {cfg} {over} {variant} k={k}")
    inp, lo, hi, S = _index_case(dsa, cfg, over, variant)
    idx = dsa.topk(S, lo, hi, k)
    torch.cuda.synchronize()
    Sc = cpu(S).numpy().reshape(-1, S.shape[-1])
    qp, pd = _rows_qpos_pad(inp)
    ref = oracle.topk(Sc, qp, pd, k)
    got = cpu(idx).numpy().reshape(ref.shape)
    bad = np.nonzero((got != ref).any(1))[0]
    assert bad.size == 0, f"rows differ: {bad[:10]} first: {got[bad[0]][:16]} vs {ref[bad[0]][:16]}"


def test_topk_long_rows_skewed(dsa):
    """Long rows where one stretch of columns holds every top score (one
    block's pairs alone set the threshold), a row whose last, partial block
    wins, and a row whose visible window leaves blocks with fewer keys than
    their pairs' ranks."""
    note("topk long rows, skewed")
    rng = np.random.default_rng(21)
    n, k = 150000, 2048
    rows = rng.standard_normal((3, n)).astype(np.float32)
    rows[0, 20000:40000] += 50.0          # the top scores all in one chunk
    rows[1, :] = rng.standard_normal(n).astype(np.float32) * 1e-3
    rows[1, 131072:] += 10.0              # the last (partial) chunk wins
    S = torch.tensor(rows, device="cuda")
    lo = torch.tensor([0, 0, 100000], dtype=torch.int32, device="cuda")
    hi = torch.tensor([n, n, 116500], dtype=torch.int32, device="cuda")
    idx = dsa.topk(S, lo, hi, k)
    torch.cuda.synchronize()
    got = cpu(idx).numpy()
    for i in range(3):
        l0, h0 = int(lo[i]), int(hi[i])
        r = rows[i]
        cand = np.arange(l0, h0)
        order = cand[np.lexsort((cand, -r[l0:h0].astype(np.float64)))][:k]
        exp = np.concatenate([order, np.full(k - order.size, INV)])
        assert (got[i] == exp).all(), i


def test_topk_edge_rows(dsa):
    note("topk edge rows")
    n = 777
    rows = []
    rows.append(np.full(n, 0.5, np.float32))                             # all equal
    rows.append(np.where(np.arange(n) % 2 == 0, 0.0, -0.0).astype(np.float32))  # +-0
    r = np.random.default_rng(3).standard_normal(n).astype(np.float32)
    rows.append(r)                                                       # empty range
    rows.append(r)                                                       # 1 visible key
    rows.append(-np.abs(r))                                              # negatives
    rows.append(np.array([np.inf, -np.inf] * (n // 2) + [1.0], np.float32))
    S = torch.tensor(np.stack(rows), device="cuda")
    lo = torch.tensor([0, 3, 5, 10, 0, 0], dtype=torch.int32, device="cuda")
    hi = torch.tensor([n, n, 5, 11, 600, n], dtype=torch.int32, device="cuda")
    for k in (1, 5, 300, 2048):
        idx = dsa.topk(S, lo, hi, k)
        torch.cuda.synchronize()
        got = cpu(idx).numpy()
        for i in range(len(rows)):
            l0, h0 = int(lo[i]), int(hi[i])
            cand = sorted(range(l0, h0), key=lambda s: (-float(rows[i][s]), s))[:k]
            exp = cand + [INV] * (k - len(cand))
            assert got[i].tolist() == exp, (i, k)


def test_topk_segmented_rows(dsa):
    """Few rows, so several blocks share each row and each writes one segment
    of its ranks: ties straddling segment boundaries and the k-th rank,
    crowded value buckets, an outlier, a value range that overflows f32, a
    visibility window, and a k that the segments do not divide."""
    note("topk segmented rows")
    rng = np.random.default_rng(33)
    n = 8192
    rows = [
        np.round(rng.standard_normal(n) * 50.0) / 50.0,      # ~400 levels: ties everywhere
        rng.integers(0, 4, n).astype(np.float64),            # 4 levels: crowded buckets
        np.concatenate([[1e30], rng.standard_normal(n - 1)]),  # one outlier
        np.concatenate([[3e38, -3e38], rng.standard_normal(n - 2)]),  # range overflows
        rng.standard_normal(n),
        rng.standard_normal(n) * 1e-30,                      # tiny values
    ]
    rows = np.stack(rows).astype(np.float32)
    S = torch.tensor(rows, device="cuda")
    lo = torch.tensor([0, 0, 0, 0, 1000, 0], dtype=torch.int32, device="cuda")
    hi = torch.tensor([n, n, n, n, 7000, n], dtype=torch.int32, device="cuda")
    for k in (2048, 1000, 256):
        idx = dsa.topk(S, lo, hi, k)
        torch.cuda.synchronize()
        got = cpu(idx).numpy()
        for i in range(rows.shape[0]):
            l0, h0 = int(lo[i]), int(hi[i])
            cand = np.arange(l0, h0)
            order = cand[np.lexsort((cand, -rows[i][l0:h0].astype(np.float64)))][:k]
            exp = np.concatenate([order, np.full(k - order.size, INV)])
            assert (got[i] == exp).all(), (i, k, np.nonzero(got[i] != exp)[0][:8])


def test_topk_long_rows_segmented_merge(dsa):
    """Rows longer than one block's cache whose chunk winners fit the merge
    cache, so the merge is split over several blocks per row: quantized
    ties, four levels (crowded buckets), an outlier, every score equal,
    plain values, and a window that leaves the last chunk short."""
    note("topk long rows, segmented merge")
    rng = np.random.default_rng(44)
    n, k = 100000, 2048
    rows = [
        np.round(rng.standard_normal(n) * 50.0) / 50.0,
        rng.integers(0, 4, n).astype(np.float64),
        np.concatenate([[1e30], rng.standard_normal(n - 1)]),
        np.full(n, 0.25),
        rng.standard_normal(n),
        rng.standard_normal(n),
    ]
    rows = np.stack(rows).astype(np.float32)
    S = torch.tensor(rows, device="cuda")
    lo = torch.tensor([0, 0, 0, 0, 0, 30000], dtype=torch.int32, device="cuda")
    hi = torch.tensor([n, n, n, n, n, 50100], dtype=torch.int32, device="cuda")
    for kk in (k, 700):
        ws = torch.empty(max(dsa.topk_workspace_size(rows.shape[0], n, kk), 1), dtype=torch.uint8,
                         device="cuda")
        idx = dsa.topk(S, lo, hi, kk, workspace=ws)
        torch.cuda.synchronize()
        got = cpu(idx).numpy()
        for i in range(rows.shape[0]):
            l0, h0 = int(lo[i]), int(hi[i])
            cand = np.arange(l0, h0)
            order = cand[np.lexsort((cand, -rows[i][l0:h0].astype(np.float64)))][:kk]
            exp = np.concatenate([order, np.full(kk - order.size, INV)])
            assert (got[i] == exp).all(), (i, kk, np.nonzero(got[i] != exp)[0][:8])


# ---------------------------------------------------------------- attention

def _oracle_sel(inp, S, k):
    Sc = cpu(S).numpy().reshape(-1, S.shape[-1])
    qp, pd = _rows_qpos_pad(inp)
    return oracle.topk(Sc, qp, pd, k).reshape(S.shape[0], S.shape[1], k)


ABSORBED_CASES = [
    (2, dict(B=3, Tk=1500), None, 512),
    # 15 splits of 66-67 keys: ragged last tiles in every split-K block
    (2, dict(B=3, Tk=1500), None, 1000),
    (2, dict(B=2, Tk=2111), "sharp", 2048),
    (3, dict(Tq=200, Tk=200), None, 64),
    (4, dict(B=2, Tk=5000), None, 2048),
]


@pytest.mark.parametrize("cfg,over,variant,k", ABSORBED_CASES)
def test_absorbed_attend_parity(dsa, cfg, over, variant, k):
    note(f"absorbed attend config {cfg} {over} {variant} k={k}")
    inp, lo, hi, S = _index_case(dsa, cfg, over, variant)
    sel = _oracle_sel(inp, S, k)
    idx = torch.tensor(sel, device="cuda")
    kd, vd = inp["kd"], inp["vd"]
    out, lse = dsa.sparse_attend(inp["q"], inp["KV"], None, idx, inp["scale_attn"], kv_heads=1,
                                 vd=vd, vis_lo=lo, vis_hi=hi)
    torch.cuda.synchronize()
    ref, lref = oracle.sparse_attend(cpu(inp["q"]), cpu(inp["KV"]), None, sel, inp["scale_attn"],
                                     kv_heads=1, q_pos=cpu(inp["q_pos"]), pad=cpu(inp["pad"]),
                                     k_row_stride=kd, vd=vd)
    check_attend(cpu(out).numpy().reshape(ref.shape), ref, cpu(lse).numpy().reshape(lref.shape),
                 lref, bf16=True, what=f"config {cfg}")


def test_absorbed_attend_set_semantics(dsa):
    """Duplicates, INVALID, out-of-range and invisible entries, empty rows."""
    note("absorbed attend: set semantics")
    inp = W.make(2, device="cuda", B=5, Tk=700)
    B, Tk = 5, 700
    rng = np.random.default_rng(5)
    sel = rng.integers(-3, Tk + 40, (B, 1, 300)).astype(np.int32)
    sel[0, 0, :] = INV                        # empty
    sel[1, 0, 150:] = sel[1, 0, :150]         # every entry twice
    sel[2, 0, :] = 17                         # one key, many times
    # distinct entries, some INVALID (-1), negative, past n_k or invisible
    sel[4, 0, :] = rng.permutation(Tk + 43)[:300] - 3
    idx = torch.tensor(sel, device="cuda")
    lo = torch.full((B, 1), 5, dtype=torch.int32, device="cuda")
    hi = torch.full((B, 1), 650, dtype=torch.int32, device="cuda")
    out, lse = dsa.sparse_attend(inp["q"], inp["KV"], None, idx, inp["scale_attn"], 1, vd=512,
                                 vis_lo=lo, vis_hi=hi)
    torch.cuda.synchronize()
    ref, lref = oracle.sparse_attend(cpu(inp["q"]), cpu(inp["KV"]), None, sel,
                                     inp["scale_attn"], 1, q_pos=np.full((B, 1), 649),
                                     pad=np.full(B, 5), k_row_stride=576, vd=512)
    check_attend(cpu(out).numpy().reshape(ref.shape), ref, cpu(lse).numpy().reshape(lref.shape),
                 lref, bf16=True, what="set semantics")
    assert torch.all(out[0] == 0) and torch.all(torch.isneginf(lse[0]))


def test_absorbed_attend_split_partials_large_values(dsa):
    """Few rows (split-K partials) with latent rows x 2^26 and queries x 2^-26
    (both exact in bf16): the scores are unchanged and |V| reaches ~10^6, past
    the fp16 range the split partials are stored in, so their per-(row, split,
    head) power-of-two scale is what keeps the result."""
    note("absorbed attend: large V through the split partials")
    inp, lo, hi, S = _index_case(dsa, 2, dict(B=2, Tk=3000), None)
    sel = _oracle_sel(inp, S, 2048)
    idx = torch.tensor(sel, device="cuda")
    q = (inp["q"].float() * 2.0 ** -26).to(torch.bfloat16)
    kv = (inp["KV"].float() * 2.0 ** 26).to(torch.bfloat16)
    assert torch.equal(q.float() * 2.0 ** 26, inp["q"].float())
    out, lse = dsa.sparse_attend(q, kv, None, idx, inp["scale_attn"], kv_heads=1, vd=512,
                                 vis_lo=lo, vis_hi=hi)
    torch.cuda.synchronize()
    assert float(cpu(out).abs().max()) > 65504.0
    ref, lref = oracle.sparse_attend(cpu(q), cpu(kv), None, sel, inp["scale_attn"],
                                     kv_heads=1, q_pos=cpu(inp["q_pos"]), pad=cpu(inp["pad"]),
                                     k_row_stride=576, vd=512)
    check_attend(cpu(out).numpy().reshape(ref.shape), ref, cpu(lse).numpy().reshape(lref.shape),
                 lref, bf16=True, what="large values")


def test_absorbed_attend_long_context_distinct(dsa):
    """n_k past the gather kernel's limit of 262144 keys (300000 keys): the
    absorbed layout then runs attend_plain_kernel, here with distinct keys,
    INVALID entries and a visibility window.  The gather kernel's own
    set-bitmap path at n_k = 262144 is covered in test_gpu_paths.py."""
    note("absorbed attend: n_k = 300000")
    B, Tk = 1, 300000
    inp = W.make(2, device="cuda", B=B, Tk=Tk)
    rng = np.random.default_rng(11)
    sel = np.full((B, 1, 512), INV, dtype=np.int32)
    sel[0, 0, :400] = rng.choice(Tk, 400, replace=False)
    idx = torch.tensor(sel, device="cuda")
    lo = torch.full((B, 1), 1000, dtype=torch.int32, device="cuda")
    hi = torch.full((B, 1), 290000, dtype=torch.int32, device="cuda")
    out, lse = dsa.sparse_attend(inp["q"], inp["KV"], None, idx, inp["scale_attn"], 1, vd=512,
                                 vis_lo=lo, vis_hi=hi)
    torch.cuda.synchronize()
    ref, lref = oracle.sparse_attend(cpu(inp["q"]), cpu(inp["KV"]), None, sel,
                                     inp["scale_attn"], 1, q_pos=np.full((B, 1), 289999),
                                     pad=np.full(B, 1000), k_row_stride=576, vd=512)
    check_attend(cpu(out).numpy().reshape(ref.shape), ref, cpu(lse).numpy().reshape(lref.shape),
                 lref, bf16=True, what="long context")


def test_attend_plain_f32_per_head_and_shared(dsa):
    note("plain attend f32 (config 1)")
    inp = W.make(1, device="cuda")
    lo, hi = _ranges(dsa, inp)
    S = dsa.index_scores(inp["q_idx"], inp["k_idx"], inp["w"], lo, hi, inp["scale_idx"])
    torch.cuda.synchronize()
    sel = _oracle_sel(inp, S, 8)
    idx = torch.tensor(sel, device="cuda")
    for K, V, kvh in ((inp["K"], inp["V"], 4), (inp["K1"], inp["V1"], 1)):
        out, lse = dsa.sparse_attend(inp["q"], K, V, idx, inp["scale_attn"], kvh, vis_lo=lo,
                                     vis_hi=hi)
        torch.cuda.synchronize()
        ref, lref = oracle.sparse_attend(cpu(inp["q"]), cpu(K), cpu(V), sel, inp["scale_attn"],
                                         kvh, q_pos=cpu(inp["q_pos"]), pad=cpu(inp["pad"]))
        check_attend(cpu(out).numpy().reshape(ref.shape), ref,
                     cpu(lse).numpy().reshape(lref.shape), lref, bf16=False,
                     what=f"config 1 kv_heads {kvh}")


def test_attend_plain_bf16_per_head_other_shape(dsa):
    note("plain attend bf16 per-head (shape outside the MFMA kernels)")
    gen = torch.Generator(device="cuda").manual_seed(11)
    B, T, H, kd, vd = 2, 50, 4, 96, 80
    q = (torch.randn(B, T, H, kd, generator=gen, device="cuda") / kd ** 0.5).bfloat16()
    K = (torch.randn(B, T, H, kd, generator=gen, device="cuda") / kd ** 0.5).bfloat16()
    V = (torch.randn(B, T, H, vd, generator=gen, device="cuda") / vd ** 0.5).bfloat16()
    sel = np.random.default_rng(2).integers(-1, T, (B, T, 20)).astype(np.int32)
    idx = torch.tensor(sel, device="cuda")
    out, lse = dsa.sparse_attend(q, K, V, idx, kd ** -0.5, H)
    torch.cuda.synchronize()
    ref, lref = oracle.sparse_attend(cpu(q), cpu(K), cpu(V), sel, kd ** -0.5, H)
    check_attend(cpu(out).numpy().reshape(ref.shape), ref, cpu(lse).numpy().reshape(lref.shape),
                 lref, bf16=True, what="plain bf16")


# ---------------------------------------------------------------- pooled path

def test_pool_keys_within_one_ulp(dsa):
    note("pool keys (config 5 shape, reduced length)")
    inp = W.make(5, device="cuda", L=1030)
    pk, npools = dsa.pool_keys(inp["k_idx"], inp["gate"], inp["pad"], 4)
    torch.cuda.synchronize()
    ref, rn, mag = oracle.pool_keys(cpu(inp["k_idx"]), cpu(inp["gate"]), cpu(inp["pad"]), 4,
                                    want_mag=True)
    assert cpu(npools).tolist() == rn.tolist()
    bf16_ulp_ok(cpu(pk), ref, mag, "pool keys")
    for b, n in enumerate(rn):
        assert torch.all(pk[b, n:] == 0)


@pytest.mark.parametrize("variant", [None, "tie"])
def test_pool_select_bit_exact(dsa, variant):
    note(f"pool select (config 5 shape, reduced) {variant}")
    L, kp, sk, width = 1030, 4, 64, 64 * 4 + 4
    inp = W.make(5, device="cuda", L=L, variant=variant)
    pk, _ = dsa.pool_keys(inp["k_idx"], inp["gate"], inp["pad"], kp)
    lo, hi = dsa.visibility_ranges(inp["pad"], inp["q_pos"], kp)
    S = dsa.index_scores(inp["q_idx"], pk, inp["w"], lo, hi, inp["scale_idx"])
    tok, pools = dsa.pool_select(S, inp["pad"], inp["q_pos"], kp, sk, width, want_pools=True)
    torch.cuda.synchronize()
    Sc = cpu(S).numpy().reshape(-1, S.shape[-1])
    qp, pd = _rows_qpos_pad(inp)
    rtok, rpools = oracle.pool_select(Sc, qp, pd, kp, sk, width, want_pools=True)
    assert np.array_equal(cpu(tok).numpy().reshape(rtok.shape), rtok)
    assert np.array_equal(cpu(pools).numpy().reshape(rpools.shape), rpools)


# ---------------------------------------------------------------- ABI contract

def test_abi_rejects_bad_arguments(dsa):
    note("ABI argument errors")
    S = torch.zeros(2, 10, device="cuda")
    lo = torch.zeros(2, dtype=torch.int32, device="cuda")
    hi = torch.full((2,), 10, dtype=torch.int32, device="cuda")
    with pytest.raises(dsa.DsaError) as e:
        dsa.topk(S, lo, hi, 4096)
    assert e.value.code == -2
    with pytest.raises(dsa.DsaError) as e:
        dsa.topk(S, lo, hi, 0)
    assert e.value.code == -1
    q = torch.zeros(1, 1, 48, 128, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(1, 8, 128, dtype=torch.bfloat16, device="cuda")
    w = torch.zeros(1, 1, 48, device="cuda")
    l1 = torch.zeros(1, 1, dtype=torch.int32, device="cuda")
    with pytest.raises(dsa.DsaError) as e:
        dsa.index_scores(q, k, w, l1, l1, 1.0)
    assert e.value.code == -2
    assert "n_heads" in str(e.value)


# ---------------------------------------------------------------- masked per-head attention

def _pooled_selection(dsa, inp, kp, sk, width):
    pk, _ = dsa.pool_keys(inp["k_idx"], inp["gate"], inp["pad"], kp)
    lo, hi = dsa.visibility_ranges(inp["pad"], inp["q_pos"], kp)
    S = dsa.index_scores(inp["q_idx"], pk, inp["w"], lo, hi, inp["scale_idx"])
    torch.cuda.synchronize()
    Sc = cpu(S).numpy().reshape(-1, S.shape[-1])
    qp, pd = _rows_qpos_pad(inp)
    return oracle.pool_select(Sc, qp, pd, kp, sk, width).reshape(inp["B"], inp["Tq"], width)


@pytest.mark.parametrize("L,sk,variant", [(700, 32, None), (333, 16, "sharp")])
def test_masked_attend_pooled_selection(dsa, L, sk, variant):
    """Per-head attention over the oracle's pool selection (config 5 shape,
    reduced length; ragged query blocks and key tiles)."""
    note(f"masked attend, pooled selection L={L} select_k={sk} {variant}")
    kp = 4
    width = sk * kp + kp
    inp = W.make(5, device="cuda", L=L, variant=variant)
    sel = _pooled_selection(dsa, inp, kp, sk, width)
    idx = torch.tensor(sel, device="cuda")
    lo, hi = dsa.visibility_ranges(inp["pad"], inp["q_pos"])
    out, lse = dsa.sparse_attend(inp["q"], inp["K"], inp["V"], idx, inp["scale_attn"],
                                 kv_heads=inp["H"], vis_lo=lo, vis_hi=hi)
    torch.cuda.synchronize()
    ref, lref = oracle.sparse_attend(cpu(inp["q"]), cpu(inp["K"]), cpu(inp["V"]), sel,
                                     inp["scale_attn"], inp["H"], q_pos=cpu(inp["q_pos"]),
                                     pad=cpu(inp["pad"]))
    check_attend(cpu(out).numpy().reshape(ref.shape), ref, cpu(lse).numpy().reshape(lref.shape),
                 lref, bf16=True, what=f"masked L={L}")
    # padded queries attend to nothing
    pads = cpu(inp["pad"]).tolist()
    for b, p in enumerate(pads):
        if p:
            assert torch.all(out[b, :p] == 0) and torch.all(torch.isneginf(lse[b, :p]))


@pytest.mark.parametrize("n_sel", [40, 37, 3001])
def test_masked_attend_set_semantics(dsa, n_sel):
    """Duplicates, INVALID and out-of-range entries; index rows of 40
    entries (the mask kernel reads four per load), of 37 (one per load) and
    of 3001 (twenty times the 150 keys: every key many times over)."""
    note(f"masked attend: duplicates / INVALID / out-of-range, no visibility ranges, n_sel={n_sel}")
    gen = torch.Generator(device="cuda").manual_seed(13)
    B, T, H, kd, vd = 2, 150, 8, 192, 256
    q = (torch.randn(B, T, H, kd, generator=gen, device="cuda") / kd ** 0.5).bfloat16()
    K = (torch.randn(B, T, H, kd, generator=gen, device="cuda") / kd ** 0.5).bfloat16()
    V = (torch.randn(B, T, H, vd, generator=gen, device="cuda") / vd ** 0.5).bfloat16()
    sel = np.random.default_rng(4).integers(-2, T + 9, (B, T, n_sel)).astype(np.int32)
    half = n_sel // 2
    sel[:, :, half:2 * half] = sel[:, :, :half]
    sel[0, 3, :] = INV
    idx = torch.tensor(sel, device="cuda")
    out, lse = dsa.sparse_attend(q, K, V, idx, kd ** -0.5, H)
    torch.cuda.synchronize()
    ref, lref = oracle.sparse_attend(cpu(q), cpu(K), cpu(V), sel, kd ** -0.5, H)
    check_attend(cpu(out).numpy().reshape(ref.shape), ref, cpu(lse).numpy().reshape(lref.shape),
                 lref, bf16=True, what="masked set semantics")
