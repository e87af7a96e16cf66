"""GPU parity for every kernel path the ABI can take, named by the kernel.

The configuration-shaped cases in test_gpu_parity.py reach the decode and
prefill indexer kernels, the bucket top-k and the split merge; the cases here
reach the rest of what the ABI accepts:

  * index_scores_mfma_kernel (8-15 queries per sequence; fp8 keys with 8 or
    more queries; 64 indexer heads; head_dim 64, bf16 and fp8) and the decode
    kernel at 64 heads / head_dim 64; the prefill kernel with one workgroup
    per query block (many query blocks per CU);
  * pool_keys_kernel (one channel per thread: widths that 16-byte loads do
    not divide) and pool_keys_vec_kernel<float>, and pool_counts_kernel
    (sequences shorter than one pool);
  * pool_select_kernel in both shared layouts and both row capacities, with
    several blocks per row when there are few rows;
  * attend_gather_kernel's set-bitmap path (more than 2048 entries per row)
    at the largest n_k the gather kernel takes (262144);
  * topk_merge_kernel with the candidates in LDS (one block per row: 256 or
    more rows, or k < 128);
  * every output element written: outputs are filled with a poison value
    before each call and none may survive.

Each case compares against the oracle at the stated criteria (scores
relative, selection bit-exact, attention per row)."""
import numpy as np
import pytest
import torch

import oracle
from sparse_attention_scores_amd import workloads as W
from tests.parity import bf16_ulp_ok, check_attend, check_scores, cpu, note

pytestmark = pytest.mark.gpu

INV = -1
POISON_I32 = 0x7EADBEEF


@pytest.fixture(scope="module")
def dsa():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    from sparse_attention_scores_amd import binding
    binding.load()
    return binding


def _nan_like(shape, dtype=torch.float32):
    return torch.full(shape, float("nan"), dtype=dtype, device="cuda")


# ---------------------------------------------------------------- indexer kernels

# (config, overrides, kernel the launcher picks)
INDEX_PATH_CASES = [
    (2, dict(B=2, Tq=9, Tk=1000), "mfma<128,32 heads> bf16, 9 queries"),
    (2, dict(B=2, Tq=12, Tk=777), "mfma<128,32 heads> bf16, 12 queries"),
    (2, dict(B=3, Tq=15, Tk=300), "mfma<128,32 heads> bf16, 15 queries"),
    (4, dict(B=2, Tq=16, Tk=3001), "mfma<128,32 heads> fp8, 16 queries"),
    (4, dict(B=2, Tq=8, Tk=1000), "mfma<128,32 heads> fp8, 8 queries"),
    (2, dict(B=2, Tq=1, Tk=1000, Hi=64), "decode<128,64 heads> bf16"),
    (3, dict(Tq=100, Tk=100, Hi=64), "mfma<128,64 heads> bf16 causal"),
    (4, dict(B=2, Tq=1, Tk=999, Hi=64), "decode<128,64 heads> fp8"),
    (2, dict(B=2, Tq=1, Tk=1000, d=64), "decode<64,32 heads> bf16"),
    (3, dict(Tq=130, Tk=130, d=64), "mfma<64,32 heads> bf16 causal"),
    (4, dict(B=2, Tq=1, Tk=1000, d=64), "mfma<64,32 heads,1 query> fp8"),
    (4, dict(B=2, Tq=9, Tk=1000, d=64), "mfma<64,32 heads> fp8, 9 queries"),
    (4, dict(B=2, Tq=1, Tk=700, d=64, Hi=64), "mfma<64,64 heads,1 query> fp8"),
    (3, dict(Tq=77, Tk=77, d=64, Hi=64), "mfma<64,64 heads> bf16 causal"),
    (4, dict(B=2, Tq=8, Tk=1000, Hi=64), "mfma<128,64 heads> fp8, 8 queries"),
    (4, dict(B=2, Tq=9, Tk=1000, d=64, Hi=64), "mfma<64,64 heads> fp8, 9 queries"),
    (2, dict(B=2, Tq=1, Tk=1000, d=64, Hi=64), "decode<64,64 heads> bf16"),
]


@pytest.mark.parametrize("cfg,over,path", INDEX_PATH_CASES, ids=[c[2] for c in INDEX_PATH_CASES])
def test_index_scores_every_kernel_path(dsa, cfg, over, path):
    note(f"index scores path {path}: config {cfg} {over}")
    inp = W.make(cfg, device="cuda", **over)
    lo, hi = dsa.visibility_ranges(inp["pad"], inp["q_pos"])
    S = _nan_like((inp["B"], inp["Tq"], inp["Tk"]))
    dsa.index_scores(inp["q_idx"], inp["k_idx"], inp["w"], lo, hi, inp["scale_idx"],
                     k_scale=inp["k_scale"], out=S)
    torch.cuda.synchronize()
    assert not torch.isnan(S).any(), f"{path}: score elements left unwritten"
    ref, A = oracle.index_scores(cpu(inp["q_idx"]), cpu(inp["k_idx"]), cpu(inp["w"]),
                                 inp["scale_idx"], cpu(inp["q_pos"]), cpu(inp["pad"]),
                                 k_scale=None if inp["k_scale"] is None else cpu(inp["k_scale"]),
                                 want_mag=True)
    check_scores(cpu(S).numpy().reshape(ref.shape), ref, A, 1e-3, path, d=inp["d"],
                 heads=inp["Hi"])


def test_index_scores_generic_kernel_left_padding(dsa):
    """The generic MFMA kernel (9 queries per sequence, bf16 and fp8 keys)
    with left padding, a wholly padded sequence and queries short of the
    end, so its partial and invisible tiles are exercised."""
    B, n_q, H, d, Tk = 4, 9, 32, 128, 1000
    gen = torch.Generator(device="cuda").manual_seed(17)
    for fp8 in (False, True):
        note(f"index scores generic kernel, padding, fp8={fp8}")
        q = (torch.randn(B, n_q, H, d, generator=gen, device="cuda") / d ** 0.5).bfloat16()
        kf = torch.randn(B, Tk, d, generator=gen, device="cuda") / d ** 0.5
        k, k_scale = W.quantize_fp8_rows(kf) if fp8 else (kf.bfloat16(), None)
        w = torch.rand(B, n_q, H, generator=gen, device="cuda")
        pad = torch.tensor([0, 37, 999, 1000], dtype=torch.int32, device="cuda")
        steps = torch.arange(n_q, dtype=torch.int32, device="cuda") * 61
        q_pos = (torch.tensor([999, 990, 999, 700], dtype=torch.int32, device="cuda")[:, None]
                 - steps[None, :]).contiguous()
        lo, hi = dsa.visibility_ranges(pad, q_pos)
        S = _nan_like((B, n_q, Tk))
        dsa.index_scores(q, k, w, lo, hi, 0.088, k_scale=k_scale, out=S)
        torch.cuda.synchronize()
        assert not torch.isnan(S).any()
        ref, A = oracle.index_scores(cpu(q), cpu(k), cpu(w), 0.088, cpu(q_pos), cpu(pad),
                                     k_scale=None if k_scale is None else cpu(k_scale),
                                     want_mag=True)
        check_scores(cpu(S).numpy().reshape(ref.shape), ref, A, 1e-3, f"padding fp8={fp8}",
                     d=d, heads=H)


# ---------------------------------------------------------------- top-k, one merge block per row

@pytest.mark.parametrize("rows,n,k", [(256, 20000, 2048), (4, 40000, 100), (3, 70000, 64),
                                      (300, 16385, 777)])
def test_topk_merge_one_block_per_row(dsa, rows, n, k):
    """Rows longer than one block's cache (the shared-threshold path) with
    256 or more rows, or k below 128, so the merge of the candidates takes
    one block per row.  Some rows carry quantised ties and a visibility
    window."""
    note(f"topk one-block merge rows={rows} n={n} k={k}")
    gen = torch.Generator(device="cuda").manual_seed(rows * 7 + k)
    S = torch.randn(rows, n, generator=gen, device="cuda")
    S[::3] = torch.round(S[::3] * 20.0) / 20.0
    lo = torch.zeros(rows, dtype=torch.int32, device="cuda")
    hi = torch.full((rows,), n, dtype=torch.int32, device="cuda")
    lo[1::4] = 1000
    hi[1::4] = n - 333
    idx = torch.full((rows, k), POISON_I32, dtype=torch.int32, device="cuda")
    dsa.topk(S, lo, hi, k, out=idx)
    torch.cuda.synchronize()
    Sc = cpu(S).numpy()
    lo_c, hi_c = cpu(lo).numpy(), cpu(hi).numpy()
    # the oracle's visible range is [pad, q_pos + 1): pad = lo, q_pos = hi - 1
    ref = oracle.topk(Sc, hi_c - 1, lo_c, k)
    got = cpu(idx).numpy()
    bad = np.nonzero((got != ref).any(1))[0]
    assert bad.size == 0, f"rows differ: {bad[:10]}"


# ---------------------------------------------------------------- gather set-bitmap path

def _absorbed_inputs(B, Tk, seed):
    gen = torch.Generator(device="cuda").manual_seed(seed)
    q = (torch.randn(B, 1, 64, 576, generator=gen, device="cuda") / 24.0).bfloat16()
    kv = (torch.randn(B, Tk, 576, generator=gen, device="cuda") / 24.0).bfloat16()
    return q, kv


@pytest.mark.parametrize("B,Tk,n_sel", [(2, 262144, 3000), (3, 5000, 4096), (1, 2500, 2049)])
def test_gather_set_bitmap_path(dsa, B, Tk, n_sel):
    """More than 2048 entries per row: attend_gather_kernel builds the set
    from its bitmap directly.  Rows hold repeats, INVALID, out-of-range and
    invisible entries; the largest case sits at the gather kernel's n_k
    limit (262144)."""
    note(f"gather set-bitmap path B={B} n_k={Tk} n_sel={n_sel}")
    q, kv = _absorbed_inputs(B, Tk, 23 + B)
    rng = np.random.default_rng(Tk + n_sel)
    sel = rng.integers(0, Tk, (B, 1, n_sel)).astype(np.int32)
    sel[:, :, 1::7] = sel[:, :, 0::7][:, :, :sel[:, :, 1::7].shape[2]]  # repeats
    sel[:, :, 2::11] = INV
    sel[:, :, 3::13] = Tk + 5                                           # out of range
    sel[0, 0, 5::17] = -7
    idx = torch.tensor(sel, device="cuda")
    lo = torch.full((B, 1), 3, dtype=torch.int32, device="cuda")
    hi = torch.full((B, 1), Tk - 100, dtype=torch.int32, device="cuda")
    out = _nan_like((B, 1, 64, 512))
    lse = _nan_like((B, 1, 64))
    dsa.sparse_attend(q, kv, None, idx, 576 ** -0.5, 1, vd=512, vis_lo=lo, vis_hi=hi, out=out,
                      lse=lse)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any() and not torch.isnan(lse).any()
    ref, lref = oracle.sparse_attend(cpu(q), cpu(kv), None, sel, 576 ** -0.5, 1,
                                     q_pos=np.full((B, 1), Tk - 101), pad=np.full(B, 3),
                                     k_row_stride=576, vd=512)
    check_attend(cpu(out).numpy().reshape(ref.shape), ref, cpu(lse).numpy().reshape(lref.shape),
                 lref, bf16=True, what=f"bitmap path n_k={Tk} n_sel={n_sel}")


# ---------------------------------------------------------------- every output element written

def test_every_output_written_decode_step(dsa):
    """Poison in every output of a decode-shaped step (ranges, scores, top-k,
    gather + split combine); nothing may survive and each stage still
    matches the oracle."""
    note("poisoned outputs: decode step")
    inp = W.make(2, device="cuda", B=3, Tk=2500)
    B, Tq, Tk = inp["B"], inp["Tq"], inp["Tk"]
    lo = torch.full((B, Tq), POISON_I32, dtype=torch.int32, device="cuda")
    hi = torch.full((B, Tq), POISON_I32, dtype=torch.int32, device="cuda")
    dsa.visibility_ranges(inp["pad"], inp["q_pos"], lo=lo, hi=hi)
    S = _nan_like((B, Tq, Tk))
    dsa.index_scores(inp["q_idx"], inp["k_idx"], inp["w"], lo, hi, inp["scale_idx"], out=S)
    idx = torch.full((B, Tq, 2048), POISON_I32, dtype=torch.int32, device="cuda")
    dsa.topk(S, lo, hi, 2048, out=idx)
    out = _nan_like((B, Tq, 64, 512))
    lse = _nan_like((B, Tq, 64))
    dsa.sparse_attend(inp["q"], inp["KV"], None, idx, inp["scale_attn"], 1, vd=512, vis_lo=lo,
                      vis_hi=hi, out=out, lse=lse)
    torch.cuda.synchronize()
    assert not (lo == POISON_I32).any() and not (hi == POISON_I32).any()
    assert not torch.isnan(S).any()
    assert not (idx == POISON_I32).any()
    assert not torch.isnan(out).any() and not torch.isnan(lse).any()
    qp = cpu(inp["q_pos"]).numpy().reshape(-1)
    pd = np.repeat(cpu(inp["pad"]).numpy(), Tq)
    ridx = oracle.topk(cpu(S).numpy().reshape(B * Tq, Tk), qp, pd, 2048)
    assert np.array_equal(cpu(idx).numpy().reshape(ridx.shape), ridx)


def test_every_output_written_pooled_step(dsa):
    """Poison in every output of a pooled step: pooled keys (rows past
    n_pools must come back zero), n_pools, pooled scores, the token rows and
    pool rows of pool select, and the per-head attention's out and lse."""
    note("poisoned outputs: pooled step")
    kp, sk = 4, 24
    width = sk * kp + kp
    inp = W.make(5, device="cuda", L=301)
    B, L, d = inp["B"], inp["L"], inp["d"]
    pk = _nan_like((B, L // kp, d), torch.bfloat16)
    npools = torch.full((B,), POISON_I32, dtype=torch.int32, device="cuda")
    dsa.pool_keys(inp["k_idx"], inp["gate"], inp["pad"], kp, out=pk, n_pools=npools)
    plo, phi = dsa.visibility_ranges(inp["pad"], inp["q_pos"], kp)
    S = _nan_like((B, L, L // kp))
    dsa.index_scores(inp["q_idx"], pk, inp["w"], plo, phi, inp["scale_idx"], out=S)
    tok = torch.full((B, L, width), POISON_I32, dtype=torch.int32, device="cuda")
    pools = torch.full((B, L, sk), POISON_I32, dtype=torch.int32, device="cuda")
    dsa.pool_select(S, inp["pad"], inp["q_pos"], kp, sk, width, out_tok=tok, out_pools=pools,
                    want_pools=True)
    lo, hi = dsa.visibility_ranges(inp["pad"], inp["q_pos"])
    out = _nan_like((B, L, inp["H"], inp["vd"]))
    lse = _nan_like((B, L, inp["H"]))
    dsa.sparse_attend(inp["q"], inp["K"], inp["V"], tok, inp["scale_attn"], inp["H"], vis_lo=lo,
                      vis_hi=hi, out=out, lse=lse)
    torch.cuda.synchronize()
    assert not torch.isnan(pk.float()).any()
    rn = oracle.pool_keys(cpu(inp["k_idx"]), cpu(inp["gate"]), cpu(inp["pad"]), kp)[1]
    assert cpu(npools).tolist() == rn.tolist()
    for b, n in enumerate(rn):
        assert torch.all(pk[b, n:] == 0)
    assert not torch.isnan(S).any()
    assert not (tok == POISON_I32).any() and not (pools == POISON_I32).any()
    assert not torch.isnan(out).any() and not torch.isnan(lse).any()
    Sc = cpu(S).numpy().reshape(-1, S.shape[-1])
    qp = cpu(inp["q_pos"]).numpy().reshape(-1)
    pd = np.repeat(cpu(inp["pad"]).numpy(), L)
    rtok, rpools = oracle.pool_select(Sc, qp, pd, kp, sk, width, want_pools=True)
    assert np.array_equal(cpu(tok).numpy().reshape(rtok.shape), rtok)
    assert np.array_equal(cpu(pools).numpy().reshape(rpools.shape), rpools)
    ref, lref = oracle.sparse_attend(cpu(inp["q"]), cpu(inp["K"]), cpu(inp["V"]),
                                     rtok.reshape(B, L, width), inp["scale_attn"], inp["H"],
                                     q_pos=cpu(inp["q_pos"]), pad=cpu(inp["pad"]))
    check_attend(cpu(out).numpy().reshape(ref.shape), ref, cpu(lse).numpy().reshape(lref.shape),
                 lref, bf16=True, what="poisoned pooled attend")


def test_every_output_written_tiny_f32(dsa):
    """Poison in the f32 configuration's scores and attention (plain kernel)."""
    note("poisoned outputs: tiny f32")
    inp = W.make(1, device="cuda")
    lo, hi = dsa.visibility_ranges(inp["pad"], inp["q_pos"])
    S = _nan_like((1, 64, 64))
    dsa.index_scores(inp["q_idx"], inp["k_idx"], inp["w"], lo, hi, inp["scale_idx"], out=S)
    idx = torch.full((1, 64, 8), POISON_I32, dtype=torch.int32, device="cuda")
    dsa.topk(S, lo, hi, 8, out=idx)
    out = _nan_like((1, 64, 4, 32))
    lse = _nan_like((1, 64, 4))
    dsa.sparse_attend(inp["q"], inp["K"], inp["V"], idx, inp["scale_attn"], 4, vis_lo=lo,
                      vis_hi=hi, out=out, lse=lse)
    torch.cuda.synchronize()
    assert not torch.isnan(S).any() and not (idx == POISON_I32).any()
    assert not torch.isnan(out).any() and not torch.isnan(lse).any()


# ---------------------------------------------------------------- pool select paths

@pytest.mark.parametrize("np_cols,sk,kp", [(4096, 512, 4), (1000, 300, 2), (4096, 600, 4),
                                           (6000, 512, 4)])
def test_pool_select_rows_of_every_kind(dsa, np_cols, sk, kp):
    """pool_select_kernel on rows that stress the selection: one outlier
    stretching the range, all scores equal, coarse ties, infinite scores
    (which send the row to the full sort), next to plain rows,
    short rows, a row with exactly select_k pools and padded queries; both
    row capacities (up to 4096 and up to 16384 pools), the lean shared
    layout for select_k up to 512 and the full one above it, kpool 4 rows
    with and without 16-byte alignment (four-token stores or single ones).
    Bit-exact against the oracle."""
    note(f"pool select paths np_cols={np_cols} select_k={sk} kpool={kp}")
    B, n_q = 2, 24
    L = np_cols * kp
    gen = torch.Generator(device="cuda").manual_seed(np_cols + sk)
    S = torch.randn(B, n_q, np_cols, generator=gen, device="cuda")
    S[:, 1] = 0.25                                    # all equal
    S[:, 2] = torch.round(S[:, 2] * 2) / 2            # coarse ties
    S[:, 3, 7] = 1e30                                 # one outlier
    S[:, 4] = torch.round(S[:, 4] * 50) / 50
    S[:, 4, 0] = -1e30
    S[:, 8, 5] = float("inf")                         # two tied +inf, then finite
    S[:, 8, 9] = float("inf")
    S[:, 9, ::3] = float("-inf")                      # a third of the row -inf
    pad = torch.tensor([0, 37], dtype=torch.int32, device="cuda")
    qp = torch.full((B, n_q), L - 1, dtype=torch.int32, device="cuda")
    qp[:, 5] = torch.tensor([3, 36], dtype=torch.int32)          # padded / before any pool
    qp[:, 6] = pad + kp * 100 + 1                                 # 100 pools and a tail
    qp[:, 7] = pad + kp * sk - 1                                  # exactly select_k pools
    width = sk * kp + kp - 1
    tok, pools = dsa.pool_select(S, pad, qp, kp, sk, width, want_pools=True)
    torch.cuda.synchronize()
    rtok, rpools = oracle.pool_select(cpu(S).numpy().reshape(B * n_q, -1),
                                      cpu(qp).numpy().reshape(-1),
                                      np.repeat(cpu(pad).numpy(), n_q), kp, sk, width,
                                      want_pools=True)
    got = cpu(tok).numpy().reshape(rtok.shape)
    bad = np.nonzero((got != rtok).any(1))[0]
    assert bad.size == 0, f"rows differ: {bad[:8]}"
    assert np.array_equal(cpu(pools).numpy().reshape(rpools.shape), rpools)


# ---------------------------------------------------------------- prefill indexer, whole query blocks

def test_prefill_index_one_workgroup_per_query_block(dsa):
    """index_scores_prefill_kernel with one workgroup per query block, the
    mode it takes with eight or more query blocks per CU: 8 sequences x 4100
    causal queries over 4100 keys (a ragged last query block; two key
    chunks, the second of 4 keys), left pads from 0 to the whole sequence.
    Every output element is written; sampled rows within the scores'
    criterion of the oracle."""
    note("prefill indexer, one workgroup per query block (8 x 4100)")
    gen = torch.Generator(device="cuda").manual_seed(4100)
    B, T, H, d = 8, 4100, 32, 128
    q = (torch.randn(B, T, H, d, generator=gen, device="cuda") / d ** 0.5).bfloat16()
    k = (torch.randn(B, T, d, generator=gen, device="cuda") / d ** 0.5).bfloat16()
    w = torch.rand(B, T, H, generator=gen, device="cuda")
    pad = torch.tensor([0, 1, 17, 33, 64, 100, 4095, 4100], dtype=torch.int32, device="cuda")
    q_pos = torch.arange(T, dtype=torch.int32, device="cuda").expand(B, T).contiguous()
    lo, hi = dsa.visibility_ranges(pad, q_pos)
    S = _nan_like((B, T, T))
    dsa.index_scores(q, k, w, lo, hi, d ** -0.5, out=S)
    torch.cuda.synchronize()
    assert not torch.isnan(S).any()
    rng = np.random.default_rng(41)
    must = [b * T + t for b in range(B) for t in (0, 15, 16, 4095, 4096, T - 1)]
    rows = np.array(sorted(set(must) | set(rng.choice(B * T, 120, replace=False).tolist())),
                    np.int64)
    ref, A = oracle.index_scores(cpu(q), cpu(k), cpu(w), d ** -0.5, cpu(q_pos), cpu(pad),
                                 rows=rows, want_mag=True)
    got = cpu(S.reshape(B * T, T)[torch.tensor(rows, device="cuda")]).numpy()
    check_scores(got, ref, A, 1e-3, "prefill indexer, whole query blocks")


# ---------------------------------------------------------------- pool keys, bf16 rows of any width

@pytest.mark.parametrize("d,kp", [(36, 4), (128, 12)])
def test_pool_keys_bf16_one_channel_per_thread(dsa, d, kp):
    """bf16 keys whose width (36) is not a multiple of 8 take one channel per
    thread (pool_keys_kernel<uint16_t>); 128-wide ones take eight
    (pool_keys_vec_kernel: configs 5 and 6 with kpool 4, here kpool 12, whose
    rows are read slot by slot).  Each value within one bf16 ulp plus
    2^-20 mag of the f64 oracle, as for config 5."""
    note(f"pool keys bf16 d={d} kpool={kp}")
    gen = torch.Generator(device="cuda").manual_seed(d + kp)
    B, L = 2, 401
    k = torch.randn(B, L, d, generator=gen, device="cuda").bfloat16()
    gate = (torch.randn(B, L, d, generator=gen, device="cuda") * 2).bfloat16()
    pad = torch.tensor([0, 9], dtype=torch.int32, device="cuda")
    pk, npools = dsa.pool_keys(k, gate, pad, kp)
    torch.cuda.synchronize()
    ref, rn, mag = oracle.pool_keys(cpu(k), cpu(gate), cpu(pad), kp, want_mag=True)
    assert cpu(npools).tolist() == rn.tolist()
    for b, n in enumerate(rn):
        bf16_ulp_ok(cpu(pk[b, :n]), ref[b, :n], mag[b, :n], f"pool keys d={d} kpool={kp}")
        assert torch.all(pk[b, n:] == 0)


# ---------------------------------------------------------------- pool keys on f32, short sequences

@pytest.mark.parametrize("L,kp,d", [(1030, 4, 128), (515, 8, 128), (3, 4, 128), (1030, 4, 6),
                                    (1030, 12, 128)])
def test_pool_keys_f32_and_sequences_shorter_than_a_pool(dsa, L, kp, d):
    """f32 keys and gates: four channels per thread (pool_keys_vec_kernel
    <float>, d a multiple of 4; the pool's rows held in registers up to
    kpool 8, read slot by slot at kpool 12) and one (pool_keys_kernel<float>,
    d = 6); and
    L < kpool, where no pool exists and only the counts are written
    (pool_counts_kernel).
    Criterion: each pooled value within 2 (kpool + 4) 2^-24 mag + 2^-23 |ref|
    of the f64 oracle, mag = sum_j softmax_j |k_j|: the kernel forms kpool
    exponentials (two ulps each), two sums of kpool terms and one quotient in
    f32, a factor 2 over those rounding steps."""
    note(f"pool keys f32 L={L} kpool={kp} d={d}")
    gen = torch.Generator(device="cuda").manual_seed(L * 7 + kp + d)
    B = 3
    k = torch.randn(B, L, d, generator=gen, device="cuda")
    gate = torch.randn(B, L, d, generator=gen, device="cuda") * 3
    pad = torch.tensor([0, min(1, L), min(13, L)], dtype=torch.int32, device="cuda")
    out = torch.full((B, L // kp, d), float("nan"), device="cuda")
    n_pools = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    pk, npools = dsa.pool_keys(k, gate, pad, kp, out=out, n_pools=n_pools)
    torch.cuda.synchronize()
    ref, rn, mag = oracle.pool_keys(cpu(k), cpu(gate), cpu(pad), kp, want_mag=True)
    assert cpu(npools).tolist() == rn.tolist()
    if L // kp == 0:
        assert pk.numel() == 0
        return
    got = cpu(pk).double().numpy()
    for b, n in enumerate(rn):
        assert np.all(got[b, n:] == 0.0), "pools past n_pools must be zero"
        g, r, m = got[b, :n], ref[b, :n], mag[b, :n]
        bound = 2 * (kp + 4) * 2.0 ** -24 * m + 2.0 ** -23 * np.abs(r)
        assert np.all(np.abs(g - r) <= bound), float((np.abs(g - r) / bound).max())
