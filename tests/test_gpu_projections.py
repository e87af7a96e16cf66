"""GPU parity of the dense projections ahead of the path against the
float64 oracle: the indexer front-end ("Another DSA attempt", batch-local
indexer commit: wq_b / wk / weights_proj, k_norm LayerNorm with bias, NEOX
rotation of the rope part) and expand_kv ("Module glm5next_dsa_ref").

Criterion, per element (derived from the arithmetic, not fitted): the GPU
accumulates the K products of bf16 operands in f32 on the matrix cores, so
a projection differs from the exact value by at most g*A with g = K*2^-24
and A = sum_k |a_k b_k|; LayerNorm maps an error e on its inputs to at most
2e|w_i|(1 + |x^_i|)/sigma on output i; the rotation mixes the errors of a
pair with |cos| and |sin|; f32 arithmetic of the norm and rotation adds a
few 2^-23 of the values; the bf16 output rounding adds half an ulp
(<= 2^-8 |value|)."""
import numpy as np
import pytest
import torch

import oracle
from sparse_attention_scores_amd import workloads as W
from tests.parity import cpu, note

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


@pytest.fixture(scope="module")
def dsa():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    from sparse_attention_scores_amd import binding
    binding.load()
    return binding


def _f64(t):
    return cpu(t).double().numpy()


def _check(got, ref, bound, what):
    err = np.abs(np.asarray(got, np.float64) - ref)
    bad = err > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {err.size} out of bound; worst "
                           f"|d| {err[bad].max():.3g} at ref {ref[bad][np.argmax(err[bad])]:.4g}")
    note(f"  {what}: worst {float((err / np.maximum(bound, 1e-300)).max()):.3g} of the bound")


def _rope_mix(e, pos, rope_dim, theta):
    """Errors after the rotation: e_i |cos| + e_j |sin| for each pair."""
    e = e.copy()
    h = rope_dim // 2
    inv = theta ** (-2.0 * np.arange(h) / rope_dim)
    ang = np.asarray(pos, np.float64).reshape((-1,) + (1,) * (e.ndim - 1)) * inv
    c, s = np.abs(np.cos(ang)), np.abs(np.sin(ang))
    a, b = e[..., :h].copy(), e[..., h:rope_dim].copy()
    e[..., :h] = a * c + b * s
    e[..., h:rope_dim] = b * c + a * s
    return e


def _frontend_case(dsa, inp, rows=None):
    T = inp["T"]
    Hi, R, th, eps = inp["Hi"], inp["rope_dim"], inp["rope_theta"], inp["norm_eps"]
    q, k, w = dsa.indexer_frontend(inp["q_lora"], inp["x"], inp["pos"], inp["wq_b"], inp["wk"],
                                   inp["k_norm_w"], inp["k_norm_b"], inp["w_proj"], Hi, R, th,
                                   eps)
    torch.cuda.synchronize()
    sel = np.arange(T) if rows is None else np.asarray(rows)
    pos = cpu(inp["pos"]).numpy()[sel]
    ql, x = inp["q_lora"][sel], inp["x"][sel]
    rq, rk, rw = oracle.indexer_frontend(cpu(ql), cpu(x), pos, cpu(inp["wq_b"]), cpu(inp["wk"]),
                                         cpu(inp["k_norm_w"]), cpu(inp["k_norm_b"]),
                                         cpu(inp["w_proj"]), Hi, R, th, eps)
    # q: projection error, rotated, then the bf16 rounding
    Aq = np.abs(_f64(ql)) @ np.abs(_f64(inp["wq_b"])).T
    yq = oracle.linear(cpu(ql), cpu(inp["wq_b"])).reshape(len(sel), Hi, 128)
    eq = _rope_mix(inp["q_lora_rank"] * U * Aq.reshape(len(sel), Hi, 128), pos, R, th)
    eq += 8 * U * _rope_mix(np.abs(yq), pos, R, th) + 2.0 ** -8 * np.abs(rq)
    _check(_f64(q[sel]), rq, eq * 1.001 + 1e-30, "q")
    # k: projection error through LayerNorm, rotated, bf16
    xk = oracle.linear(cpu(x), cpu(inp["wk"]))
    Ak = np.abs(_f64(x)) @ np.abs(_f64(inp["wk"])).T
    # input error: the projection's, plus the f32 summation of the row mean
    e = (inp["hidden"] * U * Ak.max(axis=1, keepdims=True)
         + 130 * U * np.abs(xk).mean(axis=1, keepdims=True))
    sd = np.sqrt(xk.var(axis=1, keepdims=True) + eps)
    xh = (xk - xk.mean(axis=1, keepdims=True)) / sd
    g, b = _f64(inp["k_norm_w"]), _f64(inp["k_norm_b"])
    z = oracle.layer_norm(xk, cpu(inp["k_norm_w"]), cpu(inp["k_norm_b"]), eps)
    ek = 2 * e * np.abs(g) * (1 + np.abs(xh)) / sd + 8 * U * (np.abs(g * xh) + np.abs(b))
    ek = _rope_mix(ek, pos, R, th) + 8 * U * _rope_mix(np.abs(z), pos, R, th)
    _check(_f64(k[sel]), rk, (ek + 2.0 ** -8 * np.abs(rk)) * 1.001, "k")
    # head weights: f32 output
    Aw = np.abs(_f64(x)) @ np.abs(_f64(inp["w_proj"])).T
    _check(_f64(w[sel]), rw, (inp["hidden"] * U * Aw + 2 * U * np.abs(rw)) * 1.001, "w")


@pytest.mark.parametrize("over", [
    dict(B=1, L=300),                                              # ragged against both tiles
    dict(B=3, L=37, Hi=64, rope_dim=32, q_lora_rank=512, hidden=1024),
    dict(B=1, L=130, rope_dim=128, rope_theta=50000.0, norm_eps=1e-5, q_lora_rank=128,
         hidden=192),
    dict(B=1, L=1, q_lora_rank=64, hidden=64),                    # one token
])
def test_indexer_frontend_parity(dsa, over):
    note(f"indexer front-end {over}")
    inp = W.make(7, device="cuda", **over)
    # positions far apart, including large ones (the angle is reduced in f64)
    T = inp["T"]
    inp["pos"] = torch.tensor((np.arange(T) * 7919 + 3) % 2000003, dtype=torch.int32,
                              device="cuda")
    _frontend_case(dsa, inp)


def test_indexer_frontend_layernorm_large_mean(dsa):
    """k rows whose entries share an offset tens of times their spread (a
    common component in every row of wk): the mean must be removed before
    the variance is formed (two passes)."""
    note("indexer front-end: LayerNorm with a large row mean")
    inp = W.make(7, device="cuda", B=1, L=260, q_lora_rank=128, hidden=256)
    u = torch.randn(256, device="cuda")
    inp["wk"] = (inp["wk"].float() + 4.0 * u[None, :]).bfloat16()
    _frontend_case(dsa, inp)


def test_indexer_frontend_full_size_sampled_rows(dsa):
    """65536 tokens in one launch (the pooled workload's token count), every
    output written; 96 sampled rows against the oracle."""
    note("indexer front-end: 65536 tokens, sampled rows")
    inp = W.make(7, device="cuda")
    rows = np.linspace(0, inp["T"] - 1, 96).astype(np.int64)
    _frontend_case(dsa, inp, rows=rows)


def _expand_case(dsa, inp, rows=None, strided=False):
    T, H, kd, vd = inp["T"], inp["H"], inp["kd"], inp["vd"]
    if strided:
        # outputs as slices of wider token rows (a cache with room for more)
        kbuf = torch.full((T, H * kd + 64), float("nan"), dtype=torch.bfloat16, device="cuda")
        vbuf = torch.full((T, H * vd + 8), float("nan"), dtype=torch.bfloat16, device="cuda")
        ko = kbuf.as_strided((T, H, kd), (H * kd + 64, kd, 1))
        vo = vbuf.as_strided((T, H, vd), (H * vd + 8, vd, 1))
        K, V = dsa.expand_kv(inp["latent"], inp["w_kv_b"], H, kd, vd, k_out=ko, v_out=vo)
    else:
        K, V = dsa.expand_kv(inp["latent"], inp["w_kv_b"], H, kd, vd)
    torch.cuda.synchronize()
    sel = np.arange(T) if rows is None else np.asarray(rows)
    lat = inp["latent"][sel]
    rK, rV = oracle.expand_kv(cpu(lat), cpu(inp["w_kv_b"]), H, kd, vd)
    A = (np.abs(_f64(lat)) @ np.abs(_f64(inp["w_kv_b"])).T).reshape(len(sel), H, kd + vd)
    g = inp["rank"] * U
    _check(_f64(K[sel]), rK, (g * A[..., :kd] + 2.0 ** -8 * np.abs(rK)) * 1.001, "K")
    _check(_f64(V[sel]), rV, (g * A[..., kd:] + 2.0 ** -8 * np.abs(rV)) * 1.001, "V")
    if strided:
        assert torch.isnan(kbuf[:, H * kd:].float()).all() and torch.isnan(vbuf[:, H * vd:].float()).all()


@pytest.mark.parametrize("over,strided", [
    (dict(B=1, L=300), False),
    (dict(B=1, L=77, H=4, kd=40, vd=24, rank=128), True),          # N = 256, odd widths
    (dict(B=2, L=100, H=3, kd=192, vd=256, rank=64), False),       # N = 1344: a partial tile
])
def test_expand_kv_parity(dsa, over, strided):
    note(f"expand_kv {over} strided={strided}")
    _expand_case(dsa, W.make(7, device="cuda", **over), strided=strided)


def test_expand_kv_full_size_sampled_rows(dsa):
    note("expand_kv: 65536 tokens x 64 heads, sampled rows")
    inp = W.make(7, device="cuda")
    _expand_case(dsa, inp, rows=np.linspace(0, inp["T"] - 1, 64).astype(np.int64))
