"""GPU parity of the pooled decode step ("Module glm5next_dsa_ref": pool_states,
index_scores over pools, topk_pools + expand_selection, topk_to_mask and
mla_masked_attention, at one query per sequence) and of the per-head gather
kernel that attends a few queries per sequence (attend_heads_gather_kernel):
set semantics of each index row (duplicates once, INVALID / out-of-range /
invisible entries dropped, empty rows), the largest selected set it holds
(4096), left padding, a negative scale, long key ranges.  Criteria as for
the other attention tests (per row: max |d| <= 2e-3 ||out||_inf, cosine,
lse)."""
import numpy as np
import pytest
import torch

import bench
import oracle
from sparse_attention_scores_amd import workloads as W
from tests.parity import check_attend, check_scores, cpu, note

pytestmark = pytest.mark.gpu

INV = -1


@pytest.fixture(scope="module")
def dsa():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    from sparse_attention_scores_amd import binding
    binding.load()
    return binding


def test_pooled_decode_full_size(dsa):
    """Configuration 6 in bench's launch configuration: 4 sequences x 16384
    tokens, one query at each last position."""
    note("pooled decode, 4 x 16384, last positions")
    inp = W.make(6, device="cuda")
    step = bench.PooledStep(dsa, inp)
    for f in (step.pool_keys, step.index, step.pool_select, step.attend):
        f()
    torch.cuda.synchronize()
    B, L, kp = inp["B"], inp["L"], inp["kpool"]
    NP = L // kp
    pads = cpu(inp["pad"]).numpy()
    qp = cpu(inp["q_pos"]).numpy().reshape(-1)
    ref, A = oracle.index_scores(cpu(inp["q_idx"]), cpu(step.pk), cpu(inp["w"]),
                                 inp["scale_idx"], cpu(inp["q_pos"]), pads, kpool=kp,
                                 want_mag=True)
    check_scores(cpu(step.S).numpy().reshape(B, NP), ref, A, 1e-3, "pooled decode scores")
    S = cpu(step.S).numpy().reshape(B, NP)
    tok_ref = oracle.pool_select(S, qp, pads, kp, inp["select_k"], inp["out_width"])
    assert np.array_equal(cpu(step.tok).numpy().reshape(B, -1), tok_ref)
    out_ref, lse_ref = oracle.sparse_attend(cpu(inp["q"]), cpu(inp["K"]), cpu(inp["V"]),
                                            tok_ref.reshape(B, 1, -1), inp["scale_attn"],
                                            inp["H"], q_pos=cpu(inp["q_pos"]), pad=pads)
    check_attend(cpu(step.out).numpy().reshape(out_ref.shape), out_ref,
                 cpu(step.lse).numpy().reshape(lse_ref.shape), lse_ref, bf16=True,
                 what="pooled decode attend")


def _per_head(B, n_q, n_k, H, seed):
    gen = torch.Generator(device="cuda").manual_seed(seed)
    q = (torch.randn(B, n_q, H, 192, generator=gen, device="cuda") / 192 ** 0.5).bfloat16()
    K = (torch.randn(B, n_k, H, 192, generator=gen, device="cuda") / 192 ** 0.5).bfloat16()
    V = (torch.randn(B, n_k, H, 256, generator=gen, device="cuda") / 16).bfloat16()
    return q, K, V


@pytest.mark.parametrize("B,n_q,n_k,H,n_sel,scale", [
    (3, 1, 5000, 8, 700, 192 ** -0.5),       # duplicates, INVALID, out of range, invisible
    (2, 2, 9000, 4, 4096, 192 ** -0.5),      # the largest set the kernel holds
    (1, 1, 300000, 2, 3000, -0.11),          # long key range, negative scale
    (4, 3, 2000, 16, 600, 0.0),              # zero scale: uniform weights
])
def test_heads_gather_parity(dsa, B, n_q, n_k, H, n_sel, scale):
    note(f"per-head gather B={B} n_q={n_q} n_k={n_k} H={H} n_sel={n_sel} scale={scale:.3g}")
    q, K, V = _per_head(B, n_q, n_k, H, n_k + n_sel)
    rng = np.random.default_rng(n_sel)
    sel = rng.integers(0, n_k, (B, n_q, n_sel)).astype(np.int32)
    sel[..., 1::5] = sel[..., 0::5][..., :sel[..., 1::5].shape[-1]]      # repeats
    sel[..., 2::9] = INV
    sel[..., 3::11] = n_k + 7                                             # out of range
    sel[0, 0, :] = INV                                                    # an empty row
    pad = np.array([(13 * b) % 97 for b in range(B)], np.int32)
    qpos = np.array([[n_k - 1 - 211 * t for t in range(n_q)] for _ in range(B)], np.int32)
    lo, hi = dsa.visibility_ranges(torch.tensor(pad, device="cuda"),
                                   torch.tensor(qpos, device="cuda"))
    idx = torch.tensor(sel, device="cuda")
    out = torch.full((B, n_q, H, 256), float("nan"), device="cuda")
    lse = torch.full((B, n_q, H), float("nan"), device="cuda")
    dims = dsa._AttnDims(B, n_q, n_k, H, 192, 256, H, n_sel, scale)
    assert dsa.sparse_attend_workspace_size(dims) == 0     # the gather path needs none
    dsa.sparse_attend(q, K, V, idx, scale, H, vis_lo=lo, vis_hi=hi, out=out, lse=lse)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any() and not torch.isnan(lse).any()
    ref, lref = oracle.sparse_attend(cpu(q), cpu(K), cpu(V), sel, scale, H, q_pos=qpos, pad=pad)
    check_attend(cpu(out).numpy().reshape(ref.shape), ref, cpu(lse).numpy().reshape(lref.shape),
                 lref, bf16=True, what=f"per-head gather n_sel={n_sel}")
    assert torch.all(out[0, 0] == 0) and torch.all(torch.isneginf(lse[0, 0]))
