"""Seeded synthetic workloads shaped like GLM-5.x DSA layers.

This module only draws random numbers and stores them in the input formats
(f32, bf16 with round-to-nearest-even, OCP fp8 e4m3fn with one f32 scale per
key row).  It holds none of the method's arithmetic, so both the GPU library's
tests and the CPU oracle's tests may use it.

Configurations (all inputs synthetic; no checkpoint or dataset is used):

1. tiny fp32 layer: 1 sequence, 64 tokens, all positions are causal queries;
   indexer 4 heads x dim 32, w ~ U(0,1), top_k 8; attention 4 heads, kd 48,
   vd 32, per-head K/V (also a single shared K/V head); q/k/v ~ N(0,1).
2. decode, bf16: 32 sequences x 1 query (last position) over 8192 keys;
   indexer 32 heads x 128, top_k 2048; absorbed MLA 64 heads over shared
   latent rows of 576 (V = first 512 columns).  Values ~ N(0,1)/sqrt(d).
3. causal prefill, bf16: 1 sequence of 4096 tokens; dims as 2.
4. long-context decode: 8 sequences x 1 query over 131072 keys, fp8 e4m3
   indexer keys with a per-row scale; dims as 2.
5. pooled NoPE, bf16: 4 sequences of 16384 tokens with left padding
   (0, 2, 37, 64); kpool 4; indexer 32 x 128 with gate ~ N(0,1); top 512
   pools plus the visible tail, out_width 2052; per-head attention 64 heads,
   kd 192, vd 256.
6. pooled decode: configuration 5's sequences and keys with one query per
   sequence, at its last position.
7. projections at configuration 5's token count (4 x 16384): the indexer
   front-end (q_lora rank 2048, hidden 6144 -> 32 heads x 128, rope 64,
   theta 10000, k_norm eps 1e-6) and expand_kv (latent rank 512 -> 64
   heads x (192 + 256)).  The pages give no model widths; these are
   stand-ins of the model's class.  Activations ~ N(0,1); weights
   ~ N(0, 1/fan_in); the k_norm weight ~ 1 + N(0, 0.1^2), its bias
   ~ N(0, 0.1^2); positions 0 .. 16383 per sequence.

Tensors are drawn in a fixed order from one torch.Generator on the target
device, seeded with ``1000 + config`` unless a seed is given.
"""
from __future__ import annotations

import math

import torch

FP8_MAX = 448.0  # largest finite OCP e4m3fn magnitude

# Full sizes of each configuration.
CONFIGS = {
    1: dict(B=1, Tq=64, Tk=64, Hi=4, d=32, top_k=8, H=4, kd=48, vd=32, dtype="f32",
            causal=True),
    2: dict(B=32, Tq=1, Tk=8192, Hi=32, d=128, top_k=2048, H=64, kd=576, vd=512,
            dtype="bf16", causal=False),
    3: dict(B=1, Tq=4096, Tk=4096, Hi=32, d=128, top_k=2048, H=64, kd=576, vd=512,
            dtype="bf16", causal=True),
    4: dict(B=8, Tq=1, Tk=131072, Hi=32, d=128, top_k=2048, H=64, kd=576, vd=512,
            dtype="bf16", causal=False, fp8_keys=True),
    5: dict(B=4, L=16384, pads=(0, 2, 37, 64), kpool=4, Hi=32, d=128, select_k=512,
            out_width=2052, H=64, kd=192, vd=256, dtype="bf16"),
    6: dict(B=4, L=16384, pads=(0, 2, 37, 64), kpool=4, Hi=32, d=128, select_k=512,
            out_width=2052, H=64, kd=192, vd=256, dtype="bf16", last_only=True),
    7: dict(B=4, L=16384, q_lora_rank=2048, hidden=6144, Hi=32, d=128, rope_dim=64,
            rope_theta=10000.0, norm_eps=1e-6, rank=512, H=64, kd=192, vd=256,
            dtype="bf16"),
}


def _randn(shape, gen, device, std=1.0):
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32) * std


def _rand(shape, gen, device):
    return torch.rand(shape, generator=gen, device=device, dtype=torch.float32)


def to_bf16(x: torch.Tensor) -> torch.Tensor:
    """Round float32 to bfloat16 (round to nearest even)."""
    return x.to(torch.bfloat16)


def quantize_fp8_rows(x: torch.Tensor):
    """Quantise each last-dim row to OCP e4m3fn with scale max|row|/448.

    Returns (codes as torch.float8_e4m3fn, scales float32 [...])."""
    amax = x.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
    y = (x / scale.unsqueeze(-1)).clamp(-FP8_MAX, FP8_MAX)
    return y.to(torch.float8_e4m3fn), scale.float()


def _ints(shape, lo, hi, gen, device):
    return torch.randint(lo, hi, shape, generator=gen, device=device).float()


def make(config: int, device="cpu", seed=None, variant=None, **over):
    """Build the inputs of one configuration.

    ``over`` replaces any size (e.g. ``B=2, Tk=1024``) to make a smaller case
    of the same shape family.  ``variant``:
      * ``"tie"``  -- indexer q/k drawn from {-1,0,1} and w from {0.5,1}, so
        many index scores tie exactly (top-k tie-break stress);
      * ``"sharp"`` -- attention queries x16 (peaked softmax).
    Returns a dict of tensors on ``device`` plus the sizes used."""
    cfg = dict(CONFIGS[config])
    cfg.update(over)
    seed = 1000 + config if seed is None else seed
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    out = dict(cfg)
    out["config"] = config
    out["seed"] = seed
    out["variant"] = variant
    if config in (5, 6):
        return _make_pooled(cfg, gen, device, variant, out)
    if config == 7:
        return _make_projections(cfg, gen, device, out)

    B, Tq, Tk, Hi, d = cfg["B"], cfg["Tq"], cfg["Tk"], cfg["Hi"], cfg["d"]
    H, kd, vd = cfg["H"], cfg["kd"], cfg["vd"]
    f32 = cfg["dtype"] == "f32"
    # query positions: causal prefill queries sit at 0..Tq-1 (Tq == Tk);
    # decode queries sit at the last position Tk-1.
    if cfg.get("causal"):
        q_pos = torch.arange(Tq, dtype=torch.int32, device=device).repeat(B, 1)
    else:
        q_pos = torch.full((B, Tq), Tk - 1, dtype=torch.int32, device=device)
    out["q_pos"] = q_pos
    out["pad"] = torch.zeros(B, dtype=torch.int32, device=device)

    # --- indexer inputs
    if variant == "tie":
        qi = _ints((B, Tq, Hi, d), -1, 2, gen, device)
        ki = _ints((B, Tk, d), -1, 2, gen, device)
        w = _ints((B, Tq, Hi), 1, 3, gen, device) * 0.5
    else:
        std_i = 1.0 if f32 else 1.0 / math.sqrt(d)
        qi = _randn((B, Tq, Hi, d), gen, device, std_i)
        ki = _randn((B, Tk, d), gen, device, std_i)
        w = _rand((B, Tq, Hi), gen, device)
    out["w"] = w
    out["scale_idx"] = 1.0 / math.sqrt(d)
    if f32:
        out["q_idx"], out["k_idx"], out["k_scale"] = qi, ki, None
    else:
        out["q_idx"] = to_bf16(qi)
        if cfg.get("fp8_keys"):
            out["k_idx"], out["k_scale"] = quantize_fp8_rows(ki)
        else:
            out["k_idx"], out["k_scale"] = to_bf16(ki), None
    del qi, ki

    # --- attention inputs
    out["scale_attn"] = 1.0 / math.sqrt(kd)
    qmul = 16.0 if variant == "sharp" else 1.0
    if f32:
        out["q"] = _randn((B, Tq, H, kd), gen, device) * qmul
        out["K"] = _randn((B, Tk, H, kd), gen, device)
        out["V"] = _randn((B, Tk, H, vd), gen, device)
        out["K1"] = _randn((B, Tk, 1, kd), gen, device)
        out["V1"] = _randn((B, Tk, 1, vd), gen, device)
    else:
        out["q"] = to_bf16(_randn((B, Tq, H, kd), gen, device, qmul / math.sqrt(kd)))
        # absorbed MLA: one latent row of kd per key; V is its first vd columns
        out["KV"] = to_bf16(_randn((B, Tk, kd), gen, device, 1.0 / math.sqrt(kd)))
    if cfg.get("fp8_keys") and not f32:
        # the decode token's own indexer key, to be rotated and appended to
        # the fp8 key cache (k_idx) at its last row; drawn last so that every
        # other tensor keeps its values
        out["k_new"] = to_bf16(_randn((B, 1, d), gen, device, 1.0 / math.sqrt(d)))
    return out


def _make_pooled(cfg, gen, device, variant, out):
    B, L, d, Hi = cfg["B"], cfg["L"], cfg["d"], cfg["Hi"]
    H, kd, vd = cfg["H"], cfg["kd"], cfg["vd"]
    pads = list(cfg["pads"])[:B]
    while len(pads) < B:
        pads.append(0)
    out["pad"] = torch.tensor(pads, dtype=torch.int32, device=device)
    last = cfg.get("last_only", False)
    Tq = 1 if last else L
    if last:
        out["q_pos"] = torch.full((B, 1), L - 1, dtype=torch.int32, device=device)
    else:
        out["q_pos"] = torch.arange(L, dtype=torch.int32, device=device).repeat(B, 1)
    out["Tq"] = Tq
    if variant == "tie":
        out["k_idx"] = to_bf16(_ints((B, L, d), -1, 2, gen, device))
        out["gate"] = to_bf16(_ints((B, L, d), -1, 2, gen, device))
        out["q_idx"] = to_bf16(_ints((B, Tq, Hi, d), -1, 2, gen, device))
        out["w"] = _ints((B, Tq, Hi), 1, 3, gen, device) * 0.5
    else:
        out["k_idx"] = to_bf16(_randn((B, L, d), gen, device, 1.0 / math.sqrt(d)))
        out["gate"] = to_bf16(_randn((B, L, d), gen, device))
        out["q_idx"] = to_bf16(_randn((B, Tq, Hi, d), gen, device, 1.0 / math.sqrt(d)))
        out["w"] = _rand((B, Tq, Hi), gen, device)
    out["scale_idx"] = 1.0 / math.sqrt(d)
    out["scale_attn"] = 1.0 / math.sqrt(kd)
    qmul = 16.0 if variant == "sharp" else 1.0
    out["q"] = to_bf16(_randn((B, Tq, H, kd), gen, device, qmul / math.sqrt(kd)))
    out["K"] = to_bf16(_randn((B, L, H, kd), gen, device, 1.0 / math.sqrt(kd)))
    out["V"] = to_bf16(_randn((B, L, H, vd), gen, device, 1.0 / math.sqrt(vd)))
    return out


def _make_projections(cfg, gen, device, out):
    B, L = cfg["B"], cfg["L"]
    T = B * L
    r_q, hid, Hi, d = cfg["q_lora_rank"], cfg["hidden"], cfg["Hi"], cfg["d"]
    rank, H, kd, vd = cfg["rank"], cfg["H"], cfg["kd"], cfg["vd"]
    out["T"] = T
    out["pos"] = torch.arange(L, dtype=torch.int32, device=device).repeat(B)
    out["q_lora"] = to_bf16(_randn((T, r_q), gen, device))
    out["x"] = to_bf16(_randn((T, hid), gen, device))
    out["wq_b"] = to_bf16(_randn((Hi * d, r_q), gen, device, 1.0 / math.sqrt(r_q)))
    out["wk"] = to_bf16(_randn((d, hid), gen, device, 1.0 / math.sqrt(hid)))
    out["w_proj"] = to_bf16(_randn((Hi, hid), gen, device, 1.0 / math.sqrt(hid)))
    out["k_norm_w"] = 1.0 + _randn((d,), gen, device, 0.1)
    out["k_norm_b"] = _randn((d,), gen, device, 0.1)
    out["latent"] = to_bf16(_randn((T, rank), gen, device))
    out["w_kv_b"] = to_bf16(_randn((H * (kd + vd), rank), gen, device, 1.0 / math.sqrt(rank)))
    return out
