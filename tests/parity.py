"""Shared checks for the GPU-vs-oracle parity tests (not collected).

Criteria (stated per stage):
  * index scores: |S_gpu - S_ref| <= rtol * |S_ref| on every visible
    element (rtol = 1e-3 for bf16 inputs, 1e-5 for f32 inputs), except where
    S_ref is cancellation-dominated.  That is where the kernel's own
    worst-case rounding bound gamma * A exceeds rtol * |S_ref|, with
    A = sum_h |w| |scale| sum_c |q_c k_c| and gamma = (d + heads + 4) * unit:
    unit = 2^-23 for the f32 sums of exact bf16 products, 2^-52 for the f64
    sums of the f32-input kernel (any summation order, any rounding with a
    relative error of at most unit per operation).  There |S_gpu - S_ref| <=
    gamma * A is required instead, and the count of such elements is
    reported.  Invisible scores must be exactly -FLT_MAX on both sides.
  * top-k / pool select: bit-exact against the oracle applied to the GPU's
    own scores.
  * attention (given the oracle's selection): per query row over all heads x
    vd, max|d| <= 2e-3 * ||out_ref||_inf and cosine >= 0.9999 for bf16;
    max|d| <= 1e-5 * ||out_ref||_inf for f32.  lse within 1e-4 (bf16) /
    1e-5 (f32) absolute.
  * pool keys: within one bf16 ulp of the f64 value.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

FLT_MAX = float(np.finfo(np.float32).max)


def note(msg: str):
    """Print and flush a progress line (names the case before GPU work)."""
    print(msg, flush=True)
    sys.stdout.flush()


def check_scores(S_gpu: np.ndarray, S_ref: np.ndarray, A: np.ndarray, rtol: float, what="",
                 d: int = 128, heads: int = 64):
    """Relative check of the index scores (see the module docstring).

    Returns (worst error / allowed error, cancellation-dominated count,
    visible count)."""
    S_gpu = np.asarray(S_gpu, np.float64)
    S_ref = np.asarray(S_ref, np.float64)
    inv_ref = S_ref == -FLT_MAX
    inv_gpu = S_gpu == -FLT_MAX
    assert np.array_equal(inv_ref, inv_gpu), f"{what}: visibility pattern differs"
    vis = ~inv_ref
    if not vis.any():
        return 0.0, 0, 0
    unit = 2.0 ** -52 if rtol <= 1e-5 else 2.0 ** -23
    gamma = (d + heads + 4) * unit
    err = np.abs(S_gpu[vis] - S_ref[vis])
    rel_bound = rtol * np.abs(S_ref[vis])
    rnd_bound = gamma * np.asarray(A, np.float64)[vis]
    dominated = rnd_bound > rel_bound
    bound = np.where(dominated, rnd_bound, rel_bound)
    ok = err <= bound
    if not ok.all():
        i = int(np.argmax(~ok))
        raise AssertionError(
            f"{what}: {int((~ok).sum())} of {err.size} visible scores out of tolerance; first: "
            f"|d| {err[i]:.3g} vs {'gamma*A' if dominated[i] else 'rtol*|S|'} {bound[i]:.3g} "
            f"(S_ref {S_ref[vis][i]:.6g}, rtol {rtol}, gamma {gamma:.3g})")
    ratio = np.where(bound > 0, err / np.where(bound > 0, bound, 1.0), 0.0)
    n_dom = int(dominated.sum())
    note(f"  {what}: worst {float(ratio.max()):.3g} of the allowed error; "
         f"{n_dom} of {err.size} visible scores cancellation-dominated")
    return float(ratio.max()), n_dom, int(err.size)


def check_attend(out_gpu, out_ref, lse_gpu, lse_ref, bf16: bool, what=""):
    """out_*: [rows, H, vd]; lse_*: [rows, H]."""
    og = np.asarray(out_gpu, np.float64).reshape(out_ref.shape[0], -1)
    orf = np.asarray(out_ref, np.float64).reshape(out_ref.shape[0], -1)
    worst_ratio, worst_cos = 0.0, 1.0
    for r in range(orf.shape[0]):
        ninf = np.abs(orf[r]).max()
        d = np.abs(og[r] - orf[r]).max()
        if ninf == 0.0:
            assert d == 0.0, f"{what}: row {r} should be all zero"
            continue
        ratio = d / ninf
        worst_ratio = max(worst_ratio, ratio)
        if bf16:
            cos = float((og[r] * orf[r]).sum() /
                        np.sqrt((og[r] ** 2).sum() * (orf[r] ** 2).sum()))
            worst_cos = min(worst_cos, cos)
    lim = 2e-3 if bf16 else 1e-5
    assert worst_ratio <= lim, f"{what}: max|d| = {worst_ratio:.3g} x ||out||_inf > {lim}"
    if bf16:
        assert worst_cos >= 0.9999, f"{what}: cosine {worst_cos:.7f} < 0.9999"
    lg = np.asarray(lse_gpu, np.float64)
    lr = np.asarray(lse_ref, np.float64)
    assert np.array_equal(np.isneginf(lg), np.isneginf(lr)), f"{what}: empty-set pattern differs"
    fin = np.isfinite(lr)
    if fin.any():
        tol = 1e-4 if bf16 else 1e-5
        e = float(np.abs(lg[fin] - lr[fin]).max())
        assert e <= tol, f"{what}: lse error {e:.3g} > {tol}"
    return worst_ratio, worst_cos


def bf16_ulp_ok(got_bf16: torch.Tensor, ref_f64: np.ndarray, mag=None, what=""):
    """Each bf16 value must be within one bf16 ulp of the f64 reference, plus
    (when `mag`, the magnitude sum of the terms, is given) the f32 rounding
    of a sum of that magnitude -- which dominates where the terms cancel."""
    g = got_bf16.float().double().cpu().numpy()
    r = np.asarray(ref_f64, np.float64)
    # ulp of the reference at its binade (bf16 has 8 significant bits)
    tiny = np.finfo(np.float32).tiny
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(r), tiny))) - 7)
    err = np.abs(g - r)
    bound = ulp + (0.0 if mag is None else 2.0 ** -20 * np.asarray(mag, np.float64))
    ratio = err / bound
    worst = float(ratio.max()) if err.size else 0.0
    if worst > 1.0:
        i = np.unravel_index(np.argmax(ratio), ratio.shape)
        raise AssertionError(f"{what}: {worst:.3g} x bound at {i}: got {g[i]!r} ref {r[i]!r} "
                             f"mag {None if mag is None else mag[i]!r}")
    return worst


def cpu(t):
    return t.detach().cpu()
