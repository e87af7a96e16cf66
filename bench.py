"""Benchmark of the DSA layer step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config 2] [--no-cpu]

One step = the whole hot path over one batch of synthetic inputs already
resident in HBM: lightning-indexer scores -> per-query top-k -> sparse MLA
attention (for the pooled configuration: pool keys -> pooled scores -> pool
select -> per-head attention).  Prints one JSON line with the throughput in
query tokens/s, the roofline of the dominant kernel (timed live with HIP
events on the stream the kernels run on), and the CPU oracle timed on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s

METRIC = "DSA layer tokens/s on 1 MI355X; indexer MFMA % and attend HBM GB/s of peak"

WORKLOAD_TEXT = {
    1: "tiny fp32 layer: 1 x 64 causal queries over 64 keys; indexer 4 heads x 32, top_k 8; "
       "attention 4 heads, kd 48, vd 32, per-head K/V",
    2: "decode: 32 sequences x 1 query over 8192 keys; indexer 32 heads x 128 bf16, "
       "top_k 2048; absorbed MLA 64 heads over shared 576-wide latent rows, vd 512",
    3: "causal prefill: 1 sequence x 4096 queries over 4096 keys; indexer 32 heads x 128 bf16, "
       "top_k 2048; absorbed MLA 64 heads, kd 576, vd 512",
    4: "long-context decode: 8 sequences x 1 query over 131072 keys; fp8-e4m3 indexer keys "
       "with per-row scales, 32 heads x 128, top_k 2048; absorbed MLA 64 heads, kd 576, vd 512",
    5: "pooled NoPE: 4 sequences x 16384 tokens (left pads 0, 2, 37, 64), all positions are "
       "queries; kpool 4 softmax-pooled indexer keys, 32 heads x 128; top 512 pools + visible "
       "tail (out_width 2052); per-head attention 64 heads, kd 192, vd 256",
}


# short workload names (file names under profiles/)
WORKLOAD_NAME = {1: "tiny_fp32_64", 2: "decode_b32x8192", 3: "prefill_4096",
                 4: "decode_b8x131072_fp8", 5: "pooled_b4x16384"}

# the kernels each ABI call of a stage launches (substrings of their names)
STAGE_KERNELS = {
    "index": ("index_scores",),
    "topk": ("topk_seg_kernel", "topk_chunk_kernel", "topk_merge_kernel",
             "topk_merge_seg_kernel"),
    "attend": ("attend_gather_kernel", "attend_combine_kernel", "topk_to_mask_kernel",
               "attend_masked_kernel", "attend_plain_kernel"),
    "pool_keys": ("pool_keys_kernel", "pool_counts_kernel"),
    "pool_select": ("pool_select_kernel",),
}


def measured_traffic(cfg, stage):
    """HBM bytes per call of `stage` from the rocprofv3 counter record under
    profiles/, or None when there is none or the kernel sources changed
    since it was taken."""
    from sparse_attention_scores_amd import profile_summary as ps
    path = os.path.join(ROOT, "profiles", f"dsa_step_{WORKLOAD_NAME[cfg]}_hbm_traffic.txt")
    if not os.path.exists(path):
        return None, None
    digest, ff, wf, kern = ps.read_traffic(path)
    if digest != ps.source_digest() or ff is None or wf is None:
        return None, os.path.relpath(path, ROOT)
    tot, hit = 0.0, False
    for name, (f, w) in kern.items():
        if any(pat in name for pat in STAGE_KERNELS[stage]):
            tot += f * 1024.0 * ff + w * 1024.0 * wf
            hit = True
    return (round(tot) if hit else None), os.path.relpath(path, ROOT)


def copy_probe(mib):
    """A plain streaming kernel of known traffic (y = -x over float32, `mib`
    MiB each way): its counter readings calibrate FETCH_SIZE / WRITE_SIZE."""
    import torch
    n = mib * (1 << 20) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(3):
        torch.neg(x, out=y)
    torch.cuda.synchronize()
    return n * 4


def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=2, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-rows", type=int, default=64, help="query rows in the oracle sample")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="also run a plain copy kernel of MIB MiB (counter calibration)")
    ap.add_argument("--graph", action="store_true",
                    help="replay one captured HIP graph per timed step instead of launching "
                         "the step's kernels one by one")
    return ap.parse_args()


class Step:
    """Preallocated buffers and the three ABI calls of one layer step."""

    def __init__(self, dsa, inp):
        import torch
        self.dsa, self.inp = dsa, inp
        self.lo, self.hi = dsa.visibility_ranges(inp["pad"], inp["q_pos"])
        B, Tq, Tk = inp["B"], inp["Tq"], inp["Tk"]
        dev = inp["q_pos"].device
        self.k = inp["top_k"]
        self.S = torch.empty((B, Tq, Tk), dtype=torch.float32, device=dev)
        self.idx = torch.empty((B, Tq, self.k), dtype=torch.int32, device=dev)
        self.f32 = inp["dtype"] == "f32"
        H, vd = inp["H"], inp["vd"]
        self.out = torch.empty((B, Tq, H, vd), dtype=torch.float32, device=dev)
        self.lse = torch.empty((B, Tq, H), dtype=torch.float32, device=dev)
        nt = dsa.topk_workspace_size(B * Tq, Tk, self.k)
        self.ws_topk = torch.empty(max(nt, 1), dtype=torch.uint8, device=dev)
        if self.f32:
            self.K, self.V, self.kvh = inp["K"], inp["V"], H
            self.ws_attn = None
        else:
            self.K, self.V, self.kvh = inp["KV"], None, 1
            dims = dsa._AttnDims(B, Tq, Tk, H, inp["kd"], vd, 1, self.k, inp["scale_attn"])
            na = dsa.sparse_attend_workspace_size(dims)
            self.ws_attn = torch.empty(max(na, 1), dtype=torch.uint8, device=dev)

    def index(self):
        i = self.inp
        self.dsa.index_scores(i["q_idx"], i["k_idx"], i["w"], self.lo, self.hi, i["scale_idx"],
                              k_scale=i["k_scale"], out=self.S)

    def topk(self):
        self.dsa.topk(self.S, self.lo, self.hi, self.k, out=self.idx, workspace=self.ws_topk)

    def attend(self):
        i = self.inp
        self.dsa.sparse_attend(i["q"], self.K, self.V, self.idx, i["scale_attn"], self.kvh,
                               vd=i["vd"], vis_lo=self.lo, vis_hi=self.hi, out=self.out,
                               lse=self.lse, workspace=self.ws_attn)

    stages = ("index", "topk", "attend")


class PooledStep:
    """The pooled NoPE step: pool keys -> pooled index scores -> pool select
    -> per-head attention over the selected tokens."""

    stages = ("pool_keys", "index", "pool_select", "attend")

    def __init__(self, dsa, inp):
        import torch
        self.dsa, self.inp = dsa, inp
        B, L, d, kp = inp["B"], inp["L"], inp["d"], inp["kpool"]
        dev = inp["q_pos"].device
        self.kp, self.sk, self.width = kp, inp["select_k"], inp["out_width"]
        self.plo, self.phi = dsa.visibility_ranges(inp["pad"], inp["q_pos"], kp)
        self.lo, self.hi = dsa.visibility_ranges(inp["pad"], inp["q_pos"])
        self.pk = torch.empty((B, L // kp, d), dtype=torch.bfloat16, device=dev)
        self.npools = torch.empty(B, dtype=torch.int32, device=dev)
        self.S = torch.empty((B, L, L // kp), dtype=torch.float32, device=dev)
        self.tok = torch.empty((B, L, self.width), dtype=torch.int32, device=dev)
        H, vd = inp["H"], inp["vd"]
        self.out = torch.empty((B, L, H, vd), dtype=torch.float32, device=dev)
        self.lse = torch.empty((B, L, H), dtype=torch.float32, device=dev)
        dims = dsa._AttnDims(B, L, L, H, inp["kd"], vd, H, self.width, inp["scale_attn"])
        self.ws_attn = torch.empty(max(dsa.sparse_attend_workspace_size(dims), 1),
                                   dtype=torch.uint8, device=dev)

    def pool_keys(self):
        i = self.inp
        self.dsa.pool_keys(i["k_idx"], i["gate"], i["pad"], self.kp, out=self.pk,
                           n_pools=self.npools)

    def index(self):
        i = self.inp
        self.dsa.index_scores(i["q_idx"], self.pk, i["w"], self.plo, self.phi, i["scale_idx"],
                              out=self.S)

    def pool_select(self):
        i = self.inp
        self.dsa.pool_select(self.S, i["pad"], i["q_pos"], self.kp, self.sk, self.width,
                             out_tok=self.tok)

    def attend(self):
        i = self.inp
        self.dsa.sparse_attend(i["q"], i["K"], i["V"], self.tok, i["scale_attn"], i["H"],
                               vis_lo=self.lo, vis_hi=self.hi, out=self.out, lse=self.lse,
                               workspace=self.ws_attn)


def pooled_work(inp):
    """Algorithmic bytes/flops of the pooled step (visible pool pairs and
    selected tokens only)."""
    B, L, d, Hi, kp = inp["B"], inp["L"], inp["d"], inp["Hi"], inp["kpool"]
    H, kd, vd, sk, width = inp["H"], inp["kd"], inp["vd"], inp["select_k"], inp["out_width"]
    pads = [int(p) for p in inp["pad"].cpu().tolist()]
    vis_pairs = sel_pairs = queries = 0
    for p in pads:
        for t in range(p, L):
            n_full = (t - p + 1) // kp
            vis_pairs += n_full
            sel_pairs += min(sk, n_full) * kp + (t + 1 - (p + n_full * kp))
            queries += 1
    np_ = L // kp
    pk_bytes = 2 * B * L * d * 2 + B * np_ * d * 2
    idx_bytes = B * L * Hi * d * 2 + B * np_ * d * 2 + B * L * Hi * 4 + vis_pairs * 4
    sel_bytes = vis_pairs * 4 + B * L * width * 4
    att_bytes = (B * L * H * (kd + kd + vd) * 2 + B * L * width * 4 + B * L * H * (vd + 1) * 4)
    return {"pool_keys": (pk_bytes, 0), "index": (idx_bytes, 2 * Hi * d * vis_pairs),
            "pool_select": (sel_bytes, 0),
            "attend": (att_bytes, 2 * H * (kd + vd) * sel_pairs)}, queries


def algorithmic_work(inp):
    """Bytes the method must move and flops it must do, per stage: only
    visible pairs and selected keys count, not the dense work the method
    avoids.  Index: the keys once, the queries and head weights, one f32 score
    per visible pair.  Top-k: the visible scores and the selected indices.
    Attend: the selected latent rows once (prefill: the distinct rows once),
    the queries, the indices and the f32 output and lse."""
    B, Tq, Tk, Hi, d = inp["B"], inp["Tq"], inp["Tk"], inp["Hi"], inp["d"]
    H, kd, vd, k = inp["H"], inp["kd"], inp["vd"], inp["top_k"]
    f32 = inp["dtype"] == "f32"
    eb = 4 if f32 else 2
    kb = 1 if inp.get("fp8_keys") else eb
    if inp.get("causal"):
        vis_pairs = B * Tq * (Tq + 1) // 2
        sel_pairs = B * sum(min(t + 1, k) for t in range(Tq))
    else:
        vis_pairs = B * Tq * Tk
        sel_pairs = B * Tq * min(k, Tk)
    idx_bytes = (B * Tk * d * kb + (B * Tk * 4 if inp.get("fp8_keys") else 0)
                 + B * Tq * Hi * d * eb + B * Tq * Hi * 4 + vis_pairs * 4)
    idx_flops = 2 * Hi * d * vis_pairs
    topk_bytes = vis_pairs * 4 + B * Tq * k * 4
    row_bytes = (kd * eb) if not f32 else (kd + vd) * eb * H  # f32 config: per-head K and V rows
    if inp.get("causal") and not f32:
        # the selected rows are re-read from cache; the method's own HBM bytes
        # are the distinct rows once
        gather = B * Tk * kd * eb
    else:
        gather = sel_pairs * row_bytes
    att_bytes = gather + B * Tq * H * kd * eb + B * Tq * k * 4 + B * Tq * H * (vd + 1) * 4
    att_flops = 2 * H * (kd + vd) * sel_pairs
    return {"index": (idx_bytes, idx_flops), "topk": (topk_bytes, 0),
            "attend": (att_bytes, att_flops)}


def capture_step(torch, run_once):
    """One step of kernels captured as a HIP graph (torch.cuda.CUDAGraph is
    hipGraph on ROCm).  The step only launches kernels on the current stream
    into preallocated buffers: no allocation, memset or synchronisation is
    recorded."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run_once()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run_once()
    torch.cuda.synchronize()
    return g


def cpu_baseline(cfg, rows_wanted, min_seconds=10.0, max_passes=20):
    """The oracle (as it stands) on a bounded sample of the same workload:
    up to `rows_wanted` query rows through index scores -> top-k ->
    attention, repeated until about `min_seconds` of CPU work."""
    import numpy as np

    import oracle
    from sparse_attention_scores_amd import workloads as W
    inp = W.make(cfg, device="cpu")
    B, Tq = inp["B"], inp["Tq"]
    rows = np.linspace(0, B * Tq - 1, num=min(rows_wanted, B * Tq)).round().astype(np.int64)
    rows = np.unique(rows)
    qp_all = inp["q_pos"].numpy().reshape(-1)
    pd_all = np.repeat(inp["pad"].numpy(), Tq)

    def one_pass():
        S = oracle.index_scores(inp["q_idx"], inp["k_idx"], inp["w"], inp["scale_idx"],
                                inp["q_pos"], inp["pad"], k_scale=inp["k_scale"], rows=rows)
        sel = oracle.topk(S, qp_all[rows], pd_all[rows], inp["top_k"])
        idx = np.full((B * Tq, inp["top_k"]), -1, np.int32)
        idx[rows] = sel
        idx = idx.reshape(B, Tq, -1)
        if inp["dtype"] == "f32":
            oracle.sparse_attend(inp["q"], inp["K"], inp["V"], idx, inp["scale_attn"], inp["H"],
                                 q_pos=inp["q_pos"], pad=inp["pad"], rows=rows)
        else:
            oracle.sparse_attend(inp["q"], inp["KV"], None, idx, inp["scale_attn"], 1,
                                 q_pos=inp["q_pos"], pad=inp["pad"], rows=rows,
                                 k_row_stride=inp["kd"], vd=inp["vd"])

    passes = 0
    t0 = time.perf_counter()
    while True:
        one_pass()
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or passes >= max_passes:
            break
    return {"value": round(len(rows) * passes / dt, 3), "unit": "tokens/s",
            "cores": oracle.threads(), "kind": "oracle",
            "sample": f"{len(rows)} of {B * Tq} query rows of the same workload, full step "
                      f"(index scores over all keys, top-k, attention), {passes} pass(es) in "
                      f"{dt:.1f} s"}


def main():
    args = _parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: the layer step here has no "
              "multi-GPU path (the design notes say how it would shard)", file=sys.stderr)
        sys.exit(2)
    import torch

    from sparse_attention_scores_amd import binding as dsa
    from sparse_attention_scores_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dsa.load()
    cfg = args.config
    print(f"[bench] config {cfg}: generating inputs", file=sys.stderr, flush=True)
    inp = W.make(cfg, device="cuda")
    step = PooledStep(dsa, inp) if cfg == 5 else Step(dsa, inp)
    names = type(step).stages
    stages = [getattr(step, s) for s in names]

    def run_once():
        for f in stages:
            f()

    for _ in range(args.warmup):
        run_once()
    torch.cuda.synchronize()
    K = args.steps
    # Whole-step timing: K steps launched back to back (or K replays of one
    # captured HIP graph per step), nothing recorded between them.  An event
    # recorded between two kernels holds the second back until the first has
    # fully drained, so per-stage events inside this loop would add their own
    # gaps to the step.
    graph = None
    if args.graph:
        graph = capture_step(torch, run_once)
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
    print(f"[bench] warmup {args.warmup} done; timing {K} steps "
          f"({'eager' if graph is None else 'graph replay'})", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(K):
        if graph is None:
            run_once()
        else:
            graph.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # Per-stage timing: K back-to-back launches of each stage on the step's
    # own buffers, bracketed by two HIP events on the stream the kernels run
    # on; the average launch duration feeds the stage breakdown and the
    # roofline.
    stage_ms = {}
    for name, f in zip(names, stages):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(K):
            f()
        e1.record()
        torch.cuda.synchronize()
        stage_ms[name] = e0.elapsed_time(e1) / K
    if cfg == 5:
        work, tokens = pooled_work(inp)
    else:
        work, tokens = algorithmic_work(inp), inp["B"] * inp["Tq"]
    ms_per_step = wall * 1e3 / K
    per_stage = {}
    for name in names:
        by, fl = work[name]
        t = stage_ms[name] * 1e-3
        per_stage[name] = {"ms": round(stage_ms[name], 5),
                           "alg_GBps": round(by / t / 1e9, 1),
                           "alg_TFLOPs": round(fl / t / 1e12, 2)}
    dom = max(names, key=lambda n: stage_ms[n])
    by, fl = work[dom]
    t = stage_ms[dom] * 1e-3
    hbm_bound = cfg in (1, 2, 4) or dom in ("topk", "pool_select", "pool_keys")
    if hbm_bound:
        ach = by / t / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4)}
    else:
        ach = fl / t / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": MFMA_BF16_PEAK_TFS,
                "unit": "TFLOP/s", "frac": round(ach / MFMA_BF16_PEAK_TFS, 4)}
    traffic, tsrc = measured_traffic(cfg, dom)
    roof["traffic"] = traffic
    roof["traffic_record"] = tsrc
    roof["kernel"] = dom
    roof["kernels"] = list(STAGE_KERNELS[dom])
    roof["ms_per_launch"] = round(stage_ms[dom], 5)
    roof["alg_bytes_per_launch"] = by
    roof["alg_flops_per_launch"] = fl
    result = {
        "metric": METRIC,
        "value": round(tokens * K / wall, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if inp["dtype"] == "f32" else "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD_TEXT[cfg], "config_id": cfg,
                   "query_tokens_per_step": tokens, "seed": inp["seed"],
                   "launch": "eager" if graph is None else "hip graph per step"},
        "roofline": roof,
        "stages": per_stage,
    }
    if args.copy_probe:
        copy_probe(args.copy_probe)
    if not args.no_cpu and cfg != 5:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(cfg, args.cpu_rows)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
