"""Benchmark of the DSA layer step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config 5] [--only] [--no-cpu]

One step = the whole hot path over one batch of synthetic inputs already
resident in HBM.  The headline workload is the pooled NoPE configuration
(4 x 16384 tokens, every position a query): pool keys -> pooled index scores
-> pool select -> per-head attention over the selected tokens.  The other
workloads (decode 32 x 8192, prefill 4096, long decode 8 x 131072 with fp8
indexer keys: index scores -> top-k -> absorbed sparse MLA attention) follow
in "configs".

Prints one JSON line:
  * value: query tokens/s of the headline workload (wall clock over K steps);
  * roofline: the dominant stage's bound, its achieved rate from HIP events
    on the stream the kernels run on, the published MI355X peak and the
    rate this GPU reaches in a plain copy / an MFMA-only loop
    (peaks_measured);
  * stages: every stage's average launch time and algorithmic rates;
  * configs: the same for the other workloads.  On the decode workloads
    the per-step footprint (~150 MB) fits the 256 MB last-level cache, so
    their inputs rotate over four seeded sets (more than 512 MB touched)
    and the cold figures are reported beside the repeated-input (hot) ones;
  * cpu_baseline: the CPU oracle on a stated sample of the headline
    workload, fed the same input bytes as the GPU.

Algorithmic work counts only what the method itself must move or compute:
visible pairs, selected keys, the inputs once and the outputs once, not the
dense work a kernel executes around them (algorithmic_work, pooled_work).
"""
from __future__ import annotations

import argparse
import ctypes
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
    6: "pooled decode: the pooled NoPE workload's 4 sequences x 16384 tokens with one query "
       "per sequence at its last position; per-head attention gathers each query's selected "
       "tokens",
    7: "projections at 65536 tokens: indexer front-end (q_lora 2048 and hidden 6144 -> 32 "
       "heads x 128 with NEOX rope 64, LayerNorm k, head weights) and expand_kv (latent 512 "
       "-> 64 heads x (192 + 256))",
}


# short workload names (file names under profiles/)
WORKLOAD_NAME = {1: "tiny_fp32_64", 2: "decode_b32x8192", 3: "prefill_4096",
                 4: "decode_b8x131072_fp8", 5: "pooled_b4x16384", 6: "pooled_decode_b4x16384",
                 7: "projections_65536"}

# the kernels each ABI call of a stage launches (substrings of their names)
STAGE_KERNELS = {
    "rotate_q": ("hadamard_rotate_kernel",),
    "cache_write": ("index_cache_write_kernel",),
    "index": ("index_scores",),
    "topk": ("topk_seg_kernel", "topk_chunk_kernel", "topk_merge_kernel",
             "topk_merge_seg_kernel", "topk_long_pairs_kernel", "topk_long_filter_kernel",
             "topk_long_merge_kernel", "topk_sink_prefix_kernel"),
    "attend": ("attend_gather_kernel", "attend_combine_kernel", "topk_to_mask_kernel",
               "v_scale_max_kernel", "v_to_f16_kernel", "attend_masked_kernel",
               "attend_heads_gather_kernel", "attend_plain_kernel"),
    "frontend": ("pj_rope_q_kernel", "pj_norm_k_kernel"),
    "expand_kv": ("pj_expand_kv_kernel",),
    "pool_keys": ("pool_keys_kernel", "pool_keys_vec_kernel", "pool_counts_kernel"),
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


PROBE_LIB = os.path.join(ROOT, "sparse_attention_scores_amd", "probe", "libdsa_probe.so")


def _probe():
    if not os.path.exists(PROBE_LIB):
        raise RuntimeError(f"{PROBE_LIB} is not built: run `python -m "
                           "sparse_attention_scores_amd.build`")
    lib = ctypes.CDLL(PROBE_LIB)
    lib.probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                               ctypes.c_void_p]
    lib.probe_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.probe_lds_stream.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                     ctypes.c_void_p]
    return lib


def _cur_stream(torch):
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


COPY_BLOCKS = 256 * 16


def copy_probe(mib):
    """The calibration copy kernel over `mib` MiB each way (its counter
    readings calibrate FETCH_SIZE / WRITE_SIZE: it moves exactly that many
    bytes in and out)."""
    import torch
    lib = _probe()
    nbytes = mib * (1 << 20)
    x = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(3):
        assert lib.probe_copy(x.data_ptr(), y.data_ptr(), nbytes, COPY_BLOCKS,
                              _cur_stream(torch)) == 0
    torch.cuda.synchronize()
    return nbytes


def measure_peaks():
    """What this GPU reaches in a plain 1 GiB streaming copy (bytes read +
    written / time) and in a loop of bf16 MFMAs with no memory traffic, each
    timed with HIP events on the current stream."""
    import torch
    lib = _probe()
    st = _cur_stream(torch)
    nbytes = 1 << 30
    x = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    t_copy = timed(lambda: lib.probe_copy(x.data_ptr(), y.data_ptr(), nbytes, COPY_BLOCKS, st), 10)
    t_torch = timed(lambda: y.copy_(x), 10)   # torch's own copy kernel, as a cross-check
    # direct-to-LDS tile streaming, one workgroup per CU: 32 tiles (1 MiB,
    # served by L2) and all 32768 tiles of the 1 GiB buffer (HBM)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    steps = 2000
    stream_bytes = 256 * steps * 29 * 1024
    lds_stream = {}
    for name, n_tiles in (("l2", 32), ("hbm", nbytes // 32768)):
        t = timed(lambda: lib.probe_lds_stream(x.data_ptr(), n_tiles, steps, sink.data_ptr(), st), 3)
        lds_stream[name] = round(stream_bytes / t / 1e9, 1)
    del x, y
    blocks, iters = 256 * 8, 4000
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    t_mfma = timed(lambda: lib.probe_mfma_bf16(blocks, iters, out.data_ptr(), st), 5)
    flops = blocks * 4 * iters * 4 * 32 * 32 * 16 * 2
    return {"hbm_copy_GBps": round(2 * nbytes / min(t_copy, t_torch) / 1e9, 1),
            "hbm_copy_probe_GBps": round(2 * nbytes / t_copy / 1e9, 1),
            "hbm_copy_torch_GBps": round(2 * nbytes / t_torch / 1e9, 1),
            "mfma_bf16_TFLOPs": round(flops / t_mfma / 1e12, 1),
            "lds_stream_from_l2_GBps": lds_stream["l2"],
            "lds_stream_from_hbm_GBps": lds_stream["hbm"],
            "how": "copy: 1 GiB read + 1 GiB written, the faster of a 16-byte-per-lane "
                   "span-per-workgroup kernel and torch's copy; "
                   "mfma: 2048 workgroups x 4 waves, each 4 independent chains of "
                   "v_mfma_f32_32x32x16_bf16, no memory traffic; "
                   "lds_stream: 256 workgroups of 8 waves, 29 one-KB direct-to-LDS loads per "
                   "32 KB tile, two tiles in flight, one barrier per tile, from 32 tiles (L2) "
                   "or 32768 (HBM)"}


def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=5, choices=[1, 2, 3, 4, 5, 6, 7],
                    help="headline workload (default: the pooled NoPE workload, the largest)")
    ap.add_argument("--only", action="store_true",
                    help="time the headline workload only (no configs object, no peaks)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-rows", type=int, default=48, help="query rows in the oracle sample")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="also run the calibration copy kernel over MIB MiB (counter "
                         "calibration)")
    ap.add_argument("--graph", action="store_true",
                    help="replay one captured HIP graph per timed step instead of launching "
                         "the step's kernels one by one")
    return ap.parse_args()


class Step:
    """Preallocated buffers and the ABI calls of one layer step: index scores,
    top-k and attention; with an fp8 indexer-key cache (the long-context
    decode workload) the step first rotates the queries and writes the new
    token's rotated key into the cache at its row (write-then-score)."""

    def __init__(self, dsa, inp):
        import torch
        self.dsa, self.inp = dsa, inp
        self.cached = inp.get("k_new") is not None
        self.stages = (("rotate_q", "cache_write") if self.cached else ()) + ("index", "topk",
                                                                              "attend")
        self.q_used = torch.empty_like(inp["q_idx"]) if self.cached else inp["q_idx"]
        if self.cached:
            B, Tk = inp["B"], inp["Tk"]
            self.kv_head = torch.full((B,), Tk - 1, dtype=torch.int32, device=inp["q_pos"].device)
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

    def rotate_q(self):
        self.dsa.hadamard_rotate(self.inp["q_idx"], out=self.q_used)

    def cache_write(self):
        i = self.inp
        self.dsa.index_cache_write(i["k_new"], self.kv_head, i["k_idx"], i["k_scale"])

    def index(self):
        i = self.inp
        self.dsa.index_scores(self.q_used, i["k_idx"], i["w"], self.lo, self.hi, i["scale_idx"],
                              k_scale=i["k_scale"], out=self.S)

    def topk(self):
        self.dsa.topk(self.S, self.lo, self.hi, self.k, out=self.idx, workspace=self.ws_topk)

    def attend(self):
        i = self.inp
        self.dsa.sparse_attend(i["q"], self.K, self.V, self.idx, i["scale_attn"], self.kvh,
                               vd=i["vd"], vis_lo=self.lo, vis_hi=self.hi, out=self.out,
                               lse=self.lse, workspace=self.ws_attn)



class PooledStep:
    """The pooled NoPE step: pool keys -> pooled index scores -> pool select
    -> per-head attention over the selected tokens."""

    stages = ("pool_keys", "index", "pool_select", "attend")

    def __init__(self, dsa, inp):
        import torch
        self.dsa, self.inp = dsa, inp
        B, L, d, kp, Tq = inp["B"], inp["L"], inp["d"], inp["kpool"], inp["Tq"]
        dev = inp["q_pos"].device
        self.kp, self.sk, self.width = kp, inp["select_k"], inp["out_width"]
        self.plo, self.phi = dsa.visibility_ranges(inp["pad"], inp["q_pos"], kp)
        self.lo, self.hi = dsa.visibility_ranges(inp["pad"], inp["q_pos"])
        self.pk = torch.empty((B, L // kp, d), dtype=torch.bfloat16, device=dev)
        self.npools = torch.empty(B, dtype=torch.int32, device=dev)
        self.S = torch.empty((B, Tq, L // kp), dtype=torch.float32, device=dev)
        self.tok = torch.empty((B, Tq, self.width), dtype=torch.int32, device=dev)
        H, vd = inp["H"], inp["vd"]
        self.out = torch.empty((B, Tq, H, vd), dtype=torch.float32, device=dev)
        self.lse = torch.empty((B, Tq, H), dtype=torch.float32, device=dev)
        dims = dsa._AttnDims(B, Tq, L, H, inp["kd"], vd, H, self.width, inp["scale_attn"])
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
    selected tokens only) for its queries (every position, or the last one
    of each sequence on decode).  Attend reads each query's vectors, the K
    and V rows of the selected tokens -- every token's rows once when the
    queries select more (query, token) pairs than there are tokens -- the
    index rows, and writes the f32 output and lse."""
    B, L, d, Hi, kp = inp["B"], inp["L"], inp["d"], inp["Hi"], inp["kpool"]
    H, kd, vd, sk, width = inp["H"], inp["kd"], inp["vd"], inp["select_k"], inp["out_width"]
    pads = [int(p) for p in inp["pad"].cpu().tolist()]
    qpos = inp["q_pos"].cpu().tolist()
    vis_pairs = sel_pairs = queries = 0
    for b, p in enumerate(pads):
        for t in qpos[b]:
            if t < p:
                continue
            n_full = (t - p + 1) // kp
            vis_pairs += n_full
            sel_pairs += min(sk, n_full) * kp + (t + 1 - (p + n_full * kp))
            queries += 1
    np_ = L // kp
    n_q = B * inp["Tq"]
    tokens = sum(L - p for p in pads)
    pk_bytes = 2 * B * L * d * 2 + B * np_ * d * 2
    idx_bytes = n_q * Hi * d * 2 + B * np_ * d * 2 + n_q * Hi * 4 + vis_pairs * 4
    sel_bytes = vis_pairs * 4 + n_q * width * 4
    kv_bytes = min(sel_pairs, tokens) * H * (kd + vd) * 2
    att_bytes = n_q * H * kd * 2 + kv_bytes + n_q * width * 4 + n_q * H * (vd + 1) * 4
    return {"pool_keys": (pk_bytes, 0), "index": (idx_bytes, 2 * Hi * d * vis_pairs),
            "pool_select": (sel_bytes, 0),
            "attend": (att_bytes, 2 * H * (kd + vd) * sel_pairs)}, queries


def projection_work(inp):
    """Algorithmic bytes/flops of the projections: each operand and output
    once; flops 2 x M x N x K of each product."""
    T, r_q, hid, Hi = inp["T"], inp["q_lora_rank"], inp["hidden"], inp["Hi"]
    rank, H, kd, vd = inp["rank"], inp["H"], inp["kd"], inp["vd"]
    fe_bytes = (T * r_q * 2 + T * hid * 2 + Hi * 128 * r_q * 2 + (128 + Hi) * hid * 2
                + T * Hi * 128 * 2 + T * 128 * 2 + T * Hi * 4 + T * 4)
    fe_flops = 2 * T * (r_q * Hi * 128 + hid * (128 + Hi))
    ex_bytes = T * rank * 2 + H * (kd + vd) * rank * 2 + T * H * (kd + vd) * 2
    ex_flops = 2 * T * rank * H * (kd + vd)
    return {"frontend": (fe_bytes, fe_flops), "expand_kv": (ex_bytes, ex_flops)}


class ProjStep:
    """The dense projections at the pooled workload's token count: the
    indexer front-end (q, k, head weights) and expand_kv (per-head K, V)."""

    stages = ("frontend", "expand_kv")

    def __init__(self, dsa, inp):
        import torch
        self.dsa, self.inp = dsa, inp
        T, Hi, H = inp["T"], inp["Hi"], inp["H"]
        dev = inp["pos"].device
        self.q = torch.empty((T, Hi, 128), dtype=torch.bfloat16, device=dev)
        self.k = torch.empty((T, 128), dtype=torch.bfloat16, device=dev)
        self.w = torch.empty((T, Hi), dtype=torch.float32, device=dev)
        self.K = torch.empty((T, H, inp["kd"]), dtype=torch.bfloat16, device=dev)
        self.V = torch.empty((T, H, inp["vd"]), dtype=torch.bfloat16, device=dev)

    def frontend(self):
        i = self.inp
        self.dsa.indexer_frontend(i["q_lora"], i["x"], i["pos"], i["wq_b"], i["wk"], i["k_norm_w"],
                                  i["k_norm_b"], i["w_proj"], i["Hi"], i["rope_dim"],
                                  i["rope_theta"], i["norm_eps"], q_out=self.q, k_out=self.k,
                                  w_out=self.w)

    def expand_kv(self):
        i = self.inp
        self.dsa.expand_kv(i["latent"], i["w_kv_b"], i["H"], i["kd"], i["vd"], k_out=self.K,
                           v_out=self.V)


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
    work = {"index": (idx_bytes, idx_flops), "topk": (topk_bytes, 0),
            "attend": (att_bytes, att_flops)}
    if inp.get("k_new") is not None:
        # rotation: the queries read and written once (bf16); cache write: the
        # new key read (bf16), its fp8 row and scale written; d log2 d flops
        # per row of the butterflies
        lg = max(d.bit_length() - 1, 1)
        work["rotate_q"] = (2 * B * Tq * Hi * d * 2, B * Tq * Hi * d * lg)
        work["cache_write"] = (B * d * 2 + B * (d + 4), B * d * lg)
    return work


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


# Seeded input sets per workload: the decode workloads rotate over four so
# that a step's inputs are not left in the last-level cache by the previous
# step (about 150 MB touched per step against 256 MB of cache).
ROTATE_SETS = {2: 4, 4: 4}


def executed_masked_flops(inp, qblock=32, tile=32):
    """Flops the per-head masked-tile kernel executes: every (query, key)
    pair of the key tiles each wave's 32 queries compute (from the block's
    first visible tile to the wave's last query; a wave skips the tiles in
    which none of its queries selects a key), whether selected or not."""
    B, L, H, kd, vd = inp["B"], inp["L"], inp["H"], inp["kd"], inp["vd"]
    pads = [int(p) for p in inp["pad"].cpu().tolist()]
    pairs = 0
    for p in pads:
        for q0 in range(0, L, qblock):
            q1 = min(q0 + qblock, L)
            if q1 <= p:
                continue
            lo, hi = p, q1          # keys [pad, last query + 1)
            t0, t1 = lo // tile, (hi + tile - 1) // tile
            pairs += (q1 - q0) * (t1 - t0) * tile
    return 2 * H * (kd + vd) * pairs


def _rates(by, fl, t):
    return {"alg_GBps": round(by / t / 1e9, 1), "alg_TFLOPs": round(fl / t / 1e12, 2)}


def stage_bound(cfg, stage):
    """The roofline that bounds each stage of each workload: the decode
    workloads and the selection stages stream memory; the prefill and
    pooled indexers and attends are contractions."""
    if stage in ("topk", "pool_select", "pool_keys") or cfg in (1, 2, 4, 6):
        return "hbm"
    return "mfma"


def run_workload(cfg, dsa, W, K, warmup, graph=False):
    """Times one workload: whole steps by wall clock, then each stage by HIP
    events; on the rotating workloads also with the inputs cycling over
    several seeded sets (cold) besides one set repeated (hot)."""
    import torch
    n_sets = ROTATE_SETS.get(cfg, 1)
    sets = []
    for i in range(n_sets):
        inp = W.make(cfg, device="cuda", seed=1000 + cfg + 7919 * i)
        sets.append(PooledStep(dsa, inp) if cfg in (5, 6)
                    else ProjStep(dsa, inp) if cfg == 7 else Step(dsa, inp))
    names = sets[0].stages

    def run_once(st):
        for n in names:
            getattr(st, n)()

    for _ in range(warmup):
        for st in sets:
            run_once(st)
    torch.cuda.synchronize()
    g = None
    if graph:
        g = capture_step(torch, lambda: run_once(sets[0]))
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
    print(f"[bench] config {cfg}: warmup done; timing {K} steps "
          f"({'graph replay' if g else 'eager'}, {n_sets} input set(s))", file=sys.stderr,
          flush=True)

    def wall(rotate):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(K):
            if g is not None:
                g.replay()
            else:
                run_once(sets[s % n_sets] if rotate else sets[0])
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    def stage_time(name, rotate):
        # K launches of the stage alone between two HIP events on the stream
        # the kernels run on (torch's current stream, which the binding uses)
        fns = [getattr(st, name) for st in (sets if rotate else sets[:1])]
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for s in range(K):
            fns[s % len(fns)]()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / K

    inp = sets[0].inp
    if cfg in (5, 6):
        work, tokens = pooled_work(inp)
    elif cfg == 7:
        work, tokens = projection_work(inp), inp["T"]
    else:
        work, tokens = algorithmic_work(inp), inp["B"] * inp["Tq"]
    res = {"workload": WORKLOAD_TEXT[cfg], "config_id": cfg, "query_tokens_per_step": tokens,
           "seed": inp["seed"], "launch": "hip graph per step" if g else "eager"}
    t_hot = wall(False)
    res["value"] = round(tokens * K / t_hot, 1)
    res["ms_per_step"] = round(t_hot * 1e3 / K, 5)
    if n_sets > 1:
        t_cold = wall(True)
        res["value_cold"] = round(tokens * K / t_cold, 1)
        res["ms_per_step_cold"] = round(t_cold * 1e3 / K, 5)
        res["input_sets"] = n_sets
    stages = {}
    for name in names:
        by, fl = work[name]
        ms = stage_time(name, False)
        st = {"ms": round(ms, 5), "bound": stage_bound(cfg, name), **_rates(by, fl, ms * 1e-3)}
        if n_sets > 1:
            ms_c = stage_time(name, True)
            st["ms_cold"] = round(ms_c, 5)
            st.update({k + "_cold": v for k, v in _rates(by, fl, ms_c * 1e-3).items()})
        stages[name] = st
    res["stages"] = stages
    res["_work"] = work
    res["_inp"] = inp
    res["_sets"] = sets
    return res


def roofline_of(cfg, res, peaks):
    """The dominant stage's roofline: its bound, achieved algorithmic rate
    (cold inputs where they rotate), the published peak, the measured
    peak and the recorded counter traffic."""
    stages = res["stages"]
    dom = max(stages, key=lambda n: stages[n].get("ms_cold", stages[n]["ms"]))
    st = stages[dom]
    by, fl = res["_work"][dom]
    ms = st.get("ms_cold", st["ms"])
    t = ms * 1e-3
    if st["bound"] == "hbm":
        ach = by / t / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4)}
        if "ms_cold" in st:
            roof["frac_hot"] = round(by / (st["ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
        if peaks:
            roof["peak_measured"] = peaks["hbm_copy_GBps"]
            roof["frac_of_measured"] = round(ach / peaks["hbm_copy_GBps"], 4)
    else:
        ach = fl / t / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": MFMA_BF16_PEAK_TFS,
                "unit": "TFLOP/s", "frac": round(ach / MFMA_BF16_PEAK_TFS, 4)}
        if peaks:
            roof["peak_measured"] = peaks["mfma_bf16_TFLOPs"]
            roof["frac_of_measured"] = round(ach / peaks["mfma_bf16_TFLOPs"], 4)
        if cfg == 5 and dom == "attend":
            ex = executed_masked_flops(res["_inp"])
            roof["executed_flops_per_launch"] = ex
            roof["executed_TFLOPs"] = round(ex / t / 1e12, 2)
            roof["frac_executed"] = round(ex / t / 1e12 / MFMA_BF16_PEAK_TFS, 4)
    traffic, tsrc = measured_traffic(cfg, dom)
    roof["traffic"] = traffic
    roof["traffic_record"] = tsrc
    roof["kernel"] = dom
    roof["kernels"] = list(STAGE_KERNELS[dom])
    roof["ms_per_launch"] = round(ms, 5)
    roof["alg_bytes_per_launch"] = by
    roof["alg_flops_per_launch"] = fl
    return roof


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _host(t):
    return t.detach().cpu()


def cpu_baseline(res, rows_wanted, min_seconds=10.0, max_passes=50):
    """The oracle (as it stands) on a bounded sample of the timed workload,
    fed the GPU's own input bytes copied to the host: up to `rows_wanted`
    query rows through the whole step, repeated to about `min_seconds`."""
    import numpy as np

    import oracle
    cfg = res["config_id"]
    inp = res["_inp"]
    h = {k: (_host(v) if hasattr(v, "detach") else v) for k, v in inp.items()}
    if cfg == 7:
        return _cpu_baseline_projections(inp, h, rows_wanted, min_seconds, max_passes)
    B, Tq = inp["B"], inp["Tq"]
    qp_all = h["q_pos"].numpy().reshape(-1)
    pd_all = np.repeat(h["pad"].numpy(), Tq)
    rows = np.unique(np.linspace(0, B * Tq - 1, num=min(rows_wanted, B * Tq)).round()
                     .astype(np.int64))
    if cfg in (5, 6):
        kp, sk, width = inp["kpool"], inp["select_k"], inp["out_width"]

        def one_pass():
            pk, _ = oracle.pool_keys(h["k_idx"], h["gate"], h["pad"], kp)
            S = oracle.index_scores(h["q_idx"], pk, h["w"], inp["scale_idx"], h["q_pos"],
                                    h["pad"], kpool=kp, rows=rows)
            tok = oracle.pool_select(S, qp_all[rows], pd_all[rows], kp, sk, width)
            idx = np.full((B * Tq, width), -1, np.int32)
            idx[rows] = tok
            oracle.sparse_attend(h["q"], h["K"], h["V"], idx.reshape(B, Tq, width),
                                 inp["scale_attn"], inp["H"], q_pos=h["q_pos"], pad=h["pad"],
                                 rows=rows)
        what = ("pool keys (all pools), pooled index scores over all visible pools, pool "
                "select and per-head attention")
    else:
        def one_pass():
            S = oracle.index_scores(h["q_idx"], h["k_idx"], h["w"], inp["scale_idx"],
                                    h["q_pos"], h["pad"], k_scale=h.get("k_scale"), rows=rows)
            sel = oracle.topk(S, qp_all[rows], pd_all[rows], inp["top_k"])
            idx = np.full((B * Tq, inp["top_k"]), -1, np.int32)
            idx[rows] = sel
            idx = idx.reshape(B, Tq, -1)
            if inp["dtype"] == "f32":
                oracle.sparse_attend(h["q"], h["K"], h["V"], idx, inp["scale_attn"], inp["H"],
                                     q_pos=h["q_pos"], pad=h["pad"], rows=rows)
            else:
                oracle.sparse_attend(h["q"], h["KV"], None, idx, inp["scale_attn"], 1,
                                     q_pos=h["q_pos"], pad=h["pad"], rows=rows,
                                     k_row_stride=inp["kd"], vd=inp["vd"])
        what = "index scores over all keys, top-k and attention"
    return _time_passes(one_pass, len(rows), B * Tq, what, min_seconds, max_passes)


def _time_passes(one_pass, n_rows, n_all, what, min_seconds, max_passes):
    import oracle
    passes = 0
    t0 = time.perf_counter()
    while True:
        one_pass()
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or passes >= max_passes:
            break
    return {"value": round(n_rows * passes / dt, 3), "unit": "tokens/s",
            "cores": oracle.threads(), "kind": "oracle",
            "nproc": os.cpu_count(), "cpu_model": _cpu_model(),
            "sample": f"{n_rows} of {n_all} query rows of the timed workload, evenly spaced, "
                      f"on the GPU's own input bytes: {what}; {passes} pass(es) in {dt:.1f} s"}


def _cpu_baseline_projections(inp, h, rows_wanted, min_seconds, max_passes):
    import numpy as np

    import oracle
    T = inp["T"]
    rows = np.unique(np.linspace(0, T - 1, num=min(rows_wanted, T)).round().astype(np.int64))
    pos = h["pos"].numpy()[rows]

    def one_pass():
        oracle.indexer_frontend(h["q_lora"][rows], h["x"][rows], pos, h["wq_b"], h["wk"],
                                h["k_norm_w"], h["k_norm_b"], h["w_proj"], inp["Hi"],
                                inp["rope_dim"], inp["rope_theta"], inp["norm_eps"])
        oracle.expand_kv(h["latent"][rows], h["w_kv_b"], inp["H"], inp["kd"], inp["vd"])
    return _time_passes(one_pass, len(rows), T, "indexer front-end and expand_kv", min_seconds,
                        max_passes)


def _public(res):
    return {k: v for k, v in res.items() if not k.startswith("_")}


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
    K = args.steps
    peaks = None
    if not args.only:
        print("[bench] measuring the copy and MFMA-loop peaks", file=sys.stderr, flush=True)
        peaks = measure_peaks()
    print(f"[bench] config {cfg}: generating inputs", file=sys.stderr, flush=True)
    res = run_workload(cfg, dsa, W, K, args.warmup, graph=args.graph)
    roof = roofline_of(cfg, res, peaks)
    inp = res["_inp"]
    result = {
        "metric": METRIC,
        "value": res["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if inp["dtype"] == "f32" else "bf16",
        "data": "synthetic",
        "config": {k: res[k] for k in ("workload", "config_id", "query_tokens_per_step",
                                       "seed", "launch")},
        "roofline": roof,
        "stages": res["stages"],
    }
    if peaks:
        result["peaks_measured"] = peaks
    if args.copy_probe:
        copy_probe(args.copy_probe)
    if not args.no_cpu:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(res, args.cpu_rows)
    del res, inp
    torch.cuda.empty_cache()
    if not args.only:
        configs = {}
        for c in (2, 3, 4, 5, 6, 7):
            if c == cfg:
                continue
            print(f"[bench] config {c}", file=sys.stderr, flush=True)
            r = run_workload(c, dsa, W, K, args.warmup)
            r["roofline"] = roofline_of(c, r, peaks)
            configs[str(c)] = _public(r)
            del r
            torch.cuda.empty_cache()
        result["configs"] = configs
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
