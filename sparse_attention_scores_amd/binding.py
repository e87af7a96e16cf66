"""Thin ctypes binding over libdsa.so (see include/dsa.h).

Argument marshalling only: shapes and dtypes are checked, outputs and
workspaces are allocated with torch when the caller does not pass them, and
each call enqueues libdsa's kernels on torch's current HIP stream.  There is
no fallback: if libdsa.so is missing or does not load, every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa.so")

INVALID = -1
DSA_F32, DSA_BF16, DSA_FP8_E4M3 = 0, 1, 2
_STATUS = {0: "DSA_OK", -1: "DSA_ERR_ARG", -2: "DSA_ERR_UNSUPPORTED", -3: "DSA_ERR_HIP",
           -4: "DSA_ERR_WORKSPACE"}


class DsaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{_STATUS.get(code, code)}: {msg}")
        self.code = code


class _IndexDims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q", ctypes.c_int32), ("n_k", ctypes.c_int32),
                ("n_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("scale", ctypes.c_float)]


class _AttnDims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q", ctypes.c_int32), ("n_k", ctypes.c_int32),
                ("n_heads", ctypes.c_int32), ("kd", ctypes.c_int32), ("vd", ctypes.c_int32),
                ("kv_heads", ctypes.c_int32), ("n_sel", ctypes.c_int32),
                ("scale", ctypes.c_float)]


class _CacheDims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_new", ctypes.c_int32), ("n_cache", ctypes.c_int32),
                ("head_dim", ctypes.c_int32)]


class _FrontendDims(ctypes.Structure):
    _fields_ = [("tokens", ctypes.c_int32), ("q_lora_rank", ctypes.c_int32),
                ("hidden", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("rope_dim", ctypes.c_int32),
                ("rope_theta", ctypes.c_float), ("norm_eps", ctypes.c_float)]


class _ExpandDims(ctypes.Structure):
    _fields_ = [("tokens", ctypes.c_int32), ("rank", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("kd", ctypes.c_int32), ("vd", ctypes.c_int32)]


class _PoolDims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seq", ctypes.c_int32), ("n_q", ctypes.c_int32),
                ("kpool", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("select_k", ctypes.c_int32), ("out_width", ctypes.c_int32)]


_lock = threading.Lock()
_lib = None
EXPORTS = ("dsa_last_error", "dsa_version", "dsa_visibility_ranges", "dsa_index_scores",
           "dsa_topk_workspace_size", "dsa_topk", "dsa_topk_noalloc", "dsa_index_share_source",
           "dsa_sparse_attend_workspace_size",
           "dsa_sparse_attend", "dsa_pool_keys", "dsa_pool_select_workspace_size",
           "dsa_pool_select", "dsa_hadamard_rotate", "dsa_index_cache_write",
           "dsa_indexer_frontend", "dsa_expand_kv")


def _hip_runtimes_mapped():
    """Distinct libamdhip64 files mapped into this process."""
    paths = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    paths.add(os.path.realpath(line.split()[-1]))
    except OSError:
        pass
    return paths


def load():
    """Load libdsa.so (raises if it is not built)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m "
                               "sparse_attention_scores_amd.build` (there is no CPU fallback)")
        import torch  # noqa: F401  (torch's HIP runtime must be the one libdsa binds to)
        lib = ctypes.CDLL(LIB_PATH)
        runtimes = _hip_runtimes_mapped()
        if len(runtimes) > 1:
            raise RuntimeError(f"two HIP runtimes are mapped ({sorted(runtimes)}); libdsa must "
                               "share torch's")
        P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        lib.dsa_last_error.restype = ctypes.c_char_p
        lib.dsa_version.restype = ctypes.c_char_p
        lib.dsa_visibility_ranges.argtypes = [I32, I32, P, P, I32, P, P, P]
        lib.dsa_index_scores.argtypes = [P, P, ctypes.c_int, P, ctypes.c_int, P, P, P, P, P, P]
        lib.dsa_topk_workspace_size.argtypes = [I32, I32, I32]
        lib.dsa_topk_workspace_size.restype = SZ
        lib.dsa_index_share_source.argtypes = [I32]
        lib.dsa_index_share_source.restype = I32
        lib.dsa_topk.argtypes = [P, I32, I32, I64, P, P, I32, I32, P, P, SZ, P]
        lib.dsa_topk_noalloc.argtypes = [P, I32, I32, I64, P, P, I32, I32, P, P]
        lib.dsa_sparse_attend_workspace_size.argtypes = [P]
        lib.dsa_sparse_attend_workspace_size.restype = SZ
        lib.dsa_sparse_attend.argtypes = [P, ctypes.c_int, P, P, I64, P, I64, P, P, P, P, P, P,
                                          SZ, P]
        lib.dsa_pool_keys.argtypes = [P, ctypes.c_int, P, P, P, P, P, P]
        lib.dsa_pool_select_workspace_size.argtypes = [P]
        lib.dsa_pool_select_workspace_size.restype = SZ
        lib.dsa_pool_select.argtypes = [P, P, P, P, P, P, P, SZ, P]
        lib.dsa_hadamard_rotate.argtypes = [I64, I32, P, ctypes.c_int, P, ctypes.c_int, P]
        lib.dsa_index_cache_write.argtypes = [P, P, ctypes.c_int, P, P, ctypes.c_int, P, P]
        lib.dsa_indexer_frontend.argtypes = [P] * 13
        lib.dsa_expand_kv.argtypes = [P, P, P, P, I64, P, I64, P]
        _lib = lib
        return lib


def version() -> str:
    return load().dsa_version().decode()


def _check(rc: int):
    if rc != 0:
        raise DsaError(rc, load().dsa_last_error().decode())


# torch's current HIP stream on the current device, as a raw handle (torch's
# own accessor of it, without building a Stream object per call; the public
# route is kept for torch builds that lack it)
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream():
    if _raw_stream is not None:
        return ctypes.c_void_p(_raw_stream(torch.cuda.current_device()))
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return DSA_F32
    if t.dtype == torch.bfloat16:
        return DSA_BF16
    if t.dtype == torch.float8_e4m3fn:
        return DSA_FP8_E4M3
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("libdsa takes device tensors")
            if not t.is_contiguous():
                raise ValueError("libdsa takes contiguous tensors")


def _i32(t):
    if t.dtype != torch.int32:
        raise TypeError(f"expected int32, got {t.dtype}")
    return t


def _shape(t, shape, name: str, dtype=None):
    """Raise unless t (when given) has exactly `shape` (and `dtype`): a short
    or mistyped tensor would otherwise become an out-of-bounds device read."""
    if t is None:
        return t
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    return t


def _workspace(nbytes: int, ws, device):
    if nbytes == 0:
        return None, 0
    if ws is None:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if ws.numel() * ws.element_size() < nbytes:
        raise ValueError(f"workspace needs {nbytes} bytes")
    return ws, ws.numel() * ws.element_size()


# --------------------------------------------------------------------------

def visibility_ranges(pad, q_pos, kpool: int = 0, lo=None, hi=None):
    """[vis_lo, vis_hi) per query (token keys, or pools when kpool > 0)."""
    _dev(pad, q_pos, lo, hi)
    B, n_q = q_pos.shape
    _shape(pad, (B,), "visibility_ranges: pad", torch.int32)
    lo = torch.empty((B, n_q), dtype=torch.int32, device=q_pos.device) if lo is None else lo
    hi = torch.empty((B, n_q), dtype=torch.int32, device=q_pos.device) if hi is None else hi
    _shape(lo, (B, n_q), "visibility_ranges: lo", torch.int32)
    _shape(hi, (B, n_q), "visibility_ranges: hi", torch.int32)
    _check(load().dsa_visibility_ranges(B, n_q, _p(_i32(pad)), _p(_i32(q_pos)), kpool, _p(lo),
                                        _p(hi), _stream()))
    return lo, hi


def index_scores(q, k, w, vis_lo, vis_hi, scale: float, k_scale=None, out=None):
    """Index scores [B, n_q, n_k] (f32).  q: [B,n_q,H,d]; k: [B,n_k,d]."""
    _dev(q, k, w, vis_lo, vis_hi, k_scale, out)
    B, n_q, H, d = q.shape
    n_k = k.shape[1]
    if k.shape != (B, n_k, d) or w.shape != (B, n_q, H) or w.dtype != torch.float32:
        raise ValueError("index_scores: shape/dtype mismatch")
    if k_scale is not None and (k_scale.shape != (B, n_k) or k_scale.dtype != torch.float32):
        raise ValueError("index_scores: k_scale must be f32 [B, n_k]")
    _shape(vis_lo, (B, n_q), "index_scores: vis_lo", torch.int32)
    _shape(vis_hi, (B, n_q), "index_scores: vis_hi", torch.int32)
    if out is None:
        out = torch.empty((B, n_q, n_k), dtype=torch.float32, device=q.device)
    _shape(out, (B, n_q, n_k), "index_scores: out", torch.float32)
    dims = _IndexDims(B, n_q, n_k, H, d, float(scale))
    _check(load().dsa_index_scores(ctypes.byref(dims), _p(q), _dtype_code(q), _p(k),
                                   _dtype_code(k), _p(k_scale), _p(w), _p(_i32(vis_lo)),
                                   _p(_i32(vis_hi)), _p(out), _stream()))
    return out


def index_share_source(layer: int) -> int:
    """IndexShare: the layer whose top-k rows `layer` attends with (itself
    when it is a full layer)."""
    return int(load().dsa_index_share_source(int(layer)))


def topk_workspace_size(rows: int, n_cols: int, top_k: int) -> int:
    return int(load().dsa_topk_workspace_size(rows, n_cols, top_k))


def topk(scores, vis_lo, vis_hi, top_k: int, out=None, workspace=None, n_sink: int = 0):
    """Top-k index rows [..., top_k] (int32, rank order, INVALID-padded);
    with n_sink > 0 the first n_sink visible columns of each row rank first
    (attention sinks)."""
    _dev(scores, vis_lo, vis_hi, out)
    if scores.dtype != torch.float32:
        raise TypeError(f"topk: scores must be float32, got {scores.dtype}")
    lead = scores.shape[:-1]
    n_cols = scores.shape[-1]
    rows = math.prod(lead)
    if vis_lo.numel() != rows or vis_hi.numel() != rows:
        raise ValueError(f"topk: vis_lo/vis_hi need {rows} elements, got "
                         f"{vis_lo.numel()}/{vis_hi.numel()}")
    if out is None:
        out = torch.empty((*lead, top_k), dtype=torch.int32, device=scores.device)
    if out.numel() != rows * top_k or out.dtype != torch.int32:
        raise ValueError(f"topk: out must be int32 with {rows} x {top_k} elements")
    ws, wsb = _workspace(topk_workspace_size(rows, n_cols, top_k), workspace, scores.device)
    _check(load().dsa_topk(_p(scores), rows, n_cols, n_cols, _p(_i32(vis_lo)), _p(_i32(vis_hi)),
                           top_k, int(n_sink), _p(out), _p(ws), wsb, _stream()))
    return out


def topk_noalloc(scores, vis_lo, vis_hi, top_k: int, out, n_sink: int = 0):
    """Top-k into a caller-given `out`, with no workspace: the library's own
    per-GPU scratch holds the chunk winners of long rows (nothing is
    allocated, here or in the library)."""
    _dev(scores, vis_lo, vis_hi, out)
    if scores.dtype != torch.float32:
        raise TypeError(f"topk_noalloc: scores must be float32, got {scores.dtype}")
    n_cols = scores.shape[-1]
    rows = math.prod(scores.shape[:-1])
    if vis_lo.numel() != rows or vis_hi.numel() != rows:
        raise ValueError(f"topk_noalloc: vis_lo/vis_hi need {rows} elements")
    if out.numel() != rows * top_k or out.dtype != torch.int32:
        raise ValueError(f"topk_noalloc: out must be int32 with {rows} x {top_k} elements")
    _check(load().dsa_topk_noalloc(_p(scores), rows, n_cols, n_cols, _p(_i32(vis_lo)),
                                   _p(_i32(vis_hi)), top_k, int(n_sink), _p(out), _stream()))
    return out


def _attn_dims(q, k, n_k, idx, kv_heads, vd, kd, scale):
    B, n_q, H, _ = q.shape
    return _AttnDims(B, n_q, n_k, H, kd, vd, kv_heads, idx.shape[-1], float(scale))


def sparse_attend_workspace_size(dims) -> int:
    return int(load().dsa_sparse_attend_workspace_size(ctypes.byref(dims)))


def sparse_attend(q, k, v, idx, scale: float, kv_heads: int, vd: int | None = None,
                  vis_lo=None, vis_hi=None, out=None, lse=None, workspace=None,
                  want_lse: bool = True):
    """Sparse attention over each query's selected keys.

    q: [B,n_q,H,kd].  k: [B,n_k,kv_heads,kd] or [B,n_k,kd_row] (absorbed latent
    rows).  v: [B,n_k,kv_heads,vd], or None to use the first vd columns of
    k's rows (absorbed MLA).  idx: [B,n_q,n_sel] int32.
    Returns (out [B,n_q,H,vd] f32, lse [B,n_q,H] f32 or None)."""
    _dev(q, k, v, idx, vis_lo, vis_hi, out, lse)
    B, n_q, H, kd = q.shape
    n_k = k.shape[1]
    k_row = k.stride(1)
    if v is None:
        if vd is None:
            raise ValueError("absorbed attention needs vd")
        v_ptr, v_row = _p(k), k_row
    else:
        vd = v.shape[-1] if vd is None else vd
        v_ptr, v_row = _p(v), v.stride(1)
        if v.dtype != q.dtype or v.shape[:2] != (B, n_k):
            raise ValueError("sparse_attend: v shape/dtype mismatch")
    if k.dtype != q.dtype or k.shape[0] != B or idx.dim() != 3 or idx.shape[:2] != (B, n_q):
        raise ValueError("sparse_attend: shape/dtype mismatch")
    if (vis_lo is None) != (vis_hi is None):
        raise ValueError("sparse_attend: give both vis_lo and vis_hi or neither")
    _shape(vis_lo, (B, n_q), "sparse_attend: vis_lo", torch.int32)
    _shape(vis_hi, (B, n_q), "sparse_attend: vis_hi", torch.int32)
    dims = _attn_dims(q, k, n_k, idx, kv_heads, vd, kd, scale)
    if out is None:
        out = torch.empty((B, n_q, H, vd), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, n_q, H), dtype=torch.float32, device=q.device)
    _shape(out, (B, n_q, H, vd), "sparse_attend: out", torch.float32)
    _shape(lse, (B, n_q, H), "sparse_attend: lse", torch.float32)
    ws, wsb = _workspace(sparse_attend_workspace_size(dims), workspace, q.device)
    _check(load().dsa_sparse_attend(ctypes.byref(dims), _dtype_code(q), _p(q), _p(k), k_row,
                                    v_ptr, v_row, _p(_i32(idx)), _p(vis_lo), _p(vis_hi), _p(out),
                                    _p(lse), _p(ws), wsb, _stream()))
    return out, lse


def pool_keys(k, gate, pad, kpool: int, out=None, n_pools=None):
    """Pooled indexer keys [B, seq//kpool, d] (same dtype as k) and n_pools [B]."""
    _dev(k, gate, pad, out, n_pools)
    B, L, d = k.shape
    if gate.shape != k.shape or gate.dtype != k.dtype:
        raise ValueError("pool_keys: gate must match k")
    _shape(pad, (B,), "pool_keys: pad", torch.int32)
    if out is None:
        out = torch.empty((B, L // kpool, d), dtype=k.dtype, device=k.device)
    if n_pools is None:
        n_pools = torch.empty(B, dtype=torch.int32, device=k.device)
    _shape(out, (B, L // kpool, d), "pool_keys: out", k.dtype)
    _shape(n_pools, (B,), "pool_keys: n_pools", torch.int32)
    dims = _PoolDims(B, L, 0, kpool, d, 1, 1)
    _check(load().dsa_pool_keys(ctypes.byref(dims), _dtype_code(k), _p(k), _p(gate),
                                _p(_i32(pad)), _p(out), _p(n_pools), _stream()))
    return out, n_pools


def pool_select(scores, pad, q_pos, kpool: int, select_k: int, out_width: int, out_tok=None,
                out_pools=None, want_pools: bool = False):
    """topk_pools + expand_selection.  scores: [B, n_q, seq//kpool] f32."""
    _dev(scores, pad, q_pos, out_tok, out_pools)
    if scores.dtype != torch.float32:
        raise TypeError(f"pool_select: scores must be float32, got {scores.dtype}")
    B, n_q, n_pool_cols = scores.shape
    seq = n_pool_cols * kpool
    _shape(pad, (B,), "pool_select: pad", torch.int32)
    _shape(q_pos, (B, n_q), "pool_select: q_pos", torch.int32)
    if out_tok is None:
        out_tok = torch.empty((B, n_q, out_width), dtype=torch.int32, device=scores.device)
    if out_pools is None and want_pools:
        out_pools = torch.empty((B, n_q, select_k), dtype=torch.int32, device=scores.device)
    _shape(out_tok, (B, n_q, out_width), "pool_select: out_tok", torch.int32)
    _shape(out_pools, (B, n_q, select_k), "pool_select: out_pools", torch.int32)
    dims = _PoolDims(B, seq, n_q, kpool, 0, select_k, out_width)
    _check(load().dsa_pool_select(ctypes.byref(dims), _p(scores), _p(_i32(pad)),
                                  _p(_i32(q_pos)), _p(out_tok), _p(out_pools), None, 0,
                                  _stream()))
    return (out_tok, out_pools) if want_pools else out_tok


def hadamard_rotate(x, out=None, out_dtype=None):
    """y = H_d x / sqrt(d) over the last axis (Sylvester Hadamard), as f32 or
    bf16 (default: x's dtype).  out may be x itself."""
    _dev(x, out)
    d = x.shape[-1]
    rows = math.prod(x.shape[:-1])
    if out is None:
        out = torch.empty(x.shape, dtype=out_dtype or x.dtype, device=x.device)
    _shape(out, x.shape, "hadamard_rotate: out")
    _check(load().dsa_hadamard_rotate(rows, d, _p(x), _dtype_code(x), _p(out), _dtype_code(out),
                                      _stream()))
    return out


def index_cache_write(k_new, kv_head, cache, k_scale=None):
    """Rotate the new indexer keys [B, n_new, d] and write them into the
    cache [B, n_cache, d] (float8_e4m3fn with k_scale [B, n_cache], or bf16)
    at each sequence's kv_head [B] (int32)."""
    _dev(k_new, kv_head, cache, k_scale)
    B, n_new, d = k_new.shape
    if cache.dim() != 3 or cache.shape[0] != B or cache.shape[2] != d:
        raise ValueError("index_cache_write: cache must be [B, n_cache, d]")
    n_cache = cache.shape[1]
    _shape(kv_head, (B,), "index_cache_write: kv_head", torch.int32)
    _shape(k_scale, (B, n_cache), "index_cache_write: k_scale", torch.float32)
    dims = _CacheDims(B, n_new, n_cache, d)
    _check(load().dsa_index_cache_write(ctypes.byref(dims), _p(k_new), _dtype_code(k_new),
                                        _p(kv_head), _p(cache), _dtype_code(cache), _p(k_scale),
                                        _stream()))
    return cache, k_scale


def indexer_frontend(q_lora, x, pos, wq_b, wk, k_norm_w, k_norm_b, w_proj, n_heads: int,
                     rope_dim: int, rope_theta: float, norm_eps: float, q_out=None, k_out=None,
                     w_out=None):
    """The indexer's q [T, n_heads, 128] bf16, k [T, 128] bf16 and head
    weights [T, n_heads] f32 from q_lora [T, r_q] and x [T, hidden] (bf16)
    at positions pos [T] (int32)."""
    _dev(q_lora, x, pos, wq_b, wk, k_norm_w, k_norm_b, w_proj, q_out, k_out, w_out)
    T, r_q = q_lora.shape
    hidden = x.shape[1]
    for t, nm in ((q_lora, "q_lora"), (x, "x"), (wq_b, "wq_b"), (wk, "wk"), (w_proj, "w_proj")):
        if t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise TypeError(f"indexer_frontend: {nm} must be contiguous bf16")
    _shape(x, (T, hidden), "indexer_frontend: x", torch.bfloat16)
    _shape(pos, (T,), "indexer_frontend: pos", torch.int32)
    _shape(wq_b, (n_heads * 128, r_q), "indexer_frontend: wq_b", torch.bfloat16)
    _shape(wk, (128, hidden), "indexer_frontend: wk", torch.bfloat16)
    _shape(w_proj, (n_heads, hidden), "indexer_frontend: w_proj", torch.bfloat16)
    _shape(k_norm_w, (128,), "indexer_frontend: k_norm_w", torch.float32)
    _shape(k_norm_b, (128,), "indexer_frontend: k_norm_b", torch.float32)
    dev = q_lora.device
    if q_out is None:
        q_out = torch.empty((T, n_heads, 128), dtype=torch.bfloat16, device=dev)
    if k_out is None:
        k_out = torch.empty((T, 128), dtype=torch.bfloat16, device=dev)
    if w_out is None:
        w_out = torch.empty((T, n_heads), dtype=torch.float32, device=dev)
    _shape(q_out, (T, n_heads, 128), "indexer_frontend: q_out", torch.bfloat16)
    _shape(k_out, (T, 128), "indexer_frontend: k_out", torch.bfloat16)
    _shape(w_out, (T, n_heads), "indexer_frontend: w_out", torch.float32)
    for t, nm in ((pos, "pos"), (k_norm_w, "k_norm_w"), (k_norm_b, "k_norm_b"), (q_out, "q_out"),
                  (k_out, "k_out"), (w_out, "w_out")):
        if not t.is_contiguous():
            raise ValueError(f"indexer_frontend: {nm} must be contiguous")
    dims = _FrontendDims(T, r_q, hidden, n_heads, 128, rope_dim, float(rope_theta),
                         float(norm_eps))
    _check(load().dsa_indexer_frontend(ctypes.byref(dims), _p(q_lora), _p(x), _p(pos), _p(wq_b),
                                       _p(wk), _p(k_norm_w), _p(k_norm_b), _p(w_proj), _p(q_out),
                                       _p(k_out), _p(w_out), _stream()))
    return q_out, k_out, w_out


def expand_kv(latent, w_kv_b, n_heads: int, kd: int, vd: int, k_out=None, v_out=None):
    """Per-head K [T, n_heads, kd] and V [T, n_heads, vd] (bf16) from the
    latent [T, rank] and w_kv_b [n_heads * (kd + vd), rank] (bf16).  Outputs
    may be views whose token stride is larger (e.g. [B, L, H, kd] slices)."""
    _dev(latent, w_kv_b)
    for t in (k_out, v_out):
        if t is not None and not t.is_cuda:
            raise ValueError("libdsa takes device tensors")
    T, rank = latent.shape
    for t, nm in ((latent, "latent"), (w_kv_b, "w_kv_b")):
        if t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise TypeError(f"expand_kv: {nm} must be contiguous bf16")
    _shape(w_kv_b, (n_heads * (kd + vd), rank), "expand_kv: w_kv_b", torch.bfloat16)
    dev = latent.device
    if k_out is None:
        k_out = torch.empty((T, n_heads, kd), dtype=torch.bfloat16, device=dev)
    if v_out is None:
        v_out = torch.empty((T, n_heads, vd), dtype=torch.bfloat16, device=dev)
    for t, w, nm in ((k_out, kd, "k_out"), (v_out, vd, "v_out")):
        if (t.dtype != torch.bfloat16 or t.dim() != 3 or tuple(t.shape) != (T, n_heads, w)
                or t.stride(-1) != 1 or t.stride(-2) != w):
            raise ValueError(f"expand_kv: {nm} must be bf16 [T, {n_heads}, {w}] with contiguous heads")
    dims = _ExpandDims(T, rank, n_heads, kd, vd)
    _check(load().dsa_expand_kv(ctypes.byref(dims), _p(latent), _p(w_kv_b), _p(k_out),
                                k_out.stride(-3), _p(v_out), v_out.stride(-3), _stream()))
    return k_out, v_out
