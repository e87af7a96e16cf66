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


class _PoolDims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seq", ctypes.c_int32), ("n_q", ctypes.c_int32),
                ("kpool", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("select_k", ctypes.c_int32), ("out_width", ctypes.c_int32)]


_lock = threading.Lock()
_lib = None
EXPORTS = ("dsa_last_error", "dsa_version", "dsa_visibility_ranges", "dsa_index_scores",
           "dsa_topk_workspace_size", "dsa_topk", "dsa_sparse_attend_workspace_size",
           "dsa_sparse_attend", "dsa_pool_keys", "dsa_pool_select_workspace_size",
           "dsa_pool_select")


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
        lib.dsa_topk.argtypes = [P, I32, I32, I64, P, P, I32, P, P, SZ, P]
        lib.dsa_sparse_attend_workspace_size.argtypes = [P]
        lib.dsa_sparse_attend_workspace_size.restype = SZ
        lib.dsa_sparse_attend.argtypes = [P, ctypes.c_int, P, P, I64, P, I64, P, P, P, P, P, P,
                                          SZ, P]
        lib.dsa_pool_keys.argtypes = [P, ctypes.c_int, P, P, P, P, P, P]
        lib.dsa_pool_select_workspace_size.argtypes = [P]
        lib.dsa_pool_select_workspace_size.restype = SZ
        lib.dsa_pool_select.argtypes = [P, P, P, P, P, P, P, SZ, P]
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
    _dev(pad, q_pos)
    B, n_q = q_pos.shape
    lo = torch.empty((B, n_q), dtype=torch.int32, device=q_pos.device) if lo is None else lo
    hi = torch.empty((B, n_q), dtype=torch.int32, device=q_pos.device) if hi is None else hi
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
    if out is None:
        out = torch.empty((B, n_q, n_k), dtype=torch.float32, device=q.device)
    dims = _IndexDims(B, n_q, n_k, H, d, float(scale))
    _check(load().dsa_index_scores(ctypes.byref(dims), _p(q), _dtype_code(q), _p(k),
                                   _dtype_code(k), _p(k_scale), _p(w), _p(_i32(vis_lo)),
                                   _p(_i32(vis_hi)), _p(out), _stream()))
    return out


def topk_workspace_size(rows: int, n_cols: int, top_k: int) -> int:
    return int(load().dsa_topk_workspace_size(rows, n_cols, top_k))


def topk(scores, vis_lo, vis_hi, top_k: int, out=None, workspace=None):
    """Top-k index rows [..., top_k] (int32, rank order, INVALID-padded)."""
    _dev(scores, vis_lo, vis_hi, out)
    lead = scores.shape[:-1]
    n_cols = scores.shape[-1]
    rows = math.prod(lead)
    if out is None:
        out = torch.empty((*lead, top_k), dtype=torch.int32, device=scores.device)
    ws, wsb = _workspace(topk_workspace_size(rows, n_cols, top_k), workspace, scores.device)
    _check(load().dsa_topk(_p(scores), rows, n_cols, n_cols, _p(_i32(vis_lo)), _p(_i32(vis_hi)),
                           top_k, _p(out), _p(ws), wsb, _stream()))
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
    if k.dtype != q.dtype or k.shape[0] != B or idx.shape[:2] != (B, n_q):
        raise ValueError("sparse_attend: shape/dtype mismatch")
    dims = _attn_dims(q, k, n_k, idx, kv_heads, vd, kd, scale)
    if out is None:
        out = torch.empty((B, n_q, H, vd), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, n_q, H), dtype=torch.float32, device=q.device)
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
    if out is None:
        out = torch.empty((B, L // kpool, d), dtype=k.dtype, device=k.device)
    if n_pools is None:
        n_pools = torch.empty(B, dtype=torch.int32, device=k.device)
    dims = _PoolDims(B, L, 0, kpool, d, 1, 1)
    _check(load().dsa_pool_keys(ctypes.byref(dims), _dtype_code(k), _p(k), _p(gate),
                                _p(_i32(pad)), _p(out), _p(n_pools), _stream()))
    return out, n_pools


def pool_select(scores, pad, q_pos, kpool: int, select_k: int, out_width: int, out_tok=None,
                out_pools=None, want_pools: bool = False):
    """topk_pools + expand_selection.  scores: [B, n_q, seq//kpool] f32."""
    _dev(scores, pad, q_pos, out_tok, out_pools)
    B, n_q, n_pool_cols = scores.shape
    seq = n_pool_cols * kpool
    if out_tok is None:
        out_tok = torch.empty((B, n_q, out_width), dtype=torch.int32, device=scores.device)
    if out_pools is None and want_pools:
        out_pools = torch.empty((B, n_q, select_k), dtype=torch.int32, device=scores.device)
    dims = _PoolDims(B, seq, n_q, kpool, 0, select_k, out_width)
    _check(load().dsa_pool_select(ctypes.byref(dims), _p(scores), _p(_i32(pad)),
                                  _p(_i32(q_pos)), _p(out_tok), _p(out_pools), None, 0,
                                  _stream()))
    return (out_tok, out_pools) if want_pools else out_tok
