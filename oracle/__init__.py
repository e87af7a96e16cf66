"""CPU oracle of the DSA layer step -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library
(``sparse_attention_scores_amd``) never imports it and shares no code with it.

The arithmetic lives in ``dsa_oracle.c`` (plain C, IEEE double, OpenMP over
query rows).  This module only compiles it with gcc and marshals numpy arrays.

Pins (see ``tests/test_oracle_*.py``): every function here is checked against
closed forms, the worked examples of the "Module glm5next_dsa_ref" page,
brute force on tiny inputs, and library routines (numpy / torch in float64).
Parity unpinned: numerics of real GLM-5.x checkpoints (no weights or goldens
exist here); the readings of the pages that the oracle takes are listed in the
header of each function in ``dsa_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dsa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libdsa_oracle.so")
_lock = threading.Lock()
_lib = None

INVALID = -1
F32, BF16, E4M3, F64 = 0, 1, 2, 3


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (OpenMP) into libdsa_oracle.so."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            # DSA_ORACLE_LIB names another build of dsa_oracle.c (the
            # sanitizer test loads one built with ASan/UBSan)
            path = os.environ.get("DSA_ORACLE_LIB")
            if not path:
                path = _LIB_PATH
                if not os.path.exists(path):
                    build(force=True)
            lib = ctypes.CDLL(path)
            P = ctypes.c_void_p
            I64 = ctypes.c_int64
            I32 = ctypes.c_int32
            D = ctypes.c_double
            lib.orc_bf16_value.argtypes = [ctypes.c_uint16]
            lib.orc_bf16_value.restype = D
            lib.orc_e4m3_value.argtypes = [ctypes.c_uint8]
            lib.orc_e4m3_value.restype = D
            lib.orc_token_visible.argtypes = [I32, I32, I64]
            lib.orc_pool_visible.argtypes = [I32, I32, I32, I64]
            lib.orc_index_scores.argtypes = [I64, I64, I64, I64, I64, P, ctypes.c_int, P,
                                             ctypes.c_int, P, P, D, P, P, I32, P, I64, P, P]
            lib.orc_topk.argtypes = [P, I64, I64, I64, P, P, I32, I32, I32, P]
            lib.orc_index_share_source.argtypes = [I32]
            lib.orc_index_share_source.restype = I32
            lib.orc_pool_keys.argtypes = [I64, I64, I64, I32, P, ctypes.c_int, P,
                                          ctypes.c_int, P, P, P, P]
            lib.orc_pool_select.argtypes = [P, I64, I64, I64, P, P, I32, I32, I32, P, P]
            lib.orc_topk_to_mask.argtypes = [P, I64, I64, ctypes.c_int, I32, I32, P]
            lib.orc_topk_to_mask.restype = None
            lib.orc_sparse_attend.argtypes = [I64, I64, I64, I64, I64, I64, I64, I64,
                                              P, ctypes.c_int, P, I64, P, I64, P, P, P, D,
                                              P, I64, P, P]
            lib.orc_max_threads.argtypes = []
            _lib = lib
    return _lib


def threads() -> int:
    """Number of OpenMP threads the oracle uses."""
    return int(_load().orc_max_threads())


# --------------------------------------------------------------------------
# marshalling helpers
# --------------------------------------------------------------------------

def _storage(a):
    """Return (contiguous numpy array, dtype code) for a numpy array or a CPU
    torch tensor.  bf16 tensors travel as their raw uint16 bits and float8
    e4m3fn tensors as their raw uint8 codes."""
    try:
        import torch
        if isinstance(a, torch.Tensor):
            t = a.detach().cpu().contiguous()
            if t.dtype == torch.bfloat16:
                return t.view(torch.int16).numpy().view(np.uint16), BF16
            if t.dtype == torch.float8_e4m3fn:
                return t.view(torch.uint8).numpy(), E4M3
            a = t.numpy()
    except ImportError:  # pragma: no cover
        pass
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a, F32
    if a.dtype == np.float64:
        return a, F64
    if a.dtype == np.uint16:
        return a, BF16
    if a.dtype == np.uint8:
        return a, E4M3
    raise TypeError("unsupported oracle input dtype %s" % a.dtype)


def _i32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _f32(a):
    try:
        import torch
        if isinstance(a, torch.Tensor):
            a = a.detach().cpu().float().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _rows(rows, n_all):
    if rows is None:
        return None, n_all
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    return r, len(r)


# --------------------------------------------------------------------------
# public functions
# --------------------------------------------------------------------------

def bf16_value(bits: int) -> float:
    return _load().orc_bf16_value(bits)


def e4m3_value(code: int) -> float:
    return _load().orc_e4m3_value(code)


def token_visible(pad: int, qpos: int, s: int) -> bool:
    return bool(_load().orc_token_visible(pad, qpos, s))


def pool_visible(pad: int, kpool: int, qpos: int, i: int) -> bool:
    return bool(_load().orc_pool_visible(pad, kpool, qpos, i))


def index_scores(q, k, w, scale, q_pos, pad, k_scale=None, kpool=0, rows=None,
                 want_mag=False):
    """Index scores for the given query rows.

    q: [B,Tq,H,d]; k: [B,Tk,d] (Tk pools when kpool > 0); w: [B,Tq,H];
    q_pos: [B,Tq] query positions; pad: [B] left-padding counts.
    Returns S [n_rows,Tk] float32 (and the magnitude A [n_rows,Tk] float64)."""
    qa, qt = _storage(q)
    ka, kt = _storage(k)
    B, Tq, H, d = qa.shape
    Tk = ka.shape[1]
    assert ka.shape == (B, Tk, d)
    wa = _f32(w).reshape(B, Tq, H)
    ks = None if k_scale is None else _f32(k_scale).reshape(B, Tk)
    qp = _i32(q_pos).reshape(B * Tq)
    pd = _i32(pad).reshape(B)
    r, n = _rows(rows, B * Tq)
    S = np.empty((n, Tk), np.float32)
    A = np.empty((n, Tk), np.float64) if want_mag else None
    rc = _load().orc_index_scores(B, Tq, Tk, H, d, _ptr(qa), qt, _ptr(ka), kt, _ptr(ks),
                                  _ptr(wa), float(scale), _ptr(qp), _ptr(pd), int(kpool),
                                  _ptr(r), n, _ptr(S), _ptr(A))
    if rc != 0:
        raise ValueError("oracle index_scores: NaN input")
    return (S, A) if want_mag else S


def topk(S, row_qpos, row_pad, k, kpool=0, n_sink=0):
    """Top-k per row (higher score, then smaller index), INVALID-padded.

    S: [rows, n_cols] float32; row_qpos/row_pad: per-row query position and
    sequence padding (visibility).  n_sink > 0 adds the attention-sink boost
    (1e20, in f32) to each row's first n_sink visible columns first."""
    Sa = _f32(S)
    n_rows, n_cols = Sa.shape
    out = np.empty((n_rows, k), np.int32)
    rc = _load().orc_topk(_ptr(Sa), n_rows, n_cols, n_cols, _ptr(_i32(row_qpos)),
                          _ptr(_i32(row_pad)), int(kpool), int(k), int(n_sink), _ptr(out))
    if rc != 0:
        raise ValueError("oracle topk: NaN score")
    return out


def index_share_source(layer: int) -> int:
    """IndexShare: the layer whose indexer selection `layer` uses (itself
    when it is a full layer: layer <= 1 or layer % 4 == 2)."""
    return int(_load().orc_index_share_source(int(layer)))


def pool_keys(k, gate, pad, kpool, want_mag=False):
    """Pooled indexer keys in float64: [B, L//kpool, d], and n_pools [B]
    (and, with want_mag, sum_j softmax_j |k_j| of each pooled value)."""
    ka, kt = _storage(k)
    ga, gt = _storage(gate)
    B, L, d = ka.shape
    pd = _i32(pad).reshape(B)
    pk = np.empty((B, L // kpool, d), np.float64)
    mag = np.empty((B, L // kpool, d), np.float64) if want_mag else None
    npools = np.empty(B, np.int32)
    _load().orc_pool_keys(B, L, d, int(kpool), _ptr(ka), kt, _ptr(ga), gt, _ptr(pd),
                          _ptr(pk), _ptr(npools), _ptr(mag))
    return (pk, npools, mag) if want_mag else (pk, npools)


def pool_select(S, row_qpos, row_pad, kpool, select_k, out_width, want_pools=False):
    """topk_pools + expand_selection per row. S: [rows, n_pool_cols]."""
    Sa = _f32(S)
    n_rows, n_cols = Sa.shape
    tok = np.empty((n_rows, out_width), np.int32)
    pools = np.empty((n_rows, select_k), np.int32) if want_pools else None
    rc = _load().orc_pool_select(_ptr(Sa), n_rows, n_cols, n_cols, _ptr(_i32(row_qpos)),
                                 _ptr(_i32(row_pad)), int(kpool), int(select_k),
                                 int(out_width), _ptr(tok), _ptr(pools))
    if rc == -1:
        raise ValueError("oracle pool_select: NaN score")
    if rc == -2:
        raise ValueError("oracle pool_select: out_width too small")
    return (tok, pools) if want_pools else tok


def topk_to_mask(idx_row, Tk, pad=None, qpos=None):
    """Boolean mask over Tk keys of the selected set of one index row."""
    ia = _i32(idx_row).reshape(-1)
    m = np.empty(Tk, np.uint8)
    has = pad is not None and qpos is not None
    _load().orc_topk_to_mask(_ptr(ia), len(ia), int(Tk), int(has),
                             int(pad or 0), int(qpos or 0), _ptr(m))
    return m.astype(bool)


def sparse_attend(q, K, V, idx, scale, kv_heads, q_pos=None, pad=None, rows=None,
                  k_row_stride=None, v_row_stride=None, vd=None, v_offset=0):
    """Sparse attention over each query's selected set, in float64.

    q: [B,Tq,H,kd]; K: [B,Tk,kv_heads,kd] (or any [B,Tk,...] whose rows are
    k_row_stride elements apart); V likewise, or V=None to use the first vd
    columns of K's rows (absorbed MLA).  idx: [B,Tq,n_sel].
    Returns (out [n_rows,H,vd], lse [n_rows,H])."""
    qa, qt = _storage(q)
    Ka, kt = _storage(K)
    B, Tq, H, kd = qa.shape
    Tk = Ka.shape[1]
    ks = k_row_stride if k_row_stride is not None else int(np.prod(Ka.shape[2:]))
    if V is None:
        Va, vt = Ka, kt
        vs = ks if v_row_stride is None else v_row_stride
        assert vd is not None
    else:
        Va, vt = _storage(V)
        vs = v_row_stride if v_row_stride is not None else int(np.prod(Va.shape[2:]))
        if vd is None:
            vd = Va.shape[-1]
    assert qt == kt == vt, "q, K and V must share a storage dtype"
    ia = _i32(idx).reshape(B, Tq, -1)
    n_sel = ia.shape[2]
    qp = None if q_pos is None else _i32(q_pos).reshape(B * Tq)
    pd = None if pad is None else _i32(pad).reshape(B)
    r, n = _rows(rows, B * Tq)
    out = np.empty((n, H, vd), np.float64)
    lse = np.empty((n, H), np.float64)
    vptr = _ptr(Va)
    if v_offset:
        vptr = ctypes.c_void_p(vptr.value + v_offset * Va.itemsize)
    rc = _load().orc_sparse_attend(B, Tq, Tk, H, kd, vd, int(kv_heads), n_sel, _ptr(qa), qt,
                                   _ptr(Ka), ks, vptr, vs, _ptr(ia), _ptr(qp), _ptr(pd),
                                   float(scale), _ptr(r), n, _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError("oracle sparse_attend: bad kv_heads")
    return out, lse


# --------------------------------------------------------------------------
# indexer-key cache write ("Another DSA attempt": the decode indexer-K cache
# commit and the serving-correctness commit)
# --------------------------------------------------------------------------

def hadamard_rows(x, want_f64=False):
    """Sylvester Hadamard rotation of each last-axis row, y = H x / sqrt(d):
    returns y rounded once to float32 (and the float64 value)."""
    xa, xt = _storage(x)
    d = xa.shape[-1]
    rows = int(np.prod(xa.shape[:-1])) if xa.ndim > 1 else 1
    lib = _load()
    lib.orc_hadamard_rows.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                      ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    y32 = np.empty(xa.shape, np.float32)
    y64 = np.empty(xa.shape, np.float64) if want_f64 else None
    if lib.orc_hadamard_rows(_ptr(xa), xt, rows, d, _ptr(y64), _ptr(y32)) != 0:
        raise ValueError("oracle hadamard_rows: d must be a power of two")
    return (y32, y64) if want_f64 else y32


def e4m3_encode(v):
    """OCP e4m3fn codes (uint8) of float32 values: nearest, ties to even,
    saturating at 448, sign kept."""
    lib = _load()
    lib.orc_e4m3_encode.argtypes = [ctypes.c_float]
    lib.orc_e4m3_encode.restype = ctypes.c_uint8
    a = np.asarray(v, np.float32)
    return np.array([lib.orc_e4m3_encode(float(t)) for t in a.reshape(-1)],
                    np.uint8).reshape(a.shape)


def quantize_e4m3_rows(y):
    """Per-row fp8: scale = max|row| / 448 (f32 division; 1 for a zero row),
    codes = e4m3(y / scale).  y: [..., d] float32."""
    ya = np.ascontiguousarray(np.asarray(y, np.float32))
    d = ya.shape[-1]
    rows = ya.size // d
    lib = _load()
    lib.orc_quantize_e4m3_rows.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                           ctypes.c_void_p, ctypes.c_void_p]
    lib.orc_quantize_e4m3_rows.restype = None
    codes = np.empty(ya.shape, np.uint8)
    scales = np.empty(ya.shape[:-1], np.float32)
    lib.orc_quantize_e4m3_rows(_ptr(ya), rows, d, _ptr(codes), _ptr(scales))
    return codes, scales


def index_cache_write(k_new, kv_head, cache, scales=None):
    """The cache after writing the rotated new keys of each sequence at its
    kv_head: rows kv_head[b] .. kv_head[b] + n_new - 1 of sequence b get the
    rotated rows (fp8 codes with their scales when `scales` is given, else
    bf16 bits); rows outside [0, n_cache) are not written; every other row
    keeps its value.  k_new: [B, n_new, d]; cache: [B, n_cache, d] uint8
    (fp8 codes) or uint16 (bf16 bits); scales: [B, n_cache] float32 or None.
    Returns new (cache, scales) arrays."""
    y = hadamard_rows(k_new)
    B, n_new, d = y.shape
    cache = np.array(cache, copy=True)
    scales = None if scales is None else np.array(scales, np.float32, copy=True)
    if scales is not None:
        codes, sc = quantize_e4m3_rows(y)
    else:
        import torch
        bits = torch.from_numpy(y).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    n_cache = cache.shape[1]
    heads = np.asarray(kv_head, np.int64).reshape(B)
    for b in range(B):
        for i in range(n_new):
            r = int(heads[b]) + i
            if 0 <= r < n_cache:
                if scales is not None:
                    cache[b, r] = codes[b, i]
                    scales[b, r] = sc[b, i]
                else:
                    cache[b, r] = bits[b, i]
    return cache, scales


# --------------------------------------------------------------------------
# dense projections ahead of the path: the indexer front-end ("Another DSA
# attempt": the batch-local indexer commit; the CPU crash-fix commit and the
# review on the k_norm eps) and expand_kv ("Module glm5next_dsa_ref":
# expand_kv, linear, layer_norm, and the NoPE invariant).  Plain float64
# numpy; a bf16 input is decoded exactly from its bits.
# --------------------------------------------------------------------------

def _as_f64(a):
    """float64 copy of a numpy array or CPU torch tensor (bf16 decoded from
    its bits: the 16 bits are the top half of the f32 value)."""
    arr, code = _storage(a)
    if code == BF16:
        return (arr.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if code == E4M3:
        raise TypeError("fp8 input is not a projection operand")
    return arr.astype(np.float64)


def linear(x, w):
    """y = x @ w^T ("Module glm5next_dsa_ref" linear: torch Linear layout,
    w [n, k], no bias) over the last axis of x, in float64."""
    xa, wa = _as_f64(x), _as_f64(w)
    assert xa.shape[-1] == wa.shape[1]
    return xa @ wa.T


def layer_norm(x, weight, bias, eps):
    """LayerNorm over the last axis ("Module glm5next_dsa_ref" layer_norm and
    its k_norm invariant: subtract the mean, divide by the standard deviation
    -- population variance, eps added inside the root -- then w * x + b)."""
    xa = _as_f64(x)
    mu = xa.mean(axis=-1, keepdims=True)
    var = ((xa - mu) ** 2).mean(axis=-1, keepdims=True)
    return (xa - mu) / np.sqrt(var + float(eps)) * _as_f64(weight) + _as_f64(bias)


def rope_neox(x, pos, rope_dim, theta):
    """NEOX-style rotary embedding of the first rope_dim entries of the last
    axis ("Another DSA attempt", batch-local indexer commit: the rope part is
    rotated NEOX-style, the rest passes through).  With h = rope_dim / 2,
    entries i and i + h (i < h) form one pair, rotated by the angle
    pos * theta^(-2i / rope_dim).  x: [T, ..., D]; pos: [T]."""
    xa = _as_f64(x).copy()
    h = rope_dim // 2
    assert rope_dim % 2 == 0 and rope_dim <= xa.shape[-1]
    i = np.arange(h, dtype=np.float64)
    inv = float(theta) ** (-2.0 * i / rope_dim)
    p = np.asarray(pos, np.float64).reshape((-1,) + (1,) * (xa.ndim - 1))
    ang = p * inv                                    # [T, 1.., h]
    c, s = np.cos(ang), np.sin(ang)
    a, b = xa[..., :h].copy(), xa[..., h:rope_dim].copy()
    xa[..., :h] = a * c - b * s
    xa[..., h:rope_dim] = b * c + a * s
    return xa


def indexer_frontend(q_lora, x, pos, wq_b, wk, k_norm_w, k_norm_b, w_proj, n_heads,
                     rope_dim, theta, eps):
    """The lightning indexer's inputs from the layer's activations ("Another
    DSA attempt", batch-local indexer commit): q = wq_b(q_lora) per head,
    rope part NEOX-rotated at the token's position, rest unchanged;
    k = LayerNorm-with-bias(wk(x)), rotated the same way (one key head);
    w = weights_proj(x).  The pages split each head vector as rope(64) then
    nope(64) and concatenate in that order, so the rope part is the leading
    rope_dim entries.  Returns float64 (q [T, H, d], k [T, d], w [T, H])."""
    q = linear(q_lora, wq_b)
    T = q.shape[0]
    q = rope_neox(q.reshape(T, n_heads, -1), pos, rope_dim, theta)
    k = rope_neox(layer_norm(linear(x, wk), k_norm_w, k_norm_b, eps), pos, rope_dim, theta)
    w = linear(x, w_proj)
    return q, k, w


def expand_kv(latent, w_kv_b, n_heads, kd, vd):
    """Per-head K and V from the compressed latent ("Module glm5next_dsa_ref"
    expand_kv, NoPE: K is exactly the no-rope head width kd).  The projection
    rows are head-major, each head's kd key rows followed by its vd value
    rows (torch Linear layout w [n_heads * (kd + vd), r]).  latent: [T, r].
    Returns float64 (K [T, H, kd], V [T, H, vd])."""
    y = linear(latent, w_kv_b)
    T = y.shape[0]
    y = y.reshape(T, n_heads, kd + vd)
    return y[..., :kd].copy(), y[..., kd:].copy()
