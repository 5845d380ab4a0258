"""fp64 CPU oracle for scaled dot-product and multi-head attention.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``, never by the product package.
It shares no code with the HIP path.  Functions: ``sdpa``, ``sdpa_rows``,
``mha``, ``mha_rows``, ``linear``, ``decode``, ``sdpa_bwd`` and ``round_bf16``.

The arithmetic lives in ``oracle.c`` (plain C, fp64, one query row at a time,
sums in index order).  This module only marshals numpy arrays through ctypes.
Definitions: "Attention Is All You Need" section 3.2.1 Eq. 1 (scaled
dot-product attention) and section 3.2.2 (multi-head attention), as restated on
the vlmlib.cn summary of 1706.03762 and the rockcohen.cc deep read
(sections 5.1-5.3, 6.3).
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
# A differently built copy of oracle.c (the sanitizer tier loads one built
# with -fsanitize=address,undefined); it is used as given, never rebuilt here.
_LIB_OVERRIDE = os.environ.get("ATTN_ORACLE_LIB")
_lib = None

_D = ctypes.POINTER(ctypes.c_double)
_I = ctypes.POINTER(ctypes.c_int)
_L = ctypes.POINTER(ctypes.c_int64)


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc into liboracle.so (IEEE fp64: no fast-math,
    no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-pthread",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            lib = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
                build(force=True)
            lib = ctypes.CDLL(_LIB_PATH)
        i, d = ctypes.c_int, ctypes.c_double
        lib.oracle_sdpa_f64.argtypes = [i, i, i, i, i, i, _D, _D, _D, _D, _D, d, i, _I, _I, i]
        lib.oracle_sdpa_rows_f64.argtypes = [i, i, i, i, i, i, _D, _D, _D, _L, ctypes.c_int64,
                                             _D, _D, d, i, _I, _I, i]
        lib.oracle_mha_f64.argtypes = [i, i, i, i, i, i, i, _D, _D, _D, _D, _D, _D, _D, d, i,
                                       _I, _I, i, i]
        lib.oracle_mha_rows_f64.argtypes = [i, i, i, i, i, i, i, _D, _D, _D, _D, _D, _D, _L,
                                            ctypes.c_int64, _D, d, i, _I, _I, i, i]
        lib.oracle_sdpa_bwd_f64.argtypes = [i, i, i, i, i, i, _D, _D, _D, _D, _D, _D, _D, d, i, _I, _I, i]
        lib.oracle_sdpa_window_f64.argtypes = [i, i, i, i, i, i, _D, _D, _D, _D, _D, d, i, _I, _I, i, i]
        lib.oracle_decode_f64.argtypes = [i, i, i, i, i, i, _D, _D, _D, _D, _D, d, _I, i]
        lib.oracle_linear_f64.argtypes = [i, i, i, _D, ctypes.c_int64, _L, ctypes.c_int64, _D, _D, i]
        lib.oracle_pe_f64.argtypes = [i, i, _D]
        lib.oracle_layernorm_f64.argtypes = [ctypes.c_int64, i, _D, _D, _D, d, _D]
        lib.oracle_mha_block_f64.argtypes = [i, i, i, i, i, i, i, _D, _D, i, _D, _D, _D, _D, _D, _D, d,
                                             _D, _D, d, i, _I, _I, i]
        lib.oracle_mha_block_rows_f64.argtypes = [i, i, i, i, i, i, i, _D, _D, i, _D, _D, _D, _D, _D,
                                                  _D, d, _L, ctypes.c_int64, _D, _D, d, i, _I, _I, i]
        lib.oracle_round_bf16.argtypes = [d]
        lib.oracle_round_bf16.restype = d
        for f in ("oracle_sdpa_f64", "oracle_sdpa_rows_f64", "oracle_mha_f64", "oracle_mha_rows_f64",
                  "oracle_linear_f64", "oracle_decode_f64", "oracle_sdpa_window_f64",
                  "oracle_sdpa_bwd_f64", "oracle_pe_f64", "oracle_layernorm_f64",
                  "oracle_mha_block_f64", "oracle_mha_block_rows_f64"):
            getattr(lib, f).restype = i
        _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_D)


def _lens(x, batch):
    if x is None:
        return None, None
    a = np.ascontiguousarray(x, dtype=np.int32)
    if a.shape != (batch,):
        raise ValueError("lengths must have shape [batch]")
    return a, a.ctypes.data_as(_I)


def _check(rc: int, what: str):
    if rc == -1:
        raise ValueError(f"{what}: invalid arguments")
    if rc != 0:
        raise MemoryError(f"{what}: out of memory")


def sdpa(q, k, v, scale=None, causal=False, seqlens_q=None, seqlens_kv=None, window=None,
         nthreads=None):
    """Scaled dot-product attention in fp64.

    q [B,H,n_q,d_k], k [B,H,n_kv,d_k], v [B,H,n_kv,d_v] (any float dtype; values
    are taken exactly).  scale None means 1/sqrt(d_k).  window r (optional):
    restricted attention, only keys with |i - j| <= r are legal.  Returns
    (o, lse) with o [B,H,n_q,d_v] and lse [B,H,n_q] (natural log of the softmax
    denominator including the max shift; -inf for rows without a legal key)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, n_q, d_k = q.shape
    n_kv, d_v = k.shape[2], v.shape[3]
    if k.shape != (B, H, n_kv, d_k) or v.shape != (B, H, n_kv, d_v):
        raise ValueError("shape mismatch")
    scale = 1.0 / math.sqrt(d_k) if scale is None else float(scale)
    o = np.empty((B, H, n_q, d_v))
    lse = np.empty((B, H, n_q))
    lq, plq = _lens(seqlens_q, B)
    lk, plk = _lens(seqlens_kv, B)
    if window is None:
        rc = _load().oracle_sdpa_f64(B, H, n_q, n_kv, d_k, d_v, _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                     _ptr(lse), scale, int(bool(causal)), plq, plk,
                                     nthreads or default_threads())
    else:
        rc = _load().oracle_sdpa_window_f64(B, H, n_q, n_kv, d_k, d_v, _ptr(q), _ptr(k), _ptr(v),
                                            _ptr(o), _ptr(lse), scale, int(bool(causal)), plq, plk,
                                            int(window), nthreads or default_threads())
    _check(rc, "oracle_sdpa")
    return o, lse


def sdpa_rows(q, k, v, rows, scale=None, causal=False, seqlens_q=None, seqlens_kv=None,
              nthreads=None):
    """SDPA for selected query rows only.  rows: int array of flat indices
    (b*H + h)*n_q + i.  Returns (o [nrows,d_v], lse [nrows])."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, n_q, d_k = q.shape
    n_kv, d_v = k.shape[2], v.shape[3]
    scale = 1.0 / math.sqrt(d_k) if scale is None else float(scale)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    o = np.empty((len(rows), d_v))
    lse = np.empty(len(rows))
    lq, plq = _lens(seqlens_q, B)
    lk, plk = _lens(seqlens_kv, B)
    rc = _load().oracle_sdpa_rows_f64(B, H, n_q, n_kv, d_k, d_v, _ptr(q), _ptr(k), _ptr(v),
                                      rows.ctypes.data_as(_L), len(rows), _ptr(o), _ptr(lse), scale,
                                      int(bool(causal)), plq, plk, nthreads or default_threads())
    _check(rc, "oracle_sdpa_rows_f64")
    return o, lse


def mha(x_q, x_kv, w_q, w_k, w_v, w_o, heads, scale=None, causal=False, seqlens_q=None,
        seqlens_kv=None, bf16_storage=False, nthreads=None):
    """Multi-head attention block Y = Concat(head_1..head_h) W^O in fp64.

    x_q [B,n_q,d_model], x_kv [B,n_kv,d_model]; w_q, w_k [d_model, heads*d_k];
    w_v [d_model, heads*d_v]; w_o [heads*d_v, d_model] (row-major, Y = X.W, no
    bias).  scale None means 1/sqrt(d_k).  bf16_storage=True rounds the
    projections and the concatenation to bf16 (diagnostic only)."""
    x_q, x_kv = _f64(x_q), _f64(x_kv)
    w_q, w_k, w_v, w_o = _f64(w_q), _f64(w_k), _f64(w_v), _f64(w_o)
    B, n_q, d_model = x_q.shape
    n_kv = x_kv.shape[1]
    d_k = w_q.shape[1] // heads
    d_v = w_v.shape[1] // heads
    if (w_q.shape != (d_model, heads * d_k) or w_k.shape != w_q.shape
            or w_v.shape != (d_model, heads * d_v) or w_o.shape != (heads * d_v, d_model)
            or x_kv.shape != (B, n_kv, d_model)):
        raise ValueError("shape mismatch")
    scale = 1.0 / math.sqrt(d_k) if scale is None else float(scale)
    y = np.empty((B, n_q, d_model))
    lq, plq = _lens(seqlens_q, B)
    lk, plk = _lens(seqlens_kv, B)
    rc = _load().oracle_mha_f64(B, n_q, n_kv, d_model, heads, d_k, d_v, _ptr(x_q), _ptr(x_kv),
                                _ptr(w_q), _ptr(w_k), _ptr(w_v), _ptr(w_o), _ptr(y), scale,
                                int(bool(causal)), plq, plk, int(bool(bf16_storage)),
                                nthreads or default_threads())
    _check(rc, "oracle_mha_f64")
    return y


def mha_rows(x_q, x_kv, w_q, w_k, w_v, w_o, heads, rows, scale=None, causal=False,
             seqlens_q=None, seqlens_kv=None, bf16_storage=False, nthreads=None):
    """MHA for selected output rows only: rows are flat indices b*n_q + i.
    Returns y [nrows, d_model]."""
    x_q, x_kv = _f64(x_q), _f64(x_kv)
    w_q, w_k, w_v, w_o = _f64(w_q), _f64(w_k), _f64(w_v), _f64(w_o)
    B, n_q, d_model = x_q.shape
    n_kv = x_kv.shape[1]
    d_k = w_q.shape[1] // heads
    d_v = w_v.shape[1] // heads
    scale = 1.0 / math.sqrt(d_k) if scale is None else float(scale)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    y = np.empty((len(rows), d_model))
    lq, plq = _lens(seqlens_q, B)
    lk, plk = _lens(seqlens_kv, B)
    rc = _load().oracle_mha_rows_f64(B, n_q, n_kv, d_model, heads, d_k, d_v, _ptr(x_q),
                                     _ptr(x_kv), _ptr(w_q), _ptr(w_k), _ptr(w_v), _ptr(w_o),
                                     rows.ctypes.data_as(_L), len(rows), _ptr(y), scale,
                                     int(bool(causal)), plq, plk, int(bool(bf16_storage)),
                                     nthreads or default_threads())
    _check(rc, "oracle_mha_rows_f64")
    return y


def sdpa_bwd(q, k, v, dout, scale=None, causal=False, seqlens_q=None, seqlens_kv=None, nthreads=None):
    """Gradients of sum(dout * sdpa(q, k, v)) with respect to q, k and v, in
    fp64, from the chain rule through the definition.  Returns (dq, dk, dv)."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, n_q, d_k = q.shape
    n_kv, d_v = k.shape[2], v.shape[3]
    if dout.shape != (B, H, n_q, d_v):
        raise ValueError("dout must match the output shape")
    scale = 1.0 / math.sqrt(d_k) if scale is None else float(scale)
    dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    lq, plq = _lens(seqlens_q, B)
    lk, plk = _lens(seqlens_kv, B)
    rc = _load().oracle_sdpa_bwd_f64(B, H, n_q, n_kv, d_k, d_v, _ptr(q), _ptr(k), _ptr(v), _ptr(dout),
                                     _ptr(dq), _ptr(dk), _ptr(dv), scale, int(bool(causal)), plq, plk,
                                     nthreads or default_threads())
    _check(rc, "oracle_sdpa_bwd_f64")
    return dq, dk, dv


def decode(q, k, v, scale=None, seqlens_kv=None, nthreads=None):
    """One decoding step over a key/value cache in fp64: the n_q queries are
    the newest positions L_kv[b] - n_q + i of each sequence and attend to the
    cache up to their own position (causal, aligned at the end of the cache).
    q [B,H,n_q,d_k], k [B,H,n_kv,d_k], v [B,H,n_kv,d_v]; seqlens_kv [B] or
    None (= n_kv).  Returns (o [B,H,n_q,d_v], lse [B,H,n_q])."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, n_q, d_k = q.shape
    n_kv, d_v = k.shape[2], v.shape[3]
    scale = 1.0 / math.sqrt(d_k) if scale is None else float(scale)
    o = np.empty((B, H, n_q, d_v))
    lse = np.empty((B, H, n_q))
    lk, plk = _lens(seqlens_kv, B)
    rc = _load().oracle_decode_f64(B, H, n_q, n_kv, d_k, d_v, _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                   _ptr(lse), scale, plk, nthreads or default_threads())
    _check(rc, "oracle_decode_f64")
    return o, lse


def linear(x, w, rows=None, nthreads=None):
    """One projection of the multi-head block in fp64, y = x . w (no bias;
    paper section 3.2.2).  x [M_x, K], w [K, N] row-major; rows (optional)
    selects the rows of x to compute.  Returns y [len(rows) or M_x, N]."""
    x, w = _f64(x), _f64(w)
    mx, k = x.shape
    k2, n = w.shape
    if k != k2:
        raise ValueError("inner dimensions differ")
    prow = None
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        prow = rows.ctypes.data_as(_L)
    m = mx if rows is None else len(rows)
    y = np.empty((m, n))
    rc = _load().oracle_linear_f64(m, k, n, _ptr(x), k, prow, mx, _ptr(w), _ptr(y),
                                   nthreads or default_threads())
    _check(rc, "oracle_linear_f64")
    return y


def positional_encoding(n, d_model):
    """Sinusoidal positional encoding [n, d_model] in fp64: sin on even and cos
    on odd columns of pos / 10000^(2i/d_model) (paper section 3.5)."""
    pe = np.empty((n, d_model))
    _check(_load().oracle_pe_f64(n, d_model, _ptr(pe)), "oracle_pe_f64")
    return pe


def layernorm(z, gamma, beta, eps):
    """LayerNorm over the last dimension in fp64 (population variance, eps
    inside the square root), then the gain gamma and bias beta."""
    z = _f64(z)
    d = z.shape[-1]
    gamma, beta = _f64(gamma), _f64(beta)
    if gamma.shape != (d,) or beta.shape != (d,):
        raise ValueError("gamma and beta must have shape [d]")
    y = np.empty_like(z)
    _check(_load().oracle_layernorm_f64(z.size // d, d, _ptr(z), _ptr(gamma), _ptr(beta), float(eps),
                                        _ptr(y)), "oracle_layernorm_f64")
    return y


def _block_args(x_q, x_kv, w_q, w_k, w_v, w_o, gamma, beta, heads):
    x_q = _f64(x_q)
    x_kv = None if x_kv is None else _f64(x_kv)
    w_q, w_k, w_v, w_o = _f64(w_q), _f64(w_k), _f64(w_v), _f64(w_o)
    gamma, beta = _f64(gamma), _f64(beta)
    B, n_q, d_model = x_q.shape
    n_kv = n_q if x_kv is None else x_kv.shape[1]
    d_k = w_q.shape[1] // heads
    d_v = w_v.shape[1] // heads
    if (w_q.shape != (d_model, heads * d_k) or w_k.shape != w_q.shape
            or w_v.shape != (d_model, heads * d_v) or w_o.shape != (heads * d_v, d_model)
            or (x_kv is not None and x_kv.shape != (B, n_kv, d_model))
            or gamma.shape != (d_model,) or beta.shape != (d_model,)):
        raise ValueError("shape mismatch")
    return x_q, x_kv, w_q, w_k, w_v, w_o, gamma, beta, B, n_q, n_kv, d_model, d_k, d_v


def mha_block(x_q, w_q, w_k, w_v, w_o, gamma, beta, heads, x_kv=None, add_pe=False, eps=1e-5,
              scale=None, causal=False, seqlens_q=None, seqlens_kv=None, nthreads=None):
    """The attention sublayer in fp64: h = x_q (+ PE), z = h + MultiHead(h,
    kv, kv) with kv = h (x_kv None: self-attention) or x_kv (cross-attention,
    no PE), y = LayerNorm(z) with gain gamma and bias beta.  Returns (y, z),
    both [B, n_q, d_model]."""
    (x_q, x_kv, w_q, w_k, w_v, w_o, gamma, beta, B, n_q, n_kv, d_model, d_k,
     d_v) = _block_args(x_q, x_kv, w_q, w_k, w_v, w_o, gamma, beta, heads)
    scale = 1.0 / math.sqrt(d_k) if scale is None else float(scale)
    y = np.empty((B, n_q, d_model))
    z = np.empty((B, n_q, d_model))
    lq, plq = _lens(seqlens_q, B)
    lk, plk = _lens(seqlens_kv, B)
    rc = _load().oracle_mha_block_f64(B, n_q, n_kv, d_model, heads, d_k, d_v, _ptr(x_q),
                                      None if x_kv is None else _ptr(x_kv), int(bool(add_pe)),
                                      _ptr(w_q), _ptr(w_k), _ptr(w_v), _ptr(w_o), _ptr(gamma),
                                      _ptr(beta), float(eps), _ptr(y), _ptr(z), scale,
                                      int(bool(causal)), plq, plk, nthreads or default_threads())
    _check(rc, "oracle_mha_block_f64")
    return y, z


def mha_block_rows(x_q, w_q, w_k, w_v, w_o, gamma, beta, heads, rows, x_kv=None, add_pe=False,
                   eps=1e-5, scale=None, causal=False, seqlens_q=None, seqlens_kv=None, nthreads=None):
    """mha_block for selected output rows only (flat indices b*n_q + i).
    Returns (y, z), each [len(rows), d_model]."""
    (x_q, x_kv, w_q, w_k, w_v, w_o, gamma, beta, B, n_q, n_kv, d_model, d_k,
     d_v) = _block_args(x_q, x_kv, w_q, w_k, w_v, w_o, gamma, beta, heads)
    scale = 1.0 / math.sqrt(d_k) if scale is None else float(scale)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    y = np.empty((len(rows), d_model))
    z = np.empty((len(rows), d_model))
    lq, plq = _lens(seqlens_q, B)
    lk, plk = _lens(seqlens_kv, B)
    rc = _load().oracle_mha_block_rows_f64(B, n_q, n_kv, d_model, heads, d_k, d_v, _ptr(x_q),
                                           None if x_kv is None else _ptr(x_kv), int(bool(add_pe)),
                                           _ptr(w_q), _ptr(w_k), _ptr(w_v), _ptr(w_o), _ptr(gamma),
                                           _ptr(beta), float(eps), rows.ctypes.data_as(_L), len(rows),
                                           _ptr(y), _ptr(z), scale, int(bool(causal)), plq, plk,
                                           nthreads or default_threads())
    _check(rc, "oracle_mha_block_rows_f64")
    return y, z


def round_bf16(x: float) -> float:
    """The oracle's own fp64 -> bf16 round-to-nearest-even (storage diagnostic)."""
    return _load().oracle_round_bf16(float(x))
