"""MI355X (gfx950) scaled dot-product and multi-head attention.

A thin ctypes binding over the C ABI in include/attn_sdpa.h (libattn_sdpa.so
in this package directory).  This module only marshals arguments: every step
of the computation runs in the library's HIP kernels.  PyTorch supplies the
device memory and the current stream.  If the library is missing the calls
raise; there is no fallback path.

    sdpa(q, k, v, scale=None, causal=False, seqlens_q=None, seqlens_kv=None,
         return_lse=False, out=None)
        q [B,H,n_q,d_k], k [B,H,n_kv,d_k], v [B,H,n_kv,d_v] on the GPU, bf16 or
        float32, last dimension contiguous.  Scaled dot-product attention,
        "Attention Is All You Need" section 3.2.1 Eq. 1.

    mha(x_q, x_kv, w_q, w_k, w_v, w_o, heads, ...)
        Multi-head attention block, section 3.2.2 (no bias, Y = X.W).
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn_sdpa.so")

ATTN_F32, ATTN_BF16 = 0, 1
ATTN_MASK_NONE, ATTN_MASK_CAUSAL = 0, 1
STATUS = {0: "ATTN_OK", -1: "ATTN_E_INVALID", -2: "ATTN_E_UNSUPPORTED", -3: "ATTN_E_ALIGN",
          -4: "ATTN_E_WORKSPACE", -5: "ATTN_E_HIP"}

# every entry point that include/attn_sdpa.h declares
EXPORTS = ("attn_sdpa_fwd", "attn_sdpa_window_fwd", "attn_mha_workspace_bytes", "attn_mha_fwd", "attn_decode_workspace_bytes",
           "attn_decode_fwd", "attn_linear_fwd", "attn_mha_block_workspace_bytes", "attn_mha_block_fwd",
           "attn_sdpa_bwd_workspace_bytes", "attn_sdpa_bwd", "attn_sdpa_bwd_noalloc",
           "attn_status_str", "attn_last_hip_error", "attn_hip_error_str", "attn_abi_version")


class AttnError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({msg})")
        self.status = status


class attn_strides(ctypes.Structure):
    _fields_ = [("b", ctypes.c_int64), ("h", ctypes.c_int64), ("n", ctypes.c_int64)]


_lib = None


def hip_runtimes() -> list:
    """Files of the HIP runtime (libamdhip64) mapped into this process."""
    try:
        with open("/proc/self/maps") as f:
            return sorted({line.split()[-1] for line in f if "libamdhip64" in line})
    except OSError:
        return []


def lib() -> ctypes.CDLL:
    """The loaded C-ABI library (raises if it has not been built).

    torch is imported first: the library's libamdhip64.so.7 dependency then
    resolves to the HIP runtime torch has already loaded, so torch's memory
    and streams and the library's kernels live in one runtime.  (Loaded the
    other way round, the process holds two HIP and two HSA runtimes, one from
    the ROCm installation and one shipped with torch, and the library's runtime
    has reported hipErrorNoDevice at its first launch.)  Raises if more than
    one HIP runtime is mapped after loading."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m head_attention_sdpa_amd.build` (or __graft_entry__.build())")
        import torch  # noqa: F401  (its HIP runtime first, see above)
        L = ctypes.CDLL(LIB_PATH)
        rts = hip_runtimes()
        if len(rts) > 1:
            raise ImportError(f"more than one HIP runtime is loaded in this process ({rts}): load torch "
                              "before any other HIP library so that libattn_sdpa.so binds to torch's runtime")
        i, vp, sp = ctypes.c_int, ctypes.c_void_p, ctypes.POINTER(attn_strides)
        L.attn_sdpa_fwd.argtypes = [i, i, i, i, i, i, i, vp, sp, vp, sp, vp, sp, vp, sp,
                                    ctypes.c_float, i, vp, vp, vp, vp]
        L.attn_sdpa_fwd.restype = i
        L.attn_sdpa_window_fwd.argtypes = [i, i, i, i, i, i, i, vp, sp, vp, sp, vp, sp, vp, sp,
                                           ctypes.c_float, i, i, vp, vp, vp, vp]
        L.attn_sdpa_window_fwd.restype = i
        L.attn_mha_workspace_bytes.argtypes = [i, i, i, i, i, i, i, i]
        L.attn_mha_workspace_bytes.restype = ctypes.c_size_t
        L.attn_mha_fwd.argtypes = [i, i, i, i, i, i, i, i, vp, vp, vp, vp, vp, vp, vp,
                                   ctypes.c_float, i, vp, vp, vp, ctypes.c_size_t, vp]
        L.attn_mha_fwd.restype = i
        L.attn_decode_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
        L.attn_decode_workspace_bytes.restype = ctypes.c_size_t
        L.attn_decode_fwd.argtypes = [i, i, i, i, i, i, i, vp, sp, vp, sp, vp, sp, vp, sp, ctypes.c_float,
                                      vp, vp, vp, ctypes.c_size_t, vp]
        L.attn_decode_fwd.restype = i
        L.attn_linear_fwd.argtypes = [i, i, i, i, vp, ctypes.c_int64, vp, vp, ctypes.c_int64, vp]
        L.attn_linear_fwd.restype = i
        L.attn_mha_block_workspace_bytes.argtypes = [i, i, i, i, i, i, i, i, i]
        L.attn_mha_block_workspace_bytes.restype = ctypes.c_size_t
        L.attn_mha_block_fwd.argtypes = [i, i, i, i, i, i, i, i, vp, vp, i, vp, vp, vp, vp, vp, vp,
                                         ctypes.c_float, vp, ctypes.c_float, i, vp, vp, vp, ctypes.c_size_t, vp]
        L.attn_mha_block_fwd.restype = i
        L.attn_sdpa_bwd_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
        L.attn_sdpa_bwd_workspace_bytes.restype = ctypes.c_size_t
        L.attn_sdpa_bwd.argtypes = [i, i, i, i, i, i, i, vp, sp, vp, sp, vp, sp, vp, sp, vp, sp, vp,
                                    vp, sp, vp, sp, vp, sp, ctypes.c_float, i, vp, vp, vp,
                                    ctypes.c_size_t, vp]
        L.attn_sdpa_bwd.restype = i
        L.attn_sdpa_bwd_noalloc.argtypes = [i, i, i, i, i, i, i, vp, sp, vp, sp, vp, sp, vp, sp, vp, sp, vp,
                                            vp, sp, vp, sp, vp, sp, ctypes.c_float, i, vp, vp, vp]
        L.attn_sdpa_bwd_noalloc.restype = i
        L.attn_status_str.argtypes = [i]
        L.attn_status_str.restype = ctypes.c_char_p
        L.attn_abi_version.argtypes = []
        L.attn_abi_version.restype = i
        L.attn_last_hip_error.argtypes = []
        L.attn_last_hip_error.restype = i
        L.attn_hip_error_str.argtypes = [i]
        L.attn_hip_error_str.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().attn_status_str(status).decode()


def _check(fn: str, rc: int):
    if rc != 0:
        msg = status_str(rc)
        if rc == -5:  # ATTN_E_HIP: name the HIP error behind it
            e = lib().attn_last_hip_error()
            msg += f"; HIP error {e}: {lib().attn_hip_error_str(e).decode()}"
        raise AttnError(fn, rc, msg)


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float32:
        return ATTN_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _strides4(t) -> attn_strides:
    if t.dim() == 4 and t.numel() == 0:  # empty: torch may report any strides
        _, H, n, d = t.shape
        return attn_strides(H * n * d, n * d, d)
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError("expected a [B,H,n,d] tensor with a contiguous last dimension")
    return attn_strides(t.stride(0), t.stride(1), t.stride(2))


def _lens_ptr(lens, batch, device):
    if lens is None:
        return None
    torch = _torch()
    if not (isinstance(lens, torch.Tensor) and lens.dtype == torch.int32 and lens.device == device
            and lens.is_contiguous() and lens.shape == (batch,)):
        raise ValueError("lengths must be a contiguous int32 [batch] tensor on the same device")
    return lens.data_ptr()


def _expect(t, shape, dtype, device, what):
    """t must have exactly this shape, dtype and device (checked before any
    pointer reaches the library: a smaller or mistyped tensor would be
    written or read past its end)."""
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or t.device != device:
        raise ValueError(f"{what} must be {dtype} {tuple(shape)} on {device}; got {t.dtype} "
                         f"{tuple(t.shape)} on {t.device}")


def _on_gpu(t):
    if t.device.type != "cuda":
        raise ValueError("tensors must be on the GPU")


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def sdpa(q, k, v, scale=None, causal=False, seqlens_q=None, seqlens_kv=None, return_lse=False,
         out=None, stream=None, window=None):
    """Scaled dot-product attention forward on the GPU (see module docstring).
    window r (optional): restricted attention, only keys with |i - j| <= r.
    Returns o [B,H,n_q,d_v] (and lse [B,H,n_q] fp32 if return_lse)."""
    torch = _torch()
    B, H, n_q, d_k = q.shape
    n_kv, d_v = k.shape[2], v.shape[3]
    if k.shape != (B, H, n_kv, d_k) or v.shape != (B, H, n_kv, d_v):
        raise ValueError("shape mismatch between q, k, v")
    if not (q.dtype == k.dtype == v.dtype) or not (q.device == k.device == v.device):
        raise ValueError("q, k, v must share dtype and device")
    if out is not None:
        _expect(out, (B, H, n_q, d_v), q.dtype, q.device, "out")
    _on_gpu(q)
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty((B, H, n_q, d_v), dtype=q.dtype, device=q.device)
    lse = torch.empty((B, H, n_q), dtype=torch.float32, device=q.device) if return_lse else None
    sq, sk, sv, so = _strides4(q), _strides4(k), _strides4(v), _strides4(out)
    common = (q.data_ptr(), ctypes.byref(sq), k.data_ptr(), ctypes.byref(sk),
              v.data_ptr(), ctypes.byref(sv), out.data_ptr(), ctypes.byref(so),
              0.0 if scale is None else float(scale), ATTN_MASK_CAUSAL if causal else ATTN_MASK_NONE)
    tail = (_lens_ptr(seqlens_q, B, q.device), _lens_ptr(seqlens_kv, B, q.device),
            None if lse is None else lse.data_ptr(), _stream(stream))
    if window is None:
        rc = lib().attn_sdpa_fwd(dt, B, H, n_q, n_kv, d_k, d_v, *common, *tail)
        _check("attn_sdpa_fwd", rc)
    else:
        rc = lib().attn_sdpa_window_fwd(dt, B, H, n_q, n_kv, d_k, d_v, *common, int(window), *tail)
        _check("attn_sdpa_window_fwd", rc)
    return (out, lse) if return_lse else out


def mha_workspace_bytes(batch, n_q, n_kv, d_model, heads, d_k=64, d_v=64, dtype=ATTN_BF16) -> int:
    return int(lib().attn_mha_workspace_bytes(dtype, batch, n_q, n_kv, d_model, heads, d_k, d_v))


def _check_projections(x_q, x_kv, w_q, w_k, w_v, w_o, heads, out, fn):
    """Shapes of the multi-head block's operands: x_kv [B, n_kv, d_model],
    w_q/w_k/w_v [d_model, heads*d_k], w_o [heads*d_v, d_model] with
    heads*d_k = heads*d_v = d_model (d_k = d_v = d_model/h, "Attention Is All
    You Need" section 3.2.2), out [B, n_q, d_model]; all contiguous, one
    dtype and device.  Returns (d_k, d_v)."""
    if x_q.dim() != 3 or x_kv.dim() != 3:
        raise ValueError(f"{fn}: x_q and x_kv must be [batch, n, d_model]")
    B, n_q, d_model = x_q.shape
    if heads < 1 or d_model % heads != 0:
        raise ValueError(f"{fn}: d_model = {d_model} is not a multiple of heads = {heads}")
    d_k = d_v = d_model // heads
    hd = heads * d_k
    want = {"x_kv": (x_kv, (B, x_kv.shape[1], d_model)), "w_q": (w_q, (d_model, hd)),
            "w_k": (w_k, (d_model, hd)), "w_v": (w_v, (d_model, hd)), "w_o": (w_o, (hd, d_model))}
    if out is not None:
        want["out"] = (out, (B, n_q, d_model))
    for name, (t, shape) in want.items():
        _expect(t, shape, x_q.dtype, x_q.device, f"{fn}: {name}")
        if not t.is_contiguous():
            raise ValueError(f"{fn}: {name} must be contiguous")
    if not x_q.is_contiguous():
        raise ValueError(f"{fn}: x_q must be contiguous")
    return d_k, d_v


def mha(x_q, x_kv, w_q, w_k, w_v, w_o, heads, scale=None, causal=False, seqlens_q=None,
        seqlens_kv=None, out=None, workspace=None, stream=None):
    """Multi-head attention block forward on the GPU (bf16, d_k = d_v = 64).
    x_q [B,n_q,d_model], x_kv [B,n_kv,d_model] (pass x_q itself for
    self-attention); w_q/w_k/w_v [d_model, heads*64], w_o [heads*64, d_model].
    Returns y [B,n_q,d_model]."""
    torch = _torch()
    B, n_q, d_model = x_q.shape
    n_kv = x_kv.shape[1]
    d_k, d_v = _check_projections(x_q, x_kv, w_q, w_k, w_v, w_o, heads, out, "mha")
    _on_gpu(x_q)
    dt = _dtype_code(x_q)
    nbytes = mha_workspace_bytes(B, n_q, n_kv, d_model, heads, d_k, d_v, dt)
    if nbytes == 0:
        raise AttnError("attn_mha_workspace_bytes", -2, "unsupported sizes")
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=x_q.device)
    if out is None:
        out = torch.empty((B, n_q, d_model), dtype=x_q.dtype, device=x_q.device)
    rc = lib().attn_mha_fwd(dt, B, n_q, n_kv, d_model, heads, d_k, d_v,
                            x_q.data_ptr(), x_kv.data_ptr(), w_q.data_ptr(), w_k.data_ptr(),
                            w_v.data_ptr(), w_o.data_ptr(), out.data_ptr(),
                            0.0 if scale is None else float(scale),
                            ATTN_MASK_CAUSAL if causal else ATTN_MASK_NONE,
                            _lens_ptr(seqlens_q, B, x_q.device), _lens_ptr(seqlens_kv, B, x_q.device),
                            workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                            _stream(stream))
    _check("attn_mha_fwd", rc)
    return out


def mha_block_workspace_bytes(batch, n_q, n_kv, d_model, heads, add_pe, d_k=64, d_v=64,
                              dtype=ATTN_BF16) -> int:
    return int(lib().attn_mha_block_workspace_bytes(dtype, batch, n_q, n_kv, d_model, heads, d_k, d_v,
                                                    int(bool(add_pe))))


def mha_block(x_q, w_q, w_k, w_v, w_o, ln_gamma, ln_beta, heads, x_kv=None, add_pe=False, ln_eps=1e-5,
              scale=None, causal=False, seqlens_q=None, seqlens_kv=None, out=None, workspace=None,
              stream=None):
    """The attention sublayer on the GPU (bf16, d_k = d_v = 64, d_model in
    {256, 512, 768, 1024}): y = LayerNorm(h + MultiHead(h, kv, kv)) with
    h = x_q (+ positional encoding if add_pe) and kv = h (x_kv None:
    self-attention) or x_kv.  Returns y [B, n_q, d_model]."""
    torch = _torch()
    B, n_q, d_model = x_q.shape
    xkv = x_q if x_kv is None else x_kv
    n_kv = xkv.shape[1]
    d_k, d_v = _check_projections(x_q, xkv, w_q, w_k, w_v, w_o, heads, out, "mha_block")
    for name, t in (("ln_gamma", ln_gamma), ("ln_beta", ln_beta)):
        _expect(t, (d_model,), x_q.dtype, x_q.device, f"mha_block: {name}")
    _on_gpu(x_q)
    dt = _dtype_code(x_q)
    nbytes = mha_block_workspace_bytes(B, n_q, n_kv, d_model, heads, add_pe, d_k, d_v, dt)
    if nbytes == 0:
        raise AttnError("attn_mha_block_workspace_bytes", -2, "unsupported sizes")
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=x_q.device)
    if out is None:
        out = torch.empty((B, n_q, d_model), dtype=x_q.dtype, device=x_q.device)
    rc = lib().attn_mha_block_fwd(dt, B, n_q, n_kv, d_model, heads, d_k, d_v,
                                  x_q.data_ptr(), xkv.data_ptr() or None,
                                  int(bool(add_pe)), w_q.data_ptr(), w_k.data_ptr(), w_v.data_ptr(),
                                  w_o.data_ptr(), ln_gamma.data_ptr(), ln_beta.data_ptr(), float(ln_eps),
                                  out.data_ptr(), 0.0 if scale is None else float(scale),
                                  ATTN_MASK_CAUSAL if causal else ATTN_MASK_NONE,
                                  _lens_ptr(seqlens_q, B, x_q.device), _lens_ptr(seqlens_kv, B, x_q.device),
                                  workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                  _stream(stream))
    _check("attn_mha_block_fwd", rc)
    return out


def decode_workspace_bytes(batch, heads, n_q, n_kv, d_k=64, d_v=64, dtype=ATTN_BF16) -> int:
    return int(lib().attn_decode_workspace_bytes(dtype, batch, heads, n_q, n_kv, d_k, d_v))


def decode(q, k_cache, v_cache, scale=None, seqlens_kv=None, return_lse=False, out=None,
           workspace=None, stream=None):
    """One decoding step over a key/value cache (bf16, head size 64): the n_q
    (<= 32) queries of each sequence are its newest positions and attend to
    the cache up to their own position.  q [B,H,n_q,64], k_cache/v_cache
    [B,H,n_kv,64] (any strides with a contiguous last dimension), seqlens_kv
    int32 [B] cache lengths (None = n_kv).  Returns o (and lse)."""
    torch = _torch()
    B, H, n_q, d_k = q.shape
    n_kv, d_v = k_cache.shape[2], v_cache.shape[3]
    _expect(k_cache, (B, H, n_kv, d_k), q.dtype, q.device, "decode: k_cache")
    _expect(v_cache, (B, H, n_kv, d_v), q.dtype, q.device, "decode: v_cache")
    if out is not None:
        _expect(out, (B, H, n_q, d_v), q.dtype, q.device, "decode: out")
    if workspace is not None and workspace.device != q.device:
        raise ValueError("decode: workspace must be on the device of q")
    _on_gpu(q)
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty((B, H, n_q, d_v), dtype=q.dtype, device=q.device)
    lse = torch.empty((B, H, n_q), dtype=torch.float32, device=q.device) if return_lse else None
    nbytes = decode_workspace_bytes(B, H, max(n_q, 1), n_kv, d_k, d_v, dt)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=q.device)
    sq, sk, sv, so = (_strides4(t) for t in (q, k_cache, v_cache, out))
    rc = lib().attn_decode_fwd(dt, B, H, n_q, n_kv, d_k, d_v,
                               q.data_ptr() or None, ctypes.byref(sq), k_cache.data_ptr() or None,
                               ctypes.byref(sk), v_cache.data_ptr() or None, ctypes.byref(sv),
                               out.data_ptr() or None, ctypes.byref(so),
                               0.0 if scale is None else float(scale), _lens_ptr(seqlens_kv, B, q.device),
                               None if lse is None else lse.data_ptr(), workspace.data_ptr(),
                               workspace.numel() * workspace.element_size(), _stream(stream))
    _check("attn_decode_fwd", rc)
    return (out, lse) if return_lse else out


def linear(x, w, out=None, stream=None):
    """One projection y = x . w (no bias) on the GPU, bf16.  x [m, k] with a
    contiguous last dimension (any row stride), w [k, n] contiguous; returns
    y [m, n] (or writes `out`, any row stride)."""
    torch = _torch()
    if x.dim() != 2 or w.dim() != 2 or x.shape[1] != w.shape[0]:
        raise ValueError("expected x [m, k] and w [k, n]")
    if x.stride(1) != 1 or not w.is_contiguous() or x.device != w.device or x.dtype != w.dtype:
        raise ValueError("x needs a contiguous last dimension, w must be contiguous, same device and dtype")
    m, k = x.shape
    n = w.shape[1]
    if out is None:
        out = torch.empty((m, n), dtype=x.dtype, device=x.device)
    if out.dim() != 2 or out.shape != (m, n) or out.stride(1) != 1 or out.dtype != x.dtype:
        raise ValueError("out must be [m, n] with a contiguous last dimension")
    rc = lib().attn_linear_fwd(_dtype_code(x), m, k, n, x.data_ptr() if m else None, max(x.stride(0), k),
                               w.data_ptr() if m else None, out.data_ptr() if m else None,
                               max(out.stride(0), n), _stream(stream))
    _check("attn_linear_fwd", rc)
    return out


def sdpa_bwd_workspace_bytes(batch, heads, n_q, n_kv, d_k=64, d_v=64, dtype=ATTN_BF16) -> int:
    return int(lib().attn_sdpa_bwd_workspace_bytes(dtype, batch, heads, n_q, n_kv, d_k, d_v))


def sdpa_bwd(q, k, v, o, lse, dout, scale=None, causal=False, seqlens_q=None, seqlens_kv=None,
             dq=None, dk=None, dv=None, workspace=None, stream=None, noalloc=False):
    """Gradients of scaled dot-product attention (bf16, head size 64): given
    the forward's q, k, v, its output o and lse [B,H,n_q] (fp32, contiguous)
    and the gradient dout of o, returns (dq, dk, dv).  scale, causal and the
    lengths must be those of the forward call.  noalloc=True calls
    attn_sdpa_bwd_noalloc (no workspace; the library's fixed per-device
    scratch, B*H*n_q <= 2,097,152; pass dq, dk, dv to allocate nothing here
    either)."""
    torch = _torch()
    B, H, n_q, d_k = q.shape
    n_kv, d_v = k.shape[2], v.shape[3]
    if k.shape != (B, H, n_kv, d_k) or v.shape != (B, H, n_kv, d_v):
        raise ValueError("shape mismatch between q, k, v")
    if o.shape != (B, H, n_q, d_v) or dout.shape != o.shape:
        raise ValueError("o and dout must be [B, H, n_q, d_v]")
    if not (lse.dtype == torch.float32 and lse.is_contiguous() and lse.shape == (B, H, n_q)):
        raise ValueError("lse must be a contiguous fp32 [B, H, n_q] tensor")
    for t in (k, v, o, dout, lse):
        if t.device != q.device:
            raise ValueError("all tensors must be on the same device")
    if not (q.dtype == k.dtype == v.dtype == o.dtype == dout.dtype):
        raise ValueError("q, k, v, o and dout must share one dtype")
    for name, t, like in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if t is not None:
            _expect(t, like.shape, like.dtype, like.device, f"sdpa_bwd: {name}")
    _on_gpu(q)
    dt = _dtype_code(q)
    dq = torch.empty_like(q, memory_format=torch.contiguous_format) if dq is None else dq
    dk = torch.empty_like(k, memory_format=torch.contiguous_format) if dk is None else dk
    dv = torch.empty_like(v, memory_format=torch.contiguous_format) if dv is None else dv
    st = [_strides4(t) for t in (q, k, v, o, dout, dq, dk, dv)]
    ptr = [t.data_ptr() or None for t in (q, k, v, o, dout, dq, dk, dv)]
    if noalloc:
        rc = lib().attn_sdpa_bwd_noalloc(dt, B, H, n_q, n_kv, d_k, d_v,
                                         ptr[0], ctypes.byref(st[0]), ptr[1], ctypes.byref(st[1]),
                                         ptr[2], ctypes.byref(st[2]), ptr[3], ctypes.byref(st[3]),
                                         ptr[4], ctypes.byref(st[4]), lse.data_ptr() or None,
                                         ptr[5], ctypes.byref(st[5]), ptr[6], ctypes.byref(st[6]),
                                         ptr[7], ctypes.byref(st[7]), 0.0 if scale is None else float(scale),
                                         ATTN_MASK_CAUSAL if causal else ATTN_MASK_NONE,
                                         _lens_ptr(seqlens_q, B, q.device), _lens_ptr(seqlens_kv, B, q.device),
                                         _stream(stream))
        _check("attn_sdpa_bwd_noalloc", rc)
        return dq, dk, dv
    nbytes = sdpa_bwd_workspace_bytes(B, H, n_q, n_kv, d_k, d_v, dt)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=q.device)
    rc = lib().attn_sdpa_bwd(dt, B, H, n_q, n_kv, d_k, d_v,
                             ptr[0], ctypes.byref(st[0]), ptr[1], ctypes.byref(st[1]),
                             ptr[2], ctypes.byref(st[2]), ptr[3], ctypes.byref(st[3]),
                             ptr[4], ctypes.byref(st[4]), lse.data_ptr() or None,
                             ptr[5], ctypes.byref(st[5]), ptr[6], ctypes.byref(st[6]),
                             ptr[7], ctypes.byref(st[7]), 0.0 if scale is None else float(scale),
                             ATTN_MASK_CAUSAL if causal else ATTN_MASK_NONE,
                             _lens_ptr(seqlens_q, B, q.device), _lens_ptr(seqlens_kv, B, q.device),
                             workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                             _stream(stream))
    _check("attn_sdpa_bwd", rc)
    return dq, dk, dv
