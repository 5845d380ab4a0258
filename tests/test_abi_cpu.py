"""The C-ABI library on the CPU: it loads, exports every entry point the
header declares, and rejects bad arguments with the documented status before
touching the GPU.  Every call here fails validation by construction (fake
device pointers are never dereferenced)."""
import ctypes
import os
import re

import pytest

import head_attention_sdpa_amd as attn
from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "attn_sdpa.h")
FAKE = 0x10000          # 16-byte aligned, never dereferenced
MISALIGNED = 0x10002


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_0-9]+)\s*\(", text)))


def test_library_loads_and_exports_header_symbols():
    L = attn.lib()
    names = header_functions()
    assert set(names) == set(attn.EXPORTS)
    for name in names:
        assert hasattr(L, name), name


def test_abi_version_matches_header():
    m = re.search(r"#define ATTN_ABI_VERSION (\d+)", open(HEADER).read())
    assert attn.lib().attn_abi_version() == int(m.group(1))


def test_one_hip_runtime_when_the_library_loads_first():
    """Loading the library before anything imports torch still leaves one
    HIP runtime in the process (torch's), checked in a fresh interpreter."""
    import subprocess
    import sys
    code = ("import sys; sys.path.insert(0, %r); import head_attention_sdpa_amd as attn; attn.lib(); "
            "print(repr(attn.hip_runtimes()))" % ROOT)
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr[-2000:]
    runtimes = eval(out.stdout.strip().splitlines()[-1])
    assert len(runtimes) == 1, runtimes


def test_hip_error_reporting():
    L = attn.lib()
    assert L.attn_last_hip_error() == 0   # no ATTN_E_HIP on this thread so far
    assert L.attn_hip_error_str(100).decode()   # HIP's name of hipErrorNoDevice


def test_status_strings():
    for code in (0, -1, -2, -3, -4, -5):
        assert attn.status_str(code) and attn.status_str(code) != "unknown status"
    assert attn.status_str(42) == "unknown status"


def sdpa_call(dt=1, B=2, H=2, nq=8, nkv=8, dk=64, dv=64, q=FAKE, k=FAKE, v=FAKE, o=FAKE,
              sq=None, scale=0.0, mask=0, lse=None):
    sqp = ctypes.byref(sq) if sq is not None else None
    return attn.lib().attn_sdpa_fwd(dt, B, H, nq, nkv, dk, dv, q, sqp, k, None, v, None, o, None,
                                    scale, mask, None, None, lse, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=7), -1),
    (dict(B=0), -1),
    (dict(H=-1), -1),
    (dict(nq=-1), -1),
    (dict(dk=0), -1),
    (dict(q=None), -1),
    (dict(k=None), -1),
    (dict(nkv=0, k=None, v=None, dk=32), -2),  # null K/V allowed when empty
    (dict(o=None), -1),
    (dict(scale=-1.0), -1),
    (dict(scale=float("inf")), -1),
    (dict(scale=float("nan")), -1),
    (dict(mask=3), -1),
    (dict(sq=attn.attn_strides(-8, 64, 64)), -1),
    (dict(dk=32), -2),
    (dict(dv=128), -2),
    (dict(dt=0, dk=65), -2),
    (dict(q=MISALIGNED), -3),
    (dict(o=MISALIGNED), -3),
    (dict(sq=attn.attn_strides(1024, 512, 68)), -3),
    (dict(dt=0, q=MISALIGNED), -3),
    (dict(lse=MISALIGNED), -3),
])
def test_sdpa_validation(kw, code):
    assert sdpa_call(**kw) == code


def mha_call(dt=1, B=1, nq=16, nkv=16, dm=128, H=2, dk=64, dv=64, ws=FAKE, wsb=1 << 30,
             x=FAKE, y=FAKE, scale=0.0, mask=1):
    return attn.lib().attn_mha_fwd(dt, B, nq, nkv, dm, H, dk, dv, x, x, FAKE, FAKE, FAKE, FAKE, y,
                                   scale, mask, None, None, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=5), -1),
    (dict(B=0), -1),
    (dict(x=None), -1),
    (dict(scale=-2.0), -1),
    (dict(mask=9), -1),
    (dict(dt=0), -2),
    # the heads split the model width: h * d_k = h * d_v = d_model
    (dict(dk=32), -1),
    (dict(dm=100), -1),
    (dict(dm=128, H=4), -1),
    (dict(dm=128, H=4, dk=32), -1),
    (dict(dm=128, H=4, dk=32, dv=32), -2),   # a consistent split, but head size 32 is not built
    # the attention step's 32-bit offsets: 87,297 rows of a 64-head fused QKV projection pass 2 GiB
    (dict(nq=87297, nkv=87297, dm=4096, H=64), -2),
    (dict(ws=None), -4),
    (dict(wsb=1024), -4),
    (dict(ws=FAKE + 16), -3),
    (dict(y=MISALIGNED), -3),
])
def test_mha_validation(kw, code):
    assert mha_call(**kw) == code


def test_mha_workspace_bytes():
    L = attn.lib()
    # cfg: 4 x 4096 tokens, d_model 1024, 16 heads: Q, K, V and the concatenation in bf16
    n = L.attn_mha_workspace_bytes(1, 4, 4096, 4096, 1024, 16, 64, 64)
    assert n == 4 * 4096 * 1024 * 2 * 4
    assert L.attn_mha_workspace_bytes(0, 4, 4096, 4096, 1024, 16, 64, 64) == 0  # f32 unsupported
    assert L.attn_mha_workspace_bytes(1, 4, 4096, 4096, 1000, 16, 64, 64) == 0
    assert L.attn_mha_workspace_bytes(1, 0, 4096, 4096, 1024, 16, 64, 64) == 0
    assert L.attn_mha_workspace_bytes(1, 4, 4096, 4096, 1024, 8, 64, 64) == 0   # 8 * 64 != 1024
    assert L.attn_mha_workspace_bytes(1, 4, 4096, 4096, 1024, 16, 64, 32) == 0  # 16 * 32 != 1024
    # rows x 3*64*64*2 bytes per fused projection row: 87,296 rows fit below 2 GiB, 87,297 do not
    assert L.attn_mha_workspace_bytes(1, 1, 87296, 87296, 4096, 64, 64, 64) > 0
    assert L.attn_mha_workspace_bytes(1, 1, 87297, 87297, 4096, 64, 64, 64) == 0
    # keys round up to 64 rows: 87,360 fit, 87,361 do not
    assert L.attn_mha_workspace_bytes(1, 1, 16, 87360, 4096, 64, 64, 64) > 0
    assert L.attn_mha_workspace_bytes(1, 1, 16, 87361, 4096, 64, 64, 64) == 0


def linear_call(dt=1, m=64, k=128, n=256, x=FAKE, ldx=128, w=FAKE, y=FAKE, ldy=256):
    return attn.lib().attn_linear_fwd(dt, m, k, n, x, ldx, w, y, ldy, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=5), -1),
    (dict(m=-1), -1),
    (dict(k=0), -1),
    (dict(n=0), -1),
    (dict(ldx=64), -1),
    (dict(ldy=128), -1),
    (dict(x=None), -1),
    (dict(w=None), -1),
    (dict(y=None), -1),
    (dict(dt=0), -2),
    (dict(k=96, ldx=96), -2),
    (dict(n=12, ldy=16), -2),
    (dict(x=MISALIGNED), -3),
    (dict(y=MISALIGNED), -3),
    (dict(ldx=132), -3),
    (dict(m=0, x=None, w=None, y=None), 0),   # nothing to do: no launch
])
def test_linear_validation(kw, code):
    assert linear_call(**kw) == code


def decode_call(dt=1, B=2, H=2, nq=1, nkv=100, dk=64, dv=64, q=FAKE, k=FAKE, v=FAKE, o=FAKE,
                ws=FAKE, wsb=1 << 30, scale=0.0):
    return attn.lib().attn_decode_fwd(dt, B, H, nq, nkv, dk, dv, q, None, k, None, v, None, o, None,
                                      scale, None, None, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=7), -1),
    (dict(B=0), -1),
    (dict(nkv=-1), -1),
    (dict(q=None), -1),
    (dict(k=None), -1),
    (dict(scale=-1.0), -1),
    (dict(dt=0), -2),
    (dict(nq=33), -2),
    (dict(dk=32), -2),
    (dict(q=MISALIGNED), -3),
    (dict(ws=FAKE + 64), -3),
    (dict(ws=None), -4),
    (dict(wsb=64), -4),
    (dict(nq=0, q=None, o=None), 0),   # nothing to do: no launch
])
def test_decode_validation(kw, code):
    assert decode_call(**kw) == code


def test_decode_workspace_bytes():
    L = attn.lib()
    # 16 x 16 heads, one query, 4096-key cache: 4 chunks of 16 tiles per (b, h)
    # (about 1024 workgroups); fp32 partial O (64 per row) and (m, l) per
    # (b, h, chunk, query)
    rows = 16 * 16 * 4 * 1
    assert L.attn_decode_workspace_bytes(1, 16, 16, 1, 4096, 64, 64) == rows * 64 * 4 + rows * 2 * 4
    assert L.attn_decode_workspace_bytes(0, 16, 16, 1, 4096, 64, 64) == 0   # f32 unsupported
    assert L.attn_decode_workspace_bytes(1, 16, 16, 33, 4096, 64, 64) == 0  # n_q > 32
    assert L.attn_decode_workspace_bytes(1, 16, 16, 1, 4096, 32, 32) == 0
    assert L.attn_decode_workspace_bytes(1, 1, 1, 1, 0, 64, 64) > 0         # empty cache: one chunk


def test_sdpa_window_validation():
    L = attn.lib()
    s = attn.attn_strides(64 * 128, 64 * 128, 64)
    args = (1, 1, 1, 128, 128, 64, 64, FAKE, None, FAKE, None, FAKE, None, FAKE, None, 0.0, 0)
    assert L.attn_sdpa_window_fwd(*args, -1, None, None, None, None) == -1          # negative radius
    assert L.attn_sdpa_window_fwd(1, 1, 1, 128, 128, 32, 32, *args[7:], 4, None, None, None, None) == -2
    assert L.attn_sdpa_window_fwd(*args[:7], MISALIGNED, *args[8:], 4, None, None, None, None) == -3


def bwd_call(dt=1, B=2, H=2, nq=100, nkv=100, dk=64, dv=64, q=FAKE, k=FAKE, v=FAKE, o=FAKE, do=FAKE,
             lse=FAKE, dq=FAKE, dk_=FAKE, dv_=FAKE, sdo=None, mask=1, ws=FAKE, wsb=1 << 30, scale=0.0):
    return attn.lib().attn_sdpa_bwd(dt, B, H, nq, nkv, dk, dv, q, None, k, None, v, None, o, None,
                                    do, sdo, lse, dq, None, dk_, None, dv_, None, scale, mask, None, None,
                                    ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=7), -1),
    (dict(B=0), -1),
    (dict(nq=-1), -1),
    (dict(mask=2), -1),
    (dict(q=None), -1),
    (dict(do=None), -1),
    (dict(lse=None), -1),
    (dict(dq=None), -1),
    (dict(dk_=None), -1),
    (dict(dv_=None), -1),
    (dict(scale=float("nan")), -1),
    (dict(sdo=attn.attn_strides(-1, 64, 64)), -1),
    (dict(dt=0), -2),
    (dict(dk=32, dv=32), -2),
    (dict(sdo=attn.attn_strides(64 * 100, 64 * 100, 32)), -2),  # dO rows overlap
    (dict(do=MISALIGNED), -3),
    (dict(dv_=MISALIGNED), -3),
    (dict(lse=FAKE + 2), -3),
    (dict(sdo=attn.attn_strides(64 * 100, 64 * 100, 68)), -3),
    (dict(ws=FAKE + 64), -3),
    (dict(ws=None), -4),
    (dict(wsb=2 * 2 * 100 * 8 - 1), -4),
    (dict(nq=0, nkv=0, q=None, k=None, v=None, o=None, do=None, lse=None, dq=None, dk_=None, dv_=None,
          ws=None, wsb=0), 0),   # nothing to do: no launch
])
def test_bwd_validation(kw, code):
    assert bwd_call(**kw) == code


def test_bwd_workspace_bytes():
    L = attn.lib()
    # one (lse in log2 units, D) fp32 pair per query row, rounded up to 256 bytes
    assert L.attn_sdpa_bwd_workspace_bytes(1, 4, 16, 4096, 4096, 64, 64) == 4 * 16 * 4096 * 8
    assert L.attn_sdpa_bwd_workspace_bytes(1, 1, 1, 3, 5, 64, 64) == 256
    assert L.attn_sdpa_bwd_workspace_bytes(1, 1, 1, 0, 5, 64, 64) == 0
    assert L.attn_sdpa_bwd_workspace_bytes(0, 1, 1, 3, 5, 64, 64) == 0      # f32 unsupported
    assert L.attn_sdpa_bwd_workspace_bytes(1, 1, 1, 3, 5, 32, 32) == 0


def block_call(dt=1, B=2, nq=64, nkv=64, dm=256, H=4, dk=64, dv=64, xq=FAKE, xkv=FAKE, pe=1, g=FAKE,
               b=FAKE, eps=1e-5, y=FAKE, mask=1, ws=FAKE, wsb=1 << 30, scale=0.0):
    return attn.lib().attn_mha_block_fwd(dt, B, nq, nkv, dm, H, dk, dv, xq, xkv, pe, FAKE, FAKE, FAKE, FAKE,
                                         g, b, eps, y, scale, mask, None, None, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=7), -1),
    (dict(B=0), -1),
    (dict(mask=3), -1),
    (dict(g=None), -1),
    (dict(y=None), -1),
    (dict(pe=2), -1),
    (dict(xkv=FAKE + 4096), -1),             # encoding on a cross-attention sublayer
    (dict(nkv=32), -1),                      # self-attention with n_kv != n_q
    (dict(eps=0.0), -1),
    (dict(eps=float("inf")), -1),
    (dict(scale=-1.0), -1),
    (dict(dt=0), -2),
    (dict(dm=320, H=5), -2),                 # d_model outside {256, 512, 768, 1024}
    (dict(dm=320), -1),                      # 4 heads of 64 are not 320 wide
    (dict(dm=2048, H=32), -2),
    (dict(dk=32, dv=32), -1),                # 4 heads of 32 are not 256 wide
    (dict(dk=32, dv=32, H=8), -2),           # 8 heads of 32 are, but head size 32 is not built
    (dict(g=MISALIGNED), -3),
    (dict(ws=FAKE + 64), -3),
    (dict(ws=None), -4),
    (dict(wsb=1024), -4),
    (dict(nq=0, nkv=0), 0),                  # no output rows: nothing to do
])
def test_mha_block_validation(kw, code):
    assert block_call(**kw) == code


def test_mha_block_workspace_bytes():
    L = attn.lib()
    # the MHA regions (Q | K | V and the concatenation, bf16) plus h with the encoding
    base = L.attn_mha_workspace_bytes(1, 4, 4096, 4096, 1024, 16, 64, 64)
    assert L.attn_mha_block_workspace_bytes(1, 4, 4096, 4096, 1024, 16, 64, 64, 0) == base
    assert L.attn_mha_block_workspace_bytes(1, 4, 4096, 4096, 1024, 16, 64, 64, 1) == base + 4 * 4096 * 1024 * 2
    assert L.attn_mha_block_workspace_bytes(1, 4, 4096, 4096, 320, 5, 64, 64, 0) == 0


# ---------------------------------------------------------------------------
# The binding checks every tensor whose pointer it passes against the shape,
# dtype and device the call implies, before anything reaches the library (a
# smaller or mistyped out, cache or weight would be written or read past its
# end).  The shape checks come first, so CPU tensors exercise them here.
# ---------------------------------------------------------------------------
def _t(*shape, dtype=None):
    import torch
    return torch.zeros(shape, dtype=dtype or torch.bfloat16)


def test_binding_sdpa_checks_out():
    q = _t(2, 3, 10, 64)
    with pytest.raises(ValueError, match="out must be"):
        attn.sdpa(q, q, q, out=_t(2, 3, 9, 64))
    import torch
    with pytest.raises(ValueError, match="out must be"):
        attn.sdpa(q, q, q, out=_t(2, 3, 10, 64, dtype=torch.float32))
    with pytest.raises(ValueError, match="on the GPU"):
        attn.sdpa(q, q, q, out=_t(2, 3, 10, 64))


def test_binding_decode_checks_caches_and_out():
    q = _t(2, 3, 1, 64)
    cache = _t(2, 3, 100, 64)
    with pytest.raises(ValueError, match="k_cache"):
        attn.decode(q, _t(2, 4, 100, 64), cache)
    with pytest.raises(ValueError, match="k_cache"):
        attn.decode(q, _t(1, 3, 100, 64), cache)
    with pytest.raises(ValueError, match="v_cache"):
        attn.decode(q, cache, _t(2, 3, 99, 64))
    with pytest.raises(ValueError, match="out"):
        attn.decode(q, cache, cache, out=_t(2, 3, 2, 64))
    with pytest.raises(ValueError, match="on the GPU"):
        attn.decode(q, cache, cache)


def _mha_operands(B=2, n_q=8, n_kv=6, dm=128, heads=2):
    x, xkv = _t(B, n_q, dm), _t(B, n_kv, dm)
    w = [_t(dm, dm) for _ in range(4)]
    return x, xkv, w, heads


@pytest.mark.parametrize("bad,match", [
    ("w_q", "w_q"), ("w_k", "w_k"), ("w_v", "w_v"), ("w_o", "w_o"), ("x_kv", "x_kv"), ("out", "out"),
    ("heads", "multiple of heads"),
])
def test_binding_mha_checks_operands(bad, match):
    x, xkv, w, heads = _mha_operands()
    kw = {}
    if bad == "x_kv":
        xkv = _t(2, 6, 64)
    elif bad == "out":
        kw["out"] = _t(2, 8, 64)
    elif bad == "heads":
        heads = 3
    else:
        w[("w_q", "w_k", "w_v", "w_o").index(bad)] = _t(128, 64)
    with pytest.raises(ValueError, match=match):
        attn.mha(x, xkv, *w, heads=heads, **kw)
    x, xkv, w, heads = _mha_operands(dm=256, heads=4)
    g = _t(256)
    if bad in ("w_q", "w_k", "w_v", "w_o"):
        w[("w_q", "w_k", "w_v", "w_o").index(bad)] = _t(256, 128)
        with pytest.raises(ValueError, match=match):
            attn.mha_block(x, *w, g, g, heads=4, x_kv=xkv)
    with pytest.raises(ValueError, match="ln_gamma"):
        attn.mha_block(x, *_mha_operands(dm=256, heads=4)[2], _t(128), g, heads=4)


def test_binding_mha_reaches_gpu_check_when_consistent():
    x, xkv, w, heads = _mha_operands()
    with pytest.raises(ValueError, match="on the GPU"):
        attn.mha(x, xkv, *w, heads=heads)


def test_binding_bwd_checks_gradients():
    q = _t(1, 2, 10, 64)
    k = _t(1, 2, 12, 64)
    import torch
    lse = torch.zeros((1, 2, 10), dtype=torch.float32)
    for name, bad in (("dq", _t(1, 2, 12, 64)), ("dk", _t(1, 2, 10, 64)), ("dv", _t(1, 2, 12, 32))):
        with pytest.raises(ValueError, match=name):
            attn.sdpa_bwd(q, k, k, q, lse, q, **{name: bad})
    with pytest.raises(ValueError, match="on the GPU"):
        attn.sdpa_bwd(q, k, k, q, lse, q)


def test_bwd_noalloc_rejects_sizes_beyond_its_scratch():
    """attn_sdpa_bwd_noalloc keeps its per-row terms in a fixed 16 MiB array
    (8 bytes per query row): 2,097,152 rows of batch*heads*n_q at most.  One
    row more is refused with ATTN_E_WORKSPACE before any HIP call (so this
    runs without a GPU); argument errors come first, as in attn_sdpa_bwd."""
    L = attn.lib()

    def call(B, H, n_q, dt=1, lse=FAKE):
        return L.attn_sdpa_bwd_noalloc(dt, B, H, n_q, 64, 64, 64, FAKE, None, FAKE, None, FAKE, None, FAKE, None,
                                       FAKE, None, lse, FAKE, None, FAKE, None, FAKE, None, 0.0, 1, None, None,
                                       None)
    assert call(4, 16, 32769) == -4           # 2,097,216 rows
    assert call(1, 1, 2097153) == -4
    assert call(4, 16, 32769, dt=0) == -2     # f32: unsupported, as in attn_sdpa_bwd
    assert call(4, 16, 32769, lse=None) == -1
