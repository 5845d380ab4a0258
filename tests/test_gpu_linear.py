"""GPU parity of attn_linear_fwd, one projection y = x . W of the multi-head
block (no bias), against the fp64 oracle on identical seeded bf16 inputs.

Tolerance, per element: the GPU rounds the fp32 sum to bf16 once (at most
2^-9 |y| from the fp32 value; 2^-8 |y| allowed) and accumulates K exact
bf16 x bf16 products in fp32 (at most K * 2^-24 * sum_k |x_k w_k| away from
the exact sum, the standard bound for recursive summation).  Covers both GEMM
kernels (256-column panels take the LDS-DMA kernel, other widths the general
one), ragged M, strided x and y (columns beyond n untouched), the full-size
projections of the 4 x 4096 x 1024 block on sampled rows, and m = 0."""
import numpy as np
import pytest

import attn_inputs as gen
import oracle
from gpu_helpers import announce, to_f64, to_gpu

pytestmark = pytest.mark.gpu


def attn_mod():
    import head_attention_sdpa_amd as attn
    attn.lib()
    return attn


def bound(x, w, ref, rows=None):
    K = x.shape[1]
    absprod = oracle.linear(np.abs(x), np.abs(w), rows=rows)
    return 2.0 ** -8 * np.abs(ref) + K * 2.0 ** -24 * absprod


def check(gpu, ref, tol, what):
    err = np.abs(gpu - ref)
    worst = float((err - tol).max()) if err.size else -1.0
    print(f"{what}: max err {float(err.max()) if err.size else 0.0:.3e}", flush=True)
    assert worst <= 0.0, f"{what}: error above the bound by {worst:.3e}"


CASES = [
    dict(name="dma_kernel_ragged_m", M=300, K=256, N=512),
    dict(name="dma_kernel_k32_steps", M=256, K=1024, N=256),
    dict(name="general_kernel", M=77, K=64, N=200),
    dict(name="general_kernel_n8", M=5, K=128, N=8),
]


@pytest.mark.parametrize("c", CASES, ids=[c["name"] for c in CASES])
def test_linear_vs_oracle(c):
    import torch
    attn = attn_mod()
    M, K, N = c["M"], c["K"], c["N"]
    x = gen.to_dtype(gen.normal(7000 + M, (M, K)), "bf16")
    w = gen.to_dtype(gen.xavier_uniform(7001 + N, K, N), "bf16")
    announce(f"linear {c['name']} M={M} K={K} N={N}")
    y = attn.linear(to_gpu(gen.bf16_bits(x), "bf16"), to_gpu(gen.bf16_bits(w), "bf16"))
    torch.cuda.synchronize()
    ref = oracle.linear(x, w)
    check(to_f64(y), ref, bound(x, w, ref), c["name"])


def test_linear_strided_rows_and_untouched_columns():
    """x read with a row stride of 320 elements, y written with a row stride of
    264: only the m x n block of y changes; the canary columns stay."""
    import torch
    attn = attn_mod()
    M, K, N = 300, 256, 256
    xbuf = gen.to_dtype(gen.normal(7100, (M, 320)), "bf16")
    w = gen.to_dtype(gen.xavier_uniform(7101, K, N), "bf16")
    announce("linear strided x/y with canaries")
    xg = to_gpu(gen.bf16_bits(xbuf), "bf16")
    yg = torch.full((M, 264), -7.0, dtype=torch.bfloat16, device=xg.device)
    attn.linear(xg[:, :K], to_gpu(gen.bf16_bits(w), "bf16"), out=yg[:, :N])
    torch.cuda.synchronize()
    yb = to_f64(yg)
    ref = oracle.linear(xbuf[:, :K], w)
    check(yb[:, :N], ref, bound(xbuf[:, :K], w, ref), "strided")
    assert np.all(yb[:, N:] == -7.0)


@pytest.mark.parametrize("which", ["qkv", "wo"])
def test_linear_full_size_block_projections(which):
    """The projections of the 4 x 4096 x 1024, h = 16 block at full size, in the
    launch configuration the block uses (one call per projection), checked on
    96 sampled rows: X [16384, 1024] . [W^Q | W^K | W^V] [1024, 3072], and an
    activation-like A [16384, 1024] . W^O [1024, 1024]."""
    import torch
    attn = attn_mod()
    inp = gen.config(5)
    B, n, dm = inp.x.shape
    if which == "qkv":
        x = inp.x.reshape(B * n, dm)
        w = np.concatenate([inp.w_q, inp.w_k, inp.w_v], axis=1)
    else:
        x = gen.to_dtype(0.5 * gen.normal(7200, (B * n, dm)), "bf16")
        w = inp.w_o
    announce(f"linear full-size {which} {x.shape} x {w.shape}")
    y = attn.linear(to_gpu(gen.bf16_bits(x), "bf16"), to_gpu(gen.bf16_bits(np.ascontiguousarray(w)), "bf16"))
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, B * n, 173), [0, 255, 256, B * n - 1]]))[:96]
    ref = oracle.linear(x, w, rows=rows)
    yg = to_f64(y)[rows]
    check(yg, ref, bound(x, w, ref, rows=rows), f"full {which}")


def test_linear_empty():
    import torch
    attn = attn_mod()
    announce("linear m=0")
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda:0")
    w = torch.zeros((64, 8), dtype=torch.bfloat16, device="cuda:0")
    y = attn.linear(x, w)
    assert y.shape == (0, 8)


@pytest.mark.parametrize("M,K,N", [(300, 256, 512), (256, 1024, 256), (77, 64, 200)])
def test_one_hot_rows_select_weight_rows_exactly(M, K, N):
    """x with one 1 per row (row i selects weight row (7 i) mod K): every
    product but one is an exact zero and the sum is that weight entry, so y
    equals the selected rows of W bit for bit, on both GEMM kernels."""
    import torch
    attn = attn_mod()
    announce(f"linear one-hot rows M={M} K={K} N={N}")
    sel = (7 * np.arange(M)) % K
    x = np.zeros((M, K))
    x[np.arange(M), sel] = 1.0
    w = gen.to_dtype(gen.xavier_uniform(7100 + N, K, N) * 3.0, "bf16")
    wg = to_gpu(gen.bf16_bits(w), "bf16")
    y = attn.linear(to_gpu(gen.bf16_bits(x), "bf16"), wg)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), wg[torch.from_numpy(sel).to(wg.device)].view(torch.int16))
