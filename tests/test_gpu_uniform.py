"""A closed form on the GPU, independent of the oracle: with Q = 0 every
legal score is 0, every weight is exp(0) = 1 (exactly, also after rounding to
bf16), and each output row is the plain mean of the value rows its query may
use (the legal keys: below the key length, not after the query under the
causal mask, within the radius of restricted attention, up to the query's
position for a decoding step).  The GPU sums bf16 value rows in fp32 and
rounds the mean to bf16 once, so |o - mean| <= 2^-8 |mean| + n 2^-24 max|v|."""
import numpy as np
import pytest

import attn_inputs as gen
from gpu_helpers import announce, lens_gpu, to_f64, to_gpu

pytestmark = pytest.mark.gpu


def attn_mod():
    import head_attention_sdpa_amd as attn
    attn.lib()
    return attn


def legal(i, j, causal, Lk, window=None, shift=0):
    """key j is legal for query i (query i sits at position i + shift)"""
    pos = i + shift
    ok = j < Lk
    if causal:
        ok &= j <= pos
    if window is not None:
        ok &= abs(pos - j) <= window
    return ok


def check(o, v, causal, Lq, Lk, window=None, shift=None, what=""):
    B, H, n_q, _ = o.shape
    n_kv = v.shape[2]
    worst = 0.0
    for b in range(B):
        sh = 0 if shift is None else shift[b]
        for i in range(n_q):
            keys = [j for j in range(n_kv) if legal(i, j, causal, Lk[b], window, sh)]
            if (Lq is not None and i >= Lq[b]) or not keys:
                assert np.all(o[b, :, i] == 0.0), f"{what}: row {b},{i} must be zeros"
                continue
            mean = v[b][:, keys].mean(axis=1)                    # [H, d]
            tol = 2.0 ** -8 * np.abs(mean) + len(keys) * 2.0 ** -24 * np.abs(v[b]).max() + 1e-7
            ratio = float((np.abs(o[b, :, i] - mean) / tol).max())
            worst = max(worst, ratio)
            assert ratio <= 1.0, f"{what}: row {b},{i}: error/bound {ratio:.3f}"
    print(f"{what}: max error/bound {worst:.3f}", flush=True)


@pytest.mark.parametrize("name,B,H,n_q,n_kv,causal,window,lens", [
    ("resident_causal", 3, 2, 200, 200, True, None, [200, 131, 64]),
    ("resident_cross_keys", 2, 3, 100, 300, False, None, [300, 77]),
    ("streaming_causal", 2, 2, 700, 700, True, None, [700, 453]),
    ("streaming_cross", 2, 2, 300, 900, False, None, [900, 512]),
    ("restricted_r37", 2, 2, 600, 600, False, 37, [600, 389]),
    ("restricted_causal_r100", 1, 3, 500, 500, True, 100, [500]),
])
def test_zero_queries_average_the_legal_values(name, B, H, n_q, n_kv, causal, window, lens):
    import torch
    attn = attn_mod()
    announce(f"uniform weights: {name}")
    v = gen.to_dtype(gen.normal(777 + n_kv, (B, H, n_kv, 64)), "bf16")
    k = gen.to_dtype(gen.normal(778 + n_kv, (B, H, n_kv, 64)), "bf16")
    q = np.zeros((B, H, n_q, 64))
    Lk = np.array(lens, np.int32)
    Lq = Lk if n_q == n_kv else None
    o = attn.sdpa(to_gpu(gen.bf16_bits(q), "bf16"), to_gpu(gen.bf16_bits(k), "bf16"),
                  to_gpu(gen.bf16_bits(v), "bf16"), causal=causal, window=window,
                  seqlens_q=lens_gpu(Lq), seqlens_kv=lens_gpu(Lk))
    torch.cuda.synchronize()
    check(to_f64(o), v, causal, Lq, Lk, window, what=name)


def test_zero_queries_decode_step():
    import torch
    attn = attn_mod()
    announce("uniform weights: decoding step")
    B, H, n_q, n_kv = 3, 2, 5, 3000
    v = gen.to_dtype(gen.normal(901, (B, H, n_kv, 64)), "bf16")
    k = gen.to_dtype(gen.normal(902, (B, H, n_kv, 64)), "bf16")
    q = np.zeros((B, H, n_q, 64))
    Lk = np.array([3000, 1234, 3], np.int32)
    o = attn.decode(to_gpu(gen.bf16_bits(q), "bf16"), to_gpu(gen.bf16_bits(k), "bf16"),
                    to_gpu(gen.bf16_bits(v), "bf16"), seqlens_kv=lens_gpu(Lk))
    torch.cuda.synchronize()
    # query i of sequence b sits at position Lk[b] - n_q + i and sees keys up to it
    check(to_f64(o), v, True, None, Lk, shift=Lk - n_q, what="decoding step")


@pytest.mark.parametrize("causal", [True, False])
def test_zero_queries_backward(causal):
    """Gradients with Q = 0: the weights of query i are 1/n_i over its n_i
    legal keys, so dK = scale dS^T Q is exactly zero and dV_j = sum over the
    queries i that may use key j of dO_i / n_i.  Bound for dV: the weights
    are recomputed from the forward's lse and rounded to bf16 for the product
    (relative 2^-8 each), plus one bf16 rounding of dV."""
    import torch
    attn = attn_mod()
    announce(f"uniform weights: backward causal={causal}")
    B, H, n = 2, 2, 300
    k = gen.to_dtype(gen.normal(1201, (B, H, n, 64)), "bf16")
    v = gen.to_dtype(gen.normal(1202, (B, H, n, 64)), "bf16")
    do = gen.to_dtype(gen.normal(1203, (B, H, n, 64)), "bf16")
    L = np.array([300, 211], np.int32)
    qg = to_gpu(gen.bf16_bits(np.zeros((B, H, n, 64))), "bf16")
    kg, vg, dog = (to_gpu(gen.bf16_bits(a), "bf16") for a in (k, v, do))
    o, lse = attn.sdpa(qg, kg, vg, causal=causal, seqlens_q=lens_gpu(L), seqlens_kv=lens_gpu(L), return_lse=True)
    dq, dk, dv = attn.sdpa_bwd(qg, kg, vg, o, lse, dog, causal=causal, seqlens_q=lens_gpu(L),
                               seqlens_kv=lens_gpu(L))
    torch.cuda.synchronize()
    assert bool((dk.float() == 0).all()), "dK must be exactly zero when Q = 0"
    dv = to_f64(dv)
    worst = 0.0
    for b in range(B):
        for j in range(n):
            users = [i for i in range(L[b]) if j < L[b] and (not causal or j <= i)]
            if not users:
                assert np.all(dv[b, :, j] == 0.0)
                continue
            cnt = np.array([(i + 1) if causal else L[b] for i in users], dtype=np.float64)
            terms = do[b][:, users] / cnt[None, :, None]          # [H, users, d]
            want = terms.sum(axis=1)
            tol = 2.0 ** -7 * np.abs(terms).sum(axis=1) + 2.0 ** -8 * np.abs(want) + 1e-6
            ratio = float((np.abs(dv[b, :, j] - want) / tol).max())
            worst = max(worst, ratio)
            assert ratio <= 1.0, f"dV row {b},{j}: error/bound {ratio:.3f}"
    print(f"backward causal={causal}: dK exactly 0, dV max error/bound {worst:.3f}", flush=True)
