"""GPU parity of attn_sdpa_bwd (gradients of scaled dot-product attention)
against the fp64 oracle on identical seeded inputs.

The GPU pass gets what a training step gives it: q, k, v, the GPU forward's
o (bf16) and lse, and dO.  The oracle computes the exact gradients of the
same inputs from the chain rule in fp64.

Tolerance, per element, from the arithmetic of the GPU path (u = 2^-9, the
bf16 unit roundoff; fp32 accumulation error is far below it):
  - P is recomputed from the forward's lse, whose row sum was taken over
    bf16-rounded weights: P carries a relative error up to ~u, and is
    rounded to bf16 (u) for dV = P^T dO;
  - D_i = dO_i . O_i uses the bf16 forward output, |O - O_exact| <~ 2u (|O| + P|V|),
    so |dD_i| <= 2u sum_c |dO_ic| (|O_ic| + (P|V|)_ic);
  - dS = P (dP - D) is rounded to bf16 (u) for dK and dQ, on top of P's own
    error (u) and P dD;
  - every gradient is rounded to bf16 once (u).
With the upper bound |dS_ij| <= P_ij (sum_c |dO_ic||V_jc| + |D_i|) =: A_ij:
  |ddV| <= u |dV| + 2u P^T|dO|
  |ddK| <= u |dK| + scale (2u A^T|Q| + (P dD)^T |Q|)
  |ddQ| <= u |dQ| + scale (2u A|K| + dD (P|K|))
The test takes twice these bounds (plus 1e-6) and checks every element; it
prints the largest error/bound ratio.  Gradients of padded rows and keys
must be exactly zero."""
import numpy as np
import pytest

import attn_inputs as gen
import oracle
from gpu_helpers import announce, lens_gpu, to_f64, to_gpu

pytestmark = pytest.mark.gpu

U = 2.0 ** -9


def attn_mod():
    import head_attention_sdpa_amd as attn
    attn.lib()
    return attn


def bounds(q, k, v, g, o_gpu, lse, scale, causal, Lq, Lkv, ref):
    """Per-element bounds of one (b, h) slice (valid rows and keys only)."""
    dq_ref, dk_ref, dv_ref = ref
    bq = np.full(dq_ref.shape, 1e-6)
    bk = np.full(dk_ref.shape, 1e-6)
    bv = np.full(dv_ref.shape, 1e-6)
    if Lq == 0 or Lkv == 0:
        return bq, bk, bv
    Q, K, V, G, O = q[:Lq], k[:Lkv], v[:Lkv], g[:Lq], o_gpu[:Lq]
    S = scale * (Q @ K.T)
    legal = np.ones((Lq, Lkv), dtype=bool)
    if causal:
        legal = np.arange(Lkv)[None, :] <= np.arange(Lq)[:, None]
    l = lse[:Lq, None]
    P = np.where(legal & np.isfinite(l), np.exp(np.where(legal, S, 0.0) - np.where(np.isfinite(l), l, 0.0)), 0.0)
    aG, aV, aQ, aK = np.abs(G), np.abs(V), np.abs(Q), np.abs(K)
    D = np.sum(G * O, axis=1)
    A = P * (aG @ aV.T + np.abs(D)[:, None])
    dD = 2 * U * np.sum(aG * (np.abs(O) + P @ aV), axis=1)
    bv[:Lkv] += 2 * (U * np.abs(dv_ref[:Lkv]) + 2 * U * (P.T @ aG))
    bk[:Lkv] += 2 * (U * np.abs(dk_ref[:Lkv]) + scale * (2 * U * (A.T @ aQ) + (P * dD[:, None]).T @ aQ))
    bq[:Lq] += 2 * (U * np.abs(dq_ref[:Lq]) + scale * (2 * U * (A @ aK) + dD[:, None] * (P @ aK)))
    return bq, bk, bv


def run_case(name, B, H, n_q, n_kv, causal, lq=None, lkv=None, seed=0, check_heads=None,
             strided=False, zero_dout=False, strided_grads=False):
    import torch
    attn = attn_mod()
    inp = gen.make_sdpa(name, "bf16", B, H, n_q, n_kv, 64, 64, 0.125, causal,
                        seqlens_q=None if lq is None else np.array(lq, np.int32),
                        seqlens_kv=None if lkv is None else np.array(lkv, np.int32), cfg_id=80 + seed)
    g, g_st = gen.make_dout(inp, 80 + seed)
    if zero_dout:
        g = np.where(np.isnan(g), g, 0.0)
        g_st = gen.storage(g, "bf16")
    announce(f"backward {name} B={B} H={H} n_q={n_q} n_kv={n_kv} causal={causal} lq={lq} lkv={lkv}"
             f" strided={strided}")
    q, k, v, do = (to_gpu(a, "bf16") for a in (inp.q_st, inp.k_st, inp.v_st, g_st))
    if strided:
        # q/k/v/dO as views of packed [B, n, H, 4*64] buffers (strides h = 256,
        # n = H*256), the layout a fused projection leaves behind
        def packed(t, slot, n):
            buf = torch.full((B, n, H, 4 * 64), float("nan"), dtype=torch.bfloat16, device=t.device)
            view = buf[:, :, :, 64 * slot:64 * (slot + 1)].permute(0, 2, 1, 3)
            view.copy_(t)
            return view
        q, do = packed(q, 0, n_q), packed(do, 3, n_q)
        k, v = packed(k, 1, n_kv), packed(v, 2, n_kv)
    lqg, lkg = lens_gpu(inp.seqlens_q), lens_gpu(inp.seqlens_kv)
    o, lse = attn.sdpa(q, k, v, scale=0.125, causal=causal, seqlens_q=lqg, seqlens_kv=lkg, return_lse=True)
    grads = {}
    if strided_grads:
        # dq, dk, dv written into views of packed [B, n, H, 2*64] buffers
        gq = torch.full((B, n_q, H, 128), float("nan"), dtype=torch.bfloat16, device=q.device)
        gkv = torch.full((B, n_kv, H, 256), float("nan"), dtype=torch.bfloat16, device=q.device)
        grads = dict(dq=gq[..., 64:].permute(0, 2, 1, 3), dk=gkv[..., :64].permute(0, 2, 1, 3),
                     dv=gkv[..., 128:192].permute(0, 2, 1, 3))
    dq, dk, dv = attn.sdpa_bwd(q, k, v, o, lse, do, scale=0.125, causal=causal, seqlens_q=lqg,
                               seqlens_kv=lkg, **grads)
    if strided_grads:   # the rest of the packed buffers is untouched
        assert torch.isnan(gq[..., :64]).all() and torch.isnan(gkv[..., 64:128]).all()
        assert torch.isnan(gkv[..., 192:]).all()
    torch.cuda.synchronize()
    og, lg = to_f64(o), lse.double().cpu().numpy()
    got = [to_f64(t) for t in (dq, dk, dv)]
    heads = [(b, h) for b in range(B) for h in range(H)] if check_heads is None else check_heads
    if check_heads is None:
        # one oracle call over every (b, h) (threaded inside the oracle)
        ref_all = oracle.sdpa_bwd(inp.q, inp.k, inp.v, g, scale=0.125, causal=causal,
                                  seqlens_q=inp.seqlens_q, seqlens_kv=inp.seqlens_kv)

    def check_head(bh):
        b, h = bh
        Lq = n_q if inp.seqlens_q is None else int(inp.seqlens_q[b])
        Lkv = n_kv if inp.seqlens_kv is None else int(inp.seqlens_kv[b])
        if check_heads is None:
            ref = [r[b, h] for r in ref_all]
        else:
            sl = (slice(b, b + 1), slice(h, h + 1))
            ref = oracle.sdpa_bwd(inp.q[sl], inp.k[sl], inp.v[sl], g[sl], scale=0.125, causal=causal,
                                  seqlens_q=None if inp.seqlens_q is None else inp.seqlens_q[b:b + 1],
                                  seqlens_kv=None if inp.seqlens_kv is None else inp.seqlens_kv[b:b + 1])
            ref = [r[0, 0] for r in ref]
        bnd = bounds(inp.q[b, h], inp.k[b, h], inp.v[b, h], g[b, h], og[b, h], lg[b, h], 0.125, causal,
                     Lq, Lkv, ref)
        worst, absmax = 0.0, [0.0, 0.0, 0.0]
        for i, (nm, x, r, bb) in enumerate(zip(("dq", "dk", "dv"), (t[b, h] for t in got), ref, bnd)):
            assert np.all(np.isfinite(x)), f"{nm} not finite at (b={b}, h={h})"
            if x.size == 0:
                continue
            ratio = np.abs(x - r) / bb
            worst = max(worst, float(ratio.max()))
            absmax[i] = float(np.abs(x - r).max())
            assert ratio.max() <= 1.0, (f"{nm} (b={b}, h={h}): max error/bound {ratio.max():.3f} at "
                                        f"{np.unravel_index(ratio.argmax(), ratio.shape)}")
        # padded query rows and keys past the lengths: exact zeros
        assert np.all(got[0][b, h, Lq:] == 0.0)
        assert np.all(got[1][b, h, Lkv:] == 0.0) and np.all(got[2][b, h, Lkv:] == 0.0)
        return worst, absmax

    import concurrent.futures as cf
    with cf.ThreadPoolExecutor(max_workers=min(16, len(heads))) as ex:
        results = list(ex.map(check_head, heads))
    worst = max(r[0] for r in results)
    absmax = [max(r[1][i] for r in results) for i in range(3)]
    print(f"{name}: max error/bound {worst:.3f} over {len(heads)} (b, h) slices; max|gpu-oracle| "
          f"dq {absmax[0]:.3e} dk {absmax[1]:.3e} dv {absmax[2]:.3e}", flush=True)
    return got, inp


CASES = [
    dict(name="causal_ragged", B=1, H=2, n_q=200, n_kv=200, causal=True),
    dict(name="bidir_lengths", B=2, H=2, n_q=300, n_kv=300, causal=False, lq=[300, 170], lkv=[300, 170]),
    dict(name="causal_lengths", B=2, H=2, n_q=260, n_kv=260, causal=True, lq=[260, 97], lkv=[260, 131]),
    dict(name="cross_key_lengths", B=2, H=3, n_q=257, n_kv=390, causal=False, lkv=[390, 201]),
    dict(name="cross_causal_nq_gt_nkv", B=1, H=2, n_q=333, n_kv=150, causal=True),
    dict(name="cross_causal_nq_lt_nkv", B=1, H=2, n_q=100, n_kv=300, causal=True),
    dict(name="single_query_key", B=2, H=2, n_q=1, n_kv=1, causal=False),
    dict(name="few_queries", B=1, H=2, n_q=5, n_kv=70, causal=False),
    dict(name="zero_length_sequence", B=2, H=2, n_q=150, n_kv=150, causal=True, lq=[0, 150], lkv=[150, 0]),
    dict(name="strided_packed", B=2, H=3, n_q=190, n_kv=190, causal=True, lkv=[190, 77], strided=True),
    dict(name="multi_tile", B=1, H=2, n_q=700, n_kv=700, causal=False),
    dict(name="query_lengths_only", B=2, H=2, n_q=180, n_kv=180, causal=False, lq=[180, 61]),
    dict(name="strided_gradients", B=2, H=2, n_q=150, n_kv=150, causal=True, lkv=[150, 99],
         strided_grads=True),
]


@pytest.mark.parametrize("c", CASES, ids=[c["name"] for c in CASES])
def test_bwd_vs_oracle(c):
    seed = 10 + CASES.index(c)
    c = dict(c)
    run_case(c.pop("name"), seed=seed, **c)


def _bwd_sweep(n=10, seed=4242):
    """Seeded random shapes: n_q and n_kv up to 520 (ragged against the
    128-row blocks and 64-row tiles of both kernels), causal or not, query
    and key lengths (zero included), batch*heads a multiple of 8 or not."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        B, H = int(rng.integers(1, 3)), int(rng.choice([1, 2, 4]))
        n_q, n_kv = int(rng.integers(1, 521)), int(rng.integers(1, 521))
        causal = bool(rng.integers(0, 2))
        lq = [int(x) for x in rng.integers(0, n_q + 1, size=B)] if rng.integers(0, 2) == 0 else None
        lkv = [int(x) for x in rng.integers(0, n_kv + 1, size=B)] if rng.integers(0, 2) == 0 else None
        out.append(dict(name=f"sweep{i:02d}_{B}x{H}x{n_q}x{n_kv}{'_causal' if causal else ''}"
                             f"{'_lq' if lq else ''}{'_lkv' if lkv else ''}",
                        B=B, H=H, n_q=n_q, n_kv=n_kv, causal=causal, lq=lq, lkv=lkv))
    return out


BWD_SWEEP = _bwd_sweep()


@pytest.mark.parametrize("c", BWD_SWEEP, ids=[c["name"] for c in BWD_SWEEP])
def test_bwd_random_shape_sweep(c):
    seed = 500 + BWD_SWEEP.index(c)
    c = dict(c)
    run_case(c.pop("name"), seed=seed, **c)


def test_bwd_zero_dout_gives_zero_gradients():
    """dO = 0 makes dV = P^T 0 and dS = P (0 - 0) vanish: every gradient is
    exactly zero."""
    got, _ = run_case("zero_dout", 1, 2, 130, 130, True, seed=1, zero_dout=True)
    for x in got:
        assert np.all(x == 0.0)


@pytest.mark.parametrize("n_q,n_kv", [(0, 64), (64, 0)])
def test_bwd_empty(n_q, n_kv):
    """No queries: dK = dV = 0.  No keys: every row has no legal key, dQ = 0."""
    got, _ = run_case(f"empty_{n_q}x{n_kv}", 1, 2, n_q, n_kv, False, seed=2)
    for x in got:
        assert np.all(x == 0.0)


def test_bwd_block_size_every_head():
    """The block's attention at full size, [4,16,4096,64] causal, in the
    launch configuration the benchmark times: every gradient element of all
    64 (b, h) slices checked against the oracle's exact gradients."""
    run_case("block_4x16x4096", 4, 16, 4096, 4096, True, seed=3)
