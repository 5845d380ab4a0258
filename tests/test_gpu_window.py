"""GPU parity of attn_sdpa_window_fwd, restricted self-attention (key j legal
for query i only if |i - j| <= r, on top of the key lengths and the causal
mask), against the fp64 oracle on identical seeded inputs.  Tolerances as for
attn_sdpa_fwd: 2e-2 max-abs for bf16 (fp32 accumulation), 1e-4 for fp32; lse
4e-3 (bf16) / 1e-4 (fp32) relative to max(1, |lse|)."""
import numpy as np
import pytest

import attn_inputs as gen
import oracle
from gpu_helpers import announce, lens_gpu, max_err, to_f64, to_gpu

pytestmark = pytest.mark.gpu


def attn_mod():
    import head_attention_sdpa_amd as attn
    attn.lib()
    return attn


def run_case(name, dtype, B, H, n_q, n_kv, r, causal, lq=None, lkv=None, seed=0, d=64):
    import torch
    attn = attn_mod()
    inp = gen.make_sdpa(name, dtype, B, H, n_q, n_kv, d, d, 0.125, causal,
                        seqlens_q=None if lq is None else np.array(lq, np.int32),
                        seqlens_kv=None if lkv is None else np.array(lkv, np.int32), cfg_id=70 + seed)
    announce(f"window {name} {dtype} B={B} H={H} n_q={n_q} n_kv={n_kv} r={r} causal={causal}")
    q, k, v = (to_gpu(a, dtype) for a in (inp.q_st, inp.k_st, inp.v_st))
    o, lse = attn.sdpa(q, k, v, scale=0.125, causal=causal, seqlens_q=lens_gpu(inp.seqlens_q),
                       seqlens_kv=lens_gpu(inp.seqlens_kv), return_lse=True, window=r)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.sdpa(inp.q, inp.k, inp.v, scale=0.125, causal=causal, seqlens_q=inp.seqlens_q,
                               seqlens_kv=inp.seqlens_kv, window=r)
    og, lg = to_f64(o), lse.double().cpu().numpy()
    tol, ltol = (2e-2, 4e-3) if dtype == "bf16" else (1e-4, 1e-4)
    assert np.all(np.isfinite(og))
    none = ref_lse == -np.inf
    assert np.array_equal(lg == -np.inf, none)
    assert np.all(og[none] == 0.0)
    rel = np.abs(lg[~none] - ref_lse[~none]) / np.maximum(1.0, np.abs(ref_lse[~none]))
    e = max_err(og, ref)
    print(f"{name}: max|dO| {e:.3e}  max rel dlse {float(rel.max()) if rel.size else 0.0:.3e}", flush=True)
    assert e <= tol and (rel.size == 0 or rel.max() <= ltol)
    return og, inp


CASES = [
    dict(name="r0_diagonal", B=1, H=2, n_q=130, n_kv=130, r=0, causal=False),
    dict(name="r1_causal", B=1, H=2, n_q=200, n_kv=200, r=1, causal=True),
    dict(name="r63_lengths", B=2, H=2, n_q=700, n_kv=700, r=63, causal=False, lq=[700, 333], lkv=[700, 333]),
    dict(name="r64_causal_lengths", B=2, H=2, n_q=700, n_kv=700, r=64, causal=True, lkv=[700, 400]),
    dict(name="r100_bidir", B=2, H=3, n_q=513, n_kv=513, r=100, causal=False),
    dict(name="r_wider_than_sequence", B=1, H=2, n_q=300, n_kv=300, r=1000, causal=True),
    dict(name="cross_nq_lt_nkv", B=2, H=2, n_q=300, n_kv=500, r=50, causal=False, lkv=[500, 260]),
    dict(name="cross_nq_gt_nkv", B=1, H=2, n_q=500, n_kv=300, r=37, causal=True),
]


@pytest.mark.parametrize("c", CASES, ids=[c["name"] for c in CASES])
def test_window_bf16_vs_oracle(c):
    c = dict(c)
    run_case(c.pop("name"), "bf16", seed=len(CASES), **c)


def _window_sweep(n=10, seed=91):
    """Seeded random restricted-attention shapes: n_q, n_kv up to 800, radius
    0 to 400, causal or not, lengths or not."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
        n_q, n_kv = int(rng.integers(1, 801)), int(rng.integers(1, 801))
        r = int(rng.choice([0, 1, int(rng.integers(2, 65)), int(rng.integers(65, 401))]))
        causal = bool(rng.integers(0, 2))
        lq = [int(x) for x in rng.integers(0, n_q + 1, size=B)] if rng.integers(0, 3) == 0 else None
        lkv = [int(x) for x in rng.integers(0, n_kv + 1, size=B)] if rng.integers(0, 2) == 0 else None
        out.append(dict(name=f"sweep{i:02d}_{B}x{H}x{n_q}x{n_kv}_r{r}{'_causal' if causal else ''}"
                             f"{'_lq' if lq else ''}{'_lkv' if lkv else ''}",
                        B=B, H=H, n_q=n_q, n_kv=n_kv, r=r, causal=causal, lq=lq, lkv=lkv))
    return out


WINDOW_SWEEP = _window_sweep()


@pytest.mark.parametrize("c", WINDOW_SWEEP, ids=[c["name"] for c in WINDOW_SWEEP])
def test_window_random_shape_sweep(c):
    seed = 40 + WINDOW_SWEEP.index(c)
    c = dict(c)
    run_case(c.pop("name"), "bf16", seed=seed, **c)


def test_window_zero_returns_v():
    """r = 0: every query attends to itself only, so O = V exactly (the weight
    is 1 and V is already bf16)."""
    og, inp = run_case("r0_exact", "bf16", 1, 2, 97, 97, 0, False, seed=3)
    assert np.array_equal(og, inp.v)


@pytest.mark.parametrize("r,causal", [(5, False), (3, True)])
def test_window_f32_vs_oracle(r, causal):
    run_case(f"f32_r{r}", "f32", 1, 2, 40, 40, r, causal, seed=4, d=16)


def test_window_long_sequence():
    """The block's sequence length with a 256-key radius: 16 heads x 4096."""
    run_case("long_r256", "bf16", 1, 16, 4096, 4096, 256, True, seed=5)


@pytest.mark.parametrize("dtype,causal", [("bf16", True), ("bf16", False), ("f32", True)])
def test_window_int_max_is_full_attention(dtype, causal):
    """A radius beyond every |i - j| leaves every key legal: r = 2^31 - 1
    (which the library clamps before its bound arithmetic) gives bitwise the
    same output as the radius max(n_q, n_kv), and unrestricted attention
    within tolerance of the oracle."""
    import torch
    attn = attn_mod()
    d = 64 if dtype == "bf16" else 16
    og, inp = run_case(f"int_max_{dtype}_{causal}", dtype, 2, 2, 333, 333, 2 ** 31 - 1, causal, seed=6, d=d)
    q, k, v = (to_gpu(a, dtype) for a in (inp.q_st, inp.k_st, inp.v_st))
    o2 = attn.sdpa(q, k, v, scale=0.125, causal=causal, window=333)
    torch.cuda.synchronize()
    assert np.array_equal(og, to_f64(o2))
    ref, _ = oracle.sdpa(inp.q, inp.k, inp.v, scale=0.125, causal=causal)
    assert max_err(og, ref) <= (2e-2 if dtype == "bf16" else 1e-4)
