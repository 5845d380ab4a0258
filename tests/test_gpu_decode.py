"""GPU parity of attn_decode_fwd (one decoding step over a key/value cache:
the newest n_q queries of each sequence, causal aligned at the end of the
cache) against the fp64 oracle on identical seeded inputs.  Cache rows past
the lengths hold NaN.  Tolerances as for the bf16 SDPA: 2e-2 max-abs on O
(bf16 inputs and weights, fp32 accumulation, one RNE rounding of O) and 4e-3
relative (to max(1, |lse|)) on the log-sum-exp, whose denominator sums the
bf16-rounded weights (relative error ~2^-9 in the sum)."""
import numpy as np
import pytest

import attn_inputs as gen
import oracle
from gpu_helpers import announce, lens_gpu, max_err, to_f64, to_gpu

pytestmark = pytest.mark.gpu
TOL, LSE_TOL = 2e-2, 4e-3


def attn_mod():
    import head_attention_sdpa_amd as attn
    attn.lib()
    return attn


def run(inp, strided=False):
    import torch
    attn = attn_mod()
    q, k, v = (to_gpu(a, "bf16") for a in (inp.q_st, inp.k_st, inp.v_st))
    if strided:   # the cache inside a larger buffer: [B, H, n_kv, 64] out of [B, H+1, n_kv, 128]
        B, H, n_kv, _ = k.shape
        kb = torch.zeros((B, H + 1, n_kv, 128), dtype=k.dtype, device=k.device)
        vb = torch.zeros_like(kb)
        kb[:, 1:, :, 32:96] = k
        vb[:, 1:, :, 32:96] = v
        k, v = kb[:, 1:, :, 32:96], vb[:, 1:, :, 32:96]
    o, lse = attn.decode(q, k, v, scale=inp.scale, seqlens_kv=lens_gpu(inp.seqlens_kv), return_lse=True)
    torch.cuda.synchronize()
    return to_f64(o), lse.double().cpu().numpy()


def compare(inp, o, lse, what):
    ref_o, ref_lse = oracle.decode(inp.q, inp.k, inp.v, scale=inp.scale, seqlens_kv=inp.seqlens_kv)
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    e = max_err(o, ref_o)
    none = ref_lse == -np.inf
    assert np.array_equal(lse == -np.inf, none), f"{what}: -inf lse pattern differs"
    assert np.all(o[none] == 0.0), f"{what}: rows without keys must be zeros"
    rel = np.abs(lse[~none] - ref_lse[~none]) / np.maximum(1.0, np.abs(ref_lse[~none]))
    el = float(rel.max()) if rel.size else 0.0
    print(f"{what}: max|dO| {e:.3e}  max rel dlse {el:.3e}", flush=True)
    assert e <= TOL and el <= LSE_TOL


CASES = [
    dict(name="one_query_ragged_cache", B=2, H=3, n_q=1, n_kv=300, lo=137),
    dict(name="four_queries_speculative", B=3, H=2, n_q=4, n_kv=1000, lo=3),
    dict(name="thirty_two_queries_full_tiles", B=2, H=2, n_q=32, n_kv=320, lo=320),
    dict(name="short_and_empty_sequences", B=4, H=1, n_q=2, n_kv=2048, L=[1, 0, 2, 2048]),
    dict(name="odd_queries_tail_tile", B=1, H=5, n_q=7, n_kv=4097, lo=4000),
    # up to four chunks per (b, h) run as the waves of one workgroup, merged in LDS:
    dict(name="merged_one_chunk_short_cache", B=2, H=3, n_q=5, n_kv=50, L=[50, 3]),
    dict(name="merged_two_chunks", B=2, H=2, n_q=3, n_kv=100, L=[100, 65]),
    dict(name="merged_three_chunks", B=1, H=3, n_q=7, n_kv=150, L=[150]),
    dict(name="merged_four_chunks_empty_and_short", B=3, H=1, n_q=2, n_kv=256, L=[256, 0, 70]),
    dict(name="merged_one_chunk_many_heads", B=64, H=16, n_q=1, n_kv=300, lo=1),
]


@pytest.mark.parametrize("c", CASES, ids=[c["name"] for c in CASES])
def test_decode_vs_oracle(c):
    c = dict(c)
    name = c.pop("name")
    inp = gen.decode_workload(**c)
    announce(f"decode {name} {inp.shape} L={inp.seqlens_kv.tolist()}")
    o, lse = run(inp)
    compare(inp, o, lse, name)


def _decode_sweep(n=10, seed=77):
    """Seeded random decoding steps: 1-32 new queries, caches up to 6000 rows
    (one chunk up to the split over workgroups), lengths from 0 to the
    capacity, batch*heads from 1 to 96."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        B, H = int(rng.integers(1, 7)), int(rng.integers(1, 17))
        n_q = int(rng.choice([1, 1, 2, 4, 7, 16, 32]))
        n_kv = int(rng.integers(1, 6001))
        L = [int(x) for x in rng.integers(0, n_kv + 1, size=B)]
        out.append(dict(name=f"sweep{i:02d}_{B}x{H}_q{n_q}_cache{n_kv}", B=B, H=H, n_q=n_q, n_kv=n_kv, L=L))
    return out


DECODE_SWEEP = _decode_sweep()


@pytest.mark.parametrize("c", DECODE_SWEEP, ids=[c["name"] for c in DECODE_SWEEP])
def test_decode_random_shape_sweep(c):
    c = dict(c)
    name = c.pop("name")
    inp = gen.decode_workload(**c)
    announce(f"decode {name} {inp.shape} L={inp.seqlens_kv.tolist()}")
    o, lse = run(inp)
    compare(inp, o, lse, name)


def test_decode_strided_cache():
    inp = gen.decode_workload(B=2, H=3, n_q=3, n_kv=700, lo=200)
    announce(f"decode strided cache {inp.shape}")
    o, lse = run(inp, strided=True)
    compare(inp, o, lse, "strided")


def test_decode_full_size_workload():
    """The benchmarked step at full size: 16 x 16 heads, one query, cache
    capacity 4096, lengths U{1024..4096}; every output checked."""
    inp = gen.decode_workload()
    announce(f"decode full size {inp.shape}")
    o, lse = run(inp)
    compare(inp, o, lse, "full")


def test_decode_empty_cache_and_no_queries():
    import torch
    attn = attn_mod()
    announce("decode n_kv = 0 and n_q = 0")
    q = torch.randn((2, 2, 3, 64), device="cuda:0").to(torch.bfloat16)
    kv = torch.empty((2, 2, 0, 64), dtype=torch.bfloat16, device="cuda:0")
    o, lse = attn.decode(q, kv, kv, return_lse=True)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(lse == -float("inf"))
    q0 = torch.empty((2, 2, 0, 64), dtype=torch.bfloat16, device="cuda:0")
    k = torch.randn((2, 2, 64, 64), device="cuda:0").to(torch.bfloat16)
    assert attn.decode(q0, k, k).shape == (2, 2, 0, 64)


def test_decode_matches_prefill_last_rows():
    """The decoding step and the causal prefill kernel agree on the last rows
    of a full sequence (both on the GPU, both against the oracle)."""
    import torch
    attn = attn_mod()
    n, n_q = 333, 5
    inp = gen.make_sdpa("decode_vs_prefill", "bf16", 2, 2, n, n, 64, 64, 0.125, True, cfg_id=61)
    announce("decode vs prefill last rows")
    q, k, v = (to_gpu(a, "bf16") for a in (inp.q_st, inp.k_st, inp.v_st))
    o_full = attn.sdpa(q, k, v, scale=0.125, causal=True)
    o_dec = attn.decode(q[:, :, n - n_q:].contiguous(), k, v, scale=0.125)
    torch.cuda.synchronize()
    d = max_err(to_f64(o_dec), to_f64(o_full)[:, :, n - n_q:])
    ref, _ = oracle.sdpa(inp.q, inp.k, inp.v, scale=0.125, causal=True)
    assert max_err(to_f64(o_dec), ref[:, :, n - n_q:]) <= TOL
    assert d <= 2 * TOL
