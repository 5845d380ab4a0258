"""GPU parity of attn_sdpa_fwd (HIP kernels, through the C ABI) against the fp64
oracle on identical seeded inputs, plus black-box invariants of the GPU
output.  Tolerances (max-abs over all outputs): 1e-4 for fp32 inputs, 2e-2
for bf16 inputs with fp32 accumulation."""
import math

import numpy as np
import pytest

import attn_inputs as gen
import oracle
from gpu_helpers import announce, lens_gpu, max_err, to_f64, to_gpu

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
# bf16 path: the softmax denominator sums the bf16-rounded weights (the ones
# that enter P.V), each within a relative 2^-9 of its fp32 value, so
# |d ln l| <= 2^-9 / (1 - 2^-9) ~ 2e-3; 4e-3 leaves room for fp32 score rounding.
LSE_TOL = {"f32": 1e-4, "bf16": 4e-3}


def attn_mod():
    import head_attention_sdpa_amd as attn
    attn.lib()  # raises if the HIP library is missing: no fallback
    return attn


def run_gpu(inp, **kw):
    attn = attn_mod()
    q, k, v = (to_gpu(a, inp.dtype) for a in (inp.q_st, inp.k_st, inp.v_st))
    o, lse = attn.sdpa(q, k, v, scale=inp.scale, causal=inp.causal,
                       seqlens_q=lens_gpu(inp.seqlens_q), seqlens_kv=lens_gpu(inp.seqlens_kv),
                       return_lse=True, **kw)
    import torch
    torch.cuda.synchronize()
    return to_f64(o), to_f64(lse)


def check_against_oracle(inp, o_gpu, lse_gpu):
    o_ref, lse_ref = oracle.sdpa(inp.q, inp.k, inp.v, scale=inp.scale, causal=inp.causal,
                                 seqlens_q=inp.seqlens_q, seqlens_kv=inp.seqlens_kv)
    assert not np.isnan(o_gpu).any(), "NaN in the GPU output"
    err = max_err(o_gpu, o_ref)
    print(f"  {inp.name}: max|gpu-oracle| = {err:.3e} (tol {TOL[inp.dtype]})", flush=True)
    assert err <= TOL[inp.dtype]
    # rows the ABI defines as zero are exactly zero
    zero_rows = np.isneginf(lse_ref)
    assert np.all(o_gpu[zero_rows] == 0.0)
    assert np.all(np.isneginf(lse_gpu[zero_rows]))
    fin = ~zero_rows
    if fin.any():
        # fp32 score accumulation error grows with the score magnitude
        lse_err = np.abs(lse_gpu[fin] - lse_ref[fin]) / np.maximum(1.0, np.abs(lse_ref[fin]))
        assert lse_err.max() <= LSE_TOL[inp.dtype]
    return err


# ---------------------------------------------------------------------------
# The five workloads' SDPA configs at full size, and reduced/ragged cases
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_config_full_size(cfg):
    inp = gen.config(cfg)
    announce(f"sdpa config {cfg} {inp.name} shape={inp.shape}")
    o, lse = run_gpu(inp)
    check_against_oracle(inp, o, lse)


def _case(name, dtype, B, H, nq, nkv, dk=64, dv=64, causal=False, lq=None, lkv=None, scale=None,
          cfg_id=90):
    scale = 1.0 / math.sqrt(dk) if scale is None else scale
    lq = None if lq is None else np.array(lq, np.int32)
    lkv = None if lkv is None else np.array(lkv, np.int32)
    return gen.make_sdpa(name, dtype, B, H, nq, nkv, dk, dv, scale, causal, lq, lkv, cfg_id=cfg_id)


RAGGED = [
    dict(name="bf16_ragged_bidir", dtype="bf16", B=2, H=3, nq=200, nkv=333),
    dict(name="bf16_ragged_causal", dtype="bf16", B=2, H=3, nq=333, nkv=333, causal=True),
    dict(name="bf16_causal_nq_gt_nkv", dtype="bf16", B=1, H=2, nq=300, nkv=130, causal=True),
    dict(name="bf16_causal_nq_lt_nkv", dtype="bf16", B=1, H=2, nq=70, nkv=250, causal=True),
    dict(name="bf16_lengths_both_causal", dtype="bf16", B=2, H=3, nq=200, nkv=333, causal=True,
         lq=[150, 200], lkv=[333, 17]),
    dict(name="bf16_lengths_zero_and_one", dtype="bf16", B=3, H=2, nq=65, nkv=129,
         lq=[65, 0, 65], lkv=[0, 50, 1]),
    dict(name="bf16_single", dtype="bf16", B=1, H=1, nq=1, nkv=1),
    dict(name="bf16_empty_keys", dtype="bf16", B=2, H=1, nq=5, nkv=0),
    dict(name="bf16_xcd_path_bh8", dtype="bf16", B=1, H=8, nq=513, nkv=513, causal=True),
    dict(name="bf16_scale_4", dtype="bf16", B=1, H=2, nq=100, nkv=100, scale=0.5),
    dict(name="f32_small_d_causal_lengths", dtype="f32", B=2, H=2, nq=70, nkv=90, dk=5, dv=7,
         causal=True, lkv=[90, 33], lq=[70, 50]),
    dict(name="f32_d64_multiblock", dtype="f32", B=1, H=3, nq=130, nkv=77),
    # 2048 (b, h) slices of 40 queries: a grid of 2048 one-block workgroups
    dict(name="bf16_many_heads_causal", dtype="bf16", B=16, H=128, nq=40, nkv=40, causal=True),
]


@pytest.mark.parametrize("case", RAGGED, ids=[c["name"] for c in RAGGED])
def test_ragged_and_edge_cases(case):
    inp = _case(**case)
    announce(f"sdpa {inp.name} shape={inp.shape} causal={inp.causal}")
    o, lse = run_gpu(inp)
    check_against_oracle(inp, o, lse)


# Shapes on both sides of the short-sequence kernel's limits (one workgroup per
# (batch, head) when n_q <= 256 and n_kv <= 384, eight waves up to n_q = 128,
# 2/4/6 resident key tiles): masks, lengths that leave a single active group
# of 16 queries, heads with no key, and causal masks with n_q != n_kv.
RESIDENT_EDGES = [
    dict(name="res_nq256_nkv384_len", B=2, H=3, nq=256, nkv=384, lkv=[384, 200]),
    dict(name="stream_nq257_nkv384", B=1, H=2, nq=257, nkv=384),
    dict(name="stream_nq128_nkv385", B=1, H=2, nq=128, nkv=385),
    dict(name="res_nq129_nkv130_causal", B=2, H=2, nq=129, nkv=130, causal=True),
    dict(name="res_nq128_nkv128_causal_len", B=3, H=2, nq=128, nkv=128, causal=True, lq=[128, 77, 1],
         lkv=[128, 128, 60]),
    dict(name="res_nq16_causal_len_zero", B=3, H=2, nq=16, nkv=16, causal=True, lq=[16, 7, 0]),
    dict(name="res_causal_nq_lt_nkv", B=1, H=3, nq=100, nkv=300, causal=True),
    dict(name="res_causal_nq_gt_nkv", B=1, H=3, nq=250, nkv=70, causal=True),
    dict(name="res_one_active_group", B=2, H=2, nq=256, nkv=384, lq=[10, 256], lkv=[384, 1]),
    dict(name="res_no_keys_in_one_head", B=2, H=2, nq=200, nkv=64, causal=True, lq=[200, 200], lkv=[0, 64]),
]


@pytest.mark.parametrize("case", RESIDENT_EDGES, ids=[c["name"] for c in RESIDENT_EDGES])
def test_short_sequence_kernel_edges(case):
    inp = _case(dtype="bf16", cfg_id=89, **case)
    announce(f"sdpa {inp.name} shape={inp.shape} causal={inp.causal}")
    o, lse = run_gpu(inp)
    check_against_oracle(inp, o, lse)


def _sweep_cases(n=24, seed=2024):
    """Seeded random shapes over both bf16 kernels and their limits: n_q and
    n_kv up to 700 (the short-sequence kernel takes n_q <= 256, n_kv <= 384),
    causal or not, lengths or not (including empty sequences), batch*heads
    a multiple of 8 or not (the two workgroup orders)."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        B, H = int(rng.integers(1, 4)), int(rng.choice([1, 2, 3, 8]))
        nq = int(rng.choice([int(rng.integers(1, 257)), int(rng.integers(257, 701))]))
        nkv = int(rng.choice([int(rng.integers(1, 385)), int(rng.integers(385, 701))]))
        causal = bool(rng.integers(0, 2))
        lq = [int(x) for x in rng.integers(0, nq + 1, size=B)] if rng.integers(0, 3) == 0 else None
        lkv = [int(x) for x in rng.integers(0, nkv + 1, size=B)] if rng.integers(0, 2) == 0 else None
        cases.append(dict(name=f"sweep{i:02d}_{B}x{H}x{nq}x{nkv}{'_causal' if causal else ''}"
                               f"{'_lq' if lq else ''}{'_lkv' if lkv else ''}",
                          B=B, H=H, nq=nq, nkv=nkv, causal=causal, lq=lq, lkv=lkv))
    return cases


SWEEP = _sweep_cases()


@pytest.mark.parametrize("case", SWEEP, ids=[c["name"] for c in SWEEP])
def test_random_shape_sweep(case):
    inp = _case(dtype="bf16", cfg_id=88, **case)
    announce(f"sdpa {inp.name} shape={inp.shape} causal={inp.causal}")
    o, lse = run_gpu(inp)
    check_against_oracle(inp, o, lse)


LONG = [
    # one head of 65,536 positions, causal: 1,024 key tiles, 8 MiB per operand
    dict(name="bf16_long_65536_causal", B=1, H=1, nq=65536, nkv=65536, causal=True),
    # 2,048 queries over 49,152 cached keys of which 40,001 are valid
    dict(name="bf16_long_cross_49152_len", B=1, H=1, nq=2048, nkv=49152, causal=False, lkv=[40001]),
]


@pytest.mark.parametrize("case", LONG, ids=[c["name"] for c in LONG])
def test_long_sequence_sampled_rows(case):
    """Long sequences: every query is computed on the GPU; 12 rows (first,
    tile and block edges, middle, last) are checked against the oracle row
    by row."""
    inp = _case(dtype="bf16", cfg_id=97, **case)
    announce(f"sdpa {inp.name} shape={inp.shape} causal={inp.causal}")
    o, lse = run_gpu(inp)
    n = inp.shape[2]
    rows = np.unique(np.array([0, 1, 63, 64, 127, 128, 1000, n // 2 - 1, n // 2, n - 65, n - 64, n - 1]))
    o_ref, lse_ref = oracle.sdpa_rows(inp.q, inp.k, inp.v, rows, scale=inp.scale, causal=inp.causal,
                                      seqlens_kv=inp.seqlens_kv)
    err = float(np.abs(o[0, 0, rows] - o_ref).max())
    lse_err = float((np.abs(lse[0, 0, rows] - lse_ref) / np.maximum(1.0, np.abs(lse_ref))).max())
    print(f"  {inp.name}: max|gpu-oracle| = {err:.3e}, lse rel {lse_err:.2e} over {len(rows)} rows", flush=True)
    assert not np.isnan(o).any()
    assert err <= TOL["bf16"] and lse_err <= LSE_TOL["bf16"]


# ---------------------------------------------------------------------------
# The pages' worked examples on the GPU (fp32 path)
# ---------------------------------------------------------------------------
def _run_f32(Q, K, V, causal=False):
    attn = attn_mod()
    import torch
    t = [torch.tensor(np.asarray(a, np.float32)[None, None], device="cuda") for a in (Q, K, V)]
    o = attn.sdpa(*t, causal=causal)
    torch.cuda.synchronize()
    return to_f64(o)[0, 0]


def test_p1_example_on_gpu(golden):
    """attention-paper-guide 03.2 two-token example: weights (via V = I) and
    outputs, against the closed form and the printed values."""
    announce("p1 two-token example, fp32")
    g = golden("p1_two_token_example.txt")
    e = math.exp(1 / math.sqrt(2))
    w_exact = np.array([[0.5, 0.5], [1 / (1 + e), e / (1 + e)]])
    P = _run_f32(g["Q"], g["K"], np.eye(2))
    assert np.abs(P - w_exact).max() < 1e-6
    assert np.abs(P - g["weights_printed"]).max() <= 0.005 + 1e-6
    O = _run_f32(g["Q"], g["K"], g["V"])
    assert np.abs(O - w_exact @ g["V"]).max() < 1e-5
    assert np.abs(O - g["output_printed"]).max() <= 0.05
    Oc = _run_f32(g["Q"], g["K"], g["V"], causal=True)
    assert np.array_equal(Oc[0], [10.0, 0.0])


def test_p4_ledger_on_gpu(golden):
    announce("p4 ledger, fp32")
    g = golden("p4_running_example_ledger.txt")
    A = _run_f32(g["Q"], g["K"], np.eye(4))
    assert np.abs(A - g["A"]).max() < 2e-3
    Z = _run_f32(g["Q"], g["K"], g["V"])
    assert np.abs(Z[0] - g["z0"][0]).max() < 2e-3
    Ac = _run_f32(g["Q"], g["K"], np.eye(4), causal=True)
    assert np.abs(Ac[:2] - g["causal_rows_0_1"]).max() < 2e-3
    assert np.all(Ac[np.triu_indices(4, 1)] == 0.0)


# ---------------------------------------------------------------------------
# Black-box invariants of the bf16 kernel
# ---------------------------------------------------------------------------
def _bf16_case(seed=91, B=2, H=4, n=256, causal=True):
    return _case(f"inv_{seed}", "bf16", B, H, n, n, causal=causal, cfg_id=seed)


def test_bitwise_deterministic():
    inp = _bf16_case()
    announce("determinism")
    o1, l1 = run_gpu(inp)
    o2, l2 = run_gpu(inp)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_future_keys_are_ignored_bitwise():
    """Causal: changing K[j], V[j] for j > i leaves output rows <= i bitwise unchanged."""
    inp = _bf16_case(92)
    announce("future keys ignored")
    o1, _ = run_gpu(inp)
    cut = 100
    inp2 = _bf16_case(92)
    rng = np.random.default_rng(3)
    inp2.k[:, :, cut + 1:] = gen.round_to_bf16(rng.normal(size=inp2.k[:, :, cut + 1:].shape) * 3)
    inp2.v[:, :, cut + 1:] = gen.round_to_bf16(rng.normal(size=inp2.v[:, :, cut + 1:].shape) * 3)
    inp2.k_st, inp2.v_st = gen.bf16_bits(inp2.k), gen.bf16_bits(inp2.v)
    o2, _ = run_gpu(inp2)
    assert np.array_equal(o1[:, :, :cut + 1], o2[:, :, :cut + 1])
    assert not np.array_equal(o1[:, :, cut + 1:], o2[:, :, cut + 1:])


def test_value_column_of_ones_gives_ones():
    inp = _bf16_case(93, causal=False)
    inp.v[:] = 1.0
    inp.v_st = gen.bf16_bits(inp.v)
    announce("rows sum to one")
    o, _ = run_gpu(inp)
    assert np.abs(o - 1.0).max() <= 2 ** -7


def test_large_shift_overflow_safety():
    """Scores near +1e3 (keys shifted along the query direction): the max
    subtraction keeps the kernel finite and on the oracle."""
    inp = _bf16_case(94, n=192)
    inp.q = gen.round_to_bf16(np.abs(inp.q) + 1.0)
    inp.k = gen.round_to_bf16(inp.k + 48.0)
    inp.q_st, inp.k_st = gen.bf16_bits(inp.q), gen.bf16_bits(inp.k)
    announce("large shift")
    o, lse = run_gpu(inp)
    assert np.all(np.isfinite(o))
    check_against_oracle(inp, o, lse)


def test_strided_layout_equals_contiguous():
    """[B, n, H, d] memory read through strides gives the same bits as BHND."""
    import torch
    attn = attn_mod()
    inp = _case("strided", "bf16", 2, 4, 160, 200, causal=True, cfg_id=95)
    announce("strided layout")
    q, k, v = (to_gpu(a, "bf16") for a in (inp.q_st, inp.k_st, inp.v_st))
    o_c = attn.sdpa(q, k, v, causal=True)
    qs, ks, vs = (t.transpose(1, 2).contiguous().transpose(1, 2) for t in (q, k, v))
    out = torch.empty((2, 160, 4, 64), dtype=torch.bfloat16, device="cuda").transpose(1, 2)
    o_s = attn.sdpa(qs, ks, vs, causal=True, out=out)
    torch.cuda.synchronize()
    assert qs.stride(2) == 4 * 64 and o_s.stride(2) == 4 * 64
    assert torch.equal(o_c, o_s)


def test_no_out_of_bounds_writes():
    import torch
    attn = attn_mod()
    inp = _case("guard", "bf16", 1, 2, 77, 90, causal=True, cfg_id=96)
    announce("guard canaries")
    q, k, v = (to_gpu(a, "bf16") for a in (inp.q_st, inp.k_st, inp.v_st))
    n_out = 1 * 2 * 77 * 64
    buf = torch.full((n_out + 2 * 4096,), -7.0, dtype=torch.bfloat16, device="cuda")
    out = buf[4096:4096 + n_out].view(1, 2, 77, 64)
    attn.sdpa(q, k, v, causal=True, out=out)
    torch.cuda.synchronize()
    assert torch.all(buf[:4096] == -7.0) and torch.all(buf[4096 + n_out:] == -7.0)
    assert torch.isfinite(out).all()


def test_non_default_stream():
    import torch
    attn = attn_mod()
    inp = _bf16_case(97, H=2)
    announce("non-default stream")
    ref, _ = run_gpu(inp)
    q, k, v = (to_gpu(a, "bf16") for a in (inp.q_st, inp.k_st, inp.v_st))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        o = attn.sdpa(q, k, v, scale=inp.scale, causal=True)
    s.synchronize()
    assert np.array_equal(to_f64(o), ref)


def test_permutation_equivariance_on_gpu():
    """No mask: permuting queries permutes the output rows (bitwise, since each
    query's arithmetic is independent); permuting keys with their values stays
    within tolerance (summation order changes)."""
    inp = _case("perm", "bf16", 1, 2, 96, 96, cfg_id=98)
    announce("permutation equivariance")
    o, _ = run_gpu(inp)
    perm = np.random.default_rng(5).permutation(96)
    inp2 = _case("perm", "bf16", 1, 2, 96, 96, cfg_id=98)
    inp2.q = inp2.q[:, :, perm]
    inp2.q_st = gen.bf16_bits(inp2.q)
    o2, _ = run_gpu(inp2)
    assert np.array_equal(o2, o[:, :, perm])
    inp3 = _case("perm", "bf16", 1, 2, 96, 96, cfg_id=98)
    inp3.k, inp3.v = inp3.k[:, :, perm], inp3.v[:, :, perm]
    inp3.k_st, inp3.v_st = gen.bf16_bits(inp3.k), gen.bf16_bits(inp3.v)
    o3, _ = run_gpu(inp3)
    assert max_err(o3, o) <= 2e-2


def test_api_errors_raise():
    import torch
    attn = attn_mod()
    q = torch.zeros((1, 1, 8, 32), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(attn.AttnError) as e:
        attn.sdpa(q, q, q)
    assert e.value.status == -2
