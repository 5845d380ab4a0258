"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test names the fact it pins and the plausible oracle mistake it would
catch (wrong or missing scale, transposed operands, softmax over the wrong
axis, off-by-one or reversed causal mask, padding applied to the wrong side,
mixed-up head slicing, wrong weight orientation, wrong log-sum-exp).
Runs on the CPU only.
"""
import math

import numpy as np
import pytest

import attn_inputs as gen
import oracle


def rnd(seed, shape):
    return gen.normal(seed, shape)


def weights_via_identity(q, k, **kw):
    """Attention weights P: with V = I (d_v = n_kv) the output row is the
    weight row."""
    B, H, n_q, _ = q.shape
    n_kv = k.shape[2]
    eye = np.broadcast_to(np.eye(n_kv), (B, H, n_kv, n_kv)).copy()
    o, lse = oracle.sdpa(q, k, eye, **kw)
    return o, lse


# ---------------------------------------------------------------------------
# Worked examples printed on the pages
# ---------------------------------------------------------------------------
def test_p1_two_token_example(golden):
    """attention-paper-guide section 03.2: 2 tokens, d_k = 2.  Closed form:
    row 0 scores (1,1)/sqrt2 -> weights (1/2, 1/2); row 1 scores (0,1)/sqrt2 ->
    weights (1, e^{1/sqrt2}) / (1 + e^{1/sqrt2}).  Catches a missing or wrong
    scale, Q/K swapped (K Q^T gives different rows), softmax on the wrong axis."""
    g = golden("p1_two_token_example.txt")
    Q, K, V = (g[n][None, None] for n in ("Q", "K", "V"))
    e = math.exp(1 / math.sqrt(2))
    w_exact = np.array([[0.5, 0.5], [1 / (1 + e), e / (1 + e)]])
    o_exact = w_exact @ np.array([[10.0, 0.0], [0.0, 6.0]])
    P, lse = weights_via_identity(Q, K)
    assert np.abs(P[0, 0] - w_exact).max() < 1e-12
    o, lse2 = oracle.sdpa(Q, K, V)
    assert np.abs(o[0, 0] - o_exact).max() < 1e-12
    # the page's printed values, to its printed precision
    assert np.abs(P[0, 0] - g["weights_printed"]).max() <= 0.005 + 1e-12
    assert np.abs(o[0, 0] - g["output_printed"]).max() <= 0.05
    assert abs(o[0, 0, 1, 1] - 4.02) <= 0.005  # the page's two-decimal value
    # log-sum-exp closed form: ln(2 e^{1/sqrt2}) and ln(1 + e^{1/sqrt2})
    lse_exact = [1 / math.sqrt(2) + math.log(2), math.log(1 + e)]
    assert np.abs(lse2[0, 0] - lse_exact).max() < 1e-12
    # causal: row 0 may only see key 0, so it equals V[0] exactly
    oc, _ = oracle.sdpa(Q, K, V, causal=True)
    assert np.array_equal(oc[0, 0, 0], [10.0, 0.0])
    assert np.abs(oc[0, 0, 1] - o_exact[1]).max() < 1e-12


def test_p4_ledger_from_printed_qkv(golden):
    """rockcohen.cc section 5.1 ledger: S = QK^T/sqrt2, A = softmax(S), z0;
    section 5.3 causal rows.  S is recovered from the oracle's outputs as
    log(A) + lse, so this also pins the log-sum-exp."""
    g = golden("p4_running_example_ledger.txt")
    Q, K, V = (g[n][None, None] for n in ("Q", "K", "V"))
    A, lse = weights_via_identity(Q, K)
    assert np.abs(A[0, 0] - g["A"]).max() < 2e-3
    S = np.log(A[0, 0]) + lse[0, 0][:, None]
    assert np.abs(S - g["S"]).max() < 2e-3
    o, _ = oracle.sdpa(Q, K, V)
    assert np.abs(o[0, 0, 0] - g["z0"][0]).max() < 2e-3
    Ac, _ = weights_via_identity(Q, K, causal=True)
    assert np.abs(Ac[0, 0, :2] - g["causal_rows_0_1"]).max() < 2e-3
    assert np.all(Ac[0, 0][np.triu_indices(4, 1)] == 0.0)


def test_p4_ledger_through_mha(golden):
    """The same ledger through the multi-head path with one head: projections
    X.W^Q, X.W^K, X.W^V (the page's orientation, W in R^{4x2}), then W^O that
    keeps the two attention columns.  Catches a transposed weight or a wrong
    projection operand."""
    g = golden("p4_running_example_ledger.txt")
    X = g["X"][None]
    WO = np.zeros((2, 4))
    WO[0, 0] = WO[1, 1] = 1.0
    y = oracle.mha(X, X, g["WQ"], g["WK"], g["WV"], WO, heads=1)
    assert np.abs(y[0, 0, :2] - g["z0"][0]).max() < 2e-3
    assert np.all(y[0, :, 2:] == 0.0)
    # the whole Z agrees with A.V from the printed ledger
    Z = g["A"] @ g["V"]
    assert np.abs(y[0, :, :2] - Z).max() < 2e-3
    # causal rows through the block (row 0 = V[0] of the projections)
    yc = oracle.mha(X, X, g["WQ"], g["WK"], g["WV"], WO, heads=1, causal=True)
    assert np.abs(yc[0, 0, :2] - (g["X"] @ g["WV"])[0]).max() < 1e-15


# ---------------------------------------------------------------------------
# Definition-level invariants (rockcohen.cc section 10.2, P0 and P1)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
def test_rows_sum_to_one(causal):
    B, H, n_q, n_kv, d = 2, 3, 37, 37, 16
    q, k = rnd(1, (B, H, n_q, d)), rnd(2, (B, H, n_kv, d))
    lkv = np.array([37, 5], np.int32)
    v = np.ones((B, H, n_kv, 3))
    o, _ = oracle.sdpa(q, k, v, causal=causal, seqlens_kv=lkv)
    assert np.abs(o - 1.0).max() < 1e-12
    P, _ = weights_via_identity(q, k, causal=causal, seqlens_kv=lkv)
    assert np.all(P >= 0)


def test_causal_upper_triangle_exact_zero_and_row0():
    """rockcohen.cc section 6.3: -inf at the softmax input gives weights that
    are exactly 0.0 for future keys; row 0 sees only key 0."""
    q, k = rnd(3, (1, 2, 20, 8)), rnd(4, (1, 2, 20, 8))
    P, _ = weights_via_identity(q, k, causal=True)
    iu = np.triu_indices(20, 1)
    assert np.all(P[:, :, iu[0], iu[1]] == 0.0)
    assert np.all(P[:, :, np.arange(20), np.arange(20)] > 0)  # diagonal is legal
    v = rnd(5, (1, 2, 20, 8))
    o, _ = oracle.sdpa(q, k, v, causal=True)
    assert np.array_equal(o[:, :, 0], v[:, :, 0])


def test_mask_equals_renormalising_over_legal_keys():
    """rockcohen.cc section 6.3: masking at the input equals a softmax over the
    legal set.  Causal row i == unmasked attention over keys 0..i; key padding
    == attention on the truncated K/V; padding is on keys, not queries."""
    q, k, v = rnd(6, (1, 1, 12, 8)), rnd(7, (1, 1, 12, 8)), rnd(8, (1, 1, 12, 5))
    oc, lc = oracle.sdpa(q, k, v, causal=True)
    for i in range(12):
        oi, li = oracle.sdpa(q[:, :, i:i + 1], k[:, :, :i + 1], v[:, :, :i + 1])
        assert np.abs(oc[0, 0, i] - oi[0, 0, 0]).max() < 1e-14
        assert abs(lc[0, 0, i] - li[0, 0, 0]) < 1e-14
    L = np.array([7], np.int32)
    kp, vp = k.copy(), v.copy()
    kp[:, :, 7:] = np.nan
    vp[:, :, 7:] = np.nan  # padding must never be read
    op, _ = oracle.sdpa(q, kp, vp, seqlens_kv=L)
    ot, _ = oracle.sdpa(q, k[:, :, :7], v[:, :, :7])
    assert np.abs(op - ot).max() < 1e-14
    # query lengths: rows past L_q are zero, the rest unchanged
    oq, lq = oracle.sdpa(q, k, v, seqlens_q=L)
    of, _ = oracle.sdpa(q, k, v)
    assert np.all(oq[:, :, 7:] == 0.0) and np.all(np.isneginf(lq[:, :, 7:]))
    assert np.array_equal(oq[:, :, :7], of[:, :, :7])


def test_empty_key_set_gives_zero_row():
    q, k, v = rnd(9, (2, 1, 4, 8)), rnd(10, (2, 1, 6, 8)), rnd(11, (2, 1, 6, 8))
    L = np.array([0, 6], np.int32)
    o, lse = oracle.sdpa(q, k, v, seqlens_kv=L)
    assert np.all(o[0] == 0.0) and np.all(np.isneginf(lse[0]))
    assert np.all(np.isfinite(o[1]))


def test_permutation_equivariance_and_key_invariance():
    """rockcohen.cc sections 3.4 and 6.2 (P1): without a mask,
    f(PQ, PK, PV) = P f(Q, K, V), and permuting keys with their values changes
    nothing."""
    q, k, v = rnd(12, (1, 2, 9, 8)), rnd(13, (1, 2, 9, 8)), rnd(14, (1, 2, 9, 8))
    perm = np.random.default_rng(0).permutation(9)
    o, _ = oracle.sdpa(q, k, v)
    op, _ = oracle.sdpa(q[:, :, perm], k[:, :, perm], v[:, :, perm])
    assert np.abs(op - o[:, :, perm]).max() < 1e-12
    ok, _ = oracle.sdpa(q, k[:, :, perm], v[:, :, perm])
    assert np.abs(ok - o).max() < 1e-12


def test_shift_invariance_and_overflow_safety():
    """rockcohen.cc section 3.2: adding a constant to a row of scores leaves the
    weights unchanged.  K_j + u for all j adds q.u to every score of row q.
    A large u (scores near +1e3) checks the max subtraction."""
    q, k, v = rnd(15, (1, 1, 10, 8)), rnd(16, (1, 1, 10, 8)), rnd(17, (1, 1, 10, 4))
    o, _ = oracle.sdpa(q, k, v)
    u = rnd(18, (8,))
    o1, _ = oracle.sdpa(q, k + u, v)
    assert np.abs(o1 - o).max() < 1e-12
    q2 = np.abs(q) + 1.0
    u_big = np.full(8, 400.0)  # q.u >= 3200 scaled by 1/sqrt(8): ~1e3
    o2, _ = oracle.sdpa(q2, k, v)
    o3, _ = oracle.sdpa(q2, k + u_big, v)
    assert np.all(np.isfinite(o3)) and np.abs(o3 - o2).max() < 1e-9


def test_scale_brings_score_variance_to_one():
    """vlmlib.cn summary / rockcohen.cc section 5.1 (paper footnote 4): for
    iid N(0,1) components, q.k has variance d_k; dividing by sqrt(d_k) brings
    it to 1.  Scores are recovered as log(P) + lse."""
    d = 64
    q, k = rnd(19, (1, 4, 64, d)), rnd(20, (1, 4, 64, d))
    P, lse = weights_via_identity(q, k)
    with np.errstate(divide="ignore", invalid="ignore"):   # a planted mistake may zero weights
        S = np.log(P) + lse[..., None]
        assert abs(S.var() - 1.0) < 0.1
    raw = q @ np.swapaxes(k, -1, -2)
    assert abs(np.abs(S * math.sqrt(d) - raw).max()) < 1e-10


def test_special_cases():
    q, k, v = rnd(21, (1, 1, 5, 8)), rnd(22, (1, 1, 7, 8)), rnd(23, (1, 1, 7, 6))
    # one key: the output is that value row
    o, _ = oracle.sdpa(q, k[:, :, :1], v[:, :, :1])
    assert np.array_equal(o, np.broadcast_to(v[:, :, :1], o.shape))
    # all-zero keys: uniform weights -> mean of the value rows
    o, _ = oracle.sdpa(q, np.zeros_like(k), v)
    assert np.abs(o - v.mean(axis=2, keepdims=True)).max() < 1e-14
    # value columns are independent: a column subset of V gives that subset of O
    o, _ = oracle.sdpa(q, k, v)
    o2, _ = oracle.sdpa(q, k, v[..., [1, 4]])
    assert np.array_equal(o2, o[..., [1, 4]])
    # huge scale -> softmax tends to argmax: output is the argmax row of V
    o, _ = oracle.sdpa(q, k, v, scale=1e6)
    idx = np.argmax(q[0, 0] @ k[0, 0].T, axis=1)
    assert np.abs(o[0, 0] - v[0, 0, idx]).max() < 1e-12


def test_bf16_storage_rounding_matches_torch():
    """Both roundings (generator's and the oracle's storage diagnostic) agree
    with torch's float32 -> bfloat16 conversion (round to nearest even)."""
    import torch
    x = gen.normal(24, (4096,)) * np.exp(gen.normal(25, (4096,)) * 4)
    x32 = x.astype(np.float32).astype(np.float64)  # values torch sees exactly
    ref = torch.tensor(x32, dtype=torch.float32).to(torch.bfloat16).double().numpy()
    assert np.array_equal(gen.round_to_bf16(x32), ref)
    assert np.array_equal(np.array([oracle.round_bf16(t) for t in x32[:512]]), ref[:512])
    ties = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8)])
    assert list(gen.round_to_bf16(ties)) == [1.0, 1 + 2 ** -6, -1.0]


def test_thread_count_independence():
    q, k, v = rnd(26, (2, 3, 33, 16)), rnd(27, (2, 3, 41, 16)), rnd(28, (2, 3, 41, 16))
    a, la = oracle.sdpa(q, k, v, causal=True, nthreads=1)
    b, lb = oracle.sdpa(q, k, v, causal=True, nthreads=7)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_rows_api_matches_full():
    q, k, v = rnd(29, (2, 3, 20, 8)), rnd(30, (2, 3, 25, 8)), rnd(31, (2, 3, 25, 8))
    L = np.array([25, 11], np.int32)
    o, lse = oracle.sdpa(q, k, v, causal=True, seqlens_kv=L)
    rows = np.array([0, 7, 19, 60, 101, 119])
    orr, lr = oracle.sdpa_rows(q, k, v, rows, causal=True, seqlens_kv=L)
    assert np.array_equal(orr, o.reshape(-1, 8)[rows])
    assert np.array_equal(lr, lse.reshape(-1)[rows])


# ---------------------------------------------------------------------------
# Multi-head attention (vlmlib.cn summary; rockcohen.cc section 5.2)
# ---------------------------------------------------------------------------
def _mha_case(seed, B=2, n_q=9, n_kv=11, dm=12, h=3):
    xq, xkv = rnd(seed, (B, n_q, dm)), rnd(seed + 1, (B, n_kv, dm))
    ws = [rnd(seed + 2 + t, (dm, dm)) * 0.3 for t in range(4)]
    return xq, xkv, ws, h


def test_mha_single_head_is_full_width_sdpa():
    """h = 1: MultiHead = Attention(XW^Q, XW^K, XW^V) W^O with scale
    1/sqrt(d_model) (projections by numpy matmul, Y = X.W)."""
    xq, xkv, (wq, wk, wv, wo), _ = _mha_case(40)
    y = oracle.mha(xq, xkv, wq, wk, wv, wo, heads=1, causal=False)
    o, _ = oracle.sdpa((xq @ wq)[:, None], (xkv @ wk)[:, None], (xkv @ wv)[:, None])
    assert np.abs(y - o[:, 0] @ wo).max() < 1e-12


def test_mha_concat_of_heads_on_column_slices():
    """With W^O = I the block output is Concat(head_1..head_h), head i using the
    contiguous columns [i*d_k, (i+1)*d_k) of each projection."""
    xq, xkv, (wq, wk, wv, wo), h = _mha_case(50)
    dm = wq.shape[0]
    dk = dm // h
    y = oracle.mha(xq, xkv, wq, wk, wv, np.eye(dm), heads=h, causal=True)
    for i in range(h):
        sl = slice(i * dk, (i + 1) * dk)
        o, _ = oracle.sdpa((xq @ wq[:, sl])[:, None], (xkv @ wk[:, sl])[:, None],
                           (xkv @ wv[:, sl])[:, None], causal=True)
        assert np.abs(y[:, :, sl] - o[:, 0]).max() < 1e-12
    # general W^O: Y = Concat . W^O
    y2 = oracle.mha(xq, xkv, wq, wk, wv, wo, heads=h, causal=True)
    assert np.abs(y2 - y @ wo).max() < 1e-12


def test_mha_head_isolation():
    """Perturbing head i's W^Q columns changes only head i's concat columns."""
    xq, xkv, (wq, wk, wv, _), h = _mha_case(60)
    dm = wq.shape[0]
    dk = dm // h
    y = oracle.mha(xq, xkv, wq, wk, wv, np.eye(dm), heads=h)
    wq2 = wq.copy()
    wq2[:, dk:2 * dk] += 0.5
    y2 = oracle.mha(xq, xkv, wq2, wk, wv, np.eye(dm), heads=h)
    changed = np.abs(y2 - y).max(axis=(0, 1)) > 0
    assert not changed[:dk].any() and changed[dk:2 * dk].all() and not changed[2 * dk:].any()


def test_mha_is_not_a_column_split_single_head():
    """rockcohen.cc section 5.2 / P5: per-head softmax and scale make the
    multi-head output differ from one full-width head."""
    xq, xkv, (wq, wk, wv, wo), _ = _mha_case(70, h=2)
    y1 = oracle.mha(xq, xkv, wq, wk, wv, wo, heads=1)
    y2 = oracle.mha(xq, xkv, wq, wk, wv, wo, heads=2)
    assert np.abs(y2 - y1).max() > 1e-3


def test_mha_self_attention_permutation_equivariance():
    """No mask, no positional encoding: f(PX) = P f(X) (rockcohen.cc 6.2)."""
    xq, _, (wq, wk, wv, wo), h = _mha_case(80)
    perm = np.random.default_rng(1).permutation(xq.shape[1])
    y = oracle.mha(xq, xq, wq, wk, wv, wo, heads=h)
    yp = oracle.mha(xq[:, perm], xq[:, perm], wq, wk, wv, wo, heads=h)
    assert np.abs(yp - y[:, perm]).max() < 1e-12


def test_mha_rows_and_lengths():
    xq, xkv, (wq, wk, wv, wo), h = _mha_case(90)
    Lq, Lkv = np.array([9, 4], np.int32), np.array([3, 11], np.int32)
    y = oracle.mha(xq, xkv, wq, wk, wv, wo, heads=h, seqlens_q=Lq, seqlens_kv=Lkv)
    assert np.all(y[1, 4:] == 0.0)
    rows = np.array([0, 5, 8, 9, 12, 17])
    yr = oracle.mha_rows(xq, xkv, wq, wk, wv, wo, heads=h, rows=rows, seqlens_q=Lq, seqlens_kv=Lkv)
    assert np.array_equal(yr, y.reshape(-1, y.shape[-1])[rows])
    # key padding on the block = the block on truncated keys
    yt = oracle.mha(xq[:1], xkv[:1, :3], wq, wk, wv, wo, heads=h)
    assert np.abs(y[0] - yt[0]).max() < 1e-13


def test_mha_bf16_storage_mode_is_close_but_distinct():
    xq, xkv, (wq, wk, wv, wo), h = _mha_case(100)
    y = oracle.mha(xq, xkv, wq, wk, wv, wo, heads=h)
    yr = oracle.mha(xq, xkv, wq, wk, wv, wo, heads=h, bf16_storage=True)
    d = np.abs(yr - y).max()
    assert 0 < d < 0.05


# ---------------------------------------------------------------------------
# One projection, y = x . W (paper section 3.2.2: X W_i^Q, X W_i^K, X W_i^V
# and Concat(...) W^O), which the library also exposes on its own
# ---------------------------------------------------------------------------
def test_linear_closed_form():
    """x[m, k] = m + 1 and w[k, n] = k + n give y[m, n] = (m + 1) (K(K-1)/2 + nK)
    exactly.  Catches a transposed weight (w[n][k] reads k + n too, so the
    non-square shape below is what separates them: K = 7, N = 3), a dropped or
    repeated term, and a row offset."""
    M, K, N = 4, 7, 3
    x = np.array([[m + 1.0] * K for m in range(M)])
    w = np.array([[k + n + 0.0 for n in range(N)] for k in range(K)])
    y = oracle.linear(x, w)
    ref = np.array([[(m + 1) * (K * (K - 1) / 2 + n * K) for n in range(N)] for m in range(M)])
    assert np.array_equal(y, ref)


def test_linear_special_cases():
    """Identity weights return x; a one-hot column of W copies one column of x
    (on a non-square W, so a transposed weight fails); zero weights give zeros;
    the row selection returns the selected rows of the full product."""
    x = rnd(302, (6, 8))
    assert np.array_equal(oracle.linear(x, np.eye(8)), x)
    w = np.zeros((8, 3))
    w[5, 1] = 1.0
    w[2, 2] = -2.0
    y = oracle.linear(x, w)
    assert np.array_equal(y[:, 0], np.zeros(6))
    assert np.array_equal(y[:, 1], x[:, 5])
    assert np.array_equal(y[:, 2], -2.0 * x[:, 2])
    w2 = rnd(303, (8, 5))
    full = oracle.linear(x, w2)
    assert np.array_equal(oracle.linear(x, w2, rows=[4, 0, 4]), full[[4, 0, 4]])


# ---------------------------------------------------------------------------
# One decoding step over a key/value cache (autoregressive generation:
# attention-paper-guide sections 05 and 07+, the csdn blog section 3.6)
# ---------------------------------------------------------------------------
def test_decode_last_rows_equal_full_causal_attention():
    """Generating one step at a time reproduces the decoder's masked attention:
    the newest n_q queries over the full cache give exactly the last n_q rows
    of causal self-attention over the whole sequence (the mask of rockcohen.cc
    5.3).  Catches an off-by-one or reversed alignment of the positions."""
    B, H, n, d, n_q = 2, 3, 23, 8, 4
    q, k, v = rnd(400, (B, H, n, d)), rnd(401, (B, H, n, d)), rnd(402, (B, H, n, d))
    o_full, lse_full = oracle.sdpa(q, k, v, causal=True)
    o, lse = oracle.decode(q[:, :, n - n_q:], k, v)
    assert np.array_equal(o, o_full[:, :, n - n_q:])
    assert np.array_equal(lse, lse_full[:, :, n - n_q:])


def test_decode_single_query_is_unmasked_attention_over_the_cache():
    """With one query the causal mask removes nothing inside the cache: the
    step equals unmasked attention over the first L_kv keys (and ignores what
    the cache holds beyond them, NaN included)."""
    B, H, n_kv, d = 3, 2, 17, 8
    q, k, v = rnd(410, (B, H, 1, d)), rnd(411, (B, H, n_kv, d)), rnd(412, (B, H, n_kv, d))
    L = np.array([17, 9, 1], np.int32)
    ref, ref_lse = oracle.sdpa(q, k, v, seqlens_kv=L)
    for b in range(B):
        k[b, :, L[b]:] = np.nan
        v[b, :, L[b]:] = np.nan
    o, lse = oracle.decode(q, k, v, seqlens_kv=L)
    assert np.array_equal(o, ref) and np.array_equal(lse, ref_lse)


def test_decode_per_sequence_lengths_and_short_sequences():
    """With cache lengths L_b the newest queries sit at L_b - n_q + i: equal to
    causal attention over the truncated sequence.  A sequence shorter than n_q
    leaves its first n_q - L_b queries without keys: zeros and -inf."""
    B, H, n_kv, d, n_q = 3, 2, 20, 8, 3
    q, k, v = rnd(420, (B, H, n_q, d)), rnd(421, (B, H, n_kv, d)), rnd(422, (B, H, n_kv, d))
    L = np.array([20, 11, 2], np.int32)
    o, lse = oracle.decode(q, k, v, seqlens_kv=L)
    for b in range(2):
        Lb = int(L[b])
        qq = np.concatenate([np.zeros((1, H, Lb - n_q, d)), q[b:b + 1]], axis=2)
        of, lf = oracle.sdpa(qq, k[b:b + 1, :, :Lb], v[b:b + 1, :, :Lb], causal=True)
        assert np.array_equal(o[b], of[0, :, Lb - n_q:])
        assert np.array_equal(lse[b], lf[0, :, Lb - n_q:])
    # L = 2 < n_q = 3: query 0 is position -1 (nothing), queries 1, 2 are positions 0, 1
    assert np.all(o[2, :, 0] == 0.0) and np.all(lse[2, :, 0] == -np.inf)
    of, lf = oracle.sdpa(q[2:3, :, 1:], k[2:3, :, :2], v[2:3, :, :2], causal=True)
    assert np.array_equal(o[2, :, 1:], of[0]) and np.array_equal(lse[2, :, 1:], lf[0])


# ---------------------------------------------------------------------------
# Restricted self-attention over a neighbourhood of radius r (the paper's
# proposal for very long inputs: the csdn blog section 4.3, the vlmlib.cn
# summary's limitations paragraph; reading: key j is legal iff |i - j| <= r)
# ---------------------------------------------------------------------------
def test_window_wider_than_the_sequence_is_full_attention():
    q, k, v = rnd(500, (2, 2, 19, 8)), rnd(501, (2, 2, 19, 8)), rnd(502, (2, 2, 19, 8))
    for causal in (False, True):
        full = oracle.sdpa(q, k, v, causal=causal)
        win = oracle.sdpa(q, k, v, causal=causal, window=18)
        assert np.array_equal(full[0], win[0]) and np.array_equal(full[1], win[1])
        # the largest radius the call takes: no overflow in the bounds, every key in the window
        wmax = oracle.sdpa(q, k, v, causal=causal, window=2 ** 31 - 1)
        assert np.array_equal(full[0], wmax[0]) and np.array_equal(full[1], wmax[1])


def test_window_zero_attends_to_itself():
    """r = 0 leaves the diagonal only: O[i] = V[i] exactly and lse = s_ii.
    Catches an off-by-one on either side of the band."""
    q, k, v = rnd(510, (1, 2, 9, 8)), rnd(511, (1, 2, 9, 8)), rnd(512, (1, 2, 9, 8))
    o, lse = oracle.sdpa(q, k, v, window=0, scale=0.3)
    assert np.array_equal(o, v)
    assert np.allclose(lse, 0.3 * np.einsum("bhid,bhid->bhi", q, k), rtol=0, atol=1e-13)


def test_window_equals_attention_over_the_neighbourhood():
    """Masking outside the band equals attention of each query over the sliced
    keys k[i-r .. i+r] (renormalising over the legal set, rockcohen.cc 6.3),
    with and without the causal mask and with key lengths."""
    B, H, n, d, r = 2, 2, 21, 8, 3
    q, k, v = rnd(520, (B, H, n, d)), rnd(521, (B, H, n, d)), rnd(522, (B, H, n, d))
    L = np.array([21, 12], np.int32)
    for causal in (False, True):
        o, lse = oracle.sdpa(q, k, v, causal=causal, window=r, seqlens_kv=L)
        for b in range(B):
            for i in range(n):
                lo, hi = max(0, i - r), min(int(L[b]), (i if causal else i + r) + 1)
                if hi <= lo:
                    assert np.all(o[b, :, i] == 0) and np.all(lse[b, :, i] == -np.inf)
                    continue
                ref, rl = oracle.sdpa(q[b:b + 1, :, i:i + 1], k[b:b + 1, :, lo:hi], v[b:b + 1, :, lo:hi])
                assert np.abs(o[b, :, i] - ref[0, :, 0]).max() < 1e-13
                assert np.abs(lse[b, :, i] - rl[0, :, 0]).max() < 1e-13


# ---------------------------------------------------------------------------
# Gradients of SDPA (the model is trained end to end: the vlmlib.cn summary's
# training-objective paragraph, attention-paper-guide section 05)
# ---------------------------------------------------------------------------
def _fd_grads(q, k, v, dout, h=1e-5, **kw):
    """Central finite differences of L = sum(dout * O) through the forward
    oracle (pinned above), element by element."""
    def loss(q_, k_, v_):
        return float((dout * oracle.sdpa(q_, k_, v_, **kw)[0]).sum())
    grads = []
    for which in range(3):
        base = [q, k, v]
        g = np.zeros_like(base[which])
        it = np.nditer(base[which], flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            plus = [a.copy() for a in base]
            minus = [a.copy() for a in base]
            plus[which][idx] += h
            minus[which][idx] -= h
            g[idx] = (loss(*plus) - loss(*minus)) / (2 * h)
        grads.append(g)
    return grads


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_matches_finite_differences(causal):
    """The analytic gradients agree with central differences of the forward
    (error O(h^2) ~ 1e-9).  Catches a dropped softmax-Jacobian term, a wrong
    sign, a missing scale, a transposed product or a wrong mask in the
    backward."""
    B, H, n_q, n_kv, d = 1, 2, 5, 6, 3
    q, k, v = rnd(600, (B, H, n_q, d)), rnd(601, (B, H, n_kv, d)), rnd(602, (B, H, n_kv, d))
    dout = rnd(603, (B, H, n_q, d))
    kw = dict(scale=0.7, causal=causal)
    dq, dk, dv = oracle.sdpa_bwd(q, k, v, dout, **kw)
    fq, fk, fv = _fd_grads(q, k, v, dout, **kw)
    for a, b_ in ((dq, fq), (dk, fk), (dv, fv)):
        assert np.abs(a - b_).max() < 1e-7 * (1 + np.abs(b_).max())


def test_bwd_with_lengths_matches_finite_differences():
    B, H, n_q, n_kv, d = 2, 1, 5, 6, 3
    q, k, v = rnd(610, (B, H, n_q, d)), rnd(611, (B, H, n_kv, d)), rnd(612, (B, H, n_kv, d))
    dout = rnd(613, (B, H, n_q, d))
    kw = dict(scale=0.5, causal=True, seqlens_q=np.array([5, 3], np.int32),
              seqlens_kv=np.array([6, 2], np.int32))
    dq, dk, dv = oracle.sdpa_bwd(q, k, v, dout, **kw)
    fq, fk, fv = _fd_grads(q, k, v, dout, **kw)
    for a, b_ in ((dq, fq), (dk, fk), (dv, fv)):
        assert np.abs(a - b_).max() < 1e-7 * (1 + np.abs(b_).max())
    # padded query rows and keys past the length get exactly zero gradient
    assert np.all(dq[1, :, 3:] == 0) and np.all(dk[1, :, 2:] == 0) and np.all(dv[1, :, 2:] == 0)


def test_bwd_special_cases():
    """One key: the weight is the constant 1, so dQ = dK = 0 and dV = sum_i dO_i.
    Zero dO gives zero gradients."""
    q, k, v = rnd(620, (1, 2, 4, 5)), rnd(621, (1, 2, 1, 5)), rnd(622, (1, 2, 1, 5))
    dout = rnd(623, (1, 2, 4, 5))
    dq, dk, dv = oracle.sdpa_bwd(q, k, v, dout)
    assert np.all(dq == 0) and np.all(dk == 0)
    assert np.allclose(dv[0, :, 0], dout[0].sum(axis=1), rtol=0, atol=1e-13)
    z = oracle.sdpa_bwd(q, k, v, np.zeros_like(dout))
    assert all(np.all(g == 0) for g in z)


# ---- positional encoding, LayerNorm and the attention sublayer --------------
def test_pe_closed_forms():
    """Position 0: every sine column is 0 and every cosine column 1.  The
    first pair has frequency 1 (10000^0), so its columns are sin(pos) and
    cos(pos) (the formula of paper section 3.5 on the vlmlib.cn summary and
    rockcohen.cc section 5.4)."""
    pe = oracle.positional_encoding(50, 16)
    assert np.all(pe[0, 0::2] == 0.0) and np.all(pe[0, 1::2] == 1.0)
    pos = np.arange(50)
    assert np.allclose(pe[:, 0], np.sin(pos), rtol=0, atol=1e-15)
    assert np.allclose(pe[:, 1], np.cos(pos), rtol=0, atol=1e-15)
    assert np.allclose(pe[:, 0::2] ** 2 + pe[:, 1::2] ** 2, 1.0, rtol=0, atol=1e-15)


def test_pe_wavelengths_geometric_from_2pi_to_10000_2pi():
    """rockcohen.cc section 5.4: the wavelengths form a geometric progression
    from 2*pi towards 10000*2*pi.  The angle of pair i at position 1 is its
    frequency; consecutive ratios are equal, the first frequency is 1 and the
    d/2-th power of the ratio is 1/10000."""
    d = 64
    pe = oracle.positional_encoding(2, d)
    w = np.arctan2(pe[1, 0::2], pe[1, 1::2])          # angle of each pair at pos = 1
    assert abs(w[0] - 1.0) < 1e-15
    ratio = w[1:] / w[:-1]
    assert np.allclose(ratio, ratio[0], rtol=1e-12, atol=0)
    assert abs(ratio[0] ** (d // 2) - 1e-4) < 1e-15


def test_pe_offset_is_a_linear_map():
    """For a fixed offset k, PE(pos + k) is a linear function of PE(pos) (the
    reason the paper gives for sinusoids, section 3.5: vlmlib.cn summary;
    rockcohen.cc section 5.4).  The map is built from PE(k) alone: each
    (sin, cos) pair rotates by its angle at position k."""
    d, n = 10, 60
    pe = oracle.positional_encoding(n, d)
    for k in (1, 7, 23):
        s_k, c_k = pe[k, 0::2], pe[k, 1::2]
        for pos in (0, 3, 17, n - 1 - k):
            s, c = pe[pos, 0::2], pe[pos, 1::2]
            pred = np.empty(d)
            pred[0::2] = s * c_k + c * s_k                # sin(a + b)
            pred[1::2] = c * c_k - s * s_k                # cos(a + b)
            assert np.allclose(pe[pos + k], pred, rtol=0, atol=1e-12)


def test_layernorm_scale_and_shift_invariance():
    """rockcohen.cc section 5.5 (reproduction P6): LN(c z) = LN(z) for c = 1e3
    and 1e-3, and LN(z + 1) = LN(z): LayerNorm removes the mean and the scale
    of a row (eps = 0 here)."""
    z = rnd(700, (5, 12))
    g, b = np.ones(12), np.zeros(12)
    base = oracle.layernorm(z, g, b, 0.0)
    for c in (1e3, 1e-3):
        assert np.abs(oracle.layernorm(c * z, g, b, 0.0) - base).max() < 1e-12
    assert np.abs(oracle.layernorm(z + 1.0, g, b, 0.0) - base).max() < 1e-12
    assert np.abs(oracle.layernorm(3.0 * z - 7.0, g, b, 0.0) - base).max() < 1e-12


def test_layernorm_moments_and_affine():
    """With gain 1 and bias 0 each row has mean 0 and mean square 1 (the
    population variance: dividing by d, not d - 1); the gain and bias then
    act per column; eps sits inside the square root: the row [-1, 1] has
    variance 1, so it maps to gamma*(+-1)/sqrt(1 + eps) + beta; a constant row
    maps to beta."""
    z = rnd(701, (4, 9))
    y = oracle.layernorm(z, np.ones(9), np.zeros(9), 0.0)
    assert np.abs(y.mean(axis=1)).max() < 1e-14
    assert np.abs((y ** 2).mean(axis=1) - 1.0).max() < 1e-13
    g, b = rnd(702, (9,)), rnd(703, (9,))
    assert np.abs(oracle.layernorm(z, g, b, 0.0) - (y * g + b)).max() < 1e-13
    eps = 0.25
    y2 = oracle.layernorm(np.array([[-1.0, 1.0]]), np.array([2.0, 3.0]), np.array([0.5, -0.5]), eps)
    assert np.allclose(y2, [[-2.0 / np.sqrt(1.25) + 0.5, 3.0 / np.sqrt(1.25) - 0.5]], rtol=0, atol=1e-15)
    y3 = oracle.layernorm(np.full((1, 5), 4.2), np.ones(5), np.arange(5.0), 1e-5)
    assert np.array_equal(y3, np.arange(5.0)[None, :])


def _block_inputs(seed, B=2, n=7, dm=8, heads=2, d=4):
    x = rnd(seed, (B, n, dm))
    ws = [rnd(seed + 1 + t, shape) * 0.3 for t, shape in
          enumerate([(dm, heads * d), (dm, heads * d), (dm, heads * d), (heads * d, dm)])]
    g, b = 1.0 + 0.1 * rnd(seed + 5, (dm,)), 0.1 * rnd(seed + 6, (dm,))
    return x, ws, g, b


def test_block_is_layernorm_of_residual_plus_mha():
    """The sublayer is LayerNorm(h + MultiHead(h)) with h = x + PE (paper
    section 3.1 post-LN, vlmlib.cn summary; section 3.5 for the PE), checked
    against the separately pinned parts; with W^O = 0 the attention adds
    nothing and y = LN(x + PE); with gain 0, y = beta exactly."""
    x, (wq, wk, wv, wo), g, b = _block_inputs(710)
    h = x + oracle.positional_encoding(7, 8)[None]
    y, z = oracle.mha_block(x, wq, wk, wv, wo, g, b, heads=2, add_pe=True, eps=1e-5, causal=True)
    m = oracle.mha(h, h, wq, wk, wv, wo, heads=2, causal=True)
    assert np.abs(z - (h + m)).max() < 1e-13
    assert np.abs(y - oracle.layernorm(h + m, g, b, 1e-5)).max() < 1e-13
    y0, _ = oracle.mha_block(x, wq, wk, wv, np.zeros_like(wo), g, b, heads=2, add_pe=True, eps=1e-5)
    assert np.abs(y0 - oracle.layernorm(h, g, b, 1e-5)).max() < 1e-13
    yb, _ = oracle.mha_block(x, wq, wk, wv, wo, np.zeros(8), b, heads=2, add_pe=True)
    assert np.array_equal(yb, np.broadcast_to(b, yb.shape))


def test_block_cross_and_rows():
    """Cross-attention sublayer: z = x_q + MultiHead(x_q, x_kv, x_kv), no PE;
    the row-selected form equals the full one."""
    x, (wq, wk, wv, wo), g, b = _block_inputs(720)
    xkv = rnd(727, (2, 5, 8))
    y, z = oracle.mha_block(x, wq, wk, wv, wo, g, b, heads=2, x_kv=xkv, seqlens_kv=[5, 2])
    m = oracle.mha(x, xkv, wq, wk, wv, wo, heads=2, seqlens_kv=[5, 2])
    assert np.abs(z - (x + m)).max() < 1e-13
    rows = [0, 6, 9, 13]
    yr, zr = oracle.mha_block_rows(x, wq, wk, wv, wo, g, b, heads=2, rows=rows, x_kv=xkv,
                                   seqlens_kv=[5, 2])
    assert np.array_equal(yr, y.reshape(-1, 8)[rows]) and np.array_equal(zr, z.reshape(-1, 8)[rows])
    ys, _ = oracle.mha_block(x, wq, wk, wv, wo, g, b, heads=2, add_pe=True, causal=True)
    ysr, _ = oracle.mha_block_rows(x, wq, wk, wv, wo, g, b, heads=2, rows=rows, add_pe=True, causal=True)
    assert np.array_equal(ysr, ys.reshape(-1, 8)[rows])


# ---------------------------------------------------------------------------
# Brute force at 50 digits on tiny shapes: Eq. 1 evaluated literally (no max
# shift, no reordering) in mpmath, against the oracle's fp64 stable form.
# ---------------------------------------------------------------------------
def _mp_sdpa_row(mp, q, K, V, scale, legal):
    s = [scale * mp.fsum(mp.mpf(a) * mp.mpf(b) for a, b in zip(q, K[j])) for j in legal]
    e = [mp.exp(x) for x in s]
    z = mp.fsum(e)
    o = [mp.fsum(e[t] * mp.mpf(V[j][c]) for t, j in enumerate(legal)) / z for c in range(len(V[0]))]
    return o, mp.log(z)


@pytest.mark.parametrize("n_q,n_kv,d,causal,lkv", [(2, 2, 2, False, None), (3, 4, 5, True, None),
                                                    (4, 3, 3, False, [2]), (4, 4, 4, True, [3])])
def test_sdpa_matches_50_digit_brute_force(n_q, n_kv, d, causal, lkv):
    """The oracle's fp64 result (max shift, fixed summation order) equals the
    definition evaluated at 50 significant digits to 1e-13.  Catches any
    cancellation or shift mistake that the closed forms above would not see
    at these sizes."""
    mp = pytest.importorskip("mpmath")
    mp.mp.dps = 50
    q, k, v = rnd(8101, (1, 1, n_q, d)) * 3, rnd(8102, (1, 1, n_kv, d)) * 3, rnd(8103, (1, 1, n_kv, d))
    scale = 1 / math.sqrt(d)
    lk = None if lkv is None else np.array(lkv, np.int32)
    o, lse = oracle.sdpa(q, k, v, scale=scale, causal=causal, seqlens_kv=lk)
    L = n_kv if lkv is None else lkv[0]
    for i in range(n_q):
        legal = [j for j in range(L) if not (causal and j > i)]
        if not legal:
            assert np.all(o[0, 0, i] == 0.0) and lse[0, 0, i] == -np.inf
            continue
        o_mp, lse_mp = _mp_sdpa_row(mp, q[0, 0, i], k[0, 0], v[0, 0], mp.mpf(scale), legal)
        assert max(abs(float(o_mp[c]) - o[0, 0, i, c]) for c in range(d)) <= 1e-13
        assert abs(float(lse_mp) - lse[0, 0, i]) <= 1e-13


def test_mha_matches_50_digit_brute_force():
    """MultiHead(X, X, X) = Concat(head_1, head_2) W^O with head_i =
    Attention(X W^Q_i, X W^K_i, X W^V_i) (section 3.2.2), two heads of size
    2, evaluated at 50 digits: equals the oracle to 1e-13."""
    mp = pytest.importorskip("mpmath")
    mp.mp.dps = 50
    n, dm, h = 3, 4, 2
    x = rnd(8111, (1, n, dm))
    w = [rnd(8112 + t, (dm, dm)) * 0.5 for t in range(4)]
    y = oracle.mha(x, x, *w, heads=h, causal=True)
    X = mp.matrix(x[0].tolist())
    Wq, Wk, Wv, Wo = (mp.matrix(m.tolist()) for m in w)
    Qp, Kp, Vp = X * Wq, X * Wk, X * Wv
    dk = dm // h
    cat = mp.matrix(n, dm)
    for hh in range(h):
        cols = range(hh * dk, (hh + 1) * dk)
        for i in range(n):
            row, _ = _mp_sdpa_row(mp, [Qp[i, c] for c in cols], [[Kp[j, c] for c in cols] for j in range(n)],
                                  [[Vp[j, c] for c in cols] for j in range(n)], 1 / mp.sqrt(dk),
                                  list(range(i + 1)))
            for t, c in enumerate(cols):
                cat[i, c] = row[t]
    Y = cat * Wo
    assert max(abs(float(Y[i, c]) - y[0, i, c]) for i in range(n) for c in range(dm)) <= 1e-13
