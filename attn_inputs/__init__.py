"""Seeded synthetic inputs for the attention workloads.

This module is shared by the oracle-side tests and by the GPU-side tests and
bench; it holds none of the attention arithmetic.  It produces exact fp64
values already rounded to the storage dtype, plus the storage bytes, so both
sides see bit-identical inputs.

Random numbers: SplitMix64 (G. Steele, D. Lea, C. Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014) -> doubles in (0,1) from the top
53 bits -> normals by the Box-Muller transform.  Weight init is the
Glorot-Bengio ("Xavier") uniform U(-a, a), a = sqrt(6 / (fan_in + fan_out)).
The positional encoding is the sinusoidal one of "Attention Is All You Need"
section 3.5: even dimension 2i gets sin(pos / 10000^(2i/d_model)), odd
dimension 2i+1 gets cos of the same angle, positions counted from 0.

Rounding to bf16 is round-to-nearest-even, computed directly from fp64 (no
double rounding through fp32).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def splitmix64(seed: int, n: int) -> np.ndarray:
    """The first n outputs of SplitMix64 started at state `seed` (uint64)."""
    with np.errstate(over="ignore"):
        state = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + _GOLDEN * np.arange(1, n + 1, dtype=np.uint64)
        z = state
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        return z ^ (z >> np.uint64(31))


def uniform01(seed: int, n: int) -> np.ndarray:
    """n doubles in the open interval (0, 1): ((x >> 11) + 0.5) * 2^-53."""
    return ((splitmix64(seed, n) >> np.uint64(11)).astype(np.float64) + 0.5) * (2.0 ** -53)


def normal(seed: int, shape) -> np.ndarray:
    """iid N(0,1) in fp64 via Box-Muller on consecutive uniform pairs."""
    n = int(np.prod(shape))
    pairs = (n + 1) // 2
    u = uniform01(seed, 2 * pairs)
    u1, u2 = u[0::2], u[1::2]
    r = np.sqrt(-2.0 * np.log(u1))
    z = np.empty(2 * pairs)
    z[0::2] = r * np.cos(2.0 * np.pi * u2)
    z[1::2] = r * np.sin(2.0 * np.pi * u2)
    return z[:n].reshape(shape)


def uniform(seed: int, shape, lo: float, hi: float) -> np.ndarray:
    n = int(np.prod(shape))
    return (lo + (hi - lo) * uniform01(seed, n)).reshape(shape)


def xavier_bound(fan_in: int, fan_out: int) -> float:
    return math.sqrt(6.0 / (fan_in + fan_out))


def xavier_uniform(seed: int, fan_in: int, fan_out: int) -> np.ndarray:
    """[fan_in, fan_out] weights, U(-a, a) with a = sqrt(6/(fan_in+fan_out))."""
    a = xavier_bound(fan_in, fan_out)
    return uniform(seed, (fan_in, fan_out), -a, a)


def int_uniform(seed: int, n: int, lo: int, hi: int) -> np.ndarray:
    """n integers uniform on {lo, ..., hi} (inclusive), int32."""
    u = uniform01(seed, n)
    return (lo + np.floor(u * (hi - lo + 1))).astype(np.int32)


def sinusoidal_pe(n: int, d_model: int) -> np.ndarray:
    """[n, d_model] fp64 positional encoding (sin on even, cos on odd dims)."""
    pos = np.arange(n, dtype=np.float64)[:, None]
    i2 = np.arange(0, d_model, 2, dtype=np.float64)[None, :]
    angle = pos / np.power(10000.0, i2 / d_model)
    pe = np.empty((n, d_model))
    pe[:, 0::2] = np.sin(angle)
    pe[:, 1::2] = np.cos(angle[:, : d_model // 2])
    return pe


# ---- storage rounding ------------------------------------------------------
def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """fp64 -> nearest bf16 value (ties to even), returned as fp64.  The bf16
    spacing near x is 2^(e-7) with 2^e <= |x| (e clamped at -126); x/spacing is
    exact and np.rint rounds half to even."""
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    fin = np.isfinite(x) & (x != 0)
    _, e = np.frexp(x[fin])
    ex = np.maximum(e - 1, -126)
    spacing = np.ldexp(1.0, ex - 7)
    r = np.rint(x[fin] / spacing) * spacing
    r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, x[fin]), r)
    out[fin] = r
    return out


def bf16_bits(x_bf16_exact: np.ndarray) -> np.ndarray:
    """uint16 storage of values that are already exactly bf16 (NaN -> 0x7FC0).
    Raises if a value is not exactly representable (round it first)."""
    x = np.asarray(x_bf16_exact, dtype=np.float64)
    fin = np.isfinite(x)
    if not np.array_equal(x[fin], round_to_bf16(x[fin])):
        raise ValueError("bf16_bits: values are not exactly bf16; round them first")
    f32 = x.astype(np.float32)
    bits = (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits[np.isnan(f32)] = 0x7FC0
    return bits


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def round_to_f32(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 values representable in `dtype` ('bf16' or 'f32')."""
    if dtype == "bf16":
        return round_to_bf16(x)
    if dtype == "f32":
        return round_to_f32(x)
    raise ValueError(dtype)


def storage(x_exact: np.ndarray, dtype: str) -> np.ndarray:
    """Storage array for exact values: uint16 bits for bf16, float32 for f32."""
    if dtype == "bf16":
        return bf16_bits(x_exact)
    return np.asarray(x_exact, dtype=np.float32)


# ---- the five workloads ----------------------------------------------------
@dataclass
class SDPAInputs:
    """One SDPA workload.  q/k/v are exact fp64 values ([B,H,n,d], BHND),
    with padding positions set to NaN; *_st are the storage arrays."""
    name: str
    dtype: str
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    scale: float
    causal: bool
    seqlens_q: np.ndarray | None
    seqlens_kv: np.ndarray | None
    q_st: np.ndarray = field(repr=False, default=None)
    k_st: np.ndarray = field(repr=False, default=None)
    v_st: np.ndarray = field(repr=False, default=None)

    @property
    def shape(self):
        B, H, n_q, d_k = self.q.shape
        return B, H, n_q, self.k.shape[2], d_k, self.v.shape[3]


@dataclass
class MHAInputs:
    name: str
    dtype: str
    x: np.ndarray            # [B, n, d_model], exact
    w_q: np.ndarray
    w_k: np.ndarray
    w_v: np.ndarray
    w_o: np.ndarray
    heads: int
    scale: float
    causal: bool
    x_st: np.ndarray = field(repr=False, default=None)
    w_st: tuple = field(repr=False, default=None)


def _seed(cfg: int, t: int) -> int:
    """Seed scheme: workload c uses seed 1000*c + t with t = 0 Q/X, 1 K, 2 V,
    3 lengths, 4..7 W^Q, W^K, W^V, W^O."""
    return 1000 * cfg + t


def make_sdpa(name, dtype, B, H, n_q, n_kv, d_k, d_v, scale, causal, seqlens_q=None,
              seqlens_kv=None, cfg_id=0, nan_padding=True) -> SDPAInputs:
    """iid N(0,1) Q/K/V, rounded to dtype; positions beyond the lengths are NaN."""
    q = to_dtype(normal(_seed(cfg_id, 0), (B, H, n_q, d_k)), dtype)
    k = to_dtype(normal(_seed(cfg_id, 1), (B, H, n_kv, d_k)), dtype)
    v = to_dtype(normal(_seed(cfg_id, 2), (B, H, n_kv, d_v)), dtype)
    if nan_padding:
        for b in range(B):
            if seqlens_kv is not None:
                k[b, :, seqlens_kv[b]:, :] = np.nan
                v[b, :, seqlens_kv[b]:, :] = np.nan
            if seqlens_q is not None:
                q[b, :, seqlens_q[b]:, :] = np.nan
    inp = SDPAInputs(name, dtype, q, k, v, scale, causal, seqlens_q, seqlens_kv)
    inp.q_st, inp.k_st, inp.v_st = storage(q, dtype), storage(k, dtype), storage(v, dtype)
    return inp


def config(c: int, **overrides):
    """The five named workloads (sizes as stated in each docstring line):
      1  single-head SDPA fp32, [1,1,16,64], no mask, scale 1/8
      2  encoder self-attention bf16, [32,8,128,64], lengths U{16..128} on queries
         and keys, bidirectional
      3  decoder masked self-attention bf16, [32,8,256,64], causal
      4  cross-attention bf16, Q [16,16,256,64], K/V [16,16,320,64], key lengths
         U{160..320}, no query lengths
      5  multi-head block bf16: X [4,4096,1024] = N(0,1) + PE, Xavier W [1024,1024] x4,
         h=16, d_k=64, causal
    `overrides` may shrink batch/lengths for reduced-size parity cases."""
    if c == 1:
        p = dict(B=1, H=1, n=16)
        p.update(overrides)
        return make_sdpa("sdpa_f32_1x1x16x64", "f32", p["B"], p["H"], p["n"], p["n"], 64, 64,
                         0.125, False, cfg_id=1)
    if c == 2:
        p = dict(B=32, H=8, n=128, lo=16)
        p.update(overrides)
        L = int_uniform(_seed(2, 3), p["B"], min(p["lo"], p["n"]), p["n"])
        return make_sdpa("encoder_self_bf16_32x8x128x64_padded", "bf16", p["B"], p["H"], p["n"],
                         p["n"], 64, 64, 0.125, False, seqlens_q=L, seqlens_kv=L, cfg_id=2)
    if c == 3:
        p = dict(B=32, H=8, n=256)
        p.update(overrides)
        return make_sdpa("decoder_causal_bf16_32x8x256x64", "bf16", p["B"], p["H"], p["n"], p["n"],
                         64, 64, 0.125, True, cfg_id=3)
    if c == 4:
        p = dict(B=16, H=16, n_q=256, n_kv=320, lo=160)
        p.update(overrides)
        L = int_uniform(_seed(4, 3), p["B"], min(p["lo"], p["n_kv"]), p["n_kv"])
        return make_sdpa("cross_bf16_16x16x256x320x64_padded", "bf16", p["B"], p["H"], p["n_q"],
                         p["n_kv"], 64, 64, 0.125, False, seqlens_kv=L, cfg_id=4)
    if c == 5:
        p = dict(B=4, n=4096, d_model=1024, heads=16)
        p.update(overrides)
        B, n, dm, h = p["B"], p["n"], p["d_model"], p["heads"]
        x = to_dtype(normal(_seed(5, 0), (B, n, dm)) + sinusoidal_pe(n, dm)[None], "bf16")
        ws = [to_dtype(xavier_uniform(_seed(5, 4 + t), dm, dm), "bf16") for t in range(4)]
        inp = MHAInputs("mha_block_bf16_4x4096x1024_h16_causal", "bf16", x, *ws, heads=h,
                        scale=1.0 / math.sqrt(dm // h), causal=True)
        inp.x_st = bf16_bits(x)
        inp.w_st = tuple(bf16_bits(w) for w in ws)
        return inp
    raise ValueError(c)


def decode_workload(**overrides):
    """One decoding step over a key/value cache (bf16, head size 64): B = 16
    sequences x 16 heads (the big model's head count), one new query each, a
    cache of capacity 4096 (the block's sequence length) holding L ~ U{1024..4096}
    positions per sequence; cache rows beyond L are NaN.  Seeds 1000*6 + t as
    for the named workloads.  `overrides` may shrink any size or give the
    lengths L explicitly."""
    p = dict(B=16, H=16, n_q=1, n_kv=4096, lo=1024, L=None)
    p.update(overrides)
    L = (int_uniform(_seed(6, 3), p["B"], min(p["lo"], p["n_kv"]), p["n_kv"]) if p["L"] is None
         else np.asarray(p["L"], dtype=np.int32))
    return make_sdpa(f"decode_bf16_{p['B']}x{p['H']}x{p['n_q']}q_cache{p['n_kv']}", "bf16", p["B"],
                     p["H"], p["n_q"], p["n_kv"], 64, 64, 0.125, False, seqlens_kv=L, cfg_id=6)


def make_dout(inp: SDPAInputs, cfg_id: int) -> tuple[np.ndarray, np.ndarray]:
    """Gradient at the attention output for a backward pass over `inp`: iid
    N(0,1) rounded to the inputs' dtype, seed 1000*cfg_id + 8, rows beyond the
    query lengths NaN.  Returns (exact fp64 values, storage array)."""
    B, H, n_q, _, _, d_v = inp.shape
    g = to_dtype(normal(_seed(cfg_id, 8), (B, H, n_q, d_v)), inp.dtype)
    if inp.seqlens_q is not None:
        for b in range(B):
            g[b, :, inp.seqlens_q[b]:, :] = np.nan
    return g, storage(g, inp.dtype)


def backward_workload(**overrides) -> tuple[SDPAInputs, np.ndarray, np.ndarray]:
    """Gradients of the block's attention: [4,16,4096,64] bf16, causal, scale
    1/8, Q/K/V and dO iid N(0,1) (the per-head shape of the multi-head block,
    workload 5).  Seeds 1000*8 + t.  `overrides` may shrink any size."""
    p = dict(B=4, H=16, n=4096)
    p.update(overrides)
    inp = make_sdpa(f"backward_bf16_{p['B']}x{p['H']}x{p['n']}x64_causal", "bf16", p["B"], p["H"],
                    p["n"], p["n"], 64, 64, 0.125, True, cfg_id=8)
    g, g_st = make_dout(inp, 8)
    return inp, g, g_st


def sublayer_workload(**overrides):
    """The attention sublayer of the big model at the block's shape: token
    embeddings X [4, 4096, 1024] ~ N(0,1) (the positional encoding is added by
    the sublayer itself), Xavier W^Q, W^K, W^V, W^O [1024, 1024], LayerNorm
    gain 1 + 0.1 N(0,1) and bias 0.1 N(0,1), h = 16, causal; all bf16.  Seeds
    1000*9 + t (t = 0 X, 4..7 the weights, 8 and 9 gain and bias).
    `overrides` may shrink any size.  Returns (x, [w_q, w_k, w_v, w_o], gamma,
    beta, heads) as exact fp64 values."""
    p = dict(B=4, n=4096, d_model=1024, heads=16)
    p.update(overrides)
    B, n, dm, h = p["B"], p["n"], p["d_model"], p["heads"]
    x = to_dtype(normal(_seed(9, 0), (B, n, dm)), "bf16")
    ws = [to_dtype(xavier_uniform(_seed(9, 4 + t), dm, dm), "bf16") for t in range(4)]
    gamma = to_dtype(1.0 + 0.1 * normal(_seed(9, 8), (dm,)), "bf16")
    beta = to_dtype(0.1 * normal(_seed(9, 9), (dm,)), "bf16")
    return x, ws, gamma, beta, h
