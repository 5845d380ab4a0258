"""The seeded input generator: determinism, published known answers and
distribution properties."""
import math

import numpy as np

import attn_inputs as gen


def test_splitmix64_known_answer():
    # SplitMix64 from state 0: the first four outputs of the published generator
    assert [int(x) for x in gen.splitmix64(0, 4)] == [
        0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F, 0xF88BB8A8724C81EC]


def test_uniform_open_interval_and_determinism():
    u = gen.uniform01(7, 100000)
    assert u.min() > 0 and u.max() < 1
    assert np.array_equal(u, gen.uniform01(7, 100000))
    assert abs(u.mean() - 0.5) < 5e-3


def test_normal_moments_and_ks():
    from scipy import stats
    z = gen.normal(11, (200001,))
    assert abs(z.mean()) < 0.01 and abs(z.var() - 1) < 0.01
    assert stats.kstest(z, "norm").pvalue > 1e-3


def test_xavier_bound_and_variance():
    w = gen.xavier_uniform(5, 1024, 1024)
    a = math.sqrt(6 / 2048)
    assert abs(a - 0.0541266) < 1e-6
    assert np.abs(w).max() <= a
    assert abs(w.var() - 1 / 1024) < 2e-5  # U(-a,a) variance a^2/3 = 2/(fan_in+fan_out)


def test_lengths_inclusive_range():
    L = gen.int_uniform(3, 20000, 16, 128)
    assert L.min() == 16 and L.max() == 128 and L.dtype == np.int32


def test_positional_encoding_identities():
    """Sinusoidal PE (paper section 3.5): PE(0, 2i) = 0, PE(0, 2i+1) = 1, and
    for a fixed offset k, (PE(p+k, 2i), PE(p+k, 2i+1)) is a rotation of
    (PE(p, 2i), PE(p, 2i+1)) by the angle k * omega_i (angle addition)."""
    d = 1024
    pe = gen.sinusoidal_pe(300, d)
    assert np.all(pe[0, 0::2] == 0.0) and np.all(pe[0, 1::2] == 1.0)
    omega = 1.0 / np.power(10000.0, np.arange(0, d, 2) / d)
    for k in (1, 7, 100):
        c, s = np.cos(k * omega), np.sin(k * omega)
        sin_p, cos_p = pe[:-k, 0::2], pe[:-k, 1::2]
        assert np.abs(pe[k:, 0::2] - (sin_p * c + cos_p * s)).max() < 1e-10
        assert np.abs(pe[k:, 1::2] - (cos_p * c - sin_p * s)).max() < 1e-10
    # wavelengths form a geometric progression from 2*pi to 10000*2*pi
    assert abs(omega[0] - 1.0) < 1e-15 and omega[-1] > 1e-4 * 1.0


def test_configs_shapes_padding_and_storage():
    c2 = gen.config(2, B=4)
    B, H, n_q, n_kv, dk, dv = c2.shape
    assert (H, n_q, dk) == (8, 128, 64)
    for b in range(B):
        L = c2.seqlens_kv[b]
        assert np.all(np.isnan(c2.k[b, :, L:])) and np.all(np.isfinite(c2.k[b, :, :L]))
        assert np.all(np.isnan(c2.q[b, :, L:]))
    # storage bits decode back to the exact values
    assert np.array_equal(gen.bf16_bits_to_f64(c2.q_st)[np.isfinite(c2.q)], c2.q[np.isfinite(c2.q)])
    c4 = gen.config(4, B=2)
    assert c4.seqlens_q is None and c4.shape[3] == 320
    c1 = gen.config(1)
    assert c1.q_st.dtype == np.float32 and c1.scale == 0.125
    c5 = gen.config(5, B=1, n=64)
    assert c5.x.shape == (1, 64, 1024) and c5.heads == 16
    # bf16 storage may round a weight up to the bf16 value nearest the bound
    assert np.abs(c5.w_q).max() <= gen.round_to_bf16(np.array([math.sqrt(6 / 2048)]))[0]
