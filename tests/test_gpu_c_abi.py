"""The library used from a C program through its C ABI alone, with no Python
and no torch in the GPU process: tests/c_abi/sdpa_driver (built by
__graft_entry__.build()) runs attn_sdpa_fwd on bf16 inputs this test writes,
and its O and log-sum-exp are checked against the fp64 oracle with the same
tolerances as the Python-side tests (max-abs 2e-2 on O; rows without a legal
key exactly zero)."""
import os
import struct
import subprocess

import numpy as np
import pytest

import attn_inputs as gen
import oracle
from conftest import ROOT
from gpu_helpers import announce

pytestmark = pytest.mark.gpu

DRIVER = os.path.join(ROOT, "tests", "c_abi", "sdpa_driver")
LSE_TOL = 4e-3   # the bf16 path's bound on the log-sum-exp (see test_gpu_sdpa.py)

CASES = [
    dict(name="c_abi_causal", B=2, H=3, n_q=200, n_kv=200, causal=True, lq=None, lkv=None),
    dict(name="c_abi_cross_lengths", B=2, H=2, n_q=130, n_kv=330, causal=False, lq=[130, 57], lkv=[330, 0]),
]


@pytest.mark.parametrize("c", CASES, ids=[c["name"] for c in CASES])
def test_c_program_through_the_abi(c, tmp_path):
    assert os.path.exists(DRIVER), "the C-ABI test program is missing: run __graft_entry__.build()"
    lq = None if c["lq"] is None else np.array(c["lq"], np.int32)
    lkv = None if c["lkv"] is None else np.array(c["lkv"], np.int32)
    B, H, n_q, n_kv = c["B"], c["H"], c["n_q"], c["n_kv"]
    inp = gen.make_sdpa(c["name"], "bf16", B, H, n_q, n_kv, 64, 64, 0.125, c["causal"], lq, lkv, cfg_id=95)
    fin, fout = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(fin, "wb") as f:
        f.write(struct.pack("<6if", B, H, n_q, n_kv, int(c["causal"]), int(lq is not None), 0.125))
        if lq is not None:
            f.write(lq.astype("<i4").tobytes())
            f.write(lkv.astype("<i4").tobytes())
        for a in (inp.q_st, inp.k_st, inp.v_st):
            f.write(np.ascontiguousarray(a, dtype="<u2").tobytes())
    announce(f"C driver {c['name']} B={B} H={H} n_q={n_q} n_kv={n_kv} causal={c['causal']} lq={c['lq']} lkv={c['lkv']}")
    run = subprocess.run([DRIVER, str(fin), str(fout)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stderr
    raw = open(fout, "rb").read()
    n_o = B * H * n_q * 64
    o = gen.bf16_bits_to_f64(np.frombuffer(raw[:2 * n_o], dtype="<u2")).reshape(B, H, n_q, 64)
    lse = np.frombuffer(raw[2 * n_o:], dtype="<f4").astype(np.float64).reshape(B, H, n_q)
    o_ref, lse_ref = oracle.sdpa(inp.q, inp.k, inp.v, scale=0.125, causal=c["causal"], seqlens_q=lq, seqlens_kv=lkv)
    err = float(np.abs(o - o_ref).max())
    print(f"  {c['name']}: max|C driver - oracle| = {err:.3e}", flush=True)
    assert err <= 2e-2
    zero = np.isneginf(lse_ref)
    assert np.all(o[zero] == 0.0) and np.all(np.isneginf(lse[zero]))
    ok = ~zero
    assert np.all(np.abs(lse[ok] - lse_ref[ok]) / np.maximum(1.0, np.abs(lse_ref[ok])) <= LSE_TOL)
