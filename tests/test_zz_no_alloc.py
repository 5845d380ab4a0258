"""attn_sdpa_bwd_noalloc (no workspace argument: the library's fixed
per-device scratch) against attn_sdpa_bwd with a caller workspace, through
the C ABI: the same kernels, so the gradients must agree bit for bit; two
calls in a row, the second smaller than the first (the scratch keeps the
first call's contents, which the second must not see)."""
import ctypes

import numpy as np
import pytest

import attn_inputs as gen
from gpu_helpers import announce, lens_gpu, to_gpu

pytestmark = pytest.mark.gpu


def _grads(L, attn, torch, inp, g_st, noalloc):
    B, H, n_q, n_kv, _, _ = inp.shape
    q, k, v, do = (to_gpu(a, "bf16") for a in (inp.q_st, inp.k_st, inp.v_st, g_st))
    lq, lk = lens_gpu(inp.seqlens_q), lens_gpu(inp.seqlens_kv)
    o, lse = attn.sdpa(q, k, v, scale=inp.scale, causal=inp.causal, seqlens_q=lq, seqlens_kv=lk, return_lse=True)
    # outputs prefilled with NaN: every element must be written
    dq, dk, dv = (torch.full_like(t, float("nan")) for t in (q, k, v))
    stream = torch.cuda.current_stream().cuda_stream
    common = [attn.ATTN_BF16, B, H, n_q, n_kv, 64, 64, q.data_ptr(), None, k.data_ptr(), None, v.data_ptr(), None,
              o.data_ptr(), None, do.data_ptr(), None, lse.data_ptr(), dq.data_ptr(), None, dk.data_ptr(), None,
              dv.data_ptr(), None, float(inp.scale), attn.ATTN_MASK_CAUSAL if inp.causal else attn.ATTN_MASK_NONE,
              None if lq is None else lq.data_ptr(), None if lk is None else lk.data_ptr()]
    if noalloc:
        rc = L.attn_sdpa_bwd_noalloc(*common, stream)
        assert rc == 0, attn.status_str(rc)
    else:
        nbytes = L.attn_sdpa_bwd_workspace_bytes(attn.ATTN_BF16, B, H, n_q, n_kv, 64, 64)
        ws = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device=q.device)
        rc = L.attn_sdpa_bwd(*common, ws.data_ptr(), nbytes, stream)
        assert rc == 0, attn.status_str(rc)
    torch.cuda.synchronize()
    return [t.cpu() for t in (dq, dk, dv)]


def test_noalloc_backward_equals_workspace_backward_twice():
    import torch
    import head_attention_sdpa_amd as attn
    L = attn.lib()
    cases = [  # the second call is smaller than the first
        gen.make_sdpa("noalloc_big", "bf16", 2, 4, 333, 333, 64, 64, 0.125, True,
                      seqlens_q=np.array([333, 200], np.int32), seqlens_kv=np.array([333, 150], np.int32),
                      cfg_id=61),
        gen.make_sdpa("noalloc_small", "bf16", 1, 2, 100, 130, 64, 64, 0.125, False, cfg_id=62),
    ]
    for inp in cases:
        announce(f"noalloc backward {inp.name} shape={inp.shape}")
        g, g_st = gen.make_dout(inp, 63)
        ref = _grads(L, attn, torch, inp, g_st, noalloc=False)
        got = _grads(L, attn, torch, inp, g_st, noalloc=True)
        for name, a, b in zip(("dq", "dk", "dv"), ref, got):
            assert not torch.isnan(b).any(), f"{inp.name}: {name} has unwritten elements"
            assert torch.equal(a, b), f"{inp.name}: {name} differs from the workspace entry point"
        print(f"  {inp.name}: dq, dk, dv bitwise equal to attn_sdpa_bwd", flush=True)
