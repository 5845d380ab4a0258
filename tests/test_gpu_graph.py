"""Every entry point captured into a HIP graph (torch.cuda.CUDAGraph) and
replayed: each replay, with new inputs written eagerly between replays and the
outputs poisoned with NaN before it, must give the same bits as an eager call
on the same inputs.  This is the launch path the benchmarks time, so it is
checked against the eager path, which the parity tests check against the
oracle.  The library enqueues kernels only (no memsets or copies), reads the
lengths arrays from device memory at run time, and its workspaces are the
caller's: nothing may depend on state from the capture."""
import zlib

import pytest

from gpu_helpers import announce

pytestmark = pytest.mark.gpu
REPLAYS = 3


def attn_mod():
    import head_attention_sdpa_amd as attn
    attn.lib()
    return attn


def randn(gen, shape, dtype):
    import torch
    return torch.randn(shape, generator=gen, dtype=torch.float32).to(dtype).cuda()


def check_graph(run, sets, static, outs, what):
    """run() enqueues the op on the current stream, reading `static` and
    writing `outs`; sets[i] holds the i-th replay's values of `static`."""
    import torch
    announce(f"graph replay: {what}")
    for t, v in zip(static, sets[0]):
        t.copy_(v)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for rep in range(REPLAYS):
        for t, v in zip(static, sets[rep % len(sets)]):
            t.copy_(v)
        for o in outs:
            o.fill_(float("nan")) if o.is_floating_point() else o.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in outs]
        for o in outs:
            o.fill_(float("nan")) if o.is_floating_point() else o.fill_(-1)
        run()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(got, outs)):
            ai = a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32)
            bi = b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32)
            assert torch.equal(ai, bi), f"{what}: replay {rep}, output {i} differs from the eager call"
            assert not torch.isnan(b.float()).any(), f"{what}: replay {rep}, output {i} left unwritten"
    print(f"{what}: {REPLAYS} replays bitwise equal to eager", flush=True)


def lengths(gen, batch, n):
    import torch
    return torch.randint(0, n + 1, (batch,), generator=gen, dtype=torch.int32).cuda()


@pytest.mark.parametrize("name,B,H,n_q,n_kv,causal,window,dt", [
    ("resident_causal_lengths", 8, 4, 200, 200, True, None, "bf16"),
    ("streaming_causal", 2, 4, 1000, 1000, True, None, "bf16"),
    ("streaming_cross_lengths", 2, 3, 300, 777, False, None, "bf16"),
    ("restricted_r100", 2, 2, 1500, 1500, False, 100, "bf16"),
    ("fp32_d64", 2, 2, 100, 130, True, None, "f32"),
])
def test_sdpa_graph_replay(name, B, H, n_q, n_kv, causal, window, dt):
    import torch
    attn = attn_mod()
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    gen = torch.Generator().manual_seed(zlib.crc32(name.encode()))
    sets = []
    for _ in range(REPLAYS):
        s = [randn(gen, (B, H, n, 64), dtype) for n in (n_q, n_kv, n_kv)]
        s += [lengths(gen, B, n_q), lengths(gen, B, n_kv)]
        sets.append(s)
    static = [torch.empty_like(t) for t in sets[0]]
    q, k, v, lq, lk = static
    o = torch.empty((B, H, n_q, 64), dtype=dtype, device="cuda")
    lse = torch.empty((B, H, n_q), dtype=torch.float32, device="cuda")

    def run():
        # lse through the C ABI's output argument: the binding allocates it
        # itself, so the graph case passes a preallocated one by hand
        import ctypes
        lib = attn.lib()
        sq, sk, sv, so = (attn._strides4(t) for t in (q, k, v, o))
        args = (attn._dtype_code(q), B, H, n_q, n_kv, 64, 64, q.data_ptr(), ctypes.byref(sq),
                k.data_ptr(), ctypes.byref(sk), v.data_ptr(), ctypes.byref(sv), o.data_ptr(),
                ctypes.byref(so), 0.0, attn.ATTN_MASK_CAUSAL if causal else attn.ATTN_MASK_NONE)
        tail = (lq.data_ptr(), lk.data_ptr(), lse.data_ptr(), torch.cuda.current_stream().cuda_stream)
        if window is None:
            rc = lib.attn_sdpa_fwd(*args, *tail)
        else:
            rc = lib.attn_sdpa_window_fwd(*args, window, *tail)
        assert rc == 0, attn.status_str(rc)

    check_graph(run, sets, static, [o, lse], name)


def test_decode_graph_replay_split_path():
    """Four (b, h) over a 4097-key cache: the library splits each (b, h) into
    more than four chunks, so the partial kernel writes the caller's workspace
    and the merge kernel reads it, both inside the graph."""
    import torch
    attn = attn_mod()
    B, H, n_q, n_kv = 2, 2, 3, 4097
    gen = torch.Generator().manual_seed(31)
    sets = []
    for _ in range(REPLAYS):
        sets.append([randn(gen, (B, H, n_q, 64), torch.bfloat16), randn(gen, (B, H, n_kv, 64), torch.bfloat16),
                     randn(gen, (B, H, n_kv, 64), torch.bfloat16),
                     torch.randint(n_q, n_kv + 1, (B,), generator=gen, dtype=torch.int32).cuda()])
    static = [torch.empty_like(t) for t in sets[0]]
    q, k, v, lk = static
    o = torch.empty((B, H, n_q, 64), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(max(attn.decode_workspace_bytes(B, H, n_q, n_kv), 256), dtype=torch.uint8, device="cuda")
    check_graph(lambda: attn.decode(q, k, v, seqlens_kv=lk, out=o, workspace=ws), sets, static, [o],
                "decode, split over the cache")


@pytest.mark.parametrize("noalloc", [False, True])
def test_backward_graph_replay(noalloc):
    import torch
    attn = attn_mod()
    B, H, n = 2, 3, 700
    gen = torch.Generator().manual_seed(57 + int(noalloc))
    sets = []
    for _ in range(REPLAYS):
        q, k, v, do = (randn(gen, (B, H, n, 64), torch.bfloat16) for _ in range(4))
        lq = lengths(gen, B, n)
        o, lse = attn.sdpa(q, k, v, causal=True, seqlens_q=lq, seqlens_kv=lq, return_lse=True)
        sets.append([q, k, v, o, lse, do, lq])
    torch.cuda.synchronize()
    static = [torch.empty_like(t) for t in sets[0]]
    q, k, v, o, lse, do, lq = static
    dq, dk, dv = (torch.empty((B, H, n, 64), dtype=torch.bfloat16, device="cuda") for _ in range(3))
    ws = torch.empty(max(attn.sdpa_bwd_workspace_bytes(B, H, n, n), 256), dtype=torch.uint8, device="cuda")

    def run():
        attn.sdpa_bwd(q, k, v, o, lse, do, causal=True, seqlens_q=lq, seqlens_kv=lq, dq=dq, dk=dk, dv=dv,
                      workspace=None if noalloc else ws, noalloc=noalloc)

    check_graph(run, sets, static, [dq, dk, dv], "backward" + (", no-allocation entry" if noalloc else ""))


def test_sublayer_and_linear_graph_replay():
    import torch
    attn = attn_mod()
    B, n, dm, h = 2, 300, 256, 4
    gen = torch.Generator().manual_seed(71)

    def sets_of(shapes):
        return [[randn(gen, s, torch.bfloat16) * 0.1 for s in shapes] for _ in range(REPLAYS)]

    shapes = [(B, n, dm), (dm, dm), (dm, dm), (dm, dm), (dm, dm), (dm,), (dm,)]
    sets = sets_of(shapes)
    for s in sets:
        s.append(lengths(gen, B, n))
    static = [torch.empty_like(t) for t in sets[0]]
    x, wq, wk, wv, wo, gam, bet, lq = static
    y = torch.empty((B, n, dm), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(attn.mha_block_workspace_bytes(B, n, n, dm, h, True), dtype=torch.uint8, device="cuda")
    check_graph(lambda: attn.mha_block(x, wq, wk, wv, wo, gam, bet, h, add_pe=True, causal=True, seqlens_q=lq,
                                       seqlens_kv=lq, out=y, workspace=ws),
                sets, static, [y], "attention sublayer (PE, MultiHead, residual, LayerNorm)")

    lsets = sets_of([(333, 256), (256, 200)])
    lstatic = [torch.empty_like(t) for t in lsets[0]]
    lx, lw = lstatic
    ly = torch.empty((333, 200), dtype=torch.bfloat16, device="cuda")
    check_graph(lambda: attn.linear(lx, lw, out=ly), lsets, lstatic, [ly], "projection GEMM")
