"""Calls from several host threads at once, each thread on its own stream
(the library's only host state is per thread or looked up once under a lock):
every thread's results must equal, bit for bit, the same calls made one after
another from one thread."""
import threading

import pytest

from gpu_helpers import announce

pytestmark = pytest.mark.gpu
THREADS, CALLS = 4, 6


def test_concurrent_host_threads_match_sequential_calls():
    import torch
    import head_attention_sdpa_amd as attn
    attn.lib()
    announce("four host threads, one stream each: forward, decoding step and backward")
    gen = torch.Generator().manual_seed(404)

    def rnd(*shape):
        return torch.randn(shape, generator=gen).to(torch.bfloat16).cuda()

    work = []
    for t in range(THREADS):
        q, k, v, do = rnd(2, 4, 300, 64), rnd(2, 4, 300, 64), rnd(2, 4, 300, 64), rnd(2, 4, 300, 64)
        qd, kc, vc = rnd(3, 2, 2, 64), rnd(3, 2, 2000, 64), rnd(3, 2, 2000, 64)
        work.append((q, k, v, do, qd, kc, vc))

    def calls(w):
        q, k, v, do, qd, kc, vc = w
        out = []
        for i in range(CALLS):
            o, lse = attn.sdpa(q, k, v, causal=bool(i & 1), return_lse=True)
            out += [o, lse, attn.decode(qd, kc, vc)]
            out += list(attn.sdpa_bwd(q, k, v, o, lse, do, causal=bool(i & 1)))
        return out

    ref = []
    for w in work:
        ref.append(calls(w))
    torch.cuda.synchronize()

    got = [None] * THREADS
    errors = []

    def worker(t):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                got[t] = calls(work[t])
            s.synchronize()
        except Exception as e:  # reported below, after every thread has ended
            errors.append((t, repr(e)))

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(THREADS)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for t in range(THREADS):
        for i, (a, b) in enumerate(zip(ref[t], got[t])):
            assert torch.equal(a, b), f"thread {t}, result {i} differs from the sequential call"
    print(f"{THREADS} threads x {CALLS} rounds of forward, decode and backward: bitwise equal", flush=True)
