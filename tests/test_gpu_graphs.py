"""The library's calls captured in a HIP graph (torch.cuda.CUDAGraph): the
calls only launch kernels on the caller's stream (no allocation, no memset,
no synchronisation), so a captured forward + backward, or decode, replays to
the eager result.  Each replay runs after other eager work and a host
synchronisation, with the inputs refilled in place, and is compared with an
eager call on the same inputs (bit-exact: the kernels are deterministic)."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

fa = pytest.importorskip("io_aware_exact_tiled_amd")


def _rand(shape, dtype, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    return torch.randn(*shape, generator=g).to(dtype).cuda()


@pytest.mark.parametrize("d,dtype", [(64, torch.bfloat16), (128, torch.bfloat16), (64, torch.float16)])
def test_forward_backward_graph_replays(d, dtype):
    print(f"[case] graph fwd+bwd d={d} {dtype}", flush=True)
    B, H, N = 2, 4, 300
    kw = dict(causal=True, dropout_p=0.1, seed=7, key_lens=torch.tensor([300, 211], dtype=torch.int32).cuda())
    q, k, v, do = (_rand((B, H, N, d), dtype, s) for s in range(4))
    o = torch.empty_like(q)
    lse = torch.empty(B, H, N, dtype=torch.float32, device="cuda")
    grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    fws = torch.empty(max(1, fa.fwd_workspace_bytes(B, H, N, d, dtype)), dtype=torch.uint8, device="cuda")
    bws = torch.empty(fa.bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device="cuda")

    def call():
        fa.fwd(q, k, v, out=o, lse=lse, workspace=fws, **kw)
        fa.bwd(q, k, v, o, do, lse, grads=grads, workspace=bws, **kw)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()                                         # warm-up off the default stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for r in range(3):
        for t, seed in zip((q, k, v, do), range(10 * r + 10, 10 * r + 14)):
            t.copy_(_rand(t.shape, dtype, seed))
        fa.fwd(_rand((1, 2, 64, d), dtype, 99), _rand((1, 2, 64, d), dtype, 98), _rand((1, 2, 64, d), dtype, 97))
        torch.cuda.synchronize()                       # other eager work between replays
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (o, lse) + grads]
        call()                                         # eager, same inputs
        torch.cuda.synchronize()
        want = [o, lse, *grads]
        for name, a_, b_ in zip(("O", "LSE", "dQ", "dK", "dV"), got, want):
            assert torch.equal(a_, b_), (r, name)
    print(f"[ok] graph fwd+bwd d={d} {dtype}", flush=True)


def test_decode_graph_replays():
    print("[case] graph decode", flush=True)
    B, H, Hkv, Nq, Nk, d = 4, 8, 2, 1, 3000, 128
    q = _rand((B, H, Nq, d), torch.bfloat16, 1)
    k = _rand((B, Hkv, Nk, d), torch.bfloat16, 2)
    v = _rand((B, Hkv, Nk, d), torch.bfloat16, 3)
    kl = torch.tensor([3000, 1, 1777, 2048], dtype=torch.int32).cuda()
    o = torch.empty_like(q)
    lse = torch.empty(B, H, Nq, dtype=torch.float32, device="cuda")
    ws = torch.empty(fa.decode_workspace_bytes(B, H, Hkv, Nq, Nk, d), dtype=torch.uint8, device="cuda")

    def call():
        fa.decode(q, k, v, kv_lens=kl, causal=True, out=o, lse=lse, workspace=ws)

    call()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for r in range(3):
        q.copy_(_rand(q.shape, torch.bfloat16, 20 + r))
        kl.copy_(torch.tensor([3000 - r, 1 + r, 1777, 2048 - 7 * r], dtype=torch.int32))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (o.clone(), lse.clone())
        call()
        torch.cuda.synchronize()
        assert torch.equal(got[0], o) and torch.equal(got[1], lse), r
    print("[ok] graph decode", flush=True)
