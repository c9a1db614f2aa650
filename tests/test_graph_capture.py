"""The entry points under HIP graph capture: none of them allocates, frees, synchronises or
clears memory with a memset, so a caller can capture prefill, backward and decode (with
preallocated outputs and workspaces) into one graph and replay it. The graph is replayed
several times with the program's own eager work (and a NaN fill of every output) between
replays; every replay must reproduce the eager results bit for bit.
"""
import pytest
import torch

import exact_tiled_attention_08_amd as fa
from parity_util import say, seeded

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.library()


def test_graph_replays_match_eager():
    B, H, N, d = 2, 4, 700, 128
    q = seeded((B, H, N, d), 9201, torch.bfloat16, mult=2.0)
    k = seeded((B, H, N, d), 9202, torch.bfloat16, mult=2.0)
    v = seeded((B, H, N, d), 9203, torch.bfloat16)
    do = seeded((B, H, N, d), 9204, torch.bfloat16)
    qd = seeded((B, H, 1, d), 9205, torch.bfloat16)
    bias = fa.pad_bias(seeded((B, H, N, N), 9206, torch.bfloat16))

    say("graph capture: eager reference")
    ref = []
    o, lse = fa.fwd(q, k, v, causal=1)
    ref += [o, lse, *fa.bwd(q, k, v, o, lse, do, causal=1)]
    ref += list(fa.decode(qd, k, v, num_splits=16))
    ref += list(fa.decode_noalloc(qd, k, v, num_splits=16))
    ob, lb = fa.fwd_bias(q, k, v, bias, causal=1)
    ref += [ob, lb]
    torch.cuda.synchronize()

    # static outputs and workspaces, used once eagerly before capture
    outs = [torch.empty_like(t) for t in ref]
    ws_b = torch.empty(fa.bwd_workspace_bytes(B, H, N), dtype=torch.uint8, device=DEV)
    ws_d = torch.empty(fa.decode_workspace_bytes(B, H, d, 16), dtype=torch.uint8, device=DEV)

    def work():
        fa.fwd(q, k, v, causal=1, out=outs[0], lse=outs[1])
        fa.bwd(q, k, v, outs[0], outs[1], do, causal=1, dq=outs[2], dk=outs[3], dv=outs[4],
               workspace=ws_b)
        fa.decode(qd, k, v, num_splits=16, out=outs[5], lse=outs[6], workspace=ws_d)
        fa.decode_noalloc(qd, k, v, num_splits=16, out=outs[7], lse=outs[8])
        fa.fwd_bias(q, k, v, bias, causal=1, out=outs[9], lse=outs[10])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        work()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(outs, ref))

    say("graph capture: capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    torch.cuda.synchronize()

    x = torch.randn((1024, 1024), device=DEV)
    for r in range(4):
        say(f"graph capture: replay {r}")
        for t in outs:
            t.fill_(float("nan"))
        x = torch.tanh(x @ x.T * 1e-3)  # the program's own eager work between replays
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outs, ref)):
            assert torch.equal(a, b), f"replay {r}: output {i} differs from the eager result"
