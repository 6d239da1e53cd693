"""HIP-graph capture of prefill, decode (caller workspace) and the backward.

These calls only enqueue kernels on the caller's stream: no allocation, no
memset, no host synchronisation.  A captured graph therefore replays them.
Each replay is compared bit for bit with the eager result (the kernels are
deterministic), with eager work and synchronisations between the replays.
"""

import pytest
import torch

from exact_tiled_attention_prefill_amd import (decode, decode_workspace_bytes, prefill, prefill_backward,
                                               prefill_backward_workspace_bytes)
from exact_tiled_attention_prefill_amd import inputs as I

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    dev = "cuda"
    q, k, v, scale = I.prefill_inputs(2, 8, 2, 300, 128, "bf16", seed=4)
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    o = torch.empty_like(qd)
    lse = torch.empty((2, 8, 300), dtype=torch.float32, device=dev)
    do = I.backward_inputs(2, 8, 2, 300, 128, "bf16", seed=6)[3].to(dev)
    dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
    bws = torch.empty(prefill_backward_workspace_bytes(2, 8, 300), dtype=torch.uint8, device=dev)
    zq, kc, vc, ls, dscale = I.decode_inputs(4, 8, 2, 128, 1, 1500, 1500, "bf16", seed=5)
    zqd, kcd, vcd, lsd = (t.to(dev) for t in (zq, kc, vc, ls))
    od = torch.empty_like(zqd)
    ws = torch.empty(decode_workspace_bytes(4, 8, 2, 1500, 128), dtype=torch.uint8, device=dev)

    def step():
        prefill(qd, kd, vd, causal=True, scale=scale, out=o, lse=lse)
        prefill_backward(qd, kd, vd, o, do, lse, causal=True, scale=scale, dq=dq, dk=dk, dv=dv, workspace=bws)
        decode(zqd, kcd, vcd, lsd, scale=dscale, out=od, workspace=ws)

    outs = (o, lse, dq, dk, dv, od)
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for t in outs:
            t.fill_(float("nan") if t.is_floating_point() else 0)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, r in zip(outs, ref):
            assert torch.equal(t, r), f"replay {rep} differs from the eager result"
