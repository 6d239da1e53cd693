"""GPU parity for the attention backward (fa_prefill_backward, bf16).

Inputs are seeded bf16 draws; the forward runs on the GPU (its o and lse feed
the backward, as in training) and the fp64 oracle computes the gradients
from the same q, k, v, dout.  Tolerance: the kernel rounds p and ds to bf16
before the matrix products that consume them, and each gradient to bf16 on
output (relative 2^-9 each); for gradient entries of magnitude up to
s = max(1, max|ref|) the bar is max-abs <= 2e-2 * s and mean-abs
<= 2e-3 * s, the bf16 bar of the forward scaled to the gradient's range.
"""

import numpy as np
import pytest
import torch

import oracle
from exact_tiled_attention_prefill_amd import prefill, prefill_backward, prefill_backward_workspace_bytes
from exact_tiled_attention_prefill_amd import inputs as I
from gpu_util import f64, to_dev

pytestmark = pytest.mark.gpu


def check_grad(g_gpu, ref, what):
    err = np.abs(f64(g_gpu) - ref)
    assert np.isfinite(err).all(), f"{what}: non-finite"
    s = max(1.0, float(np.abs(ref).max()))
    mx, mean = err.max(), err.mean()
    assert mx <= 2e-2 * s, f"{what}: max-abs {mx:.3e} > {2e-2 * s:.3e}"
    assert mean <= 2e-3 * s, f"{what}: mean-abs {mean:.3e} > {2e-3 * s:.3e}"


def run_backward(q, k, v, do, causal, scale, workspace=False):
    qd, kd, vd, dod = to_dev(q, k, v, do)
    o, lse = prefill(qd, kd, vd, causal=causal, scale=scale)
    ws = None
    if workspace:
        B, Hq, N, _ = q.shape
        ws = torch.empty(prefill_backward_workspace_bytes(B, Hq, N), dtype=torch.uint8, device="cuda")
    dq, dk, dv = prefill_backward(qd, kd, vd, o, dod, lse, causal=causal, scale=scale, workspace=ws)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("N", [1, 17, 64, 130, 300])
def test_backward_matches_oracle(d, causal, N):
    print(f"backward d={d} causal={causal} N={N}", flush=True)
    q, k, v, do, scale = I.backward_inputs(2, 4, 2, N, d, seed=N + d + causal)
    dq, dk, dv = run_backward(q, k, v, do, causal, scale)
    rq, rk, rv = oracle.attention_backward(q, k, v, do, causal, scale)
    check_grad(dq, rq, "dq")
    check_grad(dk, rk, "dk")
    check_grad(dv, rv, "dv")


@pytest.mark.parametrize("G", [1, 3, 8])
@pytest.mark.parametrize("scale", [-0.2, 0.0])
def test_backward_gqa_and_scale(G, scale):
    scale = float(np.float32(scale))  # the fp32 value the kernel receives, which the oracle widens
    q, k, v, do, _ = I.backward_inputs(1, G, 1, 200, 128, seed=G)
    dq, dk, dv = run_backward(q, k, v, do, True, scale, workspace=True)
    rq, rk, rv = oracle.attention_backward(q, k, v, do, True, scale)
    check_grad(dq, rq, "dq")
    check_grad(dk, rk, "dk")
    check_grad(dv, rv, "dv")


@pytest.mark.parametrize("causal", [True, False])
def test_backward_gqa_long(causal):
    """Four query heads per key/value head over 1000 rows: the dK/dV kernel's
    loop over the group's heads crosses many unmasked interior tiles of each
    head, the causal diagonal and the ragged end."""
    print(f"backward gqa long causal={causal}", flush=True)
    q, k, v, do, scale = I.backward_inputs(1, 8, 2, 1000, 128, seed=40 + causal)
    dq, dk, dv = run_backward(q, k, v, do, causal, scale, workspace=True)
    rq, rk, rv = oracle.attention_backward(q, k, v, do, causal, scale)
    check_grad(dq, rq, "dq")
    check_grad(dk, rk, "dk")
    check_grad(dv, rv, "dv")


def test_backward_deterministic():
    q, k, v, do, scale = I.backward_inputs(1, 4, 2, 257, 128, seed=3)
    a = run_backward(q, k, v, do, True, scale)
    b = run_backward(q, k, v, do, True, scale)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_backward_mha_4k_sampled_heads():
    """The B4 H32 N4096 d128 causal workload: gradients of heads (0, 0) and
    (3, 31) against the oracle on those heads (each head's gradients depend
    only on its own q, k, v, do under MHA)."""
    cfg = I.PREFILL_MHA_4K
    q, k, v, do, scale = I.backward_inputs(cfg.B, cfg.Hq, cfg.Hkv, cfg.N, cfg.d, seed=0)
    dq, dk, dv = run_backward(q, k, v, do, True, scale)
    for b, h in ((0, 0), (3, 31)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        rq, rk, rv = oracle.attention_backward(q[sl], k[sl], v[sl], do[sl], True, scale)
        check_grad(dq[sl], rq, f"dq head {b},{h}")
        check_grad(dk[sl], rk, f"dk head {b},{h}")
        check_grad(dv[sl], rv, f"dv head {b},{h}")
