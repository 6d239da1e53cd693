"""GPU parity for the 8-wave prefill launch (256 query rows per workgroup).

The launcher uses it when the average query row sees 4096 keys or more
(d = 128).  These cases are chosen to take it, with ragged query and key ends
(lengths that are not multiples of the 256-row or 64-key tiles), and are
checked on sampled rows against the fp64 oracle to the bf16 bar.
"""

import numpy as np
import pytest
import torch

import oracle
from exact_tiled_attention_prefill_amd import prefill, prefill_varlen
from exact_tiled_attention_prefill_amd import inputs as I
from gpu_util import BF16_LSE_MAX_ABS, check_bf16, check_close, f64, to_dev

pytestmark = pytest.mark.gpu


def _dense(B, Hq, Hkv, N, causal, seed, rows):
    print(f"wide dense B{B} Hq{Hq} Hkv{Hkv} N{N} causal={causal}", flush=True)
    q, k, v, scale = I.prefill_inputs(B, Hq, Hkv, N, 128, "bf16", seed=seed)
    qd, kd, vd = to_dev(q, k, v)
    o, lse = prefill(qd, kd, vd, causal=causal, scale=scale)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    heads = [(b, h) for b in range(B) for h in range(Hq)]
    ro, rl = oracle.attention_rows(q, k, v, causal, scale, rows, heads)
    check_bf16(torch.stack([o[b, h, rows] for b, h in heads]), ro, "wide dense o")
    check_close(torch.stack([lse[b, h, rows] for b, h in heads]), rl, BF16_LSE_MAX_ABS, "wide dense lse")


def test_wide_dense_noncausal_ragged():
    """N = 8269 (every row sees 8269 keys): the last query tile holds 77 rows
    and the last key tile 13 keys."""
    N = 8269
    _dense(1, 4, 2, N, False, 61, [0, 1, 255, 256, 4000, 8191, 8192, 8255, 8256, N - 1])


def test_wide_dense_causal_gqa_ragged():
    """Causal GQA (4 query heads per key/value head), N = 16461: rows see
    8231 keys on average; the paired query tiles include the ragged last one."""
    N = 16461
    _dense(1, 4, 1, N, True, 62, [0, 1, 255, 256, 511, 8000, 8230, 16383, 16384, N - 2, N - 1])


def test_wide_dense_causal_mha_near_threshold():
    """Causal MHA, N = 8300: rows see 4150.5 keys on average, just above the
    width threshold; ragged last query and key tiles."""
    N = 8300
    _dense(1, 2, 2, N, True, 65, [0, 1, 63, 64, 255, 256, 4095, 4096, 8191, 8192, N - 1])


@pytest.mark.parametrize("causal", [True, False])
def test_wide_varlen_long_prefixes(causal):
    """Packed chunks against long cached prefixes (9278 keys per row on
    average under the bottom-right causal mask): ragged chunk lengths, a
    single-row chunk, GQA."""
    print(f"wide varlen causal={causal}", flush=True)
    lens = [(300, 9000), (1000, 12000), (1, 8500), (77, 8300)]
    q, k, v, cu_q, cu_k, scale = I.varlen_inputs(lens, 8, 2, 128, seed=63 + causal)
    qd, kd, vd, cqd, ckd = to_dev(q, k, v, cu_q, cu_k)
    o, lse = prefill_varlen(qd, kd, vd, cqd, ckd, 1000, causal=causal, scale=scale)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    starts = cu_q[:-1].tolist()
    rows = sorted({r for s, (nq, _) in zip(starts, lens) for r in (s, s + nq // 2, s + nq - 1)} | {255, 256, 1299})
    ro, rl = oracle.attention_varlen(q, k, v, cu_q, cu_k, causal, scale, rows=rows)
    check_bf16(o[rows], ro[rows], "wide varlen o")
    err = np.abs(f64(lse[:, rows]) - rl[:, rows]).max()
    assert err <= BF16_LSE_MAX_ABS, f"wide varlen lse max-abs {err:.3e}"


@pytest.mark.parametrize("causal,window", [(True, -1), (True, 4500), (False, -1), (False, 4500)])
def test_wide_varlen_short_sequences_and_window(causal, window):
    """Eight-wave launch (the batch's rows see >= 4096 keys on average) over
    sequences from 1 to 200 keys beside long ones: key-tile counts 1 to 4
    take every remaining-tile path of the four-slot ring; with a 4500-key
    window the long rows start past key 0."""
    print(f"wide varlen short+long causal={causal} window={window}", flush=True)
    lens = [(1, 1), (2, 2), (63, 63), (64, 64), (65, 65), (130, 130), (200, 200), (1, 150),
            (500, 20000), (300, 18000), (257, 16000)]
    q, k, v, cu_q, cu_k, scale = I.varlen_inputs(lens, 4, 2, 128, seed=66 + causal + 2 * (window >= 0))
    qd, kd, vd, cqd, ckd = to_dev(q, k, v, cu_q, cu_k)
    o, lse = prefill_varlen(qd, kd, vd, cqd, ckd, 500, causal=causal, scale=scale, window_left=window)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    starts = cu_q[:-1].tolist()
    rows = sorted({r for s, (nq, _) in zip(starts, lens) for r in (s, s + nq // 2, s + nq - 1)} |
                  set(range(starts[8], starts[8] + 16)))
    ro, rl = oracle.attention_varlen(q, k, v, cu_q, cu_k, causal, scale, window_left=window, rows=rows)
    check_bf16(o[rows], ro[rows], "wide varlen short+long o")
    err = np.abs(f64(lse[:, rows]) - rl[:, rows]).max()
    assert err <= BF16_LSE_MAX_ABS, f"wide varlen short+long lse max-abs {err:.3e}"


@pytest.mark.parametrize("causal,n", [(True, 16500), (False, 8300)])
def test_wide_varlen_single_sequence_equals_dense(causal, n):
    """One full-length sequence long enough for the 8-wave launch: packed and
    dense prefill pick the same width and give bit-identical results."""
    print(f"wide single sequence causal={causal} n={n}", flush=True)
    hq, hkv, d = 4, 2, 128
    q, k, v, scale = I.prefill_inputs(1, hq, hkv, n, d, "bf16", seed=64 + causal)
    od, ld = prefill(*to_dev(q, k, v), causal=causal, scale=scale)
    qp, kp, vp = (x[0].transpose(0, 1).contiguous() for x in (q, k, v))  # [n, H, d]
    cu = torch.tensor([0, n], dtype=torch.int32)
    o, lse = prefill_varlen(*to_dev(qp, kp, vp, cu, cu), n, causal=causal, scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(o.cpu(), od.cpu()[0].transpose(0, 1))
    assert torch.equal(lse.cpu(), ld.cpu()[0])


def test_wide_varlen_128k_sequence_equals_dense():
    """The 131072-token causal GQA workload (Hq64 Hkv8 d128) as one packed
    sequence: its packed Q/O rows span 2 GiB, so row offsets pass 2^31 bytes.
    Packed and dense prefill must agree bit for bit."""
    print("wide varlen 128K single sequence", flush=True)
    cfg = I.PREFILL_GQA_128K
    q, k, v, scale = I.prefill_config_inputs(cfg)
    qd, kd, vd = to_dev(q, k, v)
    del q, k, v
    od, ld = prefill(qd, kd, vd, causal=True, scale=scale)
    qp, kp, vp = (x[0].transpose(0, 1).contiguous() for x in (qd, kd, vd))  # [n, H, d] on the device
    del qd, kd, vd
    cu = torch.tensor([0, cfg.N], dtype=torch.int32, device="cuda")
    o, lse = prefill_varlen(qp, kp, vp, cu, cu, cfg.N, causal=True, scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(o, od[0].transpose(0, 1))
    assert torch.equal(lse, ld[0])
