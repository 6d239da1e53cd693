"""GPU parity for packed variable-length prefill (fa_prefill_varlen).

Covers chunked prefill against a longer key prefix (bottom-right causal
alignment), sequences of mixed lengths, rows with no visible key, and left
windows.  Each case is compared element by element with the fp64 oracle
(attention_varlen) on the same seeded inputs.  Tolerances are bf16 max-abs
2e-2 and mean-abs 2e-3 on O, and 1e-3 on lse; rows without keys must give
exactly 0 and -inf.  On a single full-length sequence the result must be
bit-identical to dense fa_prefill.
"""

import numpy as np
import pytest
import torch

import oracle
from exact_tiled_attention_prefill_amd import prefill, prefill_varlen
from exact_tiled_attention_prefill_amd import inputs as I
from gpu_util import BF16_LSE_MAX_ABS, check_bf16, f64, to_dev

pytestmark = pytest.mark.gpu

# (n_q, n_k) per sequence: one row, ragged tiles, chunks against longer
# prefixes, more queries than keys, and sequences without queries or keys
MIXED = [(1, 1), (130, 130), (7, 300), (200, 1000), (0, 5), (64, 64), (129, 140), (50, 20), (5, 0), (3, 70)]


def run_varlen(q, k, v, cu_q, cu_k, causal, window, scale):
    qd, kd, vd, cqd, ckd = to_dev(q, k, v, cu_q, cu_k)
    max_q = int((cu_q[1:] - cu_q[:-1]).max())
    o, lse = prefill_varlen(qd, kd, vd, cqd, ckd, max_q, causal=causal, window_left=window, scale=scale)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def check_lse(lse_gpu, lse_ref, what):
    g = f64(lse_gpu)
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(g), empty), f"{what}: rows without keys differ"
    err = np.abs(g[~empty] - lse_ref[~empty]).max() if (~empty).any() else 0.0
    assert err <= BF16_LSE_MAX_ABS, f"{what}: lse max-abs {err:.3e}"


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("window", [-1, 0, 1, 63, 64, 200])
def test_varlen_mixed_lengths_match_oracle(d, causal, window):
    G = 4
    print(f"varlen d={d} causal={causal} window={window}", flush=True)
    q, k, v, cu_q, cu_k, scale = I.varlen_inputs(MIXED, 2 * G, 2, d, seed=d + window + 7 * causal)
    o, lse = run_varlen(q, k, v, cu_q, cu_k, causal, window, scale)
    ro, rl = oracle.attention_varlen(q, k, v, cu_q, cu_k, causal, scale, window_left=window)
    check_bf16(o, ro, "varlen o")
    check_lse(lse, rl, "varlen lse")
    empty = np.isneginf(rl)
    if empty.any():  # rows without keys: exactly zero output
        rows = np.where(empty.any(axis=0))[0]
        assert torch.all(o[rows] == 0)


@pytest.mark.parametrize("G", [1, 3, 8])
def test_varlen_gqa_groups(G):
    lens = [(300, 300), (100, 513)]
    q, k, v, cu_q, cu_k, scale = I.varlen_inputs(lens, G, 1, 128, seed=G)
    o, lse = run_varlen(q, k, v, cu_q, cu_k, True, -1, scale)
    ro, rl = oracle.attention_varlen(q, k, v, cu_q, cu_k, True, scale)
    check_bf16(o, ro, "varlen GQA o")
    check_lse(lse, rl, "varlen GQA lse")


@pytest.mark.parametrize("causal", [True, False])
def test_varlen_single_sequence_equals_dense_prefill(causal):
    """One sequence with n_q = n_k, no window: the same tiles in the same
    order as fa_prefill, so the outputs are bit-identical."""
    n, hq, hkv, d = 700, 8, 2, 128
    q, k, v, scale = I.prefill_inputs(1, hq, hkv, n, d, "bf16", seed=31)
    od, ld = prefill(*to_dev(q, k, v), causal=causal, scale=scale)
    qp, kp, vp = (x[0].transpose(0, 1).contiguous() for x in (q, k, v))  # [n, H, d]
    cu = torch.tensor([0, n], dtype=torch.int32)
    o, lse = run_varlen(qp, kp, vp, cu, cu, causal, -1, scale)
    torch.cuda.synchronize()
    assert torch.equal(o, od.cpu()[0].transpose(0, 1))
    assert torch.equal(lse, ld.cpu()[0])


def test_varlen_chunked_prefill_matches_full_causal_rows():
    """A 1000-query chunk against its 3000-key prefix (GQA, d 128) equals the
    last 1000 rows of causal attention over the whole sequence (oracle on
    sampled rows)."""
    n, nq, hq, hkv, d = 3000, 1000, 8, 2, 128
    q, k, v, cu_q, cu_k, scale = I.varlen_inputs([(nq, n)], hq, hkv, d, seed=41)
    o, lse = run_varlen(q, k, v, cu_q, cu_k, True, -1, scale)
    rows = [0, 1, 63, 64, 127, 128, 500, 998, 999]
    ro, rl = oracle.attention_varlen(q, k, v, cu_q, cu_k, True, scale, rows=rows)
    check_bf16(o[rows], ro[rows], "chunked prefill o")
    check_lse(lse[:, rows], rl[:, rows], "chunked prefill lse")


def test_varlen_out_of_range_offsets_are_clamped():
    """cu_seqlens values outside [0, total] are clamped on the device: the
    call stays in bounds and equals the oracle on the clamped offsets."""
    lens = [(40, 40), (30, 50)]
    q, k, v, cu_q, cu_k, scale = I.varlen_inputs(lens, 2, 1, 64, seed=3)
    bad_q = torch.tensor([0, 40, 500], dtype=torch.int32)   # end past total_q = 70
    bad_k = torch.tensor([-9, 40, 90], dtype=torch.int32)   # start before 0
    qd, kd, vd, cqd, ckd = to_dev(q, k, v, bad_q, bad_k)
    o, lse = prefill_varlen(qd, kd, vd, cqd, ckd, 40, causal=True, scale=scale)
    torch.cuda.synchronize()
    cq = torch.tensor([0, 40, 70], dtype=torch.int32)
    ck = torch.tensor([0, 40, 90], dtype=torch.int32)
    ro, rl = oracle.attention_varlen(q, k, v, cq, ck, True, scale)
    check_bf16(o.cpu()[:70], ro, "clamped offsets o")
