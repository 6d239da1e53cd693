"""bench.py's own arithmetic: the FLOP and byte counts its roofline figures
divide by, the row and sequence samples its parity checks use, and the
parity checks themselves (with planted errors).

Each count is checked against a quantity computed another way: visible
(query, key) pairs counted pair by pair from the mask predicate (and from
PyTorch's bottom-right causal bias), bytes summed from the tensors the
workload actually moves.
"""

import multiprocessing

import numpy as np
import pytest
import torch

import bench
import oracle
from exact_tiled_attention_prefill_amd import inputs as I


def visible_pairs_bruteforce(nq, nk, causal, window):
    """Pairs (i, j) with j <= i + (nk - nq) under the mask and j >= i + off - W with a window."""
    i = torch.arange(nq)[:, None]
    j = torch.arange(nk)[None, :]
    off = nk - nq
    vis = torch.ones(nq, nk, dtype=torch.bool)
    if causal:
        vis &= j <= i + off
    if window >= 0:
        vis &= j >= i + off - window
    return int(vis.sum())


@pytest.mark.parametrize("N", [1, 2, 7, 64, 130])
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_flops_counts_visible_pairs(N, causal):
    pairs = int(torch.tril(torch.ones(N, N)).sum()) if causal else N * N
    assert bench.prefill_flops(2, 3, N, 128, causal) == 4 * 128 * 2 * 3 * pairs


@pytest.mark.parametrize("lens", [[(5, 9)], [(9, 5)], [(64, 64), (1, 300)], [(0, 10), (10, 0)], [(33, 100), (7, 7)]])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("window", [-1, 0, 3, 40])
def test_varlen_pairs_match_the_pairwise_predicate(lens, causal, window):
    want = sum(visible_pairs_bruteforce(nq, nk, causal, window) for nq, nk in lens)
    assert bench.varlen_pairs(lens, causal, window) == want


@pytest.mark.parametrize("nq,nk", [(5, 9), (16, 16), (1, 40)])
def test_varlen_pairs_match_torch_causal_lower_right(nq, nk):
    from torch.nn.attention.bias import causal_lower_right

    mask = causal_lower_right(nq, nk)._materialize()
    assert bench.varlen_pairs([(nq, nk)], True, -1) == int(mask.sum())


def test_prefill_bytes_are_the_tensors_moved():
    B, Hq, Hkv, N, d = 2, 8, 2, 100, 64
    q = torch.empty(B, Hq, N, d, dtype=torch.bfloat16)
    kv = torch.empty(B, Hkv, N, d, dtype=torch.bfloat16)
    lse = torch.empty(B, Hq, N, dtype=torch.float32)
    moved = 2 * q.nbytes + 2 * kv.nbytes + lse.nbytes  # q, o; k, v; lse
    assert bench.prefill_bytes(B, Hq, Hkv, N, d) == moved


def test_decode_bytes_are_the_rows_read_and_written():
    lens, Hq, Hkv, d = [5, 0, 17, 1], 8, 2, 128
    kc = torch.empty(len(lens), Hkv, max(lens), d, dtype=torch.bfloat16)
    kv_read = sum(2 * kc[b, :, :n].nbytes for b, n in enumerate(lens))
    q = torch.empty(len(lens), Hq, d, dtype=torch.bfloat16)
    seqlens = torch.empty(len(lens), dtype=torch.int32)
    assert bench.decode_bytes(lens, Hq, Hkv, d) == kv_read + 2 * q.nbytes + seqlens.nbytes


def test_c5_sample_rows():
    n = I.PREFILL_GQA_128K.N
    rows = bench.c5_sample_rows(n)
    assert len(rows) == 2048 and rows == sorted(set(rows))
    assert rows[0] == 0 and rows[-1] == n - 1 and all(0 <= r < n for r in rows)
    assert {63, 64, 65, 1023, 1024, 1025, 65535, 65536, 65537}.issubset(rows)


def test_decode_sample_sequences_keep_the_extremes():
    lens = [50, 7, 900, 3, 12, 901, 40, 40]
    seqs = bench.decode_sample_sequences(lens, count=5)
    assert seqs == sorted(set(seqs)) and len(seqs) == 5
    assert {3, 1, 5, 2}.issubset(seqs)  # two shortest (3, 7) and two longest (901, 900)
    assert bench.decode_sample_sequences(lens, count=20) == list(range(len(lens)))


@pytest.fixture(scope="module")
def pool():
    p = multiprocessing.get_context("spawn").Pool(2, initializer=bench._oracle_pool_init)
    yield p
    p.close()
    p.join()


def bf16(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)


def test_prefill_parity_check_passes_rounded_oracle_and_catches_a_planted_error(pool):
    q, k, v, s = I.prefill_inputs(1, 4, 2, 150, 128, "bf16", seed=3)
    ro, rl = oracle.attention(q, k, v, True, s)
    o, lse = bf16(ro), torch.from_numpy(rl.astype(np.float32))
    rows = [0, 1, 63, 64, 149]
    err, flops, _ = bench.oracle_check(pool, q, k, v, s, o, lse, rows, heads_per_job=2)
    assert err["within_bar"] and flops == 4 * 128 * 4 * sum(r + 1 for r in rows)
    bad = o.clone()
    bad[0, 3, 64, 10] += 0.1
    assert not bench.oracle_check(pool, q, k, v, s, bad, lse, rows, heads_per_job=2)[0]["within_bar"]
    bad_lse = lse.clone()
    bad_lse[0, 1, 149] += 2e-3
    assert not bench.oracle_check(pool, q, k, v, s, o, bad_lse, rows, heads_per_job=2)[0]["within_bar"]


@pytest.mark.parametrize("window", [-1, 20])
def test_varlen_parity_check(pool, window):
    q, k, v, cq, ck, s = I.varlen_inputs([(40, 90), (25, 25)], 4, 2, 128, seed=5)
    ro, rl = oracle.attention_varlen(q, k, v, cq, ck, True, s, window_left=window)
    o, lse = bf16(ro), torch.from_numpy(rl.astype(np.float32))
    assert bench.oracle_varlen_check(pool, q, k, v, cq, ck, True, window, s, o, lse)[0]["within_bar"]
    bad = o.clone()
    bad[50, 2, 7] += 0.1
    assert not bench.oracle_varlen_check(pool, q, k, v, cq, ck, True, window, s, bad, lse)[0]["within_bar"]


def test_decode_parity_check(pool):
    q, kc, vc, dl, s = I.decode_inputs(5, 8, 2, 128, 1, 400, 400, "bf16", seed=2)
    ro, _ = oracle.decode(q, kc, vc, dl, s)
    good = bf16(ro)
    bad = good.clone()
    bad[4, 6, 9] += 0.1
    lens = dl.tolist()
    errs, _ = bench.oracle_decode_check(pool, q, kc, vc, lens, s, {"a": good, "b": bad}, list(range(5)))
    assert errs["a"]["within_bar"] and not errs["b"]["within_bar"]


def test_backward_parity_check(pool):
    q, k, v, do, s = I.backward_inputs(1, 2, 2, 70, 64, seed=4)
    refs = [bf16(r) for r in oracle.attention_backward(q, k, v, do, True, s)]
    err, _ = bench.oracle_backward_check(pool, q, k, v, do, s, refs)
    assert err["within_bar"]
    bad = [r.clone() for r in refs]
    bad[2][0, 1, 33, 5] += 0.5
    err, _ = bench.oracle_backward_check(pool, q, k, v, do, s, bad)
    assert not err["within_bar"] and err["dv"]["max_abs_over_range"] > 2e-2


def test_rooflines_state_their_goal():
    rl = bench.mfma_roofline("k", 0.49 * bench.PEAK_BF16_TFLOPS)
    assert rl["goal_frac"] == 0.5 and rl["goal_met"] is False
    assert bench.mfma_roofline("k", 0.5 * bench.PEAK_BF16_TFLOPS)["goal_met"] is True
    none = bench.mfma_roofline("k", 1.0, goal=None)
    assert none["goal_frac"] is None and none["goal_met"] is None
    hbm = bench.with_goal({"frac": 0.83}, bench.GOAL_DECODE_FRAC)
    assert hbm["goal_frac"] == 0.7 and hbm["goal_met"] is True


def test_f32_parity_check(pool):
    q, k, v, s = I.prefill_inputs(1, 1, 1, 256, 64, "f32", seed=0)
    ro, rl = oracle.attention(q, k, v, False, s)
    o, lse = torch.from_numpy(ro.astype(np.float32)), torch.from_numpy(rl.astype(np.float32))
    err, _ = bench.oracle_f32_check(pool, q, k, v, False, s, o, lse)
    assert err["within_bar"] and err["o_max_abs"] < 1e-6
    bad = o.clone()
    bad[0, 0, 200, 3] += 3e-5
    assert not bench.oracle_f32_check(pool, q, k, v, False, s, bad, lse)[0]["within_bar"]
    bad_lse = lse.clone()
    bad_lse[0, 0, 7] -= 3e-5
    assert not bench.oracle_f32_check(pool, q, k, v, False, s, o, bad_lse)[0]["within_bar"]
