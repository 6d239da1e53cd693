"""Pins for the fp64 CPU oracle (no GPU).

Each test checks the oracle against something other than itself: a closed
form, an invariant of softmax attention, 50-digit brute force, PyTorch's CPU
float64 scaled_dot_product_attention, or a number printed on the pages.  The
set is chosen so that a dropped scale, a flipped mask, a wrong head map, a
transposed operand, a missing log/max term in lse, a missing rescale in the
running softmax or a wrong merge weight each fail at least one test; the
planted-mistake tests at the bottom show that for a few of them.
"""

import math
import os

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import oracle
from oracle import exact as oatt
from exact_tiled_attention_prefill_amd.inputs import decode_inputs, prefill_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand(shape, seed):
    g = np.random.default_rng(seed)
    return g.standard_normal(shape)


# ---------------------------------------------------------------- P1 / P13
@pytest.mark.parametrize("causal", [False, True])
def test_rows_sum_to_one(causal):
    """P1: with V = 1 every output is 1 (softmax weights sum to one)."""
    q, k = rand((2, 3, 37, 8), 1), rand((2, 3, 37, 8), 2)
    o, _ = oracle.attention(q, k, np.ones_like(k), causal, 0.7)
    assert np.abs(o - 1).max() <= 1e-14


@pytest.mark.parametrize("causal", [False, True])
def test_convex_hull(causal):
    """P13: each output coordinate lies between the min and max of the V rows it sees."""
    q, k, v = rand((1, 2, 29, 5), 3), rand((1, 2, 29, 5), 4), rand((1, 2, 29, 5), 5)
    o, _ = oracle.attention(q, k, v, causal, 1.3)
    for i in range(29):
        vis = v[:, :, : i + 1] if causal else v
        assert np.all(o[:, :, i] >= vis.min(axis=2) - 1e-15)
        assert np.all(o[:, :, i] <= vis.max(axis=2) + 1e-15)


# ---------------------------------------------------------------- P2 / P3
@pytest.mark.parametrize("causal", [False, True])
def test_identical_keys_give_mean(causal):
    """P2: all keys equal -> uniform weights -> mean of the visible V rows."""
    n, d = 23, 6
    q = rand((1, 1, n, d), 6)
    k = np.repeat(rand((1, 1, 1, d), 7), n, axis=2)
    v = rand((1, 1, n, d), 8)
    o, lse = oracle.attention(q, k, v, causal, 0.9)
    for i in range(n):
        vis = v[0, 0, : i + 1] if causal else v[0, 0]
        assert np.abs(o[0, 0, i] - vis.mean(axis=0)).max() <= 1e-14
        s = 0.9 * q[0, 0, i] @ k[0, 0, 0]
        assert abs(lse[0, 0, i] - (s + math.log(len(vis)))) <= 1e-13


def test_dominant_key_selects_its_value():
    """P3: one key whose score exceeds the rest by >= 40 returns its V row."""
    n, d = 16, 4
    q = np.zeros((1, 1, n, d))
    q[..., 0] = 1.0
    k = np.zeros((1, 1, n, d))
    jstar = 11
    k[0, 0, jstar, 0] = 50.0
    v = rand((1, 1, n, d), 9)
    o, lse = oracle.attention(q, k, v, False, 1.0)
    assert np.abs(o[0, 0] - v[0, 0, jstar]).max() <= 1e-14
    assert abs(lse[0, 0, 0] - 50.0) <= 1e-14


# ---------------------------------------------------------------- P4 / P5
def test_causal_row0_is_v0():
    """P4: under the causal mask row 0 sees only key 0: o = V[0], lse = scale q0.k0."""
    q, k, v = rand((2, 2, 9, 7), 10), rand((2, 2, 9, 7), 11), rand((2, 2, 9, 7), 12)
    o, lse = oracle.attention(q, k, v, True, 0.37)
    assert np.array_equal(o[:, :, 0], v[:, :, 0])
    assert np.allclose(lse[:, :, 0], 0.37 * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]),
                       rtol=0, atol=1e-15)


@pytest.mark.parametrize("causal", [False, True])
def test_single_token(causal):
    """P5: N = 1 returns V[0] under either mask."""
    q, k, v = rand((1, 4, 1, 3), 13), rand((1, 2, 1, 3), 14), rand((1, 2, 1, 3), 15)
    o, _ = oracle.attention(q, k, v, causal, 2.0)
    assert np.array_equal(o[0, :2, 0], np.repeat(v[0, 0], 2, axis=0).reshape(2, 3))
    assert np.array_equal(o[0, 2:, 0], np.repeat(v[0, 1], 2, axis=0).reshape(2, 3))


# ---------------------------------------------------------------- P6
def _mp_attention(q, k, v, causal, scale):
    import mpmath as mp

    mp.mp.dps = 50
    n, d = q.shape
    out = []
    lses = []
    for i in range(n):
        js = range(i + 1) if causal else range(n)
        s = [mp.mpf(scale) * mp.fsum(mp.mpf(q[i, c]) * mp.mpf(k[j, c]) for c in range(d)) for j in js]
        e = [mp.e ** x for x in s]
        tot = mp.fsum(e)
        out.append([mp.fsum(e[t] * mp.mpf(v[j, c]) for t, j in enumerate(js)) / tot for c in range(d)])
        lses.append(mp.log(tot))
    return np.array(out, dtype=object), np.array(lses, dtype=object)


@pytest.mark.parametrize("d", [1, 4])
@pytest.mark.parametrize("causal", [False, True])
def test_mpmath_bruteforce_4x4(d, causal):
    """P6: hand-sized cases against a 50-digit evaluation of the definition."""
    g = np.random.default_rng(100 + d + 10 * causal)
    # values exactly representable in bf16 (multiples of 1/8 in [-4, 4])
    q = g.integers(-32, 33, (4, d)) / 8.0
    k = g.integers(-32, 33, (4, d)) / 8.0
    v = g.integers(-32, 33, (4, d)) / 8.0
    scale = 0.5
    o, lse = oracle.attention(q[None, None], k[None, None], v[None, None], causal, scale)
    mo, ml = _mp_attention(q, k, v, causal, scale)
    assert np.abs(o[0, 0] - mo.astype(float)).max() <= 1e-14
    assert np.abs(lse[0, 0] - ml.astype(float)).max() <= 1e-14


# ---------------------------------------------------------------- P7
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("bq,bk", [(1, 1), (3, 5), (64, 64), (16, 7), (70, 70)])
def test_tiled_running_softmax_equals_full(causal, bq, bk):
    """P7: tile-by-tile running softmax == materialised softmax (exactness claim)."""
    q, k, v = rand((2, 4, 70, 16), 20), rand((2, 2, 70, 16), 21), rand((2, 2, 70, 16), 22)
    o, lse = oracle.attention(q, k, v, causal, 0.25)
    ot, lt = oracle.tiled_attention(q, k, v, causal, 0.25, bq, bk)
    assert np.abs(o - ot).max() <= 1e-12
    assert np.abs(lse - lt).max() <= 1e-12


# ---------------------------------------------------------------- P8
@pytest.mark.parametrize("cuts", [[40], [1, 2, 90], [17, 34, 51, 68], [0, 100, 120]])
def test_split_merge_equals_all_keys(cuts):
    """P8: attention over disjoint key chunks merged by lse weights == over all keys."""
    n, d = 128, 8
    q = rand((3, 4, d), 30)
    kc, vc = rand((3, 2, n, d), 31), rand((3, 2, n, d), 32)
    lens = [n, n, n]
    full_o, full_lse = oracle.decode(q, kc, vc, lens, 0.3)
    edges = [0] + cuts + [n]
    parts_o, parts_l = [], []
    for a, b in zip(edges[:-1], edges[1:]):
        sub_k = kc[:, :, a:b]
        sub_v = vc[:, :, a:b]
        o_s, l_s = oracle.decode(q, sub_k, sub_v, [b - a] * 3, 0.3)
        parts_o.append(o_s)
        parts_l.append(l_s)
    mo, ml = oracle.merge_partials(np.stack(parts_o), np.stack(parts_l))
    assert np.abs(mo - full_o).max() <= 1e-12
    assert np.abs(ml - full_lse).max() <= 1e-12


# ---------------------------------------------------------------- P9
def test_decode_equals_last_causal_prefill_row():
    """P9: decode of token i against cache 0..i == causal prefill row i."""
    n, d = 33, 8
    q, k, v = rand((2, 4, n, d), 40), rand((2, 2, n, d), 41), rand((2, 2, n, d), 42)
    o, lse = oracle.attention(q, k, v, True, 0.5)
    for i in (0, 5, 31, 32):
        od, ld = oracle.decode(q[:, :, i], k, v, [i + 1, i + 1], 0.5)
        assert np.abs(od - o[:, :, i]).max() <= 1e-12
        assert np.abs(ld - lse[:, :, i]).max() <= 1e-12


def test_decode_never_reads_past_length():
    """Cache rows at or past seqlens[b] hold NaN; the result stays finite."""
    q, kc, vc, lens, scale = decode_inputs(3, 4, 2, 8, 1, 9, 12, "bf16", seed=3)
    o, lse = oracle.decode(q, kc, vc, lens, scale)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    q2 = q.clone()
    o0, l0 = oracle.decode(q2, kc, vc, [0, 1, 2], scale)
    assert np.all(o0[0] == 0) and np.all(np.isneginf(l0[0]))
    # sequence 1 has one visible entry: every head returns its V row 0
    for h in range(4):
        assert np.array_equal(o0[1, h], vc[1, h // 2, 0].double().numpy())


# ---------------------------------------------------------------- P10
@pytest.mark.parametrize("causal", [False, True])
def test_gqa_equals_mha_with_repeated_heads(causal):
    """P10: GQA with G = Hq/Hkv equals MHA on K/V heads repeated G times consecutively."""
    q, k, v = rand((2, 8, 19, 4), 50), rand((2, 2, 19, 4), 51), rand((2, 2, 19, 4), 52)
    og, lg = oracle.attention(q, k, v, causal, 0.6)
    om, lm = oracle.attention(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1), causal, 0.6)
    assert np.array_equal(og, om) and np.array_equal(lg, lm)


# ---------------------------------------------------------------- P11 / P12
def test_permutation_symmetry_noncausal():
    """P11: jointly permuting K,V rows changes nothing; permuting Q permutes O."""
    q, k, v = rand((1, 2, 31, 6), 60), rand((1, 2, 31, 6), 61), rand((1, 2, 31, 6), 62)
    o, lse = oracle.attention(q, k, v, False, 0.8)
    perm = np.random.default_rng(63).permutation(31)
    o2, l2 = oracle.attention(q, k[:, :, perm], v[:, :, perm], False, 0.8)
    assert np.abs(o - o2).max() <= 1e-13 and np.abs(lse - l2).max() <= 1e-13
    o3, l3 = oracle.attention(q[:, :, perm], k, v, False, 0.8)
    assert np.abs(o[:, :, perm] - o3).max() <= 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_affine_equivariance(causal):
    """P12: O(V A + 1 b^T) = O(V) A + b^T because the weights sum to one."""
    q, k, v = rand((1, 1, 25, 5), 70), rand((1, 1, 25, 5), 71), rand((1, 1, 25, 5), 72)
    a, bvec = rand((5, 5), 73), rand((5,), 74)
    o, _ = oracle.attention(q, k, v, causal, 0.4)
    o2, _ = oracle.attention(q, k, v @ a + bvec, causal, 0.4)
    assert np.abs(o2 - (o @ a + bvec)).max() <= 1e-12


# ---------------------------------------------------------------- P14 / P15
@pytest.mark.parametrize("causal", [False, True])
def test_lse_bounds_and_zero_scale(causal):
    """P14: max s <= lse <= max s + ln|J|; scale 0 -> lse = ln|J|, o = mean."""
    n = 21
    q, k, v = rand((1, 2, n, 4), 80), rand((1, 2, n, 4), 81), rand((1, 2, n, 4), 82)
    o, lse = oracle.attention(q, k, v, causal, 0.9)
    for h in range(2):
        s = oracle.score_matrix(q[0, h], k[0, h], 0.9, causal)
        m = s.max(axis=1)
        cnt = np.arange(1, n + 1) if causal else np.full(n, n)
        assert np.all(lse[0, h] >= m - 1e-14) and np.all(lse[0, h] <= m + np.log(cnt) + 1e-14)
    o0, l0 = oracle.attention(q, k, v, causal, 0.0)
    cnt = np.arange(1, n + 1) if causal else np.full(n, n)
    assert np.abs(l0[0] - np.log(cnt)[None]).max() <= 1e-14
    means = np.cumsum(v[0], axis=1) / cnt[None, :, None] if causal else np.broadcast_to(v[0].mean(axis=1, keepdims=True), v[0].shape)
    assert np.abs(o0[0] - means).max() <= 1e-14


def test_large_scores_are_stable():
    """P15: scores near 1e3 do not overflow; the result matches the rescaled closed form."""
    q = np.zeros((1, 1, 4, 2))
    q[..., 0] = 30.0
    k = np.zeros((1, 1, 4, 2))
    k[0, 0, :, 0] = [40.0, 40.0, 39.0, 0.0]  # scores 1200, 1200, 1170, 0
    v = rand((1, 1, 4, 2), 90)
    o, lse = oracle.attention(q, k, v, False, 1.0)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    w = np.array([1.0, 1.0, math.exp(-30.0), math.exp(-1200.0)])
    ref = (w[:, None] * v[0, 0]).sum(0) / w.sum()
    assert np.abs(o[0, 0] - ref).max() <= 1e-14
    assert abs(lse[0, 0, 0] - (1200.0 + math.log(w.sum()))) <= 1e-12


# ---------------------------------------------------------------- P16
@settings(max_examples=25, deadline=None)
@given(B=st.integers(1, 2), hkv=st.integers(1, 3), G=st.sampled_from([1, 2, 4]),
       n=st.integers(1, 70), d=st.sampled_from([1, 4, 64]), causal=st.booleans(),
       scale=st.floats(0.01, 2.0), seed=st.integers(0, 2**16))
def test_matches_torch_sdpa_float64(B, hkv, G, n, d, causal, scale, seed):
    """P16: PyTorch CPU float64 SDPA (is_causal, enable_gqa, scale=) agrees on small shapes."""
    hq = hkv * G
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, hq, n, d, generator=g, dtype=torch.float64)
    k = torch.randn(B, hkv, n, d, generator=g, dtype=torch.float64)
    v = torch.randn(B, hkv, n, d, generator=g, dtype=torch.float64)
    ref = torch.nn.functional.scaled_dot_product_attention(
        q, k, v, is_causal=causal, scale=scale, enable_gqa=True).numpy()
    o, _ = oracle.attention(q.numpy(), k.numpy(), v.numpy(), causal, scale)
    assert np.abs(o - ref).max() <= 1e-12


@pytest.mark.parametrize("per_block", [1, 2, 256])
@pytest.mark.parametrize("rows", [[0, 1, 17, 48, 49], [49, 3, 17, 0, 30, 2]])
def test_rows_variant_matches_full(per_block, rows):
    """attention_rows evaluates the same definition at chosen rows and heads,
    whatever the rows' order and however they are grouped."""
    q, k, v, scale = prefill_inputs(2, 4, 2, 50, 16, "bf16", seed=5)
    o, lse = oracle.attention(q, k, v, True, scale)
    heads = [(0, 0), (1, 3), (0, 2)]
    orr, lr = oracle.attention_rows(q, k, v, True, scale, rows, heads, rows_per_block=per_block)
    for t, (b, h) in enumerate(heads):
        assert np.abs(orr[t] - o[b, h, rows]).max() <= 1e-13
        assert np.abs(lr[t] - lse[b, h, rows]).max() <= 1e-13
    on, ln_ = oracle.attention_rows(q, k, v, False, scale, rows, heads, rows_per_block=per_block)
    of, lf = oracle.attention(q, k, v, False, scale)
    for t, (b, h) in enumerate(heads):
        assert np.abs(on[t] - of[b, h, rows]).max() <= 1e-13


# ---------------------------------------------------------------- printed numbers
def _golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                rows.append([int(x) for x in line.split()])
    return rows


def test_score_matrix_has_n_squared_entries():
    """The materialised score matrix has the sizes the pages print (1k -> 1M, 8k -> 64M)."""
    for tokens, entries in _golden("score_matrix_entries.txt"):
        x = np.zeros((tokens, 1))
        s = oracle.score_matrix(x, x, 1.0, False)
        assert s.size == entries
        del s


def test_gemm_tiling_traffic_matches_page():
    """Page-1 tiled-GEMM load counts (25 tiles -> 650 loads / 26000 MiB; 13 -> 182 / 14560)."""
    for tiles, mib, loads, total in _golden("gemm_tiling_traffic.txt"):
        assert oracle.tiled_gemm_reads(tiles, mib) == (loads, total)


# ---------------------------------------------------------------- planted mistakes
def _planted(monkeypatch, fn):
    monkeypatch.setattr(oatt, "score_matrix", fn)


def test_pins_catch_dropped_scale(monkeypatch):
    real = oatt.score_matrix
    _planted(monkeypatch, lambda q, k, scale, causal: real(q, k, 1.0, causal))
    q, k, v = (torch.randn(1, 1, 6, 4, dtype=torch.float64) for _ in range(3))
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=0.3).numpy()
    o, _ = oracle.attention(q.numpy(), k.numpy(), v.numpy(), False, 0.3)
    assert np.abs(o - ref).max() > 1e-6


def test_pins_catch_flipped_causal_mask(monkeypatch):
    def flipped(q, k, scale, causal):
        s = float(scale) * (np.asarray(q, float) @ np.asarray(k, float).T)
        if causal:
            s[np.tril(np.ones(s.shape, dtype=bool), k=-1)] = -np.inf
        return s
    _planted(monkeypatch, flipped)
    q, k, v = rand((1, 1, 9, 7), 10), rand((1, 1, 9, 7), 11), rand((1, 1, 9, 7), 12)
    o, _ = oracle.attention(q, k, v, True, 0.37)
    assert not np.array_equal(o[:, :, 0], v[:, :, 0])


def test_pins_catch_wrong_head_map(monkeypatch):
    monkeypatch.setattr(oatt, "_kv_head", lambda h, hq, hkv: h % hkv)
    g = torch.Generator().manual_seed(1)
    q = torch.randn(1, 4, 5, 3, generator=g, dtype=torch.float64)
    k = torch.randn(1, 2, 5, 3, generator=g, dtype=torch.float64)
    v = torch.randn(1, 2, 5, 3, generator=g, dtype=torch.float64)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, enable_gqa=True).numpy()
    o, _ = oracle.attention(q.numpy(), k.numpy(), v.numpy(), False, 1 / math.sqrt(3))
    assert np.abs(o - ref).max() > 1e-6


# ---------------------------------------------------------------- P17 - P19: paged decode
def _pool(logical_k, logical_v, lens, page, seed, spare=2):
    """Scatter logical caches [B,Hkv,maxlen,d] into shuffled pool pages (numpy).

    Unused pool pages and unused table entries are NaN pages, so reading
    anything outside a sequence poisons the result."""
    B, hkv, maxlen, d = logical_k.shape
    npg = [-(-n // page) for n in lens]
    used = sum(npg)
    slots = np.random.default_rng(seed).permutation(used + spare)
    kp = np.full((used + spare, hkv, page, d), np.nan)
    vp = np.full_like(kp, np.nan)
    table = np.full((B, -(-maxlen // page)), slots[used], dtype=np.int32)
    j = 0
    for b in range(B):
        for i in range(npg[b]):
            rows = min(page, maxlen - i * page)
            kp[slots[j], :, :rows] = logical_k[b, :, i * page:i * page + rows]
            vp[slots[j], :, :rows] = logical_v[b, :, i * page:i * page + rows]
            table[b, i] = slots[j]
            j += 1
    return kp, vp, table


def _paged_identical_keys_error(fn):
    """Max error of fn against the closed form for identical keys: the mean of
    the visible logical V rows (computed here from the logical rows)."""
    lens, page, d, hkv, hq = [1, 4, 5, 8, 11, 0], 4, 3, 2, 4
    B, maxlen = len(lens), 12
    k = np.repeat(rand((1, 1, 1, d), 70), B * hkv * maxlen, axis=0).reshape(B, hkv, maxlen, d)
    v = rand((B, hkv, maxlen, d), 71)
    for b, n in enumerate(lens):
        v[b, :, n:] = np.nan  # never visible
    kp, vp, table = _pool(k, v, lens, page, seed=5)
    q = rand((B, hq, d), 72)
    o, _ = fn(q, kp, vp, table, lens, 0.8)
    err = 0.0
    for b, n in enumerate(lens):
        for h in range(hq):
            want = np.zeros(d) if n == 0 else v[b, h // 2, :n].mean(axis=0)
            e = float(np.abs(o[b, h] - want).max())
            err = max(err, e if math.isfinite(e) else math.inf)  # a NaN read counts as wrong
    return err


def test_paged_identical_keys_give_mean_of_logical_rows():
    """P17: paged decode with identical keys returns the mean of the sequence's
    logical V rows 0..L-1, across page boundaries and for L = 0."""
    assert _paged_identical_keys_error(oracle.decode_paged) <= 1e-14


def test_paged_needle_selects_its_logical_row():
    """P18: one cached key scoring 50 above the rest returns its logical V row
    (closed form (e^50 v* + sum of the others) / (e^50 + L - 1))."""
    page, d, L = 4, 3, 13
    for jstar in (0, 3, 4, 7, 8, 12):
        k = np.zeros((1, 1, 16, d))
        k[0, 0, jstar, 0] = 50.0
        v = rand((1, 1, 16, d), 73 + jstar)
        kp, vp, table = _pool(k, v, [L], page, seed=jstar)
        q = np.zeros((1, 1, d))
        q[0, 0, 0] = 1.0
        o, lse = oracle.decode_paged(q, kp, vp, table, [L], 1.0)
        e = math.exp(50.0)
        want = (e * v[0, 0, jstar] + v[0, 0, :L].sum(axis=0) - v[0, 0, jstar]) / (e + L - 1)
        assert np.abs(o[0, 0] - want).max() <= 1e-14
        assert abs(lse[0, 0] - (50.0 + math.log(1 + (L - 1) * math.exp(-50.0)))) <= 1e-12


def test_paged_shared_pages_and_table_tail_never_read():
    """P19: two sequences whose tables name the same pool pages for the same
    length give identical results; table entries past the last page are never
    read (they hold an id outside the pool)."""
    page, d = 8, 4
    kp = rand((5, 1, page, d), 80)
    vp = rand((5, 1, page, d), 81)
    table = np.array([[3, 1, 4, 999], [3, 1, 4, -7]], dtype=np.int32)
    q = np.repeat(rand((1, 2, d), 82), 2, axis=0)
    o, lse = oracle.decode_paged(q, kp, vp, table, [20, 20], 0.6)
    assert np.array_equal(o[0], o[1]) and np.array_equal(lse[0], lse[1])
    with pytest.raises(IndexError):
        oracle.decode_paged(q, kp, vp, table, [20, 25], 0.6)  # 25 keys need a 4th page


def test_pins_catch_page_off_by_one():
    """A gather that takes each sequence's pages one table entry late fails P17."""
    def shifted(q, kp, vp, table, lens, scale):
        t = np.asarray(table)
        return oracle.decode_paged(q, kp, vp, np.concatenate([t[:, 1:], t[:, :1]], axis=1), lens, scale)
    assert not _paged_identical_keys_error(shifted) <= 1e-6


def test_paged_generator_matches_contiguous_cache():
    """The shared paged-cache generator keeps the logical cache: the oracle
    over its pool equals the oracle over the contiguous cache."""
    from exact_tiled_attention_prefill_amd.inputs import paged_cache
    q, kc, vc, lens, scale = decode_inputs(3, 4, 2, 8, 1, 40, 48, "bf16", seed=9)
    for page in (16, 32):
        kp, vp, table, _ = paged_cache(kc, vc, lens, page, seed=page)
        o1, l1 = oracle.decode_paged(q, kp, vp, table, lens, scale)
        o2, l2 = oracle.decode(q, kc, vc, lens, scale)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


# ---------------------------------------------------------------- P20 - P24: packed variable-length prefill
def _pack(seqs_q, seqs_k):
    """Per-sequence arrays [n, H, d] -> packed arrays and cumulative offsets."""
    cu_q = np.cumsum([0] + [len(x) for x in seqs_q])
    cu_k = np.cumsum([0] + [len(x) for x in seqs_k])
    return np.concatenate(seqs_q), np.concatenate(seqs_k), cu_q, cu_k


@pytest.mark.parametrize("lens", [[(5, 9), (7, 7), (1, 12)], [(16, 40), (33, 33)]])
@pytest.mark.parametrize("hq,hkv", [(2, 2), (4, 1)])
def test_varlen_causal_matches_torch_lower_right(lens, hq, hkv):
    """P20: causal varlen rows equal PyTorch CPU float64 SDPA with its own
    bottom-right causal bias (torch.nn.attention.bias.causal_lower_right),
    sequence by sequence, GQA by repeating K/V heads."""
    from torch.nn.attention.bias import causal_lower_right
    d, scale = 8, 0.41
    qs = [rand((nq, hq, d), 100 + i) for i, (nq, _) in enumerate(lens)]
    ks = [rand((nk, hkv, d), 200 + i) for i, (_, nk) in enumerate(lens)]
    vs = [rand((nk, hkv, d), 300 + i) for i, (_, nk) in enumerate(lens)]
    q, k, cu_q, cu_k = _pack(qs, ks)
    v = np.concatenate(vs)
    o, lse = oracle.attention_varlen(q, k, v, cu_q, cu_k, True, scale)
    for b, (nq, nk) in enumerate(lens):
        tq = torch.from_numpy(qs[b]).permute(1, 0, 2)[None]
        tk = torch.from_numpy(np.repeat(ks[b], hq // hkv, axis=1)).permute(1, 0, 2)[None]
        tv = torch.from_numpy(np.repeat(vs[b], hq // hkv, axis=1)).permute(1, 0, 2)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            tq, tk, tv, attn_mask=causal_lower_right(nq, nk), scale=scale)[0].permute(1, 0, 2).numpy()
        assert np.abs(o[cu_q[b]:cu_q[b + 1]] - ref).max() <= 1e-12


def test_varlen_window_zero_returns_diagonal_value():
    """P21: window 0 under the causal mask leaves one key per row, key i + off:
    o = V[i + off], lse = scale * q_i . k_{i + off} (closed form)."""
    d, nq, nk, scale = 5, 6, 10, 0.7
    q, k, v = rand((nq, 2, d), 400), rand((nk, 1, d), 401), rand((nk, 1, d), 402)
    o, lse = oracle.attention_varlen(q, k, v, [0, nq], [0, nk], True, scale, window_left=0)
    for i in range(nq):
        j = i + nk - nq
        for h in range(2):
            assert np.array_equal(o[i, h], v[j, 0])
            assert abs(lse[h, i] - scale * q[i, h] @ k[j, 0]) <= 1e-14


@pytest.mark.parametrize("w", [1, 3, 50])
def test_varlen_window_identical_keys_give_window_mean(w):
    """P22: identical keys -> uniform weights over the window
    [max(0, i+off-W), i+off]: o = mean of those V rows, lse = s + ln(count)."""
    d, nq, nk, scale = 4, 7, 12, 0.3
    q = rand((nq, 1, d), 410)
    k = np.repeat(rand((1, 1, d), 411), nk, axis=0)
    v = rand((nk, 1, d), 412)
    o, lse = oracle.attention_varlen(q, k, v, [0, nq], [0, nk], True, scale, window_left=w)
    for i in range(nq):
        hi = i + nk - nq
        lo = max(0, hi - w)
        assert np.abs(o[i, 0] - v[lo:hi + 1, 0].mean(axis=0)).max() <= 1e-14
        assert abs(lse[0, i] - (scale * q[i, 0] @ k[0, 0] + math.log(hi - lo + 1))) <= 1e-13


def test_varlen_rows_without_keys_and_chunking():
    """P23: causal rows with i + (n_k - n_q) < 0 see no key (o = 0, lse = -inf);
    the last n_q rows of a full causal prefill equal a chunk of n_q queries
    against the whole key prefix (dense oracle, itself pinned against SDPA)."""
    d, n, scale = 6, 20, 0.5
    q, k, v = rand((1, 2, n, d), 420), rand((1, 1, n, d), 421), rand((1, 1, n, d), 422)
    full_o, full_l = oracle.attention(q, k, v, True, scale)
    qp, kp, vp = (x[0].transpose(1, 0, 2) for x in (q, k, v))  # [n, H, d]
    for nq in (1, 7, 20):
        o, lse = oracle.attention_varlen(qp[n - nq:], kp, vp, [0, nq], [0, n], True, scale)
        assert np.abs(o - full_o[0][:, n - nq:].transpose(1, 0, 2)).max() <= 1e-13
        assert np.abs(lse - full_l[0][:, n - nq:]).max() <= 1e-13
    # more queries than keys: the first 3 rows see nothing
    o, lse = oracle.attention_varlen(qp[:8], kp[:5], vp[:5], [0, 8], [0, 5], True, scale)
    assert np.all(o[:3] == 0) and np.all(np.isneginf(lse[:, :3]))
    assert np.isfinite(lse[:, 3:]).all()


@pytest.mark.parametrize("lens", [[(5, 9), (7, 7), (12, 3)], [(16, 40), (33, 33), (50, 20)]])
@pytest.mark.parametrize("hq,hkv", [(2, 2), (4, 1)])
def test_varlen_noncausal_matches_torch_sdpa(lens, hq, hkv):
    """P20b: without the causal mask and without a window every row sees all
    n_k keys of its sequence, whatever n_q is: the rows equal PyTorch CPU
    float64 SDPA with no mask, sequence by sequence (GQA by repeating K/V
    heads), including sequences with more queries than keys."""
    d, scale = 8, 0.37
    qs = [rand((nq, hq, d), 130 + i) for i, (nq, _) in enumerate(lens)]
    ks = [rand((nk, hkv, d), 230 + i) for i, (_, nk) in enumerate(lens)]
    vs = [rand((nk, hkv, d), 330 + i) for i, (_, nk) in enumerate(lens)]
    q, k, cu_q, cu_k = _pack(qs, ks)
    v = np.concatenate(vs)
    o, lse = oracle.attention_varlen(q, k, v, cu_q, cu_k, False, scale)
    for b, (nq, nk) in enumerate(lens):
        tq = torch.from_numpy(qs[b]).permute(1, 0, 2)[None]
        tk = torch.from_numpy(np.repeat(ks[b], hq // hkv, axis=1)).permute(1, 0, 2)[None]
        tv = torch.from_numpy(np.repeat(vs[b], hq // hkv, axis=1)).permute(1, 0, 2)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale)[0].permute(1, 0, 2).numpy()
        assert np.abs(o[cu_q[b]:cu_q[b + 1]] - ref).max() <= 1e-12
        # lse: log of the row's sum of exp(scale q.k), by logsumexp of torch
        s = scale * torch.einsum("qhd,khd->hqk", torch.from_numpy(qs[b]),
                                 torch.from_numpy(np.repeat(ks[b], hq // hkv, axis=1)))
        assert np.abs(lse[:, cu_q[b]:cu_q[b + 1]] - torch.logsumexp(s, dim=-1).numpy()).max() <= 1e-12


# sequences (n_q, n_k) with the queries at the end (off > 0), aligned (off = 0)
# and with more queries than keys (off < 0, the window bound moves left)
NONCAUSAL_WINDOW_LENS = [(7, 12), (6, 6), (9, 5)]


@pytest.mark.parametrize("w", [0, 1, 3, 50])
def test_varlen_noncausal_window_identical_keys_give_tail_mean(w):
    """P22b: without the causal mask a window W >= 0 is left-only: row i of a
    sequence sees keys max(0, i + off - W) .. n_k - 1 with off = n_k - n_q
    (the queries are the last n_q positions).  With identical keys the weights
    are uniform over that range: o = the mean of those V rows and
    lse = s + ln(count) (closed form).  Every row keeps at least key n_k - 1,
    since i + off - W <= n_k - 1."""
    d, scale = 4, 0.3
    qs = [rand((nq, 1, d), 430 + i) for i, (nq, _) in enumerate(NONCAUSAL_WINDOW_LENS)]
    key = rand((1, 1, d), 440)
    ks = [np.repeat(key, nk, axis=0) for _, nk in NONCAUSAL_WINDOW_LENS]
    vs = [rand((nk, 1, d), 450 + i) for i, (_, nk) in enumerate(NONCAUSAL_WINDOW_LENS)]
    q, k, cu_q, cu_k = _pack(qs, ks)
    v = np.concatenate(vs)
    o, lse = oracle.attention_varlen(q, k, v, cu_q, cu_k, False, scale, window_left=w)
    for b, (nq, nk) in enumerate(NONCAUSAL_WINDOW_LENS):
        for i in range(nq):
            lo = max(0, i + nk - nq - w)
            row = cu_q[b] + i
            assert np.abs(o[row, 0] - vs[b][lo:, 0].mean(axis=0)).max() <= 1e-14
            assert abs(lse[0, row] - (scale * qs[b][i, 0] @ key[0, 0] + math.log(nk - lo))) <= 1e-13


def test_pins_catch_noncausal_window_from_row_index(monkeypatch):
    """A non-causal window measured from the packed row index i instead of the
    row's position i + off fails P22b (off != 0 for two of its sequences)."""
    real = oatt.varlen_visible

    def wrong(i, nq, nk, causal, w):
        lo, hi = real(i, nq, nk, causal, w)
        if not causal and w >= 0:
            lo = max(0, i - w)
        return lo, hi

    monkeypatch.setattr(oatt, "varlen_visible", wrong)
    with pytest.raises(AssertionError):
        test_varlen_noncausal_window_identical_keys_give_tail_mean(1)


def test_pins_catch_window_off_by_one(monkeypatch):
    """A window that keeps one key too many fails P21."""
    real = oatt.varlen_visible
    monkeypatch.setattr(oatt, "varlen_visible",
                        lambda i, nq, nk, c, w: real(i, nq, nk, c, w + 1 if w >= 0 else w))
    d, nq, nk = 5, 6, 10
    q, k, v = rand((nq, 1, d), 400), rand((nk, 1, d), 401), rand((nk, 1, d), 402)
    o, _ = oracle.attention_varlen(q, k, v, [0, nq], [0, nk], True, 0.7, window_left=0)
    assert not np.array_equal(o[1, 0], v[1 + nk - nq, 0])


# ---------------------------------------------------------------- P24 - P26: backward
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("hq,hkv", [(2, 2), (4, 2), (3, 1)])
def test_backward_matches_torch_autograd(causal, hq, hkv):
    """P24: dq, dk, dv equal PyTorch float64 autograd through its own
    scaled_dot_product_attention (is_causal, enable_gqa)."""
    g = torch.Generator().manual_seed(7 + hq + causal)
    q = torch.randn(2, hq, 9, 5, generator=g, dtype=torch.float64, requires_grad=True)
    k = torch.randn(2, hkv, 9, 5, generator=g, dtype=torch.float64, requires_grad=True)
    v = torch.randn(2, hkv, 9, 5, generator=g, dtype=torch.float64, requires_grad=True)
    do = torch.randn(2, hq, 9, 5, generator=g, dtype=torch.float64)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal, scale=0.37,
                                                         enable_gqa=hq != hkv)
    o.backward(do)
    dq, dk, dv = oracle.attention_backward(q.detach(), k.detach(), v.detach(), do, causal, 0.37)
    assert np.abs(dq - q.grad.numpy()).max() <= 1e-12
    assert np.abs(dk - k.grad.numpy()).max() <= 1e-12
    assert np.abs(dv - v.grad.numpy()).max() <= 1e-12


def test_backward_matches_finite_differences():
    """P25: central differences of sum(o * do) in float64 (step 1e-6) agree
    with every gradient entry to 1e-7."""
    q, k, v, do = rand((1, 2, 4, 3), 500), rand((1, 1, 4, 3), 501), rand((1, 1, 4, 3), 502), rand((1, 2, 4, 3), 503)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, True, 0.8)

    def loss(q_, k_, v_):
        o, _ = oracle.attention(q_, k_, v_, True, 0.8)
        return float((o * do).sum())
    eps = 1e-6
    for x, grad, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[which], args_m[which] = xp, xm
            fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert abs(fd - grad[idx]) <= 1e-7, (which, idx, fd, grad[idx])


def test_backward_single_key_closed_form():
    """P26: with one visible key the softmax is constant: dq = dk = 0 and
    dv = do (summed over the heads sharing the key/value head)."""
    q, k, v, do = rand((1, 4, 1, 6), 510), rand((1, 2, 1, 6), 511), rand((1, 2, 1, 6), 512), rand((1, 4, 1, 6), 513)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, False, 1.3)
    assert np.all(dq == 0) and np.all(dk == 0)
    assert np.allclose(dv[0, 0], do[0, 0] + do[0, 1], rtol=0, atol=1e-15)
    assert np.allclose(dv[0, 1], do[0, 2] + do[0, 3], rtol=0, atol=1e-15)


def test_pins_catch_missing_softmax_correction(monkeypatch):
    """A backward that drops the -rowsum(p dp) term fails P24."""
    def wrong(q, k, v, do, causal, scale):
        q, k, v, do = (oatt._f64(x) for x in (q, k, v, do))
        dq = np.zeros_like(q)
        for h in range(q.shape[1]):
            s = oatt.score_matrix(q[0, h], k[0, h], scale, causal)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            dq[0, h] = scale * ((p * (do[0, h] @ v[0, h].T)) @ k[0, h])
        return dq
    g = torch.Generator().manual_seed(3)
    q = torch.randn(1, 2, 6, 4, generator=g, dtype=torch.float64, requires_grad=True)
    k = torch.randn(1, 2, 6, 4, generator=g, dtype=torch.float64)
    v = torch.randn(1, 2, 6, 4, generator=g, dtype=torch.float64)
    do = torch.randn(1, 2, 6, 4, generator=g, dtype=torch.float64)
    torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=0.5).backward(do)
    assert np.abs(wrong(q.detach(), k, v, do, False, 0.5) - q.grad.numpy()).max() > 1e-6
