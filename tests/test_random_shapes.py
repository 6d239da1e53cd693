"""GPU parity on seeded random shapes across the entry points.

The hand-picked cases elsewhere cover tile edges and the published
workloads; these draw shapes, head groupings, masks, scales, (packed)
sequence lengths and page sizes from a fixed seed, for every entry point
including the backward and the paged decode, so that combinations nobody picked by hand
are compared element by element with the fp64 oracle too.  Each case prints
its parameters before it runs.  The scales reach 5.7x the named workloads'
1/sqrt(d), so the bf16 outputs are held to the per-element bar their
arithmetic gives (gpu_util.check_bf16_elementwise: (2^-8 + 2^-10) (|o| + a) +
1e-5 with a the oracle's output for |V|) and mean-abs 2e-3, lse to 1e-3;
fp32 to 1e-5.
"""

import random

import numpy as np
import pytest
import torch

import oracle
from exact_tiled_attention_prefill_amd import decode, decode_paged, prefill, prefill_backward, prefill_varlen
from exact_tiled_attention_prefill_amd import inputs as I
from gpu_util import BF16_LSE_MAX_ABS, F32_LSE_MAX_ABS, F32_MAX_ABS, check_bf16_elementwise, check_close, f64, to_dev

pytestmark = pytest.mark.gpu


def fp32(x):
    """A drawn scale as the fp32 value the kernels receive (the oracle widens that value)."""
    return float(np.float32(x))


def check_f32_lse(lse_gpu, lse_ref, what):
    """fp32 lse: 1e-5 plus one ulp of the fp32 output, whose half-ulp alone is 7.6e-6 at
    |lse| = 128 and 1.5e-5 at 256 (the sharp softmaxes of the larger drawn scales)."""
    err = np.abs(f64(lse_gpu) - lse_ref)
    bound = F32_LSE_MAX_ABS + 2.0 ** -23 * np.abs(lse_ref)
    assert np.isfinite(err).all() and (err <= bound).all(), f"{what}: max excess {(err - bound).max():.3e}"


def _dense_cases(n, seed):
    rng = random.Random(seed)
    cases = []
    while len(cases) < n:
        d = rng.choice([64, 128])
        hkv = rng.choice([1, 2, 3])
        g = rng.choice([1, 2, 3, 4, 8])
        b = rng.choice([1, 2, 3])
        nn = rng.choice([rng.randint(1, 200), rng.randint(200, 1500), rng.randint(1500, 3000)])
        if b * hkv * g * nn * nn > 1.2e8:  # keeps the materialised oracle to seconds
            continue
        causal = rng.random() < 0.6
        scale = rng.choice([None, rng.uniform(-0.3, 0.5)])
        cases.append((b, hkv, g, nn, d, causal, scale, rng.randint(0, 10 ** 6)))
    return cases


@pytest.mark.parametrize("B,Hkv,G,N,d,causal,scale,seed", _dense_cases(16, 2024))
def test_random_dense_prefill_bf16(B, Hkv, G, N, d, causal, scale, seed):
    print(f"dense bf16 B{B} Hkv{Hkv} G{G} N{N} d{d} causal={causal} scale={scale}", flush=True)
    q, k, v, s0 = I.prefill_inputs(B, Hkv * G, Hkv, N, d, "bf16", seed=seed)
    scale = s0 if scale is None else fp32(scale)
    o, lse = prefill(*to_dev(q, k, v), causal=causal, scale=scale)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(q, k, v, causal, scale)
    ra, _ = oracle.attention(q, k, v.abs(), causal, scale)
    check_bf16_elementwise(o, ro, ra, "o")
    check_close(lse, rl, BF16_LSE_MAX_ABS, "lse")


@pytest.mark.parametrize("B,Hkv,G,N,d,causal,scale,seed", _dense_cases(6, 77)[:6])
def test_random_dense_prefill_f32(B, Hkv, G, N, d, causal, scale, seed):
    print(f"dense f32 B{B} Hkv{Hkv} G{G} N{N} d{d} causal={causal} scale={scale}", flush=True)
    q, k, v, s0 = I.prefill_inputs(B, Hkv * G, Hkv, N, d, "f32", seed=seed)
    scale = s0 if scale is None else fp32(scale)
    o, lse = prefill(*to_dev(q, k, v), causal=causal, scale=scale)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(q, k, v, causal, scale)
    check_close(o, ro, F32_MAX_ABS, "o")
    check_f32_lse(lse, rl, "lse")


def _wide_cases(n, seed):
    rng = random.Random(seed)
    out = []
    for _ in range(n):
        causal = rng.random() < 0.5
        nn = rng.randint(16400, 20000) if causal else rng.randint(8200, 12000)
        out.append((rng.choice([1, 2]), rng.choice([1, 2, 4]), nn, causal, rng.randint(0, 10 ** 6)))
    return out


@pytest.mark.parametrize("Hkv,G,N,causal,seed", _wide_cases(4, 31337))
def test_random_wide_prefill_bf16(Hkv, G, N, causal, seed):
    """Rows long enough for the 8-wave launch (d = 128), sampled rows of every head."""
    print(f"wide bf16 Hkv{Hkv} G{G} N{N} causal={causal}", flush=True)
    q, k, v, scale = I.prefill_inputs(1, Hkv * G, Hkv, N, 128, "bf16", seed=seed)
    o, lse = prefill(*to_dev(q, k, v), causal=causal, scale=scale)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    rng = random.Random(seed)
    rows = sorted({0, 1, 255, 256, N - 2, N - 1} | {rng.randrange(N) for _ in range(30)})
    heads = [(0, h) for h in range(Hkv * G)]
    ro, rl = oracle.attention_rows(q, k, v, causal, scale, rows, heads)
    ra, _ = oracle.attention_rows(q, k, v.abs(), causal, scale, rows, heads)
    idx = torch.as_tensor(rows)
    check_bf16_elementwise(torch.stack([o[0, h][idx] for _, h in heads]), ro, ra, "wide o")
    check_close(torch.stack([lse[0, h][idx] for _, h in heads]), rl, BF16_LSE_MAX_ABS, "wide lse")


def _varlen_cases(n, seed):
    rng = random.Random(seed)
    out = []
    for _ in range(n):
        lens = []
        for _ in range(rng.randint(1, 6)):
            nk = rng.randint(0, 900)
            nq = rng.choice([nk, rng.randint(0, nk + 1), rng.randint(0, 300)])
            lens.append((nq, nk))
        if sum(a for a, _ in lens) == 0:
            lens.append((5, 9))
        if sum(b for _, b in lens) == 0:
            lens.append((3, 4))
        window = rng.choice([-1, -1, rng.randint(0, 300)])
        out.append((lens, rng.choice([1, 2]), rng.choice([1, 2, 4]), rng.choice([64, 128]), rng.random() < 0.6,
                    window, rng.randint(0, 10 ** 6)))
    return out


@pytest.mark.parametrize("lens,Hkv,G,d,causal,window,seed", _varlen_cases(10, 555))
def test_random_varlen_prefill(lens, Hkv, G, d, causal, window, seed):
    print(f"varlen {lens} Hkv{Hkv} G{G} d{d} causal={causal} window={window}", flush=True)
    q, k, v, cu_q, cu_k, scale = I.varlen_inputs(lens, Hkv * G, Hkv, d, seed=seed)
    max_q = max(1, max(nq for nq, _ in lens))
    o, lse = prefill_varlen(*to_dev(q, k, v, cu_q, cu_k), max_q, causal=causal, window_left=window, scale=scale)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_varlen(q, k, v, cu_q, cu_k, causal, scale, window_left=window)
    ra, _ = oracle.attention_varlen(q, k, v.abs(), cu_q, cu_k, causal, scale, window_left=window)
    check_bf16_elementwise(o, ro, ra, "varlen o")
    g = f64(lse)
    empty = np.isneginf(rl)
    assert np.array_equal(np.isneginf(g), empty), "rows without keys differ"
    if (~empty).any():
        assert np.abs(g[~empty] - rl[~empty]).max() <= BF16_LSE_MAX_ABS
    if empty.any():
        assert torch.all(o.cpu()[np.where(empty.any(axis=0))[0]] == 0)


def _decode_cases(n, seed):
    rng = random.Random(seed)
    out = []
    for _ in range(n):
        maxlen = rng.choice([rng.randint(1, 300), rng.randint(300, 5000), rng.randint(5000, 40000)])
        b = rng.randint(1, 12)
        lens = [rng.randint(0, maxlen) for _ in range(b)]
        out.append((lens, maxlen, rng.choice([1, 2, 4, 8]), rng.choice([1, 3, 4, 5, 8, 16]), rng.choice([64, 128]),
                    rng.choice(["bf16", "bf16", "f32"]), rng.randint(0, 10 ** 6)))
    return out


@pytest.mark.parametrize("lens,maxlen,Hkv,G,d,dtype,seed", _decode_cases(10, 909))
def test_random_decode(lens, maxlen, Hkv, G, d, dtype, seed):
    print(f"decode {dtype} B{len(lens)} maxlen{maxlen} Hkv{Hkv} G{G} d{d}", flush=True)
    q, kc, vc, ls, scale = I.decode_inputs(len(lens), Hkv * G, Hkv, d, 0, maxlen, maxlen, dtype, seed=seed,
                                           seqlens=lens)
    o = decode(*to_dev(q, kc, vc, ls), scale=scale)
    torch.cuda.synchronize()
    ro, _ = oracle.decode(q, kc, vc, ls, scale)
    if dtype == "f32":
        check_close(o, ro, F32_MAX_ABS, "decode f32")
    else:
        ra, _ = oracle.decode(q, kc, vc.abs(), ls, scale)
        check_bf16_elementwise(o, ro, ra, "decode bf16")
    for b, n in enumerate(lens):
        if n == 0:
            assert torch.all(o.cpu()[b] == 0)


def _backward_cases(n, seed):
    rng = random.Random(seed)
    out = []
    for _ in range(n):
        d = rng.choice([64, 128])
        hkv, g, b = rng.choice([1, 2]), rng.choice([1, 2, 3, 4]), rng.choice([1, 2])
        nn = rng.choice([rng.randint(1, 80), rng.randint(80, 400), rng.randint(400, 700)])
        out.append((b, hkv, g, nn, d, rng.random() < 0.6, rng.choice([None, rng.uniform(-0.3, 0.4)]),
                    rng.randint(0, 10 ** 6)))
    return out


@pytest.mark.parametrize("B,Hkv,G,N,d,causal,scale,seed", _backward_cases(8, 4242))
def test_random_backward(B, Hkv, G, N, d, causal, scale, seed):
    """dq, dk, dv against the oracle's backward, with the bar of tests/test_backward.py."""
    print(f"backward B{B} Hkv{Hkv} G{G} N{N} d{d} causal={causal} scale={scale}", flush=True)
    q, k, v, do, s0 = I.backward_inputs(B, Hkv * G, Hkv, N, d, seed=seed)
    scale = s0 if scale is None else fp32(scale)
    qd, kd, vd, dod = to_dev(q, k, v, do)
    o, lse = prefill(qd, kd, vd, causal=causal, scale=scale)
    grads = prefill_backward(qd, kd, vd, o, dod, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    for g, r, name in zip(grads, oracle.attention_backward(q, k, v, do, causal, scale), ("dq", "dk", "dv")):
        err = np.abs(f64(g) - r)
        s = max(1.0, float(np.abs(r).max()))
        assert np.isfinite(err).all(), f"{name}: non-finite"
        assert err.max() <= 2e-2 * s and err.mean() <= 2e-3 * s, (name, err.max(), err.mean(), s)


def _paged_cases(n, seed):
    rng = random.Random(seed)
    out = []
    for _ in range(n):
        maxlen = rng.choice([rng.randint(1, 300), rng.randint(300, 6000), rng.randint(6000, 20000)])
        lens = [rng.randint(0, maxlen) for _ in range(rng.randint(1, 8))]
        out.append((rng.choice([16, 32, 64, 128, 256, 512, 1024]), rng.choice([64, 128]), rng.choice([1, 2, 4]),
                    rng.choice([1, 2, 4, 8, 16]), lens, maxlen, rng.randint(0, 10 ** 6)))
    return out


@pytest.mark.parametrize("page,d,Hkv,G,lens,maxlen,seed", _paged_cases(6, 5151))
def test_random_paged_decode(page, d, Hkv, G, lens, maxlen, seed):
    """Paged decode against the oracle, and bit-identical to contiguous decode of the same cache."""
    print(f"paged decode page{page} d{d} Hkv{Hkv} G{G} B{len(lens)} maxlen{maxlen}", flush=True)
    q, kc, vc, ls, scale = I.decode_inputs(len(lens), Hkv * G, Hkv, d, 0, maxlen, maxlen, "bf16", seed=seed,
                                           seqlens=lens)
    kp, vp, table, _ = I.paged_cache(kc, vc, ls, page, seed=seed)
    o = decode_paged(*to_dev(q, kp, vp, table, ls), scale=scale)
    oc = decode(*to_dev(q, kc, vc, ls), scale=scale)
    torch.cuda.synchronize()
    ro, _ = oracle.decode_paged(q, kp, vp, table, ls, scale)
    ra, _ = oracle.decode_paged(q, kp, vp.abs(), table, ls, scale)
    check_bf16_elementwise(o, ro, ra, "paged decode o")
    assert torch.equal(o, oc), "paged and contiguous decode differ on the same logical cache"
