"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Every test draws seeded inputs on the CPU, runs libfa on the GPU and compares
element by element with the oracle on the same values.  Tolerances: fp32
max-abs 1e-5; bf16 max-abs 2e-2 and mean-abs 2e-3 on O, 1e-3 on lse.
The causal MHA 4K and GQA 16K workloads are compared over their whole
output; the 128K workload on about 100 edge and seeded rows of every head
(the oracle evaluates chosen rows), plus properties checked on every row.
"""

import numpy as np
import pytest
import torch

import oracle
from exact_tiled_attention_prefill_amd import decode, decode_workspace_bytes, prefill
from exact_tiled_attention_prefill_amd import inputs as I
from gpu_util import (BF16_LSE_MAX_ABS, F32_LSE_MAX_ABS, F32_MAX_ABS, boundary_rows, check_bf16,
                      check_causal_invariants, check_close, f64, oracle_rows_parallel, to_dev)

pytestmark = pytest.mark.gpu


def gpu_prefill(q, k, v, causal, scale):
    qd, kd, vd = to_dev(q, k, v)
    o, lse = prefill(qd, kd, vd, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def gpu_decode(q, kc, vc, lens, scale, workspace=False):
    qd, kd, vd, ld = to_dev(q, kc, vc, lens)
    ws = None
    if workspace:
        B, Hq, d = q.shape
        ws = torch.empty(decode_workspace_bytes(B, Hq, kc.shape[1], kc.shape[2], d), dtype=torch.uint8,
                         device="cuda")
    o = decode(qd, kd, vd, ld, scale=scale, workspace=ws)
    torch.cuda.synchronize()
    return o.cpu()


# ------------------------------------------------------------------ fp32
def test_fp32_noncausal_workload():
    """B1 H1 N256 d64 fp32 non-causal, seed 0: max-abs <= 1e-5 on O and lse."""
    cfg = I.PREFILL_F32_SMALL
    q, k, v, scale = I.prefill_config_inputs(cfg)
    o, lse = gpu_prefill(q, k, v, cfg.causal, scale)
    ro, rl = oracle.attention(q, k, v, cfg.causal, scale)
    check_close(o, ro, F32_MAX_ABS, "o")
    check_close(lse, rl, F32_LSE_MAX_ABS, "lse")


@pytest.mark.parametrize("N", [1, 5, 127, 128, 129, 300])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fp32_prefill_shapes(N, d, causal):
    q, k, v, scale = I.prefill_inputs(2, 4, 2, N, d, "f32", seed=N + d)
    o, lse = gpu_prefill(q, k, v, causal, scale)
    ro, rl = oracle.attention(q, k, v, causal, scale)
    check_close(o, ro, F32_MAX_ABS, "o")
    check_close(lse, rl, F32_LSE_MAX_ABS, "lse")


@pytest.mark.parametrize("d,causal,Hq,Hkv,N", [(64, True, 64, 8, 1020), (128, False, 64, 8, 1020),
                                               (64, False, 16, 4, 2000)])
def test_fp32_prefill_large_grid(d, causal, Hq, Hkv, N):
    """The launch forms past the small grids above (which take 16 waves per
    workgroup at d = 64, 8 at d = 128): 64 heads x 64 sixteen-row tiles = 4096
    workgroups take 4 waves, 16 heads x 125 tiles = 2000 workgroups at d = 64
    take 8; ragged last tiles."""
    q, k, v, scale = I.prefill_inputs(1, Hq, Hkv, N, d, "f32", seed=d + N)
    o, lse = gpu_prefill(q, k, v, causal, scale)
    ro, rl = oracle.attention(q, k, v, causal, scale)
    check_close(o, ro, F32_MAX_ABS, "o")
    check_close(lse, rl, F32_LSE_MAX_ABS, "lse")


# ------------------------------------------------------------------ bf16 prefill, small
SMALL = [  # (B, Hkv, G, N, d)
    (1, 1, 1, 1, 128), (1, 1, 1, 2, 64), (2, 1, 2, 63, 128), (1, 2, 1, 64, 64), (1, 1, 4, 65, 128),
    (2, 2, 1, 127, 128), (1, 1, 8, 128, 64), (1, 2, 2, 129, 128), (1, 1, 1, 255, 128),
    (1, 1, 4, 256, 128), (2, 1, 1, 257, 64), (1, 2, 4, 1000, 128), (1, 1, 2, 1000, 64),
    (1, 1, 1, 513, 128), (1, 2, 8, 777, 128), (1, 1, 2, 4097, 64), (2, 2, 3, 300, 128), (1, 3, 3, 129, 64),
]


@pytest.mark.parametrize("B,Hkv,G,N,d", SMALL)
@pytest.mark.parametrize("causal", [False, True])
def test_bf16_prefill_shapes(B, Hkv, G, N, d, causal):
    q, k, v, scale = I.prefill_inputs(B, Hkv * G, Hkv, N, d, "bf16", seed=7 * N + d + G)
    o, lse = gpu_prefill(q, k, v, causal, scale)
    ro, rl = oracle.attention(q, k, v, causal, scale)
    check_bf16(o, ro, "o")
    check_close(lse, rl, BF16_LSE_MAX_ABS, "lse")


def test_bf16_causal_row0_is_exact():
    """Causal row 0 sees only key 0: o must equal V[0] bit for bit."""
    q, k, v, scale = I.prefill_inputs(2, 8, 2, 300, 128, "bf16", seed=11)
    o, lse = gpu_prefill(q, k, v, True, scale)
    g = torch.arange(8) // 4
    assert torch.equal(o[:, :, 0], v[:, g, 0])
    ref = scale * (f64(q[:, :, 0]) * f64(k[:, g, 0])).sum(-1)
    assert np.abs(f64(lse[:, :, 0]) - ref).max() <= BF16_LSE_MAX_ABS


@pytest.mark.parametrize("scale", [-0.0883883, 0.0, 3.0])
def test_bf16_scale_sign_zero_and_large(scale):
    """Negative scale, zero scale (uniform weights) and scores near 1e3 (no overflow)."""
    scale = float(np.float32(scale))  # the fp32 value the kernel receives, which the oracle widens
    q, k, v, _ = I.prefill_inputs(1, 4, 2, 200, 128, "bf16", seed=13)
    for causal in (False, True):
        o, lse = gpu_prefill(q, k, v, causal, scale)
        ro, rl = oracle.attention(q, k, v, causal, scale)
        check_bf16(o, ro, f"o scale={scale}")
        check_close(lse, rl, BF16_LSE_MAX_ABS, f"lse scale={scale}")


def test_bf16_identical_keys_give_prefix_mean():
    q, k, v, scale = I.prefill_inputs(1, 2, 1, 333, 64, "bf16", seed=17)
    k = k[:, :, :1].expand(-1, -1, 333, -1).contiguous()
    o, _ = gpu_prefill(q, k, v, True, scale)
    means = np.cumsum(f64(v), axis=2) / np.arange(1, 334)[None, None, :, None]
    err = np.abs(f64(o)[:, :, :, :] - np.repeat(means, 2, axis=1))
    assert err.max() <= 2e-2


def test_bf16_deterministic_and_prefix_invariant():
    """Two runs are bitwise equal; causal O on the first n rows does not depend on N."""
    q, k, v, scale = I.prefill_inputs(1, 8, 2, 2048, 128, "bf16", seed=19)
    o1, l1 = gpu_prefill(q, k, v, True, scale)
    o2, l2 = gpu_prefill(q, k, v, True, scale)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    n = 1500
    o3, l3 = gpu_prefill(q[:, :, :n].contiguous(), k[:, :, :n].contiguous(), v[:, :, :n].contiguous(),
                         True, scale)
    assert torch.equal(o3, o1[:, :, :n])
    assert torch.equal(l3, l1[:, :, :n])


# ------------------------------------------------------------------ bf16 prefill, full workloads
def _workload_on_gpu(cfg):
    q, k, v, scale = I.prefill_config_inputs(cfg)
    qd, kd, vd = to_dev(q, k, v)
    od, lsed = prefill(qd, kd, vd, causal=cfg.causal, scale=scale)
    torch.cuda.synchronize()
    return (q, k, v, scale), (qd, kd, vd, od, lsed)


def _compare_rows(cfg, host, dev, rows, heads):
    """GPU output at (heads x rows) against the oracle, element by element."""
    q, k, v, scale = host
    od, lsed = dev[3], dev[4]
    ro, rl = oracle_rows_parallel(q, k, v, cfg.causal, scale, rows, heads)
    idx = torch.as_tensor(rows, dtype=torch.long)
    got = torch.stack([od[b, h].cpu()[idx] for b, h in heads])
    got_l = torch.stack([lsed[b, h].cpu()[idx] for b, h in heads])
    check_bf16(got, ro, f"{cfg.name} o")
    check_close(got_l, rl, BF16_LSE_MAX_ABS, f"{cfg.name} lse")


def test_causal_mha_4k_workload():
    """B4 H32 N4096 d128 causal bf16: the whole output (every row of all 128
    heads) against the oracle, and the every-row invariants."""
    cfg = I.PREFILL_MHA_4K
    host, dev = _workload_on_gpu(cfg)
    heads = [(b, h) for b in range(cfg.B) for h in range(cfg.Hq)]
    _compare_rows(cfg, host, dev, np.arange(cfg.N), heads)
    check_causal_invariants(*dev, host[3], cfg.name)


def test_causal_gqa_16k_workload():
    """B2 Hq32 Hkv8 N16384 d128 causal bf16: the whole output (every row of
    all 64 (batch, head) pairs) against the oracle, and the every-row
    invariants."""
    cfg = I.PREFILL_GQA_16K
    host, dev = _workload_on_gpu(cfg)
    heads = [(b, h) for b in range(cfg.B) for h in range(cfg.Hq)]
    _compare_rows(cfg, host, dev, np.arange(cfg.N), heads)
    check_causal_invariants(*dev, host[3], cfg.name)


def test_causal_gqa_128k_workload():
    """B1 Hq64 Hkv8 N131072 d128 causal bf16 (O(N) memory): all 64 heads on
    the tile, wave-interleave, pair-mirror and power-of-two edge rows plus
    seeded rows (about 100 per head) against the oracle, and the every-row
    invariants (row 0 exact, convex hull, lse bounds) on all 8.4M rows."""
    cfg = I.PREFILL_GQA_128K
    host, dev = _workload_on_gpu(cfg)
    rows = boundary_rows(cfg.N, extra=32, seed=5)
    assert len(rows) >= 64
    heads = [(0, h) for h in range(cfg.Hq)]
    _compare_rows(cfg, host, dev, rows, heads)
    check_causal_invariants(*dev, host[3], cfg.name)


# ------------------------------------------------------------------ decode
def test_decode_gqa_workload():
    """B64 Hq32 Hkv8 d128 bf16, lengths uniform in [1024, 32768], NaN past each length."""
    cfg = I.DECODE_GQA
    q, kc, vc, lens, scale = I.decode_config_inputs(cfg)
    o = gpu_decode(q, kc, vc, lens, scale)
    ro, _ = oracle.decode(q, kc, vc, lens, scale)
    check_bf16(o, ro, "decode o")
    o2 = gpu_decode(q, kc, vc, lens, scale, workspace=True)
    assert torch.equal(o, o2)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("G", [1, 2, 3, 4, 6, 8, 12, 16, 24, 32, 37, 48, 64])
def test_decode_lengths_and_groups(dtype, d, G):
    lens = [0, 1, 2, 511, 512, 513, 1024, 1100, 1300, 7]
    q, kc, vc, ls, scale = I.decode_inputs(len(lens), 2 * G, 2, d, 1, 1300, 1300, dtype, seed=G + d,
                                           seqlens=lens)
    o = gpu_decode(q, kc, vc, ls, scale)
    ro, _ = oracle.decode(q, kc, vc, ls, scale)
    if dtype == "f32":
        check_close(o, ro, F32_MAX_ABS, "decode f32")
    else:
        check_bf16(o, ro, "decode bf16")
    assert torch.all(o[0] == 0)  # empty sequence


def test_decode_long_chunk_boundaries():
    """B16 Hq32 Hkv4 d128 with a 32768-key cache launches 2048-key chunks:
    lengths on and around their boundaries, and empty / single-key rows."""
    lens = [0, 1, 2047, 2048, 2049, 4095, 4096, 4097, 30000, 32767, 32768, 6144, 100, 2, 8191, 16385]
    q, kc, vc, ls, scale = I.decode_inputs(len(lens), 32, 4, 128, 1, 32768, 32768, "bf16", seed=9, seqlens=lens)
    o = gpu_decode(q, kc, vc, ls, scale)
    ro, _ = oracle.decode(q, kc, vc, ls, scale)
    check_bf16(o, ro, "decode 2048-key chunks")
    assert torch.all(o[0] == 0)


def test_decode_4096_key_chunk_boundaries():
    """B32 Hq32 Hkv8 d128 with a 32768-key cache launches 4096-key chunks:
    lengths on and around their boundaries (and the 32-key tiles inside
    them), empty and single-key rows."""
    lens = [0, 1, 31, 32, 33, 4095, 4096, 4097, 8191, 8192, 8193, 12288, 16383, 16385, 20000, 24575,
            24576, 24577, 28000, 32767, 32768, 2, 100, 4000, 4127, 7000, 9000, 15000, 30000, 31000, 5, 12345]
    q, kc, vc, ls, scale = I.decode_inputs(len(lens), 32, 8, 128, 1, 32768, 32768, "bf16", seed=10, seqlens=lens)
    o = gpu_decode(q, kc, vc, ls, scale)
    ro, _ = oracle.decode(q, kc, vc, ls, scale)
    check_bf16(o, ro, "decode 4096-key chunks")
    assert torch.all(o[0] == 0)


def test_decode_512_key_chunk_boundaries():
    """B8 Hq8 Hkv1 d128 with a 65536-key cache: 8 (sequence, head-group) rows
    launch 512-key chunks (8 x 128 = 1024 workgroups); lengths on and around
    their boundaries and the full cache."""
    lens = [0, 1, 511, 512, 513, 1025, 65535, 65536]
    q, kc, vc, ls, scale = I.decode_inputs(len(lens), 8, 1, 128, 1, 65536, 65536, "bf16", seed=12, seqlens=lens)
    o = gpu_decode(q, kc, vc, ls, scale)
    ro, _ = oracle.decode(q, kc, vc, ls, scale)
    check_bf16(o, ro, "decode 512-key chunks")
    assert torch.all(o[0] == 0)


@pytest.mark.parametrize("dtype,maxlen,L", [("bf16", 300000, 300000), ("bf16", 300000, 262145),
                                            ("bf16", 300000, 262144), ("bf16", 300000, 257),
                                            ("f32", 600000, 524289), ("f32", 600000, 600000)])
def test_decode_more_than_1024_splits(dtype, maxlen, L):
    """One sequence, one KV head (8 query heads): the bf16 path takes 256-key
    chunks (1172 of them at maxlen 300000) and the fp32 path 512-key chunks
    (1172 at maxlen 600000), so the combine merges more partials than its
    1024-weight LDS batch: lengths giving one split past a batch (1025),
    exactly one batch (1024), a single split, and the full cache."""
    q, kc, vc, ls, scale = I.decode_inputs(1, 8, 1, 128, 1, maxlen, maxlen, dtype, seed=13, seqlens=[L])
    o = gpu_decode(q, kc, vc, ls, scale)
    ro, _ = oracle.decode(q, kc, vc, ls, scale)
    if dtype == "f32":
        check_close(o, ro, F32_MAX_ABS, "decode f32 long")
    else:
        check_bf16(o, ro, "decode bf16 long")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("G", [1, 4, 8])
@pytest.mark.parametrize("scale", [-0.0883883, 0.0, 3.0])
def test_decode_scale_sign_zero_and_large(dtype, G, scale):
    """Negative scale (query signs flipped, positive exponent coefficient),
    zero scale (uniform weights over the visible keys) and scores near 1e2
    (no overflow), for both decode paths."""
    scale = float(np.float32(scale))  # the fp32 value the kernel receives, which the oracle widens
    lens = [1, 31, 33, 300, 1024, 1300, 5]
    q, kc, vc, ls, _ = I.decode_inputs(len(lens), 2 * G, 2, 128, 1, 1300, 1300, dtype, seed=70 + G, seqlens=lens)
    o = gpu_decode(q, kc, vc, ls, scale)
    ro, _ = oracle.decode(q, kc, vc, ls, scale)
    if dtype == "f32":
        check_close(o, ro, F32_MAX_ABS, "decode f32 scale")
    else:
        check_bf16(o, ro, "decode bf16 scale")


@pytest.mark.parametrize("kind", ["large", "falling"])
@pytest.mark.parametrize("lens,d,G,scale", [([35, 20, 1], 128, 4, 0.1416), ([6517, 3000], 128, 4, 0.0884),
                                           ([30000, 513], 64, 8, 0.125)])
def test_decode_f32_sharp_scores(kind, lens, d, G, scale):
    """fp32 decode where rounding is amplified: q and K scaled by 4 (scores
    spread over tens of units, one or two keys carrying the weight), or scores
    falling along the cache (the first entry holds the max and the later
    chunks' weights fall to e^-60 and below).  A single split (35 keys) and
    several, both head dims, held to the fp32 bar."""
    scale = float(np.float32(scale))
    q, kc, vc, ls, _ = I.decode_inputs(len(lens), 2 * G, 2, d, 1, max(lens), max(lens), "f32", seed=90 + d,
                                       seqlens=lens)
    if kind == "large":
        q, kc = q * 4, kc * 4
    else:
        sgn = torch.sign(torch.randn((d,), generator=torch.Generator().manual_seed(d)))
        ramp = torch.linspace(6, 0, max(lens))[None, None, :, None]
        q, kc = q * 0.2 + sgn, kc * 0.2 + ramp * sgn
    o = gpu_decode(q, kc, vc, ls, scale)
    ro, _ = oracle.decode(q, kc, vc, ls, scale)
    check_close(o, ro, F32_MAX_ABS, f"decode f32 {kind}")


def test_decode_f32_merge_at_large_lse():
    """Sharp scores (q and K scaled by 4, scale 0.35, d = 64) over several
    512-key chunks, with chunk log-sum-exps up to ~200, where fp32's half-ulp
    (7.6e-6 above 128) shifts the merge weights.  On these inputs a model with
    exact chunk partials merged through fp32-stored log-sum-exps is off by
    1.02e-5 -- past the fp32 bar on its own -- and by ~1e-7 with fp64 ones."""
    lens, d, G, scale = [3471, 535, 5166], 64, 8, float(np.float32(0.35))
    q, kc, vc, ls, _ = I.decode_inputs(len(lens), 2 * G, 2, d, 1, max(lens), max(lens), "f32", seed=3,
                                       seqlens=lens)
    q, kc = q * 4, kc * 4
    o = gpu_decode(q, kc, vc, ls, scale)
    ro, rl = oracle.decode(q, kc, vc, ls, scale)
    assert np.nanmax(rl) > 128
    check_close(o, ro, F32_MAX_ABS, "decode f32 large lse")


def test_decode_matches_last_prefill_row():
    """Decode of token i against K,V[0..i] equals causal prefill row i (both on the GPU)."""
    q, k, v, scale = I.prefill_inputs(2, 8, 2, 700, 128, "bf16", seed=23)
    o, _ = gpu_prefill(q, k, v, True, scale)
    for i in (0, 1, 511, 512, 699):
        lens = torch.full((2,), i + 1, dtype=torch.int32)
        od = gpu_decode(q[:, :, i].contiguous(), k.contiguous(), v.contiguous(), lens, scale)
        assert np.abs(f64(od) - f64(o[:, :, i])).max() <= 2e-2
