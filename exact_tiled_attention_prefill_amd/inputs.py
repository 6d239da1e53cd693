"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle checks.

This module draws random numbers and lays them out; it holds none of the
attention arithmetic.  Everything is generated on the CPU with a seeded
torch.Generator so that the GPU path and the CPU oracle see identical values.

Recipe (all five workloads, seed 0 unless stated):
* prefill: one fp32 standard-normal draw per tensor, in the order Q, K, V,
  each in [B, H, N, d] layout, then rounded to bf16 (round-to-nearest-even)
  for the bf16 workloads; the fp32 workload keeps the fp32 values.
* decode: first the per-sequence lengths, uniform integers in [lmin, lmax]
  inclusive; then Q [B, Hq, d]; then for each sequence b in order its K slab
  [Hkv, L_b, d] followed by its V slab.  Cache rows at or past L_b hold NaN so
  that any read beyond a sequence's length poisons the result.
* scale = 1/sqrt(d), stored as the fp32 value handed to the kernels.
"""

import math
from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class PrefillConfig:
    name: str
    B: int
    Hq: int
    Hkv: int
    N: int
    d: int
    causal: bool
    dtype: str  # "bf16" or "f32"


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    lmin: int
    lmax: int
    maxlen: int
    dtype: str


# The five published workloads.
PREFILL_F32_SMALL = PrefillConfig("noncausal-f32-B1H1N256d64", 1, 1, 1, 256, 64, False, "f32")
PREFILL_MHA_4K = PrefillConfig("causal-mha-bf16-B4H32N4096d128", 4, 32, 32, 4096, 128, True, "bf16")
PREFILL_GQA_16K = PrefillConfig("causal-gqa-bf16-B2Hq32Hkv8N16384d128", 2, 32, 8, 16384, 128, True, "bf16")
DECODE_GQA = DecodeConfig("decode-gqa-bf16-B64Hq32Hkv8d128-L1024to32768", 64, 32, 8, 128, 1024, 32768, 32768, "bf16")
PREFILL_GQA_128K = PrefillConfig("causal-gqa-bf16-B1Hq64Hkv8N131072d128", 1, 64, 8, 131072, 128, True, "bf16")


def fp32_scale(d):
    """1/sqrt(d) rounded to fp32, returned as a Python float."""
    return float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32))


def _draw(gen, shape, dtype):
    x = torch.randn(shape, generator=gen, dtype=torch.float32)
    return x.to(torch.bfloat16) if dtype == "bf16" else x


def prefill_inputs(B, Hq, Hkv, N, d, dtype="bf16", seed=0):
    """Return (q, k, v, scale) as CPU tensors: q [B,Hq,N,d], k/v [B,Hkv,N,d]."""
    gen = torch.Generator().manual_seed(seed)
    q = _draw(gen, (B, Hq, N, d), dtype)
    k = _draw(gen, (B, Hkv, N, d), dtype)
    v = _draw(gen, (B, Hkv, N, d), dtype)
    return q, k, v, fp32_scale(d)


def prefill_config_inputs(cfg: PrefillConfig, seed=0):
    return prefill_inputs(cfg.B, cfg.Hq, cfg.Hkv, cfg.N, cfg.d, cfg.dtype, seed)


def decode_inputs(B, Hq, Hkv, d, lmin, lmax, maxlen, dtype="bf16", seed=0, seqlens=None):
    """Return (q, kcache, vcache, seqlens, scale) as CPU tensors.

    q [B,Hq,d]; kcache/vcache [B,Hkv,maxlen,d] with NaN at rows >= L_b;
    seqlens int32 [B].  If `seqlens` is given it replaces the drawn lengths
    (the draw still happens, so the rest of the stream is unchanged).
    """
    gen = torch.Generator().manual_seed(seed)
    drawn = torch.randint(lmin, lmax + 1, (B,), generator=gen, dtype=torch.int64)
    lens = drawn if seqlens is None else torch.as_tensor(seqlens, dtype=torch.int64)
    if int(lens.max()) > maxlen or int(lens.min()) < 0:
        raise ValueError("sequence lengths must lie in [0, maxlen]")
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q = _draw(gen, (B, Hq, d), dtype)
    kc = torch.full((B, Hkv, maxlen, d), float("nan"), dtype=tdt)
    vc = torch.full((B, Hkv, maxlen, d), float("nan"), dtype=tdt)
    for b in range(B):
        n = int(lens[b])
        kc[b, :, :n] = _draw(gen, (Hkv, n, d), dtype)
        vc[b, :, :n] = _draw(gen, (Hkv, n, d), dtype)
    return q, kc, vc, lens.to(torch.int32), fp32_scale(d)


def decode_config_inputs(cfg: DecodeConfig, seed=0, seqlens=None):
    return decode_inputs(cfg.B, cfg.Hq, cfg.Hkv, cfg.d, cfg.lmin, cfg.lmax, cfg.maxlen,
                         cfg.dtype, seed, seqlens)


def sample_rows(n, count, seed=0):
    """Deterministic query rows for sampled checks at large N.

    Always includes the first and last rows and rows next to powers of two
    (tile edges), then fills up with seeded uniform rows.  Sorted, unique.
    """
    rows = {0, 1, 2, 3, n - 2, n - 1}
    p = 1
    while p < n:
        for r in (p - 1, p, p + 1):
            if 0 <= r < n:
                rows.add(r)
        p *= 2
    gen = torch.Generator().manual_seed(seed + 12345)
    extra = torch.randint(0, n, (count,), generator=gen).tolist()
    for r in extra:
        if len(rows) >= count + 6:
            break
        rows.add(int(r))
    return sorted(r for r in rows if 0 <= r < n)


def paged_cache(kcache, vcache, seqlens, page_size, seed=0, spare_pages=2):
    """Scatter contiguous caches [B,Hkv,maxlen,d] into a shuffled page pool.

    Returns (kpages, vpages, block_table, num_pages) with pools
    [num_pages, Hkv, page_size, d] on the caches' device and block_table
    int32 [B, ceil(maxlen/page_size)] (CPU).  Each sequence's pages
    0 .. ceil(L_b/page_size)-1 go to seeded random pool slots; the logical
    rows past L_b (and past maxlen) keep whatever the contiguous cache held
    there, NaN for caches made by decode_inputs.  `spare_pages` extra pool
    pages are NaN, and every block-table entry past a sequence's last page
    names one of them, so a read of anything outside the sequence is NaN.
    Pure data movement: nothing here computes attention.
    """
    B, Hkv, maxlen, d = kcache.shape
    lens = [int(x) for x in torch.as_tensor(seqlens).reshape(-1).tolist()]
    npg = [-(-n // page_size) for n in lens]
    max_pages = -(-maxlen // page_size)
    used = sum(npg)
    num_pages = used + max(1, spare_pages)
    gen = torch.Generator().manual_seed(seed + 777)
    slots = torch.randperm(num_pages, generator=gen).tolist()
    kp = torch.full((num_pages, Hkv, page_size, d), float("nan"), dtype=kcache.dtype, device=kcache.device)
    vp = torch.full_like(kp, float("nan"))
    table = torch.full((B, max_pages), slots[used], dtype=torch.int32)
    if used:
        # logical page i of sequence b -> pool slot, all pages in one gather
        bi = torch.tensor([b for b in range(B) for _ in range(npg[b])], dtype=torch.long)
        pi = torch.tensor([i for b in range(B) for i in range(npg[b])], dtype=torch.long)
        dst = torch.tensor(slots[:used], dtype=torch.long)
        table[bi, pi] = dst.to(torch.int32)
        pad = max_pages * page_size - maxlen  # the last page may run past maxlen: NaN rows
        for src, pool in ((kcache, kp), (vcache, vp)):
            if pad:
                src = torch.cat([src, torch.full((B, Hkv, pad, d), float("nan"), dtype=src.dtype,
                                                 device=src.device)], dim=2)
            pages = src.reshape(B, Hkv, max_pages, page_size, d).permute(0, 2, 1, 3, 4)
            pool[dst.to(pool.device)] = pages[bi.to(pool.device), pi.to(pool.device)]
    return kp, vp, table, num_pages


def varlen_inputs(lens, Hq, Hkv, d, dtype="bf16", seed=0):
    """Packed variable-length inputs for sequences lens = [(n_q, n_k), ...].

    Returns (q [total_q,Hq,d], k, v [total_k,Hkv,d], cu_q, cu_k int32 [B+1],
    scale) as CPU tensors; Q, K, V are each one seeded N(0,1) draw of the
    packed shape, rounded to bf16 (or fp32).  The queries of a sequence are
    its last n_q positions (n_q < n_k: a chunk against a cached prefix).
    """
    gen = torch.Generator().manual_seed(seed)
    tq = sum(nq for nq, _ in lens)
    tk = sum(nk for _, nk in lens)
    q = _draw(gen, (tq, Hq, d), dtype)
    k = _draw(gen, (tk, Hkv, d), dtype)
    v = _draw(gen, (tk, Hkv, d), dtype)
    cu_q = torch.tensor([0] + [sum(nq for nq, _ in lens[:i + 1]) for i in range(len(lens))], dtype=torch.int32)
    cu_k = torch.tensor([0] + [sum(nk for _, nk in lens[:i + 1]) for i in range(len(lens))], dtype=torch.int32)
    return q, k, v, cu_q, cu_k, fp32_scale(d)


def backward_inputs(B, Hq, Hkv, N, d, dtype="bf16", seed=0):
    """(q, k, v, do, scale) for the attention backward: q, k, v as
    prefill_inputs draws them, then the upstream gradient do [B,Hq,N,d] as
    one more seeded N(0,1) draw rounded to bf16 (or fp32)."""
    gen = torch.Generator().manual_seed(seed)
    q = _draw(gen, (B, Hq, N, d), dtype)
    k = _draw(gen, (B, Hkv, N, d), dtype)
    v = _draw(gen, (B, Hkv, N, d), dtype)
    do = _draw(gen, (B, Hq, N, d), dtype)
    return q, k, v, do, fp32_scale(d)
