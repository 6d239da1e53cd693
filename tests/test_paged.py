"""GPU parity for decode against a paged KV cache (fa_decode_paged).

The pool and block table come from inputs.paged_cache: each sequence's
logical cache is scattered over shuffled pool pages, and every table entry
past a sequence's last page names a NaN page.  Checks:
- element-wise against the fp64 oracle's paged decode (bf16 tolerances:
  max-abs 2e-2, mean-abs 2e-3);
- bit-identical to fa_decode on the same logical cache.  The chunking and
  arithmetic are the same; only the addresses of the copies differ.
"""

import numpy as np
import pytest
import torch

import oracle
from exact_tiled_attention_prefill_amd import decode, decode_paged, decode_paged_workspace_bytes
from exact_tiled_attention_prefill_amd import inputs as I
from gpu_util import check_bf16, to_dev

pytestmark = pytest.mark.gpu


def run_paged(q, kp, vp, table, lens, scale, workspace=False):
    qd, kd, vd, td, ld = to_dev(q, kp, vp, table, lens)
    ws = None
    if workspace:
        B, Hq, d = q.shape
        ws = torch.empty(decode_paged_workspace_bytes(B, Hq, kp.shape[1], kp.shape[2], table.shape[1], d),
                         dtype=torch.uint8, device="cuda")
    o = decode_paged(qd, kd, vd, td, ld, scale=scale, workspace=ws)
    torch.cuda.synchronize()
    return o.cpu()


def run_contiguous(q, kc, vc, lens, scale):
    qd, kd, vd, ld = to_dev(q, kc, vc, lens)
    o = decode(qd, kd, vd, ld, scale=scale)
    torch.cuda.synchronize()
    return o.cpu()


@pytest.mark.parametrize("page", [16, 32, 64, 256, 2048])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("G", [1, 4, 8, 16, 32])
def test_paged_decode_matches_oracle(page, d, G):
    lens = [0, 1, 15, 16, 17, 511, 1024, 1025, 2000, 2048, 7]
    print(f"paged decode page={page} d={d} G={G}", flush=True)
    q, kc, vc, ls, scale = I.decode_inputs(len(lens), 2 * G, 2, d, 1, 2048, 2048, "bf16", seed=page + d + G,
                                           seqlens=lens)
    kp, vp, table, _ = I.paged_cache(kc, vc, ls, page, seed=page)
    o = run_paged(q, kp, vp, table, ls, scale)
    ro, _ = oracle.decode_paged(q, kp, vp, table, ls, scale)
    check_bf16(o, ro, "paged decode o")
    assert torch.all(o[0] == 0)  # empty sequence
    oc = run_contiguous(q, kc, vc, ls, scale)
    assert torch.equal(o, oc), "paged and contiguous decode differ on the same logical cache"
    assert torch.equal(run_paged(q, kp, vp, table, ls, scale, workspace=True), o)


def test_paged_shared_prefix_pages():
    """Sequences whose tables share pool pages (a common prefix) each see their own logical cache."""
    d, page, G = 128, 32, 4
    lens = [200, 96, 150]
    q, kc, vc, ls, scale = I.decode_inputs(3, 2 * G, 2, d, 1, 256, 256, "bf16", seed=5, seqlens=lens)
    # sequence 1 and 2 reuse sequence 0's first three pages (keys 0..95)
    for b in (1, 2):
        kc[b, :, :96] = kc[0, :, :96]
        vc[b, :, :96] = vc[0, :, :96]
    kp, vp, table, _ = I.paged_cache(kc, vc, ls, page, seed=1)
    table[1, :3] = table[0, :3]
    table[2, :3] = table[0, :3]
    o = run_paged(q, kp, vp, table, ls, scale)
    ro, _ = oracle.decode_paged(q, kp, vp, table, ls, scale)
    check_bf16(o, ro, "shared-prefix paged decode")


def test_paged_ids_outside_pool_are_clamped():
    """Ids outside [0, num_pages) are clamped into the pool (a caller error that
    must never become an out-of-bounds read)."""
    d, page = 64, 16
    lens = [40, 33]
    q, kc, vc, ls, scale = I.decode_inputs(2, 2, 1, d, 1, 48, 48, "bf16", seed=7, seqlens=lens)
    kp, vp, table, num_pages = I.paged_cache(kc, vc, ls, page, seed=3, spare_pages=1)
    kp[torch.isnan(kp)] = 0  # whichever page a clamped id lands on holds finite data
    vp[torch.isnan(vp)] = 0
    table[0, 1] = -5
    table[1, 2] = num_pages + 100
    o = run_paged(q, kp, vp, table, ls, scale)
    ro, _ = oracle.decode_paged(q, kp, vp, table.clamp(0, num_pages - 1), ls, scale)
    check_bf16(o, ro, "clamped-id paged decode")


@pytest.mark.parametrize("page", [16, 64])
def test_paged_decode_workload(page):
    """The B64 Hq32 Hkv8 d128 decode workload (4096-key chunks) in 16- and
    64-key pages -- 16-key pages give the most page ids per chunk: bit-identical
    to contiguous decode, and against the oracle on sampled sequences."""
    cfg = I.DECODE_GQA
    q, kc, vc, ls, scale = I.decode_config_inputs(cfg)
    kcd, vcd = kc.to("cuda"), vc.to("cuda")
    kp, vp, table, _ = I.paged_cache(kcd, vcd, ls, page, seed=11)
    qd, ld, td = q.to("cuda"), ls.to("cuda"), table.to("cuda")
    o = decode_paged(qd, kp, vp, td, ld, scale=scale)
    oc = decode(qd, kcd, vcd, ld, scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(o, oc)
    for b in (0, 17, 63):
        ro, _ = oracle.decode(q[b:b + 1], kc[b:b + 1], vc[b:b + 1], ls[b:b + 1], scale)
        check_bf16(o[b:b + 1].cpu(), ro, f"paged workload sequence {b}")
