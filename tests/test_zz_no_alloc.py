"""fa_decode_noalloc (the allocation-free decode entry point) through the C ABI.

Its kernels are fa_decode_ws's, with the split-KV partials in the library's
fixed per-GPU array instead of a caller workspace, so the outputs must be
bit-identical to fa_decode_ws on the same inputs -- and within the bf16 bar of
the fp64 oracle.  Two calls in a row, the second smaller, show that what the
first left in the array does not leak into the second.  Sizes beyond the
array are refused before any HIP call.
"""

import numpy as np
import pytest
import torch

import oracle
from exact_tiled_attention_prefill_amd import binding, decode, decode_noalloc, decode_workspace_bytes
from exact_tiled_attention_prefill_amd import inputs as I
from gpu_util import check_bf16, to_dev

pytestmark = pytest.mark.gpu


def _both(q, kc, vc, ls, scale):
    qd, kd, vd, ld = to_dev(q, kc, vc, ls)
    B, Hq, d = q.shape
    ws = torch.empty(decode_workspace_bytes(B, Hq, kc.shape[1], kc.shape[2], d), dtype=torch.uint8, device="cuda")
    ref = decode(qd, kd, vd, ld, scale=scale, workspace=ws)
    got = decode_noalloc(qd, kd, vd, ld, scale=scale)
    torch.cuda.synchronize()
    return got.cpu(), ref.cpu()


def test_noalloc_matches_workspace_decode_on_two_calls():
    print("noalloc: GQA decode B64 Hq32 Hkv8 d128, lengths 1024..32768", flush=True)
    cfg = I.DECODE_GQA
    q, kc, vc, ls, scale = I.decode_config_inputs(cfg)
    got, ref = _both(q, kc, vc, ls, scale)
    assert torch.equal(got, ref)
    for b in (0, 31, 63):
        ro, _ = oracle.decode(q[b:b + 1], kc[b:b + 1], vc[b:b + 1], ls[b:b + 1], scale)
        check_bf16(got[b:b + 1], ro, f"noalloc sequence {b}")
    del kc, vc

    print("noalloc: second, smaller call B4 Hq8 Hkv2 d64", flush=True)
    lens = [0, 1, 700, 2049]
    q, kc, vc, ls, scale = I.decode_inputs(len(lens), 8, 2, 64, 1, 2049, 2049, "bf16", seed=21, seqlens=lens)
    got, ref = _both(q, kc, vc, ls, scale)
    assert torch.equal(got, ref)
    ro, _ = oracle.decode(q, kc, vc, ls, scale)
    check_bf16(got, ro, "noalloc small")
    assert torch.all(got[0] == 0)


def test_noalloc_refuses_sizes_beyond_its_array():
    """B 4096 x Hq 64 x maxlen 65536 needs far more than the fixed array: the
    call returns FA_ERR_TOO_LARGE before touching the device (the pointers
    are never dereferenced)."""
    lib = binding.load_library()
    p = torch.empty(16, dtype=torch.bfloat16, device="cuda")
    sl = torch.zeros(4096, dtype=torch.int32, device="cuda")
    st = lib.fa_decode_noalloc(p.data_ptr(), p.data_ptr(), p.data_ptr(), sl.data_ptr(), p.data_ptr(), 4096, 64, 8,
                               65536, 128, 0.088, None)
    assert st == binding.FA_ERR_TOO_LARGE
