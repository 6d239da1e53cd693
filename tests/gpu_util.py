"""Helpers shared by the GPU parity tests (comparison and tolerances)."""

import os

import numpy as np
import torch

# Tolerances against the fp64 oracle on the same (bf16-rounded) inputs.
BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3
BF16_LSE_MAX_ABS = 1e-3
F32_MAX_ABS = 1e-5
F32_LSE_MAX_ABS = 1e-5


def gpu_available():
    return torch.cuda.is_available()


def to_dev(*ts):
    return [t.to("cuda") for t in ts]


def f64(t):
    return t.detach().to("cpu").double().numpy()


def check_bf16(o_gpu, o_ref, what):
    err = np.abs(f64(o_gpu) - o_ref)
    assert np.isfinite(err).all(), f"{what}: non-finite output"
    mx, mean = err.max(), err.mean()
    assert mx <= BF16_MAX_ABS, f"{what}: max-abs {mx:.3e} > {BF16_MAX_ABS}"
    assert mean <= BF16_MEAN_ABS, f"{what}: mean-abs {mean:.3e} > {BF16_MEAN_ABS}"
    return mx, mean


# bf16 paths, per output element, from their arithmetic: P is rounded to bf16
# before P.V (at most 2^-8 of each term, so at most 2^-8 * a on an element,
# with a = sum_j p_j |v_j| / l, the attention output of |V|), and the output
# is rounded to bf16 (at most 2^-8 |o|); another 2^-10 (|o| + a) and 1e-5 cover
# the fp32 arithmetic around them.  For the flat softmaxes of the named
# workloads this is tighter than BF16_MAX_ABS on most elements; it is looser
# only where a sharp softmax meets |v| of about 4.
BF16_ELEMENT_REL = 2.0 ** -8 + 2.0 ** -10


def check_bf16_elementwise(o_gpu, o_ref, a_ref, what):
    err = np.abs(f64(o_gpu) - o_ref)
    assert np.isfinite(err).all(), f"{what}: non-finite output"
    bound = BF16_ELEMENT_REL * (np.abs(o_ref) + a_ref) + 1e-5
    ratio = err / bound
    worst = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
    assert ratio[worst] <= 1.0, (f"{what}: element {tuple(int(i) for i in worst)} error {err[worst]:.3e} > "
                                 f"bound {bound[worst]:.3e} (|o| {abs(o_ref[worst]):.3e}, a {a_ref[worst]:.3e})")
    mean = err.mean()
    assert mean <= BF16_MEAN_ABS, f"{what}: mean-abs {mean:.3e} > {BF16_MEAN_ABS}"
    return err.max(), mean


def check_close(x_gpu, ref, tol, what):
    err = np.abs(f64(x_gpu) - ref)
    assert np.isfinite(err).all(), f"{what}: non-finite output"
    mx = err.max()
    assert mx <= tol, f"{what}: max-abs {mx:.3e} > {tol}"
    return mx


def oracle_rows_parallel(q, k, v, causal, scale, rows, heads, threads=16):
    """oracle.attention_rows over many heads, one head per task on a thread
    pool (numpy's matrix products and ufuncs release the GIL; BLAS is held to
    one thread per task).  Returns (o [len(heads), len(rows), d], lse)."""
    import concurrent.futures

    from threadpoolctl import threadpool_limits

    import oracle

    threads = max(1, min(threads, len(os.sched_getaffinity(0)), len(heads)))
    with threadpool_limits(limits=1):
        with concurrent.futures.ThreadPoolExecutor(threads) as ex:
            parts = list(ex.map(lambda bh: oracle.attention_rows(q, k, v, causal, scale, rows, [bh]), heads))
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])


def boundary_rows(n, extra=16, seed=0):
    """Query rows where a tiled causal kernel changes behaviour, for sampled
    checks at large N: the first and last rows of the first and last query
    tiles (both wave widths interleave rows over 4 or 8 waves), the edges of
    64-key tiles and 128/256-row query tiles at the start, at the causal
    pairing's mirror point (the middle) and at the end, rows next to powers of
    two, plus `extra` seeded uniform rows.  Sorted, unique."""
    from exact_tiled_attention_prefill_amd.inputs import sample_rows

    rows = set(range(min(n, 9))) | set(range(max(0, n - 9), n))
    for t in (64, 128, 256):
        for base in (t, 2 * t, (n // t // 2) * t, (n // t - 1) * t):
            rows.update(r for r in (base - 1, base, base + 1) if 0 <= r < n)
    rows.update(sample_rows(n, 0, seed))
    gen = torch.Generator().manual_seed(seed + 4321)
    rows.update(torch.randint(0, n, (extra,), generator=gen).tolist())
    return sorted(rows)


def check_causal_invariants(qd, kd, vd, od, lsed, scale, what):
    """Properties of dense causal attention checked on EVERY row (device
    tensors q [B,Hq,N,d], k/v [B,Hkv,N,d], o, lse [B,Hq,N]):
    * row 0 sees only key 0: o = V[0] bit for bit;
    * convex hull: each o[i, c] lies between the min and max of V[0..i, c]
      (slack: bf16 rounding of the probabilities (a weight sum within 2^-9
      of 1) and of the output, taken at 2^-8);
    * lse bounds: scale q_i.k_i <= max_j s_ij <= lse_i <= max_j s_ij + ln(i+1)
      <= |scale| |q_i| max_{j<=i} |k_j| + ln(i+1), within the 1e-3 lse bar.
    """
    B, Hq, N, d = qd.shape
    G = Hq // kd.shape[1]
    ln = torch.log(torch.arange(1, N + 1, device=qd.device, dtype=torch.float32))
    for b in range(B):
        for g in range(kd.shape[1]):
            vf = vd[b, g].float()
            vmax = torch.cummax(vf, dim=0).values
            vmin = torch.cummin(vf, dim=0).values
            vabs = torch.maximum(vmax.abs(), vmin.abs())
            kf = kd[b, g].float()
            kmax = torch.cummax(kf.norm(dim=1), dim=0).values
            for h in range(g * G, (g + 1) * G):
                assert torch.equal(od[b, h, 0], vd[b, g, 0]), f"{what}: row 0 of head {(b, h)} is not V[0]"
                of = od[b, h].float()
                slack = (vabs + of.abs()) * 2.0 ** -8 + 1e-6
                assert bool((of >= vmin - slack).all()), f"{what}: head {(b, h)} below the hull"
                assert bool((of <= vmax + slack).all()), f"{what}: head {(b, h)} above the hull"
                qf = qd[b, h].float()
                lse = lsed[b, h]
                assert bool(torch.isfinite(lse).all()), f"{what}: non-finite lse in head {(b, h)}"
                diag = scale * (qf * kf).sum(dim=1)
                upper = abs(scale) * qf.norm(dim=1) * kmax + ln
                assert bool((lse >= diag - BF16_LSE_MAX_ABS).all()), f"{what}: lse below the diagonal score"
                assert bool((lse <= upper + BF16_LSE_MAX_ABS).all()), f"{what}: lse above its bound"
    torch.cuda.synchronize()
