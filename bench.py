#!/usr/bin/env python3
"""Benchmark of the exact-attention hot path on one MI355X.

One step = one fa_prefill call on the long-context causal GQA workload
(B1 Hq64 Hkv8 N131072 d128 bf16) followed by one fa_decode call on the GQA
decode workload (B64 Hq32 Hkv8 d128 bf16, cache lengths uniform in
[1024, 32768]): the prefill covers the tiled score / mask / running-softmax /
value steps, the decode the split-KV read of a cache and its log-sum-exp
combine.  `value` is the prefill's TFLOP/s (algorithmic FLOPs =
4*d*B*Hq*N(N+1)/2 over the prefill kernel's own HIP-event time).

After the timed steps, the other workloads are timed as legs with their own
step counts: causal MHA B4 H32 N4096, causal GQA B2 Hq32 Hkv8 N16384, decode
against the same caches in 64-key pages of a shuffled pool, a packed
4096-query chunk against a 16384-key prefix, the MHA 4K workload with a
1024-key window, and the MHA 4K backward.  Inputs are seeded synthetic
tensors already resident in HBM before timing starts; kernel durations come
from HIP events recorded on the stream the kernels are launched on.

The fp64 CPU oracle runs on the host in a pool of worker processes (started
before anything touches the GPU): on sampled rows of every head of the 128K
workload (timed: that is `cpu_baseline`), on every row of the 16K and 4K
workloads; each compares its rows with the GPU's output of the timed runs
(`parity`).  The device's sustained MFMA and HBM-read rates are measured
after the timed region.

Prints ONE JSON line.  --gpus N with N > 1 exits: the kernels run on one GPU.
"""

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA (256 CU x 4096 FLOP/clk x 2.4 GHz)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_FP64_VALU_TFLOPS = 78.6  # MI355X fp64 vector: 256 CU x 4 SIMD x 16 lanes x 2 FLOP (FMA) x 2.4 GHz
# Performance goals, as fractions of those peaks: compute-bound prefill at
# least half the dense bf16 matrix rate, bandwidth-bound decode at least 70%
# of HBM bandwidth.  Each leg reports its goal and whether it was met; the
# backward has no stated goal.
GOAL_PREFILL_FRAC = 0.5
GOAL_DECODE_FRAC = 0.7
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "exact_tiled_attention_prefill_amd", "csrc")
PREFILL_SRC = os.path.join(CSRC, "prefill_bf16.hip")
DECODE_SRC = os.path.join(CSRC, "decode.hip")
BACKWARD_SRC = os.path.join(CSRC, "backward_bf16.hip")
BAR = {"o_max_abs": 2e-2, "o_mean_abs": 2e-3, "lse_max_abs": 1e-3}
# backward: the forward's bf16 bar scaled to each gradient's range s = max(1, max|ref|)
F32_BAR = {"o_max_abs": 1e-5, "lse_max_abs": 1e-5}
BWD_BAR = {"max_abs_over_range": 2e-2, "mean_abs_over_range": 2e-3}
PREFILL_KERNEL = "prefill_bf16_kernel<128, causal> (4 or 8 waves per workgroup, as the launcher picks)"


def prefill_flops(B, Hq, N, d, causal):
    pairs = N * (N + 1) // 2 if causal else N * N
    return 4 * d * B * Hq * pairs


def varlen_pairs(lens, causal, window):
    """Visible (query, key) pairs of packed sequences [(n_q, n_k), ...]."""
    total = 0
    for nq, nk in lens:
        off = nk - nq
        for i in range(nq):
            hi = min(i + off, nk - 1) if causal else nk - 1
            lo = max(0, i + off - window) if window >= 0 else 0
            total += max(hi - lo + 1, 0)
    return total


def prefill_bytes(B, Hq, Hkv, N, d, elem=2):
    return (2 * B * Hq * N * d + 2 * B * Hkv * N * d) * elem + B * Hq * N * 4


def decode_bytes(lens, Hq, Hkv, d, elem=2):
    kv = sum(int(x) for x in lens) * Hkv * d * 2 * elem
    return kv + 2 * len(lens) * Hq * d * elem + 4 * len(lens)


def source_hash(path):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def _summary(name, src):
    """Text of profiles/<name>.md if its kernel_source_sha matches `src`."""
    path = os.path.join(PROFILES, name + ".md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    h = re.search(r"kernel_source_sha:\s*([0-9a-f]+)", text)
    if not h or h.group(1) != source_hash(src):
        return None
    return text


def measured_traffic(name, src):
    """HBM bytes per launch from a committed rocprofv3 counter summary.

    profiles/<name>.md carries `traffic_bytes_per_launch: <number>` and
    `kernel_source_sha: <hash>`; the figure is used only while the kernel
    source still has that hash (otherwise null: the counters are stale).
    """
    text = _summary(name, src)
    m = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text) if text else None
    return float(m.group(1)) if m else None


def measured_counters(name, src, keys):
    """Derived rocprofv3 counter figures (MFMA busy fraction, counted MFMA
    FLOPs over algorithmic FLOPs, clock, HBM rate) from a committed summary,
    used only while the kernel source still has the summary's hash."""
    text = _summary(name, src)
    if text is None:
        return None
    out = {}
    for key in keys:
        m = re.search(key + r":\s*([0-9.eE+-]+)", text)
        if m:
            out[key] = float(m.group(1))
    return out or None


def measured_ceilings():
    """Sustained MFMA and HBM-read rates of this device from libfa_probes.so.

    Context only: the roofline fractions are against the published peaks.
    Under dense MFMA load on random operands the part is power-limited, so the
    matrix cores sustain less than the nominal rate; HBM's practical read rate
    is likewise below 8 TB/s.  Returns None if the probe library is absent.
    """
    import ctypes

    path = os.path.join(ROOT, "exact_tiled_attention_prefill_amd", "libfa_probes.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.fa_probe_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_double),
                                       ctypes.POINTER(ctypes.c_double)]
    lib.fa_probe_mfma_bf16.restype = ctypes.c_int
    lib.fa_probe_hbm_read_hint.argtypes = [ctypes.c_size_t, ctypes.c_int, ctypes.c_int,
                                           ctypes.POINTER(ctypes.c_double)]
    lib.fa_probe_hbm_read_hint.restype = ctypes.c_int
    out = {}
    for name, zero in (("mfma_bf16_random_operands", 0), ("mfma_bf16_zero_operands", 1)):
        tf, ghz = ctypes.c_double(), ctypes.c_double()
        if lib.fa_probe_mfma_bf16(zero, 20000, ctypes.byref(tf), ctypes.byref(ghz)) != 0:
            return None
        out[name] = {"tflops": tf.value, "shader_clock_ghz": ghz.value}
    reads = {}
    for name, nt in (("plain", 0), ("nontemporal", 1)):
        gbs = ctypes.c_double()
        if lib.fa_probe_hbm_read_hint(4 << 30, 5, nt, ctypes.byref(gbs)) != 0:
            return None
        reads[name] = gbs.value
    out["hbm_read_gbs"] = max(reads.values())
    out["hbm_read_gbs_by_hint"] = reads
    out["note"] = ("context only, not a roofline: whole-chip sustained v_mfma_f32_32x32x16_bf16 rate (two "
                   "waves per SIMD, operands in registers) and a 4 GiB read-only stream with 16-byte loads, "
                   "with and without the non-temporal hint (hbm_read_gbs is the faster)")
    return out


def device_memory(fn, io, workspace, n_by_n):
    """Device bytes around one call: the call's inputs and outputs, the
    caller-owned workspace it is given, torch's peak over the call (the
    library allocates nothing of its own on these paths), and what an N x N
    fp32 score buffer would take."""
    import torch

    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    before = torch.cuda.memory_allocated()
    fn()
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated()
    io_bytes = sum(t.numel() * t.element_size() for t in io)
    return {"io_bytes": io_bytes, "workspace_bytes": workspace, "allocated_before_call": before,
            "peak_during_call": peak, "extra_over_call": peak - before, "n_by_n_fp32_scores_bytes": n_by_n,
            "call_allocates_nothing": peak == before}


# ---------------------------------------------------------------- oracle pool
def _oracle_pool_init():
    """Process-pool worker start-up: one BLAS thread per worker process."""
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS", "BLIS_NUM_THREADS"):
        os.environ[var] = "1"


def _oracle_job(job):
    """Causal prefill rows of one KV group's query heads through the fp64
    oracle (run in a pool worker), and the GPU output's error on them.
    Tensors arrive as raw bf16 bits (uint16), lse as float32; q holds only the
    requested rows of each head."""
    import numpy as np

    import oracle

    n, rows, q_rows, kh, vh, o_rows, l_rows, scale = job
    bf16 = lambda a: (a.astype(np.uint32) << 16).view(np.float32)  # exact bf16 -> fp32
    d = kh.shape[1]
    k4, v4 = bf16(kh)[None, None], bf16(vh)[None, None]
    flops, emax, esum, count, lmax = 0, 0.0, 0.0, 0, 0.0
    q4 = np.zeros((1, 1, n, d), dtype=np.float32)
    for qh, oh, lh in zip(q_rows, o_rows, l_rows):
        q4[0, 0, rows] = bf16(qh)
        ro, rl = oracle.attention_rows(q4, k4, v4, True, scale, rows, [(0, 0)])
        e = np.abs(bf16(oh).astype(np.float64) - ro[0])
        el = np.abs(lh.astype(np.float64) - rl[0])
        flops += int(sum(4 * d * (int(r) + 1) for r in rows))
        emax, esum, count, lmax = max(emax, float(e.max())), esum + float(e.sum()), count + e.size, max(
            lmax, float(el.max()))
    return flops, emax, esum, count, lmax


def _oracle_f32_job(job):
    """A whole fp32 prefill through the fp64 oracle (run in a pool worker) and
    the GPU output's largest errors.  Tensors arrive as float32 arrays."""
    import numpy as np

    import oracle

    q, k, v, causal, scale, o, lse = job
    ro, rl = oracle.attention(q, k, v, causal, scale)
    return float(np.abs(o.astype(np.float64) - ro).max()), float(np.abs(lse.astype(np.float64) - rl).max())


def oracle_f32_check(pool, q, k, v, causal, scale, o_gpu, lse_gpu):
    """Compare every element of an fp32 prefill with the oracle (one job)."""
    t0 = time.perf_counter()
    eo, el = pool.apply(_oracle_f32_job, ((q.numpy(), k.numpy(), v.numpy(), causal, scale, o_gpu.numpy(),
                                           lse_gpu.numpy()),))
    err = {"o_max_abs": eo, "lse_max_abs": el}
    err["within_bar"] = all(err[key] <= F32_BAR[key] for key in F32_BAR)
    return err, time.perf_counter() - t0


def _oracle_bwd_job(job):
    """One head's dq, dk, dv through the fp64 oracle's backward (run in a pool
    worker) and the GPU gradients' errors, each over the gradient's range
    s = max(1, max|ref|).  Tensors arrive as raw bf16 bits (uint16)."""
    import numpy as np

    import oracle

    qh, kh, vh, doh, grads, scale = job
    bf16 = lambda a: (a.astype(np.uint32) << 16).view(np.float32)[None, None]  # exact bf16 -> fp32
    refs = oracle.attention_backward(bf16(qh), bf16(kh), bf16(vh), bf16(doh), True, scale)
    out = []
    for g, r in zip(grads, refs):
        e = np.abs(bf16(g).astype(np.float64) - r)
        s = max(1.0, float(np.abs(r).max()))
        out.append((float(e.max()) / s, float(e.mean()) / s))
    return out


def _oracle_varlen_job(job):
    """One packed sequence and query head through the fp64 oracle's
    attention_varlen (run in a pool worker), and the GPU output's error on its
    rows.  Tensors arrive as raw bf16 bits (uint16), lse as float32."""
    import numpy as np

    import oracle

    qh, kh, vh, causal, window, oh, lh, scale = job
    bf16 = lambda a: (a.astype(np.uint32) << 16).view(np.float32)  # exact bf16 -> fp32
    n_q, n_k = qh.shape[0], kh.shape[0]
    ro, rl = oracle.attention_varlen(bf16(qh)[:, None], bf16(kh)[:, None], bf16(vh)[:, None], [0, n_q], [0, n_k],
                                     causal, scale, window_left=window)
    e = np.abs(bf16(oh).astype(np.float64) - ro[:, 0])
    el = np.abs(lh.astype(np.float64) - rl[0])
    return float(e.max()), float(e.sum()), e.size, float(el.max())


def oracle_varlen_check(pool, q, k, v, cu_q, cu_k, causal, window, scale, o_gpu, lse_gpu):
    """Compare every row of every head of a packed prefill with the oracle,
    one (sequence, head) per job."""
    import torch

    hq, hkv = q.shape[1], k.shape[1]
    G = hq // hkv
    bits = lambda t: t.contiguous().view(torch.int16).numpy().view("uint16")
    cq, ck = cu_q.tolist(), cu_k.tolist()

    def jobs():
        for b in range(len(cq) - 1):
            for h in range(hq):
                yield (bits(q[cq[b]:cq[b + 1], h]), bits(k[ck[b]:ck[b + 1], h // G]),
                       bits(v[ck[b]:ck[b + 1], h // G]), causal, window, bits(o_gpu[cq[b]:cq[b + 1], h]),
                       lse_gpu[h, cq[b]:cq[b + 1]].numpy(), scale)

    t0 = time.perf_counter()
    res = list(pool.imap_unordered(_oracle_varlen_job, jobs(), chunksize=1))
    dt = time.perf_counter() - t0
    count = sum(r[2] for r in res)
    err = {"o_max_abs": max(r[0] for r in res), "o_mean_abs": sum(r[1] for r in res) / count,
           "lse_max_abs": max(r[3] for r in res)}
    err["within_bar"] = all(err[key] <= BAR[key] for key in BAR)
    return err, dt


def _oracle_decode_job(job):
    """One decode sequence (all query heads) through the fp64 oracle (run in a
    pool worker), and the errors of the GPU outputs given for it."""
    import numpy as np

    import oracle

    qb, kb, vb, n, outs, scale = job
    bf16 = lambda a: (a.astype(np.uint32) << 16).view(np.float32)  # exact bf16 -> fp32
    ro, _ = oracle.decode(bf16(qb)[None], bf16(kb)[None], bf16(vb)[None], np.array([n]), scale)
    res = []
    for ob in outs:
        e = np.abs(bf16(ob).astype(np.float64) - ro[0])
        res.append((float(e.max()), float(e.sum()), e.size))
    return res


def oracle_decode_check(pool, q, kcache_dev, vcache_dev, lens, scale, outs, seqs):
    """Compare the GPU decode outputs `outs` (name -> [B,Hq,d] host tensor) on
    the sequences `seqs` with the oracle; the cache rows of each sequence are
    copied from the device as its job is made."""
    import torch

    bits = lambda t: t.contiguous().view(torch.int16).numpy().view("uint16")
    names = list(outs)

    def jobs():
        for b in seqs:
            n = int(lens[b])
            yield (bits(q[b]), bits(kcache_dev[b, :, :n].cpu()), bits(vcache_dev[b, :, :n].cpu()), n,
                   [bits(outs[name][b]) for name in names], scale)

    t0 = time.perf_counter()
    res = list(pool.imap_unordered(_oracle_decode_job, jobs(), chunksize=1))
    dt = time.perf_counter() - t0
    out = {}
    for i, name in enumerate(names):
        count = sum(r[i][2] for r in res)
        err = {"o_max_abs": max(r[i][0] for r in res), "o_mean_abs": sum(r[i][1] for r in res) / count}
        err["within_bar"] = err["o_max_abs"] <= BAR["o_max_abs"] and err["o_mean_abs"] <= BAR["o_mean_abs"]
        out[name] = err
    return out, dt


def decode_sample_sequences(lens, count=16, seed=4):
    """The two shortest and two longest decode sequences and seeded others, `count` in all."""
    import torch

    order = sorted(range(len(lens)), key=lambda b: lens[b])
    seqs = set(order[:2] + order[-2:])
    gen = torch.Generator().manual_seed(seed)
    for b in torch.randperm(len(lens), generator=gen).tolist():
        if len(seqs) >= min(count, len(lens)):
            break
        seqs.add(b)
    return sorted(seqs)


def oracle_backward_check(pool, q, k, v, do, scale, grads_gpu):
    """Compare the GPU backward of every (batch, head) of an MHA causal
    workload with the oracle.  Returns the worst ratios per gradient."""
    import torch

    B, Hq = q.shape[:2]
    assert k.shape[1] == Hq, "one head per job needs MHA (each head's gradients depend on it alone)"
    bits = lambda t: t.contiguous().view(torch.int16).numpy().view("uint16")
    jobs = ((bits(q[b, h]), bits(k[b, h]), bits(v[b, h]), bits(do[b, h]), [bits(g[b, h]) for g in grads_gpu],
             scale) for b in range(B) for h in range(Hq))
    t0 = time.perf_counter()
    res = list(pool.imap_unordered(_oracle_bwd_job, jobs, chunksize=1))
    dt = time.perf_counter() - t0
    err = {}
    for i, name in enumerate(("dq", "dk", "dv")):
        err[name] = {"max_abs_over_range": max(r[i][0] for r in res),
                     "mean_abs_over_range": max(r[i][1] for r in res)}
    err["within_bar"] = all(err[n][key] <= BWD_BAR[key] for n in ("dq", "dk", "dv") for key in BWD_BAR)
    return err, dt


def oracle_check(pool, q, k, v, scale, o_gpu, lse_gpu, rows, heads_per_job):
    """Compare the GPU output at `rows` of every (batch, head) with the oracle,
    jobs of `heads_per_job` query heads of one KV group.  Returns the error
    summary, the algorithmic FLOPs evaluated and the wall time."""
    import numpy as np
    import torch

    B, Hq, N, d = q.shape
    G = Hq // k.shape[1]
    rows = np.asarray(rows, dtype=np.int64)
    idx = torch.as_tensor(rows)
    bits = lambda t: t.contiguous().view(torch.int16).numpy().view("uint16")

    def jobs():
        for b in range(B):
            for h0 in range(0, Hq, heads_per_job):
                hs = range(h0, min(h0 + heads_per_job, Hq))
                g = h0 // G
                assert all(h // G == g for h in hs)
                yield (N, rows, [bits(q[b, h][idx]) for h in hs], bits(k[b, g]), bits(v[b, g]),
                       [bits(o_gpu[b, h][idx]) for h in hs], [lse_gpu[b, h][idx].numpy() for h in hs], scale)

    t0 = time.perf_counter()
    res = list(pool.imap_unordered(_oracle_job, jobs(), chunksize=1))
    dt = time.perf_counter() - t0
    count = sum(r[3] for r in res)
    err = {"o_max_abs": max(r[1] for r in res), "o_mean_abs": sum(r[2] for r in res) / count,
           "lse_max_abs": max(r[4] for r in res)}
    err["within_bar"] = all(err[key] <= BAR[key] for key in BAR)
    return err, sum(r[0] for r in res), dt


def c5_sample_rows(n, count=2048, seed=3):
    """Rows of the 128K workload the oracle evaluates on every head: the
    first and last rows, multiples of 64 +- 1 in the first 1024 rows, rows
    next to powers of two, and seeded uniform rows up to `count`."""
    import torch

    rows = {0, 1, 2, 3, n - 2, n - 1}
    for m in range(64, 1025, 64):
        rows.update((m - 1, m, m + 1))
    p = 1
    while p < n:
        rows.update(r for r in (p - 1, p, p + 1) if 0 <= r < n)
        p *= 2
    gen = torch.Generator().manual_seed(seed)
    for r in torch.randint(0, n, (4 * count,), generator=gen).tolist():
        if len(rows) >= count:
            break
        rows.add(int(r))
    return sorted(rows)


# ---------------------------------------------------------------- timing
def time_calls(fn, stream, steps):
    """HIP-event times (ms) of `steps` back-to-back calls on `stream`."""
    import torch

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for e0, e1 in evs:
        e0.record(stream)
        fn()
        e1.record(stream)
    torch.cuda.synchronize()
    return sorted(e0.elapsed_time(e1) for e0, e1 in evs)


def warm(fn, calls, seconds=0.2):
    """Untimed warm-up: at least `calls` calls and `seconds` of wall time, so
    that the GPU's clocks have left their idle state before timing starts."""
    import torch

    t0, n = time.perf_counter(), 0
    while n < calls or time.perf_counter() - t0 < seconds:
        fn()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def stats(ms):
    k = len(ms)
    return {"ms_avg": sum(ms) / k, "ms_median": ms[k // 2], "ms_min": ms[0], "launches": k}


def with_goal(rl, goal):
    rl["goal_frac"] = goal
    rl["goal_met"] = None if goal is None else bool(rl["frac"] >= goal)
    return rl


def mfma_roofline(kernel, tflops, counters_name=None, src=PREFILL_SRC, algorithmic_bytes=None,
                  goal=GOAL_PREFILL_FRAC):
    rl = with_goal({"kernel": kernel, "bound": "mfma", "achieved": tflops, "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": tflops / PEAK_BF16_TFLOPS, "traffic": None}, goal)
    if algorithmic_bytes is not None:
        rl["algorithmic_bytes"] = algorithmic_bytes
    if counters_name is not None:
        rl["traffic"] = measured_traffic(counters_name, src)
        rl["rocprof"] = measured_counters(counters_name, src, ("mfma_busy_fraction", "mfma_flops_over_algorithmic",
                                                               "shader_clock_ghz", "traffic_over_algorithmic"))
    return rl


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle (cpu_baseline and the parity of the timed outputs)")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the MFMA / HBM ceiling probes")
    ap.add_argument("--no-legs", action="store_true", help="time only the step (128K prefill + decode)")
    ap.add_argument("--page-size", type=int, default=64, help="page size of the paged-decode leg")
    ap.add_argument("--only", choices=["step", "prefill_gqa_128k", "decode", "prefill_mha_4k", "prefill_gqa_16k",
                                       "decode_paged", "prefill_chunked", "prefill_window", "prefill_f32_small", "backward",
                                       "copy",
                                       "ceiling"],
                    default=None,
                    help="run one kernel only (for profiler runs); 'step' runs the 128K prefill and the decode; "
                         "'copy' runs a plain 1 GiB device copy used to calibrate the HBM byte counters; "
                         "'ceiling' runs only the MFMA / HBM ceiling probes")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); nothing to do for N > 1.",
              file=sys.stderr)
        sys.exit(2)
    only = args.only
    want = lambda name: only is None or only == name or (only == "step" and name in ("prefill_gqa_128k", "decode"))
    run_legs = only is not None or not args.no_legs
    leg = lambda name: want(name) and run_legs

    # The oracle's worker processes start before anything touches the GPU (a
    # process that has initialised the GPU does not start new programs).
    pool, workers = None, 0
    if only is None and not args.no_cpu_baseline:
        import multiprocessing

        workers = max(1, min(16, len(os.sched_getaffinity(0))))
        pool = multiprocessing.get_context("spawn").Pool(workers, initializer=_oracle_pool_init)

    import torch

    from exact_tiled_attention_prefill_amd import (decode, decode_paged, decode_paged_workspace_bytes,
                                                   decode_workspace_bytes, load_library, prefill, prefill_backward,
                                                   prefill_backward_workspace_bytes, prefill_varlen)
    from exact_tiled_attention_prefill_amd import inputs as I

    load_library()  # fail loudly before any work if libfa.so is missing
    dev = torch.device("cuda:0")
    if only == "ceiling":
        print(json.dumps({"ceilings": measured_ceilings()}), flush=True)
        return
    if only == "copy":
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(args.warmup + args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": 1 << 30, "launches": args.warmup + args.steps}))
        return
    stream = torch.cuda.current_stream()
    K = args.steps
    result = {
        "metric": "prefill attention TFLOP/s (% bf16 MFMA peak); decode KV-read GB/s (% HBM)",
        "value": None, "unit": "TFLOP/s", "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": None,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) rounded to bf16)",
    }
    host = {}  # CPU copies of inputs and GPU outputs for the oracle

    def prefill_setup(cfg):
        q, k, v, scale = I.prefill_config_inputs(cfg)
        qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
        od = torch.empty_like(qd)
        ld = torch.empty((cfg.B, cfg.Hq, cfg.N), dtype=torch.float32, device=dev)

        def fn():
            prefill(qd, kd, vd, causal=cfg.causal, scale=scale, out=od, lse=ld)
        mem = device_memory(fn, [qd, kd, vd, od, ld], 0, cfg.B * cfg.Hq * cfg.N * cfg.N * 4)
        return (q, k, v, scale), fn, od, ld, mem

    def prefill_record(cfg, ms, mem, counters):
        F = prefill_flops(cfg.B, cfg.Hq, cfg.N, cfg.d, cfg.causal)
        st = stats(ms)
        tf = F / (st["ms_avg"] * 1e-3) / 1e12
        return dict(workload=cfg.name, **st, tflops=tf, tokens_per_s=cfg.B * cfg.N / (st["ms_avg"] * 1e-3),
                    frac_of_peak=tf / PEAK_BF16_TFLOPS, flops_per_launch=F, device_memory=mem,
                    roofline=mfma_roofline(PREFILL_KERNEL, tf, counters,
                                           algorithmic_bytes=prefill_bytes(cfg.B, cfg.Hq, cfg.Hkv, cfg.N, cfg.d)))

    pc, dc = I.PREFILL_GQA_128K, I.DECODE_GQA
    run_p, run_d = want("prefill_gqa_128k"), want("decode")
    if run_d or leg("decode_paged"):
        dq, dk, dv, dl, dscale = I.decode_config_inputs(dc)
        lens_host = dl.tolist()
        dqd, dkd, dvd, dld = dq.to(dev), dk.to(dev), dv.to(dev), dl.to(dev)
        del dk, dv
        dod = torch.empty_like(dqd)
    # ------------------------------------------------ legs, timed before the step: after seconds of
    # sustained 128K prefill the part runs hot and clocks lower, which would
    # penalise the short legs
    legs_steps = max(1, K)
    for name, cfg, counters, steps in (("prefill_mha_4k", I.PREFILL_MHA_4K, "prefill_bf16_mha4k_counters", legs_steps),
                                       ("prefill_gqa_16k", I.PREFILL_GQA_16K, "prefill_bf16_gqa16k_counters",
                                        max(1, min(K, 10)))):
        if not leg(name):
            continue
        host[name], fn, od, ld, mem = prefill_setup(cfg)
        warm(fn, args.warmup)
        result[name] = prefill_record(cfg, time_calls(fn, stream, steps), mem, counters)
        host[name + "_out"] = (od.cpu(), ld.cpu())
        del fn, od, ld
        torch.cuda.empty_cache()
        if result["value"] is None:
            result["value"] = result[name]["tflops"]

    if leg("decode_paged"):
        kpd, vpd, table, _ = I.paged_cache(dkd, dvd, dl, args.page_size, seed=11)
        tbd = table.to(dev)
        pws = torch.empty(decode_paged_workspace_bytes(dc.B, dc.Hq, dc.Hkv, args.page_size, table.shape[1], dc.d),
                          dtype=torch.uint8, device=dev)
        pgo = torch.empty_like(dqd)

        def pgf():
            decode_paged(dqd, kpd, vpd, tbd, dld, scale=dscale, out=pgo, workspace=pws)
        warm(pgf, args.warmup)
        st = stats(time_calls(pgf, stream, legs_steps))
        nbytes = decode_bytes(lens_host, dc.Hq, dc.Hkv, dc.d) + table.numel() * 4
        gbs = nbytes / (st["ms_avg"] * 1e-3) / 1e9
        result["decode_paged"] = dict(workload=dc.name + f"-paged{args.page_size}", page_size=args.page_size, **st,
                                      GB_per_s=gbs, frac_of_hbm_peak=gbs / PEAK_HBM_GBS, bytes_per_launch=nbytes,
                                      tokens_per_s=dc.B / (st["ms_avg"] * 1e-3),
                                      roofline=with_goal({
                                          "kernel": "decode_bf16_mfma_kernel<paged> + decode_combine_kernel",
                                          "bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                          "frac": gbs / PEAK_HBM_GBS,
                                          "traffic": measured_traffic("decode_paged_counters", DECODE_SRC)},
                                          GOAL_DECODE_FRAC))
        if pool is not None:
            host["decode_paged_out"] = pgo.cpu()
        del kpd, vpd, pws
        torch.cuda.empty_cache()
        if result["value"] is None:
            result["value"], result["unit"] = gbs, "GB/s"

    # packed variable-length legs: a 4096-query chunk against a 16384-key prefix
    # (GQA B2 Hq32 Hkv8 d128, causal bottom-right), and the MHA 4K workload
    # with a 1024-key causal window
    for name, lens, hq, hkv, causal, window in (("prefill_chunked", [(4096, 16384)] * 2, 32, 8, True, -1),
                                                ("prefill_window", [(4096, 4096)] * 4, 32, 32, True, 1024)):
        if not leg(name):
            continue
        vq, vk, vv, cq, ck, vscale = I.varlen_inputs(lens, hq, hkv, 128, seed=5)
        vqd, vkd, vvd, cqd, ckd = vq.to(dev), vk.to(dev), vv.to(dev), cq.to(dev), ck.to(dev)
        vod = torch.empty_like(vqd)
        vld = torch.empty((hq, vq.shape[0]), dtype=torch.float32, device=dev)
        mq = max(nq for nq, _ in lens)

        def vf():
            prefill_varlen(vqd, vkd, vvd, cqd, ckd, mq, causal=causal, window_left=window, scale=vscale, out=vod,
                           lse=vld)
        warm(vf, args.warmup)
        st = stats(time_calls(vf, stream, legs_steps))
        flops = 4 * 128 * hq * varlen_pairs(lens, causal, window)
        tf = flops / (st["ms_avg"] * 1e-3) / 1e12
        result[name] = dict(config={"sequences": [list(x) for x in lens], "Hq": hq, "Hkv": hkv, "d": 128,
                                    "causal": causal, "window_left": window}, **st, tflops=tf,
                            flops_per_launch=flops,
                            roofline=mfma_roofline("prefill_bf16_kernel<128, causal, varlen>", tf,
                                                   name.replace("prefill_", "prefill_bf16_") + "_counters"))
        if pool is not None:
            host[name] = (vq, vk, vv, cq, ck, causal, window, vscale)
            host[name + "_out"] = (vod.cpu(), vld.cpu())
        del vqd, vkd, vvd, vod, vld
        torch.cuda.empty_cache()
        if result["value"] is None:
            result["value"] = tf

    if leg("prefill_f32_small"):
        # the small fp32 workload: one head, 256 rows, d = 64, no mask
        fc = I.PREFILL_F32_SMALL
        fq, fk, fv, fscale = I.prefill_config_inputs(fc)
        fqd, fkd, fvd = fq.to(dev), fk.to(dev), fv.to(dev)
        fod = torch.empty_like(fqd)
        fld = torch.empty((fc.B, fc.Hq, fc.N), dtype=torch.float32, device=dev)

        def ff():
            prefill(fqd, fkd, fvd, causal=fc.causal, scale=fscale, out=fod, lse=fld)
        warm(ff, args.warmup)
        st = stats(time_calls(ff, stream, legs_steps))
        F = prefill_flops(fc.B, fc.Hq, fc.N, fc.d, fc.causal)
        tf = F / (st["ms_avg"] * 1e-3) / 1e12
        result["prefill_f32_small"] = dict(
            workload=fc.name, **st, tflops=tf, flops_per_launch=F, dtype="f32 in/out, f64 sums",
            roofline=with_goal({"kernel": "prefill_f32_kernel", "bound": "alu", "achieved": tf,
                                "peak": PEAK_FP64_VALU_TFLOPS, "unit": "TFLOP/s", "frac": tf / PEAK_FP64_VALU_TFLOPS,
                                "traffic": None,
                                "note": "fp64 FMAs for the dot products and sums; at this size the launch "
                                        "fills only a few of the 256 CUs"}, None))
        if pool is not None:
            host["prefill_f32_small"] = (fq, fk, fv, fc.causal, fscale)
            host["prefill_f32_small_out"] = (fod.cpu(), fld.cpu())
        del fqd, fkd, fvd, fod, fld

    if leg("backward"):
        # backward of the MHA 4K causal workload: the forward's o and lse feed it
        bc = I.PREFILL_MHA_4K
        bq, bk, bv, bdo, bscale = I.backward_inputs(bc.B, bc.Hq, bc.Hkv, bc.N, bc.d, seed=1)
        bqd, bkd, bvd, bdod = bq.to(dev), bk.to(dev), bv.to(dev), bdo.to(dev)
        bo, blse = prefill(bqd, bkd, bvd, causal=True, scale=bscale)
        bdq, bdk, bdv = torch.empty_like(bqd), torch.empty_like(bkd), torch.empty_like(bvd)
        bws = torch.empty(prefill_backward_workspace_bytes(bc.B, bc.Hq, bc.N), dtype=torch.uint8, device=dev)

        def bwf():
            prefill_backward(bqd, bkd, bvd, bo, bdod, blse, causal=True, scale=bscale, dq=bdq, dk=bdk, dv=bdv,
                             workspace=bws)
        warm(bwf, args.warmup)
        st = stats(time_calls(bwf, stream, legs_steps))
        flops = 2.5 * prefill_flops(bc.B, bc.Hq, bc.N, bc.d, True)
        tf = flops / (st["ms_avg"] * 1e-3) / 1e12
        result["backward"] = dict(config={"workload": bc.name, "flops": "2.5 x forward (five matrix products per "
                                                                        "score)",
                                          "kernels": "dQ (with the D and lse rows) + dK/dV"}, **st, tflops=tf,
                                  flops_per_launch=flops,
                                  roofline=mfma_roofline("bwd_dq_kernel + bwd_dkdv_kernel", tf, "backward_counters",
                                                         src=BACKWARD_SRC, goal=None))
        if result["value"] is None:
            result["value"] = tf
        if pool is not None:
            host["backward"] = (bq, bk, bv, bdo, bscale)
            host["backward_out"] = (bdq.cpu(), bdk.cpu(), bdv.cpu())
        del bqd, bkd, bvd, bdod, bo, blse, bdq, bdk, bdv, bws
        torch.cuda.empty_cache()

    # ------------------------------------------------ the step (timed last): 128K prefill + decode
    if run_p:
        host["c5"], pf, pod, pld, p_mem = prefill_setup(pc)
    if run_d:
        ws = torch.empty(decode_workspace_bytes(dc.B, dc.Hq, dc.Hkv, dc.maxlen, dc.d), dtype=torch.uint8,
                         device=dev)

        def df():
            decode(dqd, dkd, dvd, dld, scale=dscale, out=dod, workspace=ws)
        d_mem = device_memory(df, [dqd, dkd, dvd, dld, dod], ws.numel(), None)
    if run_p or run_d:
        for _ in range(args.warmup):
            if run_p:
                pf()
            if run_d:
                df()
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(K):
            ev[i][0].record(stream)
            if run_p:
                pf()
            ev[i][1].record(stream)
            if run_d:
                df()
            ev[i][2].record(stream)
        torch.cuda.synchronize()
        result["ms_per_step"] = (time.perf_counter() - t0) * 1e3 / K
        p_ms = sorted(ev[i][0].elapsed_time(ev[i][1]) for i in range(K))
        d_ms = sorted(ev[i][1].elapsed_time(ev[i][2]) for i in range(K))
        result["config"] = {"workload": pc.name if run_p else dc.name,
                            "step": "one prefill of this workload + one decode of decode.workload"}
        if run_p:
            rec = prefill_record(pc, p_ms, p_mem, "prefill_bf16_gqa128k_counters")
            result["value"] = rec["tflops"]
            result["config"].update({"B": pc.B, "Hq": pc.Hq, "Hkv": pc.Hkv, "N": pc.N, "d": pc.d,
                                     "causal": pc.causal})
            result["roofline"] = rec.pop("roofline")
            result["prefill"] = rec
            host["c5_out"] = (pod.cpu(), pld.cpu())
        if run_d:
            nbytes = decode_bytes(lens_host, dc.Hq, dc.Hkv, dc.d)
            st = stats(d_ms)
            gbs = nbytes / (st["ms_avg"] * 1e-3) / 1e9
            result["decode"] = dict(workload=dc.name, **st, GB_per_s=gbs, frac_of_hbm_peak=gbs / PEAK_HBM_GBS,
                                    bytes_per_launch=nbytes, tokens_per_s=dc.B / (st["ms_avg"] * 1e-3),
                                    device_memory=d_mem,
                                    roofline=with_goal({
                                        "kernel": "decode_bf16_mfma_kernel + decode_combine_kernel",
                                        "bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                        "frac": gbs / PEAK_HBM_GBS,
                                        "traffic": measured_traffic("decode_gqa_counters", DECODE_SRC),
                                        "rocprof": measured_counters("decode_gqa_counters", DECODE_SRC,
                                                                     ("hbm_gbs_counter_run", "shader_clock_ghz"))},
                                        GOAL_DECODE_FRAC))
            if result["value"] is None:
                result["value"], result["unit"] = gbs, "GB/s"
            if pool is not None:
                host["decode_out"] = dod.cpu()
        if run_p:
            del pf
            torch.cuda.empty_cache()

    props = torch.cuda.get_device_properties(dev)
    result["device"] = {"name": props.name, "cus": props.multi_processor_count,
                        "arch": getattr(props, "gcnArchName", ""), "torch": torch.__version__,
                        "hip": getattr(torch.version, "hip", None)}
    if only is None and not args.no_ceilings:
        result["ceilings"] = measured_ceilings()

    # ------------------------------------------------ oracle: cpu_baseline and parity of the timed outputs
    if pool is not None:
        parity = {}
        if "c5_out" in host:
            q, k, v, scale = host["c5"]
            rows = c5_sample_rows(pc.N)
            err, flops, dt = oracle_check(pool, q, k, v, scale, *host["c5_out"], rows, heads_per_job=4)
            rate = flops / dt
            full = prefill_flops(pc.B, pc.Hq, pc.N, pc.d, True)
            result["cpu_baseline"] = {
                "value": rate / 1e12, "unit": "TFLOP/s", "cores": workers, "kind": "oracle",
                "host_cpu_count": os.cpu_count(), "host_affinity_cores": len(os.sched_getaffinity(0)),
                "sample": f"{len(rows)} causal query rows (first/last rows, 64-multiples +-1 below 1024, powers of "
                          f"two +-1, seeded uniform rows) of each of the {pc.B * pc.Hq} heads of the {pc.name} "
                          f"workload, fp64 numpy oracle, {workers} worker processes with 1 BLAS thread each, "
                          f"{dt:.1f} s wall (inputs pickled to the workers inside the timed span); the rate is the "
                          f"algorithmic FLOPs of those rows over wall time",
                "sample_flops": flops, "sample_seconds": dt,
                "extrapolated_full_workload_seconds": full / rate,
                "extrapolated_note": "extrapolated: the measured rate applied to the whole workload's algorithmic "
                                     "FLOPs, not timed",
                "gpu_speedup_over_oracle": result["value"] * 1e12 / rate if result["value"] else None}
            parity[pc.name] = dict(rows=f"{len(rows)} sampled rows x {pc.B * pc.Hq} heads", bar=BAR, **err)
        for name, cfg in (("prefill_gqa_16k", I.PREFILL_GQA_16K), ("prefill_mha_4k", I.PREFILL_MHA_4K)):
            if name + "_out" not in host:
                continue
            q, k, v, scale = host[name]
            err, flops, dt = oracle_check(pool, q, k, v, scale, *host[name + "_out"], range(cfg.N),
                                          heads_per_job=1)
            parity[cfg.name] = dict(rows=f"all {cfg.N} rows x {cfg.B * cfg.Hq} heads", bar=BAR, oracle_seconds=dt,
                                    **err)
        for name in ("prefill_chunked", "prefill_window"):
            if name + "_out" not in host:
                continue
            vq, vk, vv, cq, ck, causal, window, vscale = host[name]
            err, dt = oracle_varlen_check(pool, vq, vk, vv, cq, ck, causal, window, vscale, *host[name + "_out"])
            parity[name] = dict(rows=f"all {vq.shape[0]} packed rows x {vq.shape[1]} heads", bar=BAR,
                                oracle_seconds=dt, **err)
        outs = {k_: host[k_ + "_out"] for k_ in ("decode", "decode_paged") if k_ + "_out" in host}
        if outs:
            seqs = decode_sample_sequences(lens_host)
            errs, dt = oracle_decode_check(pool, dq, dkd, dvd, lens_host, dscale, outs, seqs)
            for k_, err in errs.items():
                parity[k_ + " " + dc.name] = dict(sequences=f"{len(seqs)} of {dc.B} sequences (the 2 shortest, "
                                                  f"the 2 longest, seeded others) x {dc.Hq} heads",
                                                  bar={"o_max_abs": BAR["o_max_abs"], "o_mean_abs": BAR["o_mean_abs"]},
                                                  oracle_seconds=dt, **err)
        if "prefill_f32_small_out" in host:
            err, dt = oracle_f32_check(pool, *host["prefill_f32_small"], *host["prefill_f32_small_out"])
            parity[I.PREFILL_F32_SMALL.name] = dict(rows="every element", bar=F32_BAR, oracle_seconds=dt, **err)
        if "backward_out" in host:
            bq, bk, bv, bdo, bscale = host["backward"]
            err, dt = oracle_backward_check(pool, bq, bk, bv, bdo, bscale, host["backward_out"])
            bc = I.PREFILL_MHA_4K
            parity["backward " + bc.name] = dict(heads=f"dq, dk, dv of all {bc.B * bc.Hq} heads", bar=BWD_BAR,
                                                 oracle_seconds=dt, **err)
        pool.close()
        pool.join()
        result["parity"] = parity
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
