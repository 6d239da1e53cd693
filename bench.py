#!/usr/bin/env python3
"""Benchmark of the exact-attention hot path on one MI355X.

One step = one fa_prefill call on the causal MHA workload (B4 H32 N4096
d128 bf16), one fa_decode call on the GQA decode workload (B64 Hq32 Hkv8 d128
bf16, cache lengths uniform in [1024, 32768]), one fa_decode_paged call on
the same logical caches in 64-key pages of a shuffled pool, and two
fa_prefill_varlen calls: a 4096-query chunk against a 16384-key prefix (GQA B2
Hq32 Hkv8 d128, causal) and the MHA 4K workload with a 1024-key causal window.
Inputs are seeded synthetic tensors already resident in HBM before timing
starts.

`value` is prefill TFLOP/s (algorithmic FLOPs = 4*d*B*Hq*(N(N+1)/2) over the
prefill kernel's own HIP-event time); the decode figures (KV bytes read per
second) are reported beside it.  Kernel durations come from HIP events
recorded on the stream the kernels are launched on.  A bounded sample of the
fp64 CPU oracle is timed on the host as a reported baseline, and the
device's sustained MFMA and HBM-read rates are measured after the timed
region.

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
PROFILES = os.path.join(ROOT, "profiles")
PREFILL_SRC = os.path.join(ROOT, "exact_tiled_attention_prefill_amd", "csrc", "prefill_bf16.hip")
DECODE_SRC = os.path.join(ROOT, "exact_tiled_attention_prefill_amd", "csrc", "decode.hip")


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


def prefill_waves(d, causal, n_q, n_k, window=-1):
    """Waves per prefill workgroup that the library's launcher picks (for
    the kernel labels): 8 when the average query row of sequences with n_q
    queries against n_k keys sees 8192 keys or more at d = 128, else 4."""
    keys = n_k - ((n_q - 1) / 2 if causal else 0)
    if window >= 0:
        keys = min(keys, window + 1)
    return 8 if d == 128 and keys >= 8192 else 4


def prefill_bytes(B, Hq, Hkv, N, d, elem=2):
    return (2 * B * Hq * N * d + 2 * B * Hkv * N * d) * elem + B * Hq * N * 4


def decode_bytes(lens, Hq, Hkv, d, elem=2):
    kv = sum(int(x) for x in lens) * Hkv * d * 2 * elem
    return kv + 2 * len(lens) * Hq * d * elem + 4 * len(lens)


def source_hash(path):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def measured_traffic(name, src):
    """HBM bytes per launch from a committed rocprofv3 counter summary.

    profiles/<name>.md carries a line `traffic_bytes_per_launch: <int>` and
    `kernel_source_sha: <hash>`; the figure is only used while the kernel
    source still has that hash (otherwise null: the counters are stale).
    """
    path = os.path.join(PROFILES, name + ".md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    h = re.search(r"kernel_source_sha:\s*([0-9a-f]+)", text)
    if not m or not h or h.group(1) != source_hash(src):
        return None
    return float(m.group(1))


def measured_counters(name, src, keys):
    """Derived rocprofv3 counter figures (MFMA busy fraction, counted MFMA
    FLOPs over algorithmic FLOPs, clock, HBM rate) from a committed summary,
    used only while the kernel source still has the summary's hash."""
    path = os.path.join(PROFILES, name + ".md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    h = re.search(r"kernel_source_sha:\s*([0-9a-f]+)", text)
    if not h or h.group(1) != source_hash(src):
        return None
    out = {}
    for key in keys:
        m = re.search(key + r":\s*([0-9.eE+-]+)", text)
        if m:
            out[key] = float(m.group(1))
    return out or None


def measured_ceilings():
    """Sustained MFMA and HBM-read rates of this device from libfa_probes.so.

    The nominal peaks above assume the 2.4 GHz boost clock; under dense MFMA
    load on random operands the part is power-limited, so the rate the matrix
    cores actually sustain (and HBM's practical read rate) is measured here
    and reported beside them.  Returns None if the probe library is absent.
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
    out["note"] = ("whole-chip sustained v_mfma_f32_32x32x16_bf16 rate (two waves per SIMD, operands in "
                   "registers) and a 4 GiB read-only stream with 16-byte loads, with and without the "
                   "non-temporal hint (hbm_read_gbs is the faster)")
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
    return {"io_bytes": sum(t.numel() * t.element_size() for t in io), "workspace_bytes": workspace,
            "allocated_before_call": before, "peak_during_call": peak,
            "extra_over_call": peak - before, "n_by_n_fp32_scores_bytes": n_by_n}


def _oracle_pool_init():
    """Process-pool worker start-up: one BLAS thread per worker process."""
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS", "BLIS_NUM_THREADS"):
        os.environ[var] = "1"


def _oracle_head(job):
    """One (batch, head) of the causal prefill workload through the fp64 oracle
    (run in a pool worker): every query row, and the GPU output's error on
    them.  Tensors arrive as raw bf16 bits (uint16) and lse as float32."""
    import numpy as np

    import oracle

    qh, kh, vh, oh, lh, scale = job
    bf16 = lambda a: (a.astype(np.uint32) << 16).view(np.float32)  # exact bf16 -> fp32
    n, d = qh.shape
    q4, k4, v4 = (bf16(a)[None, None] for a in (qh, kh, vh))
    ro, rl = oracle.attention_rows(q4, k4, v4, True, scale, np.arange(n), [(0, 0)])
    e = np.abs(bf16(oh).astype(np.float64) - ro[0])
    el = np.abs(lh.astype(np.float64) - rl[0])
    return 4 * d * n * (n + 1) // 2, float(e.max()), float(e.sum()), int(e.size), float(el.max())


def cpu_baseline_pool(pool, workers, q, k, v, scale, o_gpu, lse_gpu):
    """Time the fp64 oracle on the WHOLE prefill workload (every causal row of
    every (batch, head)), spread over a pool of worker processes, and report
    the GPU output's error on all of it."""
    import torch

    B, Hq, N, d = q.shape
    G = Hq // k.shape[1]
    bits = lambda t: t.contiguous().view(torch.int16).numpy().view("uint16")
    jobs = ((bits(q[b, h]), bits(k[b, h // G]), bits(v[b, h // G]), bits(o_gpu[b, h]),
             lse_gpu[b, h].contiguous().numpy(), scale) for b in range(B) for h in range(Hq))
    t0 = time.perf_counter()
    res = list(pool.imap_unordered(_oracle_head, jobs, chunksize=1))
    dt = time.perf_counter() - t0
    flops = sum(r[0] for r in res)
    count = sum(r[3] for r in res)
    o_max, o_mean, l_max = max(r[1] for r in res), sum(r[2] for r in res) / count, max(r[4] for r in res)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": workers, "kind": "oracle",
            "sample": f"the whole B{B} H{Hq} N{N} d{d} causal workload ({B * Hq} heads x {N} rows), fp64 numpy, "
                      f"{workers} worker processes with 1 BLAS thread each, {dt:.1f} s wall (inputs pickled "
                      f"to the workers inside the timed span); the rate is algorithmic FLOPs over wall time",
            "gpu_error_on_these_rows": {
                "rows": "all", "o_max_abs": o_max, "o_mean_abs": o_mean, "lse_max_abs": l_max,
                "bar": {"o_max_abs": 2e-2, "o_mean_abs": 2e-3, "lse_max_abs": 1e-3},
                "within_bar": o_max <= 2e-2 and o_mean <= 2e-3 and l_max <= 1e-3}}


def cpu_baseline(q, k, v, scale, seconds, o_gpu=None, lse_gpu=None):
    """Time the fp64 oracle on sampled causal rows of the prefill workload.

    When the GPU's output (host copies) is given, the same oracle rows also
    give the error of those rows: max-abs / mean-abs of O and max-abs of lse.
    """
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    from exact_tiled_attention_prefill_amd.inputs import sample_rows

    B, Hq, N, d = q.shape
    rows = sample_rows(N, 2048, seed=3)  # ~2100 rows spread over the sequence, per head
    heads = [(b, h) for b in range(B) for h in range(Hq)]
    done_flops, done_rows, done_heads, t0 = 0, 0, 0, time.perf_counter()
    err = {"o_max_abs": 0.0, "o_abs_sum": 0.0, "o_count": 0, "lse_max_abs": 0.0}
    with threadpool_limits(limits=1):
        for b, h in heads:
            ro, rl = oracle.attention_rows(q, k, v, True, scale, rows, [(b, h)])
            done_flops += sum(4 * d * (r + 1) for r in rows)
            done_rows += len(rows)
            done_heads += 1
            if o_gpu is not None:
                e = np.abs(o_gpu[b, h, rows].double().numpy() - ro[0])
                err["o_max_abs"] = max(err["o_max_abs"], float(e.max()))
                err["o_abs_sum"] += float(e.sum())
                err["o_count"] += e.size
                el = np.abs(lse_gpu[b, h, rows].double().numpy() - rl[0])
                err["lse_max_abs"] = max(err["lse_max_abs"], float(el.max()))
            if time.perf_counter() - t0 >= seconds:
                break
    dt = time.perf_counter() - t0
    out = {"value": done_flops / dt / 1e12, "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
           "sample": f"{done_rows} causal query rows ({len(rows)} sampled rows x {done_heads} heads) of "
                     f"the B4 H32 N4096 d128 workload, fp64 numpy, {dt:.1f} s, 1 BLAS thread; "
                     f"the rate is algorithmic FLOPs of those rows over wall time"}
    if o_gpu is not None and err["o_count"]:
        mean = err["o_abs_sum"] / err["o_count"]
        out["gpu_error_on_these_rows"] = {
            "o_max_abs": err["o_max_abs"], "o_mean_abs": mean, "lse_max_abs": err["lse_max_abs"],
            "bar": {"o_max_abs": 2e-2, "o_mean_abs": 2e-3, "lse_max_abs": 1e-3},
            "within_bar": err["o_max_abs"] <= 2e-2 and mean <= 2e-3 and err["lse_max_abs"] <= 1e-3}
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the MFMA / HBM ceiling probes")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the 16K and 128K causal GQA prefill configurations")
    ap.add_argument("--page-size", type=int, default=64, help="page size of the paged-decode leg")
    ap.add_argument("--only", choices=["prefill", "decode", "decode_paged", "prefill_chunked", "prefill_window",
                                       "backward", "prefill_gqa_16k", "prefill_gqa_128k", "copy", "ceiling"],
                    default=None,
                    help="run one kernel only (for profiler runs); 'copy' runs a plain 1 GiB device "
                         "copy used to calibrate the HBM byte counters; 'ceiling' runs only the "
                         "MFMA / HBM ceiling probes")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); nothing to do for N > 1.",
              file=sys.stderr)
        sys.exit(2)

    # The oracle's worker processes start before anything touches the GPU (a
    # process that has initialised the GPU does not start new programs).
    pool, workers = None, 0
    if args.only in (None, "prefill") and not args.no_cpu_baseline:
        try:
            import multiprocessing

            workers = max(1, min(16, len(os.sched_getaffinity(0))))
            pool = multiprocessing.get_context("spawn").Pool(workers, initializer=_oracle_pool_init)
        except Exception as exc:  # fall back to the single-thread sampled baseline
            print(f"oracle process pool unavailable ({exc}); timing a single-thread sample", file=sys.stderr)
            pool = None

    import torch

    from exact_tiled_attention_prefill_amd import (decode, decode_paged, decode_paged_workspace_bytes,
                                                   decode_workspace_bytes, load_library, prefill, prefill_backward,
                                                   prefill_backward_workspace_bytes, prefill_varlen)
    from exact_tiled_attention_prefill_amd import inputs as I

    load_library()  # fail loudly before any work if libfa.so is missing
    dev = torch.device("cuda:0")
    if args.only == "ceiling":
        print(json.dumps({"ceilings": measured_ceilings()}), flush=True)
        return
    if args.only == "copy":
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(args.warmup + args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": 1 << 30, "launches": args.warmup + args.steps}))
        return
    stream = torch.cuda.current_stream()
    out = {}
    run_prefill = args.only in (None, "prefill")
    run_decode = args.only in (None, "decode") and not args.no_decode
    run_paged = args.only in (None, "decode_paged") and not args.no_decode
    run_chunk = args.only in (None, "prefill_chunked")
    run_window = args.only in (None, "prefill_window")
    run_bwd = args.only in (None, "backward")

    pc = I.PREFILL_MHA_4K
    if run_prefill:
        q, k, v, scale = I.prefill_config_inputs(pc)
        qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
        od = torch.empty_like(qd)
        lsed = torch.empty((pc.B, pc.Hq, pc.N), dtype=torch.float32, device=dev)

        def pf():
            prefill(qd, kd, vd, causal=True, scale=scale, out=od, lse=lsed)
        p_mem = device_memory(pf, [qd, kd, vd, od, lsed], 0,
                              pc.B * pc.Hq * pc.N * pc.N * 4)

    dc = I.DECODE_GQA
    if run_decode or run_paged:
        dq, dk, dv, dl, dscale = I.decode_config_inputs(dc)
        lens_host = dl.tolist()
        dqd, dkd, dvd, dld = dq.to(dev), dk.to(dev), dv.to(dev), dl.to(dev)
        dod = torch.empty_like(dqd)
        del dk, dv
    if run_decode:
        ws = torch.empty(decode_workspace_bytes(dc.B, dc.Hq, dc.Hkv, dc.maxlen, dc.d), dtype=torch.uint8,
                         device=dev)

        def df():
            decode(dqd, dkd, dvd, dld, scale=dscale, out=dod, workspace=ws)
        d_mem = device_memory(df, [dqd, dkd, dvd, dld, dod], ws.numel(), None)
    if run_paged:
        # the same logical caches scattered over a shuffled pool of pages
        kpd, vpd, table, _ = I.paged_cache(dkd, dvd, dl, args.page_size, seed=11)
        tbd = table.to(dev)
        if not run_decode:
            del dkd, dvd
        pws = torch.empty(decode_paged_workspace_bytes(dc.B, dc.Hq, dc.Hkv, args.page_size, table.shape[1], dc.d),
                          dtype=torch.uint8, device=dev)
        pod = torch.empty_like(dqd)

        def pgf():
            decode_paged(dqd, kpd, vpd, tbd, dld, scale=dscale, out=pod, workspace=pws)

    # packed variable-length legs: a 4096-query chunk against a 16384-key prefix
    # (GQA B2 Hq32 Hkv8 d128, causal bottom-right), and the MHA 4K workload
    # with a 1024-key causal window
    vl_legs = []
    for name, on, lens, hq, hkv, causal, window in (
            ("prefill_chunked", run_chunk, [(4096, 16384)] * 2, 32, 8, True, -1),
            ("prefill_window", run_window, [(4096, 4096)] * 4, 32, 32, True, 1024)):
        if not on:
            continue
        vq, vk, vv, cq, ck, vscale = I.varlen_inputs(lens, hq, hkv, 128, seed=5)
        vqd, vkd, vvd, cqd, ckd = vq.to(dev), vk.to(dev), vv.to(dev), cq.to(dev), ck.to(dev)
        vod = torch.empty_like(vqd)
        vld = torch.empty((hq, vq.shape[0]), dtype=torch.float32, device=dev)
        mq = max(nq for nq, _ in lens)

        def vf(vqd=vqd, vkd=vkd, vvd=vvd, cqd=cqd, ckd=ckd, vod=vod, vld=vld, mq=mq, causal=causal,
               window=window, vscale=vscale):
            prefill_varlen(vqd, vkd, vvd, cqd, ckd, mq, causal=causal, window_left=window, scale=vscale,
                           out=vod, lse=vld)
        flops = 4 * 128 * hq * varlen_pairs(lens, causal, window)
        cfg = {"sequences": [list(x) for x in lens], "Hq": hq, "Hkv": hkv, "d": 128, "causal": causal,
               "window_left": window}
        waves = prefill_waves(128, causal, sum(nq for nq, _ in lens) / len(lens),
                              sum(nk for _, nk in lens) / len(lens), window)
        vl_legs.append((name, vf, flops, cfg, f"prefill_bf16_kernel<128,causal,varlen,{waves} waves>"))

    if run_bwd:
        # backward of the MHA 4K causal workload: the forward's o and lse feed it
        bq, bk, bv, bdo, bscale = I.backward_inputs(pc.B, pc.Hq, pc.Hkv, pc.N, pc.d, seed=1)
        bqd, bkd, bvd, bdod = bq.to(dev), bk.to(dev), bv.to(dev), bdo.to(dev)
        bo, blse = prefill(bqd, bkd, bvd, causal=True, scale=bscale)
        bdq, bdk, bdv = torch.empty_like(bqd), torch.empty_like(bkd), torch.empty_like(bvd)
        bws = torch.empty(prefill_backward_workspace_bytes(pc.B, pc.Hq, pc.N), dtype=torch.uint8, device=dev)

        def bwf():
            prefill_backward(bqd, bkd, bvd, bo, bdod, blse, causal=True, scale=bscale, dq=bdq, dk=bdk, dv=bdv,
                             workspace=bws)
        vl_legs.append(("backward", bwf, 2.5 * prefill_flops(pc.B, pc.Hq, pc.N, pc.d, True),
                        {"workload": pc.name, "flops": "2.5 x forward (five matrix products per score)",
                         "kernels": "dQ (with the D and lse rows) + dK/dV"}, "bwd_dq + bwd_dkdv"))

    for _ in range(args.warmup):
        for _, vf, _, _, _ in vl_legs:
            vf()
        if run_prefill:
            pf()
        if run_decode:
            df()
        if run_paged:
            pgf()
    torch.cuda.synchronize()

    # timed region: K steps, each = one prefill + one decode (+ one paged decode), events per call
    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4 + len(vl_legs))] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        for j, (_, vf, _, _, _) in enumerate(vl_legs):
            ev[i][4 + j].record(stream)
            vf()
        ev[i][0].record(stream)
        if run_prefill:
            pf()
        ev[i][1].record(stream)
        if run_decode:
            df()
        ev[i][2].record(stream)
        if run_paged:
            pgf()
        ev[i][3].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    p_ms = sorted(ev[i][0].elapsed_time(ev[i][1]) for i in range(K))
    d_ms = sorted(ev[i][1].elapsed_time(ev[i][2]) for i in range(K))
    g_ms = sorted(ev[i][2].elapsed_time(ev[i][3]) for i in range(K))
    vl_ms = []
    for j in range(len(vl_legs)):
        nxt = [(4 + j + 1) if j + 1 < len(vl_legs) else 0 for _ in range(K)]
        vl_ms.append(sorted(ev[i][4 + j].elapsed_time(ev[i][nxt[i]]) for i in range(K)))
    p_avg = sum(p_ms) / K
    d_avg = sum(d_ms) / K
    g_avg = sum(g_ms) / K

    props = torch.cuda.get_device_properties(dev)
    result = {
        "metric": "prefill attention TFLOP/s (% bf16 MFMA peak); decode KV-read GB/s (% HBM)",
        "value": None,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / K,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) rounded to bf16)",
        "config": {"workload": pc.name, "B": pc.B, "Hq": pc.Hq, "Hkv": pc.Hkv, "N": pc.N, "d": pc.d,
                   "causal": pc.causal, "step": "one prefill (this workload) + one decode (decode.workload) + one paged decode "
                                                              "(decode_paged.workload) + the prefill_chunked and "
                                                              "prefill_window legs"},
        "device": {"name": props.name, "cus": props.multi_processor_count,
                   "arch": getattr(props, "gcnArchName", ""), "torch": torch.__version__,
                   "hip": getattr(torch.version, "hip", None)},
    }
    if run_prefill:
        F = prefill_flops(pc.B, pc.Hq, pc.N, pc.d, True)
        tflops = F / (p_avg * 1e-3) / 1e12
        result["value"] = tflops
        result["prefill"] = {"ms_avg": p_avg, "ms_median": p_ms[K // 2], "ms_min": p_ms[0],
                             "tflops": tflops, "tokens_per_s": pc.B * pc.N / (p_avg * 1e-3),
                             "frac_of_peak": tflops / PEAK_BF16_TFLOPS, "flops_per_launch": F}
        traffic = measured_traffic("prefill_bf16_mha4k_counters", PREFILL_SRC)
        result["roofline"] = {"kernel": f"prefill_bf16_kernel<128,causal,{prefill_waves(pc.d, True, pc.N, pc.N)} waves>",
                              "bound": "mfma",
                              "achieved": tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                              "frac": tflops / PEAK_BF16_TFLOPS, "traffic": traffic,
                              "algorithmic_bytes": prefill_bytes(pc.B, pc.Hq, pc.Hkv, pc.N, pc.d),
                              "rocprof": measured_counters("prefill_bf16_mha4k_counters", PREFILL_SRC,
                                                           ("mfma_busy_fraction", "mfma_flops_over_algorithmic",
                                                            "shader_clock_ghz"))}
        result["prefill"]["device_memory"] = p_mem
    if run_decode:
        nbytes = decode_bytes(lens_host, dc.Hq, dc.Hkv, dc.d)
        gbs = nbytes / (d_avg * 1e-3) / 1e9
        result["decode"] = {"workload": dc.name, "ms_avg": d_avg, "ms_median": d_ms[K // 2],
                            "ms_min": d_ms[0], "GB_per_s": gbs, "frac_of_hbm_peak": gbs / PEAK_HBM_GBS,
                            "bytes_per_launch": nbytes, "tokens_per_s": dc.B / (d_avg * 1e-3),
                            "roofline": {"kernel": "decode_bf16_mfma_kernel + decode_combine_kernel",
                                         "bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS,
                                         "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
                                         "traffic": measured_traffic("decode_gqa_counters", DECODE_SRC),
                                         "rocprof": measured_counters("decode_gqa_counters", DECODE_SRC,
                                                                      ("hbm_gbs_counter_run", "shader_clock_ghz"))},
                            "device_memory": d_mem}
        if result["value"] is None:
            result["value"], result["unit"] = gbs, "GB/s"
    for (name, _, flops, cfg, kernel), ms in zip(vl_legs, vl_ms):
        avg = sum(ms) / K
        tf = flops / (avg * 1e-3) / 1e12
        result[name] = {"config": cfg, "ms_avg": avg, "ms_median": ms[K // 2], "ms_min": ms[0], "tflops": tf,
                        "flops_per_launch": flops,
                        "roofline": {"kernel": kernel, "bound": "mfma",
                                     "achieved": tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                     "frac": tf / PEAK_BF16_TFLOPS}}
        if result["value"] is None:
            result["value"] = tf
    if run_paged:
        nbytes = decode_bytes(lens_host, dc.Hq, dc.Hkv, dc.d) + table.numel() * 4
        gbs = nbytes / (g_avg * 1e-3) / 1e9
        result["decode_paged"] = {"workload": dc.name + f"-paged{args.page_size}", "page_size": args.page_size,
                                  "ms_avg": g_avg, "ms_median": g_ms[K // 2], "ms_min": g_ms[0],
                                  "GB_per_s": gbs, "frac_of_hbm_peak": gbs / PEAK_HBM_GBS,
                                  "bytes_per_launch": nbytes, "tokens_per_s": dc.B / (g_avg * 1e-3),
                                  "roofline": {"kernel": "decode_bf16_mfma_kernel<paged> + decode_combine_kernel",
                                               "bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS,
                                               "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS}}
        if result["value"] is None:
            result["value"], result["unit"] = gbs, "GB/s"
    # the other two causal GQA configurations, timed after the steps above
    # with their own (smaller) step counts: B2 Hq32 Hkv8 N16384 and
    # B1 Hq64 Hkv8 N131072 (O(N) memory: no N x N buffer exists anywhere)
    cfg_legs = []
    for name, cfg, steps in (("prefill_gqa_16k", I.PREFILL_GQA_16K, max(1, min(K, 10))),
                             ("prefill_gqa_128k", I.PREFILL_GQA_128K, max(1, min(K, 3)))):
        if not (args.only == name or (args.only is None and not args.no_configs)):
            continue
        cq, ck_, cv, cscale = I.prefill_config_inputs(cfg)
        cqd, ckd_, cvd = cq.to(dev), ck_.to(dev), cv.to(dev)
        del cq, ck_, cv
        cod = torch.empty_like(cqd)
        cld = torch.empty((cfg.B, cfg.Hq, cfg.N), dtype=torch.float32, device=dev)
        prefill(cqd, ckd_, cvd, causal=True, scale=cscale, out=cod, lse=cld)
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for e0, e1 in evs:
            e0.record(stream)
            prefill(cqd, ckd_, cvd, causal=True, scale=cscale, out=cod, lse=cld)
            e1.record(stream)
        torch.cuda.synchronize()
        ms = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
        avg = sum(ms) / steps
        F = prefill_flops(cfg.B, cfg.Hq, cfg.N, cfg.d, True)
        tf = F / (avg * 1e-3) / 1e12
        result[name] = {"workload": cfg.name, "steps": steps, "ms_avg": avg, "ms_median": ms[steps // 2],
                        "ms_min": ms[0], "tflops": tf, "tokens_per_s": cfg.B * cfg.N / (avg * 1e-3),
                        "flops_per_launch": F,
                        "roofline": {"kernel": f"prefill_bf16_kernel<128,causal,{prefill_waves(cfg.d, True, cfg.N, cfg.N)} waves>",
                                     "bound": "mfma", "achieved": tf,
                                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": tf / PEAK_BF16_TFLOPS}}
        cfg_legs.append(name)
        del cqd, ckd_, cvd, cod, cld
        torch.cuda.empty_cache()
        if result["value"] is None:
            result["value"] = tf
    if args.only is None and not args.no_ceilings:
        ceil = measured_ceilings()
        result["ceilings"] = ceil
        if ceil is not None:
            sus = ceil["mfma_bf16_random_operands"]["tflops"]
            for rl in ([result.get("roofline")] + [result[n]["roofline"] for n, _, _, _, _ in vl_legs]
                       + [result[n]["roofline"] for n in cfg_legs]):
                if rl is not None:
                    rl["measured_ceiling"] = sus
                    rl["frac_of_measured_ceiling"] = rl["achieved"] / sus
            for leg in ("decode", "decode_paged"):
                if leg in result:
                    rl = result[leg]["roofline"]
                    rl["measured_ceiling"] = ceil["hbm_read_gbs"]
                    rl["frac_of_measured_ceiling"] = rl["achieved"] / ceil["hbm_read_gbs"]
    if run_prefill and not args.no_cpu_baseline:
        if pool is not None:
            result["cpu_baseline"] = cpu_baseline_pool(pool, workers, q, k, v, scale, od.cpu(), lsed.cpu())
            pool.close()
            pool.join()
        else:
            result["cpu_baseline"] = cpu_baseline(q, k, v, scale, args.cpu_seconds, od.cpu(), lsed.cpu())
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
