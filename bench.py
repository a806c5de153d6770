#!/usr/bin/env python3
"""Throughput of the Dust LM-head estimator on one MI355X.

One step = one dust_head_estimate call over the whole batch (noise, perturbed
cross-entropy, centring, reward, error estimate and the G_W outer product),
inputs resident in HBM, outputs and workspace preallocated.  Prints one JSON
line: token-draws/s (T*K per step), the roofline of the dominant kernel (the
fused noise + cross-entropy + accumulate kernel, timed with HIP events on the
call's stream inside the timed loop) and the fp64 CPU oracle's rate on a
bounded sample of the same workload.

  python bench.py [--steps 20] [--warmup 5] [--workload paper] [--no-cpu-baseline]
                  [--copy-probe-mib 256]

The default line also carries sub-records ("workloads") for the LM head at
K = 1024 and K = 16384 (the public code's default population) and the
hidden-layer estimator, each with its own roofline and oracle baseline.  Other workloads print their
own line: linear (the hidden-layer estimator), k1024, k16384, forward
(perturbed forward), embedding, optim (SGD/Adam steps), cosine (the
cosine-versus-population sweep and its fitted law).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "token-draws/sec, LM-head Dust estimator (T=16384, V=4096) + % VALU/MFMA peak"

# MI355X peaks.  VALU: 256 CUs x 4 SIMDs x 32 lanes x 2.4 GHz = 78.64e12
# full-rate 32-bit lane operations per second, i.e. the published fp32 vector
# 157.3 TFLOP/s counted as FMAs.  fp16/bf16 dense MFMA 2.5 PFLOP/s.  HBM3E 8 TB/s.
VALU_SLOTS_PER_S = 256 * 4 * 32 * 2.4e9
FP16_MFMA_FLOPS = 2.5e15  # dense fp16 (and bf16) matrix cores
SCAN_LAUNCHES = 50  # back-to-back reward scans timed for the scan's per-launch figure
HBM_BYTES_PER_S = 8.0e12

# VALU issue slots per normal (one column of one token-draw), charged at the
# issue costs measured on gfx950 with a dependent-chain probe: 1 slot for fp32
# add/mul/fma and 32-bit logic (including v_bitop3), 2 for v_mad_u64_u32 and
# v_alignbit, 4 for the transcendentals (v_exp, v_log, v_sqrt, v_sin, v_cos).
#
# Algorithmic count, the work the method itself asks per normal (what the
# roofline divides by):
#   Philox4x32-10, a quarter block: 5 32x32->64 products (2) + 5 three-input
#     xors (1) = 15
#   uniform map: alignbit + subtract = 3
#   Box-Muller, half a pair: half of log, sqrt, sin, cos (8) + the radius
#     multiply (1) = 9
#   perturbed cross-entropy: FMA + exp2 + add = 6
#   accumulation of sum a and sum delta a: 2
# total 35.  The error estimate of the linear layer: the same noise (27) and
# one FMA, 28.
SLOTS = {"philox": 15.0, "uniform": 3.0, "box_muller": 9.0, "cross_entropy": 6.0,
         "accumulate": 2.0}
SLOTS_PER_NORMAL = sum(SLOTS.values())
SLOTS_PER_NORMAL_ERROR_ESTIMATE = SLOTS["philox"] + SLOTS["uniform"] + SLOTS["box_muller"] + 1
# The fused head kernel's own count is lower: with the column's Philox word in
# a xor, the first rounds are the same for all lanes of a wave and 4 of the 20
# products per block run on the scalar unit (16 x 2 + 18 xors = 12.5 per
# normal), the normals come scaled by 1/sqrt(2 ln 2), one multiply fewer per
# pair (Box-Muller 9), and the angle word reaches v_sin/v_cos as 1 + v (they
# reduce modulo one revolution) without the subtraction (uniform 2.5): 32 slots
# issued per normal by design.
IMPL_SLOTS_PER_NORMAL = 32.0
IMPL_SLOTS_PER_NORMAL_ERROR_ESTIMATE = 25.0

# Hardware byte counts of the head kernel (FETCH_SIZE and WRITE_SIZE from two
# rocprofv3 --pmc runs, scaled by the same counters read on a plain copy of
# known size) are kept in this summary with the hash of the kernel sources
# they were taken on; they are reported only while the sources are unchanged.
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "head_kernel_paper_traffic.json")
KERNEL_SOURCES = ["activation_perturbation_estimator_amd/csrc/dust_head.hip",
                  "activation_perturbation_estimator_amd/csrc/dust_device.hpp",
                  "activation_perturbation_estimator_amd/csrc/dust_gemm16.hpp"]


def kernel_source_hash() -> str:
    """sha256 of the kernel sources with comments and blank space removed, so
    that editing a comment does not invalidate the recorded counters."""
    import hashlib
    import re
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def measured_traffic(workload: str):
    try:
        with open(TRAFFIC_SUMMARY) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("workload") != workload or rec.get("source_sha256") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="paper",
                    help="paper (default: T=16384, V=4096, d=512, K=64), k1024, k16384, tiny, "
                         "linear (hidden layer 512->2048, K=256, gamma=0.9); the other rows: "
                         "forward, embedding, optim, cosine")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sub-workloads", action="store_true",
                    help="paper workload only: skip the K=1024, K=16384 and linear sub-records")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after timing, run one plain fp32 copy kernel (y = x * 1) over this "
                         "many MiB: the reference that scales hardware byte counters")
    return ap.parse_args()


def host_cores() -> int:
    """The cores this process may run on (its affinity mask)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def oracle_rate(run_sample, T: int, K: int, target_s: float, threads: int, n0: int):
    """Time the oracle (as it stands) on growing random token samples of the
    workload (all K draws each, seed 1) until one takes about target_s seconds
    on `threads` OpenMP threads; returns (token-draws/s, tokens, seconds)."""
    import numpy as np
    import oracle
    oracle.build(force=False)
    oracle.set_num_threads(threads)
    rng = np.random.default_rng(1)
    n = max(1, min(n0, T))
    while True:
        tok = np.sort(rng.choice(T, size=n, replace=False))
        t0 = time.perf_counter()
        run_sample(tok)
        dt = time.perf_counter() - t0
        if dt >= 0.5 * target_s or n >= T:
            break
        n = min(T, max(n + 1, int(n * min(8.0, 0.75 * target_s / max(dt, 1e-3)))))
    return len(tok) * K / dt, len(tok), dt


def cpu_baseline_record(run_sample, w, target_s: float, what: str):
    """The oracle on all host cores and on one thread, on bounded samples of the
    same workload; the rate is per token-draw, uniform over tokens, so the full
    workload's time is the sample's scaled by T / tokens ("extrapolated")."""
    cores = host_cores()
    rate, ntok, dt = oracle_rate(run_sample, w.T, w.K, target_s, cores, 2 * cores)
    rate1, ntok1, dt1 = oracle_rate(run_sample, w.T, w.K, target_s / 2, 1, 1)
    return {"value": rate, "unit": "token-draws/s", "cores": cores, "kind": "oracle",
            "sample": f"{ntok} of {w.T} tokens x all {w.K} draws of the same workload ({what}, "
                      f"fp64, OpenMP over tokens on {cores} threads), {dt:.2f} s; full workload "
                      f"extrapolated: {w.T * w.K / rate:.1f} s",
            "single_thread": {"value": rate1, "cores": 1,
                              "sample": f"{ntok1} tokens x {w.K} draws, {dt1:.2f} s"}}


def cpu_baseline(w, z, y, target_s: float):
    """The fp64 oracle, as it stands, on bounded samples of tokens of the same
    LM-head workload."""
    import numpy as np
    import oracle
    from activation_perturbation_estimator_amd import synth
    yn = y.numpy()

    def run(tok):
        zfull = np.zeros((w.T, w.V))
        zfull[tok] = synth.to_f64(z[tok])
        oracle.head_rows(zfull, yn, w.seq_len, w.sigma, w.K, w.gamma, w.philox_seed, tok)

    return cpu_baseline_record(run, w, target_s, "g_hat rows")


def time_steps(torch, step, steps: int, warmup: int, nev: int, copy_probe_mib: int = 0,
               same_as_previous=()):
    """Warm-up, then `steps` timed calls bracketed by device synchronisation;
    returns (ms per step, per-stage ms per launch) from the library's stage events.

    Each recorded event puts a few microseconds of marker between two kernels,
    so the loop records only the boundaries it needs: the first call's start,
    then each call's later boundaries; a call's start is the previous call's
    end (the calls are back to back on one stream), and the boundaries listed
    in `same_as_previous` (a stage the call skips, recorded back to back with
    the boundary before it) are not recorded."""
    for _ in range(warmup):
        step(None)
    torch.cuda.synchronize()

    def recorded(k, b):
        return k == 0 if b == 0 else b not in same_as_previous

    evs = [[torch.cuda.Event(enable_timing=True) if recorded(k, b) else None
            for b in range(nev)] for k in range(steps)]
    for row in evs:  # materialise the handles on this stream before timing
        for e in row:
            if e is not None:
                e.record()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if copy_probe_mib:
        n = copy_probe_mib * (1 << 20) // 4
        xs = torch.ones(n, dtype=torch.float32, device="cuda:0")
        ys = torch.empty_like(xs)
        torch.mul(xs, 1.0, out=ys)
        torch.cuda.synchronize()
        del xs, ys
    stage = [0.0] * (nev - 1)
    for k, row in enumerate(evs):
        # boundary b of call k: its own event, else the recorded boundary before it
        marks = [row[0] if k == 0 else evs[k - 1][nev - 1]]
        for b in range(1, nev):
            marks.append(row[b] if row[b] is not None else marks[-1])
        for s in range(nev - 1):
            if marks[s] is not marks[s + 1]:
                stage[s] += marks[s].elapsed_time(marks[s + 1])
    return wall * 1e3 / steps, [v / steps for v in stage]


def common_fields(args, w, value, ms_per_step, metric, workload_text):
    return {
        "metric": metric, "value": value, "unit": "token-draws/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": workload_text, "T": w.T, "N": w.V, "d": w.d, "K": w.K,
                   "global_batch": w.T, "seq_len": w.seq_len, "parallelism": "single GPU"},
    }


def outer_sum_fields(w, stage_ms):
    """The G_W stage (fp16 matrix-core pass over per-token power-of-two scaled
    operands, then the fixed-order sum of the token splits): one pass, so the
    executed flops are the algorithmic 2 T N d."""
    flops = 2.0 * w.T * w.V * w.d
    return {"stage_ms": stage_ms, "algorithmic_tflops": flops / (stage_ms / 1e3) / 1e12,
            "peak_fp16_tflops": FP16_MFMA_FLOPS / 1e12,
            "frac": flops / (stage_ms / 1e3) / FP16_MFMA_FLOPS}


def run_head(args, torch, dust, synth, w):
    z, y, X = synth.workload_inputs(w)
    dev = torch.device("cuda:0")
    zd, yd, Xd = z.to(dev), y.to(dev), X.to(dev)
    g = torch.empty((w.T, w.V), dtype=torch.float32, device=dev)
    G = torch.empty((w.V, w.d), dtype=torch.float32, device=dev)
    ws = torch.empty(dust.head_workspace_size(w.T, w.V, w.d, w.K, w.gamma), dtype=torch.uint8,
                     device=dev)

    def step(events):
        dust.head_estimate(zd, yd, Xd, sigma=w.sigma, K=w.K, gamma=w.gamma, seed=w.philox_seed,
                           seq_len=w.seq_len, workspace=ws, out=(g, G), stage_events=events)

    # gamma = 0: one fused kernel ends the loss and the error-estimate stages
    # together, so the boundary after the latter is not recorded
    fused = (w.gamma == 0.0)
    ms_per_step, stage = time_steps(torch, step, args.steps, args.warmup,
                                    dust.DUST_STAGE_EVENTS, args.copy_probe_mib,
                                    same_as_previous=(2,) if fused else ())
    value = w.T * w.K / (ms_per_step / 1e3)
    head_ms = stage[0]
    achieved = float(w.T) * w.K * w.V * SLOTS_PER_NORMAL / (head_ms / 1e3) / 1e12
    peak = VALU_SLOTS_PER_S / 1e12
    out = common_fields(args, w, value, ms_per_step, METRIC,
                        f"{w.name}: LM head T={w.T} ({w.T // w.seq_len}x{w.seq_len}), V={w.V}, "
                        f"d={w.d}, K={w.K}, sigma={w.sigma}, gamma={w.gamma}, "
                        f"{'bf16' if w.bf16 else 'fp32'} logits and X")
    out["roofline"] = {"bound": "alu", "kernel": "head_kernel (fused noise + CE + accumulate)"
                       if fused else "head_kernel (per-draw losses)",
                       "achieved": achieved, "peak": peak, "unit": "T VALU slots/s",
                       "frac": achieved / peak, "traffic": measured_traffic(w.name),
                       "slots_per_normal": SLOTS_PER_NORMAL,
                       "impl_slots_per_normal": IMPL_SLOTS_PER_NORMAL,
                       "impl_frac": achieved / peak * IMPL_SLOTS_PER_NORMAL / SLOTS_PER_NORMAL,
                       "launch_ms": head_ms}
    # the same kernel in HBM terms (algorithmic bytes: logits read once, g_hat written once)
    head_bytes = w.T * w.V * (2.0 if w.bf16 else 4.0) + 4.0 * w.T + 4.0 * w.T * w.V
    out["roofline"]["hbm_gbs"] = head_bytes / (head_ms / 1e3) / 1e9
    out["roofline"]["hbm_frac"] = head_bytes / (head_ms / 1e3) / HBM_BYTES_PER_S
    out["stages_ms"] = {"head": stage[0], "error_estimate": stage[1], "outer_sum": stage[2]}
    out["outer_sum"] = outer_sum_fields(w, stage[2])
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, z, y, args.cpu_seconds)
    return out


def cpu_baseline_linear(w, c, target_s: float):
    import oracle
    cd = c.double().numpy()

    def run(tok):
        oracle.linear_rows(cd, w.seq_len, w.V, w.sigma, w.gamma, w.philox_seed, tok)

    return cpu_baseline_record(run, w, target_s, "reward scan over all tokens, g_hat rows")


def run_linear(args, torch, dust, synth, w):
    X, c = synth.workload_inputs(w)
    dev = torch.device("cuda:0")
    Xd, cd = X.to(dev), c.to(dev)
    g = torch.empty((w.T, w.V), dtype=torch.float32, device=dev)
    G = torch.empty((w.V, w.d), dtype=torch.float32, device=dev)
    ws = torch.empty(dust.linear_workspace_size(w.T, w.d, w.V, w.K, w.gamma), dtype=torch.uint8,
                     device=dev)

    def step(events):
        dust.linear_estimate(Xd, cd, N=w.V, sigma=w.sigma, gamma=w.gamma, seed=w.philox_seed,
                             seq_len=w.seq_len, workspace=ws, out=(g, G), stage_events=events)

    ms_per_step, stage = time_steps(torch, step, args.steps, args.warmup,
                                    dust.DUST_STAGE_EVENTS, args.copy_probe_mib)
    value = w.T * w.K / (ms_per_step / 1e3)
    ee_ms = stage[1]
    achieved = (float(w.T) * w.K * w.V * SLOTS_PER_NORMAL_ERROR_ESTIMATE / (ee_ms / 1e3) / 1e12)
    peak = VALU_SLOTS_PER_S / 1e12
    scan_bytes = 8.0 * w.T * w.K  # read c, write r
    out = common_fields(args, w, value, ms_per_step,
                        "token-draws/sec, hidden linear layer Dust estimator "
                        f"(T={w.T}, N={w.V}, d_in={w.d})",
                        f"{w.name}: linear d_in={w.d} -> N={w.V}, T={w.T} "
                        f"({w.T // w.seq_len}x{w.seq_len}), K={w.K}, sigma={w.sigma}, "
                        f"gamma={w.gamma}, bf16 X, caller c fp32")
    out["roofline"] = {"bound": "alu", "kernel": "error_estimate_kernel (noise + r a accumulate)",
                       "achieved": achieved, "peak": peak, "unit": "T VALU slots/s",
                       "frac": achieved / peak, "traffic": None,
                       "slots_per_normal": SLOTS_PER_NORMAL_ERROR_ESTIMATE,
                       "impl_slots_per_normal": IMPL_SLOTS_PER_NORMAL_ERROR_ESTIMATE,
                       "impl_frac": achieved / peak * IMPL_SLOTS_PER_NORMAL_ERROR_ESTIMATE /
                       SLOTS_PER_NORMAL_ERROR_ESTIMATE, "launch_ms": ee_ms}
    # the accumulate pass in HBM terms too: it reads r [K,T] and writes g_hat [T,N]
    acc_bytes = 4.0 * w.K * w.T + 4.0 * w.T * w.V
    out["roofline"]["hbm_gbs"] = acc_bytes / (ee_ms / 1e3) / 1e9
    out["roofline"]["hbm_frac"] = acc_bytes / (ee_ms / 1e3) / HBM_BYTES_PER_S
    # the scan takes a few microseconds, less than a call from Python takes to
    # launch it, so the stage events around it (and back-to-back calls) time the
    # host: its per-launch time comes from a HIP graph of SCAN_LAUNCHES scans,
    # replayed between two events
    rbuf = torch.empty((w.K, w.T), dtype=torch.float32, device=dev)
    scan = lambda: dust.reward_scan(cd, seq_len=w.seq_len, gamma=w.gamma, out=rbuf)
    scan_eager_ms = _time_calls(torch, scan, SCAN_LAUNCHES, 2)
    try:
        scan_ms = _time_graph(torch, scan, SCAN_LAUNCHES)
        scan_timing = "one HIP graph of back-to-back launches"
    except RuntimeError as e:  # no graph capture here: the eager figure, which times the host
        print(f"[bench] reward scan graph capture failed ({e}); eager timing", file=sys.stderr)
        scan_ms, scan_timing = scan_eager_ms, "back-to-back calls from Python"
    del rbuf
    out["reward_scan"] = {"bound": "hbm", "achieved": scan_bytes / (scan_ms / 1e3) / 1e9,
                          "peak": HBM_BYTES_PER_S / 1e9, "unit": "GB/s",
                          "frac": scan_bytes / (scan_ms / 1e3) / HBM_BYTES_PER_S,
                          "launch_ms": scan_ms, "launches": SCAN_LAUNCHES,
                          "timing": scan_timing,
                          "eager_launch_ms": scan_eager_ms, "stage_ms": stage[0]}
    out["stages_ms"] = {"reward_scan": stage[0], "error_estimate": stage[1], "outer_sum": stage[2]}
    out["outer_sum"] = outer_sum_fields(w, stage[2])
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_linear(w, c, args.cpu_seconds)
    return out


def _time_calls(torch, fn, steps: int, warmup: int) -> float:
    """ms per call of fn (work on torch's current stream), HIP events around
    `steps` back-to-back calls after `warmup` untimed ones."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def _time_graph(torch, fn, calls: int) -> float:
    """ms per call of fn, from one HIP graph of `calls` back-to-back calls
    (captured on a side stream, replayed once untimed, then timed between two
    events on the stream that replays it)."""
    fn()  # the library loads and the kernels' code objects settle before capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(calls):
            fn()
    graph.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    del graph
    return e0.elapsed_time(e1) / calls


def _row_line(args, metric, value, unit, ms, workload, roofline, extra=None):
    out = {"metric": metric, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
           "config": {"workload": workload, "parallelism": "single GPU"}, "roofline": roofline}
    out.update(extra or {})
    return out


def run_forward(args, torch, dust, synth):
    """Perturbed forward of the hidden layer (512 -> 2048 over 8 x 2048 tokens),
    8 draws per call: one bf16 product reused for every draw, the noise added
    in the epilogue.  Bound by writing Y (4 B per token-column-draw)."""
    T, d, N, nd = 16384, 512, 2048, 8
    gen = torch.Generator().manual_seed(11)
    X = (torch.randn(T, d, generator=gen) / d ** 0.5).to(torch.bfloat16).cuda()
    W = (torch.randn(N, d, generator=gen) / d ** 0.5).to(torch.bfloat16).cuda()
    Y = torch.empty((nd, T, N), dtype=torch.float32, device="cuda:0")
    ms = _time_calls(torch, lambda: dust.perturbed_linear(X, W, sigma=0.01, seed=1, ndraw=nd,
                                                          out=Y), args.steps, args.warmup)
    ybytes = 4.0 * nd * T * N
    in_bytes = 2.0 * (T * d + N * d)
    gbs = (ybytes + in_bytes) / (ms / 1e3) / 1e9
    slots = float(nd) * T * N * (SLOTS_PER_NORMAL_ERROR_ESTIMATE) / (ms / 1e3) / 1e12
    roof = {"bound": "hbm", "kernel": "perturbed_linear_kernel (bf16 MFMA product + noise "
            "epilogue)", "achieved": gbs, "peak": HBM_BYTES_PER_S / 1e9, "unit": "GB/s",
            "frac": gbs * 1e9 / HBM_BYTES_PER_S, "traffic": None, "launch_ms": ms,
            "valu_slots_tps": slots, "valu_frac": slots * 1e12 / VALU_SLOTS_PER_S,
            "gemm_tflops": 2.0 * T * N * d / (ms / 1e3) / 1e12}
    return _row_line(args, "token-draws/sec, perturbed forward y = W x + sigma a "
                     f"(T={T}, d={d}, N={N})", T * nd / (ms / 1e3), "token-draws/s", ms,
                     f"forward: bf16 X [{T},{d}], W [{N},{d}], {nd} draws per call, Y fp32",
                     roof)


def run_embedding(args, torch, dust, synth):
    """Embedding estimate at the pages' shape: 16384 token ids (Zipf over a
    4096-token vocabulary), error estimates of width 512."""
    import numpy as np
    T, N, vocab = 16384, 512, 4096
    rng = np.random.default_rng(5)
    ids = torch.from_numpy(synth.zipf_targets(rng, T, vocab)).cuda()
    g = torch.from_numpy(rng.standard_normal((T, N)).astype(np.float32)).cuda()
    G = torch.empty((vocab, N), dtype=torch.float32, device="cuda:0")
    ws = torch.empty(dust._lib.load().dust_embedding_workspace_size(T, N, vocab), dtype=torch.uint8,
                     device="cuda:0")
    ms = _time_calls(torch, lambda: dust.embedding_grad(ids, g, vocab, out=G, workspace=ws),
                     args.steps, args.warmup)
    nbytes = 4.0 * T * N + 4.0 * vocab * N + 4.0 * T
    gbs = nbytes / (ms / 1e3) / 1e9
    roof = {"bound": "hbm", "kernel": "sort/segment/finish (dust_embedding_grad)",
            "achieved": gbs, "peak": HBM_BYTES_PER_S / 1e9, "unit": "GB/s",
            "frac": gbs * 1e9 / HBM_BYTES_PER_S, "traffic": None, "launch_ms": ms}
    return _row_line(args, f"tokens/sec, embedding estimate G_E (T={T}, N={N}, vocab={vocab})",
                     T / (ms / 1e3), "tokens/s", ms,
                     f"embedding: {T} Zipf(1.1) ids over {vocab}, g fp32 [{T},{N}]", roof)


def run_optim(args, torch, dust, synth):
    """SGD + momentum and Adam steps over 2^24 fp32 parameters (the order of
    the pages' 8 x 512 model)."""
    n = 1 << 24
    gen = torch.Generator(device="cuda:0").manual_seed(13)
    W = torch.randn(n, device="cuda:0", generator=gen)
    G = torch.randn(n, device="cuda:0", generator=gen)
    m = torch.zeros(n, device="cuda:0")
    v = torch.zeros(n, device="cuda:0")
    ms_sgd = _time_calls(torch, lambda: dust.sgd_momentum_(W, G, m, lr=1e-3, momentum=0.9),
                         args.steps, args.warmup)
    ms_adam = _time_calls(torch, lambda: dust.adam_(W, G, m, v, lr=1e-3, step=3),
                          args.steps, args.warmup)
    gbs_sgd = 20.0 * n / (ms_sgd / 1e3) / 1e9
    gbs_adam = 28.0 * n / (ms_adam / 1e3) / 1e9
    roof = {"bound": "hbm", "kernel": "adam_kernel", "achieved": gbs_adam,
            "peak": HBM_BYTES_PER_S / 1e9, "unit": "GB/s", "frac": gbs_adam * 1e9 / HBM_BYTES_PER_S,
            "traffic": None, "launch_ms": ms_adam}
    return _row_line(args, f"parameters/sec, Adam step on the estimate (n={n})",
                     n / (ms_adam / 1e3), "params/s", ms_adam,
                     f"optim: {n} fp32 parameters, 28 B (Adam) / 20 B (SGD) per parameter", roof,
                     {"sgd_momentum": {"ms": ms_sgd, "achieved_gbs": gbs_sgd,
                                       "frac": gbs_sgd * 1e9 / HBM_BYTES_PER_S}})


def run_cosine(args, torch, dust, synth):
    """The cosine-versus-population measurement at the paper shape: cosine of
    g_hat (and of G_W) with the closed-form head gradient for K = 64 .. 16384,
    and the fit of cos(K) = c_max / sqrt(1 + c/K), at the paper's sigma and at
    two large ones where the Gaussian smoothing of the loss shows (the
    first-order analysis predicts c = V + 1 and c_max -> 1 as sigma -> 0)."""
    from activation_perturbation_estimator_amd.cosine import cosine_sweep
    w = synth.WORKLOADS["paper"]
    z, y, X = synth.workload_inputs(w)
    zc, yc, Xc = z.cuda(), y.cuda(), X.cuda()
    t0 = time.perf_counter()
    sweeps = {}
    for sigma in (w.sigma, 1.0, 4.0):
        sweeps[str(sigma)] = cosine_sweep(zc, yc, Xc, [64, 256, 1024, 4096, 16384], sigma=sigma,
                                          seed=1, seq_len=w.seq_len)
    dt = time.perf_counter() - t0
    res = sweeps[str(w.sigma)]
    return {"metric": "cosine of g_hat with softmax(z) - onehot(y) versus population K",
            "value": res["fit_token"]["c"], "unit": "fitted c (law cos = c_max / sqrt(1 + c/K))",
            "n_gpus": 1, "data": "synthetic", "dtype": "f32", "higher_is_better": False,
            "config": {"workload": f"paper shape, T={w.T}, V={w.V}, sigma={w.sigma} (and 1, 4), "
                                   "K = 64, 256, 1024, 4096, 16384"},
            "sweep": res, "sweeps_by_sigma": sweeps, "predicted_c": w.V + 1, "wall_s": dt}


ROWS = {"forward": run_forward, "embedding": run_embedding, "optim": run_optim,
        "cosine": run_cosine}


# The default line's sub-records: the LM head at K = 1024, the public code's
# default population (K = 16384, the largest single-GPU head workload) and the
# hidden-layer estimator, each with its own roofline and oracle baseline
# (steps, oracle seconds).
SUB_WORKLOADS = (("k1024", 5, 4.0), ("k16384", 3, 4.0), ("linear", 10, 4.0))
SUB_KEEP = ("metric", "value", "unit", "ms_per_step", "steps", "warmup", "config", "roofline",
            "stages_ms", "outer_sum", "reward_scan", "cpu_baseline")


def run_sub_workloads(args, torch, dust, synth):
    import copy
    subs = {}
    for name, steps, cpu_s in SUB_WORKLOADS:
        a = copy.copy(args)
        a.steps, a.warmup, a.cpu_seconds, a.copy_probe_mib = steps, 1, cpu_s, 0
        w = synth.WORKLOADS[name]
        run = run_linear if w.kind == "linear" else run_head
        print(f"[bench] {name}: {steps} steps", file=sys.stderr, flush=True)
        rec = run(a, torch, dust, synth, w)
        subs[name] = {k: v for k, v in rec.items() if k in SUB_KEEP}
    return subs


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "bench.py measures one GPU; libdust has no multi-GPU path "
                                   "(the estimator would shard by sequence, with one sum "
                                   "all-reduce of G_W)", "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    import activation_perturbation_estimator_amd as dust
    from activation_perturbation_estimator_amd import synth

    if args.workload in ROWS:
        print(json.dumps(ROWS[args.workload](args, torch, dust, synth)), flush=True)
        return
    w = synth.WORKLOADS[args.workload]
    run = run_linear if w.kind == "linear" else run_head
    rec = run(args, torch, dust, synth, w)
    if args.workload == "paper" and not args.no_sub_workloads:
        rec["workloads"] = run_sub_workloads(args, torch, dust, synth)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
