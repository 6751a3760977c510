"""Benchmark: chunkwise KDA forward, B=2 H=32 T=8192 dk=dv=128 C=64, bf16, one MI355X.

One step = one gdr_chunk_fwd call over the whole batch: the whole hot path (gate
prefix sums, UT transform and WY factors in the chunk-parallel kernel; the serial
state pass and the output in the state kernel), on seeded synthetic inputs already
resident in HBM.  Prints one JSON line.

Throughput is tokens/s (B*T / mean step time; a token carries all H heads).  The
roofline entry treats the call (all its launches) as the unit: algorithmic bytes
per call (read q, k, v, log alpha, beta; write O and S_final) over the mean call
duration measured with HIP events on the launch stream, against 8 TB/s.  HBM
traffic and MFMA-busy figures come from the committed rocprofv3 counter summary,
and only while the kernel source still matches the one it was measured on.  The
CPU baseline is the fp64 oracle on the host cores.

Before the W warm-up steps the call is repeated untimed for at least --settle-ms of
device time (60 by default; the count is reported under "settle"), so that the timed
steps do not fall in the GPU's power-management transient after idle.
"""
import argparse
import hashlib
import json
import os
import platform
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
WORKLOAD = "kda"
# The headline kernels' source: the kernel file, the device headers it includes and the
# build script (its compiler flags shape the code as much as the source does).
KERNEL_SOURCES = ["chunkwise_gated_delta_amd/csrc/gdr_kda_split.hip",
                  "chunkwise_gated_delta_amd/csrc/gdr_mfma.h",
                  "chunkwise_gated_delta_amd/csrc/gdr_split_common.h",
                  "chunkwise_gated_delta_amd/csrc/gdr_common.h",
                  "chunkwise_gated_delta_amd/build.py"]
COUNTERS_FILE = "profiles/kda_split__kda_B2_H32_T8192_d128__counters.md"


def kernel_source_sha():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def committed_counters():
    """Figures from the committed counter summary, or {} when the kernels changed since.

    The summary records the sha256 of the kernel source it was measured on and a few
    machine-readable lines `key: value`.
    """
    try:
        text = open(os.path.join(ROOT, COUNTERS_FILE)).read()
    except OSError:
        return {}
    m_sha = re.search(r"Kernel source sha256 `([0-9a-f]{64})`", text)
    if not m_sha or m_sha.group(1) != kernel_source_sha():
        return {}
    out = {}
    for key in ("traffic_bytes_per_launch", "mfma_busy_frac"):
        m = re.search(rf"^{key}: ([0-9.eE+-]+)$", text, re.M)
        if m:
            out[key] = float(m.group(1))
    return out


def algorithmic_counts(P):
    """(bytes, flops) one call must move / perform at the algorithmic minimum.

    Bytes per token-head: q, k, v, O at 2*d each (bf16), log alpha 4*dk, beta 4;
    plus S_final (and S0 if given) once per (sequence, head).
    FLOP per token-head: 10*C*d + 6*d^2 -- five C x C x d products (K<-K->^T,
    At K<-, At V, Q<-K->^T, A_qk V_new) and three C x d x d products (W S^T,
    V_new^T K^, Q<- S^T), counted as full tiles.  With a and b (DPLR) the call also
    reads a, b (2*dk each) and does 18*C*d + 8*d^2.  Counting only the lower triangles
    of the C x C factors gives 5*(C+1)*d + 6*d^2 (DPLR: 9*(C+1)*d + 8*d^2), the third
    value returned.
    """
    th = P.B * P.T * P.H
    d, C = P.dk, P.chunk
    es = 2 if P.dtype.itemsize == 2 else 4
    gate_bytes = {0: 0, 1: 4, 2: 4 * P.dk}[P.gate]
    per_th = es * (2 * P.dk + 2 * P.dv) + gate_bytes + 4
    flops_th = 10 * C * d + 6 * d * d
    tri_th = 5 * (C + 1) * d + 6 * d * d
    if P.a is not None:
        per_th += 2 * es * P.dk
        flops_th = 18 * C * d + 8 * d * d
        tri_th = 9 * (C + 1) * d + 8 * d * d
    state = P.n_seq * P.H * P.dv * P.dk * 4 * (1 + (P.S0 is not None))
    return th * per_th + state, th * flops_th, th * tri_th


def settle(call, settle_ms):
    """Repeat `call` untimed until `settle_ms` of device time have passed; returns the count.

    A GPU that has been idle runs the first ~30 ms of this load through a power-management
    transient: per-call times rise by ~15% around the tenth call and return to the steady
    value by about the fiftieth (kernel traces of the first 400 calls on MI355X).  A short
    warm-up followed by a short timed window would measure that transient, not the kernels;
    the settle phase precedes the warm-up steps, which are then run and timed as asked.
    """
    import torch

    if settle_ms <= 0:
        return 0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n, batch = 0, 8
    e0.record()
    while True:
        for _ in range(batch):
            call()
        n += batch
        e1.record()
        e1.synchronize()
        if e0.elapsed_time(e1) >= settle_ms:
            return n


def time_gpu(P, steps, warmup, cold_steps, for_backward=False, settle_ms=0.0):
    import torch

    from chunkwise_gated_delta_amd import gdr

    dev = torch.device("cuda", 0)
    to = lambda t: None if t is None else t.to(dev)
    q, k, v, beta, la = to(P.q), to(P.k), to(P.v), to(P.beta), to(P.log_alpha)
    a, b, S0, cu = to(P.a), to(P.b), to(P.S0), to(P.cu_seqlens)
    out = torch.empty((P.B, P.T, P.H, P.dv), dtype=P.dtype, device=dev)
    fin = torch.empty((P.n_seq, P.H, P.dv, P.dk), dtype=torch.float32, device=dev)
    ws = None
    if for_backward:
        # the forward of a training step: it also keeps the per-chunk states for the backward
        n_seq = 0 if cu is None else P.n_seq
        gate = gdr.GATE_NONE if la is None else (gdr.GATE_HEAD if la.dim() == 3 else gdr.GATE_CHANNEL)
        ws = torch.zeros(gdr.bwd_workspace_bytes(P.B, P.H, P.T, P.dk, P.dv, n_seq=n_seq, gate=gate,
                                                 has_ab=a is not None), dtype=torch.uint8, device=dev)
    call = lambda: gdr.chunk_fwd(q, k, v, beta, log_alpha=la, a=a, b=b, S0=S0, cu_seqlens=cu,
                                 chunk_size=P.chunk, out=out, final_state=fin, clip=P.clip,
                                 workspace=ws, for_backward=for_backward)
    n_settle = settle(call, settle_ms)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)
    ev0, ev1 = ev(), ev()
    per = []
    ev0.record(stream)
    for _ in range(steps):
        e0, e1 = ev(), ev()
        e0.record(stream)
        call()
        e1.record(stream)
        per.append((e0, e1))
    ev1.record(stream)
    torch.cuda.synchronize()
    total_ms = ev0.elapsed_time(ev1)
    launch_ms = sorted(a.elapsed_time(b) for a, b in per)
    # cold: a 512 MB write between calls evicts the 256 MB memory-side cache
    scrub = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    cold = []
    for i in range(cold_steps):
        scrub.fill_(i & 0xFF)
        e0, e1 = ev(), ev()
        e0.record(stream)
        call()
        e1.record(stream)
        cold.append((e0, e1))
    torch.cuda.synchronize()
    cold_ms = sorted(a.elapsed_time(b) for a, b in cold)
    del scrub
    return total_ms / steps, launch_ms, cold_ms, out, fin, n_settle


def machine_context():
    """Measured bf16 GEMM rate and device copy bandwidth on this GPU (context only)."""
    import torch

    dev = torch.device("cuda", 0)
    n = 8192
    a = torch.randn(n, n, dtype=torch.bfloat16, device=dev)
    b = torch.randn(n, n, dtype=torch.bfloat16, device=dev)
    for _ in range(3):
        a @ b
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 10
    e0.record()
    for _ in range(reps):
        a @ b
    e1.record()
    torch.cuda.synchronize()
    gemm_tflops = 2 * n ** 3 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e12
    del a, b
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * (1 << 30) * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    return {"bf16_gemm_8192_tflops": gemm_tflops, "copy_1GiB_read_plus_write_gbs": copy_gbs}


def cpu_baseline(P, n_threads):
    """fp64 oracle on the whole workload (all host threads) and on a 2-chain sample (1 thread)."""
    import numpy as np
    import torch

    import oracle

    f64 = lambda t: None if t is None else t.to(torch.float64).numpy()
    args = dict(q=f64(P.q), k=f64(P.k), v=f64(P.v), beta=f64(P.beta),
                log_alpha=f64(P.log_alpha), a=f64(P.a), b=f64(P.b), S0=f64(P.S0),
                cu_seqlens=None if P.cu_seqlens is None else P.cu_seqlens.numpy(), clip=P.clip)
    # The whole workload, repeated until at least a second has passed (small workloads).
    reps, t = 0, time.perf_counter()
    while True:
        O, Sf = oracle.recurrence(**args, n_threads=n_threads)
        reps += 1
        if time.perf_counter() - t >= 1.0 or reps >= 1000:
            break
    dt = (time.perf_counter() - t) / reps
    chains = [(0, 0), (min(1, P.n_seq - 1), min(5, P.H - 1))]
    if P.cu_seqlens is None:
        chain_tokens = len(chains) * P.T
    else:
        lens = np.diff(P.cu_seqlens.numpy())
        chain_tokens = int(sum(lens[n] for n, _ in chains))
    reps1, t = 0, time.perf_counter()
    while True:
        oracle.recurrence(**args, chains=chains, n_threads=1)
        reps1 += 1
        if time.perf_counter() - t >= 0.3 or reps1 >= 1000:
            break
    dt1 = (time.perf_counter() - t) / reps1
    return dt, reps, dt1, chain_tokens, O, Sf


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def backward_counts(P):
    """(bytes, flops) of one backward call at the algorithmic minimum.

    Bytes per token-head: read q, k, v, dO (es*d each), log alpha (4*dk channel gate,
    4 head gate), beta 4; write dq, dk, dv (es*d each), dlog alpha (as log alpha),
    dbeta 4; plus S0, dS_final read and dS0 written once per (sequence, head).
    FLOP per token-head, the chunk products of the backward notes as full tiles:
    30*C*d + 10*d^2 + 4*C^2 (the per-chunk gradients: fifteen C x C x d and five
    C x d x d products, two C x C x C), 6*d^2 (the reverse state pass) and the
    forward quantities it recomputes, 10*C*d + 6*d^2.  With a and b (DPLR) the call
    also reads a, b and writes da, db (es*d each), and the per-chunk gradients are
    44*C*d + 14*d^2 + 10*C^2 (twenty-two C x C x d, seven C x d x d and five
    C x C x C products), plus the DPLR forward recompute, 18*C*d + 8*d^2.
    """
    th = P.B * P.T * P.H
    d, C = P.dk, P.chunk
    es = 2 if P.dtype.itemsize == 2 else 4
    gate_bytes = {0: 0, 1: 4, 2: 4 * P.dk}[P.gate]
    per_th = es * (2 * P.dk + 2 * P.dv) + es * (2 * P.dk + P.dv) + 2 * gate_bytes + 8
    state = P.n_seq * P.H * P.dv * P.dk * 4 * (2 + (P.S0 is not None))
    flops_th = 30 * C * d + 10 * d * d + 4 * C * C + 6 * d * d + 10 * C * d + 6 * d * d
    if P.a is not None:
        per_th += 4 * es * P.dk
        flops_th = 44 * C * d + 14 * d * d + 10 * C * C + 6 * d * d + 18 * C * d + 8 * d * d
    return th * per_th + state, th * flops_th


def bench_backward(args):
    """Time gdr_chunk_bwd on a workload; one JSON line."""
    import numpy as np
    import torch

    from chunkwise_gated_delta_amd import gdr, inputs

    P = inputs.make_problem(args.workload)
    dO, dSf = inputs.make_cotangents(P, seed=100)
    dev = torch.device("cuda", 0)
    to = lambda t: None if t is None else t.to(dev)
    q, k, v, beta, la = to(P.q), to(P.k), to(P.v), to(P.beta), to(P.log_alpha)
    a, b = to(P.a), to(P.b)
    S0, cu, dOd, dSd = to(P.S0), to(P.cu_seqlens), to(dO), to(dSf)
    ws = None
    if args.train_step:
        args.forward_states = True
    if args.forward_states:
        args.forward_workspace = True
    if args.forward_workspace:
        # the backward of a training step: the forward call's workspace (its per-chunk
        # factors) is handed to the backward, which then skips recomputing them
        n_seq = 0 if cu is None else P.n_seq
        gate = gdr.GATE_NONE if la is None else (gdr.GATE_HEAD if la.dim() == 3 else gdr.GATE_CHANNEL)
        need = max(gdr.workspace_bytes(P.B, P.H, P.T, P.dk, P.dv, n_seq=n_seq, gate=gate, has_ab=a is not None),
                   gdr.bwd_workspace_bytes(P.B, P.H, P.T, P.dk, P.dv, n_seq=n_seq, gate=gate,
                                           has_ab=a is not None))
        ws = torch.zeros(need, dtype=torch.uint8, device=dev)
        gdr.chunk_fwd(q, k, v, beta, log_alpha=la, a=a, b=b, S0=S0, cu_seqlens=cu,
                      chunk_size=P.chunk, workspace=ws, for_backward=args.forward_states)
    bwd = lambda: gdr.chunk_bwd(q, k, v, beta, dOd, log_alpha=la, a=a, b=b, S0=S0,
                                dS_final=dSd, cu_seqlens=cu, chunk_size=P.chunk, workspace=ws,
                                forward_workspace=args.forward_workspace,
                                forward_states=args.forward_states)
    if args.train_step:
        # one training step of the layer: the forward that keeps its states, then the backward
        def call():
            gdr.chunk_fwd(q, k, v, beta, log_alpha=la, a=a, b=b, S0=S0, cu_seqlens=cu,
                          chunk_size=P.chunk, workspace=ws, for_backward=True)
            return bwd()
    else:
        call = bwd
    n_settle = settle(call, args.settle_ms)
    for _ in range(args.warmup):
        g = call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)
    ev0, ev1 = ev(), ev()
    per = []
    ev0.record(stream)
    for _ in range(args.steps):
        e0, e1 = ev(), ev()
        e0.record(stream)
        g = call()
        e1.record(stream)
        per.append((e0, e1))
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    launch_ms = sorted(a.elapsed_time(b) for a, b in per)
    call_ms = float(np.mean(launch_ms))
    alg_bytes, alg_flops = backward_counts(P)
    if args.train_step:
        fb, ff, _ = algorithmic_counts(P)
        alg_bytes, alg_flops = alg_bytes + fb, alg_flops + ff
    tokens = P.B * P.T
    gbs = alg_bytes / (call_ms * 1e-3) / 1e9
    tflops = alg_flops / (call_ms * 1e-3) / 1e12
    result = {
        "metric": (f"tokens/s, {args.workload} chunk training step (forward keeping its states, "
                   "then all input gradients), 1xMI355X" if args.train_step else
                   f"tokens/s, {args.workload} chunk bwd (all input gradients"
                   f"{', forward states reused' if args.forward_states else (', forward workspace reused' if args.forward_workspace else '')}), 1xMI355X"),
        "value": tokens / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{args.workload} backward: B={P.B} H={P.H} T={P.T} dk={P.dk} "
                               f"dv={P.dv} C={P.chunk} n_seq={P.n_seq}, seeded dO and dS_final"},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "gdr_chunk_bwd call (all launches)", "call_ms_mean": call_ms,
                     "alg_bytes_per_launch": alg_bytes},
        "mfma": {"alg_flops_per_launch": alg_flops, "achieved_tflops": tflops,
                 "peak_tflops": BF16_MFMA_PEAK_TFLOPS, "frac": tflops / BF16_MFMA_PEAK_TFLOPS},
        "settle": {"calls": n_settle, "device_ms_min": args.settle_ms,
                   "note": "untimed calls before the warm-up steps (power-management transient)"},
    }
    if not args.no_cpu:
        import oracle

        f64 = lambda t: None if t is None else t.to(torch.float64).numpy()
        chains = [(0, 0), (min(1, P.n_seq - 1), min(5, P.H - 1))]
        cu_np = None if P.cu_seqlens is None else P.cu_seqlens.numpy()
        t = time.perf_counter()
        ref = oracle.recurrence_bwd(f64(P.q), f64(P.k), f64(P.v), f64(P.beta), f64(dO),
                                    log_alpha=f64(P.log_alpha), a=f64(P.a), b=f64(P.b),
                                    S0=f64(P.S0), dS_final=f64(dSf),
                                    cu_seqlens=cu_np, chains=chains, n_threads=2)
        dt = time.perf_counter() - t
        if cu_np is None:
            chain_tokens = len(chains) * P.T
        else:
            lens = np.diff(cu_np)
            chain_tokens = int(sum(lens[n] for n, _ in chains))
        # a token carries all H heads: chain tokens / H of them per second, scaled to the
        # two threads that ran the two chains
        result["cpu_baseline"] = {
            "value": chain_tokens / dt / P.H, "unit": "tokens/s", "cores": 2, "kind": "oracle",
            "sample": f"2 (sequence, head) chains ({chain_tokens} token-heads) of the workload, "
                      f"fp64 reverse pass with checkpoint replay, {dt:.2f} s on 2 threads"}
        errs = {}
        for key, val in g.items():
            gk = val.to(torch.float64).cpu().numpy()
            if key == "dS0":
                a = np.concatenate([gk[n, h].ravel() for n, h in chains])
                b = np.concatenate([ref[key][n, h].ravel() for n, h in chains])
            elif P.cu_seqlens is None:
                a = np.concatenate([gk[n, :, h].ravel() for n, h in chains])
                b = np.concatenate([ref[key][n, :, h].ravel() for n, h in chains])
            else:
                a = np.concatenate([gk[0, cu_np[n]:cu_np[n + 1], h].ravel() for n, h in chains])
                b = np.concatenate([ref[key][0, cu_np[n]:cu_np[n + 1], h].ravel() for n, h in chains])
            errs[key + "_rel_err"] = float(np.max(np.abs(a - b)) / np.max(np.abs(b)))
        result["parity"] = dict(errs, tol=inputs.TOLERANCE[P.dtype], chains=chains)
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--workload", default=WORKLOAD, choices=["kda", "gdn", "dplr", "kda_varlen",
                                                              "deltanet_f32", "gdn2_clip", "kda_strong"],
                    help="the benchmark line is for kda; the others time the same call on the "
                         "other workloads (reported under the same keys, metric named per workload)")
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cold-steps", type=int, default=10)
    ap.add_argument("--settle-ms", type=float, default=60.0,
                    help="before the warm-up steps, repeat the call untimed until this much device "
                         "time has passed (the GPU's power-management transient after idle); 0: off")
    ap.add_argument("--chunk", type=int, default=64, choices=[64, 128],
                    help="forward chunk size C (128: bf16 without a, b at dk = 128 only)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the GEMM / copy context measurements")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward pass (gdr_chunk_bwd) on the workload instead")
    ap.add_argument("--forward-workspace", action="store_true",
                    help="with --backward: hand the backward the workspace of a forward call on "
                         "the same inputs (GDR_BWD_FORWARD_WORKSPACE), as a training step does")
    ap.add_argument("--for-backward", action="store_true",
                    help="forward only: time gdr_chunk_fwd_for_bwd (the forward of a training "
                         "step, which also keeps the per-chunk states for the backward)")
    ap.add_argument("--train-step", action="store_true",
                    help="with --backward: time a whole training step of the layer "
                         "(gdr_chunk_fwd_for_bwd, then gdr_chunk_bwd on its states)")
    ap.add_argument("--forward-states", action="store_true",
                    help="with --backward: the forward call also kept its per-chunk states "
                         "(gdr_chunk_fwd_for_bwd, GDR_BWD_FORWARD_STATES)")
    ap.add_argument("--copy-cal", action="store_true",
                    help="run only a plain 1 GiB device-to-device copy (calibrates the HBM "
                         "traffic counters: FETCH_SIZE/WRITE_SIZE per byte actually moved)")
    args = ap.parse_args()
    if args.copy_cal:
        import torch

        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "copies": args.steps}))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); each (sequence, head) "
              "chain is independent, so N GPUs would each run this path on H/N heads.",
              file=sys.stderr)
        sys.exit(2)

    if args.backward:
        if args.chunk != 64:
            print("the backward pass runs with C = 64 only", file=sys.stderr)
            sys.exit(2)
        bench_backward(args)
        return

    import numpy as np
    import torch

    from chunkwise_gated_delta_amd import inputs

    P = inputs.make_problem(args.workload, chunk=args.chunk)
    alg_bytes, alg_flops, tri_flops = algorithmic_counts(P)
    ms, launch_ms, cold_ms, out, fin, n_settle = time_gpu(
        P, args.steps, args.warmup, args.cold_steps, for_backward=args.for_backward,
        settle_ms=args.settle_ms)
    call_ms = float(np.mean(launch_ms))
    tokens = P.B * P.T  # packed total for the varlen workload (B = 1)
    achieved_gbs = alg_bytes / (call_ms * 1e-3) / 1e9
    tflops = alg_flops / (call_ms * 1e-3) / 1e12
    headline = args.workload == WORKLOAD and not args.for_backward and args.chunk == 64
    cc = committed_counters() if headline else {}
    traffic = cc.get("traffic_bytes_per_launch")
    pct = lambda xs, f: xs[min(len(xs) - 1, int(f * len(xs)))]

    result = {
        "metric": ("tokens/s + MFMA util % for KDA chunk fwd, T=8192 H=32 d=128, 1xMI355X"
                   if headline else f"tokens/s, {args.workload} chunk fwd"
                   f"{'' if P.chunk == 64 else f' C={P.chunk}'}"
                   f"{' keeping the states for the backward' if args.for_backward else ''}, 1xMI355X"),
        "value": tokens / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if P.dtype == torch.float32 else "bf16",
        "data": "synthetic",
        "config": {"workload": ("KDA chunkwise forward (per-channel gate), B=2 H=32 T=8192 "
                                "dk=dv=128 C=64, bf16 q/k/v, fp32 gate/beta/state, S0=0"
                                if headline else f"{args.workload}: B={P.B} H={P.H} T={P.T} "
                                f"dk={P.dk} dv={P.dv} C={P.chunk} n_seq={P.n_seq}"),
                   "global_batch": P.B, "seq_len": P.T, "heads": P.H, "dk": P.dk, "dv": P.dv,
                   "chunk": P.chunk, "parallelism": "none (one GPU)"},
        "roofline": {"bound": "hbm", "achieved": achieved_gbs, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved_gbs / HBM_PEAK_GBS,
                     "traffic": None if traffic is None else int(traffic),
                     "kernel": ("gdr_chunk_fwd call: kda_prep_kernel<128, channel gate> + its "
                                "log-domain pass (flag scan) + kda_state_kernel<128>"
                                if headline else "gdr_chunk_fwd call"),
                     "call_ms_mean": call_ms, "call_ms_median": pct(launch_ms, 0.5),
                     "call_ms_p10": pct(launch_ms, 0.1), "call_ms_p90": pct(launch_ms, 0.9),
                     "call_ms_cold_mean": float(np.mean(cold_ms)) if cold_ms else None,
                     "alg_bytes_per_launch": alg_bytes},
        "mfma": {"alg_flops_per_launch": alg_flops, "achieved_tflops": tflops,
                 "peak_tflops": BF16_MFMA_PEAK_TFLOPS, "frac": tflops / BF16_MFMA_PEAK_TFLOPS,
                 "lower_triangle_flops_per_launch": tri_flops,
                 "frac_lower_triangle": tri_flops / (call_ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS,
                 "counter_busy_frac": cc.get("mfma_busy_frac")},
        "settle": {"calls": n_settle, "device_ms_min": args.settle_ms,
                   "note": "untimed calls before the warm-up steps (power-management transient)"},
    }
    if not args.no_context:
        result["context"] = machine_context()
    if not args.no_cpu:
        import oracle

        n_threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or oracle.max_threads()
        dt, reps, dt1, chain_tokens, Oref, Sref = cpu_baseline(P, n_threads)
        Og = out.to(torch.float64).cpu().numpy()
        Sg = fin.to(torch.float64).cpu().numpy()
        result["cpu_baseline"] = {
            "value": tokens / dt, "unit": "tokens/s", "cores": n_threads, "kind": "oracle",
            "sample": f"the whole workload ({P.n_seq * P.H} (sequence, head) chains, {tokens} tokens), "
                      f"fp64 token recurrence, {dt * 1e3:.1f} ms per pass on {n_threads} threads "
                      f"(mean of {reps}); one thread: 2 chains ({chain_tokens} tokens) in "
                      f"{dt1 * 1e3:.1f} ms = {chain_tokens / dt1 / P.H:.0f} tokens/s "
                      f"(a token = all {P.H} heads)",
            "cpu_model": cpu_model(), "nproc": os.cpu_count()}
        result["parity"] = {
            "O_rel_err": float(np.max(np.abs(Og - Oref)) / np.max(np.abs(Oref))),
            "S_final_rel_err": float(np.max(np.abs(Sg - Sref)) / np.max(np.abs(Sref))),
            "tol": inputs.TOLERANCE[P.dtype]}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
