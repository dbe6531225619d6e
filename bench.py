#!/usr/bin/env python3
"""Benchmark of the tree-based invariant kernels on one MI355X.

Headline step (the LM-head logprob workload): one pass of the logprob path
over a batch of M = 512 tokens -- the LM-head GEMM A [512, 4096] x
W [151936, 4096]^T (bf16, A ~N(0,1), W ~N(0,0.02); 64-wide K-block MFMA
leaves and the fixed fp32 tree; exact row maxima of each 64-column block in
its epilogue), then the tree log-softmax over the vocabulary as tp = 4
simulated vocabulary shards and the gather of the uniform random targets'
log-probabilities.  value = 2*M*V*K / step time (TFLOP/s of the invariant
GEMM, the log-softmax's time included).  Inputs are resident in HBM; W
(1.24 GB) is far larger than the 256 MB last-level cache.

The roofline object is for the dominant kernel, the LM-head GEMM (bound by
the matrix cores: 408 FLOP/B against a ridge of 312), timed back to back
with HIP events on its launch stream; hipBLASLt (torch's bf16 GEMM with an
fp32 output) on the same shape gives the non-invariant baseline and the
overhead.  Also reported: bitwise mismatches across tp and batch size,
SHA-256 fingerprints of the inputs and outputs, the library's own ceiling
microbenchmarks, the other workloads (down projection at simulated tp = 8
and tp = 1, prefill, row kernels, decoder, training side), and the CPU
oracle timed on bounded samples of every workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extra] [--no-cpu]
       python bench.py --profile lmhead|rows|downproj|decode|calib   (a few launches, for rocprofv3)
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
METRIC = "invariant GEMM TFLOP/s (% MFMA peak, overhead vs hipBLASLt); 0 bit mismatches"
M_HEAD, K_HEAD, V_HEAD, TP_HEAD = 512, 4096, 151936, 4

# The headline's LM-head GEMM kernel, as named in a rocprofv3 kernel trace.
HEAD_KERNEL = "k_gemm_ring<4, 2, 2, 4, 4, 2, false, 8, 1, 0, 3, 1, 1>"
# HBM bytes per launch of HEAD_KERNEL from two rocprofv3 --pmc runs of
# `bench.py --profile lmhead` (profiles/k_gemm_ring_lmhead_M512_K4096_N151936.md):
# FETCH_SIZE 1035959 KiB x 2.000 + WRITE_SIZE 339916 KiB x 1.000, the factors
# being what a plain 1 GiB device copy reads on the same counters
# (`bench.py --profile calib`: 524301 KiB fetched, 1048576 KiB written).  Valid
# only for the GEMM sources the counters were taken on (hash below).
HEAD_TRAFFIC_BYTES = (1035959 * 2 + 339916) * 1024
HEAD_TRAFFIC_SRC_SHA256 = "0bab4607a51a99695a34e69afac4925578617c55c219b1cb5435d7388f3232da"
# The same for the down projection's tp = 8 shard-partials kernel (profiles/
# k_gemm_ring_downproj_M256_K14336_N4096_tp8.md): FETCH_SIZE 64794 KiB x 2.000
# + WRITE_SIZE 32768 KiB x 1.000.
HEAD_TP8_TRAFFIC_BYTES = (64794 * 2 + 32768) * 1024
HEAD_TP8_TRAFFIC_SRC_SHA256 = "0bab4607a51a99695a34e69afac4925578617c55c219b1cb5435d7388f3232da"


def gemm_source_sha256(root):
    h = hashlib.sha256()
    for f in ("gemm.hip", "tbik_device.h", "tbik_internal.h"):
        with open(os.path.join(root, "tp_invariant_numerics_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def sha256_of(*ts):
    """SHA-256 of the bytes of device or host tensors (the inputs' and
    outputs' fingerprints)."""
    import torch
    h = hashlib.sha256()
    for t in ts:
        h.update(t.detach().contiguous().view(-1).view(torch.uint8).cpu().numpy().tobytes())
    return h.hexdigest()


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-extra", action="store_true", help="headline step only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baselines")
    ap.add_argument("--profile", default="",
                    choices=["", "lmhead", "rows", "downproj", "decode", "calib", "ringcopy"],
                    help="run only a few launches of one group of kernels, for rocprofv3: "
                         "lmhead (the headline's GEMM and log-softmax), rows (RMSNorm, RoPE, "
                         "SwiGLU, standalone log-softmax), downproj (tp = 8 partials + combine), "
                         "decode (tp = 1 down projection at M = 1 and M = 32), "
                         "calib (a plain 1 GiB device copy, the counters' byte scale)")
    ap.add_argument("--only", default="", help="run only one extra workload (profiling)")
    return ap.parse_args()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the tensor-parallel shards are simulated on a "
              "single MI355X (no collectives); run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    root = os.path.dirname(os.path.abspath(__file__))
    if root not in sys.path:
        sys.path.insert(0, root)
    import tp_invariant_numerics_amd as tb
    from tp_invariant_numerics_amd import inputs

    if not os.path.exists(tb._build.LIB):
        import __graft_entry__
        __graft_entry__.build()
    tb.lib()
    dev = "cuda"
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()

    def log(*a):
        print(*a, file=sys.stderr, flush=True)

    if args.profile == "calib":
        # plain copy kernel of known size for FETCH_SIZE / WRITE_SIZE scaling
        nbytes = 1 << 30
        src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("pmc-calib: copied %d bytes x5" % nbytes)
        return
    if args.profile == "ringcopy":
        # the ring-copy microbenchmark from a 1 MiB, a 32 MiB and a 1 GiB
        # window, one launch each (256 workgroups x 1024 stages of 32 KB)
        buf = torch.empty((1 << 30,), dtype=torch.uint8, device=dev).fill_(3)
        out = torch.empty((256 * 512,), dtype=torch.int32, device=dev)
        for win in (1 << 20, 32 << 20, 1 << 30):
            tb.tbik_bench_copy_lds(buf, win, 1024, 256, out=out)
        torch.cuda.synchronize()
        log("profile ringcopy: 3 launches")
        return

    def timed(fn, iters, warm=3, min_ms=25.0, max_iters=1000):
        """Average ms per call of fn() over at least iters calls, HIP events on
        the stream.  A timed region shorter than min_ms is repeated with more
        calls (up to max_iters): the first launch after a synchronisation
        costs extra, which would otherwise weigh on the mean of a short loop."""
        for _ in range(warm):
            fn()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)

        def run(n):
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(n):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1)

        total = run(iters)
        n = min(max_iters, int(math.ceil(iters * min_ms / max(total, 1e-3))))
        if n > iters:
            total, iters = run(n), n
        return total / iters

    # ------------------------------------------------------------------ headline
    M, K, V, tp = M_HEAD, K_HEAD, V_HEAD, TP_HEAD
    log("inputs: A [%d,%d], W [%d,%d], targets [%d], tp=%d" % (M, K, V, K, M, tp))
    A = inputs.normal_bf16((M, K), 1001, device=dev)
    W = inputs.normal_bf16((V, K), 1002, std=0.02, device=dev)
    tgt = inputs.uniform_int(M, V, 1003, device=dev)
    logits = torch.empty((M, V), dtype=torch.float32, device=dev)
    pm = torch.empty((M, (V + 63) // 64), dtype=torch.float32, device=dev)
    lp = torch.empty((M,), dtype=torch.float32, device=dev)
    lws = torch.empty((tb.tbik_logsoftmax_workspace_bytes(M, V, tp) // 4 + 1,),
                      dtype=torch.float32, device=dev)
    flops = 2.0 * M * V * K

    def gemm():
        tb.tbik_gemm_logits(A, W, out=logits, pmax=pm)

    if args.profile:
        profile_kernels(args.profile, tb, inputs, torch, dev, log,
                        (gemm, lambda: tb.tbik_logsoftmax_gather_pmax(logits, tgt, pm, tp, ws=lws,
                                                                      out=lp)))
        return

    # One step = the config's logprob path: the LM-head GEMM with its fused
    # row maxima, then the log-softmax + gather (one read of the logits).
    # The K timed steps are bracketed by one event pair and the wall clock.
    def step():
        gemm()
        tb.tbik_logsoftmax_gather_pmax(logits, tgt, pm, tp, ws=lws, out=lp)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e_start = torch.cuda.Event(enable_timing=True)
    e_end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e_start.record(stream)
    for _ in range(args.steps):
        step()
    e_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = e_start.elapsed_time(e_end) / args.steps
    ms_per_step = max(step_ms, wall * 1e3 / args.steps)
    value = flops / (ms_per_step * 1e-3) / 1e12
    log("step %.4f ms (events), wall %.4f ms/step: %.1f TFLOP/s"
        % (step_ms, wall * 1e3 / args.steps, value))

    # the dominant kernel alone: back-to-back launches between two HIP
    # events on the launch stream
    kern_ms = timed(gemm, max(10, args.steps), warm=2)
    lsm_ms = timed(lambda: tb.tbik_logsoftmax_gather_pmax(logits, tgt, pm, tp, ws=lws, out=lp),
                   max(10, args.steps))
    log("LM-head GEMM %.4f ms per launch; log-softmax %.4f ms" % (kern_ms, lsm_ms))
    achieved = flops / (kern_ms * 1e-3) / 1e12
    gemm_bytes = M * K * 2 + V * K * 2 + M * V * 4 + M * ((V + 63) // 64) * 4
    traffic = HEAD_TRAFFIC_BYTES if (HEAD_TRAFFIC_SRC_SHA256 is not None and
                                     gemm_source_sha256(root) == HEAD_TRAFFIC_SRC_SHA256) else None
    roofline = {"kernel": HEAD_KERNEL + " (LM-head GEMM with fused 64-column row maxima)",
                "bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic, "algorithmic_flops_per_launch": flops,
                "algorithmic_bytes_per_launch": gemm_bytes,
                "arith_intensity_flop_per_byte": round(flops / gemm_bytes, 1),
                "avg_launch_ms": round(kern_ms, 5)}
    lsm_bytes = M * V * 4
    secondary = {"kernel": "k_logsoftmax_row (tree log-softmax + gather, tp=%d, row maxima "
                           "from the GEMM)" % tp, "bound": "hbm",
                 "achieved": round(lsm_bytes / lsm_ms / 1e6, 1), "peak": PEAK_HBM_GBS,
                 "unit": "GB/s", "frac": round(lsm_bytes / lsm_ms / 1e6 / PEAK_HBM_GBS, 4),
                 "algorithmic_bytes_per_launch": lsm_bytes, "avg_launch_ms": round(lsm_ms, 5)}

    # fingerprints of what this run consumed and produced
    step()
    torch.cuda.synchronize()
    fingerprints = {"A": sha256_of(A), "W": sha256_of(W), "targets": sha256_of(tgt),
                    "logits": sha256_of(logits), "row_maxima": sha256_of(pm),
                    "logprobs": sha256_of(lp)}
    lp_head = lp.clone()

    # bitwise invariance on this workload: tp 1/2/8 logprobs and sub-batches
    mismatches = 0
    checks = 0
    for t in (1, 2, 8):
        o, _ = tb.tbik_logsoftmax_gather_pmax(logits, tgt, pm, t)
        mismatches += int((o.view(torch.int32) != lp_head.view(torch.int32)).sum().item())
        checks += M
    for lo, m in ((0, 1), (511, 1), (100, 17), (0, 256)):
        lg, p2 = tb.tbik_gemm_logits(A[lo:lo + m], W)
        mismatches += int((lg.view(torch.int32) != logits[lo:lo + m].view(torch.int32)).sum().item())
        o, _ = tb.tbik_logsoftmax_gather_pmax(lg, tgt[lo:lo + m], p2, tp)
        mismatches += int((o.view(torch.int32) != lp_head[lo:lo + m].view(torch.int32)).sum()
                          .item())
        checks += m * V + m
        del lg, p2
    log("bit mismatches across tp {1,2,4,8} and batch {1,17,256,512}: %d of %d" % (mismatches,
                                                                                   checks))

    # non-invariant baseline: hipBLASLt through torch (bf16 inputs, fp32 out
    # when the backend takes it, else bf16 out)
    blas_out = "fp32"
    try:
        torch.mm(A, W.t(), out_dtype=torch.float32)
        blas = lambda: torch.mm(A, W.t(), out_dtype=torch.float32)  # noqa: E731
    except Exception:                                                # noqa: BLE001
        blas_out = "bf16"
        blas = lambda: torch.matmul(A, W.t())  # noqa: E731
    t_blas = timed(blas, max(10, args.steps), warm=2)
    t_blas_bf16 = timed(lambda: torch.matmul(A, W.t()), max(10, args.steps), warm=2)
    hipblaslt = {"what": "torch bf16 GEMM (hipBLASLt), same shape, %s output, not tp-invariant"
                         % blas_out,
                 "ms": round(t_blas, 5), "tflops": round(flops / t_blas / 1e9, 1),
                 "ms_bf16_out": round(t_blas_bf16, 5),
                 "tflops_bf16_out": round(flops / t_blas_bf16 / 1e9, 1),
                 "tbik_gemm_ms": round(kern_ms, 5),
                 "overhead_gemm_pct": round((kern_ms / t_blas - 1) * 100, 1),
                 "overhead_step_pct": round((ms_per_step / t_blas - 1) * 100, 1)}
    log("hipBLASLt %.4f ms (%s out), %.4f ms (bf16 out); tbik GEMM %.4f ms"
        % (t_blas, blas_out, t_blas_bf16, kern_ms))
    del logits, pm, lws

    extra = {}
    if not args.no_extra:
        extra = run_extra(tb, inputs, torch, np, dev, timed, log, args)

    cpu = None
    cpu_all = None
    if not args.no_cpu:
        cpu, cpu_all = cpu_baselines(inputs, np, torch, log, (A, W, tgt, tp))

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "LM-head logprob path: M=%d tokens, K=%d, V=%d vocab; bf16 GEMM "
                               "(64-wide K-block MFMA leaves, fixed fp32 tree, fused 64-column "
                               "row maxima) + tree log-softmax over tp=%d simulated vocab shards "
                               "+ target gather" % (M, K, V, tp),
                   "M": M, "K": K, "V": V, "tp": tp,
                   "A": "bf16 ~N(0,1)", "W": "bf16 ~N(0,0.02)", "targets": "uniform int32",
                   "accumulate": "fp32 tree", "output": "fp32 logits + fp32 logprobs"},
        "pct_mfma_peak": round(value / PEAK_BF16_TFLOPS * 100, 2),
        "bit_mismatches": mismatches,
        "bit_checks": checks,
        "step_split": {"gemm_ms": round(kern_ms, 5), "logsoftmax_ms": round(lsm_ms, 5),
                       "note": "each kernel back to back on its own; the timed steps run them "
                               "in sequence with no events between"},
        "roofline": roofline,
        "roofline_logsoftmax": secondary,
        "hipblaslt": hipblaslt,
        "fingerprints_sha256": fingerprints,
        "cpu_baseline": cpu,
        "cpu_oracle_configs": cpu_all,
        "extra": extra,
    }
    print(json.dumps(out), flush=True)


def profile_kernels(what, tb, inputs, torch, dev, log, head):
    """A few launches of one group of kernels and nothing else, so that a
    rocprofv3 run of `bench.py --profile <what>` reads their counters."""
    reps = 5
    if what == "lmhead":
        for f in head:
            for _ in range(reps):
                f()
    elif what == "rows":
        x = inputs.outlier_bf16((4096, 4096), 3400, device=dev)
        r = inputs.outlier_bf16((4096, 4096), 3410, device=dev)
        w = inputs.normal_bf16((4096,), 3420, std=0.1, mean=1.0, device=dev)
        q = inputs.normal_bf16((32768, 16, 128), 3500, device=dev)
        pos = inputs.positions(32768, 32768, seed=3501).to(dev)
        c, s = tb.tbik_rope_table(1e6, 128, 32768)
        c, s = c.to(dev), s.to(dev)
        g = inputs.normal_bf16((4096, 14336), 3600, std=3.0, device=dev)
        u = inputs.normal_bf16((4096, 14336), 3601, device=dev)
        lg = torch.randn((512, 151936), device=dev) * 3
        tgt = inputs.uniform_int(512, 151936, 3302, device=dev)
        for _ in range(reps):
            tb.tbik_rmsnorm_residual(x, r, w, 1e-6)
            tb.tbik_rope(q, pos, c, s)
            tb.tbik_swiglu(g, u)
            tb.tbik_logsoftmax_gather(lg, tgt, 1)
    elif what == "downproj":
        M, K, N, tp = 256, 14336, 4096, 8
        A = inputs.normal_bf16((M, K), 1001, device=dev)
        Ws = [inputs.normal_bf16((N, K), 2001 + i, std=0.02, device=dev) for i in range(6)]
        ws = torch.empty((tp, M, N), dtype=torch.float32, device=dev)
        C = torch.empty((M, N), dtype=torch.float32, device=dev)
        for i in range(reps):
            tb.tbik_gemm_tpsim(A, Ws[i % 6], tp, ws=ws, out=C)
    elif what == "decode":
        # the tp = 1 down projection at decode batch sizes, W rotating over 5
        # copies as in the timed workload; M = 1 first, then M = 32
        K, N = 14336, 4096
        Ws = [inputs.normal_bf16((N, K), 3001 + i, std=0.02, device=dev) for i in range(5)]
        for M in (1, 32):
            A = inputs.normal_bf16((M, K), 3100 + M, device=dev)
            C = torch.empty((M, N), dtype=torch.float32, device=dev)
            nb = tb.tbik_gemm_workspace_bytes(M, N, K)
            ws = torch.empty((nb // 4,), dtype=torch.float32, device=dev)
            for i in range(reps):
                tb.tbik_gemm(A, Ws[i % 5], out=C, ws=ws)
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    log("profile %s: %d launches of each kernel" % (what, reps))


def downproj_tp8(tb, inputs, torch, dev, timed, log, args):
    """The row-parallel down projection (M = 256, K = 14336, N = 4096) as
    simulated tp = 8: the shard-partials kernel writes 8 fp32 partials, the
    combine runs the top of the tree.  HBM-bound (190 FLOP/B < 312)."""
    import time as _t
    M, K, N, tp = 256, 14336, 4096, 8
    w_bytes = N * K * 2
    n_rot = max(2, -(-600_000_000 // w_bytes))       # > 2x the 256 MB last-level cache
    A = inputs.normal_bf16((M, K), 1001, device=dev)
    Ws = [inputs.normal_bf16((N, K), 2001 + i, std=0.02, device=dev) for i in range(n_rot)]
    ws = torch.empty((tp, M, N), dtype=torch.float32, device=dev)
    C = torch.empty((M, N), dtype=torch.float32, device=dev)
    flops = 2.0 * M * N * K
    stream = torch.cuda.current_stream()
    steps = max(50, args.steps)

    def step(i):
        tb.tbik_gemm_tpsim(A, Ws[i % n_rot], tp, ws=ws, out=C)

    for i in range(10):
        step(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = _t.perf_counter()
    e0.record(stream)
    for i in range(steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = _t.perf_counter() - t0
    ms = max(e0.elapsed_time(e1) / steps, wall * 1e3 / steps)

    k = {"i": 0}

    def part_only():
        k["i"] += 1
        tb.tbik_gemm_tp_partials(A, Ws[k["i"] % n_rot], tp, ws=ws)

    kern_ms = timed(part_only, steps)
    part_bytes = M * K * 2 + N * K * 2 + tp * M * N * 4
    traffic = HEAD_TP8_TRAFFIC_BYTES if gemm_source_sha256(
        os.path.dirname(os.path.abspath(__file__))) == HEAD_TP8_TRAFFIC_SRC_SHA256 else None

    # bitwise invariance over tp and batch size on this workload
    mismatches = 0
    W0 = Ws[0]
    ref = tb.tbik_gemm(A, W0)[0]
    for t in (1, 2, 4, 8):
        Ct = tb.tbik_gemm_tpsim(A, W0, t)[0]
        mismatches += int((Ct.view(torch.int32) != ref.view(torch.int32)).sum().item())
    for m in (1, 32, 255):
        Cm = tb.tbik_gemm(A[:m], W0)[0]
        mismatches += int((Cm.view(torch.int32) != ref[:m].view(torch.int32)).sum().item())
    # negative control: each shard's partial from torch's GEMM, the shards
    # summed in rank order -- not tp-invariant (why the tree exists)
    naive = {}
    one = torch.matmul(A, W0.t()).float()
    for t in (2, 4, 8):
        ks = K // t
        acc = None
        for r in range(t):
            part = torch.matmul(A[:, r * ks:(r + 1) * ks], W0[:, r * ks:(r + 1) * ks].t()).float()
            acc = part if acc is None else acc + part
        naive["tp%d" % t] = int((acc.view(torch.int32) != one.view(torch.int32)).sum().item())
    rot = {"i": 0}

    def blas_rot():
        rot["i"] += 1
        return torch.matmul(A, Ws[rot["i"] % n_rot].t())

    def tp1_rot():
        rot["i"] += 1
        return tb.tbik_gemm(A, Ws[rot["i"] % n_rot], out=C)

    t_blas = timed(blas_rot, steps)
    t_tp1 = timed(tp1_rot, steps)
    log("down projection tp8: step %.4f ms, partials %.4f ms, hipBLASLt %.4f, tp1 %.4f"
        % (ms, kern_ms, t_blas, t_tp1))
    return {"ms_per_step": round(ms, 5), "tflops": round(flops / ms / 1e9, 1),
            "roofline": {"kernel": "tp shard partials", "bound": "hbm",
                         "achieved": round(part_bytes / kern_ms / 1e6, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(part_bytes / kern_ms / 1e6 / PEAK_HBM_GBS, 4),
                         "traffic": traffic, "algorithmic_bytes_per_launch": part_bytes,
                         "avg_launch_ms": round(kern_ms, 5),
                         "mfma_frac": round(flops / kern_ms / 1e9 / PEAK_BF16_TFLOPS, 4)},
            "bit_mismatches_tp_1_2_4_8_M_1_32_255": mismatches,
            "negative_control_mismatches": dict(naive, of=M * N),
            "hipblaslt_ms": round(t_blas, 5), "tbik_tp1_ms": round(t_tp1, 5),
            "overhead_tp1_pct": round((t_tp1 / t_blas - 1) * 100, 1),
            "overhead_tpsim_pct": round((ms / t_blas - 1) * 100, 1)}


def ceilings(tb, inputs, torch, dev, timed, log):
    """What this GPU sustains, from the library's own microbenchmarks (a
    pure matrix-core loop of the leaf instruction; non-temporal HBM read and
    copy streams over buffers of 4 GiB and 2 GiB), beside a large hipBLASLt
    GEMM for reference."""
    ceil = {}
    seed = inputs.normal_bf16((1024,), 3900, device=dev)          # 2 KB of operands
    blocks, iters = 2048, 1024
    out = torch.empty((blocks * 512,), dtype=torch.float32, device=dev)
    fl = {}

    def mf():
        _, fl["f"] = tb.tbik_bench_mfma(seed, blocks, iters, out=out)

    t = timed(mf, 5, warm=2)
    ceil["mfma_bf16_loop_tflops"] = round(fl["f"] / t / 1e9, 1)
    buf = torch.empty((1 << 32,), dtype=torch.uint8, device=dev)    # 4 GiB
    buf.fill_(7)
    red = torch.empty((65536 * 256,), dtype=torch.int32, device=dev)
    src, dst = buf[:1 << 31], buf[1 << 31:]
    # the best of a few grid sizes (one to eight workgroups of 256 per CU
    # and more): the ceiling is what the chip can sustain
    rd, cp = {}, {}
    for blocks in (1024, 2048, 4096, 8192, 16384, 32768, 65536):
        t = timed(lambda: tb.tbik_bench_hbm_read(buf, blocks, out=red), 5, warm=2)
        rd[blocks] = round((1 << 32) / t / 1e6, 1)
        t = timed(lambda: tb.tbik_bench_hbm_copy(src, dst, blocks), 5, warm=2)
        cp[blocks] = round(2 * (1 << 31) / t / 1e6, 1)
    ceil["hbm_read_4GiB_gbs"] = max(rd.values())
    ceil["hbm_copy_2GiB_gbs"] = max(cp.values())
    ceil["hbm_by_grid"] = {"read": rd, "copy_read_plus_write": cp}
    # the GEMM ring's operand copy alone (32 KB stages, 4-slot LDS ring,
    # 8 waves, one workgroup per CU): from a 1 MiB window (resident in every
    # XCD's 4 MB L2), a 32 MiB one (beyond L2, inside the last-level cache)
    # and a 1 GiB one (HBM)
    lds = {}
    outl = torch.empty((1024 * 512,), dtype=torch.int32, device=dev)
    for win, name in ((1 << 20, "l2_1MiB"), (32 << 20, "llc_32MiB"), (1 << 30, "hbm_1GiB")):
        for blocks, stages in ((256, 2048), (1024, 512)):
            nb = {}

            def cl():
                _, nb["b"] = tb.tbik_bench_copy_lds(buf, win, stages, blocks, out=outl)

            t = timed(cl, 5, warm=2)
            lds["%s_wg%d" % (name, blocks)] = round(nb["b"] / t / 1e6, 1)
    ceil["ring_copy_to_lds_gbs"] = lds
    ceil["ring_copy_l2_gbs"] = max(v for k, v in lds.items() if k.startswith("l2_"))
    del buf, src, dst
    n = 8192
    a8 = inputs.normal_bf16((n, n), 3901, device=dev)
    b8 = inputs.normal_bf16((n, n), 3902, device=dev)
    t = timed(lambda: torch.matmul(a8, b8), 10)
    ceil["hipblaslt_bf16_8192cubed_tflops"] = round(2.0 * n ** 3 / t / 1e9, 1)
    del a8, b8
    ceil["spec"] = {"bf16_mfma_tflops": PEAK_BF16_TFLOPS, "hbm_gbs": PEAK_HBM_GBS}
    log("ceilings: MFMA loop %.0f TFLOP/s, HBM read %.0f GB/s, copy %.0f GB/s, ring copy from "
        "L2 %.0f GB/s, hipBLASLt %.0f"
        % (ceil["mfma_bf16_loop_tflops"], ceil["hbm_read_4GiB_gbs"], ceil["hbm_copy_2GiB_gbs"],
           ceil["ring_copy_l2_gbs"], ceil["hipblaslt_bf16_8192cubed_tflops"]))
    return ceil


def run_extra(tb, inputs, torch, np, dev, timed, log, args):
    res = {}
    only = args.only

    def want(name):
        return not only or only == name

    # --- the row-parallel down projection at simulated tp = 8 (M = 256,
    #     K = 14336, N = 4096): shard partials + tree combine per step, W
    #     rotating over copies larger than the last-level cache
    if want("downproj_tp8"):
        res["downproj_tp8_M256_K14336_N4096"] = downproj_tp8(tb, inputs, torch, dev, timed, log,
                                                             args)

    # --- tp=1 GEMM at the other batch sizes vs hipBLASLt
    if want("gemm_m"):
        K, N = 14336, 4096
        Ws = [inputs.normal_bf16((N, K), 3001 + i, std=0.02, device=dev) for i in range(5)]
        for M in (1, 32, 256):
            A = inputs.normal_bf16((M, K), 3100 + M, device=dev)
            C = torch.empty((M, N), dtype=torch.float32, device=dev)
            k = {"i": 0}

            def ours():
                k["i"] += 1
                tb.tbik_gemm(A, Ws[k["i"] % 5], out=C)

            def blas():
                k["i"] += 1
                torch.matmul(A, Ws[k["i"] % 5].t())

            t1, t2 = timed(ours, 30), timed(blas, 30)
            byt = M * K * 2 + N * K * 2 + M * N * 4
            res["downproj_tp1_M%d" % M] = {
                "ms": round(t1, 5), "tflops": round(2 * M * N * K / t1 / 1e9, 1),
                "hbm_gbs": round(byt / t1 / 1e6, 1), "hbm_frac": round(byt / t1 / 1e6 / 8000, 4),
                "hipblaslt_ms": round(t2, 5), "overhead_pct": round((t1 / t2 - 1) * 100, 1)}
            log("downproj M=%d: %.4f ms (hipBLASLt %.4f)" % (M, t1, t2))
        del Ws

    # --- compute-bound shapes: M=4096 prefill and the LM head
    if want("prefill"):
        M, K, N = 4096, 14336, 4096
        A = inputs.normal_bf16((M, K), 3200, device=dev)
        # W (117 MB) rotates over 4 copies, so A and W together exceed twice
        # the 256 MB last-level cache and are read from HBM, not kept there
        Wr = [inputs.normal_bf16((N, K), 3201 + i, std=0.02, device=dev) for i in range(4)]
        C = torch.empty((M, N), dtype=torch.float32, device=dev)
        kr = {"i": 0}

        def tb_rot():
            kr["i"] += 1
            tb.tbik_gemm(A, Wr[kr["i"] % 4], out=C)

        def blas_rot():
            kr["i"] += 1
            return torch.matmul(A, Wr[kr["i"] % 4].t())
        t1 = timed(tb_rot, 10)
        t2 = timed(blas_rot, 10)
        fl = 2.0 * M * N * K
        res["prefill_M4096_K14336_N4096"] = {
            "ms": round(t1, 4), "tflops": round(fl / t1 / 1e9, 1),
            "mfma_frac": round(fl / t1 / 1e9 / 2500, 4), "hipblaslt_ms": round(t2, 4),
            "hipblaslt_tflops": round(fl / t2 / 1e9, 1),
            "overhead_pct": round((t1 / t2 - 1) * 100, 1)}
        log("prefill: %.3f ms = %.1f TFLOP/s (hipBLASLt %.3f ms)" % (t1, fl / t1 / 1e9, t2))
        del A, Wr, C

    if want("logsoftmax"):
        # the standalone log-softmax (its own exact row maxima: two reads of
        # the logits) on the LM head's logits
        M, K, V = 512, 4096, 151936
        A = inputs.normal_bf16((M, K), 3300, device=dev)
        W = inputs.normal_bf16((V, K), 3301, std=0.02, device=dev)
        logits = tb.tbik_gemm(A, W)[0]
        del A, W
        tgt = inputs.uniform_int(M, V, 3302, device=dev)
        nbytes = M * V * 4
        for tpv in (1, 4):
            ws = torch.empty((tb.tbik_logsoftmax_workspace_bytes(M, V, tpv) // 4,),
                             dtype=torch.float32, device=dev)
            out = torch.empty((M,), dtype=torch.float32, device=dev)
            t = timed(lambda: tb.tbik_logsoftmax_gather(logits, tgt, tpv, ws=ws, out=out), 20)
            res["logsoftmax_M512_V151936_tp%d" % tpv] = {
                "ms": round(t, 5), "gbs": round(nbytes / t / 1e6, 1),
                "hbm_frac": round(nbytes / t / 1e6 / 8000, 4),
                "note": "algorithmic bytes = one read of the fp32 logits"}
            log("logsoftmax tp=%d: %.4f ms = %.0f GB/s" % (tpv, t, nbytes / t / 1e6))
        del logits

    if want("rmsnorm"):
        rows, H = 4096, 4096
        xs = [inputs.outlier_bf16((rows, H), 3400 + i, device=dev) for i in range(4)]
        rs = [inputs.outlier_bf16((rows, H), 3410 + i, device=dev) for i in range(4)]
        w = inputs.normal_bf16((H,), 3420, std=0.1, mean=1.0, device=dev)
        y = torch.empty_like(xs[0]); ro = torch.empty_like(xs[0])
        k = {"i": 0}

        def f():
            k["i"] += 1
            tb.tbik_rmsnorm_residual(xs[k["i"] % 4], rs[k["i"] % 4], w, 1e-6, y=y, r_out=ro)

        t = timed(f, 30)
        nbytes = 4 * rows * H * 2 + H * 2
        res["rmsnorm_4096x4096"] = {"ms": round(t, 5), "gbs": round(nbytes / t / 1e6, 1),
                                    "hbm_frac": round(nbytes / t / 1e6 / 8000, 4)}
        log("rmsnorm: %.4f ms = %.0f GB/s" % (t, nbytes / t / 1e6))
        del xs, rs

    if want("rope"):
        T, heads, d = 32768, 16, 128
        x = inputs.normal_bf16((T, heads, d), 3500, device=dev)
        pos = inputs.positions(T, 32768, seed=3501).to(dev)
        c, s = tb.tbik_rope_table(1e6, d, 32768)
        c, s = c.to(dev), s.to(dev)
        y = torch.empty_like(x)
        t = timed(lambda: tb.tbik_rope(x, pos, c, s, y=y), 30)
        nbytes = 2 * T * heads * d * 2 + T * (d // 2) * 4 * 2 + T * 4
        res["rope_32768x16x128"] = {"ms": round(t, 5), "gbs": round(nbytes / t / 1e6, 1),
                                    "hbm_frac": round(nbytes / t / 1e6 / 8000, 4)}
        log("rope: %.4f ms = %.0f GB/s" % (t, nbytes / t / 1e6))
        del x, y

    if want("decoder"):
        from tp_invariant_numerics_amd.decoder import decoder_forward
        cfg = inputs.DecoderConfig()
        B, L = 8, 512
        w = inputs.decoder_weights(cfg, 3700, device=dev)
        tok = inputs.decoder_tokens(B, L, cfg.vocab, 3701, device=dev)
        for tpv in (1, 4):
            t = timed(lambda: decoder_forward(w, tok, cfg, tp=tpv), 5, warm=2)
            res["decoder_8L_d2048_tokens8x512_tp%d" % tpv] = {
                "ms": round(t, 3), "tokens_per_s": round(B * L / t * 1e3, 1),
                "note": "forward logprobs, every step in libtbik (MFMA leaves)"}
            log("decoder tp=%d: %.2f ms = %.0f tokens/s" % (tpv, t, B * L / t * 1e3))
        # Rounding-location mismatch (rounding-alignment article, "three
        # nodes"): the trainer stack is tp=1 with fp32-intermediate nodes;
        # the engine runs tp=4 with the same nodes ("aligned") or with some
        # nodes rounding every intermediate to bf16.  Gap = logprob
        # differences over the 8 x 511 predicted tokens.
        ref = decoder_forward(w, tok, cfg, tp=1).double()
        gaps = {}
        for name, nodes in (("aligned", ()), ("rope", ("rope",)), ("swiglu", ("swiglu",)),
                            ("rmsnorm", ("rmsnorm",)),
                            ("all_three", ("rmsnorm", "rope", "swiglu"))):
            lp = decoder_forward(w, tok, cfg, tp=4,
                                 rounding=dict.fromkeys(nodes, "each_op")).double()
            d_lp = (lp - ref).abs()
            d_p = (lp.exp() - ref.exp()).abs()
            gaps[name] = {"tokens_differing": int((d_lp > 0).sum().item()),
                          "tokens": int(d_lp.numel()),
                          "max_abs_dlogprob": float(d_lp.max().item()),
                          "mean_abs_dlogprob": float(d_lp.mean().item()),
                          "max_abs_dprob": float(d_p.max().item())}
            log("rounding gap engine(tp4, %s) vs trainer(tp1): %d/%d tokens differ, "
                "max |dlp| %.3g, mean %.3g" % (name, gaps[name]["tokens_differing"],
                                               gaps[name]["tokens"],
                                               gaps[name]["max_abs_dlogprob"],
                                               gaps[name]["mean_abs_dlogprob"]))
        # Negative control at the logprob level (TBIK summary page, Abstract:
        # the TP size changes the outputs of ordinary kernels): the two
        # row-parallel projections computed the usual way -- hipBLASLt on
        # each K shard, the bf16 shard outputs summed in rank order -- at
        # tp = 1, 2, 4, everything else unchanged.
        def naive_rowpar(A_, W_, out, tpn):
            ks = A_.shape[1] // tpn
            acc = None
            for t in range(tpn):
                part = torch.matmul(A_[:, t * ks:(t + 1) * ks],
                                    W_[:, t * ks:(t + 1) * ks].t().contiguous())
                acc = part if acc is None else acc + part
            out.copy_(acc)

        base = decoder_forward(w, tok, cfg, tp=1, rowpar=naive_rowpar).double()
        neg = {}
        for tpn in (2, 4):
            lp = decoder_forward(w, tok, cfg, tp=tpn, rowpar=naive_rowpar).double()
            d_lp = (lp - base).abs()
            neg["tp%d_vs_tp1" % tpn] = {"tokens_differing": int((d_lp > 0).sum().item()),
                                        "tokens": int(d_lp.numel()),
                                        "max_abs_dlogprob": float(d_lp.max().item()),
                                        "mean_abs_dlogprob": float(d_lp.mean().item())}
            log("negative control decoder (hipBLASLt shards, rank-order bf16 sum) tp%d vs tp1: "
                "%d/%d tokens differ, max |dlp| %.3g" % (tpn, neg["tp%d_vs_tp1" % tpn]
                                                         ["tokens_differing"], d_lp.numel(),
                                                         d_lp.max().item()))
        tb4 = decoder_forward(w, tok, cfg, tp=4).double()
        res["tp_logprob_gap"] = {
            "tbik_tp4_vs_tp1_tokens_differing": int((tb4 != ref).sum().item()),
            "negative_control": neg}
        res["rounding_location_gap"] = {
            "what": "engine tp=4 (nodes rounding each op to bf16) vs trainer tp=1 "
                    "(fp32-intermediate nodes); random-init weights, so the mechanism, "
                    "not the pages' RL numbers",
            "gaps": gaps}
        del w

    if want("ceilings"):
        res["measured_ceilings"] = ceilings(tb, inputs, torch, dev, timed, log)

    if want("training"):
        # Training side at the down projection's shape: Y = A W^T with
        # A [4096 tokens, 14336], W [4096, 14336].  dW = dY^T A sums over the
        # tokens (token-axis tree, dp = simulated data-parallel ranks),
        # dA = dY W sums over the 4096 outputs; both include their operand
        # transposes.  hipBLASLt on the same products for reference.
        M, d, f = 4096, 4096, 14336
        dY = inputs.normal_bf16((M, d), 3800, device=dev)
        A = inputs.normal_bf16((M, f), 3801, device=dev)
        W = inputs.normal_bf16((d, f), 3802, std=0.02, device=dev)
        dW = torch.empty((d, f), dtype=torch.float32, device=dev)
        flops = 2.0 * M * d * f
        tr = {}
        for dp in (1, 8):
            ws = torch.empty((tb.lib().tbik_gemm_wgrad_workspace_bytes(M, d, f, dp) // 4 + 4,),
                             dtype=torch.float32, device=dev)
            t = timed(lambda: tb.tbik_gemm_wgrad(dY, A, dp=dp, ws=ws, out=dW), 10)
            tr["wgrad_dp%d" % dp] = {"ms": round(t, 4), "tflops": round(flops / t / 1e9, 1)}
            log("wgrad dp=%d: %.3f ms = %.1f TFLOP/s" % (dp, t, flops / t / 1e9))
            del ws
        t = timed(lambda: torch.matmul(dY.t(), A), 10)
        tr["wgrad_hipblaslt"] = {"ms": round(t, 4), "tflops": round(flops / t / 1e9, 1)}
        wsd = torch.empty((tb.lib().tbik_gemm_dgrad_workspace_bytes(M, d, f) // 4 + 4,),
                          dtype=torch.float32, device=dev)
        t = timed(lambda: tb.tbik_gemm_dgrad(dY, W, ws=wsd, want_fp32=False, want_bf16=True), 10)
        tr["dgrad_bf16"] = {"ms": round(t, 4), "tflops": round(flops / t / 1e9, 1)}
        log("dgrad: %.3f ms = %.1f TFLOP/s" % (t, flops / t / 1e9))
        t = timed(lambda: torch.matmul(dY, W), 10)
        tr["dgrad_hipblaslt"] = {"ms": round(t, 4), "tflops": round(flops / t / 1e9, 1)}
        del dY, A, W, dW, wsd
        # backward row kernels, bytes = inputs read once + outputs written once
        rows, H = 4096, 4096
        x = inputs.outlier_bf16((rows, H), 3810, device=dev)
        r = inputs.outlier_bf16((rows, H), 3811, device=dev)
        w = inputs.normal_bf16((H,), 3812, std=0.1, mean=1.0, device=dev)
        gy = inputs.normal_bf16((rows, H), 3813, device=dev)
        gr = inputs.normal_bf16((rows, H), 3814, device=dev)
        t = timed(lambda: tb.tbik_rmsnorm_backward(x, r, w, gy, gr, dp=8), 20)
        nb = 5 * rows * H * 2 + H * 2 + H * 4
        tr["rmsnorm_backward_4096x4096"] = {"ms": round(t, 4), "gbs": round(nb / t / 1e6, 1),
                                            "hbm_frac": round(nb / t / 1e6 / 8000, 4)}
        log("rmsnorm backward: %.4f ms = %.0f GB/s" % (t, nb / t / 1e6))
        del x, r, gy, gr
        rows, cols = 4096, 14336
        g = inputs.normal_bf16((rows, cols), 3820, std=3.0, device=dev)
        u = inputs.normal_bf16((rows, cols), 3821, device=dev)
        gd = inputs.normal_bf16((rows, cols), 3822, device=dev)
        t = timed(lambda: tb.tbik_swiglu_backward(g, u, gd), 20)
        nb = 5 * rows * cols * 2
        tr["swiglu_backward_4096x14336"] = {"ms": round(t, 4), "gbs": round(nb / t / 1e6, 1),
                                            "hbm_frac": round(nb / t / 1e6 / 8000, 4)}
        log("swiglu backward: %.4f ms = %.0f GB/s" % (t, nb / t / 1e6))
        del g, u, gd
        res["training"] = tr

    if want("swiglu"):
        rows, cols = 4096, 14336
        g = inputs.normal_bf16((rows, cols), 3600, std=3.0, device=dev)
        u = inputs.normal_bf16((rows, cols), 3601, device=dev)
        o = torch.empty_like(g)
        t = timed(lambda: tb.tbik_swiglu(g, u, out=o), 30)
        nbytes = 3 * rows * cols * 2
        res["swiglu_4096x14336"] = {"ms": round(t, 5), "gbs": round(nbytes / t / 1e6, 1),
                                    "hbm_frac": round(nbytes / t / 1e6 / 8000, 4)}
        log("swiglu: %.4f ms = %.0f GB/s" % (t, nbytes / t / 1e6))
        del g, u, o
    return res


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baselines(inputs, np, torch, log, head):
    """The CPU oracle (scalar C, as it stands) timed on the host cores.

    Headline (cpu_baseline): the config's logprob path -- oracle GEMM over
    all V columns plus the oracle log-softmax + gather -- on a bounded
    number of the same rows (the GPU run's own A, W and targets), sized for
    about 12 s, scaled to the metric's unit.  cpu_oracle_configs: every
    other workload at full size where that stays within seconds, otherwise
    on a stated sample, plus a one-thread time on a row subset scaled up."""
    import oracle
    from oracle import decoder as od
    nproc = os.cpu_count() or 1
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = nproc
    nth = max(1, min(16, affinity))
    A, W, tgt, tp = head
    M, K = A.shape
    V = W.shape[0]
    log("cpu oracle: copying the headline inputs to the host")
    Ab = inputs.bits(A)
    Wb = inputs.bits(W)
    tg = tgt.cpu().numpy()

    def lp_rows(r0, r):
        lg = oracle.gemm(Ab[r0:r0 + r], Wb, nthreads=nth)
        out, _ = oracle.logsoftmax_gather(lg, tg[r0:r0 + r], tp)
        return out

    t0 = time.perf_counter()
    lp_rows(0, 2)
    dt = time.perf_counter() - t0
    rows = int(max(2, min(M, 2 * 12.0 / max(dt, 1e-3))))
    t0 = time.perf_counter()
    lp_rows(0, rows)
    dt = time.perf_counter() - t0
    fl = 2.0 * rows * V * K
    log("cpu oracle headline: %d of %d rows, %d threads: %.2f s" % (rows, M, nth, dt))
    head_line = {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": nth, "kind": "oracle",
                 "nproc": nproc, "affinity_cpus": affinity, "seconds": round(dt, 2),
                 "cpu_model": _cpu_model(),
                 "full_step_seconds_estimate": round(dt * M / rows, 1),
                 "sample": "oracle logprob path (scalar-leaf tree GEMM over all %d vocab columns "
                           "+ tree log-softmax over tp=%d shards + gather) on the first %d of the "
                           "%d rows of the benchmark's own inputs; value = GEMM flops of those "
                           "rows / time" % (V, tp, rows, M)}

    res = {"threads": nth, "nproc": nproc, "affinity_cpus": affinity, "cpu_model": _cpu_model()}
    # one thread, 4 rows x 4096 vocab columns of the same GEMM, scaled up
    t0 = time.perf_counter()
    oracle.gemm(Ab[:4], Wb[:4096], nthreads=1)
    d1 = time.perf_counter() - t0
    res["lmhead_gemm_1thread"] = {
        "sample": "4 rows x 4096 columns, K=%d, one thread" % K, "seconds": round(d1, 3),
        "gflops": round(2.0 * 4 * 4096 * K / d1 / 1e9, 3),
        "full_gemm_seconds_scaled": round(d1 * (M * V) / (4 * 4096), 1)}
    del Wb

    # config 1: the small simulated-TP GEMM at full size
    a1 = inputs.bits(inputs.normal_bf16((16, 1024), 1))
    w1 = inputs.bits(inputs.normal_bf16((256, 1024), 2))
    t0 = time.perf_counter()
    for t in (1, 2, 4):
        oracle.gemm_tpsim(a1, w1, t, nthreads=nth)
    d = (time.perf_counter() - t0) / 3
    res["tp_gemm_M16_K1024_N256"] = {"seconds_per_call": round(d, 4),
                                     "gflops": round(2.0 * 16 * 256 * 1024 / d / 1e9, 3),
                                     "sample": "full size, tp 1/2/4"}

    # config 2: the row-parallel down projection at full size, tp = 8
    a2 = inputs.bits(inputs.normal_bf16((256, 14336), 3))
    w2 = inputs.bits(inputs.normal_bf16((4096, 14336), 4, std=0.02))
    t0 = time.perf_counter()
    oracle.gemm_tpsim(a2, w2, 8, nthreads=nth)
    d = time.perf_counter() - t0
    res["downproj_M256_K14336_N4096_tp8"] = {
        "seconds": round(d, 2), "gflops": round(2.0 * 256 * 4096 * 14336 / d / 1e9, 3),
        "sample": "full size"}
    log("cpu oracle down projection: %.2f s" % d)
    del a2, w2

    # config 3: the row nodes at full size (the oracle's row nodes are one thread)
    x = inputs.bits(inputs.outlier_bf16((4096, 4096), 5))
    r = inputs.bits(inputs.outlier_bf16((4096, 4096), 6))
    w = inputs.bits(inputs.normal_bf16((4096,), 7, std=0.1, mean=1.0))
    t0 = time.perf_counter()
    oracle.rmsnorm_residual(x, r, w, 1e-6)
    d = time.perf_counter() - t0
    res["rmsnorm_4096x4096"] = {"seconds": round(d, 3),
                                "gbs": round((4 * 4096 * 4096 * 2) / d / 1e9, 3), "threads": 1}
    del x, r
    xr = inputs.bits(inputs.normal_bf16((32768, 16, 128), 8))
    pos = inputs.positions(32768, 32768, seed=9).numpy()
    c, s = oracle.rope_table(1e6, 128, 32768)
    t0 = time.perf_counter()
    oracle.rope(xr, pos, c, s)
    d = time.perf_counter() - t0
    res["rope_32768x16x128"] = {"seconds": round(d, 3),
                                "gbs": round((2 * 32768 * 16 * 128 * 2) / d / 1e9, 3),
                                "threads": 1}
    del xr
    g = inputs.bits(inputs.normal_bf16((4096, 14336), 10, std=3.0))
    u = inputs.bits(inputs.normal_bf16((4096, 14336), 11))
    t0 = time.perf_counter()
    oracle.swiglu(g, u)
    d = time.perf_counter() - t0
    res["swiglu_4096x14336"] = {"seconds": round(d, 3),
                                "gbs": round((3 * 4096 * 14336 * 2) / d / 1e9, 3), "threads": 1}
    del g, u
    log("cpu oracle row nodes done")

    # config 5: the decoder forward on one sequence of 64 tokens (full width)
    cfg = inputs.DecoderConfig()
    wt = inputs.decoder_weights(cfg, 12)
    w_np = {"emb": inputs.bits(wt["emb"]), "lm_head": inputs.bits(wt["lm_head"]),
            "final_norm": inputs.bits(wt["final_norm"]),
            "layers": [{k: inputs.bits(v) for k, v in lw.items()} for lw in wt["layers"]]}
    del wt
    tok = inputs.decoder_tokens(1, 64, cfg.vocab, 13).numpy()
    t0 = time.perf_counter()
    od.decoder_logprobs(w_np, tok, cfg, tp=4)
    d = time.perf_counter() - t0
    res["decoder_8L_d2048_1x64_tokens_tp4"] = {
        "seconds": round(d, 2), "tokens_per_s": round(64 / d, 2),
        "sample": "one sequence of 64 tokens, the shortest the 64-key leaves allow (the benchmark runs 8 x 512)"}
    log("cpu oracle decoder: %.2f s for 64 tokens" % d)
    return head_line, res


if __name__ == "__main__":
    main()
