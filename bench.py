#!/usr/bin/env python3
"""Benchmark of the tree-based invariant kernels on one MI355X.

Headline step (the row-parallel down-projection workload): one pass of the
simulated tensor-parallel GEMM over a batch of M=256 tokens,
A [256, 14336] bf16 ~N(0,1), W [4096, 14336] bf16 ~N(0,0.02), K split into
tp=8 shards: the shard-partials kernel (64-wide K-block MFMA leaves + the
in-register tree) writes 8 fp32 partials, the combine kernel runs the top
of the tree.  value = 2*M*N*K / step time (TFLOP/s).  Inputs are resident in
HBM; W rotates over several copies so every step streams W from HBM rather
than from the 256 MB last-level cache.

Also reported: the same GEMM at tp=1 for M in {1,32,256} against torch's
bf16 GEMM (hipBLASLt) -- the non-invariant baseline and overhead; a
compute-bound M=4096 prefill and the LM-head GEMM (M=512, K=4096,
N=151936) as % of the bf16 MFMA peak; the row kernels as % of HBM
bandwidth; the bitwise mismatch count across tp and M; and the CPU oracle
timed on a bounded sample.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extra]
"""
import argparse
import json
import math
import os
import sys
import time

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
METRIC = "invariant GEMM TFLOP/s (% MFMA peak, overhead vs hipBLASLt); 0 bit mismatches"

# The headline's shard-partials kernel, as named in a rocprofv3 kernel trace.
HEAD_KERNEL = "k_gemm_ring<4, 2, 2, 4, 4, 2, false, 28, 0, 0, 1, 1, 2>"
# HBM bytes per launch of HEAD_KERNEL from two rocprofv3 --pmc runs (profiles/
# k_gemm_ring_downproj_M256_K14336_N4096_tp8.md): FETCH_SIZE 64818 KiB x 2.000
# + WRITE_SIZE 32768 KiB x 1.000, the factors being what a plain 1 GiB device
# copy reads on the same counters (524303 KiB fetched, 1048576 KiB written).
# Valid only for the GEMM sources the counters were taken on (hash below).
HEAD_TRAFFIC_BYTES = (64818 * 2 + 32768) * 1024
HEAD_TRAFFIC_SRC_SHA256 = "b368286dba4f51fbc852b85d1d79d7ec4104168481bb3a3d0859460c35544994"


def gemm_source_sha256(root):
    import hashlib
    h = hashlib.sha256()
    for f in ("gemm.hip", "tbik_device.h", "tbik_internal.h"):
        with open(os.path.join(root, "tp_invariant_numerics_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--M", type=int, default=256)
    ap.add_argument("--tp", type=int, default=8)
    ap.add_argument("--no-extra", action="store_true", help="headline step only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--pmc-calib", action="store_true",
                    help="run only a plain device copy of known size (counter calibration)")
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

    if args.pmc_calib:
        # plain copy kernel of known size for FETCH_SIZE / WRITE_SIZE scaling
        nbytes = 1 << 30
        src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("pmc-calib: copied %d bytes x5" % nbytes)
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
    M, K, N, tp = args.M, 14336, 4096, args.tp
    w_bytes = N * K * 2
    n_rot = max(2, -(-600_000_000 // w_bytes))       # > 2x the 256 MB last-level cache
    log("inputs: A [%d,%d], W [%d,%d] x%d rotating copies, tp=%d" % (M, K, N, K, n_rot, tp))
    A = inputs.normal_bf16((M, K), 1001, device=dev)
    Ws = [inputs.normal_bf16((N, K), 2001 + i, std=0.02, device=dev) for i in range(n_rot)]
    ws = torch.empty((tp, M, N), dtype=torch.float32, device=dev)
    C = torch.empty((M, N), dtype=torch.float32, device=dev)
    flops = 2.0 * M * N * K

    # One step = the library's simulated-TP call: the shard-partials kernel
    # writes the tp fp32 partials into ws, the combine kernel runs the top
    # of the tree into C.  The K timed steps are bracketed by one event pair
    # and the wall clock; per-kernel events inside the loop would add their
    # own dispatch gaps to the step.
    def step(i):
        tb.tbik_gemm_tpsim(A, Ws[i % n_rot], tp, ws=ws, out=C)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e_start = torch.cuda.Event(enable_timing=True)
    e_end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e_start.record(stream)
    for i in range(args.steps):
        step(i)
    e_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = e_start.elapsed_time(e_end) / args.steps
    ms_per_step = max(step_ms, wall * 1e3 / args.steps)
    value = flops / (ms_per_step * 1e-3) / 1e12
    log("step %.4f ms (events), wall %.4f ms/step" % (step_ms, wall * 1e3 / args.steps))

    # The same step split into its two kernels, in a separately instrumented
    # pass (an event between the kernels adds a dispatch gap, so the split
    # sums to more than the step).
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        rec = ev[i]
        rec[0].record(stream)
        tb.tbik_gemm_tp_partials(A, Ws[i % n_rot], tp, ws=ws)
        rec[1].record(stream)
        tb.tbik_tree_combine(ws, out=C)
        rec[2].record(stream)
    torch.cuda.synchronize()
    part_ms = sum(a.elapsed_time(b) for a, b, c in ev) / args.steps
    comb_ms = sum(b.elapsed_time(c) for a, b, c in ev) / args.steps
    log("instrumented split: partials %.4f ms, combine %.4f ms" % (part_ms, comb_ms))

    # Average duration of the shard-partials kernel: back-to-back launches on
    # the launch stream between two HIP events (per-kernel events inside a
    # step add their own dispatch overhead to the interval).
    nb2b = max(10, args.steps)

    def part_only(i=[0]):
        i[0] += 1
        tb.tbik_gemm_tp_partials(A, Ws[i[0] % n_rot], tp, ws=ws)

    kern_ms = timed(part_only, nb2b)
    log("partials kernel back-to-back: %.4f ms per launch" % kern_ms)

    # roofline of the dominant kernel (the shard-partials GEMM): by arithmetic
    # intensity 2MNK / bytes = 190 FLOP/B < 2500e12/8e12 = 312 FLOP/B it is
    # HBM-bound; its MFMA fraction is reported beside it
    part_bytes = M * K * 2 + N * K * 2 + tp * M * N * 4
    achieved_gbs = part_bytes / (kern_ms * 1e-3) / 1e9
    traffic = HEAD_TRAFFIC_BYTES if gemm_source_sha256(root) == HEAD_TRAFFIC_SRC_SHA256 else None
    roofline = {"kernel": HEAD_KERNEL + " (tp shard partials)", "bound": "hbm",
                "achieved": round(achieved_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved_gbs / PEAK_HBM_GBS, 4), "traffic": traffic,
                "algorithmic_bytes_per_launch": part_bytes,
                "avg_launch_ms": round(kern_ms, 5),
                "in_step_event_ms": round(part_ms, 5),
                "arith_intensity_flop_per_byte": round(flops / part_bytes, 1),
                "mfma_frac": round(flops / (kern_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}

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
    log("bit mismatches across tp {1,2,4,8} and M {1,32,255,256}: %d" % mismatches)

    # negative control: the same tp split done the usual way -- each shard's
    # partial from torch's GEMM, the shards summed in rank order -- is not
    # tp-invariant (why the tree exists); count its mismatches against tp=1
    naive_mism = {}
    one = torch.matmul(A, W0.t()).float()
    for t in (2, 4, 8):
        ks = K // t
        acc = None
        for r in range(t):
            part = torch.matmul(A[:, r * ks:(r + 1) * ks], W0[:, r * ks:(r + 1) * ks].t()).float()
            acc = part if acc is None else acc + part
        naive_mism["tp%d" % t] = int((acc.view(torch.int32) != one.view(torch.int32)).sum().item())
    del one
    log("negative control (hipBLASLt per shard + sequential sum vs tp=1): %s" % naive_mism)

    # non-invariant baseline: torch bf16 GEMM (hipBLASLt), same shape
    rot = {"i": 0}

    def blas_rot():
        rot["i"] += 1
        return torch.matmul(A, Ws[rot["i"] % n_rot].t())

    t_blas = timed(blas_rot, args.steps)

    def tbik_tp1_rot():
        rot["i"] += 1
        return tb.tbik_gemm(A, Ws[rot["i"] % n_rot], out=C)

    t_tp1 = timed(tbik_tp1_rot, args.steps)
    hipblaslt = {"what": "torch.matmul bf16 (hipBLASLt), same shape, not tp-invariant",
                 "ms": round(t_blas, 5), "tflops": round(flops / t_blas / 1e9, 1),
                 "tbik_tp1_ms": round(t_tp1, 5),
                 "overhead_tp1_pct": round((t_tp1 / t_blas - 1) * 100, 1),
                 "overhead_tpsim_pct": round((ms_per_step / t_blas - 1) * 100, 1)}
    log("hipBLASLt %.4f ms; tbik tp=1 %.4f ms; tpsim step %.4f ms" % (t_blas, t_tp1, ms_per_step))

    extra = {}
    if not args.no_extra:
        extra = run_extra(tb, inputs, torch, np, dev, timed, log, args)

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(inputs, np, log, A, Ws[0], tp)

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
        "config": {"workload": "row-parallel down-proj GEMM, M=%d K=%d N=%d, simulated TP=%d "
                               "(shard partials + tree combine)" % (M, K, N, tp),
                   "M": M, "K": K, "N": N, "tp": tp, "rotating_W_copies": n_rot,
                   "A": "bf16 ~N(0,1)", "W": "bf16 ~N(0,0.02)", "accumulate": "fp32 tree"},
        "pct_mfma_peak": round(value / PEAK_BF16_TFLOPS * 100, 2),
        "bit_mismatches": mismatches,
        "step_split": {"partials_ms": round(part_ms, 5), "combine_ms": round(comb_ms, 5),
                       "note": "separately instrumented pass with an event between the two "
                               "kernels; the timed steps carry no events inside"},
        "negative_control_mismatches": {
            "what": "torch bf16 GEMM per K shard, shards summed in rank order, vs the "
                    "unsplit torch GEMM (not tp-invariant); out of %d outputs" % (M * N),
            **naive_mism},
        "roofline": roofline,
        "hipblaslt": hipblaslt,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(out), flush=True)


def run_extra(tb, inputs, torch, np, dev, timed, log, args):
    res = {}
    only = args.only

    def want(name):
        return not only or only == name

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
        W = inputs.normal_bf16((N, K), 3201, std=0.02, device=dev)
        C = torch.empty((M, N), dtype=torch.float32, device=dev)
        t1 = timed(lambda: tb.tbik_gemm(A, W, out=C), 10)
        t2 = timed(lambda: torch.matmul(A, W.t()), 10)
        fl = 2.0 * M * N * K
        res["prefill_M4096_K14336_N4096"] = {
            "ms": round(t1, 4), "tflops": round(fl / t1 / 1e9, 1),
            "mfma_frac": round(fl / t1 / 1e9 / 2500, 4), "hipblaslt_ms": round(t2, 4),
            "hipblaslt_tflops": round(fl / t2 / 1e9, 1),
            "overhead_pct": round((t1 / t2 - 1) * 100, 1)}
        log("prefill: %.3f ms = %.1f TFLOP/s (hipBLASLt %.3f ms)" % (t1, fl / t1 / 1e9, t2))
        del A, W, C

    logits = None
    if want("lmhead") or want("logsoftmax"):
        M, K, V = 512, 4096, 151936
        A = inputs.normal_bf16((M, K), 3300, device=dev)
        W = inputs.normal_bf16((V, K), 3301, std=0.02, device=dev)
        logits = torch.empty((M, V), dtype=torch.float32, device=dev)
        pm = torch.empty((M, (V + 63) // 64), dtype=torch.float32, device=dev)
        if want("lmhead"):
            # the tree GEMM with and without the fused row maxima back to back,
            # then hipBLASLt (whose large launches change the clocks seen next)
            t1 = timed(lambda: tb.tbik_gemm(A, W, out=logits), 8, warm=2)
            t_fused = timed(lambda: tb.tbik_gemm_logits(A, W, out=logits, pmax=pm), 8, warm=2)
            t2 = timed(lambda: torch.matmul(A, W.t()), 8, warm=2)
            fl = 2.0 * M * V * K
            res["lmhead_M512_K4096_N151936"] = {
                "ms": round(t1, 4), "tflops": round(fl / t1 / 1e9, 1),
                "mfma_frac": round(fl / t1 / 1e9 / 2500, 4), "hipblaslt_ms": round(t2, 4),
                "hipblaslt_tflops": round(fl / t2 / 1e9, 1),
                "overhead_pct": round((t1 / t2 - 1) * 100, 1)}
            log("lmhead: %.3f ms = %.1f TFLOP/s (hipBLASLt %.3f ms)" % (t1, fl / t1 / 1e9, t2))
        else:
            tb.tbik_gemm(A, W, out=logits)
        tgt = inputs.uniform_int(M, V, 3302, device=dev)
        nbytes = M * V * 4
        # logprob path with the row maximum fused into the LM-head GEMM
        if want("lmhead"):
            t1 = t_fused
            res["lmhead_fused_rowmax_M512_K4096_N151936"] = {
                "ms": round(t1, 4), "tflops": round(2.0 * M * V * K / t1 / 1e9, 1),
                "note": "tbik_gemm_logits: LM-head GEMM + 64-column row maxima in its epilogue"}
        else:
            tb.tbik_gemm_logits(A, W, out=logits, pmax=pm)
        for tpv in (1, 4):
            ws = torch.empty((tb.tbik_logsoftmax_workspace_bytes(M, V, tpv) // 4,),
                             dtype=torch.float32, device=dev)
            out = torch.empty((M,), dtype=torch.float32, device=dev)
            t = timed(lambda: tb.tbik_logsoftmax_gather_pmax(logits, tgt, pm, tpv, ws=ws, out=out),
                      20)
            res["logsoftmax_fused_max_M512_V151936_tp%d" % tpv] = {
                "ms": round(t, 5), "gbs": round(nbytes / t / 1e6, 1),
                "hbm_frac": round(nbytes / t / 1e6 / 8000, 4),
                "note": "row maxima from the LM-head GEMM epilogue; one read of the fp32 logits"}
            log("logsoftmax (fused max) tp=%d: %.4f ms = %.0f GB/s" % (tpv, t, nbytes / t / 1e6))
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
        del A, W, logits

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
        # measured ceilings beside the spec peaks: a large vendor GEMM for the
        # matrix cores, a 1 GiB device copy and a 2 GiB read for HBM
        n = 8192
        a8 = inputs.normal_bf16((n, n), 3900, device=dev)
        b8 = inputs.normal_bf16((n, n), 3901, device=dev)
        t = timed(lambda: torch.matmul(a8, b8), 10)
        ceil = {"hipblaslt_bf16_8192cubed_tflops": round(2.0 * n ** 3 / t / 1e9, 1)}
        del a8, b8
        src = torch.empty((1 << 30,), dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        t = timed(lambda: dst.copy_(src), 20)
        ceil["copy_1GiB_gbs"] = round(2 * (1 << 30) / t / 1e6, 1)
        del src, dst
        rd = torch.ones((1 << 29,), dtype=torch.float32, device=dev)       # 2 GiB
        t = timed(lambda: torch.sum(rd), 20)
        ceil["read_2GiB_sum_gbs"] = round((1 << 31) / t / 1e6, 1)
        del rd
        ceil["spec"] = {"bf16_mfma_tflops": PEAK_BF16_TFLOPS, "hbm_gbs": PEAK_HBM_GBS}
        res["measured_ceilings"] = ceil
        log("ceilings: hipBLASLt 8192^3 %.0f TFLOP/s, copy %.0f GB/s, read %.0f GB/s"
            % (ceil["hipblaslt_bf16_8192cubed_tflops"], ceil["copy_1GiB_gbs"],
               ceil["read_2GiB_sum_gbs"]))

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


def cpu_baseline(inputs, np, log, A, W, tp):
    """The CPU oracle (scalar C, as it stands) on a bounded sample of the
    headline workload: all M rows x a block of output columns, simulated tp."""
    import oracle
    nth = min(16, os.cpu_count() or 1)
    Ab = inputs.bits(A)
    M, K = Ab.shape
    # a short calibration run, then one run sized for about 12 s of CPU work
    cols = 8
    t0 = time.perf_counter()
    oracle.gemm_tpsim(Ab, inputs.bits(W[:cols]), tp, nthreads=nth)
    dt = time.perf_counter() - t0
    cols = int(min(W.shape[0], max(8, cols * 12.0 / max(dt, 1e-3))))
    Wb = inputs.bits(W[:cols])
    t0 = time.perf_counter()
    oracle.gemm_tpsim(Ab, Wb, tp, nthreads=nth)
    dt = time.perf_counter() - t0
    fl = 2.0 * M * cols * K
    log("cpu oracle: %d x %d outputs, K=%d, tp=%d, %d threads: %.2f s" % (M, cols, K, tp, nth, dt))
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": nth, "kind": "oracle",
            "seconds": round(dt, 2),
            "cpu_model": _cpu_model(),
            "sample": "oracle tpsim GEMM (scalar leaves, same tree) on A[%d,%d] x W[:%d] "
                      "(all rows, first %d output columns), tp=%d" % (M, K, cols, cols, tp)}


if __name__ == "__main__":
    main()
