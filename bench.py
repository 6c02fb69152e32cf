#!/usr/bin/env python3
"""Throughput of one training step of the INT8 W8A8 linear layer on one GPU.

Workload: 12000 tokens, 5376 -> 7168, block-Hadamard rotation 128, bf16
activations with 1% outlier channels, bf16 dY, seeded synthetic data (the
headline shape of OneTrainer PR #1681's measurements).  A step is the whole
path: rotate + quantize X, forward product, both dY quantizations (one
call), dX product with the un-rotation in its epilogue, dW product, and the
SGD stochastic requant.
Metric: int8 TOPS counting the three products (3 * 2 * M * N * K ops) over
the wall time of the full step, and its fraction of the dense INT8 MFMA peak.

The timed steps carry one event per step boundary and none between calls;
ms_per_step is the median step, and the mean over the bracketed K steps is
reported beside it.  Per-call durations come from HIP events recorded on the
launch stream between the calls of as many steps again, run after the timed
ones; the dominant call is reported against its roofline.  The memory-bound
calls are also timed on their own, cycling through more than 512 MB of
buffer copies so the 256 MB infinity cache cannot serve them, next to the
library's streaming copy (the device's practical read+write ceiling).  The
forward of 2048 tokens (rotate, quantize, forward product) is timed on its
own as well.  The CPU baseline runs the oracle, compiled for the host CPU,
on a bounded token sample.

The default warmup is 50 steps (about 75 ms): after 5 steps from idle, the
clocks have not settled, and the same GPU timed its steps about 4% slower.
The workloads that do not use the headline layer (the 2048-token forward, the
matrix-core ceiling, the MLP products and step) run before the warmup, so the
warmup and timed steps start on a device at the clocks a training loop holds;
the timed region is still exactly the K steps.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

M, K, N, HAD = 12000, 5376, 7168, 128
LR = 1e-3
SEED = 0
PEAK_INT8_TOPS = 5000.0       # MI355X dense INT8 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
GEMM_OPS = 2.0 * M * N * K
METRIC = "INT8 linear fwd+bwd TOPS at 12000x5376->7168; % of INT8 MFMA peak"

# Algorithmic bytes per launch of the memory-bound calls (read once + write once).
# quantize_dy reads dY twice (the column scales must be known before any
# column code is written) and writes both code arrays.
ALG_BYTES = {
    "quantize_x": M * K * 2 + M * K + 4 * M,
    "quantize_dy": 2 * (M * N * 2) + 2 * (M * N) + 8 * M + 8 * N,
    "sgd_requant": N * K * (1 + 4 + 1) + 8 * N,
    # AdamW: codes in and out, gradient in, both fp32 moments in and out.
    "adamw_requant": N * K * (1 + 4 + 8 + 8 + 1) + 8 * N,
    # Weight-normalized SGD: codes in and out, gradient in.
    "wn_sgd_requant": N * K * (1 + 4 + 1) + 16 * N,
}
GEMMS = ("fwd", "bwd_dx", "bwd_dw")
COPY_BYTES = 512 << 20        # calibration copy: reads and writes this many bytes
# Kernel symbols behind each call, as rocprofv3 names them (a call's traffic
# is the sum over its kernels).
KERNEL_OF = {"fwd": ["gemm_kernel<2, 4, false, false, 2, 2>"],
             "bwd_dx": ["gemm_kernel<2, 4, false, true, 3, 0>"],
             "bwd_dw": ["gemm_kernel<2, 4, true, true, 1, 2>"],
             "quantize_x": ["quant_rows_kernel<true, 256, 3, 128>"],
             "quantize_dy": ["grad_stats_kernel<true>", "grad_scales_kernel",
                             "grad_codes_kernel<true>"],
             "sgd_requant": ["sgd_requant_kernel<256, 3, false>"]}


def code_only(src):
    """C/C++ source text without its comments (string and character literals
    kept) and with whitespace runs collapsed: edits to comments or layout do
    not change the kernels."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def source_digest(read=None):
    """Digest of the kernel sources (csrc/, comments and layout ignored) that
    the committed counter summaries must have been taken on.  read(name)
    returns a file's text (default: the working tree's)."""
    csrc = os.path.join(ROOT, "w8a8_integer_linear_amd", "csrc")
    if read is None:
        def read(name):
            with open(os.path.join(csrc, name), encoding="utf-8") as fh:
                return fh.read()
    h = hashlib.sha256()
    for f in sorted(os.listdir(csrc)):
        h.update(f.encode() + code_only(read(f)).encode())
    return h.hexdigest()[:16]


def traffic_for(call):
    """Measured HBM bytes per call (summed over its kernels) from the committed
    counter summary, or None when the summary is absent, lacks one of the
    kernels, or was taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_digest") != source_digest():
        return None
    total = 0
    for key in KERNEL_OF.get(call, []):
        hits = [ent for name, ent in rec.get("kernels", {}).items() if key in name]
        if len(hits) != 1:
            return None
        total += hits[0].get("bytes_per_launch", 0)
    return total or None


def host_cpu():
    """(logical CPUs, CPU model name) of the host."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return os.cpu_count(), model


def cpu_baseline(d, tokens):
    """The oracle's full step on the first `tokens` rows (weight prep untimed),
    with the oracle compiled -O3 -march=native for this host."""
    import oracle
    flags = oracle.use_host_build()
    qw, sw = oracle.prepare_weight(d["w"], had_block=HAD)
    x, dy = d["x"][:tokens], d["dy"][:tokens]
    t0 = time.perf_counter()
    qx, sx = oracle.quantize_rows(x, had_block=HAD)
    oracle.fwd(qx, sx, qw, sw)
    qg1, sg1 = oracle.quantize_rows(dy, prescale=sw)
    qg2, sg2 = oracle.quantize_cols(dy, prescale=sx)
    dx = oracle.bwd_dx(qg1, sg1, qw)
    oracle.hadamard(dx, HAD)
    dw = oracle.bwd_dw(qg2, sg2, qx)
    oracle.sgd_requant(qw, sw, dw, LR, SEED, 0)
    t = time.perf_counter() - t0
    ops = 3 * 2.0 * tokens * N * K
    ncpu, model = host_cpu()
    return {"value": round(ops / t / 1e12, 6), "unit": "TOPS", "cores": oracle.threads(),
            "kind": "oracle",
            "sample": f"{tokens} of {M} tokens at full 5376->7168 width, all eight steps "
                      f"(SGD requant over the whole weight), {t:.2f} s",
            "host_cpus": ncpu, "cpu_model": model, "build": " ".join(flags)}


def median(v):
    s = sorted(v)
    n = len(s)
    return s[n // 2] if n % 2 else 0.5 * (s[n // 2 - 1] + s[n // 2])


def timed_calls(torch, fns, reps):
    """Median device time (ms) of calls fns[i % len(fns)], each bracketed by
    events on the current stream, after one untimed pass over fns."""
    for fn in fns:
        fn()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record()
    for i in range(reps):
        fns[i % len(fns)]()
        ev[i + 1].record()
    torch.cuda.synchronize()
    return median([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)])


def memory_bound_rotating(torch, layer, d, reps=24):
    """The memory-bound calls of the step on their own, each cycling through
    enough copies of its operands (more than 512 MB in all) that the 256 MB
    infinity cache cannot hold the next call's data, against the library's
    streaming copy of 512 MiB (the same cycling), the device's practical
    read+write ceiling.  GB/s count algorithmic bytes."""
    import numpy as np
    from w8a8_integer_linear_amd import _native as nat
    x = torch.from_numpy(d["x"].view(np.int16)).view(torch.bfloat16).cuda()
    dy = torch.from_numpy(d["dy"].view(np.int16)).view(torch.bfloat16).cuda()
    res = {}

    copy_n = 512 << 20
    bufs = [torch.empty(copy_n, dtype=torch.uint8, device="cuda") for _ in range(4)]
    copy_fns = [lambda i=i: nat.qlin_stream_copy(bufs[2 * i], bufs[2 * i + 1]) for i in range(2)]
    ms = timed_calls(torch, copy_fns, reps)
    ceiling = 2 * copy_n / (ms * 1e-3) / 1e9
    res["stream_copy"] = {"ms": round(ms, 4), "gbs": round(ceiling, 1),
                          "frac_hbm": round(ceiling / PEAK_HBM_GBS, 4),
                          "bytes": 2 * copy_n}
    del bufs, copy_fns

    def entry(name, fns, footprint):
        ms = timed_calls(torch, fns, reps)
        gbs = ALG_BYTES[name] / (ms * 1e-3) / 1e9
        res[name] = {"ms": round(ms, 4), "gbs": round(gbs, 1),
                     "frac_hbm": round(gbs / PEAK_HBM_GBS, 4),
                     "frac_ceiling": round(gbs / ceiling, 4),
                     "rotating_mb": round(footprint / 1e6, 1)}

    xs = [x] + [x.clone() for _ in range(2)]
    qxs = [torch.empty((M, K), dtype=torch.int8, device="cuda") for _ in xs]
    sxs = [torch.empty(M, dtype=torch.float32, device="cuda") for _ in xs]
    entry("quantize_x", [lambda i=i: nat.qlin_quantize_rows(xs[i], had_block=HAD, q=qxs[i],
                                                            s=sxs[i]) for i in range(len(xs))],
          len(xs) * ALG_BYTES["quantize_x"])
    del xs, qxs

    dys = [dy] + [dy.clone() for _ in range(2)]
    outs = [(torch.empty((M, N), dtype=torch.int8, device="cuda"),
             torch.empty(M, dtype=torch.float32, device="cuda"),
             torch.empty((M, N), dtype=torch.int8, device="cuda"),
             torch.empty(N, dtype=torch.float32, device="cuda"),
             torch.empty(N, dtype=torch.float32, device="cuda")) for _ in dys]
    entry("quantize_dy",
          [lambda i=i: nat.qlin_quantize_grad(dys[i], layer.sw, sxs[0], q1=outs[i][0],
                                              s1=outs[i][1], q2=outs[i][2], s2=outs[i][3],
                                              col_sum=outs[i][4]) for i in range(len(dys))],
          len(dys) * (M * N * 2 + 2 * M * N))
    del dys, outs

    ws = [(layer.qw.clone(), layer.sw.clone(), layer.dw.clone()) for _ in range(3)]
    entry("sgd_requant",
          [lambda i=i: nat.qlin_sgd_requant(ws[i][0], ws[i][1], ws[i][2], LR, SEED, i)
           for i in range(len(ws))], len(ws) * ALG_BYTES["sgd_requant"])
    del ws
    return res


def forward_2048(torch, reps=50):
    """The forward workload of 2048 tokens (5376 -> 7168, rotation 128):
    rotate + quantize X, then the forward product with its fused dequant, per
    call (median of `reps`, each bracketed by events).  TOPS count 2 M N K."""
    import numpy as np

    import workloads
    from w8a8_integer_linear_amd import LinearW8A8Training
    m = 2048
    d2 = workloads.linear(m, K, N, seed=SEED, with_dy=False)
    layer = LinearW8A8Training(torch.from_numpy(d2["w"]).cuda(), had_block=HAD, max_tokens=m)
    x = torch.from_numpy(d2["x"].view(np.int16)).view(torch.bfloat16).cuda()
    ms = timed_calls(torch, [lambda: layer.forward(x)], reps)
    tops = 2.0 * m * N * K / (ms * 1e-3) / 1e12
    return {"ms": round(ms, 4), "tops": round(tops, 1),
            "frac_mfma": round(tops / PEAK_INT8_TOPS, 4), "shape": [m, K, N],
            "context_rtx5090_ms": 1.27}


def replay_skinny(torch, nat, qx, sx, qws, sw, y, eager, reps, nbytes):
    """The skinny calls replayed from a HIP graph, without the host's per-call
    launch cost: one call per weight copy, in the order that ends on the copy
    the eager loop ended on, so each replay must reproduce `eager` exactly
    (checked after the first replay and after the timed ones)."""
    copies = len(qws)
    try:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(copies):
                nat.qlin_fwd(qx, sx, qws[(reps + i) % copies], sw, y=y)
        graph.replay()
        torch.cuda.synchronize()
        if not torch.equal(y, eager):
            return {"ms_graph": None, "graph_error": "replay differs from the eager output"}
        n_rep = max(1, reps // copies)
        b = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        b.record()
        for _ in range(n_rep):
            graph.replay()
        e.record()
        torch.cuda.synchronize()
        if not torch.equal(y, eager):
            return {"ms_graph": None, "graph_error": "replay differs from the eager output"}
    except RuntimeError as err:      # capture not available: report, do not fail the bench
        return {"ms_graph": None, "graph_error": str(err)[:200]}
    ms_graph = b.elapsed_time(e) / (n_rep * copies)
    return {"ms_graph": round(ms_graph, 5),
            "gbs_graph": round(nbytes / (ms_graph * 1e-3) / 1e9, 1)}


def skinny_forward(torch, reps=240, copies=24):
    """The weight-streaming forward for M <= 16 rows (4096 -> 4096, no rotation,
    seeded inputs of the skinny workload): HBM GB/s per call, where a call moves
    the weight once plus the small activation and output arrays.  Calls cycle
    through `copies` copies of the weight (403 MB, more than the 256 MB
    infinity cache), so each call streams its weight from HBM.  `ms` times the
    calls as launched from Python; `ms_graph` times them replayed from a HIP
    graph."""
    import numpy as np

    import workloads
    from w8a8_integer_linear_amd import _native as nat
    res = {}
    for m in (1, 4, 16):
        d = workloads.skinny(m)
        kk = d["w"].shape[1]
        nn = d["w"].shape[0]
        x = torch.from_numpy(d["x"].view(np.int16)).view(torch.bfloat16).cuda()
        w = torch.from_numpy(d["w"]).cuda()
        qw, sw = nat.qlin_quantize_rows(w)
        qws = [qw.clone() for _ in range(copies)]
        qx, sx = nat.qlin_quantize_rows(x)
        y = torch.empty((m, nn), dtype=torch.float32, device="cuda")
        for i in range(copies):
            nat.qlin_fwd(qx, sx, qws[i], sw, y=y)
        torch.cuda.synchronize()
        b = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        b.record()
        for i in range(reps):
            nat.qlin_fwd(qx, sx, qws[i % copies], sw, y=y)
        e.record()
        torch.cuda.synchronize()
        ms = b.elapsed_time(e) / reps
        eager = y.clone()          # the last call used copy (reps - 1) % copies
        nbytes = nn * kk + m * kk + 4 * (m + nn) + 4 * m * nn
        gbs = nbytes / (ms * 1e-3) / 1e9
        graph_res = replay_skinny(torch, nat, qx, sx, qws, sw, y, eager, reps, nbytes)
        res[f"skinny_fwd_m{m}"] = {"ms": round(ms, 5), "gbs": round(gbs, 1),
                                   "frac_hbm": round(gbs / PEAK_HBM_GBS, 4), **graph_res,
                                   "shape": [m, kk, nn]}
    return res


def mlp_products(torch, reps=10):
    """The six products of the transformer MLP workload (8192 tokens, fc1
    4096 -> 14336, fc2 14336 -> 4096, dX rotated back with blocks of 128),
    each timed over `reps` calls through the same entry point as the step,
    with its workspace for split tails.  Operands are seeded codes in
    [-127, 127] and positive scales: a product's time does not depend on
    the values.  TOPS count 2 M N K per call."""
    from w8a8_integer_linear_amd import _native as nat
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    M = 8192

    def codes(r, c):
        return torch.randint(-127, 128, (r, c), dtype=torch.int8, device="cuda", generator=g)

    def scales(n):
        return torch.rand(n, device="cuda", generator=g) * 1e-2 + 1e-3

    res = {}
    for name, K, N in (("fc1", 4096, 14336), ("fc2", 14336, 4096)):
        qx, sx, qw, sw = codes(M, K), scales(M), codes(N, K), scales(N)
        qg1, sg1, qg2, sg2 = codes(M, N), scales(M), codes(N, M), scales(N)
        out = {0: torch.empty(M, N, device="cuda"), 1: torch.empty(M, K, device="cuda"),
               2: torch.empty(N, K, device="cuda")}
        ws = torch.zeros(max(nat.qlin_product_ws_bytes(op, M, N, K) for op in range(3)) + 16,
                         dtype=torch.uint8, device="cuda")
        calls = {
            "fwd": lambda: nat.qlin_product_ws(nat.QLIN_OP_FWD, qx, sx, qw, M, N, K, scol=sw,
                                               out=out[0], workspace=ws),
            "dx": lambda: nat.qlin_product_ws(nat.QLIN_OP_DX, qg1, sg1, qw, M, N, K,
                                              had_block=HAD, out=out[1], workspace=ws),
            "dw": lambda: nat.qlin_product_ws(nat.QLIN_OP_DW, qg2, sg2, qx, M, N, K,
                                              out=out[2], workspace=ws),
        }
        for op, fn in calls.items():
            fn()
            fn()
            torch.cuda.synchronize()
            b = torch.cuda.Event(enable_timing=True)
            e = torch.cuda.Event(enable_timing=True)
            b.record()
            for _ in range(reps):
                fn()
            e.record()
            torch.cuda.synchronize()
            ms = b.elapsed_time(e) / reps
            tops = 2.0 * M * N * K / (ms * 1e-3) / 1e12
            res[f"mlp_{name}_{op}"] = {"ms": round(ms, 4), "tops": round(tops, 1),
                                       "frac_mfma": round(tops / PEAK_INT8_TOPS, 4),
                                       "shape": [M, K, N]}
        del out, ws
    return res


def mlp_step(torch, reps=10, warm=3):
    """One training step of the transformer MLP workload (8192 tokens, fc1
    4096 -> 14336, exact erf-GELU in fp32, fc2 14336 -> 4096, rotation 128 on
    both inputs, seeded inputs): both forwards, both backwards with the GELU's
    derivative between them, and both SGD stochastic requants (seeds 0 and
    1).  The GELU and its derivative are torch's own fused fp32 kernels (they
    sit outside the INT8 path) and are part of the step's time.  Median of
    `reps` steps, each bracketed by events.  TOPS count the six products (2 M
    N K each)."""
    import numpy as np

    import workloads
    from w8a8_integer_linear_amd import LinearW8A8Training
    d = workloads.mlp()
    dev = lambda a: (torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
                     if a.dtype == np.uint16 else torch.from_numpy(a).cuda())
    m, dm, hm = d["x"].shape[0], d["x"].shape[1], d["w1"].shape[0]
    fc1 = LinearW8A8Training(dev(d["w1"]), had_block=HAD, max_tokens=m)
    fc2 = LinearW8A8Training(dev(d["w2"]), had_block=HAD, max_tokens=m)
    x, dy2 = dev(d["x"]), dev(d["dy2"])

    def step(i):
        h = fc1.forward(x)
        a = torch.nn.functional.gelu(h)
        fc2.forward(a)
        da = fc2.backward(dy2)
        dh = torch.ops.aten.gelu_backward(da, h)
        fc1.backward(dh)
        fc2.sgd_step(d["lr"], d["seeds"][1], i)
        fc1.sgd_step(d["lr"], d["seeds"][0], i)

    for i in range(warm):
        step(i)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record()
    for i in range(reps):
        step(warm + i)
        ev[i + 1].record()
    torch.cuda.synchronize()
    ms = median([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)])
    ops = 6 * 2.0 * m * dm * hm
    tops = ops / (ms * 1e-3) / 1e12
    return {"ms": round(ms, 4), "tops": round(tops, 1),
            "frac_mfma": round(tops / PEAK_INT8_TOPS, 4), "shape": [m, dm, hm]}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--cpu-tokens", type=int, default=4096,
                    help="token sample of the oracle CPU baseline (0 skips it)")
    ap.add_argument("--no-mlp", action="store_true",
                    help="skip the MLP workload's products, whose kernels share names with "
                         "the step's (for per-kernel profiler summaries of the step)")
    ap.add_argument("--step-kernels-only", action="store_true",
                    help="also skip the timings whose kernels share names with the step's "
                         "(the 2048-token forward and the memory-bound calls on rotating "
                         "buffers): implies --no-mlp")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="before the steps, run a plain device copy of 512 MiB (three times) "
                         "whose counter readings calibrate HBM byte counters")
    ap.add_argument("--mfma-ceiling-seconds", type=float, default=0.0,
                    help="only run the matrix-core ceiling kernel back to back for this many "
                         "seconds (for power sampling) and print its JSON line")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the layer's data-"
              "parallel sharding is not built here.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import workloads
    from w8a8_integer_linear_amd import LinearW8A8Training

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.mfma_ceiling_seconds > 0:
        print(json.dumps({"mfma_ceiling": mfma_ceiling(torch, warm_s=args.mfma_ceiling_seconds)}),
              flush=True)
        return

    print(f"[bench] generating inputs {M}x{K}->{N}", file=sys.stderr, flush=True)
    d = workloads.linear(M, K, N, seed=SEED)

    def dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    x, dy = dev(d["x"]), dev(d["dy"])
    layer = LinearW8A8Training(dev(d["w"]), had_block=HAD, max_tokens=M)
    torch.cuda.synchronize()
    if args.copy_calibration:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # The workloads that do not use the headline layer run first, so that the
    # warmup and timed steps start on a device already at the clocks and power
    # a training loop holds (after a few steps from idle they run about 4%
    # slower).  Their figures go into the same line.
    pre = {}
    if not args.step_kernels_only:
        print("[bench] forward of 2048 tokens", file=sys.stderr, flush=True)
        pre["forward_2048"] = forward_2048(torch)
        print("[bench] matrix-core ceiling", file=sys.stderr, flush=True)
        pre["mfma_ceiling"] = mfma_ceiling(torch)
        if not args.no_mlp:
            pre_mlp = mlp_products(torch)
            print("[bench] MLP training step", file=sys.stderr, flush=True)
            pre_mlp["mlp_step"] = mlp_step(torch)
            pre["mlp"] = pre_mlp
        torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    marks = []

    def tick(label):
        ev = torch.cuda.Event(enable_timing=True)
        ev.record(stream)
        marks.append((label, ev))

    def step(i):
        if layer.timer is not None:
            tick("start")
        layer.forward(x)
        layer.backward(dy)
        layer.sgd_step(LR, SEED, i)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # The timed steps carry no per-call events; the per-call breakdown comes
    # from as many steps again, run after them with an event between calls.
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    bounds = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    bounds[0].record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
        bounds[i + 1].record(stream)
    torch.cuda.synchronize()
    ms_mean = bounds[0].elapsed_time(bounds[-1]) / args.steps
    ms_per_step = median([bounds[i].elapsed_time(bounds[i + 1]) for i in range(args.steps)])

    print(f"[bench] per-call events over {args.steps} more steps", file=sys.stderr, flush=True)
    layer.timer = tick
    e_begin = torch.cuda.Event(enable_timing=True)
    e_end = torch.cuda.Event(enable_timing=True)
    e_begin.record(stream)
    for i in range(args.steps):
        step(args.warmup + args.steps + i)
    e_end.record(stream)
    torch.cuda.synchronize()
    print(f"[bench] {ms_per_step:.4f} ms per step (median; mean {ms_mean:.4f}); with per-call events "
          f"{e_begin.elapsed_time(e_end) / args.steps:.4f}", file=sys.stderr, flush=True)

    per = {}
    for (_, a), (label, b) in zip(marks[:-1], marks[1:]):
        if label == "start":
            continue
        per.setdefault(label, []).append(a.elapsed_time(b))
    avg = {k: sum(v) / len(v) for k, v in per.items()}

    breakdown = {}
    for k, ms in avg.items():
        if k in GEMMS:
            breakdown[k] = {"ms": round(ms, 4), "tops": round(GEMM_OPS / (ms * 1e-3) / 1e12, 1),
                            "frac_mfma": round(GEMM_OPS / (ms * 1e-3) / 1e12 / PEAK_INT8_TOPS, 4)}
        else:
            gbs = ALG_BYTES[k] / (ms * 1e-3) / 1e9
            breakdown[k] = {"ms": round(ms, 4), "gbs": round(gbs, 1),
                            "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}
    dominant = max(avg, key=avg.get)
    if dominant in GEMMS:
        ach = GEMM_OPS / (avg[dominant] * 1e-3) / 1e12
        traffic = traffic_for(dominant)
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_INT8_TOPS,
                "unit": "TFLOP/s", "frac": round(ach / PEAK_INT8_TOPS, 4), "traffic": traffic,
                "kernel": dominant, "ms_per_launch": round(avg[dominant], 4)}
    else:
        ach = ALG_BYTES[dominant] / (avg[dominant] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4),
                "traffic": traffic_for(dominant),
                "kernel": dominant,
                "ms_per_launch": round(avg[dominant], 4)}

    tops = 3 * GEMM_OPS / (ms_per_step * 1e-3) / 1e12
    out = {
        "metric": METRIC, "value": round(tops, 2), "unit": "TOPS", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_mean": round(ms_mean, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "INT8 W8A8 linear training step, 12000 tokens, 5376->7168, "
                               "Hadamard block 128, bf16 X (1% x8 outlier channels), bf16 dY, "
                               "SGD lr 1e-3 with Philox stochastic requant",
                   "tokens": M, "in_features": K, "out_features": N, "had_block": HAD},
        "pct_of_int8_peak": round(100 * tops / PEAK_INT8_TOPS, 2),
        "roofline": roof,
        "breakdown": breakdown,
    }
    # Outside the timed step: the AdamW update on the same weight (the second
    # optimizer of the update row), timed over a few calls after the step.
    layer.timer = None
    layer.adamw_step(LR, SEED, 1, weight_decay=0.01)
    torch.cuda.synchronize()
    a_begin = torch.cuda.Event(enable_timing=True)
    a_end = torch.cuda.Event(enable_timing=True)
    a_begin.record(stream)
    for t in range(2, 12):
        layer.adamw_step(LR, SEED, t, weight_decay=0.01)
    a_end.record(stream)
    torch.cuda.synchronize()
    a_ms = a_begin.elapsed_time(a_end) / 10
    a_gbs = ALG_BYTES["adamw_requant"] / (a_ms * 1e-3) / 1e9
    out["extras"] = {"adamw_requant": {"ms": round(a_ms, 4), "gbs": round(a_gbs, 1),
                                       "frac_hbm": round(a_gbs / PEAK_HBM_GBS, 4),
                                       "shape": [N, K]}}
    out["extras"].update(wn_update(torch, layer))
    if not args.step_kernels_only:
        print("[bench] memory-bound calls on rotating buffers", file=sys.stderr, flush=True)
        out["memory_bound_rotating"] = memory_bound_rotating(torch, layer, d)
        out["forward_2048"] = pre["forward_2048"]
        ceil = pre["mfma_ceiling"]
        out["mfma_ceiling"] = ceil
        for k in GEMMS:
            if k in breakdown:
                breakdown[k]["frac_ceiling"] = round(breakdown[k]["tops"] / ceil["tops"], 4)
    out["extras"].update(skinny_forward(torch))
    if "mlp" in pre:
        out["extras"].update(pre["mlp"])
    if args.cpu_tokens > 0:
        print(f"[bench] cpu baseline on {args.cpu_tokens} tokens", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(d, args.cpu_tokens)
    print(json.dumps(out), flush=True)


def mfma_ceiling(torch, warm_s=1.0, reps=20, iters=1000):
    """The library's matrix-core ceiling kernel (the products' register tile
    and MFMA sequence on random fragments, no memory traffic, one workgroup of
    8 waves per compute unit): run back to back for about a second so that
    power and clocks settle where the products run, then `reps` launches timed
    with an event between launches.  Int8 TOPS of the median launch."""
    import time
    from w8a8_integer_linear_amd import _native as nat
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    g = torch.Generator(device="cuda").manual_seed(3)
    frags = torch.randint(-128, 128, (nat.MFMA_CEILING_FRAG_BYTES,), dtype=torch.int32,
                          device="cuda", generator=g).to(torch.int8)
    out = torch.empty(cus * 512 * 4, dtype=torch.int32, device="cuda")
    ops = 2.0 * 16 * 16 * 64 * 64 * 8 * cus * iters
    t0 = time.time()
    while time.time() - t0 < warm_s:
        for _ in range(10):
            nat.qlin_mfma_ceiling(frags, out, cus, iters)
        torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record()
    for i in range(reps):
        nat.qlin_mfma_ceiling(frags, out, cus, iters)
        ev[i + 1].record()
    torch.cuda.synchronize()
    ms = median([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)])
    tops = ops / (ms * 1e-3) / 1e12
    return {"ms_per_launch": round(ms, 4), "tops": round(tops, 1),
            "frac_peak": round(tops / PEAK_INT8_TOPS, 4), "workgroups": cus, "iters": iters}


def wn_update(torch, layer):
    """The weight-normalized SGD step (trained magnitude, INT8 direction) on
    a copy of the headline weight's state, timed over ten calls."""
    from w8a8_integer_linear_amd import _native as nat
    q, s = layer.qw.clone(), layer.sw.clone()
    g, sw = nat.qlin_wn_init(q, s)
    nat.qlin_wn_sgd_requant(q, s, g, sw, layer.dw, LR, SEED, 1)
    torch.cuda.synchronize()
    b = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    b.record()
    for t in range(2, 12):
        nat.qlin_wn_sgd_requant(q, s, g, sw, layer.dw, LR, SEED, t)
    e.record()
    torch.cuda.synchronize()
    ms = b.elapsed_time(e) / 10
    gbs = ALG_BYTES["wn_sgd_requant"] / (ms * 1e-3) / 1e9
    return {"wn_sgd_requant": {"ms": round(ms, 4), "gbs": round(gbs, 1),
                               "frac_hbm": round(gbs / PEAK_HBM_GBS, 4), "shape": [N, K]}}


if __name__ == "__main__":
    main()
