#!/usr/bin/env python3
"""Packed ternary-code matmul benchmark on one MI355X.

Headline workload (one JSON line on stdout): the Route B GEMV, uint8 codes
[8192, 8192] into a 243-entry fp32 code book, one fp32 layer scale, bf16
activations at M tokens (default 1), bf16 output.  One step is one pass of
the whole decode path over a batch: eight different code matrices (eight
"layers", 512 MiB of codes, more than twice the 256 MB Infinity Cache, so
every launch streams its codes from HBM), replayed from a captured HIP graph
so host launch overhead is not timed.

  value        whole-step throughput: algorithmic bytes of the eight launches
               / wall time of the step (GB/s), wall time bracketed by
               torch.cuda.synchronize() on both sides.
  roofline     the GEMV kernel alone: algorithmic bytes of one launch / its
               average duration, from HIP events recorded on the launch
               stream around the timed steps; peak 8000 GB/s of HBM.
  cpu_baseline the CPU oracle (float64 decode + matmul) timed on this host
               over a bounded sample of the same workload.
  extra        the other packed-matmul workloads, timed the same way (per
               launch, HIP events, rotating buffers): ternary GEMV at
               M = 1, 4, 16 (and tq_pack / tq_unpack on its matrix, per
               call), the two-plane MoE grouped GEMV, the Route B
               prefill at M = 2048 (TFLOP/s) with and without a workspace
               (rb_matmul_ws), Route B GEMV at M = 4 and 16.  One entry
               is context, not this library: the vendor fp16 GEMM of the
               prefill's shape with nothing to decode
               (context_vendor_fp16_gemm_M2048).

Inputs are the seeded synthetic workloads of workloads.py; the pages'
published numbers are end-to-end decode rates on other hardware, so
vs_baseline is null.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
# HBM bytes of one headline launch (M = 1) from the hardware byte counters
# FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0 (the factors that make a 512 MiB device
# copy read and write 512 MiB), in profiles/hbm_traffic_rb_gemv_tq_wave.md.
# The figure belongs to the kernel source it was measured on: any other
# source of rb_gemv.hip reports null.
MEASURED_TRAFFIC = {"rb_gemv.hip": ("9908ab656a4fabaa", 67668937)}
BF16_MFMA_PEAK_TFLOPS = 2500.0
METRIC = "packed matmul: weight GB/s vs HBM peak at M=1–16; TFLOP/s at M=2048"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--M", type=int, default=1, help="tokens of the headline GEMV")
    ap.add_argument("--layers", type=int, default=8, help="code matrices per step")
    ap.add_argument("--no-graph", action="store_true", help="eager launches instead of a graph")
    ap.add_argument("--settle-s", type=float, default=0.5,
                    help="warm-up continues untimed until this many seconds of work have run")
    ap.add_argument("--quick", action="store_true", help="headline only (no extra workloads)")
    ap.add_argument("--extras", default="routeb,ternary,moe,encode,prefill,blocks,alphabet",
                    help="comma list of extra workloads to time "
                         "(routeb, ternary, moe, encode, prefill, blocks, alphabet)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 512 MiB device-to-device copy five times (a kernel of "
                         "known traffic, for scaling hardware byte counters) and exit")
    return ap.parse_args()


def bits16(a):
    return np.ascontiguousarray(a).view(np.int16)


def measured_traffic(src, M):
    """Counter-derived HBM bytes per launch, or None when the kernel source
    differs from the measured one or the launch is not the measured M = 1."""
    import hashlib
    if M != 1 or src not in MEASURED_TRAFFIC:
        return None
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "decode_matmul_amd", "csrc", src)
    try:
        digest = hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]
    except OSError:
        return None
    want, nbytes = MEASURED_TRAFFIC[src]
    return nbytes if digest == want else None


def progress(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class Timed:
    """Captures `fn` (which enqueues work on the current stream) into a HIP
    graph, or runs it eagerly, and times repetitions with HIP events."""

    def __init__(self, torch, fn, use_graph):
        self.torch = torch
        self.fn = fn
        self.graph = None
        torch.cuda.synchronize()
        fn()                                   # eager warm-up (loads code objects)
        torch.cuda.synchronize()
        if use_graph:
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                fn()
            torch.cuda.current_stream().wait_stream(s)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                fn()
            torch.cuda.synchronize()
            self.graph = g

    def run(self):
        if self.graph is not None:
            self.graph.replay()
        else:
            self.fn()

    def time(self, reps, warmup, settle_s=0.0):
        """`warmup` untimed repetitions, continued (untimed) until `settle_s`
        seconds of back-to-back work have passed: the GPU raises its clocks
        over the first tenths of a second under load, and a few warm-up steps
        of a ~0.15 ms step would otherwise time the ramp.  Then `reps` timed
        repetitions."""
        torch = self.torch
        t_start = time.perf_counter()
        for _ in range(warmup):
            self.run()
        torch.cuda.synchronize()
        while time.perf_counter() - t_start < settle_s:
            for _ in range(8):
                self.run()
            torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        for _ in range(reps):
            self.run()
        e1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return wall, e0.elapsed_time(e1) / 1e3          # seconds


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return 1


def host_cpu():
    """(cores this process may run on, CPU model name from /proc/cpuinfo)."""
    try:
        cores = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        cores = os.cpu_count() or 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return cores, model


def cpu_baseline_routeb(d, M, seconds):
    """The oracle itself on the headline workload: float64 decode of the whole
    8192 x 8192 code matrix (numpy indexing, one thread) and the float64
    matmul with M tokens (numpy's BLAS, its own thread pool), repeated until
    `seconds` have passed.  Each step is timed on its own."""
    import oracle
    table = oracle.rb_table(d["ladder"])
    reps = 0
    t_dec = t_mm = 0.0
    t0 = time.perf_counter()
    while True:
        a = time.perf_counter()
        w = oracle.rb_weights(d["codes"], table, d["alpha"])
        b = time.perf_counter()
        oracle.matmul_ref(d["x"][:M], w)
        c = time.perf_counter()
        t_dec += b - a
        t_mm += c - b
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 50:
            break
    code_bytes = d["codes"].nbytes * reps
    host_cores, model = host_cpu()
    mm_threads = blas_threads()
    return {
        "value": round(code_bytes / el / 1e9, 4),
        "unit": "GB/s",
        # threads the oracle actually ran on (the matmul's BLAS pool; the
        # decode step is single-threaded)
        "cores": mm_threads,
        "kind": "oracle",
        "sample": f"{reps} full passes of the float64 oracle (decode 8192x8192 codes, "
                  f"matmul at M={M}) in {el:.1f} s",
        "host_cores": host_cores,
        "cpu_model": model,
        "threads_per_step": {"decode": 1, "matmul": mm_threads},
        "seconds_per_step": {"decode": round(t_dec / reps, 4), "matmul": round(t_mm / reps, 4)},
    }


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library runs the packed matmul on a single "
              "MI355X and has no multi-GPU path; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads
    import decode_matmul_amd as dmm

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    use_graph = not args.no_graph

    if args.calibrate_copy:
        src = torch.ones(1 << 29, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": src.numel(), "copies": 5}), flush=True)
        return

    def to_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    # ---------------------------------------------------------- headline
    progress("headline: generating routeb_gemv inputs")
    M, L = args.M, args.layers
    N = K = 8192
    d = workloads.routeb_gemv(M=max(M, 4))
    table = to_dev(dmm.rb_table(d["ladder"]))
    alpha = float(d["alpha"])
    c0 = to_dev(d["codes"])
    bufs = [c0] + [((c0.to(torch.int32) + 37 * i) % 243).to(torch.uint8) for i in range(1, L)]
    x = to_dev(bits16(d["x"][:M]))
    ys = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(L)]

    def step():
        for i in range(L):
            dmm.rb_matmul(x, bufs[i], table, alpha, ys[i])

    progress("headline: capturing and timing")
    t = Timed(torch, step, use_graph)
    # the graph must reproduce the eager result bit for bit
    ref = [y.clone() for y in ys]
    t.run()
    torch.cuda.synchronize()
    graph_ok = all(torch.equal(a.view(torch.int16), b.view(torch.int16)) for a, b in zip(ref, ys))
    wall, gpu = t.time(args.steps, args.warmup, args.settle_s)

    bytes_launch = N * K + 243 * 4 + M * K * 2 + M * N * 2
    per_launch = gpu / (args.steps * L)
    achieved = bytes_launch / per_launch / 1e9
    value = bytes_launch * L * args.steps / wall / 1e9

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"routeb_gemv: uint8 codes N=K=8192 into a 243-entry fp32 code book, "
                        f"fp32 layer scale, bf16 x at M={M}, bf16 y; {L} code matrices per step",
            "M": M, "N": N, "K": K, "layers_per_step": L,
            "graph": use_graph, "graph_matches_eager": bool(graph_ok),
            "warmup_settle_s": args.settle_s,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic("rb_gemv.hip", M),
            "kernel": "rb_gemv_tiled_kernel",
            "bytes_per_launch": bytes_launch,
            "us_per_launch": round(per_launch * 1e6, 3),
            "tok_s_equiv_per_layer": round(M / per_launch, 1),
            # context: decode steps per second of a model whose packed weights
            # (31.0 GB, the Route B page's Gemma 4 31B checkpoint) stream at
            # this rate
            "steps_per_s_31GB_model": round(achieved * 1e9 / 31.0e9, 1),
        },
    }
    del bufs, ys

    # ---------------------------------------------------------- extras
    extra = {}
    if not args.quick:
        extra = run_extras(torch, dmm, workloads, to_dev, use_graph, args)
    out["extra"] = extra

    # ---------------------------------------------------------- cpu
    if not args.no_cpu:
        progress("cpu baseline: timing the oracle")
        out["cpu_baseline"] = cpu_baseline_routeb(d, M, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


def _timed_launches(torch, fn, n_launch, use_graph, reps=20, warmup=3, settle_s=0.2):
    t = Timed(torch, fn, use_graph)
    wall, gpu = t.time(reps, warmup, settle_s)
    return gpu / (reps * n_launch)


def run_extras(torch, dmm, workloads, to_dev, use_graph, args):
    res = {}
    sel = set(args.extras.split(","))
    dev = torch.device("cuda:0")

    if "routeb" in sel:
        progress("extra: routeb_gemv M=4,16")
        # Route B GEMV at M = 4 (same codes as the headline, 8 layers)
        d = workloads.routeb_gemv(M=4)
        table = to_dev(dmm.rb_table(d["ladder"]))
        c0 = to_dev(d["codes"])
        bufs = [c0] + [((c0.to(torch.int32) + 37 * i) % 243).to(torch.uint8) for i in range(1, 8)]
        for M in (4, 16):
            x = to_dev(bits16(workloads.routeb_gemv(M=M, N=1)["x"]))
            ys = [torch.empty((M, 8192), dtype=torch.bfloat16, device=dev) for _ in range(8)]
            fn = lambda: [dmm.rb_matmul(x, bufs[i], table, float(d["alpha"]), ys[i]) for i in range(8)]
            sec = _timed_launches(torch, fn, 8, use_graph)
            b = 8192 * 8192 + 972 + M * 8192 * 4
            res[f"routeb_gemv_M{M}"] = _rec(b, sec, M, 2 * M * 8192 * 8192)
        del bufs

    if "ternary" in sel:
        progress("extra: ternary_gemv")
        # ternary GEMV 14336 x 4096, codes packed on the GPU, 37 rotating copies
        d = workloads.ternary_gemv()
        W = to_dev(d["W"])
        cs, ss = dmm.packed_shape(14336, 4096, 64)
        c = torch.empty(cs, dtype=torch.uint8, device=dev)
        s = torch.empty(ss, dtype=torch.int16, device=dev)
        st = dmm.tq_pack(W, 64, 1, c, s)
        assert int(st.item()) == 0
        # the packer and the unpacker on this matrix (W fp32, 234.9 MB)
        pst = torch.zeros(1, dtype=torch.int32, device=dev)
        c_again, s_again = torch.empty_like(c), torch.empty_like(s)
        sec = _timed_launches(torch, lambda: dmm.tq_pack(W, 64, 1, c_again, s_again, status=pst), 1,
                              use_graph, reps=10)
        assert torch.equal(c_again, c) and torch.equal(s_again, s)   # packing is deterministic
        res["tq_pack_ternary_gemv"] = _rec_bytes(W.numel() * 4 + c.numel() + s.numel() * 2, sec)
        # four calls per replay into rotating outputs (as the GEMV legs do), so
        # that the replay's own launch cost is shared; each call also clears
        # its status word first
        Wus = [torch.empty((14336, 4096), dtype=torch.bfloat16, device=dev) for _ in range(4)]
        sec = _timed_launches(torch, lambda: [dmm.tq_unpack(c, s, 14336, 4096, 64, Wus[i], status=pst)
                                              for i in range(4)], 4, use_graph, reps=10)
        res["tq_unpack_ternary_gemv_bf16"] = _rec_bytes(c.numel() + s.numel() * 2 + Wus[0].numel() * 2, sec)
        del W, Wus, c_again, s_again
        R = 37
        cc = [c] + [c.clone() for _ in range(R - 1)]
        sc = [s] + [s.clone() for _ in range(R - 1)]
        for M in (1, 4, 16):
            x = to_dev(bits16(d["x"][:M]))
            ys = [torch.empty((M, 14336), dtype=torch.bfloat16, device=dev) for _ in range(R)]
            fn = lambda: [dmm.tq_matmul(x, cc[i], sc[i], 14336, 64, ys[i]) for i in range(R)]
            sec = _timed_launches(torch, fn, R, use_graph)
            b = c.numel() + s.numel() * 2 + M * 4096 * 2 + M * 14336 * 2
            res[f"ternary_gemv_M{M}"] = _rec(b, sec, M, 2 * M * 14336 * 4096)
        del cc, sc
        # ternary prefill: the same package at M = 2048 tokens (MFMA bound)
        progress("extra: ternary_prefill")
        Mp = 2048
        rng = np.random.default_rng(6)
        xp = to_dev(bits16(workloads.bf16_bits(rng.standard_normal((Mp, 4096)).astype(np.float32))))
        yp = torch.empty((Mp, 14336), dtype=torch.bfloat16, device=dev)
        fn = lambda: dmm.tq_matmul(xp, c, s, 14336, 64, yp)
        sec = _timed_launches(torch, fn, 1, use_graph, reps=5, warmup=1)
        flops = 2.0 * Mp * 14336 * 4096
        res["ternary_prefill_M2048"] = _prefill_rec(sec, flops)
        # the same call with a workspace (activations converted once, inside the call)
        wsp = torch.empty(dmm.tq_prefill_workspace_bytes(Mp, 4096), dtype=torch.uint8, device=dev)
        fn = lambda: dmm.tq_matmul_ws(xp, c, s, 14336, 64, yp, wsp)
        sec = _timed_launches(torch, fn, 1, use_graph, reps=5, warmup=1)
        res["ternary_prefill_ws_M2048"] = _prefill_rec(sec, flops)
        del xp, yp, wsp

    if "moe" in sel:
        progress("extra: moe_two_plane (generating 2 GiB of weights)")
        # two-plane MoE: 64 experts 2048 x 4096, 16 tokens, top-8, 3 rotating copies
        d = workloads.moe_two_plane()
        W = to_dev(d["W"].reshape(-1, 4096))
        cs, ss = dmm.packed_shape(64 * 2048, 4096, 64)
        pk = []
        for r in range(3):
            c1 = torch.empty(cs, dtype=torch.uint8, device=dev)
            s1 = torch.empty(ss, dtype=torch.int16, device=dev)
            c2 = torch.empty(cs, dtype=torch.uint8, device=dev)
            s2 = torch.empty(ss, dtype=torch.int16, device=dev)
            if r == 0:
                st = dmm.tq_pack(W, 64, 2, c1, s1, c2, s2)
                assert int(st.item()) == 0
            else:
                c1.copy_(pk[0][0]); s1.copy_(pk[0][1]); c2.copy_(pk[0][2]); s2.copy_(pk[0][3])
            pk.append((c1, s1, c2, s2))
        del W
        x = to_dev(bits16(d["x"]))
        ids = to_dev(d["ids"])
        ys = [torch.empty((16, 8, 2048), dtype=torch.bfloat16, device=dev) for _ in range(3)]
        fn = lambda: [dmm.tq_matmul(x, pk[i][0], pk[i][1], 2048, 64, ys[i], pk[i][2], pk[i][3],
                                    n_experts=64, expert_ids=ids, top_k=8) for i in range(3)]
        sec = _timed_launches(torch, fn, 3, use_graph)
        touched = len(set(d["ids"].reshape(-1).tolist()))
        b = touched * 2 * 2048 * 64 * 15 + 16 * 4096 * 2 + 16 * 8 * 4 + 16 * 8 * 2048 * 2
        rec = _rec(b, sec, 16, 2 * 16 * 8 * 2048 * 4096)
        rec["touched_experts"] = touched
        res["moe_two_plane_T16"] = rec
        # the same experts stored hot-first: plane 2 for experts 0 .. 15 only
        n_hot = 16
        hot = [(p[0], p[1], p[2][:n_hot * 2048], p[3][:n_hot * 2048]) for p in pk]
        fn = lambda: [dmm.tq_matmul_hot(x, hot[i][0], hot[i][1], 2048, 64, ys[i], n_hot, 64, ids,
                                        8, hot[i][2], hot[i][3]) for i in range(3)]
        sec = _timed_launches(torch, fn, 3, use_graph)
        used = set(d["ids"].reshape(-1).tolist())
        planes = sum(2 if e < n_hot else 1 for e in used)
        b = planes * 2048 * 64 * 15 + 16 * 4096 * 2 + 16 * 8 * 4 + 16 * 8 * 2048 * 2
        rec = _rec(b, sec, 16, 2 * 16 * 8 * 2048 * 4096)
        rec["touched_experts"] = touched
        rec["hot_experts"] = n_hot
        res["moe_hot_prefix16_T16"] = rec
        del pk, hot

    if "encode" in sel:
        progress("extra: routeb_encode")
        # Route B encoder with per-row scales, W fp32 8192 x 8192
        d = workloads.routeb_encode()
        N, K = d["W"].shape
        W = to_dev(d["W"])
        codes = torch.empty((N, K), dtype=torch.uint8, device=dev)
        alpha = torch.empty(1 + N, dtype=torch.float32, device=dev)
        rs = torch.empty(N, dtype=torch.float16, device=dev)
        st = torch.zeros(1, dtype=torch.int32, device=dev)
        lad = d["ladder"]
        fn = lambda: dmm.rb_encode(W, lad, codes, alpha, row_scale=rs, status=st)
        sec = _timed_launches(torch, fn, 1, use_graph, reps=10, warmup=2)
        nbytes = 4 * N * K + N * K + 6 * N + 4          # W once, codes, rho, alpha_n, alpha
        gbs = nbytes / sec / 1e9
        res["routeb_encode_per_row"] = {
            "us_per_call": round(sec * 1e6, 2),
            "bytes_per_call": int(nbytes),
            "GBs": round(gbs, 1),
            "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "weights_per_s": round(N * K / sec, 1),
        }
        del W, codes

    if "prefill" in sel:
        progress("extra: routeb_prefill")
        # Route B prefill M = 2048 (MFMA bound)
        d = workloads.routeb_prefill()
        table = to_dev(dmm.rb_table(d["ladder"]))
        cd = to_dev(d["codes"])
        x = to_dev(bits16(d["x"]))
        rho = to_dev(bits16(d["row_scale"]))
        y = torch.empty((2048, 8192), dtype=torch.bfloat16, device=dev)
        fn = lambda: dmm.rb_matmul(x, cd, table, float(d["alpha"]), y, rho)
        sec = _timed_launches(torch, fn, 1, use_graph, reps=10, warmup=2)
        flops = 2.0 * 2048 * 8192 * 8192
        res["routeb_prefill_M2048"] = _prefill_rec(sec, flops)
        # the same call with a workspace: the activations are converted once
        # (a pre-pass kernel, inside the timed call) instead of per N-tile
        ws = torch.empty(dmm.rb_prefill_workspace_bytes(2048, 8192), dtype=torch.uint8, device=dev)
        fn = lambda: dmm.rb_matmul_ws(x, cd, table, 0, float(d["alpha"]), y, ws, rho)
        sec = _timed_launches(torch, fn, 1, use_graph, reps=10, warmup=2)
        res["routeb_prefill_ws_M2048"] = _prefill_rec(sec, flops)
        del ws
        # context only, not this library: the vendor fp16 GEMM (torch.matmul,
        # hipBLASLt) of the same shape with weights already in fp16, i.e. the
        # rate of a plain GEMM on this part with nothing to decode
        wf = torch.randn(8192, 8192, device=dev, dtype=torch.float16).t().contiguous()
        xf = torch.randn(2048, 8192, device=dev, dtype=torch.float16)
        yf = torch.empty((2048, 8192), dtype=torch.float16, device=dev)
        fn = lambda: torch.matmul(xf, wf, out=yf)
        sec = _timed_launches(torch, fn, 1, use_graph, reps=10, warmup=2)
        rec = _prefill_rec(sec, flops)
        rec["what"] = "torch.matmul fp16 2048x8192 @ 8192x8192, no decode (vendor library, context)"
        res["context_vendor_fp16_gemm_M2048"] = rec
        del wf, xf, yf

    if "blocks" in sel:
        progress("extra: routeb_blocks (one code book per 32 rows)")
        d = workloads.routeb_blocks(M=2048)
        tables = to_dev(np.stack([dmm.rb_table(a) for a in d["ladders"]]))
        c0 = to_dev(d["codes"])
        bufs = [c0] + [c0.clone() for _ in range(7)]
        x1 = to_dev(bits16(d["x"][:1]))
        ys = [torch.empty((1, 8192), dtype=torch.bfloat16, device=dev) for _ in range(8)]
        fn = lambda: [dmm.rb_matmul_blocks(x1, bufs[i], tables, 32, float(d["alpha"]), ys[i])
                      for i in range(8)]
        sec = _timed_launches(torch, fn, 8, use_graph)
        b = 8192 * 8192 + 256 * 972 + 8192 * 4
        res["routeb_blocks32_gemv_M1"] = _rec(b, sec, 1, 2 * 8192 * 8192)
        del bufs, ys
        x = to_dev(bits16(d["x"]))
        y = torch.empty((2048, 8192), dtype=torch.bfloat16, device=dev)
        fn = lambda: dmm.rb_matmul_blocks(x, c0, tables, 32, float(d["alpha"]), y)
        sec = _timed_launches(torch, fn, 1, use_graph, reps=10, warmup=2)
        res["routeb_blocks32_prefill_M2048"] = _prefill_rec(sec, 2.0 * 2048 * 8192 * 8192)
        del x, y, c0

    if "alphabet" in sel:
        progress("extra: routeb_alphabet (7-bit indices)")
        d = workloads.routeb_alphabet(M=2048)
        table = to_dev(dmm.rb_table(d["ladder"]))
        codes = to_dev(d["codes"])
        L = dmm.rb7_row_bytes(8192)
        used = torch.empty(128, dtype=torch.uint8, device=dev)
        n_used = torch.empty(1, dtype=torch.int32, device=dev)
        c7 = torch.empty((8192, L), dtype=torch.uint8, device=dev)
        st = torch.zeros(1, dtype=torch.int32, device=dev)
        fn = lambda: dmm.rb_truncate(codes, used, n_used, c7, st)
        sec = _timed_launches(torch, fn, 1, use_graph, reps=10, warmup=2)
        assert int(st.item()) == 0 and int(n_used.item()) == 60
        res["routeb_truncate"] = {"us_per_call": round(sec * 1e6, 2),
                                  "codes_per_s": round(8192 * 8192 / sec, 1)}
        del codes
        bufs = [c7] + [c7.clone() for _ in range(7)]
        x1 = to_dev(bits16(d["x"][:1]))
        ys = [torch.empty((1, 8192), dtype=torch.bfloat16, device=dev) for _ in range(8)]
        fn = lambda: [dmm.rb_matmul7(x1, bufs[i], 8192, used, table, 0, float(d["alpha"]), ys[i])
                      for i in range(8)]
        sec = _timed_launches(torch, fn, 8, use_graph)
        b = 8192 * L + 128 + 972 + 8192 * 4
        rec = _rec(b, sec, 1, 2 * 8192 * 8192)
        rec["codes_used"] = 60
        res["routeb7_gemv_M1"] = rec
        del bufs, ys
        x = to_dev(bits16(d["x"]))
        y = torch.empty((2048, 8192), dtype=torch.bfloat16, device=dev)
        fn = lambda: dmm.rb_matmul7(x, c7, 8192, used, table, 0, float(d["alpha"]), y)
        sec = _timed_launches(torch, fn, 1, use_graph, reps=10, warmup=2)
        res["routeb7_prefill_M2048"] = _prefill_rec(sec, 2.0 * 2048 * 8192 * 8192)
        del x, y, c7
    return res


def _prefill_rec(sec, flops):
    return {
        "us_per_launch": round(sec * 1e6, 2),
        "tflops": round(flops / sec / 1e12, 2),
        "frac_bf16_mfma_peak": round(flops / sec / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
    }


def _rec_bytes(bytes_call, sec):
    gbs = bytes_call / sec / 1e9
    return {"us_per_call": round(sec * 1e6, 2), "bytes_per_call": int(bytes_call),
            "GBs": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}


def _rec(bytes_launch, sec, M, flops):
    gbs = bytes_launch / sec / 1e9
    return {
        "us_per_launch": round(sec * 1e6, 3),
        "bytes_per_launch": int(bytes_launch),
        "GBs": round(gbs, 1),
        "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
        "tflops": round(flops / sec / 1e12, 3),
        "tok_s_equiv": round(M / sec, 1),
    }


if __name__ == "__main__":
    main()
