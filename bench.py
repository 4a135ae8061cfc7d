"""Throughput of the fused dequantize-and-multiply path on one MI355X.

Workload (one "step"): the decode products of a ~1B-parameter dense transformer
with Q8_0 weights -- QKV 3072x2048, O 2048x2048, gate and up 6144x2048, down
2048x6144 and the output head 65536x2048 -- at batch 1 and again at batch 8
(Phobos README "Inference": Q8_0 ~1B models decoded on the GPU).  Each batch
size is one grouped launch over the six matrices (README "Components": kernel
fusion).  Weights and activations are seeded synthetic tensors with the model's
shapes, resident in HBM before the timed region.  The weights are cycled over
enough distinct device copies (>= 1 GiB); step c runs its batch-1 launch on
copy c and its batch-8 launch on copy c + copies/2, so no launch finds its
weights in the 256 MB last-level cache.  Steps are replayed from HIP graphs --
one graph runs a step on each weight copy in turn -- so the host's launch cost
is not what is measured.

Prints one JSON line: weight GB/s of the step (value), the dominant launch's
achieved bandwidth against the 8 TB/s HBM peak (roofline: HIP events on the
launch stream around graph replays of that launch alone, back to back over the
weight copies, so the time per launch includes the in-graph gaps between
dependent kernels), and the CPU oracle on bounded samples of every
configuration, 1 thread and all threads (cpu_baseline).  Secondary figures
(the 1024x1024 and Q4_K GEMVs, routed MoE, pp512 GEMM TFLOP/s) are reported
under "secondary" unless --no-secondary is given.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "dequant-GEMV weight GB/s (% HBM peak) + pp512 quant-GEMM TOPS (% MFMA peak)"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
ROTATE_BYTES = 1 << 30


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=300)
    p.add_argument("--warmup", type=int, default=30)
    p.add_argument("--copies", type=int, default=0, help="weight copies to cycle (0 = auto, >= 1 GiB)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-secondary", action="store_true")
    p.add_argument("--cpu-reps", type=int, default=5, help="timed oracle runs per sample (median)")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run a plain device copy of known size (HBM counter calibration)")
    p.add_argument("--only", choices=["small", "q4k", "moe", "moe_prompt", "ffn", "gemm", "sweep",
                                      "hbm"],
                   default=None,
                   help="run one secondary workload only (for profiling)")
    return p.parse_args()


def capture(torch, fns):
    """One HIP graph per closure (each closure launches on the current stream)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for f in fns:
            f()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for f in fns:
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            f()
        graphs.append(gr)
    torch.cuda.synchronize()
    return graphs


def replay_ms(torch, graphs, reps, per_graph=1, warm_ms=20.0):
    """ms per call over `reps` replays (round robin over `graphs`, each of
    `per_graph` calls), after about warm_ms of untimed replays: the kernels run
    a few percent faster once the shader clock has settled under load."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    graphs[0].replay()
    torch.cuda.synchronize()
    e0.record()
    graphs[0].replay()
    e1.record()
    torch.cuda.synchronize()
    one = max(e0.elapsed_time(e1), 1e-3)
    for i in range(max(len(graphs), int(warm_ms / one) + 1)):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    e0.record()
    for i in range(reps):
        graphs[i % len(graphs)].replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (reps * per_graph)


def steady_ms(torch, graph, per_graph, warm_ms=25.0, timed_ms=25.0):
    """ms per call of a graph of `per_graph` calls at steady state: replayed for
    about warm_ms first, then timed over about timed_ms (compute-bound kernels
    speed up over the first tens of milliseconds as the shader clock settles)."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    graph.replay()
    torch.cuda.synchronize()
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    one = max(e0.elapsed_time(e1), 1e-3)
    return replay_ms(torch, [graph], int(timed_ms / one) + 1, per_graph, warm_ms)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path would shard rows, experts or output columns across GPUs)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import quantized_gguf_q8_amd as g
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")

    if args.calibrate_copy:
        print(json.dumps(calibrate_copy(torch)), flush=True)
        return
    if args.only:
        print(json.dumps(secondary(g, torch, synth, only=args.only)), flush=True)
        return

    # ---- inputs: one host copy of the weights, C device copies ----
    shapes = list(synth.DENSE_1B_LAYER_SET)
    host_w = [synth.q8_0_matrix(n, k, seed=0, tensor_id=synth.tid(1, n, k)) for _, n, k in shapes]
    set_bytes = sum(w.nbytes for w in host_w)
    copies = args.copies or max(2, -(-ROTATE_BYTES // set_bytes))
    dev_sets = [[torch.from_numpy(w).to(dev) for w in host_w] for _ in range(copies)]
    del host_w
    xs, ys = {}, {}
    for name, n, k in shapes:
        for b in (1, 8):
            xs[(name, b)] = torch.from_numpy(
                synth.normal_f32((b, k), seed=0, tensor_id=synth.tid(1, n, k) + b)).to(dev)
            ys[(name, b)] = torch.empty((b, n), dtype=torch.float32, device=dev)
    groups = []   # per copy: (batch-1 group, batch-8 group)
    for wset in dev_sets:
        # batch 1: vector units, no workspace; batch 8: matrix cores with a workspace
        groups.append(tuple(
            g.GemvGroup(g.Q8_0, [(w, n, k, xs[(name, b)], ys[(name, b)])
                                 for (name, n, k), w in zip(shapes, wset)],
                        ws=None if b == 1 else "auto") for b in (1, 8)))
    torch.cuda.synchronize()
    weight_bytes_step = 2 * set_bytes

    def step_fn(c):
        # batch 8 on the copy half a cycle away: its weights were last read
        # about copies/2 * 194 MB earlier, past the last-level cache
        g1 = groups[c][0]
        g8 = groups[(c + copies // 2) % copies][1]
        return lambda: (g1(), g8())

    # One graph runs a step on every weight copy in turn (`copies` steps per
    # replay, as a serving loop captures many layers per graph); single-step
    # graphs make up a step count that is not a multiple of `copies`.
    def all_copies():
        for c in range(copies):
            step_fn(c)()

    graphs = capture(torch, [step_fn(c) for c in range(copies)] + [all_copies])
    single, multi = graphs[:copies], graphs[copies]

    def run_steps(n):
        for _ in range(n // copies):
            multi.replay()
        for i in range(n % copies):
            single[i].replay()

    run_steps(args.warmup)
    torch.cuda.synchronize()

    # ---- timed region: exactly K steps ----
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run_steps(args.steps)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    value = weight_bytes_step / (ms_step * 1e-3) / 1e9

    # ---- per-launch times: each launch kind alone, back to back over the
    # weight copies in one graph, HIP events on the launch stream around the
    # replays (the time per launch includes the in-graph gaps between its
    # kernels and the next launch's) ----
    del graphs
    agg = {}
    alg = {}
    for b_i, label in ((0, "gemv_q8_0_grouped_b1"), (1, "gemv_q8_0_grouped_b8")):
        grp0 = groups[0][b_i]
        alg[label] = grp0.weight_bytes + sum(
            xs[(name, grp0.batch)].numel() * 4 + ys[(name, grp0.batch)].numel() * 4
            for name, _, _ in shapes)
        lgraph = capture(torch, [lambda: [groups[c][b_i]() for c in range(copies)]])
        reps = max(2, args.steps // copies)
        ms = replay_ms(torch, lgraph, reps, copies)
        agg[label] = (ms * reps * copies, reps * copies)
        del lgraph
    dom = max(agg, key=lambda k: agg[k][0] / agg[k][1])
    dom_ms, dom_n = agg[dom]
    avg_ms = dom_ms / dom_n
    achieved = alg[dom] / (avg_ms * 1e-3) / 1e9
    per_kernel = {k: {"launches": c, "avg_us": round(t * 1e3 / c, 3),
                      "alg_bytes": alg[k], "GB/s": round(alg[k] / (t / c * 1e-3) / 1e9, 1)}
                  for k, (t, c) in agg.items()}

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "dense ~1B decode layer set, Q8_0 weights: qkv 3072x2048, o 2048x2048, "
                        "gate 6144x2048, up 6144x2048, down 2048x6144, head 65536x2048; "
                        "batch 1 then batch 8 per step, one grouped launch per batch "
                        "(batch 8 on the matrix cores)",
            "weight_format": "q8_0",
            "weight_bytes_per_step": weight_bytes_step,
            "weight_copies_cycled": copies,
            "frac_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        },
        "roofline": {
            "bound": "hbm",
            "kernel": dom,
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(dom),
            "alg_bytes_per_launch": alg[dom],
            "avg_launch_us": round(avg_ms * 1e3, 3),
            "launches": dom_n,
            "timing": "HIP events around graph replays of this launch alone over the weight "
                      "copies; includes in-graph launch gaps (kernel-only durations: rocprof "
                      "summary under profiles/)",
        },
        "kernels": per_kernel,
    }
    if not args.no_secondary:
        result["secondary"] = secondary(g, torch, synth)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(synth, args.cpu_reps,
                                              result.get("secondary"), value, alg, per_kernel)
    print(json.dumps(result), flush=True)


# --------------------------------------------------------------------------- #
COPY_BYTES = 512 << 20
COPY_REPS = 4
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_q8_0_layer_set.json")


def calibrate_copy(torch):
    """A plain device-to-device copy of COPY_BYTES, COPY_REPS times: the HBM
    counters of its kernel (FETCH_SIZE, WRITE_SIZE) against the known bytes give
    the counters' scale factors."""
    dev = torch.device("cuda:0")
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(COPY_REPS):
        dst.copy_(src)
    torch.cuda.synchronize()
    return {"copy_bytes_read": COPY_BYTES, "copy_bytes_written": COPY_BYTES, "reps": COPY_REPS}


# The sources the layer-set launches are built from (their kernels, the shared
# device helpers, the dispatch and its plans) and the build flags.
LAYER_SET_SOURCES = ("api.hip", "gemv.hip", "gemv_core.h", "gemv_mfma.hip", "gemv_mfma_core.h",
                     "ggq_device.h", "ggq_launch.h")


def kernel_sources_digest():
    """sha256 over the layer-set launches' sources and build flags; counter-derived
    traffic is reported only while it matches the sources the counters were taken from."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "quantized_gguf_q8_amd", "csrc")
    for name in LAYER_SET_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    with open(os.path.join(ROOT, "quantized_gguf_q8_amd", "build.py"), "rb") as f:
        h.update(b"build.py\0" + f.read())   # compiler flags change the code too
    return h.hexdigest()


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the calibrated counter runs
    recorded in TRAFFIC_FILE, or None when absent or taken on other sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("sources_sha256") != kernel_sources_digest():
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else k.get("bytes_per_launch")


# --------------------------------------------------------------------------- #
def secondary(g, torch, synth, only=None):
    dev = torch.device("cuda:0")
    out = {}
    if only in (None, "hbm"):
        # What plain streams reach on this device, as a reference for the
        # weight GB/s figures: a 1 GiB device copy (bytes read + written) and a
        # library sum over 1 GiB (bytes read), 10 back-to-back eager calls each
        # (the sum is kept out of graphs: it may record a memset node).
        src = torch.ones((1 << 30) // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        acc = torch.empty((), dtype=torch.float32, device=dev)

        def eager_ms(fn, reps=10):
            fn()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / reps

        copy_ms = eager_ms(lambda: dst.copy_(src))
        read_ms = eager_ms(lambda: torch.sum(src, dim=0, out=acc))
        out["hbm_reference"] = {
            "copy_GB/s": round(2 * src.nbytes / (copy_ms * 1e-3) / 1e9, 1),
            "sum_read_GB/s": round(src.nbytes / (read_ms * 1e-3) / 1e9, 1),
            "note": "torch device copy (read + write bytes) and torch.sum (read bytes), 1 GiB each",
        }
        del src, dst, acc
    if only in (None, "small"):
        # the 1024 x 1024 Q8_0 single-token product (batch 1 on the vector
        # units; batch 8 through the single-launch matrix-core path); one
        # call is one launch, replayed 16 to a graph over >= 1 GiB of copies
        res = {}
        n = k = 1024
        w = synth.q8_0_matrix(n, k, seed=0, tensor_id=synth.tid(3, n, k))
        copies = max(2, -(-ROTATE_BYTES // w.nbytes))
        wd = torch.from_numpy(w).to(dev)
        cps = [wd.clone() for _ in range(copies)]
        for b in (1, 8):
            x = torch.from_numpy(synth.normal_f32((b, k), 0, synth.tid(3, n, k) + b)).to(dev)
            y = torch.empty((b, n), dtype=torch.float32, device=dev)
            calls = [g.GemvGroup(g.Q8_0, [(c, n, k, x, y)], ws=None if b == 1 else "auto")
                     for c in cps]
            per = 16
            fns = [(lambda j0: (lambda: [calls[(j0 + j) % copies]() for j in range(per)]))(j0)
                   for j0 in range(0, copies, per)]
            graphs = capture(torch, fns)
            ms = replay_ms(torch, graphs, 2 * len(graphs), per)
            gbs = w.nbytes / (ms * 1e-3) / 1e9
            res[f"q8_0_{n}x{k}_b{b}"] = {"us": round(ms * 1e3, 3), "GB/s": round(gbs, 1),
                                        "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                                        "alg_bytes": int(w.nbytes + 8 * b * k)}
            del graphs, calls
        del cps, wd
        out["q8_0_gemv_small"] = res
    if only in (None, "q4k"):
        res = {}
        for name, n, k in synth.Q4K_FFN_PAIR:
            w = synth.q4_k_matrix(n, k, seed=0, tensor_id=synth.tid(2, n, k))
            copies = max(2, -(-ROTATE_BYTES // w.nbytes))
            wd = torch.from_numpy(w).to(dev)
            cps = [wd.clone() for _ in range(copies)]
            for b in (1, 4, 16):
                # with a workspace every batch takes the single-launch
                # matrix-core kernel (batch 1 included, at these sizes)
                x = torch.from_numpy(synth.normal_f32((b, k), 0, synth.tid(2, n, k) + 1)).to(dev)
                y = torch.empty((b, n), dtype=torch.float32, device=dev)
                calls = [g.GemvGroup(g.Q4_K, [(c, n, k, x, y)], ws="auto") for c in cps]
                per = 16
                fns = [(lambda j0: (lambda: [calls[(j0 + j) % copies]() for j in range(per)]))(j0)
                       for j0 in range(0, copies, per)]
                graphs = capture(torch, fns)
                ms = replay_ms(torch, graphs, 4 * len(graphs), per)
                gbs = w.nbytes / (ms * 1e-3) / 1e9
                res[f"{name}_{n}x{k}_b{b}"] = {"us": round(ms * 1e3, 3), "GB/s": round(gbs, 1),
                                               "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}
                del graphs
            del cps, wd
        out["q4k_gemv"] = res
    if only in (None, "moe"):
        res = {}
        e, h, f, k = synth.MOE_EXPERTS, synth.MOE_HIDDEN, synth.MOE_FFN, synth.MOE_TOP_K
        for t in (1, 16):
            mo = synth.moe_layer(seed=0, n_tokens=t)
            wr = torch.from_numpy(mo["wr"]).to(dev)
            layer_bytes = mo["wg"].nbytes + mo["wu"].nbytes + mo["wd"].nbytes
            copies = max(2, -(-ROTATE_BYTES // layer_bytes))
            sets = [tuple(torch.from_numpy(mo[key]).to(dev) for key in ("wg", "wu", "wd"))
                    for _ in range(copies)]
            x = torch.from_numpy(mo["x"]).to(dev)
            idx0, _, _ = g.moe_route(wr, x, k)
            distinct = int(torch.unique(idx0).numel())
            ws = torch.empty(g.moe_workspace_size(e, t, k, h, f), dtype=torch.uint8, device=dev)
            y = torch.empty((t, h), dtype=torch.float32, device=dev)
            per_expert = mo["wg"][0].nbytes + mo["wu"][0].nbytes + mo["wd"][0].nbytes
            alg = distinct * per_expert + mo["wr"].nbytes

            # the layer as one call (moe_layer_gemv: for one token the router and
            # the selection are one launch), and as moe_route then moe_expert_gemv
            lws = torch.zeros(g.moe_layer_workspace_size(e, t, k, h, f), dtype=torch.uint8,
                              device=dev)
            outs = (y, torch.empty((t, k), dtype=torch.int32, device=dev),
                    torch.empty((t, k), dtype=torch.float32, device=dev),
                    torch.empty((t, e), dtype=torch.float32, device=dev))

            def layer(c):
                def run():
                    wg_, wu_, wd_ = sets[c]
                    g.moe_layer_gemv(g.Q4_K, wr, wg_, wu_, wd_, e, h, f, x, k, out=outs, ws=lws)
                return run

            def two_calls(c):
                def run():
                    wg_, wu_, wd_ = sets[c]
                    ii, pp, _ = g.moe_route(wr, x, k)
                    g.moe_expert_gemv(g.Q4_K, wg_, wu_, wd_, e, h, f, x, ii, pp, y, ws)
                return run

            # one graph runs the layer once on every weight copy
            graphs = capture(torch, [lambda: [layer(c)() for c in range(copies)]])
            ms = replay_ms(torch, graphs, 50, copies)
            del graphs
            graphs = capture(torch, [lambda: [two_calls(c)() for c in range(copies)]])
            ms2 = replay_ms(torch, graphs, 50, copies)
            gbs = alg / (ms * 1e-3) / 1e9
            res[f"t{t}"] = {"us": round(ms * 1e3, 3), "distinct_experts": distinct,
                            "alg_bytes": alg, "GB/s": round(gbs, 1),
                            "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                            "route_then_experts_us": round(ms2 * 1e3, 3)}
            del graphs, sets
        out["moe_q4k"] = res
    if only in (None, "moe_prompt"):
        # The same routed layer at prompt batch through moe_expert_gemm (grouped
        # matrix-core products), against the decode path (moe_expert_gemv) on
        # the same tokens.
        res = {}
        e, h, f, k = synth.MOE_EXPERTS, synth.MOE_HIDDEN, synth.MOE_FFN, synth.MOE_TOP_K
        for t in (64, 512):
            mo = synth.moe_layer(seed=0, n_tokens=t)
            wr = torch.from_numpy(mo["wr"]).to(dev)
            layer_bytes = mo["wg"].nbytes + mo["wu"].nbytes + mo["wd"].nbytes
            copies = max(2, -(-ROTATE_BYTES // layer_bytes))
            sets = [tuple(torch.from_numpy(mo[key]).to(dev) for key in ("wg", "wu", "wd"))
                    for _ in range(copies)]
            x = torch.from_numpy(mo["x"]).to(dev)
            idx0, _, _ = g.moe_route(wr, x, k)
            distinct = int(torch.unique(idx0).numel())
            ws = torch.empty(max(g.moe_gemm_workspace_size(e, t, k, h, f),
                                 g.moe_workspace_size(e, t, k, h, f)), dtype=torch.uint8,
                             device=dev)
            y = torch.empty((t, h), dtype=torch.float32, device=dev)
            per_expert = mo["wg"][0].nbytes + mo["wu"][0].nbytes + mo["wd"][0].nbytes
            alg = distinct * per_expert + mo["wr"].nbytes
            flop = 2.0 * t * k * 3 * h * f

            def layer(c, fn):
                def run():
                    wg_, wu_, wd_ = sets[c]
                    ii, pp, _ = g.moe_route(wr, x, k)
                    fn(g.Q4_K, wg_, wu_, wd_, e, h, f, x, ii, pp, y, ws)
                return run

            graphs = capture(torch, [lambda: [layer(c, g.moe_expert_gemm)() for c in range(copies)]])
            ms = replay_ms(torch, graphs, 20, copies)
            del graphs
            graphs = capture(torch, [lambda: [layer(c, g.moe_expert_gemv)() for c in range(copies)]])
            ms_gemv = replay_ms(torch, graphs, 3, copies)
            del graphs
            gbs = alg / (ms * 1e-3) / 1e9
            tflops = flop / (ms * 1e-3) / 1e12
            res[f"t{t}"] = {"us": round(ms * 1e3, 2), "distinct_experts": distinct,
                            "alg_bytes": alg, "GB/s": round(gbs, 1),
                            "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                            "TFLOP/s": round(tflops, 1),
                            "frac_bf16_peak": round(tflops / BF16_PEAK_TFLOPS, 4),
                            "decode_path_us": round(ms_gemv * 1e3, 2)}
            del sets
        out["moe_q4k_prompt"] = res
    if only in (None, "ffn"):
        # Dense FFN gate/up of the ~1B layer set fused with SiLU*up
        # (quant_gemv_swiglu) against the same two products as one grouped GEMV
        # that writes g and u (the activation left to a later pass).
        res = {}
        n, k = next((n, k) for name, n, k in synth.DENSE_1B_LAYER_SET if name == "gate")
        tid = synth.tid(1, n, k)
        wgh = synth.q8_0_matrix(n, k, 0, tid)
        wuh = synth.q8_0_matrix(n, k, 0, synth.tid(1, n, k) + 7)
        pair = wgh.nbytes + wuh.nbytes
        copies = max(2, -(-ROTATE_BYTES // pair))
        cps = [(torch.from_numpy(wgh).to(dev), torch.from_numpy(wuh).to(dev)) for _ in range(copies)]
        for b in (1, 8):
            x = torch.from_numpy(synth.normal_f32((b, k), 0, tid + 1)).to(dev)
            hh = torch.empty((b, n), dtype=torch.float32, device=dev)
            yg = torch.empty((b, n), dtype=torch.float32, device=dev)
            yu = torch.empty((b, n), dtype=torch.float32, device=dev)
            ws = None if b == 1 else torch.zeros(g.quant_gemv_workspace_size(g.Q8_0, k, b),
                                                 dtype=torch.uint8, device=dev)
            graphs = capture(torch, [lambda: [g.quant_gemv_swiglu(g.Q8_0, a_, u_, n, k, x, hh, ws)
                                              for a_, u_ in cps]])
            fused = replay_ms(torch, graphs, 10, copies)
            del graphs
            calls = [g.GemvGroup(g.Q8_0, [(a_, n, k, x, yg), (u_, n, k, x, yu)],
                                 ws=None if b == 1 else "auto") for a_, u_ in cps]
            graphs = capture(torch, [lambda: [c() for c in calls]])
            grouped = replay_ms(torch, graphs, 10, copies)
            del graphs, calls
            res[f"gate_up_{n}x{k}_b{b}"] = {
                "fused_us": round(fused * 1e3, 2),
                "fused_GB/s": round(pair / (fused * 1e-3) / 1e9, 1),
                "fused_frac_hbm": round(pair / (fused * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "grouped_two_gemv_us": round(grouped * 1e3, 2)}
        del cps
        out["ffn_swiglu_q8_0"] = res
    if only in (None, "sweep"):
        # Batch and prompt sweep on the Q4_K up projection: the decode GEMV
        # (batch 1..16, matrix cores from 2) against the GEMM at M = batch, then
        # the GEMM from just past the GEMV's 16 rows to pp2048.
        res = {}
        name, fmt, n, k = synth.PP512_GEMMS[0]
        tid = synth.tid(4, n, k)
        wh = synth.quant_matrix(fmt, n, k, seed=0, tensor_id=tid)
        copies = max(2, -(-ROTATE_BYTES // wh.nbytes))
        cps = [torch.from_numpy(wh).to(dev) for _ in range(copies)]
        for m in (1, 4, 16, 17, 32, 64, 128, 256, 512, 1024, 2048):
            a = torch.from_numpy(synth.normal_f32((m, k), 1, tid + m)).to(dev)
            c = torch.empty((m, n), dtype=torch.float32, device=dev)
            row = {}
            if m <= 16:
                calls = [g.GemvGroup(fmt, [(cw, n, k, a, c)], ws=None if m == 1 else "auto")
                         for cw in cps]
                graphs = capture(torch, [lambda: [call() for call in calls]])
                ms = replay_ms(torch, graphs, 10, copies)
                row["gemv_us"] = round(ms * 1e3, 2)
                row["gemv_GB/s"] = round(wh.nbytes / (ms * 1e-3) / 1e9, 1)
                del graphs, calls
            wsg = torch.zeros(g.quant_gemm_workspace_size(fmt, m, n, k), dtype=torch.uint8,
                              device=dev)
            graphs = capture(torch, [lambda: [g.quant_gemm(fmt, cw, n, k, a, c, wsg)
                                              for cw in cps]])
            ms = steady_ms(torch, graphs[0], copies)
            tflops = 2.0 * m * n * k / (ms * 1e-3) / 1e12
            row["gemm_us"] = round(ms * 1e3, 2)
            row["gemm_TFLOP/s"] = round(tflops, 1)
            row["gemm_frac_bf16_peak"] = round(tflops / BF16_PEAK_TFLOPS, 4)
            row["gemm_weight_GB/s"] = round(wh.nbytes / (ms * 1e-3) / 1e9, 1)
            res[f"m{m}"] = row
            del graphs, wsg
        del cps
        out["sweep_q4k_up"] = res
    if only in (None, "gemm"):
        # one call per weight copy (>= 1 GiB of copies, so every call reads its
        # weights from HBM), at steady state (see steady_ms)
        res = {}
        m = synth.PP512_M
        for name, fmt, n, k in synth.PP512_GEMMS:
            tid = synth.tid(4, n, k)
            wh = torch.from_numpy(synth.quant_matrix(fmt, n, k, seed=0, tensor_id=tid))
            copies = max(2, -(-ROTATE_BYTES // wh.nbytes))
            cps = [wh.to(dev) for _ in range(copies)]
            a = torch.from_numpy(synth.normal_f32((m, k), 0, tid + 1)).to(dev)
            c = torch.empty((m, n), dtype=torch.float32, device=dev)
            ws = torch.zeros(g.quant_gemm_workspace_size(fmt, m, n, k), dtype=torch.uint8,
                             device=dev)
            graphs = capture(torch, [lambda: [g.quant_gemm(fmt, cw, n, k, a, c, ws)
                                              for cw in cps]])
            ms = steady_ms(torch, graphs[0], copies)
            tflops = 2.0 * m * n * k / (ms * 1e-3) / 1e12
            res[name] = {"shape": f"{m}x{n}x{k}", "us": round(ms * 1e3, 2),
                         "TFLOP/s": round(tflops, 1),
                         "frac_bf16_peak": round(tflops / BF16_PEAK_TFLOPS, 4)}
            del graphs, cps
        out["pp512_gemm"] = res
    return out


def _cpu_info():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, os.cpu_count() or 1


def _median_time(fn, reps):
    fn()   # warm-up
    ts = []
    for _ in range(reps):
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
    ts.sort()
    return ts[len(ts) // 2]


def cpu_baseline(synth, reps, secondary, value, alg, per_kernel):
    """The oracle (plain C, fp64 accumulation) on bounded samples of every
    configuration, with 1 thread and with all the threads the host gives one GPU
    (rows or columns split across threads), median of `reps` runs after one
    warm-up.  Rates use the same algorithmic units as the GPU figures (weight
    bytes of the sample, or 2*M*N*K flop), so each row sits next to its GPU
    number.  A reported baseline, not the target."""
    import numpy as np
    import oracle

    model, nproc = _cpu_info()
    # the machine's CPU share for one GPU is 16 threads, whatever nproc reports
    full = max(1, min(nproc, 16))
    rows = []
    sec = secondary or {}

    def add(config, unit, work, sample, fn_for, gpu=None):
        r = {"config": config, "unit": unit, "sample": sample}
        for th in (1, full):
            t = _median_time(lambda: fn_for(th), reps)
            r[f"threads_{th}"] = round(work / t / (1e9 if unit in ("GB/s", "GFLOP/s") else 1), 3)
        r["gpu"] = gpu
        rows.append(r)
        return r

    # the 1024 x 1024 Q8_0 GEMV: the whole matrix, batch 1
    n = k = 1024
    w = synth.q8_0_matrix(n, k, seed=0, tensor_id=synth.tid(3, n, k))
    x = synth.normal_f32((1, k), 0, synth.tid(3, n, k) + 1)
    add("q8_0_gemv_1024x1024_b1", "GB/s", w.nbytes, "whole matrix",
        lambda th: oracle.gemv(synth.FMT_Q8_0, w, n, k, x, threads=th),
        sec.get("q8_0_gemv_small", {}).get("q8_0_1024x1024_b1", {}).get("GB/s"))
    # the layer set at batch 1 and 8: the first 1/8 of every matrix's rows
    sets = []
    for name, n, k in synth.DENSE_1B_LAYER_SET:
        w = synth.q8_0_matrix(n, k, seed=0, tensor_id=synth.tid(1, n, k))
        sets.append((name, n // 8, k, np.ascontiguousarray(w[: n // 8])))
    wb = sum(ws.nbytes for _, _, _, ws in sets)
    for b in (1, 8):
        xs = {name: synth.normal_f32((b, k), seed=0, tensor_id=synth.tid(1, n * 8, k) + b)
              for name, n, k, _ in sets}

        def run(th, xs=xs):
            for name, n, k, ws in sets:
                oracle.gemv(synth.FMT_Q8_0, ws, n, k, xs[name], threads=th)
        label = f"gemv_q8_0_grouped_b{b}"
        gpu = per_kernel.get(label, {}).get("GB/s")
        add(f"q8_0_layer_set_b{b}", "GB/s", wb, f"first 1/8 of each matrix's rows ({wb} B)",
            run, gpu)
    # the Q4_K pair at batch 1, 4, 16: the first 1/16 of the rows
    for name, n, k in synth.Q4K_FFN_PAIR:
        w = synth.q4_k_matrix(n, k, seed=0, tensor_id=synth.tid(2, n, k))
        ns = n // 16
        ws = np.ascontiguousarray(w[:ns])
        for b in (1, 4, 16):
            x = synth.normal_f32((b, k), 0, synth.tid(2, n, k) + 1)
            add(f"q4k_gemv_{n}x{k}_b{b}", "GB/s", ws.nbytes, f"first {ns} of {n} rows",
                lambda th, ws=ws, ns=ns, k=k, x=x: oracle.gemv(synth.FMT_Q4_K, ws, ns, k, x,
                                                              threads=th),
                sec.get("q4k_gemv", {}).get(f"{name}_{n}x{k}_b{b}", {}).get("GB/s"))
    # the routed layer: 1 token (whole layer) and the first 4 of 16 tokens
    e, h, f, top = synth.MOE_EXPERTS, synth.MOE_HIDDEN, synth.MOE_FFN, synth.MOE_TOP_K
    for t, ts in ((1, 1), (16, 4)):
        mo = synth.moe_layer(seed=0, n_tokens=t)
        xs = mo["x"][:ts]
        lg, _ = oracle.router_logits(mo["wr"], xs)
        idx = oracle.topk(lg, top)
        probs = oracle.route_probs(lg, idx)
        per_expert = mo["wg"][0].nbytes + mo["wu"][0].nbytes + mo["wd"][0].nbytes
        work = len(set(idx.ravel().tolist())) * per_expert + mo["wr"].nbytes

        def run(th, mo=mo, xs=xs):
            l2, _ = oracle.router_logits(mo["wr"], xs)
            i2 = oracle.topk(l2, top)
            oracle.moe(synth.FMT_Q4_K, mo["wg"], mo["wu"], mo["wd"], e, h, f, xs, i2,
                       oracle.route_probs(l2, i2), threads=th)
        add(f"moe_q4k_t{t}", "GB/s", work,
            f"tokens 0..{ts - 1} of {t}: routing and expert layer, {work} weight bytes", run,
            sec.get("moe_q4k", {}).get(f"t{t}", {}).get("GB/s"))
    # the pp512 GEMMs: 16 output columns of all 512 rows
    for name, fmt, n, k in synth.PP512_GEMMS:
        tid = synth.tid(4, n, k)
        w = synth.quant_matrix(fmt, n, k, seed=0, tensor_id=tid)
        a = synth.normal_f32((synth.PP512_M, k), 0, tid + 1)
        cols = list(range(16))
        add(f"pp512_gemm_{name}", "GFLOP/s", 2.0 * synth.PP512_M * len(cols) * k,
            f"{len(cols)} of {n} output columns, all {synth.PP512_M} rows",
            lambda th, w=w, n=n, k=k, a=a, fmt=fmt: oracle.gemm_columns(fmt, w, n, k, a, cols,
                                                                        threads=th),
            (lambda r: None if r is None else round(r * 1e3, 1))(
                sec.get("pp512_gemm", {}).get(name, {}).get("TFLOP/s")))
    head = next(r for r in rows if r["config"] == "q8_0_layer_set_b1")
    head8 = next(r for r in rows if r["config"] == "q8_0_layer_set_b8")
    # the headline rate: the layer-set step (batch 1 then batch 8) with all threads
    step = 2.0 / (1.0 / head[f"threads_{full}"] + 1.0 / head8[f"threads_{full}"])
    return {"value": round(step, 3), "unit": "GB/s", "cores": full, "kind": "oracle",
            "sample": "layer set, batch 1 then batch 8, first 1/8 of each matrix's rows; "
                      f"median of {reps} runs after one warm-up, {full} threads",
            "nproc": nproc, "cpu_model": model, "gpu_value": round(value, 2),
            "configs": rows}


if __name__ == "__main__":
    main()
