"""Benchmark of the routed MoE layer on one MI355X.

A step is one moe_layer_forward call (router, top-k, alignment, routed experts, shared
expert, combine) over one batch of synthetic tokens, on one of L layer replicas that all
stay resident in HBM; the replicas are cycled so that each step streams its experts from
HBM rather than from the 256 MB Infinity Cache.  Prints one JSON line.

Default workload: the Qwen3.6-35B-A3B-like decode/verify layer (hidden 2048, 256 experts,
top-8, intermediate 512, one shared expert of 512 with a sigmoid gate, bf16 weights) on a
T=8 verify block (a DFlash block-8 verify pass).
"""
import argparse
import hashlib
import re
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + achieved HBM GB/s (% of peak) at T=8 verify block, bf16"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
MFMA_FP8_PEAK_TFLOPS = 5000.0

WORKLOADS = {
    # name: (recipe, T, description)
    "qwen36_T8": ("qwen36_a3b", 8, "Qwen3.6-35B-A3B-like MoE layer, T=8 verify block"),
    "qwen36_T1": ("qwen36_a3b", 1, "Qwen3.6-35B-A3B-like MoE layer, T=1 decode"),
    "qwen36_T12": ("qwen36_a3b", 12, "Qwen3.6-35B-A3B-like MoE layer, T=12 verify block"),
    "qwen36_T16": ("qwen36_a3b", 16, "Qwen3.6-35B-A3B-like MoE layer, T=16 verify block"),
    "qwen36_T32": ("qwen36_a3b", 32, "Qwen3.6-35B-A3B-like MoE layer, T=32 (two 16-position blocks)"),
    "qwen36_zipf_T32": ("qwen36_a3b_zipf", 32, "Qwen3.6-35B-A3B-like MoE layer, T=32, Zipf(1.1) expert load"),
    "qwen36_T64": ("qwen36_a3b", 64, "Qwen3.6-35B-A3B-like MoE layer, T=64 (the largest verify block of the decode path)"),
    "flash_fp8_T1": ("flash_next_fp8", 1, "Qwen3.8-Flash-Next-like fp8 MoE layer, T=1 decode"),
    "qwen36_mxfp4_T8": ("qwen36_a3b_mxfp4", 8, "Qwen3.6-35B-A3B-like MoE layer with MXFP4 (4-bit) experts, "
                        "T=8 verify block"),
    "qwen36_mxfp4_T1": ("qwen36_a3b_mxfp4", 1, "Qwen3.6-35B-A3B-like MoE layer with MXFP4 (4-bit) experts, T=1 decode"),
    "flash_fp8_T6": ("flash_next_fp8", 6, "Qwen3.8-Flash-Next-like fp8 MoE layer, T=6 MTP verify block"),
    "prefill_T4096": ("prefill", 4096, "Qwen3.6-35B-A3B-like MoE layer, 4096-token prefill chunk"),
    "prefill_fp8_T4096": ("prefill_fp8", 4096, "Qwen3.6-35B-A3B-like MoE layer with fp8 e4m3 experts, 4096-token prefill chunk"),
    "prefill_fp8a8_T4096": ("prefill_fp8a8", 4096, "Qwen3.6-35B-A3B-like MoE layer with fp8 e4m3 experts and fp8 "
                            "activations (per-row scales), 4096-token prefill chunk"),
}

def plan_stages(plan):
    """The stage names of a plan string, in the order the library attaches stage events:
    "... stages: 0 name ...; 1 name ...; ..."."""
    body = plan.split("stages:", 1)[1]
    names = re.findall(r"(?:^|;)\s*(\d+) ([a-z_0-9]+)", body)
    assert [int(i) for i, _ in names] == list(range(len(names))), plan
    return [n for _, n in names]



def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=2400)
    p.add_argument("--warmup", type=int, default=320)
    p.add_argument("--workload", default="qwen36_T8", choices=sorted(WORKLOADS))
    p.add_argument("--replicas", type=int, default=0, help="layer replicas in HBM (0: 16 decode, 2 prefill)")
    p.add_argument("--rounds", type=int, default=3, help="the K timed steps are split into this many rounds")
    p.add_argument("--no-stream-read", action="store_true", help="skip the streaming-read context measurement")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="target wall time of each leg of the oracle baseline (one thread, all threads)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--four-kernel", action="store_true", help="run decode blocks as four kernels, not the fused one")
    p.add_argument("--no-graph", action="store_true",
                   help="time eager calls instead of replays of one captured HIP graph per replica")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                   help="only run a plain device copy of MIB MiB (5 times) for the HBM counter calibration")
    return p.parse_args()


# sources each dominant kernel is built from: a counter summary is valid only for this text
CSRC = "speculative_verify_moe_amd/csrc/"
KERNEL_SOURCES = {
    "moe_decode_fused": [CSRC + "fused.hip", CSRC + "topk.h", CSRC + "device.h", CSRC + "mxfp4.h"],
    "gemv_gate_up": [CSRC + "gemv.hip", CSRC + "device.h", CSRC + "mxfp4.h"],
    "gemm_gate_up_mfma": [CSRC + "gemm.hip", CSRC + "device.h"],
}


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_summary(path):
    """`key: value` lines of a committed profile summary (other lines are ignored)."""
    d = {}
    with open(path) as f:
        for ln in f:
            if ":" in ln and not ln.startswith((" ", "#", "|")):
                key, val = ln.split(":", 1)
                d[key.strip()] = val.strip()
    return d


def load_traffic(kernel, workload, src_hash):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it still matches the source."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_pmc.txt")
    if not os.path.exists(path):
        return None
    d = read_summary(path)
    if d.get("source_hash") != src_hash or "hbm_bytes_per_launch" not in d:
        return None
    return int(float(d["hbm_bytes_per_launch"]))


def calibrate_copy(mib):
    """A plain device-to-device copy of known size, for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    n = mib * (1 << 20)
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "copies": 5}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus}). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return

    import torch
    import speculative_verify_moe_amd as moe
    from synth import configs

    recipe, T, desc = WORKLOADS[args.workload]
    cfg = configs.CONFIGS[recipe]
    prefill = T > 64
    L_rep = args.replicas or (2 if prefill else 16)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.four_kernel:
        moe.moe_set_option(moe.MOE_OPT_DECODE_FUSED, 0)

    # ---- inputs: replica 0's expert banks, copied to L distinct HBM buffers; each replica has
    # its own router, bias and tokens (so each step touches its own set of experts)
    t0 = time.time()
    host = configs.make_layer(cfg, seed=0, replica=0)
    base = moe.Layer.from_host(host, device=dev)
    layers, xs, outs, wss, host_routers, host_x = [], [], [], [], [], []
    for r in range(L_rep):
        hr = configs.make_layer(cfg, seed=0, replica=r, with_experts=False)
        act8 = base.routed.wtype == moe.MOE_W_FP8_E4M3_A8
        mx = base.routed.wtype == moe.MOE_W_MXFP4
        routed = moe.Bank(base.routed.w_gate_up.clone(), base.routed.w_down.clone(),
                          None if base.routed.s_gate_up is None else base.routed.s_gate_up.clone(),
                          None if base.routed.s_down is None else base.routed.s_down.clone(), act8, mx)
        shared = None
        if base.shared is not None:
            shared = moe.Bank(base.shared.w_gate_up.clone(), base.shared.w_down.clone(),
                              None if base.shared.s_gate_up is None else base.shared.s_gate_up.clone(),
                              None if base.shared.s_down is None else base.shared.s_down.clone(), act8, mx)
        rb = None if hr["router_b"] is None else torch.from_numpy(hr["router_b"]).to(dev)
        sg = None if cfg.I_s == 0 else torch.from_numpy(hr["shared_gate_w"]).to(dev)
        lay = moe.Layer(torch.from_numpy(hr["router_w"]).to(dev), rb, routed, cfg.k, shared, sg, cfg.renormalize)
        xb = configs.make_tokens(cfg, T, seed=0, replica=r)
        layers.append(lay)
        xs.append(torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(dev))
        outs.append(torch.empty((T, cfg.H), dtype=torch.bfloat16, device=dev))
        wss.append(torch.zeros((moe.moe_layer_workspace_size(T, lay),), dtype=torch.uint8, device=dev))
        host_routers.append(hr)
        host_x.append(xb)
    del base
    torch.cuda.synchronize()
    setup_s = time.time() - t0
    plan = moe.moe_describe_plan(T, layers[0])
    fused = "decode-fused" in plan
    stages = plan_stages(plan)
    nst = len(stages)
    # stages on the library's second stream (the shared expert at prefill) overlap the others:
    # then a layer's kernel time is the span from the first stage's start to the last one's end
    overlapped = "second stream" in plan

    # realised routing per replica (touched experts) for the algorithmic byte counts
    touched = []
    for r in range(L_rep):
        ids = torch.empty((T, cfg.k), dtype=torch.int32, device=dev)
        moe.moe_layer_forward(xs[r], layers[r], out=outs[r], ids_out=ids, ws=wss[r])
        torch.cuda.synchronize()
        touched.append(len(np.unique(ids.cpu().numpy())))

    H, I, I_s, E, k = cfg.H, cfg.I, cfg.I_s, cfg.E, cfg.k

    def mat(rows, cols):
        # bytes of a weight matrix with its scales: bf16; fp8 codes + one fp32 per row; MXFP4
        # codes (half a byte) + one E8M0 byte per 32 weights
        if cfg.wtype == "bf16":
            return rows * cols * 2
        if cfg.wtype == "mxfp4":
            return rows * cols // 2 + rows * cols // 32
        return rows * cols + rows * 4

    def gate_up_bytes(nt):
        # weights of every touched expert (+ shared) once, tokens read, h written
        w = nt * mat(2 * I, H) + (mat(2 * I_s, H) if I_s else 0)
        return w + T * H * 2 + T * k * I * 2 + T * I_s * 2

    def layer_bytes(nt):
        w = nt * (mat(2 * I, H) + mat(H, I)) + ((mat(2 * I_s, H) + mat(H, I_s)) if I_s else 0)
        router = E * H * 4 + (E * 4 if host_routers[0]["router_b"] is not None else 0) + (H * 4 if I_s else 0)
        return w + router + 2 * T * H * 2

    flops_layer = 2 * T * k * 3 * H * I + (2 * T * 3 * H * I_s if I_s else 0)

    # ---- HIP graphs: one of the L replicas' calls in a row (steps i .. i+L-1 for i a multiple
    # of L), and one of the first K mod L of them, so that K steps are K // L replays of the
    # first and one of the second; the timed steps carry no per-call host overhead (the layer
    # call allocates nothing and captures as is)
    K = args.steps
    n_rounds = max(1, min(args.rounds, K))
    round_steps = [K * (i + 1) // n_rounds - K * i // n_rounds for i in range(n_rounds)]
    graphs = {}
    if not args.no_graph:
        cap = torch.cuda.Stream()
        for n in sorted(({L_rep} | {m % L_rep for m in round_steps}) - {0}):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                for r in range(n):
                    moe.moe_layer_forward(xs[r], layers[r], out=outs[r], ws=wss[r])
            graphs[n] = g
        torch.cuda.synchronize()

    def run_steps(n_steps):
        if graphs:
            for _ in range(n_steps // L_rep):
                graphs[L_rep].replay()
            if n_steps % L_rep:
                graphs[n_steps % L_rep].replay()
        else:
            for i in range(n_steps):
                r = i % L_rep
                moe.moe_layer_forward(xs[r], layers[r], out=outs[r], ws=wss[r])

    # ---- warmup (whole rounds of the replicas)
    run_steps(-(-args.warmup // L_rep) * L_rep)
    torch.cuda.synchronize()

    # ---- timed region: exactly K steps, in rounds, each bracketed by a device synchronisation
    round_s = []
    for m in round_steps:
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        run_steps(m)
        torch.cuda.synchronize()
        round_s.append(time.perf_counter() - t_start)
    elapsed = float(sum(round_s))
    round_rate = np.array([T * m / t for m, t in zip(round_steps, round_s)])
    cv = float(round_rate.std() / round_rate.mean()) if n_rounds > 1 else 0.0

    # ---- cold single call: a 1 GiB scratch write first (caches hold other data), then one
    # eager call on replica 0, its kernels timed by the stage events and the host clock
    scratch = torch.empty((1 << 30,), dtype=torch.uint8, device=dev)
    cold_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * nst)]
    cold_h = moe.stage_event_handles(cold_ev)
    scratch.fill_(1)
    torch.cuda.synchronize()
    moe.moe_set_stage_events(cold_h)
    t_c0 = time.perf_counter()
    moe.moe_layer_forward(xs[0], layers[0], out=outs[0], ws=wss[0])
    torch.cuda.synchronize()
    cold_wall_us = (time.perf_counter() - t_c0) * 1e6
    moe.moe_set_stage_events(None)
    cold_gpu_us = sum(cold_ev[2 * j].elapsed_time(cold_ev[2 * j + 1]) for j in range(nst)) * 1e3
    del scratch

    # ---- kernel durations: the same K steps once more as eager calls, with HIP events on every
    # stage's kernels (attached to the kernel dispatches by the library, on the launch stream).
    # stage s of step i: events[i][2s] at its first kernel's start, events[i][2s+1] at its last
    # kernel's end
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * nst)] for _ in range(K)]
    stream = torch.cuda.current_stream()
    for evs in events:
        for ev in evs:
            ev.record(stream)
    handles = [moe.stage_event_handles(evs) for evs in events]
    torch.cuda.synchronize()
    for i in range(K):
        r = i % L_rep
        moe.moe_set_stage_events(handles[i])
        moe.moe_layer_forward(xs[r], layers[r], out=outs[r], ws=wss[r])
    moe.moe_set_stage_events(None)
    torch.cuda.synchronize()

    stage_ms = np.zeros((K, nst))
    for i in range(K):
        for s in range(nst):
            stage_ms[i, s] = events[i][2 * s].elapsed_time(events[i][2 * s + 1])
    # kernel time per layer: the stages' own durations; the span from the first stage's start to
    # the last one's end also holds the eager pass's launch gaps, which graph replays do not have
    span_ms = np.array([events[i][0].elapsed_time(events[i][2 * nst - 1]) for i in range(K)])
    gpu_ms = span_ms if overlapped else stage_ms.sum(axis=1)
    nt_steps = np.array([touched[i % L_rep] for i in range(K)])

    ms_per_step = elapsed * 1e3 / K
    value = T * K / elapsed

    # dominant kernel: the fused layer kernel, the gate/up expert stream (four-kernel decode) or
    # the gate/up MFMA GEMM (prefill)
    dom = 0 if fused else (stages.index("gemm_gate_up_mfma") if prefill else stages.index("gemv_gate_up"))
    # the matrix cores' dense peak for the operand type the prefill GEMMs run in
    mfma_peak = MFMA_FP8_PEAK_TFLOPS if cfg.wtype == "fp8a8" else MFMA_BF16_PEAK_TFLOPS
    dom_name = stages[dom]
    dom_ms = stage_ms[:, dom]
    src_hash = source_hash(KERNEL_SOURCES[dom_name])
    if not prefill:
        per = layer_bytes if fused else gate_up_bytes
        alg_bytes = np.array([per(n) for n in nt_steps], dtype=np.float64)
        achieved = alg_bytes.sum() / (dom_ms.sum() * 1e-3) / 1e9
        traffic = load_traffic(dom_name, args.workload, src_hash)
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                    "kernel": dom_name, "avg_us": round(float(dom_ms.mean()) * 1e3, 2),
                    "alg_bytes_per_launch": int(alg_bytes.mean())}
    else:
        # gate/up GEMM flops: every routed slot, and every token through the shared expert when
        # the same launch carries it (not when the shared expert has stages of its own)
        fl = 2 * T * k * 2 * H * I + (0 if "shared_gate_up_mfma" in stages else 2 * T * 2 * H * I_s)
        achieved = fl / (dom_ms.mean() * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": mfma_peak,
                    "unit": "TFLOP/s", "frac": round(achieved / mfma_peak, 4),
                    "traffic": load_traffic(dom_name, args.workload, src_hash), "kernel": dom_name,
                    "avg_us": round(float(dom_ms.mean()) * 1e3, 2), "alg_flops_per_launch": int(fl)}

    lb = np.array([layer_bytes(n) for n in nt_steps], dtype=np.float64)
    layer = {"us_per_layer_wall": round(ms_per_step * 1e3, 2),
             "us_per_layer_gpu": round(float(gpu_ms.mean()) * 1e3, 2),
             "us_per_layer_eager_span": round(float(span_ms.mean()) * 1e3, 2),
             "alg_bytes_per_layer": int(lb.mean()),
             "hbm_gbs_gpu": round(lb.sum() / (gpu_ms.sum() * 1e-3) / 1e9, 1),
             "hbm_frac_gpu": round(lb.sum() / (gpu_ms.sum() * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
             "mfma_frac_gpu": round(flops_layer / (gpu_ms.mean() * 1e-3) / 1e12 / mfma_peak, 4),
             "touched_experts_mean": round(float(nt_steps.mean()), 2),
             "stage_us": {s: round(float(stage_ms[:, j].mean()) * 1e3, 2) for j, s in enumerate(stages)}}

    # ---- context: the read rate this device attains on a plain streaming read (the library's
    # measurement aid), best over a small sweep of launch shapes; the judged fractions above
    # stay against the nominal peak
    stream = None
    if not args.no_stream_read:
        stream = stream_read_context(moe, torch, achieved_layer_gbs=lb.sum() / (gpu_ms.sum() * 1e-3) / 1e9)

    # ---- CPU baseline: the fp64 oracle, as it stands, on a bounded sample of the same workload:
    # whole layer calls (router, top-k, experts, shared, combine) on the replicas in turn, first
    # on one thread, then on all the host threads the process may use (one call per thread at
    # a time; the oracle's C calls run outside Python's lock)
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        from concurrent.futures import ThreadPoolExecutor
        sample_T = 16 if prefill else T

        def oracle_call(r):
            hr = host_routers[r % L_rep]
            hl = dict(host)
            hl["router_w"], hl["router_b"] = hr["router_w"], hr["router_b"]
            if I_s:
                hl["shared_gate_w"] = hr["shared_gate_w"]
            xb = host_x[r % L_rep][:sample_T]
            lg = oracle.router_logits(xb, hr["router_w"], hr["router_b"]).astype(np.float32)
            ids, w = oracle.route_topk(lg, k, cfg.renormalize)
            oracle.moe_layer(xb, hl, ids, w, rounding=True, threads=1)

        def leg(n_threads):
            n_calls, t_c = 0, time.perf_counter()
            if n_threads == 1:
                while time.perf_counter() - t_c < args.cpu_seconds:
                    oracle_call(n_calls)
                    n_calls += 1
            else:
                with ThreadPoolExecutor(max_workers=n_threads) as pool:
                    while time.perf_counter() - t_c < args.cpu_seconds:
                        list(pool.map(oracle_call, range(n_calls, n_calls + n_threads)))
                        n_calls += n_threads
            return n_calls, time.perf_counter() - t_c

        n1, s1 = leg(1)
        nth = oracle.default_threads()
        nn, sn = leg(nth) if nth > 1 else (n1, s1)
        what = (f"oracle layer calls of {sample_T} tokens each (router, top-k, experts, shared, combine; fp64) "
                f"on the replicas in turn")
        cpu = {"value": round(nn * sample_T / sn, 3), "unit": "tokens/s", "cores": nth, "kind": "oracle",
               "sample": f"{nn} {what}, {sn:.1f} s on {nth} host threads (one call per thread)",
               "cpu": _cpu_model(),
               "single_thread": {"value": round(n1 * sample_T / s1, 3), "unit": "tokens/s", "cores": 1,
                                 "sample": f"{n1} {what}, {s1:.1f} s on one thread"}}

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": {"bf16": "bf16", "fp8": "fp8-e4m3 weights, bf16 activations",
                                               "fp8a8": "fp8-e4m3 weights and activations (row scales), "
                                                        "fp32 accumulate",
                                               "mxfp4": "mxfp4 (e2m1 + e8m0 block scales) weights, bf16 "
                                                        "activations"}[cfg.wtype],
        "data": "synthetic",
        "config": {"workload": desc, "T": T, "hidden": H, "experts": E, "top_k": k, "inter": I,
                   "shared_inter": I_s, "weights": cfg.wtype, "replicas": L_rep,
                   "path": plan.split()[0].split("=")[1]},
        "roofline": roofline, "layer": layer, "cpu_baseline": cpu, "stream_read": stream,
        "rounds": [round(float(v), 1) for v in round_rate], "round_steps": round_steps,
        "median_round_value": round(float(np.median(round_rate)), 1), "cv": round(cv, 4),
        "valid": cv <= 0.03,
        "cold": {"us_kernels": round(cold_gpu_us, 2), "us_wall": round(cold_wall_us, 2),
                 "after": "a 1 GiB device write; one eager call on replica 0"},
        "setup_s": round(setup_s, 1), "device": torch.cuda.get_device_name(0),
        "timing": (f"{n_rounds} rounds of " + ("HIP graph replays (one graph per round of the replicas)"
                                                  if graphs else "eager calls")
                   + "; value = all K steps over the summed round times; the line is invalid when the rounds' "
                     "coefficient of variation exceeds 3%; kernel durations from HIP events on a second pass "
                     "of the same steps"),
    }
    print(json.dumps(line), flush=True)


def stream_read_context(moe, torch, achieved_layer_gbs, gib=4):
    """Best read rate of moe_measure_stream_read over a few launch shapes on a gib-GiB buffer
    (5 timed launches each, after 2 untimed), with the layer's HBM rate as a fraction of it."""
    nbytes = gib << 30
    buf = torch.empty((nbytes,), dtype=torch.uint8, device="cuda:0")
    sink = torch.empty((8192,), dtype=torch.int32, device="cuda:0")
    best = None
    for blocks in (1024, 2048, 4096, 8192):
        for depth in (4, 8, 16):
            for _ in range(2):
                moe.moe_measure_stream_read(buf, blocks, depth, sink)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(5):
                moe.moe_measure_stream_read(buf, blocks, depth, sink)
            e1.record()
            torch.cuda.synchronize()
            gbs = 5 * nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9
            if best is None or gbs > best[0]:
                best = (gbs, blocks, depth)
    del buf, sink
    torch.cuda.empty_cache()
    gbs, blocks, depth = best
    return {"GBps": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4), "blocks": blocks, "depth": depth,
            "bytes": nbytes, "layer_frac_of_attained": round(achieved_layer_gbs / gbs, 4),
            "what": "moe_measure_stream_read: plain non-temporal 16-byte reads, best of 12 launch shapes "
                    "(blocks x loads in flight per thread), 5 launches each"}


def _cpu_model():
    """The host CPU as /proc/cpuinfo names it, with its family/model/stepping numbers (some
    hypervisors shorten the model name) and the logical CPUs this process may run on."""
    fields = {}
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ":" not in ln:
                    if fields:
                        break  # the first processor's block is enough
                    continue
                key, val = ln.split(":", 1)
                fields.setdefault(key.strip(), val.strip())
    except OSError:
        pass
    name = fields.get("model name", "unknown")
    ids = ", ".join(f"{k} {fields[k]}" for k in ("vendor_id", "cpu family", "model", "stepping") if k in fields)
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count() or 0
    return f"{name} ({ids}; {usable} logical CPUs usable, {os.cpu_count()} online)"


if __name__ == "__main__":
    main()
