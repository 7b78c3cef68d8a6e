#!/usr/bin/env python3
"""Benchmark of the gated-delta-rule decode path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2] [--rotate R]
                    [--cpu-seconds S] [--no-cpu-baseline]

One step is the whole path over one batch: the gate front end (g = decay_scale *
softplus(a + dt_bias), beta = sigmoid(b)) and the decode step, in place on the state pool,
in the HIP library through its C ABI. By default the step is one launch of
rgdr_decode_gated (the gate computed in the decode kernel's prologue); the two-launch chain
la_gate -> rgdr_decode is timed as well and reported as `unfused_ms_per_step`. The default
workload is the batched GQA decode shape (B=64, H_q=16, H_v=32, T=1, D_k=D_v=128, a
256-slot pool, 64 slots in use), with gate inputs that reproduce its g/beta recipe.

Measurement:
  * R independent buffer sets (pool and every per-step input/output) are rotated so that
    consecutive steps stream their state from HBM, not from the 256 MB Infinity Cache;
    R is chosen so one rotation touches >= 1 GiB of distinct state.
  * W eager warmup steps; then the K timed steps are captured in one HIP graph (so
    Python launch overhead is not measured), replayed untimed until 25 ms of work have run
    (upload, and the shader clock settling under load), and timed with events on the
    launch stream around a single replay.
  * The decode kernel's average duration: K back-to-back decode launches over the same
    rotation, captured in a graph and timed with events around each of 5 replays; the
    median replay's per-launch mean is the duration (what rocprofv3's kernel trace
    reports as the average); its roofline uses the method's algorithmic bytes per launch.
    The gate kernel is timed the same way.
  * copy_reference: a plain 256 MiB device copy (torch elementwise, read + write), timed
    the same way, as the box's practical streaming rate.
  * cpu_baseline: the fp64 C oracle repeats the same step on the host for about
    --cpu-seconds, on one thread and on one thread per host core (batch entries split
    into contiguous slices, each slice with its own compact copy of its state slots).

Prints ONE JSON line on stdout; progress goes to stderr.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "achieved HBM GB/s (% of peak) + token·head steps/sec, gated-delta decode"
HBM_PEAK_GBS = 8000.0
KERNEL_REPLAYS = 5  # kernel durations: median over this many replays of the K-launch graph
WARM_MS = 25.0      # untimed graph replays before any timed one, in wall-clock milliseconds


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def decode_bytes(inp):
    """Algorithmic bytes of one decode call: the state tile of every served (b, h) read and
    written once (bf16), per valid token-head q+k (shared over H_v/H_q heads), v, out,
    beta, g, gk, and 12 B of index data per batch entry."""
    import numpy as np
    lens = np.clip(inp.actual_seq_lengths, 0, inp.T)
    valid = (inp.ssm_state_indices >= 0) & (inp.ssm_state_indices < inp.N_slots)
    n_pairs = int(valid.sum()) * inp.Hv
    tok_heads = int(lens[valid].sum()) * inp.Hv
    per_tok = (4 * inp.Dk * inp.Hq / inp.Hv + 2 * inp.Dv + 2 * inp.Dv + 2 + 4 + 4 * inp.Dk)
    return int(n_pairs * 4 * inp.Dk * inp.Dv + tok_heads * per_tok + 12 * inp.B), tok_heads


def gate_bytes(inp):
    n = inp.B * inp.T * inp.Hv
    return n * (4 + 4 + 4 + 2) + 2 * 4 * inp.Hv  # a, b in; decay fp32, beta bf16 out; 2 [H]


def fused_bytes(inp, decode_b, tok_heads):
    """The fused step reads the raw gate projections a, b (fp32) instead of g (fp32) and
    beta (bf16) for each valid token-head, and the two per-head vectors once."""
    return decode_b + tok_heads * (4 + 4 - 4 - 2) + 2 * 4 * inp.Hv


KERNEL_SOURCES = ("gated_delta_rule_rgdr_amd/csrc/rgdr_decode.hip",
                  "gated_delta_rule_rgdr_amd/csrc/rgdr_common.h")
TRAFFIC_PROFILES = {2: "profiles/rgdr_decode_b64_gqa_d128.md",
                    3: "profiles/rgdr_decode_varlen_b32_t8_d128.md",
                    4: "profiles/rgdr_decode_b256_gqa_d128.md"}


def kernel_code_digest():
    """sha256 of the decode kernel sources with comments and whitespace removed: an edit to
    comments keeps the committed counter summaries valid, an edit to code does not."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        text = open(os.path.join(ROOT, f)).read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def measured_traffic(wid=2):
    """HBM bytes per fused call from the committed rocprofv3 counter summary of workload
    `wid`, or None when there is none or the decode kernel's code has changed since those
    counters were taken."""
    import re
    if wid not in TRAFFIC_PROFILES:
        return None
    path = os.path.join(ROOT, TRAFFIC_PROFILES[wid])
    if not os.path.exists(path):
        return None
    text = open(path).read()
    mt = re.search(r"^traffic_bytes_per_call:\s*(\d+)", text, re.M)
    mh = re.search(r"^kernel_code_sha256:\s*([0-9a-f]{64})", text, re.M)
    if not (mt and mh):
        return None
    return int(mt.group(1)) if kernel_code_digest() == mh.group(1) else None


def cpu_baseline(inp, step_bytes, tok_heads, seconds):
    """Time the oracle on the host: the whole step (gate, then decode) over the workload,
    first on one thread, then on one thread per host core. Each thread takes a contiguous
    slice of batch entries with a compact copy of the state slots they name (prepared before
    the clock starts); the oracle runs unchanged on each slice (its C calls release the
    GIL). Each mode repeats the step for about `seconds`."""
    import concurrent.futures as cf
    import platform

    import numpy as np

    import oracle

    def slices(n):
        out = []
        for bs in np.array_split(np.arange(inp.B), n):
            if len(bs) == 0:
                continue
            idx = inp.ssm_state_indices[bs]
            valid = (idx >= 0) & (idx < inp.N_slots)
            pool = inp.state[idx[valid]]
            if pool.shape[0] == 0:
                pool = np.zeros((1,) + inp.state.shape[1:], np.uint16)
            cidx = np.full(len(bs), -1, np.int32)
            cidx[valid] = np.arange(int(valid.sum()), dtype=np.int32)
            out.append(dict(a=inp.gate_a[bs], b=inp.gate_b[bs], q=inp.query[bs], k=inp.key[bs],
                            v=inp.value[bs], gk=inp.gk[bs], lens=inp.actual_seq_lengths[bs],
                            nacc=inp.num_accepted_tokens[bs], pool=pool, idx=cidx))
        return out

    def run(sl):
        d64, b64 = oracle.la_gate(sl["a"], inp.dt_bias, inp.decay_scale, sl["b"])
        g32 = np.ascontiguousarray(d64.astype(np.float32).transpose(0, 2, 1))
        beta_bits = np.ascontiguousarray(oracle.f64_to_bf16(b64).transpose(0, 2, 1))
        oracle.rgdr_bf16(sl["q"], sl["k"], sl["v"], beta_bits, sl["pool"], sl["lens"],
                         sl["idx"], g32, sl["gk"], sl["nacc"], inp.scale)

    def timed(n):
        parts = slices(n)
        t0 = time.perf_counter()
        reps = 0
        with cf.ThreadPoolExecutor(max_workers=len(parts)) as ex:
            while True:
                list(ex.map(run, parts))
                reps += 1
                el = time.perf_counter() - t0
                if el >= seconds:
                    return reps, el, len(parts)

    oracle.default()
    cores = max(1, min(len(os.sched_getaffinity(0)), 16))
    r1, e1, _ = timed(1)
    log(f"cpu oracle, 1 thread: {r1} steps in {e1:.1f} s")
    rn, en, used = timed(cores)
    log(f"cpu oracle, {used} threads: {rn} steps in {en:.1f} s")
    model = platform.processor() or "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": round(step_bytes * rn / en / 1e9, 4), "unit": "GB/s", "cores": used,
            "kind": "oracle",
            "sample": f"{rn} full steps of this workload (gate + decode, fp64 C oracle) on "
                      f"{used} threads in {en:.1f} s, batch entries split into {used} slices",
            "token_head_steps_per_s": round(tok_heads * rn / en, 1),
            "single_thread": {"value": round(step_bytes * r1 / e1 / 1e9, 4),
                              "token_head_steps_per_s": round(tok_heads * r1 / e1, 1),
                              "sample": f"{r1} full steps on 1 thread in {e1:.1f} s"},
            "cpu_model": model}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=2, choices=[0, 1, 2, 3, 4])
    ap.add_argument("--rotate", type=int, default=0, help="buffer sets (0: auto, >= 1 GiB)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB copy (read 256 MiB, write 256 MiB) five "
                         "times, as the reference for the HBM byte counters")
    ap.add_argument("--eager-only", action="store_true",
                    help="profiling pass: W + K eager steps, no graphs, no JSON line")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for {args.gpus}): the decode path has "
              "no cross-GPU work (each GPU would serve its own state slots or heads on its "
              "own), so more GPUs only repeat the one-GPU figure", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gated_delta_rule_rgdr_amd as rg
    import workloads

    rg.library()  # fails loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wid = args.workload
    inp = workloads.make_workload(wid, gate_inputs=True)
    B, Hq, Hv, T, Dk, Dv, N = inp.B, inp.Hq, inp.Hv, inp.T, inp.Dk, inp.Dv, inp.N_slots
    dbytes, tok_heads = decode_bytes(inp)
    gbytes = gate_bytes(inp)
    step_bytes = fused_bytes(inp, dbytes, tok_heads)
    touched = int(((inp.ssm_state_indices >= 0) & (inp.ssm_state_indices < N)).sum()) \
        * Hv * Dk * Dv * 2
    R = args.rotate or max(2, math.ceil((1 << 30) / max(touched, 1)))
    R = min(R, args.steps) if args.steps > 0 else R
    log(f"workload {wid}: {workloads.WORKLOAD_NAMES[wid]}; fused step bytes {step_bytes}, "
        f"unfused decode {dbytes} + gate {gbytes}; rotation sets {R}")

    def bits(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)

    base = dict(q=bits(inp.query), k=bits(inp.key), v=bits(inp.value), pool=bits(inp.state),
                gk=torch.from_numpy(inp.gk).to(dev), a=torch.from_numpy(inp.gate_a).to(dev),
                b=torch.from_numpy(inp.gate_b).to(dev))
    dt = torch.from_numpy(inp.dt_bias).to(dev)
    ds = torch.from_numpy(inp.decay_scale).to(dev)
    lens = torch.from_numpy(inp.actual_seq_lengths).to(dev)
    idx = torch.from_numpy(inp.ssm_state_indices).to(dev)
    nacc = torch.from_numpy(inp.num_accepted_tokens).to(dev)
    sets = []
    for _ in range(R):
        s = {k_: v_.clone() for k_, v_ in base.items()}
        s["g"] = torch.empty((B, T, Hv), dtype=torch.float32, device=dev)
        s["beta"] = torch.empty((B, T, Hv), dtype=torch.bfloat16, device=dev)
        s["out"] = torch.empty((B, Hv, T, Dv), dtype=torch.bfloat16, device=dev)
        if T != 1:
            s["gT"] = torch.empty((B, Hv, T), dtype=torch.float32, device=dev)
            s["betaT"] = torch.empty((B, Hv, T), dtype=torch.bfloat16, device=dev)
        sets.append(s)
    del base
    torch.cuda.synchronize()

    # g and beta come out of the gate as [B, T, H_v]; the decode reads [B, H_v, T]. With
    # T = 1 these are the same bytes. For T > 1 the unfused chain transposes them with torch
    # (part of the chain's time), while the decode kernel's own timing reads copies that
    # were transposed once beforehand.
    if T != 1:
        log("note: T > 1; the unfused chain transposes g/beta with torch between its kernels")

    def gate(s):
        rg.la_gate(s["a"], dt, ds, s["b"], decay_dtype=torch.float32,
                   beta_dtype=torch.bfloat16, decay_out=s["g"], beta_out=s["beta"])

    def transpose(s):
        s["gT"].copy_(s["g"].transpose(1, 2))
        s["betaT"].copy_(s["beta"].transpose(1, 2))

    def decode(s):
        g_ = s["g"].view(B, Hv, T) if T == 1 else s["gT"]
        be = s["beta"].view(B, Hv, T) if T == 1 else s["betaT"]
        rg.rgdr_decode(s["q"], s["k"], s["v"], be, s["pool"], lens, idx, g_, s["gk"], nacc,
                       inp.scale, out=s["out"])

    def fused(s):
        rg.rgdr_decode_gated(s["q"], s["k"], s["v"], s["a"], s["b"], dt, ds, s["pool"], lens, idx,
                             s["gk"], nacc, inp.scale, out=s["out"])

    def step(i):
        fused(sets[i % R])

    def unfused_step(i):
        s = sets[i % R]
        gate(s)
        if T != 1:
            transpose(s)
        decode(s)

    def copy_calibration():
        # A plain elementwise copy of known size: 64 Mi fp32 elements read and written once.
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        log("copy calibration: 5 x (read 256 MiB + write 256 MiB)")

    stream = torch.cuda.current_stream()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"warmup: {args.warmup} eager steps done")
    if args.eager_only:
        for i in range(args.steps):
            step(args.warmup + i)
            unfused_step(args.warmup + i)
        torch.cuda.synchronize()
        log(f"eager pass: {args.steps} steps done")
        if args.copy_calibration:
            copy_calibration()
        return

    # K timed steps in one graph.
    K = args.steps

    def warm_replays(graph):
        # Untimed replays (the first also uploads the graph) until WARM_MS of work have run
        # back to back: the shader clock takes a few milliseconds of load to settle, and a
        # replay timed straight after capture runs up to 10% slow on the latency-bound
        # multi-token kernels.
        t0 = time.perf_counter()
        while True:
            graph.replay()
            torch.cuda.synchronize()
            if (time.perf_counter() - t0) * 1e3 >= WARM_MS:
                break

    def graph_ms(body, first):
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):
            with torch.cuda.graph(graph, stream=cap):
                for i in range(K):
                    body(first + i)
        stream.wait_stream(cap)
        warm_replays(graph)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        graph.replay()
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1)

    total_ms = graph_ms(step, args.warmup)
    ms_per_step = total_ms / K
    log(f"timed: {K} steps in {total_ms:.3f} ms ({ms_per_step * 1e3:.2f} us/step)")
    for i in range(args.warmup):
        unfused_step(i)
    unfused_ms = graph_ms(unfused_step, args.warmup) / K
    log(f"unfused chain (la_gate + rgdr_decode): {unfused_ms * 1e3:.2f} us/step")

    # Kernel durations: K back-to-back launches of one kernel, captured in a graph, timed
    # with events on the launch stream around one replay (no per-launch event overhead;
    # this is the duration rocprofv3's kernel trace reports).
    def kernel_avg_us(fn):
        g = torch.cuda.CUDAGraph()
        c = torch.cuda.Stream()
        c.wait_stream(stream)
        with torch.cuda.stream(c):
            with torch.cuda.graph(g, stream=c):
                for i in range(K):
                    fn(sets[i % R])
        stream.wait_stream(c)
        warm_replays(g)
        per = []
        for _ in range(KERNEL_REPLAYS):
            a0 = torch.cuda.Event(enable_timing=True)
            a1 = torch.cuda.Event(enable_timing=True)
            a0.record(stream)
            g.replay()
            a1.record(stream)
            a1.synchronize()
            per.append(a0.elapsed_time(a1) * 1e3 / K)
        del g
        return float(sorted(per)[len(per) // 2]), per

    fused_us, fused_all = kernel_avg_us(fused)
    dec_us, _ = kernel_avg_us(decode)
    gate_us, _ = kernel_avg_us(gate)
    log(f"fused decode kernel: {fused_us:.2f} us per launch; unfused: decode {dec_us:.2f} us, "
        f"gate {gate_us:.2f} us (medians of {KERNEL_REPLAYS} replays; fused replays: "
        + " ".join(f"{x:.2f}" for x in fused_all) + ")")

    # The box's practical streaming rate: a plain 256 MiB copy (read + write), graph-timed.
    csrc = torch.ones(64 << 20, dtype=torch.float32, device=dev)
    cdst = torch.empty_like(csrc)
    cg = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    cs.wait_stream(stream)
    with torch.cuda.stream(cs):
        with torch.cuda.graph(cg, stream=cs):
            for _ in range(20):
                torch.mul(csrc, 1.0, out=cdst)
    stream.wait_stream(cs)
    cg.replay()
    torch.cuda.synchronize()
    c0 = torch.cuda.Event(enable_timing=True)
    c1 = torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    cg.replay()
    c1.record(stream)
    c1.synchronize()
    copy_us = c0.elapsed_time(c1) * 1e3 / 20
    copy_gbs = 2 * csrc.numel() * 4 / (copy_us * 1e-6) / 1e9
    del cg, csrc, cdst
    log(f"copy reference: 256 MiB read + 256 MiB write in {copy_us:.1f} us ({copy_gbs:.0f} GB/s)")

    if args.copy_calibration:
        copy_calibration()

    kernel_gbs = step_bytes / (fused_us * 1e-6) / 1e9
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    steps_per_s = tok_heads / (ms_per_step * 1e-3)

    traffic = measured_traffic(wid)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(inp, step_bytes, tok_heads, args.cpu_seconds)
    n_pairs = int(((inp.ssm_state_indices >= 0) & (inp.ssm_state_indices < N)).sum()) * Hv

    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "storage_dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": workloads.WORKLOAD_NAMES[wid] + " (gate + decode step)",
                   "step": "rgdr_decode_gated (gate fused into the decode kernel)",
                   "B": B, "H_q": Hq, "H_v": Hv, "T": T, "D_k": Dk, "D_v": Dv,
                   "N_slots": N, "rotation_sets": R, "parallelism": "none (1 GPU)"},
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "token_head_steps_per_s": round(steps_per_s, 1),
        "step_bytes": step_bytes,
        "bytes_per_state_element": round(step_bytes / (n_pairs * Dk * Dv), 4),
        "copy_reference": {"gbs": round(copy_gbs, 1), "us": round(copy_us, 2),
                           "what": "torch elementwise copy, 256 MiB read + 256 MiB write"},
        "roofline": {"kernel": "rgdr_decode_gated", "bound": "hbm",
                     "achieved": round(kernel_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(kernel_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "bytes_per_launch": step_bytes, "avg_launch_us": round(fused_us, 3),
                     "launch_us_replays": [round(x, 3) for x in fused_all]},
        "unfused_ms_per_step": round(unfused_ms, 6),
        "unfused_kernels_avg_us": {"la_gate": round(gate_us, 3), "rgdr_decode": round(dec_us, 3)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
