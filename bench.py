#!/usr/bin/env python3
"""Benchmark of the gated-delta-rule path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2] [--rotate R]
                    [--extra 1,3,4,5,6] [--snapshots 3] [--cpu-seconds S] [--no-cpu-baseline]

One step is the whole path over one batch: the gate front end (g = decay_scale *
softplus(a + dt_bias), beta = sigmoid(b)) and the recurrence, in place on the state pool,
in the HIP library through its C ABI. By default the step is one launch of
rgdr_decode_gated (the gate computed in the decode kernel's prologue); the two-launch chain
la_gate -> rgdr_decode is timed as well and reported as `unfused_ms_per_step`. The default
workload is the batched GQA decode shape (B=64, H_q=16, H_v=32, T=1, D_k=D_v=128, a
256-slot pool, 64 slots in use), with gate inputs that reproduce its g/beta recipe.
Workloads 5 and 6 (T = 1024; D = 128, and the example page's head size D_k = 64, D_v = 512)
run the long-sequence entries, rgdr_prefill_gated and rgdr_prefill.

Measurement:
  * R independent buffer sets (pool and every per-step input/output) are rotated so that
    consecutive steps stream their data from HBM, not from the 256 MB Infinity Cache: one
    rotation touches >= 1 GiB of distinct state (decode) or of step data (long sequences).
  * W eager warmup steps; then the K timed steps are captured in one HIP graph (so
    Python launch overhead is not measured), replayed untimed until 25 ms of work have run
    (upload, and the shader clock settling under load), and timed with events on the
    launch stream around a single replay.
  * The fused kernel's average duration: K back-to-back calls over the same rotation,
    captured in a graph and timed with events around each of 5 replays; the median replay's
    per-call mean is the duration (what rocprofv3's kernel trace reports as the average);
    its roofline uses the method's algorithmic bytes per call. The unfused kernels are
    timed the same way.
  * `workloads`: the same kernel timing for the other workloads (--extra), so one line
    carries every workload's fused-call duration, roofline fraction and counter traffic;
    and `<id>_snapshots` (--snapshots): rgdr_decode_snapshots, the step that also stores
    the state after every token, at that workload.
  * copy_reference: a plain 256 MiB device copy (torch elementwise, read + write), timed
    the same way, as the box's practical streaming rate.
  * cpu_baseline: the fp64 C oracle repeats the step on the host for about --cpu-seconds,
    on one thread and on one thread per core of the GPU's host share (batch entries split
    into contiguous slices, each slice with its own compact copy of its state slots); where
    one full step would take longer than that, on a sample of the step's batch entries.

Prints ONE JSON line on stdout; progress goes to stderr.
"""
import argparse
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "achieved HBM GB/s (% of peak) + token·head steps/sec, gated-delta decode"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 matrix-core peak of MI355X
KERNEL_REPLAYS = 5  # kernel durations: median over this many replays of the K-call graph
WARM_MS = 25.0      # untimed graph replays before any timed one, in wall-clock milliseconds
# The host share of one GPU on the benchmark boxes: the threaded CPU baseline uses at most
# this many threads, whatever the process's affinity mask shows.
HOST_CORES_PER_GPU = 16
PREFILL_WORKLOADS = (5, 6, 7)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def decode_bytes(inp):
    """Algorithmic bytes of one call: the state tile of every served (b, h) read and
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


def prefill_mfma_flops(inp, cus):
    """Matrix-core flops the long-sequence kernel executes per call (not the method's
    algorithmic flops). Per chunk of up to 32 tokens and per 128-column item: each of its four
    waves issues 24 x (D_k / 32) products of 16x16x32 for [c k | c scale q]^T S, 6 x (D_k / 16)
    for the rank-32 update and 36 of 16x16x16 for the blockwise solve and the outputs; the
    item's M and N blocks take 18 x (D_k / 32) of 16x16x32. The library's other tile widths
    scale each wave's share with the columns and keep the M and N blocks: 256-column items
    at D_k = 64 when D_v is a multiple of 256 and the call has more 128-column items than
    the device's `cus` compute units hold at two per unit; 64-column items at D_k = 128
    when it has at most cus / 2 of them. Chunks split at the accepted prefix's end; chunks shortened by the
    decay range (rare at these decays) are not counted."""
    import numpy as np
    lens = np.clip(inp.actual_seq_lengths, 0, inp.T)
    nacc = np.clip(inp.num_accepted_tokens, 0, lens)
    valid = (inp.ssm_state_indices >= 0) & (inp.ssm_state_indices < inp.N_slots)
    chunks = 0
    for L, n, ok in zip(lens, nacc, valid):
        if ok and L > 0:
            chunks += -(-int(L) // 32) + (1 if 0 < n < L and n % 32 else 0)
    narrow_items = inp.B * inp.Hv * -(-inp.Dv // 128)
    if inp.Dk == 64 and inp.Dv % 256 == 0 and narrow_items > 2 * cus:
        nc = 4                                  # column sets per lane
    elif inp.Dk == 128 and 2 * narrow_items <= cus:
        nc = 1
    else:
        nc = 2
    items = inp.Hv * -(-inp.Dv // (64 * nc))
    npb, nrb = inp.Dk // 32, inp.Dk // 16
    big = 4 * (12 * npb + 3 * nrb) * nc + 18 * npb  # 16x16x32 products per item and chunk
    small = 4 * 18 * nc                         # 16x16x16 products
    return chunks * items * (big * 16 * 16 * 32 * 2 + small * 16 * 16 * 16 * 2)


def segmented_mfma_flops(inp, cus):
    """Matrix-core flops the segmented form's two passes execute per call (the scan's fp32
    products run on the VALU and are not counted). Segments as the library cuts them: the
    second pass's items per segment (128-column tiles) fill two per compute unit, at most
    16 segments, each a multiple of 32 tokens; the prefix [0, n) and the rest [n, L) are
    cut separately. Each segment is walked in chunks of up to 32 tokens; the first pass
    carries D_v + D_k columns and computes no outputs, the second carries D_v."""
    import numpy as np
    per = inp.B * inp.Hv * -(-inp.Dv // 128)
    want = min(16, 2 * cus // per)
    sl = -(-(-(-inp.T // want)) // 32) * 32
    lens = np.clip(inp.actual_seq_lengths, 0, inp.T)
    nacc = np.clip(inp.num_accepted_tokens, 0, lens)
    valid = (inp.ssm_state_indices >= 0) & (inp.ssm_state_indices < inp.N_slots)
    chunks = 0
    for L, n, ok in zip(lens, nacc, valid):
        if not ok:
            continue
        for a0, a1 in ((0, int(n)), (int(n), int(L))):
            for t0 in range(a0, a1, sl):
                chunks += -(-(min(t0 + sl, a1) - t0) // 32)
    npb, nrb = inp.Dk // 32, inp.Dk // 16
    # second pass: the single pass's products at 128-column tiles; first pass: no outputs,
    # so [c scale q]^T S and the N U products are not issued (the M and N blocks are)
    big_b, small_b = 4 * (12 * npb + 3 * nrb) * 2 + 18 * npb, 4 * 18 * 2
    big_a, small_a = 4 * (6 * npb + 3 * nrb) * 2 + 18 * npb, 4 * 9 * 2
    fl = lambda big, small: big * 16 * 16 * 32 * 2 + small * 16 * 16 * 16 * 2
    items_a = inp.Hv * -(-(inp.Dv + inp.Dk) // 128)
    items_b = inp.Hv * -(-inp.Dv // 128)
    return chunks * (items_a * fl(big_a, small_a) + items_b * fl(big_b, small_b))


SOURCES_COMMON = ("gated_delta_rule_rgdr_amd/csrc/rgdr_device.h",
                  "gated_delta_rule_rgdr_amd/csrc/rgdr_common.h")
SOURCES_DECODE = ("gated_delta_rule_rgdr_amd/csrc/rgdr_decode.hip",) + SOURCES_COMMON
SOURCES_PREFILL = ("gated_delta_rule_rgdr_amd/csrc/rgdr_prefill.hip",) + SOURCES_COMMON
# Counter summaries by (workload, batch size; None = the workload's own).
TRAFFIC_PROFILES = {(2, 16): "profiles/rgdr_decode_b16_gqa_d128.md",
                    1: "profiles/rgdr_decode_b1_h64_dk64_dv512.md",
                    2: "profiles/rgdr_decode_b64_gqa_d128.md",
                    3: "profiles/rgdr_decode_varlen_b32_t8_d128.md",
                    4: "profiles/rgdr_decode_b256_gqa_d128.md",
                    5: "profiles/rgdr_prefill_b16_t1024_gqa_d128.md",
                    6: "profiles/rgdr_prefill_b4_h64_t1024_dk64_dv512.md",
                    7: "profiles/rgdr_prefill_segmented_b1_t8192_gqa_d128.md",
                    (3, "snapshots"): "profiles/rgdr_decode_snapshots_varlen_b32_t8_d128.md"}


def kernel_code_digest(wid=2):
    """sha256 of the sources of the kernel that serves workload `wid`, with comments and
    whitespace removed: an edit to comments keeps the committed counter summaries valid, an
    edit to code does not."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in (SOURCES_PREFILL if wid in PREFILL_WORKLOADS else SOURCES_DECODE):
        text = open(os.path.join(ROOT, f)).read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def measured_traffic(wid=2, batch=None):
    """HBM bytes per fused call from the committed rocprofv3 counter summary of workload
    `wid` (at batch size `batch`, if it replaces the workload's; "snapshots" for the
    rgdr_decode_snapshots call), or None when there is none or the kernel's code has
    changed since those counters were taken."""
    import re
    key = wid if batch is None else (wid, batch)
    if key not in TRAFFIC_PROFILES:
        return None
    path = os.path.join(ROOT, TRAFFIC_PROFILES[key])
    if not os.path.exists(path):
        return None
    text = open(path).read()
    mt = re.search(r"^traffic_bytes_per_call:\s*(\d+)", text, re.M)
    mh = re.search(r"^kernel_code_sha256:\s*([0-9a-f]{64})", text, re.M)
    if not (mt and mh):
        return None
    return int(mt.group(1)) if kernel_code_digest(wid) == mh.group(1) else None


def cpu_baseline(inp, seconds):
    """Time the oracle on the host: the whole step (gate, then the recurrence), first on one
    thread, then on one thread per core of the GPU's host share. Each thread takes a
    contiguous slice of batch entries with a compact copy of the state slots they name
    (prepared before the clock starts); the oracle runs unchanged on each slice (its C calls
    release the GIL). Each mode repeats its sample for about `seconds`. The sample is the
    whole batch unless one pass would exceed about 1e9 state-element updates per thread
    (several seconds of the oracle); then it is the first entries of the batch, sized to
    that, and the rate is that sample's algorithmic bytes over its time."""
    import concurrent.futures as cf
    import platform

    import numpy as np

    import oracle

    lens = np.clip(inp.actual_seq_lengths, 0, inp.T)
    per_entry = np.maximum(lens, 1).astype(np.float64) * inp.Hv * inp.Dk * inp.Dv
    budget = 1e9

    def sample_size(threads):
        total = 0.0
        for n_ent in range(1, inp.B + 1):
            total += per_entry[n_ent - 1]
            if total > budget * threads:
                return max(n_ent - 1, min(threads, inp.B))
        return inp.B

    def sub(inp_, bs):
        import copy
        s = copy.copy(inp_)
        for name in ("query", "key", "value", "beta", "g", "gk", "ssm_state_indices",
                     "actual_seq_lengths", "num_accepted_tokens", "gate_a", "gate_b"):
            setattr(s, name, getattr(inp_, name)[bs])
        s.B = len(bs)
        return s

    def slices(entries, n):
        out = []
        for bs in np.array_split(entries, n):
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
        entries = np.arange(sample_size(n))
        parts = slices(entries, n)
        s = sub(inp, entries)
        db, th = decode_bytes(s)
        sbytes = fused_bytes(s, db, th)
        t0 = time.perf_counter()
        reps = 0
        with cf.ThreadPoolExecutor(max_workers=len(parts)) as ex:
            while True:
                list(ex.map(run, parts))
                reps += 1
                el = time.perf_counter() - t0
                if el >= seconds:
                    return reps, el, len(parts), len(entries), sbytes, th

    oracle.default()
    affinity = len(os.sched_getaffinity(0))
    cores = max(1, min(affinity, HOST_CORES_PER_GPU))
    r1, e1, _, n1, b1, th1 = timed(1)
    log(f"cpu oracle, 1 thread: {r1} passes over {n1} entries in {e1:.1f} s")
    rn, en, used, nn, bn, thn = timed(cores)
    log(f"cpu oracle, {used} threads: {rn} passes over {nn} entries in {en:.1f} s "
        f"(affinity mask: {affinity} cores)")
    model = platform.processor() or "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    what = "full steps of this workload" if nn == inp.B else \
        f"passes over the first {nn} of the step's {inp.B} batch entries"
    what1 = "full steps" if n1 == inp.B else f"passes over the first {n1} entries"
    return {"value": round(bn * rn / en / 1e9, 4), "unit": "GB/s", "cores": used,
            "kind": "oracle",
            "sample": f"{rn} {what} (gate + recurrence, fp64 C oracle) on {used} threads in "
                      f"{en:.1f} s, entries split into {used} slices",
            "token_head_steps_per_s": round(thn * rn / en, 1),
            "single_thread": {"value": round(b1 * r1 / e1 / 1e9, 4),
                              "token_head_steps_per_s": round(th1 * r1 / e1, 1),
                              "sample": f"{r1} {what1} on 1 thread in {e1:.1f} s"},
            "cpu_model": model, "affinity_cores": affinity,
            "threads_cap": f"at most {HOST_CORES_PER_GPU} threads: the host share of one GPU"}


class Workload:
    """Device buffers of one workload, rotated over R sets, and its calls."""

    def __init__(self, wid, dev, rotate=0, steps=200, batch=None):
        import numpy as np
        import torch

        import gated_delta_rule_rgdr_amd as rg
        import workloads
        self.rg, self.torch = rg, torch
        self.cus = torch.cuda.get_device_properties(dev).multi_processor_count
        self.wid = wid
        self.batch = batch
        self.name = workloads.WORKLOAD_NAMES[wid]
        if batch is not None:
            self.name = re.sub(r"B=\d+", f"B={batch}", self.name)
        self.prefill = wid in PREFILL_WORKLOADS
        inp = self.inp = workloads.make_workload(wid, gate_inputs=True, batch=batch)
        B, Hv, T, Dk, Dv, N = inp.B, inp.Hv, inp.T, inp.Dk, inp.Dv, inp.N_slots
        self.dbytes, self.tok_heads = decode_bytes(inp)
        self.gbytes = gate_bytes(inp)
        self.step_bytes = fused_bytes(inp, self.dbytes, self.tok_heads)
        self.n_pairs = int(((inp.ssm_state_indices >= 0) & (inp.ssm_state_indices < N)).sum()) * Hv
        touched = self.n_pairs * Dk * Dv * 2
        if self.prefill:
            touched = self.step_bytes  # every step streams far more than its state
        R = rotate or max(2, math.ceil((1 << 30) / max(touched, 1)))
        self.R = min(R, steps) if steps > 0 else R

        def bits(x):
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)

        base = dict(q=bits(inp.query), k=bits(inp.key), v=bits(inp.value), pool=bits(inp.state),
                    gk=torch.from_numpy(inp.gk).to(dev), a=torch.from_numpy(inp.gate_a).to(dev),
                    b=torch.from_numpy(inp.gate_b).to(dev))
        self.dt = torch.from_numpy(inp.dt_bias).to(dev)
        self.ds = torch.from_numpy(inp.decay_scale).to(dev)
        self.lens = torch.from_numpy(inp.actual_seq_lengths).to(dev)
        self.idx = torch.from_numpy(inp.ssm_state_indices).to(dev)
        self.nacc = torch.from_numpy(inp.num_accepted_tokens).to(dev)
        self.sets = []
        for _ in range(self.R):
            s = {k_: v_.clone() for k_, v_ in base.items()}
            s["g"] = torch.empty((B, T, Hv), dtype=torch.float32, device=dev)
            s["beta"] = torch.empty((B, T, Hv), dtype=torch.bfloat16, device=dev)
            s["out"] = torch.empty((B, Hv, T, Dv), dtype=torch.bfloat16, device=dev)
            if T != 1:
                s["gT"] = torch.empty((B, Hv, T), dtype=torch.float32, device=dev)
                s["betaT"] = torch.empty((B, Hv, T), dtype=torch.bfloat16, device=dev)
            self.sets.append(s)
        del base
        torch.cuda.synchronize()
        self.fused_fn = rg.rgdr_prefill_gated if self.prefill else rg.rgdr_decode_gated
        self.decode_fn = rg.rgdr_prefill if self.prefill else rg.rgdr_decode
        self.fused_name = "rgdr_prefill_gated" if self.prefill else "rgdr_decode_gated"
        self.decode_name = "rgdr_prefill" if self.prefill else "rgdr_decode"
        # Long sequences with too few (entry, head) pairs to fill the device take the
        # segmented form, through the workspace entries (one workspace, every call in order
        # on one stream).
        self.ws_bytes = rg.rgdr_prefill_workspace_size(B, Hv, T, Dk, Dv, dev) if self.prefill else 0
        self.ws = None
        if self.ws_bytes:
            self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)
            ws = self.ws
            self.single_fused_fn = self.fused_fn
            self.fused_fn = lambda *a_, **k_: rg.rgdr_prefill_gated_ws(*a_, workspace=ws, **k_)
            self.decode_fn = lambda *a_, **k_: rg.rgdr_prefill_ws(*a_, workspace=ws, **k_)
            self.fused_name = "rgdr_prefill_gated_ws (segmented)"
            self.decode_name = "rgdr_prefill_ws (segmented)"

    # g and beta come out of the gate as [B, T, H_v]; the recurrence reads [B, H_v, T]. With
    # T = 1 these are the same bytes. For T > 1 the unfused chain transposes them with torch
    # (part of the chain's time), while the unfused kernel's own timing reads copies that
    # were transposed once beforehand.
    def gate(self, s):
        self.rg.la_gate(s["a"], self.dt, self.ds, s["b"], decay_dtype=self.torch.float32,
                        beta_dtype=self.torch.bfloat16, decay_out=s["g"], beta_out=s["beta"])

    def transpose(self, s):
        s["gT"].copy_(s["g"].transpose(1, 2))
        s["betaT"].copy_(s["beta"].transpose(1, 2))

    def decode(self, s):
        inp = self.inp
        B, Hv, T = inp.B, inp.Hv, inp.T
        g_ = s["g"].view(B, Hv, T) if T == 1 else s["gT"]
        be = s["beta"].view(B, Hv, T) if T == 1 else s["betaT"]
        self.decode_fn(s["q"], s["k"], s["v"], be, s["pool"], self.lens, self.idx, g_, s["gk"],
                       self.nacc, inp.scale, out=s["out"])

    def fused(self, s):
        self.fused_fn(s["q"], s["k"], s["v"], s["a"], s["b"], self.dt, self.ds, s["pool"],
                      self.lens, self.idx, s["gk"], self.nacc, self.inp.scale, out=s["out"])

    def single_fused(self, s):
        """The single-pass fused call (segmented workloads: the form the workspace replaces)."""
        self.single_fused_fn(s["q"], s["k"], s["v"], s["a"], s["b"], self.dt, self.ds,
                             s["pool"], self.lens, self.idx, s["gk"], self.nacc, self.inp.scale,
                             out=s["out"])

    def step(self, i):
        self.fused(self.sets[i % self.R])

    def unfused_step(self, i):
        s = self.sets[i % self.R]
        self.gate(s)
        if self.inp.T != 1:
            self.transpose(s)
        self.decode(s)

    def free(self):
        self.sets = []
        self.ws = None
        self.fused_fn = self.decode_fn = None
        self.torch.cuda.synchronize()
        self.torch.cuda.empty_cache()


def warm_replays(torch, graph):
    # Untimed replays (the first also uploads the graph) until WARM_MS of work have run back
    # to back: the shader clock takes a few milliseconds of load to settle, and a replay
    # timed straight after capture runs up to 10% slow on the latency-bound multi-token
    # kernels.
    t0 = time.perf_counter()
    while True:
        graph.replay()
        torch.cuda.synchronize()
        if (time.perf_counter() - t0) * 1e3 >= WARM_MS:
            break


def capture(torch, stream, body, n):
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            for i in range(n):
                body(i)
    stream.wait_stream(cap)
    return graph


def graph_ms(torch, stream, body, n):
    """Wall time of n calls of body(i) captured in one graph, timed around one replay."""
    graph = capture(torch, stream, body, n)
    warm_replays(torch, graph)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    graph.replay()
    e1.record(stream)
    e1.synchronize()
    return e0.elapsed_time(e1)


def kernel_avg_us(torch, stream, fn, sets, n):
    """K back-to-back calls of one kernel, captured in a graph, timed with events on the
    launch stream around each of KERNEL_REPLAYS replays (no per-launch event overhead; this
    is the duration rocprofv3's kernel trace reports). Returns the median per-call time and
    every replay's."""
    g = capture(torch, stream, lambda i: fn(sets[i % len(sets)]), n)
    warm_replays(torch, g)
    per = []
    for _ in range(KERNEL_REPLAYS):
        a0 = torch.cuda.Event(enable_timing=True)
        a1 = torch.cuda.Event(enable_timing=True)
        a0.record(stream)
        g.replay()
        a1.record(stream)
        a1.synchronize()
        per.append(a0.elapsed_time(a1) * 1e3 / n)
    del g
    return float(sorted(per)[len(per) // 2]), per


def roofline(wl, us):
    gbs = wl.step_bytes / (us * 1e-6) / 1e9
    r = {"kernel": wl.fused_name, "bound": "hbm", "achieved": round(gbs, 2),
         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
         "traffic": measured_traffic(wl.wid, wl.batch), "bytes_per_launch": wl.step_bytes,
         "avg_launch_us": round(us, 3)}
    if wl.prefill:
        fl = (segmented_mfma_flops(wl.inp, wl.cus) if wl.ws_bytes
              else prefill_mfma_flops(wl.inp, wl.cus))
        tf = fl / (us * 1e-6) / 1e12
        r["mfma_executed"] = {"flops_per_launch": fl, "achieved_tflops": round(tf, 1),
                              "peak_tflops": MFMA_BF16_PEAK_TFLOPS,
                              "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                              "what": "bf16 matrix-core flops issued (split operands), not "
                                      "the method's algorithmic flops"}
    return r


def extra_entry(torch, stream, wl, n):
    """Fused-call duration and roofline of one more workload (kernel timing only)."""
    for i in range(3):
        wl.step(i)
    torch.cuda.synchronize()
    us, per = kernel_avg_us(torch, stream, wl.fused, wl.sets, n)
    inp = wl.inp
    r = roofline(wl, us)
    r["launch_us_replays"] = [round(x, 3) for x in per]
    if wl.ws_bytes:  # the segmented form: three launches per call; the single pass beside it
        r["launches_per_call"] = 3
        r["workspace_bytes"] = wl.ws_bytes
        sus, _ = kernel_avg_us(torch, stream, wl.single_fused, wl.sets, max(4, n // 4))
        r["single_pass_us"] = round(sus, 3)
    return {"workload": wl.name, "config": {"B": inp.B, "H_q": inp.Hq, "H_v": inp.Hv,
                                            "T": inp.T, "D_k": inp.Dk, "D_v": inp.Dv,
                                            "N_slots": inp.N_slots, "rotation_sets": wl.R,
                                            "calls_timed": n},
            "call_us": round(us, 3),
            "token_head_steps_per_s": round(wl.tok_heads / (us * 1e-6), 1),
            "roofline": r}


def snapshot_setup(torch, wl):
    """The rgdr_decode_snapshots call at workload `wl` (g and beta from the gate beforehand,
    as that entry takes them, and a snapshot buffer per buffer set) and its algorithmic
    bytes: the decode's plus D_k * D_v * 2 per written snapshot (every token t < L of every
    served entry and value head)."""
    import numpy as np
    inp = wl.inp
    B, Hv, T, Dk, Dv = inp.B, inp.Hv, inp.T, inp.Dk, inp.Dv
    for s in wl.sets:
        wl.gate(s)
        if T != 1:
            wl.transpose(s)
        s["snap"] = torch.empty((B, T, Hv, Dk, Dv), dtype=torch.bfloat16, device=s["q"].device)
    torch.cuda.synchronize()

    def call(s):
        g_ = s["g"].view(B, Hv, T) if T == 1 else s["gT"]
        be = s["beta"].view(B, Hv, T) if T == 1 else s["betaT"]
        wl.rg.rgdr_decode_snapshots(s["q"], s["k"], s["v"], be, s["pool"], wl.lens, wl.idx, g_,
                                    s["gk"], wl.nacc, inp.scale, out=s["out"],
                                    state_snapshots=s["snap"])

    lens = np.clip(inp.actual_seq_lengths, 0, T)
    valid = (inp.ssm_state_indices >= 0) & (inp.ssm_state_indices < inp.N_slots)
    return call, wl.dbytes + int(lens[valid].sum()) * Hv * Dk * Dv * 2


def snapshot_entry(torch, stream, wl, n):
    """Duration and roofline of rgdr_decode_snapshots at one workload: the decode step that
    also stores the state after every token (see snapshot_setup for its bytes)."""
    inp = wl.inp
    B, Hv, T, Dk, Dv = inp.B, inp.Hv, inp.T, inp.Dk, inp.Dv
    call, by = snapshot_setup(torch, wl)
    for s in wl.sets[:3]:
        call(s)
    torch.cuda.synchronize()
    us, per = kernel_avg_us(torch, stream, call, wl.sets, n)
    gbs = by / (us * 1e-6) / 1e9
    return {"workload": wl.name, "call": "rgdr_decode_snapshots (state after every token)",
            "config": {"B": B, "H_q": inp.Hq, "H_v": Hv, "T": T, "D_k": Dk, "D_v": Dv,
                       "N_slots": inp.N_slots, "rotation_sets": wl.R, "calls_timed": n},
            "call_us": round(us, 3),
            "roofline": {"kernel": "rgdr_decode_snapshots", "bound": "hbm",
                         "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic(wl.wid, "snapshots"),
                         "bytes_per_launch": by, "avg_launch_us": round(us, 3),
                         "launch_us_replays": [round(x, 3) for x in per]}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=2, choices=[0, 1, 2, 3, 4, 5, 6, 7])
    ap.add_argument("--rotate", type=int, default=0, help="buffer sets (0: auto, >= 1 GiB)")
    ap.add_argument("--batch", type=int, default=None,
                    help="replace the workload's batch size B (same recipe otherwise)")
    ap.add_argument("--extra", default="1,3,4,5,6,7",
                    help="other workloads whose fused-call duration the line also carries "
                         "(comma-separated ids; empty for none)")
    ap.add_argument("--snapshots", default="3",
                    help="workload at which the line also carries rgdr_decode_snapshots "
                         "(the state after every token); empty for none")
    ap.add_argument("--extra-steps", type=int, default=50,
                    help="calls per timed graph replay for the --extra workloads")
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

    import torch

    import gated_delta_rule_rgdr_amd as rg

    rg.library()  # fails loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wid = args.workload
    wl = Workload(wid, dev, args.rotate, args.steps, args.batch)
    inp = wl.inp
    B, Hq, Hv, T, Dk, Dv, N = inp.B, inp.Hq, inp.Hv, inp.T, inp.Dk, inp.Dv, inp.N_slots
    log(f"workload {wid}: {wl.name}; fused step bytes {wl.step_bytes}, unfused "
        f"{wl.decode_name} {wl.dbytes} + gate {wl.gbytes}; rotation sets {wl.R}")
    if T != 1:
        log("note: T > 1; the unfused chain transposes g/beta with torch between its kernels")

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
        wl.step(i)
    torch.cuda.synchronize()
    log(f"warmup: {args.warmup} eager steps done")
    if args.eager_only:
        for i in range(args.steps):
            wl.step(args.warmup + i)
            wl.unfused_step(args.warmup + i)
        torch.cuda.synchronize()
        log(f"eager pass: {args.steps} steps done")
        if args.snapshots.strip() == str(wid) and not wl.prefill:
            call, _ = snapshot_setup(torch, wl)
            for i in range(args.steps):
                call(wl.sets[i % len(wl.sets)])
            torch.cuda.synchronize()
            log(f"eager pass: {args.steps} rgdr_decode_snapshots calls done")
        if args.copy_calibration:
            copy_calibration()
        return

    K = args.steps
    total_ms = graph_ms(torch, stream, lambda i: wl.step(args.warmup + i), K)
    ms_per_step = total_ms / K
    log(f"timed: {K} steps in {total_ms:.3f} ms ({ms_per_step * 1e3:.2f} us/step)")
    for i in range(args.warmup):
        wl.unfused_step(i)
    unfused_ms = graph_ms(torch, stream, lambda i: wl.unfused_step(args.warmup + i), K) / K
    log(f"unfused chain (la_gate + {wl.decode_name}): {unfused_ms * 1e3:.2f} us/step")

    fused_us, fused_all = kernel_avg_us(torch, stream, wl.fused, wl.sets, K)
    dec_us, _ = kernel_avg_us(torch, stream, wl.decode, wl.sets, K)
    gate_us, _ = kernel_avg_us(torch, stream, wl.gate, wl.sets, K)
    log(f"fused kernel: {fused_us:.2f} us per call; unfused: {wl.decode_name} {dec_us:.2f} us, "
        f"gate {gate_us:.2f} us (medians of {KERNEL_REPLAYS} replays; fused replays: "
        + " ".join(f"{x:.2f}" for x in fused_all) + ")")

    # The box's practical streaming rate: a plain 256 MiB copy (read + write), graph-timed.
    csrc = torch.ones(64 << 20, dtype=torch.float32, device=dev)
    cdst = torch.empty_like(csrc)
    cg = capture(torch, stream, lambda i: torch.mul(csrc, 1.0, out=cdst), 20)
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

    value = wl.step_bytes / (ms_per_step * 1e-3) / 1e9
    steps_per_s = wl.tok_heads / (ms_per_step * 1e-3)
    roof = roofline(wl, fused_us)
    roof["launch_us_replays"] = [round(x, 3) for x in fused_all]
    wl.free()

    extras = {}
    for tok in [t for t in args.extra.split(",") if t.strip()]:
        ew = int(tok)
        if ew == wid or ew not in range(8):
            continue
        e = Workload(ew, dev, 0, args.extra_steps)
        extras[str(ew)] = extra_entry(torch, stream, e, args.extra_steps)
        log(f"workload {ew} ({e.name}): {e.fused_name} {extras[str(ew)]['call_us']:.2f} us "
            f"per call, {100 * extras[str(ew)]['roofline']['frac']:.1f}% of 8 TB/s")
        e.free()
        del e

    if args.snapshots.strip():
        sw = int(args.snapshots)
        e = Workload(sw, dev, 0, args.extra_steps)
        if not e.prefill:
            extras[f"{sw}_snapshots"] = snapshot_entry(torch, stream, e, args.extra_steps)
            log(f"workload {sw} with per-token states: rgdr_decode_snapshots "
                f"{extras[f'{sw}_snapshots']['call_us']:.2f} us per call, "
                f"{100 * extras[f'{sw}_snapshots']['roofline']['frac']:.1f}% of 8 TB/s")
        e.free()
        del e

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(inp, args.cpu_seconds)

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
        "config": {"workload": wl.name + " (gate + recurrence step)",
                   "step": f"{wl.fused_name} (gate fused into the kernel)",
                   "B": B, "H_q": Hq, "H_v": Hv, "T": T, "D_k": Dk, "D_v": Dv,
                   "N_slots": N, "rotation_sets": wl.R, "parallelism": "none (1 GPU)"},
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "token_head_steps_per_s": round(steps_per_s, 1),
        "step_bytes": wl.step_bytes,
        "bytes_per_state_element": round(wl.step_bytes / (wl.n_pairs * Dk * Dv), 4),
        "copy_reference": {"gbs": round(copy_gbs, 1), "us": round(copy_us, 2),
                           "what": "torch elementwise copy, 256 MiB read + 256 MiB write"},
        "roofline": roof,
        "unfused_ms_per_step": round(unfused_ms, 6),
        "unfused_kernels_avg_us": {"la_gate": round(gate_us, 3),
                                   wl.decode_name: round(dec_us, 3)},
        "workloads": extras,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
