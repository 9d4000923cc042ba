#!/usr/bin/env python3
"""Benchmark one MoE layer's expert path on one MI355X.

A step is one pass of the whole path over one batch: softmax top-k gate ->
dispatch permutation -> grouped SwiGLU FFN -> combine, plus the expert
statistics over the workload's layer stack.  Inputs are synthetic, already in
HBM when the timed region starts.  The default workload is the largest one
that fits one GPU: the GPT-OSS-120B-shaped mixed batch (64 decode tokens ahead
of a 4096-token prefill chunk, E=128, top-4, d=I=2880, bf16, 6.4 GB of expert
weights), whose FFN runs as one persistent launch with the decode tiles first.

Expert weights rotate over several copies (one per simulated layer) so that
each step streams its weights from HBM rather than from the 256 MB last-level
cache, as a model cycling through its layers would.

Prints ONE JSON line: MoE-layer tokens/s, the dominant kernel's roofline (the
grouped FFN: HBM-bound at decode sizes, MFMA-bound at prefill sizes), and the
CPU oracle timed on this host as a reported baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3        # MI355X fp32 vector
METRIC = "MoE-layer tokens/s; decode HBM GB/s and prefill MFMA util vs MI355X peak"
FFN_SOURCE = os.path.join(ROOT, "top_expert_routing_amd", "csrc", "ffn.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "ffn_traffic.json")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="gptoss_mixed")
    ap.add_argument("--weight-copies", type=int, default=0,
                    help="expert-weight copies to rotate over (0: enough to exceed 3 GiB)")
    ap.add_argument("--router", action="store_true",
                    help="put the router projection (x . W_r^T, seeded N(0, 0.02^2) weights) in front of the "
                         "gate; the gate then routes on its logits")
    ap.add_argument("--signature", action="store_true",
                    help="also time the signature recording at KV-block granularity (16-token blocks, every "
                         "layer of the statistics stack) and its device-to-host staging into pinned memory")
    ap.add_argument("--fp8-weights", action="store_true",
                    help="expert weights as E4M3 codes with per-row scales (moe_grouped_ffn_fp8w); the CPU "
                         "baseline leg is skipped in this mode")
    ap.add_argument("--unpacked-weights", action="store_true",
                    help="keep the [E+S][rows][K] weight layout (moe_grouped_ffn) on bf16 workloads; by "
                         "default their weights are pre-packed once before timing (pack_weights) and the FFN "
                         "runs moe_grouped_ffn_packed")
    ap.add_argument("--fused-combine", action="store_true",
                    help="run the FFN and the combine as one moe_grouped_ffn_combine call (the combine folded "
                         "into the down projection; bf16 decode-sized batches)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="rough CPU budget of the oracle leg")
    ap.add_argument("--json-out", default="", help="also append the JSON line to this file")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (scale for HBM byte counters) and exit")
    ap.add_argument("--eager", action="store_true",
                    help="time eager launches instead of replaying captured HIP graphs")
    ap.add_argument("--write-traffic", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="record the FFN's HBM traffic for --workload from rocprofv3 --pmc counter CSVs "
                         "(FETCH_SIZE and WRITE_SIZE runs of this bench and of --copy-calibration) into "
                         "profiles/ffn_traffic.json, then exit (no GPU needed)")
    return ap.parse_args()


def ffn_source_hash() -> str:
    with open(FFN_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_for(workload: str):
    """HBM bytes per FFN call from the committed rocprofv3 counter summary,
    each counter scaled by its copy-kernel factor; None if absent or stale."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("ffn_source_sha256_16") != ffn_source_hash():
        return None
    w = rec.get("workloads", {}).get(workload)
    if not w:
        return None
    return (w["fetch_kib_per_call"] * rec["fetch_scale"] + w["write_kib_per_call"] * rec["write_scale"]) * 1024.0


def _counter_per_dispatch(csv_path: str, counter: str, name_part: str):
    """Sum of `counter` over the dispatches whose kernel name contains
    name_part, and the number of those dispatches."""
    import csv
    per = {}
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter or name_part not in r["Kernel_Name"]:
                continue
            per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    return sum(per.values()), len(per)


def write_traffic(workload: str, fetch_csv: str, write_csv: str, copy_fetch_csv: str, copy_write_csv: str):
    """An FFN call is two dispatches: the gate/up and down launches, or the
    queue reset and the persistent queue launch.  The copy calibration runs
    three 1 GiB copies (each reads and writes 2**30 bytes)."""
    fk, fn = _counter_per_dispatch(fetch_csv, "FETCH_SIZE", "ffn_")
    wk, wn = _counter_per_dispatch(write_csv, "WRITE_SIZE", "ffn_")
    cf, cfn = _counter_per_dispatch(copy_fetch_csv, "FETCH_SIZE", "copyBuffer")
    cw, cwn = _counter_per_dispatch(copy_write_csv, "WRITE_SIZE", "copyBuffer")
    if not (fn and wn and cfn and cwn) or fn % 2 or wn % 2:
        raise SystemExit("unexpected dispatch counts in the counter CSVs")
    _, qf = _counter_per_dispatch(fetch_csv, "FETCH_SIZE", "ffn_queue_bf16")
    _, qw = _counter_per_dispatch(write_csv, "WRITE_SIZE", "ffn_queue_bf16")
    if (qf and 2 * qf != fn) or (qw and 2 * qw != wn):
        raise SystemExit("queue launches without their reset in the counter CSVs")
    copy_kib = 3 * 2**30 / 1024.0
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        rec = {}
    if rec.get("ffn_source_sha256_16") != ffn_source_hash():
        rec = {"workloads": {}}
    rec.update({
        "ffn_source_sha256_16": ffn_source_hash(),
        "fetch_scale": round(copy_kib / cf, 4),
        "write_scale": round(copy_kib / cw, 4),
        "note": "KiB per FFN call (two dispatches: both phase launches, or queue reset + queue launch) from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE; "
                "scales = bytes a 1 GiB copy moves / what the same counter reports for it",
    })
    rec.setdefault("workloads", {})[workload] = {
        "fetch_kib_per_call": round(fk / (fn / 2), 1),
        "write_kib_per_call": round(wk / (wn / 2), 1),
        "commands": [f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir> -o p -- python bench.py "
                     f"--workload {workload} --steps 4 --warmup 2 --no-cpu-baseline --eager",
                     "the same with --pmc WRITE_SIZE",
                     "rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) ... -- python bench.py --copy-calibration"],
    }
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec["workloads"][workload]))


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, budget_s: float, w_router=None):
    """Time the CPU oracle (as it stands) on a bounded sample of the workload
    (with `w_router`, the sample's logits come from the oracle's router), once
    with one BLAS thread and once with all of them."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle import moe_oracle as O

    def host(t):
        t = t.detach().contiguous().cpu()
        return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()

    s = wl.spec
    logits, x = host(wl.logits), host(wl.x)
    wg, wu, wd = host(wl.w_gate), host(wl.w_up), host(wl.w_down)
    # sample: the first n tokens (whole batch when it is small), whole layer path
    n = s.T if s.T <= 256 else 256
    toks = np.arange(n)
    wr = None if w_router is None else host(w_router)

    def timed(budget):
        t0 = time.perf_counter()
        done = passes = 0
        while True:
            lg = logits
            if wr is not None:
                lg = logits.copy()
                lg[:n] = O.router(x[:n], wr, s.dtype)
            O.moe_layer(lg, x, wg, wu, wd, s.k, s.dtype, n_shared=s.S, n_priority=s.n_priority, tokens=toks)
            ids, _ = O.gate(lg[:n], s.k)
            O.stats(ids[None], s.E, np.arange(n + 1, dtype=np.int32))
            done += n
            passes += 1
            el = time.perf_counter() - t0
            if el >= budget or passes >= 20 or el * (passes + 1) / passes > 2.5 * budget:
                return done / el, passes, el

    threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    with threadpool_limits(limits=1, user_api="blas"):
        v1, p1, e1 = timed(budget_s / 2)
    vn, pn, en = timed(budget_s / 2)
    return {"value": round(vn, 1), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {n} of {s.T} tokens, whole layer path (gate, permute, FFN on their rows, "
                      f"combine) plus their statistics{', router first' if wr is not None else ''}; "
                      f"{pn} pass(es) in {en:.1f} s with {threads} BLAS threads, {p1} in {e1:.1f} s with 1",
            "one_thread": {"value": round(v1, 1), "unit": "tokens/s", "cores": 1},
            "nproc": os.cpu_count(), "cpu_model": _cpu_model(),
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}


def decode_segment(layer, wl, s, dev, expert_bytes, packed):
    """One FFN call of the layer with the per-tile timeline: when the priority
    (decode) segment's last tile and the whole call's last tile ended, from the
    call's first tile start.  Against the time the decode segment's distinct
    experts' weights take to stream at the HBM peak."""
    import numpy as np
    import torch
    import top_expert_routing_amd as moe
    trace = torch.zeros((1 << 17, 4), dtype=torch.int64, device=dev)
    ffn = moe.grouped_ffn_packed if packed else moe.grouped_ffn
    ffn(wl.x, layer.perm["group_offsets"], s.E, s.S, layer.nseg, layer.w_gate, layer.w_up, layer.w_down,
        layer.h_sorted, layer.ffn_ws, x_rows=layer.perm["sorted_token"], trace=trace)
    torch.cuda.synchronize()
    tr = trace.cpu().numpy().view(np.uint64)
    rec = tr[tr[:, 1] != 0]
    if len(rec) == 0:
        return None
    prio = ((rec[:, 2] >> 1) & 1) == 1
    t0 = int(rec[:, 0].min())
    u_dec = int(np.unique(layer.topk_ids[: s.n_priority].cpu().numpy()).size)
    return {"completion_us": round((int(rec[prio, 1].max()) - t0) / 100.0, 1) if prio.any() else None,
            "ffn_us": round((int(rec[:, 1].max()) - t0) / 100.0, 1),
            "priority_tiles": int(prio.sum()), "tiles": int(len(rec)),
            "decode_union": u_dec,
            "hbm_bound_us": round(u_dec * expert_bytes / (PEAK_HBM_GBS * 1e3), 1),
            "clock": "s_memrealtime, 100 MHz; tile stamps of one traced call (a wait for each tile's stores "
                     "before its end stamp)"}


def signature_recording(s, stats_ids, req_offsets, stream, K, dev, logits_stack=None, block=16):
    """Per-KV-block expert counts over the statistics layer stack and their
    copy into pinned host memory, timed with HIP events on `stream` over K
    repetitions, two ways: recorded at the gate (moe_gate_record for each
    layer, against moe_gate alone) and by moe_stats with block offsets from
    the stacked ids; the staging is moe_stage_to_host.  The ELDR page
    ("Overhead" paragraph of its evidence section) times the same two steps on
    MI300X: 0.48 ms for the on-GPU scatter and 0.21 ms for the signature's D2H
    staging per request.  With `logits_stack` ([L][T][E]) it also times the
    continuous (softmax-probability) request signature over the same layers."""
    import torch
    import top_expert_routing_amd as moe
    offs = list(range(0, s.T, block)) + [s.T]
    boffs = torch.tensor(offs, dtype=torch.int32, device=dev)
    nb = len(offs) - 1
    L = stats_ids.shape[0]
    R = req_offsets.numel() - 1 if req_offsets is not None else nb
    out = {}
    ws = torch.empty(max(moe.stats_workspace_bytes(L, s.T, s.k, s.E, nb), 256), dtype=torch.uint8, device=dev)
    rec_g = torch.empty((nb, L, s.E), dtype=torch.int32, device=dev)
    ids = torch.empty((s.T, s.k), dtype=torch.int32, device=dev)
    wts = torch.empty((s.T, s.k), dtype=torch.float32, device=dev)

    def gates(record):
        for l in range(L):
            if record:
                moe.gate_record(logits_stack[l], s.k, block, l, rec_g, True, ids, wts)
            else:
                moe.gate(logits_stack[l], s.k, True, ids, wts)

    with torch.cuda.stream(stream):
        moe.stats(stats_ids, s.E, boffs, affinity=False, signature=False, out=out, workspace=ws)
        gates(True)
    host = torch.empty(out["req_counts"].shape, dtype=torch.int32, pin_memory=True)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(K)]
    with torch.cuda.stream(stream):
        for i in range(K):
            ev[i][0].record(stream)
            gates(False)
            ev[i][1].record(stream)
            gates(True)
            ev[i][2].record(stream)
            moe.stats(stats_ids, s.E, boffs, affinity=False, signature=False, out=out, workspace=ws)
            ev[i][3].record(stream)
            moe.stage_to_host(rec_g, host)
            ev[i][4].record(stream)
    torch.cuda.synchronize()
    ms = [sum(e[a].elapsed_time(e[a + 1]) for e in ev) / K * 1e3 for a in range(4)]
    gate_us, gate_rec_us, stats_us, d2h = ms
    if not torch.equal(host, out["req_counts"].cpu()) or not torch.equal(rec_g, out["req_counts"]):
        raise RuntimeError("block counts recorded at the gate, by moe_stats and on the host differ")
    # the continuous alternative the page compares against: per-request sums of
    # softmax probabilities from the recorded layers' logits
    prob = None
    if req_offsets is not None:
        psig = torch.empty((R, L, s.E), dtype=torch.float32, device=dev)
        pe = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
        with torch.cuda.stream(stream):
            moe.prob_signature(logits_stack, req_offsets, psig)
            for i in range(K):
                pe[i][0].record(stream)
                moe.prob_signature(logits_stack, req_offsets, psig)
                pe[i][1].record(stream)
        torch.cuda.synchronize()
        prob = round(sum(a.elapsed_time(b) for a, b in pe) / K * 1e3, 2)
    rec = gate_rec_us - gate_us
    return {"kv_block_tokens": block, "blocks": nb, "requests": R, "layers": L,
            "gate_us": round(gate_us, 2), "gate_record_us": round(gate_rec_us, 2),
            "record_at_gate_us": round(rec, 2), "record_by_stats_us": round(stats_us, 2),
            "d2h_us": round(d2h, 2), "d2h_bytes": host.numel() * 4,
            "per_request_us": round((max(rec, 0.0) + d2h) / max(R, 1), 3), "prob_signature_us": prob,
            "pages_mi300x_per_request_us": {"scatter": 480.0, "d2h_staging": 210.0}}


def main():
    args = parse()
    if args.write_traffic:
        write_traffic(args.workload, *args.write_traffic)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the expert path here has no multi-GPU mode "
              "(no collectives, no sharding); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import top_expert_routing_amd as moe
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        # known traffic: each copy reads 1 GiB and writes 1 GiB
        src = torch.empty(2**30, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": 2**30, "copies": 3}), flush=True)
        return
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    moe.load()

    wl = workloads.make(args.workload, dev)
    s = wl.spec
    esize = 4 if s.dtype == "f32" else 2
    fp8 = bool(args.fp8_weights)
    if fp8 and s.dtype != "bf16":
        print("--fp8-weights needs a bf16 workload", file=sys.stderr)
        sys.exit(2)
    # bf16 batches run on pre-packed weights unless asked otherwise
    packable = not fp8 and s.dtype == "bf16" and s.d % 32 == 0 and s.I % 32 == 0
    packed = packable and not args.unpacked_weights
    # FP8 codes are packed too when d and I are multiples of 64
    fp8_packed = fp8 and s.d % 64 == 0 and s.I % 64 == 0 and not args.unpacked_weights
    # expert weight bytes (fp8: codes plus one fp32 scale per weight row)
    expert_bytes = 3 * s.d * s.I + (2 * s.I + s.d) * 4 if fp8 else 3 * s.d * s.I * esize
    all_w = (s.E + s.S) * expert_bytes
    copies = args.weight_copies or max(1, int(np.ceil(3 * 2**30 / all_w)))
    if fp8:
        q = [moe.quantize_fp8_rows(w) for w in (wl.w_gate, wl.w_up, wl.w_down)]
        if fp8_packed:
            q = [(moe.pack_fp8_codes(c), sc) for c, sc in q]
        base = (q[0][0], q[0][1], q[1][0], q[1][1], q[2][0], q[2][1])
        wsets = [base] + [tuple(t.clone() for t in base) for _ in range(copies - 1)]
    else:
        base = (wl.w_gate, wl.w_up, wl.w_down)
        if packed:
            base = tuple(moe.pack_weights(w) for w in base)
        wsets = [base]
        for _ in range(copies - 1):
            wsets.append(tuple(w.clone() for w in base))

    # the gate writes the routing layer's ids straight into layer 0 of the
    # statistics stack
    stats_ids = torch.empty((s.stats_layers, s.T, s.k), dtype=torch.int32, device=dev)
    w_router = None
    if args.router:
        g = torch.Generator().manual_seed(1234)
        w_router = (torch.randn((s.E, s.d), generator=g) * 0.02).to(wl.torch_dtype).to(dev)
    w16 = (wl.w_gate, wl.w_up, wl.w_down) if fp8 else wsets[0]     # the layer's bf16 / fp32 weights
    layer = moe.MoeLayer(s.E, s.k, s.d, s.I, s.T, wl.torch_dtype, *w16, packed_weights=packed or fp8_packed,
                         n_shared=s.S, n_priority=s.n_priority, renormalize=bool(s.renormalize),
                         stats_layers=s.stats_layers, req_offsets=wl.req_offsets, device=dev,
                         topk_ids=stats_ids[0], w_router=w_router, fp8_weights=wsets[0] if fp8 else None,
                         fused_combine=args.fused_combine)
    for l in range(1, s.stats_layers):      # the other layers' ids, produced before timing
        moe.gate(wl.stats_logits[l].contiguous(), s.k, True, stats_ids[l],
                 torch.empty((s.T, s.k), device=dev))
    # One stream, in path order: (router,) gate, statistics (they need only the gate's
    # ids), permute, FFN, combine.  (A second stream for the statistics costs
    # two cross-queue waits per step, more than the statistics themselves.)
    stream = torch.cuda.Stream(dev)
    call_sets = []
    for ws in wsets:
        if fp8:
            layer.fp8_weights = ws
        else:
            layer.w_gate, layer.w_up, layer.w_down = ws
        call_sets.append(layer.bound_calls(wl.logits, wl.x, stats_ids, stream.cuda_stream))
    names = [c[0] for c in call_sets[0]]
    first = [names.index(n) for n in ("moe_router", "moe_gate", "moe_stats") if n in names]
    order = first + [j for j in range(len(names)) if j not in first]

    def step(i, ev=None):
        """One layer step on `stream`."""
        calls = call_sets[i % copies]
        for j in order:
            name, fn, a = calls[j]
            if ev is not None:
                ev[j][0].record(stream)
            st = fn(*a)
            if st != 0:
                raise moe.MoeError(name, st)
            if ev is not None:
                ev[j][1].record(stream)

    # Everything above ran on the default stream and returned before the GPU
    # finished: the weight preparation frees large temporaries whose kernels are
    # still queued, and the layer's buffers may reuse that memory.  The steps run
    # on `stream`, which is not ordered after those kernels, so wait for them
    # here (otherwise a late write of a freed temporary can land in the layer's
    # index buffers while the steps use them).
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            step(i)
    torch.cuda.synchronize()

    # headline: K steps replayed from captured HIP graphs, or eager launches
    # with --eager.  One graph holds `copies` consecutive steps (one per weight
    # copy, like the consecutive layers of a captured forward pass);
    # single-step graphs cover a remainder, so exactly K steps run.
    K = args.steps
    multi, singles = None, []
    if not args.eager:
        multi = torch.cuda.CUDAGraph()
        with torch.cuda.graph(multi, stream=stream):
            for c in range(copies):
                step(c)
        for c in range(copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                step(c)
            singles.append(g)
        for i in range(max(1, args.warmup // copies)):
            multi.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        if multi is not None:
            reps, rem = divmod(K, copies)
            for _ in range(reps):
                multi.replay()
            for c in range(rem):
                singles[c].replay()
        else:
            for i in range(K):
                step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    # per-call durations: K eager steps with HIP events around every call, on
    # the stream each call runs on
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in names]
           for _ in range(K)]
    with torch.cuda.stream(stream):
        for i in range(K):
            step(i, evs[i])
    torch.cuda.synchronize()
    diag = int(layer.ffn_ws[-4:].view(torch.int32).item())
    if diag != 0:
        raise RuntimeError("the FFN's diagnostic word is set: a wait of the persistent tile queue gave up")
    per_call = {n: 0.0 for n in names}
    for e in evs:
        for j, n in enumerate(names):
            per_call[n] += e[j][0].elapsed_time(e[j][1]) / K     # ms

    # algorithmic work of the FFN call
    union = int(layer.stats_out["union_size"][0].item()) if layer.stats_out else s.E
    used_experts = union + s.S
    N = s.N
    ffn_bytes = used_experts * expert_bytes + 2 * N * s.d * esize
    ffn_flops = 2.0 * N * 3 * s.d * s.I
    ffn_name = ("moe_grouped_ffn_fp8w_packed" if fp8_packed else "moe_grouped_ffn_fp8w") if fp8 else \
        "moe_grouped_ffn_combine" if args.fused_combine else \
        "moe_grouped_ffn_packed" if packed else "moe_grouped_ffn"
    ffn_s = per_call[ffn_name] * 1e-3
    peak_flops = PEAK_F32_TFLOPS if s.dtype == "f32" else PEAK_BF16_TFLOPS
    intensity = ffn_flops / ffn_bytes
    ridge = peak_flops * 1e12 / (PEAK_HBM_GBS * 1e9)
    if intensity < ridge:
        achieved = ffn_bytes / ffn_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4)}
    else:
        achieved = ffn_flops / ffn_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak_flops, "unit": "TFLOP/s",
                "frac": round(achieved / peak_flops, 4)}
    # the committed counters are for the default mode of each workload
    traffic = None if fp8 or args.unpacked_weights or args.fused_combine else traffic_for(args.workload)
    roof["traffic"] = None if traffic is None else round(traffic)
    # the library's path choice for batches with a priority segment: bf16
    # prefill-sized groups, or packed FP8 codes on 128-row GEMM tiles
    avg = s.N // s.G
    queue = (s.n_priority > 0 and os.environ.get("LIBMOE_FFN_QUEUE", "1") != "0" and
             ((not fp8 and s.dtype == "bf16" and s.d % 32 == 0 and s.I % 32 == 0 and avg > 48) or
              (fp8_packed and s.d >= 128 and s.I >= 128 and 48 < avg < 256)))
    roof["kernel"] = (f"{ffn_name} (" + ("one persistent launch: decode-priority tile queues" if queue else
                                         "gate/up launch + down launch with the combine in its epilogue + "
                                         "conversion launch" if args.fused_combine else
                                         "gate/up launch + down launch") + "), HIP events over K eager steps")
    roof["algorithmic_bytes"] = int(ffn_bytes)
    roof["algorithmic_flops"] = int(ffn_flops)
    roof["avg_call_us"] = round(ffn_s * 1e6, 2)

    # the FFN against the other roof as well (MFMA for decode-bound batches,
    # HBM for compute-bound ones)
    roof["hbm_frac"] = round(ffn_bytes / ffn_s / 1e9 / PEAK_HBM_GBS, 4)
    roof["mfma_frac"] = round(ffn_flops / ffn_s / 1e12 / peak_flops, 4)

    signature = None
    if args.signature:
        # the recorded layers' logits; layer 0 is the routing layer, whose gate
        # read the router's logits when the router runs in front
        rec_logits = wl.stats_logits.contiguous()
        if layer.logits is not None:
            rec_logits = rec_logits.clone()
            rec_logits[0].copy_(layer.logits)
        signature = signature_recording(s, stats_ids, wl.req_offsets, stream, K, dev, rec_logits)
    dseg = decode_segment(layer, wl, s, dev, expert_bytes, packed) if queue else None

    tokens_per_s = s.T * K / elapsed
    out = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(elapsed / K * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": s.dtype, "data": "synthetic",
        "config": {"workload": args.workload, "T": s.T, "E": s.E, "k": s.k, "n_shared": s.S, "d": s.d,
                   "I": s.I, "n_priority": s.n_priority, "stats_layers": s.stats_layers,
                   "weight_copies": copies, "union": union, "router": bool(args.router),
                   "expert_weights": ("fp8_e4m3 + fp32 row scales" + (", packed 16x64 blocks" if fp8_packed else ""))
                   if fp8 else
                   f"{s.dtype}, packed 16x32 blocks" if packed else s.dtype},
        "roofline": roof,
        "per_call_us": {n: round(v * 1e3, 2) for n, v in per_call.items()},
        "timing": "eager launches" if args.eager else
                  f"captured HIP graphs of {copies} consecutive steps (one per weight copy) replayed",
    }
    if signature is not None:
        out["signature_recording"] = signature
    if dseg is not None:
        out["decode_segment"] = dseg
    if not args.no_cpu_baseline and not fp8:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds, w_router)
    line = json.dumps(out)
    print(line, flush=True)
    if args.json_out:
        with open(args.json_out, "a") as f:
            f.write(line + "\n")


if __name__ == "__main__":
    main()
