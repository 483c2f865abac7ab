#!/usr/bin/env python3
"""Benchmark of the gated delta rule hot path on one MI355X.

One step is one pass of the whole path over one batch: a mixed step whose front is
the standard decode batch (64 cached rows, 16 key / 32 value heads, d_k = d_v = 128,
bf16 q/k/v, fp32 states in a 256-slot cache) and whose prefill part is the long
prefill (16 sequences x 8192 tokens, same heads, zero initial states, states exported
on the 1088-token prefix-cache grid).  The step is issued as its two launches --
gdn_recurrent_decode (one kernel) then gdn_chunk_prefill (one kernel) -- which is
exactly what gdn_mixed_step enqueues (checked bitwise before timing), so that HIP
events on the launch stream time each kernel.  Inputs are resident in HBM before the
timed region starts.

Timing: the prefill alone and the decode alone (over disjoint slot sets of the
cache) are timed back to back first, which also brings the GPU to its steady state;
then W warm-up steps, then exactly K steps between one pair of HIP events
(ms_per_step, value).  Per-kernel medians with 10th/90th percentiles come from a
second pass of K steps with an event between the two launches.

Prints one JSON line: value = prefill tokens per second of the whole step; the
decode part's state bandwidth and its fraction of the 8 TB/s HBM peak; the dominant
kernel's roofline; the other standard workloads (the single fp32 sequence, the
varlen prefill exporting every 64 tokens, the mixed step of 32 cached rows and four
fresh prefills), each timed call by call with the caches flushed in between; and
the fp64 CPU oracle timed on bounded samples of the same workload, on every host
core and on one.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GDN prefill tokens/s + decode state GB/s (frac of HBM peak) on 1 MI355X"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3        # MI355X fp32 (matrix and vector)
CHUNK = 64
KERNEL_SOURCES = {"decode_kernel": "gdn_decode.hip", "chunk_kernel": "gdn_prefill_bf16.hip",
                  "stream_copy_kernel": "gdn_probe.hip", "state_rmw_kernel": "gdn_probe.hip"}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the single-sequence, varlen and mixed-step workloads")
    ap.add_argument("--secondary-calls", type=int, default=50,
                    help="timed calls of each secondary workload")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="first run one plain device-to-device copy of this many MiB, a reference "
                         "dispatch of known traffic for hardware byte counters")
    ap.add_argument("--ingest-sq-counters", metavar="SQ_CSV",
                    help="no GPU work: turn the counter_collection.csv of a rocprofv3 --pmc run with "
                         "SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE, SQ_INSTS_* (the bf16 and, if taken, the fp16 "
                         "MFMA op counts) and SQ_WAVES into profiles/mfma_counters.json")
    ap.add_argument("--ingest-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU work: turn the counter_collection.csv files of a rocprofv3 --pmc FETCH_SIZE "
                         "run and a --pmc WRITE_SIZE run of this bench into profiles/hbm_traffic.json")
    return ap.parse_args()


def source_digest(kernel):
    """sha256 of the HIP source a kernel is built from; hardware byte counters taken
    on another version of the source no longer describe the kernel."""
    path = os.path.join(ROOT, "gated_deltanet_rule_amd", "csrc", KERNEL_SOURCES[kernel])
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic(kernel):
    """HBM bytes per launch from the committed counter profile (FETCH_SIZE and
    WRITE_SIZE, each scaled by what the counter reads for a copy of known size), or
    None when there is none for the current source of the kernel."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(kernel)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256") != source_digest(kernel):
        return None
    return rec.get("bytes_per_launch")


def ingest_counters(fetch_csv, write_csv, copy_mib=1024):
    """HBM bytes per launch of each library kernel from two rocprofv3 counter runs.
    Each counter (KiB per dispatch) is scaled by what it reads for the plain copies of
    copy_mib MiB that the bench dispatches (a copy reads and writes copy_mib MiB), so the
    figures are in bytes whatever unit or sampling the counter uses on this chip."""
    import csv
    out = {}
    per = {}
    for tag, path in (("fetch", fetch_csv), ("write", write_csv)):
        rows = list(csv.DictReader(open(path)))
        copies = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]]
        big = [c for c in copies if c > 0.5 * max(copies)]
        factor = (copy_mib * 1024.0) / float(np.median(big))
        for kernel in KERNEL_SOURCES:
            vals = [float(r["Counter_Value"]) for r in rows if kernel in r["Kernel_Name"]]
            if vals:
                per.setdefault(kernel, {})[tag] = (len(vals), float(np.mean(vals)), factor)
    for kernel, d in per.items():
        if "fetch" not in d or "write" not in d:
            continue
        nf, fk, ff = d["fetch"]
        nw, wk, wf = d["write"]
        out[kernel] = {"source": "gated_deltanet_rule_amd/csrc/" + KERNEL_SOURCES[kernel],
                       "source_sha256": source_digest(kernel), "dispatches": [nf, nw],
                       "fetch_kib": round(fk, 1), "write_kib": round(wk, 1),
                       "fetch_factor": round(ff, 4), "write_factor": round(wf, 4),
                       "bytes_per_launch": int(round((fk * ff + wk * wf) * 1024))}
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))


SIMDS = 1024          # 256 compute units x 4 SIMDs
XCDS = 8


def ingest_sq_counters(sq_csv, chunks_per_wave=128):
    """MFMA utilisation of each library kernel from one rocprofv3 counter run: busy
    cycles of the matrix cores summed over all SIMDs, over the GPU-active cycles (the
    GRBM counter summed over the XCDs, divided by their number) times the SIMD count;
    the instruction counts per wave (and per chunk for the prefill kernel, whose
    waves each walk chunks_per_wave chunks at the bench's shape)."""
    import csv
    per = {}
    for r in csv.DictReader(open(sq_csv)):
        kernel = next((k for k in KERNEL_SOURCES if k in r["Kernel_Name"]), None)
        if kernel:
            d = per.setdefault(kernel, {}).setdefault(int(r["Dispatch_Id"]), {})
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    out = {}
    for kernel, disp in per.items():
        mean = lambda c: float(np.mean([d[c] for d in disp.values()]))
        active = mean("GRBM_GUI_ACTIVE") / XCDS
        waves = mean("SQ_WAVES")
        units = waves * (chunks_per_wave if kernel == "chunk_kernel" else 1)
        rec = {"source": "gated_deltanet_rule_amd/csrc/" + KERNEL_SOURCES[kernel],
               "source_sha256": source_digest(kernel), "dispatches": len(disp),
               "mfma_busy_frac": round(mean("SQ_VALU_MFMA_BUSY_CYCLES") / (active * SIMDS), 4),
               "gpu_active_cycles_per_xcd": round(active),
               "mfma_insts_per_unit": round(mean("SQ_INSTS_MFMA") / units, 1),
               "valu_insts_per_unit": round((mean("SQ_INSTS_VALU") - mean("SQ_INSTS_MFMA")) / units, 1),
               "lds_insts_per_unit": round(mean("SQ_INSTS_LDS") / units, 1),
               "unit": "wave and chunk" if kernel == "chunk_kernel" else "wave",
               "executed_bf16_mfma_flop": mean("SQ_INSTS_VALU_MFMA_MOPS_BF16") * 512}
        if "SQ_INSTS_VALU_MFMA_MOPS_F16" in next(iter(disp.values())):
            rec["executed_f16_mfma_flop"] = mean("SQ_INSTS_VALU_MFMA_MOPS_F16") * 512
        if "SQ_VALU_MFMA_COEXEC_CYCLES" in next(iter(disp.values())):
            busy = mean("SQ_VALU_MFMA_BUSY_CYCLES")
            rec["valu_coexec_frac_of_mfma_busy"] = round(mean("SQ_VALU_MFMA_COEXEC_CYCLES") / busy, 4) if busy else None
        out[kernel] = rec
    path = os.path.join(ROOT, "profiles", "mfma_counters.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))


def measured_mfma_util(kernel):
    """MFMA busy fraction from the committed counter profile, or None when there is
    none for the current source of the kernel."""
    try:
        with open(os.path.join(ROOT, "profiles", "mfma_counters.json")) as f:
            rec = json.load(f).get(kernel)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256") != source_digest(kernel):
        return None
    return rec.get("mfma_busy_frac")


def algorithmic_flops_per_token(H_k, H_v, d_k, d_v, C=CHUNK):
    """Flops per prefill token of the chunked form, triangles counted once, K K^T and
    Q K^T once per key head: H_k 2 C d_k + H_v (C (d_k + d_v) + C d_v + 6 d_k d_v)."""
    return H_k * 2 * C * d_k + H_v * (C * (d_k + d_v) + C * d_v + 6 * d_k * d_v)


def algorithmic_bytes_per_token(H_k, H_v, d_k, d_v, elem):
    """HBM bytes every prefill token must move: q and k (H_k d_k each), v and o (H_v
    d_v each) at elem bytes per element, and the fp32 g and beta of every value head."""
    return 2 * H_k * d_k * elem + 2 * H_v * d_v * elem + 8 * H_v


def stats(ts):
    """Median, 10th and 90th percentile of a list of durations (ms)."""
    a = np.sort(np.asarray(ts, dtype=np.float64))
    return {"median": round(float(np.median(a)), 5), "p10": round(float(np.percentile(a, 10)), 5),
            "p90": round(float(np.percentile(a, 90)), 5), "n": int(a.size)}


def time_calls(torch, fn, n, warmup, flush=None):
    """Durations (ms) of n calls of fn, each between a pair of HIP events recorded on
    the stream the library launches on (torch's current stream); flush() runs before
    every call, outside the events."""
    for _ in range(warmup):
        if flush:
            flush()
        fn()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    torch.cuda.synchronize()
    for e0, e1 in ev:
        if flush:
            flush()
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    return [e0.elapsed_time(e1) for e0, e1 in ev]


def time_loop(torch, fn, n):
    """Average duration (ms) of n calls of fn issued back to back between one pair of events."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(n):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def prefill_inputs(torch, binding, w, dev, B=0):
    """A workload's tensors on the device, with an export buffer for its grid."""
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    t = {x: torch.from_numpy(getattr(w, x)).to(dev, dt) for x in ("q", "k", "v")}
    t.update({x: torch.from_numpy(getattr(w, x)).to(dev) for x in ("g", "beta", "pool")})
    i32 = lambda a: torch.as_tensor(np.asarray(a, dtype=np.int32), device=dev)
    t["o"] = torch.empty_like(t["v"])
    t["cu"] = i32(w.cu_seqlens())
    t["init_slot"], t["final_slot"] = i32(w.init_slot), i32(w.final_slot)
    t["slot_in"], t["slot_out"] = i32(w.slot_in), i32(w.slot_out)
    kw = dict(scale=w.scale, workspace=binding.alloc_workspace(w.H_v, dt, w.num_seqs, w.prefill_tokens, dev))
    if w.export_grid:
        offs = binding.export_offsets(w.lengths, None, w.export_grid)
        kw.update(export_grid=w.export_grid, export_offsets=i32(offs),
                  export_states=torch.empty((max(offs[-1], 1), w.H_v, w.d_k, w.d_v), dtype=torch.float32,
                                            device=dev))
    n_states = (kw["export_states"].shape[0] if w.export_grid else 0) + w.num_seqs
    return t, kw, n_states


def prefill_figures(ms, w, n_states, elem):
    """Throughput and roofline fractions of one prefill launch of ms milliseconds."""
    T = w.prefill_tokens
    bytes_ = algorithmic_bytes_per_token(w.H_k, w.H_v, w.d_k, w.d_v, elem) * T + 4 * w.H_v * w.d_k * w.d_v * n_states
    flops = algorithmic_flops_per_token(w.H_k, w.H_v, w.d_k, w.d_v) * T
    gbps = bytes_ / (ms * 1e-3) / 1e9
    tflops = flops / (ms * 1e-3) / 1e12
    peak_t = BF16_PEAK_TFLOPS if elem == 2 else FP32_PEAK_TFLOPS
    return {"tokens_per_s": round(T / (ms * 1e-3), 1), "bytes_per_launch": int(bytes_),
            "flops_per_launch": int(flops), "achieved_GB_per_s": round(gbps, 1),
            "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4), "mfma_tflops": round(tflops, 3),
            "mfma_frac": round(tflops / peak_t, 4),
            # time a launch could take at best: its bytes at the HBM peak or its flops at
            # the matrix peak, whichever is longer
            "floor_ms": round(max(bytes_ / (HBM_PEAK_GBPS * 1e9), flops / (peak_t * 1e12)) * 1e3, 5)}


def secondary_configs(torch, binding, W, dev, n, warmup):
    """The other standard workloads, each timed call by call with the caches flushed
    (a 1 GiB fill) before every call: the single fp32 sequence, the varlen prefill
    with exports every 64 tokens, and the mixed step."""
    scratch = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    flush = lambda: scratch.fill_(1.0)
    out = {}

    w0 = W.config(0)
    t, kw, ns = prefill_inputs(torch, binding, w0, dev)
    run0 = lambda: binding.gdn_chunk_prefill(t["q"], t["k"], t["v"], t["g"], t["beta"], t["o"], t["cu"], t["pool"],
                                             t["init_slot"], t["final_slot"], **kw)
    st = stats(time_calls(torch, run0, n, warmup, flush))
    out["single_sequence_fp32"] = dict(
        {"workload": W.CONFIG_DESCRIPTIONS[0], "bound": "latency", "kernel": "scan_kernel", "ms": st},
        **{k: v for k, v in prefill_figures(st["median"], w0, ns, 4).items()
           if k in ("tokens_per_s", "flops_per_launch", "floor_ms")})
    del t, kw

    w2 = W.config(2, fill_pool=False)
    t, kw, ns = prefill_inputs(torch, binding, w2, dev)
    run2 = lambda: binding.gdn_chunk_prefill(t["q"], t["k"], t["v"], t["g"], t["beta"], t["o"], t["cu"], t["pool"],
                                             t["init_slot"], t["final_slot"], **kw)
    st = stats(time_calls(torch, run2, n, warmup, flush))
    fig = prefill_figures(st["median"], w2, ns, 2)
    out["varlen_prefill_export64"] = dict(
        {"workload": W.CONFIG_DESCRIPTIONS[2], "lengths": w2.lengths, "prefill_tokens": w2.prefill_tokens,
         "exported_states": ns - w2.num_seqs, "bound": "hbm", "kernel": "chunk_kernel", "ms": st}, **fig)
    del t, kw

    w3 = W.config(3)
    t, kw, ns = prefill_inputs(torch, binding, w3, dev)
    B = w3.num_decode_rows
    run3 = lambda: binding.gdn_mixed_step(t["q"], t["k"], t["v"], t["g"], t["beta"], t["o"], t["pool"], t["slot_in"],
                                          t["slot_out"], t["cu"], t["init_slot"], t["final_slot"], **kw)
    st = stats(time_calls(torch, run3, n, warmup, flush))
    dec_bytes = 2 * 4 * w3.d_k * w3.d_v * B * w3.H_v
    pre = prefill_figures(st["median"], w3, ns, 2)
    step_bytes = dec_bytes + pre["bytes_per_launch"]
    out["mixed_step"] = {
        "workload": W.CONFIG_DESCRIPTIONS[3], "bound": "latency", "kernels": ["decode_kernel", "chunk_kernel"],
        "step_ms": st, "decode_rows": B, "prefill_tokens": w3.prefill_tokens,
        "tokens_per_s": round((B + w3.prefill_tokens) / (st["median"] * 1e-3), 1),
        "bytes_per_step": int(step_bytes),
        "hbm_floor_ms": round(step_bytes / (HBM_PEAK_GBPS * 1e9) * 1e3, 5)}
    del t, kw, scratch
    torch.cuda.synchronize()
    return out


def main():
    args = parse()
    if args.ingest_counters:
        ingest_counters(*args.ingest_counters)
        return
    if args.ingest_sq_counters:
        ingest_sq_counters(args.ingest_sq_counters)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(requested --gpus %d, WORLD_SIZE %d)" % (args.gpus, world), file=sys.stderr)
        sys.exit(2)

    import torch
    from gated_deltanet_rule_amd import binding
    from gated_deltanet_rule_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 18                # float32 elements
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    copy_gbps = copy_bandwidth(torch, dev)
    t_gen = time.time()
    wd = W.config(1)                                           # decode batch
    wp = W.config(4, fill_pool=False)                          # long prefill
    H_k, H_v, d_k, d_v = wd.H_k, wd.H_v, wd.d_k, wd.d_v
    B, N = wd.num_decode_rows, wp.num_seqs
    Tp = wp.prefill_tokens
    bf = torch.bfloat16

    def cat(name, dtype):
        a = torch.from_numpy(getattr(wd, name)).to(dev, dtype)
        b = torch.from_numpy(getattr(wp, name)).to(dev, dtype)
        return torch.cat([a, b]).contiguous()

    q, k, v = cat("q", bf), cat("k", bf), cat("v", bf)
    g, beta = cat("g", torch.float32), cat("beta", torch.float32)
    num_slots = wd.pool.shape[0] + N
    pool = torch.empty((num_slots, H_v, d_k, d_v), dtype=torch.float32, device=dev)
    pool[:wd.pool.shape[0]] = torch.from_numpy(wd.pool).to(dev)
    pool[wd.pool.shape[0]:] = 0
    o = torch.empty_like(v)
    i32 = lambda a: torch.as_tensor(np.asarray(a, dtype=np.int32), device=dev)
    slot_in, slot_out = i32(wd.slot_in), i32(wd.slot_out)
    cu = i32(wp.cu_seqlens())
    init_slot = i32(np.full(N, -1))
    final_slot = i32(np.arange(wd.pool.shape[0], num_slots))
    grid = wp.export_grid
    offs = binding.export_offsets(wp.lengths, None, grid)
    exp_offs = i32(offs)
    exports = torch.empty((offs[-1], H_v, d_k, d_v), dtype=torch.float32, device=dev)
    ws = binding.alloc_workspace(H_v, bf, N, Tp, dev)
    torch.cuda.synchronize()
    gen_s = time.time() - t_gen

    dq, dk_, dv_, dg, db, do = q[:B], k[:B], v[:B], g[:B], beta[:B], o[:B]
    pq, pk, pv, pg, pb, po = q[B:], k[B:], v[B:], g[B:], beta[B:], o[B:]
    pre = dict(scale=wp.scale, workspace=ws, export_grid=grid, export_states=exports, export_offsets=exp_offs)

    def stage_decode():
        binding.gdn_recurrent_decode(dq, dk_, dv_, dg, db, do, pool, slot_in, slot_out, scale=wd.scale)

    def stage_prefill():
        binding.gdn_chunk_prefill(pq, pk, pv, pg, pb, po, cu, pool, init_slot, final_slot, **pre)

    def step():
        stage_decode()
        stage_prefill()

    # the staged step is the mixed step: check bitwise once, from the same pool
    pool0 = pool.clone()
    binding.gdn_mixed_step(q, k, v, g, beta, o, pool, slot_in, slot_out, cu, init_slot, final_slot, **pre)
    torch.cuda.synchronize()
    ref = (o.clone(), pool.clone(), exports.clone())
    pool.copy_(pool0)
    step()
    torch.cuda.synchronize()
    same = torch.equal(o, ref[0]) and torch.equal(pool, ref[1]) and torch.equal(exports, ref[2])
    if not same:
        print("staged step differs from gdn_mixed_step", file=sys.stderr)
        sys.exit(1)
    del pool0, ref

    # The prefill alone and the decode alone, back to back, before the step's warm-up: a
    # GPU fresh from the input generation needs some 30 steps of this workload to settle
    # (four consecutive 20-step loops measured 1.26, 1.06, 1.04 and 1.03 ms per step), and
    # these two passes bring it there; their own figures are taken while it settles.
    K = args.steps
    t_pre_b2b = time_loop(torch, stage_prefill, K)
    t_dec_b2b = decode_back_to_back(torch, binding, wd, dq, dk_, dv_, dg, db, do, pool, dev)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # The timed region: exactly K steps between one pair of events, nothing else in it.
    ms_step = time_loop(torch, step, K)

    # Per-kernel figures: K steps with an event between the two launches (median and
    # spread per kernel); the back-to-back passes ran before the warm-up.
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    for e in ev:
        e[0].record()
        stage_decode()
        e[1].record()
        stage_prefill()
        e[2].record()
    torch.cuda.synchronize()
    st_dec = stats([e[0].elapsed_time(e[1]) for e in ev])
    st_pre = stats([e[1].elapsed_time(e[2]) for e in ev])
    t_copy_ref, t_rmw_ref = decode_floors(torch, wd, pool, dev)
    t_dec, t_pre = st_dec["median"], st_pre["median"]

    # ---- figures
    value = Tp / (ms_step * 1e-3)
    dec_bytes = 2 * 4 * d_k * d_v * B * H_v                # fp32 state read + write per (row, head)
    dec_gbps = dec_bytes / (t_dec * 1e-3) / 1e9
    f_tok = algorithmic_flops_per_token(H_k, H_v, d_k, d_v)
    pre_flops = f_tok * Tp
    pre_tflops = pre_flops / (t_pre * 1e-3) / 1e12
    state_bytes = 4 * H_v * d_k * d_v
    b_tok = algorithmic_bytes_per_token(H_k, H_v, d_k, d_v, 2)
    pre_bytes = b_tok * Tp + state_bytes * (offs[-1] + N)  # activations + exports + final states
    pre_gbps = pre_bytes / (t_pre * 1e-3) / 1e9
    kernels = {
        "decode_kernel": {"ms": st_dec, "bound": "hbm", "achieved": round(dec_gbps, 1),
                          "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(dec_gbps / HBM_PEAK_GBPS, 4),
                          "bytes_per_launch": dec_bytes, "traffic": measured_traffic("decode_kernel")},
        # arithmetic intensity pre_flops / pre_bytes (about 156 flop/B) is below the bf16
        # ridge (2500 / 8 = 312 flop/B): HBM binds, MFMA use is reported beside it
        "chunk_kernel": {"ms": st_pre, "bound": "hbm", "achieved": round(pre_gbps, 1),
                        "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(pre_gbps / HBM_PEAK_GBPS, 4),
                        "bytes_per_launch": pre_bytes, "traffic": measured_traffic("chunk_kernel"),
                        "mfma_tflops": round(pre_tflops, 2), "mfma_frac": round(pre_tflops / BF16_PEAK_TFLOPS, 4),
                        "mfma_busy_frac_counters": measured_mfma_util("chunk_kernel"),
                        "flops_per_launch": pre_flops, "back_to_back_ms": round(t_pre_b2b, 5)},
    }
    dominant = "chunk_kernel" if t_pre >= t_dec else "decode_kernel"
    roof = kernels[dominant]
    roofline = {"kernel": dominant, "bound": roof["bound"], "achieved": roof["achieved"], "peak": roof["peak"],
                "unit": roof["unit"], "frac": roof["frac"], "traffic": roof["traffic"]}

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "mixed step: 64 cached decode rows (256-slot fp32 state cache) ahead of 16 x 8192-token "
                               "prefills exporting states every 1088 tokens; 16 key / 32 value heads, d_k = d_v = 128, "
                               "bf16 q/k/v, fp32 gates and states",
                   "global_batch": B + N, "seq_len": 8192, "prefill_tokens": Tp, "decode_rows": B,
                   "parallelism": "single GPU"},
        "decode": {"state_GB_per_s": round(dec_gbps, 1), "frac_of_hbm_peak": round(dec_gbps / HBM_PEAK_GBPS, 4),
                   "ms": t_dec, "state_bytes": dec_bytes,
                   # the same launch timed back to back over 4 disjoint 64-slot sets of the
                   # 256-slot cache (every launch's states cold), without a pair of events
                   # around each launch
                   "back_to_back_ms": round(t_dec_b2b, 5),
                   "back_to_back_frac_of_hbm_peak": round(dec_bytes / (t_dec_b2b * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                   # the same bytes in two reference patterns, timed the same way: a plain
                   # streaming copy, and the decode's read-reduce-write dependency
                   # without its arithmetic (libgdn_probe.so)
                   "stream_copy_ms": round(t_copy_ref, 5),
                   "stream_copy_frac_of_hbm_peak": round(dec_bytes / (t_copy_ref * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                   "state_rmw_ms": round(t_rmw_ref, 5),
                   "state_rmw_frac_of_hbm_peak": round(dec_bytes / (t_rmw_ref * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                   "back_to_back_frac_of_state_rmw": round(t_rmw_ref / t_dec_b2b, 4)},
        "prefill": {"tokens_per_s": round(Tp / (t_pre * 1e-3), 1), "ms": t_pre,
                    "hbm_frac": round(pre_gbps / HBM_PEAK_GBPS, 4),
                    "mfma_frac": round(pre_tflops / BF16_PEAK_TFLOPS, 4), "flops_per_token": f_tok,
                    "bytes_per_token": b_tok},
        "copy_GB_per_s": round(copy_gbps, 1),
        "roofline": roofline,
        "kernels": kernels,
    }
    if not args.no_secondary:
        out["other_workloads"] = secondary_configs(torch, binding, W, dev, args.secondary_calls, args.warmup)

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wp, wd)
    print("input generation %.1f s; step %.3f ms = decode %.4f + prefill %.4f ms" % (
        gen_s, ms_step, t_dec, t_pre), file=sys.stderr)
    print(json.dumps(out), flush=True)


def decode_back_to_back(torch, binding, wd, q, k, v, g, beta, o, pool, dev, rounds=5):
    """Average duration of the decode launch over rounds x 4 launches issued back to
    back, each on a different one of 4 disjoint 64-slot sets that cover the 256-slot
    cache (in place), so that no launch finds its states in a cache.  Returns ms."""
    B = wd.num_decode_rows
    slots = wd.pool.shape[0]
    nsets = slots // B
    perm = np.concatenate([wd.slot_in, np.setdiff1d(np.arange(slots), wd.slot_in)]).astype(np.int32)
    sets = [torch.as_tensor(perm[i * B:(i + 1) * B], device=dev) for i in range(nsets)]
    for s in sets:
        binding.gdn_recurrent_decode(q, k, v, g, beta, o, pool, s, s, scale=wd.scale)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(rounds):
        for s in sets:
            binding.gdn_recurrent_decode(q, k, v, g, beta, o, pool, s, s, scale=wd.scale)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (rounds * nsets)


def probe_library():
    """libgdn_probe.so: the memory-pattern reference kernels (a streaming copy and the
    decode's read-reduce-write pattern without its arithmetic)."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "gated_deltanet_rule_amd", "libgdn_probe.so"))
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    lib.gdn_probe_stream_copy.restype = i32
    lib.gdn_probe_stream_copy.argtypes = [vp, vp, sz, vp]
    lib.gdn_probe_state_rmw.restype = i32
    lib.gdn_probe_state_rmw.argtypes = [vp, i32, i32, vp, i32, vp]
    return lib


def decode_floors(torch, wd, pool, dev, rounds=5):
    """What HBM delivers for the decode batch's bytes (2 x 128 MiB of state per launch)
    in two reference patterns, each timed back to back like the decode: a streaming
    copy of 128 MiB rotating over 4 disjoint source/destination pairs of a 1 GiB
    buffer, and the decode's read-reduce-write pattern without its arithmetic over the
    same 4 disjoint 64-slot sets of the cache.  Returns (copy ms, rmw ms)."""
    import ctypes
    lib = probe_library()
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    B, H_v = wd.num_decode_rows, wd.H_v
    nbytes = 4 * wd.d_k * wd.d_v * B * H_v
    buf = torch.empty(8 * nbytes // 4, dtype=torch.float32, device=dev)
    pairs = [(buf.data_ptr() + i * nbytes, buf.data_ptr() + (i + 4) * nbytes) for i in range(4)]
    slots = wd.pool.shape[0]
    perm = np.concatenate([wd.slot_in, np.setdiff1d(np.arange(slots), wd.slot_in)]).astype(np.int32)
    sets = [torch.as_tensor(perm[i * B:(i + 1) * B], device=dev) for i in range(slots // B)]

    def copy():
        for sp, dp in pairs:
            assert lib.gdn_probe_stream_copy(ctypes.c_void_p(sp), ctypes.c_void_p(dp), nbytes, stream) == 0

    def rmw():
        for st in sets:
            assert lib.gdn_probe_state_rmw(ctypes.c_void_p(pool.data_ptr()), pool.shape[0], H_v,
                                           ctypes.c_void_p(st.data_ptr()), B, stream) == 0

    copy()
    rmw()
    t_copy = time_loop(torch, copy, rounds) / len(pairs)
    t_rmw = time_loop(torch, rmw, rounds) / len(sets)
    del buf
    return t_copy, t_rmw


def copy_bandwidth(torch, dev, mib=1024, reps=10):
    """Achievable HBM bandwidth of a plain device-to-device copy (read + write bytes
    per second), the practical ceiling next to the 8 TB/s peak."""
    src = torch.ones(mib << 18, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    gbps = 2 * (mib << 20) * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    return gbps


def _median_runs(fn, runs=3, single_if_over_s=60.0):
    """Median wall time (s) of up to `runs` calls of fn; one call when the first takes
    longer than single_if_over_s."""
    ts = []
    for _ in range(runs):
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
        if ts[0] > single_if_over_s:
            break
    return float(np.median(ts)), len(ts)


def cpu_baseline(wp, wd, all_core_seqs=4, one_thread_tokens=2048):
    """The oracle as it stands (fp64 sequential recurrence, OpenMP over (sequence,
    head) units) on bounded samples of the same workloads: every host core on
    all_core_seqs of the 16 long sequences (all 32 heads, exports on the 1088 grid),
    and one thread on the first one_thread_tokens tokens of one sequence; each the
    median of 3 runs (one run if a run exceeds 60 s).  Decode likewise on the whole
    64-row batch."""
    import oracle
    L = wp.lengths[0]
    n_seqs = max(1, min(all_core_seqs, wp.num_seqs))
    T = n_seqs * L
    cu = np.arange(n_seqs + 1, dtype=np.int32) * L
    cores = oracle.num_threads()
    pre_s, pre_runs = _median_runs(lambda: oracle.prefill(wp.q[:T], wp.k[:T], wp.v[:T], wp.g[:T], wp.beta[:T], cu,
                                                          scale=wp.scale, export_grid=wp.export_grid))
    B = wd.num_decode_rows
    compact = wd.pool[wd.slot_in].astype(np.float64)
    idx = np.arange(B, dtype=np.int32)
    dec = lambda: oracle.decode(wd.q, wd.k, wd.v, wd.g, wd.beta, compact.copy(), idx, idx, scale=wd.scale)
    dec_s, dec_runs = _median_runs(dec)
    dec_bytes = 2 * 4 * wd.d_k * wd.d_v * B * wd.H_v
    T1 = min(one_thread_tokens, L)
    oracle.set_num_threads(1)
    try:
        one_s, one_runs = _median_runs(lambda: oracle.prefill(
            wp.q[:T1], wp.k[:T1], wp.v[:T1], wp.g[:T1], wp.beta[:T1], np.array([0, T1], dtype=np.int32),
            scale=wp.scale, export_grid=wp.export_grid))
        dec1_s, dec1_runs = _median_runs(dec)
    finally:
        oracle.set_num_threads(cores)
    return {"value": round(T / pre_s, 1), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": "prefill of %d of the 16 long sequences (%d tokens, all 32 heads, exports on the 1088 grid), "
                      "median of %d runs of %.2f s" % (n_seqs, T, pre_runs, pre_s),
            "decode_state_GB_per_s": round(dec_bytes / dec_s / 1e9, 3),
            "decode_sample": "the 64-row decode batch, median of %d runs of %.3f s" % (dec_runs, dec_s),
            "one_thread": {"value": round(T1 / one_s, 1), "unit": "tokens/s", "cores": 1,
                           "sample": "prefill of the first %d tokens of one long sequence (all 32 heads), median of "
                                     "%d runs of %.2f s" % (T1, one_runs, one_s),
                           "decode_state_GB_per_s": round(dec_bytes / dec1_s / 1e9, 3)}}


if __name__ == "__main__":
    main()
