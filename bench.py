#!/usr/bin/env python3
"""Throughput of the MoE expert layer with per-request LoRA deltas on one MI355X.

A step is one pass of the whole hot path over one batch: moe_lora_info (the
per-batch metadata), moe_lora_align and moe_lora_forward.  The default workload
is the largest layer that fits one GPU: 256 routed experts, top-8, hidden 7168,
moe intermediate 2048 (22.5 GB of expert weights), 8 adapter slots of rank 32,
one prefill batch of 16384 tokens in 64 requests, bf16 (--config picks another).
Inputs are synthetic and resident in HBM before timing starts.

Prints one JSON line with tokens/s, the roofline of the dominant kernel (the
gate_up GEMM, timed with HIP events around its launch inside the timed region),
the median of graph replays of [align -> forward], and the CPU oracle timed on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 vector / MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="c4p")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=-1,
                    help="tokens of the batch the CPU oracle runs on (0: all of them; -1: as "
                         "many as about 1.5 TFLOP of oracle work)")
    ap.add_argument("--graph-replays", type=int, default=50,
                    help="HIP-graph replays of [align -> forward] timed one by one (median)")
    ap.add_argument("--cpu-min-seconds", type=float, default=10.0,
                    help="repeat the oracle pass over the sample until this much time has passed")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="HBM traffic per launch measured with rocprofv3 counters")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (3 times) and exit: "
                         "the reference kernel that scales FETCH_SIZE / WRITE_SIZE counters")
    ap.add_argument("--traffic-from", default=None, metavar="DIR",
                    help="host only: read the rocprofv3 counter CSVs under DIR/{fetch,write,"
                         "cfetch,cwrite} (and, when present, DIR/mfma and DIR/tcc), write the "
                         "calibrated per-launch HBM traffic, MFMA utilisation and L2 hit rate of "
                         "every layer kernel of --config to --traffic and exit")
    return ap.parse_args()


# kernel name (rocprofv3, mangled or not) -> forward stage or metadata kernel
def _stage_of(kname):
    if "gate_up_fixup_kernel" in kname:   # finishes the gate_up tail tiles split into K pieces
        return "gate_up_fixup"
    if "gemm_kernel" in kname or "gemm_big_kernel" in kname:
        gate_up = ("Lb1E" in kname) or kname.rstrip(") ").split("(")[0].endswith("true>")
        return "gate_up_gemm" if gate_up else "down_gemm"
    if "shrink_reduce" in kname:
        return "shrink_reduce"
    if "shrink_kernel" in kname or "shrink4_kernel" in kname:
        return "shrink_gate_up" if ("Li2E" in kname or ", 2>" in kname or ", 2," in kname) \
            else "shrink_down"
    for key in ("combine", "plan", "tile_table", "info", "align_count", "align_scan", "align_scatter"):
        if key + "_kernel" in kname:
            return key
    return None


def kernel_source_hash():
    """Hash of the kernel sources and build script: counters taken on other code are stale."""
    import hashlib
    h = hashlib.sha256()
    pkg = os.path.join(ROOT, "moe_expert_layer_segment_amd")
    csrc = os.path.join(pkg, "csrc")
    for name in sorted(os.listdir(csrc)) + ["../build.py"]:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def traffic_from_counters(args):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) -> bytes per launch, each scaled by what
    the same counter reads for a plain copy of known size."""
    import csv
    import collections

    def per_kernel(sub, counter):
        path = os.path.join(args.traffic_from, sub, "run_counter_collection.csv")
        agg = collections.defaultdict(list)
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    agg[r["Kernel_Name"]].append(float(r["Counter_Value"]))
        return agg

    def copy_kib(d):
        vals = [max(v) for k, v in d.items() if "copy" in k.lower() or "elementwise" in k.lower()]
        assert vals, "no copy kernel in the calibration run"
        return max(vals)

    mib = 1024
    f_scale = mib * 1024 / copy_kib(per_kernel("cfetch", "FETCH_SIZE"))
    w_scale = mib * 1024 / copy_kib(per_kernel("cwrite", "WRITE_SIZE"))
    fetch, write = per_kernel("fetch", "FETCH_SIZE"), per_kernel("write", "WRITE_SIZE")
    stages = {}
    for kname, vals in fetch.items():
        st = _stage_of(kname)
        if st is None:
            continue
        wv = write.get(kname, [0.0])
        fb = float(np.mean(vals)) * f_scale * 1024
        wb = float(np.mean(wv)) * w_scale * 1024
        stages[st] = dict(bytes=round(fb + wb), fetch_bytes=round(fb), write_bytes=round(wb),
                          dispatches=len(vals))

    def optional(sub, counter):
        path = os.path.join(args.traffic_from, sub, "run_counter_collection.csv")
        return per_kernel(sub, counter) if os.path.exists(path) else {}

    # MFMA utilisation: MFMA-busy cycles summed over the 1024 SIMDs against the
    # GPU-active cycles (GRBM_GUI_ACTIVE, summed over the 8 XCDs) of the dispatch
    busy, active = optional("mfma", "SQ_VALU_MFMA_BUSY_CYCLES"), optional("mfma", "GRBM_GUI_ACTIVE")
    for kname, vals in busy.items():
        st = _stage_of(kname)
        if st in stages and kname in active:
            cyc = float(np.mean(active[kname])) / 8
            stages[st]["mfma_busy_frac"] = round(float(np.mean(vals)) / (cyc * 1024), 4)
            stages[st]["gpu_cycles"] = round(cyc)
    hit, miss = optional("tcc", "TCC_HIT_sum"), optional("tcc", "TCC_MISS_sum")
    for kname, vals in hit.items():
        st = _stage_of(kname)
        if st in stages and kname in miss:
            h, m = float(np.mean(vals)), float(np.mean(miss[kname]))
            stages[st]["l2_hit_rate"] = round(h / max(h + m, 1.0), 4)
            stages[st]["l2_requests"] = round(h + m)
    from moe_expert_layer_segment_amd import workloads
    spec = workloads.config(args.config)
    out = {}
    if os.path.exists(args.traffic):
        with open(args.traffic) as f:
            out = json.load(f)
    out[spec.name] = dict(stages=stages, fetch_scale=round(f_scale, 4),
                          write_scale=round(w_scale, 4), copy_calibration_mib=mib,
                          source_hash=kernel_source_hash())
    with open(args.traffic, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
    print(json.dumps(out[spec.name]))


def copy_calibration(mib):
    """A plain device-to-device copy of known size, for counter calibration."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_mib": mib, "bytes_read": n * 4, "bytes_written": n * 4}))


class HipEvents:
    """Raw hipEvent_t handles through libamdhip64 (recorded by the library on
    the stream its kernels run on).  Created without the system-scope fence: a
    default event record writes back and invalidates the caches, which idles
    the GPU for microseconds and starts the next kernel with a cold L2; these
    events only time work."""

    DISABLE_SYSTEM_FENCE = 0x20000000   # hipEventDisableSystemFence

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreateWithFlags(ctypes.byref(e), self.DISABLE_SYSTEM_FENCE) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            out.append(e.value)
        return out

    def record(self, e, stream):
        if self.hip.hipEventRecord(ctypes.c_void_p(e), ctypes.c_void_p(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(ctypes.c_void_p(e))


def timed_steps(args, torch, hip, step, stages, kernel):
    """Time args.steps steps between two events on the launch stream.  Inside
    the timed region only the dominant kernel is bracketed by HIP events (its
    live duration for the roofline): every event recorded between kernels
    leaves the GPU idle for several microseconds, which a marker at each stage
    boundary would add to the step.  The per-stage breakdown comes from
    further, untimed steps with an event pair around every stage.
    Returns (ms per step, kernel ms, {stage: ms})."""
    nst = len(stages)
    ki = stages.index(kernel)
    ev = []
    for _ in range(args.steps):
        pair = hip.create(2)
        e = [None] * (2 * nst)
        e[2 * ki], e[2 * ki + 1] = pair
        ev.append(e)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for st in range(args.steps):
        step(ev[st])
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    k_ms = float(np.mean([hip.elapsed_ms(e[2 * ki], e[2 * ki + 1]) for e in ev]))
    for e in ev:
        hip.destroy([e[2 * ki], e[2 * ki + 1]])
    nb = max(1, min(args.steps, 10))
    evb = [hip.create(2 * nst) for _ in range(nb)]
    evm = [hip.create(3) for _ in range(nb)]   # before info, after info, after align
    for st in range(nb):
        step(evb[st], evm[st])
    torch.cuda.synchronize()
    stage_ms = {name: float(np.mean([hip.elapsed_ms(e[2 * i], e[2 * i + 1]) for e in evb]))
                for i, name in enumerate(stages)}
    stage_ms["info"] = float(np.mean([hip.elapsed_ms(e[0], e[1]) for e in evm]))
    stage_ms["align"] = float(np.mean([hip.elapsed_ms(e[1], e[2]) for e in evm]))
    for e in evb + evm:
        hip.destroy(e)
    return ms, k_ms, stage_ms


def graph_replays(torch, hip, fn, n):
    """Capture fn ([align -> forward]) in a HIP graph and time n replays one by
    one, each between two fence-free events on the replay stream; returns
    (median ms, min ms, max ms).  The library launches kernels only (no
    allocation, memset or host synchronisation), so the capture holds the same
    kernels the eager step runs."""
    if n <= 0:
        return None
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up on the capture stream
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream().cuda_stream
    evs = [hip.create(2) for _ in range(n)]
    for a, b in evs:
        hip.record(a, stream)
        g.replay()
        hip.record(b, stream)
    torch.cuda.synchronize()
    ms = np.array([hip.elapsed_ms(a, b) for a, b in evs])
    for e in evs:
        hip.destroy(e)
    del g
    return float(np.median(ms)), float(ms.min()), float(ms.max())


def default_cpu_sample(spec):
    """Tokens of the batch for the CPU oracle: about 1.5 TFLOP of float64 work
    (10-30 s on the host's cores with the oracle's per-expert BLAS products)."""
    per_token = 6.0 * spec.hidden * spec.inter * spec.top_k
    return int(min(spec.num_tokens, max(64, 1.5e12 // per_token)))


def metadata_rates(binding, spec, stage_ms, BM):
    """info and align: latency-bound, reported in us with the GB/s of their
    algorithmic bytes as evidence (info: the request arrays, the slot ranks and
    the two outputs; align: 8 B read and 4 B written per pair plus the tile
    tables and expert offsets)."""
    T, k, E, L = spec.num_tokens, spec.top_k, spec.num_experts, spec.num_loras
    bs, P = spec.num_reqs, spec.num_tokens * spec.top_k
    cap = binding.moe_lora_align_capacity_rows(T, k, E, L, BM)
    info_b = 4 * (bs + 1) + 4 * bs + 4 * L + 4 * T + 4 * L
    align_b = 12 * P + 8 * (cap // BM) + 4 * (E + 1) + 4
    out = {}
    for name, nbytes in (("info", info_b), ("align", align_b)):
        ms = stage_ms[name]
        out[name] = {"us": round(ms * 1e3, 2), "bytes": int(nbytes),
                     "gbs": round(nbytes / (ms * 1e-3) / 1e9, 2) if ms > 0 else None}
    return out


def counts(spec, meta):
    """FLOPs and bytes the method itself must do for this batch (padding,
    intermediates and pool rows beyond each slot's rank excluded)."""
    T, k, E, H, I = spec.num_tokens, spec.top_k, spec.num_experts, spec.hidden, spec.inter
    ids = meta["topk_ids"]
    indptr = meta["seg_indptr"]
    wi = meta["weight_indices"]
    ranks = meta["lora_ranks"]
    mapping = np.repeat(wi, np.diff(indptr))
    used = set(int(v) for v in wi if v >= 0)
    on_slot = np.array([(l in used and ranks[l] > 0) for l in range(len(ranks))], dtype=bool)
    tok = np.repeat(np.arange(T), k)
    e_of = ids.reshape(-1)
    l_of = mapping[tok]
    r_of = np.where((l_of >= 0) & on_slot[np.maximum(l_of, 0)] if len(ranks) else False,
                    ranks[np.maximum(l_of, 0)] if len(ranks) else 0, 0)
    P = T * k
    esz = 2 if spec.dtype == "bf16" else 4
    fp8 = spec.weights == "fp8"
    wsz = 1 if fp8 else esz                       # bytes per expert weight
    fl_gate_up_base = 4.0 * H * I * P
    fl_gate_up_expand = 4.0 * float(np.sum(r_of)) * I
    fl_shrink = 4.0 * float(np.sum(r_of)) * H + 2.0 * float(np.sum(r_of)) * I
    fl_down = 2.0 * H * I * P + 2.0 * float(np.sum(r_of)) * H
    total_flops = fl_gate_up_base + fl_gate_up_expand + fl_shrink + fl_down
    active = np.unique(e_of)
    # expert weights (+ their fp32 128 x 128 block scales when fp8)
    w_bytes = len(active) * 3.0 * H * I * (wsz + (4.0 / (128 * 128) if fp8 else 0.0))
    buckets = set(zip(e_of[r_of > 0].tolist(), l_of[r_of > 0].tolist()))
    lora_bytes = sum(3.0 * ranks[l] * (H + I) * esz for (_, l) in buckets)
    io_bytes = 2.0 * T * H * esz + 8.0 * P
    gate_up_bytes = len(active) * 2.0 * H * I * (wsz + (4.0 / (128 * 128) if fp8 else 0.0)) + T * H * esz
    return dict(total_flops=total_flops, gate_up_flops=fl_gate_up_base + fl_gate_up_expand,
                total_bytes=w_bytes + lora_bytes + io_bytes, gate_up_bytes=gate_up_bytes,
                active_experts=int(len(active)), lora_buckets=len(buckets))


def cpu_baseline(spec, inp, n_tokens, min_seconds):
    """The oracle as it stands, on a bounded sample of the workload's tokens, repeated
    (at most 8 passes) until min_seconds have passed."""
    import oracle
    import torch

    T = spec.num_tokens
    n_tokens = T if n_tokens <= 0 else min(n_tokens, T)
    sample = np.unique(np.linspace(0, T - 1, n_tokens).astype(np.int64))
    m = inp["meta"]

    class View:
        def __init__(self, t):
            self.t = t

        def __getitem__(self, idx):
            idx = idx if isinstance(idx, tuple) else (idx,)
            return self.t[tuple(int(i) for i in idx)].float().cpu().numpy()

    x_host = inp["x"][torch.as_tensor(sample, device=inp["x"].device)].float().cpu().numpy()
    # the oracle indexes x by token id; give it a dict view over the sample
    xs = {int(t): x_host[i] for i, t in enumerate(sample)}

    class XView:
        def __getitem__(self, t):
            return xs[int(t)]

    class Fp8View:
        """fp8 expert weights, dequantized by the oracle one expert at a time"""
        def __init__(self, codes, scales):
            self.codes, self.scales = codes, scales

        def __getitem__(self, idx):
            idx = idx if isinstance(idx, tuple) else (idx,)
            e = int(idx[0])
            w = oracle.dequantize_block_fp8(self.codes[e].cpu().numpy(), self.scales[e].cpu().numpy())
            return w[tuple(int(i) for i in idx[1:])] if len(idx) > 1 else w

    if "w_gate_up_scale" in inp:
        w_gu = Fp8View(inp["w_gate_up"], inp["w_gate_up_scale"])
        w_d = Fp8View(inp["w_down"], inp["w_down_scale"])
    else:
        w_gu, w_d = View(inp["w_gate_up"]), View(inp["w_down"])
    pools = {n: View(inp[n]) for n in ("a_gate", "a_up", "b_gate", "b_up", "a_down", "b_down")
             if n in inp}
    t0 = time.perf_counter()
    passes = 0
    while passes < 8 and (passes == 0 or time.perf_counter() - t0 < min_seconds):
        en, mp = oracle.moe_lora_info(T, m["seg_indptr"], m["weight_indices"], m["lora_ranks"],
                                      m["max_seg_len"])
        oracle.moe_lora_forward(XView(), m["topk_ids"], m["topk_weights"], w_gu, w_d,
                                m["lora_ranks"], m["scaling"], mp, en, tokens=sample, **pools)
        passes += 1
    dt = time.perf_counter() - t0
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    omp = os.environ.get("OMP_NUM_THREADS")
    if omp and omp.isdigit():
        cores = min(cores, int(omp))
    return dict(value=passes * len(sample) / dt, unit="tokens/s", cores=cores, kind="oracle",
                sample=f"{len(sample)} of {T} tokens (evenly spaced) of the same batch, "
                       f"{passes} pass(es); float64 numpy oracle incl. per-expert upcast of the "
                       f"touched weights; {dt:.1f} s")


def dense_main(args, torch, binding, workloads, dev):
    """The second workload: the dense two-slice LoRA projection (info + align +
    dense forward per step), one JSON line in the same shape as the layer's."""
    spec = workloads.dense_config(args.config)
    print(f"[bench] generating {spec.name} on {dev}", file=sys.stderr, flush=True)
    inp = workloads.generate_dense(spec, device=dev, canary=False)
    T, H, N0, N1, L = spec.num_tokens, spec.hidden, spec.out0, spec.out1, spec.num_loras
    N = N0 + N1
    BM = 16
    pools = {n: inp[n] for n in ("a0", "a1", "b0", "b1")} if L > 0 else None
    en_buf = torch.empty(max(L, 1), dtype=torch.int32, device=dev)
    mp_buf = torch.empty(max(T, 1), dtype=torch.int32, device=dev)
    en, mp = binding.moe_lora_info(T, inp["seg_indptr"], inp["lora_ranks"], inp["weight_indices"],
                                   en_buf, mp_buf, max_len=inp["meta"]["max_seg_len"])
    al = binding.moe_lora_align(inp["topk_ids"], mp, en if L > 0 else None, 1, L, BM)
    al_ws = torch.empty(binding.moe_lora_align_workspace_bytes(T, 1, 1, L, BM), dtype=torch.uint8,
                        device=dev)
    y = torch.empty((T, N), dtype=inp["x"].dtype, device=dev)
    ws = torch.empty(binding.moe_lora_dense_workspace_bytes(
        inp["x"], inp["w"], N0, al, inp["lora_ranks"], inp["scaling"], pools), dtype=torch.uint8,
        device=dev)
    hip = HipEvents()

    def step(events=None, meta_events=None):
        stream = torch.cuda.current_stream().cuda_stream
        if meta_events:
            hip.record(meta_events[0], stream)
        binding.moe_lora_info(T, inp["seg_indptr"], inp["lora_ranks"], inp["weight_indices"],
                              en_buf, mp_buf, max_len=inp["meta"]["max_seg_len"])
        if meta_events:
            hip.record(meta_events[1], stream)
        binding.moe_lora_align(inp["topk_ids"], mp, en if L > 0 else None, 1, L, BM, out=al,
                               workspace=al_ws)
        if meta_events:
            hip.record(meta_events[2], stream)
        binding.moe_lora_dense_forward(inp["x"], inp["w"], N0, al,
                                       inp["lora_ranks"] if L > 0 else None,
                                       inp["scaling"] if L > 0 else None, pools, y=y,
                                       workspace=ws, events=events)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ms, g_ms, stage_ms = timed_steps(args, torch, hip, step, binding.DENSE_STAGES, "gemm")

    m = inp["meta"]
    ranks = np.asarray(m["lora_ranks"])
    tok_slot = np.repeat(np.asarray(m["weight_indices"]), np.diff(np.asarray(m["seg_indptr"])))
    used = set(int(v) for v in tok_slot if v >= 0)
    r_tok = np.array([ranks[l] if (l >= 0 and l in used and ranks[l] > 0) else 0 for l in tok_slot])
    esz = 2 if spec.dtype == "bf16" else 4
    gemm_flops = 2.0 * T * H * N + 2.0 * float(np.sum(r_tok)) * N
    total_flops = gemm_flops + 2.0 * float(np.sum(r_tok)) * H * (2 if N1 > 0 else 1)
    gemm_bytes = N * H * esz + T * H * esz + 4.0 * T * N
    peak = PEAK_BF16_TFLOPS if spec.dtype == "bf16" else PEAK_FP32_TFLOPS
    if gemm_flops / gemm_bytes >= peak * 1e12 / (PEAK_HBM_GBS * 1e9):
        a = gemm_flops / (g_ms * 1e-3) / 1e12
        roofline = dict(bound="mfma", achieved=round(a, 2), peak=peak, unit="TFLOP/s",
                        frac=round(a / peak, 4), traffic=None, kernel="dense_gemm",
                        kernel_ms=round(g_ms, 4), kernel_flops=gemm_flops)
    else:
        gbs = gemm_bytes / (g_ms * 1e-3) / 1e9
        roofline = dict(bound="hbm", achieved=round(gbs, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                        frac=round(gbs / PEAK_HBM_GBS, 4), traffic=None, kernel="dense_gemm",
                        kernel_ms=round(g_ms, 4), kernel_bytes=gemm_bytes)
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        n = T if args.cpu_sample_tokens <= 0 else min(args.cpu_sample_tokens, T)
        sample = np.unique(np.linspace(0, T - 1, n).astype(np.int64))
        xh = inp["x"].float().cpu().numpy()
        wh = inp["w"].float().cpu().numpy()
        ph = {k: v.float().cpu().numpy() for k, v in (pools or {}).items()}
        t0, passes = time.perf_counter(), 0
        while passes < 8 and (passes == 0 or time.perf_counter() - t0 < args.cpu_min_seconds):
            en_o, mp_o = oracle.moe_lora_info(T, m["seg_indptr"], m["weight_indices"],
                                              m["lora_ranks"], m["max_seg_len"])
            oracle.dense_lora_forward(xh, wh, N0, m["lora_ranks"], m["scaling"], mp_o, en_o,
                                      tokens=sample, **ph)
            passes += 1
        dt = time.perf_counter() - t0
        try:
            cores = len(os.sched_getaffinity(0))
        except AttributeError:
            cores = os.cpu_count() or 1
        omp = os.environ.get("OMP_NUM_THREADS")
        if omp and omp.isdigit():
            cores = min(cores, int(omp))
        cpu = dict(value=passes * len(sample) / dt, unit="tokens/s", cores=cores, kind="oracle",
                   sample=f"{len(sample)} of {T} tokens (evenly spaced), {passes} pass(es); "
                          f"float64 numpy oracle; {dt:.1f} s")
    out = {
        "metric": "dense LoRA projection tokens/s", "value": round(T / (ms * 1e-3), 1),
        "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if spec.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": spec.name, "hidden": H, "out0": N0, "out1": N1, "tokens": T,
                   "requests": spec.num_reqs, "adapter_slots": L, "lora_ranks": list(spec.lora_ranks),
                   "block_m": BM, "parallelism": "tp1"},
        "roofline": roofline, "cpu_baseline": cpu,
        "stages_ms": {k: round(v, 4) for k, v in stage_ms.items()},
    }
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.traffic_from:
        traffic_from_counters(args)
        return
    if args.copy_calibration_mib:
        copy_calibration(args.copy_calibration_mib)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the layer runs at TP=1 on a single MI355X; there is "
              "no multi-GPU path (the per-rank kernels run at their shard shapes with "
              "--config c1_tp2, c1_tp4, c1_tp8, c4p_ep8 or c4d_ep8).", file=sys.stderr)
        sys.exit(2)

    import torch
    from moe_expert_layer_segment_amd import binding, workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.config in workloads.DENSE_CONFIG_NAMES:
        dense_main(args, torch, binding, workloads, dev)
        return
    spec = workloads.config(args.config)
    print(f"[bench] generating {spec.name} on {dev}", file=sys.stderr, flush=True)
    inp = workloads.generate(spec, device=dev, canary=False)
    torch.cuda.synchronize()

    T, k, E = spec.num_tokens, spec.top_k, spec.num_experts
    L = spec.num_loras
    BM = 16
    pools = {n: inp[n] for n in binding._POOLS} if L > 0 else None
    en_buf = torch.empty(max(L, 1), dtype=torch.int32, device=dev)
    mp_buf = torch.empty(max(T, 1), dtype=torch.int32, device=dev)
    en, mp = binding.moe_lora_info(T, inp["seg_indptr"], inp["lora_ranks"], inp["weight_indices"],
                                   en_buf, mp_buf, max_len=inp["meta"]["max_seg_len"])
    al = binding.moe_lora_align(inp["topk_ids"], mp, en if L > 0 else None, E, L, BM)
    al_ws = torch.empty(binding.moe_lora_align_workspace_bytes(T, k, E, L, BM), dtype=torch.uint8,
                        device=dev)
    y = torch.empty_like(inp["x"])
    w_scales = ((inp["w_gate_up_scale"], inp["w_down_scale"]) if "w_gate_up_scale" in inp
                else None)
    fws = torch.empty(binding.moe_lora_forward_workspace_bytes(
        inp["x"], inp["topk_weights"], inp["w_gate_up"], inp["w_down"], al, k,
        inp["lora_ranks"], inp["scaling"], pools, w_scales), dtype=torch.uint8, device=dev)

    hip = HipEvents()

    def step(events=None, meta_events=None):
        stream = torch.cuda.current_stream().cuda_stream
        if meta_events:
            hip.record(meta_events[0], stream)
        binding.moe_lora_info(T, inp["seg_indptr"], inp["lora_ranks"], inp["weight_indices"],
                              en_buf, mp_buf, max_len=inp["meta"]["max_seg_len"])
        if meta_events:
            hip.record(meta_events[1], stream)
        binding.moe_lora_align(inp["topk_ids"], mp, en if L > 0 else None, E, L, BM, out=al,
                               workspace=al_ws)
        if meta_events:
            hip.record(meta_events[2], stream)
        binding.moe_lora_forward(inp["x"], inp["topk_weights"], inp["w_gate_up"], inp["w_down"],
                                 al, k, inp["lora_ranks"] if L > 0 else None,
                                 inp["scaling"] if L > 0 else None, pools, y=y, workspace=fws,
                                 events=events, w_scales=w_scales)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

    t0 = time.perf_counter()
    ms, gu_ms, stage_ms = timed_steps(args, torch, hip, step, binding.FORWARD_STAGES, "gate_up_gemm")
    wall = time.perf_counter() - t0
    print(f"[bench] timed {args.steps} steps: {ms:.3f} ms/step (wall {wall:.2f} s)",
          file=sys.stderr, flush=True)

    def align_forward():
        binding.moe_lora_align(inp["topk_ids"], mp, en if L > 0 else None, E, L, BM, out=al,
                               workspace=al_ws)
        binding.moe_lora_forward(inp["x"], inp["topk_weights"], inp["w_gate_up"], inp["w_down"],
                                 al, k, inp["lora_ranks"] if L > 0 else None,
                                 inp["scaling"] if L > 0 else None, pools, y=y, workspace=fws,
                                 w_scales=w_scales)

    graph = None
    if args.graph_replays > 0:
        gmed, gmin, gmax = graph_replays(torch, hip, align_forward, args.graph_replays)
        graph = {"what": "align + forward captured in one HIP graph; info once per batch",
                 "replays": args.graph_replays, "median_ms": round(gmed, 4),
                 "min_ms": round(gmin, 4), "max_ms": round(gmax, 4),
                 "tokens_per_s": round(T / (gmed * 1e-3), 1)}
        print(f"[bench] {args.graph_replays} graph replays: median {gmed:.3f} ms", file=sys.stderr,
              flush=True)

    # the router step before the layer (not part of the step): its time on this
    # workload's router logits, events on the current stream (the launch stream)
    logits = torch.from_numpy(workloads.router_logits(spec).astype(np.float32)).to(dev)
    r_ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    r_w = torch.empty((T, k), dtype=torch.float32, device=dev)
    for _ in range(3):
        binding.moe_lora_route(logits, k, r_ids, r_w)
    r_start, r_stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    r_start.record()
    for _ in range(20):
        binding.moe_lora_route(logits, k, r_ids, r_w)
    r_stop.record()
    torch.cuda.synchronize()
    router_ms = r_start.elapsed_time(r_stop) / 20

    c = counts(spec, inp["meta"])
    achieved = c["gate_up_flops"] / (gu_ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if spec.dtype == "bf16" else PEAK_FP32_TFLOPS
    traffic = None
    if os.path.exists(args.traffic):
        with open(args.traffic) as f:
            rec = json.load(f).get(spec.name, {})
        # counters taken on other kernel code say nothing about this one
        if rec.get("source_hash") == kernel_source_hash():
            traffic = rec.get("stages", {}).get("gate_up_gemm", {}).get("bytes")
    if c["gate_up_flops"] / c["gate_up_bytes"] >= peak * 1e12 / (PEAK_HBM_GBS * 1e9):
        roofline = dict(bound="mfma", achieved=round(achieved, 2), peak=peak, unit="TFLOP/s",
                        frac=round(achieved / peak, 4), traffic=traffic,
                        kernel="gate_up_gemm", kernel_ms=round(gu_ms, 4),
                        kernel_flops=c["gate_up_flops"])
    else:
        # below the ridge point (decode): the weight stream bounds the kernel
        gbs = c["gate_up_bytes"] / (gu_ms * 1e-3) / 1e9
        roofline = dict(bound="hbm", achieved=round(gbs, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                        frac=round(gbs / PEAK_HBM_GBS, 4), traffic=traffic,
                        kernel="gate_up_gemm", kernel_ms=round(gu_ms, 4),
                        kernel_bytes=c["gate_up_bytes"])

    cpu = None
    if not args.no_cpu_baseline:
        n_cpu = default_cpu_sample(spec) if args.cpu_sample_tokens < 0 else args.cpu_sample_tokens
        print(f"[bench] timing the CPU oracle on a sample of {n_cpu or T} tokens", file=sys.stderr,
              flush=True)
        cpu = cpu_baseline(spec, inp, n_cpu, args.cpu_min_seconds)

    tok_s = T / (ms * 1e-3)
    out = {
        "metric": "MoE-LoRA layer tokens/s",
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("bf16" if spec.dtype == "bf16" else "f32") + (" (fp8 e4m3 weights)" if spec.weights == "fp8" else ""),
        "data": "synthetic",
        "config": {"workload": spec.name, "experts": E, "top_k": k, "hidden": spec.hidden,
                   "intermediate": spec.inter, "tokens": T, "requests": spec.num_reqs,
                   "adapter_slots": L, "lora_ranks": list(spec.lora_ranks),
                   "block_m": BM, "parallelism": "tp1"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "layer": {"tflops": round(c["total_flops"] / (ms * 1e-3) / 1e12, 2),
                  "gbs": round(c["total_bytes"] / (ms * 1e-3) / 1e9, 1),
                  "algorithmic_flops": c["total_flops"], "algorithmic_bytes": c["total_bytes"],
                  "active_experts": c["active_experts"], "lora_buckets": c["lora_buckets"]},
        "graph": graph,
        "stages_ms": {kk: round(v, 4) for kk, v in stage_ms.items()},
        "metadata": metadata_rates(binding, spec, stage_ms, BM),
        "router_ms": round(router_ms, 4),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
