"""Benchmark of the fused MoE forward on one MI355X.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--workload NAME]
                    [--no-cpu-baseline] [--copy-probe]

One step is one moe_forward call (route, slot map, permute, grouped GEMM 1
with SwiGLU, grouped GEMM 2, combine) over the whole synthetic batch, inputs
and weights resident in HBM. The default workload is the redundant-slot
layer (T=16384, H=4096, I=1024, 64 experts in 80 slots, top-8, Zipf(1.2)
expert popularity), the largest of the layer shapes. Prints one JSON line.

Timing: HIP events on the stream the kernels run on (torch's current
stream), recorded by moe_forward itself at every stage boundary of every
timed step; ms_per_step is the device time from the first to the last event.
The dominant kernel (grouped GEMM 1) is timed by the events around it.

--copy-probe runs only a plain device copy of a known size (for scaling the
HBM byte counters of a profiler run) and exits.

On bf16 workloads the line also carries `dense_reference`, one dense bf16
GEMM of the gate/up product's FLOPs through torch.matmul, timed after the
steps for context (--no-dense-reference skips it). On bf16 and FP8 workloads
it carries `mfma_ceiling`: the sustained bf16 and FP8 MFMA rates of the chip
measured just before (moe_expert_dispatch_amd/probe/mfma_ceiling, a separate
process), with the MFMAs alone and with the operand movement of the GEMM's
K-loop; the chip lowers its clock under load, so the peak figures are not
reached by either (--no-mfma-ceiling skips it).
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

METRIC = "fused-MoE layer tokens/sec; grouped-GEMM TFLOP/s as % of bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PEAK_F32_TFLOPS = 157.3  # MI355X fp32 vector (FMA) peak
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
TRAFFIC_DIR = os.path.join(ROOT, "profiles")  # <workload>_gate_up_traffic.json
# the GEMM kernels and the item order they share
GEMM_SRC = [os.path.join(ROOT, "moe_expert_dispatch_amd", "csrc", f)
            for f in ("gemm_mfma.hip", "item_order.h")]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="redundant_slots_zipf")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--no-mfma-ceiling", action="store_true")
    ap.add_argument("--no-dense-reference", action="store_true")
    ap.add_argument("--a2a", action="store_true",
                    help="time the all-to-all dispatch path on an expert-parallel workload")
    ap.add_argument("--ep-rank", type=int, default=0,
                    help="expert-parallel share to time (workloads with ep_size > 1)")
    return ap.parse_args()


def copy_probe():
    import torch
    n = 1 << 30  # 1 GiB read + 1 GiB written per copy
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "launches": 5}), flush=True)


def run_a2a(args):
    """All-to-all path of an expert-parallel workload on one GPU: dispatch to
    ep_size blocks, each rank's fused forward over its block (f32 partials),
    gather-sum. Prints one JSON line (not the layer's headline metric)."""
    import torch

    import moe_expert_dispatch_amd as moe
    from workloads import CONFIGS, make_inputs

    moe.lib()
    dev = torch.device("cuda:0")
    name = args.workload if CONFIGS[args.workload].ep_size > 1 else "ep_share_256_bf16"
    cfg = CONFIGS[name]
    R, T, El = cfg.ep_size, cfg.T, cfg.E_local
    inp = make_inputs(cfg)
    x = inp.x.to(dev)
    ids, w = moe.route(inp.logits.to(dev), cfg.K, cfg.renormalize)
    wgu = [inp.w_gate_up[r * El:(r + 1) * El].contiguous().to(dev) for r in range(R)]
    wd = [inp.w_down[r * El:(r + 1) * El].contiguous().to(dev) for r in range(R)]
    fc = [moe.ForwardConfig(T=T, H=cfg.H, I=cfg.I, E_global=cfg.E, K=cfg.K, renormalize=False,
                            S=El, dtype=torch.bfloat16, out_dtype=torch.float32, ep_size=R,
                            ep_rank=r) for r in range(R)]
    fws = torch.empty(moe.forward_workspace_size(fc[0]), dtype=torch.uint8, device=dev)
    dws = torch.empty(max(moe.a2a_dispatch_workspace_size(T, R, T), 1), dtype=torch.uint8,
                      device=dev)
    partial = torch.empty(R * T, cfg.H, dtype=torch.float32, device=dev)
    state = {}

    def dispatch():
        state["d"] = moe.a2a_dispatch(x, ids, w, cfg.E, R, T, ws=dws)

    def experts():
        _, _, _, sx, sids, sw = state["d"]
        for r in range(R):
            blk = slice(r * T, (r + 1) * T)
            moe.forward(fc[r], sx[blk], wgu[r], wd[r], topk_ids=sids[blk], topk_w=sw[blk],
                        out=partial[blk], ws=fws)

    def gather():
        state["out"] = moe.a2a_combine(partial, state["d"][1], out_dtype=torch.bfloat16)

    for _ in range(args.warmup):
        dispatch(); experts(); gather()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for e in ev:
        e[0].record(); dispatch(); e[1].record(); experts(); e[2].record(); gather(); e[3].record()
    torch.cuda.synchronize()
    t_d = sum(e[0].elapsed_time(e[1]) for e in ev) / args.steps
    t_x = sum(e[1].elapsed_time(e[2]) for e in ev) / args.steps
    t_g = sum(e[2].elapsed_time(e[3]) for e in ev) / args.steps
    sent = int((state["d"][1] >= 0).sum().item())  # (token, rank) messages
    eb = 2
    # dispatch: read each token row and its routing once, write one row per
    # message, the routing of every send row (ids, weights, token) and the
    # token positions
    d_bytes = (T * cfg.H * eb + sent * cfg.H * eb + T * cfg.K * 8 + R * T * (cfg.K * 8 + 4)
               + T * R * 4)
    g_bytes = sent * cfg.H * 4 + T * cfg.H * eb + T * R * 4
    step = t_d + t_x + t_g
    res = {"metric": "all-to-all expert-parallel layer tokens/sec (dispatch, per-rank experts, "
                     "gather-sum; one GPU)",
           "value": T / (step * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": step, "higher_is_better": True,
           "dtype": "bf16", "data": "synthetic",
           "config": {"workload": name, "tokens": T, "hidden": cfg.H, "experts": cfg.E,
                      "top_k": cfg.K, "ranks": R, "messages": sent},
           "stage_ms": {"dispatch": t_d, "rank_forwards": t_x, "gather_sum": t_g},
           "dispatch_gbps": d_bytes / (t_d * 1e6), "gather_sum_gbps": g_bytes / (t_g * 1e6),
           "dispatch_frac_of_hbm": d_bytes / (t_d * 1e6) / PEAK_HBM_GBPS,
           "gather_sum_frac_of_hbm": g_bytes / (t_g * 1e6) / PEAK_HBM_GBPS}
    print(json.dumps(res), flush=True)


def mfma_ceiling():
    """Runs the MFMA ceiling program as a child process (before this process
    touches the GPU) and returns its two rates, or a reason it could not."""
    import subprocess
    prog = os.path.join(ROOT, "moe_expert_dispatch_amd", "probe", "mfma_ceiling")
    if not os.path.exists(prog):
        return {"error": "program not built"}
    try:
        res = subprocess.run([prog], capture_output=True, text=True, timeout=120)
    except subprocess.TimeoutExpired:
        return {"error": "timed out"}
    if res.returncode != 0:
        return {"error": f"exit status {res.returncode}: {res.stderr.strip()[-200:]}"}
    rates = {}
    for line in res.stdout.splitlines():
        rec = json.loads(line)
        rates[rec["mode"] + "_tflops"] = rec["tflops"]
    rates["program"] = "moe_expert_dispatch_amd/probe/mfma_ceiling"
    return rates


def ceiling_with_frac(ceiling, gu_tflops, fp8):
    """The ceiling program's rates plus the gate/up GEMM's rate as a fraction
    of the operand-movement rate of its own precision."""
    key = "fp8_operand_movement_tflops" if fp8 else "operand_movement_tflops"
    if not ceiling or key not in ceiling:
        return ceiling
    return dict(ceiling, gate_up_frac_of_operand_movement=gu_tflops / ceiling[key])


def kernel_source_digest(paths):
    """SHA-256 of source files with their comments and whitespace removed: it
    changes when the code does, not when a comment does."""
    import re
    src = ""
    for path in paths:
        with open(path) as f:
            src += f.read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    return hashlib.sha256(re.sub(r"\s+", "", src).encode()).hexdigest()


def gemm_traffic(workload):
    """HBM traffic of grouped GEMM 1 from the committed profiler summary, or
    None if the kernel source changed since the counters were taken or they
    were taken on another workload."""
    try:
        with open(os.path.join(TRAFFIC_DIR, f"{workload}_gate_up_traffic.json")) as f:
            rec = json.load(f)
        sha = kernel_source_digest(GEMM_SRC)
        if rec.get("kernel_source_sha256") != sha or rec.get("workload") != workload:
            return None
        return rec.get("bytes_per_launch")
    except (OSError, ValueError):
        return None


def staged_permute_ms(moe, x, slot, mask, S, reps=10):
    """Device time of one moe_permute call with its row gather (x_perm
    written), averaged over `reps` calls on the current stream."""
    import torch
    T, K = slot.shape
    ws = torch.empty(max(moe.permute_workspace_size(T, K, S), 1), dtype=torch.uint8,
                     device=x.device)
    for _ in range(2):
        moe.permute(x, slot, mask, S, ws=ws)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        moe.permute(x, slot, mask, S, ws=ws)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def dense_reference(M, K, N, reps=10):
    """A library rate for context: one dense bf16 GEMM [M, K] x [K, N] of the
    gate/up product's FLOPs through torch.matmul (the BLAS library torch
    selects, named in the result), timed with events outside the timed
    steps. Not part of the path."""
    import torch
    g = torch.Generator(device="cuda").manual_seed(0)
    a = torch.randn(M, K, device="cuda", dtype=torch.bfloat16, generator=g)
    b = torch.randn(K, N, device="cuda", dtype=torch.bfloat16, generator=g)
    c = torch.empty(M, N, device="cuda", dtype=torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b, out=c)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch.matmul(a, b, out=c)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b, c
    torch.cuda.empty_cache()
    lib = str(torch.backends.cuda.preferred_blas_library()).split(".")[-1]
    if torch.version.hip:  # torch keeps the CUDA names for the ROCm libraries
        lib = {"Cublaslt": "hipBLASLt", "Cublas": "rocBLAS", "Ck": "composable_kernel"}.get(lib, lib)
    return {"library": f"torch.matmul bf16 ({lib})", "shape_mkn": [M, K, N], "ms": ms,
            "tflops": 2.0 * M * K * N / (ms * 1e9)}


def cpu_baseline(inp, seconds, rank=0):
    """The oracle, as it stands, on a bounded sample of the same workload."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle
    cfg = inp.cfg
    blas_threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    block = 64
    done = 0
    t0 = time.perf_counter()
    while True:
        tok = np.arange(done, min(done + block, cfg.T))
        if cfg.dtype == "fp8":
            oracle.fp8_forward(inp.x, inp.logits, inp.w_gate_up.numpy(), inp.w_gate_up_scale,
                               inp.w_down.numpy(), inp.w_down_scale, cfg.a1_scale, cfg.a2_scale,
                               cfg.K, cfg.renormalize, cfg.ep_size, rank, tokens=tok)
        elif cfg.num_expert_group:
            ids, w = oracle.route_grouped(inp.logits.numpy()[tok], cfg.K, cfg.renormalize,
                                          cfg.num_expert_group, cfg.topk_group)
            oracle.forward(inp.x[tok], None, inp.w_gate_up, inp.w_down, cfg.K, False,
                           cfg.ep_size, rank, topk=(ids, w))
        else:
            oracle.forward(inp.x, inp.logits, inp.w_gate_up, inp.w_down, cfg.K,
                           cfg.renormalize, cfg.ep_size, rank, tokens=tok,
                           routing_on_input=cfg.routing_on_input,
                           shared=np.zeros((cfg.T, cfg.H)) if cfg.shared_expert else None)
        done += tok.size
        el = time.perf_counter() - t0
        if el >= seconds or done >= cfg.T:
            break
    host_cores = os.cpu_count() or 1
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = host_cores
    # `cores` is the thread count the oracle ran with: numpy's BLAS threads
    # (its matmuls); everything else in it is single-threaded numpy
    return {"value": done / el, "unit": "tokens/s", "cores": int(blas_threads), "kind": "oracle",
            "host_cores": int(host_cores), "cores_usable": int(usable),
            "sample": (f"first {done} of {cfg.T} tokens of the same workload through the fp64 "
                       f"numpy oracle (route, EP mask / slot map, per-expert SwiGLU MLP, "
                       f"combine), {el:.1f} s wall; {int(blas_threads)} BLAS threads on a host "
                       f"with {host_cores} logical cores ({usable} usable by this process)")}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(expert-parallel shares run in sequence on one device); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import moe_expert_dispatch_amd as moe
    from workloads import CONFIGS, build_slot_table, identity_slot_table, make_inputs, slot_weights

    if args.copy_probe:
        copy_probe()
        return
    if args.a2a:
        run_a2a(args)
        return
    cfg = CONFIGS[args.workload]
    ceiling = None
    if cfg.dtype in ("bf16", "fp8") and not args.no_mfma_ceiling:
        ceiling = mfma_ceiling()
    moe.lib()
    dev = torch.device("cuda:0")
    rank = args.ep_rank
    if not 0 <= rank < cfg.ep_size:
        print(f"--ep-rank must be in [0, {cfg.ep_size}) for {cfg.name}", file=sys.stderr)
        sys.exit(2)
    fp8 = cfg.dtype == "fp8"
    tdt = torch.bfloat16 if cfg.dtype in ("bf16", "fp8") else torch.float32  # x and out
    t_gen = time.perf_counter()
    inp = make_inputs(cfg)
    wgu_h, wd_h = inp.share_weights(rank)
    sgu_h, sd_h = inp.share_scales(rank) if fp8 else (None, None)
    if cfg.n_replicated:
        ro, rs, se = build_slot_table(cfg.E_local, inp.replicated_experts())
        wgu_h, wd_h = slot_weights(wgu_h, se), slot_weights(wd_h, se)
        if fp8:
            sgu_h, sd_h = slot_weights(sgu_h, se), slot_weights(sd_h, se)
        S = int(se.numel())
    else:
        ro, rs = identity_slot_table(cfg.E_local)
        S = cfg.E_local
    wgu, wd = wgu_h.contiguous().to(dev), wd_h.contiguous().to(dev)
    sgu = sgu_h.contiguous().to(dev) if fp8 else None
    sd = sd_h.contiguous().to(dev) if fp8 else None
    x = inp.x.to(dev)
    logits = inp.logits.to(dev)
    ro, rs = ro.to(dev), rs.to(dev)
    gen_s = time.perf_counter() - t_gen

    fc = moe.ForwardConfig(T=cfg.T, H=cfg.H, I=cfg.I, E_global=cfg.E, K=cfg.K,
                           renormalize=cfg.renormalize, S=S, dtype=moe.FP8 if fp8 else tdt,
                           out_dtype=tdt, ep_size=cfg.ep_size,
                           ep_rank=rank, num_expert_group=cfg.num_expert_group,
                           topk_group=cfg.topk_group, routing_on_input=cfg.routing_on_input,
                           a1_scale=cfg.a1_scale, a2_scale=cfg.a2_scale)
    shared = None
    if cfg.shared_expert:  # stands for the shared expert's output (not computed here)
        shared = torch.randn(cfg.T, cfg.H, generator=torch.Generator().manual_seed(1)).to(
            tdt).to(dev)
    ws = torch.empty(moe.forward_workspace_size(fc), dtype=torch.uint8, device=dev)
    out = torch.empty(cfg.T, cfg.H, dtype=tdt, device=dev)

    # included pairs of this batch (all pairs when ep_size == 1)
    ids, w = moe.route(logits, cfg.K, cfg.renormalize, num_groups=cfg.num_expert_group,
                       topk_groups=cfg.topk_group)
    slot, wm, mask = moe.slot_map(ids, w, cfg.E, cfg.ep_size, rank, ro, rs)
    P_in = int(mask.sum().item())

    def step(events=None):
        moe.forward(fc, x, wgu, wd, logits=logits, rep_off=ro, rep_slots=rs, out=out, ws=ws,
                    events=events, shared_out=shared, w_gate_up_scale=sgu, w_down_scale=sd)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # one set of stage events per timed step (created by a first record)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(moe.NUM_EVENTS)]
           for _ in range(args.steps)]
    for row in ev:
        for e in row:
            e.record()
    torch.cuda.synchronize()

    t0 = time.perf_counter()
    for i in range(args.steps):
        step([e.cuda_event for e in ev[i]])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    names = ["route_slot_map", "permute", "gemm_gate_up", "gemm_down", "combine"]
    stage_ms = {n: 0.0 for n in names}
    for row in ev:
        for j, n in enumerate(names):
            stage_ms[n] += row[j].elapsed_time(row[j + 1]) / args.steps
    ms_per_step = ev[0][0].elapsed_time(ev[-1][-1]) / args.steps

    eb = {"bf16": 2, "fp8": 2, "f32": 4}[cfg.dtype]  # x, Y and out element bytes
    wb = 1 if fp8 else eb                             # weight and A element bytes
    fl_gu = 4.0 * cfg.H * cfg.I * P_in       # gate and up products
    fl_dn = 2.0 * cfg.H * cfg.I * P_in
    gemm_tflops = (fl_gu + fl_dn) / ((stage_ms["gemm_gate_up"] + stage_ms["gemm_down"]) * 1e9)
    gu_tflops = fl_gu / (stage_ms["gemm_gate_up"] * 1e9)
    P = cfg.T * cfg.K
    # Permutation: count and scatter each read slot + mask (5 B per pair), the
    # scatter writes pair_row (4 B per pair) and sorted_pairs (4 B per included
    # pair). For bf16 with H a multiple of 64 (>= 128) the row gather is folded
    # into the gate/up GEMM; otherwise permute also copies the rows.
    fused_gather = fp8 or (cfg.dtype == "bf16" and cfg.H % 64 == 0 and cfg.H >= 128
                           and cfg.T * cfg.H * 2 < 2 ** 31 and not cfg.routing_on_input)
    permute_bytes = 2 * 5 * P + 4 * P + 4 * P_in
    if not fused_gather:
        permute_bytes += cfg.T * cfg.H * eb + P_in * cfg.H * eb
    if fp8:  # the permute stage also quantizes x (read bf16, write codes)
        permute_bytes += cfg.T * cfg.H * (2 + 1)
    combine_bytes = P_in * cfg.H * eb + 8 * P + cfg.T * cfg.H * eb
    if cfg.shared_expert:
        combine_bytes += cfg.T * cfg.H * eb
    # GEMM floor: the larger of the compute time at peak and the time to stream
    # every slot's weights plus the activations (x or x_perm read, A written and
    # read, Y written) at HBM peak.
    peak_tf = {"bf16": PEAK_BF16_TFLOPS, "fp8": PEAK_FP8_TFLOPS, "f32": PEAK_F32_TFLOPS}[cfg.dtype]
    gemm_bytes = (S * 3 * cfg.H * cfg.I * wb
                  + (cfg.T if fused_gather else P_in) * cfg.H * wb
                  + 2 * P_in * cfg.I * wb + P_in * cfg.H * eb)
    gemm_floor_ms = max((fl_gu + fl_dn) / (peak_tf * 1e9), gemm_bytes / (PEAK_HBM_GBPS * 1e6))
    gemm_ms = stage_ms["gemm_gate_up"] + stage_ms["gemm_down"]
    traffic = gemm_traffic(cfg.name) if cfg.dtype in ("bf16", "fp8") else None

    # The standalone permutation with its row gather, timed after (not inside)
    # the steps: moe_forward folds the gather into the gate/up GEMM, so this is
    # where the permutation's HBM rate is measured.
    sp_ms = staged_permute_ms(moe, x, slot, mask, S)
    dense = None
    if cfg.dtype == "bf16" and not args.no_dense_reference:
        # the gate/up product's FLOPs as one dense GEMM: [P_in, H] x [H, 2I]
        dense = dense_reference(P_in, cfg.H, 2 * cfg.I)
        dense["gate_up_vs_dense"] = gu_tflops / dense["tflops"]
    xb = x.element_size()
    sp_bytes = 2 * 5 * P + 4 * P + 4 * P_in + cfg.T * cfg.H * xb + P_in * cfg.H * xb

    res = {
        "metric": METRIC,
        "value": cfg.T / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "fp8": "fp8_e4m3", "f32": "f32"}[cfg.dtype],
        "data": "synthetic",
        "config": {"workload": cfg.name, "tokens": cfg.T, "hidden": cfg.H,
                   "intermediate": cfg.I, "experts": cfg.E, "slots": S, "top_k": cfg.K,
                   "renormalize": cfg.renormalize, "ep_size": cfg.ep_size, "ep_rank": rank,
                   "included_pairs": P_in, "parallelism": "single GPU"},
        "roofline": ({"bound": "mfma", "kernel": "grouped_gemm_dma_kernel bf16 gate/up + SwiGLU",
                      "achieved": gu_tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                      "frac": gu_tflops / PEAK_BF16_TFLOPS, "traffic": traffic}
                     if cfg.dtype == "bf16" else
                     {"bound": "mfma", "kernel": "grouped_gemm_dma_kernel FP8 (E4M3) gate/up + SwiGLU",
                      "achieved": gu_tflops, "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                      "frac": gu_tflops / PEAK_FP8_TFLOPS, "traffic": traffic}
                     if fp8 else
                     {"bound": "alu", "kernel": "grouped_gemm_f32 gate/up + SwiGLU (FMA)",
                      "achieved": gu_tflops, "peak": PEAK_F32_TFLOPS, "unit": "TFLOP/s",
                      "frac": gu_tflops / PEAK_F32_TFLOPS, "traffic": None}),
        "mfma_ceiling": ceiling_with_frac(ceiling, gu_tflops, fp8),
        "dense_reference": dense,
        "grouped_gemm_tflops": gemm_tflops,
        "grouped_gemm_frac_of_bf16_peak": gemm_tflops / PEAK_BF16_TFLOPS,
        "grouped_gemm_frac_of_peak": gemm_tflops / peak_tf,
        "grouped_gemm_floor_ms": gemm_floor_ms,
        "grouped_gemm_frac_of_roofline": gemm_floor_ms / gemm_ms,
        "stage_ms": stage_ms,
        "permute_gbps": permute_bytes / (stage_ms["permute"] * 1e6),
        "permute_stage_moves": ("indices only (row gather folded into the gate/up GEMM)"
                                if fused_gather and not fp8 else
                                "indices and quantized x" if fp8 else "indices and rows"),
        "staged_permute": {"call": "moe_permute with its row gather, outside the timed steps",
                           "ms": sp_ms, "bytes": sp_bytes,
                           "gbps": sp_bytes / (sp_ms * 1e6),
                           "frac_of_hbm": sp_bytes / (sp_ms * 1e6) / PEAK_HBM_GBPS},
        "combine_frac_of_hbm": combine_bytes / (stage_ms["combine"] * 1e6) / PEAK_HBM_GBPS,
        "combine_gbps": combine_bytes / (stage_ms["combine"] * 1e6),
        "host_wall_ms_per_step": wall * 1e3 / args.steps,
        "input_generation_s": gen_s,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds, rank)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
