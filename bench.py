"""Benchmark of the routed-expert layer (forward + backward) on one MI355X.

A step is one pass of the whole layer over one batch of synthetic input:
  route (top-k + softmax) -> permute -> gate/up GEMM + SiTU-GLU -> down GEMM + combine
  -> backward (dA GEMM + SiTU-GLU' + dp partials, dW_down, dW_gu, dX + combine, dp).
`value` is the layer's useful GEMM throughput, 18 R d H FLOP per step over the measured step
time (TFLOP/s), on the large-context workload (98304 tokens dispatched to 28 local experts,
top-16: R = 1,572,864 routed rows), the largest that fits one GPU. HIP events on the
library's stream bracket every stage of every timed step; `roofline` is the stage that is one
kernel and takes the longest. The JSON line also carries the one-rank shard workload as a
secondary key, the standalone streaming SiTU-GLU rate on its own workload, the MXFP8-store
and W4A8 variants, peak HBM against the naive six-fp32-copies footprint, and the fp64 CPU
oracle's rate on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload large|shard|skew|tiny]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE expert fwd+bwd TFLOP/s (% bf16 MFMA peak); SiTU-GLU GB/s (% HBM)"
PROFILES = os.path.join(ROOT, "profiles")
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA (the W4A8 MFMA takes an fp8 operand)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E

# The stages of one step, in launch order: (name, kernels in it, FLOP per launch as a multiple
# of R d H). Stages that are one kernel can carry the roofline.
STAGES = [("route_permute", "route + permute count/scan/scatter", 0.0),
          ("gate_up", "gate/up GEMM + SiTU-GLU epilogue", 4.0),
          ("down_combine", "down GEMM + combine", 2.0),
          ("dA", "dA GEMM + SiTU-GLU' + dp partials", 2.0),
          ("dW_down", "dW_down GEMM (fp32)", 2.0),
          ("dW_gu", "dW_gu GEMM (fp32)", 4.0),
          ("dX_combine", "dX GEMM + combine", 4.0),
          ("dp", "dp row reduce + scatter", 0.0)]
SINGLE_KERNEL = ("gate_up", "dA", "dW_down", "dW_gu")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="large")
    ap.add_argument("--secondary", default="shard",
                    help="second layer workload reported as an extra key ('none' to skip)")
    ap.add_argument("--bwd-passes", type=int, default=0,
                    help="column windows of the backward's dX combine (0: LayerBuffers' "
                         "default, the fewest that keep the backward within the forward's "
                         "memory when that saves 1 GiB or more)")
    ap.add_argument("--combine-passes", type=int, default=1,
                    help="passes over the output columns per combine (less fp32 row memory)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-situ", action="store_true")
    ap.add_argument("--no-variants", action="store_true", help="skip the MXFP8-store and W4A8 legs")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run 3 plain 1 GiB device copies (counter calibration)")
    ap.add_argument("--print-digest", action="store_true",
                    help="print the digest of the kernel sources and exit")
    ap.add_argument("--blas-reference", action="store_true",
                    help="only time torch's bf16 GEMMs (hipBLASLt) on the layer's shapes, as context")
    ap.add_argument("--blas-rows", type=int, default=16456,
                    help="routed rows R for --blas-reference (16456: the shard workload; "
                         "1572864: the large-context workload)")
    return ap.parse_args()


def kernel_source_digest():
    """sha256 over the HIP sources and the build flags of the library."""
    import hashlib
    pkg = os.path.join(ROOT, "sparse_moe_expert_top_amd")
    h = hashlib.sha256()
    files = [os.path.join(pkg, "csrc", f) for f in sorted(os.listdir(os.path.join(pkg, "csrc")))]
    for f in files + [os.path.join(pkg, "build.py")]:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def committed_traffic(workload, stage):
    """HBM bytes per launch of a stage's kernel from the committed counter summary
    profiles/<stage>_<workload>_counters.md, or None when it is missing or was taken on other
    kernel sources (its source_sha256 must match the current digest)."""
    path = os.path.join(PROFILES, f"{stage}_{workload}_counters.md")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith(("#", "|", " ", "`")):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != kernel_source_digest():
        return None
    try:
        return {"fetch": float(kv["fetch_bytes_per_launch"]),
                "write": float(kv["write_bytes_per_launch"])}
    except (KeyError, ValueError):
        return None


def calibrate_copy():
    """Three plain device copies of 1 GiB: FETCH_SIZE / WRITE_SIZE of these dispatches give
    the counters' scale (bytes per counted KiB)."""
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_read": n, "bytes_written": n,
                      "dispatches": 3}), flush=True)


def blas_reference(cfg, R):
    """torch's bf16 GEMMs (hipBLASLt) on dense and per-expert batched forms of the layer's
    contractions with R rows spread evenly over the experts; contiguous operands. Context for
    the grouped kernels' TFLOP/s, not part of the path."""
    import torch
    dev = "cuda"
    d, H, E = cfg.d, cfg.H, cfg.E_loc
    Re = R // E
    g = torch.Generator(device=dev).manual_seed(0)
    rnd = lambda *sh: torch.randn(*sh, device=dev, dtype=torch.bfloat16, generator=g)
    a, w = rnd(R, d), rnd(d, 2 * H)
    ab, wb = rnd(E, Re, d), rnd(E, d, 2 * H)
    ah, wd = rnd(E, Re, H), rnd(E, H, d)
    dht, xb = rnd(E, 2 * H, Re), rnd(E, Re, d)
    sq = rnd(8192, 8192), rnd(8192, 8192)
    cases = [("dense gate/up-sized [R,d]x[d,2H]", lambda: a @ w, 4.0 * R * d * H),
             ("batched gate/up [E,R/E,d]x[E,d,2H]", lambda: torch.bmm(ab, wb), 4.0 * E * Re * d * H),
             ("batched down [E,R/E,H]x[E,H,d]", lambda: torch.bmm(ah, wd), 2.0 * E * Re * d * H),
             ("batched dW_gu [E,2H,R/E]x[E,R/E,d], bf16 out", lambda: torch.bmm(dht, xb), 4.0 * E * Re * d * H),
             ("dense 8192^3", lambda: sq[0] @ sq[1], 2.0 * 8192 ** 3)]
    out = {}
    for name, fn, flop in cases:
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(20):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 20
        out[name] = {"ms": round(ms, 4), "TFLOP/s": round(flop / (ms * 1e-3) / 1e12, 1)}
    print(json.dumps({"blas_reference": out, "rows_per_expert": Re}))


def bf16_dev(u16, torch):
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).cuda().view(torch.bfloat16)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def cpu_baseline(cfg, inp, target_s):
    """Time the fp64 oracle (as it stands) on a row sample of one expert of the same input:
    the first n routed rows of local expert 0, run as a layer of those n tokens with that one
    expert (its rows are independent of the rest). n is sized from a warm timing so the run
    takes about target_s seconds."""
    import oracle
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        pools = [p for p in threadpool_info() if p.get("user_api") == "blas"] or threadpool_info()
        threads = max((p.get("num_threads", 1) for p in pools), default=1)
        blas = ",".join(sorted({f"{p.get('internal_api', '?')} {p.get('version', '')}".strip()
                                for p in pools})) or blas
    except Exception:                                     # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    idx, gates = oracle.route_topk(inp["logits"], cfg.k)
    perm = oracle.permute(idx, gates, cfg.e_lo, cfg.E_loc)
    off = perm["offsets"]
    e0 = int(np.argmax(np.diff(off) > 0))                 # first local expert with rows
    r0, n_e = int(off[e0]), int(off[e0 + 1] - off[e0])

    def sub(n):
        rows = r0 + np.arange(n)
        tok = perm["row_token"][rows]
        slot = np.full((n, cfg.k), -1, np.int32)
        slot[np.arange(n), np.argmax(idx[tok] == cfg.e_lo + e0, axis=1)] = np.arange(n)
        p = dict(offsets=np.array([0, n], np.int32), row_token=np.arange(n, dtype=np.int32),
                 row_gate=perm["row_gate"][rows], slot_row=slot, R=n)
        return p, inp["x"][tok], inp["dy"][tok]

    w_gu, w_down = inp["w_gu"][e0:e0 + 1], inp["w_down"][e0:e0 + 1]

    def run(n):
        p, x, dy = sub(n)
        t0 = time.perf_counter()
        oracle.expert_layer_fwd(x, w_gu, w_down, p, cfg.H, mode="S", keep=False)
        oracle.expert_layer_bwd(x, dy, w_gu, w_down, p, cfg.H, mode="S")
        return time.perf_counter() - t0

    n0 = min(1024, n_e)
    run(n0)                                   # first call pays thread-pool and page-in start-up
    t1 = run(n0)
    n = int(max(n0, min(n_e, n0 * target_s / max(t1, 1e-3))))
    dt = run(n)
    flop = 18.0 * n * cfg.d * cfg.H
    return dict(value=flop / dt / 1e12, unit="TFLOP/s", cores=int(threads), kind="oracle",
                host_cpus=len(os.sched_getaffinity(0)), blas=blas,
                sample=f"fp64 oracle forward+backward of the first {n} routed rows of local "
                       f"expert {e0} (of {n_e}; {perm['R']} rows in all) of the same input, as "
                       f"a layer of those {n} tokens; {dt:.1f} s",
                seconds=round(dt, 2))


def streaming_leg(moe, cfg, t, R, torch, iters=20, warmup=3):
    """Route and permute of the workload, each timed alone with HIP events (median of
    `iters` after `warmup`), the Infinity Cache flushed by a 1 GiB write before each launch.
    Algorithmic bytes: route 4TE + 8Tk (logits in; indices and gates out), permute
    12R + 12Tk (indices and gates in; slot map, row token, gate out; offsets aside)."""
    stream = torch.cuda.current_stream()
    T, E, k = cfg.T, cfg.E, cfg.k
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    gates = torch.empty((T, k), dtype=torch.float32, device="cuda")
    perm = dict(offsets=torch.empty(cfg.E_loc + 1, dtype=torch.int32, device="cuda"),
                row_token=torch.empty(max(R, 1), dtype=torch.int32, device="cuda"),
                row_gate=torch.empty(max(R, 1), dtype=torch.float32, device="cuda"),
                slot_row=torch.empty((T, k), dtype=torch.int32, device="cuda"),
                status=torch.empty(1, dtype=torch.int32, device="cuda"))
    ws = torch.empty(max(moe.workspace_size(moe.MOE_WS_PERMUTE, T=T, E_loc=cfg.E_loc), 256),
                     dtype=torch.uint8, device="cuda")
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    ops = {"route": lambda: moe.moe_route_topk(t["logits"], k, topk_idx=idx, gates=gates),
           "permute": lambda: moe.moe_permute(idx, gates, cfg.e_lo, cfg.E_loc, R, out=perm, ws=ws)}
    by = {"route": 4.0 * T * E + 8.0 * T * k, "permute": 12.0 * R + 12.0 * T * k}
    out = {}
    for name, fn in ops.items():
        ms = []
        for i in range(warmup + iters):
            flush.zero_()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            if i >= warmup:
                ms.append(e0.elapsed_time(e1))
        m = float(np.median(ms))
        out[name] = {"us": round(m * 1e3, 1), "algorithmic_bytes": by[name],
                     "GB/s": round(by[name] / (m * 1e-3) / 1e9, 1),
                     "frac_hbm": round(by[name] / (m * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    assert int(perm["offsets"][-1].item()) == R
    del flush, idx, gates, perm, ws
    torch.cuda.empty_cache()
    return out


def load_workload(cfg, torch):
    from moe_inputs import layer_inputs
    log(f"generating inputs for {cfg.name}")
    inp = layer_inputs(cfg, seed=0)
    t = dict(x=bf16_dev(inp["x"], torch), dy=bf16_dev(inp["dy"], torch),
             w_gu=bf16_dev(inp["w_gu"], torch), w_down=bf16_dev(inp["w_down"], torch),
             logits=torch.from_numpy(inp["logits"]).cuda())
    return inp, t


def timed_steps(moe, buf, t, steps, warmup, torch):
    """W warm-up steps, then `steps` timed steps with HIP events between the stages, on the
    stream the library launches on. Returns (ms per step from the host clock around the
    synchronized loop, mean ms per stage)."""
    stream = torch.cuda.current_stream()
    bwd = [moe.MOE_BWD_DA, moe.MOE_BWD_DW_DOWN, moe.MOE_BWD_DW_GU, moe.MOE_BWD_DX, moe.MOE_BWD_DP]

    def step(ev):
        ev[0].record(stream)
        buf.route(t["logits"])
        ev[1].record(stream)
        buf.gate_up(t["x"], t["w_gu"])
        ev[2].record(stream)
        buf.down_combine(t["w_down"])
        ev[3].record(stream)
        for i, st in enumerate(bwd):
            buf.backward(t["dy"], t["x"], t["w_gu"], t["w_down"], stages=st)
            ev[4 + i].record(stream)

    mk = lambda: [torch.cuda.Event(enable_timing=True) for _ in range(len(STAGES) + 1)]
    for _ in range(warmup):
        step(mk())
    torch.cuda.synchronize()
    evs = [mk() for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / steps
    stage_ms = {name: float(np.mean([ev[j].elapsed_time(ev[j + 1]) for ev in evs]))
                for j, (name, _, _) in enumerate(STAGES)}
    return ms_step, stage_ms


def layer_leg(moe, cfg, t, steps, warmup, passes, torch, h_store="bf16", bwd_passes=0):
    shape = moe.LayerShape(T=cfg.T, E=cfg.E, k=cfg.k, e_lo=cfg.e_lo, E_loc=cfg.E_loc, d=cfg.d,
                           H=cfg.H, beta=cfg.beta, linear_beta=cfg.linear_beta)
    R = moe.LayerBuffers.routed_rows(shape, t["logits"])
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    buf = moe.LayerBuffers(shape, R_cap=R, h_store=h_store, combine_passes=passes,
                           bwd_passes=bwd_passes or None)
    ms_step, stage_ms = timed_steps(moe, buf, t, steps, warmup, torch)
    assert buf.rows() == R and not buf.overflowed()
    peak = torch.cuda.max_memory_allocated() / 1e9
    layer_leg.bwd_passes = buf.bwd_passes
    del buf
    torch.cuda.empty_cache()
    return R, ms_step, stage_ms, peak


def stage_report(stage_ms, R, cfg):
    rdh = float(R) * cfg.d * cfg.H
    out = {}
    for name, what, mult in STAGES:
        ms = stage_ms[name]
        e = {"ms": round(ms, 4), "kernels": what}
        if mult:
            e["TFLOP/s"] = round(mult * rdh / (ms * 1e-3) / 1e12, 1)
        out[name] = e
    return out


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU (asked for --gpus {args.gpus}, WORLD_SIZE "
              f"{world}); this layer is measured on one GPU's share of experts", file=sys.stderr)
        sys.exit(2)
    if args.print_digest:
        print(kernel_source_digest())
        return
    if args.calibrate_copy:
        calibrate_copy()
        return

    import torch
    import sparse_moe_expert_top_amd as moe
    from moe_inputs import LAYER_CONFIGS, SITU_CONFIGS, situ_inputs

    torch.cuda.set_device(0)
    cfg = LAYER_CONFIGS[args.workload]
    if args.blas_reference:
        blas_reference(cfg, args.blas_rows)
        return
    inp, t = load_workload(cfg, torch)
    input_gb = sum(v.numel() * v.element_size() for v in t.values()) / 1e9

    log(f"{cfg.name}: {args.warmup} warm-up + {args.steps} timed steps")
    R, ms_step, stage_ms, peak_gb = layer_leg(moe, cfg, t, args.steps, args.warmup,
                                              args.combine_passes, torch,
                                              bwd_passes=args.bwd_passes)
    bwd_passes = layer_leg.bwd_passes
    log(f"{cfg.name}: route and permute alone")
    streaming = streaming_leg(moe, cfg, t, R, torch)
    rdh = float(R) * cfg.d * cfg.H
    flop_step = 18.0 * rdh
    value = flop_step / (ms_step * 1e-3) / 1e12
    stages = stage_report(stage_ms, R, cfg)
    dom = max(SINGLE_KERNEL, key=lambda n: stage_ms[n])
    dom_mult = dict((n, m) for n, _, m in STAGES)[dom]
    dom_flop = dom_mult * rdh
    dom_tf = dom_flop / (stage_ms[dom] * 1e-3) / 1e12
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {cfg.note}; T={cfg.T} d={cfg.d} H={cfg.H} "
                               f"E={cfg.E} k={cfg.k} local experts {cfg.e_lo}..{cfg.e_lo + cfg.E_loc - 1}",
                   "routed_rows": R, "flop_per_step": flop_step, "row_capacity": R,
                   "combine_passes": args.combine_passes, "bwd_combine_passes": bwd_passes},
        "mfma_frac": round(value / PEAK_BF16_TFLOPS, 4),
        "roofline": {"kernel": f"{dom}: {dict((n, w) for n, w, _ in STAGES)[dom]}",
                     "bound": "mfma", "achieved": round(dom_tf, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(dom_tf / PEAK_BF16_TFLOPS, 4),
                     "avg_launch_ms": round(stage_ms[dom], 4), "flop_per_launch": dom_flop,
                     "traffic": None},
        "stages": stages,
        "streaming": streaming,
        "peak_hbm_GB": round(peak_gb, 2),
        "inputs_and_weights_GB": round(input_gb, 2),
        "saved_activation_GB": round((R * 2 * cfg.H * 2 + cfg.T * cfg.d * 2) / 1e9, 3),
        "naive_saved_fp32_GB": round(6 * R * cfg.H * 4 / 1e9, 3),
    }
    tr = committed_traffic(cfg.name, dom)
    if tr is not None:
        # algorithmic bytes of the weight-gradient and row GEMMs: each operand once, output once
        alg = {"gate_up": 2.0 * (cfg.E_loc * 2 * cfg.H * cfg.d + R * cfg.d + R * 3 * cfg.H),
               "dA": 2.0 * (cfg.E_loc * cfg.d * cfg.H + R * cfg.d + 2 * R * 2 * cfg.H + R * cfg.H) + 4.0 * R,
               "dW_down": 2.0 * (R * cfg.d + R * cfg.H) + 4.0 * cfg.E_loc * cfg.d * cfg.H,
               "dW_gu": 2.0 * (R * 2 * cfg.H + R * cfg.d) + 4.0 * cfg.E_loc * 2 * cfg.H * cfg.d}[dom]
        out["roofline"].update(traffic=tr["fetch"] + tr["write"], traffic_fetch_bytes=tr["fetch"],
                               traffic_write_bytes=tr["write"],
                               algorithmic_bytes_per_launch=alg,
                               traffic_vs_algorithmic=round((tr["fetch"] + tr["write"]) / alg, 3))

    if not args.no_variants:
        # the same step with the saved h stored as MXFP8 (E4M3 codes + one scale byte per 32)
        log(f"{cfg.name}: MXFP8-store steps")
        n_mx = max(1, args.steps // 2)
        _, ms_mx, _, peak_mx = layer_leg(moe, cfg, t, n_mx, max(1, args.warmup // 2),
                                         args.combine_passes, torch, h_store="mxfp8",
                                         bwd_passes=args.bwd_passes)
        out["mxfp8_h"] = {"ms_per_step": round(ms_mx, 4),
                          "value": round(flop_step / (ms_mx * 1e-3) / 1e12, 2),
                          "saved_activation_GB": round((R * 2 * cfg.H * (1 + 1 / 32) + cfg.T * cfg.d * 2) / 1e9, 3),
                          "peak_hbm_GB": round(peak_mx, 2), "steps": n_mx}

        # W4A8 forward (rollouts): MXFP4 weights quantized once, x quantized to MXFP8 each step
        log(f"{cfg.name}: W4A8 forward")
        shape = moe.LayerShape(T=cfg.T, E=cfg.E, k=cfg.k, e_lo=cfg.e_lo, E_loc=cfg.E_loc,
                               d=cfg.d, H=cfg.H, beta=cfg.beta, linear_beta=cfg.linear_beta)
        w4 = moe.W4A8Weights(t["w_gu"], t["w_down"])
        b4 = moe.LayerBuffers(shape, R_cap=R)
        stream = torch.cuda.current_stream()
        for _ in range(args.warmup):
            b4.forward_w4a8(t["x"], t["logits"], w4)
        torch.cuda.synchronize()
        ev4 = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(args.steps)]
        t0 = time.perf_counter()
        for i in range(args.steps):
            b4.route(t["logits"])
            moe.moe_mxfp8_quantize(t["x"], codes=b4.x_codes, scales=b4.x_scales)
            ev4[i][0].record(stream)
            moe.moe_grouped_gemm_gate_up_w4a8(b4.x_codes, b4.x_scales, b4.perm["row_token"],
                                              b4.perm["offsets"], w4.gu_codes, w4.gu_scales,
                                              b4.R_cap, cfg.beta, cfg.linear_beta,
                                              a_codes=b4.a_codes, a_scales=b4.a_scales)
            ev4[i][1].record(stream)
            moe.moe_grouped_gemm_down_combine_w4a8(b4.a_codes, b4.a_scales, b4.perm["offsets"],
                                                   b4.perm["row_gate"], b4.perm["slot_row"],
                                                   w4.down_codes, w4.down_scales, b4.R_cap,
                                                   y=b4.y, ws=b4.ws_down)
            ev4[i][2].record(stream)
        torch.cuda.synchronize()
        ms_w4 = (time.perf_counter() - t0) * 1e3 / args.steps
        assert b4.rows() == R
        gu4_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev4]))
        dn4_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev4]))
        flop_gu = 4.0 * rdh
        out["w4a8_fwd"] = {
            "ms_per_step": round(ms_w4, 4), "value": round(6.0 * rdh / (ms_w4 * 1e-3) / 1e12, 2),
            "unit": "TFLOP/s (forward, 6 R d H)", "steps": args.steps,
            "bf16_fwd_ms": round(stage_ms["route_permute"] + stage_ms["gate_up"] + stage_ms["down_combine"], 4),
            "gate_up_ms": round(gu4_ms, 4),
            "gate_up_TFLOPs": round(flop_gu / (gu4_ms * 1e-3) / 1e12, 2),
            "gate_up_frac_fp8_peak": round(flop_gu / (gu4_ms * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4),
            "down_combine_ms": round(dn4_ms, 4),
            "weights_GB": round(cfg.E_loc * 3 * cfg.H * cfg.d * (0.5 + 1 / 32) / 1e9, 3),
            "bf16_weights_GB": round(cfg.E_loc * 3 * cfg.H * cfg.d * 2 / 1e9, 3),
        }
        del b4, w4
        torch.cuda.empty_cache()

    if not args.no_cpu_baseline:
        log("CPU oracle baseline")
        out["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_seconds)
    del inp, t
    torch.cuda.empty_cache()

    if args.secondary != "none" and args.secondary != cfg.name:
        c2 = LAYER_CONFIGS[args.secondary]
        _, t2 = load_workload(c2, torch)
        log(f"{c2.name}: {args.warmup} warm-up + {args.steps} timed steps")
        R2, ms2, st2, peak2 = layer_leg(moe, c2, t2, args.steps, args.warmup,
                                        args.combine_passes, torch, bwd_passes=args.bwd_passes)
        out[c2.name] = {"workload": f"{c2.name}: {c2.note}", "routed_rows": R2,
                        "ms_per_step": round(ms2, 4),
                        "value": round(18.0 * R2 * c2.d * c2.H / (ms2 * 1e-3) / 1e12, 2),
                        "unit": "TFLOP/s", "stages": stage_report(st2, R2, c2),
                        "peak_hbm_GB": round(peak2, 2),
                        "naive_saved_fp32_GB": round(6 * R2 * c2.H * 4 / 1e9, 3)}
        del t2
        torch.cuda.empty_cache()

    if not args.no_situ:
        sc = SITU_CONFIGS["situ"]
        Rs, Hs = sc["R"], sc["H"]
        log("SiTU-GLU streaming")
        stream = torch.cuda.current_stream()
        si = situ_inputs(Rs, Hs, seed=0, h_std=sc["h_std"])
        h, da = bf16_dev(si["h"], torch), bf16_dev(si["da"], torch)
        a = torch.empty((Rs, Hs), dtype=torch.bfloat16, device="cuda")
        dh = torch.empty_like(h)
        flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        tf, tb = [], []
        for i in range(3 + 20):
            flush.zero_()
            e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
            e0.record(stream)
            moe.situ_glu_fwd(h, a=a)
            e1.record(stream)
            moe.situ_glu_bwd(h, da, dh=dh)
            e2.record(stream)
            torch.cuda.synchronize()
            if i >= 3:
                tf.append(e0.elapsed_time(e1))
                tb.append(e1.elapsed_time(e2))
        fwd_b, bwd_b = 6.0 * Hs * Rs, 10.0 * Hs * Rs
        mf, mb = float(np.median(tf)), float(np.median(tb))
        gbs_f, gbs_b = fwd_b / mf / 1e6, bwd_b / mb / 1e6
        out["situ_glu"] = {"workload": f"h bf16 [{Rs}, {2 * Hs}] N(0,9), da bf16 [{Rs}, {Hs}]",
                           "fwd_GBs": round(gbs_f, 1), "bwd_GBs": round(gbs_b, 1),
                           "fwd_ms": round(mf, 4), "bwd_ms": round(mb, 4),
                           "GBs": round((fwd_b + bwd_b) / (mf + mb) / 1e6, 1),
                           "frac_hbm": round((fwd_b + bwd_b) / (mf + mb) / 1e6 / PEAK_HBM_GBS, 4)}
        del h, da, a, dh, flush
        torch.cuda.empty_cache()

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
