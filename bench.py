"""Benchmark of the routed-expert layer (forward + backward) on one MI355X.

A step is one pass of the whole layer over one batch of synthetic input:
  route (top-k + softmax) -> permute -> gate/up GEMM + SiTU-GLU -> down GEMM + combine
  -> backward (re-dispatch, dA GEMM + SiTU-GLU' + dp, dW_down, dW_gu, dX + combine, dp).
`value` is the layer's useful GEMM throughput, 18 R d H FLOP per step over the measured step
time (TFLOP/s); the JSON line also carries the standalone streaming SiTU-GLU rate (GB/s) on
its own workload, the roofline of the dominant kernel, and the fp64 CPU oracle's rate on a
bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload shard|large|skew|tiny]
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
# HBM counters of the gate/up GEMM on the shard workload, taken with rocprofv3 (FETCH_SIZE and
# WRITE_SIZE passes over `bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-situ`, scaled by
# the same counters over `bench.py --calibrate-copy`). They describe the kernel sources whose
# digest they record; for any other sources `traffic` is null.
COUNTERS_FILE = os.path.join(ROOT, "profiles", "gate_up_shard_counters.md")
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA (the W4A8 MFMA takes an fp8 operand)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
SHARD_ROWS = 16456             # routed local rows of the shard workload's seed-0 logits


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="shard")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-situ", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run 3 plain 1 GiB device copies (counter calibration)")
    ap.add_argument("--print-digest", action="store_true",
                    help="print the digest of the kernel sources and exit")
    ap.add_argument("--blas-reference", action="store_true",
                    help="only time torch's bf16 GEMMs (hipBLASLt) on the layer's shapes, as context")
    return ap.parse_args()


def blas_reference(cfg, R):
    """torch's bf16 GEMMs (hipBLASLt) on dense and per-expert batched forms of the layer's
    contractions with the shard workload's mean rows per expert; contiguous operands. Context
    for the grouped kernels' TFLOP/s, not part of the path."""
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


def committed_traffic(workload):
    """HBM bytes per gate/up launch from the committed counter summary, or None when the
    summary is missing, is for another workload, or was taken on other kernel sources."""
    if workload != "shard" or not os.path.exists(COUNTERS_FILE):
        return None
    kv = {}
    with open(COUNTERS_FILE) as fh:
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


def bf16_dev(u16, torch):
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).cuda().view(torch.bfloat16)


def cpu_baseline(cfg, inp, target_s):
    """Time the fp64 oracle (as it stands) on the first n local experts of the same input."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:                                     # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    idx, gates = oracle.route_topk(inp["logits"], cfg.k)
    perm = oracle.permute(idx, gates, cfg.e_lo, cfg.E_loc)

    def sub(n):
        off = perm["offsets"][: n + 1]
        R = int(off[-1])
        keep = np.zeros(perm["R"] + 1, bool)
        keep[:R] = True
        sr = np.where((perm["slot_row"] >= 0) & (perm["slot_row"] < R), perm["slot_row"], -1)
        return dict(offsets=off, row_token=perm["row_token"][:R], row_gate=perm["row_gate"][:R],
                    slot_row=sr.astype(np.int32), R=R)

    def run(n):
        p = sub(n)
        w_gu, w_down = inp["w_gu"][:n], inp["w_down"][:n]
        t0 = time.perf_counter()
        oracle.expert_layer_fwd(inp["x"], w_gu, w_down, p, cfg.H, mode="S", keep=False)
        oracle.expert_layer_bwd(inp["x"], inp["dy"], w_gu, w_down, p, cfg.H, mode="S")
        return time.perf_counter() - t0, p["R"]

    run(1)                                   # first call pays thread-pool and page-in start-up
    t1, _ = run(1)
    t2, _ = run(2)
    per = max(t2 - t1, 1e-3)                 # each call also has a fixed cost (the combine over T)
    n = int(max(1, min(cfg.E_loc, (target_s - (t1 - per)) / per)))
    dt, R = run(n)
    flop = 18.0 * R * cfg.d * cfg.H
    return dict(value=flop / dt / 1e12, unit="TFLOP/s", cores=int(threads), kind="oracle",
                sample=f"fp64 oracle forward+backward of local experts 0..{n - 1} "
                       f"({R} routed rows of {perm['R']}) of the same input; {dt:.1f} s",
                seconds=round(dt, 2))


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
    from moe_inputs import LAYER_CONFIGS, SITU_CONFIGS, layer_inputs, situ_inputs

    torch.cuda.set_device(0)
    cfg = LAYER_CONFIGS[args.workload]
    if args.blas_reference:
        blas_reference(cfg, SHARD_ROWS)
        return
    print(f"[bench] generating inputs for {cfg.name}", file=sys.stderr, flush=True)
    inp = layer_inputs(cfg, seed=0)
    x, dy = bf16_dev(inp["x"], torch), bf16_dev(inp["dy"], torch)
    w_gu, w_down = bf16_dev(inp["w_gu"], torch), bf16_dev(inp["w_down"], torch)
    logits = torch.from_numpy(inp["logits"]).cuda()
    shape = moe.LayerShape(T=cfg.T, E=cfg.E, k=cfg.k, e_lo=cfg.e_lo, E_loc=cfg.E_loc, d=cfg.d,
                           H=cfg.H, beta=cfg.beta, linear_beta=cfg.linear_beta)
    torch.cuda.reset_peak_memory_stats()
    buf = moe.LayerBuffers(shape)
    stream = torch.cuda.current_stream()

    print("[bench] warmup", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        buf.step(x, logits, w_gu, w_down, dy)
    torch.cuda.synchronize()
    R = buf.rows()
    assert not buf.overflowed()
    flop_step = 18.0 * R * cfg.d * cfg.H
    flop_gu = 4.0 * R * cfg.d * cfg.H

    # timed region: K full steps; HIP events bracket every gate/up GEMM launch on its stream
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        buf.route(logits)
        ev[i][0].record(stream)
        moe.moe_grouped_gemm_gate_up(x, buf.perm["row_token"], buf.perm["offsets"], w_gu,
                                     buf.R_cap, cfg.beta, cfg.linear_beta, h=buf.h, a=buf.a)
        ev[i][1].record(stream)
        moe.moe_grouped_gemm_down_combine(buf.a, buf.perm["offsets"], buf.perm["row_gate"],
                                          buf.perm["slot_row"], w_down, buf.R_cap, y=buf.y,
                                          ws=buf.ws_down)
        buf.backward(dy, x, w_gu, w_down)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = elapsed * 1e3 / args.steps
    gu_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))

    # one more step with events between the phases (breakdown only, not the headline)
    evs[0].record(stream)
    buf.route(logits)
    evs[1].record(stream)
    moe.moe_grouped_gemm_gate_up(x, buf.perm["row_token"], buf.perm["offsets"], w_gu, buf.R_cap,
                                 cfg.beta, cfg.linear_beta, h=buf.h, a=buf.a)
    evs[2].record(stream)
    moe.moe_grouped_gemm_down_combine(buf.a, buf.perm["offsets"], buf.perm["row_gate"],
                                      buf.perm["slot_row"], w_down, buf.R_cap, y=buf.y,
                                      ws=buf.ws_down)
    evs[3].record(stream)
    buf.backward(dy, x, w_gu, w_down)
    evs[4].record(stream)
    torch.cuda.synchronize()
    phases = dict(route_permute=evs[0].elapsed_time(evs[1]), gate_up=evs[1].elapsed_time(evs[2]),
                  down_combine=evs[2].elapsed_time(evs[3]), backward=evs[3].elapsed_time(evs[4]))
    peak_gb = torch.cuda.max_memory_allocated() / 1e9

    # gate/up moves each local expert's [2H, d] weights once, the R gathered rows of x, and
    # writes h [R, 2H] and a [R, H]
    gu_bytes = 2.0 * (cfg.E_loc * 2 * cfg.H * cfg.d + R * cfg.d + R * 3 * cfg.H)
    value = flop_step / (ms_step * 1e-3) / 1e12
    gu_tflops = flop_gu / (gu_ms * 1e-3) / 1e12
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {cfg.note}; T={cfg.T} d={cfg.d} H={cfg.H} "
                               f"E={cfg.E} k={cfg.k} local experts {cfg.e_lo}..{cfg.e_lo + cfg.E_loc - 1}",
                   "routed_rows": R, "flop_per_step": flop_step, "row_capacity": buf.R_cap},
        "mfma_frac": round(value / PEAK_BF16_TFLOPS, 4),
        "roofline": {"kernel": "grouped GEMM gate/up + SiTU-GLU epilogue", "bound": "mfma",
                     "achieved": round(gu_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(gu_tflops / PEAK_BF16_TFLOPS, 4),
                     "avg_launch_ms": round(gu_ms, 4), "flop_per_launch": flop_gu,
                     "algorithmic_bytes_per_launch": gu_bytes, "traffic": None},
        "phase_ms": {k: round(v, 4) for k, v in phases.items()},
        "peak_hbm_GB": round(peak_gb, 2),
        "saved_activation_GB": round((R * 2 * cfg.H * 2 + cfg.T * cfg.d * 2) / 1e9, 3),
        "naive_saved_fp32_GB": round(6 * R * cfg.H * 4 / 1e9, 3),
    }
    # the same step with the saved h stored as MXFP8 (E4M3 codes + one scale byte per 32)
    del buf
    torch.cuda.empty_cache()
    bmx = moe.LayerBuffers(shape, h_store="mxfp8")
    for _ in range(args.warmup):
        bmx.step(x, logits, w_gu, w_down, dy)
    torch.cuda.synchronize()
    n_mx = max(1, args.steps // 2)
    t0 = time.perf_counter()
    for _ in range(n_mx):
        bmx.step(x, logits, w_gu, w_down, dy)
    torch.cuda.synchronize()
    ms_mx = (time.perf_counter() - t0) * 1e3 / n_mx
    out["mxfp8_h"] = {"ms_per_step": round(ms_mx, 4),
                      "value": round(flop_step / (ms_mx * 1e-3) / 1e12, 2),
                      "saved_activation_GB": round((R * 2 * cfg.H * (1 + 1 / 32) + cfg.T * cfg.d * 2) / 1e9, 3),
                      "steps": n_mx}
    del bmx
    torch.cuda.empty_cache()

    # W4A8 forward (rollouts): MXFP4 weights quantized once, x quantized to MXFP8 each step
    print("[bench] W4A8 forward", file=sys.stderr, flush=True)
    w4 = moe.W4A8Weights(w_gu, w_down)
    b4 = moe.LayerBuffers(shape)
    for _ in range(args.warmup):
        b4.forward_w4a8(x, logits, w4)
    torch.cuda.synchronize()
    assert b4.rows() == R
    ev4 = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        b4.route(logits)
        moe.moe_mxfp8_quantize(x, codes=b4.x_codes, scales=b4.x_scales)
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
    gu4_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev4]))
    dn4_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev4]))
    flop_fwd = 6.0 * R * cfg.d * cfg.H
    out["w4a8_fwd"] = {
        "ms_per_step": round(ms_w4, 4), "value": round(flop_fwd / (ms_w4 * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s (forward, 6 R d H)", "steps": args.steps,
        "bf16_fwd_ms": round(phases["route_permute"] + phases["gate_up"] + phases["down_combine"], 4),
        "gate_up_ms": round(gu4_ms, 4),
        "gate_up_TFLOPs": round(flop_gu / (gu4_ms * 1e-3) / 1e12, 2),
        "gate_up_frac_fp8_peak": round(flop_gu / (gu4_ms * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4),
        "down_combine_ms": round(dn4_ms, 4),
        "weights_GB": round(cfg.E_loc * 3 * cfg.H * cfg.d * (0.5 + 1 / 32) / 1e9, 3),
        "bf16_weights_GB": round(cfg.E_loc * 3 * cfg.H * cfg.d * 2 / 1e9, 3),
    }
    del b4, w4
    torch.cuda.empty_cache()

    tr = committed_traffic(args.workload)
    if tr is not None:
        out["roofline"]["traffic"] = tr["fetch"] + tr["write"]
        out["roofline"].update(traffic_fetch_bytes=tr["fetch"], traffic_write_bytes=tr["write"],
                               traffic_vs_algorithmic=round((tr["fetch"] + tr["write"]) / gu_bytes, 3))

    if not args.no_situ:
        sc = SITU_CONFIGS["situ"]
        Rs, Hs = sc["R"], sc["H"]
        print("[bench] SiTU-GLU streaming", file=sys.stderr, flush=True)
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

    if not args.no_cpu_baseline:
        print("[bench] CPU oracle baseline", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
