#!/usr/bin/env python3
"""Benchmark of the prefill sparse-MoE layer on one MI355X.

One step = the whole layer over one prompt of synthetic tokens already resident
in HBM: routing (router logits, top-k, histogram, scan, scatter, block map),
the grouped gate/up + SwiGLU GEMM, the grouped down GEMM and the weighted
combine, chunk by chunk.  The step enqueues the library's four entry points
(the same kernels moe_layer_forward enqueues) so HIP events on the launch
stream can time each kernel inside the timed region.

Prints one JSON line; see --help for options.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE prefill layer tokens/s at 4K tokens; % of bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
# fp32 vector FMA without packed math: 256 CUs x 4 SIMDs x 16 lanes x 2 flop x 2.4 GHz
# (the published 157.3 TFLOP/s counts packed fp32 ops, which this library does not use)
PEAK_FP32_VALU_TFLOPS = 78.6
def run_gdn(args, shape, torch, B, gen):
    """The Gated DeltaNet prefill scan (gdn_prefill_scan): tokens/s and, as
    its roofline, fp32 vector arithmetic: 7*DK flops per state row and token
    (recall S.k: 2 DK, update alpha*S + c*k: 3 DK, output S.q: 2 DK) over the
    kernel's time."""
    import numpy as np

    dev = "cuda:0"
    torch.cuda.set_device(0)
    inp = gen.make_gdn(shape)
    T, HK, HV, DK, DV = shape.T, shape.HK, shape.HV, shape.DK, shape.DV
    u16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)  # noqa: E731
    q, k, v = u16(inp.q), u16(inp.k), u16(inp.v)
    al = torch.from_numpy(inp.alpha).to(dev)
    be = torch.from_numpy(inp.beta).to(dev)
    si = torch.from_numpy(inp.state_in).to(dev) if inp.state_in is not None else None
    o = torch.empty((T, HV, DV), dtype=torch.float32, device=dev)
    so = torch.empty((HV, DV, DK), dtype=torch.float32, device=dev)
    desc = B.gdn_desc(T, HK, HV, DK, DV)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        B.gdn_prefill_scan(desc, q, k, v, al, be, si, o, so, stream)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for a, b in evs:
        a.record(stream)
        B.gdn_prefill_scan(desc, q, k, v, al, be, si, o, so, stream)
        b.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    scan_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    flop = 7.0 * DK * DV * HV * T
    achieved = flop / (scan_ms * 1e-3) / 1e12
    hbm = 2 * T * HK * DK * 2 + T * HV * DV * 2 + 2 * T * HV * 4 + T * HV * DV * 4 + 2 * HV * DV * DK * 4
    res = {
        "metric": "Gated DeltaNet prefill scan tokens/s",
        "value": round(T * args.steps / elapsed, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: T={T} key heads={HK} value heads={HV} DK={DK} DV={DV}, "
                               "gated delta rule, fp32 state", "tokens": T, "seed": shape.seed},
        "roofline": {"kernel": "gdn_scan_kernel", "bound": "alu", "achieved": round(achieved, 2),
                     "peak": PEAK_FP32_VALU_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP32_VALU_TFLOPS, 4),
                     "traffic": load_traffic("gdn_scan", args.workload), "flop_per_launch": flop,
                     "avg_launch_ms": round(scan_ms, 4)},
        "hbm_bytes_algorithmic": hbm,
        "hbm_GBs": round(hbm / (scan_ms * 1e-3) / 1e9, 1),
    }
    if not args.no_cpu_baseline:
        import oracle.gdn as G

        G.set_threads(os.cpu_count() or 1)  # every host core; the oracle splits over value heads
        threads = min(os.cpu_count() or 1, HV)
        t1 = time.perf_counter()
        G.scan(inp.q, inp.k, inp.v, inp.alpha, inp.beta, inp.state_in)
        dt = time.perf_counter() - t1
        res["cpu_baseline"] = {"value": round(T / dt, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
                               "sample": f"all {T} tokens, fp64 gated delta rule over {HV} heads, {dt:.1f} s"}
    print(json.dumps(res), flush=True)
    return 0


def run_gqa(args, shape, torch, B, gen):
    """Batch-1 GQA decode attention (gqa_decode_attention): decode steps/s and,
    as its roofline, the HBM bytes the step must move (the K and V cache of
    the context once, q, out) over the step's time."""
    import numpy as np

    dev = "cuda:0"
    torch.cuda.set_device(0)
    inp = gen.make_gqa(shape)
    L, HQ, HKV, D = shape.L, shape.HQ, shape.HKV, shape.D
    u16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)  # noqa: E731
    q, k, v = u16(inp.q), u16(inp.k), u16(inp.v)
    desc = B.gqa_desc(L, HQ, HKV, D, inp.scale)
    nbytes = B.gqa_decode_workspace_size(desc)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
    out = torch.empty((HQ, D), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        B.gqa_decode_attention(desc, q, k, v, out, ws, nbytes, stream)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for a, b in evs:
        a.record(stream)
        B.gqa_decode_attention(desc, q, k, v, out, ws, nbytes, stream)
        b.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    step_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    hbm = 2 * L * HKV * D * 2 + HQ * D * 2 + HQ * D * 4
    achieved = hbm / (step_ms * 1e-3) / 1e9
    res = {
        "metric": "GQA decode attention steps/s (batch 1)",
        "value": round(args.steps / elapsed, 1),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: context {L} tokens, {HQ} query heads over {HKV} KV heads, "
                               f"head dim {D}, KV cache in 32-token blocks", "context": L, "seed": shape.seed},
        "roofline": {"kernel": "gqa_split_kernel + gqa_combine_kernel", "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": load_traffic("gqa_decode", args.workload), "bytes_per_launch": hbm,
                     "avg_launch_ms": round(step_ms, 4)},
        "workspace_bytes": nbytes,
    }
    if not args.no_cpu_baseline:
        import oracle.gqa as OA

        OA.set_threads(os.cpu_count() or 1)  # every host core; the oracle splits over query heads
        threads = min(os.cpu_count() or 1, HQ)
        t1 = time.perf_counter()
        reps = 0
        while True:
            OA.decode(L, inp.q, inp.k, inp.v, HKV, inp.scale)
            reps += 1
            dt = time.perf_counter() - t1
            if dt > 2.0 or reps >= 50:
                break
        res["cpu_baseline"] = {"value": round(reps / dt, 2), "unit": "steps/s", "cores": threads, "kind": "oracle",
                               "sample": f"{reps} whole decode steps over the {L}-token context, fp64, {dt:.1f} s"}
    print(json.dumps(res), flush=True)
    return 0


PROFILES = os.path.join(ROOT, "profiles")


def source_digest(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def load_traffic(kernel: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 --pmc summaries, if they
    were taken on the current kernel source; otherwise None."""
    p = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        tab = json.load(f)
    ent = tab.get(f"{kernel}@{workload}")
    if not ent:
        return None
    src = os.path.join(ROOT, "q4_grouped_expert_amd", "csrc", ent["source"])
    if not os.path.exists(src) or source_digest(src) != ent["source_sha256_16"]:
        return None
    return ent["hbm_bytes_per_launch"]


def measure_temp_memory(torch, B, dl, chunks, out):
    """Peak temporary device memory of the layer over the whole prompt: the
    workspace moe_layer_forward needs is allocated inside a
    torch.cuda.max_memory_allocated window and the prompt runs chunk by chunk
    through it (routing results inside the workspace); the library itself
    allocates nothing."""
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    nbytes = B.moe_layer_workspace_size(dl.desc(dl.chunk))
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=out.device)
    for c0, c1 in chunks:
        B.moe_layer_forward(dl.desc(c1 - c0), dl.x[c0:c1], dl.w_router, dl.router_bias, dl.gate_up.desc,
                            dl.down.desc, dl.s_gate_up.desc if dl.has_shared else None,
                            dl.s_down.desc if dl.has_shared else None, out[c0:c1], None, ws, nbytes)
    torch.cuda.synchronize()
    delta = torch.cuda.max_memory_allocated() - base
    del ws
    return {"workspace_bytes": nbytes, "peak_allocated_delta_bytes": int(delta), "chunks": len(chunks),
            "chunk_tokens": dl.chunk}


def copy_calibration(args, torch) -> int:
    """A plain copy of known size: reads and writes n bytes per launch."""
    n = args.copy_calibration_mib << 20
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    print(json.dumps({"copy_bytes_per_launch": n, "launches": args.steps, "ms_per_launch": round(dt * 1e3, 4),
                      "read_plus_write_GBs": round(2 * n / dt / 1e9, 1)}), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100,
                    help="untimed steps first; the GPU takes some tens of milliseconds of load to reach its steady clock")
    ap.add_argument("--workload", default="prefill4096",
                    help="prefill4096 (default), prefill512, skew2048, long16384, tiny; decode1, decode4, "
                         "decode16 (decode-shape layer); gdn4096, gdn512, gdn_tiny (Gated DeltaNet prefill scan); "
                         "attn32k, attn128k, attn3840, attn_tiny (batch-1 GQA decode attention)")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the CPU oracle timing")
    ap.add_argument("--variant", default="fused", choices=["fused", "unfused_dequant", "host_sync"],
                    help="fused: the layer as built (default); unfused_dequant: a separate kernel writes the bf16 "
                         "weights of the experts with rows, then a bf16 grouped GEMM reads them; host_sync: the "
                         "host reads the tile count after routing and sizes the GEMM launches from it")
    ap.add_argument("--cpu-sample-tokens", type=int, default=4096,
                    help="tokens of the workload the CPU oracle is timed on (from the first)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="instead of the layer, run a plain device-to-device copy of this many MiB "
                         "(--steps times); its counter readings scale the HBM byte counters")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this layer is built and measured on one GPU; multi-GPU runs are not "
                                   "part of it (token chunks shard with no exchange, experts would need an "
                                   "all-to-all); run with --gpus 1"}), flush=True)
        return 2

    import numpy as np
    import torch

    from q4_grouped_expert_amd import binding as B
    from q4_grouped_expert_amd import inputs as gen
    from q4_grouped_expert_amd.device import DeviceLayer

    if args.copy_calibration_mib:
        return copy_calibration(args, torch)
    if args.workload in gen.GQA_WORKLOADS:
        B.lib()  # raises if the HIP library is missing
        return run_gqa(args, gen.GQA_WORKLOADS[args.workload], torch, B, gen)
    if args.workload in gen.GDN_WORKLOADS:
        B.lib()  # raises if the HIP library is missing
        return run_gdn(args, gen.GDN_WORKLOADS[args.workload], torch, B, gen)
    if args.workload not in gen.WORKLOADS:
        print(f"unknown workload {args.workload}", file=sys.stderr)
        return 2
    shape = gen.WORKLOADS[args.workload]
    B.lib()  # raises if the HIP library is missing
    if args.workload.startswith("decode"):
        return run_decode(args, shape, torch, B, gen)
    dev = "cuda:0"
    torch.cuda.set_device(0)
    inp = gen.make_layer(shape)
    dl = DeviceLayer(inp, dev)
    T, H, I, E, K = shape.T, shape.H, shape.I, shape.E, shape.K
    chunk = dl.chunk
    chunks = [(c0, min(T, c0 + chunk)) for c0 in range(0, T, chunk)]
    rows_max = chunk * K + (chunk if dl.has_shared else 0)
    route = dl.new_route(chunk)
    rdesc = B.route_desc(route)
    h = torch.empty((rows_max, I), dtype=torch.int16, device=dev)
    # the library's default staging of the down GEMM's rows: bf16 y
    down_mode, y_dtype = B.MOE_GEMM_DOWN_BF16, B.MOE_DTYPE_BF16
    y = torch.empty((rows_max, H), dtype=torch.int16, device=dev)
    out = torch.empty((T, H), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    sgu = dl.s_gate_up.desc if dl.has_shared else None
    sdn = dl.s_down.desc if dl.has_shared else None

    variant = args.variant
    if variant == "unfused_dequant":
        # bf16 weight buffers the separate dequant kernel writes (experts with rows)
        i16 = dict(dtype=torch.int16, device=dev)
        wgu, wdn = torch.empty((E, 2 * I, H), **i16), torch.empty((E, H, I), **i16)
        bgu, bdn = B.bf16_desc(wgu, E, 2 * I, H), B.bf16_desc(wdn, E, H, I)
        bgu_s = bdn_s = None
        if dl.has_shared:
            wgu_s, wdn_s = torch.empty((1, 2 * I, H), **i16), torch.empty((1, H, I), **i16)
            bgu_s, bdn_s = B.bf16_desc(wgu_s, 1, 2 * I, H), B.bf16_desc(wdn_s, 1, H, I)

        def dequant(w, w_bf, s_w, s_bf):
            B.moe_dequant_q4_to_bf16(w, route["counts"], w_bf, stream)
            if s_w is not None:
                B.moe_dequant_q4_to_bf16(s_w, None, s_bf, stream)

    # phase names of one chunk, timed with events between them
    names = {"fused": ["route", "gemm_gate_up", "gemm_down", "combine"],
             "unfused_dequant": ["route", "dequant_gate_up", "gemm_gate_up", "dequant_down", "gemm_down",
                                 "combine"],
             "host_sync": ["layer"]}[variant]

    def step(events=None, only=None):
        """One pass over all chunks.  events[chunk][i] is recorded after phase
        i - 1; with `only`, just the events that bracket that phase."""
        for ci, (c0, c1) in enumerate(chunks):
            d = dl.desc(c1 - c0)
            ev = events[ci] if events is not None else None

            def mark(i):
                if ev and (only is None or i in only):
                    ev[i].record(stream)
            mark(0)
            if variant == "host_sync":
                B.moe_layer_forward_host_sync(d, dl.x[c0:c1], dl.w_router, dl.router_bias, dl.gate_up.desc,
                                              dl.down.desc, sgu, sdn, out[c0:c1], rdesc, dl.ws, dl.ws_bytes, stream)
                mark(1)
                continue
            B.moe_route(d, dl.x[c0:c1], dl.w_router, dl.router_bias, rdesc, dl.route_ws, dl.route_ws_bytes, stream)
            mark(1)
            if variant == "fused":
                B.moe_grouped_gemm_q4(d, B.MOE_GEMM_GATE_UP_SWIGLU, dl.x[c0:c1], dl.gate_up.desc, sgu, rdesc, h,
                                      stream=stream)
                mark(2)
                B.moe_grouped_gemm_q4(d, down_mode, h, dl.down.desc, sdn, rdesc, y, stream=stream)
                mark(3)
            else:
                dequant(dl.gate_up.desc, wgu, sgu, wgu_s if dl.has_shared else None)
                mark(2)
                B.moe_grouped_gemm_bf16(d, B.MOE_GEMM_GATE_UP_SWIGLU, dl.x[c0:c1], bgu, bgu_s, rdesc, h,
                                        stream=stream)
                mark(3)
                dequant(dl.down.desc, wdn, sdn, wdn_s if dl.has_shared else None)
                mark(4)
                B.moe_grouped_gemm_bf16(d, down_mode, h, bdn, bdn_s, rdesc, y, stream=stream)
                mark(5)
            B.moe_combine(d, y, rdesc, out[c0:c1], y_dtype=y_dtype, stream=stream)
            mark(len(names))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    assert torch.isfinite(out).all().item(), "non-finite layer output"

    def phase_times(evs, phases):
        per = {n: [] for n in phases}
        for ev_step in evs:
            for ev in ev_step:
                for n in phases:
                    i = names.index(n)
                    per[n].append(ev[i].elapsed_time(ev[i + 1]))
        return {n: float(np.mean(v)) for n, v in per.items()}

    def new_events():
        return [[[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in chunks]
                for _ in range(args.steps)]

    if variant != "fused":
        evs = new_events()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(args.steps):
            step(evs[s])
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        return report_variant(args, shape, dl, chunk, T, elapsed, phase_times(evs, names))

    def layer_step():
        """One step as the library runs it: moe_layer_forward chunk by chunk
        through one workspace (routing results, h and y inside it)."""
        for c0, c1 in chunks:
            B.moe_layer_forward(dl.desc(c1 - c0), dl.x[c0:c1], dl.w_router, dl.router_bias, dl.gate_up.desc,
                                dl.down.desc, sgu, sdn, out[c0:c1], None, dl.ws, dl.ws_bytes, stream)

    # The timed steps are the library's layer entry point with nothing else
    # on the stream: a recorded event waits for the kernel before it and the
    # next kernel for the event, a gap of several microseconds each.  Passes
    # over the same steps then record (a) an event pair around each step for
    # the per-step median, (b) events around the gate/up launch only (the
    # roofline's kernel) and (c) events between all phases for the breakdown;
    # (b) and (c) enqueue the four entry points the layer is made of.
    for _ in range(args.warmup):
        layer_step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        layer_step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    step_evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in range(args.steps)]
    for s in range(args.steps):
        step_evs[s][0].record(stream)
        layer_step()
        step_evs[s][1].record(stream)
    torch.cuda.synchronize()
    step_ms = [a.elapsed_time(b) for a, b in step_evs]
    gu = names.index("gemm_gate_up")
    evs = new_events()
    for s in range(args.steps):
        step(evs[s], only=(gu, gu + 1))
    torch.cuda.synchronize()
    gu_ms_timed = phase_times(evs, ["gemm_gate_up"])["gemm_gate_up"]
    evs_all = new_events()
    for s in range(args.steps):
        step(evs_all[s])
    torch.cuda.synchronize()
    kernels_ms = phase_times(evs_all, names)

    # algorithmic work of the dominant kernel (gate/up GEMM) per launch
    counts_last = route["counts"].cpu().numpy()
    rows_per_launch = [(c1 - c0) * K + ((c1 - c0) if dl.has_shared else 0) for c0, c1 in chunks]
    flop_gu = float(np.mean([2.0 * r * H * 2 * I for r in rows_per_launch]))
    gu_ms = gu_ms_timed
    achieved_tflops = flop_gu / (gu_ms * 1e-3) / 1e12
    flop_dn = float(np.mean([2.0 * r * I * H for r in rows_per_launch]))
    traffic = load_traffic("gemm_gate_up", args.workload)

    # per-kernel rates over the algorithmic bytes each one must move (per launch = per chunk)
    n_ne = int((counts_last > 0).sum()) + (1 if dl.has_shared else 0)
    wb_gu = 2 * I * H // 2 + 2 * I * (H // 64) * 4      # codes + bf16 scale and bias, one expert
    wb_dn = H * I // 2 + H * (I // 64) * 4
    rows_m = float(np.mean(rows_per_launch))
    Tc = float(np.mean([c1 - c0 for c0, c1 in chunks]))
    Rc = Tc * K
    route_bytes = Tc * H * 2 + E * H * 2 + Rc * 8 + 2 * Rc * 4 + (2 * E + 1) * 4
    comb_bytes = rows_m * H * 2 + Tc * H * 4 + Rc * 8  # bf16 y rows in, fp32 out

    def rate(b, ms):
        return round(b / (ms * 1e-3) / 1e9, 1)

    kernels = {
        "route": {"ms": round(kernels_ms["route"], 4), "GBs": rate(route_bytes, kernels_ms["route"]),
                  "router_TFLOPs": round(2 * Tc * H * E / (kernels_ms["route"] * 1e-3) / 1e12, 2)},
        "gemm_gate_up": {"ms": round(gu_ms, 4), "TFLOPs": round(achieved_tflops, 2),
                         "mfma_frac": round(achieved_tflops / PEAK_BF16_TFLOPS, 4),
                         "weight_GBs": rate(n_ne * wb_gu, gu_ms)},
        "gemm_down": {"ms": round(kernels_ms["gemm_down"], 4),
                      "TFLOPs": round(flop_dn / (kernels_ms["gemm_down"] * 1e-3) / 1e12, 2),
                      "mfma_frac": round(flop_dn / (kernels_ms["gemm_down"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                      "weight_GBs": rate(n_ne * wb_dn, kernels_ms["gemm_down"])},
        "combine": {"ms": round(kernels_ms["combine"], 4), "GBs": rate(comb_bytes, kernels_ms["combine"])},
    }

    ms_per_step = elapsed * 1e3 / args.steps
    value = T * args.steps / elapsed
    total_flop = flop_gu * len(chunks) + flop_dn * len(chunks)
    dn_ms = kernels_ms["gemm_down"]
    med_step_ms = float(np.median(step_ms))
    temp_mem = measure_temp_memory(torch, B, dl, chunks, out)
    res = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{args.workload}: T={T} H={H} I={I} E={E} top-{K}"
                        f"{' + 1 shared' if dl.has_shared else ''}, SwiGLU, Q4 groupwise-affine g=64 "
                        f"(bf16 scale+bias), chunk={chunk}"
                        + (f", Zipf({shape.zipf_s}) router bias" if shape.zipf_s else ""),
            "tokens": T, "chunk": chunk, "seed": shape.seed, "norm_topk": 1,
        },
        "roofline": {
            "kernel": "gemm_q4_kernel<gate_up+SwiGLU>",
            "bound": "mfma",
            "achieved": round(achieved_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "flop_per_launch": flop_gu,
            "avg_launch_ms": round(gu_ms, 4),
            # the other GEMM and the whole layer against the same bf16 dense peak
            "gemm_down_frac": round(flop_dn / (dn_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "gemm_down_avg_launch_ms": round(dn_ms, 4),
            "layer_gemm_frac": round(total_flop / (med_step_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        },
        "kernels": kernels,
        "kernels_note": "per-phase HIP-event means from a pass of the same steps with an event between every "
                        "phase; the gate/up time (roofline) from a pass whose events bracket only that launch; "
                        "the timed steps call moe_layer_forward with no events between them",
        "layer_gemm_tflops": round(total_flop / (ms_per_step * 1e-3) / 1e12, 2),
        "step_ms_median": round(med_step_ms, 4),
        "step_ms_mean": round(float(np.mean(step_ms)), 4),
        "step_ms_note": "HIP events on the launch stream around each step, in a pass of the same steps after "
                        "the timed one (each event pair adds a gap to its step)",
        "temporary_memory": temp_mem,
        "nonempty_experts_last_chunk": int((counts_last > 0).sum()),
    }

    if not args.no_cpu_baseline:
        import oracle

        S = min(args.cpu_sample_tokens, T)
        nthreads = os.cpu_count() or 1  # every host core
        xs = np.ascontiguousarray(inp.x[:S])
        t1 = time.perf_counter()
        oracle.layer_forward(inp, x=xs, nthreads=nthreads)
        dt = time.perf_counter() - t1
        res["cpu_baseline"] = {"value": round(S / dt, 2), "unit": "tokens/s", "cores": nthreads, "kind": "oracle",
                               "sample": f"first {S} of the {T} tokens, whole layer (routing, dequant of every "
                                         f"expert with rows, SwiGLU FFN, combine), {dt:.1f} s"}
    print(json.dumps(res), flush=True)
    return 0


def run_decode(args, shape, torch, B, gen):
    """The decode-shape layer (moe_decode_forward, at most 16 tokens): layer
    tokens/s and, as its roofline, the HBM bytes the call must move (the Q4
    weights of every expert with rows plus the shared expert, x and out) over
    the layer's time."""
    import numpy as np

    from q4_grouped_expert_amd.device import DeviceLayer

    dev = "cuda:0"
    torch.cuda.set_device(0)
    inp = gen.make_layer(shape)
    dl = DeviceLayer(inp, dev)
    T, H, I, E, K = shape.T, shape.H, shape.I, shape.E, shape.K
    route = dl.new_route(T)
    out = torch.empty((T, H), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    dl.decode_router()  # the prepared router copy is per model, outside the step
    for _ in range(args.warmup):
        dl.decode(dl.x, out, route, stream)
    torch.cuda.synchronize()
    # timed calls back to back with nothing else on the stream; then the same
    # calls each between an event pair for the per-call duration
    t0 = time.perf_counter()
    for _ in range(args.steps):
        dl.decode(dl.x, out, route, stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a, b in evs:
        a.record(stream)
        dl.decode(dl.x, out, route, stream)
        b.record(stream)
    torch.cuda.synchronize()
    layer_ms = float(np.median([a.elapsed_time(b) for a, b in evs]))
    counts = route["counts"].cpu().numpy()
    n_ne = int((counts > 0).sum()) + (1 if dl.has_shared else 0)
    wbytes = n_ne * ((2 * I * H + H * I) // 2 + (2 * I * (H // 64) + H * (I // 64)) * 4)
    hbm_bytes = wbytes + T * H * 2 + T * H * 4
    achieved = hbm_bytes / (layer_ms * 1e-3) / 1e9
    res = {
        "metric": "MoE decode layer tokens/s (1-16 tokens per call)",
        "value": round(T * args.steps / elapsed, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: T={T} H={H} I={I} E={E} top-{K}"
                               f"{' + 1 shared' if dl.has_shared else ''}, decode path", "tokens": T,
                   "seed": shape.seed, "norm_topk": 1},
        "roofline": {"kernel": "decode layer (router, grouping, split-reduction GEMVs, combine)", "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None,
                     "bytes_per_launch": hbm_bytes, "avg_launch_ms": round(layer_ms, 4),
                     "avg_launch_note": "median of HIP-event pairs around single calls"},
        "experts_read": n_ne,
    }
    if not args.no_cpu_baseline:
        import oracle

        nthreads = os.cpu_count() or 1  # every host core
        t1 = time.perf_counter()
        reps = 0
        while True:
            oracle.layer_forward(inp, nthreads=nthreads)
            reps += 1
            dt = time.perf_counter() - t1
            if dt > 2.0 or reps >= 20:
                break
        res["cpu_baseline"] = {"value": round(T * reps / dt, 2), "unit": "tokens/s", "cores": nthreads,
                               "kind": "oracle", "sample": f"{reps} whole calls of the {T}-token layer, {dt:.1f} s"}
    print(json.dumps(res), flush=True)
    return 0


def report_variant(args, shape, dl, chunk, T, elapsed, kernels_ms):
    """One JSON line for an ablation variant: layer tokens/s and the per-phase
    means of the variant (no roofline entry: that is the fused layer's)."""
    ms_per_step = elapsed * 1e3 / args.steps
    res = {
        "metric": METRIC,
        "value": round(T * args.steps / elapsed, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{args.workload}: T={T} H={shape.H} I={shape.I} E={shape.E} top-{shape.K}"
                        f"{' + 1 shared' if dl.has_shared else ''}, chunk={chunk}",
            "variant": args.variant, "tokens": T, "chunk": chunk, "seed": shape.seed, "norm_topk": 1,
        },
        "phases_ms": {n: round(v, 4) for n, v in kernels_ms.items()},
    }
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
