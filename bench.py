#!/usr/bin/env python3
"""Benchmark of the Gemma 4 interleaved attention block on one MI355X.

One step = the whole hot path once over synthetic, seeded bf16 inputs already
resident in HBM:
  - prefill of one 5:1 interleave group at long context (B=1, S=262144):
    5 sliding-window local layers (Hq=16, Hkv=8, d=256, window 1024, full
    RoPE) then 1 global layer (Hq=16, Hkv=2, d=512, K=V, p-RoPE p=0.25);
  - one decode step of the same 5:1 group for a batch of 64 sequences with
    cache lengths uniform in [4096, 65536]: 5 local layers (Hq=16, Hkv=8,
    d=256, 512-slot ring cache) then 1 global layer (Hq=16, Hkv=2, d=512, K=V
    linear cache).
value = algorithmic attention FLOPs of the step / step time (TFLOP/s); only
(query, key) pairs the mask keeps are counted.  Per-kind times come from HIP
events recorded on the stream the kernels run on.  Prints one JSON line.
"""
import argparse
import json
import math
import os
import sys
import time

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E peak


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--only", choices=["all", "local", "global", "decode", "fp8", "vision", "multi"], default="all",
                    help="restrict the step to one kernel kind (profiling runs)")
    ap.add_argument("--seq", type=int, default=None, help="override the prefill length")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the stand-alone local (B=4, S=8192) and global (S=32768) timings")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="finish with one plain device copy of MIB MiB (scale for HBM counters)")
    return ap.parse_args()


PROFILES = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles")
TRAFFIC_SUMMARY = os.path.join(PROFILES, "prefill_global_kv512_s262144_hbm_traffic.txt")
DECODE_TRAFFIC_SUMMARY = os.path.join(PROFILES, "decode_global_kv512_b64_hbm_traffic.txt")
MFMA_SUMMARY = os.path.join(PROFILES, "prefill_global_kv512_s262144_mfma_busy.txt")
# the other kernels' counter summaries: (entry, file, figure)
OTHER_COUNTERS = [
    ("local_prefill_hbm_bytes_per_launch", "prefill_local_d256_w1024_s262144_hbm_traffic.txt",
     "hbm_bytes_per_launch"),
    ("local_prefill_mfma_busy", "prefill_local_d256_w1024_s262144_mfma_busy.txt",
     "mfma_busy_fraction_at_2.4GHz"),
    ("local_decode_hbm_bytes_per_launch", "decode_local_d256_ring512_b64_hbm_traffic.txt",
     "hbm_bytes_per_launch"),
    ("decode_multi_global_q4_hbm_bytes_per_launch",
     "decode_multi_q4_global_kv512_b64_hbm_traffic.txt", "hbm_bytes_per_launch"),
    ("decode_fp8_global_hbm_bytes_per_launch", "decode_fp8_global_kv512_b64_hbm_traffic.txt",
     "hbm_bytes_per_launch"),
    ("decode_fp8_local_hbm_bytes_per_launch", "decode_fp8_local_d256_ring512_b64_hbm_traffic.txt",
     "hbm_bytes_per_launch"),
    ("vision_budget280_b4_mfma_busy", "prefill_vision_budget280_b4_mfma_busy.txt",
     "mfma_busy_fraction_at_2.4GHz"),
    ("vision_budget1120_b1_mfma_busy", "prefill_vision_budget1120_b1_mfma_busy.txt",
     "mfma_busy_fraction_at_2.4GHz"),
]


def measured_traffic(path=TRAFFIC_SUMMARY, key="hbm_bytes_per_launch"):
    """One figure (HBM bytes per launch by default) of a committed rocprofv3
    counter summary, or None when the kernel sources it names changed since."""
    try:
        text = open(path).read()
    except OSError:
        return None
    vals = dict(line.split(":", 1) for line in text.splitlines()
                if ":" in line and line.split(":", 1)[0] in ("source_sha256", key, "sources"))
    from attention_g4attn_amd.profsum import source_hash
    sources = [f.strip() for f in vals.get("sources", "").split(",") if f.strip()]
    if not sources or vals.get("source_sha256", "").strip() != source_hash(sources):
        return None
    try:
        return float(vals[key])
    except (KeyError, ValueError):
        return None


def prefill_flops(layer):
    """4 * d * Hq * B * sum_i n_i, n_i = keys row i sees."""
    S, W = layer.S, layer.window
    if W == 0 or W >= S:
        pairs = S * (S + 1) // 2
    else:
        pairs = W * (W + 1) // 2 + (S - W) * W
    return 4.0 * layer.d * layer.Hq * layer.B * pairs


def decode_cost(layer, lengths):
    """(FLOPs, bytes): cache rows read once (K and V, or one tensor for K=V),
    plus q and out."""
    n = [min(int(L), layer.window) if layer.window > 0 else int(L) for L in lengths]
    rows = sum(n)
    tensors = 1 if layer.kind == "global" else 2
    byts = rows * layer.Hkv * layer.d * 2 * tensors + layer.B * layer.Hq * layer.d * (2 + 4)
    flops = 4.0 * layer.d * sum(n) * layer.Hq
    return flops, byts


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; "
                          "sharding across GPUs is not implemented", "n_gpus": args.gpus}))
        sys.exit(2)
    import numpy as np
    import torch

    import attention_g4attn_amd as g4
    from attention_g4attn_amd import inputs

    dev = "cuda"
    torch.cuda.set_device(0)
    S = args.seq or inputs.GROUP_S
    loc = inputs.local(1, S)
    glo = inputs.global_(1, S)
    dloc, dglo = inputs.DECODE_LOCAL, inputs.DECODE_GLOBAL
    lengths = inputs.decode_lengths(dloc.B)
    bf = torch.bfloat16
    run_local = args.only in ("all", "local")
    run_global = args.only in ("all", "global")
    run_decode = args.only in ("all", "decode")

    t_setup = time.time()
    L_in = [inputs.prefill_inputs(loc, 5, i, bf, dev) for i in range(5)] if run_local else []
    L_out = [torch.empty((1, S, loc.Hq, loc.d), dtype=torch.float32, device=dev) for _ in L_in]
    G_in = inputs.prefill_inputs(glo, 5, 5, bf, dev) if run_global else None
    G_out = torch.empty((1, S, glo.Hq, glo.d), dtype=torch.float32, device=dev) if run_global else None
    D_loc = [inputs.decode_inputs(dloc, 4, i, bf, dev, lengths) for i in range(5)] if run_decode else []
    D_glo = inputs.decode_inputs(dglo, 4, 5, bf, dev, lengths) if run_decode else None
    D_out_l = [torch.empty((dloc.B, dloc.Hq, dloc.d), dtype=torch.float32, device=dev) for _ in D_loc]
    D_out_g = torch.empty((dglo.B, dglo.Hq, dglo.d), dtype=torch.float32, device=dev) if run_decode else None
    ws_l = torch.empty(g4.decode_workspace_bytes(dloc.B, dloc.Hq, dloc.Hkv, dloc.d, dloc.capacity,
                                                 dloc.window), dtype=torch.uint8, device=dev)
    ws_g = torch.empty(g4.decode_workspace_bytes(dglo.B, dglo.Hq, dglo.Hkv, dglo.d, dglo.capacity,
                                                 dglo.window), dtype=torch.uint8, device=dev)
    # prefill workspaces (rotated key slabs), allocated once outside the timed region
    pws_l = torch.empty(max(16, g4.prefill_workspace_bytes(1, S, loc.Hkv, loc.d, loc.p)),
                        dtype=torch.uint8, device=dev)
    pws_g = torch.empty(max(16, g4.prefill_workspace_bytes(1, S, glo.Hkv, glo.d, glo.p)),
                        dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    print(f"# setup {time.time() - t_setup:.1f}s", file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream()
    kinds = ["local_prefill", "global_prefill", "local_decode", "global_decode"]

    # Each run of launches of one kind (the 5 local prefills, the global
    # prefill, the 5 local decodes, the global decode) is bracketed by one
    # event pair on the launch stream, and its time divided by the launches
    # in it.  An event pair around every single launch adds the event
    # packets' own cost to each: about 5 us on a 55 us decode launch.
    def step(record):
        ev = []
        def mark():
            if record:
                e = torch.cuda.Event(enable_timing=True)
                e.record(stream)
                ev.append(e)
        if L_in:
            mark()
            for (q, k, v, pos), out in zip(L_in, L_out):
                g4.local_prefill(q, k, v, pos, loc.window, loc.theta, loc.p, out=out,
                                 workspace=pws_l)
            mark()
        if G_in is not None:
            q, kv, _, pos = G_in
            mark()
            g4.global_prefill(q, kv, pos, 0, glo.theta, glo.p, out=G_out, workspace=pws_g)
            mark()
        if D_loc:
            mark()
            for (q, kc, vc, pos, _), out in zip(D_loc, D_out_l):
                g4.decode(q, kc, vc, pos, dloc.window, dloc.theta, dloc.p, out=out,
                          workspace=ws_l)
            mark()
        if D_glo is not None:
            q, kc, _, pos, _ = D_glo
            mark()
            g4.decode(q, kc, None, pos, 0, dglo.theta, dglo.p, out=D_out_g, workspace=ws_g)
            mark()
        return ev

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    per_kind = {k: [] for k in kinds}
    t0 = time.perf_counter()
    all_ev = []
    for _ in range(args.steps):
        all_ev.append(step(True))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for ev in all_ev:
        pairs = iter([ev[i].elapsed_time(ev[i + 1]) for i in range(0, len(ev), 2)])
        if L_in:
            per_kind["local_prefill"].append(next(pairs) / len(L_in))
        if G_in is not None:
            per_kind["global_prefill"].append(next(pairs))
        if D_loc:
            per_kind["local_decode"].append(next(pairs) / len(D_loc))
        if D_glo is not None:
            per_kind["global_decode"].append(next(pairs))
    print(f"# timed {args.steps} steps in {wall:.2f}s", file=sys.stderr, flush=True)
    # fp8, vision, multi: that side timing alone (for counter runs)
    side = args.only in ("fp8", "vision", "multi")
    extra = {} if args.no_configs or side else time_configs(g4, inputs, torch)
    nxt = {} if args.no_configs or side else time_next(g4, inputs, torch)
    if args.only == "fp8":
        nxt["fp8"] = time_fp8(g4, inputs, torch)
    elif args.only == "vision":
        nxt["vision"] = time_vision(g4, inputs, torch)
    elif args.only == "multi":
        nxt.update(time_next(g4, inputs, torch))
    elif not args.no_configs:
        nxt["fp8"] = time_fp8(g4, inputs, torch)
        nxt["vision"] = time_vision(g4, inputs, torch)

    fl_loc, fl_glo = prefill_flops(loc), prefill_flops(glo)
    (fdl, bdl), (fdg, bdg) = decode_cost(dloc, lengths), decode_cost(dglo, lengths)
    step_flops = 5 * fl_loc * run_local + fl_glo * run_global + (5 * fdl + fdg) * run_decode
    ms_step = wall * 1e3 / args.steps

    def mean(x):
        return float(np.mean(x)) if x else None

    kind_rep = {}
    if run_local:
        t = mean(per_kind["local_prefill"])
        kind_rep["local_prefill"] = {"ms": t, "tflops": fl_loc / t / 1e9,
                                     "frac_mfma": fl_loc / t / 1e9 / MFMA_BF16_PEAK_TFLOPS}
    if run_global:
        t = mean(per_kind["global_prefill"])
        kind_rep["global_prefill"] = {"ms": t, "tflops": fl_glo / t / 1e9,
                                      "frac_mfma": fl_glo / t / 1e9 / MFMA_BF16_PEAK_TFLOPS}
    if run_decode:
        tl, tg = mean(per_kind["local_decode"]), mean(per_kind["global_decode"])
        kind_rep["local_decode"] = {"us": tl * 1e3, "GBps": bdl / tl / 1e6,
                                    "frac_hbm": bdl / tl / 1e6 / HBM_PEAK_GBS,
                                    "tok_per_s": dloc.B / tl * 1e3}
        kind_rep["global_decode"] = {"us": tg * 1e3, "GBps": bdg / tg / 1e6,
                                     "frac_hbm": bdg / tg / 1e6 / HBM_PEAK_GBS,
                                     "tok_per_s": dglo.B / tg * 1e3}
        kind_rep["group_decode_tok_per_s"] = dloc.B / (5 * tl + tg) * 1e3

    if not args.no_configs and not side:
        nxt["schedules"] = time_schedules(g4, inputs, torch)

    roof = None
    if run_global:
        t = mean(per_kind["global_prefill"])
        ach = fl_glo / t / 1e9
        roof = {"bound": "mfma", "achieved": ach, "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": ach / MFMA_BF16_PEAK_TFLOPS,
                "traffic": measured_traffic() if S == inputs.GROUP_S else None,
                # matrix-core busy fraction of the same launch from its counters
                "mfma_busy": (measured_traffic(MFMA_SUMMARY, "mfma_busy_fraction_at_2.4GHz")
                              if S == inputs.GROUP_S else None),
                "kernel": "g4a::pf::prefill_kernel<512, 8, true, false, 128, 3, 1, true, false>",
                "flops_per_launch": fl_glo, "ms_per_launch": t}
    roof_dec = None
    if run_decode:
        tg = mean(per_kind["global_decode"])
        ach = bdg / tg / 1e6
        roof_dec = {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": ach / HBM_PEAK_GBS, "bytes_per_launch": bdg,
                    "traffic": measured_traffic(DECODE_TRAFFIC_SUMMARY),
                    "kernel": "g4a::decode_split_kernel<512, 8, true, 4, 4, false> + decode_merge_kernel"}

    cpu = None
    if not args.no_cpu_baseline and run_global and run_local:
        cpu = cpu_baseline(args, loc, glo, L_in[0], G_in, L_out[0], G_out, 5 * fl_loc + fl_glo)

    rec = {
        "metric": "attention TFLOP/s (prefill) + decode tok/s, as % of MFMA / HBM roofline",
        "value": step_flops / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"gemma4 5:1 interleave group prefill S={S} (5 local W=1024 "
                               f"Hq16/Hkv8/d256 + 1 global K=V p=0.25 Hq16/Hkv2/d512) + "
                               f"batch-64 decode of the group (cache 4096..65536)",
                   "global_batch": 1, "seq_len": S, "parallelism": "none (1 GPU)",
                   "only": args.only},
        "kinds": kind_rep,
        "configs": extra,
        "next": nxt,
        "roofline": roof,
        "roofline_decode": roof_dec,
        "cpu_baseline": cpu,
        # figures of the committed counter summaries (None once the kernel changed)
        "counters": {k: measured_traffic(os.path.join(PROFILES, f), key)
                     for k, f, key in OTHER_COUNTERS},
    }
    if args.copy_calibration > 0:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty(n, dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        rec["copy_calibration_bytes"] = n
    print(json.dumps(rec), flush=True)


def time_configs(g4, inputs, torch, reps=5):
    """Stand-alone timings of the local prefill (B=4, S=8192) and the global
    prefill (S=32768) shapes, outside the timed step."""
    res = {}
    for name, layer, wl in (("local_prefill_b4_s8192", inputs.LOCAL_PREFILL, 2),
                            ("global_prefill_s32768", inputs.GLOBAL_PREFILL, 3)):
        q, k, v, pos = inputs.prefill_inputs(layer, wl, 0, torch.bfloat16, "cuda")
        out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
        ws = torch.empty(max(16, g4.prefill_workspace_bytes(layer.B, layer.S, layer.Hkv, layer.d,
                                                            layer.p)),
                         dtype=torch.uint8, device="cuda")

        def call(r):
            if layer.kind == "global":
                g4.global_prefill(q, k, pos, 0, layer.theta, layer.p, out=out, workspace=ws)
            else:
                g4.local_prefill(q, k, v, pos, layer.window, layer.theta, layer.p, out=out,
                                 workspace=ws)
        ms = _event_time(torch, call, reps)
        fl = prefill_flops(layer)
        res[name] = {"ms": ms, "tflops": fl / ms / 1e9,
                     "frac_mfma": fl / ms / 1e9 / MFMA_BF16_PEAK_TFLOPS}
        del q, k, v, pos, out, ws
    return res


def _event_time(torch, call, reps, warm_s=0.05, min_s=0.1):
    """Mean ms of call(r), r = 0, 1, ..., timed with events on the current
    stream.  Calls first run for about warm_s seconds, so that a short kernel
    is timed at the clock the GPU holds under load rather than while the
    clock ramps up from idle; then at least reps calls, and enough to last
    about min_s seconds, are timed."""
    t0 = time.perf_counter()
    n = 0
    while True:
        call(n)
        torch.cuda.synchronize()
        n += 1
        if time.perf_counter() - t0 >= warm_s:
            break
    est = (time.perf_counter() - t0) / n
    reps = max(reps, min(int(math.ceil(min_s / est)), 20000))
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for r in range(reps):
        call(r)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def time_next(g4, inputs, torch, q_len=4, reps=8):
    """The steps on either side of the path: filling the decode caches from a
    prefill, and decoding q_len tokens per sequence at once (the verify step
    of speculative decoding), at the decode and group shapes.  Rates count
    every cache row once (the algorithmic bytes)."""
    res = {}
    # local: a ring of window + q_len - 1 slots per (sequence, kv head); four
    # distinct caches in turn, as distinct layers are (beyond the last-level cache)
    base = inputs.DECODE_LOCAL
    loc = inputs.DecodeLayer(base.kind, base.B, base.Hq, base.Hkv, base.d,
                             base.window + q_len - 1, base.window, base.theta, base.p)
    caches = [inputs.decode_inputs(loc, 60 + i, 0, torch.bfloat16, "cuda")[1:3] for i in range(4)]
    q = inputs.randn((loc.B, q_len, loc.Hq, loc.d), 6001, torch.bfloat16, "cuda")
    pos = torch.full((loc.B,), 100000, dtype=torch.int32, device="cuda")
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    ws = torch.empty(max(16, g4.decode_multi_workspace_bytes(loc.B, q_len, loc.Hq, loc.Hkv, loc.d,
                                                              loc.capacity, loc.window)),
                     dtype=torch.uint8, device="cuda")
    ms = _event_time(torch, lambda r: g4.decode_multi(q, caches[r % 4][0], caches[r % 4][1], pos,
                                                      loc.window, loc.theta, loc.p, out=out,
                                                      workspace=ws), reps)
    byts = loc.B * loc.Hkv * loc.capacity * loc.d * 2 * 2 + q.numel() * (2 + 4)
    res[f"decode_multi_local_q{q_len}"] = {"us": ms * 1e3, "GBps": byts / ms / 1e6,
                                          "frac_hbm": byts / ms / 1e6 / HBM_PEAK_GBS,
                                          "tok_per_s": loc.B * q_len / ms * 1e3}
    del caches, q, out, ws
    # global: the K=V linear cache of the decode shape, lengths as there
    glo = inputs.DECODE_GLOBAL
    _, kc, _, pos, lengths = inputs.decode_inputs(glo, 61, 0, torch.bfloat16, "cuda")
    q = inputs.randn((glo.B, q_len, glo.Hq, glo.d), 6101, torch.bfloat16, "cuda")
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    ws = torch.empty(max(16, g4.decode_multi_workspace_bytes(glo.B, q_len, glo.Hq, glo.Hkv, glo.d,
                                                              glo.capacity, 0)),
                     dtype=torch.uint8, device="cuda")
    ms = _event_time(torch, lambda r: g4.decode_multi(q, kc, None, pos, 0, glo.theta, glo.p,
                                                      out=out, workspace=ws), reps)
    byts = int(lengths.sum()) * glo.Hkv * glo.d * 2 + q.numel() * (2 + 4)
    res[f"decode_multi_global_q{q_len}"] = {"us": ms * 1e3, "GBps": byts / ms / 1e6,
                                           "frac_hbm": byts / ms / 1e6 / HBM_PEAK_GBS,
                                           "tok_per_s": glo.B * q_len / ms * 1e3,
                                           "column_blocks": (glo.Hq // glo.Hkv * q_len + 15) // 16}
    del kc, q, out, ws
    # cache fill of the group's global prefill rows (K=V, linear cache)
    gl = inputs.global_(1, inputs.GROUP_S)
    k = inputs.randn((gl.B, gl.S, gl.Hkv, gl.d), 6201, torch.bfloat16, "cuda")
    p = inputs.positions(gl.B, gl.S, "cuda")
    kc = torch.empty((gl.B, gl.Hkv, gl.S, gl.d), dtype=torch.bfloat16, device="cuda")
    ms = _event_time(torch, lambda r: g4.fill_cache(k, None, p, kc, None, 0), reps)
    byts = 2 * k.numel() * 2 + p.numel() * 4
    res["fill_cache_global_s262144"] = {"us": ms * 1e3, "GBps": byts / ms / 1e6,
                                        "frac_hbm": byts / ms / 1e6 / HBM_PEAK_GBS}
    del k, p, kc
    return res


def time_fp8(g4, inputs, torch, reps=8):
    """Decode over FP8 E4M3 caches (one byte per element, a scale per KV head)
    at the decode shapes, and the quantizing fill of the group's global
    prefill rows.  Rates count every cache row once at one byte per element
    (the algorithmic bytes of the fp8 cache)."""
    res = {}
    loc = inputs.DECODE_LOCAL
    sets = [inputs.decode_inputs_fp8(loc, 70 + i, 0, "cuda") for i in range(4)]
    out = torch.empty(sets[0][0].shape, dtype=torch.float32, device="cuda")
    ws = torch.empty(max(16, g4.decode_fp8_workspace_bytes(loc.B, 1, loc.Hq, loc.Hkv, loc.d,
                                                            loc.capacity, loc.window)),
                     dtype=torch.uint8, device="cuda")

    def run_loc(r):
        q, kc, vc, ks, vs, pos, _ = sets[r % 4]
        g4.decode_fp8(q, kc, vc, ks, vs, pos, loc.window, loc.theta, loc.p, out=out, workspace=ws)

    ms = _event_time(torch, run_loc, reps)
    byts = loc.B * loc.Hkv * loc.capacity * loc.d * 2 + sets[0][0].numel() * (2 + 4)
    res["decode_fp8_local"] = {"us": ms * 1e3, "GBps": byts / ms / 1e6,
                               "frac_hbm": byts / ms / 1e6 / HBM_PEAK_GBS,
                               "tok_per_s": loc.B / ms * 1e3}
    del sets, out, ws
    glo = inputs.DECODE_GLOBAL
    q, kc, _, ks, _, pos, lengths = inputs.decode_inputs_fp8(glo, 71, 0, "cuda")
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    ws = torch.empty(max(16, g4.decode_fp8_workspace_bytes(glo.B, 1, glo.Hq, glo.Hkv, glo.d,
                                                            glo.capacity, 0)),
                     dtype=torch.uint8, device="cuda")
    ms = _event_time(torch, lambda r: g4.decode_fp8(q, kc, None, ks, None, pos, 0, glo.theta,
                                                    glo.p, out=out, workspace=ws), reps)
    byts = int(lengths.sum()) * glo.Hkv * glo.d + q.numel() * (2 + 4)
    res["decode_fp8_global"] = {"us": ms * 1e3, "GBps": byts / ms / 1e6,
                                "frac_hbm": byts / ms / 1e6 / HBM_PEAK_GBS,
                                "tok_per_s": glo.B / ms * 1e3}
    del q, kc, out, ws
    gl = inputs.global_(1, inputs.GROUP_S)
    k = inputs.randn((gl.B, gl.S, gl.Hkv, gl.d), 6201, torch.bfloat16, "cuda")
    p = inputs.positions(gl.B, gl.S, "cuda")
    ks = inputs.kv_scales(gl.Hkv, 6202, "cuda", 0.01, 0.02)
    kc = torch.empty((gl.B, gl.Hkv, gl.S, gl.d), dtype=torch.uint8, device="cuda")
    ms = _event_time(torch, lambda r: g4.fill_cache_fp8(k, None, p, kc, None, 0, ks), reps)
    byts = k.numel() * (2 + 1) + p.numel() * 4
    res["fill_cache_fp8_global_s262144"] = {"us": ms * 1e3, "GBps": byts / ms / 1e6,
                                            "frac_hbm": byts / ms / 1e6 / HBM_PEAK_GBS}
    del k, p, kc
    return res


def time_vision(g4, inputs, torch, reps=5):
    """Vision-encoder attention (2D RoPE, no causal mask) at the budget-280
    batch (4 images up to 2520 patches) and one budget-1120 image (10080
    patches).  FLOPs count 4*d per (valid query, valid key) pair per head."""
    res = {}
    for name, layer in (("budget280_b4", inputs.VISION_280), ("budget1120_b1", inputs.VISION_1120)):
        q, k, v, pos2, lengths = inputs.vision_inputs(layer, 9, torch.bfloat16, "cuda")
        out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
        ws = torch.empty(g4.prefill_workspace_bytes(layer.B, layer.S, layer.Hkv, layer.d, 1.0),
                         dtype=torch.uint8, device="cuda")
        ms = _event_time(torch, lambda r: g4.vision_prefill(q, k, v, pos2, layer.theta,
                                                            lengths=lengths, out=out,
                                                            workspace=ws), reps)
        flops = sum((w * h) ** 2 for w, h in layer.grids) * layer.Hq * 4 * layer.d
        res[name] = {"ms": ms, "tflops": flops / ms / 1e9,
                     "frac_mfma": flops / ms / 1e9 / MFMA_BF16_PEAK_TFLOPS,
                     "patches": [w * h for w, h in layer.grids]}
        del q, k, v, pos2, lengths, out, ws
    return res


# Full-depth attention schedules of the pages' model sizes ("Guia visual do
# Gemma 4", section "Intercalacao de camadas de atencao": window 512 for
# E2B/E4B and 1024 for the large models, 4:1 interleave for E2B and 5:1 for
# the others, the last layer always global; layer counts 35 (E2B), 42 (E4B)
# and 60 (31B) from the same page and the techtoday page; context 128K for the
# small models and 256K for the medium ones: "Visao geral do modelo Gemma 4",
# section "Recursos").  The pages give no head counts for these sizes, so the
# layers use this block's head geometry.
SCHEDULES = {
    "e2b_128k": dict(layers=35, ratio=4, window=512, S=131072),
    "e4b_128k": dict(layers=42, ratio=5, window=512, S=131072),
    "31b_256k": dict(layers=60, ratio=5, window=1024, S=262144),
}


def time_schedules(g4, inputs, torch, reps=2, dec_reps=4):
    """Prefill and one batch-64 decode step of every layer of each schedule.
    Every layer kind is timed at the schedule's own geometry: the local prefill
    at its window and context, the global prefill at the context, the local
    decode over full rings of `window` slots, and the global decode over
    linear K=V caches of the context's length with cache lengths uniform in
    [4096, context].  Layers of one kind at one geometry cost the same, so a
    stack's time is the per-layer time times its layer count."""
    res, pre_cache, dec_cache = {}, {}, {}

    def prefill_ms(layer):
        key = (layer.kind, layer.S, layer.window)
        if key not in pre_cache:
            q, k, v, pos = inputs.prefill_inputs(layer, 80, 0, torch.bfloat16, "cuda")
            out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
            ws = torch.empty(max(16, g4.prefill_workspace_bytes(layer.B, layer.S, layer.Hkv,
                                                                layer.d, layer.p)),
                             dtype=torch.uint8, device="cuda")
            if layer.kind == "global":
                f = lambda r: g4.global_prefill(q, k, pos, 0, layer.theta, layer.p, out=out,
                                                workspace=ws)
            else:
                f = lambda r: g4.local_prefill(q, k, v, pos, layer.window, layer.theta, layer.p,
                                               out=out, workspace=ws)
            pre_cache[key] = _event_time(torch, f, reps)
            del q, k, v, pos, out, ws
        return pre_cache[key]

    def decode_us(layer, lengths):
        """(us per call, algorithmic bytes) of one batch-64 decode launch; ring
        layers rotate over two cache copies (distinct layers' caches)."""
        key = (layer.kind, layer.capacity, layer.window)
        if key not in dec_cache:
            ncopy = 2 if layer.window > 0 else 1
            sets = [inputs.decode_inputs(layer, 82 + i, 0, torch.bfloat16, "cuda", lengths)
                    for i in range(ncopy)]
            out = torch.empty(sets[0][0].shape, dtype=torch.float32, device="cuda")
            ws = torch.empty(max(16, g4.decode_workspace_bytes(layer.B, layer.Hq, layer.Hkv,
                                                               layer.d, layer.capacity,
                                                               layer.window)),
                             dtype=torch.uint8, device="cuda")

            def f(r):
                q, kc, vc, pos, _ = sets[r % ncopy]
                g4.decode(q, kc, vc, pos, layer.window, layer.theta, layer.p, out=out,
                          workspace=ws)
            ms = _event_time(torch, f, dec_reps)
            _, byts = decode_cost(layer, lengths)
            dec_cache[key] = (ms * 1e3, byts)
            del sets, out, ws
            torch.cuda.empty_cache()
        return dec_cache[key]

    for name, sc in SCHEDULES.items():
        n_glob = sc["layers"] // (sc["ratio"] + 1)
        n_loc = sc["layers"] - n_glob
        loc = inputs.local(1, sc["S"], window=sc["window"])
        glo = inputs.global_(1, sc["S"])
        t_pre = n_loc * prefill_ms(loc) + n_glob * prefill_ms(glo)
        fl = n_loc * prefill_flops(loc) + n_glob * prefill_flops(glo)
        entry = {"layers": sc["layers"], "local_layers": n_loc, "global_layers": n_glob,
                 "window": sc["window"], "context": sc["S"], "prefill_ms": t_pre,
                 "prefill_tflops": fl / t_pre / 1e9}
        b = inputs.DECODE_LOCAL.B
        dl = inputs.DecodeLayer("local", b, 16, 8, 256, sc["window"], sc["window"],
                                inputs.LOCAL_THETA, 1.0)
        dg = inputs.DecodeLayer("global", b, 16, 2, 512, sc["S"], 0, inputs.GLOBAL_THETA, 0.25)
        lengths = inputs.decode_lengths(b, 4009, 4096, sc["S"])
        tl, bl = decode_us(dl, lengths)
        tg, bg = decode_us(dg, lengths)
        step = n_loc * tl + n_glob * tg
        entry.update({"decode_step_us": step, "decode_tok_per_s": b / step * 1e6,
                      "decode_local_us": tl, "decode_local_frac_hbm": bl / tl / 1e3 / HBM_PEAK_GBS,
                      "decode_global_us": tg,
                      "decode_global_frac_hbm": bg / tg / 1e3 / HBM_PEAK_GBS,
                      "decode_global_mean_len": float(lengths.double().mean()),
                      "decode_note": f"batch {b}; local ring of {sc['window']} slots, global "
                                     f"K=V cache of {sc['S']} rows, lengths U[4096, {sc['S']}]; "
                                     f"each kind timed at this geometry"})
        res[name] = entry
    return res


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(args, loc, glo, L0, G0, Lout, Gout, step_prefill_flops):
    """The fp64 oracle, untuned, on a bounded sample of rows of the same
    workload (first local layer and the global layer), on every host thread
    and then on one; also reports the parity of those rows against the GPU
    outputs of the run.  The rates are measured over the row sample; the time
    of the whole prefill group is extrapolated from them by the ratio of
    algorithmic FLOPs."""
    import numpy as np
    import torch

    import oracle
    from tests.helpers import to_oracle

    S = loc.S
    threads = oracle.threads()
    qg, kvg, _, posg = G0
    ql, kl, vl, posl = L0
    t0 = time.time()
    kvg_h, kl_h, vl_h = to_oracle(kvg), to_oracle(kl), to_oracle(vl)
    posg_h, posl_h = posg.cpu().numpy(), posl.cpu().numpy()
    qg_h, ql_h = to_oracle(qg), to_oracle(ql)
    print(f"# host copies {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    def run(rows_g, rows_l):
        t = time.time()
        og = oracle.prefill(qg_h, kvg_h, kvg_h, posg_h, 0, glo.theta, glo.p, rows=rows_g)
        ol = oracle.prefill(ql_h, kl_h, vl_h, posl_h, loc.window, loc.theta, loc.p, rows=rows_l)
        return time.time() - t, og, ol

    def flops(rows_g, rows_l):
        f = sum(4.0 * glo.d * glo.Hq * (int(r) + 1) for r in rows_g)
        f += sum(4.0 * loc.d * loc.Hq * min(int(r) + 1, loc.window) for r in rows_l)
        return f

    rng = np.random.default_rng(7)
    # calibration run, then a sample sized for about args.cpu_seconds of oracle time;
    # global rows (2^18 keys each) dominate, local rows ride along 8 per global row
    n_g = 4
    for _ in range(5):
        rows_g = np.unique(np.concatenate([[0, 1, S - 1], rng.choice(S, n_g, replace=False)]))
        rows_l = np.unique(np.concatenate([[0, 1, 1023, 1024, S - 1],
                                           rng.choice(S, 8 * n_g, replace=False)]))
        t, og, ol = run(rows_g, rows_l)
        if t >= 0.6 * args.cpu_seconds or n_g >= 4096:
            break
        n_g = max(n_g + 1, min(4096, int(n_g * args.cpu_seconds / max(t, 1e-3))))
    f = flops(rows_g, rows_l)
    print(f"# oracle sample on {threads} threads: {t:.1f}s", file=sys.stderr, flush=True)
    got_g = Gout.view(S, glo.Hq, glo.d)[torch.as_tensor(rows_g, device=Gout.device)]
    got_l = Lout.view(S, loc.Hq, loc.d)[torch.as_tensor(rows_l, device=Lout.device)]
    eg = np.abs(got_g.double().cpu().numpy() - og)
    el = np.abs(got_l.double().cpu().numpy() - ol)
    # one thread: a smaller sample of the same kinds of rows, about a third of
    # the CPU seconds
    oracle.set_threads(1)
    try:
        n1 = max(1, int(len(rows_g) * args.cpu_seconds / 3 / max(t * threads, 1e-3)))
        r1g = rng.choice(S, n1, replace=False)
        r1l = rng.choice(S, 8 * n1, replace=False)
        t1, _, _ = run(r1g, r1l)
        f1 = flops(r1g, r1l)
    finally:
        oracle.set_threads(threads)
    print(f"# oracle sample on 1 thread: {t1:.1f}s", file=sys.stderr, flush=True)
    rate, rate1 = f / t, f1 / t1
    return {"value": rate / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(), "seconds": t,
            "sample": f"row sample: {len(rows_g)} query rows (all 16 heads) of the global layer "
                      f"and {len(rows_l)} rows of the first local layer, S={S}; fp64, OpenMP on "
                      f"{threads} threads; the rate is the sample's algorithmic FLOPs over its "
                      f"time",
            "one_thread": {"value": rate1 / 1e12, "unit": "TFLOP/s", "seconds": t1,
                           "sample": f"{len(r1g)} global rows and {len(r1l)} local rows"},
            "extrapolated_group_prefill_s": step_prefill_flops / rate,
            "extrapolated_group_prefill_s_one_thread": step_prefill_flops / rate1,
            "extrapolation": "whole prefill of the 5:1 group (5 local + 1 global layer) at the "
                             "sample's rate, scaled by algorithmic FLOPs; not measured",
            "parity_sample": {"global_max_abs": float(eg.max()), "global_mean_abs": float(eg.mean()),
                              "local_max_abs": float(el.max()), "local_mean_abs": float(el.mean())}}


if __name__ == "__main__":
    main()
