"""Benchmark: steady-state decode steps/s of the fused importance-aware KV step.

Headline workload ``headkv32k``: batch 4, 32 q / 8 KV heads, D = 128, bf16, a
32768-token prefilled cache per (batch, KV head), per-KV-head budgets from one
Dirichlet(0.5) draw (total about 8 * 2048, clamped to [64, 8192]), 4 sinks,
128 recent.  Every layer copy first takes the compression step (32769 -> its
budget); the timed region is K steady decode steps (attend over budget + 1
tokens, accumulate, evict one), captured in one HIP graph.

Cold measurement: the steps cycle over L independent layer copies (like
successive layers of a model), so the ~34 MB a step touches is not resident
in the 256 MB Infinity Cache when the step starts.  "warm" repeats steps on
one layer copy (its rows stay resident).

Besides the headline the JSON line carries:
  roofline   the whole step's algorithmic bytes / its graph-timed duration
             against 8 TB/s; the attention launch (HIP events per launch) as
             roofline.attend; roofline.floor: a plain cold read of the same
             K and V rows in the cache layout in one launch (the streaming
             floor), and the cost of one dependent empty launch;
  whole_run  the workload as the pages run it: the compression step plus its
             steady steps (64 steps in all for headkv32k);
  workloads  the same measurement on the other seeded workloads (llama8b,
             longctx128k budgeted and full attention, twostage);
  budget_sweep  llama8b at budgets 128 ... 4096, and Stage II (twostage) at 1024 ... 4096;
  cpu_baseline  the CPU oracle on a bounded sample of the headline workload.

--workload selects another headline workload with the same protocol:
llama8b, longctx128k, longctx128k_full (no eviction), twostage (Stage II,
exact top-k_T V side), hikv_dualbank (HiKV's dual-bank Stage I; also times
the bank initialisation's prompt scores), hikv_hier (dual bank plus HiKV's
chunked Stage II V side), tiny.  --accumulate overrides the importance
accumulation (H2O probabilities, HiKV's recent window, Kelle's logits);
--prefill times the prompt scores on any workload; --quick leaves out the
other workloads and the sweep.

Prints one JSON line (stdout).  Diagnostics go to stderr.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 matrix-core peak of MI355X
FP32_PEAK_TFLOPS = 157.3         # fp32 vector peak
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "hbm_traffic_headkv32k.md")
KERNEL_SOURCES = ("importance_aware_kv_amd/csrc/step.hip", "importance_aware_kv_amd/csrc/hikv_common.h",
                  "importance_aware_kv_amd/csrc/hikv_dev.h", "importance_aware_kv_amd/csrc/hikv_block.h")
SWEEP_BUDGETS = (128, 256, 512, 1024, 2048, 3072, 4096)
STAGE2_BUDGETS = (1024, 2048, 3072, 4096)
SUB_WORKLOADS = ("llama8b", "longctx128k", "longctx128k_full", "twostage")


def measured_traffic():
    """HBM bytes per steady step (and per attention launch) of the headline
    workload from the committed counter record, or None when the kernel
    sources changed since the counters were taken."""
    import hashlib
    try:
        text = open(TRAFFIC_RECORD).read()
    except OSError:
        return None
    tag = "<!-- traffic: "
    if tag not in text:
        return None
    rec = json.loads(text.split(tag, 1)[1].split(" -->", 1)[0])
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return rec if h.hexdigest() == rec["sources_sha256"] else None


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def pct(xs, q):
    import numpy as np
    return float(np.percentile(np.asarray(xs, dtype=np.float64), q))


def host_cpu():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count()
    return model, os.cpu_count(), avail


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=512)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--layers", type=int, default=16)
    ap.add_argument("--workload", default="headkv32k")
    ap.add_argument("--prefill", action="store_true",
                    help="also time hikv_prefill_scores over every prompt query (on by default for the "
                         "HiKV dual-bank workloads, with the recent bank's window)")
    ap.add_argument("--accumulate", choices=["all", "recent", "logit"], default=None,
                    help="override the workload's importance accumulation (H2O probabilities, HiKV's "
                         "recent window only, Kelle's pre-softmax logits)")
    ap.add_argument("--budget", type=int, default=None,
                    help="one budget for every unit in place of the workload's own (a measurement at another size)")
    ap.add_argument("--quick", action="store_true", help="the headline workload only (no sub-workloads, no sweep)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-hint", action="store_true", help="do not pass host lengths")
    ap.add_argument("--block-tokens", type=int, default=0,
                    help="evict whole blocks of this many positions (policy block_tokens; 0: single tokens)")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="after the run, copy this many bytes device-to-device 4 times (a plain copy "
                         "kernel of known size, for calibrating memory counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (this path has no "
              "multi-GPU mode).", file=sys.stderr)
        sys.exit(2)

    import torch

    from importance_aware_kv_amd import hikv as H

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    H.lib()  # raises when the HIP library is missing: no fallback
    H.calib_lib()
    dev_name = torch.cuda.get_device_name(0)
    log(f"[bench] device {dev_name}")
    t_all = time.time()

    acc = None if args.accumulate is None else {"all": H.HIKV_ACC_ALL, "recent": H.HIKV_ACC_RECENT,
                                                "logit": H.HIKV_ACC_LOGIT}[args.accumulate]
    head = run_workload(args.workload, steps=args.steps, warmup=args.warmup, layers=args.layers,
                        hint=not args.no_hint, accumulate=acc, prefill=args.prefill, detail=True,
                        keep_data=not args.no_cpu_baseline, block_tokens=args.block_tokens, budget_all=args.budget)
    launch_us = launch_floor_us()
    log(f"[bench] dependent empty launch in a graph: {launch_us:.2f} us")

    if args.copy_bytes > 0:
        n = args.copy_bytes // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy calibration: 4 x {n * 4} bytes device-to-device")
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(head["w"], head["data"], args.cpu_seconds, args.block_tokens)
        log(f"[bench] cpu oracle: {cpu}")
    head.pop("data", None)
    w = head.pop("w")

    subs, sweep = None, None
    if not args.quick and args.workload == "headkv32k" and not args.block_tokens and args.budget is None:
        subs = {}
        for name in SUB_WORKLOADS:
            r = run_workload(name, steps=128, warmup=16, layers=args.layers, hint=not args.no_hint, detail=False)
            r.pop("w")
            subs[name] = r
        # block-granular eviction (blocks of 16 positions) on llama8b's shape
        r = run_workload("llama8b", steps=128, warmup=16, layers=args.layers, detail=False, block_tokens=16)
        r.pop("w")
        r["what"] = ("llama8b with whole blocks of 16 positions evicted (policy block_tokens 16; no length "
                     "hints: the device's plan); bytes counted with the single-token lengths, within a "
                     "block of the device's")
        subs["llama8b_blocks16"] = r
        pts = []
        for b in SWEEP_BUDGETS:
            r = run_workload("llama8b", steps=128, warmup=16, layers=args.layers, hint=not args.no_hint,
                             budget_all=b, detail=False)
            r.pop("w")
            pts.append({"budget": b, **{k: r[k] for k in ("us_per_step", "steps_per_s", "achieved_gbs", "frac",
                                                        "bytes_per_step", "compression_step_us")}})
        sweep = {"workload": "llama8b (batch 8, 32 q / 8 KV heads, D 128, bf16, 8192-token prefill, sinks 4, "
                             "recent 128), one budget for every unit", "points": pts}
        # Stage II (r = 32, k_T = 256) on the same shape at the larger budgets
        pts2 = []
        for b in STAGE2_BUDGETS:
            r = run_workload("twostage", steps=128, warmup=16, layers=args.layers, hint=not args.no_hint,
                             budget_all=b, detail=False)
            r.pop("w")
            pts2.append({"budget": b, **{k: r[k] for k in ("us_per_step", "steps_per_s", "bytes_per_step",
                                                         "compression_step_us")}})
        sweep["stage2"] = {"workload": "twostage (the same shape; Stage II, r = 32 channels, k_T = 256 tokens)",
                           "bytes": "Stage I's algorithmic bytes of the same budget", "points": pts2}

    tr = measured_traffic() if args.workload == "headkv32k" and not args.block_tokens and args.budget is None else None
    line = {
        "metric": "decode steps/s and achieved KV HBM GB/s (fraction of 8 TB/s) per budget",
        "value": round(head["steps_per_s"], 1),
        "unit": "decode steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["us_per_step"] / 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.el == 2 else "f32",
        "data": "synthetic",
        "config": {
            "workload": head["text"],
            "global_batch": w.batch,
            "seq_len": w.ctx,
            "layers_cycled": args.layers,
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": head["achieved_gbs"],
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": head["frac"],
            "traffic": None if tr is None else tr["step_bytes"],
            "scope": "the whole steady step (every launch of it), graph-timed, cold",
            "bytes_per_step": head["bytes_per_step"],
            "us_per_step": head["us_per_step"],
            "attend": {**head["attend"], "traffic": None if tr is None else tr["attend_bytes"]},
            "floor": head["floor"],
            "launch_floor_us": round(launch_us, 3),
        },
        "step_us_p50": head["step_us_p50"],
        "step_us_p90": head["step_us_p90"],
        "warm": head["warm"],
        ("first_step_us" if w.name.endswith("_full") else "compression_step_us"):
            head["first_step_us" if w.name.endswith("_full") else "compression_step_us"],
        "compression": head["compression"],
        "whole_run": head["whole_run"],
        "workloads": subs,
        "budget_sweep": sweep,
        "cpu_baseline": cpu,
        "wall_s": round(time.time() - t_all, 1),
    }
    if "prefill_scores" in head:
        line["prefill_scores"] = head["prefill_scores"]
    print(json.dumps(line), flush=True)


def launch_floor_us(n=256):
    """One dependent empty launch, from n of them back to back in a HIP graph."""
    import torch

    from importance_aware_kv_amd import hikv as H
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        H.check(H.hikv_calib_empty(4, s), "hikv_calib_empty")
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            H.check(H.hikv_calib_empty(n, s), "hikv_calib_empty")
        torch.cuda.synchronize()
        g.replay()  # first replay uploads the graph
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        g.replay()
        e1.record(s)
        torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / n


def stream_floor(caches, lens, rb, log, what):
    """The streaming floor: a plain read of rows [0, lens[u]) of every unit's K
    and V (one launch, cycling over the layer copies so that every launch
    reads cold rows), for a few tile counts; the fastest is the floor."""
    import numpy as np
    import torch

    from importance_aware_kv_amd import hikv as H
    lens = np.asarray(lens, dtype=np.int64).reshape(-1)
    total = int(lens.sum())
    nbytes = total * 2 * rb
    cap = caches[0].shape.capacity
    best = None
    for target in (512, 1024, 2048, 4096):
        T = max(16, -(-total // target))
        tl = [(u, t0, min(int(lens[u]), t0 + T)) for u in range(len(lens)) for t0 in range(0, int(lens[u]), T)]
        tiles = torch.tensor(tl, dtype=torch.int32, device="cuda")
        sink = torch.zeros(len(tl), dtype=torch.int32, device="cuda")
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in caches]
        for e_a, e_b in evs:
            e_a.record()
            e_b.record()
        torch.cuda.synchronize()
        torch.cuda._sleep(50_000_000)
        for c, (e_a, e_b) in zip(caches, evs):
            H.check(H.hikv_calib_stream(c.k, c.v, cap, rb, tiles, sink, e_a.cuda_event, e_b.cuda_event),
                    "hikv_calib_stream")
        torch.cuda.synchronize()
        us = [e_a.elapsed_time(e_b) * 1e3 for e_a, e_b in evs]
        mean = sum(us) / len(us)
        if best is None or mean < best["us"]:
            best = {"us": round(mean, 3), "tiles": len(tl)}
    gbs = nbytes / (best["us"] * 1e-6) / 1e9
    best.update({"bytes": nbytes, "achieved": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
                 "what": f"plain cold read of {what} in the cache layout, one launch of 16-byte loads "
                         "(HIP events; the fastest of 512-4096 equal tiles)"})
    log(f"[bench] streaming floor ({what}): {best['us']:.2f} us for {nbytes / 1e6:.2f} MB -> {gbs:.0f} GB/s "
        f"({gbs / HBM_PEAK_GBS:.1%}), {best['tiles']} tiles")
    return best


def run_workload(name, *, steps, warmup, layers, hint=True, budget_all=None, accumulate=None, prefill=False,
                 detail=False, keep_data=False, block_tokens=0):
    """Compression step and cold steady steps of one seeded workload on `layers`
    layer copies (the timed steps: one HIP graph).  With detail: the attention
    launch timed per launch with HIP events, per-step times, warm steps, the
    streaming floors and the prompt scores where the workload asks for them."""
    import numpy as np
    import torch

    from importance_aware_kv_amd import bytes_model as BM
    from importance_aware_kv_amd import hikv as H
    from importance_aware_kv_amd import workloads as W

    n_inputs = 256
    full = name.endswith("_full")
    base_name = name[:-5] if full else name
    own_steps = W.workload(base_name, full=full).steps  # the workload's own step count
    w = W.workload(base_name, steps=n_inputs, full=full)
    if budget_all is not None:
        w.budget_all, w.budgets = budget_all, None
    if accumulate is not None:
        w.accumulate = accumulate
    warm_steps = steps if detail else 0
    # compression step + warm-up + timed steps (+ the same number again for
    # the per-launch timing replay) over the copies, + warm steps on copy 0
    per_layer_steps = 1 + (warmup + (2 if detail else 1) * steps + (16 if detail else 0) + layers - 1) // layers \
        + warm_steps
    w.capacity = w.ctx + per_layer_steps + 1
    if full:  # full attention: the budget is the whole capacity, nothing is ever evicted
        w.budget_all = w.capacity
    stage2 = w.stage2_channels > 0
    # Stage I and, for bf16 K with D = 128, Stage II with the exact top-k_T V
    # side run in two launches and leave a one-token eviction pending; the
    # other Stage II variants evict in place
    pending_path = (not stage2) or (w.stage2_v == H.HIKV_S2V_TOPK and w.el == 2 and w.head_dim == 128
                                    and w.stage2_tokens <= 2048)
    if block_tokens:
        # Whole blocks leave lengths the host cannot foresee (they depend on
        # the device's importance): no length hints, no pending eviction, and
        # the host's lengths below (for the byte count) are the single-token
        # ones, within a block of the device's.
        hint, pending_path = False, False
    t0 = time.time()
    d = W.generate(w)
    tag = (name if budget_all is None else f"{name}@{budget_all}") + (f"/blocks{block_tokens}" if block_tokens else "")
    log(f"[bench] {tag}: inputs generated in {time.time() - t0:.1f}s")
    B, Hq, Hkv, D = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim
    budget = w.budget_array()
    rb = D * w.el

    caches = [H.DeviceCache(d, Hq)]
    for _ in range(1, layers):
        caches.append(caches[0].clone())
    budget_t = torch.from_numpy(budget).cuda()
    b_arr, b_all = (budget_t, 0) if w.budgets is not None else (None, w.budget_all)
    pol = H.make_policy(b_arr, b_all, w.n_sink, w.n_recent, w.stage2_channels, w.stage2_tokens,
                        accumulate=w.accumulate, stage2_v=w.stage2_v, block_tokens=block_tokens)
    # One workspace (scratch) serves every layer copy, as it would every layer
    # of a model; each cache carries its own pending-eviction state.
    ws = H.workspace(caches[0].shape, pol)

    def device_status(what):
        H.check(H.hikv_device_status(ws), what)

    # The caller's host copy of every layer's lengths (a serving loop tracks
    # them anyway); passed as the length hint so the tile plan is made on the
    # host.  hint=False measures the device-derived plan instead.
    host_len = [np.full((B, Hkv), w.ctx, dtype=np.int32) for _ in range(layers)]
    q_all = H.to_device(d["q"])
    kn_all = H.to_device(d["k_new"])
    vn_all = H.to_device(d["v_new"])
    pos_all = torch.from_numpy(
        (w.ctx + np.arange(per_layer_steps + 1, dtype=np.int32))[:, None].repeat(B, 1).copy()).cuda()
    out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    layer_step = [0] * layers
    live_log, moves_log = [], []  # tokens attended / units moving rows per step, in launch order

    def step(li, events=None):
        c = caches[li]
        n = layer_step[li]
        layer_step[li] += 1
        # live tokens of the step (a pending eviction's dead slot is not one)
        live_now = host_len[li] + 1 - ((host_len[li] > budget) & pending_path)
        live_log.append(int(live_now.sum()))
        moves_log.append(int((live_now > budget).sum()))
        p = pol
        if hint:
            p = H.make_policy(b_arr, b_all, w.n_sink, w.n_recent, w.stage2_channels, w.stage2_tokens,
                              budget_hint=budget if b_arr is not None else None,
                              len_hint=host_len[li], accumulate=w.accumulate, stage2_v=w.stage2_v, block_tokens=block_tokens)
        dbg = None
        if events is not None:
            dbg = H.hikv_debug(None, None, None, events[0].cuda_event, events[1].cuda_event)
        code = H.hikv_decode_step(c.shape, c.cache, p, q_all[n % n_inputs], kn_all[n % n_inputs],
                                  vn_all[n % n_inputs], pos_all[n], out, ws, debug=dbg)
        if code != 0:
            raise RuntimeError(f"hikv_decode_step: {H.status_string(code)}")
        # The caller's copy of len[] after the step: a unit over its budget by one
        # keeps budget + 1 slots with that eviction pending (the next step writes
        # its new token into the dead slot); a bulk cut leaves exactly the budget.
        old = host_len[li]
        if not pending_path:
            host_len[li] = np.minimum(old + 1, budget).astype(np.int32)
        else:
            pending = old > budget
            live = old + 1 - pending
            host_len[li] = np.where(live > budget + 1, budget, np.where(pending, old, old + 1)).astype(np.int32)

    res = {"w": w, "text": workload_text(w, budget, full)
           + (f", whole blocks of {block_tokens} positions evicted" if block_tokens else "")}
    stream = torch.cuda.current_stream()
    if detail and (prefill or w.accumulate == H.HIKV_ACC_RECENT) and not full:
        res["prefill_scores"] = measure_prefill(w, caches[0], budget, log)
    comp_floor = None
    if detail:
        comp_floor = stream_floor(caches, host_len[0], rb, log, "every prefilled K and V row")

    # Compression step of every layer copy (ctx + 1 tokens -> budget), queued
    # behind a GPU-side wait so that the steps run back to back.
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(100_000_000)
    e0.record(stream)
    for li in range(layers):
        step(li)
    e1.record(stream)
    torch.cuda.synchronize()
    comp_us = e0.elapsed_time(e1) * 1e3 / layers
    device_status("device status after compression")
    live_after = np.minimum(w.ctx + 1, budget)
    if not block_tokens:
        assert np.array_equal(caches[0].len.cpu().numpy(), live_after), "compression did not reach the budgets"
    # (the rows the cut relocates are not counted: the bytes are what any
    # layout must move, every live row read once and the importance updated)
    comp_bytes = BM.decode_step_bytes(B, Hq, Hkv, D, w.el, np.full((B, Hkv), w.ctx + 1), 0)
    log(f"[bench] {tag} {'first' if full else 'compression'} step: {comp_us:.1f} us/layer "
        f"({comp_bytes / comp_us / 1e3:.0f} GB/s algorithmic)")

    # Warm-up steady steps, eager.
    for i in range(warmup):
        step(i % layers)
    torch.cuda.synchronize()
    device_status("device status after warm-up")

    # Timed steady steps: one HIP graph, replayed once.
    mark = len(live_log)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            step((warmup + i) % layers)
    torch.cuda.synchronize()
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_start.record()
    g.replay()
    t_end.record()
    torch.cuda.synchronize()
    us_step = t_start.elapsed_time(t_end) * 1e3 / steps
    device_status("device status after timed steps")
    del g
    # bytes of the average timed step (every step is alike in the budgeted steady
    # state; a full-attention step attends one token more than the one before)
    live_avg = sum(live_log[mark:]) / steps
    moves_avg = sum(moves_log[mark:]) / steps
    step_bytes = int(BM.decode_step_bytes(B, Hq, Hkv, D, w.el, [0], 0) + live_avg * (2 * rb + 12)
                     + moves_avg * 2 * (2 * rb + 8))
    gbs = step_bytes / (us_step * 1e-6) / 1e9
    log(f"[bench] {tag} steady step: {us_step:.2f} us, {1e6 / us_step:.0f} steps/s, {step_bytes / 1e6:.2f} MB/step "
        f"algorithmic -> {gbs:.0f} GB/s ({gbs / HBM_PEAK_GBS:.1%} of 8 TB/s)")
    res.update({
        "us_per_step": round(us_step, 3), "steps_per_s": round(1e6 / us_step, 1),
        "bytes_per_step": step_bytes, "achieved_gbs": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
        ("first_step_us" if full else "compression_step_us"): round(comp_us, 2),
    })
    own_bytes = comp_bytes + (own_steps - 1) * step_bytes
    own_us = comp_us + (own_steps - 1) * us_step
    res["whole_run"] = {"steps": own_steps, "us": round(own_us, 1), "bytes": own_bytes,
                        "achieved_gbs": round(own_bytes / (own_us * 1e-6) / 1e9, 1),
                        "frac": round(own_bytes / (own_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                        "what": f"the {'first' if full else 'compression'} step and {own_steps - 1} steady steps "
                                "(cold), their algorithmic bytes over their summed times"}
    res["compression"] = {"us": round(comp_us, 2), "bytes": comp_bytes,
                          "achieved_gbs": round(comp_bytes / (comp_us * 1e-6) / 1e9, 1), "floor": comp_floor}

    if detail:
        # The attention launch: the same steps run once more, launched eagerly
        # and back to back behind a GPU-side wait, with a pair of HIP events
        # around every attention launch (recorded by the dispatch itself, on
        # the stream that launch uses).
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for e_a, e_b in evs:
            e_a.record(stream)
            e_b.record(stream)
        torch.cuda.synchronize()
        base2 = warmup + steps
        torch.cuda._sleep(500_000_000)
        t_enq = time.perf_counter()
        for i in range(steps):
            step((base2 + i) % layers, events=evs[i])
        t_enq = time.perf_counter() - t_enq
        torch.cuda.synchronize()
        log(f"[bench] timing replay: {steps} steps enqueued in {t_enq * 1e3:.1f} ms behind a GPU wait")
        device_status("device status after the timing replay")
        att = [e_a.elapsed_time(e_b) * 1e3 for e_a, e_b in evs]
        attend_us = sum(att) / steps
        live_rep = sum(live_log[-steps:]) / steps
        if stage2:  # the reduced-channel logits pass reads every live K row whole, and q
            attend_bytes = int(live_rep * D * w.el + B * Hq * D * w.el)
        else:
            attend_bytes = int(BM.attend_bytes(B, Hq, Hkv, D, w.el, [0]) + live_rep * 2 * rb)
        attend_gbs = attend_bytes / (attend_us * 1e-6) / 1e9
        log(f"[bench] attention launch: {attend_us:.2f} us (p50 {pct(att, 50):.2f}, p90 {pct(att, 90):.2f}), "
            f"{attend_bytes / 1e6:.2f} MB algorithmic -> {attend_gbs:.0f} GB/s ({attend_gbs / HBM_PEAK_GBS:.1%})")
        res["attend"] = {"kernel": kernel_text(w), "achieved": round(attend_gbs, 1),
                         "frac": round(attend_gbs / HBM_PEAK_GBS, 4), "bytes_per_launch": attend_bytes,
                         "us_per_launch": round(attend_us, 3), "p50_us": round(pct(att, 50), 3),
                         "p90_us": round(pct(att, 90), 3)}
        # Spread of the step time: a graph of 16 cold steps replayed 32 times,
        # each replay timed (events outside the graph): p50 / p90 of the
        # replays' per-step means.  (Budgeted steady state only: the graph
        # carries the steps' lengths, which full attention grows every step.)
        res["step_us_p50"] = res["step_us_p90"] = None
        if not full:
            # (each replay appends tokens at positions one past the previous
            # replay's: the graph reads them from rows of pos_all, bumped between
            # replays, so that positions stay distinct)
            rows = []
            for i in range(16):
                li = i % layers
                rows.append(layer_step[li] + sum(1 for k in range(i) if k % layers == li))
            rows_t = torch.tensor(rows, dtype=torch.long, device="cuda")
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(16):
                    step(i % layers)
            torch.cuda.synchronize()
            reps = []
            for _ in range(32):
                pos_all[rows_t] += 1
                t_start.record()
                g.replay()
                t_end.record()
                torch.cuda.synchronize()
                reps.append(t_start.elapsed_time(t_end) * 1e3 / 16)
            device_status("device status after the replays")
            del g
            pos_all[min(rows) + 1:] += 32  # later steps stay past the replayed positions
            res["step_us_p50"] = round(pct(reps, 50), 3)
            res["step_us_p90"] = round(pct(reps, 90), 3)
            log(f"[bench] 32 replays of 16 cold steps: per-step p50 {res['step_us_p50']:.2f} us, "
                f"p90 {res['step_us_p90']:.2f} us")
        # The streaming floor of the steady step: the same K and V rows (the
        # live rows of a step), cold.
        res["floor"] = stream_floor(caches, host_len[0], rb, log, "a steady step's K and V rows")
        # Warm: steps repeated on one layer copy (its ~step bytes stay resident).
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(warm_steps):
                step(0)
        torch.cuda.synchronize()
        t_start.record()
        g.replay()
        t_end.record()
        torch.cuda.synchronize()
        device_status("device status after warm steps")
        warm_us = t_start.elapsed_time(t_end) * 1e3 / warm_steps
        del g
        res["warm"] = {"us_per_step": round(warm_us, 3), "steps_per_s": round(1e6 / warm_us, 1),
                       "what": "steady steps repeated on one layer copy (its rows resident in the Infinity "
                               "Cache), graph-timed"}
        log(f"[bench] warm steady step: {warm_us:.2f} us")
    if keep_data:
        res["data"] = d
    del caches, ws, q_all, kn_all, vn_all
    torch.cuda.empty_cache()
    return res


def measure_prefill(w, layer, budget, log, reps=3):
    """Prompt-side scores as HiKV initialises its banks (Sec. III-D): every
    prompt query adds its causal attention row to the tokens within the
    window (the recent bank's size) of it; window 0 (other workloads) counts
    every query.  Timed on a copy of one layer's prefilled cache, with seeded
    synthetic prompt queries; the decode measurement does not use it."""
    import torch

    from importance_aware_kv_amd import hikv as H
    B, Hq, D, L = w.batch, w.n_q_heads, w.head_dim, w.ctx
    c = layer.clone()
    c.imp.zero_()
    window = int(min(w.n_recent, int(budget.min()) - w.n_sink)) if w.accumulate == H.HIKV_ACC_RECENT else 0
    gen = torch.Generator(device="cuda")
    gen.manual_seed(w.seed + 17)
    qdt = torch.bfloat16 if w.el == 2 else torch.float32
    qo = torch.randn((B, Hq, L, D), generator=gen, device="cuda", dtype=torch.float32).to(qdt)
    qpos = torch.arange(L, dtype=torch.int32, device="cuda").repeat(B, 1).contiguous()
    ws = torch.zeros(H.hikv_prefill_workspace_bytes(c.shape, L), dtype=torch.uint8, device="cuda")

    def call():
        H.check(H.hikv_prefill_scores(c.shape, c.cache, qo, qpos, L, window, ws), "hikv_prefill_scores")

    call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        call()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    causal = L * (L + 1) // 2                                   # (query, visible key) pairs
    inwin = causal if window == 0 else window * (window + 1) // 2 + (L - window) * window
    flops = 2 * D * (causal + inwin) * B * Hq                  # q.k for the statistics, again for the sums
    tf = flops / (us * 1e-6) / 1e12
    peak = MFMA_BF16_PEAK_TFLOPS if w.el == 2 else FP32_PEAK_TFLOPS
    log(f"[bench] prefill scores: {L} queries, window {window}: {us:.1f} us, {tf:.1f} TFLOP/s")
    del qo
    return {"queries": L, "window": window, "us": round(us, 1), "bound": "mfma" if w.el == 2 else "alu",
            "achieved": round(tf, 2), "peak": peak, "unit": "TFLOP/s", "frac": round(tf / peak, 4),
            "flops": flops}


def workload_text(w, budget, full):
    heads = f"{w.n_q_heads} q / {w.n_kv_heads} KV heads"
    dt = "bf16" if w.el == 2 else "fp32"
    if full:
        pol = "budget = capacity (full attention, no eviction)"
    elif w.budgets is not None:
        pol = "per-KV-head budgets " + ",".join(map(str, budget[0]))
    else:
        pol = f"budget {w.budget_all}"
    s2 = f", Stage II r = {w.stage2_channels}, k_T = {w.stage2_tokens}" if w.stage2_channels else ""
    if w.stage2_channels and w.stage2_v:
        s2 = (f", Stage II r = {w.stage2_channels} channels and, on the V side, the top {w.stage2_channels} "
              f"entries of P per chunk of {w.head_dim} positions (HiKV)")
    if w.accumulate == 1:
        s2 += ", HiKV dual bank (scores accumulate only in the recent window, frozen outside it)"
    elif w.accumulate == 2:
        s2 += ", Kelle importance (pre-softmax logits summed)"
    return (f"{w.name} {'decode' if full else 'steady state'}: batch {w.batch}, {heads}, D {w.head_dim}, "
            f"{dt} KV, {w.ctx}-token prefill, {pol}, sinks {w.n_sink}, recent {w.n_recent}{s2}")


def kernel_text(w):
    if w.stage2_channels and w.stage2_v == 0 and w.el == 2 and w.head_dim == 128:
        return (f"k_attend_s2<{w.group},2> (Stage II: exact and reduced-channel logits of every live K row on "
                "matrix cores, K only; HIP events per launch)")
    if w.stage2_channels:
        return (f"k_attn_tiles<2,{w.head_dim},{w.group},false,true> (Stage II reduced-channel logits over "
                "every live K row; HIP events per launch)")
    if w.el == 2 and w.head_dim == 128:
        return (f"k_attend_mfma<{w.group},2> (split-K attention over the live K/V rows on matrix cores; "
                "HIP events per launch)")
    return (f"k_attend<{w.el},{w.head_dim},{w.group}> (split-K attention over the live K/V rows; "
            "HIP events per launch)")


def cpu_baseline(w, d, seconds, block_tokens=0):
    """The CPU oracle, as it stands, on a bounded sample of the same workload:
    its own compression step, then steady steps until `seconds` have passed."""
    from oracle import ref
    st = ref.copy_state(d)
    budget = w.budget_array()
    kw = dict(budget=budget, n_sink=w.n_sink, n_recent=w.n_recent, debug=False,
              stage2_channels=w.stage2_channels, stage2_tokens=w.stage2_tokens,
              accumulate=w.accumulate, stage2_v=w.stage2_v, block_tokens=block_tokens)
    tc = time.perf_counter()
    ref.decode_step(st, w.n_q_heads, d["q"][0], d["k_new"][0], d["v_new"][0], d["new_pos"][0], **kw)
    tc = time.perf_counter() - tc
    n = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds and n + 1 < d["q"].shape[0]:
        t = n + 1
        ref.decode_step(st, w.n_q_heads, d["q"][t], d["k_new"][t], d["v_new"][t], d["new_pos"][t], **kw)
        n += 1
    dt = time.perf_counter() - t0
    model, ncpu, avail = host_cpu()
    return {"value": round(n / dt, 2), "unit": "decode steps/s", "cores": 1, "kind": "oracle",
            "cpu_model": model, "nproc": ncpu, "cpus_available": avail,
            "compression_step_s": round(tc, 2),
            "sample": f"{n} steady decode steps of the same workload after the oracle's own "
                      f"compression step ({tc:.1f}s), single-threaded fp64 C++ ({dt:.1f}s)"}


if __name__ == "__main__":
    main()
