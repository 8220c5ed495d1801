"""Benchmark: steady-state decode steps/s of the fused importance-aware KV step.

Workload ``headkv32k``: batch 4, 32 q / 8 KV heads, D = 128, bf16, a
32768-token prefilled cache per (batch, KV head), per-KV-head budgets from one
Dirichlet(0.5) draw (total about 8 * 2048, clamped to [64, 8192]), 4 sinks,
128 recent.  Every layer copy first takes the compression step (32769 -> its
budget); the timed region is K steady decode steps (attend over budget + 1
tokens, accumulate, evict one, compact), captured in one HIP graph.

Cold measurement: the steps cycle over L independent layer copies (like
successive layers of a model), so the ~34 MB a step touches is not resident
in the 256 MB Infinity Cache when the step starts.

--workload selects another seeded workload with the same protocol: llama8b,
longctx128k, longctx128k_full (no eviction), twostage (Stage II, exact
top-k_T V side), hikv_dualbank (HiKV's dual-bank Stage I; also times the
bank initialisation's prompt scores), hikv_hier (dual bank plus HiKV's
chunked Stage II V side), tiny.  --accumulate overrides the importance
accumulation (H2O probabilities, HiKV's recent window, Kelle's logits);
--prefill times the prompt scores on any workload.

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
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "k_attend_mfma_hbm_traffic_headkv32k.md")
KERNEL_SOURCES = ("importance_aware_kv_amd/csrc/step.hip", "importance_aware_kv_amd/csrc/hikv_common.h",
                  "importance_aware_kv_amd/csrc/hikv_block.h")


def measured_traffic():
    """HBM bytes per attention launch from the committed counter record, or None
    when the kernel sources changed since the counters were taken."""
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
    return rec["traffic_bytes"] if h.hexdigest() == rec["sources_sha256"] else None


def log(*a):
    print(*a, file=sys.stderr, flush=True)


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
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-hint", action="store_true", help="do not pass host lengths")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="after the run, copy this many bytes device-to-device 4 times (a plain copy "
                         "kernel of known size, for calibrating memory counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (this path has no "
              "multi-GPU mode).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from importance_aware_kv_amd import bytes_model as BM
    from importance_aware_kv_amd import hikv as H
    from importance_aware_kv_amd import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    H.lib()  # raises when the HIP library is missing: no fallback
    dev_name = torch.cuda.get_device_name(0)

    n_inputs = 256
    full = args.workload.endswith("_full")
    w = W.workload(args.workload[:-5] if full else args.workload, steps=n_inputs, full=full)
    if args.accumulate is not None:
        w.accumulate = {"all": H.HIKV_ACC_ALL, "recent": H.HIKV_ACC_RECENT, "logit": H.HIKV_ACC_LOGIT}[args.accumulate]
    # compression step + warm-up + the timed steps + the same number again for
    # the per-kernel timing replay
    per_layer_steps = 1 + (args.warmup + 2 * args.steps + args.layers - 1) // args.layers
    w.capacity = w.ctx + per_layer_steps + 1
    if full:  # full attention: the budget is the whole capacity, nothing is ever evicted
        w.budget_all = w.capacity
    stage2 = w.stage2_channels > 0
    t0 = time.time()
    d = W.generate(w)
    log(f"[bench] {w.name}: inputs generated in {time.time() - t0:.1f}s on {dev_name}")
    B, Hq, Hkv, D, G = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.group
    budget = w.budget_array()

    layers = [H.DeviceCache(d, Hq)]
    for _ in range(1, args.layers):
        c = H.DeviceCache.__new__(H.DeviceCache)
        c.torch = torch
        c.dtype, c.shape = layers[0].dtype, layers[0].shape
        for f in ("k", "v", "pos", "imp", "len", "evict"):
            setattr(c, f, getattr(layers[0], f).clone())
        c.cache = c.make_cache()
        layers.append(c)
    budget_t = torch.from_numpy(budget).cuda()
    # per-KV-head budgets go as a device array; one budget for every unit as budget_all
    b_arr, b_all = (budget_t, 0) if w.budgets is not None else (None, w.budget_all)
    pol = H.make_policy(b_arr, b_all, w.n_sink, w.n_recent, w.stage2_channels, w.stage2_tokens,
                        accumulate=w.accumulate, stage2_v=w.stage2_v)
    # One workspace (scratch) serves every layer copy, as it would every layer
    # of a model; each cache carries its own pending-eviction state.
    wss = [H.workspace(layers[0].shape, pol)]

    def device_status(what):
        for wsl in wss:
            H.check(H.hikv_device_status(wsl), what)
    # The caller's host copy of every layer's lengths (a serving loop tracks
    # them anyway); passed as the length hint so the tile plan is made on the
    # host.  --no-hint measures the device-derived plan instead.
    host_len = [np.full((B, Hkv), w.ctx, dtype=np.int32) for _ in range(args.layers)]
    q_all = H.to_device(d["q"])
    kn_all = H.to_device(d["k_new"])
    vn_all = H.to_device(d["v_new"])
    pos_all = torch.from_numpy(
        (w.ctx + np.arange(per_layer_steps + 1, dtype=np.int32))[:, None].repeat(B, 1).copy()).cuda()
    out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    layer_step = [0] * args.layers

    live_log = []  # tokens attended per step (sum over units), in launch order

    def step(li, events=None):
        c = layers[li]
        n = layer_step[li]
        layer_step[li] += 1
        # live tokens of the step (a pending eviction's dead slot is not one;
        # the Stage II path evicts in place and leaves none pending)
        live_now = host_len[li] + 1 - ((host_len[li] > budget) & (not stage2))
        live_log.append(int(live_now.sum()))
        moves_log.append(int((live_now > budget).sum()))
        p = pol
        if not args.no_hint:
            p = H.make_policy(b_arr, b_all, w.n_sink, w.n_recent, w.stage2_channels, w.stage2_tokens,
                              budget_hint=budget if b_arr is not None else None,
                              len_hint=host_len[li], accumulate=w.accumulate, stage2_v=w.stage2_v)
        dbg = None
        if events is not None:
            dbg = H.hikv_debug(None, None, None, events[0].cuda_event, events[1].cuda_event)
        code = H.hikv_decode_step(c.shape, c.cache, p, q_all[n % n_inputs], kn_all[n % n_inputs],
                                  vn_all[n % n_inputs], pos_all[n], out, wss[0], debug=dbg)
        if code != 0:
            raise RuntimeError(f"hikv_decode_step: {H.status_string(code)}")
        # The caller's copy of len[] after the step: a unit over its budget by one
        # keeps budget + 1 slots with that eviction pending (the next step writes
        # its new token into the dead slot); a bulk cut leaves exactly the budget.
        old = host_len[li]
        if stage2:
            host_len[li] = np.minimum(old + 1, budget).astype(np.int32)
        else:
            pending = old > budget
            live = old + 1 - pending
            host_len[li] = np.where(live > budget + 1, budget, np.where(pending, old, old + 1)).astype(np.int32)

    moves_log = []
    stream = torch.cuda.current_stream()
    prefill = None
    if (args.prefill or w.accumulate == H.HIKV_ACC_RECENT) and not full:
        prefill = measure_prefill(w, layers[0], budget, log)
    # Compression step of every layer copy (32769 tokens -> budget), queued
    # behind a GPU-side wait so that the steps run back to back.
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(100_000_000)
    e0.record(stream)
    for li in range(args.layers):
        step(li)
    e1.record(stream)
    torch.cuda.synchronize()
    comp_ms = e0.elapsed_time(e1) / args.layers
    device_status("device status after compression")
    live_after = np.minimum(w.ctx + 1, budget)
    assert np.array_equal(layers[0].len.cpu().numpy(), live_after), "compression did not reach the budgets"
    comp_bytes = BM.decode_step_bytes(B, Hq, Hkv, D, w.el, np.full((B, Hkv), w.ctx + 1),
                                      int(np.minimum(budget, w.ctx + 1).sum()))
    log(f"[bench] {'first' if full else 'compression'} step: {comp_ms * 1e3:.1f} us/layer "
        f"({comp_bytes / comp_ms / 1e6:.0f} GB/s algorithmic)")

    # Warm-up steady steps, eager.
    for i in range(args.warmup):
        step(i % args.layers)
    torch.cuda.synchronize()
    device_status("device status after warm-up")

    # Timed steady steps: one HIP graph, replayed once.
    base = args.warmup
    mark = len(live_log)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(args.steps):
            step((base + i) % args.layers)
    torch.cuda.synchronize()
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_start.record()
    g.replay()
    t_end.record()
    torch.cuda.synchronize()
    ms_total = t_start.elapsed_time(t_end)
    device_status("device status after timed steps")
    ms_step = ms_total / args.steps
    steps_per_s = 1e3 / ms_step
    # bytes of the average timed step (every step is alike in the budgeted steady
    # state; a full-attention step attends one token more than the one before)
    live_avg = sum(live_log[mark:]) / args.steps
    moves_avg = sum(moves_log[mark:]) / args.steps
    step_bytes = int(BM.decode_step_bytes(B, Hq, Hkv, D, w.el, [0], 0) + live_avg * (2 * D * w.el + 12)
                     + moves_avg * 2 * (2 * D * w.el + 8))
    gbs = step_bytes / (ms_step * 1e-3) / 1e9
    log(f"[bench] steady step: {ms_step * 1e3:.2f} us, {steps_per_s:.0f} steps/s, "
        f"{step_bytes / 1e6:.2f} MB/step algorithmic -> {gbs:.0f} GB/s ({gbs / HBM_PEAK_GBS:.1%} of 8 TB/s)")

    # The dominant kernel, the attention launch: the same steps run once more,
    # launched eagerly and back to back, with a pair of HIP events around every
    # attention launch, recorded by the library on the stream that launch uses
    # (event nodes inside a captured graph do not bracket the kernel's
    # execution).
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for e_a, e_b in evs:  # materialise the events
        e_a.record(stream)
        e_b.record(stream)
    torch.cuda.synchronize()
    base2 = base + args.steps
    # A GPU-side wait ahead of the replay lets the host enqueue every step
    # before the first runs, so the launches run back to back as in the graph
    # (no idle gaps while the host catches up).
    sleep_cycles = 500_000_000
    torch.cuda._sleep(sleep_cycles)
    t_enq = time.perf_counter()
    for i in range(args.steps):
        step((base2 + i) % args.layers, events=evs[i])
    t_enq = time.perf_counter() - t_enq
    torch.cuda.synchronize()
    log(f"[bench] timing replay: {args.steps} steps enqueued in {t_enq * 1e3:.1f} ms behind a "
        f"~{sleep_cycles / 2.4e6:.0f} ms GPU wait (the host blocks once the hardware queue is full)")
    device_status("device status after the timing replay")
    attend_ms = sum(e_a.elapsed_time(e_b) for e_a, e_b in evs) / args.steps
    live_rep = sum(live_log[-args.steps:]) / args.steps
    if stage2:  # the reduced-channel logits pass reads every live K row whole, and q
        attend_bytes = int(live_rep * D * w.el + B * Hq * D * w.el)
    else:
        attend_bytes = int(BM.attend_bytes(B, Hq, Hkv, D, w.el, [0]) + live_rep * 2 * D * w.el)
    attend_gbs = attend_bytes / (attend_ms * 1e-3) / 1e9
    log(f"[bench] attention launch: {attend_ms * 1e3:.2f} us, {attend_bytes / 1e6:.2f} MB algorithmic -> "
        f"{attend_gbs:.0f} GB/s ({attend_gbs / HBM_PEAK_GBS:.1%} of 8 TB/s)")

    if args.copy_bytes > 0:
        n = args.copy_bytes // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy calibration: 4 x {n * 4} bytes device-to-device")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, d, args.cpu_seconds)
        log(f"[bench] cpu oracle: {cpu}")

    line = {
        "metric": "decode steps/s and achieved KV HBM GB/s (fraction of 8 TB/s) per budget",
        "value": round(steps_per_s, 1),
        "unit": "decode steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.el == 2 else "f32",
        "data": "synthetic",
        "config": {
            "workload": workload_text(w, budget, full),
            "global_batch": B,
            "seq_len": w.ctx,
            "layers_cycled": args.layers,
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(attend_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(attend_gbs / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic() if args.workload == "headkv32k" else None,
            "kernel": kernel_text(w),
            "bytes_per_launch": attend_bytes,
            "us_per_launch": round(attend_ms * 1e3, 3),
            "whole_step": {"achieved": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
                           "bytes_per_step": step_bytes},
        },
        ("first_step_us" if full else "compression_step_us"): round(comp_ms * 1e3, 2),
        "cpu_baseline": cpu,
    }
    if prefill is not None:
        line["prefill_scores"] = prefill
    print(json.dumps(line), flush=True)


def measure_prefill(w, layer, budget, log, reps=3):
    """Prompt-side scores as HiKV initialises its banks (Sec. III-D): every
    prompt query adds its causal attention row to the tokens within the
    window (the recent bank's size) of it; window 0 (other workloads) counts
    every query.  Timed on a copy of one layer's prefilled cache, with seeded
    synthetic prompt queries; the decode measurement does not use it."""
    import torch

    from importance_aware_kv_amd import hikv as H
    B, Hq, D, L = w.batch, w.n_q_heads, w.head_dim, w.ctx
    c = H.DeviceCache.__new__(H.DeviceCache)
    c.torch = torch
    c.dtype, c.shape = layer.dtype, layer.shape
    for f in ("k", "v", "pos", "imp", "len", "evict"):
        setattr(c, f, getattr(layer, f).clone())
    c.imp.zero_()
    c.cache = c.make_cache()
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
    if w.stage2_channels:
        return (f"k_attn_tiles<2,{w.head_dim},{w.group},false,true> (Stage II reduced-channel logits over "
                "every live K row; HIP events per launch)")
    if w.el == 2 and w.head_dim == 128:
        return (f"k_attend_mfma<{w.group},3> (split-K attention over the live K/V rows on matrix cores; "
                "HIP events per launch)")
    return (f"k_attend<{w.el},{w.head_dim},{w.group}> (split-K attention over the live K/V rows; "
            "HIP events per launch)")


def cpu_baseline(w, d, seconds):
    """The CPU oracle, as it stands, on a bounded sample of the same workload:
    its own compression step, then steady steps until `seconds` have passed."""
    import numpy as np

    from oracle import ref
    st = ref.copy_state(d)
    budget = w.budget_array()
    kw = dict(budget=budget, n_sink=w.n_sink, n_recent=w.n_recent, debug=False,
              stage2_channels=w.stage2_channels, stage2_tokens=w.stage2_tokens,
              accumulate=w.accumulate, stage2_v=w.stage2_v)
    ref.decode_step(st, w.n_q_heads, d["q"][0], d["k_new"][0], d["v_new"][0], d["new_pos"][0], **kw)
    n = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds and n + 1 < d["q"].shape[0]:
        t = n + 1
        ref.decode_step(st, w.n_q_heads, d["q"][t], d["k_new"][t], d["v_new"][t], d["new_pos"][t], **kw)
        n += 1
    dt = time.perf_counter() - t0
    return {"value": round(n / dt, 2), "unit": "decode steps/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} steady decode steps of the same workload after the oracle's own "
                      f"compression step, single-threaded fp64 C++ ({dt:.1f}s)"}


if __name__ == "__main__":
    main()
