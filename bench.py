"""Benchmark: batch-1 GPT-2 124M greedy decode on one MI355X.

One bench step = one whole greedy run of the workload (default: the fp32 124M
model, 10 prompt ids + 60 greedy ids = 69 one-token forward passes, chained on
the device by gpt2_generate).  `value` is forward passes (decoded tokens) per
second over the timed steps, with weights and prompt already resident on the
GPU.  Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--config 2..5] [--only] [--no-cpu-baseline]
                  [--prefill-only] [--timeline CONFIG]

The headline workload (--config, default 2) gives the line's value and roofline;
the other three 124M workloads are timed in the same run, each in
"other_configs" with its own value, per-pass time and roofline (--only skips
them).  "prefill" times gpt2_prefill on the fp32 124M model: one call takes a
1024-id prompt through every layer at once (GEMMs and attention on the matrix
cores), so it is rated in tokens/s and against the fp32 matrix-core peak.
"prefill_then_decode" runs the headline workload with its prompt prefilled,
"sampled" with temperature sampling instead of the greedy pick.
"""
import argparse
import contextlib
import gc
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E peak, GB/s
MFMA_F32_PEAK_TFS = 157.3  # MI355X dense fp32 matrix-core peak, TFLOP/s
PREFILL_N = 1024       # prompt ids per timed prefill call


@contextlib.contextmanager
def no_gc():
    """Python's garbage collector off inside a timed loop (a collection pause
    there would count as device time between the events around a launch)."""
    gc.collect()
    gc.disable()
    try:
        yield
    finally:
        gc.enable()


def bytes_per_step(cfg, p):
    """Algorithmic bytes of one forward pass at position p: every weight once
    (block matrices in their storage type, the head, biases and LayerNorm
    parameters, the two embedding rows) plus the K and V rows 0..p read by
    attention."""
    E, F, V, L = cfg.n_embd, 4 * cfg.n_embd, cfg.vocab, cfg.n_layer
    elems = L * (3 * E * E + E * E + F * E + E * F)
    if cfg.wdtype == "fp32":
        mats = elems * 4
        head = V * E * 4
    elif cfg.wdtype == "fp16":
        mats = elems * 2
        head = V * E * 2
    else:
        mats = elems // 2 + elems // 32 * 8
        head = V * E * 4
    small = (L * (2 * E + 3 * E + E + 2 * E + F + E) + 2 * E) * 4 + 2 * E * 4
    kv = L * 2 * E * 4 * (p + 1)
    return mats + head + small + kv


def kernel_source_hash(files=("decode_kernel.hip", "dec_internal.h")):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "transformer_decode_token_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


PREFILL_SOURCES = ("prefill.hip",)


def load_prefill_traffic(cfg_key, n):
    """Memory-side bytes of one gpt2_prefill call (every kernel of the call),
    measured with rocprofv3 counters for this exact prefill source
    (profiles/prefill_traffic.json), else None."""
    path = os.path.join(ROOT, "profiles", "prefill_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    e = d.get(f"{cfg_key}/{n}")
    if not e or e.get("source_hash") != kernel_source_hash(PREFILL_SOURCES):
        return None
    return e


def load_traffic(cfg_key):
    """HBM bytes per launch measured with rocprofv3 counters for this exact
    kernel source (profiles/decode_traffic.json), else None."""
    path = os.path.join(ROOT, "profiles", "decode_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    e = d.get(str(cfg_key))
    if not e or e.get("kernel_hash") != kernel_source_hash():
        return None
    return e


def cpu_info():
    """The host CPU's model name and the number of CPUs this process may use."""
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
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count()
    return model, n


def cpu_baseline(cfg, seconds=10.0):
    """The oracle (fp32 build), single-threaded, on the GPU host: the same greedy
    run from position 0, repeated until about `seconds` of work."""
    import synth
    from oracle import Oracle
    model = synth.make_model(cfg)
    orc = Oracle(model)
    prompt = [int(t) for t in synth.make_prompt(cfg)]
    t0 = time.perf_counter()
    n = runs = 0
    while (time.perf_counter() - t0) < seconds:
        orc.reset()
        toks = list(prompt)
        for pos in range(cfg.n_steps):
            am, _ = orc.step(toks[pos], pos, want_logits=False)
            if pos + 1 >= len(toks):
                toks.append(am)
            n += 1
            if (time.perf_counter() - t0) >= seconds:
                break
        runs += 1
    dt = time.perf_counter() - t0
    orc.close()
    # the algorithmic bytes of the passes timed (the same accounting as the GPU roofline)
    done, byts = 0, 0
    while done < n:
        k = min(cfg.n_steps, n - done)
        byts += sum(bytes_per_step(cfg, p) for p in range(k))
        done += k
    model, ncpu = cpu_info()
    return {"value": round(n / dt, 3), "unit": "tok/s", "cores": 1, "kind": "oracle",
            "gb_per_s": round(byts / dt / 1e9, 3), "cpu": model, "cpus_available": ncpu,
            "sample": f"{n} forward passes: the {cfg.n_steps}-pass greedy run from position 0, "
                      f"repeated ({runs} started), {dt:.1f} s, one thread"}


def stream_read_ceiling(torch, gib=4):
    """A measured streaming-read rate of this GPU (context for the 8 TB/s vendor
    peak): torch's sum over a `gib` GiB fp32 tensor, best of 5."""
    x = torch.ones((gib << 30) // 4, dtype=torch.float32, device="cuda")
    x.sum()
    torch.cuda.synchronize()
    best = None
    for _ in range(5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        x.sum()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b)
        best = ms if best is None else min(best, ms)
    del x
    torch.cuda.empty_cache()
    return round((gib << 30) / (best * 1e-3) / 1e9, 1)


def time_config(cfg, steps, warmup, sync_steps, torch, g2):
    """Load one workload, time `steps` device-chained greedy runs of it (HIP
    events on the library's stream, and the host clock around the loop), and the
    synchronous one-token call.  Returns a dict of measurements."""
    import synth
    model = synth.make_model(cfg)
    prompt = synth.make_prompt(cfg)
    ctx = g2.gpt2_load(cfg.n_layer, cfg.n_embd, cfg.n_head, cfg.n_positions, cfg.vocab, model.t,
                       wdtype=cfg.wdtype, ln_eps=cfg.ln_eps, q4_group=cfg.q4_group)
    del model
    stream = torch.cuda.current_stream()
    g2.gpt2_set_stream(ctx, stream.cuda_stream)
    for _ in range(warmup):
        g2.gpt2_reset(ctx)
        g2.gpt2_generate(ctx, prompt, cfg.n_new)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    # torch creates an event at its first record: do that outside the timed loop
    for ev in starts + ends:
        ev.record(stream)
    with no_gc():
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            g2.gpt2_reset(ctx)
            starts[i].record(stream)
            g2.gpt2_generate(ctx, prompt, cfg.n_new)
            ends[i].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    times = [a.elapsed_time(b) for a, b in zip(starts, ends)]
    ms_launch = float(np.mean(times))
    ms_median = float(np.median(times))
    # synchronous one-token calls (host round trip per token)
    g2.gpt2_reset(ctx)
    torch.cuda.synchronize()
    ns = min(sync_steps, cfg.n_steps)
    ts = time.perf_counter()
    for pos in range(ns):
        g2.gpt2_step(ctx, int(prompt[pos % len(prompt)]), pos, want_logits=False)
    sync_tok_s = ns / (time.perf_counter() - ts) if ns else None
    ctx.close()
    torch.cuda.synchronize()
    return {"wall_s": wall, "ms_launch": ms_launch, "ms_median": ms_median, "sync_tok_s": sync_tok_s}


def roofline(cfg, ms_launch):
    """HBM roofline of the decode kernel for one launch of the workload:
    algorithmic bytes (every weight once per pass + the K/V rows read) per event-
    timed launch, and the rocprofv3-counted DRAM-side bytes when they were taken
    for this kernel source."""
    alg_bytes = sum(bytes_per_step(cfg, p) for p in range(cfg.n_steps))
    achieved = alg_bytes / (ms_launch * 1e-3) / 1e9
    tr = load_traffic(cfg.key)
    out = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
           "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": tr["bytes_per_launch"] if tr else None}
    if tr:
        # the same launch's bytes fetched from the memory side (FETCH_SIZE, calibrated),
        # which for fp16/int4 include memory-side-cache hits
        out["dram_read_bytes"] = tr["fetch_bytes"]
        out["dram_read_frac"] = round(tr["fetch_bytes"] / (ms_launch * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
        out["dram_read_over_algorithmic"] = round(tr["fetch_bytes"] / alg_bytes, 3)
    return out, alg_bytes


def config_line(cfg, m):
    """The per-workload figures of one time_config result."""
    rf, alg = roofline(cfg, m["ms_launch"])
    return {
        "workload": workload_name(cfg),
        "value": round(cfg.n_steps * m["steps"] / m["wall_s"], 2),
        "unit": "tok/s",
        "ms_per_step": round(m["wall_s"] * 1e3 / m["steps"], 4),
        "generated_tok_per_s": round(cfg.n_new * m["steps"] / m["wall_s"], 2),
        "decode_kernel_ms_per_launch": round(m["ms_launch"], 4),
        "median_us_per_token": round(m["ms_median"] * 1e3 / cfg.n_steps, 2),
        "us_per_token": round(m["ms_launch"] * 1e3 / cfg.n_steps, 2),
        "algorithmic_bytes_per_launch": alg,
        "roofline": rf,
        "sync_step_tok_per_s": round(m["sync_tok_s"], 1) if m["sync_tok_s"] else None,
    }


def prefill_flops(cfg, n, p0=0):
    """Algorithmic flops of one gpt2_prefill call of n ids from position p0:
    2 per multiply-add of the four block linears for every row, the causal
    attention (q.k and the weighted value sum over keys 0..p0+t for row t), and
    the head for the last row."""
    E, V, L = cfg.n_embd, cfg.vocab, cfg.n_layer
    linears = 2 * n * L * (3 * E * E + E * E + 4 * E * E + 4 * E * E)
    keys = sum(p0 + t + 1 for t in range(n))
    attention = L * 2 * 2 * E * keys
    return linears + attention + 2 * V * E


def time_prefill(cfg, n, steps, warmup, torch, g2):
    """Time `steps` gpt2_prefill calls of one seeded n-id prompt from position 0
    (HIP events on the library's stream, and the host clock around the loop)."""
    import synth
    model = synth.make_model(cfg)
    ctx = g2.gpt2_load(cfg.n_layer, cfg.n_embd, cfg.n_head, cfg.n_positions, cfg.vocab, model.t,
                       wdtype=cfg.wdtype, ln_eps=cfg.ln_eps, q4_group=cfg.q4_group)
    del model
    prompt = np.random.default_rng(20241).integers(0, cfg.vocab, n).astype(np.int32)
    stream = torch.cuda.current_stream()
    g2.gpt2_set_stream(ctx, stream.cuda_stream)
    for _ in range(warmup):
        g2.gpt2_reset(ctx)
        g2.gpt2_prefill(ctx, prompt, want_logits=False)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for ev in starts + ends:
        ev.record(stream)
    with no_gc():
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            g2.gpt2_reset(ctx)
            starts[i].record(stream)
            g2.gpt2_prefill(ctx, prompt, want_logits=False)
            ends[i].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    ms = float(np.mean([a.elapsed_time(b) for a, b in zip(starts, ends)]))
    ctx.close()
    torch.cuda.synchronize()
    flops = prefill_flops(cfg, n)
    achieved = flops / (ms * 1e-3) / 1e12
    tr = load_prefill_traffic(cfg.key, n)
    return {
        "workload": f"{cfg.name}: one {n}-id prompt from position 0 through every layer in one gpt2_prefill "
                    f"call (then its last row's logits and argmax), batch 1",
        "value": round(n * steps / wall, 1),
        "unit": "tok/s",
        "ms_per_call": round(wall * 1e3 / steps, 4),
        "event_ms_per_call": round(ms, 4),
        "flops_per_call": flops,
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_F32_PEAK_TFS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_F32_PEAK_TFS, 4),
                     "traffic": tr["bytes_per_call"] if tr else None},
        "roofline_note": "algorithmic flops of the whole call (linears, causal attention, head) over its "
                         "event-timed duration, against the dense fp32 matrix-core peak",
    }


def time_prefill_then_decode(cfg, steps, warmup, torch, g2):
    """The headline workload as an application would run it: the prompt in one
    gpt2_prefill call (its argmax is the first new id), then the other
    n_new - 1 ids by gpt2_generate chained on the device: the same 69
    positions.  Host clock around `steps` runs, each after a reset; also
    whether the ids equal those of the one-pass-per-id run."""
    import synth
    model = synth.make_model(cfg)
    prompt = synth.make_prompt(cfg)
    ctx = g2.gpt2_load(cfg.n_layer, cfg.n_embd, cfg.n_head, cfg.n_positions, cfg.vocab, model.t,
                       wdtype=cfg.wdtype, ln_eps=cfg.ln_eps, q4_group=cfg.q4_group)
    del model

    def run():
        g2.gpt2_reset(ctx)
        first, _ = g2.gpt2_prefill(ctx, prompt, want_logits=False)
        rest = g2.gpt2_generate(ctx, np.array([first], np.int32), cfg.n_new - 1)
        return [int(first)] + [int(i) for i in rest]

    g2.gpt2_reset(ctx)
    reference = [int(i) for i in g2.gpt2_generate(ctx, prompt, cfg.n_new)]
    ids = None
    for _ in range(warmup):
        ids = run()
    with no_gc():
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            ids = run()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    ctx.close()
    return {
        "workload": f"{cfg.name}: the {cfg.n_prompt}-id prompt in one gpt2_prefill call, then {cfg.n_new - 1} "
                    f"greedy ids by gpt2_generate ({cfg.n_new} new ids, positions 0..{cfg.n_steps - 1}), batch 1",
        "ms_per_run": round(wall * 1e3 / steps, 4),
        "generated_tok_per_s": round(cfg.n_new * steps / wall, 2),
        "same_ids_as_one_pass_per_id": ids == reference,
    }


def time_sampled(cfg, steps, warmup, torch, g2, temperature=0.8, seed=20241):
    """The headline workload with temperature sampling instead of the greedy
    pick (gpt2_generate_sample: softmax(logits / T) and one xorshift64* draw
    per id, chained on the device); event-timed like the greedy runs."""
    import synth
    model = synth.make_model(cfg)
    prompt = synth.make_prompt(cfg)
    ctx = g2.gpt2_load(cfg.n_layer, cfg.n_embd, cfg.n_head, cfg.n_positions, cfg.vocab, model.t,
                       wdtype=cfg.wdtype, ln_eps=cfg.ln_eps, q4_group=cfg.q4_group)
    del model
    stream = torch.cuda.current_stream()
    g2.gpt2_set_stream(ctx, stream.cuda_stream)
    for _ in range(warmup):
        g2.gpt2_reset(ctx)
        g2.gpt2_generate_sample(ctx, prompt, cfg.n_new, temperature, seed)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for ev in starts + ends:
        ev.record(stream)
    with no_gc():
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            g2.gpt2_reset(ctx)
            starts[i].record(stream)
            g2.gpt2_generate_sample(ctx, prompt, cfg.n_new, temperature, seed + i)
            ends[i].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    ms = float(np.mean([a.elapsed_time(b) for a, b in zip(starts, ends)]))
    ctx.close()
    return {
        "workload": f"{cfg.name}: {cfg.n_prompt} prompt ids + {cfg.n_new} ids drawn at temperature {temperature} "
                    f"= {cfg.n_steps} one-token forward passes, batch 1",
        "value": round(cfg.n_steps * steps / wall, 2),
        "unit": "tok/s",
        "ms_per_step": round(wall * 1e3 / steps, 4),
        "us_per_token": round(ms * 1e3 / cfg.n_steps, 2),
    }


def timeline(cfg, torch, g2):
    """Per-phase timeline of one traced greedy run (gpt2_debug_trace: a variant
    of the kernel that stamps the device wall clock when each workgroup's
    inputs are ready, passes its two barriers and has published; about 2 us
    per pass slower than the untraced kernel).  Medians over the passes from
    the 13th on, in us from the previous phase's last publish to the last
    workgroup's event, per phase kind; the stamps' tick rate is taken from
    the launch's event-timed duration."""
    import synth
    model = synth.make_model(cfg)
    prompt = synth.make_prompt(cfg)
    ctx = g2.gpt2_load(cfg.n_layer, cfg.n_embd, cfg.n_head, cfg.n_positions, cfg.vocab, model.t,
                       wdtype=cfg.wdtype, ln_eps=cfg.ln_eps, q4_group=cfg.q4_group)
    del model
    stream = torch.cuda.current_stream()
    g2.gpt2_set_stream(ctx, stream.cuda_stream)
    L, ns = cfg.n_layer, cfg.n_steps
    g2.gpt2_generate(ctx, prompt, cfg.n_new)
    g2.gpt2_reset(ctx)
    g2.gpt2_debug_trace(ctx, ns)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    g2.gpt2_generate(ctx, prompt, cfg.n_new)
    b.record(stream)
    torch.cuda.synchronize()
    rec = g2.gpt2_debug_trace(ctx, 0, fetch=True).astype(np.float64)  # [ns][5L+1][G][4]
    ctx.close()
    launch_us = a.elapsed_time(b) * 1e3
    stamps = rec[rec > 0]
    # (the stamps span nearly the whole launch, so this overstates the tick by about 1%)
    us_per_tick = launch_us / (stamps.max() - stamps.min())

    def last(st, ph, k):
        v = rec[st, ph, :, k]
        v = v[v > 0]
        return v.max() if v.size else np.nan

    names = ["qkv", "attention", "attention_projection", "fc", "mlp_projection"]
    rows = {nm: [] for nm in names}
    per_layer, head, token = [], [], []
    for st in range(12, ns):
        for l in range(L):
            for i, nm in enumerate(names):
                ph = 5 * l + i
                prev = last(st, ph - 1, 3) if ph > 0 else last(st - 1, 5 * L, 3)
                rows[nm].append([(last(st, ph, k) - prev) * us_per_tick for k in range(4)])
            if l > 0:
                per_layer.append((last(st, 5 * l + 4, 3) - last(st, 5 * (l - 1) + 4, 3)) * us_per_tick)
        head.append((last(st, 5 * L, 3) - last(st, 5 * L - 1, 3)) * us_per_tick)
        token.append((last(st, 5 * L, 3) - last(st - 1, 5 * L, 3)) * us_per_tick)
    return {
        "workload": workload_name(cfg) + " (traced kernel)",
        "us_per_tick": round(us_per_tick, 5),
        "us_per_token": round(float(np.median(token)), 2),
        "us_per_layer": round(float(np.median(per_layer)), 2),
        "us_head": round(float(np.median(head)), 2),
        # (a negative 'inputs ready' is a stamp taken before the inputs were in:
        # in the eight-wave kernels the dot waves poll the inputs of sets Q, A
        # and F, and barrier 1 marks their arrival; reported as null)
        "phases_us_ready_barrier1_barrier2_published": {
            nm: [None if (k == 0 and x < 0) else round(float(x), 2)
                 for k, x in enumerate(np.nanmedian(np.array(rows[nm]), axis=0))] for nm in names},
    }


def workload_name(cfg):
    return (f"{cfg.name}: {cfg.n_prompt} prompt ids + {cfg.n_new} greedy ids = {cfg.n_steps} one-token "
            f"forward passes, batch 1")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=2, help="the headline workload (2..5)")
    ap.add_argument("--only", action="store_true",
                    help="time the headline workload alone (no per-config lines for the others)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--timeline", type=int, default=0, metavar="CONFIG",
                    help="print the per-phase timeline of a traced greedy run of this workload (2..5)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="time only gpt2_prefill (fp32 124M, one 1024-id prompt per call) and print its line")
    ap.add_argument("--sync-steps", type=int, default=30,
                    help="gpt2_step calls timed for the synchronous per-token rate")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run plain device-to-device copies of MIB MiB (a known-size "
                         "reference for the FETCH_SIZE / WRITE_SIZE counters), then exit")
    args = ap.parse_args()
    if args.calibrate_copy:
        import torch
        n = args.calibrate_copy * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n * 4, "copies": 3}), flush=True)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on one GPU only (batch-1 decode of one sequence does "
              "not shard usefully); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import transformer_decode_token_amd as g2

    torch.cuda.init()
    if args.timeline:
        print(json.dumps({"timeline": timeline(synth.CONFIGS[args.timeline], torch, g2)}), flush=True)
        return
    if args.prefill_only:
        print(f"[bench] prefill: {args.warmup} warm-up + {args.steps} timed calls of {PREFILL_N} ids",
              file=sys.stderr, flush=True)
        print(json.dumps({"prefill": time_prefill(synth.CONFIGS[2], PREFILL_N, args.steps, args.warmup, torch, g2)}),
              flush=True)
        return
    head_cfg = synth.CONFIGS[args.config]
    others = [] if args.only else [k for k in (2, 3, 4, 5) if k != args.config]
    results = {}
    for k in [args.config] + others:
        cfg = synth.CONFIGS[k]
        print(f"[bench] config {k} {cfg.name}: {args.warmup} warm-up + {args.steps} timed runs of "
              f"{cfg.n_steps} passes", file=sys.stderr, flush=True)
        m = time_config(cfg, args.steps, args.warmup, args.sync_steps, torch, g2)
        m["steps"] = args.steps
        results[k] = config_line(cfg, m)
        print(f"[bench] config {k}: {results[k]['us_per_token']} us per pass, "
              f"{results[k]['roofline']['frac']} of the HBM peak", file=sys.stderr, flush=True)
    h = results[args.config]
    out = {
        "metric": "batch-1 decode tok/s GPT-2 124M fp32/fp16/int4; achieved HBM GB/s vs peak",
        "value": h["value"],
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": h["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"fp32": "f32", "fp16": "f16 weights, f32 math", "int4": "u4 weights, f32 math"}[head_cfg.wdtype],
        "data": "synthetic (seeded random weights of the GPT-2 124M shape; seeded prompt ids)",
        "config": {"workload": h["workload"],
                   "n_layer": head_cfg.n_layer, "n_embd": head_cfg.n_embd, "n_head": head_cfg.n_head,
                   "vocab": head_cfg.vocab, "weights": head_cfg.wdtype, "parallelism": "single GPU"},
        "roofline": h["roofline"],
        "roofline_note": "frac = algorithmic bytes (each weight once per pass + K/V rows read) over the "
                         "event-timed launch; dram_read_frac = the counted FETCH_SIZE bytes over the same time",
        "generated_tok_per_s": h["generated_tok_per_s"],
        "decode_kernel_ms_per_launch": h["decode_kernel_ms_per_launch"],
        "us_per_token": h["us_per_token"],
        "median_us_per_token": h["median_us_per_token"],
        "algorithmic_bytes_per_launch": h["algorithmic_bytes_per_launch"],
        "sync_step_tok_per_s": h["sync_step_tok_per_s"],
        "other_configs": {str(k): results[k] for k in others},
    }
    if not args.only:
        print(f"[bench] prefill: {args.warmup} warm-up + {args.steps} timed calls of {PREFILL_N} ids",
              file=sys.stderr, flush=True)
        out["prefill"] = time_prefill(synth.CONFIGS[2], PREFILL_N, args.steps, args.warmup, torch, g2)
        # the same prompt with fp16 and int4 block matrices (widened or decoded
        # into the GEMM stages; products and sums in fp32, as for fp32 weights)
        out["prefill_other_weights"] = {}
        for k in (3, 4):
            c = synth.CONFIGS[k]
            print(f"[bench] prefill, {c.name}", file=sys.stderr, flush=True)
            r = time_prefill(c, PREFILL_N, args.steps, args.warmup, torch, g2)
            out["prefill_other_weights"][c.name] = {key: r[key] for key in
                                                    ("value", "unit", "ms_per_call", "event_ms_per_call")}
            out["prefill_other_weights"][c.name]["roofline_frac"] = r["roofline"]["frac"]
        print("[bench] prompt by prefill, then decode", file=sys.stderr, flush=True)
        out["prefill_then_decode"] = time_prefill_then_decode(head_cfg, args.steps, args.warmup, torch, g2)
        print("[bench] sampled run", file=sys.stderr, flush=True)
        out["sampled"] = time_sampled(head_cfg, args.steps, args.warmup, torch, g2)
    if not args.only:
        print("[bench] streaming-read ceiling", file=sys.stderr, flush=True)
        out["measured_stream_read_GBs"] = stream_read_ceiling(torch)
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(head_cfg)
        if not args.only:
            # the other weight types' oracle rates (shorter samples: context only)
            out["cpu_baseline_other"] = {str(k): cpu_baseline(synth.CONFIGS[k], seconds=4.0)
                                         for k in (3, 4) if k != args.config}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
