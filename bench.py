"""Benchmark of the window+sink chunk-attention hot path on one MI355X.

One step = one pass of the stack workload: 30 layers of 12 heads x 128 (1560 tokens/frame,
chunk 3 frames = 4680 query rows, sink 3 + window 9 frames), 80 chunks streamed from an empty
cache, 4 denoise steps per chunk; every denoise step runs ll_attn_chunk on each of the 30
layers, and after the last step one ll_cache_commit_layers commits the chunk's K/V into all
30 layers. Inputs are synthetic bf16 N(0, 0.25), generated on the GPU before timing (resident
in HBM) and cycled through a pool of 8 sets (values do not change the work). Prints ONE JSON
line.

value = query rows attended per second over the whole step (attention + commits);
roofline = the attention kernel against the bf16 dense MFMA peak: average algorithmic flops
per launch over the pass, divided by the average launch duration from HIP events recorded on
the launch stream around each chunk's 120 attention launches in the timed region; extra rows
report the single-layer stream, the commits, the FP4 store, the recache and the other
workloads, each timed on its own after the main loop.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 (published)
HBM_PEAK_GBS = 8000.0              # MI355X HBM3E (published)
# GPU spin ahead of each timed batch of the cache and codec rows (gpu_hold): longer than the
# host needs to enqueue a batch (30 Python-level commit calls)
HOLD_MS = 3.0


# hipDeviceAttribute_t values of the ROCm 7 HIP runtime (hip_runtime_api.h); they are only
# trusted when the multiprocessor count read this way equals torch's
HIP_ATTR_CLOCK_KHZ, HIP_ATTR_LDS_PER_CU, HIP_ATTR_MEM_CLOCK_KHZ = 5, 10002, 60
HIP_ATTR_MEM_BUS_BITS, HIP_ATTR_CUS = 59, 63


def device_info(torch):
    """The device the peaks above are meant for, as the runtime reports it: name, architecture,
    compute units, L2 and HBM sizes (torch), peak shader clock, LDS per CU and memory clock and
    bus width (HIP attributes, through the runtime torch already loaded), and the bf16 dense
    MFMA peak they imply (4096 bf16 flop per clock per CU). The HBM peak stays the published
    8 TB/s: the transfers per reported memory clock depend on the memory type."""
    prop = torch.cuda.get_device_properties(0)
    info = {"name": prop.name, "arch": prop.gcnArchName, "compute_units": prop.multi_processor_count,
            "l2_bytes_per_xcd": prop.L2_cache_size, "hbm_bytes": prop.total_memory}
    try:
        hip = ctypes.CDLL("libamdhip64.so.7")
    except OSError:
        return info

    def attr(code):
        v = ctypes.c_int(0)
        return v.value if hip.hipDeviceGetAttribute(ctypes.byref(v), ctypes.c_int(code), ctypes.c_int(0)) == 0 else None

    if attr(HIP_ATTR_CUS) != prop.multi_processor_count:
        return info
    clk, lds = attr(HIP_ATTR_CLOCK_KHZ), attr(HIP_ATTR_LDS_PER_CU)
    mclk, bus = attr(HIP_ATTR_MEM_CLOCK_KHZ), attr(HIP_ATTR_MEM_BUS_BITS)
    info.update({"peak_clock_ghz": clk / 1e6 if clk else None, "lds_bytes_per_cu": lds,
                 "mem_clock_ghz": mclk / 1e6 if mclk else None, "mem_bus_bits": bus})
    if clk:
        info["bf16_dense_peak_tflops_from_clock"] = round(prop.multi_processor_count * 4096 * clk * 1e3 / 1e12, 1)
    return info


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extra", action="store_true", help="skip the FP4 / recache rows")
    ap.add_argument("--row", choices=["share", "recache", "vendor-flash", "steady"], default=None,
                    help="run only this workload (for profiling) and print its row: the 3-head "
                         "share streams, the 30-layer recache, the vendor flash attention "
                         "on the steady chunk's shape, or 40 steady 12-head chunk calls")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration)")
    return ap.parse_args()


def copy_calibration(mib):
    """A plain device-to-device copy of known size, for scaling FETCH_SIZE / WRITE_SIZE."""
    import torch
    n = mib * (1 << 20)
    a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "bytes_written": n, "launches": 3}))


def code_hash(path):
    """sha256 prefix of a C++/HIP source with its comments and whitespace removed: it changes
    with the code, not with the commentary."""
    import hashlib
    import re
    text = open(path, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = re.sub(r"\s+", " ", text).strip()
    return hashlib.sha256(text.encode("utf-8")).hexdigest()[:16]


def counter_traffic(avg_flops_per_launch):
    """HBM bytes per attention launch from the committed FETCH_SIZE / WRITE_SIZE summary, but only
    while the kernel code is the one the counters were taken on (else None)."""
    src = os.path.join(ROOT, "windowed_attention_kv_amd", "csrc", "attn_bf16.hip")
    prof = os.path.join(ROOT, "profiles", "attn_commit_traffic_counters.md")
    try:
        sha = code_hash(src)
        kv = {}
        for line in open(prof):
            if ":" in line and line.startswith("    "):
                k, v = line.strip().split(":", 1)
                kv[k.strip()] = v.strip()
        if kv.get("source_sha256_prefix") != sha:
            return None
        return round((float(kv["fetch_kib_per_launch"]) * float(kv["read_scale"])
                      + float(kv["write_kib_per_launch"]) * float(kv["write_scale"])) * 1024)
    except (OSError, KeyError, ValueError):
        return None


def visible_keys(chunk, C, S, W, T):
    s = chunk * C
    frames = set(range(min(S, s + C))) | set(range(max(0, s - W), s)) | set(range(s, s + C))
    return len(frames) * T


def gen_inputs(torch, n_chunks, n, H, D, seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out = []
    for _ in range(n_chunks):
        trip = []
        for _ in range(3):
            x = torch.randn((n, H, D), generator=g, device=device, dtype=torch.float32) * 0.5
            trip.append(x.to(torch.bfloat16))
        out.append(tuple(trip))
    return out


_SLEEP_CYCLES_PER_MS = None


def progress(msg):
    """One progress line on stderr (stdout carries only the JSON result line)."""
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def gpu_hold(torch, ms):
    """Enqueue a GPU spin of about `ms` milliseconds (torch's sleep kernel, its cycle count
    calibrated once with events). A start event recorded after it fires only when the spin
    ends, by which time the host has enqueued the timed calls: the events then measure the
    GPU's own time for back-to-back launches, not the host's argument marshalling between
    them. Returns False (and enqueues nothing) if the spin cannot be calibrated."""
    global _SLEEP_CYCLES_PER_MS
    if _SLEEP_CYCLES_PER_MS is None:
        _SLEEP_CYCLES_PER_MS = 0.0
        try:
            torch.cuda._sleep(1 << 20)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            torch.cuda._sleep(1 << 24)
            b.record()
            b.synchronize()
            el = a.elapsed_time(b)
            if el > 0.05:
                _SLEEP_CYCLES_PER_MS = (1 << 24) / el
        except (AttributeError, RuntimeError):
            pass
    if _SLEEP_CYCLES_PER_MS <= 0:
        return False
    torch.cuda._sleep(int(ms * _SLEEP_CYCLES_PER_MS))
    return True


class EventTimer:
    """Pairs of HIP events recorded on the current (launch) stream."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = []

    def start(self, hold_ms=0.0):
        """Record a start event; with hold_ms, behind a GPU spin of that length (gpu_hold)."""
        if hold_ms > 0:
            gpu_hold(self.torch, hold_ms)
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    def stop(self, s, tag):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        self.pairs.append((tag, s, e))

    def totals(self):
        out = {}
        for tag, s, e in self.pairs:
            ms = s.elapsed_time(e)
            t = out.setdefault(tag, [0.0, 0])
            t[0] += ms
            t[1] += 1
        return out


def run_stream(cache, inputs, timer=None):
    for c, (q, k, v) in enumerate(inputs):
        if timer:
            s = timer.start()
        cache.attn_chunk(0, q, k, v, out=_OUT[0])
        if timer:
            timer.stop(s, "attn")
            s = timer.start()
        cache.commit(0, k, v)
        if timer:
            timer.stop(s, "commit")


_OUT = [None]


def host_cores():
    """Host CPU counts of the machine the oracle runs on: logical CPUs, CPUs this process may
    use, and physical cores from lscpu (None where unavailable)."""
    import subprocess
    info = {"logical_cpus": os.cpu_count(), "usable_cpus": len(os.sched_getaffinity(0))}
    try:
        out = subprocess.run(["lscpu", "-p=CORE,SOCKET"], capture_output=True, text=True,
                             timeout=10).stdout
        cores = {tuple(l.split(",")) for l in out.splitlines() if l and not l.startswith("#")}
        info["physical_cores_lscpu"] = len(cores) or None
        model = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in model.splitlines():
            if line.startswith("Model name:"):
                info["model"] = line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        info["physical_cores_lscpu"] = None
    return info


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        return None


def cpu_baseline(shape):
    """The fp64 oracle as it stands, timed on bounded samples of the workloads (input drawing
    excluded), each scaled to its whole workload by algorithmic flops or by heads (every
    steady chunk, head and layer does the same work):
      - the stack (the headline): layer 0, 4 denoise steps, chunks 0-7 (fill-up and steady
        chunks, attention and commit), 1 of 12 heads, scaled by flops to 30 layers x 80 chunks
        x 12 heads;
      - the tiny config in full; the FP4 stack (1 denoise step of chunks 0-7 over an FP4
        store, codec included, 1 head, scaled by flops); one layer of the prompt-switch recache
        (1 head, scaled by heads); one steady chunk call (23,400 keys, 1 head) on 1 thread."""
    from oracle.model import LayerModel
    from windowed_attention_kv_amd import synth
    n, T, C, S, W = shape.n_query, shape.tokens_per_frame, shape.chunk_frames, shape.sink_frames, shape.window_frames
    L, steps, chunks = 30, 4, 80
    D = shape.head_dim

    def flops(chunk_ids, heads, n_steps):
        return sum(n_steps * n * visible_keys(c, C, S, W, T) * heads * 4 * D for c in chunk_ids)

    sub1 = synth.shrink(shape, heads=1)
    stack_flops = L * flops(range(chunks), shape.heads, steps)
    # the stack: layer 0, 4 steps, chunks 0-7, 1 head
    sub_chunks = 8
    ins = [[synth.chunk_inputs(sub1, 0, st, c) for st in range(steps)] for c in range(sub_chunks)]
    m = LayerModel(S, W, C, T, 1, D)
    t0 = time.perf_counter()
    for c in range(sub_chunks):
        for st in range(steps):
            q, k, v = ins[c][st]
            m.attn_chunk(q.values, k.values, v.values)
        m.commit(k.values, v.values)
    dt = time.perf_counter() - t0
    sub_flops = flops(range(sub_chunks), 1, steps)
    stack_s = dt * stack_flops / sub_flops
    rows_stack = n * L * steps * chunks
    extra = {}
    # the tiny config, whole stream
    tiny = synth.CONFIGS["tiny"]
    tins = [synth.chunk_inputs(tiny, 0, 0, c) for c in range(tiny.chunks)]
    mt = LayerModel(tiny.sink_frames, tiny.window_frames, tiny.chunk_frames, tiny.tokens_per_frame,
                    tiny.heads, tiny.head_dim)
    t0 = time.perf_counter()
    for q, k, v in tins:
        mt.attn_chunk(q.values, k.values, v.values)
        mt.commit(k.values, v.values)
    dtt = time.perf_counter() - t0
    extra["tiny_config"] = {"value": round(tiny.n_query * tiny.chunks / dtt, 1), "unit": "query-tokens/s",
                            "sample": f"the whole 8-chunk fp32 stream, {dtt:.3f} s measured"}
    # FP4 stack: 1 step of chunks 0-7 over an FP4 store (codec included), 1 head
    m4 = LayerModel(S, W, C, T, 1, D, kv_format="fp4")
    t0 = time.perf_counter()
    for c in range(sub_chunks):
        q, k, v = ins[c][steps - 1]
        m4.attn_chunk(q.values, k.values, v.values)
        m4.commit(k.values, v.values, k.bits, v.bits)
    dt4 = time.perf_counter() - t0
    fp4_s = dt4 * stack_flops / flops(range(sub_chunks), 1, 1)
    extra["fp4_stack"] = {"value": round(rows_stack / fp4_s, 1), "unit": "query-tokens/s",
                          "sample": (f"1 denoise step of chunks 0-{sub_chunks - 1} over an FP4 store "
                                     f"(codec included), layer 0, 1/{shape.heads} heads, {dt4:.1f} s "
                                     "measured, scaled by flops to the FP4 stack")}
    # one layer of the prompt-switch recache (12 held frames, 512 text tokens), 1 head
    mr = LayerModel(S, W, C, T, 1, D)
    for c in range(4):
        mr.commit(ins[c][0][1].values, ins[c][0][2].values)
    rows = len(mr.held()) * T
    rin = synth.recache_inputs(sub1, 0, rows, 512)
    t0 = time.perf_counter()
    mr.recache(*(x.values for x in rin))
    dtr = time.perf_counter() - t0
    extra["recache_30_layers"] = {"value": round(rows / (dtr * shape.heads), 1),
                                  "unit": "query-tokens/s",
                                  "sample": (f"one layer's recache ({rows} rows: block-causal self + 512-key "
                                             f"cross), 1/{shape.heads} heads, {dtr:.1f} s measured, "
                                             "scaled by heads (30 layers: the same rate)")}
    # one steady chunk call on one thread, 1 head
    q, k, v = ins[sub_chunks - 1][0]
    single = None
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            m.attn_chunk(q.values, k.values, v.values)
            dt1 = time.perf_counter() - t0
        single = {"value": round(n / (dt1 * shape.heads), 1), "unit": "query-tokens/s", "cores": 1,
                  "sample": (f"one steady chunk call (4680 rows x 23,400 keys), 1/{shape.heads} heads, "
                             f"BLAS limited to 1 thread, {dt1:.1f} s measured, scaled by heads")}
    except Exception as e:  # threadpoolctl missing: the leg is reported as not run
        single = {"value": None, "note": f"not run: {e}"}
    extra["steady_call_1_thread"] = single
    threads = _blas_threads()
    return {"value": round(rows_stack / stack_s, 1), "unit": "query-tokens/s",
            "cores": threads if threads else os.cpu_count(), "kind": "oracle",
            "sample": (f"fp64 oracle on the stack: layer 0, {steps} denoise steps, chunks 0-{sub_chunks - 1} "
                       f"(attention + commit), 1/{shape.heads} heads x {n} rows, {dt:.1f} s measured "
                       f"({sub_flops / 1e12:.2f} TFLOP), scaled by algorithmic flops to the whole stack "
                       f"({stack_flops / 1e15:.3f} PFLOP): {stack_s / 3600:.1f} h"),
            "cores_note": "BLAS threads the oracle's matrix products used (threadpoolctl)",
            "host": host_cores(), "other_workloads": extra}


def stack_pass(cache, pool, out, L, steps, chunks, timer=None):
    """One pass of the stack workload on `cache`: per chunk, 4 denoise steps of attention
    over the L layers, then one batched commit of the last step's K/V into all layers.
    Inputs cycle through `pool`. With a timer, each chunk's attention launches and its
    commit launch are bracketed by events."""
    i = 0
    for c in range(chunks):
        if timer:
            s = timer.start()
        last_k, last_v = [], []
        for st in range(steps):
            for layer in range(L):
                q, k, v = pool[i % len(pool)]
                i += 1
                cache.attn_chunk(layer, q, k, v, out=out)
                if st == steps - 1:
                    last_k.append(k)
                    last_v.append(v)
        if timer:
            timer.stop(s, "attn")
            s = timer.start()
        cache.commit_layers(0, last_k, last_v)
        if timer:
            timer.stop(s, "commit")


def stack_flops(shape, attn_flops, L=30, steps=4, chunks=80):
    n, H, D, T = shape.n_query, shape.heads, shape.head_dim, shape.tokens_per_frame
    C, S, W = shape.chunk_frames, shape.sink_frames, shape.window_frames
    return sum(L * steps * attn_flops(n, visible_keys(c, C, S, W, T), H, D) for c in range(chunks))


def stack_row(torch, shape, Cache, attn_flops, kv_format, pool):
    """One pass of the stack workload from an empty cache with the given KV store, timed as
    a whole with events."""
    L, steps, chunks = 30, 4, 80
    n, H, D, T = shape.n_query, shape.heads, shape.head_dim, shape.tokens_per_frame
    C, S, W = shape.chunk_frames, shape.sink_frames, shape.window_frames
    cache = Cache(L, H, D, T, C, S, W, kv_format=kv_format)
    out = torch.empty((n, H, D), dtype=torch.bfloat16, device="cuda")
    flops = stack_flops(shape, attn_flops)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    stack_pass(cache, pool, out, L, steps, chunks)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1)
    rows = n * L * steps * chunks
    return {"ms": round(ms, 2), "query_rows": rows, "query_tokens_per_s": round(rows / ms * 1e3, 1),
            "tflops": round(flops / ms / 1e9, 1),
            "frac_bf16_peak": round(flops / ms / 1e9 / MFMA_BF16_PEAK_TFLOPS, 4),
            "pflop": round(flops / 1e15, 4),
            "work": f"{L} layers x {steps} steps x {chunks} chunks, {kv_format} KV, attention + batched commits"}


def composite_row(torch, shape, Cache, attn_flops, pool):
    """The interactive composite: the dense stack stream (30 layers x 4 steps x 80 chunks)
    with a prompt switch at every sixth of the stream (six prompts, five switches), where all
    30 layers are recached with a new 512-token prompt before the next chunk. Timed end to end
    with events; inputs cycle through resident synthetic sets."""
    L, steps, chunks, n_text = 30, 4, 80, 512
    n, H, D, T = shape.n_query, shape.heads, shape.head_dim, shape.tokens_per_frame
    C, S, W = shape.chunk_frames, shape.sink_frames, shape.window_frames
    switches = [round(chunks * j / 6) for j in range(1, 6)]
    cache = Cache(L, H, D, T, C, S, W)
    out = torch.empty((n, H, D), dtype=torch.bfloat16, device="cuda")
    rows = (S + W) * T
    g = torch.Generator(device="cuda")
    g.manual_seed(13)
    big = [(torch.randn((rows, H, D), generator=g, device="cuda") * 0.5).to(torch.bfloat16)
           for _ in range(4)]
    txt = [(torch.randn((n_text, H, D), generator=g, device="cuda") * 0.5).to(torch.bfloat16)
           for _ in range(2)]
    o = torch.empty_like(big[0])
    ox = torch.empty_like(big[0])
    flops = 0.0
    qrows = 0
    for c in range(chunks):
        flops += L * steps * attn_flops(n, visible_keys(c, C, S, W, T), H, D)
        qrows += L * steps * n
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    i = 0
    for c in range(chunks):
        if c in switches:
            held = cache.held_rows(0)
            for layer in range(L):
                cache.recache(layer, big[0][:held], big[1][:held], big[2][:held], big[3][:held],
                              txt[0], txt[1], out=o[:held], out_x=ox[:held])
        last_k, last_v = [], []
        for st in range(steps):
            for layer in range(L):
                q, k, v = pool[i % len(pool)]
                i += 1
                cache.attn_chunk(layer, q, k, v, out=out)
                if st == steps - 1:
                    last_k.append(k)
                    last_v.append(v)
        cache.commit_layers(0, last_k, last_v)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1)
    # recache flops: held frames in groups of one chunk, group j seeing groups 0..j (block
    # causal), plus the cross-attention to n_text keys
    for c in switches:
        F = c * C
        held_frames = min(F, S) + min(max(F - S, 0), W)
        groups = held_frames // C
        self_pairs = sum(C * T * (j + 1) * C * T for j in range(groups))
        flops += L * (self_pairs + held_frames * T * n_text) * H * 4 * D
        qrows += L * 2 * held_frames * T
    return {"ms": round(ms, 2), "query_rows": qrows, "query_tokens_per_s": round(qrows / ms * 1e3, 1),
            "tflops": round(flops / ms / 1e9, 1),
            "frac_bf16_peak": round(flops / ms / 1e9 / MFMA_BF16_PEAK_TFLOPS, 4),
            "pflop": round(flops / 1e15, 4), "switches_at_chunk": switches,
            "work": (f"{L} layers x {steps} steps x {chunks} chunks, dense KV, attention + batched commits, "
                     f"{len(switches)} prompt switches each recaching {L} layers ({n_text} text tokens)")}


def commit_batch_row(torch, shape, Cache, kv_format, pairs, batched=False):
    """Per-layer commit time of 30 steady commits (one per layer of a 30-layer cache), either
    30 back-to-back ll_cache_commit calls or one ll_cache_commit_layers call for all 30
    layers (the stack workload's pattern). Every layer commits its own K/V pair (30 distinct
    pairs, 862 MB: more than the caches hold, as in the stack); events bracket each batch,
    recorded behind a GPU spin that covers the host's enqueueing of the batch (gpu_hold)."""
    L = 30
    n, H, D = shape.n_query, shape.heads, shape.head_dim
    cache = Cache(L, H, D, shape.tokens_per_frame, shape.chunk_frames, shape.sink_frames,
                  shape.window_frames, kv_format=kv_format)
    ks, vs = [p[0] for p in pairs[:L]], [p[1] for p in pairs[:L]]
    # warm every layer past the commit that moves the sink frames out of the window (timed
    # in its own row), so each timed commit is a steady-state one
    for _ in range(shape.window_frames // shape.chunk_frames + 1):
        for layer in range(L):
            cache.commit(layer, ks[layer], vs[layer])
    tm = EventTimer(torch)
    for rep in range(10):
        s = tm.start(HOLD_MS)
        if batched:
            cache.commit_layers(0, ks, vs)
        else:
            for layer in range(L):
                cache.commit(layer, ks[layer], vs[layer])
        tm.stop(s, "batch")
    torch.cuda.synchronize()
    ms = tm.totals()["batch"][0] / (10 * L)
    if kv_format == "fp4":
        nbytes = 2 * n * H * D * 2 + 2 * n * H * (D // 2 + D // 16)
    else:
        nbytes = 2 * 2 * n * H * D * 2
    gbs = nbytes / ms / 1e6
    return {"us_per_commit": round(ms * 1e3, 3), "bytes": nbytes, "gbs": round(gbs, 1),
            "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}


def copy_ceiling_row(torch, pairs):
    """Context for the commit rows: a plain device copy (torch's copy kernel) of the bytes the
    batched commit moves: 30 distinct K/V pairs (2 x 14.38 MB each) copied back to back into
    30 destination pairs; per-pair time, events bracketing each batch of 30 (behind a GPU spin,
    as in commit_batch_row)."""
    dst = [(torch.empty_like(k), torch.empty_like(v)) for k, v in pairs]
    for (k, v), (dk, dv) in zip(pairs, dst):
        dk.copy_(k)
        dv.copy_(v)
    tm = EventTimer(torch)
    for rep in range(10):
        s = tm.start(HOLD_MS)
        for (k, v), (dk, dv) in zip(pairs, dst):
            dk.copy_(k)
            dv.copy_(v)
        tm.stop(s, "batch")
    torch.cuda.synchronize()
    ms = tm.totals()["batch"][0] / (10 * len(pairs))
    k = pairs[0][0]
    nbytes = 2 * 2 * k.numel() * k.element_size()
    gbs = nbytes / ms / 1e6
    return {"us_per_pair": round(ms * 1e3, 3), "bytes": nbytes, "gbs": round(gbs, 1),
            "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}


def quant_chunk_row(torch, k, v):
    """Context for the FP4 commit row: ll_kv_quant over exactly the bytes a quantising commit
    moves (one chunk's K and V: 2 x 14.38 MB of bf16 read, 2 x 4.04 MB of codes and scales
    written), without the slot scatter; 30 back-to-back launches into 30 output buffers, called
    through the C ABI with prepared arguments, events bracketing each batch like
    commit_batch_row."""
    import ctypes
    from windowed_attention_kv_amd import _lib
    lib = _lib.lib()
    x = torch.cat([k.reshape(-1, k.shape[-1]), v.reshape(-1, v.shape[-1])]).contiguous()
    rows, D = x.shape
    outs = [(torch.empty((rows, D // 2), dtype=torch.uint8, device="cuda"),
             torch.empty((rows, D // 16), dtype=torch.uint8, device="cuda")) for _ in range(30)]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    args = [(ctypes.c_void_p(x.data_ptr()), rows, D, ctypes.c_void_p(pk.data_ptr()),
             ctypes.c_void_p(sc.data_ptr()), stream) for pk, sc in outs]
    for a in args[:3]:
        _lib.check(lib, lib.ll_kv_quant(*a))
    tm = EventTimer(torch)
    for rep in range(10):
        s = tm.start(HOLD_MS)
        for a in args:
            lib.ll_kv_quant(*a)
        tm.stop(s, "batch")
    torch.cuda.synchronize()
    for a in args:
        _lib.check(lib, lib.ll_kv_quant(*a))
    ms = tm.totals()["batch"][0] / (10 * 30)
    nbytes = x.numel() * 2 + outs[0][0].numel() + outs[0][1].numel()
    gbs = nbytes / ms / 1e6
    return {"us_per_quant": round(ms * 1e3, 3), "bytes": nbytes, "gbs": round(gbs, 1),
            "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}


def spill_commit_row(torch, shape, Cache, k, v):
    """The commit that retires a shot's sink frames from the window (multi-shot sink): with
    S = C = 3 and W = 9, the fourth commit after a shot boundary also moves the shot's first 3
    frames from their window slots to the sink slots. Per-commit time of 30 such commits (one
    per layer), events behind a GPU spin as in commit_batch_row; bytes = the plain commit's
    plus the moved frames read and written."""
    L = 30
    n, H, D, T = shape.n_query, shape.heads, shape.head_dim, shape.tokens_per_frame
    C, S, W = shape.chunk_frames, shape.sink_frames, shape.window_frames
    cache = Cache(L, H, D, T, C, S, W)
    tm = EventTimer(torch)
    for rep in range(11):
        for layer in range(L):
            cache.new_shot(layer)
            for _ in range(W // C):
                cache.commit(layer, k, v)
        s = tm.start(HOLD_MS)
        for layer in range(L):
            cache.commit(layer, k, v)
        tm.stop(s, "spill" if rep else "warm")
    torch.cuda.synchronize()
    ms = tm.totals()["spill"][0] / (10 * L)
    moved = 2 * 2 * S * T * H * D * 2
    nbytes = 2 * 2 * n * H * D * 2 + moved
    gbs = nbytes / ms / 1e6
    return {"us_per_commit": round(ms * 1e3, 3), "bytes": nbytes, "gbs": round(gbs, 1),
            "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
            "note": f"commit that moves {S} sink frames (K and V) to the sink slots"}


def extra_rows(torch, shape, Cache, kv_quant, attn_flops):
    """Commit batches, FP4 stream, standalone quant, recache and the 30-layer stacks."""
    res = {}
    n, H, D = shape.n_query, shape.heads, shape.head_dim
    inputs = gen_inputs(torch, shape.chunks, n, H, D, 7, "cuda")
    out = torch.empty((n, H, D), dtype=torch.bfloat16, device="cuda")
    res["layer_stream"] = layer_stream_row(torch, shape, Cache, attn_flops, inputs)
    progress("row done: single-layer stream")
    # 30 distinct (K, V) pairs for the commit rows (the 20 chunks' q, k, v tensors, paired up)
    flat = [t for trip in inputs for t in trip]
    pairs = [(flat[2 * i], flat[2 * i + 1]) for i in range(30)]
    res["commit_layers_30_dense"] = commit_batch_row(torch, shape, Cache, "dense", pairs, batched=True)
    res["commit_layers_30_fp4"] = commit_batch_row(torch, shape, Cache, "fp4", pairs, batched=True)
    res["commit_30_layers"] = commit_batch_row(torch, shape, Cache, "dense", pairs)
    res["fp4_commit_30_layers"] = commit_batch_row(torch, shape, Cache, "fp4", pairs)
    res["spill_commit_30_layers"] = spill_commit_row(torch, shape, Cache, inputs[0][1], inputs[0][2])
    res["plain_copy_same_bytes"] = copy_ceiling_row(torch, pairs)
    del pairs, flat
    res["kv_quant_same_bytes_as_fp4_commit"] = quant_chunk_row(torch, inputs[0][1], inputs[0][2])
    progress("rows done: commits, copy ceiling, codec")
    # FP4 KV store at the layer shape: steady-state attention (15 visible frames)
    c4 = Cache(1, H, D, shape.tokens_per_frame, shape.chunk_frames, shape.sink_frames,
               shape.window_frames, kv_format="fp4")
    for rep in range(3):
        c4.reset()
        tm = EventTimer(torch)
        for c, (q, k, v) in enumerate(inputs):
            s = tm.start()
            c4.attn_chunk(0, q, k, v, out=out)
            tm.stop(s, "attn_steady" if c >= 4 else "attn_fill")
            c4.commit(0, k, v)
        torch.cuda.synchronize()
    tot = tm.totals()
    steady_flops = attn_flops(n, 23400, H, D)
    ms = tot["attn_steady"][0] / tot["attn_steady"][1]
    res["fp4_attention_steady"] = {"ms": round(ms, 4), "tflops": round(steady_flops / ms / 1e9, 1),
                                   "frac_bf16_peak": round(steady_flops / ms / 1e9 / MFMA_BF16_PEAK_TFLOPS, 4)}
    # dense steady-state attention for comparison
    cd = Cache(1, H, D, shape.tokens_per_frame, shape.chunk_frames, shape.sink_frames,
               shape.window_frames)
    tm = EventTimer(torch)
    for c, (q, k, v) in enumerate(inputs):
        s = tm.start()
        cd.attn_chunk(0, q, k, v, out=out)
        tm.stop(s, "attn_steady" if c >= 4 else "attn_fill")
        cd.commit(0, k, v)
    torch.cuda.synchronize()
    tot = tm.totals()
    ms = tot["attn_steady"][0] / tot["attn_steady"][1]
    res["attention_steady"] = {"ms": round(ms, 4), "tflops": round(steady_flops / ms / 1e9, 1),
                               "frac_bf16_peak": round(steady_flops / ms / 1e9 / MFMA_BF16_PEAK_TFLOPS, 4),
                               "keys": 23400}
    # the chunk's text cross-attention (512 text tokens) fused into the same launch
    gx = torch.Generator(device="cuda")
    gx.manual_seed(17)
    qx = (torch.randn((n, H, D), generator=gx, device="cuda") * 0.5).to(torch.bfloat16)
    ktx = (torch.randn((512, H, D), generator=gx, device="cuda") * 0.5).to(torch.bfloat16)
    vtx = (torch.randn((512, H, D), generator=gx, device="cuda") * 0.5).to(torch.bfloat16)
    ox = torch.empty_like(out)
    tm = EventTimer(torch)
    for rep in range(2):
        cd.reset()
        for c, (q, k, v) in enumerate(inputs):
            s = tm.start()
            cd.attn_chunk_cross(0, q, k, v, qx, ktx, vtx, out=out, out_x=ox)
            tm.stop(s, "fused_steady" if c >= 4 and rep > 0 else "fused_other")
            cd.commit(0, k, v)
    torch.cuda.synchronize()
    tot = tm.totals()
    ms_f = tot["fused_steady"][0] / tot["fused_steady"][1]
    fused_flops = steady_flops + attn_flops(n, 512, H, D)
    res["attention_cross_fused_steady"] = {
        "ms": round(ms_f, 4), "tflops": round(fused_flops / ms_f / 1e9, 1),
        "frac_bf16_peak": round(fused_flops / ms_f / 1e9 / MFMA_BF16_PEAK_TFLOPS, 4),
        "cross_us_over_self_only": round((ms_f - res["attention_steady"]["ms"]) * 1e3, 1),
        "note": "self (23400 keys) + text cross-attention (512 keys) in one launch"}
    del qx, ktx, vtx, ox
    res.update(share_rows(torch, shape, Cache, attn_flops, inputs))
    # standalone quant of one 12-frame cache (K and V): 2 x 18720 x 1536 elements
    x = torch.randn((2 * 18720 * H, D), device="cuda").mul_(0.5).to(torch.bfloat16)
    pk = torch.empty((x.shape[0], D // 2), dtype=torch.uint8, device="cuda")
    sc = torch.empty((x.shape[0], D // 16), dtype=torch.uint8, device="cuda")
    for _ in range(3):
        kv_quant(x, pk, sc)
    tm = EventTimer(torch)
    for _ in range(10):
        s = tm.start(HOLD_MS)
        kv_quant(x, pk, sc)
        tm.stop(s, "quant")
    torch.cuda.synchronize()
    ms = tm.totals()["quant"][0] / 10
    qbytes = x.numel() * 2 + pk.numel() + sc.numel()
    res["kv_quant_12_frames"] = {"ms": round(ms, 5), "bytes": qbytes, "gbs": round(qbytes / ms / 1e6, 1),
                                 "frac_hbm": round(qbytes / ms / 1e6 / HBM_PEAK_GBS, 4)}
    del x, pk, sc
    res["recache_30_layers"] = recache_row(torch, shape, Cache, inputs)
    progress("row done: 30-layer recache")
    pool = gen_inputs(torch, 8, n, H, D, 21, "cuda")
    res["stack_fp4"] = stack_row(torch, shape, Cache, attn_flops, "fp4", pool)
    progress("row done: FP4 stack")
    res["interactive_composite"] = composite_row(torch, shape, Cache, attn_flops, pool)
    progress("row done: interactive composite")
    res["gemm_bf16_ceiling"] = gemm_ceiling_row(torch)
    res["vendor_flash_attention_same_shape"] = sdpa_context_row(torch, shape, attn_flops)
    progress("rows done: vendor context rows")
    return res


def share_rows(torch, shape, Cache, attn_flops, inputs):
    """One GPU's share of the heads under 4-way sequence parallelism: the layer shape at 3
    heads (57 query blocks on 256 CUs, so chunk attention runs with the split schedule),
    20-chunk streams over a dense and an FP4 cache; steady chunks timed."""
    res = {}
    n, D, Hs = shape.n_query, shape.head_dim, 3
    share_in = [tuple(t[:, :Hs].contiguous() for t in trip) for trip in inputs]
    outs = torch.empty((n, Hs, D), dtype=torch.bfloat16, device="cuda")
    share_flops = attn_flops(n, 23400, Hs, D)
    for kv_format, row in (("dense", "share_3_heads_steady"), ("fp4", "fp4_share_3_heads_steady")):
        cs = Cache(1, Hs, D, shape.tokens_per_frame, shape.chunk_frames, shape.sink_frames,
                   shape.window_frames, kv_format=kv_format)
        for rep in range(2):
            cs.reset()
            tm = EventTimer(torch)
            for c, (q, k, v) in enumerate(share_in):
                s = tm.start()
                cs.attn_chunk(0, q, k, v, out=outs)
                tm.stop(s, "attn_steady" if c >= 4 else "attn_fill")
                cs.commit(0, k, v)
            torch.cuda.synchronize()
        tot = tm.totals()
        ms = tot["attn_steady"][0] / tot["attn_steady"][1]
        res[row] = {"ms": round(ms, 4), "tflops": round(share_flops / ms / 1e9, 1),
                    "frac_bf16_peak": round(share_flops / ms / 1e9 / MFMA_BF16_PEAK_TFLOPS, 4),
                    "note": (f"3 of 12 heads (4-way sequence-parallel share), {kv_format} cache, "
                             "split schedule")}
    del share_in, outs, cs
    return res


def steady_calls_row(torch, shape, Cache, attn_flops, inputs, calls=40):
    """The steady chunk call alone (12 heads, 4680 query rows over 23,400 keys): a layer is
    filled with 5 chunks, then the 6th chunk's attention runs `calls` times back to back,
    events around the batch (behind a GPU spin, gpu_hold), so that a profiler sees those
    launches only."""
    n, H, D = shape.n_query, shape.heads, shape.head_dim
    cache = Cache(1, H, D, shape.tokens_per_frame, shape.chunk_frames, shape.sink_frames,
                  shape.window_frames)
    out = torch.empty((n, H, D), dtype=torch.bfloat16, device="cuda")
    for q, k, v in inputs[:5]:
        cache.attn_chunk(0, q, k, v, out=out)
        cache.commit(0, k, v)
    q, k, v = inputs[5]
    tm = EventTimer(torch)
    s = tm.start(HOLD_MS)
    for _ in range(calls):
        cache.attn_chunk(0, q, k, v, out=out)
    tm.stop(s, "steady")
    torch.cuda.synchronize()
    ms = tm.totals()["steady"][0] / calls
    fl = attn_flops(n, 23400, H, D)
    return {"calls": calls, "ms": round(ms, 4), "tflops": round(fl / ms / 1e9, 1),
            "frac_bf16_peak": round(fl / ms / 1e9 / MFMA_BF16_PEAK_TFLOPS, 4)}


def recache_row(torch, shape, Cache, inputs):
    """The prompt-switch recache (12 held frames, 512 text tokens) of every layer of a
    filled 30-layer cache: per layer block-causal self + cross + slot rewrite."""
    H, D = shape.heads, shape.head_dim
    L = 30
    cr = Cache(L, H, D, shape.tokens_per_frame, shape.chunk_frames, shape.sink_frames,
               shape.window_frames)
    for c in range(10):
        for layer in range(L):
            cr.commit(layer, inputs[c][1], inputs[c][2])
    rows = 12 * shape.tokens_per_frame
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    big = [(torch.randn((rows, H, D), generator=g, device="cuda") * 0.5).to(torch.bfloat16)
           for _ in range(4)]
    txt = [(torch.randn((512, H, D), generator=g, device="cuda") * 0.5).to(torch.bfloat16)
           for _ in range(2)]
    o = torch.empty_like(big[0])
    ox = torch.empty_like(big[0])
    cr.recache(0, big[0], big[1], big[2], big[3], txt[0], txt[1], out=o, out_x=ox)
    torch.cuda.synchronize()
    tm = EventTimer(torch)
    for _ in range(2):
        s = tm.start()
        for layer in range(L):
            cr.recache(layer, big[0], big[1], big[2], big[3], txt[0], txt[1], out=o, out_x=ox)
        tm.stop(s, "recache")
    torch.cuda.synchronize()
    ms = tm.totals()["recache"][0] / 2
    # visible pairs: group g of 4680 rows sees (g+1)*4680 keys; cross: 512 keys
    self_pairs = sum(4680 * (gg + 1) * 4680 for gg in range(4))
    fl = L * (self_pairs + rows * 512) * H * 4 * D
    row = {"ms": round(ms, 3), "tflops": round(fl / ms / 1e9, 1),
           "frac_bf16_peak": round(fl / ms / 1e9 / MFMA_BF16_PEAK_TFLOPS, 4),
           "query_tokens_per_s": round(L * rows / ms * 1e3, 1),
           "note": "per layer: block-causal self + cross (512 text keys) + slot rewrite"}
    del cr, big, txt, o, ox
    return row


def layer_stream_row(torch, shape, Cache, attn_flops, inputs, passes=5):
    """The single-layer workload: 20 chunks streamed from an empty 1-layer cache, each chunk
    ll_attn_chunk then ll_cache_commit; events around every attention and commit launch."""
    n, H, D, T = shape.n_query, shape.heads, shape.head_dim, shape.tokens_per_frame
    C, S, W = shape.chunk_frames, shape.sink_frames, shape.window_frames
    cache = Cache(1, H, D, T, C, S, W)
    _OUT[0] = torch.empty((n, H, D), dtype=torch.bfloat16, device="cuda")
    run_stream(cache, inputs)
    torch.cuda.synchronize()
    timer = EventTimer(torch)
    t0 = time.perf_counter()
    for _ in range(passes):
        cache.reset()
        run_stream(cache, inputs, timer)
    torch.cuda.synchronize()
    ms_pass = (time.perf_counter() - t0) * 1e3 / passes
    tot = timer.totals()
    flops = sum(attn_flops(n, visible_keys(c, C, S, W, T), H, D) for c in range(shape.chunks))
    attn_ms = tot["attn"][0] / tot["attn"][1]
    commit_ms = tot["commit"][0] / tot["commit"][1]
    commit_bytes = 2 * 2 * n * H * D * 2
    return {"ms_per_stream": round(ms_pass, 3), "query_tokens_per_s": round(n * shape.chunks / ms_pass * 1e3, 1),
            "attention_avg_launch_ms": round(attn_ms, 4),
            "attention_tflops": round(flops / shape.chunks / attn_ms / 1e9, 1),
            "frac_bf16_peak": round(flops / shape.chunks / attn_ms / 1e9 / MFMA_BF16_PEAK_TFLOPS, 4),
            "commit_avg_launch_ms": round(commit_ms, 5),
            "commit_frac_hbm": round(commit_bytes / commit_ms / 1e6 / HBM_PEAK_GBS, 4),
            "work": "1 layer, 20 chunks streamed from an empty cache (attention + commit per chunk)"}


def gemm_ceiling_row(torch, m=8192):
    """Context for the attention roofline: a plain bf16 GEMM (torch.matmul, the vendor BLAS)
    of m x m x m on the same device, its sustained rate and fraction of the dense bf16 peak."""
    a = torch.randn((m, m), device="cuda").to(torch.bfloat16)
    b = torch.randn((m, m), device="cuda").to(torch.bfloat16)
    c = torch.empty((m, m), device="cuda", dtype=torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b, out=c)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    reps = 20
    e0.record()
    for _ in range(reps):
        torch.matmul(a, b, out=c)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    tf = 2.0 * m ** 3 / ms / 1e9
    return {"ms": round(ms, 4), "tflops": round(tf, 1), "frac_bf16_peak": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
            "note": f"torch.matmul bf16 {m}x{m}x{m}: the vendor GEMM's sustained rate on this device"}


def sdpa_context_row(torch, shape, attn_flops):
    """Context for the attention roofline: torch's fused attention (scaled_dot_product_attention
    restricted to its flash backend, so it can never fall back to the unfused path) on the
    steady chunk's shape: 4680 queries x 23400 keys x 12 heads x 128, bf16, no mask. Timed with
    each flash library the torch build offers (AOTriton, CK); a library it lacks is reported as
    unavailable."""
    from torch.nn.attention import SDPBackend, sdpa_kernel
    n, H, D = shape.n_query, shape.heads, shape.head_dim
    keys = (shape.sink_frames + shape.window_frames + shape.chunk_frames) * shape.tokens_per_frame
    g = torch.Generator(device="cuda")
    g.manual_seed(23)
    q = (torch.randn((1, H, n, D), generator=g, device="cuda") * 0.5).to(torch.bfloat16)
    k = (torch.randn((1, H, keys, D), generator=g, device="cuda") * 0.5).to(torch.bfloat16)
    v = (torch.randn((1, H, keys, D), generator=g, device="cuda") * 0.5).to(torch.bfloat16)
    flops = attn_flops(n, keys, H, D)
    res = {"keys": keys,
           "note": "torch.nn.functional.scaled_dot_product_attention, flash backend only, same shape "
                   "as the steady chunk call"}
    pick = getattr(torch.backends.cuda, "preferred_rocm_fa_library", None)
    before = pick() if pick else None
    for lib in ("aotriton", "ck"):
        try:
            if pick:
                pick(lib)
            elif lib != "aotriton":
                raise RuntimeError("this torch build has no flash-library switch")
            with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
                for _ in range(3):
                    o = torch.nn.functional.scaled_dot_product_attention(q, k, v)
                torch.cuda.synchronize()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                reps = 10
                e0.record()
                for _ in range(reps):
                    o = torch.nn.functional.scaled_dot_product_attention(q, k, v)
                e1.record()
                torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            res[lib] = {"ms": round(ms, 4), "tflops": round(flops / ms / 1e9, 1),
                        "frac_bf16_peak": round(flops / ms / 1e9 / MFMA_BF16_PEAK_TFLOPS, 4)}
            del o
        except RuntimeError as e:
            res[lib] = {"unavailable": str(e).splitlines()[0][:200]}
    if pick and before is not None:
        pick(before)
    del q, k, v
    return res


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the library has no "
              "multi-GPU path; the hot path shards by head with no communication inside it",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from windowed_attention_kv_amd import Cache, attn_flops, kv_quant, synth

    layer_shape = synth.CONFIGS["layer"]
    if args.row:
        torch.cuda.set_device(0)
        ls = layer_shape
        inputs = gen_inputs(torch, ls.chunks, ls.n_query, ls.heads, ls.head_dim, 7, "cuda")
        if args.row == "share":
            rows = share_rows(torch, ls, Cache, attn_flops, inputs)
        elif args.row == "vendor-flash":
            rows = {"vendor_flash_attention_same_shape": sdpa_context_row(torch, ls, attn_flops)}
        elif args.row == "steady":
            rows = {"attention_steady_calls": steady_calls_row(torch, ls, Cache, attn_flops, inputs)}
        else:
            rows = {"recache_30_layers": recache_row(torch, ls, Cache, inputs)}
        print(json.dumps({"row": args.row, "rows": rows}), flush=True)
        return
    shape = synth.CONFIGS["stack"]
    L, steps, chunks = shape.layers, shape.steps, shape.chunks
    n, H, D, T = shape.n_query, shape.heads, shape.head_dim, shape.tokens_per_frame
    C, S, W = shape.chunk_frames, shape.sink_frames, shape.window_frames
    torch.cuda.set_device(0)
    pool = gen_inputs(torch, 8, n, H, D, 1234, "cuda")
    out = torch.empty((n, H, D), dtype=torch.bfloat16, device="cuda")
    cache = Cache(L, H, D, T, C, S, W)
    flops_step = stack_flops(shape, attn_flops, L, steps, chunks)
    launches = L * steps * chunks

    for w in range(args.warmup):
        cache.reset()
        stack_pass(cache, pool, out, L, steps, chunks)
        torch.cuda.synchronize()
        progress(f"warm-up stack pass {w + 1}/{args.warmup} done")

    timer = EventTimer(torch)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for st in range(args.steps):
        cache.reset()
        stack_pass(cache, pool, out, L, steps, chunks, timer)
        # enqueued, not synchronised: the host runs at most a launch queue ahead of the GPU
        progress(f"timed stack pass {st + 1}/{args.steps} enqueued")
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    progress(f"timed passes done: {wall * 1e3 / args.steps:.1f} ms per pass")
    tot = timer.totals()
    ms_step = wall * 1e3 / args.steps
    # average attention launch: each chunk's 120 back-to-back attention launches are bracketed
    # by one pair of events, so the launch gaps between them are included
    attn_ms = tot["attn"][0] / (launches * args.steps)
    attn_flops_launch = flops_step / launches              # average algorithmic flops per launch
    achieved = attn_flops_launch / attn_ms / 1e9           # TFLOP/s
    commit_ms = tot["commit"][0] / tot["commit"][1]        # one batched commit of 30 layers
    commit_bytes = L * 2 * 2 * n * H * D * 2               # read + write of K and V, every layer
    rows_step = n * launches

    line = {
        "metric": "query-tokens/s and TFLOP/s for window+sink chunk attention (% bf16 MFMA peak)",
        "value": round(rows_step / (ms_step / 1e3), 1),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": (f"stack: {L} layers x {steps} denoise steps x {chunks} chunks streamed from an "
                                "empty cache; per layer 12 heads x 128, 1560 tok/frame, chunk 3 frames (4680 "
                                "query rows), sink 3 + window 9 frames; chunk attention for every step and "
                                "layer, one batched commit of all layers per chunk"),
                   "query_rows_per_step": rows_step,
                   "attention_launches_per_step": launches,
                   "attention_pflop_per_step": round(flops_step / 1e15, 4),
                   "tflops_whole_step": round(flops_step / (ms_step / 1e3) / 1e12, 1)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": counter_traffic(attn_flops_launch),
                     "traffic_unit": "bytes per launch (FETCH_SIZE x read scale + WRITE_SIZE x write scale)",
                     # Q and O (n x H x D bf16 each) + the visible keys' K and V: per launch the
                     # K/V bytes are 2 * keys * H * D * 2 = flops_per_launch / n
                     "algorithmic_bytes_per_launch": round(2 * n * H * D * 2 + attn_flops_launch / n),
                     "kernel": "attn_bf16_direct_kernel<8,2,false,false>",
                     "avg_launch_ms": round(attn_ms, 4),
                     "avg_flops_per_launch": attn_flops_launch},
        "device": device_info(torch),
        "rows": {"commit_layers_in_stack": {
            "avg_launch_ms": round(commit_ms, 4), "layers_per_launch": L, "bytes": commit_bytes,
            "us_per_layer": round(commit_ms * 1e3 / L, 3),
            "gbs": round(commit_bytes / commit_ms / 1e6, 1),
            "frac_hbm": round(commit_bytes / commit_ms / 1e6 / HBM_PEAK_GBS, 4)}},
    }
    del cache
    if not args.no_extra:
        line["rows"].update(extra_rows(torch, layer_shape, Cache, kv_quant, attn_flops))
    if not args.no_cpu:
        progress("CPU oracle baseline")
        line["cpu_baseline"] = cpu_baseline(layer_shape)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
