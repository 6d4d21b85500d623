"""Benchmark of the window+sink chunk-attention hot path on one MI355X.

One step = one pass of the layer workload (12 heads x 128, 1560 tokens/frame, chunk 3
frames = 4680 query rows, sink 3 + window 9 frames, 20 chunks streamed from an empty cache):
for each chunk, ll_attn_chunk then ll_cache_commit. Inputs are synthetic bf16 N(0, 0.25),
generated on the GPU before timing (resident in HBM). Prints ONE JSON line.

value = query rows attended per second over the whole step (attention + commit);
roofline = the attention kernel against the bf16 dense MFMA peak, from HIP events recorded on
the launch stream around every attention launch inside the timed region; extra rows report
the commit, the FP4 path and the recache, each timed on its own after the main loop.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 (published)
HBM_PEAK_GBS = 8000.0              # MI355X HBM3E (published)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extra", action="store_true", help="skip the FP4 / recache rows")
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


class EventTimer:
    """Pairs of HIP events recorded on the current (launch) stream."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = []

    def start(self):
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


def cpu_baseline(shape):
    """The fp64 oracle on a bounded sample of the same workload: the whole 20-chunk stream
    (fill-up and steady chunks, attention and commit, inputs drawn beforehand) for 2 of the 12
    heads and all 4680 rows of each chunk, scaled to 12 heads (heads are independent and cost
    the same)."""
    from oracle.model import LayerModel
    from windowed_attention_kv_amd import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    Hs = 2
    sub = synth.shrink(shape, heads=Hs)
    m = LayerModel(sub.sink_frames, sub.window_frames, sub.chunk_frames, sub.tokens_per_frame,
                   Hs, sub.head_dim)
    inputs = [synth.chunk_inputs(sub, 0, 0, c) for c in range(shape.chunks)]
    t0 = time.perf_counter()
    for q, k, v in inputs:
        m.attn_chunk(q.values, k.values, v.values)
        m.commit(k.values, v.values)
    dt = time.perf_counter() - t0
    stream_time = dt * shape.heads / Hs
    extra = {}
    # the same stream over the oracle's FP4 store (codec included), for 1 of the 12 heads
    sub1 = synth.shrink(shape, heads=1)
    m4 = LayerModel(sub1.sink_frames, sub1.window_frames, sub1.chunk_frames,
                    sub1.tokens_per_frame, 1, sub1.head_dim, kv_format="fp4")
    inputs1 = [synth.chunk_inputs(sub1, 0, 0, c) for c in range(shape.chunks)]
    t0 = time.perf_counter()
    for q, k, v in inputs1:
        m4.attn_chunk(q.values, k.values, v.values)
        m4.commit(k.values, v.values, k.bits, v.bits)
    dt4 = time.perf_counter() - t0
    extra["fp4_stream"] = {"value": round(shape.n_query * shape.chunks / (dt4 * shape.heads), 3),
                           "unit": "query-tokens/s",
                           "sample": f"the {shape.chunks}-chunk stream over an FP4 store, 1/{shape.heads} heads, "
                                     f"{dt4:.1f} s measured, scaled by heads"}
    # one layer of the prompt-switch recache (12 held frames, 512 text tokens), 1 head
    mr = LayerModel(sub1.sink_frames, sub1.window_frames, sub1.chunk_frames,
                    sub1.tokens_per_frame, 1, sub1.head_dim)
    for q, k, v in inputs1[:4]:
        mr.commit(k.values, v.values)
    rows = len(mr.held()) * sub1.tokens_per_frame
    rin = synth.recache_inputs(sub1, 0, rows, 512)
    t0 = time.perf_counter()
    mr.recache(*(x.values for x in rin))
    dtr = time.perf_counter() - t0
    extra["recache_30_layers"] = {"value": round(rows / (dtr * shape.heads), 3),
                                  "unit": "query-tokens/s",
                                  "sample": f"one layer's recache ({rows} rows: block-causal self + 512-key "
                                            f"cross), 1/{shape.heads} heads, {dtr:.1f} s measured, "
                                            "scaled by heads (30 layers: the same rate)"}
    return {"value": round(shape.n_query * shape.chunks / stream_time, 3), "unit": "query-tokens/s",
            "cores": int(threads), "kind": "oracle",
            "sample": (f"fp64 oracle, the whole {shape.chunks}-chunk stream (attention + commit) "
                       f"for {Hs}/{shape.heads} heads x {shape.n_query} rows, {dt:.1f} s measured, "
                       f"scaled by heads to {shape.heads}"),
            "other_workloads": extra}


def stack_row(torch, shape, Cache, attn_flops, kv_format, pool):
    """The stack workload: L layers x 4 denoise steps x 80 chunks (only the last step of a
    chunk commits), one pass from an empty cache. Inputs cycle through a pool of resident
    synthetic sets (values do not change the work). Timed as a whole with events."""
    L, steps, chunks = 30, 4, 80
    n, H, D, T = shape.n_query, shape.heads, shape.head_dim, shape.tokens_per_frame
    C, S, W = shape.chunk_frames, shape.sink_frames, shape.window_frames
    cache = Cache(L, H, D, T, C, S, W, kv_format=kv_format)
    out = torch.empty((n, H, D), dtype=torch.bfloat16, device="cuda")
    flops = 0.0
    for c in range(chunks):
        flops += L * steps * attn_flops(n, visible_keys(c, C, S, W, T), H, D)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    i = 0
    for c in range(chunks):
        for st in range(steps):
            for layer in range(L):
                q, k, v = pool[i % len(pool)]
                i += 1
                cache.attn_chunk(layer, q, k, v, out=out)
                if st == steps - 1:
                    cache.commit(layer, k, v)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1)
    rows = n * L * steps * chunks
    return {"ms": round(ms, 2), "query_rows": rows, "query_tokens_per_s": round(rows / ms * 1e3, 1),
            "tflops": round(flops / ms / 1e9, 1),
            "frac_bf16_peak": round(flops / ms / 1e9 / MFMA_BF16_PEAK_TFLOPS, 4),
            "pflop": round(flops / 1e15, 4),
            "work": f"{L} layers x {steps} steps x {chunks} chunks, {kv_format} KV, attention + commits"}


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
        for st in range(steps):
            for layer in range(L):
                q, k, v = pool[i % len(pool)]
                i += 1
                cache.attn_chunk(layer, q, k, v, out=out)
                if st == steps - 1:
                    cache.commit(layer, k, v)
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
            "work": (f"{L} layers x {steps} steps x {chunks} chunks, dense KV, attention + commits, "
                     f"{len(switches)} prompt switches each recaching {L} layers ({n_text} text tokens)")}


def commit_batch_row(torch, shape, Cache, kv_format, k, v):
    """Per-commit time of 30 back-to-back steady commits (one per layer of a 30-layer cache),
    the pattern of the stack workload; events bracket each batch of 30."""
    L = 30
    n, H, D = shape.n_query, shape.heads, shape.head_dim
    cache = Cache(L, H, D, shape.tokens_per_frame, shape.chunk_frames, shape.sink_frames,
                  shape.window_frames, kv_format=kv_format)
    # warm every layer past the commit that moves the sink frames out of the window (timed
    # in its own row), so each timed commit is a steady-state one
    for _ in range(shape.window_frames // shape.chunk_frames + 1):
        for layer in range(L):
            cache.commit(layer, k, v)
    tm = EventTimer(torch)
    for rep in range(10):
        s = tm.start()
        for layer in range(L):
            cache.commit(layer, k, v)
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


def copy_ceiling_row(torch, k, v):
    """Context for the commit rows: a plain device copy (torch's copy kernel) of the same K and V
    a dense commit moves, 2 x 14.38 MB read and written; per-copy time of 30 back-to-back pairs
    of copies, events bracketing each batch like commit_batch_row."""
    dk, dv = torch.empty_like(k), torch.empty_like(v)
    for _ in range(3):
        dk.copy_(k)
        dv.copy_(v)
    tm = EventTimer(torch)
    for rep in range(10):
        s = tm.start()
        for _ in range(30):
            dk.copy_(k)
            dv.copy_(v)
        tm.stop(s, "batch")
    torch.cuda.synchronize()
    ms = tm.totals()["batch"][0] / (10 * 30)
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
        s = tm.start()
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
    per layer); bytes = the plain commit's plus the moved frames read and written."""
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
        s = tm.start()
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
    res["commit_30_layers"] = commit_batch_row(torch, shape, Cache, "dense", inputs[0][1], inputs[0][2])
    res["fp4_commit_30_layers"] = commit_batch_row(torch, shape, Cache, "fp4", inputs[0][1], inputs[0][2])
    res["spill_commit_30_layers"] = spill_commit_row(torch, shape, Cache, inputs[0][1], inputs[0][2])
    res["plain_copy_same_bytes"] = copy_ceiling_row(torch, inputs[0][1], inputs[0][2])
    res["kv_quant_same_bytes_as_fp4_commit"] = quant_chunk_row(torch, inputs[0][1], inputs[0][2])
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
    # one GPU's share of the heads under 4-way sequence parallelism: the layer shape at 3
    # heads (57 query blocks on 256 CUs, so chunk attention runs with the split schedule)
    Hs = 3
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
    # standalone quant of one 12-frame cache (K and V): 2 x 18720 x 1536 elements
    x = torch.randn((2 * 18720 * H, D), device="cuda").mul_(0.5).to(torch.bfloat16)
    pk = torch.empty((x.shape[0], D // 2), dtype=torch.uint8, device="cuda")
    sc = torch.empty((x.shape[0], D // 16), dtype=torch.uint8, device="cuda")
    for _ in range(3):
        kv_quant(x, pk, sc)
    tm = EventTimer(torch)
    for _ in range(10):
        s = tm.start()
        kv_quant(x, pk, sc)
        tm.stop(s, "quant")
    torch.cuda.synchronize()
    ms = tm.totals()["quant"][0] / 10
    qbytes = x.numel() * 2 + pk.numel() + sc.numel()
    res["kv_quant_12_frames"] = {"ms": round(ms, 5), "bytes": qbytes, "gbs": round(qbytes / ms / 1e6, 1),
                                 "frac_hbm": round(qbytes / ms / 1e6 / HBM_PEAK_GBS, 4)}
    del x, pk, sc
    # recache at the prompt-switch shape (12 held frames, 512 text tokens), 30 layers
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
    res["recache_30_layers"] = {"ms": round(ms, 3), "tflops": round(fl / ms / 1e9, 1),
                                "frac_bf16_peak": round(fl / ms / 1e9 / MFMA_BF16_PEAK_TFLOPS, 4),
                                "query_tokens_per_s": round(L * rows / ms * 1e3, 1),
                                "note": "per layer: block-causal self + cross (512 text keys) + slot rewrite"}
    del cr, big, txt, o, ox
    pool = gen_inputs(torch, 8, n, H, D, 21, "cuda")
    res["stack_dense"] = stack_row(torch, shape, Cache, attn_flops, "dense", pool)
    res["stack_fp4"] = stack_row(torch, shape, Cache, attn_flops, "fp4", pool)
    res["interactive_composite"] = composite_row(torch, shape, Cache, attn_flops, pool)
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

    shape = synth.CONFIGS["layer"]
    n, H, D, T = shape.n_query, shape.heads, shape.head_dim, shape.tokens_per_frame
    C, S, W = shape.chunk_frames, shape.sink_frames, shape.window_frames
    torch.cuda.set_device(0)
    inputs = gen_inputs(torch, shape.chunks, n, H, D, 1234, "cuda")
    _OUT[0] = torch.empty((n, H, D), dtype=torch.bfloat16, device="cuda")
    cache = Cache(1, H, D, T, C, S, W)
    flops_step = sum(attn_flops(n, visible_keys(c, C, S, W, T), H, D) for c in range(shape.chunks))

    for _ in range(args.warmup):
        cache.reset()
        run_stream(cache, inputs)
    torch.cuda.synchronize()

    timer = EventTimer(torch)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        cache.reset()
        run_stream(cache, inputs, timer)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    tot = timer.totals()
    ms_step = wall * 1e3 / args.steps
    attn_ms = tot["attn"][0] / tot["attn"][1]            # average attention launch
    attn_flops_launch = flops_step / shape.chunks          # average algorithmic flops per launch
    achieved = attn_flops_launch / attn_ms / 1e9           # TFLOP/s
    commit_ms = tot["commit"][0] / tot["commit"][1]
    commit_bytes = 2 * 2 * n * H * D * 2                   # read + write of K and V

    line = {
        "metric": "query-tokens/s and TFLOP/s for window+sink chunk attention (% bf16 MFMA peak)",
        "value": round(n * shape.chunks / (ms_step / 1e3), 1),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "layer: 12 heads x 128, 1560 tok/frame, chunk 3 (4680 q), sink 3, "
                               "window 9, 20 chunks streamed (attn + commit per chunk)",
                   "query_rows_per_step": n * shape.chunks,
                   "attention_tflop_per_step": round(flops_step / 1e12, 4),
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
        "rows": {"commit": {"avg_launch_ms": round(commit_ms, 5), "bytes": commit_bytes,
                            "gbs": round(commit_bytes / commit_ms / 1e6, 1),
                            "frac_hbm": round(commit_bytes / commit_ms / 1e6 / HBM_PEAK_GBS, 4)}},
    }
    if not args.no_extra:
        line["rows"].update(extra_rows(torch, shape, Cache, kv_quant, attn_flops))
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(shape)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
