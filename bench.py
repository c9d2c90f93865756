#!/usr/bin/env python3
"""Benchmark of the decode attention block on one MI355X.

One step = one decode step of the whole block (fused qkv+g GEMV, split + RoPE
+ KV-slot write, split-K attention with the headwise gate, o_proj) over one
batch, with weights and KV cache already resident in HBM.  The default
workload is the full (causal) layer at 32K context: hidden 2560, position
32767, 32768-row fp16 cache.  To keep the 256 MiB Infinity Cache from serving
"HBM" reads, the step rotates over several copies of weights and cache whose
total exceeds 1 GiB.

Prints ONE JSON line with the throughput (tokens/s), a roofline object for
the dominant kernel (for one sequence over more than one attention chunk the
whole block is one launch of block_fused_kernel: the block's algorithmic HBM
bytes over that launch's average duration, timed with HIP events around the
timed region on the stream it is launched on; otherwise the split-K pass
attn_partial_kernel with its K/V bytes), and the fp64 CPU oracle timed on the
host as a baseline.  `--calibrate-copy MIB` only runs a
plain device copy of known size, to scale rocprofv3's HBM byte counters.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode attn-block tokens/s + achieved HBM GB/s (% peak) at 32K ctx"
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, AMD published
# what the path computes in: bf16 weights and fp16 K/V as stored, every
# product accumulated in fp32
DTYPE = "bf16w+fp16kv->fp32acc"
PROFILE_DIR = os.path.join(ROOT, "profiles")
KERNEL_SRC = os.path.join(ROOT, "gqa_attention_block_amd", "csrc", "gqa_kernels.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def workloads():
    import synth
    return {
        "full32k": synth.headline_full_pos32767,
        "cfg1": synth.cfg1_sliding_pos63,
        "cfg2": synth.cfg2_full_pos4095,
        "cfg3": synth.cfg3_sliding_ring_pos32767,
        "cfg5": synth.cfg5_batched_full,
    }


def attended_rows(case):
    """K/V rows the block reads, from the library's own window function."""
    import gqa_attention_block_amd as gqa
    n = 0
    for s in case.seqs:
        sl, ks, _ = gqa.kv_window(case.is_full, s.position, case.arch.sliding_window,
                                  s.ring_capacity)
        n += sl - ks
    return n


def block_bytes(case) -> int:
    """Algorithmic HBM bytes of one block step: each weight once (bf16), each
    attended K/V row once (fp16, all KV heads), the slot row written, x in and
    out as fp32."""
    a = case.arch
    h, b = a.hidden, case.batch
    w = 2 * (a.qkv_rows + a.num_heads) * h + 2 * h * a.q_dim
    kv_row = 2 * 2 * a.num_kv_heads * a.head_dim          # K and V, fp16
    return w + kv_row * attended_rows(case) + kv_row * b + 4 * h * b * 2


def attention_bytes(case) -> int:
    """Algorithmic HBM bytes of the attention step: attended K/V rows (fp16,
    all KV heads), fp32 q and gate logits in, gated attention out."""
    a = case.arch
    b = case.batch
    kv_row = 2 * 2 * a.num_kv_heads * a.head_dim
    return kv_row * attended_rows(case) + 4 * b * (a.q_dim + a.num_heads + a.q_dim)


def kv_bytes(case) -> int:
    """Algorithmic HBM bytes of the split-K pass: the
    attended K/V rows, fp16, all KV heads, each read once.  The q it reads
    (16 KB) and the partials it writes are workspace traffic, not counted."""
    a = case.arch
    return 2 * 2 * a.num_kv_heads * a.head_dim * attended_rows(case)


def source_digest() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def counted_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` from a committed rocprofv3 PMC summary
    of the same kernel source, or None."""
    path = os.path.join(PROFILE_DIR, f"{kernel}_{workload}_hbm_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    t = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m or not t or m.group(1) != source_digest():
        return None
    return float(t.group(1))


def synth_sinks(case):
    import synth
    return synth.random_sinks(case.arch, 0, 1)


def cpu_baseline(case, seconds: float, sinks=None):
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:                       # pragma: no cover
        cores = os.cpu_count() or 1
    runs, t0 = 0, time.perf_counter()
    while True:
        oracle.block_decode(case.arch, case.is_full, case.w_qkv, case.w_g, case.w_o, case.x,
                            case.seqs, sinks)
        runs += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    tok = case.batch * runs / el
    return {"value": tok, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{runs} full fp64 oracle block steps of this workload ({el:.1f} s)"}


def calibrate_copy(mib: int, reps: int):
    """A plain device-to-device copy of known size, for scaling the HBM byte
    counters (FETCH_SIZE / WRITE_SIZE) read by rocprofv3 --pmc."""
    import torch
    n = mib << 20
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_read": n, "bytes_written": n,
                      "reps": reps}), flush=True)


def stack_bytes(st) -> int:
    """Algorithmic HBM bytes of one token through the stack: per layer the
    block's bytes (block_bytes) plus the RMSNorm (h in, x out, bf16 w) and the
    residual add (h and o in, h out), fp32 [1][hidden]."""
    import numpy as np
    import synth
    total = 0
    h = st.arch.hidden
    for L in st.layers:
        c = synth.BlockCase(name="layer", arch=st.arch, is_full=L.is_full, w_qkv=L.w_qkv, w_g=L.w_g,
                            w_o=L.w_o, x=np.zeros((1, h), np.float32), seqs=[L.cache])
        total += block_bytes(c) + (4 * h * 2 + 2 * h) + 4 * h * 3
        if hasattr(L, "w_gate"):
            # the MLP: post-attention norm (h in, x out, bf16 w), gate/up (bf16
            # weights, x in, two [inter] fp32 out), activation (2 in, 1 out),
            # down (bf16 weights, act in) with the residual add (h in and out)
            inter = int(L.w_gate.shape[0])
            total += (4 * h * 2 + 2 * h) + (2 * 2 * inter * h + 4 * h + 2 * 4 * inter) \
                + 3 * 4 * inter + (2 * h * inter + 4 * inter + 2 * 4 * h)
    return total


def bench_stack(args):
    """The 36-layer stack (RMSNorm -> block -> residual add per layer) at
    position 8191: 9 full layers over 8192 rows, 27 sliding layers over a
    wrapped 512-slot ring.  The stack runs as one gqa_attention_stack_decode
    call per token (one persistent launch for all 36 layers), or with
    --layer-calls as one gqa_attention_layer_decode call per layer.  With
    --workload decoder every layer also runs its MLP (gqa_mlp_decode:
    post-attention norm, erf-GELU gated MLP with intermediate 3 x hidden,
    residual add), i.e. a whole decode step, layer call by layer call.  One
    step = one token through all 36 layers."""
    import numpy as np
    import torch
    import gqa_attention_block_amd as gqa
    import synth
    mlp = args.workload == "decoder"
    st = synth.decoder_stack() if mlp else synth.cfg4_stack()
    a = gqa.Arch(hidden=st.arch.hidden)
    up = lambda arr: torch.from_numpy(arr.view(np.int16) if arr.dtype == np.uint16 else arr).to("cuda:0")  # noqa: E731
    layers = [dict(w_norm=up(L.w_norm), w_qkv=up(L.w_qkv), w_g=up(L.w_g), w_o=up(L.w_o),
                   seq=gqa.KvSeq(k=up(L.cache.k), v=up(L.cache.v), position=L.cache.position,
                                 ring_capacity=L.cache.ring_capacity), full=L.is_full,
                   mlp=(up(L.w_post), up(L.w_gate), up(L.w_up), up(L.w_down)) if mlp else None)
              for L in st.layers]
    h0 = up(st.h)
    h = h0.clone()
    ws = torch.empty(gqa.workspace_size(a, 1, st.layers[0].cache.position + 1), dtype=torch.uint8,
                     device="cuda:0")

    ws_mlp = (torch.empty(gqa.mlp_workspace_size(a, int(st.layers[0].w_gate.shape[0]), 1), dtype=torch.uint8,
                          device="cuda:0") if mlp else None)

    # per layer: h += block(RMSNorm(h) * w) [, then h += mlp(h)], each call
    # marshalled once (the binding's prepared calls); the attention-only stack
    # as one call for all layers unless --layer-calls
    one_call = not mlp and not args.layer_calls
    calls = []
    if one_call:
        calls.append(gqa.PreparedStack(a, [gqa.StackLayer(w_norm=L["w_norm"], w_qkv=L["w_qkv"], w_g=L["w_g"],
                                                          w_o=L["w_o"], is_full=L["full"], seq=L["seq"])
                                           for L in layers], h, ws))
    else:
        for L in layers:
            calls.append(gqa.PreparedLayer(a, L["w_norm"], L["w_qkv"], L["w_g"], L["w_o"], L["full"], [L["seq"]], h,
                                           ws))
            if mlp:
                calls.append(gqa.PreparedMlp(a, *L["mlp"], h, ws_mlp))
    launch = ("one_launch_stack" if one_call else "layer_calls") + ("+hip_graph" if args.graph else "")

    def step():
        for c in calls:
            c.step()

    run = step
    if args.graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=side):
                step()
        torch.cuda.current_stream().wait_stream(side)
        run = g.replay
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run()
    submitted = time.perf_counter() - t0
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    assert torch.isfinite(h).all(), "non-finite residual stream"
    ms = 1e3 * elapsed / args.steps
    sb = stack_bytes(st)
    log(f"stack ({launch}): {ms * 1e3:.1f} us/token, host submit "
        f"{submitted / args.steps * 1e6:.1f} us/token, {sb / 1e9:.3f} GB/token -> "
        f"{sb / (ms * 1e-3) / 1e9:.1f} GB/s")
    cpu = None
    if args.cpu_seconds > 0:
        import oracle
        # bounded sample: the fp64 oracle over the first layers, scaled to 36
        done, t0 = 0, time.perf_counter()
        while done < len(st.layers) and time.perf_counter() - t0 < args.cpu_seconds:
            (oracle.decoder_stack_decode if mlp else oracle.stack_decode)(st.arch, st.h, st.layers[done:done + 1])
            done += 1
        el = time.perf_counter() - t0
        try:
            from threadpoolctl import threadpool_info
            cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        except Exception:                   # pragma: no cover
            cores = os.cpu_count() or 1
        cpu = {"value": 1.0 / (el / done * len(st.layers)), "unit": "tokens/s", "cores": int(cores),
               "kind": "oracle", "sample": f"{done} of {len(st.layers)} layers in {el:.1f} s, scaled to 36"}
    line = {
        "metric": METRIC, "value": round(1e3 / ms, 3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": DTYPE,
        "data": "synthetic",
        "config": {"workload": st.name, "hidden": a.hidden, "batch": 1, "layers": len(st.layers),
                   "positions": [st.layers[0].cache.position], "weights": "bf16", "kv_cache": "fp16",
                   "stack_bytes_per_token": sb, "launch": launch},
        "block_hbm_gbs": round(sb / (ms * 1e-3) / 1e9, 1),
        "block_frac_of_peak": round(sb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "host_submit_us_per_step": round(submitted / args.steps * 1e6, 3),
        "roofline": None,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def bench_head(args):
    """The ends of the decode step, batch 1: the embedding gather of the next
    token and the final RMSNorm + tied head over a 65536-token table at hidden
    2560 (the pages print no vocabulary size).  One step = gather + head."""
    import torch
    import gqa_attention_block_amd as gqa
    import synth
    hid, vocab = 2560, 65536
    hc = synth.head_case(hid, vocab, 1)
    a = gqa.Arch(hidden=hid)
    up = lambda arr: torch.from_numpy(arr.view("int16") if arr.dtype.name == "uint16" else arr).to("cuda:0")  # noqa: E731
    table, w_final, h = up(hc.embed), up(hc.w_final), up(hc.h)
    he = torch.empty_like(h)
    logits = torch.empty((1, vocab), dtype=torch.float32, device="cuda:0")
    ws = torch.empty(gqa.lm_head_workspace_size(a, 1), dtype=torch.uint8, device="cuda:0")
    ids = [int(hc.ids[0])]

    def step():
        gqa.embed_tokens(a, table, ids, he)
        gqa.lm_head(a, w_final, table, h, logits, ws)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = 1e3 * (time.perf_counter() - t0) / args.steps
    alg = 2 * vocab * hid + 2 * hid + 4 * hid + (4 * hid * 2 + 2 * hid) + 4 * hid + 4 * vocab
    log(f"head (gather + final norm + tied head, vocab {vocab}): {ms * 1e3:.2f} us/token, "
        f"{alg / 1e6:.1f} MB -> {alg / (ms * 1e-3) / 1e9:.1f} GB/s")
    line = {
        "metric": METRIC, "value": round(1e3 / ms, 3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": DTYPE,
        "data": "synthetic",
        "config": {"workload": f"head_h{hid}_vocab{vocab}", "hidden": hid, "vocab": vocab, "batch": 1,
                   "weights": "bf16", "algorithmic_bytes_per_step": alg},
        "block_hbm_gbs": round(alg / (ms * 1e-3) / 1e9, 1),
        "block_frac_of_peak": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "roofline": None, "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def bench_chunk(args):
    """Several tokens of one sequence per call (gqa_attention_block_chunk): a
    full layer, hidden 2560, 32 tokens at positions 4096 .. 4127 (a chunk of
    prefill at 4K context).  One step = one call = 32 tokens."""
    import numpy as np
    import torch
    import gqa_attention_block_amd as gqa
    import synth
    m, p0, hid = 32, 4096, 2560
    case = synth.block_case("chunk_full_h2560_p4096_m32", hid, True, [p0], capacities=[p0 + m], seed=0,
                            case_id=40)
    x = synth.random_hidden(hid, m, 0, 40, tensor_id=90)
    a = gqa.Arch(hidden=hid)
    up = lambda arr: torch.from_numpy(arr.view(np.int16) if arr.dtype == np.uint16 else arr).to("cuda:0")  # noqa: E731
    w = [up(case.w_qkv), up(case.w_g), up(case.w_o)]
    seq = gqa.KvSeq(k=up(case.seqs[0].k), v=up(case.seqs[0].v), position=p0, ring_capacity=0)
    xd = up(x)
    out = torch.empty((m, hid), dtype=torch.float32, device="cuda:0")
    ws = torch.empty(gqa.workspace_size(a, m, p0 + m), dtype=torch.uint8, device="cuda:0")

    def step():
        gqa.attention_block_chunk(a, w[0], w[1], w[2], True, seq, xd, out, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    assert torch.isfinite(out).all(), "non-finite chunk output"
    ms = 1e3 * elapsed / args.steps
    wbytes = case.w_qkv.nbytes + case.w_g.nbytes + case.w_o.nbytes
    kv_union = 4096 * (p0 + m)                              # K + V rows of every window, once
    kv_per_token = sum(4096 * (p0 + t + 1) for t in range(m))  # what per-token attention reads
    io = 8 * m * hid
    alg = wbytes + kv_union + io
    log(f"chunk ({m} tokens at {p0}): {ms * 1e3:.2f} us/call, {m / (ms * 1e-3):.1f} tokens/s; "
        f"algorithmic {alg / 1e6:.1f} MB -> {alg / (ms * 1e-3) / 1e9:.1f} GB/s; the per-token attention "
        f"reads {(wbytes + kv_per_token + io) / 1e6:.1f} MB")
    line = {
        "metric": METRIC, "value": round(m / (ms * 1e-3), 3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": DTYPE,
        "data": "synthetic",
        "config": {"workload": case.name, "hidden": hid, "tokens_per_call": m, "positions": [p0, p0 + m - 1],
                   "weights": "bf16", "kv_cache": "fp16", "algorithmic_bytes_per_call": alg},
        "block_hbm_gbs": round(alg / (ms * 1e-3) / 1e9, 1),
        "block_frac_of_peak": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "roofline": None,
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="full32k", choices=sorted(list(workloads()) + ["cfg4", "chunk", "decoder", "head"]),
                    help="cfg4 is the 36-layer stack at position 8191, chunk 32 tokens of one sequence "
                         "per call (neither has a dominant-kernel roofline)")
    ap.add_argument("--copies", type=int, default=0, help="weight/cache copies rotated (0: auto)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU oracle sample length (0 skips the baseline)")
    ap.add_argument("--graph", action="store_true",
                    help="replay one captured HIP graph per step instead of launching from the host")
    ap.add_argument("--layer-calls", action="store_true",
                    help="cfg4: one gqa_attention_layer_decode call per layer instead of one stack call per token")
    ap.add_argument("--sinks", action="store_true",
                    help="block workloads: pass per-head attention-sink logits (seeded, fp32 [Hq])")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration) and exit")
    args = ap.parse_args()
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy, 5)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU (asked for --gpus {args.gpus}, WORLD_SIZE "
              f"{world}); the block is a single-GPU decode step and sharding it across GPUs "
              "is not implemented", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gqa_attention_block_amd as gqa

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.workload in ("cfg4", "decoder"):
        bench_stack(args)
        return
    if args.workload == "head":
        bench_head(args)
        return
    if args.workload == "chunk":
        bench_chunk(args)
        return
    case = workloads()[args.workload]()
    a = gqa.Arch(hidden=case.arch.hidden)
    per_copy = (case.w_qkv.nbytes + case.w_g.nbytes + case.w_o.nbytes
                + sum(s.k.nbytes + s.v.nbytes for s in case.seqs))
    copies = args.copies or max(2, min(64, math.ceil((1 << 30) / per_copy)))
    log(f"workload {case.name}: batch {case.batch}, {per_copy / 1e6:.1f} MB per copy, "
        f"{copies} copies")

    def up(arr, dt=None):
        t = torch.from_numpy(arr.view(np.int16) if arr.dtype == np.uint16 else arr)
        return t.to("cuda:0")

    base = dict(w_qkv=up(case.w_qkv), w_g=up(case.w_g), w_o=up(case.w_o),
                k=[up(s.k) for s in case.seqs], v=[up(s.v) for s in case.seqs])
    sets = []
    for c in range(copies):
        cl = (lambda t: t) if c == 0 else (lambda t: t.clone())
        sets.append(dict(w_qkv=cl(base["w_qkv"]), w_g=cl(base["w_g"]), w_o=cl(base["w_o"]),
                         seqs=[gqa.KvSeq(k=cl(base["k"][i]), v=cl(base["v"][i]),
                                         position=s.position, ring_capacity=s.ring_capacity)
                               for i, s in enumerate(case.seqs)]))
    x = up(case.x)
    sinks_np = synth_sinks(case) if args.sinks else None
    sinks = up(sinks_np) if args.sinks else None
    out = torch.empty((case.batch, a.hidden), dtype=torch.float32, device="cuda:0")
    ws = torch.empty(gqa.workspace_size(a, case.batch, max(s.position + 1 for s in case.seqs)),
                     dtype=torch.uint8, device="cuda:0")
    torch.cuda.synchronize()

    # each copy's block call marshalled once (the binding's prepared call):
    # a step enqueues the same gqa_attention_block_decode
    prepared = [gqa.PreparedBlock(a, s["w_qkv"], s["w_g"], s["w_o"], case.is_full, s["seqs"], x, out, ws,
                                  sinks=sinks)
                for s in sets]

    def block_step(c):
        prepared[c].step()

    # the attention step (split-K attention over the window, merge + gate),
    # on a q produced once by the projection step
    q = torch.empty((case.batch, a.q_dim), dtype=torch.float32, device="cuda:0")
    gl = torch.empty((case.batch, a.num_heads), dtype=torch.float32, device="cuda:0")
    attn = torch.empty((case.batch, a.q_dim), dtype=torch.float32, device="cuda:0")
    gqa.qkv_rope_kv(a, sets[0]["w_qkv"], sets[0]["w_g"], case.is_full, sets[0]["seqs"], x, q, gl)

    def attn_step(c):
        gqa.attention_gated(a, case.is_full, sets[c]["seqs"], q, gl, attn, ws, sinks=sinks)

    for c in range(copies):          # eager warm-up of every copy (also caches the CU count)
        block_step(c)
        attn_step(c)
    torch.cuda.synchronize()

    if not args.graph:
        run_block = block_step
        run_attn = attn_step
    else:
        # one HIP graph per copy: a decode step is replayed the way a serving
        # loop would replay it, without per-kernel host launch cost
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        gb, ga = [], []
        with torch.cuda.stream(side):
            for c in range(copies):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=side):
                    block_step(c)
                gb.append(g)
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=side):
                    attn_step(c)
                ga.append(g)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        run_block = lambda c: gb[c].replay()   # noqa: E731
        run_attn = lambda c: ga[c].replay()    # noqa: E731

    for i in range(args.warmup):
        run_block(i % copies)
    torch.cuda.synchronize()
    # HIP events on the stream the block is launched on, around the timed
    # region: with one launch per step, their average is that kernel's
    # average launch duration (back to back, inter-launch gaps included)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for i in range(args.steps):
        run_block(i % copies)
    ev1.record()
    submitted = time.perf_counter() - t0
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    launch_s = ev0.elapsed_time(ev1) * 1e-3 / args.steps
    assert torch.isfinite(out).all(), "non-finite block output"
    ms_per_step = 1e3 * elapsed / args.steps
    tokens_per_s = case.batch * args.steps / elapsed
    bb = block_bytes(case)
    log(f"host submit time {submitted / args.steps * 1e6:.2f} us/step (the GPU is the bound "
        f"while this stays below the step time)")
    log(f"block ({'graph' if args.graph else 'eager'}): {ms_per_step * 1e3:.2f} us/step, "
        f"{tokens_per_s:.1f} tokens/s, {bb / 1e6:.2f} MB/step -> "
        f"{bb / (ms_per_step * 1e-3) / 1e9:.1f} GB/s")

    # one sequence whose window takes more than one chunk: the whole block is
    # one launch of block_fused_kernel (the library's rule, restated here for
    # the report); else the split-K pass is the dominant kernel
    plan = gqa.split_plan(a, case.is_full, [s.position for s in case.seqs], case.seqs[0].ring_capacity,
                          capacities=[s.k.shape[0] for s in case.seqs])
    one_launch = (case.batch == 1 and not plan.direct and plan.groups == 1 and plan.max_group_chunks <= 256
                  and a.hidden <= 4096 and a.q_dim <= 4096)
    # the split-K pass alone, launched back to back over the copies; one event
    # pair around the whole run gives its average duration
    part_o = torch.empty((1024, a.num_heads, a.head_dim), dtype=torch.float32, device="cuda:0")
    part_ml = torch.empty((part_o.shape[0], a.num_heads, 2), dtype=torch.float32, device="cuda:0")

    def part_step(c):
        return gqa.attention_partials(a, case.is_full, sets[c]["seqs"], q, part_o, part_ml)

    chunk_rows, begin = part_step(0)
    n_runs = max(args.steps, 20)

    def timed(fn):
        for i in range(args.warmup):
            fn(i % copies)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(n_runs):
            fn(i % copies)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / n_runs

    part_s = timed(part_step)
    pb = kv_bytes(case)
    achieved = pb / part_s / 1e9
    log(f"attn_partial_kernel: {part_s * 1e6:.2f} us avg over {n_runs} back-to-back launches, "
        f"{begin[-1]} chunks of {chunk_rows} rows, {pb / 1e6:.2f} MB of K/V -> {achieved:.1f} GB/s = "
        f"{achieved / HBM_PEAK_GBS:.3f} of peak")
    att_s = timed(attn_step)
    ab = attention_bytes(case)
    log(f"attention step (partials + combine): {att_s * 1e6:.2f} us avg, {ab / 1e6:.2f} MB -> "
        f"{ab / att_s / 1e9:.1f} GB/s")

    split_k = {"kernel": "attn_partial_kernel", "achieved": round(achieved, 1), "unit": "GB/s",
               "frac": round(achieved / HBM_PEAK_GBS, 4), "us_per_launch": round(part_s * 1e6, 3),
               "kv_bytes_per_launch": pb}
    if one_launch:
        kname, kbytes, ks = "block_fused_kernel", bb, launch_s
    else:
        kname, kbytes, ks = "attn_partial_kernel", pb, part_s
    kach = kbytes / ks / 1e9
    log(f"{kname}: {ks * 1e6:.2f} us per launch, {kbytes / 1e6:.2f} MB -> {kach:.1f} GB/s = "
        f"{kach / HBM_PEAK_GBS:.3f} of peak")
    roofline = {"kernel": kname, "bound": "hbm", "achieved": round(kach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(kach / HBM_PEAK_GBS, 4), "traffic": counted_traffic(args.workload, kname),
                "us_per_launch": round(ks * 1e6, 3), "algorithmic_bytes_per_launch": kbytes}
    # the block as a whole (what the metric names): its algorithmic bytes over
    # the wall time of a step
    block_gbs = bb / (ms_per_step * 1e-3) / 1e9
    block_roofline = {"bound": "hbm", "achieved": round(block_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                      "frac": round(block_gbs / HBM_PEAK_GBS, 4), "us_per_step": round(ms_per_step * 1e3, 3),
                      "algorithmic_bytes_per_step": bb}
    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(case, args.cpu_seconds, sinks_np)
        log(f"cpu oracle: {cpu['value']:.3f} tokens/s on {cpu['cores']} threads ({cpu['sample']})")

    line = {
        "metric": METRIC, "value": round(tokens_per_s, 2), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": DTYPE,
        "data": "synthetic",
        "config": {"workload": case.name, "hidden": a.hidden, "batch": case.batch,
                   "positions": [s.position for s in case.seqs][:4],
                   "kv_rows_attended": attended_rows(case), "weights": "bf16",
                   "kv_cache": "fp16", "block_bytes_per_step": bb, "copies_rotated": copies,
                   "launch": "hip_graph" if args.graph else "eager",
                   "attention_chunk_rows": chunk_rows, "sinks": bool(args.sinks)},
        "attention_step_us": round(att_s * 1e6, 3),
        "host_submit_us_per_step": round(submitted / args.steps * 1e6, 3),
        "block_hbm_gbs": round(bb / (ms_per_step * 1e-3) / 1e9, 1),
        "block_frac_of_peak": round(bb / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "roofline": roofline,
        "block_roofline": block_roofline,
        "split_k_pass": split_k,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
