"""SPLA decode benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload llama_gqa_128k]

A step is one pass of the whole decode hot path for one SPLA attention layer:
spla_decode_step, i.e. the append of the step's token for every sequence
(page write, S_all / z_all update, statistics of a completed block) fused
into the launch of the Taylor block scorer, then top-k, attend + residual
linear attention and combine (plus the chunk appends of workloads that have
them, through spla_append_kv).  Inputs (the prefilled state and every step's
q, k, v) are resident in HBM before the timed region starts.

The per-step footprint of the 128K workload (~26 MB) fits the 256 MB
Infinity Cache, so the state is replicated into L_rot independent layer
instances (device copies, L_rot = max(2, ceil(512 MB / bytes per step))) and
each timed step runs every instance in turn on one stream; t_step = timed
time / (K * L_rot).  Every instance sees identical inputs, so their outputs
must be bitwise equal (checked after the run).

The timed steps start where a block completion falls in their middle (a few
untimed lead-in steps after the warm-up move it there), so the statistics
work of a completed block is part of what is timed.

Prints one JSON line (rank 0) with the throughput, a roofline entry for the
kernel that takes the largest share of the step's time (its launch duration
from HIP events that hipExtLaunchKernel stamps with the kernel's own begin /
end on its launch stream; its HBM traffic from the committed rocprofv3
counter summary when that was taken on the current kernel sources), the
same figures for every kernel of the step and for the step as a whole, and a
CPU baseline (the fp64 oracle timed on a bounded sample of the same
workload, with all host threads and with one).
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published

CSRC = "block_sparse_linear_amd/csrc/"
# sources of each decode kernel (by launch-plan name); a counter summary of a
# kernel is used only while the hash of its sources matches the one it was
# taken on
_COMMON = ["decode_common.h", "spla_common.h", "append_items.h"]
KERNEL_SOURCES = {
    "score": ["score.hip", "score_parts.h"],
    "step_score": ["score.hip", "score_parts.h"],
    "select": ["select.hip", "select_core.h"],
    "attend": ["attend.hip", "attend_mfma.h"],
    "select_attend": ["select_attend.hip", "select_core.h", "attend_mfma.h", "combine_body.h", "xcd_sync.h"],
    "combine": ["combine.hip", "combine_body.h", "xcd_sync.h"],
    "step_fused": ["step_fused.hip", "score_parts.h", "select_core.h", "attend_mfma.h", "xcd_sync.h"],
}
PMC_SUMMARY = "profiles/decode_{workload}_pmc.txt"
# plain copy of known size run by every bench (outside the timed region) so the
# HBM byte counters can be scaled: reads and writes CALIB_BYTES each
CALIB_BYTES = 512 << 20


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def step_bytes(w, lens, s_kv: int, chunk_lens=None) -> dict:
    """Algorithmic bytes of one decode step (after the step's append) for
    sequence lengths ``lens``: candidate statistics, selected K/V rows,
    S_all / z_all read + write, q in, o out, gate, the new k / v read and
    written into the pages, and the statistics of a block the token completes.

    ``chunk_lens``: {sequence: length before its chunk} of the step's chunk
    appends (ragged serving workload), each adding its n tokens' K and V read
    and written into the pages, S_all / z_all read + write, and for every
    block the chunk completes its keys read (those not in the chunk) and its
    mean and variance written."""
    d, G, H, B, bk, k = w.head_dim, w.n_kv_heads, w.n_q_heads, w.batch, w.block_size, w.top_k
    stats = kv = state = 0
    for T in lens:
        nb = -(-T // bk)
        if nb > k:
            stats += G * (nb - 2) * 2 * d * 4
            ntok = (k - 1) * bk + (T - (nb - 1) * bk)
        else:
            ntok = T
        kv += G * ntok * 2 * d * s_kv
        state += G * 2 * (d * d * 4 + d * 4)
        if T % bk == 0:  # the step's token completes block T / bk - 1
            state += G * ((bk - 1) * d * s_kv + 2 * d * 4)
    io = B * H * d * (s_kv + 4) + H * 4 + B * G * d * 2 * s_kv * 2
    chunk = 0
    for _, t0 in sorted((chunk_lens or {}).items()):
        n = w.chunk_len
        chunk += 4 * n * G * d * s_kv + G * 2 * (d * d * 4 + d * 4)
        for j in range(t0 // bk, (t0 + n) // bk):  # blocks the chunk completes
            chunk += G * (max(0, t0 - j * bk) * d * s_kv + 2 * d * 4)
    return {"stats": stats, "kv": kv, "state": state, "io": io, "chunk": chunk,
            "total": stats + kv + state + io + chunk}


def step_score_bytes(w, lens, s_kv: int) -> int:
    """Algorithmic bytes of one launch of the fused first kernel of a decode
    step (lens: after the step's append): mean and variance of every candidate
    block and the queries (scorer), S_all / z_all read + write, the new k / v
    read and written into the pages (append)."""
    d, G, bk, k = w.head_dim, w.n_kv_heads, w.block_size, w.top_k
    tot = 0
    for T in lens:
        nb = -(-T // bk)
        if nb > k:
            tot += G * (nb - 2) * 2 * d * 4
    tot += w.batch * w.n_q_heads * d * s_kv
    tot += w.batch * G * 2 * (d * d * 4 + d * 4)
    tot += w.batch * G * d * 2 * s_kv * 2
    for T in lens:
        if T % bk == 0:  # the token completes a block: its other keys read, mean and variance written
            tot += G * ((bk - 1) * d * s_kv + 2 * d * 4)
    return tot


def kernel_bytes(name: str, w, lens, s_kv: int, merged: bool = False) -> int:
    """Algorithmic bytes of one launch of decode kernel ``name`` (a launch-plan
    name) for sequence lengths ``lens`` (after the step's append): what the
    method must move through that kernel, not its scratch traffic beyond the
    partial records it hands to the next kernel.  merged: the plan has no
    combine kernel, so the fused select + attend also merges the records (it
    reads the o_bar / phi(q).z partials and writes the outputs)."""
    d, G, H, bk, k = w.head_dim, w.n_kv_heads, w.n_q_heads, w.block_size, w.top_k
    r = H // G
    chunks = d * d // 1024
    rec = (2 * d + 4) * 4  # one partial record: acc[d], o_tilde[d] and its header m, l, sum w, pad
    lg = kv = recs = 0
    for T in lens:
        nb = -(-T // bk)
        used = min(nb, k)
        if nb > k:
            lg += G * (nb - 2) * 4
            ntok = (k - 1) * bk + (T - (nb - 1) * bk)
        else:
            ntok = T
        kv += G * ntok * 2 * d * s_kv
        recs += G * r * used * rec
    B = w.batch
    if name == "step_score":
        return step_score_bytes(w, lens, s_kv)
    if name == "select":
        return lg + B * G * k * 4 * 2
    if name == "attend":
        return kv + recs + B * H * d * s_kv
    if name == "select_attend":
        merge = B * G * chunks * r * (d + 1) * 4 + B * H * d * 4 + H * 4 if merged else 0
        return lg + kv + recs + B * H * d * s_kv + merge
    if name == "combine":
        return recs + B * G * chunks * r * (d + 1) * 4 + B * H * d * 4 + H * 4
    if name == "step_fused":
        # the first kernel's bytes, then the selected K/V and the records (the
        # scores it hands over inside the kernel are not counted)
        return step_score_bytes(w, lens, s_kv) + kv + recs
    raise ValueError(name)


def kernel_source_hash(name: str) -> str:
    """sha256 prefix of the sources of decode kernel ``name``."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[name] + _COMMON:
        with open(os.path.join(ROOT, CSRC + p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_pmc_summary(path: str) -> dict:
    """The key = value fields of a counter summary: {"": global fields,
    kernel symbol: that kernel's fields} ([section] lines open a kernel)."""
    out = {"": {}}
    cur = out[""]
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("[") and line.endswith("]"):
                cur = out.setdefault(line[1:-1].strip(), {})
            elif "=" in line:
                k, v = line.split("=", 1)
                cur[k.strip()] = v.strip()
    return out


def read_traffic(workload: str, name: str):
    """HBM bytes per launch of decode kernel ``name`` from the committed
    counter summary (FETCH_SIZE and WRITE_SIZE per dispatch, each scaled by
    what the counter reads for the calibration copy), or None when there is
    no summary of it for this workload or its sources changed since."""
    p = os.path.join(ROOT, PMC_SUMMARY.format(workload=workload))
    if not os.path.exists(p):
        return None, "no counter summary"
    s = read_pmc_summary(p)
    g, kv = s[""], s.get("k_" + name)
    if kv is None:
        return None, f"no counters of k_{name}"
    if kv.get("source_sha256") != kernel_source_hash(name):
        return None, "kernel changed since the counters were taken"
    fetch_scale = float(g["copy_bytes"]) / (float(g["copy_fetch_kib"]) * 1024.0)
    write_scale = float(g["copy_bytes"]) / (float(g["copy_write_kib"]) * 1024.0)
    fetch = float(kv["fetch_kib_per_dispatch"]) * 1024.0 * fetch_scale
    write = float(kv["write_kib_per_dispatch"]) * 1024.0 * write_scale
    return {"bytes": fetch + write, "fetch": fetch, "write": write,
            "fetch_scale": fetch_scale, "write_scale": write_scale}, None


RLA_FORMS = {0: "plain", 1: "normalized", 2: "rmsnorm"}
RLA_EPS = 1e-6


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(w, n_steps: int, budget_s: float, rla_form: int = 0) -> dict:
    """Time the fp64 oracle's append + decode per step on the host cores: the
    first steps after an untimed prefill with every BLAS thread the process
    may use, up to budget_s / 2 of oracle time, then the following steps with
    one thread for as long again."""
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import SplaOracle

    threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    o = SplaOracle(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.block_size, w.top_k,
                   w.max_tokens(n_steps))
    t0 = time.time()
    for b in range(w.batch):
        for _, k, v in w.prefill_chunks(b):
            o.append([b], [k.shape[0]], k, v)
    log(f"oracle prefill {time.time() - t0:.1f}s")
    gate = w.gate()
    gamma = w.rla_gamma() if rla_form == 2 else None
    mix = w.mixture_state()
    s = 0

    def sample(limit_s):
        nonlocal s
        done, spent = 0, 0.0
        while s < n_steps:
            st = w.step(s, mix)
            t = time.perf_counter()
            cs = [int(x) for x in st["chunk_seqs"]]
            if cs:
                o.append(cs, [w.chunk_len] * len(cs), st["chunk_k"], st["chunk_v"])
            o.append(list(range(w.batch)), [1] * w.batch, st["k"], st["v"])
            o.decode(st["q"], gate, rla_mode=rla_form, gamma=gamma, eps=RLA_EPS)
            spent += time.perf_counter() - t
            done += 1
            s += 1
            if spent >= limit_s:
                break
        return done, spent

    done, spent = sample(budget_s / 2)
    with threadpool_limits(1):
        done1, spent1 = sample(budget_s / 2)
    t_step = spent / done
    res = {"value": w.batch / t_step, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
           "cpu_model": cpu_model(),
           "sample": f"{w.name}: fp64 NumPy oracle append+decode of decode steps 0..{done - 1} after an untimed "
                     f"prefill, {threads} BLAS threads ({spent:.1f}s timed, {t_step * 1e3:.1f} ms/step)"}
    if done1:
        t1 = spent1 / done1
        res["value_1_thread"] = w.batch / t1
        res["sample_1_thread"] = (f"steps {done}..{done + done1 - 1}, 1 BLAS thread ({spent1:.1f}s timed, "
                                  f"{t1 * 1e3:.1f} ms/step)")
    return res


def run_prefill(args) -> int:
    """Chunked prefill: time spla_prefill of args.prefill tokens appended to
    sequence 0 of the workload (after its untimed prefill), each timed call on
    a fresh copy of the prefilled state (the copy is outside the timed region).
    Prints one JSON line: tokens/s of the prefilled tokens."""
    import numpy as np
    import torch

    from block_sparse_linear_amd import SplaLayer
    from workloads import WORKLOADS

    w = WORKLOADS[args.workload]
    n = args.prefill
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tdt = torch.bfloat16 if w.kv_dtype == "bf16" else torch.float32
    mb = -(-(max(w.t0) + n) // w.block_size) + 1
    L = SplaLayer(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.block_size, w.top_k, mb,
                  kv_dtype=w.kv_dtype, device="cuda:0")
    L.set_fused_select(args.fused_select)
    gamma = torch.from_numpy(w.rla_gamma()).to(dev) if args.rla_form == 2 else None
    L.set_rla_output(args.rla_form, gamma, RLA_EPS)
    t0 = time.time()
    for b in range(w.batch):
        for _, k, v in w.prefill_chunks(b):
            L.append([b], [k.shape[0]], torch.from_numpy(k).to(dev).to(tdt), torch.from_numpy(v).to(dev).to(tdt))
    torch.cuda.synchronize()
    log(f"prefill of the context {time.time() - t0:.1f}s lens={L.lens[:4]}")
    seq = 0
    rng = np.random.default_rng([w.seed, 99])
    kk = torch.from_numpy(w.round(rng.standard_normal((n, w.n_kv_heads, w.head_dim)).astype(np.float32))).to(dev).to(tdt)
    vv = torch.from_numpy(w.round(rng.standard_normal((n, w.n_kv_heads, w.head_dim)).astype(np.float32))).to(dev).to(tdt)
    qq = torch.from_numpy(w.prefill_queries(seq, L.lens[seq], n)).to(dev).to(tdt)
    gate = torch.from_numpy(w.gate()).to(dev)
    out = torch.empty((n, w.n_q_heads, w.head_dim), dtype=torch.float32, device=dev)
    ws = torch.empty(L.handle.prefill_workspace_bytes(args.prefill_chunk) // 4 + 64, dtype=torch.int32, device=dev)
    snap = L.snapshot()
    times = []
    for it in range(args.warmup + args.steps):
        L.restore(snap)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        L.prefill(seq, kk, vv, qq, gate, out=out, workspace=ws)
        e1.record()
        torch.cuda.synchronize()
        if it >= args.warmup:
            times.append(e0.elapsed_time(e1) * 1e-3)
    t_call = float(np.median(times))
    log(f"prefill of {n} tokens: median {t_call * 1e3:.3f} ms over {len(times)} calls "
        f"(min {min(times) * 1e3:.3f}, max {max(times) * 1e3:.3f})")
    result = {
        "metric": f"SPLA chunked-prefill tokens/s ({n} tokens onto {max(w.t0)} context, GQA "
                  f"{w.n_q_heads}/{w.n_kv_heads}x{w.head_dim})",
        "value": n / t_call, "unit": "tokens/s", "n_gpus": 1, "steps": len(times), "warmup": args.warmup,
        "ms_per_call": t_call * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.kv_dtype, "data": "synthetic (seeded; see workloads/)",
        "config": {"workload": w.name, "mode": "prefill", "prefill_tokens": n, "group": args.prefill_chunk,
                   "context": max(w.t0), "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
                   "head_dim": w.head_dim, "block_size": w.block_size, "top_k": w.top_k,
                   "rla_output": RLA_FORMS[args.rla_form]},
    }
    print(json.dumps(result), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="llama_gqa_128k")
    ap.add_argument("--lrot", type=int, default=0, help="layer instances (0 = auto)")
    ap.add_argument("--prof-steps", type=int, default=16, help="steps of the per-kernel event pass")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle work to time")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--fused-select", type=int, default=-1, choices=(-1, 0, 1),
                    help="selector placement: -1 automatic, 0 stand-alone kernel, 1 fused into attend")
    ap.add_argument("--fused-merge", type=int, default=-1, choices=(-1, 0, 1),
                    help="1: the fused select + attend merges the records; -1 automatic, 0: combine kernel")
    ap.add_argument("--step-kernel", type=int, default=-1, choices=(-1, 0, 1),
                    help="1: decode step in one kernel plus the combine; -1 automatic, 0: separate kernels")
    ap.add_argument("--rla-form", type=int, default=0, choices=sorted(RLA_FORMS),
                    help="output form of the RLA branch: 0 plain, 1 normalised (o_rla / D), 2 RMS-normalised")
    ap.add_argument("--prefill", type=int, default=0,
                    help="time chunked prefill of this many tokens instead of decode steps")
    ap.add_argument("--prefill-chunk", type=int, default=256, help="tokens per group of prefill launches")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "one GPU per process only; --gpus must be 1"}))
        log("the SPLA decode library runs on one GPU per process and has no collectives")
        return 2
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        log("WORLD_SIZE > 1 is not supported")
        return 2
    if args.prefill > 0:
        return run_prefill(args)

    import numpy as np
    import torch

    from block_sparse_linear_amd import SplaLayer
    from workloads import WORKLOADS

    w = WORKLOADS[args.workload]
    K, W, P = args.steps, args.warmup, args.prof_steps
    bk = w.block_size

    # sequence lengths after each step's appends (chunk, then the token), and
    # each step's chunk appends as {sequence: length before the chunk}
    def simulate(n):
        lens, after, chunks = list(w.t0), [], []
        for s in range(n):
            cs = {int(b): lens[int(b)] for b in w.chunk_plan(s)}
            for b in cs:
                lens[b] += w.chunk_len
            lens = [t + 1 for t in lens]
            after.append(list(lens))
            chunks.append(cs)
        return after, chunks

    # untimed lead-in steps after the warm-up, so that a token of the timed
    # steps completes a block (at the middle step, or as near as 2 Bk steps allow)
    lead = 0
    after, _ = simulate(W + 2 * bk + K)
    mid = K // 2
    for x in range(2 * bk):
        if any(t % bk == 0 for t in after[W + x + mid]):
            lead = x
            break
    W0 = W + lead
    total_steps = W0 + K + P
    if total_steps > w.steps:
        # the workload's draws over more steps than it states (the mixture's
        # centre ids run on: the first w.steps steps are unchanged)
        w = dataclasses.replace(w, steps=total_steps)
    after, chunk_lens = simulate(total_steps)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    s_kv = 2 if w.kv_dtype == "bf16" else 4
    tdt = torch.bfloat16 if w.kv_dtype == "bf16" else torch.float32
    mb = w.max_blocks_per_seq(total_steps)

    gamma = torch.from_numpy(w.rla_gamma()).to(dev) if args.rla_form == 2 else None

    def new_layer():
        layer = SplaLayer(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.block_size, w.top_k, mb,
                          kv_dtype=w.kv_dtype, device="cuda:0")
        layer.set_fused_select(args.fused_select)
        layer.set_step_kernel(args.step_kernel)
        layer.set_fused_merge(args.fused_merge)
        layer.set_rla_output(args.rla_form, gamma, RLA_EPS)
        return layer

    t0 = time.time()
    base = new_layer()
    for b in range(w.batch):
        for _, k, v in w.prefill_chunks(b):
            base.append([b], [k.shape[0]], torch.from_numpy(k).to(dev).to(tdt),
                        torch.from_numpy(v).to(dev).to(tdt))
    torch.cuda.synchronize()
    log(f"prefill {time.time() - t0:.1f}s lens={base.lens[:4]}")

    # per-step inputs, resident on the device
    mix = w.mixture_state()
    steps_in = []
    for s in range(total_steps):
        st = w.step(s, mix)
        steps_in.append({
            "q": torch.from_numpy(st["q"]).to(dev).to(tdt),
            "k": torch.from_numpy(st["k"]).to(dev).to(tdt),
            "v": torch.from_numpy(st["v"]).to(dev).to(tdt),
            "cs": [int(x) for x in st["chunk_seqs"]],
            "ck": torch.from_numpy(st["chunk_k"]).to(dev).to(tdt),
            "cv": torch.from_numpy(st["chunk_v"]).to(dev).to(tdt),
        })
    gate = torch.from_numpy(w.gate()).to(dev)

    timed = range(W0, W0 + K)
    sbs = [step_bytes(w, after[s], s_kv, chunk_lens[s]) for s in timed]
    bytes_avg = float(np.mean([x["total"] for x in sbs]))
    L = args.lrot or max(2, math.ceil(512e6 / bytes_avg))
    layers = [base]
    for _ in range(L - 1):
        x = new_layer()
        for dst, src in zip(x.state_tensors(), base.state_tensors()):
            dst.copy_(src)
        x._bind(base.lens)
        layers.append(x)
    torch.cuda.synchronize()
    parts = {k: float(np.mean([x[k] for x in sbs])) for k in sbs[0]}
    completions = [s - W0 for s in timed if any(t % bk == 0 for t in after[s])]
    log(f"L_rot={L} lead-in {lead} steps; timed steps {W0}..{W0 + K - 1}, block completions at timed steps "
        f"{completions[:8]}; mean step bytes {parts}")
    outs = [torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32, device=dev) for _ in layers]

    def run_step(s, layer, out, kernel_events=None):
        # chunk appends (ragged serving preset), then the fused decode step:
        # append of the token of every sequence + decode
        x = steps_in[s]
        if x["cs"]:
            layer.append(x["cs"], [w.chunk_len] * len(x["cs"]), x["ck"], x["cv"])
        layer.decode_step(x["k"], x["v"], x["q"], gate, out=out, kernel_events=kernel_events)

    for s in range(W0):
        for layer, out in zip(layers, outs):
            run_step(s, layer, out)
    torch.cuda.synchronize()

    # one HIP graph per timed step holding every instance's append + decode
    # (captured ahead of the timed region; replay order = step order)
    graphs = []
    for s in timed:
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for layer, out in zip(layers, outs):
                run_step(s, layer, out)
        graphs.append(gr)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for gr in graphs:
        gr.replay()
    end.record()
    torch.cuda.synchronize()
    elapsed_ms = start.elapsed_time(end)
    t_step = elapsed_ms / 1e3 / (K * L)
    if layers[0].lens != after[W0 + K - 1]:
        raise RuntimeError(f"lengths after the timed steps {layers[0].lens[:4]} != {after[W0 + K - 1][:4]}")
    for o in outs[1:]:
        if not torch.equal(o, outs[0]):
            log("WARNING: layer instances disagree bitwise")
    log(f"timed {K} steps x {L} instances: {elapsed_ms:.2f} ms, t_step {t_step * 1e6:.2f} us")
    del graphs

    # per-kernel durations: every kernel of the step (append+score, select,
    # attend, combine) is launched through hipExtLaunchKernel with a pair of
    # HIP events, which take that kernel's begin and end timestamps on its
    # launch stream.  The steps are enqueued while a spin kernel holds the
    # GPU, so that the GPU then runs them back to back as in the graphs.
    names = layers[0].launch_plan(step=True)  # e.g. step_score, select_attend, combine
    import ctypes
    prof = range(W0 + K, W0 + K + P)
    ev_sets = []
    for s in prof:
        ev_sets.append([[torch.cuda.Event(enable_timing=True) for _ in range(2 * len(names))] for _ in layers])
    for sets in ev_sets:
        for evs in sets:
            for e in evs:
                e.record()  # materialise the handles
    torch.cuda.synchronize()
    torch.cuda._sleep(int(2.4e9 * 0.3))
    for s, sets in zip(prof, ev_sets):
        for layer, out, evs in zip(layers, outs, sets):
            if layer.launch_plan(step=True) != names:
                raise RuntimeError("the launch plan changed during the per-kernel pass")
            handles = (ctypes.c_void_p * len(evs))(*[e.cuda_event for e in evs])
            run_step(s, layer, out, kernel_events=handles)
    torch.cuda.synchronize()
    durs = {n: [] for n in names}
    launch_bytes = {n: [] for n in names}
    for s, sets in zip(prof, ev_sets):
        for evs in sets:
            for i, n in enumerate(names):
                durs[n].append(evs[2 * i].elapsed_time(evs[2 * i + 1]) * 1e-3)
        for n in names:
            launch_bytes[n].append(kernel_bytes(n, w, after[s], s_kv, merged="combine" not in names))
    avg = {n: float(np.mean(v)) for n, v in durs.items()}
    nbytes = {n: float(np.mean(v)) for n, v in launch_bytes.items()}

    # calibration copy for the HBM byte counters (see CALIB_BYTES)
    calib = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device=dev)
    calib_out = torch.empty_like(calib)
    torch.neg(calib, out=calib_out)
    torch.cuda.synchronize()
    # its time gives the copy bandwidth this machine reaches (read + write)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(4):
        torch.neg(calib, out=calib_out)
    c1.record()
    torch.cuda.synchronize()
    probe_gbs = 4 * 2 * CALIB_BYTES / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del calib, calib_out
    log("kernel us (HIP events): " + ", ".join(f"{n}={avg[n] * 1e6:.2f}" for n in names))

    def roof(n):
        achieved = nbytes[n] / avg[n] / 1e9
        traffic, why = read_traffic(w.name, n)
        if traffic is None:
            log(f"k_{n} traffic: null ({why})")
        return {"kernel": "k_" + n, "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": traffic["bytes"] if traffic else None,
                "bytes_per_launch": nbytes[n], "us": avg[n] * 1e6, "share_of_step": avg[n] / t_step}

    # the kernel that takes the largest share of the step's time
    dominant = max(names, key=lambda n: avg[n])
    top = roof(dominant)
    top["copy_probe_GBps"] = probe_gbs
    result = {
        "metric": "SPLA decode tokens/s at 128K ctx GQA 32/8x128; achieved HBM GB/s vs peak",
        "value": w.batch / t_step,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": t_step * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.kv_dtype,
        "data": "synthetic (seeded; see workloads/)",
        "config": {"workload": w.name, "batch": w.batch, "context": max(w.t0), "n_q_heads": w.n_q_heads,
                   "n_kv_heads": w.n_kv_heads, "head_dim": w.head_dim, "block_size": w.block_size,
                   "top_k": w.top_k, "l_rot": L, "lead_in_steps": lead, "rla_output": RLA_FORMS[args.rla_form]},
        "step_bytes": bytes_avg,
        "step_bytes_parts": parts,
        "step_GBps": bytes_avg / t_step / 1e9,
        "step_frac_of_peak": bytes_avg / t_step / 1e9 / HBM_PEAK_GBS,
        "kernel_us": {n: avg[n] * 1e6 for n in names},
        "kernels": names,
        # the kernel with the largest share of the step's time
        "roofline": top,
        # the whole step: algorithmic bytes per step over the graph-timed step
        "step_roofline": {"bound": "hbm", "achieved": bytes_avg / t_step / 1e9, "peak": HBM_PEAK_GBS,
                          "unit": "GB/s", "frac": bytes_avg / t_step / 1e9 / HBM_PEAK_GBS,
                          "bytes_per_step": bytes_avg, "us": t_step * 1e6},
        # every kernel of the step against the same HBM peak
        "kernel_rooflines": [roof(n) for n in names],
    }
    if not args.no_cpu_baseline:
        # room for both samples (the steps the GPU ran and 200 more)
        result["cpu_baseline"] = cpu_baseline(w, total_steps + 200, args.cpu_budget, args.rla_form)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
