"""Benchmark of the MSA hot path on one MI355X; prints ONE JSON line.

Headline (``value``): causal prefill tokens/s at N = 131072 (32 query heads / 4 KV
groups, d_h 128, index d_idx 64, blocks of 64, top_k 32, bf16): one step is the index
branch (block scores, top-k) plus the sparse prefill attention over all 131072 rows.
The same line carries, each with the roofline of its dominant kernel and the fp64
oracle timed on a bounded sample on the host cores:
  decode         the 1M-token decode (batch 4, one new token each, same heads), as the
                 two calls msa_index_topk + msa_sparse_attn_decode, and also as one
                 msa_decode_step call (decode_step_call);
  index_kl       the index branch's alignment loss on the prefill's selection;
  attn_backward  the main branch's backward (dq, dk, dv) for that selection;
  index_project  the index branch's two projections from hidden states of width h_q * d_h;
  chunked_prefill  the last 8192 rows of a 1M-token context against all 1M keys (the same
                 step as the headline; here the index kernel holds 94% of the FLOPs).
index_kl, attn_backward and index_project are timed apart from the step.

Inputs are seeded synthetic tensors already resident in HBM when timing starts. Kernel
durations come from HIP events recorded on the stream the library launches on.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--decode-steps KD] [--no-cpu]
                    [--sections prefill,chunk,decode]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MSA attn: prefill tok/s @128K, decode tok/s @1M; % of MFMA/HBM roofline"
PEAK_BF16_FLOPS = 2.5e15   # MI355X dense bf16 MFMA
PEAK_HBM_BYTES = 8.0e12    # MI355X HBM3E


# ------------------------------------------------------------------ algorithmic work

def prefill_work(w):
    """Algorithmic FLOPs of one step: index scores R*(p+1)*2*d_idx per row plus main
    branch H_q*T_p*4*d_h, T_p = visible tokens of the selected blocks."""
    p = w.q_start + np.arange(w.n_q, dtype=np.int64)
    b = p // w.block_size
    t_p = (np.minimum(w.top_k, b + 1) - 1) * w.block_size + (p - b * w.block_size + 1)
    index = float(w.batch * w.h_kv * np.sum(p + 1) * 2 * w.d_idx)
    main = float(w.batch * w.h_q * np.sum(t_p) * 4 * w.d_h)
    return index, main


def kl_work(w):
    """Algorithmic FLOPs of msa_index_kl: per (row, group) and selected visible token, the
    G heads' q.k (2*d_h each) and the index score q_idx.k_idx (2*d_idx)."""
    p = w.q_start + np.arange(w.n_q, dtype=np.int64)
    b = p // w.block_size
    t_p = (np.minimum(w.top_k, b + 1) - 1) * w.block_size + (p - b * w.block_size + 1)
    G = w.h_q // w.h_kv
    return float(w.batch * w.h_kv * np.sum(t_p) * (2 * w.d_h * G + 2 * w.d_idx))


def bwd_work(w):
    """Algorithmic FLOPs of msa_sparse_attn_backward: per (row, head) and selected visible
    token, q.k (recomputed), dout.v, and the three products that give dv, dk and dq
    (2*d_h each)."""
    p = w.q_start + np.arange(w.n_q, dtype=np.int64)
    b = p // w.block_size
    t_p = (np.minimum(w.top_k, b + 1) - 1) * w.block_size + (p - b * w.block_size + 1)
    return float(w.batch * w.h_q * np.sum(t_p) * 10 * w.d_h)


def project_work(w, d_model):
    """Algorithmic work of msa_index_project: FLOPs 2*d_model per output, (h_kv + 1)*d_idx
    outputs per row; bytes: x, both weights and both outputs once each."""
    es = 2 if w.dtype == "bf16" else 4
    cols = (w.h_kv + 1) * w.d_idx
    rows = w.batch * w.n_q
    flops = float(2 * rows * d_model * cols)
    nbytes = float(es * (rows * d_model + cols * d_model + rows * cols))
    return flops, nbytes


def decode_work(w):
    """Algorithmic HBM bytes of one decode step: the whole k_idx cache, the selected K/V
    blocks, q, q_idx, o and sel (block-score scratch and split partials excluded)."""
    L, e = w.n_k, 2
    nb = -(-L // w.block_size)
    sel_blocks = min(w.top_k, nb)
    kv_tokens = (sel_blocks - 1) * w.block_size + (L - (nb - 1) * w.block_size)
    k_idx = L * w.d_idx * e
    kv = w.h_kv * kv_tokens * w.d_h * e * 2
    small = (w.h_q * w.d_h * e * 2) + (w.h_kv * w.d_idx * e) + (w.h_kv * w.top_k * 4)
    per_seq = dict(k_idx=k_idx, kv=kv, small=small)
    index_kernel = w.batch * (k_idx + w.h_kv * w.d_idx * e)
    return w.batch * (k_idx + kv + small), index_kernel, per_seq


# ------------------------------------------------------------------ GPU timing

def time_step(w, inputs, steps, warmup, decode, extras=True):
    import torch
    from block_sparse_gqa_msa_amd import binding as msa

    s = msa.shape_of(w)
    R, n = w.h_kv, w.n_q
    nb = -(-w.n_k // w.block_size)
    scores = torch.empty((w.batch, R, n, nb), dtype=torch.float32, device="cuda")
    sel = torch.empty((w.batch, R, n, w.top_k), dtype=torch.int32, device="cuda")
    o = torch.empty((w.batch, w.h_q, n, w.d_h), dtype=inputs["q"].dtype, device="cuda")
    lse = torch.empty((w.batch, w.h_q, n), dtype=torch.float32, device="cuda")
    ws_topk = torch.empty(max(1, msa.msa_topk_workspace_size(s)), dtype=torch.uint8, device="cuda")
    ws_attn = torch.empty(max(1, msa.msa_sparse_attn_workspace_size(s)), dtype=torch.uint8,
                          device="cuda")
    attn = msa.msa_sparse_attn_decode if decode else msa.msa_sparse_attn_prefill
    stream = torch.cuda.current_stream()

    ws_index = torch.empty(max(1, msa.msa_index_topk_workspace_size(s)), dtype=torch.uint8,
                           device="cuda")

    if decode:
        # msa_index_topk runs the first selection stage inside the index kernel
        # (index_select_decode) and merges the per-range winners in topk_pass2
        stages = [
            ("index_topk", lambda: msa.msa_index_topk(s, inputs["q_idx"], inputs["k_idx"], sel,
                                                       None, ws_index)),
            ("attention", lambda: msa.msa_sparse_attn_decode(s, inputs["q"], inputs["k"],
                                                             inputs["v"], sel, o, lse, ws_attn)),
        ]
    else:
        # prefill: every stage is its own call so each kernel is timed alone
        stages = [
            ("index_scores", lambda: msa.msa_index_block_scores(s, inputs["q_idx"],
                                                                inputs["k_idx"], scores)),
            ("topk", lambda: msa.msa_topk_from_block_scores(s, scores, sel, ws_topk)),
            ("attn_plan", lambda: msa.msa_sparse_attn_prefill_plan(s, sel, ws_attn)),
            ("attn_partials", lambda: msa.msa_sparse_attn_prefill_partials(
                s, inputs["q"], inputs["k"], inputs["v"], ws_attn)),
            ("attn_merge", lambda: msa.msa_sparse_attn_prefill_merge(s, sel, o, lse, ws_attn)),
        ]

    def step(ev=None):
        for i, (_, call) in enumerate(stages):
            if ev:
                ev[i].record(stream)
            call()
        if ev:
            ev[-1].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # The timed region: exactly `steps` steps with nothing else enqueued between them.
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    # Per-stage times from a second pass with an event before each stage (the events and
    # their host-side cost stay out of the timed region above).
    n_ev = len(stages) + 1
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(steps)]
    for i in range(steps):
        step(events[i])
    torch.cuda.synchronize()
    times = {name: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in events])) * 1e-3
             for i, (name, _) in enumerate(stages)}
    if not decode and extras:
        # the alignment loss of the same step (sel and lse from the last step above)
        kl = torch.empty((w.batch, R, n), dtype=torch.float32, device="cuda")
        kl_call = lambda: msa.msa_index_kl(s, inputs["q"], inputs["k"], inputs["q_idx"],
                                           inputs["k_idx"], sel, lse, kl, None, ws_attn)
        for _ in range(max(1, warmup)):
            kl_call()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        ev[0].record(stream)
        for _ in range(steps):
            kl_call()
        ev[1].record(stream)
        torch.cuda.synchronize()
        times["index_kl"] = ev[0].elapsed_time(ev[1]) * 1e-3 / steps
        del kl
        # the main branch's backward for the same selection, o and lse
        from block_sparse_gqa_msa_amd.inputs import generate_dout
        dout = generate_dout(w, device="cuda")
        dq = torch.empty_like(inputs["q"])
        dk = torch.empty_like(inputs["k"])
        dv = torch.empty_like(inputs["v"])
        ws_bwd = torch.empty(msa.msa_sparse_attn_backward_workspace_size(s), dtype=torch.uint8,
                             device="cuda")
        bwd_call = lambda: msa.msa_sparse_attn_backward(s, inputs["q"], inputs["k"], inputs["v"],
                                                        sel, o, lse, dout, dq, dk, dv, ws_bwd)
        for _ in range(max(1, warmup)):
            bwd_call()
        torch.cuda.synchronize()
        ev[0].record(stream)
        for _ in range(steps):
            bwd_call()
        ev[1].record(stream)
        torch.cuda.synchronize()
        # the same backward as its three staged calls, with an event around each, so the
        # per-block gradient kernel is timed alone
        bst = [("bwd_plan", lambda: msa.msa_sparse_attn_backward_plan(s, sel, o, dout, ws_bwd)),
               ("bwd_partials", lambda: msa.msa_sparse_attn_backward_partials(
                   s, inputs["q"], inputs["k"], inputs["v"], lse, dout, ws_bwd)),
               ("bwd_merge", lambda: msa.msa_sparse_attn_backward_merge(s, sel, dq, dk, dv,
                                                                        ws_bwd))]
        sev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(bst) + 1)]
               for _ in range(steps)]
        for i in range(steps):
            for j, (_, call) in enumerate(bst):
                sev[i][j].record(stream)
                call()
            sev[i][-1].record(stream)
        torch.cuda.synchronize()
        for j, (name, _) in enumerate(bst):
            times[name] = float(np.mean([e[j].elapsed_time(e[j + 1]) for e in sev])) * 1e-3
        times["attn_backward"] = ev[0].elapsed_time(ev[1]) * 1e-3 / steps
        del dout, dq, dk, dv, ws_bwd
        # the index branch's projections of the step's rows (hidden width h_q * d_h)
        from block_sparse_gqa_msa_amd.inputs import generate_hidden
        hid = generate_hidden(w, w.h_q * w.d_h, device="cuda")
        q_idx_p = torch.empty_like(inputs["q_idx"])
        k_idx_p = torch.empty_like(inputs["k_idx"])
        proj_call = lambda: msa.msa_index_project(s, hid["x"], hid["w_q"], hid["w_k"], q_idx_p,
                                                  k_idx_p)
        for _ in range(max(1, warmup)):
            proj_call()
        torch.cuda.synchronize()
        ev[0].record(stream)
        for _ in range(steps):
            proj_call()
        ev[1].record(stream)
        torch.cuda.synchronize()
        times["index_project"] = ev[0].elapsed_time(ev[1]) * 1e-3 / steps
        del hid, q_idx_p, k_idx_p
    return wall, times


def time_decode_step(w, inputs, steps, warmup):
    """Seconds per decode step made as one msa_decode_step call (index kernel, then one
    kernel for the final selection, the attention and the merge), same inputs."""
    import torch
    from block_sparse_gqa_msa_amd import binding as msa

    s = msa.shape_of(w)
    sel = torch.empty((w.batch, w.h_kv, 1, w.top_k), dtype=torch.int32, device="cuda")
    o = torch.empty((w.batch, w.h_q, 1, w.d_h), dtype=inputs["q"].dtype, device="cuda")
    lse = torch.empty((w.batch, w.h_q, 1), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(1, msa.msa_decode_step_workspace_size(s)), dtype=torch.uint8,
                     device="cuda")
    call = lambda: msa.msa_decode_step(s, inputs["q"], inputs["k"], inputs["v"],
                                       inputs["q_idx"], inputs["k_idx"], sel, o, lse, ws)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


# ------------------------------------------------------------------ CPU baseline

def cpu_baseline_prefill(w, inputs, target_s=12.0, seed=0):
    import oracle
    orc = oracle.get()
    cpu = {k: inputs[k].cpu() for k in ("q", "k", "v", "q_idx", "k_idx")}
    rng = np.random.default_rng(seed)
    probe = np.sort(rng.choice(w.n_q, size=16, replace=False))
    t0 = time.perf_counter()
    orc.run(w, cpu, rows=probe)
    dt = time.perf_counter() - t0
    n = int(min(w.n_q, max(16, 16 * target_s / max(dt, 1e-3))))
    rows = np.sort(rng.choice(w.n_q, size=n, replace=False))
    t0 = time.perf_counter()
    orc.run(w, cpu, rows=rows)
    dt = time.perf_counter() - t0
    return dict(value=n / dt, unit="tok/s", cores=orc.max_threads(), kind="oracle",
                sample=f"{n} query rows drawn uniformly (seed {seed}) from the {w.n_q}-row "
                       f"prefill, all {w.h_kv} groups and {w.h_q} heads; {dt:.1f} s")


def cpu_baseline_kl(w, inputs, target_s=6.0, seed=1):
    import oracle
    orc = oracle.get()
    cpu = {k: inputs[k].cpu() for k in ("q", "k", "q_idx", "k_idx")}
    rng = np.random.default_rng(seed)
    probe = np.sort(rng.choice(w.n_q, size=8, replace=False))
    sel = orc.run(w, cpu, rows=probe, attention=False)["sel"]
    t0 = time.perf_counter()
    orc.kl(w, cpu, sel, rows=probe)
    dt = time.perf_counter() - t0
    n = int(min(w.n_q, max(8, 8 * target_s / max(dt, 1e-3))))
    rows = np.sort(rng.choice(w.n_q, size=n, replace=False))
    sel = orc.run(w, cpu, rows=rows, attention=False)["sel"]
    t0 = time.perf_counter()
    orc.kl(w, cpu, sel, rows=rows)
    dt = time.perf_counter() - t0
    return dict(value=n / dt, unit="tok/s", cores=orc.max_threads(), kind="oracle",
                sample=f"{n} query rows drawn uniformly (seed {seed}) from the {w.n_q}-row "
                       f"prefill, all {w.h_kv} groups (loss only; their selections are "
                       f"computed first and not timed); {dt:.1f} s")


def cpu_baseline_bwd(w, inputs, target_s=12.0):
    """The oracle's backward on the last m rows of the prefill (their selections computed
    first, untimed), m sized for about target_s seconds."""
    import oracle
    from block_sparse_gqa_msa_amd.inputs import generate_dout
    orc = oracle.get()
    dout_all = generate_dout(w, device="cuda")

    def sub(m):
        ws = w.replace(n_q=m, q_start=w.q_start + w.n_q - m)
        cpu = {k: inputs[k].cpu() for k in ("k", "v", "k_idx")}
        cpu["q"] = inputs["q"][:, :, -m:].cpu()
        cpu["q_idx"] = inputs["q_idx"][:, :, -m:].cpu()
        sel = orc.run(ws, cpu, attention=False)["sel"]
        return ws, cpu, sel, dout_all[:, :, -m:].cpu()

    ws, cpu, sel, do = sub(32)
    t0 = time.perf_counter()
    orc.attn_bwd(ws, cpu, sel, do)
    dt = time.perf_counter() - t0
    m = int(min(w.n_q, max(32, 32 * target_s / max(dt, 1e-3))))
    ws, cpu, sel, do = sub(m)
    t0 = time.perf_counter()
    orc.attn_bwd(ws, cpu, sel, do)
    dt = time.perf_counter() - t0
    return dict(value=m / dt, unit="tok/s", cores=orc.max_threads(), kind="oracle",
                sample=f"the last {m} rows of the {w.n_q}-row prefill, all {w.h_kv} groups and "
                       f"{w.h_q} heads (dq of those rows, their dk and dv contributions; "
                       f"selections computed first and not timed); {dt:.1f} s")


def cpu_baseline_project(w, d_model, target_s=6.0, seed=4):
    """The oracle's projections of uniformly drawn rows of the step's hidden states."""
    import oracle
    import torch
    from block_sparse_gqa_msa_amd.inputs import generate_hidden
    orc = oracle.get()
    hid = generate_hidden(w, d_model, device="cuda")
    wq, wk = hid["w_q"].cpu(), hid["w_k"].cpu()
    rng = np.random.default_rng(seed)

    def rows_x(m):
        rows = torch.as_tensor(np.sort(rng.choice(w.n_q, size=m, replace=False)), device="cuda")
        return hid["x"][:, rows].cpu()

    x = rows_x(256)
    t0 = time.perf_counter()
    orc.project(x, wq, wk, w.h_kv, w.d_idx)
    dt = time.perf_counter() - t0
    m = int(min(w.n_q, max(256, 256 * target_s / max(dt, 1e-3))))
    x = rows_x(m)
    t0 = time.perf_counter()
    orc.project(x, wq, wk, w.h_kv, w.d_idx)
    dt = time.perf_counter() - t0
    return dict(value=w.batch * m / dt, unit="tok/s", cores=orc.max_threads(), kind="oracle",
                sample=f"{m} rows drawn uniformly (seed {seed}) from the {w.n_q}-row prefill's "
                       f"hidden states (d_model {d_model}); {dt:.1f} s")


def cpu_baseline_decode(w, inputs, target_s=6.0):
    import oracle
    orc = oracle.get()
    wb = w.replace(batch=1)
    cpu = {k: inputs[k][0:1].cpu() for k in ("q", "k", "v", "q_idx", "k_idx")}
    n, t0 = 0, time.perf_counter()
    while True:  # the step of one sequence, repeated for a few seconds
        orc.run(wb, cpu)
        n += 1
        dt = time.perf_counter() - t0
        if dt >= target_s:
            break
    return dict(value=n / dt, unit="tok/s", cores=orc.max_threads(), kind="oracle",
                sample=f"sequence 0 of {w.batch} (one decode token over {w.n_k} cached tokens), "
                       f"{n} repetitions in {dt:.1f} s")


# ------------------------------------------------------------------ counters

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def source_digest(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from the FETCH_SIZE / WRITE_SIZE
    counter runs recorded in profiles/traffic.json (each scaled by what the counter
    reads for a plain copy of known size), or None when there is no record or the
    kernel's sources have changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)["kernels"][f"{kernel}@{workload}"]
    except (OSError, KeyError, ValueError):
        return None
    if source_digest(rec["sources"]) != rec["source_digest"]:
        return None
    return rec["traffic_bytes"]


def copy_calibration(n_bytes=1 << 30, reps=5):
    """A plain device-to-device copy of known size, for scaling the HBM byte counters."""
    import torch
    src = torch.ones(n_bytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n_bytes, "copy_bytes_written": n_bytes, "reps": reps}))


# ------------------------------------------------------------------ main

def run_chunk(args, wc, time_step, generate, log):
    """The headline step on a chunked prefill: timing, per-stage times and the index
    kernel's roofline (its FLOPs dominate there)."""
    import torch
    inp = generate(wc, device="cuda")
    log(f"[bench] chunked prefill {wc.name}: warmup {args.warmup}, steps {args.steps}")
    cwall, ckt = time_step(wc, inp, args.steps, args.warmup, decode=False, extras=False)
    c_index, c_main = prefill_work(wc)
    t_ci = ckt["index_scores"]
    chunk = dict(
        workload=wc.name, value=wc.batch * wc.n_q / cwall, unit="tok/s",
        ms_per_step=cwall * 1e3,
        config={"batch": wc.batch, "rows": wc.n_q, "q_start": wc.q_start, "kv_len": wc.n_k,
                "top_k": wc.top_k},
        roofline=dict(kernel="index_pool_prefill", bound="mfma", achieved=c_index / t_ci / 1e12,
                      peak=PEAK_BF16_FLOPS / 1e12, unit="TFLOP/s",
                      frac=c_index / t_ci / PEAK_BF16_FLOPS,
                      traffic=measured_traffic("index_pool_prefill", wc.name),
                      per_launch_flops=c_index, avg_launch_ms=t_ci * 1e3),
        path_mfma=dict(flops=c_index + c_main, tflops=(c_index + c_main) / cwall / 1e12,
                       mfma_frac=(c_index + c_main) / cwall / PEAK_BF16_FLOPS),
        kernel_ms={k: v * 1e3 for k, v in ckt.items()})
    log(f"[bench] chunked prefill {cwall * 1e3:.2f} ms/step, kernels (ms): "
        + ", ".join(f"{k} {v * 1e3:.3f}" for k, v in ckt.items()))
    del inp
    torch.cuda.empty_cache()
    return chunk


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=200)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--prefill", default="prefill_128k")
    ap.add_argument("--chunk", default="chunk_1m")
    ap.add_argument("--sections", default="prefill,chunk,decode",
                    help="comma-separated subset of prefill, chunk, decode (for profiling runs; "
                         "the JSON line needs prefill)")
    ap.add_argument("--decode", default="decode_1m_b4")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 1 GiB device copy (to scale the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the MSA library has no multi-GPU path; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    sections = set(args.sections.split(","))
    if not sections <= {"prefill", "chunk", "decode"}:
        ap.error(f"unknown section in --sections {args.sections}")
    if "prefill" in sections and "decode" not in sections:
        ap.error("the JSON line carries prefill and decode: --sections needs both or no prefill")

    if args.calibrate_copy:
        copy_calibration()
        return

    import torch
    from block_sparse_gqa_msa_amd import binding as msa
    from block_sparse_gqa_msa_amd.inputs import WORKLOADS, generate

    msa.load_library()
    log = lambda m: print(m, file=sys.stderr, flush=True)
    if "prefill" not in sections:  # a profiling run: time the other sections, print no line
        if "chunk" in sections:
            log(json.dumps(run_chunk(args, WORKLOADS[args.chunk], time_step, generate, log)))
        if "decode" in sections:
            wd = WORKLOADS[args.decode]
            inp = generate(wd, device="cuda")
            dwall, dkt = time_step(wd, inp, args.decode_steps, args.warmup, decode=True)
            fused = time_decode_step(wd, inp, args.decode_steps, args.warmup)
            log(f"[bench] decode {dwall * 1e6:.1f} us/step, one call {fused * 1e6:.1f} us/step")
        return

    # ---- prefill at 128K
    wp = WORKLOADS[args.prefill]
    inp = generate(wp, device="cuda")
    log(f"[bench] prefill {wp.name}: warmup {args.warmup}, steps {args.steps}")
    wall, kt = time_step(wp, inp, args.steps, args.warmup, decode=False)
    f_index, f_main = prefill_work(wp)
    tok_s = wp.batch * wp.n_q / wall
    # dominant kernel by time: the index kernel (index FLOPs) or kv_attend (main-branch FLOPs)
    cand = [dict(kernel="index_pool_prefill", stage="index_scores", flops=f_index),
            dict(kernel="kv_attend", stage="attn_partials", flops=f_main)]
    dom = max(cand, key=lambda c: kt[c["stage"]])
    t_dom = kt[dom["stage"]]
    roof = dict(kernel=dom["kernel"], bound="mfma", achieved=dom["flops"] / t_dom / 1e12,
                peak=PEAK_BF16_FLOPS / 1e12, unit="TFLOP/s",
                frac=dom["flops"] / t_dom / PEAK_BF16_FLOPS,
                traffic=measured_traffic(dom["kernel"], wp.name),
                per_launch_flops=dom["flops"], avg_launch_ms=t_dom * 1e3)
    path = dict(flops=f_index + f_main, tflops=(f_index + f_main) / wall / 1e12,
                mfma_frac=(f_index + f_main) / wall / PEAK_BF16_FLOPS)
    t_kl = kt.pop("index_kl")
    log(f"[bench] prefill {wall * 1e3:.2f} ms/step, kernels (ms): "
        + ", ".join(f"{k} {v * 1e3:.3f}" for k, v in kt.items()))
    f_kl = kl_work(wp)
    kl = dict(workload=wp.name, value=wp.batch * wp.n_q / t_kl, unit="tok/s",
              ms_per_call=t_kl * 1e3,
              roofline=dict(kernel="kv_kl", bound="mfma", achieved=f_kl / t_kl / 1e12,
                            peak=PEAK_BF16_FLOPS / 1e12, unit="TFLOP/s",
                            frac=f_kl / t_kl / PEAK_BF16_FLOPS,
                            traffic=measured_traffic("kv_kl", wp.name),
                            per_launch_flops=f_kl, avg_launch_ms=t_kl * 1e3))
    log(f"[bench] alignment loss {t_kl * 1e3:.2f} ms/call")
    t_bwd = kt.pop("attn_backward")
    t_bst = {k: kt.pop(k) for k in ("bwd_plan", "bwd_partials", "bwd_merge")}
    t_kvb = t_bst["bwd_partials"]  # the kv_bwd kernel alone
    f_bwd = bwd_work(wp)
    bwd = dict(workload=wp.name, value=wp.batch * wp.n_q / t_bwd, unit="tok/s",
               ms_per_call=t_bwd * 1e3,
               roofline=dict(kernel="kv_bwd", bound="mfma", achieved=f_bwd / t_kvb / 1e12,
                             peak=PEAK_BF16_FLOPS / 1e12, unit="TFLOP/s",
                             frac=f_bwd / t_kvb / PEAK_BF16_FLOPS,
                             traffic=measured_traffic("kv_bwd", wp.name),
                             per_launch_flops=f_bwd, avg_launch_ms=t_kvb * 1e3),
               call_mfma=dict(tflops=f_bwd / t_bwd / 1e12, mfma_frac=f_bwd / t_bwd / PEAK_BF16_FLOPS),
               stage_ms={k: v * 1e3 for k, v in t_bst.items()})
    log(f"[bench] attention backward {t_bwd * 1e3:.2f} ms/call")
    t_pj = kt.pop("index_project")
    d_model = wp.h_q * wp.d_h
    f_pj, b_pj = project_work(wp, d_model)
    # the bound is the larger of the two ideal times (bytes at the HBM peak, FLOPs at MFMA's)
    if b_pj / PEAK_HBM_BYTES >= f_pj / PEAK_BF16_FLOPS:
        pj_roof = dict(kernel="index_project", bound="hbm", achieved=b_pj / t_pj / 1e9,
                       peak=PEAK_HBM_BYTES / 1e9, unit="GB/s", frac=b_pj / t_pj / PEAK_HBM_BYTES,
                       per_launch_bytes=b_pj)
    else:
        pj_roof = dict(kernel="index_project", bound="mfma", achieved=f_pj / t_pj / 1e12,
                       peak=PEAK_BF16_FLOPS / 1e12, unit="TFLOP/s",
                       frac=f_pj / t_pj / PEAK_BF16_FLOPS, per_launch_flops=f_pj)
    pj_roof.update(traffic=measured_traffic("index_project", wp.name), avg_launch_ms=t_pj * 1e3,
                   tflops=f_pj / t_pj / 1e12, mfma_frac=f_pj / t_pj / PEAK_BF16_FLOPS)
    proj = dict(workload=wp.name, d_model=d_model, value=wp.batch * wp.n_q / t_pj, unit="tok/s",
                ms_per_call=t_pj * 1e3, roofline=pj_roof)
    log(f"[bench] index projections {t_pj * 1e3:.3f} ms/call")
    cpu_p = None
    if not args.no_cpu:
        log("[bench] oracle CPU baseline (prefill sample)")
        cpu_p = cpu_baseline_prefill(wp, inp)
        log("[bench] oracle CPU baseline (alignment loss sample)")
        kl["cpu_baseline"] = cpu_baseline_kl(wp, inp)
        log("[bench] oracle CPU baseline (backward sample)")
        bwd["cpu_baseline"] = cpu_baseline_bwd(wp, inp)
        log("[bench] oracle CPU baseline (projection sample)")
        proj["cpu_baseline"] = cpu_baseline_project(wp, d_model)
    del inp
    torch.cuda.empty_cache()

    # ---- chunked prefill: the last rows of a 1M context (the index kernel dominates)
    chunk = None
    if "chunk" in sections:
        chunk = run_chunk(args, WORKLOADS[args.chunk], time_step, generate, log)

    # ---- decode at 1M
    wd = WORKLOADS[args.decode]
    inp = generate(wd, device="cuda")
    log(f"[bench] decode {wd.name}: warmup {args.warmup}, steps {args.decode_steps}")
    dwall, dkt = time_step(wd, inp, args.decode_steps, args.warmup, decode=True)
    fused_ms = time_decode_step(wd, inp, args.decode_steps, args.warmup) * 1e3
    log(f"[bench] decode as one msa_decode_step call: {fused_ms * 1e3:.1f} us/step")
    d_bytes, d_index_bytes, _ = decode_work(wd)
    t_idx = dkt["index_topk"]
    droof = dict(kernel="index_select_decode+topk_merge_wide", bound="hbm",
                 achieved=d_index_bytes / t_idx / 1e9, peak=PEAK_HBM_BYTES / 1e9,
                 unit="GB/s", frac=d_index_bytes / t_idx / PEAK_HBM_BYTES,
                 traffic=measured_traffic("index_select_decode", wd.name),
                 per_launch_bytes=d_index_bytes, avg_launch_ms=t_idx * 1e3)
    log(f"[bench] decode {dwall * 1e6:.1f} us/step, kernels (us): "
        + ", ".join(f"{k} {v * 1e6:.1f}" for k, v in dkt.items()))
    cpu_d = None
    if not args.no_cpu:
        log("[bench] oracle CPU baseline (decode sample)")
        cpu_d = cpu_baseline_decode(wd, inp)

    line = {
        "metric": METRIC,
        "value": tok_s,
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wp.name, "batch": wp.batch, "seq_len": wp.n_q, "h_q": wp.h_q,
                   "h_kv": wp.h_kv, "d_h": wp.d_h, "d_idx": wp.d_idx,
                   "block_size": wp.block_size, "top_k": wp.top_k, "parallelism": "none"},
        "roofline": roof,
        "path_mfma": path,
        "kernel_ms": {k: v * 1e3 for k, v in kt.items()},
        "cpu_baseline": cpu_p,
        "index_kl": kl,
        "attn_backward": bwd,
        "index_project": proj,
        "chunked_prefill": chunk,
        "decode": {
            "workload": wd.name, "value": wd.batch / dwall, "unit": "tok/s",
            "steps": args.decode_steps, "ms_per_step": dwall * 1e3,
            "config": {"batch": wd.batch, "kv_len": wd.n_k, "h_q": wd.h_q, "h_kv": wd.h_kv,
                       "d_h": wd.d_h, "d_idx": wd.d_idx, "block_size": wd.block_size,
                       "top_k": wd.top_k},
            "roofline": droof,
            "path_hbm": dict(bytes=d_bytes, gbs=d_bytes / dwall / 1e9,
                             hbm_frac=d_bytes / dwall / PEAK_HBM_BYTES),
            "kernel_ms": {k: v * 1e3 for k, v in dkt.items()},
            "decode_step_call": {"ms_per_step": fused_ms, "value": wd.batch / (fused_ms * 1e-3),
                                 "hbm_frac": d_bytes / (fused_ms * 1e-3) / PEAK_HBM_BYTES},
            "cpu_baseline": cpu_d,
        },
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
