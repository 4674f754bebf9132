"""Benchmark of the MSA hot path on one MI355X; prints ONE JSON line.

Headline (``value``): causal prefill tokens/s at N = 131072 (32 query heads / 4 KV
groups, d_h 128, index d_idx 64, blocks of 64, top_k 32, bf16): one step is the index
branch (block scores, top-k) plus the sparse prefill attention over all 131072 rows.
Every workload of the measured set has a leg of its own in the same line, each with its
throughput, the roofline of its dominant kernel, the fp64 oracle timed on a bounded sample
on the host cores, and a correctness block comparing the outputs of the timed run with
the oracle on that sample:
  prefill_512_f32    the tiny fp32 prefill (parity only: no roofline applies)
  prefill_8k         causal prefill N = 8192, top_k 16
  prefill_128k       the headline (top-level keys), plus, on its selection and outputs:
                     index_kl (alignment loss), attn_backward (dq, dk, dv) and
                     index_project (the index branch's two projections)
  prefill_128k_hot   the same step with every row choosing the same blocks (all index
                     inputs zero: ties everywhere, lowest block index first), the
                     most skewed block popularity there is
  chunk_1m           the last 8192 rows of a 1M-token context against all 1M keys
  decode_256k_b32    decode, 32 sequences of 262144 cached tokens
  decode_1m_b4       decode, 4 sequences of 1048576 cached tokens (the metric's
                     "decode tok/s @1M"); also as one msa_decode_step call
Step times are medians over at least 20 repetitions: prefill steps one by one, decode
steps in repetitions of 10 (HIP events on the library's stream); the mean over the
timed region's wall clock is reported beside them.

Inputs are seeded synthetic tensors already resident in HBM when timing starts.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--decode-steps KD] [--no-cpu]
                    [--sections LEG,...] [--no-extras]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MSA attn: prefill tok/s @128K, decode tok/s @1M; % of MFMA/HBM roofline"
PEAK_BF16_FLOPS = 2.5e15   # MI355X dense bf16 MFMA
PEAK_HBM_BYTES = 8.0e12    # MI355X HBM3E
DECODE_REP = 10            # decode steps per timed repetition

# Legs in the order they run, and the short names --sections also accepts.
LEGS = ["prefill_128k", "prefill_128k_hot", "chunk_1m", "prefill_8k", "prefill_512_f32",
        "decode_256k_b32", "decode_1m_b4"]
ALIASES = {"prefill": "prefill_128k", "hot": "prefill_128k_hot", "chunk": "chunk_1m",
           "c1": "prefill_512_f32", "c2": "prefill_8k", "c3": "prefill_128k",
           "c4": "decode_256k_b32", "c5a": "chunk_1m", "c5b": "decode_1m_b4",
           "decode": "decode_1m_b4"}
HEADLINE, HEADLINE_DECODE = "prefill_128k", "decode_1m_b4"
PARITY_ONLY = {"prefill_512_f32"}
# Output tolerances the correctness blocks are judged against (O max-abs, O mean-abs).
TOL = {"f32": dict(o_max_abs=1e-5, o_mean_abs=1e-5), "bf16": dict(o_max_abs=2e-2, o_mean_abs=1e-2)}
# The loss: |kl - ref| <= atol + rtol |ref|. dq: |dq - ref| <= atol max|ref| + rtol |ref| and
# mean error <= mean * mean|ref|. Projections: |x - ref| <= rtol |ref| + atol max|ref|.
KL_TOL = {"f32": dict(atol=2e-5, rtol=2e-5), "bf16": dict(atol=2e-4, rtol=2e-5)}
BWD_TOL = {"f32": dict(atol=2e-5, rtol=2e-5, mean=2e-5), "bf16": dict(atol=1e-2, rtol=1e-2, mean=6e-3)}
PROJ_TOL = {"f32": dict(rtol=1e-5, atol=1e-6), "bf16": dict(rtol=4e-3, atol=1e-4)}


# ------------------------------------------------------------------ algorithmic work

def _visible_tokens(w):
    p = w.q_start + np.arange(w.n_q, dtype=np.int64)
    b = p // w.block_size
    return p, (np.minimum(w.top_k, b + 1) - 1) * w.block_size + (p - b * w.block_size + 1)


def prefill_work(w):
    """Algorithmic FLOPs of one step: index scores R*(p+1)*2*d_idx per row plus main
    branch H_q*T_p*4*d_h, T_p = visible tokens of the selected blocks."""
    p, t_p = _visible_tokens(w)
    index = float(w.batch * w.h_kv * np.sum(p + 1) * 2 * w.d_idx)
    main = float(w.batch * w.h_q * np.sum(t_p) * 4 * w.d_h)
    return index, main


def kl_work(w):
    """Algorithmic FLOPs of msa_index_kl: per (row, group) and selected visible token, the
    G heads' q.k (2*d_h each) and the index score q_idx.k_idx (2*d_idx)."""
    _, t_p = _visible_tokens(w)
    G = w.h_q // w.h_kv
    return float(w.batch * w.h_kv * np.sum(t_p) * (2 * w.d_h * G + 2 * w.d_idx))


def bwd_work(w):
    """Algorithmic FLOPs of msa_sparse_attn_backward: per (row, head) and selected visible
    token, q.k (recomputed), dout.v, and the three products that give dv, dk and dq
    (2*d_h each)."""
    _, t_p = _visible_tokens(w)
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

def timed_reps(step, steps, warmup, per=1):
    """Run `warmup` untimed steps, then exactly `steps` timed ones (synchronised on both
    sides) with a HIP event on the current stream before every `per` steps. Returns the
    median seconds per step over the repetitions, the mean from the wall clock, and the
    number of repetitions."""
    import torch
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    n_rep = steps // per
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n_rep + 1)]
    t0 = time.perf_counter()
    for i in range(n_rep * per):
        if i % per == 0:
            ev[i // per].record(stream)
        step()
    ev[n_rep].record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / (n_rep * per)
    reps = [ev[i].elapsed_time(ev[i + 1]) * 1e-3 / per for i in range(n_rep)]
    return float(np.median(reps)), wall, n_rep


def stage_medians(stages, steps):
    """Per-stage medians from a pass of `steps` steps with an event before each stage (kept
    out of the timed region: recording many events per short step costs host time)."""
    import torch
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
          for _ in range(steps)]
    for i in range(steps):
        for j, (_, call) in enumerate(stages):
            ev[i][j].record(stream)
            call()
        ev[i][-1].record(stream)
    torch.cuda.synchronize()
    return {name: float(np.median([e[j].elapsed_time(e[j + 1]) for e in ev])) * 1e-3
            for j, (name, _) in enumerate(stages)}


class PrefillRun:
    """Output buffers and the five staged calls of one prefill step (each stage its own
    call so that every kernel is timed alone; together they are the whole step)."""

    def __init__(self, w, inputs):
        import torch
        from block_sparse_gqa_msa_amd import binding as msa
        self.w, self.inputs, s = w, inputs, msa.shape_of(w)
        self.s = s
        R, n = w.h_kv, w.n_q
        dev = "cuda"
        self.sel = torch.empty((w.batch, R, n, w.top_k), dtype=torch.int32, device=dev)
        self.o = torch.empty((w.batch, w.h_q, n, w.d_h), dtype=inputs["q"].dtype, device=dev)
        self.lse = torch.empty((w.batch, w.h_q, n), dtype=torch.float32, device=dev)
        # block maxima, top-k candidates and run scores: msa_index_topk's workspace, which
        # its two stages share
        self.ws_index = torch.empty(max(1, msa.msa_index_topk_workspace_size(s)),
                                    dtype=torch.uint8, device=dev)
        self.ws_attn = torch.empty(max(1, msa.msa_sparse_attn_workspace_size(s)),
                                   dtype=torch.uint8, device=dev)
        i = inputs
        self.stages = [
            ("index_scores", lambda: msa.msa_index_topk_scores(s, i["q_idx"], i["k_idx"], None,
                                                               self.ws_index)),
            ("topk", lambda: msa.msa_index_topk_select(s, self.sel, None, self.ws_index)),
            ("attn_plan", lambda: msa.msa_sparse_attn_prefill_plan(s, self.sel, self.ws_attn)),
            ("attn_partials", lambda: msa.msa_sparse_attn_prefill_partials(
                s, i["q"], i["k"], i["v"], self.ws_attn)),
            ("attn_merge", lambda: msa.msa_sparse_attn_prefill_merge(s, self.sel, self.o,
                                                                     self.lse, self.ws_attn)),
        ]

    def step(self):
        for _, call in self.stages:
            call()


class DecodeRun:
    """Buffers and calls of one decode step: msa_index_topk + msa_sparse_attn_decode, and
    the same step as one msa_decode_step call."""

    def __init__(self, w, inputs):
        import torch
        from block_sparse_gqa_msa_amd import binding as msa
        self.w, self.inputs, s = w, inputs, msa.shape_of(w)
        self.s = s
        dev = "cuda"
        self.sel = torch.empty((w.batch, w.h_kv, 1, w.top_k), dtype=torch.int32, device=dev)
        self.o = torch.empty((w.batch, w.h_q, 1, w.d_h), dtype=inputs["q"].dtype, device=dev)
        self.lse = torch.empty((w.batch, w.h_q, 1), dtype=torch.float32, device=dev)
        self.ws_index = torch.empty(max(1, msa.msa_index_topk_workspace_size(s)),
                                    dtype=torch.uint8, device=dev)
        self.ws_attn = torch.empty(max(1, msa.msa_sparse_attn_workspace_size(s)),
                                   dtype=torch.uint8, device=dev)
        self.ws_step = torch.empty(max(1, msa.msa_decode_step_workspace_size(s)),
                                   dtype=torch.uint8, device=dev)
        i = inputs
        self.stages = [
            ("index_topk", lambda: msa.msa_index_topk(s, i["q_idx"], i["k_idx"], self.sel, None,
                                                      self.ws_index)),
            ("attention", lambda: msa.msa_sparse_attn_decode(s, i["q"], i["k"], i["v"], self.sel,
                                                             self.o, self.lse, self.ws_attn)),
        ]
        self.one_call = lambda: msa.msa_decode_step(s, i["q"], i["k"], i["v"], i["q_idx"],
                                                    i["k_idx"], self.sel, self.o, self.lse,
                                                    self.ws_step)

    def step(self):
        for _, call in self.stages:
            call()


# ------------------------------------------------------------------ oracle: baseline and parity

def correctness(w, sel, o, lse, rows, ref, seqs=None):
    """The timed run's outputs against the oracle's at the sampled rows (prefill) or
    sequences (decode): (row, group) selections that differ, O max / mean abs error,
    LSE max abs error."""
    import torch
    if seqs is not None:
        idx = torch.as_tensor(seqs, device=sel.device, dtype=torch.long)
        sel, o, lse = sel[idx], o[idx], lse[idx]
    if rows is not None:
        idx = torch.as_tensor(rows, device=sel.device, dtype=torch.long)
        sel, o, lse = sel[:, :, idx], o[:, :, idx], lse[:, :, idx]
    g_sel = sel.cpu().numpy()
    err = np.abs(o.float().cpu().numpy().astype(np.float64) - ref["o"])
    lerr = np.abs(lse.cpu().numpy().astype(np.float64) - ref["lse"])
    tol = TOL[w.dtype]
    out = dict(rows_checked=int(g_sel.shape[0] * g_sel.shape[1] * g_sel.shape[2]),
               sel_mismatch=int((g_sel != ref["sel"]).any(-1).sum()),
               o_max_abs=float(err.max()), o_mean_abs=float(err.mean()),
               lse_max_abs=float(lerr.max()), tol=tol)
    out["pass"] = bool(out["sel_mismatch"] == 0 and out["o_max_abs"] <= tol["o_max_abs"]
                       and out["o_mean_abs"] <= tol["o_mean_abs"])
    return out


def oracle_prefill(w, inputs, target_s, seed=0, full=False):
    """The oracle on uniformly drawn rows of the prefill (all rows when `full`), sized for
    about `target_s` seconds from a 16-row probe. Returns the baseline record, the rows
    and the oracle's outputs for them."""
    import oracle
    orc = oracle.get()
    cpu = {k: inputs[k].cpu() for k in ("q", "k", "v", "q_idx", "k_idx")}
    rng = np.random.default_rng(seed)
    if full:
        rows = np.arange(w.n_q)
    else:
        probe = np.sort(rng.choice(w.n_q, size=min(16, w.n_q), replace=False))
        t0 = time.perf_counter()
        orc.run(w, cpu, rows=probe)
        dt = time.perf_counter() - t0
        n = int(min(w.n_q, max(16, 16 * target_s / max(dt, 1e-3))))
        rows = np.sort(rng.choice(w.n_q, size=n, replace=False))
    t0 = time.perf_counter()
    ref = orc.run(w, cpu, rows=rows)
    dt = time.perf_counter() - t0
    what = (f"all {w.n_q} rows" if len(rows) == w.n_q else
            f"{len(rows)} query rows drawn uniformly (seed {seed}) from the {w.n_q}-row prefill")
    base = dict(value=w.batch * len(rows) / dt, unit="tok/s", cores=orc.max_threads(),
                kind="oracle", sample=f"{what}, all {w.h_kv} groups and {w.h_q} heads; {dt:.1f} s")
    return base, rows, ref


def oracle_decode(w, inputs, target_s, seqs):
    """Baseline: the oracle's step of sequence 0 repeated for about `target_s` seconds.
    Parity: the oracle once on the sequences `seqs`."""
    import oracle
    orc = oracle.get()
    idx = list(seqs)
    cpu = {k: inputs[k][idx].cpu() for k in ("q", "k", "v", "q_idx", "k_idx")}
    ref = orc.run(w.replace(batch=len(idx)), cpu)
    one = {k: v[0:1] for k, v in cpu.items()}
    wb = w.replace(batch=1)
    n, t0 = 0, time.perf_counter()
    while True:
        orc.run(wb, one)
        n += 1
        dt = time.perf_counter() - t0
        if dt >= target_s:
            break
    base = dict(value=n / dt, unit="tok/s", cores=orc.max_threads(), kind="oracle",
                sample=f"sequence 0 of {w.batch} (one decode token over {w.n_k} cached tokens), "
                       f"{n} repetitions in {dt:.1f} s")
    return base, ref


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
    ref = orc.kl(w, cpu, sel, rows=rows)
    dt = time.perf_counter() - t0
    base = dict(value=n / dt, unit="tok/s", cores=orc.max_threads(), kind="oracle",
                sample=f"{n} query rows drawn uniformly (seed {seed}) from the {w.n_q}-row "
                       f"prefill, all {w.h_kv} groups (loss only; their selections are "
                       f"computed first and not timed); {dt:.1f} s")
    return base, rows, ref


def cpu_baseline_bwd(w, inputs, target_s=10.0):
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
    ref = orc.attn_bwd(ws, cpu, sel, do)
    dt = time.perf_counter() - t0
    base = dict(value=m / dt, unit="tok/s", cores=orc.max_threads(), kind="oracle",
                sample=f"the last {m} rows of the {w.n_q}-row prefill, all {w.h_kv} groups and "
                       f"{w.h_q} heads (dq of those rows, their dk and dv contributions; "
                       f"selections computed first and not timed); {dt:.1f} s")
    return base, m, ref["dq"]


def cpu_baseline_project(w, d_model, target_s=5.0, seed=4):
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
    rows = np.sort(rng.choice(w.n_q, size=m, replace=False))
    x = hid["x"][:, torch.as_tensor(rows, device="cuda")].cpu()
    t0 = time.perf_counter()
    ref = orc.project(x, wq, wk, w.h_kv, w.d_idx)
    dt = time.perf_counter() - t0
    base = dict(value=w.batch * m / dt, unit="tok/s", cores=orc.max_threads(), kind="oracle",
                sample=f"{m} rows drawn uniformly (seed {seed}) from the {w.n_q}-row prefill's "
                       f"hidden states (d_model {d_model}); {dt:.1f} s")
    return base, rows, ref


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


def mfma_roofline(kernel, flops, seconds, workload):
    return dict(kernel=kernel, bound="mfma", achieved=flops / seconds / 1e12,
                peak=PEAK_BF16_FLOPS / 1e12, unit="TFLOP/s", frac=flops / seconds / PEAK_BF16_FLOPS,
                traffic=measured_traffic(kernel, workload), per_launch_flops=flops,
                avg_launch_ms=seconds * 1e3)


# ------------------------------------------------------------------ legs

def prefill_leg(w, args, log, cpu_s=8.0, extras=False):
    """One prefill workload: median step time, per-stage medians, the dominant kernel's
    roofline, the whole step's MFMA fraction, the oracle baseline and parity."""
    import torch
    from block_sparse_gqa_msa_amd.inputs import generate
    inp = generate(w, device="cuda")
    run = PrefillRun(w, inp)
    log(f"[bench] {w.name}: warmup {args.warmup}, steps {args.steps}")
    med, wall, reps = timed_reps(run.step, args.steps, args.warmup)
    kt = stage_medians(run.stages, args.steps)
    f_index, f_main = prefill_work(w)
    leg = dict(workload=w.name, value=w.batch * w.n_q / med, unit="tok/s",
               ms_per_step=med * 1e3, ms_per_step_mean=wall * 1e3, reps=reps,
               config={"batch": w.batch, "rows": w.n_q, "q_start": w.q_start, "kv_len": w.n_k,
                       "h_q": w.h_q, "h_kv": w.h_kv, "d_h": w.d_h, "d_idx": w.d_idx,
                       "block_size": w.block_size, "top_k": w.top_k, "dtype": w.dtype},
               kernel_ms={k: v * 1e3 for k, v in kt.items()})
    if w.name in PARITY_ONLY:
        leg["roofline"] = None
        leg["parity_only"] = True
    else:
        # dominant kernel by time: the index kernel (index FLOPs) or kv_attend (main FLOPs)
        cand = [("index_pool_prefill", "index_scores", f_index), ("kv_attend", "attn_partials", f_main)]
        kern, stage, flops = max(cand, key=lambda c: kt[c[1]])
        leg["roofline"] = mfma_roofline(kern, flops, kt[stage], w.name)
        leg["path_mfma"] = dict(flops=f_index + f_main, tflops=(f_index + f_main) / med / 1e12,
                                mfma_frac=(f_index + f_main) / med / PEAK_BF16_FLOPS)
    log(f"[bench] {w.name} {med * 1e3:.3f} ms/step (mean {wall * 1e3:.3f}), kernels (ms): "
        + ", ".join(f"{k} {v * 1e3:.3f}" for k, v in kt.items()))
    if extras:
        leg.update(prefill_extras(w, inp, run, args, log))
    if not args.no_cpu:
        log(f"[bench] oracle on {w.name}")
        base, rows, ref = oracle_prefill(w, inp, cpu_s, full=w.name in PARITY_ONLY)
        leg["cpu_baseline"] = base
        leg["correctness"] = correctness(w, run.sel, run.o, run.lse, rows, ref)
        log(f"[bench] {w.name} parity: {json.dumps(leg['correctness'])}")
    del run, inp
    torch.cuda.empty_cache()
    return leg


def prefill_extras(w, inp, run, args, log):
    """The alignment loss, the backward and the index projections on the prefill's last
    step (its selection, o and lse), each with its oracle baseline and a parity block on
    the rows the oracle computed."""
    import torch
    from block_sparse_gqa_msa_amd import binding as msa
    from block_sparse_gqa_msa_amd.inputs import generate_dout, generate_hidden
    s, R, n = run.s, w.h_kv, w.n_q
    out = {}
    # the alignment loss of the same step
    kl = torch.empty((w.batch, R, n), dtype=torch.float32, device="cuda")
    kl_call = lambda: msa.msa_index_kl(s, inp["q"], inp["k"], inp["q_idx"], inp["k_idx"], run.sel,
                                       run.lse, kl, None, run.ws_attn)
    t_kl, _, reps = timed_reps(kl_call, args.steps, max(1, args.warmup))
    f_kl = kl_work(w)
    out["index_kl"] = dict(workload=w.name, value=w.batch * n / t_kl, unit="tok/s",
                           ms_per_call=t_kl * 1e3, reps=reps,
                           roofline=mfma_roofline("kv_kl", f_kl, t_kl, w.name))
    log(f"[bench] alignment loss {t_kl * 1e3:.2f} ms/call")
    # the main branch's backward for the same selection, o and lse
    dout = generate_dout(w, device="cuda")
    dq, dk, dv = (torch.empty_like(inp[x]) for x in ("q", "k", "v"))
    ws_bwd = torch.empty(msa.msa_sparse_attn_backward_workspace_size(s), dtype=torch.uint8,
                         device="cuda")
    bwd_call = lambda: msa.msa_sparse_attn_backward(s, inp["q"], inp["k"], inp["v"], run.sel,
                                                    run.o, run.lse, dout, dq, dk, dv, ws_bwd)
    t_bwd, _, reps = timed_reps(bwd_call, args.steps, max(1, args.warmup))
    # the same backward as its three staged calls, so the per-block kernel is timed alone
    bst = [("bwd_plan", lambda: msa.msa_sparse_attn_backward_plan(s, run.sel, run.o, dout, ws_bwd)),
           ("bwd_partials", lambda: msa.msa_sparse_attn_backward_partials(
               s, inp["q"], inp["k"], inp["v"], run.lse, dout, ws_bwd)),
           ("bwd_merge", lambda: msa.msa_sparse_attn_backward_merge(s, run.sel, dq, dk, dv, ws_bwd))]
    t_bst = stage_medians(bst, args.steps)
    del dout, dk, dv, ws_bwd
    f_bwd = bwd_work(w)
    out["attn_backward"] = dict(
        workload=w.name, value=w.batch * n / t_bwd, unit="tok/s", ms_per_call=t_bwd * 1e3,
        reps=reps, roofline=mfma_roofline("kv_bwd", f_bwd, t_bst["bwd_partials"], w.name),
        call_mfma=dict(tflops=f_bwd / t_bwd / 1e12, mfma_frac=f_bwd / t_bwd / PEAK_BF16_FLOPS),
        stage_ms={k: v * 1e3 for k, v in t_bst.items()})
    log(f"[bench] attention backward {t_bwd * 1e3:.2f} ms/call")
    # the index branch's projections of the step's rows (hidden width h_q * d_h)
    d_model = w.h_q * w.d_h
    hid = generate_hidden(w, d_model, device="cuda")
    q_idx_p, k_idx_p = torch.empty_like(inp["q_idx"]), torch.empty_like(inp["k_idx"])
    proj_call = lambda: msa.msa_index_project(s, hid["x"], hid["w_q"], hid["w_k"], q_idx_p, k_idx_p)
    t_pj, _, reps = timed_reps(proj_call, args.steps, max(1, args.warmup))
    del hid
    f_pj, b_pj = project_work(w, d_model)
    # the bound is the larger of the two ideal times (bytes at the HBM peak, FLOPs at MFMA's)
    if b_pj / PEAK_HBM_BYTES >= f_pj / PEAK_BF16_FLOPS:
        roof = dict(kernel="index_project", bound="hbm", achieved=b_pj / t_pj / 1e9,
                    peak=PEAK_HBM_BYTES / 1e9, unit="GB/s", frac=b_pj / t_pj / PEAK_HBM_BYTES,
                    per_launch_bytes=b_pj)
    else:
        roof = dict(kernel="index_project", bound="mfma", achieved=f_pj / t_pj / 1e12,
                    peak=PEAK_BF16_FLOPS / 1e12, unit="TFLOP/s",
                    frac=f_pj / t_pj / PEAK_BF16_FLOPS, per_launch_flops=f_pj)
    roof.update(traffic=measured_traffic("index_project", w.name), avg_launch_ms=t_pj * 1e3,
                tflops=f_pj / t_pj / 1e12, mfma_frac=f_pj / t_pj / PEAK_BF16_FLOPS)
    out["index_project"] = dict(workload=w.name, d_model=d_model, value=w.batch * n / t_pj,
                                unit="tok/s", ms_per_call=t_pj * 1e3, reps=reps, roofline=roof)
    log(f"[bench] index projections {t_pj * 1e3:.3f} ms/call")
    if not args.no_cpu:
        log("[bench] oracle baselines and parity of the alignment loss, the backward, the projections")
        base, rows, ref = cpu_baseline_kl(w, inp)
        got = kl[:, :, torch.as_tensor(rows, device="cuda")].cpu().numpy().astype(np.float64)
        err = np.abs(got - ref["kl"])
        tol = KL_TOL[w.dtype]
        out["index_kl"]["cpu_baseline"] = base
        out["index_kl"]["correctness"] = dict(
            rows_checked=int(got.size), kl_max_abs=float(err.max()),
            worst_over_bound=float((err / (tol["atol"] + tol["rtol"] * np.abs(ref["kl"]))).max()),
            tol=tol, **{"pass": bool((err <= tol["atol"] + tol["rtol"] * np.abs(ref["kl"])).all())})
        base, m, ref_dq = cpu_baseline_bwd(w, inp)
        got = dq[:, :, -m:].float().cpu().numpy().astype(np.float64)
        err = np.abs(got - ref_dq)
        tol, scale = BWD_TOL[w.dtype], np.abs(ref_dq).max()
        ok = (err <= tol["atol"] * scale + tol["rtol"] * np.abs(ref_dq)).all() and \
            err.mean() <= tol["mean"] * np.abs(ref_dq).mean()
        out["attn_backward"]["cpu_baseline"] = base
        out["attn_backward"]["correctness"] = dict(
            rows_checked=int(m * w.batch * w.h_q), tensor="dq of the last rows",
            dq_max_abs_over_max_ref=float(err.max() / scale),
            dq_mean_abs_over_mean_ref=float(err.mean() / np.abs(ref_dq).mean()),
            tol=tol, **{"pass": bool(ok)})
        base, rows, ref = cpu_baseline_project(w, d_model)
        ridx = torch.as_tensor(rows, device="cuda")
        ok, worst = True, 0.0
        for got_t, want in ((q_idx_p[:, :, ridx], ref["q_idx"]), (k_idx_p[:, ridx], ref["k_idx"])):
            got = got_t.float().cpu().numpy().astype(np.float64)
            tol = PROJ_TOL[w.dtype]
            bound = tol["rtol"] * np.abs(want) + tol["atol"] * np.abs(want).max()
            worst = max(worst, float((np.abs(got - want) / bound).max()))
            ok = ok and bool((np.abs(got - want) <= bound).all())
        out["index_project"]["cpu_baseline"] = base
        out["index_project"]["correctness"] = dict(rows_checked=int(len(rows) * w.batch),
                                                   worst_over_bound=worst, tol=PROJ_TOL[w.dtype],
                                                   **{"pass": ok})
        for key in ("index_kl", "attn_backward", "index_project"):
            log(f"[bench] {key} parity: {json.dumps(out[key]['correctness'])}")
    del kl, dq, q_idx_p, k_idx_p
    torch.cuda.empty_cache()
    return out


def decode_leg(w, args, log, parity_seqs, cpu_s=5.0):
    """One decode workload: median step time (repetitions of DECODE_REP steps) of the step as
    one msa_decode_step call, the same step as two calls (msa_index_topk, then
    msa_sparse_attn_decode) beside it, the index kernel's HBM roofline, the whole step's HBM
    fraction, the oracle baseline and parity on `parity_seqs` (of the one-call outputs)."""
    import torch
    from block_sparse_gqa_msa_amd.inputs import generate
    inp = generate(w, device="cuda")
    run = DecodeRun(w, inp)
    steps = max(DECODE_REP, args.decode_steps // DECODE_REP * DECODE_REP)
    log(f"[bench] {w.name}: warmup {args.warmup}, steps {steps}")
    two, two_wall, _ = timed_reps(run.step, steps, args.warmup, per=DECODE_REP)
    kt = stage_medians(run.stages, steps)
    med, wall, reps = timed_reps(run.one_call, steps, args.warmup, per=DECODE_REP)
    d_bytes, d_index_bytes, _ = decode_work(w)
    t_idx = kt["index_topk"]
    leg = dict(
        workload=w.name, value=w.batch / med, unit="tok/s", steps=steps, reps=reps,
        ms_per_step=med * 1e3, ms_per_step_mean=wall * 1e3, path="msa_decode_step",
        config={"batch": w.batch, "kv_len": w.n_k, "h_q": w.h_q, "h_kv": w.h_kv, "d_h": w.d_h,
                "d_idx": w.d_idx, "block_size": w.block_size, "top_k": w.top_k},
        roofline=dict(kernel="index_select_decode+topk_merge_wide", bound="hbm",
                      achieved=d_index_bytes / t_idx / 1e9, peak=PEAK_HBM_BYTES / 1e9,
                      unit="GB/s", frac=d_index_bytes / t_idx / PEAK_HBM_BYTES,
                      traffic=measured_traffic("index_select_decode", w.name),
                      per_launch_bytes=d_index_bytes, avg_launch_ms=t_idx * 1e3),
        path_hbm=dict(bytes=d_bytes, gbs=d_bytes / med / 1e9, hbm_frac=d_bytes / med / PEAK_HBM_BYTES),
        kernel_ms={k: v * 1e3 for k, v in kt.items()},
        two_calls={"ms_per_step": two * 1e3, "ms_per_step_mean": two_wall * 1e3,
                   "value": w.batch / two, "hbm_frac": d_bytes / two / PEAK_HBM_BYTES})
    log(f"[bench] {w.name} {med * 1e6:.1f} us/step as one call (mean {wall * 1e6:.1f}), "
        f"two calls {two * 1e6:.1f} us/step, their kernels (us): "
        + ", ".join(f"{k} {v * 1e6:.1f}" for k, v in kt.items()))
    if not args.no_cpu:
        log(f"[bench] oracle on {w.name}")
        run.one_call()  # the reported path's outputs (its timed loop ran last as well)
        torch.cuda.synchronize()
        base, ref = oracle_decode(w, inp, cpu_s, parity_seqs)
        leg["cpu_baseline"] = base
        leg["correctness"] = correctness(w, run.sel, run.o, run.lse, None, ref, seqs=parity_seqs)
        leg["correctness"]["sequences"] = list(parity_seqs)
        log(f"[bench] {w.name} parity: {json.dumps(leg['correctness'])}")
    del run, inp
    torch.cuda.empty_cache()
    return leg


def run_leg(name, args, log):
    from block_sparse_gqa_msa_amd.inputs import WORKLOADS
    w = WORKLOADS[name]
    if w.decode:
        seqs = list(range(w.batch)) if w.batch <= 4 else list(range(0, w.batch, w.batch // 8))
        return decode_leg(w, args, log, seqs)
    cpu_s = {"prefill_128k": 8.0, "prefill_128k_hot": 3.0, "chunk_1m": 6.0, "prefill_8k": 6.0}.get(name, 2.0)
    return prefill_leg(w, args, log, cpu_s=cpu_s,
                       extras=(name == HEADLINE and not args.no_extras))


# ------------------------------------------------------------------ main

def parse_sections(text, ap):
    if text == "all":
        return list(LEGS)
    want = []
    for part in text.split(","):
        name = ALIASES.get(part, part)
        if name not in LEGS:
            ap.error(f"unknown leg {part!r} in --sections (legs: {', '.join(LEGS)}, "
                     f"or {', '.join(ALIASES)})")
        want.append(name)
    return [n for n in LEGS if n in want]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=200)
    ap.add_argument("--no-cpu", action="store_true",
                    help="skip the oracle (CPU baselines and correctness blocks)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the alignment loss, backward and projections of the 128K prefill")
    ap.add_argument("--sections", default="all",
                    help="comma-separated legs to run (for profiling runs; the JSON line needs "
                         f"{HEADLINE} and {HEADLINE_DECODE}, otherwise each leg is logged)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 1 GiB device copy (to scale the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the MSA library has no multi-GPU path; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    legs = parse_sections(args.sections, ap)
    if args.steps < 1 or args.decode_steps < 1:
        ap.error("--steps and --decode-steps must be positive")

    if args.calibrate_copy:
        copy_calibration()
        return

    from block_sparse_gqa_msa_amd import binding as msa
    msa.load_library()
    log = lambda m: print(m, file=sys.stderr, flush=True)
    out = {}
    for name in legs:
        out[name] = run_leg(name, args, log)
        if HEADLINE not in legs or HEADLINE_DECODE not in legs:
            log(json.dumps({name: out[name]}))
    if HEADLINE not in legs or HEADLINE_DECODE not in legs:
        return  # a profiling run: no headline line

    head = out.pop(HEADLINE)
    w = head
    line = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "ms_per_step_mean": head["ms_per_step_mean"],
        "statistic": f"median over {head['reps']} timed steps",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": dict(workload=w["workload"], seq_len=w["config"]["rows"],
                       parallelism="none", **{k: v for k, v in w["config"].items()
                                              if k not in ("rows", "dtype")}),
        "roofline": head["roofline"],
        "path_mfma": head["path_mfma"],
        "kernel_ms": head["kernel_ms"],
        "cpu_baseline": head.get("cpu_baseline"),
        "correctness": head.get("correctness"),
        "index_kl": head.get("index_kl"),
        "attn_backward": head.get("attn_backward"),
        "index_project": head.get("index_project"),
        "decode": out.pop(HEADLINE_DECODE),
        "chunked_prefill": out.pop("chunk_1m", None),
    }
    line.update(out)  # the remaining legs under their workload names
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
