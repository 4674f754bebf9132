"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI, run the
oracle on the same input bits, and compare with the stated tolerances."""
from __future__ import annotations

import sys
import time

import numpy as np
import torch

import oracle
from block_sparse_gqa_msa_amd import binding as msa
from block_sparse_gqa_msa_amd.inputs import Workload, generate

# Tolerances on the main-branch output O (and a derived bound for LSE).
TOL = {"f32": dict(o_max=1e-5, o_mean=1e-5, lse=1e-5),
       "bf16": dict(o_max=2e-2, o_mean=1e-2, lse=1e-3)}


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_cpu(inputs, keys=("q", "k", "v", "q_idx", "k_idx")):
    return {k: inputs[k].cpu() for k in keys if k in inputs}


def run_gpu(w: Workload, inputs, block_scores=False, kv_capacity=0):
    s = msa.shape_of(w, kv_capacity=kv_capacity)
    buf = msa.Buffers(s, block_scores=block_scores)
    msa.msa_step(buf, inputs)
    torch.cuda.synchronize()
    return buf


def check_selection_invariants(w: Workload, sel: torch.Tensor):
    """Properties every row's selection has at any size: count min(k, local+1), the local
    block present and last, strictly ascending, -1 padding, every entry visible."""
    sel = sel.cpu().numpy()
    B, R, n, k = sel.shape
    t = np.arange(n)
    local = (w.q_start + t) // w.block_size                          # [n]
    count = np.minimum(k, local + 1)
    valid = sel >= 0
    assert np.array_equal(valid.sum(-1), np.broadcast_to(count, (B, R, n))), "selection count"
    # valid entries first, then padding
    assert np.all(valid[..., :-1] | ~valid[..., 1:]), "padding not at the end"
    last = np.take_along_axis(sel, (count - 1)[None, None, :, None].repeat(B, 0).repeat(R, 1), -1)[..., 0]
    assert np.array_equal(last, np.broadcast_to(local, (B, R, n))), "local block not last"
    d = np.diff(sel, axis=-1)
    both = valid[..., 1:] & valid[..., :-1]
    assert np.all(d[both] > 0), "selection not strictly ascending"
    assert np.all(sel[valid] >= 0)


def compare(w: Workload, buf, ref, rows=None, seqs=None, label=""):
    """Compare GPU outputs (optionally at sampled rows / sequences) with oracle outputs."""
    sel = buf.sel
    o = buf.o
    lse = buf.lse
    if seqs is not None:
        sel, o, lse = sel[seqs], o[seqs], lse[seqs]
    if rows is not None:
        ridx = torch.as_tensor(rows, device=sel.device, dtype=torch.long)
        sel, o, lse = sel[:, :, ridx], o[:, :, ridx], lse[:, :, ridx]
    g_sel = sel.cpu().numpy()
    mism = int((g_sel != ref["sel"]).any(-1).sum())
    assert mism == 0, f"{label}: {mism} (row, group) selections differ from the oracle"
    g_o = o.float().cpu().numpy().astype(np.float64)
    err = np.abs(g_o - ref["o"])
    tol = TOL[w.dtype]
    log(f"{label}: sel exact on {g_sel.shape[0] * g_sel.shape[1] * g_sel.shape[2]} rows, "
        f"O max-abs {err.max():.3e} mean-abs {err.mean():.3e}")
    assert err.max() <= tol["o_max"], f"{label}: O max-abs {err.max()}"
    assert err.mean() <= tol["o_mean"], f"{label}: O mean-abs {err.mean()}"
    lerr = np.abs(lse.cpu().numpy().astype(np.float64) - ref["lse"]).max()
    assert lerr <= tol["lse"], f"{label}: LSE max-abs {lerr}"
    return err.max(), err.mean()


def sample_rows(w: Workload, n_random=64, seed=0):
    """First rows (take-all selections), rows at block edges, random rows and the last rows."""
    n = w.n_q
    rows = set(range(min(n, 48)))
    bs = w.block_size
    first_block_edge = (-w.q_start) % bs
    for e in range(first_block_edge, n, max(bs, n // 16)):
        rows.update(x for x in (e - 1, e, e + 1) if 0 <= x < n)
    rng = np.random.default_rng(seed)
    rows.update(rng.integers(0, n, size=min(n_random, n)).tolist())
    rows.update(range(max(0, n - 40), n))
    return sorted(rows)


def oracle_run(w: Workload, cpu_inputs, rows=None, block_scores=False):
    t0 = time.time()
    out = oracle.get().run(w, cpu_inputs, rows=rows, block_scores=block_scores)
    log(f"  oracle {w.name}: {len(rows) if rows is not None else w.n_q} rows in {time.time() - t0:.1f}s")
    return out
