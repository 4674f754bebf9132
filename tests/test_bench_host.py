"""Host logic of bench.py (CPU only): the algorithmic work models that every roofline
figure divides by, checked against counts taken from the oracle's own selections, and the
command-line contract (one GPU; sections)."""
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
from block_sparse_gqa_msa_amd.inputs import Workload, generate

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def W(n_q, n_k, top_k, block_size=16, batch=1, seed=5):
    return Workload("host", "f32", batch, n_q, n_k, n_k - n_q, 4, 2, 16, 8, block_size, top_k,
                    3, 1.0, 2, seed)


def visible_selected_tokens(w, sel):
    """Tokens j <= p inside the selected blocks, per (b, r, t), counted one by one."""
    p = w.q_start + np.arange(w.n_q)
    out = np.zeros(sel.shape[:3], dtype=np.int64)
    for b in range(sel.shape[0]):
        for r in range(sel.shape[1]):
            for t in range(sel.shape[2]):
                for c in sel[b, r, t]:
                    if c < 0:
                        continue
                    lo, hi = c * w.block_size, min((c + 1) * w.block_size, p[t] + 1)
                    out[b, r, t] += max(0, hi - lo)
    return out


@pytest.fixture(scope="module")
def orc():
    oracle.build()
    return oracle.get()


@pytest.mark.parametrize("n_q,n_k,top_k", [(70, 70, 3), (40, 130, 4), (1, 97, 5), (33, 33, 40)])
def test_work_models_match_the_oracles_selection(orc, n_q, n_k, top_k):
    w = W(n_q, n_k, top_k)
    inp = generate(w)
    ref = orc.run(w, inp, attention=False)
    tok = visible_selected_tokens(w, ref["sel"])  # [B, R, n_q]
    G = w.h_q // w.h_kv
    f_index, f_main = bench.prefill_work(w)
    p = w.q_start + np.arange(w.n_q)
    assert f_index == w.batch * w.h_kv * float(np.sum(p + 1)) * 2 * w.d_idx
    assert f_main == float(tok.sum()) * G * 4 * w.d_h
    assert bench.kl_work(w) == float(tok.sum()) * (2 * w.d_h * G + 2 * w.d_idx)
    assert bench.bwd_work(w) == float(tok.sum()) * G * 10 * w.d_h
    if n_q == 1:  # decode: the selected K/V bytes are the visible tokens' rows
        total, index_bytes, per_seq = bench.decode_work(w)
        assert per_seq["kv"] * w.h_kv == tok[0].sum() * w.h_kv * w.d_h * 2 * 2
        assert per_seq["k_idx"] == w.n_k * w.d_idx * 2


def _bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_bench_refuses_more_than_one_gpu():
    r = _bench("--gpus", "2")
    assert r.returncode == 2 and "one GPU" in r.stderr


@pytest.mark.parametrize("sections", ["decode,bogus", "prefill_2k", ""])
def test_bench_rejects_unknown_legs(sections):
    r = _bench("--sections", sections)
    assert r.returncode == 2 and "--sections" in r.stderr


def test_bench_sections_run_in_leg_order():
    import argparse
    ap = argparse.ArgumentParser()
    assert bench.parse_sections("c5b,c1,prefill", ap) == ["prefill_128k", "prefill_512_f32",
                                                          "decode_1m_b4"]
    assert bench.parse_sections("all", ap) == bench.LEGS
    from block_sparse_gqa_msa_amd.inputs import WORKLOADS
    assert all(name in WORKLOADS for name in bench.LEGS)


def test_correctness_block_counts_what_differs():
    """The bench's parity block: a planted selection difference and output error are
    reported as such, on sampled rows."""
    import torch
    w = W(8, 8, 2)
    B, H, R, n, k, d = w.batch, w.h_q, w.h_kv, w.n_q, w.top_k, w.d_h
    rng = np.random.default_rng(0)
    ref = dict(sel=rng.integers(0, 4, (B, R, n, k)).astype(np.int32),
               o=rng.standard_normal((B, H, n, d)), lse=rng.standard_normal((B, H, n)))
    sel = torch.as_tensor(ref["sel"]).clone()
    o = torch.as_tensor(ref["o"], dtype=torch.float32).clone()
    lse = torch.as_tensor(ref["lse"], dtype=torch.float32).clone()
    rows = [1, 3, 6]
    sub = dict(sel=ref["sel"][:, :, rows], o=ref["o"][:, :, rows], lse=ref["lse"][:, :, rows])
    c = bench.correctness(w, sel, o, lse, rows, sub)
    assert c["sel_mismatch"] == 0 and c["o_max_abs"] < 1e-6 and c["pass"]
    sel[0, 1, 3, 0] += 1         # a checked row
    sel[0, 0, 2, 0] += 1         # a row outside the sample
    o[0, 2, 6, 5] += 0.5
    c = bench.correctness(w, sel, o, lse, rows, sub)
    assert c["rows_checked"] == B * R * len(rows)
    assert c["sel_mismatch"] == 1 and abs(c["o_max_abs"] - 0.5) < 1e-6 and not c["pass"]
