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


@pytest.mark.parametrize("sections", ["prefill", "prefill,chunk", "decode,bogus"])
def test_bench_rejects_section_sets(sections):
    r = _bench("--sections", sections)
    assert r.returncode == 2 and "--sections" in r.stderr
