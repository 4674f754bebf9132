"""GPU parity of the top-k for rows with more than 2048 candidate blocks, where the index
kernel also writes the largest score of every aligned run of 32 blocks and the top-k reads
only the runs that can hold a winner (plus the tail after the last whole run), falling back
to ranking every chunk when ties at the bound leave too many runs.

Each case compares, on the same inputs: the oracle's selection; msa_index_topk; its two
stages (msa_index_topk_scores, msa_index_topk_select); and the route without run scores
(msa_index_block_scores, msa_topk_from_block_scores), which ranks every candidate."""
from __future__ import annotations

import pytest
import torch

from block_sparse_gqa_msa_amd import binding as msa
from block_sparse_gqa_msa_amd.inputs import Workload, generate
from gpu_cases import check_selection_invariants, compare, log, oracle_run, run_gpu, to_cpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    msa.load_library()  # raises if libmsa.so is missing: no fallback


def W(name, n_q, q_start, block_size=32, top_k=16, h_q=8, h_kv=2, d_h=64, d_idx=32,
      idx_range=4, needles=8, seed=11):
    return Workload(name, "bf16", 1, n_q, q_start + n_q, q_start, h_q, h_kv, d_h, d_idx,
                    block_size, top_k, idx_range, 0.5, needles, seed)


def all_routes(w: Workload, inp):
    """sel from msa_index_topk, from its two stages, and from the route without run scores."""
    s = msa.shape_of(w)
    B, R, n, k = w.batch, w.h_kv, w.n_q, w.top_k
    nb = -(-w.n_k // w.block_size)
    dev = inp["q_idx"].device
    ws = torch.empty(max(1, msa.msa_index_topk_workspace_size(s)), dtype=torch.uint8, device=dev)
    out = {}
    sel = torch.full((B, R, n, k), -7, dtype=torch.int32, device=dev)
    msa.msa_index_topk(s, inp["q_idx"], inp["k_idx"], sel, None, ws)
    out["fused"] = sel
    sel = torch.full((B, R, n, k), -7, dtype=torch.int32, device=dev)
    ws.fill_(0xAB)  # stale workspace: the stages must not depend on its contents
    msa.msa_index_topk_scores(s, inp["q_idx"], inp["k_idx"], None, ws)
    msa.msa_index_topk_select(s, sel, None, ws)
    out["staged"] = sel
    scores = torch.empty((B, R, n, nb), dtype=torch.float32, device=dev)
    wst = torch.empty(max(1, msa.msa_topk_workspace_size(s)), dtype=torch.uint8, device=dev)
    sel = torch.full((B, R, n, k), -7, dtype=torch.int32, device=dev)
    msa.msa_index_block_scores(s, inp["q_idx"], inp["k_idx"], scores)
    msa.msa_topk_from_block_scores(s, scores, sel, wst)
    out["chunked"] = sel
    torch.cuda.synchronize()
    return out


def check_case(w: Workload, inp):
    log(f"case {w.name}: {w}")
    routes = all_routes(w, inp)
    ref = oracle_run(w, to_cpu(inp))
    for name, sel in routes.items():
        check_selection_invariants(w, sel)
        g = sel.cpu().numpy()
        mism = int((g != ref["sel"]).any(-1).sum())
        assert mism == 0, f"{w.name} ({name}): {mism} (row, group) selections differ from the oracle"
    # the whole step through msa_index_topk, with and without block scores requested
    for want_scores in (False, True):
        buf = run_gpu(w, inp, block_scores=want_scores)
        compare(w, buf, ref, label=f"{w.name} (block scores {want_scores})")


# local blocks 2200 .. 2218 of 32 tokens: rows with a 24-block tail, and rows whose local
# block starts a run (local = 2208: no tail)
def test_runs_tail_and_no_tail():
    w = W("runs_tail_mix", n_q=600, q_start=70400)
    check_case(w, generate(w, device="cuda"))


@pytest.mark.parametrize("top_k", [2, 33, 64])
def test_runs_top_k(top_k):
    """k = 2 (one winner), 33 (32 runs plus the tail: phase 2 with 32 slots) and 64 (63
    winners, 63 or 64 runs)."""
    w = W(f"runs_k{top_k}", n_q=160, q_start=140000, block_size=64, top_k=top_k, d_idx=64)
    check_case(w, generate(w, device="cuda"))


def test_runs_many_ties_at_bound():
    """Index values in {0, 1}: many runs share the bound, so phase 2 takes more runs than
    winners (or the chunked fallback takes over)."""
    w = W("runs_few_values", n_q=256, q_start=70000, top_k=32, idx_range=1)
    inp = generate(w, device="cuda")
    inp["q_idx"].abs_()
    inp["k_idx"].abs_()
    check_case(w, inp)


def test_runs_all_ties_fallback():
    """All index keys zero: every run key ties, so every row takes the chunked fallback
    inside the top-k wave; the lowest blocks win."""
    w = W("runs_all_ties", n_q=128, q_start=70000, top_k=16)
    inp = generate(w, device="cuda")
    inp["k_idx"].zero_()
    check_case(w, inp)


def test_runs_many_chunks():
    """About 32800 candidate blocks (17 chunks of 2048): 1025 run keys per row in phase 1."""
    w = W("runs_many_chunks", n_q=40, q_start=(1 << 20) + 56, top_k=16)
    check_case(w, generate(w, device="cuda"))


def test_runs_batch_ragged():
    """Two sequences, rows not a multiple of the index kernel's row tile, four groups."""
    w = Workload("runs_batch2", "bf16", 2, 333, 67000 + 333, 67000, 16, 4, 64, 32, 32, 12, 4,
                 0.5, 6, 5)
    check_case(w, generate(w, device="cuda"))


def test_runs_equal_full_ranking_every_row_1m_chunk():
    """The 1M-context chunk (8192 rows, 16384 key blocks): on every row and group, the
    selection read through run keys equals the one that ranks every candidate."""
    from block_sparse_gqa_msa_amd.inputs import WORKLOADS
    w = WORKLOADS["chunk_1m"]
    log(f"case {w.name}: {w}")
    inp = generate(w, device="cuda")
    routes = all_routes(w, inp)
    ref = routes["chunked"]
    check_selection_invariants(w, ref)
    for name in ("fused", "staged"):
        diff = int((routes[name] != ref).any(-1).sum())
        assert diff == 0, f"{name}: {diff} (row, group) selections differ from the full ranking"
