"""GPU parity of the index branch's projections (msa_index_project) with the fp64 oracle.

Integer inputs (x in [-2, 2], weights in [-1, 1], d_model <= 128) make every output an
integer of magnitude <= 256, exact in fp32 and bf16, so those cases must match bit for bit.
Gaussian inputs: |got - ref| <= RTOL * |ref| + ATOL * max|ref| per tensor (bf16: the
output's rounding, 2^-9 relative, plus fp32 accumulation; fp32: accumulation only).
The k_idx cache must change only in the rows of the call's positions.
"""
import dataclasses

import numpy as np
import pytest
import torch

from block_sparse_gqa_msa_amd import binding as msa
from block_sparse_gqa_msa_amd.inputs import WORKLOADS, Workload, generate_hidden
from gpu_cases import log

pytestmark = pytest.mark.gpu

PROJ_TOL = {"f32": (1e-5, 1e-6), "bf16": (4e-3, 1e-4)}  # (rtol, atol as a fraction of max|ref|)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    msa.load_library()


def W(name, dtype="bf16", batch=1, n_q=256, n_k=256, q_start=0, h_q=32, h_kv=4, d_h=128,
      d_idx=64, block_size=64, top_k=8, idx_range=4, qkv_scale=0.5, needles=0, seed=7):
    return Workload(name, dtype, batch, n_q, n_k, q_start, h_q, h_kv, d_h, d_idx, block_size,
                    top_k, idx_range, qkv_scale, needles, seed)


SENTINEL = 5.0


def gpu_project(w, hid, cap=None):
    cap = cap or w.n_k
    s = msa.shape_of(w, kv_capacity=cap if cap != w.n_k else 0)
    dt = hid["x"].dtype
    q_idx = torch.full((w.batch, w.h_kv, w.n_q, w.d_idx), float("nan"), dtype=dt, device="cuda")
    k_idx = torch.full((w.batch, cap, w.d_idx), SENTINEL, dtype=dt, device="cuda")
    msa.msa_index_project(s, hid["x"], hid["w_q"], hid["w_k"], q_idx, k_idx)
    torch.cuda.synchronize()
    return q_idx, k_idx


def check(w, name, got, want, exact, label):
    g = got.float().cpu().numpy().astype(np.float64)
    assert np.isfinite(g).all(), f"{label}: {name} not finite"
    err = np.abs(g - want)
    log(f"{label}: {name} max-abs err {err.max():.3e} (max|ref| {np.abs(want).max():.3e})")
    if exact:
        assert np.array_equal(g, want), f"{label}: {name} not exact"
        return
    rtol, atol = PROJ_TOL[w.dtype]
    bound = rtol * np.abs(want) + atol * np.abs(want).max()
    worst = np.unravel_index((err - bound).argmax(), err.shape)
    assert (err <= bound).all(), f"{label}: {name} worst at {worst}: {g[worst]} vs {want[worst]}"


def check_cache(w, k_idx, want_rows, exact, label, rows=None):
    """Rows q_start .. q_start + n_q - 1 hold the projections; every other row is unchanged."""
    lo, hi = w.q_start, w.q_start + w.n_q
    outside = torch.cat([k_idx[:, :lo], k_idx[:, hi:]], dim=1)
    assert (outside == SENTINEL).all(), f"{label}: k_idx rows outside the call's positions changed"
    got = k_idx[:, lo:hi] if rows is None else k_idx[:, lo + torch.as_tensor(rows, device="cuda")]
    check(w, "k_idx", got, want_rows, exact, label)


SMALL = [
    (W("proj_int_bf16", n_q=300, n_k=300), 128, True),
    (W("proj_int_f32_r2_d32", dtype="f32", n_q=257, n_k=400, q_start=100, h_kv=2, d_idx=32), 64, True),
    (W("proj_int_bf16_r16", batch=2, n_q=130, n_k=200, q_start=70, h_q=32, h_kv=16), 128, True),
    (W("proj_gauss_bf16", batch=2, n_q=500, n_k=700, q_start=200), 1024, False),
    (W("proj_gauss_f32", dtype="f32", n_q=333, n_k=333, h_kv=8, d_idx=32), 320, False),
    (W("proj_gauss_bf16_r1_d32", n_q=64, n_k=64, h_q=8, h_kv=1, d_idx=32), 4096, False),
    (W("proj_decode", batch=3, n_q=1, n_k=5000, q_start=4999), 512, False),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: c[0].name)
def test_project_small_full_oracle(case):
    import oracle
    w, d_model, integer = case
    log(f"case {w.name}: d_model {d_model}, integer {integer}: {w}")
    hid = generate_hidden(w, d_model, device="cuda", integer=integer)
    q_idx, k_idx = gpu_project(w, hid)
    ref = oracle.get().project(hid["x"].cpu(), hid["w_q"].cpu(), hid["w_k"].cpu(), w.h_kv, w.d_idx)
    check(w, "q_idx", q_idx, ref["q_idx"], integer, w.name)
    check_cache(w, k_idx, ref["k_idx"], integer, w.name)


def test_project_kv_capacity_stride():
    """A cache allocated longer than n_k: the rows land at the capacity stride."""
    import oracle
    w = W("proj_cap", batch=2, n_q=100, n_k=300, q_start=200)
    hid = generate_hidden(w, 256, device="cuda")
    q_idx, k_idx = gpu_project(w, hid, cap=w.n_k + 77)
    ref = oracle.get().project(hid["x"].cpu(), hid["w_q"].cpu(), hid["w_k"].cpu(), w.h_kv, w.d_idx)
    check(w, "q_idx", q_idx, ref["q_idx"], False, w.name)
    check_cache(w, k_idx, ref["k_idx"], False, w.name)


def test_project_then_select_matches_oracle():
    """Integer hidden states and weights: the projections are exact, so the block selection
    that msa_index_topk makes from them is the oracle's selection from the oracle's
    projections, bit for bit (a chunked prefill whose earlier cache rows are given)."""
    import oracle
    orc = oracle.get()
    w = W("proj_select", n_q=512, n_k=1536, q_start=1024, h_q=8, h_kv=2, d_h=64, d_idx=32,
          block_size=32, top_k=8)
    hid = generate_hidden(w, 128, device="cuda", integer=True)
    # the earlier cache rows: integer index keys as the library would have appended them
    earlier = dataclasses.replace(w, n_q=w.q_start, q_start=0)
    hid_e = generate_hidden(earlier, 128, device="cuda", integer=True, seed=99)
    hid_e["w_q"], hid_e["w_k"] = hid["w_q"], hid["w_k"]
    _, k_early = gpu_project(earlier, hid_e, cap=w.n_k)
    s = msa.shape_of(w)
    q_idx = torch.empty((w.batch, w.h_kv, w.n_q, w.d_idx), dtype=torch.bfloat16, device="cuda")
    k_idx = k_early.clone()
    msa.msa_index_project(s, hid["x"], hid["w_q"], hid["w_k"], q_idx, k_idx)
    sel = torch.empty((w.batch, w.h_kv, w.n_q, w.top_k), dtype=torch.int32, device="cuda")
    ws = torch.empty(max(1, msa.msa_index_topk_workspace_size(s)), dtype=torch.uint8, device="cuda")
    msa.msa_index_topk(s, q_idx, k_idx, sel, None, ws)
    torch.cuda.synchronize()
    # the oracle's projections of both chunks, then its selection
    pe = orc.project(hid_e["x"].cpu(), hid["w_q"].cpu(), hid["w_k"].cpu(), w.h_kv, w.d_idx)
    pc = orc.project(hid["x"].cpu(), hid["w_q"].cpu(), hid["w_k"].cpu(), w.h_kv, w.d_idx)
    k_all = np.concatenate([pe["k_idx"], pc["k_idx"]], axis=1)
    inputs = dict(q=torch.zeros(w.batch, w.h_q, w.n_q, w.d_h), k=torch.zeros(w.batch, w.h_kv, w.n_k, w.d_h),
                  v=torch.zeros(w.batch, w.h_kv, w.n_k, w.d_h),
                  q_idx=torch.from_numpy(pc["q_idx"]).float(), k_idx=torch.from_numpy(k_all).float())
    wf = dataclasses.replace(w, dtype="f32")
    ref = orc.run(wf, inputs, attention=False)["sel"]
    assert np.array_equal(sel.cpu().numpy(), ref), "selection from the projections differs"
    log(f"{w.name}: selection from the GPU projections equals the oracle's")


@pytest.mark.parametrize("name", ["prefill_128k", "chunk_1m", "decode_1m_b4"])
def test_project_workload_sampled_rows(name):
    """The workloads' shapes at full size with d_model = h_q * d_h: sampled rows against
    the oracle, and the cache rows outside the call's positions untouched."""
    import oracle
    w = WORKLOADS[name]
    d_model = w.h_q * w.d_h
    log(f"case {name}: d_model {d_model}")
    hid = generate_hidden(w, d_model, device="cuda")
    q_idx, k_idx = gpu_project(w, hid)
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([np.arange(min(w.n_q, 70)), rng.integers(0, w.n_q, 64),
                                     np.arange(max(0, w.n_q - 70), w.n_q)]))
    ridx = torch.as_tensor(rows, device="cuda")
    ref = oracle.get().project(hid["x"][:, ridx].cpu(), hid["w_q"].cpu(), hid["w_k"].cpu(),
                               w.h_kv, w.d_idx)
    check(w, "q_idx", q_idx[:, :, ridx], ref["q_idx"], False, f"{name} ({len(rows)} rows)")
    check_cache(w, k_idx, ref["k_idx"], False, f"{name} ({len(rows)} rows)", rows=rows)
