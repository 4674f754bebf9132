"""GPU parity of the main-branch backward (msa_sparse_attn_backward) with the fp64 oracle.

The GPU path takes its own forward's selection, o and lse (the selection is checked
against the oracle's, which the oracle side uses); the oracle recomputes everything from
the input bits. Small shapes are compared in full, element by element; the prefill
workloads run at full size with sampled rows of dq (each against the oracle on the
equivalent problem that holds only that row's selected blocks), sampled blocks of dk and
dv (summed from the same per-row problems of every row that chose the block) and, on all
of dk and dv, properties that hold at any size.

Tolerance per tensor X in {dq, dk, dv}: |X - ref| <= ATOL * max|ref| + RTOL * |ref|, and the
mean error <= MEAN * mean|ref|. bf16: the kernel rounds P and dS to bf16 for the matrix
cores, stores dq partials per selection in bf16 and takes D from the bf16 forward output
(relative 2^-9 each), then rounds the result to bf16; fp32 keeps every step in fp32.
"""
import dataclasses

import numpy as np
import pytest
import torch

from block_sparse_gqa_msa_amd import binding as msa
from block_sparse_gqa_msa_amd.inputs import WORKLOADS, Workload, generate, generate_dout
from gpu_cases import log, run_gpu, sample_rows, to_cpu

pytestmark = pytest.mark.gpu

BWD_TOL = {"f32": dict(atol=2e-5, rtol=2e-5, mean=2e-5),
           "bf16": dict(atol=1e-2, rtol=1e-2, mean=6e-3)}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    msa.load_library()


def W(name, dtype="bf16", batch=1, n_q=256, n_k=256, q_start=0, h_q=32, h_kv=4, d_h=128,
      d_idx=64, block_size=64, top_k=8, idx_range=4, qkv_scale=0.5, needles=0, seed=7):
    return Workload(name, dtype, batch, n_q, n_k, q_start, h_q, h_kv, d_h, d_idx, block_size,
                    top_k, idx_range, qkv_scale, needles, seed)


def gpu_bwd(w, inp, buf, dout, kv_capacity=0, fill=float("nan")):
    s = msa.shape_of(w, kv_capacity=kv_capacity)
    cap = kv_capacity or w.n_k
    dq = torch.full_like(inp["q"], fill)
    dk = torch.full((w.batch, w.h_kv, cap, w.d_h), fill, dtype=inp["q"].dtype, device="cuda")
    dv = torch.full_like(dk, fill)
    ws = torch.empty(max(1, msa.msa_sparse_attn_backward_workspace_size(s)), dtype=torch.uint8,
                     device="cuda")
    msa.msa_sparse_attn_backward(s, inp["q"], inp["k"], inp["v"], buf.sel, buf.o, buf.lse, dout,
                                 dq, dk, dv, ws)
    torch.cuda.synchronize()
    return dq, dk, dv


def check(w, name, got, want, label):
    tol = BWD_TOL[w.dtype]
    g = got.float().cpu().numpy().astype(np.float64) if torch.is_tensor(got) else got
    assert np.isfinite(g).all(), f"{label}: {name} not finite"
    err = np.abs(g - want)
    scale = np.abs(want).max()
    bound = tol["atol"] * scale + tol["rtol"] * np.abs(want)
    mean_ok = err.mean() <= tol["mean"] * max(np.abs(want).mean(), 1e-30)
    log(f"{label}: {name} max-abs err {err.max():.3e} (max|ref| {scale:.3e}), mean err "
        f"{err.mean():.3e} (mean|ref| {np.abs(want).mean():.3e})")
    worst = np.unravel_index((err - bound).argmax(), err.shape)
    assert (err <= bound).all(), f"{label}: {name} worst at {worst}: {g[worst]} vs {want[worst]}"
    assert mean_ok, f"{label}: {name} mean error {err.mean()} too large"


def oracle_sel(w, cpu, rows=None):
    import oracle
    return oracle.get().run(w, cpu, rows=rows, attention=False)["sel"]


SMALL = [
    WORKLOADS["prefill_512_f32"],
    W("bwd_ragged_bf16", batch=2, n_q=1000, n_k=1000, top_k=8, needles=4),
    W("bwd_chunk_g4_d64_bs32", n_q=300, n_k=1500, q_start=1200, h_q=8, h_kv=2, d_h=64, d_idx=32,
      block_size=32, top_k=5, needles=3),
    W("bwd_g1_r8_f32", dtype="f32", n_q=700, n_k=700, h_q=8, h_kv=8, d_h=64, d_idx=64, top_k=3,
      idx_range=3, qkv_scale=1.0),
    W("bwd_g16_r1_bs32", n_q=520, n_k=520, h_q=16, h_kv=1, d_h=128, d_idx=32, block_size=32,
      top_k=4),
    W("bwd_g2_r16_f32", dtype="f32", n_q=300, n_k=300, h_q=32, h_kv=16, d_h=64, d_idx=64,
      block_size=32, top_k=6, idx_range=3, qkv_scale=1.0),
    W("bwd_f32_d128_bs64", dtype="f32", n_q=640, n_k=640, h_q=8, h_kv=2, d_h=128, d_idx=64,
      top_k=4, idx_range=3, qkv_scale=1.0),
    W("bwd_f32_d128_bs32", dtype="f32", n_q=500, n_k=520, q_start=20, h_q=4, h_kv=2, d_h=128,
      d_idx=32, block_size=32, top_k=5, idx_range=3, qkv_scale=1.0),
    W("bwd_k1_local_only", n_q=777, n_k=777, top_k=1, block_size=32),
    W("bwd_k32_long_lists", n_q=1600, n_k=1600, h_q=16, h_kv=2, top_k=20, needles=6),
    W("bwd_batch3_chunk", batch=3, n_q=333, n_k=2000, q_start=1667, h_q=16, h_kv=2, d_h=128,
      d_idx=64, block_size=64, top_k=7, needles=5),
    W("bwd_bf16_d64_bs64_g8", n_q=900, n_k=900, h_q=32, h_kv=4, d_h=64, d_idx=32,
      block_size=64, top_k=10, needles=4),
    # one row at the end of a long cache (the decode shape): a single entry per list
    W("bwd_decode_row", batch=3, n_q=1, n_k=5000, q_start=4999, top_k=16, needles=4),
    # one group and many rows: the longest list (block 0, 1132 entries) spans more than one
    # run of 8 chunks x 128 entries; the first rows' selections are shorter than top_k
    W("bwd_long_list_runs", n_q=2600, n_k=2600, h_q=8, h_kv=1, d_h=64, d_idx=32,
      block_size=32, top_k=12, needles=1),
]


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_bwd_small_full_oracle(w):
    import oracle
    log(f"case {w.name}: {w}")
    inp = generate(w, device="cuda")
    dout = generate_dout(w, device="cuda")
    buf = run_gpu(w, inp)
    dq, dk, dv = gpu_bwd(w, inp, buf, dout)
    cpu = to_cpu(inp)
    sel = oracle_sel(w, cpu)
    assert np.array_equal(buf.sel.cpu().numpy(), sel), "selections differ"
    ref = oracle.get().attn_bwd(w, cpu, sel, dout.cpu())
    for name, got in (("dq", dq), ("dk", dk), ("dv", dv)):
        check(w, name, got, ref[name], w.name)
    # dq has a fixed summation order: a second call gives the same bits
    dq2, _, _ = gpu_bwd(w, inp, buf, dout)
    assert torch.equal(dq, dq2), "dq differs between two calls"


def test_bwd_kv_capacity_stride():
    """k, v (and dk, dv) with a token stride above n_k: rows past n_k are neither read as
    keys nor written."""
    import oracle
    w = W("bwd_cap", n_q=200, n_k=400, q_start=200, top_k=4, needles=2)
    inp = generate(w, device="cuda")
    dout = generate_dout(w, device="cuda")
    cap = w.n_k + 136
    big = dict(q=inp["q"], q_idx=inp["q_idx"])
    for key in ("k", "v"):
        x = torch.full((w.batch, w.h_kv, cap, w.d_h), 2.0, dtype=inp[key].dtype, device="cuda")
        x[:, :, : w.n_k] = inp[key]
        big[key] = x
    x = torch.full((w.batch, cap, w.d_idx), 3.0, dtype=inp["k_idx"].dtype, device="cuda")
    x[:, : w.n_k] = inp["k_idx"]
    big["k_idx"] = x
    buf = run_gpu(w, big, kv_capacity=cap)
    dq, dk, dv = gpu_bwd(w, big, buf, dout, kv_capacity=cap, fill=7.0)
    assert (dk[:, :, w.n_k:] == 7.0).all() and (dv[:, :, w.n_k:] == 7.0).all(), \
        "rows past n_k were written"
    cpu = to_cpu(inp)
    sel = oracle_sel(w, cpu)
    ref = oracle.get().attn_bwd(w, cpu, sel, dout.cpu())
    check(w, "dq", dq, ref["dq"], w.name)
    check(w, "dk", dk[:, :, : w.n_k], ref["dk"], w.name)
    check(w, "dv", dv[:, :, : w.n_k], ref["dv"], w.name)


def test_bwd_staged_calls_equal_single_call():
    """_plan, _partials and _merge on one workspace give the single call's dq bit for bit,
    and its dk, dv up to the order of a list's rows (the list build's atomics)."""
    w = W("bwd_staged", batch=2, n_q=700, n_k=900, q_start=200, h_q=16, h_kv=2, top_k=6,
          needles=3)
    inp = generate(w, device="cuda")
    dout = generate_dout(w, device="cuda")
    buf = run_gpu(w, inp)
    dq, dk, dv = gpu_bwd(w, inp, buf, dout)
    s = msa.shape_of(w)
    ws = torch.empty(msa.msa_sparse_attn_backward_workspace_size(s), dtype=torch.uint8,
                     device="cuda")
    dq2, dk2, dv2 = (torch.full_like(x, float("nan")) for x in (dq, dk, dv))
    msa.msa_sparse_attn_backward_plan(s, buf.sel, buf.o, dout, ws)
    msa.msa_sparse_attn_backward_partials(s, inp["q"], inp["k"], inp["v"], buf.lse, dout, ws)
    msa.msa_sparse_attn_backward_merge(s, buf.sel, dq2, dk2, dv2, ws)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq2), "staged dq differs"
    for a, b in ((dk, dk2), (dv, dv2)):
        assert torch.isfinite(b).all()
        assert (a.float() - b.float()).abs().max().item() <= 1e-2 * a.float().abs().max().item()


# ------------------------------------------------------------------ full-size workloads

def row_problem(w, cpu, dout_cpu, sel_row, b, r, t):
    """The equivalent problem that holds only row t's selected blocks (in ascending order,
    so the row's local block is last and every other one is fully visible): one sequence,
    one group, the row's G heads. Returns (workload, inputs, sel, dout, blocks)."""
    G, BS = w.h_q // w.h_kv, w.block_size
    blocks = [int(c) for c in sel_row if c >= 0]
    p = w.q_start + t
    assert blocks == sorted(blocks) and blocks[-1] == p // BS
    nv = len(blocks)
    kc = torch.zeros((1, 1, nv * BS, w.d_h), dtype=cpu["k"].dtype)
    vc = torch.zeros_like(kc)
    for i, c in enumerate(blocks):
        hi = min((c + 1) * BS, w.n_k)
        kc[0, 0, i * BS: i * BS + hi - c * BS] = cpu["k"][b, r, c * BS: hi]
        vc[0, 0, i * BS: i * BS + hi - c * BS] = cpu["v"][b, r, c * BS: hi]
    ws = dataclasses.replace(w, batch=1, n_q=1, n_k=nv * BS, q_start=(nv - 1) * BS + p % BS,
                             h_q=G, h_kv=1, top_k=nv)
    inp = dict(q=cpu["q"][b:b + 1, r * G:(r + 1) * G, t:t + 1].contiguous(), k=kc, v=vc)
    sel = np.arange(nv, dtype=np.int32).reshape(1, 1, 1, nv)
    do = dout_cpu[b:b + 1, r * G:(r + 1) * G, t:t + 1].contiguous()
    return ws, inp, sel, do, blocks


@pytest.mark.parametrize("name", ["prefill_8k", "prefill_128k", "chunk_1m"])
def test_bwd_workload_sampled(name):
    """Full-size prefill workloads: dq at sampled rows and dk, dv at two sampled blocks per
    workload against the oracle; on every key, dk and dv are exactly 0 where no row of
    the group selected the key's block or no row sees the key, sum_j dv_j equals the sum
    of the group's dout rows, and sum_j dk_j is 0 (each row's dS sums to 0)."""
    import oracle
    orc = oracle.get()
    w = WORKLOADS[name]
    log(f"case {name}: {w}")
    G, BS = w.h_q // w.h_kv, w.block_size
    inp = generate(w, device="cuda")
    dout = generate_dout(w, device="cuda")
    buf = run_gpu(w, inp)
    dq, dk, dv = gpu_bwd(w, inp, buf, dout)
    for x in (dq, dk, dv):
        assert torch.isfinite(x).all()
    cpu = to_cpu(inp)
    dout_cpu = dout.cpu()
    sel_all = buf.sel.cpu().numpy()

    # sampled rows of dq (the selection of those rows is checked against the oracle's)
    rows = sample_rows(w, n_random=24 if name == "prefill_8k" else 12)
    sel_ref = oracle_sel(w, cpu, rows=rows)
    assert np.array_equal(sel_all[:, :, rows], sel_ref), "selections differ"
    got, want = [], []
    for b in range(w.batch):
        for r in range(w.h_kv):
            for i, t in enumerate(rows):
                ws, pin, psel, pdo, _ = row_problem(w, cpu, dout_cpu, sel_ref[b, r, i], b, r, t)
                ref = orc.attn_bwd(ws, pin, psel, pdo)
                want.append(ref["dq"][0, :, 0])
                got.append(dq[b, r * G:(r + 1) * G, t].float().cpu().numpy())
    check(w, "dq (sampled rows)", np.stack(got).astype(np.float64), np.stack(want),
          f"{name} ({len(rows)} rows)")

    # exact zeros and sums over every key of each (b, r)
    B, R = w.batch, w.h_kv
    for b in range(B):
        for r in range(R):
            chosen = np.zeros(w.n_blocks, bool)
            s = sel_all[b, r]
            chosen[s[s >= 0]] = True
            key_chosen = np.repeat(chosen, BS)[: w.n_k]
            key_chosen[w.q_start + w.n_q:] = False  # after the last row: seen by no row
            mask = torch.as_tensor(~key_chosen, device="cuda")
            assert (dk[b, r][mask] == 0).all() and (dv[b, r][mask] == 0).all(), \
                "keys no row sees have nonzero gradients"
            dv_sum = dv[b, r].double().sum(0).cpu().numpy()
            want_sum = dout[b, r * G:(r + 1) * G].double().sum((0, 1)).cpu().numpy()
            dv_abs = dv[b, r].double().abs().sum(0).cpu().numpy()
            assert (np.abs(dv_sum - want_sum) <= 1e-2 * dv_abs + 1e-3).all(), "sum of dv"
            dk_sum = dk[b, r].double().sum(0).cpu().numpy()
            dk_abs = dk[b, r].double().abs().sum(0).cpu().numpy()
            assert (np.abs(dk_sum) <= 1e-2 * dk_abs + 1e-3).all(), "sum of dk"
    log(f"{name}: zero and sum properties hold on all {w.n_k} keys")

    # two sampled blocks of group 0, sequence 0: one picked by few rows, one by more
    b, r = 0, 0
    s = sel_all[b, r]
    counts = np.bincount(s[s >= 0].ravel(), minlength=w.n_blocks)
    lo_blk = int(w.q_start // BS)
    cand = [c for c in range(lo_blk, w.n_blocks) if 0 < counts[c] <= 96]
    rng = np.random.default_rng(1)
    picks = [cand[-1], int(rng.choice(cand))] if cand else []
    for c in picks:
        tt = np.nonzero((s == c).any(-1))[0]
        want_k = np.zeros((BS, w.d_h))
        want_v = np.zeros((BS, w.d_h))
        for t in tt:
            ws, pin, psel, pdo, blocks = row_problem(w, cpu, dout_cpu, s[t], b, r, int(t))
            ref = orc.attn_bwd(ws, pin, psel, pdo)
            i = blocks.index(c)
            want_k += ref["dk"][0, 0, i * BS:(i + 1) * BS]
            want_v += ref["dv"][0, 0, i * BS:(i + 1) * BS]
        hi = min((c + 1) * BS, w.n_k) - c * BS
        check(w, "dk (block)", dk[b, r, c * BS: c * BS + hi], want_k[:hi], f"{name} block {c} ({len(tt)} rows)")
        check(w, "dv (block)", dv[b, r, c * BS: c * BS + hi], want_v[:hi], f"{name} block {c} ({len(tt)} rows)")
