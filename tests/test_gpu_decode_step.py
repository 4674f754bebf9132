"""GPU parity of msa_decode_step, the whole decode step in two launches (index kernel, then
one kernel for the final top-k, the attention over the selected blocks and the log-sum-exp
merge), against the fp64 oracle and against the two calls it stands for.

Selections must match the oracle bit for bit; O and LSE within the decode tolerances
(1e-5 for fp32, 2e-2 max-abs / 1e-2 mean-abs and 1e-3 LSE for bf16). The workspace starts
filled with 0xff bytes: the call clears its own arrival counters.
"""
import numpy as np
import pytest
import torch

from block_sparse_gqa_msa_amd import binding as msa
from block_sparse_gqa_msa_amd.inputs import WORKLOADS, Workload, generate
from gpu_cases import check_selection_invariants, compare, log, oracle_run, run_gpu, to_cpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    msa.load_library()  # raises if libmsa.so is missing: no fallback


def W(name, dtype="bf16", batch=1, n_k=256, h_q=32, h_kv=4, d_h=128, d_idx=64, block_size=64,
      top_k=8, idx_range=4, qkv_scale=0.5, needles=0, seed=11):
    return Workload(name, dtype, batch, 1, n_k, n_k - 1, h_q, h_kv, d_h, d_idx, block_size, top_k,
                    idx_range, qkv_scale, needles, seed)


class Step:
    """Outputs of one msa_decode_step call (the attribute names compare() reads)."""

    def __init__(self, w: Workload, ws=None):
        s = msa.shape_of(w)
        dt = torch.float32 if w.dtype == "f32" else torch.bfloat16
        self.sel = torch.full((w.batch, w.h_kv, 1, w.top_k), -7, dtype=torch.int32, device="cuda")
        self.o = torch.full((w.batch, w.h_q, 1, w.d_h), float("nan"), dtype=dt, device="cuda")
        self.lse = torch.full((w.batch, w.h_q, 1), float("nan"), device="cuda")
        need = msa.msa_decode_step_workspace_size(s)
        if ws is None:
            ws = torch.full((max(1, need),), 0xff, dtype=torch.uint8, device="cuda")
        assert ws.numel() >= need
        self.ws = ws

    def run(self, w: Workload, inp):
        msa.msa_decode_step(msa.shape_of(w), inp["q"], inp["k"], inp["v"], inp["q_idx"],
                            inp["k_idx"], self.sel, self.o, self.lse, self.ws)
        torch.cuda.synchronize()
        return self


CASES = [
    W("step_ragged_bf16", batch=3, n_k=5000, top_k=16, needles=4),
    W("step_f32_g2", dtype="f32", batch=2, n_k=3001, h_q=8, h_kv=4, d_h=64, d_idx=32,
      block_size=32, top_k=4, idx_range=3, qkv_scale=1.0),
    W("step_f32_d128_bs64", dtype="f32", batch=2, n_k=7000, h_q=8, h_kv=2, d_h=128, top_k=9,
      idx_range=3, qkv_scale=1.0),
    W("step_few_blocks", batch=2, n_k=200, top_k=8),          # every block selected
    W("step_k1", batch=2, n_k=3000, top_k=1),                  # falls back to the two calls
    W("step_k2", batch=2, n_k=3000, top_k=2),                  # one block per sub-range
    W("step_ties", batch=2, n_k=70000, d_idx=32, top_k=32, idx_range=0),  # all scores equal
    W("step_g1_r8", batch=2, n_k=9000, h_q=8, h_kv=8, d_h=64, top_k=12, needles=4),
    W("step_g16_r1", batch=2, n_k=4100, h_q=16, h_kv=1, d_h=128, top_k=9, needles=2),
    W("step_k48", batch=2, n_k=40000, top_k=48, needles=6),
    W("step_k64_bs32", batch=1, n_k=30000, h_q=16, h_kv=2, d_h=64, d_idx=32, block_size=32,
      top_k=64, needles=6),
    W("step_many_ranges", batch=2, n_k=140000, block_size=32, top_k=32, needles=8),  # 18 ranges
]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_decode_step_full_oracle(w):
    log(f"case {w.name}: {w}")
    inp = generate(w, device="cuda")
    ref = oracle_run(w, to_cpu(inp))
    got = Step(w).run(w, inp)
    check_selection_invariants(w, got.sel)
    compare(w, got, ref, label=f"{w.name} (decode step)")
    two = run_gpu(w, inp)  # msa_index_topk + msa_sparse_attn_decode
    assert torch.equal(got.sel, two.sel), f"{w.name}: selection differs from the two calls"


def test_decode_step_reuses_workspace():
    """Three calls on one workspace (counters left by the previous call), the last one with a
    smaller batch and a different cache length: each equals its own fresh two-call result."""
    big = W("reuse_big", batch=4, n_k=20000, top_k=32, needles=4, seed=21)
    small = W("reuse_small", batch=2, n_k=9000, top_k=32, needles=4, seed=22)
    ws = torch.full((msa.msa_decode_step_workspace_size(msa.shape_of(big)),), 0xff,
                    dtype=torch.uint8, device="cuda")
    for w in (big, big, small):
        inp = generate(w, device="cuda")
        got = Step(w, ws).run(w, inp)
        two = run_gpu(w, inp)
        assert torch.equal(got.sel, two.sel), w.name
        err = (got.o.float() - two.o.float()).abs().max().item()
        lerr = (got.lse - two.lse).abs().max().item()
        log(f"{w.name}: sel equal, O max-abs vs two calls {err:.2e}, LSE {lerr:.2e}")
        assert err <= 2e-3 and lerr <= 1e-4, w.name


@pytest.mark.parametrize("name,seqs", [("decode_256k_b32", [0, 17, 31]),
                                       ("decode_1m_b4", [1, 2])])
def test_decode_step_workload_full_size(name, seqs):
    """The two decode workloads at full size: every selection checked for its invariants and
    equal to the two calls' selection; sampled sequences against the oracle."""
    w = WORKLOADS[name]
    log(f"case {name}: {w}")
    inp = generate(w, device="cuda")
    got = Step(w).run(w, inp)
    check_selection_invariants(w, got.sel)
    two = run_gpu(w, inp)
    assert torch.equal(got.sel, two.sel), f"{name}: selection differs from the two calls"
    import oracle
    orc = oracle.get()
    outs = []
    for b in seqs:
        wb = w.replace(batch=1)
        outs.append(orc.run(wb, {k: inp[k][b:b + 1].cpu() for k in ("q", "k", "v", "q_idx", "k_idx")}))
        log(f"  oracle sequence {b} done")
    ref = {k: np.concatenate([o[k] for o in outs], axis=0) for k in ("sel", "o", "lse")}
    compare(w, got, ref, seqs=torch.as_tensor(seqs, device="cuda"), label=f"{name} (decode step)")


def test_decode_step_kv_capacity_stride():
    """Caches allocated longer than the valid length (kv_capacity > n_k), the slack filled
    with values that would change the result if read."""
    w = W("step_capacity", batch=2, n_k=9000, top_k=16, needles=3, seed=23)
    inp = generate(w, device="cuda")
    cap = w.n_k + 200
    big = {"q": inp["q"], "q_idx": inp["q_idx"]}
    for key in ("k", "v"):
        x = torch.full((w.batch, w.h_kv, cap, w.d_h), 9.0, dtype=inp[key].dtype, device="cuda")
        x[:, :, : w.n_k] = inp[key]
        big[key] = x
    x = torch.full((w.batch, cap, w.d_idx), 4.0, dtype=inp["k_idx"].dtype, device="cuda")
    x[:, : w.n_k] = inp["k_idx"]
    big["k_idx"] = x
    s = msa.shape_of(w, kv_capacity=cap)
    got = Step(w)
    got.ws = torch.full((msa.msa_decode_step_workspace_size(s),), 0xff, dtype=torch.uint8,
                        device="cuda")
    msa.msa_decode_step(s, big["q"], big["k"], big["v"], big["q_idx"], big["k_idx"], got.sel,
                        got.o, got.lse, got.ws)
    torch.cuda.synchronize()
    ref = oracle_run(w, to_cpu(inp))
    compare(w, got, ref, label=w.name)
