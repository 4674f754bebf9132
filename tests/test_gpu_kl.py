"""GPU parity of the index-branch alignment loss (msa_index_kl) with the fp64 oracle.

The GPU path takes the selection and the main-branch LSE of the GPU forward step (the
selection is bit-exact with the oracle's, checked here again); the oracle computes the
teacher from scratch. Both sides see the same input bits. Tolerance: |kl - ref| <=
KL_ATOL + KL_RTOL * |ref|, and the same for lse_idx (see the derivation in the design
notes: fp32 sums over at most 4096 tokens of terms whose size is bounded by the index
score range, plus the forward LSE's own rounding carried into the teacher's weights).
"""
import numpy as np
import pytest
import torch

from block_sparse_gqa_msa_amd import binding as msa
from block_sparse_gqa_msa_amd.inputs import WORKLOADS, Workload, generate
from gpu_cases import log, run_gpu, sample_rows, to_cpu

pytestmark = pytest.mark.gpu

KL_TOL = {"f32": (2e-5, 2e-5), "bf16": (2e-4, 2e-5)}  # (atol, rtol)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    msa.load_library()


def W(name, dtype="bf16", batch=1, n_q=256, n_k=256, q_start=0, h_q=32, h_kv=4, d_h=128,
      d_idx=64, block_size=64, top_k=8, idx_range=4, qkv_scale=0.5, needles=0, seed=7):
    return Workload(name, dtype, batch, n_q, n_k, q_start, h_q, h_kv, d_h, d_idx, block_size,
                    top_k, idx_range, qkv_scale, needles, seed)


def gpu_kl(w, inp, buf):
    s = msa.shape_of(w)
    kl = torch.full((w.batch, w.h_kv, w.n_q), float("nan"), device="cuda")
    lse_idx = torch.full_like(kl, float("nan"))
    ws = torch.empty(max(1, msa.msa_sparse_attn_workspace_size(s)), dtype=torch.uint8,
                     device="cuda")
    msa.msa_index_kl(s, inp["q"], inp["k"], inp["q_idx"], inp["k_idx"], buf.sel, buf.lse, kl,
                     lse_idx, ws)
    torch.cuda.synchronize()
    return kl, lse_idx


def check(w, kl, lse_idx, ref, label):
    atol, rtol = KL_TOL[w.dtype]
    for name, got in (("kl", kl), ("lse_idx", lse_idx)):
        g = got.cpu().numpy().astype(np.float64)
        want = ref[name]
        assert np.isfinite(g).all(), f"{label}: {name} not finite"
        err = np.abs(g - want)
        bound = atol + rtol * np.abs(want)
        log(f"{label}: {name} max-abs err {err.max():.3e} (ref range {want.min():.3g} .. "
            f"{want.max():.3g})")
        assert (err <= bound).all(), f"{label}: {name} worst {err.max()} at {np.unravel_index(err.argmax(), err.shape)}"


SMALL = [
    WORKLOADS["prefill_512_f32"],
    W("kl_ragged_bf16", batch=2, n_q=1000, n_k=1000, top_k=8, needles=4),
    W("kl_chunk_g4", n_q=300, n_k=1500, q_start=1200, h_q=8, h_kv=2, d_h=64, d_idx=32,
      block_size=32, top_k=5, needles=3),
    W("kl_g1_r8_f32", dtype="f32", n_q=700, n_k=700, h_q=8, h_kv=8, d_h=64, d_idx=64, top_k=3,
      idx_range=3, qkv_scale=1.0),
    W("kl_g16_r1", n_q=520, n_k=520, h_q=16, h_kv=1, d_h=128, d_idx=32, block_size=32, top_k=4),
    W("kl_k64", n_q=4200, n_k=4200, top_k=64, needles=8),
    W("kl_decode", batch=3, n_q=1, n_k=5000, q_start=4999, top_k=16, needles=4),
]


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_kl_small_full_oracle(w):
    import oracle
    log(f"case {w.name}: {w}")
    inp = generate(w, device="cuda")
    buf = run_gpu(w, inp)
    kl, lse_idx = gpu_kl(w, inp, buf)
    cpu = to_cpu(inp)
    orc = oracle.get()
    sel = orc.run(w, cpu, attention=False)["sel"]
    assert np.array_equal(buf.sel.cpu().numpy(), sel), "selections differ"
    ref = orc.kl(w, cpu, sel)
    check(w, kl, lse_idx, ref, w.name)


def test_kl_kv_capacity_stride():
    """Caches allocated longer than the valid length (kv_capacity > n_k): the loss reads K
    and K_idx with the capacity stride; padding past n_k holds values that would change it."""
    import oracle
    for w in (W("kl_cap_prefill", n_q=200, n_k=400, q_start=200, top_k=4),
              W("kl_cap_decode", batch=2, n_q=1, n_k=900, q_start=899, top_k=6)):
        inp = generate(w, device="cuda")
        cap = w.n_k + 136
        big = dict(q=inp["q"], q_idx=inp["q_idx"])
        for key in ("k", "v"):
            x = torch.full((w.batch, w.h_kv, cap, w.d_h), 2.0, dtype=inp[key].dtype, device="cuda")
            x[:, :, : w.n_k] = inp[key]
            big[key] = x
        x = torch.full((w.batch, cap, w.d_idx), 3.0, dtype=inp["k_idx"].dtype, device="cuda")
        x[:, : w.n_k] = inp["k_idx"]
        big["k_idx"] = x
        s = msa.shape_of(w, kv_capacity=cap)
        buf = msa.Buffers(s)
        msa.msa_step(buf, big)
        kl = torch.empty((w.batch, w.h_kv, w.n_q), device="cuda")
        lse_idx = torch.empty_like(kl)
        msa.msa_index_kl(s, big["q"], big["k"], big["q_idx"], big["k_idx"], buf.sel, buf.lse, kl,
                         lse_idx, buf.ws_attn)
        torch.cuda.synchronize()
        cpu = to_cpu(inp)
        sel = oracle.get().run(w, cpu, attention=False)["sel"]
        assert np.array_equal(buf.sel.cpu().numpy(), sel)
        check(w, kl, lse_idx, oracle.get().kl(w, cpu, sel), w.name)


@pytest.mark.parametrize("name", ["prefill_8k", "prefill_128k", "chunk_1m"])
def test_kl_workload_sampled_rows(name):
    """The prefill workloads at full size: every row's loss is finite and >= -atol, and
    sampled rows match the oracle."""
    import oracle
    w = WORKLOADS[name]
    log(f"case {name}: {w}")
    inp = generate(w, device="cuda")
    buf = run_gpu(w, inp)
    kl, lse_idx = gpu_kl(w, inp, buf)
    atol, _ = KL_TOL[w.dtype]
    assert torch.isfinite(kl).all() and kl.min().item() >= -atol
    rows = sample_rows(w, n_random=64 if name == "prefill_8k" else 24)
    cpu = to_cpu(inp)
    orc = oracle.get()
    ridx = torch.as_tensor(rows, device="cuda")
    sel = buf.sel[:, :, ridx].cpu().numpy()
    sel_ref = orc.run(w, cpu, rows=rows, attention=False)["sel"]
    assert np.array_equal(sel, sel_ref), "selections differ"
    ref = orc.kl(w, cpu, sel_ref, rows=rows)
    check(w, kl[:, :, ridx], lse_idx[:, :, ridx], ref, f"{name} ({len(rows)} rows)")
