"""msa_decode_step_noalloc (the decode step on the library's own per-GPU scratch array)
against msa_decode_step with a caller workspace: same kernels, so selections, outputs and
LSE must be identical, on consecutive calls whose second input is smaller (the scratch keeps
the first call's contents) and on the fallback path of two calls (top_k 1)."""
import pytest
import torch

from gpu_cases import log
from block_sparse_gqa_msa_amd import binding as msa
from block_sparse_gqa_msa_amd.inputs import WORKLOADS, generate

pytestmark = pytest.mark.gpu

BASE = WORKLOADS["decode_1m_b4"]


def decode_case(name, batch, n_k, top_k, dtype="bf16", d_h=128, seed=7):
    return BASE.replace(name=name, batch=batch, n_k=n_k, q_start=n_k - 1, top_k=top_k,
                        dtype=dtype, d_h=d_h, needles=4, seed=seed)


def both_ways(w):
    inp = generate(w, device="cuda")
    s = msa.shape_of(w)
    out = {}
    for how in ("workspace", "noalloc"):
        sel = torch.full((w.batch, w.h_kv, 1, w.top_k), -7, dtype=torch.int32, device="cuda")
        o = torch.full((w.batch, w.h_q, 1, w.d_h), 7.0, dtype=inp["q"].dtype, device="cuda")
        lse = torch.full((w.batch, w.h_q, 1), 7.0, dtype=torch.float32, device="cuda")
        if how == "workspace":
            ws = torch.empty(max(1, msa.msa_decode_step_workspace_size(s)), dtype=torch.uint8,
                             device="cuda")
            msa.msa_decode_step(s, inp["q"], inp["k"], inp["v"], inp["q_idx"], inp["k_idx"], sel,
                                o, lse, ws)
        else:
            msa.msa_decode_step_noalloc(s, inp["q"], inp["k"], inp["v"], inp["q_idx"],
                                        inp["k_idx"], sel, o, lse)
        torch.cuda.synchronize()
        out[how] = (sel, o, lse)
    (s1, o1, l1), (s2, o2, l2) = out["workspace"], out["noalloc"]
    assert torch.equal(s1, s2), f"{w.name}: selections differ"
    assert torch.equal(o1, o2), f"{w.name}: o differs, max {(o1.float() - o2.float()).abs().max()}"
    assert torch.equal(l1, l2), f"{w.name}: lse differs"
    log(f"{w.name}: noalloc step equals the workspace step (sel, o, lse bit for bit)")


def test_noalloc_step_equals_workspace_step_twice():
    log("noalloc: batch 3 x 5000 tokens, top_k 16, then batch 1 x 2000 tokens, top_k 8")
    both_ways(decode_case("noalloc_a", 3, 5000, 16))
    both_ways(decode_case("noalloc_b", 1, 2000, 8, seed=8))


def test_noalloc_fallback_and_fp32():
    log("noalloc: top_k 1 (two-call fallback), then fp32 d_h 64")
    both_ways(decode_case("noalloc_k1", 2, 3000, 1))
    both_ways(decode_case("noalloc_f32", 2, 3000, 8, dtype="f32", d_h=64))


def test_noalloc_full_size_decode():
    w = WORKLOADS["decode_256k_b32"]
    need = msa.msa_decode_step_workspace_size(msa.shape_of(w))
    assert need <= msa.DECODE_STEP_SCRATCH_BYTES
    log(f"noalloc: {w.name} ({need} of {msa.DECODE_STEP_SCRATCH_BYTES} scratch bytes), then a "
        f"smaller step")
    both_ways(w)
    both_ways(decode_case("noalloc_small", 2, 4096, 32, seed=9))
