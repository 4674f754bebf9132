"""The library's calls captured in a HIP graph (through torch.cuda.CUDAGraph) and replayed.

Each entry point enqueues only kernels on the caller's stream (no memory allocation, no
memset node, no synchronisation), so a captured step can be replayed: each replay below
follows new inputs copied into the captured buffers, eager work and a synchronisation,
and must give the bits the same calls give eagerly on those inputs.
"""
import pytest
import torch

from block_sparse_gqa_msa_amd import binding as msa
from block_sparse_gqa_msa_amd.inputs import Workload, generate
from gpu_cases import log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    msa.load_library()  # raises if libmsa.so is missing: no fallback


def W(name, batch, n_q, n_k, top_k, seed, block_size=64, needles=4):
    return Workload(name, "bf16", batch, n_q, n_k, n_k - n_q, 32, 4, 128, 64, block_size, top_k,
                    4, 0.5, needles, seed)


def _outputs(w):
    return dict(sel=torch.empty((w.batch, w.h_kv, w.n_q, w.top_k), dtype=torch.int32, device="cuda"),
                o=torch.empty((w.batch, w.h_q, w.n_q, w.d_h), dtype=torch.bfloat16, device="cuda"),
                lse=torch.empty((w.batch, w.h_q, w.n_q), dtype=torch.float32, device="cuda"))


def _replay_matches_eager(w, step, workspaces):
    """Capture step(inputs, outputs) once, then for three new input sets: copy them into
    the captured buffers, replay, and compare with the eager call on the same inputs."""
    static_in = generate(w, device="cuda")
    static_out = _outputs(w)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up off the capture
        step(static_in, static_out, workspaces)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(static_in, static_out, workspaces)
    torch.cuda.synchronize()
    eager_out = _outputs(w)
    for rnd in range(3):
        fresh = generate(w, device="cuda", seed=w.seed + 100 + rnd)
        for key in ("q", "k", "v", "q_idx", "k_idx"):
            static_in[key].copy_(fresh[key])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        step(fresh, eager_out, workspaces)  # eager work between the replays
        torch.cuda.synchronize()
        for key in ("sel", "o", "lse"):
            a, b = static_out[key], eager_out[key]
            same = torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b)
            assert same, f"{w.name} replay {rnd}: {key} differs from the eager call"
        log(f"{w.name}: replay {rnd} equals the eager call bit for bit")


def test_graph_decode_step():
    w = W("graph_decode", batch=3, n_q=1, n_k=40000, top_k=32, seed=31)
    s = msa.shape_of(w)
    ws = torch.empty(msa.msa_decode_step_workspace_size(s), dtype=torch.uint8, device="cuda")

    def step(inp, out, wsp):
        msa.msa_decode_step(s, inp["q"], inp["k"], inp["v"], inp["q_idx"], inp["k_idx"],
                            out["sel"], out["o"], out["lse"], wsp)

    _replay_matches_eager(w, step, ws)


def test_graph_decode_two_calls():
    w = W("graph_decode_two", batch=2, n_q=1, n_k=30000, top_k=16, seed=32)
    s = msa.shape_of(w)
    wi = torch.empty(msa.msa_index_topk_workspace_size(s), dtype=torch.uint8, device="cuda")
    wa = torch.empty(msa.msa_sparse_attn_workspace_size(s), dtype=torch.uint8, device="cuda")

    def step(inp, out, wsp):
        msa.msa_index_topk(s, inp["q_idx"], inp["k_idx"], out["sel"], None, wsp[0])
        msa.msa_sparse_attn_decode(s, inp["q"], inp["k"], inp["v"], out["sel"], out["o"],
                                   out["lse"], wsp[1])

    _replay_matches_eager(w, step, (wi, wa))


def test_graph_prefill_step():
    w = W("graph_prefill", batch=1, n_q=3000, n_k=3000, top_k=16, seed=33)
    s = msa.shape_of(w)
    wi = torch.empty(msa.msa_index_topk_workspace_size(s), dtype=torch.uint8, device="cuda")
    wa = torch.empty(msa.msa_sparse_attn_workspace_size(s), dtype=torch.uint8, device="cuda")

    def step(inp, out, wsp):
        msa.msa_index_topk(s, inp["q_idx"], inp["k_idx"], out["sel"], None, wsp[0])
        msa.msa_sparse_attn_prefill(s, inp["q"], inp["k"], inp["v"], out["sel"], out["o"],
                                    out["lse"], wsp[1])

    _replay_matches_eager(w, step, (wi, wa))
