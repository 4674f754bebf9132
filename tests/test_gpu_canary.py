"""Output canaries: every output of the step is a window of a larger buffer whose guard
regions (before and after) and the window itself are pre-filled with sentinels. After the
call the guards must be untouched (no write outside an output) and the window fully
overwritten (no sentinel left in sel, o, lse, block scores, kl, dq / dk / dv): each entry
point writes exactly its outputs, for prefill, chunked prefill, decode (both decode
paths), the loss and the backward, on ragged shapes."""
import numpy as np
import pytest
import torch

from gpu_cases import log
from block_sparse_gqa_msa_amd import binding as msa
from block_sparse_gqa_msa_amd.inputs import Workload, generate, generate_dout

pytestmark = pytest.mark.gpu

GUARD = 4096  # elements on each side


def W(name, dtype="bf16", batch=1, n_q=256, n_k=256, q_start=0, h_q=32, h_kv=4, d_h=128,
      d_idx=64, block_size=64, top_k=8, idx_range=4, qkv_scale=0.5, needles=0, seed=11):
    return Workload(name, dtype, batch, n_q, n_k, q_start, h_q, h_kv, d_h, d_idx, block_size,
                    top_k, idx_range, qkv_scale, needles, seed)
SENT_I = 0x7EADBEEF


def guarded(shape, dtype):
    """A window of `shape` inside a buffer with GUARD elements of sentinel on each side; the
    window holds the sentinel too."""
    n = int(np.prod(shape))
    buf = torch.empty(n + 2 * GUARD, dtype=dtype, device="cuda")
    if dtype.is_floating_point:
        buf.fill_(float("nan"))
    else:
        buf.fill_(SENT_I)
    return buf, buf[GUARD:GUARD + n].view(shape)


def check(name, buf, win):
    lo, hi = buf[:GUARD], buf[-GUARD:]
    if buf.dtype.is_floating_point:
        assert torch.isnan(lo.float()).all() and torch.isnan(hi.float()).all(), f"{name}: write outside the output"
        assert not torch.isnan(win.float()).any(), f"{name}: output not fully written"
    else:
        assert (lo == SENT_I).all() and (hi == SENT_I).all(), f"{name}: write outside the output"
        assert not (win == SENT_I).any(), f"{name}: output not fully written"


CASES = [
    W("canary_prefill", batch=2, n_q=700, n_k=700, top_k=6, needles=3),
    W("canary_chunk", n_q=130, n_k=1000, q_start=870, h_q=16, h_kv=2, d_h=64, d_idx=32,
      block_size=32, top_k=5, needles=2),
    W("canary_f32", dtype="f32", n_q=300, n_k=300, h_q=8, h_kv=4, d_h=64, d_idx=32,
      block_size=32, top_k=4, idx_range=3, qkv_scale=1.0),
]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_prefill_outputs_exactly_written(w):
    log(f"case {w.name}: {w}")
    inp = generate(w, device="cuda")
    s = msa.shape_of(w)
    et = inp["q"].dtype
    B, R, H, n, k = w.batch, w.h_kv, w.h_q, w.n_q, w.top_k
    nb = -(-w.n_k // w.block_size)
    sel_b, sel = guarded((B, R, n, k), torch.int32)
    bs_b, bs = guarded((B, R, n, nb), torch.float32)
    o_b, o = guarded((B, H, n, w.d_h), et)
    lse_b, lse = guarded((B, H, n), torch.float32)
    ws_i = torch.empty(max(1, msa.msa_index_topk_workspace_size(s)), dtype=torch.uint8, device="cuda")
    ws_a = torch.empty(max(1, msa.msa_sparse_attn_workspace_size(s)), dtype=torch.uint8, device="cuda")
    msa.msa_index_topk(s, inp["q_idx"], inp["k_idx"], sel, bs, ws_i)
    msa.msa_sparse_attn_prefill(s, inp["q"], inp["k"], inp["v"], sel, o, lse, ws_a)
    torch.cuda.synchronize()
    # sel's padding is -1, never the sentinel; block scores past the local block are -inf
    for name, b_, w_ in (("sel", sel_b, sel), ("block_scores", bs_b, bs), ("o", o_b, o), ("lse", lse_b, lse)):
        check(f"{w.name} {name}", b_, w_)
    kl_b, kl = guarded((B, R, n), torch.float32)
    li_b, li = guarded((B, R, n), torch.float32)
    msa.msa_index_kl(s, inp["q"], inp["k"], inp["q_idx"], inp["k_idx"], sel, lse, kl, li, ws_a)
    torch.cuda.synchronize()
    check(f"{w.name} kl", kl_b, kl)
    check(f"{w.name} lse_idx", li_b, li)
    dout = generate_dout(w, device="cuda")
    grads = [guarded(tuple(inp[x].shape), et) for x in ("q", "k", "v")]
    ws_b = torch.empty(msa.msa_sparse_attn_backward_workspace_size(s), dtype=torch.uint8, device="cuda")
    msa.msa_sparse_attn_backward(s, inp["q"], inp["k"], inp["v"], sel, o, lse, dout,
                                 *[g[1] for g in grads], ws_b)
    torch.cuda.synchronize()
    for name, (b_, w_) in zip(("dq", "dk", "dv"), grads):
        check(f"{w.name} {name}", b_, w_)
    log(f"{w.name}: every output written exactly")


@pytest.mark.parametrize("one_call", [False, True], ids=["two_calls", "decode_step"])
def test_decode_outputs_exactly_written(one_call):
    w = W("canary_decode", batch=3, n_q=1, n_k=4100, q_start=4099, top_k=12, needles=3)
    log(f"case {w.name} one_call={one_call}: {w}")
    inp = generate(w, device="cuda")
    s = msa.shape_of(w)
    et = inp["q"].dtype
    sel_b, sel = guarded((w.batch, w.h_kv, 1, w.top_k), torch.int32)
    o_b, o = guarded((w.batch, w.h_q, 1, w.d_h), et)
    lse_b, lse = guarded((w.batch, w.h_q, 1), torch.float32)
    if one_call:
        ws = torch.empty(max(1, msa.msa_decode_step_workspace_size(s)), dtype=torch.uint8, device="cuda")
        msa.msa_decode_step(s, inp["q"], inp["k"], inp["v"], inp["q_idx"], inp["k_idx"], sel, o, lse, ws)
    else:
        ws_i = torch.empty(max(1, msa.msa_index_topk_workspace_size(s)), dtype=torch.uint8, device="cuda")
        ws_a = torch.empty(max(1, msa.msa_sparse_attn_workspace_size(s)), dtype=torch.uint8, device="cuda")
        msa.msa_index_topk(s, inp["q_idx"], inp["k_idx"], sel, None, ws_i)
        msa.msa_sparse_attn_decode(s, inp["q"], inp["k"], inp["v"], sel, o, lse, ws_a)
    torch.cuda.synchronize()
    for name, b_, w_ in (("sel", sel_b, sel), ("o", o_b, o), ("lse", lse_b, lse)):
        check(f"{w.name} {name}", b_, w_)
