"""GPU parity: the HIP path through the C ABI against the fp64 oracle on the same input bits.

Block selections (and block scores, when requested) must match bit for bit: index
inputs are integers, so every fp32 score is exact. O must be within 1e-5 max-abs
(fp32) or 2e-2 max-abs and 1e-2 mean-abs (bf16); LSE within 1e-5 (fp32) / 1e-3 (bf16).
Small shapes are compared in full; the six workloads run at full size with sampled
rows (sampled sequences for decode) checked against the oracle and selection
invariants checked on every row.
"""
import numpy as np
import pytest
import torch

from block_sparse_gqa_msa_amd import binding as msa
from block_sparse_gqa_msa_amd.inputs import WORKLOADS, Workload, generate
from gpu_cases import (check_selection_invariants, compare, log, oracle_run, run_gpu,
                       sample_rows, to_cpu)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    msa.load_library()  # raises if libmsa.so is missing: no fallback


def W(name, dtype="bf16", batch=1, n_q=256, n_k=256, q_start=0, h_q=32, h_kv=4, d_h=128,
      d_idx=64, block_size=64, top_k=8, idx_range=4, qkv_scale=0.5, needles=0, seed=7):
    return Workload(name, dtype, batch, n_q, n_k, q_start, h_q, h_kv, d_h, d_idx, block_size,
                    top_k, idx_range, qkv_scale, needles, seed)


SMALL = [
    WORKLOADS["prefill_512_f32"],
    W("ragged_tail_bf16", batch=2, n_q=1000, n_k=1000, top_k=8, needles=4),
    W("chunk_unaligned_g4", n_q=300, n_k=1500, q_start=1200, h_q=8, h_kv=2, d_h=64, d_idx=32,
      block_size=32, top_k=5, needles=3),
    W("g1_r8_f32", dtype="f32", n_q=700, n_k=700, h_q=8, h_kv=8, d_h=64, d_idx=64, top_k=3,
      idx_range=3, qkv_scale=1.0),
    W("g16_r1", n_q=520, n_k=520, h_q=16, h_kv=1, d_h=128, d_idx=32, block_size=32, top_k=4),
    W("g2_r16_f32", dtype="f32", n_q=300, n_k=300, h_q=32, h_kv=16, d_h=64, d_idx=64,
      block_size=32, top_k=6, idx_range=3, qkv_scale=1.0),
    W("k64_near_dense", n_q=4200, n_k=4200, top_k=64, needles=8),
    W("k1_local_only", n_q=777, n_k=777, top_k=1, block_size=32),
    W("f32_d128_bs64", dtype="f32", n_q=640, n_k=640, h_q=8, h_kv=2, d_h=128, d_idx=64,
      top_k=4, idx_range=3, qkv_scale=1.0),
    W("prefill_two_level_topk", n_q=64, n_k=70064, q_start=70000, block_size=32, d_idx=32,
      top_k=32, needles=16),
    W("batch3_unaligned_chunk", batch=3, n_q=333, n_k=2000, q_start=1667, h_q=16, h_kv=2,
      d_h=128, d_idx=64, block_size=64, top_k=7, needles=5),
    W("bf16_d64_bs64_g8", n_q=1500, n_k=1500, h_q=32, h_kv=4, d_h=64, d_idx=32, block_size=64,
      top_k=10, needles=4),
    # k = 48 over ~257 blocks: about 80 candidates reach the first bound, more than one
    # per lane, so the exact m-th comes from the second bitwise search, not the ranking
    W("k48_mid_candidates", n_q=64, n_k=16448, q_start=16384, h_q=8, h_kv=2, d_h=64,
      d_idx=32, block_size=64, top_k=48, needles=8),
    # 18751 key blocks: the list build's LDS histograms take 73 KiB per workgroup (more
    # than the 64 KiB of the 1M-context workloads)
    W("prefill_hist_73k_lds", n_q=48, n_k=600032, q_start=599984, h_q=8, h_kv=2, d_h=64,
      d_idx=32, block_size=32, top_k=12, needles=8),
    # more than 32768 key blocks: the list build falls back to per-entry counters
    W("prefill_many_blocks", n_q=40, n_k=(1 << 20) + 96, q_start=(1 << 20) + 56, h_q=8,
      h_kv=2, d_h=64, d_idx=32, block_size=32, top_k=16, needles=8),
]


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_small_full_oracle(w):
    log(f"case {w.name}: {w}")
    inp = generate(w, device="cuda")
    buf = run_gpu(w, inp, block_scores=True)
    check_selection_invariants(w, buf.sel)
    ref = oracle_run(w, to_cpu(inp), block_scores=True)
    bs_gpu = buf.block_scores.cpu().numpy().astype(np.float64)
    assert np.array_equal(bs_gpu, ref["block_scores"]), "block scores differ"
    compare(w, buf, ref, label=w.name)


def test_heavy_ties_use_exact_fallback():
    """All index keys zero: every block score is 0, so the tie-break alone decides
    (lowest blocks first) and the wide-tie path of the top-k kernel runs."""
    w = W("all_ties", n_q=3000, n_k=3000, block_size=32, d_idx=32, top_k=16)
    inp = generate(w, device="cuda")
    inp["k_idx"].zero_()
    buf = run_gpu(w, inp)
    ref = oracle_run(w, to_cpu(inp))
    compare(w, buf, ref, label=w.name)


def test_few_distinct_scores():
    """Index values in {0, 1}: many ties at the threshold but a short candidate list."""
    w = W("few_values", n_q=2500, n_k=2500, block_size=32, d_idx=32, top_k=12, idx_range=1)
    inp = generate(w, device="cuda")
    inp["q_idx"].abs_()
    inp["k_idx"].abs_()
    buf = run_gpu(w, inp)
    ref = oracle_run(w, to_cpu(inp))
    compare(w, buf, ref, label=w.name)


@pytest.mark.parametrize("q_start", [20000, 80000], ids=["one_chunk", "two_chunks"])
def test_signed_zero_scores_tie(q_start):
    """Block scores of -0 and +0 are equal scores: the ties at zero go to the lowest blocks,
    whatever the signs (caller scores through msa_topk_from_block_scores; 32-token blocks,
    about 625 or 2500 candidates). Expected by construction: five blocks with distinct
    positive scores, then the lowest-index zero blocks, then the local block."""
    w = W("signed_zeros", n_q=48, n_k=q_start + 48, q_start=q_start, h_kv=2, h_q=8,
          block_size=32, top_k=16)
    s = msa.shape_of(w)
    nb = -(-w.n_k // w.block_size)
    rng = np.random.default_rng(5)
    scores = np.full((1, w.h_kv, w.n_q, nb), -1.0, dtype=np.float32)
    expect = np.full((1, w.h_kv, w.n_q, w.top_k), -1, dtype=np.int32)
    for r in range(w.h_kv):
        for t in range(w.n_q):
            local = (q_start + t) // w.block_size
            picks = rng.choice(local, size=45, replace=False)
            pos, zer = picks[:5], picks[5:]
            scores[0, r, t, pos] = rng.uniform(1.0, 2.0, size=5).astype(np.float32)
            scores[0, r, t, zer] = np.where(rng.random(40) < 0.5, -0.0, 0.0).astype(np.float32)
            chosen = np.concatenate([pos, np.sort(zer)[:w.top_k - 1 - 5], [local]])
            expect[0, r, t] = np.sort(chosen)
    assert np.signbit(scores[scores == 0]).any() and (~np.signbit(scores[scores == 0])).any()
    sc = torch.from_numpy(scores).cuda()
    sel = torch.full((1, w.h_kv, w.n_q, w.top_k), -7, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(1, msa.msa_topk_workspace_size(s)), dtype=torch.uint8, device="cuda")
    msa.msa_topk_from_block_scores(s, sc, sel, ws)
    torch.cuda.synchronize()
    got = sel.cpu().numpy()
    bad = int((got != expect).any(-1).sum())
    assert bad == 0, f"{bad} (row, group) selections differ from the expected ties at zero"


DECODE_SMALL = [
    W("decode_ragged_bf16", batch=3, n_q=1, n_k=5000, q_start=4999, top_k=16, needles=4),
    W("decode_f32_g2", dtype="f32", batch=2, n_q=1, n_k=3001, q_start=3000, h_q=8, h_kv=4,
      d_h=64, d_idx=32, block_size=32, top_k=4, idx_range=3, qkv_scale=1.0),
    W("decode_two_level_topk", batch=2, n_q=1, n_k=140000, q_start=139999, block_size=32,
      top_k=32, needles=8),
    W("decode_few_blocks", batch=2, n_q=1, n_k=200, q_start=199, top_k=8),
    W("decode_k1", batch=2, n_q=1, n_k=3000, q_start=2999, top_k=1),
    W("decode_ties", batch=2, n_q=1, n_k=70000, q_start=69999, d_idx=32, top_k=32,
      idx_range=0),  # all index scores equal: lowest blocks win every tie
    W("decode_g1_r8", batch=2, n_q=1, n_k=9000, q_start=8999, h_q=8, h_kv=8, d_h=64,
      top_k=12, needles=4),
    W("decode_g16_r1_f32", dtype="f32", batch=2, n_q=1, n_k=4100, q_start=4099, h_q=16, h_kv=1,
      d_h=128, d_idx=64, block_size=64, top_k=9, idx_range=3, qkv_scale=1.0),
    W("decode_k48", batch=2, n_q=1, n_k=40000, q_start=39999, block_size=64, top_k=48,
      needles=6),  # more candidates than lanes at the first bound: second bitwise search
]


@pytest.mark.parametrize("w", DECODE_SMALL, ids=lambda w: w.name)
def test_decode_full_oracle(w):
    """Both decode selection paths: with block scores requested (index kernel, then top-k
    passes over the scores) and without (selection fused into the index kernel)."""
    log(f"case {w.name}: {w}")
    inp = generate(w, device="cuda")
    ref = oracle_run(w, to_cpu(inp), block_scores=True)
    for want_scores in (True, False):
        buf = run_gpu(w, inp, block_scores=want_scores)
        check_selection_invariants(w, buf.sel)
        if want_scores:
            assert np.array_equal(buf.block_scores.cpu().numpy().astype(np.float64),
                                  ref["block_scores"])
        compare(w, buf, ref, label=f"{w.name} (block scores {want_scores})")


def test_kv_capacity_stride():
    """Caches allocated longer than the valid length (kv_capacity > n_k), prefill and decode."""
    for w in (W("cap_prefill", n_q=200, n_k=400, q_start=200, top_k=4),
              W("cap_decode", batch=2, n_q=1, n_k=900, q_start=899, top_k=6)):
        inp = generate(w, device="cuda")
        cap = w.n_k + 136
        big = {}
        for key in ("k", "v"):
            x = torch.zeros(w.batch, w.h_kv, cap, w.d_h, dtype=inp[key].dtype, device="cuda")
            x[:, :, : w.n_k] = inp[key]
            big[key] = x
        x = torch.full((w.batch, cap, w.d_idx), 3.0, dtype=inp["k_idx"].dtype, device="cuda")
        x[:, : w.n_k] = inp["k_idx"]
        big["k_idx"] = x
        big["q"], big["q_idx"] = inp["q"], inp["q_idx"]
        buf = run_gpu(w, big, kv_capacity=cap)
        ref = oracle_run(w, to_cpu(inp))
        compare(w, buf, ref, label=w.name)


def test_decode_equals_prefill_last_row():
    """The split decode path and the prefill path agree on the same row."""
    w = W("consistency", batch=2, n_q=1, n_k=4096 + 77, q_start=4096 + 76, top_k=16, needles=4)
    inp = generate(w, device="cuda")
    dec = run_gpu(w, inp)
    s = msa.shape_of(w)
    buf = msa.Buffers(s)
    msa.msa_index_topk(s, inp["q_idx"], inp["k_idx"], buf.sel, None, buf.ws_index)
    msa.msa_sparse_attn_prefill(s, inp["q"], inp["k"], inp["v"], buf.sel, buf.o, buf.lse,
                                buf.ws_attn)
    torch.cuda.synchronize()
    assert torch.equal(dec.sel, buf.sel)
    assert (dec.o.float() - buf.o.float()).abs().max().item() <= 1e-2
    assert (dec.lse - buf.lse).abs().max().item() <= 1e-4


def test_chunked_equals_full_rows():
    """A chunk at q_start > 0 gives the same selections as the matching rows of a full prefill."""
    w = W("full", n_q=2000, n_k=2000, top_k=8, needles=6)
    inp = generate(w, device="cuda")
    full = run_gpu(w, inp)
    start = 1333
    wc = w.replace(name="chunk", n_q=w.n_q - start, q_start=start)
    ic = dict(inp)
    ic["q"] = inp["q"][:, :, start:].contiguous()
    ic["q_idx"] = inp["q_idx"][:, :, start:].contiguous()
    part = run_gpu(wc, ic)
    assert torch.equal(part.sel, full.sel[:, :, start:])
    assert torch.equal(part.o, full.o[:, :, start:])


# ---------------------------------------------------------------- full-size workloads

@pytest.mark.parametrize("name", ["prefill_8k", "prefill_128k", "chunk_1m"])
def test_prefill_workload_full_size(name):
    w = WORKLOADS[name]
    log(f"case {name}: {w}")
    inp = generate(w, device="cuda")
    buf = run_gpu(w, inp)
    check_selection_invariants(w, buf.sel)
    rows = sample_rows(w, n_random=64 if w.n_q > 10000 else 128)
    ref = oracle_run(w, to_cpu(inp), rows=rows)
    compare(w, buf, ref, rows=rows, label=name)
    if name == "prefill_8k":  # every row's selection (index branch only)
        import oracle
        full = oracle.get().run(w, to_cpu(inp, ("q_idx", "k_idx")), attention=False)
        assert np.array_equal(buf.sel.cpu().numpy(), full["sel"]), "selections differ"


@pytest.mark.parametrize("shape", [
    # 512 key blocks per row, key chunks of 32 blocks: the counted flush without run keys
    dict(name="counted_flush_32k", n_q=32768, n_k=32768, q_start=0, block_size=64, h_kv=4,
         h_q=32, top_k=16, sampled=True),
    # 2208 blocks of 32 keys (rows past one top-k chunk: run keys, key chunks of 32+
    # blocks), 656 rows in row tiles of 128 (the last one ragged: the spare destination)
    dict(name="counted_flush_runs", n_q=656, n_k=70656, q_start=70000, block_size=32,
         h_kv=2, h_q=8, top_k=24, sampled=False),
], ids=lambda d: d["name"])
def test_counted_flush_block_scores(shape):
    """The maxima flushed with a fixed number of stores per lane (rows a whole number of
    32-block runs, a workspace for the spare destination): block scores bit-exact against
    the oracle, -inf past each row's local block, then the selection and the outputs."""
    d = dict(shape)
    name, sampled = d.pop("name"), d.pop("sampled")
    w = W(name, d_h=64, d_idx=64, needles=8, **d)
    assert (-(-w.n_k // w.block_size)) % 32 == 0
    log(f"case {w.name}: {w}")
    inp = generate(w, device="cuda")
    buf = run_gpu(w, inp, block_scores=True)
    check_selection_invariants(w, buf.sel)
    rows = sample_rows(w, n_random=96) if sampled else None
    ref = oracle_run(w, to_cpu(inp), rows=rows, block_scores=True)
    bs = buf.block_scores
    if rows is not None:
        bs = bs[:, :, torch.as_tensor(rows, device=bs.device)]
    assert np.array_equal(bs.cpu().numpy().astype(np.float64), ref["block_scores"]), \
        "block scores differ"
    compare(w, buf, ref, rows=rows, label=name)


def test_segments_with_small_list_batches():
    """Several row segments (16 heads per group: 4 KiB of Q per row, 16384 rows per
    segment) in a call with few selections, so the list build takes its smallest batches
    (2048 entries, 1024 rows) and the last segment ends inside a batch."""
    w = W("segments_small_batches", n_q=40000, n_k=40000, h_q=16, h_kv=1, d_h=128,
          d_idx=32, block_size=64, top_k=2, needles=4)
    log(f"case {w.name}: {w}")
    inp = generate(w, device="cuda")
    buf = run_gpu(w, inp)
    check_selection_invariants(w, buf.sel)
    rows = sorted(set(sample_rows(w, n_random=96)) |
                  {x for e in (16384, 32768) for x in range(e - 3, e + 3)})
    ref = oracle_run(w, to_cpu(inp), rows=rows)
    compare(w, buf, ref, rows=rows, label=w.name)


@pytest.mark.parametrize("name,seqs", [("decode_256k_b32", [0, 13, 31]),
                                       ("decode_1m_b4", [0, 3])])
def test_decode_workload_full_size(name, seqs):
    w = WORKLOADS[name]
    log(f"case {name}: {w}")
    inp = generate(w, device="cuda")
    buf = run_gpu(w, inp)
    check_selection_invariants(w, buf.sel)
    import oracle
    orc = oracle.get()
    outs = []
    for b in seqs:
        wb = w.replace(batch=1)
        cb = {k: inp[k][b:b + 1].cpu() for k in ("q", "k", "v", "q_idx", "k_idx")}
        outs.append(orc.run(wb, cb))
        log(f"  oracle sequence {b} done")
    ref = {k: np.concatenate([o[k] for o in outs], axis=0) for k in ("sel", "o", "lse")}
    compare(w, buf, ref, seqs=torch.as_tensor(seqs, device="cuda"), label=name)


def test_split_index_calls_equal_fused():
    """msa_index_block_scores + msa_topk_from_block_scores select exactly what
    msa_index_topk selects, and the block scores agree on every visible block."""
    for w in (W("split_prefill", n_q=3000, n_k=3000, top_k=16, needles=6),
              W("split_decode", batch=2, n_q=1, n_k=150000, q_start=149999, block_size=32,
                top_k=32, needles=8)):
        inp = generate(w, device="cuda")
        fused = run_gpu(w, inp, block_scores=True)
        s = msa.shape_of(w)
        nb = -(-w.n_k // w.block_size)
        scores = torch.full((w.batch, w.h_kv, w.n_q, nb), float("nan"), device="cuda")
        sel = torch.empty_like(fused.sel)
        ws = torch.empty(max(1, msa.msa_topk_workspace_size(s)), dtype=torch.uint8, device="cuda")
        msa.msa_index_block_scores(s, inp["q_idx"], inp["k_idx"], scores)
        msa.msa_topk_from_block_scores(s, scores, sel, ws)
        torch.cuda.synchronize()
        assert torch.equal(sel, fused.sel), w.name
        local = (w.q_start + torch.arange(w.n_q, device="cuda")) // w.block_size
        vis = torch.arange(nb, device="cuda")[None, :] <= local[:, None]
        assert torch.equal(scores[..., vis], fused.block_scores[..., vis]), w.name


def test_staged_prefill_calls_equal_single_call():
    """_plan, _partials and _merge in order on one workspace give the same bits as
    msa_sparse_attn_prefill, for a prefill and for a chunk of rows at q_start > 0."""
    for w in (W("staged_prefill", n_q=2000, n_k=2000, top_k=16, needles=6),
              W("staged_chunk_f32", dtype="f32", n_q=300, n_k=1500, q_start=1200, h_q=8,
                h_kv=2, d_h=64, d_idx=32, block_size=32, top_k=5, idx_range=3, qkv_scale=1.0)):
        inp = generate(w, device="cuda")
        one = run_gpu(w, inp)
        s = msa.shape_of(w)
        o = torch.full_like(one.o, float("nan"))
        lse = torch.full_like(one.lse, float("nan"))
        ws = torch.empty(msa.msa_sparse_attn_workspace_size(s), dtype=torch.uint8, device="cuda")
        msa.msa_sparse_attn_prefill_plan(s, one.sel, ws)
        msa.msa_sparse_attn_prefill_partials(s, inp["q"], inp["k"], inp["v"], ws)
        msa.msa_sparse_attn_prefill_merge(s, one.sel, o, lse, ws)
        torch.cuda.synchronize()
        assert torch.equal(o, one.o), w.name
        assert torch.equal(lse, one.lse), w.name


def test_empty_step_is_noop():
    """batch == 0 and n_q == 0 shapes go through the whole step on the GPU as no-ops."""
    for w in (W("empty_batch", batch=0), W("empty_rows", n_q=0, n_k=512, q_start=512),
              W("empty_decode", batch=0, n_q=1, n_k=4096, q_start=4095)):
        s = msa.shape_of(w)
        buf = msa.Buffers(s)
        inp = generate(w, device="cuda")
        msa.msa_step(buf, inp)
        torch.cuda.synchronize()
        assert buf.sel.numel() == 0 and buf.o.numel() == 0, w.name
