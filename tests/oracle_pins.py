"""Pins for the fp64 oracle: checks against what the MSA definition and plain
mathematics fix, none of which re-types the oracle's own code.

Definitions pinned (page "MiniMax-M3: MSA 技术报告速读", section 核心机制):
  index-branch token scores and causal block max-pool, the per-group TopK with
  the local block forced in, and the main-branch sparse softmax attention; and
  (section 训练) the index-branch distribution P^idx, the group-averaged teacher
  P^(r) over the selected tokens and the alignment loss KL(P^(r) || P^idx); the
  gradients of the main-branch equation for a fixed selection; and (section 核心机制,
  索引分支) the index branch's two projections: one index query head per group, one index
  key shared by the groups.

Each pin takes an ``oracle.Oracle`` and raises AssertionError on a mismatch, so
the same pins also run against deliberately broken oracle builds.
"""
from __future__ import annotations

import itertools
import math
from types import SimpleNamespace

import numpy as np
import torch


def shape(**kw):
    base = dict(dtype="f32", batch=1, n_q=8, n_k=8, q_start=0, h_q=2, h_kv=1, d_h=4, d_idx=2,
                block_size=2, top_k=2)
    base.update(kw)
    return SimpleNamespace(**base)


def rand_inputs(w, seed, idx_values=(-2, 3), cont_idx=False):
    """Small fp32 inputs: Gaussian q, k, v; integer (or Gaussian) index inputs."""
    g = torch.Generator().manual_seed(seed)
    B, R, H = w.batch, w.h_kv, w.h_q
    out = dict(
        q=torch.randn(B, H, w.n_q, w.d_h, generator=g),
        k=torch.randn(B, R, w.n_k, w.d_h, generator=g),
        v=torch.randn(B, R, w.n_k, w.d_h, generator=g),
    )
    if cont_idx:
        out["q_idx"] = torch.randn(B, R, w.n_q, w.d_idx, generator=g)
        out["k_idx"] = torch.randn(B, w.n_k, w.d_idx, generator=g)
    else:
        lo, hi = idx_values
        out["q_idx"] = torch.randint(lo, hi, (B, R, w.n_q, w.d_idx), generator=g).float()
        out["k_idx"] = torch.randint(lo, hi, (B, w.n_k, w.d_idx), generator=g).float()
    return out


def exact_block_max(w, inp):
    """Causal block maxima in exact int64 arithmetic (integer-valued index inputs)."""
    qi = inp["q_idx"].numpy().astype(np.int64)      # [B,R,n_q,d]
    ki = inp["k_idx"].numpy().astype(np.int64)      # [B,n_k,d]
    s = np.einsum("brtd,bjd->brtj", qi, ki).astype(np.float64)
    pos = w.q_start + np.arange(w.n_q)
    j = np.arange(w.n_k)
    s[:, :, j[None, :] > pos[:, None]] = -np.inf     # keys after the query are invisible
    nb = -(-w.n_k // w.block_size)
    pad = nb * w.block_size - w.n_k
    s = np.concatenate([s, np.full(s.shape[:-1] + (pad,), -np.inf)], axis=-1)
    return s.reshape(s.shape[:-1] + (nb, w.block_size)).max(axis=-1)


def visible_token_mask(w, sel):
    """[B,R,n_q,n_k] bool: token j attended by row t of group r under selection ``sel``."""
    B, R, n, k = sel.shape
    mask = np.zeros((B, R, n, w.n_k), bool)
    for b, r, t in itertools.product(range(B), range(R), range(n)):
        p = w.q_start + t
        for c in sel[b, r, t]:
            if c >= 0:
                lo, hi = c * w.block_size, min((c + 1) * w.block_size, p + 1)
                mask[b, r, t, lo:hi] = True
    return mask


def sdpa_reference(w, inp, mask_brtj):
    """Attention output and LSE with torch's SDPA (fp64) under a token mask, GQA via repeat."""
    G = w.h_q // w.h_kv
    q = inp["q"].double()
    k = inp["k"].double().repeat_interleave(G, dim=1)
    v = inp["v"].double().repeat_interleave(G, dim=1)
    m = torch.from_numpy(mask_brtj).repeat_interleave(G, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=m)
    z = (q @ k.transpose(-1, -2)) / math.sqrt(w.d_h)
    lse = torch.logsumexp(z.masked_fill(~m, -math.inf), dim=-1)
    return o.numpy(), lse.numpy()


def causal_mask(w):
    pos = w.q_start + np.arange(w.n_q)
    m = np.arange(w.n_k)[None, :] <= pos[:, None]
    return np.broadcast_to(m, (w.batch, w.h_kv, w.n_q, w.n_k)).copy()


# ----------------------------------------------------------------------------- pins

def pin_block_scores_exact(orc):
    """Block scores equal exact integer causal block maxima (ragged last block, q_start>0)."""
    for kw in (dict(batch=2, h_kv=3, h_q=3, n_q=37, n_k=37, d_idx=5, block_size=8, top_k=3),
               dict(batch=1, h_kv=2, h_q=4, n_q=9, n_k=30, q_start=21, d_idx=3, block_size=4,
                    top_k=2)):
        w = shape(**kw)
        inp = rand_inputs(w, seed=11)
        got = orc.run(w, inp, attention=False, block_scores=True)["block_scores"]
        want = exact_block_max(w, inp)
        assert np.array_equal(got, want), "block scores differ from exact causal block maxima"


def pin_topk_bruteforce(orc):
    """Selections equal the unique subset no unselected block beats (exhaustive search).

    Block c beats block u when its score is higher, or equal with a lower index.
    The query's own block is always in, top_k counts it, and a query that sees
    top_k blocks or fewer takes them all. Heavy ties come from index values in {-1,0,1}.
    """
    for top_k in (1, 2, 3, 4, 9, 10):
        w = shape(batch=1, h_kv=2, h_q=2, n_q=18, n_k=18, d_idx=2, block_size=2, top_k=top_k)
        inp = rand_inputs(w, seed=5 + top_k, idx_values=(-1, 2))
        sel = orc.run(w, inp, attention=False)["sel"]
        bm = exact_block_max(w, inp)
        for r, t in itertools.product(range(w.h_kv), range(w.n_q)):
            p = w.q_start + t
            local = p // w.block_size
            m = min(top_k - 1, local)
            valid = []
            for sub in itertools.combinations(range(local), m):
                rest = [u for u in range(local) if u not in sub]
                if all(bm[0, r, t, c] > bm[0, r, t, u] or
                       (bm[0, r, t, c] == bm[0, r, t, u] and c < u) for c in sub for u in rest):
                    valid.append(sub)
            assert len(valid) == 1
            want = sorted(valid[0] + (local,))
            want += [-1] * (top_k - len(want))
            assert list(sel[0, r, t]) == want, (top_k, r, t, list(sel[0, r, t]), want)


def pin_dense_when_k_covers(orc):
    """k >= number of blocks: the step equals dense causal GQA attention (torch SDPA, fp64)."""
    for kw in (dict(batch=2, h_q=6, h_kv=3, n_q=40, n_k=40, d_h=8, d_idx=3, block_size=8,
                    top_k=5),
               dict(batch=1, h_q=4, h_kv=2, n_q=10, n_k=29, q_start=19, d_h=6, d_idx=2,
                    block_size=4, top_k=8)):
        w = shape(**kw)
        inp = rand_inputs(w, seed=3)
        out = orc.run(w, inp)
        o, lse = sdpa_reference(w, inp, causal_mask(w))
        assert np.allclose(out["o"], o, rtol=0, atol=1e-12)
        assert np.allclose(out["lse"], lse, rtol=0, atol=1e-12)


def pin_local_block_only(orc):
    """k = 1: each query attends exactly to the visible part of its own block."""
    w = shape(batch=1, h_q=4, h_kv=2, n_q=21, n_k=21, d_h=5, d_idx=2, block_size=4, top_k=1)
    inp = rand_inputs(w, seed=4)
    out = orc.run(w, inp)
    pos = np.arange(w.n_q)[:, None]
    j = np.arange(w.n_k)[None, :]
    m = (j <= pos) & (j // w.block_size == pos // w.block_size)
    o, lse = sdpa_reference(w, inp, np.broadcast_to(m, (1, 2, w.n_q, w.n_k)).copy())
    assert np.allclose(out["o"], o, rtol=0, atol=1e-12)
    assert np.allclose(out["lse"], lse, rtol=0, atol=1e-12)


def pin_token_level(orc):
    """block_size = 1: selection is the query token plus torch.topk of earlier token scores."""
    w = shape(batch=1, h_q=2, h_kv=2, n_q=24, n_k=24, d_h=4, d_idx=3, block_size=1, top_k=5)
    inp = rand_inputs(w, seed=9, cont_idx=True)   # continuous scores: no ties
    out = orc.run(w, inp)
    s = torch.einsum("brtd,bjd->brtj", inp["q_idx"].double(), inp["k_idx"].double())
    want = np.full((1, 2, w.n_q, w.top_k), -1, np.int32)
    for r, t in itertools.product(range(2), range(w.n_q)):
        if t + 1 <= w.top_k:
            chosen = list(range(t + 1))
        else:
            chosen = torch.topk(s[0, r, t, :t], w.top_k - 1).indices.tolist() + [t]
        chosen = sorted(chosen)
        want[0, r, t, :len(chosen)] = chosen
    assert np.array_equal(out["sel"], want)
    o, lse = sdpa_reference(w, inp, visible_token_mask(w, want))
    assert np.allclose(out["o"], o, rtol=0, atol=1e-12)
    assert np.allclose(out["lse"], lse, rtol=0, atol=1e-12)


def pin_zero_query_closed_form(orc):
    """q = 0: uniform weights, so lse = ln|T| with |T| = (min(k, b+1)-1)*bs + (p - b*bs + 1)
    and o = mean of v over the attended tokens."""
    w = shape(batch=1, h_q=2, h_kv=1, n_q=45, n_k=45, d_h=3, d_idx=2, block_size=4, top_k=3)
    inp = rand_inputs(w, seed=6)
    inp["q"].zero_()
    out = orc.run(w, inp)
    v = inp["v"].double().numpy()
    mask = visible_token_mask(w, out["sel"])
    for t in range(w.n_q):
        p = t
        b = p // w.block_size
        n_tok = (min(w.top_k, b + 1) - 1) * w.block_size + (p - b * w.block_size + 1)
        assert mask[0, 0, t].sum() == n_tok
        for h in range(w.h_q):
            assert abs(out["lse"][0, h, t] - math.log(n_tok)) < 1e-12
            assert np.allclose(out["o"][0, h, t], v[0, 0, mask[0, 0, t]].mean(axis=0), atol=1e-12)


def pin_group_map_and_ones(orc):
    """v = r + 1 on group r: head h must output h // (H_q/H_kv) + 1 exactly (softmax sums to 1)."""
    w = shape(batch=2, h_q=6, h_kv=3, n_q=20, n_k=20, d_h=4, d_idx=2, block_size=4, top_k=2)
    inp = rand_inputs(w, seed=8)
    for r in range(w.h_kv):
        inp["v"][:, r] = float(r + 1)
    out = orc.run(w, inp)
    G = w.h_q // w.h_kv
    for h in range(w.h_q):
        assert np.allclose(out["o"][:, h], h // G + 1, rtol=0, atol=1e-13)


def pin_entry_point_consistency(orc):
    """A chunk at q_start > 0 and a single decode row equal the matching rows of the full
    prefill (causality is by absolute position)."""
    w = shape(batch=2, h_q=4, h_kv=2, n_q=33, n_k=33, d_h=4, d_idx=3, block_size=4, top_k=3)
    inp = rand_inputs(w, seed=10)
    full = orc.run(w, inp, block_scores=True)
    for start in (20, 32):
        wc = shape(**{**vars(w), "n_q": w.n_q - start, "q_start": start})
        ic = dict(inp)
        ic["q"] = inp["q"][:, :, start:].contiguous()
        ic["q_idx"] = inp["q_idx"][:, :, start:].contiguous()
        part = orc.run(wc, ic, block_scores=True)
        for key in ("sel", "block_scores", "o", "lse"):
            a, b = part[key], full[key][:, :, start:]
            assert np.array_equal(a, b), key


def pin_bf16_storage_widening(orc):
    """bf16 storage is widened exactly: bf16 inputs give bit-identical results to the same
    values stored as fp32."""
    w = shape(batch=1, h_q=4, h_kv=2, n_q=19, n_k=19, d_h=8, d_idx=4, block_size=4, top_k=3)
    inp = rand_inputs(w, seed=12)
    as_bf16 = {k: x.to(torch.bfloat16) for k, x in inp.items()}
    as_f32 = {k: x.float() for k, x in as_bf16.items()}
    a = orc.run(shape(**{**vars(w), "dtype": "bf16"}), as_bf16, block_scores=True)
    b = orc.run(w, as_f32, block_scores=True)
    for key in a:
        assert np.array_equal(a[key], b[key]), key


def pin_general_sparse(orc):
    """General sparse selections (neither dense, local-only nor token-level): the selection
    satisfies the threshold property against exact integer block maxima (every selected
    earlier block beats every unselected visible one under (score desc, block asc), the
    local block is in, the count is min(k, local+1), ascending), and the attention output
    equals torch's fp64 SDPA under the token mask of that selection."""
    for kw in (dict(batch=2, h_q=8, h_kv=2, n_q=70, n_k=70, d_h=8, d_idx=4, block_size=4,
                    top_k=5),
               dict(batch=1, h_q=6, h_kv=3, n_q=33, n_k=101, q_start=68, d_h=5, d_idx=3,
                    block_size=8, top_k=4)):
        w = shape(**kw)
        inp = rand_inputs(w, seed=21, idx_values=(-3, 4))
        out = orc.run(w, inp)
        m = exact_block_max(w, inp)
        sel = out["sel"]
        for b, r, t in itertools.product(range(w.batch), range(w.h_kv), range(w.n_q)):
            local = (w.q_start + t) // w.block_size
            row = sel[b, r, t]
            chosen = [int(c) for c in row if c >= 0]
            assert len(chosen) == min(w.top_k, local + 1)
            assert chosen == sorted(set(chosen)) and local in chosen
            assert list(row[len(chosen):]) == [-1] * (w.top_k - len(chosen))
            picked = [c for c in chosen if c != local]
            others = [c for c in range(local) if c not in chosen]
            for c in picked:
                for c2 in others:
                    mc, mc2 = m[b, r, t, c], m[b, r, t, c2]
                    assert mc > mc2 or (mc == mc2 and c < c2), (b, r, t, c, c2)
        o, lse = sdpa_reference(w, inp, visible_token_mask(w, sel))
        assert np.allclose(out["o"], o, rtol=0, atol=1e-12)
        assert np.allclose(out["lse"], lse, rtol=0, atol=1e-12)


# ----------------------------------------------------------------- alignment loss pins

def pin_kl_two_tokens_closed_form(orc):
    """Two selected tokens, one head: both distributions are Bernoulli, and
    KL(a || b) = a ln(a/b) + (1-a) ln((1-a)/(1-b)) with a = sigmoid(z1 - z0), b =
    sigmoid(s1 - s0), worked by hand: d_h = d_idx = 1, q = 2, k = (0, 1), q_idx = 1,
    k_idx = (0, 3), so z = (0, 2) and s = (0, 3)."""
    w = shape(n_q=2, n_k=2, h_q=1, h_kv=1, d_h=1, d_idx=1, block_size=1, top_k=2)
    inp = dict(q=torch.tensor([2.0, 2.0]).reshape(1, 1, 2, 1),
               k=torch.tensor([0.0, 1.0]).reshape(1, 1, 2, 1),
               v=torch.zeros(1, 1, 2, 1),
               q_idx=torch.tensor([1.0, 1.0]).reshape(1, 1, 2, 1),
               k_idx=torch.tensor([0.0, 3.0]).reshape(1, 2, 1))
    sel = orc.run(w, inp, attention=False)["sel"]
    assert sel[0, 0, 1].tolist() == [0, 1]
    out = orc.kl(w, inp, sel)
    a, b = 1 / (1 + math.exp(-2)), 1 / (1 + math.exp(-3))
    want = a * math.log(a / b) + (1 - a) * math.log((1 - a) / (1 - b))
    assert abs(out["kl"][0, 0, 1] - want) < 1e-14, (out["kl"][0, 0, 1], want)
    assert abs(out["lse_idx"][0, 0, 1] - math.log(1 + math.exp(3))) < 1e-14
    assert out["kl"][0, 0, 0] == 0.0  # row 0 sees one token: both distributions are {1}


def pin_kl_student_equals_teacher(orc):
    """Index branch identical to the main branch (one group, d_idx = d_h, q_idx = q of a
    head, k_idx = k): the student equals every head's distribution, so the loss is 0 for
    one head and for G identical heads (the teacher is their mean), on sparse selections."""
    for G in (1, 3):
        w = shape(batch=2, h_q=G, h_kv=1, n_q=40, n_k=40, d_h=6, d_idx=6, block_size=4,
                  top_k=3)
        g = torch.Generator().manual_seed(5)
        q1 = torch.randn(2, 1, 40, 6, generator=g)
        k = torch.randn(2, 1, 40, 6, generator=g)
        inp = dict(q=q1.repeat(1, G, 1, 1), k=k, v=torch.zeros_like(k), q_idx=q1.clone(),
                   k_idx=k[:, 0].clone())
        sel = orc.run(w, inp, attention=False)["sel"]
        local = (w.q_start + np.arange(w.n_q)) // w.block_size
        assert ((sel >= 0).sum(-1) < local + 1).any()  # some selections leave blocks out
        out = orc.kl(w, inp, sel)
        assert np.abs(out["kl"]).max() < 1e-12, np.abs(out["kl"]).max()


def pin_kl_uniform_teacher(orc):
    """q = 0 makes every head's distribution uniform over the selected tokens T, so the
    loss is KL(U || P^idx) = -ln|T| - mean_T log P^idx, with log P^idx from scipy's
    log_softmax of exact integer index scores / sqrt(d_idx) over T."""
    from scipy.special import log_softmax
    w = shape(batch=2, h_q=4, h_kv=2, n_q=50, n_k=50, d_h=4, d_idx=3, block_size=4, top_k=4)
    inp = rand_inputs(w, seed=9, idx_values=(-3, 4))
    inp["q"] = torch.zeros_like(inp["q"])
    sel = orc.run(w, inp, attention=False)["sel"]
    out = orc.kl(w, inp, sel)
    mask = visible_token_mask(w, sel)
    qi = inp["q_idx"].numpy().astype(np.int64)
    ki = inp["k_idx"].numpy().astype(np.int64)
    s = np.einsum("brtd,bjd->brtj", qi, ki) / math.sqrt(w.d_idx)
    for b, r, t in itertools.product(range(w.batch), range(w.h_kv), range(w.n_q)):
        m = mask[b, r, t]
        assert m.any(), (b, r, t)  # every row selects at least its own block
        logq = log_softmax(s[b, r, t][m])
        want = -math.log(m.sum()) - logq.mean()
        assert abs(out["kl"][b, r, t] - want) < 1e-12, (b, r, t)
        assert abs(out["lse_idx"][b, r, t] - np.log(np.exp(s[b, r, t][m]).sum())) < 1e-12


def pin_kl_dense_scipy(orc):
    """k covering every block: T is the whole causal prefix, and the loss is scipy's
    relative entropy of the mean of the G heads' softmaxes (scipy) against the softmax of
    the index scores, per row; it is also never negative."""
    from scipy.special import softmax
    from scipy.stats import entropy
    w = shape(batch=1, h_q=4, h_kv=2, n_q=24, n_k=24, d_h=5, d_idx=3, block_size=4, top_k=6)
    inp = rand_inputs(w, seed=13, idx_values=(-2, 3))
    sel = orc.run(w, inp, attention=False)["sel"]
    out = orc.kl(w, inp, sel)
    G = w.h_q // w.h_kv
    q = inp["q"].double().numpy()
    k = inp["k"].double().numpy()
    qi = inp["q_idx"].double().numpy()
    ki = inp["k_idx"].double().numpy()
    for r, t in itertools.product(range(w.h_kv), range(w.n_q)):
        n = t + 1
        heads = [softmax(q[0, r * G + l, t] @ k[0, r, :n].T / math.sqrt(w.d_h)) for l in range(G)]
        teacher = np.mean(heads, axis=0)
        student = softmax(qi[0, r, t] @ ki[0, :n].T / math.sqrt(w.d_idx))
        assert abs(out["kl"][0, r, t] - entropy(teacher, student)) < 1e-12, (r, t)
    assert out["kl"].min() >= -1e-15


# ----------------------------------------------------------------- main-branch gradient pins

def pin_bwd_autograd(orc):
    """General sparse selections: dq, dk, dv equal torch autograd (fp64) through SDPA under
    the selection's token mask, GQA by repeating K/V over each group's heads."""
    for kw in (dict(batch=2, h_q=8, h_kv=2, n_q=40, n_k=40, d_h=8, d_idx=4, block_size=4,
                    top_k=3),
               dict(batch=1, h_q=6, h_kv=3, n_q=21, n_k=61, q_start=40, d_h=5, d_idx=3,
                    block_size=8, top_k=4)):
        w = shape(**kw)
        inp = rand_inputs(w, seed=31, idx_values=(-3, 4))
        g = torch.Generator().manual_seed(32)
        dout = torch.randn(w.batch, w.h_q, w.n_q, w.d_h, generator=g)
        sel = orc.run(w, inp, attention=False)["sel"]
        got = orc.attn_bwd(w, inp, sel, dout)
        G = w.h_q // w.h_kv
        q = inp["q"].double().requires_grad_()
        k = inp["k"].double().requires_grad_()
        v = inp["v"].double().requires_grad_()
        m = torch.from_numpy(visible_token_mask(w, sel)).repeat_interleave(G, dim=1)
        o = torch.nn.functional.scaled_dot_product_attention(
            q, k.repeat_interleave(G, dim=1), v.repeat_interleave(G, dim=1), attn_mask=m)
        (o * dout.double()).sum().backward()
        for name, ref in (("dq", q.grad), ("dk", k.grad), ("dv", v.grad)):
            assert np.allclose(got[name], ref.numpy(), rtol=0, atol=1e-12), name


def pin_bwd_finite_difference(orc):
    """Central differences of L = sum(dout * O) through the (pinned) forward oracle, for a
    spread of q, k and v coordinates; the selection does not depend on them."""
    w = shape(batch=1, h_q=4, h_kv=2, n_q=12, n_k=12, d_h=3, d_idx=2, block_size=2, top_k=3)
    inp = rand_inputs(w, seed=41, idx_values=(-2, 3))
    g = torch.Generator().manual_seed(42)
    dout = torch.randn(w.batch, w.h_q, w.n_q, w.d_h, generator=g)
    sel = orc.run(w, inp, attention=False)["sel"]
    got = orc.attn_bwd(w, inp, sel, dout)
    eps = 2.0 ** -10  # x +- eps is exact in fp32 for these magnitudes
    rng = np.random.default_rng(43)

    def loss(x):
        return float((orc.run(w, x)["o"] * dout.double().numpy()).sum())

    for name, grad in (("q", "dq"), ("k", "dk"), ("v", "dv")):
        shp = tuple(inp[name].shape)
        for _ in range(6):
            idx = tuple(int(rng.integers(0, n)) for n in shp)
            plus = dict(inp)
            minus = dict(inp)
            plus[name] = inp[name].clone()
            minus[name] = inp[name].clone()
            plus[name][idx] += eps
            minus[name][idx] -= eps
            fd = (loss(plus) - loss(minus)) / (2 * eps)
            assert abs(fd - got[grad][idx]) < 2e-5 * (1 + abs(fd)), (name, idx, fd, got[grad][idx])


def pin_project_selector_weights(orc):
    """Weights whose rows each pick one input coordinate: every output is exactly one
    element of x, which fixes the output layout (group-major index queries, one shared
    index key per row) and the weight orientation (a row per output)."""
    B, n, dm, R, DI = 2, 5, 24, 3, 4
    g = torch.Generator().manual_seed(51)
    x = torch.randn(B, n, dm, generator=g)
    pq = torch.randperm(dm, generator=g)[: R * DI]
    pk = torch.randperm(dm, generator=g)[:DI]
    w_q = torch.zeros(R * DI, dm)
    w_q[torch.arange(R * DI), pq] = 1.0
    w_k = torch.zeros(DI, dm)
    w_k[torch.arange(DI), pk] = 1.0
    out = orc.project(x, w_q, w_k, R, DI)
    xd = x.double().numpy()
    for r in range(R):
        for d in range(DI):
            assert np.array_equal(out["q_idx"][:, r, :, d], xd[:, :, int(pq[r * DI + d])]), (r, d)
    for d in range(DI):
        assert np.array_equal(out["k_idx"][:, :, d], xd[:, :, int(pk[d])]), d


def pin_project_integer_bruteforce(orc):
    """Small integer inputs: exact sums, against explicit Python loops over the definition."""
    B, n, dm, R, DI = 1, 3, 7, 2, 3
    g = torch.Generator().manual_seed(52)
    x = torch.randint(-3, 4, (B, n, dm), generator=g).float()
    w_q = torch.randint(-2, 3, (R * DI, dm), generator=g).float()
    w_k = torch.randint(-2, 3, (DI, dm), generator=g).float()
    out = orc.project(x, w_q, w_k, R, DI)
    for b in range(B):
        for t in range(n):
            for r in range(R):
                for d in range(DI):
                    want = sum(float(x[b, t, i]) * float(w_q[r * DI + d, i]) for i in range(dm))
                    assert out["q_idx"][b, r, t, d] == want
            for d in range(DI):
                want = sum(float(x[b, t, i]) * float(w_k[d, i]) for i in range(dm))
                assert out["k_idx"][b, t, d] == want


def pin_project_matmul(orc):
    """Gaussian inputs in bf16 storage against numpy's fp64 matrix product of the same
    bf16 values (widened by torch): the whole reduction, nothing dropped."""
    B, n, dm, R, DI = 2, 9, 96, 4, 8
    g = torch.Generator().manual_seed(53)
    x = torch.randn(B, n, dm, generator=g).bfloat16()
    w_q = (torch.randn(R * DI, dm, generator=g) / 8).bfloat16()
    w_k = (torch.randn(DI, dm, generator=g) / 8).bfloat16()
    out = orc.project(x, w_q, w_k, R, DI)
    xd, wq, wk = (a.double().numpy() for a in (x, w_q, w_k))
    want_q = np.matmul(xd, wq.T).reshape(B, n, R, DI).transpose(0, 2, 1, 3)
    want_k = np.matmul(xd, wk.T)
    assert np.abs(out["q_idx"] - want_q).max() <= 1e-12 * np.abs(want_q).max()
    assert np.abs(out["k_idx"] - want_k).max() <= 1e-12 * np.abs(want_k).max()


PINS = [pin_block_scores_exact, pin_topk_bruteforce, pin_dense_when_k_covers,
        pin_local_block_only, pin_token_level, pin_zero_query_closed_form,
        pin_group_map_and_ones, pin_entry_point_consistency, pin_bf16_storage_widening,
        pin_general_sparse, pin_kl_two_tokens_closed_form, pin_kl_student_equals_teacher,
        pin_kl_uniform_teacher, pin_kl_dense_scipy, pin_bwd_autograd, pin_bwd_finite_difference,
        pin_project_selector_weights, pin_project_integer_bruteforce, pin_project_matmul]
