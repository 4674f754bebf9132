"""Host-side checks of libmsa.so (no GPU needed): it loads, exports every function that
include/msa.h declares, sizes workspaces, and rejects bad arguments with the documented
code and a message before anything reaches the GPU."""
import ctypes
import os
import re

import pytest

from block_sparse_gqa_msa_amd import binding as msa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msa.h")


@pytest.fixture(scope="module")
def lib():
    return msa.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(msa_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert set(names) == set(msa.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), f"libmsa.so does not export {n}"


def test_header_struct_matches_binding():
    text = open(HEADER).read()
    body = text[text.index("typedef struct {"):text.index("} msa_shape;")]
    fields = re.findall(r"int32_t\s+(\w+);", body)
    assert fields == [n for n, _ in msa.MsaShape._fields_]


def test_abi_version(lib):
    assert msa.msa_abi_version() == 1


def good(**kw):
    f = dict(batch=1, n_q=128, n_k=128, q_start=0, h_q=32, h_kv=4, d_h=128, d_idx=64,
             block_size=64, top_k=8, dtype="bf16")
    f.update(kw)
    return msa.make_shape(**f)


def test_workspace_sizes(lib):
    s = good(batch=2, n_q=1000, n_k=1000)
    nb = -(-1000 // 64)
    assert msa.msa_index_topk_workspace_size(s) >= 2 * 4 * 1000 * nb * 4
    # prefill: per-block lists plus one bf16 partial per (row, group, slot, head)
    assert msa.msa_sparse_attn_workspace_size(s) >= 2 * 4 * 1000 * 8 * 8 * 128 * 2
    d = good(batch=4, n_q=1, n_k=1 << 20, q_start=(1 << 20) - 1, top_k=32)
    # decode partials: (b, h, split) x (d_h + 2) floats
    assert msa.msa_sparse_attn_workspace_size(d) >= 4 * 32 * 32 * 130 * 4
    # chunked prefill at 1M keys needs the two-level candidate buffers
    c = good(n_q=8192, n_k=1 << 20, q_start=(1 << 20) - 8192, top_k=32)
    rows = 4 * 8192
    assert msa.msa_index_topk_workspace_size(c) >= rows * (1 << 14) * 4 + 2 * rows * 8 * 31 * 4


BAD = [
    (dict(batch=-1), msa.MSA_ERR_INVALID_ARG),
    (dict(n_q=-1), msa.MSA_ERR_INVALID_ARG),
    (dict(q_start=-1), msa.MSA_ERR_INVALID_ARG),
    (dict(n_q=100, n_k=120, q_start=30), msa.MSA_ERR_INVALID_ARG),   # q_start + n_q > n_k
    (dict(h_q=30), msa.MSA_ERR_INVALID_ARG),                        # not a multiple of h_kv
    (dict(top_k=0), msa.MSA_ERR_INVALID_ARG),
    (dict(kv_capacity=64), msa.MSA_ERR_INVALID_ARG),                # below n_k
    (dict(dtype=7), msa.MSA_ERR_UNSUPPORTED),
    (dict(block_size=16), msa.MSA_ERR_UNSUPPORTED),
    (dict(top_k=65), msa.MSA_ERR_UNSUPPORTED),
    (dict(h_q=24, h_kv=3), msa.MSA_ERR_UNSUPPORTED),
    (dict(h_q=96, h_kv=4), msa.MSA_ERR_UNSUPPORTED),                # 24 heads per group
    (dict(d_idx=48), msa.MSA_ERR_UNSUPPORTED),
]


@pytest.mark.parametrize("kw,code", BAD, ids=[str(b[0]) for b in BAD])
def test_index_topk_rejects(lib, kw, code):
    s = good(**kw)
    dummy = 1 << 20  # never dereferenced: validation fails first
    rc = lib.msa_index_topk(ctypes.byref(s), dummy, dummy, dummy, None, dummy, 1 << 40, None)
    assert rc == code
    assert msa.msa_last_error() != ""


def test_attention_rejects(lib):
    dummy = 1 << 20
    s = good(d_h=96)
    assert lib.msa_sparse_attn_prefill(ctypes.byref(s), dummy, dummy, dummy, dummy, dummy, None,
                                       None, 0, None) == msa.MSA_ERR_UNSUPPORTED
    s = good()
    assert lib.msa_sparse_attn_prefill(ctypes.byref(s), None, dummy, dummy, dummy, dummy, None,
                                       None, 0, None) == msa.MSA_ERR_INVALID_ARG
    assert "non-NULL" in msa.msa_last_error()
    assert lib.msa_sparse_attn_prefill(ctypes.byref(s), dummy, dummy, dummy, dummy, dummy, None,
                                       dummy, 100, None) == msa.MSA_ERR_WORKSPACE
    # decode needs n_q == 1 at the last position
    assert lib.msa_sparse_attn_decode(ctypes.byref(s), dummy, dummy, dummy, dummy, dummy, None,
                                      dummy, 1 << 30, None) == msa.MSA_ERR_INVALID_ARG
    d = good(n_q=1, n_k=5000, q_start=4999)
    assert lib.msa_sparse_attn_decode(ctypes.byref(d), dummy, dummy, dummy, dummy, dummy, None,
                                      dummy, 16, None) == msa.MSA_ERR_WORKSPACE
    # one head per group with a large top_k is supported; it only needs its workspace
    g = good(h_q=4, h_kv=4, top_k=64)
    assert lib.msa_sparse_attn_prefill(ctypes.byref(g), dummy, dummy, dummy, dummy, dummy, None,
                                       None, 0, None) == msa.MSA_ERR_WORKSPACE


def test_prefill_stage_calls_reject(lib):
    dummy = 1 << 20
    s = good()
    need = msa.msa_sparse_attn_workspace_size(s)
    ok = ctypes.c_size_t(need)
    assert lib.msa_sparse_attn_prefill_plan(ctypes.byref(s), None, dummy, ok, None) \
        == msa.MSA_ERR_INVALID_ARG
    assert lib.msa_sparse_attn_prefill_partials(ctypes.byref(s), dummy, None, dummy, dummy, ok,
                                                None) == msa.MSA_ERR_INVALID_ARG
    assert lib.msa_sparse_attn_prefill_merge(ctypes.byref(s), dummy, None, None, dummy, ok,
                                             None) == msa.MSA_ERR_INVALID_ARG
    small = ctypes.c_size_t(need - 1)
    assert lib.msa_sparse_attn_prefill_plan(ctypes.byref(s), dummy, dummy, small, None) \
        == msa.MSA_ERR_WORKSPACE
    assert lib.msa_sparse_attn_prefill_partials(ctypes.byref(s), dummy, dummy, dummy, None, ok,
                                                None) == msa.MSA_ERR_WORKSPACE
    assert lib.msa_sparse_attn_prefill_merge(ctypes.byref(s), dummy, dummy, None, dummy, small,
                                             None) == msa.MSA_ERR_WORKSPACE
    d = good(d_h=96)
    assert lib.msa_sparse_attn_prefill_plan(ctypes.byref(d), dummy, dummy, ok, None) \
        == msa.MSA_ERR_UNSUPPORTED
    assert lib.msa_sparse_attn_prefill_plan(None, dummy, dummy, ok, None) \
        == msa.MSA_ERR_INVALID_ARG


def test_index_workspace_too_small(lib):
    s = good()
    need = msa.msa_index_topk_workspace_size(s)
    dummy = 1 << 20
    rc = lib.msa_index_topk(ctypes.byref(s), dummy, dummy, dummy, None, dummy, need - 1, None)
    assert rc == msa.MSA_ERR_WORKSPACE
    rc = lib.msa_index_topk(ctypes.byref(s), dummy, dummy, dummy, None, None, need, None)
    assert rc == msa.MSA_ERR_WORKSPACE


def test_null_shape_and_bytes(lib):
    assert lib.msa_index_topk(None, 1, 1, 1, None, None, 0, None) == msa.MSA_ERR_INVALID_ARG
    n = ctypes.c_size_t()
    assert lib.msa_index_topk_workspace_size(None, ctypes.byref(n)) == msa.MSA_ERR_INVALID_ARG
    s = good()
    assert lib.msa_sparse_attn_workspace_size(ctypes.byref(s), None) == msa.MSA_ERR_INVALID_ARG


def test_too_many_candidate_blocks(lib):
    # 2^30 keys in blocks of 32 with k = 64: more chunk winners than one merge pass takes
    s = good(n_q=1, n_k=(1 << 30), q_start=(1 << 30) - 1, block_size=32, top_k=64)
    with pytest.raises(msa.MsaError) as e:
        msa.msa_index_topk_workspace_size(s)
    assert e.value.code == msa.MSA_ERR_UNSUPPORTED


def test_missing_library_raises(tmp_path):
    with pytest.raises(msa.MsaLibraryMissing):
        msa._lib_saved = msa._lib
        try:
            msa._lib = None
            msa.load_library(str(tmp_path / "nope.so"))
        finally:
            msa._lib = msa._lib_saved


def test_empty_calls_are_noops(lib):
    """batch == 0 or n_q == 0: every entry point validates the shape, touches no pointer,
    enqueues nothing (no GPU needed) and returns MSA_OK; workspace sizes are 0."""
    for kw in (dict(batch=0), dict(n_q=0), dict(n_q=0, n_k=0), dict(n_q=0, q_start=128)):
        s = good(**kw)
        assert msa.msa_index_topk_workspace_size(s) == 0
        assert msa.msa_topk_workspace_size(s) == 0
        assert msa.msa_sparse_attn_workspace_size(s) == 0
        sb = ctypes.byref(s)
        assert lib.msa_index_topk(sb, None, None, None, None, None, 0, None) == msa.MSA_OK
        assert lib.msa_index_block_scores(sb, None, None, None, None) == msa.MSA_OK
        assert lib.msa_topk_from_block_scores(sb, None, None, None, 0, None) == msa.MSA_OK
        assert lib.msa_sparse_attn_prefill(sb, None, None, None, None, None, None, None, 0,
                                           None) == msa.MSA_OK
        assert lib.msa_sparse_attn_prefill_plan(sb, None, None, 0, None) == msa.MSA_OK
        assert lib.msa_sparse_attn_prefill_partials(sb, None, None, None, None, 0, None) == msa.MSA_OK
        assert lib.msa_sparse_attn_prefill_merge(sb, None, None, None, None, 0, None) == msa.MSA_OK
    d = good(batch=0, n_q=1, n_k=5000, q_start=4999)
    assert lib.msa_sparse_attn_decode(ctypes.byref(d), None, None, None, None, None, None, None, 0,
                                      None) == msa.MSA_OK
    # the supported set is still checked
    s = good(n_q=0, d_h=96)
    assert lib.msa_sparse_attn_prefill(ctypes.byref(s), None, None, None, None, None, None, None, 0,
                                       None) == msa.MSA_ERR_UNSUPPORTED
    s = good(batch=0, d_idx=48)
    assert lib.msa_index_topk(ctypes.byref(s), None, None, None, None, None, 0, None) \
        == msa.MSA_ERR_UNSUPPORTED


def test_index_kl_rejects(lib):
    dummy = 1 << 20
    s = good()
    need = msa.msa_sparse_attn_workspace_size(s)
    sb = ctypes.byref(s)
    args = [dummy] * 7  # q, k, q_idx, k_idx, sel, lse, kl
    for i in range(7):
        a = list(args)
        a[i] = None
        assert lib.msa_index_kl(sb, *a, None, dummy, need, None) == msa.MSA_ERR_INVALID_ARG
        assert "non-NULL" in msa.msa_last_error()
    assert lib.msa_index_kl(sb, *args, None, dummy, need - 1, None) == msa.MSA_ERR_WORKSPACE
    assert lib.msa_index_kl(sb, *args, None, None, need, None) == msa.MSA_ERR_WORKSPACE
    for bad in (dict(d_idx=48), dict(d_h=96)):
        x = good(**bad)
        assert lib.msa_index_kl(ctypes.byref(x), *args, None, dummy, need, None) \
            == msa.MSA_ERR_UNSUPPORTED
    e = good(n_q=0)
    assert lib.msa_index_kl(ctypes.byref(e), *([None] * 8), None, 0, None) == msa.MSA_OK


def test_backward_rejects(lib):
    dummy = 1 << 20
    s = good()
    need = msa.msa_sparse_attn_backward_workspace_size(s)
    # at least the prefill's lists and partials, D and one fp32 dk/dv partial per list
    assert need > msa.msa_sparse_attn_workspace_size(s)
    sb = ctypes.byref(s)
    args = [dummy] * 10  # q, k, v, sel, o, lse, dout, dq, dk, dv
    for i in range(10):
        a = list(args)
        a[i] = None
        assert lib.msa_sparse_attn_backward(sb, *a, dummy, need, None) == msa.MSA_ERR_INVALID_ARG
        assert "non-NULL" in msa.msa_last_error()
    assert lib.msa_sparse_attn_backward(sb, *args, dummy, need - 1, None) == msa.MSA_ERR_WORKSPACE
    assert lib.msa_sparse_attn_backward(sb, *args, None, need, None) == msa.MSA_ERR_WORKSPACE
    for bad, code in ((dict(d_h=96), msa.MSA_ERR_UNSUPPORTED),
                      (dict(block_size=16), msa.MSA_ERR_UNSUPPORTED),
                      (dict(h_q=12), msa.MSA_ERR_UNSUPPORTED),
                      (dict(h_q=30), msa.MSA_ERR_INVALID_ARG),
                      (dict(q_start=10), msa.MSA_ERR_INVALID_ARG)):
        x = good(**bad)
        assert lib.msa_sparse_attn_backward(ctypes.byref(x), *args, dummy, need, None) == code
    n = ctypes.c_size_t()
    assert lib.msa_sparse_attn_backward_workspace_size(sb, None) == msa.MSA_ERR_INVALID_ARG
    assert lib.msa_sparse_attn_backward_workspace_size(None, ctypes.byref(n)) \
        == msa.MSA_ERR_INVALID_ARG
    for kw in (dict(batch=0), dict(n_q=0)):
        e = good(**kw)
        assert msa.msa_sparse_attn_backward_workspace_size(e) == 0
        assert lib.msa_sparse_attn_backward(ctypes.byref(e), *([None] * 10), None, 0, None) \
            == msa.MSA_OK


def test_index_project_rejects(lib):
    dummy = 1 << 20
    s = good()
    sb = ctypes.byref(s)
    args = [dummy] * 5  # x, w_qidx, w_kidx, q_idx, k_idx
    for i in range(5):
        a = list(args)
        a[i] = None
        assert lib.msa_index_project(sb, 256, *a, None) == msa.MSA_ERR_INVALID_ARG
        assert "non-NULL" in msa.msa_last_error()
    for dm in (0, 32, 96, -64):
        assert lib.msa_index_project(sb, dm, *args, None) == msa.MSA_ERR_UNSUPPORTED
        assert "d_model" in msa.msa_last_error()
    x = good(d_idx=48)
    assert lib.msa_index_project(ctypes.byref(x), 256, *args, None) == msa.MSA_ERR_UNSUPPORTED
    x = good(q_start=10)  # q_start + n_q > n_k
    assert lib.msa_index_project(ctypes.byref(x), 256, *args, None) == msa.MSA_ERR_INVALID_ARG
    for kw in (dict(batch=0), dict(n_q=0)):
        e = good(**kw)
        assert lib.msa_index_project(ctypes.byref(e), 256, *([None] * 5), None) == msa.MSA_OK
    # the supported set is checked on empty calls too
    e = good(n_q=0)
    assert lib.msa_index_project(ctypes.byref(e), 100, *([None] * 5), None) == msa.MSA_ERR_UNSUPPORTED


def test_backward_stage_calls_reject(lib):
    dummy = 1 << 20
    s = good()
    need = msa.msa_sparse_attn_backward_workspace_size(s)
    sb = ctypes.byref(s)
    calls = [(lib.msa_sparse_attn_backward_plan, 3), (lib.msa_sparse_attn_backward_partials, 5),
             (lib.msa_sparse_attn_backward_merge, 4)]
    for fn, n in calls:
        for i in range(n):
            a = [dummy] * n
            a[i] = None
            assert fn(sb, *a, dummy, need, None) == msa.MSA_ERR_INVALID_ARG
            assert "non-NULL" in msa.msa_last_error()
        assert fn(sb, *([dummy] * n), dummy, need - 1, None) == msa.MSA_ERR_WORKSPACE
        x = good(d_h=96)
        assert fn(ctypes.byref(x), *([dummy] * n), dummy, need, None) == msa.MSA_ERR_UNSUPPORTED
        e = good(n_q=0)
        assert fn(ctypes.byref(e), *([None] * n), None, 0, None) == msa.MSA_OK


def test_decode_step_rejects(lib):
    """msa_decode_step: decode shape only, every pointer required (lse optional), workspace
    sized by msa_decode_step_workspace_size and at least the two calls' workspaces it
    contains, supported set of both halves checked."""
    dummy = 1 << 20
    d = good(batch=2, n_q=1, n_k=5000, q_start=4999, top_k=16)
    need = msa.msa_decode_step_workspace_size(d)
    assert need >= msa.msa_index_topk_workspace_size(d) + msa.msa_sparse_attn_workspace_size(d)
    db = ctypes.byref(d)
    args = lambda ws_bytes, **none: [db] + [None if k in none else dummy for k in (
        "q", "k", "v", "q_idx", "k_idx", "sel", "o")] + [None, dummy, ws_bytes, None]
    assert lib.msa_decode_step(*args(need - 1)) == msa.MSA_ERR_WORKSPACE
    for name in ("q", "k", "v", "q_idx", "k_idx", "sel", "o"):
        assert lib.msa_decode_step(*args(need, **{name: True})) == msa.MSA_ERR_INVALID_ARG, name
    p = good(n_q=64, n_k=5000, q_start=100)  # not a decode shape
    assert lib.msa_decode_step(ctypes.byref(p), dummy, dummy, dummy, dummy, dummy, dummy, dummy,
                               None, dummy, need, None) == msa.MSA_ERR_INVALID_ARG
    for kw in (dict(d_h=96), dict(d_idx=48), dict(block_size=16), dict(top_k=65)):
        bad = good(batch=2, n_q=1, n_k=5000, q_start=4999, **{"top_k": 16, **kw})
        assert lib.msa_decode_step(ctypes.byref(bad), dummy, dummy, dummy, dummy, dummy, dummy,
                                   dummy, None, dummy, need, None) == msa.MSA_ERR_UNSUPPORTED, kw
        n = ctypes.c_size_t()
        assert lib.msa_decode_step_workspace_size(ctypes.byref(bad), ctypes.byref(n)) \
            == msa.MSA_ERR_UNSUPPORTED, kw
    assert lib.msa_decode_step_workspace_size(db, None) == msa.MSA_ERR_INVALID_ARG
    # empty calls: size 0, no pointer touched
    e = good(batch=0, n_q=1, n_k=5000, q_start=4999)
    assert msa.msa_decode_step_workspace_size(e) == 0
    assert lib.msa_decode_step(ctypes.byref(e), None, None, None, None, None, None, None, None,
                               None, 0, None) == msa.MSA_OK


def test_decode_step_noalloc_rejects(lib):
    """msa_decode_step_noalloc: the same validation as msa_decode_step, and shapes whose
    workspace exceeds its scratch array are refused before anything is enqueued."""
    dummy = 1 << 20
    d = good(batch=2, n_q=1, n_k=5000, q_start=4999, top_k=16)
    db = ctypes.byref(d)
    args = lambda **none: [db] + [None if k in none else dummy for k in (
        "q", "k", "v", "q_idx", "k_idx", "sel", "o")] + [None, None]
    for name in ("q", "k", "v", "q_idx", "k_idx", "sel", "o"):
        assert lib.msa_decode_step_noalloc(*args(**{name: True})) == msa.MSA_ERR_INVALID_ARG, name
    p = good(n_q=64, n_k=5000, q_start=100)  # not a decode shape
    assert lib.msa_decode_step_noalloc(ctypes.byref(p), *([dummy] * 7), None, None) \
        == msa.MSA_ERR_INVALID_ARG
    big = good(batch=64, n_q=1, n_k=1 << 20, q_start=(1 << 20) - 1, top_k=32)
    assert msa.msa_decode_step_workspace_size(big) > msa.DECODE_STEP_SCRATCH_BYTES
    assert lib.msa_decode_step_noalloc(ctypes.byref(big), *([dummy] * 7), None, None) \
        == msa.MSA_ERR_WORKSPACE
    assert b"scratch" in lib.msa_last_error()
    from block_sparse_gqa_msa_amd.inputs import WORKLOADS
    for name in ("decode_256k_b32", "decode_1m_b4"):
        assert msa.msa_decode_step_workspace_size(msa.shape_of(WORKLOADS[name])) \
            <= msa.DECODE_STEP_SCRATCH_BYTES, name
    e = good(batch=0, n_q=1, n_k=5000, q_start=4999)
    assert lib.msa_decode_step_noalloc(ctypes.byref(e), *([None] * 9)) == msa.MSA_OK
