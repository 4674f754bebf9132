"""ctypes binding of libmsa.so (include/msa.h): argument marshalling only.

Each C entry point has a Python function of the same name taking an ``MsaShape``
and torch tensors (or raw device pointers as ints). The functions check that
tensors are contiguous, on the GPU and of the expected dtype, pass
``data_ptr()`` and the current HIP stream, and raise ``MsaError`` with the
library's message when a call returns an error code. Every step of the
computation runs in the library's HIP kernels; if the library is missing,
loading it raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmsa.so")

MSA_F32, MSA_BF16 = 0, 1
MSA_OK, MSA_ERR_INVALID_ARG, MSA_ERR_UNSUPPORTED, MSA_ERR_WORKSPACE, MSA_ERR_HIP = 0, -1, -2, -3, -4
EXPORTS = ("msa_index_topk_workspace_size", "msa_index_topk", "msa_index_topk_scores",
           "msa_index_topk_select", "msa_index_block_scores",
           "msa_topk_workspace_size", "msa_topk_from_block_scores",
           "msa_sparse_attn_workspace_size", "msa_sparse_attn_prefill",
           "msa_sparse_attn_prefill_plan", "msa_sparse_attn_prefill_partials",
           "msa_sparse_attn_prefill_merge", "msa_sparse_attn_decode", "msa_index_kl",
           "msa_sparse_attn_backward_workspace_size", "msa_sparse_attn_backward",
           "msa_sparse_attn_backward_plan", "msa_sparse_attn_backward_partials",
           "msa_sparse_attn_backward_merge", "msa_index_project",
           "msa_decode_step_workspace_size", "msa_decode_step", "msa_decode_step_noalloc",
           "msa_last_error", "msa_abi_version")
DECODE_STEP_SCRATCH_BYTES = 32 << 20  # MSA_DECODE_STEP_SCRATCH_BYTES


class MsaShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "n_q", "n_k", "q_start", "h_q", "h_kv", "d_h", "d_idx", "block_size", "top_k",
        "dtype", "kv_capacity")]

    def __repr__(self):
        return "MsaShape(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"


class MsaError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"[{code}] {message}")
        self.code = code
        self.message = message


class MsaLibraryMissing(ImportError):
    pass


_lib: Optional[ctypes.CDLL] = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmsa.so once; raise MsaLibraryMissing if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise MsaLibraryMissing(
            f"{path} is missing: build it with `python -m block_sparse_gqa_msa_amd.build`")
    # torch's HIP runtime first: the library's libamdhip64 dependency then binds to the
    # same runtime instance that owns the tensors and streams it is handed (a second
    # runtime loaded beside it sees no device).
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    P, S, I = ctypes.c_void_p, ctypes.POINTER(MsaShape), ctypes.c_int
    sz = ctypes.POINTER(ctypes.c_size_t)
    lib.msa_index_topk_workspace_size.argtypes = [S, sz]
    lib.msa_sparse_attn_workspace_size.argtypes = [S, sz]
    lib.msa_topk_workspace_size.argtypes = [S, sz]
    lib.msa_index_block_scores.argtypes = [S, P, P, P, P]
    lib.msa_topk_from_block_scores.argtypes = [S, P, P, P, ctypes.c_size_t, P]
    lib.msa_index_topk.argtypes = [S, P, P, P, P, P, ctypes.c_size_t, P]
    lib.msa_index_topk_scores.argtypes = [S, P, P, P, P, ctypes.c_size_t, P]
    lib.msa_index_topk_select.argtypes = [S, P, P, P, ctypes.c_size_t, P]
    lib.msa_sparse_attn_prefill.argtypes = [S, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.msa_sparse_attn_prefill_plan.argtypes = [S, P, P, ctypes.c_size_t, P]
    lib.msa_sparse_attn_prefill_partials.argtypes = [S, P, P, P, P, ctypes.c_size_t, P]
    lib.msa_sparse_attn_prefill_merge.argtypes = [S, P, P, P, P, ctypes.c_size_t, P]
    lib.msa_sparse_attn_decode.argtypes = [S, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.msa_index_kl.argtypes = [S, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.msa_sparse_attn_backward_workspace_size.argtypes = [S, sz]
    lib.msa_index_project.argtypes = [S, ctypes.c_int32, P, P, P, P, P, P]
    lib.msa_sparse_attn_backward_plan.argtypes = [S, P, P, P, P, ctypes.c_size_t, P]
    lib.msa_sparse_attn_backward_partials.argtypes = [S, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.msa_sparse_attn_backward_merge.argtypes = [S, P, P, P, P, P, ctypes.c_size_t, P]
    lib.msa_sparse_attn_backward.argtypes = [S, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.msa_decode_step_workspace_size.argtypes = [S, sz]
    lib.msa_decode_step.argtypes = [S, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.msa_decode_step_noalloc.argtypes = [S, P, P, P, P, P, P, P, P, P]
    for f in EXPORTS:
        if f == "msa_last_error":
            continue
        getattr(lib, f).restype = I
    lib.msa_last_error.restype = ctypes.c_char_p
    lib.msa_last_error.argtypes = []
    lib.msa_abi_version.argtypes = []
    _lib = lib
    return lib


def make_shape(batch, n_q, n_k, q_start, h_q, h_kv, d_h, d_idx, block_size, top_k, dtype,
               kv_capacity=0) -> MsaShape:
    dt = {"f32": MSA_F32, "bf16": MSA_BF16}.get(dtype, dtype)
    return MsaShape(batch, n_q, n_k, q_start, h_q, h_kv, d_h, d_idx, block_size, top_k, dt,
                    kv_capacity)


def shape_of(w, **over) -> MsaShape:
    """MsaShape for a workload object (block_sparse_gqa_msa_amd.inputs.Workload or alike)."""
    f = dict(batch=w.batch, n_q=w.n_q, n_k=w.n_k, q_start=w.q_start, h_q=w.h_q, h_kv=w.h_kv,
             d_h=w.d_h, d_idx=w.d_idx, block_size=w.block_size, top_k=w.top_k, dtype=w.dtype)
    f.update(over)
    return make_shape(**f)


def _elem_dtype(shape: MsaShape):
    import torch
    return torch.float32 if shape.dtype == MSA_F32 else torch.bfloat16


def _ptr(x, want=None, name="tensor"):
    """Device pointer of a contiguous GPU tensor (or pass through an int / None)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not x.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if want is not None and x.dtype != want:
        raise TypeError(f"{name} has dtype {x.dtype}, expected {want}")
    return x.data_ptr()


def _stream(stream, *tensors):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    for t in tensors:
        if t is not None and not isinstance(t, int):
            return torch.cuda.current_stream(t.device).cuda_stream
    return 0


def _check(rc: int):
    if rc != MSA_OK:
        raise MsaError(rc, load_library().msa_last_error().decode())


def _ws(workspace):
    if workspace is None:
        return None, 0
    if isinstance(workspace, tuple):
        return workspace
    return _ptr(workspace, name="workspace"), workspace.numel() * workspace.element_size()


# ----------------------------------------------------------------- C entry points

def msa_abi_version() -> int:
    return int(load_library().msa_abi_version())


def msa_last_error() -> str:
    return load_library().msa_last_error().decode()


def msa_index_topk_workspace_size(shape: MsaShape) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().msa_index_topk_workspace_size(ctypes.byref(shape), ctypes.byref(n)))
    return int(n.value)


def msa_sparse_attn_workspace_size(shape: MsaShape) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().msa_sparse_attn_workspace_size(ctypes.byref(shape), ctypes.byref(n)))
    return int(n.value)


def msa_index_topk(shape: MsaShape, q_idx, k_idx, sel, block_scores=None, workspace=None,
                   stream=None) -> None:
    import torch
    et = _elem_dtype(shape)
    wp, wn = _ws(workspace)
    _check(load_library().msa_index_topk(
        ctypes.byref(shape), _ptr(q_idx, et, "q_idx"), _ptr(k_idx, et, "k_idx"),
        _ptr(sel, torch.int32, "sel"), _ptr(block_scores, torch.float32, "block_scores"),
        wp, wn, _stream(stream, sel)))


def msa_index_topk_scores(shape: MsaShape, q_idx, k_idx, block_scores=None, workspace=None,
                          stream=None) -> None:
    import torch
    et = _elem_dtype(shape)
    wp, wn = _ws(workspace)
    _check(load_library().msa_index_topk_scores(
        ctypes.byref(shape), _ptr(q_idx, et, "q_idx"), _ptr(k_idx, et, "k_idx"),
        _ptr(block_scores, torch.float32, "block_scores"), wp, wn, _stream(stream, q_idx)))


def msa_index_topk_select(shape: MsaShape, sel, block_scores=None, workspace=None,
                          stream=None) -> None:
    import torch
    wp, wn = _ws(workspace)
    _check(load_library().msa_index_topk_select(
        ctypes.byref(shape), _ptr(block_scores, torch.float32, "block_scores"),
        _ptr(sel, torch.int32, "sel"), wp, wn, _stream(stream, sel)))


def msa_index_block_scores(shape: MsaShape, q_idx, k_idx, block_scores, stream=None) -> None:
    import torch
    et = _elem_dtype(shape)
    _check(load_library().msa_index_block_scores(
        ctypes.byref(shape), _ptr(q_idx, et, "q_idx"), _ptr(k_idx, et, "k_idx"),
        _ptr(block_scores, torch.float32, "block_scores"), _stream(stream, block_scores)))


def msa_topk_workspace_size(shape: MsaShape) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().msa_topk_workspace_size(ctypes.byref(shape), ctypes.byref(n)))
    return int(n.value)


def msa_topk_from_block_scores(shape: MsaShape, block_scores, sel, workspace=None,
                               stream=None) -> None:
    import torch
    wp, wn = _ws(workspace)
    _check(load_library().msa_topk_from_block_scores(
        ctypes.byref(shape), _ptr(block_scores, torch.float32, "block_scores"),
        _ptr(sel, torch.int32, "sel"), wp, wn, _stream(stream, sel)))


def msa_sparse_attn_prefill(shape: MsaShape, q, k, v, sel, o, lse=None, workspace=None,
                            stream=None) -> None:
    import torch
    et = _elem_dtype(shape)
    wp, wn = _ws(workspace)
    _check(load_library().msa_sparse_attn_prefill(
        ctypes.byref(shape), _ptr(q, et, "q"), _ptr(k, et, "k"), _ptr(v, et, "v"),
        _ptr(sel, torch.int32, "sel"), _ptr(o, et, "o"), _ptr(lse, torch.float32, "lse"),
        wp, wn, _stream(stream, o)))


def msa_sparse_attn_prefill_plan(shape: MsaShape, sel, workspace=None, stream=None) -> None:
    import torch
    wp, wn = _ws(workspace)
    _check(load_library().msa_sparse_attn_prefill_plan(
        ctypes.byref(shape), _ptr(sel, torch.int32, "sel"), wp, wn, _stream(stream, sel)))


def msa_sparse_attn_prefill_partials(shape: MsaShape, q, k, v, workspace=None,
                                     stream=None) -> None:
    et = _elem_dtype(shape)
    wp, wn = _ws(workspace)
    _check(load_library().msa_sparse_attn_prefill_partials(
        ctypes.byref(shape), _ptr(q, et, "q"), _ptr(k, et, "k"), _ptr(v, et, "v"), wp, wn,
        _stream(stream, q)))


def msa_sparse_attn_prefill_merge(shape: MsaShape, sel, o, lse=None, workspace=None,
                                  stream=None) -> None:
    import torch
    et = _elem_dtype(shape)
    wp, wn = _ws(workspace)
    _check(load_library().msa_sparse_attn_prefill_merge(
        ctypes.byref(shape), _ptr(sel, torch.int32, "sel"), _ptr(o, et, "o"),
        _ptr(lse, torch.float32, "lse"), wp, wn, _stream(stream, o)))


def msa_sparse_attn_decode(shape: MsaShape, q, k_cache, v_cache, sel, o, lse=None,
                           workspace=None, stream=None) -> None:
    import torch
    et = _elem_dtype(shape)
    wp, wn = _ws(workspace)
    _check(load_library().msa_sparse_attn_decode(
        ctypes.byref(shape), _ptr(q, et, "q"), _ptr(k_cache, et, "k_cache"),
        _ptr(v_cache, et, "v_cache"), _ptr(sel, torch.int32, "sel"), _ptr(o, et, "o"),
        _ptr(lse, torch.float32, "lse"), wp, wn, _stream(stream, o)))


def msa_decode_step_workspace_size(shape: MsaShape) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().msa_decode_step_workspace_size(ctypes.byref(shape), ctypes.byref(n)))
    return int(n.value)


def msa_decode_step(shape: MsaShape, q, k_cache, v_cache, q_idx, k_idx, sel, o, lse=None,
                    workspace=None, stream=None) -> None:
    import torch
    et = _elem_dtype(shape)
    wp, wn = _ws(workspace)
    _check(load_library().msa_decode_step(
        ctypes.byref(shape), _ptr(q, et, "q"), _ptr(k_cache, et, "k_cache"),
        _ptr(v_cache, et, "v_cache"), _ptr(q_idx, et, "q_idx"), _ptr(k_idx, et, "k_idx"),
        _ptr(sel, torch.int32, "sel"), _ptr(o, et, "o"), _ptr(lse, torch.float32, "lse"), wp, wn,
        _stream(stream, o)))


def msa_decode_step_noalloc(shape: MsaShape, q, k_cache, v_cache, q_idx, k_idx, sel, o, lse=None,
                            stream=None) -> None:
    """msa_decode_step on the library's own per-GPU scratch array (no workspace argument)."""
    import torch
    et = _elem_dtype(shape)
    _check(load_library().msa_decode_step_noalloc(
        ctypes.byref(shape), _ptr(q, et, "q"), _ptr(k_cache, et, "k_cache"),
        _ptr(v_cache, et, "v_cache"), _ptr(q_idx, et, "q_idx"), _ptr(k_idx, et, "k_idx"),
        _ptr(sel, torch.int32, "sel"), _ptr(o, et, "o"), _ptr(lse, torch.float32, "lse"),
        _stream(stream, o)))


def msa_index_kl(shape: MsaShape, q, k, q_idx, k_idx, sel, lse, kl, lse_idx=None,
                 workspace=None, stream=None) -> None:
    import torch
    et = _elem_dtype(shape)
    wp, wn = _ws(workspace)
    _check(load_library().msa_index_kl(
        ctypes.byref(shape), _ptr(q, et, "q"), _ptr(k, et, "k"), _ptr(q_idx, et, "q_idx"),
        _ptr(k_idx, et, "k_idx"), _ptr(sel, torch.int32, "sel"), _ptr(lse, torch.float32, "lse"),
        _ptr(kl, torch.float32, "kl"), _ptr(lse_idx, torch.float32, "lse_idx"), wp, wn,
        _stream(stream, kl)))


def msa_sparse_attn_backward_workspace_size(shape: MsaShape) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().msa_sparse_attn_backward_workspace_size(ctypes.byref(shape),
                                                                  ctypes.byref(n)))
    return int(n.value)


def msa_sparse_attn_backward(shape: MsaShape, q, k, v, sel, o, lse, dout, dq, dk, dv,
                             workspace=None, stream=None) -> None:
    import torch
    et = _elem_dtype(shape)
    wp, wn = _ws(workspace)
    _check(load_library().msa_sparse_attn_backward(
        ctypes.byref(shape), _ptr(q, et, "q"), _ptr(k, et, "k"), _ptr(v, et, "v"),
        _ptr(sel, torch.int32, "sel"), _ptr(o, et, "o"), _ptr(lse, torch.float32, "lse"),
        _ptr(dout, et, "dout"), _ptr(dq, et, "dq"), _ptr(dk, et, "dk"), _ptr(dv, et, "dv"),
        wp, wn, _stream(stream, dq)))


def msa_sparse_attn_backward_plan(shape: MsaShape, sel, o, dout, workspace=None,
                                  stream=None) -> None:
    import torch
    et = _elem_dtype(shape)
    wp, wn = _ws(workspace)
    _check(load_library().msa_sparse_attn_backward_plan(
        ctypes.byref(shape), _ptr(sel, torch.int32, "sel"), _ptr(o, et, "o"),
        _ptr(dout, et, "dout"), wp, wn, _stream(stream, dout)))


def msa_sparse_attn_backward_partials(shape: MsaShape, q, k, v, lse, dout, workspace=None,
                                      stream=None) -> None:
    import torch
    et = _elem_dtype(shape)
    wp, wn = _ws(workspace)
    _check(load_library().msa_sparse_attn_backward_partials(
        ctypes.byref(shape), _ptr(q, et, "q"), _ptr(k, et, "k"), _ptr(v, et, "v"),
        _ptr(lse, torch.float32, "lse"), _ptr(dout, et, "dout"), wp, wn, _stream(stream, q)))


def msa_sparse_attn_backward_merge(shape: MsaShape, sel, dq, dk, dv, workspace=None,
                                   stream=None) -> None:
    import torch
    et = _elem_dtype(shape)
    wp, wn = _ws(workspace)
    _check(load_library().msa_sparse_attn_backward_merge(
        ctypes.byref(shape), _ptr(sel, torch.int32, "sel"), _ptr(dq, et, "dq"),
        _ptr(dk, et, "dk"), _ptr(dv, et, "dv"), wp, wn, _stream(stream, dq)))


def msa_index_project(shape: MsaShape, x, w_qidx, w_kidx, q_idx, k_idx, stream=None) -> None:
    """x [B, n_q, d_model]; writes q_idx [B, h_kv, n_q, d_idx] and the k_idx cache rows
    q_start .. q_start + n_q - 1. d_model is taken from x."""
    et = _elem_dtype(shape)
    if x.dim() != 3:
        raise ValueError("x must be [batch, n_q, d_model]")
    _check(load_library().msa_index_project(
        ctypes.byref(shape), int(x.shape[-1]), _ptr(x, et, "x"), _ptr(w_qidx, et, "w_qidx"),
        _ptr(w_kidx, et, "w_kidx"), _ptr(q_idx, et, "q_idx"), _ptr(k_idx, et, "k_idx"),
        _stream(stream, q_idx)))


# ----------------------------------------------------------------- allocation helpers

class Buffers:
    """Output and workspace tensors for one MSA step of a given shape (allocated once, reused)."""

    def __init__(self, shape: MsaShape, device="cuda", block_scores=False, lse=True):
        import torch
        B, R, H, n = shape.batch, shape.h_kv, shape.h_q, shape.n_q
        nb = -(-shape.n_k // shape.block_size)
        self.shape = shape
        self.sel = torch.empty((B, R, n, shape.top_k), dtype=torch.int32, device=device)
        self.o = torch.empty((B, H, n, shape.d_h), dtype=_elem_dtype(shape), device=device)
        self.lse = torch.empty((B, H, n), dtype=torch.float32, device=device) if lse else None
        self.block_scores = (torch.empty((B, R, n, nb), dtype=torch.float32, device=device)
                             if block_scores else None)
        wi = msa_index_topk_workspace_size(shape)
        wa = msa_sparse_attn_workspace_size(shape)
        self.ws_index = torch.empty(max(wi, 1), dtype=torch.uint8, device=device)
        self.ws_attn = torch.empty(max(wa, 1), dtype=torch.uint8, device=device)
        self.decode = shape.n_q == 1 and shape.q_start == shape.n_k - 1


def msa_step(buf: Buffers, inputs, stream=None) -> Buffers:
    """One MSA step (index branch, then main branch) into ``buf``; decode shapes use the
    split decode path."""
    s = buf.shape
    msa_index_topk(s, inputs["q_idx"], inputs["k_idx"], buf.sel, buf.block_scores, buf.ws_index,
                   stream)
    attn = msa_sparse_attn_decode if buf.decode else msa_sparse_attn_prefill
    attn(s, inputs["q"], inputs["k"], inputs["v"], buf.sel, buf.o, buf.lse, buf.ws_attn, stream)
    return buf
