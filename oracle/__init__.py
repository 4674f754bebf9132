"""ctypes wrapper of the fp64 CPU oracle (oracle/msa_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, by __graft_entry__.smoke() and by
the CPU-baseline leg of bench.py, never by the library path. It shares no code
with the HIP path; both are fed by block_sparse_gqa_msa_amd.inputs only.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "msa_oracle.c")
LIB = os.path.join(HERE, "libmsa_oracle.so")


def build(src: str = SRC, out: str = LIB, extra_flags: Sequence[str] = ()) -> str:
    """Compile the oracle with gcc: -O2, OpenMP, no fast-math (IEEE double throughout)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math",
           "-ffp-contract=off", *extra_flags, src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


class Oracle:
    """A loaded oracle library (the default build, or a variant built from other source)."""

    def __init__(self, path: str = LIB):
        if not os.path.exists(path):
            build(out=path)
        self.lib = ctypes.CDLL(path)
        f = self.lib.msa_oracle_run
        i, p = ctypes.c_int, ctypes.c_void_p
        f.argtypes = [i] * 10 + [i, p, p, p, p, p, i, p, p, p, p, p, i]
        f.restype = i
        g = self.lib.msa_oracle_kl
        g.argtypes = [i] * 11 + [p, p, p, p, i, p, p, p, p, i]
        g.restype = i
        bw = self.lib.msa_oracle_attn_bwd
        bw.argtypes = [i] * 10 + [p, p, p, p, p, p, p, p, i]
        bw.restype = i
        pj = self.lib.msa_oracle_project
        pj.argtypes = [i] * 6 + [p, p, p, p, p, i]
        pj.restype = i
        self.lib.msa_oracle_max_threads.restype = i

    def max_threads(self) -> int:
        return int(self.lib.msa_oracle_max_threads())

    def run(self, w, inputs: Dict, rows: Optional[Sequence[int]] = None, attention: bool = True,
            block_scores: bool = False, n_threads: int = 0) -> Dict[str, np.ndarray]:
        """Run the oracle on workload ``w`` (a Workload or any object with the same fields).

        ``inputs`` maps q, k, v, q_idx, k_idx to CPU torch tensors or numpy arrays in the
        layouts of block_sparse_gqa_msa_amd.inputs (bf16 tensors are passed as raw bits).
        ``rows`` lists query rows (default: all). Returns sel [B,R,n,k] int32 and, as
        requested, block_scores [B,R,n,nb], o [B,H_q,n,d_h], lse [B,H_q,n] in float64.
        """
        rows_arr = np.arange(w.n_q, dtype=np.int32) if rows is None else np.asarray(rows, np.int32)
        rows_arr = np.ascontiguousarray(rows_arr)
        n = len(rows_arr)
        B, R, H, k = w.batch, w.h_kv, w.h_q, w.top_k
        nb = -(-w.n_k // w.block_size)
        typ = 0 if w.dtype == "f32" else 1
        keep = []

        def ptr(name):
            if name not in inputs or inputs[name] is None:
                return None
            a = _as_numpy(inputs[name], typ)
            keep.append(a)
            return a.ctypes.data

        sel = np.empty((B, R, n, k), np.int32)
        bm = np.empty((B, R, n, nb), np.float64) if block_scores else None
        o = np.empty((B, H, n, w.d_h), np.float64) if attention else None
        lse = np.empty((B, H, n), np.float64) if attention else None
        rc = self.lib.msa_oracle_run(
            B, w.n_q, w.n_k, w.q_start, H, R, w.d_h, w.d_idx, w.block_size, k, typ,
            ptr("q_idx"), ptr("k_idx"), ptr("q") if attention else None,
            ptr("k") if attention else None, ptr("v") if attention else None,
            n, rows_arr.ctypes.data, sel.ctypes.data,
            None if bm is None else bm.ctypes.data,
            None if o is None else o.ctypes.data,
            None if lse is None else lse.ctypes.data, int(n_threads))
        if rc != 0:
            raise RuntimeError(f"msa_oracle_run failed with code {rc}")
        out = dict(sel=sel)
        if bm is not None:
            out["block_scores"] = bm
        if attention:
            out["o"], out["lse"] = o, lse
        return out


    def kl(self, w, inputs: Dict, sel: np.ndarray, rows: Optional[Sequence[int]] = None,
           n_threads: int = 0) -> Dict[str, np.ndarray]:
        """The index-branch alignment loss L_KL and the student's normaliser lse_idx,
        [B, R, n] float64, for the listed rows (default: all) given their selections
        ``sel`` [B, R, n, k] (as ``run`` returns them for the same rows)."""
        rows_arr = np.arange(w.n_q, dtype=np.int32) if rows is None else np.asarray(rows, np.int32)
        rows_arr = np.ascontiguousarray(rows_arr)
        n = len(rows_arr)
        B, R, H, k = w.batch, w.h_kv, w.h_q, w.top_k
        typ = 0 if w.dtype == "f32" else 1
        arrs = {name: _as_numpy(inputs[name], typ) for name in ("q_idx", "k_idx", "q", "k")}
        sel = np.ascontiguousarray(sel, dtype=np.int32)
        if sel.shape != (B, R, n, k):
            raise ValueError(f"sel has shape {sel.shape}, expected {(B, R, n, k)}")
        kl = np.empty((B, R, n), np.float64)
        lse = np.empty((B, R, n), np.float64)
        rc = self.lib.msa_oracle_kl(
            B, w.n_q, w.n_k, w.q_start, H, R, w.d_h, w.d_idx, w.block_size, k, typ,
            arrs["q_idx"].ctypes.data, arrs["k_idx"].ctypes.data, arrs["q"].ctypes.data,
            arrs["k"].ctypes.data, n, rows_arr.ctypes.data, sel.ctypes.data, kl.ctypes.data,
            lse.ctypes.data, int(n_threads))
        if rc != 0:
            raise RuntimeError(f"msa_oracle_kl failed with code {rc}")
        return dict(kl=kl, lse_idx=lse)


    def attn_bwd(self, w, inputs: Dict, sel: np.ndarray, dout, n_threads: int = 0
                 ) -> Dict[str, np.ndarray]:
        """Gradients of the main branch for every row, given the selections ``sel``
        [B, R, n_q, k] (held fixed) and the output gradient ``dout`` [B, H_q, n_q, d_h] in
        the inputs' storage type: dq [B, H_q, n_q, d_h], dk and dv [B, R, n_k, d_h], float64."""
        B, R, H, k = w.batch, w.h_kv, w.h_q, w.top_k
        typ = 0 if w.dtype == "f32" else 1
        arrs = {name: _as_numpy(inputs[name], typ) for name in ("q", "k", "v")}
        do = _as_numpy(dout, typ)
        sel = np.ascontiguousarray(sel, dtype=np.int32)
        if sel.shape != (B, R, w.n_q, k):
            raise ValueError(f"sel has shape {sel.shape}, expected {(B, R, w.n_q, k)}")
        dq = np.empty((B, H, w.n_q, w.d_h), np.float64)
        dk = np.empty((B, R, w.n_k, w.d_h), np.float64)
        dv = np.empty((B, R, w.n_k, w.d_h), np.float64)
        rc = self.lib.msa_oracle_attn_bwd(
            B, w.n_q, w.n_k, w.q_start, H, R, w.d_h, w.block_size, k, typ,
            arrs["q"].ctypes.data, arrs["k"].ctypes.data, arrs["v"].ctypes.data,
            sel.ctypes.data, do.ctypes.data, dq.ctypes.data, dk.ctypes.data, dv.ctypes.data,
            int(n_threads))
        if rc != 0:
            raise RuntimeError(f"msa_oracle_attn_bwd failed with code {rc}")
        return dict(dq=dq, dk=dk, dv=dv)


    def project(self, x, w_q, w_k, h_kv: int, d_idx: int, n_threads: int = 0
                ) -> Dict[str, np.ndarray]:
        """The index branch's projections of hidden states ``x`` [B, n, d_model]:
        q_idx [B, h_kv, n, d_idx] = per group r, x w_q[r*d_idx:(r+1)*d_idx]^T, and
        k_idx [B, n, d_idx] = x w_k^T, float64. ``w_q`` [h_kv*d_idx, d_model] and ``w_k``
        [d_idx, d_model] share the storage type of ``x`` (fp32, or bf16 passed as raw bits)."""
        typ = 1 if _is_bf16(x) else 0
        xs, wq, wk = (_as_numpy(a, typ) for a in (x, w_q, w_k))
        B, n, dm = xs.shape
        if wq.shape != (h_kv * d_idx, dm) or wk.shape != (d_idx, dm):
            raise ValueError(f"weights {wq.shape}, {wk.shape} do not match x {xs.shape}")
        q = np.empty((B, h_kv, n, d_idx), np.float64)
        k = np.empty((B, n, d_idx), np.float64)
        rc = self.lib.msa_oracle_project(B, n, dm, h_kv, d_idx, typ, xs.ctypes.data,
                                         wq.ctypes.data, wk.ctypes.data, q.ctypes.data,
                                         k.ctypes.data, int(n_threads))
        if rc != 0:
            raise RuntimeError(f"msa_oracle_project failed with code {rc}")
        return dict(q_idx=q, k_idx=k)


def _is_bf16(x) -> bool:
    try:
        import torch
        return isinstance(x, torch.Tensor) and x.dtype == torch.bfloat16
    except ImportError:
        return False


def _as_numpy(x, typ: int) -> np.ndarray:
    """Contiguous numpy view of a CPU tensor/array: float32, or the raw uint16 bits of bf16."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().contiguous()
            if x.dtype == torch.bfloat16:
                if typ != 1:
                    raise TypeError("bf16 tensor passed for an fp32 workload")
                return x.view(torch.int16).numpy().view(np.uint16)
            if x.dtype != torch.float32 or typ != 0:
                raise TypeError(f"unexpected dtype {x.dtype}")
            return x.numpy()
    except ImportError:
        pass
    a = np.ascontiguousarray(x)
    want = np.float32 if typ == 0 else np.uint16
    if a.dtype != want:
        raise TypeError(f"expected {want}, got {a.dtype}")
    return a


_default: Optional[Oracle] = None


def get() -> Oracle:
    """The default oracle library (built on first use if missing)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default
