"""MSA forward oracle -- TEST INFRASTRUCTURE ONLY.

Python access to the plain fp64 CPU reference in ``msa_oracle.c``.  Only
the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline leg
may import this package; the GPU library never does, and the two share no
code.  Inputs are numpy arrays: bf16 tensors are passed as their uint16 bit
patterns.

What it computes follows the MiniMax Sparse Attention explainer
(minimax-sparse-attention-danialwang.pages.dev): Index Branch scores,
block max pooling and forced-local Top-k (Figure 1 caption; section 05,
part 1), the inverted block->query index (section 05, part 2) and exact
softmax attention over the selected blocks (section 02).
"""
from __future__ import annotations

from .frontend import index_frontend  # noqa: F401  (fp64 numpy, see frontend.py)

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "msa_oracle.c")
_LIB = os.path.join(_HERE, "libmsa_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain -O2, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-Wextra",
                               "-shared", "-fPIC", "-pthread", "-o", tmp, _SRC,
                               "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i64, i32, f64 = ctypes.c_int64, ctypes.c_int, ctypes.c_double
        lib.oracle_block_scores.argtypes = [P, P, i64, i32, i32, i32, i32, P]
        lib.oracle_block_scores.restype = None
        lib.oracle_select.argtypes = [P, P, P, i64, i32, i32, i32, i32, P, i32]
        lib.oracle_select.restype = None
        lib.oracle_attend.argtypes = [P, P, P, P, P, i64, i32, i32, i32, i32,
                                      i32, f64, P, P, i32]
        lib.oracle_attend.restype = None
        lib.oracle_invert.argtypes = [P, i64, i64, i32, i32, i64, P, P, P]
        lib.oracle_invert.restype = i64
        lib.oracle_attend_backward_dq_rows.argtypes = [P, P, P, P, P, P, i64, i32, i32, i32,
                                                       i32, i32, f64, P, i32]
        lib.oracle_attend_backward_dq_rows.restype = None
        lib.oracle_decode_one.argtypes = [P, P, P, P, P, i64, i32, i32, i32,
                                          i32, i32, i32, f64, P, P, P, i32]
        lib.oracle_decode_one.restype = None
        lib.oracle_index_kl.argtypes = [P, P, P, P, P, P, i64, i32, i32, i32, i32,
                                        i32, i32, f64, P, i32]
        lib.oracle_index_kl.restype = None
        lib.oracle_attend_backward.argtypes = [P, P, P, P, P, i64, i32, i32, i32, i32, i32,
                                               f64, P, P, P, i32]
        lib.oracle_attend_backward.restype = None
        _lib = lib
    return _lib


def threads() -> int:
    """Host threads the oracle uses: the cores this process may run on."""
    return len(os.sched_getaffinity(0))


def _u16(a):
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint16, a.dtype
    return a


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def block_scores(q_row, k_idx, i, r, B_k=128):
    """Pooled block scores P[0..lb(i)] of one query row and group (fp64).

    q_row: uint16 [H_kv, d_idx] (that row's index query); k_idx: uint16
    [Nk, H_kv, d_idx].
    """
    q_row, k_idx = _u16(q_row), _u16(k_idx)
    H_kv, d_idx = q_row.shape
    out = np.empty(i // B_k + 1, dtype=np.float64)
    _load().oracle_block_scores(_ptr(q_row), _ptr(k_idx), i, r, H_kv, d_idx,
                                B_k, _ptr(out))
    return out


def select(q_rows, k_idx, rows, k, B_k=128, nthreads=None):
    """Block selection for query positions ``rows``.

    q_rows: uint16 [nrows, H_kv, d_idx] (index queries of those rows);
    k_idx: uint16 [Nk, H_kv, d_idx].  Returns int32 [nrows, H_kv, k],
    ascending block ids, -1 padded.
    """
    q_rows, k_idx = _u16(q_rows), _u16(k_idx)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    nrows, H_kv, d_idx = q_rows.shape
    assert rows.shape == (nrows,) and (nrows == 0 or rows.max() < k_idx.shape[0])
    sel = np.empty((nrows, H_kv, k), dtype=np.int32)
    _load().oracle_select(_ptr(q_rows), _ptr(k_idx), _ptr(rows), nrows, H_kv,
                          d_idx, B_k, k, _ptr(sel), nthreads or threads())
    return sel


def attend(Q_rows, K, V, sel, rows, scale, B_k=128, nthreads=None):
    """Exact attention of the given rows over their selected blocks.

    Q_rows: uint16 [nrows, H_q, d_h]; K, V: uint16 [Nk, H_kv, d_h]; sel:
    int32 [nrows, H_kv, k].  Returns (O fp64 [nrows, H_q, d_h], lse fp64
    [nrows, H_q]).
    """
    Q_rows, K, V = _u16(Q_rows), _u16(K), _u16(V)
    sel = np.ascontiguousarray(sel, dtype=np.int32)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    nrows, H_q, d_h = Q_rows.shape
    H_kv = K.shape[1]
    k = sel.shape[2]
    assert sel.shape == (nrows, H_kv, k) and K.shape == V.shape
    O = np.empty((nrows, H_q, d_h), dtype=np.float64)
    lse = np.empty((nrows, H_q), dtype=np.float64)
    _load().oracle_attend(_ptr(Q_rows), _ptr(K), _ptr(V), _ptr(sel), _ptr(rows),
                          nrows, H_q, H_kv, d_h, B_k, k, float(scale), _ptr(O),
                          _ptr(lse), nthreads or threads())
    return O, lse


def invert(sel, q_start, nblk):
    """Inverted index of a selection table for positions q_start.. .

    sel: int32 [Nq, H_kv, k].  Returns (row_ptr int64 [H_kv*nblk+1], col
    int64 [nnz], slot int32 [nnz]).
    """
    sel = np.ascontiguousarray(sel, dtype=np.int32)
    Nq, H_kv, k = sel.shape
    cap = int((sel >= 0).sum())
    row_ptr = np.empty(H_kv * nblk + 1, dtype=np.int64)
    col = np.empty(max(cap, 1), dtype=np.int64)
    slot = np.empty(max(cap, 1), dtype=np.int32)
    nnz = _load().oracle_invert(_ptr(sel), q_start, Nq, H_kv, k, nblk,
                                _ptr(row_ptr), _ptr(col), _ptr(slot))
    assert nnz == cap
    return row_ptr, col[:nnz], slot[:nnz]


def index_kl(q_rows, k_idx, Q_rows, K, sel, rows, scale, B_k=128, nthreads=None):
    """Index-alignment KL(teacher || student) of each (row, group) over the
    tokens of its selection.

    q_rows: uint16 [nrows, H_kv, d_idx]; k_idx: uint16 [Nk, H_kv, d_idx];
    Q_rows: uint16 [nrows, H_q, d_h]; K: uint16 [Nk, H_kv, d_h]; sel: int32
    [nrows, H_kv, k].  Returns fp64 [nrows, H_kv].
    """
    q_rows, k_idx, Q_rows, K = _u16(q_rows), _u16(k_idx), _u16(Q_rows), _u16(K)
    sel = np.ascontiguousarray(sel, dtype=np.int32)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    nrows, H_kv, d_idx = q_rows.shape
    H_q, d_h = Q_rows.shape[1], Q_rows.shape[2]
    k = sel.shape[2]
    assert sel.shape == (nrows, H_kv, k) and Q_rows.shape[0] == nrows
    assert K.shape[1] == H_kv and k_idx.shape[1] == H_kv
    kl = np.empty((nrows, H_kv), dtype=np.float64)
    _load().oracle_index_kl(_ptr(q_rows), _ptr(k_idx), _ptr(Q_rows), _ptr(K), _ptr(sel),
                            _ptr(rows), nrows, H_q, H_kv, d_h, d_idx, B_k, k, float(scale),
                            _ptr(kl), nthreads or threads())
    return kl


def attend_backward(Q, K, V, dO, sel, scale, B_k=128, nthreads=None):
    """Main Branch gradients for every row 0..N-1 given the output gradient.

    Q, dO: uint16 [N, H_q, d_h]; K, V: uint16 [N, H_kv, d_h]; sel: int32
    [N, H_kv, k].  Returns (dQ [N, H_q, d_h], dK [N, H_kv, d_h],
    dV [N, H_kv, d_h]), fp64.
    """
    Q, K, V, dO = _u16(Q), _u16(K), _u16(V), _u16(dO)
    sel = np.ascontiguousarray(sel, dtype=np.int32)
    N, H_q, d_h = Q.shape
    H_kv = K.shape[1]
    k = sel.shape[2]
    assert dO.shape == Q.shape and K.shape == V.shape == (N, H_kv, d_h)
    assert sel.shape == (N, H_kv, k)
    dQ = np.empty((N, H_q, d_h), dtype=np.float64)
    dK = np.empty((N, H_kv, d_h), dtype=np.float64)
    dV = np.empty((N, H_kv, d_h), dtype=np.float64)
    _load().oracle_attend_backward(_ptr(Q), _ptr(K), _ptr(V), _ptr(dO), _ptr(sel), N, H_q,
                                   H_kv, d_h, B_k, k, float(scale), _ptr(dQ), _ptr(dK),
                                   _ptr(dV), nthreads or threads())
    return dQ, dK, dV


def attend_backward_dq_rows(Q_rows, K, V, dO_rows, sel_rows, rows, scale, B_k=128,
                            nthreads=None):
    """dQ of the given query rows only (no dK/dV), fp64.

    Q_rows, dO_rows: uint16 [R, H_q, d_h]; K, V: uint16 [Nk, H_kv, d_h];
    sel_rows: int32 [R, H_kv, k]; rows: their positions.
    """
    Q_rows, K, V, dO_rows = _u16(Q_rows), _u16(K), _u16(V), _u16(dO_rows)
    sel_rows = np.ascontiguousarray(sel_rows, dtype=np.int32)
    pos = np.ascontiguousarray(rows, dtype=np.int64)
    R, H_q, d_h = Q_rows.shape
    H_kv = K.shape[1]
    k = sel_rows.shape[2]
    assert dO_rows.shape == Q_rows.shape and sel_rows.shape == (R, H_kv, k) and pos.shape == (R,)
    assert pos.max() < K.shape[0]
    dQ = np.empty((R, H_q, d_h), dtype=np.float64)
    _load().oracle_attend_backward_dq_rows(_ptr(Q_rows), _ptr(K), _ptr(V), _ptr(dO_rows),
                                           _ptr(sel_rows), _ptr(pos), R, H_q, H_kv, d_h, B_k,
                                           k, float(scale), _ptr(dQ), nthreads or threads())
    return dQ


def decode_one(q, q_idx, K, V, k_idx, k, scale, B_k=128, nthreads=None):
    """Decode for one sequence whose query is the last cache row.

    q uint16 [H_q, d_h], q_idx [H_kv, d_idx], K/V [N, H_kv, d_h], k_idx
    [N, H_kv, d_idx].  Returns (sel [H_kv, k], O [H_q, d_h], lse [H_q]).
    """
    q, q_idx, K, V, k_idx = map(_u16, (q, q_idx, K, V, k_idx))
    N, H_kv, d_h = K.shape
    H_q = q.shape[0]
    d_idx = q_idx.shape[1]
    sel = np.empty((H_kv, k), dtype=np.int32)
    O = np.empty((H_q, d_h), dtype=np.float64)
    lse = np.empty(H_q, dtype=np.float64)
    _load().oracle_decode_one(_ptr(q), _ptr(q_idx), _ptr(K), _ptr(V), _ptr(k_idx),
                              N, H_q, H_kv, d_h, d_idx, B_k, k, float(scale),
                              _ptr(sel), _ptr(O), _ptr(lse), nthreads or threads())
    return sel, O, lse


def prefill_rows(inp, rows, k, scale, B_k=128, nthreads=None):
    """Select + attend for the given query rows of a prefill input dict
    (uint16 arrays Q, K, V, q_idx, k_idx).  Returns (sel, O, lse)."""
    rows = np.asarray(rows, dtype=np.int64)
    sel = select(inp["q_idx"][rows], inp["k_idx"], rows, k, B_k, nthreads)
    O, lse = attend(inp["Q"][rows], inp["K"], inp["V"], sel, rows, scale, B_k,
                    nthreads)
    return sel, O, lse
