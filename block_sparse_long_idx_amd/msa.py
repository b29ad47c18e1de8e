"""ctypes binding of libmsa (include/msa.h): argument marshalling only.

Every step of the MSA forward path runs in libmsa's HIP kernels; torch
supplies device memory (outputs and workspaces) and the current stream.
There is no CPU fallback: if libmsa.so is missing or no GPU is present the
calls raise.
"""
from __future__ import annotations

import ctypes
import math
import os
import re

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmsa.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "msa.h")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, -1, -2, -3, -4
OPT_INDEX_FUSED, OPT_ATTN_CHUNK = 1, 2
B_K = 128

_lib = None


class MsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"libmsa status {status}: {message}")
        self.status = status


def load():
    """Load libmsa.so (built in-tree by __graft_entry__.build())."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(LIB_PATH)
    P, i64, i32, sz, f32 = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                            ctypes.c_size_t, ctypes.c_float)
    sigs = {
        "msa_last_error": ([], ctypes.c_char_p),
        "msa_selection_nnz": ([i64, i64, i32, i32, i32], i64),
        "msa_index_topk_workspace_bytes": ([i64, i64, i32, i32, i32], sz),
        "msa_index_topk": ([P, P, i64, i64, i64, i32, i32, i32, i32, P, P, sz, P], i32),
        "msa_invert_index_workspace_bytes": ([i64, i64, i32, i32, i32], sz),
        "msa_invert_index": ([P, i64, i64, i32, i32, i32, P, P, P, P, sz, P], i32),
        "msa_sparse_attn_fwd_workspace_bytes": ([i64, i64, i32, i32, i32, i32, i32], sz),
        "msa_sparse_attn_fwd": ([P, P, P, P, P, P, i64, i64, i64, i32, i32, i32, i32,
                                 i32, f32, P, P, P, sz, P], i32),
        "msa_prefill_workspace_bytes": ([i64, i64, i32, i32, i32, i32, i32, i32], sz),
        "msa_prefill": ([P, P, P, P, P, i64, i64, i32, i32, i32, i32, i32, i32, f32, P,
                         P, P, P, sz, P], i32),
        "msa_decode_workspace_bytes": ([i32, i64, i32, i32, i32, i32, i32, i32], sz),
        "msa_decode": ([P, P, P, P, P, i32, i64, i32, i32, i32, i32, i32, i32, f32, P, P,
                        P, P, sz, P], i32),
        "msa_index_kl_workspace_bytes": ([i64, i64, i32, i32, i32], sz),
        "msa_index_kl": ([P, P, P, P, P, P, P, P, i64, i64, i64, i32, i32, i32, i32, i32,
                          i32, f32, P, P, P, sz, P], i32),
        "msa_prefill_cached_workspace_bytes": ([i64, i64, i64, i32, i32, i32, i32, i32, i32],
                                               sz),
        "msa_prefill_cached": ([P, P, P, P, P, i64, i64, i64, i32, i32, i32, i32, i32, i32,
                                f32, P, P, P, P, sz, P], i32),
        "msa_prefill_varlen_workspace_bytes": ([P, i32, i64, i32, i32, i32, i32, i32, i32], sz),
        "msa_prefill_varlen": ([P, P, P, P, P, P, i32, i64, i32, i32, i32, i32, i32, i32, f32,
                                P, P, P, P, sz, P], i32),
        "msa_index_frontend": ([P, P, P, P, P, i64, i64, i32, i32, i32, i32, f32, f32, P, P,
                                P], i32),
        "msa_sparse_attn_bwd_workspace_bytes": ([i64, i64, i32, i32, i32, i32, i32], sz),
        "msa_sparse_attn_bwd": ([P, P, P, P, P, P, P, P, P, i64, i64, i64, i32, i32, i32,
                                 i32, i32, f32, P, P, P, P, sz, P], i32),
        "msa_decode_static_scratch_bytes": ([], sz),
        "msa_decode_static": ([P, P, P, P, P, i32, i64, i32, i32, i32, i32, i32, i32, f32, P,
                               P, P, P], i32),
        "msa_set_option": ([i32, i64], i32),
        "msa_get_option": ([i32], i64),
    }
    for name, (args, res) in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def header_functions():
    """Names of the functions declared in include/msa.h."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(msa_[a-z_]+)\s*\(", text)))


def _check(status: int):
    if status != OK:
        raise MsaError(status, load().msa_last_error().decode())


def _ptr(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _need_cuda(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("libmsa works on GPU tensors only")
            if not t.is_contiguous():
                raise ValueError("tensors must be contiguous")


def _expect(name, t, dtype, shape, min_rows=None):
    """Raise ValueError unless tensor `t` has this dtype and rank, the sizes
    in `shape` (None = any) and at least `min_rows` leading rows.  The
    library reads rows by position, so a short tensor would be read past
    its end on the device."""
    if t is None:
        return
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if t.dim() != len(shape) or any(e is not None and a != e for a, e in zip(t.shape, shape)):
        want = "[" + ", ".join("*" if e is None else str(e) for e in shape) + "]"
        raise ValueError(f"{name} has shape {list(t.shape)}, expected {want}")
    if min_rows is not None and t.shape[0] < min_rows:
        raise ValueError(f"{name} has {t.shape[0]} rows, needs at least {min_rows}")


def _expect_csr(row_ptr, col, slot, q_start, Nq, H_kv, k, B_k):
    nblk = (q_start + Nq + B_k - 1) // B_k
    nnz = load().msa_selection_nnz(q_start, Nq, H_kv, B_k, k)
    _expect("row_ptr", row_ptr, torch.int32, (None,), H_kv * nblk + 1)
    _expect("col", col, torch.int32, (None,), nnz)
    _expect("slot", slot, torch.uint8, (None,), nnz)


def _workspace(nbytes, device):
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def set_option(option: int, value: int):
    _check(load().msa_set_option(option, value))


def get_option(option: int) -> int:
    return load().msa_get_option(option)


def selection_nnz(q_start, Nq, H_kv, k, B_k=B_K) -> int:
    return load().msa_selection_nnz(q_start, Nq, H_kv, B_k, k)


def index_topk(q_idx, k_idx, k, q_start=0, Nq=None, B_k=B_K, sel=None, ws=None):
    """Index Branch for query rows [q_start, q_start+Nq): returns sel int32
    [Nq, H_kv, k].  q_idx/k_idx: bf16 [N, H_kv, d_idx] on the GPU."""
    _need_cuda(q_idx, k_idx, sel)
    N, H_kv, d_idx = k_idx.shape
    Nq = q_idx.shape[0] - q_start if Nq is None else Nq
    _expect("k_idx", k_idx, torch.bfloat16, (None, H_kv, d_idx), q_start + Nq)
    _expect("q_idx", q_idx, torch.bfloat16, (None, H_kv, d_idx), q_start + Nq)
    _expect("sel", sel, torch.int32, (Nq, H_kv, k))
    lib = load()
    if sel is None:
        sel = torch.empty((Nq, H_kv, k), dtype=torch.int32, device=k_idx.device)
    need = lib.msa_index_topk_workspace_bytes(q_start, Nq, H_kv, B_k, k)
    if ws is None:
        ws = _workspace(need, k_idx.device)
    _check(lib.msa_index_topk(_ptr(q_idx), _ptr(k_idx), q_start, Nq, N, H_kv, d_idx, B_k,
                              k, _ptr(sel), _ptr(ws), ws.numel(), _stream(k_idx)))
    return sel


def invert_index(sel, q_start=0, B_k=B_K, ws=None, row_ptr=None, col=None, slot=None):
    """Inverted index of sel [Nq, H_kv, k]: (row_ptr, col int32, slot uint8).
    Preallocated outputs may be passed (col/slot with >= nnz entries)."""
    _need_cuda(sel, row_ptr, col, slot)
    _expect("sel", sel, torch.int32, (None, None, None))
    Nq, H_kv, k = sel.shape
    _expect("row_ptr", row_ptr, torch.int32, (None,))
    _expect("col", col, torch.int32, (None,))
    _expect("slot", slot, torch.uint8, (None,))
    lib = load()
    nblk = (q_start + Nq + B_k - 1) // B_k
    nnz = lib.msa_selection_nnz(q_start, Nq, H_kv, B_k, k)
    dev = sel.device
    if row_ptr is None:
        row_ptr = torch.empty(H_kv * nblk + 1, dtype=torch.int32, device=dev)
    if col is None:
        col = torch.empty(max(nnz, 1), dtype=torch.int32, device=dev)
    if slot is None:
        slot = torch.empty(max(nnz, 1), dtype=torch.uint8, device=dev)
    if row_ptr.numel() < H_kv * nblk + 1 or col.numel() < nnz or slot.numel() < nnz:
        raise ValueError("preallocated inverted-index outputs are too small")
    need = lib.msa_invert_index_workspace_bytes(q_start, Nq, H_kv, B_k, k)
    if ws is None:
        ws = _workspace(need, dev)
    _check(lib.msa_invert_index(_ptr(sel), q_start, Nq, H_kv, B_k, k, _ptr(row_ptr),
                                _ptr(col), _ptr(slot), _ptr(ws), ws.numel(), _stream(sel)))
    return row_ptr, col[:nnz], slot[:nnz]


def sparse_attn_fwd(Q, K, V, row_ptr, col, slot, k, q_start=0, Nq=None, scale=None,
                    B_k=B_K, want_lse=True, O=None, lse=None, ws=None):
    """Main Branch for query rows [q_start, q_start+Nq): (O fp32, lse fp32)."""
    _need_cuda(Q, K, V, row_ptr, col, slot, O, lse)
    Nk, H_kv, d_h = K.shape
    H_q = Q.shape[1]
    Nq = Q.shape[0] - q_start if Nq is None else Nq
    _expect("K", K, torch.bfloat16, (None, H_kv, d_h), q_start + Nq)
    _expect("V", V, torch.bfloat16, (Nk, H_kv, d_h))
    _expect("Q", Q, torch.bfloat16, (None, H_q, d_h), q_start + Nq)
    _expect_csr(row_ptr, col, slot, q_start, Nq, H_kv, k, B_k)
    _expect("O", O, torch.float32, (Nq, H_q, d_h))
    _expect("lse", lse, torch.float32, (Nq, H_q))
    scale = 1.0 / math.sqrt(d_h) if scale is None else scale
    lib = load()
    dev = Q.device
    if O is None:
        O = torch.empty((Nq, H_q, d_h), dtype=torch.float32, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((Nq, H_q), dtype=torch.float32, device=dev)
    need = lib.msa_sparse_attn_fwd_workspace_bytes(q_start, Nq, H_q, H_kv, d_h, B_k, k)
    if ws is None:
        ws = _workspace(need, dev)
    _check(lib.msa_sparse_attn_fwd(_ptr(Q), _ptr(K), _ptr(V), _ptr(row_ptr), _ptr(col),
                                   _ptr(slot), q_start, Nq, Nk, H_q, H_kv, d_h, B_k, k,
                                   scale, _ptr(O), _ptr(lse), _ptr(ws), ws.numel(),
                                   _stream(Q)))
    return O, lse


def sparse_attn_bwd(Q, K, V, O, lse, dO, row_ptr, col, slot, k, q_start=0, Nq=None,
                    scale=None, B_k=B_K, dQ=None, dK=None, dV=None, ws=None):
    """Main Branch backward for rows [q_start, q_start+Nq): returns (dQ, dK, dV).
    dK and dV are added to (fresh zero tensors when not given)."""
    _need_cuda(Q, K, V, O, lse, dO, row_ptr, col, slot, dQ, dK, dV)
    Nk, H_kv, d_h = K.shape
    H_q = Q.shape[1]
    Nq = Q.shape[0] - q_start if Nq is None else Nq
    _expect("K", K, torch.bfloat16, (None, H_kv, d_h), q_start + Nq)
    _expect("V", V, torch.bfloat16, (Nk, H_kv, d_h))
    _expect("Q", Q, torch.bfloat16, (None, H_q, d_h), q_start + Nq)
    _expect("O", O, torch.float32, (Nq, H_q, d_h))
    _expect("lse", lse, torch.float32, (Nq, H_q))
    _expect("dO", dO, torch.bfloat16, (Nq, H_q, d_h))
    _expect_csr(row_ptr, col, slot, q_start, Nq, H_kv, k, B_k)
    _expect("dQ", dQ, torch.float32, (Nq, H_q, d_h))
    _expect("dK", dK, torch.float32, (Nk, H_kv, d_h))
    _expect("dV", dV, torch.float32, (Nk, H_kv, d_h))
    scale = 1.0 / math.sqrt(d_h) if scale is None else scale
    lib = load()
    dev = Q.device
    if dQ is None:
        dQ = torch.empty((Nq, H_q, d_h), dtype=torch.float32, device=dev)
    if dK is None:
        dK = torch.zeros((Nk, H_kv, d_h), dtype=torch.float32, device=dev)
    if dV is None:
        dV = torch.zeros((Nk, H_kv, d_h), dtype=torch.float32, device=dev)
    if ws is None:
        ws = _workspace(lib.msa_sparse_attn_bwd_workspace_bytes(q_start, Nq, H_q, H_kv, d_h,
                                                                B_k, k), dev)
    _check(lib.msa_sparse_attn_bwd(_ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(lse), _ptr(dO),
                                   _ptr(row_ptr), _ptr(col), _ptr(slot), q_start, Nq, Nk, H_q,
                                   H_kv, d_h, B_k, k, scale, _ptr(dQ), _ptr(dK), _ptr(dV),
                                   _ptr(ws), ws.numel(), _stream(Q)))
    return dQ, dK, dV


def prefill_cached(Q, K, V, q_idx, k_idx, k, q_start, chunk=0, scale=None, B_k=B_K,
                   sel=None, O=None, lse=None, want_lse=True, ws=None):
    """Chunked prefill against a KV cache: Q/q_idx hold the Nq new tokens
    (positions q_start..), K/V/k_idx the cache with them appended.
    Returns (sel, O, lse) for the new tokens."""
    _need_cuda(Q, K, V, q_idx, k_idx, sel, O, lse)
    Nq, H_q, d_h = Q.shape
    H_kv, d_idx = k_idx.shape[1], k_idx.shape[2]
    if K.shape[0] < q_start + Nq or k_idx.shape[0] < q_start + Nq:
        raise ValueError("the cache must hold q_start + Nq keys")
    _expect("Q", Q, torch.bfloat16, (Nq, H_q, d_h))
    _expect("K", K, torch.bfloat16, (None, H_kv, d_h))
    _expect("V", V, torch.bfloat16, tuple(K.shape))
    _expect("q_idx", q_idx, torch.bfloat16, (Nq, H_kv, d_idx))
    _expect("k_idx", k_idx, torch.bfloat16, (None, H_kv, d_idx))
    _expect("sel", sel, torch.int32, (Nq, H_kv, k))
    _expect("O", O, torch.float32, (Nq, H_q, d_h))
    _expect("lse", lse, torch.float32, (Nq, H_q))
    scale = 1.0 / math.sqrt(d_h) if scale is None else scale
    lib = load()
    dev = Q.device
    if sel is None:
        sel = torch.empty((Nq, H_kv, k), dtype=torch.int32, device=dev)
    if O is None:
        O = torch.empty((Nq, H_q, d_h), dtype=torch.float32, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((Nq, H_q), dtype=torch.float32, device=dev)
    if ws is None:
        ws = _workspace(lib.msa_prefill_cached_workspace_bytes(q_start, Nq, chunk, H_q, H_kv,
                                                               d_h, d_idx, B_k, k), dev)
    _check(lib.msa_prefill_cached(_ptr(Q), _ptr(K), _ptr(V), _ptr(q_idx), _ptr(k_idx), q_start,
                                  Nq, chunk, H_q, H_kv, d_h, d_idx, B_k, k, scale, _ptr(sel),
                                  _ptr(O), _ptr(lse), _ptr(ws), ws.numel(), _stream(Q)))
    return sel, O, lse


def prefill_varlen(Q, K, V, q_idx, k_idx, cu_seqlens, k, chunk=0, scale=None, B_k=B_K,
                   sel=None, O=None, lse=None, want_lse=True, ws=None):
    """Varlen batched prefill of packed sequences; cu_seqlens is a host
    sequence of B+1 prefix sums.  Returns (sel, O, lse) for all tokens."""
    _need_cuda(Q, K, V, q_idx, k_idx, sel, O, lse)
    T, H_q, d_h = Q.shape
    H_kv, d_idx = k_idx.shape[1], k_idx.shape[2]
    _expect("Q", Q, torch.bfloat16, (T, H_q, d_h))
    _expect("K", K, torch.bfloat16, (T, H_kv, d_h))
    _expect("V", V, torch.bfloat16, (T, H_kv, d_h))
    _expect("q_idx", q_idx, torch.bfloat16, (T, H_kv, d_idx))
    _expect("k_idx", k_idx, torch.bfloat16, (T, H_kv, d_idx))
    _expect("sel", sel, torch.int32, (T, H_kv, k))
    _expect("O", O, torch.float32, (T, H_q, d_h))
    _expect("lse", lse, torch.float32, (T, H_q))
    cu = (ctypes.c_int64 * len(cu_seqlens))(*[int(x) for x in cu_seqlens])
    B = len(cu_seqlens) - 1
    if int(cu_seqlens[-1]) != T:
        raise ValueError("cu_seqlens[-1] must equal the number of packed tokens")
    scale = 1.0 / math.sqrt(d_h) if scale is None else scale
    lib = load()
    dev = Q.device
    if sel is None:
        sel = torch.empty((T, H_kv, k), dtype=torch.int32, device=dev)
    if O is None:
        O = torch.empty((T, H_q, d_h), dtype=torch.float32, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((T, H_q), dtype=torch.float32, device=dev)
    if ws is None:
        ws = _workspace(lib.msa_prefill_varlen_workspace_bytes(cu, B, chunk, H_q, H_kv, d_h,
                                                               d_idx, B_k, k), dev)
    _check(lib.msa_prefill_varlen(_ptr(Q), _ptr(K), _ptr(V), _ptr(q_idx), _ptr(k_idx), cu, B,
                                  chunk, H_q, H_kv, d_h, d_idx, B_k, k, scale, _ptr(sel),
                                  _ptr(O), _ptr(lse), _ptr(ws), ws.numel(), _stream(Q)))
    return sel, O, lse


def index_frontend(hidden, Wq, Wk, gq, gk, H_kv, d_idx, pos0=0, rope_dim=64,
                   rope_theta=10000.0, eps=1e-6, q_idx=None, k_idx=None):
    """Index Branch front-end: hidden [N, d_model] bf16 -> (q_idx, k_idx)
    [N, H_kv, d_idx] bf16 by linear projection, per-group RMS norm and RoPE
    over the first rope_dim entries at positions pos0 + i."""
    _need_cuda(hidden, Wq, Wk, gq, gk, q_idx, k_idx)
    _expect("hidden", hidden, torch.bfloat16, (None, None))
    N, d_model = hidden.shape
    _expect("Wq", Wq, torch.bfloat16, (H_kv * d_idx, d_model))
    _expect("Wk", Wk, torch.bfloat16, (H_kv * d_idx, d_model))
    _expect("gq", gq, torch.float32, (d_idx,))
    _expect("gk", gk, torch.float32, (d_idx,))
    _expect("q_idx", q_idx, torch.bfloat16, (N, H_kv, d_idx))
    _expect("k_idx", k_idx, torch.bfloat16, (N, H_kv, d_idx))
    dev = hidden.device
    if q_idx is None:
        q_idx = torch.empty((N, H_kv, d_idx), dtype=torch.bfloat16, device=dev)
    if k_idx is None:
        k_idx = torch.empty((N, H_kv, d_idx), dtype=torch.bfloat16, device=dev)
    _check(load().msa_index_frontend(_ptr(hidden), _ptr(Wq), _ptr(Wk), _ptr(gq), _ptr(gk), N,
                                     pos0, d_model, H_kv, d_idx, min(rope_dim, d_idx),
                                     rope_theta, eps, _ptr(q_idx), _ptr(k_idx), _stream(hidden)))
    return q_idx, k_idx


def index_kl_workspace_bytes(q_start, Nq, H_kv, k, B_k=B_K) -> int:
    return load().msa_index_kl_workspace_bytes(q_start, Nq, H_kv, B_k, k)


def index_kl(Q, K, q_idx, k_idx, lse, row_ptr, col, slot, k, q_start=0, Nq=None, scale=None,
             B_k=B_K, want_sum=True, kl=None, kl_sum=None, ws=None):
    """Index-alignment KL(teacher || student) per (query, group) for rows
    [q_start, q_start+Nq): (kl fp32 [Nq, H_kv], kl_sum fp64 [1] or None).
    `lse` is the Main Branch's [Nq, H_q] output for the same rows."""
    _need_cuda(Q, K, q_idx, k_idx, lse, row_ptr, col, slot, kl, kl_sum)
    Nk, H_kv, d_h = K.shape
    H_q = Q.shape[1]
    d_idx = k_idx.shape[2]
    Nq = Q.shape[0] - q_start if Nq is None else Nq
    _expect("K", K, torch.bfloat16, (None, H_kv, d_h), q_start + Nq)
    _expect("Q", Q, torch.bfloat16, (None, H_q, d_h), q_start + Nq)
    _expect("q_idx", q_idx, torch.bfloat16, (None, H_kv, d_idx), q_start + Nq)
    _expect("k_idx", k_idx, torch.bfloat16, (None, H_kv, d_idx), Nk)
    _expect("lse", lse, torch.float32, (Nq, H_q))
    _expect_csr(row_ptr, col, slot, q_start, Nq, H_kv, k, B_k)
    _expect("kl", kl, torch.float32, (Nq, H_kv))
    _expect("kl_sum", kl_sum, torch.float64, (None,), 1)
    scale = 1.0 / math.sqrt(d_h) if scale is None else scale
    lib = load()
    dev = Q.device
    if kl is None:
        kl = torch.empty((Nq, H_kv), dtype=torch.float32, device=dev)
    if kl_sum is None and want_sum:
        kl_sum = torch.empty(1, dtype=torch.float64, device=dev)
    if ws is None:
        ws = _workspace(lib.msa_index_kl_workspace_bytes(q_start, Nq, H_kv, B_k, k), dev)
    _check(lib.msa_index_kl(_ptr(Q), _ptr(K), _ptr(q_idx), _ptr(k_idx), _ptr(lse),
                            _ptr(row_ptr), _ptr(col), _ptr(slot), q_start, Nq, Nk, H_q, H_kv,
                            d_h, d_idx, B_k, k, scale, _ptr(kl), _ptr(kl_sum), _ptr(ws),
                            ws.numel(), _stream(Q)))
    return kl, kl_sum


def prefill_workspace_bytes(N, H_q, H_kv, d_h, d_idx, k, chunk=0, B_k=B_K) -> int:
    return load().msa_prefill_workspace_bytes(N, chunk, H_q, H_kv, d_h, d_idx, B_k, k)


def prefill(Q, K, V, q_idx, k_idx, k, scale=None, chunk=0, B_k=B_K, want_sel=True,
            want_lse=True, sel=None, O=None, lse=None, ws=None):
    """Whole prefill over query chunks: (sel, O, lse)."""
    _need_cuda(Q, K, V, q_idx, k_idx, sel, O, lse)
    N, H_q, d_h = Q.shape
    H_kv, d_idx = k_idx.shape[1], k_idx.shape[2]
    _expect("Q", Q, torch.bfloat16, (N, H_q, d_h))
    _expect("K", K, torch.bfloat16, (N, H_kv, d_h))
    _expect("V", V, torch.bfloat16, (N, H_kv, d_h))
    _expect("q_idx", q_idx, torch.bfloat16, (N, H_kv, d_idx))
    _expect("k_idx", k_idx, torch.bfloat16, (N, H_kv, d_idx))
    _expect("sel", sel, torch.int32, (N, H_kv, k))
    _expect("O", O, torch.float32, (N, H_q, d_h))
    _expect("lse", lse, torch.float32, (N, H_q))
    scale = 1.0 / math.sqrt(d_h) if scale is None else scale
    lib = load()
    dev = Q.device
    if sel is None and want_sel:
        sel = torch.empty((N, H_kv, k), dtype=torch.int32, device=dev)
    if O is None:
        O = torch.empty((N, H_q, d_h), dtype=torch.float32, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((N, H_q), dtype=torch.float32, device=dev)
    if ws is None:
        ws = _workspace(lib.msa_prefill_workspace_bytes(N, chunk, H_q, H_kv, d_h, d_idx,
                                                        B_k, k), dev)
    _check(lib.msa_prefill(_ptr(Q), _ptr(K), _ptr(V), _ptr(q_idx), _ptr(k_idx), N, chunk,
                           H_q, H_kv, d_h, d_idx, B_k, k, scale, _ptr(sel), _ptr(O),
                           _ptr(lse), _ptr(ws), ws.numel(), _stream(Q)))
    return sel, O, lse


def decode_workspace_bytes(B, N, H_q, H_kv, d_h, d_idx, k, B_k=B_K) -> int:
    return load().msa_decode_workspace_bytes(B, N, H_q, H_kv, d_h, d_idx, B_k, k)


def decode_static(q, q_idx, K, V, k_idx, k, sel, O, lse=None, scale=None, B_k=B_K):
    """Decode step through msa_decode_static: no workspace, no allocation.
    The caller passes every output (sel int32 [B, H_kv, k], O fp32
    [B, H_q, d_h], lse fp32 [B, H_q] or None)."""
    _need_cuda(q, q_idx, K, V, k_idx, sel, O, lse)
    B, N, H_kv, d_h = K.shape
    H_q = q.shape[1]
    d_idx = k_idx.shape[3]
    _expect("K", K, torch.bfloat16, (B, N, H_kv, d_h))
    _expect("V", V, torch.bfloat16, (B, N, H_kv, d_h))
    _expect("k_idx", k_idx, torch.bfloat16, (B, N, H_kv, d_idx))
    _expect("q", q, torch.bfloat16, (B, H_q, d_h))
    _expect("q_idx", q_idx, torch.bfloat16, (B, H_kv, d_idx))
    _expect("sel", sel, torch.int32, (B, H_kv, k))
    _expect("O", O, torch.float32, (B, H_q, d_h))
    _expect("lse", lse, torch.float32, (B, H_q))
    scale = 1.0 / math.sqrt(d_h) if scale is None else scale
    _check(load().msa_decode_static(_ptr(q), _ptr(q_idx), _ptr(K), _ptr(V), _ptr(k_idx), B, N,
                                    H_q, H_kv, d_h, d_idx, B_k, k, scale, _ptr(sel), _ptr(O),
                                    _ptr(lse), _stream(q)))
    return sel, O, lse


def decode(q, q_idx, K, V, k_idx, k, scale=None, B_k=B_K, want_lse=True, sel=None,
           O=None, lse=None, ws=None):
    """Decode step for B sequences (query = last cache row): (sel, O, lse)."""
    _need_cuda(q, q_idx, K, V, k_idx, sel, O, lse)
    B, N, H_kv, d_h = K.shape
    H_q = q.shape[1]
    d_idx = k_idx.shape[3]
    _expect("K", K, torch.bfloat16, (B, N, H_kv, d_h))
    _expect("V", V, torch.bfloat16, (B, N, H_kv, d_h))
    _expect("k_idx", k_idx, torch.bfloat16, (B, N, H_kv, d_idx))
    _expect("q", q, torch.bfloat16, (B, H_q, d_h))
    _expect("q_idx", q_idx, torch.bfloat16, (B, H_kv, d_idx))
    _expect("sel", sel, torch.int32, (B, H_kv, k))
    _expect("O", O, torch.float32, (B, H_q, d_h))
    _expect("lse", lse, torch.float32, (B, H_q))
    scale = 1.0 / math.sqrt(d_h) if scale is None else scale
    lib = load()
    dev = q.device
    if sel is None:
        sel = torch.empty((B, H_kv, k), dtype=torch.int32, device=dev)
    if O is None:
        O = torch.empty((B, H_q, d_h), dtype=torch.float32, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((B, H_q), dtype=torch.float32, device=dev)
    if ws is None:
        ws = _workspace(lib.msa_decode_workspace_bytes(B, N, H_q, H_kv, d_h, d_idx, B_k, k),
                        dev)
    _check(lib.msa_decode(_ptr(q), _ptr(q_idx), _ptr(K), _ptr(V), _ptr(k_idx), B, N, H_q,
                          H_kv, d_h, d_idx, B_k, k, scale, _ptr(sel), _ptr(O), _ptr(lse),
                          _ptr(ws), ws.numel(), _stream(q)))
    return sel, O, lse
