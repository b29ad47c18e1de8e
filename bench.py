#!/usr/bin/env python3
"""MSA forward benchmark on one MI355X.

One step = the whole MSA prefill of a synthetic sequence (the fused Index
Branch over all queries in one launch, then the inverted index and the
KV-outer Main Branch per query chunk), with all inputs resident in HBM.  Default workload: N = 1,048,576 tokens, 64 query
heads, 4 KV heads, d_h 128, d_idx 64, k 16, B_k 128, query chunks of 65,536.

Prints one JSON line: prefill tokens/s (value), effective TFLOP/s by the
MSA FLOP formula 4*H_q*d_h*N*k*B_k + H_kv*d_idx*N^2 (as a fraction of the
2.5 PFLOP/s bf16 MFMA peak), per-stage times, the roofline of the dominant
kernel, the CPU oracle timed on sampled rows, and the index-alignment KL
pass, Main Branch backward, cached and varlen prefill, index front-end,
128K-prefill and 32 x 1M decode figures.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def formula_flops(cfg):
    """MSA attention FLOPs: Main 4*H_q*d_h*N*k*B_k + Index H_kv*d_idx*N^2."""
    main = 4.0 * cfg.H_q * cfg.d_h * cfg.N * cfg.k * cfg.B_k
    index = float(cfg.H_kv) * cfg.d_idx * cfg.N * cfg.N
    return main, index


def stored_traffic(kernel):
    """HBM bytes per launch of `kernel` measured with rocprofv3 FETCH_SIZE /
    WRITE_SIZE (calibrated on a plain copy), from profiles/; None once the
    kernel's sources differ from the ones that were profiled."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "prefill_1m_hbm_traffic.md")
    srcs = [os.path.join(ROOT, "block_sparse_long_idx_amd", "csrc", f)
            for f in ("index_topk.hip", "common.h")]
    try:
        h = hashlib.sha256()
        for f in srcs:
            with open(f, "rb") as fh:
                h.update(fh.read())
        with open(path) as fh:
            for line in fh:
                parts = line.split()
                if len(parts) >= 5 and parts[0] == "traffic" and parts[1] == kernel:
                    kv = dict(x.split("=") for x in parts[2:])
                    if kv["sources"] != h.hexdigest()[:16] or kv.get("launch") != "whole":
                        return None
                    return float(kv["fetch_bytes"]) + float(kv["write_bytes"])
    except OSError:
        return None
    return None


def chunks_of(cfg):
    c = cfg.chunk or cfg.N
    return [(q0, min(c, cfg.N - q0)) for q0 in range(0, cfg.N, c)]


class Prefill:
    """Preallocated buffers and the per-chunk call sequence of one step."""

    def __init__(self, cfg, t, whole_index=True):
        import torch
        from block_sparse_long_idx_amd import msa
        self.cfg, self.t, self.msa = cfg, t, msa
        dev = t["Q"].device
        lib = msa.load()
        self.chunks = chunks_of(cfg)
        ws_i = ws_v = ws_a = nnz = 0
        for q0, nq in self.chunks:
            ws_i = max(ws_i, lib.msa_index_topk_workspace_bytes(q0, nq, cfg.H_kv, cfg.B_k, cfg.k))
            ws_v = max(ws_v, lib.msa_invert_index_workspace_bytes(q0, nq, cfg.H_kv, cfg.B_k, cfg.k))
            ws_a = max(ws_a, lib.msa_sparse_attn_fwd_workspace_bytes(
                q0, nq, cfg.H_q, cfg.H_kv, cfg.d_h, cfg.B_k, cfg.k))
            nnz = max(nnz, msa.selection_nnz(q0, nq, cfg.H_kv, cfg.k))
        fused = msa.get_option(msa.OPT_INDEX_FUSED)
        self.whole_index = bool(fused) and whole_index
        u8 = torch.uint8
        self.ws_i = torch.empty(1 if fused else ws_i, dtype=u8, device=dev)
        self.ws_v = torch.empty(ws_v, dtype=u8, device=dev)
        self.ws_a = torch.empty(ws_a, dtype=u8, device=dev)
        self.sel = torch.empty((cfg.N, cfg.H_kv, cfg.k), dtype=torch.int32, device=dev)
        self.O = torch.empty((cfg.N, cfg.H_q, cfg.d_h), dtype=torch.float32, device=dev)
        self.lse = torch.empty((cfg.N, cfg.H_q), dtype=torch.float32, device=dev)
        self.row_ptr = torch.empty(cfg.H_kv * cfg.nblk + 1, dtype=torch.int32, device=dev)
        self.col = torch.empty(nnz, dtype=torch.int32, device=dev)
        self.slot = torch.empty(nnz, dtype=torch.uint8, device=dev)
        self.events = []

    def step(self, record=False):
        """One prefill.  The fused Index Branch runs once over the whole
        sequence (it keeps no per-chunk state); the inverted index and the
        Main Branch run per query chunk."""
        import torch
        cfg, t, msa = self.cfg, self.t, self.msa

        def ev():
            return torch.cuda.Event(enable_timing=True)
        rec = []
        if self.whole_index:
            e = (ev(), ev()) if record else None
            if record:
                e[0].record()
            msa.index_topk(t["q_idx"], t["k_idx"], cfg.k, q_start=0, Nq=cfg.N, sel=self.sel,
                           ws=self.ws_i)
            if record:
                e[1].record()
                rec.append((0, e[0], e[1]))
        for q0, nq in self.chunks:
            e = [ev() for _ in range(4)] if record else None
            if record:
                e[0].record()
            sel_c = self.sel[q0:q0 + nq]
            if not self.whole_index:
                msa.index_topk(t["q_idx"], t["k_idx"], cfg.k, q_start=q0, Nq=nq, sel=sel_c,
                               ws=self.ws_i)
            if record:
                e[1].record()
            rp, col, slot = msa.invert_index(sel_c, q_start=q0, ws=self.ws_v,
                                             row_ptr=self.row_ptr, col=self.col,
                                             slot=self.slot)
            if record:
                e[2].record()
            msa.sparse_attn_fwd(t["Q"], t["K"], t["V"], rp, col, slot, cfg.k, q_start=q0,
                                Nq=nq, scale=cfg.scale, O=self.O[q0:q0 + nq],
                                lse=self.lse[q0:q0 + nq], ws=self.ws_a)
            if record:
                e[3].record()
                rec += [(0, e[0], e[1]), (1, e[1], e[2]), (2, e[2], e[3])]
        if record:
            self.events.append(rec)

    def stage_ms(self):
        """Total ms per stage over the recorded steps."""
        tot = [0.0, 0.0, 0.0]
        for rec in self.events:
            for stage, a, b in rec:
                tot[stage] += a.elapsed_time(b)
        return tot


def time_prefill(cfg, t, steps, warmup, whole_index=True):
    import torch
    pf = Prefill(cfg, t, whole_index)
    for _ in range(warmup):
        pf.step()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        pf.step(record=True)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    st = [x / steps for x in pf.stage_ms()]
    return pf, ms, st


def time_kl(pf, cfg, t, reps=2):
    """The index-alignment KL pass (msa_index_kl) over every chunk of a step,
    from the step's lse.  Each chunk's inverted index is rebuilt first (its
    buffers are shared between chunks); only the KL calls are timed."""
    import torch
    msa = pf.msa
    lib = msa.load()
    ws = max(lib.msa_index_kl_workspace_bytes(q0, nq, cfg.H_kv, cfg.B_k, cfg.k)
             for q0, nq in pf.chunks)
    ws = torch.empty(ws, dtype=torch.uint8, device=t["Q"].device)
    kl = torch.empty((cfg.N, cfg.H_kv), dtype=torch.float32, device=t["Q"].device)
    sums = torch.empty(len(pf.chunks), dtype=torch.float64, device=t["Q"].device)
    total_ms, nnz = 0.0, 0
    for rep in range(reps + 1):
        ms = 0.0
        for c, (q0, nq) in enumerate(pf.chunks):
            rp, col, slot = msa.invert_index(pf.sel[q0:q0 + nq], q_start=q0, ws=pf.ws_v,
                                             row_ptr=pf.row_ptr, col=pf.col, slot=pf.slot)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            msa.index_kl(t["Q"], t["K"], t["q_idx"], t["k_idx"], pf.lse[q0:q0 + nq], rp, col,
                         slot, cfg.k, q_start=q0, Nq=nq, scale=cfg.scale, kl=kl[q0:q0 + nq],
                         kl_sum=sums[c:c + 1], ws=ws)
            b.record()
            b.synchronize()
            ms += a.elapsed_time(b)
            if rep == 0:
                nnz += msa.selection_nnz(q0, nq, cfg.H_kv, cfg.k)
        if rep > 0:
            total_ms += ms
    ms = total_ms / reps
    G = cfg.H_q // cfg.H_kv
    # per (query, group, selected block): the group's Q rows, q_idx, its lse
    # values and the 12-byte partial
    nbytes = nnz * (2 * G * cfg.d_h + 2 * cfg.d_idx + 4 * G + 12)
    return {"ms_per_step": round(ms, 3),
            "kl_mean": float(sums.sum().item() / (cfg.N * cfg.H_kv)),
            "GB_per_s": round(nbytes / (ms / 1e3) / 1e9, 1),
            "frac_hbm_peak": round(nbytes / (ms / 1e3) / 1e9 / PEAK_HBM_GBS, 4),
            "bytes_per_step": nbytes}


def time_bwd(pf, cfg, t, reps=2):
    """The Main Branch backward (msa_sparse_attn_bwd) over every chunk of a
    step, from the step's O and lse and a seeded output gradient.  Each
    chunk's inverted index is rebuilt first (its buffers are shared between
    chunks); only the backward calls are timed."""
    import torch
    from block_sparse_long_idx_amd.synth import make_grad_output
    msa = pf.msa
    lib = msa.load()
    dev = t["Q"].device
    dO = make_grad_output(cfg.N, cfg.H_q, cfg.d_h, seed=cfg.seed + 17, device=dev)
    ws = max(lib.msa_sparse_attn_bwd_workspace_bytes(q0, nq, cfg.H_q, cfg.H_kv, cfg.d_h,
                                                     cfg.B_k, cfg.k) for q0, nq in pf.chunks)
    ws = torch.empty(ws, dtype=torch.uint8, device=dev)
    dQ = torch.empty((cfg.N, cfg.H_q, cfg.d_h), dtype=torch.float32, device=dev)
    dK = torch.empty((cfg.N, cfg.H_kv, cfg.d_h), dtype=torch.float32, device=dev)
    dV = torch.empty_like(dK)
    total_ms, nnz = 0.0, 0
    for rep in range(reps + 1):
        dK.zero_()
        dV.zero_()
        ms = 0.0
        for q0, nq in pf.chunks:
            rp, col, slot = msa.invert_index(pf.sel[q0:q0 + nq], q_start=q0, ws=pf.ws_v,
                                             row_ptr=pf.row_ptr, col=pf.col, slot=pf.slot)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            msa.sparse_attn_bwd(t["Q"], t["K"], t["V"], pf.O[q0:q0 + nq], pf.lse[q0:q0 + nq],
                                dO[q0:q0 + nq], rp, col, slot, cfg.k, q_start=q0, Nq=nq,
                                scale=cfg.scale, dQ=dQ[q0:q0 + nq], dK=dK, dV=dV, ws=ws)
            b.record()
            b.synchronize()
            ms += a.elapsed_time(b)
            if rep == 0:
                nnz += msa.selection_nnz(q0, nq, cfg.H_kv, cfg.k)
        if rep > 0:
            total_ms += ms
    ms = total_ms / reps
    G = cfg.H_q // cfg.H_kv
    d = cfg.d_h
    # per (query, head, selected block): the fused pass reads Q, dO, lse and
    # delta once and writes a bf16 dQ partial, which the reduce reads back.
    # Per (query, head): delta reads O (fp32) and dO and writes delta; the
    # reduce writes dQ (fp32).
    pairs = nnz * G
    nbytes = pairs * (8 * d + 8) + cfg.N * cfg.H_q * (6 * d + 4 * d + 4)
    flops = 10.0 * cfg.H_q * d * cfg.N * cfg.k * cfg.B_k
    ok = bool(torch.isfinite(dQ).all().item() and torch.isfinite(dK).all().item()
              and torch.isfinite(dV).all().item())
    del dO, ws
    return {"ms_per_step": round(ms, 3),
            "effective_tflops": round(flops / (ms / 1e3) / 1e12, 2),
            "frac_bf16_peak": round(flops / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "formula_tflop_per_step": round(flops / 1e12, 3),
            "GB_per_s": round(nbytes / (ms / 1e3) / 1e9, 1),
            "frac_hbm_peak": round(nbytes / (ms / 1e3) / 1e9 / PEAK_HBM_GBS, 4),
            "bytes_per_step": nbytes, "finite": ok}


def time_frontend(cfg, reps=3):
    """The Index Branch front-end (msa_index_frontend: both projections of
    the hidden states, RMS norm and RoPE) over the whole sequence."""
    import torch
    from block_sparse_long_idx_amd import msa
    from block_sparse_long_idx_amd.synth import make_frontend_inputs
    t = make_frontend_inputs(cfg.N, cfg.d_model, cfg.H_kv, cfg.d_idx, seed=cfg.seed + 29,
                             device="cuda")
    q = torch.empty((cfg.N, cfg.H_kv, cfg.d_idx), dtype=torch.bfloat16, device="cuda")
    k = torch.empty_like(q)

    def run():
        msa.index_frontend(t["hidden"], t["Wq"], t["Wk"], t["gq"], t["gk"], cfg.H_kv, cfg.d_idx,
                           q_idx=q, k_idx=k)
    run()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        run()
    b.record()
    b.synchronize()
    ms = a.elapsed_time(b) / reps
    cols = cfg.H_kv * cfg.d_idx
    flops = 2.0 * 2 * cfg.N * cfg.d_model * cols
    # hidden read once, both outputs written, both weights read
    nbytes = 2 * cfg.N * cfg.d_model + 2 * 2 * cfg.N * cols + 2 * 2 * cols * cfg.d_model
    del t, q, k
    return {"ms_per_step": round(ms, 3), "d_model": cfg.d_model,
            "effective_tflops": round(flops / (ms / 1e3) / 1e12, 2),
            "frac_bf16_peak": round(flops / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "GB_per_s": round(nbytes / (ms / 1e3) / 1e9, 1), "bytes_per_step": nbytes}


VARLEN_FRACTIONS = (3 / 8, 1 / 4, 1 / 8, 1 / 8, 1 / 16, 1 / 32, 1 / 64, 1 / 64)


def time_cached(cfg, t, reps=3):
    """Chunked prefill against a KV cache: the last query chunk of the
    sequence (its own Q/q_idx rows only) against the cache of all keys."""
    import torch
    from block_sparse_long_idx_amd import msa
    c = cfg.chunk or cfg.N
    q0 = cfg.N - c
    Qc, qic = t["Q"][q0:], t["q_idx"][q0:]
    lib = msa.load()
    ws = torch.empty(lib.msa_prefill_cached_workspace_bytes(q0, c, 0, cfg.H_q, cfg.H_kv, cfg.d_h,
                                                            cfg.d_idx, cfg.B_k, cfg.k),
                     dtype=torch.uint8, device="cuda")
    sel = torch.empty((c, cfg.H_kv, cfg.k), dtype=torch.int32, device="cuda")
    O = torch.empty((c, cfg.H_q, cfg.d_h), dtype=torch.float32, device="cuda")
    lse = torch.empty((c, cfg.H_q), dtype=torch.float32, device="cuda")

    def run():
        msa.prefill_cached(Qc, t["K"], t["V"], qic, t["k_idx"], cfg.k, q_start=q0,
                           scale=cfg.scale, sel=sel, O=O, lse=lse, ws=ws)
    run()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        run()
    b.record()
    b.synchronize()
    ms = a.elapsed_time(b) / reps
    del ws, sel, O, lse
    return {"new_tokens": c, "cached_tokens": q0, "ms": round(ms, 3),
            "tokens_per_s": round(c / (ms / 1e3), 1)}


def time_varlen(cfg, reps=2):
    """Varlen batched prefill: eight packed sequences whose lengths sum to
    N (fractions VARLEN_FRACTIONS), each with its own positions and prefix."""
    import torch
    from block_sparse_long_idx_amd import msa
    from block_sparse_long_idx_amd.synth import make_prefill_inputs
    lens = [int(cfg.N * f) for f in VARLEN_FRACTIONS]
    lens[0] += cfg.N - sum(lens)
    packed = None
    for b, L in enumerate(lens):
        s = make_prefill_inputs(L, cfg.H_q, cfg.H_kv, cfg.d_h, cfg.d_idx,
                                n_hot=max(1, cfg.n_hot * L // cfg.N), seed=cfg.seed + 100 + b,
                                device="cuda")
        if packed is None:
            packed = {key: torch.empty((cfg.N,) + v.shape[1:], dtype=v.dtype, device="cuda")
                      for key, v in s.items()}
        t0 = sum(lens[:b])
        for key, v in s.items():
            packed[key][t0:t0 + L] = v
        del s
    cu = [0]
    for L in lens:
        cu.append(cu[-1] + L)
    chunk = cfg.chunk or 0
    lib = msa.load()
    import ctypes
    cua = (ctypes.c_int64 * len(cu))(*cu)
    ws = torch.empty(lib.msa_prefill_varlen_workspace_bytes(cua, len(lens), chunk, cfg.H_q,
                                                            cfg.H_kv, cfg.d_h, cfg.d_idx,
                                                            cfg.B_k, cfg.k),
                     dtype=torch.uint8, device="cuda")
    O = torch.empty((cfg.N, cfg.H_q, cfg.d_h), dtype=torch.float32, device="cuda")

    def run():
        msa.prefill_varlen(packed["Q"], packed["K"], packed["V"], packed["q_idx"],
                           packed["k_idx"], cu, cfg.k, chunk=chunk, scale=cfg.scale,
                           want_lse=False, sel=None, O=O, ws=ws)
    run()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        run()
    b.record()
    b.synchronize()
    ms = a.elapsed_time(b) / reps
    flops = sum(4.0 * cfg.H_q * cfg.d_h * L * cfg.k * cfg.B_k + float(cfg.H_kv) * cfg.d_idx * L * L
                for L in lens)
    del packed, ws, O
    return {"lengths": lens, "ms_per_step": round(ms, 3),
            "tokens_per_s": round(cfg.N / (ms / 1e3), 1),
            "effective_tflops": round(flops / (ms / 1e3) / 1e12, 2),
            "frac_bf16_peak": round(flops / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4)}


def cpu_baseline(cfg, t, n_rows):
    """The oracle, as it stands, on n_rows query rows spread over the sequence."""
    import numpy as np
    import torch
    import oracle
    from block_sparse_long_idx_amd.synth import bf16_bits, sample_rows
    rows = np.array(sample_rows(cfg.N, n_rows))
    rt = torch.from_numpy(rows).to(t["Q"].device)
    k_idx, K, V = bf16_bits(t["k_idx"]), bf16_bits(t["K"]), bf16_bits(t["V"])
    q_rows, Q_rows = bf16_bits(t["q_idx"][rt]), bf16_bits(t["Q"][rt])
    oracle.build(force=False)
    nthreads = oracle.threads()
    t0 = time.perf_counter()
    sel = oracle.select(q_rows, k_idx, rows, cfg.k, nthreads=nthreads)
    oracle.attend(Q_rows, K, V, sel, rows, cfg.scale, nthreads=nthreads)
    dt = time.perf_counter() - t0

    # Extrapolation to every row of the sequence by the oracle's own cost per
    # row: selection scores i+1 keys per group (d_idx multiply-adds each),
    # attention touches min(k*B_k, i+1) keys per head (2 d_h each).
    def row_cost(i):
        i = np.asarray(i, dtype=np.float64)
        return (i + 1) * cfg.d_idx * cfg.H_kv + \
            np.minimum(cfg.k * cfg.B_k, i + 1) * 2 * cfg.d_h * cfg.H_q

    full_s = dt * float(row_cost(np.arange(cfg.N)).sum()) / float(row_cost(rows).sum())
    return {"value": round(len(rows) / dt, 3), "unit": "tokens/s", "cores": nthreads,
            "kind": "oracle",
            "sample": f"{len(rows)} query rows evenly spaced over positions 0..{cfg.N - 1} "
                      f"of the same workload (all heads and groups), {dt:.1f} s wall",
            "extrapolated_all_rows_s": round(full_s, 1),
            "extrapolation": "sample wall time scaled by the oracle's per-row work "
                             "(i+1 index scores per group + min(k*B_k, i+1) keys per head) "
                             "summed over all N rows vs the sampled rows"}


def time_decode(cfg, steps, warmup):
    import torch
    from block_sparse_long_idx_amd import msa
    from block_sparse_long_idx_amd.synth import inputs_for
    t = inputs_for(cfg, device="cuda")
    dev = t["q"].device
    B, N = cfg.batch, cfg.N
    ws = torch.empty(msa.decode_workspace_bytes(B, N, cfg.H_q, cfg.H_kv, cfg.d_h, cfg.d_idx, cfg.k),
                     dtype=torch.uint8, device=dev)
    sel = torch.empty((B, cfg.H_kv, cfg.k), dtype=torch.int32, device=dev)
    O = torch.empty((B, cfg.H_q, cfg.d_h), dtype=torch.float32, device=dev)
    lse = torch.empty((B, cfg.H_q), dtype=torch.float32, device=dev)

    def one():
        msa.decode(t["q"], t["q_idx"], t["K"], t["V"], t["k_idx"], cfg.k, scale=cfg.scale,
                   sel=sel, O=O, lse=lse, ws=ws)

    for _ in range(warmup):
        one()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(steps):
        one()
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / steps
    nbytes = (B * N * cfg.H_kv * cfg.d_idx * 2                       # k_idx scan
              + B * cfg.H_kv * cfg.k * cfg.B_k * cfg.d_h * 2 * 2      # selected K and V
              + B * (cfg.H_q * cfg.d_h * 2 + cfg.H_kv * cfg.d_idx * 2)  # q, q_idx
              + B * cfg.H_q * (cfg.d_h + 1) * 4)                      # O, lse
    del t
    return {"workload": f"decode B={B} x N={N}", "ms_per_step": round(ms, 4),
            "tokens_per_s": round(B / (ms / 1e3), 1),
            "GB_per_s": round(nbytes / (ms / 1e3) / 1e9, 1),
            "frac_hbm_peak": round(nbytes / (ms / 1e3) / 1e9 / PEAK_HBM_GBS, 4),
            "bytes_per_step": nbytes}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="1m", choices=["tiny", "8k", "128k", "1m"])
    ap.add_argument("--fused", type=int, default=1, help="fused Index-Branch kernel (1/0)")
    ap.add_argument("--attn-chunk", type=int, default=0, help="positions per work item")
    ap.add_argument("--chunk", type=int, default=0,
                    help="query positions per Main Branch pass (0 = the workload's)")
    ap.add_argument("--cpu-rows", type=int, default=1024)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the 128K and decode legs")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); "
              "this build has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        # A plain copy of known size: reads and writes exactly 1 GiB each, so
        # FETCH_SIZE / WRITE_SIZE of this dispatch calibrate the counters.
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": src.numel() * 4, "copy_bytes_written": dst.numel() * 4}))
        return
    from block_sparse_long_idx_amd import msa
    from block_sparse_long_idx_amd.synth import CONFIGS, inputs_for
    msa.load()
    msa.set_option(msa.OPT_INDEX_FUSED, args.fused)
    if args.attn_chunk:
        msa.set_option(msa.OPT_ATTN_CHUNK, args.attn_chunk)
    cfg = CONFIGS[args.workload]
    if args.chunk:
        import dataclasses
        cfg = dataclasses.replace(cfg, chunk=args.chunk)
    log(f"[bench] workload {cfg.name}: generating inputs on the GPU")
    t = inputs_for(cfg, device="cuda")
    torch.cuda.synchronize()
    log(f"[bench] timing {args.warmup} warmup + {args.steps} steps")
    pf, ms, stages = time_prefill(cfg, t, args.steps, args.warmup)
    main_f, index_f = formula_flops(cfg)
    tflops = (main_f + index_f) / (ms / 1e3) / 1e12
    stage_names = ["index_topk", "invert_index", "sparse_attn_fwd"]
    log(f"[bench] {ms:.2f} ms/step; stages " +
        ", ".join(f"{n} {s:.2f} ms" for n, s in zip(stage_names, stages)))

    # Roofline of the dominant kernel.  With the fused Index Branch that is
    # its single launch per step, the largest kernel of the step: the Main
    # Branch stage is three kernels per query chunk (work list, KV-outer
    # attention, combine), the largest of which takes ~2/3 of the stage.
    if args.fused:
        ach = index_f / (stages[0] / 1e3) / 1e12
        roof = {"kernel": "index_topk_fused_kernel", "bound": "mfma",
                "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                "traffic": stored_traffic("index_topk_fused_kernel") if cfg.name == "1m" else None,
                "per_launch": "one launch per step over all N queries; achieved = "
                              "algorithmic flops (H_kv*d_idx*N^2) / its event time; traffic "
                              "in HBM bytes per launch"}
    else:
        roof = {"kernel": "index_pool_kernel + topk_kernel", "bound": "mfma", "achieved": None,
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": None, "traffic": None}
    # The Main Branch stage against HBM: per non-local (query, head, block) Q
    # is gathered (2 d_h B), the bf16 partial written and read back (4 d_h B)
    # with its fp32 lse (8 B); per (query, head) the combine reads the local
    # block's Q (2 d_h B) and writes O (4 d_h B) and lse (4 B).
    main_bytes = 0
    for q0, nq in chunks_of(cfg):
        nl = (msa.selection_nnz(q0, nq, cfg.H_kv, cfg.k) - nq * cfg.H_kv) * (cfg.H_q // cfg.H_kv)
        main_bytes += nl * (6 * cfg.d_h + 8) + nq * cfg.H_q * (6 * cfg.d_h + 4)
    main_gbs = main_bytes / (stages[2] / 1e3) / 1e9
    roof_main = {"stage": "sparse_attn_fwd", "kernels": "build_items_kernel, "
                 "attn_kv_outer_kernel, combine_local_kernel per query chunk",
                 "bound": "hbm", "achieved": round(main_gbs, 1), "peak": PEAK_HBM_GBS,
                 "unit": "GB/s", "frac": round(main_gbs / PEAK_HBM_GBS, 4),
                 "algorithmic_bytes_per_step": main_bytes}

    # The inverted index against HBM: per chunk the selection table is read
    # (4 B per (query, group, slot)), col and slot written (5 B per entry)
    # and row_ptr written (4 B per bucket).
    inv_bytes = 0
    for q0, nq in chunks_of(cfg):
        nblk_c = -(-(q0 + nq) // cfg.B_k)
        inv_bytes += 4 * nq * cfg.H_kv * cfg.k + 5 * msa.selection_nnz(q0, nq, cfg.H_kv, cfg.k) \
            + 4 * (cfg.H_kv * nblk_c + 1)
    inv_gbs = inv_bytes / (stages[1] / 1e3) / 1e9
    roof_inv = {"stage": "invert_index", "kernels": "csr_hist_kernel, csr_scan_kernel, "
                "csr_scatter_kernel per query chunk", "bound": "hbm",
                "achieved": round(inv_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(inv_gbs / PEAK_HBM_GBS, 4), "algorithmic_bytes_per_step": inv_bytes}

    out = {
        "metric": "MSA prefill tokens/s + effective TFLOP/s (% bf16 MFMA peak) at 128K and 1M",
        "value": round(cfg.N / (ms / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"MSA prefill N={cfg.N}", "N": cfg.N, "H_q": cfg.H_q,
                   "H_kv": cfg.H_kv, "d_h": cfg.d_h, "d_idx": cfg.d_idx, "k": cfg.k,
                   "B_k": cfg.B_k, "query_chunk": cfg.chunk or cfg.N,
                   "index_variant": "fused" if args.fused else "two-kernel",
                   "index_launch": "whole sequence" if args.fused else "per query chunk",
                   "attn_chunk": msa.get_option(msa.OPT_ATTN_CHUNK)},
        "effective_tflops": round(tflops, 2),
        "frac_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "formula_tflop_per_step": {"main": round(main_f / 1e12, 3),
                                   "index": round(index_f / 1e12, 3)},
        "stage_ms": {n: round(s, 3) for n, s in zip(stage_names, stages)},
        "roofline": roof,
        "roofline_main_branch": roof_main,
        "roofline_invert_index": roof_inv,
    }
    if not args.no_cpu_baseline:
        log(f"[bench] CPU oracle on {args.cpu_rows} sampled rows")
        out["cpu_baseline"] = cpu_baseline(cfg, t, args.cpu_rows)
    kl_leg = bwd_leg = cached_leg = chunked_leg = None
    if not args.no_extra and args.fused:
        log("[bench] per-chunk index leg")
        _, ms_c, st_c = time_prefill(cfg, t, 2, 1, whole_index=False)
        chunked_leg = {"ms_per_step": round(ms_c, 3),
                       "tokens_per_s": round(cfg.N / (ms_c / 1e3), 1),
                       "stage_ms": {n: round(x, 3) for n, x in zip(stage_names, st_c)}}
    if not args.no_extra:
        log("[bench] index KL leg")
        kl_leg = time_kl(pf, cfg, t)
        log("[bench] Main Branch backward leg")
        bwd_leg = time_bwd(pf, cfg, t)
        log("[bench] cached-prefill leg")
        cached_leg = time_cached(cfg, t)
    del pf, t
    torch.cuda.empty_cache()
    if not args.no_extra:
        extra = {f"index_kl_{cfg.name}": kl_leg, f"attn_bwd_{cfg.name}": bwd_leg,
                 f"prefill_cached_{cfg.name}": cached_leg}
        if chunked_leg:
            extra[f"prefill_{cfg.name}_index_per_chunk"] = chunked_leg
        log("[bench] varlen batch leg")
        extra[f"prefill_varlen_{cfg.name}"] = time_varlen(cfg)
        torch.cuda.empty_cache()
        log("[bench] index front-end leg")
        extra[f"index_frontend_{cfg.name}"] = time_frontend(cfg)
        torch.cuda.empty_cache()
        if cfg.name != "128k":
            c2 = CONFIGS["128k"]
            log("[bench] 128K prefill leg")
            t2 = inputs_for(c2, device="cuda")
            _, ms2, st2 = time_prefill(c2, t2, max(3, args.steps), 1)
            f2 = sum(formula_flops(c2))
            extra["prefill_128k"] = {
                "ms_per_step": round(ms2, 3), "tokens_per_s": round(c2.N / (ms2 / 1e3), 1),
                "effective_tflops": round(f2 / (ms2 / 1e3) / 1e12, 2),
                "frac_bf16_peak": round(f2 / (ms2 / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                "stage_ms": {n: round(s, 3) for n, s in zip(stage_names, st2)}}
            del t2
            torch.cuda.empty_cache()
        log("[bench] decode leg")
        extra["decode_32x1m"] = time_decode(CONFIGS["decode_1m"], max(5, args.steps), 2)
        torch.cuda.empty_cache()
        out["extra"] = extra
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
