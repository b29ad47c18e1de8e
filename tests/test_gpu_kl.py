"""GPU parity of the index-alignment KL (msa_index_kl) against the CPU
oracle, through the C ABI.

The teacher probabilities use the forward's lse (fp32) and the kernel sums
in fp32, so the KL value carries rounding relative to the scale of the
index scores: KL = sum t ln t - sum t s + ln sum exp(s) cancels two terms
of the size of the largest index score |s|max.  Bar: |KL - KL_ref| <=
KL_ATOL + KL_REL * (|KL_ref| + S_max), where S_max bounds |s| on these
inputs (d_idx * 3 * 5 for the integer index tensors, whose entries lie in
[-3, 5] after hot-block planting) and KL_REL is five fp32 units of
roundoff (5 * 2^-24).
"""
import math
import sys

import numpy as np
import pytest
import torch

from block_sparse_long_idx_amd import msa
from block_sparse_long_idx_amd.synth import CONFIGS, bf16_bits, inputs_for, make_prefill_inputs

pytestmark = pytest.mark.gpu

KL_ATOL, KL_REL = 1e-4, 3e-7


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _u16(t):
    return {k: bf16_bits(v) for k, v in t.items()}


def assert_kl_close(kl, kl_ref, d_idx):
    kl = np.asarray(kl, dtype=np.float64)
    s_max = d_idx * 3 * 5
    err = np.abs(kl - kl_ref)
    bound = KL_ATOL + KL_REL * (np.abs(kl_ref) + s_max)
    print(f"[kl] max err {err.max():.3e}, max err/bound {(err / bound).max():.3f}", flush=True)
    assert np.isfinite(kl).all()
    assert (err <= bound).all(), (err.max(), np.unravel_index(err.argmax(), err.shape))


KL_CASES = [
    # N, H_q, H_kv, d_h, d_idx, k, n_hot, q_start, Nq
    (1024, 4, 1, 64, 32, 4, 0, 0, 1024),
    (1000, 8, 2, 128, 64, 4, 2, 0, 1000),       # ragged last block
    (2000, 16, 4, 64, 128, 5, 3, 700, 1300),    # unaligned q_start
    (3000, 6, 2, 128, 64, 32, 4, 0, 3000),      # k = 32, G = 3
    (777, 2, 2, 64, 32, 1, 0, 0, 777),          # k = 1: local block only
    (600, 64, 1, 128, 64, 3, 1, 0, 600),        # G = 64
]


@pytest.mark.parametrize("case", KL_CASES, ids=lambda c: "N%d_Hq%d_Hkv%d_dh%d_di%d_k%d_qs%d" % (c[0], c[1], c[2], c[3], c[4], c[5], c[7]))
def test_index_kl_stage(oracle_lib, case):
    """Fed the oracle's selection, inverted index and lse."""
    N, H_q, H_kv, d_h, d_idx, k, n_hot, q_start, Nq = case
    say("index_kl", case)
    t = make_prefill_inputs(N, H_q, H_kv, d_h, d_idx, n_hot=n_hot, seed=N + k + 1)
    u = _u16(t)
    rows = np.arange(q_start, q_start + Nq)
    scale = 1.0 / math.sqrt(d_h)
    sel, _, lse_ref = oracle_lib.prefill_rows(u, rows, k, scale)
    kl_ref = oracle_lib.index_kl(u["q_idx"][rows], u["k_idx"], u["Q"][rows], u["K"], sel, rows,
                                 scale)
    nblk = (q_start + Nq + 127) // 128
    rp, col, slot = oracle_lib.invert(sel, q_start, nblk)
    d = {key: v.cuda() for key, v in t.items()}
    kl, kl_sum = msa.index_kl(
        d["Q"], d["K"], d["q_idx"], d["k_idx"],
        torch.from_numpy(lse_ref.astype(np.float32)).cuda(),
        torch.from_numpy(rp.astype(np.int32)).cuda(),
        torch.from_numpy(col.astype(np.int32)).cuda(),
        torch.from_numpy(slot.astype(np.uint8)).cuda(), k, q_start=q_start, Nq=Nq, scale=scale)
    torch.cuda.synchronize()
    kl_h = kl.cpu().numpy()
    assert_kl_close(kl_h, kl_ref, d_idx)
    # the fixed-order total equals the sum of the per-row values
    assert abs(kl_sum.item() - kl_h.astype(np.float64).sum()) <= 1e-9 * max(1.0, abs(kl_sum.item()))


def test_index_kl_end_to_end_8k(oracle_lib):
    """The whole GPU chain (selection, inverted index, Main Branch lse, KL) on
    the 8K workload against the oracle on every 8th row."""
    cfg = CONFIGS["8k"]
    say("index_kl e2e", cfg.name)
    t = inputs_for(cfg, device="cuda")
    sel = msa.index_topk(t["q_idx"], t["k_idx"], cfg.k)
    rp, col, slot = msa.invert_index(sel, q_start=0)
    _, lse = msa.sparse_attn_fwd(t["Q"], t["K"], t["V"], rp, col, slot, cfg.k, scale=cfg.scale)
    kl, kl_sum = msa.index_kl(t["Q"], t["K"], t["q_idx"], t["k_idx"], lse, rp, col, slot, cfg.k,
                              scale=cfg.scale)
    kl2, kl_sum2 = msa.index_kl(t["Q"], t["K"], t["q_idx"], t["k_idx"], lse, rp, col, slot,
                                cfg.k, scale=cfg.scale)
    torch.cuda.synchronize()
    assert torch.equal(kl, kl2) and torch.equal(kl_sum, kl_sum2)   # deterministic
    rows = np.arange(0, cfg.N, 8)
    u = {key: bf16_bits(t[key]) for key in ("Q", "K", "q_idx", "k_idx")}
    sel_ref = oracle_lib.select(u["q_idx"][rows], u["k_idx"], rows, cfg.k)
    np.testing.assert_array_equal(sel.cpu().numpy()[rows], sel_ref)
    kl_ref = oracle_lib.index_kl(u["q_idx"][rows], u["k_idx"], u["Q"][rows], u["K"], sel_ref,
                                 rows, cfg.scale)
    assert_kl_close(kl.cpu().numpy()[rows], kl_ref, cfg.d_idx)


@pytest.mark.slow
def test_index_kl_1m_sampled(oracle_lib):
    """The 1M workload's KL pass over every chunk, after the GPU selection
    and forward, checked on sampled rows (each (row, group) value depends on
    that row alone)."""
    from block_sparse_long_idx_amd.synth import sample_rows
    cfg = CONFIGS["1m"]
    say("index_kl 1m sampled")
    t = inputs_for(cfg, device="cuda")
    sel = msa.index_topk(t["q_idx"], t["k_idx"], cfg.k)
    kl = torch.empty((cfg.N, cfg.H_kv), dtype=torch.float32, device="cuda")
    for q0 in range(0, cfg.N, cfg.chunk):
        rp, col, slot = msa.invert_index(sel[q0:q0 + cfg.chunk], q_start=q0)
        _, lse = msa.sparse_attn_fwd(t["Q"], t["K"], t["V"], rp, col, slot, cfg.k, q_start=q0,
                                     Nq=cfg.chunk, scale=cfg.scale)
        msa.index_kl(t["Q"], t["K"], t["q_idx"], t["k_idx"], lse, rp, col, slot, cfg.k,
                     q_start=q0, Nq=cfg.chunk, scale=cfg.scale, want_sum=False,
                     kl=kl[q0:q0 + cfg.chunk])
        del rp, col, slot, lse
    torch.cuda.synchronize()
    rows = np.array(sample_rows(cfg.N, 64))
    rt = torch.from_numpy(rows).cuda()
    u = {key: bf16_bits(t[key][rt]) for key in ("Q", "q_idx")}
    K, kx = bf16_bits(t["K"]), bf16_bits(t["k_idx"])
    sel_ref = oracle_lib.select(u["q_idx"], kx, rows, cfg.k)
    np.testing.assert_array_equal(sel[rt].cpu().numpy(), sel_ref)
    kl_ref = oracle_lib.index_kl(u["q_idx"], kx, u["Q"], K, sel_ref, rows, cfg.scale)
    assert_kl_close(kl[rt].cpu().numpy(), kl_ref, cfg.d_idx)
