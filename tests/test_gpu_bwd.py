"""GPU parity of the Main Branch backward (msa_sparse_attn_bwd) against the
CPU oracle, through the C ABI.

The kernels feed bf16 P and dS to the MFMAs (as the forward feeds bf16 P)
and keep per-(row, block) dQ partials in bf16, so every gradient carries
bf16 rounding relative to its own scale.  Bar, per tensor: relative L2
error <= REL_L2 and max-abs error <= MAX_REL * max|reference|.
"""
import math
import sys

import numpy as np
import pytest
import torch

from block_sparse_long_idx_amd import msa
from block_sparse_long_idx_amd.synth import bf16_bits, make_prefill_inputs

pytestmark = pytest.mark.gpu

# About twice the errors these shapes measure (rel-L2 2.4e-3 for dQ, 1.7e-3
# for dK and dV), so a precision regression of the bf16 partials fails.
REL_L2, MAX_REL = 5e-3, 1e-2


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def assert_grad_close(name, got, ref):
    got = np.asarray(got, dtype=np.float64)
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    mx = np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30)
    print(f"[bwd] {name}: rel-L2 {rel:.2e}, max/max|ref| {mx:.2e}", flush=True)
    assert np.isfinite(got).all(), name
    assert rel <= REL_L2 and mx <= MAX_REL, (name, rel, mx)


BWD_CASES = [
    # N, H_q, H_kv, d_h, d_idx, k, n_hot, chunk
    (1024, 4, 1, 64, 32, 4, 0, 0),        # the tiny workload's shapes
    (1000, 8, 2, 128, 64, 4, 2, 0),       # ragged last block
    (2000, 16, 4, 64, 64, 5, 3, 768),     # three chunks, dK/dV accumulated
    (2600, 6, 2, 128, 32, 16, 4, 1000),   # G = 3, k = 16, chunks not on block edges
    (777, 2, 2, 64, 32, 1, 0, 0),         # k = 1: local block only
    (600, 64, 1, 128, 64, 3, 1, 0),       # G = 64
    (4500, 4, 4, 128, 64, 32, 3, 1500),   # G = 1, k = 32 (rows past 4096 fill every slot)
]


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: "N%d_Hq%d_Hkv%d_dh%d_k%d_chunk%d" % (c[0], c[1], c[2], c[3], c[5], c[7]))
def test_attn_bwd(oracle_lib, case):
    """Fed the oracle's selection, inverted index, O and lse; the output
    gradient is a seeded bf16 tensor."""
    N, H_q, H_kv, d_h, d_idx, k, n_hot, chunk = case
    say("attn_bwd", case)
    t = make_prefill_inputs(N, H_q, H_kv, d_h, d_idx, n_hot=n_hot, seed=N + 3 * k)
    gen = torch.Generator().manual_seed(N + 7)
    dO = torch.randn((N, H_q, d_h), generator=gen).to(torch.bfloat16)
    u = {key: bf16_bits(v) for key, v in t.items()}
    scale = 1.0 / math.sqrt(d_h)
    rows = np.arange(N)
    sel, O_ref, lse_ref = oracle_lib.prefill_rows(u, rows, k, scale)
    dQ_ref, dK_ref, dV_ref = oracle_lib.attend_backward(u["Q"], u["K"], u["V"], bf16_bits(dO),
                                                        sel, scale)
    d = {key: v.cuda() for key, v in t.items()}
    dOd = dO.cuda()
    O = torch.from_numpy(O_ref.astype(np.float32)).cuda()
    lse = torch.from_numpy(lse_ref.astype(np.float32)).cuda()
    dQ = torch.empty((N, H_q, d_h), dtype=torch.float32, device="cuda")
    dK = torch.zeros((N, H_kv, d_h), dtype=torch.float32, device="cuda")
    dV = torch.zeros((N, H_kv, d_h), dtype=torch.float32, device="cuda")
    c = chunk or N
    for q0 in range(0, N, c):
        nq = min(c, N - q0)
        nblk = (q0 + nq + 127) // 128
        rp, col, slot = oracle_lib.invert(sel[q0:q0 + nq], q0, nblk)
        msa.sparse_attn_bwd(d["Q"], d["K"], d["V"], O[q0:q0 + nq], lse[q0:q0 + nq],
                            dOd[q0:q0 + nq], torch.from_numpy(rp.astype(np.int32)).cuda(),
                            torch.from_numpy(col.astype(np.int32)).cuda(),
                            torch.from_numpy(slot.astype(np.uint8)).cuda(), k, q_start=q0,
                            Nq=nq, scale=scale, dQ=dQ[q0:q0 + nq], dK=dK, dV=dV)
    torch.cuda.synchronize()
    assert_grad_close("dQ", dQ.cpu().numpy(), dQ_ref)
    assert_grad_close("dK", dK.cpu().numpy(), dK_ref)
    assert_grad_close("dV", dV.cpu().numpy(), dV_ref)


def test_attn_bwd_deterministic():
    """Two runs of the whole chain give bitwise-identical gradients."""
    N, H_q, H_kv, d_h, d_idx, k = 3000, 16, 4, 128, 64, 8
    t = make_prefill_inputs(N, H_q, H_kv, d_h, d_idx, n_hot=4, seed=77)
    d = {key: v.cuda() for key, v in t.items()}
    dO = torch.randn((N, H_q, d_h), generator=torch.Generator().manual_seed(78)).to(
        torch.bfloat16).cuda()
    sel = msa.index_topk(d["q_idx"], d["k_idx"], k)
    rp, col, slot = msa.invert_index(sel, q_start=0)
    O, lse = msa.sparse_attn_fwd(d["Q"], d["K"], d["V"], rp, col, slot, k)
    outs = [msa.sparse_attn_bwd(d["Q"], d["K"], d["V"], O, lse, dO, rp, col, slot, k)
            for _ in range(2)]
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_attn_bwd_8k_group0(oracle_lib):
    """The 8K workload's full shape (64 query heads, 4 groups, d_h 128,
    k 16) through the GPU backward; groups are independent, so group 0 is
    checked against the oracle run on that group alone."""
    from block_sparse_long_idx_amd.synth import CONFIGS, inputs_for, make_grad_output
    cfg = CONFIGS["8k"]
    say("attn_bwd 8k group 0")
    t = inputs_for(cfg)
    dO = make_grad_output(cfg.N, cfg.H_q, cfg.d_h, seed=cfg.seed + 17)
    u = {key: bf16_bits(v) for key, v in t.items()}
    rows = np.arange(cfg.N)
    sel = oracle_lib.select(u["q_idx"], u["k_idx"], rows, cfg.k)
    rp, col, slot = oracle_lib.invert(sel, 0, cfg.nblk)
    d = {key: v.cuda() for key, v in t.items()}
    rp_d = torch.from_numpy(rp.astype(np.int32)).cuda()
    col_d = torch.from_numpy(col.astype(np.int32)).cuda()
    slot_d = torch.from_numpy(slot.astype(np.uint8)).cuda()
    O, lse = msa.sparse_attn_fwd(d["Q"], d["K"], d["V"], rp_d, col_d, slot_d, cfg.k,
                                 scale=cfg.scale)
    dQ, dK, dV = msa.sparse_attn_bwd(d["Q"], d["K"], d["V"], O, lse, dO.cuda(), rp_d, col_d,
                                     slot_d, cfg.k, scale=cfg.scale)
    torch.cuda.synchronize()
    G = cfg.H_q // cfg.H_kv
    dQ_ref, dK_ref, dV_ref = oracle_lib.attend_backward(
        np.ascontiguousarray(u["Q"][:, :G]), np.ascontiguousarray(u["K"][:, :1]),
        np.ascontiguousarray(u["V"][:, :1]), np.ascontiguousarray(bf16_bits(dO)[:, :G]),
        np.ascontiguousarray(sel[:, :1]), cfg.scale)
    assert_grad_close("dQ", dQ[:, :G].cpu().numpy(), dQ_ref)
    assert_grad_close("dK", dK[:, :1].cpu().numpy(), dK_ref)
    assert_grad_close("dV", dV[:, :1].cpu().numpy(), dV_ref)


@pytest.mark.slow
def test_attn_bwd_1m_sampled(oracle_lib):
    """The 1M workload's backward in the benchmark's launch shape (16 query
    chunks of 65,536, dK/dV accumulated across them) after the GPU forward:
    dQ on sampled rows against the oracle, and the exact identity
    sum_j dV[j, r] = sum of dO over group r's (row, head) pairs."""
    from block_sparse_long_idx_amd.synth import CONFIGS, inputs_for, make_grad_output, sample_rows
    cfg = CONFIGS["1m"]
    say("attn_bwd 1m sampled")
    t = inputs_for(cfg, device="cuda")
    dO = make_grad_output(cfg.N, cfg.H_q, cfg.d_h, seed=cfg.seed + 17, device="cuda")
    sel = msa.index_topk(t["q_idx"], t["k_idx"], cfg.k)
    O = torch.empty((cfg.N, cfg.H_q, cfg.d_h), dtype=torch.float32, device="cuda")
    lse = torch.empty((cfg.N, cfg.H_q), dtype=torch.float32, device="cuda")
    dQ = torch.empty_like(O)
    dK = torch.zeros((cfg.N, cfg.H_kv, cfg.d_h), dtype=torch.float32, device="cuda")
    dV = torch.zeros_like(dK)
    for q0 in range(0, cfg.N, cfg.chunk):
        rp, col, slot = msa.invert_index(sel[q0:q0 + cfg.chunk], q_start=q0)
        msa.sparse_attn_fwd(t["Q"], t["K"], t["V"], rp, col, slot, cfg.k, q_start=q0,
                            Nq=cfg.chunk, scale=cfg.scale, O=O[q0:q0 + cfg.chunk],
                            lse=lse[q0:q0 + cfg.chunk])
        msa.sparse_attn_bwd(t["Q"], t["K"], t["V"], O[q0:q0 + cfg.chunk],
                            lse[q0:q0 + cfg.chunk], dO[q0:q0 + cfg.chunk], rp, col, slot,
                            cfg.k, q_start=q0, Nq=cfg.chunk, scale=cfg.scale,
                            dQ=dQ[q0:q0 + cfg.chunk], dK=dK, dV=dV)
        del rp, col, slot
    torch.cuda.synchronize()
    rows = np.array(sample_rows(cfg.N, 48))
    rt = torch.from_numpy(rows).cuda()
    u = {key: bf16_bits(t[key][rt]) for key in ("Q", "q_idx")}
    K, V, kx = bf16_bits(t["K"]), bf16_bits(t["V"]), bf16_bits(t["k_idx"])
    sel_ref = oracle_lib.select(u["q_idx"], kx, rows, cfg.k)
    np.testing.assert_array_equal(sel[rt].cpu().numpy(), sel_ref)
    dq_ref = oracle_lib.attend_backward_dq_rows(u["Q"], K, V, bf16_bits(dO[rt]), sel_ref, rows,
                                                cfg.scale)
    assert_grad_close("dQ (sampled rows)", dQ[rt].cpu().numpy(), dq_ref)
    # sum_j p_j = 1 for every (row, head): the dV column sums are the dO sums
    G = cfg.H_q // cfg.H_kv
    got = dV.double().sum(0)                                     # [H_kv, d_h]
    want = torch.zeros((cfg.H_kv, cfg.d_h), dtype=torch.float64, device="cuda")
    scale_ref = torch.zeros_like(want)
    for q0 in range(0, cfg.N, cfg.chunk):                        # bounded temporaries
        g = dO[q0:q0 + cfg.chunk].double().view(-1, cfg.H_kv, G, cfg.d_h)
        want += g.sum((0, 2))
        scale_ref += g.abs().sum((0, 2))
        del g
    err = ((got - want).abs() / scale_ref).max().item()
    print(f"[bwd] 1M dV column sums: max |err| / sum|dO| = {err:.2e}", flush=True)
    # bf16 P perturbs each row's sum of p by ~2^-9 with random sign; over
    # 2^24 (row, head) pairs that averages to ~1e-6 of sum|dO| at most
    assert err <= 1e-5, err
