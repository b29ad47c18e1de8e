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

REL_L2, MAX_REL = 1e-2, 2e-2


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
