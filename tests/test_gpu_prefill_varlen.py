"""GPU parity of the second prefill workload against the CPU oracle,
through the C ABI: chunked prefill against a KV cache (msa_prefill_cached)
and varlen batched prefill of packed sequences (msa_prefill_varlen).

Selections are bit-exact (the index inputs are integer-valued, so every
index score is exact); O and lse meet the bar of the single-sequence
prefill tests (max-abs 1e-2 and relative L2 5e-3 on O, 1e-3 on lse).
"""
import math
import sys

import numpy as np
import pytest
import torch

from block_sparse_long_idx_amd import msa
from block_sparse_long_idx_amd.synth import bf16_bits, make_prefill_inputs

pytestmark = pytest.mark.gpu

ATOL, RTOL_L2, LSE_ATOL = 1e-2, 5e-3, 1e-3


@pytest.fixture(params=[0, 1], ids=["twokernel", "fused"])
def index_variant(request):
    """Both Index Branch variants: per-chunk score GEMM + Top-k kernel, and
    the fused kernel (run once over each span)."""
    old = msa.get_option(msa.OPT_INDEX_FUSED)
    msa.set_option(msa.OPT_INDEX_FUSED, request.param)
    yield request.param
    msa.set_option(msa.OPT_INDEX_FUSED, old)


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def assert_attn_close(O, O_ref, lse, lse_ref):
    O = np.asarray(O, dtype=np.float64)
    err = np.abs(O - O_ref).max()
    rel = np.linalg.norm(O - O_ref) / np.linalg.norm(O_ref)
    lerr = np.abs(np.asarray(lse, dtype=np.float64) - lse_ref).max()
    print(f"[prefill] O max-abs {err:.2e} rel-L2 {rel:.2e}, lse {lerr:.2e}", flush=True)
    assert np.isfinite(O).all()
    assert err <= ATOL and rel <= RTOL_L2 and lerr <= LSE_ATOL, (err, rel, lerr)


@pytest.mark.parametrize("splits,inner", [((1000, 2100, 3000), 0), ((1, 700, 3000), 512),
                                          ((2999, 3000), 0)])
def test_prefill_cached(oracle_lib, splits, inner, index_variant):
    """A 3000-token sequence arriving in pieces; each piece is attended with
    only its own Q/q_idx rows and a cache holding exactly the keys so far."""
    N, H_q, H_kv, d_h, d_idx, k = 3000, 16, 4, 64, 64, 6
    say("cached", splits, inner)
    t = make_prefill_inputs(N, H_q, H_kv, d_h, d_idx, n_hot=3, seed=91)
    u = {key: bf16_bits(v) for key, v in t.items()}
    scale = 1.0 / math.sqrt(d_h)
    q0 = 0
    for q1 in splits:
        # fresh, exactly-sized device buffers: nothing before the chunk's first
        # query row, nothing after the last cached key
        Qc = t["Q"][q0:q1].contiguous().cuda()
        qic = t["q_idx"][q0:q1].contiguous().cuda()
        Kc, Vc = t["K"][:q1].contiguous().cuda(), t["V"][:q1].contiguous().cuda()
        kic = t["k_idx"][:q1].contiguous().cuda()
        sel, O, lse = msa.prefill_cached(Qc, Kc, Vc, qic, kic, k, q_start=q0, chunk=inner,
                                         scale=scale)
        torch.cuda.synchronize()
        rows = np.arange(q0, q1)
        sel_ref, O_ref, lse_ref = oracle_lib.prefill_rows(u, rows, k, scale)
        np.testing.assert_array_equal(sel.cpu().numpy(), sel_ref)
        assert_attn_close(O.cpu().numpy(), O_ref, lse.cpu().numpy(), lse_ref)
        q0 = q1


@pytest.mark.parametrize("lens,inner", [((1000, 129, 1, 2600, 0, 777), 0),
                                        ((300, 2048, 513), 1024)])
def test_prefill_varlen(oracle_lib, lens, inner, index_variant):
    """Independently generated sequences packed back to back: each one's
    rows must equal the oracle on that sequence alone."""
    H_q, H_kv, d_h, d_idx, k = 8, 2, 128, 32, 5
    say("varlen", lens, inner)
    seqs = [make_prefill_inputs(L, H_q, H_kv, d_h, d_idx, n_hot=2, seed=100 + i)
            for i, L in enumerate(lens) if L > 0]
    packed = {key: torch.cat([s[key] for s in seqs]).cuda() for key in seqs[0]}
    cu = np.concatenate([[0], np.cumsum(lens)])
    scale = 1.0 / math.sqrt(d_h)
    sel, O, lse = msa.prefill_varlen(packed["Q"], packed["K"], packed["V"], packed["q_idx"],
                                     packed["k_idx"], cu.tolist(), k, chunk=inner, scale=scale)
    torch.cuda.synchronize()
    sel, O, lse = sel.cpu().numpy(), O.cpu().numpy(), lse.cpu().numpy()
    n = 0
    for b, L in enumerate(lens):
        if L == 0:
            continue
        s = seqs[n]
        n += 1
        u = {key: bf16_bits(v) for key, v in s.items()}
        rows = np.arange(L)
        sel_ref, O_ref, lse_ref = oracle_lib.prefill_rows(u, rows, k, scale)
        t0 = cu[b]
        np.testing.assert_array_equal(sel[t0:t0 + L], sel_ref)
        assert_attn_close(O[t0:t0 + L], O_ref, lse[t0:t0 + L], lse_ref)


def test_varlen_equals_per_sequence_prefill():
    """The batch gives each sequence bit for bit what msa_prefill gives it."""
    lens = (4096, 1500, 2222)
    H_q, H_kv, d_h, d_idx, k = 16, 4, 128, 64, 8
    say("varlen vs prefill", lens)
    seqs = [make_prefill_inputs(L, H_q, H_kv, d_h, d_idx, n_hot=4, seed=200 + i, device="cuda")
            for i, L in enumerate(lens)]
    packed = {key: torch.cat([s[key] for s in seqs]) for key in seqs[0]}
    cu = np.concatenate([[0], np.cumsum(lens)]).tolist()
    sel, O, lse = msa.prefill_varlen(packed["Q"], packed["K"], packed["V"], packed["q_idx"],
                                     packed["k_idx"], cu, k)
    for b, s in enumerate(seqs):
        sel1, O1, lse1 = msa.prefill(s["Q"], s["K"], s["V"], s["q_idx"], s["k_idx"], k)
        sl = slice(cu[b], cu[b + 1])
        assert torch.equal(sel[sl], sel1) and torch.equal(O[sl], O1) and torch.equal(lse[sl], lse1)
