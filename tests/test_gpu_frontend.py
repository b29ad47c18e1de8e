"""GPU parity of the Index Branch front-end (msa_index_frontend: Linear,
per-group RMS norm and RoPE) against the fp64 oracle, through the C ABI.

The kernel accumulates in fp32 and rounds to bf16 once.  Its error before
that rounding scales with the size of the operands, not of the result: a
rotated entry a cos - b sin of a unit-RMS vector can be tiny while its
fp32 error is ~1e-6 (|a| + |b|).  Bar: |out - ref| <= 1 ulp_bf16 of
max(|ref|, 2^-6) -- one bf16 unit in the last place, or 2^-14 absolute
for entries below 2^-6 -- and at least EXACT_FRAC of the elements equal
to bf16(ref).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from block_sparse_long_idx_amd import msa
from block_sparse_long_idx_amd.synth import CONFIGS, bf16_bits, make_frontend_inputs, sample_rows

pytestmark = pytest.mark.gpu

EXACT_FRAC = 0.97


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def assert_bf16_close(got, ref):
    got = got.float().cpu().numpy().astype(np.float64)
    m, e = np.frexp(np.maximum(np.abs(ref), 2.0 ** -6))
    ulp = np.ldexp(1.0, e - 8)
    err = np.abs(got - ref)
    rounded = torch.from_numpy(ref).to(torch.float32).to(torch.bfloat16).float().numpy()
    exact = np.mean(got == rounded)
    small = np.abs(ref) < 2.0 ** -6
    print(f"[fe] max err/bound {np.max(err / ulp):.3f}, exact {exact:.4f}, max abs err on "
          f"|ref| < 2^-6: {np.max(err[small], initial=0):.2e}", flush=True)
    assert np.isfinite(got).all()
    assert (err <= ulp).all(), np.unravel_index(np.argmax(err / ulp), err.shape)
    assert exact >= EXACT_FRAC, exact


FE_CASES = [
    # N, d_model, H_kv, d_idx, rope_dim, pos0
    (1000, 256, 4, 64, 64, 0),
    (777, 512, 2, 128, 64, 12345),       # RoPE on half the entries, ragged row tile
    (300, 128, 1, 32, 32, 0),            # tiny: 32 columns in a 256-column tile
    (513, 3072, 4, 64, 64, 1048000),     # the model width; positions near 2^20
    (200, 64, 3, 64, 0, 7),              # no RoPE; 192 columns
    (130, 192, 64, 32, 32, 5),           # 2048 columns: eight column tiles
]


@pytest.mark.parametrize("case", FE_CASES, ids=lambda c: "N%d_dm%d_Hkv%d_di%d_R%d_p%d" % c)
def test_frontend(case):
    N, d_model, H_kv, d_idx, rope_dim, pos0 = case
    say("frontend", case)
    t = make_frontend_inputs(N, d_model, H_kv, d_idx, seed=N + d_model)
    d = {k: v.cuda() for k, v in t.items()}
    q, k = msa.index_frontend(d["hidden"], d["Wq"], d["Wk"], d["gq"], d["gk"], H_kv, d_idx,
                              pos0=pos0, rope_dim=rope_dim)
    torch.cuda.synchronize()
    pos = pos0 + np.arange(N)
    u = {key: bf16_bits(t[key]) for key in ("hidden", "Wq", "Wk")}
    for out, W, g in ((q, "Wq", "gq"), (k, "Wk", "gk")):
        ref = oracle.index_frontend(u["hidden"], u[W], t[g].numpy(), pos, H_kv, d_idx, rope_dim)
        assert_bf16_close(out, ref)


def test_frontend_1m_sampled_rows():
    """The 1M workload's front-end (hidden width 3072, positions 0..2^20-1)
    in the launch shape the benchmark times, checked on sampled rows."""
    cfg = CONFIGS["1m"]
    say("frontend 1m sampled")
    t = make_frontend_inputs(cfg.N, cfg.d_model, cfg.H_kv, cfg.d_idx, seed=cfg.seed + 29,
                             device="cuda")
    q, k = msa.index_frontend(t["hidden"], t["Wq"], t["Wk"], t["gq"], t["gk"], cfg.H_kv,
                              cfg.d_idx)
    torch.cuda.synchronize()
    rows = np.array(sample_rows(cfg.N, 384))
    rt = torch.from_numpy(rows).cuda()
    hid = bf16_bits(t["hidden"][rt])
    for out, W, g in ((q, "Wq", "gq"), (k, "Wk", "gk")):
        ref = oracle.index_frontend(hid, bf16_bits(t[W]), t[g].cpu().numpy(), rows, cfg.H_kv,
                                    cfg.d_idx)
        assert_bf16_close(out[rt], ref)


def test_frontend_feeds_the_index_branch(oracle_lib):
    """hidden -> front-end -> Top-k on the GPU against the oracle's
    selection on the same front-end outputs.  These index vectors are not
    integer-valued, so the GPU's fp32 block scores and the oracle's fp64
    ones may order two blocks differently when their scores agree to fp32
    rounding: selections must match except for blocks whose fp64 score is
    within SCORE_TOL of the boundary (k-th) score."""
    N, d_model, H_kv, d_idx, k = 2000, 256, 4, 64, 5
    SCORE_TOL = 1e-4
    say("frontend -> topk", N)
    t = make_frontend_inputs(N, d_model, H_kv, d_idx, seed=61, device="cuda")
    q, kx = msa.index_frontend(t["hidden"], t["Wq"], t["Wk"], t["gq"], t["gk"], H_kv, d_idx)
    sel = msa.index_topk(q, kx, k)
    torch.cuda.synchronize()
    rows = np.arange(0, N, 3)
    qb, kb = bf16_bits(q), bf16_bits(kx)
    ref = oracle_lib.select(qb[rows], kb, rows, k)
    got = sel.cpu().numpy()[rows]
    n_diff = 0
    for n, i in enumerate(rows):
        for r in range(H_kv):
            a, b = set(got[n, r].tolist()), set(ref[n, r].tolist())
            if a == b:
                continue
            n_diff += 1
            sc = oracle_lib.block_scores(qb[i], kb, int(i), r)
            lb = i // 128
            others = np.delete(sc, lb)
            kth = np.sort(others)[::-1][min(k - 1, len(others)) - 1]
            assert lb in a, (i, r)
            for blk in a ^ b:
                assert blk >= 0 and abs(sc[blk] - kth) <= SCORE_TOL * (1 + abs(kth)), (i, r, blk)
    print(f"[fe] selections differing at near-ties: {n_diff}", flush=True)
    assert n_diff <= len(rows) * H_kv // 100


def test_frontend_rejects_bad_shapes():
    t = make_frontend_inputs(64, 96, 1, 64, seed=1, device="cuda")
    with pytest.raises(RuntimeError):
        msa.index_frontend(t["hidden"], t["Wq"], t["Wk"], t["gq"], t["gk"], 1, 64)  # d_model 96
