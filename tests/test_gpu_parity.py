"""GPU parity of libmsa against the CPU oracle, through the C ABI.

Bar: block selections and the inverted index bit-exact; attention output
within max-abs 1e-2 and relative L2 5e-3 of the fp64 oracle; lse within
1e-3.  Inputs are seeded synthetic tensors (block_sparse_long_idx_amd.synth).
Each stage is also fed the oracle's own upstream result, so no oracle input
ever comes from the GPU path.
"""
import math
import sys

import numpy as np
import pytest
import torch

from block_sparse_long_idx_amd import msa
from block_sparse_long_idx_amd.synth import (CONFIGS, MsaConfig, bf16_bits,
                                             inputs_for, make_decode_inputs,
                                             make_prefill_inputs, sample_rows)

pytestmark = pytest.mark.gpu

ATOL, RTOL_L2, LSE_ATOL = 1e-2, 5e-3, 1e-3


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def assert_attn_close(O, O_ref, lse=None, lse_ref=None):
    O = np.asarray(O, dtype=np.float64)
    err = np.abs(O - O_ref).max()
    rel = np.linalg.norm(O - O_ref) / np.linalg.norm(O_ref)
    assert np.isfinite(O).all()
    assert err <= ATOL and rel <= RTOL_L2, (err, rel)
    if lse is not None:
        lerr = np.abs(np.asarray(lse, dtype=np.float64) - lse_ref).max()
        assert lerr <= LSE_ATOL, lerr


def _u16(t):
    return {k: bf16_bits(v) for k, v in t.items()}


def _dev(t):
    return {k: v.cuda() for k, v in t.items()}


# ----------------------------------------------------------------- stages
STAGE_CASES = [
    # N, H_q, H_kv, d_h, d_idx, k, n_hot, q_start, Nq
    (1024, 4, 1, 64, 32, 4, 0, 0, 1024),        # the tiny workload
    (1000, 8, 2, 128, 64, 4, 2, 0, 1000),       # ragged last block
    (2000, 16, 4, 64, 128, 5, 3, 700, 1300),    # unaligned q_start
    (5000, 6, 2, 128, 64, 32, 4, 0, 5000),      # k = 32, G = 3
    (777, 2, 2, 64, 32, 1, 0, 0, 777),          # k = 1: local block only
    (600, 64, 1, 128, 64, 3, 1, 0, 600),        # G = 64 (> 32 rows per position)
    # H_kv = 64: enough 512-query tiles for the 8-wave Index work-groups
    (2600, 64, 64, 64, 64, 8, 2, 0, 2600),
    (3000, 64, 64, 64, 32, 16, 3, 333, 2667),   # d_idx 32, unaligned q_start
]


@pytest.mark.parametrize("case", STAGE_CASES, ids=lambda c: "N%d_Hq%d_Hkv%d_dh%d_di%d_k%d_qs%d" % (c[0], c[1], c[2], c[3], c[4], c[5], c[7]))
def test_index_topk_stage(oracle_lib, case):
    N, H_q, H_kv, d_h, d_idx, k, n_hot, q_start, Nq = case
    say("index_topk", case)
    t = make_prefill_inputs(N, H_q, H_kv, d_h, d_idx, n_hot=n_hot, seed=N + k)
    u = _u16(t)
    rows = np.arange(q_start, q_start + Nq)
    ref = oracle_lib.select(u["q_idx"][rows], u["k_idx"], rows, k)
    d = _dev(t)
    old = msa.get_option(msa.OPT_INDEX_FUSED)
    try:
        for fused in (0, 1):
            msa.set_option(msa.OPT_INDEX_FUSED, fused)
            sel = msa.index_topk(d["q_idx"], d["k_idx"], k, q_start=q_start, Nq=Nq)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(sel.cpu().numpy(), ref, err_msg=f"fused={fused}")
    finally:
        msa.set_option(msa.OPT_INDEX_FUSED, old)


# Shapes that take the fused kernel's 128-queries-per-wave form (1024-query
# tiles, two Top-k lists per lane): chosen when ceil(Nq/1024) * H_kv covers
# every compute unit (256 on MI355X), d_idx <= 64 and k <= 16.  Both end in
# a ragged tile; the second starts off a block edge.
WIDE_CASES = [
    # N, H_kv, d_idx, k, n_hot, q_start, Nq
    (4200, 64, 64, 16, 3, 0, 4200),
    (4600, 64, 32, 8, 2, 700, 3900),
]


@pytest.mark.parametrize("case", WIDE_CASES, ids=lambda c: "N%d_Hkv%d_di%d_k%d_qs%d" % (c[0], c[1], c[2], c[3], c[5]))
def test_index_topk_wide_tiles(oracle_lib, case):
    N, H_kv, d_idx, k, n_hot, q_start, Nq = case
    say("index_topk wide tiles", case)
    t = make_prefill_inputs(N, H_kv, H_kv, 64, d_idx, n_hot=n_hot, seed=N + 5 * k)
    rows = np.arange(q_start, q_start + Nq)
    ref = oracle_lib.select(bf16_bits(t["q_idx"])[rows], bf16_bits(t["k_idx"]), rows, k)
    old = msa.get_option(msa.OPT_INDEX_FUSED)
    try:
        msa.set_option(msa.OPT_INDEX_FUSED, 1)
        sel = msa.index_topk(t["q_idx"].cuda(), t["k_idx"].cuda(), k, q_start=q_start, Nq=Nq)
        torch.cuda.synchronize()
    finally:
        msa.set_option(msa.OPT_INDEX_FUSED, old)
    np.testing.assert_array_equal(sel.cpu().numpy(), ref)


# Rows of more than 128 visible blocks, the two-kernel Top-k's thresholded
# path (shorter rows are ranked whole).  "tiled" makes every key block a copy
# of the first, so all of a query's blocks score alike, apart from blocks
# whose keys are doubled (they outscore the rest wherever a query's best key
# scores above zero).  More than 128 blocks then share the (k-1)-th best
# score, the LDS pack overflows and the register-list path runs; ties go to
# the lower block index.
TOPK_LONG_CASES = [
    # N, H_kv, d_idx, k, tiled, doubled blocks, q_start
    (20000, 2, 64, 16, False, (), 17000),
    (20000, 1, 32, 16, True, (), 18500),
    (20000, 2, 64, 32, True, (), 19000),
    (20000, 2, 32, 8, True, (5, 40, 77), 18000),
]


@pytest.mark.parametrize("case", TOPK_LONG_CASES,
                         ids=lambda c: "N%d_Hkv%d_di%d_k%d_tiled%d_hot%d" % (c[:5] + (len(c[5]),)))
def test_index_topk_long_rows(oracle_lib, case):
    N, H_kv, d_idx, k, tiled, hot, q_start = case
    say("index_topk long rows", case)
    t = make_prefill_inputs(N, H_kv, H_kv, 64, d_idx, seed=N + 7 * k)
    ki = t["k_idx"]
    if tiled:
        ki = ki[:128].repeat((N + 127) // 128, 1, 1)[:N].contiguous()
    for b in hot:
        ki[b * 128:(b + 1) * 128] *= 2
    qi = t["q_idx"]
    rows = np.arange(q_start, N)
    uq, uk = bf16_bits(qi), bf16_bits(ki)
    ref = oracle_lib.select(uq[rows], uk, rows, k)
    if tiled:
        # the case reaches the overflow path: the last row has more than 128
        # blocks scoring at least its (k-1)-th best
        i = N - 1
        P = oracle_lib.block_scores(uq[i], uk, i, 0)[:i // 128]
        assert (P >= np.sort(P)[::-1][k - 2]).sum() > 128
    old = msa.get_option(msa.OPT_INDEX_FUSED)
    try:
        for fused in (0, 1):
            msa.set_option(msa.OPT_INDEX_FUSED, fused)
            sel = msa.index_topk(qi.cuda(), ki.cuda(), k, q_start=q_start, Nq=N - q_start)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(sel.cpu().numpy(), ref, err_msg=f"fused={fused}")
    finally:
        msa.set_option(msa.OPT_INDEX_FUSED, old)


@pytest.mark.parametrize("case", STAGE_CASES, ids=lambda c: "N%d_k%d_qs%d" % (c[0], c[5], c[7]))
def test_invert_stage(oracle_lib, case):
    N, H_q, H_kv, d_h, d_idx, k, n_hot, q_start, Nq = case
    say("invert", case)
    t = make_prefill_inputs(N, H_q, H_kv, d_h, d_idx, n_hot=n_hot, seed=N + k)
    u = _u16(t)
    rows = np.arange(q_start, q_start + Nq)
    sel = oracle_lib.select(u["q_idx"][rows], u["k_idx"], rows, k)
    nblk = (q_start + Nq + 127) // 128
    rp, col, slot = oracle_lib.invert(sel, q_start, nblk)
    g_rp, g_col, g_slot = msa.invert_index(torch.from_numpy(sel).cuda(), q_start=q_start)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(g_rp.cpu().numpy(), rp)
    np.testing.assert_array_equal(g_col.cpu().numpy(), col)
    np.testing.assert_array_equal(g_slot.cpu().numpy(), slot)


@pytest.mark.parametrize("case", STAGE_CASES, ids=lambda c: "N%d_Hq%d_dh%d_k%d_qs%d" % (c[0], c[1], c[3], c[5], c[7]))
def test_attn_stage(oracle_lib, case):
    N, H_q, H_kv, d_h, d_idx, k, n_hot, q_start, Nq = case
    say("attn", case)
    t = make_prefill_inputs(N, H_q, H_kv, d_h, d_idx, n_hot=n_hot, seed=N + k)
    u = _u16(t)
    rows = np.arange(q_start, q_start + Nq)
    scale = 1.0 / math.sqrt(d_h)
    sel, O_ref, lse_ref = oracle_lib.prefill_rows(u, rows, k, scale)
    nblk = (q_start + Nq + 127) // 128
    rp, col, slot = oracle_lib.invert(sel, q_start, nblk)
    d = _dev(t)
    O, lse = msa.sparse_attn_fwd(
        d["Q"], d["K"], d["V"], torch.from_numpy(rp.astype(np.int32)).cuda(),
        torch.from_numpy(col.astype(np.int32)).cuda(),
        torch.from_numpy(slot.astype(np.uint8)).cuda(), k, q_start=q_start, Nq=Nq,
        scale=scale)
    torch.cuda.synchronize()
    assert_attn_close(O.cpu().numpy(), O_ref, lse.cpu().numpy(), lse_ref)


# --------------------------------------------------------------- end to end
E2E_CASES = [
    # N, H_q, H_kv, d_h, d_idx, k, n_hot, chunk
    (1024, 4, 1, 64, 32, 4, 0, 0),
    (2000, 16, 4, 64, 128, 5, 3, 384),
    (2000, 16, 4, 64, 128, 5, 3, 300),      # chunks not aligned to blocks
    (3000, 8, 2, 128, 64, 8, 2, 1000),
]


@pytest.fixture(params=[0, 1], ids=["twokernel", "fused"])
def index_variant(request):
    old = msa.get_option(msa.OPT_INDEX_FUSED)
    msa.set_option(msa.OPT_INDEX_FUSED, request.param)
    yield request.param
    msa.set_option(msa.OPT_INDEX_FUSED, old)


@pytest.mark.parametrize("case", E2E_CASES, ids=lambda c: "N%d_k%d_chunk%d" % (c[0], c[5], c[7]))
def test_prefill_end_to_end(oracle_lib, case, index_variant):
    N, H_q, H_kv, d_h, d_idx, k, n_hot, chunk = case
    say("prefill", case, "fused", index_variant)
    t = make_prefill_inputs(N, H_q, H_kv, d_h, d_idx, n_hot=n_hot, seed=7 * N + k)
    u = _u16(t)
    rows = np.arange(N)
    scale = 1.0 / math.sqrt(d_h)
    sel_ref, O_ref, lse_ref = oracle_lib.prefill_rows(u, rows, k, scale)
    d = _dev(t)
    sel, O, lse = msa.prefill(d["Q"], d["K"], d["V"], d["q_idx"], d["k_idx"], k,
                              scale=scale, chunk=chunk)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(sel.cpu().numpy(), sel_ref)
    assert_attn_close(O.cpu().numpy(), O_ref, lse.cpu().numpy(), lse_ref)


def test_prefill_is_deterministic():
    N, H_q, H_kv, d_h, d_idx, k = 3000, 16, 4, 128, 64, 8
    say("determinism", N)
    d = _dev(make_prefill_inputs(N, H_q, H_kv, d_h, d_idx, n_hot=3, seed=99))
    outs = []
    for _ in range(2):
        outs.append(msa.prefill(d["Q"], d["K"], d["V"], d["q_idx"], d["k_idx"], k,
                                chunk=1024))
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_prefill_chunking_does_not_change_results():
    N, H_q, H_kv, d_h, d_idx, k = 2500, 8, 2, 64, 64, 6
    say("chunk invariance", N)
    d = _dev(make_prefill_inputs(N, H_q, H_kv, d_h, d_idx, n_hot=2, seed=5))
    s1, O1, l1 = msa.prefill(d["Q"], d["K"], d["V"], d["q_idx"], d["k_idx"], k, chunk=0)
    s2, O2, l2 = msa.prefill(d["Q"], d["K"], d["V"], d["q_idx"], d["k_idx"], k, chunk=640)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2)
    assert torch.equal(O1, O2) and torch.equal(l1, l2)


# ------------------------------------------------------------------- decode
DECODE_CASES = [
    # B, N, H_q, H_kv, d_h, d_idx, k
    (3, 5000, 16, 4, 128, 64, 8),
    (2, 300, 8, 2, 64, 32, 4),          # fewer blocks than k
    (2, 4096, 64, 4, 128, 64, 16),
    (1, 129, 4, 1, 64, 128, 2),         # local block of one token
    # G > 16: scores in their own LDS buffer beside K, V and q
    (2, 3000, 64, 2, 128, 64, 8),       # G = 32
    (2, 2000, 64, 1, 64, 128, 4),       # G = 64, d_h 64
    (1, 4100, 64, 1, 128, 64, 16),      # G = 64, d_h 128 (the largest LDS footprint)
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: "B%d_N%d_k%d" % (c[0], c[1], c[6]))
def test_decode(oracle_lib, case):
    B, N, H_q, H_kv, d_h, d_idx, k = case
    say("decode", case)
    t = make_decode_inputs(B, N, H_q, H_kv, d_h, d_idx, seed=N)
    scale = 1.0 / math.sqrt(d_h)
    d = _dev(t)
    sel, O, lse = msa.decode(d["q"], d["q_idx"], d["K"], d["V"], d["k_idx"], k, scale=scale)
    torch.cuda.synchronize()
    sel, O, lse = sel.cpu().numpy(), O.cpu().numpy(), lse.cpu().numpy()
    for b in range(B):
        u = {n: bf16_bits(t[n][b]) for n in t}
        s_ref, O_ref, l_ref = oracle_lib.decode_one(u["q"], u["q_idx"], u["K"], u["V"],
                                                    u["k_idx"], k, scale)
        np.testing.assert_array_equal(sel[b], s_ref)
        assert_attn_close(O[b], O_ref, lse[b], l_ref)


# Decode over more than 128 blocks with every key block a copy of the first
# (all blocks score alike for each sequence), apart from sequence 1, whose
# blocks 7 and 150 have their keys doubled: the Top-k's threshold passes
# more than 128 blocks and its register-list path picks the lowest ids (and
# the doubled blocks first where the best key scores above zero).
def test_decode_ties(oracle_lib):
    B, N, H_q, H_kv, d_h, d_idx, k = 2, 20000, 16, 2, 128, 64, 16
    say("decode ties", (B, N, H_q, H_kv, d_h, d_idx, k))
    t = make_decode_inputs(B, N, H_q, H_kv, d_h, d_idx, seed=77)
    nb = (N + 127) // 128
    t["k_idx"] = t["k_idx"][:, :128].repeat(1, nb, 1, 1)[:, :N].contiguous()
    for blk in (7, 150):
        t["k_idx"][1, blk * 128:(blk + 1) * 128] *= 2
    scale = 1.0 / math.sqrt(d_h)
    d = _dev(t)
    sel, O, lse = msa.decode(d["q"], d["q_idx"], d["K"], d["V"], d["k_idx"], k, scale=scale)
    torch.cuda.synchronize()
    sel, O, lse = sel.cpu().numpy(), O.cpu().numpy(), lse.cpu().numpy()
    for b in range(B):
        u = {n: bf16_bits(t[n][b]) for n in t}
        s_ref, O_ref, l_ref = oracle_lib.decode_one(u["q"], u["q_idx"], u["K"], u["V"],
                                                    u["k_idx"], k, scale)
        if b == 0:
            assert (s_ref[:, :k - 1] == np.arange(k - 1)).all()  # all tied: lowest ids
        np.testing.assert_array_equal(sel[b], s_ref)
        assert_attn_close(O[b], O_ref, lse[b], l_ref)


# ------------------------------------------------------ full-size workloads
# Oracle results of the full-size workloads, shared by the two Index Branch
# variants (the inputs are seeded, so both runs see the same tensors).
_ORACLE_CACHE = {}


def _full_prefill_check(oracle_lib, cfg, n_rows, attn_rows=None):
    say("full prefill", cfg.name, "rows", n_rows)
    t = inputs_for(cfg, device="cuda")
    sel, O, lse = msa.prefill(t["Q"], t["K"], t["V"], t["q_idx"], t["k_idx"], cfg.k,
                              scale=cfg.scale, chunk=cfg.chunk or 0)
    torch.cuda.synchronize()
    rows = np.array(sample_rows(cfg.N, n_rows))
    rows_t = torch.from_numpy(rows).cuda()
    arows = rows if attn_rows is None else np.array(sample_rows(cfg.N, attn_rows))
    ar_t = torch.from_numpy(arows).cuda()
    key = (cfg.name, n_rows, attn_rows)
    if key not in _ORACLE_CACHE:
        k_idx = bf16_bits(t["k_idx"])
        say("oracle select", len(rows))
        sel_ref = oracle_lib.select(bf16_bits(t["q_idx"][rows_t]), k_idx, rows, cfg.k)
        sel_a = sel_ref if attn_rows is None else \
            oracle_lib.select(bf16_bits(t["q_idx"][ar_t]), k_idx, arows, cfg.k)
        say("oracle attend", len(arows))
        O_ref, lse_ref = oracle_lib.attend(bf16_bits(t["Q"][ar_t]), bf16_bits(t["K"]),
                                           bf16_bits(t["V"]), sel_a, arows, cfg.scale)
        _ORACLE_CACHE.clear()
        _ORACLE_CACHE[key] = (sel_ref, O_ref, lse_ref)
    sel_ref, O_ref, lse_ref = _ORACLE_CACHE[key]
    np.testing.assert_array_equal(sel[rows_t].cpu().numpy(), sel_ref)
    assert_attn_close(O[ar_t].cpu().numpy(), O_ref, lse[ar_t].cpu().numpy(), lse_ref)
    return t, sel


@pytest.mark.slow
def test_full_8k(oracle_lib, index_variant):
    """Every row of the 8K workload: selection, inverted index, O and lse."""
    cfg = CONFIGS["8k"]
    t, sel = _full_prefill_check(oracle_lib, cfg, cfg.N)
    # inverted index of the full selection, bit-exact
    sel_np = sel.cpu().numpy()
    rp, col, slot = oracle_lib.invert(sel_np, 0, cfg.nblk)
    g_rp, g_col, g_slot = msa.invert_index(torch.from_numpy(sel_np).cuda())
    np.testing.assert_array_equal(g_rp.cpu().numpy(), rp)
    np.testing.assert_array_equal(g_col.cpu().numpy(), col)
    np.testing.assert_array_equal(g_slot.cpu().numpy(), slot)


def test_full_128k(oracle_lib, index_variant):
    _full_prefill_check(oracle_lib, CONFIGS["128k"], 512)


@pytest.mark.slow
def test_full_1m(oracle_lib, index_variant):
    """The fused variant is the configuration the benchmark times: one
    Index Branch launch over all 1,048,576 queries, then the inverted index
    and the Main Branch per 65,536-query chunk."""
    _full_prefill_check(oracle_lib, CONFIGS["1m"], 256)


# The largest key range the library accepts: 16,384 blocks of 128 tokens.
# k = 32 runs the 64-queries-per-wave index kernel, k = 16 the
# 128-queries-per-wave one.
MAX_BLOCK_CASES = [
    MsaConfig("max_blocks_k32", N=16384 * 128, H_q=4, H_kv=1, d_h=64, d_idx=32,
              k=32, n_hot=16, chunk=131072, seed=1006),
    MsaConfig("max_blocks_k16", N=16384 * 128 - 77, H_q=8, H_kv=2, d_h=128,
              d_idx=64, k=16, n_hot=8, chunk=131072, seed=1007),
]


@pytest.mark.slow
@pytest.mark.parametrize("cfg", MAX_BLOCK_CASES, ids=lambda c: c.name)
def test_max_block_count(oracle_lib, index_variant, cfg):
    assert cfg.nblk == 16384
    _full_prefill_check(oracle_lib, cfg, 96)


@pytest.mark.slow
def test_decode_max_block_count(oracle_lib):
    B, N, H_q, H_kv, d_h, d_idx, k = 2, 16384 * 128, 8, 2, 128, 64, 32
    say("decode max blocks", B, N)
    t = make_decode_inputs(B, N, H_q, H_kv, d_h, d_idx, seed=1008, device="cuda")
    scale = 1.0 / math.sqrt(d_h)
    sel, O, lse = msa.decode(t["q"], t["q_idx"], t["K"], t["V"], t["k_idx"], k, scale=scale)
    torch.cuda.synchronize()
    for b in range(B):
        u = {n: bf16_bits(t[n][b]) for n in t}
        s_ref, O_ref, l_ref = oracle_lib.decode_one(u["q"], u["q_idx"], u["K"], u["V"],
                                                    u["k_idx"], k, scale)
        np.testing.assert_array_equal(sel[b].cpu().numpy(), s_ref)
        assert_attn_close(O[b].cpu().numpy(), O_ref, lse[b].cpu().numpy(), l_ref)


@pytest.mark.slow
def test_full_decode_1m(oracle_lib):
    cfg = CONFIGS["decode_1m"]
    say("full decode", cfg.name)
    t = inputs_for(cfg, device="cuda")
    sel, O, lse = msa.decode(t["q"], t["q_idx"], t["K"], t["V"], t["k_idx"], cfg.k,
                             scale=cfg.scale)
    torch.cuda.synchronize()
    sel, O, lse = sel.cpu(), O.cpu(), lse.cpu()
    for b in range(cfg.batch):
        say("oracle decode seq", b)
        u = {n: bf16_bits(t[n][b]) for n in t}
        s_ref, O_ref, l_ref = oracle_lib.decode_one(u["q"], u["q_idx"], u["K"], u["V"],
                                                    u["k_idx"], cfg.k, cfg.scale)
        np.testing.assert_array_equal(sel[b].cpu().numpy(), s_ref)
        assert_attn_close(O[b].cpu().numpy(), O_ref, lse[b].cpu().numpy(), l_ref)
