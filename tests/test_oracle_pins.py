"""Pins for the CPU oracle: checks against what the MSA pages and plain
mathematics fix, never against the oracle's own formulas retyped.

Source: MiniMax Sparse Attention explainer
(minimax-sparse-attention-danialwang.pages.dev).

  (a) dense reduction: when k*B_k covers every visible token, MSA is
      dense causal GQA attention (section 02 + section 01) -> textbook
      numpy softmax attention and torch's SDPA in float64.
  (b) order preservation: Top-k on raw block scores equals Top-k after a
      token softmax (section 05, part 1).
  (c) forced local block, cardinality min(k, lb+1) (Figure 1 caption).
  (d) brute force over every candidate block set.
  plus inverted-index invariants, closed forms and special cases.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from block_sparse_long_idx_amd.synth import (bf16_bits, make_prefill_inputs,
                                             make_decode_inputs)

HERE = os.path.dirname(os.path.abspath(__file__))


def _np_inputs(N, H_q, H_kv, d_h, d_idx, n_hot=0, seed=7):
    t = make_prefill_inputs(N, H_q, H_kv, d_h, d_idx, n_hot=n_hot, seed=seed)
    u16 = {k: bf16_bits(v) for k, v in t.items()}
    f64 = {k: v.double().numpy() for k, v in t.items()}
    return t, u16, f64


def _dense_causal_gqa_numpy(Q, K, V, scale):
    """Textbook dense causal GQA attention in fp64 (independent of the oracle)."""
    N, H_q, d_h = Q.shape
    H_kv = K.shape[1]
    G = H_q // H_kv
    O = np.zeros_like(Q)
    lse = np.zeros((N, H_q))
    mask = np.tril(np.ones((N, N), dtype=bool))
    for h in range(H_q):
        r = h // G
        S = (Q[:, h, :] @ K[:, r, :].T) * scale
        S = np.where(mask, S, -np.inf)
        m = S.max(axis=1, keepdims=True)
        E = np.exp(S - m)
        l = E.sum(axis=1, keepdims=True)
        O[:, h, :] = (E @ V[:, r, :]) / l
        lse[:, h] = (m + np.log(l))[:, 0]
    return O, lse


# --------------------------------------------------------------------- (a)
@pytest.mark.parametrize("N,H_q,H_kv,d_h,d_idx,k", [
    (512, 4, 2, 64, 32, 4),      # k*B_k = N exactly
    (1000, 8, 2, 32, 16, 8),     # ragged last block, k*B_k > N
    (1024, 4, 1, 64, 32, 8),     # the tiny workload's shapes with k = nblk
])
def test_dense_reduction_numpy(oracle_lib, N, H_q, H_kv, d_h, d_idx, k):
    t, u16, f64 = _np_inputs(N, H_q, H_kv, d_h, d_idx, seed=N + k)
    rows = np.arange(N)
    scale = 1.0 / math.sqrt(d_h)
    sel, O, lse = oracle_lib.prefill_rows(u16, rows, k, scale)
    # every visible block is selected
    nb = (N + 127) // 128
    for i in range(0, N, 37):
        got = sel[i, 0]
        assert list(got[got >= 0]) == list(range(i // 128 + 1))
    O_ref, lse_ref = _dense_causal_gqa_numpy(f64["Q"], f64["K"], f64["V"], scale)
    np.testing.assert_allclose(O, O_ref, rtol=0, atol=1e-10)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-10)
    assert nb <= k


def test_dense_reduction_torch_sdpa(oracle_lib):
    """Same reduction against a library routine: torch SDPA in float64."""
    N, H_q, H_kv, d_h, d_idx, k = 640, 8, 2, 64, 32, 5
    t, u16, f64 = _np_inputs(N, H_q, H_kv, d_h, d_idx, seed=3)
    scale = 1.0 / math.sqrt(d_h)
    _, O, _ = oracle_lib.prefill_rows(u16, np.arange(N), k, scale)
    G = H_q // H_kv
    q = torch.from_numpy(f64["Q"]).permute(1, 0, 2)
    kk = torch.from_numpy(f64["K"]).repeat_interleave(G, dim=1).permute(1, 0, 2)
    vv = torch.from_numpy(f64["V"]).repeat_interleave(G, dim=1).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(
        q, kk, vv, is_causal=True, scale=scale).permute(1, 0, 2).numpy()
    np.testing.assert_allclose(O, ref, rtol=0, atol=1e-10)


# --------------------------------------------------------------------- (b)
def _select_via_softmax(q_idx, k_idx, i, r, k, B_k=128):
    """Selection computed the slow way: token softmax (fp64), block max of
    the probabilities, then a stable sort by (probability desc, block asc)."""
    s = k_idx[: i + 1, r, :] @ q_idx[i, r, :]
    p = np.exp(s - s.max())
    p /= p.sum()
    lb = i // B_k
    pooled = np.array([p[b * B_k:min((b + 1) * B_k, i + 1)].max()
                       for b in range(lb)])
    order = np.lexsort((np.arange(lb), -pooled))   # primary: -pooled
    chosen = sorted(list(order[: k - 1]) + [lb])
    return chosen + [-1] * (k - len(chosen))


def test_order_preservation_softmax(oracle_lib):
    N, H_q, H_kv, d_h, d_idx, k = 1024, 4, 1, 64, 32, 4
    t, u16, f64 = _np_inputs(N, H_q, H_kv, d_h, d_idx, seed=11)
    rows = np.arange(N)
    sel = oracle_lib.select(u16["q_idx"], u16["k_idx"], rows, k)
    for i in range(N):
        ref = _select_via_softmax(f64["q_idx"], f64["k_idx"], i, 0, k)
        assert list(sel[i, 0]) == ref, i


# --------------------------------------------------------------------- (c)
@pytest.mark.parametrize("k", [1, 2, 4, 16])
def test_local_block_and_cardinality(oracle_lib, k):
    N, H_kv, d_idx = 3000, 3, 16
    t, u16, _ = _np_inputs(N, 3, H_kv, 16, d_idx, n_hot=4, seed=k)
    rows = np.arange(0, N, 7)
    sel = oracle_lib.select(u16["q_idx"][rows], u16["k_idx"], rows, k)
    for n, i in enumerate(rows):
        lb = i // 128
        for r in range(H_kv):
            row = sel[n, r]
            valid = row[row >= 0]
            assert len(valid) == min(k, lb + 1)
            assert (row[len(valid):] == -1).all()
            assert lb in valid
            assert (np.diff(valid) > 0).all()          # ascending, no dups
            assert valid.min() >= 0 and valid.max() <= lb


# --------------------------------------------------------------------- (d)
def _pooled_numpy(q_idx, k_idx, i, r, B_k=128):
    s = k_idx[: i + 1, r, :] @ q_idx[i, r, :]
    lb = i // B_k
    return np.array([s[b * B_k:min((b + 1) * B_k, i + 1)].max()
                     for b in range(lb + 1)])


def test_block_scores_against_numpy(oracle_lib):
    N, H_kv, d_idx = 2000, 2, 32
    t, u16, f64 = _np_inputs(N, 2, H_kv, 16, d_idx, n_hot=3, seed=5)
    for i in (0, 1, 127, 128, 255, 256, 999, 1999):
        for r in range(H_kv):
            P = oracle_lib.block_scores(u16["q_idx"][i], u16["k_idx"], i, r)
            np.testing.assert_array_equal(P, _pooled_numpy(f64["q_idx"],
                                                           f64["k_idx"], i, r))


def test_bruteforce_selection(oracle_lib):
    """Sel = the k-set containing the local block with the largest score
    sum; among equal sums the lexicographically smallest sorted tuple
    (which is exactly 'ties go to the lower block index')."""
    N, H_kv, d_idx, k = 1024, 2, 8, 4   # small d_idx => many score ties
    t, u16, f64 = _np_inputs(N, 2, H_kv, 16, d_idx, seed=21)
    rows = np.arange(0, N, 3)
    sel = oracle_lib.select(u16["q_idx"][rows], u16["k_idx"], rows, k)
    n_ties = 0
    for n, i in enumerate(rows):
        lb = i // 128
        for r in range(H_kv):
            P = _pooled_numpy(f64["q_idx"], f64["k_idx"], i, r)
            if lb < k:
                best = tuple(range(lb + 1))
            else:
                best, best_sum = None, -np.inf
                for comb in itertools.combinations(range(lb), k - 1):
                    ssum = P[list(comb)].sum()
                    tup = tuple(sorted(comb + (lb,)))
                    if ssum > best_sum or (ssum == best_sum and tup < best):
                        best, best_sum = tup, ssum
                n_ties += len(set(P[:lb])) < lb
            got = tuple(int(b) for b in sel[n, r] if b >= 0)
            assert got == best, (i, r, got, best)
    assert n_ties > 0   # the case exercised tie-breaking


# ----------------------------------------------------------- inverted index
def _nnz_closed_form(q_start, Nq, k, H_kv, B_k=128):
    return H_kv * sum(min(k, i // B_k + 1) for i in range(q_start, q_start + Nq))


@pytest.mark.parametrize("q_start,Nq,k", [(0, 1024, 4), (256, 700, 3),
                                          (0, 8192, 16)])
def test_invert_invariants(oracle_lib, q_start, Nq, k):
    H_kv, d_idx = 2, 16
    N = q_start + Nq
    t, u16, _ = _np_inputs(N, 2, H_kv, 16, d_idx, n_hot=5, seed=q_start + k)
    rows = np.arange(q_start, N)
    sel = oracle_lib.select(u16["q_idx"][rows], u16["k_idx"], rows, k)
    nblk = (N + 127) // 128
    row_ptr, col, slot = oracle_lib.invert(sel, q_start, nblk)
    assert len(col) == _nnz_closed_form(q_start, Nq, k, H_kv)
    if q_start == 0 and Nq % 128 == 0 and Nq // 128 >= k:
        nb = Nq // 128
        assert len(col) == H_kv * 128 * (k * (k - 1) // 2 + k * (nb - k + 1))
    assert row_ptr[0] == 0 and (np.diff(row_ptr) >= 0).all()
    # transpose back: rebuilds sel exactly
    back = -np.ones_like(sel)
    for bucket in range(H_kv * nblk):
        r, b = divmod(bucket, nblk)
        seg = slice(row_ptr[bucket], row_ptr[bucket + 1])
        c = col[seg]
        assert (np.diff(c) > 0).all()          # ascending positions
        for i, s in zip(c, slot[seg]):
            assert back[i - q_start, r, s] == -1
            back[i - q_start, r, s] = b
    np.testing.assert_array_equal(back, sel)


def test_invert_worked_example(oracle_lib):
    """Hand-built 3-query selection and its inverted index."""
    sel = np.array([[[0, -1]], [[0, 1]], [[1, 2]]], dtype=np.int32)
    row_ptr, col, slot = oracle_lib.invert(sel, 10, 3)
    assert list(row_ptr) == [0, 2, 4, 5]
    assert list(col) == [10, 11, 11, 12, 12]
    assert list(slot) == [0, 0, 1, 0, 1]


# ------------------------------------------------------------ special cases
def test_constant_values_give_constant_output(oracle_lib):
    N, H_q, H_kv, d_h, d_idx, k = 1500, 4, 2, 32, 16, 3
    t, u16, _ = _np_inputs(N, H_q, H_kv, d_h, d_idx, seed=9)
    Vc = torch.full_like(t["V"], 1.75)
    u16["V"] = bf16_bits(Vc)
    rows = np.arange(0, N, 11)
    _, O, _ = oracle_lib.prefill_rows(u16, rows, k, 0.2)
    np.testing.assert_allclose(O, 1.75, rtol=0, atol=1e-12)


def test_zero_query_gives_mean_of_selected_values(oracle_lib):
    N, H_q, H_kv, d_h, d_idx, k = 1500, 4, 2, 32, 16, 3
    t, u16, f64 = _np_inputs(N, H_q, H_kv, d_h, d_idx, seed=10)
    u16["Q"] = np.zeros_like(u16["Q"])
    rows = np.arange(0, N, 13)
    sel, O, lse = oracle_lib.prefill_rows(u16, rows, k, 0.125)
    G = H_q // H_kv
    for n, i in enumerate(rows):
        for h in range(H_q):
            r = h // G
            toks = [j for b in sel[n, r] if b >= 0
                    for j in range(b * 128, min(b * 128 + 128, i + 1))]
            np.testing.assert_allclose(O[n, h], f64["V"][toks, r].mean(axis=0),
                                       rtol=0, atol=1e-12)
            assert abs(lse[n, h] - math.log(len(toks))) < 1e-12


def test_lse_is_logsumexp_over_selected_tokens(oracle_lib):
    from scipy.special import logsumexp
    N, H_q, H_kv, d_h, d_idx, k = 2100, 4, 2, 64, 16, 4
    t, u16, f64 = _np_inputs(N, H_q, H_kv, d_h, d_idx, n_hot=3, seed=12)
    rows = np.array([0, 5, 130, 700, 2099])
    scale = 1 / 8
    sel, O, lse = oracle_lib.prefill_rows(u16, rows, k, scale)
    G = H_q // H_kv
    for n, i in enumerate(rows):
        for h in range(H_q):
            r = h // G
            toks = [j for b in sel[n, r] if b >= 0
                    for j in range(b * 128, min(b * 128 + 128, i + 1))]
            s = f64["K"][toks, r] @ f64["Q"][i, h] * scale
            assert abs(lse[n, h] - logsumexp(s)) < 1e-10
            w = np.exp(s - logsumexp(s))
            np.testing.assert_allclose(O[n, h], w @ f64["V"][toks, r], atol=1e-10)


def test_decode_equals_last_prefill_row(oracle_lib):
    B, N, H_q, H_kv, d_h, d_idx, k = 2, 1300, 8, 2, 64, 32, 4
    d = make_decode_inputs(B, N, H_q, H_kv, d_h, d_idx, seed=4)
    for b in range(B):
        u = {n: bf16_bits(d[n][b]) for n in ("q", "q_idx", "K", "V", "k_idx")}
        sel, O, lse = oracle_lib.decode_one(u["q"], u["q_idx"], u["K"], u["V"],
                                            u["k_idx"], k, 0.125)
        rows = np.array([N - 1])
        sel2 = oracle_lib.select(u["q_idx"][None], u["k_idx"], rows, k)
        O2, lse2 = oracle_lib.attend(u["q"][None], u["K"], u["V"], sel2, rows,
                                     0.125)
        np.testing.assert_array_equal(sel, sel2[0])
        np.testing.assert_array_equal(O, O2[0])
        np.testing.assert_array_equal(lse, lse2[0])
        assert sel[0, -1] == (N - 1) // 128


# --------------------------------------------------------------- golden
def test_golden_hand_worked_selection(oracle_lib):
    """A hand-worked selection with integer index vectors (fixture file
    states each step)."""
    with open(os.path.join(HERE, "golden", "hand_select.json")) as f:
        g = json.load(f)
    k_idx = np.array(g["k_idx"], dtype=np.float32)          # [N, 1, d]
    q_idx = np.array(g["q_idx"], dtype=np.float32)
    to16 = lambda a: bf16_bits(torch.from_numpy(a).to(torch.bfloat16))
    rows = np.array(g["rows"], dtype=np.int64)
    sel = oracle_lib.select(to16(q_idx[rows]), to16(k_idx), rows, g["k"],
                            B_k=g["B_k"])
    assert sel[:, 0, :].tolist() == g["expected_sel"]
    for i, P in zip(g["rows"], g["expected_block_scores"]):
        got = oracle_lib.block_scores(to16(q_idx[i]), to16(k_idx), i, 0,
                                      B_k=g["B_k"])
        assert got.tolist() == P
