"""Pins for the oracle's index-alignment KL ("MiniMax Sparse Attention"
explainer, section 03 "KL Loss": on the token set of the selected blocks,
the student is the softmax of the index scores, the teacher is the mean of
the group's head attention distributions, and the loss is KL(teacher ||
student)).  Each check rests on mathematics the oracle does not share:
Gibbs' inequality, closed forms, a textbook scipy evaluation and exact
special cases.
"""
import math

import numpy as np
import pytest
from scipy.special import logsumexp, rel_entr, softmax

from block_sparse_long_idx_amd.synth import bf16_bits, make_prefill_inputs


def _inputs(N, H_q, H_kv, d_h, d_idx, seed, n_hot=0):
    t = make_prefill_inputs(N, H_q, H_kv, d_h, d_idx, n_hot=n_hot, seed=seed)
    return {k: bf16_bits(v) for k, v in t.items()}, {k: v.double().numpy() for k, v in t.items()}


def _tokens(sel_row, i, B_k=128):
    return [j for b in sel_row if b >= 0 for j in range(b * B_k, min((b + 1) * B_k, i + 1))]


def test_kl_vanishes_when_student_is_the_teacher(oracle_lib):
    """G = 1, index projections equal to the attention's (q_idx = Q, k_idx = K)
    and scale 1: the two distributions coincide, so KL = 0."""
    N, H, d = 640, 2, 64
    u, _ = _inputs(N, H, H, d, d, seed=31)
    rows = np.arange(0, N, 7)
    sel = oracle_lib.select(u["Q"][rows], u["K"], rows, 3)
    kl = oracle_lib.index_kl(u["Q"][rows], u["K"], u["Q"][rows], u["K"], sel, rows, scale=1.0)
    np.testing.assert_allclose(kl, 0.0, atol=1e-10)


def test_kl_is_nonnegative_and_positive_in_general(oracle_lib):
    """Gibbs' inequality: KL >= 0, and unrelated projections give KL > 0."""
    N = 700
    u, _ = _inputs(N, 8, 2, 32, 32, seed=32, n_hot=2)
    rows = np.arange(N)
    sel = oracle_lib.select(u["q_idx"], u["k_idx"], rows, 3)
    kl = oracle_lib.index_kl(u["q_idx"], u["k_idx"], u["Q"], u["K"], sel, rows,
                             scale=1 / math.sqrt(32))
    assert kl.min() >= -1e-12
    assert (kl[128:] > 1e-6).all()   # rows past the first block see > 1 token


def test_kl_uniform_teacher_closed_form(oracle_lib):
    """Q = 0 makes every head's attention uniform over T, so the teacher is
    U(T) and KL(U || u) = -ln|T| - mean_j ln u_j, ln u_j = s_j - logsumexp(s)."""
    N, H_q, H_kv, d_h, d_idx = 500, 4, 2, 32, 16
    u, f = _inputs(N, H_q, H_kv, d_h, d_idx, seed=33, n_hot=1)
    rows = np.arange(0, N, 3)
    Qz = np.zeros_like(u["Q"][rows])
    sel = oracle_lib.select(u["q_idx"][rows], u["k_idx"], rows, 2)
    kl = oracle_lib.index_kl(u["q_idx"][rows], u["k_idx"], Qz, u["K"], sel, rows, scale=0.2)
    for n, i in enumerate(rows):
        for r in range(H_kv):
            T = _tokens(sel[n, r], i)
            s = f["k_idx"][T, r, :] @ f["q_idx"][i, r, :]
            expect = -math.log(len(T)) - np.mean(s - logsumexp(s))
            assert abs(kl[n, r] - expect) < 1e-9, (i, r)


def test_kl_matches_a_scipy_evaluation(oracle_lib):
    """Brute force with scipy on a small case: per-head softmax, head mean,
    student softmax and rel_entr, all over the same token sets."""
    N, H_q, H_kv, d_h, d_idx, k = 400, 6, 2, 16, 8, 2
    u, f = _inputs(N, H_q, H_kv, d_h, d_idx, seed=34, n_hot=1)
    rows = np.arange(0, N, 5)
    scale = 0.3
    sel = oracle_lib.select(u["q_idx"][rows], u["k_idx"], rows, k)
    kl = oracle_lib.index_kl(u["q_idx"][rows], u["k_idx"], u["Q"][rows], u["K"], sel, rows,
                             scale=scale)
    G = H_q // H_kv
    for n, i in enumerate(rows):
        for r in range(H_kv):
            T = _tokens(sel[n, r], i)
            teacher = np.mean([softmax(scale * (f["K"][T, r, :] @ f["Q"][i, r * G + g, :]))
                               for g in range(G)], axis=0)
            student = softmax(f["k_idx"][T, r, :] @ f["q_idx"][i, r, :])
            expect = rel_entr(teacher, student).sum()
            assert abs(kl[n, r] - expect) < 1e-9 * max(1.0, abs(expect)), (i, r)


def test_kl_teacher_is_the_head_mean(oracle_lib):
    """Two identical heads in a group give the same teacher as one head: a
    group of copies must average to the copy (catches a sum in place of a
    mean, or a wrong head -> group map)."""
    N, d_h, d_idx = 450, 32, 16
    u, _ = _inputs(N, 2, 2, d_h, d_idx, seed=35, n_hot=1)
    rows = np.arange(0, N, 4)
    sel = oracle_lib.select(u["q_idx"][rows], u["k_idx"], rows, 2)
    one = oracle_lib.index_kl(u["q_idx"][rows], u["k_idx"], u["Q"][rows], u["K"], sel, rows,
                              scale=0.25)
    # heads (0, 0, 1, 1): group r gets two copies of head r
    Q2 = np.repeat(u["Q"][rows], 2, axis=1)
    two = oracle_lib.index_kl(u["q_idx"][rows], u["k_idx"], Q2, u["K"], sel, rows, scale=0.25)
    np.testing.assert_allclose(two, one, rtol=0, atol=1e-12)
