"""Pins for the oracle's Main Branch backward (gradients of exact softmax
attention over each row's selected token set; "MiniMax Sparse Attention"
explainer, section 02).  Checked against torch autograd in float64 -- an
independent implementation of the same calculus -- and against two exact
sums every softmax-attention backward satisfies.
"""
import math

import numpy as np
import pytest
import torch

from block_sparse_long_idx_amd.synth import bf16_bits, make_prefill_inputs


def _inputs(N, H_q, H_kv, d_h, d_idx, seed, n_hot=0):
    t = make_prefill_inputs(N, H_q, H_kv, d_h, d_idx, n_hot=n_hot, seed=seed)
    g = torch.Generator().manual_seed(seed + 1)
    t["dO"] = torch.randn((N, H_q, d_h), generator=g).to(torch.bfloat16)
    return t, {k: bf16_bits(v) for k, v in t.items()}


def _mask_from_sel(sel, N, B_k=128):
    """[H_kv, N, N] boolean: token j is in row i's selected set for group r."""
    H_kv = sel.shape[1]
    M = np.zeros((H_kv, N, N), dtype=bool)
    for i in range(N):
        for r in range(H_kv):
            for b in sel[i, r]:
                if b >= 0:
                    M[r, i, b * B_k:min((b + 1) * B_k, i + 1)] = True
    return M


def _torch_grads(t, M, scale):
    """Masked softmax attention in float64 with torch autograd."""
    Q = t["Q"].double().requires_grad_(True)
    K = t["K"].double().requires_grad_(True)
    V = t["V"].double().requires_grad_(True)
    N, H_q, d_h = Q.shape
    H_kv = K.shape[1]
    G = H_q // H_kv
    Kh = K.repeat_interleave(G, dim=1)   # [N, H_q, d]
    Vh = V.repeat_interleave(G, dim=1)
    S = torch.einsum("ihd,jhd->hij", Q, Kh) * scale
    Mh = torch.from_numpy(M).repeat_interleave(G, dim=0)
    S = S.masked_fill(~Mh, float("-inf"))
    P = torch.softmax(S, dim=-1)
    O = torch.einsum("hij,jhd->ihd", P, Vh)
    (O * t["dO"].double()).sum().backward()
    return Q.grad.numpy(), K.grad.numpy(), V.grad.numpy()


def test_backward_dense_reduction_matches_torch_sdpa(oracle_lib):
    """k * B_k covers every row's prefix: MSA is dense causal GQA, whose
    gradients torch's SDPA autograd gives directly."""
    N, H_q, H_kv, d_h, k = 384, 4, 2, 32, 3
    t, u = _inputs(N, H_q, H_kv, d_h, 16, seed=41)
    rows = np.arange(N)
    sel = oracle_lib.select(u["q_idx"], u["k_idx"], rows, k)
    scale = 1 / math.sqrt(d_h)
    dQ, dK, dV = oracle_lib.attend_backward(u["Q"], u["K"], u["V"], u["dO"], sel, scale)
    Q = t["Q"].double().permute(1, 0, 2).unsqueeze(0).requires_grad_(True)
    K = t["K"].double().permute(1, 0, 2).unsqueeze(0).requires_grad_(True)
    V = t["V"].double().permute(1, 0, 2).unsqueeze(0).requires_grad_(True)
    G = H_q // H_kv
    O = torch.nn.functional.scaled_dot_product_attention(
        Q, K.repeat_interleave(G, dim=1), V.repeat_interleave(G, dim=1), is_causal=True,
        scale=scale)
    (O * t["dO"].double().permute(1, 0, 2).unsqueeze(0)).sum().backward()
    np.testing.assert_allclose(dQ, Q.grad[0].permute(1, 0, 2).numpy(), rtol=0, atol=1e-10)
    np.testing.assert_allclose(dK, K.grad[0].permute(1, 0, 2).numpy(), rtol=0, atol=1e-10)
    np.testing.assert_allclose(dV, V.grad[0].permute(1, 0, 2).numpy(), rtol=0, atol=1e-10)


@pytest.mark.parametrize("N,H_q,H_kv,d_h,k,n_hot", [
    (700, 4, 2, 32, 2, 1),      # sparse: 2 of up to 6 blocks
    (900, 6, 2, 16, 3, 2),      # G = 3, ragged last block
])
def test_backward_sparse_matches_torch_masked_autograd(oracle_lib, N, H_q, H_kv, d_h, k, n_hot):
    t, u = _inputs(N, H_q, H_kv, d_h, 16, seed=N + k, n_hot=n_hot)
    rows = np.arange(N)
    sel = oracle_lib.select(u["q_idx"], u["k_idx"], rows, k)
    scale = 1 / math.sqrt(d_h)
    dQ, dK, dV = oracle_lib.attend_backward(u["Q"], u["K"], u["V"], u["dO"], sel, scale)
    tQ, tK, tV = _torch_grads(t, _mask_from_sel(sel, N), scale)
    np.testing.assert_allclose(dQ, tQ, rtol=0, atol=1e-10)
    np.testing.assert_allclose(dK, tK, rtol=0, atol=1e-10)
    np.testing.assert_allclose(dV, tV, rtol=0, atol=1e-10)


def test_backward_exact_sums(oracle_lib):
    """sum_j p_j = 1 gives sum_j dV[j, r] = sum over the group's (i, h) of dO;
    sum_j ds_j = dO.O - dO.O = 0 gives sum_j dK[j, r] = 0."""
    N, H_q, H_kv, d_h, k = 1000, 8, 2, 32, 3
    t, u = _inputs(N, H_q, H_kv, d_h, 16, seed=43, n_hot=2)
    rows = np.arange(N)
    sel = oracle_lib.select(u["q_idx"], u["k_idx"], rows, k)
    _, dK, dV = oracle_lib.attend_backward(u["Q"], u["K"], u["V"], u["dO"], sel, 0.17)
    dO = t["dO"].double().numpy()
    G = H_q // H_kv
    for r in range(H_kv):
        np.testing.assert_allclose(dV[:, r, :].sum(0), dO[:, r * G:(r + 1) * G, :].sum((0, 1)),
                                   rtol=0, atol=1e-9)
        np.testing.assert_allclose(dK[:, r, :].sum(0), 0.0, atol=1e-9)


def test_backward_dq_rows_matches_torch_on_sampled_rows(oracle_lib):
    """The rows-only dQ entry point (used where only sampled rows can be
    checked) against torch autograd on those rows."""
    N, H_q, H_kv, d_h, k = 800, 6, 2, 32, 3
    t, u = _inputs(N, H_q, H_kv, d_h, 16, seed=47, n_hot=2)
    rows = np.array([0, 5, 127, 128, 300, 511, 640, 799])
    sel = oracle_lib.select(u["q_idx"], u["k_idx"], np.arange(N), k)
    scale = 1 / math.sqrt(d_h)
    dq = oracle_lib.attend_backward_dq_rows(u["Q"][rows], u["K"], u["V"], u["dO"][rows],
                                            sel[rows], rows, scale)
    tQ, _, _ = _torch_grads(t, _mask_from_sel(sel, N), scale)
    np.testing.assert_allclose(dq, tQ[rows], rtol=0, atol=1e-10)
