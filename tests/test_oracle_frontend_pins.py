"""Pins for the oracle's Index Branch front-end (hidden -> Linear -> Norm &
RoPE -> Q^idx / K^idx; "MiniMax Sparse Attention" explainer, Figure 1
caption, RoPE width 64 from section 06).  The checks lean on torch's own
linear and rms_norm, on RoPE written as a complex rotation, and on the
invariants a correct RMS norm and rotary embedding must satisfy.
"""
import numpy as np
import pytest
import torch

import oracle
from block_sparse_long_idx_amd.synth import bf16_bits, make_frontend_inputs


def _inputs(N, d_model, H_kv, d_idx, seed):
    t = make_frontend_inputs(N, d_model, H_kv, d_idx, seed=seed)
    return t, {k: bf16_bits(t[k]) for k in ("hidden", "Wq", "Wk")}


def _torch_normed(t, W, gamma, H_kv, d_idx, eps=1e-6):
    y = torch.nn.functional.linear(t["hidden"].double(), t[W].double())
    y = y.view(y.shape[0], H_kv, d_idx)
    return torch.nn.functional.rms_norm(y, (d_idx,), weight=t[gamma].double(), eps=eps)


@pytest.mark.parametrize("d_idx,rope_dim", [(64, 64), (128, 64), (32, 32)])
def test_position_zero_is_linear_then_rms_norm(d_idx, rope_dim):
    """At position 0 every rotation is the identity: the output is torch's
    linear followed by torch's rms_norm."""
    N, d_model, H_kv = 96, 256, 4
    t, u = _inputs(N, d_model, H_kv, d_idx, seed=51)
    got = oracle.index_frontend(u["hidden"], u["Wq"], t["gq"].numpy(), np.zeros(N, np.int64),
                                H_kv, d_idx, rope_dim)
    ref = _torch_normed(t, "Wq", "gq", H_kv, d_idx).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("d_idx,rope_dim", [(64, 64), (128, 64), (32, 32)])
def test_rope_is_the_complex_rotation(d_idx, rope_dim):
    """Pair (j, j + rope_dim/2) as the complex number a + ib, multiplied by
    exp(i * pos * theta^(-2j/rope_dim)); entries past rope_dim unchanged."""
    N, d_model, H_kv, theta = 200, 128, 2, 10000.0
    t, u = _inputs(N, d_model, H_kv, d_idx, seed=52)
    pos = np.random.default_rng(3).integers(0, 1 << 20, N)
    got = oracle.index_frontend(u["hidden"], u["Wk"], t["gk"].numpy(), pos, H_kv, d_idx,
                                rope_dim, theta)
    y = _torch_normed(t, "Wk", "gk", H_kv, d_idx)
    half = rope_dim // 2
    freqs = 1.0 / theta ** (torch.arange(0, rope_dim, 2, dtype=torch.float64) / rope_dim)
    rot = torch.polar(torch.ones(N, half, dtype=torch.float64),
                      torch.from_numpy(pos).double()[:, None] * freqs[None, :])
    z = torch.complex(y[..., :half], y[..., half:rope_dim]) * rot[:, None, :]
    ref = y.clone()
    ref[..., :half] = z.real
    ref[..., half:rope_dim] = z.imag
    np.testing.assert_allclose(got, ref.numpy(), rtol=0, atol=1e-9)


def test_rope_scores_depend_on_relative_position_only():
    """<RoPE_p(u), RoPE_p'(v)> = <RoPE_{p+s}(u), RoPE_{p'+s}(v)>: the property
    that makes the index score a function of the distance."""
    rng = np.random.default_rng(4)
    u, v = rng.standard_normal((1, 1, 64)), rng.standard_normal((1, 1, 64))
    for p, q, s in [(5, 2, 100), (1000, 17, 70000), (0, 0, 12345)]:
        a = np.sum(oracle.frontend.rope(u, [p], 64, 1e4) * oracle.frontend.rope(v, [q], 64, 1e4))
        b = np.sum(oracle.frontend.rope(u, [p + s], 64, 1e4) * oracle.frontend.rope(v, [q + s], 64, 1e4))
        assert abs(a - b) < 1e-9 * (1 + abs(a))


def test_rms_norm_is_scale_free():
    """Scaling a token's hidden state leaves its normalised projection (and
    so the output) unchanged, up to the eps term."""
    N, d_model, H_kv, d_idx = 40, 128, 2, 64
    t, u = _inputs(N, d_model, H_kv, d_idx, seed=53)
    pos = np.arange(N) * 977
    a = oracle.index_frontend(u["hidden"], u["Wq"], t["gq"].numpy(), pos, H_kv, d_idx, eps=0.0)
    h2 = bf16_bits((t["hidden"].float() * 4.0).to(torch.bfloat16))   # exact in bf16
    b = oracle.index_frontend(h2, u["Wq"], t["gq"].numpy(), pos, H_kv, d_idx, eps=0.0)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)
    # and with gamma = 1 each group's vector has unit mean square
    c = oracle.index_frontend(u["hidden"], u["Wq"], np.ones(d_idx), np.zeros(N, np.int64), H_kv,
                              d_idx, eps=0.0)
    np.testing.assert_allclose(np.mean(c * c, axis=-1), 1.0, rtol=1e-12)
