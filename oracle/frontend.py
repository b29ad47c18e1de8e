"""Index Branch front-end oracle -- TEST INFRASTRUCTURE ONLY.

Plain fp64 numpy reference of the step that turns hidden states into the
index projections (MiniMax Sparse Attention explainer, Figure 1 caption:
hidden states pass a linear projection and then "Norm & RoPE" to give the
light-weight Q^idx and K^idx; section 06 gives the model's RoPE width of
64).  The pages fix neither the norm nor the RoPE variant; the readings
taken are the plain ones:

* Linear: y = x W^T with W stored [H_kv * d_idx, d_model] (one d_idx slice
  per GQA group), no bias.
* Norm: RMS normalisation of each group's d_idx vector,
  y * gamma / sqrt(mean(y^2) + eps), with one gamma of length d_idx shared
  by the groups.
* RoPE: rotate-half pairing over the first rope_dim entries, pair
  (j, j + rope_dim/2) turned by the angle pos * theta^(-2j/rope_dim),
  theta = 10000 by default; entries past rope_dim pass unchanged.

Only tests, ``__graft_entry__.smoke()`` and the benchmark's CPU leg may use
this module; it shares no code with the GPU library.
"""
from __future__ import annotations

import numpy as np


def _bf16_to_f64(bits):
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def linear(hidden, W):
    """x W^T in fp64 (the library matmul is the whole Linear step)."""
    return _bf16_to_f64(hidden) @ _bf16_to_f64(W).T


def rms_norm(y, gamma, eps):
    """RMS-normalise the last axis and scale by gamma."""
    ms = np.mean(y * y, axis=-1, keepdims=True)
    return y / np.sqrt(ms + eps) * np.asarray(gamma, dtype=np.float64)


def rope(y, pos, rope_dim, theta):
    """Rotate-half RoPE over the first rope_dim entries of the last axis.
    y [N, ..., d], pos [N] integer positions."""
    if rope_dim == 0:
        return y
    half = rope_dim // 2
    j = np.arange(half, dtype=np.float64)
    inv_freq = theta ** (-2.0 * j / rope_dim)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv_freq[None, :]
    shape = (y.shape[0],) + (1,) * (y.ndim - 2) + (half,)
    c, s = np.cos(ang).reshape(shape), np.sin(ang).reshape(shape)
    out = y.copy()
    a, b = y[..., :half], y[..., half:rope_dim]
    out[..., :half] = a * c - b * s
    out[..., half:rope_dim] = b * c + a * s
    return out


def index_frontend(hidden, W, gamma, pos, H_kv, d_idx, rope_dim=64, theta=10000.0, eps=1e-6):
    """hidden [N, d_model] and W [H_kv*d_idx, d_model] as bf16 bit patterns,
    gamma [d_idx], pos [N]: the fp64 projection [N, H_kv, d_idx] before any
    rounding to bf16."""
    N = hidden.shape[0]
    y = linear(hidden, W).reshape(N, H_kv, d_idx)
    y = rms_norm(y, gamma, eps)
    return rope(y, pos, min(rope_dim, d_idx), theta)
