"""Seeded synthetic inputs for the MSA forward path.

This module only draws random tensors with the shapes and value
distributions of the MSA workloads; it holds none of the method's
arithmetic, so both the GPU path and the CPU oracle may consume what it
produces.

Workload shapes follow the MiniMax Sparse Attention write-up
(minimax-sparse-attention-danialwang.pages.dev): 64 query heads, 4 KV
heads, head dim 128 (section 06, model description), block size 128 and
k = 16 blocks per (query, group) (section 04, complexity).  The index
inputs are integer-valued bf16 so that every index score is exact in
fp32; that makes block selection comparable bit for bit.

Recipe (all draws from one ``torch.Generator`` seeded with ``seed``, in
this order):
  Q ~ bf16(N(0,1)) [N, H_q, d_h]; K, V ~ bf16(N(0,1)) [N, H_kv, d_h];
  q_idx, k_idx ~ bf16(uniform integer in {-3..3}) [N, H_kv, d_idx];
  then, per group r, ``n_hot`` distinct blocks from ``randperm(nblk)``
  whose 128 tokens get +2 added to k_idx[:, r, :] (values stay integers
  in [-1, 5]).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

B_K = 128


@dataclasses.dataclass(frozen=True)
class MsaConfig:
    name: str
    N: int
    H_q: int
    H_kv: int
    d_h: int
    d_idx: int
    k: int
    B_k: int = B_K
    n_hot: int = 0
    chunk: Optional[int] = None  # query chunk for prefill (None = whole N)
    batch: int = 1               # decode: number of sequences
    decode: bool = False
    seed: int = 1000
    d_model: int = 3072          # hidden width feeding the index front-end (section 06)

    @property
    def G(self) -> int:
        return self.H_q // self.H_kv

    @property
    def nblk(self) -> int:
        return (self.N + self.B_k - 1) // self.B_k

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d_h)


# The five workloads: tiny, 8K, 128K, 1M prefill and 32 x 1M decode.
CONFIGS = {
    "tiny": MsaConfig("tiny", N=1024, H_q=4, H_kv=1, d_h=64, d_idx=32, k=4,
                      n_hot=0, seed=1001),
    "8k": MsaConfig("8k", N=8192, H_q=64, H_kv=4, d_h=128, d_idx=64, k=16,
                    n_hot=8, seed=1002),
    "128k": MsaConfig("128k", N=131072, H_q=64, H_kv=4, d_h=128, d_idx=64,
                      k=16, n_hot=32, seed=1003),
    "1m": MsaConfig("1m", N=1048576, H_q=64, H_kv=4, d_h=128, d_idx=64, k=16,
                    n_hot=64, chunk=65536, seed=1004),
    "decode_1m": MsaConfig("decode_1m", N=1048576, H_q=64, H_kv=4, d_h=128,
                           d_idx=64, k=16, n_hot=0, batch=32, decode=True,
                           seed=1005),
}


def _randn_bf16(shape, gen, device):
    return torch.randn(shape, generator=gen, device=device,
                       dtype=torch.bfloat16)


def _randint_bf16(shape, gen, device):
    # uniform over the 7 integers -3..3, stored exactly in bf16
    return torch.randint(-3, 4, shape, generator=gen, device=device,
                         dtype=torch.int8).to(torch.bfloat16)


def make_prefill_inputs(N, H_q, H_kv, d_h, d_idx, *, n_hot=0, seed=0,
                        device="cpu", B_k=B_K):
    """Return dict(Q, K, V, q_idx, k_idx) of bf16 tensors, token-major."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    Q = _randn_bf16((N, H_q, d_h), gen, device)
    K = _randn_bf16((N, H_kv, d_h), gen, device)
    V = _randn_bf16((N, H_kv, d_h), gen, device)
    q_idx = _randint_bf16((N, H_kv, d_idx), gen, device)
    k_idx = _randint_bf16((N, H_kv, d_idx), gen, device)
    if n_hot:
        nblk = (N + B_k - 1) // B_k
        for r in range(H_kv):
            hot = torch.randperm(nblk, generator=gen, device=device)[:n_hot]
            for b in hot.tolist():
                k_idx[b * B_k:(b + 1) * B_k, r, :] += 2
    return dict(Q=Q, K=K, V=V, q_idx=q_idx, k_idx=k_idx)


def make_grad_output(N, H_q, d_h, *, seed=0, device="cpu"):
    """A seeded standard-normal bf16 output gradient dO [N, H_q, d_h]."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    return _randn_bf16((N, H_q, d_h), gen, device)


def make_frontend_inputs(N, d_model, H_kv, d_idx, *, seed=0, device="cpu"):
    """Hidden states and synthetic index-projection weights:
    hidden [N, d_model] bf16 ~ N(0, 1); Wq, Wk [H_kv*d_idx, d_model] bf16
    ~ N(0, 1/d_model); gq, gk [d_idx] fp32 ~ 1 + 0.1 N(0, 1)."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    hidden = _randn_bf16((N, d_model), gen, device)
    s = d_model ** -0.5
    Wq = (torch.randn((H_kv * d_idx, d_model), generator=gen, device=device) * s).to(torch.bfloat16)
    Wk = (torch.randn((H_kv * d_idx, d_model), generator=gen, device=device) * s).to(torch.bfloat16)
    gq = 1.0 + 0.1 * torch.randn((d_idx,), generator=gen, device=device)
    gk = 1.0 + 0.1 * torch.randn((d_idx,), generator=gen, device=device)
    return dict(hidden=hidden, Wq=Wq, Wk=Wk, gq=gq, gk=gk)


def make_decode_inputs(B, N, H_q, H_kv, d_h, d_idx, *, seed=0, device="cpu",
                       seqs=None):
    """Decode inputs for a batch of B sequences, each with an N-token cache.

    Sequence b is drawn from its own generator seeded ``seed * 5 + b`` so a
    single sequence can be regenerated alone.  ``seqs`` restricts which
    sequences are materialised (default: all).  Returns dict of stacked
    tensors q [B', H_q, d_h], q_idx [B', H_kv, d_idx], K, V [B', N, H_kv,
    d_h], k_idx [B', N, H_kv, d_idx].
    """
    seqs = list(range(B)) if seqs is None else list(seqs)
    nb = len(seqs)
    out = dict(
        q=torch.empty((nb, H_q, d_h), dtype=torch.bfloat16, device=device),
        q_idx=torch.empty((nb, H_kv, d_idx), dtype=torch.bfloat16,
                          device=device),
        K=torch.empty((nb, N, H_kv, d_h), dtype=torch.bfloat16, device=device),
        V=torch.empty((nb, N, H_kv, d_h), dtype=torch.bfloat16, device=device),
        k_idx=torch.empty((nb, N, H_kv, d_idx), dtype=torch.bfloat16,
                          device=device),
    )
    for n, b in enumerate(seqs):
        gen = torch.Generator(device=device)
        gen.manual_seed(seed * 5 + b)
        out["q"][n] = _randn_bf16((H_q, d_h), gen, device)
        out["K"][n] = _randn_bf16((N, H_kv, d_h), gen, device)
        out["V"][n] = _randn_bf16((N, H_kv, d_h), gen, device)
        out["q_idx"][n] = _randint_bf16((H_kv, d_idx), gen, device)
        out["k_idx"][n] = _randint_bf16((N, H_kv, d_idx), gen, device)
    return out


def inputs_for(cfg: MsaConfig, device="cpu", seqs=None):
    if cfg.decode:
        return make_decode_inputs(cfg.batch, cfg.N, cfg.H_q, cfg.H_kv, cfg.d_h,
                                  cfg.d_idx, seed=cfg.seed, device=device,
                                  seqs=seqs)
    return make_prefill_inputs(cfg.N, cfg.H_q, cfg.H_kv, cfg.d_h, cfg.d_idx,
                               n_hot=cfg.n_hot, seed=cfg.seed, device=device,
                               B_k=cfg.B_k)


def sample_rows(N: int, S: int):
    """S query rows spread evenly over [0, N-1], including both ends."""
    if S >= N:
        return list(range(N))
    return sorted(set(int(round(x)) for x in
                      torch.linspace(0, N - 1, S, dtype=torch.float64).tolist()))


def bf16_bits(t: torch.Tensor):
    """bf16 tensor -> numpy uint16 array of its bit patterns (host copy)."""
    import numpy as np
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
