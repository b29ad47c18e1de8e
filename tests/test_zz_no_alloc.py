"""msa_decode_static (decode with the library's fixed device scratch, no
workspace and no allocation) against msa_decode with a caller workspace,
through the C ABI.  Both run the same kernels, so selections and outputs
must agree bit for bit.  Two calls in a row, the second on a smaller input,
since every call on a GPU shares that GPU's scratch."""
import math
import sys

import pytest
import torch

from block_sparse_long_idx_amd import msa
from block_sparse_long_idx_amd.synth import make_decode_inputs

pytestmark = pytest.mark.gpu


def _outputs(B, H_q, H_kv, d_h, k, dev):
    return (torch.full((B, H_kv, k), -7, dtype=torch.int32, device=dev),
            torch.full((B, H_q, d_h), float("nan"), dtype=torch.float32, device=dev),
            torch.full((B, H_q), float("nan"), dtype=torch.float32, device=dev))


def test_decode_static_matches_workspace_decode():
    dev = torch.device("cuda:0")
    cases = [
        # B, N, H_q, H_kv, d_h, d_idx, k, seed: the second is smaller
        (4, 70000, 64, 4, 128, 64, 16, 11),
        (2, 3000, 16, 4, 64, 32, 8, 12),
    ]
    for B, N, H_q, H_kv, d_h, d_idx, k, seed in cases:
        print("[case] decode_static", (B, N, H_q, H_kv, d_h, d_idx, k), flush=True)
        sys.stdout.flush()
        need = msa.decode_workspace_bytes(B, N, H_q, H_kv, d_h, d_idx, k)
        assert 0 < need <= msa.load().msa_decode_static_scratch_bytes()
        t = make_decode_inputs(B, N, H_q, H_kv, d_h, d_idx, seed=seed, device=dev)
        scale = 1.0 / math.sqrt(d_h)
        ref = msa.decode(t["q"], t["q_idx"], t["K"], t["V"], t["k_idx"], k, scale=scale)
        sel, O, lse = _outputs(B, H_q, H_kv, d_h, k, dev)
        msa.decode_static(t["q"], t["q_idx"], t["K"], t["V"], t["k_idx"], k, sel, O, lse,
                          scale=scale)
        torch.cuda.synchronize()
        assert torch.equal(sel, ref[0])
        assert torch.equal(O, ref[1])
        assert torch.equal(lse, ref[2])
