"""CPU checks of the Python binding's argument validation.

The library addresses rows by position, so a tensor with the wrong dtype or
too few rows would be read past its end on the device.  The binding refuses
such calls with ValueError before anything reaches libmsa.  The device check
is bypassed here (CPU tensors), so every case must fail on dtype or shape.
"""
import pytest
import torch

from block_sparse_long_idx_amd import msa

bf16 = torch.bfloat16


@pytest.fixture(autouse=True)
def _no_device_check(monkeypatch):
    monkeypatch.setattr(msa, "_need_cuda", lambda *ts: None)


def _t(shape, dtype=bf16):
    return torch.zeros(shape, dtype=dtype)


def _prefill_args(N=256, H_q=8, H_kv=2, d_h=64, d_idx=32):
    return dict(Q=_t((N, H_q, d_h)), K=_t((N, H_kv, d_h)), V=_t((N, H_kv, d_h)),
                q_idx=_t((N, H_kv, d_idx)), k_idx=_t((N, H_kv, d_idx)))


@pytest.mark.parametrize("bad", [
    dict(Q=_t((256, 8, 64), torch.float32)),        # fp32 Q
    dict(K=_t((200, 2, 64))),                       # K shorter than Q
    dict(V=_t((256, 2, 128))),                      # V head dim differs
    dict(q_idx=_t((256, 2, 64))),                   # q_idx width differs from k_idx
    dict(k_idx=_t((256, 2, 32), torch.float16)),    # fp16 index keys
    dict(O=_t((256, 8, 64), bf16)),                 # bf16 output
    dict(lse=_t((255, 8), torch.float32)),          # lse one row short
    dict(sel=_t((256, 2, 5), torch.int32)),         # sel width is not k
])
def test_prefill_rejects(bad):
    a = _prefill_args()
    a.update(bad)
    with pytest.raises(ValueError):
        msa.prefill(a["Q"], a["K"], a["V"], a["q_idx"], a["k_idx"], 4,
                    sel=a.get("sel"), O=a.get("O"), lse=a.get("lse"))


def test_index_topk_rejects_short_rows():
    q = _t((300, 2, 32))
    k = _t((300, 2, 32))
    with pytest.raises(ValueError):
        msa.index_topk(q, k, 4, q_start=200, Nq=200)     # rows 200..399 > 300
    with pytest.raises(ValueError):
        msa.index_topk(q.float(), k, 4)


def test_sparse_attn_rejects_short_csr():
    Q, K, V = _t((512, 4, 64)), _t((512, 1, 64)), _t((512, 1, 64))
    nnz = msa.selection_nnz(0, 512, 1, 4)
    rp = _t((1 * 4 + 1,), torch.int32)
    col = _t((nnz - 1,), torch.int32)          # one entry short
    slot = _t((nnz,), torch.uint8)
    with pytest.raises(ValueError):
        msa.sparse_attn_fwd(Q, K, V, rp, col, slot, 4)
    with pytest.raises(ValueError):                # int64 row_ptr
        msa.sparse_attn_fwd(Q, K, V, rp.long(), _t((nnz,), torch.int32), slot, 4)


def test_decode_rejects_mismatch():
    B, N = 2, 1000
    q, qi = _t((B, 8, 64)), _t((B, 2, 32))
    K, V, ki = _t((B, N, 2, 64)), _t((B, N, 2, 64)), _t((B, N, 2, 32))
    with pytest.raises(ValueError):
        msa.decode(q, qi, K, _t((B, N - 1, 2, 64)), ki, 4)
    with pytest.raises(ValueError):
        msa.decode(_t((B + 1, 8, 64)), qi, K, V, ki, 4)
    with pytest.raises(ValueError):
        msa.decode(q, qi, K, V, ki.float(), 4)


def test_frontend_rejects_weight_shape():
    h = _t((100, 128))
    W = _t((2 * 32, 128))
    g = _t((32,), torch.float32)
    with pytest.raises(ValueError):
        msa.index_frontend(h, W, _t((2 * 32, 64)), g, g, 2, 32)
    with pytest.raises(ValueError):
        msa.index_frontend(h, W, W, g.double(), g, 2, 32)


def test_backward_rejects_dO_dtype():
    N, H_q, H_kv, d = 256, 4, 1, 64
    Q, K, V = _t((N, H_q, d)), _t((N, H_kv, d)), _t((N, H_kv, d))
    O, lse = _t((N, H_q, d), torch.float32), _t((N, H_q), torch.float32)
    nnz = msa.selection_nnz(0, N, H_kv, 4)
    rp, col, slot = _t((3,), torch.int32), _t((nnz,), torch.int32), _t((nnz,), torch.uint8)
    with pytest.raises(ValueError):
        msa.sparse_attn_bwd(Q, K, V, O, lse, _t((N, H_q, d), torch.float32), rp, col, slot, 4)
