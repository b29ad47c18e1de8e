"""CPU checks of the C ABI: the library loads, exports what include/msa.h
declares, sizes workspaces, and rejects bad arguments on the host before
any device work (none of these calls reaches the GPU)."""
import ctypes

import pytest

from block_sparse_long_idx_amd import msa

FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first
NULL = ctypes.c_void_p(0)


@pytest.fixture(scope="module")
def lib():
    return msa.load()


def test_exports_every_declared_symbol(lib):
    names = msa.header_functions()
    assert len(names) >= 14
    for name in names:
        assert hasattr(lib, name), name


def test_selection_nnz_closed_form(lib):
    for q_start, Nq, H_kv, k in [(0, 1024, 1, 4), (0, 8192, 4, 16), (300, 5000, 3, 7),
                                 (65536 * 3, 65536, 4, 16), (0, 1, 2, 1)]:
        brute = H_kv * sum(min(k, i // 128 + 1) for i in range(q_start, q_start + Nq))
        assert msa.selection_nnz(q_start, Nq, H_kv, k) == brute
    # the budget formula for aligned full-size sequences
    nb = 8192 // 128
    assert msa.selection_nnz(0, 8192, 1, 16) == 128 * (16 * 15 // 2 + 16 * (nb - 16 + 1))


def test_workspace_sizes(lib):
    assert lib.msa_index_topk_workspace_bytes(0, 8192, 4, 128, 16) >= 4 * 8192 * 64 * 4
    assert lib.msa_index_topk_workspace_bytes(0, 8192, 4, 64, 16) == 0   # unsupported B_k
    assert lib.msa_invert_index_workspace_bytes(0, 8192, 4, 128, 16) > 0
    assert lib.msa_sparse_attn_fwd_workspace_bytes(0, 8192, 64, 4, 128, 128, 16) > \
        2 * 8192 * 15 * 64 * 128
    assert lib.msa_sparse_attn_fwd_workspace_bytes(0, 8192, 64, 4, 96, 128, 16) == 0
    assert lib.msa_prefill_workspace_bytes(1 << 20, 65536, 64, 4, 128, 64, 128, 16) > 0
    assert lib.msa_decode_workspace_bytes(32, 1 << 20, 64, 4, 128, 64, 128, 16) > 0
    # decode's index scan needs H_kv * d_idx to divide 512
    assert lib.msa_decode_workspace_bytes(2, 1024, 12, 3, 128, 64, 128, 4) == 0
    assert lib.msa_decode_workspace_bytes(2, 1024, 64, 8, 128, 128, 128, 4) == 0


def _err(lib):
    return lib.msa_last_error().decode()


@pytest.mark.parametrize("args,status", [
    # q_idx, k_idx, q_start, Nq, Nk, H_kv, d_idx, B_k, k, sel, ws, ws_bytes
    ((FAKE, FAKE, 0, 0, 128, 1, 64, 128, 4, FAKE, FAKE, 1 << 30), msa.ERR_INVALID_ARG),
    ((FAKE, FAKE, 0, 128, 128, 1, 64, 64, 4, FAKE, FAKE, 1 << 30), msa.ERR_UNSUPPORTED),
    ((FAKE, FAKE, 0, 128, 128, 1, 64, 128, 33, FAKE, FAKE, 1 << 30), msa.ERR_UNSUPPORTED),
    ((FAKE, FAKE, 0, 128, 128, 1, 64, 128, 0, FAKE, FAKE, 1 << 30), msa.ERR_UNSUPPORTED),
    ((FAKE, FAKE, 0, 128, 128, 1, 48, 128, 4, FAKE, FAKE, 1 << 30), msa.ERR_UNSUPPORTED),
    ((NULL, FAKE, 0, 128, 128, 1, 64, 128, 4, FAKE, FAKE, 1 << 30), msa.ERR_INVALID_ARG),
    ((FAKE, FAKE, 0, 128, 100, 1, 64, 128, 4, FAKE, FAKE, 1 << 30), msa.ERR_INVALID_ARG),
    ((FAKE, FAKE, 0, 128, 128, 1, 64, 128, 4, FAKE, FAKE, 16), msa.ERR_WORKSPACE),
    ((FAKE, FAKE, 0, 1 << 22, 1 << 22, 1, 64, 128, 4, FAKE, FAKE, 1 << 40),
     msa.ERR_UNSUPPORTED),   # more than 16384 blocks
])
def test_index_topk_rejects(lib, args, status):
    # the two-kernel variant, which alone needs the score workspace; every
    # other check is the same for both
    old = msa.get_option(msa.OPT_INDEX_FUSED)
    msa.set_option(msa.OPT_INDEX_FUSED, 0)
    try:
        assert lib.msa_index_topk(*args, NULL) == status
        assert _err(lib)
    finally:
        msa.set_option(msa.OPT_INDEX_FUSED, old)


def test_index_fused_is_default(lib):
    assert msa.get_option(msa.OPT_INDEX_FUSED) == 1


def test_invert_rejects(lib):
    assert lib.msa_invert_index(NULL, 0, 128, 1, 128, 4, FAKE, FAKE, FAKE, FAKE, 1 << 30,
                                NULL) == msa.ERR_INVALID_ARG
    assert lib.msa_invert_index(FAKE, 0, 128, 1, 128, 4, FAKE, FAKE, FAKE, FAKE, 4,
                                NULL) == msa.ERR_WORKSPACE


def test_attn_rejects(lib):
    base = [FAKE] * 6
    # H_q not a multiple of H_kv
    assert lib.msa_sparse_attn_fwd(*base, 0, 128, 128, 6, 4, 128, 128, 4, 0.1, FAKE, NULL,
                                   FAKE, 1 << 30, NULL) == msa.ERR_INVALID_ARG
    # d_h unsupported
    assert lib.msa_sparse_attn_fwd(*base, 0, 128, 128, 8, 4, 96, 128, 4, 0.1, FAKE, NULL,
                                   FAKE, 1 << 30, NULL) == msa.ERR_UNSUPPORTED
    # more than 64 query heads per KV head
    assert lib.msa_sparse_attn_fwd(*base, 0, 128, 128, 130, 2, 128, 128, 4, 0.1, FAKE, NULL,
                                   FAKE, 1 << 30, NULL) == msa.ERR_UNSUPPORTED
    # bad scale
    assert lib.msa_sparse_attn_fwd(*base, 0, 128, 128, 8, 4, 128, 128, 4, -1.0, FAKE, NULL,
                                   FAKE, 1 << 30, NULL) == msa.ERR_INVALID_ARG
    # workspace too small
    assert lib.msa_sparse_attn_fwd(*base, 0, 128, 128, 8, 4, 128, 128, 4, 0.1, FAKE, NULL,
                                   FAKE, 8, NULL) == msa.ERR_WORKSPACE


def test_prefill_and_decode_reject(lib):
    five = [FAKE] * 5
    assert lib.msa_prefill(*five, 0, 0, 8, 4, 128, 64, 128, 4, 0.1, NULL, FAKE, NULL, FAKE,
                           1 << 30, NULL) == msa.ERR_INVALID_ARG
    assert lib.msa_prefill(*five, 1024, -1, 8, 4, 128, 64, 128, 4, 0.1, NULL, FAKE, NULL,
                           FAKE, 1 << 30, NULL) == msa.ERR_INVALID_ARG
    assert lib.msa_prefill(*five, 1024, 0, 8, 4, 128, 64, 128, 4, 0.1, NULL, FAKE, NULL,
                           FAKE, 64, NULL) == msa.ERR_WORKSPACE
    assert lib.msa_decode(*five, 2, 1024, 12, 3, 128, 64, 128, 4, 0.1, FAKE, FAKE, NULL,
                          FAKE, 1 << 30, NULL) == msa.ERR_UNSUPPORTED   # H_kv * d_idx = 192 does not divide 512
    assert lib.msa_decode(*five, 0, 1024, 8, 4, 128, 64, 128, 4, 0.1, FAKE, FAKE, NULL,
                          FAKE, 1 << 30, NULL) == msa.ERR_INVALID_ARG
    assert lib.msa_decode(*five, 2, 1024, 65, 1, 128, 64, 128, 4, 0.1, FAKE, FAKE, NULL,
                          FAKE, 1 << 30, NULL) == msa.ERR_UNSUPPORTED   # G = 65


def test_decode_static_limits(lib):
    """The fixed-scratch decode refuses, on the host, shapes whose decode
    workspace exceeds its scratch, and bad arguments, before any HIP call."""
    cap = lib.msa_decode_static_scratch_bytes()
    assert cap == 64 << 20
    assert lib.msa_decode_workspace_bytes(32, 1 << 20, 64, 4, 128, 64, 128, 16) <= cap
    big = (256, 1 << 21, 64, 4, 128, 64, 128, 32)
    assert lib.msa_decode_workspace_bytes(*big) > cap
    B, N, H_q, H_kv, d_h, d_idx, B_k, k = big
    five = (FAKE,) * 5
    assert lib.msa_decode_static(*five, B, N, H_q, H_kv, d_h, d_idx, B_k, k, 0.1, FAKE, FAKE,
                                 NULL, NULL) == msa.ERR_WORKSPACE
    assert "scratch" in _err(lib)
    assert lib.msa_decode_static(*five, 0, 1024, 8, 4, 128, 64, 128, 4, 0.1, FAKE, FAKE, NULL,
                                 NULL) == msa.ERR_INVALID_ARG
    assert lib.msa_decode_static(*five, 2, 1024, 12, 3, 128, 64, 128, 4, 0.1, FAKE, FAKE, NULL,
                                 NULL) == msa.ERR_UNSUPPORTED


def test_options(lib):
    assert msa.get_option(msa.OPT_ATTN_CHUNK) >= 1
    with pytest.raises(msa.MsaError):
        msa.set_option(99, 1)
    with pytest.raises(msa.MsaError):
        msa.set_option(msa.OPT_ATTN_CHUNK, 0)
    with pytest.raises(msa.MsaError):
        msa.set_option(msa.OPT_ATTN_CHUNK, 127)     # below the smallest work item
    # workspace sizes do not depend on the item size
    sizes = []
    for item in (128, 2048):
        old_item = msa.get_option(msa.OPT_ATTN_CHUNK)
        msa.set_option(msa.OPT_ATTN_CHUNK, item)
        sizes.append((lib.msa_sparse_attn_fwd_workspace_bytes(0, 65536, 64, 4, 128, 128, 16),
                      lib.msa_index_kl_workspace_bytes(0, 65536, 4, 128, 16),
                      lib.msa_prefill_workspace_bytes(1 << 20, 65536, 64, 4, 128, 64, 128, 16)))
        msa.set_option(msa.OPT_ATTN_CHUNK, old_item)
    assert sizes[0] == sizes[1]
    old = msa.get_option(msa.OPT_ATTN_CHUNK)
    msa.set_option(msa.OPT_ATTN_CHUNK, 512)
    assert msa.get_option(msa.OPT_ATTN_CHUNK) == 512
    msa.set_option(msa.OPT_ATTN_CHUNK, old)


@pytest.mark.parametrize("N,d_model,H_kv,d_idx,rope,theta,eps", [
    (0, 256, 4, 64, 64, 1e4, 1e-6),        # no rows
    (10, 96, 4, 64, 64, 1e4, 1e-6),        # d_model not a multiple of 64
    (10, 256, 4, 48, 32, 1e4, 1e-6),       # unsupported d_idx
    (10, 256, 4, 32, 64, 1e4, 1e-6),       # rope_dim > d_idx
    (10, 256, 4, 64, 16, 1e4, 1e-6),       # unsupported rope_dim
    (10, 256, 0, 64, 64, 1e4, 1e-6),       # no groups
    (10, 256, 4, 64, 64, 1.0, 1e-6),       # theta <= 1
    (10, 256, 4, 64, 64, 1e4, -1.0),       # negative eps
])
def test_frontend_rejects(lib, N, d_model, H_kv, d_idx, rope, theta, eps):
    st = lib.msa_index_frontend(FAKE, FAKE, FAKE, FAKE, FAKE, N, 0, d_model, H_kv, d_idx, rope,
                                theta, eps, FAKE, FAKE, NULL)
    assert st != msa.OK
    st = lib.msa_index_frontend(FAKE, NULL, FAKE, FAKE, FAKE, 10, 0, 256, 4, 64, 64, 1e4, 1e-6,
                                FAKE, FAKE, NULL)
    assert st == msa.ERR_INVALID_ARG


def test_varlen_and_cached_reject(lib):
    bad = [(0, 5, 3), (0, 5, 3, 2), (1, 5), (0, 0)]   # decreasing, cu[0] != 0, no tokens
    for cu in bad:
        arr = (ctypes.c_int64 * len(cu))(*cu)
        B = len(cu) - 1
        assert lib.msa_prefill_varlen_workspace_bytes(arr, B, 0, 16, 4, 128, 64, 128, 8) == 0
        st = lib.msa_prefill_varlen(FAKE, FAKE, FAKE, FAKE, FAKE, arr, B, 0, 16, 4, 128, 64,
                                    128, 8, 0.1, NULL, FAKE, NULL, FAKE, 1 << 30, NULL)
        assert st == msa.ERR_INVALID_ARG
    arr = (ctypes.c_int64 * 3)(0, 100, 300)
    assert lib.msa_prefill_varlen_workspace_bytes(arr, 2, 0, 16, 4, 128, 64, 128, 8) > 0
    # the cached form validates like the stage calls
    assert lib.msa_prefill_cached_workspace_bytes(1000, 500, 0, 16, 4, 128, 64, 128, 8) > 0
    assert lib.msa_prefill_cached_workspace_bytes(-1, 500, 0, 16, 4, 128, 64, 128, 8) == 0
    st = lib.msa_prefill_cached(FAKE, FAKE, FAKE, FAKE, FAKE, 1000, 0, 0, 16, 4, 128, 64, 128, 8,
                                0.1, NULL, FAKE, NULL, FAKE, 1 << 30, NULL)
    assert st == msa.ERR_INVALID_ARG


def test_empty_chunks_rejected(lib):
    """Every chunk-level entry point refuses Nq = 0 (and the front-end N = 0)
    on the host, before any device work."""
    E = msa.ERR_INVALID_ARG
    assert lib.msa_invert_index(FAKE, 0, 0, 4, 128, 16, FAKE, FAKE, FAKE, FAKE,
                                1 << 30, NULL) == E
    assert ">= 1" in _err(lib), _err(lib)
    assert lib.msa_sparse_attn_fwd(*[FAKE] * 6, 0, 0, 128, 8, 4, 128, 128, 4, 0.1, FAKE,
                                   NULL, FAKE, 1 << 30, NULL) == E
    assert ">= 1" in _err(lib), _err(lib)
    assert lib.msa_sparse_attn_bwd(*[FAKE] * 9, 0, 0, 128, 8, 4, 128, 128, 4, 0.1, FAKE,
                                   FAKE, FAKE, FAKE, 1 << 30, NULL) == E
    assert ">= 1" in _err(lib), _err(lib)
    assert lib.msa_index_kl(*[FAKE] * 8, 0, 0, 128, 8, 4, 128, 64, 128, 4, 0.1, FAKE,
                            NULL, FAKE, 1 << 30, NULL) == E
    assert ">= 1" in _err(lib), _err(lib)
    assert lib.msa_prefill_cached(*[FAKE] * 5, 128, 0, 0, 8, 4, 128, 64, 128, 4, 0.1, NULL,
                                  FAKE, NULL, FAKE, 1 << 30, NULL) == E
    assert ">= 1" in _err(lib), _err(lib)
    assert lib.msa_index_frontend(*[FAKE] * 5, 0, 0, 256, 4, 64, 64, 1e4, 1e-6, FAKE, FAKE,
                                  NULL) == E
    assert ">= 1" in _err(lib), _err(lib)
