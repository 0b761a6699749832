"""Host-side checks of the C ABI: the library loads, exports every entry point include/dsa.h
declares, and rejects bad arguments before launching anything (no GPU needed)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")


@pytest.fixture(scope="module")
def dsa():
    lib_path = os.path.join(ROOT, "dsa_sparse_attention_indexer_amd", "libdsa.so")
    if not os.path.exists(lib_path):
        import __graft_entry__
        __graft_entry__._builder().build()
    import dsa_sparse_attention_indexer_amd as m
    return m


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z_]+)\s*\(", text)))


def test_header_declares_the_four_stages():
    fns = declared_functions()
    for f in ("dsa_indexer_scores", "dsa_topk", "dsa_sparse_mla_decode", "dsa_sparse_mla_prefill"):
        assert f in fns


def test_library_exports_every_declared_function(dsa):
    lib = ctypes.CDLL(dsa.LIB_PATH)
    for f in declared_functions():
        assert hasattr(lib, f), f"{f} declared in dsa.h but not exported"
    assert set(declared_functions()) == set(dsa.EXPORTED)
    assert dsa.lib().dsa_abi_version() == 3


def test_topk_rejects_bad_arguments_listing_every_reason(dsa):
    L = dsa.lib()
    st = L.dsa_topk(None, 6, None, 3, 0, None, None, None, 0, None)
    assert st == dsa.DSA_ERR_ARG
    msg = L.dsa_last_error().decode()
    for frag in ("multiple of 4", "k must be", "non-NULL", "top-k workspace"):
        assert frag in msg, msg


def test_indexer_topk_requires_its_workspace(dsa):
    L = dsa.lib()
    d = dsa.IndexerDesc(2, 64, 128, 64, 1, 100, dsa.DSA_BF16, dsa.DSA_FP8_E4M3FN)
    st = L.dsa_indexer_topk(ctypes.byref(d), None, None, None, None, None, None, None, None, None, None, 100, 2048,
                            None, None, None, 0, None, 0, None, None)
    msg = L.dsa_last_error().decode()
    assert st == dsa.DSA_ERR_ARG and "top-k workspace" in msg and "non-NULL" in msg, msg


def test_indexer_rejects_unsupported_shapes(dsa):
    L = dsa.lib()
    d = dsa.IndexerDesc(1, 64, 96, 32, 1, 100, dsa.DSA_BF16, dsa.DSA_BF16)
    st = L.dsa_indexer_scores(ctypes.byref(d), None, None, None, None, None, None, None, None, None, None, 50, None, 0,
                              None, None)
    assert st == dsa.DSA_ERR_ARG            # the NULLs and ld < max_ctx are argument errors
    msg = L.dsa_last_error().decode()
    for frag in ("head_dim", "num_heads", "rope_dim", "k_dtype", "ld_scores", "non-NULL", "workspace"):
        assert frag in msg, msg
    d = dsa.IndexerDesc(0, 64, 128, 64, 1, 100, dsa.DSA_BF16, dsa.DSA_FP8_E4M3FN)
    st = L.dsa_indexer_scores(ctypes.byref(d), None, None, None, None, None, None, None, None, None, None, 100, None, 0,
                              None, None)
    assert st == dsa.DSA_ERR_UNSUPPORTED and "num_heads" in L.dsa_last_error().decode()


def test_mla_rejects_bad_dtype_combinations(dsa):
    L = dsa.lib()
    d = dsa.MlaDesc(4, 64, 512, 64, 1, 1000, 2048, dsa.DSA_F32, dsa.DSA_FP8_E4M3FN, 64, 0.07, 0)
    st = L.dsa_sparse_mla_decode(ctypes.byref(d), None, None, None, None, None, None, None, None, None, 0, None, None)
    msg = L.dsa_last_error().decode()
    assert st == dsa.DSA_ERR_ARG and "BF16 queries" in msg and "non-NULL" in msg
    d = dsa.MlaDesc(0, 64, 256, 32, 1, 1000, 2048, dsa.DSA_BF16, dsa.DSA_FP8_E4M3FN, 32, 0.07, 0)
    st = L.dsa_sparse_mla_prefill(ctypes.byref(d), None, None, None, None, None, None, None, None, None, 0, None, None)
    msg = L.dsa_last_error().decode()
    assert st == dsa.DSA_ERR_UNSUPPORTED and "kv_lora" in msg and "rope_dim" in msg and "kv_scale_block" in msg


def test_workspace_queries(dsa):
    assert dsa.dsa_topk_workspace_size(16, 131072, 2048) == 16 * (4096 + 4 + 2 * 512 + 2 * 16384) * 4
    assert dsa.dsa_topk_workspace_size(0, 131072, 2048) == 0
    assert dsa.dsa_block_select_workspace_size(4, 524288, 128) == 4 * 4096 * 4
    d = dsa.MlaDesc(16, 64, 512, 64, 16, 131072, 2048, dsa.DSA_BF16, dsa.DSA_FP8_E4M3FN, 64, 0.07, 0)
    # automatic splits at batch 16 run each query as two 32-head halves: 32 x 8 splits of 256 keys,
    # partials for 16 queries x 8 splits x 64 heads
    assert dsa.dsa_sparse_mla_workspace_size(d) == 16 * 8 * 64 * 514 * 4
    d.num_splits = 16   # explicit splits: no head split
    assert dsa.dsa_sparse_mla_workspace_size(d) == 16 * 16 * 64 * 514 * 4
    d.num_q = 64
    d.num_splits = 0    # batch 64: 4 splits of 512 keys, no head split
    assert dsa.dsa_sparse_mla_workspace_size(d) == 64 * 4 * 64 * 514 * 4
    d.num_q = 16
    d.num_splits = 1
    assert dsa.dsa_sparse_mla_workspace_size(d) == 0


def test_zero_queries_is_a_no_op(dsa):
    L = dsa.lib()
    assert L.dsa_topk(None, 8, None, 0, 2048, None, None, None, 0, None) == dsa.DSA_OK
    assert L.dsa_last_error().decode() == ""


def test_cache_writers_validate_arguments(dsa):
    d = dsa.IndexKDesc(16, 6144, 6144, 64, 1e-6, 1000)
    assert dsa.dsa_index_k_insert_workspace_size(d) > 0
    # geometry: T = 16 is one token tile, so the hidden dim's 24 blocks of 256 are 24 slices
    assert dsa.dsa_index_k_insert_workspace_size(d) == 24 * 16 * 128 * 4
    assert dsa.dsa_index_k_insert_workspace_size(dsa.IndexKDesc(4096, 6144, 6144, 64, 1e-6, 1)) == 4 * 4096 * 128 * 4
    bad = dsa.IndexKDesc(16, 100, 96, 32, -1.0, 1000)
    st = dsa.lib().dsa_index_k_insert(ctypes.byref(bad), *([None] * 10), 0, None, None)
    msg = dsa.lib().dsa_last_error().decode()
    assert st in (dsa.DSA_ERR_ARG, dsa.DSA_ERR_UNSUPPORTED)
    for frag in ("hidden must be a multiple of 32", "ld_x must be", "rope_dim must be 0 or 64", "eps must be",
                 "must be non-NULL", "workspace"):
        assert frag in msg, (frag, msg)
    st = dsa.lib().dsa_latent_insert(4, 16, None, 100, None, None, None, 10, None, None, None)
    msg = dsa.lib().dsa_last_error().decode()
    assert st == dsa.DSA_ERR_ARG and "ld_kv must be >= 576" in msg and "rope_dim must be 0 or 64" in msg
    zero = dsa.IndexKDesc(0, 6144, 6144, 64, 1e-6, 0)
    assert dsa.lib().dsa_index_k_insert(ctypes.byref(zero), *([None] * 10), 0, None, None) == dsa.DSA_OK
    assert dsa.lib().dsa_latent_insert(0, 64, None, 576, None, None, None, 0, None, None, None) == dsa.DSA_OK


def test_noalloc_mla_rejects_oversized_partials_before_touching_the_gpu(dsa):
    L = dsa.lib()
    assert L.dsa_sparse_mla_noalloc_max_bytes() == 64 << 20
    d = dsa.MlaDesc(16, 64, 512, 64, 16, 4096, 2048, dsa.DSA_BF16, dsa.DSA_FP8_E4M3FN, 64, 0.07, 64)
    st = L.dsa_sparse_mla_decode_noalloc(ctypes.byref(d), None, None, None, None, None, None, None, None, None, None)
    msg = L.dsa_last_error().decode()
    assert st == dsa.DSA_ERR_UNSUPPORTED and "67108864 bytes" in msg, msg


def test_mla_rejects_a_zero_topk_without_dividing_by_zero(dsa):
    L = dsa.lib()
    d = dsa.MlaDesc(2, 64, 512, 64, 1, 100, 0, dsa.DSA_BF16, dsa.DSA_FP8_E4M3FN, 64, 0.07, 0)
    st = L.dsa_sparse_mla_decode(ctypes.byref(d), None, None, None, None, None, None, None, None, None, 0, None, None)
    assert st == dsa.DSA_ERR_ARG and "topk" in L.dsa_last_error().decode()
    assert L.dsa_sparse_mla_workspace_size(ctypes.byref(d)) == 0


def test_timing_hook_rejects_bad_arguments_and_disarms_cleanly(dsa):
    L = dsa.lib()
    assert L.dsa_timing_begin(None, 4) == dsa.DSA_ERR_ARG
    arr = (ctypes.c_void_p * 2)()
    assert L.dsa_timing_begin(arr, 0) == dsa.DSA_ERR_ARG
    assert L.dsa_timing_begin(arr, 65537) == dsa.DSA_ERR_ARG
    assert L.dsa_timing_begin(arr, 1) == dsa.DSA_OK
    assert L.dsa_timing_end() == 0          # nothing launched while armed
    assert L.dsa_timing_kernel_name(0) is None
    assert L.dsa_timing_end() == 0          # ending twice is harmless


def test_block_select_without_scores_only_where_the_kernel_writes_block_maxima(dsa):
    """No score buffer is accepted only where the fp8 decode score kernel writes the block maxima
    (128-token blocks); elsewhere (fp32 keys, 100-token blocks, many queries per sequence) the
    call fails on the host, before any launch."""
    L = dsa.lib()
    fake = ctypes.c_void_p(1 << 20)   # aligned, never dereferenced: validation fails first
    cases = [(dsa.DSA_F32, 128, 4, 4), (dsa.DSA_FP8_E4M3FN, 100, 4, 4), (dsa.DSA_FP8_E4M3FN, 128, 64, 4)]
    for k_dtype, block, T, B in cases:
        d = dsa.IndexerDesc(T, 4, 128, 64, B, 8192, dsa.DSA_BF16, k_dtype)
        st = L.dsa_indexer_block_select(ctypes.byref(d), fake, fake, fake, fake, None, None, fake, fake, fake,
                                        None, 8192, block, 16, 2048, fake, None, fake, 1 << 30, fake, 1 << 30,
                                        None, None)
        msg = L.dsa_last_error().decode()
        assert st == dsa.DSA_ERR_ARG and "scores may be NULL only" in msg, (k_dtype, block, T, msg)
