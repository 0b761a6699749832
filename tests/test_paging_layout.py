"""The paged layout rule as the tests restate it (tests/paging_util.py), pinned on the CPU to the
page's description: 16-token x 16-byte tiles within a cache block ("Day 0 support for Mistral
Large 4 on vLLM", "ROCm implementation details", "DSA indexer on AITER"), and the C ABI's host
checks of a paging argument."""
import ctypes
import os

import numpy as np
import pytest

from tests.paging_util import key_byte_offsets, shuffled_table, slots_of

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("page", [32, 64, 256])
def test_block_bytes_are_a_permutation_and_32_row_groups_are_4k_ranges(page):
    off = key_byte_offsets(np.arange(page), page)             # block 0, every row
    assert sorted(off.reshape(-1).tolist()) == list(range(page * 128))
    for g in range(page // 32):
        grp = off[32 * g:32 * g + 32].reshape(-1)
        assert grp.min() == 4096 * g and grp.max() == 4096 * g + 4095
    blk3 = key_byte_offsets(3 * page + np.arange(page), page)
    assert np.array_equal(blk3, off + 3 * page * 128)


def test_tile_positions_by_hand():
    off = key_byte_offsets(np.arange(64), 64)
    assert off[0, 0] == 0 and off[0, 15] == 15            # row 0: the first 16 bytes of tile (0, 0)
    assert off[1, 0] == 16                                # row 1 follows row 0 inside the tile
    assert off[15, 15] == 255                             # the tile is 16 rows x 16 bytes
    assert off[0, 16] == 256                              # the next 16 bytes: the next tile
    assert off[0, 127] == 7 * 256 + 15                    # 8 tiles side by side per 16-row group
    assert off[16, 0] == 2048                             # rows 16..31: the next group of tiles
    assert off[17, 127] == 256 * 15 + 16 + 15


def test_shuffled_table_uses_every_block_once():
    table, nb = shuffled_table([300, 64, 1], 64, 3, seed=5)
    used = [table[0, :5], table[1, :1], table[2, :1]]
    flat = np.concatenate(used)
    assert len(set(flat.tolist())) == flat.size and flat.max() < nb and flat.min() >= 0
    assert slots_of(table, 64, 0, [0, 63, 64, 299]).tolist() == [table[0, 0] * 64, table[0, 0] * 64 + 63,
                                                                 table[0, 1] * 64, table[0, 4] * 64 + 43]


@pytest.fixture(scope="module")
def dsa():
    lib_path = os.path.join(ROOT, "dsa_sparse_attention_indexer_amd", "libdsa.so")
    if not os.path.exists(lib_path):
        pytest.skip("libdsa.so not built")
    import dsa_sparse_attention_indexer_amd as m
    return m


def _pg(dsa, page, bps, nblocks, nseq, table=1):
    return dsa.PagingDesc(table, page, bps, nblocks, nseq)


def test_paging_arguments_are_checked_before_launch(dsa):
    L = dsa.lib()
    d = dsa.IndexerDesc(0, 32, 128, 64, 2, 1000, 1, 2)   # no queries (nothing else to check), fp8 keys
    args = [ctypes.byref(d)] + [None] * 10 + [1000, None, 0, None]

    def call(pg):
        return L.dsa_indexer_scores(*args, ctypes.byref(pg))
    assert call(_pg(dsa, 48, 40, 100, 2)) == dsa.DSA_ERR_UNSUPPORTED      # not a multiple of 32
    assert call(_pg(dsa, 64, 15, 100, 2)) == dsa.DSA_ERR_ARG              # 15 * 64 < max_ctx
    assert call(_pg(dsa, 64, 16, 0, 2)) == dsa.DSA_ERR_ARG                # empty pool
    assert call(_pg(dsa, 64, 16, 100, 3)) == dsa.DSA_ERR_ARG              # table rows != num_seqs
    assert call(_pg(dsa, 64, 16, 100, 2, table=None)) == dsa.DSA_ERR_ARG  # no table
    assert call(_pg(dsa, 64, 16, 100, 2)) == dsa.DSA_OK
    f32 = dsa.IndexerDesc(0, 32, 128, 64, 2, 1000, 0, 0)                 # f32 keys are never paged
    assert L.dsa_indexer_scores(ctypes.byref(f32), *args[1:], ctypes.byref(_pg(dsa, 64, 16, 100, 2))) \
        == dsa.DSA_ERR_UNSUPPORTED


def test_paged_latent_pool_must_fit_32_bit_offsets(dsa):
    L = dsa.lib()
    d = dsa.MlaDesc(0, 64, 512, 64, 2, 4096, 2048, 1, 2, 64, 0.07, 0)
    big = _pg(dsa, 64, 64, (1 << 32) // (576 * 64) + 1, 2)
    st = L.dsa_sparse_mla_decode(ctypes.byref(d), *([None] * 9), 0, None, ctypes.byref(big))
    assert st == dsa.DSA_ERR_UNSUPPORTED and "pool" in L.dsa_last_error().decode()


def test_paged_slots_rejects_a_missing_layout(dsa):
    L = dsa.lib()
    assert L.dsa_paged_slots(None, 4, None, None, None, None) == dsa.DSA_ERR_ARG
    assert L.dsa_paged_slots(ctypes.byref(_pg(dsa, 64, 4, 8, 1)), 0, None, None, None, None) == dsa.DSA_OK
