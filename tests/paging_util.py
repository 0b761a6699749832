"""Paged cache layouts built and read on the CPU, for the paging tests.

The rule ("Day 0 support for Mistral Large 4 on vLLM", "ROCm implementation details", "DSA
indexer on AITER": keys in cache blocks, stored in 16x16 tiles within a block): token p of
sequence b lives in block table[b][p // page], row i = p % page; byte d of its FP8 index key is
byte 256 * (8 * (i // 16) + d // 16) + 16 * (i % 16) + d % 16 of the block's page * 128 bytes,
and every other per-token array (key scale, latent row, latent scales) keeps one whole row per
pool slot block * page + i.  These helpers restate that rule with numpy index arithmetic, apart
from the library, so that a layout mistake shared by the library's writer and readers still
shows up.
"""
import numpy as np
import torch


def shuffled_table(seq_lens, page, spare_blocks, seed, bad_tail=True):
    """A block table that hands out the pool's blocks in a random order: [B][bps] int32 and the
    pool's block count.  Table entries past a sequence's last block hold out-of-range values
    (the kernels must never use them for visible positions)."""
    rng = np.random.default_rng(seed)
    bps = max((n + page - 1) // page for n in seq_lens)
    need = sum((n + page - 1) // page for n in seq_lens)
    nblocks = need + spare_blocks
    perm = rng.permutation(nblocks)
    table = np.full((len(seq_lens), bps), -1, dtype=np.int32)
    k = 0
    for b, n in enumerate(seq_lens):
        used = (n + page - 1) // page
        table[b, :used] = perm[k:k + used]
        k += used
        if bad_tail:
            table[b, used:] = rng.choice([-5, nblocks, 1 << 30], size=bps - used)
    return table, nblocks


def slots_of(table, page, b, positions):
    positions = np.asarray(positions, dtype=np.int64)
    return table[b, positions // page].astype(np.int64) * page + positions % page


def key_byte_offsets(slot, page):
    """Byte offset in the pool of each of the 128 key bytes of each slot: [n][128]."""
    slot = np.asarray(slot, dtype=np.int64)
    blk, i = slot // page, slot % page
    d = np.arange(128, dtype=np.int64)
    return (blk * page * 128)[:, None] + 256 * (8 * (i // 16)[:, None] + d[None, :] // 16) \
        + 16 * (i % 16)[:, None] + d[None, :] % 16


def pool_from_contiguous(keys, kscale, kv, kvscale, seq_lens, table, page, nblocks, seed):
    """Paged pools holding the first seq_lens[b] tokens of contiguous caches [B][max_ctx][...] (on
    their own device), every other byte random (FP8 NaN codes included).  Returns (k_pool
    [rows][128] uint8, k_scale [rows] f32, kv_pool [rows][576] uint8, kv_scale [rows][9] f32)."""
    dev = keys.device
    g = torch.Generator(device=dev)
    g.manual_seed(int(seed))
    rows = nblocks * page
    kp = torch.randint(0, 256, (rows * 128,), generator=g, dtype=torch.uint8, device=dev)
    ks = torch.randn(rows, generator=g, dtype=torch.float32, device=dev)
    vp = torch.randint(0, 256, (rows, 576), generator=g, dtype=torch.uint8, device=dev)
    vs = torch.randn((rows, 9), generator=g, dtype=torch.float32, device=dev)
    keys = keys.view(torch.uint8)
    kv = kv.view(torch.uint8)
    for b, n in enumerate(seq_lens):
        sl = slots_of(table, page, b, np.arange(n))
        off = torch.from_numpy(key_byte_offsets(sl, page)).to(dev)
        kp[off.reshape(-1)] = keys[b, :n].reshape(-1)
        slt = torch.from_numpy(sl).to(dev)
        ks[slt] = kscale[b, :n]
        vp[slt] = kv[b, :n]
        vs[slt] = kvscale[b, :n]
    return kp.reshape(rows, 128), ks, vp, vs


def key_rows_from_pool(pool, slots, page):
    """The 128-byte keys of the given slots, read back out of a tiled pool ([rows][128] uint8)."""
    flat = pool.reshape(-1).cpu().numpy()
    return flat[key_byte_offsets(slots, page)]
