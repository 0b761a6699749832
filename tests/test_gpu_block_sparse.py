"""GPU parity of the block-sparse selection (the MiniMax Sparse Attention steps of "vLLM adds NVFP4
serving for MiniMax M3.1 Flash at 76 concurrent sequences": block maxima of the index scores, the
most recent block kept, the best of the rest by (score desc, block asc)).

Every selection is the oracle's block_select_row of the GPU's own fp32 scores, bit for bit; the
fused call (block maxima written by the score kernel) is also checked against the separate calls.
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import dsa_oracle as O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    assert torch.cuda.is_available(), "GPU tests need the MI355X"
    import dsa_sparse_attention_indexer_amd as m
    return m


def _pick(dsa, sc, lens, block=128, nblocks=16):
    T = len(lens)
    qp = torch.as_tensor([n - 1 for n in lens], dtype=torch.int32).cuda()
    idx = torch.empty(T, max(2048, nblocks * block), dtype=torch.int32, device="cuda")
    ln = torch.empty(T, dtype=torch.int32, device="cuda")
    dsa.dsa_block_select(torch.from_numpy(sc).cuda(), qp, idx, ln, block=block, nblocks=nblocks)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), ln.cpu().numpy()


def test_block_pick_ties_at_the_threshold(dsa):
    """A few block maxima equal to the threshold (the lower blocks are kept), in several rows:
    the radix path ranks them in one wave; a row with 80 tied maxima takes the argmax rounds."""
    rng = np.random.default_rng(31)
    n = 128 * 300
    lens = [n, n, n, n - 50]
    sc = rng.standard_normal((4, n)).astype(np.float32) - 10.0
    for t, (ntie, take_rank) in enumerate([(5, 12), (3, 14), (80, 5), (2, 0)]):
        blocks = rng.permutation(299)[: 14 + ntie]
        top = blocks[:take_rank]                    # strictly above the tie
        tie = blocks[take_rank:take_rank + ntie]
        for r, j in enumerate(top):
            sc[t, 128 * j + 7] = 100.0 - r
        for j in tie:
            sc[t, 128 * j + 100] = 50.0
    gi, gl = _pick(dsa, sc, lens)
    for t, n_ in enumerate(lens):
        ref, rl = O.block_select_row(sc[t, :n_].astype(np.float64), n_ - 1)
        assert gl[t] == rl and np.array_equal(gi[t], ref), f"row {t}"


FUSED_CASES = [
    # 4096-key score chunks (many queries), 128-token blocks; ragged, partial recent blocks
    ("chunks4096_b128", dict(seq_lens=[20000, 17001, 9000, 4097] * 32, max_ctx=20000, num_heads=4), 128, 16),
    # 1024-key chunks, 64-token blocks, 32 kept
    ("chunks1024_b64", dict(seq_lens=[30000, 12345], max_ctx=30000, num_heads=4), 64, 32),
    # 100-token blocks: not whole tiles, so the separate block-max pass runs
    ("unfused_b100", dict(seq_lens=[9000, 4000], max_ctx=9000, num_heads=4), 100, 16),
    # fewer blocks than kept: every block
    ("short_rows", dict(seq_lens=[1500, 700], max_ctx=1500, num_heads=32), 128, 16),
]


@pytest.mark.parametrize("name,kw,block,nblocks", FUSED_CASES, ids=[c[0] for c in FUSED_CASES])
def test_fused_block_select_matches_oracle(dsa, name, kw, block, nblocks):
    g = workloads.make_workload(name=name, seed=1601, device="cuda", **kw)
    T = g.num_q
    ld = (g.max_ctx + 3) // 4 * 4
    scores = torch.empty(T, ld, dtype=torch.float32, device="cuda")
    k = max(2048, block * nblocks)
    idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
    ln = torch.empty(T, dtype=torch.int32, device="cuda")
    dsa.dsa_indexer_block_select(g.index_q, g.index_w, g.q_seq, g.q_pos, g.index_k, scores, idx, ln, block=block,
                                 nblocks=nblocks, k_scale=g.index_k_scale, ssmax_s=g.ssmax_s, ssmax_b=g.ssmax_b,
                                 inv_freq=g.inv_freq)
    sep_idx = torch.empty_like(idx)
    sep_ln = torch.empty_like(ln)
    dsa.dsa_block_select(scores, g.q_pos, sep_idx, sep_ln, block=block, nblocks=nblocks)
    torch.cuda.synchronize()
    assert torch.equal(idx, sep_idx) and torch.equal(ln, sep_ln)
    sc, gi, gl = scores.cpu().numpy(), idx.cpu().numpy(), ln.cpu().numpy()
    for t in range(T):
        n = int(g.q_pos[t]) + 1
        ref, rl = O.block_select_row(sc[t, :n].astype(np.float64), n - 1, block=block, nblocks=nblocks, topk=k)
        assert gl[t] == rl and np.array_equal(gi[t], ref), f"{name} q{t}"
    one = workloads.slice_query(g, 0)
    s = O.index_scores(one, 0)
    tol = 2e-6 * np.sqrt(np.mean(s * s)) + 2e-6 * np.abs(s)
    assert np.all(np.abs(sc[0, :s.shape[0]] - s) <= tol)
    # without a score buffer: the same selection where the score kernel writes the block maxima,
    # a clear error where the separate block-max pass would need the scores
    nidx = torch.full_like(idx, -7)
    nln = torch.full_like(ln, -7)
    args = (g.index_q, g.index_w, g.q_seq, g.q_pos, g.index_k, None, nidx, nln)
    kw = dict(block=block, nblocks=nblocks, k_scale=g.index_k_scale, ssmax_s=g.ssmax_s, ssmax_b=g.ssmax_b,
              inv_freq=g.inv_freq, ld=ld)
    if block % 32 == 0:
        dsa.dsa_indexer_block_select(*args, **kw)
        torch.cuda.synchronize()
        assert torch.equal(nidx, idx) and torch.equal(nln, ln), f"{name}: selection without scores differs"
    else:
        with pytest.raises(dsa.DsaError, match="scores may be NULL only"):
            dsa.dsa_indexer_block_select(*args, **kw)
