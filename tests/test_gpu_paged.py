"""GPU parity of the paged cache layout ("Day 0 support for Mistral Large 4 on vLLM", "ROCm
implementation details", "DSA indexer on AITER": cache blocks, keys in 16x16 tiles within a block,
one layout rule for the writer and every reader).

Block tables are shuffled (blocks handed out in random order, out-of-range entries past each
sequence's last block, random bytes in every unused row).  The writers' bytes are read back by
the test's own restatement of the rule; the readers see pools built by that restatement and must
return exactly what they return on the same data in contiguous caches, and match the oracle.
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import dsa_oracle as O
from tests.paging_util import key_rows_from_pool, pool_from_contiguous, shuffled_table, slots_of
from tests.parity_util import check_attention, check_selection, mla_lse_bound

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    assert torch.cuda.is_available(), "GPU tests need the MI355X"
    import dsa_sparse_attention_indexer_amd as m
    return m


def _paging(dsa, table, page, nblocks, max_ctx):
    return dsa.Paging(torch.from_numpy(table).cuda(), page, nblocks, max_ctx)


def test_paged_slots_follow_the_rule(dsa):
    lens = [700, 64, 1, 2049]
    table, nb = shuffled_table(lens, 64, 5, seed=71)
    pg = _paging(dsa, table, 64, nb, max(lens))
    rng = np.random.default_rng(72)
    seq = rng.integers(0, len(lens), size=500).astype(np.int32)
    pos = np.array([rng.integers(-2, lens[s]) for s in seq], dtype=np.int32)
    got = dsa.dsa_paged_slots(pg, torch.from_numpy(seq).cuda(), torch.from_numpy(pos).cuda()).cpu().numpy()
    want = np.array([-1 if p < 0 else slots_of(table, 64, s, [p])[0] for s, p in zip(seq, pos)])
    assert np.array_equal(got, want)


@pytest.mark.parametrize("page", [32, 64, 256])
def test_paged_key_writer_places_bytes_in_tiles(dsa, page):
    """The key writer into a paged pool writes, at each token's tiles, exactly the bytes it writes
    into a contiguous cache; every other byte of the pool is untouched."""
    lens = [300, 129, 70]
    table, nb = shuffled_table(lens, page, 2, seed=73 + page)
    pos = [p for n in lens for p in range(n)]
    seqs = [b for b, n in enumerate(lens) for _ in range(n)]
    bt = workloads.make_insert_batch(name=f"paged{page}", seed=74, positions=pos, seqs=seqs, num_seqs=len(lens),
                                     max_ctx=max(lens), hidden=256, rope=True)
    dev = "cuda"
    T = bt.num_tokens
    contig = torch.zeros((T, 128), dtype=torch.uint8, device=dev)
    cscale = torch.zeros(T, dtype=torch.float32, device=dev)
    dense = torch.arange(T, dtype=torch.int64, device=dev)
    args = (bt.x.to(dev), bt.wk.to(dev), bt.ln_w.to(dev), bt.ln_b.to(dev), bt.pos.to(dev))
    dsa.dsa_index_k_insert(*args, dense, contig, cscale, inv_freq=bt.inv_freq.to(dev), eps=bt.eps)
    pg = _paging(dsa, table, page, nb, max(lens))
    rows = nb * page
    pool = torch.full((rows, 128), 0x5A, dtype=torch.uint8, device=dev)
    pscale = torch.full((rows,), -7.0, dtype=torch.float32, device=dev)
    slot = dsa.dsa_paged_slots(pg, torch.tensor(seqs, dtype=torch.int32, device=dev), bt.pos.to(dev))
    dsa.dsa_index_k_insert(*args, slot, pool, pscale, inv_freq=bt.inv_freq.to(dev), eps=bt.eps, paging=pg)
    torch.cuda.synchronize()
    sl = slot.cpu().numpy()
    assert np.array_equal(sl, np.concatenate([slots_of(table, page, b, range(n)) for b, n in enumerate(lens)]))
    got = key_rows_from_pool(pool.cpu(), sl, page)
    assert np.array_equal(got, contig.cpu().numpy())
    assert np.array_equal(pscale.cpu().numpy()[sl], cscale.cpu().numpy())
    untouched = np.ones(rows, dtype=bool)
    untouched[sl] = False
    # a slot's bytes are spread over its tiles: check the untouched slots' bytes through the rule
    rest = key_rows_from_pool(pool.cpu(), np.nonzero(untouched)[0], page)
    assert np.all(rest == 0x5A) and np.all(pscale.cpu().numpy()[untouched] == -7.0)


def _paged_inputs(dsa, g, page, spare, seed):
    """Paged pools of the (GPU) workload g's caches, on a shuffled table."""
    lens = [int(x) for x in g.seq_len.tolist()]
    table, nb = shuffled_table(lens, page, spare, seed)
    kp, ks, vp, vs = pool_from_contiguous(g.index_k, g.index_k_scale, g.kv, g.kv_scale, lens, table, page, nb,
                                          seed + 1)
    return _paging(dsa, table, page, nb, g.max_ctx), kp, ks, vp, vs


def _mla_ref(wl, t, idx, ln):
    idx = np.asarray(idx)
    sel = idx[:ln][idx[:ln] >= 0]
    rows = O.cache_rows(wl, int(wl.q_seq[t]), sel)
    ro, rl = O.mla_attend(wl.mla_q[t], rows, wl.rope_dim, wl.softmax_scale)
    return ro, rl, mla_lse_bound(O.to_f64(wl.mla_q[t]), rows, wl.rope_dim, wl.softmax_scale, wl.fp8)


PAGED_CASES = [
    # decode (4096-key score chunks, emitted candidates), ragged lengths ending inside blocks
    ("decode_4096_chunks", lambda: workloads.make_workload(name="pd", seed=81, seq_lens=[10000, 9000, 8191, 4100] * 50,
                                                           max_ctx=10000, device="cuda"), 64, False),
    # decode with 1024-key chunks, 32-token blocks
    ("decode_1024_chunks_page32", lambda: workloads.make_workload(name="pd2", seed=82, seq_lens=[5000, 3001],
                                                                  max_ctx=5000), 32, False),
    # verify blocks (grouped kernel, shared key stream), NoPE
    ("verify_b3x4_nope", lambda: workloads.verify_blocks(seed=83, tokens=4, seq_lens=[9000, 4097, 12000],
                                                         rope=False), 128, False),
    # interleaved sequences: grouped kernel, private streams
    ("grouped_private", lambda: workloads.make_workload(name="pi", seed=84, seq_lens=[6000, 5000], max_ctx=6000,
                                                        q_positions=[5999, 4999, 5998, 4998, 5000, 100],
                                                        q_seqs=[0, 1, 0, 1, 0, 1]), 256, False),
    # chunked prefill (one MLA workgroup per query)
    ("prefill_300", lambda: workloads.make_workload(name="pp", seed=85, seq_lens=[8300], max_ctx=8300,
                                                    q_positions=list(range(8000, 8300))), 64, True),
    # query tiles (16+ queries per sequence, 8192-key ranges): two sequences whose runs of queries
    # do not align with the 8-query groups, ranges past the shorter sequence, 64-token blocks
    ("prefill_query_tiles", lambda: _qtile_workload(), 64, True),
]


def _qtile_workload():
    rng = np.random.default_rng(87)
    lens = [70001, 20000]
    seqs = [0] * 100 + [1] * 50 + [0] * 140 + [1] * 180
    pos = [int(rng.integers(0, lens[b])) for b in seqs]
    pos[0], pos[1] = lens[0] - 1, 0
    return workloads.make_workload(name="pq", seed=87, seq_lens=lens, max_ctx=lens[0], q_positions=pos, q_seqs=seqs)


@pytest.mark.parametrize("name,make,page,prefill", PAGED_CASES, ids=[c[0] for c in PAGED_CASES])
def test_paged_readers_match_contiguous(dsa, name, make, page, prefill):
    g = make().to("cuda")
    pg, kp, ks, vp, vs = _paged_inputs(dsa, g, page, 3, seed=90)
    from dsa_sparse_attention_indexer_amd import pipeline as P
    ref = P.alloc_buffers(g, prefill=prefill)
    P.layer_step(g, ref, prefill=prefill)
    pb = P.alloc_buffers(g, prefill=prefill)
    dsa.dsa_indexer_topk(g.index_q, g.index_w, g.q_seq, g.q_pos, kp, pb.scores, g.topk, pb.idx, pb.length,
                         k_scale=ks, ssmax_s=g.ssmax_s, ssmax_b=g.ssmax_b, inv_freq=g.inv_freq, ws=pb.ws_index,
                         topk_ws=pb.ws_topk, paging=pg)
    mla = dsa.dsa_sparse_mla_prefill if prefill else dsa.dsa_sparse_mla_decode
    kw = {} if prefill else {"ws": pb.ws_mla}
    mla(g.mla_q, vp, vs, g.q_seq, pb.idx, pb.length, pb.out, pb.lse, softmax_scale=g.softmax_scale, paging=pg, **kw)
    torch.cuda.synchronize()
    sr, sp = ref.scores.cpu().numpy(), pb.scores.cpu().numpy()
    for t in range(g.num_q):
        n = int(g.q_pos[t]) + 1
        assert np.array_equal(sr[t, :n], sp[t, :n]), f"{name} q{t}: paged scores differ"
    assert torch.equal(ref.idx, pb.idx) and torch.equal(ref.length, pb.length), f"{name}: paged selection differs"
    assert torch.equal(ref.out, pb.out) and torch.equal(ref.lse, pb.lse), f"{name}: paged attention differs"
    idx, ln = pb.idx.cpu().numpy(), pb.length.cpu().numpy()
    out, lse = pb.out.cpu().numpy(), pb.lse.cpu().numpy()
    for t in sorted({0, g.num_q - 1}):
        one = workloads.slice_query(g, t)
        check_selection(idx[t], ln[t], O.index_scores(one, 0), g.topk, f"{name} q{t}", rms_admitted_ok=False)
        ro, rl, bound = _mla_ref(one, 0, idx[t], int(ln[t]))
        check_attention(out[t], lse[t], ro, rl, True, f"{name} q{t}", lse_abs=bound)


def test_paged_noalloc_decode_matches_workspace_call(dsa):
    g = workloads.make_workload(name="pn", seed=86, seq_lens=[7000, 2500], max_ctx=7000).to("cuda")
    pg, kp, ks, vp, vs = _paged_inputs(dsa, g, 64, 2, seed=91)
    from dsa_sparse_attention_indexer_amd import pipeline as P
    b1, b2 = P.alloc_buffers(g), P.alloc_buffers(g)
    dsa.dsa_indexer_topk(g.index_q, g.index_w, g.q_seq, g.q_pos, kp, b1.scores, g.topk, b1.idx, b1.length,
                         k_scale=ks, ssmax_s=g.ssmax_s, ssmax_b=g.ssmax_b, inv_freq=g.inv_freq, paging=pg)
    dsa.dsa_sparse_mla_decode(g.mla_q, vp, vs, g.q_seq, b1.idx, b1.length, b1.out, b1.lse,
                              softmax_scale=g.softmax_scale, ws=b1.ws_mla, paging=pg)
    dsa.dsa_sparse_mla_decode_noalloc(g.mla_q, vp, vs, g.q_seq, b1.idx, b1.length, b2.out, b2.lse,
                                      softmax_scale=g.softmax_scale, paging=pg)
    torch.cuda.synchronize()
    assert torch.equal(b1.out, b2.out) and torch.equal(b1.lse, b2.lse)
