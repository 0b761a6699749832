"""Which kernels each call shape launches: the library's timing hook names every dispatch, so the
routing rules (decode stream vs. grouped vs. query-tile score kernels, the per-row vs. segmented
top-k, the MLA head split) are checked on small inputs shaped like the workloads they serve.  The
numerical results of every path are checked against the oracle elsewhere; this file guards the
routing, so that a rule change cannot silently send a benchmarked shape down another path."""
import numpy as np
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    assert torch.cuda.is_available(), "GPU tests need the MI355X"
    import dsa_sparse_attention_indexer_amd as m
    return m


def _launched(dsa, fn):
    timer = dsa.KernelTimer(64)
    with timer:
        fn()
        torch.cuda.synchronize()
    return [name for name, _ in timer.results()]


def _has(names, part):
    return any(part in n for n in names)


def _step(dsa, wl, prefill=False):
    from dsa_sparse_attention_indexer_amd import pipeline as P
    buf = P.alloc_buffers(wl, prefill=prefill)
    return _launched(dsa, lambda: P.layer_step(wl, buf, prefill=prefill))


def test_decode_batch16_uses_the_fused_stream_and_head_split(dsa):
    wl = workloads.make_workload(name="d16", seed=1, seq_lens=[9000] * 16, max_ctx=9000, device="cuda")
    names = _step(dsa, wl)
    assert _has(names, "k_index_scores_fp8") and not _has(names, "grouped") and not _has(names, "qtile"), names
    assert _has(names, "k_topk_resolve") and not _has(names, "k_topk_hist"), names
    assert _has(names, "k_mla_fp8_wsILi64ELi1E") and _has(names, "k_mla_combine"), names   # two 32-head halves


def test_decode_batch64_keeps_whole_head_tiles(dsa):
    wl = workloads.make_workload(name="d64", seed=2, seq_lens=[3000] * 64, max_ctx=3000, device="cuda")
    names = _step(dsa, wl)
    assert _has(names, "k_mla_fp8_wsILi64ELi2E"), names


def test_verify_blocks_use_the_grouped_kernel(dsa):
    wl = workloads.verify_blocks(device="cuda", batch=16, tokens=4, ctx=9000)
    names = _step(dsa, wl)
    assert _has(names, "k_index_scores_fp8_grouped") and not _has(names, "qtile"), names
    assert _has(names, "k_topk_emit") and _has(names, "k_topk_resolve") and not _has(names, "k_topk_hist"), names


@pytest.mark.parametrize("paged", [False, True])
def test_long_prefill_chunk_uses_query_tiles_and_the_per_row_top_k(dsa, paged):
    n = 65536
    wl = workloads.make_workload(name="pf", seed=3, seq_lens=[n], max_ctx=n, device="cuda",
                                 q_positions=list(range(n - 512, n)))
    if not paged:
        names = _step(dsa, wl, prefill=True)
        assert _has(names, "k_index_scores_fp8_qtileILb0E") and _has(names, "k_topk_direct"), names
        return
    from tests.paging_util import pool_from_contiguous, shuffled_table
    from dsa_sparse_attention_indexer_amd import pipeline as P
    table, nb = shuffled_table([n], 64, 2, seed=5)
    kp, ks, _, _ = pool_from_contiguous(wl.index_k, wl.index_k_scale, wl.kv, wl.kv_scale, [n], table, 64, nb, 6)
    pg = dsa.Paging(torch.from_numpy(table).cuda(), 64, nb, n)
    buf = P.alloc_buffers(wl, prefill=True)
    names = _launched(dsa, lambda: dsa.dsa_indexer_topk(
        wl.index_q, wl.index_w, wl.q_seq, wl.q_pos, kp, buf.scores, wl.topk, buf.idx, buf.length, k_scale=ks,
        ssmax_s=wl.ssmax_s, ssmax_b=wl.ssmax_b, inv_freq=wl.inv_freq, ws=buf.ws_index, topk_ws=buf.ws_topk,
        paging=pg))
    assert _has(names, "k_index_scores_fp8_qtileILb1E") and _has(names, "k_topk_direct"), names


def test_short_prefill_chunk_keeps_the_grouped_kernel(dsa):
    wl = workloads.make_workload(name="ps", seed=4, seq_lens=[6000], max_ctx=6000, device="cuda",
                                 q_positions=list(range(5700, 6000)))
    names = _step(dsa, wl, prefill=True)
    assert _has(names, "k_index_scores_fp8_grouped") and not _has(names, "qtile"), names


def test_separate_top_k_routing_by_row_count(dsa):
    rng = np.random.default_rng(9)
    for rows, direct in ((16, False), (160, True)):
        sc = torch.as_tensor(rng.standard_normal((rows, 20000)).astype(np.float32)).cuda()
        qp = torch.full((rows,), 19999, dtype=torch.int32, device="cuda")
        idx = torch.empty(rows, 2048, dtype=torch.int32, device="cuda")
        ln = torch.empty(rows, dtype=torch.int32, device="cuda")
        names = _launched(dsa, lambda: dsa.dsa_topk(sc, qp, 2048, idx, ln))
        assert _has(names, "k_topk_direct") == direct and _has(names, "k_topk_emit") == (not direct), names
        assert not _has(names, "k_topk_hist"), names
