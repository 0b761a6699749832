"""GPU parity of the grouped path: several queries per sequence (multi-token verify blocks and
chunked prefill), where four consecutive queries of one sequence share one key stream through LDS,
and the top-k selection runs over the scores written.

Every selection is the oracle's top-k of the GPU's own scores, bit for bit, and lies in the tie
band of the oracle's float64 scores; every attention output matches the oracle's attention over
that selection.  Verify-block tokens attend causally: token j of a block sees the keys up to its
own position only.
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import dsa_oracle as O
from tests.parity_util import check_attention, check_selection, mla_lse_bound

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    assert torch.cuda.is_available(), "GPU tests need the MI355X"
    import dsa_sparse_attention_indexer_amd as m
    return m


def _pipe():
    from dsa_sparse_attention_indexer_amd import pipeline
    return pipeline


def _grouped(dsa, wl):
    """The score call takes the grouped kernel exactly when it needs a query-prep workspace."""
    return dsa.dsa_indexer_workspace_size(dsa.indexer_desc(wl.index_q, wl.index_k, wl.inv_freq)) > 0


def _prefill(seed, n, q0, q1):
    return workloads.make_workload(name=f"prefill_{q0}_{q1}", seed=seed, seq_lens=[n], max_ctx=n,
                                   q_positions=list(range(q0, q1)))


def _interleaved(seed):
    # two sequences, queries alternating between them: every group of four consecutive queries
    # reads two sequences, so each wave streams its own keys
    pos = [8999 - i for i in range(6)] + [6999 - i for i in range(6)]
    seqs = [0] * 6 + [1] * 6
    order = [0, 6, 1, 7, 2, 8, 3, 9, 4, 10, 5, 11]
    return workloads.make_workload(name="interleaved", seed=seed, seq_lens=[9000, 7000], max_ctx=9000,
                                   q_positions=[pos[i] for i in order], q_seqs=[seqs[i] for i in order])


GROUPED_CASES = [
    # four tokens per sequence: every group of four queries is one sequence's verify block
    ("verify_b4x4", lambda: workloads.verify_blocks(seed=1515, tokens=4, seq_lens=[20000, 9000, 30000, 4500])),
    # three tokens per sequence: groups of four straddle two sequences (private streams)
    ("verify_b3x3", lambda: workloads.verify_blocks(seed=1516, tokens=3, seq_lens=[12000, 5000, 8000])),
    # two tokens per sequence, NoPE layer, four index heads
    ("verify_b3x2_nope_h4", lambda: workloads.verify_blocks(seed=1517, tokens=2, seq_lens=[7000, 3000, 5200],
                                                           rope=False, num_heads=4)),
    # a prefill chunk whose rows cross k = 2048 (rows of <= k keys take everything) and end inside
    # a 1024-key chunk, 70 queries (the last group is partial)
    ("prefill_across_k", lambda: _prefill(1518, 2100, 2010, 2080)),
    ("prefill_600_on_9000", lambda: _prefill(1519, 9600, 9000, 9600)),
    ("interleaved_sequences", lambda: _interleaved(1520)),
]


@pytest.mark.parametrize("name,make", GROUPED_CASES, ids=[c[0] for c in GROUPED_CASES])
def test_grouped_index_topk_matches_oracle(dsa, name, make):
    wl = make()
    g = wl.to("cuda")
    assert _grouped(dsa, g), "this layout takes the grouped score kernel"
    P = _pipe()
    fus, sep = P.alloc_buffers(g, prefill=True), P.alloc_buffers(g, prefill=True)
    P.index_and_select(g, fus)
    P.index_scores(g, sep)
    P.select(g, sep)
    torch.cuda.synchronize()
    idx, ln = fus.idx.cpu().numpy(), fus.length.cpu().numpy()
    sc = fus.scores.cpu().numpy()
    ssep = sep.scores.cpu().numpy()
    for t in range(wl.num_q):
        n = int(wl.q_pos[t]) + 1
        assert np.array_equal(sc[t, :n], ssep[t, :n]), f"{name} q{t}: the one-call path writes the same scores"
        ref, rl = O.topk_row(sc[t, :n].astype(np.float64), wl.topk)
        assert ln[t] == rl and np.array_equal(idx[t, :wl.topk], ref), f"{name} q{t}: selection differs"
        assert idx[t, :rl].max() < n, f"{name} q{t}: a key past the query's position"
    assert torch.equal(fus.idx, sep.idx) and torch.equal(fus.length, sep.length)
    for t in sorted({0, wl.num_q // 2, wl.num_q - 1}):
        check_selection(idx[t], ln[t], O.index_scores(wl, t), wl.topk, f"{name} q{t}", rms_admitted_ok=False)


def test_grouped_repeat_calls_self_clean(dsa):
    """Three calls in a row on one workspace (each selection clears the bookkeeping it used), then
    a decode-shaped call (whose score kernel emits its own candidates) on the same workspace."""
    P = _pipe()
    wl = workloads.verify_blocks(seed=1521, tokens=4, seq_lens=[15000, 6000]).to("cuda")
    buf = P.alloc_buffers(wl, prefill=True)
    first = None
    for _ in range(3):
        P.index_and_select(wl, buf)
        torch.cuda.synchronize()
        if first is None:
            first = buf.idx.clone()
        assert torch.equal(first, buf.idx)
    dec = workloads.make_workload(name="dec", seed=1522, seq_lens=[15000, 6000], max_ctx=15000).to("cuda")
    bd = P.alloc_buffers(dec)
    bd.ws_topk = buf.ws_topk
    P.index_and_select(dec, bd)
    torch.cuda.synchronize()
    sc, idx = bd.scores.cpu().numpy(), bd.idx.cpu().numpy()
    for t in range(dec.num_q):
        ref, rl = O.topk_row(sc[t, :int(dec.q_pos[t]) + 1].astype(np.float64), dec.topk)
        assert np.array_equal(idx[t, :dec.topk], ref)


def _mla_ref(wl, t, idx, ln):
    idx = np.asarray(idx)
    sel = idx[:ln][idx[:ln] >= 0]
    rows = O.cache_rows(wl, int(wl.q_seq[t]), sel)
    ro, rl = O.mla_attend(wl.mla_q[t], rows, wl.rope_dim, wl.softmax_scale)
    return ro, rl, mla_lse_bound(O.to_f64(wl.mla_q[t]), rows, wl.rope_dim, wl.softmax_scale, wl.fp8)


VERIFY_STEP_CASES = [
    ("b4x4_rope", dict(seed=1530, tokens=4, seq_lens=[20000, 9000, 30000, 4500]), 0),
    ("b2x4_rope_split5", dict(seed=1531, tokens=4, seq_lens=[16000, 12000]), 5),
    ("b3x3_nope", dict(seed=1532, tokens=3, seq_lens=[12000, 5000, 8000], rope=False), 0),
]


@pytest.mark.parametrize("name,kw,splits", VERIFY_STEP_CASES, ids=[c[0] for c in VERIFY_STEP_CASES])
def test_verify_block_layer_step(dsa, name, kw, splits):
    """A decode step over verify blocks: per-token selections (causal) and attention outputs
    against the oracle; the MLA runs split across workgroups with a sequence's tokens grouped on
    one XCD."""
    wl = workloads.verify_blocks(**kw)
    g = wl.to("cuda")
    P = _pipe()
    buf = P.alloc_buffers(g, num_splits=splits)
    P.layer_step(g, buf, num_splits=splits)
    torch.cuda.synchronize()
    idx, ln = buf.idx.cpu().numpy(), buf.length.cpu().numpy()
    out, lse = buf.out.cpu().numpy(), buf.lse.cpu().numpy()
    for t in range(wl.num_q):
        s = O.index_scores(wl, t)
        assert len(s) == int(wl.q_pos[t]) + 1
        check_selection(idx[t], ln[t], s, wl.topk, f"{name} q{t}", rms_admitted_ok=False)
        ro, rl, bound = _mla_ref(wl, t, idx[t], int(ln[t]))
        check_attention(out[t], lse[t], ro, rl, True, f"{name} q{t}", lse_abs=bound)
