"""GPU parity: every stage of the HIP path against the float64 CPU oracle, through the C ABI.

Small cases span several tiles and ragged tails and finish in seconds on the oracle; the
full-size configurations are checked on sampled queries in the same launch configuration the
benchmark times.
"""
import math

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


def _score_tol(ref):
    # fp32 / two-term fp16 scores agree with float64 to ~1e-6 of the row's RMS
    return 2e-6 * math.sqrt(float(np.mean(ref * ref))) + 2e-6 * np.abs(ref)


# ---------------------------------------------------------------------------------------------
# index scores
# ---------------------------------------------------------------------------------------------

SCORE_CASES = [
    # name, kwargs for make_workload
    ("fp32_rope", dict(seq_lens=[3000], max_ctx=3000, fp8=False, q_dtype=torch.float32)),
    ("fp8_rope_ragged", dict(seq_lens=[700, 2049, 4100, 1], max_ctx=4104)),
    ("fp8_nope", dict(seq_lens=[1500, 2600], max_ctx=2600, rope=False)),
    ("fp8_h4", dict(seq_lens=[5000, 333], max_ctx=5000, num_heads=4)),
    ("fp8_f32q_nossmax", dict(seq_lens=[1025], max_ctx=1028, q_dtype=torch.float32, ssmax=False)),
    ("f32_bf16q_h7", dict(seq_lens=[900], max_ctx=900, fp8=False, num_heads=7)),
    # >= 256 queries take the grouped many-query path (queries prepared once, 4 per workgroup)
    ("fp8_prefill_grouped", dict(seq_lens=[6000], max_ctx=6000, q_positions=list(range(5699, 6000)))),
    ("fp8_grouped_mixed_seqs", dict(seq_lens=[3000, 2500, 1200], max_ctx=3000,
                                    q_positions=[(37 * i) % 1100 + 50 for i in range(258)],
                                    q_seqs=[i % 3 for i in range(258)])),
]


@pytest.mark.parametrize("name,kw", SCORE_CASES, ids=[c[0] for c in SCORE_CASES])
def test_index_scores_match_oracle(dsa, name, kw):
    wl = workloads.make_workload(name=name, seed=101, **kw)
    g = wl.to("cuda")
    buf = _pipe().alloc_buffers(g)
    _pipe().index_scores(g, buf)
    torch.cuda.synchronize()
    sc = buf.scores.cpu().numpy()
    for t in range(wl.num_q):
        ref = O.index_scores(wl, t)
        got = sc[t, :ref.shape[0]].astype(np.float64)
        err = np.abs(got - ref)
        assert np.all(err <= _score_tol(ref)), f"{name} q{t}: max err {err.max():.3g} rms {np.sqrt(np.mean(ref**2)):.3g}"


def _qtile_case(name):
    """Workloads of the query-tile score kernel (sequences averaging 16 or more queries, 8-query
    groups x 8192-key ranges filling 512 or more workgroups): a ragged prefill-like chunk and three
    sequences whose queries interleave, so that groups span sequences."""
    rng = np.random.default_rng(17)
    if name == "qtile_one_seq":
        pos = np.sort(rng.choice(70001, size=461, replace=False))
        pos[0], pos[-1] = 0, 70000
        return workloads.make_workload(name=name, seed=31, seq_lens=[70001], max_ctx=70001,
                                       q_positions=pos.tolist())
    lens = [40000, 17000, 9000]
    seqs = np.repeat(np.arange(3), [420, 260, 141])          # runs of one sequence ...
    cut = rng.choice(seqs.size, size=60, replace=False)        # ... with 60 queries moved around
    seqs[np.sort(cut)] = rng.permutation(seqs[cut])
    pos = np.array([rng.integers(0, lens[b]) for b in seqs])
    pos[:3] = [lens[seqs[0]] - 1, 0, 8191]
    return workloads.make_workload(name=name, seed=32, seq_lens=lens, max_ctx=40000,
                                   q_positions=pos.tolist(), q_seqs=seqs.tolist())


@pytest.mark.parametrize("name", ["qtile_one_seq", "qtile_mixed_seqs"])
def test_index_scores_query_tiles_match_oracle(dsa, name):
    wl = _qtile_case(name)
    T, B = wl.num_q, wl.num_seqs
    assert T >= 16 * B and -(-T // 8) * -(-wl.max_ctx // 8192) >= 512   # the query-tile kernel's range
    g = wl.to("cuda")
    buf = _pipe().alloc_buffers(g)
    buf.scores.fill_(float("nan"))
    _pipe().index_scores(g, buf)
    torch.cuda.synchronize()
    sc = buf.scores.cpu().numpy()
    keys = [O.cache_keys(wl, b, int(wl.seq_len[b])) for b in range(B)]   # decoded once per sequence
    s_s = None if wl.ssmax_s is None else O.to_f64(wl.ssmax_s)
    s_b = None if wl.ssmax_b is None else O.to_f64(wl.ssmax_b)
    inv = None if wl.inv_freq is None else O.to_f64(wl.inv_freq)
    for t in range(T):
        p, b = int(wl.q_pos[t]), int(wl.q_seq[t])
        qp = O.index_query(wl.index_q[t], p, s_s, s_b, inv)
        ref = O.index_scores_row(qp, O.to_f64(wl.index_w[t]), keys[b][:p + 1])
        got = sc[t, :p + 1].astype(np.float64)
        err = np.abs(got - ref)
        assert np.all(err <= _score_tol(ref)), f"{name} q{t} (seq {b}, p {p}): max err {err.max():.3g}"
        assert np.all(np.isnan(sc[t, p + 1:])), f"{name} q{t}: columns past p written"


def test_index_scores_exact_on_integers(dsa):
    """Integer q, fp8 keys and weights, unit scales, no RoPE / SSMax: S * 64 is an exact integer."""
    T, H, L = 2, 32, 700
    gen = torch.Generator().manual_seed(5)
    wl = workloads.make_workload(name="int", seed=5, seq_lens=[L, L], max_ctx=L, rope=False, ssmax=False,
                                 q_dtype=torch.float32)
    wl.index_q = torch.randint(-3, 4, (T, H, 128), generator=gen).float()
    wl.index_w = torch.randint(-5, 6, (T, H), generator=gen).float()
    keys = torch.randint(-8, 9, (2, L, 128), generator=gen).float()
    wl.index_k = keys.to(torch.float8_e4m3fn).view(torch.uint8)
    wl.index_k_scale = torch.ones(2, L)
    g = wl.to("cuda")
    buf = _pipe().alloc_buffers(g)
    _pipe().index_scores(g, buf)
    torch.cuda.synchronize()
    sc = buf.scores.cpu().numpy().astype(np.float64)
    q = wl.index_q.numpy().astype(np.int64)
    w = wl.index_w.numpy().astype(np.int64)
    k = keys.numpy().astype(np.int64)
    for t in range(T):
        dots = q[t] @ k[t].T                                   # exact integers [H][L]
        exact = (w[t][:, None] * np.maximum(dots, 0)).sum(0)   # = 64 * S, exactly
        assert np.array_equal(sc[t, :L] * 64.0, exact.astype(np.float64)), f"q{t}"
        assert np.allclose(O.index_scores(wl, t) * 64.0, exact, rtol=0, atol=1e-9)


def test_index_scores_position_zero_and_untouched_tail(dsa):
    wl = workloads.make_workload(name="p0", seed=7, seq_lens=[1, 300], max_ctx=300)
    g = wl.to("cuda")
    buf = _pipe().alloc_buffers(g)
    buf.scores.fill_(12345.0)
    _pipe().index_scores(g, buf)
    torch.cuda.synchronize()
    sc = buf.scores.cpu().numpy()
    assert np.all(sc[0, 1:] == 12345.0) and np.all(sc[1, 300:] == 12345.0)
    ref = O.index_scores(wl, 0)
    assert abs(sc[0, 0] - ref[0]) <= _score_tol(ref)[0]


# ---------------------------------------------------------------------------------------------
# top-k: bit-exact on the GPU's own fp32 scores
# ---------------------------------------------------------------------------------------------

def _run_topk(dsa, rows, qpos, k, ld=None):
    T = len(rows)
    ld = ld or max(4, (max(len(r) for r in rows) + 3) // 4 * 4)
    sc = torch.full((T, ld), float("nan"), dtype=torch.float32)
    for t, r in enumerate(rows):
        sc[t, :len(r)] = torch.as_tensor(r, dtype=torch.float32)
    sc = sc.cuda()
    qp = torch.as_tensor(qpos, dtype=torch.int32).cuda()
    idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
    ln = torch.empty(T, dtype=torch.int32, device="cuda")
    dsa.dsa_topk(sc, qp, k, idx, ln)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), ln.cpu().numpy()


TOPK_CASES = [
    ("random_mixed_lengths", 2048, [5000, 2047, 2048, 2049, 4096, 4097, 12289, 1, 0]),
    ("small_k", 16, [15, 16, 17, 100, 4095, 4096, 4097, 9000]),
    ("k1", 1, [1, 2, 5000]),
    ("big_row", 2048, [131072]),
    ("k_above_lds_resolve", 5000, [4999, 5000, 5001, 20000]),   # k > 4096: the streaming finish
]


@pytest.mark.parametrize("name,k,lens", TOPK_CASES, ids=[c[0] for c in TOPK_CASES])
@pytest.mark.parametrize("dist", ["normal", "ties3", "allequal", "signed_zero"])
def test_topk_bit_exact(dsa, name, k, lens, dist):
    rng = np.random.default_rng(len(lens) * 1000 + k)
    rows = []
    for n in lens:
        if dist == "normal":
            r = rng.standard_normal(n).astype(np.float32)
        elif dist == "ties3":
            r = rng.choice(np.array([-1.5, 0.25, 3.0], np.float32), n)
        elif dist == "allequal":
            r = np.full(n, 0.5, np.float32)
        else:
            r = rng.choice(np.array([-0.0, 0.0, 1.0, -2.0], np.float32), n)
        rows.append(r)
    qpos = [n - 1 for n in lens]
    idx, ln = _run_topk(dsa, rows, qpos, k)
    for t, r in enumerate(rows):
        ref, rl = O.topk_row(r.astype(np.float64), k)
        assert ln[t] == rl, f"{name}/{dist} row {t}: len {ln[t]} != {rl}"
        assert np.array_equal(idx[t], ref), f"{name}/{dist} row {t} (n={len(r)}): selections differ"


def test_topk_heavy_threshold_bin_overflow(dsa):
    """More than the candidate buffer's worth of keys share the threshold's top bits."""
    rng = np.random.default_rng(3)
    n = 60000
    r = (1.0 + rng.integers(0, 4, n) * 2.0 ** -20).astype(np.float32)    # 4 values in one top-11-bit bin
    r[rng.choice(n, 100, replace=False)] = 7.0
    idx, ln = _run_topk(dsa, [r], [n - 1], 2048)
    ref, _ = O.topk_row(r.astype(np.float64), 2048)
    assert np.array_equal(idx[0], ref)


@pytest.mark.parametrize("dist", ["normal", "ties3", "heavy_bin"])
def test_topk_many_rows(dsa, dist):
    """Hundreds of rows of mixed lengths in one call, including rows whose threshold bin holds more
    keys than the candidate buffer (the streaming finish)."""
    rng = np.random.default_rng(77)
    lens = rng.integers(0, 40000, 300).tolist() + [40000, 2048, 2049, 16384, 16385, 32769]
    rows = []
    for n in lens:
        if dist == "normal":
            r = rng.standard_normal(n).astype(np.float32)
        elif dist == "ties3":
            r = rng.choice(np.array([-1.5, 0.25, 3.0], np.float32), n)
        else:   # more than the candidate buffer's worth of keys in the threshold's top bits
            r = (1.0 + rng.integers(0, 4, n) * 2.0 ** -20).astype(np.float32)
            r[rng.choice(n, min(n, 100), replace=False)] = 7.0
        rows.append(r)
    idx, ln = _run_topk(dsa, rows, [n - 1 for n in lens], 2048)
    for t, r in enumerate(rows):
        ref, rl = O.topk_row(r.astype(np.float64), 2048)
        assert ln[t] == rl, f"{dist} row {t}: len {ln[t]} != {rl}"
        assert np.array_equal(idx[t], ref), f"{dist} row {t} (n={len(r)}): selections differ"


def test_topk_sample_misleads_threshold(dsa):
    """Rows (128 or more: the one-workgroup-per-row kernel) whose sampled columns -- the first 1024
    of every 8192 -- hold far higher scores than the rest: the threshold taken from the sample lies
    above the k-th key, so fewer than k keys reach the candidate list and the row must still come
    out exact.  Mixed with ordinary rows and rows whose unsampled tail holds the top keys."""
    rng = np.random.default_rng(78)
    rows, pos = [], []
    for i in range(160):
        n = int(rng.integers(20000, 70000))
        r = rng.standard_normal(n).astype(np.float32)
        c = np.arange(n)
        if i % 3 == 0:
            r[(c % 8192) < 1024] += 50.0           # the sample holds the largest scores
        elif i % 3 == 1:
            r[(c % 8192) >= 1024] += 50.0          # the top keys all lie outside the sample
        rows.append(r)
        pos.append(n - 1)
    idx, ln = _run_topk(dsa, rows, pos, 2048)
    for t, r in enumerate(rows):
        ref, rl = O.topk_row(r.astype(np.float64), 2048)
        assert ln[t] == rl and np.array_equal(idx[t], ref), f"row {t} (n={len(r)}): selections differ"


def test_topk_row_shorter_than_ld_and_deterministic(dsa):
    rng = np.random.default_rng(11)
    rows = [rng.standard_normal(9000).astype(np.float32) for _ in range(3)]
    a, _ = _run_topk(dsa, rows, [8999, 4000, 2100], 2048, ld=9000)
    b, _ = _run_topk(dsa, rows, [8999, 4000, 2100], 2048, ld=9000)
    assert np.array_equal(a, b)
    for t, p in enumerate([8999, 4000, 2100]):
        ref, _ = O.topk_row(rows[t][:p + 1].astype(np.float64), 2048)
        assert np.array_equal(a[t], ref)


# ---------------------------------------------------------------------------------------------
# block selection: bit-exact on the GPU's own fp32 scores
# ---------------------------------------------------------------------------------------------

def test_block_select_bit_exact(dsa):
    rng = np.random.default_rng(21)
    lens = [128 * 40 + 17, 128 * 16, 128 * 16 + 1, 1000, 128 * 100]
    T = len(lens)
    ld = (max(lens) + 3) // 4 * 4
    sc = rng.standard_normal((T, ld)).astype(np.float32)
    sc[0, 128 * 40:] -= 50.0                        # the recent block scores lowest: still kept
    sc[4, :] = np.round(sc[4, :])                   # many equal block maxima: lower block wins
    qp = torch.as_tensor([n - 1 for n in lens], dtype=torch.int32).cuda()
    idx = torch.empty(T, 2048, dtype=torch.int32, device="cuda")
    ln = torch.empty(T, dtype=torch.int32, device="cuda")
    dsa.dsa_block_select(torch.from_numpy(sc).cuda(), qp, idx, ln)
    torch.cuda.synchronize()
    gi, gl = idx.cpu().numpy(), ln.cpu().numpy()
    for t, n in enumerate(lens):
        ref, rl = O.block_select_row(sc[t, :n].astype(np.float64), n - 1)
        assert gl[t] == rl and np.array_equal(gi[t], ref), f"row {t}"


def test_block_select_many_blocks(dsa):
    """More block maxima than the picker keeps in registers (1-key blocks over 20000 keys)."""
    rng = np.random.default_rng(23)
    n = 20000
    sc = rng.standard_normal((2, n)).astype(np.float32)
    sc[1, :] = np.round(sc[1, :] * 4)                 # ties between single-key blocks
    qp = torch.as_tensor([n - 1, 17000], dtype=torch.int32).cuda()
    idx = torch.empty(2, 2048, dtype=torch.int32, device="cuda")
    ln = torch.empty(2, dtype=torch.int32, device="cuda")
    dsa.dsa_block_select(torch.from_numpy(sc).cuda(), qp, idx, ln, block=1, nblocks=16)
    torch.cuda.synchronize()
    gi, gl = idx.cpu().numpy(), ln.cpu().numpy()
    for t, p in enumerate([n - 1, 17000]):
        ref, rl = O.block_select_row(sc[t, :p + 1].astype(np.float64), p, block=1, nblocks=16)
        assert gl[t] == rl and np.array_equal(gi[t], ref), f"row {t}"


# ---------------------------------------------------------------------------------------------
# sparse MLA on a given selection
# ---------------------------------------------------------------------------------------------

def _mla_ref(wl, t, idx, ln):
    """The oracle's attention for query t over idx[:ln] and the LSE bound for the kernel's rounding."""
    idx = np.asarray(idx)
    sel = idx[:ln][idx[:ln] >= 0]
    rows = O.cache_rows(wl, int(wl.q_seq[t]), sel)
    ro, rl = O.mla_attend(wl.mla_q[t], rows, wl.rope_dim, wl.softmax_scale)
    return ro, rl, mla_lse_bound(O.to_f64(wl.mla_q[t]), rows, wl.rope_dim, wl.softmax_scale, wl.fp8)


MLA_CASES = [
    ("fp8_rope_decode", dict(seq_lens=[3000, 2500, 900], max_ctx=3000), False, 0),
    ("fp8_nope_decode", dict(seq_lens=[2600, 2100], max_ctx=2600, rope=False), False, 0),
    ("fp8_rope_prefill", dict(seq_lens=[2600], max_ctx=2600, q_positions=[2100, 2300, 2599, 100]), True, 0),
    ("fp8_rope_split3", dict(seq_lens=[4000, 3000], max_ctx=4000), False, 3),
    ("f32_rope_decode", dict(seq_lens=[2500, 3000], max_ctx=3000, fp8=False, q_dtype=torch.float32), False, 0),
    ("f32_nope_prefill", dict(seq_lens=[2200], max_ctx=2200, fp8=False, q_dtype=torch.float32, rope=False,
                              q_positions=[2199, 50]), True, 0),
    # selections wider than the 2048 slots staged in LDS at a time (and top-k above 4096)
    ("fp8_topk4100_prefill", dict(seq_lens=[6000], max_ctx=6000, q_positions=[5999, 4500, 3000], topk=4100), True, 0),
    ("fp8_topk4100_decode", dict(seq_lens=[6000, 5000], max_ctx=6000, topk=4100), False, 0),
    # the other head counts of the fp8 path, 32 splits (two batches of partials in the combine) and
    # one split (the decode writes its output directly)
    ("fp8_rope_h48_split32", dict(seq_lens=[3000, 2200], max_ctx=3000, mla_heads=48), False, 32),
    ("fp8_nope_h32", dict(seq_lens=[2600, 1500], max_ctx=2600, rope=False, mla_heads=32), False, 0),
    ("fp8_rope_h16_split1", dict(seq_lens=[2500], max_ctx=2500, mla_heads=16), False, 1),
]


@pytest.mark.parametrize("name,kw,prefill,splits", MLA_CASES, ids=[c[0] for c in MLA_CASES])
def test_sparse_mla_matches_oracle(dsa, name, kw, prefill, splits):
    wl = workloads.make_workload(name=name, seed=202, **kw)
    g = wl.to("cuda")
    P = _pipe()
    buf = P.alloc_buffers(g, prefill=prefill, num_splits=splits)
    P.layer_step(g, buf, prefill=prefill, num_splits=splits)
    torch.cuda.synchronize()
    idx, ln = buf.idx.cpu().numpy(), buf.length.cpu().numpy()
    out, lse = buf.out.cpu().numpy(), buf.lse.cpu().numpy()
    for t in range(wl.num_q):
        ro, rl, bound = _mla_ref(wl, t, idx[t], int(ln[t]))
        check_attention(out[t], lse[t], ro, rl, wl.fp8, f"{name} q{t}", lse_abs=bound)


def test_sparse_mla_ragged_lists_and_empty(dsa):
    """-1 entries inside a list are skipped; len = 0 gives zeros and -inf."""
    wl = workloads.make_workload(name="rag", seed=303, seq_lens=[3000, 3000, 3000], max_ctx=3000)
    rng = np.random.default_rng(0)
    idx = np.full((3, 2048), -1, np.int32)
    idx[0, :1500] = np.sort(rng.choice(3000, 1500, replace=False))
    idx[0, 100:140] = -1
    idx[1, :77] = np.sort(rng.choice(3000, 77, replace=False))
    lens = np.array([1500, 77, 0], np.int32)
    g = wl.to("cuda")
    for prefill in (False, True):
        out = torch.empty(3, 64, 512, device="cuda")
        lse = torch.empty(3, 64, device="cuda")
        fn = dsa.dsa_sparse_mla_prefill if prefill else dsa.dsa_sparse_mla_decode
        fn(g.mla_q, g.kv, g.kv_scale, g.q_seq, torch.from_numpy(idx).cuda(), torch.from_numpy(lens).cuda(), out, lse,
           softmax_scale=wl.softmax_scale)
        torch.cuda.synchronize()
        o, l = out.cpu().numpy(), lse.cpu().numpy()
        for t in range(2):
            sel = idx[t, :lens[t]]
            ro, rl = O.mla_attend(wl.mla_q[t], O.cache_rows(wl, t, sel[sel >= 0]), 64, wl.softmax_scale)
            check_attention(o[t], l[t], ro, rl, True, f"prefill={prefill} q{t}")
        assert np.all(o[2] == 0) and np.all(np.isneginf(l[2]))


@pytest.mark.parametrize("rope", [True, False], ids=["rope", "nope"])
def test_sparse_mla_head_split_matches_oracle(dsa, rope):
    """Automatic splits at 8..32 queries run each query as two 32-head halves (the halves share the
    row lists; their partials and statistics are separate): 12 queries, peaked softmax, ragged and
    empty lists, -1 holes; every query against the oracle, and the same call with explicit splits
    (no head split) agrees to the same tolerance."""
    T, n = 12, 6000
    wl = workloads.make_workload(name="hsplit", seed=1717, seq_lens=[n] * T, max_ctx=n, rope=rope, mla_q_std=16.0)
    rng = np.random.default_rng(17)
    lens = np.array([2048, 2048, 1999, 1024, 777, 300, 256, 255, 64, 63, 1, 0], np.int32)
    idx = np.full((T, 2048), -1, np.int32)
    for t in range(T):
        idx[t, :lens[t]] = np.sort(rng.choice(n, lens[t], replace=False))
    idx[0, 500:530] = -1
    g = wl.to("cuda")
    it, lt = torch.from_numpy(idx).cuda(), torch.from_numpy(lens).cuda()
    res = []
    for splits in (0, 8):
        out = torch.empty(T, 64, 512, device="cuda")
        lse = torch.empty(T, 64, device="cuda")
        dsa.dsa_sparse_mla_decode(g.mla_q, g.kv, g.kv_scale, g.q_seq, it, lt, out, lse,
                                  softmax_scale=wl.softmax_scale, num_splits=splits)
        torch.cuda.synchronize()
        res.append((out.cpu().numpy(), lse.cpu().numpy()))
    for (o, l), tag in zip(res, ("auto (head split)", "explicit 8 splits")):
        for t in range(T):
            if lens[t] == 0:
                assert np.all(o[t] == 0) and np.all(np.isneginf(l[t])), f"{tag} q{t}"
                continue
            sel = idx[t, :lens[t]]
            rows = O.cache_rows(wl, t, sel[sel >= 0])
            ro, rl = O.mla_attend(wl.mla_q[t], rows, wl.rope_dim, wl.softmax_scale)
            bound = mla_lse_bound(O.to_f64(wl.mla_q[t]), rows, wl.rope_dim, wl.softmax_scale, True)
            check_attention(o[t], l[t], ro, rl, True, f"{tag} q{t}", lse_abs=bound)


def test_sparse_equals_dense_when_selection_covers_context(dsa):
    wl = workloads.make_workload(name="dense", seed=404, seq_lens=[1800, 2048], max_ctx=2048)
    g = wl.to("cuda")
    P = _pipe()
    buf = P.alloc_buffers(g)
    P.layer_step(g, buf)
    torch.cuda.synchronize()
    out, lse = buf.out.cpu().numpy(), buf.lse.cpu().numpy()
    ln = buf.length.cpu().numpy()
    for t in range(2):
        assert ln[t] == int(wl.q_pos[t]) + 1
        ro, rl = O.dense_mla_row(wl, t)
        check_attention(out[t], lse[t], ro, rl, True, f"dense q{t}")


# ---------------------------------------------------------------------------------------------
# end to end on small workloads: selection within the band, attention within tolerance
# ---------------------------------------------------------------------------------------------

E2E_CASES = [
    ("rope", dict(seq_lens=[9000, 4097, 12000], max_ctx=12000), False),
    ("nope", dict(seq_lens=[7000, 2049], max_ctx=7000, rope=False), False),
    ("prefill", dict(seq_lens=[6000], max_ctx=6000, q_positions=[1000, 2047, 2048, 4095, 5999]), False),
    ("block", dict(seq_lens=[128 * 70 + 5, 128 * 30], max_ctx=128 * 70 + 8, num_heads=4), True),
]


@pytest.mark.parametrize("name,kw,block", E2E_CASES, ids=[c[0] for c in E2E_CASES])
def test_layer_step_end_to_end(dsa, name, kw, block):
    wl = workloads.make_workload(name=name, seed=505, **kw)
    g = wl.to("cuda")
    P = _pipe()
    prefill = "q_positions" in kw
    buf = P.alloc_buffers(g, prefill=prefill, block_sparse=block)
    P.layer_step(g, buf, prefill=prefill, block_sparse=block)
    torch.cuda.synchronize()
    idx, ln = buf.idx.cpu().numpy(), buf.length.cpu().numpy()
    out, lse = buf.out.cpu().numpy(), buf.lse.cpu().numpy()
    for t in range(wl.num_q):
        s = O.index_scores(wl, t)
        if block:
            ref, rl = O.block_select_row(s, int(wl.q_pos[t]))
            assert ln[t] == rl and np.array_equal(idx[t], ref), f"{name} q{t}: block selection differs"
        else:
            check_selection(idx[t], ln[t], s, wl.topk, f"{name} q{t}", rms_admitted_ok=False)
        ro, rl, bound = _mla_ref(wl, t, idx[t], int(ln[t]))
        check_attention(out[t], lse[t], ro, rl, True, f"{name} q{t}", lse_abs=bound)


def test_shared_indexer_layer_reuses_selection(dsa):
    a = workloads.make_workload(name="a", seed=606, seq_lens=[5000, 6000], max_ctx=6000)
    c = workloads.make_workload(name="c", seed=607, seq_lens=[5000, 6000], max_ctx=6000)
    ga, gc = a.to("cuda"), c.to("cuda")
    P = _pipe()
    ba, bc = P.alloc_buffers(ga), P.alloc_buffers(gc)
    P.layer_step(ga, ba)
    idx_before = ba.idx.clone()
    P.layer_step(gc, bc, shared_from=ba)
    torch.cuda.synchronize()
    assert torch.equal(idx_before, ba.idx)
    idx, ln = ba.idx.cpu().numpy(), ba.length.cpu().numpy()
    out, lse = bc.out.cpu().numpy(), bc.lse.cpu().numpy()
    for t in range(2):
        ro, rl = O.sparse_mla_row(c, t, idx[t], int(ln[t]))
        check_attention(out[t], lse[t], ro, rl, True, f"shared q{t}")


def test_repeat_runs_are_bit_identical(dsa):
    wl = workloads.make_workload(name="rep", seed=707, seq_lens=[20000, 9000], max_ctx=20000)
    g = wl.to("cuda")
    P = _pipe()
    buf = P.alloc_buffers(g)
    res = []
    for _ in range(3):
        P.layer_step(g, buf)
        torch.cuda.synchronize()
        res.append((buf.scores.clone(), buf.idx.clone(), buf.out.clone(), buf.lse.clone()))
    for r in res[1:]:
        for x, y in zip(res[0], r):
            assert torch.equal(x, y)


# ---------------------------------------------------------------------------------------------
# fused scores + top-k: identical to the two separate calls; one workspace serves every call
# ---------------------------------------------------------------------------------------------

FUSED_CASES = [
    ("ragged", dict(seq_lens=[9000, 2048, 2049, 1, 4097], max_ctx=9000), False),
    ("prefill_positions", dict(seq_lens=[7000], max_ctx=7000, q_positions=[0, 2047, 2048, 5000, 6999]), False),
    ("constant_keys", dict(seq_lens=[6000, 3000], max_ctx=6000), True),   # every score ties
    # paths where the histogram comes from a pass after the scores: fp32 keys, and 300 queries
    # (the grouped score kernel)
    ("f32_keys", dict(seq_lens=[5000, 2500], max_ctx=5000, fp8=False, q_dtype=torch.float32), False),
    ("grouped_300_queries", dict(seq_lens=[6000], max_ctx=6000, q_positions=list(range(2000, 6000, 13))[:300]), False),
]


@pytest.mark.parametrize("name,kw,constant", FUSED_CASES, ids=[c[0] for c in FUSED_CASES])
def test_fused_index_topk_equals_separate_calls(dsa, name, kw, constant):
    wl = workloads.make_workload(name=name, seed=808, **kw)
    g = wl.to("cuda")
    if constant:
        g.index_k[:] = g.index_k[0, 0]
        g.index_k_scale[:] = g.index_k_scale[0, 0]
    P = _pipe()
    sep, fus, spl = P.alloc_buffers(g), P.alloc_buffers(g), P.alloc_buffers(g)
    P.index_scores(g, sep)
    P.select(g, sep)
    P.index_and_select(g, fus)
    P.index_scores_hist(g, spl)   # the same in two calls (dsa_indexer_scores_hist + dsa_topk_hist)
    P.select_hist(g, spl)
    torch.cuda.synchronize()
    for t in range(wl.num_q):
        n = int(wl.q_pos[t]) + 1
        assert torch.equal(sep.scores[t, :n], fus.scores[t, :n]), f"{name} q{t}: scores differ"
        assert torch.equal(sep.scores[t, :n], spl.scores[t, :n]), f"{name} q{t}: split-call scores differ"
    assert torch.equal(sep.idx, fus.idx) and torch.equal(sep.length, fus.length), f"{name}: selections differ"
    assert torch.equal(sep.idx, spl.idx) and torch.equal(sep.length, spl.length), f"{name}: split-call selections differ"
    if constant:   # all scores equal: the lowest k columns win
        idx = fus.idx.cpu().numpy()
        for t in range(wl.num_q):
            n = int(wl.q_pos[t]) + 1
            assert np.array_equal(idx[t], np.arange(wl.topk)) if n > wl.topk else idx[t, 0] == 0


FUSED_ORACLE_CASES = [
    # 4096-key chunks (many workgroups) and 1024-key chunks (few), ragged rows
    ("chunks4096", dict(seq_lens=[40000] * 12 + [9000, 2049, 2048, 100000], max_ctx=100000)),
    ("chunks1024", dict(seq_lens=[20000, 7000, 4097], max_ctx=20000)),
    ("nope_h4", dict(seq_lens=[30000, 12000], max_ctx=30000, rope=False, num_heads=4)),
]


@pytest.mark.parametrize("name,kw", FUSED_ORACLE_CASES, ids=[c[0] for c in FUSED_ORACLE_CASES])
def test_fused_index_topk_matches_oracle(dsa, name, kw):
    """dsa_indexer_topk (score chunks emit their own candidates): the selection is the oracle's
    top-k of the GPU's scores bit for bit, and within the tie band of the oracle's own scores."""
    wl = workloads.make_workload(name=name, seed=1313, **kw)
    g = wl.to("cuda")
    P = _pipe()
    buf = P.alloc_buffers(g)
    P.index_and_select(g, buf)
    torch.cuda.synchronize()
    _check_rows_exact(wl, buf, wl.topk, f"fused {name}")
    idx, ln = buf.idx.cpu().numpy(), buf.length.cpu().numpy()
    for t in (0, wl.num_q - 1):
        check_selection(idx[t], ln[t], O.index_scores(wl, t), wl.topk, f"fused {name} q{t}", rms_admitted_ok=False)


def test_fused_index_topk_clustered_top_keys(dsa):
    """The top keys of each row are packed into the last 3000 positions with distinct, increasing
    scores: the chunks there hold far more of the top k than their share, emit only digits above
    the row's k-th digit, and the row must take the exact passes; the result is still the oracle's
    selection of the GPU's scores."""
    n = 20000
    wl = workloads.make_workload(name="clustered", seed=1414, seq_lens=[n, n], max_ctx=n)
    for t in range(2):
        s = O.index_scores(wl, t)
        best = int(np.argmax(s))
        assert s[best] > 0
        lo = n - 3000
        wl.index_k[t, lo:n] = wl.index_k[t, best]
        wl.index_k_scale[t, lo:n] = wl.index_k_scale[t, best] * torch.linspace(1.0, 2.0, 3000)
    g = wl.to("cuda")
    P = _pipe()
    fus, sep = P.alloc_buffers(g), P.alloc_buffers(g)
    P.index_and_select(g, fus)
    P.index_scores(g, sep)
    P.select(g, sep)
    torch.cuda.synchronize()
    _check_rows_exact(wl, fus, wl.topk, "clustered fused")
    assert torch.equal(fus.idx, sep.idx)
    idx = fus.idx.cpu().numpy()
    assert np.all(idx[:, 0] >= n - 3000), "the top keys are the packed ones"


def test_fused_index_topk_overflow_ties_and_stale_workspace(dsa):
    """Fused selection on 1024-key chunks (98 per row, so each chunk's item region holds 167):
    row 0 has 2000 keys that tie for the top score, so the chunks holding them emit more candidates
    than their regions hold and the row takes the exact passes; row 1 takes the emitted path.  Then
    the same call on a workspace holding a stale histogram (an interrupted split call) and on one
    of random bytes.  Every selection is the oracle's top-k of the GPU's scores."""
    n0, n1 = 100000, 60000
    wl = workloads.make_workload(name="overflow", seed=1515, seq_lens=[n0, n1], max_ctx=n0)
    s = O.index_scores(wl, 0)
    best = int(np.argmax(s))
    wl.index_k[0, 50000:52000] = wl.index_k[0, best]
    wl.index_k_scale[0, 50000:52000] = wl.index_k_scale[0, best]
    g = wl.to("cuda")
    P = _pipe()
    buf = P.alloc_buffers(g)
    P.index_and_select(g, buf)
    torch.cuda.synchronize()
    _check_rows_exact(wl, buf, wl.topk, "tied block")
    idx = buf.idx.cpu().numpy()
    assert np.isin(np.arange(50000, 52000), idx[0]).all(), "the tied top keys are all kept"
    P.index_scores_hist(g, buf)   # a histogram left behind by an interrupted split call
    P.index_and_select(g, buf)
    torch.cuda.synchronize()
    _check_rows_exact(wl, buf, wl.topk, "stale histogram")
    gen = torch.Generator(device="cuda").manual_seed(7)
    buf.ws_topk.copy_(torch.randint(0, 256, buf.ws_topk.shape, generator=gen, device="cuda", dtype=torch.int32)
                      .to(torch.uint8))
    P.index_and_select(g, buf)
    torch.cuda.synchronize()
    _check_rows_exact(wl, buf, wl.topk, "random workspace")
    P.index_and_select(g, buf)
    torch.cuda.synchronize()
    _check_rows_exact(wl, buf, wl.topk, "after recovery")


def test_fused_workspace_reused_across_shapes(dsa):
    P = _pipe()
    big = workloads.make_workload(name="big", seed=909, seq_lens=[12000, 8000, 5000], max_ctx=12000).to("cuda")
    small = workloads.make_workload(name="small", seed=910, seq_lens=[3000], max_ctx=3000).to("cuda")
    bb, bs = P.alloc_buffers(big), P.alloc_buffers(small)
    shared_ws = bb.ws_topk
    for i, (wl, buf) in enumerate(((big, bb), (small, bs), (big, bb), (small, bs))):
        buf.ws_topk = shared_ws
        if i % 2:   # the separate top-k call shares the same workspace
            P.index_scores(wl, buf)
            P.select(wl, buf)
        else:
            P.index_and_select(wl, buf)
        torch.cuda.synchronize()
        idx, ln = buf.idx.cpu().numpy(), buf.length.cpu().numpy()
        sc = buf.scores.cpu().numpy()
        for t in range(wl.num_q):
            n = int(wl.q_pos[t]) + 1
            ref, rl = O.topk_row(sc[t, :n].astype(np.float64), wl.topk)
            assert ln[t] == rl and np.array_equal(idx[t], ref), f"call {i} q{t}: selection differs"


def _check_rows_exact(wl, buf, k, where):
    """The selection equals the oracle's top-k of the GPU's own scores, bit for bit."""
    idx, ln = buf.idx.cpu().numpy(), buf.length.cpu().numpy()
    sc = buf.scores.cpu().numpy()
    for t in range(wl.num_q):
        n = min(int(wl.q_pos[t]) + 1, wl.max_ctx)
        ref, rl = O.topk_row(sc[t, :n].astype(np.float64), k)
        assert ln[t] == rl and np.array_equal(idx[t, :k], ref), f"{where} q{t}: selection differs"


def test_topk_workspace_stale_state_self_heals(dsa):
    """The top-k workspace carries a histogram between the two halves of a selection.  Whatever an
    earlier call left in it (an interrupted scores_hist, a histogram built for another k, two
    histograms piled up, none at all, or random bytes), every later selection is exact, and the
    call after a recovery finds the workspace clean again."""
    P = _pipe()
    wl = workloads.make_workload(name="stale", seed=1212, seq_lens=[20000, 9000, 3000, 2049], max_ctx=20000).to("cuda")
    buf = P.alloc_buffers(wl)
    k = wl.topk

    def pair():
        P.index_scores_hist(wl, buf)
        P.select_hist(wl, buf)
        torch.cuda.synchronize()
        _check_rows_exact(wl, buf, k, "pair")

    pair()
    # 1. interrupted: scores + histogram, no selection; then a normal pair on the same workspace
    P.index_scores_hist(wl, buf)
    torch.cuda.synchronize()
    pair()
    # 2. scores + histogram twice (the histogram counts every key twice), then the selection
    P.index_scores_hist(wl, buf)
    P.index_scores_hist(wl, buf)
    P.select_hist(wl, buf)
    torch.cuda.synchronize()
    _check_rows_exact(wl, buf, k, "double histogram")
    pair()
    # 3. a selection with no histogram before it (the previous selection cleared it)
    P.select_hist(wl, buf)
    torch.cuda.synchronize()
    _check_rows_exact(wl, buf, k, "no histogram")
    # 4. histogram built for k = 2048, selection with k = 4000 (rows of 3000 and 2049 keys take
    #    every key and must clear what the histogram left), then matched calls again
    idx_big = torch.empty(wl.num_q, 4000, dtype=torch.int32, device="cuda")
    P.index_scores_hist(wl, buf)
    dsa.dsa_topk_hist(buf.scores, wl.q_pos, 4000, idx_big, buf.length, wl.max_ctx, buf.ws_topk)
    torch.cuda.synchronize()
    sc = buf.scores.cpu().numpy()
    ib = idx_big.cpu().numpy()
    for t in range(wl.num_q):
        n = int(wl.q_pos[t]) + 1
        ref, rl = O.topk_row(sc[t, :n].astype(np.float64), 4000)
        assert np.array_equal(ib[t], ref), f"k mismatch q{t}"
    pair()
    pair()
    # 5. the separate top-k call after an interrupted fused half
    P.index_scores_hist(wl, buf)
    P.select(wl, buf)
    torch.cuda.synchronize()
    _check_rows_exact(wl, buf, k, "separate call after an interrupted half")
    pair()
    # 6. a workspace of random bytes (never cleared)
    gen = torch.Generator(device="cuda").manual_seed(5)
    buf.ws_topk.copy_(torch.randint(0, 256, buf.ws_topk.shape, generator=gen, device="cuda", dtype=torch.int32)
                      .to(torch.uint8))
    pair()
    pair()
    P.select(wl, buf)
    torch.cuda.synchronize()
    _check_rows_exact(wl, buf, k, "separate call on a used workspace")


# ---------------------------------------------------------------------------------------------
# sparse MLA with peaked softmax: logits spread over many binades, so the running maximum moves
# after the first tile (the lazy rescale of the accumulators) and the split combine weighs
# partials that differ by many powers of two
# ---------------------------------------------------------------------------------------------

def _log2_range(wl, t, idx, ln):
    """Per-head spread (log2) of the logits over the selection, and how far (log2) the maximum over
    the whole list exceeds the maximum over its first 32 keys."""
    sel = np.asarray(idx)[:ln]
    rows = O.cache_rows(wl, int(wl.q_seq[t]), sel[sel >= 0])
    q = O.to_f64(wl.mla_q[t])
    d = 512 + wl.rope_dim
    z = wl.softmax_scale * (q[:, :d] @ rows[:, :d].T) / math.log(2.0)
    return z.max(1) - z.min(1), z.max(1) - z[:, :32].max(1)


PEAKED_CASES = [
    # name, make_workload kwargs, prefill, splits
    ("fp8_rope_decode_auto", dict(seq_lens=[3000, 2500, 2100], max_ctx=3000), False, 0),
    ("fp8_rope_decode_split1", dict(seq_lens=[3000, 2500], max_ctx=3000), False, 1),
    ("fp8_rope_decode_split3", dict(seq_lens=[4000, 3000], max_ctx=4000), False, 3),
    ("fp8_rope_decode_split32", dict(seq_lens=[3000, 2200], max_ctx=3000), False, 32),
    ("fp8_rope_prefill", dict(seq_lens=[2600], max_ctx=2600, q_positions=[2100, 2599, 100]), True, 0),
    ("fp8_nope_decode", dict(seq_lens=[2600, 2100], max_ctx=2600, rope=False), False, 0),
    ("fp8_nope_prefill", dict(seq_lens=[2600], max_ctx=2600, rope=False, q_positions=[2599, 2300]), True, 0),
    ("f32_rope_decode", dict(seq_lens=[2500, 3000], max_ctx=3000, fp8=False, q_dtype=torch.float32), False, 0),
    ("f32_nope_prefill", dict(seq_lens=[2200], max_ctx=2200, fp8=False, q_dtype=torch.float32, rope=False,
                              q_positions=[2199, 2000]), True, 0),
]


@pytest.mark.parametrize("name,kw,prefill,splits", PEAKED_CASES, ids=[c[0] for c in PEAKED_CASES])
def test_sparse_mla_peaked_softmax(dsa, name, kw, prefill, splits):
    """Queries ~N(0, 64^2): per-head logits span tens of binades over the selection."""
    wl = workloads.make_workload(name=name, seed=222, mla_q_std=64.0, **kw)
    g = wl.to("cuda")
    P = _pipe()
    buf = P.alloc_buffers(g, prefill=prefill, num_splits=splits)
    P.layer_step(g, buf, prefill=prefill, num_splits=splits)
    torch.cuda.synchronize()
    idx, ln = buf.idx.cpu().numpy(), buf.length.cpu().numpy()
    out, lse = buf.out.cpu().numpy(), buf.lse.cpu().numpy()
    spread = []
    for t in range(wl.num_q):
        rng_, late = _log2_range(wl, t, idx[t], int(ln[t]))
        spread.append(np.median(rng_))
        ro, rl, bound = _mla_ref(wl, t, idx[t], int(ln[t]))
        check_attention(out[t], lse[t], ro, rl, wl.fp8, f"{name} q{t}", lse_abs=bound)
        # zeroed logits would put the LSE at ln(len): far outside the bound
        assert np.all(np.abs(np.log(float(ln[t])) - rl) > 10 * (bound + 1e-3)), f"{name} q{t}: LSE check is blind"
    assert min(spread) > 20.0, f"{name}: logits not peaked enough ({spread})"


LATE_PEAK_CASES = [
    # name, fp8, rope, prefill, splits, list lengths
    ("fp8_rope_decode_auto", True, True, False, 0, [2048, 1500]),
    ("fp8_rope_decode_split1", True, True, False, 1, [2048, 700]),
    ("fp8_rope_decode_split3", True, True, False, 3, [2048, 1999]),
    ("fp8_rope_decode_split32", True, True, False, 32, [2048, 2047]),
    ("fp8_rope_prefill", True, True, True, 0, [2048, 1200]),
    ("fp8_nope_decode", True, False, False, 0, [2048, 1800]),
    ("f32_rope_decode", False, True, False, 0, [2048, 1500]),
    ("f32_rope_prefill", False, True, True, 0, [2048, 333]),
]


@pytest.mark.parametrize("name,fp8,rope,prefill,splits,lens", LATE_PEAK_CASES, ids=[c[0] for c in LATE_PEAK_CASES])
def test_sparse_mla_peak_in_last_tile_of_last_split(dsa, name, fp8, rope, prefill, splits, lens):
    """Every head's largest logit is the list's last key (the last tile of the last split), by a
    margin that grows across the heads from 2 to 60 natural-log units over the others: the
    running maximum jumps in the last tile, and the split combine weighs that split's partial
    against the others by up to 2^-80."""
    n = 4000
    T = len(lens)
    wl = workloads.make_workload(name=name, seed=333 + splits, seq_lens=[n] * T, max_ctx=n, fp8=fp8, rope=rope,
                                 q_dtype=torch.bfloat16 if fp8 else torch.float32)
    rng = np.random.default_rng(44 + splits)
    idx = np.full((T, 2048), -1, np.int32)
    d = 512 + wl.rope_dim
    q = O.to_f64(wl.mla_q).copy()
    for t, L in enumerate(lens):
        sel = np.sort(rng.choice(n, L, replace=False))
        idx[t, :L] = sel
        c = O.cache_rows(wl, t, sel[-1:])[0, :d]           # the peak key: the last slot of the list
        margin = np.linspace(2.0, 60.0, wl.mla_heads)       # nats above a typical logit
        q[t, :, :d] = 0.5 * q[t, :, :d] + (margin / (wl.softmax_scale * float(c @ c)))[:, None] * c[None, :]
    wl.mla_q = torch.from_numpy(q).to(wl.mla_q.dtype)
    lens_t = torch.as_tensor(lens, dtype=torch.int32)
    g = wl.to("cuda")
    out = torch.empty(T, wl.mla_heads, 512, device="cuda")
    lse = torch.empty(T, wl.mla_heads, device="cuda")
    ws = None
    if not prefill:
        need = dsa.dsa_sparse_mla_workspace_size(dsa.mla_desc(g.mla_q, g.kv, torch.empty(T, 2048, dtype=torch.int32),
                                                              wl.softmax_scale, splits))
        ws = torch.empty(max(16, need), dtype=torch.uint8, device="cuda")
        dsa.dsa_sparse_mla_decode(g.mla_q, g.kv, g.kv_scale, g.q_seq, torch.from_numpy(idx).cuda(), lens_t.cuda(),
                                  out, lse, softmax_scale=wl.softmax_scale, num_splits=splits, ws=ws)
    else:
        dsa.dsa_sparse_mla_prefill(g.mla_q, g.kv, g.kv_scale, g.q_seq, torch.from_numpy(idx).cuda(), lens_t.cuda(),
                                   out, lse, softmax_scale=wl.softmax_scale)
    torch.cuda.synchronize()
    o, l = out.cpu().numpy(), lse.cpu().numpy()
    for t, L in enumerate(lens):
        _, late = _log2_range(wl, t, idx[t], L)
        assert np.median(late) > 8.0, f"{name} q{t}: the peak does not move the running maximum ({np.median(late)})"
        ro, rl, bound = _mla_ref(wl, t, idx[t], L)
        check_attention(o[t], l[t], ro, rl, fp8, f"{name} q{t}", lse_abs=bound)


def test_topk_one_segment_holds_the_top_keys(dsa):
    """Fewer than 128 rows (segments that emit their own candidates): rows whose top keys crowd one
    8192-column segment, so that segment's own threshold lies above the row's k-th key and the row
    must take the exact passes; mixed with ordinary rows and rows whose top keys sit in the last,
    partial segment."""
    rng = np.random.default_rng(79)
    rows, pos = [], []
    for i in range(24):
        n = int(rng.integers(20000, 70000))
        r = rng.standard_normal(n).astype(np.float32)
        if i % 3 == 0:
            s0 = 8192 * int(rng.integers(0, n // 8192))
            r[s0:s0 + 8192] += 50.0                 # one whole segment above every other key
        elif i % 3 == 1:
            r[-3000:] += 50.0                       # the recent keys
        rows.append(r)
        pos.append(n - 1)
    idx, ln = _run_topk(dsa, rows, pos, 2048)
    for t, r in enumerate(rows):
        ref, rl = O.topk_row(r.astype(np.float64), 2048)
        assert ln[t] == rl and np.array_equal(idx[t], ref), f"row {t} (n={len(r)}): selections differ"


def test_topk_few_rows_on_a_random_workspace(dsa):
    """The one-pass selection for few rows adds each segment's histogram into the workspace: on a
    workspace of random bytes (an earlier call that never finished) every row is still exact, the
    call leaves the rows' histograms cleared, and the next call on it is exact too."""
    rng = np.random.default_rng(80)
    rows = [rng.standard_normal(int(rng.integers(9000, 60000))).astype(np.float32) for _ in range(12)]
    rows[3][:5000] += 50.0                           # one row whose top keys crowd its first segment
    T = len(rows)
    ld = (max(len(r) for r in rows) + 3) // 4 * 4
    sc = torch.full((T, ld), float("nan"), dtype=torch.float32)
    for t, r in enumerate(rows):
        sc[t, :len(r)] = torch.as_tensor(r)
    sc = sc.cuda()
    qp = torch.as_tensor([len(r) - 1 for r in rows], dtype=torch.int32).cuda()
    ws = torch.as_tensor(rng.integers(0, 256, dsa.dsa_topk_workspace_size(T, ld, 2048), dtype=np.uint8)).cuda()
    for call in range(2):
        idx = torch.empty(T, 2048, dtype=torch.int32, device="cuda")
        ln = torch.empty(T, dtype=torch.int32, device="cuda")
        dsa.dsa_topk(sc, qp, 2048, idx, ln, ws=ws)
        torch.cuda.synchronize()
        gi, gl = idx.cpu().numpy(), ln.cpu().numpy()
        for t, r in enumerate(rows):
            ref, rl = O.topk_row(r.astype(np.float64), 2048)
            assert gl[t] == rl and np.array_equal(gi[t], ref), f"call {call} row {t}: selections differ"
        hist = ws.view(torch.int32)[:4096].cpu().numpy()   # row 0's histogram words
        assert call == 0 or not hist.any(), "the histogram is not cleared"
