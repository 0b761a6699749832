"""The no-allocation sparse MLA decode entry point against the one that takes a workspace.

dsa_sparse_mla_decode_noalloc runs the same kernels with the split partials in the library's
per-GPU scratch buffer.  Two calls in a row (the second smaller, reusing what the first left in
the buffer), then an fp32-cache call: each must give exactly the outputs of dsa_sparse_mla_decode
on the same inputs, and those outputs must match the float64 oracle.
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import dsa_oracle as O
from tests.parity_util import check_attention, mla_lse_bound

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    assert torch.cuda.is_available(), "GPU tests need the MI355X"
    import dsa_sparse_attention_indexer_amd as m
    return m


def _lists(n_ctx, lens, seed):
    rng = np.random.default_rng(seed)
    idx = np.full((len(lens), 2048), -1, np.int32)
    for t, L in enumerate(lens):
        idx[t, :L] = np.sort(rng.choice(n_ctx, L, replace=False))
    return idx


def _both(dsa, wl, idx, lens, splits):
    g = wl.to("cuda")
    T, H = wl.num_q, wl.mla_heads
    it, lt = torch.from_numpy(idx).cuda(), torch.as_tensor(lens, dtype=torch.int32).cuda()
    out_ws, lse_ws = torch.empty(T, H, 512, device="cuda"), torch.empty(T, H, device="cuda")
    out_na, lse_na = torch.full((T, H, 512), 7.0, device="cuda"), torch.full((T, H), 7.0, device="cuda")
    dsa.dsa_sparse_mla_decode(g.mla_q, g.kv, g.kv_scale, g.q_seq, it, lt, out_ws, lse_ws,
                              softmax_scale=wl.softmax_scale, num_splits=splits)
    dsa.dsa_sparse_mla_decode_noalloc(g.mla_q, g.kv, g.kv_scale, g.q_seq, it, lt, out_na, lse_na,
                                      softmax_scale=wl.softmax_scale, num_splits=splits)
    torch.cuda.synchronize()
    assert torch.equal(out_ws, out_na) and torch.equal(lse_ws, lse_na), "no-allocation outputs differ"
    o, l = out_na.cpu().numpy(), lse_na.cpu().numpy()
    for t, L in enumerate(lens):
        sel = idx[t, :L]
        rows = O.cache_rows(wl, int(wl.q_seq[t]), sel)
        ro, rl = O.mla_attend(wl.mla_q[t], rows, wl.rope_dim, wl.softmax_scale)
        if L == 0:
            assert np.all(o[t] == 0) and np.all(np.isneginf(l[t]))
            continue
        bound = mla_lse_bound(O.to_f64(wl.mla_q[t]), rows, wl.rope_dim, wl.softmax_scale, wl.fp8)
        check_attention(o[t], l[t], ro, rl, wl.fp8, f"noalloc q{t}", lse_abs=bound)


def test_noalloc_decode_matches_the_workspace_entry_point(dsa):
    assert dsa.lib().dsa_sparse_mla_noalloc_max_bytes() == 64 << 20
    # call 1: four 4000-row sequences, automatic splits (each query as two 32-head halves, 32 splits
    # each: 16.8 MB of partials)
    big = workloads.make_workload(name="na1", seed=71, seq_lens=[4000] * 4, max_ctx=4000, mla_q_std=8.0)
    lens1 = [2048, 1999, 2048, 77]
    _both(dsa, big, _lists(4000, lens1, 1), lens1, 0)
    # call 2: smaller (two queries, three splits, one empty list); the buffer holds call 1's partials
    small = workloads.make_workload(name="na2", seed=72, seq_lens=[2500, 3000], max_ctx=3000, rope=False)
    lens2 = [1500, 0]
    _both(dsa, small, _lists(2500, lens2, 2), lens2, 3)
    # call 3: the fp32 cache path (fp32 partials) through the same buffer
    f32 = workloads.make_workload(name="na3", seed=73, seq_lens=[3000, 3000], max_ctx=3000, fp8=False,
                                  q_dtype=torch.float32)
    lens3 = [2048, 1024]
    _both(dsa, f32, _lists(3000, lens3, 3), lens3, 0)


def test_noalloc_decode_rejects_partials_above_its_buffer(dsa):
    wl = workloads.make_workload(name="na4", seed=74, seq_lens=[3000] * 16, max_ctx=3000).to("cuda")
    idx = torch.zeros(16, 2048, dtype=torch.int32, device="cuda")
    lens = torch.full((16,), 2048, dtype=torch.int32, device="cuda")
    out = torch.full((16, 64, 512), 3.0, device="cuda")
    with pytest.raises(dsa.DsaError) as e:   # 16 queries x 64 splits x 64 heads: 134 MB of partials
        dsa.dsa_sparse_mla_decode_noalloc(wl.mla_q, wl.kv, wl.kv_scale, wl.q_seq, idx, lens, out,
                                          softmax_scale=wl.softmax_scale, num_splits=64)
    assert e.value.status == dsa.DSA_ERR_UNSUPPORTED and "bytes" in str(e.value)
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)   # nothing was launched
