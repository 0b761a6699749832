"""GPU parity at the full benchmark sizes, on sampled queries.

Each workload is generated on the GPU with its full shape (batch, context, heads, fp8 caches) and
run through the same layer step, launch configuration and buffers the benchmark uses; the float64
oracle then recomputes a few sampled queries one by one (index scores over the whole context,
the selection, the sparse attention) from a CPU copy of that query's own sequence.
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import dsa_oracle as O
from tests.parity_util import check_attention, check_block_selection, check_selection, mla_lse_bound

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pipe():
    assert torch.cuda.is_available(), "GPU tests need the MI355X"
    from dsa_sparse_attention_indexer_amd import pipeline
    return pipeline


def _score_tol(ref):
    return 2e-6 * float(np.sqrt(np.mean(ref * ref))) + 2e-6 * np.abs(ref)


def _check_queries(wl, buf, samples, *, block=False, fp8=True, where=""):
    torch.cuda.synchronize()
    for t in samples:
        sub = workloads.slice_query(wl, t)
        n = int(sub.q_pos[0]) + 1
        ref = O.index_scores(sub, 0)
        got = buf.scores[t, :n].cpu().numpy().astype(np.float64)
        assert np.all(np.abs(got - ref[:n]) <= _score_tol(ref[:n])), f"{where} q{t}: index scores"
        idx, ln = buf.idx[t].cpu().numpy(), int(buf.length[t])
        if block:
            check_block_selection(idx, ln, ref, n - 1, where=f"{where} q{t}")
        else:
            check_selection(idx, ln, ref, wl.topk, f"{where} q{t}", rms_admitted_ok=False)
        ro, rl = O.sparse_mla_row(sub, 0, idx, ln)
        bound = mla_lse_bound(O.to_f64(sub.mla_q[0]), O.cache_rows(sub, 0, idx[:ln][idx[:ln] >= 0]), sub.rope_dim,
                              sub.softmax_scale, fp8)
        check_attention(buf.out[t].cpu().numpy(), buf.lse[t].cpu().numpy(), ro, rl, fp8, f"{where} q{t}",
                        lse_abs=bound)
        print(f"{where} q{t}: ok (n={n}, len={ln})", flush=True)


def test_config0_decode_b1_ctx8192_f32(pipe):
    wl = workloads.config0(device="cuda")
    buf = pipe.alloc_buffers(wl)
    pipe.layer_step(wl, buf)
    _check_queries(wl, buf, [0], fp8=False, where="b1 8K f32")


def test_config1_decode_b64_ctx16k_32k(pipe):
    wl = workloads.config1(device="cuda")
    buf = pipe.alloc_buffers(wl)
    pipe.layer_step(wl, buf)
    _check_queries(wl, buf, [0, 37, 63], where="b64 16K-32K")


@pytest.mark.parametrize("variant", ["a", "b"])
def test_config2_decode_b16_ctx128k(pipe, variant):
    wl = workloads.config2(variant, device="cuda")
    buf = pipe.alloc_buffers(wl)
    pipe.layer_step(wl, buf)
    _check_queries(wl, buf, [0, 15], where=f"b16 128K {variant}")


def test_config2c_shared_indexer_at_128k(pipe):
    wa = workloads.config2("a", device="cuda")
    ba, bc = pipe.alloc_buffers(wa), pipe.alloc_buffers(wa)
    pipe.layer_step(wa, ba)
    pipe.layer_step(wa, bc, shared_from=ba)
    torch.cuda.synchronize()
    assert torch.equal(ba.out, bc.out) and torch.equal(ba.lse, bc.lse)
    for t in (3,):
        sub = workloads.slice_query(wa, t)
        ro, rl = O.sparse_mla_row(sub, 0, ba.idx[t].cpu().numpy(), int(ba.length[t]))
        check_attention(bc.out[t].cpu().numpy(), bc.lse[t].cpu().numpy(), ro, rl, True, f"shared q{t}")


def test_config3_chunked_prefill_4096_on_61440(pipe):
    wl = workloads.config3(device="cuda")
    buf = pipe.alloc_buffers(wl, prefill=True)
    pipe.layer_step(wl, buf, prefill=True)
    _check_queries(wl, buf, [0, 2048, 4095], where="prefill")


def test_config4_block_sparse_b4_ctx512k(pipe):
    wl = workloads.config4(device="cuda")
    buf = pipe.alloc_buffers(wl, block_sparse=True)
    pipe.layer_step(wl, buf, block_sparse=True)   # the selection from block maxima alone: no score rows
    pipe.index_scores(wl, buf)                     # the score rows, for the score check below
    _check_queries(wl, buf, [0, 3], block=True, where="block 512K")
