"""Pins for the CPU oracle: each checks it against something other than itself.

The pages print no worked numeric example for the path, so the oracle is pinned by
library routines (torch's fp8 / bf16 codecs, numpy / scipy sorting and log-sum-exp),
closed forms chosen so the answer is known by construction, invariants of the
definitions, and brute force on tiny inputs.  A dropped scale, a wrong sign, a swapped
pair or head index, or a transposed product each fails at least one test here.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import workloads
from oracle import dsa_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------------------------
# Storage formats
# ---------------------------------------------------------------------------------------------

def test_e4m3fn_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = O.decode_e4m3fn(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    both_nan = np.isnan(ours) & np.isnan(ref)
    assert np.all(both_nan | (ours == ref))
    assert np.isnan(ours).sum() == 2            # 0x7F and 0xFF only


@pytest.mark.parametrize("code,value", [(0x38, 1.0), (0xB8, -1.0), (0x7E, 448.0), (0x01, 2.0 ** -9),
                                        (0x08, 2.0 ** -6), (0x07, 7 * 2.0 ** -9), (0x00, 0.0),
                                        (0x3C, 1.5), (0x40, 2.0), (0x30, 0.5)])
def test_e4m3fn_hand_values(code, value):
    assert O.decode_e4m3fn(np.array([code], np.uint8))[0] == value


def test_bf16_decode_matches_torch():
    x = torch.randn(4096, generator=torch.Generator().manual_seed(5)) * 100
    b = x.to(torch.bfloat16)
    ours = O.to_f64(b)
    assert np.array_equal(ours, b.to(torch.float64).numpy())


def test_quantiser_roundtrip_within_half_ulp():
    x = torch.randn(64, 576, generator=torch.Generator().manual_seed(7)) / 24
    codes, scales = workloads.quantize_e4m3(x, 64)
    v = O.dequant_rows(codes.numpy(), scales.numpy(), 64)
    err = np.abs(v - x.double().numpy()) / np.repeat(scales.double().numpy(), 64, axis=1)
    # E4M3 has 3 mantissa bits: relative half-ulp is 2^-4; in scaled units at most 448 * 2^-4 = 16 (top binade)
    assert err.max() <= 16.0 + 1e-9
    # the largest magnitude of each block maps exactly to +-448
    assert np.all(np.isclose(np.abs(v).reshape(64, 9, 64).max(-1),
                             np.abs(x.double().numpy()).reshape(64, 9, 64).max(-1), rtol=1e-6))


# ---------------------------------------------------------------------------------------------
# RoPE (interleaved pairs) and SSMax
# ---------------------------------------------------------------------------------------------

def test_rope_rotates_e0_to_cos_sin_and_keeps_pairs():
    th = np.array([0.3, 1.1])
    x = np.zeros(6); x[0] = 1.0
    y = O.rope_interleaved(x, th)
    assert np.allclose(y, [math.cos(0.3), math.sin(0.3), 0, 0, 0, 0], atol=1e-15)
    x = np.zeros(6); x[3] = 1.0          # second element of pair 1: (0,1) -> (-sin, cos)
    y = O.rope_interleaved(x, th)
    assert np.allclose(y, [0, 0, -math.sin(1.1), math.cos(1.1), 0, 0], atol=1e-15)
    x = np.zeros(6); x[5] = 2.0          # beyond the rotary dims: untouched
    assert np.array_equal(O.rope_interleaved(x, th), x)


def test_rope_identity_norm_composition():
    rng = np.random.default_rng(0)
    q = rng.standard_normal((32, 128))
    inv = workloads.inv_freq_table().double().numpy()
    assert np.array_equal(O.rope_interleaved(q, O.rope_angles(0, inv)), q)
    assert np.array_equal(O.rope_interleaved(q, np.zeros(32)), q)
    r = O.rope_interleaved(q, O.rope_angles(1000, inv))
    pair = lambda a: a[:, :64].reshape(32, 32, 2)
    assert np.allclose(np.linalg.norm(pair(r), axis=-1), np.linalg.norm(pair(q), axis=-1), rtol=1e-13)
    assert np.array_equal(r[:, 64:], q[:, 64:])
    a, b = O.rope_angles(700, inv), O.rope_angles(300, inv)
    assert np.allclose(O.rope_interleaved(O.rope_interleaved(q, a), b), O.rope_interleaved(q, a + b), atol=1e-12)
    assert np.allclose(O.rope_interleaved(O.rope_interleaved(q, a), -a), q, atol=1e-12)


def test_rope_angle_uses_absolute_position():
    # pair 0 angle at position p is p * inv_freq[0]; choose inv_freq[0] so the angle is pi/2 at p=4
    inv = np.zeros(32); inv[0] = math.pi / 8
    q = np.zeros((1, 128)); q[0, 0] = 1.0
    y = O.index_query(q, 4, inv_freq=inv)
    assert np.allclose(y[0, :2], [0.0, 1.0], atol=1e-15)


def test_ssmax_closed_form():
    s = np.array([0.1, 0.2]); b = np.array([1.0, 0.5])
    assert np.allclose(O.ssmax_multiplier(s, b, 0), b)                 # ln(1) = 0 -> m = b
    pe = math.e ** 3 - 1                                                # ln(pe+1) = 3
    m = s * math.log(pe + 1) + b
    assert np.allclose(m, [1.3, 1.1])
    q = np.ones((2, 128))
    y = O.index_query(q, 1023, ssmax_s=s, ssmax_b=b)
    assert np.allclose(y[:, 0], s * math.log(1024) + b)
    assert np.allclose(y, y[:, :1])                                     # a per-head scalar, no rotation


# ---------------------------------------------------------------------------------------------
# Index scores
# ---------------------------------------------------------------------------------------------

def test_scores_single_head_unit_query_picks_relu_of_one_key_dim():
    # w = sqrt(H) sqrt(D) on head 0 only, q_0 = e_i:  S(t) = max(k_t[i], 0) exactly.
    rng = np.random.default_rng(1)
    H, D, n = 32, 128, 50
    keys = rng.standard_normal((n, D))
    for i in (0, 5, 127):
        q = np.zeros((H, D)); q[0, i] = 1.0
        w = np.zeros(H); w[0] = math.sqrt(H) * math.sqrt(D)
        S = O.index_scores_row(q, w, keys)
        assert np.allclose(S, np.maximum(keys[:, i], 0.0), rtol=1e-14, atol=0)


def test_scores_exact_on_integers():
    # integer q, k, w: S * sqrt(32) * sqrt(128) = S * 64 is an exact integer, known by enumeration
    rng = np.random.default_rng(2)
    H, D, n = 32, 128, 40
    q = rng.integers(-3, 4, (H, D)).astype(np.float64)
    k = rng.integers(-3, 4, (n, D)).astype(np.float64)
    w = rng.integers(-5, 6, H).astype(np.float64)
    S = O.index_scores_row(q, w, k) * 64.0
    for t in range(n):
        acc = 0
        for h in range(H):
            d = sum(int(q[h, j]) * int(k[t, j]) for j in range(D))
            acc += int(w[h]) * max(d, 0)
        assert S[t] == pytest.approx(acc, abs=1e-9)


def test_scores_linear_in_weights_and_homogeneous_in_query():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((32, 128)); k = rng.standard_normal((64, 128))
    w1, w2 = rng.standard_normal(32), rng.standard_normal(32)
    assert np.allclose(O.index_scores_row(q, w1 + w2, k),
                       O.index_scores_row(q, w1, k) + O.index_scores_row(q, w2, k), atol=1e-12)
    assert np.allclose(O.index_scores_row(2.5 * q, w1, k), 2.5 * O.index_scores_row(q, w1, k), atol=1e-12)
    # SSMax with s = 0, b = 2.5 is the same as scaling the query
    assert np.allclose(O.index_query(q, 77, np.zeros(32), np.full(32, 2.5)), 2.5 * q)


def test_relu_nonnegativity_and_all_zero_rows_select_lowest_indices():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((32, 128)); k = rng.standard_normal((5000, 128))
    w = np.abs(rng.standard_normal(32))
    assert np.all(O.index_scores_row(q, w, k) >= 0)
    # every head's dot is <= 0 when all keys point against head 0 and other heads are zero
    q0 = np.zeros((32, 128)); q0[0] = 1.0
    kneg = -np.abs(k)
    S = O.index_scores_row(q0, rng.standard_normal(32), kneg)
    assert np.all(S == 0)
    idx, n = O.topk_row(S, 2048)
    assert n == 2048 and np.array_equal(idx, np.arange(2048))


def test_workload_scores_use_query_position_and_sequence():
    wl = workloads.make_workload(name="t", seed=11, seq_lens=[40, 70], max_ctx=80, fp8=True)
    s0 = O.index_scores(wl, 0); s1 = O.index_scores(wl, 1)
    assert s0.shape == (40,) and s1.shape == (70,)
    # recompute query 1 by hand: rotate with angle p*inv_freq, scale by SSMax, decode fp8 x scale
    p = 69
    q = O.to_f64(wl.index_q[1])
    inv = wl.inv_freq.double().numpy()
    qr = q.copy()
    for j in range(32):
        a = p * inv[j]
        x, y = q[:, 2 * j], q[:, 2 * j + 1]
        qr[:, 2 * j] = x * math.cos(a) - y * math.sin(a)
        qr[:, 2 * j + 1] = x * math.sin(a) + y * math.cos(a)
    m = wl.ssmax_s.double().numpy() * math.log(p + 1) + wl.ssmax_b.double().numpy()
    qr *= m[:, None]
    keys = torch.from_numpy(wl.index_k[1, :70].numpy()).view(torch.float8_e4m3fn).double().numpy()
    keys *= wl.index_k_scale[1, :70].double().numpy()[:, None]
    w = wl.index_w[1].double().numpy()
    ref = np.array([sum(w[h] / math.sqrt(32) * max(float(qr[h] @ keys[t]) / math.sqrt(128), 0) for h in range(32))
                    for t in range(70)])
    assert np.allclose(s1, ref, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------------------------
# Top-k
# ---------------------------------------------------------------------------------------------

def _brute_topk(s, k):
    order = sorted(range(len(s)), key=lambda t: (-s[t], t))
    keep = sorted(order[:k])
    return keep


@pytest.mark.parametrize("n,k", [(1, 1), (5, 3), (16, 16), (15, 16), (17, 16), (200, 7), (64, 1)])
@pytest.mark.parametrize("alphabet", [None, 3, 1])
def test_topk_brute_force(n, k, alphabet):
    rng = np.random.default_rng(n * 31 + k)
    if alphabet is None:
        s = rng.standard_normal(n)
    else:
        s = rng.integers(0, alphabet, n).astype(np.float64)
    idx, ln = O.topk_row(s, k)
    assert ln == min(n, k)
    want = list(range(n)) if n <= k else _brute_topk(list(s), k)
    assert list(idx[:ln]) == want
    assert np.all(idx[ln:] == -1)


def test_topk_signed_zero_is_one_value():
    s = np.array([-0.0, 0.0, -0.0, 0.0, -1.0, 1.0])
    idx, ln = O.topk_row(s, 3)
    assert list(idx) == [0, 1, 5]


def test_topk_exhaustive_tiny():
    # every score vector over a 3-letter alphabet of length 6, every k
    for s in itertools.product([-1.0, 0.0, 2.0], repeat=6):
        for k in range(1, 7):
            idx, ln = O.topk_row(np.array(s), k)
            chosen = set(idx[:ln].tolist())
            # defining property: no unchosen key beats a chosen one, and among equals lower index wins
            for a in chosen:
                for b in set(range(6)) - chosen:
                    assert s[a] > s[b] or (s[a] == s[b] and a < b)


@pytest.mark.parametrize("alphabet", [None, 2, 3, 7])
@pytest.mark.parametrize("k", [1, 2, 5, 16, 63, 64])
def test_kth_score_is_the_kth_entry_of_the_brute_force_order(alphabet, k):
    """kth_score(s, k) is the score of the k-th key in the (score desc, index asc) order that
    defines the selection, i.e. the lowest selected score: at most k-1 keys score above it and
    at least k score at or above it.  Checked against a plain sort by a Python key function,
    on tie-heavy rows and on rows one shorter, equal to and one longer than k."""
    rng = np.random.default_rng(100 * k + (alphabet or 0))
    for n in (k - 1, k, k + 1, 3 * k + 5, 200):
        if n < 1:
            continue
        s = rng.standard_normal(n) if alphabet is None else rng.integers(-1, alphabet - 1, n).astype(np.float64)
        got = O.kth_score(s, k)
        if n <= k:
            assert got is None
            continue
        order = sorted(range(n), key=lambda t: (-s[t], t))
        assert got == s[order[k - 1]]
        assert np.sum(s > got) <= k - 1 and np.sum(s >= got) >= k
        # the selection's lowest score is this value, and no unselected key scores above it
        idx, ln = O.topk_row(s, k)
        assert min(s[idx[:ln]]) == got and np.all(np.delete(s, idx[:ln]) <= got)


def test_kth_score_hand_values():
    s = np.array([3.0, 1.0, 3.0, 2.0, 3.0, 0.5])
    assert O.kth_score(s, 1) == 3.0 and O.kth_score(s, 3) == 3.0
    assert O.kth_score(s, 4) == 2.0 and O.kth_score(s, 5) == 1.0
    assert O.kth_score(s, 6) is None
    assert O.kth_score(np.array([-0.0, 0.0, -1.0]), 2) == 0.0


# ---------------------------------------------------------------------------------------------
# Block select
# ---------------------------------------------------------------------------------------------

def test_block_select_brute_force_and_forced_recent_block():
    rng = np.random.default_rng(9)
    pos = 128 * 20 + 37
    s = rng.standard_normal(pos + 1)
    s[128 * 20:] -= 100.0                      # the recent (partial) block scores lowest
    idx, ln = O.block_select_row(s, pos)
    nb = 21
    bmax = [max(s[j * 128:min(pos + 1, (j + 1) * 128)]) for j in range(nb)]
    best = sorted(range(20), key=lambda j: (-bmax[j], j))[:15]
    want = [t for j in sorted(best + [20]) for t in range(j * 128, min(pos + 1, (j + 1) * 128))]
    assert list(idx[:ln]) == want and ln == 15 * 128 + 38
    assert np.all(idx[ln:] == -1)


def test_block_select_short_context_takes_everything():
    s = np.random.default_rng(1).standard_normal(1000)
    idx, ln = O.block_select_row(s, 999)
    assert ln == 1000 and np.array_equal(idx[:1000], np.arange(1000))


# ---------------------------------------------------------------------------------------------
# Sparse MLA
# ---------------------------------------------------------------------------------------------

def _tiny_wl(fp8=True, rope=True, n=300, seed=21):
    return workloads.make_workload(name="t", seed=seed, seq_lens=[n], max_ctx=n, fp8=fp8, rope=rope,
                                   q_dtype=torch.bfloat16 if fp8 else torch.float32)


@pytest.mark.parametrize("fp8,rope", [(True, True), (False, True), (True, False)])
def test_sparse_equals_dense_when_k_covers_context(fp8, rope):
    wl = _tiny_wl(fp8, rope)
    s = O.index_scores(wl, 0)
    idx, n = O.topk_row(s, 2048)
    assert n == 300
    o1, l1 = O.sparse_mla_row(wl, 0, idx, n)
    o2, l2 = O.dense_mla_row(wl, 0)
    assert np.allclose(o1, o2, rtol=1e-12, atol=1e-15) and np.allclose(l1, l2, rtol=1e-12)


def test_mla_matches_scipy_softmax_and_logsumexp():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((64, 576)); rows = rng.standard_normal((37, 576)) / 24
    o, lse = O.mla_attend(q, rows, 64, 1 / math.sqrt(192))
    z = (q @ rows.T) / math.sqrt(192)
    assert np.allclose(lse, scipy.special.logsumexp(z, axis=1), rtol=1e-13)
    assert np.allclose(o, scipy.special.softmax(z, axis=1) @ rows[:, :512], rtol=1e-12, atol=1e-15)
    # NoPE: the rope part of the rows is ignored and q has 512 dims
    o0, l0 = O.mla_attend(q[:, :512], rows, 0, 0.1)
    z0 = 0.1 * (q[:, :512] @ rows[:, :512].T)
    assert np.allclose(l0, scipy.special.logsumexp(z0, axis=1), rtol=1e-13)


def test_mla_special_cases():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((64, 576)); rows = rng.standard_normal((20, 576))
    sig = 0.07
    # one key: output is that row's latent, LSE is its logit
    o, l = O.mla_attend(q, rows[:1], 64, sig)
    assert np.allclose(o, np.broadcast_to(rows[0, :512], (64, 512)))
    assert np.allclose(l, sig * (q @ rows[0]))
    # identical rows: output is the row, LSE = z + ln m
    same = np.repeat(rows[:1], 9, axis=0)
    o, l = O.mla_attend(q, same, 64, sig)
    assert np.allclose(o, np.broadcast_to(rows[0, :512], (64, 512)))
    assert np.allclose(l, sig * (q @ rows[0]) + math.log(9))
    # q = 0: uniform weights -> mean of rows, LSE = ln m
    o, l = O.mla_attend(np.zeros((64, 576)), rows, 64, sig)
    assert np.allclose(o, np.broadcast_to(rows[:, :512].mean(0), (64, 512)))
    assert np.allclose(l, math.log(20))
    # order of the index list does not matter
    perm = rng.permutation(20)
    a = O.mla_attend(q, rows, 64, sig); b = O.mla_attend(q, rows[perm], 64, sig)
    assert np.allclose(a[0], b[0], rtol=1e-12) and np.allclose(a[1], b[1], rtol=1e-13)
    # two keys: the weight of key 0 is the logistic of the logit gap (textbook closed form)
    o, l = O.mla_attend(q[:1], rows[:2], 64, sig)
    z = sig * (rows[:2] @ q[0])
    w0 = 1 / (1 + math.exp(z[1] - z[0]))
    assert np.allclose(o[0], w0 * rows[0, :512] + (1 - w0) * rows[1, :512], rtol=1e-12)


def test_mla_empty_selection():
    o, l = O.mla_attend(np.ones((64, 576)), np.zeros((0, 576)), 64, 0.1)
    assert np.all(o == 0) and np.all(np.isneginf(l))


def test_shared_indexer_layer_reuses_selection_verbatim():
    wl = workloads.make_workload(name="t", seed=12, seq_lens=[3000, 2500], max_ctx=3000)
    full = O.decode_layer(wl, [0, 1])
    other = workloads.make_workload(name="t2", seed=13, seq_lens=[3000, 2500], max_ctx=3000)
    shared = O.decode_layer(other, [0, 1], idx_override=(full["idx"], full["len"]))
    for i in range(2):
        o, l = O.sparse_mla_row(other, i, full["idx"][i], full["len"][i])
        assert np.array_equal(shared["out"][i], o) and shared["scores"][i] is None


# ---------------------------------------------------------------------------------------------
# Layout constants against the pages' byte counts
# ---------------------------------------------------------------------------------------------

def test_cache_byte_arithmetic_matches_pages():
    g = json.load(open(os.path.join(GOLDEN, "cache_bytes.json")))
    idx_bytes = workloads.INDEX_HEAD_DIM * 1 + 4           # fp8 key row + one fp32 scale
    assert idx_bytes == g["indexer_bytes_per_token_per_layer"]
    assert workloads.KV_ROW * 1 == g["latent_bytes_rocm_e4m3"]
    assert workloads.KV_ROW * 2 == g["latent_bytes_bf16"]
    assert g["kv_owner_layers"] == g["layers"] - g["kv_consumer_layers"]
    assert g["kv_owner_layers"] * g["latent_bytes_fp8_ds_mla"] == g["total_latent_fp8_ds_mla"]
    assert g["indexer_layers"] * idx_bytes == g["total_indexer"]
    assert g["total_latent_fp8_ds_mla"] + g["total_indexer"] == g["total_fp8_ds_mla"]
    assert g["kv_owner_layers"] * workloads.KV_ROW + g["total_indexer"] == g["total_rocm_e4m3"]
    assert g["kv_owner_layers"] * 2 * workloads.KV_ROW + g["total_indexer"] == g["total_bf16"]
    assert round(g["total_bf16"] / g["total_rocm_e4m3"], 2) == g["capacity_ratio_bf16_over_e4m3"]


# ---------------------------------------------------------------------------------------------
# Cache writers: the E4M3FN encoder, the quantiser, the indexer key path and latent rows
# ---------------------------------------------------------------------------------------------

def _e4m3_magnitudes():
    return torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_e4m3fn_encoder_matches_torch_cast_on_ties_and_random_values():
    m = _e4m3_magnitudes()
    mids = (m[:-1] + m[1:]) / 2                          # every tie between neighbours
    rng = np.random.default_rng(7)
    rand = np.concatenate([rng.normal(0, s, 20000) for s in (1e-3, 0.05, 1.0, 30.0, 150.0)])
    v = np.concatenate([m, mids, -mids, rand, [0.0, -0.0, 448.0, -448.0]])
    v = v[np.abs(v) <= 448.0]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = O.encode_e4m3fn(v)
    # torch rounds from float64 directly (no double rounding), so codes agree bit for bit
    assert np.array_equal(ours, ref)


def test_e4m3fn_encoder_ties_go_to_even_code_and_saturates():
    m = _e4m3_magnitudes()
    for c in range(126):
        mid = (m[c] + m[c + 1]) / 2
        assert O.encode_e4m3fn(mid) == (c if c % 2 == 0 else c + 1)
        assert O.encode_e4m3fn(-mid) == 0x80 | (c if c % 2 == 0 else c + 1)
        assert O.decode_e4m3fn(O.encode_e4m3fn(m[c])) == m[c]          # exact values round-trip
    assert O.encode_e4m3fn(449.0) == 0x7E and O.encode_e4m3fn(-1e9) == 0xFE
    assert O.encode_e4m3fn(np.nan) == 0x7F


def test_quantiser_maps_the_group_maximum_to_448_and_bounds_the_error():
    rng = np.random.default_rng(8)
    x = rng.normal(0, 3.0, (50, 128))
    x[3] = 0.0
    codes, scale = O.quantize_e4m3_rows(x, 128)
    assert scale.shape == (50, 1) and scale[3, 0] == 1.0 and np.all(codes[3] & 0x7F == 0)
    for r in (0, 1, 2, 10, 49):
        j = int(np.argmax(np.abs(x[r])))
        assert codes[r, j] & 0x7F == 0x7E                # |x| = amax -> 448
        assert np.isclose(scale[r, 0], np.abs(x[r]).max() / 448.0, rtol=0, atol=0)
    back = O.decode_e4m3fn(codes) * scale
    # relative half-spacing of E4M3 normals is 2^-4; subnormals are at most 2^-10 x scale off
    err = np.abs(back - x)
    assert np.all(err <= np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * scale) + 1e-12)
    # the same quantiser also produces the synthetic caches' format: 64-element groups
    c64, s64 = O.quantize_e4m3_rows(x[:, :128], 64)
    assert s64.shape == (50, 2)
    assert np.array_equal(c64[:, :64], O.quantize_e4m3_rows(x[:, :64], 64)[0])


def test_quantiser_agrees_with_torch_cast_of_the_float64_quotient():
    """The float64 quantiser against torch's E4M3FN cast of the same float64 quotient.  torch
    rounds a float64 through float32 first, so the two may differ only where the quotient lies
    within float32 rounding of a midpoint between two codes (double rounding); none of these
    values does, so every code must match."""
    rng = np.random.default_rng(9)
    x = rng.normal(0, 1.0, (200, 576))
    x[5, :64] = 0.0                                   # an all-zero group: scale 1, codes 0
    codes, scale = O.quantize_e4m3_rows(x, 64)
    xt = torch.from_numpy(x).reshape(200, 9, 64)
    amax = xt.abs().amax(-1)
    st = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    quot = xt / st.unsqueeze(-1)
    ref = quot.to(torch.float8_e4m3fn).view(torch.uint8).reshape(200, 576).numpy()
    mags = O.decode_e4m3fn(np.arange(127, dtype=np.uint8))
    mids = (mags[1:] + mags[:-1]) / 2
    q = np.abs(quot.reshape(200, 576).numpy())
    near_mid = np.min(np.abs(q[..., None] - mids), axis=-1) <= 2.0 ** -23 * q
    assert not near_mid.any()
    assert np.array_equal(codes, ref)
    assert np.array_equal(scale, st.numpy())
    assert scale[5, 0] == 1.0 and np.all(codes[5, :64] == 0)


def test_layer_norm_matches_torch_layer_norm():
    rng = np.random.default_rng(10)
    y = rng.normal(0.3, 2.0, (7, 128))
    w, b = rng.uniform(0.5, 1.5, 128), rng.normal(0, 0.2, 128)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(y), (128,), torch.from_numpy(w), torch.from_numpy(b),
                                         eps=1e-5).numpy()
    assert np.allclose(O.layer_norm(y, w, b, 1e-5), ref, rtol=1e-12, atol=1e-12)


def test_index_key_with_identity_projection_is_layer_norm_then_rope():
    rng = np.random.default_rng(11)
    x = rng.normal(0, 1, 128)
    eye = np.eye(128)
    one, zero = np.ones(128), np.zeros(128)
    k0 = O.index_key(x, eye, one, zero, 1e-6, pos=0, inv_freq=workloads.inv_freq_table().numpy())
    k_norope = O.index_key(x, eye, one, zero, 1e-6, pos=0)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x), (128,), eps=1e-6).numpy()
    assert np.allclose(k0, ref, atol=1e-12) and np.allclose(k_norope, ref, atol=1e-12)   # pos 0: no turn
    # closed forms of a unit LayerNorm: zero mean, mean square var / (var + eps)
    var = x.var()
    assert abs(k_norope.mean()) < 1e-12 and np.isclose((k_norope ** 2).mean(), var / (var + 1e-6), rtol=1e-12)


def test_index_key_projection_orientation_and_rope_pairs():
    rng = np.random.default_rng(12)
    D = 96
    x = rng.normal(0, 1, D)
    wk = rng.normal(0, 1, (128, D))
    w, b = rng.uniform(0.5, 1.5, 128), rng.normal(0, 0.1, 128)
    invf = workloads.inv_freq_table().numpy().astype(np.float64)
    pos = 777
    k = O.index_key(x, wk, w, b, 1e-6, pos, invf)
    # brute force: output o is the dot of wk's row o with x (wk is [out][in])
    y = np.array([sum(wk[o, i] * x[i] for i in range(D)) for o in range(128)])
    base = O.layer_norm(y, w, b, 1e-6)
    assert np.allclose(k[64:], base[64:], rtol=1e-12, atol=1e-12)          # dims past 64 unrotated
    for j in (0, 5, 31):
        a = pos * invf[j]
        c, s = math.cos(a), math.sin(a)
        assert np.isclose(k[2 * j], base[2 * j] * c - base[2 * j + 1] * s, atol=1e-12)
        assert np.isclose(k[2 * j + 1], base[2 * j] * s + base[2 * j + 1] * c, atol=1e-12)
    # a transposed projection gives a different key
    wk_sq = rng.normal(0, 1, (128, 128))
    xs = rng.normal(0, 1, 128)
    assert not np.allclose(O.index_key(xs, wk_sq, w, b, 1e-6, 0), O.index_key(xs, wk_sq.T, w, b, 1e-6, 0))


def test_latent_row_rotates_only_the_rotary_slice():
    rng = np.random.default_rng(13)
    kv = rng.normal(0, 1, 576)
    invf = workloads.inv_freq_table().numpy().astype(np.float64)
    r = O.latent_row(kv, 1234, invf)
    assert np.array_equal(r[:512], kv[:512])
    pe, rpe = kv[512:].reshape(32, 2), r[512:].reshape(32, 2)
    assert np.allclose(np.linalg.norm(pe, axis=1), np.linalg.norm(rpe, axis=1), rtol=1e-12)
    a = 1234 * invf[3]
    assert np.isclose(r[512 + 6], kv[512 + 6] * math.cos(a) - kv[512 + 7] * math.sin(a), atol=1e-12)
    assert np.array_equal(O.latent_row(kv, 1234, None), kv)                  # NoPE layer: as given
