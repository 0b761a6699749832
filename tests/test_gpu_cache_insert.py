"""GPU parity of the cache writers (indexer key path, latent rows) against the float64 oracle.

The codes are integers decided by floating point.  The kernel decides them from its float32
values and scale; the expected code is the oracle's, decided in float64 on its own scale.  Where
the oracle's quotient lies within the kernel's float32 error of a rounding midpoint, either
neighbour is accepted (such cases are counted and bounded).  For values exact in float32 (the
latent groups that are not rotated) that error is only the float32 rounding of the scale and the
quotient.  Scales agree to float32 accuracy.  Rows that are not written keep their bytes.
"""
import zlib

import numpy as np
import pytest
import torch

import workloads
from oracle import dsa_oracle as O

pytestmark = pytest.mark.gpu

SENTINEL = 0x5A


@pytest.fixture(scope="module")
def dsa():
    assert torch.cuda.is_available(), "GPU tests need the MI355X"
    import dsa_sparse_attention_indexer_amd as m
    return m


_MAGS = O.decode_e4m3fn(np.arange(127, dtype=np.uint8))


def check_codes(codes, scale, ref, what, rel_err=2e-6):
    """codes [n] uint8 and scale (kernel) against the float64 values ref [n] of one group.

    The expected code is the oracle's: the nearest E4M3FN value of ref / (max|ref| / 448), in
    float64.  rel_err bounds the kernel's float32 error of ref relative to max|ref| (0 for values
    exact in float32); a code may be the other neighbour only where the oracle's quotient lies
    within the kernel's error of a rounding midpoint: that value error over the scale, the scale's
    own error and the float32 rounding of the quotient.  Returns the number of such cases."""
    amax = float(np.abs(ref).max())
    want_scale = amax / 448.0 if amax > 0 else 1.0
    assert abs(scale - want_scale) <= (4 * rel_err + 2.0 ** -23) * want_scale, (what, scale, want_scale)
    v = np.asarray(ref, dtype=np.float64) / want_scale
    near = O.encode_e4m3fn(v)
    bad = codes != near
    # -0 / +0: both decode to zero
    bad &= ~((codes & 0x7F) == 0) | ~((near & 0x7F) == 0)
    n_band = 0
    if bad.any():
        for i in np.nonzero(bad)[0]:
            a, b = O.decode_e4m3fn(codes[i]), O.decode_e4m3fn(near[i])
            assert np.sign(a) == np.sign(b) or a == 0 or b == 0, (what, i, a, b)
            ia = int(codes[i]) & 0x7F
            ib = int(near[i]) & 0x7F
            assert abs(ia - ib) == 1, (what, i, v[i], a, b)              # a neighbour
            mid = (_MAGS[ia] + _MAGS[ib]) / 2
            band = (rel_err * amax) / want_scale + (4 * rel_err + 2.0 ** -22) * abs(v[i])
            assert abs(abs(v[i]) - mid) <= band, (what, i, v[i], a, b, band)
            n_band += 1
    return n_band


def _fresh_cache(n, width, dev):
    cache = torch.full((n, width), SENTINEL, dtype=torch.uint8, device=dev)
    return cache


def _compact(b, nslots, limit=1 << 20):
    """Far positions: renumber the written slots densely so the cache stays small (the slot is
    only a row number to the writers)."""
    if nslots <= limit:
        return nslots
    uniq = sorted(set(int(s) for s in b.slot.tolist() if s >= 0))
    remap = {s: i for i, s in enumerate(uniq)}
    b.slot = torch.tensor([remap.get(int(s), -1) for s in b.slot.tolist()], dtype=torch.int64)
    return len(uniq) + 3


def _run_key(dsa, b, nslots, x=None):
    dev = "cuda"
    x = b.x.to(dev) if x is None else x
    k_cache = _fresh_cache(nslots, 128, dev)
    k_scale = torch.full((nslots,), -7.0, dtype=torch.float32, device=dev)
    dsa.dsa_index_k_insert(x, b.wk.to(dev), b.ln_w.to(dev), b.ln_b.to(dev), b.pos.to(dev), b.slot.to(dev),
                           k_cache, k_scale, inv_freq=None if b.inv_freq is None else b.inv_freq.to(dev),
                           eps=b.eps)
    torch.cuda.synchronize()
    return k_cache.cpu().numpy(), k_scale.cpu().numpy()


def _check_key_tokens(b, kc, ks, tokens, nslots):
    invf = None if b.inv_freq is None else b.inv_freq.numpy()
    written = set()
    n_band = 0
    for t in tokens:
        sl = int(b.slot[t])
        if sl < 0 or sl >= nslots:
            continue
        written.add(sl)
        ref = O.index_key(b.x[t], b.wk, b.ln_w, b.ln_b, b.eps, int(b.pos[t]), invf)
        n_band += check_codes(kc[sl], float(ks[sl]), ref, f"{b.name} token {t}")
    return written, n_band


KEY_CASES = [
    # name, positions, seqs, num_seqs, max_ctx, hidden, rope, skip
    ("ragged_one_tile_rope", list(range(100, 137)), [0] * 37, 1, 400, 6144, True, ()),
    ("three_tiles_nope_two_seqs", [5 * i for i in range(75)] * 2, [0] * 75 + [1] * 75, 2, 400, 6144, False, (3, 80)),
    ("small_hidden_one_step", list(range(70)), [0] * 70, 1, 80, 32, True, ()),
    ("hidden_96_odd_steps", list(range(0, 130, 2)), [0] * 65, 1, 200, 96, True, (0,)),
    ("hidden_4160", [1 << 20] * 3 + [7, 9], [0, 1, 2, 3, 3], 4, (1 << 20) + 1, 4160, True, ()),
    ("single_token", [5], [0], 1, 10, 6144, True, ()),
    ("tile_plus_one_nope", list(range(65)), [0] * 65, 1, 70, 6144, False, (64,)),
]


@pytest.mark.parametrize("case", KEY_CASES, ids=[c[0] for c in KEY_CASES])
def test_index_k_insert_matches_oracle(dsa, case):
    name, pos, seqs, B, max_ctx, hidden, rope, skip = case
    b = workloads.make_insert_batch(name=name, seed=zlib.crc32(name.encode()) % 1000, positions=pos, seqs=seqs, num_seqs=B,
                                    max_ctx=max_ctx, hidden=hidden, rope=rope, skip=skip)
    nslots = _compact(b, B * max_ctx)
    print(f"case {name}: T={b.num_tokens} hidden={hidden} rope={rope} slots={nslots}", flush=True)
    kc, ks = _run_key(dsa, b, nslots)
    written, n_band = _check_key_tokens(b, kc, ks, range(b.num_tokens), nslots)
    untouched = np.array([i for i in range(nslots) if i not in written])
    assert np.all(kc[untouched] == SENTINEL) and np.all(ks[untouched] == -7.0)
    assert n_band <= max(2, b.num_tokens * 128 // 2000), n_band


def test_index_k_insert_out_of_range_slot_is_skipped_and_strided_x(dsa):
    b = workloads.make_insert_batch(name="oob", seed=31, positions=list(range(40)), seqs=[0] * 40, num_seqs=1,
                                    max_ctx=40, hidden=6144)
    b.slot[7] = 40            # == num_slots: skipped
    b.slot[8] = 1 << 40       # far out: skipped
    wide = torch.zeros((40, 6144 + 64), dtype=torch.bfloat16)
    wide[:, :6144] = b.x
    x = wide.to("cuda")[:, :6144]          # row stride 6208 elements
    kc, ks = _run_key(dsa, b, 40, x=x)
    written, _ = _check_key_tokens(b, kc, ks, range(40), 40)
    assert 7 not in written and np.all(kc[7] == SENTINEL) and ks[7] == -7.0


@pytest.mark.parametrize("shape", ["decode_b16_ctx131072", "prefill_4096_on_61440"])
def test_index_k_insert_full_size(dsa, shape):
    b = workloads.insert_decode() if shape.startswith("decode") else workloads.insert_prefill()
    nslots = b.num_seqs * b.max_ctx   # the readers' full layout, as the benchmark writes it
    print(f"case {shape}: T={b.num_tokens} slots={nslots}", flush=True)
    kc, ks = _run_key(dsa, b, nslots)
    T = b.num_tokens
    sample = sorted(set([0, 1, T - 1] + list(range(0, T, max(1, T // 40)))))
    written, n_band = _check_key_tokens(b, kc, ks, sample, nslots)
    assert n_band <= 3
    # every token's row was written (not left at the sentinel scale) and nothing else was
    slots = b.slot.numpy()
    assert np.all(ks[slots] > 0)
    mask = np.ones(nslots, dtype=bool)
    mask[slots] = False
    assert np.all(ks[mask] == -7.0)


LATENT_CASES = [
    ("rope_ragged", list(range(300, 337)), [0] * 37, 1, 400, True, ()),
    ("nope_two_seqs_skip", list(range(90)) * 2, [0] * 90 + [1] * 90, 2, 100, False, (4, 95)),
    ("rope_decode_b16", [131071] * 16, list(range(16)), 16, 131072, True, ()),
    ("single_token_far", [(1 << 26) - 1], [0], 1, 1 << 26, True, ()),
]


@pytest.mark.parametrize("case", LATENT_CASES, ids=[c[0] for c in LATENT_CASES])
def test_latent_insert_matches_oracle(dsa, case):
    name, pos, seqs, B, max_ctx, rope, skip = case
    b = workloads.make_insert_batch(name=name, seed=zlib.crc32(name.encode()) % 1000 + 7, positions=pos, seqs=seqs, num_seqs=B,
                                    max_ctx=max_ctx, hidden=32, rope=rope, skip=skip)
    nslots = _compact(b, B * max_ctx)
    print(f"case latent {name}: T={b.num_tokens} slots={nslots}", flush=True)
    dev = "cuda"
    kv_cache = _fresh_cache(nslots, 576, dev)
    kv_scale = torch.full((nslots, 9), -7.0, dtype=torch.float32, device=dev)
    dsa.dsa_latent_insert(b.kv.to(dev), b.pos.to(dev), b.slot.to(dev), kv_cache, kv_scale,
                          inv_freq=None if b.inv_freq is None else b.inv_freq.to(dev))
    torch.cuda.synchronize()
    kc, ks = kv_cache.cpu().numpy(), kv_scale.cpu().numpy()
    invf = None if b.inv_freq is None else b.inv_freq.numpy()
    written = set()
    n_band = 0
    for t in range(b.num_tokens):
        sl = int(b.slot[t])
        if sl < 0:
            continue
        written.add(sl)
        ref = O.latent_row(b.kv[t], int(b.pos[t]), invf)
        for g in range(9):
            rotated = g == 8 and rope
            # the latent groups are bf16 values, exact in float32: their only error is the float32
            # rounding of the scale and the quotient; the rotated group also carries the rotation's
            nb = check_codes(kc[sl, 64 * g:64 * g + 64], float(ks[sl, g]), ref[64 * g:64 * g + 64],
                             f"{name} token {t} group {g}", rel_err=1e-6 if rotated else 0.0)
            n_band += nb
    assert n_band <= max(2, b.num_tokens // 4), n_band
    rows = np.array(sorted(written))
    mask = np.ones(nslots, dtype=bool)
    mask[rows] = False
    assert np.all(ks[mask] == -7.0) and np.all(kc[mask] == SENTINEL)


def test_written_caches_feed_the_readers(dsa):
    """Keys and latents written by the writers are what the score and attention kernels read:
    scoring the written cache on the GPU matches the oracle scoring the same bytes."""
    B, L = 2, 3000
    pos = list(range(L)) * B
    seqs = [0] * L + [1] * L
    b = workloads.make_insert_batch(name="feed", seed=40, positions=pos, seqs=seqs, num_seqs=B, max_ctx=L,
                                    hidden=256, rope=True)
    dev = "cuda"
    k_cache = torch.zeros((B, L, 128), dtype=torch.uint8, device=dev)
    k_scale = torch.zeros((B, L), dtype=torch.float32, device=dev)
    dsa.dsa_index_k_insert(b.x.to(dev), b.wk.to(dev), b.ln_w.to(dev), b.ln_b.to(dev), b.pos.to(dev),
                           b.slot.to(dev), k_cache, k_scale, inv_freq=b.inv_freq.to(dev), eps=b.eps)
    wl = workloads.make_workload(name="feed_q", seed=41, seq_lens=[L, L - 500], max_ctx=L)
    wl.index_k, wl.index_k_scale = k_cache.cpu(), k_scale.cpu()
    scores = torch.full((wl.num_q, L), float("nan"), dtype=torch.float32, device=dev)
    g = wl.to(dev)
    dsa.dsa_indexer_scores(g.index_q, g.index_w, g.q_seq, g.q_pos, g.index_k, scores, k_scale=g.index_k_scale,
                           ssmax_s=g.ssmax_s, ssmax_b=g.ssmax_b, inv_freq=g.inv_freq)
    torch.cuda.synchronize()
    s = scores.cpu().numpy()
    for t in range(wl.num_q):
        ref = O.index_scores(wl, t)
        n = ref.shape[0]
        tol = 2e-6 * np.sqrt(np.mean(ref * ref)) + 2e-6 * np.abs(ref)
        assert np.all(np.abs(s[t, :n] - ref) <= tol)
