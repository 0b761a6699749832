"""Comparison helpers shared by the GPU parity tests (no method arithmetic lives here)."""
import math

import numpy as np

# Selection: sets must be equal except for keys whose oracle score lies within this relative
# band of the oracle's k-th score (ties broken toward the lower index elsewhere).
SELECT_BAND = 1e-5
# Attention on fp8 caches with fp32 accumulation: per element |d| <= ATOL + RTOL |ref|, plus a
# relative-RMS bound (outputs are ~1e-3, so the absolute bound alone would pass zeros).
ATOL, RTOL, REL_RMS_FP8 = 2e-2, 1e-2, 1e-2
REL_RMS_F32 = 1e-5


def check_selection(gpu_idx, gpu_len, scores, k, where="", rms_admitted_ok=True):
    """GPU selection vs the oracle's scores: equal size, differences only inside the tie band.

    The band is SELECT_BAND * max(|k-th|, row RMS); the RMS floor covers a k-th score near 0.
    Returns (keys that differ, keys admitted only by the RMS floor).  With
    rms_admitted_ok=False a difference that only the RMS floor admits fails the check."""
    from oracle import dsa_oracle as O
    s = np.asarray(scores, dtype=np.float64)
    n = s.shape[0]
    gi = np.asarray(gpu_idx)
    gl = int(gpu_len)
    assert gl == min(n, k), f"{where}: len {gl} != {min(n, k)}"
    assert np.all(gi[gl:] == -1), f"{where}: padding is not -1"
    sel = gi[:gl]
    assert np.all(np.diff(sel) > 0), f"{where}: selection not strictly ascending"
    if n <= k:
        assert np.array_equal(sel, np.arange(n)), f"{where}: n <= k must select every key"
        return 0, 0
    ref, _ = O.topk_row(s, k)
    kth = O.kth_score(s, k)
    rms = math.sqrt(float(np.mean(s * s)))
    band = SELECT_BAND * max(abs(kth), rms)
    rel_band = SELECT_BAND * abs(kth)
    diff = np.setxor1d(sel, ref)
    outside = [int(t) for t in diff if abs(s[t] - kth) > band]
    assert not outside, (f"{where}: {len(outside)} keys differ outside the band (k-th {kth:.9g}, band {band:.3g}); "
                         f"e.g. {[(t, s[t]) for t in outside[:5]]}")
    rms_only = [int(t) for t in diff if abs(s[t] - kth) > rel_band]
    assert rms_admitted_ok or not rms_only, (
        f"{where}: {len(rms_only)} differing keys lie outside 1e-5 of the k-th score ({kth:.9g}) and are "
        f"admitted only by the RMS floor: {[(t, s[t]) for t in rms_only[:5]]}")
    return len(diff), len(rms_only)


def mla_lse_bound(q, rows, rope_dim, sigma, fp8, kv_lora=512):
    """Bound on |LSE_gpu - LSE_ref| per head from the rounding the kernels do.

    Every logit z_t = sigma * sum_d q_d c_{t,d}.  The fp8 path multiplies q (exact bf16) with
    bf16(code * scale), whose relative rounding error is at most 2^-9 per element, and
    accumulates in fp32; so |dz_t| <= 1.1 * 2^-9 * sigma * sum_d |q_d c_{t,d}| (the 1.1 covers
    the fp32 accumulation, 576 terms at 2^-24 each).  The fp32 path's error is fp32 rounding of
    the same sum: at most 600 * 2^-24 of it.  The LSE moves by at most max_t |dz_t|; the
    exponentials and the log add about 1e-6."""
    q = np.asarray(q, dtype=np.float64)
    rows = np.asarray(rows, dtype=np.float64)
    dq = kv_lora + rope_dim
    if rows.shape[0] == 0:
        return np.zeros(q.shape[0])
    mag = np.abs(q[:, :dq]) @ np.abs(rows[:, :dq]).T          # [G][m]
    u = 1.1 * 2.0 ** -9 if fp8 else 600 * 2.0 ** -24
    return u * sigma * mag.max(axis=1)


def check_attention(out, lse, ref_out, ref_lse, fp8, where="", lse_abs=None):
    """Attention output and LSE against the oracle.  lse_abs (per head, from mla_lse_bound) is
    the absolute LSE bound; without it the LSE must agree to 1e-2 (1e-5 on the fp32 path)
    relative to max(1, |LSE|)."""
    out = np.asarray(out, dtype=np.float64)
    ref_out = np.asarray(ref_out, dtype=np.float64)
    d = np.abs(out - ref_out)
    assert np.all(d <= ATOL + RTOL * np.abs(ref_out)), f"{where}: max abs err {d.max():.3g}"
    rel = np.linalg.norm(out - ref_out) / max(np.linalg.norm(ref_out), 1e-300)
    lim = REL_RMS_FP8 if fp8 else REL_RMS_F32
    assert rel <= lim, f"{where}: rel-RMS {rel:.3g} > {lim}"
    if lse is not None:
        lse = np.asarray(lse, dtype=np.float64)
        ref_lse = np.asarray(ref_lse, dtype=np.float64)
        fin = np.isfinite(ref_lse)
        assert np.array_equal(np.isfinite(lse), fin), f"{where}: lse finiteness differs"
        if fin.any():
            dl = np.abs(lse[fin] - ref_lse[fin])
            if lse_abs is not None:
                lim_h = np.asarray(lse_abs, dtype=np.float64)[fin] + 1e-6 * (1.0 + np.abs(ref_lse[fin]))
                assert np.all(dl <= lim_h), f"{where}: lse err {dl.max():.3g} above its bound {lim_h[np.argmax(dl - lim_h)]:.3g}"
            else:
                lim_lse = 1e-2 if fp8 else 1e-5
                assert dl.max() <= lim_lse * max(1.0, np.abs(ref_lse[fin]).max()), f"{where}: lse err {dl.max():.3g}"
    return rel


def check_block_selection(gpu_idx, gpu_len, scores, pos, block=128, nblocks=16, where=""):
    """Block-sparse selection vs the oracle's scores: the block holding `pos` is kept, the other
    kept blocks may differ from the oracle's only where block maxima lie inside the tie band, and
    the list is every visible key of the kept blocks, ascending, -1 padded."""
    s = np.asarray(scores, dtype=np.float64)[: pos + 1]
    n = pos + 1
    nb = (n + block - 1) // block
    bmax = np.array([s[j * block: min(n, (j + 1) * block)].max() for j in range(nb)])
    gi = np.asarray(gpu_idx)
    gl = int(gpu_len)
    assert np.all(gi[gl:] == -1), f"{where}: padding is not -1"
    chosen = sorted(set(int(x) // block for x in gi[:gl]))
    want = [t for j in chosen for t in range(j * block, min(n, (j + 1) * block))]
    assert gl == len(want) and np.array_equal(gi[:gl], want), f"{where}: not the full ascending key list of its blocks"
    recent = pos // block
    assert recent in chosen, f"{where}: most recent block missing"
    assert len(chosen) == min(nb, nblocks), f"{where}: {len(chosen)} blocks kept"
    if nb <= nblocks:
        return 0
    others = np.array([j for j in range(nb) if j != recent])
    vals = np.sort(bmax[others])[::-1]
    kth = vals[nblocks - 2]
    rms = math.sqrt(float(np.mean(s * s)))
    band = SELECT_BAND * max(abs(kth), rms)
    picked = [j for j in chosen if j != recent]
    bad = [j for j in picked if bmax[j] < kth - band]
    bad += [int(j) for j in others if j not in picked and bmax[j] > kth + band]
    assert not bad, f"{where}: blocks {bad[:5]} disagree with the oracle outside the band"
    from oracle import dsa_oracle as O
    ref, rl = O.block_select_row(s, pos, block, nblocks, topk=len(gi))
    return len(set(chosen) ^ set(int(x) // block for x in ref[:rl]))
