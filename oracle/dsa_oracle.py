"""Plain, slow CPU oracle for the DSA decode / prefill path, in float64.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU-baseline
leg of the benchmark may import this module.  The product path (the HIP library and
its Python binding) never imports, calls or falls back to it, and it shares no code,
table or constant generator with that path: it decodes the fp8 / bf16 bytes itself
and follows the definitions below with numpy, one query at a time.

What it computes, and where the pages say so:

* Lightning-indexer query prep -- "mistral-large4.md" (colibri), section
  "What differs from GLM-5.2", bullets "SSMax", "The indexer" and "RoPE and the rest":
  the index query is rotated on its first 64 dims on RoPE layers, in interleaved pairs
  (2j, 2j+1), and every head's query is multiplied by s*log(position+1)+b with that
  head's own s and b.  The log is natural, the position is the query token's 0-based
  absolute position, and the rotation angle is position * inv_freq[j].
* Index scores -- same page and bullet: each cached key t gets
  S(t) = sum_h (w_h / sqrt(H)) * relu(q'_h . k_t / sqrt(128)), with H = 32 index heads
  on Mistral Large 4 (the page divides by sqrt(32)).  Keys are read from the fp8 cache
  as code * per-token fp32 scale ("Day 0 support for Mistral Large 4 on vLLM",
  "ROCm implementation details", "DSA indexer on AITER": FP8 keys with one scale).
* Top-k -- the 2048 highest scores per query are kept (same pages; "Highlights" and the
  architecture table).  Ties go to the lower key index; a query that sees n <= k keys
  takes all of them; the selection is emitted ascending and padded with -1 up to k,
  with its length reported separately (the -1 slots and the top-k length bound of the
  "Top-k compaction" bullet in "Long context: decode and prefill context parallelism").
* Sparse MLA -- absorbed multi-head latent attention over the selected keys only:
  per head g, z_t = sigma * (q_g[:512] . c_t[:512] + q_g[512:] . c_t[512:576]),
  P = softmax(z), O_g = sum_t P_t c_t[:512] (V is the latent), LSE_g = log sum exp z.
  NoPE layers are MLA with zero rope dims on the same cache layout ("NoPE, SSMax and
  LeRoPE" on the vLLM page; "NoPE layers" bullet on the colibri page).
* Cache writers -- the indexer key of a token is k = LayerNorm(wk(x)), rotated on its
  first 64 dims on RoPE layers ("mistral-large4.md", "What differs from GLM-5.2", bullet
  "The indexer"), quantised to FP8 with one scale per token and written into the index
  cache ("Day 0 support for Mistral Large 4 on vLLM", "ROCm implementation details",
  "DSA indexer on AITER": 132 bytes per token, one layout shared by writer and readers).
  A latent row (512 latent + 64 rotary dims, "Model architecture") has its rotary slice
  rotated at the token's position and is stored as FP8 with one scale per 64 elements.
  The quantiser is scale = amax / 448 (1 for an all-zero group) and code = the nearest
  E4M3FN value of x / scale, ties to the even code, saturated at +-448.
* Block-sparse selection -- "vLLM adds NVFP4 serving for MiniMax M3.1 Flash at 76
  concurrent sequences", the three MiniMax Sparse Attention steps: 128-token blocks,
  16 blocks selected with the most recent block always kept, exact attention over the
  selected keys.  The block score is the maximum index score over the block's visible
  keys.

Every function works on float64 copies of its inputs.  Sorting and matrix products use
numpy's own routines; nothing is blocked, fused or reordered beyond the definitions.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

# ----------------------------------------------------------------------------------------------
# Storage formats
# ----------------------------------------------------------------------------------------------


def decode_e4m3fn(codes) -> np.ndarray:
    """OCP FP8 E4M3FN: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits.

    Exponent field 0 is subnormal (m * 2^-9); S.1111.111 is NaN; there are no infinities;
    the largest finite magnitude is 1.75 * 2^8 = 448.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64))
    sub = m * 2.0 ** -9
    v = np.where(e == 0, sub, normal)
    v = np.where((e == 15) & (m == 7), np.nan, v)
    return sign * v


def encode_e4m3fn(v) -> np.ndarray:
    """Nearest E4M3FN code of each value: ties go to the even code (even mantissa), magnitudes
    above 448 saturate to 448, the sign is kept (also for zero), NaN gives 0x7F.

    The candidates are the 127 finite non-negative magnitudes of decode_e4m3fn, in code order
    (which is increasing magnitude).
    """
    v = np.asarray(v, dtype=np.float64)
    mags = decode_e4m3fn(np.arange(127, dtype=np.uint8))      # codes 0x00..0x7E
    a = np.minimum(np.abs(v), 448.0)
    hi = np.clip(np.searchsorted(mags, a, side="left"), 0, 126)  # mags[hi] >= a
    lo = np.maximum(hi - 1, 0)
    d_lo = a - mags[lo]
    d_hi = mags[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(np.signbit(v), code | 0x80, code).astype(np.uint8)
    return np.where(np.isnan(v), np.uint8(0x7F), code).astype(np.uint8)


def quantize_e4m3_rows(x, block: int):
    """Codes and scales of the rows of x, one scale per `block` elements along the last dim.

    scale = amax / 448 (1 where amax is 0); code = encode_e4m3fn(x / scale), everything in
    float64.  Returns (uint8 codes, float64 scales).
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    assert d % block == 0
    xb = x.reshape(*x.shape[:-1], d // block, block)
    amax = np.abs(xb).max(axis=-1)
    scale = np.where(amax > 0, amax / 448.0, 1.0)
    return encode_e4m3fn(xb / scale[..., None]).reshape(x.shape), scale


def decode_bf16(bits) -> np.ndarray:
    """bfloat16 is the top half of an IEEE binary32: widen the bits and reinterpret."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def to_f64(x) -> np.ndarray:
    """Float64 view of a query / cache tensor given as float32 values or bf16 bit patterns.

    Accepts numpy arrays or torch CPU tensors.  bf16 torch tensors are decoded from their
    raw bits by decode_bf16, so torch's own conversion is never used on the values.
    """
    try:
        import torch  # noqa: F401  (only to recognise torch tensors)
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu()
            if x.dtype == torch.bfloat16:
                return decode_bf16(x.view(torch.int16).numpy().view(np.uint16))
            x = x.numpy()
    except ImportError:  # pragma: no cover
        pass
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return decode_bf16(x)
    return x.astype(np.float64)


def dequant_rows(codes, scales, block: int) -> np.ndarray:
    """Cached value = decoded E4M3FN code x the fp32 scale of its `block`-element group."""
    v = decode_e4m3fn(codes)
    s = np.asarray(scales, dtype=np.float64)
    d = v.shape[-1]
    assert d % block == 0 and s.shape[-1] == d // block
    return (v.reshape(*v.shape[:-1], d // block, block) * s[..., None]).reshape(v.shape)


# ----------------------------------------------------------------------------------------------
# Index query prep: interleaved RoPE, then SSMax
# ----------------------------------------------------------------------------------------------


def rope_interleaved(x: np.ndarray, angles: np.ndarray) -> np.ndarray:
    """Rotate pairs (2j, 2j+1) of the last dim by angles[j]; dims past 2*len(angles) untouched.

    x'_{2j}   = x_{2j} cos a_j - x_{2j+1} sin a_j
    x'_{2j+1} = x_{2j} sin a_j + x_{2j+1} cos a_j
    """
    x = np.array(x, dtype=np.float64, copy=True)
    a = np.asarray(angles, dtype=np.float64)
    r = 2 * a.shape[-1]
    ev = x[..., 0:r:2].copy()
    od = x[..., 1:r:2].copy()
    c, s = np.cos(a), np.sin(a)
    x[..., 0:r:2] = ev * c - od * s
    x[..., 1:r:2] = ev * s + od * c
    return x


def rope_angles(pos: int, inv_freq) -> np.ndarray:
    """Angle of pair j at absolute position pos: pos * inv_freq[j], formed in float64."""
    return float(pos) * np.asarray(inv_freq, dtype=np.float64)


def ssmax_multiplier(s, b, pos: int) -> np.ndarray:
    """SSMax query multiplier s * ln(pos + 1) + b, per head."""
    return np.asarray(s, dtype=np.float64) * math.log(pos + 1.0) + np.asarray(b, dtype=np.float64)


def index_query(q_heads, pos: int, ssmax_s=None, ssmax_b=None, inv_freq=None) -> np.ndarray:
    """q' for one query token: RoPE on the first 2*len(inv_freq) dims (if given), then x m_h."""
    q = to_f64(q_heads)
    if inv_freq is not None:
        q = rope_interleaved(q, rope_angles(pos, inv_freq))
    if ssmax_s is not None:
        q = q * ssmax_multiplier(ssmax_s, ssmax_b, pos)[:, None]
    return q


# ----------------------------------------------------------------------------------------------
# Index scores
# ----------------------------------------------------------------------------------------------


def index_scores_row(qp: np.ndarray, w, keys: np.ndarray) -> np.ndarray:
    """S(t) = sum_h (w_h / sqrt(H)) relu(q'_h . k_t / sqrt(D)) for every row k_t of `keys`."""
    qp = np.asarray(qp, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    H, D = qp.shape
    dots = qp @ np.asarray(keys, dtype=np.float64).T          # [H][n]
    head = np.maximum(dots / math.sqrt(D), 0.0)
    return (w / math.sqrt(H)) @ head                          # [n]


def cache_keys(wl, seq: int, n: int) -> np.ndarray:
    """The first n cached index keys of sequence `seq` as float64 values."""
    k = wl.index_k[seq, :n]
    if wl.index_k_scale is None:
        return to_f64(k)
    codes = k.cpu().numpy() if hasattr(k, "cpu") else np.asarray(k)
    sc = wl.index_k_scale[seq, :n]
    sc = sc.cpu().numpy() if hasattr(sc, "cpu") else np.asarray(sc)
    return decode_e4m3fn(codes) * sc.astype(np.float64)[:, None]


def index_scores(wl, query: int) -> np.ndarray:
    """Scores of every key visible to query `query` (positions 0..q_pos) of workload `wl`."""
    p = int(wl.q_pos[query])
    b = int(wl.q_seq[query])
    qp = index_query(wl.index_q[query], p,
                     None if wl.ssmax_s is None else to_f64(wl.ssmax_s),
                     None if wl.ssmax_b is None else to_f64(wl.ssmax_b),
                     None if wl.inv_freq is None else to_f64(wl.inv_freq))
    return index_scores_row(qp, to_f64(wl.index_w[query]), cache_keys(wl, b, p + 1))


# ----------------------------------------------------------------------------------------------
# Selection
# ----------------------------------------------------------------------------------------------


def topk_row(scores, k: int):
    """Keep the k highest scores; ties to the lower index; ascending, -1 padded; returns (idx, len)."""
    s = np.asarray(scores, dtype=np.float64)
    n = s.shape[0]
    out = np.full(k, -1, dtype=np.int32)
    if n <= k:
        out[:n] = np.arange(n, dtype=np.int32)
        return out, n
    t = np.arange(n)
    order = np.lexsort((t, -s))          # primary: score descending; secondary: index ascending
    keep = np.sort(order[:k])
    out[:] = keep.astype(np.int32)
    return out, k


def kth_score(scores, k: int) -> Optional[float]:
    """The k-th highest score (None when there are at most k scores)."""
    s = np.asarray(scores, dtype=np.float64)
    if s.shape[0] <= k:
        return None
    return float(-np.sort(-s, kind="stable")[k - 1])


def block_select_row(scores, pos: int, block: int = 128, nblocks: int = 16, topk: int = 2048):
    """Block-sparse selection over the visible keys 0..pos.

    Block j's score is the max of its visible keys' scores.  The block holding `pos` (the most
    recent one, possibly partial) is always kept; the other nblocks-1 come from the rest by
    (score desc, block asc).  The selection is every visible key of the kept blocks, ascending,
    -1 padded to `topk`.
    """
    s = np.asarray(scores, dtype=np.float64)[: pos + 1]
    n = pos + 1
    nb = (n + block - 1) // block
    bmax = np.array([s[j * block: min(n, (j + 1) * block)].max() for j in range(nb)])
    recent = pos // block
    if nb <= nblocks:
        chosen = list(range(nb))
    else:
        others = [j for j in range(nb) if j != recent]
        others.sort(key=lambda j: (-bmax[j], j))
        chosen = sorted(others[: nblocks - 1] + [recent])
    idx = [t for j in chosen for t in range(j * block, min(n, (j + 1) * block))]
    out = np.full(topk, -1, dtype=np.int32)
    assert len(idx) <= topk
    out[: len(idx)] = idx
    return out, len(idx)


# ----------------------------------------------------------------------------------------------
# Sparse MLA (absorbed form, V = latent)
# ----------------------------------------------------------------------------------------------


def cache_rows(wl, seq: int, rows) -> np.ndarray:
    """Selected latent rows of sequence `seq` as float64 [m][576]."""
    rows = np.asarray(rows, dtype=np.int64)
    if wl.kv_scale is None:
        return to_f64(wl.kv[seq][rows])
    codes = wl.kv[seq].cpu().numpy()[rows] if hasattr(wl.kv, "cpu") else np.asarray(wl.kv[seq])[rows]
    sc = wl.kv_scale[seq].cpu().numpy()[rows] if hasattr(wl.kv_scale, "cpu") else np.asarray(wl.kv_scale[seq])[rows]
    return dequant_rows(codes, sc, 64)


def mla_attend(q, rows: np.ndarray, rope_dim: int, sigma: float, kv_lora: int = 512):
    """Exact attention of every head of q [G][kv_lora+rope_dim] over the latent rows [m][576].

    Returns (O [G][kv_lora], LSE [G]).  With no rows, O = 0 and LSE = -inf.
    """
    q = to_f64(q)
    rows = np.asarray(rows, dtype=np.float64)
    G = q.shape[0]
    if rows.shape[0] == 0:
        return np.zeros((G, kv_lora)), np.full(G, -np.inf)
    z = q[:, :kv_lora] @ rows[:, :kv_lora].T
    if rope_dim:
        z = z + q[:, kv_lora:kv_lora + rope_dim] @ rows[:, kv_lora:kv_lora + rope_dim].T
    z = sigma * z                                         # [G][m]
    zmax = z.max(axis=1, keepdims=True)
    e = np.exp(z - zmax)
    l = e.sum(axis=1, keepdims=True)
    out = (e / l) @ rows[:, :kv_lora]
    lse = zmax[:, 0] + np.log(l[:, 0])
    return out, lse


def sparse_mla_row(wl, query: int, idx, length: Optional[int] = None):
    """Sparse MLA for one query over idx[:length] (the -1 slots beyond are ignored)."""
    idx = np.asarray(idx, dtype=np.int64)
    if length is None:
        length = int((idx >= 0).sum())
    sel = idx[:length]
    rows = cache_rows(wl, int(wl.q_seq[query]), sel)
    return mla_attend(wl.mla_q[query], rows, wl.rope_dim, wl.softmax_scale)


def dense_mla_row(wl, query: int):
    """Dense MLA over every visible key 0..q_pos, computed without any index list."""
    p = int(wl.q_pos[query])
    rows = cache_rows(wl, int(wl.q_seq[query]), np.arange(p + 1))
    return mla_attend(wl.mla_q[query], rows, wl.rope_dim, wl.softmax_scale)


# ----------------------------------------------------------------------------------------------
# Cache writers: the indexer key path and latent rows
# ----------------------------------------------------------------------------------------------


def layer_norm(y, weight, bias, eps: float) -> np.ndarray:
    """LayerNorm over the last dim: (y - mean) / sqrt(var + eps) * weight + bias, with the
    population variance (mean of squared deviations)."""
    y = np.asarray(y, dtype=np.float64)
    mu = y.mean(axis=-1, keepdims=True)
    var = ((y - mu) ** 2).mean(axis=-1, keepdims=True)
    out = (y - mu) / np.sqrt(var + eps) * to_f64(weight)
    return out + (0.0 if bias is None else to_f64(bias))


def index_key(x, wk, ln_w, ln_b, eps: float, pos: int, inv_freq=None) -> np.ndarray:
    """Indexer key of one token before quantisation: LayerNorm(wk(x)), then RoPE on the first
    2*len(inv_freq) dims at the token's position (no rotation when inv_freq is None).

    x [D] (the token's hidden state), wk [128][D] (the projection's weight: output dim first).
    """
    y = to_f64(wk) @ to_f64(x)
    k = layer_norm(y, ln_w, ln_b, eps)
    if inv_freq is not None:
        k = rope_interleaved(k, rope_angles(pos, inv_freq))
    return k


def latent_row(kv, pos: int, inv_freq=None, kv_lora: int = 512) -> np.ndarray:
    """A latent cache row before quantisation: the 512 latent dims as given, the rotary slice
    (dims 512..575) rotated at the token's position (unrotated when inv_freq is None)."""
    r = np.array(to_f64(kv), copy=True)
    if inv_freq is not None:
        r[kv_lora:] = rope_interleaved(r[kv_lora:], rope_angles(pos, inv_freq))
    return r


# ----------------------------------------------------------------------------------------------
# One layer step for a set of queries
# ----------------------------------------------------------------------------------------------


def decode_layer(wl, queries: Sequence[int], topk: Optional[int] = None, block_sparse: bool = False,
                 idx_override=None):
    """Scores -> selection -> sparse MLA for the listed queries.

    idx_override: a shared-indexer layer reuses another layer's selection ([T][k], lengths) and
    skips scoring.  Returns dict(scores=list, idx=[q][k], len=[q], out=[q][G][512], lse=[q][G]).
    """
    k = wl.topk if topk is None else topk
    res = dict(scores=[], idx=[], len=[], out=[], lse=[])
    for i, t in enumerate(queries):
        if idx_override is not None:
            idx, n = idx_override[0][i], int(idx_override[1][i])
            s = None
        else:
            s = index_scores(wl, t)
            if block_sparse:
                idx, n = block_select_row(s, int(wl.q_pos[t]), topk=k)
            else:
                idx, n = topk_row(s, k)
        o, l = sparse_mla_row(wl, t, idx, n)
        res["scores"].append(s)
        res["idx"].append(np.asarray(idx))
        res["len"].append(n)
        res["out"].append(o)
        res["lse"].append(l)
    return res
