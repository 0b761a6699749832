"""Python binding of libdsa, the MI355X (gfx950) DSA hot path: lightning-indexer scores, top-k /
block selection and sparse absorbed-MLA attention.

Every function here only marshals arguments: it checks tensor dtypes, shapes, devices and
contiguity, passes raw device pointers and the current HIP stream to the C ABI in
``include/dsa.h`` and raises on a non-OK status with the library's error text.  All arithmetic
runs in the library's HIP kernels.  There is no CPU or PyTorch fallback: if ``libdsa.so`` is
missing, importing this package raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa.so")

DSA_OK, DSA_ERR_ARG, DSA_ERR_UNSUPPORTED, DSA_ERR_HIP = 0, 1, 2, 3
DSA_F32, DSA_BF16, DSA_FP8_E4M3FN = 0, 1, 2
ABI_VERSION = 3


class DsaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"[status {status}] {msg}")
        self.status = status


class IndexerDesc(ctypes.Structure):
    _fields_ = [("num_q", ctypes.c_int32), ("num_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("rope_dim", ctypes.c_int32), ("num_seqs", ctypes.c_int32), ("max_ctx", ctypes.c_int32),
                ("q_dtype", ctypes.c_int32), ("k_dtype", ctypes.c_int32)]


class MlaDesc(ctypes.Structure):
    _fields_ = [("num_q", ctypes.c_int32), ("num_heads", ctypes.c_int32), ("kv_lora", ctypes.c_int32),
                ("rope_dim", ctypes.c_int32), ("num_seqs", ctypes.c_int32), ("max_ctx", ctypes.c_int32),
                ("topk", ctypes.c_int32), ("q_dtype", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
                ("kv_scale_block", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
                ("num_splits", ctypes.c_int32)]


class PagingDesc(ctypes.Structure):
    _fields_ = [("block_table", ctypes.c_void_p), ("page_size", ctypes.c_int32), ("blocks_per_seq", ctypes.c_int32),
                ("num_blocks", ctypes.c_int32), ("num_seqs", ctypes.c_int32)]


class IndexKDesc(ctypes.Structure):
    _fields_ = [("num_tokens", ctypes.c_int32), ("hidden", ctypes.c_int32), ("ld_x", ctypes.c_int64),
                ("rope_dim", ctypes.c_int32), ("eps", ctypes.c_float), ("num_slots", ctypes.c_int64)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python dsa_sparse_attention_indexer_amd/build.py` "
                          "(there is no fallback path)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    PG = ctypes.POINTER(PagingDesc)
    sig = {
        "dsa_last_error": (ctypes.c_char_p, []),
        "dsa_abi_version": (I32, []),
        "dsa_timing_begin": (I32, [P, I32]),
        "dsa_timing_end": (I32, []),
        "dsa_timing_kernel_name": (ctypes.c_char_p, [I32]),
        "dsa_indexer_workspace_size": (SZ, [ctypes.POINTER(IndexerDesc)]),
        "dsa_indexer_scores": (I32, [ctypes.POINTER(IndexerDesc), P, P, P, P, P, P, P, P, P, P, I64, P, SZ, P, PG]),
        "dsa_indexer_topk": (I32, [ctypes.POINTER(IndexerDesc), P, P, P, P, P, P, P, P, P, P, I64, I32, P, P, P, SZ,
                                   P, SZ, P, PG]),
        "dsa_indexer_scores_hist": (I32, [ctypes.POINTER(IndexerDesc), P, P, P, P, P, P, P, P, P, P, I64, I32, P, SZ,
                                          P, SZ, P, PG]),
        "dsa_topk_hist": (I32, [ctypes.POINTER(IndexerDesc), P, I64, P, I32, P, P, P, SZ, P]),
        "dsa_topk_workspace_size": (SZ, [I32, I64, I32]),
        "dsa_topk": (I32, [P, I64, P, I32, I32, P, P, P, SZ, P]),
        "dsa_block_select_workspace_size": (SZ, [I32, I64, I32]),
        "dsa_block_select": (I32, [P, I64, P, I32, I32, I32, I32, P, P, P, SZ, P]),
        "dsa_indexer_block_select": (I32, [ctypes.POINTER(IndexerDesc), P, P, P, P, P, P, P, P, P, P, I64, I32, I32,
                                           I32, P, P, P, SZ, P, SZ, P, PG]),
        "dsa_sparse_mla_workspace_size": (SZ, [ctypes.POINTER(MlaDesc)]),
        "dsa_sparse_mla_decode": (I32, [ctypes.POINTER(MlaDesc), P, P, P, P, P, P, P, P, P, SZ, P, PG]),
        "dsa_sparse_mla_prefill": (I32, [ctypes.POINTER(MlaDesc), P, P, P, P, P, P, P, P, P, SZ, P, PG]),
        "dsa_sparse_mla_noalloc_max_bytes": (SZ, []),
        "dsa_sparse_mla_decode_noalloc": (I32, [ctypes.POINTER(MlaDesc), P, P, P, P, P, P, P, P, P, PG]),
        "dsa_index_k_insert_workspace_size": (SZ, [ctypes.POINTER(IndexKDesc)]),
        "dsa_index_k_insert": (I32, [ctypes.POINTER(IndexKDesc), P, P, P, P, P, P, P, P, P, P, SZ, P, PG]),
        "dsa_paged_slots": (I32, [PG, I32, P, P, P, P]),
        "dsa_latent_insert": (I32, [I32, I32, P, I64, P, P, P, I64, P, P, P]),
    }
    for name, (res, args) in sig.items():
        if not hasattr(lib, name):
            raise ImportError(f"{LIB_PATH} does not export {name}: it is stale, rebuild it")
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    if lib.dsa_abi_version() != ABI_VERSION:
        raise ImportError(f"libdsa ABI version {lib.dsa_abi_version()} != {ABI_VERSION}")
    return lib


_lib = _load()
EXPORTED = ["dsa_last_error", "dsa_abi_version", "dsa_indexer_workspace_size", "dsa_indexer_scores", "dsa_indexer_topk",
            "dsa_indexer_scores_hist", "dsa_topk_hist",
            "dsa_topk_workspace_size", "dsa_topk", "dsa_block_select_workspace_size", "dsa_block_select", "dsa_sparse_mla_workspace_size",
            "dsa_sparse_mla_decode", "dsa_sparse_mla_prefill", "dsa_sparse_mla_noalloc_max_bytes",
            "dsa_sparse_mla_decode_noalloc", "dsa_index_k_insert_workspace_size",
            "dsa_index_k_insert", "dsa_latent_insert", "dsa_timing_begin", "dsa_timing_end",
            "dsa_timing_kernel_name", "dsa_paged_slots", "dsa_indexer_block_select"]


def lib():
    return _lib


def _check(status: int):
    if status != DSA_OK:
        raise DsaError(status, _lib.dsa_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(name, t, dtype=None, shape=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


class Paging:
    """A paged cache layout (the header's "Paged caches"): block_table [num_seqs][blocks_per_seq]
    i32 on the GPU, page_size tokens per block, num_blocks blocks in the pool, and max_ctx, the
    longest sequence the table describes (at most blocks_per_seq * page_size)."""

    def __init__(self, block_table: torch.Tensor, page_size: int, num_blocks: int, max_ctx: int):
        _dev("block_table", block_table, torch.int32)
        if block_table.dim() != 2:
            raise ValueError("block_table must be [num_seqs][blocks_per_seq]")
        self.block_table, self.page_size, self.num_blocks = block_table, int(page_size), int(num_blocks)
        self.num_seqs, self.blocks_per_seq = int(block_table.shape[0]), int(block_table.shape[1])
        self.max_ctx = int(max_ctx)
        self.desc = PagingDesc(block_table.data_ptr(), self.page_size, self.blocks_per_seq, self.num_blocks,
                               self.num_seqs)

    @property
    def pool_rows(self) -> int:
        return self.num_blocks * self.page_size


def _pg(paging):
    return None if paging is None else ctypes.byref(paging.desc)


def _seq_dims(cache, paging):
    """(num_seqs, max_ctx) of a contiguous cache [B][max_ctx][row], or of a paged one."""
    if paging is None:
        return int(cache.shape[0]), int(cache.shape[1])
    if cache.shape[0] * (cache.shape[1] if cache.dim() == 3 else 1) != paging.pool_rows:
        raise ValueError("a paged cache must hold num_blocks * page_size rows")
    return paging.num_seqs, paging.max_ctx


def _rows_of(cache, paging):
    return cache.shape[:2] if paging is None else (paging.pool_rows,)


def _qdtype(t):
    return {torch.float32: DSA_F32, torch.bfloat16: DSA_BF16}[t.dtype]


def _kdtype(t):
    return {torch.float32: DSA_F32, torch.uint8: DSA_FP8_E4M3FN, torch.float8_e4m3fn: DSA_FP8_E4M3FN}[t.dtype]


# ------------------------------------------------------------------------------------------------
# 1. indexer scores
# ------------------------------------------------------------------------------------------------

def dsa_indexer_workspace_size(desc: IndexerDesc) -> int:
    return int(_lib.dsa_indexer_workspace_size(ctypes.byref(desc)))


def indexer_desc(q, k_cache, inv_freq=None, paging=None) -> IndexerDesc:
    T, H, D = q.shape
    B, max_ctx = _seq_dims(k_cache, paging)
    rope = 0 if inv_freq is None else 2 * int(inv_freq.numel())
    return IndexerDesc(T, H, D, rope, B, max_ctx, _qdtype(q), _kdtype(k_cache))


def dsa_indexer_scores(q, w, q_seq, q_pos, k_cache, scores, k_scale=None, ssmax_s=None, ssmax_b=None,
                       inv_freq=None, ws=None, stream=None, paging=None):
    """Fills scores[t, 0..q_pos[t]] with the lightning-indexer score of every visible key.

    q [T][H][128] f32|bf16, w [T][H] f32, q_seq/q_pos [T] i32, k_cache [B][max_ctx][128] f32 or
    fp8 bytes (uint8 / float8_e4m3fn), k_scale [B][max_ctx] f32 (fp8 only), ssmax_s/b [H] f32,
    inv_freq [32] f32 on RoPE layers (None on NoPE layers), scores [T][ld] f32 with ld >= max_ctx.
    """
    T, H, D = q.shape
    B, max_ctx = _seq_dims(k_cache, paging)
    _dev("q", q, (torch.float32, torch.bfloat16))
    _dev("w", w, torch.float32, (T, H))
    _dev("q_seq", q_seq, torch.int32, (T,))
    _dev("q_pos", q_pos, torch.int32, (T,))
    _dev("k_cache", k_cache, (torch.float32, torch.uint8, torch.float8_e4m3fn))
    _dev("k_scale", k_scale, torch.float32, _rows_of(k_cache, paging))
    _dev("ssmax_s", ssmax_s, torch.float32, (H,))
    _dev("ssmax_b", ssmax_b, torch.float32, (H,))
    _dev("inv_freq", inv_freq, torch.float32)
    _dev("scores", scores, torch.float32)
    if scores.dim() != 2 or scores.shape[0] != T:
        raise ValueError("scores must be [T][ld]")
    d = indexer_desc(q, k_cache, inv_freq, paging)
    if ws is None:
        ws = torch.empty(max(16, dsa_indexer_workspace_size(d)), dtype=torch.uint8, device=q.device)
    _dev("ws", ws, torch.uint8)
    _check(_lib.dsa_indexer_scores(ctypes.byref(d), _ptr(q), _ptr(w), _ptr(q_seq), _ptr(q_pos), _ptr(ssmax_s),
                                   _ptr(ssmax_b), _ptr(inv_freq), _ptr(k_cache), _ptr(k_scale), _ptr(scores),
                                   scores.shape[1], _ptr(ws), ws.numel(), _stream(stream), _pg(paging)))
    return scores


def dsa_indexer_topk(q, w, q_seq, q_pos, k_cache, scores, k, idx, length=None, k_scale=None, ssmax_s=None,
                     ssmax_b=None, inv_freq=None, ws=None, topk_ws=None, stream=None, paging=None):
    """Scores and top-k selection in one call (the fp8 score kernel also builds the first radix
    digit's histogram).  Arguments as dsa_indexer_scores plus dsa_topk's."""
    T, H, D = q.shape
    B, max_ctx = _seq_dims(k_cache, paging)
    _dev("q", q, (torch.float32, torch.bfloat16))
    _dev("w", w, torch.float32, (T, H))
    _dev("q_seq", q_seq, torch.int32, (T,))
    _dev("q_pos", q_pos, torch.int32, (T,))
    _dev("k_cache", k_cache, (torch.float32, torch.uint8, torch.float8_e4m3fn))
    _dev("k_scale", k_scale, torch.float32, _rows_of(k_cache, paging))
    _dev("ssmax_s", ssmax_s, torch.float32, (H,))
    _dev("ssmax_b", ssmax_b, torch.float32, (H,))
    _dev("inv_freq", inv_freq, torch.float32)
    _dev("scores", scores, torch.float32)
    _dev("idx", idx, torch.int32, (T, k))
    _dev("length", length, torch.int32, (T,))
    if scores.dim() != 2 or scores.shape[0] != T:
        raise ValueError("scores must be [T][ld]")
    ld = scores.shape[1]
    d = indexer_desc(q, k_cache, inv_freq, paging)
    if ws is None:
        ws = torch.empty(max(16, dsa_indexer_workspace_size(d)), dtype=torch.uint8, device=q.device)
    if topk_ws is None:
        topk_ws = topk_workspace(T, ld, k, q.device)
    _dev("ws", ws, torch.uint8)
    _dev("topk_ws", topk_ws, torch.uint8)
    _check(_lib.dsa_indexer_topk(ctypes.byref(d), _ptr(q), _ptr(w), _ptr(q_seq), _ptr(q_pos), _ptr(ssmax_s),
                                 _ptr(ssmax_b), _ptr(inv_freq), _ptr(k_cache), _ptr(k_scale), _ptr(scores), ld, k,
                                 _ptr(idx), _ptr(length), _ptr(ws), ws.numel(), _ptr(topk_ws), topk_ws.numel(),
                                 _stream(stream), _pg(paging)))
    return idx, length


def dsa_indexer_scores_hist(q, w, q_seq, q_pos, k_cache, scores, k, topk_ws, k_scale=None, ssmax_s=None,
                            ssmax_b=None, inv_freq=None, ws=None, stream=None, paging=None):
    """First half of dsa_indexer_topk: the scores, plus each row's first-digit histogram left in
    topk_ws for dsa_topk_hist.  Arguments as dsa_indexer_topk (no index outputs)."""
    T, H, D = q.shape
    B, max_ctx = _seq_dims(k_cache, paging)
    _dev("q", q, (torch.float32, torch.bfloat16))
    _dev("w", w, torch.float32, (T, H))
    _dev("q_seq", q_seq, torch.int32, (T,))
    _dev("q_pos", q_pos, torch.int32, (T,))
    _dev("k_cache", k_cache, (torch.float32, torch.uint8, torch.float8_e4m3fn))
    _dev("k_scale", k_scale, torch.float32, _rows_of(k_cache, paging))
    _dev("ssmax_s", ssmax_s, torch.float32, (H,))
    _dev("ssmax_b", ssmax_b, torch.float32, (H,))
    _dev("inv_freq", inv_freq, torch.float32)
    _dev("scores", scores, torch.float32)
    _dev("topk_ws", topk_ws, torch.uint8)
    if scores.dim() != 2 or scores.shape[0] != T:
        raise ValueError("scores must be [T][ld]")
    d = indexer_desc(q, k_cache, inv_freq, paging)
    if ws is None:
        ws = torch.empty(max(16, dsa_indexer_workspace_size(d)), dtype=torch.uint8, device=q.device)
    _dev("ws", ws, torch.uint8)
    _check(_lib.dsa_indexer_scores_hist(ctypes.byref(d), _ptr(q), _ptr(w), _ptr(q_seq), _ptr(q_pos), _ptr(ssmax_s),
                                        _ptr(ssmax_b), _ptr(inv_freq), _ptr(k_cache), _ptr(k_scale), _ptr(scores),
                                        scores.shape[1], k, _ptr(ws), ws.numel(), _ptr(topk_ws), topk_ws.numel(),
                                        _stream(stream), _pg(paging)))
    return scores


def dsa_topk_hist(scores, q_pos, k, idx, length, max_ctx, topk_ws, stream=None):
    """Second half of dsa_indexer_topk: the top-k of each row from the scores and the histogram a
    preceding dsa_indexer_scores_hist left in topk_ws (rows hold min(q_pos + 1, max_ctx) scores)."""
    T = scores.shape[0]
    _dev("scores", scores, torch.float32)
    _dev("q_pos", q_pos, torch.int32, (T,))
    _dev("idx", idx, torch.int32, (T, k))
    _dev("length", length, torch.int32, (T,))
    _dev("topk_ws", topk_ws, torch.uint8)
    d = IndexerDesc(T, 0, 128, 0, 1, max_ctx, DSA_F32, DSA_F32)   # only num_q and max_ctx are read
    _check(_lib.dsa_topk_hist(ctypes.byref(d), _ptr(scores), scores.shape[1], _ptr(q_pos), k, _ptr(idx),
                              _ptr(length), _ptr(topk_ws), topk_ws.numel(), _stream(stream)))
    return idx, length


# ------------------------------------------------------------------------------------------------
# 2. selection
# ------------------------------------------------------------------------------------------------

def dsa_topk_workspace_size(num_q: int, ld: int, k: int) -> int:
    return int(_lib.dsa_topk_workspace_size(num_q, ld, k))


def topk_workspace(num_q: int, ld: int, k: int, device) -> torch.Tensor:
    """A zero-filled top-k workspace (every call clears what it used; stale contents only slow a
    call down)."""
    return torch.zeros(max(16, dsa_topk_workspace_size(num_q, ld, k)), dtype=torch.uint8, device=device)


def dsa_topk(scores, q_pos, k, idx, length=None, ws=None, stream=None):
    """Top-k of each score row (n = q_pos + 1 columns): idx [T][k] ascending, -1 padded; length [T]."""
    T, ld = scores.shape
    _dev("scores", scores, torch.float32)
    _dev("q_pos", q_pos, torch.int32, (T,))
    _dev("idx", idx, torch.int32, (T, k))
    _dev("length", length, torch.int32, (T,))
    if ws is None:
        ws = topk_workspace(T, ld, k, scores.device)
    _dev("ws", ws, torch.uint8)
    _check(_lib.dsa_topk(_ptr(scores), ld, _ptr(q_pos), T, k, _ptr(idx), _ptr(length), _ptr(ws), ws.numel(),
                         _stream(stream)))
    return idx, length


def dsa_block_select_workspace_size(num_q: int, ld: int, block: int) -> int:
    return int(_lib.dsa_block_select_workspace_size(num_q, ld, block))


def dsa_block_select(scores, q_pos, idx, length=None, block=128, nblocks=16, ws=None, stream=None):
    """Block-sparse selection: best `nblocks` blocks of `block` keys, the query's own block forced."""
    T, ld = scores.shape
    topk = idx.shape[1]
    _dev("scores", scores, torch.float32)
    _dev("q_pos", q_pos, torch.int32, (T,))
    _dev("idx", idx, torch.int32, (T, topk))
    _dev("length", length, torch.int32, (T,))
    need = dsa_block_select_workspace_size(T, ld, block)
    if ws is None:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=scores.device)
    _dev("ws", ws, torch.uint8)
    _check(_lib.dsa_block_select(_ptr(scores), ld, _ptr(q_pos), T, block, nblocks, topk, _ptr(idx),
                                 _ptr(length), _ptr(ws), ws.numel(), _stream(stream)))
    return idx, length


def dsa_indexer_block_select(q, w, q_seq, q_pos, k_cache, scores, idx, length=None, block=128, nblocks=16,
                             k_scale=None, ssmax_s=None, ssmax_b=None, inv_freq=None, ws=None, bs_ws=None,
                             stream=None, paging=None, ld=None):
    """Scores and block-sparse selection in one call (dsa_indexer_scores then dsa_block_select; the
    fp8 decode score kernel writes the block maxima itself).  scores may be None where the score
    kernel writes the block maxima (the scores are then not written); ld then gives the row stride
    the block workspace is sized for (default max_ctx rounded up to 4)."""
    T, H, D = q.shape
    B, max_ctx = _seq_dims(k_cache, paging)
    _dev("q", q, (torch.float32, torch.bfloat16))
    _dev("w", w, torch.float32, (T, H))
    _dev("q_seq", q_seq, torch.int32, (T,))
    _dev("q_pos", q_pos, torch.int32, (T,))
    _dev("k_cache", k_cache, (torch.float32, torch.uint8, torch.float8_e4m3fn))
    _dev("k_scale", k_scale, torch.float32, _rows_of(k_cache, paging))
    _dev("ssmax_s", ssmax_s, torch.float32, (H,))
    _dev("ssmax_b", ssmax_b, torch.float32, (H,))
    _dev("inv_freq", inv_freq, torch.float32)
    _dev("scores", scores, torch.float32)
    _dev("idx", idx, torch.int32)
    _dev("length", length, torch.int32, (T,))
    if (scores is not None and (scores.dim() != 2 or scores.shape[0] != T)) or idx.dim() != 2 or idx.shape[0] != T:
        raise ValueError("scores must be [T][ld] and idx [T][topk]")
    if scores is not None:
        ld = scores.shape[1]
    elif ld is None:
        ld = (max_ctx + 3) // 4 * 4
    d = indexer_desc(q, k_cache, inv_freq, paging)
    if ws is None:
        ws = torch.empty(max(16, dsa_indexer_workspace_size(d)), dtype=torch.uint8, device=q.device)
    if bs_ws is None:
        bs_ws = torch.empty(max(16, dsa_block_select_workspace_size(T, ld, block)), dtype=torch.uint8,
                            device=q.device)
    _dev("ws", ws, torch.uint8)
    _dev("bs_ws", bs_ws, torch.uint8)
    _check(_lib.dsa_indexer_block_select(ctypes.byref(d), _ptr(q), _ptr(w), _ptr(q_seq), _ptr(q_pos), _ptr(ssmax_s),
                                         _ptr(ssmax_b), _ptr(inv_freq), _ptr(k_cache), _ptr(k_scale), _ptr(scores),
                                         ld, block, nblocks, idx.shape[1], _ptr(idx), _ptr(length), _ptr(ws),
                                         ws.numel(), _ptr(bs_ws), bs_ws.numel(), _stream(stream), _pg(paging)))
    return idx, length


# ------------------------------------------------------------------------------------------------
# 3. sparse MLA
# ------------------------------------------------------------------------------------------------

def mla_desc(q, kv, idx, softmax_scale, num_splits=0, paging=None) -> MlaDesc:
    T, H, DQ = q.shape
    B, max_ctx = _seq_dims(kv, paging)
    rope = DQ - 512
    return MlaDesc(T, H, 512, rope, B, max_ctx, idx.shape[1], _qdtype(q), _kdtype(kv), 64, float(softmax_scale),
                   int(num_splits))


def dsa_sparse_mla_workspace_size(desc: MlaDesc) -> int:
    return int(_lib.dsa_sparse_mla_workspace_size(ctypes.byref(desc)))


def _mla(fn, q, kv, kv_scale, q_seq, idx, length, out, lse, softmax_scale, num_splits, ws, stream, paging=None):
    T, H, DQ = q.shape
    row = kv.shape[-1]
    _dev("q", q, (torch.float32, torch.bfloat16))
    _dev("kv", kv, (torch.float32, torch.uint8, torch.float8_e4m3fn))
    _dev("kv_scale", kv_scale, torch.float32, (*_rows_of(kv, paging), row // 64))
    _dev("q_seq", q_seq, torch.int32, (T,))
    _dev("idx", idx, torch.int32)
    _dev("length", length, torch.int32, (T,))
    _dev("out", out, torch.float32, (T, H, 512))
    _dev("lse", lse, torch.float32, (T, H))
    if row != 576 or DQ not in (512, 576):
        raise ValueError("kv rows must be 576 wide and q 512 (NoPE) or 576 (RoPE) wide")
    d = mla_desc(q, kv, idx, softmax_scale, num_splits, paging)
    need = dsa_sparse_mla_workspace_size(d)
    if ws is None and need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    _dev("ws", ws, torch.uint8)
    _check(fn(ctypes.byref(d), _ptr(q), _ptr(kv), _ptr(kv_scale), _ptr(q_seq), _ptr(idx), _ptr(length), _ptr(out),
              _ptr(lse), _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream), _pg(paging)))
    return out, lse


def dsa_sparse_mla_decode(q, kv, kv_scale, q_seq, idx, length, out, lse=None, softmax_scale=None, num_splits=0,
                          ws=None, stream=None, paging=None):
    """Sparse MLA for decode (each query's selection split over several workgroups)."""
    return _mla(_lib.dsa_sparse_mla_decode, q, kv, kv_scale, q_seq, idx, length, out, lse, softmax_scale,
                num_splits, ws, stream, paging)


def dsa_sparse_mla_decode_noalloc(q, kv, kv_scale, q_seq, idx, length, out, lse=None, softmax_scale=None,
                                  num_splits=0, stream=None, paging=None):
    """dsa_sparse_mla_decode with the split partials in the library's per-GPU scratch buffer (no
    workspace argument, nothing allocated)."""
    T, H, DQ = q.shape
    row = kv.shape[-1]
    _dev("q", q, (torch.float32, torch.bfloat16))
    _dev("kv", kv, (torch.float32, torch.uint8, torch.float8_e4m3fn))
    _dev("kv_scale", kv_scale, torch.float32, (*_rows_of(kv, paging), row // 64))
    _dev("q_seq", q_seq, torch.int32, (T,))
    _dev("idx", idx, torch.int32)
    _dev("length", length, torch.int32, (T,))
    _dev("out", out, torch.float32, (T, H, 512))
    _dev("lse", lse, torch.float32, (T, H))
    if row != 576 or DQ not in (512, 576):
        raise ValueError("kv rows must be 576 wide and q 512 (NoPE) or 576 (RoPE) wide")
    d = mla_desc(q, kv, idx, softmax_scale, num_splits, paging)
    _check(_lib.dsa_sparse_mla_decode_noalloc(ctypes.byref(d), _ptr(q), _ptr(kv), _ptr(kv_scale), _ptr(q_seq),
                                              _ptr(idx), _ptr(length), _ptr(out), _ptr(lse), _stream(stream),
                                              _pg(paging)))
    return out, lse


def dsa_sparse_mla_prefill(q, kv, kv_scale, q_seq, idx, length, out, lse=None, softmax_scale=None, ws=None,
                           stream=None, paging=None):
    """Sparse MLA for chunked prefill (one workgroup per query)."""
    return _mla(_lib.dsa_sparse_mla_prefill, q, kv, kv_scale, q_seq, idx, length, out, lse, softmax_scale, 0,
                ws, stream, paging)


# ------------------------------------------------------------------------------------------------
# 0. cache writers
# ------------------------------------------------------------------------------------------------

def index_k_desc(x, hidden, rope_dim, eps, num_slots) -> IndexKDesc:
    return IndexKDesc(x.shape[0], int(hidden), x.stride(0), int(rope_dim), float(eps), int(num_slots))


def dsa_index_k_insert_workspace_size(desc: IndexKDesc) -> int:
    return int(_lib.dsa_index_k_insert_workspace_size(ctypes.byref(desc)))


def dsa_index_k_insert(x, wk, ln_w, ln_b, pos, slot, k_cache, k_scale, inv_freq=None, eps=1e-6, ws=None,
                       stream=None, paging=None):
    """Indexer keys of x's tokens (LayerNorm of the key projection, RoPE when inv_freq is given,
    FP8 with one scale per token) written into k_cache / k_scale at rows `slot` (-1 = skip).

    x [T][hidden] bf16 (rows may be strided), wk [128][hidden] bf16, ln_w / ln_b [128] f32,
    pos [T] i32, slot [T] i64, k_cache [..., 128] uint8 / float8_e4m3fn, k_scale [...] f32; with
    paging, k_cache is the paged pool and a slot's key bytes go to its block's 16x16 tiles."""
    T, hidden = x.shape
    if x.dtype != torch.bfloat16 or not x.is_cuda or x.stride(1) != 1:
        raise ValueError("x must be a bf16 GPU tensor with unit column stride")
    _dev("wk", wk, torch.bfloat16, (128, hidden))
    _dev("ln_w", ln_w, torch.float32, (128,))
    _dev("ln_b", ln_b, torch.float32, (128,))
    _dev("pos", pos, torch.int32, (T,))
    _dev("slot", slot, torch.int64, (T,))
    _dev("inv_freq", inv_freq, torch.float32, (32,))
    _dev("k_cache", k_cache, (torch.uint8, torch.float8_e4m3fn))
    _dev("k_scale", k_scale, torch.float32)
    if k_cache.shape[-1] != 128 or k_cache.numel() // 128 != k_scale.numel():
        raise ValueError("k_cache must hold 128-byte rows, one k_scale per row")
    d = index_k_desc(x, hidden, 64 if inv_freq is not None else 0, eps, k_scale.numel())
    need = dsa_index_k_insert_workspace_size(d)
    if ws is None and need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=x.device)
    _dev("ws", ws, torch.uint8)
    _check(_lib.dsa_index_k_insert(ctypes.byref(d), _ptr(x), _ptr(wk), _ptr(ln_w), _ptr(ln_b), _ptr(pos),
                                   _ptr(inv_freq), _ptr(slot), _ptr(k_cache), _ptr(k_scale), _ptr(ws),
                                   0 if ws is None else ws.numel(), _stream(stream), _pg(paging)))
    return k_cache, k_scale


def dsa_paged_slots(paging, seq, pos, slot=None, stream=None):
    """Pool slot of each (seq[j], pos[j]) by the paged layout rule (-1 where pos[j] < 0)."""
    n = int(pos.numel())
    _dev("seq", seq, torch.int32, (n,))
    _dev("pos", pos, torch.int32, (n,))
    if slot is None:
        slot = torch.empty(n, dtype=torch.int64, device=pos.device)
    _dev("slot", slot, torch.int64, (n,))
    _check(_lib.dsa_paged_slots(_pg(paging), n, _ptr(seq), _ptr(pos), _ptr(slot), _stream(stream)))
    return slot


def dsa_latent_insert(kv, pos, slot, kv_cache, kv_scale, inv_freq=None, stream=None):
    """Latent rows kv [T][576] bf16 (rotary slice rotated when inv_freq is given) written as FP8
    with one scale per 64 elements into kv_cache [..., 576] / kv_scale [..., 9] at rows `slot`."""
    T = kv.shape[0]
    if kv.dtype != torch.bfloat16 or not kv.is_cuda or kv.stride(1) != 1 or kv.shape[1] != 576:
        raise ValueError("kv must be a [T][576] bf16 GPU tensor with unit column stride")
    _dev("pos", pos, torch.int32, (T,))
    _dev("slot", slot, torch.int64, (T,))
    _dev("inv_freq", inv_freq, torch.float32, (32,))
    _dev("kv_cache", kv_cache, (torch.uint8, torch.float8_e4m3fn))
    _dev("kv_scale", kv_scale, torch.float32)
    if kv_cache.shape[-1] != 576 or kv_cache.numel() // 576 * 9 != kv_scale.numel():
        raise ValueError("kv_cache must hold 576-byte rows, nine kv_scale entries per row")
    _check(_lib.dsa_latent_insert(T, 64 if inv_freq is not None else 0, _ptr(kv), kv.stride(0), _ptr(pos),
                                  _ptr(inv_freq), _ptr(slot), kv_cache.numel() // 576, _ptr(kv_cache),
                                  _ptr(kv_scale), _stream(stream)))
    return kv_cache, kv_scale


class KernelTimer:
    """Each library kernel's own device duration inside a running pipeline (dsa_timing_begin /
    dsa_timing_end): within the `with` block, up to `capacity` kernels the library enqueues record
    their dispatch's start and stop timestamps into a pair of events; no work is added to the
    stream.  After the block, results() synchronises and returns [(kernel name, microseconds)]
    in launch order."""

    def __init__(self, capacity: int, stream=None):
        self.capacity = int(capacity)
        self.events = [torch.cuda.Event(enable_timing=True) for _ in range(2 * self.capacity)]
        for e in self.events:   # torch creates its events on first record
            e.record(stream)
        self._handles = (ctypes.c_void_p * len(self.events))(*[e.cuda_event for e in self.events])
        self.count = 0
        self.names = []

    def __enter__(self):
        torch.cuda.synchronize()
        _check(_lib.dsa_timing_begin(self._handles, self.capacity))
        return self

    def __exit__(self, *exc):
        self.count = _lib.dsa_timing_end()
        self.names = [(_lib.dsa_timing_kernel_name(i) or b"?").decode() for i in range(self.count)]
        return False

    def results(self):
        torch.cuda.synchronize()
        return [(self.names[i], self.events[2 * i].elapsed_time(self.events[2 * i + 1]) * 1e3)
                for i in range(self.count)]
