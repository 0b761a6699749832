"""One DSA layer step over device-resident inputs, built from the C-ABI calls.

A layer step is: index scores (with the query's RoPE and SSMax) -> top-k (or block) selection ->
sparse MLA.  A shared-indexer layer skips the first two and reuses another layer's selection
("Day 0 support for Mistral Large 4 on vLLM", the architecture table: 28 of the 72 layers reuse
the top-k of the nearest earlier indexer layer).  Buffers are allocated once and reused, so a
timed step only enqueues kernels.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

from . import (dsa_block_select, dsa_block_select_workspace_size, dsa_indexer_block_select, dsa_indexer_scores,
               dsa_indexer_scores_hist,
               dsa_indexer_topk, dsa_indexer_workspace_size, dsa_sparse_mla_decode, dsa_sparse_mla_prefill,
               dsa_sparse_mla_workspace_size, dsa_topk, dsa_topk_hist, indexer_desc, mla_desc, topk_workspace)


@dataclasses.dataclass
class StepBuffers:
    scores: torch.Tensor
    idx: torch.Tensor
    length: torch.Tensor
    out: torch.Tensor
    lse: torch.Tensor
    ws_index: torch.Tensor
    ws_topk: torch.Tensor
    ws_block: Optional[torch.Tensor]
    ws_mla: Optional[torch.Tensor]


def _ld(max_ctx: int) -> int:
    return (max_ctx + 3) // 4 * 4


def alloc_buffers(wl, *, prefill: bool = False, block_sparse: bool = False, num_splits: int = 0) -> StepBuffers:
    dev = wl.index_q.device
    T, k = wl.num_q, wl.topk
    ld = _ld(wl.max_ctx)
    scores = torch.empty(T, ld, dtype=torch.float32, device=dev)
    idx = torch.empty(T, k, dtype=torch.int32, device=dev)
    length = torch.empty(T, dtype=torch.int32, device=dev)
    out = torch.empty(T, wl.mla_heads, 512, dtype=torch.float32, device=dev)
    lse = torch.empty(T, wl.mla_heads, dtype=torch.float32, device=dev)
    ws_index = torch.empty(max(16, dsa_indexer_workspace_size(indexer_desc(wl.index_q, wl.index_k, wl.inv_freq))),
                           dtype=torch.uint8, device=dev)
    ws_topk = topk_workspace(T, ld, k, dev)
    ws_block = None
    if block_sparse:
        ws_block = torch.empty(max(16, dsa_block_select_workspace_size(T, ld, 128)), dtype=torch.uint8, device=dev)
    ws_mla = None
    if not prefill:
        need = dsa_sparse_mla_workspace_size(mla_desc(wl.mla_q, wl.kv, idx, wl.softmax_scale, num_splits))
        if need:
            ws_mla = torch.empty(need, dtype=torch.uint8, device=dev)
    return StepBuffers(scores, idx, length, out, lse, ws_index, ws_topk, ws_block, ws_mla)


def index_scores(wl, buf: StepBuffers, stream=None):
    return dsa_indexer_scores(wl.index_q, wl.index_w, wl.q_seq, wl.q_pos, wl.index_k, buf.scores,
                              k_scale=wl.index_k_scale, ssmax_s=wl.ssmax_s, ssmax_b=wl.ssmax_b,
                              inv_freq=wl.inv_freq, ws=buf.ws_index, stream=stream)


def select(wl, buf: StepBuffers, *, block_sparse: bool = False, stream=None):
    if block_sparse:
        return dsa_block_select(buf.scores, wl.q_pos, buf.idx, buf.length, block=128, nblocks=16, ws=buf.ws_block,
                                stream=stream)
    return dsa_topk(buf.scores, wl.q_pos, wl.topk, buf.idx, buf.length, ws=buf.ws_topk, stream=stream)


def attend(wl, buf: StepBuffers, *, prefill: bool = False, num_splits: int = 0, idx=None, length=None,
           stream=None):
    idx = buf.idx if idx is None else idx
    length = buf.length if length is None else length
    if prefill:
        return dsa_sparse_mla_prefill(wl.mla_q, wl.kv, wl.kv_scale, wl.q_seq, idx, length, buf.out, buf.lse,
                                      softmax_scale=wl.softmax_scale, stream=stream)
    return dsa_sparse_mla_decode(wl.mla_q, wl.kv, wl.kv_scale, wl.q_seq, idx, length, buf.out, buf.lse,
                                 softmax_scale=wl.softmax_scale, num_splits=num_splits, ws=buf.ws_mla,
                                 stream=stream)


def index_and_select(wl, buf: StepBuffers, stream=None):
    """Scores and top-k in one call (histogram of the first radix digit fused into the scores)."""
    return dsa_indexer_topk(wl.index_q, wl.index_w, wl.q_seq, wl.q_pos, wl.index_k, buf.scores, wl.topk, buf.idx,
                            buf.length, k_scale=wl.index_k_scale, ssmax_s=wl.ssmax_s, ssmax_b=wl.ssmax_b,
                            inv_freq=wl.inv_freq, ws=buf.ws_index, topk_ws=buf.ws_topk, stream=stream)


def index_and_select_blocks(wl, buf: StepBuffers, stream=None, keep_scores: bool = False):
    """Scores and block-sparse selection in one call (the block maxima from the score kernel).  The
    selection needs only the block maxima, so the score rows are written only with keep_scores."""
    return dsa_indexer_block_select(wl.index_q, wl.index_w, wl.q_seq, wl.q_pos, wl.index_k,
                                    buf.scores if keep_scores else None, buf.idx, buf.length, block=128, nblocks=16,
                                    k_scale=wl.index_k_scale, ssmax_s=wl.ssmax_s, ssmax_b=wl.ssmax_b,
                                    inv_freq=wl.inv_freq, ws=buf.ws_index, bs_ws=buf.ws_block, stream=stream,
                                    ld=buf.scores.shape[1])


def index_scores_hist(wl, buf: StepBuffers, stream=None):
    """The scores plus the first-digit histogram (first half of index_and_select)."""
    return dsa_indexer_scores_hist(wl.index_q, wl.index_w, wl.q_seq, wl.q_pos, wl.index_k, buf.scores, wl.topk,
                                   buf.ws_topk, k_scale=wl.index_k_scale, ssmax_s=wl.ssmax_s, ssmax_b=wl.ssmax_b,
                                   inv_freq=wl.inv_freq, ws=buf.ws_index, stream=stream)


def select_hist(wl, buf: StepBuffers, stream=None):
    """The top-k from the scores and histogram index_scores_hist left (second half)."""
    return dsa_topk_hist(buf.scores, wl.q_pos, wl.topk, buf.idx, buf.length, wl.max_ctx, buf.ws_topk, stream=stream)


def layer_step(wl, buf: StepBuffers, *, prefill: bool = False, block_sparse: bool = False,
               shared_from: Optional[StepBuffers] = None, num_splits: int = 0, fused: bool = True, stream=None):
    """Scores -> selection -> sparse MLA; with shared_from, only the MLA over that selection.

    fused (default): one dsa_indexer_topk (dsa_indexer_block_select) call -- the score kernel also
    builds the first radix digit's histogram and emits each chunk's candidates (the block maxima),
    and the selection continues from them; else dsa_indexer_scores and dsa_topk (dsa_block_select)."""
    if shared_from is not None:
        return attend(wl, buf, prefill=prefill, num_splits=num_splits, idx=shared_from.idx,
                      length=shared_from.length, stream=stream)
    if fused and block_sparse:
        # the fp8 decode score kernel (fewer than 256 queries and than two per sequence) writes the
        # 128-key block maxima itself; elsewhere a separate pass reads them from the scores
        fp8 = wl.index_k.dtype in (torch.uint8, torch.float8_e4m3fn)
        decode = wl.num_q < 256 and wl.num_q < 2 * wl.num_seqs
        index_and_select_blocks(wl, buf, stream, keep_scores=not (fp8 and decode))
    elif fused:
        index_and_select(wl, buf, stream)
    else:
        index_scores(wl, buf, stream)
        select(wl, buf, block_sparse=block_sparse, stream=stream)
    return attend(wl, buf, prefill=prefill, num_splits=num_splits, stream=stream)
