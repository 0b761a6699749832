"""Seeded synthetic inputs for the DSA decode / prefill path.

This module only draws random numbers and packs them into the cache formats the
kernels and the oracle both read (fp8 E4M3FN codes plus fp32 scales, bf16 or
fp32 queries).  It holds none of the method's arithmetic: no RoPE, no SSMax, no
scoring, no selection, no attention.  Both the HIP path and the CPU oracle take
their inputs from here and nothing else is shared between them.

Workload shapes follow the pages' model (Mistral Large 4 as described in
"Day 0 support for Mistral Large 4 on vLLM", Highlights and the architecture
table: 32 index heads, top-k 2048, 64 MLA heads, KV LoRA rank 512, RoPE dim 64)
and the decode / prefill / block-sparse settings of the five measured
configurations (8K fp32 check, 64 x 16-32K fp8, 16 x 128K fp8 in RoPE / NoPE /
shared-indexer variants, a 4096-token chunked prefill over a 61440 prefix, and
a 4 x 512K block-sparse scan).

Generation order per workload is fixed: positions, index query, index weights,
SSMax s and b, index keys, MLA query, latent cache.  Everything is drawn from
one ``torch.Generator`` seeded with the workload seed, on the device the caller
asks for (CPU for small cases, the GPU for full-size ones).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

E4M3_MAX = 448.0
INDEX_HEAD_DIM = 128
ROPE_DIM = 64
KV_LORA = 512
KV_ROW = KV_LORA + ROPE_DIM  # 576 latent elements per cached token
KV_SCALE_BLOCK = 64
TOPK = 2048


def inv_freq_table(rope_dim: int = ROPE_DIM, base: float = 10000.0) -> torch.Tensor:
    """Synthetic stand-in for the YaRN + LeRoPE frequency table: base^(-2j/rope_dim)."""
    j = torch.arange(rope_dim // 2, dtype=torch.float64)
    return (base ** (-2.0 * j / rope_dim)).to(torch.float32)


def quantize_e4m3(x: torch.Tensor, block: int):
    """Quantise the last dim of x to E4M3FN codes with one fp32 scale per `block` elements.

    scale = amax / 448 (1 where amax == 0); code = RNE(x / scale), saturated to +-448.
    Returns (uint8 codes shaped like x, fp32 scales shaped x[..., D // block]).
    """
    d = x.shape[-1]
    assert d % block == 0
    xb = x.float().reshape(*x.shape[:-1], d // block, block)
    amax = xb.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
    y = (xb / scale.unsqueeze(-1)).clamp_(-E4M3_MAX, E4M3_MAX)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8).reshape(x.shape)
    return codes.contiguous(), scale.contiguous()


@dataclasses.dataclass
class Workload:
    """One batch of inputs for index scoring, selection and sparse MLA.

    Layouts (row-major, contiguous):
      q_seq, q_pos     [T] int32          sequence id and 0-based position of each query
      seq_len          [B] int32          cached tokens per sequence
      index_q          [T][H][128]        f32 or bf16
      index_w          [T][H] f32         weights_proj(x) per head
      ssmax_s/b        [H] f32            per-head SSMax parameters (None: no SSMax)
      inv_freq         [rope/2] f32       rotary frequencies (None on NoPE layers)
      index_k          [B][max_ctx][128]  f32, or uint8 E4M3FN codes
      index_k_scale    [B][max_ctx] f32   per-token key scale (None for f32 keys)
      mla_q            [T][64][512+rope]  f32 or bf16
      kv               [B][max_ctx][576]  f32, or uint8 E4M3FN codes
      kv_scale         [B][max_ctx][9]    per-64-element latent scales (None for f32)
    """
    name: str
    num_heads: int
    rope_dim: int
    softmax_scale: float
    topk: int
    q_seq: torch.Tensor
    q_pos: torch.Tensor
    seq_len: torch.Tensor
    max_ctx: int
    index_q: torch.Tensor
    index_w: torch.Tensor
    ssmax_s: Optional[torch.Tensor]
    ssmax_b: Optional[torch.Tensor]
    inv_freq: Optional[torch.Tensor]
    index_k: torch.Tensor
    index_k_scale: Optional[torch.Tensor]
    mla_q: torch.Tensor
    kv: torch.Tensor
    kv_scale: Optional[torch.Tensor]
    mla_heads: int = 64

    @property
    def num_q(self) -> int:
        return int(self.q_pos.shape[0])

    @property
    def num_seqs(self) -> int:
        return int(self.seq_len.shape[0])

    @property
    def fp8(self) -> bool:
        return self.index_k.dtype == torch.uint8

    def to(self, device) -> "Workload":
        kw = {}
        for f in dataclasses.fields(self):
            v = getattr(self, f.name)
            kw[f.name] = v.to(device) if isinstance(v, torch.Tensor) else v
        return Workload(**kw)


def _normal(gen, shape, device, std=1.0):
    return torch.randn(*shape, generator=gen, device=device, dtype=torch.float32).mul_(std)


def _uniform(gen, shape, device, lo, hi):
    return torch.rand(*shape, generator=gen, device=device, dtype=torch.float32).mul_(hi - lo).add_(lo)


def make_workload(*, name: str, seed: int, seq_lens, max_ctx: int, q_positions=None, q_seqs=None,
                  num_heads: int = 32, mla_heads: int = 64, rope: bool = True, fp8: bool = True,
                  q_dtype: torch.dtype = torch.bfloat16, ssmax: bool = True, topk: int = TOPK,
                  device="cpu", mla_q_std: float = 1.0) -> Workload:
    """Draw one workload.

    seq_lens: per-sequence cached lengths (list or tensor) or an int (all equal).
    q_positions / q_seqs: explicit query placement; default is decode, one query per
    sequence at position seq_len - 1 (its own key already in the cache).
    """
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(int(seed))
    if isinstance(seq_lens, int):
        seq_len = torch.full((1,), seq_lens, dtype=torch.int32)
    else:
        seq_len = torch.as_tensor(seq_lens, dtype=torch.int32).flatten()
    B = int(seq_len.shape[0])
    assert int(seq_len.max()) <= max_ctx
    if q_positions is None:
        q_pos = (seq_len - 1).to(torch.int32)
        q_seq = torch.arange(B, dtype=torch.int32)
    else:
        q_pos = torch.as_tensor(q_positions, dtype=torch.int32).flatten()
        q_seq = (torch.zeros_like(q_pos) if q_seqs is None
                 else torch.as_tensor(q_seqs, dtype=torch.int32).flatten())
    T = int(q_pos.shape[0])
    rope_dim = ROPE_DIM if rope else 0

    index_q = _normal(gen, (T, num_heads, INDEX_HEAD_DIM), dev)
    index_w = _normal(gen, (T, num_heads), dev)
    if ssmax:
        ssmax_s = _uniform(gen, (num_heads,), dev, 0.05, 0.2)
        ssmax_b = _uniform(gen, (num_heads,), dev, 0.9, 1.1)
    else:
        ssmax_s = ssmax_b = None
    keys = _normal(gen, (B, max_ctx, INDEX_HEAD_DIM), dev)
    if fp8:
        index_k, index_k_scale = quantize_e4m3(keys, INDEX_HEAD_DIM)
        index_k_scale = index_k_scale.reshape(B, max_ctx)
    else:
        index_k, index_k_scale = keys, None
    del keys
    mla_q = _normal(gen, (T, mla_heads, KV_LORA + rope_dim), dev, mla_q_std)
    latent = _normal(gen, (B, max_ctx, KV_ROW), dev, 1.0 / math.sqrt(KV_ROW))
    if fp8:
        kv, kv_scale = quantize_e4m3(latent, KV_SCALE_BLOCK)
    else:
        kv, kv_scale = latent, None
    del latent
    if q_dtype == torch.bfloat16:
        index_q = index_q.to(torch.bfloat16)
        mla_q = mla_q.to(torch.bfloat16)
    # RoPE layers: the un-absorbed qk head is 128 NoPE + 64 rope dims -> 1/sqrt(192);
    # NoPE layers have 128 qk dims and no rope part -> 1/sqrt(128).
    softmax_scale = 1.0 / math.sqrt(192.0) if rope else 1.0 / math.sqrt(128.0)
    return Workload(name=name, num_heads=num_heads, rope_dim=rope_dim, softmax_scale=softmax_scale,
                    topk=topk, q_seq=q_seq.to(dev), q_pos=q_pos.to(dev), seq_len=seq_len.to(dev),
                    max_ctx=max_ctx, index_q=index_q.contiguous(), index_w=index_w.contiguous(),
                    ssmax_s=ssmax_s, ssmax_b=ssmax_b,
                    inv_freq=inv_freq_table().to(dev) if rope else None,
                    index_k=index_k.contiguous(), index_k_scale=index_k_scale,
                    mla_q=mla_q.contiguous(), kv=kv.contiguous(), kv_scale=kv_scale,
                    mla_heads=mla_heads)


# ---- the measured configurations -------------------------------------------------------------

def config0(device="cpu", seed=0):
    """Single decode step, batch 1, context 8192, RoPE layer, fp32 everywhere."""
    return make_workload(name="decode_b1_ctx8192_f32", seed=seed, seq_lens=[8192], max_ctx=8192,
                         fp8=False, q_dtype=torch.float32, device=device)


def config1(device="cpu", seed=1, batch=64, lo=16384, hi=32768):
    """Decode, batch 64, per-sequence context uniform in [16K, 32K], fp8 caches."""
    g = torch.Generator().manual_seed(seed + 1000)
    lens = torch.randint(lo, hi + 1, (batch,), generator=g, dtype=torch.int64).to(torch.int32)
    return make_workload(name=f"decode_b{batch}_ctx{lo}-{hi}_fp8", seed=seed, seq_lens=lens,
                         max_ctx=hi, device=device)


def config2(variant="a", device="cpu", seed=2, batch=16, ctx=131072):
    """Decode, batch 16, context 131072, fp8 caches; variant a = RoPE layer, b = NoPE layer.

    Variant c (shared indexer) uses variant a's caches and selection; it has no inputs of
    its own beyond a's.
    """
    rope = variant != "b"
    return make_workload(name=f"decode_b{batch}_ctx{ctx}_fp8_{'rope' if rope else 'nope'}",
                         seed=seed + (10 if not rope else 0), seq_lens=[ctx] * batch, max_ctx=ctx,
                         rope=rope, device=device)


def config3(device="cpu", seed=3, prefix=61440, chunk=4096):
    """Chunked causal prefill: `chunk` new query tokens appended to a `prefix`-token prefix."""
    total = prefix + chunk
    return make_workload(name=f"prefill_{chunk}_on_{prefix}_fp8", seed=seed, seq_lens=[total],
                         max_ctx=total, q_positions=torch.arange(prefix, total, dtype=torch.int32),
                         device=device)


def config4(device="cpu", seed=4, batch=4, ctx=524288):
    """Block-sparse long-context decode: 4 index heads, 128-token blocks, top-16 blocks."""
    return make_workload(name=f"blocksparse_b{batch}_ctx{ctx}_fp8", seed=seed, seq_lens=[ctx] * batch,
                         max_ctx=ctx, num_heads=4, device=device)


def verify_blocks(device="cpu", seed=5, batch=16, tokens=4, ctx=131072, seq_lens=None, max_ctx=None,
                  drift=0.25, **kw):
    """Multi-token decode: each of `batch` sequences verifies a block of `tokens` consecutive query
    tokens at its last positions (a speculative-decoding verify block; the block's own keys are
    already in the caches and each token attends causally, up to its own position).  Query t is
    token t % tokens of sequence t // tokens.  Neighbouring tokens of a text select largely the
    same keys; here every token's index queries and head weights are its block's first token's
    plus drift * N(0, 1), which gives that overlap.  The attention queries are independent."""
    lens = [ctx] * batch if seq_lens is None else list(seq_lens)
    B = len(lens)
    pos = [n - tokens + j for n in lens for j in range(tokens)]
    seqs = [b for b in range(B) for _ in range(tokens)]
    wl = make_workload(name=f"verify_b{B}x{tokens}_ctx{max(lens)}_fp8", seed=seed, seq_lens=lens,
                       max_ctx=max(lens) if max_ctx is None else max_ctx, q_positions=pos, q_seqs=seqs,
                       device=device, **kw)
    gen = torch.Generator(device=torch.device(device))
    gen.manual_seed(int(seed) + 7)
    T, H, D = wl.index_q.shape
    anchor_q = wl.index_q.float().reshape(B, tokens, H, D)[:, :1]
    anchor_w = wl.index_w.float().reshape(B, tokens, H)[:, :1]
    q = anchor_q + drift * _normal(gen, (B, tokens, H, D), wl.index_q.device)
    w = anchor_w + drift * _normal(gen, (B, tokens, H), wl.index_q.device)
    q[:, 0], w[:, 0] = anchor_q[:, 0], anchor_w[:, 0]
    return dataclasses.replace(wl, index_q=q.reshape(T, H, D).to(wl.index_q.dtype).contiguous(),
                               index_w=w.reshape(T, H).contiguous())


HIDDEN = 6144   # Mistral Large 4 hidden size (the indexer key projection's input width)


@dataclasses.dataclass
class InsertBatch:
    """Inputs of the cache writers for T new tokens.

    Layouts (row-major, contiguous):
      x          [T][hidden] bf16      hidden states entering the indexer key projection
      wk         [128][hidden] bf16    that projection's weight (output dim first)
      ln_w, ln_b [128] f32             the key LayerNorm's weight and bias
      eps        float                 LayerNorm epsilon
      kv         [T][576] bf16         latent rows (512 latent + 64 rotary dims) to be cached
      pos        [T] int32             0-based position of each token in its sequence
      seq        [T] int32             its sequence
      slot       [T] int64             destination cache row: seq * max_ctx + pos, -1 = skip
      inv_freq   [32] f32 or None      rotary frequencies (None on NoPE layers)
    """
    name: str
    x: torch.Tensor
    wk: torch.Tensor
    ln_w: torch.Tensor
    ln_b: torch.Tensor
    eps: float
    kv: torch.Tensor
    pos: torch.Tensor
    seq: torch.Tensor
    slot: torch.Tensor
    inv_freq: Optional[torch.Tensor]
    num_seqs: int
    max_ctx: int

    @property
    def num_tokens(self) -> int:
        return int(self.pos.shape[0])


def make_insert_batch(*, name: str, seed: int, positions, seqs, num_seqs: int, max_ctx: int,
                      hidden: int = HIDDEN, rope: bool = True, skip=(), device="cpu") -> InsertBatch:
    """Draw the cache writers' inputs: x ~ N(0, 1), wk ~ N(0, 1/hidden) (so each projected
    output is about unit-variance), LayerNorm weight U(0.9, 1.1) and bias N(0, 0.1^2),
    eps 1e-6, latent rows N(0, 1/576).  Tokens listed in `skip` get slot -1 (padding)."""
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(int(seed))
    pos = torch.as_tensor(positions, dtype=torch.int32).flatten()
    seq = torch.as_tensor(seqs, dtype=torch.int32).flatten()
    assert pos.shape == seq.shape and int(pos.max()) < max_ctx and int(seq.max()) < num_seqs
    T = int(pos.shape[0])
    x = _normal(gen, (T, hidden), dev).to(torch.bfloat16)
    wk = _normal(gen, (INDEX_HEAD_DIM, hidden), dev, 1.0 / math.sqrt(hidden)).to(torch.bfloat16)
    ln_w = _uniform(gen, (INDEX_HEAD_DIM,), dev, 0.9, 1.1)
    ln_b = _normal(gen, (INDEX_HEAD_DIM,), dev, 0.1)
    kv = _normal(gen, (T, KV_ROW), dev, 1.0 / math.sqrt(KV_ROW)).to(torch.bfloat16)
    slot = seq.to(torch.int64) * max_ctx + pos.to(torch.int64)
    for t in skip:
        slot[t] = -1
    return InsertBatch(name=name, x=x, wk=wk, ln_w=ln_w, ln_b=ln_b, eps=1e-6, kv=kv, pos=pos.to(dev),
                       seq=seq.to(dev), slot=slot.to(dev), inv_freq=inv_freq_table().to(dev) if rope else None,
                       num_seqs=num_seqs, max_ctx=max_ctx)


def insert_decode(device="cpu", seed=20, batch=16, ctx=131072, rope=True):
    """One decode step's new tokens: the last position of each of `batch` sequences."""
    return make_insert_batch(name=f"insert_decode_b{batch}_ctx{ctx}", seed=seed, positions=[ctx - 1] * batch,
                             seqs=list(range(batch)), num_seqs=batch, max_ctx=ctx, rope=rope, device=device)


def insert_prefill(device="cpu", seed=21, prefix=61440, chunk=4096, rope=True):
    """A prefill chunk's new tokens: positions prefix .. prefix + chunk - 1 of one sequence."""
    total = prefix + chunk
    return make_insert_batch(name=f"insert_prefill_{chunk}_on_{prefix}", seed=seed,
                             positions=list(range(prefix, total)), seqs=[0] * chunk, num_seqs=1,
                             max_ctx=total, rope=rope, device=device)


def slice_query(wl: Workload, t: int) -> Workload:
    """Query t and its own sequence only (B = 1), copied to the CPU: what the oracle needs to
    recompute one query of a large workload."""
    b = int(wl.q_seq[t])
    sl = lambda x: None if x is None else x[b:b + 1].cpu()
    cpu = lambda x: None if x is None else x.cpu()
    return Workload(name=f"{wl.name}[q{t}]", num_heads=wl.num_heads, rope_dim=wl.rope_dim,
                    softmax_scale=wl.softmax_scale, topk=wl.topk, q_seq=torch.zeros(1, dtype=torch.int32),
                    q_pos=wl.q_pos[t:t + 1].cpu(), seq_len=wl.seq_len[b:b + 1].cpu(), max_ctx=wl.max_ctx,
                    index_q=wl.index_q[t:t + 1].cpu(), index_w=wl.index_w[t:t + 1].cpu(),
                    ssmax_s=cpu(wl.ssmax_s), ssmax_b=cpu(wl.ssmax_b), inv_freq=cpu(wl.inv_freq),
                    index_k=sl(wl.index_k), index_k_scale=sl(wl.index_k_scale), mla_q=wl.mla_q[t:t + 1].cpu(),
                    kv=sl(wl.kv), kv_scale=sl(wl.kv_scale), mla_heads=wl.mla_heads)
