/*
 * dsa.h -- C ABI of the DSA (DeepSeek-style sparse attention) hot path for MI355X (gfx950).
 *
 * Three stages, as Mistral Large 4 runs them on every decode step
 * ("Day 0 support for Mistral Large 4 on vLLM", Highlights, the architecture table and
 * "Sparse MLA + DSA indexer"; formulas from "mistral-large4.md", section
 * "What differs from GLM-5.2"):
 *
 *   1. dsa_indexer_scores   lightning-indexer score of every visible cached key per query
 *   2. dsa_topk             keep the k (= 2048) highest-scoring keys per query
 *      dsa_block_select     block-sparse alternative: top-16 128-token blocks, recent block kept
 *   3. dsa_sparse_mla_decode / dsa_sparse_mla_prefill
 *                           exact absorbed-MLA attention over the selected keys only
 *   0. dsa_index_k_insert / dsa_latent_insert
 *                           the writers that put each new token's indexer key and latent row
 *                           into the FP8 caches that stages 1 and 3 read
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor pointer is a DEVICE pointer (HIP global memory); sizes and descriptors are
 *    host values.  Tensors are dense row-major with the layouts given per argument.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls only enqueue work: they never
 *    allocate, free or synchronise, and keep no state besides the loaded code object and the
 *    calling thread's error string.  The caller owns every buffer, including workspaces sized
 *    by the *_workspace_size queries.
 *  - Errors: every host-checkable condition (null pointers, unsupported sizes or dtype
 *    combinations, a workspace that is too small) is checked before anything is launched.
 *    A failing call returns DSA_ERR_ARG or DSA_ERR_UNSUPPORTED, launches nothing, and
 *    dsa_last_error() lists every violated condition.  A failed launch returns DSA_ERR_HIP with
 *    the HIP error text.
 *  - Data-dependent preconditions are the caller's: 0 <= q_pos[t] < max_ctx, 0 <= q_seq[t] <
 *    num_seqs, cache scales finite and >= 0, index entries in [0, max_ctx) or -1.  The kernels
 *    clamp positions and sequence ids and skip out-of-range indices so that a violation never
 *    reads outside the given buffers, but the results of such a call are unspecified.
 *  - Keys visible to a query at 0-based position p are cache rows 0..p of its sequence (its own
 *    key is already in the cache).  Index lists hold row numbers within the query's sequence.
 */
#ifndef DSA_H_
#define DSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DSA_OK = 0,
  DSA_ERR_ARG = 1,          /* a null pointer, a bad size or an inconsistent argument        */
  DSA_ERR_UNSUPPORTED = 2,  /* well-formed but outside what the kernels implement            */
  DSA_ERR_HIP = 3           /* the HIP runtime reported an error while launching             */
} dsa_status_t;

typedef enum {
  DSA_F32 = 0,              /* IEEE binary32                                                  */
  DSA_BF16 = 1,             /* bfloat16, stored as 16-bit patterns                            */
  DSA_FP8_E4M3FN = 2        /* OCP FP8 E4M3FN bytes (bias 7, max 448, no infinities)          */
} dsa_dtype_t;

/* Text of the last failure on the calling thread ("" after a success).  Owned by the library. */
const char* dsa_last_error(void);

/* ABI version of this header (bumped on any incompatible change). */
int32_t dsa_abi_version(void);
#define DSA_ABI_VERSION 3

/* ============================================================================================
 * Paged caches
 * --------------------------------------------------------------------------------------------
 * "Day 0 support for Mistral Large 4 on vLLM", "ROCm implementation details", "DSA indexer on
 * AITER": the index-key cache is kept in cache blocks, the keys of a block stored in 16x16 tiles,
 * and one layout rule is shared by the writer and every reader.  Here that rule is:
 *
 *   A paged cache is a pool of num_blocks blocks of page_size tokens.  Token p of sequence b lives
 *   in block k = block_table[b * blocks_per_seq + p / page_size], row i = p % page_size, and its
 *   pool slot is k * page_size + i.
 *   Index keys: byte d (0..127) of the FP8 key of slot s (block k, row i) is at byte
 *       k * page_size * 128 + 256 * (8 * (i / 16) + d / 16) + 16 * (i % 16) + d % 16
 *     of k_cache: tiles of 16 tokens x 16 bytes, the 8 tiles of a 16-token group side by side (so
 *     each 32-token group of a block is one contiguous 4 KiB range); its scale is k_scale[s].
 *   Latent rows: kv_cache[s][0..576) and kv_scale[s][0..9) (whole rows: the sparse attention
 *     gathers one row per selected token).
 *
 * Entry points that take `const dsa_paging_t* paging` read (or write) contiguous caches
 * [num_seqs][max_ctx] when it is NULL, and the pool through the rule above otherwise; the caches
 * then hold num_blocks * page_size rows, and num_seqs / max_ctx keep describing the sequences.
 * page_size is a multiple of 32 in [32, 8192]; blocks_per_seq * page_size >= max_ctx; FP8 caches
 * only.  The table is device data the host does not read: kernels clamp each entry into
 * [0, num_blocks), so a bad entry reads or writes another block of the pool, never outside it.
 * dsa_paged_slots writes slot[j] for (seq[j], pos[j]) by the same rule (for the cache writers,
 * which take slots); pos[j] < 0 gives -1 (the writers skip it).
 * ==========================================================================================*/
typedef struct {
  const int32_t* block_table;   /* [num_seqs][blocks_per_seq] i32, device                          */
  int32_t page_size;            /* tokens per block                                                */
  int32_t blocks_per_seq;       /* table columns                                                   */
  int32_t num_blocks;           /* blocks in the pool                                              */
  int32_t num_seqs;             /* table rows                                                      */
} dsa_paging_t;

dsa_status_t dsa_paged_slots(const dsa_paging_t* paging, int32_t n, const int32_t* seq, const int32_t* pos,
                             int64_t* slot, void* stream);

/* ============================================================================================
 * 1. Lightning-indexer scores
 * --------------------------------------------------------------------------------------------
 * Defined by "mistral-large4.md", "What differs from GLM-5.2", bullets "The indexer", "SSMax"
 * and "RoPE and the rest".  For query t at position p = q_pos[t] in sequence b = q_seq[t]:
 *
 *   q'_h  = m_h * RoPE_p(q[t][h])             m_h = s_h * ln(p + 1) + b_h   (SSMax)
 *           RoPE_p rotates pairs (2j, 2j+1), j < rope_dim/2, by the angle p * inv_freq[j]
 *   S(i)  = sum_h (w[t][h] / sqrt(H)) * max(0, q'_h . k_i / sqrt(head_dim)),   i = 0..p
 *   k_i   = key row i of sequence b, times its per-token scale for fp8 keys
 *
 * Arguments
 *   q        [num_q][num_heads][head_dim]  q_dtype (F32 or BF16)
 *   w        [num_q][num_heads] f32        weights_proj(x) per head
 *   q_seq    [num_q] i32                   sequence of each query
 *   q_pos    [num_q] i32                   0-based position of each query
 *   ssmax_s, ssmax_b  [num_heads] f32      per-head SSMax parameters; both NULL = no SSMax
 *   inv_freq [rope_dim/2] f32              rotary frequencies; NULL iff rope_dim == 0
 *   k_cache  [num_seqs][max_ctx][head_dim] k_dtype (F32, or FP8_E4M3FN bytes)
 *   k_scale  [num_seqs][max_ctx] f32       per-token key scale (FP8 keys; NULL for F32 keys)
 *   scores   [num_q][ld_scores] f32        row t gets S(0..p); entries past p are not written
 *   ld_scores >= max_ctx
 *   ws       device workspace of at least dsa_indexer_workspace_size(desc) bytes, 16-byte
 *            aligned: the queries prepared once each (about 20 KiB per query) on the fp32-key
 *            path and, on the fp8 path, from 256 queries or two queries per sequence on (chunked
 *            prefill, multi-token verify blocks: four consecutive queries of one sequence then
 *            share one key stream, or eight when the sequences average 16 or more queries);
 *            0 bytes otherwise (the fp8 decode kernel prepares its query while its first key
 *            tiles are in flight), and then ws may be NULL.
 *   paging   NULL, or the paged layout of k_cache / k_scale (see "Paged caches").
 *
 * Supported: head_dim == 128; 1 <= num_heads <= 32; rope_dim in {0, 64}; q_dtype F32 or BF16;
 * k_dtype F32 (fp32 vector path) or FP8_E4M3FN (matrix-core path).  Both paths form the rotary
 * angles p * inv_freq[j] exactly and reduce them to [-pi, pi] in float64, then evaluate sine,
 * cosine, the SSMax factor and the rotation in float32 (about 1e-7 relative).  The FP8 path
 * splits q' into two fp16 terms (22 significant bits) and accumulates in fp32; its scores agree
 * with the real-number definition to about 1e-6 of the score scale.
 * ==========================================================================================*/
typedef struct {
  int32_t num_q;       /* T: query tokens                                                   */
  int32_t num_heads;   /* H: index heads (32 on Mistral Large 4; 4 in the block-sparse scan) */
  int32_t head_dim;    /* 128                                                                */
  int32_t rope_dim;    /* 64 on RoPE layers, 0 on NoPE layers                               */
  int32_t num_seqs;    /* B: sequences in the cache                                         */
  int32_t max_ctx;     /* rows per sequence in the cache                                     */
  dsa_dtype_t q_dtype;
  dsa_dtype_t k_dtype;
} dsa_indexer_desc_t;

size_t dsa_indexer_workspace_size(const dsa_indexer_desc_t* desc);
dsa_status_t dsa_indexer_scores(const dsa_indexer_desc_t* desc, const void* q, const float* w,
                                const int32_t* q_seq, const int32_t* q_pos,
                                const float* ssmax_s, const float* ssmax_b, const float* inv_freq,
                                const void* k_cache, const float* k_scale,
                                float* scores, int64_t ld_scores,
                                void* ws, size_t ws_bytes, void* stream,
                                const dsa_paging_t* paging);

/* ============================================================================================
 * 2a. Top-k selection
 * --------------------------------------------------------------------------------------------
 * Keep the k highest scores of each row ("the top 2048 keys kept": "mistral-large4.md", bullet
 * "The indexer"; top-k 2048 in the vLLM page's architecture table).  Row t has n = q_pos[t]+1
 * valid scores (columns 0..n-1 of scores[t]).
 *   - n <= k: every column is selected.
 *   - otherwise the k largest are selected; equal scores go to the lower column; -0.0 == +0.0.
 *   - idx[t][0..len) lists the selected columns in ascending order, idx[t][len..k) = -1, and
 *     len[t] = min(n, k) (the -1 slots and top-k length of the vLLM page's "Top-k compaction").
 * Scores must not be NaN.  Selection is exact: it depends only on the fp32 score values.
 *
 * Arguments
 *   scores   [num_q][ld_scores] f32;  q_pos [num_q] i32 (n = q_pos + 1, clamped to ld_scores)
 *   idx      [num_q][k] i32;          len [num_q] i32 (may be NULL)
 *   ws       device workspace of at least dsa_topk_workspace_size(num_q, ld_scores, k) bytes,
 *            16-byte aligned (about 148 KiB per query: the row's first-digit histogram and the
 *            keys that survive it).  With many rows (128 or more) dsa_topk selects each row in one
 *            kernel (two passes over the row, the candidates kept on chip) and only clears the
 *            workspace rows; with fewer, and on the fused and split calls below, the workspace
 *            carries the rows' histograms and candidates between kernels.  Its contents never decide a
 *            selection: the histogram only steers a fast path whose premise (the k-th largest key
 *            lies in the bin it names) is checked against the scores themselves, and rows that
 *            fail the check are selected by exact passes over the row.  Every call clears what it
 *            used, so a workspace that is zero-filled once (hipMemset) keeps every call on the
 *            fast path; stale or random contents cost one slower call, never a wrong one.  Calls
 *            that overlap in time must not share a workspace.
 * Supported: 1 <= k <= 65536; ld_scores <= 4194304 and a multiple of 4; scores 16-byte aligned.
 * ==========================================================================================*/
dsa_status_t dsa_topk(const float* scores, int64_t ld_scores, const int32_t* q_pos, int32_t num_q,
                      int32_t k, int32_t* idx, int32_t* len, void* ws, size_t ws_bytes, void* stream);

/* Scores and top-k in one call: dsa_indexer_scores followed by dsa_topk, with the first radix
 * digit's histogram built inside the fp8 decode score kernel and each score chunk's candidates
 * emitted by it (the scores are still written to `scores`); scores from the grouped or fp32 score
 * kernels are selected as dsa_topk does.
 * Same arguments, conventions and results as the two calls made in sequence, except that a row
 * holds min(q_pos + 1, max_ctx) scores (the score kernel's clamp).  `topk_ws` follows dsa_topk's
 * workspace rules. */
size_t dsa_topk_workspace_size(int32_t num_q, int64_t ld_scores, int32_t k);
dsa_status_t dsa_indexer_topk(const dsa_indexer_desc_t* desc, const void* q, const float* w,
                              const int32_t* q_seq, const int32_t* q_pos,
                              const float* ssmax_s, const float* ssmax_b, const float* inv_freq,
                              const void* k_cache, const float* k_scale,
                              float* scores, int64_t ld_scores, int32_t k, int32_t* idx, int32_t* len,
                              void* ws, size_t ws_bytes, void* topk_ws, size_t topk_ws_bytes, void* stream,
                              const dsa_paging_t* paging);

/* The two halves of dsa_indexer_topk as separate calls, for callers that schedule or time the
 * score stream and the selection apart.  dsa_indexer_scores_hist writes the scores (as
 * dsa_indexer_scores) and leaves each row's first-radix-digit histogram in `topk_ws` (built inside
 * the fp8 score kernel, else by a histogram pass after it); dsa_topk_hist then selects k columns of
 * each row from those scores and that histogram and leaves the workspace zeroed.  Issued back to
 * back with the same arguments they give exactly dsa_indexer_topk's results (rows hold
 * min(q_pos + 1, max_ctx) scores).  dsa_topk_hist is meant to follow a dsa_indexer_scores_hist call
 * on the same scores and workspace with the same k.  If it does not (the histogram is missing,
 * doubled, left by an interrupted call or built for another k), its selection is still exact: the
 * rows whose histogram does not match their scores are selected by exact passes over the row. */
dsa_status_t dsa_indexer_scores_hist(const dsa_indexer_desc_t* desc, const void* q, const float* w,
                                     const int32_t* q_seq, const int32_t* q_pos,
                                     const float* ssmax_s, const float* ssmax_b, const float* inv_freq,
                                     const void* k_cache, const float* k_scale,
                                     float* scores, int64_t ld_scores, int32_t k,
                                     void* ws, size_t ws_bytes, void* topk_ws, size_t topk_ws_bytes, void* stream,
                                     const dsa_paging_t* paging);
dsa_status_t dsa_topk_hist(const dsa_indexer_desc_t* desc, const float* scores, int64_t ld_scores,
                           const int32_t* q_pos, int32_t k, int32_t* idx, int32_t* len,
                           void* topk_ws, size_t topk_ws_bytes, void* stream);

/* ============================================================================================
 * 2b. Block-sparse selection
 * --------------------------------------------------------------------------------------------
 * The MiniMax Sparse Attention steps ("vLLM adds NVFP4 serving for MiniMax M3.1 Flash at 76
 * concurrent sequences"): the cache is cut into `block`-token blocks; a block's score is the
 * largest index score among its visible keys; the block holding the query position (the most
 * recent one) is always kept and the other nblocks-1 are the best of the rest (ties to the
 * lower block); the selection is every visible key of the kept blocks, ascending.
 *   idx [num_q][topk] i32 (-1 padded), len [num_q] i32 (may be NULL).
 * Supported: block in [1, 4096], nblocks >= 1, nblocks * block <= topk, nblocks <= 64.
 * ==========================================================================================*/
size_t dsa_block_select_workspace_size(int32_t num_q, int64_t ld_scores, int32_t block);
dsa_status_t dsa_block_select(const float* scores, int64_t ld_scores, const int32_t* q_pos,
                              int32_t num_q, int32_t block, int32_t nblocks, int32_t topk,
                              int32_t* idx, int32_t* len, void* ws, size_t ws_bytes, void* stream);

/* Scores and block selection in one call: dsa_indexer_scores, then dsa_block_select over the
 * scores, with the same arguments and results (scores written as dsa_indexer_scores writes them).
 * bs_ws is dsa_block_select's workspace (dsa_block_select_workspace_size(num_q, ld_scores, block)
 * bytes); it receives each block's maximum.  On the fp8 decode path (fewer than two queries per
 * sequence) with block a multiple of 32 that divides the score kernel's chunk (4096 keys, or
 * 1024 when the query count is small; 128 always does), the score kernel writes the maxima itself
 * and the selection never reads the scores back; otherwise a separate pass takes them.  On that
 * path `scores` may be NULL: the selection needs only the maxima, and no score row is written (the
 * stores, 4 bytes per key mixed into the key stream, cost the score kernel about 12 % of its
 * time); ld_scores then only sizes the rows of bs_ws.  NULL elsewhere is an error. */
dsa_status_t dsa_indexer_block_select(const dsa_indexer_desc_t* desc, const void* q, const float* w,
                                      const int32_t* q_seq, const int32_t* q_pos,
                                      const float* ssmax_s, const float* ssmax_b, const float* inv_freq,
                                      const void* k_cache, const float* k_scale, float* scores, int64_t ld_scores,
                                      int32_t block, int32_t nblocks, int32_t topk, int32_t* idx, int32_t* len,
                                      void* ws, size_t ws_bytes, void* bs_ws, size_t bs_ws_bytes, void* stream,
                                      const dsa_paging_t* paging);

/* ============================================================================================
 * 3. Sparse MLA (absorbed form, V = latent)
 * --------------------------------------------------------------------------------------------
 * For query t and head g over the selected rows r in idx[t][0..len[t]) (entries < 0 skipped):
 *   z_r  = softmax_scale * (q[t][g][0:kv_lora] . c_r[0:kv_lora]
 *                           + q[t][g][kv_lora:kv_lora+rope_dim] . c_r[kv_lora:kv_lora+rope_dim])
 *   out[t][g] = sum_r softmax(z)_r * c_r[0:kv_lora],   lse[t][g] = ln sum_r exp(z_r)
 * ("Day 0 support for Mistral Large 4 on vLLM": MLA with KV LoRA rank 512 and RoPE dim 64,
 * one latent KV head shared by all heads; NoPE layers are the same with zero RoPE dims on the
 * same cache layout.)  q arrives final: SSMax and RoPE of the MLA query are applied upstream.
 * A query with no selected row gets out = 0 and lse = -inf.
 *
 * Arguments
 *   q        [num_q][num_heads][kv_lora + rope_dim]  q_dtype
 *   kv       [num_seqs][max_ctx][kv_lora + 64]       kv_dtype (the row is 576 wide on every layer)
 *   kv_scale [num_seqs][max_ctx][(kv_lora+64)/kv_scale_block] f32 for FP8, NULL for F32
 *   q_seq    [num_q] i32;  idx [num_q][topk] i32;  len [num_q] i32 or NULL (then -1 ends a list)
 *   out      [num_q][num_heads][kv_lora] f32;        lse [num_q][num_heads] f32 or NULL
 *   ws       workspace of dsa_sparse_mla_workspace_size(desc) bytes (0 is allowed when the
 *            query count alone fills the GPU and no split is needed)
 *   paging   NULL, or the paged layout of kv / kv_scale (see "Paged caches"; FP8 path only, the
 *            pool below 2^32 bytes of latent rows)
 * Decode queries of one sequence that are consecutive and equally many per sequence (2..8, the
 * tokens of a multi-token verify block) run on one XCD, next to each other, so that the latent
 * rows their selections share are gathered through one L2.
 * Supported: num_heads a multiple of 16 up to 128; kv_lora == 512; rope_dim in {0, 64};
 * kv_scale_block == 64; (q F32, kv F32) on the fp32 path, (q BF16, kv FP8) on the matrix-core
 * path (fp8 x scale rounded to bf16, bf16 probabilities, fp32 accumulation).
 *
 * _decode splits each query's selection over several workgroups (split-K with an exact
 * log-sum-exp merge) so that a handful of queries still fills the GPU; _prefill gives each
 * query one workgroup (chunked prefill: thousands of queries).  Both compute the same values.
 * ==========================================================================================*/
typedef struct {
  int32_t num_q;            /* T                                                             */
  int32_t num_heads;        /* 64                                                            */
  int32_t kv_lora;          /* 512                                                           */
  int32_t rope_dim;         /* 64 (RoPE layer) or 0 (NoPE layer)                             */
  int32_t num_seqs;         /* B                                                             */
  int32_t max_ctx;          /* rows per sequence                                             */
  int32_t topk;             /* width of an index row (2048)                                  */
  dsa_dtype_t q_dtype;
  dsa_dtype_t kv_dtype;
  int32_t kv_scale_block;   /* 64                                                            */
  float softmax_scale;      /* 1/sqrt(192) on RoPE layers, 1/sqrt(128) on NoPE layers        */
  int32_t num_splits;       /* decode only: 0 = choose automatically, else 1..64             */
} dsa_mla_desc_t;

size_t dsa_sparse_mla_workspace_size(const dsa_mla_desc_t* desc);
dsa_status_t dsa_sparse_mla_decode(const dsa_mla_desc_t* desc, const void* q, const void* kv,
                                   const float* kv_scale, const int32_t* q_seq, const int32_t* idx,
                                   const int32_t* len, float* out, float* lse,
                                   void* ws, size_t ws_bytes, void* stream,
                                   const dsa_paging_t* paging);
dsa_status_t dsa_sparse_mla_prefill(const dsa_mla_desc_t* desc, const void* q, const void* kv,
                                    const float* kv_scale, const int32_t* q_seq, const int32_t* idx,
                                    const int32_t* len, float* out, float* lse,
                                    void* ws, size_t ws_bytes, void* stream,
                                    const dsa_paging_t* paging);

/* Sparse MLA decode that allocates nothing, for callers that cannot allocate device memory or
 * size a workspace: code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  The same computation, kernels and results as dsa_sparse_mla_decode, with the split
 * partials kept in a scratch buffer the library holds on each GPU for the life of the process
 * (dsa_sparse_mla_noalloc_max_bytes() bytes, 64 MiB; it is looked up on a device's first call).
 * A call whose partials need more (dsa_sparse_mla_workspace_size(desc) above that; about 4 * 514 *
 * num_heads bytes per query and split, e.g. 256 query-splits of 64 heads = 33.7 MB) returns
 * DSA_ERR_UNSUPPORTED before launching anything.  Every call on a GPU shares that GPU's buffer:
 * calls that overlap in time on one GPU (other streams, other threads) race and give undefined
 * results; calls in stream order do not.  The buffer is fully rewritten before it is read, so no
 * call depends on what an earlier one left in it.  No hipMalloc, hipFree or other allocation. */
size_t dsa_sparse_mla_noalloc_max_bytes(void);
dsa_status_t dsa_sparse_mla_decode_noalloc(const dsa_mla_desc_t* desc, const void* q, const void* kv,
                                           const float* kv_scale, const int32_t* q_seq, const int32_t* idx,
                                           const int32_t* len, float* out, float* lse, void* stream,
                                           const dsa_paging_t* paging);

/* ============================================================================================
 * 0. Cache writers
 * --------------------------------------------------------------------------------------------
 * Indexer key ("mistral-large4.md", "What differs from GLM-5.2", bullet "The indexer";
 * "Day 0 support for Mistral Large 4 on vLLM", "ROCm implementation details", "DSA indexer on
 * AITER": the key is quantised to FP8 with one scale per token and written straight into the
 * index cache, in the layout its readers use).  For token t with hidden state x[t]:
 *
 *   y     = wk . x[t]                                  (128 outputs; wk is [128][hidden])
 *   k     = (y - mean(y)) / sqrt(var(y) + eps) * ln_w + ln_b     (var: mean squared deviation)
 *   k     = RoPE_p(k) on RoPE layers: pairs (2j, 2j+1), j < 32, rotated by p * inv_freq[j],
 *           p = pos[t]
 *   scale = max|k| / 448 (1 if k = 0);  code_i = E4M3FN(k_i / scale), round to nearest even,
 *           saturated to +-448
 *   k_cache[slot[t]][0..128) = codes, k_scale[slot[t]] = scale
 *
 * Arguments (device pointers unless noted)
 *   desc     host descriptor below
 *   x        [num_tokens][ld_x] BF16, 16-byte aligned     hidden states
 *   wk       [128][hidden] BF16, 16-byte aligned          key projection weight (output dim first)
 *   ln_w     [128] f32;  ln_b [128] f32 or NULL (no bias)
 *   pos      [num_tokens] i32;  inv_freq [32] f32 (RoPE layers; ignored when rope_dim = 0)
 *   slot     [num_tokens] i64  destination row; in the readers' contiguous layout
 *            seq * max_ctx + position, in a paged cache the token's pool slot (dsa_paged_slots).
 *            A negative slot (padding token) or one >= num_slots is skipped.
 *   paging   NULL (k_cache rows are 128 contiguous bytes per slot) or the paged layout: the key
 *            bytes of a slot go to their 16x16 tiles (see "Paged caches"; num_slots is then
 *            num_blocks * page_size).
 *   k_cache  [num_slots][128] E4M3FN bytes, 2-byte aligned;  k_scale [num_slots] f32 (the index cache and its
 *            per-token scales as dsa_indexer_scores reads them)
 *   ws       workspace of dsa_index_k_insert_workspace_size(desc) bytes, 16-byte aligned
 *            (partial projections; its contents need not be initialised)
 * Supported: hidden a multiple of 32; rope_dim 0 or 64.  Rows whose slot is not written keep
 * their contents.  Two tokens with the same slot race (either row may remain).
 * ==========================================================================================*/
typedef struct {
  int32_t num_tokens;       /* T                                                             */
  int32_t hidden;           /* width of x and wk rows (6144 on Mistral Large 4)              */
  int64_t ld_x;             /* row stride of x in elements, >= hidden, a multiple of 8       */
  int32_t rope_dim;         /* 64 (RoPE layer) or 0 (NoPE layer)                             */
  float eps;                /* LayerNorm epsilon                                             */
  int64_t num_slots;        /* rows of k_cache                                               */
} dsa_index_k_desc_t;

size_t dsa_index_k_insert_workspace_size(const dsa_index_k_desc_t* desc);
dsa_status_t dsa_index_k_insert(const dsa_index_k_desc_t* desc, const void* x, const void* wk,
                                const float* ln_w, const float* ln_b, const int32_t* pos,
                                const float* inv_freq, const int64_t* slot, uint8_t* k_cache,
                                float* k_scale, void* ws, size_t ws_bytes, void* stream,
                                const dsa_paging_t* paging);

/* Latent row ("Day 0 support for Mistral Large 4 on vLLM", "Model architecture": 512 latent
 * dims and 64 rotary dims per token; "ROCm implementation details", "FP8 latent cache": the row
 * is stored as E4M3 codes).  For token t, row r = kv[t][0..576):
 *   r[512..576) rotated at p = pos[t] on RoPE layers (pairs (512+2j, 512+2j+1) by p * inv_freq[j]);
 *   on NoPE layers (rope_dim = 0) the row is stored as given (the readers ignore that slice);
 *   per 64-element group g: scale_g = max|r_g| / 448 (1 if 0), codes as for the key;
 *   kv_cache[slot[t]][0..576) = codes, kv_scale[slot[t]][g] = scale_g.
 * The latent part arrives final (any normalisation of it is applied upstream).
 *   kv       [num_tokens][ld_kv] BF16 (ld_kv >= 576, a multiple of 8), 16-byte aligned;
 *            pos, inv_freq, slot as above
 *   kv_cache [num_slots][576] E4M3FN bytes, 8-byte aligned;  kv_scale [num_slots][9] f32 (the latent cache as
 *            dsa_sparse_mla_decode / _prefill read it, with kv_scale_block = 64)
 * No workspace.  Skipped slots and races as above.
 * ==========================================================================================*/
dsa_status_t dsa_latent_insert(int32_t num_tokens, int32_t rope_dim, const void* kv, int64_t ld_kv,
                               const int32_t* pos, const float* inv_freq, const int64_t* slot,
                               int64_t num_slots, uint8_t* kv_cache, float* kv_scale, void* stream);

/* ============================================================================================
 * Kernel timing (measurement, not serving)
 * --------------------------------------------------------------------------------------------
 * For benchmarks that need each kernel's own duration inside a running pipeline without adding
 * work to the stream.  After dsa_timing_begin(events, capacity), each kernel the library enqueues
 * (from any entry point, on any stream) takes the next pair events[2i], events[2i+1] as its start
 * and stop events (hipExtLaunchKernel's: the timestamps of the kernel's own dispatch, no marker
 * packets), until `capacity` kernels have taken one; later kernels are enqueued untimed.
 *   events   2 * capacity hipEvent_t handles, created by the caller (timing enabled), which must
 *            stay valid until the stream has passed the last timed kernel; read them with
 *            hipEventElapsedTime after synchronising.
 * dsa_timing_end() disarms the hook and returns how many kernels took a pair;
 * dsa_timing_kernel_name(i) names the kernel of pair i (owned by the runtime; NULL if i is out
 * of range).  The hook is process-wide state: arm it from the thread that enqueues the work and
 * do not call the library from other threads meanwhile.  Returns DSA_ERR_ARG for a NULL array
 * or capacity < 1 or > 65536.
 * ==========================================================================================*/
dsa_status_t dsa_timing_begin(void* const* events, int32_t capacity);
int32_t dsa_timing_end(void);
const char* dsa_timing_kernel_name(int32_t i);

#ifdef __cplusplus
}
#endif
#endif /* DSA_H_ */
