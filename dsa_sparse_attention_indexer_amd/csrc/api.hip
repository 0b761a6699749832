// C ABI of libdsa: argument validation (default-deny: every violated condition is reported and
// nothing is launched) and dispatch to the gfx950 kernels.  See include/dsa.h for the contract.

#include "topk_common.h"

#include <stdarg.h>
#include <stdio.h>
#include <mutex>
#include <vector>
#include <string>

namespace {

thread_local std::string g_err;

struct Checker {
  std::string msg;
  bool unsupported = false;
  bool arg = false;
  void fail(bool is_arg, const char* fmt, ...) {
    char buf[256];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    if (!msg.empty()) msg += "; ";
    msg += buf;
    if (is_arg) arg = true; else unsupported = true;
  }
  void need(bool ok, const char* what) { if (!ok) fail(true, "%s", what); }
  void support(bool ok, const char* what) { if (!ok) fail(false, "%s", what); }
  dsa_status_t finish(const char* fn) {
    if (msg.empty()) { g_err.clear(); return DSA_OK; }
    g_err = std::string(fn) + ": " + msg;
    return arg ? DSA_ERR_ARG : DSA_ERR_UNSUPPORTED;
  }
};

dsa_status_t hip_status(const char* fn, hipError_t e) {
  if (e == hipSuccess) { g_err.clear(); return DSA_OK; }
  g_err = std::string(fn) + ": HIP launch failed: " + hipGetErrorString(e);
  return DSA_ERR_HIP;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace

// Kernel timing hook state (dsa_timing_begin / _end).
struct TimingHook {
  std::mutex mu;
  void* const* events = nullptr;
  int cap = 0, used = 0;
  std::vector<const void*> fns;
};
static TimingHook g_timing;

namespace dsa {
bool timing_take(const void* fn, hipEvent_t* start, hipEvent_t* stop) {
  std::lock_guard<std::mutex> lk(g_timing.mu);
  if (!g_timing.events || g_timing.used >= g_timing.cap) return false;
  const int i = g_timing.used++;
  g_timing.fns[(size_t)i] = fn;
  *start = (hipEvent_t)g_timing.events[2 * i];
  *stop = (hipEvent_t)g_timing.events[2 * i + 1];
  return true;
}
}  // namespace dsa

extern "C" {

const char* dsa_last_error(void) { return g_err.c_str(); }

int32_t dsa_abi_version(void) { return DSA_ABI_VERSION; }

dsa_status_t dsa_timing_begin(void* const* events, int32_t capacity) {
  Checker ck;
  ck.need(events != nullptr, "events is NULL");
  ck.need(capacity >= 1 && capacity <= 65536, "capacity must be in [1, 65536]");
  dsa_status_t st = ck.finish("dsa_timing_begin");
  if (st != DSA_OK) return st;
  std::lock_guard<std::mutex> lk(g_timing.mu);
  g_timing.events = events;
  g_timing.cap = capacity;
  g_timing.used = 0;
  g_timing.fns.assign((size_t)capacity, nullptr);
  return DSA_OK;
}

int32_t dsa_timing_end(void) {
  std::lock_guard<std::mutex> lk(g_timing.mu);
  g_timing.events = nullptr;
  return g_timing.used;
}

const char* dsa_timing_kernel_name(int32_t i) {
  std::lock_guard<std::mutex> lk(g_timing.mu);
  if (i < 0 || i >= g_timing.used || (size_t)i >= g_timing.fns.size()) return nullptr;
  return hipKernelNameRefByPtr(g_timing.fns[(size_t)i], nullptr);
}

size_t dsa_indexer_workspace_size(const dsa_indexer_desc_t* d) {
  if (!d || d->num_q <= 0) return 0;
  return dsa::indexer_ws_bytes(d->num_q, d->num_seqs, d->k_dtype);
}

}  // extern "C"

namespace {

// The paged layout's host conditions (the header's "Paged caches"); NULL = contiguous caches.
dsa::Paging check_paging(Checker& ck, const dsa_paging_t* pg, int32_t num_seqs, int32_t max_ctx, bool fp8) {
  if (!pg) return dsa::Paging{nullptr, 0, 0, 0};
  ck.support(fp8, "paged caches are FP8 only");
  ck.need(pg->block_table != nullptr, "paging->block_table must be non-NULL");
  ck.support(pg->page_size >= 32 && pg->page_size <= 8192 && pg->page_size % 32 == 0,
             "paging->page_size must be a multiple of 32 in [32, 8192]");
  ck.need(pg->blocks_per_seq >= 1, "paging->blocks_per_seq must be >= 1");
  ck.need(pg->num_blocks >= 1, "paging->num_blocks must be >= 1");
  ck.need(pg->num_seqs == num_seqs, "paging->num_seqs must equal the descriptor's num_seqs");
  ck.need((int64_t)pg->blocks_per_seq * pg->page_size >= max_ctx, "paging: blocks_per_seq * page_size must be >= max_ctx");
  ck.need((int64_t)pg->num_blocks * pg->page_size <= ((int64_t)1 << 31) - 1, "paging: the pool must hold < 2^31 rows");
  return dsa::Paging{pg->block_table, pg->page_size, pg->blocks_per_seq, pg->num_blocks};
}

void check_indexer(Checker& ck, const dsa_indexer_desc_t* d, const void* q, const float* w, const int32_t* q_seq,
                   const int32_t* q_pos, const float* ssmax_s, const float* ssmax_b, const float* inv_freq,
                   const void* k_cache, const float* k_scale, const float* scores, int64_t ld_scores, const void* ws,
                   size_t ws_bytes, bool scores_optional = false) {
  ck.need(d->num_q >= 0 && d->num_q <= 65535, "num_q must be in [0, 65535]");
  ck.need(d->num_seqs >= 1, "num_seqs must be >= 1");
  ck.need(d->max_ctx >= 1 && d->max_ctx <= (1 << 26), "max_ctx must be in [1, 2^26]");
  ck.support(d->head_dim == 128, "head_dim must be 128");
  ck.support(d->num_heads >= 1 && d->num_heads <= 32, "num_heads must be in [1, 32]");
  ck.support(d->rope_dim == 0 || d->rope_dim == 64, "rope_dim must be 0 or 64");
  ck.support(d->q_dtype == DSA_F32 || d->q_dtype == DSA_BF16, "q_dtype must be F32 or BF16");
  ck.support(d->k_dtype == DSA_F32 || d->k_dtype == DSA_FP8_E4M3FN, "k_dtype must be F32 or FP8_E4M3FN");
  ck.need(ld_scores >= d->max_ctx, "ld_scores must be >= max_ctx");
  if (d->num_q > 0) {
    ck.need(q && w && q_seq && q_pos && k_cache, "q, w, q_seq, q_pos and k_cache must be non-NULL");
    ck.need(scores || scores_optional, "scores must be non-NULL");
    ck.need((ssmax_s == nullptr) == (ssmax_b == nullptr), "ssmax_s and ssmax_b must be both NULL or both set");
    ck.need((inv_freq != nullptr) == (d->rope_dim > 0), "inv_freq must be set iff rope_dim > 0");
    ck.need(d->k_dtype != DSA_FP8_E4M3FN || k_scale != nullptr, "k_scale is required for FP8 keys");
    ck.need(aligned(k_cache, 16), "k_cache must be 16-byte aligned");
    ck.need(aligned(q, 16), "q must be 16-byte aligned");
    const size_t need = dsa_indexer_workspace_size(d);
    ck.need(need == 0 || (ws != nullptr && ws_bytes >= need && aligned(ws, 16)),
            "workspace missing, misaligned or smaller than dsa_indexer_workspace_size()");
  }
}

void check_topk(Checker& ck, int32_t num_q, int64_t ld_scores, int32_t k, const void* scores, const int32_t* q_pos,
                const int32_t* idx, bool with_idx = true) {
  ck.need(num_q >= 0 && num_q <= 65535, "num_q must be in [0, 65535]");
  ck.need(ld_scores >= 1, "ld_scores must be >= 1");
  ck.support(ld_scores <= dsa::kTopkMaxCols, "ld_scores must be <= 4194304");
  ck.need(ld_scores % 4 == 0, "ld_scores must be a multiple of 4");
  ck.support(k >= 1 && k <= 65536, "k must be in [1, 65536]");
  if (num_q > 0) {
    ck.need(scores && q_pos && (idx || !with_idx), with_idx ? "scores, q_pos and idx must be non-NULL"
                                                              : "scores and q_pos must be non-NULL");
    ck.need(aligned(scores, 16), "scores must be 16-byte aligned");
  }
}

void check_topk_ws(Checker& ck, int32_t num_q, const void* ws, size_t ws_bytes) {
  if (num_q <= 0) return;
  ck.need(ws != nullptr && ws_bytes >= dsa::topk_ws_bytes(num_q),
          "top-k workspace missing or smaller than dsa_topk_workspace_size()");
  ck.need(aligned(ws, 16), "top-k workspace must be 16-byte aligned");
}

dsa::IndexerLaunch indexer_launch(const dsa_indexer_desc_t* d, const void* q, const float* w, const int32_t* q_seq,
                                  const int32_t* q_pos, const float* ssmax_s, const float* ssmax_b,
                                  const float* inv_freq, const void* k_cache, const float* k_scale, float* scores,
                                  int64_t ld_scores) {
  return dsa::IndexerLaunch{d->num_q, d->num_heads, d->rope_dim, d->num_seqs, d->max_ctx, d->q_dtype, d->k_dtype,
                            q, w, q_seq, q_pos, ssmax_s, ssmax_b, inv_freq, k_cache, k_scale, scores, ld_scores,
                            nullptr, 0, 0, dsa::Paging{nullptr, 0, 0, 0}, nullptr, 0, 0};
}

}  // namespace

extern "C" {

dsa_status_t dsa_indexer_scores(const dsa_indexer_desc_t* d, const void* q, const float* w,
                                const int32_t* q_seq, const int32_t* q_pos,
                                const float* ssmax_s, const float* ssmax_b, const float* inv_freq,
                                const void* k_cache, const float* k_scale,
                                float* scores, int64_t ld_scores, void* ws, size_t ws_bytes, void* stream,
                                const dsa_paging_t* paging) {
  Checker ck;
  if (!d) { ck.need(false, "desc is NULL"); return ck.finish("dsa_indexer_scores"); }
  check_indexer(ck, d, q, w, q_seq, q_pos, ssmax_s, ssmax_b, inv_freq, k_cache, k_scale, scores, ld_scores, ws,
                ws_bytes);
  const dsa::Paging pg = check_paging(ck, paging, d->num_seqs, d->max_ctx, d->k_dtype == DSA_FP8_E4M3FN);
  dsa_status_t st = ck.finish("dsa_indexer_scores");
  if (st != DSA_OK || d->num_q == 0) return st;
  dsa::IndexerLaunch a = indexer_launch(d, q, w, q_seq, q_pos, ssmax_s, ssmax_b, inv_freq, k_cache, k_scale, scores,
                                        ld_scores);
  a.pg = pg;
  return hip_status("dsa_indexer_scores", dsa::launch_indexer(a, ws, (hipStream_t)stream));
}

dsa_status_t dsa_indexer_topk(const dsa_indexer_desc_t* d, const void* q, const float* w,
                              const int32_t* q_seq, const int32_t* q_pos,
                              const float* ssmax_s, const float* ssmax_b, const float* inv_freq,
                              const void* k_cache, const float* k_scale,
                              float* scores, int64_t ld_scores, int32_t k, int32_t* idx, int32_t* len,
                              void* ws, size_t ws_bytes, void* topk_ws, size_t topk_ws_bytes, void* stream,
                              const dsa_paging_t* paging) {
  Checker ck;
  if (!d) { ck.need(false, "desc is NULL"); return ck.finish("dsa_indexer_topk"); }
  check_indexer(ck, d, q, w, q_seq, q_pos, ssmax_s, ssmax_b, inv_freq, k_cache, k_scale, scores, ld_scores, ws,
                ws_bytes);
  const dsa::Paging pg = check_paging(ck, paging, d->num_seqs, d->max_ctx, d->k_dtype == DSA_FP8_E4M3FN);
  check_topk(ck, d->num_q, ld_scores, k, scores, q_pos, idx);
  check_topk_ws(ck, d->num_q, topk_ws, topk_ws_bytes);
  dsa_status_t st = ck.finish("dsa_indexer_topk");
  if (st != DSA_OK || d->num_q == 0) return st;
  dsa::IndexerLaunch a = indexer_launch(d, q, w, q_seq, q_pos, ssmax_s, ssmax_b, inv_freq, k_cache, k_scale, scores,
                                        ld_scores);
  a.pg = pg;
  // The decode score kernel builds the first digit's histogram, and its chunks emit their own
  // candidates when the row's chunks fit the segment table.  The grouped kernel (several queries
  // per sequence) only writes scores: its workgroups are bound by matrix work, and a per-chunk
  // selection tail there costs more than the separate passes over the scores.
  const bool fused = d->k_dtype == DSA_FP8_E4M3FN && !dsa::indexer_grouped(d->num_q, d->num_seqs, d->k_dtype);
  const int chunk = dsa::indexer_chunk(d->num_q, d->max_ctx);
  const bool emit = fused && k <= dsa::kTkFastK && (d->max_ctx + chunk - 1) / chunk <= dsa::kTkMaxSeg;
  if (fused) { a.topk_ws = topk_ws; a.topk_k = k; a.topk_emit = emit; }
  hipError_t e = dsa::launch_indexer(a, ws, (hipStream_t)stream);
  if (e != hipSuccess) return hip_status("dsa_indexer_topk", e);
  dsa::TopkLaunch tk{scores, ld_scores, d->max_ctx, q_pos, d->num_q, k, idx, len, topk_ws, emit ? chunk : 0, emit};
  // scores nobody histogrammed (grouped or fp32 score kernels): as dsa_topk
  if (fused) return hip_status("dsa_indexer_topk", dsa::launch_topk(tk, true, (hipStream_t)stream));
  return hip_status("dsa_indexer_topk", dsa::topk_direct_pays(d->num_q) ? dsa::launch_topk_direct(tk, (hipStream_t)stream)
                                                                         : dsa::launch_topk(tk, false, (hipStream_t)stream));
}

dsa_status_t dsa_indexer_scores_hist(const dsa_indexer_desc_t* d, const void* q, const float* w,
                                     const int32_t* q_seq, const int32_t* q_pos,
                                     const float* ssmax_s, const float* ssmax_b, const float* inv_freq,
                                     const void* k_cache, const float* k_scale,
                                     float* scores, int64_t ld_scores, int32_t k,
                                     void* ws, size_t ws_bytes, void* topk_ws, size_t topk_ws_bytes, void* stream,
                                     const dsa_paging_t* paging) {
  Checker ck;
  if (!d) { ck.need(false, "desc is NULL"); return ck.finish("dsa_indexer_scores_hist"); }
  check_indexer(ck, d, q, w, q_seq, q_pos, ssmax_s, ssmax_b, inv_freq, k_cache, k_scale, scores, ld_scores, ws,
                ws_bytes);
  const dsa::Paging pg = check_paging(ck, paging, d->num_seqs, d->max_ctx, d->k_dtype == DSA_FP8_E4M3FN);
  check_topk(ck, d->num_q, ld_scores, k, scores, q_pos, nullptr, false);   // no index output in this half
  check_topk_ws(ck, d->num_q, topk_ws, topk_ws_bytes);
  dsa_status_t st = ck.finish("dsa_indexer_scores_hist");
  if (st != DSA_OK || d->num_q == 0) return st;
  dsa::IndexerLaunch a = indexer_launch(d, q, w, q_seq, q_pos, ssmax_s, ssmax_b, inv_freq, k_cache, k_scale, scores,
                                        ld_scores);
  a.pg = pg;
  const bool fused = d->k_dtype == DSA_FP8_E4M3FN && !dsa::indexer_grouped(d->num_q, d->num_seqs, d->k_dtype);
  if (fused) { a.topk_ws = topk_ws; a.topk_k = k; }
  hipError_t e = dsa::launch_indexer(a, ws, (hipStream_t)stream);
  if (e != hipSuccess || fused) return hip_status("dsa_indexer_scores_hist", e);
  dsa::TopkLaunch tk{scores, ld_scores, d->max_ctx, q_pos, d->num_q, k, nullptr, nullptr, topk_ws, 0, 0};
  return hip_status("dsa_indexer_scores_hist", dsa::launch_topk_hist(tk, (hipStream_t)stream));
}

dsa_status_t dsa_topk_hist(const dsa_indexer_desc_t* d, const float* scores, int64_t ld_scores,
                           const int32_t* q_pos, int32_t k, int32_t* idx, int32_t* len,
                           void* topk_ws, size_t topk_ws_bytes, void* stream) {
  Checker ck;
  if (!d) { ck.need(false, "desc is NULL"); return ck.finish("dsa_topk_hist"); }
  ck.need(d->max_ctx >= 1 && d->max_ctx <= (1 << 26), "max_ctx must be in [1, 2^26]");
  ck.need(ld_scores >= d->max_ctx, "ld_scores must be >= max_ctx");
  check_topk(ck, d->num_q, ld_scores, k, scores, q_pos, idx);
  check_topk_ws(ck, d->num_q, topk_ws, topk_ws_bytes);
  dsa_status_t st = ck.finish("dsa_topk_hist");
  if (st != DSA_OK || d->num_q == 0) return st;
  dsa::TopkLaunch tk{scores, ld_scores, d->max_ctx, q_pos, d->num_q, k, idx, len, topk_ws, 0, 0};
  return hip_status("dsa_topk_hist", dsa::launch_topk(tk, true, (hipStream_t)stream));
}

size_t dsa_topk_workspace_size(int32_t num_q, int64_t ld_scores, int32_t k) {
  if (num_q <= 0 || ld_scores <= 0 || k <= 0) return 0;
  return dsa::topk_ws_bytes(num_q);
}

dsa_status_t dsa_topk(const float* scores, int64_t ld_scores, const int32_t* q_pos, int32_t num_q,
                      int32_t k, int32_t* idx, int32_t* len, void* ws, size_t ws_bytes, void* stream) {
  Checker ck;
  check_topk(ck, num_q, ld_scores, k, scores, q_pos, idx);
  check_topk_ws(ck, num_q, ws, ws_bytes);
  dsa_status_t st = ck.finish("dsa_topk");
  if (st != DSA_OK || num_q == 0) return st;
  dsa::TopkLaunch a{scores, ld_scores, ld_scores, q_pos, num_q, k, idx, len, ws, 0, 0};
  return hip_status("dsa_topk", dsa::topk_direct_pays(num_q) ? dsa::launch_topk_direct(a, (hipStream_t)stream)
                                                              : dsa::launch_topk(a, false, (hipStream_t)stream));
}

size_t dsa_block_select_workspace_size(int32_t num_q, int64_t ld_scores, int32_t block) {
  if (num_q <= 0 || ld_scores <= 0 || block <= 0) return 0;
  return dsa::block_select_ws_bytes(num_q, ld_scores, block);
}

dsa_status_t dsa_block_select(const float* scores, int64_t ld_scores, const int32_t* q_pos,
                              int32_t num_q, int32_t block, int32_t nblocks, int32_t topk,
                              int32_t* idx, int32_t* len, void* ws, size_t ws_bytes, void* stream) {
  Checker ck;
  ck.need(num_q >= 0 && num_q <= 65535, "num_q must be in [0, 65535]");
  ck.need(ld_scores >= 1 && ld_scores <= (int64_t(1) << 30), "ld_scores must be in [1, 2^30]");
  ck.support(block >= 1 && block <= 4096, "block must be in [1, 4096]");
  ck.support(nblocks >= 1 && nblocks <= 64, "nblocks must be in [1, 64]");
  ck.need(topk >= 1, "topk must be >= 1");
  ck.need((int64_t)nblocks * block <= topk, "nblocks * block must be <= topk");
  if (num_q > 0) {
    ck.need(scores && q_pos && idx, "scores, q_pos and idx must be non-NULL");
    ck.need(block <= 0 || (ws != nullptr && ws_bytes >= dsa_block_select_workspace_size(num_q, ld_scores, block)),
            "workspace missing or smaller than dsa_block_select_workspace_size()");
  }
  dsa_status_t st = ck.finish("dsa_block_select");
  if (st != DSA_OK || num_q == 0) return st;
  dsa::BlockSelectLaunch a{scores, ld_scores, q_pos, num_q, block, nblocks, topk, idx, len, ws};
  return hip_status("dsa_block_select", dsa::launch_block_select(a, (hipStream_t)stream));
}

dsa_status_t dsa_indexer_block_select(const dsa_indexer_desc_t* d, const void* q, const float* w,
                                      const int32_t* q_seq, const int32_t* q_pos,
                                      const float* ssmax_s, const float* ssmax_b, const float* inv_freq,
                                      const void* k_cache, const float* k_scale, float* scores, int64_t ld_scores,
                                      int32_t block, int32_t nblocks, int32_t topk, int32_t* idx, int32_t* len,
                                      void* ws, size_t ws_bytes, void* bs_ws, size_t bs_ws_bytes, void* stream,
                                      const dsa_paging_t* paging) {
  const char* fn = "dsa_indexer_block_select";
  Checker ck;
  if (!d) { ck.need(false, "desc is NULL"); return ck.finish(fn); }
  check_indexer(ck, d, q, w, q_seq, q_pos, ssmax_s, ssmax_b, inv_freq, k_cache, k_scale, scores, ld_scores, ws,
                ws_bytes, true);
  const dsa::Paging pg = check_paging(ck, paging, d->num_seqs, d->max_ctx, d->k_dtype == DSA_FP8_E4M3FN);
  ck.need(ld_scores <= (int64_t(1) << 30), "ld_scores must be <= 2^30");
  // the decode score kernel emits the block maxima itself where its chunks hold whole blocks; only
  // then can the scores be left unwritten
  const bool fused = block >= 1 && dsa::indexer_block_max_fused(d->num_q, d->num_seqs, d->max_ctx, d->k_dtype, block);
  ck.need(scores != nullptr || fused || d->num_q == 0,
          "scores may be NULL only on the fp8 decode path with block a multiple of 32 that divides the score chunk");
  ck.support(block >= 1 && block <= 4096, "block must be in [1, 4096]");
  ck.support(nblocks >= 1 && nblocks <= 64, "nblocks must be in [1, 64]");
  ck.need(topk >= 1, "topk must be >= 1");
  ck.need((int64_t)nblocks * block <= topk, "nblocks * block must be <= topk");
  if (d->num_q > 0) {
    ck.need(idx != nullptr, "idx must be non-NULL");
    ck.need(block <= 0 || (bs_ws != nullptr && bs_ws_bytes >= dsa_block_select_workspace_size(d->num_q, ld_scores, block)),
            "block workspace missing or smaller than dsa_block_select_workspace_size()");
  }
  dsa_status_t st = ck.finish(fn);
  if (st != DSA_OK || d->num_q == 0) return st;
  dsa::IndexerLaunch a = indexer_launch(d, q, w, q_seq, q_pos, ssmax_s, ssmax_b, inv_freq, k_cache, k_scale, scores,
                                        ld_scores);
  a.pg = pg;
  if (fused) {
    a.bmax = static_cast<uint32_t*>(bs_ws);
    a.bblock = block;
    a.bld = (ld_scores + block - 1) / block;
  }
  hipError_t e = dsa::launch_indexer(a, ws, (hipStream_t)stream);
  if (e != hipSuccess) return hip_status(fn, e);
  dsa::BlockSelectLaunch b{scores, ld_scores, q_pos, d->num_q, block, nblocks, topk, idx, len, bs_ws};
  return hip_status(fn, fused ? dsa::launch_block_pick(b, (hipStream_t)stream)
                              : dsa::launch_block_select(b, (hipStream_t)stream));
}

}  // extern "C"

namespace {

// Head split of the fp8 decode kernel: small batches (automatic splits, 64 heads, at most 32
// queries) run each query as two 32-head halves.  A workgroup then loads half the query, its split
// partials are half as large and twice as many keys go to each split, so the kernel's fixed costs
// (query load, first gathers, partial stores, the combine's reads) shrink while the tile loop stays
// about as long (each tile carries half the P.V work).
int mla_hsplit(const dsa_mla_desc_t* d, bool decode) {
  const bool fp8 = d->kv_dtype == DSA_FP8_E4M3FN;
  // (measured, 2048 keys per query: batch 8 24.8 -> 18.8 us, 16 27.8 -> 23.5, 32 34.8 -> 32.2; batch 4,
  // whose splits are single tiles either way, 24.3 -> 26.5: not split)
  return (fp8 && decode && d->num_splits == 0 && d->num_heads == 64 && d->num_q >= 8 && d->num_q <= 32) ? 2 : 1;
}

int auto_splits(const dsa_mla_desc_t* d, bool decode) {
  if (!decode) return 1;
  if (d->num_splits > 0) return d->num_splits;
  // As many workgroups as cover the 256 CUs once without a second round (the fp8 kernel's LDS holds
  // one workgroup per CU); each split keeps >= 64 selected keys (one tile of the fp8 kernel).
  const int nq = d->num_q * mla_hsplit(d, decode);   // (virtual) queries
  int s = 256 / (nq > 0 ? nq : 1);
  const int max_by_keys = (d->topk + 63) / 64;
  if (s > max_by_keys) s = max_by_keys;
  if (s > 64) s = 64;
  if (s < 1) s = 1;
  return s;
}

void split_geometry(const dsa_mla_desc_t* d, bool decode, int* splits, int* per_split) {
  if (d->topk < 1 || d->num_splits < 0) {   // an invalid descriptor (rejected by the caller's checks)
    *splits = 1;
    *per_split = 32;
    return;
  }
  int s = auto_splits(d, decode);
  int per = (d->topk + s - 1) / s;
  per = (per + 63) / 64 * 64;   // whole 64-key tiles per split
  s = (d->topk + per - 1) / per;
  if (s < 1) s = 1;
  *splits = s;
  *per_split = per;
}

size_t mla_ws_bytes(const dsa_mla_desc_t* d, bool decode) {
  int s, per;
  split_geometry(d, decode, &s, &per);
  if (s <= 1) return 0;
  // (with a head split: hs x num_q virtual queries of num_heads / hs heads, the same product)
  return (size_t)d->num_q * s * d->num_heads * ((size_t)d->kv_lora + 2) * sizeof(float);
}

dsa_status_t mla_call(const char* fn, bool decode, const dsa_mla_desc_t* d, const void* q, const void* kv,
                      const float* kv_scale, const int32_t* q_seq, const int32_t* idx, const int32_t* len,
                      float* out, float* lse, void* ws, size_t ws_bytes, void* stream, const dsa_paging_t* paging) {
  Checker ck;
  if (!d) { ck.need(false, "desc is NULL"); return ck.finish(fn); }
  ck.need(d->num_q >= 0 && d->num_q <= 65535, "num_q must be in [0, 65535]");
  ck.need(d->num_seqs >= 1, "num_seqs must be >= 1");
  ck.need(d->max_ctx >= 1 && d->max_ctx <= (1 << 26), "max_ctx must be in [1, 2^26]");
  ck.need(d->topk >= 1 && d->topk <= (1 << 20), "topk must be in [1, 2^20]");
  ck.support(d->kv_lora == 512, "kv_lora must be 512");
  ck.support(d->rope_dim == 0 || d->rope_dim == 64, "rope_dim must be 0 or 64");
  ck.support(d->kv_scale_block == 64, "kv_scale_block must be 64");
  ck.need(d->num_splits >= 0 && d->num_splits <= 64, "num_splits must be in [0, 64]");
  ck.need(d->softmax_scale > 0.f, "softmax_scale must be > 0");
  const bool fp8 = d->kv_dtype == DSA_FP8_E4M3FN;
  if (fp8) {
    ck.support(d->q_dtype == DSA_BF16, "the FP8 cache path takes BF16 queries");
    ck.support(d->num_heads >= 16 && d->num_heads <= 64 && d->num_heads % 16 == 0,
               "num_heads must be 16, 32, 48 or 64 on the FP8 path");
    // the kernel addresses a sequence's latent rows (a paged pool) with 32-bit byte offsets
    ck.support((uint64_t)d->max_ctx * 576 < (uint64_t(1) << 32), "max_ctx must be <= 7456540 on the FP8 path");
    ck.support(!paging || (uint64_t)paging->num_blocks * (uint64_t)paging->page_size * 576 < (uint64_t(1) << 32),
               "a paged latent pool must hold fewer than 7456540 rows");
  } else {
    ck.support(d->kv_dtype == DSA_F32, "kv_dtype must be F32 or FP8_E4M3FN");
    ck.support(d->q_dtype == DSA_F32, "the F32 cache path takes F32 queries");
    ck.support(d->num_heads >= 1 && d->num_heads <= 64, "num_heads must be in [1, 64] on the F32 path");
  }
  if (d->num_q > 0) {
    ck.need(q && kv && q_seq && idx && out, "q, kv, q_seq, idx and out must be non-NULL");
    ck.need(!fp8 || kv_scale != nullptr, "kv_scale is required for an FP8 cache");
    ck.need(aligned(q, 16) && aligned(kv, 16) && aligned(out, 16), "q, kv and out must be 16-byte aligned");
    const size_t need = mla_ws_bytes(d, decode);
    ck.need(need == 0 || (ws != nullptr && ws_bytes >= need && aligned(ws, 16)),
            "workspace missing, misaligned or smaller than dsa_sparse_mla_workspace_size()");
  }
  const dsa::Paging pg = check_paging(ck, paging, d->num_seqs, d->max_ctx, fp8);
  dsa_status_t st = ck.finish(fn);
  if (st != DSA_OK || d->num_q == 0) return st;
  dsa::MlaLaunch a{};
  a.pg = pg;
  a.pool_rows = pg.table ? (int64_t)pg.nblocks * pg.page : 0;
  a.hs = mla_hsplit(d, decode);
  a.T = d->num_q * a.hs; a.H = d->num_heads / a.hs; a.kv_lora = d->kv_lora; a.rope_dim = d->rope_dim;
  a.B = d->num_seqs; a.max_ctx = d->max_ctx; a.topk = d->topk;
  split_geometry(d, decode, &a.splits, &a.per_split);
  a.q_dtype = d->q_dtype; a.kv_dtype = d->kv_dtype; a.softmax_scale = d->softmax_scale;
  a.q = q; a.kv = kv; a.kv_scale = kv_scale; a.q_seq = q_seq; a.idx = idx; a.len = len;
  a.out = out; a.lse = lse; a.ws = reinterpret_cast<float*>(ws);
  return hip_status(fn, dsa::launch_sparse_mla(a, (hipStream_t)stream));
}

}  // namespace

extern "C" {

size_t dsa_sparse_mla_workspace_size(const dsa_mla_desc_t* d) {
  if (!d || d->num_q <= 0 || d->topk <= 0) return 0;
  return mla_ws_bytes(d, true);
}

dsa_status_t dsa_sparse_mla_decode(const dsa_mla_desc_t* d, const void* q, const void* kv, const float* kv_scale,
                                   const int32_t* q_seq, const int32_t* idx, const int32_t* len, float* out,
                                   float* lse, void* ws, size_t ws_bytes, void* stream, const dsa_paging_t* paging) {
  return mla_call("dsa_sparse_mla_decode", true, d, q, kv, kv_scale, q_seq, idx, len, out, lse, ws, ws_bytes, stream,
                  paging);
}

dsa_status_t dsa_sparse_mla_prefill(const dsa_mla_desc_t* d, const void* q, const void* kv, const float* kv_scale,
                                    const int32_t* q_seq, const int32_t* idx, const int32_t* len, float* out,
                                    float* lse, void* ws, size_t ws_bytes, void* stream, const dsa_paging_t* paging) {
  return mla_call("dsa_sparse_mla_prefill", false, d, q, kv, kv_scale, q_seq, idx, len, out, lse, ws, ws_bytes, stream,
                  paging);
}

}  // extern "C"

// ---- sparse MLA decode without allocation ----------------------------------------------------

// Split partials and statistics of dsa_sparse_mla_decode_noalloc, one copy per GPU for the life of
// the process.  In host code this name is a host-side stand-in, not device memory: the device
// address is looked up once per device with hipGetSymbolAddress, and only that address is handed
// to kernels.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The device address of `scratch` on the current device (looked up on its first use there).
hipError_t scratch_on_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

size_t dsa_sparse_mla_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

dsa_status_t dsa_sparse_mla_decode_noalloc(const dsa_mla_desc_t* d, const void* q, const void* kv,
                                           const float* kv_scale, const int32_t* q_seq, const int32_t* idx,
                                           const int32_t* len, float* out, float* lse, void* stream,
                                           const dsa_paging_t* paging) {
  const char* fn = "dsa_sparse_mla_decode_noalloc";
  Checker ck;
  if (!d) { ck.need(false, "desc is NULL"); return ck.finish(fn); }
  const size_t need = d->num_q > 0 ? mla_ws_bytes(d, true) : 0;
  if (need > kNoAllocScratchBytes) {
    ck.fail(false, "needs %zu bytes of split partials, above the %zu bytes this entry point holds per GPU "
            "(use fewer queries or splits, or dsa_sparse_mla_decode with a workspace)", need, kNoAllocScratchBytes);
    return ck.finish(fn);
  }
  void* ws = nullptr;
  if (need > 0) {
    const hipError_t e = scratch_on_current_device(&ws);
    if (e != hipSuccess) {
      g_err = std::string(fn) + ": device address of the scratch buffer: " + hipGetErrorString(e);
      return DSA_ERR_HIP;
    }
  }
  return mla_call(fn, true, d, q, kv, kv_scale, q_seq, idx, len, out, lse, ws, need > 0 ? kNoAllocScratchBytes : 0,
                  stream, paging);
}

}  // extern "C"

// ---- cache writers --------------------------------------------------------------------------

namespace {

size_t kinsert_ws_bytes(const dsa_index_k_desc_t* d) {
  if (!d || d->num_tokens <= 0 || d->hidden < 32 || d->hidden % 32 != 0) return 0;
  return (size_t)dsa::kinsert_splits(d->num_tokens, d->hidden) * d->num_tokens * 128 * sizeof(float);
}

}  // namespace

extern "C" {

size_t dsa_index_k_insert_workspace_size(const dsa_index_k_desc_t* d) { return kinsert_ws_bytes(d); }

dsa_status_t dsa_index_k_insert(const dsa_index_k_desc_t* d, const void* x, const void* wk, const float* ln_w,
                                const float* ln_b, const int32_t* pos, const float* inv_freq, const int64_t* slot,
                                uint8_t* k_cache, float* k_scale, void* ws, size_t ws_bytes, void* stream,
                                const dsa_paging_t* paging) {
  const char* fn = "dsa_index_k_insert";
  Checker ck;
  if (!d) { ck.need(false, "desc is NULL"); return ck.finish(fn); }
  ck.need(d->num_tokens >= 0 && d->num_tokens <= (1 << 24), "num_tokens must be in [0, 2^24]");
  ck.support(d->hidden >= 32 && d->hidden <= (1 << 20) && d->hidden % 32 == 0,
             "hidden must be a multiple of 32 in [32, 2^20]");
  ck.need(d->ld_x >= d->hidden && d->ld_x % 8 == 0, "ld_x must be >= hidden and a multiple of 8");
  ck.support(d->rope_dim == 0 || d->rope_dim == 64, "rope_dim must be 0 or 64");
  ck.need(d->eps >= 0.f, "eps must be >= 0");
  ck.need(d->num_slots >= 0, "num_slots must be >= 0");
  if (d->num_tokens > 0) {
    ck.need(x && wk && ln_w && pos && slot && k_cache && k_scale, "x, wk, ln_w, pos, slot, k_cache and k_scale must be non-NULL");
    ck.need(d->rope_dim == 0 || inv_freq != nullptr, "inv_freq is required when rope_dim is 64");
    ck.need(aligned(x, 16) && aligned(wk, 16), "x and wk must be 16-byte aligned");
    ck.need(aligned(k_cache, 2) && aligned(k_scale, 4), "k_cache must be 2-byte and k_scale 4-byte aligned");
    const size_t need = kinsert_ws_bytes(d);
    ck.need(ws != nullptr && ws_bytes >= need && aligned(ws, 16),
            "workspace missing, misaligned or smaller than dsa_index_k_insert_workspace_size()");
  }
  if (paging) {   // the writer needs the block size only (slots come in); the pool is the cache
    ck.support(paging->page_size >= 32 && paging->page_size <= 8192 && paging->page_size % 32 == 0,
               "paging->page_size must be a multiple of 32 in [32, 8192]");
    ck.need(paging->num_blocks >= 1 && (int64_t)paging->num_blocks * paging->page_size == d->num_slots,
            "num_slots must be paging->num_blocks * paging->page_size");
  }
  dsa_status_t st = ck.finish(fn);
  if (st != DSA_OK || d->num_tokens == 0) return st;
  dsa::KInsertLaunch a{};
  a.page = paging ? paging->page_size : 0;
  a.T = d->num_tokens; a.D = d->hidden; a.rope_dim = d->rope_dim;
  a.splits = dsa::kinsert_splits(a.T, a.D);
  a.ld_x = d->ld_x; a.nslots = d->num_slots; a.eps = d->eps;
  a.x = static_cast<const uint16_t*>(x); a.wk = static_cast<const uint16_t*>(wk);
  a.ln_w = ln_w; a.ln_b = ln_b; a.pos = pos; a.inv_freq = inv_freq; a.slot = slot;
  a.k_cache = k_cache; a.k_scale = k_scale; a.ws = static_cast<float*>(ws);
  return hip_status(fn, dsa::launch_index_k_insert(a, (hipStream_t)stream));
}

dsa_status_t dsa_latent_insert(int32_t num_tokens, int32_t rope_dim, const void* kv, int64_t ld_kv,
                               const int32_t* pos, const float* inv_freq, const int64_t* slot, int64_t num_slots,
                               uint8_t* kv_cache, float* kv_scale, void* stream) {
  const char* fn = "dsa_latent_insert";
  Checker ck;
  ck.need(num_tokens >= 0 && num_tokens <= (1 << 24), "num_tokens must be in [0, 2^24]");
  ck.support(rope_dim == 0 || rope_dim == 64, "rope_dim must be 0 or 64");
  ck.need(ld_kv >= 576, "ld_kv must be >= 576");
  ck.need(num_slots >= 0, "num_slots must be >= 0");
  if (num_tokens > 0) {
    ck.need(kv && pos && slot && kv_cache && kv_scale, "kv, pos, slot, kv_cache and kv_scale must be non-NULL");
    ck.need(aligned(kv, 16) && ld_kv % 8 == 0 && aligned(kv_cache, 8) && aligned(kv_scale, 4),
            "kv must be 16-byte aligned with ld_kv a multiple of 8, kv_cache 8-byte and kv_scale 4-byte aligned");
    ck.need(rope_dim == 0 || inv_freq != nullptr, "inv_freq is required when rope_dim is 64");
  }
  dsa_status_t st = ck.finish(fn);
  if (st != DSA_OK || num_tokens == 0) return st;
  dsa::LatentInsertLaunch a{};
  a.T = num_tokens; a.rope_dim = rope_dim; a.ld_kv = ld_kv; a.nslots = num_slots;
  a.kv = static_cast<const uint16_t*>(kv); a.pos = pos; a.inv_freq = inv_freq; a.slot = slot;
  a.kv_cache = kv_cache; a.kv_scale = kv_scale;
  return hip_status(fn, dsa::launch_latent_insert(a, (hipStream_t)stream));
}

dsa_status_t dsa_paged_slots(const dsa_paging_t* paging, int32_t n, const int32_t* seq, const int32_t* pos,
                             int64_t* slot, void* stream) {
  const char* fn = "dsa_paged_slots";
  Checker ck;
  ck.need(paging != nullptr, "paging is NULL");
  ck.need(n >= 0, "n must be >= 0");
  if (!paging) return ck.finish(fn);
  const dsa::Paging pg = check_paging(ck, paging, paging->num_seqs, 1, true);
  ck.need(paging->num_seqs >= 1, "paging->num_seqs must be >= 1");
  if (n > 0) ck.need(seq && pos && slot, "seq, pos and slot must be non-NULL");
  dsa_status_t st = ck.finish(fn);
  if (st != DSA_OK || n == 0) return st;
  return hip_status(fn, dsa::launch_paged_slots(pg, paging->num_seqs, n, seq, pos, slot, (hipStream_t)stream));
}

}  // extern "C"
