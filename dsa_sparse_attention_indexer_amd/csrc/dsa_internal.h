// Internal declarations shared by the HIP translation units of libdsa (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/dsa.h"

namespace dsa {

// Every kernel of the library is enqueued through launch(): normally a plain launch; while the
// timing hook (dsa_timing_begin) has a free pair of events, a launch that records the kernel's own
// start and stop timestamps into them.
bool timing_take(const void* fn, hipEvent_t* start, hipEvent_t* stop);

template <typename... Params, typename... Args>
inline void launch(void (*kernel)(Params...), dim3 grid, dim3 block, uint32_t shmem, hipStream_t s, Args... args) {
  hipEvent_t e0, e1;
  if (timing_take(reinterpret_cast<const void*>(kernel), &e0, &e1))
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, s, e0, e1, 0u, static_cast<Params>(args)...);
  else
    hipLaunchKernelGGL(kernel, grid, block, shmem, s, static_cast<Params>(args)...);
}

// ---- launch parameter blocks (host-validated, passed by value to the launchers) -------------

// Paged cache layout (the header's "Paged caches"): table == nullptr means contiguous caches.
struct Paging {
  const int32_t* table;   // [num_seqs][bps]
  int page;               // tokens per block (a multiple of 32)
  int bps;                // table columns
  int nblocks;            // blocks in the pool
};

struct IndexerLaunch {
  int T, H, rope_dim, B, max_ctx;
  dsa_dtype_t q_dtype, k_dtype;
  const void* q;
  const float* w;
  const int32_t* q_seq;
  const int32_t* q_pos;
  const float* ssmax_s;
  const float* ssmax_b;
  const float* inv_freq;
  const void* k_cache;
  const float* k_scale;
  float* scores;
  int64_t ld;
  // optional fused first top-k digit: when set, the score kernel adds the histogram of its
  // scores' first radix digit into this per-row workspace for a k-selection; NULL = scores only
  void* topk_ws;
  int topk_k;
  // with topk_ws: each score chunk also appends its own top-k candidates (every score at or above
  // the bin of the chunk's kq-th largest) to the row's item list, so the selection needs no second
  // pass over the scores (dsa_indexer_topk only: the emitted items are consumed in the same call)
  int topk_emit;
  Paging pg;
  // optional block maxima (block-sparse selection; the decode kernel without the top-k digit): the
  // largest score key of each visible `bblock`-key block, bmax[t * bld + block]; NULL = none
  uint32_t* bmax;
  int bblock;
  int64_t bld;
};

struct TopkLaunch {
  const float* scores;
  int64_t ld;
  int64_t ncap;   // a row holds min(q_pos + 1, ncap) scores
  const int32_t* q_pos;
  int T, k;
  int32_t* idx;
  int32_t* len;
  void* ws;       // per-row first-digit histograms (fused path only)
  int seg;        // columns per entry of the row's item table (a collect segment or a score chunk)
  int emitted;    // the score kernel emitted the items (no collect pass)
};

struct BlockSelectLaunch {
  const float* scores;
  int64_t ld;
  const int32_t* q_pos;
  int T, block, nblocks, topk;
  int32_t* idx;
  int32_t* len;
  void* ws;
};

struct MlaLaunch {
  int T, H, kv_lora, rope_dim, B, max_ctx, topk, splits, per_split;
  dsa_dtype_t q_dtype, kv_dtype;
  float softmax_scale;
  const void* q;
  const void* kv;
  const float* kv_scale;
  const int32_t* q_seq;
  const int32_t* idx;
  const int32_t* len;
  float* out;
  float* lse;
  float* ws;  // split partials: [T][H][splits][kv_lora] O, then [T][H][splits] m and l
  Paging pg;
  int64_t pool_rows;  // rows of kv / kv_scale when paged
  // head split (fp8 path): T and H above count virtual queries of H heads each, hs of them per real
  // query (the [T][64][...] query, output and LSE arrays read as [hs T][64 / hs][...]); the row
  // indices, lengths and sequence of virtual query t are those of real query t / hs
  int hs;
};

struct KInsertLaunch {
  int T, D, rope_dim, splits;   // split s sums the 256-dim blocks s, s + splits, ... of the hidden dim
  int64_t ld_x, nslots;
  float eps;
  const uint16_t* x;      // [T][ld_x] bf16
  const uint16_t* wk;     // [128][D] bf16
  const float* ln_w;
  const float* ln_b;      // NULL = no bias
  const int32_t* pos;
  const float* inv_freq;
  const int64_t* slot;
  uint8_t* k_cache;       // [nslots][128] E4M3FN
  float* k_scale;         // [nslots]
  float* ws;              // [splits][T][128] partial projections
  int page;               // > 0: k_cache is paged with this block size (key bytes in 16x16 tiles)
};

struct LatentInsertLaunch {
  int T, rope_dim;
  int64_t ld_kv, nslots;
  const uint16_t* kv;     // [T][ld_kv] bf16, 576 used
  const int32_t* pos;
  const float* inv_freq;
  const int64_t* slot;
  uint8_t* kv_cache;      // [nslots][576] E4M3FN
  float* kv_scale;        // [nslots][9]
};

// ---- sizes shared between validation and the kernels ----------------------------------------

constexpr int64_t kTopkMaxCols = int64_t(1) << 22;   // columns a top-k row may have

size_t topk_ws_bytes(int T);
size_t indexer_ws_bytes(int T, int B, dsa_dtype_t k_dtype);
// the grouped score kernel (fp8 keys; many queries, or several per sequence): it writes the
// scores only, and the selection runs as separate kernels over them
bool indexer_grouped(int T, int B, dsa_dtype_t k_dtype);
int indexer_chunk(int T, int max_ctx);              // keys per workgroup of the fp8 decode score kernel
size_t block_select_ws_bytes(int T, int64_t ld, int block);
// the decode score kernel can emit the block maxima itself (blocks of whole 32-key tiles that
// divide its chunk)
bool indexer_block_max_fused(int T, int B, int max_ctx, dsa_dtype_t k_dtype, int block);
int kinsert_splits(int T, int D);   // hidden-dim splits of the key projection

// ---- launchers (return the HIP status of the last launch) -----------------------------------

hipError_t launch_indexer(const IndexerLaunch& a, void* ws, hipStream_t s);
hipError_t launch_topk(const TopkLaunch& a, bool hist_given, hipStream_t s);
hipError_t launch_topk_hist(const TopkLaunch& a, hipStream_t s);   // the first-digit histogram only
// one kernel per call, no workspace needed (a.ws, if given, has each row's bookkeeping cleared):
// for scores that no kernel histogrammed.  One workgroup streams each row twice, so it pays when
// there are enough rows to fill the CUs (measured: 4096 rows of 61K 583 us against 723 us for the
// histogram + collect + resolve kernels; 64 rows of 131K 60 us against 32 us)
hipError_t launch_topk_direct(const TopkLaunch& a, hipStream_t s);
inline bool topk_direct_pays(int num_q) { return num_q >= 128; }
hipError_t launch_block_select(const BlockSelectLaunch& a, hipStream_t s);
hipError_t launch_block_pick(const BlockSelectLaunch& a, hipStream_t s);   // maxima already in a.ws
hipError_t launch_sparse_mla(const MlaLaunch& a, hipStream_t s);
hipError_t launch_index_k_insert(const KInsertLaunch& a, hipStream_t s);
hipError_t launch_latent_insert(const LatentInsertLaunch& a, hipStream_t s);
hipError_t launch_paged_slots(const Paging& pg, int nseq, int n, const int32_t* seq, const int32_t* pos, int64_t* slot,
                              hipStream_t s);

}  // namespace dsa

// ---- small device helpers --------------------------------------------------------------------

#if defined(__HIP_DEVICE_COMPILE__) || defined(__HIPCC__)
namespace dsa {

// Order-preserving map float -> u32 (larger float -> larger key); -0.0 maps like +0.0.
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// The paged layout rule, shared by the cache writers and every reader.  Block of position p of
// sequence b (the table entry clamped into the pool), and the pool slot of (b, p):
__device__ __forceinline__ int paged_block(const Paging& pg, int b, int p) {
  return clampi(pg.table[(size_t)b * pg.bps + min(p / pg.page, pg.bps - 1)], 0, pg.nblocks - 1);
}
__device__ __forceinline__ int64_t paged_slot(const Paging& pg, int b, int p) {
  return (int64_t)paged_block(pg, b, p) * pg.page + p % pg.page;
}
// Byte d of the key in row i of a block, from the block's first byte: 16-token x 16-byte tiles,
// the 8 tiles of a 16-token group side by side (a 32-row group is one contiguous 4 KiB range).
__device__ __forceinline__ uint32_t key_tile_byte(int i, int d) {
  return 256u * (8u * (uint32_t)(i >> 4) + (uint32_t)(d >> 4)) + 16u * (uint32_t)(i & 15) + (uint32_t)(d & 15);
}

// Sine and cosine of the RoPE angle p * inv_freq.  The product is exact in float64 (24-bit times
// 26-bit); it is reduced to [-pi, pi] in float64 with a two-term 2*pi (error far below float32
// resolution up to p = 2^26), and the sine and cosine of the reduced angle are taken in float32
// (about one ulp).
__device__ __forceinline__ void rope_sincos(int p, float inv_freq, float* sn, float* cs) {
  constexpr double kInv2Pi = 0.15915494309189535;
  constexpr double k2PiHi = 6.283185307179586;
  constexpr double k2PiLo = 2.4492935982947064e-16;
  const double ang = (double)p * (double)inv_freq;
  const double k = rint(ang * kInv2Pi);
  const double r = fma(-k, k2PiLo, fma(-k, k2PiHi, ang));
  sincosf((float)r, sn, cs);
}

}  // namespace dsa
#endif
