// Device-side pieces of the exact top-k shared by the index-score kernel (which can build the
// first radix digit's histogram while it scores) and the top-k kernels.
//
// Per-row workspace (32-bit words), zero before first use; the resolve kernel that finishes a row
// clears its histogram and counter again, so one zeroed workspace serves any sequence of calls:
//   hist   [kTkBins]        counts of the first radix digit (score-key bits 31..20)
//   ctr    [4]              ctr[0]: items appended by the collect kernel
//   table  [kTkMaxSeg][2]   per segment: first item, item count (written by every live segment)
//   items  [kTkItemCap][2]  (key, column) of every score whose first digit is >= the threshold
//                           digit, in column order within each segment
#pragma once

#include "dsa_internal.h"

namespace dsa {

constexpr int kTkBins = 4096;       // first digit: key bits 31..20
constexpr int kTkShift0 = 20;
constexpr int kTkSeg = 8192;        // columns per collect workgroup
constexpr int kTkMaxSeg = (int)(kTopkMaxCols / kTkSeg);
constexpr int kTkItemCap = 16384;   // items per row resolved in LDS
constexpr int kTkFastK = 4096;      // largest k resolved in LDS

constexpr size_t kTkOffCtr = kTkBins;
constexpr size_t kTkOffTable = kTkOffCtr + 4;
constexpr size_t kTkOffItems = kTkOffTable + 2 * (size_t)kTkMaxSeg;
constexpr size_t kTkRowWords = kTkOffItems + 2 * (size_t)kTkItemCap;

__host__ __device__ inline size_t tk_total_words(int T) { return (size_t)T * kTkRowWords; }

__device__ inline uint32_t* tk_row(void* ws, int t) { return reinterpret_cast<uint32_t*>(ws) + (size_t)t * kTkRowWords; }
__device__ inline uint32_t* tk_hist(void* ws, int t) { return tk_row(ws, t); }

// Block-wide exclusive prefix sum (blockDim.x a multiple of 64, at most 1024 threads).
__device__ inline uint32_t tk_excl_scan(uint32_t v, uint32_t* total, uint32_t* sbuf /* >= 17 words */) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) sbuf[wave] = x;
  __syncthreads();
  if (tid == 0) {
    uint32_t run = 0;
    for (int w = 0; w < nw; ++w) { const uint32_t s = sbuf[w]; sbuf[w] = run; run += s; }
    sbuf[16] = run;
  }
  __syncthreads();
  const uint32_t r = sbuf[wave] + x - v;
  if (total) *total = sbuf[16];
  __syncthreads();
  return r;
}

// The bin of an nb-bin histogram (nb a multiple of blockDim.x) holding the need-th largest key:
// returns it and the count still needed inside it, identically in every thread.
__device__ inline void tk_find_bin(const uint32_t* h, int nb, uint32_t need, uint32_t* sbuf, int* bin_out,
                                   uint32_t* need_out) {
  const int tid = threadIdx.x;
  const int per = nb / (int)blockDim.x;
  const int hi = nb - per * tid;   // thread 0 owns the top bins
  uint32_t local = 0;
  for (int i = 1; i <= per; ++i) local += h[hi - i];
  uint32_t above = tk_excl_scan(local, nullptr, sbuf);
  for (int i = 1; i <= per; ++i) {
    const uint32_t c = h[hi - i];
    if (above < need && need <= above + c) { sbuf[20] = (uint32_t)(hi - i); sbuf[21] = need - above; }
    above += c;
  }
  __syncthreads();
  *bin_out = (int)sbuf[20];
  *need_out = sbuf[21];
  __syncthreads();
}

}  // namespace dsa
