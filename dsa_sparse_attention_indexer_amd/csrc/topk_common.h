// Device-side pieces of the exact top-k shared by the index-score kernel (which can build the
// first radix digit's histogram while it scores) and the top-k kernels.
//
// Per-row workspace (32-bit words):
//   hist   [kTkBins]        counts of the first radix digit (score-key bits 31..20)
//   ctr    [4]              reserved (cleared by every selection)
//   table  [kTkMaxSeg][2]   per segment: first item, item count | (lowest digit emitted << 16),
//                           written by every live segment (a collect segment or, on the fused path,
//                           a score chunk)
//   items  [kTkItemCap][2]  (key, column) of every score whose first digit is >= the segment's
//                           lowest emitted digit, in column order within each segment; segment
//                           s of a row of S (collect segments or score chunks) owns slots
//                           s * (kTkItemCap / S) onwards
// Collected rows: the histogram only steers the fast path: the resolve kernel checks against the
// collected items that the digit it names holds the k-th largest key, and otherwise selects by
// exact passes over the row.  Emitted rows (score chunks that emit their own candidates) add only
// their bins at or above their lowest emitted digit: with L the largest such digit of the row's
// segments, the histogram is exact from L up and the items at or above L are exactly the row's
// keys there; the resolve kernel drops the bins below L and proceeds as above (b0 below L means
// fewer than k keys at or above L: exact passes).  The
// resolve kernel that finishes a row clears its histogram and counter, so stale
// contents (an interrupted call, a different k, a workspace never cleared) cost speed, never
// correctness.
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

// Block-wide exclusive prefix sum over NT threads (a multiple of 64, at most 1024); *total, if
// given, gets the sum.  sbuf: at least NT/64 words.
// Inclusive prefix sum over the 64 lanes of a wave with DPP moves (no LDS round trips): shifts by
// 1, 2, 4 and 8 lanes within each 16-lane row (lanes shifted in from outside the row read 0), then
// the total of row 0 is added to row 1 and of row 2 to row 3 (row_bcast:15), and the total of rows
// 0-1 to rows 2 and 3 (row_bcast:31).
__device__ inline uint32_t tk_wave_incl_scan(uint32_t x) {
  x += __builtin_amdgcn_update_dpp(0u, x, 0x111, 0xf, 0xf, true);    // row_shr:1
  x += __builtin_amdgcn_update_dpp(0u, x, 0x112, 0xf, 0xf, true);    // row_shr:2
  x += __builtin_amdgcn_update_dpp(0u, x, 0x114, 0xf, 0xf, true);    // row_shr:4
  x += __builtin_amdgcn_update_dpp(0u, x, 0x118, 0xf, 0xf, true);    // row_shr:8
  x += __builtin_amdgcn_update_dpp(0u, x, 0x142, 0xa, 0xf, false);   // row_bcast:15 -> rows 1, 3
  x += __builtin_amdgcn_update_dpp(0u, x, 0x143, 0xc, 0xf, false);   // row_bcast:31 -> rows 2, 3
  return x;
}

// Maximum over the 64 lanes of a wave with DPP moves (the same row shifts and broadcasts as the
// scan above); every lane gets it.
__device__ inline uint32_t tk_wave_max(uint32_t x) {
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0u, x, 0x111, 0xf, 0xf, true));    // row_shr:1
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0u, x, 0x112, 0xf, 0xf, true));    // row_shr:2
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0u, x, 0x114, 0xf, 0xf, true));    // row_shr:4
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0u, x, 0x118, 0xf, 0xf, true));    // row_shr:8
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0u, x, 0x142, 0xa, 0xf, false));   // row_bcast:15
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0u, x, 0x143, 0xc, 0xf, false));   // row_bcast:31
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

template <int NT>
__device__ inline uint32_t tk_excl_scan(uint32_t v, uint32_t* total, uint32_t* sbuf) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t x = tk_wave_incl_scan(v);
  if (lane == 63) sbuf[wave] = x;
  __syncthreads();
  uint32_t off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t s = sbuf[w];
    off += w < wave ? s : 0u;
    tot += s;
  }
  __syncthreads();
  if (total) *total = tot;
  return off + x - v;
}

// The bin of an NB-bin histogram (16-byte aligned) that holds the need-th largest key: returns it
// and the count still needed inside it, identically in every thread.  If the histogram holds
// fewer than need keys, bin 0 and need are returned.  Thread i owns NB/NT consecutive bins counted
// from the top.  sbuf: at least 22 words.
template <int NB, int NT>
__device__ inline void tk_find_bin(const uint32_t* h, uint32_t need, uint32_t* sbuf, int* bin_out,
                                   uint32_t* need_out) {
  static_assert(NB % NT == 0, "bins per thread");
  constexpr int PER = NB / NT;
  const int lo = NB - PER * ((int)threadIdx.x + 1);
  uint32_t c[PER];
  if constexpr (PER % 4 == 0) {
#pragma unroll
    for (int q = 0; q < PER / 4; ++q) {
      const uint4 x = *reinterpret_cast<const uint4*>(h + lo + 4 * q);
      c[4 * q] = x.x; c[4 * q + 1] = x.y; c[4 * q + 2] = x.z; c[4 * q + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < PER; ++i) c[i] = h[lo + i];
  }
  uint32_t local = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) local += c[i];
  if (threadIdx.x == 0) { sbuf[20] = 0u; sbuf[21] = need; }   // ordered before the finder by the scan's barrier
  uint32_t above = tk_excl_scan<NT>(local, nullptr, sbuf);
#pragma unroll
  for (int i = PER - 1; i >= 0; --i) {
    if (above < need && need <= above + c[i]) { sbuf[20] = (uint32_t)(lo + i); sbuf[21] = need - above; }
    above += c[i];
  }
  __syncthreads();
  *bin_out = (int)sbuf[20];
  *need_out = sbuf[21];
  __syncthreads();
}

// The bin of an NB-bin histogram (16-byte aligned, in LDS) that holds the need-th largest key, found
// by one wave with no barrier: lane l sums the NB/64 bins counted l-th from the top, a prefix sum
// over the lanes names the lane whose bins hold it, and a second prefix sum over that lane's bins
// (one per lane) names the bin.  Returns the bin and the count still needed inside it in every lane;
// fewer than need keys in the histogram: bin 0 and need.
template <int NB>
__device__ inline void tk_wave_find_bin(const uint32_t* h, uint32_t need, int* bin_out, uint32_t* need_out) {
  constexpr int PER = NB / 64;
  static_assert(PER % 4 == 0 && PER <= 64, "bins per lane");
  const int lane = threadIdx.x & 63;
  const int lo = NB - PER * (lane + 1);
  uint32_t sum = 0;
#pragma unroll
  for (int q = 0; q < PER / 4; ++q) {
    const uint4 x = *reinterpret_cast<const uint4*>(h + lo + 4 * q);
    sum += x.x + x.y + x.z + x.w;
  }
  const uint32_t incl = tk_wave_incl_scan(sum);
  const uint64_t m = __ballot(incl - sum < need && need <= incl);
  if (m == 0) {
    *bin_out = 0;
    *need_out = need;
    return;
  }
  const int l0 = __builtin_ctzll(m);
  const uint32_t ab = (uint32_t)__builtin_amdgcn_readlane((int)(incl - sum), l0);
  const int lo0 = NB - PER * (l0 + 1);
  const uint32_t c = lane < PER ? h[lo0 + PER - 1 - lane] : 0u;   // lane i: the i-th of those bins from the top
  const uint32_t inc2 = ab + tk_wave_incl_scan(c);
  const uint64_t m2 = __ballot(lane < PER && inc2 - c < need && need <= inc2);
  const int i = __builtin_ctzll(m2);
  *bin_out = lo0 + PER - 1 - i;
  *need_out = need - ((uint32_t)__builtin_amdgcn_readlane((int)inc2, i) - (uint32_t)__builtin_amdgcn_readlane((int)c, i));
}

// Sum over the 64 lanes of a wave (every lane gets it).
__device__ inline uint32_t tk_wave_sum(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_readlane((int)tk_wave_incl_scan(x), 63);
}

__device__ inline uint32_t tk_lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Element (q, e) of thread tid stands for column c0 + 4*NT*q + 4*tid + e: each float4 load of a
// wave covers 1 KiB of contiguous scores.  Loads keys; bit 4q+e of the mask is set when the
// column is < n (n >= 1).  Every load is an unconditional float4 (a slice at or past n reads the
// row's last aligned float4 instead, which is in range because rows are a multiple of 4 long, and
// is masked out), so all of them are in flight together.
template <int Q, int NT>
__device__ __forceinline__ uint32_t tk_load_slices(const float* row, int n, int c0, uint32_t key[Q][4]) {
  float4 v[Q];
  const int clast = (n - 1) & ~3;
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int c = c0 + 4 * NT * q + 4 * (int)threadIdx.x;
    v[q] = *reinterpret_cast<const float4*>(row + min(c, clast));
  }
  uint32_t mask = 0;
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int c = c0 + 4 * NT * q + 4 * (int)threadIdx.x;
    key[q][0] = score_key(v[q].x);
    key[q][1] = score_key(v[q].y);
    key[q][2] = score_key(v[q].z);
    key[q][3] = score_key(v[q].w);
#pragma unroll
    for (int e = 0; e < 4; ++e) mask |= (c + e < n ? 1u : 0u) << (4 * q + e);
  }
  return mask;
}

// Ordered compaction over the workgroup for the layout above (column order = slice, wave, lane,
// element).  fl[q] holds this thread's 4-bit selection of slice q; returns in pos[q] the slot of
// its first selected element of slice q, and the workgroup's total.  wsum: Q * NT/64 LDS words.
template <int Q, int NT>
__device__ uint32_t tk_ordered_slots(const uint32_t fl[Q], uint32_t pos[Q], uint32_t* wsum) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t below[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    uint32_t bl = 0, wt = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint64_t b = __ballot((fl[q] >> e) & 1u);
      bl += tk_lanes_below(b);
      wt += (uint32_t)__popcll(b);
    }
    below[q] = bl;
    if (lane == 0) wsum[q * NW + wave] = wt;
  }
  __syncthreads();
  uint32_t run = 0;
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    uint32_t tq = 0, pw = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const uint32_t x = wsum[q * NW + w];
      pw += w < wave ? x : 0u;
      tq += x;
    }
    pos[q] = run + pw + below[q];
    run += tq;
  }
  __syncthreads();
  return run;
}

}  // namespace dsa
