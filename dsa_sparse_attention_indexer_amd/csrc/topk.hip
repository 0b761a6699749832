// Exact per-row top-k selection on gfx950 (radix select over order-preserving u32 score keys).
//
// Keeps the k highest scores of each row, equal scores going to the lower column, and emits the
// kept columns in ascending order with -1 padding and the row length ("mistral-large4.md", bullet
// "The indexer": the top 2048 keys are kept; the -1 slots and top-k length bound follow the vLLM
// page's "Top-k compaction" bullet).
//
// Up to three launches; rows are cut into 8192-column segments:
//   hist     one workgroup per segment histograms the first digit (key bits 31..20) in LDS and
//            adds it to the row's histogram.  The fused path skips it: the index-score kernel
//            has already built that histogram.
//   collect  one workgroup per segment finds, from the row's histogram, the bin b0 that holds
//            the k-th largest key and writes every key whose first digit is >= b0 (all keys
//            above b0 plus the candidates inside it; a few thousand per row) to the segment's own
//            region of the row's item list, in column order, with ballot/mbcnt compaction.
//   resolve  one workgroup per row loads the histogram, the segment table and every item region
//            in one round of loads and places the items in LDS in column order, checks from them
//            that the histogram's bin b0 really holds the k-th largest key (fewer than k items
//            above b0, at least k at or above it), finds the exact k-th key among the candidates
//            (bits 19..10, then 9..0; each histogram searched by one wave), and with one ordered
//            pass keeps the keys above it and the lowest columns among the keys equal to it.  The
//            output is ascending by construction: no sort and no merge.
// On the fused score + top-k path the score kernel emits each chunk's candidates itself (see
// emit_candidates in the index kernels) into the same kind of regions, and only the resolve kernel
// runs; a chunk that emitted only digits above the row's b0 sends the row to the exact passes.
// With many rows and no histogram (the grouped and fp32 score kernels, the separate call), one
// kernel per row (direct) streams the row twice and keeps the candidates on chip; with fewer rows,
// the emit kernel's segments pick their own thresholds and emit as the score kernel does, so the
// scores are read once and no row histogram pass comes first.
// If a row's items do not fit in LDS (heavy ties), k is large, or the check fails (a histogram
// left over from an interrupted call, or built for another k), the resolve workgroup instead
// selects by exact passes over the row, first digit included.  Every decision is made on the
// integer keys, so the result is exact and deterministic; the histogram only decides how fast.

#include "topk_common.h"

namespace dsa {
namespace {

constexpr int kCT = 512;                   // hist / collect threads
constexpr int kCQ = kTkSeg / (4 * kCT);    // float4 slices per collect thread (4)
constexpr int kRT = 1024;                  // resolve threads
constexpr int kSQ = 4;                     // float4 slices per resolve thread and streaming round

__device__ inline int row_n(const TopkLaunch& a, int t) {
  int64_t n = (int64_t)a.q_pos[t] + 1;
  if (n < 0) n = 0;
  if (n > a.ncap) n = a.ncap;
  return (int)n;
}

// ------------------------------------------------------------------------------------------
// hist: first-digit histogram of one segment, added into the row's
// ------------------------------------------------------------------------------------------

__global__ void __launch_bounds__(kCT) k_topk_hist(TopkLaunch a) {
  __shared__ uint32_t lh[kTkBins];
  const int t = blockIdx.y;
  const int n = row_n(a, t);
  const int c0 = blockIdx.x * kTkSeg;
  if (n <= a.k || c0 >= n) return;
  const float* row = a.scores + (size_t)t * a.ld;
  uint32_t key[kCQ][4];
  const uint32_t mask = tk_load_slices<kCQ, kCT>(row, n, c0, key);
  for (int i = threadIdx.x; i < kTkBins; i += kCT) lh[i] = 0;
  __syncthreads();
#pragma unroll
  for (int q = 0; q < kCQ; ++q)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if ((mask >> (4 * q + e)) & 1u) atomicAdd(&lh[key[q][e] >> kTkShift0], 1u);
  __syncthreads();
  uint32_t* gh = tk_hist(a.ws, t);
  for (int i = threadIdx.x; i < kTkBins; i += kCT)
    if (lh[i]) atomicAdd(&gh[i], lh[i]);
}

// ------------------------------------------------------------------------------------------
// emit: one pass over the scores with no row histogram first.  Each segment histograms its own
// keys in LDS, takes lb, the first digit of its kq-th largest key (kq: twice the segment's share
// of the k plus 32), adds its bins from lb up into the row's histogram and writes every key whose
// digit is >= lb, in column order, to its region, with the entry (first item, count | lb << 16):
// the bookkeeping of the score kernel's own emission, which the resolve kernel checks the same way
// (a segment that held more of the row's top k than it emitted sends the row to the exact passes).
// ------------------------------------------------------------------------------------------

__global__ void __launch_bounds__(kCT) k_topk_emit(TopkLaunch a) {
  __shared__ __attribute__((aligned(16))) uint32_t lh[kTkBins];
  __shared__ uint32_t sbuf[32];
  __shared__ uint32_t wsum[kCQ * (kCT / 64)];
  const int t = blockIdx.y;
  const int n = row_n(a, t);
  const int seg = blockIdx.x;
  const int c0 = seg * kTkSeg;
  if (n <= a.k || a.k > kTkFastK || c0 >= n) return;
  const float* row = a.scores + (size_t)t * a.ld;
  uint32_t key[kCQ][4];
  const uint32_t mask = tk_load_slices<kCQ, kCT>(row, n, c0, key);
  for (int i = threadIdx.x; i < kTkBins; i += kCT) lh[i] = 0;
  __syncthreads();
#pragma unroll
  for (int q = 0; q < kCQ; ++q)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if ((mask >> (4 * q + e)) & 1u) atomicAdd(&lh[key[q][e] >> kTkShift0], 1u);
  __syncthreads();
  const uint32_t nrow = (uint32_t)min(kTkSeg, n - c0);
  const uint32_t share = (uint32_t)(((uint64_t)a.k * kTkSeg + (uint64_t)n - 1) / (uint64_t)n);
  const uint32_t kq = min(nrow, 2u * share + 32u);
  int lb;
  uint32_t unused;
  tk_find_bin<kTkBins, kCT>(lh, kq, sbuf, &lb, &unused);
  uint32_t* rw = tk_row(a.ws, t);
  uint32_t* gh = tk_hist(a.ws, t);
  for (int i = lb + (int)threadIdx.x; i < kTkBins; i += kCT)
    if (lh[i]) atomicAdd(&gh[i], lh[i]);
  uint32_t fl[kCQ];
#pragma unroll
  for (int q = 0; q < kCQ; ++q) {
    fl[q] = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      fl[q] |= (((mask >> (4 * q + e)) & 1u) && (key[q][e] >> kTkShift0) >= (uint32_t)lb ? 1u : 0u) << e;
  }
  uint32_t pos[kCQ];
  const uint32_t total = tk_ordered_slots<kCQ, kCT>(fl, pos, wsum);
  const uint32_t cap = (uint32_t)kTkItemCap / (uint32_t)((n + kTkSeg - 1) / kTkSeg);
  const uint32_t st = (uint32_t)seg * cap;
  const bool fits = total <= cap;
  if (threadIdx.x == 0)
    *reinterpret_cast<uint2*>(rw + kTkOffTable + 2 * seg) =
        make_uint2(fits ? st : (uint32_t)kTkItemCap, (fits ? total : 0xFFFFu) | ((uint32_t)lb << 16));
  if (!fits) return;
  uint2* items = reinterpret_cast<uint2*>(rw + kTkOffItems);
#pragma unroll
  for (int q = 0; q < kCQ; ++q) {
    uint32_t p = st + pos[q];
    const uint32_t cq = (uint32_t)(c0 + 4 * kCT * q + 4 * (int)threadIdx.x);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if ((fl[q] >> e) & 1u) items[p++] = make_uint2(key[q][e], cq + e);
  }
}

// ------------------------------------------------------------------------------------------
// collect: the keys of one segment whose first digit is >= b0, in column order
// ------------------------------------------------------------------------------------------

__global__ void __launch_bounds__(kCT) k_topk_collect(TopkLaunch a) {
  __shared__ __attribute__((aligned(16))) uint32_t hist[kTkBins];
  __shared__ uint32_t sbuf[32];
  __shared__ uint32_t wsum[kCQ * (kCT / 64)];
  const int t = blockIdx.y;
  const int n = row_n(a, t);
  const int seg = blockIdx.x;
  const int c0 = seg * kTkSeg;
  if (n <= a.k || a.k > kTkFastK || c0 >= n) return;
  const float* row = a.scores + (size_t)t * a.ld;
  uint32_t* rw = tk_row(a.ws, t);
  uint32_t key[kCQ][4];
  const uint32_t mask = tk_load_slices<kCQ, kCT>(row, n, c0, key);
  const uint4* gh = reinterpret_cast<const uint4*>(rw);
#pragma unroll
  for (int j = 0; j < kTkBins / (4 * kCT); ++j) {
    const uint4 h = gh[threadIdx.x + kCT * j];
    uint32_t* d = hist + 4 * (threadIdx.x + kCT * j);
    d[0] = h.x; d[1] = h.y; d[2] = h.z; d[3] = h.w;
  }
  __syncthreads();
  int b0;
  uint32_t need0;
  tk_find_bin<kTkBins, kCT>(hist, (uint32_t)a.k, sbuf, &b0, &need0);
  uint32_t fl[kCQ];
#pragma unroll
  for (int q = 0; q < kCQ; ++q) {
    fl[q] = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      fl[q] |= (((mask >> (4 * q + e)) & 1u) && (key[q][e] >> kTkShift0) >= (uint32_t)b0 ? 1u : 0u) << e;
  }
  uint32_t pos[kCQ];
  const uint32_t total = tk_ordered_slots<kCQ, kCT>(fl, pos, wsum);
  // segment s of the row's S owns items s * cap .. s * cap + cap - 1 (cap = kTkItemCap / S); a
  // segment with more candidates writes none and an entry that claims more items than the list
  // has, and the resolve kernel then streams the row
  const uint32_t cap = (uint32_t)kTkItemCap / (uint32_t)((n + kTkSeg - 1) / kTkSeg);
  const uint32_t st = (uint32_t)seg * cap;
  const bool fits = total <= cap;
  if (threadIdx.x == 0)
    *reinterpret_cast<uint2*>(rw + kTkOffTable + 2 * seg) =
        make_uint2(fits ? st : (uint32_t)kTkItemCap, fits ? total : 0xFFFFu);
  if (!fits) return;
  uint2* items = reinterpret_cast<uint2*>(rw + kTkOffItems);
#pragma unroll
  for (int q = 0; q < kCQ; ++q) {
    uint32_t p = st + pos[q];
    const uint32_t cq = (uint32_t)(c0 + 4 * kCT * q + 4 * (int)threadIdx.x);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if ((fl[q] >> e) & 1u) items[p++] = make_uint2(key[q][e], cq + e);
  }
}

// ------------------------------------------------------------------------------------------
// resolve: one workgroup per row
// ------------------------------------------------------------------------------------------

struct ResolveSmem {
  uint32_t key[kTkItemCap];
  uint32_t col[kTkItemCap];
  uint32_t hist[kTkBins];
  uint32_t tst[kTkMaxSeg];    // per segment: first item in the workspace (emitted rows: its count)
  uint32_t tpre[kTkMaxSeg];   // per segment: first item in column order
  uint32_t sbuf[32];
  uint32_t wsum[kSQ * (kRT / 64)];
  uint32_t hist1[1024];       // emitted rows: the second digit of the candidates inside b0
  uint32_t wtot[kRT / 64];    // per wave: a sum
  uint32_t wmax[kRT / 64];    // per wave: a maximum
  uint32_t res[8];            // results handed from one wave to the workgroup
};

// Among keys[0..cnt) whose bits above shift + bits equal prefix: the bits-wide digit at shift
// that holds the need-th largest key, and the count still needed inside it.
template <int BITS>
__device__ void lds_digit(const uint32_t* keys, int cnt, uint32_t prefix, int shift, uint32_t need,
                          ResolveSmem& sm, int* digit, uint32_t* need_out) {
  constexpr int nb = 1 << BITS;
  constexpr int bits = BITS;
  for (int i = threadIdx.x; i < nb; i += kRT) sm.hist[i] = 0;
  __syncthreads();
  const int hs = shift + bits;
  for (int i = threadIdx.x; i < cnt; i += kRT) {
    const uint32_t k = keys[i];
    if ((k >> hs) == prefix) atomicAdd(&sm.hist[(k >> shift) & (nb - 1)], 1u);
  }
  __syncthreads();
  tk_find_bin<nb, kRT>(sm.hist, need, sm.sbuf, digit, need_out);
}

// The same over the row in memory (streaming finish).  shift + BITS == 32 is the first digit (no
// prefix).
template <int BITS>
__device__ void row_digit(const float* row, int n, uint32_t prefix, int shift, uint32_t need,
                          ResolveSmem& sm, int* digit, uint32_t* need_out) {
  constexpr int nb = 1 << BITS;
  constexpr int bits = BITS;
  static_assert(nb <= kTkBins, "digit histogram fits");
  for (int i = threadIdx.x; i < nb; i += kRT) sm.hist[i] = 0;
  __syncthreads();
  const bool top = shift + bits >= 32;
  const int hs = top ? 0 : shift + bits;
  for (int c0 = 0; c0 < n; c0 += 4 * kRT * kSQ) {
    uint32_t key[kSQ][4];
    const uint32_t mask = tk_load_slices<kSQ, kRT>(row, n, c0, key);
#pragma unroll
    for (int q = 0; q < kSQ; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (((mask >> (4 * q + e)) & 1u) && (top || (key[q][e] >> hs) == prefix))
          atomicAdd(&sm.hist[(key[q][e] >> shift) & (nb - 1)], 1u);
  }
  __syncthreads();
  tk_find_bin<nb, kRT>(sm.hist, need, sm.sbuf, digit, need_out);
}

// Streaming finish: the exact k-th key from three passes over the row (first digit, then bits
// 19..10 and 9..0), then one ordered pass that emits every key above it and the lowest columns
// among the keys equal to it.  It reads nothing from the workspace.
__device__ __forceinline__ void finish_streaming(const TopkLaunch& a, int t, int n, ResolveSmem& sm) {
  const float* row = a.scores + (size_t)t * a.ld;
  int b0i, d1, d2;
  uint32_t need0, need1, need2;
  row_digit<12>(row, n, 0u, kTkShift0, (uint32_t)a.k, sm, &b0i, &need0);
  const uint32_t b0 = (uint32_t)b0i;
  row_digit<10>(row, n, b0, 10, need0, sm, &d1, &need1);
  row_digit<10>(row, n, (b0 << 10) | (uint32_t)d1, 0, need1, sm, &d2, &need2);
  const uint32_t thr = (b0 << 20) | ((uint32_t)d1 << 10) | (uint32_t)d2;
  int32_t* out = a.idx + (size_t)t * a.k;
  uint32_t base = 0, eq_seen = 0;
  for (int c0 = 0; c0 < n; c0 += 4 * kRT * kSQ) {
    uint32_t key[kSQ][4];
    const uint32_t mask = tk_load_slices<kSQ, kRT>(row, n, c0, key);
    uint32_t gt[kSQ], eq[kSQ], epos[kSQ], spos[kSQ];
#pragma unroll
    for (int q = 0; q < kSQ; ++q) {
      gt[q] = eq[q] = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool in = (mask >> (4 * q + e)) & 1u;
        gt[q] |= (in && key[q][e] > thr ? 1u : 0u) << e;
        eq[q] |= (in && key[q][e] == thr ? 1u : 0u) << e;
      }
    }
    const uint32_t eq_tot = tk_ordered_slots<kSQ, kRT>(eq, epos, sm.wsum);
#pragma unroll
    for (int q = 0; q < kSQ; ++q) {
      uint32_t r = eq_seen + epos[q];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if ((eq[q] >> e) & 1u) {
          if (r < need2) gt[q] |= 1u << e;
          ++r;
        }
    }
    const uint32_t sel_tot = tk_ordered_slots<kSQ, kRT>(gt, spos, sm.wsum);
#pragma unroll
    for (int q = 0; q < kSQ; ++q) {
      uint32_t p = base + spos[q];
      const int cq = c0 + 4 * kRT * q + 4 * (int)threadIdx.x;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if ((gt[q] >> e) & 1u) {
          if (p < (uint32_t)a.k) out[p] = cq + e;
          ++p;
        }
    }
    base += sel_tot;
    eq_seen += eq_tot;
  }
}

// The selection from the row's candidates in LDS (sm.key / sm.col[0, total), in column order: every
// key whose first digit is >= b0, where b0 holds the k-th largest key and need0 of its keys are
// still needed): the exact k-th key from two more 10-bit digits, then one ordered pass that keeps
// the keys above it and the lowest columns among the keys equal to it.  Writes the row's output
// and length.
__device__ __forceinline__ void select_from_items(const TopkLaunch& a, int t, uint32_t total, uint32_t b0,
                                                  uint32_t need0, ResolveSmem& sm) {
  const int tid = threadIdx.x;
  int32_t* out = a.idx + (size_t)t * a.k;

  // the exact k-th key among the candidates (the items inside b0): bits 19..10 first
  int d1;
  uint32_t need1;
  lds_digit<10>(sm.key, (int)total, b0, 10, need0, sm, &d1, &need1);
  const uint32_t pre22 = (b0 << 10) | (uint32_t)d1;
  uint32_t thr, need2;
  const uint32_t c1 = sm.hist[d1];   // keys sharing the top 22 bits of the k-th key
  __syncthreads();                   // read before the histogram is reused below
  if (c1 <= 64u) {
    // typically a handful of keys share the top 22 bits: collect them and rank them in one wave
    if (tid == 0) sm.sbuf[25] = 0;
    __syncthreads();
    for (uint32_t i = tid; i < total; i += kRT) {
      const uint32_t k = sm.key[i];
      if ((k >> 10) == pre22) sm.wsum[atomicAdd(&sm.sbuf[25], 1u)] = k;
    }
    __syncthreads();
    if (tid < 64) {
      const uint32_t c = sm.sbuf[25];
      const uint32_t mine = tid < (int)c ? sm.wsum[tid] : 0u;
      uint32_t above = 0, same = 0;
      for (uint32_t j = 0; j < c; ++j) {
        const uint32_t o = sm.wsum[j];
        above += o > mine ? 1u : 0u;
        same += o == mine ? 1u : 0u;
      }
      if (tid < (int)c && above < need1 && need1 <= above + same) { sm.sbuf[26] = mine; sm.sbuf[27] = need1 - above; }
    }
    __syncthreads();
    thr = sm.sbuf[26];
    need2 = sm.sbuf[27];
  } else {
    int d2;
    lds_digit<10>(sm.key, (int)total, pre22, 0, need1, sm, &d2, &need2);
    thr = (pre22 << 10) | (uint32_t)d2;
  }

  // One ordered pass: keys above thr, and the need2 lowest columns among the keys equal to it.
  // Item i goes to slot (#keys above thr before i) + min(#keys equal to thr before i, need2); both
  // counts come from one scan of a packed pair (each at most 16384, so no carry crosses).
  const uint32_t per = (total + kRT - 1) / kRT;
  const uint32_t i0 = min(total, per * tid), i1 = min(total, i0 + per);
  uint32_t ngt = 0, neq = 0;
  for (uint32_t i = i0; i < i1; ++i) {
    const uint32_t k = sm.key[i];
    ngt += k > thr ? 1u : 0u;
    neq += k == thr ? 1u : 0u;
  }
  const uint32_t pk = tk_excl_scan<kRT>((neq << 16) | ngt, nullptr, sm.sbuf);
  uint32_t gt = pk & 0xFFFFu, eq = pk >> 16;
  for (uint32_t i = i0; i < i1; ++i) {
    const uint32_t k = sm.key[i];
    if (k > thr) {
      const uint32_t p = gt + min(eq, need2);
      if (p < (uint32_t)a.k) out[p] = (int32_t)sm.col[i];
      ++gt;
    } else if (k == thr) {
      if (eq < need2 && gt + eq < (uint32_t)a.k) out[gt + eq] = (int32_t)sm.col[i];
      ++eq;
    }
  }
  if (tid == 0 && a.len) a.len[t] = a.k;
}

// A row's candidates are in fixed regions of its item list (segment s of S -- a collect segment or
// a score chunk -- owns items s * cap .. s * cap + cap - 1, cap = kTkItemCap / S), and its table
// entry gives (first item, count | lowest digit emitted << 16; 0 for collect segments, which emit
// every key from the row's b0 up).  The histogram, the table and every item
// region are loaded in one round of loads; the searches over a histogram run in one wave while the
// other waves place the items in column order, so the row takes nine workgroup barriers.  Returns
// false (the row is then selected by the exact passes) on the same conditions as the general path.
__device__ __forceinline__ bool resolve_items(const TopkLaunch& a, int t, int n, ResolveSmem& sm) {
  constexpr int IPT = kTkItemCap / kRT;   // item slots per thread
  static_assert(IPT % 2 == 0 && kTkMaxSeg <= kRT, "item slots and table entries per thread");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t* rw = tk_row(a.ws, t);
  int32_t* out = a.idx + (size_t)t * a.k;
  const int S = (n + a.seg - 1) / a.seg;
  const uint32_t cap = (uint32_t)kTkItemCap / (uint32_t)S;

  // one round of loads: this thread's four histogram bins, its table entry and item slots
  // 2 * tid + 2 * kRT * u + {0, 1}
  const uint4 h = reinterpret_cast<const uint4*>(rw)[tid];
  uint2 te = make_uint2(0u, 0u);
  if (tid < S) te = reinterpret_cast<const uint2*>(rw + kTkOffTable)[tid];
  uint4 raw[IPT / 2];
  {
    const uint4* src = reinterpret_cast<const uint4*>(rw + kTkOffItems);
#pragma unroll
    for (int u = 0; u < IPT / 2; ++u) raw[u] = src[tid + kRT * u];
  }
  const uint32_t cnt_s = tid < S ? te.y & 0xFFFFu : 0u;
  const uint32_t low_s = tid < S ? te.y >> 16 : 0u;
  const bool bad = tid < S && (te.x != (uint32_t)tid * cap || cnt_s > cap);
  {   // per-wave sums of the counts (segment prefix sums) and maxima of the lowest emitted digits
    const uint32_t incl = tk_wave_incl_scan(cnt_s);
    const uint32_t mx = tk_wave_max(low_s);
    if (lane == 63) sm.wtot[wave] = incl;
    if (lane == 0) sm.wmax[wave] = mx;
    if (tid < S) sm.tpre[tid] = incl - cnt_s;   // within the wave; the waves before are added below
  }
  const bool overflow = __syncthreads_or(bad) != 0;                          // barrier 1
  // the workspace histogram and counter are cleared for the next call (their values are in registers)
  reinterpret_cast<uint4*>(rw)[tid] = make_uint4(0u, 0u, 0u, 0u);
  if (tid == 0) rw[kTkOffCtr] = 0u;
  if (overflow) {
    return false;
  }
  uint32_t L = 0, woff = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kRT / 64; ++w) {
    const uint32_t x = sm.wtot[w];
    woff += w < wave ? x : 0u;
    total += x;
    L = max(L, sm.wmax[w]);
  }
  if (tid < S) {
    sm.tpre[tid] += woff;
    sm.tst[tid] = cnt_s;
  }
  // the histogram from L up (each chunk added its bins from its own lowest digit up)
  {
    const uint32_t b = 4u * (uint32_t)tid;
    sm.hist[b] = b < L ? 0u : h.x;
    sm.hist[b + 1] = b + 1 < L ? 0u : h.y;
    sm.hist[b + 2] = b + 2 < L ? 0u : h.z;
    sm.hist[b + 3] = b + 3 < L ? 0u : h.w;
  }
  sm.hist1[tid] = 0u;
  if (tid == 0) sm.res[5] = 0u;
  __syncthreads();                                                            // barrier 2
  // wave 0: the first digit b0 of the k-th largest key; every wave: the items into column order
  if (wave == 0) {
    int b0;
    uint32_t need0;
    tk_wave_find_bin<kTkBins>(sm.hist, (uint32_t)a.k, &b0, &need0);
    if (lane == 0) sm.res[0] = (uint32_t)b0;
  }
  {
    const float rcap = 1.0f / (float)cap;
#pragma unroll
    for (int u = 0; u < IPT / 2; ++u) {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const uint32_t slot = 2u * (uint32_t)(tid + kRT * u) + (uint32_t)e;
        uint32_t sg = (uint32_t)((float)slot * rcap);
        if (sg * cap > slot) --sg;
        else if ((sg + 1) * cap <= slot) ++sg;
        const uint32_t j = slot - sg * cap;
        if (sg < (uint32_t)S && j < sm.tst[sg]) {
          const uint32_t p = sm.tpre[sg] + j;
          sm.key[p] = e ? raw[u].z : raw[u].x;
          sm.col[p] = e ? raw[u].w : raw[u].y;
        }
      }
    }
  }
  __syncthreads();                                                            // barrier 3
  const uint32_t b0 = sm.res[0];
  if (L > b0) {   // fewer than k keys at or above L: some chunk may hold keys of the top k it did not emit
    return false;
  }
  // this thread's contiguous range of the items: counts above b0 and at or above it (a check of the
  // histogram against the items), and the second-digit histogram of the items inside b0
  const uint32_t per = (total + kRT - 1) / kRT;
  const uint32_t i0 = min(total, per * (uint32_t)tid), i1 = min(total, i0 + per);
  {
    uint32_t gt = 0, ge = 0;
    for (uint32_t i = i0; i < i1; ++i) {
      const uint32_t k = sm.key[i];
      const uint32_t d = k >> kTkShift0;
      gt += d > b0 ? 1u : 0u;
      ge += d >= b0 ? 1u : 0u;
      if (d == b0) atomicAdd(&sm.hist1[(k >> 10) & 1023u], 1u);
    }
    sm.hist[tid] = 0u;   // the first 1024 bins become the third digit's histogram
    const uint32_t ws = tk_wave_sum((ge << 16) | gt);   // each count is at most 16384
    if (lane == 0) sm.wtot[wave] = ws;
  }
  __syncthreads();                                                            // barrier 4
  uint32_t above_b0 = 0, atleast_b0 = 0;
#pragma unroll
  for (int w = 0; w < kRT / 64; ++w) {
    const uint32_t x = sm.wtot[w];
    above_b0 += x & 0xFFFFu;
    atleast_b0 += x >> 16;
  }
  if (!(above_b0 < (uint32_t)a.k && (uint32_t)a.k <= atleast_b0)) {
    return false;
  }
  const uint32_t need0 = (uint32_t)a.k - above_b0;
  if (wave == 0) {   // the second digit (bits 19..10) of the k-th key among the candidates inside b0
    int d1;
    uint32_t need1;
    tk_wave_find_bin<1024>(sm.hist1, need0, &d1, &need1);
    if (lane == 0) {
      sm.res[1] = (uint32_t)d1;
      sm.res[2] = need1;
      sm.res[3] = sm.hist1[d1];
    }
  }
  __syncthreads();                                                            // barrier 5
  const uint32_t pre22 = (b0 << 10) | sm.res[1];
  const uint32_t need1 = sm.res[2];
  const uint32_t c1 = sm.res[3];   // keys sharing the top 22 bits of the k-th key
  if (c1 <= 64u) {   // typically a handful: collected and ranked in one wave
    for (uint32_t i = i0; i < i1; ++i) {
      const uint32_t k = sm.key[i];
      if ((k >> 10) == pre22) sm.wsum[atomicAdd(&sm.res[5], 1u)] = k;
    }
    __syncthreads();                                                          // barrier 6
    if (wave == 0) {
      const uint32_t c = sm.res[5];
      const uint32_t mine = lane < (int)c ? sm.wsum[lane] : 0u;
      uint32_t above = 0, same = 0;
      for (uint32_t j = 0; j < c; ++j) {
        const uint32_t o = sm.wsum[j];
        above += o > mine ? 1u : 0u;
        same += o == mine ? 1u : 0u;
      }
      if (lane < (int)c && above < need1 && need1 <= above + same) {
        sm.res[6] = mine;
        sm.res[7] = need1 - above;
      }
    }
  } else {           // the third digit (bits 9..0) among the keys sharing the top 22 bits
    for (uint32_t i = i0; i < i1; ++i) {
      const uint32_t k = sm.key[i];
      if ((k >> 10) == pre22) atomicAdd(&sm.hist[k & 1023u], 1u);
    }
    __syncthreads();                                                          // barrier 6
    if (wave == 0) {
      int d2;
      uint32_t need2;
      tk_wave_find_bin<1024>(sm.hist, need1, &d2, &need2);
      if (lane == 0) {
        sm.res[6] = (pre22 << 10) | (uint32_t)d2;
        sm.res[7] = need2;
      }
    }
  }
  __syncthreads();                                                            // barrier 7
  const uint32_t thr = sm.res[6], need2 = sm.res[7];
  // One ordered pass: keys above thr, and the need2 lowest columns among the keys equal to it.
  // Item i goes to slot (#keys above thr before i) + min(#keys equal to thr before i, need2); both
  // counts come from one scan of a packed pair (each at most 16384, so no carry crosses).
  uint32_t ngt = 0, neq = 0;
  for (uint32_t i = i0; i < i1; ++i) {
    const uint32_t k = sm.key[i];
    ngt += k > thr ? 1u : 0u;
    neq += k == thr ? 1u : 0u;
  }
  const uint32_t pk = tk_excl_scan<kRT>((neq << 16) | ngt, nullptr, sm.sbuf);   // barriers 8, 9
  uint32_t gt = pk & 0xFFFFu, eq = pk >> 16;
  for (uint32_t i = i0; i < i1; ++i) {
    const uint32_t k = sm.key[i];
    if (k > thr) {
      const uint32_t p = gt + min(eq, need2);
      if (p < (uint32_t)a.k) out[p] = (int32_t)sm.col[i];
      ++gt;
    } else if (k == thr) {
      if (eq < need2 && gt + eq < (uint32_t)a.k) out[gt + eq] = (int32_t)sm.col[i];
      ++eq;
    }
  }
  if (tid == 0 && a.len) a.len[t] = a.k;
  return true;
}

__global__ void __launch_bounds__(kRT) k_topk_resolve(TopkLaunch a) {
  __shared__ __attribute__((aligned(16))) ResolveSmem sm;
  static_assert(kTkBins == 4 * kRT, "one uint4 of histogram per thread");
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int n = row_n(a, t);
  int32_t* out = a.idx + (size_t)t * a.k;
  uint32_t* rw = tk_row(a.ws, t);
  if (n <= a.k) {   // every visible column, then padding; a histogram left by an earlier call is cleared
    for (int i = tid; i < a.k; i += kRT) out[i] = i < n ? i : -1;
    reinterpret_cast<uint4*>(rw)[tid] = make_uint4(0u, 0u, 0u, 0u);
    if (tid == 0) {
      rw[kTkOffCtr] = 0u;
      if (a.len) a.len[t] = n;
    }
    return;
  }

  const bool done = a.k <= kTkFastK && resolve_items(a, t, n, sm);
  if (!done) {
    finish_streaming(a, t, n, sm);
    if (tid == 0 && a.len) a.len[t] = a.k;
  }
}

// ------------------------------------------------------------------------------------------
// direct: one workgroup per row, no workspace, for rows whose scores no kernel has histogrammed
// (the scores of the grouped and fp32 score kernels, and the separate top-k call)
// ------------------------------------------------------------------------------------------

// Raw float4 slices of a row (layout of tk_load_slices: element (q, e) of thread tid is column
// c0 + 4*kRT*q + 4*tid + e; slices past the row read its last aligned float4 and are masked later).
template <int Q>
__device__ __forceinline__ void row_slices(const float* row, int n, int c0, float4 (&v)[Q]) {
  const int clast = (n - 1) & ~3;
#pragma unroll
  for (int q = 0; q < Q; ++q)
    v[q] = *reinterpret_cast<const float4*>(row + min(c0 + 4 * kRT * q + 4 * (int)threadIdx.x, clast));
}

// Two passes over the row: the first digit's histogram in LDS gives b0 (the digit holding the k-th
// largest key), then every key whose first digit is >= b0 goes straight into LDS in column order
// (the ordered compaction of the collect kernel, without the global item list), and the selection
// finishes there.  Each pass issues the next round's loads before it works on the current round.
// Returns false when the candidates do not fit in LDS (heavy ties: exact passes).
__device__ __forceinline__ bool direct_fast(const TopkLaunch& a, int t, int n, ResolveSmem& sm) {
  constexpr int Q = 2;                 // float4 slices per thread and round
  constexpr int STEP = 4 * kRT * Q;    // columns per round
  const float* row = a.scores + (size_t)t * a.ld;
  const int tid = threadIdx.x;
  auto keys_of = [&](const float4 (&v)[Q], int c0, uint32_t (&key)[Q][4]) {
    uint32_t mask = 0;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int c = c0 + 4 * kRT * q + 4 * tid;
      key[q][0] = score_key(v[q].x);
      key[q][1] = score_key(v[q].y);
      key[q][2] = score_key(v[q].z);
      key[q][3] = score_key(v[q].w);
#pragma unroll
      for (int e = 0; e < 4; ++e) mask |= (c + e < n ? 1u : 0u) << (4 * q + e);
    }
    return mask;
  };
  // pass 1: the first digit's histogram of a sample -- the first 1024 columns of every 8192 (a
  // contiguous eighth of the row, whole memory lines) -- and from it a low digit bs above which the
  // row should hold about twice k keys.  Pass 2 keeps every key at or above bs, so whenever at least
  // k are kept the k-th key is among them and their histogram is exact from bs up; otherwise (or if
  // they overflow) the row takes the exact passes.
  for (int i = tid; i < kTkBins; i += kRT) sm.hist[i] = 0;
  __syncthreads();
  constexpr int kBlk = 8192, kSam = 1024;
  static_assert(kRT == 4 * (kSam / 4), "four sample blocks per round");
  const int nblk = (n + kBlk - 1) / kBlk;
  for (int s0 = 0; s0 < nblk; s0 += 4) {
    const int sb = s0 + (tid >> 8);
    const int c = kBlk * sb + 4 * (tid & 255);
    if (sb < nblk && c < n) {
      const float4 v = *reinterpret_cast<const float4*>(row + c);
      const float ve[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (c + e < n) atomicAdd(&sm.hist[score_key(ve[e]) >> kTkShift0], 1u);
    }
  }
  __syncthreads();
  const uint32_t ns = (uint32_t)((nblk - 1) * kSam + min(kSam, n - kBlk * (nblk - 1)));   // sampled columns
  const uint32_t want = (uint32_t)min((uint64_t)ns, (2ull * (uint64_t)a.k * ns + (uint64_t)n - 1) / (uint64_t)n + 64u);
  int bsi;
  uint32_t unused;
  tk_find_bin<kTkBins, kRT>(sm.hist, want, sm.sbuf, &bsi, &unused);
  const uint32_t bs = (uint32_t)bsi;
  __syncthreads();   // the sample's histogram is read; it now counts the candidates
  for (int i = tid; i < kTkBins; i += kRT) sm.hist[i] = 0;
  __syncthreads();
  // pass 2: the candidates into LDS in column order, and their first digits' histogram
  uint32_t base = 0;
  {
    float4 cur[Q], nxt[Q];
    row_slices<Q>(row, n, 0, cur);
    for (int c0 = 0; c0 < n; c0 += STEP) {
      row_slices<Q>(row, n, c0 + STEP, nxt);   // unconditional (clamped past the row): stays in flight
      uint32_t key[Q][4];
      const uint32_t mask = keys_of(cur, c0, key);
      uint32_t fl[Q], pos[Q];
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        fl[q] = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          fl[q] |= (((mask >> (4 * q + e)) & 1u) && (key[q][e] >> kTkShift0) >= bs ? 1u : 0u) << e;
      }
      const uint32_t tot = tk_ordered_slots<Q, kRT>(fl, pos, sm.wsum);
      if (base + tot > (uint32_t)kTkItemCap) return false;   // (block-uniform)
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        uint32_t p = base + pos[q];
        const uint32_t cq = (uint32_t)(c0 + 4 * kRT * q + 4 * tid);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if ((fl[q] >> e) & 1u) {
            sm.key[p] = key[q][e];
            sm.col[p] = cq + e;
            atomicAdd(&sm.hist[key[q][e] >> kTkShift0], 1u);
            ++p;
          }
      }
      base += tot;
#pragma unroll
      for (int q = 0; q < Q; ++q) cur[q] = nxt[q];
    }
  }
  __syncthreads();   // the items and their histogram are in LDS for every thread
  if (base < (uint32_t)a.k) return false;   // bs was above the k-th key: exact passes (block-uniform)
  int b0i;
  uint32_t need0;
  tk_find_bin<kTkBins, kRT>(sm.hist, (uint32_t)a.k, sm.sbuf, &b0i, &need0);
  select_from_items(a, t, base, (uint32_t)b0i, need0, sm);
  return true;
}

__global__ void __launch_bounds__(kRT) k_topk_direct(TopkLaunch a) {
  __shared__ __attribute__((aligned(16))) ResolveSmem sm;
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int n = row_n(a, t);
  int32_t* out = a.idx + (size_t)t * a.k;
  if (a.ws) {   // a workspace given with the call: leave its row clean, as the resolve kernel does
    uint32_t* rw = tk_row(a.ws, t);
    reinterpret_cast<uint4*>(rw)[tid] = make_uint4(0u, 0u, 0u, 0u);
    if (tid == 0) rw[kTkOffCtr] = 0u;
  }
  if (n <= a.k) {   // every visible column, then padding
    for (int i = tid; i < a.k; i += kRT) out[i] = i < n ? i : -1;
    if (tid == 0 && a.len) a.len[t] = n;
    return;
  }
  const bool done = a.k <= kTkFastK && direct_fast(a, t, n, sm);
  if (!done) {
    finish_streaming(a, t, n, sm);
    if (tid == 0 && a.len) a.len[t] = a.k;
  }
}

}  // namespace

size_t topk_ws_bytes(int T) { return tk_total_words(T) * sizeof(uint32_t); }

hipError_t launch_topk_direct(const TopkLaunch& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  launch(k_topk_direct, dim3(a.T), dim3(kRT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_topk_hist(const TopkLaunch& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const int64_t cols = a.ld < a.ncap ? a.ld : a.ncap;
  const dim3 seg_grid((unsigned)((cols + kTkSeg - 1) / kTkSeg), (unsigned)a.T);
  launch(k_topk_hist, seg_grid, dim3(kCT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_topk(const TopkLaunch& a, bool hist_given, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const int64_t cols = a.ld < a.ncap ? a.ld : a.ncap;
  const dim3 seg_grid((unsigned)((cols + kTkSeg - 1) / kTkSeg), (unsigned)a.T);
  TopkLaunch r = a;
  if (!hist_given && !a.emitted && a.k <= kTkFastK) {   // one pass: segments emit their own candidates
    r.seg = kTkSeg;
    r.emitted = 1;
    launch(k_topk_emit, seg_grid, dim3(kCT), 0, s, r);
    launch(k_topk_resolve, dim3(a.T), dim3(kRT), 0, s, r);
    return hipGetLastError();
  }
  if (!hist_given) launch(k_topk_hist, seg_grid, dim3(kCT), 0, s, a);
  if (!a.emitted) {
    r.seg = kTkSeg;
    if (a.k <= kTkFastK) launch(k_topk_collect, seg_grid, dim3(kCT), 0, s, r);
  }
  launch(k_topk_resolve, dim3(a.T), dim3(kRT), 0, s, r);
  return hipGetLastError();
}

}  // namespace dsa
