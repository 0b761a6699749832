// Exact per-row top-k selection on gfx950 (radix select over order-preserving u32 keys).
//
// Keeps the k highest scores of each row, equal scores going to the lower column, and emits the
// kept columns in ascending order with -1 padding and the row length ("mistral-large4.md", bullet
// "The indexer": the top 2048 keys are kept; the -1 slots and top-k length bound follow the vLLM
// page's "Top-k compaction" bullet).
//
// A row is cut into 4096-score segments, each handled by one workgroup, so that 16 long rows
// still fill the GPU.  Five launches:
//   1. init     zero the row's digit-0 histogram and candidate counter
//   2. hist     each segment builds an LDS histogram of key bits 31..21 and adds it to the row's
//   3. collect  every segment finds the threshold bin b0 from the row histogram, counts its keys
//               above b0 and appends the keys inside b0 (wave ballot + one atomic per wave)
//   4. resolve  one workgroup per row finishes the radix select on the candidates (bits 20..10,
//               then 9..0) in LDS -- or, when the threshold bin overflowed the candidate buffer
//               (heavy ties), by re-reading the row -- giving the exact k-th key `thr`, how many
//               keys equal to thr are kept (lowest columns first), and per-segment counts
//   5. emit     each segment computes its output offset from the per-segment counts and writes
//               its kept columns in order (block-wide prefix sums)
// Every decision is made on the integer keys, so the result is exact and deterministic.

#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kT = kTopkThreads;
constexpr int kSeg = kTopkSeg;
constexpr int kBins0 = kTopkBins0;
constexpr int kCap = kTopkCap;
constexpr int kResolveThreads = 1024;

// Per-row workspace layout (u32 words).
struct RowWs {
  uint32_t* hist;     // [2048]
  uint32_t* ctrl;     // [16]: 0 cand_cnt, 1 b0, 2 need0, 3 thr, 4 need_eq
  uint32_t* gt;       // [nseg]  keys above the threshold (after resolve: above thr)
  uint32_t* eq;       // [nseg]  keys equal to thr
  uint32_t* ckey;     // [kCap]
  uint32_t* cidx;     // [kCap]
};

__host__ __device__ inline int64_t nseg_of(int64_t ld) { return (ld + kSeg - 1) / kSeg; }
__host__ __device__ inline size_t row_words(int64_t ld) {
  const int64_t ns = nseg_of(ld);
  size_t w = kBins0 + 16 + 2 * (size_t)ns;
  w = (w + 63) & ~size_t(63);
  return w + 2 * (size_t)kCap;
}

__device__ inline RowWs row_ws(void* ws, int64_t ld, int t) {
  uint32_t* base = reinterpret_cast<uint32_t*>(ws) + (size_t)t * row_words(ld);
  const int64_t ns = nseg_of(ld);
  RowWs r;
  r.hist = base;
  r.ctrl = base + kBins0;
  r.gt = r.ctrl + 16;
  r.eq = r.gt + ns;
  size_t off = (kBins0 + 16 + 2 * (size_t)ns + 63) & ~size_t(63);
  r.ckey = base + off;
  r.cidx = r.ckey + kCap;
  return r;
}

__device__ inline int row_n(const TopkLaunch& a, int t) {
  int64_t n = (int64_t)a.q_pos[t] + 1;
  if (n < 0) n = 0;
  if (n > a.ld) n = a.ld;
  return (int)n;
}

// Block-wide exclusive prefix sum over blockDim.x threads (multiple of 64, <= 1024).
__device__ uint32_t block_excl_scan(uint32_t v, uint32_t* total, uint32_t* sbuf /* >= 17 words */) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) sbuf[wave] = x;
  __syncthreads();
  if (tid == 0) {
    uint32_t run = 0;
    for (int w = 0; w < nw; ++w) { uint32_t s = sbuf[w]; sbuf[w] = run; run += s; }
    sbuf[16] = run;
  }
  __syncthreads();
  const uint32_t r = sbuf[wave] + x - v;
  if (total) *total = sbuf[16];
  __syncthreads();
  return r;
}

// Finds the bin holding the `need`-th largest key of a histogram with nb bins (nb a multiple of
// blockDim.x).  Returns the bin through *bin and the count still needed inside it through *need_in;
// exactly one thread writes them.
__device__ void find_bin(const uint32_t* h, int nb, uint32_t need, uint32_t* sbuf, int* bin, uint32_t* need_in) {
  const int tid = threadIdx.x;
  const int per = nb / (int)blockDim.x;
  const int hi = nb - per * tid;           // thread 0 owns the top bins
  uint32_t local = 0;
  for (int i = 1; i <= per; ++i) local += h[hi - i];
  uint32_t above = block_excl_scan(local, nullptr, sbuf);
  for (int i = 1; i <= per; ++i) {
    const uint32_t c = h[hi - i];
    if (above < need && need <= above + c) { *bin = hi - i; *need_in = need - above; }
    above += c;
  }
  __syncthreads();
}

__global__ void __launch_bounds__(kT) k_topk_init(TopkLaunch a) {
  RowWs r = row_ws(a.ws, a.ld, blockIdx.x);
  for (int i = threadIdx.x; i < kBins0; i += kT) r.hist[i] = 0;
  if (threadIdx.x < 16) r.ctrl[threadIdx.x] = 0;
}

// Loads this thread's 16 scores of segment `seg` (coalesced float4s), as keys; invalid -> flagged.
__device__ __forceinline__ void load_keys16(const float* row, int n, int s0, uint32_t key[16], bool ok[16], int col[16]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = s0 + 1024 * i + 4 * threadIdx.x;
    if (c + 3 < n) {
      const float4 v = *reinterpret_cast<const float4*>(row + c);
      key[4 * i + 0] = score_key(v.x); key[4 * i + 1] = score_key(v.y);
      key[4 * i + 2] = score_key(v.z); key[4 * i + 3] = score_key(v.w);
#pragma unroll
      for (int j = 0; j < 4; ++j) ok[4 * i + j] = true;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ok[4 * i + j] = c + j < n;
        key[4 * i + j] = ok[4 * i + j] ? score_key(row[c + j]) : 0u;
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) col[4 * i + j] = c + j;
  }
}

__global__ void __launch_bounds__(kT) k_topk_hist(TopkLaunch a) {
  __shared__ uint32_t lh[kBins0];
  const int t = blockIdx.y, seg = blockIdx.x;
  const int n = row_n(a, t);
  if (n <= a.k || seg * kSeg >= n) return;
  for (int i = threadIdx.x; i < kBins0; i += kT) lh[i] = 0;
  __syncthreads();
  uint32_t key[16]; bool ok[16]; int col[16];
  load_keys16(a.scores + (size_t)t * a.ld, n, seg * kSeg, key, ok, col);
#pragma unroll
  for (int i = 0; i < 16; ++i)
    if (ok[i]) atomicAdd(&lh[key[i] >> 21], 1u);
  __syncthreads();
  RowWs r = row_ws(a.ws, a.ld, t);
  for (int i = threadIdx.x; i < kBins0; i += kT)
    if (lh[i]) atomicAdd(&r.hist[i], lh[i]);
}

__global__ void __launch_bounds__(kT) k_topk_collect(TopkLaunch a) {
  __shared__ uint32_t lh[kBins0];
  __shared__ uint32_t sbuf[24];
  __shared__ int s_bin;
  __shared__ uint32_t s_need;
  const int t = blockIdx.y, seg = blockIdx.x;
  const int n = row_n(a, t);
  if (n <= a.k || seg * kSeg >= n) return;
  RowWs r = row_ws(a.ws, a.ld, t);
  for (int i = threadIdx.x; i < kBins0; i += kT) lh[i] = r.hist[i];
  __syncthreads();
  int bin = -1; uint32_t need = 0;
  find_bin(lh, kBins0, (uint32_t)a.k, sbuf, &bin, &need);
  if (bin >= 0) { s_bin = bin; s_need = need; }
  __syncthreads();
  const uint32_t b0 = (uint32_t)s_bin;
  uint32_t key[16]; bool ok[16]; int col[16];
  load_keys16(a.scores + (size_t)t * a.ld, n, seg * kSeg, key, ok, col);
  uint32_t gt = 0;
  const int lane = threadIdx.x & 63;
  const uint64_t below = (1ull << lane) - 1ull;
  // one returning atomic per wave: count this wave's candidates first, then place them
  uint64_t masks[16];
  uint32_t wave_cnt = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t d = key[i] >> 21;
    gt += (ok[i] && d > b0) ? 1u : 0u;
    masks[i] = __ballot(ok[i] && d == b0);
    wave_cnt += (uint32_t)__popcll(masks[i]);
  }
  if (wave_cnt) {
    uint32_t base = 0;
    if (lane == 0) base = atomicAdd(&r.ctrl[0], wave_cnt);
    base = __shfl(base, 0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if ((masks[i] >> lane) & 1ull) {
        const uint32_t pos = base + (uint32_t)__popcll(masks[i] & below);
        if (pos < (uint32_t)kCap) { r.ckey[pos] = key[i]; r.cidx[pos] = (uint32_t)col[i]; }
      }
      base += (uint32_t)__popcll(masks[i]);
    }
  }
  uint32_t tot;
  block_excl_scan(gt, &tot, sbuf);
  if (threadIdx.x == 0) {
    r.gt[seg] = tot;
    r.eq[seg] = 0;
    if (seg == 0) { r.ctrl[1] = b0; r.ctrl[2] = s_need; }
  }
}

// Radix step over keys held in LDS: among keys whose bits above `shift+bits` equal `prefix`,
// histogram the `bits`-wide digit at `shift`, and find the digit holding the need-th largest.
__device__ void lds_radix_step(const uint32_t* keys, int cnt, uint32_t prefix, int hi_shift, int shift, int bits,
                               uint32_t* hist, uint32_t* sbuf, uint32_t need, int* digit, uint32_t* need_out) {
  const int nb = 1 << bits;
  for (int i = threadIdx.x; i < nb; i += blockDim.x) hist[i] = 0;
  __syncthreads();
  for (int i = threadIdx.x; i < cnt; i += blockDim.x) {
    const uint32_t k = keys[i];
    if ((k >> hi_shift) == prefix) atomicAdd(&hist[(k >> shift) & (nb - 1)], 1u);
  }
  __syncthreads();
  __shared__ int s_d;
  __shared__ uint32_t s_n;
  int d = -1; uint32_t nn = 0;
  find_bin(hist, nb, need, sbuf, &d, &nn);
  if (d >= 0) { s_d = d; s_n = nn; }
  __syncthreads();
  *digit = s_d;
  *need_out = s_n;
  __syncthreads();
}

// Same as lds_radix_step but streaming the whole row from global memory.
__device__ void row_radix_step(const float* row, int n, uint32_t prefix, int hi_shift, int shift, int bits,
                               uint32_t* hist, uint32_t* sbuf, uint32_t need, int* digit, uint32_t* need_out) {
  const int nb = 1 << bits;
  for (int i = threadIdx.x; i < nb; i += blockDim.x) hist[i] = 0;
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const uint32_t k = score_key(row[i]);
    if ((k >> hi_shift) == prefix) atomicAdd(&hist[(k >> shift) & (nb - 1)], 1u);
  }
  __syncthreads();
  __shared__ int s_d;
  __shared__ uint32_t s_n;
  int d = -1; uint32_t nn = 0;
  find_bin(hist, nb, need, sbuf, &d, &nn);
  if (d >= 0) { s_d = d; s_n = nn; }
  __syncthreads();
  *digit = s_d;
  *need_out = s_n;
  __syncthreads();
}

__global__ void __launch_bounds__(kResolveThreads) k_topk_resolve(TopkLaunch a) {
  __shared__ uint32_t skey[kCap];
  __shared__ uint32_t sidx[kCap];
  __shared__ uint32_t hist[8 * kResolveThreads];
  __shared__ uint32_t sbuf[24];
  const int t = blockIdx.x;
  const int n = row_n(a, t);
  if (n <= a.k) return;
  RowWs r = row_ws(a.ws, a.ld, t);
  const uint32_t cnt = r.ctrl[0];
  const uint32_t b0 = r.ctrl[1];
  const uint32_t need0 = r.ctrl[2];
  const int ns = (int)((n + kSeg - 1) / kSeg);
  int d1, d2;
  uint32_t need1, need2;
  uint32_t thr;
  uint32_t* gtc = hist;                // reused after the radix steps: [ns] gt counts
  uint32_t* eqc = hist + kTopkMaxSegs; // [ns] eq counts (hist holds 8192 words; ns <= 1024)
  if (cnt <= (uint32_t)kCap) {
    for (uint32_t i = threadIdx.x; i < cnt; i += kResolveThreads) { skey[i] = r.ckey[i]; sidx[i] = r.cidx[i]; }
    __syncthreads();
    lds_radix_step(skey, (int)cnt, b0, 21, 10, 11, hist, sbuf, need0, &d1, &need1);
    lds_radix_step(skey, (int)cnt, (b0 << 11) | (uint32_t)d1, 10, 0, 10, hist, sbuf, need1, &d2, &need2);
    thr = (b0 << 21) | ((uint32_t)d1 << 10) | (uint32_t)d2;
    for (int i = threadIdx.x; i < 2 * kTopkMaxSegs; i += kResolveThreads) hist[i] = 0;
    __syncthreads();
    for (uint32_t i = threadIdx.x; i < cnt; i += kResolveThreads) {
      const uint32_t k = skey[i];
      const int s = (int)(sidx[i] / kSeg);
      if (k > thr) atomicAdd(&gtc[s], 1u);
      else if (k == thr) atomicAdd(&eqc[s], 1u);
    }
    __syncthreads();
    for (int s = threadIdx.x; s < ns; s += kResolveThreads) { r.gt[s] += gtc[s]; r.eq[s] = eqc[s]; }
  } else {
    const float* row = a.scores + (size_t)t * a.ld;
    row_radix_step(row, n, b0, 21, 10, 11, hist, sbuf, need0, &d1, &need1);
    row_radix_step(row, n, (b0 << 11) | (uint32_t)d1, 10, 0, 10, hist, sbuf, need1, &d2, &need2);
    thr = (b0 << 21) | ((uint32_t)d1 << 10) | (uint32_t)d2;
    for (int i = threadIdx.x; i < 2 * kTopkMaxSegs; i += kResolveThreads) hist[i] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += kResolveThreads) {
      const uint32_t k = score_key(row[i]);
      if (k > thr) atomicAdd(&gtc[i / kSeg], 1u);
      else if (k == thr) atomicAdd(&eqc[i / kSeg], 1u);
    }
    __syncthreads();
    for (int s = threadIdx.x; s < ns; s += kResolveThreads) { r.gt[s] = gtc[s]; r.eq[s] = eqc[s]; }
  }
  if (threadIdx.x == 0) { r.ctrl[3] = thr; r.ctrl[4] = need2; }
}

__global__ void __launch_bounds__(kT) k_topk_emit(TopkLaunch a) {
  __shared__ uint32_t sbuf[24];
  __shared__ uint32_t s_base, s_eqb;
  const int t = blockIdx.y, seg = blockIdx.x;
  const int n = row_n(a, t);
  int32_t* out = a.idx + (size_t)t * a.k;
  const int s0 = seg * kSeg;
  if (n <= a.k) {
    for (int i = s0 + threadIdx.x; i < min(n, s0 + kSeg); i += kT) out[i] = i;
    if (seg == 0) {
      for (int i = n + threadIdx.x; i < a.k; i += kT) out[i] = -1;
      if (threadIdx.x == 0 && a.len) a.len[t] = n;
    }
    return;
  }
  if (s0 >= n) return;
  RowWs r = row_ws(a.ws, a.ld, t);
  const uint32_t thr = r.ctrl[3];
  const uint32_t need_eq = r.ctrl[4];
  // Offsets of this segment: eq keys are taken lowest column first, so segment s keeps
  // min(eq_s, need_eq - eq_before_s) of its eq keys.
  {
    uint32_t eqb = 0, base = 0;
    // each thread sums a contiguous run of the earlier segments; two block scans merge them
    const int per = (seg + kT - 1) / kT;
    const int lo = threadIdx.x * per, hi = min(seg, lo + per);
    uint32_t e_local = 0;
    for (int s = lo; s < hi; ++s) e_local += r.eq[s];
    uint32_t e_tot;
    const uint32_t e_before = block_excl_scan(e_local, &e_tot, sbuf);
    uint32_t sel_local = 0, run = e_before;
    for (int s = lo; s < hi; ++s) {
      const uint32_t e = r.eq[s];
      const uint32_t rem = need_eq > run ? need_eq - run : 0u;
      sel_local += r.gt[s] + (e < rem ? e : rem);
      run += e;
    }
    uint32_t sel_tot;
    block_excl_scan(sel_local, &sel_tot, sbuf);
    eqb = e_tot;
    base = sel_tot;
    if (threadIdx.x == 0) { s_base = base; s_eqb = eqb; }
    __syncthreads();
  }
  const uint32_t base = s_base, eqb = s_eqb;
  // This thread's 16 contiguous scores.
  const float* row = a.scores + (size_t)t * a.ld;
  const int c0 = s0 + 16 * threadIdx.x;
  uint32_t key[16];
  bool ok[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    ok[i] = c0 + i < n;
    key[i] = ok[i] ? score_key(row[c0 + i]) : 0u;
  }
  uint32_t neq = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) neq += (ok[i] && key[i] == thr) ? 1u : 0u;
  uint32_t tmp;
  uint32_t eq_rank = eqb + block_excl_scan(neq, &tmp, sbuf);
  uint32_t sel_mask = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    bool sel = false;
    if (ok[i]) {
      if (key[i] > thr) sel = true;
      else if (key[i] == thr) { sel = eq_rank < need_eq; ++eq_rank; }
    }
    sel_mask |= sel ? (1u << i) : 0u;
  }
  uint32_t pos = base + block_excl_scan((uint32_t)__popc(sel_mask), &tmp, sbuf);
#pragma unroll
  for (int i = 0; i < 16; ++i)
    if (sel_mask & (1u << i)) {
      if (pos < (uint32_t)a.k) out[pos] = c0 + i;   // always true when the counts are consistent
      ++pos;
    }
  if (seg == 0 && threadIdx.x == 0 && a.len) a.len[t] = a.k;
}

}  // namespace

size_t topk_row_bytes(int64_t ld) { return row_words(ld) * sizeof(uint32_t); }

hipError_t launch_topk(const TopkLaunch& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const int ns = (int)nseg_of(a.ld);
  hipLaunchKernelGGL(k_topk_init, dim3(a.T), dim3(kT), 0, s, a);
  hipLaunchKernelGGL(k_topk_hist, dim3(ns, a.T), dim3(kT), 0, s, a);
  hipLaunchKernelGGL(k_topk_collect, dim3(ns, a.T), dim3(kT), 0, s, a);
  hipLaunchKernelGGL(k_topk_resolve, dim3(a.T), dim3(kResolveThreads), 0, s, a);
  hipLaunchKernelGGL(k_topk_emit, dim3(ns, a.T), dim3(kT), 0, s, a);
  return hipGetLastError();
}

}  // namespace dsa
