// Block-sparse key selection on gfx950 (the MiniMax Sparse Attention steps of "vLLM adds NVFP4
// serving for MiniMax M3.1 Flash at 76 concurrent sequences": 128-token blocks, the index keys
// scanned, 16 blocks kept with the most recent block always among them, exact attention over the
// kept blocks' keys).
//
// A block's score is the largest index score among its visible keys.  Two launches:
//   1. block_max  one wave per block reduces its visible scores (block maxima -> workspace); the
//                 fp8 decode score kernel can write these maxima itself (dsa_indexer_block_select)
//   2. select     one workgroup per query: the block holding the query position is forced in, the
//                 other nblocks-1 are the largest maxima by (score desc, block asc): the
//                 (nblocks-1)-th largest score key by three radix passes over LDS histograms with
//                 the maxima in registers, every key above it, and the lowest blocks among the
//                 keys equal to it (ranked in one wave; when more than 64 keys tie, nblocks-1
//                 rounds of block-wide argmax over (score, -block) packed into one u64 instead).
//                 The kept blocks are then ranked and expanded into ascending key indices with -1
//                 padding.

#include "topk_common.h"

namespace dsa {
namespace {

constexpr int kT = 256;
constexpr int kMaxBlocksKept = 64;

__host__ __device__ inline int64_t nblk_of(int64_t ld, int block) { return (ld + block - 1) / block; }

__global__ void __launch_bounds__(kT) k_block_max(BlockSelectLaunch a) {
  const int t = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t j = (int64_t)blockIdx.x * (kT / 64) + wave;
  int64_t n = (int64_t)a.q_pos[t] + 1;
  n = n < 0 ? 0 : (n > a.ld ? a.ld : n);
  const int64_t lo = j * a.block;
  if (lo >= n) return;
  const int64_t hi = lo + a.block < n ? lo + a.block : n;
  const float* row = a.scores + (size_t)t * a.ld;
  uint32_t best = 0;   // key 0 is below every real score key
  for (int64_t i = lo + lane; i < hi; i += 64) {
    const uint32_t k = score_key(row[i]);
    best = k > best ? k : best;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t y = __shfl_xor(best, o);
    best = y > best ? y : best;
  }
  if (lane == 0) reinterpret_cast<uint32_t*>(a.ws)[(size_t)t * nblk_of(a.ld, a.block) + j] = best;
}

constexpr int kPT = 1024;       // pick threads: 16 waves
constexpr int kPickPer = 16;    // block maxima per thread kept in registers (nb <= 16384)

// Block-wide maximum of one u64 per thread; every thread gets the result.
__device__ uint64_t block_max_u64(uint64_t v, uint64_t* sbuf) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint64_t y = __shfl_xor(v, o);
    v = y > v ? y : v;
  }
  if (lane == 0) sbuf[wave] = v;
  __syncthreads();
  uint64_t r = sbuf[0];
#pragma unroll
  for (int w = 1; w < kPT / 64; ++w) r = sbuf[w] > r ? sbuf[w] : r;
  __syncthreads();
  return r;
}

// Higher score first, then lower block: the score key above the inverted block id.  Every non-NaN
// score key is >= 1, so 0 marks "not a candidate".
__device__ inline uint64_t pack_block(uint32_t key, int64_t j) {
  return (uint64_t)key << 32 | (uint64_t)(0xFFFFFFFFu - (uint32_t)j);
}

struct PickSmem {
  uint32_t hist[4096];   // first digit
  uint32_t h1[1024];     // second and third digits
  uint32_t h2[1024];
  uint32_t res[2];       // a digit search's result: bin, count still needed
  uint32_t sbuf[32];
  int eq[kMaxBlocksKept];
  int cnt, neq;
};

__global__ void __launch_bounds__(kPT) k_block_pick(BlockSelectLaunch a) {
  __shared__ uint64_t sbuf[kPT / 64];
  __shared__ __attribute__((aligned(16))) PickSmem ps;
  __shared__ int chosen[kMaxBlocksKept];
  __shared__ int sorted[kMaxBlocksKept];
  __shared__ int offs[kMaxBlocksKept + 1];
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  int64_t n = (int64_t)a.q_pos[t] + 1;
  n = n < 0 ? 0 : (n > a.ld ? a.ld : n);
  const int64_t nb = (n + a.block - 1) / a.block;
  const uint32_t* bmax = reinterpret_cast<const uint32_t*>(a.ws) + (size_t)t * nblk_of(a.ld, a.block);
  int m;
  if (nb <= a.nblocks) {
    m = (int)nb;
    if (tid < m) chosen[tid] = tid;
  } else {
    m = a.nblocks;
    const int recent = (int)((n - 1) / a.block);
    if (tid == 0) chosen[0] = recent;
    bool done = false;
    if (nb <= (int64_t)kPT * kPickPer) {
      // Exact select of the m-1 largest candidates (score desc, block asc) with the maxima in
      // registers: the (m-1)-th largest key by three radix passes (12, 10 and 10 bits) over LDS
      // histograms, every key above it, and the lowest blocks among the keys equal to it.
      uint32_t v[kPickPer];
#pragma unroll
      for (int i = 0; i < kPickPer; ++i) {
        const int64_t j = tid + (int64_t)kPT * i;
        v[i] = (j < nb && j != recent) ? bmax[j] : 0u;   // every candidate key is >= 1
      }
      uint32_t need = (uint32_t)(m - 1), prefix = 0;
      // the three histograms are cleared together; each digit's bin is then found by one wave
      for (int i = tid; i < 4096; i += kPT) ps.hist[i] = 0u;
      for (int i = tid; i < 1024; i += kPT) { ps.h1[i] = 0u; ps.h2[i] = 0u; }
      __syncthreads();
#pragma unroll 1
      for (int pass = 0; pass < 3; ++pass) {
        const int shift = pass == 0 ? 20 : (pass == 1 ? 10 : 0);
        const int nbins = pass == 0 ? 4096 : 1024;
        uint32_t* h = pass == 0 ? ps.hist : (pass == 1 ? ps.h1 : ps.h2);
#pragma unroll
        for (int i = 0; i < kPickPer; ++i) {
          const uint32_t k = v[i];
          const bool in = k != 0u && (pass == 0 || (k >> (shift + 10)) == prefix);
          if (in) atomicAdd(&h[(k >> shift) & (uint32_t)(nbins - 1)], 1u);
        }
        __syncthreads();
        if (tid < 64) {
          int bin;
          uint32_t left;
          if (pass == 0) tk_wave_find_bin<4096>(h, need, &bin, &left);
          else tk_wave_find_bin<1024>(h, need, &bin, &left);
          if (tid == 0) { ps.res[0] = (uint32_t)bin; ps.res[1] = left; }
        }
        __syncthreads();
        need = ps.res[1];
        prefix = (prefix << (pass == 0 ? 12 : 10)) | ps.res[0];
      }
      const uint32_t thr = prefix;   // the (m-1)-th largest key; `need` of the keys equal to it are kept
      if (tid == 0) { ps.cnt = 1; ps.neq = 0; }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < kPickPer; ++i) {
        const int j = tid + kPT * i;
        if (v[i] > thr) chosen[atomicAdd(&ps.cnt, 1)] = j;
        else if (v[i] == thr && v[i] != 0u) {
          const int e = atomicAdd(&ps.neq, 1);
          if (e < kMaxBlocksKept) ps.eq[e] = j;
        }
      }
      __syncthreads();
      const int neq = ps.neq;
      if (neq <= kMaxBlocksKept) {   // typically a handful of ties: rank them by block in one wave
        if (tid < neq) {
          const int j = ps.eq[tid];
          int rank = 0;
          for (int i = 0; i < neq; ++i) rank += ps.eq[i] < j ? 1 : 0;
          if (rank < (int)need) chosen[ps.cnt + rank] = j;
        }
        done = true;
      }
      __syncthreads();
    }
    if (!done && nb <= (int64_t)kPT * kPickPer) {
      // many equal maxima: nblocks-1 rounds of block-wide argmax over (score, -block)
      uint64_t v[kPickPer];
#pragma unroll
      for (int i = 0; i < kPickPer; ++i) {
        const int64_t j = tid + (int64_t)kPT * i;
        v[i] = (j < nb && j != recent) ? pack_block(bmax[j], j) : 0ull;
      }
      for (int r = 1; r < m; ++r) {
        uint64_t best = 0;
#pragma unroll
        for (int i = 0; i < kPickPer; ++i) best = v[i] > best ? v[i] : best;
        best = block_max_u64(best, sbuf);
        const int j = (int)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFull));
        if (tid == 0) chosen[r] = j;
        if (j % kPT == tid) {
#pragma unroll
          for (int i = 0; i < kPickPer; ++i)
            if (i == j / kPT) v[i] = 0ull;
        }
      }
    } else if (!done) {
      // very many blocks: rescan the maxima from memory each round
      for (int r = 1; r < m; ++r) {
        __syncthreads();
        uint64_t best = 0;
        for (int64_t j = tid; j < nb; j += kPT) {
          bool taken = j == recent;
          for (int c = 1; c < r; ++c) taken |= (chosen[c] == (int)j);
          if (taken) continue;
          const uint64_t v = pack_block(bmax[j], j);
          best = v > best ? v : best;
        }
        best = block_max_u64(best, sbuf);
        if (tid == 0) chosen[r] = (int)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFull));
      }
    }
  }
  __syncthreads();
  // ascending: each chosen block's rank among the chosen ones (distinct ids)
  if (tid < m) {
    const int v = chosen[tid];
    int rank = 0;
    for (int i = 0; i < m; ++i) rank += chosen[i] < v ? 1 : 0;
    sorted[rank] = v;
  }
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int i = 0; i < m; ++i) {
      offs[i] = run;
      const int64_t lo = (int64_t)sorted[i] * a.block;
      run += (int)((lo + a.block <= n) ? a.block : (n - lo));
    }
    offs[m] = run;
  }
  __syncthreads();
  int32_t* out = a.idx + (size_t)t * a.topk;
  const int total = offs[m];
  for (int e = tid; e < a.topk; e += kPT) {
    int32_t val = -1;
    if (e < total) {
      int lo = 0, hi = m - 1;   // the last kept block whose first slot is <= e
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (offs[mid] <= e) lo = mid; else hi = mid - 1;
      }
      val = (int32_t)((int64_t)sorted[lo] * a.block + (e - offs[lo]));
    }
    out[e] = val;
  }
  if (tid == 0 && a.len) a.len[t] = total;
}

}  // namespace

size_t block_select_ws_bytes(int T, int64_t ld, int block) {
  return (size_t)T * (size_t)nblk_of(ld, block) * sizeof(uint32_t);
}

hipError_t launch_block_select(const BlockSelectLaunch& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const int64_t nb = nblk_of(a.ld, a.block);
  dim3 g1((unsigned)((nb + 3) / 4), a.T);
  launch(k_block_max, g1, dim3(kT), 0, s, a);
  launch(k_block_pick, dim3(a.T), dim3(kPT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_block_pick(const BlockSelectLaunch& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  launch(k_block_pick, dim3(a.T), dim3(kPT), 0, s, a);
  return hipGetLastError();
}

}  // namespace dsa
