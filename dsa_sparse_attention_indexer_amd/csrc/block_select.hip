// Block-sparse key selection on gfx950 (the MiniMax Sparse Attention steps of "vLLM adds NVFP4
// serving for MiniMax M3.1 Flash at 76 concurrent sequences": 128-token blocks, the index keys
// scanned, 16 blocks kept with the most recent block always among them, exact attention over the
// kept blocks' keys).
//
// A block's score is the largest index score among its visible keys.  Two launches:
//   1. block_max  one wave per block reduces its visible scores (block maxima -> workspace)
//   2. select     one workgroup per query: the block holding the query position is forced in, the
//                 other nblocks-1 are taken by repeated block-wide argmax over (score, -block)
//                 packed into one u64 (so equal scores go to the lower block), then the kept
//                 blocks are expanded into ascending key indices with -1 padding.

#include "dsa_internal.h"

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
  for (int w = 1; w < kT / 64; ++w) r = sbuf[w] > r ? sbuf[w] : r;
  __syncthreads();
  return r;
}

__global__ void __launch_bounds__(kT) k_block_pick(BlockSelectLaunch a) {
  __shared__ uint64_t sbuf[kT / 64];
  __shared__ int chosen[kMaxBlocksKept];
  __shared__ int nchosen;
  __shared__ int offs[kMaxBlocksKept + 1];
  const int t = blockIdx.x;
  int64_t n = (int64_t)a.q_pos[t] + 1;
  n = n < 0 ? 0 : (n > a.ld ? a.ld : n);
  const int64_t nb = (n + a.block - 1) / a.block;
  const uint32_t* bmax = reinterpret_cast<const uint32_t*>(a.ws) + (size_t)t * nblk_of(a.ld, a.block);
  if (threadIdx.x == 0) nchosen = 0;
  __syncthreads();
  if (nb <= a.nblocks) {
    if (threadIdx.x < nb) chosen[threadIdx.x] = (int)threadIdx.x;
    if (threadIdx.x == 0) nchosen = (int)nb;
  } else {
    const int recent = (int)((n - 1) / a.block);
    if (threadIdx.x == 0) { chosen[0] = recent; nchosen = 1; }
    __syncthreads();
    for (int r = 1; r < a.nblocks; ++r) {
      uint64_t best = 0;
      for (int64_t j = threadIdx.x; j < nb; j += kT) {
        bool taken = false;
        for (int c = 0; c < r; ++c) taken |= (chosen[c] == (int)j);
        if (taken) continue;
        // higher score first, then lower block: the score key above the inverted block id
        // (every non-NaN score key is >= 1, so 0 never wins)
        const uint64_t v = (uint64_t)bmax[j] << 32 | (uint64_t)(0xFFFFFFFFu - (uint32_t)j);
        best = v > best ? v : best;
      }
      best = block_max_u64(best, sbuf);
      if (threadIdx.x == 0) { chosen[r] = (int)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFull)); nchosen = r + 1; }
      __syncthreads();
    }
  }
  __syncthreads();
  const int m = nchosen;
  if (threadIdx.x == 0) {
    // ascending order (m <= 64: insertion sort), then output offsets
    for (int i = 1; i < m; ++i) {
      const int v = chosen[i];
      int j = i - 1;
      while (j >= 0 && chosen[j] > v) { chosen[j + 1] = chosen[j]; --j; }
      chosen[j + 1] = v;
    }
    int run = 0;
    for (int i = 0; i < m; ++i) {
      offs[i] = run;
      const int64_t lo = (int64_t)chosen[i] * a.block;
      const int64_t cnt = (lo + a.block <= n) ? a.block : (n - lo);
      run += (int)cnt;
    }
    offs[m] = run;
  }
  __syncthreads();
  int32_t* out = a.idx + (size_t)t * a.topk;
  for (int i = 0; i < m; ++i) {
    const int64_t lo = (int64_t)chosen[i] * a.block;
    const int cnt = offs[i + 1] - offs[i];
    for (int e = threadIdx.x; e < cnt; e += kT) out[offs[i] + e] = (int32_t)(lo + e);
  }
  for (int e = offs[m] + threadIdx.x; e < a.topk; e += kT) out[e] = -1;
  if (threadIdx.x == 0 && a.len) a.len[t] = offs[m];
}

}  // namespace

size_t block_select_ws_bytes(int T, int64_t ld, int block) {
  return (size_t)T * (size_t)nblk_of(ld, block) * sizeof(uint32_t);
}

hipError_t launch_block_select(const BlockSelectLaunch& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const int64_t nb = nblk_of(a.ld, a.block);
  dim3 g1((unsigned)((nb + 3) / 4), a.T);
  hipLaunchKernelGGL(k_block_max, g1, dim3(kT), 0, s, a);
  hipLaunchKernelGGL(k_block_pick, dim3(a.T), dim3(kT), 0, s, a);
  return hipGetLastError();
}

}  // namespace dsa
