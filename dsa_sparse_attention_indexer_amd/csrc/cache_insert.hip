// Cache writers of the DSA path on gfx950: the step just before scoring, which puts each new
// token's indexer key and latent row into the FP8 caches that the score and attention kernels read.
//
// Indexer key ("mistral-large4.md", "What differs from GLM-5.2", bullet "The indexer": the key is
// the LayerNorm of the key projection of the token's hidden state, rotated on its first 64 dims on
// RoPE layers; "Day 0 support for Mistral Large 4 on vLLM", "ROCm implementation details", "DSA
// indexer on AITER": the key is quantised to FP8 with one scale per token and written straight
// into the index cache, 132 bytes per token, in the one layout that the readers use):
//   k_kproj    partial projections y = x . wk^T over a slice of the hidden dim for a tile of 64
//              tokens.  Wave w owns outputs 32w..32w+31 (two 16-row M blocks of
//              v_mfma_f32_16x16x32_bf16, weight rows as M) against the tile's four 16-token N
//              blocks.  Both operands pass through LDS in 256-dim blocks loaded one block ahead
//              with whole 512-byte row segments per 32 threads (operands read straight from global
//              memory as 16-byte pieces of 64 rows, one MFMA step per load, reached only ≈1.2 TB/s
//              on the token rows).  The hidden dim is cut into slices that interleave its 256-dim
//              blocks, so that a decode step's handful of tokens still spreads the weight's read
//              over many CUs and the slices of one tile read neighbouring pieces of the same rows;
//              the fp32 partials go to the workspace, [slice][token][128].
//   k_kfinish  one wave per token (one workgroup per token when there are more than four
//              slices, its waves summing interleaved slices), lane j holding dims 2j and 2j+1
//              (exactly one RoPE pair): the slices' sum, LayerNorm with the
//              population variance, the rotation of pairs j < rope_dim/2 by p * inv_freq[j],
//              scale = amax / 448 (1 for an all-zero key) and the codes of k / scale, clamped to
//              +-448 and rounded to nearest even by v_cvt_pk_fp8_f32; one 128-byte row (in a paged
//              cache: its eight 16-byte pieces in the block's 16x16 tiles) and its scale stored at
//              the token's slot.
// Latent row ("Day 0 support for Mistral Large 4 on vLLM", "Model architecture": 512 latent and 64
// rotary dims per token; FP8 with one scale per 64 elements, the layout the attention kernels read):
//   k_latent   one wave per token, 8 lanes per 64-element group (16-byte loads, 8-byte code
//              stores): the rotary group rotated at the token's position on RoPE layers (each lane's
//              four pairs are its own), each group's scale and codes as above.
// Tokens whose slot is negative (padding) or not below the cache's row count are skipped.

#include "dsa_internal.h"

#include <math.h>

#include <algorithm>

namespace dsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kKeyDim = 128;
constexpr int kTileTok = 64;       // tokens per projection tile
constexpr int kNB = kTileTok / 16;  // 16-token MFMA blocks per tile
constexpr int kStep = 32;          // hidden dims per MFMA step
constexpr int kProjThreads = 256;  // 4 waves x 32 outputs
constexpr int kFinThreads = 256;   // key finish: one token per workgroup; latent: 4 tokens
constexpr int kLatRow = 576;
constexpr int kLatGroup = 64;

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

// Two E4M3FN codes of v0 / scale and v1 / scale (clamped to +-448, round to nearest even) in the
// low 16 bits, v0's code in the low byte.
__device__ __forceinline__ uint32_t fp8_pair(float v0, float v1, float scale) {
  const float a = fminf(fmaxf(v0 / scale, -448.f), 448.f);
  const float b = fminf(fmaxf(v1 / scale, -448.f), 448.f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

// LDS tiles of one macro step: kMacro hidden dims of the tile's 64 token rows and of the 128
// weight rows, rows padded by 16 bytes (consecutive rows start 4 banks apart).
constexpr int kMacro = 256;
constexpr int kRowPad = kMacro + 8;
struct ProjSmem {
  uint16_t x[kTileTok][kRowPad];
  uint16_t w[kKeyDim][kRowPad];
};
constexpr int kXPieces = kTileTok * kMacro / 8 / kProjThreads;   // 16-byte pieces per thread
constexpr int kWPieces = kKeyDim * kMacro / 8 / kProjThreads;

// Global -> registers -> LDS, one macro step ahead: 32 consecutive threads read one row's
// kMacro dims (512 contiguous bytes), so every load instruction covers whole row segments.
// Token rows past the end read the last token's row; pieces past the slice read its last piece
// again (in bounds; their steps are not computed), so no load is predicated.
__device__ __forceinline__ void proj_load(const KInsertLaunch& a, int t0, int kc, int kend, u32x4 (&xr)[kXPieces],
                                          u32x4 (&wr)[kWPieces]) {
#pragma unroll
  for (int i = 0; i < kXPieces; ++i) {
    const int pc = i * kProjThreads + (int)threadIdx.x;
    const int row = pc >> 5, col = min(kc + (pc & 31) * 8, kend - 8);
    xr[i] = *reinterpret_cast<const u32x4*>(a.x + (size_t)min(t0 + row, a.T - 1) * a.ld_x + col);
  }
#pragma unroll
  for (int i = 0; i < kWPieces; ++i) {
    const int pc = i * kProjThreads + (int)threadIdx.x;
    const int row = pc >> 5, col = min(kc + (pc & 31) * 8, kend - 8);
    wr[i] = *reinterpret_cast<const u32x4*>(a.wk + (size_t)row * a.D + col);
  }
}

__device__ __forceinline__ void proj_store(ProjSmem& sm, const u32x4 (&xr)[kXPieces], const u32x4 (&wr)[kWPieces]) {
#pragma unroll
  for (int i = 0; i < kXPieces; ++i) {
    const int pc = i * kProjThreads + (int)threadIdx.x;
    *reinterpret_cast<u32x4*>(&sm.x[pc >> 5][(pc & 31) * 8]) = xr[i];
  }
#pragma unroll
  for (int i = 0; i < kWPieces; ++i) {
    const int pc = i * kProjThreads + (int)threadIdx.x;
    *reinterpret_cast<u32x4*>(&sm.w[pc >> 5][(pc & 31) * 8]) = wr[i];
  }
}

__global__ void __launch_bounds__(kProjThreads) k_kproj(KInsertLaunch a) {
  __shared__ __attribute__((aligned(16))) ProjSmem sm;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t0 = blockIdx.x * kTileTok;
  const int split = blockIdx.y;
  const int r = lane & 15, kg = (lane >> 4) * 8;   // operand row within a block, its 8 dims
  float4v acc[2][kNB];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) acc[mb][nb] = float4v{0.f, 0.f, 0.f, 0.f};

  // this slice: the 256-dim blocks split, split + splits, ... (the slices of one tile read
  // neighbouring blocks of the same rows at about the same time), walked from a starting block
  // that depends on the tile, so that the tiles, which share the weight, do not all read the same
  // weight block at the same time
  const int nblk = (a.D + kMacro - 1) / kMacro;
  const int n = (nblk - split + a.splits - 1) / a.splits;
  const int rot = (int)(blockIdx.x % (unsigned)n);
  auto kat = [&](int j) {
    const int jj = j + rot;
    return (split + (jj >= n ? jj - n : jj) * a.splits) * kMacro;
  };
  u32x4 xr[kXPieces], wr[kWPieces];
  proj_load(a, t0, kat(0), min(a.D, kat(0) + kMacro), xr, wr);
  proj_store(sm, xr, wr);
  __syncthreads();
  for (int j = 0; j < n; ++j) {
    const int kc = kat(j);
    const bool more = j + 1 < n;
    if (more) {   // in flight during this block's products
      const int kn = kat(j + 1);
      proj_load(a, t0, kn, min(a.D, kn + kMacro), xr, wr);
    }
    const int nsteps = min(kMacro, a.D - kc) / kStep;
    for (int u = 0; u < nsteps; ++u) {
      bf16x8 wa[2], xb[kNB];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
        wa[mb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&sm.w[32 * wave + 16 * mb + r][u * kStep + kg]));
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb)
        xb[nb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&sm.x[16 * nb + r][u * kStep + kg]));
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[mb], xb[nb], acc[mb][nb], 0, 0, 0);
    }
    if (more) {
      __syncthreads();   // every wave is done reading this macro step's tiles
      proj_store(sm, xr, wr);
      __syncthreads();
    }
  }
  // C block (mb, nb): lane holds outputs 32*wave + 16*mb + 4*(lane/16) + 0..3 of token
  // t0 + 16*nb + lane%16: one 16-byte store into [split][token][128]
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    const int t = t0 + 16 * nb + r;
    if (t < a.T) {
      float* dst = a.ws + ((size_t)split * a.T + t) * kKeyDim + 32 * wave + 4 * (lane >> 4);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) *reinterpret_cast<float4v*>(dst + 16 * mb) = acc[mb][nb];
    }
  }
}

__global__ void __launch_bounds__(kFinThreads) k_kfinish(KInsertLaunch a) {
  __shared__ float2 red[kFinThreads / 64][kKeyDim / 2];
  constexpr int W = kFinThreads / 64;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // up to W slices: one wave per token; more: one workgroup per token, wave w summing the slices
  // w, w + W, ... and wave 0 adding the W sums
  const bool per_wave = a.splits <= W;
  const int t = per_wave ? blockIdx.x * W + wave : blockIdx.x;
  if (t >= a.T) return;
  const int64_t slot = a.slot[t];
  if (slot < 0 || slot >= a.nslots) return;
  const float2* part = reinterpret_cast<const float2*>(a.ws) + (size_t)t * (kKeyDim / 2) + lane;
  const size_t sstride = (size_t)a.T * (kKeyDim / 2);
  float y0 = 0.f, y1 = 0.f;
  if (per_wave) {
    float2 v[W];
#pragma unroll
    for (int i = 0; i < W; ++i) v[i] = part[(size_t)min(i, a.splits - 1) * sstride];
#pragma unroll
    for (int i = 0; i < W; ++i)
      if (i < a.splits) { y0 += v[i].x; y1 += v[i].y; }
  } else {
    int s = wave;
    for (; s + 3 * W < a.splits; s += 4 * W) {
      float2 v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = part[(size_t)(s + i * W) * sstride];
#pragma unroll
      for (int i = 0; i < 4; ++i) { y0 += v[i].x; y1 += v[i].y; }
    }
    for (; s < a.splits; s += W) {
      const float2 v = part[(size_t)s * sstride];
      y0 += v.x;
      y1 += v.y;
    }
    red[wave][lane] = make_float2(y0, y1);
    __syncthreads();
    if (wave != 0) return;
    y0 = 0.f;
    y1 = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) { y0 += red[w][lane].x; y1 += red[w][lane].y; }
  }
  // LayerNorm over the 128 dims
  const float mean = wave_sum(y0 + y1) * (1.f / kKeyDim);
  const float d0 = y0 - mean, d1 = y1 - mean;
  const float var = wave_sum(d0 * d0 + d1 * d1) * (1.f / kKeyDim);
  const float rstd = 1.f / sqrtf(var + a.eps);
  const float b0 = a.ln_b ? a.ln_b[2 * lane] : 0.f, b1 = a.ln_b ? a.ln_b[2 * lane + 1] : 0.f;
  float k0 = d0 * rstd * a.ln_w[2 * lane] + b0;
  float k1 = d1 * rstd * a.ln_w[2 * lane + 1] + b1;
  // RoPE: pair (2j, 2j+1) is lane j's
  if (lane < a.rope_dim / 2) {
    float sn, cs;
    rope_sincos(a.pos[t], a.inv_freq[lane], &sn, &cs);
    const float r0 = k0 * cs - k1 * sn;
    const float r1 = k0 * sn + k1 * cs;
    k0 = r0;
    k1 = r1;
  }
  const float amax = wave_max(fmaxf(fabsf(k0), fabsf(k1)));
  const float scale = amax > 0.f ? amax / 448.f : 1.f;
  // contiguous rows, or the paged layout's 16x16 tiles (bytes 2 lane and 2 lane + 1 share a tile row)
  uint8_t* dst = a.page > 0 ? a.k_cache + (slot / a.page) * a.page * kKeyDim + key_tile_byte((int)(slot % a.page), 2 * lane)
                            : a.k_cache + slot * kKeyDim + 2 * lane;
  *reinterpret_cast<uint16_t*>(dst) = (uint16_t)fp8_pair(k0, k1, scale);
  if (lane == 0) a.k_scale[slot] = scale;
}

// Max over the 8 lanes 8i..8i+7 of a wave (xor shuffles within the group).
__device__ __forceinline__ float group8_max(float x) {
#pragma unroll
  for (int o = 4; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

// Eight codes of v[0..8) / scale, byte i = code of v[i].
__device__ __forceinline__ uint2 fp8_eight(const float (&v)[8], float scale) {
  float q[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) q[i] = fminf(fmaxf(v[i] / scale, -448.f), 448.f);
  uint32_t w0 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
  w0 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], (int)w0, true);
  uint32_t w1 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q[4], q[5], 0, false);
  w1 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q[6], q[7], (int)w1, true);
  return make_uint2(w0, w1);
}

__device__ __forceinline__ void bf16x8_to_f32(const u32x4& raw, float (&v)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(raw[i] << 16);
    v[2 * i + 1] = __uint_as_float(raw[i] & 0xFFFF0000u);
  }
}

__global__ void __launch_bounds__(kFinThreads) k_latent(LatentInsertLaunch a) {
  // one wave per token: lane l holds latent elements 8l..8l+7 (64-element group l/8, its eight
  // lanes reduce the group's maximum), and lanes 0..7 also hold the rotary group's elements
  // 512+8l..512+8l+7, whose four RoPE pairs are all the lane's own
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * (kFinThreads / 64) + wave;
  if (t >= a.T) return;
  const int64_t slot = a.slot[t];
  if (slot < 0 || slot >= a.nslots) return;
  const uint16_t* src = a.kv + (size_t)t * a.ld_kv;
  constexpr int G = kLatRow / kLatGroup;
  const u32x4 raw = *reinterpret_cast<const u32x4*>(src + 8 * lane);
  const u32x4 rraw = *reinterpret_cast<const u32x4*>(src + 512 + 8 * (lane & 7));
  float v[8], r[8];
  bf16x8_to_f32(raw, v);
  bf16x8_to_f32(rraw, r);
  if (a.rope_dim) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float sn, cs;
      rope_sincos(a.pos[t], a.inv_freq[4 * (lane & 7) + i], &sn, &cs);
      const float e = r[2 * i], o = r[2 * i + 1];
      r[2 * i] = e * cs - o * sn;
      r[2 * i + 1] = e * sn + o * cs;
    }
  }
  float m = 0.f, mr = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) { m = fmaxf(m, fabsf(v[i])); mr = fmaxf(mr, fabsf(r[i])); }
  m = group8_max(m);
  mr = group8_max(mr);
  const float scale = m > 0.f ? m / 448.f : 1.f;
  const float rscale = mr > 0.f ? mr / 448.f : 1.f;
  uint8_t* dst = a.kv_cache + slot * kLatRow;
  *reinterpret_cast<uint2*>(dst + 8 * lane) = fp8_eight(v, scale);
  if (lane < 8) *reinterpret_cast<uint2*>(dst + 512 + 8 * lane) = fp8_eight(r, rscale);
  if ((lane & 7) == 0) a.kv_scale[slot * G + (lane >> 3)] = scale;
  if (lane == 0) a.kv_scale[slot * G + G - 1] = rscale;
}

}  // namespace

int kinsert_splits(int T, int D) {
  const int blocks = (D + kMacro - 1) / kMacro;
  const int tiles = (T + kTileTok - 1) / kTileTok;
  const int s = (256 + tiles - 1) / tiles;       // about one workgroup per CU
  return std::max(1, std::min(s, blocks));
}

hipError_t launch_index_k_insert(const KInsertLaunch& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const dim3 g1((unsigned)((a.T + kTileTok - 1) / kTileTok), (unsigned)a.splits);
  launch(k_kproj, g1, dim3(kProjThreads), 0, s, a);
  const int W = kFinThreads / 64;
  const unsigned g2 = a.splits <= W ? (unsigned)((a.T + W - 1) / W) : (unsigned)a.T;
  launch(k_kfinish, dim3(g2), dim3(kFinThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_latent_insert(const LatentInsertLaunch& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const dim3 g((unsigned)((a.T + kFinThreads / 64 - 1) / (kFinThreads / 64)));
  launch(k_latent, g, dim3(kFinThreads), 0, s, a);
  return hipGetLastError();
}

namespace {
// Pool slot of each (sequence, position) by the paged layout rule; negative positions give -1.
__global__ void __launch_bounds__(256) k_paged_slots(Paging pg, int nseq, int n, const int32_t* seq,
                                                      const int32_t* pos, int64_t* slot) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= n) return;
  const int p = pos[j];
  slot[j] = p < 0 ? -1 : paged_slot(pg, clampi(seq[j], 0, nseq - 1), p);
}
}  // namespace

hipError_t launch_paged_slots(const Paging& pg, int nseq, int n, const int32_t* seq, const int32_t* pos, int64_t* slot,
                              hipStream_t s) {
  if (n == 0) return hipSuccess;
  launch(k_paged_slots, dim3((n + 255) / 256), dim3(256), 0, s, pg, nseq, n, seq, pos, slot);
  return hipGetLastError();
}

}  // namespace dsa
