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
//              blocks; every operand is 8 consecutive bf16 of one row, loaded straight from global
//              memory (16 bytes per lane).  The hidden dim is cut into slices so that a decode
//              step's handful of tokens still spreads the weight's read over many CUs; the fp32
//              partials go to the workspace, [slice][token][128].
//   k_kfinish  one workgroup per token: its four waves sum interleaved slices, then one wave, lane
//              j holding dims 2j and 2j+1 (exactly one RoPE pair), applies LayerNorm with the
//              population variance, the rotation of pairs j < rope_dim/2 by p * inv_freq[j],
//              scale = amax / 448 (1 for an all-zero key) and the codes of k / scale, clamped to
//              +-448 and rounded to nearest even by v_cvt_pk_fp8_f32; one 128-byte row and its
//              scale stored at the token's slot.
// Latent row ("Day 0 support for Mistral Large 4 on vLLM", "Model architecture": 512 latent and 64
// rotary dims per token; FP8 with one scale per 64 elements, the layout the attention kernels read):
//   k_latent   one wave per token: per 64-element group the bf16 values, the rotary group rotated
//              at the token's position on RoPE layers, the group's scale and codes as above.
// Tokens whose slot is negative (padding) or not below the cache's row count are skipped.

#include "dsa_internal.h"

#include <math.h>

namespace dsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));

constexpr int kKeyDim = 128;
constexpr int kTileTok = 64;       // tokens per projection tile
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

__device__ __forceinline__ bf16x8 load8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

__global__ void __launch_bounds__(kProjThreads) k_kproj(KInsertLaunch a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t0 = blockIdx.x * kTileTok;
  const int split = blockIdx.y;
  const int kbeg = split * a.steps_per_split * kStep;
  const int kend = min(a.D, kbeg + a.steps_per_split * kStep);
  const int r = lane & 15, kg = (lane >> 4) * 8;   // operand row within a block, its 8 dims
  // A operands: weight rows 32*wave + 16*mb + r; B operands: token rows t0 + 16*nb + r (tokens
  // past the end read the last token's row and are not stored)
  const uint16_t* wrow[2];
  const uint16_t* xrow[4];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) wrow[mb] = a.wk + (size_t)(32 * wave + 16 * mb + r) * a.D + kg;
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) xrow[nb] = a.x + (size_t)min(t0 + 16 * nb + r, a.T - 1) * a.ld_x + kg;
  float4v acc[2][4];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = float4v{0.f, 0.f, 0.f, 0.f};
  bf16x8 wa[2], xb[4];
  if (kbeg < kend) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) wa[mb] = load8(wrow[mb] + kbeg);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) xb[nb] = load8(xrow[nb] + kbeg);
  }
  for (int k = kbeg; k < kend; k += kStep) {
    // the next step's operands are in flight while this step's products run
    const int kn = k + kStep < kend ? k + kStep : k;
    bf16x8 wn[2], xn[4];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) wn[mb] = load8(wrow[mb] + kn);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) xn[nb] = load8(xrow[nb] + kn);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[mb], xb[nb], acc[mb][nb], 0, 0, 0);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) wa[mb] = wn[mb];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) xb[nb] = xn[nb];
  }
  // C block (mb, nb): lane holds outputs 32*wave + 16*mb + 4*(lane/16) + 0..3 of token
  // t0 + 16*nb + lane%16: one 16-byte store into [split][token][128]
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
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
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x;
  const int64_t slot = a.slot[t];
  if (slot < 0 || slot >= a.nslots) return;
  // wave w sums the slices s = w, w + 4, ...; wave 0 then adds the four sums
  const float2* part = reinterpret_cast<const float2*>(a.ws) + (size_t)t * (kKeyDim / 2) + lane;
  const size_t sstride = (size_t)a.T * (kKeyDim / 2);
  constexpr int W = kFinThreads / 64;
  float y0 = 0.f, y1 = 0.f;
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
  reinterpret_cast<uint16_t*>(a.k_cache + slot * kKeyDim)[lane] = (uint16_t)fp8_pair(k0, k1, scale);
  if (lane == 0) a.k_scale[slot] = scale;
}

__global__ void __launch_bounds__(kFinThreads) k_latent(LatentInsertLaunch a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * (kFinThreads / 64) + wave;
  if (t >= a.T) return;
  const int64_t slot = a.slot[t];
  if (slot < 0 || slot >= a.nslots) return;
  const uint16_t* src = a.kv + (size_t)t * a.ld_kv;
  constexpr int G = kLatRow / kLatGroup;
  float v[G];
#pragma unroll
  for (int g = 0; g < G; ++g) v[g] = __uint_as_float((uint32_t)src[g * kLatGroup + lane] << 16);
  if (a.rope_dim) {
    // the rotary group: lanes 2j and 2j+1 hold pair j
    float sn, cs;
    rope_sincos(a.pos[t], a.inv_freq[lane >> 1], &sn, &cs);
    const float other = __shfl_xor(v[G - 1], 1);
    v[G - 1] = (lane & 1) ? other * sn + v[G - 1] * cs : v[G - 1] * cs - other * sn;
  }
  uint8_t* dst = a.kv_cache + slot * kLatRow;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float amax = wave_max(fabsf(v[g]));
    const float scale = amax > 0.f ? amax / 448.f : 1.f;
    dst[g * kLatGroup + lane] = (uint8_t)fp8_pair(v[g], 0.f, scale);
    if (lane == 0) a.kv_scale[slot * G + g] = scale;
  }
}

}  // namespace

void kinsert_geometry(int T, int D, int* splits, int* steps_per_split) {
  const int steps = D / kStep;
  const int tiles = (T + kTileTok - 1) / kTileTok;
  int s = (256 + tiles - 1) / tiles;             // about one workgroup per CU
  s = std::min(s, std::max(1, steps / 2));       // at least two steps per slice
  s = std::max(s, 1);
  const int per = (steps + s - 1) / s;
  *steps_per_split = per;
  *splits = (steps + per - 1) / per;             // no empty slice
}

hipError_t launch_index_k_insert(const KInsertLaunch& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const dim3 g1((unsigned)((a.T + kTileTok - 1) / kTileTok), (unsigned)a.splits);
  hipLaunchKernelGGL(k_kproj, g1, dim3(kProjThreads), 0, s, a);
  hipLaunchKernelGGL(k_kfinish, dim3((unsigned)a.T), dim3(kFinThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_latent_insert(const LatentInsertLaunch& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const dim3 g((unsigned)((a.T + kFinThreads / 64 - 1) / (kFinThreads / 64)));
  hipLaunchKernelGGL(k_latent, g, dim3(kFinThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace dsa
