// Sparse absorbed-MLA attention on gfx950: exact softmax attention of every head over the keys
// the indexer selected ("Day 0 support for Mistral Large 4 on vLLM": MLA with KV LoRA rank 512
// and RoPE dim 64, one latent KV head shared by all 64 heads, V = the latent; NoPE layers are
// the same with zero RoPE dims on the same cache layout).
//
// fp8 cache, bf16 query (matrix-core path), one workgroup = 4 waves = up to 64 heads:
//   * 32-key tiles are gathered by row index into LDS as raw fp8 bytes plus their per-64 scales,
//     then dequantised once per workgroup to bf16 (code * scale, rounded to nearest even) in two
//     layouts: key-major rows for Q.K^T and a dim-major transpose for P.V.
//   * wave w owns heads 16w..16w+15.  Its bf16 query stays in registers as the B operand of
//     v_mfma_f32_16x16x32_bf16 (S^T = K Q^T, keys as M).  The key rows are placed in LDS in an
//     order that makes the S^T accumulator of each lane hold exactly the 8 consecutive keys that
//     the P.V step needs in its B operand, so probabilities go from accumulators to MFMA operands
//     without touching LDS.
//   * online softmax in the log2 domain with fp32 statistics; O^T = V^T P^T accumulates in fp32.
// fp32 cache, fp32 query: the same tiling with fp32 vector FMAs (8 lanes per head).
//
// Decode splits a query's selection over `splits` workgroups; each writes an unnormalised partial
// output with its running max and sum, and a combine kernel merges them exactly.

#include "dsa_internal.h"

#include <math.h>

namespace dsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kTileK = 32;
constexpr int kRow = 576;                 // latent row: 512 + 64
constexpr int kLora = 512;
constexpr int kBlocks = kRow / 64;        // scales per row
constexpr int kKsStride = kRow + 8;       // bf16 per key-major row (1168 B: rows shift by 4 banks)
constexpr int kVtStride = kTileK + 8;     // bf16 per dim-major row (80 B)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct Fp8Smem {
  uint8_t raw[kTileK][kRow];
  float sc[kTileK][kBlocks];
  int row[kTileK];
  int valid[kTileK];
  uint16_t ks[kTileK][kKsStride];
  uint16_t vt[kLora][kVtStride];
};

// Key kappa (0..31) of a tile lives in key-major LDS row 16*((kappa>>2)&1) + 4*(kappa>>3) + (kappa&3).
__device__ __forceinline__ int ks_row_of_key(int kappa) {
  return 16 * ((kappa >> 2) & 1) + 4 * (kappa >> 3) + (kappa & 3);
}

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return (uint32_t)float_to_bf16_bits(lo) | ((uint32_t)float_to_bf16_bits(hi) << 16);
}

__device__ __forceinline__ void write_partial_or_final(const MlaLaunch& a, int t, int split, int head,
                                                       float m_log2, float l_tot, const float* o, int d0,
                                                       int ndim) {
  // o: ndim consecutive output dims starting at d0 for this head (unnormalised)
  if (a.splits == 1) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    float* dst = a.out + ((size_t)t * a.H + head) * a.kv_lora + d0;
    for (int i = 0; i < ndim; i += 4)
      *reinterpret_cast<float4*>(dst + i) = make_float4(o[i] * inv, o[i + 1] * inv, o[i + 2] * inv, o[i + 3] * inv);
  } else {
    float* dst = a.ws + (((size_t)t * a.splits + split) * a.H + head) * a.kv_lora + d0;
    for (int i = 0; i < ndim; i += 4)
      *reinterpret_cast<float4*>(dst + i) = make_float4(o[i], o[i + 1], o[i + 2], o[i + 3]);
  }
}

__device__ __forceinline__ void write_stats(const MlaLaunch& a, int t, int split, int head, float m_log2, float l_tot) {
  if (a.splits == 1) {
    if (a.lse) a.lse[(size_t)t * a.H + head] = l_tot > 0.f ? (m_log2 + log2f(l_tot)) * kLn2 : -INFINITY;
  } else {
    float* stats = a.ws + (size_t)a.T * a.splits * a.H * a.kv_lora;
    const size_t i = ((size_t)t * a.splits + split) * a.H + head;
    stats[2 * i] = m_log2;
    stats[2 * i + 1] = l_tot;
  }
}

template <int ROPE>
__global__ void __launch_bounds__(kThreads)
k_mla_fp8(MlaLaunch a) {
  constexpr int DQ = kLora + ROPE;
  constexpr int KSTEPS = DQ / 32;
  __shared__ Fp8Smem sm;
  const int t = blockIdx.y, split = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int b = clampi(a.q_seq[t], 0, a.B - 1);
  const int L = a.len ? clampi(a.len[t], 0, a.topk) : a.topk;
  const int slot0 = split * a.per_split;
  const int slot1 = min(L, slot0 + a.per_split);
  const bool active = 16 * wave < a.H;
  const int head = 16 * wave + c;
  const float zscale = a.softmax_scale * kLog2e;

  bf16x8 qreg[KSTEPS];
  if (active) {
    const uint16_t* qh = reinterpret_cast<const uint16_t*>(a.q) + ((size_t)t * a.H + head) * DQ;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s)
      qreg[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qh + 32 * s + 8 * g));
  }
  float m_run = -INFINITY, l_run = 0.f;
  float4v oacc[kLora / 16];
#pragma unroll
  for (int md = 0; md < kLora / 16; ++md) oacc[md] = float4v{0.f, 0.f, 0.f, 0.f};

  const int32_t* irow = a.idx + (size_t)t * a.topk;
  const uint8_t* kvseq = reinterpret_cast<const uint8_t*>(a.kv) + (size_t)b * a.max_ctx * kRow;
  const float* scseq = a.kv_scale + (size_t)b * a.max_ctx * kBlocks;

  for (int tb = slot0; tb < slot1; tb += kTileK) {
    if (tid < kTileK) {
      const int slot = tb + tid;
      const int r = slot < slot1 ? irow[slot] : -1;
      const bool ok = r >= 0 && r < a.max_ctx;
      sm.valid[tid] = ok;
      sm.row[tid] = ok ? r : 0;
    }
    __syncthreads();
    for (int ch = tid; ch < kTileK * (kRow / 16); ch += kThreads) {
      const int r = ch / (kRow / 16), cc = ch % (kRow / 16);
      const u32x4 v = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(kvseq + (size_t)sm.row[r] * kRow) + cc);
      *reinterpret_cast<u32x4*>(&sm.raw[r][16 * cc]) = v;
    }
    for (int e = tid; e < kTileK * kBlocks; e += kThreads) {
      const int r = e / kBlocks, blk = e % kBlocks;
      sm.sc[r][blk] = scseq[(size_t)sm.row[r] * kBlocks + blk];
    }
    __syncthreads();
    // key-major bf16 rows (Q.K^T operand)
    for (int it = tid; it < kTileK * (DQ / 8); it += kThreads) {
      const int r = it / (DQ / 8), grp = it % (DQ / 8);
      const uint2 raw8 = *reinterpret_cast<const uint2*>(&sm.raw[r][8 * grp]);
      const float s = sm.sc[r][grp >> 3];
      u32x4 pk;
      pk[0] = pack2(__builtin_amdgcn_cvt_f32_fp8(raw8.x, 0) * s, __builtin_amdgcn_cvt_f32_fp8(raw8.x, 1) * s);
      pk[1] = pack2(__builtin_amdgcn_cvt_f32_fp8(raw8.x, 2) * s, __builtin_amdgcn_cvt_f32_fp8(raw8.x, 3) * s);
      pk[2] = pack2(__builtin_amdgcn_cvt_f32_fp8(raw8.y, 0) * s, __builtin_amdgcn_cvt_f32_fp8(raw8.y, 1) * s);
      pk[3] = pack2(__builtin_amdgcn_cvt_f32_fp8(raw8.y, 2) * s, __builtin_amdgcn_cvt_f32_fp8(raw8.y, 3) * s);
      *reinterpret_cast<u32x4*>(&sm.ks[ks_row_of_key(r)][8 * grp]) = pk;
    }
    // dim-major bf16 transpose of the latent part (P.V operand)
    for (int it = tid; it < kLora * (kTileK / 8); it += kThreads) {
      const int d = it % kLora, oct = it / kLora;
      float v[8];
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const int r = 8 * oct + kk;
        v[kk] = __builtin_amdgcn_cvt_f32_fp8((uint32_t)sm.raw[r][d], 0) * sm.sc[r][d >> 6];
      }
      u32x4 pk;
      pk[0] = pack2(v[0], v[1]); pk[1] = pack2(v[2], v[3]);
      pk[2] = pack2(v[4], v[5]); pk[3] = pack2(v[6], v[7]);
      *reinterpret_cast<u32x4*>(&sm.vt[d][8 * oct]) = pk;
    }
    __syncthreads();
    if (active) {
      float4v sacc[2] = {float4v{0.f, 0.f, 0.f, 0.f}, float4v{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const bf16x8 kop = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&sm.ks[16 * mb + c][32 * s + 8 * g]));
          sacc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qreg[s], sacc[mb], 0, 0, 0);
        }
      }
      // this lane: head c, keys 8g + 4mb + i
      float z[8];
      float tmax = -INFINITY;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int kappa = 8 * g + 4 * mb + i;
          const float v = sm.valid[kappa] ? sacc[mb][i] * zscale : -INFINITY;
          z[4 * mb + i] = v;
          tmax = fmaxf(tmax, v);
        }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      const float m_new = fmaxf(m_run, tmax);
      float alpha = 1.f;
      float p[8];
      if (m_new == -INFINITY) {
#pragma unroll
        for (int e = 0; e < 8; ++e) p[e] = 0.f;
      } else {
        alpha = exp2f(m_run - m_new);
#pragma unroll
        for (int e = 0; e < 8; ++e) p[e] = exp2f(z[e] - m_new);
      }
      float psum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) psum += p[e];
      l_run = l_run * alpha + psum;
      m_run = m_new;
      if (__ballot(alpha != 1.f)) {
#pragma unroll
        for (int md = 0; md < kLora / 16; ++md) oacc[md] *= alpha;
      }
      u32x4 pk;
      pk[0] = pack2(p[0], p[1]); pk[1] = pack2(p[2], p[3]);
      pk[2] = pack2(p[4], p[5]); pk[3] = pack2(p[6], p[7]);
      const bf16x8 pop = __builtin_bit_cast(bf16x8, pk);
#pragma unroll
      for (int md = 0; md < kLora / 16; ++md) {
        const bf16x8 vop = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&sm.vt[16 * md + c][8 * g]));
        oacc[md] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop, oacc[md], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  if (!active) return;
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  // oacc[md][i] = O^T[dim 16md + 4g + i][head c]
#pragma unroll
  for (int md = 0; md < kLora / 16; ++md) {
    float o[4] = {oacc[md][0], oacc[md][1], oacc[md][2], oacc[md][3]};
    write_partial_or_final(a, t, split, head, m_run, l_tot, o, 16 * md + 4 * g, 4);
  }
  if (g == 0) write_stats(a, t, split, head, m_run, l_tot);
}

// ---------------------------------------------------------------------------------------------
// fp32 path: 512 threads, 8 lanes per head, 16-key tiles
// ---------------------------------------------------------------------------------------------

constexpr int kF32Threads = 512;
constexpr int kF32Tile = 16;

template <int ROPE>
__global__ void __launch_bounds__(kF32Threads)
k_mla_f32(MlaLaunch a) {
  constexpr int DQ = kLora + ROPE;
  constexpr int QPART = DQ / 8;      // query dims per lane
  constexpr int OPART = kLora / 8;   // output dims per lane
  __shared__ float kt[kF32Tile][kRow];
  __shared__ int srow[kF32Tile];
  __shared__ int svalid[kF32Tile];
  const int t = blockIdx.y, split = blockIdx.x;
  const int tid = threadIdx.x;
  const int head = tid >> 3, part = tid & 7;
  const bool active = head < a.H;
  const int b = clampi(a.q_seq[t], 0, a.B - 1);
  const int L = a.len ? clampi(a.len[t], 0, a.topk) : a.topk;
  const int slot0 = split * a.per_split;
  const int slot1 = min(L, slot0 + a.per_split);
  const float zscale = a.softmax_scale * kLog2e;

  float qr[QPART];
  if (active) {
    const float* qh = reinterpret_cast<const float*>(a.q) + ((size_t)t * a.H + head) * DQ + part * QPART;
#pragma unroll
    for (int d = 0; d < QPART; ++d) qr[d] = qh[d];
  }
  float o[OPART];
#pragma unroll
  for (int d = 0; d < OPART; ++d) o[d] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const int32_t* irow = a.idx + (size_t)t * a.topk;
  const float* kvseq = reinterpret_cast<const float*>(a.kv) + (size_t)b * a.max_ctx * kRow;

  for (int tb = slot0; tb < slot1; tb += kF32Tile) {
    if (tid < kF32Tile) {
      const int slot = tb + tid;
      const int r = slot < slot1 ? irow[slot] : -1;
      const bool ok = r >= 0 && r < a.max_ctx;
      svalid[tid] = ok;
      srow[tid] = ok ? r : 0;
    }
    __syncthreads();
    for (int e = tid; e < kF32Tile * (kRow / 4); e += kF32Threads) {
      const int r = e / (kRow / 4), c4 = e % (kRow / 4);
      *reinterpret_cast<float4*>(&kt[r][4 * c4]) =
          reinterpret_cast<const float4*>(kvseq + (size_t)srow[r] * kRow)[c4];
    }
    __syncthreads();
    if (active) {
      float z[kF32Tile];
#pragma unroll
      for (int k = 0; k < kF32Tile; ++k) {
        // query dim d pairs with latent row dim d (0..511 latent, 512..575 rope key)
        float acc = 0.f;
#pragma unroll
        for (int d = 0; d < QPART; ++d) acc = fmaf(qr[d], kt[k][part * QPART + d], acc);
        acc += __shfl_xor(acc, 1);
        acc += __shfl_xor(acc, 2);
        acc += __shfl_xor(acc, 4);
        z[k] = svalid[k] ? acc * zscale : -INFINITY;
      }
      float tmax = -INFINITY;
#pragma unroll
      for (int k = 0; k < kF32Tile; ++k) tmax = fmaxf(tmax, z[k]);
      const float m_new = fmaxf(m_run, tmax);
      float alpha = 1.f;
      float p[kF32Tile];
      if (m_new == -INFINITY) {
#pragma unroll
        for (int k = 0; k < kF32Tile; ++k) p[k] = 0.f;
      } else {
        alpha = exp2f(m_run - m_new);
#pragma unroll
        for (int k = 0; k < kF32Tile; ++k) p[k] = exp2f(z[k] - m_new);
      }
      float psum = 0.f;
#pragma unroll
      for (int k = 0; k < kF32Tile; ++k) psum += p[k];
      l_run = l_run * alpha + psum;
      m_run = m_new;
#pragma unroll
      for (int d = 0; d < OPART; ++d) {
        float acc = o[d] * alpha;
#pragma unroll
        for (int k = 0; k < kF32Tile; ++k) acc = fmaf(p[k], kt[k][part * OPART + d], acc);
        o[d] = acc;
      }
    }
    __syncthreads();
  }
  if (!active) return;
  write_partial_or_final(a, t, split, head, m_run, l_run, o, part * OPART, OPART);
  if (part == 0) write_stats(a, t, split, head, m_run, l_run);
}

// Merge split partials: out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s;  lse = ln2 (M + log2 L).
__global__ void __launch_bounds__(kThreads) k_mla_combine(MlaLaunch a) {
  __shared__ float wts[128][65];
  const int t = blockIdx.x;
  const float* stats = a.ws + (size_t)a.T * a.splits * a.H * a.kv_lora;
  for (int h = threadIdx.x; h < a.H; h += kThreads) {
    float M = -INFINITY;
    for (int s = 0; s < a.splits; ++s) M = fmaxf(M, stats[2 * (((size_t)t * a.splits + s) * a.H + h)]);
    float Ls = 0.f;
    for (int s = 0; s < a.splits; ++s) {
      const size_t i = ((size_t)t * a.splits + s) * a.H + h;
      const float w = (M == -INFINITY) ? 0.f : exp2f(stats[2 * i] - M);
      wts[h][s] = w;
      Ls += w * stats[2 * i + 1];
    }
    const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
    for (int s = 0; s < a.splits; ++s) wts[h][s] *= inv;
    if (a.lse) a.lse[(size_t)t * a.H + h] = Ls > 0.f ? (M + log2f(Ls)) * kLn2 : -INFINITY;
  }
  __syncthreads();
  const int n4 = a.H * a.kv_lora / 4;
  for (int e = threadIdx.x; e < n4; e += kThreads) {
    const int h = (4 * e) / a.kv_lora;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s = 0; s < a.splits; ++s) {
      const float w = wts[h][s];
      const float4 v = reinterpret_cast<const float4*>(a.ws + (((size_t)t * a.splits + s) * a.H) * a.kv_lora)[e];
      acc.x = fmaf(w, v.x, acc.x); acc.y = fmaf(w, v.y, acc.y);
      acc.z = fmaf(w, v.z, acc.z); acc.w = fmaf(w, v.w, acc.w);
    }
    reinterpret_cast<float4*>(a.out + (size_t)t * a.H * a.kv_lora)[e] = acc;
  }
}

}  // namespace

hipError_t launch_sparse_mla(const MlaLaunch& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  dim3 grid(a.splits, a.T);
  if (a.kv_dtype == DSA_FP8_E4M3FN) {
    if (a.rope_dim == 64) hipLaunchKernelGGL(k_mla_fp8<64>, grid, dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL(k_mla_fp8<0>, grid, dim3(kThreads), 0, s, a);
  } else {
    if (a.rope_dim == 64) hipLaunchKernelGGL(k_mla_f32<64>, grid, dim3(kF32Threads), 0, s, a);
    else hipLaunchKernelGGL(k_mla_f32<0>, grid, dim3(kF32Threads), 0, s, a);
  }
  if (a.splits > 1) hipLaunchKernelGGL(k_mla_combine, dim3(a.T), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace dsa
