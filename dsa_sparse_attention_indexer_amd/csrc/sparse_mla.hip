// Sparse absorbed-MLA attention on gfx950: exact softmax attention of every head over the keys
// the indexer selected ("Day 0 support for Mistral Large 4 on vLLM": MLA with KV LoRA rank 512
// and RoPE dim 64, one latent KV head shared by all 64 heads, V = the latent; NoPE layers are
// the same with zero RoPE dims on the same cache layout).
//
// fp8 cache, bf16 query (matrix-core path), one workgroup = 4 waves = up to 64 heads:
//   * 32-key tiles are gathered by row index straight from HBM into registers (16 bytes per lane,
//     issued one tile ahead of the compute), dequantised once per workgroup to bf16 (code * scale,
//     v_cvt_pk_f32_fp8 / v_cvt_pk_bf16_f32, round to nearest even) and stored key-major in LDS.
//   * wave w owns heads 16w..16w+15.  Its bf16 query stays in registers as the B operand of
//     v_mfma_f32_16x16x32_bf16 (S^T = K Q^T, keys as M).  The key rows are placed in LDS in an
//     order that makes the S^T accumulator of each lane hold exactly the 8 consecutive keys that
//     the P.V step needs in its B operand, so probabilities go from accumulators to MFMA operands
//     without touching LDS.
//   * P.V (O^T = V^T P^T) reads its V^T operand from the same key-major tile with
//     ds_read_b64_tr_b16: a 16-lane group that points lane j at row 4*(j/4)+.., dims 4*(j%4)..+3
//     gets back, per lane, four consecutive keys of one dim -- the MFMA operand layout.
//   * online softmax in the log2 domain with fp32 statistics; fp32 accumulation.
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
typedef short short8v __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
constexpr int kTileK = 32;
constexpr int kRow = 576;                 // latent row: 512 + 64
constexpr int kLora = 512;
constexpr int kBlocks = kRow / 64;        // scales per row
constexpr int kKsStride = kRow + 8;       // bf16 per key-major row (1168 B: rows shift by 4 banks)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

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

typedef short short4v __attribute__((ext_vector_type(4)));
typedef float float2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t cvt2_bf16(float2v v) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// 16 fp8 codes times one scale -> 16 bf16 (8 dwords), nearest even.
__device__ __forceinline__ void dequant16(const u32x4 raw, float s, u32x4& lo, u32x4& hi) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float2v a = __builtin_amdgcn_cvt_pk_f32_fp8(raw[w], false) * s;
    const float2v b = __builtin_amdgcn_cvt_pk_f32_fp8(raw[w], true) * s;
    const uint32_t pa = cvt2_bf16(a), pb = cvt2_bf16(b);
    if (w < 2) { lo[2 * w] = pa; lo[2 * w + 1] = pb; } else { hi[2 * w - 4] = pa; hi[2 * w - 3] = pb; }
  }
}

template <int ROPE>
__global__ void __launch_bounds__(kThreads)
k_mla_fp8(MlaLaunch a) {
  constexpr int DQ = kLora + ROPE;
  constexpr int KSTEPS = DQ / 32;
  constexpr int CHUNKS = DQ / 16;                     // 16-byte chunks of a row that are used
  constexpr int NCH = kTileK * CHUNKS;
  constexpr int PER = (NCH + kThreads - 1) / kThreads;
  __shared__ uint16_t ks[kTileK][kKsStride];
  __shared__ int srow[2][kTileK];
  __shared__ int svalid[2][kTileK];
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
  const int32_t* irow = a.idx + (size_t)t * a.topk;
  const uint8_t* kvseq = reinterpret_cast<const uint8_t*>(a.kv) + (size_t)b * a.max_ctx * kRow;
  const float* scseq = a.kv_scale + (size_t)b * a.max_ctx * kBlocks;

  auto fetch_idx = [&](int tile_base) -> int {   // row of slot tile_base + tid (tid < 32), -1 if none
    const int slot = tile_base + tid;
    const int r = slot < slot1 ? irow[slot] : -1;
    return (r >= 0 && r < a.max_ctx) ? r : -1;
  };
  u32x4 raw[PER];
  float rsc[PER];
  auto issue_loads = [&](int buf) {
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      const int ch = tid + kThreads * m;
      if (ch < NCH) {
        const int r = ch / CHUNKS, cc = ch % CHUNKS;
        const int row = srow[buf][r];
        raw[m] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kvseq + (size_t)row * kRow) + cc);
        rsc[m] = scseq[(size_t)row * kBlocks + (cc >> 2)];
      }
    }
  };

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

  // prologue: rows of tile 0 -> LDS, its data in flight, rows of tile 1 in a register
  if (slot0 < slot1) {
    if (tid < kTileK) {
      const int r = fetch_idx(slot0);
      srow[0][tid] = r < 0 ? 0 : r;
      svalid[0][tid] = r >= 0;
    }
    __syncthreads();
    issue_loads(0);
  }
  int next_row = -1;
  if (tid < kTileK && slot0 + kTileK < slot1) next_row = fetch_idx(slot0 + kTileK);

  int cur = 0;
  for (int tb = slot0; tb < slot1; tb += kTileK, cur ^= 1) {
    __syncthreads();                       // the previous tile's readers of ks are done
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      const int ch = tid + kThreads * m;
      if (ch < NCH) {
        const int r = ch / CHUNKS, cc = ch % CHUNKS;
        u32x4 lo, hi;
        dequant16(raw[m], rsc[m], lo, hi);
        uint16_t* dst = &ks[ks_row_of_key(r)][16 * cc];
        *reinterpret_cast<u32x4*>(dst) = lo;
        *reinterpret_cast<u32x4*>(dst + 8) = hi;
      }
    }
    const bool more = tb + kTileK < slot1;
    if (tid < kTileK && more) {
      srow[cur ^ 1][tid] = next_row < 0 ? 0 : next_row;
      svalid[cur ^ 1][tid] = next_row >= 0;
    }
    __syncthreads();                       // ks and the next tile's rows are ready
    if (more) {
      issue_loads(cur ^ 1);
      if (tid < kTileK) next_row = tb + 2 * kTileK < slot1 ? fetch_idx(tb + 2 * kTileK) : -1;
    }
    if (active) {
      float4v sacc[2] = {float4v{0.f, 0.f, 0.f, 0.f}, float4v{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const bf16x8 kop = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&ks[16 * mb + c][32 * s + 8 * g]));
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
          const float v = svalid[cur][kappa] ? sacc[mb][i] * zscale : -INFINITY;
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
#pragma unroll
      for (int e = 0; e < 4; ++e) pk[e] = cvt2_bf16(float2v{p[2 * e], p[2 * e + 1]});
      const bf16x8 pop = __builtin_bit_cast(bf16x8, pk);
      // V^T operand rows: LDS rows 16h + 4g + j/4 hold keys 8g + 4h + j/4
      const int trow = 4 * g + (c >> 2), tcol = 4 * (c & 3);
#pragma unroll
      for (int md = 0; md < kLora / 16; ++md) {
        typedef __attribute__((address_space(3))) short4v* lds_s4p;
        const short4v v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4p)(&ks[trow][16 * md + tcol]));
        const short4v v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4p)(&ks[16 + trow][16 * md + tcol]));
        const short8v vv = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
        oacc[md] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vv), pop, oacc[md], 0, 0, 0);
      }
    }
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
// One workgroup per (query, 4 heads).
constexpr int kCombineHeads = 4;

__global__ void __launch_bounds__(kThreads) k_mla_combine(MlaLaunch a) {
  __shared__ float sm_m[kCombineHeads][64], sm_l[kCombineHeads][64];
  __shared__ float wts[kCombineHeads][64];
  const int t = blockIdx.y, h0 = blockIdx.x * kCombineHeads;
  const int nh = min(kCombineHeads, a.H - h0);
  const float* stats = a.ws + (size_t)a.T * a.splits * a.H * a.kv_lora;
  // all (head, split) statistics in one parallel load
  for (int e = threadIdx.x; e < nh * a.splits; e += kThreads) {
    const int hl = e / a.splits, s = e % a.splits;
    const size_t i = ((size_t)t * a.splits + s) * a.H + h0 + hl;
    sm_m[hl][s] = stats[2 * i];
    sm_l[hl][s] = stats[2 * i + 1];
  }
  __syncthreads();
  if (threadIdx.x < nh) {
    const int hl = threadIdx.x;
    float M = -INFINITY;
    for (int s = 0; s < a.splits; ++s) M = fmaxf(M, sm_m[hl][s]);
    float Ls = 0.f;
    for (int s = 0; s < a.splits; ++s) {
      const float w = (M == -INFINITY) ? 0.f : exp2f(sm_m[hl][s] - M);
      wts[hl][s] = w;
      Ls += w * sm_l[hl][s];
    }
    const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
    for (int s = 0; s < a.splits; ++s) wts[hl][s] *= inv;
    if (a.lse) a.lse[(size_t)t * a.H + h0 + hl] = Ls > 0.f ? (M + log2f(Ls)) * kLn2 : -INFINITY;
  }
  __syncthreads();
  const int n4 = nh * a.kv_lora / 4;
  for (int e = threadIdx.x; e < n4; e += kThreads) {
    const int hl = (4 * e) / a.kv_lora;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s = 0; s < a.splits; ++s) {
      const float w = wts[hl][s];
      const float4 v = reinterpret_cast<const float4*>(a.ws + (((size_t)t * a.splits + s) * a.H + h0) * a.kv_lora)[e];
      acc.x = fmaf(w, v.x, acc.x); acc.y = fmaf(w, v.y, acc.y);
      acc.z = fmaf(w, v.z, acc.z); acc.w = fmaf(w, v.w, acc.w);
    }
    reinterpret_cast<float4*>(a.out + ((size_t)t * a.H + h0) * a.kv_lora)[e] = acc;
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
  if (a.splits > 1)
    hipLaunchKernelGGL(k_mla_combine, dim3((a.H + kCombineHeads - 1) / kCombineHeads, a.T), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace dsa
