// Lightning-indexer scores on gfx950.
//
// Definition ("mistral-large4.md", "What differs from GLM-5.2", bullets "The indexer", "SSMax",
// "RoPE and the rest"): for a query at position p, each index head's query is rotated on its
// first 64 dims in interleaved pairs (angle p * inv_freq[j]) and multiplied by the head's SSMax
// factor s*ln(p+1)+b; key i then scores  S(i) = sum_h w_h/sqrt(H) * relu(q'_h . k_i / sqrt(128)).
//
// Two kernels:
//  * fp8 keys (the serving format, 128 B + one fp32 scale per token, as the vLLM page's
//    "DSA indexer on AITER" describes): a bandwidth-bound stream over the key cache.  Each wave
//    owns the 32 (zero-padded) heads of one query as the A operand of v_mfma_f32_32x32x16_f16 and
//    streams 32-key tiles as the B operand straight from HBM (16-byte loads per lane, the fp8
//    bytes converted exactly to fp16 by v_cvt_scalef32_pk_f16_fp8 with unit scale).  q' is formed
//    in float64, scaled by a power of two per head and split into two fp16 terms (hi + lo) whose
//    products accumulate into one fp32 accumulator, so the dot product keeps ~22 bits of q'.
//    ReLU, the head weights and the per-token scale are applied in registers; the two halves of
//    the wave are summed with v_permlane32_swap, and lanes 0..31 store 32 consecutive scores.
//  * fp32 keys (the reference-precision path): one thread per key, fp32 FMAs against q' in LDS.
//
// Query prep (RoPE angles formed and evaluated in float64, SSMax in float64) runs once per query in
// its own small kernel, which writes the prepared operands to the caller's workspace.

#include "dsa_internal.h"

#include <math.h>

namespace dsa {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float16v __attribute__((ext_vector_type(16)));

constexpr int kD = 128;          // index head dim
constexpr int kHPad = 32;        // heads padded to the MFMA M dimension
constexpr int kThreads = 256;    // 4 waves
constexpr int kTile = 32;        // keys per MFMA N tile
constexpr int kQsStride = kD + 1;  // double row stride in LDS (odd: per-head reductions avoid conflicts)

struct PrepSmem {
  double qs[kHPad][kQsStride];   // q' (rotated, SSMax-scaled), float64
  double cs[32], sn[32];         // cos / sin of the 32 rotary angles
  double mh[kHPad];              // SSMax multipliers
  float coef[kHPad];             // w_h / (sqrt(H) sqrt(128)) * 2^-e_h   (fp8 path)
  int ex[kHPad];                 // per-head power-of-two exponent e_h   (fp8 path)
};

__device__ __forceinline__ double load_q(const void* q, dsa_dtype_t dt, size_t i) {
  if (dt == DSA_BF16) return (double)bf16_bits_to_float(reinterpret_cast<const uint16_t*>(q)[i]);
  return (double)reinterpret_cast<const float*>(q)[i];
}

// Fills sm.qs with q' for query t (heads >= H zeroed).  All 256 threads participate.
__device__ void prep_query(PrepSmem& sm, const IndexerLaunch& a, int t, int p) {
  const int tid = threadIdx.x;
  const int npairs = a.rope_dim / 2;
  if (tid < npairs) {
    // p * inv_freq[j] is exact in float64 (24-bit times 31-bit); sin/cos evaluated in float64.
    double ang = (double)p * (double)a.inv_freq[tid];
    double s, c;
    sincos(ang, &s, &c);
    sm.cs[tid] = c;
    sm.sn[tid] = s;
  }
  if (tid < kHPad) {
    double m = 1.0;
    if (a.ssmax_s != nullptr && tid < a.H)
      m = (double)a.ssmax_s[tid] * log((double)p + 1.0) + (double)a.ssmax_b[tid];
    sm.mh[tid] = m;
  }
  __syncthreads();
  // 32 heads x 64 pairs = 2048 pairs, 8 per thread.
  for (int e = tid; e < kHPad * (kD / 2); e += kThreads) {
    const int h = e >> 6, j = e & 63;
    double x0 = 0.0, x1 = 0.0;
    if (h < a.H) {
      const size_t base = ((size_t)t * a.H + h) * kD + 2 * j;
      x0 = load_q(a.q, a.q_dtype, base);
      x1 = load_q(a.q, a.q_dtype, base + 1);
      if (j < npairs) {
        const double c = sm.cs[j], s = sm.sn[j];
        const double r0 = x0 * c - x1 * s;
        const double r1 = x0 * s + x1 * c;
        x0 = r0;
        x1 = r1;
      }
      x0 *= sm.mh[h];
      x1 *= sm.mh[h];
    }
    sm.qs[h][2 * j] = x0;
    sm.qs[h][2 * j + 1] = x1;
  }
  __syncthreads();
}

// ------------------------------------------------------------------------------------------
// Query prep: one workgroup per query writes the prepared query to the workspace
// ------------------------------------------------------------------------------------------

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Per-query workspace record.  fp8 keys: the MFMA A operands of every lane of a wave
// (j = 2*s + term, term 0 = hi, 1 = lo) and each lane's 16 accumulator-row weights.
// fp32 keys: q' as fp32 [32][128] and the 32 head weights.
struct QPrepFp8 {
  u32x4 a[16][64];
  float cf[16][64];
};
struct QPrepF32 {
  float q[kHPad][kD];
  float coef[kHPad];
};
constexpr size_t kQPrepBytes = sizeof(QPrepFp8) > sizeof(QPrepF32) ? sizeof(QPrepFp8) : sizeof(QPrepF32);

__device__ __forceinline__ uint32_t pack_half2(_Float16 lo, _Float16 hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
}

__global__ void __launch_bounds__(kThreads) k_index_qprep(IndexerLaunch a, void* ws) {
  __shared__ PrepSmem sm;
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int p = clampi(a.q_pos[t], -1, a.max_ctx - 1);
  prep_query(sm, a, t, p < 0 ? 0 : p);
  uint8_t* rec = reinterpret_cast<uint8_t*>(ws) + (size_t)t * kQPrepBytes;
  const double inv_norm = 1.0 / (sqrt((double)a.H) * sqrt((double)kD));
  if (a.k_dtype != DSA_FP8_E4M3FN) {
    QPrepF32* o = reinterpret_cast<QPrepF32*>(rec);
    for (int e = tid; e < kHPad * kD; e += kThreads) o->q[e / kD][e % kD] = (float)sm.qs[e / kD][e % kD];
    if (tid < kHPad) o->coef[tid] = tid < a.H ? (float)((double)a.w[(size_t)t * a.H + tid] * inv_norm) : 0.f;
    return;
  }
  // Per-head power-of-two scale: max|q'_h| * 2^e_h in [2^14, 2^15) keeps both fp16 terms normal.
  {
    const int h = tid >> 3, part = tid & 7;   // 32 heads x 8 lanes
    double mx = 0.0;
    for (int d = part * 16; d < part * 16 + 16; ++d) mx = fmax(mx, fabs(sm.qs[h][d]));
    mx = fmax(mx, __shfl_xor(mx, 1));
    mx = fmax(mx, __shfl_xor(mx, 2));
    mx = fmax(mx, __shfl_xor(mx, 4));
    if (part == 0) {
      int e = 0;
      if (mx > 0.0) {
        int x;
        frexp(mx, &x);   // mx = f * 2^x, f in [0.5, 1)
        e = 15 - x;
      }
      sm.ex[h] = e;
      const double wv = h < a.H ? (double)a.w[(size_t)t * a.H + h] * inv_norm : 0.0;
      sm.coef[h] = (float)ldexp(wv, -e);
    }
  }
  __syncthreads();
  QPrepFp8* o = reinterpret_cast<QPrepFp8*>(rec);
  // A operand of lane l (row m = l & 31, half g = l >> 5) for K-step s: q'[m][32(s>>1) + 16g + 8(s&1) + i]
  {
    const int l = tid & 63, sg = tid >> 6;
    const int m = l & 31, g = l >> 5;
    const int e = sm.ex[m];
#pragma unroll
    for (int ss = 0; ss < 2; ++ss) {
      const int s = 2 * sg + ss;
      const int base = 32 * (s >> 1) + 16 * g + 8 * (s & 1);
      _Float16 hi[8], lo[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const double v = ldexp(sm.qs[m][base + i], e);
        hi[i] = (_Float16)(float)v;                        // |v| < 2^15: normal, exact residual below
        lo[i] = (_Float16)(float)(v - (double)(float)hi[i]);
      }
      u32x4 h4, l4;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        h4[i] = pack_half2(hi[2 * i], hi[2 * i + 1]);
        l4[i] = pack_half2(lo[2 * i], lo[2 * i + 1]);
      }
      o->a[2 * s][l] = h4;
      o->a[2 * s + 1][l] = l4;
    }
  }
  if (tid < 64) {
    const int g = tid >> 5;
    // accumulator row r of a lane in half g is head 8(r>>2) + 4g + (r&3)
#pragma unroll
    for (int r = 0; r < 16; ++r) o->cf[r][tid] = sm.coef[8 * (r >> 2) + 4 * g + (r & 3)];
  }
}

// ------------------------------------------------------------------------------------------
// fp8 keys: MFMA stream
// ------------------------------------------------------------------------------------------

__device__ __forceinline__ half8 fp8x8_to_half8(uint32_t d0, uint32_t d1) {
  half2v a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d0, 1.0f, false);
  half2v b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d0, 1.0f, true);
  half2v c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d1, 1.0f, false);
  half2v d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d1, 1.0f, true);
  half8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

struct KeyTile {
  u32x4 x[4];   // 64 bytes of this lane's key row: bytes [32c + 16g, +16) for c = 0..3
  float sc;     // the row's fp8 scale
};

// Buffer resource (gfx9 raw buffer, no swizzle) over `bytes` bytes from `base`.  Accesses at or past
// `bytes` are dropped by the hardware (loads return 0, stores do nothing), which keeps tail
// handling free of branches -- and the compiler's wait counts static.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ void load_tile(KeyTile& kt, __amdgpu_buffer_rsrc_t krs, __amdgpu_buffer_rsrc_t srs,
                                          uint32_t rel_row, int g) {
  const uint32_t off = rel_row * kD + 16u * g;
#pragma unroll
  for (int c = 0; c < 4; ++c)
    kt.x[c] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, off + 32u * c, 0, 0));
  kt.sc = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(srs, rel_row * 4u, 0, 0));
}

// One 32-key tile: 16 MFMAs (8 K-steps x hi/lo), ReLU + head weights, halves summed across the wave.
__device__ __forceinline__ float tile_scores(const KeyTile& kt, const half8* ahi, const half8* alo, const float* cf) {
  float16v acc = {};
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const half8 b0 = fp8x8_to_half8(kt.x[c][0], kt.x[c][1]);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ahi[2 * c], b0, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(alo[2 * c], b0, acc, 0, 0, 0);
    const half8 b1 = fp8x8_to_half8(kt.x[c][2], kt.x[c][3]);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ahi[2 * c + 1], b1, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(alo[2 * c + 1], b1, acc, 0, 0, 0);
  }
  float part = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) part = fmaf(cf[r], fmaxf(acc[r], 0.f), part);
  // lanes l and l^32 hold the two halves of key column l&31's head sum
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part), false, false);
  return (__uint_as_float(sw[0]) + __uint_as_float(sw[1])) * kt.sc;
}

template <int TPW>   // 32-key tiles per wave; a workgroup covers 4 * 32 * TPW keys
__global__ void __launch_bounds__(kThreads)
k_index_scores_fp8(IndexerLaunch a, const void* ws) {
  constexpr int chunk = 4 * kTile * TPW;
  const int t = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform (scalar) loop control
  const int g = lane >> 5, col = lane & 31;
  const int b = clampi(a.q_seq[t], 0, a.B - 1);
  const int p = clampi(a.q_pos[t], -1, a.max_ctx - 1);
  const int n = p + 1;
  const int c0 = blockIdx.x * chunk;
  if (c0 >= n) return;
  const int c1 = min(n, c0 + chunk);
  const uint32_t nrow = (uint32_t)(c1 - c0);
  const uint8_t* kseq = reinterpret_cast<const uint8_t*>(a.k_cache) + ((size_t)b * a.max_ctx + c0) * kD;
  const float* sseq = a.k_scale + (size_t)b * a.max_ctx + c0;
  float* srow = a.scores + (size_t)t * a.ld + c0;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kseq, nrow * kD);
  const __amdgpu_buffer_rsrc_t srs = make_rsrc(sseq, nrow * 4u);
  const __amdgpu_buffer_rsrc_t ors = make_rsrc(srow, nrow * 4u);
  constexpr uint32_t kStride = 4 * kTile;   // the 4 waves interleave 32-key tiles

  // Prepared query first (L2-resident), then three key tiles in flight per wave.  The loop is
  // unrolled three ways so the tile buffers rotate by name: a buffer is refilled right after it is
  // consumed and the two younger loads stay outstanding across the MFMAs.
  const QPrepFp8* qp = reinterpret_cast<const QPrepFp8*>(reinterpret_cast<const uint8_t*>(ws) + (size_t)t * kQPrepBytes);
  half8 ahi[8], alo[8];
  float cf[16];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    ahi[s] = __builtin_bit_cast(half8, qp->a[2 * s][lane]);
    alo[s] = __builtin_bit_cast(half8, qp->a[2 * s + 1][lane]);
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) cf[r] = qp->cf[r][lane];

  // rel: this wave's current tile, relative to the chunk start (rows past the chunk read as zero)
  uint32_t rel = wave * kTile;
  KeyTile tb[3];
#pragma unroll
  for (int i = 0; i < 3; ++i) load_tile(tb[i], krs, srs, rel + i * kStride + col, g);
  // only lanes 0..31 store (lanes 32..63 hold the same columns); the others aim past the range
  const uint32_t out_off = g == 0 ? 4u * col : 0x80000000u;

  // Fully unrolled: straight-line code gives the compiler exact wait counts, so two tiles stay in
  // flight behind the one being multiplied.  Past the chunk the loads read zeros and the stores
  // are dropped, so there is no per-tile guard.
#pragma unroll
  for (int it = 0; it < TPW; ++it) {
    KeyTile& cur = tb[it % 3];
    const float sc = tile_scores(cur, ahi, alo, cf);
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, sc), ors, out_off + 4u * rel, 0, 0);
    if (it + 3 < TPW) load_tile(cur, krs, srs, rel + 3 * kStride + col, g);
    rel += kStride;
  }
}

// ------------------------------------------------------------------------------------------
// fp32 keys: vector FMAs
// ------------------------------------------------------------------------------------------

__global__ void __launch_bounds__(kThreads)
k_index_scores_f32(IndexerLaunch a, const void* ws) {
  __shared__ float qf[kHPad][kD];
  __shared__ float coef[kHPad];
  const int t = blockIdx.y;
  const int tid = threadIdx.x;
  const int b = clampi(a.q_seq[t], 0, a.B - 1);
  const int p = clampi(a.q_pos[t], -1, a.max_ctx - 1);
  const int n = p + 1;
  const int c0 = blockIdx.x * kThreads;
  if (c0 >= n) return;
  const QPrepF32* qp = reinterpret_cast<const QPrepF32*>(reinterpret_cast<const uint8_t*>(ws) + (size_t)t * kQPrepBytes);
  for (int e = tid; e < kHPad * kD; e += kThreads) qf[e / kD][e % kD] = qp->q[e / kD][e % kD];
  if (tid < kHPad) coef[tid] = qp->coef[tid];
  __syncthreads();
  const int row = c0 + tid;
  if (row >= n) return;
  const float4* kr = reinterpret_cast<const float4*>(
      reinterpret_cast<const float*>(a.k_cache) + ((size_t)b * a.max_ctx + row) * kD);
  float acc[kHPad];
#pragma unroll
  for (int h = 0; h < kHPad; ++h) acc[h] = 0.f;
  for (int d4 = 0; d4 < kD / 4; ++d4) {
    const float4 k = kr[d4];
#pragma unroll
    for (int h = 0; h < kHPad; ++h) {
      acc[h] = fmaf(qf[h][4 * d4 + 0], k.x, acc[h]);
      acc[h] = fmaf(qf[h][4 * d4 + 1], k.y, acc[h]);
      acc[h] = fmaf(qf[h][4 * d4 + 2], k.z, acc[h]);
      acc[h] = fmaf(qf[h][4 * d4 + 3], k.w, acc[h]);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int h = 0; h < kHPad; ++h) s = fmaf(coef[h], fmaxf(acc[h], 0.f), s);
  a.scores[(size_t)t * a.ld + row] = s;
}

}  // namespace

size_t indexer_ws_bytes(int T) { return (size_t)T * kQPrepBytes; }

hipError_t launch_indexer(const IndexerLaunch& a, void* ws, hipStream_t s) {
  if (a.T == 0 || a.max_ctx == 0) return hipSuccess;
  hipLaunchKernelGGL(k_index_qprep, dim3(a.T), dim3(kThreads), 0, s, a, ws);
  if (a.k_dtype == DSA_FP8_E4M3FN) {
    // 4096-key chunks (32 tiles per wave) when that still gives >= 512 workgroups, else 1024.
    const int64_t big = (int64_t)a.T * ((a.max_ctx + 4095) / 4096);
    if (big >= 512) {
      dim3 grid((a.max_ctx + 4095) / 4096, a.T);
      hipLaunchKernelGGL(k_index_scores_fp8<32>, grid, dim3(kThreads), 0, s, a, (const void*)ws);
    } else {
      dim3 grid((a.max_ctx + 1023) / 1024, a.T);
      hipLaunchKernelGGL(k_index_scores_fp8<8>, grid, dim3(kThreads), 0, s, a, (const void*)ws);
    }
  } else {
    dim3 grid((a.max_ctx + kThreads - 1) / kThreads, a.T);
    hipLaunchKernelGGL(k_index_scores_f32, grid, dim3(kThreads), 0, s, a, (const void*)ws);
  }
  return hipGetLastError();
}

}  // namespace dsa
