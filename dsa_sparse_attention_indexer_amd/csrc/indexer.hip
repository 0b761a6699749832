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
// Query prep (RoPE angles formed and evaluated in float64, SSMax in float64) happens inside each
// workgroup; the first key tile is already in flight while it runs.

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

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct KeyTile {
  u32x4 x[4];   // 64 bytes of this lane's key row: bytes [32c + 16g, +16) for c = 0..3
  float sc;     // the row's fp8 scale
};

__device__ __forceinline__ void load_tile(KeyTile& kt, const uint8_t* kseq, const float* sseq,
                                          int row, int g) {
  const u32x4* p = reinterpret_cast<const u32x4*>(kseq + (size_t)row * kD + 16 * g);
#pragma unroll
  for (int c = 0; c < 4; ++c) kt.x[c] = __builtin_nontemporal_load(p + 2 * c);
  kt.sc = sseq[row];
}

__global__ void __launch_bounds__(kThreads)
k_index_scores_fp8(IndexerLaunch a, int chunk) {
  __shared__ PrepSmem sm;
  const int t = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, col = lane & 31;

  const int b = clampi(a.q_seq[t], 0, a.B - 1);
  const int p = clampi(a.q_pos[t], -1, a.max_ctx - 1);
  const int n = p + 1;
  const int c0 = blockIdx.x * chunk;
  if (c0 >= n) return;
  const int c1 = min(n, c0 + chunk);

  const uint8_t* kseq = reinterpret_cast<const uint8_t*>(a.k_cache) + (size_t)b * a.max_ctx * kD;
  const float* sseq = a.k_scale + (size_t)b * a.max_ctx;
  float* srow = a.scores + (size_t)t * a.ld;

  // First tile of this wave goes out before the query prep.
  int kb = c0 + wave * kTile;
  KeyTile cur;
  load_tile(cur, kseq, sseq, min(kb + col, n - 1), g);

  prep_query(sm, a, t, p);

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
      double wv = 0.0;
      if (h < a.H) wv = (double)a.w[(size_t)t * a.H + h] / (sqrt((double)a.H) * sqrt((double)kD));
      sm.coef[h] = (float)ldexp(wv, -e);
    }
  }
  __syncthreads();

  // A operands: lane (row m = col, half g); K-step s covers dims [32(s>>1) + 16g + 8(s&1), +8).
  half8 ahi[8], alo[8];
  {
    const int e = sm.ex[col];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int base = 32 * (s >> 1) + 16 * g + 8 * (s & 1);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const double v = ldexp(sm.qs[col][base + i], e);
        const _Float16 hi = (_Float16)v;
        ahi[s][i] = hi;
        alo[s][i] = (_Float16)(v - (double)hi);
      }
    }
  }
  // Accumulator row r of this lane is head 8(r>>2) + 4g + (r&3).
  float cf[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) cf[r] = sm.coef[8 * (r >> 2) + 4 * g + (r & 3)];

  for (; kb < c1; kb += 4 * kTile) {
    const int nkb = kb + 4 * kTile;
    KeyTile nxt;
    if (nkb < c1) load_tile(nxt, kseq, sseq, min(nkb + col, n - 1), g);

    float16v acc = {};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const half8 b0 = fp8x8_to_half8(cur.x[c][0], cur.x[c][1]);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ahi[2 * c], b0, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(alo[2 * c], b0, acc, 0, 0, 0);
      const half8 b1 = fp8x8_to_half8(cur.x[c][2], cur.x[c][3]);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ahi[2 * c + 1], b1, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(alo[2 * c + 1], b1, acc, 0, 0, 0);
    }
    float part = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) part = fmaf(cf[r], fmaxf(acc[r], 0.f), part);
    // lanes l and l^32 hold the two halves of key column l&31's head sum
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part), false, false);
    const float tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    const int row = kb + col;
    if (g == 0 && row < c1) srow[row] = tot * cur.sc;
    if (nkb < c1) cur = nxt;
  }
}

// ------------------------------------------------------------------------------------------
// fp32 keys: vector FMAs
// ------------------------------------------------------------------------------------------

__global__ void __launch_bounds__(kThreads)
k_index_scores_f32(IndexerLaunch a) {
  __shared__ PrepSmem sm;
  __shared__ float qf[kHPad][kD];
  const int t = blockIdx.y;
  const int tid = threadIdx.x;
  const int b = clampi(a.q_seq[t], 0, a.B - 1);
  const int p = clampi(a.q_pos[t], -1, a.max_ctx - 1);
  const int n = p + 1;
  const int c0 = blockIdx.x * kThreads;
  if (c0 >= n) return;
  prep_query(sm, a, t, p);
  for (int e = tid; e < kHPad * kD; e += kThreads) qf[e / kD][e % kD] = (float)sm.qs[e / kD][e % kD];
  if (tid < kHPad) {
    double wv = 0.0;
    if (tid < a.H) wv = (double)a.w[(size_t)t * a.H + tid] / (sqrt((double)a.H) * sqrt((double)kD));
    sm.coef[tid] = (float)wv;
  }
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
  for (int h = 0; h < kHPad; ++h) s = fmaf(sm.coef[h], fmaxf(acc[h], 0.f), s);
  a.scores[(size_t)t * a.ld + row] = s;
}

}  // namespace

hipError_t launch_indexer(const IndexerLaunch& a, hipStream_t s) {
  if (a.T == 0 || a.max_ctx == 0) return hipSuccess;
  if (a.k_dtype == DSA_FP8_E4M3FN) {
    // ~2K workgroups over the largest context; chunks are multiples of the 4-wave tile stride.
    int chunk = 1024;
    while (chunk > 128 && (int64_t)a.T * ((a.max_ctx + chunk - 1) / chunk) < 2048) chunk /= 2;
    dim3 grid((a.max_ctx + chunk - 1) / chunk, a.T);
    hipLaunchKernelGGL(k_index_scores_fp8, grid, dim3(kThreads), 0, s, a, chunk);
  } else {
    dim3 grid((a.max_ctx + kThreads - 1) / kThreads, a.T);
    hipLaunchKernelGGL(k_index_scores_f32, grid, dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace dsa
