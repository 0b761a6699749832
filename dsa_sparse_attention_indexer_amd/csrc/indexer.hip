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
// Query prep (RoPE angles formed and evaluated in float64, SSMax in float64): on the fp8 path each
// workgroup prepares its query in LDS while its first key tiles are in flight; on the fp32 path a
// small kernel prepares each query once into the caller's workspace.

#include "topk_common.h"

#include <math.h>

namespace dsa {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 128;          // index head dim
constexpr int kHPad = 32;        // heads padded to the MFMA M dimension
constexpr int kThreads = 256;    // 4 waves
constexpr int kTile = 32;        // keys per MFMA N tile
constexpr int kQsStride = kD + 1;  // double row stride in LDS (odd: per-head reductions avoid conflicts)
constexpr int kDepth = 5;        // key tiles in flight per wave in the fp8 stream

struct PrepSmem {
  double qs[kHPad][kQsStride];   // q' (rotated, SSMax-scaled), float64
  double cs[32], sn[32];         // cos / sin of the 32 rotary angles
  double mh[kHPad];              // SSMax multipliers
  double wv[kHPad];              // raw head weights
  float coef[kHPad];             // w_h / (sqrt(H) sqrt(128)) * 2^-e_h   (fp8 path)
  int ex[kHPad];                 // per-head power-of-two exponent e_h   (fp8 path)
};

// Query prep in two phases so the fp8 kernel can put its key loads between them.
// Load phase: thread (h = tid / 8, part = tid % 8) owns dims [16 part, 16 part + 16) of head h and
// issues its 16 elements as two (bf16) or four (f32) 16-byte loads; threads < 32 also fetch one
// rotary frequency, one head's SSMax pair and one head weight.
struct PrepIn {
  u32x4 raw[4];   // the 16 query elements as loaded: 2 (bf16) or 4 (f32) 16-byte chunks
  float invf, ss, sb, wv;
};

template <bool BF16Q>
__device__ inline PrepIn prep_load(const IndexerLaunch& a, int t) {
  // Every load is unconditional (indices clamped into range, values masked afterwards) so that the
  // compiler can issue them together, ahead of the key stream.
  const int tid = threadIdx.x;
  const int h = tid >> 3, part = tid & 7;
  const int hc = min(h, a.H - 1);
  PrepIn in;
  const size_t base = ((size_t)t * a.H + hc) * kD + 16 * part;
  if (BF16Q) {
    const u32x4* src = reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(a.q) + base);
    in.raw[0] = src[0];
    in.raw[1] = src[1];
  } else {
    const u32x4* src = reinterpret_cast<const u32x4*>(reinterpret_cast<const float*>(a.q) + base);
#pragma unroll
    for (int i = 0; i < 4; ++i) in.raw[i] = src[i];
  }
  const int th = min(tid, a.H - 1);
  const float* pf = a.rope_dim > 0 ? a.inv_freq : a.w;            // a.w is a valid dummy source
  const float* ps = a.ssmax_s ? a.ssmax_s : a.w;
  const float* pb = a.ssmax_s ? a.ssmax_b : a.w;
  in.invf = pf[a.rope_dim > 0 ? min(tid, a.rope_dim / 2 - 1) : 0];
  in.ss = ps[th];
  in.sb = pb[th];
  in.wv = a.w[(size_t)t * a.H + th];
  return in;
}

// Compute phase: fills sm.qs with q' (heads >= H zeroed) and sm.wv with the raw head weights.
template <bool BF16Q>
__device__ void prep_compute(PrepSmem& sm, const PrepIn& in, const IndexerLaunch& a, int p) {
  const int tid = threadIdx.x;
  const int h = tid >> 3, part = tid & 7;
  const int npairs = a.rope_dim / 2;
  if (tid < npairs) {
    // p * inv_freq[j] is exact in float64 (24-bit times 31-bit); sin/cos evaluated in float64.
    const double ang = (double)p * (double)in.invf;
    double sn, cs;
    sincos(ang, &sn, &cs);
    sm.cs[tid] = cs;
    sm.sn[tid] = sn;
  }
  if (tid < kHPad) {
    sm.mh[tid] = (a.ssmax_s != nullptr && tid < a.H) ? (double)in.ss * log((double)p + 1.0) + (double)in.sb : 1.0;
    sm.wv[tid] = tid < a.H ? (double)in.wv : 0.0;
  }
  float x[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (BF16Q) {
      const uint32_t w = in.raw[i >> 2][i & 3];
      x[2 * i] = __uint_as_float(w << 16);
      x[2 * i + 1] = __uint_as_float(w & 0xFFFF0000u);
    } else {
      x[2 * i] = __uint_as_float(in.raw[i >> 1][2 * (i & 1)]);
      x[2 * i + 1] = __uint_as_float(in.raw[i >> 1][2 * (i & 1) + 1]);
    }
  }
  __syncthreads();
  const double m = h < a.H ? sm.mh[h] : 0.0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int j = 8 * part + i;          // pair (2j, 2j + 1)
    double x0 = (double)x[2 * i], x1 = (double)x[2 * i + 1];
    if (j < npairs) {
      const double c = sm.cs[j], sn = sm.sn[j];
      const double r0 = x0 * c - x1 * sn;
      const double r1 = x0 * sn + x1 * c;
      x0 = r0;
      x1 = r1;
    }
    sm.qs[h][2 * j] = x0 * m;
    sm.qs[h][2 * j + 1] = x1 * m;
  }
  __syncthreads();
}

__device__ inline void prep_query(PrepSmem& sm, const IndexerLaunch& a, int t, int p) {
  if (a.q_dtype == DSA_BF16) {
    const PrepIn in = prep_load<true>(a, t);
    prep_compute<true>(sm, in, a, p);
  } else {
    const PrepIn in = prep_load<false>(a, t);
    prep_compute<false>(sm, in, a, p);
  }
}

// ------------------------------------------------------------------------------------------
// Query prep: one workgroup per query writes the prepared query to the workspace
// ------------------------------------------------------------------------------------------

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

// From q' in sm.qs: per-head power-of-two scales, head weights and the hi/lo fp16 MFMA A operands
// of every lane, written to `o` (LDS or global).  All 256 threads participate.
__device__ void build_fp8_operands(PrepSmem& sm, QPrepFp8* o, const IndexerLaunch& a, int t) {
  const int tid = threadIdx.x;
  const double inv_norm = 1.0 / (sqrt((double)a.H) * sqrt((double)kD));
  // max|q'_h| * 2^e_h in [2^14, 2^15) keeps both fp16 terms normal
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
      const double wv = h < a.H ? sm.wv[h] * inv_norm : 0.0;
      sm.coef[h] = (float)ldexp(wv, -e);
    }
  }
  __syncthreads();
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
  __syncthreads();
}

// fp32 keys: q' as fp32 and the head weights, one workgroup per query, to the workspace.
__global__ void __launch_bounds__(kThreads) k_index_qprep(IndexerLaunch a, void* ws) {
  __shared__ PrepSmem sm;
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int p = clampi(a.q_pos[t], -1, a.max_ctx - 1);
  prep_query(sm, a, t, p < 0 ? 0 : p);
  QPrepF32* o = reinterpret_cast<QPrepF32*>(reinterpret_cast<uint8_t*>(ws) + (size_t)t * kQPrepBytes);
  const double inv_norm = 1.0 / (sqrt((double)a.H) * sqrt((double)kD));
  for (int e = tid; e < kHPad * kD; e += kThreads) o->q[e / kD][e % kD] = (float)sm.qs[e / kD][e % kD];
  if (tid < kHPad) o->coef[tid] = tid < a.H ? (float)(sm.wv[tid] * inv_norm) : 0.f;
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

// TPW: 32-key tiles per wave (a workgroup covers 4 * 32 * TPW keys).  HIST: also histogram the
// first top-k digit of this chunk's scores into the top-k workspace (the fused selection path).
template <int TPW, bool HIST, bool BF16Q>
__global__ void __launch_bounds__(kThreads)
k_index_scores_fp8(IndexerLaunch a) {
  constexpr int chunk = 4 * kTile * TPW;
  __shared__ PrepSmem sm;
  __shared__ QPrepFp8 qa;
  __shared__ uint32_t lh[HIST ? kTkBins : 1];
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

  // The first key tiles go out first; the query prep (float64 RoPE and SSMax, power-of-two scaling,
  // hi/lo fp16 split) runs in LDS while they are in flight.
  const PrepIn pin = prep_load<BF16Q>(a, t);
  __builtin_amdgcn_sched_barrier(0);
  uint32_t rel = wave * kTile;
  KeyTile tb[kDepth];
#pragma unroll
  for (int i = 0; i < kDepth; ++i) load_tile(tb[i], krs, srs, rel + i * kStride + col, g);
  __builtin_amdgcn_sched_barrier(0);
  prep_compute<BF16Q>(sm, pin, a, p);
  build_fp8_operands(sm, &qa, a, t);
  half8 ahi[8], alo[8];
  float cf[16];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    ahi[s] = __builtin_bit_cast(half8, qa.a[2 * s][lane]);
    alo[s] = __builtin_bit_cast(half8, qa.a[2 * s + 1][lane]);
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) cf[r] = qa.cf[r][lane];

  // only lanes 0..31 store (lanes 32..63 hold the same columns); the others aim past the range
  const uint32_t out_off = g == 0 ? 4u * col : 0x80000000u;
  const bool hist = HIST && n > a.topk_k;
  if (hist) {
    for (int i = threadIdx.x; i < kTkBins; i += kThreads) lh[i] = 0;
    __syncthreads();
  }

  // Fully unrolled: straight-line code gives the compiler exact wait counts, so kDepth - 1 tiles
  // stay in flight behind the one being multiplied.  Past the chunk the loads read zeros and the stores
  // are dropped, so there is no per-tile guard.
#pragma unroll
  for (int it = 0; it < TPW; ++it) {
    KeyTile& cur = tb[it % kDepth];
    const float sc = tile_scores(cur, ahi, alo, cf);
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, sc), ors, out_off + 4u * rel, 0, 0);
    if (hist && g == 0 && rel + col < nrow) atomicAdd(&lh[score_key(sc) >> kTkShift0], 1u);
    if (it + kDepth < TPW) load_tile(cur, krs, srs, rel + kDepth * kStride + col, g);
    rel += kStride;
  }
  if (hist) {   // this chunk's counts into the row's histogram (read by the next kernel)
    __syncthreads();
    uint32_t* gh = tk_hist(a.topk_ws, t);
    for (int i = threadIdx.x; i < kTkBins; i += kThreads)
      if (lh[i]) atomicAdd(&gh[i], lh[i]);
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

size_t indexer_ws_bytes(int T, dsa_dtype_t k_dtype) { return k_dtype == DSA_FP8_E4M3FN ? 0 : (size_t)T * kQPrepBytes; }

hipError_t launch_indexer(const IndexerLaunch& a, void* ws, hipStream_t s) {
  if (a.T == 0 || a.max_ctx == 0) return hipSuccess;
  if (a.k_dtype == DSA_FP8_E4M3FN) {
    // 4096-key chunks (32 tiles per wave) when that still gives >= 512 workgroups, else 1024.
    const int64_t big = (int64_t)a.T * ((a.max_ctx + 4095) / 4096);
    const bool hist = a.topk_ws != nullptr;
    const bool bf = a.q_dtype == DSA_BF16;
    auto go = [&](auto kernel, int chunk) {
      dim3 grid((a.max_ctx + chunk - 1) / chunk, a.T);
      hipLaunchKernelGGL(kernel, grid, dim3(kThreads), 0, s, a);
    };
    if (big >= 512) {
      if (hist) bf ? go(k_index_scores_fp8<32, true, true>, 4096) : go(k_index_scores_fp8<32, true, false>, 4096);
      else bf ? go(k_index_scores_fp8<32, false, true>, 4096) : go(k_index_scores_fp8<32, false, false>, 4096);
    } else {
      if (hist) bf ? go(k_index_scores_fp8<8, true, true>, 1024) : go(k_index_scores_fp8<8, true, false>, 1024);
      else bf ? go(k_index_scores_fp8<8, false, true>, 1024) : go(k_index_scores_fp8<8, false, false>, 1024);
    }
  } else {
    hipLaunchKernelGGL(k_index_qprep, dim3(a.T), dim3(kThreads), 0, s, a, ws);
    dim3 grid((a.max_ctx + kThreads - 1) / kThreads, a.T);
    hipLaunchKernelGGL(k_index_scores_f32, grid, dim3(kThreads), 0, s, a, (const void*)ws);
  }
  return hipGetLastError();
}

}  // namespace dsa
