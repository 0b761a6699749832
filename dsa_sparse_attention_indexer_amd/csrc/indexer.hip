// Lightning-indexer scores on gfx950.
//
// Definition ("mistral-large4.md", "What differs from GLM-5.2", bullets "The indexer", "SSMax",
// "RoPE and the rest"): for a query at position p, each index head's query is rotated on its
// first 64 dims in interleaved pairs (angle p * inv_freq[j]) and multiplied by the head's SSMax
// factor s*ln(p+1)+b; key i then scores  S(i) = sum_h w_h/sqrt(H) * relu(q'_h . k_i / sqrt(128)).
//
// Two key formats:
//  * fp8 keys (the serving format, 128 B + one fp32 scale per token, as the vLLM page's
//    "DSA indexer on AITER" describes): a bandwidth-bound stream over the key cache.  Each wave
//    owns the 32 (zero-padded) heads of one query as the A operand of v_mfma_f32_32x32x16_f16 and
//    streams 32-key tiles as the B operand straight from HBM (16-byte loads per lane, the fp8
//    bytes converted exactly to fp16 by v_cvt_scalef32_pk_f16_fp8 with unit scale).  q' is formed
//    in float32, scaled by a power of two per head and split into two fp16 terms (hi + lo) whose
//    products accumulate into one fp32 accumulator, so the dot product keeps ~22 bits of q'.
//    ReLU, the head weights and the per-token scale are applied in registers; the two halves of
//    the wave are summed with v_permlane32_swap, and lanes 0..31 store 32 consecutive scores.
//    With many queries (several per sequence), the queries are prepared once into a workspace and
//    consecutive queries of a sequence share one key stream through LDS: four per workgroup over
//    1024-key chunks (verify blocks, large batches), or eight -- two per wave -- over 8192-key
//    ranges where the sequences hold 16 or more queries each (chunked prefill).
//  * fp32 keys (the reference-precision path): one thread per key, fp32 FMAs against q' in LDS.
//
// Query prep (RoPE angles formed and reduced to [-pi, pi] in float64, then sine, cosine, SSMax and
// the rotation in float32, about 1e-7 relative): on the fp8 path each
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
constexpr int kQsStride = kD + 1;  // row stride of q' in LDS (odd: per-head reductions avoid conflicts)
constexpr int kDepth = 5;        // key tiles in flight per wave in the fp8 stream

struct PrepSmem {
  float qs[kHPad][kQsStride];    // q' (rotated, SSMax-scaled)
  float cs[32], sn[32];          // cos / sin of the 32 rotary angles
  float mh[kHPad];               // SSMax multipliers
  float wv[kHPad];               // raw head weights
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
    float sn, cs;
    rope_sincos(p, in.invf, &sn, &cs);
    sm.cs[tid] = cs;
    sm.sn[tid] = sn;
  }
  if (tid < kHPad) {
    sm.mh[tid] = (a.ssmax_s != nullptr && tid < a.H) ? fmaf(in.ss, logf((float)p + 1.f), in.sb) : 1.f;
    sm.wv[tid] = tid < a.H ? in.wv : 0.f;
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
  const float m = h < a.H ? sm.mh[h] : 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int j = 8 * part + i;          // pair (2j, 2j + 1)
    float x0 = x[2 * i], x1 = x[2 * i + 1];
    if (j < npairs) {
      const float c = sm.cs[j], sn = sm.sn[j];
      const float r0 = fmaf(x0, c, -x1 * sn);
      const float r1 = fmaf(x0, sn, x1 * c);
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
__device__ void prep_scales(PrepSmem& sm, const IndexerLaunch& a) {
  const int tid = threadIdx.x;
  const float inv_norm = 1.f / sqrtf((float)(a.H * kD));   // one rounding (exact for H = 32)
  // max|q'_h| * 2^e_h in [2^14, 2^15) keeps both fp16 terms normal
  {
    const int h = tid >> 3, part = tid & 7;   // 32 heads x 8 lanes
    float mx = 0.f;
#pragma unroll
    for (int d = 0; d < 16; ++d) mx = fmaxf(mx, fabsf(sm.qs[h][16 * part + d]));
    mx = fmaxf(mx, __shfl_xor(mx, 1));
    mx = fmaxf(mx, __shfl_xor(mx, 2));
    mx = fmaxf(mx, __shfl_xor(mx, 4));
    if (part == 0) {
      int e = 0;
      if (mx > 0.f) {
        int x;
        frexpf(mx, &x);   // mx = f * 2^x, f in [0.5, 1)
        e = 15 - x;
      }
      sm.ex[h] = e;
      const float wv = h < a.H ? sm.wv[h] * inv_norm : 0.f;
      sm.coef[h] = ldexpf(wv, -e);
    }
  }
  __syncthreads();
}

// hi/lo fp16 split of q' * 2^e (exact power-of-two scaling; the residual v - hi is exact in fp32).
__device__ __forceinline__ void split_half8(const float* v, u32x4& h4, u32x4& l4) {
  _Float16 hi[8], lo[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    hi[i] = (_Float16)v[i];                           // |v| < 2^15: normal
    lo[i] = (_Float16)(v[i] - (float)hi[i]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h4[i] = pack_half2(hi[2 * i], hi[2 * i + 1]);
    l4[i] = pack_half2(lo[2 * i], lo[2 * i + 1]);
  }
}

__device__ void build_fp8_operands(PrepSmem& sm, QPrepFp8* o, const IndexerLaunch& a, int t) {
  const int tid = threadIdx.x;
  prep_scales(sm, a);
  // A operand of lane l (row m = l & 31, half g = l >> 5) for K-step s: q'[m][32(s>>1) + 16g + 8(s&1) + i]
  {
    const int l = tid & 63, sg = tid >> 6;
    const int m = l & 31, g = l >> 5;
    const int e = sm.ex[m];
#pragma unroll
    for (int ss = 0; ss < 2; ++ss) {
      const int s = 2 * sg + ss;
      const int base = 32 * (s >> 1) + 16 * g + 8 * (s & 1);
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = ldexpf(sm.qs[m][base + i], e);
      u32x4 h4, l4;
      split_half8(v, h4, l4);
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

// Many queries (prefill): each query's MFMA operands prepared once, one workgroup per query, into
// the workspace; the grouped stream kernel below loads them.
__global__ void __launch_bounds__(kThreads) k_index_qprep_fp8(IndexerLaunch a, void* ws) {
  __shared__ PrepSmem sm;
  const int t = blockIdx.x;
  const int p = clampi(a.q_pos[t], -1, a.max_ctx - 1);
  prep_query(sm, a, t, p < 0 ? 0 : p);
  build_fp8_operands(sm, reinterpret_cast<QPrepFp8*>(reinterpret_cast<uint8_t*>(ws) + (size_t)t * kQPrepBytes), a, t);
}

// fp32 keys: q' as fp32 and the head weights, one workgroup per query, to the workspace.
__global__ void __launch_bounds__(kThreads) k_index_qprep(IndexerLaunch a, void* ws) {
  __shared__ PrepSmem sm;
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int p = clampi(a.q_pos[t], -1, a.max_ctx - 1);
  prep_query(sm, a, t, p < 0 ? 0 : p);
  QPrepF32* o = reinterpret_cast<QPrepF32*>(reinterpret_cast<uint8_t*>(ws) + (size_t)t * kQPrepBytes);
  const float inv_norm = 1.f / sqrtf((float)(a.H * kD));   // one rounding (exact for H = 32)
  for (int e = tid; e < kHPad * kD; e += kThreads) o->q[e / kD][e % kD] = sm.qs[e / kD][e % kD];
  if (tid < kHPad) o->coef[tid] = tid < a.H ? sm.wv[tid] * inv_norm : 0.f;
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

// Cache policy of the score stores: non-temporal.  The scores are written once and read by the
// selection (or the caller) after the kernel; kept out of the L2 as dirty lines, they neither compete
// with the key stream there nor have to be written back at the end of the kernel (measured: the
// kernel and the hand-over to the next one are both shorter).
constexpr int kStreamStore = 2;   // the nt bit of the buffer store's cache-policy operand

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

// max(x, 0) as one instruction: a signed integer max of the bit pattern with 0 (negative floats,
// -0 included, have the sign bit set, so they become +0; non-negative floats keep their bits).
// fmaxf would add a NaN-quieting max first, which the ReLU does not need (a NaN score only arises
// from NaN key codes, which no writer produces).  Written in C, not assembly, so that the compiler
// sees the read of the MFMA result and keeps the wait states it needs.
__device__ __forceinline__ float relu1(float x) {
  return __builtin_bit_cast(float, max(__builtin_bit_cast(int, x), 0));
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
  for (int r = 0; r < 16; ++r) part = fmaf(cf[r], relu1(acc[r]), part);
  // lanes l and l^32 hold the two halves of key column l&31's head sum
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part), false, false);
  return (__uint_as_float(sw[0]) + __uint_as_float(sw[1])) * kt.sc;
}

// Two tiles at once with independent accumulators (the MFMA chains interleave; used where the
// matrix cores, not memory, bound the stream).  The matrix chains are issued at raised wave priority,
// so that the SIMD's other wave does not hold them up with vector work; the epilogue runs at the
// normal priority (measured: the grouped kernel 3-9 % faster; the decode stream slower, so
// tile_scores keeps the normal priority).
__device__ __forceinline__ void tile_scores2(const KeyTile& k0, const KeyTile& k1, const half8* ahi, const half8* alo,
                                             const float* cf, float& s0, float& s1) {
  float16v a0 = {}, a1 = {};
  __builtin_amdgcn_s_setprio(1);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const half8 x0 = fp8x8_to_half8(k0.x[c][2 * h], k0.x[c][2 * h + 1]);
      const half8 x1 = fp8x8_to_half8(k1.x[c][2 * h], k1.x[c][2 * h + 1]);
      a0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(ahi[2 * c + h], x0, a0, 0, 0, 0);
      a1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(ahi[2 * c + h], x1, a1, 0, 0, 0);
      a0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(alo[2 * c + h], x0, a0, 0, 0, 0);
      a1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(alo[2 * c + h], x1, a1, 0, 0, 0);
    }
  }
  __builtin_amdgcn_s_setprio(0);
  float p0 = 0.f, p1 = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    p0 = fmaf(cf[r], relu1(a0[r]), p0);
    p1 = fmaf(cf[r], relu1(a1[r]), p1);
  }
  const auto w0 = __builtin_amdgcn_permlane32_swap(__float_as_uint(p0), __float_as_uint(p0), false, false);
  const auto w1 = __builtin_amdgcn_permlane32_swap(__float_as_uint(p1), __float_as_uint(p1), false, false);
  s0 = (__uint_as_float(w0[0]) + __uint_as_float(w0[1])) * k0.sc;
  s1 = (__uint_as_float(w1[0]) + __uint_as_float(w1[1])) * k1.sc;
}

// 16-byte slot of (row r, chunk k) of a 32-row key tile in LDS: chunks are XOR-swizzled by row pair
// so that the 16 lanes of a ds_read_b128 quarter (rows col..col+15, one chunk) hit 16 different
// bank groups.
__device__ __forceinline__ int tile_slot(int r, int k) { return 8 * r + (k ^ ((r >> 1) & 7)); }

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt out of range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Raw buffer descriptor words (as make_rsrc builds them) for the inline-assembly loads below.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t p = (uint64_t)(uintptr_t)base;
  return i32x4{__builtin_amdgcn_readfirstlane((int)(uint32_t)p), __builtin_amdgcn_readfirstlane((int)(uint32_t)(p >> 32) & 0xFFFF),
               __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000};
}

typedef __attribute__((address_space(3))) void* lds_vp;

// Streaming buffer loads straight into LDS, non-temporal (the key stream is read once): lane l's 16
// (4) bytes at byte voff of the buffer land at LDS byte lds + 16*l (4*l); offsets past the buffer
// read zero.  Inline assembly keeps the compiler from treating them as LDS writes (it would make
// every later LDS read wait for all of them); callers wait with wait_vm.
__device__ __forceinline__ void bdma16(i32x4 rs, uint32_t voff, void* lds) {
  const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_vp)lds);
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds" ::"v"(voff), "s"(rs), "s"(base)
               : "memory", "m0");
}
__device__ __forceinline__ void bdma4(i32x4 rs, uint32_t voff, void* lds) {
  const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_vp)lds);
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dword %0, %1, 0 offen nt lds" ::"v"(voff), "s"(rs), "s"(base)
               : "memory", "m0");
}

constexpr int kRing = 3;   // key tiles in flight per wave (its own LDS ring)

struct WaveRing {
  u32x4 key[kRing][kTile * kD / 16];
  float sc[kRing][kTile];
};

// Query-prep inputs loaded with assembly loads, so that the compiler does not wait for the key
// gathers issued after them (it cannot see those and would drain the whole load counter before
// the first use).  prep_landed<N> waits until at most N later operations are outstanding; the
// values are tied to that wait so that nothing reads them earlier.
__device__ __forceinline__ u32x4 aload16(const void* p) {
  u32x4 v;
  asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(v) : "v"(p) : "memory");
  return v;
}
__device__ __forceinline__ float aload4(const float* p) {
  float v;
  asm volatile("global_load_dword %0, %1, off" : "=v"(v) : "v"(p) : "memory");
  return v;
}

template <bool BF16Q>
__device__ __forceinline__ PrepIn prep_issue(const IndexerLaunch& a, int t) {
  const int tid = threadIdx.x;
  const int h = tid >> 3, part = tid & 7;
  const int hc = min(h, a.H - 1);
  PrepIn in;
  const size_t base = ((size_t)t * a.H + hc) * kD + 16 * part;
  if (BF16Q) {
    const u32x4* src = reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(a.q) + base);
    in.raw[0] = aload16(src);
    in.raw[1] = aload16(src + 1);
  } else {
    const u32x4* src = reinterpret_cast<const u32x4*>(reinterpret_cast<const float*>(a.q) + base);
#pragma unroll
    for (int i = 0; i < 4; ++i) in.raw[i] = aload16(src + i);
  }
  const int th = min(tid, a.H - 1);
  const float* pf = a.rope_dim > 0 ? a.inv_freq : a.w;
  const float* ps = a.ssmax_s ? a.ssmax_s : a.w;
  const float* pb = a.ssmax_s ? a.ssmax_b : a.w;
  in.invf = aload4(pf + (a.rope_dim > 0 ? min(tid, a.rope_dim / 2 - 1) : 0));
  in.ss = aload4(ps + th);
  in.sb = aload4(pb + th);
  in.wv = aload4(a.w + (size_t)t * a.H + th);
  return in;
}

template <int N, bool BF16Q>
__device__ __forceinline__ void prep_landed(PrepIn& in) {
  wait_vm<N>();
  if (BF16Q)
    asm volatile("" : "+v"(in.raw[0]), "+v"(in.raw[1]), "+v"(in.invf), "+v"(in.ss), "+v"(in.sb), "+v"(in.wv));
  else
    asm volatile("" : "+v"(in.raw[0]), "+v"(in.raw[1]), "+v"(in.raw[2]), "+v"(in.raw[3]), "+v"(in.invf),
                 "+v"(in.ss), "+v"(in.sb), "+v"(in.wv));
}

// Vector-memory operations issued after tile it's gathers and before its wait, per wave of the
// decode kernel: iteration m issues the gathers of tile m + kRing (five loads, when that tile
// exists) right after reading its slot, then stores its 32 scores (one store); tiles 0..kRing-1
// are gathered before the loop.
constexpr int kLoadsPerTile = 5;   // four 16-byte row loads and one scale load
constexpr int ring_wait(int it, int tpw) {
  int n = 0;
  if (it < kRing) {
    for (int j = it + 1; j < kRing && j < tpw; ++j) n += kLoadsPerTile;
    for (int m = 0; m < it; ++m) n += (m + kRing < tpw ? kLoadsPerTile : 0) + 1;
  } else {
    n += 1;   // the store of iteration it - kRing, issued after that iteration's gathers
    for (int m = it - kRing + 1; m < it; ++m) n += (m + kRing < tpw ? kLoadsPerTile : 0) + 1;
  }
  return n;
}
static_assert(ring_wait(0, 32) == 10 && ring_wait(1, 32) == 11 && ring_wait(2, 32) == 12 && ring_wait(3, 32) == 13 &&
                      ring_wait(29, 32) == 13 && ring_wait(30, 32) == 8 && ring_wait(31, 32) == 3,
              "ring wait counts");

// Fused selection: this chunk's candidates for the row's top-k, in column order, in the chunk's own
// region of the row's item list (chunk c of a row of S chunks owns items c * cap .. c * cap + cap - 1,
// cap = kTkItemCap / S, so no counter is involved).  kq is twice the chunk's expected share of the k
// (its share of the row's keys) plus 32; every score whose first digit is >= lb, the digit of the
// chunk's kq-th largest score (from the chunk's histogram in LDS), is emitted, and the chunk's table
// entry records (first item, count | lb << 16); the chunk's histogram bins from lb up are added into
// the row's.  A chunk with more candidates than its region holds writes none and an entry that
// claims more items than the list has.  With L the largest lb of the row's chunks, the row histogram
// is exact from L up and the items at or above L are exactly the row's keys there; when at least k
// keys lie at or above L the selection kernel finds the row's top k among the items, and otherwise
// selects from the scores directly.  The chunk's scores are read from the copy the score loop kept
// in LDS (sc, chunk-relative columns), not from memory.
struct EmitSmem {
  uint32_t sbuf[32];
  uint32_t wsum[16];
};

// Bin b of the chunk histogram, whose 16-bit counters sit two to a word (bin 2i low, 2i + 1 high).
__device__ __forceinline__ uint32_t packed_bin(const uint32_t* h2, int b) {
  return (h2[b >> 1] >> ((b & 1) << 4)) & 0xFFFFu;
}

// One wave's search of the packed kTkBins-bin histogram for the bin that holds the need-th largest
// key (bins counted from the top); 0 when fewer than need keys are counted.  Lane l sums bins
// kTkBins - 64 (l + 1) .. kTkBins - 64 l - 1; a scan over the lanes picks the lane, a second scan
// over that lane's 64 bins (one per lane) picks the bin.
__device__ inline int packed_find_bin(const uint32_t* h2, uint32_t need) {
  constexpr int PER = kTkBins / 64;
  static_assert(PER == 64, "one bin per lane in the second scan");
  const int lane = threadIdx.x & 63;
  const int lo = kTkBins - PER * (lane + 1);
  uint32_t sum = 0;
#pragma unroll
  for (int q = 0; q < PER / 8; ++q) {
    const uint4 x = *reinterpret_cast<const uint4*>(h2 + lo / 2 + 4 * q);
    sum += (x.x & 0xFFFFu) + (x.x >> 16) + (x.y & 0xFFFFu) + (x.y >> 16) + (x.z & 0xFFFFu) + (x.z >> 16) +
           (x.w & 0xFFFFu) + (x.w >> 16);
  }
  const uint32_t incl = tk_wave_incl_scan(sum);
  const uint64_t m = __ballot(incl - sum < need && need <= incl);
  if (m == 0) return 0;
  const int l0 = __builtin_ctzll(m);
  const uint32_t ab = (uint32_t)__builtin_amdgcn_readlane((int)(incl - sum), l0);
  const int b = kTkBins - PER * l0 - 1 - lane;   // lane i: the i-th of those bins from the top
  const uint32_t c = packed_bin(h2, b);
  const uint32_t inc2 = ab + tk_wave_incl_scan(c);
  const uint64_t m2 = __ballot(inc2 - c < need && need <= inc2);
  return kTkBins - PER * l0 - 1 - __builtin_ctzll(m2);
}

template <int TPW>
__device__ void emit_candidates(const IndexerLaunch& a, int t, int n, int c0, uint32_t nrow, const uint32_t* lh2,
                                const float* sc, EmitSmem& em) {
  constexpr int chunk = 4 * kTile * TPW;
  constexpr int Q = chunk / (4 * kThreads);
  static_assert(Q * (kThreads / 64) <= 16, "wsum size");
  const uint32_t share = (uint32_t)(((uint64_t)a.topk_k * chunk + (uint64_t)n - 1) / (uint64_t)n);
  const uint32_t kq = min(nrow, 2u * share + 32u);
  if (threadIdx.x < 64) {   // wave 0 finds lb; the barrier hands it to the others
    const int b = packed_find_bin(lh2, kq);
    if (threadIdx.x == 0) em.sbuf[0] = (uint32_t)b;
  }
  __syncthreads();
  const int lb = (int)em.sbuf[0];
  uint32_t* gh = tk_hist(a.topk_ws, t);   // the row's histogram, from lb up (exact above the row's largest lb)
  for (int i = lb + (int)threadIdx.x; i < kTkBins; i += kThreads) {
    const uint32_t c = packed_bin(lh2, i);
    if (c) atomicAdd(&gh[i], c);
  }
  uint32_t key[Q][4];
  uint32_t mask = 0;
#pragma unroll
  for (int q = 0; q < Q; ++q) {   // the slice layout of the selection kernels: column 4*(256q + thread) + e
    const int l = 4 * kThreads * q + 4 * (int)threadIdx.x;
    const float4 v = *reinterpret_cast<const float4*>(sc + l);
    key[q][0] = score_key(v.x);
    key[q][1] = score_key(v.y);
    key[q][2] = score_key(v.z);
    key[q][3] = score_key(v.w);
#pragma unroll
    for (int e = 0; e < 4; ++e) mask |= ((uint32_t)(l + e) < nrow ? 1u : 0u) << (4 * q + e);
  }
  uint32_t fl[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    fl[q] = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      fl[q] |= (((mask >> (4 * q + e)) & 1u) && (key[q][e] >> kTkShift0) >= (uint32_t)lb ? 1u : 0u) << e;
  }
  uint32_t pos[Q];
  const uint32_t total = tk_ordered_slots<Q, kThreads>(fl, pos, em.wsum);
  uint32_t* rw = tk_row(a.topk_ws, t);
  const uint32_t cap = (uint32_t)kTkItemCap / (uint32_t)((n + chunk - 1) / chunk);
  const uint32_t st = (uint32_t)blockIdx.x * cap;
  const bool fits = total <= cap;
  if (threadIdx.x == 0)
    *reinterpret_cast<uint2*>(rw + kTkOffTable + 2 * blockIdx.x) =
        make_uint2(fits ? st : (uint32_t)kTkItemCap, (fits ? total : 0xFFFFu) | ((uint32_t)lb << 16));
  if (!fits) return;
  uint2* items = reinterpret_cast<uint2*>(rw + kTkOffItems);
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    uint32_t p = st + pos[q];
    const uint32_t cq = (uint32_t)(c0 + 4 * kThreads * q + 4 * (int)threadIdx.x);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if ((fl[q] >> e) & 1u) items[p++] = make_uint2(key[q][e], cq + e);
  }
}

// TPW: 32-key tiles per wave (a workgroup covers 4 * 32 * TPW keys).  HIST: also histogram the
// first top-k digit of this chunk's scores into the top-k workspace (the fused selection path).
//
// Each wave streams its tiles through a private ring of kRing LDS slots: every load instruction
// reads whole 128-byte key rows (8 lanes per row) with the non-temporal policy, which the memory
// system serves markedly faster than the per-lane operand pattern; the MFMA operands are then read
// from LDS (swizzled, conflict-free).  The ring is private, so no barrier is involved: a wave waits
// for its own loads with vmcnt.
template <int TPW, bool HIST, bool BF16Q, bool PAGED>
__global__ void __launch_bounds__(kThreads)
k_index_scores_fp8(IndexerLaunch a) {
  constexpr int chunk = 4 * kTile * TPW;
  __shared__ __attribute__((aligned(16))) WaveRing ring[4];
  // query prep, then (fused path) the chunk's histogram and scores, which reuse the prep's space.
  // The histogram's counters are 16-bit, two to a word (a chunk holds at most 4096 keys), so that
  // the scores fit beside it and two workgroups still share a CU; it is searched packed.
  __shared__ __attribute__((aligned(16))) union PrepOrHist {
    PrepSmem sm;
    struct {
      uint32_t lh2[HIST ? kTkBins / 2 : 1];
      float sc[HIST ? chunk : 1];
    } h;
  } pu;
  static_assert(!HIST || chunk < 65536, "16-bit histogram counters");
  PrepSmem& sm = pu.sm;
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
  const i32x4 krs = rsrc_words(kseq, PAGED ? 0u : nrow * kD);
  const i32x4 srs = rsrc_words(sseq, PAGED ? 0u : nrow * 4u);
  // without a score buffer (block maxima only) the range is empty and the stores write nothing
  const __amdgpu_buffer_rsrc_t ors = make_rsrc(srow, a.scores ? nrow * 4u : 0u);
  constexpr uint32_t kStride = 4 * kTile;   // the 4 waves interleave 32-key tiles
  WaveRing& wr = ring[wave];
  // paged caches: lane j holds the block of this wave's tile j (a tile's 32 rows lie in one block;
  // tiles past the row's end read its last block and are never stored)
  int blk = 0;
  if (PAGED && lane < TPW) blk = paged_block(a.pg, b, min(c0 + wave * kTile + lane * (int)kStride, n - 1));

  // tile j of this wave (rows wave*32 + j*128 .. of the chunk) into ring slot j % kRing: load c
  // brings rows 8c..8c+7, lane l the 16-byte chunk stored at slot position 64c + l
  const int lr = lane >> 3, lj = lane & 7;
  auto issue = [&](int j) {
    const uint32_t row0 = wave * kTile + (uint32_t)j * kStride;
    if (PAGED) {   // the tile's 32 rows: one contiguous 4 KiB range of 16x16 tiles in its block
      const int bj = __builtin_amdgcn_readlane(blk, j);
      const size_t r0 = (size_t)bj * a.pg.page + (size_t)((c0 + (int)row0) % a.pg.page);
      const i32x4 trs = rsrc_words(reinterpret_cast<const uint8_t*>(a.k_cache) + r0 * kD, kTile * kD);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int r = 8 * c + lr;
        const int k = lj ^ ((r >> 1) & 7);
        bdma16(trs, key_tile_byte(r, 16 * k), &wr.key[j % kRing][64 * c]);
      }
      if (lane < kTile) bdma4(rsrc_words(a.k_scale + r0, kTile * 4u), lane * 4u, &wr.sc[j % kRing][0]);
      return;
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int r = 8 * c + lr;
      const int k = lj ^ ((r >> 1) & 7);     // the chunk whose swizzled slot is position 64c + l
      bdma16(krs, (row0 + r) * kD + 16u * k, &wr.key[j % kRing][64 * c]);
    }
    if (lane < kTile) bdma4(srs, (row0 + lane) * 4u, &wr.sc[j % kRing][0]);   // 32 scales: lanes 0..31
  };

  // The query-prep inputs go out, then the first key tiles; the prep (RoPE and SSMax, power-of-two
  // scaling, hi/lo fp16 split) runs as soon as its inputs have landed, while the tiles are in flight.
  PrepIn pin = prep_issue<BF16Q>(a, t);
#pragma unroll
  for (int i = 0; i < kRing; ++i)
    if (i < TPW) issue(i);
  prep_landed<5 * (kRing < TPW ? kRing : TPW), BF16Q>(pin);
  prep_compute<BF16Q>(sm, pin, a, p);
  prep_scales(sm, a);
  // this lane's MFMA A operands (row m = lane & 31, half g) for the 8 K-steps, and its 16
  // accumulator-row weights (row r of a lane in half g is head 8(r>>2) + 4g + (r&3))
  half8 ahi[8], alo[8];
  float cf[16];
  {
    const int m = lane & 31;
    const int e = sm.ex[m];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int base = 32 * (s >> 1) + 16 * g + 8 * (s & 1);
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = ldexpf(sm.qs[m][base + i], e);
      u32x4 h4, l4;
      split_half8(v, h4, l4);
      ahi[s] = __builtin_bit_cast(half8, h4);
      alo[s] = __builtin_bit_cast(half8, l4);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) cf[r] = sm.coef[8 * (r >> 2) + 4 * g + (r & 3)];
  }

  // only lanes 0..31 store (lanes 32..63 hold the same columns); the others aim past the range.
  // On the fused path every lane aims past it: the chunk's scores are stored from LDS at the end,
  // in one burst, and the dropped per-tile store keeps the ring's wait counts (which count it).
  const bool hist = HIST && n > a.topk_k;
  const uint32_t out_off = (g == 0 && !hist) ? 4u * col : 0x80000000u;
  if (HIST) {
    __syncthreads();   // every wave is done with the prep space
    if (hist)
      for (int i = threadIdx.x; i < kTkBins / 2; i += kThreads) pu.h.lh2[i] = 0;
    __syncthreads();
  }
  // block maxima (block-sparse selection): the largest score key of each block of the chunk
  __shared__ uint32_t sbm[HIST ? 1 : chunk / kTile];
  const bool bm = !HIST && a.bmax != nullptr;
  if (!HIST && bm) {
    for (int i = threadIdx.x; i < chunk / kTile; i += kThreads) sbm[i] = 0u;
    __syncthreads();
  }

  // Every wait's vmcnt is a compile-time count (ring_wait): the first kRing tiles and the last two
  // are unrolled, and the tiles between run as a rolled loop of kRing-tile groups whose waits are all
  // ring_wait's steady value (each copy in a group also knows its ring slot).  A slot is refilled as
  // soon as its contents are in registers, before the tile's matrix work, so the next gather is in
  // flight while this tile is scored.  The rolled middle keeps the kernel's code small: it is
  // fetched again after the other kernels of a step have run.
  uint32_t rel = wave * kTile;
  auto step = [&](auto slot_c, auto wait_c, int it) {
    constexpr int S = decltype(slot_c)::value;
    wait_vm<decltype(wait_c)::value>();
    asm volatile("" ::: "memory");           // the ring reads below stay after the wait
    KeyTile cur;
    const u32x4* slot = wr.key[S];
#pragma unroll
    for (int c = 0; c < 4; ++c) cur.x[c] = slot[tile_slot(col, 2 * c + g)];
    cur.sc = wr.sc[S][col];
    if (it + kRing < TPW) {
      __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));   // lgkmcnt(0): the slot's contents are in registers
      issue(it + kRing);
    }
    const float sc = tile_scores(cur, ahi, alo, cf);
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, sc), ors, out_off + 4u * rel, 0, kStreamStore);
    if (hist && g == 0) {
      pu.h.sc[rel + col] = sc;
      if (rel + col < nrow) {
        const uint32_t d = score_key(sc) >> kTkShift0;
        atomicAdd(&pu.h.lh2[d >> 1], 1u << ((d & 1u) << 4));
      }
    }
    if (!HIST && bm) {   // a 32-key tile lies in one block: its maximum, then the block's
      const uint32_t kk = tk_wave_max((g == 0 && rel + col < nrow) ? score_key(sc) : 0u);
      if (lane == 0) atomicMax(&sbm[rel / (uint32_t)a.bblock], kk);
    }
    rel += kStride;
  };
  static_assert(kRing == 3 && TPW >= kRing + 2 && (TPW - 2 - kRing) % kRing == 0, "loop split");
  static_assert(ring_wait(kRing, TPW) == ring_wait(TPW - 3, TPW), "steady wait count");
  step(std::integral_constant<int, 0>(), std::integral_constant<int, ring_wait(0, TPW)>(), 0);
  step(std::integral_constant<int, 1>(), std::integral_constant<int, ring_wait(1, TPW)>(), 1);
  step(std::integral_constant<int, 2>(), std::integral_constant<int, ring_wait(2, TPW)>(), 2);
  constexpr int kSteady = ring_wait(kRing, TPW);
#pragma unroll 1
  for (int it = kRing; it < TPW - 2; it += kRing) {
    step(std::integral_constant<int, 0>(), std::integral_constant<int, kSteady>(), it);
    step(std::integral_constant<int, 1>(), std::integral_constant<int, kSteady>(), it + 1);
    step(std::integral_constant<int, 2>(), std::integral_constant<int, kSteady>(), it + 2);
  }
  step(std::integral_constant<int, (TPW - 2) % kRing>(), std::integral_constant<int, ring_wait(TPW - 2, TPW)>(), TPW - 2);
  step(std::integral_constant<int, (TPW - 1) % kRing>(), std::integral_constant<int, ring_wait(TPW - 1, TPW)>(), TPW - 1);
  if (!HIST && bm) {   // the chunk's blocks that hold visible keys
    __syncthreads();
    const int nbc = ((int)nrow + a.bblock - 1) / a.bblock;
    for (int i = threadIdx.x; i < nbc; i += kThreads) a.bmax[(size_t)t * a.bld + c0 / a.bblock + i] = sbm[i];
  }
  if (hist) {
    __syncthreads();   // every wave's counts and scores are in LDS
    // 4-byte stores (a wave's instruction covers two whole lines): the range check drops each
    // column past the row, where a wider store straddling the end would be dropped whole
    for (int i = (int)threadIdx.x; i < chunk; i += kThreads)
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, pu.h.sc[i]), ors, 4u * (uint32_t)i, 0,
                                            kStreamStore);
    if (a.topk_emit) {   // this chunk's candidates and its histogram from their lowest digit up
      __shared__ EmitSmem em;
      emit_candidates<TPW>(a, t, n, c0, nrow, pu.h.lh2, pu.h.sc, em);
    } else {             // this chunk's counts into the row's histogram (read by the next kernel)
      uint32_t* gh = tk_hist(a.topk_ws, t);
      for (int i = threadIdx.x; i < kTkBins; i += kThreads) {
        const uint32_t c = packed_bin(pu.h.lh2, i);
        if (c) atomicAdd(&gh[i], c);
      }
    }
  }
}

// Grouped variant for many queries, or several per sequence (chunked prefill, multi-token verify
// blocks).  Workgroup (x, y) scores key chunk x for the four queries 4y..4y+3, one per wave, with
// operands prepared once per query in the workspace.  When the four queries read the same sequence
// (consecutive queries of a prefill chunk or of a verify block), each 32-key tile
// is gathered once into an LDS ring (global_load_lds, one 16-byte chunk per lane) and all four waves
// read their MFMA B operands from it, so the key stream is read from memory once per four queries.
// Otherwise every wave streams its own keys from memory as the decode kernel does.
constexpr int kGroup = 4;
constexpr int kRingTiles = 8;                    // key tiles in flight per workgroup
constexpr int kTileBytes = kTile * kD;           // 4 KiB

__device__ __forceinline__ void dma16(const void* g, void* lds) {
  const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_vp)lds);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(base) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* g, void* lds) {
  const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_vp)lds);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(base) : "memory", "m0");
}
// Barrier for LDS hand-offs that does not wait for global loads in flight.
__device__ __forceinline__ void lds_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}


struct SharedTiles {
  u32x4 key[kRingTiles][kTile * kD / 16];
  float sc[kRingTiles][kTile];
};

// Tile it of a paged chunk (this lane's row col, half g): the tile's 4 KiB of 16x16 tiles in its
// block, whose id lane `it` of blk holds.
__device__ __forceinline__ void load_tile_paged(KeyTile& kt, const IndexerLaunch& a, int blk, int it, int c0, int col,
                                                int g) {
  const int bj = __builtin_amdgcn_readlane(blk, it);
  const size_t r0 = (size_t)bj * a.pg.page + (size_t)((c0 + kTile * it) % a.pg.page);
  const __amdgpu_buffer_rsrc_t trs = make_rsrc(reinterpret_cast<const uint8_t*>(a.k_cache) + r0 * kD, kTile * kD);
#pragma unroll
  for (int c = 0; c < 4; ++c)
    kt.x[c] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(trs, key_tile_byte(col, 32 * c + 16 * g), 0, 0));
  kt.sc = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(a.k_scale + r0, kTile * 4u),
                                                                         4u * col, 0, 0));
}

// The block of each of the chunk's tiles for sequence b, tile j in lane j (the last block of the
// row for tiles past it; their scores are never stored).
template <int TPW>
__device__ __forceinline__ int chunk_blocks(const IndexerLaunch& a, int b, int c0, int n) {
  static_assert(TPW <= 64, "one tile per lane");
  const int lane = threadIdx.x & 63;
  return lane < TPW ? paged_block(a.pg, b, min(c0 + kTile * lane, n - 1)) : 0;
}

// Waves of mismatched sequences: each streams its own keys (as the decode kernel does).
template <int TPW, bool PAGED>
__device__ void grouped_private_stream(const IndexerLaunch& a, int t, int c0, const half8* ahi, const half8* alo,
                                       const float* cf) {
  const int lane = threadIdx.x & 63, g = lane >> 5, col = lane & 31;
  const int b = clampi(a.q_seq[t], 0, a.B - 1);
  const int n = clampi(a.q_pos[t], -1, a.max_ctx - 1) + 1;
  if (c0 >= n) return;
  const uint32_t nrow = (uint32_t)(min(n, c0 + kTile * TPW) - c0);
  const __amdgpu_buffer_rsrc_t krs =
      make_rsrc(reinterpret_cast<const uint8_t*>(a.k_cache) + ((size_t)b * a.max_ctx + c0) * kD, PAGED ? 0u : nrow * kD);
  const __amdgpu_buffer_rsrc_t srs = make_rsrc(a.k_scale + (size_t)b * a.max_ctx + c0, PAGED ? 0u : nrow * 4u);
  const __amdgpu_buffer_rsrc_t ors = make_rsrc(a.scores + (size_t)t * a.ld + c0, nrow * 4u);
  const uint32_t out_off = g == 0 ? 4u * col : 0x80000000u;
  const int blk = PAGED ? chunk_blocks<TPW>(a, b, c0, n) : 0;
  auto load = [&](KeyTile& kt, int it) {
    if (PAGED) load_tile_paged(kt, a, blk, it, c0, col, g);
    else load_tile(kt, krs, srs, it * kTile + col, g);
  };
  KeyTile tb[kDepth];
#pragma unroll
  for (int i = 0; i < kDepth; ++i) load(tb[i], i);
  uint32_t rel = 0;
#pragma unroll
  for (int it = 0; it < TPW; ++it) {
    KeyTile& cur = tb[it % kDepth];
    const float sc = tile_scores(cur, ahi, alo, cf);
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, sc), ors, out_off + 4u * rel, 0, kStreamStore);
    if (it + kDepth < TPW) load(cur, it + kDepth);
    rel += kTile;
  }
}

template <int TPW, bool PAGED>
__global__ void __launch_bounds__(kThreads)
k_index_scores_fp8_grouped(IndexerLaunch a, const void* ws) {
  static_assert(TPW >= kRingTiles, "ring shorter than the chunk");
  __shared__ __attribute__((aligned(16))) SharedTiles st;
  __shared__ int sseq[kGroup], sn[kGroup];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 5, col = lane & 31;
  const int t = kGroup * blockIdx.y + wave;
  const bool live = t < a.T;
  const int c0 = blockIdx.x * kTile * TPW;
  if (lane == 0) {
    sseq[wave] = live ? clampi(a.q_seq[t], 0, a.B - 1) : -1;
    sn[wave] = live ? clampi(a.q_pos[t], -1, a.max_ctx - 1) + 1 : 0;
  }
  __syncthreads();
  int b = -1, nmax = 0;
  bool uniform = true;
#pragma unroll
  for (int w = 0; w < kGroup; ++w) {
    const int sw = sseq[w];
    if (sw >= 0) {
      uniform = uniform && (b < 0 || sw == b);
      b = b < 0 ? sw : b;
      nmax = max(nmax, sn[w]);
    }
  }
  if (c0 >= nmax) return;   // every query of the group has fewer keys than the chunk start

  half8 ahi[8], alo[8];
  float cf[16];
  auto load_operands = [&]() {
    if (!live) return;
    const QPrepFp8* qp = reinterpret_cast<const QPrepFp8*>(reinterpret_cast<const uint8_t*>(ws) + (size_t)t * kQPrepBytes);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      ahi[s] = __builtin_bit_cast(half8, qp->a[2 * s][lane]);
      alo[s] = __builtin_bit_cast(half8, qp->a[2 * s + 1][lane]);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) cf[r] = qp->cf[r][lane];
  };
  if (!uniform) {
    load_operands();
    if (live) grouped_private_stream<TPW, PAGED>(a, t, c0, ahi, alo, cf);
    return;
  }

  // shared stream: rows c0.. of sequence b, up to the longest query of the group
  const int rows = min(nmax - c0, kTile * TPW);
  const int ntiles = (rows + kTile - 1) / kTile;
  const uint8_t* kseq = reinterpret_cast<const uint8_t*>(a.k_cache) + ((size_t)b * a.max_ctx + c0) * kD;
  const float* sseqp = a.k_scale + (size_t)b * a.max_ctx + c0;
  const int n = live ? sn[wave] : 0;
  const uint32_t nrow = (uint32_t)max(0, min(n - c0, kTile * TPW));
  const __amdgpu_buffer_rsrc_t ors = make_rsrc(a.scores + (size_t)(live ? t : 0) * a.ld + c0, nrow * 4u);
  const uint32_t out_off = g == 0 ? 4u * col : 0x80000000u;
  // this lane's slot q = 64 * wave + lane of each tile holds row q/8's chunk (q%8) ^ swizzle
  const int q = 64 * wave + lane;
  const int qr = q >> 3, qk = (q & 7) ^ ((qr >> 1) & 7);
  const int blk = PAGED ? chunk_blocks<TPW>(a, b, c0, nmax) : 0;
  auto issue = [&](int tau) {
    const int slot = tau % kRingTiles;
    if (PAGED) {   // the tile's rows are one 4 KiB range of 16x16 tiles in its block
      const size_t r0 = (size_t)__builtin_amdgcn_readlane(blk, tau) * a.pg.page + (size_t)((c0 + kTile * tau) % a.pg.page);
      dma16(reinterpret_cast<const uint8_t*>(a.k_cache) + r0 * kD + key_tile_byte(qr, 16 * qk), &st.key[slot][64 * wave]);
      if (lane < kTile / kGroup) dma4(a.k_scale + r0 + (kTile / kGroup) * wave + lane, &st.sc[slot][(kTile / kGroup) * wave]);
      return;
    }
    const int r = min(kTile * tau + qr, rows - 1);   // rows past the group's range read a valid row
    dma16(kseq + (size_t)r * kD + 16 * qk, &st.key[slot][64 * wave]);
    if (lane < kTile / kGroup) dma4(sseqp + min(kTile * tau + (kTile / kGroup) * wave + lane, rows - 1),
                                    &st.sc[slot][(kTile / kGroup) * wave]);
  };
  constexpr int LPT = 2;   // LDS-direct loads per wave and tile
#pragma unroll
  for (int i = 0; i < kRingTiles; ++i)
    if (i < ntiles) issue(i);
  load_operands();
  wait_vm<0>();   // operands and the first tiles are in (tells the compiler too: no waits below)
  // Two tiles per step: one barrier per pair, and their MFMA chains interleave.
  for (int tau = 0; tau < ntiles; tau += 2) {
    // gathers issued so far: the first ring's worth, then two per step from step 1 on (after the
    // wait); tiles tau and tau + 1 have landed once at most the later ones are outstanding
    const int step = tau >> 1;
    const int issued = min(ntiles, kRingTiles + 2 * max(step - 1, 0));
    const int later = issued - min(tau + 1, ntiles - 1) - 1;
    switch (later) {
      case 7: wait_vm<7 * LPT>(); break;
      case 6: wait_vm<6 * LPT>(); break;
      case 5: wait_vm<5 * LPT>(); break;
      case 4: wait_vm<4 * LPT>(); break;
      case 3: wait_vm<3 * LPT>(); break;
      case 2: wait_vm<2 * LPT>(); break;
      case 1: wait_vm<LPT>(); break;
      default: wait_vm<0>(); break;
    }
    lds_sync();   // tiles tau, tau + 1 are in LDS for every wave; every wave is done with the last pair
    if (step >= 1) {
      if (tau - 2 + kRingTiles < ntiles) issue(tau - 2 + kRingTiles);
      if (tau - 1 + kRingTiles < ntiles) issue(tau - 1 + kRingTiles);
    }
    const uint32_t rel = (uint32_t)(kTile * tau);
    if (rel < nrow) {
      KeyTile k0, k1;
      const int s0 = tau % kRingTiles, s1 = (tau + 1) % kRingTiles;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        k0.x[c] = st.key[s0][tile_slot(col, 2 * c + g)];
        k1.x[c] = st.key[s1][tile_slot(col, 2 * c + g)];
      }
      k0.sc = st.sc[s0][col];
      k1.sc = st.sc[s1][col];
      float r0, r1;
      tile_scores2(k0, k1, ahi, alo, cf, r0, r1);   // past the last tile, k1 holds stale data: not stored
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, r0), ors, out_off + 4u * rel, 0, kStreamStore);
      if (tau + 1 < ntiles)
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, r1), ors, out_off + 4u * (rel + kTile), 0,
                                              kStreamStore);
    }
  }
}

// ------------------------------------------------------------------------------------------
// Many queries per sequence (chunked prefill): query tiles over long key ranges
// ------------------------------------------------------------------------------------------

constexpr int kQtPerWave = 2;                      // queries per wave (their operands stay in registers)
constexpr int kQtQueries = kQtPerWave * kGroup;    // 8 consecutive queries per workgroup
constexpr int kQtRange = 8192;                     // keys per workgroup (256 tiles)

// One 32-key tile for two queries: the tile's fp16 B operands are converted once and feed both
// queries' MFMA chains (independent accumulators, interleaved).  Raised wave priority for the matrix
// chains, as in tile_scores2.
__device__ __forceinline__ void tile_scores_q2(const KeyTile& k, const half8* ah0, const half8* al0, const half8* ah1,
                                               const half8* al1, const float* cf0, const float* cf1, float& s0,
                                               float& s1) {
  float16v a0 = {}, a1 = {};
  __builtin_amdgcn_s_setprio(1);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const half8 x = fp8x8_to_half8(k.x[c][2 * h], k.x[c][2 * h + 1]);
      a0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah0[2 * c + h], x, a0, 0, 0, 0);
      a1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah1[2 * c + h], x, a1, 0, 0, 0);
      a0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(al0[2 * c + h], x, a0, 0, 0, 0);
      a1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(al1[2 * c + h], x, a1, 0, 0, 0);
    }
  }
  __builtin_amdgcn_s_setprio(0);
  float p0 = 0.f, p1 = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    p0 = fmaf(cf0[r], relu1(a0[r]), p0);
    p1 = fmaf(cf1[r], relu1(a1[r]), p1);
  }
  const auto w0 = __builtin_amdgcn_permlane32_swap(__float_as_uint(p0), __float_as_uint(p0), false, false);
  const auto w1 = __builtin_amdgcn_permlane32_swap(__float_as_uint(p1), __float_as_uint(p1), false, false);
  s0 = (__uint_as_float(w0[0]) + __uint_as_float(w0[1])) * k.sc;
  s1 = (__uint_as_float(w1[0]) + __uint_as_float(w1[1])) * k.sc;
}

// A workgroup scores 8 consecutive queries (two per wave) over one 8192-key range of their
// sequence: each 32-key tile is gathered once into the eight-tile LDS ring and feeds 8 queries, so
// the key stream per flop is half that of the four-query grouped kernel and the query operands are
// loaded once per 256 tiles instead of once per 32.  Work items (range, group) are listed
// range-major and cut into 8 contiguous parts, one per XCD (workgroups go to the XCDs round-robin
// by linear id): the workgroups of one XCD share a few key ranges, which its L2 holds.  A group
// whose queries read several sequences makes one pass per sequence.  PAGED: the range's tiles are
// 4 KiB ranges of 16x16 tiles in their cache blocks (a block holds whole 32-key tiles); each lane
// holds the block ids of tiles lane, 64 + lane, 128 + lane and 192 + lane of the range, read once
// per pass.
template <bool PAGED>
__global__ void __launch_bounds__(kThreads)
k_index_scores_fp8_qtile(IndexerLaunch a, const void* ws, int n_ranges, int n_groups) {
  static_assert(kQtRange % (2 * kTile) == 0, "ranges are whole tile pairs");
  __shared__ __attribute__((aligned(16))) SharedTiles st;
  __shared__ int sseq[kQtQueries], sn[kQtQueries];
  const int total = n_ranges * n_groups;
  const int per_xcd = (total + 7) / 8;
  const int item = (int)(blockIdx.x % 8u) * per_xcd + (int)(blockIdx.x / 8u);
  if (item >= total) return;
  const int range = item / n_groups, grp = item % n_groups;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 5, col = lane & 31;
  const int c0 = range * kQtRange;
  if (threadIdx.x < kQtQueries) {
    const int t = kQtQueries * grp + threadIdx.x;
    sseq[threadIdx.x] = t < a.T ? clampi(a.q_seq[t], 0, a.B - 1) : -1;
    sn[threadIdx.x] = t < a.T ? clampi(a.q_pos[t], -1, a.max_ctx - 1) + 1 : 0;
  }
  __syncthreads();

  half8 ahi[kQtPerWave][8], alo[kQtPerWave][8];
  float cf[kQtPerWave][16];
  int tq[kQtPerWave];
#pragma unroll
  for (int j = 0; j < kQtPerWave; ++j) {   // (a query past T loads the last one's operands; never stored)
    tq[j] = kQtQueries * grp + kQtPerWave * wave + j;
    const QPrepFp8* qp = reinterpret_cast<const QPrepFp8*>(reinterpret_cast<const uint8_t*>(ws) +
                                                           (size_t)min(tq[j], a.T - 1) * kQPrepBytes);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ahi[j][e] = __builtin_bit_cast(half8, qp->a[2 * e][lane]);
      alo[j][e] = __builtin_bit_cast(half8, qp->a[2 * e + 1][lane]);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) cf[j][r] = qp->cf[r][lane];
  }
  const uint32_t out_off = g == 0 ? 4u * col : 0x80000000u;
  const int q = 64 * wave + lane;
  const int qr = q >> 3, qk = (q & 7) ^ ((qr >> 1) & 7);
  constexpr int LPT = 2;   // LDS-direct loads per wave and tile

  // One pass of the shared stream per sequence among the group's queries (one pass when the
  // group's queries share a sequence, as in a prefill chunk); each pass stores only its queries.
  uint32_t done = 0;
#pragma unroll
  for (int i = 0; i < kQtQueries; ++i) done |= sseq[i] < 0 ? 1u << i : 0u;
  for (int pass = 0; done != (1u << kQtQueries) - 1; ++pass) {
    const int first = __builtin_ctz(~done);
    const int b = sseq[first];
    uint32_t mask = 0;
    int nmax = 0;
#pragma unroll
    for (int i = 0; i < kQtQueries; ++i)
      if (!((done >> i) & 1u) && sseq[i] == b) {
        mask |= 1u << i;
        nmax = max(nmax, sn[i]);
      }
    done |= mask;
    if (c0 >= nmax) continue;   // no query of this sequence sees the range
    if (pass > 0) __syncthreads();   // every wave is done with the ring of the last pass

    const int rows = min(nmax - c0, kQtRange);
    const int ntiles = (rows + kTile - 1) / kTile;
    const uint8_t* kseq = reinterpret_cast<const uint8_t*>(a.k_cache) + ((size_t)b * a.max_ctx + c0) * kD;
    const float* sseqp = a.k_scale + (size_t)b * a.max_ctx + c0;
    __amdgpu_buffer_rsrc_t ors[kQtPerWave];
    uint32_t nrow = 0;
#pragma unroll
    for (int j = 0; j < kQtPerWave; ++j) {
      const int i = kQtPerWave * wave + j;
      const uint32_t nr = (mask >> i) & 1u ? (uint32_t)max(0, min(sn[i] - c0, kQtRange)) : 0u;
      ors[j] = make_rsrc(a.scores + (size_t)min(tq[j], a.T - 1) * a.ld + c0, nr * 4u);
      nrow = max(nrow, nr);
    }
    int blk[kQtRange / kTile / 64] = {};   // PAGED: block of tile 64 u + lane (past the rows: the last row's)
    if (PAGED) {
#pragma unroll
      for (int u = 0; u < kQtRange / kTile / 64; ++u) blk[u] = paged_block(a.pg, b, min(c0 + kTile * (64 * u + lane), nmax - 1));
    }
    auto issue = [&](int tau) {
      const int slot = tau % kRingTiles;
      if (PAGED) {   // the tile's rows are one 4 KiB range of 16x16 tiles in its block
        static_assert(kQtRange / kTile / 64 == 4, "four block ids per lane");
        const int w = tau >> 6;   // (uniform)
        const int bw = w == 0 ? blk[0] : w == 1 ? blk[1] : w == 2 ? blk[2] : blk[3];
        const size_t r0 = (size_t)__builtin_amdgcn_readlane(bw, tau & 63) * a.pg.page + (size_t)((c0 + kTile * tau) % a.pg.page);
        dma16(reinterpret_cast<const uint8_t*>(a.k_cache) + r0 * kD + key_tile_byte(qr, 16 * qk), &st.key[slot][64 * wave]);
        if (lane < kTile / kGroup) dma4(a.k_scale + r0 + (kTile / kGroup) * wave + lane, &st.sc[slot][(kTile / kGroup) * wave]);
        return;
      }
      const int r = min(kTile * tau + qr, rows - 1);   // rows past the group's range read a valid row
      dma16(kseq + (size_t)r * kD + 16 * qk, &st.key[slot][64 * wave]);
      if (lane < kTile / kGroup)
        dma4(sseqp + min(kTile * tau + (kTile / kGroup) * wave + lane, rows - 1), &st.sc[slot][(kTile / kGroup) * wave]);
    };
#pragma unroll
    for (int i = 0; i < kRingTiles; ++i)
      if (i < ntiles) issue(i);
    wait_vm<0>();   // (the first pass: the operands too)
#pragma unroll 1
    for (int tau = 0; tau < ntiles; tau += 2) {
      // gathers issued so far: the first ring's worth, then two per step from step 1 on (after the
      // wait); tiles tau and tau + 1 have landed once at most the later ones are outstanding (the
      // score stores issued since count as later too, which only makes the wait stricter)
      const int step = tau >> 1;
      const int issued = min(ntiles, kRingTiles + 2 * max(step - 1, 0));
      const int later = issued - min(tau + 1, ntiles - 1) - 1;
      switch (later) {
        case 7: wait_vm<7 * LPT>(); break;
        case 6: wait_vm<6 * LPT>(); break;
        case 5: wait_vm<5 * LPT>(); break;
        case 4: wait_vm<4 * LPT>(); break;
        case 3: wait_vm<3 * LPT>(); break;
        case 2: wait_vm<2 * LPT>(); break;
        case 1: wait_vm<LPT>(); break;
        default: wait_vm<0>(); break;
      }
      lds_sync();   // tiles tau, tau + 1 are in LDS for every wave; every wave is done with the last pair
      if (step >= 1) {
        if (tau - 2 + kRingTiles < ntiles) issue(tau - 2 + kRingTiles);
        if (tau - 1 + kRingTiles < ntiles) issue(tau - 1 + kRingTiles);
      }
#pragma unroll 1
      for (int e = 0; e < 2; ++e) {
        const uint32_t rel = (uint32_t)(kTile * (tau + e));
        if (tau + e < ntiles && rel < nrow) {
          const int sl = (tau + e) % kRingTiles;
          KeyTile k;
#pragma unroll
          for (int c = 0; c < 4; ++c) k.x[c] = st.key[sl][tile_slot(col, 2 * c + g)];
          k.sc = st.sc[sl][col];
          float r0, r1;
          tile_scores_q2(k, ahi[0], alo[0], ahi[1], alo[1], cf[0], cf[1], r0, r1);
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, r0), ors[0], out_off + 4u * rel, 0,
                                                kStreamStore);
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, r1), ors[1], out_off + 4u * rel, 0,
                                                kStreamStore);
        }
      }
    }
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

// fp8 keys take the grouped path (queries prepared once into the workspace) from this many queries on
constexpr int kGroupedMinQueries = 256;

// ... or when there are at least two queries per sequence (verify blocks of several tokens per
// sequence, chunked prefill): consecutive queries of one sequence then share one key stream.
bool indexer_block_max_fused(int T, int B, int max_ctx, dsa_dtype_t k_dtype, int block) {
  return k_dtype == DSA_FP8_E4M3FN && !indexer_grouped(T, B, k_dtype) && block % kTile == 0 &&
         indexer_chunk(T, max_ctx) % block == 0;
}

bool indexer_grouped(int T, int B, dsa_dtype_t k_dtype) {
  return k_dtype == DSA_FP8_E4M3FN && (T >= kGroupedMinQueries || (B > 0 && T >= 2 * B));
}

size_t indexer_ws_bytes(int T, int B, dsa_dtype_t k_dtype) {
  if (k_dtype == DSA_FP8_E4M3FN && !indexer_grouped(T, B, k_dtype)) return 0;
  return (size_t)T * kQPrepBytes;
}

// 4096-key chunks (32 tiles per wave) when that still gives >= 512 workgroups, else 1024
int indexer_chunk(int T, int max_ctx) {
  const int64_t big = (int64_t)T * ((max_ctx + 4095) / 4096);
  return big >= 512 ? 4096 : 1024;
}

// Query tiles (8 queries of a sequence over 8192-key ranges) where sequences average 16 or more
// queries and the work items fill two workgroups per CU.
static bool indexer_qtile(const IndexerLaunch& a) {
  const int64_t items = (int64_t)((a.T + kQtQueries - 1) / kQtQueries) * ((a.max_ctx + kQtRange - 1) / kQtRange);
  return a.B > 0 && a.T >= 16 * a.B && items >= 512;
}

hipError_t launch_indexer(const IndexerLaunch& a, void* ws, hipStream_t s) {
  if (a.T == 0 || a.max_ctx == 0) return hipSuccess;
  if (indexer_grouped(a.T, a.B, a.k_dtype) && indexer_qtile(a)) {
    launch(k_index_qprep_fp8, dim3(a.T), dim3(kThreads), 0, s, a, ws);
    const int n_ranges = (a.max_ctx + kQtRange - 1) / kQtRange, n_groups = (a.T + kQtQueries - 1) / kQtQueries;
    const int per_xcd = (n_ranges * n_groups + 7) / 8;
    if (a.pg.table)
      launch(k_index_scores_fp8_qtile<true>, dim3(8 * per_xcd), dim3(kThreads), 0, s, a, (const void*)ws, n_ranges, n_groups);
    else
      launch(k_index_scores_fp8_qtile<false>, dim3(8 * per_xcd), dim3(kThreads), 0, s, a, (const void*)ws, n_ranges, n_groups);
  } else if (indexer_grouped(a.T, a.B, a.k_dtype)) {
    launch(k_index_qprep_fp8, dim3(a.T), dim3(kThreads), 0, s, a, ws);
    dim3 grid((a.max_ctx + kTile * 32 - 1) / (kTile * 32), (a.T + kGroup - 1) / kGroup);
    if (a.pg.table) launch(k_index_scores_fp8_grouped<32, true>, grid, dim3(kThreads), 0, s, a, (const void*)ws);
    else launch(k_index_scores_fp8_grouped<32, false>, grid, dim3(kThreads), 0, s, a, (const void*)ws);
  } else if (a.k_dtype == DSA_FP8_E4M3FN) {
    const bool hist = a.topk_ws != nullptr;
    const bool bf = a.q_dtype == DSA_BF16;
    const bool pg = a.pg.table != nullptr;
    auto go = [&](auto kernel, int chunk) {
      dim3 grid((a.max_ctx + chunk - 1) / chunk, a.T);
      launch(kernel, grid, dim3(kThreads), 0, s, a);
    };
    if (indexer_chunk(a.T, a.max_ctx) == 4096) {
      if (pg) {
        if (hist) bf ? go(k_index_scores_fp8<32, true, true, true>, 4096) : go(k_index_scores_fp8<32, true, false, true>, 4096);
        else bf ? go(k_index_scores_fp8<32, false, true, true>, 4096) : go(k_index_scores_fp8<32, false, false, true>, 4096);
      } else {
        if (hist) bf ? go(k_index_scores_fp8<32, true, true, false>, 4096) : go(k_index_scores_fp8<32, true, false, false>, 4096);
        else bf ? go(k_index_scores_fp8<32, false, true, false>, 4096) : go(k_index_scores_fp8<32, false, false, false>, 4096);
      }
    } else {
      if (pg) {
        if (hist) bf ? go(k_index_scores_fp8<8, true, true, true>, 1024) : go(k_index_scores_fp8<8, true, false, true>, 1024);
        else bf ? go(k_index_scores_fp8<8, false, true, true>, 1024) : go(k_index_scores_fp8<8, false, false, true>, 1024);
      } else {
        if (hist) bf ? go(k_index_scores_fp8<8, true, true, false>, 1024) : go(k_index_scores_fp8<8, true, false, false>, 1024);
        else bf ? go(k_index_scores_fp8<8, false, true, false>, 1024) : go(k_index_scores_fp8<8, false, false, false>, 1024);
      }
    }
  } else {
    launch(k_index_qprep, dim3(a.T), dim3(kThreads), 0, s, a, ws);
    dim3 grid((a.max_ctx + kThreads - 1) / kThreads, a.T);
    launch(k_index_scores_f32, grid, dim3(kThreads), 0, s, a, (const void*)ws);
  }
  return hipGetLastError();
}

}  // namespace dsa
