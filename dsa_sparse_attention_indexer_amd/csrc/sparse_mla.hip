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
constexpr int kRowsChunk = 2048;          // selection slots staged in LDS at a time (fp8 path)
constexpr float kLazyLog2 = 8.f;          // the running maximum lags the true one by at most this (log2)
constexpr float kNoMax = -1.0e30f;        // running maximum before the first valid key (fp8 path)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Key kappa (0..31) of a tile lives in key-major LDS row 16*((kappa>>2)&1) + 4*(kappa>>3) + (kappa&3).
__device__ __forceinline__ int ks_row_of_key(int kappa) {
  return 16 * ((kappa >> 2) & 1) + 4 * (kappa >> 3) + (kappa & 3);
}

typedef float float2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t cvt2_bf16(float2v v) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Split partials: the fp32 path keeps them unnormalised in fp32; the fp8 path (whose error budget
// is set by its bf16 operands) stores them normalised by their own sum, as bf16, which halves the
// partial traffic; the combine knows the format from the cache dtype.
__device__ __forceinline__ bool bf16_partials(const MlaLaunch& a) { return a.kv_dtype == DSA_FP8_E4M3FN; }

__device__ __forceinline__ void write_partial_or_final(const MlaLaunch& a, int t, int split, int head,
                                                       float m_log2, float l_tot, const float* o, int d0,
                                                       int ndim) {
  // o: ndim consecutive output dims starting at d0 for this head (unnormalised)
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (a.splits == 1) {
    float* dst = a.out + ((size_t)t * a.H + head) * a.kv_lora + d0;
    for (int i = 0; i < ndim; i += 4)
      *reinterpret_cast<float4*>(dst + i) = make_float4(o[i] * inv, o[i + 1] * inv, o[i + 2] * inv, o[i + 3] * inv);
  } else if (bf16_partials(a)) {
    uint16_t* dst = reinterpret_cast<uint16_t*>(a.ws) + (((size_t)t * a.H + head) * a.splits + split) * a.kv_lora + d0;
    for (int i = 0; i < ndim; i += 4)
      *reinterpret_cast<uint2*>(dst + i) = make_uint2(cvt2_bf16(float2v{o[i] * inv, o[i + 1] * inv}),
                                                      cvt2_bf16(float2v{o[i + 2] * inv, o[i + 3] * inv}));
  } else {
    float* dst = a.ws + (((size_t)t * a.H + head) * a.splits + split) * a.kv_lora + d0;
    for (int i = 0; i < ndim; i += 4)
      *reinterpret_cast<float4*>(dst + i) = make_float4(o[i], o[i + 1], o[i + 2], o[i + 3]);
  }
}

__device__ __forceinline__ void write_stats(const MlaLaunch& a, int t, int split, int head, float m_log2, float l_tot) {
  if (a.splits == 1) {
    if (a.lse) a.lse[(size_t)t * a.H + head] = l_tot > 0.f ? (m_log2 + log2f(l_tot)) * kLn2 : -INFINITY;
  } else {
    float* stats = a.ws + (size_t)a.T * a.splits * a.H * a.kv_lora;
    const size_t i = ((size_t)t * a.H + head) * a.splits + split;
    stats[2 * i] = m_log2;
    stats[2 * i + 1] = l_tot;
  }
}

typedef short short4v __attribute__((ext_vector_type(4)));

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

typedef __attribute__((address_space(3))) void* lds_void_ptr;

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding: vmcnt in bits 3:0 and
// 15:14, expcnt in 6:4 and lgkmcnt in 11:8 left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt out of range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Gathers straight into LDS: lane l's 16 (4) bytes from global address g land at LDS byte
// lds + 16*l (4*l); lds must be the same in every lane.  Written as inline assembly so that the
// compiler does not track these loads as LDS writes -- it would otherwise make later LDS accesses
// wait for every gather in flight.  The callers wait for them explicitly (wait_vmcnt) before a
// barrier, and vmcnt counts them like any other vector-memory load.
__device__ __forceinline__ void gather16_to_lds(const void* g, void* lds) {
  const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_ptr)lds);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(base) : "memory", "m0");
}
__device__ __forceinline__ void gather4_to_lds(const void* g, void* lds) {
  const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_ptr)lds);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(base) : "memory", "m0");
}

// Maximum over lanes l and l ^ 16 (ds_swizzle swap of 16-lane halves) and over l and l ^ 32
// (v_permlane32_swap), without the address arithmetic of a bpermute shuffle.
__device__ __forceinline__ float max_xor16(float x) {
  return fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x401F)));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x),
                                                  false, false);
  return fmaxf(__builtin_bit_cast(float, r[0]), __builtin_bit_cast(float, r[1]));
}

// Workgroup barrier for hand-offs through LDS: this wave's LDS operations are complete before it,
// but global loads in flight (the gathers of later tiles) are not waited for, as __syncthreads
// would.  The empty asm statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Workgroups are dispatched to the 8 XCDs round-robin by linear id.  A 1-D grid of
// 8 * inner * ceil(T / 8) workgroups is mapped so that every workgroup of query t runs on XCD t % 8:
// the splits of a query share one L2 for the query and the row indices, and the combine that reads
// their partials runs on the XCD whose L2 they were written to.  Returns false for the padding.
__device__ __forceinline__ bool xcd_query_map(int inner, int T, int* t, int* j) {
  const int id = blockIdx.x, x = id & 7, r = id >> 3;
  *j = r % inner;
  *t = 8 * (r / inner) + x;
  return *t < T;
}
inline unsigned xcd_grid(int inner, int T) { return (unsigned)(8 * inner * ((T + 7) / 8)); }

constexpr int kMlaThreads = 512;   // fp8 path: 8 waves = 4 head groups x 2 halves
constexpr int kSlots = 3;          // raw tiles in LDS: the next one to dequantise plus two in flight

template <int V>
struct IntC {
  static constexpr int value = V;
};

template <int ROPE>
struct MlaFp8 {
  static constexpr int DQ = kLora + ROPE;               // bytes of a latent row that are used
  static constexpr int KSTEPS = DQ / 32;
  static constexpr int CHUNKS = DQ / 16;                // 16-byte chunks per used row
  static constexpr int NSC = DQ / 64;                   // scales per used row
  static constexpr int WROWS = kTileK / 8;              // rows of a tile each wave gathers
  static constexpr int WCH = WROWS * CHUNKS;            // chunks per wave and tile
  static constexpr int WCHI = (WCH + 63) / 64;          // chunk loads per wave and tile
  static constexpr int WSC = WROWS * NSC;               // scale words per wave and tile
  static constexpr int WSCI = (WSC + 63) / 64;          // scale loads per wave and tile
  static constexpr int LPT = WCHI + WSCI;               // LDS-direct loads per wave and tile
  static constexpr int NCH = kTileK * CHUNKS;
  static constexpr int FULL = NCH / kMlaThreads;        // whole chunks each thread dequantises
  static constexpr int REM = NCH - FULL * kMlaThreads;  // the rest, split into 4-byte quarters
  static_assert(4 * REM <= kMlaThreads, "at most one quarter chunk per thread");
  static constexpr int ODIM = kLora / 2;                // output dims per wave
};

// Wave w = 4 * half + hg owns heads 16hg..16hg+15.  For each 32-key tile it computes the partial
// S^T over its half of the query dims (K-steps KH*half..KH*half+KH-1) for all 32 keys, adds the
// other half's partial through LDS, and accumulates O^T for output dims 256*half..256*half+255.
// Per lane: the query slice (KH operands) and 64 accumulator registers.
//
// Tiles are software-pipelined over two bf16 buffers (ks0, ks1) and kSlots raw slots, two
// barriers per tile tau:
//   B0  ks[tau & 1] holds tile tau, tile tau+1's gathers are in their slot, the other bf16 buffer
//       and tile tau's slot are free;
//   phase 1: gathers of tile tau+3 into tile tau's slot; the partial QK^T of tile tau on the
//       matrix cores while the same waves dequantise tile tau+1 into the other buffer (independent
//       instruction streams the compiler interleaves); partial scores to LDS;
//   B1  both halves' partial scores are in LDS;
//   phase 2: online softmax and PV of tile tau.
template <int ROPE>
__global__ void __launch_bounds__(kMlaThreads)
k_mla_fp8(MlaLaunch a) {
  int t, split;
  if (!xcd_query_map(a.splits, a.T, &t, &split)) return;
  using C = MlaFp8<ROPE>;
  constexpr int DQ = C::DQ, KSTEPS = C::KSTEPS, CHUNKS = C::CHUNKS, NSC = C::NSC, WROWS = C::WROWS;
  constexpr int LPT = C::LPT;
  constexpr int MD = C::ODIM / 16;                      // 16-dim output tiles per wave
  // Raw fp8 rows and scales of a tile, gathered straight into LDS.
  struct Slot {
    uint8_t raw[kTileK * DQ];
    float sc[kTileK * NSC];
  };
  typedef uint16_t KsTile[kTileK][kKsStride];
  __shared__ __attribute__((aligned(16))) Slot sl[kSlots];
  __shared__ __attribute__((aligned(16))) KsTile ks0, ks1;
  __shared__ __attribute__((aligned(16))) float4v xz[2][4][2][64];   // partial scores swapped between halves
  __shared__ int rows[kRowsChunk];                      // row of every slot of the current chunk, -1 if none
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hg = wave & 3, half = wave >> 2;
  const int c = lane & 15, g = lane >> 4;
  const int slot0 = split * a.per_split;
  const bool active = 16 * hg < a.H;
  const int head = 16 * hg + c;
  const float zscale = a.softmax_scale * kLog2e;
  const int32_t* irow = a.idx + (size_t)t * a.topk;

  // The first chunk's row indices and the query are loaded before the selection length and the
  // sequence are known, so that all of these loads are in flight together.
  const int slot_end = min(slot0 + a.per_split, a.topk);   // this split's slots before the length cut
  constexpr int RPT = kRowsChunk / kMlaThreads;
  int rv[RPT];
  auto load_rows = [&](int cb) {   // unconditional loads (slot clamped into the row): all in flight together
#pragma unroll
    for (int u = 0; u < RPT; ++u) rv[u] = irow[min(cb + tid + kMlaThreads * u, a.topk - 1)];
#pragma unroll
    for (int u = 0; u < RPT; ++u) rv[u] = cb + tid + kMlaThreads * u < slot_end ? rv[u] : -1;
  };
  load_rows(slot0);
  constexpr int KH = KSTEPS / 2;                        // K-steps per half
  static_assert(KSTEPS % 2 == 0, "query dims split in two halves");
  bf16x8 qreg[KH];                                      // zero in waves without heads
#pragma unroll
  for (int s = 0; s < KH; ++s) qreg[s] = bf16x8{};
  if (active) {
    const uint16_t* qh = reinterpret_cast<const uint16_t*>(a.q) + ((size_t)t * a.H + head) * DQ + 32 * KH * half;
#pragma unroll
    for (int s = 0; s < KH; ++s)
      qreg[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qh + 32 * s + 8 * g));
  }
  const int b = clampi(a.q_seq[t], 0, a.B - 1);
  const int L = a.len ? clampi(a.len[t], 0, a.topk) : a.topk;
  const int slot1 = min(L, slot0 + a.per_split);
  const uint8_t* kvseq = reinterpret_cast<const uint8_t*>(a.kv) + (size_t)b * a.max_ctx * kRow;
  const float* scseq = a.kv_scale + (size_t)b * a.max_ctx * kBlocks;

  float m_run = kNoMax, l_run = 0.f;
  float4v oacc[MD];
#pragma unroll
  for (int md = 0; md < MD; ++md) oacc[md] = float4v{0.f, 0.f, 0.f, 0.f};

  // Wave w gathers rows WROWS*w.. of tile tau: their chunks and scales are contiguous in the slot,
  // and lane l of a load lands at 16*l (4*l) bytes from the load's base.
  auto issue = [&](Slot& s, int tau) {
    const int* tr = rows + kTileK * tau + WROWS * wave;
    // every row index first: the gathers are opaque to the compiler, which keeps LDS reads after them
    int rc[C::WCHI], rs[C::WSCI];
#pragma unroll
    for (int j = 0; j < C::WCHI; ++j) {
      const int i = 64 * j + lane;
      rc[j] = max(tr[i < C::WCH ? i / CHUNKS : 0], 0);
    }
#pragma unroll
    for (int j = 0; j < C::WSCI; ++j) {
      const int i = 64 * j + lane;
      rs[j] = max(tr[i < C::WSC ? i / NSC : 0], 0);
    }
#pragma unroll
    for (int j = 0; j < C::WCHI; ++j) {
      const int i = 64 * j + lane;
      if (i < C::WCH)
        gather16_to_lds(kvseq + (size_t)rc[j] * kRow + 16 * (i % CHUNKS), s.raw + WROWS * wave * DQ + 1024 * j);
    }
#pragma unroll
    for (int j = 0; j < C::WSCI; ++j) {
      const int i = 64 * j + lane;
      if (i < C::WSC)
        gather4_to_lds(scseq + (size_t)rs[j] * kBlocks + i % NSC, s.sc + WROWS * wave * NSC + 64 * j);
    }
  };

  // fp8 tile -> bf16 key-major tile (code * scale, nearest even); the same share for every thread:
  // FULL 16-byte chunks, then one 4-byte quarter of the rest.
  auto dequant = [&](const Slot& s, KsTile& ks) {
#pragma unroll
    for (int m = 0; m < C::FULL; ++m) {
      const int ch = tid + kMlaThreads * m;
      const int r = ch / CHUNKS, cc = ch % CHUNKS;
      const u32x4 v = *reinterpret_cast<const u32x4*>(s.raw + 16 * ch);
      u32x4 lo, hi;
      dequant16(v, s.sc[r * NSC + (cc >> 2)], lo, hi);
      u32x4* dst = reinterpret_cast<u32x4*>(&ks[ks_row_of_key(r)][16 * cc]);
      dst[0] = lo;
      dst[1] = hi;
    }
    if (C::REM > 0 && tid < 4 * C::REM) {
      const int ch = C::FULL * kMlaThreads + (tid >> 2), qd = tid & 3;
      const int r = ch / CHUNKS, cc = ch % CHUNKS;
      const uint32_t v = *reinterpret_cast<const uint32_t*>(s.raw + 16 * ch + 4 * qd);
      const float sc = s.sc[r * NSC + (cc >> 2)];
      const float2v lo = __builtin_amdgcn_cvt_pk_f32_fp8(v, false) * sc;
      const float2v hi = __builtin_amdgcn_cvt_pk_f32_fp8(v, true) * sc;
      *reinterpret_cast<uint2*>(&ks[ks_row_of_key(r)][16 * cc + 4 * qd]) = make_uint2(cvt2_bf16(lo), cvt2_bf16(hi));
    }
  };

  // partial S^T over this half's query dims: lane (c, g) gets keys 8g + 4mb + i of head c
  auto qk = [&](const KsTile& ks, float4v* sacc) {
    constexpr int KB = 3;   // K operands read a batch ahead of their MFMAs
#pragma unroll
    for (int s0 = 0; s0 < KH; s0 += KB) {
      bf16x8 kop[2][KB];
#pragma unroll
      for (int j = 0; j < KB; ++j)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
          if (s0 + j < KH)
            kop[mb][j] = __builtin_bit_cast(
                bf16x8, *reinterpret_cast<const u32x4*>(&ks[16 * mb + c][32 * (KH * half + s0 + j) + 8 * g]));
#pragma unroll
      for (int j = 0; j < KB; ++j)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
          if (s0 + j < KH) sacc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[mb][j], qreg[s0 + j], sacc[mb], 0, 0, 0);
    }
  };

  // online softmax of tile tau's scores and O^T += V^T P^T
  auto attend = [&](const KsTile& ks, const float4v* sacc, uint32_t vmask) {
    float z[8];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const float4v other = xz[half ^ 1][hg][mb][lane];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float dot = sacc[mb][i] + other[i];   // the same sum in both halves (addition commutes)
        z[4 * mb + i] = ((vmask >> (4 * mb + i)) & 1u) ? dot * zscale : -INFINITY;
      }
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; ++e) tmax = fmaxf(tmax, z[e]);
    tmax = max_xor16(tmax);
    tmax = max_xor32(tmax);
    // Lazy rescaling: the reference maximum m_run only moves when the tile's maximum exceeds it by
    // more than 2^kLazyLog2 (or on the first keys), so probabilities stay below 2^kLazyLog2 and the
    // accumulators are rescaled rarely instead of on every tile.  O and l share m_run, so the
    // normalised result is the same softmax.  Before the first valid key m_run is kNoMax (finite),
    // so every exponent below is a plain hardware exp2 of a non-NaN argument.
    const bool bump = tmax > m_run + kLazyLog2;
    if (__ballot(bump)) {
      const float m_new = bump ? tmax : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);   // 0 when m_run is kNoMax
      l_run *= alpha;
      if (__ballot(bump && m_run != kNoMax)) {   // the accumulators hold keys to rescale
#pragma unroll
        for (int md = 0; md < MD; ++md) oacc[md] *= alpha;
      }
      m_run = m_new;
    }
    float p[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) p[e] = __builtin_amdgcn_exp2f(z[e] - m_run);
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) psum += p[e];
    l_run += psum;
    u32x4 pk;
#pragma unroll
    for (int e = 0; e < 4; ++e) pk[e] = cvt2_bf16(float2v{p[2 * e], p[2 * e + 1]});
    const bf16x8 pop = __builtin_bit_cast(bf16x8, pk);
    // V^T operand rows: LDS rows 16h + 4g + j/4 hold keys 8g + 4h + j/4
    const int trow = 4 * g + (c >> 2), tcol = 4 * (c & 3) + C::ODIM * half;
    typedef __attribute__((address_space(3))) short4v* lds_s4p;
    constexpr int VB = 4;   // V^T operands read a batch ahead of their MFMAs
#pragma unroll
    for (int md0 = 0; md0 < MD; md0 += VB) {
      short8v vv[VB];
#pragma unroll
      for (int j = 0; j < VB; ++j) {
        const short4v v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4p)(&ks[trow][16 * (md0 + j) + tcol]));
        const short4v v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4p)(&ks[16 + trow][16 * (md0 + j) + tcol]));
        vv[j] = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
      }
#pragma unroll
      for (int j = 0; j < VB; ++j)
        oacc[md0 + j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vv[j]), pop, oacc[md0 + j], 0, 0, 0);
    }
  };

  // One tile; KBC selects the bf16 buffer of tile tau (the other one receives tile tau+1), st is
  // tile tau's slot.
  auto step = [&](auto KBC, int tau, int ntiles, int st) {
    KsTile& kcur = decltype(KBC)::value ? ks1 : ks0;
    KsTile& knext = decltype(KBC)::value ? ks0 : ks1;
    if (tau + 2 < ntiles) wait_vmcnt<LPT>();   // tile tau+1's gathers are done, tile tau+2's may not be
    else wait_vmcnt<0>();
    lds_barrier();
    if (tau + 3 < ntiles) issue(sl[st], tau + 3);
    // validity of this lane's 8 keys (8g + e) of tile tau
    uint32_t vmask = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) vmask |= (rows[kTileK * tau + 8 * g + e] >= 0 ? 1u : 0u) << e;
    float4v sacc[2] = {float4v{0.f, 0.f, 0.f, 0.f}, float4v{0.f, 0.f, 0.f, 0.f}};
    qk(kcur, sacc);
    // the next tile (after the last one: stale slot contents into a buffer nobody reads)
    dequant(sl[st == kSlots - 1 ? 0 : st + 1], knext);
    xz[half][hg][0][lane] = sacc[0];
    xz[half][hg][1][lane] = sacc[1];
    lds_barrier();                         // both halves' partial scores are in LDS
    if (active) attend(kcur, sacc, vmask);
  };

  for (int cb = slot0; cb < slot1; cb += kRowsChunk) {   // chunks of the split's slots (one, normally)
    if (cb != slot0) load_rows(cb);
    const int nslot = min(kRowsChunk, slot1 - cb);
    const int ntiles = (nslot + kTileK - 1) / kTileK;
    __syncthreads();                       // the previous chunk is completely consumed
#pragma unroll
    for (int u = 0; u < RPT; ++u) {
      const int i = tid + kMlaThreads * u;
      if (i < ntiles * kTileK) rows[i] = (i < nslot && rv[u] >= 0 && rv[u] < a.max_ctx) ? rv[u] : -1;
    }
    __syncthreads();
    wait_vmcnt<0>();   // the query loads are done (tells the compiler too: no waits for them below)
    issue(sl[0], 0);
    if (1 < ntiles) issue(sl[1], 1);
    if (2 < ntiles) issue(sl[2], 2);
    if (ntiles > 2) wait_vmcnt<2 * LPT>();
    else if (ntiles > 1) wait_vmcnt<LPT>();
    else wait_vmcnt<0>();
    lds_barrier();                         // tile 0 is in its slot
    dequant(sl[0], ks0);
    int st = 0;
    for (int tau = 0; tau < ntiles; tau += 2) {
      step(IntC<0>(), tau, ntiles, st);
      st = st == kSlots - 1 ? 0 : st + 1;
      if (tau + 1 < ntiles) {
        step(IntC<1>(), tau + 1, ntiles, st);
        st = st == kSlots - 1 ? 0 : st + 1;
      }
    }
  }
  if (!active) return;
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  // oacc[md][i] = O^T[dim ODIM*half + 16md + 4g + i][head c]
  if (a.splits > 1 && bf16_partials(a)) {
    // bf16 split partials leave through LDS so that every store covers whole lines: this wave's
    // 16 heads x 256 dims in two rounds of 8 heads, each head row then stored as 32 lanes x 16
    // contiguous bytes, non-temporally (the partials stream out during the kernel instead of being
    // written back from L2 when it ends).  The raw slots are free: every wave has passed the last
    // tile's second barrier, after which no gather or dequantisation touches them.  No branch
    // depends on the lane: in each round the lanes of the other round's heads write a discard row
    // (row 8), and a wave barrier keeps the round's writes before its reads.
    constexpr int kStageRow = 2 * C::ODIM + 16;            // bytes per staged head row (padded)
    constexpr int kStageWords = kStageRow / 4;
    static_assert(8 * 9 * kStageRow <= (int)sizeof(sl), "staging space");
    uint32_t* stage = static_cast<uint32_t*>(__builtin_assume_aligned(
        reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(&sl[0]) + wave * 9 * kStageRow), 16));
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const size_t hstride = (size_t)a.splits * a.kv_lora;   // bf16 between consecutive heads' partials
    uint16_t* dst0 = reinterpret_cast<uint16_t*>(a.ws) + (((size_t)t * a.H + 16 * hg) * a.splits + split) * a.kv_lora +
                     C::ODIM * half;
#pragma unroll
    for (int ph = 0; ph < 2; ++ph) {
      const int wrow = (c >> 3) == ph ? (c & 7) : 8;
#pragma unroll
      for (int md = 0; md < MD; ++md) {
        uint32_t* w = stage + wrow * kStageWords + (16 * md + 4 * g) / 2;
        w[0] = cvt2_bf16(float2v{oacc[md][0] * inv, oacc[md][1] * inv});
        w[1] = cvt2_bf16(float2v{oacc[md][2] * inv, oacc[md][3] * inv});
      }
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int row = 2 * k + (lane >> 5), ch = lane & 31;
        const uint32_t* r = stage + row * kStageWords + 4 * ch;
        const u32x4 v = {r[0], r[1], r[2], r[3]};
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dst0 + (size_t)(8 * ph + row) * hstride + 8 * ch));
      }
      __builtin_amdgcn_wave_barrier();
    }
  } else {
#pragma unroll
    for (int md = 0; md < MD; ++md) {
      float o[4] = {oacc[md][0], oacc[md][1], oacc[md][2], oacc[md][3]};
      write_partial_or_final(a, t, split, head, m_run, l_tot, o, C::ODIM * half + 16 * md + 4 * g, 4);
    }
  }
  if (g == 0 && half == 0) write_stats(a, t, split, head, m_run, l_tot);
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
// One wave per (query, head), 8 of the 512 output dims per lane.  The first batch of partials is
// loaded before the split statistics are reduced, so both sets of loads are in flight together;
// split s's weight is then read from lane s.
constexpr int kCombineHeads = 4;                      // waves (heads) per workgroup
constexpr int kCombineThreads = 64 * kCombineHeads;

// Maximum and sum over the 64 lanes of a wave with DPP moves (no LDS round trips): row shifts by
// 1, 2, 4 and 8 lanes, then row broadcasts of lanes 15 and 31, leave the result in lane 63, which
// is read into a scalar.
__device__ __forceinline__ float wave_max(float x) {
  int v = __builtin_bit_cast(int, x);
  auto step = [&](auto CTRL, auto RMASK) {
    const int o = __builtin_amdgcn_update_dpp(v, v, decltype(CTRL)::value, decltype(RMASK)::value, 0xf, false);
    v = __builtin_bit_cast(int, fmaxf(__builtin_bit_cast(float, v), __builtin_bit_cast(float, o)));
  };
  step(IntC<0x111>(), IntC<0xf>());   // row_shr:1 (lanes without a source keep their own value)
  step(IntC<0x112>(), IntC<0xf>());   // row_shr:2
  step(IntC<0x114>(), IntC<0xf>());   // row_shr:4
  step(IntC<0x118>(), IntC<0xf>());   // row_shr:8
  step(IntC<0x142>(), IntC<0xa>());   // row_bcast:15 into rows 1 and 3
  step(IntC<0x143>(), IntC<0xc>());   // row_bcast:31 into rows 2 and 3
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(v, 63));
}
__device__ __forceinline__ float wave_sum(float x) {
  auto step = [&](auto CTRL, auto RMASK) {
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), decltype(CTRL)::value,
                                                               decltype(RMASK)::value, 0xf, true));
  };
  step(IntC<0x111>(), IntC<0xf>());   // row_shr:1 (lanes without a source add 0)
  step(IntC<0x112>(), IntC<0xf>());
  step(IntC<0x114>(), IntC<0xf>());
  step(IntC<0x118>(), IntC<0xf>());
  step(IntC<0x142>(), IntC<0xa>());
  step(IntC<0x143>(), IntC<0xc>());
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}

template <bool BF16>
__global__ void __launch_bounds__(kCombineThreads) k_mla_combine(MlaLaunch a) {
  constexpr int SB = BF16 ? 16 : 8;                   // splits per batch of loads
  constexpr int NV = BF16 ? 1 : 2;                    // 16-byte loads per split and lane
  int t, hq;
  if (!xcd_query_map((a.H + kCombineHeads - 1) / kCombineHeads, a.T, &t, &hq)) return;
  const int lane = threadIdx.x & 63;
  const int h = hq * kCombineHeads + (threadIdx.x >> 6);
  if (h >= a.H) return;                               // whole waves; the kernel has no barriers
  const float* stats = a.ws + (size_t)a.T * a.splits * a.H * a.kv_lora;
  const size_t base = ((size_t)t * a.H + h) * a.splits * a.kv_lora + 8 * lane;   // split 0, this lane's dims
  const size_t sstride = (size_t)a.kv_lora;                                      // elements between splits
  // split statistics: lane s holds split s (splits <= 64)
  float m = -INFINITY, l = 0.f;
  if (lane < a.splits) {
    const size_t i = ((size_t)t * a.H + h) * a.splits + lane;
    m = stats[2 * i];
    l = stats[2 * i + 1];
  }
  // A batch of SB splits: every load is unconditional (split indices past the end are clamped to
  // the last split, whose weight below is then 0 for them), so the whole batch is in flight at
  // once; the values are decoded where they are used.
  u32x4 raw[SB][NV];
  auto load = [&](int s0) {
#pragma unroll
    for (int j = 0; j < SB; ++j) {
      const size_t off = base + (size_t)min(s0 + j, a.splits - 1) * sstride;
      if (BF16) {
        raw[j][0] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(a.ws) + off);
      } else {
        raw[j][0] = *reinterpret_cast<const u32x4*>(a.ws + off);
        raw[j][NV - 1] = *reinterpret_cast<const u32x4*>(a.ws + off + 4);
      }
    }
  };
  auto value = [&](int j, int e) -> float {
    if (BF16) {
      const uint32_t w2 = raw[j][0][e >> 1];
      return __uint_as_float((e & 1) ? (w2 & 0xFFFF0000u) : (w2 << 16));
    }
    return __uint_as_float(raw[j][e >> 2][e & 3]);
  };
  load(0);
  const float M = wave_max(m);
  const float w = (M == -INFINITY || lane >= a.splits) ? 0.f : exp2f(m - M);
  const float Ls = wave_sum(w * l);
  // normalised (bf16) partials carry their own sum l
  const float wt = Ls > 0.f ? (BF16 ? w * l : w) / Ls : 0.f;
  if (lane == 0 && a.lse) a.lse[(size_t)t * a.H + h] = Ls > 0.f ? (M + log2f(Ls)) * kLn2 : -INFINITY;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < a.splits; s0 += SB) {
    if (s0 > 0) load(s0);
#pragma unroll
    for (int j = 0; j < SB; ++j) {
      const float wj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wt), min(s0 + j, 63)));
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(wj, value(j, e), acc[e]);
    }
  }
  float* outp = a.out + ((size_t)t * a.H + h) * a.kv_lora + 8 * lane;
  *reinterpret_cast<float4*>(outp) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  *reinterpret_cast<float4*>(outp + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
}

}  // namespace

hipError_t launch_sparse_mla(const MlaLaunch& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  dim3 grid(a.splits, a.T);
  if (a.kv_dtype == DSA_FP8_E4M3FN) {
    const dim3 xgrid(xcd_grid(a.splits, a.T));
    if (a.rope_dim == 64) hipLaunchKernelGGL(k_mla_fp8<64>, xgrid, dim3(kMlaThreads), 0, s, a);
    else hipLaunchKernelGGL(k_mla_fp8<0>, xgrid, dim3(kMlaThreads), 0, s, a);
  } else {
    if (a.rope_dim == 64) hipLaunchKernelGGL(k_mla_f32<64>, grid, dim3(kF32Threads), 0, s, a);
    else hipLaunchKernelGGL(k_mla_f32<0>, grid, dim3(kF32Threads), 0, s, a);
  }
  if (a.splits > 1) {
    const dim3 cgrid(xcd_grid((a.H + kCombineHeads - 1) / kCombineHeads, a.T));
    if (a.kv_dtype == DSA_FP8_E4M3FN) hipLaunchKernelGGL(k_mla_combine<true>, cgrid, dim3(kCombineThreads), 0, s, a);
    else hipLaunchKernelGGL(k_mla_combine<false>, cgrid, dim3(kCombineThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace dsa
