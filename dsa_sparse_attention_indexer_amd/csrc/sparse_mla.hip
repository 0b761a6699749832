// Sparse absorbed-MLA attention on gfx950: exact softmax attention of every head over the keys
// the indexer selected ("Day 0 support for Mistral Large 4 on vLLM": MLA with KV LoRA rank 512
// and RoPE dim 64, one latent KV head shared by all 64 heads, V = the latent; NoPE layers are
// the same with zero RoPE dims on the same cache layout).
//
// fp8 cache, bf16 query (matrix-core path): see the wave-specialised kernel k_mla_fp8_ws below
// (8 waves per workgroup: 4 for the logits and softmax, 4 for P.V; fp8 codes converted exactly to
// bf16 in registers, the fp32 block scales applied in fp32).
// fp32 cache, fp32 query: 16-key tiles with fp32 vector FMAs (8 lanes per head).
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

constexpr int kRow = 576;                 // latent row: 512 + 64
constexpr int kLora = 512;
constexpr int kBlocks = kRow / 64;        // scales per row
constexpr int kRowsChunk = 2048;          // selection slots staged in LDS at a time (fp8 path)
constexpr float kLazyLog2 = 8.f;          // the running maximum lags the true one by at most this (log2)
constexpr float kNoMax = -1.0e30f;        // running maximum before the first valid key (fp8 path)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

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

typedef __attribute__((address_space(3))) void* lds_void_ptr;

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding: vmcnt in bits 3:0 and
// 15:14, expcnt in 6:4 and lgkmcnt in 11:8 left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt out of range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Maximum over lanes l and l ^ 32 (v_permlane32_swap), without the address arithmetic of a bpermute
// shuffle.
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

// Workgroups are dispatched to the 8 XCDs round-robin by linear id.  Queries are taken in groups of
// G consecutive ones (G = T / B when every sequence has the same 2..8 queries, as in multi-token
// decode where consecutive queries are one sequence's verify block; else 1), and a 1-D grid of
// 8 * inner * G * ceil(T / 8G) workgroups is mapped so that every workgroup of group q runs on XCD
// q % 8, the G queries' workgroups for the same inner index next to each other in dispatch order.
// The splits of a query share one L2 for the query and the row indices, the combine that reads
// their partials runs on the XCD whose L2 they were written to, and the tokens of one verify block
// gather their (largely common) latent rows through one L2 at about the same time.  Returns false
// for the padding.
__host__ __device__ inline int mla_group(int T, int B) {
  return (B > 0 && T % B == 0 && T / B >= 2 && T / B <= 8) ? T / B : 1;
}
__device__ __forceinline__ bool xcd_query_map(int inner, int T, int G, int* t, int* j) {
  const int id = blockIdx.x, x = id & 7, r = id >> 3;
  const int per = inner * G;
  const int rem = r % per;
  *j = rem / G;
  *t = G * (8 * (r / per) + x) + rem % G;
  return *t < T;
}
inline unsigned xcd_grid(int inner, int T, int G) { return (unsigned)(8 * inner * G * ((T + 8 * G - 1) / (8 * G))); }

constexpr int kMlaThreads = 512;   // fp8 path: 8 waves

template <int V>
struct IntC {
  static constexpr int value = V;
};

// ---------------------------------------------------------------------------------------------
// fp8 cache, bf16 query: wave-specialised kernel on v_mfma_f32_32x32x16_bf16
//
// One workgroup of 8 waves per (query, split); 64-key tiles.  The fp8 rows and their scales are
// gathered into a ring of three LDS slots and never dequantised as a whole: every fp8 code is
// converted exactly to bf16 in registers (v_cvt_scalef32_pk_bf16_fp8 with unit scale), and the
// per-(key, 64-element block) fp32 scales are applied in fp32:
//   * QK waves 0..3, wave = (head group hg of 32 heads, key half kg of 32 keys): S^T[32 keys x 32
//     heads] block by block -- for each 64-dim block an accumulator of 4 MFMAs (K codes as A, the
//     bf16 query as B, held in registers), then S^T += scale(key, block) * block accumulator.
//     The logits are exact up to fp32 accumulation.  Online softmax (lazy rescale) per head with the
//     other key half's maximum exchanged through LDS; P (fp32) goes to LDS in the lane order of the
//     PV operand.
//   * PV waves 4..7, wave = 128 output dims of all 64 heads: O^T[128 dims x 64 heads] +=
//     V^T . (P scale(key, block))^T, V^T read from the fp8 slot with ds_read_b64_tr_b8 (8 keys of one
//     dim per lane) and converted exactly; the V scales are folded into the bf16 P operand.
//     The PV waves also issue the gathers.
// Each SIMD holds one QK and one PV wave, so one wave's matrix work overlaps the other's vector
// work.  Tile tau: phase A -- QK(tau) || PV(tau-1) and the gathers of tile tau+2; phase B --
// softmax(tau) || the PV waves read tile tau's V bytes into registers (its slot is then free).
// Within a 32-key half, tile key kappa sits in LDS row lrow(kappa) (bits 2 and 3 swapped), so that
// the rows behind a QK lane's accumulator run in key order and the P values of a lane are the 8
// consecutive keys the PV operand needs.
// ---------------------------------------------------------------------------------------------

typedef float float16v __attribute__((ext_vector_type(16)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2* lds_i2p;

constexpr int kT2 = 64;        // keys per tile
constexpr int kS2 = 3;         // raw tiles in LDS

__device__ __forceinline__ int perm23(int x) { return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1); }
__device__ __forceinline__ int lrow(int k) { return (k & ~31) | perm23(k & 31); }   // an involution

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer descriptor words over `bytes` bytes from `base` (loads past the end read zero).
__device__ __forceinline__ i32x4 buffer_words(const void* base, uint32_t bytes) {
  const uint64_t p = (uint64_t)(uintptr_t)base;
  return i32x4{__builtin_amdgcn_readfirstlane((int)(uint32_t)p), __builtin_amdgcn_readfirstlane((int)(uint32_t)(p >> 32) & 0xFFFF),
               __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000};
}
// Gathers through a buffer descriptor straight into LDS: lane l's 16 (4) bytes at byte voff of the
// buffer land at LDS byte lds + 16*l (4*l).  One 32-bit offset per lane; waited for with vmcnt.
__device__ __forceinline__ void bgather16(i32x4 rs, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rs), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void bgather4(i32x4 rs, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dword %0, %1, 0 offen lds" ::"v"(voff), "s"(rs), "s"(lds) : "memory", "m0");
}

// Slot layout.  Codes: [row group i = R/16][64-byte segment j][16 rows][4 chunks of 16 bytes], the
// chunks of a segment rotated by row (swz) so that 16 consecutive rows reading the same chunk, and
// the 8 rows of a transposing read, hit different banks.  PV wave pw gathers row group pw: one
// 64-lane load per segment, four lanes per row, every load of a lane from the same cache row.
// Scales: [row group][block][16 keys] (by tile key, not LDS row).
__device__ __forceinline__ int swz(int m16) { return ((m16 >> 1) + (m16 >> 3)) & 3; }

template <int ROPE>
struct M2 {
  static constexpr int DQ = kLora + ROPE;        // used bytes of a latent row
  static constexpr int NB = DQ / 64;             // scale blocks used
  static constexpr int NJ = DQ / 64;             // 64-byte segments per row
  static constexpr int CODES = kT2 * DQ;
  static constexpr int SLOT = CODES + NB * kT2 * 4;
  static constexpr int NP = DQ / 32;             // 32-dim pairs of K-steps
  static constexpr int NSC = (NB + 3) / 4;       // scale loads per PV wave and tile
  static constexpr int LPT = NJ + NSC;           // LDS-direct loads per PV wave and tile
  // byte offset of 16-byte chunk c of LDS row R
  static __device__ __forceinline__ int pos(int R, int c) {
    return (((R >> 4) * NJ + (c >> 2)) * 16 + (R & 15)) * 64 + 16 * ((c & 3) ^ swz(R & 15));
  }
};

// 8 fp8 codes (two dwords) -> 8 bf16, exact
__device__ __forceinline__ bf16x8 codes_bf16(uint32_t lo, uint32_t hi) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

template <int ROPE>
struct Mla2Smem {
  using C = M2<ROPE>;
  uint8_t slot[kS2][C::SLOT];          // codes [64 LDS rows][RS], then scales [NB][64 keys]
  float pbuf[2][4][64][8];             // P of the current tile: [head tile][K-step][lane][8 keys]
  float scl[4][2][64];                 // per PV wave: V scales of its two blocks, current tile
  int rows[kRowsChunk];                // cache row of every slot of the chunk, -1 if none
  float xmax[2][2][32];                // QK: per (head group, key half) tile maxima
  float alpha[64];                     // rescale factor of the tile, per head
  float lsum[2][2][32];                // epilogue: softmax sums per (head group, key half)
  int flags[2];                        // per head group: the tile moved the running maximum
};

// NHT: head tiles of 32 (2 for up to 64 heads, 1 for up to 32: the P.V waves then do half the work)
template <int ROPE, int NHT>
__global__ void __launch_bounds__(kMlaThreads)
k_mla_fp8_ws(MlaLaunch a) {
  using C = M2<ROPE>;
  int t, split;
  if (!xcd_query_map(a.splits, a.T, mla_group(a.T, a.B), &t, &split)) return;
  __shared__ __attribute__((aligned(16))) Mla2Smem<ROPE> sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int slot0 = split * a.per_split;
  const int tr = t / a.hs;                               // the real query (head split)
  const int32_t* irow = a.idx + (size_t)tr * a.topk;
  const int slot_end = min(slot0 + a.per_split, a.topk);
  // The row indices are loaded and staged by the PV waves alone, so that the first gathers (which
  // need them) do not wait behind the QK waves' query loads.
  constexpr int kPvThreads = kMlaThreads / 2;
  constexpr int RPT = kRowsChunk / kPvThreads;
  const int ptid = tid - kPvThreads;                     // PV thread index (PV waves only)
  int rv[RPT];
  auto load_rows = [&](int cb) {   // unconditional loads (slot clamped into the row): all in flight together
#pragma unroll
    for (int u = 0; u < RPT; ++u) rv[u] = irow[min(cb + ptid + kPvThreads * u, a.topk - 1)];
#pragma unroll
    for (int u = 0; u < RPT; ++u) rv[u] = cb + ptid + kPvThreads * u < slot_end ? rv[u] : -1;
  };
  constexpr int nht = NHT;                               // head tiles of 32
  const int b = clampi(a.q_seq[tr], 0, a.B - 1);
  const int L = a.len ? clampi(a.len[tr], 0, a.topk) : a.topk;
  const int slot1 = min(L, slot0 + a.per_split);
  // contiguous caches: the query's sequence; paged: the whole pool (rows are pool slots)
  const bool paged = a.pg.table != nullptr;
  const uint8_t* kvseq = reinterpret_cast<const uint8_t*>(a.kv) + (paged ? 0 : (size_t)b * a.max_ctx * kRow);
  const float* scseq = a.kv_scale + (paged ? 0 : (size_t)b * a.max_ctx * kBlocks);
  const int64_t seq_rows = paged ? a.pool_rows : a.max_ctx;
  const float zscale = a.softmax_scale * kLog2e;

  // the rows of chunk cb into LDS (PV waves; callers hold a barrier before and after): the cache
  // row of each selected position (its pool slot on a paged cache), -1 for none
  auto store_rows = [&](int nslot, int ntiles) {
    // The slot addresses come from a copy of the thread index made here: formed once and kept live
    // across the kernel they are spilled, and each reload then costs a scratch round trip.
    int pt;
    asm volatile("v_mov_b32 %0, %1" : "=v"(pt) : "v"(ptid));
    int* rp = sm.rows + pt;
#pragma unroll
    for (int u = 0; u < RPT; ++u) {
      const int i = ptid + kPvThreads * u;
      const bool ok = i < nslot && rv[u] >= 0 && rv[u] < a.max_ctx;
      if (i < ntiles * kT2) rp[kPvThreads * u] = ok ? (paged ? (int)paged_slot(a.pg, b, rv[u]) : rv[u]) : -1;
    }
  };

  if (wave < 4) {
    // ======================================= QK waves =======================================
    const int hg = wave & 1, kg = wave >> 1;
    const int m = lane & 31, h = lane >> 5;
    const int head = 32 * hg + m;
    const bool active = 32 * hg < a.H;
    bf16x8 qreg[2 * C::NP];                              // K-step (p, e): dims 32p + 16h + 8e + 0..7
#pragma unroll
    for (int s = 0; s < 2 * C::NP; ++s) qreg[s] = bf16x8{};
    if (active && head < a.H) {
      const uint16_t* qh = reinterpret_cast<const uint16_t*>(a.q) + ((size_t)t * a.H + head) * C::DQ + 16 * h;
#pragma unroll
      for (int p = 0; p < C::NP; ++p) {
        qreg[2 * p] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qh + 32 * p));
        qreg[2 * p + 1] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qh + 32 * p + 8));
      }
    }
    float m_run = kNoMax, l_run = 0.f;
    for (int cb = slot0; cb < slot1; cb += kRowsChunk) {
      const int nslot = min(kRowsChunk, slot1 - cb);
      const int ntiles = (nslot + kT2 - 1) / kT2;
      lds_barrier();                                     // R: the chunk's rows are in LDS
      for (int tau = 0; tau < ntiles; ++tau) {
        lds_barrier();                                   // A: tile tau is in its slot
        const uint8_t* codes = sm.slot[tau % kS2];
        const float* scs = reinterpret_cast<const float*>(codes + C::CODES);
        // validity of this lane's 16 keys: 32kg + 16(r/8) + 8h + r%8
        const uint64_t vmask = __ballot(sm.rows[kT2 * tau + lane] >= 0);
        const uint32_t vbits = (uint32_t)((vmask >> (32 * kg + 8 * h)) & 0xFFull) |
                               ((uint32_t)((vmask >> (32 * kg + 16 + 8 * h)) & 0xFFull) << 8);
        float16v S = {};
        if (active) {
#pragma unroll
          for (int bl = 0; bl < C::NB; ++bl) {
            float16v ab = {};
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) {
              const int p = 2 * bl + pp;                 // dims 32p + 16h .. + 15: chunk 2p + h
              const u32x4 raw = *reinterpret_cast<const u32x4*>(codes + C::pos(32 * kg + m, 2 * p + h));
              ab = __builtin_amdgcn_mfma_f32_32x32x16_bf16(codes_bf16(raw[0], raw[1]), qreg[2 * p], ab, 0, 0, 0);
              ab = __builtin_amdgcn_mfma_f32_32x32x16_bf16(codes_bf16(raw[2], raw[3]), qreg[2 * p + 1], ab, 0, 0, 0);
            }
            const float* sb0 = scs + ((2 * kg) * C::NB + bl) * 16 + 8 * h;       // keys 32kg + 8h + 0..7
            const float* sb1 = scs + ((2 * kg + 1) * C::NB + bl) * 16 + 8 * h;   // keys 32kg + 16 + 8h + 0..7
            const float4 s0 = *reinterpret_cast<const float4*>(sb0);
            const float4 s1 = *reinterpret_cast<const float4*>(sb0 + 4);
            const float4 s2 = *reinterpret_cast<const float4*>(sb1);
            const float4 s3 = *reinterpret_cast<const float4*>(sb1 + 4);
            const float sv[16] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w,
                                  s2.x, s2.y, s2.z, s2.w, s3.x, s3.y, s3.z, s3.w};
#pragma unroll
            for (int r = 0; r < 16; ++r) S[r] = fmaf(sv[r], ab[r], S[r]);
          }
        }
        float z[16];
        float tmax = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          z[r] = ((vbits >> r) & 1u) ? S[r] * zscale : -INFINITY;
          tmax = fmaxf(tmax, z[r]);
        }
        tmax = max_xor32(tmax);                          // this key half's 32 keys, per head
        if (lane < 32) sm.xmax[hg][kg][m] = tmax;
        lds_barrier();                                   // B: both key halves' maxima are in LDS
        if (active) {
          const float t64 = fmaxf(tmax, sm.xmax[hg][kg ^ 1][m]);
          // lazy rescale: the reference maximum m_run only moves when the tile's maximum exceeds it
          // by more than 2^kLazyLog2 (or on the first keys), so probabilities stay below 2^kLazyLog2
          // and the accumulators are rescaled rarely; O and l share m_run, so the normalised result
          // is the same softmax.  Both key halves take the same decision from the same maxima.
          const bool bump = t64 > m_run + kLazyLog2;
          const uint64_t any = __ballot(bump);
          if (any) {
            const float m_new = bump ? t64 : m_run;
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            l_run *= alpha;
            m_run = m_new;
            if (kg == 0 && lane < 32) sm.alpha[head] = alpha;
          }
          if (kg == 0 && lane == 0) sm.flags[hg] = any != 0;
          float p[16];
          float psum = 0.f;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            p[r] = __builtin_amdgcn_exp2f(z[r] - m_run);
            psum += p[r];
          }
          l_run += psum;
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            float* dst = &sm.pbuf[hg][2 * kg + j][lane][0];
            *reinterpret_cast<float4*>(dst) = make_float4(p[8 * j], p[8 * j + 1], p[8 * j + 2], p[8 * j + 3]);
            *reinterpret_cast<float4*>(dst + 4) = make_float4(p[8 * j + 4], p[8 * j + 5], p[8 * j + 6], p[8 * j + 7]);
          }
        }
      }
      lds_barrier();                                     // F: the chunk's last P is in LDS
    }
    // epilogue: softmax sums per head (both lane halves, then both key halves)
    const float l_half = l_run + __shfl_xor(l_run, 32);
    if (lane < 32) sm.lsum[hg][kg][m] = l_half;
    lds_barrier();                                       // G
    if (active && kg == 0 && lane < 32 && head < a.H) {
      const float l_tot = sm.lsum[hg][0][m] + sm.lsum[hg][1][m];
      write_stats(a, t, split, head, m_run, l_tot);
    }
  } else {
    // ======================================= PV waves =======================================
    const int pw = wave - 4;                             // output dims 128pw .. 128pw + 127
    const int c16 = lane & 15, g16 = lane >> 4, h = lane >> 5;
    float16v O[NHT][4];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) O[ht][dt] = float16v{};
    i32x2 vraw[4][4];                                    // V^T bytes of the tile: [K-step J][dim tile]

    // This wave's gathers of tile tau: LDS rows 16pw .. 16pw + 15, one load per 64-byte segment
    // (lane: row 16pw + lane/4, chunk lane%4 of the segment, rotated by swz) and the scales of the
    // same 16 keys.  The latent rows and scales of the query's sequence are addressed through
    // buffer descriptors (32-bit offsets: the host checks that a sequence's rows, or a paged pool, span less than
    // 4 GiB).  Both row indices are read before the first load goes out.
    const i32x4 kv_rs = buffer_words(kvseq, (uint32_t)((uint64_t)seq_rows * kRow));
    const i32x4 sc_rs = buffer_words(scseq, (uint32_t)((uint64_t)seq_rows * kBlocks * 4));
    const uint32_t lds_slots = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_ptr)&sm.slot[0][0]);
    const int g_row = lrow(16 * pw + (lane >> 2));           // tile key in LDS row 16pw + lane/4
    const int g_chunk = (lane & 3) ^ swz(lane >> 2);          // its chunk within each segment
    auto issue = [&](int tau) {
      const uint32_t base = lds_slots + (uint32_t)(C::SLOT * (tau % kS2));
      const int* tr = sm.rows + kT2 * tau;
      const uint32_t rc = (uint32_t)max(tr[g_row], 0);
      const uint32_t rs = (uint32_t)max(tr[16 * pw + (lane & 15)], 0);
      const uint32_t voff = rc * kRow + 16 * g_chunk;
#pragma unroll
      for (int j = 0; j < C::NJ; ++j) bgather16(kv_rs, voff + 64 * j, base + 1024 * (pw * C::NJ + j));
#pragma unroll
      for (int k = 0; k < C::NSC; ++k) {
        const int bl = 4 * k + (lane >> 4);
        if (bl < C::NB) bgather4(sc_rs, (rs * kBlocks + bl) * 4, base + C::CODES + 64 * (pw * C::NB + 4 * k));
      }
    };
    // PV of the tile whose V bytes are in vraw (its P, scales and rescale factors in LDS)
    auto pv = [&]() {
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) {
        if (ht < nht && sm.flags[ht]) {
          const float al = sm.alpha[32 * ht + (lane & 31)];
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) O[ht][dt] *= al;
        }
      }
#pragma unroll
      for (int J = 0; J < 4; ++J) {
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) {
          const bf16x8 v0 = codes_bf16((uint32_t)vraw[J][2 * bb][0], (uint32_t)vraw[J][2 * bb][1]);
          const bf16x8 v1 = codes_bf16((uint32_t)vraw[J][2 * bb + 1][0], (uint32_t)vraw[J][2 * bb + 1][1]);
          const float* sp = &sm.scl[pw][bb][16 * J + 8 * h];
          const float4 s0 = *reinterpret_cast<const float4*>(sp);
          const float4 s1 = *reinterpret_cast<const float4*>(sp + 4);
          // every head tile of the workgroup (NHT), branch-free
#pragma unroll
          for (int ht = 0; ht < NHT; ++ht) {
            const float* pp = &sm.pbuf[ht][J][lane][0];
            const float4 p0 = *reinterpret_cast<const float4*>(pp);
            const float4 p1 = *reinterpret_cast<const float4*>(pp + 4);
            u32x4 pk;
            pk[0] = cvt2_bf16(float2v{p0.x * s0.x, p0.y * s0.y});
            pk[1] = cvt2_bf16(float2v{p0.z * s0.z, p0.w * s0.w});
            pk[2] = cvt2_bf16(float2v{p1.x * s1.x, p1.y * s1.y});
            pk[3] = cvt2_bf16(float2v{p1.z * s1.z, p1.w * s1.w});
            const bf16x8 pop = __builtin_bit_cast(bf16x8, pk);
            O[ht][2 * bb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v0, pop, O[ht][2 * bb], 0, 0, 0);
            O[ht][2 * bb + 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v1, pop, O[ht][2 * bb + 1], 0, 0, 0);
          }
        }
      }
    };
    // tile tau's V bytes (8 keys of one dim per lane) and this wave's V scales, out of its slot
    auto preload = [&](int tau) {
      const uint8_t* codes = sm.slot[tau % kS2];
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        const int R = lrow(16 * J + 8 * (g16 >> 1) + (c16 >> 1));
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {   // dims 128pw + 32dt + 16(g16&1) + 8(c16&1): chunk 8pw + 2dt + (g16&1)
          const uint8_t* src = codes + C::pos(R, 8 * pw + 2 * dt + (g16 & 1)) + 8 * (c16 & 1);
          vraw[J][dt] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i2p)(src));
        }
      }
      const float* scs = reinterpret_cast<const float*>(codes + C::CODES);
      sm.scl[pw][0][lane] = scs[((lane >> 4) * C::NB + 2 * pw) * 16 + (lane & 15)];
      sm.scl[pw][1][lane] = scs[((lane >> 4) * C::NB + 2 * pw + 1) * 16 + (lane & 15)];
    };

    load_rows(slot0);
    for (int cb = slot0; cb < slot1; cb += kRowsChunk) {
      if (cb != slot0) load_rows(cb);
      const int nslot = min(kRowsChunk, slot1 - cb);
      const int ntiles = (nslot + kT2 - 1) / kT2;
      store_rows(nslot, ntiles);
      lds_barrier();                                     // R
      issue(0);
      if (1 < ntiles) issue(1);
      for (int tau = 0; tau < ntiles; ++tau) {
        // tile tau has landed; tile tau + 1 (issued later) may still be in flight
        if (tau + 1 < ntiles) wait_vmcnt<C::LPT>();
        else wait_vmcnt<0>();
        lds_barrier();                                   // A
        if (tau >= 1) pv();
        // into the slot of tile tau - 1 (free: its V bytes were read in the last phase B); after the
        // PV, whose V registers are then dead
        if (tau + 2 < ntiles) issue(tau + 2);
        lds_barrier();                                   // B
        preload(tau);
      }
      lds_barrier();                                     // F: the last tile's P is in LDS
      if (ntiles > 0) pv();
    }
    lds_barrier();                                       // G: the softmax sums are in LDS
    // normalise and store: lane (head 32ht + lane%32, half h) holds, for dim tile dt, dims
    // 128pw + 32dt + 8A + 4h + 0..3 in registers 4A..4A+3
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      const int head = 32 * ht + (lane & 31);
      if (ht >= nht || head >= a.H) continue;
      const float l_tot = sm.lsum[ht][0][lane & 31] + sm.lsum[ht][1][lane & 31];
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
        for (int A = 0; A < 4; ++A) {
          const int d0 = 128 * pw + 32 * dt + 8 * A + 4 * h;
          const float v0 = O[ht][dt][4 * A] * inv, v1 = O[ht][dt][4 * A + 1] * inv;
          const float v2 = O[ht][dt][4 * A + 2] * inv, v3 = O[ht][dt][4 * A + 3] * inv;
          if (a.splits == 1) {
            *reinterpret_cast<float4*>(a.out + ((size_t)t * a.H + head) * a.kv_lora + d0) = make_float4(v0, v1, v2, v3);
          } else {
            uint16_t* dst = reinterpret_cast<uint16_t*>(a.ws) + (((size_t)t * a.H + head) * a.splits + split) * a.kv_lora + d0;
            *reinterpret_cast<uint2*>(dst) = make_uint2(cvt2_bf16(float2v{v0, v1}), cvt2_bf16(float2v{v2, v3}));
          }
        }
      }
    }
  }
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
  if (!xcd_query_map((a.H + kCombineHeads - 1) / kCombineHeads, a.T, mla_group(a.T, a.B), &t, &hq)) return;
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
    const dim3 xgrid(xcd_grid(a.splits, a.T, mla_group(a.T, a.B)));
    if (a.H > 32) {
      if (a.rope_dim == 64) launch(k_mla_fp8_ws<64, 2>, xgrid, dim3(kMlaThreads), 0, s, a);
      else launch(k_mla_fp8_ws<0, 2>, xgrid, dim3(kMlaThreads), 0, s, a);
    } else {
      if (a.rope_dim == 64) launch(k_mla_fp8_ws<64, 1>, xgrid, dim3(kMlaThreads), 0, s, a);
      else launch(k_mla_fp8_ws<0, 1>, xgrid, dim3(kMlaThreads), 0, s, a);
    }
  } else {
    if (a.rope_dim == 64) launch(k_mla_f32<64>, grid, dim3(kF32Threads), 0, s, a);
    else launch(k_mla_f32<0>, grid, dim3(kF32Threads), 0, s, a);
  }
  if (a.splits > 1) {
    const dim3 cgrid(xcd_grid((a.H + kCombineHeads - 1) / kCombineHeads, a.T, mla_group(a.T, a.B)));
    if (a.kv_dtype == DSA_FP8_E4M3FN) launch(k_mla_combine<true>, cgrid, dim3(kCombineThreads), 0, s, a);
    else launch(k_mla_combine<false>, cgrid, dim3(kCombineThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace dsa
