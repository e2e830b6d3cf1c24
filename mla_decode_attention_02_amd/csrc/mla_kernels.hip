// HIP kernels for MLA decode over a paged latent KV cache, written for
// gfx950 (MI355X, CDNA4).
//
// Method (TokenSpeed code-audit article, complete technology list, MLA
// kernel entries): each token stores one row of 512 latent + 64 rope values
// that serves as the key of every head and, through its latent part, as the
// value; a split kernel writes per-chunk fp32 partial results, and a
// reduction kernel merges them by log-sum-exp rescaling and casts to bf16.
// The tiled online softmax is the FlashAttention rewrite of the plain
// softmax ("推理优化" tag page, FlashAttention article: blockwise on-chip
// accumulation, identical result).
//
// Kernels in this file:
//   mla_split_mfma<FP8, WAVES, STAGES>  the hot path: Dc = 512, Dr = 64,
//       bf16 queries, bf16 or FP8-E4M3 KV, pages of a multiple of 32 tokens.
//   mla_split_generic                  any widths / dtypes, VALU only.
//   mla_combine_kernel                 log-sum-exp merge of split partials.
//   mla_gather_kernel                  test hook for the page-table loader.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include <mutex>
#include <type_traits>

#include "mla_internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef int intx2 __attribute__((vector_size(8)));
typedef unsigned uintx4 __attribute__((ext_vector_type(4)));
typedef unsigned uintx2 __attribute__((ext_vector_type(2)));
#define LDS_AS __attribute__((address_space(3)))

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

template <typename T>
__device__ __forceinline__ T uniform_load(const T* p) {
  // wave-uniform address: read through the scalar cache
  return *(const __attribute__((address_space(4))) T*)p;
}

// ------------------------------------------------------------------ loader
// Physical row of logical token j of request b: the block table maps the
// request's logical page j / P to a physical page, and j mod P is the slot in
// it ("推理优化" tag page, PagedAttention article).  The decode kernels, the
// append kernel and the gather hook resolve rows through this routine;
// kUniform reads the table entry through the scalar cache (b and j the same
// in every lane).
// (kv_page_entry and kv_row_of_page are its two halves, for callers that
// read the entry ahead of its use.)
__device__ __forceinline__ const int32_t* kv_page_entry(const int32_t* __restrict__ page_table, int MP,
                                                        int P, int b, int j) {
  return page_table + (int64_t)b * MP + j / P;
}
__device__ __forceinline__ int64_t kv_row_of_page(int page, int P, int j) { return (int64_t)page * P + (j % P); }
template <bool kUniform = false>
__device__ __forceinline__ int64_t kv_row_index(const int32_t* __restrict__ page_table, int MP,
                                                int P, int b, int j) {
  const int32_t* entry = kv_page_entry(page_table, MP, P, b, j);
  return kv_row_of_page(kUniform ? uniform_load(entry) : *entry, P, j);
}

// Split plan: chunk k of a request of length L, with S chunks, covers
// [k C, min((k+1) C, L)) where C = P * ceil(ceil(L / S) / P) (page aligned).
__device__ __forceinline__ void chunk_span(int L, int S, int P, int k, int* cb, int* ce) {
  const int per = (L + S - 1) / S;
  const int C = ((per + P - 1) / P) * P;
  const int64_t b0 = (int64_t)k * C;
  *cb = (int)(b0 < L ? b0 : L);
  const int64_t e0 = b0 + C;
  *ce = (int)(e0 < L ? e0 : L);
}

// Wavefront-wide reductions (64 lanes) by cross-lane shuffles.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Exchange between the two 32-lane halves of a wave (v_permlane32_swap):
// returns {own-half value, other-half value} combined by the caller.
__device__ __forceinline__ float half_swap_max(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

// OCP E4M3: sign, 4 exponent bits (bias 7), 3 mantissa bits; S.1111.111 is
// NaN; exponent 0 is subnormal (m * 2^-9).
__device__ __forceinline__ float e4m3_to_float(uint8_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  float mag;
  if (e == 15u && m == 7u) return __builtin_nanf("");
  if (e == 0u)
    mag = (float)m * (1.0f / 512.0f);
  else
    mag = __uint_as_float(((e + 120u) << 23) | (m << 20));
  return (c & 0x80u) ? -mag : mag;
}

// Eight E4M3 codes (little-endian in two dwords) -> eight bf16 (exact).
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(unsigned lo, unsigned hi) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// ----------------------------------------------------- MFMA tile geometry
// A tile is 32 consecutive tokens of one page.  In LDS:
//   latent rows: bf16 -> row r starts at 16 * B(r) bytes with
//     B(r) = 64 r + 64 (r >> 4) + 4 (r & 3) + 17 ((r >> 2) & 3), rows stored
//     whole and in order; fp8 -> rows r and r + 16 share a 1056 B block
//     (r & 15), 512 B each, with 16-byte chunk c at c ^ ((r >> 3) & 1)
//   rope rows:   r * 128 B (bf16) or r * 64 B (fp8), 16-byte chunks XOR
//     swizzled by row
//   scales:      32 fp32 (fp8 only), stored 8 times over so that one
//     full-wave load fills them
// These placements keep both LDS access patterns free of bank conflicts on a
// 64-bank LDS -- the QK^T read (16 lanes = 16 rows, one logical 16-byte chunk)
// and the transposed PV read (bf16: 4 rows x two 32-byte runs per 32 lanes;
// fp8: 8 rows x 2 chunks) -- and every read address is one base register
// plus an immediate.  The bf16 rows carry no XOR: the transposed read takes a
// row's 32 bytes from four lanes that must lie contiguous and in order.
template <bool FP8>
struct Tile {
  static constexpr int kRowBytes = FP8 ? 576 : 1152;  // stored row stride in HBM
  static constexpr int kLat = FP8 ? 512 : 1024;       // latent bytes per row
  static constexpr int kRope = FP8 ? 64 : 128;        // rope bytes per row
  static constexpr int kLatBytes = FP8 ? 16 * 1056 : 16 * 2176;
  static constexpr int kRopeBytes = 32 * kRope;
  static constexpr int kScaleBytes = FP8 ? 1024 : 0;  // 8 copies of the 32 scales
  static constexpr int kStage = kLatBytes + kRopeBytes + kScaleBytes;

  static __device__ __forceinline__ int lat_base(int r) {
    return FP8 ? ((r & 15) * 1056 + (r >> 4) * 512)
               : 16 * (64 * r + 64 * (r >> 4) + 4 * (r & 3) + 17 * ((r >> 2) & 3));
  }
  static __device__ __forceinline__ int xlat(int r) { return FP8 ? ((r >> 3) & 1) : 0; }
  static __device__ __forceinline__ int xrope(int r) { return FP8 ? ((r >> 2) & 3) : ((r >> 1) & 7); }

  // Direct HBM -> LDS loads per wave per tile (equal for every wave).
  template <int WAVES>
  static constexpr int loads_per_wave() {
    if (!FP8) return 36 / WAVES;
    return 16 / WAVES + (WAVES == 4 ? 1 : (WAVES == 2 ? 2 : 3));
  }
};

// One 64-lane direct HBM -> LDS load of 16 bytes per lane: lane i reads
// gbase + voff (gbase wave-uniform) and writes LDS address lds + 16 i.
// Issued through inline assembly so that the compiler does not guard every
// later LDS read with a wait for all outstanding loads; the kernel orders
// them itself with s_waitcnt vmcnt + a workgroup barrier before a stage is
// read, and a barrier before a stage is refilled.  The load takes its LDS
// address from M0, and a scalar write of M0 needs one wait state before a
// direct-to-LDS load reads it.
__device__ __forceinline__ void lds_dma16(const void* gbase, uint32_t voff, uint32_t lds) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds);  // wave-uniform by construction
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(gbase), "s"(m0v)
               : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(LDS_AS const void* p) {
  return (uint32_t)(uintptr_t)p;
}

// Direct-to-LDS load number q (0 <= q < loads_per_wave) of one tile for this
// wave.  `tile_g` is the first row of the tile in HBM (32 rows, contiguous
// within one page).
// Lane id passed through an empty asm statement: offsets computed from it are
// recomputed where they are used (a few VALU operations) instead of being
// kept live through the tile loop, where registers are the scarce resource.
__device__ __forceinline__ int fresh_lane() {
  int l = __lane_id();
  asm volatile("" : "+v"(l));
  return l;
}

template <bool FP8, int WAVES>
__device__ __forceinline__ void issue_piece(const char* tile_g, const float* scale_g,
                                            LDS_AS char* st, int wave, int /*lane*/, int q) {
  using G = Tile<FP8>;
  const int lane = fresh_lane();
  if constexpr (!FP8) {
    if (q < 32 / WAVES) {  // latent rows
      const int r = wave + q * WAVES;
      const int c = lane ^ G::xlat(r);
      lds_dma16(tile_g, r * G::kRowBytes + 16 * c, lds_addr(st + G::lat_base(r)));
    } else {  // rope: 8 rows per load
      const int qq = wave + (q - 32 / WAVES) * WAVES;
      const int r = 8 * qq + (lane >> 3);
      const int c = (lane & 7) ^ G::xrope(r);
      lds_dma16(tile_g, r * G::kRowBytes + G::kLat + 16 * c,
                lds_addr(st + G::kLatBytes + 1024 * qq));
    }
  } else {
    if (q < 16 / WAVES) {  // latent rows pr and pr + 16
      const int pr = wave + q * WAVES;
      const int r = pr + 16 * (lane >> 5);
      const int c = (lane & 31) ^ G::xlat(r);
      lds_dma16(tile_g, r * G::kRowBytes + 16 * c, lds_addr(st + pr * 1056));
    } else {
      // rope (2 loads) and scales (1 load: lane l reads scale chunk l mod 8),
      // spread so that every wave issues the same count; duplicate scale
      // loads write the same bytes.
      const int e = q - 16 / WAVES;
      int job;  // 0, 1 = rope halves; 2 = scales
      if (WAVES == 4) job = wave < 2 ? wave : 2;
      else if (WAVES == 2) job = e == 0 ? wave : 2;
      else job = e;
      if (job < 2) {
        const int r = 16 * job + (lane >> 2);
        const int c = (lane & 3) ^ G::xrope(r);
        lds_dma16(tile_g, r * G::kRowBytes + G::kLat + 16 * c,
                  lds_addr(st + G::kLatBytes + 1024 * job));
      } else {
        lds_dma16(scale_g, 16 * (lane & 7), lds_addr(st + G::kLatBytes + G::kRopeBytes));
      }
    }
  }
}

// All direct-to-LDS loads of one tile for this wave.
template <bool FP8, int WAVES>
__device__ __forceinline__ void issue_tile(const char* tile_g, const float* scale_g,
                                           LDS_AS char* st, int wave, int lane) {
#pragma unroll
  for (int q = 0; q < Tile<FP8>::template loads_per_wave<WAVES>(); ++q)
    issue_piece<FP8, WAVES>(tile_g, scale_g, st, wave, lane, q);
}

// Zero the rows r >= valid of a loaded tile (their slots are past the end of
// the request and may hold anything, NaN included); called by all threads.
template <bool FP8, int WAVES>
__device__ __forceinline__ void zero_tail_rows(LDS_AS char* st, int valid, int tid) {
  using G = Tile<FP8>;
  const int nrows = 32 - valid;
  constexpr int lat_chunks = G::kLat / 16, rope_chunks = G::kRope / 16;
  for (int x = tid; x < nrows * lat_chunks; x += 64 * WAVES) {
    const int r = valid + x / lat_chunks, c = x % lat_chunks;
    *(LDS_AS uintx4*)(st + G::lat_base(r) + 16 * c) = uintx4{0, 0, 0, 0};
  }
  for (int x = tid; x < nrows * rope_chunks; x += 64 * WAVES) {
    const int r = valid + x / rope_chunks, c = x % rope_chunks;
    *(LDS_AS uintx4*)(st + G::kLatBytes + r * G::kRope + 16 * c) = uintx4{0, 0, 0, 0};
  }
  if (FP8)
    for (int r = valid + tid; r < 32; r += 64 * WAVES)
      *(LDS_AS float*)(st + G::kLatBytes + G::kRopeBytes + 4 * r) = 0.0f;
}

// Token slot m of the QK^T A-operand is fed from tile row swap_bits23(m), so
// that in the MFMA accumulator lane-half h, register i holds tile token
// 16 (i / 8) + 8 h + (i % 8): eight consecutive tokens per PV step, matching
// what the transposed LDS reads deliver for the value operand.
__device__ __forceinline__ int swap_bits23(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// Latent/rope dims held by query-fragment kk for lane half h.
template <bool FP8>
__device__ __forceinline__ int qfrag_dim(int kk, int h) {
  return FP8 ? (32 * (kk >> 1) + 16 * h + 8 * (kk & 1)) : (16 * kk + 8 * h);
}

template <int N>
__device__ __forceinline__ void wait_ahead(int ahead) {
  // wait until at most `ahead` later tiles' loads (N each) are outstanding
  switch (ahead) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<N>(); break;
    case 2: wait_vmcnt<(2 * N < 64 ? 2 * N : 0)>(); break;
    case 3: wait_vmcnt<(3 * N < 64 ? 3 * N : 0)>(); break;
    case 4: wait_vmcnt<(4 * N < 64 ? 4 * N : 0)>(); break;
    default: wait_vmcnt<(5 * N < 64 ? 5 * N : 0)>(); break;
  }
}

// Score-tile MFMAs in inline assembly, with the accumulator constrained to
// VGPRs.  The output accumulators take all 256 AGPRs; the compiler's builtin
// would put this accumulator in AGPRs as well and shuffle output blocks out
// of the way.  The compiler does not know these are MFMAs, so it models none
// of their hazards, and the helpers cover them:
//   - each MFMA starts with two wait states (enough for a VALU write of an
//     operand just before);
//   - the chain accumulates in place, so the only writer of the accumulator
//     while an MFMA may still read it is the next MFMA of the same chain;
//   - the last MFMA waits out its result latency inside the same statement,
//     so no instruction the compiler places after it (a copy of the
//     accumulator included) can read the result early.
// A and B are read when an MFMA issues; only the accumulator is read later.
__device__ __forceinline__ void mfma_v0(floatx16& c, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_v(floatx16& c, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}
// mfma_drain() waits out the MFMA result latency before any other
// instruction may read or write an accumulator the asm MFMAs above wrote.
__device__ __forceinline__ void mfma_drain() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }
__device__ __forceinline__ void mfma_v_last(floatx16& c, const bf16x8& a, const bf16x8& b) {
  asm volatile(
      "s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\t"
      "s_nop 7\n\ts_nop 7\n\ts_nop 7"
      : "+v"(c)
      : "v"(a), "v"(b));
}

// ------------------------------------------------------- MFMA split kernel
// One workgroup = WAVES wavefronts = 32 * WAVES query rows (row r = t * H + h
// of one request: the query-token fold puts drafts and heads on one axis) over
// one chunk of one request.  Each wave keeps its 32 query rows in registers
// as the B operand of S^T = K Q^T (v_mfma_f32_32x32x16_bf16, K = the 576-deep
// dot split in 36 steps), so a row's 32 token scores sit in one lane pair and
// the softmax max/sum needs one half-swap; then O^T += V^T P^T with the value
// operand read transposed from the same LDS tile (ds_read_b64_tr_b16 / _b8).
// O^T for the wave's 32 rows x 512 latent columns is 16 accumulators (256
// registers per lane).
//
// Software pipeline, per tile i: one barrier (tile i has landed, every wave
// is done with tile i - 2, whose stage is refilled with tile i + STAGES - 2),
// then the scores of tile i, then the value product of tile i - 1 with the
// softmax of tile i interleaved between its MFMAs.
template <bool FP8, int WAVES, int STAGES>
__global__ void __launch_bounds__(64 * WAVES, 1)
mla_split_mfma(SplitParams p, int groups) {
  using G = Tile<FP8>;
  constexpr int kRows = 32 * WAVES;
  constexpr int kLoads = G::template loads_per_wave<WAVES>();
  constexpr int kDepth = STAGES - 2;  // tiles loading ahead of the one being scored
  static_assert(kDepth >= 1 && kDepth - 1 <= 5, "stage count");
  static_assert((kDepth - 1) * kLoads < 64, "vmcnt range");
  extern __shared__ __attribute__((aligned(1024))) char smem_raw[];
  LDS_AS char* smem = (LDS_AS char*)(LDS_AS void*)smem_raw;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int h = lane >> 5, n = lane & 31;

  const int M = p.T * p.H;
  // Work of this workgroup: a list of segments, each a run of 32-token tiles
  // of one unit (request b, row group g).
  //   Uniform chunks (p.NB == 0): one segment, chunk s of unit (b, g).  The
  //   block mapping is XCD-aware: consecutive hardware block ids go to
  //   different XCDs (id mod 8), so the row groups of one (request, chunk)
  //   are given ids 8 apart and share that XCD's L2 while they read the same
  //   pages.
  //   Balanced (p.NB > 0): the units' tiles, laid end to end (unit-major,
  //   each unit's preceded by kUnitStartCost positions for the cost of
  //   starting it; prefix sums in p.tile_prefix), are cut into NB equal
  //   contiguous ranges, one per workgroup; a range crosses unit boundaries
  //   freely, so every workgroup gets the same work whatever the length mix,
  //   a workgroup that starts a unit inside its range that many tiles fewer.
  int ub = 0, ug = 0, us = 0;
  int wx = 0, wx1 = 0;
  int wu = 0, wk = 0, wsu = 0;  // balanced: current unit and its first tile
  if (p.NB == 0 && p.Sp > 0) {
    // Cascade: chunk s runs on XCD s mod 8, where its workgroups for every
    // request and row group take consecutive slots, so that the workgroups
    // reading one shared-prefix chunk run together and share that XCD's L2.
    const int x = blockIdx.x;
    const int xcd = x & 7, slot = x >> 3;
    const int per = p.B * groups;
    const int sl8 = slot / per, rem = slot - sl8 * per;
    us = 8 * sl8 + xcd;
    if (us >= p.S) return;
    ub = rem / groups;
    ug = rem - ub * groups;
  } else if (p.NB == 0) {
    const int x = blockIdx.x;
    const int xcd = x & 7, slot = x >> 3;
    const int k8 = slot / groups;
    ug = slot - k8 * groups;
    const int unit = 8 * k8 + xcd;
    if (unit >= p.B * p.S) return;
    ub = unit / p.S;
    us = unit - ub * p.S;
  } else {
    // Plan, in every workgroup: each thread sums the tiles of a run of
    // units, a block-wide scan gives the runs' offsets, and the thread whose
    // run holds this workgroup's first tile finds its unit.  Workgroup 0
    // also writes the prefix sums for the merge.
    volatile LDS_AS int* ps = (volatile LDS_AS int*)(smem + STAGES * G::kStage + 8 * WAVES);
    const int U = p.B * groups;
    const int per = (U + 64 * WAVES - 1) / (64 * WAVES);
    const int u0 = tid * per < U ? tid * per : U;
    const int u1 = u0 + per < U ? u0 + per : U;
    auto unit_tiles = [&](int u) {  // the unit's positions: tiles + start cost
      const int Lu = p.seq_lens[u / groups];
      return Lu > 0 ? ((Lu + 31) >> 5) + kUnitStartCost : 0;
    };
    int run_sum = 0;
    for (int u = u0; u < u1; ++u) run_sum += unit_tiles(u);
    int incl = run_sum;  // inclusive scan within the wave
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_up(incl, off, 64);
      if (lane >= off) incl += v;
    }
    if (lane == 63) ps[wave] = incl;
    __syncthreads();
    int W = 0, before = 0;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      const int v = ps[w];
      before += w < wave ? v : 0;
      W += v;
    }
    W = __builtin_amdgcn_readfirstlane(W);  // the same in every lane
    const int excl = before + incl - run_sum;
    if (blockIdx.x == 0) {
      int run = excl;
      for (int u = u0; u < u1; ++u) {
        p.tile_prefix[u] = run;
        run += unit_tiles(u);
      }
      if (tid == 0) p.tile_prefix[U] = W;
    }
    // no workgroup with an empty range (a range may still hold only a unit's
    // start positions: its workgroup then has no segment)
    const int64_t nb = W < p.NB ? W : p.NB;
    // Ranges are dealt so that each XCD (hardware block id mod 8; the grid
    // is NB workgroups) runs a contiguous run of NB / 8 of them: the few
    // workgroups that share a unit, and so read its query rows, then mostly
    // share one L2.
    wk = (p.NB & 7) == 0 ? (int)(blockIdx.x & 7) * (p.NB >> 3) + (int)(blockIdx.x >> 3) : (int)blockIdx.x;
    if (wk >= nb) return;
    // (W < 2^30, so the bounds fit in int32; read back as wave-uniform values)
    wx = __builtin_amdgcn_readfirstlane((int)(wk * (int64_t)W / nb));
    wx1 = __builtin_amdgcn_readfirstlane((int)((wk + 1) * (int64_t)W / nb));
    if (excl <= wx && wx < excl + run_sum) {
      int run = excl, fu = u0, fr = excl;
      bool found = false;
      for (int u = u0; u < u1; ++u) {
        const int tu = unit_tiles(u);
        const bool hit = !found && wx < run + tu;
        fu = hit ? u : fu;
        fr = hit ? run : fr;
        found = found || hit;
        run += tu;
      }
      ps[WAVES] = fu;
      ps[WAVES + 1] = fr;
    }
    __syncthreads();
    wu = __builtin_amdgcn_readfirstlane(ps[WAVES]);
    wsu = __builtin_amdgcn_readfirstlane(ps[WAVES + 1]);
  }

  for (bool more_segments = true; more_segments;) {
  int b, g, L, cb, ce;
  // destination: rows [drow, drow + kRows) of out/lse when the segment is a
  // whole unit (final_out), else of the partial buffers
  bool final_out;
  int64_t drow;
  if (p.NB == 0) {
    more_segments = false;
    b = ub;
    g = ug;
    L = uniform_load(p.seq_lens + b);
    if (p.Sp == 0) {
      chunk_span(L, p.S, p.P, us, &cb, &ce);
    } else if (us < p.Sp) {  // shared-prefix chunk: the same bounds for every request
      chunk_span(p.prefix_len, p.Sp, p.P, us, &cb, &ce);
      cb = cb < L ? cb : L;
      ce = ce < L ? ce : L;
    } else {  // suffix chunk of [prefix_len, L)
      const int Ls = L > p.prefix_len ? L - p.prefix_len : 0;
      chunk_span(Ls, p.S - p.Sp, p.P, us - p.Sp, &cb, &ce);
      cb += p.prefix_len;
      ce += p.prefix_len;
    }
    final_out = p.write_final;
    drow = final_out ? (int64_t)b * M + (int64_t)g * kRows
                     : ((int64_t)b * p.S + us) * M + (int64_t)g * kRows;
  } else {
    // Unit wu occupies positions [su, eu): kUnitStartCost positions, then
    // its tiles from ts = su + kUnitStartCost on.
    int su = wsu, eu;
    for (;;) {  // skip units that end at or before wx (and units without tiles)
      b = wu / groups;
      L = uniform_load(p.seq_lens + b);
      eu = su + (L > 0 ? ((L + 31) >> 5) + kUnitStartCost : 0);
      if (eu > wx) break;
      ++wu;
      su = eu;
    }
    const int ts = su + kUnitStartCost;
    const int s0 = wx > ts ? (int)wx : ts;
    const int e = (int)(wx1 < eu ? wx1 : eu);
    if (s0 >= e) break;  // the range ends inside the unit's start cost: none of its tiles here
    g = wu - b * groups;
    cb = 32 * (s0 - ts);
    ce = 32 * (e - ts);
    if (ce > L) ce = L;
    // Partial slots: [NB][2][kRows] rows.  Slot 0 holds the segment that
    // continues a unit begun in an earlier workgroup, slot 1 the one that
    // starts a unit and continues into later workgroups.
    final_out = s0 == ts && e == eu;
    drow = final_out ? (int64_t)b * M + (int64_t)g * kRows
                     : ((int64_t)wk * 2 + (s0 > ts ? 0 : 1)) * kRows;
    wx = e;
    ++wu;
    wsu = eu;
    more_segments = wx < wx1;
  }
  // the previous segment's waves are done with every stage (and with the
  // restart words, cleared here) before this one refills them
  __syncthreads();
  if (tid < 2) ((volatile LDS_AS uint32_t*)(smem + STAGES * G::kStage))[tid] = 0;

  const int lr = 32 * wave + n;  // this lane's row within the group
  const int gr = g * kRows + lr;  // this lane's query row
  const bool row_ok = gr < M;
  const int t = row_ok ? gr / p.H : 0;
  const int vis = p.causal ? (L - p.T + 1 + t) : L;
  const int lim = vis < ce ? vis : ce;  // tokens >= lim are masked for this row

  // ---- query fragments (B operand), staged through LDS: each wave copies
  // its 32 rows into its own region of the idle stages with whole-row
  // direct-to-LDS loads (one 1 KB latent row per load, eight 128-byte rope
  // rows per load) and reads its fragments from there; loaded straight into
  // the fragment layout, every load would touch 32 rows.  Padding rows
  // (gr >= M) reuse row M - 1: they are computed like any row and never
  // written out.
  bf16x8 qf[36];
  {
    constexpr int kQPitch = 1024 + 16;  // latent row pitch (conflict-free fragment reads)
    constexpr int kQWave = 32 * kQPitch + 32 * 128;
    static_assert(WAVES * kQWave <= STAGES * G::kStage, "query staging fits the stages");
    LDS_AS char* qst = smem + wave * kQWave;
    LDS_AS char* qrs = qst + 32 * kQPitch;
    const int64_t qrow0 = (int64_t)b * M;
    const int wr0 = g * kRows + 32 * wave;
    const int ql = fresh_lane();
#pragma unroll 4
    for (int r = 0; r < 32; ++r) {
      const int rr = wr0 + r < M ? wr0 + r : M - 1;
      lds_dma16((const char*)p.q_abs + (qrow0 + rr) * 1024, 16 * ql, lds_addr(qst + r * kQPitch));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int rb = wr0 + 8 * j < M ? wr0 + 8 * j : M - 1;
      const int rl = wr0 + 8 * j + (ql >> 3) < M ? wr0 + 8 * j + (ql >> 3) : M - 1;
      lds_dma16((const char*)p.q_rope + (qrow0 + rb) * 128, (rl - rb) * 128 + 16 * (ql & 7),
                lds_addr(qrs + 1024 * j));
    }
    wait_vmcnt<0>();
#pragma unroll
    for (int kk = 0; kk < 32; ++kk)
      qf[kk] = *(const LDS_AS bf16x8*)(qst + n * kQPitch + 2 * qfrag_dim<FP8>(kk, h));
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      qf[32 + kk] = *(const LDS_AS bf16x8*)(qrs + n * 128 + 2 * qfrag_dim<FP8>(kk, h));
    __syncthreads();  // every wave has its fragments before the stages refill
  }

  floatx16 acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = floatx16{};
  // Softmax reference: p = 2^(z - m_ref) in the log2 domain.  m_ref is the
  // row maximum of the chunk's first tile and is never moved while
  // accumulating: any reference within 2^60 of the true maximum keeps every p
  // and every partial sum finite and normal in fp32/bf16, so O needs no
  // rescaling.  If a later tile's maximum exceeds m_ref by more than that,
  // the workgroup restarts the chunk with m_ref = the largest maximum seen
  // (zeroing the accumulators), which real attention logits never trigger.
  float m_ref = neg_inf();
  float m_seen = neg_inf();  // largest tile maximum seen so far
  float l_part = 0.0f;       // this lane-half's share of the normaliser (odd
  float l_part2 = 0.0f;      // and even scores in two sums)
  const float scale_log2 = p.scale * kLog2e;
  constexpr float kRestartMargin = 60.0f;

  const int ntiles = (ce - cb + 31) >> 5;

  const char* kv = (const char*)p.kv;
  const int rho = swap_bits23(n);  // tile row feeding A-operand slot n

  auto stage_of = [&](int i) -> LDS_AS char* { return smem + (i % STAGES) * G::kStage; };
  // the two halves of kv_row_index, the entry read a step ahead of its use
  auto page_of = [&](int i) { return uniform_load(kv_page_entry(p.page_table, p.MP, p.P, b, cb + 32 * i)); };
  auto row_of = [&](int i, int page) { return kv_row_of_page(page, p.P, cb + 32 * i); };
  auto issue = [&](int i) {
    const int64_t row0 = row_of(i, page_of(i));
    issue_tile<FP8, WAVES>(kv + row0 * G::kRowBytes, FP8 ? p.kv_scales + row0 : nullptr,
                           stage_of(i), wave, lane);
  };

  // per-lane LDS read offsets (stage relative)
  const int k_off = G::lat_base(rho) + 16 * (FP8 ? (h ^ G::xlat(rho)) : 0);
  const int grp = lane >> 4, sl = lane & 15, dh = grp & 1;

  // S^T = K Q^T for one tile (32 tokens x 32 rows) in one accumulation chain
  // (back-to-back dependent MFMAs still issue every 32 cycles), K operands
  // read from LDS a few steps ahead of the MFMA using them.
  // The loads of a later tile are issued a few at a time between the MFMAs,
  // not in one burst that would stall on the vector-memory issue queue.
  struct Loader {
    const char* tg;
    const float* sg;
    LDS_AS char* dst;
  };
  // The kLoads direct-to-LDS loads of a later tile go out between the score
  // MFMAs, one every kQkEvery steps of the score loop: early in the step, so
  // that they have the most time to land, and spread, so that the CU's load
  // issue never bursts.  (Issued between the value MFMAs too, as earlier
  // versions did, they left the speculative-decode shape 2 % slower.)
  constexpr int kQkSteps = FP8 ? 18 : 36;
  constexpr int kQkLoads = kLoads;
  constexpr int kQkEvery = kQkSteps / kQkLoads;
  static_assert(kQkEvery * kQkLoads <= kQkSteps, "load spread");
  auto scores = [&](LDS_AS char* st, floatx16& sacc, const Loader& ld, auto with_loads) {
    constexpr bool kLd = decltype(with_loads)::value;
    floatx16 s0;
    const LDS_AS char* ropep = st + G::kLatBytes + rho * G::kRope;
    const int swr = G::xrope(rho);
    if constexpr (!FP8) {
      const LDS_AS char* rowp = st + k_off + 16 * h;
      auto kaddr = [&](int kk) -> const LDS_AS bf16x8* {
        return kk < 32 ? (const LDS_AS bf16x8*)(rowp + 32 * kk)
                       : (const LDS_AS bf16x8*)(ropep + 16 * ((2 * (kk - 32) + h) ^ swr));
      };
      constexpr int kAhead = 4;
      bf16x8 ring[kAhead];
#pragma unroll
      for (int kk = 0; kk < kAhead; ++kk) ring[kk] = *kaddr(kk);
#pragma unroll
      for (int kk = 0; kk < 36; ++kk) {
        const bf16x8 a = ring[kk % kAhead];
        if (kk + kAhead < 36) ring[kk % kAhead] = *kaddr(kk + kAhead);
        if (kLd && kk % kQkEvery == kQkEvery - 1 && kk / kQkEvery < kQkLoads)
          issue_piece<FP8, WAVES>(ld.tg, ld.sg, ld.dst, wave, lane, kk / kQkEvery);
        if (kk == 0) mfma_v0(s0, a, qf[0]);
        else if (kk < 35) mfma_v(s0, a, qf[kk]);
        else mfma_v_last(s0, a, qf[kk]);
      }
    } else {
      const LDS_AS char* rowp = st + k_off;
      auto kaddr = [&](int kk) -> const LDS_AS uintx4* {
        return kk < 16 ? (const LDS_AS uintx4*)(rowp + 32 * kk)
                       : (const LDS_AS uintx4*)(ropep + 16 * ((2 * (kk - 16) + h) ^ swr));
      };
      constexpr int kAhead = 2;
      uintx4 ring[kAhead];
#pragma unroll
      for (int kk = 0; kk < kAhead; ++kk) ring[kk] = *kaddr(kk);
#pragma unroll
      for (int kk = 0; kk < 18; ++kk) {
        const uintx4 raw = ring[kk % kAhead];
        if (kk + kAhead < 18) ring[kk % kAhead] = *kaddr(kk + kAhead);
        if (kLd && kk % kQkEvery == 1 && kk / kQkEvery < kQkLoads)
          issue_piece<FP8, WAVES>(ld.tg, ld.sg, ld.dst, wave, lane, kk / kQkEvery);
        const int q0 = kk < 16 ? 2 * kk : 32 + 2 * (kk - 16);
        const bf16x8 a0 = e4m3x8_to_bf16(raw[0], raw[1]);
        const bf16x8 a1 = e4m3x8_to_bf16(raw[2], raw[3]);
        if (kk == 0) mfma_v0(s0, a0, qf[q0]);
        else mfma_v(s0, a0, qf[q0]);
        if (kk < 17) mfma_v(s0, a1, qf[q0 + 1]);
        else mfma_v_last(s0, a1, qf[q0 + 1]);
      }
    }
    sacc = s0;
  };

  // Restart requests: byte [i % 2][wave] is written by every wave while it
  // handles tile i and read by all waves after the barrier that opens tile
  // i + 1 (the four bytes of a tile in one 32-bit read, which the barrier
  // orders after the writes); it is next written for tile i + 2, after the
  // following barrier.  Both words are cleared before step 0.
  static_assert(WAVES == 4, "one byte per wave in a 32-bit restart word");
  volatile LDS_AS uint8_t* req = (volatile LDS_AS uint8_t*)(smem + STAGES * G::kStage);
  auto restart_word = [&](int i) -> int {
    return (int)*(const LDS_AS uint32_t*)(smem + STAGES * G::kStage + 4 * (i & 1));
  };

  // One step of the softmax of tile i (32 steps per tile, interleaved with the
  // 32 MFMAs of the value product of tile i - 1); each step works on two
  // scores so that its instructions form two independent chains:
  //   steps 0..7    mask scores 2k, 2k+1 (FP8: times the token scale) and
  //                 fold them into two running maxima;
  //   step 8        the row maximum across both halves and the lane pair,
  //                 times s = scale * log2 e (s > 0: max(s z) = s max(z)
  //                 exactly, rounding being monotonic);
  //   step 9        the reference maximum and the restart request;
  //   steps 10..17  p = 2^(s z - m_ref) for scores 2(k-10), 2(k-10)+1;
  //   steps 18..25  round two weights to bf16 for the value product (FP8:
  //                 times the token scale) and add the rounded weights to the
  //                 normaliser, exactly as the product sees them;
  //   step 26       publish this wave's restart request.
  struct SoftmaxState {
    float mx_a, mx_b, mu;
    bool over;
  };
  // running maximum without the NaN canonicalisation fmaxf implies; the
  // volatile statement also keeps the step's work in its step
  auto vmax = [](float& m, float x) { asm volatile("v_max_f32 %0, %0, %1" : "+v"(m) : "v"(x)); };
  auto softmax_step = [&](int k, const float (&tscv)[16], int lim_rel, floatx16& z,
                          bf16x8 (&pb)[2], SoftmaxState& sm, int i) {
    if (k < 8) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int e = 2 * k + u;
        const int tok = 16 * (e >> 3) + 8 * h + (e & 7);
        float v = z[e];
        if constexpr (FP8) v *= tscv[e];
        z[e] = tok < lim_rel ? v : neg_inf();
      }
      vmax(sm.mx_a, z[2 * k]);
      vmax(sm.mx_b, z[2 * k + 1]);
    } else if (k == 8) {
      float mx = sm.mx_a;
      vmax(mx, sm.mx_b);
      sm.mx_a = half_swap_max(mx) * scale_log2;
      asm volatile("" : "+v"(sm.mx_a));
    } else if (k == 9) {
      const float mx = sm.mx_a;
      m_seen = fmaxf(m_seen, mx);
      m_ref = m_ref == neg_inf() ? mx : m_ref;  // first tile with a visible token
      sm.over = mx > m_ref + kRestartMargin;
      sm.mu = m_ref == neg_inf() ? 0.0f : m_ref;
      asm volatile("" : "+v"(sm.mu));
    } else if (k < 18) {
      const int e = 2 * (k - 10);
#pragma unroll
      for (int u = 0; u < 2; ++u) z[e + u] = fast_exp2(__builtin_fmaf(z[e + u], scale_log2, -sm.mu));
      asm volatile("" : "+v"(z));
    } else if (k < 26) {
      const int e = 2 * (k - 18), q = e >> 3, j = e & 7;
      const __bf16 w0 = (__bf16)z[e], w1 = (__bf16)z[e + 1];
      l_part += (float)w0;  // the normaliser sums the weights exactly as PV sees them
      l_part2 += (float)w1;
      if constexpr (FP8) {
        pb[q][j] = (__bf16)((float)w0 * tscv[e]);
        pb[q][j + 1] = (__bf16)((float)w1 * tscv[e + 1]);
      } else {
        pb[q][j] = w0;
        pb[q][j + 1] = w1;
      }
      asm volatile("" : "+v"(l_part), "+v"(l_part2));
    } else if (k == 26) {
      req[(i & 1) * WAVES + wave] = __builtin_amdgcn_ballot_w64(sm.over) != 0 ? 1 : 0;
    }
  };

  // O^T += V^T P^T for the tile in stage sv with weights pw, one softmax step
  // of tile i after each MFMA (each step is its own scheduling region, so the
  // VALU work sits between the MFMAs instead of after them).
  auto values_softmax = [&](LDS_AS char* sv, const bf16x8 (&pw)[2], LDS_AS char* st, int i,
                            floatx16& z, bf16x8 (&pb)[2]) {
    const int lim_rel = lim - (cb + 32 * i);
    SoftmaxState sm{neg_inf(), neg_inf(), 0.0f, false};
    // FP8: the scales of this lane's 16 tokens (two runs of 8), read up front
    // so that no step waits on an LDS read behind the value prefetches
    float tscv[16];
    if constexpr (FP8) {
      const LDS_AS float* tsc = (const LDS_AS float*)(st + G::kLatBytes + G::kRopeBytes);
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const floatx4 u0 = *(const LDS_AS floatx4*)(tsc + 16 * r + 8 * h);
        const floatx4 u1 = *(const LDS_AS floatx4*)(tsc + 16 * r + 8 * h + 4);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          tscv[8 * r + c] = u0[c];
          tscv[8 * r + 4 + c] = u1[c];
        }
      }
    } else {
#pragma unroll
      for (int c = 0; c < 16; ++c) tscv[c] = 1.0f;
    }
    if constexpr (!FP8) {
      // Rows r0 = 8h + (sl >> 2) (+4, +16, +20) of the tile: r0 & 15 <= 11,
      // so B(r0 + 4) = B(r0) + 273 and B(r0 + 16) = B(r0) + 1088, and all
      // four reads are one base register plus immediates.
      const int ln = fresh_lane(), lh = ln >> 5, lsl = ln & 15, ldh = (ln >> 4) & 1;
      const LDS_AS char* vb =
          sv + G::lat_base(8 * lh + (lsl >> 2)) + 16 * (2 * ldh + ((lsl & 3) >> 1)) + 8 * (lsl & 1);
      // whole-vector reinterpretation of the two transposed reads
      // (element-wise bf16 inserts were miscompiled into a broadcast)
      auto vread = [&](int x2) -> bf16x8 {
        const int q = x2 >> 4, db = x2 & 15;
        const LDS_AS char* b0 = vb + 16 * 1088 * q + 64 * db;
        const shortx4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS shortx4*)b0);
        const shortx4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS shortx4*)(b0 + 16 * 273));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      constexpr int kAhead = 5;  // value operands in flight ahead of their MFMA
      bf16x8 ring[kAhead];
#pragma unroll
      for (int x2 = 0; x2 < kAhead; ++x2) ring[x2] = vread(x2);
#pragma unroll
      for (int x2 = 0; x2 < 32; ++x2) {
        const bf16x8 a = ring[x2 % kAhead];
        if (x2 + kAhead < 32) ring[x2 % kAhead] = vread(x2 + kAhead);
        acc[x2 & 15] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pw[x2 >> 4], acc[x2 & 15], 0, 0, 0);
        softmax_step(x2, tscv, lim_rel, z, pb, sm, i);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      // rows r0 = 8h + (sl >> 1) and r0 + 16 share a block, 512 B apart,
      // with the same chunk swizzle: one base register plus immediates
      const int ln = fresh_lane(), lsl = ln & 15, ldh = (ln >> 4) & 1;
      const int r0 = 8 * (ln >> 5) + (lsl >> 1);
      const LDS_AS char* vb = sv + G::lat_base(r0) + 16 * (ldh ^ G::xlat(r0)) + 8 * (lsl & 1);
      auto vread = [&](int x2) -> intx2 {
        return __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS intx2*)(vb + 512 * (x2 >> 4) + 32 * (x2 & 15)));
      };
      constexpr int kAhead = 3;
      intx2 ring[kAhead];
#pragma unroll
      for (int x2 = 0; x2 < kAhead; ++x2) ring[x2] = vread(x2);
#pragma unroll
      for (int x2 = 0; x2 < 32; ++x2) {
        const intx2 v = ring[x2 % kAhead];
        if (x2 + kAhead < 32) ring[x2 % kAhead] = vread(x2 + kAhead);
        acc[x2 & 15] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            e4m3x8_to_bf16((unsigned)v[0], (unsigned)v[1]), pw[x2 >> 4], acc[x2 & 15], 0, 0, 0);
        softmax_step(x2, tscv, lim_rel, z, pb, sm, i);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // The value product "of tile -1" in the first step reads the last stage with
  // zero weights: clear it so that it holds no NaN.
  auto clear_stage = [&](LDS_AS char* st) {
    for (int o = 16 * tid; o < G::kStage; o += 16 * 64 * WAVES)
      *(LDS_AS uintx4*)(st + o) = uintx4{0, 0, 0, 0};
  };
  clear_stage(stage_of(STAGES - 1));
#pragma unroll
  for (int i = 0; i < kDepth; ++i)
    if (i < ntiles) issue(i);

  bf16x8 pprev[2] = {bf16x8{}, bf16x8{}};
  // page of the next tile to load, read one step ahead of its use
  int pg_next = kDepth < ntiles ? page_of(kDepth) : 0;
  for (; ntiles > 0;) {
    bool restart = false;
    // Step i scores tile i (if i < ntiles) and accumulates the values of
    // tile i - 1; step ntiles only finishes the last tile.
    for (int i = 0; i <= ntiles; ++i) {
      const int ahead_tiles = ntiles - 1 - i;
      wait_ahead<kLoads>(ahead_tiles < 0 ? 0 : (ahead_tiles < kDepth - 1 ? ahead_tiles : kDepth - 1));
      __syncthreads();
      // restart requests of tile i - 1: read now, acted on after the scores
      const int asked = restart_word(i - 1);  // zero for i = 0 (cleared per segment)
      // tile i + kDepth goes to the stage freed by tile i - 2
      const int64_t row0 = row_of(i + kDepth, pg_next);
      const Loader ld{kv + row0 * G::kRowBytes, FP8 ? p.kv_scales + row0 : nullptr,
                      stage_of(i + kDepth)};
      LDS_AS char* st = stage_of(i);
      const int ts = cb + 32 * i;
      if (i < ntiles && ts + 32 > L) {  // last tile of the request: clear slots past its end
        zero_tail_rows<FP8, WAVES>(st, L - ts, tid);
        __syncthreads();
      }
      // step ntiles scores whatever its stage holds: every token is masked.
      // One uniform branch per step picks the variant with or without loads,
      // so that the MFMA loop itself has no branches.
      floatx16 z;
      if (i + kDepth < ntiles)
        scores(st, z, ld, std::true_type{});
      else
        scores(st, z, ld, std::false_type{});
      if (__builtin_amdgcn_readfirstlane(asked) != 0) {
        restart = true;
        break;
      }
      __builtin_amdgcn_sched_barrier(0);
      bf16x8 pcur[2];
      values_softmax(stage_of(i + STAGES - 1), pprev, st, i, z, pcur);
      pprev[0] = pcur[0];
      pprev[1] = pcur[1];
      // branch-free: past the last tile this re-reads a valid entry and is unused
      pg_next = page_of(i + kDepth + 1 < ntiles ? i + kDepth + 1 : 0);
    }
    if (!restart) break;
    // Rare path: drain the pipeline, reset, and run the chunk again (the
    // restart words are cleared too: step 0 reads them).
    wait_vmcnt<0>();
    __syncthreads();
    if (tid < 2) ((volatile LDS_AS uint32_t*)(smem + STAGES * G::kStage))[tid] = 0;
    clear_stage(stage_of(STAGES - 1));
    m_ref = m_seen;
    l_part = 0.0f;
    l_part2 = 0.0f;
    pprev[0] = bf16x8{};
    pprev[1] = bf16x8{};
#pragma unroll
    for (int db = 0; db < 16; ++db) acc[db] = floatx16{};
#pragma unroll
    for (int i = 0; i < kDepth; ++i)
      if (i < ntiles) issue(i);
    pg_next = kDepth < ntiles ? page_of(kDepth) : 0;
  }

  // ---- epilogue: normalise and write (lane pair n, n+32 shares row gr)
  const float l_tot = half_swap_sum(l_part + l_part2);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  const float lse_v = l_tot > 0.0f ? (m_ref + __log2f(l_tot)) * kLn2 : neg_inf();
  // The rows go out through LDS: each wave writes its normalised rows into
  // its own region of the (now idle) stages, row r at r * kPitch, then reads
  // them back a row at a time, so that every store writes 1 KB of one row.
  // Stored straight from the accumulator layout, one instruction would write
  // 32 bytes into each of 32 rows (32 partial cache lines).  fp32 rows go in
  // two passes of 256 columns, bf16 rows in one.  The 16-byte pad keeps the
  // row-scattered writes free of bank conflicts.
  constexpr int kPitch = 1024 + 16;
  static_assert(WAVES * 32 * kPitch <= STAGES * G::kStage, "output staging fits the stages");
  // (the destination row is taken through an empty asm statement so that
  // no address of it is computed before, and kept live through, the loop)
  asm volatile("" : "+s"(drow));
  __syncthreads();  // every wave is done with the stages
  LDS_AS char* wst = smem + wave * 32 * kPitch;
  const int wrow0 = g * kRows + 32 * wave;  // query row of this wave's staged row 0
  auto stage_out = [&](int db0, int ndb, auto cvt) {
    constexpr int esz = sizeof(decltype(cvt(floatx4{}))) / 4;
#pragma unroll
    for (int db = 0; db < ndb; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const floatx4 v = floatx4{acc[db0 + db][4 * g4 + 0], acc[db0 + db][4 * g4 + 1],
                                  acc[db0 + db][4 * g4 + 2], acc[db0 + db][4 * g4 + 3]} * inv;
        *(decltype(cvt(v))*)(wst + n * kPitch + esz * (32 * db + 8 * g4 + 4 * h)) = cvt(v);
      }
  };
  auto drain = [&](char* dst, int64_t row_bytes) {  // dst: this wave's row 0 at this pass's column
#pragma unroll 1
    for (int r0 = 0; r0 < 32; r0 += 8) {  // eight rows in flight at a time
      uintx4 v[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) v[r] = *(const LDS_AS uintx4*)(wst + (r0 + r) * kPitch + 16 * lane);
#pragma unroll
      for (int r = 0; r < 8; ++r)
        if (wrow0 + r0 + r < M) *(uintx4*)(dst + (r0 + r) * row_bytes + 16 * lane) = v[r];
    }
  };
  auto to_bf16 = [](floatx4 v) { return bf16x4{(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]}; };
  auto to_f32 = [](floatx4 v) { return v; };
  const int64_t orow0 = drow + 32 * wave;
  if (final_out && p.out_dtype == kBF16) {
    stage_out(0, 16, to_bf16);
    drain((char*)((__bf16*)p.out + orow0 * 512), 1024);
  } else if (!final_out && p.NB > 0) {  // balanced slots hold bf16 partials
    stage_out(0, 16, to_bf16);
    drain((char*)((__bf16*)p.part_o + orow0 * 512), 1024);
  } else {
    float* base = final_out ? (float*)p.out + orow0 * 512 : p.part_o + orow0 * 512;
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      stage_out(8 * pass, 8, to_f32);
      drain((char*)(base + 256 * pass), 2048);
    }
  }
  if (row_ok && h == 0) {
    const int64_t orow = drow + lr;
    if (!final_out) p.part_lse[orow] = lse_v;
    else if (p.lse) p.lse[orow] = lse_v;
  }
  }  // segments
}

// --------------------------------------------- MFMA split kernel, wave pairs
// One workgroup = NP pairs of wavefronts (NP = 4: 8 waves, 128 query rows,
// the unit of the balanced work list, the one launched; NP = 2: 4 waves, 64
// rows) over rows of one request b (row r = t * H + h, the query-token fold).  Pair p (waves p and
// p + NP) owns rows 32p .. 32p + 31 of the workgroup and splits both
// contractions in halves: role 0 (wave p + NP) forms the partial scores over
// dims [0, 288) of the 576-deep dot and owns output columns [0, 256); role 1
// (wave p) takes dims [288, 576) and columns [256, 512).  A wave so
// holds 15 query fragments in registers (3 more in LDS) and 128 fp32
// accumulators, 252 VGPRs in all: with NP = 4 two waves share each SIMD.
//
// Scores are S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (a row's 32 token
// scores sit in one lane pair), values O^T += V^T P^T with V read transposed
// from the same LDS tile.  Step i (tile i, 32 tokens), one workgroup barrier:
//   role 1  issues the direct HBM -> LDS loads of tile i + 1 (its share of
//           the tile; the stage tile i - 2 left), scores tile i (18 MFMAs,
//           one chain), writes its partial score tile to the pair's LDS slot
//           and marks it ready, then runs its half of tile i - 1's value
//           product (16 MFMAs) with the weights role 0 left in the slot;
//   role 0  scores tile i, waits for the mark, adds the partial, runs the
//           softmax (lazy reference, see kRescaleMargin), writes the bf16
//           weights to the slot and runs its half of tile i's value product.
// LDS: three tile stages, one 4 KB exchange slot per pair (partial scores,
// then weights, at the end 1 / normaliser), the kept query fragments, one
// restart word and one ready mark per pair.
// E4M3 KV (the quantisation article's FP8 table; code-audit article, FP8 KV
// cache entry): the stages hold codes and per-token scales; each wave
// converts to bf16 only the key half it scores and the value columns it
// owns, at the operand read; role 0 multiplies the summed scores and the
// weights by the token scales (the normaliser takes the weights alone).
constexpr int kXchgSlot = 4096;
constexpr int kRowPitch = 1024 + 16;             // staged query / output rows
constexpr int kQRegion = 32 * kRowPitch + 32 * 128;
// Of a wave's 18 query fragments (16 dims each) the first kQReg stay in
// registers and the last kQLds are re-read from LDS every tile: registers are
// what limits a wave pair per SIMD, and three 16-byte reads per tile are cheap.
constexpr int kQLds = 3, kQReg = 18 - kQLds;
// Softmax reference margin (log2 domain): a tile whose maximum exceeds the
// reference by more than this makes the workgroup run its segment again with
// a larger reference; below it every weight and partial sum stays under 2^60.
constexpr float kRescaleMargin = 60.0f;

template <int NP, bool FP8 = false>
struct PairLds {
  static_assert(NP == 2 || NP == 4, "two or four pairs per workgroup");
  static_assert(!FP8 || NP == 4, "E4M3 tiles: four pairs");
  static constexpr int kCStage = Tile<FP8>::kStage;
  static constexpr int kXchg = 3 * kCStage;             // exchange slots, one per pair
  static constexpr int kQKeep = kXchg + NP * kXchgSlot;  // per wave: the query fragments kept in LDS
  static constexpr int kRestart = kQKeep + 2 * NP * kQLds * 1024;  // one restart word per pair (4 words)
  static constexpr int kReady = kRestart + 16;  // per pair: tiles whose partial scores are in the slot
  static constexpr int kPipe = kReady + 16;
  static constexpr int kBytes = kPipe > NP * kQRegion ? kPipe : NP * kQRegion;
  static_assert(NP * 32 * kRowPitch <= kBytes, "output staging fits");
  static_assert(kBytes <= 160 * 1024, "fits the LDS");
};

// One segment: a run of tiles [cb, ce) of unit (b, g); its rows go to out /
// lse (final_out) or to partial rows starting at drow.
struct PairSegment {
  int b, g, L, cb, ce;
  bool final_out;
  int64_t drow;
};

// Direct HBM -> LDS loads of one tile by role-1 wave bw (0 .. NP - 1),
// kPairLoads<NP, FP8> of them.  bf16: load k < 32 / NP is latent row
// bw + NP k, the rest the rope of the 8-row groups c = bw + NP j (rows
// 8c .. 8c + 7).  E4M3 (NP = 4): load k < 4 is latent rows pr = bw + 4k and
// pr + 16 (one 1056-byte block), the last one the rope of rows 16 bw ..
// 16 bw + 15 (bw < 2) or the tile's 32 token scales (bw >= 2; both such
// waves write the same bytes).  Rows at or past `valid` (slots past the
// request's end, which may hold anything) are loaded from row valid - 1
// instead: their scores are masked and their weights are exactly 0, so a
// finite duplicate row contributes nothing.  (Scales past the end are not
// replaced; the softmax zeroes those tokens' scales.)
template <int NP, bool FP8>
constexpr int kPairLoads = FP8 ? 16 / NP + 1 : 32 / NP + 4 / NP;
template <int NP, bool FP8>
__device__ __forceinline__ void pair_issue_piece(const char* tile_g, const float* scale_g, LDS_AS char* st, int bw,
                                                 int valid, int k) {
  using G = Tile<FP8>;
  const int lane = fresh_lane();
  if constexpr (!FP8) {
    if (k < 32 / NP) {
      const int r = bw + NP * k;  // wave-uniform
      const int rs = r < valid ? r : valid - 1;
      lds_dma16(tile_g, rs * G::kRowBytes + 16 * lane, lds_addr(st + G::lat_base(r)));
    } else {
      const int c8 = bw + NP * (k - 32 / NP);
      const int r = 8 * c8 + (lane >> 3);
      const int rs = r < valid ? r : valid - 1;
      const int c = (lane & 7) ^ G::xrope(r);
      lds_dma16(tile_g, rs * G::kRowBytes + G::kLat + 16 * c, lds_addr(st + G::kLatBytes + 1024 * c8));
    }
  } else {
    static_assert(NP == 4, "E4M3 tiles: four loading waves");
    if (k < 4) {
      const int pr = bw + 4 * k;
      const int r = pr + 16 * (lane >> 5);
      const int rs = r < valid ? r : valid - 1;
      const int c = (lane & 31) ^ G::xlat(r);
      lds_dma16(tile_g, rs * G::kRowBytes + 16 * c, lds_addr(st + pr * 1056));
    } else if (bw < 2) {
      const int r = 16 * bw + (lane >> 2);
      const int rs = r < valid ? r : valid - 1;
      const int c = (lane & 3) ^ G::xrope(r);
      lds_dma16(tile_g, rs * G::kRowBytes + G::kLat + 16 * c, lds_addr(st + G::kLatBytes + 1024 * bw));
    } else {
      lds_dma16(scale_g, 16 * (lane & 7), lds_addr(st + G::kLatBytes + G::kRopeBytes));
    }
  }
}
template <int NP, bool FP8>
__device__ __forceinline__ void pair_issue_tile(const char* tile_g, const float* scale_g, LDS_AS char* st, int bw,
                                                int valid) {
#pragma unroll
  for (int k = 0; k < kPairLoads<NP, FP8>; ++k) pair_issue_piece<NP, FP8>(tile_g, scale_g, st, bw, valid, k);
}

template <int NP, int ROLE, bool FP8>
__device__ __forceinline__ void pair_segment(const SplitParams& p, LDS_AS char* smem, const PairSegment& sg,
                                             int pair, int tid) {
  using G = Tile<FP8>;  // layout of the stages the MFMAs read
  using Lds = PairLds<NP, FP8>;
  constexpr int kRows = 32 * NP;  // rows of a workgroup
  constexpr int kBase = 18 * ROLE;  // first 16-dim step of this wave's half of the dot
  // Output columns: role 0 owns the 32-column blocks [0, 8), role 1 [8, 16).
  constexpr int kNB = 8;               // 32-column output blocks of this wave
  constexpr int kCol0 = ROLE ? 8 : 0;  // its first block
  const int M = p.T * p.H;
  const int b = sg.b, g = sg.g, L = sg.L, cb = sg.cb, ce = sg.ce;

  // ---- query fragments: the pair stages its 32 rows through LDS with
  // whole-row direct-to-LDS loads (role 0 latent rows 0..15, role 1 rows
  // 16..31 and the rope rows), then each wave reads the fragments of its half
  // of the dot.  Padding rows (gr >= M) reuse row M - 1 and are never written.
  bf16x8 qf[kQReg];
  {
    LDS_AS char* qst = smem + pair * kQRegion;
    LDS_AS char* qrs = qst + 32 * kRowPitch;
    const int64_t qrow0 = (int64_t)b * M;
    const int wr0 = g * kRows + 32 * pair;
    const int ql = fresh_lane();
#pragma unroll 4
    for (int r = 16 * ROLE; r < 16 * ROLE + 16; ++r) {
      const int rr = wr0 + r < M ? wr0 + r : M - 1;
      lds_dma16((const char*)p.q_abs + (qrow0 + rr) * 1024, 16 * ql, lds_addr(qst + r * kRowPitch));
    }
    if (ROLE == 1) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int rb = wr0 + 8 * j < M ? wr0 + 8 * j : M - 1;
        const int rl = wr0 + 8 * j + (ql >> 3) < M ? wr0 + 8 * j + (ql >> 3) : M - 1;
        lds_dma16((const char*)p.q_rope + (qrow0 + rb) * 128, (rl - rb) * 128 + 16 * (ql & 7),
                  lds_addr(qrs + 1024 * j));
      }
    }
    wait_vmcnt<0>();
    __syncthreads();
    const int ln = fresh_lane(), h = ln >> 5, n = ln & 31;
    bf16x8 kept[kQLds];
#pragma unroll
    for (int s = 0; s < 18; ++s) {
      const int kk = kBase + s;
      const bf16x8 f = kk < 32 ? *(const LDS_AS bf16x8*)(qst + n * kRowPitch + 2 * qfrag_dim<FP8>(kk, h))
                               : *(const LDS_AS bf16x8*)(qrs + n * 128 + 2 * qfrag_dim<FP8>(kk - 32, h));
      if (s < kQReg) qf[s] = f;
      else kept[s - kQReg] = f;
    }
    __syncthreads();  // every wave has its fragments before the stages refill
    // no restart requests, no partial scores yet (cleared only now: the query
    // staging may cover these words; the first step's barrier orders the
    // clear before every read)
    if (tid < 8) ((volatile LDS_AS uint32_t*)(smem + Lds::kRestart))[tid] = 0u;
    LDS_AS char* qkeep = smem + Lds::kQKeep + (pair + NP * ROLE) * (kQLds * 1024);
#pragma unroll
    for (int j = 0; j < kQLds; ++j) *(LDS_AS bf16x8*)(qkeep + 1024 * j + 16 * ln) = kept[j];
  }

  floatx16 acc[kNB];
  // role 0: softmax state of this lane's row.  p = 2^(s z - m_ref): m_ref is
  // the first tile's maximum and never moves while accumulating, so neither
  // wave ever rescales its accumulators.  A later tile maximum more than the
  // margin above it makes the whole workgroup run the segment again with
  // m_ref = the largest tile maximum seen (m_seen); real attention logits
  // never do.  l: the normaliser share of this lane half.
  float m_ref = neg_inf(), m_seen = neg_inf(), l_run = 0.0f;
  int lim = 0;  // tokens >= lim are masked for this lane's row
  if (ROLE == 0) {
    const int gr = g * kRows + 32 * pair + (fresh_lane() & 31);
    const int t = gr < M ? gr / p.H : 0;
    const int vis = p.causal ? (L - p.T + 1 + t) : L;
    lim = vis < ce ? vis : ce;
  }
  const float scale_log2 = p.scale * kLog2e;
  const int ntiles = (ce - cb + 31) >> 5;
  const char* kv = (const char*)p.kv;
  const int xs_off = Lds::kXchg + pair * kXchgSlot;  // the pair's exchange slot
  const int pr_slot = pair;
  const int qk_off = Lds::kQKeep + (pair + NP * ROLE) * (kQLds * 1024);

  // The scores of the tile in st: this wave's 18 dot steps, one MFMA chain,
  // key operands read from LDS a few steps ahead.  E4M3 tiles: one 16-byte
  // read per two steps (16 codes), converted to bf16 where used; each wave
  // converts only the half of the keys it scores.
  auto scores = [&](const LDS_AS char* st, floatx16& S) {
    const int ln = fresh_lane(), h = ln >> 5, n = ln & 31;
    const int rho = swap_bits23(n);  // tile row feeding A-operand slot n
    const LDS_AS char* qk = smem + qk_off + 16 * ln;
    constexpr int kAhead = 2;  // kept fragments are read this many steps before use
    bf16x8 qk_ring[kAhead];  // kept fragments in flight
    auto q_of = [&](int s) -> bf16x8 {  // this wave's query fragment of step s
      const bf16x8 q = s < kQReg ? qf[s < kQReg ? s : 0] : qk_ring[(s < kQReg ? 0 : s - kQReg) % kAhead];
      const int t = s + kAhead;  // the kept fragment read now
      if (t >= kQReg && t < 18) qk_ring[(t - kQReg) % kAhead] = *(const LDS_AS bf16x8*)(qk + 1024 * (t - kQReg));
      return q;
    };
    auto chain = [&](int s, const bf16x8& a, const bf16x8& q) {
      if (s == 0) mfma_v0(S, a, q);
      else if (s < 17) mfma_v(S, a, q);
      else mfma_v_last(S, a, q);
    };
    if constexpr (!FP8) {
      const LDS_AS char* kb = st + G::lat_base(rho) + 16 * h;
      const LDS_AS char* rb = st + G::kLatBytes + rho * 128;
      const int swr = G::xrope(rho);
      auto kread = [&](int kk) -> bf16x8 {
        return kk < 32 ? *(const LDS_AS bf16x8*)(kb + 32 * kk)
                       : *(const LDS_AS bf16x8*)(rb + 16 * ((2 * (kk - 32) + h) ^ swr));
      };
      constexpr int KR = 4;  // key fragments in flight
      bf16x8 kring[KR];
#pragma unroll
      for (int r = 0; r < KR; ++r) kring[r] = kread(kBase + r);
#pragma unroll
      for (int s = 0; s < 18; ++s) {
        const bf16x8 a = kring[s % KR];
        if (s + KR < 18) kring[s % KR] = kread(kBase + s + KR);
        chain(s, a, q_of(s));
        __builtin_amdgcn_sched_barrier(0);  // keep the operand rings as written
      }
    } else {
      // chunk c (16 codes of row rho): dims 32 c + 16 h .. + 15 for c < 16,
      // rope dims 32 (c - 16) + 16 h .. + 15 after; steps 2c and 2c + 1 take
      // its first and last eight (the query fragments hold the same dims)
      const LDS_AS char* kb = st + G::lat_base(rho) + 16 * (h ^ G::xlat(rho));
      const LDS_AS char* rb = st + G::kLatBytes + rho * G::kRope;
      const int swr = G::xrope(rho);
      auto kread = [&](int c) -> uintx4 {
        return c < 16 ? *(const LDS_AS uintx4*)(kb + 32 * c)
                      : *(const LDS_AS uintx4*)(rb + 16 * ((2 * (c - 16) + h) ^ swr));
      };
      constexpr int KR = 2;  // key chunks in flight (four steps)
      constexpr int kC0 = 9 * ROLE;  // this wave's first chunk
      uintx4 kring[KR];
#pragma unroll
      for (int r = 0; r < KR; ++r) kring[r] = kread(kC0 + r);
#pragma unroll
      for (int c = 0; c < 9; ++c) {
        const uintx4 raw = kring[c % KR];
        if (c + KR < 9) kring[c % KR] = kread(kC0 + c + KR);
        const bf16x8 a0 = e4m3x8_to_bf16(raw[0], raw[1]);
        const bf16x8 a1 = e4m3x8_to_bf16(raw[2], raw[3]);
        chain(2 * c, a0, q_of(2 * c));
        chain(2 * c + 1, a1, q_of(2 * c + 1));
        __builtin_amdgcn_sched_barrier(0);  // keep the operand rings as written
      }
    }
  };
  // This wave's half of the value product of the tile in sv with weights pw
  // (token 16q + 8h + j of this lane's row in pw[q][j]).  The value operand
  // of lane (lh, lsl) comes from rows r0 = 8 lh + (lsl >> 2) (+4, +16, +20)
  // of the tile: B(r0 + 4) = B(r0) + 273 and B(r0 + 16) = B(r0) + 1088
  // (r0 & 15 <= 11), so every read is one base register plus an immediate.
  // (hook(s) runs after value MFMA s: role 1 issues its tile loads there)
  auto values = [&](const LDS_AS char* sv, const bf16x8 (&pw)[2], auto&& hook) {
    constexpr int VR = 2;
    if constexpr (!FP8) {
      const int ln = fresh_lane(), lh = ln >> 5, lsl = ln & 15, ldh = (ln >> 4) & 1;
      const LDS_AS char* vb =
          sv + G::lat_base(8 * lh + (lsl >> 2)) + 16 * (2 * ldh + ((lsl & 3) >> 1)) + 8 * (lsl & 1);
      auto vread = [&](int x) -> bf16x8 {  // x: token half x / kNB, column block x % kNB
        const LDS_AS char* b0 = vb + 16 * 1088 * (x / kNB) + 64 * (kCol0 + x % kNB);
        const shortx4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS shortx4*)b0);
        const shortx4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS shortx4*)(b0 + 16 * 273));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      bf16x8 vring[VR];
#pragma unroll
      for (int r = 0; r < VR; ++r) vring[r] = vread(r);
#pragma unroll
      for (int s = 0; s < 2 * kNB; ++s) {
        const bf16x8 v = vring[s % VR];
        if (s + VR < 2 * kNB) vring[s % VR] = vread(s + VR);
        mfma_v(acc[s % kNB], v, pw[s / kNB]);
        hook(s);
      }
    } else {
      // E4M3: rows r0 = 8 lh + (lsl >> 1) and r0 + 16 share a block, 512 B
      // apart, with the same chunk swizzle; one 8-byte transposed read gives
      // eight tokens' codes of one column, converted where used
      const int ln = fresh_lane(), lsl = ln & 15, ldh = (ln >> 4) & 1;
      const int r0 = 8 * (ln >> 5) + (lsl >> 1);
      const LDS_AS char* vb = sv + G::lat_base(r0) + 16 * (ldh ^ G::xlat(r0)) + 8 * (lsl & 1);
      auto vread = [&](int x) -> intx2 {  // x: token half x / kNB, column block x % kNB
        return __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS intx2*)(vb + 512 * (x / kNB) + 32 * (kCol0 + x % kNB)));
      };
      intx2 vring[VR];
#pragma unroll
      for (int r = 0; r < VR; ++r) vring[r] = vread(r);
#pragma unroll
      for (int s = 0; s < 2 * kNB; ++s) {
        const intx2 v = vring[s % VR];
        if (s + VR < 2 * kNB) vring[s % VR] = vread(s + VR);
        mfma_v(acc[s % kNB], e4m3x8_to_bf16((unsigned)v[0], (unsigned)v[1]), pw[s / kNB]);
        hook(s);
      }
    }
  };
  auto no_hook = [](int) {};
  // Role 0, phase B: softmax of tile i from this wave's partial scores S and
  // the partner's (from the slot); writes the bf16 weights to the slot.
  // E4M3 (ts: the tile's 32 token scales in LDS, 8 copies; any copy
  // serves): the scores are code-domain dots times the token's scale, the
  // value product takes the weights times the scale and the normaliser the
  // weights alone.  The scales are read where used, eight at a time (registers
  // are scarce here); a masked token's weight stays 0 whatever its scale
  // (past the request's end it may hold anything).
  auto softmax = [&](auto with_mask, floatx16& S, const floatx4 (&sb)[4], int i, bf16x8 (&pw)[2],
                     const LDS_AS float* ts) {
    constexpr bool kMask = decltype(with_mask)::value;
    const int ln = fresh_lane();
    // token 16 (e >> 3) + 8 h + (e & 7) is visible iff 16 (e >> 3) + (e & 7)
    // < lim - (cb + 32 i) - 8 h: one bound, compared against immediates
    const int lim_h = lim - (cb + 32 * i) - 8 * (ln >> 5);
    auto scale8 = [&](int r, float (&sc)[8]) {  // scales of tokens 16 r + 8 h + j
      const floatx4 u0 = *(const LDS_AS floatx4*)(ts + 16 * r + 8 * (ln >> 5));
      const floatx4 u1 = *(const LDS_AS floatx4*)(ts + 16 * r + 8 * (ln >> 5) + 4);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        sc[c] = u0[c];
        sc[4 + c] = u1[c];
      }
    };
    float mx_a = neg_inf(), mx_b = neg_inf();
    float sc[8];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float v = S[e] + sb[e >> 2][e & 3];
      if constexpr (FP8) {
        if ((e & 7) == 0) scale8(e >> 3, sc);
        v *= sc[e & 7];
      }
      if constexpr (kMask) v = 16 * (e >> 3) + (e & 7) < lim_h ? v : neg_inf();
      S[e] = v;
      if (e & 1) mx_b = __builtin_fmaxf(mx_b, v);
      else mx_a = __builtin_fmaxf(mx_a, v);
    }
    // row maximum (both lane halves), times s = scale * log2 e > 0
    const float mx = half_swap_max(__builtin_fmaxf(mx_a, mx_b)) * scale_log2;
    if (m_ref == neg_inf()) m_ref = mx;  // first tile with a visible token: nothing accumulated yet
    m_seen = __builtin_fmaxf(m_seen, mx);
    // a maximum past the margin asks for a run with a larger reference (read
    // by every wave after the next barrier); this tile's weights are then unused
    if (__builtin_amdgcn_ballot_w64(mx > m_ref + kRescaleMargin) != 0 && ln == 0)
      *(volatile LDS_AS uint32_t*)(smem + Lds::kRestart + 4 * (xs_off - Lds::kXchg) / kXchgSlot) = 1u;
    const float mu = m_ref == neg_inf() ? 0.0f : m_ref;
#pragma unroll
    for (int e = 0; e < 16; ++e) pw[e >> 3][e & 7] = (__bf16)fast_exp2(__builtin_fmaf(S[e], scale_log2, -mu));
    // the normaliser sums the weights as the value product sees them (bf16),
    // two at a time
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    float la = 0.0f, lb = 0.0f;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      la = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pw[0][2 * d], pw[0][2 * d + 1]}, ones, la, false);
      lb = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pw[1][2 * d], pw[1][2 * d + 1]}, ones, lb, false);
    }
    l_run += la + lb;
    if constexpr (FP8) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        if ((e & 7) == 0) scale8(e >> 3, sc);
        float w = (float)pw[e >> 3][e & 7] * sc[e & 7];
        if constexpr (kMask) w = 16 * (e >> 3) + (e & 7) < lim_h ? w : 0.0f;
        pw[e >> 3][e & 7] = (__bf16)w;
      }
    }
    // slot: weights [0, 2048) (the partner's partial scores there were read above)
    LDS_AS char* xw = smem + xs_off + 16 * ln;
    *(LDS_AS bf16x8*)xw = pw[0];
    *(LDS_AS bf16x8*)(xw + 1024) = pw[1];
  };

  // ---- the tile loop, one workgroup barrier per step.  Step i: both waves
  // score tile i.  Role 1 first issues the loads of tile i + 1 (into the stage
  // tile i - 2 left); after its scores it hands over the partial scores, marks
  // them ready and goes straight on to its half of tile i - 1's value product.
  // Role 0 waits for the mark only, then runs the softmax of tile i and its
  // half of tile i's value product.
  // Role 1 reads the page of tile i + 2 during step i with a vector load (a
  // scalar one would be waited for at the next LDS wait): it lands with the
  // tile loads, which step i + 1 waits for anyway.
  auto entry_of = [&](int i) { return kv_page_entry(p.page_table, p.MP, p.P, b, cb + 32 * i); };
  auto row_at = [&](int i, int page) { return kv_row_of_page(page, p.P, cb + 32 * i); };
  auto tile_at = [&](int i, int page) { return kv + row_at(i, page) * G::kRowBytes; };
  auto scales_at = [&](int i, int page) { return FP8 ? p.kv_scales + row_at(i, page) : nullptr; };
  auto page_ahead = [&](int i) {  // entries of tiles past the last are never read
    return i < ntiles ? entry_of(i)[fresh_lane() >> 6] : 0;  // (lane >> 6 == 0: one vector load)
  };
  for (;;) {  // once, unless a tile asks for a larger softmax reference
#pragma unroll
    for (int db = 0; db < kNB; ++db) acc[db] = floatx16{};
    l_run = 0.0f;
    int pg_next = 0;  // role 1: page of tile i + 1 (in flight during step i - 1)
    if (ROLE == 1 && 0 < ntiles) {
      const int pg0 = uniform_load(entry_of(0));
      pair_issue_tile<NP, FP8>(tile_at(0, pg0), scales_at(0, pg0), smem, pair, L - cb);
      pg_next = page_ahead(1);
    }
    int so_cur = 0;  // stage offsets of tiles i and i - 1 (three stages, rotating)
    int so_prev = 2 * Lds::kCStage;
    bool restart = false;
    for (int i = 0; i <= ntiles; ++i) {
      if (ROLE == 1) wait_vmcnt<0>();  // tile i has landed
      __syncthreads();  // tile i is in its stage; every wave is done with step i - 1
      // requests made by the softmax of tile i - 1: read now, acted on after
      // the scores, so that the read's latency is not in front of them
      const uintx4 rq = *(const LDS_AS uintx4*)(smem + Lds::kRestart);
      const int so_next = so_cur == 2 * Lds::kCStage ? 0 : so_cur + Lds::kCStage;
      // (initialised here so that it is not carried from step to step)
      bf16x8 pw[2] = {bf16x8{}, bf16x8{}};  // role 0: the weights of tile i; role 1: those of tile i - 1
      // role 1: the weights of tile i - 1 from the slot, read after its scores
      // (not held through them) and before its partial scores overwrite the
      // slot (LDS serves one wave's accesses in order)
      auto read_weights = [&]() {
        if (ROLE == 1 && i >= 1) {
          const int ln = fresh_lane();
          pw[0] = *(const LDS_AS bf16x8*)(smem + xs_off + 16 * ln);
          pw[1] = *(const LDS_AS bf16x8*)(smem + xs_off + 1024 + 16 * ln);
        }
      };
      floatx16 S = __builtin_nondeterministic_value(S);  // defined by the scores when used
      if (i < ntiles) {
        scores(smem + so_cur, S);
        read_weights();
        if (ROLE == 1) {
          LDS_AS char* xw = smem + xs_off + 16 * fresh_lane();
#pragma unroll
          for (int k = 0; k < 4; ++k)
            *(LDS_AS floatx4*)(xw + 1024 * k) = floatx4{S[4 * k], S[4 * k + 1], S[4 * k + 2], S[4 * k + 3]};
          // (LDS carries one wave's accesses in order: the mark lands after the scores)
          *(volatile LDS_AS int*)(smem + Lds::kReady + 4 * pr_slot) = i + 1;
        }
      } else {
        read_weights();
      }
      if (__builtin_amdgcn_readfirstlane((int)(rq[0] | rq[1] | rq[2] | rq[3])) != 0) {
        restart = true;
        break;
      }
      if (ROLE == 0) {
        if (i == ntiles) break;
        // the partner's partial scores of tile i, read together with its
        // ready mark (one LDS round trip): LDS serves the partner's accesses
        // in order, so when the mark read sees tile i the reads after it see
        // the scores.  The partner is the older wave of the SIMD and usually
        // done first; otherwise read again until the mark shows (it marks
        // the scores right after its own score chain, so this wait ends).
        floatx4 sb[4];
        const volatile LDS_AS char* xs = smem + xs_off + 16 * fresh_lane();
        for (;;) {
          const int mark = *(const volatile LDS_AS int*)(smem + Lds::kReady + 4 * pr_slot);
#pragma unroll
          for (int k = 0; k < 4; ++k) sb[k] = *(const volatile LDS_AS floatx4*)(xs + 1024 * k);
          if (__builtin_amdgcn_readfirstlane(mark) > i) break;
          __builtin_amdgcn_s_sleep(1);
        }
        const LDS_AS float* ts = (const LDS_AS float*)(smem + so_cur + G::kLatBytes + G::kRopeBytes);
        const bool full = __builtin_amdgcn_ballot_w64(lim - (cb + 32 * i) < 32) == 0;
        if (__builtin_amdgcn_readfirstlane((int)full))
          softmax(std::false_type{}, S, sb, i, pw, ts);
        else
          softmax(std::true_type{}, S, sb, i, pw, ts);
        values(smem + so_cur, pw, no_hook);
      } else {
        // the loads of tile i + 1 go out between the value MFMAs of tile
        // i - 1: issuing them takes a while, and here no wave waits on it
        const bool load_next = i + 1 < ntiles;
        const int pgn = __builtin_amdgcn_readfirstlane(pg_next);
        const char* tg = tile_at(load_next ? i + 1 : 0, pgn);
        const float* sgl = scales_at(load_next ? i + 1 : 0, pgn);
        const int vnext = L - (cb + 32 * (i + 1));
        auto issue = [&](int k) {
          if (load_next && k < kPairLoads<NP, FP8>) pair_issue_piece<NP, FP8>(tg, sgl, smem + so_next, pair, vnext, k);
        };
        if (i >= 1) values(smem + so_prev, pw, issue);
        else issue(0);
#pragma unroll
        for (int k = i >= 1 ? 16 : 1; k < kPairLoads<NP, FP8>; ++k) issue(k);
        pg_next = page_ahead(i + 2);
        if (i == ntiles) break;
      }
      so_prev = so_cur;
      so_cur = so_next;
    }
    if (!restart) break;
    // rare path: every wave has read the requests before they are cleared;
    // the next run starts with the largest maximum seen as its reference
    mfma_drain();  // no value MFMA still writes the accumulators zeroed next
    wait_vmcnt<0>();  // the loads role 1 issued this step have landed
    __syncthreads();
    if (tid < 8) ((volatile LDS_AS uint32_t*)(smem + Lds::kRestart))[tid] = 0u;
    m_ref = m_seen;
  }

  // ---- epilogue: role 0 forms 1 / normaliser and lse and hands 1 / l to role 1
  mfma_drain();  // the last value MFMAs' results are in the accumulators
  int pr = pair;
  asm volatile("" : "+s"(pr));  // recomputed here, not kept through the loop
  const int ln = fresh_lane(), h = ln >> 5, n = ln & 31;
  LDS_AS char* xe = smem + Lds::kXchg + pr * kXchgSlot + 2304 + 4 * ln;
  float inv = 0.0f, lse_v = neg_inf();
  if (ROLE == 0) {
    const float l_tot = half_swap_sum(l_run);
    inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    lse_v = l_tot > 0.0f ? (m_ref + __log2f(l_tot)) * kLn2 : neg_inf();
    *(LDS_AS float*)xe = inv;
  }
  __syncthreads();
  if (ROLE == 1) inv = *(const LDS_AS float*)xe;
  int64_t drow = sg.drow;
  asm volatile("" : "+s"(drow));
  __syncthreads();  // the slots are read before the staging below overwrites them

  // The pair's rows go out through LDS: each wave writes its normalised
  // columns of the 32 rows at pitch kRowPitch, then each wave stores 16 whole
  // rows (role 0 rows 0..15, role 1 rows 16..31), 1 KB per store.
  LDS_AS char* wst = smem + pr * 32 * kRowPitch;
  const int wrow0 = g * kRows + 32 * pr;  // unit row of staged row 0
  auto stage_bf16 = [&]() {
#pragma unroll
    for (int db = 0; db < kNB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const floatx4 v = floatx4{acc[db][4 * g4], acc[db][4 * g4 + 1], acc[db][4 * g4 + 2], acc[db][4 * g4 + 3]} * inv;
        *(LDS_AS bf16x4*)(wst + n * kRowPitch + 2 * (32 * (kCol0 + db) + 8 * g4 + 4 * h)) =
            bf16x4{(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
      }
  };
  auto stage_f32 = [&](int half) {  // this wave's blocks among columns [256 half, 256 half + 256)
#pragma unroll
    for (int db = 0; db < kNB; ++db) {
      const int cb32 = kCol0 + db - 8 * half;
      if (cb32 < 0 || cb32 >= 8) continue;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const floatx4 v = floatx4{acc[db][4 * g4], acc[db][4 * g4 + 1], acc[db][4 * g4 + 2], acc[db][4 * g4 + 3]} * inv;
        *(LDS_AS floatx4*)(wst + n * kRowPitch + 4 * (32 * cb32 + 8 * g4 + 4 * h)) = v;
      }
    }
  };
  auto drain = [&](char* dst, int64_t row_bytes) {  // dst: staged row 0's destination
#pragma unroll 1
    for (int r0 = 16 * ROLE; r0 < 16 * ROLE + 16; r0 += 8) {
      uintx4 v[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) v[r] = *(const LDS_AS uintx4*)(wst + (r0 + r) * kRowPitch + 16 * ln);
#pragma unroll
      for (int r = 0; r < 8; ++r)
        if (wrow0 + r0 + r < M) *(uintx4*)(dst + (r0 + r) * row_bytes + 16 * ln) = v[r];
    }
  };
  const int64_t orow0 = drow + 32 * pr;
  if (sg.final_out && p.out_dtype == kBF16) {
    stage_bf16();
    __syncthreads();
    drain((char*)((__bf16*)p.out + orow0 * 512), 1024);
  } else if (!sg.final_out && p.NB > 0) {  // balanced slots hold bf16 partials
    stage_bf16();
    __syncthreads();
    drain((char*)((__bf16*)p.part_o + orow0 * 512), 1024);
  } else {
    float* base = sg.final_out ? (float*)p.out + orow0 * 512 : p.part_o + orow0 * 512;
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      stage_f32(pass);
      __syncthreads();
      drain((char*)(base + 256 * pass), 2048);
      __syncthreads();
    }
  }
  if (ROLE == 0 && h == 0 && wrow0 + n < M) {
    const int64_t orow = drow + 32 * pr + n;
    if (!sg.final_out) p.part_lse[orow] = lse_v;
    else if (p.lse) p.lse[orow] = lse_v;
  }
}

template <int NP, bool FP8>
__global__ void __launch_bounds__(128 * NP, 1)
mla_split_pair(SplitParams p, int groups) {
  using Lds = PairLds<NP, FP8>;
  constexpr int kWaves = 2 * NP;
  constexpr int kRows = 32 * NP;
  extern __shared__ __attribute__((aligned(1024))) char smem_raw[];
  LDS_AS char* smem = (LDS_AS char*)(LDS_AS void*)smem_raw;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  // Role 1 is the older wave of its SIMD: where both are ready to issue, the
  // older one goes first, so its score chain (which role 0 waits for) finishes
  // first.
  const int pair = wave & (NP - 1), role = 1 - wave / NP;

  // Work of this workgroup: a list of segments, each a run of 32-token tiles
  // of one unit (request b, row group g).
  //   Uniform chunks (p.NB == 0): one segment, chunk s of unit (b, g).  The
  //   block mapping is XCD-aware: consecutive hardware block ids go to
  //   different XCDs (id mod 8), so the row groups of one (request, chunk)
  //   are given ids 8 apart and share that XCD's L2 while they read the same
  //   pages.
  //   Balanced (p.NB > 0): the units' tiles, laid end to end (unit-major,
  //   each unit's preceded by kUnitStartCost positions for the cost of
  //   starting it; prefix sums in p.tile_prefix), are cut into NB equal
  //   contiguous ranges, one per workgroup; a range crosses unit boundaries
  //   freely, so every workgroup gets the same work whatever the length mix,
  //   a workgroup that starts a unit inside its range that many tiles fewer.
  int ub = 0, ug = 0, us = 0;
  int wx = 0, wx1 = 0;
  int wu = 0, wk = 0, wsu = 0;  // balanced: current unit and its first position
  if (p.NB == 0 && p.Sp > 0) {
    // Cascade: chunk s runs on XCD s mod 8, where its workgroups for every
    // request and row group take consecutive slots, so that the workgroups
    // reading one shared-prefix chunk run together and share that XCD's L2.
    const int x = blockIdx.x;
    const int xcd = x & 7, slot = x >> 3;
    const int per = p.B * groups;
    const int sl8 = slot / per, rem = slot - sl8 * per;
    us = 8 * sl8 + xcd;
    if (us >= p.S) return;
    ub = rem / groups;
    ug = rem - ub * groups;
  } else if (p.NB == 0) {
    const int x = blockIdx.x;
    const int xcd = x & 7, slot = x >> 3;
    const int k8 = slot / groups;
    ug = slot - k8 * groups;
    const int unit = 8 * k8 + xcd;
    if (unit >= p.B * p.S) return;
    ub = unit / p.S;
    us = unit - ub * p.S;
  } else {
    // Plan, in every workgroup: each thread sums the positions of a run of
    // units, a block-wide scan gives the runs' offsets, and the thread whose
    // run holds this workgroup's first position finds its unit.  Workgroup 0
    // also writes the prefix sums for the merge.  (The scratch words sit in
    // the exchange slots, unused until the first tile.)
    volatile LDS_AS int* ps = (volatile LDS_AS int*)(smem + Lds::kXchg);
    const int U = p.B * groups;
    const int per = (U + 64 * kWaves - 1) / (64 * kWaves);
    const int u0 = tid * per < U ? tid * per : U;
    const int u1 = u0 + per < U ? u0 + per : U;
    auto unit_tiles = [&](int u) {  // the unit's positions: tiles + start cost
      const int Lu = p.seq_lens[u / groups];
      return Lu > 0 ? ((Lu + 31) >> 5) + kUnitStartCost : 0;
    };
    int run_sum = 0;
    for (int u = u0; u < u1; ++u) run_sum += unit_tiles(u);
    int incl = run_sum;  // inclusive scan within the wave
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_up(incl, off, 64);
      if (lane >= off) incl += v;
    }
    if (lane == 63) ps[wave] = incl;
    __syncthreads();
    int W = 0, before = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const int v = ps[w];
      before += w < wave ? v : 0;
      W += v;
    }
    W = __builtin_amdgcn_readfirstlane(W);  // the same in every lane
    const int excl = before + incl - run_sum;
    if (blockIdx.x == 0) {
      int run = excl;
      for (int u = u0; u < u1; ++u) {
        p.tile_prefix[u] = run;
        run += unit_tiles(u);
      }
      if (tid == 0) p.tile_prefix[U] = W;
    }
    // no workgroup with an empty range (a range may still hold only a unit's
    // start positions: its workgroup then has no segment)
    const int64_t nb = W < p.NB ? W : p.NB;
    // Ranges are dealt so that each XCD (hardware block id mod 8; the grid
    // is NB workgroups) runs a contiguous run of NB / 8 of them: the few
    // workgroups that share a unit, and so read its query rows, mostly share
    // one L2.
    wk = (p.NB & 7) == 0 ? (int)(blockIdx.x & 7) * (p.NB >> 3) + (int)(blockIdx.x >> 3) : (int)blockIdx.x;
    if (wk >= nb) return;
    // (W < 2^30, so the bounds fit in int32; read back as wave-uniform values)
    wx = __builtin_amdgcn_readfirstlane((int)(wk * (int64_t)W / nb));
    wx1 = __builtin_amdgcn_readfirstlane((int)((wk + 1) * (int64_t)W / nb));
    if (excl <= wx && wx < excl + run_sum) {
      int run = excl, fu = u0, fr = excl;
      bool found = false;
      for (int u = u0; u < u1; ++u) {
        const int tu = unit_tiles(u);
        const bool hit = !found && wx < run + tu;
        fu = hit ? u : fu;
        fr = hit ? run : fr;
        found = found || hit;
        run += tu;
      }
      ps[kWaves] = fu;
      ps[kWaves + 1] = fr;
    }
    __syncthreads();
    wu = __builtin_amdgcn_readfirstlane(ps[kWaves]);
    wsu = __builtin_amdgcn_readfirstlane(ps[kWaves + 1]);
  }

  const int M = p.T * p.H;
  for (bool more_segments = true; more_segments;) {
    PairSegment sg;
    if (p.NB == 0) {
      more_segments = false;
      sg.b = ub;
      sg.g = ug;
      sg.L = uniform_load(p.seq_lens + ub);
      if (p.Sp == 0) {
        chunk_span(sg.L, p.S, p.P, us, &sg.cb, &sg.ce);
      } else if (us < p.Sp) {  // shared-prefix chunk: the same bounds for every request
        chunk_span(p.prefix_len, p.Sp, p.P, us, &sg.cb, &sg.ce);
        sg.cb = sg.cb < sg.L ? sg.cb : sg.L;
        sg.ce = sg.ce < sg.L ? sg.ce : sg.L;
      } else {  // suffix chunk of [prefix_len, L)
        const int Ls = sg.L > p.prefix_len ? sg.L - p.prefix_len : 0;
        chunk_span(Ls, p.S - p.Sp, p.P, us - p.Sp, &sg.cb, &sg.ce);
        sg.cb += p.prefix_len;
        sg.ce += p.prefix_len;
      }
      sg.final_out = p.write_final;
      sg.drow = sg.final_out ? (int64_t)ub * M + (int64_t)ug * kRows
                             : ((int64_t)ub * p.S + us) * M + (int64_t)ug * kRows;
    } else {
      // Unit wu occupies positions [su, eu): kUnitStartCost positions, then
      // its tiles from ts = su + kUnitStartCost on.
      int su = wsu, eu, L, b;
      for (;;) {  // skip units that end at or before wx (and units without tiles)
        b = wu / groups;
        L = uniform_load(p.seq_lens + b);
        eu = su + (L > 0 ? ((L + 31) >> 5) + kUnitStartCost : 0);
        if (eu > wx) break;
        ++wu;
        su = eu;
      }
      const int ts = su + kUnitStartCost;
      const int s0 = wx > ts ? (int)wx : ts;
      const int e = (int)(wx1 < eu ? wx1 : eu);
      if (s0 >= e) break;  // the range ends inside the unit's start cost: none of its tiles here
      sg.b = b;
      sg.L = L;
      sg.g = wu - b * groups;
      sg.cb = 32 * (s0 - ts);
      sg.ce = 32 * (e - ts);
      if (sg.ce > L) sg.ce = L;
      // Partial slots: [NB][2][kRows] rows.  Slot 0 holds the segment that
      // continues a unit begun in an earlier workgroup, slot 1 the one that
      // starts a unit and continues into later workgroups.
      sg.final_out = s0 == ts && e == eu;
      sg.drow = sg.final_out ? (int64_t)b * M + (int64_t)sg.g * kRows
                             : ((int64_t)wk * 2 + (s0 > ts ? 0 : 1)) * kRows;
      wx = e;
      ++wu;
      wsu = eu;
      more_segments = wx < wx1;
    }
    // the previous segment's waves are done with all of the LDS
    __syncthreads();
    if (role == 0)
      pair_segment<NP, 0, FP8>(p, smem, sg, pair, tid);
    else
      pair_segment<NP, 1, FP8>(p, smem, sg, pair, tid);
  }
}

template <int NP, bool FP8>
hipError_t launch_pair(const SplitParams& p, hipStream_t stream) {
  constexpr int kRows = 32 * NP;
  const int M = p.T * p.H;
  const int groups = (M + kRows - 1) / kRows;
  if (p.NB > 0 && kRows != kBalancedRows) return hipErrorInvalidValue;  // balanced units are 128 rows
  const int units = p.B * p.S;
  const int64_t blocks = p.NB > 0   ? (int64_t)p.NB
                         : p.Sp > 0 ? 8LL * ((p.S + 7) / 8) * p.B * groups  // cascade: chunk-major per XCD
                                    : 8LL * groups * ((units + 7) / 8);
  const size_t lds = (size_t)PairLds<NP, FP8>::kBytes;
  static std::once_flag once;
  static hipError_t attr_err = hipSuccess;
  std::call_once(once, [&] {
    attr_err = hipFuncSetAttribute((const void*)mla_split_pair<NP, FP8>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                   (int)lds);
  });
  if (attr_err != hipSuccess) return attr_err;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((mla_split_pair<NP, FP8>), dim3((unsigned)blocks), dim3(128 * NP), lds, stream, p,
                     groups);
  return hipGetLastError();
}

// ---------------------------------------------------- generic split kernel
// Any widths and dtypes, VALU only: one wavefront per query row, 64 tokens at
// a time (lane j scores token j), online softmax with wavefront reductions,
// then the latent accumulation with each lane owning columns lane + 64 k.
constexpr int kGenericMaxDc = 1024;

__device__ __forceinline__ float kv_value(const SplitParams& p, int64_t row, int d) {
  const int D = p.Dc + p.Dr;
  const int64_t i = row * D + d;
  if (p.kv_dtype == kF32) return ((const float*)p.kv)[i];
  if (p.kv_dtype == kBF16) return bf16_bits_to_float(((const uint16_t*)p.kv)[i]);
  return e4m3_to_float(((const uint8_t*)p.kv)[i]) * p.kv_scales[row];
}

__device__ __forceinline__ float q_value(const SplitParams& p, const void* base, int64_t i) {
  return p.q_dtype == kF32 ? ((const float*)base)[i] : bf16_bits_to_float(((const uint16_t*)base)[i]);
}

__global__ void __launch_bounds__(256) mla_split_generic(SplitParams p) {
  extern __shared__ float gsm[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int M = p.T * p.H, D = p.Dc + p.Dr;
  const int gr = blockIdx.x * 4 + wave;
  const int s = blockIdx.y, b = blockIdx.z;
  if (gr >= M) return;
  float* q = gsm + wave * D;
  for (int d = lane; d < p.Dc; d += 64) q[d] = q_value(p, p.q_abs, ((int64_t)b * M + gr) * p.Dc + d);
  for (int e = lane; e < p.Dr; e += 64) q[p.Dc + e] = q_value(p, p.q_rope, ((int64_t)b * M + gr) * p.Dr + e);
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");

  const int t = gr / p.H;
  const int L = p.seq_lens[b];
  int cb, ce;
  chunk_span(L, p.S, p.P, s, &cb, &ce);
  const int vis = p.causal ? (L - p.T + 1 + t) : L;
  const int lim = vis < ce ? vis : ce;
  const float scale_log2 = p.scale * kLog2e;
  constexpr int kPer = kGenericMaxDc / 64;
  float acc[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) acc[k] = 0.0f;
  float m = neg_inf(), l = 0.0f;
  for (int j0 = cb; j0 < lim; j0 += 64) {
    const int j = j0 + lane;
    const bool ok = j < lim;
    const int64_t row = ok ? kv_row_index(p.page_table, p.MP, p.P, b, j) : 0;
    float z = neg_inf();
    if (ok) {
      float dot = 0.0f;
      for (int d = 0; d < D; ++d) dot += q[d] * kv_value(p, row, d);
      z = dot * scale_log2;
    }
    const float mx = wave_max(z);
    const float m_new = fmaxf(m, mx);
    const float alpha = m == neg_inf() ? 0.0f : fast_exp2(m - m_new);
    const float pj = ok ? fast_exp2(z - m_new) : 0.0f;
    l = l * alpha + wave_sum(pj);
#pragma unroll
    for (int k = 0; k < kPer; ++k) acc[k] *= alpha;
    m = m_new;
    const int cnt = lim - j0 < 64 ? lim - j0 : 64;
    for (int jj = 0; jj < cnt; ++jj) {
      const float w = __shfl(pj, jj, 64);
      const int64_t r = ((int64_t)__shfl((int)(row >> 32), jj, 64) << 32) |
                        (uint32_t)__shfl((int)(row & 0xffffffff), jj, 64);
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const int d = lane + 64 * k;
        if (d < p.Dc) acc[k] += w * kv_value(p, r, d);
      }
    }
  }
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  const float lse_v = l > 0.0f ? (m + __log2f(l)) * kLn2 : neg_inf();
  if (p.write_final) {
    const int64_t ob = ((int64_t)b * M + gr) * p.Dc;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int d = lane + 64 * k;
      if (d < p.Dc) {
        if (p.out_dtype == kBF16) ((__bf16*)p.out)[ob + d] = (__bf16)(acc[k] * inv);
        else ((float*)p.out)[ob + d] = acc[k] * inv;
      }
    }
    if (p.lse && lane == 0) p.lse[(int64_t)b * M + gr] = lse_v;
  } else {
    const int64_t prow = ((int64_t)b * p.S + s) * M + gr;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int d = lane + 64 * k;
      if (d < p.Dc) p.part_o[prow * p.Dc + d] = acc[k] * inv;
    }
    if (lane == 0) p.part_lse[prow] = lse_v;
  }
}

// ----------------------------------------------------------- combine kernel
// Log-sum-exp merge of one output row (one wavefront) from ns partial rows,
// partial j at row slot_row(j) of po / pl: M = max_j lse_j, w_j =
// exp(lse_j - M), out = sum_j w_j o_j / sum_j w_j, lse = M + ln sum_j w_j.
// Partials with lse = -inf weigh nothing (their rows may hold anything, NaN
// included); with none left, out = 0 and lse = -inf.  The normalised weights of 64 partials
// at a time sit one per lane and are broadcast by shuffles, and each lane
// accumulates 8 columns, so several partial rows are in flight per wave.
__device__ __forceinline__ floatx4 load4(const float* p) { return *(const floatx4*)p; }
__device__ __forceinline__ floatx4 load4(const __bf16* p) {
  const bf16x4 v = *(const bf16x4*)p;
  return floatx4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}

template <typename PT, typename SlotRow>
__device__ __forceinline__ void merge_row(int ns, int Dc, SlotRow slot_row, const PT* __restrict__ po,
                                          const float* __restrict__ pl, int out_dtype, void* out,
                                          int64_t out_row, float* lse) {
  const int lane = threadIdx.x & 63;
  float mx = neg_inf();
  for (int j = lane; j < ns; j += 64) mx = fmaxf(mx, pl[slot_row(j)]);
  mx = wave_max(mx);
  float wsum = 0.0f;
  for (int j = lane; j < ns; j += 64) {
    const float v = pl[slot_row(j)];
    wsum += v == neg_inf() ? 0.0f : fast_exp2((v - mx) * kLog2e);
  }
  wsum = wave_sum(wsum);
  const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
  const int64_t ob = out_row * Dc;
  auto put4 = [&](int d, floatx4 a) {
    if (out_dtype == kBF16)
      *(bf16x4*)((__bf16*)out + ob + d) = bf16x4{(__bf16)a[0], (__bf16)a[1], (__bf16)a[2], (__bf16)a[3]};
    else
      *(floatx4*)((float*)out + ob + d) = a;
  };
  if ((Dc & 3) == 0) {
    for (int d0 = 0; d0 < Dc; d0 += 512) {
      const int da = d0 + 4 * lane, db = da + 256;
      const bool oka = da < Dc, okb = db < Dc;
      floatx4 a = floatx4{0.0f, 0.0f, 0.0f, 0.0f}, c = a;
      for (int j0 = 0; j0 < ns; j0 += 64) {
        float wj = 0.0f;
        if (j0 + lane < ns) {
          const float v = pl[slot_row(j0 + lane)];
          wj = v == neg_inf() ? 0.0f : fast_exp2((v - mx) * kLog2e) * inv;
        }
        const int cnt = ns - j0 < 64 ? ns - j0 : 64;
        // four partial rows per round, all loads issued before the first
        // use; every slot row lies inside the partial buffer, so rows are
        // read unconditionally (a round past the end re-reads the last one)
        // and a zero-weight row is dropped by a select, never multiplied in
        for (int jj = 0; jj < cnt; jj += 4) {
          floatx4 x[4], y[4];
          float w[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int j = jj + q < cnt ? jj + q : cnt - 1;
            w[q] = jj + q < cnt ? __shfl(wj, j, 64) : 0.0f;
            const PT* row = po + slot_row(j0 + j) * Dc;
            x[q] = oka ? load4(row + da) : floatx4{};
            y[q] = okb ? load4(row + db) : floatx4{};
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const bool live = w[q] != 0.0f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              a[e] = live ? __builtin_fmaf(w[q], x[q][e], a[e]) : a[e];
              c[e] = live ? __builtin_fmaf(w[q], y[q][e], c[e]) : c[e];
            }
          }
        }
      }
      if (oka) put4(da, a);
      if (okb) put4(db, c);
    }
  } else {
    for (int d = lane; d < Dc; d += 64) {
      float a = 0.0f;
      for (int j = 0; j < ns; ++j) {
        const float v = pl[slot_row(j)];
        if (v == neg_inf()) continue;
        a += fast_exp2((v - mx) * kLog2e) * inv * (float)po[slot_row(j) * Dc + d];
      }
      if (out_dtype == kBF16) ((__bf16*)out)[ob + d] = (__bf16)a;
      else ((float*)out)[ob + d] = a;
    }
  }
  if (lse && lane == 0) lse[out_row] = wsum > 0.0f ? mx + __logf(wsum) : neg_inf();
}

// Uniform plan: partials [B, S, rows, Dc] / [B, S, rows]; one wavefront per
// (request, row).
__global__ void __launch_bounds__(256)
mla_combine_kernel(int B, int S, int rows, int Dc, const float* __restrict__ po,
                   const float* __restrict__ pl, int out_dtype, void* out, float* lse) {
  const int wave = threadIdx.x >> 6;
  const int64_t idx = (int64_t)blockIdx.x * 4 + wave;
  if (idx >= (int64_t)B * rows) return;
  const int b = (int)(idx / rows), r = (int)(idx - (int64_t)b * rows);
  merge_row(S, Dc, [&](int k) { return ((int64_t)b * S + k) * rows + r; }, po, pl, out_dtype, out,
            idx, lse);
}

// ------------------------------------------------------- balanced merge
// Merge for the balanced work list (same arithmetic as mla_combine_kernel).
// With W positions cut into nb = min(NB, W) ranges [k W / nb, (k+1) W / nb),
// position x lies in range ceil((x+1) nb / W) - 1.  A unit at positions
// [su, eu) has its tiles at [su + kUnitStartCost, eu); when they lie in
// ranges k1 < k2 its partials are in slot 1 of workgroup k1 and in slot 0 of
// workgroups k1+1 .. k2 (slot rows [k][2][kBalancedRows]).  One wave per
// output row.
__global__ void __launch_bounds__(256)
mla_combine_balanced_kernel(int B, int M, int Dc, int NB, const int32_t* __restrict__ prefix,
                            const __bf16* __restrict__ po, const float* __restrict__ pl,
                            int out_dtype, void* out, float* lse) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t idx = (int64_t)blockIdx.x * 4 + wave;
  if (idx >= (int64_t)B * M) return;
  const int b = (int)(idx / M), r = (int)(idx - (int64_t)b * M);
  const int groups = (M + kBalancedRows - 1) / kBalancedRows;
  const int g = r / kBalancedRows, lr = r - g * kBalancedRows;
  const int u = b * groups + g;
  const int64_t W = prefix[B * groups];
  const int64_t su = prefix[u], eu = prefix[u + 1];
  const int64_t ob = idx * Dc;
  auto store = [&](int d, float a) {
    if (out_dtype == kBF16) ((__bf16*)out)[ob + d] = (__bf16)a;
    else ((float*)out)[ob + d] = a;
  };
  if (su == eu) {  // no visible token: out = 0, lse = -inf
    for (int d = lane; d < Dc; d += 64) store(d, 0.0f);
    if (lse && lane == 0) lse[idx] = neg_inf();
    return;
  }
  const int64_t nb = W < NB ? W : NB;
  const int k1 = (int)(((su + kUnitStartCost + 1) * nb + W - 1) / W - 1);  // range of the first tile
  const int k2 = (int)((eu * nb + W - 1) / W - 1);
  if (k1 == k2) return;  // written by the split kernel
  const int ns = k2 - k1 + 1;
  merge_row(ns, Dc,
            [&](int j) -> int64_t {
              const int64_t slot = j == 0 ? 2LL * k1 + 1 : 2LL * (k1 + j);
              return slot * kBalancedRows + lr;
            },
            po, pl, out_dtype, out, idx, lse);
}

// Balanced-plan merge, four rows per wavefront (M a multiple of 4 and Dc a
// multiple of 8; the rows share their unit and so their slots).  A merge of
// one row per wavefront spends its life waiting on three dependent loads
// (tile prefix, slot lse, slot rows) with a few KB in flight; four rows per
// wave put 4x the rows' loads in flight behind the same waits and quarter
// the number of waves.  Each lane owns 8 consecutive columns of the four
// rows; partial rows are read four slots at a time as raw bf16, a zero-weight
// slot is dropped by a select (its row may hold anything).
constexpr int kMergeRows = 4;

__global__ void __launch_bounds__(256)
mla_combine_balanced4_kernel(int B, int M, int Dc, int NB, const int32_t* __restrict__ prefix,
                             const __bf16* __restrict__ po, const float* __restrict__ pl, int out_dtype,
                             void* out, float* lse) {
  const int lane = threadIdx.x & 63;
  const int64_t idx0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * kMergeRows;
  if (idx0 >= (int64_t)B * M) return;
  const int b = (int)(idx0 / M), r0 = (int)(idx0 - (int64_t)b * M);
  const int groups = (M + kBalancedRows - 1) / kBalancedRows;
  const int g = r0 / kBalancedRows, lr0 = r0 - g * kBalancedRows;
  const int u = b * groups + g;
  const int64_t W = prefix[B * groups];
  const int64_t su = prefix[u], eu = prefix[u + 1];
  if (su == eu) {  // no visible token: out = 0, lse = -inf
    for (int rr = 0; rr < kMergeRows; ++rr) {
      const int64_t ob = (idx0 + rr) * Dc;
      for (int d = lane; d < Dc; d += 64) {
        if (out_dtype == kBF16) ((__bf16*)out)[ob + d] = (__bf16)0.0f;
        else ((float*)out)[ob + d] = 0.0f;
      }
      if (lse && lane == 0) lse[idx0 + rr] = neg_inf();
    }
    return;
  }
  const int64_t nb = W < NB ? W : NB;
  const int k1 = (int)(((su + kUnitStartCost + 1) * nb + W - 1) / W - 1);  // range of the first tile
  const int k2 = (int)((eu * nb + W - 1) / W - 1);
  if (k1 == k2) return;  // written by the split kernel
  const int ns = k2 - k1 + 1;
  auto slot_row = [&](int j) -> int64_t {  // row lr0 of partial j's slot
    const int64_t slot = j == 0 ? 2LL * k1 + 1 : 2LL * (k1 + j);
    return slot * kBalancedRows + lr0;
  };
  auto weight = [](float v, float mx) { return v == neg_inf() ? 0.0f : fast_exp2((v - mx) * kLog2e); };
  // Few partials (a unit spread over at most kFewSlots workgroups) and
  // Dc <= 512: the partials' lse and all their rows are requested together
  // right after the tile prefix, so the wave waits on one dependent round of
  // loads instead of one for the lse and one per four partials; partials past
  // ns are not read.  Same arithmetic, in the same order, as the general path.
  constexpr int kFewSlots = 8;
  if (ns <= kFewSlots && Dc <= 512) {
    const int d = 8 * lane;
    const bool ok = d < Dc;
    float v[kMergeRows];
#pragma unroll
    for (int rr = 0; rr < kMergeRows; ++rr) v[rr] = lane < ns ? pl[slot_row(lane) + rr] : neg_inf();
    bf16x8 raw[kFewSlots][kMergeRows];
#pragma unroll
    for (int j = 0; j < kFewSlots; ++j) {
      const __bf16* row = po + slot_row(j < ns ? j : 0) * Dc + d;
#pragma unroll
      for (int rr = 0; rr < kMergeRows; ++rr)
        raw[j][rr] = ok && j < ns ? *(const bf16x8*)(row + (int64_t)rr * Dc) : bf16x8{};
    }
    float m[kMergeRows], ws[kMergeRows], wl[kMergeRows], acc[kMergeRows][8];
#pragma unroll
    for (int rr = 0; rr < kMergeRows; ++rr) {
      m[rr] = wave_max(v[rr]);
      const float w = weight(v[rr], m[rr]);
      ws[rr] = wave_sum(w);
      wl[rr] = w * (ws[rr] > 0.0f ? 1.0f / ws[rr] : 0.0f);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[rr][e] = 0.0f;
    }
#pragma unroll
    for (int j = 0; j < kFewSlots; ++j) {
      if (j >= ns) break;
#pragma unroll
      for (int rr = 0; rr < kMergeRows; ++rr) {
        const float w = __shfl(wl[rr], j, 64);
        const bool live = w != 0.0f;  // a zero-weight partial's row may hold anything
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[rr][e] = live ? __builtin_fmaf(w, (float)raw[j][rr][e], acc[rr][e]) : acc[rr][e];
      }
    }
    if (ok) {
#pragma unroll
      for (int rr = 0; rr < kMergeRows; ++rr) {
        const int64_t ob = (idx0 + rr) * Dc + d;
        if (out_dtype == kBF16) {
          bf16x8 o;
#pragma unroll
          for (int e = 0; e < 8; ++e) o[e] = (__bf16)acc[rr][e];
          *(bf16x8*)((__bf16*)out + ob) = o;
        } else {
          *(floatx4*)((float*)out + ob) = floatx4{acc[rr][0], acc[rr][1], acc[rr][2], acc[rr][3]};
          *(floatx4*)((float*)out + ob + 4) = floatx4{acc[rr][4], acc[rr][5], acc[rr][6], acc[rr][7]};
        }
      }
    }
    if (lse && lane == 0) {
#pragma unroll
      for (int rr = 0; rr < kMergeRows; ++rr) lse[idx0 + rr] = ws[rr] > 0.0f ? m[rr] + __logf(ws[rr]) : neg_inf();
    }
    return;
  }
  // lane j holds the four rows' lse of partial j (the first 64; more are re-read)
  float v0[kMergeRows], mx[kMergeRows], inv[kMergeRows], w0[kMergeRows], wsum[kMergeRows];
#pragma unroll
  for (int rr = 0; rr < kMergeRows; ++rr) v0[rr] = lane < ns ? pl[slot_row(lane) + rr] : neg_inf();
#pragma unroll
  for (int rr = 0; rr < kMergeRows; ++rr) {
    float m = v0[rr];
    for (int j = lane + 64; j < ns; j += 64) m = fmaxf(m, pl[slot_row(j) + rr]);
    mx[rr] = wave_max(m);
    w0[rr] = weight(v0[rr], mx[rr]);
    float sm = w0[rr];
    for (int j = lane + 64; j < ns; j += 64) sm += weight(pl[slot_row(j) + rr], mx[rr]);
    wsum[rr] = wave_sum(sm);
    inv[rr] = wsum[rr] > 0.0f ? 1.0f / wsum[rr] : 0.0f;
  }
  for (int d0 = 0; d0 < Dc; d0 += 512) {
    const int d = d0 + 8 * lane;
    const bool ok = d < Dc;
    float acc[kMergeRows][8];
#pragma unroll
    for (int rr = 0; rr < kMergeRows; ++rr)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[rr][e] = 0.0f;
    for (int j0 = 0; j0 < ns; j0 += 64) {
      float wj[kMergeRows];
#pragma unroll
      for (int rr = 0; rr < kMergeRows; ++rr)
        wj[rr] = (j0 == 0 ? w0[rr] : (j0 + lane < ns ? weight(pl[slot_row(j0 + lane) + rr], mx[rr]) : 0.0f)) *
                 inv[rr];
      const int cnt = ns - j0 < 64 ? ns - j0 : 64;
      for (int jj = 0; jj < cnt; jj += 4) {
        bf16x8 raw[4][kMergeRows];
        float w[4][kMergeRows];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int j = jj + q < cnt ? jj + q : cnt - 1;  // past the end: re-read the last, weight 0
          const __bf16* row = po + slot_row(j0 + j) * Dc + d;
#pragma unroll
          for (int rr = 0; rr < kMergeRows; ++rr) {
            w[q][rr] = jj + q < cnt ? __shfl(wj[rr], j, 64) : 0.0f;
            raw[q][rr] = ok ? *(const bf16x8*)(row + (int64_t)rr * Dc) : bf16x8{};
          }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int rr = 0; rr < kMergeRows; ++rr) {
            const bool live = w[q][rr] != 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e)
              acc[rr][e] = live ? __builtin_fmaf(w[q][rr], (float)raw[q][rr][e], acc[rr][e]) : acc[rr][e];
          }
      }
    }
    if (ok) {
#pragma unroll
      for (int rr = 0; rr < kMergeRows; ++rr) {
        const int64_t ob = (idx0 + rr) * Dc + d;
        if (out_dtype == kBF16) {
          bf16x8 o;
#pragma unroll
          for (int e = 0; e < 8; ++e) o[e] = (__bf16)acc[rr][e];
          *(bf16x8*)((__bf16*)out + ob) = o;
        } else {
          *(floatx4*)((float*)out + ob) = floatx4{acc[rr][0], acc[rr][1], acc[rr][2], acc[rr][3]};
          *(floatx4*)((float*)out + ob + 4) = floatx4{acc[rr][4], acc[rr][5], acc[rr][6], acc[rr][7]};
        }
      }
    }
  }
  if (lse && lane == 0) {
#pragma unroll
    for (int rr = 0; rr < kMergeRows; ++rr) lse[idx0 + rr] = wsum[rr] > 0.0f ? mx[rr] + __logf(wsum[rr]) : neg_inf();
  }
}

// Balanced-plan merge for units that span many workgroups (a few long
// requests): the partials of a row-quad are spread over WV = 2, 4 or 8
// wavefronts (M a multiple of 4, Dc a multiple of 8 and at most 512).  Every
// wavefront reads the four rows' lse of the first 64 partials (lane j holds
// partial j) and, in the same round trip, the rows of its own share of the
// partials (j = wave, wave + WV, ...; eight partials in flight), so a
// row-quad costs two dependent memory round trips (tile prefix, then lse
// plus rows) when it has at most 8 WV partials; the wavefronts' sums are
// added through LDS.  Same weights as the kernels above (normalised once per
// row); the partials are summed in a different order.
constexpr int kWideSlotsInFlight = 8;

template <int WV>
struct WideMerge {
  static_assert(WV == 2 || WV == 4 || WV == 8, "two, four or eight wavefronts per row-quad");
  static constexpr int kQuads = WV >= 4 ? 1 : 4 / WV;  // row-quads per workgroup
  static constexpr int kThreads = kQuads * WV * 64;
  static constexpr int kRed = kQuads * WV * kMergeRows * 512;  // floats of LDS
};

template <int WV>
__global__ void __launch_bounds__(WideMerge<WV>::kThreads)
mla_combine_balanced_wide_kernel(int B, int M, int Dc, int NB, const int32_t* __restrict__ prefix,
                                 const __bf16* __restrict__ po, const float* __restrict__ pl, int out_dtype,
                                 void* out, float* lse) {
  using G = WideMerge<WV>;
  __shared__ float red[G::kRed];  // [quad][wavefront][row][column]
  const int lane = threadIdx.x & 63;
  const int quad = (threadIdx.x >> 6) / WV, wave = (threadIdx.x >> 6) % WV;
  const int64_t idx0 = ((int64_t)blockIdx.x * G::kQuads + quad) * kMergeRows;  // the quad's first row
  const int d = 8 * lane;
  const bool ok = d < Dc;
  bool merged = false;  // this quad's rows are written by this kernel from partials
  float mx[kMergeRows], wsum[kMergeRows];
  float acc[kMergeRows][8];
#pragma unroll
  for (int rr = 0; rr < kMergeRows; ++rr) {
    mx[rr] = neg_inf();
    wsum[rr] = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[rr][e] = 0.0f;
  }
  if (idx0 < (int64_t)B * M) {
    const int b = (int)(idx0 / M), r0 = (int)(idx0 - (int64_t)b * M);
    const int groups = (M + kBalancedRows - 1) / kBalancedRows;
    const int g = r0 / kBalancedRows, lr0 = r0 - g * kBalancedRows;
    const int u = b * groups + g;
    const int64_t W = prefix[B * groups];
    const int64_t su = prefix[u], eu = prefix[u + 1];
    const int64_t nb = W < NB ? W : NB;
    const int k1 = su == eu ? 0 : (int)(((su + kUnitStartCost + 1) * nb + W - 1) / W - 1);
    const int k2 = su == eu ? 0 : (int)((eu * nb + W - 1) / W - 1);
    if (su == eu) {  // no visible token: out = 0, lse = -inf (wavefront 0 of the quad)
      if (wave == 0) {
        for (int rr = 0; rr < kMergeRows; ++rr) {
          const int64_t ob = (idx0 + rr) * Dc;
          for (int c = lane; c < Dc; c += 64) {
            if (out_dtype == kBF16) ((__bf16*)out)[ob + c] = (__bf16)0.0f;
            else ((float*)out)[ob + c] = 0.0f;
          }
        }
        if (lse && lane < kMergeRows) lse[idx0 + lane] = neg_inf();
      }
    } else if (k1 != k2) {  // k1 == k2: written by the split kernel
      merged = true;
      const int ns = k2 - k1 + 1;
      auto slot_row = [&](int j) -> int64_t {  // row lr0 of partial j's slot
        const int64_t slot = j == 0 ? 2LL * k1 + 1 : 2LL * (k1 + j);
        return slot * kBalancedRows + lr0;
      };
      auto weight = [](float v, float m) { return v == neg_inf() ? 0.0f : fast_exp2((v - m) * kLog2e); };
      float l0[kMergeRows];  // lse of partial `lane` (first 64 partials)
      {
        const int64_t row = slot_row(lane < ns ? lane : 0);
#pragma unroll
        for (int rr = 0; rr < kMergeRows; ++rr) l0[rr] = lane < ns ? pl[row + rr] : neg_inf();
      }
      bf16x8 raw[kWideSlotsInFlight][kMergeRows];
      auto load_batch = [&](int jb) {
#pragma unroll
        for (int q = 0; q < kWideSlotsInFlight; ++q) {
          const int j = jb + WV * q;
          const bool live = ok && j < ns;
          const int64_t row = slot_row(j < ns ? j : 0);
#pragma unroll
          for (int rr = 0; rr < kMergeRows; ++rr)
            raw[q][rr] = live ? *(const bf16x8*)(po + (row + rr) * Dc + d) : bf16x8{};
        }
      };
      load_batch(wave);  // in flight with the lse loads
      float inv[kMergeRows], wl[kMergeRows];
#pragma unroll
      for (int rr = 0; rr < kMergeRows; ++rr) {
        float m = l0[rr];
        for (int j = lane + 64; j < ns; j += 64) m = fmaxf(m, pl[slot_row(j) + rr]);
        mx[rr] = wave_max(m);
        float sm = weight(l0[rr], mx[rr]);
        for (int j = lane + 64; j < ns; j += 64) sm += weight(pl[slot_row(j) + rr], mx[rr]);
        wsum[rr] = wave_sum(sm);
        inv[rr] = wsum[rr] > 0.0f ? 1.0f / wsum[rr] : 0.0f;
        wl[rr] = weight(l0[rr], mx[rr]) * inv[rr];  // weight of partial `lane`
      }
      for (int jb = wave;;) {
#pragma unroll
        for (int q = 0; q < kWideSlotsInFlight; ++q) {
          const int j = jb + WV * q;
          if (j >= ns) break;  // uniform over the wavefront
#pragma unroll
          for (int rr = 0; rr < kMergeRows; ++rr) {
            const float w = j < 64 ? __shfl(wl[rr], j, 64) : weight(pl[slot_row(j) + rr], mx[rr]) * inv[rr];
            if (w != 0.0f) {  // a zero-weight partial's row may hold anything
#pragma unroll
              for (int e = 0; e < 8; ++e) acc[rr][e] = __builtin_fmaf(w, (float)raw[q][rr][e], acc[rr][e]);
            }
          }
        }
        jb += WV * kWideSlotsInFlight;
        if (jb >= ns) break;
        load_batch(jb);
      }
    }
  }
  {
    float* qred = red + quad * (WV * kMergeRows * 512);
    if (merged && ok) {
#pragma unroll
      for (int rr = 0; rr < kMergeRows; ++rr)
#pragma unroll
        for (int e = 0; e < 8; ++e) qred[(wave * kMergeRows + rr) * 512 + d + e] = acc[rr][e];
    }
    __syncthreads();  // reached by every thread: no early return above
    if (merged) {
      // the quad's threads finish 4 rows x 128 column-quads
      for (int it = wave * 64 + lane; it < kMergeRows * 128; it += WV * 64) {
        const int rr = it >> 7, c = 4 * (it & 127);
        if (c >= Dc) continue;
        float a[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float s = 0.0f;
#pragma unroll
          for (int v = 0; v < WV; ++v) s += qred[(v * kMergeRows + rr) * 512 + c + e];
          a[e] = s;
        }
        const int64_t ob = (idx0 + rr) * Dc + c;
        if (out_dtype == kBF16) {
          *(bf16x4*)((__bf16*)out + ob) = bf16x4{(__bf16)a[0], (__bf16)a[1], (__bf16)a[2], (__bf16)a[3]};
        } else {
          *(floatx4*)((float*)out + ob) = floatx4{a[0], a[1], a[2], a[3]};
        }
      }
    }
  }
  if (merged && lse && wave == 0 && lane == 0) {
#pragma unroll
    for (int rr = 0; rr < kMergeRows; ++rr) lse[idx0 + rr] = wsum[rr] > 0.0f ? mx[rr] + __logf(wsum[rr]) : neg_inf();
  }
}

// ------------------------------------------------------------- KV append
// Paged KV append with packing: token t of request b is stored at logical
// position pos[b] + t, i.e. page page_table[b][pos / P], slot pos mod P
// (PagedAttention article on the "推理优化" tag page), as fp32, as bf16
// (nearest, ties to even) or as OCP E4M3 codes with one fp32 scale per row:
// s = absmax / 448 (448 = largest finite E4M3, FP8 format table of the
// quantisation article on the same page; s = 1 for an all-zero row) and each
// value v stored as the E4M3 code nearest to v / s, ties to even, magnitudes
// past 448 saturating, the sign kept.

// E4M3 code of an fp32 value: below 2^-6 the format's values are the
// multiples of 2^-9 (codes 0..8 per sign, 8 being 2^-6 itself); from 2^e
// (e = -6..8) on the step is 2^(e-3) and the code is (e + 7) << 3 | mantissa.
__device__ __forceinline__ uint32_t e4m3_encode(float q) {
  const uint32_t u = __float_as_uint(q);
  const uint32_t mag = u & 0x7FFFFFFFu;
  if (mag > 0x7F800000u) return 0x7Fu;  // NaN
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = __uint_as_float(mag);
  if (a >= 448.0f) return sign | 0x7Eu;
  const int e = (int)(mag >> 23) - 127;  // exponent of a normal fp32 (fp32 subnormals: < -6)
  if (e < -6) return sign | (uint32_t)__builtin_rintf(__builtin_ldexpf(a, 9));  // exact scaling
  const float m = __builtin_rintf(__builtin_ldexpf(a, 3 - e));               // 8 .. 16
  uint32_t code = m == 16.0f ? (uint32_t)(e + 8) << 3 : ((uint32_t)(e + 7) << 3) | ((uint32_t)m - 8u);
  return sign | (code > 0x7Eu ? 0x7Eu : code);
}

// Four E4M3 codes (byte k = code of q[k]) with the hardware's
// round-to-nearest-even conversion on the range where it is exact for every
// fp32 input, and the format's rule outside it: magnitudes at or below 2^-10
// (half the smallest subnormal step; fp32 subnormals included) become +-0,
// magnitudes at or past 448 saturate, NaN gives 0x7F.
__device__ __forceinline__ uint32_t e4m3_encode4(const float (&q)[4]) {
  float c[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float a = fabsf(q[k]);
    c[k] = a <= 0x1p-10f ? __builtin_copysignf(0.0f, q[k]) : (a >= 448.0f ? __builtin_copysignf(448.0f, q[k]) : q[k]);
  }
  uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
  w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], (int)w, true);
#pragma unroll
  for (int k = 0; k < 4; ++k)
    if (q[k] != q[k]) w = (w & ~(0xFFu << (8 * k))) | (0x7Fu << (8 * k));
  return w;
}

// bf16 bits of an fp32 value: nearest, ties to even; NaN stays NaN.
__device__ __forceinline__ uint32_t bf16_encode(float v) {
  const uint32_t u = __float_as_uint(v);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// One wavefront per appended row; 4 rows per workgroup.
__global__ void __launch_bounds__(256)
mla_append_kernel(int B, int T, int D, int P, int MP, int src_dtype, int kv_dtype,
                  const void* __restrict__ src, const int32_t* __restrict__ page_table,
                  const int32_t* __restrict__ pos0, void* __restrict__ kv, float* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int64_t idx = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (idx >= (int64_t)B * T) return;
  const int b = (int)(idx / T), t = (int)(idx - (int64_t)b * T);
  const int pos = pos0[b] + t;
  const int64_t row = kv_row_index(page_table, MP, P, b, pos);  // the write side of the same mapping
  auto value = [&](int d) -> float {
    return src_dtype == kF32 ? ((const float*)src)[idx * D + d]
                             : bf16_bits_to_float(((const uint16_t*)src)[idx * D + d]);
  };
  if (kv_dtype == kF32) {
    for (int d = lane; d < D; d += 64) ((float*)kv)[row * D + d] = value(d);
    return;
  }
  if (kv_dtype == kBF16) {
    for (int d = lane; d < D; d += 64) ((uint16_t*)kv)[row * D + d] = (uint16_t)bf16_encode(value(d));
    return;
  }
  if ((D & 3) == 0 && D <= 1024) {
    // the row in registers: up to four 4-value chunks per lane, one read
    float v[4][4];
    float amax = 0.0f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int d = 4 * (lane + 64 * c);
      if (d < D) {
        if (src_dtype == kF32) {
          const floatx4 f = *(const floatx4*)((const float*)src + idx * D + d);
#pragma unroll
          for (int k = 0; k < 4; ++k) v[c][k] = f[k];
        } else {
          const uintx2 w = *(const uintx2*)((const uint16_t*)src + idx * D + d);
          v[c][0] = __uint_as_float(w[0] << 16);
          v[c][1] = __uint_as_float(w[0] & 0xFFFF0000u);
          v[c][2] = __uint_as_float(w[1] << 16);
          v[c][3] = __uint_as_float(w[1] & 0xFFFF0000u);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) amax = fmaxf(amax, fabsf(v[c][k]));
      }
    }
    amax = wave_max(amax);
    const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int d = 4 * (lane + 64 * c);
      if (d < D) {
        float q[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) q[k] = v[c][k] / s;
        *(uint32_t*)((uint8_t*)kv + row * D + d) = e4m3_encode4(q);
      }
    }
    if (lane == 0) scales[row] = s;
    return;
  }
  float amax = 0.0f;
  for (int d = lane; d < D; d += 64) amax = fmaxf(amax, fabsf(value(d)));
  amax = wave_max(amax);
  const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
  for (int d = lane; d < D; d += 64) ((uint8_t*)kv + row * D)[d] = (uint8_t)e4m3_encode(value(d) / s);
  if (lane == 0) scales[row] = s;
}

// ------------------------------------------------- greedy chain verification
// Greedy verification of a linear chain of drafts (TokenSpeed code-audit
// article, technology list, speculative decoding: greedy linear-chain
// verification).  Request b has T positions; position 0 holds the last
// accepted token and positions 1..T-1 the drafts d[0..T-2].  The target's
// token at position t is p_t = argmax_v logits[b][t][v] (stored values
// compared exactly, the smallest index among equal maxima, NaN never wins, 0
// when every entry is NaN).  Draft i passes iff d[i] == p_i and every draft
// before it passed; with n passing, out = d[0..n-1], p_n, then -1.
// One workgroup per request; the rows are scanned one after another by all
// threads, each keeping the first maximum of its own (increasing) indices.
struct ArgMax {
  float v;
  int i;  // kNone: nothing seen yet
};
constexpr int kNone = 0x7FFFFFFF;
__device__ __forceinline__ ArgMax better(ArgMax a, ArgMax b) {
  if (a.i == kNone) return b;
  if (b.i == kNone) return a;
  if (b.v > a.v) return b;
  if (a.v > b.v) return a;
  return b.i < a.i ? b : a;
}
__device__ __forceinline__ void take(ArgMax& a, float v, int i) {
  if (v == v && (a.i == kNone || v > a.v)) a = ArgMax{v, i};  // indices arrive in increasing order
}

__global__ void __launch_bounds__(1024)
mla_verify_kernel(int T, int V, int dtype, const void* __restrict__ logits, const int32_t* __restrict__ draft,
                  int32_t* __restrict__ argmax, int32_t* __restrict__ accept_len, int32_t* __restrict__ out) {
  __shared__ float red_v[16];
  __shared__ int red_i[16];
  __shared__ int best_sh[64];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int t = 0; t < T; ++t) {  // T <= 64 (checked on the host)
    const int64_t base = ((int64_t)b * T + t) * V;
    ArgMax a{0.0f, kNone};
    if (dtype == kBF16 && (V & 7) == 0) {
      const uintx4* row = (const uintx4*)((const uint16_t*)logits + base);
      const int nc = V >> 3;
      auto take8 = [&](const uintx4& w, int c) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          take(a, __uint_as_float(w[k] << 16), 8 * c + 2 * k);
          take(a, __uint_as_float(w[k] & 0xFFFF0000u), 8 * c + 2 * k + 1);
        }
      };
      int c = tid;
      for (; c + 3 * 1024 < nc; c += 4 * 1024) {  // four 16-byte loads in flight per thread
        uintx4 w[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) w[u] = row[c + u * 1024];
#pragma unroll
        for (int u = 0; u < 4; ++u) take8(w[u], c + u * 1024);
      }
      for (; c < nc; c += 1024) take8(row[c], c);
    } else if (dtype == kF32 && (V & 3) == 0) {
      const floatx4* row = (const floatx4*)((const float*)logits + base);
      const int nc = V >> 2;
      for (int c = tid; c < nc; c += 1024) {
        const floatx4 w = row[c];
#pragma unroll
        for (int k = 0; k < 4; ++k) take(a, w[k], 4 * c + k);
      }
    } else {
      for (int v = tid; v < V; v += 1024)
        take(a, dtype == kF32 ? ((const float*)logits)[base + v]
                              : bf16_bits_to_float(((const uint16_t*)logits)[base + v]), v);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const ArgMax o{__shfl_xor(a.v, off, 64), __shfl_xor(a.i, off, 64)};
      a = better(a, o);
    }
    if (lane == 0) {
      red_v[wave] = a.v;
      red_i[wave] = a.i;
    }
    __syncthreads();
    if (tid == 0) {
      ArgMax m{red_v[0], red_i[0]};
      for (int w = 1; w < 16; ++w) m = better(m, ArgMax{red_v[w], red_i[w]});
      best_sh[t] = m.i == kNone ? 0 : m.i;
      argmax[(int64_t)b * T + t] = best_sh[t];
    }
    __syncthreads();
  }
  if (tid == 0) {  // the run of leading matches
    int n = 0;
    while (n < T - 1 && draft[(int64_t)b * (T - 1) + n] == best_sh[n]) ++n;
    accept_len[b] = n;
    for (int i = 0; i < T; ++i)
      out[(int64_t)b * T + i] = i < n ? draft[(int64_t)b * (T - 1) + i] : (i == n ? best_sh[n] : -1);
  }
}

// ------------------------------------------------------------ gather hook
// ---------------------------------------------------------------------------
// Per-head projection on either side of the latent attention (the absorbed
// projections of MLA: q_abs = W_UK^T q_nope forms the query, W_UV o the
// head's value output):  out[m][g][n] = sum_k w[g][n][k] * x[m][g][k].
//
// It is a batch of G small GEMMs that at decode batch sizes streams its
// weights once from HBM (about 73 flops per byte at M = 64, well under the
// chip's bf16 ridge), so the design goal is bytes in flight, not MFMA rate.
// One workgroup owns a 32 (m) x 64 (n) output tile of one head.  The k range
// is cut into 32-wide chunks dealt round-robin to the four waves, so even a
// short k loop (k = 128: one chunk per wave) keeps every wave loading; each
// wave issues all loads of its chunks (up to four) before its first MFMA, and
// the register budget follows the chunks a wave holds (more resident
// workgroups when k is short).  Operands
// go from HBM straight into the MFMA layout: both are k-contiguous, so lane
// (i, half) reads 16 contiguous bytes of row i per MFMA step.  The four
// partial tiles are summed through LDS, which also turns the accumulator
// layout into 16-byte row stores.  Tiles are numbered head-major and dealt in
// contiguous ranges per XCD, so the tiles that share a head's x rows and
// weight rows share one L2.
constexpr int kPjWaves = 4, kPjTileM = 32, kPjTileN = 64, kPjChunk = 32;

__device__ __forceinline__ bf16x8 pj_load(const __bf16* row, int k, int K, bool valid) {
  if (valid && k < K) return *(const bf16x8*)(row + k);
  return bf16x8{};
}

template <typename OutT, int kPjGroup>
__global__ void __launch_bounds__(64 * kPjWaves)
mla_project_kernel(int M, int G, int K, int N, const __bf16* __restrict__ x, const __bf16* __restrict__ w,
                   OutT* __restrict__ out, int tiles_m, int tiles_n, int per_xcd, int tiles) {
  constexpr int kPitch = kPjTileN + 4;  // floats; the pad spreads the row-scattered writes
  __shared__ float red[kPjWaves][kPjTileM][kPitch];
  const int bid = blockIdx.x;
  const int u = (bid & 7) * per_xcd + (bid >> 3);
  if (u >= tiles) return;  // whole workgroup, before any barrier
  const int per_head = tiles_m * tiles_n;
  const int g = u / per_head;
  const int mt = (u - g * per_head) / tiles_n;
  const int nt = u - g * per_head - mt * tiles_n;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = lane & 31, half = lane >> 5;
  // MFMA operand A = weight rows (output columns n), B = x rows (output rows m)
  const int m = mt * kPjTileM + i;
  const int n0 = nt * kPjTileN + i, n1 = n0 + 32;
  const bool vm = m < M, vn0 = n0 < N, vn1 = n1 < N;
  const __bf16* xr = x + ((int64_t)(vm ? m : 0) * G + g) * K + 8 * half;
  const __bf16* w0 = w + ((int64_t)g * N + (vn0 ? n0 : 0)) * K + 8 * half;
  const __bf16* w1 = w + ((int64_t)g * N + (vn1 ? n1 : 0)) * K + 8 * half;
  const int Kh = K - 8 * half;  // a piece at k (relative to this lane's base) exists iff k < Kh
  floatx16 acc0 = {}, acc1 = {};
  const int nch = (K + kPjChunk - 1) / kPjChunk;
  for (int c0 = wave; c0 < nch; c0 += kPjWaves * kPjGroup) {
    bf16x8 xa[kPjGroup][2], wa[kPjGroup][2], wb[kPjGroup][2];
#pragma unroll
    for (int s = 0; s < kPjGroup; ++s)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int k = (c0 + kPjWaves * s) * kPjChunk + 16 * st;
        xa[s][st] = pj_load(xr, k, Kh, vm);
        wa[s][st] = pj_load(w0, k, Kh, vn0);
        wb[s][st] = pj_load(w1, k, Kh, vn1);
      }
#pragma unroll
    for (int s = 0; s < kPjGroup; ++s) {
      if (c0 + kPjWaves * s >= nch) break;  // wave-uniform
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa[s][st], xa[s][st], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wb[s][st], xa[s][st], acc1, 0, 0, 0);
      }
    }
  }
  // accumulator register r of lane (i, half) holds output row m = i and
  // column n = 8 (r / 4) + 4 half + r % 4 (+ 32 for acc1)
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int nl = 8 * q + 4 * half;
    *(floatx4*)&red[wave][i][nl] = floatx4{acc0[4 * q], acc0[4 * q + 1], acc0[4 * q + 2], acc0[4 * q + 3]};
    *(floatx4*)&red[wave][i][nl + 32] = floatx4{acc1[4 * q], acc1[4 * q + 1], acc1[4 * q + 2], acc1[4 * q + 3]};
  }
  __syncthreads();
  const int t = threadIdx.x;
  const int ml = t >> 3, nl = 8 * (t & 7);
  const int mo = mt * kPjTileM + ml, no = nt * kPjTileN + nl;
  if (mo >= M || no >= N) return;  // N is a multiple of 8: a piece is all in or all out
  floatx4 s0 = *(const floatx4*)&red[0][ml][nl], s1 = *(const floatx4*)&red[0][ml][nl + 4];
#pragma unroll
  for (int v = 1; v < kPjWaves; ++v) {
    s0 += *(const floatx4*)&red[v][ml][nl];
    s1 += *(const floatx4*)&red[v][ml][nl + 4];
  }
  OutT* dst = out + ((int64_t)mo * G + g) * N + no;
  if constexpr (sizeof(OutT) == 4) {
    *(floatx4*)dst = s0;
    *(floatx4*)(dst + 4) = s1;
  } else {
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      o[e] = (__bf16)s0[e];
      o[4 + e] = (__bf16)s1[e];
    }
    *(bf16x8*)dst = o;
  }
}

// Staged form for k a multiple of 64: a 64 (m) x 64 (n) output tile per
// workgroup, its operands streamed through a ring of LDS stages by direct
// HBM -> LDS loads.  A stage holds 64 k of the tile's 64 x rows and 64 weight
// rows (128 bytes of each row, 16 KB); each 64-lane load moves eight whole
// 128-byte rows, so every request is a full cache line (the register-direct
// form above reads 32 rows x 32 bytes per instruction).  In LDS, row r's
// 16-byte column c sits at r * 128 + 16 (c ^ (r & 7)): the loads place it
// there by permuting their source addresses within the row, and the MFMA
// operand reads (32 rows, one logical column per half-wave) then hit eight
// distinct 16-byte bank groups per eight lanes.  Waves form a 2 x 2 grid of
// 32 x 32 MFMA tiles.  Rows past M or N load a clamped in-range row whose
// results are never stored.
constexpr int kPsTileN = 64;
template <int TM>
constexpr int ps_stage_bytes() { return (TM + kPsTileN) * 128; }

template <typename OutT, int STAGES, int TM>
__global__ void __launch_bounds__(256)
mla_project_staged(int M, int G, int K, int N, const __bf16* __restrict__ x, const __bf16* __restrict__ w,
                   OutT* __restrict__ out, int tiles_m, int tiles_n, int per_xcd, int tiles) {
  static_assert(TM == 64 || TM == 128, "tile rows");
  constexpr int kStage = ps_stage_bytes<TM>();
  constexpr int kLoads = (TM + kPsTileN) / 32;  // 8-row loads per wave per stage
  constexpr int kMt = TM / 64;                  // 32-row m subtiles per wave
  extern __shared__ __attribute__((aligned(1024))) char pj_smem_raw[];
  LDS_AS char* smem = (LDS_AS char*)pj_smem_raw;
  const int bid = blockIdx.x;
  const int u = (bid & 7) * per_xcd + (bid >> 3);
  if (u >= tiles) return;  // whole workgroup, before any barrier
  const int per_head = tiles_m * tiles_n;
  const int g = u / per_head;
  const int mt = (u - g * per_head) / tiles_n;
  const int nt = u - g * per_head - mt * tiles_n;
  const int m0 = mt * TM, n0 = nt * kPsTileN;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // Load j (0 <= j < (TM + 64) / 8) of a stage moves tile rows 8 j .. 8 j + 7:
  // the TM x rows first, then the 64 weight rows; wave v issues loads
  // kLoads v .. kLoads v + kLoads - 1.  Lane L takes row 8 j + L / 8, physical
  // column L % 8.
  const int lr = lane >> 3, lc = (lane & 7) ^ lr;  // (8 j + lr) & 7 == lr
  const char* xb = (const char*)(x + ((int64_t)m0 * G + g) * K);
  const char* wb = (const char*)(w + ((int64_t)g * N + n0) * K);
  uint32_t voff[kLoads];
#pragma unroll
  for (int q = 0; q < kLoads; ++q) {
    const int j = kLoads * wave + q;
    if (j < TM / 8) {
      const int r = 8 * j + lr;
      const int rm = (m0 + r < M ? r : M - 1 - m0);
      voff[q] = (uint32_t)((int64_t)rm * G * K * 2 + 16 * lc);
    } else {
      const int r = 8 * (j - TM / 8) + lr;
      const int rn = (n0 + r < N ? r : N - 1 - n0);
      voff[q] = (uint32_t)((int64_t)rn * K * 2 + 16 * lc);
    }
  }
  const int nst = K / 64;
  auto issue = [&](int t) {
    LDS_AS char* slot = smem + (t % STAGES) * kStage;
#pragma unroll
    for (int q = 0; q < kLoads; ++q) {
      const int j = kLoads * wave + q;
      lds_dma16((j < TM / 8 ? xb : wb) + 128 * t, voff[q], lds_addr(slot + 1024 * j));
    }
  };
  // all STAGES slots are filled up front; after that, step t refills the slot
  // that step t - 1 read
#pragma unroll
  for (int t = 0; t < STAGES; ++t)
    if (t < nst) issue(t);
  const int i = lane & 31, h = lane >> 5;
  const int wm = wave & 1, wn = wave >> 1;
  // operand rows: A = weight row 32 wn + i, B = x rows TM / 2 wm + 32 mi + i
  // (all equal to i modulo 8)
  const int ra = TM * 128 + (32 * wn + i) * 128, rb = ((TM / 2) * wm + i) * 128;
  floatx16 acc[kMt];
#pragma unroll
  for (int mi = 0; mi < kMt; ++mi) acc[mi] = floatx16{};
  for (int t = 0; t < nst; ++t) {
    // stages issued so far: min(nst, STAGES) at t = 0, min(nst, t + STAGES - 1) after
    const int issued = t == 0 ? STAGES : t + STAGES - 1;
    const int ahead = (issued < nst ? issued : nst) - 1 - t;
    wait_ahead<kLoads>(ahead);
    __syncthreads();  // stage t is in LDS for every wave; slot (t - 1) % STAGES is free
    if (t >= 1 && t + STAGES - 1 < nst) issue(t + STAGES - 1);
    const LDS_AS char* slot = smem + (t % STAGES) * kStage;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int col = 16 * ((2 * s + h) ^ (i & 7));
      const bf16x8 a = *(const LDS_AS bf16x8*)(slot + ra + col);
#pragma unroll
      for (int mi = 0; mi < kMt; ++mi) {
        const bf16x8 b = *(const LDS_AS bf16x8*)(slot + rb + 32 * 128 * mi + col);
        acc[mi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[mi], 0, 0, 0);
      }
    }
  }
  // D[n][m]: register r of lane (i, h) holds n = 32 wn + 8 (r / 4) + 4 h + r % 4,
  // m = TM / 2 wm + 32 mi + i.  Staged as [m][n] OutT rows (pitch + 16 bytes),
  // then stored as 16-byte pieces of whole rows.
  constexpr int kRowB = kPsTileN * (int)sizeof(OutT), kPitchB = kRowB + 16;
  static_assert(TM * kPitchB <= STAGES * kStage, "output staging fits the stages");
  __syncthreads();  // every wave is done with the stages
#pragma unroll
  for (int mi = 0; mi < kMt; ++mi)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int nl = 32 * wn + 8 * q + 4 * h;
      LDS_AS char* dst = smem + ((TM / 2) * wm + 32 * mi + i) * kPitchB + nl * (int)sizeof(OutT);
      const floatx16& a = acc[mi];
      if constexpr (sizeof(OutT) == 4) {
        *(LDS_AS floatx4*)dst = floatx4{a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]};
      } else {
        *(LDS_AS bf16x4*)dst =
            bf16x4{(__bf16)a[4 * q], (__bf16)a[4 * q + 1], (__bf16)a[4 * q + 2], (__bf16)a[4 * q + 3]};
      }
    }
  __syncthreads();
  constexpr int kPieces = TM * kRowB / 16, kPerRow = kRowB / 16;
#pragma unroll
  for (int e = threadIdx.x; e < kPieces; e += 256) {
    const int ml = e / kPerRow, pc = e - ml * kPerRow;
    const int mo = m0 + ml, no = n0 + pc * (16 / (int)sizeof(OutT));
    if (mo < M && no < N)  // N is a multiple of 8: a piece is all in or all out
      *(uintx4*)(out + ((int64_t)mo * G + g) * N + no) = *(const LDS_AS uintx4*)(smem + ml * kPitchB + 16 * pc);
  }
}

__global__ void mla_gather_kernel(int D, int elt, int P, int MP, const char* __restrict__ kv,
                                  const int32_t* __restrict__ page_table, int n,
                                  const int32_t* __restrict__ req, const int32_t* __restrict__ tok,
                                  char* __restrict__ out) {
  const int rb = D * elt;
  const int64_t total = (int64_t)n * rb;
  for (int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; x < total;
       x += (int64_t)gridDim.x * blockDim.x) {
    const int i = (int)(x / rb), byte = (int)(x - (int64_t)i * rb);
    const int64_t row = kv_row_index(page_table, MP, P, req[i], tok[i]);
    out[x] = kv[row * rb + byte];
  }
}

// ------------------------------------------------------------- launchers
template <bool FP8, int WAVES, int STAGES>
hipError_t launch_mfma(const SplitParams& p, hipStream_t stream) {
  constexpr int kRows = 32 * WAVES;
  const int M = p.T * p.H;
  const int groups = (M + kRows - 1) / kRows;
  static_assert(kRows == kBalancedRows, "balanced units are one workgroup of rows");
  const int units = p.B * p.S;
  const int64_t blocks = p.NB > 0   ? (int64_t)p.NB
                         : p.Sp > 0 ? 8LL * ((p.S + 7) / 8) * p.B * groups  // cascade: chunk-major per XCD
                                    : 8LL * groups * ((units + 7) / 8);
  // + restart requests + plan scratch
  const size_t lds = (size_t)STAGES * Tile<FP8>::kStage + 8 * WAVES + 4 * (WAVES + 2);
  static std::once_flag once;
  static hipError_t attr_err = hipSuccess;
  std::call_once(once, [&] {
    attr_err = hipFuncSetAttribute((const void*)mla_split_mfma<FP8, WAVES, STAGES>,
                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  });
  if (attr_err != hipSuccess) return attr_err;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((mla_split_mfma<FP8, WAVES, STAGES>), dim3((unsigned)blocks), dim3(64 * WAVES),
                     lds, stream, p, groups);
  return hipGetLastError();
}

}  // namespace

Kernel pick_kernel(const SplitParams& p) {
  if (p.force_generic) return Kernel::kGeneric;
  // the MFMA kernel folds the scale into its exponent and takes the row
  // maximum before scaling, which needs scale > 0
  const bool mfma_shape = p.Dc == 512 && p.Dr == 64 && p.q_dtype == kBF16 && p.P % 32 == 0 &&
                          (p.kv_dtype == kBF16 || p.kv_dtype == kFP8) && p.scale > 0.0f;
  if (!mfma_shape) return Kernel::kGeneric;
  return p.kv_dtype == kFP8 ? Kernel::kMfmaFp8 : Kernel::kMfmaBf16;
}

// bf16 and E4M3 KV: the wave-pair kernel with 128-row workgroups.
// (Workgroups of two pairs would fill the chip where a uniform plan has fewer
// units than compute units, but one wave per SIMD runs them slower than half
// the chip runs the four-pair ones.)  The environment variable
// MLA_MFMA_KERNEL=four (read at each launch) selects the four-wave kernel
// instead, for either KV format.
bool four_wave_selected() {
  const char* sel = getenv("MLA_MFMA_KERNEL");
  return sel && sel[0] == 'f';
}
hipError_t launch_bf16_mfma(const SplitParams& p, hipStream_t stream) {
  if (four_wave_selected()) return launch_mfma<false, 4, 4>(p, stream);
  return launch_pair<4, false>(p, stream);
}
hipError_t launch_fp8_mfma(const SplitParams& p, hipStream_t stream) {
  if (four_wave_selected()) return launch_mfma<true, 4, 8>(p, stream);
  return launch_pair<4, true>(p, stream);
}

hipError_t launch_split(const SplitParams& p, hipStream_t stream) {
  switch (pick_kernel(p)) {
    case Kernel::kMfmaBf16: return launch_bf16_mfma(p, stream);
    case Kernel::kMfmaFp8: return launch_fp8_mfma(p, stream);
    default: break;
  }
  const int M = p.T * p.H;
  if (p.B == 0 || M == 0) return hipSuccess;
  dim3 grid((unsigned)((M + 3) / 4), (unsigned)p.S, (unsigned)p.B);
  const size_t lds = sizeof(float) * 4 * (size_t)(p.Dc + p.Dr);
  hipLaunchKernelGGL(mla_split_generic, grid, dim3(256), lds, stream, p);
  return hipGetLastError();
}

hipError_t launch_combine(int32_t B, int32_t S, int32_t rows, int32_t Dc, const float* part_o,
                          const float* part_lse, int32_t out_dtype, void* out, float* lse,
                          hipStream_t stream) {
  const int64_t n = (int64_t)B * rows;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(mla_combine_kernel, dim3((unsigned)((n + 3) / 4)), dim3(256), 0, stream, B, S,
                     rows, Dc, part_o, part_lse, out_dtype, out, lse);
  return hipGetLastError();
}

hipError_t launch_combine_balanced(int32_t B, int32_t M, int32_t Dc, int32_t NB,
                                   const int32_t* tile_prefix, const void* part_o,
                                   const float* part_lse, int32_t out_dtype, void* out, float* lse,
                                   hipStream_t stream) {
  const int64_t n = (int64_t)B * M;
  if (n == 0) return hipSuccess;
  if (M % kMergeRows == 0 && Dc % 8 == 0 && Dc <= 512) {
    // wavefronts per row-quad from the average number of partials per unit
    // (measured: the single-wavefront merge is faster up to about 8)
    const int64_t units = (int64_t)B * ((M + kBalancedRows - 1) / kBalancedRows);
    const int64_t per_unit = NB / units + 1;
    const int64_t quads = n / kMergeRows;
    auto grid = [&](int q) { return dim3((unsigned)((quads + q - 1) / q)); };
    if (per_unit > 32)
      hipLaunchKernelGGL(mla_combine_balanced_wide_kernel<8>, grid(WideMerge<8>::kQuads), dim3(WideMerge<8>::kThreads),
                         0, stream, B, M, Dc, NB, tile_prefix, (const __bf16*)part_o, part_lse, out_dtype, out, lse);
    else if (per_unit > 16)
      hipLaunchKernelGGL(mla_combine_balanced_wide_kernel<4>, grid(WideMerge<4>::kQuads), dim3(WideMerge<4>::kThreads),
                         0, stream, B, M, Dc, NB, tile_prefix, (const __bf16*)part_o, part_lse, out_dtype, out, lse);
    else if (per_unit > 8)
      hipLaunchKernelGGL(mla_combine_balanced_wide_kernel<2>, grid(WideMerge<2>::kQuads), dim3(WideMerge<2>::kThreads),
                         0, stream, B, M, Dc, NB, tile_prefix, (const __bf16*)part_o, part_lse, out_dtype, out, lse);
    else  // a few partials per unit: one wavefront per row-quad
      hipLaunchKernelGGL(mla_combine_balanced4_kernel, dim3((unsigned)((quads + 3) / 4)), dim3(256), 0, stream, B, M,
                         Dc, NB, tile_prefix, (const __bf16*)part_o, part_lse, out_dtype, out, lse);
    return hipGetLastError();
  }
  if (M % kMergeRows == 0 && Dc % 8 == 0) {
    const int64_t waves = n / kMergeRows;
    hipLaunchKernelGGL(mla_combine_balanced4_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, stream, B, M,
                       Dc, NB, tile_prefix, (const __bf16*)part_o, part_lse, out_dtype, out, lse);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(mla_combine_balanced_kernel, dim3((unsigned)((n + 3) / 4)), dim3(256), 0, stream,
                     B, M, Dc, NB, tile_prefix, (const __bf16*)part_o, part_lse, out_dtype, out, lse);
  return hipGetLastError();
}

hipError_t launch_append(int32_t B, int32_t T, int32_t D, int32_t P, int32_t MP, int32_t src_dtype,
                         int32_t kv_dtype, const void* src, const int32_t* page_table,
                         const int32_t* positions, void* kv, float* kv_scales, hipStream_t stream) {
  const int64_t n = (int64_t)B * T;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(mla_append_kernel, dim3((unsigned)((n + 3) / 4)), dim3(256), 0, stream, B, T, D, P,
                     MP, src_dtype, kv_dtype, src, page_table, positions, kv, kv_scales);
  return hipGetLastError();
}

hipError_t launch_verify(int32_t B, int32_t T, int32_t V, int32_t dtype, const void* logits,
                         const int32_t* draft, int32_t* argmax, int32_t* accept_len, int32_t* out,
                         hipStream_t stream) {
  if (B == 0) return hipSuccess;
  hipLaunchKernelGGL(mla_verify_kernel, dim3((unsigned)B), dim3(1024), 0, stream, T, V, dtype, logits, draft,
                     argmax, accept_len, out);
  return hipGetLastError();
}

template <int S, int TM>
hipError_t launch_staged(hipStream_t stream, int M, int G, int K, int N, const void* x, const void* w,
                         int32_t out_dtype, void* out) {
  const int tm = (M + TM - 1) / TM, tn = (N + kPsTileN - 1) / kPsTileN;
  const int64_t tl = (int64_t)G * tm * tn, px = (tl + 7) / 8;
  const dim3 grid((unsigned)(8 * px));
  const size_t lds = (size_t)S * ps_stage_bytes<TM>();
  static std::once_flag once;
  static hipError_t attr_err = hipSuccess;
  std::call_once(once, [&] {
    const hipError_t e1 = hipFuncSetAttribute((const void*)mla_project_staged<float, S, TM>,
                                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    const hipError_t e2 = hipFuncSetAttribute((const void*)mla_project_staged<__bf16, S, TM>,
                                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    attr_err = e1 != hipSuccess ? e1 : e2;
  });
  if (attr_err != hipSuccess) return attr_err;
  if (out_dtype == kF32)
    hipLaunchKernelGGL((mla_project_staged<float, S, TM>), grid, dim3(256), lds, stream, M, G, K, N,
                       (const __bf16*)x, (const __bf16*)w, (float*)out, tm, tn, (int)px, (int)tl);
  else
    hipLaunchKernelGGL((mla_project_staged<__bf16, S, TM>), grid, dim3(256), lds, stream, M, G, K, N,
                       (const __bf16*)x, (const __bf16*)w, (__bf16*)out, tm, tn, (int)px, (int)tl);
  return hipGetLastError();
}

hipError_t launch_project(int32_t M, int32_t G, int32_t K, int32_t N, const void* x, const void* w,
                          int32_t out_dtype, void* out, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const int tiles_m = (M + kPjTileM - 1) / kPjTileM, tiles_n = (N + kPjTileN - 1) / kPjTileN;
  const int64_t tiles = (int64_t)G * tiles_m * tiles_n;
  const int64_t per_xcd = (tiles + 7) / 8;
  const dim3 grid((unsigned)(8 * per_xcd)), block(64 * kPjWaves);
  // staged form: k a multiple of 64, and every row offset within a tile's
  // 128 rows fits the loads' 32-bit offsets.  Two stages hold all of
  // k <= 128 (more resident workgroups), four stream longer k.  With k <= 128
  // and more than 64 rows, 128-row tiles read each weight row once per 128
  // token rows (A/B on one box: 1024 rows x 64 heads, k 128 -> n 512, 6 %
  // faster); with four stages their 96 KB of LDS leaves one workgroup per CU,
  // and 64-row tiles are faster.
  if (K % 64 == 0 && (int64_t)128 * G * K * 2 < ((int64_t)1 << 31)) {
    if (K <= 128)
      return M > 64 ? launch_staged<2, 128>(stream, M, G, K, N, x, w, out_dtype, out)
                    : launch_staged<2, 64>(stream, M, G, K, N, x, w, out_dtype, out);
    return launch_staged<4, 64>(stream, M, G, K, N, x, w, out_dtype, out);
  }
  const int nch = (K + kPjChunk - 1) / kPjChunk, per_wave = (nch + kPjWaves - 1) / kPjWaves;
#define PJ_LAUNCH(T, GR) hipLaunchKernelGGL((mla_project_kernel<T, GR>), grid, block, 0, stream, M, G, K, N, (const __bf16*)x, \
                       (const __bf16*)w, (T*)out, tiles_m, tiles_n, (int)per_xcd, (int)tiles)
  if (out_dtype == kF32) {
    if (per_wave <= 1) PJ_LAUNCH(float, 1); else if (per_wave <= 2) PJ_LAUNCH(float, 2); else PJ_LAUNCH(float, 4);
  } else {
    if (per_wave <= 1) PJ_LAUNCH(__bf16, 1); else if (per_wave <= 2) PJ_LAUNCH(__bf16, 2); else PJ_LAUNCH(__bf16, 4);
  }
#undef PJ_LAUNCH
  return hipGetLastError();
}

hipError_t launch_gather(int32_t Dc, int32_t Dr, int32_t P, int32_t MP, int32_t kv_dtype,
                         const void* kv, const int32_t* page_table, int32_t n, const int32_t* req,
                         const int32_t* tok, void* out, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int elt = kv_dtype == kF32 ? 4 : (kv_dtype == kBF16 ? 2 : 1);
  const int64_t total = (int64_t)n * (Dc + Dr) * elt;
  const int64_t blocks64 = (total + 255) / 256;
  const unsigned blocks = (unsigned)(blocks64 < 4096 ? blocks64 : 4096);
  hipLaunchKernelGGL(mla_gather_kernel, dim3(blocks), dim3(256), 0, stream, Dc + Dr, elt, P, MP,
                     (const char*)kv, page_table, n, req, tok, (char*)out);
  return hipGetLastError();
}

// ------------------------------------------------------ streaming read probe
// Measurement hook: reads n16 16-byte words once (grid-stride, eight loads in
// flight per thread) and writes the XOR of everything each workgroup read to
// sink[workgroup], which keeps every load live and makes the result checkable.
__global__ void __launch_bounds__(256)
mla_stream_read_kernel(const uintx4* __restrict__ src, int64_t n16, unsigned* __restrict__ sink) {
  __shared__ unsigned part[4];
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  unsigned acc = 0;
  for (; i + 7 * stride < n16; i += 8 * stride) {
    uintx4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const uintx4 v = src[i];
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc ^= (unsigned)__shfl_xor((int)acc, off, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

hipError_t launch_stream_read(const void* src, int64_t n16, unsigned* sink, int32_t blocks,
                              hipStream_t stream) {
  hipLaunchKernelGGL(mla_stream_read_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     (const uintx4*)src, n16, sink);
  return hipGetLastError();
}

// ------------------------------------------------------- static scratch
// Device memory for mla_decode_no_alloc, the entry point for callers that
// cannot allocate: the workspace of one decode (balanced work list slots and
// tile prefix, or uniform-plan partials) lives in this file-scope array, one
// copy per device, held until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the
// symbol): the device address comes from hipGetSymbolAddress, taken once per
// device with that device current and kept in per_device below.
static __device__ __attribute__((aligned(256))) unsigned char scratch[kStaticScratchBytes];

hipError_t static_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* per_device[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (per_device[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    per_device[dev] = p;
  }
  *ptr = per_device[dev];
  return hipSuccess;
}

}  // namespace mla
