// Internal interface between the C-ABI layer (mla_api.cpp) and the HIP
// kernels (mla_kernels.hip).  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace mla {

enum DType : int32_t { kF32 = 0, kBF16 = 1, kFP8 = 2 };

// One split-stage launch: every argument already validated on the host.
struct SplitParams {
  int32_t B, T, H, Dc, Dr, P, NP, MP;
  int32_t q_dtype, kv_dtype, out_dtype, causal;
  int32_t S;                   // chunks per request
  const void* q_abs;
  const void* q_rope;
  const void* kv;
  const float* kv_scales;
  const int32_t* page_table;
  const int32_t* seq_lens;
  float scale;
  bool write_final;            // S == 1: write out/lse directly
  void* out;                   // [B, T*H, Dc] out_dtype (write_final)
  float* lse;                  // [B, T*H] or nullptr (write_final)
  float* part_o;               // uniform: [B, S, T*H, Dc] fp32 (!write_final);
                               // balanced: slot rows [2 NB, 128, Dc] bf16
  float* part_lse;             // [B, S, T*H] fp32 (!write_final)
  bool force_generic;          // run the VALU kernel even where the MFMA one applies
  // Balanced work list (MFMA kernels only; NB == 0 selects uniform chunks):
  // the 32-token tiles of all units (request, group of kBalancedRows rows),
  // each unit with tiles preceded by kUnitStartCost positions that stand for
  // the cost of starting a segment, are cut into NB equal contiguous ranges
  // of positions, one per workgroup.
  int32_t NB;
  int32_t* tile_prefix;        // [B * groups + 1] exclusive prefix of positions per
                               // unit (tiles + kUnitStartCost, 0 for a unit
                               // without tiles), written by workgroup 0 for the merge
  // Cascade (uniform chunks only; Sp == 0 disables it): chunks 0..Sp-1 split
  // the first prefix_len tokens (a prefix every request shares) with the same
  // page-aligned bounds for all requests, chunks Sp..S-1 split [prefix_len, L_b).
  int32_t Sp;
  int32_t prefix_len;
};

// Rows per unit of the balanced work list (the MFMA kernels' workgroup rows).
constexpr int32_t kBalancedRows = 128;

// Positions the balanced work list charges for starting a unit, in tiles: a
// workgroup whose range holds the start of a unit pays a second prologue
// (query staging, pipeline fill) and epilogue, and so gets that many fewer
// tiles.  4 measured best of 0, 2, 4, 6, 8 on the DeepSeek-shaped batch.
constexpr int32_t kUnitStartCost = 4;

// Number of units (request, row group) of the balanced work list.
inline int64_t balanced_units(int32_t B, int32_t T, int32_t H) {
  return (int64_t)B * (((int64_t)T * H + kBalancedRows - 1) / kBalancedRows);
}

// Merge for the balanced work list: for each unit that spans several
// workgroups, merge its partial slots into out/lse; units without tiles get
// out = 0, lse = -inf; the others were written by the split kernel.
hipError_t launch_combine_balanced(int32_t B, int32_t M, int32_t Dc, int32_t NB,
                                   const int32_t* tile_prefix, const void* part_o,
                                   const float* part_lse, int32_t out_dtype, void* out, float* lse,
                                   hipStream_t stream);

enum class Kernel { kMfmaBf16, kMfmaFp8, kGeneric };

// Which kernel serves this shape (host-side decision, no HIP call).
Kernel pick_kernel(const SplitParams& p);

hipError_t launch_split(const SplitParams& p, hipStream_t stream);

hipError_t launch_combine(int32_t B, int32_t S, int32_t rows, int32_t Dc, const float* part_o,
                          const float* part_lse, int32_t out_dtype, void* out, float* lse,
                          hipStream_t stream);

// Paged KV append with packing (see mla_append_kv); arguments validated.
hipError_t launch_append(int32_t B, int32_t T, int32_t D, int32_t P, int32_t MP, int32_t src_dtype,
                         int32_t kv_dtype, const void* src, const int32_t* page_table,
                         const int32_t* positions, void* kv, float* kv_scales, hipStream_t stream);

// Greedy chain verification (see mla_verify_greedy); T <= 64, arguments validated.
hipError_t launch_verify(int32_t B, int32_t T, int32_t V, int32_t dtype, const void* logits,
                         const int32_t* draft, int32_t* argmax, int32_t* accept_len, int32_t* out,
                         hipStream_t stream);

// Per-head projection (see mla_project); arguments validated, bf16 x and w.
hipError_t launch_project(int32_t M, int32_t G, int32_t K, int32_t N, const void* x, const void* w,
                          int32_t out_dtype, void* out, hipStream_t stream);

hipError_t launch_gather(int32_t Dc, int32_t Dr, int32_t P, int32_t MP, int32_t kv_dtype,
                         const void* kv, const int32_t* page_table, int32_t n,
                         const int32_t* req, const int32_t* tok, void* out, hipStream_t stream);
hipError_t launch_stream_read(const void* src, int64_t n16, unsigned* sink, int32_t blocks,
                              hipStream_t stream);

// Size of the library's static device scratch (mla_decode_no_alloc).
constexpr size_t kStaticScratchBytes = (size_t)72 << 20;

// Device address of the static scratch on the current device (looked up once
// per device, then cached).
hipError_t static_scratch(void** ptr);

}  // namespace mla
