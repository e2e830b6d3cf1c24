// C-ABI layer of the MLA decode library: argument validation, split
// planning, checked mode and kernel dispatch.  Declared in include/mla.h.
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdlib.h>

#include <vector>

#include "../../include/mla.h"
#include "mla_internal.h"

namespace {

using mla::SplitParams;

// Largest chunk count the planner picks by itself, and the number of
// workgroups it aims for (256 CUs, one 4-wave MFMA workgroup each, two waves
// of workgroups so that short and long chunks even out).
constexpr int32_t kAutoMaxSplits = 64;
constexpr int64_t kTargetWorkgroups = 512;
constexpr int32_t kMaxSplits = 1 << 16;

bool env_checked_mode() {
  static const bool on = [] {
    const char* v = getenv("MLA_CHECK");
    return v && v[0] == '1';
  }();
  return on;
}

// MLA_KERNEL=generic routes every call to the VALU kernel (cross-checks).
bool env_force_generic() {
  const char* v = getenv("MLA_KERNEL");
  return v && v[0] == 'g';
}

// MLA_PLAN=uniform turns the balanced work list off (comparisons, tests).
bool env_force_uniform() {
  const char* v = getenv("MLA_PLAN");
  return v && v[0] == 'u';
}

bool valid_dtype(int32_t d) { return d == MLA_DTYPE_F32 || d == MLA_DTYPE_BF16 || d == MLA_DTYPE_FP8_E4M3; }

int validate_problem(const mla_problem* pr) {
  if (!pr) return MLA_ERR_INVALID_ARG;
  if (pr->batch < 0 || pr->q_len < 1 || pr->num_heads < 1 || pr->d_latent < 1 || pr->d_rope < 0 ||
      pr->page_size < 1 || pr->num_pages < 1 || pr->max_pages_per_seq < 1 || pr->max_seq_len < 0 ||
      pr->num_splits < 0 || pr->num_splits > kMaxSplits)
    return MLA_ERR_INVALID_ARG;
  if ((int64_t)pr->max_pages_per_seq * pr->page_size > INT32_MAX) return MLA_ERR_INVALID_ARG;
  if ((int64_t)pr->max_seq_len > (int64_t)pr->max_pages_per_seq * pr->page_size) return MLA_ERR_INVALID_ARG;
  if ((int64_t)pr->q_len * pr->num_heads > INT32_MAX / 4) return MLA_ERR_INVALID_ARG;
  if (pr->causal != 0 && pr->causal != 1) return MLA_ERR_INVALID_ARG;
  if (!valid_dtype(pr->q_dtype) || !valid_dtype(pr->kv_dtype) || !valid_dtype(pr->out_dtype))
    return MLA_ERR_INVALID_ARG;
  if (pr->q_dtype == MLA_DTYPE_FP8_E4M3 || pr->out_dtype == MLA_DTYPE_FP8_E4M3) return MLA_ERR_UNSUPPORTED;
  if (pr->d_latent > 1024 || pr->d_latent + pr->d_rope > 4096) return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

int32_t effective_max_len(const mla_problem* pr) {
  return pr->max_seq_len > 0 ? pr->max_seq_len : pr->max_pages_per_seq * pr->page_size;
}

// Chunks per request: forced, or enough (page-aligned) chunks that the grid
// reaches about kTargetWorkgroups workgroups, never more than the pages of
// the longest request.
int32_t plan_splits(const mla_problem* pr) {
  const int32_t max_pages = (effective_max_len(pr) + pr->page_size - 1) / pr->page_size;
  const int32_t cap = max_pages > 0 ? max_pages : 1;
  if (pr->num_splits > 0) return pr->num_splits;
  const int64_t rows = (int64_t)pr->q_len * pr->num_heads;
  const int64_t groups = (rows + 127) / 128;
  const int64_t units = (int64_t)(pr->batch > 0 ? pr->batch : 1) * groups;
  int64_t s = (kTargetWorkgroups + units - 1) / units;
  if (s > kAutoMaxSplits) s = kAutoMaxSplits;
  if (s > cap) s = cap;
  if (s < 1) s = 1;
  return (int32_t)s;
}

size_t partial_bytes(const mla_problem* pr, int32_t S) {
  const size_t rows = (size_t)pr->batch * S * pr->q_len * pr->num_heads;
  const size_t o = rows * pr->d_latent * sizeof(float);
  const size_t o_aligned = (o + 255) & ~(size_t)255;
  return o_aligned + rows * sizeof(float);
}

// The balanced work list's tile indices are int32: all tiles of all units
// must fit.
bool balanced_size_ok(const mla_problem* pr) {
  const int64_t units = mla::balanced_units(pr->batch, pr->q_len, pr->num_heads);
  // positions per unit: its tiles plus the start cost
  const int64_t max_pos = ((int64_t)pr->max_pages_per_seq * pr->page_size + 31) / 32 + mla::kUnitStartCost;
  return units < (int64_t)INT32_MAX / 2 && units * max_pos < (int64_t)INT32_MAX / 2;
}

// Balanced work list (used by mla_decode when the library chooses the plan,
// the uniform plan would split, and the MFMA kernels serve the shape): one
// workgroup per compute unit, partial slots [NB][2][kBalancedRows].
bool balanced_shape(const mla_problem* pr) {
  if (pr->num_splits != 0 || plan_splits(pr) <= 1) return false;
  if (!(pr->d_latent == 512 && pr->d_rope == 64 && pr->q_dtype == MLA_DTYPE_BF16 &&
        pr->page_size % 32 == 0 &&
        (pr->kv_dtype == MLA_DTYPE_BF16 || pr->kv_dtype == MLA_DTYPE_FP8_E4M3)))
    return false;
  return balanced_size_ok(pr);
}

int32_t device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return cus;
}

struct BalancedLayout {
  size_t prefix_off, lse_off, o_off, total;
};

BalancedLayout balanced_layout(const mla_problem* pr, int32_t NB) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t units = (size_t)mla::balanced_units(pr->batch, pr->q_len, pr->num_heads);
  const size_t slot_rows = (size_t)NB * 2 * mla::kBalancedRows;
  BalancedLayout l;
  l.prefix_off = 0;
  l.lse_off = up((units + 1) * sizeof(int32_t));
  l.o_off = l.lse_off + up(slot_rows * sizeof(float));
  l.total = l.o_off + slot_rows * (size_t)pr->d_latent * sizeof(uint16_t);  // bf16 slot rows
  return l;
}

// Workspace for everything mla_decode may run: the uniform plan's partials
// and, where it may apply, the balanced work list's.
size_t decode_workspace(const mla_problem* pr, int32_t S, int32_t NB) {
  size_t need = S > 1 ? partial_bytes(pr, S) : 0;
  if (NB > 0 && balanced_shape(pr)) {
    const size_t bal = balanced_layout(pr, NB).total;
    if (bal > need) need = bal;
  }
  return need;
}

SplitParams make_params(const mla_problem* pr, const void* q_abs, const void* q_rope, const void* kv,
                        const float* kv_scales, const int32_t* page_table, const int32_t* seq_lens,
                        float scale, int32_t S) {
  SplitParams p{};
  p.B = pr->batch;
  p.T = pr->q_len;
  p.H = pr->num_heads;
  p.Dc = pr->d_latent;
  p.Dr = pr->d_rope;
  p.P = pr->page_size;
  p.NP = pr->num_pages;
  p.MP = pr->max_pages_per_seq;
  p.q_dtype = pr->q_dtype;
  p.kv_dtype = pr->kv_dtype;
  p.out_dtype = pr->out_dtype;
  p.causal = pr->causal;
  p.S = S;
  p.q_abs = q_abs;
  p.q_rope = q_rope;
  p.kv = kv;
  p.kv_scales = kv_scales;
  p.page_table = page_table;
  p.seq_lens = seq_lens;
  p.scale = scale;
  p.force_generic = env_force_generic();
  return p;
}

int validate_inputs(const mla_problem* pr, const void* q_abs, const void* q_rope, const void* kv,
                    const float* kv_scales, const int32_t* page_table, const int32_t* seq_lens) {
  if (pr->batch == 0) return MLA_OK;
  if (!q_abs || !kv || !page_table || !seq_lens) return MLA_ERR_INVALID_ARG;
  if (pr->d_rope > 0 && !q_rope) return MLA_ERR_INVALID_ARG;
  if ((pr->kv_dtype == MLA_DTYPE_FP8_E4M3) != (kv_scales != nullptr)) return MLA_ERR_INVALID_ARG;
  return MLA_OK;
}

int run_checked_mode(const mla_problem* pr, const int32_t* page_table, const int32_t* seq_lens,
                     hipStream_t stream) {
  if (!env_checked_mode() || pr->batch == 0) return MLA_OK;
  std::vector<int32_t> pt((size_t)pr->batch * pr->max_pages_per_seq), sl((size_t)pr->batch);
  if (hipMemcpyAsync(pt.data(), page_table, pt.size() * sizeof(int32_t), hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipMemcpyAsync(sl.data(), seq_lens, sl.size() * sizeof(int32_t), hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return MLA_ERR_HIP;
  return mla_check_tables(pr, pt.data(), sl.data());
}

// Cascade plan: chunks of about the same length for the shared prefix and
// for each request's suffix, sized so that the grid reaches about
// kTargetWorkgroups workgroups.
void cascade_plan(const mla_problem* pr, int32_t prefix_len, int32_t* Sp, int32_t* Ss) {
  const int64_t P = pr->page_size;
  const int64_t max_len = effective_max_len(pr);
  const int64_t groups = ((int64_t)pr->q_len * pr->num_heads + 127) / 128;
  const int64_t units = (int64_t)(pr->batch > 0 ? pr->batch : 1) * groups;
  int64_t chunk = (units * max_len + kTargetWorkgroups - 1) / kTargetWorkgroups;
  chunk = (chunk + P - 1) / P * P;
  if (chunk < P) chunk = P;
  const int64_t suffix = max_len > prefix_len ? max_len - prefix_len : 0;
  int64_t sp = (prefix_len + chunk - 1) / chunk, ss = (suffix + chunk - 1) / chunk;
  if (sp < 1) sp = 1;
  if (ss < 1) ss = 1;
  *Sp = (int32_t)(sp < kAutoMaxSplits ? sp : kAutoMaxSplits);
  *Ss = (int32_t)(ss < kAutoMaxSplits ? ss : kAutoMaxSplits);
}

int cascade_check(const mla_problem* pr, int32_t prefix_len) {
  const int rc = validate_problem(pr);
  if (rc) return rc;
  if (prefix_len < 0 || prefix_len % pr->page_size != 0 ||
      (int64_t)prefix_len > (int64_t)pr->max_pages_per_seq * pr->page_size)
    return MLA_ERR_INVALID_ARG;
  return MLA_OK;
}

}  // namespace

extern "C" {

int mla_num_splits(const mla_problem* problem, int32_t* num_splits) {
  const int rc = validate_problem(problem);
  if (rc) return rc;
  if (!num_splits) return MLA_ERR_INVALID_ARG;
  *num_splits = plan_splits(problem);
  return MLA_OK;
}

int mla_workspace_size(const mla_problem* problem, size_t* bytes) {
  const int rc = validate_problem(problem);
  if (rc) return rc;
  if (!bytes) return MLA_ERR_INVALID_ARG;
  const int32_t S = plan_splits(problem);
  *bytes = decode_workspace(problem, S, balanced_shape(problem) ? device_cus() : 0);
  return MLA_OK;
}

int mla_check_tables(const mla_problem* problem, const int32_t* page_table_host,
                     const int32_t* seq_lens_host) {
  const int rc = validate_problem(problem);
  if (rc) return rc;
  if (problem->batch > 0 && (!page_table_host || !seq_lens_host)) return MLA_ERR_INVALID_ARG;
  const int64_t cap = (int64_t)problem->max_pages_per_seq * problem->page_size;
  for (int32_t b = 0; b < problem->batch; ++b) {
    const int32_t L = seq_lens_host[b];
    if (L < 0 || L > cap) return MLA_ERR_CHECK;
    const int32_t used = (int32_t)(((int64_t)L + problem->page_size - 1) / problem->page_size);
    for (int32_t e = 0; e < used; ++e) {
      const int32_t page = page_table_host[(int64_t)b * problem->max_pages_per_seq + e];
      if (page < 0 || page >= problem->num_pages) return MLA_ERR_CHECK;
    }
  }
  return MLA_OK;
}

int mla_decode_split(const mla_problem* problem, const void* q_absorbed, const void* q_rope,
                     const void* kv_pages, const float* kv_scales, const int32_t* page_table,
                     const int32_t* seq_lens, float scale, int32_t num_splits, float* partial_o,
                     float* partial_lse, hipStream_t stream) {
  int rc = validate_problem(problem);
  if (rc) return rc;
  if (num_splits < 1 || num_splits > kMaxSplits) return MLA_ERR_INVALID_ARG;
  rc = validate_inputs(problem, q_absorbed, q_rope, kv_pages, kv_scales, page_table, seq_lens);
  if (rc) return rc;
  if (problem->batch == 0) return MLA_OK;
  if (!partial_o || !partial_lse) return MLA_ERR_INVALID_ARG;
  rc = run_checked_mode(problem, page_table, seq_lens, stream);
  if (rc) return rc;
  SplitParams p = make_params(problem, q_absorbed, q_rope, kv_pages, kv_scales, page_table,
                              seq_lens, scale, num_splits);
  p.write_final = false;
  p.part_o = partial_o;
  p.part_lse = partial_lse;
  return mla::launch_split(p, stream) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // extern "C"

namespace {

// mla_decode with the workspace either the caller's (static_scratch false)
// or the library's static device scratch (true: workspace arguments unused).
int decode_impl(const mla_problem* problem, const void* q_absorbed, const void* q_rope,
                const void* kv_pages, const float* kv_scales, const int32_t* page_table,
                const int32_t* seq_lens, float scale, void* out, float* lse, void* workspace,
                size_t workspace_bytes, bool static_scratch, hipStream_t stream) {
  int rc = validate_problem(problem);
  if (rc) return rc;
  rc = validate_inputs(problem, q_absorbed, q_rope, kv_pages, kv_scales, page_table, seq_lens);
  if (rc) return rc;
  if (problem->batch == 0) return MLA_OK;
  if (!out) return MLA_ERR_INVALID_ARG;
  const int32_t S = plan_splits(problem);
  const int32_t NB = balanced_shape(problem) && !env_force_uniform() ? device_cus() : 0;
  SplitParams p = make_params(problem, q_absorbed, q_rope, kv_pages, kv_scales, page_table,
                              seq_lens, scale, S);
  const bool balanced = NB > 0 && mla::pick_kernel(p) != mla::Kernel::kGeneric;
  if (static_scratch) {
    // the workspace of the plan this call runs
    static_assert(mla::kStaticScratchBytes == MLA_STATIC_SCRATCH_BYTES, "header and library agree");
    const size_t need = balanced ? balanced_layout(problem, NB).total : (S > 1 ? partial_bytes(problem, S) : 0);
    if (need > mla::kStaticScratchBytes) return MLA_ERR_SCRATCH;
    workspace = nullptr;
    workspace_bytes = mla::kStaticScratchBytes;
    if (need > 0 && mla::static_scratch(&workspace) != hipSuccess) return MLA_ERR_HIP;
  } else {
    // the caller's workspace is sized by mla_workspace_size(): every plan this
    // problem may take
    const size_t need = decode_workspace(problem, S, NB);
    if (need > 0 && (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255) != 0))
      return MLA_ERR_WORKSPACE;
  }
  rc = run_checked_mode(problem, page_table, seq_lens, stream);
  if (rc) return rc;
  if (balanced) {
    // the stages of mla_decode_split_balanced and mla_combine_balanced,
    // arguments already validated
    const BalancedLayout l = balanced_layout(problem, NB);
    const int32_t M = problem->q_len * problem->num_heads;
    int32_t* prefix = (int32_t*)((char*)workspace + l.prefix_off);
    p.NB = NB;
    p.tile_prefix = prefix;
    p.write_final = false;
    p.out = out;
    p.lse = lse;
    p.part_lse = (float*)((char*)workspace + l.lse_off);
    p.part_o = (float*)((char*)workspace + l.o_off);
    if (mla::launch_split(p, stream) != hipSuccess ||
        mla::launch_combine_balanced(problem->batch, M, problem->d_latent, NB, prefix, p.part_o,
                                     p.part_lse, problem->out_dtype, out, lse, stream) != hipSuccess)
      return MLA_ERR_HIP;
    return MLA_OK;
  }
  if (S == 1) {
    p.write_final = true;
    p.out = out;
    p.lse = lse;
    return mla::launch_split(p, stream) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
  }
  const int32_t rows = problem->q_len * problem->num_heads;
  const size_t o_bytes = (size_t)problem->batch * S * rows * problem->d_latent * sizeof(float);
  p.write_final = false;
  p.part_o = (float*)workspace;
  p.part_lse = (float*)((char*)workspace + ((o_bytes + 255) & ~(size_t)255));
  if (mla::launch_split(p, stream) != hipSuccess) return MLA_ERR_HIP;
  return mla::launch_combine(problem->batch, S, rows, problem->d_latent, p.part_o, p.part_lse,
                             problem->out_dtype, out, lse, stream) == hipSuccess
             ? MLA_OK
             : MLA_ERR_HIP;
}

}  // namespace

extern "C" {

int mla_decode(const mla_problem* problem, const void* q_absorbed, const void* q_rope,
               const void* kv_pages, const float* kv_scales, const int32_t* page_table,
               const int32_t* seq_lens, float scale, void* out, float* lse, void* workspace,
               size_t workspace_bytes, hipStream_t stream) {
  return decode_impl(problem, q_absorbed, q_rope, kv_pages, kv_scales, page_table, seq_lens, scale, out,
                     lse, workspace, workspace_bytes, false, stream);
}

int mla_decode_no_alloc(const mla_problem* problem, const void* q_absorbed, const void* q_rope,
                        const void* kv_pages, const float* kv_scales, const int32_t* page_table,
                        const int32_t* seq_lens, float scale, void* out, float* lse, hipStream_t stream) {
  return decode_impl(problem, q_absorbed, q_rope, kv_pages, kv_scales, page_table, seq_lens, scale, out,
                     lse, nullptr, 0, true, stream);
}

int mla_balanced_workgroups(int32_t* num_workgroups) {
  if (!num_workgroups) return MLA_ERR_INVALID_ARG;
  const int32_t cus = device_cus();
  if (cus <= 0) return MLA_ERR_HIP;
  *num_workgroups = cus;
  return MLA_OK;
}

int mla_decode_split_balanced(const mla_problem* problem, const void* q_absorbed,
                              const void* q_rope, const void* kv_pages, const float* kv_scales,
                              const int32_t* page_table, const int32_t* seq_lens, float scale,
                              int32_t num_workgroups, int32_t* tile_prefix, void* out,
                              float* lse, void* slot_o, float* slot_lse, hipStream_t stream) {
  int rc = validate_problem(problem);
  if (rc) return rc;
  rc = validate_inputs(problem, q_absorbed, q_rope, kv_pages, kv_scales, page_table, seq_lens);
  if (rc) return rc;
  if (problem->batch == 0) return MLA_OK;
  if (num_workgroups < 1 || !tile_prefix || !out || !slot_o || !slot_lse) return MLA_ERR_INVALID_ARG;
  if (!balanced_size_ok(problem)) return MLA_ERR_UNSUPPORTED;
  SplitParams p = make_params(problem, q_absorbed, q_rope, kv_pages, kv_scales, page_table,
                              seq_lens, scale, 1);
  if (mla::pick_kernel(p) == mla::Kernel::kGeneric) return MLA_ERR_UNSUPPORTED;
  rc = run_checked_mode(problem, page_table, seq_lens, stream);
  if (rc) return rc;
  p.NB = num_workgroups;
  p.tile_prefix = tile_prefix;
  p.write_final = false;
  p.out = out;
  p.lse = lse;
  p.part_o = (float*)slot_o;  // bf16 slot rows in balanced mode
  p.part_lse = slot_lse;
  return mla::launch_split(p, stream) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int mla_combine_balanced(const mla_problem* problem, int32_t num_workgroups,
                         const int32_t* tile_prefix, const void* slot_o, const float* slot_lse,
                         void* out, float* lse, hipStream_t stream) {
  const int rc = validate_problem(problem);
  if (rc) return rc;
  if (problem->batch == 0) return MLA_OK;
  if (num_workgroups < 1 || !tile_prefix || !slot_o || !slot_lse || !out) return MLA_ERR_INVALID_ARG;
  const int32_t M = problem->q_len * problem->num_heads;
  return mla::launch_combine_balanced(problem->batch, M, problem->d_latent, num_workgroups,
                                      tile_prefix, slot_o, slot_lse, problem->out_dtype, out, lse,
                                      stream) == hipSuccess
             ? MLA_OK
             : MLA_ERR_HIP;
}

int mla_cascade_workspace_size(const mla_problem* problem, int32_t prefix_len, size_t* bytes) {
  const int rc = cascade_check(problem, prefix_len);
  if (rc) return rc;
  if (!bytes) return MLA_ERR_INVALID_ARG;
  int32_t Sp, Ss;
  cascade_plan(problem, prefix_len, &Sp, &Ss);
  *bytes = partial_bytes(problem, Sp + Ss);
  return MLA_OK;
}

int mla_decode_cascade(const mla_problem* problem, const void* q_absorbed, const void* q_rope,
                       const void* kv_pages, const float* kv_scales, const int32_t* page_table,
                       const int32_t* seq_lens, float scale, int32_t prefix_len, void* out, float* lse,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int rc = cascade_check(problem, prefix_len);
  if (rc) return rc;
  rc = validate_inputs(problem, q_absorbed, q_rope, kv_pages, kv_scales, page_table, seq_lens);
  if (rc) return rc;
  if (problem->batch == 0) return MLA_OK;
  if (!out) return MLA_ERR_INVALID_ARG;
  int32_t Sp, Ss;
  cascade_plan(problem, prefix_len, &Sp, &Ss);
  const int32_t S = Sp + Ss;
  const size_t need = partial_bytes(problem, S);
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255) != 0) return MLA_ERR_WORKSPACE;
  SplitParams p = make_params(problem, q_absorbed, q_rope, kv_pages, kv_scales, page_table, seq_lens,
                              scale, S);
  if (mla::pick_kernel(p) == mla::Kernel::kGeneric) return MLA_ERR_UNSUPPORTED;
  rc = run_checked_mode(problem, page_table, seq_lens, stream);
  if (rc) return rc;
  const int32_t rows = problem->q_len * problem->num_heads;
  const size_t o_bytes = (size_t)problem->batch * S * rows * problem->d_latent * sizeof(float);
  p.Sp = Sp;
  p.prefix_len = prefix_len;
  p.write_final = false;
  p.part_o = (float*)workspace;
  p.part_lse = (float*)((char*)workspace + ((o_bytes + 255) & ~(size_t)255));
  if (mla::launch_split(p, stream) != hipSuccess) return MLA_ERR_HIP;
  return mla::launch_combine(problem->batch, S, rows, problem->d_latent, p.part_o, p.part_lse,
                             problem->out_dtype, out, lse, stream) == hipSuccess
             ? MLA_OK
             : MLA_ERR_HIP;
}

int mla_combine(int32_t batch, int32_t num_splits, int32_t rows, int32_t d_latent,
                const float* partial_o, const float* partial_lse, int32_t out_dtype, void* out,
                float* lse, hipStream_t stream) {
  if (batch < 0 || num_splits < 1 || num_splits > kMaxSplits || rows < 1 || d_latent < 1)
    return MLA_ERR_INVALID_ARG;
  if (out_dtype != MLA_DTYPE_F32 && out_dtype != MLA_DTYPE_BF16) return MLA_ERR_UNSUPPORTED;
  if (batch == 0) return MLA_OK;
  if (!partial_o || !partial_lse || !out) return MLA_ERR_INVALID_ARG;
  return mla::launch_combine(batch, num_splits, rows, d_latent, partial_o, partial_lse, out_dtype,
                             out, lse, stream) == hipSuccess
             ? MLA_OK
             : MLA_ERR_HIP;
}

int mla_append_kv(const mla_problem* problem, const void* rows, int32_t src_dtype,
                  const int32_t* page_table, const int32_t* positions, void* kv_pages, float* kv_scales,
                  hipStream_t stream) {
  const int rc = validate_problem(problem);
  if (rc) return rc;
  if (src_dtype != MLA_DTYPE_F32 && src_dtype != MLA_DTYPE_BF16) return MLA_ERR_UNSUPPORTED;
  if (problem->batch == 0) return MLA_OK;
  if (!rows || !page_table || !positions || !kv_pages) return MLA_ERR_INVALID_ARG;
  if ((problem->kv_dtype == MLA_DTYPE_FP8_E4M3) != (kv_scales != nullptr)) return MLA_ERR_INVALID_ARG;
  if ((int64_t)problem->batch * problem->q_len > INT32_MAX) return MLA_ERR_INVALID_ARG;
  return mla::launch_append(problem->batch, problem->q_len, problem->d_latent + problem->d_rope,
                            problem->page_size, problem->max_pages_per_seq, src_dtype,
                            problem->kv_dtype, rows, page_table, positions, kv_pages, kv_scales,
                            stream) == hipSuccess
             ? MLA_OK
             : MLA_ERR_HIP;
}

int mla_verify_greedy(int32_t batch, int32_t num_positions, int32_t vocab, const void* logits,
                      int32_t logits_dtype, const int32_t* draft, int32_t* argmax, int32_t* accept_len,
                      int32_t* out_tokens, hipStream_t stream) {
  if (batch < 0 || num_positions < 1 || vocab < 1) return MLA_ERR_INVALID_ARG;
  if (logits_dtype != MLA_DTYPE_F32 && logits_dtype != MLA_DTYPE_BF16) return MLA_ERR_UNSUPPORTED;
  if (num_positions > 64) return MLA_ERR_UNSUPPORTED;
  if ((int64_t)batch * num_positions * vocab > (int64_t)1 << 40) return MLA_ERR_INVALID_ARG;
  if (batch == 0) return MLA_OK;
  if (!logits || !argmax || !accept_len || !out_tokens || (num_positions > 1 && !draft))
    return MLA_ERR_INVALID_ARG;
  return mla::launch_verify(batch, num_positions, vocab, logits_dtype, logits, draft, argmax, accept_len,
                            out_tokens, stream) == hipSuccess
             ? MLA_OK
             : MLA_ERR_HIP;
}

int mla_project(int32_t rows, int32_t heads, int32_t in_dim, int32_t out_dim, const void* x,
                const void* w, int32_t out_dtype, void* out, hipStream_t stream) {
  if (rows < 0 || heads < 1 || in_dim < 8 || out_dim < 8) return MLA_ERR_INVALID_ARG;
  if (in_dim % 8 != 0 || out_dim % 8 != 0) return MLA_ERR_UNSUPPORTED;
  if (out_dtype != MLA_DTYPE_F32 && out_dtype != MLA_DTYPE_BF16) return MLA_ERR_UNSUPPORTED;
  const int64_t tiles = (int64_t)heads * ((rows + 31) / 32) * ((out_dim + 63) / 64);
  if ((int64_t)rows * heads * in_dim > (int64_t)1 << 40 || (int64_t)rows * heads * out_dim > (int64_t)1 << 40 ||
      (int64_t)heads * out_dim * in_dim > (int64_t)1 << 40 || tiles > (int64_t)1 << 28)
    return MLA_ERR_INVALID_ARG;
  if (rows == 0) return MLA_OK;
  if (!x || !w || !out) return MLA_ERR_INVALID_ARG;
  if (((uintptr_t)x | (uintptr_t)w | (uintptr_t)out) % 16 != 0) return MLA_ERR_INVALID_ARG;
  return mla::launch_project(rows, heads, in_dim, out_dim, x, w, out_dtype, out, stream) == hipSuccess
             ? MLA_OK
             : MLA_ERR_HIP;
}

int mla_gather_rows(const mla_problem* problem, const void* kv_pages, const int32_t* page_table,
                    int32_t n, const int32_t* req, const int32_t* tok, void* out,
                    hipStream_t stream) {
  const int rc = validate_problem(problem);
  if (rc) return rc;
  if (n < 0) return MLA_ERR_INVALID_ARG;
  if (n == 0) return MLA_OK;
  if (!kv_pages || !page_table || !req || !tok || !out) return MLA_ERR_INVALID_ARG;
  return mla::launch_gather(problem->d_latent, problem->d_rope, problem->page_size,
                            problem->max_pages_per_seq, problem->kv_dtype, kv_pages, page_table, n,
                            req, tok, out, stream) == hipSuccess
             ? MLA_OK
             : MLA_ERR_HIP;
}

int mla_stream_read(const void* src, size_t bytes, uint32_t* sink, int32_t sink_len,
                    hipStream_t stream) {
  if ((!src && bytes) || !sink || sink_len < 1 || sink_len > 65536) return MLA_ERR_INVALID_ARG;
  if (bytes % 16 != 0 || (uintptr_t)src % 16 != 0 || (uintptr_t)sink % 4 != 0) return MLA_ERR_INVALID_ARG;
  return mla::launch_stream_read(src, (int64_t)(bytes / 16), sink, sink_len, stream) == hipSuccess
             ? MLA_OK
             : MLA_ERR_HIP;
}

const char* mla_status_string(int status) {
  switch (status) {
    case MLA_OK: return "ok";
    case MLA_ERR_INVALID_ARG: return "invalid argument";
    case MLA_ERR_UNSUPPORTED: return "unsupported combination";
    case MLA_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case MLA_ERR_HIP: return "HIP runtime or launch failure";
    case MLA_ERR_CHECK: return "checked mode: page id or seq_len out of range";
    case MLA_ERR_SCRATCH: return "problem needs more workspace than the static scratch of mla_decode_no_alloc holds";
    default: return "unknown status";
  }
}

}  // extern "C"
