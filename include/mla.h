/*
 * mla.h -- C ABI of the MI355X (gfx950) library for Multi-head Latent
 * Attention decode over a paged, prefix-shared latent KV cache.
 *
 * The operation (TokenSpeed code-audit article, complete technology list,
 * MLA kernel entry): every token stores ONE row of d_latent latent values
 * followed by d_rope rope values (512 + 64 in DeepSeek-style models); that row
 * is the key of every query head, and its latent part is the value.  The
 * per-head key and value up-projections are absorbed into the query (the
 * query arrives as q_absorbed, d_latent wide, plus q_rope, d_rope wide) and
 * into the caller's output projection, so for request b, query token t, head h
 *
 *   z_j   = scale * ( q_absorbed[b,t,h,:] . c_j  +  q_rope[b,t,h,:] . k_j )
 *   o     = sum_j softmax(z)_j * c_j              (d_latent wide)
 *   lse   = ln sum_j exp(z_j)
 *
 * over the visible tokens j of request b.  Rows live in fixed-size pages
 * found through a per-request block table (the "推理优化" tag page,
 * PagedAttention article: logical block -> physical block); several requests
 * may point at the same physical pages for a shared prefix (TokenSpeed 580
 * tok/s zero-copy article: prefix KV shared by reference, never copied).
 *
 * Long contexts run in two stages, as the code-audit article describes the
 * Blackwell kernel: a split stage writes fp32 partial results per chunk of
 * the sequence into a workspace, and a reduction stage merges them by
 * log-sum-exp rescaling and casts to the output type.  mla_decode() runs both;
 * mla_decode_split() and mla_combine() expose them separately.  (The uniform
 * plan's partials are fp32 as described; the balanced work list, mla_decode's
 * default where it would split, keeps its few per-workgroup partial rows in
 * bf16 with fp32 log-sum-exp: see mla_decode_split_balanced.)
 *
 * Conventions for every entry point:
 *   - All array arguments are DEVICE pointers unless marked "host"; the
 *     caller owns every buffer.  The library allocates no device memory
 *     (its one static device array, the scratch of mla_decode_no_alloc, comes
 *     with the loaded code object), keeps no state between calls (that
 *     array's contents aside) and never synchronises the stream (except in
 *     checked mode, see MLA_CHECK below).
 *   - Work is enqueued on `stream` in order; results are ready when the
 *     stream reaches that point.  Calls on different streams may overlap.
 *   - Every function returns an mla_status code; no C++ exception crosses
 *     the ABI.  Arguments are validated on the host before any HIP call, so
 *     a non-zero status means nothing was enqueued.  Device faults, if any,
 *     surface at the caller's next synchronisation.
 *   - Contents of page-table entries at or past ceil(seq_len/page_size) and of
 *     page slots at or past seq_len are never used (they may hold anything,
 *     including -1 and NaN).  In-range entries must be valid page ids: this
 *     is a precondition (not clamped), checked only in checked mode.
 *   - Checked mode: with the environment variable MLA_CHECK=1 at library
 *     load time, mla_decode() and mla_decode_split() copy page_table and
 *     seq_lens to the host (synchronising the stream) and return
 *     MLA_ERR_CHECK if any used page id is outside [0, num_pages) or any
 *     seq_len is outside [0, max_pages_per_seq * page_size].  Never use it
 *     under graph capture.
 *   - Kernel selection for comparisons (read at each call): MLA_KERNEL=generic
 *     runs every decode on the VALU kernel; MLA_MFMA_KERNEL=four runs bf16
 *     and E4M3 KV on the four-wave MFMA kernel instead of the wave-pair
 *     kernel.  Results agree up to rounding.
 */
#ifndef MLA_DECODE_H_
#define MLA_DECODE_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_DTYPE_F32 = 0,      /* IEEE binary32 */
  MLA_DTYPE_BF16 = 1,     /* bfloat16 (upper half of binary32) */
  MLA_DTYPE_FP8_E4M3 = 2  /* OCP FP8 E4M3: 4 exponent bits, 3 mantissa bits, max 448
                             ("推理优化" tag page, quantisation article, FP8 table);
                             KV only, with one fp32 scale per token */
} mla_dtype;

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = -1, /* null pointer, bad size, inconsistent shape */
  MLA_ERR_UNSUPPORTED = -2, /* well-formed, but no kernel for this combination */
  MLA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than mla_workspace_size() */
  MLA_ERR_HIP = -4,         /* a HIP runtime call or kernel launch failed */
  MLA_ERR_CHECK = -5,       /* checked mode found a bad page id or seq_len */
  MLA_ERR_SCRATCH = -6      /* mla_decode_no_alloc: the problem needs more workspace than
                               MLA_STATIC_SCRATCH_BYTES */
} mla_status;

/* Shape and types of one decode call (host struct, passed by pointer). */
typedef struct {
  int32_t batch;             /* B >= 0: requests */
  int32_t q_len;             /* T >= 1: query tokens per request (1 = plain decode;
                                >1 = speculative drafts, folded with the heads into
                                one row axis of T*H rows as the code-audit article's
                                fold_sq_factor does) */
  int32_t num_heads;         /* H >= 1 */
  int32_t d_latent;          /* Dc >= 1: latent width, also the output width */
  int32_t d_rope;            /* Dr >= 0: rope width */
  int32_t page_size;         /* P >= 1: tokens per page */
  int32_t num_pages;         /* NP >= 1: physical pages in kv_pages */
  int32_t max_pages_per_seq; /* MP >= 1: columns of page_table */
  int32_t max_seq_len;       /* host-known upper bound on seq_lens, used only to plan
                                splits; 0 means MP * P */
  int32_t q_dtype;           /* mla_dtype of q_absorbed and q_rope: F32 or BF16 */
  int32_t kv_dtype;          /* mla_dtype of kv_pages: F32, BF16 or FP8_E4M3 */
  int32_t out_dtype;         /* mla_dtype of out: F32 or BF16 */
  int32_t causal;            /* 0: every query token sees j < L_b.  1: query token t
                                sees j <= L_b - T + t (the T drafts are the last T
                                stored rows and form a linear chain) */
  int32_t num_splits;        /* 0: the library chooses; >= 1 forces S chunks */
} mla_problem;

/*
 * Number of sequence chunks S of the uniform split plan for this problem
 * (>= 1), written to *num_splits: the split-KV plan of the code-audit
 * article's MLA entries (the split stage covers one chunk of the sequence
 * per workgroup and the reduction stage merges the chunks).  Chunk k of request b covers tokens
 * [k C_b, min((k+1) C_b, L_b)) with C_b = P * ceil(ceil(L_b / S) / P), so
 * chunks are page aligned and empty chunks are allowed.  mla_decode() runs
 * this plan when num_splits is forced, when S == 1, or when the shape takes
 * the generic kernel; otherwise (the library chooses and would split, on the
 * MFMA kernels: Dc 512, Dr 64, bf16 queries, bf16 or FP8 KV, P a multiple of
 * 32, scale > 0) it runs a balanced work list instead: the 32-token tiles of
 * all requests, laid end to end, are cut into one equal contiguous range per
 * compute unit, a range may cover several requests, and only requests that
 * straddle ranges go through the log-sum-exp merge.  Both plans compute the
 * same result up to rounding.  The environment variable MLA_PLAN=uniform
 * (read at each call) turns the balanced work list off.
 */
int mla_num_splits(const mla_problem* problem, int32_t* num_splits);

/* Bytes of device workspace mla_decode() needs on the current device (0 when
 * it never splits), to *bytes: the buffer the split stage writes its partial
 * results (and their log-sum-exp) into for the reduction stage, the
 * workspace of the code-audit article's MLA entries.  The balanced work list's share depends on the
 * device's compute-unit count, so size the workspace on the device that runs
 * the call. */
int mla_workspace_size(const mla_problem* problem, size_t* bytes);

/*
 * Full decode: split stage plus (when S > 1) the merge, on `stream`.
 *   q_absorbed [B, T, H, Dc]  q_dtype, row-major
 *   q_rope     [B, T, H, Dr]  q_dtype (may be NULL when Dr == 0)
 *   kv_pages   [NP, P, Dc+Dr] kv_dtype; row = Dc latent values then Dr rope values
 *   kv_scales  [NP, P] fp32 per-token scale for FP8_E4M3 KV (stored value =
 *              e4m3(code) * scale); must be NULL for other KV types
 *   page_table [B, MP] int32 physical page ids
 *   seq_lens   [B] int32, 0 <= L_b <= MP * P
 *   scale      softmax scale applied to the full (Dc + Dr)-deep dot product
 *   out        [B, T, H, Dc] out_dtype
 *   lse        [B, T, H] fp32 natural-log log-sum-exp, or NULL
 *   workspace  >= mla_workspace_size() bytes, 256-byte aligned (NULL if 0)
 * Rows with no visible token get out = 0 and lse = -inf.
 */
int mla_decode(const mla_problem* problem, const void* q_absorbed, const void* q_rope,
               const void* kv_pages, const float* kv_scales, const int32_t* page_table,
               const int32_t* seq_lens, float scale, void* out, float* lse, void* workspace,
               size_t workspace_bytes, hipStream_t stream);

/* Size of the library's static device scratch used by mla_decode_no_alloc
 * (72 MiB: the balanced work list's slots for 256 compute units take 64 MiB). */
#define MLA_STATIC_SCRATCH_BYTES ((size_t)72 << 20)

/*
 * mla_decode for callers that cannot allocate device memory: code recorded
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, plan, kernels and results as mla_decode()
 * (bitwise), but the workspace is a static device array inside the library
 * (MLA_STATIC_SCRATCH_BYTES, one copy per device, held until the process
 * ends), so no workspace is passed; the caller still owns q, kv, tables and
 * out/lse.  Nothing is allocated or freed by this call (the array's device
 * address is looked up once per device on the first call there).  Returns
 * MLA_ERR_SCRATCH, with nothing enqueued, when the workspace of the plan
 * this call runs exceeds MLA_STATIC_SCRATCH_BYTES: the balanced work list's
 * (64 MiB of bf16 slots and 256 KiB of slot lse for 256 compute units, plus
 * 4 bytes of tile prefix per row group) fits up to about two million row
 * groups; the uniform plan's while B * S * T * H * (d_latent + 1) * 4 bytes
 * does.  Every call on a device shares that device's array and leaves its
 * contents behind; nothing in it has to start at zero (every word a call
 * reads there was written earlier in the same call).  Calls that overlap on
 * one device (other streams, other host threads) race and must be serialised
 * by the caller.
 */
int mla_decode_no_alloc(const mla_problem* problem, const void* q_absorbed, const void* q_rope,
                        const void* kv_pages, const float* kv_scales, const int32_t* page_table,
                        const int32_t* seq_lens, float scale, void* out, float* lse, hipStream_t stream);

/*
 * Split stage only, with S = num_splits >= 1 chunks (problem->num_splits is
 * ignored).  Writes, per request b, chunk k and row r = t * H + h:
 *   partial_o   [B, S, T*H, Dc] fp32: that chunk's softmax-weighted latent sum,
 *               already divided by the chunk's own normaliser
 *   partial_lse [B, S, T*H] fp32: the chunk's natural-log log-sum-exp, -inf
 *               (with partial_o = 0) when the chunk sees no token
 */
int mla_decode_split(const mla_problem* problem, const void* q_absorbed, const void* q_rope,
                     const void* kv_pages, const float* kv_scales, const int32_t* page_table,
                     const int32_t* seq_lens, float scale, int32_t num_splits,
                     float* partial_o, float* partial_lse, hipStream_t stream);

/*
 * Merge stage: for each of batch*rows rows, M = max_k lse_k,
 * w_k = exp(lse_k - M), out = sum_k w_k o_k / sum_k w_k cast to out_dtype,
 * lse = M + ln sum_k w_k (written if lse != NULL); chunks with lse = -inf
 * weigh nothing and a row with no live chunk gives out = 0, lse = -inf
 * (code-audit article: reduction kernel doing log-sum-exp rescale-merge and
 * the cast to BF16).  Layouts are those of mla_decode_split().
 */
int mla_combine(int32_t batch, int32_t num_splits, int32_t rows, int32_t d_latent,
                const float* partial_o, const float* partial_lse, int32_t out_dtype,
                void* out, float* lse, hipStream_t stream);

/*
 * The balanced work list stage by stage (mla_decode() runs these two, with
 * num_workgroups from mla_balanced_workgroups(), when it picks that plan).
 * A unit is (request b, row group g): the T*H rows of a request in groups of
 * 128 (U = B * ceil(T*H / 128) units, u = b * ceil(T*H / 128) + g), with
 * ceil(L_b / 32) tiles of 32 tokens.  With W tiles in all, workgroup k of
 * nb = min(num_workgroups, W) takes the tiles [k W / nb, (k+1) W / nb) of
 * the units laid end to end; each maximal run of one unit's tiles in that
 * range is a segment.  This is the code-audit article's two-stage
 * split/reduce decode with the chunk bounds chosen for equal work per
 * compute unit instead of equal chunks per request.  The plan is computed on
 * the device from seq_lens (no host synchronisation).
 */

/* Workgroups of the balanced work list on the current device (its compute
 * units), to *num_workgroups. */
int mla_balanced_workgroups(int32_t* num_workgroups);

/*
 * Split stage of the balanced work list on the MFMA kernels (Dc 512, Dr 64,
 * bf16 queries, bf16 or FP8 KV, P a multiple of 32, scale > 0; else
 * MLA_ERR_UNSUPPORTED, as when W could exceed 2^30).  Inputs as for
 * mla_decode().  The units' 32-token tiles, each unit's preceded by a fixed
 * start cost of 4 positions (a workgroup that starts a unit inside its range
 * gets that many tiles fewer), are cut into num_workgroups equal ranges of
 * positions.  Writes tile_prefix [U + 1] int32 (tile_prefix[u] = positions of
 * the units before u, a unit without tiles counting 0; tile_prefix[U] = W)
 * for the merge stage.  A segment
 * that is a whole unit writes its rows of out [B, T, H, Dc] (out_dtype) and
 * lse (if not NULL) directly.  Any other segment writes its normalised
 * partial, rounded to bf16, and its natural-log lse (fp32) to a slot: slot 2k
 * if it continues a unit begun in an earlier workgroup, 2k + 1 if it starts a
 * unit that continues in later ones, with
 *   slot_o   [2 * num_workgroups, 128, Dc] bf16 (row = unit row r - 128 g)
 *   slot_lse [2 * num_workgroups, 128] fp32
 * Slots and out rows that no segment writes are left untouched.
 */
int mla_decode_split_balanced(const mla_problem* problem, const void* q_absorbed,
                              const void* q_rope, const void* kv_pages, const float* kv_scales,
                              const int32_t* page_table, const int32_t* seq_lens, float scale,
                              int32_t num_workgroups, int32_t* tile_prefix, void* out,
                              float* lse, void* slot_o, float* slot_lse, hipStream_t stream);

/*
 * Merge stage of the balanced work list, after mla_decode_split_balanced()
 * with the same num_workgroups: for every unit whose tiles span workgroups
 * k1 < k2, merge slot 2 k1 + 1 and slots 2k (k1 < k <= k2) as mla_combine()
 * does into out/lse; units without tiles get out = 0 and lse = -inf; other
 * units' rows are left as the split stage wrote them.
 */
int mla_combine_balanced(const mla_problem* problem, int32_t num_workgroups,
                         const int32_t* tile_prefix, const void* slot_o, const float* slot_lse,
                         void* out, float* lse, hipStream_t stream);

/*
 * Cascade decode over a shared prefix (the zero-copy article: requests share
 * prefix KV by reference; the pages stress prefix reuse): the first
 * prefix_len tokens (a multiple of page_size) are split into chunks with the
 * same bounds for every request, each request's remaining tokens
 * [prefix_len, L_b) into chunks of its own, and the chunk partials are merged
 * by log-sum-exp as in mla_combine().  The workgroups that read one prefix
 * chunk for the different requests are dealt onto one XCD and run together,
 * so when the requests' tables alias the prefix pages each prefix tile is
 * read from HBM once and served from that XCD's L2 to the others.  Results
 * never depend on the aliasing (every workgroup reads through its own
 * request's table): they equal mla_decode()'s up to rounding for any
 * prefix_len, including requests shorter than the prefix.  MFMA-kernel
 * shapes only (else MLA_ERR_UNSUPPORTED); workspace from
 * mla_cascade_workspace_size(); other arguments as for mla_decode().
 */
int mla_cascade_workspace_size(const mla_problem* problem, int32_t prefix_len, size_t* bytes);
int mla_decode_cascade(const mla_problem* problem, const void* q_absorbed, const void* q_rope,
                       const void* kv_pages, const float* kv_scales, const int32_t* page_table,
                       const int32_t* seq_lens, float scale, int32_t prefix_len, void* out, float* lse,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Paged KV append with packing: the write that fills the cache the decode
 * reads.  problem->batch = B requests, problem->q_len = T new tokens each,
 * rows of D = d_latent + d_rope values; page_size, num_pages,
 * max_pages_per_seq and kv_dtype describe the cache (other fields unused).
 *   rows       [B, T, D] src_dtype (F32 or BF16), device
 *   positions  [B] int32: token t of request b goes to logical position
 *              positions[b] + t, i.e. page page_table[b][pos / P], slot pos mod P
 *              ("推理优化" tag page, PagedAttention article)
 *   kv_pages   [NP, P, D] kv_dtype; kv_scales [NP, P] fp32 for FP8_E4M3 (else NULL)
 * Stored as: F32 the value; BF16 the nearest bf16 (ties to even, NaN stays
 * NaN); FP8_E4M3 one fp32 scale per row s = absmax / 448 computed in fp32
 * (448 = largest finite E4M3, quantisation article's FP8 table on the same
 * page; s = 1 for an all-zero row) and per value the E4M3 code nearest to
 * the fp32 quotient v / s (ties to even, magnitudes past 448 saturate, the
 * sign kept; NaN gives 0x7F).  Only the appended slots are written.
 * Preconditions (not checked on the device): positions[b] + T <= MP * P and
 * the page-table entries covering those positions are valid page ids; the
 * appended slots of different requests are distinct.
 */
int mla_append_kv(const mla_problem* problem, const void* rows, int32_t src_dtype,
                  const int32_t* page_table, const int32_t* positions, void* kv_pages,
                  float* kv_scales, hipStream_t stream);

/*
 * Greedy verification of a linear chain of speculative drafts, the step after
 * the speculative-decode attention (TokenSpeed code-audit article, complete
 * technology list, speculative decoding: greedy linear-chain verification).
 * Request b has T = num_positions (1..64) positions: position 0 holds the
 * last accepted token, positions 1..T-1 the drafts.
 *   logits     [B, T, vocab] logits_dtype (F32 or BF16), device
 *   draft      [B, T-1] int32 draft tokens (may be NULL when T == 1)
 *   argmax     [B, T] int32 out: p_t = argmax_v logits[b][t][v], stored values
 *              compared exactly, the smallest v among equal maxima, NaN never
 *              chosen (0 if every entry is NaN)
 *   accept_len [B] int32 out: n = number of leading drafts with
 *              draft[b][i] == p_i (a draft after a mismatch never passes)
 *   out_tokens [B, T] int32 out: draft[b][0..n-1], then p_n (the target's own
 *              token, the bonus token when every draft passes), then -1
 */
int mla_verify_greedy(int32_t batch, int32_t num_positions, int32_t vocab, const void* logits,
                      int32_t logits_dtype, const int32_t* draft, int32_t* argmax, int32_t* accept_len,
                      int32_t* out_tokens, hipStream_t stream);

/*
 * Per-head projection on either side of the latent attention: the absorbed
 * up-projections of MLA (TokenSpeed code-audit article, MLA entry: keys and
 * values are stored as one low-rank latent per token and decompressed per
 * head by up-projection matrices, which folding into the query and the
 * output avoids).  For every row m and head g
 *
 *   out[m, g, n] = sum_k w[g, n, k] * x[m, g, k]      (fp32 accumulation)
 *
 *   x    [rows, heads, in_dim]  BF16, device (row-major, in_dim contiguous)
 *   w    [heads, out_dim, in_dim] BF16, device (in_dim contiguous)
 *   out  [rows, heads, out_dim] out_dtype (F32 or BF16, nearest-even), device
 * Query side: x = q_nope [B*T, H, d_nope] and w[h] = W_UK[h] transposed,
 * stored [H, d_latent, d_nope] once at weight-load time; out is q_absorbed
 * [B*T, H, d_latent], the layout mla_decode() reads.  Value side: x = the
 * attention output o [B*T, H, d_latent] and w = W_UV [H, d_v, d_latent] as
 * is; out is the per-head value [B*T, H, d_v] that feeds the output
 * projection.  in_dim and out_dim must be multiples of 8 (else
 * MLA_ERR_UNSUPPORTED) and x, w, out 16-byte aligned (else
 * MLA_ERR_INVALID_ARG); rows = 0 enqueues nothing.  out must not overlap x or w.
 */
int mla_project(int32_t rows, int32_t heads, int32_t in_dim, int32_t out_dim, const void* x,
                const void* w, int32_t out_dtype, void* out, hipStream_t stream);

/*
 * Test hook for the page-table loader: copies, bit for bit, the stored rows
 * of logical token tok[i] of request req[i] (i < n) into out [n, Dc+Dr]
 * (kv_dtype elements), resolving pages with the same device address routine
 * the decode kernels use.  req/tok are device arrays; entries must satisfy
 * 0 <= req < B and 0 <= tok < MP * P with a valid page id (precondition).
 */
int mla_gather_rows(const mla_problem* problem, const void* kv_pages, const int32_t* page_table,
                    int32_t n, const int32_t* req, const int32_t* tok, void* out,
                    hipStream_t stream);

/*
 * Measurement hook: a plain streaming read, the reference point for the
 * decode kernels' HBM rates (read bandwidth a simple kernel reaches on this
 * device).  Reads the `bytes` bytes of src (device memory, 16-byte aligned,
 * bytes a multiple of 16) once, in sink_len workgroups, and writes to sink[k]
 * (device array of sink_len uint32) the XOR of the 32-bit words workgroup k
 * read; the XOR over all of sink is the XOR of every 32-bit word of src.
 * sink_len must lie in [1, 65536]; src may be NULL when bytes is 0 (sink is
 * then all zeros); bad pointers, alignment or sizes give
 * MLA_ERR_INVALID_ARG, a launch failure MLA_ERR_HIP.  Caller owns both
 * buffers; nothing is allocated.
 */
int mla_stream_read(const void* src, size_t bytes, uint32_t* sink, int32_t sink_len,
                    hipStream_t stream);

/*
 * Host-side table check (the one checked mode runs): page_table_host [B, MP]
 * and seq_lens_host [B] are HOST arrays.  Returns MLA_OK, MLA_ERR_CHECK or
 * MLA_ERR_INVALID_ARG.
 */
int mla_check_tables(const mla_problem* problem, const int32_t* page_table_host,
                     const int32_t* seq_lens_host);

/* Static description of a status code (never NULL). */
const char* mla_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H_ */
