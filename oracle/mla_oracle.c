/*
 * CPU oracle for MLA decode over a paged latent KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  The tests, the package smoke check and the
 * benchmark's CPU-baseline leg load this library; the GPU path never does, and
 * the two share no code, header or table.  It is plain C, fp64 throughout, with
 * OpenMP only across independent query rows.
 *
 * What it computes, per request b, query token t and head h (notation of the
 * pages: one stored row per token = 512 latent values c_j followed by 64 rope
 * values k_j, and that single row is used as the key and, through its latent
 * part, as the value -- TokenSpeed code-audit article, technology list, MLA
 * kernel entry):
 *
 *   row(j)  = kv[ page_table[b][j / P] ][ j mod P ][ 0 : Dc+Dr ]
 *             (paged storage: a block table maps a request's logical block to
 *             a physical one -- "推理优化" tag page, PagedAttention article)
 *   V       = { j : 0 <= j < L_b, and j <= L_b - T + t when causal }
 *   z_j     = scale * ( q_abs . c_j + q_rope . k_j )
 *   m       = max_{j in V} z_j,   l = sum_{j in V} exp(z_j - m)
 *   p_j     = exp(z_j - m) / l
 *   o       = sum_{j in V} p_j c_j        (Dc wide)
 *   lse     = m + ln l                    (natural log)
 *   V empty -> o = 0, lse = -inf.
 *
 * The three passes (scores; max and normaliser; weighted sum) are kept apart on
 * purpose: tiled online softmax and split-KV merging are exact rewrites of this
 * result (FlashAttention article on the "推理优化" tag page: same output,
 * different memory order; TokenSpeed code-audit article: split kernel with fp32
 * partials merged by log-sum-exp rescaling), and the oracle is the definition
 * they are checked against.  Tokens are visited in logical order, so paged and
 * contiguous layouts give bit-identical results.
 *
 * Stored values are decoded exactly: fp32 as is, bf16 as the upper half of a
 * binary32, FP8 as OCP E4M3 (4 exponent bits with bias 7, 3 mantissa bits,
 * largest finite 448, S.1111.111 = NaN, no infinities -- FP8 format table of
 * the quantisation article on the "推理优化" tag page) times the row's fp32
 * per-token scale.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_E4M3 = 2 };
enum { ORC_OK = 0, ORC_BAD_ARG = -1, ORC_BAD_PAGE = -2, ORC_NO_MEM = -3 };

typedef struct {
  int32_t batch, q_len, num_heads, d_latent, d_rope;
  int32_t page_size, num_pages, max_pages_per_seq;
  int32_t q_dtype, kv_dtype;
  int32_t causal;
} orc_problem;

double orc_bf16_value(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

double orc_e4m3_value(uint8_t code) {
  int negative = code >> 7;
  int e = (code >> 3) & 15;
  int m = code & 7;
  double mag;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    mag = ldexp((double)m, -9); /* subnormal: (m/8) * 2^(1-7) */
  else
    mag = ldexp(1.0 + (double)m / 8.0, e - 7);
  return negative ? -mag : mag;
}

static size_t elem_bytes(int dtype) {
  switch (dtype) {
    case ORC_F32: return 4;
    case ORC_BF16: return 2;
    case ORC_E4M3: return 1;
    default: return 0;
  }
}

static double elem_value(int dtype, const void* base, size_t i) {
  if (dtype == ORC_F32) return (double)((const float*)base)[i];
  if (dtype == ORC_BF16) return orc_bf16_value(((const uint16_t*)base)[i]);
  return orc_e4m3_value(((const uint8_t*)base)[i]);
}

static int check_problem(const orc_problem* pr) {
  if (!pr) return ORC_BAD_ARG;
  if (pr->batch < 0 || pr->q_len <= 0 || pr->num_heads <= 0 || pr->d_latent <= 0 ||
      pr->d_rope < 0 || pr->page_size <= 0 || pr->num_pages <= 0 ||
      pr->max_pages_per_seq <= 0)
    return ORC_BAD_ARG;
  if (pr->q_dtype != ORC_F32 && pr->q_dtype != ORC_BF16) return ORC_BAD_ARG;
  if (!elem_bytes(pr->kv_dtype)) return ORC_BAD_ARG;
  return ORC_OK;
}

/* Physical row index of logical token j of request b, or -1 for a bad page id. */
static int64_t physical_row(const orc_problem* pr, const int32_t* page_table, int b, int j) {
  int32_t page = page_table[(int64_t)b * pr->max_pages_per_seq + j / pr->page_size];
  if (page < 0 || page >= pr->num_pages) return -1;
  return (int64_t)page * pr->page_size + j % pr->page_size;
}

static void decode_row(const orc_problem* pr, const void* kv, const float* kv_scales,
                       int64_t r, double* out) {
  int D = pr->d_latent + pr->d_rope;
  if (pr->kv_dtype == ORC_E4M3) {
    double s = (double)kv_scales[r];
    for (int d = 0; d < D; ++d)
      out[d] = orc_e4m3_value(((const uint8_t*)kv)[r * D + d]) * s;
  } else {
    for (int d = 0; d < D; ++d) out[d] = elem_value(pr->kv_dtype, kv, (size_t)(r * D + d));
  }
}

/* Last visible logical token + 1 for query token t of a request of length L. */
static int visible_end(const orc_problem* pr, int L, int t) {
  return pr->causal ? L - pr->q_len + 1 + t : L;
}

typedef struct {
  const orc_problem* pr;
  const void *q_abs, *q_rope, *kv;
  const float* kv_scales;
  const int32_t* page_table;
  double scale;
} orc_inputs;

/* Scores z_j for j in [begin, end) into z; returns ORC_OK or ORC_BAD_PAGE. */
static int pass_scores(const orc_inputs* in, int b, int t, int h, int begin, int end,
                       double* q, double* row, double* z) {
  const orc_problem* pr = in->pr;
  int Dc = pr->d_latent, Dr = pr->d_rope;
  size_t qi = ((size_t)b * pr->q_len + t) * pr->num_heads + h;
  for (int d = 0; d < Dc; ++d) q[d] = elem_value(pr->q_dtype, in->q_abs, qi * Dc + d);
  for (int e = 0; e < Dr; ++e) q[Dc + e] = elem_value(pr->q_dtype, in->q_rope, qi * Dr + e);
  for (int j = begin; j < end; ++j) {
    int64_t r = physical_row(pr, in->page_table, b, j);
    if (r < 0) return ORC_BAD_PAGE;
    decode_row(pr, in->kv, in->kv_scales, r, row);
    double s = 0.0;
    for (int d = 0; d < Dc + Dr; ++d) s += q[d] * row[d];
    z[j - begin] = in->scale * s;
  }
  return ORC_OK;
}

/* One query row restricted to tokens [jb, je) of the visible set. */
static int attend_row(const orc_inputs* in, int b, int L, int t, int h, int jb, int je,
                      double* o, double* lse, double* q, double* row, double* z) {
  const orc_problem* pr = in->pr;
  int Dc = pr->d_latent;
  int begin = jb < 0 ? 0 : jb;
  int end = visible_end(pr, L, t);
  if (end > je) end = je;
  if (end > L) end = L;
  for (int d = 0; d < Dc; ++d) o[d] = 0.0;
  if (end <= begin) {
    *lse = -INFINITY;
    return ORC_OK;
  }
  /* pass 1: scores */
  int rc = pass_scores(in, b, t, h, begin, end, q, row, z);
  if (rc) return rc;
  /* pass 2: maximum and normaliser */
  double m = -INFINITY;
  for (int j = 0; j < end - begin; ++j)
    if (z[j] > m) m = z[j];
  double l = 0.0;
  for (int j = 0; j < end - begin; ++j) l += exp(z[j] - m);
  /* pass 3: probabilities and the weighted sum of latent rows */
  for (int j = begin; j < end; ++j) {
    double p = exp(z[j - begin] - m) / l;
    decode_row(pr, in->kv, in->kv_scales, physical_row(pr, in->page_table, b, j), row);
    for (int d = 0; d < Dc; ++d) o[d] += p * row[d];
  }
  *lse = m + log(l);
  return ORC_OK;
}

/*
 * Attention for the requests listed in req_ids (NULL: all, in order), each
 * restricted to tokens [tok_begin[i], tok_end[i]) (NULL: the whole request).
 * out: [n_req, T, H, Dc] fp64, lse: [n_req, T, H] fp64.
 */
int orc_attend(const orc_problem* pr, const void* q_abs, const void* q_rope, const void* kv,
               const float* kv_scales, const int32_t* page_table, const int32_t* seq_lens,
               float scale, int32_t n_req, const int32_t* req_ids, const int32_t* tok_begin,
               const int32_t* tok_end, double* out, double* lse, int32_t n_threads) {
  int rc = check_problem(pr);
  if (rc) return rc;
  if (!q_abs || !kv || !page_table || !seq_lens || !out || !lse || n_req < 0) return ORC_BAD_ARG;
  if (pr->d_rope > 0 && !q_rope) return ORC_BAD_ARG;
  if (pr->kv_dtype == ORC_E4M3 && !kv_scales) return ORC_BAD_ARG;
  int maxL = 0;
  for (int i = 0; i < n_req; ++i) {
    int b = req_ids ? req_ids[i] : i;
    if (b < 0 || b >= pr->batch) return ORC_BAD_ARG;
    int L = seq_lens[b];
    if (L < 0 || (int64_t)L > (int64_t)pr->max_pages_per_seq * pr->page_size) return ORC_BAD_ARG;
    if (L > maxL) maxL = L;
  }
  orc_inputs in = {pr, q_abs, q_rope, kv, kv_scales, page_table, (double)scale};
  int T = pr->q_len, H = pr->num_heads, Dc = pr->d_latent, D = pr->d_latent + pr->d_rope;
  int64_t rows = (int64_t)n_req * T * H;
  int status = ORC_OK;
#ifdef _OPENMP
  if (n_threads > 0) omp_set_num_threads(n_threads);
#else
  (void)n_threads;
#endif
#pragma omp parallel
  {
    double* q = (double*)malloc(sizeof(double) * (size_t)D);
    double* row = (double*)malloc(sizeof(double) * (size_t)D);
    double* z = (double*)malloc(sizeof(double) * (size_t)(maxL > 0 ? maxL : 1));
    int local = (q && row && z) ? ORC_OK : ORC_NO_MEM;
#pragma omp for schedule(dynamic, 1)
    for (int64_t x = 0; x < rows; ++x) {
      if (local) continue;
      int i = (int)(x / (T * H));
      int t = (int)((x / H) % T);
      int h = (int)(x % H);
      int b = req_ids ? req_ids[i] : i;
      int jb = tok_begin ? tok_begin[i] : 0;
      int je = tok_end ? tok_end[i] : seq_lens[b];
      int r = attend_row(&in, b, seq_lens[b], t, h, jb, je, out + x * Dc, lse + x, q, row, z);
      if (r) local = r;
    }
    if (local) {
#pragma omp critical
      status = local;
    }
    free(q);
    free(row);
    free(z);
  }
  return status;
}

/* Probabilities p_j of one query row over logical tokens j < L_b (0 where not visible). */
int orc_probs(const orc_problem* pr, const void* q_abs, const void* q_rope, const void* kv,
              const float* kv_scales, const int32_t* page_table, const int32_t* seq_lens,
              float scale, int32_t b, int32_t t, int32_t h, double* p) {
  int rc = check_problem(pr);
  if (rc) return rc;
  if (b < 0 || b >= pr->batch || t < 0 || t >= pr->q_len || h < 0 || h >= pr->num_heads || !p)
    return ORC_BAD_ARG;
  int L = seq_lens[b];
  int D = pr->d_latent + pr->d_rope;
  orc_inputs in = {pr, q_abs, q_rope, kv, kv_scales, page_table, (double)scale};
  for (int j = 0; j < L; ++j) p[j] = 0.0;
  int end = visible_end(pr, L, t);
  if (end <= 0) return ORC_OK;
  double* q = (double*)malloc(sizeof(double) * (size_t)D);
  double* row = (double*)malloc(sizeof(double) * (size_t)D);
  double* z = (double*)malloc(sizeof(double) * (size_t)end);
  if (!q || !row || !z) {
    free(q); free(row); free(z);
    return ORC_NO_MEM;
  }
  rc = pass_scores(&in, b, t, h, 0, end, q, row, z);
  if (!rc) {
    double m = -INFINITY, l = 0.0;
    for (int j = 0; j < end; ++j)
      if (z[j] > m) m = z[j];
    for (int j = 0; j < end; ++j) l += exp(z[j] - m);
    for (int j = 0; j < end; ++j) p[j] = exp(z[j] - m) / l;
  }
  free(q); free(row); free(z);
  return rc;
}

/*
 * Token range of chunk k when a request of length L is cut into S page-aligned
 * chunks: C = P * ceil(ceil(L / S) / P), chunk k = [k C, (k+1) C) clipped to L.
 */
void orc_chunk_bounds(int32_t L, int32_t S, int32_t P, int32_t k, int32_t* begin, int32_t* end) {
  int64_t per = ((int64_t)L + S - 1) / S;
  int64_t C = ((per + P - 1) / P) * P;
  int64_t b0 = (int64_t)k * C, e0 = b0 + C;
  if (b0 > L) b0 = L;
  if (e0 > L) e0 = L;
  *begin = (int32_t)b0;
  *end = (int32_t)e0;
}

/*
 * Merge of per-chunk results (o_k normalised within its chunk, lse_k its
 * log-sum-exp): M = max_k lse_k, w_k = exp(lse_k - M),
 * o = sum_k w_k o_k / sum_k w_k, lse = M + ln sum_k w_k; chunks with
 * lse = -inf weigh nothing, and all-empty rows give o = 0, lse = -inf.
 * o_parts: [n_rows, S, Dc]; lse_parts: [n_rows, S].
 */
int orc_combine(int32_t n_rows, int32_t S, int32_t Dc, const double* o_parts,
                const double* lse_parts, double* out, double* lse) {
  if (n_rows < 0 || S <= 0 || Dc <= 0 || !o_parts || !lse_parts || !out || !lse) return ORC_BAD_ARG;
  for (int64_t r = 0; r < n_rows; ++r) {
    const double* ls = lse_parts + r * S;
    double M = -INFINITY;
    for (int k = 0; k < S; ++k)
      if (ls[k] > M) M = ls[k];
    double* o = out + r * Dc;
    for (int d = 0; d < Dc; ++d) o[d] = 0.0;
    if (M == -INFINITY) {
      lse[r] = -INFINITY;
      continue;
    }
    double wsum = 0.0;
    for (int k = 0; k < S; ++k) {
      if (ls[k] == -INFINITY) continue;
      double w = exp(ls[k] - M);
      wsum += w;
      const double* ok = o_parts + (r * S + k) * Dc;
      for (int d = 0; d < Dc; ++d) o[d] += w * ok[d];
    }
    for (int d = 0; d < Dc; ++d) o[d] /= wsum;
    lse[r] = M + log(wsum);
  }
  return ORC_OK;
}

/* Raw bytes of the stored rows of (b[i], j[i]) through the page table; out: [n, D*elt]. */
int orc_gather_rows(const orc_problem* pr, const void* kv, const int32_t* page_table, int32_t n,
                    const int32_t* b, const int32_t* j, uint8_t* out) {
  int rc = check_problem(pr);
  if (rc) return rc;
  if (!kv || !page_table || !b || !j || !out || n < 0) return ORC_BAD_ARG;
  size_t rb = elem_bytes(pr->kv_dtype) * (size_t)(pr->d_latent + pr->d_rope);
  for (int i = 0; i < n; ++i) {
    if (b[i] < 0 || b[i] >= pr->batch || j[i] < 0 ||
        j[i] >= pr->max_pages_per_seq * pr->page_size)
      return ORC_BAD_ARG;
    int64_t r = physical_row(pr, page_table, b[i], j[i]);
    if (r < 0) return ORC_BAD_PAGE;
    memcpy(out + (size_t)i * rb, (const uint8_t*)kv + (size_t)r * rb, rb);
  }
  return ORC_OK;
}

/*
 * Paged KV append with FP8 packing (the write that produces the cache the
 * decode reads).  Each new row is a token's Dc + Dr values; token t of
 * request b lands at logical position pos0[b] + t, i.e. in page
 * page_table[b][pos / P], slot pos mod P (PagedAttention article on the
 * "推理优化" tag page), and is stored as
 *   - fp32: the value itself;
 *   - bf16: the value rounded to the nearest bf16, ties to even (the upper
 *     half of binary32 after rounding; NaN stays NaN);
 *   - E4M3: one fp32 scale per row, s = absmax / 448 computed in fp32 (448 =
 *     largest finite E4M3, FP8 format table of the quantisation article on
 *     the same tag page), s = 1 for an all-zero row; each value v becomes the
 *     E4M3 code nearest to the fp32 quotient q = v / s (ties to even, |q| >
 *     448 saturates to 448, the sign kept, so -0 gives the code of -0), and s
 *     goes to scales[page][slot].
 * The E4M3 code of q is found from the format's definition: below 2^-6 the
 * values are multiples of 2^-9 (codes 0..7 per sign), from 2^e (e = -6..8)
 * on the step is 2^(e-3); the code of a value is (e + 7) << 3 | mantissa.
 * src: [n_req, T, D] fp32 holding the exact source values.
 */
static uint8_t e4m3_code_of(float q) {
  if (isnan(q)) return 0x7F;
  const uint8_t sign = signbit(q) ? 0x80 : 0x00;
  const double a = fabs((double)q);
  if (a >= 448.0) return sign | 0x7E;
  if (a < ldexp(1.0, -6)) {  /* subnormal range: multiples of 2^-9 (code 8 = 2^-6) */
    const double m = nearbyint(ldexp(a, 9)); /* exact scaling; ties to even */
    return sign | (uint8_t)m;
  }
  int e;
  frexp(a, &e);  /* a = f * 2^e, f in [0.5, 1): a in [2^(e-1), 2^e) */
  e -= 1;        /* a in [2^e, 2^(e+1)) */
  double m = nearbyint(ldexp(a, 3 - e)); /* 8 .. 16 */
  if (m == 16.0) {
    m = 8.0;
    e += 1;
  }
  int code = ((e + 7) << 3) | ((int)m - 8);
  if (code > 0x7E) code = 0x7E;
  return sign | (uint8_t)code;
}

static uint16_t bf16_bits_of(float v) {
  uint32_t u;
  memcpy(&u, &v, 4);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);  /* NaN stays NaN */
  const uint32_t lsb = (u >> 16) & 1u;
  return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

int orc_append_rows(int32_t n_req, int32_t T, int32_t D, const float* src, const int32_t* page_table,
                    int32_t MP, int32_t P, int32_t NP, const int32_t* pos0, int32_t dst_dtype, void* kv,
                    float* scales) {
  if (n_req < 0 || T < 1 || D < 1 || P < 1 || MP < 1 || NP < 1 || !src || !page_table || !pos0 || !kv)
    return ORC_BAD_ARG;
  if (dst_dtype != ORC_F32 && dst_dtype != ORC_BF16 && dst_dtype != ORC_E4M3) return ORC_BAD_ARG;
  if (dst_dtype == ORC_E4M3 && !scales) return ORC_BAD_ARG;
  for (int b = 0; b < n_req; ++b) {
    for (int t = 0; t < T; ++t) {
      const int64_t pos = (int64_t)pos0[b] + t;
      if (pos < 0 || pos >= (int64_t)MP * P) return ORC_BAD_ARG;
      const int32_t page = page_table[(size_t)b * MP + pos / P];
      if (page < 0 || page >= NP) return ORC_BAD_PAGE;
      const size_t row = (size_t)page * P + (size_t)(pos % P);
      const float* x = src + ((size_t)b * T + t) * D;
      if (dst_dtype == ORC_F32) {
        memcpy((float*)kv + row * D, x, sizeof(float) * (size_t)D);
      } else if (dst_dtype == ORC_BF16) {
        uint16_t* o = (uint16_t*)kv + row * D;
        for (int d = 0; d < D; ++d) o[d] = bf16_bits_of(x[d]);
      } else {
        float amax = 0.0f;
        for (int d = 0; d < D; ++d) {
          const float a = fabsf(x[d]);
          if (a > amax) amax = a;
        }
        const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
        uint8_t* o = (uint8_t*)kv + row * D;
        for (int d = 0; d < D; ++d) o[d] = e4m3_code_of(x[d] / s);
        scales[row] = s;
      }
    }
  }
  return ORC_OK;
}

/*
 * Greedy verification of a linear chain of drafts (TokenSpeed code-audit
 * article, complete technology list: speculative decoding entries, greedy
 * linear-chain verification).  Request b has T query positions: position 0
 * holds the last accepted token, positions 1..T-1 the drafts d[b][0..T-2].
 * The target's prediction at position t is p_t = argmax_v logits[b][t][v]
 * (values compared exactly as stored; the smallest v among equal maxima;
 * NaN never wins).  Draft i is accepted iff d[b][i] == p_i and every draft
 * before it was accepted (a running product of matches), so n = number of
 * leading matches, 0 <= n <= T-1.  The step emits the n accepted drafts and
 * then the target's own token at the first unaccepted position, p_n (the
 * bonus token when all drafts pass); out[b] = d[0..n-1], p_n, then -1.
 * logits: [B, T, V] as fp64 values of the stored numbers.
 */
int orc_verify_greedy(int32_t B, int32_t T, int32_t V, const double* logits, const int32_t* draft,
                      int32_t* argmax, int32_t* accept_len, int32_t* out) {
  if (B < 0 || T < 1 || V < 1 || !logits || (T > 1 && !draft) || !argmax || !accept_len || !out)
    return ORC_BAD_ARG;
  for (int b = 0; b < B; ++b) {
    for (int t = 0; t < T; ++t) {
      const double* row = logits + ((size_t)b * T + t) * V;
      int best = -1;
      for (int v = 0; v < V; ++v) {
        if (isnan(row[v])) continue;
        if (best < 0 || row[v] > row[best]) best = v;
      }
      argmax[(size_t)b * T + t] = best < 0 ? 0 : best;
    }
    int n = 0;
    while (n < T - 1 && draft[(size_t)b * (T - 1) + n] == argmax[(size_t)b * T + n]) ++n;
    accept_len[b] = n;
    for (int i = 0; i < T; ++i) {
      int32_t tok = -1;
      if (i < n) tok = draft[(size_t)b * (T - 1) + i];
      else if (i == n) tok = argmax[(size_t)b * T + n];
      out[(size_t)b * T + i] = tok;
    }
  }
  return ORC_OK;
}

/*
 * Per-head projection on either side of the latent attention (the absorbed
 * projections of the code-audit article's MLA entry): for row m and head g,
 *   out[m][g][n] = sum_k W[g][n][k] * x[m][g][k]
 * in fp64, k in order.  With W[g] = W_UK^g transposed (d_latent x d_nope)
 * and x = q_nope this forms the absorbed query q_abs = W_UK^T q_nope; with
 * W[g] = W_UV^g (d_v x d_latent) and x = the attention output o it forms the
 * head's value output W_UV o.  x: [M, G, K], W: [G, N, K], out: [M, G, N].
 */
int orc_project(int32_t M, int32_t G, int32_t K, int32_t N, const double* x, const double* w, double* out) {
  if (M < 0 || G < 1 || K < 1 || N < 1 || !x || !w || !out) return ORC_BAD_ARG;
#ifdef _OPENMP
#pragma omp parallel for collapse(2) schedule(static)
#endif
  for (int m = 0; m < M; ++m)
    for (int g = 0; g < G; ++g) {
      const double* xr = x + ((size_t)m * G + g) * K;
      for (int n = 0; n < N; ++n) {
        const double* wr = w + ((size_t)g * N + n) * K;
        double acc = 0.0;
        for (int k = 0; k < K; ++k) acc += wr[k] * xr[k];
        out[((size_t)m * G + g) * N + n] = acc;
      }
    }
  return ORC_OK;
}

/* E4M3 code of one fp32 value (for pinning the encoder on its own). */
uint8_t orc_e4m3_code(float q) { return e4m3_code_of(q); }
uint16_t orc_bf16_bits(float v) { return bf16_bits_of(v); }

int orc_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
