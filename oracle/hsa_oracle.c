/*
 * hsa_oracle.c - plain, slow, double-precision CPU oracle for hierarchical
 * sparse attention (HSA) and its dynamic variant (DHSA).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code with
 * the GPU library: no kernels, headers, helpers or constants.
 *
 * Every input element (bf16 or fp32) is exactly representable in double, and
 * all arithmetic below is done in double.  Each step follows the pages in
 * their order; loops are written for clarity, not speed (OpenMP over
 * independent query rows only).
 *
 * Sources (web pages; cited by title and section):
 *  [HSA]  "Understanding and Improving Length Generalization in Hierarchical
 *         Sparse Attention Models" (ai.info summary of arXiv 2510.17196):
 *         Methodology (chunking layer, landmark per chunk, retrieval of the
 *         top-few chunks; chunk size 64, Top-K 8, receptive field 512);
 *         Key Contributions 1 (landmark aggregation f, intra-chunk g).
 *  [HiLS] mlsift "length extrapolation" page, HiLS abstract: each query
 *         attends independently inside every retrieved chunk and the chunk
 *         outputs are fused according to the chunk retrieval scores.
 *  [DHSA] pith.science review of arXiv 2510.24606 (Dynamic Hierarchical
 *         Sparse Attention): "What carries the argument" (sqrt|C|-scaled mean
 *         pooling of queries and keys, chunk similarity S_c, tiling of S_c
 *         into the token map S_t, TopK with budget N_b into mask M);
 *         Referee report, major comment 2 (Eq. 4 and the tiling rule) and
 *         minor comment on Algorithm 1 (top N_b preceding keys).
 *
 * Readings where the pages are silent (each one is a stated choice):
 *  - a chunk is available to query t when all of its tokens precede t,
 *    (c+1)*S <= t; a query with no available chunk outputs zero;
 *  - landmark = (sum of the chunk's S keys) / sqrt(S) (the sqrt(S)-scaled
 *    mean), and both retrieval scores and in-chunk logits use 1/sqrt(d);
 *  - with grouped query heads (head h uses KV head h / (Hq/Hkv)) the chunk
 *    selection is shared by the group and ranks the sum of the group's
 *    per-head scores; each head fuses with its own per-head scores;
 *  - ties rank the lower chunk index (DHSA: lower token index) first;
 *  - a trailing partial chunk (L not a multiple of S) has no landmark and is
 *    never available;
 *  - DHSA: S_c = q_hat . k_hat with no 1/sqrt(d); query i may keep keys
 *    j <= i; it keeps the first min(N_b, i+1) of them in (score desc, j asc)
 *    order; attention logits use 1/sqrt(d);
 *  - DHSA decode (the decode-time update of [DHSA] Referee report, minor
 *    comment on Algorithm 2, where the last chunk holds the current query):
 *    the new query i sits in the current chunk [b_n, i], which is pooled
 *    like any chunk over the tokens it has so far (its queries and keys
 *    b_n..i); the complete chunks 0..n-1 and the current one are scored,
 *    tiled to tokens j <= i and cut at min(N_b, i+1) exactly as in prefill,
 *    so a decode step equals prefill row i of the sequence cut at i+1.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F32 = 0, OR_BF16 = 1 };

/* Number of threads the oracle's parallel loops use. */
int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

enum {
  OR_OK = 0,
  OR_EINVAL = 1,
  OR_ENOMEM = 2,
};

/* One input element as a double (bf16 bits widen exactly). */
static double ld(const void* p, int dtype, int64_t i) {
  if (dtype == OR_F32) return (double)((const float*)p)[i];
  uint32_t b = (uint32_t)((const uint16_t*)p)[i] << 16;
  float f;
  memcpy(&f, &b, sizeof f);
  return (double)f;
}

/* ------------------------------------------------------------------------ */
/* Landmarks: [HSA] Methodology, landmark vector per chunk; mean pooling     */
/* scaled by sqrt(S) (the same sqrt|C| scaling as [DHSA]).                   */
/* ------------------------------------------------------------------------ */

/* lmk[b,h,c,:] = sum_{j<S} K[b,h,c*S+j,:] / sqrt(S) for c < floor(L/S). */
int oracle_landmarks(const void* K, int dtype, int64_t B, int64_t H, int64_t L, int64_t d,
                     int64_t S, double* lmk) {
  if (!K || !lmk || B < 0 || H < 0 || L < 0 || d <= 0 || S <= 0) return OR_EINVAL;
  const int64_t n = L / S;
  const double rs = sqrt((double)S);
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t bh = 0; bh < B * H; ++bh)
    for (int64_t c = 0; c < n; ++c)
      for (int64_t x = 0; x < d; ++x) {
        double acc = 0.0;
        for (int64_t j = 0; j < S; ++j) acc += ld(K, dtype, (bh * L + c * S + j) * d + x);
        lmk[(bh * n + c) * d + x] = acc / rs;
      }
  return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Shared helpers of the HSA steps.                                          */
/* ------------------------------------------------------------------------ */

typedef struct {
  double score;
  int64_t idx;
} cand_t;

/* Total order: larger score first, then lower index. */
static int cand_cmp(const void* a, const void* b) {
  const cand_t* x = (const cand_t*)a;
  const cand_t* y = (const cand_t*)b;
  if (x->score > y->score) return -1;
  if (x->score < y->score) return 1;
  return (x->idx < y->idx) ? -1 : (x->idx > y->idx);
}

/* Softmax attention of one query over keys/values rows [j0, j1) of a [N,d]
 * slab (K and V at element offset base): o = sum_j p_j v_j,
 * p = softmax_j(q . k_j / sqrt(d)).  Returns the log-sum-exp. */
static double attend_rows(const double* q, const void* K, const void* V, int dtype,
                          int64_t base, int64_t j0, int64_t j1, int64_t d, double* o,
                          double* work) {
  const double sc = 1.0 / sqrt((double)d);
  double mx = -INFINITY;
  for (int64_t j = j0; j < j1; ++j) {
    double a = 0.0;
    for (int64_t x = 0; x < d; ++x) a += q[x] * ld(K, dtype, base + j * d + x);
    a *= sc;
    work[j - j0] = a;
    if (a > mx) mx = a;
  }
  double z = 0.0;
  for (int64_t j = j0; j < j1; ++j) {
    work[j - j0] = exp(work[j - j0] - mx);
    z += work[j - j0];
  }
  for (int64_t x = 0; x < d; ++x) o[x] = 0.0;
  for (int64_t j = j0; j < j1; ++j) {
    const double p = work[j - j0] / z;
    for (int64_t x = 0; x < d; ++x) o[x] += p * ld(V, dtype, base + j * d + x);
  }
  return mx + log(z);
}

/* ------------------------------------------------------------------------ */
/* HSA prefill: [HSA] Methodology + [HiLS] abstract.                         */
/* ------------------------------------------------------------------------ */

/*
 * Q [B,Hq,L,d], K and V [B,Hkv,L,d] (dtype), for the query positions
 * rows[0..n_rows) (rows == NULL: all L positions).  Outputs, all indexed by
 * row r rather than by position:
 *   out    [B,Hq,n_rows,d]       fused output (zero if no chunk is available)
 *   sel    [B,Hkv,n_rows,topk]   selected chunks in rank order, -1 padded
 *   w      [B,Hq,n_rows,topk]    fusion weights in the same order, 0 padded
 *   margin [B,Hkv,n_rows]        sigma_(K) - sigma_(K+1) of the group-summed
 *                                scores, +inf when at most K are available
 *   sel_score [B,Hkv,n_rows,topk] group-summed score of each selected chunk,
 *                                -inf padded
 * Any output pointer may be NULL.  include_current_chunk (oracle-only switch
 * used to pin the dense-causal reduction) also makes the chunk holding t
 * available, with its keys restricted to j <= t.
 *
 * interval R >= 1 is the retrieval interval ([HSA] Key Contributions 4 and
 * Main Findings: retrieval refreshed every R tokens, per-token vs per-8-token
 * retrieval).  Row t reuses the selection made at the first token of its
 * block, t0 = floor(t/R)*R: the chunks available at t0 ranked by the group
 * sum of q_t0 . lambda_c / sqrt(d).  The row then attends inside those
 * chunks with its own query and fuses with its own per-head scores.  R = 1
 * is per-token retrieval.  sel, margin and sel_score describe t0's
 * selection.
 */
int oracle_hsa_prefill(const void* Q, const void* K, const void* V, int dtype, int64_t B,
                       int64_t L, int64_t Hq, int64_t Hkv, int64_t d, int64_t S, int64_t topk,
                       const int64_t* rows, int64_t n_rows, int include_current_chunk,
                       int64_t interval, double* out, int32_t* sel, double* w, double* margin,
                       double* sel_score) {
  if (!Q || !K || !V || B < 0 || L < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || d <= 0 ||
      S <= 0 || topk <= 0 || interval <= 0)
    return OR_EINVAL;
  if (!rows) n_rows = L;
  const int64_t G = Hq / Hkv;
  const int64_t n = L / S;
  const double sc = 1.0 / sqrt((double)d);

  /* Step 1: landmarks of every complete chunk. */
  double* lmk = (double*)malloc((size_t)(B * Hkv * (n > 0 ? n : 1) * d) * sizeof(double));
  if (!lmk) return OR_ENOMEM;
  oracle_landmarks(K, dtype, B, Hkv, L, d, S, lmk);

  int err = OR_OK;
#pragma omp parallel
  {
    cand_t* cand = (cand_t*)malloc((size_t)(n + 1) * sizeof(cand_t));
    double* sh = (double*)malloc((size_t)(G * (n + 1)) * sizeof(double));
    double* qv = (double*)malloc((size_t)(G * d) * sizeof(double));
    double* qs = (double*)malloc((size_t)(G * d) * sizeof(double));
    double* oc = (double*)malloc((size_t)d * sizeof(double));
    double* work = (double*)malloc((size_t)(S + 1) * sizeof(double));
    if (!cand || !sh || !qv || !qs || !oc || !work) {
#pragma omp atomic write
      err = OR_ENOMEM;
    } else {
#pragma omp for collapse(3) schedule(dynamic, 16)
      for (int64_t b = 0; b < B; ++b)
        for (int64_t g = 0; g < Hkv; ++g)
          for (int64_t r = 0; r < n_rows; ++r) {
            const int64_t t = rows ? rows[r] : r;
            const int64_t t0 = t / interval * interval;  /* where the selection is made */
            const int64_t kv_base = (b * Hkv + g) * L * d;
            /* Step 2: available chunks A(t0). */
            int64_t navail = include_current_chunk ? (t0 / S + 1) : (t0 / S);
            if (navail > n) navail = n;
            if (navail < 0) navail = 0;
            /* Query rows of the group's heads at t (attention, fusion) and
             * at t0 (selection). */
            for (int64_t hh = 0; hh < G; ++hh)
              for (int64_t x = 0; x < d; ++x) {
                qv[hh * d + x] = ld(Q, dtype, ((b * Hq + g * G + hh) * L + t) * d + x);
                qs[hh * d + x] = ld(Q, dtype, ((b * Hq + g * G + hh) * L + t0) * d + x);
              }
            /* Step 3: per-head scores s_h(t,c) of the row and the group sum
             * sigma at t0.  sigma = (sum over heads of q . lambda) / sqrt(d):
             * the positive factor is applied once to the summed dot products,
             * so scores that are exactly equal stay equal for the tie rule
             * (rounding each head's scaled term first could split them). */
            for (int64_t c = 0; c < navail; ++c) {
              const double* lc = lmk + ((b * Hkv + g) * n + c) * d;
              double sigma = 0.0;
              for (int64_t hh = 0; hh < G; ++hh) {
                double s = 0.0, s0 = 0.0;
                for (int64_t x = 0; x < d; ++x) s += qv[hh * d + x] * lc[x];
                for (int64_t x = 0; x < d; ++x) s0 += qs[hh * d + x] * lc[x];
                sh[hh * (n + 1) + c] = s * sc;
                sigma += s0;
              }
              cand[c].score = sigma * sc;
              cand[c].idx = c;
            }
            /* Step 4: top-min(K, |A|) by (sigma desc, c asc). */
            qsort(cand, (size_t)navail, sizeof(cand_t), cand_cmp);
            const int64_t m = navail < topk ? navail : topk;
            if (margin)
              margin[(b * Hkv + g) * n_rows + r] =
                  navail > topk ? cand[topk - 1].score - cand[topk].score : INFINITY;
            if (sel)
              for (int64_t k = 0; k < topk; ++k)
                sel[((b * Hkv + g) * n_rows + r) * topk + k] = k < m ? (int32_t)cand[k].idx : -1;
            if (sel_score)
              for (int64_t k = 0; k < topk; ++k)
                sel_score[((b * Hkv + g) * n_rows + r) * topk + k] =
                    k < m ? cand[k].score : -INFINITY;
            for (int64_t hh = 0; hh < G; ++hh) {
              const int64_t h = g * G + hh;
              double* orow = out ? out + ((b * Hq + h) * n_rows + r) * d : NULL;
              double* wrow = w ? w + ((b * Hq + h) * n_rows + r) * topk : NULL;
              if (orow)
                for (int64_t x = 0; x < d; ++x) orow[x] = 0.0;
              if (wrow)
                for (int64_t k = 0; k < topk; ++k) wrow[k] = 0.0;
              if (m == 0) continue;
              /* Step 6 weights: softmax over the kept chunks of this head's
               * own scores. */
              double smax = -INFINITY;
              for (int64_t k = 0; k < m; ++k) {
                const double s = sh[hh * (n + 1) + cand[k].idx];
                if (s > smax) smax = s;
              }
              double zs = 0.0;
              for (int64_t k = 0; k < m; ++k) zs += exp(sh[hh * (n + 1) + cand[k].idx] - smax);
              for (int64_t k = 0; k < m; ++k) {
                const int64_t c = cand[k].idx;
                const double wk = exp(sh[hh * (n + 1) + c] - smax) / zs;
                if (wrow) wrow[k] = wk;
                if (!orow) continue;
                /* Step 5: attention inside chunk c (keys j <= t only when the
                 * chunk holds t, which happens only with the switch on). */
                int64_t j1 = (c + 1) * S;
                if (j1 > t + 1) j1 = t + 1;
                attend_rows(qv + hh * d, K, V, dtype, kv_base, c * S, j1, d, oc, work);
                for (int64_t x = 0; x < d; ++x) orow[x] += wk * oc[x];
              }
            }
          }
    }
    free(cand);
    free(sh);
    free(qv);
    free(qs);
    free(oc);
    free(work);
  }
  free(lmk);
  return err;
}

/* ------------------------------------------------------------------------ */
/* HSA decode: one query per sequence at position n_ctx, all complete chunks */
/* of the context available.  Split into the selection step and the          */
/* attend+fuse step so huge caches need only the selected chunks on the host.*/
/* ------------------------------------------------------------------------ */

/*
 * q [B,Hq,d] (dtype), lmk [B,Hkv,n_lmk,d] fp32 landmarks as handed to the GPU
 * (n_lmk >= floor(n_ctx/S)).  Outputs sel [B,Hkv,topk] (-1 padded), margin
 * [B,Hkv] and sel_score [B,Hkv,topk] (-inf padded); any may be NULL
 * (group-summed scores as in prefill).
 */
int oracle_hsa_decode_select(const void* q, int dtype, const float* lmk, int64_t B,
                             int64_t Hq, int64_t Hkv, int64_t d, int64_t S, int64_t n_ctx,
                             int64_t n_lmk, int64_t topk, int32_t* sel, double* margin,
                             double* sel_score) {
  if (!q || !lmk || B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || d <= 0 || S <= 0 ||
      topk <= 0 || n_ctx < 0 || n_lmk < n_ctx / S)
    return OR_EINVAL;
  const int64_t G = Hq / Hkv;
  const int64_t navail = n_ctx / S;
  const double sc = 1.0 / sqrt((double)d);
  int err = OR_OK;
  for (int64_t b = 0; b < B; ++b)
    for (int64_t g = 0; g < Hkv; ++g) {
      cand_t* cand = (cand_t*)malloc((size_t)(navail + 1) * sizeof(cand_t));
      if (!cand) return OR_ENOMEM;
#pragma omp parallel for schedule(static)
      for (int64_t c = 0; c < navail; ++c) {
        const float* lc = lmk + ((b * Hkv + g) * n_lmk + c) * d;
        /* group sum of the dot products, scaled once (as in prefill) */
        double sigma = 0.0;
        for (int64_t hh = 0; hh < G; ++hh) {
          double s = 0.0;
          for (int64_t x = 0; x < d; ++x) s += ld(q, dtype, (b * Hq + g * G + hh) * d + x) * (double)lc[x];
          sigma += s;
        }
        cand[c].score = sigma * sc;
        cand[c].idx = c;
      }
      qsort(cand, (size_t)navail, sizeof(cand_t), cand_cmp);
      const int64_t m = navail < topk ? navail : topk;
      if (sel)
        for (int64_t k = 0; k < topk; ++k)
          sel[(b * Hkv + g) * topk + k] = k < m ? (int32_t)cand[k].idx : -1;
      if (margin)
        margin[b * Hkv + g] = navail > topk ? cand[topk - 1].score - cand[topk].score : INFINITY;
      if (sel_score)
        for (int64_t k = 0; k < topk; ++k)
          sel_score[(b * Hkv + g) * topk + k] = k < m ? cand[k].score : -INFINITY;
      free(cand);
    }
  return err;
}

/*
 * Attend + fuse for decode, given the selection.  Kc, Vc hold the selected
 * chunks packed in selection order: [B,Hkv,topk,S,d] (dtype; slots whose sel
 * entry is -1 are ignored), lmk_sel [B,Hkv,topk,d] fp32 their landmarks.
 * out [B,Hq,d] (zero when nothing is selected), w [B,Hq,topk] (may be NULL).
 */
int oracle_hsa_decode_attend(const void* q, const void* Kc, const void* Vc, int dtype,
                             const float* lmk_sel, const int32_t* sel, int64_t B, int64_t Hq,
                             int64_t Hkv, int64_t d, int64_t S, int64_t topk, double* out,
                             double* w) {
  if (!q || !Kc || !Vc || !lmk_sel || !sel || !out || B < 0 || Hq <= 0 || Hkv <= 0 ||
      Hq % Hkv || d <= 0 || S <= 0 || topk <= 0)
    return OR_EINVAL;
  const int64_t G = Hq / Hkv;
  const double sc = 1.0 / sqrt((double)d);
  int err = OR_OK;
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t b = 0; b < B; ++b)
    for (int64_t h = 0; h < Hq; ++h) {
      const int64_t g = h / G;
      double* qv = (double*)malloc((size_t)d * sizeof(double));
      double* oc = (double*)malloc((size_t)d * sizeof(double));
      double* work = (double*)malloc((size_t)S * sizeof(double));
      double* sh = (double*)malloc((size_t)topk * sizeof(double));
      if (!qv || !oc || !work || !sh) {
#pragma omp atomic write
        err = OR_ENOMEM;
      } else {
        for (int64_t x = 0; x < d; ++x) qv[x] = ld(q, dtype, (b * Hq + h) * d + x);
        double* orow = out + (b * Hq + h) * d;
        for (int64_t x = 0; x < d; ++x) orow[x] = 0.0;
        if (w)
          for (int64_t k = 0; k < topk; ++k) w[(b * Hq + h) * topk + k] = 0.0;
        int64_t m = 0;
        while (m < topk && sel[(b * Hkv + g) * topk + m] >= 0) ++m;
        double smax = -INFINITY;
        for (int64_t k = 0; k < m; ++k) {
          const float* lc = lmk_sel + ((b * Hkv + g) * topk + k) * d;
          double s = 0.0;
          for (int64_t x = 0; x < d; ++x) s += qv[x] * (double)lc[x];
          sh[k] = s * sc;
          if (sh[k] > smax) smax = sh[k];
        }
        double zs = 0.0;
        for (int64_t k = 0; k < m; ++k) zs += exp(sh[k] - smax);
        for (int64_t k = 0; k < m; ++k) {
          const double wk = exp(sh[k] - smax) / zs;
          if (w) w[(b * Hq + h) * topk + k] = wk;
          const int64_t base = ((b * Hkv + g) * topk + k) * S * d;
          attend_rows(qv, Kc, Vc, dtype, base, 0, S, d, oc, work);
          for (int64_t x = 0; x < d; ++x) orow[x] += wk * oc[x];
        }
      }
      free(qv);
      free(oc);
      free(work);
      free(sh);
    }
  return err;
}

/* ------------------------------------------------------------------------ */
/* DHSA prefill: [DHSA] "What carries the argument", Eq. 4, tiling rule,     */
/* TopK with budget N_b over preceding keys, masked softmax attention.       */
/* ------------------------------------------------------------------------ */

typedef struct {
  double score;
  int64_t j;
} tok_t;

static int tok_cmp(const void* a, const void* b) {
  const tok_t* x = (const tok_t*)a;
  const tok_t* y = (const tok_t*)b;
  if (x->score > y->score) return -1;
  if (x->score < y->score) return 1;
  return (x->j < y->j) ? -1 : (x->j > y->j);
}

/*
 * Q, K, V [B,H,L,d] (dtype); offsets [nc+1] with 0 = b_0 < ... < b_nc = L
 * (chunk l holds tokens [b_l, b_{l+1})); budget N_b > 0.  For query positions
 * rows[0..n_rows) (NULL: all):
 *   out    [B,H,n_rows,d]   attention over the kept keys
 *   Sc     [B,H,nc,nc]      chunk similarity (every l,k; may be NULL)
 *   n_kept [B,H,n_rows]     min(N_b, i+1) (may be NULL)
 *   kept   [B,H,n_rows,L]   1 where key j is kept for the row (may be NULL)
 *   margin [B,H,n_rows]     smallest score gap between the cut chunk and its
 *                           neighbours in the chunk ranking; +inf when every
 *                           causal key is kept
 */
int oracle_dhsa_prefill(const void* Q, const void* K, const void* V, int dtype, int64_t B,
                        int64_t L, int64_t H, int64_t d, const int32_t* offsets, int64_t nc,
                        int64_t budget, const int64_t* rows, int64_t n_rows, double* out,
                        double* Sc, int32_t* n_kept, uint8_t* kept, double* margin) {
  if (!Q || !K || !V || !offsets || B < 0 || L < 0 || H <= 0 || d <= 0 || nc < 0 ||
      budget <= 0)
    return OR_EINVAL;
  if (offsets[0] != 0 || offsets[nc] != L) return OR_EINVAL;
  for (int64_t l = 0; l < nc; ++l)
    if (offsets[l + 1] <= offsets[l]) return OR_EINVAL;
  if (!rows) n_rows = L;
  const double sc = 1.0 / sqrt((double)d);
  int64_t* chunk_of = (int64_t*)malloc((size_t)(L + 1) * sizeof(int64_t));
  double* qh = (double*)malloc((size_t)((nc + 1) * d) * sizeof(double));
  double* kh = (double*)malloc((size_t)((nc + 1) * d) * sizeof(double));
  double* sc_m = (double*)malloc((size_t)((nc + 1) * (nc + 1)) * sizeof(double));
  if (!chunk_of || !qh || !kh || !sc_m) {
    free(chunk_of); free(qh); free(kh); free(sc_m);
    return OR_ENOMEM;
  }
  for (int64_t l = 0; l < nc; ++l)
    for (int64_t i = offsets[l]; i < offsets[l + 1]; ++i) chunk_of[i] = l;

  int err = OR_OK;
  for (int64_t b = 0; b < B; ++b)
    for (int64_t h = 0; h < H; ++h) {
      const int64_t base = (b * H + h) * L * d;
      /* Eq. 4: q_hat_l = sqrt|C_l| * mean(Q over C_l) = sum / sqrt|C_l|. */
#pragma omp parallel for schedule(static)
      for (int64_t l = 0; l < nc; ++l) {
        const int64_t len = offsets[l + 1] - offsets[l];
        for (int64_t x = 0; x < d; ++x) {
          double aq = 0.0, ak = 0.0;
          for (int64_t i = offsets[l]; i < offsets[l + 1]; ++i) {
            aq += ld(Q, dtype, base + i * d + x);
            ak += ld(K, dtype, base + i * d + x);
          }
          qh[l * d + x] = aq / sqrt((double)len);
          kh[l * d + x] = ak / sqrt((double)len);
        }
      }
      /* S_c[l,k] = q_hat_l . k_hat_k. */
#pragma omp parallel for collapse(2) schedule(static)
      for (int64_t l = 0; l < nc; ++l)
        for (int64_t k = 0; k < nc; ++k) {
          double s = 0.0;
          for (int64_t x = 0; x < d; ++x) s += qh[l * d + x] * kh[k * d + x];
          sc_m[l * nc + k] = s;
        }
      if (Sc) memcpy(Sc + (b * H + h) * nc * nc, sc_m, (size_t)(nc * nc) * sizeof(double));

#pragma omp parallel
      {
        tok_t* tok = (tok_t*)malloc((size_t)(L + 1) * sizeof(tok_t));
        double* qv = (double*)malloc((size_t)d * sizeof(double));
        double* logit = (double*)malloc((size_t)(L + 1) * sizeof(double));
        if (!tok || !qv || !logit) {
#pragma omp atomic write
          err = OR_ENOMEM;
        } else {
#pragma omp for schedule(dynamic, 8)
          for (int64_t r = 0; r < n_rows; ++r) {
            const int64_t i = rows ? rows[r] : r;
            const int64_t l = chunk_of[i];
            /* Upsampling by tiling: S_t[i,j] = S_c[chunk(i), chunk(j)],
             * candidates j <= i. */
            for (int64_t j = 0; j <= i; ++j) {
              tok[j].score = sc_m[l * nc + chunk_of[j]];
              tok[j].j = j;
            }
            qsort(tok, (size_t)(i + 1), sizeof(tok_t), tok_cmp);
            const int64_t keep = (i + 1) < budget ? (i + 1) : budget;
            if (n_kept) n_kept[(b * H + h) * n_rows + r] = (int32_t)keep;
            uint8_t* krow = kept ? kept + ((b * H + h) * n_rows + r) * L : NULL;
            if (krow) {
              memset(krow, 0, (size_t)L);
              for (int64_t p = 0; p < keep; ++p) krow[tok[p].j] = 1;
            }
            if (margin) {
              double mg = INFINITY;
              if (keep < i + 1) {
                /* Chunk ranking around the cut: the chunk of the first
                 * dropped token (cut chunk), the chunk ranked just above it
                 * and the one just below. */
                const int64_t ccut = chunk_of[tok[keep].j];
                const double scut = tok[keep].score;
                int64_t p = keep;
                while (p > 0 && chunk_of[tok[p - 1].j] == ccut) --p;
                if (p > 0) mg = fmin(mg, tok[p - 1].score - scut);
                p = keep;
                while (p <= i && chunk_of[tok[p].j] == ccut) ++p;
                if (p <= i) mg = fmin(mg, scut - tok[p].score);
              }
              margin[(b * H + h) * n_rows + r] = mg;
            }
            /* Masked softmax attention over the kept keys. */
            for (int64_t x = 0; x < d; ++x) qv[x] = ld(Q, dtype, base + i * d + x);
            double mx = -INFINITY;
            for (int64_t p = 0; p < keep; ++p) {
              double a = 0.0;
              for (int64_t x = 0; x < d; ++x) a += qv[x] * ld(K, dtype, base + tok[p].j * d + x);
              logit[p] = a * sc;
              if (logit[p] > mx) mx = logit[p];
            }
            double z = 0.0;
            for (int64_t p = 0; p < keep; ++p) {
              logit[p] = exp(logit[p] - mx);
              z += logit[p];
            }
            if (out) {
              double* orow = out + ((b * H + h) * n_rows + r) * d;
              for (int64_t x = 0; x < d; ++x) orow[x] = 0.0;
              for (int64_t p = 0; p < keep; ++p) {
                const double pw = logit[p] / z;
                for (int64_t x = 0; x < d; ++x)
                  orow[x] += pw * ld(V, dtype, base + tok[p].j * d + x);
              }
            }
          }
        }
        free(tok);
        free(qv);
        free(logit);
      }
    }
  free(chunk_of);
  free(qh);
  free(kh);
  free(sc_m);
  return err;
}


/*
 * DHSA pooled chunk keys ([DHSA] "What carries the argument", Eq. 4):
 * k_hat_k = (sum of the keys of chunk k) / sqrt|C_k| for chunks
 * k = 0..n-1 with boundaries offsets[0..n] (0 = b_0 < ... < b_n <= N).
 *   K     [B,H,N,d] dtype
 *   khat  [B,H,n,d]
 */
int oracle_dhsa_chunk_keys(const void* K, int dtype, int64_t B, int64_t H, int64_t N, int64_t d,
                           const int32_t* offsets, int64_t n, double* khat) {
  if (!K || !offsets || !khat || B < 0 || H <= 0 || N < 0 || d <= 0 || n < 0) return OR_EINVAL;
  if (offsets[0] != 0 || offsets[n] > N) return OR_EINVAL;
  for (int64_t k = 0; k < n; ++k)
    if (offsets[k + 1] <= offsets[k]) return OR_EINVAL;
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t bh = 0; bh < B * H; ++bh)
    for (int64_t k = 0; k < n; ++k) {
      const int64_t len = offsets[k + 1] - offsets[k];
      for (int64_t x = 0; x < d; ++x) {
        double a = 0.0;
        for (int64_t j = offsets[k]; j < offsets[k + 1]; ++j) a += ld(K, dtype, (bh * N + j) * d + x);
        khat[(bh * n + k) * d + x] = a / sqrt((double)len);
      }
    }
  return OR_OK;
}

/*
 * DHSA decode: one new query at position pos = b_n + m - 1 per (b, h).
 *   Qcur   [B,H,m,d] dtype: the queries of the current chunk b_n..pos (the
 *          last row is the new query)
 *   K, V   [B,H,N,d] dtype caches; rows 0..pos are used
 *   offsets[0..n] boundaries of the n complete chunks (b_n <= pos < N)
 *   budget N_b >= 1
 * Outputs (any may be NULL):
 *   out    [B,H,d]
 *   Sc     [B,H,n+1]  chunk scores q_hat . k_hat_k, k = n is the current chunk
 *   n_kept [B,H]      number of kept keys, min(N_b, pos+1)
 *   kept   [B,H,pos+1] 1 where key j is kept
 *   margin [B,H]      as in oracle_dhsa_prefill
 */
int oracle_dhsa_decode(const void* Qcur, const void* K, const void* V, int dtype, int64_t B,
                       int64_t H, int64_t d, int64_t m, int64_t N, const int32_t* offsets,
                       int64_t n, int64_t budget, double* out, double* Sc, int32_t* n_kept,
                       uint8_t* kept, double* margin) {
  if (!Qcur || !K || !V || !offsets || B < 0 || H <= 0 || d <= 0 || m < 1 || n < 0 ||
      budget <= 0)
    return OR_EINVAL;
  if (offsets[0] != 0) return OR_EINVAL;
  for (int64_t k = 0; k < n; ++k)
    if (offsets[k + 1] <= offsets[k]) return OR_EINVAL;
  const int64_t pos = offsets[n] + m - 1;
  if (pos >= N) return OR_EINVAL;
  const int64_t nc = n + 1;  /* complete chunks plus the current one */
  const double sc = 1.0 / sqrt((double)d);
  int64_t* chunk_of = (int64_t*)malloc((size_t)(pos + 1) * sizeof(int64_t));
  int64_t* bnd = (int64_t*)malloc((size_t)(nc + 1) * sizeof(int64_t));
  if (!chunk_of || !bnd) {
    free(chunk_of); free(bnd);
    return OR_ENOMEM;
  }
  for (int64_t k = 0; k <= n; ++k) bnd[k] = offsets[k];
  bnd[nc] = pos + 1;
  for (int64_t k = 0; k < nc; ++k)
    for (int64_t j = bnd[k]; j < bnd[k + 1]; ++j) chunk_of[j] = k;
  int err = OR_OK;
#pragma omp parallel
  {
    double* qh = (double*)malloc((size_t)d * sizeof(double));
    double* kh = (double*)malloc((size_t)d * sizeof(double));
    double* scv = (double*)malloc((size_t)nc * sizeof(double));
    double* logit = (double*)malloc((size_t)(pos + 1) * sizeof(double));
    tok_t* tok = (tok_t*)malloc((size_t)(pos + 1) * sizeof(tok_t));
    if (!qh || !kh || !scv || !logit || !tok) {
#pragma omp atomic write
      err = OR_ENOMEM;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t bh = 0; bh < B * H; ++bh) {
        const int64_t kvb = bh * N * d;
        /* the current chunk's pooled query: its m queries / sqrt(m) */
        for (int64_t x = 0; x < d; ++x) {
          double a = 0.0;
          for (int64_t r = 0; r < m; ++r) a += ld(Qcur, dtype, (bh * m + r) * d + x);
          qh[x] = a / sqrt((double)m);
        }
        /* S_c over the complete chunks and the current one */
        for (int64_t k = 0; k < nc; ++k) {
          const int64_t len = bnd[k + 1] - bnd[k];
          for (int64_t x = 0; x < d; ++x) {
            double a = 0.0;
            for (int64_t j = bnd[k]; j < bnd[k + 1]; ++j) a += ld(K, dtype, kvb + j * d + x);
            kh[x] = a / sqrt((double)len);
          }
          double s = 0.0;
          for (int64_t x = 0; x < d; ++x) s += qh[x] * kh[x];
          scv[k] = s;
        }
        if (Sc) memcpy(Sc + bh * nc, scv, (size_t)nc * sizeof(double));
        /* tiling to the tokens j <= pos and the top-N_b cut */
        for (int64_t j = 0; j <= pos; ++j) {
          tok[j].score = scv[chunk_of[j]];
          tok[j].j = j;
        }
        qsort(tok, (size_t)(pos + 1), sizeof(tok_t), tok_cmp);
        const int64_t keep = (pos + 1) < budget ? (pos + 1) : budget;
        if (n_kept) n_kept[bh] = (int32_t)keep;
        if (kept) {
          uint8_t* krow = kept + bh * (pos + 1);
          memset(krow, 0, (size_t)(pos + 1));
          for (int64_t p = 0; p < keep; ++p) krow[tok[p].j] = 1;
        }
        if (margin) {
          double mg = INFINITY;
          if (keep < pos + 1) {
            const int64_t ccut = chunk_of[tok[keep].j];
            const double scut = tok[keep].score;
            int64_t p = keep;
            while (p > 0 && chunk_of[tok[p - 1].j] == ccut) --p;
            if (p > 0) mg = fmin(mg, tok[p - 1].score - scut);
            p = keep;
            while (p <= pos && chunk_of[tok[p].j] == ccut) ++p;
            if (p <= pos) mg = fmin(mg, scut - tok[p].score);
          }
          margin[bh] = mg;
        }
        /* softmax attention of the new query over the kept keys */
        const int64_t qb = (bh * m + m - 1) * d;
        double mx = -INFINITY;
        for (int64_t p = 0; p < keep; ++p) {
          double a = 0.0;
          for (int64_t x = 0; x < d; ++x)
            a += ld(Qcur, dtype, qb + x) * ld(K, dtype, kvb + tok[p].j * d + x);
          logit[p] = a * sc;
          if (logit[p] > mx) mx = logit[p];
        }
        double z = 0.0;
        for (int64_t p = 0; p < keep; ++p) {
          logit[p] = exp(logit[p] - mx);
          z += logit[p];
        }
        if (out) {
          double* orow = out + bh * d;
          for (int64_t x = 0; x < d; ++x) orow[x] = 0.0;
          for (int64_t p = 0; p < keep; ++p) {
            const double pw = logit[p] / z;
            for (int64_t x = 0; x < d; ++x) orow[x] += pw * ld(V, dtype, kvb + tok[p].j * d + x);
          }
        }
      }
    }
    free(qh);
    free(kh);
    free(scv);
    free(logit);
    free(tok);
  }
  free(chunk_of);
  free(bnd);
  return err;
}

/* ------------------------------------------------------------------------ */
/* Sliding-window attention, the local part of the upper layers ([HSA]       */
/* Methodology: upper layers combine local self-attention with HSA; a 512-   */
/* token window by default).                                                 */
/* ------------------------------------------------------------------------ */

/*
 * Q [B,Hq,L,d], K and V [B,Hkv,L,d] (head h uses KV head h / (Hq/Hkv)).  Row t
 * attends keys j in [max(0, t-W+1), t]: out_t = softmax(q_t . k_j / sqrt d) v.
 *   out [B,Hq,n_rows,d] for the positions rows[0..n_rows) (NULL: all L).
 */
int oracle_swa_prefill(const void* Q, const void* K, const void* V, int dtype, int64_t B,
                       int64_t L, int64_t Hq, int64_t Hkv, int64_t d, int64_t W,
                       const int64_t* rows, int64_t n_rows, double* out) {
  if (!Q || !K || !V || !out || B < 0 || L < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || d <= 0 ||
      W <= 0)
    return OR_EINVAL;
  if (!rows) n_rows = L;
  const int64_t G = Hq / Hkv;
  int err = OR_OK;
#pragma omp parallel
  {
    double* qv = (double*)malloc((size_t)d * sizeof(double));
    double* work = (double*)malloc((size_t)(W + 1) * sizeof(double));
    if (!qv || !work) {
#pragma omp atomic write
      err = OR_ENOMEM;
    } else {
#pragma omp for collapse(3) schedule(dynamic, 16)
      for (int64_t b = 0; b < B; ++b)
        for (int64_t h = 0; h < Hq; ++h)
          for (int64_t r = 0; r < n_rows; ++r) {
            const int64_t t = rows ? rows[r] : r;
            for (int64_t x = 0; x < d; ++x) qv[x] = ld(Q, dtype, ((b * Hq + h) * L + t) * d + x);
            const int64_t j0 = t - W + 1 > 0 ? t - W + 1 : 0;
            attend_rows(qv, K, V, dtype, (b * Hkv + h / G) * L * d, j0, t + 1, d,
                        out + ((b * Hq + h) * n_rows + r) * d, work);
          }
    }
    free(qv);
    free(work);
  }
  return err;
}

/*
 * One new query per sequence at position pos: q [B,Hq,d], caches
 * [B,Hkv,N,d] holding tokens 0..pos (pos < N); keys j in
 * [max(0, pos-W+1), pos].  out [B,Hq,d].
 */
int oracle_swa_decode(const void* q, const void* K, const void* V, int dtype, int64_t B,
                      int64_t Hq, int64_t Hkv, int64_t d, int64_t N, int64_t pos, int64_t W,
                      double* out) {
  if (!q || !K || !V || !out || B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || d <= 0 || W <= 0 ||
      pos < 0 || pos >= N)
    return OR_EINVAL;
  const int64_t G = Hq / Hkv;
  double* qv = (double*)malloc((size_t)d * sizeof(double));
  double* work = (double*)malloc((size_t)(W + 1) * sizeof(double));
  if (!qv || !work) {
    free(qv);
    free(work);
    return OR_ENOMEM;
  }
  for (int64_t b = 0; b < B; ++b)
    for (int64_t h = 0; h < Hq; ++h) {
      for (int64_t x = 0; x < d; ++x) qv[x] = ld(q, dtype, (b * Hq + h) * d + x);
      const int64_t j0 = pos - W + 1 > 0 ? pos - W + 1 : 0;
      attend_rows(qv, K, V, dtype, (b * Hkv + h / G) * N * d, j0, pos + 1, d,
                  out + (b * Hq + h) * d, work);
    }
  free(qv);
  free(work);
  return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* HSA prefill backward ([HiLS] abstract: retrieval learned end to end, the  */
/* gradient reaching the retrieval scores through the fusion weights).       */
/* ------------------------------------------------------------------------ */

/* p_j = softmax_j(q . k_j / sqrt(d)) over keys rows [j0, j1) of a slab. */
static void chunk_probs(const double* q, const void* K, int dtype, int64_t base, int64_t j0,
                        int64_t j1, int64_t d, double* p) {
  const double sc = 1.0 / sqrt((double)d);
  double mx = -INFINITY;
  for (int64_t j = j0; j < j1; ++j) {
    double a = 0.0;
    for (int64_t x = 0; x < d; ++x) a += q[x] * ld(K, dtype, base + j * d + x);
    p[j - j0] = a * sc;
    if (p[j - j0] > mx) mx = p[j - j0];
  }
  double z = 0.0;
  for (int64_t j = j0; j < j1; ++j) {
    p[j - j0] = exp(p[j - j0] - mx);
    z += p[j - j0];
  }
  for (int64_t j = j0; j < j1; ++j) p[j - j0] /= z;
}

/*
 * Gradients of sum over (b, h, t, x) of dO * out, out being HSA prefill with
 * per-token retrieval (oracle_hsa_prefill, interval 1), with respect to Q, K
 * and V.  The top-K selection is piecewise constant in the inputs and is
 * held fixed (its derivative is zero wherever the ranking does not change).
 * Per row t and head h with the selected chunks c_1..c_m:
 *   s_k = q . lambda_ck / sqrt(d),  w = softmax(s),
 *   o_k = sum_j p_kj v_j with p_k = softmax_j(q . k_j / sqrt(d)) over chunk c_k,
 *   out = sum_k w_k o_k.
 * Chain rule, in the forward's order reversed:
 *   fusion     dw_k = dO . o_k,  ds_k = w_k (dw_k - sum_k' w_k' dw_k'),
 *              the chunk outputs receive do_k = w_k dO;
 *   chunk k    dp_j = do_k . v_j,  dz_j = p_kj (dp_j - do_k . o_k),
 *              dq += dz_j k_j / sqrt(d),  dk_j += dz_j q / sqrt(d),
 *              dv_j += p_kj do_k;
 *   retrieval  dq += ds_k lambda_ck / sqrt(d),  dlambda_ck += ds_k q / sqrt(d);
 *   landmarks  lambda_c = sum_{j in c} k_j / sqrt(S): dk_j += dlambda_c / sqrt(S).
 * dO has Q's shape and dtype.  dQ [B,Hq,L,d], dK and dV [B,Hkv,L,d] (double)
 * are overwritten.  rows[0..n_rows) (NULL: every position) lists the query
 * positions whose terms are taken: the result is then the gradient of the
 * same sum with dO set to zero at every other position (dQ is zero there).
 */
int oracle_hsa_prefill_backward(const void* Q, const void* K, const void* V, const void* dO,
                                int dtype, int64_t B, int64_t L, int64_t Hq, int64_t Hkv,
                                int64_t d, int64_t S, int64_t topk, const int64_t* rows,
                                int64_t n_rows, double* dQ, double* dK, double* dV) {
  if (!Q || !K || !V || !dO || !dQ || !dK || !dV || B < 0 || L < 0 || Hq <= 0 || Hkv <= 0 ||
      Hq % Hkv || d <= 0 || S <= 0 || topk <= 0 || (rows && n_rows < 0))
    return OR_EINVAL;
  if (rows)
    for (int64_t r = 0; r < n_rows; ++r)
      if (rows[r] < 0 || rows[r] >= L) return OR_EINVAL;
  const int64_t G = Hq / Hkv;
  const int64_t n = L / S;
  const double sc = 1.0 / sqrt((double)d);
  const double rs = 1.0 / sqrt((double)S);
  memset(dQ, 0, (size_t)(B * Hq * L * d) * sizeof(double));
  memset(dK, 0, (size_t)(B * Hkv * L * d) * sizeof(double));
  memset(dV, 0, (size_t)(B * Hkv * L * d) * sizeof(double));
  double* lmk = (double*)malloc((size_t)(B * Hkv * (n > 0 ? n : 1) * d) * sizeof(double));
  if (!lmk) return OR_ENOMEM;
  oracle_landmarks(K, dtype, B, Hkv, L, d, S, lmk);
  const int64_t m_max = topk < n ? topk : n;
  int err = OR_OK;
  /* each (b, group) owns its slabs of dK, dV and its landmark gradients */
#pragma omp parallel
  {
    cand_t* cand = (cand_t*)malloc((size_t)(n + 1) * sizeof(cand_t));
    double* qv = (double*)malloc((size_t)(G * d) * sizeof(double));
    double* dov = (double*)malloc((size_t)d * sizeof(double));
    double* s = (double*)malloc((size_t)(m_max + 1) * sizeof(double));
    double* w = (double*)malloc((size_t)(m_max + 1) * sizeof(double));
    double* dw = (double*)malloc((size_t)(m_max + 1) * sizeof(double));
    double* o = (double*)malloc((size_t)((m_max + 1) * d) * sizeof(double));
    double* p = (double*)malloc((size_t)((m_max + 1) * S) * sizeof(double));
    double* dlmk = (double*)malloc((size_t)((n > 0 ? n : 1) * d) * sizeof(double));
    if (!cand || !qv || !dov || !s || !w || !dw || !o || !p || !dlmk) {
#pragma omp atomic write
      err = OR_ENOMEM;
    } else {
#pragma omp for collapse(2) schedule(dynamic, 1)
      for (int64_t b = 0; b < B; ++b)
        for (int64_t g = 0; g < Hkv; ++g) {
          const int64_t kv_base = (b * Hkv + g) * L * d;
          const double* lg = lmk + (b * Hkv + g) * n * d;
          for (int64_t x = 0; x < n * d; ++x) dlmk[x] = 0.0;
          const int64_t nr = rows ? n_rows : L;
          for (int64_t ri = 0; ri < nr; ++ri) {
            const int64_t t = rows ? rows[ri] : ri;
            const int64_t navail = t / S < n ? t / S : n;
            for (int64_t hh = 0; hh < G; ++hh)
              for (int64_t x = 0; x < d; ++x)
                qv[hh * d + x] = ld(Q, dtype, ((b * Hq + g * G + hh) * L + t) * d + x);
            /* the forward's selection: group-summed scores (the summed dot
             * products scaled once, as in the forward), top-K */
            for (int64_t c = 0; c < navail; ++c) {
              double sigma = 0.0;
              for (int64_t hh = 0; hh < G; ++hh) {
                double a = 0.0;
                for (int64_t x = 0; x < d; ++x) a += qv[hh * d + x] * lg[c * d + x];
                sigma += a;
              }
              cand[c].score = sigma * sc;
              cand[c].idx = c;
            }
            qsort(cand, (size_t)navail, sizeof(cand_t), cand_cmp);
            const int64_t m = navail < topk ? navail : topk;
            if (m == 0) continue;
            for (int64_t hh = 0; hh < G; ++hh) {
              const int64_t h = g * G + hh;
              const double* q = qv + hh * d;
              double* dq = dQ + ((b * Hq + h) * L + t) * d;
              for (int64_t x = 0; x < d; ++x) dov[x] = ld(dO, dtype, ((b * Hq + h) * L + t) * d + x);
              /* forward quantities of the row */
              double smax = -INFINITY;
              for (int64_t k = 0; k < m; ++k) {
                const int64_t c = cand[k].idx;
                double a = 0.0;
                for (int64_t x = 0; x < d; ++x) a += q[x] * lg[c * d + x];
                s[k] = a * sc;
                if (s[k] > smax) smax = s[k];
              }
              double zs = 0.0;
              for (int64_t k = 0; k < m; ++k) zs += exp(s[k] - smax);
              for (int64_t k = 0; k < m; ++k) {
                const int64_t c = cand[k].idx;
                w[k] = exp(s[k] - smax) / zs;
                chunk_probs(q, K, dtype, kv_base, c * S, (c + 1) * S, d, p + k * S);
                for (int64_t x = 0; x < d; ++x) {
                  double a = 0.0;
                  for (int64_t j = 0; j < S; ++j)
                    a += p[k * S + j] * ld(V, dtype, kv_base + (c * S + j) * d + x);
                  o[k * d + x] = a;
                }
              }
              /* fusion */
              double wdw = 0.0;
              for (int64_t k = 0; k < m; ++k) {
                double a = 0.0;
                for (int64_t x = 0; x < d; ++x) a += dov[x] * o[k * d + x];
                dw[k] = a;
                wdw += w[k] * a;
              }
              for (int64_t k = 0; k < m; ++k) {
                const int64_t c = cand[k].idx;
                const double ds = w[k] * (dw[k] - wdw);
                /* retrieval scores */
                for (int64_t x = 0; x < d; ++x) {
                  dq[x] += ds * sc * lg[c * d + x];
                  dlmk[c * d + x] += ds * sc * q[x];
                }
                /* attention inside chunk c with do = w_k dO; do . o_k = w_k dw_k */
                const double D = w[k] * dw[k];
                for (int64_t j = 0; j < S; ++j) {
                  const int64_t row = kv_base + (c * S + j) * d;
                  double dp = 0.0;
                  for (int64_t x = 0; x < d; ++x) dp += w[k] * dov[x] * ld(V, dtype, row + x);
                  const double pj = p[k * S + j];
                  const double dz = pj * (dp - D);
                  for (int64_t x = 0; x < d; ++x) {
                    dq[x] += dz * sc * ld(K, dtype, row + x);
                    dK[row + x] += dz * sc * q[x];
                    dV[row + x] += pj * w[k] * dov[x];
                  }
                }
              }
            }
          }
          /* landmark pooling */
          for (int64_t c = 0; c < n; ++c)
            for (int64_t j = 0; j < S; ++j)
              for (int64_t x = 0; x < d; ++x)
                dK[kv_base + (c * S + j) * d + x] += dlmk[c * d + x] * rs;
        }
    }
    free(cand);
    free(qv);
    free(dov);
    free(s);
    free(w);
    free(dw);
    free(o);
    free(p);
    free(dlmk);
  }
  free(lmk);
  return err;
}
