/*
 * MoBA causal prefill forward -- CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY. The tests, the smoke check and the CPU-baseline
 * leg of the benchmark are the only callers. The GPU library never links,
 * loads or calls this file, and this file uses nothing from the GPU library.
 *
 * What it computes is the plain definition of MoBA prefill: dense softmax
 * attention under MoBA's block mask. That is the mask-based "moba_naive"
 * formulation (MoBA: Mixture of Block Attention for Long-Context LLMs,
 * README, "Implementation Details"); the efficient implementation described on
 * the same page reaches the same result up to rounding, because merging the
 * softmax of disjoint key sets through their log-sum-exp is exact (Kimi发布MoBA
 * 突破性实现无限上下文, "PyTorch实现关键要点").
 *
 * Arithmetic is fp64 throughout. Inputs arrive as fp32 arrays; every bf16 and
 * every fp32 value converts to fp64 exactly, so no input rounding happens here.
 *
 * Per sequence n of a packed batch (boundaries in cu_seqlens), with local
 * positions t in [0, S_n):
 *   1. Blocks. Block b covers [b*B, min((b+1)*B, S_n)); the remainder forms a
 *      shorter final block. Blocks restart at every sequence start.
 *      (Kimi article, "MoBA：基于块的混合注意力机制": the sequence is cut into
 *      spans of equal length.)
 *   2. Pool. Kbar[b,g] = mean of K[s,g,:] over the tokens s of block b, using the
 *      block's true length. (Same section: each query looks at a pooled, e.g.
 *      mean-pooled, representation of every block's keys.)
 *   3. Gate. For row (t,h): i = t / B, g = h / (Hq/Hkv). The score of block j is
 *      the unscaled dot product q[t,h] . Kbar[j,g]; only j < i are candidates.
 *      The query's own block (j = i) is forced and not gated; future blocks are
 *      masked. (README, "Parameter-less Gating Mechanism"; Kimi article,
 *      "PyTorch实现关键要点": score = query times pooled keys, then the causal
 *      mask, then top-k; README FAQ, issue #27: the current block is always
 *      attended and is excluded from the top-k because pooling a whole block
 *      would leak future tokens.)
 *   4. Select. top-k counts the own block, so min(topk-1, i) past blocks are
 *      kept (README FAQ, issue #27: moba_topk is reduced by one and capped by the
 *      number of candidate chunks). Candidates are ranked by score, highest
 *      first; equal scores rank the lower block index first (the pages are
 *      silent on ties; this is the reading taken). The kept ids are reported in
 *      ascending order, padded with -1 up to topk-1 entries.
 *   5. Attend. The key set is A = {s : i*B <= s <= t} (own block, causal) united
 *      with every token of every selected block. With scale c:
 *        out = sum_{s in A} softmax_s(c * q . k_s) * v_s,
 *        lse = m + log(sum_{s in A} exp(c * q . k_s - m)),  m = max logit.
 *
 * The oracle takes any subset of rows ("sampled mode"): it pools every block,
 * then runs steps 3-5 for just the requested (token, head) rows. A row's result
 * does not depend on which other rows are requested.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_BAD_ARG 1
#define ORACLE_NO_MEMORY 2

static int64_t num_blocks_of(int64_t len, int64_t block) {
  return (len + block - 1) / block;
}

/* Sequence n with cu[n] <= tok < cu[n+1] (empty sequences are skipped). */
static int32_t seq_of_token(const int32_t* cu, int32_t nseq, int64_t tok) {
  int32_t lo = 0, hi = nseq - 1;
  while (lo < hi) {
    int32_t mid = (lo + hi + 1) / 2;
    if ((int64_t)cu[mid] <= tok) lo = mid; else hi = mid - 1;
  }
  return lo;
}

static int check_layout(const int32_t* cu, int32_t nseq, int32_t hq, int32_t hkv,
                        int32_t d, int32_t block) {
  if (!cu || nseq < 1 || hq < 1 || hkv < 1 || d < 1 || block < 1) return 0;
  if (hq % hkv != 0) return 0;
  if (cu[0] != 0) return 0;
  for (int32_t n = 0; n < nseq; ++n)
    if (cu[n + 1] < cu[n]) return 0;
  return 1;
}

/* Total number of blocks over all sequences, and the first global block id of
 * each sequence (block_base must hold nseq entries). */
static int64_t count_blocks(const int32_t* cu, int32_t nseq, int32_t block,
                            int64_t* block_base) {
  int64_t total = 0;
  for (int32_t n = 0; n < nseq; ++n) {
    if (block_base) block_base[n] = total;
    total += num_blocks_of((int64_t)cu[n + 1] - cu[n], block);
  }
  return total;
}

int64_t moba_oracle_num_blocks(const int32_t* cu_seqlens, int32_t nseq, int32_t block) {
  if (!cu_seqlens || nseq < 1 || block < 1) return -1;
  return count_blocks(cu_seqlens, nseq, block, NULL);
}

/* Step 2: mean-pool every block of K.
 * k:    [T, hkv, d] fp32, T = cu_seqlens[nseq].
 * kbar: [NB, hkv, d] fp64 out, blocks numbered sequence by sequence. */
int moba_oracle_pool(const float* k, const int32_t* cu_seqlens, int32_t nseq,
                     int32_t hkv, int32_t d, int32_t block, double* kbar) {
  if (!k || !kbar || !check_layout(cu_seqlens, nseq, hkv, hkv, d, block))
    return ORACLE_BAD_ARG;
  int64_t gb = 0;
  for (int32_t n = 0; n < nseq; ++n) {
    int64_t start = cu_seqlens[n], len = (int64_t)cu_seqlens[n + 1] - start;
    int64_t nb = num_blocks_of(len, block);
    for (int64_t b = 0; b < nb; ++b, ++gb) {
      int64_t s0 = start + b * block;
      int64_t s1 = start + ((b + 1) * block < len ? (b + 1) * block : len);
      for (int32_t g = 0; g < hkv; ++g) {
        double* dst = kbar + (gb * hkv + g) * d;
        for (int32_t e = 0; e < d; ++e) dst[e] = 0.0;
        for (int64_t s = s0; s < s1; ++s) {
          const float* src = k + (s * hkv + g) * d;
          for (int32_t e = 0; e < d; ++e) dst[e] += (double)src[e];
        }
        for (int32_t e = 0; e < d; ++e) dst[e] /= (double)(s1 - s0);
      }
    }
  }
  return ORACLE_OK;
}

static double dot(const float* a, const double* b, int32_t d) {
  double acc = 0.0;
  for (int32_t e = 0; e < d; ++e) acc += (double)a[e] * b[e];
  return acc;
}

static double dot_ff(const float* a, const float* b, int32_t d) {
  double acc = 0.0;
  for (int32_t e = 0; e < d; ++e) acc += (double)a[e] * (double)b[e];
  return acc;
}

/* Steps 3-4 for one row: gate scores sigma[j] of the past blocks j < i (the
 * unscaled dot product with the pooled keys of the row's kv head; kbar_g points
 * at block 0 of the row's sequence for that head, consecutive blocks hkv*d
 * apart), then nsel times the best remaining candidate; a strict '>' keeps the
 * lower index when scores tie. chosen[0..nsel) in the order taken, taken[j]
 * marks the kept blocks. */
static void gate_and_select(const float* q, const double* kbar_g, int64_t i, int32_t hkv,
                            int32_t d, int64_t nsel, double* sigma, char* taken,
                            int32_t* chosen) {
  for (int64_t j = 0; j < i; ++j) {
    sigma[j] = dot(q, kbar_g + j * hkv * d, d);
    taken[j] = 0;
  }
  for (int64_t m = 0; m < nsel; ++m) {
    int64_t best = -1;
    for (int64_t j = 0; j < i; ++j)
      if (!taken[j] && (best < 0 || sigma[j] > sigma[best])) best = j;
    taken[best] = 1;
    chosen[m] = (int32_t)best;
  }
}

/* Step 5 for one row: the attended key set A is the own block's prefix
 * {s : i*B <= s <= t} (causal) followed by every token of each chosen past
 * block (chosen[0..nsel), sequence-local ids, all complete blocks). Logits
 * c * q . k_s are stored first, then a softmax with the maximum taken out, then
 * the weighted sum of V; lse = max + log(sum of weights). `logit` has room for
 * block * (nsel + 1) values. Token indices are packed: the row's sequence starts
 * at token `start` and the row is token `tok`. */
static void attend_row(const float* q, const float* k, const float* v, int32_t hkv, int32_t d,
                       int32_t g, int64_t start, int64_t i, int64_t tok, int32_t block,
                       const int32_t* chosen, int64_t nsel, double scale, double* logit,
                       double* o, double* lse_row) {
  int64_t na = 0;
  for (int64_t s = start + i * block; s <= tok; ++s)
    logit[na++] = scale * dot_ff(q, k + (s * hkv + g) * d, d);
  for (int64_t m = 0; m < nsel; ++m) {
    int64_t s0 = start + (int64_t)chosen[m] * block;
    for (int64_t s = s0; s < s0 + block; ++s)   /* past blocks are full */
      logit[na++] = scale * dot_ff(q, k + (s * hkv + g) * d, d);
  }
  double mx = -INFINITY;
  for (int64_t a = 0; a < na; ++a) if (logit[a] > mx) mx = logit[a];
  double denom = 0.0;
  for (int32_t e = 0; e < d; ++e) o[e] = 0.0;
  int64_t a = 0;
  for (int64_t s = start + i * block; s <= tok; ++s, ++a) {
    double w = exp(logit[a] - mx);
    denom += w;
    const float* vs = v + (s * hkv + g) * d;
    for (int32_t e = 0; e < d; ++e) o[e] += w * (double)vs[e];
  }
  for (int64_t m = 0; m < nsel; ++m) {
    int64_t s0 = start + (int64_t)chosen[m] * block;
    for (int64_t s = s0; s < s0 + block; ++s, ++a) {
      double w = exp(logit[a] - mx);
      denom += w;
      const float* vs = v + (s * hkv + g) * d;
      for (int32_t e = 0; e < d; ++e) o[e] += w * (double)vs[e];
    }
  }
  for (int32_t e = 0; e < d; ++e) o[e] /= denom;
  *lse_row = mx + log(denom);
}

/* Steps 3-5 for a list of rows.
 *
 * q_rows:   [nrows, d] fp32, the query vector of each requested row.
 * row_tok:  [nrows] packed token index of the row (0 <= tok < T).
 * row_head: [nrows] query head of the row (0 <= h < hq).
 * k, v:     [T, hkv, d] fp32.
 * scale:    softmax scale; <= 0 selects 1/sqrt(d).
 * out:      [nrows, d] fp64.         lse: [nrows] fp64.
 * sel:      [nrows, topk-1] int32 (may be NULL when topk == 1).
 * margin:   [nrows] fp64 or NULL: score of the last kept block minus the best
 *           score left out; +inf when every candidate is kept.
 * nthreads: OpenMP threads; <= 0 uses the runtime default.
 */
int moba_oracle_rows(const float* q_rows, const int32_t* row_tok, const int32_t* row_head,
                     int64_t nrows, const float* k, const float* v,
                     const int32_t* cu_seqlens, int32_t nseq, int32_t hq, int32_t hkv,
                     int32_t d, int32_t block, int32_t topk, double scale,
                     double* out, double* lse, int32_t* sel, double* margin,
                     int32_t nthreads) {
  if (!q_rows || !row_tok || !row_head || !k || !v || !out || !lse || nrows < 0 ||
      topk < 1 || !check_layout(cu_seqlens, nseq, hq, hkv, d, block))
    return ORACLE_BAD_ARG;
  if (topk > 1 && !sel) return ORACLE_BAD_ARG;
  const int64_t T = cu_seqlens[nseq];
  for (int64_t r = 0; r < nrows; ++r)
    if (row_tok[r] < 0 || row_tok[r] >= T || row_head[r] < 0 || row_head[r] >= hq)
      return ORACLE_BAD_ARG;
  if (scale <= 0.0) scale = 1.0 / sqrt((double)d);

  int64_t* block_base = (int64_t*)malloc(sizeof(int64_t) * (size_t)nseq);
  if (!block_base) return ORACLE_NO_MEMORY;
  const int64_t nb_total = count_blocks(cu_seqlens, nseq, block, block_base);
  double* kbar = (double*)malloc(sizeof(double) * (size_t)(nb_total * hkv * d));
  if (!kbar) { free(block_base); return ORACLE_NO_MEMORY; }
  moba_oracle_pool(k, cu_seqlens, nseq, hkv, d, block, kbar);

  int64_t max_blocks = 0;
  for (int32_t n = 0; n < nseq; ++n) {
    int64_t nb = num_blocks_of((int64_t)cu_seqlens[n + 1] - cu_seqlens[n], block);
    if (nb > max_blocks) max_blocks = nb;
  }
  const int32_t group = hq / hkv;
  int failed = 0;

#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads)
#endif
  {
    double* sigma = (double*)malloc(sizeof(double) * (size_t)(max_blocks + 1));
    char* taken = (char*)malloc((size_t)(max_blocks + 1));
    int32_t* chosen = (int32_t*)malloc(sizeof(int32_t) * (size_t)topk);
    double* logit = (double*)malloc(sizeof(double) * (size_t)block * (size_t)topk);
    if (!sigma || !taken || !chosen || !logit) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
      failed = 1;
    } else {
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 4)
#endif
      for (int64_t r = 0; r < nrows; ++r) {
        const float* q = q_rows + r * d;
        const int64_t tok = row_tok[r];
        const int32_t h = row_head[r];
        const int32_t n = seq_of_token(cu_seqlens, nseq, tok);
        const int64_t start = cu_seqlens[n];
        const int64_t t = tok - start;
        const int64_t i = t / block;
        const int32_t g = h / group;
        const int64_t nsel = (topk - 1 < i) ? topk - 1 : i;

        /* Steps 3-4: gate scores of the past blocks j < i, then selection. */
        gate_and_select(q, kbar + (block_base[n] * hkv + g) * d, i, hkv, d, nsel, sigma, taken,
                        chosen);
        if (margin) {
          double worst_kept = INFINITY, best_left = -INFINITY;
          for (int64_t j = 0; j < i; ++j) {
            if (taken[j] && sigma[j] < worst_kept) worst_kept = sigma[j];
            if (!taken[j] && sigma[j] > best_left) best_left = sigma[j];
          }
          margin[r] = (nsel < i) ? worst_kept - best_left : INFINITY;
        }
        if (topk > 1) {
          int32_t* srow = sel + r * (topk - 1);
          int64_t w = 0;
          for (int64_t j = 0; j < i; ++j)
            if (taken[j]) srow[w++] = (int32_t)j;
          for (; w < topk - 1; ++w) srow[w] = -1;
        }

        /* Step 5 over the own-block prefix and the blocks just chosen. */
        attend_row(q, k, v, hkv, d, g, start, i, tok, block, chosen, nsel, scale, logit,
                   out + r * d, lse + r);
      }
    }
    free(sigma);
    free(taken);
    free(chosen);
    free(logit);
  }
  free(kbar);
  free(block_base);
  return failed ? ORACLE_NO_MEMORY : ORACLE_OK;
}

/* Step 5 alone for a list of rows, with the kept past blocks given instead of
 * gated: sel_in [nrows, topk-1] int32 lists sequence-local block ids (entries
 * < 0 are skipped; every other entry must be a distinct past block of the row,
 * 0 <= j < i, else the call fails with ORACLE_BAD_ARG). This evaluates the
 * attention a row would get from that selection: it serves to check a GPU's
 * output on rows whose selection is one of several valid top-(topk-1) sets
 * (scores tied within rounding). Other arguments as moba_oracle_rows. */
int moba_oracle_rows_given_sel(const float* q_rows, const int32_t* row_tok,
                               const int32_t* row_head, int64_t nrows, const float* k,
                               const float* v, const int32_t* cu_seqlens, int32_t nseq,
                               int32_t hq, int32_t hkv, int32_t d, int32_t block, int32_t topk,
                               const int32_t* sel_in, double scale, double* out, double* lse,
                               int32_t nthreads) {
  if (!q_rows || !row_tok || !row_head || !k || !v || !out || !lse || nrows < 0 ||
      topk < 1 || !check_layout(cu_seqlens, nseq, hq, hkv, d, block))
    return ORACLE_BAD_ARG;
  if (topk > 1 && !sel_in) return ORACLE_BAD_ARG;
  const int64_t T = cu_seqlens[nseq];
  const int32_t ks = topk - 1;
  for (int64_t r = 0; r < nrows; ++r) {
    if (row_tok[r] < 0 || row_tok[r] >= T || row_head[r] < 0 || row_head[r] >= hq)
      return ORACLE_BAD_ARG;
    const int32_t n = seq_of_token(cu_seqlens, nseq, row_tok[r]);
    const int64_t i = (row_tok[r] - (int64_t)cu_seqlens[n]) / block;
    for (int32_t a = 0; a < ks; ++a) {
      const int32_t j = sel_in[r * ks + a];
      if (j < 0) continue;
      if (j >= i) return ORACLE_BAD_ARG;
      for (int32_t b = 0; b < a; ++b)
        if (sel_in[r * ks + b] == j) return ORACLE_BAD_ARG;
    }
  }
  if (scale <= 0.0) scale = 1.0 / sqrt((double)d);
  const int32_t group = hq / hkv;
  int failed = 0;
#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads)
#endif
  {
    double* logit = (double*)malloc(sizeof(double) * (size_t)block * (size_t)topk);
    int32_t* chosen = (int32_t*)malloc(sizeof(int32_t) * (size_t)topk);
    if (!logit || !chosen) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
      failed = 1;
    } else {
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 4)
#endif
      for (int64_t r = 0; r < nrows; ++r) {
        const int64_t tok = row_tok[r];
        const int32_t n = seq_of_token(cu_seqlens, nseq, tok);
        const int64_t start = cu_seqlens[n];
        const int64_t i = (tok - start) / block;
        int64_t nsel = 0;
        for (int32_t a = 0; a < ks; ++a)
          if (sel_in[r * ks + a] >= 0) chosen[nsel++] = sel_in[r * ks + a];
        attend_row(q_rows + r * d, k, v, hkv, d, row_head[r] / group, start, i, tok, block,
                   chosen, nsel, scale, logit, out + r * d, lse + r);
      }
    }
    free(logit);
    free(chosen);
  }
  return failed ? ORACLE_NO_MEMORY : ORACLE_OK;
}

/* Plain causal softmax attention for a list of rows: key set {s : 0 <= s <= t}
 * of the row's own sequence. This is the comparison point that MoBA replaces
 * (full attention; README, "Seamlessly Transition between Full and Sparse
 * Attention"). Same argument conventions as moba_oracle_rows. */
int moba_oracle_causal_rows(const float* q_rows, const int32_t* row_tok,
                            const int32_t* row_head, int64_t nrows, const float* k,
                            const float* v, const int32_t* cu_seqlens, int32_t nseq,
                            int32_t hq, int32_t hkv, int32_t d, double scale,
                            double* out, double* lse, int32_t nthreads) {
  if (!q_rows || !row_tok || !row_head || !k || !v || !out || !lse || nrows < 0 ||
      !check_layout(cu_seqlens, nseq, hq, hkv, d, 1))
    return ORACLE_BAD_ARG;
  const int64_t T = cu_seqlens[nseq];
  for (int64_t r = 0; r < nrows; ++r)
    if (row_tok[r] < 0 || row_tok[r] >= T || row_head[r] < 0 || row_head[r] >= hq)
      return ORACLE_BAD_ARG;
  if (scale <= 0.0) scale = 1.0 / sqrt((double)d);
  const int32_t group = hq / hkv;
  int64_t max_len = 0;
  for (int32_t n = 0; n < nseq; ++n)
    if ((int64_t)cu_seqlens[n + 1] - cu_seqlens[n] > max_len)
      max_len = (int64_t)cu_seqlens[n + 1] - cu_seqlens[n];
  int failed = 0;
#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads)
#endif
  {
    double* logit = (double*)malloc(sizeof(double) * (size_t)(max_len + 1));
    if (!logit) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
      failed = 1;
    } else {
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
      for (int64_t r = 0; r < nrows; ++r) {
        const float* q = q_rows + r * d;
        const int64_t tok = row_tok[r];
        const int32_t g = row_head[r] / group;
        const int64_t start = cu_seqlens[seq_of_token(cu_seqlens, nseq, tok)];
        double mx = -INFINITY;
        for (int64_t s = start; s <= tok; ++s) {
          logit[s - start] = scale * dot_ff(q, k + (s * hkv + g) * d, d);
          if (logit[s - start] > mx) mx = logit[s - start];
        }
        double denom = 0.0;
        double* o = out + r * d;
        for (int32_t e = 0; e < d; ++e) o[e] = 0.0;
        for (int64_t s = start; s <= tok; ++s) {
          double w = exp(logit[s - start] - mx);
          denom += w;
          const float* vs = v + (s * hkv + g) * d;
          for (int32_t e = 0; e < d; ++e) o[e] += w * (double)vs[e];
        }
        for (int32_t e = 0; e < d; ++e) o[e] /= denom;
        lse[r] = mx + log(denom);
      }
    }
    free(logit);
  }
  return failed ? ORACLE_NO_MEMORY : ORACLE_OK;
}

/* Backward of step 5 for one row, with the selection of steps 1-4 held fixed
 * (top-k is piecewise constant in its inputs, so no gradient reaches the gate;
 * README, "Trainable Block Sparse Attention": MoBA is trained through its
 * attention). For a row r with attended set A_r, logits l_s = c * q_r . k_s,
 * probabilities p_s = softmax over A_r, output o_r = sum p_s v_s, and the loss
 * gradient dO_r, the chain rule gives
 *   dP_s = dO_r . v_s,   Delta_r = sum_{s in A_r} p_s dP_s  (= dO_r . o_r),
 *   dS_s = p_s (dP_s - Delta_r),
 *   dq_r = c sum_s dS_s k_s,   dk_s += c dS_s q_r,   dv_s += p_s dO_r.
 * qr, dor: the row's query and output gradient; kbar_g as in gate_and_select;
 * t: the row's position in its sequence (start = first token). dqr is written;
 * dk, dv ([T, hkv, d]) are accumulated into unless NULL. key, p, dp hold
 * block * topk entries; sigma, taken, chosen as in gate_and_select. */
static void row_backward(const float* qr, const float* dor, const float* k, const float* v,
                         const double* kbar_g, int64_t start, int64_t t, int32_t g,
                         int32_t hkv, int32_t d, int32_t block, int32_t topk, double scale,
                         double* dqr, double* dk, double* dv, double* sigma, char* taken,
                         int32_t* chosen, int64_t* key, double* p, double* dp) {
  const int64_t tok = start + t, i = t / block;
  const int64_t nsel = (topk - 1 < i) ? topk - 1 : i;
  gate_and_select(qr, kbar_g, i, hkv, d, nsel, sigma, taken, chosen);
  /* the attended keys: own block up to t, then the kept blocks */
  int64_t na = 0;
  for (int64_t s = start + i * block; s <= tok; ++s) key[na++] = s;
  for (int64_t m = 0; m < nsel; ++m)
    for (int64_t s = start + (int64_t)chosen[m] * block;
         s < start + ((int64_t)chosen[m] + 1) * block; ++s)
      key[na++] = s;
  double mx = -INFINITY;
  for (int64_t a = 0; a < na; ++a) {
    p[a] = scale * dot_ff(qr, k + (key[a] * hkv + g) * d, d);
    if (p[a] > mx) mx = p[a];
  }
  double denom = 0.0;
  for (int64_t a = 0; a < na; ++a) {
    p[a] = exp(p[a] - mx);
    denom += p[a];
  }
  double delta = 0.0;
  for (int64_t a = 0; a < na; ++a) {
    p[a] /= denom;
    dp[a] = dot_ff(dor, v + (key[a] * hkv + g) * d, d);
    delta += p[a] * dp[a];
  }
  for (int32_t e = 0; e < d; ++e) dqr[e] = 0.0;
  for (int64_t a = 0; a < na; ++a) {
    const double ds = p[a] * (dp[a] - delta);
    const float* ks = k + (key[a] * hkv + g) * d;
    for (int32_t e = 0; e < d; ++e) dqr[e] += scale * ds * (double)ks[e];
    if (dk) {
      double* dks = dk + (key[a] * hkv + g) * d;
      double* dvs = dv + (key[a] * hkv + g) * d;
      for (int32_t e = 0; e < d; ++e) {
        dks[e] += scale * ds * (double)qr[e];
        dvs[e] += p[a] * (double)dor[e];
      }
    }
  }
}

/* Backward (row_backward) for every row of a batch: dk and dv summed over
 * every row (all q heads of the kv group) that attends each key. Work is split
 * over (sequence, kv head) pairs, each owning its keys' gradients, so the sums
 * need no locking.
 *
 * q, dout: [T, hq, d] fp32;  k, v: [T, hkv, d] fp32.
 * dq: [T, hq, d] fp64;  dk, dv: [T, hkv, d] fp64 (fully written).
 */
int moba_oracle_backward(const float* q, const float* k, const float* v, const float* dout,
                         const int32_t* cu_seqlens, int32_t nseq, int32_t hq, int32_t hkv,
                         int32_t d, int32_t block, int32_t topk, double scale, double* dq,
                         double* dk, double* dv, int32_t nthreads) {
  if (!q || !k || !v || !dout || !dq || !dk || !dv || topk < 1 ||
      !check_layout(cu_seqlens, nseq, hq, hkv, d, block))
    return ORACLE_BAD_ARG;
  if (scale <= 0.0) scale = 1.0 / sqrt((double)d);
  const int64_t T = cu_seqlens[nseq];
  int64_t* block_base = (int64_t*)malloc(sizeof(int64_t) * (size_t)(nseq > 0 ? nseq : 1));
  if (!block_base) return ORACLE_NO_MEMORY;
  const int64_t nb_total = count_blocks(cu_seqlens, nseq, block, block_base);
  double* kbar = (double*)malloc(sizeof(double) * (size_t)(nb_total * hkv * d + 1));
  if (!kbar) { free(block_base); return ORACLE_NO_MEMORY; }
  moba_oracle_pool(k, cu_seqlens, nseq, hkv, d, block, kbar);
  memset(dk, 0, sizeof(double) * (size_t)(T * hkv * d));
  memset(dv, 0, sizeof(double) * (size_t)(T * hkv * d));
  int64_t max_blocks = 0;
  for (int32_t n = 0; n < nseq; ++n) {
    int64_t nb = num_blocks_of((int64_t)cu_seqlens[n + 1] - cu_seqlens[n], block);
    if (nb > max_blocks) max_blocks = nb;
  }
  const int32_t group = hq / hkv;
  int failed = 0;

#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads)
#endif
  {
    double* sigma = (double*)malloc(sizeof(double) * (size_t)(max_blocks + 1));
    char* taken = (char*)malloc((size_t)(max_blocks + 1));
    int32_t* chosen = (int32_t*)malloc(sizeof(int32_t) * (size_t)topk);
    int64_t* key = (int64_t*)malloc(sizeof(int64_t) * (size_t)block * (size_t)topk);
    double* p = (double*)malloc(sizeof(double) * (size_t)block * (size_t)topk);
    double* dp = (double*)malloc(sizeof(double) * (size_t)block * (size_t)topk);
    if (!sigma || !taken || !chosen || !key || !p || !dp) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
      failed = 1;
    } else {
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
      for (int64_t unit = 0; unit < (int64_t)nseq * hkv; ++unit) {
        const int32_t n = (int32_t)(unit / hkv), g = (int32_t)(unit % hkv);
        const int64_t start = cu_seqlens[n], len = (int64_t)cu_seqlens[n + 1] - start;
        for (int64_t t = 0; t < len; ++t)
          for (int32_t h = g * group; h < (g + 1) * group; ++h) {
            const int64_t r = (start + t) * hq + h;
            row_backward(q + r * d, dout + r * d, k, v, kbar + (block_base[n] * hkv + g) * d,
                         start, t, g, hkv, d, block, topk, scale, dq + r * d, dk, dv, sigma,
                         taken, chosen, key, p, dp);
          }
      }
    }
    free(sigma);
    free(taken);
    free(chosen);
    free(key);
    free(p);
    free(dp);
  }
  free(kbar);
  free(block_base);
  return failed ? ORACLE_NO_MEMORY : ORACLE_OK;
}

/* dq (row_backward) of a list of rows only, each from its own inputs: for
 * checks of sampled rows of batches too large for moba_oracle_backward.
 * q_rows, dout_rows: [nrows, d] fp32, the rows' query and output gradient;
 * row_tok, row_head as in moba_oracle_rows; dq: [nrows, d] fp64. */
int moba_oracle_dq_rows(const float* q_rows, const float* dout_rows, const int32_t* row_tok,
                        const int32_t* row_head, int64_t nrows, const float* k, const float* v,
                        const int32_t* cu_seqlens, int32_t nseq, int32_t hq, int32_t hkv,
                        int32_t d, int32_t block, int32_t topk, double scale, double* dq,
                        int32_t nthreads) {
  if (!q_rows || !dout_rows || !row_tok || !row_head || !k || !v || !dq || nrows < 0 ||
      topk < 1 || !check_layout(cu_seqlens, nseq, hq, hkv, d, block))
    return ORACLE_BAD_ARG;
  const int64_t T = cu_seqlens[nseq];
  for (int64_t r = 0; r < nrows; ++r)
    if (row_tok[r] < 0 || row_tok[r] >= T || row_head[r] < 0 || row_head[r] >= hq)
      return ORACLE_BAD_ARG;
  if (scale <= 0.0) scale = 1.0 / sqrt((double)d);
  int64_t* block_base = (int64_t*)malloc(sizeof(int64_t) * (size_t)(nseq > 0 ? nseq : 1));
  if (!block_base) return ORACLE_NO_MEMORY;
  const int64_t nb_total = count_blocks(cu_seqlens, nseq, block, block_base);
  double* kbar = (double*)malloc(sizeof(double) * (size_t)(nb_total * hkv * d + 1));
  if (!kbar) { free(block_base); return ORACLE_NO_MEMORY; }
  moba_oracle_pool(k, cu_seqlens, nseq, hkv, d, block, kbar);
  int64_t max_blocks = 0;
  for (int32_t n = 0; n < nseq; ++n) {
    int64_t nb = num_blocks_of((int64_t)cu_seqlens[n + 1] - cu_seqlens[n], block);
    if (nb > max_blocks) max_blocks = nb;
  }
  const int32_t group = hq / hkv;
  int failed = 0;

#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads)
#endif
  {
    double* sigma = (double*)malloc(sizeof(double) * (size_t)(max_blocks + 1));
    char* taken = (char*)malloc((size_t)(max_blocks + 1));
    int32_t* chosen = (int32_t*)malloc(sizeof(int32_t) * (size_t)topk);
    int64_t* key = (int64_t*)malloc(sizeof(int64_t) * (size_t)block * (size_t)topk);
    double* p = (double*)malloc(sizeof(double) * (size_t)block * (size_t)topk);
    double* dp = (double*)malloc(sizeof(double) * (size_t)block * (size_t)topk);
    if (!sigma || !taken || !chosen || !key || !p || !dp) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
      failed = 1;
    } else {
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 4)
#endif
      for (int64_t r = 0; r < nrows; ++r) {
        const int64_t tok = row_tok[r];
        const int32_t n = seq_of_token(cu_seqlens, nseq, tok);
        const int32_t g = row_head[r] / group;
        row_backward(q_rows + r * d, dout_rows + r * d, k, v,
                     kbar + (block_base[n] * hkv + g) * d, cu_seqlens[n], tok - cu_seqlens[n],
                     g, hkv, d, block, topk, scale, dq + r * d, NULL, NULL, sigma, taken,
                     chosen, key, p, dp);
      }
    }
    free(sigma);
    free(taken);
    free(chosen);
    free(key);
    free(p);
    free(dp);
  }
  free(kbar);
  free(block_base);
  return failed ? ORACLE_NO_MEMORY : ORACLE_OK;
}
