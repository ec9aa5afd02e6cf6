/*
 * ksa_oracle.c -- plain, slow, fp64 CPU oracle for one decode step of
 * block top-k sparse attention and of the vote-union (LessIsMore-style)
 * token selection.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg do.  It shares no source, header or helper with the HIP path.
 *
 * Pages followed (cited by page title and section):
 *   [KIN-5]  Kinetics explainer on news.43u.com.cn, section 五 (from theory to
 *            practice: block top-k attention): history tokens are cut into
 *            blocks, every block gets its average representation, the K'
 *            most relevant blocks are chosen and attention runs over them.
 *   [KIN-4]  same page, section 四: dense attention looks at every history
 *            token.
 *   [LIM-2]  LessIsMore explainer on techwalker.com ("少即是多" revolution),
 *            section 二: every head gets the same number of votes, picks the
 *            tokens it rates as important, votes are tallied per token and
 *            tokens are ranked by their vote total; the budget is split 75 %
 *            voted history / 25 % most recent tokens.
 *   [LIM-5]  same page, section 五: a token-selection layer computes the full
 *            score matrix, lets each head pick, aggregates and sorts the picks
 *            and finally adds the most recent tokens; sparse layers attend the
 *            chosen set only, the set being shared by all heads of a GQA group.
 *
 * Readings taken where the pages are silent:
 *   summary = arithmetic mean of the block's keys, summed in fp64 in token
 *   order, divided by the block's token count in fp64 and stored rounded
 *   to nearest-even in the KV dtype; the group score of a block is the mean
 *   over the group's query heads of q_h . summary, times sm_scale; ranking
 *   uses the unscaled sum over heads; every ranking breaks ties by lowest
 *   index; every index list is returned in ascending order; attention is an
 *   exact two-pass softmax over the chosen tokens only; votes are taken
 *   over history tokens [0, T-W) only, each head picking N-W tokens.
 *
 * All arithmetic is fp64.  Inputs are the exact bytes the GPU saw: fp32, or
 * bf16 given as raw 16-bit patterns (widened here by a 16-bit shift).
 * OpenMP only spreads independent rows over cores; it does not change the
 * order of any sum.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F32 = 0, ORC_BF16 = 1 };

/* Shape of one decode step.  Layouts (row-major, last index fastest):
 *   q        [B, Hq, D]
 *   k, v     [B, Hkv, Tcap, D]
 *   summary  [B, Hkv, NBcap, D], NBcap = ceil(Tcap / Bs)
 * Query head h reads KV head h / (Hq / Hkv). */
typedef struct {
  int64_t B, Hq, Hkv, D, T, Tcap, Bs;
  int32_t dtype;
  double sm_scale; /* <= 0 means 1/sqrt(D) */
} orc_shape;

static double orc_scale(const orc_shape* s) {
  return s->sm_scale > 0.0 ? s->sm_scale : 1.0 / sqrt((double)s->D);
}

static int64_t orc_nblocks(int64_t n, int64_t bs) { return (n + bs - 1) / bs; }

/* Element i of a KV-dtype buffer as a double (exact). */
static double orc_get(const void* base, int32_t dtype, int64_t i) {
  if (dtype == ORC_BF16) {
    uint32_t w = (uint32_t)((const uint16_t*)base)[i] << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
  }
  return (double)((const float*)base)[i];
}

/* Round x to the nearest bf16 value, ties to even, and return its bit
 * pattern.  bf16 keeps 8 significant bits and fp32's exponent range; below
 * 2^-126 its grid is uniform with spacing 2^-133.  Scaling by a power of two
 * is exact, and rint() rounds to nearest-even in the default rounding mode. */
static uint16_t orc_bf16_bits(double x) {
  if (x == 0.0) return signbit(x) ? 0x8000u : 0x0000u;
  int e;
  (void)frexp(x, &e); /* |x| = m * 2^e with 0.5 <= m < 1 */
  int q = e - 8;      /* weight of the last kept bit */
  if (q < -133) q = -133;
  double r = ldexp(rint(ldexp(x, -q)), q);
  float f = (float)r; /* exact: r has at most 8 significant bits */
  uint32_t w;
  memcpy(&w, &f, sizeof w);
  return (uint16_t)(w >> 16);
}

/* ---------------------------------------------------------------------- */
/* Block summaries [KIN-5]: mean key of each block.                        */
/* Blocks [first_block, first_block + num_blocks) of every (b, g) are      */
/* written to `summ` (KV dtype); `mean64` (nullable, [B,Hkv,NBcap,D])       */
/* receives the unrounded fp64 means.  Block j holds tokens                */
/* [j*Bs, min((j+1)*Bs, T)).                                                */
void orc_block_summaries(const orc_shape* s, const void* k, int64_t first_block,
                         int64_t num_blocks, void* summ, double* mean64) {
  const int64_t NBcap = orc_nblocks(s->Tcap, s->Bs);
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t b = 0; b < s->B; ++b)
    for (int64_t g = 0; g < s->Hkv; ++g)
      for (int64_t j = first_block; j < first_block + num_blocks; ++j) {
        int64_t t0 = j * s->Bs;
        int64_t t1 = t0 + s->Bs < s->T ? t0 + s->Bs : s->T;
        int64_t n = t1 - t0;
        if (n <= 0) continue;
        for (int64_t d = 0; d < s->D; ++d) {
          double sum = 0.0;
          for (int64_t t = t0; t < t1; ++t)
            sum += orc_get(k, s->dtype, ((b * s->Hkv + g) * s->Tcap + t) * s->D + d);
          double mean = sum / (double)n;
          int64_t o = ((b * s->Hkv + g) * NBcap + j) * s->D + d;
          if (mean64) mean64[o] = mean;
          if (s->dtype == ORC_BF16)
            ((uint16_t*)summ)[o] = orc_bf16_bits(mean);
          else
            ((float*)summ)[o] = (float)mean; /* C conversion: nearest-even */
        }
      }
}

/* ---------------------------------------------------------------------- */
/* Group relevance of every block [KIN-5] ("most relevant" blocks), from   */
/* the STORED summaries.  raw[b,g,j] = sum over the group's heads h of      */
/* q_h . summary_j (this is what ranks); scaled = sm_scale * raw / G.       */
/* Only blocks j < NB(T) are scored.  raw and scaled are [B, Hkv, NB].      */
void orc_group_scores(const orc_shape* s, const void* q, const void* summ,
                      double* raw, double* scaled) {
  const int64_t NB = orc_nblocks(s->T, s->Bs);
  const int64_t NBcap = orc_nblocks(s->Tcap, s->Bs);
  const int64_t G = s->Hq / s->Hkv;
  const double sc = orc_scale(s);
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t b = 0; b < s->B; ++b)
    for (int64_t g = 0; g < s->Hkv; ++g)
      for (int64_t j = 0; j < NB; ++j) {
        double acc = 0.0;
        for (int64_t hh = 0; hh < G; ++hh) {
          int64_t h = g * G + hh;
          for (int64_t d = 0; d < s->D; ++d)
            acc += orc_get(q, s->dtype, (b * s->Hq + h) * s->D + d) *
                   orc_get(summ, s->dtype, ((b * s->Hkv + g) * NBcap + j) * s->D + d);
        }
        int64_t o = (b * s->Hkv + g) * NB + j;
        if (raw) raw[o] = acc;
        if (scaled) scaled[o] = sc * acc / (double)G;
      }
}

/* The MAX group aggregation of the selection variants: raw[b,g,j] = the   */
/* largest over the group's heads h of q_h . summary_j (the block counts as  */
/* relevant as its most interested head finds it); scaled = sm_scale * raw. */
void orc_group_scores_max(const orc_shape* s, const void* q, const void* summ,
                          double* raw, double* scaled) {
  const int64_t NB = orc_nblocks(s->T, s->Bs);
  const int64_t NBcap = orc_nblocks(s->Tcap, s->Bs);
  const int64_t G = s->Hq / s->Hkv;
  const double sc = orc_scale(s);
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t b = 0; b < s->B; ++b)
    for (int64_t g = 0; g < s->Hkv; ++g)
      for (int64_t j = 0; j < NB; ++j) {
        double best = 0.0;
        for (int64_t hh = 0; hh < G; ++hh) {
          int64_t h = g * G + hh;
          double acc = 0.0;
          for (int64_t d = 0; d < s->D; ++d)
            acc += orc_get(q, s->dtype, (b * s->Hq + h) * s->D + d) *
                   orc_get(summ, s->dtype, ((b * s->Hkv + g) * NBcap + j) * s->D + d);
          if (hh == 0 || acc > best) best = acc;
        }
        int64_t o = (b * s->Hkv + g) * NB + j;
        if (raw) raw[o] = best;
        if (scaled) scaled[o] = sc * best;
      }
}

/* (value, index) pair ordered by value descending, then index ascending. */
typedef struct {
  double val;
  int64_t idx;
} orc_rank;

static int orc_cmp_desc(const void* a, const void* b) {
  const orc_rank* x = (const orc_rank*)a;
  const orc_rank* y = (const orc_rank*)b;
  if (x->val > y->val) return -1;
  if (x->val < y->val) return 1;
  return (x->idx > y->idx) - (x->idx < y->idx);
}

static int orc_cmp_i32(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

/* Top-k [KIN-5]: for each of `rows` rows of `n` scores, the first
 * k_eff = min(k, n) indices in (score desc, index asc) order, written to
 * out[row, 0:k_eff] in ascending index order.  -0.0 and +0.0 compare equal
 * (C comparison).  Returns k_eff. */
int64_t orc_topk(int64_t rows, int64_t n, const double* scores, int64_t k, int32_t* out) {
  const int64_t keff = k < n ? k : n;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    orc_rank* a = (orc_rank*)malloc((size_t)n * sizeof(orc_rank));
    for (int64_t j = 0; j < n; ++j) {
      a[j].val = scores[r * n + j];
      a[j].idx = j;
    }
    qsort(a, (size_t)n, sizeof(orc_rank), orc_cmp_desc);
    for (int64_t i = 0; i < keff; ++i) out[r * keff + i] = (int32_t)a[i].idx;
    qsort(out + r * keff, (size_t)keff, sizeof(int32_t), orc_cmp_i32);
    free(a);
  }
  return keff;
}

/* ---------------------------------------------------------------------- */
/* Exact softmax attention of query head h of sequence b over the listed    */
/* tokens of its KV head ([KIN-4], [KIN-5]): two passes, fp64.              */
static void orc_attend_one(const orc_shape* s, const void* q, const void* k, const void* v,
                           int64_t b, int64_t h, const int64_t* tok, int64_t ntok,
                           double* logit, double* out, double* lse) {
  const int64_t G = s->Hq / s->Hkv;
  const int64_t g = h / G;
  const double sc = orc_scale(s);
  double m = -INFINITY;
  for (int64_t i = 0; i < ntok; ++i) {
    double dot = 0.0;
    for (int64_t d = 0; d < s->D; ++d)
      dot += orc_get(q, s->dtype, (b * s->Hq + h) * s->D + d) *
             orc_get(k, s->dtype, ((b * s->Hkv + g) * s->Tcap + tok[i]) * s->D + d);
    logit[i] = sc * dot;
    if (logit[i] > m) m = logit[i];
  }
  double z = 0.0;
  for (int64_t i = 0; i < ntok; ++i) {
    logit[i] = exp(logit[i] - m); /* now the unnormalised weight */
    z += logit[i];
  }
  for (int64_t d = 0; d < s->D; ++d) {
    double acc = 0.0;
    for (int64_t i = 0; i < ntok; ++i)
      acc += logit[i] * orc_get(v, s->dtype, ((b * s->Hkv + g) * s->Tcap + tok[i]) * s->D + d);
    out[(b * s->Hq + h) * s->D + d] = acc / z;
  }
  if (lse) lse[b * s->Hq + h] = m + log(z);
}

/* Attention over the tokens of selected blocks [KIN-5].  block_idx is
 * [B, Hkv, count]; blocks are visited in the listed order and contribute
 * their tokens below T.  out [B, Hq, D], lse [B, Hq] (nullable). */
void orc_attend_blocks(const orc_shape* s, const void* q, const void* k, const void* v,
                       const int32_t* block_idx, int64_t count, double* out, double* lse) {
  const int64_t G = s->Hq / s->Hkv;
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int64_t b = 0; b < s->B; ++b)
    for (int64_t h = 0; h < s->Hq; ++h) {
      int64_t g = h / G;
      int64_t* tok = (int64_t*)malloc((size_t)(count * s->Bs) * sizeof(int64_t));
      double* wk = (double*)malloc((size_t)(count * s->Bs) * sizeof(double));
      int64_t n = 0;
      for (int64_t i = 0; i < count; ++i) {
        int64_t j = block_idx[(b * s->Hkv + g) * count + i];
        for (int64_t t = j * s->Bs; t < (j + 1) * s->Bs && t < s->T; ++t) tok[n++] = t;
      }
      orc_attend_one(s, q, k, v, b, h, tok, n, wk, out, lse);
      free(tok);
      free(wk);
    }
}

/* Attention over one token list per sequence, shared by every head of the
 * sequence [LIM-5].  token_idx is [B, count]. */
void orc_attend_tokens(const orc_shape* s, const void* q, const void* k, const void* v,
                       const int32_t* token_idx, int64_t count, double* out, double* lse) {
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int64_t b = 0; b < s->B; ++b)
    for (int64_t h = 0; h < s->Hq; ++h) {
      int64_t* tok = (int64_t*)malloc((size_t)count * sizeof(int64_t));
      double* wk = (double*)malloc((size_t)count * sizeof(double));
      for (int64_t i = 0; i < count; ++i) tok[i] = token_idx[b * count + i];
      orc_attend_one(s, q, k, v, b, h, tok, count, wk, out, lse);
      free(tok);
      free(wk);
    }
}

/* Dense decode attention over tokens [0, T) [KIN-4]. */
void orc_attend_dense(const orc_shape* s, const void* q, const void* k, const void* v,
                      double* out, double* lse) {
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int64_t b = 0; b < s->B; ++b)
    for (int64_t h = 0; h < s->Hq; ++h) {
      int64_t* tok = (int64_t*)malloc((size_t)s->T * sizeof(int64_t));
      double* wk = (double*)malloc((size_t)s->T * sizeof(double));
      for (int64_t t = 0; t < s->T; ++t) tok[t] = t;
      orc_attend_one(s, q, k, v, b, h, tok, s->T, wk, out, lse);
      free(tok);
      free(wk);
    }
}

/* ---------------------------------------------------------------------- */
/* Vote-union selection [LIM-2], [LIM-5], split into its steps so that     */
/* each can be fed the GPU's own intermediate.                             */

/* Full per-head score matrix [LIM-5]: logits[b,h,t] = q_h . k_{g(h),t} for
 * every head and every t < T (unscaled: a positive scale does not change a
 * head's ranking).  logits is [B, Hq, T]. */
void orc_head_logits(const orc_shape* s, const void* q, const void* k, double* logits) {
  const int64_t G = s->Hq / s->Hkv;
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t b = 0; b < s->B; ++b)
    for (int64_t h = 0; h < s->Hq; ++h) {
      int64_t g = h / G;
      for (int64_t t = 0; t < s->T; ++t) {
        double dot = 0.0;
        for (int64_t d = 0; d < s->D; ++d)
          dot += orc_get(q, s->dtype, (b * s->Hq + h) * s->D + d) *
                 orc_get(k, s->dtype, ((b * s->Hkv + g) * s->Tcap + t) * s->D + d);
        logits[(b * s->Hq + h) * s->T + t] = dot;
      }
    }
}

/* Equal votes per head [LIM-2]: with T > N, every head h picks the first
 * N-W history tokens t < T-W in (logit desc, t asc) order, and votes[b,t]
 * counts the heads that picked t.  Tokens t >= T-W get 0 votes; with T <= N
 * no vote is taken and every count is 0.  logits [B,Hq,T], votes [B,T]. */
void orc_votes(int64_t B, int64_t Hq, int64_t T, const double* logits, int64_t N, int64_t W,
               int32_t* votes) {
  memset(votes, 0, (size_t)(B * T) * sizeof(int32_t));
  if (T <= N) return;
  const int64_t C = T - W, Kv = N - W;
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < B; ++b) {
    orc_rank* a = (orc_rank*)malloc((size_t)C * sizeof(orc_rank));
    for (int64_t h = 0; h < Hq; ++h) {
      for (int64_t t = 0; t < C; ++t) {
        a[t].val = logits[(b * Hq + h) * T + t];
        a[t].idx = t;
      }
      qsort(a, (size_t)C, sizeof(orc_rank), orc_cmp_desc);
      for (int64_t i = 0; i < Kv; ++i) votes[b * T + a[i].idx] += 1;
    }
    free(a);
  }
}

/* Shared token set from the vote counts [LIM-2], [LIM-5]: with T > N, the
 * first N-W history tokens in (votes desc, t asc) order, in ascending order,
 * followed by the W most recent tokens [T-W, T); with T <= N, all of
 * [0, T).  token_idx is [B, min(N, T)]; returns min(N, T). */
int64_t orc_set_from_votes(int64_t B, int64_t T, const int32_t* votes, int64_t N, int64_t W,
                           int32_t* token_idx) {
  const int64_t n_out = N < T ? N : T;
  if (T <= N) {
    for (int64_t b = 0; b < B; ++b)
      for (int64_t t = 0; t < T; ++t) token_idx[b * n_out + t] = (int32_t)t;
    return n_out;
  }
  const int64_t C = T - W, Kv = N - W;
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < B; ++b) {
    orc_rank* a = (orc_rank*)malloc((size_t)C * sizeof(orc_rank));
    for (int64_t t = 0; t < C; ++t) {
      a[t].val = (double)votes[b * T + t];
      a[t].idx = t;
    }
    qsort(a, (size_t)C, sizeof(orc_rank), orc_cmp_desc);
    int32_t* row = token_idx + b * n_out;
    for (int64_t i = 0; i < Kv; ++i) row[i] = (int32_t)a[i].idx;
    qsort(row, (size_t)Kv, sizeof(int32_t), orc_cmp_i32);
    for (int64_t i = 0; i < W; ++i) row[Kv + i] = (int32_t)(C + i);
    free(a);
  }
  return n_out;
}

/* Whole vote-union selection: logits -> votes -> set.  logits_ws is a
 * caller buffer of B*Hq*T doubles; votes [B,T]; token_idx [B,min(N,T)]. */
int64_t orc_vote_select(const orc_shape* s, const void* q, const void* k, int64_t N, int64_t W,
                        double* logits_ws, int32_t* votes, int32_t* token_idx) {
  if (s->T > N) orc_head_logits(s, q, k, logits_ws);
  orc_votes(s->B, s->Hq, s->T, logits_ws, N, W, votes);
  return orc_set_from_votes(s->B, s->T, votes, N, W, token_idx);
}
