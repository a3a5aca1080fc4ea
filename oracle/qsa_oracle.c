/*
 * CPU oracle for Qwen Sparse Attention (QSA).
 *
 * TEST INFRASTRUCTURE ONLY. This file is the plain, slow, obviously correct
 * statement of what the GPU path computes. Only the tests, the package smoke
 * check and the benchmark's CPU-baseline leg load it. It shares no code, header,
 * table or helper with the GPU library, and the product path never calls it.
 *
 * Sources (web pages about the Qwen3.8-Flash-Next release):
 *   [EXPLAINER] "用125亿分之6的参数，打平3970亿的旗舰模型", section
 *               "稀疏注意力：给检索建索引，也得先学会省纸" (how QSA works).
 *   [DIGEST]    "On the Design of Qwen3.8-Next Architecture: Evaluation,
 *               Efficiency, and Training Stability" (agihunt.info digest of
 *               arXiv 2608.30320), paragraph on token mixing.
 *   [NEWS]      "Qwen3.8-Flash发布并开源…" (AITOP100), section 二, item 1
 *               (attention mechanism).
 *
 * The method, step by step, as those passages describe it:
 *   O1 compress  r consecutive tokens form a micro-block; the block's indexer
 *                key is the mean of its r token keys  [EXPLAINER].
 *   O2 score     a lightweight multi-query indexer (many query heads, one
 *                shared key) scores every block for each query  [EXPLAINER].
 *                The pages give no formula; the reading taken here is
 *                s(t, j) = sum_h w_h * max(0, q_{t,h} . c_j), w_h = 1/H.
 *   O3 select    the highest-scoring blocks are kept, up to a token budget
 *                (deployed: 2048 tokens at r = 4, so k = 512 blocks)  [DIGEST],
 *                [EXPLAINER]. Readings: candidates are the complete blocks
 *                before the query's own block; the query's own (diagonal)
 *                block is always kept and counts towards k; ties go to the
 *                lower block index.
 *   O4 expand    kept blocks are expanded back to their tokens  [DIGEST],
 *                [EXPLAINER]; tokens after the query are dropped (causal).
 *   O5 attend    exact softmax attention over only those tokens  [NEWS],
 *                [EXPLAINER]; GQA: query head h reads KV head h / (Hq/Hkv).
 *   O6 dense     O5 with every token 0..t: the full attention QSA replaces.
 *   O7 distill   forward of the indexer's KL loss against the dense
 *                attention mass per block  [EXPLAINER].
 *   O8 gdn       the gated delta rule of the recurrent layers between the
 *                attention layers  [EXPLAINER], [DIGEST].
 *
 * Arithmetic: inputs are bf16 bit patterns widened exactly. O1 follows the
 * fixed fp32 rule (left-to-right fp32 sum, divide by r, round to nearest even
 * bf16) so that the stored block keys are a unique byte pattern. O2, O5 to
 * O8 work in double; O2 rounds each score once to fp32. Every value is
 * computed by one thread in a fixed order, so results do not depend on the
 * thread count. Build without -ffast-math and with -ffp-contract=off.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double widen(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

static float widen_f(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* fp32 -> bf16, round to nearest, ties to even (NaN kept quiet). */
static uint16_t round_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if (isnan(f)) return (uint16_t)((u >> 16) | 0x0040u);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

/* ---------------------------------------------------------------- O1 ---- */
/* keys: [L][d] token keys of one sequence. out: [L / r][d] block keys.
   A trailing partial block (L mod r tokens) is not a block and is skipped. */
void qsa_ref_compress(const uint16_t* keys, int64_t L, int d, int r, uint16_t* out) {
  const int64_t nblk = L / r;
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < nblk; ++j) {
    for (int i = 0; i < d; ++i) {
      float sum = widen_f(keys[(j * r) * d + i]);
      for (int m = 1; m < r; ++m) sum = sum + widen_f(keys[(j * r + m) * d + i]);
      float mean = sum / (float)r;
      out[j * d + i] = round_bf16(mean);
    }
  }
}

/* ---------------------------------------------------------------- O2 ---- */
static float score_block(const uint16_t* q, const uint16_t* c, int H, int d, double w) {
  double s = 0.0;
  for (int h = 0; h < H; ++h) {
    double x = 0.0;
    for (int i = 0; i < d; ++i) x += widen(q[h * d + i]) * widen(c[i]);
    if (x > 0.0) s += w * x;
  }
  return (float)s;
}

/* q: [H][d] indexer query of one token; blocks: [n][d]. out: [n] fp32 scores. */
void qsa_ref_scores(const uint16_t* q, const uint16_t* blocks, int64_t n, int H, int d, double w,
                    float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < n; ++j) out[j] = score_block(q, blocks + j * d, H, d, w);
}

/* ---------------------------------------------------------------- O3 ---- */
typedef struct {
  float s;
  int32_t j;
} cand_t;

/* Order: higher score first; equal scores, lower block index first. */
static int by_score_then_index(const void* pa, const void* pb) {
  const cand_t* a = (const cand_t*)pa;
  const cand_t* b = (const cand_t*)pb;
  if (a->s > b->s) return -1;
  if (a->s < b->s) return 1;
  return (a->j > b->j) - (a->j < b->j);
}

static int ascending_i32(const void* pa, const void* pb) {
  int32_t a = *(const int32_t*)pa, b = *(const int32_t*)pb;
  return (a > b) - (a < b);
}

/* Block selection for the queries at positions t0 .. t0 + nq - 1 of one
   sequence. idx_q: [nq][H][d]; blocks: the sequence's block keys, at least
   (t0 + nq - 1) / r of them. For query t with own block b = t / r:
     scored candidates: blocks 0 .. b-1 (all complete, all before t);
     kept: the first min(k - 1, b) candidates in (score desc, index asc)
           order, plus block b itself;
     sel[i][0 .. n-1]: kept blocks ascending, the rest -1; cnt[i] = n.
   band (nullable, [nq][2]): score of the last kept and of the first dropped
   scored candidate in that order (NaN where there is none).
   Returns the number of (query, block) pairs scored. */
int64_t qsa_ref_select(const uint16_t* idx_q, const uint16_t* blocks, int64_t t0, int nq, int H,
                       int d, int r, int k, double w, int32_t* sel, int32_t* cnt, float* band) {
  int64_t pairs = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : pairs)
  for (int i = 0; i < nq; ++i) {
    const int64_t t = t0 + i;
    const int64_t b = t / r;
    cand_t* c = (cand_t*)malloc(sizeof(cand_t) * (size_t)(b > 0 ? b : 1));
    for (int64_t j = 0; j < b; ++j) {
      c[j].s = score_block(idx_q + (int64_t)i * H * d, blocks + j * d, H, d, w);
      c[j].j = (int32_t)j;
    }
    pairs += b;
    qsort(c, (size_t)b, sizeof(cand_t), by_score_then_index);
    const int64_t m = b < (int64_t)(k - 1) ? b : (int64_t)(k - 1);
    int32_t* row = sel + (int64_t)i * k;
    for (int64_t x = 0; x < m; ++x) row[x] = c[x].j;
    row[m] = (int32_t)b;
    qsort(row, (size_t)(m + 1), sizeof(int32_t), ascending_i32);
    for (int64_t x = m + 1; x < k; ++x) row[x] = -1;
    cnt[i] = (int32_t)(m + 1);
    if (band) {
      band[2 * i + 0] = m > 0 ? c[m - 1].s : NAN;
      band[2 * i + 1] = b > m ? c[m].s : NAN;
    }
    free(c);
  }
  return pairs;
}

/* ------------------------------------------------------------ O4 + O5 --- */
/* Exact softmax attention of one query over an explicit token list.
   q: [Hq][D]; K, V: [*][Hkv][D] (row = token); out: [Hq][D]; lse: [Hq]. */
static void attend_list(const uint16_t* q, const uint16_t* K, const uint16_t* V, int Hq, int Hkv,
                        int D, double scale, const int64_t* tok, int64_t ntok, double* out,
                        double* lse) {
  const int G = Hq / Hkv;
  double* logit = (double*)malloc(sizeof(double) * (size_t)(ntok > 0 ? ntok : 1));
  for (int h = 0; h < Hq; ++h) {
    const int g = h / G;
    double mx = -INFINITY;
    for (int64_t x = 0; x < ntok; ++x) {
      const uint16_t* krow = K + (tok[x] * Hkv + g) * D;
      double dot = 0.0;
      for (int i = 0; i < D; ++i) dot += widen(q[h * D + i]) * widen(krow[i]);
      logit[x] = scale * dot;
      if (logit[x] > mx) mx = logit[x];
    }
    double z = 0.0;
    for (int i = 0; i < D; ++i) out[h * D + i] = 0.0;
    for (int64_t x = 0; x < ntok; ++x) {
      const double p = exp(logit[x] - mx);
      z += p;
      const uint16_t* vrow = V + (tok[x] * Hkv + g) * D;
      for (int i = 0; i < D; ++i) out[h * D + i] += p * widen(vrow[i]);
    }
    for (int i = 0; i < D; ++i) out[h * D + i] /= z;
    lse[h] = mx + log(z);
  }
  free(logit);
}

void qsa_ref_attend_tokens(const uint16_t* q, const uint16_t* K, const uint16_t* V, int Hq, int Hkv,
                           int D, double scale, const int64_t* tok, int64_t ntok, double* out,
                           double* lse) {
  attend_list(q, K, V, Hq, Hkv, D, scale, tok, ntok, out, lse);
}

/* Sparse attention (O4 expand + O5) for queries t0 .. t0 + nq - 1.
   Q: [nq][Hq][D]; K, V: [L][Hkv][D]; sel/cnt as written by qsa_ref_select.
   out: [nq][Hq][D]; lse: [nq][Hq]. */
void qsa_ref_sparse_attn(const uint16_t* Q, const uint16_t* K, const uint16_t* V, int64_t t0, int nq,
                         int Hq, int Hkv, int D, double scale, int r, int k, const int32_t* sel,
                         const int32_t* cnt, double* out, double* lse) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int i = 0; i < nq; ++i) {
    const int64_t t = t0 + i;
    int64_t* tok = (int64_t*)malloc(sizeof(int64_t) * (size_t)k * (size_t)r);
    int64_t n = 0;
    for (int x = 0; x < cnt[i]; ++x) {
      const int64_t j = sel[(int64_t)i * k + x];
      for (int m = 0; m < r; ++m) {
        const int64_t s = j * r + m;
        if (s <= t) tok[n++] = s;
      }
    }
    attend_list(Q + (int64_t)i * Hq * D, K, V, Hq, Hkv, D, scale, tok, n,
                out + (int64_t)i * Hq * D, lse + (int64_t)i * Hq);
    free(tok);
  }
}

/* ---------------------------------------------------------------- O6 ---- */
/* Dense causal attention: every token 0 .. t. Same layouts as above. */
void qsa_ref_dense_attn(const uint16_t* Q, const uint16_t* K, const uint16_t* V, int64_t t0, int nq,
                        int Hq, int Hkv, int D, double scale, double* out, double* lse) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int i = 0; i < nq; ++i) {
    const int64_t t = t0 + i;
    int64_t* tok = (int64_t*)malloc(sizeof(int64_t) * (size_t)(t + 1));
    for (int64_t s = 0; s <= t; ++s) tok[s] = s;
    attend_list(Q + (int64_t)i * Hq * D, K, V, Hq, Hkv, D, scale, tok, t + 1,
                out + (int64_t)i * Hq * D, lse + (int64_t)i * Hq);
    free(tok);
  }
}

/* ---------------------------------------------------------------- O7 ---- */
/* Forward of the indexer's dense-distillation loss. [EXPLAINER] describes a
   first training stage in which only the indexer learns, with a KL divergence
   that pulls it towards the full-attention model's attention distribution.
   The pages give no formula; the reading taken here, for query t with own
   block b_t and candidate blocks j < b_t:
     target     P_j = M_j / sum_{j' < b_t} M_{j'},
                M_j = sum_h sum_{s in block j} a_h(s), a_h the dense causal
                softmax of query head h over the tokens s <= t (as in O6);
     indexer    Q_j = exp(s_j) / sum_{j' < b_t} exp(s_{j'}), s_j the O2 score
                (rounded to fp32, used as a logit);
     loss       KL_t = sum_j P_j (ln P_j - ln Q_j), with 0 ln 0 = 0;
                KL_t = 0 when b_t = 0 (no candidate).
   Q: [nq][Hq][D]; K: [L][Hkv][D]; idx_q: [nq][Hi][di]; blocks: [*][di].
   kl: [nq] (double). */
void qsa_ref_distill_kl(const uint16_t* Q, const uint16_t* K, const uint16_t* idx_q,
                        const uint16_t* blocks, int64_t t0, int nq, int Hq, int Hkv, int D,
                        double scale, int Hi, int di, double w, int r, double* kl) {
  const int G = Hq / Hkv;
#pragma omp parallel for schedule(dynamic, 1)
  for (int i = 0; i < nq; ++i) {
    const int64_t t = t0 + i;
    const int64_t bt = t / r;
    if (bt == 0) {
      kl[i] = 0.0;
      continue;
    }
    double* logit = (double*)malloc(sizeof(double) * (size_t)(t + 1));
    double* mass = (double*)calloc((size_t)bt, sizeof(double));
    for (int h = 0; h < Hq; ++h) {
      const int g = h / G;
      const uint16_t* q = Q + ((int64_t)i * Hq + h) * D;
      double mx = -INFINITY;
      for (int64_t s = 0; s <= t; ++s) {
        const uint16_t* krow = K + (s * Hkv + g) * D;
        double dot = 0.0;
        for (int x = 0; x < D; ++x) dot += widen(q[x]) * widen(krow[x]);
        logit[s] = scale * dot;
        if (logit[s] > mx) mx = logit[s];
      }
      double z = 0.0;
      for (int64_t s = 0; s <= t; ++s) z += exp(logit[s] - mx);
      for (int64_t s = 0; s < bt * r; ++s) mass[s / r] += exp(logit[s] - mx) / z;
    }
    double msum = 0.0;
    for (int64_t j = 0; j < bt; ++j) msum += mass[j];
    // indexer logits and their log-sum-exp
    float* sc = (float*)malloc(sizeof(float) * (size_t)bt);
    double smax = -INFINITY;
    for (int64_t j = 0; j < bt; ++j) {
      sc[j] = score_block(idx_q + (int64_t)i * Hi * di, blocks + j * di, Hi, di, w);
      if (sc[j] > smax) smax = sc[j];
    }
    double zs = 0.0;
    for (int64_t j = 0; j < bt; ++j) zs += exp((double)sc[j] - smax);
    const double lse_s = smax + log(zs);
    double acc = 0.0;
    for (int64_t j = 0; j < bt; ++j) {
      const double p = mass[j] / msum;
      if (p > 0.0) acc += p * (log(p) - ((double)sc[j] - lse_s));
    }
    kl[i] = acc;
    free(sc);
    free(mass);
    free(logit);
  }
}

/* ---------------------------------------------------------------- O8 ---- */
/* Gated DeltaNet token mixing, the recurrent layer three of every four layers
   use. [EXPLAINER] (section on the memory/efficiency trade-off) and [DIGEST]
   (token-mixing paragraph) describe it: a matrix state holds the compressed
   prefix; for each token the layer forms the error between the token's value
   and what the memory already returns for its key, then a decay gate sets
   how much of the old memory is kept and a write gate how much of the
   correction is written. The pages give no formula; the reading taken here,
   per value head h with state S (dv x dk, zero or a given initial state):
     a_t = exp(g_t)                      decay gate, g_t <= 0 given
     e_t = v_t - a_t S_{t-1} k_t         error against the decayed memory
     S_t = a_t S_{t-1} + b_t e_t k_t^T   b_t in [0, 1]: write gate
     o_t = S_t (scale q_t)
   q, k are the token's key-head vectors (key head h / (Hv / Hqk)); they
   arrive already normalised (that happens before the mixing).
   q, k: [T][Hqk][dk]; v: [T][Hv][dv] bf16; g, beta: [T][Hv] fp32;
   S0: [Hv][dv][dk] fp32 or NULL; o: [T][Hv][dv], S_out: [Hv][dv][dk] double.
   Only the value heads listed in heads[0 .. n_heads) are computed. Each row of
   the state evolves on its own (row i only ever sees v_t[i]), so one thread
   runs one (head, row) pair over every token, in token order. */
void qsa_ref_gdn(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* g,
                 const float* beta, const float* S0, int64_t T, int Hqk, int Hv, int dk, int dv,
                 double scale, const int32_t* heads, int n_heads, double* o, double* S_out) {
  const int grp = Hv / Hqk;
#pragma omp parallel for collapse(2) schedule(dynamic, 4)
  for (int hi = 0; hi < n_heads; ++hi) {
    for (int i = 0; i < dv; ++i) {
      const int h = heads[hi];
      const int hk = h / grp;
      double* s = (double*)malloc(sizeof(double) * (size_t)dk);
      for (int c = 0; c < dk; ++c) s[c] = S0 ? (double)S0[((int64_t)h * dv + i) * dk + c] : 0.0;
      for (int64_t t = 0; t < T; ++t) {
        const uint16_t* kt = k + (t * Hqk + hk) * dk;
        const uint16_t* qt = q + (t * Hqk + hk) * dk;
        const double a = exp((double)g[t * Hv + h]);
        const double b = (double)beta[t * Hv + h];
        double sk = 0.0;
        for (int c = 0; c < dk; ++c) sk += s[c] * widen(kt[c]);
        const double e = widen(v[(t * Hv + h) * dv + i]) - a * sk;
        double sq = 0.0;
        for (int c = 0; c < dk; ++c) {
          s[c] = a * s[c] + b * e * widen(kt[c]);
          sq += s[c] * widen(qt[c]);
        }
        o[(t * Hv + h) * dv + i] = scale * sq;
      }
      for (int c = 0; c < dk; ++c) S_out[((int64_t)h * dv + i) * dk + c] = s[c];
      free(s);
    }
  }
}
