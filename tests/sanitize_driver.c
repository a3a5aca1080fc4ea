/* Runs the oracle and the input generator on small, ragged inputs so that a
   build with the address and undefined-behaviour sanitizers can check them.
   Exit status 0 means every call ran without a sanitizer report. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void qsa_gen_init(void);
void qsa_gen_normal_bf16(uint64_t seed, uint32_t stream, uint64_t e0, uint64_t n, float scale, uint16_t* out);
void qsa_gen_int_bf16(uint64_t seed, uint32_t stream, uint64_t e0, uint64_t n, int lo, int hi, uint16_t* out);
void qsa_gen_needle_dir(uint64_t seed, int d, double* u);
int64_t qsa_gen_needle_offset(uint64_t seed, int64_t b, int64_t w, int64_t window, int r);
void qsa_gen_idx_keys_bf16(uint64_t seed, int64_t b, int64_t L, int64_t s0, int64_t ns, int d, int64_t window, int r,
                           uint16_t* out);
void qsa_ref_compress(const uint16_t* keys, int64_t L, int d, int r, uint16_t* out);
int64_t qsa_ref_select(const uint16_t* idx_q, const uint16_t* blocks, int64_t t0, int nq, int H, int d, int r, int k,
                       double w, int32_t* sel, int32_t* cnt, float* band);
void qsa_ref_sparse_attn(const uint16_t* Q, const uint16_t* K, const uint16_t* V, int64_t t0, int nq, int Hq, int Hkv,
                         int D, double scale, int r, int k, const int32_t* sel, const int32_t* cnt, double* out,
                         double* lse);
void qsa_ref_dense_attn(const uint16_t* Q, const uint16_t* K, const uint16_t* V, int64_t t0, int nq, int Hq, int Hkv,
                        int D, double scale, double* out, double* lse);
void qsa_ref_distill_kl(const uint16_t* Q, const uint16_t* K, const uint16_t* idx_q, const uint16_t* blocks,
                        int64_t t0, int nq, int Hq, int Hkv, int D, double scale, int Hi, int di, double w, int r,
                        double* kl);
void qsa_ref_gdn(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* g, const float* beta,
                 const float* S0, int64_t T, int Hqk, int Hv, int dk, int dv, double scale, const int32_t* heads,
                 int n_heads, double* o, double* S_out);

static void* xmalloc(size_t n) {
  void* p = malloc(n ? n : 1);
  if (!p) exit(3);
  return p;
}

int main(void) {
  const int L = 203, r = 4, d = 64, Hi = 4, Hq = 8, Hkv = 2, D = 128, k = 9, t0 = 150, nq = L - 150;
  qsa_gen_init();
  uint16_t* ik = xmalloc(sizeof(uint16_t) * L * d);
  uint16_t* iq = xmalloc(sizeof(uint16_t) * nq * Hi * d);
  uint16_t* Q = xmalloc(sizeof(uint16_t) * nq * Hq * D);
  uint16_t* K = xmalloc(sizeof(uint16_t) * L * Hkv * D);
  uint16_t* V = xmalloc(sizeof(uint16_t) * L * Hkv * D);
  qsa_gen_idx_keys_bf16(5, 0, L, 0, L, d, 64, r, ik);
  qsa_gen_int_bf16(5, 4, 0, (uint64_t)nq * Hi * d, -2, 2, iq);
  qsa_gen_normal_bf16(5, 1, 0, (uint64_t)nq * Hq * D, 1.0f, Q);
  qsa_gen_normal_bf16(5, 2, 0, (uint64_t)L * Hkv * D, 1.0f, K);
  qsa_gen_normal_bf16(5, 3, 0, (uint64_t)L * Hkv * D, 1.0f, V);
  double u[64];
  qsa_gen_needle_dir(5, d, u);
  (void)qsa_gen_needle_offset(5, 0, 1, 64, r);

  const int nb = L / r;
  uint16_t* blocks = xmalloc(sizeof(uint16_t) * nb * d);
  qsa_ref_compress(ik, L, d, r, blocks);
  int32_t* sel = xmalloc(sizeof(int32_t) * nq * k);
  int32_t* cnt = xmalloc(sizeof(int32_t) * nq);
  float* band = xmalloc(sizeof(float) * nq * 2);
  (void)qsa_ref_select(iq, blocks, t0, nq, Hi, d, r, k, 1.0 / Hi, sel, cnt, band);
  double* out = xmalloc(sizeof(double) * nq * Hq * D);
  double* lse = xmalloc(sizeof(double) * nq * Hq);
  qsa_ref_sparse_attn(Q, K, V, t0, nq, Hq, Hkv, D, 1.0 / sqrt((double)D), r, k, sel, cnt, out, lse);
  qsa_ref_dense_attn(Q, K, V, t0, nq, Hq, Hkv, D, 1.0 / sqrt((double)D), out, lse);

  /* distillation loss: 8 query heads per KV head, 8 indexer heads */
  const int Hq8 = 8 * Hkv;
  uint16_t* Q8 = xmalloc(sizeof(uint16_t) * nq * Hq8 * D);
  uint16_t* iq8 = xmalloc(sizeof(uint16_t) * nq * 8 * d);
  qsa_gen_normal_bf16(6, 1, 0, (uint64_t)nq * Hq8 * D, 1.0f, Q8);
  qsa_gen_normal_bf16(6, 4, 0, (uint64_t)nq * 8 * d, 1.0f, iq8);
  double* kl = xmalloc(sizeof(double) * nq);
  qsa_ref_distill_kl(Q8, K, iq8, blocks, t0, nq, Hq8, Hkv, D, 1.0 / sqrt((double)D), 8, d, 1.0 / 8, r, kl);

  /* gated delta rule: 37 tokens, 2 key heads, 4 value heads, dims 16 x 8 */
  const int T = 37, Hqk = 2, Hv = 4, dk = 16, dv = 8;
  uint16_t* gq = xmalloc(sizeof(uint16_t) * T * Hqk * dk);
  uint16_t* gk = xmalloc(sizeof(uint16_t) * T * Hqk * dk);
  uint16_t* gv = xmalloc(sizeof(uint16_t) * T * Hv * dv);
  qsa_gen_normal_bf16(7, 8, 0, (uint64_t)T * Hqk * dk, 0.25f, gq);
  qsa_gen_normal_bf16(7, 9, 0, (uint64_t)T * Hqk * dk, 0.25f, gk);
  qsa_gen_normal_bf16(7, 10, 0, (uint64_t)T * Hv * dv, 1.0f, gv);
  float* gg = xmalloc(sizeof(float) * T * Hv);
  float* gb = xmalloc(sizeof(float) * T * Hv);
  float* S0 = xmalloc(sizeof(float) * Hv * dv * dk);
  for (int i = 0; i < T * Hv; ++i) {
    gg[i] = -0.05f * (float)(i % 7);
    gb[i] = 0.1f * (float)(i % 10);
  }
  for (int i = 0; i < Hv * dv * dk; ++i) S0[i] = 0.01f * (float)(i % 13);
  int32_t heads[3] = {0, 2, 3};
  double* go = xmalloc(sizeof(double) * T * Hv * dv);
  double* gs = xmalloc(sizeof(double) * Hv * dv * dk);
  qsa_ref_gdn(gq, gk, gv, gg, gb, S0, T, Hqk, Hv, dk, dv, 0.5, heads, 3, go, gs);
  qsa_ref_gdn(gq, gk, gv, gg, gb, NULL, T, Hqk, Hv, dk, dv, 0.5, heads, 3, go, gs);

  double chk = lse[0] + kl[nq - 1] + go[0] + gs[0];
  printf("sanitized run done (%g)\n", chk);
  free(ik); free(iq); free(Q); free(K); free(V); free(blocks); free(sel); free(cnt); free(band);
  free(out); free(lse); free(Q8); free(iq8); free(kl); free(gq); free(gk); free(gv); free(gg); free(gb);
  free(S0); free(go); free(gs);
  return 0;
}
