/* Drives every function of oracle/moe_oracle.c on tiny inputs (and a few
 * invalid calls), for a build under AddressSanitizer and UndefinedBehavior-
 * Sanitizer: any out-of-bounds access, use of freed memory, leak, signed
 * overflow or misaligned access aborts the run.  Exit status 0 = clean. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int orc_router_logits(int32_t, int32_t, int32_t, const uint16_t *, const uint16_t *, double *);
int orc_route_topk(int32_t, int32_t, int32_t, const void *, int32_t, const float *, int32_t,
                   int32_t *, float *, double *);
int orc_eplb_phys(int32_t, int32_t, int32_t, int32_t, const int32_t *, const int32_t *,
                  const int32_t *, int32_t *);
int orc_quant_tokens(int32_t, int32_t, const void *, int32_t, int8_t *, float *);
int orc_quant_blocks(int32_t, int32_t, int32_t, const uint16_t *, int8_t *, float *);
int orc_dispatch_layout(const int32_t *, const int32_t *, const int32_t *, uint32_t, int32_t *,
                        int32_t *, int32_t *, int32_t *, int32_t *, int32_t *, int32_t *);
int orc_dispatch_rows(const int32_t *, const int8_t *, const float *, const int32_t *,
                      const int32_t *, uint32_t, int64_t, int64_t, uint8_t *);
int orc_expert_ffn(int32_t, int32_t, int32_t, const int8_t *, const float *, const int8_t *,
                   const float *, const int8_t *, const float *, int32_t *, int8_t *, float *,
                   int32_t *, uint16_t *);
int orc_combine(int32_t, int32_t, int32_t, int32_t, const void *, int64_t, int64_t, int32_t,
                const int32_t *, const float *, int32_t, void *);
int orc_eplb_plan(int32_t, int32_t, const int64_t *, int32_t, int32_t, const int32_t *,
                  const int32_t *, int32_t *, int32_t *, int32_t *, int32_t *, int32_t *, double *);
int orc_static_buffer(int64_t, int64_t, int64_t, int64_t, int64_t, int64_t *);

static uint32_t rng = 12345u;
static uint32_t next(void) { rng = rng * 1664525u + 1013904223u; return rng >> 8; }
static float unif(void) { return (float)(next() & 0xffff) / 65536.0f * 2.0f - 1.0f; }
static uint16_t bf16(float f) { uint32_t u; memcpy(&u, &f, 4); return (uint16_t)(u >> 16); }

#define CHECK(x) do { int rc_ = (x); if (rc_ != 0) { printf("FAIL %s -> %d\n", #x, rc_); return 1; } } while (0)
#define EXPECT_ERR(x) do { if ((x) == 0) { printf("FAIL %s accepted\n", #x); return 1; } } while (0)

int main(void) {
  enum { T = 12, H = 32, E = 6, P = 6, K = 2, D = 3, EPP = 2, S = 3, LB = 4, MSG = 48 };
  /* gate logits and routing */
  uint16_t xb[T * H], wr[E * H];
  for (int i = 0; i < T * H; ++i) xb[i] = bf16(unif());
  for (int i = 0; i < E * H; ++i) wr[i] = bf16(unif());
  double logits64[T * E];
  CHECK(orc_router_logits(T, E, H, xb, wr, logits64));
  float lg[T * E], bias[E];
  for (int i = 0; i < T * E; ++i) lg[i] = (float)logits64[i];
  for (int e = 0; e < E; ++e) bias[e] = 0.1f * (float)e;
  int32_t ids[T * K];
  float sc[T * K];
  double tw[T * K];
  CHECK(orc_route_topk(T, E, K, lg, 0, bias, 0, ids, sc, tw));
  uint16_t lgb[T * E];
  for (int i = 0; i < T * E; ++i) lgb[i] = bf16(lg[i]);
  CHECK(orc_route_topk(T, E, K, lgb, 1, NULL, 1, ids, sc, tw));
  int32_t phys[T * K];
  CHECK(orc_eplb_phys(T, K, LB, E, ids, NULL, NULL, phys));
  int32_t ro[E + 1], rs[P];
  for (int e = 0; e <= E; ++e) ro[e] = e;
  for (int p = 0; p < P; ++p) rs[p] = p;
  CHECK(orc_eplb_phys(T, K, LB, E, ids, ro, rs, phys));
  /* quantization */
  float xf[T * H];
  for (int i = 0; i < T * H; ++i) xf[i] = unif() * 3.0f;
  for (int h = 0; h < H; ++h) xf[5 * H + h] = 0.0f; /* an all-zero token */
  int8_t q[T * H];
  float s[T];
  CHECK(orc_quant_tokens(T, H, xf, 0, q, s));
  CHECK(orc_quant_tokens(T, H, xb, 1, q, s));
  int8_t qb[T * H];
  float sb[T * 3];
  CHECK(orc_quant_blocks(T, H, 12, xb, qb, sb)); /* blocks of 12, 12 and 8 columns */
  /* dispatch layout and rows */
  const int32_t geom[10] = {T, H, E, P, K, D, EPP, S, LB, MSG};
  int32_t sp[P];
  for (int p = 0; p < P; ++p) sp[p] = p / EPP;
  int32_t meta[D * S * 4], scnt[P], soff[P + 1], srows[T * K], drow[T * K], rrow[T * K], sloc[P];
  CHECK(orc_dispatch_layout(geom, phys, sp, 7u, meta, scnt, soff, srows, drow, rrow, sloc));
  uint8_t *rows = malloc((size_t)T * K * MSG);
  CHECK(orc_dispatch_rows(geom, q, s, phys, sloc, 7u, 0, T, rows));
  CHECK(orc_dispatch_rows(geom, q, s, phys, sloc, 7u, 3, 9, rows));
  /* expert FFN */
  enum { N = 3, HF = 64, I = 32 };
  int8_t qr[N * HF], wgu[2 * I * HF], wd[HF * I];
  float sr[N], sgu[2 * I], sd[HF];
  for (int i = 0; i < N * HF; ++i) qr[i] = (int8_t)((int)(next() % 255) - 127);
  for (int i = 0; i < 2 * I * HF; ++i) wgu[i] = (int8_t)((int)(next() % 255) - 127);
  for (int i = 0; i < HF * I; ++i) wd[i] = (int8_t)((int)(next() % 255) - 127);
  for (int i = 0; i < N; ++i) sr[i] = 0.01f;
  for (int i = 0; i < 2 * I; ++i) sgu[i] = 1e-3f;
  for (int i = 0; i < HF; ++i) sd[i] = 1e-3f;
  int32_t acc_gu[N * 2 * I], acc_d[N * HF];
  int8_t hq[N * I];
  float hs[N];
  uint16_t y[N * HF];
  CHECK(orc_expert_ffn(N, HF, I, qr, sr, wgu, sgu, wd, sd, acc_gu, hq, hs, acc_d, y));
  CHECK(orc_expert_ffn(N, HF, I, qr, sr, wgu, sgu, wd, sd, NULL, hq, hs, NULL, y));
  /* combine in its three modes */
  int32_t ident[T * K];
  float w32[T * K];
  for (int i = 0; i < T * K; ++i) { ident[i] = i; w32[i] = (float)tw[i]; }
  float outf[T * H];
  uint16_t outb[T * H];
  CHECK(orc_combine(T, K, H, 0, rows, MSG, H, 0, ident, w32, 0, outf));
  uint16_t ret[T * K * H];
  for (int i = 0; i < T * K * H; ++i) ret[i] = bf16(unif());
  CHECK(orc_combine(T, K, H, 1, ret, H * 2, 0, 0, ident, w32, 1, outb));
  uint8_t *q8rows = calloc((size_t)T * K, 64);
  int8_t qq[T * K * H];
  float ss[T * K * 2];
  CHECK(orc_quant_blocks(T * K, H, 16, ret, qq, ss));
  for (int r = 0; r < T * K; ++r) {
    memcpy(q8rows + (size_t)r * 64, qq + r * H, H);
    memcpy(q8rows + (size_t)r * 64 + H, ss + 2 * r, 8);
  }
  CHECK(orc_combine(T, K, H, 2, q8rows, 64, H, 16, ident, w32, 0, outf));
  /* replica planner */
  int64_t counts[2 * E];
  for (int i = 0; i < 2 * E; ++i) counts[i] = (int64_t)(next() % 100);
  int32_t prim[E], freec[9], ro2[E + 1], rs2[E + 3], sp2[E + 3], sl2[E + 3], sel[3];
  double tail[4];
  for (int e = 0; e < E; ++e) prim[e] = e;
  for (int d = 0; d < 9; ++d) freec[d] = d >= E;
  CHECK(orc_eplb_plan(2, E, counts, 3, 9, prim, freec, ro2, rs2, sp2, sl2, sel, tail));
  int32_t nofree[9] = {0};
  EXPECT_ERR(orc_eplb_plan(2, E, counts, 3, 9, prim, nofree, ro2, rs2, sp2, sl2, sel, tail));
  int64_t sz[2];
  CHECK(orc_static_buffer(320, 96, 8, 1, 7680, sz));
  /* invalid arguments are refused */
  EXPECT_ERR(orc_route_topk(T, E, E + 1, lg, 0, NULL, 0, ids, sc, tw));
  EXPECT_ERR(orc_quant_tokens(T, 0, xf, 0, q, s));
  EXPECT_ERR(orc_combine(T, 0, H, 0, rows, MSG, H, 0, ident, w32, 0, outf));
  free(rows);
  free(q8rows);
  printf("oracle driver ok\n");
  return 0;
}
