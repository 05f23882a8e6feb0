/* Runs every entry point of the CPU oracle on small seeded problems, for a
 * build with AddressSanitizer and UndefinedBehaviorSanitizer (any report
 * aborts the run). Covers plain, ragged, causal, merged/subdivided block
 * sizes, GQA union, paged, fp32, e4m3 K/V, backward, block selection, the
 * reference planner with tables and forced regimes, and malformed tables. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../oracle/bsa_ref.h"

static uint64_t rng = 0x9e3779b97f4a7c15ull;
static uint32_t next_u32(void) {
  rng ^= rng << 13, rng ^= rng >> 7, rng ^= rng << 17;
  return (uint32_t)(rng >> 16);
}
static double unit(void) { return (next_u32() & 0xffffff) / 16777216.0; }

static uint16_t to_bf16(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  return (uint16_t)((u + 0x7fff + ((u >> 16) & 1)) >> 16);
}

static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

static int failures = 0;
#define CHECK(c, ...)                 \
  do {                                \
    if (!(c)) {                       \
      fprintf(stderr, __VA_ARGS__);   \
      fprintf(stderr, "\n");          \
      ++failures;                     \
    }                                 \
  } while (0)

static void run_case(int batch, int hq, int hkv, int64_t sq, int64_t skv, int d, int dtype,
                     const int32_t *bq, const int32_t *bk, int bcast, int causal, int64_t off,
                     int uni, int paged, int page, double density) {
  ref_problem p;
  memset(&p, 0, sizeof p);
  p.batch = batch, p.hq = hq, p.hkv = hkv, p.sq = sq, p.skv = skv, p.d = d, p.dtype = dtype;
  p.bq = bq, p.bk = bk, p.mask_broadcast = bcast, p.causal = causal, p.causal_offset = off;
  p.gqa_union = uni, p.paged = paged;
  int64_t msize = 0;
  for (int h = 0; h < hq; ++h) msize += cdiv(sq, bq[h]) * cdiv(skv, bk[h]);
  const int64_t nm = (bcast ? 1 : batch) * msize;
  uint8_t *mask = malloc(nm > 0 ? nm : 1);
  for (int64_t i = 0; i < nm; ++i) mask[i] = unit() < density;
  int32_t *table = NULL;
  int64_t kv_rows = (int64_t)batch * hkv * skv;
  if (paged) {
    p.page_size = page, p.pages_per_seq = (int32_t)cdiv(skv, page);
    p.num_pages = batch * p.pages_per_seq + 2;
    table = malloc(sizeof(int32_t) * batch * p.pages_per_seq + 4);
    for (int i = 0; i < batch * p.pages_per_seq; ++i) table[i] = i;
    for (int i = batch * p.pages_per_seq - 1; i > 0; --i) {  /* shuffle */
      const int j = next_u32() % (i + 1), t = table[i];
      table[i] = table[j], table[j] = t;
    }
    kv_rows = (int64_t)p.num_pages * page * hkv;
  }
  const int64_t nq = (int64_t)batch * hq * sq;
  const size_t esz = dtype == 0 ? 2 : 4;
  void *q = malloc(esz * (nq * d + 1)), *k = malloc(esz * (kv_rows * d + 1)), *v = malloc(esz * (kv_rows * d + 1));
  void *dout = malloc(esz * (nq * d + 1));
  for (int64_t i = 0; i < nq * d; ++i) {
    const float a = (float)(2 * unit() - 1), b = (float)(2 * unit() - 1);
    if (dtype == 0) ((uint16_t *)q)[i] = to_bf16(a), ((uint16_t *)dout)[i] = to_bf16(b);
    else ((float *)q)[i] = a, ((float *)dout)[i] = b;
  }
  for (int64_t i = 0; i < kv_rows * d; ++i) {
    const float a = (float)(2 * unit() - 1), b = (float)(2 * unit() - 1);
    if (dtype == 0) ((uint16_t *)k)[i] = to_bf16(a), ((uint16_t *)v)[i] = to_bf16(b);
    else ((float *)k)[i] = a, ((float *)v)[i] = b;
  }
  double *o0 = malloc(sizeof(double) * (nq * d + 1)), *o1 = malloc(sizeof(double) * (nq * d + 1));
  double *l0 = malloc(sizeof(double) * (nq + 1)), *l1 = malloc(sizeof(double) * (nq + 1));
  CHECK(ref_forward(&p, mask, table, q, k, v, 0, NULL, nq, o0, l0, 1) == 0, "forward mode 0");
  CHECK(ref_forward(&p, mask, table, q, k, v, 1, NULL, nq, o1, l1, 1) == 0, "forward mode 1");
  CHECK(memcmp(o0, o1, sizeof(double) * nq * d) == 0 && memcmp(l0, l1, sizeof(double) * nq) == 0,
        "modes differ");
  /* a few rows by index */
  int64_t rows[6] = {0, 0, 0, batch - 1, hq - 1, sq > 0 ? sq - 1 : 0};
  if (sq > 0) CHECK(ref_forward(&p, mask, table, q, k, v, 1, rows, 2, o0, l0, 1) == 0, "rows");

  int64_t *feat = malloc(sizeof(int64_t) * 4 * (bcast ? 1 : batch) * hq);
  CHECK(ref_features(&p, mask, feat) == 0, "features");

  static const char *luts[] = {
      NULL,
      "bsa-lut 1\nrule * * * * 0 1000000 0 1000000 0 1000000 0 100000000 -> 256 64 lpt 3 1\n",
      "bsa-lut 2\nrule * * * * 0 1000000 0 1000000 0 1000000 0 100000000 0 10 -> 128 128 dealt 2 2\n"
      "rule * * * * 0 1000000 0 1000000 0 1000000 0 100000000 0 100000000 -> 128 64 local 0 0\n",
  };
  for (int t = 0; t < 3; ++t) {
    size_t n = 0;
    const int rc = ref_plan(&p, mask, table, luts[t], NULL, NULL, &n);
    CHECK(rc == 0 || rc == -3, "plan size rc %d", rc);
    if (rc == 0) {
      uint8_t *img = malloc(n);
      CHECK(ref_plan(&p, mask, table, luts[t], NULL, img, &n) == 0, "plan image");
      free(img);
    }
  }
  const int32_t forces[3][5] = {{128, 64, 0, 0, 1}, {256, 64, 1, 2, 2}, {128, 128, 2, 5, 0}};
  for (int f = 0; f < 3; ++f) {
    size_t n = 0;
    const int rc = ref_plan(&p, mask, table, NULL, forces[f], NULL, &n);
    CHECK(rc == 0 || rc == -3, "forced plan rc %d", rc);
    if (rc == 0) {
      uint8_t *img = malloc(n);
      CHECK(ref_plan(&p, mask, table, NULL, forces[f], img, &n) == 0, "forced plan image");
      size_t small = n / 2;
      CHECK(ref_plan(&p, mask, table, NULL, forces[f], img, &small) == -4, "capacity check");
      free(img);
    }
  }
  /* malformed tables: truncated at every character, then byte flips */
  const char *good = luts[2];
  const size_t gl = strlen(good);
  char *buf = malloc(gl + 1);
  for (size_t cut = 0; cut < gl; cut += 3) {
    memcpy(buf, good, cut);
    buf[cut] = 0;
    size_t n = 0;
    const int rc = ref_plan(&p, mask, table, buf, NULL, NULL, &n);
    CHECK(rc == 0 || rc == -2 || rc == -3, "truncated table rc %d", rc);
  }
  for (int it = 0; it < 200; ++it) {
    memcpy(buf, good, gl + 1);
    for (int f = 0; f < 3; ++f) buf[next_u32() % gl] = (char)(32 + next_u32() % 95);
    size_t n = 0;
    const int rc = ref_plan(&p, mask, table, buf, NULL, NULL, &n);
    CHECK(rc == 0 || rc == -2 || rc == -3, "mutated table rc %d", rc);
  }
  free(buf);

  if (!paged && dtype == 0) {
    double *dq = malloc(sizeof(double) * (nq * d + 1));
    const int64_t nk = (int64_t)batch * hkv * skv;
    double *dk = malloc(sizeof(double) * (nk * d + 1)), *dv = malloc(sizeof(double) * (nk * d + 1));
    CHECK(ref_backward(&p, mask, q, k, v, dout, NULL, nq, 0, skv, dq, dk, dv, 1) == 0, "backward");
    free(dq), free(dk), free(dv);
  }
  if (dtype == 0) {
    uint8_t *k8 = malloc(kv_rows * d + 1), *v8 = malloc(kv_rows * d + 1);
    for (int64_t i = 0; i < kv_rows * d; ++i) k8[i] = (uint8_t)next_u32(), v8[i] = (uint8_t)next_u32();
    for (int64_t i = 0; i < kv_rows * d; ++i) {  /* no NaN codes */
      if ((k8[i] & 0x7f) == 0x7f) k8[i] ^= 1;
      if ((v8[i] & 0x7f) == 0x7f) v8[i] ^= 1;
    }
    float *ks = malloc(sizeof(float) * hkv), *vs = malloc(sizeof(float) * hkv);
    for (int g = 0; g < hkv; ++g) ks[g] = 0.01f * (g + 1), vs[g] = 0.02f * (g + 1);
    CHECK(ref_forward_kv8(&p, mask, table, q, k8, v8, ks, vs, 1, NULL, nq, o1, l1, 1) == 0, "kv8");
    free(k8), free(v8), free(ks), free(vs);
  }
  if (!bcast) {
    uint8_t *sel = malloc(nm > 0 ? nm : 1);
    CHECK(ref_select(&p, table, q, k, 3, 0, sel) == 0, "select keep");
    CHECK(ref_select(&p, table, q, k, 1, 2, sel) == 0, "select top_k");
    free(sel);
  }
  for (int c = 0; c < 256; ++c) (void)ref_e4m3((uint8_t)c);
  free(mask), free(table), free(q), free(k), free(v), free(dout);
  free(o0), free(o1), free(l0), free(l1), free(feat);
}

int main(void) {
  const int32_t b64[4] = {64, 64, 64, 64}, b32[4] = {32, 32, 32, 32};
  const int32_t mixq[3] = {16, 32, 256}, mixk[3] = {64, 16, 512};
  const int32_t b128[8] = {128, 128, 128, 128, 128, 128, 128, 128};
  run_case(1, 2, 2, 256, 256, 64, 1, b64, b64, 0, 0, 0, 0, 0, 0, 0.5);       /* fp32 */
  run_case(2, 3, 3, 301, 333, 64, 0, mixq, mixk, 0, 0, 0, 0, 0, 0, 0.4);     /* ragged, mixed */
  run_case(2, 4, 2, 200, 260, 128, 0, b32, b64, 1, 1, 60, 0, 0, 0, 0.6);     /* causal, GQA */
  run_case(2, 8, 2, 200, 900, 128, 0, b128, b128, 0, 1, 700, 1, 1, 64, 0.1); /* union, paged */
  run_case(1, 4, 1, 5, 700, 64, 0, b64, b64, 0, 1, 695, 1, 1, 128, 0.2);     /* decode-like */
  run_case(1, 2, 2, 64, 0, 64, 0, b64, b64, 0, 0, 0, 0, 0, 0, 0.5);          /* no keys */
  run_case(1, 2, 2, 0, 64, 64, 0, b64, b64, 0, 0, 0, 0, 0, 0, 0.5);          /* no queries */
  if (failures) {
    fprintf(stderr, "%d failures\n", failures);
    return 1;
  }
  printf("oracle harness ok\n");
  return 0;
}
