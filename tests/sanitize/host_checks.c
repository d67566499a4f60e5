/*
 * Host-side checks under AddressSanitizer and UndefinedBehaviorSanitizer:
 * every argument-validation path of the C ABI that returns before a launch
 * (the launchers are linked as stubs that abort), and the oracle's functions
 * on small inputs with exactly sized buffers.  Exit status 0 when every
 * check holds; the sanitizers abort the run on the first report.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kvq.h"
#include "oracle.c"

static int fails = 0;
#define CHECK(cond)                                                          \
  do {                                                                       \
    if (!(cond)) {                                                           \
      fprintf(stderr, "FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond);        \
      ++fails;                                                               \
    }                                                                        \
  } while (0)

/* non-null, 16-byte aligned stand-ins for device pointers: never dereferenced */
#define DEV(n) ((void*)(uintptr_t)(4096u * (n)))

static void desc(kvq_cache* c, int mode, int bits, int group) {
  memset(c, 0, sizeof *c);
  c->batch = 2;
  c->kv_heads = 3;
  c->max_seq = 256;
  c->head_dim = 128;
  c->mode = mode;
  c->chunk_tokens = 32;
  const float thr[4] = {-1.5f, -0.5f, 0.5f, 1.5f};
  kvq_tensor* ts[2] = {&c->k, &c->v};
  for (int i = 0; i < 2; ++i) {
    ts[i]->bits = bits;
    ts[i]->group = group;
    memcpy(ts[i]->thr, thr, sizeof thr);
  }
}

static void api_checks(void) {
  kvq_cache c;
  kvq_cache_bytes_t b;
  size_t n = 0;
  /* sizes of every mode */
  desc(&c, KVQ_MODE_UNIFORM, 4, 64);
  CHECK(kvq_cache_bytes(&c, &b) == KVQ_OK && b.k.codes == 2u * 3 * 256 * 64);
  c.k.axis = KVQ_AXIS_CHANNEL;
  CHECK(kvq_cache_bytes(&c, &b) == KVQ_OK && b.k.codes16 == 2u * 3 * 64 * 128 * 2);
  c.page_tokens = 64;
  c.num_pages = 9;
  CHECK(kvq_cache_bytes(&c, &b) == KVQ_OK && b.k.scale == 9u * 3 * 1 * 128 * 4);
  desc(&c, KVQ_MODE_UNIFORM, 8, 128);
  c.k.format = c.v.format = KVQ_FMT_E4M3;
  CHECK(kvq_cache_bytes(&c, &b) == KVQ_OK && b.k.zero == 0);
  c.k.format = c.v.format = KVQ_FMT_E5M2;
  CHECK(kvq_cache_bytes(&c, &b) == KVQ_OK);
  desc(&c, KVQ_MODE_OAKEN, 4, 64);
  c.k.sparse_cap = c.v.sparse_cap = 1004;
  CHECK(kvq_cache_bytes(&c, &b) == KVQ_OK && b.k.sparse == 2u * 3 * 1004 * 2);
  c.k.sparse_cap = 1002;
  CHECK(kvq_cache_bytes(&c, &b) == KVQ_ERR_ALIGNMENT);
  desc(&c, KVQ_MODE_CHUNK_MIXED, 4, 32);
  CHECK(kvq_cache_bytes(&c, &b) == KVQ_OK && b.perm == 2u * 8 * 4);
  desc(&c, KVQ_MODE_DSQ, 4, 32);
  c.dsq_sig = 13;
  CHECK(kvq_cache_bytes(&c, &b) == KVQ_OK && b.dsq_mask == 2u * 3 * 4 * 8);
  /* refused configurations */
  desc(&c, KVQ_MODE_UNIFORM, 4, 64);
  c.head_dim = 64;
  CHECK(kvq_cache_bytes(&c, &b) == KVQ_ERR_UNSUPPORTED);
  desc(&c, KVQ_MODE_UNIFORM, 4, 64);
  c.max_seq = 100;
  CHECK(kvq_cache_bytes(&c, &b) == KVQ_ERR_INVALID_ARG);
  CHECK(kvq_cache_bytes(NULL, &b) == KVQ_ERR_INVALID_ARG);
  CHECK(kvq_cache_bytes(&c, NULL) == KVQ_ERR_INVALID_ARG);
  /* entry points that refuse before any launch (no buffers attached) */
  desc(&c, KVQ_MODE_UNIFORM, 4, 64);
  CHECK(kvq_quant_append(&c, DEV(1), DEV(2), 0, DEV(3), NULL) == KVQ_OK); /* nothing to do */
  CHECK(kvq_quant_append(&c, DEV(1), DEV(2), -1, DEV(3), NULL) == KVQ_ERR_INVALID_ARG);
  CHECK(kvq_quant_append(&c, DEV(1), DEV(2), 257, DEV(3), NULL) == KVQ_ERR_CAPACITY);
  CHECK(kvq_quant_append(&c, DEV(1), DEV(2), 1, DEV(3), NULL) == KVQ_ERR_INVALID_ARG);
  CHECK(kvq_quant_append(&c, (void*)((char*)DEV(1) + 2), DEV(2), 1, DEV(3), NULL) == KVQ_ERR_ALIGNMENT);
  CHECK(kvq_reorder_chunks(&c, DEV(1), 8, NULL) == KVQ_ERR_INVALID_ARG);
  CHECK(kvq_dsq_append(&c, DEV(1), DEV(2), DEV(3), 64, DEV(4), NULL) == KVQ_ERR_INVALID_ARG);
  CHECK(kvq_decode_workspace_bytes(&c, 6, 256, 4, &n) == KVQ_OK && n > 0);
  CHECK(kvq_decode_workspace_bytes(&c, 5, 256, 4, &n) == KVQ_ERR_INVALID_ARG);
  CHECK(kvq_decode_attn(&c, DEV(1), 6, DEV(2), 256, 0.1f, DEV(3), NULL, 0, 0, NULL) == KVQ_ERR_INVALID_ARG);
  CHECK(kvq_decode_attn(&c, DEV(1), 6, DEV(2), 257, 0.1f, DEV(3), NULL, 0, 0, NULL) == KVQ_ERR_CAPACITY);
  CHECK(kvq_decode_attn(&c, DEV(1), 6, DEV(2), 256, NAN, DEV(3), NULL, 0, 0, NULL) == KVQ_ERR_INVALID_ARG);
  CHECK(kvq_decode_attn(&c, (void*)((char*)DEV(1) + 8), 6, DEV(2), 256, 0.1f, DEV(3), NULL, 0, 0, NULL) ==
        KVQ_ERR_ALIGNMENT);
  CHECK(kvq_decode_workspace_bytes(&c, 6, 256, 4, &n) == KVQ_OK);
  CHECK(kvq_decode_attn(&c, DEV(1), 6, DEV(2), 256, 0.1f, DEV(3), DEV(4), n - 1, 4, NULL) == KVQ_ERR_WORKSPACE);
  /* the no-alloc entry point: a plan beyond its fixed array, then one within it (no buffers) */
  desc(&c, KVQ_MODE_UNIFORM, 4, 64);
  c.batch = 16;
  c.kv_heads = 32;
  c.max_seq = 65536;
  CHECK(kvq_decode_workspace_bytes(&c, 32, 65536, 1024, &n) == KVQ_OK && n > KVQ_STATIC_SCRATCH_BYTES);
  CHECK(kvq_decode_attn_noalloc(&c, DEV(1), 32, DEV(2), 65536, 0.1f, DEV(3), 1024, NULL) == KVQ_ERR_WORKSPACE);
  CHECK(kvq_decode_attn_noalloc(&c, DEV(1), 32, DEV(2), 65536, 0.1f, DEV(3), 4, NULL) == KVQ_ERR_INVALID_ARG);
  /* preparation entry points */
  CHECK(kvq_chunk_bits(DEV(1), DEV(2), 0, 8, 16, 0.6, 0.1, NULL, DEV(3), NULL) == KVQ_OK);
  CHECK(kvq_chunk_bits(DEV(1), DEV(2), 2, 8, 16, 2.0, 0.1, NULL, DEV(3), NULL) == KVQ_ERR_INVALID_ARG);
  CHECK(kvq_chunk_bits((const double*)((char*)DEV(1) + 4), DEV(2), 2, 8, 16, 0.6, 0.1, NULL, DEV(3), NULL) ==
        KVQ_ERR_ALIGNMENT);
  CHECK(kvq_hist_f16(NULL, 16, DEV(1), NULL) == KVQ_ERR_INVALID_ARG);
  const int32_t p_bp[9] = {250, 1500, 8500, 9750, 1, 2, 3, 4, 5};
  CHECK(kvq_hist_percentiles(DEV(1), 9, p_bp, DEV(2), NULL) == KVQ_ERR_INVALID_ARG);
  for (int s = -8; s <= 1; ++s) CHECK(kvq_status_string(s) != NULL);
}

/* fp16 bits of moderate values: exponent field 10..20 (|x| in [2^-5, 2^6)), either sign */
static void fill_f16(uint16_t* x, long n, uint32_t seed) {
  uint32_t s = seed;
  for (long i = 0; i < n; ++i) {
    s = s * 1664525u + 1013904223u;
    const uint16_t e = (uint16_t)(10 + (s >> 8) % 11);
    x[i] = (uint16_t)(((s >> 31) << 15) | (e << 10) | ((s >> 12) & 0x3FF));
  }
}

static void oracle_checks(void) {
  enum { R = 8, D = 128 };
  uint16_t x[R * D];
  fill_f16(x, R * D, 1);
  float out[R * D];
  /* asymmetric INT4, groups of 64: the half-step bound */
  {
    uint8_t codes[R * D], zero[R * 2];
    float scale[R * 2];
    ora_quant_rows(x, R, D, 64, 4, 0, codes, scale, zero);
    ora_dequant_rows(codes, scale, zero, R, D, 64, 0, out);
    for (int i = 0; i < R * D; ++i) {
      CHECK(codes[i] <= 15);
      CHECK(fabsf(out[i] - ora_f16_to_f32(x[i])) <= 0.5f * scale[i / 64] * 1.0001f + 1e-6f);
    }
  }
  /* symmetric INT8 per row */
  {
    uint8_t codes[R * D], zero[R];
    float scale[R];
    ora_quant_rows(x, R, D, 128, 8, 1, codes, scale, zero);
    ora_dequant_rows(codes, scale, zero, R, D, 128, 1, out);
    for (int i = 0; i < R * D; ++i) CHECK(fabsf(out[i] - ora_f16_to_f32(x[i])) <= 0.5f * scale[i / 128] * 1.0001f);
  }
  /* FP8 both formats */
  {
    uint8_t codes[R * D];
    float scale[R];
    ora_quant_rows_e4m3(x, R, D, 128, codes, scale);
    ora_dequant_rows_e4m3(codes, scale, R, D, 128, out);
    ora_quant_rows_e5m2(x, R, D, 128, codes, scale);
    ora_dequant_rows_e5m2(codes, scale, R, D, 128, out);
    for (int i = 0; i < R * D; ++i) CHECK(isfinite(out[i]));
  }
  /* K per channel over 64-token blocks: one slice of 128 tokens */
  {
    static uint16_t xt[128 * D];
    static uint8_t codes[128 * D];
    static float scale[2 * D], outc[128 * D];
    static uint8_t zero[2 * D];
    fill_f16(xt, 128 * D, 2);
    ora_quant_channel_blocks(xt, 1, 128, D, 64, 4, codes, scale, zero);
    ora_dequant_channel_blocks(codes, scale, zero, 1, 128, D, 64, outc);
    for (int t = 0; t < 128; ++t)
      for (int d = 0; d < D; ++d)
        CHECK(fabsf(outc[t * D + d] - ora_f16_to_f32(xt[t * D + d])) <= 0.5f * scale[(t / 64) * D + d] * 1.0001f);
  }
  /* Oaken rows */
  {
    const float thr[4] = {-8.0f, -1.0f, 1.0f, 8.0f};
    uint8_t codes[R * D], zero[R * 2];
    float scale[R * 2], oscale[R * 2];
    uint16_t entries[R * D];
    int counts[R];
    ora_oaken_rows(x, R, D, 64, thr, codes, scale, zero, oscale, entries, counts);
    ora_oaken_dequant_rows(codes, scale, zero, oscale, entries, counts, R, D, 64, thr, out);
    for (int r = 0; r < R; ++r) CHECK(counts[r] >= 0 && counts[r] <= D);
    for (int i = 0; i < R * D; ++i) CHECK(isfinite(out[i]));
  }
  /* calibration histogram and a percentile */
  {
    static uint64_t hist[65536];
    ora_hist_f16(x, R * D, hist);
    const float p = ora_hist_percentile(hist, 5000);
    CHECK(isfinite(p));
  }
  /* Cocktail chunk search and reorder */
  {
    double qe[16], ce[8 * 16], sims[8];
    uint8_t bits[2 * 8];
    for (int i = 0; i < 16; ++i) qe[i] = sin(0.7 * i + 0.1);
    for (int i = 0; i < 8 * 16; ++i) ce[i] = cos(0.3 * i);
    ora_chunk_bits(qe, ce, 8, 16, 0.6, 0.1, sims, bits);
    memcpy(bits + 8, bits, 8);
    int32_t perm[2 * 8], seg[2 * 4];
    ora_reorder(bits, 2, 8, perm, seg);
    for (int b = 0; b < 2; ++b) CHECK(seg[b * 4 + 0] + seg[b * 4 + 1] + seg[b * 4 + 2] == seg[b * 4 + 3]);
  }
  /* attention and the log-sum-exp merge */
  {
    uint16_t q[2 * D];
    float kh[8 * D], vh[8 * D];
    double o[2 * D], m[2] = {0.5, 1.5}, l[2] = {2.0, 3.0}, po[2 * D], mo[D];
    fill_f16(q, 2 * D, 3);
    for (int i = 0; i < 8 * D; ++i) {
      kh[i] = 0.01f * (float)(i % 13);
      vh[i] = 0.02f * (float)(i % 7);
    }
    ora_attention(q, 2, 1, D, kh, vh, 8, 1.0 / sqrt(128.0), o);
    for (int i = 0; i < 2 * D; ++i) po[i] = o[i];
    ora_lse_merge(2, m, l, po, D, mo);
    for (int i = 0; i < D; ++i) CHECK(isfinite(mo[i]));
  }
  /* DSQ: one group of 64 tokens, 13 significant, INT2 groups of 32 */
  {
    enum { T = 64, NS = 13, NO = 64 - 13, G2 = 32 };
    static uint16_t k[T * D], v[T * D];
    static float score[T], kscale[D], vscale[D], base[D], ks2[NO * 4], vs2[NO * 4], kh[T * D], vh[T * D];
    static int8_t ksig[NS * D], vsig[NS * D];
    static uint8_t kc2[NO * D], vc2[NO * D], kz2[NO * 4], vz2[NO * 4];
    uint64_t mask = 0;
    fill_f16(k, T * D, 4);
    fill_f16(v, T * D, 5);
    for (int t = 0; t < T; ++t) score[t] = (float)((t * 37) % 64);
    ora_dsq_group(k, v, score, T, D, NS, G2, &mask, ksig, kscale, vsig, vscale, base, kc2, ks2, kz2, vc2, vs2,
                  vz2);
    int pop = 0;
    for (int t = 0; t < 64; ++t) pop += (int)((mask >> t) & 1u);
    CHECK(pop == NS);
    ora_dsq_dequant_group(mask, T, D, G2, ksig, kscale, vsig, vscale, base, kc2, ks2, kz2, vc2, vs2, vz2, kh, vh);
    for (int i = 0; i < T * D; ++i) CHECK(isfinite(kh[i]) && isfinite(vh[i]));
  }
}

int main(void) {
  api_checks();
  oracle_checks();
  if (fails) {
    fprintf(stderr, "%d checks failed\n", fails);
    return 1;
  }
  printf("host checks passed\n");
  return 0;
}
