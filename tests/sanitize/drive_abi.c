/* Drives libkvq's C ABI on the host, built with AddressSanitizer and
 * UndefinedBehaviorSanitizer against launch stand-ins that never touch the
 * device (tests/sanitize/kvq_launch_stubs.cpp): layouts of many
 * configurations, the fill-state machine through prefills, appends and lazy
 * flushes (uniform, ragged and paged KIVI, FP8, FP16), decode planning under
 * several workgroup targets, multi-layer and allocation-free decodes, and
 * the error paths. Device pointers are aligned placeholders. Exit status 0 =
 * every check held and no sanitizer report. */
#define _POSIX_C_SOURCE 200809L
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kvq.h"

extern long kvq_stub_launches[8];

static int failures = 0;
#define CHECK(c)                                                         \
  do {                                                                   \
    if (!(c)) {                                                          \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c); \
      ++failures;                                                        \
    }                                                                    \
  } while (0)

#define P(i) ((void*)(uintptr_t)(0x10000000u + 0x100000u * (i)))

static kvq_config cfg(int fmt, int bits, int G, int R, int B, int H, int C) {
  kvq_config c;
  memset(&c, 0, sizeof c);
  c.format = fmt;
  c.bits = bits;
  c.group_size = G;
  c.residual_length = R;
  c.batch = B;
  c.num_kv_heads = H;
  c.head_dim = 128;
  c.capacity = C;
  return c;
}

static void set_buffers(kvq_cache* c) {
  c->k_codes = P(1);
  c->v_codes = P(2);
  c->k_scale = (float*)P(3);
  c->k_zero = (float*)P(4);
  c->v_scale = (float*)P(5);
  c->v_zero = (float*)P(6);
  c->k_resid = P(7);
  c->v_resid = P(8);
  c->tensor_scale = (float*)P(9);
}

/* n_quant of a KIVI prefill of S tokens: G·max(0, min(⌊S/G⌋, ⌈(S−R)/G⌉)) */
static int64_t split_nq(int64_t S, int64_t G, int64_t R) {
  int64_t need = S > R ? (S - R + G - 1) / G : 0;
  if (need > S / G) need = S / G;
  return need * G;
}

static int decode_ok(const kvq_cache* c, int hq) {
  const size_t ws = kvq_decode_workspace_bytes(&c->cfg, hq);
  if (ws == 0) return 0;
  const kvq_status st = kvq_decode_attention(c, (const float*)P(20), hq, (float*)P(21), P(22),
                                             ws, NULL);
  if (st != KVQ_OK) fprintf(stderr, "decode status %d (%s)\n", st, kvq_status_str(st));
  return st == KVQ_OK && kvq_decode_bytes(c, hq) >= 0;
}

static void uniform_kivi(int bits, int G, int R, int B, int H, int hq, int S, int steps) {
  const int C = S + steps;
  kvq_config k = cfg(KVQ_FMT_KIVI, bits, G, R, B, H, C);
  kvq_cache c;
  CHECK(kvq_cache_init(&c, &k) == KVQ_OK);
  set_buffers(&c);
  CHECK(kvq_prefill_quantize(&c, P(30), P(31), S, NULL) == KVQ_OK);
  int64_t nq = split_nq(S, G, R), nr = S - nq;
  const int64_t rcap = R > 0 ? R : G;
  CHECK(c.n_quant == nq && c.n_resid == nr);
  CHECK(decode_ok(&c, hq));
  const size_t ws = kvq_decode_workspace_bytes(&c.cfg, hq);
  /* the fused step with a short workspace is refused before it appends */
  CHECK(kvq_append_decode(&c, P(32), P(33), (const float*)P(20), hq, (float*)P(21), P(22), 64,
                          NULL) == KVQ_ERR_WORKSPACE);
  CHECK(c.n_quant == nq && c.n_resid == nr);
  for (int i = 0; i < steps; ++i) {
    /* odd steps: append and decode in one call */
    if (i % 2)
      CHECK(kvq_append_decode(&c, P(32), P(33), (const float*)P(20), hq, (float*)P(21), P(22), ws,
                              NULL) == KVQ_OK);
    else
      CHECK(kvq_append_token(&c, P(32), P(33), NULL) == KVQ_OK);
    if (nr == rcap) {
      nq += rcap;
      nr = 0;
    }
    ++nr;
    CHECK(c.n_quant == nq && c.n_resid == nr);
    if (i % 17 == 0 || i == steps - 1) CHECK(decode_ok(&c, hq));
  }
  /* full: one more append is refused and changes nothing */
  CHECK(kvq_append_token(&c, P(32), P(33), NULL) == KVQ_ERR_CAPACITY);
  CHECK(kvq_append_decode(&c, P(32), P(33), (const float*)P(20), hq, (float*)P(21), P(22), ws,
                          NULL) == KVQ_ERR_CAPACITY);
  CHECK(c.n_quant == nq && c.n_resid == nr);
  /* the allocation-free decode plans the same call */
  CHECK(kvq_decode_attention_static(&c, (const float*)P(20), hq, (float*)P(21), NULL) == KVQ_OK);
  /* a corrupted fill state is refused */
  c.n_quant += 1;
  CHECK(kvq_decode_attention(&c, (const float*)P(20), hq, (float*)P(21), P(22), 1u << 30, NULL) ==
        KVQ_ERR_STATE);
}

static void ragged_kivi(int paged, int B, int H, int hq, int steps) {
  const int G = 32, R = 128, Pt = 64;
  int64_t lens[KVQ_MAX_RAGGED_BATCH];
  int64_t maxlen = 0;
  for (int b = 0; b < B; ++b) {
    lens[b] = 1 + (b * 977) % 3000;
    if (lens[b] > maxlen) maxlen = lens[b];
  }
  const int C = (int)maxlen + steps;
  kvq_config k = cfg(KVQ_FMT_KIVI, 2, G, R, B, H, C);
  if (paged) {
    k.page_tokens = Pt;
    k.num_pages = B * ((C + Pt - 1) / Pt);
  }
  kvq_layout lay;
  CHECK(kvq_layout_query(&k, &lay) == KVQ_OK);
  kvq_cache c;
  CHECK(kvq_cache_init(&c, &k) == KVQ_OK);
  set_buffers(&c);
  int64_t* nq = calloc(B, sizeof(int64_t));
  int32_t* nr = calloc(B, sizeof(int32_t));
  c.seq_n_quant = nq;
  c.seq_n_resid = nr;
  if (paged) {
    /* a paged cache needs its table before anything runs */
    CHECK(kvq_prefill_quantize_ragged(&c, P(30), P(31), maxlen, lens, NULL) == KVQ_ERR_INVALID_ARG);
    c.block_table = (const int32_t*)P(40);
  }
  CHECK(kvq_prefill_quantize_ragged(&c, P(30), P(31), maxlen, lens, NULL) == KVQ_OK);
  for (int b = 0; b < B; ++b) {
    CHECK(nq[b] == split_nq(lens[b], G, R) && nr[b] == lens[b] - nq[b]);
  }
  CHECK(decode_ok(&c, hq));
  for (int i = 0; i < steps; ++i) {
    int64_t want_q[KVQ_MAX_RAGGED_BATCH];
    int32_t want_r[KVQ_MAX_RAGGED_BATCH];
    for (int b = 0; b < B; ++b) {
      want_q[b] = nq[b] + (nr[b] == R ? R : 0);
      want_r[b] = (nr[b] == R ? 0 : nr[b]) + 1;
    }
    if (i % 3 == 1)
      CHECK(kvq_append_decode(&c, P(32), P(33), (const float*)P(20), hq, (float*)P(21), P(22),
                              kvq_decode_workspace_bytes(&c.cfg, hq), NULL) == KVQ_OK);
    else
      CHECK(kvq_append_token(&c, P(32), P(33), NULL) == KVQ_OK);
    for (int b = 0; b < B; ++b) CHECK(nq[b] == want_q[b] && nr[b] == want_r[b]);
    if (i % 29 == 0) CHECK(decode_ok(&c, hq));
  }
  /* the contiguous prefill is not for ragged caches */
  CHECK(kvq_prefill_quantize(&c, P(30), P(31), 10, NULL) == KVQ_ERR_INVALID_ARG);
  CHECK(kvq_cache_reset(&c) == KVQ_OK);
  for (int b = 0; b < B; ++b) CHECK(nq[b] == 0 && nr[b] == 0);
  free(nq);
  free(nr);
}

static void dense(int fmt, int B, int H, int hq, int S, int steps, int per_head, int qf8) {
  kvq_config k = cfg(fmt, fmt == KVQ_FMT_FP16 ? 16 : 8, 0, 0, B, H, S + steps);
  k.scale_per_head = per_head;
  k.fp8_attention = qf8;
  kvq_cache c;
  CHECK(kvq_cache_init(&c, &k) == KVQ_OK);
  set_buffers(&c);
  if (fmt != KVQ_FMT_FP16) CHECK(kvq_append_token(&c, P(32), P(33), NULL) == KVQ_ERR_STATE);
  CHECK(kvq_prefill_quantize(&c, P(30), P(31), S, NULL) == KVQ_OK);
  CHECK(c.n_quant == S && c.n_resid == 0);
  for (int i = 0; i < steps; ++i) {
    if (i % 2)
      CHECK(kvq_append_decode(&c, P(32), P(33), (const float*)P(20), hq, (float*)P(21), P(22),
                              kvq_decode_workspace_bytes(&c.cfg, hq), NULL) == KVQ_OK);
    else
      CHECK(kvq_append_token(&c, P(32), P(33), NULL) == KVQ_OK);
    CHECK(c.n_quant == S + i + 1);
    if (i % 7 == 0) CHECK(decode_ok(&c, hq));
  }
  CHECK(kvq_append_token(&c, P(32), P(33), NULL) == KVQ_ERR_CAPACITY);
}

static void layers(void) {
  kvq_cache cs[3];
  kvq_config a = cfg(KVQ_FMT_KIVI, 2, 32, 128, 2, 4, 900);
  kvq_config b = cfg(KVQ_FMT_FP16, 16, 0, 0, 2, 8, 300);
  kvq_config d = cfg(KVQ_FMT_FP8_E4M3, 8, 0, 0, 2, 2, 500);
  const kvq_config* all[3] = {&a, &b, &d};
  const int S[3] = {800, 300, 17};
  const kvq_cache* ptrs[3];
  size_t ws = 0;
  for (int l = 0; l < 3; ++l) {
    CHECK(kvq_cache_init(&cs[l], all[l]) == KVQ_OK);
    set_buffers(&cs[l]);
    CHECK(kvq_prefill_quantize(&cs[l], P(30), P(31), S[l], NULL) == KVQ_OK);
    ptrs[l] = &cs[l];
    const size_t w = kvq_decode_workspace_bytes(all[l], 16);
    if (w > ws) ws = w;
  }
  CHECK(kvq_decode_attention_layers(ptrs, 3, (const float*)P(20), 16, (float*)P(21), P(22), ws,
                                    NULL) == KVQ_OK);
  CHECK(kvq_decode_attention_layers(ptrs, 3, (const float*)P(20), 16, (float*)P(21), P(22), 16,
                                    NULL) == KVQ_ERR_WORKSPACE);
  ptrs[1] = NULL;
  CHECK(kvq_decode_attention_layers(ptrs, 3, (const float*)P(20), 16, (float*)P(21), P(22), ws,
                                    NULL) == KVQ_ERR_INVALID_ARG);
}

static void layouts(void) {
  const int fmts[4] = {KVQ_FMT_KIVI, KVQ_FMT_FP8_E4M3, KVQ_FMT_FP8_E5M2, KVQ_FMT_FP16};
  for (int f = 0; f < 4; ++f)
    for (int G = 32; G <= 128; G *= 2)
      for (int R = 0; R <= 256; R += 64)
        for (int bits = 2; bits <= 16; bits *= 2)
          for (int C = 1; C < 5000; C = C * 3 + 7) {
            kvq_config k = cfg(fmts[f], bits, G, R, 3, 5, C);
            kvq_layout lay;
            const kvq_status st = kvq_layout_query(&k, &lay);
            CHECK(st == KVQ_OK || st == KVQ_ERR_UNSUPPORTED);
            if (st == KVQ_OK) CHECK(lay.k_codes > 0 && lay.v_codes > 0);
            (void)kvq_decode_workspace_bytes(&k, 10);
            (void)kvq_decode_workspace_bytes(&k, 15);
          }
  CHECK(kvq_layout_query(NULL, NULL) == KVQ_ERR_INVALID_ARG);
  CHECK(kvq_cache_init(NULL, NULL) == KVQ_ERR_INVALID_ARG);
  CHECK(kvq_decode_bytes(NULL, 8) == -1);
  CHECK(kvq_theoretical_bytes_layers(0, 1, NULL, NULL, NULL, 2.0) == -1.0);
  for (int s = -1; s < 9; ++s) CHECK(kvq_status_str((kvq_status)s) != NULL);
}

int main(void) {
  static const char* targets[4] = {NULL, "64", "1000", "4096"};
  layouts();
  for (int t = 0; t < 4; ++t) {
    if (targets[t]) setenv("KVQ_DECODE_TARGET_WORKGROUPS", targets[t], 1);
    else unsetenv("KVQ_DECODE_TARGET_WORKGROUPS");
    uniform_kivi(2, 32, 128, 2, 4, 32, 1000, 300);
    uniform_kivi(4, 64, 64, 3, 2, 6, 333, 140);
    uniform_kivi(2, 128, 0, 1, 1, 1, 5, 260);
    uniform_kivi(2, 32, 128, 16, 8, 64, 4096, 40);    /* GQA 8, 128 (b, h) blocks */
    uniform_kivi(4, 32, 128, 64, 32, 32, 300, 10);    /* more blocks than units */
    ragged_kivi(0, 7, 2, 16, 140);
    ragged_kivi(1, 5, 3, 12, 140);
    ragged_kivi(1, KVQ_MAX_RAGGED_BATCH, 1, 8, 3);
    dense(KVQ_FMT_FP8_E4M3, 2, 4, 8, 100, 40, 0, 0);
    dense(KVQ_FMT_FP8_E5M2, 3, 2, 4, 33, 20, 1, 1);
    dense(KVQ_FMT_FP16, 2, 2, 8, 64, 30, 0, 0);
    layers();
  }
  CHECK(kvq_stub_launches[0] > 0 && kvq_stub_launches[1] > 0 && kvq_stub_launches[6] > 0);
  fprintf(stderr, "launches: quantize %ld copy %ld vtiles %ld fp8 %ld/%ld decode %ld\n",
          kvq_stub_launches[0], kvq_stub_launches[1], kvq_stub_launches[2], kvq_stub_launches[3],
          kvq_stub_launches[4], kvq_stub_launches[6]);
  if (failures) fprintf(stderr, "%d check(s) failed\n", failures);
  return failures ? 1 : 0;
}
