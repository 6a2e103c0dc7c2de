// Host-side checks of the C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code (no GPU is used or needed):
// the host Lloyd-Max solver over a range of dimensions and bit widths, and
// every entry point's synchronous argument checks with invalid arguments
// (each must return its status before anything is launched).
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "tq.h"

static int g_fail = 0;

#define EXPECT(cond, what)                                              \
  do {                                                                  \
    if (!(cond)) {                                                      \
      fprintf(stderr, "FAIL %s:%d: %s\n", __FILE__, __LINE__, what);    \
      ++g_fail;                                                         \
    }                                                                   \
  } while (0)

static void codebooks() {
  // Every width the kernels take (0..4) over a spread of dimensions, and
  // 5 bits at the kernels' d = 128 (larger widths only take longer).
  const int dims[] = {3, 4, 16, 32, 96, 128, 200, 1536, 65536};
  for (int d : dims) {
    for (int b = 0; b <= (d == 128 ? 5 : 4); ++b) {
      const int K = 1 << b;
      std::vector<double> c(K + 2, NAN), t(K + 2, NAN);
      double mse = -1.0;
      const int st = tq_codebook(d, b, c.data() + 1, t.data() + 1, &mse);
      if (st == TQ_ERR_NO_CONVERGE) continue;
      EXPECT(st == TQ_OK, "tq_codebook status");
      EXPECT(isnan(c[0]) && isnan(c[K + 1]) && isnan(t[0]) && isnan(t[K]), "tq_codebook wrote outside");
      for (int i = 0; i + 1 < K; ++i) EXPECT(c[1 + i] < c[2 + i], "centroids ascending");
      for (int i = 0; i < K; ++i) EXPECT(c[1 + i] == -c[K - i], "centroids antisymmetric");
      EXPECT(mse >= 0.0 && mse <= 1.0 + 1e-12, "distortion in [0, 1]");
    }
  }
  double c[4], t[4];
  EXPECT(tq_codebook(128, 3, nullptr, t, nullptr) == TQ_ERR_INVALID_ARG, "null centroids");
  EXPECT(tq_codebook(1, 1, c, t, nullptr) == TQ_ERR_INVALID_ARG, "d < 2");
  EXPECT(tq_codebook(128, 9, c, t, nullptr) == TQ_ERR_UNSUPPORTED, "bits > 8");
  EXPECT(tq_codebook(65537, 1, c, t, nullptr) == TQ_ERR_UNSUPPORTED, "d > 65536");
  EXPECT(tq_codebook(128, 2, c, nullptr, nullptr) == TQ_ERR_INVALID_ARG, "null boundaries");
  for (int s = 1; s >= -6; --s) EXPECT(tq_status_string(s) != nullptr && strlen(tq_status_string(s)) > 0, "status text");
}

// Fake, aligned device addresses: the argument checks never dereference them.
static void* fake(size_t off = 0) { return reinterpret_cast<void*>(uintptr_t(1) << 20 | off); }

static tq_quantizer quant(int d, int bits, int variant) {
  tq_quantizer q;
  memset(&q, 0, sizeof q);
  q.d = d;
  q.bits = bits;
  q.variant = variant;
  q.rot = static_cast<const float*>(fake());
  q.proj = variant == TQ_PROD ? static_cast<const float*>(fake()) : nullptr;
  q.centroids = static_cast<const float*>(fake());
  q.boundaries = static_cast<const float*>(fake());
  q.prep = fake();
  return q;
}

static void argument_checks() {
  tq_quantizer q = quant(128, 3, TQ_MSE), q64 = quant(64, 3, TQ_MSE), q5 = quant(128, 5, TQ_MSE);
  tq_quantizer prod = quant(128, 3, TQ_PROD);
  tq_packed pk = {static_cast<uint8_t*>(fake()), static_cast<float*>(fake()), nullptr, nullptr};
  const void* x = fake();
  // encode
  EXPECT(tq_encode(nullptr, x, TQ_BF16, 10, 128, &pk, nullptr, nullptr) == TQ_ERR_INVALID_ARG, "encode null q");
  EXPECT(tq_encode(&q64, x, TQ_BF16, 10, 128, &pk, nullptr, nullptr) == TQ_ERR_UNSUPPORTED, "encode d");
  EXPECT(tq_encode(&q5, x, TQ_BF16, 10, 128, &pk, nullptr, nullptr) == TQ_ERR_UNSUPPORTED, "encode bits");
  EXPECT(tq_encode(&q, x, 7, 10, 128, &pk, nullptr, nullptr) == TQ_ERR_UNSUPPORTED, "encode dtype");
  EXPECT(tq_encode(&q, x, TQ_BF16, -1, 128, &pk, nullptr, nullptr) == TQ_ERR_INVALID_ARG, "encode n");
  EXPECT(tq_encode(&q, x, TQ_BF16, 10, 100, &pk, nullptr, nullptr) == TQ_ERR_INVALID_ARG, "encode stride");
  EXPECT(tq_encode(&q, nullptr, TQ_BF16, 10, 128, &pk, nullptr, nullptr) == TQ_ERR_INVALID_ARG, "encode x");
  EXPECT(tq_encode(&q, fake(4), TQ_BF16, 10, 128, &pk, nullptr, nullptr) == TQ_ERR_INVALID_ARG, "encode align");
  EXPECT(tq_encode(&q, x, TQ_BF16, 0, 128, &pk, nullptr, nullptr) == TQ_OK, "encode n = 0");
  EXPECT(tq_encode(&prod, x, TQ_BF16, 10, 128, &pk, nullptr, nullptr) == TQ_ERR_INVALID_ARG, "encode sketch arrays");
  tq_quantizer bad_prep = q;
  bad_prep.prep = fake(16);
  EXPECT(tq_prepare(&bad_prep, nullptr) == TQ_ERR_WORKSPACE, "prepare alignment");
  EXPECT(tq_prepare(nullptr, nullptr) == TQ_ERR_INVALID_ARG, "prepare null");
  // decode
  const size_t ws = tq_attn_decode_workspace(1, 32, 8, 1000);
  EXPECT(ws > 0, "workspace size");
  EXPECT(tq_attn_decode_workspace(1, 30, 8, 1000) == 0, "workspace of a bad shape");
  const float* qv = static_cast<const float*>(fake());
  float* out = static_cast<float*>(fake());
  EXPECT(tq_attn_decode(&q, &q, qv, 1, 30, 8, nullptr, 1000, &pk, &pk, 0.1f, out, fake(), ws, nullptr) ==
             TQ_ERR_INVALID_ARG, "decode Hq % Hkv");
  EXPECT(tq_attn_decode(&q, &q, qv, 0, 32, 8, nullptr, 1000, &pk, &pk, 0.1f, out, fake(), ws, nullptr) ==
             TQ_ERR_INVALID_ARG, "decode B");
  EXPECT(tq_attn_decode(&q, &q, qv, 1, 32, 8, nullptr, 0, &pk, &pk, 0.1f, out, fake(), ws, nullptr) ==
             TQ_ERR_INVALID_ARG, "decode max_ctx");
  EXPECT(tq_attn_decode(&q, &q, nullptr, 1, 32, 8, nullptr, 1000, &pk, &pk, 0.1f, out, fake(), ws, nullptr) ==
             TQ_ERR_INVALID_ARG, "decode query");
  EXPECT(tq_attn_decode(&q, &q, qv, 1, 32, 8, nullptr, 1000, &pk, &pk, 0.1f, out, fake(), ws - 1, nullptr) ==
             TQ_ERR_WORKSPACE, "decode workspace size");
  EXPECT(tq_attn_decode(&q, &q, qv, 1, 32, 8, nullptr, 1000, &pk, &pk, 0.1f, out, fake(128), ws, nullptr) ==
             TQ_ERR_WORKSPACE, "decode workspace alignment");
  EXPECT(tq_attn_decode(&q, &prod, qv, 1, 32, 8, nullptr, 1000, &pk, &pk, 0.1f, out, fake(), ws, nullptr) ==
             TQ_ERR_UNSUPPORTED, "decode prod values");
  EXPECT(tq_attn_decode(&prod, &q, qv, 1, 32, 8, nullptr, 1000, &pk, &pk, 0.1f, out, fake(), ws, nullptr) ==
             TQ_ERR_INVALID_ARG, "decode sketch arrays");
  for (int ph : {0, 4})
    EXPECT(tq_attn_decode_phase(ph, &q, &q, qv, 1, 32, 8, nullptr, 1000, &pk, &pk, 0.1f, out, fake(), ws,
                                nullptr) == TQ_ERR_INVALID_ARG, "decode phase");
  EXPECT(tq_attn_decode_noalloc(&q, &q, qv, 1, 30, 8, nullptr, 1000, &pk, &pk, 0.1f, out, nullptr) ==
             TQ_ERR_INVALID_ARG, "noalloc Hq % Hkv");
  EXPECT(tq_attn_decode_noalloc(&q, &q, qv, 128, 128, 8, nullptr, 1024, &pk, &pk, 0.1f, out, nullptr) ==
             TQ_ERR_WORKSPACE, "noalloc beyond the scratch");
  // decode step
  EXPECT(tq_decode_step(&q, &q, x, x, 9, 128, qv, 1, 32, 8, nullptr, 1000, &pk, &pk, 0.1f, out, fake(), ws,
                        nullptr) == TQ_ERR_UNSUPPORTED, "step dtype");
  EXPECT(tq_decode_step(&q, &q, nullptr, x, TQ_BF16, 128, qv, 1, 32, 8, nullptr, 1000, &pk, &pk, 0.1f, out,
                        fake(), ws, nullptr) == TQ_ERR_INVALID_ARG, "step rows");
  EXPECT(tq_decode_step(&q, &q, x, x, TQ_BF16, 100, qv, 1, 32, 8, nullptr, 1000, &pk, &pk, 0.1f, out, fake(), ws,
                        nullptr) == TQ_ERR_INVALID_ARG, "step stride");
  EXPECT(tq_decode_step_phase(5, &q, &q, x, x, TQ_BF16, 128, qv, 1, 32, 8, nullptr, 1000, &pk, &pk, 0.1f, out,
                              fake(), ws, nullptr) == TQ_ERR_INVALID_ARG, "step phase");
  // search
  const size_t sws = tq_search_workspace(4, 1000, 10);
  EXPECT(sws > 0 && tq_search_workspace(4, 1000, 33) == 0, "search workspace");
  float* sc = static_cast<float*>(fake());
  int64_t* ix = static_cast<int64_t*>(fake());
  EXPECT(tq_search(&q, qv, 4, &pk, 1000, 0, sc, ix, fake(), sws, nullptr) == TQ_ERR_INVALID_ARG, "search k");
  EXPECT(tq_search(&q, qv, 4, &pk, 1000, 33, sc, ix, fake(), sws, nullptr) == TQ_ERR_UNSUPPORTED, "search k > 32");
  EXPECT(tq_search(&q, qv, 4, &pk, 5, 10, sc, ix, fake(), sws, nullptr) == TQ_ERR_INVALID_ARG, "search k > n");
  EXPECT(tq_search(&q, qv, 4, &pk, 1000, 10, sc, ix, fake(), sws - 8, nullptr) == TQ_ERR_WORKSPACE,
         "search workspace size");
  // outlier-channel split: Π_o, Π_r and a host channel list; tq_prepare
  // checks the list (32 distinct channels in [0, 128)) before device work
  {
    tq_quantizer sq = quant(128, 2, TQ_MSE);
    sq.rot = nullptr;
    sq.split = TQ_SPLIT_OUTLIER32;
    sq.centroids_o = static_cast<const float*>(fake());
    sq.boundaries_o = static_cast<const float*>(fake());
    sq.rot_o = static_cast<const float*>(fake());
    sq.rot_r = static_cast<const float*>(fake());
    int32_t* ch = new int32_t[32];   // exactly 32 entries: a read past them is an ASan error
    for (int j = 0; j < 32; ++j) ch[j] = 4 * j;
    ch[31] = 0;
    sq.channels_o = ch;
    EXPECT(tq_prepare(&sq, nullptr) == TQ_ERR_INVALID_ARG, "split duplicate channel");
    ch[31] = 128;
    EXPECT(tq_prepare(&sq, nullptr) == TQ_ERR_INVALID_ARG, "split channel out of range");
    ch[31] = 124;
    sq.rot_o = nullptr;
    EXPECT(tq_prepare(&sq, nullptr) == TQ_ERR_INVALID_ARG, "split without rot_o");
    sq.rot_o = static_cast<const float*>(fake());
    sq.channels_o = nullptr;
    EXPECT(tq_prepare(&sq, nullptr) == TQ_ERR_INVALID_ARG, "split without channels");
    EXPECT(tq_encode(&sq, x, TQ_BF16, 0, 128, &pk, nullptr, nullptr) == TQ_ERR_INVALID_ARG, "split encode channels");
    delete[] ch;
  }
  // chunked encode and search
  EXPECT(tq_encode_chunked(&q, x, TQ_BF16, 8, 0, 256, &pk, nullptr) == TQ_ERR_INVALID_ARG, "chunked encode chunks");
  EXPECT(tq_encode_chunked(&q, x, TQ_BF16, 8, 65, 65 * 128, &pk, nullptr) == TQ_ERR_UNSUPPORTED,
         "chunked encode chunks > 64");
  EXPECT(tq_encode_chunked(&q, x, TQ_BF16, 8, 2, 128, &pk, nullptr) == TQ_ERR_INVALID_ARG, "chunked encode stride");
  const size_t cws = tq_search_chunked_workspace(4, 1000, 10, 12);
  EXPECT(cws > sws && tq_search_chunked_workspace(4, 1000, 10, 1) == sws &&
             tq_search_chunked_workspace(4, 1000, 10, 0) == 0 && tq_search_chunked_workspace(4, 1000, 10, 65) == 0,
         "chunked search workspace");
  EXPECT(tq_search_chunked(&q, qv, 4, 0, &pk, 1000, 10, sc, ix, fake(), cws, nullptr) == TQ_ERR_INVALID_ARG,
         "chunked search chunks");
  EXPECT(tq_search_chunked(&q, qv, 4, 65, &pk, 1000, 10, sc, ix, fake(), cws, nullptr) == TQ_ERR_UNSUPPORTED,
         "chunked search chunks > 64");
  EXPECT(tq_search_chunked(&q, qv, 4, 12, &pk, 1000, 10, sc, ix, fake(), cws - 8, nullptr) == TQ_ERR_WORKSPACE,
         "chunked search workspace size");
  // read probe
  uint32_t* xo = static_cast<uint32_t*>(fake());
  EXPECT(tq_read_probe(nullptr, 16, xo, nullptr) == TQ_ERR_INVALID_ARG, "probe null");
  EXPECT(tq_read_probe(fake(), 17, xo, nullptr) == TQ_ERR_INVALID_ARG, "probe size");
  EXPECT(tq_read_probe(fake(8), 16, xo, nullptr) == TQ_ERR_INVALID_ARG, "probe alignment");
}

int main() {
  codebooks();
  argument_checks();
  if (g_fail) {
    fprintf(stderr, "%d host check(s) failed\n", g_fail);
    return 1;
  }
  printf("host checks passed\n");
  return 0;
}
