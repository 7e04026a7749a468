// Host-side paths of the library that run without a GPU -- configuration
// checks, workspace sizing (also with the TTE_DEBUG guards), pack
// validation on fixed and on random offset arrays, model creation's refusals
// and its no-device error, and the per-kernel entry points' shape refusals
// -- driven against a build whose host code carries AddressSanitizer and
// UndefinedBehaviorSanitizer.  Exits non-zero on any failed expectation; the
// sanitizers abort on any memory error or undefined behaviour they see.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <string>
#include <vector>

#include "tte.h"

static int failures = 0;

#define EXPECT(cond)                                                                                           \
  do {                                                                                                         \
    if (!(cond)) {                                                                                             \
      std::fprintf(stderr, "FAILED %s:%d: %s (last error: %s)\n", __FILE__, __LINE__, #cond, tte_last_error()); \
      ++failures;                                                                                              \
    }                                                                                                          \
  } while (0)

static tte_config base_config() {
  tte_config c;
  std::memset(&c, 0, sizeof c);
  c.vocab = 102400;
  c.hidden = 768;
  c.n_heads = 12;
  c.head_dim = 64;
  c.intermediate = 3072;
  c.n_layers = 25;
  c.global_every = 3;
  c.window = 64;
  c.rope_base_global = 160000.f;
  c.rope_base_local = 10000.f;
  c.ln_eps = 1e-5f;
  c.max_tokens = 2048;
  c.max_text_len = 512;
  c.max_texts = 256;
  c.precision = TTE_BF16;
  c.flags = 0;
  return c;
}

static void configs() {
  size_t a = 0, b = 0;
  tte_config c = base_config();
  EXPECT(tte_workspace_size(&c, &a) == TTE_OK && a > 0 && a % 256 == 0);
  c.max_tokens = 4096;
  EXPECT(tte_workspace_size(&c, &b) == TTE_OK && b > a);
  for (int p = TTE_FP32; p <= TTE_INT4; ++p) {
    c = base_config();
    c.precision = p;
    EXPECT(tte_workspace_size(&c, &a) == TTE_OK);
  }
  c = base_config();
  c.flags = TTE_FLAG_SPLIT_K | TTE_FLAG_GRAPH;
  EXPECT(tte_workspace_size(&c, &a) == TTE_OK);
  EXPECT(tte_workspace_size(nullptr, &a) == TTE_E_INVALID);
  c = base_config();
  EXPECT(tte_workspace_size(&c, nullptr) == TTE_E_INVALID);
  struct Bad {
    const char* what;
    void (*apply)(tte_config&);
  } bad[] = {
      {"head_dim", [](tte_config& x) { x.head_dim = 32; }},
      {"hidden", [](tte_config& x) { x.hidden = 700; }},
      {"intermediate", [](tte_config& x) { x.intermediate = 3000; }},
      {"precision", [](tte_config& x) { x.precision = 7; }},
      {"max_tokens", [](tte_config& x) { x.max_tokens = 0; }},
      {"max_tokens big", [](tte_config& x) { x.max_tokens = (1 << 24) + 1; }},
      {"global_every", [](tte_config& x) { x.global_every = 0; }},
      {"window", [](tte_config& x) { x.window = -1; }},
      {"ln_eps", [](tte_config& x) { x.ln_eps = 0.f; }},
      {"n_layers", [](tte_config& x) { x.n_layers = 0; }},
      {"max_texts", [](tte_config& x) { x.max_texts = 0; }},
      {"flags", [](tte_config& x) { x.flags = 4; }},
      {"int4 widths", [](tte_config& x) { x.precision = TTE_INT4; x.intermediate = 3072 + 128; }},
  };
  for (const Bad& k : bad) {
    c = base_config();
    k.apply(c);
    const tte_status st = tte_workspace_size(&c, &a);
    if (st != TTE_E_INVALID) std::fprintf(stderr, "config case %s\n", k.what);
    EXPECT(st == TTE_E_INVALID);
    EXPECT(std::strlen(tte_last_error()) > 0);
  }
}

static void packs() {
  const tte_config c = base_config();
  struct Case {
    int32_t T;
    std::vector<int32_t> off;
    bool ok;
  } cases[] = {
      {10, {0, 3, 10}, true},   {0, {0}, true},          {10, {1, 3, 10}, false},
      {10, {0, 3, 3, 10}, false}, {10, {0, 6, 4, 10}, false}, {10, {0, 3, 9}, false},
      {3000, {0, 500, 1000, 1500, 2000, 2500, 3000}, false}, {600, {0, 600}, false},
  };
  for (const Case& k : cases) {
    const tte_status st = tte_check_pack(&c, k.T, k.off.data(), (int32_t)k.off.size() - 1);
    EXPECT((st == TTE_OK) == k.ok);
  }
  EXPECT(tte_check_pack(&c, 5, nullptr, 2) == TTE_E_INVALID);
  EXPECT(tte_check_pack(&c, -1, nullptr, 0) == TTE_E_INVALID);
  EXPECT(tte_check_pack(&c, 3, nullptr, 0) == TTE_E_INVALID);
  // random offset arrays, valid and not: the validator reads exactly
  // n_texts + 1 entries (the arrays are sized so; ASan sees any read beyond)
  std::mt19937 rng(7);
  int valid = 0;
  for (int it = 0; it < 20000; ++it) {
    const int n = 1 + (int)(rng() % 300);
    std::vector<int32_t> off((size_t)n + 1);
    off[0] = (rng() % 50 == 0) ? 1 : 0;
    for (int b = 1; b <= n; ++b) {
      const int len = (int)(rng() % 24) - (rng() % 97 == 0 ? 30 : 0);
      off[b] = off[b - 1] + len;
    }
    const int32_t T = (rng() % 40 == 0) ? off[n] + 1 : off[n];
    const tte_status st = tte_check_pack(&c, T, off.data(), n);
    EXPECT(st == TTE_OK || st == TTE_E_INVALID);
    valid += st == TTE_OK;
  }
  EXPECT(valid > 1000);
}

static void create_and_run_refusals() {
  tte_config c = base_config();
  std::vector<tte_layer_weights> layers((size_t)c.n_layers);
  const void* fake = reinterpret_cast<const void*>(uintptr_t(256));
  const float* ffake = reinterpret_cast<const float*>(uintptr_t(256));
  for (auto& L : layers) {
    std::memset(&L, 0, sizeof L);
    L.wqkv = L.wo = L.wi = L.wo2 = fake;
    L.attn_norm = L.mlp_norm = ffake;
  }
  tte_weights w;
  std::memset(&w, 0, sizeof w);
  w.tok_emb = fake;
  w.emb_norm = w.final_norm = ffake;
  w.layers = layers.data();
  tte_model* m = reinterpret_cast<tte_model*>(uintptr_t(1));
  EXPECT(tte_create(&c, nullptr, nullptr, 0, &m) == TTE_E_INVALID);
  EXPECT(tte_create(&c, &w, nullptr, 0, nullptr) == TTE_E_INVALID);
  layers[3].wo2 = nullptr;
  EXPECT(tte_create(&c, &w, nullptr, 0, &m) == TTE_E_INVALID);
  EXPECT(std::string(tte_last_error()).find("layer 3") != std::string::npos);
  layers[3].wo2 = fake;
  c.precision = TTE_INT8;  // scales missing
  EXPECT(tte_create(&c, &w, nullptr, 0, &m) == TTE_E_INVALID);
  c.precision = TTE_BF16;
  // complete weights: without a GPU the device check refuses (with one,
  // the NULL workspace does)
  const tte_status st = tte_create(&c, &w, nullptr, 0, &m);
  EXPECT(st == TTE_E_DEVICE || st == TTE_E_INVALID);
  EXPECT(tte_embed(nullptr, nullptr, 0, nullptr, 0, nullptr, nullptr) == TTE_E_INVALID);
  EXPECT(tte_embed_tokens(nullptr, nullptr, 0, nullptr, 0, nullptr, nullptr) == TTE_E_INVALID);
  EXPECT(tte_destroy(nullptr) == TTE_E_INVALID);
  int32_t a = 0, b = 0;
  int64_t r = 0;
  EXPECT(tte_graph_stats(nullptr, &a, &b, &r) == TTE_E_INVALID);
}

static void op_refusals() {
  EXPECT(tte_op_gemm(TTE_BF16, TTE_EPI_STORE, nullptr, nullptr, nullptr, nullptr, 16, 100, 128, nullptr, 0, nullptr) ==
         TTE_E_UNSUPPORTED);
  EXPECT(tte_op_gemm(TTE_BF16, TTE_EPI_STORE, nullptr, nullptr, nullptr, nullptr, 16, 128, 96, nullptr, 0, nullptr) ==
         TTE_E_UNSUPPORTED);
  EXPECT(tte_op_gemm(TTE_INT8, TTE_EPI_RESIDUAL, nullptr, nullptr, nullptr, nullptr, 16, 128, 128, nullptr, 1,
                     nullptr) == TTE_E_INVALID);
  EXPECT(tte_op_gemm(TTE_FP32, TTE_EPI_RESIDUAL, nullptr, nullptr, nullptr, nullptr, 16, 128, 128, nullptr, 1,
                     nullptr) == TTE_E_INVALID);
  EXPECT(tte_op_gemm(TTE_BF16, TTE_EPI_RESIDUAL, nullptr, nullptr, nullptr, nullptr, 0, 128, 128, nullptr, 1,
                     nullptr) == TTE_OK);
  EXPECT(tte_op_gemm_splitk(TTE_BF16, nullptr, nullptr, nullptr, nullptr, 16, 128, 320, 2, nullptr, nullptr) ==
         TTE_E_UNSUPPORTED);
  EXPECT(tte_op_gemm_splitk(TTE_BF16, nullptr, nullptr, nullptr, nullptr, 16, 128, 512, 0, nullptr, nullptr) ==
         TTE_E_INVALID);
  EXPECT(tte_op_resid_ln(nullptr, nullptr, 1, nullptr, 4, 768, 1e-5f, 3, nullptr, nullptr, nullptr) == TTE_E_INVALID);
  // weights past 32-bit byte offsets are refused before any launch
  const void* fake = reinterpret_cast<const void*>(uintptr_t(256));
  const float* ffake = reinterpret_cast<const float*>(uintptr_t(256));
  void* out = reinterpret_cast<void*>(uintptr_t(256));
  EXPECT(tte_op_gemm(TTE_BF16, TTE_EPI_STORE, fake, ffake, fake, ffake, 16, 65536, 32768, out, 0, nullptr) ==
         TTE_E_UNSUPPORTED);
  EXPECT(tte_op_gemm(TTE_BF16, TTE_EPI_STORE, fake, ffake, fake, ffake, 0, 65536 - 128, 32768, out, 0, nullptr) ==
         TTE_OK);
  EXPECT(tte_similarity(nullptr, 4, 100, nullptr, nullptr) == TTE_E_UNSUPPORTED);
  EXPECT(tte_similarity(nullptr, -1, 128, nullptr, nullptr) == TTE_E_INVALID);
  EXPECT(tte_similarity(nullptr, 0, 128, nullptr, nullptr) == TTE_OK);
  EXPECT(tte_similarity(nullptr, 3, 128, nullptr, nullptr) == TTE_E_INVALID);
  EXPECT(tte_op_pool(nullptr, nullptr, 0, nullptr, 0, nullptr, nullptr) == TTE_E_INVALID);
  EXPECT(tte_op_pool_static(nullptr, nullptr, 0, nullptr, 0, nullptr, nullptr) == TTE_E_INVALID);
}

int main() {
  configs();
  packs();
  create_and_run_refusals();
  op_refusals();
  std::printf("host checks done, %d failed\n", failures);
  return failures == 0 ? 0 : 1;
}
