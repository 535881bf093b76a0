// Host-side argument validation of the C ABI (include/ae.h), run in a build
// of the library whose host code carries AddressSanitizer and UBSan: every
// check that must reject a call before any HIP work, on a machine with or
// without a GPU.  Configs that pass every check then need a device: without
// one they end in AE_ERR_HIP, with one the handle is created and destroyed.
// Prints "failed checks: N".
#include <cstdio>
#include <cstring>
#include <vector>

#include "ae.h"

static int g_failed = 0;

#define CHECK(cond)                                                  \
  do {                                                               \
    if (!(cond)) {                                                   \
      std::printf("FAILED: %s (line %d)\n", #cond, __LINE__);        \
      ++g_failed;                                                    \
    }                                                                \
  } while (0)

static ae_config base() {
  ae_config c;
  std::memset(&c, 0, sizeof(c));
  c.n_layers = 2; c.width = 128; c.n_q_heads = 2; c.n_kv_heads = 1; c.head_dim = 64; c.mlp_dim = 512;
  c.action_horizon = 8; c.action_dim = 7; c.max_prefix_len = 64; c.max_batch = 2; c.max_steps = 4;
  c.act_dtype = AE_BF16; c.proj_weight_dtype = AE_BF16; c.rope_theta = 10000.0f; c.rms_eps = 1e-6f;
  c.use_graphs = 1; c.graph_cache_size = 4; c.graph_cache_evict = 1;
  return c;
}

static ae_status create(const ae_config& c, ae_handle** h) {
  *h = reinterpret_cast<ae_handle*>(0x1);  // must come back NULL on failure
  return ae_create(&c, h);
}

int main() {
  ae_handle* h = nullptr;
  // invalid values: INVALID_ARGUMENT, handle NULL
  struct Bad {
    const char* what;
    void (*edit)(ae_config&);
  };
  const Bad invalid[] = {
      {"n_layers 0", [](ae_config& c) { c.n_layers = 0; }},
      {"width 100", [](ae_config& c) { c.width = 100; }},
      {"width 8192", [](ae_config& c) { c.width = 8192; }},
      {"n_kv_heads 3", [](ae_config& c) { c.n_kv_heads = 3; }},
      {"mlp_dim 48", [](ae_config& c) { c.mlp_dim = 48; }},
      {"action_dim 65", [](ae_config& c) { c.action_dim = 65; }},
      {"max_batch 0", [](ae_config& c) { c.max_batch = 0; }},
      {"max_steps 65", [](ae_config& c) { c.max_steps = 65; }},
      {"max_prefix_len -1", [](ae_config& c) { c.max_prefix_len = -1; }},
      {"act_dtype 7", [](ae_config& c) { c.act_dtype = 7; }},
      {"rope_theta 0", [](ae_config& c) { c.rope_theta = 0.0f; }},
      {"use_graphs 2", [](ae_config& c) { c.use_graphs = 2; }},
      {"graph_cache_size 65", [](ae_config& c) { c.graph_cache_size = 65; }},
      {"context_width 100", [](ae_config& c) { c.context_width = 100; }},
      {"state without context", [](ae_config& c) { c.state_dim = 14; }},
      {"block_type 2", [](ae_config& c) { c.block_type = 2; }},
      {"fp8_rowwise 2", [](ae_config& c) { c.fp8_rowwise = 2; }},
      {"fp8_rowwise with bf16 projections", [](ae_config& c) { c.fp8_rowwise = 1; }},
      {"exec_path 3", [](ae_config& c) { c.exec_path = 3; }},
  };
  for (const Bad& b : invalid) {
    ae_config c = base();
    b.edit(c);
    const ae_status s = create(c, &h);
    if (s != AE_ERR_INVALID_ARGUMENT || h != nullptr) std::printf("  (%s)\n", b.what);
    CHECK(s == AE_ERR_INVALID_ARGUMENT);
    CHECK(h == nullptr);
  }
  // valid but not implemented: UNSUPPORTED
  const Bad unsupported[] = {
      {"head_dim 96", [](ae_config& c) { c.head_dim = 96; }},
      {"fp8 with fp32 activations", [](ae_config& c) { c.act_dtype = AE_F32; c.proj_weight_dtype = AE_FP8_E4M3; }},
      {"fp8 output projection without row-wise scales",
       [](ae_config& c) { c.proj_weight_dtype = AE_FP8_E4M3; c.fp8_oproj = 1; }},
      {"DiT block in fp32", [](ae_config& c) { c.block_type = AE_BLOCK_DIT; c.act_dtype = AE_F32; c.proj_weight_dtype = AE_F32; }},
      {"context preparation in fp32", [](ae_config& c) { c.context_width = 128; c.act_dtype = AE_F32; c.proj_weight_dtype = AE_F32; }},
  };
  for (const Bad& b : unsupported) {
    ae_config c = base();
    b.edit(c);
    const ae_status s = create(c, &h);
    if (s != AE_ERR_UNSUPPORTED || h != nullptr) std::printf("  (%s)\n", b.what);
    CHECK(s == AE_ERR_UNSUPPORTED);
    CHECK(h == nullptr);
  }
  // null arguments, every entry point
  CHECK(ae_create(nullptr, nullptr) == AE_ERR_INVALID_ARGUMENT);
  CHECK(ae_create(nullptr, &h) == AE_ERR_INVALID_ARGUMENT);
  CHECK(ae_load_weights(nullptr, nullptr, 0, nullptr) == AE_ERR_INVALID_ARGUMENT);
  CHECK(ae_set_prefix_kv(nullptr, 1, 0, nullptr, nullptr, nullptr, nullptr) == AE_ERR_INVALID_ARGUMENT);
  CHECK(ae_prepare_prefix(nullptr, 1, 0, nullptr, nullptr, nullptr, nullptr) == AE_ERR_INVALID_ARGUMENT);
  CHECK(ae_set_prefix_buckets(nullptr, nullptr, 0) == AE_ERR_INVALID_ARGUMENT);
  CHECK(ae_denoise(nullptr, nullptr, 1, 1, nullptr, nullptr) == AE_ERR_INVALID_ARGUMENT);
  CHECK(ae_denoise_static(nullptr, nullptr, 1, 1, nullptr, nullptr) == AE_ERR_INVALID_ARGUMENT);
  CHECK(ae_get_stats(nullptr, nullptr) == AE_ERR_INVALID_ARGUMENT);
  CHECK(std::strcmp(ae_last_error(nullptr), "null handle") == 0);
  CHECK(std::strcmp(ae_status_string(AE_OK), "ok") == 0);
  CHECK(std::strcmp(ae_status_string(99), "unknown status") == 0);
  ae_destroy(nullptr);
  // valid configs: no GPU -> HIP error and a NULL handle; a GPU -> a handle
  {
    ae_config c = base();
    const ae_status s = create(c, &h);
    CHECK(s == AE_OK || s == AE_ERR_HIP);
    if (s == AE_OK) {
      CHECK(h != nullptr);
      // a handle rejects calls before any work: no weights, bad buckets
      const int bad_buckets[2] = {32, 16};
      CHECK(ae_set_prefix_buckets(h, bad_buckets, 2) == AE_ERR_INVALID_ARGUMENT);
      std::vector<float> dummy(1);
      CHECK(ae_denoise(h, dummy.data(), 1, 1, dummy.data(), nullptr) == AE_ERR_NOT_READY);
      ae_destroy(h);
    } else {
      CHECK(h == nullptr);
    }
  }
  std::printf("failed checks: %d\n", g_failed);
  return g_failed == 0 ? 0 : 1;
}
