// Host-only validation of the C ABI under AddressSanitizer: the config checks of fm_query, the
// weight specification, the device check and the kernel-level entry points' argument checks,
// over the presets and a seeded sweep of malformed configs (every field pushed to 0, to
// negative values, to one past its limits and to large values), with message buffers from
// 0 bytes up. None of these touches a GPU. Built as a shared library whose fm_host_validation()
// returns 0 when every call returned a defined status; AddressSanitizer reports any invalid
// memory access.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "fm.h"

namespace {

fm_config pi05() {
  fm_config c;
  std::memset(&c, 0, sizeof c);
  c.arch = FM_ARCH_PREFIX_JOINT; c.dtype = FM_BF16; c.n_layers = 18; c.hidden = 1024; c.n_heads = 8;
  c.head_dim = 256; c.n_kv_heads = 1; c.mlp_dim = 4096; c.mlp_gated = 1; c.action_horizon = 50;
  c.action_dim = 32; c.max_prefix_len = 816; c.max_batch = 8; c.max_steps = 10;
  c.rope_base = 10000.f; c.norm_eps = 1e-6f;
  return c;
}

fm_config dit() {
  fm_config c;
  std::memset(&c, 0, sizeof c);
  c.arch = FM_ARCH_DIT_CROSS; c.dtype = FM_BF16; c.n_layers = 32; c.hidden = 1536; c.n_heads = 24;
  c.head_dim = 64; c.n_kv_heads = 24; c.mlp_dim = 6144; c.mlp_gated = 0; c.action_horizon = 40;
  c.action_dim = 32; c.state_tokens = 1; c.state_dim = 64; c.ctx_len_max = 600; c.ctx_dim = 2048;
  c.max_batch = 1; c.max_steps = 4; c.rope_base = 0.f; c.norm_eps = 1e-6f;
  return c;
}

uint64_t g_state = 0x9E3779B97F4A7C15ull;
uint32_t rnd() {   // xorshift64*
  g_state ^= g_state >> 12; g_state ^= g_state << 25; g_state ^= g_state >> 27;
  return (uint32_t)((g_state * 2685821657736338717ull) >> 32);
}

int g_calls = 0, g_bad = 0;
void expect_status(fm_status s, const char* what) {
  ++g_calls;
  if ((int)s < (int)FM_OK || (int)s > (int)FM_ERR_DEVICE) {
    std::fprintf(stderr, "%s: undefined status %d\n", what, (int)s);
    ++g_bad;
  }
}

// fm_query with message buffers of several sizes, then every weight spec of an accepted config
void query_all(const fm_config& c) {
  static const int kLens[] = {0, 1, 7, 64, 512};
  for (int len : kLens) {
    std::vector<char> msg((size_t)len + 1, 'x');   // one guard byte past the given length
    fm_plan_info info;
    const fm_status s = fm_query(&c, &info, len ? msg.data() : nullptr, len);
    expect_status(s, "fm_query");
    if (msg[(size_t)len] != 'x') { std::fprintf(stderr, "fm_query wrote past msg_len %d\n", len); ++g_bad; }
    if (s == FM_OK && len == 64) {
      // an accepted config may have thousands of layers: the first and last specs suffice there
      for (int i = -2; i < info.n_weights + 2; ++i) {
        if (i == 64 && info.n_weights > 128) i = info.n_weights - 64;
        const char* name = nullptr;
        int32_t nd = 0;
        int64_t shape[4];
        const fm_status w = fm_weight_spec(&c, i, &name, &nd, shape);
        expect_status(w, "fm_weight_spec");
        if (w == FM_OK && (!name || nd < 1 || nd > 4)) { std::fprintf(stderr, "weight spec %d malformed\n", i); ++g_bad; }
      }
    }
  }
}

}  // namespace

extern "C" int fm_host_validation() {
  // presets and the NULL forms
  query_all(pi05());
  query_all(dit());
  expect_status(fm_query(nullptr, nullptr, nullptr, 0), "fm_query(NULL)");
  {
    fm_config c = pi05();
    expect_status(fm_query(&c, nullptr, nullptr, 0), "fm_query(info NULL)");
    expect_status(fm_weight_spec(nullptr, 0, nullptr, nullptr, nullptr), "fm_weight_spec(NULL)");
  }
  (void)fm_last_error(nullptr);
  // the device check over arch names, XCD and CU counts
  const char* archs[] = {"gfx950", "gfx950:sramecc+:xnack-", "gfx942", "", "gfx95"};
  for (const char* a : archs)
    for (int xcc : {0, 1, 4, 8, 16})
      for (int cus : {0, 32, 255, 256, 304}) {
        char msg[48];
        expect_status(fm_device_supported(a, xcc, cus, msg, (int32_t)sizeof msg), "fm_device_supported");
        expect_status(fm_device_supported(a, xcc, cus, nullptr, 0), "fm_device_supported(msg NULL)");
      }
  expect_status(fm_device_supported(nullptr, 8, 256, nullptr, 0), "fm_device_supported(NULL)");
  // malformed configs: each field of each preset set to an edge value, and seeded random mixes
  const int32_t edges[] = {0, -1, 1, 2, 3, 7, 33, 63, 65, 255, 257, 4097, 65536, 1 << 30, -(1 << 30)};
  for (int preset = 0; preset < 2; ++preset) {
    const fm_config base = preset ? dit() : pi05();
    const int nint = 18;   // the int32_t fields, in declaration order
    for (int f = 0; f < nint; ++f)
      for (int32_t e : edges) {
        fm_config c = base;
        reinterpret_cast<int32_t*>(&c)[f] = e;
        query_all(c);
      }
    for (float v : {-1.f, 0.f, 1e-12f, 1e30f}) {
      fm_config c = base;
      c.norm_eps = v;
      query_all(c);
      c = base;
      c.rope_base = v;
      query_all(c);
    }
    for (int it = 0; it < 2000; ++it) {
      fm_config c = base;
      for (int k = 0; k < 3; ++k) reinterpret_cast<int32_t*>(&c)[rnd() % nint] = edges[rnd() % (sizeof edges / sizeof edges[0])];
      query_all(c);
    }
  }
  // kernel-level entry points: argument checks that refuse before any device call
  expect_status(fm_op_linear(FM_BF16, 4, 4, 33, nullptr, nullptr, nullptr, 0, nullptr, 0, nullptr), "fm_op_linear");
  expect_status(fm_op_linear(7, 4, 4, 32, nullptr, nullptr, nullptr, 0, nullptr, 0, nullptr), "fm_op_linear dtype");
  expect_status(fm_op_attention(FM_BF16, 1, 1, 1, 1, 1, 96, nullptr, nullptr, nullptr, nullptr, nullptr), "fm_op_attention");
  expect_status(fm_op_attention_noalloc(FM_F32, 1, 1, 2, 3, 1, 64, nullptr, nullptr, nullptr, nullptr, nullptr),
                "fm_op_attention_noalloc");
  expect_status(fm_op_quantize_fp8(4, 3, nullptr, nullptr, nullptr, nullptr, nullptr), "fm_op_quantize_fp8");
  std::printf("host validation: %d calls, %d with an undefined status\n", g_calls, g_bad);
  return g_bad ? 1 : 0;
}
