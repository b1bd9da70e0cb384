// Drives every entry point of the C ABI through its argument checks and its
// planner (valid shapes reach the launch stubs), under ASan/UBSan.  Exits 0
// when every status is the expected one; a sanitizer report aborts the run.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <thread>
#include <vector>

#include "spec_verify.h"
#include "sv_ceilings.h"

static int g_fail = 0;
#define EXPECT(expr, want)                                                                \
  do {                                                                                    \
    const int got_ = (int)(expr);                                                         \
    if (got_ != (int)(want)) {                                                            \
      std::printf("FAIL line %d: %s -> %d, want %d (%s)\n", __LINE__, #expr, got_,        \
                  (int)(want), sv_last_error());                                          \
      ++g_fail;                                                                           \
    }                                                                                     \
    (void)std::strlen(sv_last_error());                                                   \
  } while (0)

// Never dereferenced: the launch stubs ignore their pointers.
static void* const F = reinterpret_cast<void*>(0x100000);
static char* fp(size_t off = 0) { return static_cast<char*>(F) + off; }

static sv_attn_params attn(int B, int D, int Hq, int Hkv, int hd, int maxb, int nb, int maxlen,
                           int dtype = SV_KV_BF16, int split = 0) {
  sv_attn_params p;
  std::memset(&p, 0, sizeof(p));
  p.batch = B; p.draft_len = D; p.num_q_heads = Hq; p.num_kv_heads = Hkv; p.head_dim = hd;
  p.block_size = 16; p.max_blocks_per_seq = maxb; p.num_blocks = nb; p.max_kv_len = maxlen;
  p.kv_dtype = (sv_kv_dtype)dtype; p.sm_scale = 0.088f; p.split_tokens = split;
  return p;
}

static void attention() {
  size_t ws = 0;
  // a grid of shapes through the planner: stream-K and split paths, bf16 and e4m3
  const int Bs[] = {1, 7, 32, 2048, 2049, 5000};
  const int Ds[] = {0, 3, 15, 16, 31, 63};
  const int Gs[] = {1, 4, 8, 64};
  for (int B : Bs)
    for (int D : Ds)
      for (int G : Gs)
        for (int hd : {64, 128})
          for (int dt : {SV_KV_BF16, SV_KV_FP8_E4M3})
            for (int split : {0, 64, 1 << 20}) {
              const int maxlen = 16 * 64 + D + 1;
              sv_attn_params p = attn(B, D, 2 * G, 2, hd, 80, 1000, maxlen, dt, split);
              const sv_status s = spec_verify_attn_workspace_size(&p, &ws);
              if (s != SV_OK && s != SV_ERR_UNSUPPORTED) {
                std::printf("FAIL planner status %d for B=%d D=%d G=%d\n", s, B, D, G);
                ++g_fail;
              }
              if (s == SV_OK) {
                const float* ks = dt == SV_KV_FP8_E4M3 ? (const float*)F : nullptr;
                EXPECT(spec_verify_attn(&p, F, F, F, ks, ks, (const int32_t*)F, (const int32_t*)F,
                                        fp(1 << 20), ws ? fp(1 << 22) : nullptr, ws, nullptr),
                       SV_OK);
                if (ws) {
                  EXPECT(spec_verify_attn(&p, F, F, F, ks, ks, (const int32_t*)F,
                                          (const int32_t*)F, fp(1 << 20), fp(1 << 22), ws - 1,
                                          nullptr),
                         SV_ERR_WORKSPACE);
                }
              }
            }
  sv_attn_params p = attn(4, 15, 64, 8, 128, 64, 256, 1000);
  EXPECT(spec_verify_attn_workspace_size(nullptr, &ws), SV_ERR_INVALID);
  EXPECT(spec_verify_attn_workspace_size(&p, nullptr), SV_ERR_INVALID);
  EXPECT(spec_verify_attn_workspace_size(&p, &ws), SV_OK);
  EXPECT(spec_verify_attn(&p, nullptr, F, F, nullptr, nullptr, (const int32_t*)F,
                          (const int32_t*)F, F, F, ws, nullptr), SV_ERR_INVALID);
  EXPECT(spec_verify_attn(&p, fp(2), F, F, nullptr, nullptr, (const int32_t*)F,
                          (const int32_t*)F, F, F, ws, nullptr), SV_ERR_INVALID);
  EXPECT(spec_verify_attn(&p, F, F, F, (const float*)F, nullptr, (const int32_t*)F,
                          (const int32_t*)F, F, F, ws, nullptr), SV_ERR_INVALID);
  EXPECT(spec_verify_attn(&p, F, F, F, nullptr, nullptr, (const int32_t*)F, (const int32_t*)F, F,
                          nullptr, ws, nullptr), SV_ERR_WORKSPACE);
  EXPECT(spec_verify_attn_tree(&p, F, F, F, nullptr, nullptr, (const int32_t*)F,
                               (const int32_t*)F, nullptr, F, F, ws, nullptr), SV_ERR_INVALID);
  EXPECT(spec_verify_attn_tree(&p, F, F, F, nullptr, nullptr, (const int32_t*)F,
                               (const int32_t*)F, (const uint64_t*)fp(4), F, F, ws, nullptr),
         SV_ERR_INVALID);
  EXPECT(spec_verify_attn_tree(&p, F, F, F, nullptr, nullptr, (const int32_t*)F,
                               (const int32_t*)F, (const uint64_t*)F, F, F, ws, nullptr), SV_OK);
  // invalid shapes
  const sv_attn_params bad[] = {
      attn(0, 15, 64, 8, 128, 64, 256, 1000), attn(4, -1, 64, 8, 128, 64, 256, 1000),
      attn(4, 64, 64, 8, 128, 64, 256, 1000), attn(4, 15, 64, 7, 128, 64, 256, 1000),
      attn(4, 15, 64, 8, 96, 64, 256, 1000),  attn(4, 15, 64, 8, 128, 10, 256, 1000),
      attn(4, 15, 64, 8, 128, 64, 0, 1000),   attn(4, 15, 64, 8, 128, 64, 256, 10),
      attn(4, 15, 64, 8, 128, 64, 256, 1000, 7), attn(4, 15, 64, 8, 128, 64, 256, 1000, 0, 48)};
  for (const sv_attn_params& b : bad) {
    const sv_status s = spec_verify_attn_workspace_size(&b, &ws);
    if (s != SV_ERR_INVALID && s != SV_ERR_UNSUPPORTED) {
      std::printf("FAIL bad shape accepted (status %d)\n", s);
      ++g_fail;
    }
  }
  // the 2^31 stream-K tile count (2048 sequences x 32 row tiles of 256 x 32768 tiles)
  sv_attn_params big = attn(2048, 63, 128, 1, 64, 65536, 1 << 20, 1 << 20);
  EXPECT(spec_verify_attn_workspace_size(&big, &ws), SV_ERR_UNSUPPORTED);
}

static void acceptance() {
  size_t ws = 0;
  for (int B : {1, 3, 32, 4096})
    for (int D : {0, 1, 15, 63})
      for (int V : {1, 4095, 4096, 4097, 128256}) {
        const sv_status s = spec_accept_workspace_size(B, D, V, &ws);
        if (s != SV_OK) {
          if (B * (D + 1) <= 65535) { std::printf("FAIL accept ws %d %d %d\n", B, D, V); ++g_fail; }
          continue;
        }
        const int32_t* dr = D ? (const int32_t*)F : nullptr;
        EXPECT(spec_accept(B, D, V, (const float*)F, dr, (int32_t*)F, (int32_t*)F, (int32_t*)F,
                           (const int32_t*)F, (int32_t*)F, fp(1 << 20), ws, nullptr), SV_OK);
        EXPECT(spec_accept(B, D, V, (const float*)F, dr, (int32_t*)F, (int32_t*)F, (int32_t*)F,
                           (const int32_t*)F, (int32_t*)F, fp(1 << 20), ws - 1, nullptr),
               SV_ERR_WORKSPACE);
        EXPECT(spec_accept_tree(B, D, V, (const float*)F, dr, dr, (int32_t*)F, (int32_t*)F,
                                (int32_t*)F, (int32_t*)F, (const int32_t*)F, (int32_t*)F,
                                fp(1 << 20), ws, nullptr), SV_OK);
        const size_t need_na = (size_t)B * (D + 1) * ((V + 4095) / 4096) * 8;
        EXPECT(spec_accept_noalloc(B, D, V, (const float*)F, dr, (int32_t*)F, (int32_t*)F,
                                   (int32_t*)F, (const int32_t*)F, (int32_t*)F, nullptr),
               need_na <= (4u << 20) ? SV_OK : SV_ERR_UNSUPPORTED);
        if (B * (2 * D + 1) <= 65535) {
          EXPECT(spec_accept_sampled_workspace_size(B, D, V, &ws), SV_OK);
          EXPECT(spec_accept_sampled(B, D, V, 1.f, (const float*)F, D ? (const float*)F : nullptr,
                                     dr, D ? (const float*)F : nullptr, (const float*)F,
                                     (int32_t*)F, (int32_t*)F, (const int32_t*)F, (int32_t*)F,
                                     fp(1 << 20), ws, nullptr), SV_OK);
        }
      }
  EXPECT(spec_accept_workspace_size(0, 1, 1, &ws), SV_ERR_INVALID);
  EXPECT(spec_accept_workspace_size(1, 64, 1, &ws), SV_ERR_INVALID);
  EXPECT(spec_accept_workspace_size(1, 1, 0, &ws), SV_ERR_INVALID);
  EXPECT(spec_accept_workspace_size(1, 1, 1, nullptr), SV_ERR_INVALID);
  EXPECT(spec_accept(2, 3, 10, (const float*)fp(4), (const int32_t*)F, (int32_t*)F, (int32_t*)F,
                     (int32_t*)F, (const int32_t*)F, (int32_t*)F, F, 1 << 20, nullptr),
         SV_ERR_INVALID);
  EXPECT(spec_accept(2, 3, 10, (const float*)F, nullptr, (int32_t*)F, (int32_t*)F, (int32_t*)F,
                     (const int32_t*)F, (int32_t*)F, F, 1 << 20, nullptr), SV_ERR_INVALID);
  EXPECT(spec_accept_sampled(2, 3, 10, 0.f, (const float*)F, (const float*)F, (const int32_t*)F,
                             (const float*)F, (const float*)F, (int32_t*)F, (int32_t*)F,
                             (const int32_t*)F, (int32_t*)F, F, 1 << 20, nullptr), SV_ERR_INVALID);
}

static void append_signals_ceilings() {
  sv_append_params a;
  std::memset(&a, 0, sizeof(a));
  a.batch = 4; a.num_new = 16; a.num_kv_heads = 8; a.head_dim = 128; a.block_size = 16;
  a.max_blocks_per_seq = 64; a.num_blocks = 256; a.kv_dtype = SV_KV_BF16;
  EXPECT(spec_kv_append(&a, F, F, F, F, nullptr, nullptr, (const int32_t*)F, (const int32_t*)F,
                        (int32_t*)F, nullptr), SV_OK);
  EXPECT(spec_kv_commit_tree(&a, F, F, F, F, nullptr, nullptr, (const int32_t*)F,
                             (const int32_t*)F, (const int32_t*)F, nullptr), SV_OK);
  a.kv_dtype = SV_KV_FP8_E4M3;
  EXPECT(spec_kv_append(&a, F, F, F, F, nullptr, nullptr, (const int32_t*)F, (const int32_t*)F,
                        (int32_t*)F, nullptr), SV_ERR_INVALID);
  a.num_new = 65;
  EXPECT(spec_kv_commit_tree(&a, F, F, F, F, (float*)F, (float*)F, (const int32_t*)F,
                             (const int32_t*)F, (const int32_t*)F, nullptr), SV_ERR_INVALID);
  EXPECT(spec_kv_append(nullptr, F, F, F, F, nullptr, nullptr, (const int32_t*)F,
                        (const int32_t*)F, (int32_t*)F, nullptr), SV_ERR_INVALID);
  size_t ws = 0;
  EXPECT(spec_draft_signals_workspace_size(32, 128256, &ws), SV_OK);
  EXPECT(spec_draft_signals(32, 128256, 1.f, (const float*)F, (float*)F, (float*)F, (int32_t*)F,
                            15, 0.05f, 8, F, ws, nullptr), SV_OK);
  EXPECT(spec_draft_signals(32, 128256, 1.f, (const float*)F, (float*)F, (float*)F, (int32_t*)F,
                            14, 0.05f, 200, F, ws, nullptr), SV_ERR_INVALID);
  for (int s = -1; s < 7; ++s) (void)std::strlen(sv_status_string((sv_status)s));
  EXPECT(sv_abi_version(), SV_ABI_VERSION);
  float* sink = (float*)F;
  EXPECT(sv_ceiling_read(F, 1 << 20, 64, sink, nullptr), SV_OK);
  EXPECT(sv_ceiling_read(F, 1000, 64, sink, nullptr), SV_ERR_INVALID);
  EXPECT(sv_ceiling_mfma_bf16(64, 16, sink, nullptr), SV_OK);
  EXPECT(sv_ceiling_exp2(0, 16, sink, nullptr), SV_ERR_INVALID);
}

int main() {
  attention();
  acceptance();
  append_signals_ceilings();
  // the error message is per thread: concurrent failing and passing calls
  std::vector<std::thread> th;
  for (int t = 0; t < 8; ++t)
    th.emplace_back([t] {
      size_t ws;
      for (int i = 0; i < 200; ++i) {
        if ((i + t) % 2) {
          EXPECT(spec_accept_workspace_size(0, 1, 1, &ws), SV_ERR_INVALID);
          if (std::strstr(sv_last_error(), "batch") == nullptr) ++g_fail;
        } else {
          EXPECT(spec_accept_workspace_size(4, 3, 100, &ws), SV_OK);
        }
      }
    });
  for (auto& x : th) x.join();
  std::printf("%s (%d failures)\n", g_fail ? "FAILED" : "ok", g_fail);
  return g_fail ? 1 : 0;
}
