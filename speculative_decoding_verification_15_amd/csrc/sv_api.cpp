// C ABI entry points (include/spec_verify.h): argument checks, workspace
// sizing and dispatch to the gfx950 kernels.  Every check the host can make
// runs before the first HIP call, so invalid calls return an error without
// touching the device.
#include "spec_verify.h"
#include "sv_ceilings.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "sv_internal.h"

namespace {

thread_local char g_err[512] = "";

sv_status fail(sv_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr int kMaxDraft = 63;
constexpr int kMaxGridYZ = 65535;

// Validates the shape in `p` and fills `plan`.  No pointer is looked at.
sv_status make_attn_plan(const sv_attn_params* p, sv::AttnPlan& plan) {
  if (!p) return fail(SV_ERR_INVALID, "params is NULL");
  if (p->batch < 1) return fail(SV_ERR_INVALID, "batch must be >= 1 (got %d)", p->batch);
  if (p->draft_len < 0 || p->draft_len > kMaxDraft)
    return fail(SV_ERR_INVALID, "draft_len must be in [0, %d] (got %d)", kMaxDraft, p->draft_len);
  if (p->num_q_heads < 1 || p->num_kv_heads < 1)
    return fail(SV_ERR_INVALID, "head counts must be >= 1 (H_q=%d, H_kv=%d)", p->num_q_heads,
                p->num_kv_heads);
  if (p->num_q_heads % p->num_kv_heads != 0)
    return fail(SV_ERR_INVALID, "num_q_heads (%d) must be a multiple of num_kv_heads (%d)",
                p->num_q_heads, p->num_kv_heads);
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(SV_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", p->head_dim);
  if (p->block_size != 16)
    return fail(SV_ERR_UNSUPPORTED, "block_size must be 16 (got %d)", p->block_size);
  if (p->kv_dtype != SV_KV_BF16 && p->kv_dtype != SV_KV_FP8_E4M3)
    return fail(SV_ERR_INVALID, "unknown kv_dtype %d", p->kv_dtype);
  if (!(p->sm_scale > 0.f) || !std::isfinite(p->sm_scale))
    return fail(SV_ERR_INVALID, "sm_scale must be finite and > 0");
  const int R = p->draft_len + 1;
  if (p->max_kv_len < R)
    return fail(SV_ERR_INVALID, "max_kv_len (%d) must be >= 1 + draft_len (%d)", p->max_kv_len, R);
  if (p->num_blocks < 1) return fail(SV_ERR_INVALID, "num_blocks must be >= 1");
  const long long need_blocks = (p->max_kv_len + 15LL) / 16;
  if (p->max_blocks_per_seq < need_blocks)
    return fail(SV_ERR_INVALID, "max_blocks_per_seq (%d) < ceil(max_kv_len / 16) (%lld)",
                p->max_blocks_per_seq, need_blocks);
  if (p->split_tokens < 0 || p->split_tokens % sv::kAttnTile != 0)
    return fail(SV_ERR_INVALID, "split_tokens must be 0 or a positive multiple of %d (got %d)",
                sv::kAttnTile, p->split_tokens);
  // index arithmetic inside the kernels uses 32-bit row counts
  const long long q_elems = (long long)p->batch * R * p->num_q_heads * p->head_dim;
  if (q_elems >= (1LL << 31)) return fail(SV_ERR_UNSUPPORTED, "q/out larger than 2^31 elements");
  // ... and 32-bit block strides and scale indices
  if ((long long)p->num_kv_heads * p->head_dim * 32 >= (1LL << 31))
    return fail(SV_ERR_UNSUPPORTED, "a cache block of num_kv_heads * head_dim * 32 bytes is 2^31 or more");
  if ((long long)p->num_blocks * p->num_kv_heads >= (1LL << 32))
    return fail(SV_ERR_UNSUPPORTED, "num_blocks * num_kv_heads must be below 2^32");

  plan = sv::AttnPlan{};
  plan.B = p->batch;
  plan.R = R;
  plan.H_q = p->num_q_heads;
  plan.H_kv = p->num_kv_heads;
  plan.hd = p->head_dim;
  plan.max_blocks = p->max_blocks_per_seq;
  plan.num_blocks = p->num_blocks;
  plan.max_kv_len = p->max_kv_len;
  plan.fp8 = p->kv_dtype == SV_KV_FP8_E4M3;
  plan.sm_scale = p->sm_scale;
  sv::plan_attention(plan, p->split_tokens);
  const long long units = (long long)plan.s_max * plan.B * plan.H_kv;
  if (((units + 7) / 8) * 8 * plan.m_tiles >= (1LL << 31))
    return fail(SV_ERR_UNSUPPORTED, "too many workgroups for one launch");
  const long long ws_rows = (long long)plan.B * plan.H_kv * plan.s_max * plan.M;
  if (ws_rows >= (1LL << 31)) return fail(SV_ERR_UNSUPPORTED, "split workspace too large");
  if (plan.streamk) {
    // the stream-K work list counts 32-key tiles of every unit in int32
    const long long tiles = (long long)plan.B * plan.H_kv * plan.m_tiles *
                            ((plan.max_kv_len + 31LL) / 32);
    if (tiles >= (1LL << 31))
      return fail(SV_ERR_UNSUPPORTED, "%lld key tiles in one call (batch * num_kv_heads * row tiles "
                  "* ceil(max_kv_len / 32)) exceed the 2^31 the work list can count", tiles);
  }
  return SV_OK;
}

}  // namespace

extern "C" {

sv_status spec_verify_attn_workspace_size(const sv_attn_params* p, size_t* bytes) {
  if (!bytes) return fail(SV_ERR_INVALID, "bytes is NULL");
  sv::AttnPlan plan;
  sv_status s = make_attn_plan(p, plan);
  if (s != SV_OK) return s;
  *bytes = plan.ws_bytes;
  return SV_OK;
}

static sv_status run_attn(const sv_attn_params* p, const void* q, const void* k_cache,
                          const void* v_cache, const float* k_scale, const float* v_scale,
                          const int32_t* block_table, const int32_t* kv_lens,
                          const uint64_t* tree_mask, void* out, void* workspace,
                          size_t workspace_bytes, void* stream) {
  sv::AttnPlan plan;
  sv_status s = make_attn_plan(p, plan);
  if (s != SV_OK) return s;
  if (!q || !k_cache || !v_cache || !block_table || !kv_lens || !out)
    return fail(SV_ERR_INVALID, "a required pointer is NULL");
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16))
    return fail(SV_ERR_INVALID, "q, k_cache, v_cache and out must be 16-byte aligned");
  if (!aligned(block_table, 4) || !aligned(kv_lens, 4))
    return fail(SV_ERR_INVALID, "block_table and kv_lens must be 4-byte aligned");
  if (plan.fp8) {
    if (!k_scale || !v_scale) return fail(SV_ERR_INVALID, "e4m3 caches need k_scale and v_scale");
    if (!aligned(k_scale, 4) || !aligned(v_scale, 4))
      return fail(SV_ERR_INVALID, "k_scale and v_scale must be 4-byte aligned");
  } else if (k_scale || v_scale) {
    return fail(SV_ERR_INVALID, "k_scale and v_scale must be NULL for bf16 caches");
  }
  if (tree_mask && !aligned(tree_mask, 8))
    return fail(SV_ERR_INVALID, "tree_mask must be 8-byte aligned");
  if (plan.ws_bytes > 0) {
    if (!workspace) return fail(SV_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", plan.ws_bytes);
    if (workspace_bytes < plan.ws_bytes)
      return fail(SV_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", workspace_bytes,
                  plan.ws_bytes);
    if (!aligned(workspace, 256)) return fail(SV_ERR_INVALID, "workspace must be 256-byte aligned");
  }
  sv::AttnPtrs ptrs{q, k_cache, v_cache, k_scale, v_scale, block_table, kv_lens, out, workspace,
                    tree_mask};
  hipError_t e = sv::launch_attention(plan, ptrs, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SV_ERR_LAUNCH, "launch failed: %s", hipGetErrorString(e));
  g_err[0] = '\0';
  return SV_OK;
}

sv_status spec_verify_attn(const sv_attn_params* p, const void* q, const void* k_cache,
                           const void* v_cache, const float* k_scale, const float* v_scale,
                           const int32_t* block_table, const int32_t* kv_lens, void* out,
                           void* workspace, size_t workspace_bytes, void* stream) {
  return run_attn(p, q, k_cache, v_cache, k_scale, v_scale, block_table, kv_lens, nullptr, out,
                  workspace, workspace_bytes, stream);
}

sv_status spec_verify_attn_tree(const sv_attn_params* p, const void* q, const void* k_cache,
                                const void* v_cache, const float* k_scale, const float* v_scale,
                                const int32_t* block_table, const int32_t* kv_lens,
                                const uint64_t* tree_mask, void* out, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (!tree_mask) return fail(SV_ERR_INVALID, "tree_mask is NULL");
  return run_attn(p, q, k_cache, v_cache, k_scale, v_scale, block_table, kv_lens, tree_mask, out,
                  workspace, workspace_bytes, stream);
}

static sv_status check_accept_shape(int32_t batch, int32_t draft_len, int32_t vocab) {
  if (batch < 1) return fail(SV_ERR_INVALID, "batch must be >= 1 (got %d)", batch);
  if (draft_len < 0 || draft_len > kMaxDraft)
    return fail(SV_ERR_INVALID, "draft_len must be in [0, %d] (got %d)", kMaxDraft, draft_len);
  if (vocab < 1) return fail(SV_ERR_INVALID, "vocab must be >= 1 (got %d)", vocab);
  const long long rows = (long long)batch * (draft_len + 1);
  if (rows > kMaxGridYZ) return fail(SV_ERR_UNSUPPORTED, "batch * (1 + draft_len) > %d", kMaxGridYZ);
  if (batch > 2147483647 / 64) return fail(SV_ERR_UNSUPPORTED, "batch too large");
  return SV_OK;
}

sv_status spec_accept_workspace_size(int32_t batch, int32_t draft_len, int32_t vocab,
                                     size_t* bytes) {
  if (!bytes) return fail(SV_ERR_INVALID, "bytes is NULL");
  sv_status s = check_accept_shape(batch, draft_len, vocab);
  if (s != SV_OK) return s;
  *bytes = sv::accept_workspace_bytes(batch, draft_len, vocab);
  return SV_OK;
}

sv_status spec_accept(int32_t batch, int32_t draft_len, int32_t vocab, const float* logits,
                      const int32_t* draft, int32_t* target_tokens, int32_t* accept_len,
                      int32_t* out_tokens, const int32_t* kv_lens_in, int32_t* kv_lens_out,
                      void* workspace, size_t workspace_bytes, void* stream) {
  sv_status s = check_accept_shape(batch, draft_len, vocab);
  if (s != SV_OK) return s;
  if (!logits || !target_tokens || !accept_len || !out_tokens || !kv_lens_in || !kv_lens_out)
    return fail(SV_ERR_INVALID, "a required pointer is NULL");
  if (draft_len > 0 && !draft) return fail(SV_ERR_INVALID, "draft is NULL with draft_len > 0");
  if (!aligned(logits, 16)) return fail(SV_ERR_INVALID, "logits must be 16-byte aligned");
  if (!aligned(target_tokens, 4) || !aligned(accept_len, 4) || !aligned(out_tokens, 4) ||
      !aligned(kv_lens_in, 4) || !aligned(kv_lens_out, 4) || (draft && !aligned(draft, 4)))
    return fail(SV_ERR_INVALID, "int32 arrays must be 4-byte aligned");
  const size_t need = sv::accept_workspace_bytes(batch, draft_len, vocab);
  if (!workspace) return fail(SV_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", need);
  if (workspace_bytes < need)
    return fail(SV_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", workspace_bytes, need);
  if (!aligned(workspace, 256)) return fail(SV_ERR_INVALID, "workspace must be 256-byte aligned");
  hipError_t e = sv::launch_accept(batch, draft_len, vocab, logits, draft, target_tokens,
                                   accept_len, out_tokens, kv_lens_in, kv_lens_out, workspace,
                                   static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SV_ERR_LAUNCH, "launch failed: %s", hipGetErrorString(e));
  g_err[0] = '\0';
  return SV_OK;
}

sv_status spec_accept_noalloc(int32_t batch, int32_t draft_len, int32_t vocab, const float* logits,
                              const int32_t* draft, int32_t* target_tokens, int32_t* accept_len,
                              int32_t* out_tokens, const int32_t* kv_lens_in,
                              int32_t* kv_lens_out, void* stream) {
  sv_status s = check_accept_shape(batch, draft_len, vocab);
  if (s != SV_OK) return s;
  if (!logits || !target_tokens || !accept_len || !out_tokens || !kv_lens_in || !kv_lens_out)
    return fail(SV_ERR_INVALID, "a required pointer is NULL");
  if (draft_len > 0 && !draft) return fail(SV_ERR_INVALID, "draft is NULL with draft_len > 0");
  if (!aligned(logits, 16)) return fail(SV_ERR_INVALID, "logits must be 16-byte aligned");
  if (!aligned(target_tokens, 4) || !aligned(accept_len, 4) || !aligned(out_tokens, 4) ||
      !aligned(kv_lens_in, 4) || !aligned(kv_lens_out, 4) || (draft && !aligned(draft, 4)))
    return fail(SV_ERR_INVALID, "int32 arrays must be 4-byte aligned");
  const size_t need = sv::accept_workspace_bytes(batch, draft_len, vocab);
  if (need > sv::kAcceptScratchBytes)
    return fail(SV_ERR_UNSUPPORTED, "batch %d, draft_len %d, vocab %d need %zu bytes of scratch "
                "(8 per 4096-logit chunk of every row); the fixed array holds %zu", batch,
                draft_len, vocab, need, sv::kAcceptScratchBytes);
  void* scratch = nullptr;
  hipError_t e = sv::accept_scratch(&scratch);
  if (e != hipSuccess)
    return fail(SV_ERR_LAUNCH, "scratch set-up failed: %s", hipGetErrorString(e));
  e = sv::launch_accept(batch, draft_len, vocab, logits, draft, target_tokens, accept_len,
                        out_tokens, kv_lens_in, kv_lens_out, scratch,
                        static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SV_ERR_LAUNCH, "launch failed: %s", hipGetErrorString(e));
  g_err[0] = '\0';
  return SV_OK;
}

sv_status spec_accept_tree(int32_t batch, int32_t draft_len, int32_t vocab, const float* logits,
                           const int32_t* tokens, const int32_t* parents, int32_t* target_tokens,
                           int32_t* accept_len, int32_t* out_tokens, int32_t* accept_path,
                           const int32_t* kv_lens_in, int32_t* kv_lens_out, void* workspace,
                           size_t workspace_bytes, void* stream) {
  sv_status s = check_accept_shape(batch, draft_len, vocab);
  if (s != SV_OK) return s;
  if (!logits || !target_tokens || !accept_len || !out_tokens || !accept_path || !kv_lens_in ||
      !kv_lens_out)
    return fail(SV_ERR_INVALID, "a required pointer is NULL");
  if (draft_len > 0 && (!tokens || !parents))
    return fail(SV_ERR_INVALID, "tokens and parents are required with draft_len > 0");
  if (!aligned(logits, 16)) return fail(SV_ERR_INVALID, "logits must be 16-byte aligned");
  if (!aligned(target_tokens, 4) || !aligned(accept_len, 4) || !aligned(out_tokens, 4) ||
      !aligned(accept_path, 4) || !aligned(kv_lens_in, 4) || !aligned(kv_lens_out, 4) ||
      (tokens && !aligned(tokens, 4)) || (parents && !aligned(parents, 4)))
    return fail(SV_ERR_INVALID, "int32 arrays must be 4-byte aligned");
  const size_t need = sv::accept_workspace_bytes(batch, draft_len, vocab);
  if (!workspace) return fail(SV_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", need);
  if (workspace_bytes < need)
    return fail(SV_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", workspace_bytes, need);
  if (!aligned(workspace, 256)) return fail(SV_ERR_INVALID, "workspace must be 256-byte aligned");
  hipError_t e = sv::launch_accept_tree(batch, draft_len + 1, vocab, logits, tokens, parents,
                                        target_tokens, accept_len, out_tokens, accept_path,
                                        kv_lens_in, kv_lens_out, workspace,
                                        static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SV_ERR_LAUNCH, "launch failed: %s", hipGetErrorString(e));
  g_err[0] = '\0';
  return SV_OK;
}

static sv_status check_sampled_shape(int32_t batch, int32_t draft_len, int32_t vocab,
                                     float temperature) {
  sv_status s = check_accept_shape(batch, draft_len, vocab);
  if (s != SV_OK) return s;
  if (!(temperature > 0.f) || !std::isfinite(temperature))
    return fail(SV_ERR_INVALID, "temperature must be finite and > 0");
  const long long rows = (long long)batch * (2 * draft_len + 1);
  if (rows > kMaxGridYZ)
    return fail(SV_ERR_UNSUPPORTED, "batch * (1 + 2 draft_len) > %d", kMaxGridYZ);
  return SV_OK;
}

sv_status spec_accept_sampled_workspace_size(int32_t batch, int32_t draft_len, int32_t vocab,
                                             size_t* bytes) {
  if (!bytes) return fail(SV_ERR_INVALID, "bytes is NULL");
  sv_status s = check_sampled_shape(batch, draft_len, vocab, 1.f);
  if (s != SV_OK) return s;
  *bytes = sv::accept_sampled_workspace_bytes(batch, draft_len, vocab);
  return SV_OK;
}

sv_status spec_accept_sampled(int32_t batch, int32_t draft_len, int32_t vocab, float temperature,
                              const float* target_logits, const float* draft_logits,
                              const int32_t* draft, const float* u_accept, const float* u_sample,
                              int32_t* accept_len, int32_t* out_tokens, const int32_t* kv_lens_in,
                              int32_t* kv_lens_out, void* workspace, size_t workspace_bytes,
                              void* stream) {
  sv_status s = check_sampled_shape(batch, draft_len, vocab, temperature);
  if (s != SV_OK) return s;
  if (!target_logits || !u_sample || !accept_len || !out_tokens || !kv_lens_in || !kv_lens_out)
    return fail(SV_ERR_INVALID, "a required pointer is NULL");
  if (draft_len > 0 && (!draft_logits || !draft || !u_accept))
    return fail(SV_ERR_INVALID, "draft_logits, draft and u_accept are required with draft_len > 0");
  if (!aligned(target_logits, 16) || (draft_logits && !aligned(draft_logits, 16)))
    return fail(SV_ERR_INVALID, "logits must be 16-byte aligned");
  if (!aligned(u_sample, 4) || (u_accept && !aligned(u_accept, 4)))
    return fail(SV_ERR_INVALID, "uniform arrays must be 4-byte aligned");
  if (!aligned(accept_len, 4) || !aligned(out_tokens, 4) || !aligned(kv_lens_in, 4) ||
      !aligned(kv_lens_out, 4) || (draft && !aligned(draft, 4)))
    return fail(SV_ERR_INVALID, "int32 arrays must be 4-byte aligned");
  const size_t need = sv::accept_sampled_workspace_bytes(batch, draft_len, vocab);
  if (!workspace) return fail(SV_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", need);
  if (workspace_bytes < need)
    return fail(SV_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", workspace_bytes, need);
  if (!aligned(workspace, 256)) return fail(SV_ERR_INVALID, "workspace must be 256-byte aligned");
  hipError_t e = sv::launch_accept_sampled(batch, draft_len, vocab, temperature, target_logits,
                                           draft_logits, draft, u_accept, u_sample, accept_len,
                                           out_tokens, kv_lens_in, kv_lens_out, workspace,
                                           static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SV_ERR_LAUNCH, "launch failed: %s", hipGetErrorString(e));
  g_err[0] = '\0';
  return SV_OK;
}

static sv_status run_append(const sv_append_params* p, const void* k_new, const void* v_new,
                            void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                            const int32_t* block_table, const int32_t* kv_lens_in,
                            int32_t* kv_lens_out, const int32_t* path, void* stream) {
  if (!p) return fail(SV_ERR_INVALID, "params is NULL");
  if (p->batch < 1) return fail(SV_ERR_INVALID, "batch must be >= 1 (got %d)", p->batch);
  if (p->num_new < 1) return fail(SV_ERR_INVALID, "num_new must be >= 1 (got %d)", p->num_new);
  if (path && p->num_new > 64)
    return fail(SV_ERR_INVALID, "a tree has at most 64 nodes (num_new = %d)", p->num_new);
  if (p->num_kv_heads < 1) return fail(SV_ERR_INVALID, "num_kv_heads must be >= 1");
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(SV_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", p->head_dim);
  if (p->block_size != 16)
    return fail(SV_ERR_UNSUPPORTED, "block_size must be 16 (got %d)", p->block_size);
  if (p->kv_dtype != SV_KV_BF16 && p->kv_dtype != SV_KV_FP8_E4M3)
    return fail(SV_ERR_INVALID, "unknown kv_dtype %d", p->kv_dtype);
  if (p->num_blocks < 1) return fail(SV_ERR_INVALID, "num_blocks must be >= 1");
  if (p->max_blocks_per_seq < 1 || (long long)p->max_blocks_per_seq * 16 >= (1LL << 31))
    return fail(SV_ERR_INVALID, "max_blocks_per_seq must be in [1, 2^27) (got %d)",
                p->max_blocks_per_seq);
  if ((long long)p->num_new > (long long)p->max_blocks_per_seq * 16)
    return fail(SV_ERR_INVALID, "num_new (%d) exceeds the table's %lld tokens", p->num_new,
                (long long)p->max_blocks_per_seq * 16);
  const bool fp8 = p->kv_dtype == SV_KV_FP8_E4M3;
  if (!k_new || !v_new || !k_cache || !v_cache || !block_table || !kv_lens_in ||
      (!path && !kv_lens_out))
    return fail(SV_ERR_INVALID, "a required pointer is NULL");
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16))
    return fail(SV_ERR_INVALID, "k_new, v_new, k_cache and v_cache must be 16-byte aligned");
  if (!aligned(block_table, 4) || !aligned(kv_lens_in, 4) || (kv_lens_out && !aligned(kv_lens_out, 4)) ||
      (path && !aligned(path, 4)))
    return fail(SV_ERR_INVALID, "block_table, kv_lens and accept_path must be 4-byte aligned");
  if (fp8) {
    if (!k_scale || !v_scale) return fail(SV_ERR_INVALID, "e4m3 caches need k_scale and v_scale");
    if (!aligned(k_scale, 4) || !aligned(v_scale, 4))
      return fail(SV_ERR_INVALID, "k_scale and v_scale must be 4-byte aligned");
  } else if (k_scale || v_scale) {
    return fail(SV_ERR_INVALID, "k_scale and v_scale must be NULL for bf16 caches");
  }
  sv::AppendPlan plan{p->batch, p->num_new, p->num_kv_heads, p->head_dim, p->max_blocks_per_seq,
                      p->num_blocks, fp8};
  hipError_t e = sv::launch_kv_append(plan, k_new, v_new, k_cache, v_cache, k_scale, v_scale,
                                      block_table, kv_lens_in, kv_lens_out, path,
                                      static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SV_ERR_LAUNCH, "launch failed: %s", hipGetErrorString(e));
  g_err[0] = '\0';
  return SV_OK;
}

sv_status spec_kv_append(const sv_append_params* p, const void* k_new, const void* v_new,
                         void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                         const int32_t* block_table, const int32_t* kv_lens_in,
                         int32_t* kv_lens_out, void* stream) {
  return run_append(p, k_new, v_new, k_cache, v_cache, k_scale, v_scale, block_table, kv_lens_in,
                    kv_lens_out, nullptr, stream);
}

sv_status spec_kv_commit_tree(const sv_append_params* p, const void* k_new, const void* v_new,
                              void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                              const int32_t* block_table, const int32_t* accept_path,
                              const int32_t* kv_lens, void* stream) {
  if (!accept_path) return fail(SV_ERR_INVALID, "accept_path is NULL");
  return run_append(p, k_new, v_new, k_cache, v_cache, k_scale, v_scale, block_table, kv_lens,
                    nullptr, accept_path, stream);
}

static sv_status check_draft_signals(int32_t rows, int32_t vocab, float temperature,
                                     int32_t max_draft_len, float rho, int32_t group_size) {
  if (rows < 1 || rows > kMaxGridYZ)
    return fail(SV_ERR_INVALID, "rows must be in [1, %d] (got %d)", kMaxGridYZ, rows);
  if (vocab < 1) return fail(SV_ERR_INVALID, "vocab must be >= 1 (got %d)", vocab);
  if (!(temperature > 0.f) || !std::isfinite(temperature))
    return fail(SV_ERR_INVALID, "temperature must be finite and > 0");
  if (max_draft_len < 0 || max_draft_len > kMaxDraft)
    return fail(SV_ERR_INVALID, "max_draft_len must be in [0, %d] (got %d)", kMaxDraft,
                max_draft_len);
  if (!(rho >= 0.f) || !std::isfinite(rho)) return fail(SV_ERR_INVALID, "rho must be finite and >= 0");
  if (group_size < 0 || group_size > 1024)
    return fail(SV_ERR_INVALID, "group_size must be in [0, 1024] (got %d)", group_size);
  if (group_size > 0) {
    // the tile rule must leave at least one draft length to choose from
    bool any = false;
    for (int d = 0; d <= max_draft_len && !any; ++d) {
      const int rows = group_size * (d + 1);
      any = rows <= 128 || rows % 128 == 0;
    }
    if (!any)
      return fail(SV_ERR_INVALID, "no draft length in [0, %d] passes the tile rule for group_size "
                  "%d (G (1 + D) <= 128 or a multiple of 128)", max_draft_len, group_size);
  }
  return SV_OK;
}

sv_status spec_draft_signals_workspace_size(int32_t rows, int32_t vocab, size_t* bytes) {
  if (!bytes) return fail(SV_ERR_INVALID, "bytes is NULL");
  sv_status s = check_draft_signals(rows, vocab, 1.f, 0, 0.f, 0);
  if (s != SV_OK) return s;
  *bytes = sv::draft_signals_workspace_bytes(rows, vocab);
  return SV_OK;
}

sv_status spec_draft_signals(int32_t rows, int32_t vocab, float temperature,
                             const float* draft_logits, float* confidence, float* entropy,
                             int32_t* next_draft_len, int32_t max_draft_len, float rho,
                             int32_t group_size, void* workspace, size_t workspace_bytes,
                             void* stream) {
  sv_status s = check_draft_signals(rows, vocab, temperature, max_draft_len, rho, group_size);
  if (s != SV_OK) return s;
  if (!draft_logits || !confidence || !entropy)
    return fail(SV_ERR_INVALID, "a required pointer is NULL");
  if (!aligned(draft_logits, 16)) return fail(SV_ERR_INVALID, "draft_logits must be 16-byte aligned");
  if (!aligned(confidence, 4) || !aligned(entropy, 4) ||
      (next_draft_len && !aligned(next_draft_len, 4)))
    return fail(SV_ERR_INVALID, "output arrays must be 4-byte aligned");
  const size_t need = sv::draft_signals_workspace_bytes(rows, vocab);
  if (!workspace) return fail(SV_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", need);
  if (workspace_bytes < need)
    return fail(SV_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", workspace_bytes, need);
  if (!aligned(workspace, 256)) return fail(SV_ERR_INVALID, "workspace must be 256-byte aligned");
  hipError_t e = sv::launch_draft_signals(rows, vocab, temperature, draft_logits, confidence,
                                          entropy, next_draft_len, max_draft_len, rho, group_size,
                                          workspace, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SV_ERR_LAUNCH, "launch failed: %s", hipGetErrorString(e));
  g_err[0] = '\0';
  return SV_OK;
}

static sv_status check_ceiling_grid(int32_t workgroups, int32_t iters, const float* sink) {
  if (workgroups < 1 || workgroups > 65536)
    return fail(SV_ERR_INVALID, "workgroups must be in [1, 65536] (got %d)", workgroups);
  if (iters < 1 || iters > (1 << 20))
    return fail(SV_ERR_INVALID, "iters must be in [1, 2^20] (got %d)", iters);
  if (!sink || !aligned(sink, 4)) return fail(SV_ERR_INVALID, "sink must be a 4-byte aligned pointer");
  return SV_OK;
}

sv_status sv_ceiling_read(const void* src, size_t bytes, int32_t workgroups, float* sink,
                          void* stream) {
  sv_status s = check_ceiling_grid(workgroups, 1, sink);
  if (s != SV_OK) return s;
  if (!src || !aligned(src, 16)) return fail(SV_ERR_INVALID, "src must be a 16-byte aligned pointer");
  if (bytes == 0 || bytes % 16 != 0)
    return fail(SV_ERR_INVALID, "bytes must be a positive multiple of 16 (got %zu)", bytes);
  hipError_t e = sv::launch_ceiling_read(src, bytes, workgroups, sink, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SV_ERR_LAUNCH, "launch failed: %s", hipGetErrorString(e));
  g_err[0] = '\0';
  return SV_OK;
}

sv_status sv_ceiling_mfma_bf16(int32_t workgroups, int32_t iters, float* sink, void* stream) {
  sv_status s = check_ceiling_grid(workgroups, iters, sink);
  if (s != SV_OK) return s;
  hipError_t e = sv::launch_ceiling_mfma(workgroups, iters, sink, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SV_ERR_LAUNCH, "launch failed: %s", hipGetErrorString(e));
  g_err[0] = '\0';
  return SV_OK;
}

sv_status sv_ceiling_exp2(int32_t workgroups, int32_t iters, float* sink, void* stream) {
  sv_status s = check_ceiling_grid(workgroups, iters, sink);
  if (s != SV_OK) return s;
  hipError_t e = sv::launch_ceiling_exp2(workgroups, iters, sink, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SV_ERR_LAUNCH, "launch failed: %s", hipGetErrorString(e));
  g_err[0] = '\0';
  return SV_OK;
}

const char* sv_status_string(sv_status s) {
  switch (s) {
    case SV_OK: return "SV_OK";
    case SV_ERR_INVALID: return "SV_ERR_INVALID: invalid argument";
    case SV_ERR_WORKSPACE: return "SV_ERR_WORKSPACE: workspace missing or too small";
    case SV_ERR_UNSUPPORTED: return "SV_ERR_UNSUPPORTED: configuration not supported";
    case SV_ERR_LAUNCH: return "SV_ERR_LAUNCH: kernel launch failed";
  }
  return "unknown sv_status";
}

const char* sv_last_error(void) { return g_err; }

int32_t sv_abi_version(void) { return SV_ABI_VERSION; }

}  // extern "C"
