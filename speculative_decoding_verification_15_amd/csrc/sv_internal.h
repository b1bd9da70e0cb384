// Host-side interface between the C ABI layer (sv_api.cpp) and the kernel
// launchers (attention: sv_attn_plan.h; acceptance, sampled acceptance and KV
// append below).  Arguments reaching these launchers
// have already been validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "sv_attn_plan.h"

namespace sv {

constexpr int kArgmaxThreads = 256;
constexpr int kArgmaxChunk = kArgmaxThreads * 4 * 4;  // logits per workgroup

inline int argmax_chunks(int vocab) { return (vocab + kArgmaxChunk - 1) / kArgmaxChunk; }
inline size_t accept_workspace_bytes(int B, int D, int V) {
  return (size_t)B * (size_t)(D + 1) * (size_t)argmax_chunks(V) * 8u;
}

// spec_accept_noalloc: the library's fixed device array for the chunk results
// (4 MiB per device); `ptr` receives this device's address of it.
constexpr size_t kAcceptScratchBytes = 4u << 20;
hipError_t accept_scratch(void** ptr);

hipError_t launch_accept(int B, int D, int V, const float* logits, const int32_t* draft,
                         int32_t* target, int32_t* accept_len, int32_t* out_tokens,
                         const int32_t* kv_in, int32_t* kv_out, void* ws, hipStream_t stream);

// Draft-tree acceptance: same argmax workspace as greedy acceptance (R = 1 + D rows).
hipError_t launch_accept_tree(int B, int R, int V, const float* logits, const int32_t* tokens,
                              const int32_t* parents, int32_t* target, int32_t* accept_len,
                              int32_t* out_tokens, int32_t* accept_path, const int32_t* kv_in,
                              int32_t* kv_out, void* ws, hipStream_t stream);

// Stochastic acceptance: one (max, fp64 sum) record of 16 bytes per 4096-logit
// chunk of every target row (B (1 + D)) and draft row (B D); a 32-byte draw
// record per sequence; two fp64 weight sums per chunk of each sequence's drawn row.
inline size_t accept_sampled_workspace_bytes(int B, int D, int V) {
  const size_t chunks = (size_t)argmax_chunks(V);
  return (size_t)B * (size_t)(2 * D + 1) * chunks * 16u + (size_t)B * 32u + (size_t)B * chunks * 16u;
}

hipError_t launch_accept_sampled(int B, int D, int V, float tau, const float* zt, const float* zd,
                                 const int32_t* draft, const float* u_accept,
                                 const float* u_sample, int32_t* accept_len, int32_t* out_tokens,
                                 const int32_t* kv_in, int32_t* kv_out, void* ws,
                                 hipStream_t stream);

// Draft signals (sv_draft.hip): one 32-byte record per 4096-logit chunk of every row.
size_t draft_signals_workspace_bytes(int rows, int V);
hipError_t launch_draft_signals(int rows, int V, float tau, const float* logits,
                                float* confidence, float* entropy, int32_t* next_len,
                                int max_draft_len, float rho, int G, void* ws,
                                hipStream_t stream);

// KV append (sv_append.hip): one workgroup per sequence.
struct AppendPlan {
  int B, R, H_kv, hd, max_blocks, num_blocks;
  bool fp8;
};

hipError_t launch_kv_append(const AppendPlan& plan, const void* k_new, const void* v_new,
                            void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                            const int32_t* table, const int32_t* kv_in, int32_t* kv_out,
                            const int32_t* path, hipStream_t stream);

// Machine ceilings (sv_ceil.hip, C header sv_ceilings.h).
hipError_t launch_ceiling_read(const void* src, size_t bytes, int wgs, float* sink,
                               hipStream_t stream);
hipError_t launch_ceiling_mfma(int wgs, int iters, float* sink, hipStream_t stream);
hipError_t launch_ceiling_exp2(int wgs, int iters, float* sink, hipStream_t stream);

}  // namespace sv
