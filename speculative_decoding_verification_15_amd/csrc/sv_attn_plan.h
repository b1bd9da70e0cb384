// Host-side plan (sv_plan.cpp) and launcher (sv_attn.hip) of spec_verify_attn,
// shared with the C ABI layer.  Arguments reaching them have been validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sv {

// Keys per attention tile iteration; split boundaries are multiples of it.
constexpr int kAttnTile = 64;
// Batches up to this size take the stream-K path (its prefix table lives in LDS).
constexpr int kStreamMaxBatch = 2048;
// Query rows per wave (one 32-wide MFMA operand).
constexpr int kRowsPerWave = 32;
// Stream-K: rows per unit of 4 waves x 32 (8-wave units: 256), keys per tile
// of the bf16 kernel and of the e4m3 kernel.
constexpr int kStreamRows = 128;
constexpr int kSkKeys = 32;
constexpr int kSk8Keys = 64;
// Stream-K grid: workgroups per CU (4-wave units), MI355X compute units, and
// the least keys per workgroup range.
#ifndef SV_STREAM_WPE
#define SV_STREAM_WPE 2
#endif
constexpr int kStreamWPE = SV_STREAM_WPE;
constexpr int kStreamCUs = 256;
constexpr int kStreamDefaultMinKeys = 512;

struct AttnPlan {
  int B, R, H_q, H_kv, G, M, hd;
  int max_blocks, num_blocks, max_kv_len;
  bool fp8;
  float sm_scale;
  int split_tokens;  // keys per split (multiple of kAttnTile)
  int s_max;         // ceil(max_kv_len / split_tokens)
  int waves;         // waves per workgroup (each owns 32 query rows)
  int m_tiles;       // ceil(M / (32 * waves))
  // stream-K path (bf16 cache, 128-row tiles): persistent workgroups, the least
  // number of 64-key tiles per workgroup, and the metadata block in the workspace
  bool streamk;
  int sk_wgs, min_tiles;
  int sk_rows;       // rows per stream-K unit: 32 per wave, 4 or 8 waves
  size_t ws_meta_offset;
  size_t ws_o_bytes, ws_ml_offset, ws_bytes;
  size_t ws_f_offset;  // stream-K: per-slot-row power-of-two factors
};

struct AttnPtrs {
  const void* q;
  const void* k;
  const void* v;
  const float* k_scale;
  const float* v_scale;
  const int32_t* block_table;
  const int32_t* kv_lens;
  void* out;
  void* ws;
  const uint64_t* tree_mask;  // NULL: causal chain; else [B][R] ancestor masks
};

// Fills split/grid/workspace fields of `plan` from its shape fields.
void plan_attention(AttnPlan& plan, int split_tokens_request);
hipError_t launch_attention(const AttnPlan& plan, const AttnPtrs& ptrs, hipStream_t stream);

}  // namespace sv
