// Work split and workspace layout of spec_verify_attn (host code only, no HIP
// calls): which kernel family runs, how many workgroups, and where the split
// or stream-K partial results go in the caller's workspace.
#include "sv_attn_plan.h"

namespace sv {

void plan_attention(AttnPlan& p, int split_request) {
  p.sk_rows = 0;
  p.sk_wgs = 0;
  p.G = p.H_q / p.H_kv;
  p.M = p.G * p.R;
  // Batches up to kStreamMaxBatch go through the stream-K ring whatever M is:
  // waves beyond M still move their share of every tile (the K/V stream, not
  // the MFMA work, sets the pace when few rows share a KV head).  bf16 units
  // hold 128 rows (4 waves, two workgroups per CU) or, for 129 .. 255 rows per
  // KV head, 256 rows (8 waves, one workgroup per CU), so that those rows
  // stream their K and V once instead of twice.  From 256 rows on, the 128-row
  // units of a KV head run on one XCD at the same time (ranges numbered XCD by
  // XCD) and share its K/V through L2, and two 4-wave workgroups per CU hide
  // latency better (measured); below 256 the second unit would be partly
  // empty, and stream-K, which balances tiles, would give its light ranges the
  // same share.  e4m3 units hold 128.
  p.streamk = p.B <= kStreamMaxBatch;
  const int waves_needed = (p.M + kRowsPerWave - 1) / kRowsPerWave;
  if (p.streamk)
    p.waves = (!p.fp8 && p.M > kStreamRows && p.M < 2 * kStreamRows) ? 8 : 4;
  else
    p.waves = waves_needed > 2 ? 4 : waves_needed;
  p.m_tiles = (p.M + kRowsPerWave * p.waves - 1) / (kRowsPerWave * p.waves);
  if (p.streamk) {
    // one split per unit as far as the row context goes; ranges come from min_tiles
    p.split_tokens = (p.max_kv_len + kAttnTile - 1) / kAttnTile * kAttnTile;
    p.s_max = 1;
    p.sk_rows = p.waves * kRowsPerWave;
    p.sk_wgs = p.waves == 8 ? kStreamCUs : kStreamCUs * kStreamWPE;
    p.min_tiles = (split_request > 0 ? split_request : kStreamDefaultMinKeys) /
                  (p.fp8 ? kSk8Keys : kSkKeys);
    const size_t slots = (size_t)p.sk_wgs * 2 * p.sk_rows;
    p.ws_meta_offset = 0;
    const size_t meta_bytes = ((size_t)(p.B + 3) * sizeof(int) + 255) / 256 * 256;
    p.ws_o_bytes = slots * p.hd * sizeof(uint16_t);   // fp16 O / (l f)
    p.ws_ml_offset = meta_bytes + p.ws_o_bytes;
    p.ws_f_offset = p.ws_ml_offset + slots * 2 * sizeof(float);   // (m, l) pairs
    p.ws_bytes = p.ws_f_offset + slots * sizeof(float);
    return;
  }
  int split = split_request;
  if (split <= 0) {
    // Aim at roughly 2048 workgroups for the longest sequences (8 per compute
    // unit) so ragged lengths still fill the chip, with splits of >= 256 keys.
    const long long units = (long long)p.B * p.H_kv * p.m_tiles;
    long long per_unit = units >= 2048 ? 1 : (2048 + units - 1) / units;
    long long s = (p.max_kv_len + per_unit - 1) / per_unit;
    s = ((s + kAttnTile - 1) / kAttnTile) * kAttnTile;
    if (s < 256) s = 256;
    split = (int)s;
  }
  p.split_tokens = split;
  p.s_max = (p.max_kv_len + split - 1) / split;
  p.ws_meta_offset = 0;
  if (p.s_max <= 1) {
    p.ws_o_bytes = p.ws_ml_offset = p.ws_bytes = 0;
    return;
  }
  const size_t rows = (size_t)p.B * p.H_kv * p.s_max * p.M;
  p.ws_o_bytes = rows * p.hd * sizeof(float);
  p.ws_ml_offset = (p.ws_o_bytes + 255) / 256 * 256;
  p.ws_bytes = p.ws_ml_offset + rows * 2 * sizeof(float);   // (m, l) pairs
}

}  // namespace sv
