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
  // hold 256 rows (8 waves, one workgroup per CU) for 129 .. 255 rows per KV
  // head, so that those rows stream their K and V once instead of twice, and
  // past 256 rows whenever they pad the rows to no more than 128-row units do
  // (M a multiple of 256, or M mod 256 above 128): the 8-wave loop (segment
  // tests off the per-tile path) then runs faster than two 4-wave workgroups
  // (MQA with 512, 1024, 1536 and 2048 rows: 56.0 -> 55.4, 90.8 -> 84.7, 125.1
  // -> 117.3 and 149.2 -> 144.8 us), while 1088 rows in 256-row units
  // measured 88.3 -> 91.5 us.  Otherwise units hold 128 rows (4 waves, two
  // workgroups per CU), also at exactly 256 rows (MQA: 43.8 against 44.0
  // us).  The units of a KV head run on one XCD at the same time (ranges
  // numbered XCD by XCD) and share its K/V through L2.  e4m3 units hold 128.
  p.streamk = p.B <= kStreamMaxBatch;
  const int waves_needed = (p.M + kRowsPerWave - 1) / kRowsPerWave;
  const bool pads_as_128 = p.M % (2 * kStreamRows) == 0 || p.M % (2 * kStreamRows) > kStreamRows;
  if (p.streamk)
    p.waves = (!p.fp8 && p.M > kStreamRows && p.M != 2 * kStreamRows && pads_as_128) ? 8 : 4;
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
