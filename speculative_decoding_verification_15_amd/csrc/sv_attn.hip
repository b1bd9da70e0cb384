// Verification attention on gfx950: the R = D + 1 newest positions of every
// sequence attend over the sequence's paged KV cache.
//
// What is computed (C header, spec_verify_attn): for query head h, KV head
// kvh = h / G ("GPU and LLM" ch. 5, section "GQA"), position i,
//     out = softmax(sm_scale * q . K[0 .. L-R+i]) . V[0 .. L-R+i]
// with a running max m and running sum l per query row, rescaling by
// exp(m - m_new) whenever the max grows, and a final division by l ("GPU and
// LLM" ch. 5, section "Online softmax: carry the max and the sum").  Long key
// ranges are cut into splits whose (O, m, l) states are merged by the same rule
// in sv_attn_combine.
//
// Work decomposition.  One workgroup owns (sequence b, KV head kvh, split s,
// row tile).  The M = G * R query rows that read kvh are stacked as
// m = position * G + group-member, so the rows of one KV head are one operand
// of the score product; each wave owns 32 of them.
//
// Scores are computed transposed, S^T[key][row] = K . Q^T, with
// v_mfma_f32_32x32x16_bf16: a lane then holds one query row and 16 keys of a
// 32-key block, so the row max and row sum are in-lane reductions plus one
// exchange between the two 32-lane halves, and the output accumulator
// O^T[d][row] is rescaled with a per-lane factor.  The probabilities leave the
// score accumulator already in the B-operand layout of O^T += V^T . P^T when
// the K rows of a block are fed in the order pi(i) = i with bits 2 and 3
// swapped: then the 8 keys one lane contributes to a PV step are 8 consecutive
// token slots, which the V layout [blk][kvh][hd][16] stores as one 16-byte
// vector per dimension.
//
// Keys past L (poison slots of the last block) have their scores masked to
// -inf and their V values zeroed before the product, so NaN poison cannot
// reach a row.  All softmax arithmetic runs in the log2 domain
// (x = s * sm_scale * log2 e, exp2).
#include "sv_device.h"
#include "sv_internal.h"

namespace sv {

struct AttnArgs {
  const uint16_t* q;
  const uint8_t* k;
  const uint8_t* v;
  const float* k_scale;
  const float* v_scale;
  const int32_t* block_table;
  const int32_t* kv_lens;
  uint16_t* out;
  float* ws_o;    // [B][H_kv][s_max][M][hd] unnormalised O of each split
  f32x2* ws_ml;   // [B][H_kv][s_max][M] (m, l) of each split, log2 domain
  int R, H_q, H_kv, G, M;
  int max_blocks, num_blocks, max_kv_len;
  int split_tokens, s_max;
  float c;        // sm_scale * log2(e)
};

// Row i of the 32-key score block holds key pi(i) of that block.
__device__ __forceinline__ int key_of_row(int i) {
  return (i & 0x13) | ((i & 4) << 1) | ((i & 8) >> 1);
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  __bf16 b = (__bf16)x;
  return __builtin_bit_cast(uint16_t, b);
}

template <int HD, bool FP8>
struct KV {
  static constexpr int kElem = FP8 ? 1 : 2;
  static constexpr size_t kBlockBytes = (size_t)HD * 16 * kElem;  // one (block, head)
};

template <int HD, bool FP8, int NW>
__global__ __launch_bounds__(kWave * NW) void sv_attn_partial(AttnArgs a) {
  constexpr int KS = HD / 16;   // k-steps of the score product
  constexpr int DB = HD / 32;   // 32-wide blocks of the output dims
  using KVT = KV<HD, FP8>;

  const int split = blockIdx.x;
  const int kvh = blockIdx.y % a.H_kv;
  const int mt = blockIdx.y / a.H_kv;
  const int b = blockIdx.z;
  const int L = min(max(a.kv_lens[b], 0), a.max_kv_len);
  const int n_splits = (L + a.split_tokens - 1) / a.split_tokens;
  if (split >= n_splits) return;
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int m0 = (mt * NW + wave) * kRowsPerWave;
  if (m0 >= a.M) return;

  const int ql = lane & 31;   // query row within the wave (B/C column)
  const int hh = lane >> 5;   // half of the wave
  const int m = m0 + ql;
  const bool row_ok = m < a.M;
  const int pos = row_ok ? m / a.G : a.R - 1;
  const int head = kvh * a.G + (row_ok ? m % a.G : 0);
  const int P = L - a.R;               // context before the new positions
  const int vis_last = P + pos;        // last key this row may see
  const int k_begin = split * a.split_tokens;
  const int k_end = min(k_begin + a.split_tokens, L);

  // Q^T operand: lane (row ql, half hh) supplies 8 dims per k-step.
  bf16x8 qop[KS];
  {
    const uint16_t* qrow = a.q + ((size_t)(b * a.R + pos) * a.H_q + head) * HD;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      // bf16 K vectors hold 8 dims: k-step ks, half hh reads dims 16ks + 8hh.
      // e4m3 K vectors hold 16 dims and serve two k-steps: k-step 2c + e, half
      // hh reads dims 16(2c + hh) + 8e.
      const int d0 = FP8 ? (32 * (ks / 2) + 16 * hh + 8 * (ks % 2)) : (16 * ks + 8 * hh);
      bf16x8 z = {};
      qop[ks] = row_ok ? *reinterpret_cast<const bf16x8*>(qrow + d0) : z;
    }
  }

  const int32_t* tbl = a.block_table + (size_t)b * a.max_blocks;
  const int n_blk_seq = (L + 15) / 16;
  auto phys = [&](int logical) -> size_t {
    int j = min(logical, n_blk_seq - 1);
    int p = tbl[j];
    p = min(max(p, 0), a.num_blocks - 1);
    return (size_t)p;
  };

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  float m_run = -INFINITY;   // running max (log2 domain), same in both halves
  float l_run = 0.f;         // running sum over this lane's keys only

  const int krow = key_of_row(ql);   // key (within the 32-key block) of A-row ql

  for (int kt = k_begin; kt < k_end; kt += kAttnTile) {
    f32x16 x[2];
    size_t blk[2][2];
    bool live[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const int t0 = kt + 32 * sb;
      live[sb] = t0 < k_end;
      blk[sb][0] = phys(t0 / 16);
      blk[sb][1] = phys(t0 / 16 + 1);
      x[sb] = f32x16{};
      if (!live[sb]) continue;
      const uint8_t* kb = a.k + (blk[sb][krow >> 4] * a.H_kv + kvh) * KVT::kBlockBytes;
      const int slot = krow & 15;
      if constexpr (!FP8) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 kv8 = *reinterpret_cast<const bf16x8*>(kb + ((2 * ks + hh) * 16 + slot) * 16);
          x[sb] = mfma32x32x16(kv8, qop[ks], x[sb]);
        }
      } else {
#pragma unroll
        for (int cc = 0; cc < KS / 2; ++cc) {
          const u32x4 raw = *reinterpret_cast<const u32x4*>(kb + ((2 * cc + hh) * 16 + slot) * 16);
          x[sb] = mfma32x32x16(e4m3x8_to_bf16(raw[0], raw[1]), qop[2 * cc], x[sb]);
          x[sb] = mfma32x32x16(e4m3x8_to_bf16(raw[2], raw[3]), qop[2 * cc + 1], x[sb]);
        }
      }
    }

    // Scale to the log2 domain, mask, and take the tile max.
    float tmax = -INFINITY;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const int t0 = kt + 32 * sb;
      float c0 = a.c, c1 = a.c;
      if constexpr (FP8) {
        c0 *= a.k_scale[blk[sb][0] * a.H_kv + kvh];
        c1 *= a.k_scale[blk[sb][1] * a.H_kv + kvh];
      }
      const bool need_mask = t0 + 31 > P;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float s = x[sb][v] * (v < 8 ? c0 : c1);
        if (need_mask) {
          const int key = t0 + key_of_row(8 * (v >> 2) + 4 * hh + (v & 3));
          if (key > vis_last) s = -INFINITY;
        }
        if (!live[sb]) s = -INFINITY;
        x[sb][v] = s;
        tmax = fmaxf(tmax, s);
      }
    }
    tmax = halves_max(tmax);
    const float m_new = fmaxf(m_run, tmax);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    float psum = 0.f;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float p = fast_exp2(x[sb][v] - m_use);
        x[sb][v] = p;
        psum += p;
      }
    l_run = l_run * alpha + psum;
    if (__ballot(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;
    }
    m_run = m_new;

    // O^T += V^T . P^T over the live 16-key halves of each 32-key block.
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      if (!live[sb]) continue;
      const int t0 = kt + 32 * sb;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int tk = t0 + 16 * kk;   // first key of this cache block
        if (tk >= k_end) continue;
        float vs = 1.f;
        if constexpr (FP8) vs = a.v_scale[blk[sb][kk] * a.H_kv + kvh];
        bf16x8 pop;
#pragma unroll
        for (int j = 0; j < 8; ++j) pop[j] = (__bf16)(x[sb][8 * kk + j] * vs);
        const uint8_t* vb = a.v + (blk[sb][kk] * a.H_kv + kvh) * KVT::kBlockBytes;
        const bool tail = tk + 16 > L;   // block holds slots past L: zero them
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int d = 32 * db + ql;
          bf16x8 vop;
          if constexpr (!FP8) {
            vop = *reinterpret_cast<const bf16x8*>(vb + (d * 16 + 8 * hh) * 2);
          } else {
            const u32x2 raw = *reinterpret_cast<const u32x2*>(vb + d * 16 + 8 * hh);
            vop = e4m3x8_to_bf16(raw[0], raw[1]);
          }
          if (tail) {
#pragma unroll
            for (int j = 0; j < 8; ++j)
              if (tk + 8 * hh + j >= L) vop[j] = (__bf16)0.f;
          }
          o[db] = mfma32x32x16(vop, pop, o[db]);
        }
      }
    }
  }

  const float l_tot = halves_sum(l_run);
  if (!row_ok) return;
  if (n_splits == 1) {
    const float inv = 1.f / l_tot;
    uint16_t* orow = a.out + ((size_t)(b * a.R + pos) * a.H_q + head) * HD;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int d = 32 * db + 8 * r + 4 * hh;
        uint16_t e0 = f32_to_bf16_bits(o[db][4 * r + 0] * inv);
        uint16_t e1 = f32_to_bf16_bits(o[db][4 * r + 1] * inv);
        uint16_t e2 = f32_to_bf16_bits(o[db][4 * r + 2] * inv);
        uint16_t e3 = f32_to_bf16_bits(o[db][4 * r + 3] * inv);
        u32x2 w = {(uint32_t)e0 | ((uint32_t)e1 << 16), (uint32_t)e2 | ((uint32_t)e3 << 16)};
        *reinterpret_cast<u32x2*>(orow + d) = w;
      }
  } else {
    const size_t srow = ((size_t)(b * a.H_kv + kvh) * a.s_max + split) * a.M + m;
    float* dst = a.ws_o + srow * HD;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int d = 32 * db + 8 * r + 4 * hh;
        f32x4 w = {o[db][4 * r], o[db][4 * r + 1], o[db][4 * r + 2], o[db][4 * r + 3]};
        *reinterpret_cast<f32x4*>(dst + d) = w;
      }
    if (hh == 0) a.ws_ml[srow] = f32x2{m_run, l_tot};
  }
}

// Merge the split states of every query row whose sequence used more than one
// split: m = max_s m_s, w_s = 2^(m_s - m), out = sum_s w_s O_s / sum_s w_s l_s.
// One wave per (b, kvh, row); lanes own consecutive output dims.
template <int HD>
__global__ __launch_bounds__(256) void sv_attn_combine(AttnArgs a, int total_rows) {
  constexpr int PER = HD / kWave;   // dims per lane (1 or 2)
  const int row = blockIdx.x * 4 + threadIdx.x / kWave;
  if (row >= total_rows) return;
  const int lane = threadIdx.x % kWave;
  const int m = row % a.M;
  const int bk = row / a.M;
  const int kvh = bk % a.H_kv;
  const int b = bk / a.H_kv;
  const int L = min(max(a.kv_lens[b], 0), a.max_kv_len);
  const int n = (L + a.split_tokens - 1) / a.split_tokens;
  if (n <= 1) return;
  const size_t base = (size_t)bk * a.s_max * a.M + m;
  float mx = -INFINITY;
  for (int s = 0; s < n; ++s) mx = fmaxf(mx, a.ws_ml[base + (size_t)s * a.M][0]);
  const float mu = (mx == -INFINITY) ? 0.f : mx;
  float acc[PER] = {};
  float l = 0.f;
  for (int s = 0; s < n; ++s) {
    const size_t r = base + (size_t)s * a.M;
    const f32x2 ml = a.ws_ml[r];
    const float w = fast_exp2(ml[0] - mu);
    l += w * ml[1];
    const float* src = a.ws_o + r * HD + lane * PER;
    if constexpr (PER == 2) {
      const f32x2 v = *reinterpret_cast<const f32x2*>(src);
      acc[0] += w * v[0];
      acc[1] += w * v[1];
    } else {
      acc[0] += w * src[0];
    }
  }
  const float inv = 1.f / l;
  const int pos = m / a.G;
  const int head = kvh * a.G + m % a.G;
  uint16_t* orow = a.out + ((size_t)(b * a.R + pos) * a.H_q + head) * HD + lane * PER;
  if constexpr (PER == 2) {
    *reinterpret_cast<uint32_t*>(orow) =
        (uint32_t)f32_to_bf16_bits(acc[0] * inv) | ((uint32_t)f32_to_bf16_bits(acc[1] * inv) << 16);
  } else {
    orow[0] = f32_to_bf16_bits(acc[0] * inv);
  }
}

void plan_attention(AttnPlan& p, int split_request) {
  p.G = p.H_q / p.H_kv;
  p.M = p.G * p.R;
  const int waves_needed = (p.M + kRowsPerWave - 1) / kRowsPerWave;
  p.waves = waves_needed >= 4 ? 4 : (waves_needed >= 2 ? 2 : 1);
  p.m_tiles = (p.M + kRowsPerWave * p.waves - 1) / (kRowsPerWave * p.waves);
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
  if (p.s_max <= 1) {
    p.ws_o_bytes = p.ws_ml_offset = p.ws_bytes = 0;
    return;
  }
  const size_t rows = (size_t)p.B * p.H_kv * p.s_max * p.M;
  p.ws_o_bytes = rows * p.hd * sizeof(float);
  p.ws_ml_offset = (p.ws_o_bytes + 255) / 256 * 256;
  p.ws_bytes = p.ws_ml_offset + rows * sizeof(f32x2);
}

template <int HD, bool FP8>
static hipError_t launch_typed(const AttnPlan& p, const AttnArgs& a, hipStream_t stream) {
  dim3 grid(p.s_max, p.H_kv * p.m_tiles, p.B);
  switch (p.waves) {
    case 1: sv_attn_partial<HD, FP8, 1><<<grid, kWave * 1, 0, stream>>>(a); break;
    case 2: sv_attn_partial<HD, FP8, 2><<<grid, kWave * 2, 0, stream>>>(a); break;
    default: sv_attn_partial<HD, FP8, 4><<<grid, kWave * 4, 0, stream>>>(a); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.s_max <= 1) return e;
  const int total = p.B * p.H_kv * p.M;
  sv_attn_combine<HD><<<(total + 3) / 4, 256, 0, stream>>>(a, total);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnPlan& p, const AttnPtrs& ptr, hipStream_t stream) {
  AttnArgs a;
  a.q = static_cast<const uint16_t*>(ptr.q);
  a.k = static_cast<const uint8_t*>(ptr.k);
  a.v = static_cast<const uint8_t*>(ptr.v);
  a.k_scale = ptr.k_scale;
  a.v_scale = ptr.v_scale;
  a.block_table = ptr.block_table;
  a.kv_lens = ptr.kv_lens;
  a.out = static_cast<uint16_t*>(ptr.out);
  a.ws_o = static_cast<float*>(ptr.ws);
  a.ws_ml = p.ws_bytes ? reinterpret_cast<f32x2*>(static_cast<char*>(ptr.ws) + p.ws_ml_offset)
                       : nullptr;
  a.R = p.R;
  a.H_q = p.H_q;
  a.H_kv = p.H_kv;
  a.G = p.G;
  a.M = p.M;
  a.max_blocks = p.max_blocks;
  a.num_blocks = p.num_blocks;
  a.max_kv_len = p.max_kv_len;
  a.split_tokens = p.split_tokens;
  a.s_max = p.s_max;
  a.c = p.sm_scale * kLog2e;
  if (p.hd == 128) return p.fp8 ? launch_typed<128, true>(p, a, stream) : launch_typed<128, false>(p, a, stream);
  return p.fp8 ? launch_typed<64, true>(p, a, stream) : launch_typed<64, false>(p, a, stream);
}

}  // namespace sv
