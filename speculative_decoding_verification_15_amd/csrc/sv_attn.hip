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
// Two partial kernels share that tile arithmetic:
//   sv_attn_partial_lds     (M > 64) four waves own 128 rows and share each
//                           64-key tile through LDS.  All 256 threads fetch the
//                           tile with coalesced 16-byte loads into registers
//                           while the previous tile is being computed, convert
//                           e4m3 to bf16 once, and write it to the other half
//                           of a double buffer.
//   sv_attn_partial_direct  (M <= 64) one or two waves, each streaming its K/V
//                           operands straight from HBM in MFMA layout.
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

// Everything one lane needs to know about its query row and key range.
struct RowCtx {
  int b, kvh, split, L, n_splits, k_begin, k_end;
  int m, pos, head, P, vis_last;
  int ql, hh;
  bool row_ok;
};

__device__ __forceinline__ RowCtx make_row_ctx(const AttnArgs& a, int split, int kvh, int b,
                                               int L, int m0, int lane) {
  RowCtx r;
  r.b = b;
  r.kvh = kvh;
  r.split = split;
  r.L = L;
  r.n_splits = (L + a.split_tokens - 1) / a.split_tokens;
  r.k_begin = split * a.split_tokens;
  r.k_end = min(r.k_begin + a.split_tokens, L);
  r.ql = lane & 31;
  r.hh = lane >> 5;
  r.m = m0 + r.ql;
  r.row_ok = r.m < a.M;
  r.pos = r.row_ok ? r.m / a.G : a.R - 1;
  r.head = kvh * a.G + (r.row_ok ? r.m % a.G : 0);
  r.P = L - a.R;
  r.vis_last = r.P + r.pos;
  return r;
}

__device__ __forceinline__ int clamp_len(const AttnArgs& a, int b) {
  return min(max(a.kv_lens[b], 0), a.max_kv_len);
}

// Physical block of logical block j of a sequence with n_blk blocks, clamped so
// that a bad table entry or a block past the sequence never leaves the cache.
__device__ __forceinline__ size_t phys_block(const AttnArgs& a, const int32_t* tbl, int j,
                                             int n_blk) {
  int p = tbl[min(j, n_blk - 1)];
  return (size_t)min(max(p, 0), a.num_blocks - 1);
}

// Q^T operand: lane (row ql, half hh) supplies dims 16ks + 8hh .. +8 in k-step
// ks (FP8_LAYOUT: the e4m3 K vector of 16 dims serves k-steps 2c and 2c + 1,
// so half hh of k-step 2c + e holds dims 16(2c + hh) + 8e .. +8).
template <int HD, bool FP8_LAYOUT>
__device__ __forceinline__ void load_q(const AttnArgs& a, const RowCtx& r, bf16x8 (&qop)[HD / 16]) {
  const uint16_t* qrow = a.q + ((size_t)(r.b * a.R + r.pos) * a.H_q + r.head) * HD;
#pragma unroll
  for (int ks = 0; ks < HD / 16; ++ks) {
    const int d0 = FP8_LAYOUT ? (32 * (ks / 2) + 16 * r.hh + 8 * (ks % 2)) : (16 * ks + 8 * r.hh);
    bf16x8 z = {};
    qop[ks] = r.row_ok ? *reinterpret_cast<const bf16x8*>(qrow + d0) : z;
  }
}

// Online-softmax update for one 64-key tile whose raw scores q.k are in x
// (two 32-key sub-blocks).  cs[sb][half] scales the scores of the 16-key block
// `half` of sub-block sb into the log2 domain.  On return x holds the
// probabilities exp2(x - m_new), o has been rescaled, and m_run / l_run updated.
template <int DB>
__device__ __forceinline__ void softmax_tile(f32x16 (&x)[2], const float (&cs)[2][2],
                                             const bool (&live)[2], int kt, const RowCtx& r,
                                             float& m_run, float& l_run, f32x16 (&o)[DB]) {
  float tmax = -INFINITY;
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    const int t0 = kt + 32 * sb;
    const bool need_mask = t0 + 31 > r.P;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      float s = x[sb][v] * (v < 8 ? cs[sb][0] : cs[sb][1]);
      if (need_mask) {
        const int key = t0 + key_of_row(8 * (v >> 2) + 4 * r.hh + (v & 3));
        if (key > r.vis_last) s = -INFINITY;
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
}

// P^T operand for PV step (sub-block sb, 16-key block kk): the 8 probabilities
// this lane holds for keys 16kk + 8hh .. +8, times the block's V scale.
__device__ __forceinline__ bf16x8 p_operand(const f32x16& x, int kk, float vs) {
  bf16x8 p;
#pragma unroll
  for (int j = 0; j < 8; ++j) p[j] = (__bf16)(x[8 * kk + j] * vs);
  return p;
}

// Final division by l (single split) or the split's unnormalised state.
template <int HD>
__device__ __forceinline__ void write_result(const AttnArgs& a, const RowCtx& r,
                                             const f32x16 (&o)[HD / 32], float m_run,
                                             float l_run) {
  constexpr int DB = HD / 32;
  const float l_tot = halves_sum(l_run);
  if (!r.row_ok) return;
  if (r.n_splits == 1) {
    const float inv = 1.f / l_tot;
    uint16_t* orow = a.out + ((size_t)(r.b * a.R + r.pos) * a.H_q + r.head) * HD;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = 32 * db + 8 * q4 + 4 * r.hh;
        const uint32_t e0 = f32_to_bf16_bits(o[db][4 * q4 + 0] * inv);
        const uint32_t e1 = f32_to_bf16_bits(o[db][4 * q4 + 1] * inv);
        const uint32_t e2 = f32_to_bf16_bits(o[db][4 * q4 + 2] * inv);
        const uint32_t e3 = f32_to_bf16_bits(o[db][4 * q4 + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + d) = u32x2{e0 | (e1 << 16), e2 | (e3 << 16)};
      }
  } else {
    const size_t srow = ((size_t)(r.b * a.H_kv + r.kvh) * a.s_max + r.split) * a.M + r.m;
    float* dst = a.ws_o + srow * HD;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = 32 * db + 8 * q4 + 4 * r.hh;
        *reinterpret_cast<f32x4*>(dst + d) =
            f32x4{o[db][4 * q4], o[db][4 * q4 + 1], o[db][4 * q4 + 2], o[db][4 * q4 + 3]};
      }
    if (r.hh == 0) a.ws_ml[srow] = f32x2{m_run, l_tot};
  }
}

// ---------------------------------------------------------------------------
// LDS-staged partial kernel: 4 waves x 32 rows, 64-key tiles, double buffer.
//
// LDS image of one tile (always bf16, whatever the cache stores):
//   K: 4 blocks x [hd/8 vectors][16 slot positions] x 16 B.  Slot position s
//      holds key pi16(s) (bits 2 and 3 swapped), so MFMA row i of a 32-key
//      block reads position i & 15 of block i / 16 -- eight consecutive lanes
//      read 128 contiguous bytes.
//   V: 4 blocks x [hd dims][2 halves] x 16 B.  Half position hs of dim d holds
//      token slots 8h .. 8h + 7 with h = hs ^ ((d >> 2) & 1), which spreads
//      eight consecutive dims over all banks.
// ---------------------------------------------------------------------------
constexpr int kLdsThreads = 256;

template <int HD>
struct LdsTile {
  static constexpr int kBlk = HD * 16 * 2;       // bytes of one block of K or V as bf16
  static constexpr int kStage = 8 * kBlk;        // 4 K blocks + 4 V blocks
  static constexpr int kPos = kBlk / 16;         // 16-byte vectors per block
};

__device__ __forceinline__ int swap23(int s) { return (s & 3) | ((s & 4) << 1) | ((s & 8) >> 1); }
__device__ __forceinline__ int vhalf_swz(int d) { return (d >> 2) & 1; }

// Zero the bf16 elements of an 8-slot V vector whose keys are >= L.
__device__ __forceinline__ u32x4 zero_tail(u32x4 v, int key0, int L) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    uint32_t w = v[e];
    if (key0 + 2 * e >= L) w &= 0xFFFF0000u;
    if (key0 + 2 * e + 1 >= L) w &= 0x0000FFFFu;
    v[e] = w;
  }
  return v;
}

__device__ __forceinline__ u32x4 bf16x8_bits(bf16x8 x) { return __builtin_bit_cast(u32x4, x); }

template <int HD, bool FP8>
struct Stager {
  // bf16: one 16-byte vector per (u, thread); e4m3: one 16-byte vector of codes
  static constexpr int kGlobalVec = FP8 ? (2 * 4 * HD) : (2 * 4 * 2 * HD);   // per tile
  static constexpr int kPerThread = kGlobalVec / kLdsThreads;
  u32x4 raw[kPerThread];
};

template <int HD, bool FP8>
__global__ __attribute__((amdgpu_flat_work_group_size(kLdsThreads, kLdsThreads),
                          amdgpu_waves_per_eu(2, 2)))
void sv_attn_partial_lds(AttnArgs a) {
  constexpr int KS = HD / 16;
  constexpr int DB = HD / 32;
  using T = LdsTile<HD>;
  using S = Stager<HD, FP8>;
  constexpr int kGlobBlk = FP8 ? HD : 2 * HD;      // 16-byte vectors per cache block
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * T::kStage];

  const int split = blockIdx.x;
  const int kvh = blockIdx.y % a.H_kv;
  const int mt = blockIdx.y / a.H_kv;
  const int b = blockIdx.z;
  const int L = clamp_len(a, b);
  if (split * a.split_tokens >= L) return;           // whole workgroup: no barrier yet
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const int m0 = (mt * 4 + wave) * kRowsPerWave;
  const bool active = m0 < a.M;                       // inactive waves still load
  const RowCtx r = make_row_ctx(a, split, kvh, b, L, m0, lane);

  bf16x8 qop[KS];
  if (active) load_q<HD, false>(a, r, qop);

  const int32_t* tbl = a.block_table + (size_t)b * a.max_blocks;
  const int n_blk = (L + 15) / 16;
  const int ntiles = (r.k_end - r.k_begin + kAttnTile - 1) / kAttnTile;
  const size_t kv_stride = (size_t)a.H_kv * (FP8 ? HD * 16 : HD * 32);   // bytes per physical block
  const size_t head_off = (size_t)kvh * (FP8 ? HD * 16 : HD * 32);

  S st;
  // Fetch tile `t` (cache blocks 4 * (k_begin/16 + 4t) ...) into registers.
  auto fetch = [&](int t) {
    const int lb0 = r.k_begin / 16 + 4 * t;
#pragma unroll
    for (int u = 0; u < S::kPerThread; ++u) {
      const int qv = tid + kLdsThreads * u;
      const int bk = qv / kGlobBlk;                  // 0..7: K blocks 0..3, V blocks 0..3
      const int p = qv % kGlobBlk;
      const int blk = bk & 3;
      const size_t pb = phys_block(a, tbl, lb0 + blk, n_blk);
      const uint8_t* base = (bk < 4 ? a.k : a.v) + pb * kv_stride + head_off;
      int off;
      if constexpr (!FP8) {
        off = bk < 4 ? ((p >> 4) * 16 + swap23(p & 15)) * 16
                     : ((p >> 1) * 2 + ((p & 1) ^ vhalf_swz(p >> 1))) * 16;
      } else {
        off = p * 16;   // K: (vector c, slot) ; V: dim d -- both 16 codes
      }
      st.raw[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + off));
    }
  };
  // Write the fetched tile `t` into LDS stage `stage` (e4m3 decoded to bf16,
  // V slots at or past L zeroed).
  auto commit = [&](int t, int stage) {
    uint8_t* sbase = smem + stage * T::kStage;
    const int key_tile = r.k_begin + kAttnTile * t;
    const bool tail = key_tile + kAttnTile > L;
#pragma unroll
    for (int u = 0; u < S::kPerThread; ++u) {
      const int qv = tid + kLdsThreads * u;
      const int bk = qv / kGlobBlk;
      const int p = qv % kGlobBlk;
      const int blk = bk & 3;
      uint8_t* dst = sbase + bk * T::kBlk;
      if constexpr (!FP8) {
        u32x4 v = st.raw[u];
        if (bk >= 4 && tail) {
          const int d = p >> 1;
          const int h = (p & 1) ^ vhalf_swz(d);
          v = zero_tail(v, key_tile + 16 * blk + 8 * h, L);
        }
        *reinterpret_cast<u32x4*>(dst + p * 16) = v;
      } else {
        const bf16x8 lo = e4m3x8_to_bf16(st.raw[u][0], st.raw[u][1]);
        const bf16x8 hi = e4m3x8_to_bf16(st.raw[u][2], st.raw[u][3]);
        if (bk < 4) {
          // codes of 16 dims (vector c8 = p / 16) of slot p % 16
          const int c8 = p >> 4;
          const int s = swap23(p & 15);
          *reinterpret_cast<u32x4*>(dst + ((2 * c8) * 16 + s) * 16) = bf16x8_bits(lo);
          *reinterpret_cast<u32x4*>(dst + ((2 * c8 + 1) * 16 + s) * 16) = bf16x8_bits(hi);
        } else {
          // codes of 16 slots of dim d = p
          const int d = p;
          u32x4 v0 = bf16x8_bits(lo), v1 = bf16x8_bits(hi);
          if (tail) {
            v0 = zero_tail(v0, key_tile + 16 * blk, L);
            v1 = zero_tail(v1, key_tile + 16 * blk + 8, L);
          }
          const int sw = vhalf_swz(d);
          *reinterpret_cast<u32x4*>(dst + (2 * d + sw) * 16) = v0;
          *reinterpret_cast<u32x4*>(dst + (2 * d + (1 ^ sw)) * 16) = v1;
        }
      }
    }
  };

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  if (ntiles > 0) {
    fetch(0);
    commit(0, 0);
  }
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    if (t + 1 < ntiles) fetch(t + 1);
    if (active) {
      const uint8_t* sk = smem + (t & 1) * T::kStage;
      const uint8_t* sv = sk + 4 * T::kBlk;
      const int kt = r.k_begin + kAttnTile * t;
      const int lb0 = kt / 16;
      f32x16 x[2];
      bool live[2];
      float cs[2][2];
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        live[sb] = kt + 32 * sb < r.k_end;
        x[sb] = f32x16{};
        if constexpr (FP8) {
          cs[sb][0] = a.c * a.k_scale[phys_block(a, tbl, lb0 + 2 * sb, n_blk) * a.H_kv + kvh];
          cs[sb][1] = a.c * a.k_scale[phys_block(a, tbl, lb0 + 2 * sb + 1, n_blk) * a.H_kv + kvh];
        } else {
          cs[sb][0] = cs[sb][1] = a.c;
        }
        if (!live[sb]) continue;
        const uint8_t* kb = sk + (2 * sb + (r.ql >> 4)) * T::kBlk + (r.ql & 15) * 16;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 kop = *reinterpret_cast<const bf16x8*>(kb + (2 * ks + r.hh) * 256);
          x[sb] = mfma32x32x16(kop, qop[ks], x[sb]);
        }
      }
      softmax_tile<DB>(x, cs, live, kt, r, m_run, l_run, o);
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        if (!live[sb]) continue;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          if (kt + 32 * sb + 16 * kk >= r.k_end) continue;
          float vs = 1.f;
          if constexpr (FP8) vs = a.v_scale[phys_block(a, tbl, lb0 + 2 * sb + kk, n_blk) * a.H_kv + kvh];
          const bf16x8 pop = p_operand(x[sb], kk, vs);
          const uint8_t* vb = sv + (2 * sb + kk) * T::kBlk;
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const int d = 32 * db + r.ql;
            const bf16x8 vop =
                *reinterpret_cast<const bf16x8*>(vb + (2 * d + (r.hh ^ vhalf_swz(d))) * 16);
            o[db] = mfma32x32x16(vop, pop, o[db]);
          }
        }
      }
    }
    if (t + 1 < ntiles) commit(t + 1, (t + 1) & 1);
    __syncthreads();
  }
  if (active) write_result<HD>(a, r, o, m_run, l_run);
}

// ---------------------------------------------------------------------------
// Direct partial kernel (M <= 64): every wave streams its own operands.
// ---------------------------------------------------------------------------
template <int HD, bool FP8, int NW>
__global__ __launch_bounds__(kWave * NW) void sv_attn_partial_direct(AttnArgs a) {
  constexpr int KS = HD / 16;
  constexpr int DB = HD / 32;
  constexpr size_t kBlockBytes = (size_t)HD * 16 * (FP8 ? 1 : 2);

  const int split = blockIdx.x;
  const int kvh = blockIdx.y % a.H_kv;
  const int mt = blockIdx.y / a.H_kv;
  const int b = blockIdx.z;
  const int L = clamp_len(a, b);
  if (split * a.split_tokens >= L) return;
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int m0 = (mt * NW + wave) * kRowsPerWave;
  if (m0 >= a.M) return;
  const RowCtx r = make_row_ctx(a, split, kvh, b, L, m0, lane);

  bf16x8 qop[KS];
  load_q<HD, FP8>(a, r, qop);

  const int32_t* tbl = a.block_table + (size_t)b * a.max_blocks;
  const int n_blk = (L + 15) / 16;
  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const int krow = key_of_row(r.ql);   // key (within the 32-key block) of A-row ql

  for (int kt = r.k_begin; kt < r.k_end; kt += kAttnTile) {
    f32x16 x[2];
    size_t blk[2][2];
    bool live[2];
    float cs[2][2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const int t0 = kt + 32 * sb;
      live[sb] = t0 < r.k_end;
      blk[sb][0] = phys_block(a, tbl, t0 / 16, n_blk);
      blk[sb][1] = phys_block(a, tbl, t0 / 16 + 1, n_blk);
      cs[sb][0] = cs[sb][1] = a.c;
      if constexpr (FP8) {
        cs[sb][0] *= a.k_scale[blk[sb][0] * a.H_kv + kvh];
        cs[sb][1] *= a.k_scale[blk[sb][1] * a.H_kv + kvh];
      }
      x[sb] = f32x16{};
      if (!live[sb]) continue;
      const uint8_t* kb = a.k + (blk[sb][krow >> 4] * a.H_kv + kvh) * kBlockBytes;
      const int slot = krow & 15;
      if constexpr (!FP8) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 k8 = *reinterpret_cast<const bf16x8*>(kb + ((2 * ks + r.hh) * 16 + slot) * 16);
          x[sb] = mfma32x32x16(k8, qop[ks], x[sb]);
        }
      } else {
#pragma unroll
        for (int cc = 0; cc < KS / 2; ++cc) {
          const u32x4 raw = *reinterpret_cast<const u32x4*>(kb + ((2 * cc + r.hh) * 16 + slot) * 16);
          x[sb] = mfma32x32x16(e4m3x8_to_bf16(raw[0], raw[1]), qop[2 * cc], x[sb]);
          x[sb] = mfma32x32x16(e4m3x8_to_bf16(raw[2], raw[3]), qop[2 * cc + 1], x[sb]);
        }
      }
    }
    softmax_tile<DB>(x, cs, live, kt, r, m_run, l_run, o);
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      if (!live[sb]) continue;
      const int t0 = kt + 32 * sb;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int tk = t0 + 16 * kk;   // first key of this cache block
        if (tk >= r.k_end) continue;
        float vs = 1.f;
        if constexpr (FP8) vs = a.v_scale[blk[sb][kk] * a.H_kv + kvh];
        const bf16x8 pop = p_operand(x[sb], kk, vs);
        const uint8_t* vb = a.v + (blk[sb][kk] * a.H_kv + kvh) * kBlockBytes;
        const bool tail = tk + 16 > L;   // block holds slots past L: zero them
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int d = 32 * db + r.ql;
          bf16x8 vop;
          if constexpr (!FP8) {
            vop = *reinterpret_cast<const bf16x8*>(vb + (d * 16 + 8 * r.hh) * 2);
          } else {
            const u32x2 raw = *reinterpret_cast<const u32x2*>(vb + d * 16 + 8 * r.hh);
            vop = e4m3x8_to_bf16(raw[0], raw[1]);
          }
          if (tail) {
#pragma unroll
            for (int j = 0; j < 8; ++j)
              if (tk + 8 * r.hh + j >= L) vop[j] = (__bf16)0.f;
          }
          o[db] = mfma32x32x16(vop, pop, o[db]);
        }
      }
    }
  }
  write_result<HD>(a, r, o, m_run, l_run);
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
  const int L = clamp_len(a, b);
  const int n = (L + a.split_tokens - 1) / a.split_tokens;
  if (n <= 1) return;
  const size_t base = (size_t)bk * a.s_max * a.M + m;
  float mx = -INFINITY;
  for (int s = 0; s < n; ++s) mx = fmaxf(mx, a.ws_ml[base + (size_t)s * a.M][0]);
  const float mu = (mx == -INFINITY) ? 0.f : mx;
  float acc[PER] = {};
  float l = 0.f;
  for (int s = 0; s < n; ++s) {
    const size_t rr = base + (size_t)s * a.M;
    const f32x2 ml = a.ws_ml[rr];
    const float w = fast_exp2(ml[0] - mu);
    l += w * ml[1];
    const float* src = a.ws_o + rr * HD + lane * PER;
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
  p.waves = waves_needed > 2 ? 4 : waves_needed;
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
    case 1: sv_attn_partial_direct<HD, FP8, 1><<<grid, kWave * 1, 0, stream>>>(a); break;
    case 2: sv_attn_partial_direct<HD, FP8, 2><<<grid, kWave * 2, 0, stream>>>(a); break;
    default: sv_attn_partial_lds<HD, FP8><<<grid, kLdsThreads, 0, stream>>>(a); break;
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
  if (p.hd == 128)
    return p.fp8 ? launch_typed<128, true>(p, a, stream) : launch_typed<128, false>(p, a, stream);
  return p.fp8 ? launch_typed<64, true>(p, a, stream) : launch_typed<64, false>(p, a, stream);
}

}  // namespace sv
