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
#include "sv_attn_plan.h"

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
  float* ws_o;    // split path: [B][H_kv][s_max][M][hd] unnormalised O of each split;
                  // stream-K: fp16 O / (l f) of each segment slot (sk_partial_o)
  f32x2* ws_ml;   // [B][H_kv][s_max][M] (m, l) of each split, log2 domain
  float* ws_f;    // stream-K: power-of-two factor f of each slot row
  int B, R, H_q, H_kv, G, M;
  int max_blocks, num_blocks, max_kv_len;
  int split_tokens;
  union {
    int s_max;         // split path: splits per sequence
    uint32_t tree_lo;  // stream-K tree variants: low word of the ancestor-mask pointer
  };
  int m_tiles;
  int min_tiles;  // stream-K: least tiles per workgroup
  float c;        // sm_scale * log2(e)
  int* sk_meta;   // stream-K: [W, Wp, pref[0..B]] written by workgroup 0 for the merge
  int sk_rows;    // stream-K: rows per unit (128 or 256)
  uint32_t tree_hi;  // stream-K tree variants: high word of the ancestor-mask pointer
                     // (the struct's trailing padding, so the layout is unchanged)
};

// Tree variants: [B][R] ancestor masks, bit j of mask[b][i] = node j is node i
// or one of its ancestors.
__device__ __forceinline__ const uint64_t* tree_masks(const AttnArgs& a) {
  return reinterpret_cast<const uint64_t*>(((uint64_t)a.tree_hi << 32) | a.tree_lo);
}

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

// The same for a wave-uniform b, read with a scalar load (no vector memory
// counter involved).
__device__ __forceinline__ int clamp_len_s(const AttnArgs& a, int b) {
  const __attribute__((address_space(4))) int32_t* kl =
      (const __attribute__((address_space(4))) int32_t*)a.kv_lens;
  return min(max(kl[b], 0), a.max_kv_len);
}

// Work item of this workgroup.  The grid is one-dimensional and the hardware
// hands consecutive workgroup ids to the 8 XCDs in turn, so the id is decoded
// as (xcd = id % 8, k = id / 8): unit u = (k / m_tiles) * 8 + xcd, row tile
// mt = k % m_tiles.  All row tiles of a unit (same sequence, KV head and
// split, hence the same K/V) run on one XCD and share its L2, and units --
// ordered split-major, (sequence, KV head) minor -- are dealt round-robin over
// the XCDs, so short sequences' missing splits do not pile up on one XCD.
struct Work {
  int split, kvh, mt, b;
  bool valid;
};

__device__ __forceinline__ Work decode_work(const AttnArgs& a, int m_tiles) {
  constexpr int kXcds = 8;
  const int id = blockIdx.x;
  const int k = id / kXcds;
  const int unit = (k / m_tiles) * kXcds + id % kXcds;
  const int bk_units = a.B * a.H_kv;
  Work w;
  w.mt = k % m_tiles;
  w.split = unit / bk_units;
  const int bk = unit % bk_units;
  w.b = bk / a.H_kv;
  w.kvh = bk % a.H_kv;
  w.valid = w.split < a.s_max;
  return w;
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
// Q^T operands of the row for lanes whose row exists, and those of the row's
// position clamp for the others (callers zero them with row_ok once the loads
// have landed): no register is written before the loads retire.
template <int HD>
__device__ __forceinline__ void load_q_raw(const AttnArgs& a, const RowCtx& r,
                                           bf16x8 (&qop)[HD / 16]) {
  const uint16_t* qrow = a.q + ((size_t)(r.b * a.R + r.pos) * a.H_q + r.head) * HD;
#pragma unroll
  for (int ks = 0; ks < HD / 16; ++ks)
    qop[ks] = *reinterpret_cast<const bf16x8*>(qrow + 16 * ks + 8 * r.hh);
}

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
// (two 32-key sub-blocks).  cs[sb][half] > 0 scales the scores of 16-key block
// `half` of sub-block sb into the log2 domain.
//
// The reference m_ref against which exponentials are taken follows the running
// max lazily: it moves (and O, l are rescaled by 2^(m_ref - m_new)) only when
// the tile max exceeds it by more than kLazyRescale, so probabilities stay
// below 2^kLazyRescale.  O / l is the same for any reference, so the result is
// unchanged; it only saves the O rescale on the many tiles whose max grows a
// little.  MASKED tiles apply the causal limit (key <= P + pos) and drop dead
// sub-blocks; unmasked tiles have every key live and visible to every row.
// On return x holds the probabilities.
constexpr float kLazyRescale = 8.f;

template <bool MASKED>
__device__ __forceinline__ bool softmax_core(f32x16 (&x)[2], const float (&cs)[2][2],
                                             const bool (&live)[2], int kt, const RowCtx& r,
                                             float& m_ref, float& l_run, float& alpha) {
  float tmax = -INFINITY;
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      float hm = -INFINITY;
#pragma unroll
      for (int v = 8 * half; v < 8 * half + 8; ++v) {
        if constexpr (MASKED) {
          const int key = kt + 32 * sb + key_of_row(8 * (v >> 2) + 4 * r.hh + (v & 3));
          if (!live[sb] || key > r.vis_last) x[sb][v] = -INFINITY;
        }
        hm = fmaxf(hm, x[sb][v]);
      }
      tmax = fmaxf(tmax, hm * cs[sb][half]);
    }
  }
  tmax = halves_max(tmax);
  bool move = false;
  alpha = 1.f;
  if (m_ref == -INFINITY) {
    m_ref = tmax;                  // first visible keys of this row: O and l are still 0
  } else if (tmax > m_ref + kLazyRescale) {
    alpha = fast_exp2(m_ref - tmax);
    m_ref = tmax;
    move = true;
  }
  const float m_neg = (m_ref == -INFINITY) ? 0.f : -m_ref;
  float psum = 0.f;
#pragma unroll
  for (int sb = 0; sb < 2; ++sb)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float p = fast_exp2(__builtin_fmaf(x[sb][v], cs[sb][v >> 3], m_neg));
      x[sb][v] = p;
      psum += p;
    }
  l_run = l_run * alpha + psum;
  return __ballot(move) != 0;
}

// Online-softmax update for one 32-key sub-block (scores x, scale c into the
// log2 domain; MASKED: masked scores are already -inf, and a row may have no
// visible key yet).  Returns the probabilities as the PV B operands of its two
// 16-key halves, with l accumulated from those bf16 values (the same numbers
// the PV product multiplies), and whether O must be rescaled by alpha (lazy
// reference, see softmax_core).
template <bool MASKED = false>
__device__ __forceinline__ bool softmax_sub(const f32x16& x, float c, float& m_ref, float& l_run,
                                            float& alpha, bf16x8& p0, bf16x8& p1) {
  float hm = fmaximum(x[0], x[1]);
#pragma unroll
  for (int v = 2; v < 16; ++v) hm = fmaximum(hm, x[v]);
  const float tmax = halves_maximum(hm * c);
  // Selects rather than branches, so that the caller can overlap this VALU
  // work with MFMAs of its own basic block.
  const bool first = m_ref == -INFINITY;     // no visible key yet: O and l are 0
  const bool move = !first && tmax > m_ref + kLazyRescale;
  alpha = move ? fast_exp2(m_ref - tmax) : 1.f;
  m_ref = (first || move) ? tmax : m_ref;
  const float m_neg = (MASKED && m_ref == -INFINITY) ? 0.f : -m_ref;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    p0[j] = (__bf16)fast_exp2(__builtin_fmaf(x[j], c, m_neg));
    p1[j] = (__bf16)fast_exp2(__builtin_fmaf(x[8 + j], c, m_neg));
  }
  const bf16x2 one = {(__bf16)1.f, (__bf16)1.f};
  float psum = 0.f;
#pragma unroll
  for (int j = 0; j < 8; j += 2) {
    psum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{p0[j], p0[j + 1]}, one, psum, false);
    psum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{p1[j], p1[j + 1]}, one, psum, false);
  }
  l_run = l_run * alpha + psum;
  return __ballot(move) != 0;
}

// Running maximum of a stream-K segment before its first visible key: finite,
// so that the first tile with one simply moves the reference (alpha = 0 then
// scales O and l, both still 0) and no per-tile test for a first key is
// needed.  A tile whose keys are all masked leaves it there (its scores are
// -inf, exp2(-inf + 1e30) = 0), and a segment that never sees a key stores
// m = kNoMax with l = 0, which the merge weighs by 0.
constexpr float kNoMax = -1e30f;

// softmax_sub for the stream-K kernels (running maximum starting at kNoMax).
__device__ __forceinline__ bool softmax_sub_sk(const f32x16& x, float c, float& m_ref,
                                               float& l_run, float& alpha, bf16x8& p0,
                                               bf16x8& p1) {
  float hm = fmaximum(x[0], x[1]);
#pragma unroll
  for (int v = 2; v < 16; ++v) hm = fmaximum(hm, x[v]);
  const float tmax = halves_maximum(hm * c);
  const bool move = tmax > m_ref + kLazyRescale;
  alpha = move ? fast_exp2(m_ref - tmax) : 1.f;
  m_ref = move ? tmax : m_ref;
  const float m_neg = -m_ref;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    p0[j] = (__bf16)fast_exp2(__builtin_fmaf(x[j], c, m_neg));
    p1[j] = (__bf16)fast_exp2(__builtin_fmaf(x[8 + j], c, m_neg));
  }
  const bf16x2 one = {(__bf16)1.f, (__bf16)1.f};
  float psum = 0.f;
#pragma unroll
  for (int j = 0; j < 8; j += 2) {
    psum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{p0[j], p0[j + 1]}, one, psum, false);
    psum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{p1[j], p1[j + 1]}, one, psum, false);
  }
  l_run = l_run * alpha + psum;
  return __ballot(move) != 0;
}

// softmax_sub for a tile decoded from e4m3 codes: the scores of key block b
// (16 keys: registers 8b .. 8b + 7) are scaled by cb = c * (K mantissa of
// block b), and the probabilities of block b are returned times the block's V
// mantissa mvb (as the PV product needs them), while l accumulates the
// probabilities themselves.
__device__ __forceinline__ bool softmax_sub_fp8(const f32x16& x, float c0, float c1, float mv0,
                                                float mv1, float& m_ref, float& l_run,
                                                float& alpha, bf16x8& p0, bf16x8& p1) {
  float h0 = x[0], h1 = x[8];
#pragma unroll
  for (int v = 1; v < 8; ++v) {
    h0 = fmaximum(h0, x[v]);
    h1 = fmaximum(h1, x[8 + v]);
  }
  const float tmax = halves_maximum(fmaximum(h0 * c0, h1 * c1));
  const bool move = tmax > m_ref + kLazyRescale;   // the running maximum starts at kNoMax
  alpha = move ? fast_exp2(m_ref - tmax) : 1.f;
  m_ref = move ? tmax : m_ref;
  const float m_neg = -m_ref;
  const float a0 = m_neg + __builtin_amdgcn_logf(mv0), a1 = m_neg + __builtin_amdgcn_logf(mv1);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    p0[j] = (__bf16)fast_exp2(__builtin_fmaf(x[j], c0, a0));
    p1[j] = (__bf16)fast_exp2(__builtin_fmaf(x[8 + j], c1, a1));
  }
  const bf16x2 one = {(__bf16)1.f, (__bf16)1.f};
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int j = 0; j < 8; j += 2) {
    s0 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{p0[j], p0[j + 1]}, one, s0, false);
    s1 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{p1[j], p1[j + 1]}, one, s1, false);
  }
  l_run = l_run * alpha + s0 * __builtin_amdgcn_rcpf(mv0) + s1 * __builtin_amdgcn_rcpf(mv1);
  return __ballot(move) != 0;
}

// Online-softmax update plus the O rescale in place (used by the direct kernel).
template <int DB, bool MASKED>
__device__ __forceinline__ void softmax_tile(f32x16 (&x)[2], const float (&cs)[2][2],
                                             const bool (&live)[2], int kt, const RowCtx& r,
                                             float& m_ref, float& l_run, f32x16 (&o)[DB]) {
  float alpha;
  softmax_core<MASKED>(x, cs, live, kt, r, m_ref, l_run, alpha);
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] *= alpha;
}

// P^T operand for PV step (sub-block sb, 16-key block kk): the 8 probabilities
// this lane holds for keys 16kk + 8hh .. +8, times the block's V scale.
__device__ __forceinline__ bf16x8 p_operand(const f32x16& x, int kk, float vs) {
  bf16x8 p;
#pragma unroll
  for (int j = 0; j < 8; ++j) p[j] = (__bf16)(x[8 * kk + j] * vs);
  return p;
}

// Output row of this lane (accumulator layout: register 4 q4 + e of block db
// holds dim 32 db + 8 q4 + 4 hh + e), times inv, as bf16.  Lanes whose row
// does not exist must not call it.
template <int HD>
__device__ __forceinline__ void store_row_bf16(const AttnArgs& a, const RowCtx& r,
                                               const f32x16 (&o)[HD / 32], float inv) {
  uint16_t* orow = a.out + ((size_t)(r.b * a.R + r.pos) * a.H_q + r.head) * HD;
#pragma unroll
  for (int db = 0; db < HD / 32; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d = 32 * db + 8 * q4 + 4 * r.hh;
      const uint32_t e0 = f32_to_bf16_bits(o[db][4 * q4 + 0] * inv);
      const uint32_t e1 = f32_to_bf16_bits(o[db][4 * q4 + 1] * inv);
      const uint32_t e2 = f32_to_bf16_bits(o[db][4 * q4 + 2] * inv);
      const uint32_t e3 = f32_to_bf16_bits(o[db][4 * q4 + 3] * inv);
      *reinterpret_cast<u32x2*>(orow + d) = u32x2{e0 | (e1 << 16), e2 | (e3 << 16)};
    }
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
    store_row_bf16<HD>(a, r, o, 1.f / l_tot);
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
//      token slots 8h .. 8h + 7 with h = hs ^ vhalf_swz(d), which spreads eight
//      (and sixteen) consecutive dims over distinct banks.
// ---------------------------------------------------------------------------
constexpr int kLdsThreads = 256;
#ifndef SV_RING_STAGES
#define SV_RING_STAGES 2
#define SV_RING_WPE 2
#endif
#ifndef SV_STREAM_WPE
#define SV_STREAM_WPE 2
#endif

template <int HD>
struct LdsTile {
  static constexpr int kBlk = HD * 16 * 2;       // bytes of one block of K or V as bf16
  static constexpr int kStage = 8 * kBlk;        // 4 K blocks + 4 V blocks
  static constexpr int kPos = kBlk / 16;         // 16-byte vectors per block
};

__device__ __forceinline__ int swap23(int s) { return (s & 3) | ((s & 4) << 1) | ((s & 8) >> 1); }
// Eight consecutive dims (and sixteen) land on distinct 16-byte bank groups.
__device__ __forceinline__ int vhalf_swz(int d) { return ((d >> 2) ^ (d >> 3)) & 1; }

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
  // 16-byte global vectors of one tile: bf16 K and V blocks, or e4m3 codes
  static constexpr int kGlobBlk = FP8 ? HD : 2 * HD;         // vectors per cache block
  static constexpr int kPerThread = 8 * kGlobBlk / kLdsThreads;
  static constexpr int kBlkStep = kLdsThreads / kGlobBlk;    // blocks covered per u step
  u32x4 raw[kPerThread];
};

// One 64-key tile: S^T = K . Q^T on the LDS image, online-softmax update, and
// O^T += V^T . P^T.
// One 64-key tile on the LDS image of the register-staged kernel.  V slots at
// or past L were zeroed when the tile was staged; masked tiles still run every
// MFMA (see ring_tile) and exclude keys by selects on the scores.
template <int HD, bool FP8, bool MASKED>
__device__ __forceinline__ void lds_tile(const AttnArgs& a, const RowCtx& r, const uint8_t* stage,
                                         int k_lds, int v_lds, const bf16x8 (&qop)[HD / 16],
                                         const float (&cs)[2][2], const float (&vs)[4], int kt,
                                         float& m_ref, float& l_run, f32x16 (&o)[HD / 32]) {
  constexpr int KS = HD / 16;
  constexpr int DB = HD / 32;
  constexpr int BLK = LdsTile<HD>::kBlk;
  f32x16 x[2];
  bool live[2];
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    live[sb] = MASKED ? (kt + 32 * sb < r.k_end) : true;
    x[sb] = f32x16{};
    const uint8_t* kb = stage + k_lds + 2 * sb * BLK;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 kop = *reinterpret_cast<const bf16x8*>(kb + ks * 512);
      x[sb] = mfma32x32x16(kop, qop[ks], x[sb]);
    }
  }
  softmax_tile<DB, MASKED>(x, cs, live, kt, r, m_ref, l_run, o);
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const bf16x8 pop = p_operand(x[sb], kk, FP8 ? vs[2 * sb + kk] : 1.f);
      const uint8_t* vb = stage + v_lds + (4 + 2 * sb + kk) * BLK;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const bf16x8 vop = *reinterpret_cast<const bf16x8*>(vb + db * 1024);
        o[db] = mfma32x32x16(vop, pop, o[db]);
      }
    }
  }
}

template <int HD, bool FP8>
__global__ __attribute__((amdgpu_flat_work_group_size(kLdsThreads, kLdsThreads),
                          amdgpu_waves_per_eu(2, 2)))
void sv_attn_partial_lds(AttnArgs a) {
  constexpr int KS = HD / 16;
  constexpr int DB = HD / 32;
  using T = LdsTile<HD>;
  using S = Stager<HD, FP8>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * T::kStage];

  const Work wk = decode_work(a, a.m_tiles);
  if (!wk.valid) return;
  const int split = wk.split, kvh = wk.kvh, mt = wk.mt, b = wk.b;
  const int L = clamp_len(a, b);
  if (split * a.split_tokens >= L) return;           // whole workgroup: no barrier yet
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int m0 = (mt * 4 + wave) * kRowsPerWave;
  const bool active = m0 < a.M;                       // inactive waves still load
  const RowCtx r = make_row_ctx(a, split, kvh, b, L, m0, lane);

  bf16x8 qop[KS];
  if (active) load_q<HD, false>(a, r, qop);

  const int32_t* tbl = a.block_table + (size_t)b * a.max_blocks;
  const int n_blk = (L + 15) / 16;
  const int ntiles = (r.k_end - r.k_begin + kAttnTile - 1) / kAttnTile;
  const size_t blk_stride = (size_t)a.H_kv * (FP8 ? HD * 16 : HD * 32);   // bytes per physical block
  const size_t head_off = (size_t)kvh * (FP8 ? HD * 16 : HD * 32);

  // Per-thread, loop-invariant parts of the tile copy.  Thread tid moves
  // vector p of cache block bk(u) = u * kBlkStep + wave / (kGlobBlk / 64).
  const int p = tid % S::kGlobBlk;
  const int bk_wave = wave / (S::kGlobBlk / kWave);
  int g_off_k, g_off_v;      // byte offsets inside a global (block, head) chunk
  int l_off_k0, l_off_k1, l_off_v0, l_off_v1;   // byte offsets inside an LDS block image
  if constexpr (!FP8) {
    g_off_k = ((p >> 4) * 16 + swap23(p & 15)) * 16;
    g_off_v = ((p >> 1) * 2 + ((p & 1) ^ vhalf_swz(p >> 1))) * 16;
    l_off_k0 = l_off_v0 = p * 16;
    l_off_k1 = l_off_v1 = 0;
  } else {
    g_off_k = g_off_v = p * 16;                     // K: (vector p/16, slot p%16); V: dim p
    l_off_k0 = ((2 * (p >> 4)) * 16 + swap23(p & 15)) * 16;
    l_off_k1 = l_off_k0 + 256;
    l_off_v0 = (2 * p + vhalf_swz(p)) * 16;
    l_off_v1 = (2 * p + (1 ^ vhalf_swz(p))) * 16;
  }
  // MFMA operand reads inside a stage.
  const int k_lds = (r.ql >> 4) * T::kBlk + (r.ql & 15) * 16 + r.hh * 256;
  const int v_lds = (2 * r.ql + (r.hh ^ vhalf_swz(r.ql))) * 16;

  S st;
  auto fetch = [&](int t) {
    const int lb0 = r.k_begin / 16 + 4 * t;
#pragma unroll
    for (int u = 0; u < S::kPerThread; ++u) {
      const int bk = u * S::kBlkStep + bk_wave;                // wave-uniform
      const uint8_t* base = (bk < 4 ? a.k : a.v) + phys_block(a, tbl, lb0 + (bk & 3), n_blk) * blk_stride + head_off;
      st.raw[u] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(base + (bk < 4 ? g_off_k : g_off_v)));
    }
  };
  auto commit = [&](int t, int stage) {
    uint8_t* sbase = smem + stage * T::kStage;
    const int key_tile = r.k_begin + kAttnTile * t;
    const bool tail = key_tile + kAttnTile > L;
#pragma unroll
    for (int u = 0; u < S::kPerThread; ++u) {
      const int bk = u * S::kBlkStep + bk_wave;
      uint8_t* dst = sbase + bk * T::kBlk;
      const int key_blk = key_tile + 16 * (bk & 3);
      if constexpr (!FP8) {
        u32x4 v = st.raw[u];
        if (bk >= 4 && tail) v = zero_tail(v, key_blk + 8 * ((p & 1) ^ vhalf_swz(p >> 1)), L);
        *reinterpret_cast<u32x4*>(dst + l_off_k0) = v;
      } else {
        const u32x4 lo = bf16x8_bits(e4m3x8_to_bf16(st.raw[u][0], st.raw[u][1]));
        const u32x4 hi = bf16x8_bits(e4m3x8_to_bf16(st.raw[u][2], st.raw[u][3]));
        if (bk < 4) {
          *reinterpret_cast<u32x4*>(dst + l_off_k0) = lo;
          *reinterpret_cast<u32x4*>(dst + l_off_k1) = hi;
        } else {
          *reinterpret_cast<u32x4*>(dst + l_off_v0) = tail ? zero_tail(lo, key_blk, L) : lo;
          *reinterpret_cast<u32x4*>(dst + l_off_v1) = tail ? zero_tail(hi, key_blk + 8, L) : hi;
        }
      }
    }
  };

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  float m_ref = -INFINITY, l_run = 0.f;

  fetch(0);
  commit(0, 0);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    if (t + 1 < ntiles) fetch(t + 1);
    if (active) {
      const int kt = r.k_begin + kAttnTile * t;
      const int lb0 = kt / 16;
      float cs[2][2], vs[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (FP8) {
          const size_t pb = phys_block(a, tbl, lb0 + j, n_blk) * a.H_kv + kvh;
          cs[j >> 1][j & 1] = a.c * a.k_scale[pb];
          vs[j] = a.v_scale[pb];
        } else {
          cs[j >> 1][j & 1] = a.c;
          vs[j] = 1.f;
        }
      }
      const uint8_t* stage = smem + (t & 1) * T::kStage;
      // every key of the tile exists and every row may see it
      if (kt + kAttnTile <= r.k_end && kt + kAttnTile - 1 <= r.P)
        lds_tile<HD, FP8, false>(a, r, stage, k_lds, v_lds, qop, cs, vs, kt, m_ref, l_run, o);
      else
        lds_tile<HD, FP8, true>(a, r, stage, k_lds, v_lds, qop, cs, vs, kt, m_ref, l_run, o);
    }
    if (t + 1 < ntiles) commit(t + 1, (t + 1) & 1);
    __syncthreads();
  }
  if (active) write_result<HD>(a, r, o, m_ref, l_run);
}

// ---------------------------------------------------------------------------
// Ring partial kernel (bf16 cache, M > 64): the same tile arithmetic on an
// NS-stage LDS ring filled by direct global->LDS loads (global_load_lds_dwordx4:
// lane i of a load writes 16 bytes at the wave's LDS base + 16 i), so NS - 1
// tiles are in flight while one is computed and no registers hold staging data.
// Each wave moves K block w and V block w of every tile; the gather addresses
// carry the slot / half swizzles of the LDS image.  One barrier per tile: the
// tile's loads are waited for with s_waitcnt vmcnt, then the barrier publishes
// them and frees the stage computed in the previous iteration for refilling.
// ---------------------------------------------------------------------------
template <int HD>
struct Ring {
  static constexpr int kLoadsPerBlock = LdsTile<HD>::kBlk / 1024;  // 1 KB per wave load
  static constexpr int kLoadsPerTile = 2 * kLoadsPerBlock;         // per thread: K and V
};

#define SV_LDS __attribute__((address_space(3)))
#define SV_CONST __attribute__((address_space(4)))

// s_waitcnt with vmcnt = n and the other counters left open.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// LDS byte address of a shared-memory location (the value M0 takes).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(SV_LDS const void*)p;
}

// 16 bytes per lane from global memory into LDS (global_load_lds_dwordx4: lane
// i's bytes land at lds + 16 i; NT: non-temporal, for data read exactly once).
// Written as inline assembly so that the compiler does not track it: its own
// bookkeeping makes every later LDS read wait for all such loads in flight (it
// cannot tell which ring stage a load fills), which would drain the ring each
// tile.  Callers order these loads with s_waitcnt vmcnt and a barrier
// themselves; loads unknown to the compiler only make its own vmcnt waits more
// conservative, never less.  The statement sets M0, so a kernel using it must
// hold no other value in M0 (no LDS-DMA builtins, no indirect register
// indexing); the stream-K kernel has no other M0 user.
template <bool NT>
__device__ __forceinline__ void dma_to_lds16(const void* src, uint32_t lds) {
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
                 :
                 : "v"(src), "s"(lds)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "s"(lds)
                 : "memory", "m0");
}

// N such loads of consecutive 1 KB pieces: piece j of the wave's source (src +
// 1024 j + 16 i for lane i) lands at lds + 1024 j + 16 i.  One M0 value serves
// all of them: the instruction's immediate offset is added to both the global
// and the LDS address.
#define SV_DMA1(off, nt) "\n\tglobal_load_lds_dwordx4 %0, off offset:" #off nt
template <bool NT, int N>
__device__ __forceinline__ void dma_to_lds16_run(const void* src, uint32_t lds) {
  static_assert(N == 1 || N == 2 || N == 4, "1, 2 or 4 pieces");
  if constexpr (NT && N == 4)
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0" SV_DMA1(0, " nt") SV_DMA1(1024, " nt")
                 SV_DMA1(2048, " nt") SV_DMA1(3072, " nt") : : "v"(src), "s"(lds) : "memory", "m0");
  else if constexpr (N == 4)
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0" SV_DMA1(0, "") SV_DMA1(1024, "")
                 SV_DMA1(2048, "") SV_DMA1(3072, "") : : "v"(src), "s"(lds) : "memory", "m0");
  else if constexpr (NT && N == 2)
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0" SV_DMA1(0, " nt") SV_DMA1(1024, " nt")
                 : : "v"(src), "s"(lds) : "memory", "m0");
  else if constexpr (N == 2)
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0" SV_DMA1(0, "") SV_DMA1(1024, "")
                 : : "v"(src), "s"(lds) : "memory", "m0");
  else
    dma_to_lds16<NT>(src, lds);
}
#undef SV_DMA1

// One 64-key tile of the bf16 LDS image.  Masked tiles (the causal tail or the
// end of the sequence) run every MFMA like unmasked ones: keys past the end are
// excluded by selects on the scores and their V values are zeroed by selects,
// never by skipping work -- MFMA instructions do not observe the EXEC mask, so a
// branch the compiler turns into lane masking would still multiply poison V
// by zero probabilities (NaN).
template <int HD, bool MASKED>
__device__ __forceinline__ void ring_tile(const RowCtx& r, const uint8_t* stage, int k_lds,
                                          int v_lds, const bf16x8 (&qop)[HD / 16], float c,
                                          int kt, float& m_ref, float& l_run,
                                          f32x16 (&o)[HD / 32]) {
  constexpr int KS = HD / 16;
  constexpr int DB = HD / 32;
  constexpr int BLK = LdsTile<HD>::kBlk;
  f32x16 x[2];
  bool live[2];
  const float cs[2][2] = {{c, c}, {c, c}};
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    live[sb] = MASKED ? (kt + 32 * sb < r.k_end) : true;
    x[sb] = f32x16{};
    const uint8_t* kb = stage + k_lds + 2 * sb * BLK;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 kop = *reinterpret_cast<const bf16x8*>(kb + ks * 512);
      x[sb] = mfma32x32x16(kop, qop[ks], x[sb]);
    }
  }
  if constexpr (!MASKED) {
    // Sub-block by sub-block: the VALU softmax of one sub-block is independent
    // of the other sub-block's MFMAs, so the two overlap within the wave.
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      float alpha;
      bf16x8 p[2];
      if (softmax_sub(x[sb], c, m_ref, l_run, alpha, p[0], p[1])) {
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] *= alpha;
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const uint8_t* vb = stage + v_lds + (4 + 2 * sb + kk) * BLK;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const bf16x8 vop = *reinterpret_cast<const bf16x8*>(vb + db * 1024);
          o[db] = mfma32x32x16(vop, p[kk], o[db]);
        }
      }
    }
    return;
  }
  float alpha;
  const bool rescale = softmax_core<MASKED>(x, cs, live, kt, r, m_ref, l_run, alpha);
  if (rescale) {
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] *= alpha;
  }
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int key0 = kt + 32 * sb + 16 * kk + 8 * r.hh;   // first key of this lane's 8
      const bf16x8 pop = p_operand(x[sb], kk, 1.f);
      const uint8_t* vb = stage + v_lds + (4 + 2 * sb + kk) * BLK;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        bf16x8 vop = *reinterpret_cast<const bf16x8*>(vb + db * 1024);
        if constexpr (MASKED) {
#pragma unroll
          for (int j = 0; j < 8; ++j) vop[j] = key0 + j < r.L ? vop[j] : (__bf16)0.f;
        }
        o[db] = mfma32x32x16(vop, pop, o[db]);
      }
    }
  }
}

// NS stages of LDS per workgroup; WPE workgroups (waves per SIMD) per CU.
template <int HD, int NS, int WPE>
__global__ __attribute__((amdgpu_flat_work_group_size(kLdsThreads, kLdsThreads),
                          amdgpu_waves_per_eu(WPE, WPE)))
void sv_attn_partial_ring(AttnArgs a) {
  constexpr int KS = HD / 16;
  constexpr int DB = HD / 32;
  constexpr int BLK = LdsTile<HD>::kBlk;
  constexpr int STAGE = LdsTile<HD>::kStage;
  constexpr int LPB = Ring<HD>::kLoadsPerBlock;
  constexpr int LPT = Ring<HD>::kLoadsPerTile;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NS * STAGE];

  const Work wk = decode_work(a, a.m_tiles);
  if (!wk.valid) return;
  const int split = wk.split, kvh = wk.kvh, mt = wk.mt, b = wk.b;
  const int L = clamp_len(a, b);
  if (split * a.split_tokens >= L) return;           // whole workgroup: no barrier yet
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int m0 = (mt * 4 + wave) * kRowsPerWave;
  const bool active = m0 < a.M;                       // inactive waves still load
  const RowCtx r = make_row_ctx(a, split, kvh, b, L, m0, lane);

  bf16x8 qop[KS];
  if (active) load_q<HD, false>(a, r, qop);

  const int32_t* tbl = a.block_table + (size_t)b * a.max_blocks;
  const int n_blk = (L + 15) / 16;
  const int ntiles = (r.k_end - r.k_begin + kAttnTile - 1) / kAttnTile;
  const size_t blk_stride = (size_t)a.H_kv * HD * 32;
  const uint8_t* kbase = a.k + (size_t)kvh * HD * 32;
  const uint8_t* vbase = a.v + (size_t)kvh * HD * 32;

  // Gather offsets of this lane for the j-th 1 KB load of a block image.
  int g_k[LPB], g_v[LPB];
#pragma unroll
  for (int j = 0; j < LPB; ++j) {
    const int p = j * kWave + lane;                    // 16-byte position in the LDS image
    g_k[j] = ((p >> 4) * 16 + swap23(p & 15)) * 16;
    g_v[j] = ((p >> 1) * 2 + ((p & 1) ^ vhalf_swz(p >> 1))) * 16;
  }
  auto issue = [&](int t) {
    const int stage = t % NS;
    const size_t pb = phys_block(a, tbl, r.k_begin / 16 + 4 * t + wave, n_blk) * blk_stride;
    const uint8_t* gk = kbase + pb;
    const uint8_t* gv = vbase + pb;
    SV_LDS uint8_t* lk = (SV_LDS uint8_t*)(smem + stage * STAGE + wave * BLK);
    SV_LDS uint8_t* lv = lk + 4 * BLK;
#pragma unroll
    for (int j = 0; j < LPB; ++j)
      __builtin_amdgcn_global_load_lds((const void*)(gk + g_k[j]), (SV_LDS void*)(lk + j * 1024), 16, 0, 0);
#pragma unroll
    for (int j = 0; j < LPB; ++j)
      __builtin_amdgcn_global_load_lds((const void*)(gv + g_v[j]), (SV_LDS void*)(lv + j * 1024), 16, 0, 0);
  };

  const int k_lds = (r.ql >> 4) * BLK + (r.ql & 15) * 16 + r.hh * 256;
  const int v_lds = (2 * r.ql + (r.hh ^ vhalf_swz(r.ql))) * 16;

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  float m_ref = -INFINITY, l_run = 0.f;

  // Prologue: tiles 0 .. NS-2 in flight (tiles past the end load clamped,
  // valid blocks and are never computed, keeping the wait counts uniform).
#pragma unroll
  for (int t = 0; t < NS - 1; ++t) issue(t);
  for (int t = 0; t < ntiles; ++t) {
    wait_vmcnt<(NS - 2) * LPT>();                     // this wave's loads of tile t landed
    __builtin_amdgcn_s_barrier();                     // ... and every other wave's
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    issue(t + NS - 1);                                // refills the stage freed by tile t-1
    if (active) {
      const int kt = r.k_begin + kAttnTile * t;
      const uint8_t* stage = smem + (t % NS) * STAGE;
      if (kt + kAttnTile <= r.k_end && kt + kAttnTile - 1 <= r.P)
        ring_tile<HD, false>(r, stage, k_lds, v_lds, qop, a.c, kt, m_ref, l_run, o);
      else
        ring_tile<HD, true>(r, stage, k_lds, v_lds, qop, a.c, kt, m_ref, l_run, o);
    }
  }
  wait_vmcnt<0>();                                    // drain loads issued past the end
  if (active) write_result<HD>(a, r, o, m_ref, l_run);
}

// ---------------------------------------------------------------------------
// Stream-K persistent kernel (bf16 cache, row tiles of 128).
//
// Work is the list of (sequence b, KV head, row tile, 32-key tile) in that
// order: unit u = (b, kvh, mt) owns T_b = ceil(L_b / 32) consecutive tiles.
// A fixed grid of P workgroups splits the W tiles of the whole batch into equal
// contiguous ranges of Wp = max(ceil(W / P), min_tiles) tiles, so every
// workgroup streams the same number of tiles regardless of how ragged the
// lengths are, and its LDS ring stays full across unit boundaries.  A unit
// whose tiles all fall in one range is finished in place (O / l written as
// bf16); a unit cut by range boundaries leaves one unnormalised (O, m, l)
// segment per range -- at most the first and the last segment of each range
// -- which sv_attn_streamk_merge combines with the split-merge rule.
// Every workgroup computes the per-sequence tile prefix from kv_lens in LDS;
// workgroup 0 also stores it (with W and Wp) for the merge kernel.
//
// A tile is one 32-key sub-block (16 KB of K and V at hd 128); the 64 KB ring
// of each of the two workgroups on a compute unit holds four stages: the tile
// being computed, the next one (whose scores are computed early) and two in
// flight.  (A fifth stage, which LDS would allow now that the prefix table
// lives in the ring, measured no faster.)
// ---------------------------------------------------------------------------
constexpr int kStreamRows = 128;          // rows per unit of 4 waves x 32 (8-wave units: 256)
constexpr int kSkKeys = 32;               // keys per stream-K tile

#ifndef SV_STREAM_RING_BYTES
#define SV_STREAM_RING_BYTES 65536
#endif

template <int HD>
struct SkTile {
  static constexpr int kBlk = LdsTile<HD>::kBlk;   // one 16-key block of K or V
  static constexpr int kStage = 4 * kBlk;          // K blocks 0, 1, then V blocks 0, 1
  static constexpr int kLoads = kBlk / 1024;       // 1 KB wave loads per block
  static constexpr int kStages = SV_STREAM_RING_BYTES / kStage;
  static constexpr int kStages8 = 2 * SV_STREAM_RING_BYTES / kStage;   // one 8-wave workgroup per CU
};

// pref[b] = tiles of all units of sequences before b, for b = 0 .. B.
__device__ __forceinline__ void build_prefix(const AttnArgs& a, int* pref, int* wsum) {
  const int tid = threadIdx.x;
  const int lane = tid % kWave, wave = tid / kWave;
  const int per_seq = a.H_kv * a.m_tiles;
  const int nthreads = (int)blockDim.x;
  const int chunk = (a.B + nthreads - 1) / nthreads;
  const int lo = min(tid * chunk, a.B), hi = min(lo + chunk, a.B);
  int sum = 0;
  for (int b = lo; b < hi; ++b) {
    sum += ((clamp_len(a, b) + kSkKeys - 1) / kSkKeys) * per_seq;
    pref[b + 1] = sum;                      // inclusive within this thread's chunk
  }
  // exclusive scan of the per-thread sums: within each wave, then across waves
  int incl = sum;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int v = __shfl_up(incl, off);
    if (lane >= off) incl += v;
  }
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += wsum[w];
  const int excl = base + incl - sum;
  for (int b = lo; b < hi; ++b) pref[b + 1] += excl;
  if (tid == 0) pref[0] = 0;
  __syncthreads();
}

// Position in the work list: sequence b, unit ul = kvh * m_tiles + mt within
// the sequence, tile within the unit, and the unit's tile count T; kvh, mt and
// the offset of sequence b's block-table row are kept alongside, so that the
// per-tile path does no division or wide multiply.
struct Cursor {
  int b, tile, T;
  int kvh, mt;
  const int32_t* row;
};

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ Cursor cursor_at(const AttnArgs& a, const int* pref, int g) {
  int lo = 0, hi = a.B;                     // pref[lo] <= g < pref[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (uniform(pref[mid]) <= g) lo = mid; else hi = mid;
  }
  const int per_seq = a.H_kv * a.m_tiles;
  Cursor c;
  c.b = lo;
  c.T = uniform((pref[lo + 1] - pref[lo]) / per_seq);
  const int r = g - uniform(pref[lo]);
  const int ul = r / c.T;                   // unit within the sequence: kvh * m_tiles + mt
  c.tile = r % c.T;
  c.kvh = ul / a.m_tiles;
  c.mt = ul % a.m_tiles;
  c.row = a.block_table + (size_t)c.b * a.max_blocks;
  return c;
}

// Tiles of each unit of sequence b (the per-sequence count build_prefix sums).
__device__ __forceinline__ int unit_tiles(const AttnArgs& a, int b) {
  return (clamp_len_s(a, b) + kSkKeys - 1) / kSkKeys;
}

// Advances to the next tile of the work list.  The tile count of a new
// sequence comes from kv_lens (a scalar load, once per sequence), so the
// prefix table is needed only to place a range's first tile.
__device__ __forceinline__ void cursor_next(const AttnArgs& a, Cursor& c) {
  if (++c.tile < c.T) return;
  c.tile = 0;
  if (++c.mt < a.m_tiles) return;
  c.mt = 0;
  if (++c.kvh < a.H_kv) return;
  c.kvh = 0;
  do {
    ++c.b;
  } while (c.b < a.B && (c.T = unit_tiles(a, c.b)) == 0);
  c.row = a.block_table + (size_t)c.b * a.max_blocks;
}

// Partial O of one wave in a segment slot: O / (l f) of its rows as fp16, in
// the accumulator layout: f16x8 number (db * 2 + h) * 64 + lane holds
// registers 8 h .. 8 h + 7 of accumulator block db of that lane (row 32 w +
// lane % 32; register 4 q4 + e is dim 32 db + 8 q4 + 4 (lane / 32) + e).  f is
// the row's power of two (ws_f) that puts its largest |O / l| in [2^14, 2^15).
template <int HD>
__device__ __forceinline__ f16x8* sk_partial_o(const AttnArgs& a, int slot, int wave) {
  return reinterpret_cast<f16x8*>(a.ws_o) + ((size_t)slot * a.sk_rows + wave * kRowsPerWave) * (HD / 8);
}

// Zeroes the V values of keys >= L in the tile image at stage (keys kt ..
// kt + 31), so that poison past the end of the sequence never meets the zero
// probabilities of those keys in the PV product (MFMA instructions do not
// observe the EXEC mask, so lane masking could not keep it out).
template <int HD>
__device__ __forceinline__ void sk_zero_v_tail(uint8_t* stage, int kt, int L) {
  constexpr int BLK = SkTile<HD>::kBlk;
  constexpr int POS = 2 * HD;                // 16-byte vectors per V block image
  for (int i = threadIdx.x; i < 2 * POS; i += blockDim.x) {
    const int bk = i / POS, p = i % POS;
    const int d = p >> 1, h = (p & 1) ^ vhalf_swz(d);
    const int key0 = kt + 16 * bk + 8 * h;
    if (key0 + 8 > L) {
      u32x4* v = reinterpret_cast<u32x4*>(stage + (2 + bk) * BLK + p * 16);
      *v = zero_tail(*v, key0, L);
    }
  }
}

// Scores of one 32-key tile, transposed (keys x rows), from the K image of a
// ring stage.
template <int HD>
__device__ __forceinline__ f32x16 sk_scores(const uint8_t* stage, int k_lds,
                                            const bf16x8 (&qop)[HD / 16]) {
  f32x16 x = f32x16{};
#pragma unroll
  for (int ks = 0; ks < HD / 16; ++ks) {
    const bf16x8 kop = *reinterpret_cast<const bf16x8*>(stage + k_lds + ks * 512);
    x = mfma32x32x16(kop, qop[ks], x);
  }
  return x;
}

// Tiles that reach past a row's last visible key (the causal tail, which
// covers keys past the end) exclude those keys by a select on the scores.
__device__ __forceinline__ void sk_mask(f32x16& x, const RowCtx& r, int kt) {
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int key = kt + key_of_row(8 * (v >> 2) + 4 * r.hh + (v & 3));
    x[v] = key > r.vis_last ? -INFINITY : x[v];
  }
}

// Tree verification: new position j (key P + j) holds draft-tree node j, and
// node i sees the context and the nodes set in its ancestor mask (itself and
// its ancestors).  The mask is read here, on the tiles that reach past P only;
// the load's wait is the compiler's own, which only adds to the ring's waits.
__device__ __forceinline__ void sk_mask_tree(f32x16& x, const RowCtx& r, int kt, const AttnArgs& a) {
  const uint64_t live = a.R == 64 ? ~0ull : ((1ull << a.R) - 1);
  const uint64_t anc = tree_masks(a)[(size_t)r.b * a.R + r.pos] & live;
  // The shift amount is clamped into [0, 63] before the shift: the selects
  // below evaluate the shift for every key, and an out-of-range amount (a
  // context key, j < 0) must not reach it.
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int j = kt + key_of_row(8 * (v >> 2) + 4 * r.hh + (v & 3)) - r.P;
    const uint32_t sh = (uint32_t)min(max(j, 0), 63);
    const bool in_tree = ((anc >> sh) & 1ull) != 0;
    const bool hidden = j >= 0 && (j >= a.R || !in_tree);
    x[v] = hidden ? -INFINITY : x[v];
  }
}

// V operands of one tile (V past the end of the sequence already zeroed).
template <int HD>
__device__ __forceinline__ void sk_read_v(const uint8_t* stage, int v_lds,
                                          bf16x8 (&vop)[2][HD / 32]) {
  constexpr int BLK = SkTile<HD>::kBlk;
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int db = 0; db < HD / 32; ++db)
      vop[kk][db] = *reinterpret_cast<const bf16x8*>(stage + v_lds + (2 + kk) * BLK + db * 1024);
}

// O += P V for one tile.
template <int HD>
__device__ __forceinline__ void sk_pv(const bf16x8 (&vop)[2][HD / 32], const bf16x8 (&p)[2],
                                      f32x16 (&o)[HD / 32]) {
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int db = 0; db < HD / 32; ++db) o[db] = mfma32x32x16(vop[kk][db], p[kk], o[db]);
}

// Ends a segment of a stream-K range: the unit's output rows when the segment
// covers the whole unit, else (O / l in fp16 with a power-of-two factor per
// row, m, l) in segment slot `slot` (the range's first segment or its last
// one).  Two bytes per element instead of fp32 O halve the writes in the
// middle of the K/V stream (they cost the reads several times their size) and
// the merge's reads; the per-row factor keeps fp16's 11-bit precision relative
// to the row's largest value whatever V's range.  Stored in the accumulator
// layout (sk_partial_o), every store instruction writing 1 KB of consecutive
// bytes, non-temporal.
template <int HD>
__device__ __forceinline__ void sk_segment_end(const AttnArgs& a, RowCtx& r,
                                               const f32x16 (&o)[HD / 32], float m_ref,
                                               float l_run, bool whole, int slot, int wave,
                                               int lane) {
  if (whole) {
    r.n_splits = 1;
    write_result<HD>(a, r, o, m_ref, l_run);
    return;
  }
  const float l_tot = halves_sum(l_run);
  float mx = 0.f;                             // largest |O| of the row (both half-waves)
#pragma unroll
  for (int db = 0; db < HD / 32; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) mx = fmaxf(mx, fabsf(o[db][e]));
  mx = halves_max(mx);
  // O / l * 2^(15 - ex) with |O| / l < 2^ex: the row's values below 2^15, so
  // the fp16 result is finite; f = 2^(ex - 15) undoes it.  l = 0 or O = 0
  // (no visible key, or all-zero V): factor 1 and zeros.
  const float ol = (l_tot > 0.f) ? mx / l_tot : 0.f;
  // (ex clamped: with l >= 1 whenever a key is visible, 2^(15 - ex) / l stays finite)
  const int ex = (ol > 0.f) ? min(max(__builtin_amdgcn_frexp_expf(ol), -100), 127) : 15;
  const float inv = (l_tot > 0.f) ? __builtin_amdgcn_ldexpf(1.f / l_tot, 15 - ex) : 0.f;
  f16x8* dst = sk_partial_o<HD>(a, slot, wave) + lane;
#pragma unroll
  for (int db = 0; db < HD / 32; ++db)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      f16x8 v;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = (_Float16)(o[db][8 * h + e] * inv);
      __builtin_nontemporal_store(v, dst + (db * 2 + h) * kWave);
    }
  if (lane < 32)
    __builtin_nontemporal_store(__builtin_amdgcn_ldexpf(1.f, ex - 15),
                                a.ws_f + (size_t)slot * a.sk_rows + wave * kRowsPerWave + lane);
  if (lane < 32)
    __builtin_nontemporal_store(f32x2{m_ref, l_tot},
                                a.ws_ml + (size_t)slot * a.sk_rows + wave * kRowsPerWave + lane);
}

// NT: K/V loads are non-temporal, for row tilings where each unit's K and V are
// read by that unit alone (one row tile per KV head).  WAVES = 4 (units of 128
// rows, two workgroups per CU) or 8 (units of 256 rows, one per CU), so that
// up to 256 rows of one KV head stream its K and V once.
// TREE: draft-tree verification (ancestor masks instead of the causal chain).
template <int HD, int NS, int WPE, bool NT, int WAVES, bool TREE>
__global__ __attribute__((amdgpu_flat_work_group_size(WAVES * 64, WAVES * 64),
                          amdgpu_waves_per_eu(WPE, WPE)))
void sv_attn_streamk(AttnArgs a) {
  constexpr int KS = HD / 16;
  constexpr int DB = HD / 32;
  constexpr int BLK = SkTile<HD>::kBlk;
  constexpr int STAGE = SkTile<HD>::kStage;
  constexpr int LPB = SkTile<HD>::kLoads;
  static_assert(NS >= 3, "the ring holds the computed tile, the next one and one in flight");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NS * STAGE];
  // The prefix table only places the range's first tile: it lives in the ring
  // until the ring's first loads are issued.
  constexpr int ROWS = WAVES * kRowsPerWave;
  constexpr int WPB = WAVES / 4;               // waves sharing one block image of a tile
  constexpr int LPW = LPB / WPB;               // 1 KB loads per wave per tile
  static_assert(WAVES == 4 || WAVES == 8, "4 or 8 waves");
  static_assert((kStreamMaxBatch + 1 + WAVES) * 4 <= NS * STAGE, "prefix table fits");
  int* s_pref = reinterpret_cast<int*>(smem);
  int* s_wsum = s_pref + kStreamMaxBatch + 1;

  build_prefix(a, s_pref, s_wsum);
  const int W = uniform(s_pref[a.B]);
  const int Wp = max((W + (int)gridDim.x - 1) / (int)gridDim.x, a.min_tiles);
  const int tid = threadIdx.x;
  if (blockIdx.x == 0) {
    for (int b = tid; b <= a.B; b += WAVES * kWave) a.sk_meta[2 + b] = s_pref[b];
    if (tid == 0) {
      a.sk_meta[0] = W;
      a.sk_meta[1] = Wp;
    }
  }
  const int g0 = (int)blockIdx.x * Wp;
  const int g1 = min(g0 + Wp, W);
  if (g0 >= g1) return;                       // whole workgroup, after the last barrier use

  const int wave = uniform(tid / kWave);
  const int lane = tid % kWave;
  const int ql = lane & 31, hh = lane >> 5;
  const size_t blk_stride = (size_t)a.H_kv * HD * 32;

  // Wave w moves 1 KB chunks j0 .. j0 + LPW - 1 of block image bw of every
  // tile (bw: K block 0, K block 1, V block 0, V block 1); gather offsets of
  // this lane for each of its loads.
  const int bw = wave / WPB;
  const int j0 = (wave % WPB) * LPW;
  // The permutations act within 1 KB pieces (K: 16-byte vectors within 256
  // bytes; V: the two halves of a key pair, chosen by key bits 2 and 3), so
  // chunk j starts 1 KB after chunk 0 and one offset serves all of them.
  const bool moves_v = bw >= 2;
  const uint8_t* src = moves_v ? a.v : a.k;
  const uint32_t blk_stride32 = (uint32_t)blk_stride;   // below 2^32 (the planner checks)
  const int p0 = j0 * kWave + lane;
  const int g_off = moves_v ? ((p0 >> 1) * 2 + ((p0 & 1) ^ vhalf_swz(p0 >> 1))) * 16
                            : ((p0 >> 4) * 16 + swap23(p0 & 15)) * 16;
  const int k_lds = (ql >> 4) * BLK + (ql & 15) * 16 + hh * 256;
  const int v_lds = (2 * ql + (hh ^ vhalf_swz(ql))) * 16;

  // Table entry of the cache block this wave moves for the tile at c, read
  // with a scalar load: vector memory operations complete in issue order, so a
  // vector load of the entry would make its first use wait for every tile load
  // issued before it.  Scalar loads are counted apart from them.  The entry is
  // read one tile before its tile's loads are issued.  Entries past the
  // sequence's last block may be read (the column is clamped to the table's
  // width only); they only feed keys past the end, which are masked.
  auto entry = [&](const Cursor& c) -> int {
    const SV_CONST int32_t* row = (const SV_CONST int32_t*)c.row;
    return row[(unsigned)min(2 * c.tile + (bw & 1), a.max_blocks - 1)];
  };
  // Loads of one tile into ring stage `stage`: this wave's chunks of block bw.
  auto issue = [&](const Cursor& c, int raw, int stage) {
    const uint32_t pb = (uint32_t)min(max(raw, 0), a.num_blocks - 1);
    const uint8_t* g = src + ((uint64_t)pb * blk_stride32 + (uint32_t)(c.kvh * HD * 32));
    const uint32_t l = lds_addr(smem) + stage * STAGE + bw * BLK + j0 * 1024;
    dma_to_lds16_run<NT, LPW>(g + g_off, l);
  };

  Cursor ci = cursor_at(a, s_pref, g0);      // next tile to load (index gi)
  Cursor cc = ci;                             // tile being computed
  __syncthreads();                            // the prefix table is dead: the ring may fill

  // Row context of the segment of the tile at c; whether this wave has rows.
  auto seg_ctx = [&](const Cursor& c, RowCtx& rr) -> bool {
    const int m0 = c.mt * ROWS + wave * kRowsPerWave;
    const int L = clamp_len_s(a, c.b);
    rr = make_row_ctx(a, 0, c.kvh, c.b, L, m0, lane);
    rr.k_end = L;
    return m0 < a.M;
  };
  RowCtx r, rn;                                // segment of tile g; the next segment
  bool active = seg_ctx(cc, r), active_n = false;
  int seg_start = g0;
  bf16x8 qop[KS], qn[KS];
  if (active) load_q<HD, false>(a, r, qop);
  wait_vmcnt<0>();                             // Q before the ring's loads, waited once

  int gi = g0;
  int ent = entry(ci);                        // table entry of the tile at ci
#pragma unroll
  for (int k = 0; k < NS - 1; ++k) {         // past the range: the last tile again
    issue(ci, ent, k);
    if (gi + 1 < g1) cursor_next(a, ci);
    ++gi;
    ent = entry(ci);
  }

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  f32x16 xn;                                   // scores of tile g + 1, when have_xn
  bool have_xn = false;
  float m_ref = kNoMax, l_run = 0.f;
  for (int g = g0; g < g1; ++g) {
    const unsigned t = (unsigned)(g - g0);    // unsigned: stage indices are cheap remainders
    // This wave's loads of tiles g and g + 1 landed: loads retire in issue
    // order, so at most tile g + 2's loads (and stores issued after them) are
    // still counted.
    wait_vmcnt<(NS - 3) * LPW>();
    __builtin_amdgcn_s_barrier();              // ... and every other wave's
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");

    if (g != g0 && cc.tile == 0) {             // a new segment, prepared one tile ago
      seg_start = g;
      r = rn;
      active = active_n;
      const bf16x8 z = {};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qop[ks] = r.row_ok ? qn[ks] : z;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] = f32x16{};
      m_ref = kNoMax;
      l_run = 0.f;
      have_xn = false;
    }
    // The next tile starts a segment: its row context and Q are loaded now,
    // ahead of this tile's ring loads, so that using them next tile waits for
    // nothing issued later.
    if (g + 1 < g1 && cc.tile + 1 == cc.T) {
      Cursor cn = cc;
      cursor_next(a, cn);
      active_n = seg_ctx(cn, rn);
      if (active_n) load_q_raw<HD>(a, rn, qn);
    }
    issue(ci, ent, (t + NS - 1) % NS);         // refills the stage freed by tile g - 1
    if (gi + 1 < g1) cursor_next(a, ci);
    ++gi;
    ent = entry(ci);

    const int kt = cc.tile * kSkKeys;
    uint8_t* stage = smem + (t % NS) * STAGE;
    if (kt + kSkKeys > r.L) {                  // the sequence's last tile (same for all waves)
      sk_zero_v_tail<HD>(stage, kt, r.L);
      __syncthreads();
    }
    if (active) {
      // Software pipeline within the wave: the scores of tile g + 1 are
      // computed (MFMA) while the softmax of tile g runs (VALU); they are kept
      // when tile g + 1 continues this segment, which has the same Q.
      f32x16 x = have_xn ? xn : sk_scores<HD>(stage, k_lds, qop);
      if (kt + kSkKeys - 1 > r.P) {            // unless every key is visible to every row
        if constexpr (TREE) sk_mask_tree(x, r, kt, a);
        else sk_mask(x, r, kt);
      }
      xn = sk_scores<HD>(smem + ((t + 1) % NS) * STAGE, k_lds, qop);
      bf16x8 vop[2][DB];
      sk_read_v<HD>(stage, v_lds, vop);
      float alpha;
      bf16x8 p[2];
      const bool rescale = softmax_sub_sk(x, a.c, m_ref, l_run, alpha, p[0], p[1]);
      // Keep the probabilities and V operands in this block (ahead of the
      // rescale branch), and interleave: the next tile's K reads and this
      // tile's V reads first, then each of the next tile's score MFMAs
      // followed by a share of this tile's softmax VALU work.
      asm volatile("" : : "v"(p[0]), "v"(p[1]), "v"(l_run));
      __builtin_amdgcn_sched_group_barrier(0x100, KS + 2 * DB, 0);  // DS reads
#pragma unroll
      for (int i = 0; i < KS; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 10, 0);         // ten VALU
      }
      if (rescale) {
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] *= alpha;
      }
      sk_pv<HD>(vop, p, o);
    }
    have_xn = g + 1 < g1 && cc.tile + 1 < cc.T;
    if (cc.tile == cc.T - 1 || g == g1 - 1) {  // the segment ends
      if (active)
        sk_segment_end<HD>(a, r, o, m_ref, l_run,
                           cc.tile == cc.T - 1 && seg_start == g - cc.tile,
                           (int)blockIdx.x * 2 + (seg_start == g0 ? 0 : 1), wave, lane);
    }
    if (g + 1 < g1) cursor_next(a, cc);
  }
  wait_vmcnt<0>();                             // drain loads issued past the range
}

// Stream-K kernel for e4m3 caches.  The same work list, ranges, segments and
// merge as the bf16 kernel; what differs is the tile supply.  A 16-key block
// of e4m3 K or V is hd x 16 codes (half the bf16 bytes): the codes of NS8
// tiles stream through a DMA ring, and at every tile each wave decodes the
// block it moved for the next tile -- codes times the block's scale, rounded
// once to bf16 -- into one of two bf16 images laid out like a bf16 ring
// stage (V past the end of the sequence zeroed), on which the tile is then
// computed exactly as in the bf16 kernel.
template <int HD>
struct SkTile8 {
  static constexpr int kBlk = HD * 16;       // bytes of one block of e4m3 K or V
  static constexpr int kStage = 4 * kBlk;    // K blocks 0, 1, then V blocks 0, 1
  static constexpr int kLoads = kBlk / 1024; // 1 KB wave loads per block
  static constexpr int kStages = 3;
};

template <int HD, int WPE, bool NT, bool TREE>
__global__ __attribute__((amdgpu_flat_work_group_size(kLdsThreads, kLdsThreads),
                          amdgpu_waves_per_eu(WPE, WPE)))
void sv_attn_streamk_fp8(AttnArgs a) {
  constexpr int KS = HD / 16;
  constexpr int DB = HD / 32;
  constexpr int BLK = SkTile<HD>::kBlk;      // bf16 image
  constexpr int STAGE = SkTile<HD>::kStage;
  constexpr int BLK8 = SkTile8<HD>::kBlk;    // e4m3 ring
  constexpr int STAGE8 = SkTile8<HD>::kStage;
  constexpr int LPB = SkTile8<HD>::kLoads;
  constexpr int NS8 = SkTile8<HD>::kStages;
  __shared__ __attribute__((aligned(1024))) uint8_t ring8[NS8 * STAGE8];
  __shared__ __attribute__((aligned(1024))) uint8_t img[3 * STAGE];
  __shared__ f32x4 s_mant[3];                 // per image: mantissas of K0, K1, V0, V1 scales
  __shared__ float s_sink[kLdsThreads];       // put_mant's stores by lanes other than 0
  // the prefix table lives in the images until the first tile is decoded
  static_assert((kStreamMaxBatch + 1 + kLdsThreads / kWave) * 4 <= 3 * STAGE, "prefix table fits");
  static_assert(NS8 == 3, "the prologue below fills a three-stage code ring");
  int* s_pref = reinterpret_cast<int*>(img);
  int* s_wsum = s_pref + kStreamMaxBatch + 1;

  build_prefix(a, s_pref, s_wsum);
  const int W = uniform(s_pref[a.B]);
  const int Wp = max((W + (int)gridDim.x - 1) / (int)gridDim.x, a.min_tiles);
  const int tid = threadIdx.x;
  if (blockIdx.x == 0) {
    for (int b = tid; b <= a.B; b += kLdsThreads) a.sk_meta[2 + b] = s_pref[b];
    if (tid == 0) {
      a.sk_meta[0] = W;
      a.sk_meta[1] = Wp;
    }
  }
  const int g0 = (int)blockIdx.x * Wp;
  const int g1 = min(g0 + Wp, W);
  if (g0 >= g1) return;                       // whole workgroup, after the last barrier use

  const int wave = uniform(tid / kWave);
  const int lane = tid % kWave;
  const int ql = lane & 31, hh = lane >> 5;
  const size_t blk_stride = (size_t)a.H_kv * BLK8;

  // Wave w moves (and decodes) block w % 2 of the tile's K (w < 2) or V (w >= 2).
  const bool moves_v = wave >= 2;
  const uint8_t* src = moves_v ? a.v : a.k;
  const SV_CONST float* scales = (const SV_CONST float*)(moves_v ? a.v_scale : a.k_scale);
  const int k_lds = (ql >> 4) * BLK + (ql & 15) * 16 + hh * 256;
  const int v_lds = (2 * ql + (hh ^ vhalf_swz(ql))) * 16;

  // Table entry of this wave's block of the tile at c (a scalar load, as in
  // the bf16 kernel; entries past the sequence's last block may be read).
  auto entry = [&](const Cursor& c) -> int {
    const SV_CONST int32_t* row = (const SV_CONST int32_t*)c.row;
    return row[(unsigned)min(2 * c.tile + (wave & 1), a.max_blocks - 1)];
  };
  // Codes of one tile into ring stage `stage` (linear copy of the block); the
  // block's scale is returned (a scalar load, first used a tile later).
  // K codes land in the ring with the slots of each 16-dim group permuted like
  // the image (bits 2 and 3 of the slot swapped), so that the decode reads and
  // writes 16-byte vectors in lane order (writes in image order spread eight
  // consecutive lanes over two 64-byte halves of 128 bytes: a bank conflict).
  // The permutation stays inside 256 bytes, so one offset serves every 1 KB piece.
  const uint32_t blk_stride32 = (uint32_t)blk_stride;   // below 2^32 (the planner checks)
  const int g_off8 = moves_v ? lane * 16 : ((lane >> 4) * 16 + swap23(lane & 15)) * 16;
  auto issue = [&](const Cursor& c, int raw, int stage) -> float {
    const uint32_t pb = (uint32_t)min(max(raw, 0), a.num_blocks - 1);
    const uint8_t* g = src + ((uint64_t)pb * blk_stride32 + (uint32_t)(c.kvh * BLK8));
    const uint32_t l = lds_addr(ring8) + stage * STAGE8 + wave * BLK8;
    dma_to_lds16_run<NT, LPB>(g + g_off8, l);
    return scales[pb * (uint32_t)a.H_kv + (uint32_t)c.kvh];
  };
  // Decoding this wave's block of a tile: the codes of ring stage `stage`
  // (read first, so that the conversion can overlap MFMA work), then their
  // bf16 values into image `im`.  V past the end of the sequence is zeroed
  // later, on the image, for the sequence's last tile only.
  auto dec_read = [&](int stage, u32x4 (&raw)[LPB]) {
    const uint8_t* s8 = ring8 + stage * STAGE8 + wave * BLK8;
#pragma unroll
    for (int j = 0; j < LPB; ++j) raw[j] = *reinterpret_cast<const u32x4*>(s8 + (j * kWave + lane) * 16);
  };
  // Image offsets of the two bf16 vectors each code vector becomes (K: 16
  // dims of the key slot image position p % 16 holds; V: 16 key slots of dim
  // p), fixed per lane.
  int off_lo[LPB], off_hi[LPB];
#pragma unroll
  for (int j = 0; j < LPB; ++j) {
    const int p = j * kWave + lane;
    const int k_off = ((2 * (p >> 4)) * 16 + (p & 15)) * 16;
    off_lo[j] = wave * BLK + (moves_v ? (2 * p + vhalf_swz(p)) * 16 : k_off);
    off_hi[j] = wave * BLK + (moves_v ? (2 * p + (1 ^ vhalf_swz(p))) * 16 : k_off + 256);
  }
  // The scale's power of two goes into the conversion; its mantissa is kept
  // for the softmax (put_mant, a store by one lane: kept out of the compute
  // block, whose instruction schedule a branch would split).
  auto dec_write = [&](const u32x4 (&raw)[LPB], int im, float scale) {
    uint8_t* dst = img + im * STAGE;             // K blocks 0, 1 then V blocks 0, 1
    float pow2, mant;
    split_scale(scale, pow2, mant);
#pragma unroll
    for (int j = 0; j < LPB; ++j) {
      u32x4 lo, hi;
      e4m3x16_pow2_bf16(raw[j], pow2, lo, hi);
      *reinterpret_cast<u32x4*>(dst + off_lo[j]) = lo;
      *reinterpret_cast<u32x4*>(dst + off_hi[j]) = hi;
    }
  };
  auto put_mant = [&](int im, float scale) {
    float pow2, mant;
    split_scale(scale, pow2, mant);
    // lane 0 stores into the slot, the others into sinks of their own: one
    // store, no branch
    float* dst = lane == 0 ? reinterpret_cast<float*>(&s_mant[im]) + wave : &s_sink[tid];
    *dst = mant;
  };

  Cursor ci = cursor_at(a, s_pref, g0);      // next tile to load (index gi)
  Cursor cc = ci;                             // tile being computed
  __syncthreads();                            // the prefix table is dead: images may be written
  auto seg_ctx = [&](const Cursor& c, RowCtx& rr) -> bool {
    const int m0 = c.mt * kStreamRows + wave * kRowsPerWave;
    const int L = clamp_len_s(a, c.b);
    rr = make_row_ctx(a, 0, c.kvh, c.b, L, m0, lane);
    rr.k_end = L;
    return m0 < a.M;
  };
  RowCtx r, rn;                                // segment of tile g; the next segment
  bool active = seg_ctx(cc, r), active_n = false;
  int seg_start = g0;
  bf16x8 qop[KS], qn[KS];
  if (active) load_q<HD, false>(a, r, qop);
  wait_vmcnt<0>();                             // Q before the ring's loads, waited once

  // Tile t of the range (t = g - g0) is decoded into image t % 3 two tiles
  // ahead of its computation; its scores are computed (MFMA) one tile ahead,
  // under the softmax of the tile before it, as in the bf16 kernel.  sq holds
  // the scales of the tiles loaded but not yet decoded, oldest first.  The
  // code ring has three stages too: i0, i1, i2 = t, t + 1, t + 2 modulo 3
  // index both, rotated once per tile.
  int gi = g0;
  int ent = entry(ci);
  float sq[NS8];
  auto load_next = [&](int stage) -> float {  // past the range: the last tile again
    const float sc = issue(ci, ent, stage);
    if (gi + 1 < g1) cursor_next(a, ci);
    ++gi;
    ent = entry(ci);
    return sc;
  };
  auto decode_now = [&](int stage, int im, float scale) {
    u32x4 raw[LPB];
    dec_read(stage, raw);
    dec_write(raw, im, scale);
    put_mant(im, scale);
  };
#pragma unroll
  for (int k = 0; k < NS8; ++k) sq[k] = load_next(k);   // tiles 0, 1, 2
  wait_vmcnt<2 * LPB>();                       // this wave's codes of tile 0
  decode_now(0, 0, sq[0]);
  sq[0] = sq[1];
  sq[1] = sq[2];
  sq[2] = load_next(0);                        // tile 3
  wait_vmcnt<2 * LPB>();                       // ... of tile 1
  decode_now(1, 1, sq[0]);
  sq[0] = sq[1];
  sq[1] = sq[2];
  sq[2] = load_next(1);                        // tile 4

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  f32x16 xn;                                   // scores of tile g + 1, when have_xn
  bool have_xn = false;
  float m_ref = kNoMax, l_run = 0.f;
  int i0 = 0, i1 = 1, i2 = 2;
  for (int g = g0; g < g1; ++g) {
    // this wave's codes of tile g + 2 landed (tiles g + 3, g + 4 may not have:
    // loads retire in issue order)
    wait_vmcnt<2 * LPB>();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();              // images of tiles g, g + 1 complete; tile g - 1's free
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");

    if (g != g0 && cc.tile == 0) {             // a new segment, prepared one tile ago
      seg_start = g;
      r = rn;
      active = active_n;
      const bf16x8 z = {};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qop[ks] = r.row_ok ? qn[ks] : z;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] = f32x16{};
      m_ref = kNoMax;
      l_run = 0.f;
      have_xn = false;
    }
    if (g + 1 < g1 && cc.tile + 1 == cc.T) {   // the next tile starts a segment
      Cursor cn = cc;
      cursor_next(a, cn);
      active_n = seg_ctx(cn, rn);
      if (active_n) load_q_raw<HD>(a, rn, qn);
    }
    // codes of tile g + 2 (decoded in this tile's compute block; past the
    // range the stage holds the last tile again: decoded, never used)
    u32x4 raw[LPB];
    dec_read(i2, raw);
    const float dscale = sq[0];
    put_mant(i2, dscale);                      // tile g - 1, the image's last user, is done

    const int kt = cc.tile * kSkKeys;
    uint8_t* im = img + i0 * STAGE;
    if (kt + kSkKeys > r.L) {                  // the sequence's last tile (same for all waves)
      sk_zero_v_tail<HD>(im, kt, r.L);
      __syncthreads();
    }
    if (active) {
      f32x16 x = have_xn ? xn : sk_scores<HD>(im, k_lds, qop);
      if (kt + kSkKeys - 1 > r.P) {            // unless every key is visible to every row
        if constexpr (TREE) sk_mask_tree(x, r, kt, a);
        else sk_mask(x, r, kt);
      }
      xn = sk_scores<HD>(img + i1 * STAGE, k_lds, qop);
      const f32x4 mt4 = s_mant[i0];
      float alpha;
      bf16x8 p[2];
      const bool rescale = softmax_sub_fp8(x, a.c * mt4[0], a.c * mt4[1], mt4[2], mt4[3], m_ref,
                                           l_run, alpha, p[0], p[1]);
      dec_write(raw, i2, dscale);
      // probabilities and the decode stay ahead of the rescale branch; the
      // next tile's score MFMAs interleave with the VALU work
      asm volatile("" : : "v"(p[0]), "v"(p[1]), "v"(l_run));
      __builtin_amdgcn_sched_group_barrier(0x100, KS, 0);           // DS reads
#pragma unroll
      for (int i = 0; i < KS; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);         // VALU
      }
      if (rescale) {
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] *= alpha;
      }
      // V reads all issued ahead of the PV MFMAs (the score operands are dead)
      bf16x8 vop[2][DB];
      sk_read_v<HD>(im, v_lds, vop);
      sk_pv<HD>(vop, p, o);
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * DB, 0);       // DS reads
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * DB, 0);       // MFMA
    } else {
      dec_write(raw, i2, dscale);
    }
    have_xn = g + 1 < g1 && cc.tile + 1 < cc.T;
    // refill the stage just decoded (its codes were consumed above)
    sq[0] = sq[1];
    sq[1] = sq[2];
    sq[2] = load_next(i2);
    if (cc.tile == cc.T - 1 || g == g1 - 1) {  // the segment ends
      if (active)
        sk_segment_end<HD>(a, r, o, m_ref, l_run,
                           cc.tile == cc.T - 1 && seg_start == g - cc.tile,
                           (int)blockIdx.x * 2 + (seg_start == g0 ? 0 : 1), wave, lane);
    }
    if (g + 1 < g1) cursor_next(a, cc);
    const int i_next = i0;
    i0 = i1;
    i1 = i2;
    i2 = i_next;
  }
  wait_vmcnt<0>();                             // drain loads issued past the range
}

// Combines the segments of units that straddle range boundaries.  One
// workgroup per (unit, 32-row block w); its wave db takes the 32-dim block db,
// laid out like wave w of the stream-K workgroup (lane l holds row 32 w + l %
// 32 in the accumulator layout), so every partial-O read is 1 KB of
// consecutive bytes.  A unit's tiles [C, C + T) were split over ranges i = C /
// Wp .. (C + T - 1) / Wp, and range i holds its segment in slot 0 when the
// range starts inside the unit, else (the unit began earlier) in slot 1.  The
// segments are merged four at a time with the split-merge rule applied online
// (running max mu; the sums so far rescaled by 2^(mu_old - mu_new)), so that
// the (m, l) and O reads of four segments are in flight together.  A slot
// holds O / (l f), so segment s enters the sum of l with weight 2^(m_s - mu)
// l_s and that of O with the same weight times f_s.
constexpr int kMergeBatch = 4;

template <int HD>
__global__ __launch_bounds__(HD / 32 * kWave) void sv_attn_streamk_merge(AttnArgs a) {
  const int waves = a.sk_rows / kRowsPerWave;
  const int db = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int wave = blockIdx.x % waves;
  const int unit = blockIdx.x / waves;
  const int per_seq = a.H_kv * a.m_tiles;
  const int b = unit / per_seq;
  const int ul = unit % per_seq;
  const int kvh = ul / a.m_tiles;
  const int mt = ul % a.m_tiles;
  const int m0 = mt * a.sk_rows + wave * kRowsPerWave;
  if (b >= a.B || m0 >= a.M) return;
  const int Wp = a.sk_meta[1];
  const int* pref = a.sk_meta + 2;
  const int T = (pref[b + 1] - pref[b]) / per_seq;
  if (T == 0) return;
  const int C = pref[b] + ul * T;
  const int i0 = C / Wp, i1 = (C + T - 1) / Wp;
  if (i0 == i1) return;                       // finished in place
  const int row = wave * kRowsPerWave + lane % 32;
  auto slot_of = [&](int i) { return i * 2 + (i * Wp >= C ? 0 : 1); };
  float mu = -INFINITY, l = 0.f;
  f32x4 acc[4] = {};
  for (int i = i0; i <= i1; i += kMergeBatch) {
    f32x2 ml[kMergeBatch];
    float fs[kMergeBatch];
    f16x8 src[kMergeBatch][2];
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) {   // past i1: segment i1 again, weight 0
      const int slot = slot_of(min(i + k, i1));
      ml[k] = a.ws_ml[(size_t)slot * a.sk_rows + row];
      fs[k] = a.ws_f[(size_t)slot * a.sk_rows + row];
      const f16x8* s = sk_partial_o<HD>(a, slot, wave) + lane + db * 2 * kWave;
#pragma unroll
      for (int h = 0; h < 2; ++h) src[k][h] = s[h * kWave];
    }
    float mc = mu;
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k)
      if (i + k <= i1) mc = fmaxf(mc, ml[k][0]);
    const float base = (mc == -INFINITY) ? 0.f : mc;   // exp2(-inf - base) = 0 below
    const float f = fast_exp2(mu - base);
    l *= f;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) acc[q4] *= f;
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) {
      const float w = (i + k <= i1) ? fast_exp2(ml[k][0] - base) * ml[k][1] : 0.f;
      const float wf = w * fs[k];
      l += w;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[q4][e] += wf * (float)src[k][q4 >> 1][4 * (q4 & 1) + e];
    }
    mu = mc;
  }
  const RowCtx r = make_row_ctx(a, 0, kvh, b, clamp_len(a, b), m0, lane);
  if (!r.row_ok) return;
  const float inv = 1.f / l;
  uint16_t* orow = a.out + ((size_t)(r.b * a.R + r.pos) * a.H_q + r.head) * HD;
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    const int d = 32 * db + 8 * q4 + 4 * r.hh;
    const uint32_t e0 = f32_to_bf16_bits(acc[q4][0] * inv);
    const uint32_t e1 = f32_to_bf16_bits(acc[q4][1] * inv);
    const uint32_t e2 = f32_to_bf16_bits(acc[q4][2] * inv);
    const uint32_t e3 = f32_to_bf16_bits(acc[q4][3] * inv);
    *reinterpret_cast<u32x2*>(orow + d) = u32x2{e0 | (e1 << 16), e2 | (e3 << 16)};
  }
}

// ---------------------------------------------------------------------------
// Direct partial kernel (M <= 64): every wave streams its own operands.
// ---------------------------------------------------------------------------
template <int HD, bool FP8, int NW>
__global__ __launch_bounds__(kWave * NW) void sv_attn_partial_direct(AttnArgs a) {
  constexpr int KS = HD / 16;
  constexpr int DB = HD / 32;
  constexpr size_t kBlockBytes = (size_t)HD * 16 * (FP8 ? 1 : 2);

  const Work wk = decode_work(a, a.m_tiles);
  if (!wk.valid) return;
  const int split = wk.split, kvh = wk.kvh, mt = wk.mt, b = wk.b;
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
      // dead sub-blocks still run (on a clamped, valid block): see ring_tile
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
    const bool masked = !(kt + kAttnTile <= r.k_end && kt + kAttnTile - 1 <= r.P);
    if (!masked)
      softmax_tile<DB, false>(x, cs, live, kt, r, m_run, l_run, o);
    else
      softmax_tile<DB, true>(x, cs, live, kt, r, m_run, l_run, o);
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const int t0 = kt + 32 * sb;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int tk = t0 + 16 * kk;   // first key of this cache block
        float vs = 1.f;
        if constexpr (FP8) vs = a.v_scale[blk[sb][kk] * a.H_kv + kvh];
        const bf16x8 pop = p_operand(x[sb], kk, vs);
        const uint8_t* vb = a.v + (blk[sb][kk] * a.H_kv + kvh) * kBlockBytes;
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
          if (masked) {   // slots at or past L (poison, or a clamped block) become 0
#pragma unroll
            for (int j = 0; j < 8; ++j) vop[j] = tk + 8 * r.hh + j < L ? vop[j] : (__bf16)0.f;
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

// Stream-K variant: LDS stages per workgroup and workgroups per CU.
constexpr int kStreamWPE = SV_STREAM_WPE;
constexpr int kStreamCUs = 256;            // MI355X compute units
constexpr int kStreamDefaultMinKeys = 512;  // least keys per workgroup range

void plan_attention(AttnPlan& p, int split_request) {
  p.sk_rows = 0;
  p.sk_wgs = 0;
  p.G = p.H_q / p.H_kv;
  p.M = p.G * p.R;
  // Batches up to kStreamMaxBatch go through the stream-K ring whatever M is:
  // waves beyond M still move their share of every tile (the K/V stream, not
  // the MFMA work, sets the pace when few rows share a KV head).  bf16 units
  // hold 128 rows (4 waves, two workgroups per CU) or, for 129 .. 256 rows per
  // KV head, 256 rows (8 waves, one workgroup per CU), so that those rows
  // stream their K and V once instead of twice.  Beyond 256 rows (MQA-like
  // heads) the row tiles of a KV head share its K/V through L2 and two 4-wave
  // workgroups per CU hide latency better (measured); e4m3 units hold 128.
  p.streamk = p.B <= kStreamMaxBatch;
  const int waves_needed = (p.M + kRowsPerWave - 1) / kRowsPerWave;
  if (p.streamk)
    p.waves = (!p.fp8 && p.M > kStreamRows && p.M <= 2 * kStreamRows) ? 8 : 4;
  else
    p.waves = waves_needed > 2 ? 4 : waves_needed;
  p.m_tiles = (p.M + kRowsPerWave * p.waves - 1) / (kRowsPerWave * p.waves);
  if (p.streamk) {
    // one split per unit as far as the row context goes; ranges come from min_tiles
    p.split_tokens = (p.max_kv_len + kAttnTile - 1) / kAttnTile * kAttnTile;
    p.s_max = 1;
    p.sk_rows = p.waves * kRowsPerWave;
    p.sk_wgs = p.waves == 8 ? kStreamCUs : kStreamCUs * kStreamWPE;
    p.min_tiles = (split_request > 0 ? split_request : kStreamDefaultMinKeys) / kSkKeys;
    const size_t slots = (size_t)p.sk_wgs * 2 * p.sk_rows;
    p.ws_meta_offset = 0;
    const size_t meta_bytes = ((size_t)(p.B + 3) * sizeof(int) + 255) / 256 * 256;
    p.ws_o_bytes = slots * p.hd * sizeof(uint16_t);   // fp16 O / (l f)
    p.ws_ml_offset = meta_bytes + p.ws_o_bytes;
    p.ws_f_offset = p.ws_ml_offset + slots * sizeof(f32x2);
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
  p.ws_bytes = p.ws_ml_offset + rows * sizeof(f32x2);
}

template <int HD, bool TREE>
static hipError_t launch_streamk(const AttnPlan& p, const AttnArgs& a, hipStream_t stream) {
  // Row tiles of one KV head share its K/V through L2; a lone row tile reads
  // them once, so they stream past the caches.
  constexpr int S4 = SkTile<HD>::kStages, S8 = SkTile<HD>::kStages8;
  if (p.fp8 && p.m_tiles == 1)
    sv_attn_streamk_fp8<HD, kStreamWPE, true, TREE><<<p.sk_wgs, kLdsThreads, 0, stream>>>(a);
  else if (p.fp8)
    sv_attn_streamk_fp8<HD, kStreamWPE, false, TREE><<<p.sk_wgs, kLdsThreads, 0, stream>>>(a);
  else if (p.waves == 8 && p.m_tiles == 1)
    sv_attn_streamk<HD, S8, 2, true, 8, TREE><<<p.sk_wgs, 8 * kWave, 0, stream>>>(a);
  else if (p.waves == 8)
    sv_attn_streamk<HD, S8, 2, false, 8, TREE><<<p.sk_wgs, 8 * kWave, 0, stream>>>(a);
  else if (p.m_tiles == 1)
    sv_attn_streamk<HD, S4, kStreamWPE, true, 4, TREE><<<p.sk_wgs, kLdsThreads, 0, stream>>>(a);
  else
    sv_attn_streamk<HD, S4, kStreamWPE, false, 4, TREE><<<p.sk_wgs, kLdsThreads, 0, stream>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int units = p.B * p.H_kv * p.m_tiles;
  sv_attn_streamk_merge<HD><<<units * (p.sk_rows / kRowsPerWave), HD / 32 * kWave, 0, stream>>>(a);
  return hipGetLastError();
}

// Partial kernel for row tiles of 128: the LDS ring for bf16 caches, the
// register-staged double buffer (which decodes e4m3 once per tile) for e4m3.
template <int HD, bool FP8>
struct launch_wide;
template <int HD>
struct launch_wide<HD, false> {
  static void run(dim3 grid, const AttnArgs& a, hipStream_t stream) {
    sv_attn_partial_ring<HD, SV_RING_STAGES, SV_RING_WPE><<<grid, kLdsThreads, 0, stream>>>(a);
  }
};
template <int HD>
struct launch_wide<HD, true> {
  static void run(dim3 grid, const AttnArgs& a, hipStream_t stream) {
    sv_attn_partial_lds<HD, true><<<grid, kLdsThreads, 0, stream>>>(a);
  }
};

template <int HD, bool FP8>
static hipError_t launch_typed(const AttnPlan& p, const AttnArgs& a, hipStream_t stream) {
  const long long units = (long long)p.s_max * p.B * p.H_kv;
  dim3 grid((unsigned)(((units + 7) / 8) * 8 * p.m_tiles));
  switch (p.waves) {
    case 1: sv_attn_partial_direct<HD, FP8, 1><<<grid, kWave * 1, 0, stream>>>(a); break;
    case 2: sv_attn_partial_direct<HD, FP8, 2><<<grid, kWave * 2, 0, stream>>>(a); break;
    default: launch_wide<HD, FP8>::run(grid, a, stream); break;
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
  char* ws = static_cast<char*>(ptr.ws);
  if (p.streamk) {
    a.sk_meta = reinterpret_cast<int*>(ws + p.ws_meta_offset);
    a.ws_o = reinterpret_cast<float*>(ws + ((size_t)(p.B + 3) * sizeof(int) + 255) / 256 * 256);
  } else {
    a.sk_meta = nullptr;
    a.ws_o = reinterpret_cast<float*>(ws);
  }
  a.ws_ml = p.ws_bytes ? reinterpret_cast<f32x2*>(ws + p.ws_ml_offset) : nullptr;
  a.ws_f = p.streamk ? reinterpret_cast<float*>(ws + p.ws_f_offset) : nullptr;
  a.min_tiles = p.min_tiles;
  a.sk_rows = p.sk_rows;
  a.B = p.B;
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
  a.m_tiles = p.m_tiles;
  a.c = p.sm_scale * kLog2e;
  a.tree_hi = 0;
  if (ptr.tree_mask) {
    if (!p.streamk) return hipErrorInvalidValue;   // the host rejects trees off the stream-K path
    const uint64_t tm = reinterpret_cast<uint64_t>(ptr.tree_mask);
    a.tree_lo = (uint32_t)tm;
    a.tree_hi = (uint32_t)(tm >> 32);
    return p.hd == 128 ? launch_streamk<128, true>(p, a, stream) : launch_streamk<64, true>(p, a, stream);
  }
  if (p.streamk)
    return p.hd == 128 ? launch_streamk<128, false>(p, a, stream) : launch_streamk<64, false>(p, a, stream);
  if (p.hd == 128)
    return p.fp8 ? launch_typed<128, true>(p, a, stream) : launch_typed<128, false>(p, a, stream);
  return p.fp8 ? launch_typed<64, true>(p, a, stream) : launch_typed<64, false>(p, a, stream);
}

}  // namespace sv
