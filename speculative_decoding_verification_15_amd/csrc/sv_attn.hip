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

#include <type_traits>

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
  int s_max;      // split path: splits per sequence
  int m_tiles;
  int min_tiles;  // stream-K: least tiles per workgroup
  float c;        // sm_scale * log2(e)
  int* sk_meta;   // stream-K: [W, Wp, pref[0..B]] written by workgroup 0 for the merge
  int sk_rows;    // stream-K: rows per unit (128 or 256)
  const uint64_t* tree;  // NULL: causal chain; else [B][R] ancestor masks
};

// Tree verification: [B][R] ancestor masks, bit j of mask[b][i] = node j is
// node i or one of its ancestors.
__device__ __forceinline__ const uint64_t* tree_masks(const AttnArgs& a) { return a.tree; }

// Row i of the 32-key score block holds key pi(i) of that block.
__device__ __forceinline__ int key_of_row(int i) {
  return (i & 0x13) | ((i & 4) << 1) | ((i & 8) >> 1);
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  __bf16 b = (__bf16)x;
  return __builtin_bit_cast(uint16_t, b);
}

// Everything one lane needs to know about its query row and key range.  anc:
// the new positions the row may see (bit j: key P + j), the positions up to its
// own for a causal chain, its ancestor mask for a draft tree (split-path
// kernels; the stream-K kernels mask trees themselves).
struct RowCtx {
  int b, kvh, split, L, n_splits, k_begin, k_end;
  int m, pos, head, P, vis_last, R;
  int ql, hh;
  bool row_ok;
  uint64_t anc;
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
  r.R = a.R;
  r.anc = (2ull << r.pos) - 1ull;   // positions 0 .. pos (all 64 bits for pos = 63)
  return r;
}

// Split-path kernels: the row's ancestor mask replaces the chain mask for a tree.
__device__ __forceinline__ void load_row_anc(const AttnArgs& a, RowCtx& r) {
  if (a.tree) r.anc = a.tree[(size_t)r.b * a.R + r.pos];
}

// Whether key `key` (at or past the first new position P) is hidden from the
// row: past the end, or a new position outside the row's mask.  Every term is
// evaluated for every key, the shift amount clamped into [0, 63] first.
__device__ __forceinline__ bool row_hides(const RowCtx& r, int key) {
  const int j = key - r.P;
  const uint32_t s = (uint32_t)min(max(j, 0), 63);
  const bool in = ((r.anc >> s) & 1ull) != 0;
  return (j >= 0) & ((j >= r.R) | !in);
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
          if (!live[sb] || row_hides(r, key)) x[sb][v] = -INFINITY;
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
  RowCtx r = make_row_ctx(a, split, kvh, b, L, m0, lane);
  load_row_anc(a, r);

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

// 4 bytes per active lane from global memory into LDS (global_load_lds_dword:
// lane i's dword lands at lds + 4 i), with the same M0 contract as
// dma_to_lds16.  Counted by vmcnt like the tile loads, so it is ordered with
// them by the same waits.
__device__ __forceinline__ void dma_to_lds4(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
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
  RowCtx r = make_row_ctx(a, split, kvh, b, L, m0, lane);
  load_row_anc(a, r);

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

// pref[b] = tiles of KEYS keys of all units of sequences before b, for b = 0 .. B.
template <int KEYS>
__device__ __forceinline__ void build_prefix(const AttnArgs& a, int* pref, int* wsum) {
  const int tid = threadIdx.x;
  const int lane = tid % kWave, wave = tid / kWave;
  const int per_seq = a.H_kv * a.m_tiles;
  const int nthreads = (int)blockDim.x;
  const int chunk = (a.B + nthreads - 1) / nthreads;
  const int lo = min(tid * chunk, a.B), hi = min(lo + chunk, a.B);
  int sum = 0;
  for (int b = lo; b < hi; ++b) {
    sum += ((clamp_len(a, b) + KEYS - 1) / KEYS) * per_seq;
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
template <int KEYS>
__device__ __forceinline__ int unit_tiles(const AttnArgs& a, int b) {
  return (clamp_len_s(a, b) + KEYS - 1) / KEYS;
}

// Advances to the next tile of the work list.  The tile count of a new
// sequence comes from kv_lens (a scalar load, once per sequence), so the
// prefix table is needed only to place a range's first tile.
template <int KEYS>
__device__ __forceinline__ void cursor_next(const AttnArgs& a, Cursor& c) {
  if (++c.tile < c.T) return;
  c.tile = 0;
  if (++c.mt < a.m_tiles) return;
  c.mt = 0;
  if (++c.kvh < a.H_kv) return;
  c.kvh = 0;
  do {
    ++c.b;
  } while (c.b < a.B && (c.T = unit_tiles<KEYS>(a, c.b)) == 0);
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

// Work-list range of this workgroup (W tiles in ranges of Wp).  Workgroups go
// to the 8 XCDs in turn (workgroup i to XCD i % 8), each XCD with its own L2.
// When a KV head's rows span several units (m_tiles > 1), consecutive units
// stream the same K/V tiles at the same time, so the ranges that hold tiles
// are dealt out XCD by XCD, ceil(nr / 8) consecutive ones to each: they run on
// one XCD and share its L2 (MQA with 2048 rows: 153-156 against 161-164 us),
// and every XCD gets a share however few ranges there are.  Workgroups left
// over get range nr, past the last tile.  With one unit per KV head
// consecutive ranges share no K/V, and the plain order is kept.
__device__ __forceinline__ int sk_range(const AttnArgs& a, int W, int Wp) {
  const int n = (int)gridDim.x, i = (int)blockIdx.x;
  if (a.m_tiles <= 1 || n % 8 != 0) return i;
  const int nr = Wp > 0 ? (W + Wp - 1) / Wp : 0;   // ranges holding tiles (<= n)
  const int per = (nr + 7) / 8;                // ranges per XCD
  const int k = i / 8;
  const int r = (i % 8) * per + k;
  return k < per && r < nr ? r : nr;
}

// NT: K/V loads are non-temporal, for row tilings where each unit's K and V are
// read by that unit alone (one row tile per KV head).  WAVES = 4 (units of 128
// rows, two workgroups per CU) or 8 (units of 256 rows, one per CU, for 129 ..
// 255 rows per KV head), so that those rows stream their K and V once.
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

  build_prefix<kSkKeys>(a, s_pref, s_wsum);
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
  const int rng = sk_range(a, W, Wp);
  const int g0 = rng * Wp;
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
  bf16x8 qop[KS], qn[KS];
  if (active) load_q<HD, false>(a, r, qop);
  wait_vmcnt<0>();                             // Q before the ring's loads, waited once

  int gi = g0;
  int ent = entry(ci);                        // table entry of the tile at ci
#pragma unroll
  for (int k = 0; k < NS - 1; ++k) {         // past the range: the last tile again
    issue(ci, ent, k);
    if (gi + 1 < g1) cursor_next<kSkKeys>(a, ci);
    ++gi;
    ent = entry(ci);
  }

  // Two forms of the tile loop, chosen by measurement (outputs are bit-identical):
  // 8-wave units (129 .. 255 rows per KV head) run a loop over the range's segments with
  // an inner loop over their tiles, so that the per-tile path carries no segment tests
  // (gqa8 D = 16: 151 -> 138 us); 4-wave units keep one loop over tiles with the tests
  // inline, which measured 1-2% faster for them (70B-like 375 against 379-383 us).
  if constexpr (WAVES == 8) {
    f32x16 o[DB];
    f32x16 xn;                                   // scores of the next tile, when have_xn
    bool have_xn = false;
    float m_ref = kNoMax, l_run = 0.f;
    unsigned t = 0;                              // tiles computed so far (unsigned: stage
                                                 // indices are cheap remainders)
    int g = g0;                                  // work-list index of the tile being computed

    // One tile of the current segment, unit tile tt.  MASKED: the tile reaches
    // past some row's last visible key (key P + pos), which also covers the
    // sequence's last tile (keys past L) and the unit's last tile, where the
    // next segment is prepared; every other tile of a segment takes the plain
    // path, with none of those tests.
    auto step = [&](const int tt, auto masked_tag) {
      constexpr bool MASKED = decltype(masked_tag)::value;
      // This wave's loads of tiles g and g + 1 landed: loads retire in issue
      // order, so at most tile g + 2's loads (and stores issued after them) are
      // still counted.
      wait_vmcnt<(NS - 3) * LPW>();
      __builtin_amdgcn_s_barrier();              // ... and every other wave's
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
      if (MASKED && tt + 1 == cc.T && g + 1 < g1) {
        // The next tile starts a segment: its row context and Q are loaded now,
        // ahead of this tile's ring loads, so that using them next tile waits
        // for nothing issued later.
        Cursor cn = cc;
        cn.tile = tt;
        cursor_next<kSkKeys>(a, cn);
        active_n = seg_ctx(cn, rn);
        if (active_n) load_q_raw<HD>(a, rn, qn);
      }
      issue(ci, ent, (t + NS - 1) % NS);         // refills the stage freed by tile g - 1
      if (gi + 1 < g1) cursor_next<kSkKeys>(a, ci);
      ++gi;
      ent = entry(ci);

      const int kt = tt * kSkKeys;
      uint8_t* stage = smem + (t % NS) * STAGE;
      if (MASKED && kt + kSkKeys > r.L) {        // the sequence's last tile (same for all waves)
        sk_zero_v_tail<HD>(stage, kt, r.L);
        __syncthreads();
      }
      if (active) {
        // Software pipeline within the wave: the scores of tile g + 1 are
        // computed (MFMA) while the softmax of tile g runs (VALU); they are kept
        // when tile g + 1 continues this segment, which has the same Q.
        f32x16 x = have_xn ? xn : sk_scores<HD>(stage, k_lds, qop);
        if constexpr (MASKED) {
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
      have_xn = true;                            // the next tile of this segment has it
      ++g;
      ++t;
    };

    // Segments: the tiles of one unit inside this range, [cc.tile, cc.tile + n).
    // A segment ends at its unit's last tile or at the range's end.
    for (;;) {
      const int seg_start = g;
      const int tt0 = cc.tile;
      const int n = min(g1 - g, cc.T - tt0);
      // Tiles whose 32 keys every row of the unit sees (32 tt + 31 <= P): plain.
      const int n_plain = min(max(max(r.P + 1, 0) / kSkKeys - tt0, 0), n);
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] = f32x16{};
      m_ref = kNoMax;
      l_run = 0.f;
      have_xn = false;
      for (int i = 0; i < n_plain; ++i) step(tt0 + i, std::false_type{});
      for (int i = n_plain; i < n; ++i) step(tt0 + i, std::true_type{});
      if (active)
        sk_segment_end<HD>(a, r, o, m_ref, l_run, tt0 == 0 && tt0 + n == cc.T,
                           rng * 2 + (seg_start == g0 ? 0 : 1), wave, lane);
      if (g >= g1) break;
      // the next segment starts at tile 0 of the next unit, prepared during
      // this segment's last tile
      cc.tile = tt0 + n - 1;
      cursor_next<kSkKeys>(a, cc);
      r = rn;
      active = active_n;
      const bf16x8 z = {};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qop[ks] = r.row_ok ? qn[ks] : z;
    }
  } else {
    int seg_start = g0;
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
        cursor_next<kSkKeys>(a, cn);
        active_n = seg_ctx(cn, rn);
        if (active_n) load_q_raw<HD>(a, rn, qn);
      }
      issue(ci, ent, (t + NS - 1) % NS);         // refills the stage freed by tile g - 1
      if (gi + 1 < g1) cursor_next<kSkKeys>(a, ci);
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
                             rng * 2 + (seg_start == g0 ? 0 : 1), wave, lane);
      }
      if (g + 1 < g1) cursor_next<kSkKeys>(a, cc);
    }
  }
  wait_vmcnt<0>();                             // drain loads issued past the range
}

// Stream-K kernel for e4m3 caches, on the fp8 matrix cores.  The same work
// list, ranges, segments and merge as the bf16 kernel, with 64-key tiles
// (four 16-key blocks).  The codes are DMA'd into the ring as they are stored
// and fed to v_mfma_scale_f32_32x32x64_f8f6f4 as they are: nothing is decoded.
//
//   scores  S^T = K . Q^T: A = the K codes of 32 keys x 64 dims, B = Q.  Q is
//           scaled per row by a power of two 2^-E (its largest |value| into
//           [128, 256)) and split into two e4m3 terms, hi = e4m3(q) and lo =
//           e4m3(q - hi), whose products are summed in the same accumulator:
//           with 4 + 4 significant bits the pair carries Q to about 2^-8,
//           the precision of bf16 (a single e4m3 term would not).
//   scale   the K scale of a key's block multiplies its score together with
//           sm_scale log2(e) 2^E; log2 of the V scale of the block is added to
//           the exponent, so that the probabilities come out multiplied by the
//           V scale (the exact decode(code) * scale value of every V element,
//           applied in fp32) and the running maximum covers that factor too.
//           l sums the probabilities themselves (each block's sum times the
//           reciprocal of its V scale).
//   PV      O^T += V^T . P^T: A = the V codes of 32 dims x 64 keys, B = the
//           probabilities, again as two e4m3 terms, each row's values scaled
//           by a power of two that puts the tile's largest into (2^7, 2^8] and
//           that the MFMA's block scale undoes (without it the small
//           probabilities of a row would fall into e4m3's subnormals and lose
//           their precision).
//
// Stage layout: K blocks 0..3 as stored ([hd / 16][16 slots][16 dims] each),
// then V as [dim / 8][block 0..3][dim % 8][16 slots], so that the four blocks'
// slot rows of one dim lie 128 bytes apart and a lane's V operand is two
// 16-byte-pair reads (ds_read2_b64) straight into its eight registers.
//
// Operand bytes.  For the f8f6f4 MFMA, lane l supplies 32 bytes of A row l %
// 32 and of B column l % 32, and byte e of lane half h = l / 32 is the same
// k index in both operands (any one-to-one choice of k(h, e) gives the same
// product).  Scores use k(h, e) = dim 64 kb + 32 h + e.  The score
// accumulator of a 32-key half sh puts key 32 sh + 16 (v / 8) + 8 h + v % 8
// in register v of lane half h (rows fed in the order key_of_row), so PV uses
// k(h, e) = key 16 (e / 8) + 8 h + e % 8: byte e of the probability operand is
// then register e % 16 of accumulator e / 16, and byte e of the V operand is
// slot 8 h + e % 8 of block e / 8 -- eight consecutive bytes of a block's
// slot row of that dim.
template <int HD>
struct Sk8 {
  static constexpr int kKeys = kSk8Keys;           // keys per tile
  static constexpr int kBlk = HD * 16;             // bytes of one 16-key block of K or V codes
  static constexpr int kStage = 8 * kBlk;          // K blocks 0..3, then V blocks 0..3
  static constexpr int kStages = SV_STREAM_RING_BYTES / kStage;
  static constexpr int kLoads = kBlk / 1024;       // 1 KB DMA pieces per block
  static constexpr int kKb = HD / 64;              // 64-dim k-blocks of the score product
  static constexpr int kDb = HD / 32;              // 32-dim blocks of O
};

typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) int i32x4;

// D(32x32, fp32) += A(32x64, e4m3) * B(64x32, e4m3), block scales 1.
__device__ __forceinline__ f32x16 mfma32x32x64_e4m3(const i32x8& a, const i32x8& b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}
// The same with B scaled by E8M0 exponents sb (low byte): the exponent of lane
// j scales the first 16 bytes of B column j in both lane halves (lanes j and
// j + 32), that of lane j + 32 the last 16 bytes, each by 2^(sb - 127).  The
// callers give lanes j and j + 32 the same exponent: one factor per column.
__device__ __forceinline__ f32x16 mfma32x32x64_e4m3_sb(const i32x8& a, const i32x8& b, f32x16 c,
                                                      int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, sb);
}

// Four fp32 values as four e4m3 codes (round to nearest even; the callers keep
// every magnitude below 448) in one dword, first value in the lowest byte.
// `old` is any dword whose value is no longer needed: the conversions write
// into it in place (both of its halves are overwritten).
__device__ __forceinline__ int e4m3x4(float a, float b, float c, float d, int old) {
  const int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

// x as hi + lo in e4m3 (hi = e4m3(x), lo = e4m3(x - hi)), four values at a
// time: the dwords of hi (element 0) and lo (element 1), written over the
// dead dwords old_hi and old_lo.
__device__ __forceinline__ u32x2 e4m3_split4(float a, float b, float c, float d, int old_hi,
                                             int old_lo) {
  const int hi = e4m3x4(a, b, c, d, old_hi);
  const f32x2 h01 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, false);
  const f32x2 h23 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, true);
  const int lo = e4m3x4(a - h01[0], b - h01[1], c - h23[0], d - h23[1], old_lo);
  return u32x2{(uint32_t)hi, (uint32_t)lo};
}

// Q operands of this lane's row (row_ok: else zeros) as hi and lo e4m3 terms
// per 64-dim k-block, and the row's score factor c 2^E.
template <int HD>
__device__ __forceinline__ void load_q_e4m3(const AttnArgs& a, const RowCtx& r,
                                            i32x8 (&qhi)[HD / 64], i32x8 (&qlo)[HD / 64],
                                            float& c_row) {
  constexpr int KB = HD / 64;
  const uint16_t* qrow = a.q + ((size_t)(r.b * a.R + r.pos) * a.H_q + r.head) * HD;
  bf16x8 raw[KB][4];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x8 z = {};
      raw[kb][j] = r.row_ok ? *reinterpret_cast<const bf16x8*>(qrow + 64 * kb + 32 * r.hh + 8 * j) : z;
    }
  float amax = 0.f;
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf((float)raw[kb][j][e]));
  amax = halves_max(amax);
  // amax in [2^(ex-1), 2^ex): q 2^(8-ex) has its largest magnitude in [128, 256)
  const int ex = amax > 0.f ? __builtin_amdgcn_frexp_expf(amax) : 8;
  c_row = __builtin_amdgcn_ldexpf(a.c, ex - 8);
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = __builtin_amdgcn_ldexpf((float)raw[kb][j][e], 8 - ex);
      const u32x2 a0 = e4m3_split4(v[0], v[1], v[2], v[3], qhi[kb][2 * j], qlo[kb][2 * j]);
      const u32x2 a1 = e4m3_split4(v[4], v[5], v[6], v[7], qhi[kb][2 * j + 1],
                                   qlo[kb][2 * j + 1]);
      qhi[kb][2 * j] = (int)a0[0];
      qlo[kb][2 * j] = (int)a0[1];
      qhi[kb][2 * j + 1] = (int)a1[0];
      qlo[kb][2 * j + 1] = (int)a1[1];
    }
}

// Scores of one 32-key half sh of a tile (keys 32 sh + key_of_row(i) in row i).
template <int HD>
__device__ __forceinline__ f32x16 sk8_scores(const uint8_t* stage, int k_lds, int sh,
                                             const i32x8 (&qhi)[HD / 64],
                                             const i32x8 (&qlo)[HD / 64]) {
  constexpr int BLK = Sk8<HD>::kBlk;
  f32x16 x = f32x16{};
#pragma unroll
  for (int kb = 0; kb < HD / 64; ++kb) {
    const uint8_t* p = stage + 2 * sh * BLK + k_lds + kb * 1024;
    const u32x4 k0 = *reinterpret_cast<const u32x4*>(p);
    const u32x4 k1 = *reinterpret_cast<const u32x4*>(p + 256);
    const i32x8 kop = {(int)k0[0], (int)k0[1], (int)k0[2], (int)k0[3],
                       (int)k1[0], (int)k1[1], (int)k1[2], (int)k1[3]};
    x = mfma32x32x64_e4m3(kop, qhi[kb], x);
    x = mfma32x32x64_e4m3(kop, qlo[kb], x);
  }
  return x;
}

// Key of score register v of lane half hh in half sh of a tile starting at kt.
__device__ __forceinline__ int sk8_key(int kt, int sh, int v, int hh) {
  return kt + 32 * sh + 16 * (v >> 3) + 8 * hh + (v & 7);
}

__device__ __forceinline__ void sk8_mask(f32x16& x, const RowCtx& r, int kt, int sh) {
#pragma unroll
  for (int v = 0; v < 16; ++v) x[v] = sk8_key(kt, sh, v, r.hh) > r.vis_last ? -INFINITY : x[v];
}

// Tree variant: key P + j (a new position, j >= 0) is visible only for the
// nodes of the row's ancestor mask anc; every term is evaluated for every key
// (no short-circuit branches around the scores), the shift amount clamped
// into [0, 63] first.
__device__ __forceinline__ void sk8_mask_tree(f32x16& x, const RowCtx& r, int kt, int sh,
                                              uint64_t anc, int R) {
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int j = sk8_key(kt, sh, v, r.hh) - r.P;
    const uint32_t s = (uint32_t)min(max(j, 0), 63);
    const bool in_tree = ((anc >> s) & 1ull) != 0;
    const bool hidden = (j >= 0) & ((j >= R) | !in_tree);
    x[v] = hidden ? -INFINITY : x[v];
  }
}

// Byte offset of the 16 slot codes of V dim d, block bk in a stage's V part.
__device__ __forceinline__ int sk8_v_off(int d, int bk) {
  return ((d >> 3) * 4 + bk) * 128 + (d & 7) * 16;
}

// Zeroes the V codes of keys >= L in the tile image at stage (keys kt .. kt +
// 63): poison past the end of the sequence (NaN codes included) must not meet
// the zero probabilities of those keys in the PV product.
template <int HD>
__device__ __forceinline__ void sk8_zero_v_tail(uint8_t* stage, int kt, int L) {
  constexpr int BLK = Sk8<HD>::kBlk;
  for (int i = threadIdx.x; i < 4 * HD; i += blockDim.x) {
    const int bk = i / HD, d = i % HD;
    const int live = L - (kt + 16 * bk);             // slots of this block before the end
    if (live < 16) {
      u32x4* p = reinterpret_cast<u32x4*>(stage + 4 * BLK + sk8_v_off(d, bk));
      u32x4 v = *p;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        uint32_t m = 0;
#pragma unroll
        for (int by = 0; by < 4; ++by)
          if (4 * w + by < live) m |= 0xFFu << (8 * by);
        v[w] &= m;
      }
      *p = v;
    }
  }
}

// Online-softmax update for one 64-key tile (x[sh]: scores of half sh) with the
// per-block factors cb (K scale * c 2^E), lv (log2 of the V scale) and rv (its
// reciprocal); the probabilities come out as the PV operand's hi and lo e4m3
// terms, written over the previous tile's (dead) operands.  A row's 64
// probabilities are multiplied by a power of two 2^s that puts the tile's
// largest in (2^7, 2^8] -- well inside e4m3's normal range, so that small ones
// keep their 4 + 4 bits instead of falling into subnormals -- and sb receives
// the E8M0 exponent 127 - s that the PV MFMA applies to undo it (the same in
// both lanes of the row).  Returns whether O must be rescaled by alpha (lazy
// reference, as in softmax_sub).
__device__ __forceinline__ bool softmax_tile8(const f32x16 (&x)[2], const float (&cb)[4],
                                              const float (&lv)[4], const float (&rv)[4],
                                              float& m_ref, float& l_run, float& alpha,
                                              i32x8& phi, i32x8& plo, int& sb) {
  float hm[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const f32x16& xs = x[b >> 1];
    const int o = 8 * (b & 1);
    float m = fmaximum(xs[o], xs[o + 1]);
#pragma unroll
    for (int v = 2; v < 8; ++v) m = fmaximum(m, xs[o + v]);
    hm[b] = __builtin_fmaf(m, cb[b], lv[b]);
  }
  const float lane_max = fmaximum(fmaximum(hm[0], hm[1]), fmaximum(hm[2], hm[3]));
  const float tmax = halves_maximum(lane_max);
  const bool move = tmax > m_ref + kLazyRescale;   // the running maximum starts at kNoMax
  alpha = move ? fast_exp2(m_ref - tmax) : 1.f;
  m_ref = move ? tmax : m_ref;
  // tmax - m_ref <= kLazyRescale, so s >= 0; a row with every key of the tile
  // masked (tmax = -inf) takes the largest s, its probabilities are all 0
  const float gap = m_ref - tmax;
  const int sh = gap < 100.f ? (int)__builtin_floorf(gap) + 8 : 108;
  sb = 127 - sh;
  const float shf = (float)sh;
  float p[32];
  float s[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const f32x16& xs = x[b >> 1];
    const int o = 8 * (b & 1);
    const float ab = (lv[b] - m_ref) + shf;
    s[b] = 0.f;
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const float pv = fast_exp2(__builtin_fmaf(xs[o + v], cb[b], ab));
      p[8 * b + v] = pv;
      s[b] += pv;
    }
  }
  l_run = l_run * alpha +
          __builtin_amdgcn_ldexpf((s[0] * rv[0] + s[1] * rv[1]) + (s[2] * rv[2] + s[3] * rv[3]), -sh);
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    const u32x2 hl = e4m3_split4(p[4 * w], p[4 * w + 1], p[4 * w + 2], p[4 * w + 3], phi[w], plo[w]);
    phi[w] = (int)hl[0];
    plo[w] = (int)hl[1];
  }
  return __ballot(move) != 0;
}

// O^T += V^T . P^T for one tile (V codes of the stage, keys >= L zeroed).
template <int HD>
__device__ __forceinline__ void sk8_pv(const uint8_t* stage, int v_lds, const i32x8& phi,
                                       const i32x8& plo, int sb, f32x16 (&o)[HD / 32]) {
  constexpr int BLK = Sk8<HD>::kBlk;
#pragma unroll
  for (int db = 0; db < HD / 32; ++db) {
    i32x8 vop;
#pragma unroll
    for (int b = 0; b < 4; ++b) {   // dims 32 db .. lie 4 x 512 bytes further per block of 32
      const u32x2 w = *reinterpret_cast<const u32x2*>(stage + 4 * BLK + v_lds + db * 2048 + b * 128);
      vop[2 * b] = (int)w[0];
      vop[2 * b + 1] = (int)w[1];
    }
    o[db] = mfma32x32x64_e4m3_sb(vop, phi, o[db], sb);
    o[db] = mfma32x32x64_e4m3_sb(vop, plo, o[db], sb);
  }
}

template <int HD, bool NT, bool TREE>
__global__ __attribute__((amdgpu_flat_work_group_size(kLdsThreads, kLdsThreads),
                          amdgpu_waves_per_eu(2, 2)))
void sv_attn_streamk_f8(AttnArgs a) {
  using T8 = Sk8<HD>;
  constexpr int KEYS = T8::kKeys;
  constexpr int KB = T8::kKb;
  constexpr int DB = T8::kDb;
  constexpr int BLK = T8::kBlk;
  constexpr int STAGE = T8::kStage;
  constexpr int NS = T8::kStages;
  constexpr int LPB = T8::kLoads;
  static_assert(NS >= 4, "the ring holds the computed tile, the next one and two in flight");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NS * STAGE];
  // per stage: K and V scale of block w at [2 w] and [2 w + 1], DMA'd by wave w
  __shared__ __attribute__((aligned(16))) float s_sc[NS][8];
  static_assert((kStreamMaxBatch + 1 + 4) * 4 <= NS * STAGE, "prefix table fits");
  int* s_pref = reinterpret_cast<int*>(smem);
  int* s_wsum = s_pref + kStreamMaxBatch + 1;

  build_prefix<KEYS>(a, s_pref, s_wsum);
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
  const int rng = sk_range(a, W, Wp);
  const int g0 = rng * Wp;
  const int g1 = min(g0 + Wp, W);
  if (g0 >= g1) return;                       // whole workgroup, after the last barrier use

  const int wave = uniform(tid / kWave);
  const int lane = tid % kWave;
  const int ql = lane & 31, hh = lane >> 5;
  const uint32_t blk_stride32 = (uint32_t)a.H_kv * BLK;   // below 2^32 (the planner checks)
  const float* ksc = a.k_scale;
  const float* vsc = a.v_scale;

  // Operand offsets of this lane inside a stage: K row ql of a 32-key half is
  // key key_of_row(ql) (block ql / 16 of the half, slot key_of_row(ql) % 16),
  // dims 32 hh .. of each k-block; V dim ql of each 32-dim block, slots 8 hh ..
  const int k_lds = (ql >> 4) * BLK + ((2 * hh) * 16 + (key_of_row(ql) & 15)) * 16;
  const int v_lds = sk8_v_off(ql, 0) + 8 * hh;

  // Table entries of the tile's four blocks, read with scalar loads one tile
  // ahead (as in the bf16 kernel).  Wave w moves K block w as stored, and 1 KB
  // pieces of the V part: lane i of piece j holds V dim 8 (2 j + i / 32) + i % 8
  // of block (i / 8) % 4, so its source block is chosen per lane.
  auto entry = [&](const Cursor& c) -> i32x4 {
    const SV_CONST int32_t* row = (const SV_CONST int32_t*)c.row;
    const unsigned last = (unsigned)(a.max_blocks - 1);
    const unsigned j = 4u * (unsigned)c.tile;
    return i32x4{row[min(j, last)], row[min(j + 1, last)], row[min(j + 2, last)], row[min(j + 3, last)]};
  };
  constexpr int VPW = BLK / 1024;             // V pieces per wave (4 waves x VPW = 4 BLK / 1 KB)
  const int vb_lane = (lane >> 3) & 3;        // block of this lane's V piece rows
  const int vd_lane = (lane & 7) + 8 * (lane >> 5);   // dim within a piece's 16 dims
  // Loads of one tile into stage `stage`, then this wave's block's K and V
  // scales into s_sc[stage] (lanes 0 and 1).  The scales are DMA'd rather than
  // read with scalar loads: the blocks are scattered, so those loads missed
  // the caches, and every LDS wait of the iteration (one counter covers LDS
  // and scalar loads) then waited for them as well.  As vector-memory loads
  // they complete in order with the tile's own and are covered by the ring's
  // waits.
  auto issue = [&](const Cursor& c, const i32x4& raw, int stage) {
    const uint32_t last = (uint32_t)(a.num_blocks - 1);
    const uint32_t pw = (uint32_t)min(max(raw[wave], 0), (int)last);
    const uint32_t head = (uint32_t)(c.kvh * BLK);
    const uint32_t l = lds_addr(smem) + stage * STAGE;
    dma_to_lds16_run<NT, LPB>(a.k + ((uint64_t)pw * blk_stride32 + head + (uint32_t)lane * 16u),
                              l + wave * BLK);
    const int rl = vb_lane == 0 ? raw[0] : vb_lane == 1 ? raw[1] : vb_lane == 2 ? raw[2] : raw[3];
    const uint32_t pl = (uint32_t)min(max(rl, 0), (int)last);
    const uint8_t* vsrc = a.v + ((uint64_t)pl * blk_stride32 + head);
#pragma unroll
    for (int j = 0; j < VPW; ++j) {
      const int piece = wave * VPW + j;
      dma_to_lds16<NT>(vsrc + (16 * piece + vd_lane) * 16, l + 4 * BLK + piece * 1024);
    }
    const uint32_t si = pw * (uint32_t)a.H_kv + (uint32_t)c.kvh;
    if (lane < 2) dma_to_lds4((lane == 0 ? ksc : vsc) + si, lds_addr(&s_sc[stage][2 * wave]));
  };

  Cursor ci = cursor_at(a, s_pref, g0);      // next tile to load (index gi)
  Cursor cc = ci;                             // tile being computed
  __syncthreads();                            // the prefix table is dead: the ring may fill

  auto seg_ctx = [&](const Cursor& c, RowCtx& rr) -> bool {
    const int m0 = c.mt * kStreamRows + wave * kRowsPerWave;
    const int L = clamp_len_s(a, c.b);
    rr = make_row_ctx(a, 0, c.kvh, c.b, L, m0, lane);
    rr.k_end = L;
    return m0 < a.M;
  };
  RowCtx r;
  bool active = seg_ctx(cc, r);
  i32x8 qhi[KB], qlo[KB];
  float c_row = a.c;
  uint64_t anc = 0;
  if (active) load_q_e4m3<HD>(a, r, qhi, qlo, c_row);
  if constexpr (TREE) anc = tree_masks(a)[(size_t)r.b * a.R + r.pos];
  wait_vmcnt<0>();                             // Q before the ring's loads, waited once

  int gi = g0;
  i32x4 ent = entry(ci);
#pragma unroll
  for (int k = 0; k < NS - 1; ++k) {         // past the range: the last tile again
    issue(ci, ent, k);
    if (gi + 1 < g1) cursor_next<KEYS>(a, ci);
    ++gi;
    ent = entry(ci);
  }

  f32x16 o[DB];
  f32x16 xn[2];                                // scores of the next tile, when have_xn
  bool have_xn = false;
  float m_ref = kNoMax, l_run = 0.f;
  i32x8 phi = {}, plo = {};                    // probability operands (hi, lo) of the last tile
  unsigned t = 0;                              // tiles computed so far
  int g = g0;                                  // work-list index of the tile being computed

  // One tile of the current segment, unit tile tt (MASKED: the tile reaches
  // past some row's last visible key, which covers the sequence's last tile).
  auto step = [&](const int tt, auto masked_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    // This wave's loads of tiles g and g + 1 landed (tile g + 2's -- K, V and
    // the scales, 2 LPB + 1 loads -- may not have: loads retire in issue
    // order) ...
    wait_vmcnt<(NS - 3) * (2 * LPB + 1)>();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();              // ... and every other wave's; stage g - 1 is free
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    issue(ci, ent, (t + NS - 1) % NS);        // refills the stage of tile g - 1
    if (gi + 1 < g1) cursor_next<KEYS>(a, ci);
    ++gi;
    ent = entry(ci);

    const int kt = tt * KEYS;
    uint8_t* stage = smem + (t % NS) * STAGE;
    if (MASKED && kt + KEYS > r.L) {           // the sequence's last tile (same for all waves)
      sk8_zero_v_tail<HD>(stage, kt, r.L);
      __syncthreads();
    }
    if (active) {
      f32x16 x[2];
      if (have_xn) {
        x[0] = xn[0];
        x[1] = xn[1];
      } else {
        x[0] = sk8_scores<HD>(stage, k_lds, 0, qhi, qlo);
        x[1] = sk8_scores<HD>(stage, k_lds, 1, qhi, qlo);
      }
      if constexpr (MASKED) {
        if constexpr (TREE) {
          sk8_mask_tree(x[0], r, kt, 0, anc, a.R);
          sk8_mask_tree(x[1], r, kt, 1, anc, a.R);
        } else {
          sk8_mask(x[0], r, kt, 0);
          sk8_mask(x[1], r, kt, 1);
        }
      }
      const uint8_t* nstage = smem + ((t + 1) % NS) * STAGE;
      xn[0] = sk8_scores<HD>(nstage, k_lds, 0, qhi, qlo);
      xn[1] = sk8_scores<HD>(nstage, k_lds, 1, qhi, qlo);
      const f32x4 sc01 = *reinterpret_cast<const f32x4*>(&s_sc[t % NS][0]);
      const f32x4 sc23 = *reinterpret_cast<const f32x4*>(&s_sc[t % NS][4]);
      const float cb[4] = {c_row * sc01[0], c_row * sc01[2], c_row * sc23[0], c_row * sc23[2]};
      const float lv[4] = {__builtin_amdgcn_logf(sc01[1]), __builtin_amdgcn_logf(sc01[3]),
                           __builtin_amdgcn_logf(sc23[1]), __builtin_amdgcn_logf(sc23[3])};
      const float rv[4] = {__builtin_amdgcn_rcpf(sc01[1]), __builtin_amdgcn_rcpf(sc01[3]),
                           __builtin_amdgcn_rcpf(sc23[1]), __builtin_amdgcn_rcpf(sc23[3])};
      float alpha;
      int sb;
      const bool rescale = softmax_tile8(x, cb, lv, rv, m_ref, l_run, alpha, phi, plo, sb);
      // Keep the probabilities in this block, ahead of the rescale branch.
      // (Schedule groups that interleave the next tile's score MFMAs with the
      // softmax, as in the bf16 kernel, measured slower here.)
      asm volatile("" : : "v"(phi), "v"(plo), "v"(l_run));
      if (rescale) {
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] *= alpha;
      }
      sk8_pv<HD>(stage, v_lds, phi, plo, sb, o);
    }
    have_xn = true;
    ++g;
    ++t;
  };

  // Segments: the tiles of one unit inside this range; the per-tile path
  // carries no segment tests (e4m3 long context: 333 -> 327 us, bit-identical).
  for (;;) {
    const int seg_start = g;
    const int tt0 = cc.tile;
    const int n = min(g1 - g, cc.T - tt0);
    const int n_plain = min(max(max(r.P + 1, 0) / KEYS - tt0, 0), n);
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = f32x16{};
    m_ref = kNoMax;
    l_run = 0.f;
    have_xn = false;
    for (int i = 0; i < n_plain; ++i) step(tt0 + i, std::false_type{});
    for (int i = n_plain; i < n; ++i) step(tt0 + i, std::true_type{});
    if (active)
      sk_segment_end<HD>(a, r, o, m_ref, l_run, tt0 == 0 && tt0 + n == cc.T,
                         rng * 2 + (seg_start == g0 ? 0 : 1), wave, lane);
    if (g >= g1) break;
    cc.tile = tt0 + n - 1;
    cursor_next<KEYS>(a, cc);
    active = seg_ctx(cc, r);
    if (active) load_q_e4m3<HD>(a, r, qhi, qlo, c_row);
    if constexpr (TREE) anc = tree_masks(a)[(size_t)r.b * a.R + r.pos];
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
  RowCtx r = make_row_ctx(a, split, kvh, b, L, m0, lane);
  load_row_anc(a, r);

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

template <int HD, bool TREE>
static hipError_t launch_streamk(const AttnPlan& p, const AttnArgs& a, hipStream_t stream) {
  // Row tiles of one KV head share its K/V through L2; a lone row tile reads
  // them once, so they stream past the caches.
  // Units of at most 64 rows (two of the four waves compute, or fewer) stream
  // faster with one tile fewer in flight: 3 stages for hd 128.
  constexpr int S4 = SkTile<HD>::kStages, S8 = SkTile<HD>::kStages8;
  constexpr int S3 = HD == 128 ? 3 : S4;
  const bool few_rows = p.M <= 2 * kRowsPerWave;
  if (p.fp8 && p.m_tiles == 1)
    sv_attn_streamk_f8<HD, true, TREE><<<p.sk_wgs, kLdsThreads, 0, stream>>>(a);
  else if (p.fp8)
    sv_attn_streamk_f8<HD, false, TREE><<<p.sk_wgs, kLdsThreads, 0, stream>>>(a);
  else if (p.waves == 8 && p.m_tiles == 1)
    sv_attn_streamk<HD, S8, 2, true, 8, TREE><<<p.sk_wgs, 8 * kWave, 0, stream>>>(a);
  else if (p.waves == 8)
    sv_attn_streamk<HD, S8, 2, false, 8, TREE><<<p.sk_wgs, 8 * kWave, 0, stream>>>(a);
  else if (p.m_tiles == 1 && few_rows)
    sv_attn_streamk<HD, S3, kStreamWPE, true, 4, TREE><<<p.sk_wgs, kLdsThreads, 0, stream>>>(a);
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
  a.tree = ptr.tree_mask;
  if (ptr.tree_mask && p.streamk)
    return p.hd == 128 ? launch_streamk<128, true>(p, a, stream) : launch_streamk<64, true>(p, a, stream);
  if (p.streamk)
    return p.hd == 128 ? launch_streamk<128, false>(p, a, stream) : launch_streamk<64, false>(p, a, stream);
  if (p.hd == 128)
    return p.fp8 ? launch_typed<128, true>(p, a, stream) : launch_typed<128, false>(p, a, stream);
  return p.fp8 ? launch_typed<64, true>(p, a, stream) : launch_typed<64, false>(p, a, stream);
}

}  // namespace sv
