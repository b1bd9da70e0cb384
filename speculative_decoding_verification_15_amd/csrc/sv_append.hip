// KV append on gfx950: the K and V rows of the R = 1 + D new positions of every
// sequence are written into its paged cache at token positions
// kv_in[b] .. kv_in[b] + R - 1, and kv_out[b] = kv_in[b] + R.  It is the step
// before verification attention; rejected drafts are undone afterwards by the
// acceptance commit, which lowers the length, and the next append overwrites
// them.
//
//   - 16-token blocks found through a block table: "GPU and LLM" ch. 5,
//     section "PagedAttention (2)".
//   - FP8 storage of the KV data with scaling factors, kept up to date as the
//     cache grows: novita.ai blog "Revolutionizing LLM inference ...", sections
//     "Proprietary FP8 quantization scheme" and "KVCache quantization".
//
// e4m3 caches keep one fp32 scale per (block, KV head), amax / 448 of the
// block's values.  A block that starts in this append takes amax / 448 of its
// new values.  A block that already holds tokens keeps its scale and codes when
// the new values fit under its largest held value (largest decoded code times
// the scale, in fp32); otherwise the scale becomes amax_new / 448 and the held
// codes are re-encoded from their fp32 values.  Encoding = fp32 quotient
// x / scale, rounded to the nearest e4m3 value with ties to the even code and
// magnitudes above 448 saturated; the sign bit is the quotient's.
//
// Tree commit (path != NULL): after a tree acceptance has committed the length
// to L - R + AL, the accepted nodes' rows (path[1 .. AL-1]) are appended by the
// same rule at positions length - (AL - 1) .., right behind the root; the
// lengths are not written.
//
// Launch: one workgroup of 16 waves per sequence.  A wave takes one task at a
// time: (block touched, KV head, K or V).  The workgroup reads kv_in[b] before
// its barrier and one thread writes kv_out[b] after it, so kv_out may alias
// kv_in.
#include "sv_device.h"
#include "sv_internal.h"

namespace sv {

namespace {

constexpr int kAppendWaves = 16;
constexpr int kBlock = 16;

struct AppendArgs {
  const uint16_t* k_new;   // [B][R][H_kv][hd] bf16 bits
  const uint16_t* v_new;
  void* k_cache;
  void* v_cache;
  float* k_scale;          // [num_blocks][H_kv], e4m3 only
  float* v_scale;
  const int32_t* table;    // [B][max_blocks]
  const int32_t* kv_in;
  int32_t* kv_out;         // NULL in the tree commit (lengths already committed)
  const int32_t* path;     // tree commit: [B][R] accepted nodes, root first, -1 padded; else NULL
  int R, H_kv, hd, max_blocks, num_blocks;
};

// Row of k_new / v_new that the i-th appended position of sequence b takes:
// i itself, or in the tree commit the (i + 1)-th accepted node.
__device__ __forceinline__ int src_row(const AppendArgs& p, int b, int i) {
  if (!p.path) return i;
  return min(max(p.path[(size_t)b * p.R + 1 + i], 0), p.R - 1);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}

// fp32 -> OCP e4m3 code: nearest value, ties to the even mantissa, magnitudes of
// 448 and above give 448, the sign bit copied from y (finite y).
__device__ __forceinline__ uint32_t e4m3_encode(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  uint32_t mag;
  if (a >= 0x43E00000u) {                  // |y| >= 448
    mag = 0x7Eu;
  } else if (a < 0x3C800000u) {            // |y| < 2^-6: multiples of 2^-9
    mag = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);   // exact scaling; 8 -> 2^-6
  } else {                                 // exponent field 1..15, 3 mantissa bits kept
    const uint32_t m = a & 0x7FFFFFu;
    uint32_t q = (((a >> 23) - 120u) << 3) | (m >> 20);
    const uint32_t rem = m & 0xFFFFFu;
    q += (rem > 0x80000u) || (rem == 0x80000u && (q & 1u));   // a carry moves the exponent up
    mag = q > 0x7Eu ? 0x7Eu : q;
  }
  return sign | mag;
}

// Decoded e4m3 byte `sel` of word w (exact fp32).
template <int SEL>
__device__ __forceinline__ float e4m3_byte(uint32_t w) {
  return __builtin_amdgcn_cvt_f32_fp8((int)w, SEL);
}

__device__ __forceinline__ void decode16(const u32x4 raw, float (&x)[16]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[4 * i + 0] = e4m3_byte<0>(raw[i]);
    x[4 * i + 1] = e4m3_byte<1>(raw[i]);
    x[4 * i + 2] = e4m3_byte<2>(raw[i]);
    x[4 * i + 3] = e4m3_byte<3>(raw[i]);
  }
}

__device__ __forceinline__ u32x4 encode16(const float (&x)[16], float s) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t w = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) w |= e4m3_encode(__fdiv_rn(x[4 * i + k], s)) << (8 * k);
    r[i] = w;
  }
  return r;
}

// Scale of a block after the append (see the file comment).  a = held slots.
__device__ __forceinline__ float next_scale(int a, float amax_new, float held_max, float s_old,
                                            bool& reencode) {
  reencode = false;
  if (a > 0) {
    const float a_held = __fmul_rn(held_max, s_old);
    if (amax_new <= a_held) return s_old;
    reencode = true;
  }
  return amax_new == 0.f ? 1.f : __fdiv_rn(amax_new, 448.f);
}

// e4m3 K block [hd/16][16 slots][16 dims]: lane owns 16-byte chunks e = lane + 64 k
// (chunk e = dims 16 (e / 16) .. +16 of slot e % 16); a chunk is held, new or untouched.
template <int HD>
__device__ void append_k_fp8(const AppendArgs& p, int b, int c, int P, int a, int n, size_t blk,
                             int h, int lane) {
  constexpr int CH = HD / 64;
  uint8_t* base = static_cast<uint8_t*>(p.k_cache) + (blk * p.H_kv + h) * (size_t)(HD * kBlock);
  float* scale = p.k_scale + blk * p.H_kv + h;
  const float s_old = a > 0 ? *scale : 1.f;     // issued ahead of the block's loads
  float x[CH][16];
  bool held[CH], isnew[CH];
  float nmax = 0.f, hmax = 0.f;
#pragma unroll
  for (int k = 0; k < CH; ++k) {
    const int e = lane + 64 * k, slot = e & 15, d16 = e >> 4;
    held[k] = slot < a;
    isnew[k] = slot >= a && slot < a + n;
    if (held[k]) {
      decode16(*reinterpret_cast<const u32x4*>(base + e * 16), x[k]);
#pragma unroll
      for (int i = 0; i < 16; ++i) hmax = fmaxf(hmax, fabsf(x[k][i]));
    } else if (isnew[k]) {
      const uint16_t* src = p.k_new + (((size_t)b * p.R + src_row(p, b, P + slot - c)) * p.H_kv + h) * HD + d16 * 16;
      const u32x4 w0 = *reinterpret_cast<const u32x4*>(src);
      const u32x4 w1 = *reinterpret_cast<const u32x4*>(src + 8);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[k][2 * i] = bf16_to_f32(w0[i] & 0xFFFFu);
        x[k][2 * i + 1] = bf16_to_f32(w0[i] >> 16);
        x[k][8 + 2 * i] = bf16_to_f32(w1[i] & 0xFFFFu);
        x[k][8 + 2 * i + 1] = bf16_to_f32(w1[i] >> 16);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) nmax = fmaxf(nmax, fabsf(x[k][i]));
    }
  }
  nmax = wave_max(nmax);
  hmax = wave_max(hmax);
  bool reencode;
  const float s = next_scale(a, nmax, hmax, s_old, reencode);
#pragma unroll
  for (int k = 0; k < CH; ++k) {
    const int e = lane + 64 * k;
    if (held[k] && reencode) {
#pragma unroll
      for (int i = 0; i < 16; ++i) x[k][i] = __fmul_rn(x[k][i], s_old);
    }
    if (isnew[k] || (held[k] && reencode))
      *reinterpret_cast<u32x4*>(base + e * 16) = encode16(x[k], s);
  }
  if (lane == 0) *scale = s;
}

// e4m3 V block [hd][16 slots]: lane owns dims d = lane + 64 k, one 16-byte row each,
// read, updated in the written slots, and stored whole.
template <int HD>
__device__ void append_v_fp8(const AppendArgs& p, int b, int c, int P, int a, int n, size_t blk,
                             int h, int lane) {
  constexpr int CH = HD / 64;
  uint8_t* base = static_cast<uint8_t*>(p.v_cache) + (blk * p.H_kv + h) * (size_t)(HD * kBlock);
  float* scale = p.v_scale + blk * p.H_kv + h;
  const float s_old = a > 0 ? *scale : 1.f;     // issued ahead of the block's loads
  u32x4 raw[CH];
  float x[CH][16];
  float nmax = 0.f, hmax = 0.f;
#pragma unroll
  for (int k = 0; k < CH; ++k) {
    const int d = lane + 64 * k;
    raw[k] = *reinterpret_cast<const u32x4*>(base + d * 16);
    decode16(raw[k], x[k]);
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      if (t < a) {
        hmax = fmaxf(hmax, fabsf(x[k][t]));
      } else if (t < a + n) {
        x[k][t] = bf16_to_f32(p.v_new[(((size_t)b * p.R + src_row(p, b, P + t - c)) * p.H_kv + h) * HD + d]);
        nmax = fmaxf(nmax, fabsf(x[k][t]));
      }
    }
  }
  nmax = wave_max(nmax);
  hmax = wave_max(hmax);
  bool reencode;
  const float s = next_scale(a, nmax, hmax, s_old, reencode);
#pragma unroll
  for (int k = 0; k < CH; ++k) {
    const int d = lane + 64 * k;
    u32x4 out = raw[k];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const bool put_new = t >= a && t < a + n;
      const bool put_held = t < a && reencode;
      if (put_new || put_held) {
        const float y = put_held ? __fmul_rn(x[k][t], s_old) : x[k][t];
        const uint32_t code = e4m3_encode(__fdiv_rn(y, s));
        const int wi = t >> 2, sh = 8 * (t & 3);
        out[wi] = (out[wi] & ~(0xFFu << sh)) | (code << sh);
      }
    }
    *reinterpret_cast<u32x4*>(base + d * 16) = out;
  }
  if (lane == 0) *scale = s;
}

// bf16 K block [hd/8][16 slots][8 dims]: one 16-byte vector per (new slot, 8 dims).
// Every load is issued before the first store (fixed trip counts, guarded), so
// a task costs one memory round trip rather than one per vector.
template <int HD>
__device__ void append_k_bf16(const AppendArgs& p, int b, int c, int P, int a, int n, size_t blk,
                              int h, int lane) {
  constexpr int V8 = HD / 8;
  constexpr int IT = kBlock * V8 / 64;       // vectors per lane for a full block
  uint16_t* base = static_cast<uint16_t*>(p.k_cache) + (blk * p.H_kv + h) * (size_t)(HD * kBlock);
  u32x4 val[IT];
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const int e = lane + 64 * i, s = e / V8, d8 = e % V8;
    if (s < n)
      val[i] = *reinterpret_cast<const u32x4*>(
          p.k_new + (((size_t)b * p.R + src_row(p, b, P + a + s - c)) * p.H_kv + h) * HD + d8 * 8);
  }
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const int e = lane + 64 * i, s = e / V8, d8 = e % V8;
    if (s < n) *reinterpret_cast<u32x4*>(base + d8 * 128 + (a + s) * 8) = val[i];
  }
}

// bf16 V block [hd][16 slots]: lane owns dims d = lane + 64 k, one 2-byte store per new slot;
// all loads first, as for K.
template <int HD>
__device__ void append_v_bf16(const AppendArgs& p, int b, int c, int P, int a, int n, size_t blk,
                              int h, int lane) {
  uint16_t* base = static_cast<uint16_t*>(p.v_cache) + (blk * p.H_kv + h) * (size_t)(HD * kBlock);
  uint16_t val[HD / 64][kBlock];
#pragma unroll
  for (int s = 0; s < kBlock; ++s) {
    if (s < n) {
      const uint16_t* src = p.v_new + (((size_t)b * p.R + src_row(p, b, P + a + s - c)) * p.H_kv + h) * HD;
#pragma unroll
      for (int k = 0; k < HD / 64; ++k) val[k][s] = src[lane + 64 * k];
    }
  }
#pragma unroll
  for (int k = 0; k < HD / 64; ++k)
#pragma unroll
    for (int s = 0; s < kBlock; ++s)
      if (s < n) base[(lane + 64 * k) * 16 + a + s] = val[k][s];
}

template <int HD, bool FP8>
__global__ __launch_bounds__(kAppendWaves * 64) void sv_kv_append(AppendArgs p) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int cap = p.max_blocks * kBlock;
  // rows appended: all R, or in the tree commit the accepted nodes after the
  // root (up to the first -1), placed right behind the root
  int rows = p.R;
  if (p.path) {
    rows = 0;
    while (rows + 1 < p.R && p.path[(size_t)b * p.R + rows + 1] >= 0) ++rows;
  }
  const int start = p.path ? p.kv_in[b] - rows : p.kv_in[b];
  const int c = min(max(start, 0), cap - rows);         // in-bounds even for bad lengths
  const int span = (rows + 30) / kBlock;                // most blocks [c, c + rows) can touch
  const int tasks = span * p.H_kv * 2;
  for (int t = wave; t < tasks; t += kAppendWaves) {
    const int j = t / (2 * p.H_kv);
    const int h = (t >> 1) % p.H_kv;
    const bool is_v = t & 1;
    const int jb = c / kBlock + j;
    const int P = jb * kBlock;
    const int lo = max(c, P), hi = min(c + rows, P + kBlock);
    if (lo >= hi) continue;
    const int a = lo - P;          // held slots 0 .. a-1 (non-zero only in the first block)
    const int n = hi - lo;         // new slots a .. a+n-1
    int blk = p.table[(size_t)b * p.max_blocks + jb];
    blk = min(max(blk, 0), p.num_blocks - 1);
    if constexpr (FP8) {
      if (is_v) append_v_fp8<HD>(p, b, c, P, a, n, (size_t)blk, h, lane);
      else append_k_fp8<HD>(p, b, c, P, a, n, (size_t)blk, h, lane);
    } else {
      if (is_v) append_v_bf16<HD>(p, b, c, P, a, n, (size_t)blk, h, lane);
      else append_k_bf16<HD>(p, b, c, P, a, n, (size_t)blk, h, lane);
    }
  }
  __syncthreads();
  if (threadIdx.x == 0 && p.kv_out) p.kv_out[b] = c + p.R;
}

}  // namespace

hipError_t launch_kv_append(const AppendPlan& pl, const void* k_new, const void* v_new,
                            void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                            const int32_t* table, const int32_t* kv_in, int32_t* kv_out,
                            const int32_t* path, hipStream_t stream) {
  AppendArgs a{static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
               k_cache, v_cache, k_scale, v_scale, table, kv_in, kv_out, path,
               pl.R, pl.H_kv, pl.hd, pl.max_blocks, pl.num_blocks};
  const dim3 grid(pl.B), block(kAppendWaves * 64);
  if (pl.hd == 128) {
    if (pl.fp8) sv_kv_append<128, true><<<grid, block, 0, stream>>>(a);
    else sv_kv_append<128, false><<<grid, block, 0, stream>>>(a);
  } else {
    if (pl.fp8) sv_kv_append<64, true><<<grid, block, 0, stream>>>(a);
    else sv_kv_append<64, false><<<grid, block, 0, stream>>>(a);
  }
  return hipGetLastError();
}

}  // namespace sv
