// Greedy acceptance on gfx950: per-row vocabulary argmax, then the
// first-mismatch prefix, acceptance length and KV-length commit.
//
// The target's own token at a verified position is the argmax of its logits
// there, and drafts are kept up to the first one that differs from it, after
// which the target's token is emitted ("GPU and LLM" ch. 5, section
// "Speculative decoding (2): verify in one pass"; NVIDIA co-design summary,
// section "Basic structure of speculative decoding": AL in 1 .. 1 + D).
//
// Pass 1 (sv_argmax_partial) streams the logits once: every workgroup reduces a
// chunk of 4096 logits of one row to (max value, lowest index holding it).
// Pass 2 (sv_accept_finalize) reduces the chunk results of each row and runs
// the prefix scan for one sequence per wave.  Ties resolve to the lower index
// everywhere; values are compared as floats, never as bit patterns, so -0 and
// +0 tie.
#include "sv_device.h"
#include "sv_internal.h"

namespace sv {

struct ArgmaxPart {
  float value;
  int32_t index;
};

// (v, i) beats (bv, bi): larger value, or the same value at a lower index.
__device__ __forceinline__ bool beats(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

__device__ __forceinline__ void consider(float v, int i, float& bv, int& bi) {
  if (beats(v, i, bv, bi)) { bv = v; bi = i; }
}

__device__ __forceinline__ void wave_argmax(float& bv, int& bi) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    float ov = __shfl_xor(bv, off);
    int oi = __shfl_xor(bi, off);
    consider(ov, oi, bv, bi);
  }
}

// grid = (chunks per row, rows); 256 threads.  VEC: rows start 16-byte aligned
// (V % 4 == 0), so whole float4 loads are used.
template <bool VEC>
__global__ __launch_bounds__(kArgmaxThreads) void sv_argmax_partial(
    const float* __restrict__ logits, int V, int chunks, ArgmaxPart* __restrict__ part) {
  const int chunk = blockIdx.x;
  const size_t row = blockIdx.y;
  const float* x = logits + row * (size_t)V;
  const int base = chunk * kArgmaxChunk;
  const int t = threadIdx.x;
  float bv = -INFINITY;
  int bi = INT32_MAX;
  if constexpr (VEC) {
    constexpr int U = kArgmaxChunk / (kArgmaxThreads * 4);
    f32x4 buf[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i0 = base + (u * kArgmaxThreads + t) * 4;
      if (i0 + 3 < V) {
        buf[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(x + i0));
      } else {
        f32x4 r;
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = (i0 + e < V) ? x[i0 + e] : -INFINITY;
        buf[u] = r;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i0 = base + (u * kArgmaxThreads + t) * 4;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (i0 + e < V) consider(buf[u][e], i0 + e, bv, bi);
    }
  } else {
    constexpr int U = kArgmaxChunk / kArgmaxThreads;
#pragma unroll 8
    for (int u = 0; u < U; ++u) {
      const int i = base + u * kArgmaxThreads + t;
      if (i < V) consider(x[i], i, bv, bi);
    }
  }
  wave_argmax(bv, bi);
  __shared__ float sv_[kArgmaxThreads / kWave];
  __shared__ int si_[kArgmaxThreads / kWave];
  const int w = t / kWave;
  if ((t % kWave) == 0) { sv_[w] = bv; si_[w] = bi; }
  __syncthreads();
  if (t == 0) {
#pragma unroll
    for (int k = 1; k < kArgmaxThreads / kWave; ++k) consider(sv_[k], si_[k], bv, bi);
    part[row * chunks + chunk] = ArgmaxPart{bv, bi};
  }
}

// grid = B; one wave per sequence; lane j handles row j (R <= 64).
__global__ __launch_bounds__(kWave) void sv_accept_finalize(
    const ArgmaxPart* __restrict__ part, int chunks, int D, const int32_t* __restrict__ draft,
    int32_t* __restrict__ target, int32_t* __restrict__ accept_len,
    int32_t* __restrict__ out_tokens, const int32_t* kv_in, int32_t* kv_out) {
  const int b = blockIdx.x;
  const int j = threadIdx.x;
  const int R = D + 1;
  int tok = 0;
  if (j < R) {
    const ArgmaxPart* p = part + ((size_t)b * R + j) * chunks;
    float bv = -INFINITY;
    int bi = INT32_MAX;
    for (int c = 0; c < chunks; ++c) consider(p[c].value, p[c].index, bv, bi);
    tok = bi;
    target[(size_t)b * R + j] = tok;
  }
  const bool mismatch = (j < D) && (draft[(size_t)b * D + j] != tok);
  const unsigned long long mask = __ballot(mismatch);
  const int n = mask ? (__ffsll((long long)mask) - 1) : D;
  const int tok_n = __shfl(tok, n);
  if (j < R) {
    int o = -1;
    if (j < n) o = draft[(size_t)b * D + j];
    else if (j == n) o = tok_n;
    out_tokens[(size_t)b * R + j] = o;
  }
  if (j == 0) {
    const int kv = kv_in[b];
    accept_len[b] = n + 1;
    kv_out[b] = kv - R + n + 1;
  }
}

hipError_t launch_accept(int B, int D, int V, const float* logits, const int32_t* draft,
                         int32_t* target, int32_t* accept_len, int32_t* out_tokens,
                         const int32_t* kv_in, int32_t* kv_out, void* ws, hipStream_t stream) {
  const int R = D + 1;
  const int chunks = argmax_chunks(V);
  auto* part = static_cast<ArgmaxPart*>(ws);
  dim3 grid(chunks, B * R);
  if (V % 4 == 0)
    sv_argmax_partial<true><<<grid, kArgmaxThreads, 0, stream>>>(logits, V, chunks, part);
  else
    sv_argmax_partial<false><<<grid, kArgmaxThreads, 0, stream>>>(logits, V, chunks, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  sv_accept_finalize<<<B, kWave, 0, stream>>>(part, chunks, D, draft, target, accept_len,
                                               out_tokens, kv_in, kv_out);
  return hipGetLastError();
}

}  // namespace sv
