// Stochastic (lossless) acceptance on gfx950.
//
// The acceptance rule keeps the output distribution of the large model alone
// ("GPU and LLM" ch. 5, section "Speculative decoding (2): verify in one
// pass"); the rule is the one of the paper the pages cite for speculative
// decoding (Leviathan et al., ICML 2023, cited in "Speculative decoding (1)"):
// draft d_j, drawn from the draft distribution q_j, is kept with probability
// min(1, p_j(d_j) / q_j(d_j)); at the first draft not kept the emitted token is
// drawn from max(0, p_j - q_j), renormalised; when all D drafts are kept, the
// bonus token is drawn from p_D.  p_j = softmax(target row j / tau), q_j =
// softmax(draft row j / tau).  Keeping is the test u_j * q_j(d_j) < p_j(d_j);
// a draw with uniform u takes the first index whose running sum exceeds u
// times the total.
//
// Pass 1 (sv_sample_stats) streams every target and draft row once: each
// workgroup reduces 4096 logits of one row to (max m, sum of e^((z - m) / tau)),
// the sum accumulated in fp64.  Every weight is exp((z - m) / tau) with a
// correctly rounded division and the accurate exponential, so its error is a
// few ulp and independent from one logit to the next: a rounded log2(e) / tau
// would scale every exponent by the same factor and shift all the draw's
// boundaries the same way.  Pass 2
// (sv_sample_decide, one workgroup per sequence) combines the chunks of its
// rows, runs the keep tests in order, and draws the emitted token from the one
// row it needs: a first pass sums the weights of each thread's contiguous
// segment (fp64), an exclusive scan places the segments, and the thread whose
// segment holds u * total walks it again to find the index.
#include "sv_device.h"
#include "sv_internal.h"

namespace sv {

struct SampleStat {
  float m;       // chunk maximum (-inf: nothing finite in the chunk)
  float pad;
  double s;      // sum over the chunk of e^((z - m) / tau)
};

__device__ __forceinline__ float block_max(float v, float* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  const int w = threadIdx.x / kWave;
  if (threadIdx.x % kWave == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < kArgmaxThreads / kWave; ++i) r = fmaxf(r, red[i]);
  return r;
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// grid = (chunks, B * (1 + D) + B * D); rows below rows_t are target rows
// (b * R + j), the others draft rows (b * D + j).  VEC: V % 4 == 0, so rows
// start 16-byte aligned and whole float4 loads are used.
template <bool VEC>
__global__ __launch_bounds__(kArgmaxThreads) void sv_sample_stats(
    const float* __restrict__ zt, const float* __restrict__ zd, int rows_t, int V, int chunks,
    float tau, SampleStat* __restrict__ st) {
  constexpr int U = kArgmaxChunk / kArgmaxThreads;   // logits per thread
  __shared__ float red_m[kArgmaxThreads / kWave];
  __shared__ double red_s[kArgmaxThreads / kWave];
  const int chunk = blockIdx.x;
  const int row = blockIdx.y;
  const float* x = row < rows_t ? zt + (size_t)row * V : zd + (size_t)(row - rows_t) * V;
  const int base = chunk * kArgmaxChunk;
  const int t = threadIdx.x;
  float v[U];
  if constexpr (VEC) {
#pragma unroll
    for (int u = 0; u < U / 4; ++u) {
      const int i0 = base + (u * kArgmaxThreads + t) * 4;
      f32x4 r;
      if (i0 + 3 < V) {
        r = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(x + i0));
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = (i0 + e < V) ? x[i0 + e] : -INFINITY;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * u + e] = r[e];
    }
  } else {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = base + u * kArgmaxThreads + t;
      v[u] = i < V ? x[i] : -INFINITY;
    }
  }
  float m = v[0];
#pragma unroll
  for (int u = 1; u < U; ++u) m = fmaxf(m, v[u]);
  m = block_max(m, red_m);
  double s = 0.0;
  if (m != -INFINITY) {
#pragma unroll
    for (int u = 0; u < U; ++u) s += (double)expf((v[u] - m) / tau);
  }
  s = wave_sum(s);
  if (t % kWave == 0) red_s[t / kWave] = s;
  __syncthreads();
  if (t == 0) {
    double tot = red_s[0];
#pragma unroll
    for (int i = 1; i < kArgmaxThreads / kWave; ++i) tot += red_s[i];
    st[(size_t)row * chunks + chunk] = SampleStat{m, 0.f, tot};
  }
}

// grid = B, 256 threads.
__global__ __launch_bounds__(kArgmaxThreads) void sv_sample_decide(
    const float* __restrict__ zt, const float* __restrict__ zd, const int32_t* __restrict__ draft,
    const float* __restrict__ u_accept, const float* __restrict__ u_sample, int D, int V,
    int chunks, float tau, const SampleStat* __restrict__ st, int32_t* __restrict__ accept_len,
    int32_t* __restrict__ out_tokens, const int32_t* __restrict__ kv_in,
    int32_t* __restrict__ kv_out) {
  constexpr int kThreads = kArgmaxThreads;
  __shared__ float s_M[2 * 64 + 1];         // per row r: target rows 0 .. D, draft rows R + j
  __shared__ double s_S[2 * 64 + 1];
  __shared__ double s_part[kThreads];       // segment sums, then their exclusive prefixes
  __shared__ double s_total;
  __shared__ int s_n, s_tok;
  const int b = blockIdx.x;
  const int R = D + 1;
  const int t = threadIdx.x;
  const int lane = t % kWave, wave = t / kWave;
  const int B = gridDim.x;

  // Row normalisers: max M over the chunks and S = sum_c s_c e^((m_c - M) / tau).
  for (int r = wave; r < R + D; r += kThreads / kWave) {
    const size_t row = r < R ? (size_t)b * R + r : (size_t)B * R + (size_t)b * D + (r - R);
    const SampleStat* sr = st + row * chunks;
    float mc = -INFINITY;
    for (int c = lane; c < chunks; c += kWave) mc = fmaxf(mc, sr[c].m);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mc = fmaxf(mc, __shfl_xor(mc, off));
    double sc = 0.0;
    for (int c = lane; c < chunks; c += kWave) {
      const SampleStat x = sr[c];
      if (x.s > 0.0) sc += x.s * (double)expf((x.m - mc) / tau);
    }
    sc = wave_sum(sc);
    if (lane == 0) {
      s_M[r] = mc;
      s_S[r] = sc;
    }
  }
  if (t == 0) s_tok = -1;
  __syncthreads();

  // Keep tests, in order, up to the first draft not kept.
  if (t == 0) {
    int n = D;
    for (int j = 0; j < D; ++j) {
      const int d = min(max(draft[(size_t)b * D + j], 0), V - 1);
      const double p = (double)expf((zt[((size_t)b * R + j) * V + d] - s_M[j]) / tau) / s_S[j];
      const double q =
          (double)expf((zd[((size_t)b * D + j) * V + d] - s_M[R + j]) / tau) / s_S[R + j];
      if (!((double)u_accept[(size_t)b * D + j] * q < p)) {
        n = j;
        break;
      }
    }
    s_n = n;
  }
  __syncthreads();
  const int n = s_n;

  // The row to draw from: the residual max(0, p_n - q_n) after a draft not
  // kept, else p_D; a residual that is zero everywhere falls back to p_n.
  const float* zr = zt + ((size_t)b * R + n) * V;
  const float Mp = s_M[n];
  // Weights in fp64 (fp32 exponentials times fp64 1 / S): a rounded fp32 1 / S
  // would scale all of p, or all of q, by one factor and move every boundary of
  // the residual together.
  const double invSp = 1.0 / s_S[n];
  bool resid = n < D;
  const float* yr = resid ? zd + ((size_t)b * D + n) * V : zr;
  const float Mq = resid ? s_M[R + n] : 0.f;
  const double invSq = resid ? 1.0 / s_S[R + n] : 0.0;
  auto weight = [&](int v) -> double {
    const double p = (double)expf((zr[v] - Mp) / tau) * invSp;
    if (!resid) return p;
    const double q = (double)expf((yr[v] - Mq) / tau) * invSq;
    return fmax(p - q, 0.0);
  };
  const int seg = (V + kThreads - 1) / kThreads;
  const int v0 = min(t * seg, V), v1 = min(v0 + seg, V);
  double own = 0.0, pre = 0.0;
  for (int pass = 0; pass < 2; ++pass) {
    own = 0.0;
    for (int v = v0; v < v1; ++v) own += weight(v);
    s_part[t] = own;
    __syncthreads();
    if (t == 0) {                            // exclusive prefix, in thread order
      double run = 0.0;
      for (int i = 0; i < kThreads; ++i) {
        const double x = s_part[i];
        s_part[i] = run;
        run += x;
      }
      s_total = run;
    }
    __syncthreads();
    pre = s_part[t];
    if (!(resid && s_total == 0.0)) break;   // uniform: s_total is shared
    resid = false;                           // p_n == q_n: draw from p_n
    __syncthreads();                         // everyone has read s_part / s_total
  }
  const double T = (double)u_sample[b] * s_total;
  // The segments tile [0, total) in thread order; exactly one with own > 0
  // holds T.  Its walk repeats the same weights; should rounding keep the
  // running sum from passing T, the segment's last positive weight is taken.
  if (own > 0.0 && pre <= T && T < pre + own) {
    double run = pre;
    int tok = -1, last = -1;
    for (int v = v0; v < v1; ++v) {
      const double w = weight(v);
      if (w > 0.0) last = v;
      run += w;
      if (run > T) {
        tok = v;
        break;
      }
    }
    s_tok = tok >= 0 ? tok : last;
  }
  __syncthreads();
  if (t == 0) {
    const int tok = s_tok;
    accept_len[b] = n + 1;
    kv_out[b] = kv_in[b] - R + n + 1;
    for (int j = 0; j < R; ++j)
      out_tokens[(size_t)b * R + j] = j < n ? draft[(size_t)b * D + j] : (j == n ? tok : -1);
  }
}

hipError_t launch_accept_sampled(int B, int D, int V, float tau, const float* zt, const float* zd,
                                 const int32_t* draft, const float* u_accept,
                                 const float* u_sample, int32_t* accept_len, int32_t* out_tokens,
                                 const int32_t* kv_in, int32_t* kv_out, void* ws,
                                 hipStream_t stream) {
  const int R = D + 1;
  const int chunks = argmax_chunks(V);
  auto* st = static_cast<SampleStat*>(ws);
  dim3 grid(chunks, B * (R + D));
  if (V % 4 == 0)
    sv_sample_stats<true><<<grid, kArgmaxThreads, 0, stream>>>(zt, zd, B * R, V, chunks, tau, st);
  else
    sv_sample_stats<false><<<grid, kArgmaxThreads, 0, stream>>>(zt, zd, B * R, V, chunks, tau, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  sv_sample_decide<<<B, kArgmaxThreads, 0, stream>>>(zt, zd, draft, u_accept, u_sample, D, V,
                                                     chunks, tau, st, accept_len, out_tokens,
                                                     kv_in, kv_out);
  return hipGetLastError();
}

}  // namespace sv
