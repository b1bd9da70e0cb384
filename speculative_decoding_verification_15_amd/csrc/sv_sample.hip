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
// boundaries the same way.
// Pass 2 (sv_sample_keep, one workgroup per sequence) combines the chunks of its
// rows, runs the keep tests in order and writes every output but the emitted
// token.  The emitted token is drawn from the one row it needs in two passes
// that read it coalesced: sv_sample_chunk_sums (one workgroup per 4096-logit
// chunk) sums the weights of each chunk in fp64; sv_sample_draw (one workgroup
// per sequence) finds the chunk holding u * total from the chunk sums in index
// order, sums 16 consecutive weights per thread inside it, places the threads'
// segments by an exclusive prefix in thread order, and the thread whose segment
// holds the target walks it again to find the index.
#include "sv_device.h"
#include "sv_internal.h"

namespace sv {

// x / tau; with UNIT_TAU (tau == 1) the division, exact then, is left out.
template <bool UNIT_TAU>
__device__ __forceinline__ float over_tau(float x, float tau) {
  if constexpr (UNIT_TAU) return x;
  else return x / tau;
}

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
template <bool VEC, bool UNIT_TAU>
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
    for (int u = 0; u < U; ++u) s += (double)expf(over_tau<UNIT_TAU>(v[u] - m, tau));
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

// What the draw of sequence b needs, written by sv_sample_keep.
struct DrawInfo {
  int32_t n;       // first draft not kept (D if all kept): the emitted token's row
  int32_t resid;   // 1: draw from max(0, p_n - q_n); 0: draw from p_n (= p_D)
  float Mp, Mq;    // row maxima of target row n and draft row n
  double invSp;    // 1 / S of target row n
  double invSq;    // 1 / S of draft row n (resid only)
};

// The unnormalised weights of the emitted token's distribution at index v:
// p_n(v), and max(0, p_n(v) - q_n(v)) when drawing from the residual.  fp32
// exponentials (correctly rounded division, accurate exp) times an fp64 1 / S:
// a rounded fp32 1 / S would scale all of p, or all of q, by one factor and move
// every boundary of the residual together.
template <bool UNIT_TAU = false>
__device__ __forceinline__ double weight_p(float z, const DrawInfo& d, float tau) {
  return (double)expf(over_tau<UNIT_TAU>(z - d.Mp, tau)) * d.invSp;
}
template <bool UNIT_TAU = false>
__device__ __forceinline__ double weight_r(float z, float y, const DrawInfo& d, float tau) {
  const double q = (double)expf(over_tau<UNIT_TAU>(y - d.Mq, tau)) * d.invSq;
  return fmax(weight_p<UNIT_TAU>(z, d, tau) - q, 0.0);
}

// grid = B, 1024 threads: row normalisers (max M over the chunks and
// S = sum_c s_c e^((m_c - M) / tau)), the keep tests in order, and every output
// but the emitted token.
constexpr int kKeepThreads = 1024;   // 16 waves: the row normalisers of up to 127 rows, 8 per wave

__global__ __launch_bounds__(kKeepThreads) void sv_sample_keep(
    const float* __restrict__ zt, const float* __restrict__ zd, const int32_t* __restrict__ draft,
    const float* __restrict__ u_accept, int D, int V, int chunks, float tau,
    const SampleStat* __restrict__ st, DrawInfo* __restrict__ info,
    int32_t* __restrict__ accept_len, int32_t* __restrict__ out_tokens,
    const int32_t* __restrict__ kv_in, int32_t* __restrict__ kv_out) {
  constexpr int kThreads = kKeepThreads;
  __shared__ float s_M[2 * 64 + 1];         // per row r: target rows 0 .. D, draft rows R + j
  __shared__ double s_S[2 * 64 + 1];
  __shared__ bool s_keep[64];
  const int b = blockIdx.x;
  const int R = D + 1;
  const int t = threadIdx.x;
  const int lane = t % kWave, wave = t / kWave;
  const int B = gridDim.x;

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
  __syncthreads();
  // every keep test's inputs fetched at once (thread j: draft j), tested in order below
  if (t < D) {
    const int j = t;
    const int d = min(max(draft[(size_t)b * D + j], 0), V - 1);
    const double p = (double)expf((zt[((size_t)b * R + j) * V + d] - s_M[j]) / tau) / s_S[j];
    const double q = (double)expf((zd[((size_t)b * D + j) * V + d] - s_M[R + j]) / tau) / s_S[R + j];
    s_keep[j] = (double)u_accept[(size_t)b * D + j] * q < p;
  }
  __syncthreads();
  if (t != 0) return;
  int n = D;
  for (int j = 0; j < D; ++j) {
    if (!s_keep[j]) {
      n = j;
      break;
    }
  }
  const bool resid = n < D;
  info[b] = DrawInfo{n, resid ? 1 : 0, s_M[n], resid ? s_M[R + n] : 0.f, 1.0 / s_S[n],
                     resid ? 1.0 / s_S[R + n] : 0.0};
  accept_len[b] = n + 1;
  const int k = kv_in[b];
  kv_out[b] = k - R + n + 1;
  for (int j = 0; j < R; ++j)
    if (j != n) out_tokens[(size_t)b * R + j] = j < n ? draft[(size_t)b * D + j] : -1;
}

// grid = (chunks, B), 256 threads: the sums of the draw weights over each
// 4096-logit chunk of the emitted token's row, read coalesced.  Per chunk:
// {sum of the drawn weights, sum of p_n} (the second serves when the residual is
// zero everywhere, p_n == q_n).
template <bool VEC, bool UNIT_TAU>
__global__ __launch_bounds__(kArgmaxThreads) void sv_sample_chunk_sums(
    const float* __restrict__ zt, const float* __restrict__ zd, int D, int V, int chunks,
    float tau, const DrawInfo* __restrict__ info, double2* __restrict__ sums) {
  constexpr int U = kArgmaxChunk / kArgmaxThreads;
  __shared__ double red_w[kArgmaxThreads / kWave], red_p[kArgmaxThreads / kWave];
  const int chunk = blockIdx.x, b = blockIdx.y;
  const int R = D + 1;
  const DrawInfo di = info[b];
  const float* zr = zt + ((size_t)b * R + di.n) * V;
  const float* yr = di.resid ? zd + ((size_t)b * D + di.n) * V : zr;
  const int base = chunk * kArgmaxChunk;
  const int t = threadIdx.x;
  double sw = 0.0, sp = 0.0;
  if constexpr (VEC) {
#pragma unroll
    for (int u = 0; u < U / 4; ++u) {
      const int i0 = base + (u * kArgmaxThreads + t) * 4;
      if (i0 >= V) continue;
      f32x4 z4, y4;
      if (i0 + 3 < V) {
        z4 = *reinterpret_cast<const f32x4*>(zr + i0);
        y4 = *reinterpret_cast<const f32x4*>(yr + i0);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          z4[e] = (i0 + e < V) ? zr[i0 + e] : -INFINITY;
          y4[e] = (i0 + e < V) ? yr[i0 + e] : -INFINITY;
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (z4[e] == -INFINITY) continue;
        const double p = weight_p<UNIT_TAU>(z4[e], di, tau);
        sp += p;
        sw += di.resid ? weight_r<UNIT_TAU>(z4[e], y4[e], di, tau) : p;
      }
    }
  } else {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = base + u * kArgmaxThreads + t;
      if (i >= V || zr[i] == -INFINITY) continue;
      const double p = weight_p<UNIT_TAU>(zr[i], di, tau);
      sp += p;
      sw += di.resid ? weight_r<UNIT_TAU>(zr[i], yr[i], di, tau) : p;
    }
  }
  sw = wave_sum(sw);
  sp = wave_sum(sp);
  if (t % kWave == 0) {
    red_w[t / kWave] = sw;
    red_p[t / kWave] = sp;
  }
  __syncthreads();
  if (t == 0) {
    double a = red_w[0], c = red_p[0];
#pragma unroll
    for (int i = 1; i < kArgmaxThreads / kWave; ++i) {
      a += red_w[i];
      c += red_p[i];
    }
    sums[(size_t)b * chunks + chunk] = double2{a, c};
  }
}

// grid = B, 256 threads: the chunk holding u * total (chunk sums in index
// order), then inside it 16 consecutive logits per thread: thread sums, their
// exclusive prefix in thread order, and a walk by the thread whose segment holds
// the target.  Should rounding keep every running sum short of the target, the
// last positive weight in reach is taken.
__global__ __launch_bounds__(kArgmaxThreads) void sv_sample_draw(
    const float* __restrict__ zt, const float* __restrict__ zd, const float* __restrict__ u_sample,
    int D, int V, int chunks, float tau, const DrawInfo* __restrict__ info,
    const double2* __restrict__ sums, int32_t* __restrict__ out_tokens) {
  constexpr int kThreads = kArgmaxThreads;
  constexpr int kPer = kArgmaxChunk / kThreads;      // 16 logits per thread
  constexpr int kStagedChunks = 1024;              // vocabularies up to 4M logits
  __shared__ double2 s_sums[kStagedChunks];
  __shared__ double s_own[kThreads], s_part[kThreads];
  __shared__ double s_off;
  __shared__ int s_chunk, s_tok, s_resid, s_sel;
  const int b = blockIdx.x;
  const int R = D + 1;
  const int t = threadIdx.x;
  DrawInfo di = info[b];
  // the chunk sums, staged in LDS by all threads (one global round trip),
  // then summed by thread 0 in chunk order
  const double2* sb = sums + (size_t)b * chunks;
  const bool staged = chunks <= kStagedChunks;
  if (staged)
    for (int c = t; c < chunks; c += kThreads) s_sums[c] = sb[c];
  __syncthreads();
  auto chunk_sum = [&](int c) -> double2 { return staged ? s_sums[c] : sb[c]; };
  if (t == 0) {
    double tot_w = 0.0;
    for (int c = 0; c < chunks; ++c) tot_w += chunk_sum(c).x;
    const bool use_w = !(di.resid && tot_w == 0.0);   // p_n == q_n: draw from p_n
    double total = 0.0;
    for (int c = 0; c < chunks; ++c) total += use_w ? chunk_sum(c).x : chunk_sum(c).y;
    const double T = (double)u_sample[b] * total;
    double run = 0.0;
    int pick = -1, last = 0;
    double off = 0.0, last_off = 0.0;
    for (int c = 0; c < chunks; ++c) {
      const double w = use_w ? chunk_sum(c).x : chunk_sum(c).y;
      if (w > 0.0) {
        last = c;
        last_off = run;
        if (T < run + w) {
          pick = c;
          off = run;
          break;
        }
      }
      run += w;
    }
    s_chunk = pick >= 0 ? pick : last;
    s_off = T - (pick >= 0 ? off : last_off);          // target inside the chunk
    s_resid = use_w ? di.resid : 0;
    s_tok = -1;
  }
  __syncthreads();
  di.resid = s_resid;
  const int chunk = s_chunk;
  const double Tc = s_off;
  const float* zr = zt + ((size_t)b * R + di.n) * V;
  const float* yr = di.resid ? zd + ((size_t)b * D + di.n) * V : zr;
  const int v0 = min(chunk * kArgmaxChunk + t * kPer, V), v1 = min(v0 + kPer, V);
  // this thread's logits, loaded together (16-byte vectors where the row
  // allows; -inf past its end), and their weights, kept for the walk below
  float zv[kPer], yv[kPer];
  if (V % 4 == 0 && v1 - v0 == kPer) {
#pragma unroll
    for (int k = 0; k < kPer; k += 4) {
      const f32x4 a4 = *reinterpret_cast<const f32x4*>(zr + v0 + k);
      const f32x4 b4 = *reinterpret_cast<const f32x4*>(yr + v0 + k);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        zv[k + e] = a4[e];
        yv[k + e] = b4[e];
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      zv[k] = v0 + k < v1 ? zr[v0 + k] : -INFINITY;
      yv[k] = v0 + k < v1 ? yr[v0 + k] : -INFINITY;
    }
  }
  double wv[kPer];
  double own = 0.0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    wv[k] = zv[k] == -INFINITY ? 0.0
                               : (di.resid ? weight_r(zv[k], yv[k], di, tau) : weight_p(zv[k], di, tau));
    own += wv[k];
  }
  s_own[t] = own;
  __syncthreads();
  if (t == 0) {
    // exclusive prefix in thread order; the first segment with weight whose end
    // passes Tc holds it (else the last segment with weight)
    double run = 0.0;
    int sel = -1, last = -1;
    for (int i = 0; i < kThreads; ++i) {
      const double x = s_own[i];
      s_part[i] = run;
      if (x > 0.0) {
        last = i;
        if (sel < 0 && Tc < run + x) sel = i;
      }
      run += x;
    }
    s_sel = sel >= 0 ? sel : last;
  }
  __syncthreads();
  if (t == s_sel) {
    double run = s_part[t];
    int tok = -1, last = -1;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      if (v0 + k >= v1) break;
      const double w = wv[k];
      if (w > 0.0) last = v0 + k;
      run += w;
      if (run > Tc) {
        tok = v0 + k;
        break;
      }
    }
    s_tok = tok >= 0 ? tok : last;
  }
  __syncthreads();
  if (t == 0) out_tokens[(size_t)b * R + di.n] = s_tok >= 0 ? s_tok : chunk * kArgmaxChunk;
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
  // tau == 1: the exact division by tau is left out of the per-logit work
  const bool unit = tau == 1.f;
  if (V % 4 == 0 && unit)
    sv_sample_stats<true, true><<<grid, kArgmaxThreads, 0, stream>>>(zt, zd, B * R, V, chunks, tau, st);
  else if (V % 4 == 0)
    sv_sample_stats<true, false><<<grid, kArgmaxThreads, 0, stream>>>(zt, zd, B * R, V, chunks, tau, st);
  else if (unit)
    sv_sample_stats<false, true><<<grid, kArgmaxThreads, 0, stream>>>(zt, zd, B * R, V, chunks, tau, st);
  else
    sv_sample_stats<false, false><<<grid, kArgmaxThreads, 0, stream>>>(zt, zd, B * R, V, chunks, tau, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // workspace after the chunk statistics: DrawInfo[B], then {sum w, sum p}[B][chunks]
  const size_t st_bytes = (size_t)B * (R + D) * chunks * sizeof(SampleStat);
  auto* info = reinterpret_cast<DrawInfo*>(static_cast<char*>(ws) + st_bytes);
  auto* sums = reinterpret_cast<double2*>(static_cast<char*>(ws) + st_bytes + (size_t)B * sizeof(DrawInfo));
  sv_sample_keep<<<B, kKeepThreads, 0, stream>>>(zt, zd, draft, u_accept, D, V, chunks, tau, st,
                                                   info, accept_len, out_tokens, kv_in, kv_out);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid3(chunks, B);
  if (V % 4 == 0 && unit)
    sv_sample_chunk_sums<true, true><<<grid3, kArgmaxThreads, 0, stream>>>(zt, zd, D, V, chunks,
                                                                           tau, info, sums);
  else if (V % 4 == 0)
    sv_sample_chunk_sums<true, false><<<grid3, kArgmaxThreads, 0, stream>>>(zt, zd, D, V, chunks,
                                                                            tau, info, sums);
  else if (unit)
    sv_sample_chunk_sums<false, true><<<grid3, kArgmaxThreads, 0, stream>>>(zt, zd, D, V, chunks,
                                                                            tau, info, sums);
  else
    sv_sample_chunk_sums<false, false><<<grid3, kArgmaxThreads, 0, stream>>>(zt, zd, D, V, chunks,
                                                                             tau, info, sums);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  sv_sample_draw<<<B, kArgmaxThreads, 0, stream>>>(zt, zd, u_sample, D, V, chunks, tau, info, sums,
                                                   out_tokens);
  return hipGetLastError();
}

}  // namespace sv
