// Draft-side signals and the next draft length, on gfx950.
//
// Two signals of the draft model's next-token distribution predict how many
// drafts the target will accept: its confidence (largest probability) and its
// entropy (SpecKV summary, arXiv 2605.02888, section "Technical core").  The
// next draft length is the D that maximises expected tokens per unit time,
//     f(D) = E(alpha, D) / (1 + rho D),   E(alpha, D) = sum_{i=0..D} alpha^i,
// with alpha = confidence: the expected-token formula of "GPU and LLM" ch. 5,
// section "Speculative decoding (2)", and the drafting cost rho D of the NVIDIA
// co-design summary, guideline 4.  With a group size G > 0, lengths above
// 128/G - 1 are allowed only when G (1 + D) fills whole 128-row tiles
// (guideline 3).  Ties go to the shorter draft.
//
// Pass 1 (sv_draft_stats) streams every row once: each workgroup reduces a chunk
// of 4096 logits to (m = max z, S = sum e^x, T = sum x e^x) with x = (z - m) / tau,
// the sums in fp64.  Pass 2 (sv_draft_decide, one wave per row) merges the
// chunks with the online-softmax rule -- for chunk maximum m_c below the row
// maximum M, d = (m_c - M) / tau, S += e^d S_c, T += e^d (T_c + d S_c) -- then
//     confidence = 1 / S,   entropy = ln S - T / S,
// and evaluates f(D) in fp64 from the stored fp32 confidence in a fixed order
// (a^(D+1) by repeated products, 1 + rho D as a rounded product then a sum, no
// fused operations), so the decision is reproducible from the returned value.
#include "sv_device.h"
#include "sv_internal.h"

namespace sv {

namespace {

struct DraftStat {
  float m;       // chunk maximum (-inf: nothing finite)
  float pad;
  double s;      // sum e^x
  double t;      // sum x e^x
  double pad2;
};

constexpr int kTileRows = 128;

// grid = (chunks, rows), 256 threads.  VEC: V % 4 == 0 (rows 16-byte aligned).
template <bool VEC>
__global__ __launch_bounds__(kArgmaxThreads) void sv_draft_stats(const float* __restrict__ z,
                                                                 int V, int chunks, float tau,
                                                                 DraftStat* __restrict__ st) {
  constexpr int U = kArgmaxChunk / kArgmaxThreads;   // logits per thread
  __shared__ float red_m[kArgmaxThreads / kWave];
  __shared__ double red_s[kArgmaxThreads / kWave], red_t[kArgmaxThreads / kWave];
  const int chunk = blockIdx.x;
  const int row = blockIdx.y;
  const float* x = z + (size_t)row * V;
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
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if (t % kWave == 0) red_m[t / kWave] = m;
  __syncthreads();
  m = red_m[0];
#pragma unroll
  for (int i = 1; i < kArgmaxThreads / kWave; ++i) m = fmaxf(m, red_m[i]);
  double s = 0.0, tt = 0.0;
  if (m != -INFINITY) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (v[u] == -INFINITY) continue;
      const float xv = (v[u] - m) / tau;
      const double e = (double)expf(xv);
      s += e;
      tt += e * (double)xv;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    s += __shfl_xor(s, off);
    tt += __shfl_xor(tt, off);
  }
  if (t % kWave == 0) {
    red_s[t / kWave] = s;
    red_t[t / kWave] = tt;
  }
  __syncthreads();
  if (t == 0) {
    double S = red_s[0], T = red_t[0];
#pragma unroll
    for (int i = 1; i < kArgmaxThreads / kWave; ++i) {
      S += red_s[i];
      T += red_t[i];
    }
    st[(size_t)row * chunks + chunk] = DraftStat{m, 0.f, S, T, 0.0};
  }
}

// The next draft length from the stored confidence (fp64, fixed order, no
// contraction into fused multiply-adds).
__device__ int choose_draft_len(float confidence, int max_draft_len, float rho, int G) {
#pragma clang fp contract(off)
  const double a = fmin((double)confidence, 1.0);
  const double r = (double)rho;
  int best = -1;
  double best_f = -1.0;
  double P = 1.0;
  for (int D = 0; D <= max_draft_len; ++D) {
    P = P * a;
    const int rows = G * (D + 1);
    if (G > 0 && rows > kTileRows && rows % kTileRows != 0) continue;
    const double E = (a == 1.0) ? (double)(D + 1) : (1.0 - P) / (1.0 - a);
    const double prod = r * (double)D;
    const double cost = 1.0 + prod;
    const double f = E / cost;
    if (f > best_f) {
      best = D;
      best_f = f;
    }
  }
  return best;
}

// grid = ceil(rows / 4), 4 waves; one wave per row.
__global__ __launch_bounds__(256) void sv_draft_decide(const DraftStat* __restrict__ st, int rows,
                                                       int chunks, float tau, int max_draft_len,
                                                       float rho, int G,
                                                       float* __restrict__ confidence,
                                                       float* __restrict__ entropy,
                                                       int32_t* __restrict__ next_len) {
  const int lane = threadIdx.x % kWave;
  const int row = blockIdx.x * 4 + threadIdx.x / kWave;
  if (row >= rows) return;                              // whole waves leave together
  const DraftStat* sr = st + (size_t)row * chunks;
  float M = -INFINITY;
  for (int c = lane; c < chunks; c += kWave) M = fmaxf(M, sr[c].m);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  double S = 0.0, T = 0.0;
  for (int c = lane; c < chunks; c += kWave) {
    const DraftStat x = sr[c];
    if (!(x.s > 0.0)) continue;
    const double d = (double)((x.m - M) / tau);
    const double w = exp(d);
    S += w * x.s;
    T += w * (x.t + d * x.s);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    S += __shfl_xor(S, off);
    T += __shfl_xor(T, off);
  }
  if (lane == 0) {
    const float c = (float)(1.0 / S);
    confidence[row] = c;
    entropy[row] = (float)(log(S) - T / S);
    if (next_len) next_len[row] = choose_draft_len(c, max_draft_len, rho, G);
  }
}

}  // namespace

size_t draft_signals_workspace_bytes(int rows, int V) {
  return (size_t)rows * (size_t)argmax_chunks(V) * sizeof(DraftStat);
}

hipError_t launch_draft_signals(int rows, int V, float tau, const float* logits,
                                float* confidence, float* entropy, int32_t* next_len,
                                int max_draft_len, float rho, int G, void* ws,
                                hipStream_t stream) {
  const int chunks = argmax_chunks(V);
  DraftStat* st = static_cast<DraftStat*>(ws);
  const dim3 grid1(chunks, rows);
  if (V % 4 == 0)
    sv_draft_stats<true><<<grid1, kArgmaxThreads, 0, stream>>>(logits, V, chunks, tau, st);
  else
    sv_draft_stats<false><<<grid1, kArgmaxThreads, 0, stream>>>(logits, V, chunks, tau, st);
  sv_draft_decide<<<(rows + 3) / 4, 256, 0, stream>>>(st, rows, chunks, tau, max_draft_len, rho, G,
                                                      confidence, entropy, next_len);
  return hipGetLastError();
}

}  // namespace sv
