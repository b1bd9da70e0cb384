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

#include <mutex>

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

// (max, lowest index) over the chunk results p[0 .. chunks) of one row.  The
// loads go out sixteen at a time (past the end the last chunk is read again,
// which cannot change the result), so the reduction waits for one round trip
// per sixteen chunks rather than one per chunk.
__device__ __forceinline__ int reduce_parts(const ArgmaxPart* __restrict__ p, int chunks) {
  constexpr int kBatch = 16;
  float bv = -INFINITY;
  int bi = INT32_MAX;
  for (int c0 = 0; c0 < chunks; c0 += kBatch) {
    ArgmaxPart q[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) q[k] = p[min(c0 + k, chunks - 1)];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) consider(q[k].value, q[k].index, bv, bi);
  }
  return bi;
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
    tok = reduce_parts(part + ((size_t)b * R + j) * chunks, chunks);
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

// Draft-tree acceptance (nodes in topological order, parent[j] < j, node 0 the
// root = the last committed token).  grid = B; one wave per sequence; lane j holds tree
// node j (R <= 64): its row's argmax a_j, its parent and its token.  From the
// root, the walk steps to the lowest-indexed child c of the current node i with
// token[c] == a_i (one ballot per step) until no child matches.
__global__ __launch_bounds__(kWave) void sv_accept_tree_finalize(
    const ArgmaxPart* __restrict__ part, int chunks, int R, const int32_t* __restrict__ tokens,
    const int32_t* __restrict__ parents, int32_t* __restrict__ target,
    int32_t* __restrict__ accept_len, int32_t* __restrict__ out_tokens,
    int32_t* __restrict__ accept_path, const int32_t* kv_in, int32_t* kv_out) {
  const int b = blockIdx.x;
  const int j = threadIdx.x;
  int a = 0, par = -2, tok = -1;
  if (j < R) {
    a = reduce_parts(part + ((size_t)b * R + j) * chunks, chunks);
    target[(size_t)b * R + j] = a;
    if (j > 0) {
      par = parents[(size_t)b * R + j];
      tok = tokens[(size_t)b * R + j];
    }
  }
  // walk: at most R - 1 steps, the node index grows at each one
  int cur = 0, len = 1;
  unsigned long long path = 1ull;           // nodes on the path (node 0, the root)
  for (int step = 1; step < R; ++step) {
    const int a_cur = __shfl(a, cur);
    const unsigned long long m = __ballot(j < R && j > cur && par == cur && tok == a_cur);
    if (!m) break;
    cur = __ffsll((long long)m) - 1;
    path |= 1ull << cur;
    ++len;
  }
  const int a_last = __shfl(a, cur);
  // Path nodes grow with their place on the path, so a node's place is the
  // number of path nodes below it.  Every address below is written once.
  if (j < R) {
    const bool on_path = (path >> j) & 1ull;
    const int place = __popcll(path & ((1ull << j) - 1ull));
    if (on_path) {
      accept_path[(size_t)b * R + place] = j;
      if (place > 0) out_tokens[(size_t)b * R + place - 1] = tok;
    }
    if (j >= len) {
      accept_path[(size_t)b * R + j] = -1;
      out_tokens[(size_t)b * R + j] = -1;
    }
    if (j == len - 1) out_tokens[(size_t)b * R + j] = a_last;
  }
  if (j == 0) {
    accept_len[b] = len;
    kv_out[b] = kv_in[b] - R + len;
  }
}

hipError_t launch_accept_tree(int B, int R, int V, const float* logits, const int32_t* tokens,
                              const int32_t* parents, int32_t* target, int32_t* accept_len,
                              int32_t* out_tokens, int32_t* accept_path, const int32_t* kv_in,
                              int32_t* kv_out, void* ws, hipStream_t stream) {
  const int chunks = argmax_chunks(V);
  auto* part = static_cast<ArgmaxPart*>(ws);
  dim3 grid(chunks, B * R);
  if (V % 4 == 0)
    sv_argmax_partial<true><<<grid, kArgmaxThreads, 0, stream>>>(logits, V, chunks, part);
  else
    sv_argmax_partial<false><<<grid, kArgmaxThreads, 0, stream>>>(logits, V, chunks, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  sv_accept_tree_finalize<<<B, kWave, 0, stream>>>(part, chunks, R, tokens, parents, target,
                                                    accept_len, out_tokens, accept_path, kv_in,
                                                    kv_out);
  return hipGetLastError();
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

// ---------------------------------------------------------------------------
// Acceptance without a workspace argument (spec_accept_noalloc): the chunk
// results live in this fixed device array instead of a caller's workspace.
// Each GPU the library runs on holds its own copy until the process ends.  Its
// address on a device comes from hipGetSymbolAddress (in host code the array's
// name is only a stand-in, never a device address), taken once per device with
// that device current and kept.  Every call overwrites the entries it reads
// before reading them, so nothing needs clearing between calls.
// ---------------------------------------------------------------------------
static __device__ __attribute__((aligned(256))) unsigned char scratch[kAcceptScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};
}  // namespace

hipError_t accept_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return hipSuccess;
}

}  // namespace sv
