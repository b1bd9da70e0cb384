// Machine ceilings for the roofline figures (C header sv_ceilings.h): a
// streaming read, a bf16 matrix-core loop and a vector exponential loop, each a
// single kernel whose rate the caller times.
#include "sv_device.h"
#include "sv_internal.h"

namespace sv {

constexpr int kCeilThreads = 256;

// Every 16-byte vector of src read once, 16 KB at a time per workgroup:
// workgroup w takes the chunks w, w + gridDim.x, ..., each thread four
// vectors 4 KB apart inside a chunk (a wave reads 1 KB runs), all four in
// flight; vectors past the last whole chunk go round the grid one per thread.
// The words are folded with XOR (no float work) and one value per workgroup
// is stored so the loads stay.  (A grid-stride pattern whose four loads per
// thread lie a grid apart read ~12% slower on these GPUs.)
constexpr size_t kCeilChunk = 1024;         // 16-byte vectors per chunk

__global__ __launch_bounds__(kCeilThreads) void sv_ceil_read(const u32x4* __restrict__ src,
                                                             size_t n, float* __restrict__ sink) {
  const size_t chunks = n / kCeilChunk;
  uint32_t acc = 0;
  for (size_t c = blockIdx.x; c < chunks; c += gridDim.x) {
    const u32x4* p = src + c * kCeilChunk + threadIdx.x;
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(p + u * kCeilThreads);
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (size_t i = chunks * kCeilChunk + (size_t)blockIdx.x * kCeilThreads + threadIdx.x; i < n;
       i += (size_t)gridDim.x * kCeilThreads) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off);
  __shared__ uint32_t part[kCeilThreads / kWave];
  if (threadIdx.x % kWave == 0) part[threadIdx.x / kWave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
#pragma unroll
    for (int w = 0; w < kCeilThreads / kWave; ++w) r ^= part[w];
    sink[blockIdx.x] = __uint_as_float(r);
  }
}

// Four independent accumulators per wave, each advanced by one 32x32x16 bf16
// MFMA per iteration.  Operands come from the thread index so nothing folds.
__global__ __launch_bounds__(kCeilThreads) void sv_ceil_mfma(int iters, float* __restrict__ sink) {
  const float base = 1e-3f * (float)(threadIdx.x % kWave + 1);
  bf16x8 a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (__bf16)(base + 1e-4f * j);
    b[j] = (__bf16)(base - 1e-4f * j);
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = mfma32x32x16(a, b, c0);
    c1 = mfma32x32x16(b, a, c1);
    c2 = mfma32x32x16(a, a, c2);
    c3 = mfma32x32x16(b, b, c3);
  }
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) s += (c0[e] + c1[e]) + (c2[e] + c3[e]);
  if (threadIdx.x % kWave == 0) sink[blockIdx.x * (kCeilThreads / kWave) + threadIdx.x / kWave] = s;
}

// Eight independent chains x <- 2^(-x) per thread (values stay in [0.5, 1]).
__global__ __launch_bounds__(kCeilThreads) void sv_ceil_exp2(int iters, float* __restrict__ sink) {
  float x[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) x[k] = (float)(threadIdx.x % kWave) * (1.f / 64.f) + 0.01f * k;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = fast_exp2(-x[k]);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) s += x[k];
  sink[(size_t)blockIdx.x * kCeilThreads + threadIdx.x] = s;
}

hipError_t launch_ceiling_read(const void* src, size_t bytes, int wgs, float* sink,
                               hipStream_t stream) {
  sv_ceil_read<<<wgs, kCeilThreads, 0, stream>>>(static_cast<const u32x4*>(src), bytes / 16, sink);
  return hipGetLastError();
}

hipError_t launch_ceiling_mfma(int wgs, int iters, float* sink, hipStream_t stream) {
  sv_ceil_mfma<<<wgs, kCeilThreads, 0, stream>>>(iters, sink);
  return hipGetLastError();
}

hipError_t launch_ceiling_exp2(int wgs, int iters, float* sink, hipStream_t stream) {
  sv_ceil_exp2<<<wgs, kCeilThreads, 0, stream>>>(iters, sink);
  return hipGetLastError();
}

}  // namespace sv
