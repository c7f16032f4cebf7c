// Pooling pre-pass: per 64-token block, the fp32 mean of k and of v over the
// block's valid tokens (page "Sol-Attn: Accelerating Video Generation
// Inference via On-the-Fly Attention Sparsification", §2 "Block-Sparse
// Attention": mean-pooled blocks; §3 "Approximate correction": pooled keys and
// summed values, the latter being n_j times the mean stored here).
//
// One workgroup per (block j, head) and tensor (grid x = head * Nk + j, grid y
// = tensor). Each thread streams 16-byte chunks of rows, the partial sums meet
// in LDS, and thread c writes column c. The pass is a pure HBM stream: every
// input byte is read once. The forward pools k and v here; its pooled queries
// are summed inside the fused kernel from the Q tiles it loads anyway. The
// top-k / top-p mask builders pool q with this kernel.
#include "common.h"
#include "kernels.h"

namespace sol {

template <int D>
__global__ __launch_bounds__(256) void pool_kernel(PoolSet set, int N, int Nk, unsigned* hdr) {
  constexpr int CH = D / 8;      // 16-byte chunks per row
  constexpr int RPP = 256 / CH;  // rows covered per pass
  __shared__ float part[RPP][D];

  const int bh = blockIdx.x / Nk, j = blockIdx.x - bh * Nk, which = blockIdx.y;
  const int tid = threadIdx.x;
  const int c = tid % CH, r0 = tid / CH;
  const int nj = min(kBlk, N - j * kBlk);
  const uint16_t* src = set.src[which] + ((size_t)bh * N + (size_t)j * kBlk) * D;
  float* dst = set.dst[which] + ((size_t)bh * Nk + j) * D;

  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  // every row load of the block in flight before the first add
  constexpr int PASSES = kBlk / RPP;
  uint4 u[PASSES];
#pragma unroll
  for (int i = 0; i < PASSES; ++i) {
    const int r = r0 + i * RPP;
    u[i] = r < nj ? *reinterpret_cast<const uint4*>(src + (size_t)r * D + c * 8) : make_uint4(0u, 0u, 0u, 0u);
  }
#pragma unroll
  for (int i = 0; i < PASSES; ++i) {
    acc[0] += bf16lo(u[i].x); acc[1] += bf16hi(u[i].x);
    acc[2] += bf16lo(u[i].y); acc[3] += bf16hi(u[i].y);
    acc[4] += bf16lo(u[i].z); acc[5] += bf16hi(u[i].z);
    acc[6] += bf16lo(u[i].w); acc[7] += bf16hi(u[i].w);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[r0][c * 8 + e] = acc[e];
  __syncthreads();
  if (tid < D) {
    float s = 0.f;
#pragma unroll 8
    for (int r = 0; r < RPP; ++r) s += part[r][tid];
    dst[tid] = s / (float)nj;
  }

  if (hdr != nullptr && blockIdx.x == 0 && blockIdx.y == 0)
    for (int w = tid; w < kHdrWords; w += 256) hdr[w] = w == kHdrMin ? 0xffffffffu : 0u;
}

__global__ __launch_bounds__(256) void to_bf16_kernel(const float* __restrict__ a, uint16_t* __restrict__ a_hi,
                                                      uint16_t* __restrict__ a_lo, const float* __restrict__ b,
                                                      uint16_t* __restrict__ b16, size_t n) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) {
    const uint32_t hi = pack_bf16x2(a[i], 0.f) & 0xffffu;
    a_hi[i] = (uint16_t)hi;
    a_lo[i] = (uint16_t)(pack_bf16x2(a[i] - __uint_as_float(hi << 16), 0.f) & 0xffffu);
    b16[i] = (uint16_t)(pack_bf16x2(b[i], 0.f) & 0xffffu);
  }
}

hipError_t launch_to_bf16(const float* a, uint16_t* a_hi, uint16_t* a_lo, const float* b, uint16_t* b16, size_t n,
                          hipStream_t stream) {
  hipLaunchKernelGGL(to_bf16_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a, a_hi, a_lo, b, b16,
                     n);
  return hipGetLastError();
}

template <int D>
__global__ __launch_bounds__(256) void kstats_kernel(const float* __restrict__ kpool, float* __restrict__ stats, int Nk) {
  constexpr int G = 256 / D;  // row groups
  __shared__ float part[G][D];
  __shared__ float mean[D];
  const int tid = threadIdx.x, c = tid % D, rg = tid / D;
  const float* kp = kpool + (size_t)blockIdx.x * Nk * D;
  float s = 0.f;
  for (int j = rg; j < Nk; j += G) s += kp[(size_t)j * D + c];
  part[rg][c] = s;
  __syncthreads();
  if (tid < D) {
    float t = 0.f;
#pragma unroll
    for (int g = 0; g < G; ++g) t += part[g][tid];
    mean[tid] = t / (float)Nk;
  }
  __syncthreads();
  const float m = mean[c];
  float v = 0.f;
  for (int j = rg; j < Nk; j += G) {
    const float x = kp[(size_t)j * D + c] - m;
    v += x * x;
  }
  part[rg][c] = v;
  __syncthreads();
  if (tid < D) {
    float t = 0.f;
#pragma unroll
    for (int g = 0; g < G; ++g) t += part[g][tid];
    stats[(size_t)blockIdx.x * 2 * D + tid] = mean[tid];
    stats[(size_t)blockIdx.x * 2 * D + D + tid] = t / (float)Nk;
  }
}

hipError_t launch_kstats(const float* kpool, float* stats, int BH, int Nk, int d, hipStream_t stream) {
  if (d == 128)
    hipLaunchKernelGGL(kstats_kernel<128>, dim3(BH), dim3(256), 0, stream, kpool, stats, Nk);
  else
    hipLaunchKernelGGL(kstats_kernel<64>, dim3(BH), dim3(256), 0, stream, kpool, stats, Nk);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void reset_kernel(unsigned* hdr) {
  for (int w = threadIdx.x; w < kHdrWords; w += 256) hdr[w] = w == kHdrMin ? 0xffffffffu : 0u;
}

hipError_t launch_reset(unsigned* hdr, hipStream_t stream) {
  hipLaunchKernelGGL(reset_kernel, dim3(1), dim3(256), 0, stream, hdr);
  return hipGetLastError();
}

hipError_t launch_pool(const PoolSet& set, int BH, int N, int Nk, int d, unsigned* hdr, hipStream_t stream) {
  const dim3 grid((unsigned)(BH * Nk), (unsigned)set.n), block(256);
  if (d == 128)
    hipLaunchKernelGGL(pool_kernel<128>, grid, block, 0, stream, set, N, Nk, hdr);
  else
    hipLaunchKernelGGL(pool_kernel<64>, grid, block, 0, stream, set, N, Nk, hdr);
  return hipGetLastError();
}

}  // namespace sol
