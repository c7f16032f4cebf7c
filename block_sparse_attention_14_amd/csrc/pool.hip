// Pooling pre-pass: per 64-token block, the fp32 mean of k and of v over the
// block's valid tokens (page "Sol-Attn: Accelerating Video Generation
// Inference via On-the-Fly Attention Sparsification", §2 "Block-Sparse
// Attention": mean-pooled blocks; §3 "Approximate correction": pooled keys and
// summed values, the latter being n_j times the mean stored here).
//
// One workgroup per (block j, head) and tensor (grid x = head * Nk + j). Each thread streams 16-byte
// chunks of rows, the partial sums meet in LDS, and thread c writes column c.
// The pass is a pure HBM stream: every input byte is read once.
#include "common.h"
#include "kernels.h"

namespace sol {

template <int D>
__global__ __launch_bounds__(256) void pool_kernel(const uint16_t* __restrict__ k,
                                                   const uint16_t* __restrict__ v,
                                                   float* __restrict__ kpool,
                                                   float* __restrict__ vmean, int N, int Nk,
                                                   unsigned* queue, sol_attn_stats* stats) {
  constexpr int CH = D / 8;      // 16-byte chunks per row
  constexpr int RPP = 256 / CH;  // rows covered per pass
  __shared__ float part[RPP][D];

  const int bh = blockIdx.x / Nk, j = blockIdx.x - bh * Nk, which = blockIdx.y;
  const int tid = threadIdx.x;
  const int c = tid % CH, r0 = tid / CH;
  const int nj = min(kBlk, N - j * kBlk);
  const uint16_t* src = (which ? v : k) + ((size_t)bh * N + (size_t)j * kBlk) * D;
  float* dst = (which ? vmean : kpool) + ((size_t)bh * Nk + j) * D;

  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  for (int r = r0; r < nj; r += RPP) {
    const uint4 u = *reinterpret_cast<const uint4*>(src + (size_t)r * D + c * 8);
    acc[0] += bf16lo(u.x); acc[1] += bf16hi(u.x);
    acc[2] += bf16lo(u.y); acc[3] += bf16hi(u.y);
    acc[4] += bf16lo(u.z); acc[5] += bf16hi(u.z);
    acc[6] += bf16lo(u.w); acc[7] += bf16hi(u.w);
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

  if (queue != nullptr && j == 0 && bh == 0 && which == 0 && tid == 0) {
    queue[kQueueTicket] = 0u;
    if (stats != nullptr) {
      stats->kept_blocks = 0ull;
      stats->total_blocks = 0ull;
      stats->kept_pairs = 0ull;
      stats->min_kept = 0xffffffffu;
      stats->max_kept = 0u;
    }
  }
}

__global__ void reset_kernel(unsigned* queue, sol_attn_stats* stats) {
  if (threadIdx.x == 0) {
    queue[kQueueTicket] = 0u;
    if (stats != nullptr) {
      stats->kept_blocks = 0ull;
      stats->total_blocks = 0ull;
      stats->kept_pairs = 0ull;
      stats->min_kept = 0xffffffffu;
      stats->max_kept = 0u;
    }
  }
}

hipError_t launch_pool(const uint16_t* k, const uint16_t* v, float* kpool, float* vmean, int BH,
                       int N, int Nk, int d, unsigned* queue, sol_attn_stats* stats,
                       hipStream_t stream) {
  const dim3 grid((unsigned)(BH * Nk), 2), block(256);
  if (d == 128)
    hipLaunchKernelGGL(pool_kernel<128>, grid, block, 0, stream, k, v, kpool, vmean, N, Nk, queue, stats);
  else
    hipLaunchKernelGGL(pool_kernel<64>, grid, block, 0, stream, k, v, kpool, vmean, N, Nk, queue, stats);
  return hipGetLastError();
}

hipError_t launch_reset(unsigned* queue, sol_attn_stats* stats, hipStream_t stream) {
  hipLaunchKernelGGL(reset_kernel, dim3(1), dim3(64), 0, stream, queue, stats);
  return hipGetLastError();
}

}  // namespace sol
