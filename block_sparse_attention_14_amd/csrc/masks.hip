// Kept-block masks without attention: the on-chip threshold router, and the
// top-k / top-p routers it is compared with (page "Sol-Attn: Accelerating
// Video Generation Inference via On-the-Fly Attention Sparsification",
// §2 "Block-Sparse Attention": top-k imposes a fixed budget, top-p a dynamic
// one, and both traverse the proxy scores; §3 "On-the-fly sparsification" and
// §4 "Efficient On-the-Fly Sparsification": threshold routing consumes the
// scores on chip instead of materialising and traversing the proxy map).
//
// The threshold router is the fused forward kernel stopped after its routing
// (api.hip): it consumes the scores on chip and writes only the kept-block
// bitmap. The top-k / top-p routers here first write the full proxy map
// (fp32 [BH][Nq][Nk]) to device memory, then read it back one row per
// workgroup, sort the row, and write the bitmap. All three produce the same
// bitmap layout as sol_attn_forward_debug.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace sol {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxMaskWords = (SOL_ATTN_MAX_N / kBlk + 31) / 32;  // bitmap words of the longest row

// ---------------------------------------------------------------------------
// top-k / top-p routers: the proxy map in device memory, then a sort per row
// ---------------------------------------------------------------------------

// map[bh][i][j] = qpool[bh][i] . kpool[bh][j] * scale, fp32. 64 x 64 output
// tile per workgroup, each thread 4 x 4 outputs, d in LDS chunks of 32.
template <int D>
__global__ __launch_bounds__(kThreads) void proxy_map_kernel(const float* __restrict__ qpool,
                                                             const float* __restrict__ kpool, float* __restrict__ map,
                                                             int Nq, int Nk, float scale) {
  constexpr int KC = 32;
  __shared__ float As[KC][64 + 4];
  __shared__ float Bs[KC][64 + 4];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int bh = blockIdx.z, i0 = blockIdx.y * 64, j0 = blockIdx.x * 64;
  const float* qp = qpool + (size_t)bh * Nq * D;
  const float* kp = kpool + (size_t)bh * Nk * D;
  float acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.f;
  // loader: 64 rows x 32 columns per operand, 8 floats per thread
  const int lr = tid >> 2, lc = (tid & 3) * 8;
  for (int c0 = 0; c0 < D; c0 += KC) {
    {
      const int i = i0 + lr, j = j0 + lr;
      float4 a0 = make_float4(0.f, 0.f, 0.f, 0.f), a1 = a0, b0 = a0, b1 = a0;
      if (i < Nq) {
        a0 = *reinterpret_cast<const float4*>(qp + (size_t)i * D + c0 + lc);
        a1 = *reinterpret_cast<const float4*>(qp + (size_t)i * D + c0 + lc + 4);
      }
      if (j < Nk) {
        b0 = *reinterpret_cast<const float4*>(kp + (size_t)j * D + c0 + lc);
        b1 = *reinterpret_cast<const float4*>(kp + (size_t)j * D + c0 + lc + 4);
      }
      const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
      const float bv[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        As[lc + e][lr] = av[e];
        Bs[lc + e][lr] = bv[e];
      }
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < KC; ++kk) {
      const float4 a = *reinterpret_cast<const float4*>(&As[kk][4 * ty]);
      const float4 b = *reinterpret_cast<const float4*>(&Bs[kk][4 * tx]);
      const float av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[r][c] += av[r] * bv[c];
    }
    __syncthreads();
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = i0 + 4 * ty + r;
    if (i >= Nq) continue;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int j = j0 + 4 * tx + c;
      if (j < Nk) map[((size_t)bh * Nq + i) * Nk + j] = acc[r][c] * scale;
    }
  }
}

// a goes before b: higher score first, equal scores by lower block index
__device__ __forceinline__ bool before(float ka, int ia, float kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
}

// One workgroup per row (query block): the row is sorted in LDS (bitonic
// network over the next power of two, padding last), then the kept prefix is
// chosen: the first `k` entries (top-k) or the shortest prefix whose share of
// the row's softmax mass reaches `p` (top-p).
__global__ __launch_bounds__(kThreads) void sort_mask_kernel(const float* __restrict__ map, uint32_t* __restrict__ bitmap,
                                                             int Nq, int Nk, int n2, int nwords, int topk, float topp,
                                                             int mode) {
  extern __shared__ __align__(16) unsigned char dyn[];
  float* key = reinterpret_cast<float*>(dyn);  // [n2]
  int* idx = reinterpret_cast<int*>(key + n2);  // [n2]
  __shared__ float part[kThreads];
  __shared__ int cut;
  __shared__ uint32_t bits[kMaxMaskWords];
  const int tid = threadIdx.x;
  const int row = blockIdx.x, bh = blockIdx.y;
  const float* s = map + ((size_t)bh * Nq + row) * Nk;
  for (int t = tid; t < n2; t += kThreads) {
    key[t] = t < Nk ? s[t] : -INFINITY;
    idx[t] = t;
  }
  for (int w = tid; w < nwords; w += kThreads) bits[w] = 0u;
  if (tid == 0) cut = n2;
  __syncthreads();
  for (int size = 2; size <= n2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = tid; t < n2 / 2; t += kThreads) {
        const int i = 2 * t - (t & (stride - 1));  // lower element of the t-th pair
        const int l = i + stride;
        const bool first = (i & size) == 0;       // this pair's run is ordered forwards
        const float ki = key[i], kl = key[l];
        const int ii = idx[i], il = idx[l];
        const bool ok = first ? before(ki, ii, kl, il) : before(kl, il, ki, ii);
        if (!ok) {
          key[i] = kl;
          key[l] = ki;
          idx[i] = il;
          idx[l] = ii;
        }
      }
      __syncthreads();
    }
  }
  int keep_n;
  if (mode == 0) {
    keep_n = min(max(topk, 0), Nk);
  } else {
    // shares of exp(s - s_max) in sorted order: thread t owns positions [t*C, (t+1)*C)
    const int C = n2 / kThreads > 0 ? n2 / kThreads : 1;
    const float top = key[0];
    float local = 0.f;
    for (int c = 0; c < C; ++c) {
      const int pos = tid * C + c;
      if (pos < Nk) local += __expf(key[pos] - top);
    }
    part[tid] = local;
    __syncthreads();
    for (int off = 1; off < kThreads; off <<= 1) {  // inclusive scan of the per-thread sums
      const float v = tid >= off ? part[tid - off] : 0.f;
      __syncthreads();
      part[tid] += v;
      __syncthreads();
    }
    const float total = part[kThreads - 1];
    const float goal = topp * total;
    float run = part[tid] - local;
    for (int c = 0; c < C; ++c) {
      const int pos = tid * C + c;
      if (pos < Nk) {
        run += __expf(key[pos] - top);
        if (run >= goal) {
          atomicMin(&cut, pos);
          break;
        }
      }
    }
    __syncthreads();
    keep_n = topp >= 1.f ? Nk : min(cut + 1, Nk);
  }
  for (int pos = tid; pos < keep_n; pos += kThreads) {
    const int j = idx[pos];
    atomicOr(&bits[j >> 5], 1u << (j & 31));
  }
  __syncthreads();
  uint32_t* out = bitmap + ((size_t)bh * Nq + row) * nwords;
  for (int w = tid; w < nwords; w += kThreads) out[w] = bits[w];
}

}  // namespace

hipError_t launch_proxy_map(const float* qpool, const float* kpool, float* map, int BH, int Nq, int Nk, int d,
                            float scale, hipStream_t stream) {
  const dim3 grid((Nk + 63) / 64, (Nq + 63) / 64, BH);
  if (d == 128)
    hipLaunchKernelGGL(proxy_map_kernel<128>, grid, dim3(kThreads), 0, stream, qpool, kpool, map, Nq, Nk, scale);
  else
    hipLaunchKernelGGL(proxy_map_kernel<64>, grid, dim3(kThreads), 0, stream, qpool, kpool, map, Nq, Nk, scale);
  return hipGetLastError();
}

hipError_t launch_sort_mask(const float* map, uint32_t* bitmap, int BH, int Nq, int Nk, int topk, float topp,
                            int mode, hipStream_t stream) {
  int n2 = 1;
  while (n2 < Nk) n2 <<= 1;
  if (n2 < 2 * kThreads) n2 = 2 * kThreads;  // at least one pair per thread
  const int nwords = (Nk + 31) / 32;
  const size_t dyn = (size_t)n2 * (sizeof(float) + sizeof(int));
  hipLaunchKernelGGL(sort_mask_kernel, dim3(Nq, BH), dim3(kThreads), dyn, stream, map, bitmap, Nq, Nk, n2, nwords,
                     topk, topp, mode);
  return hipGetLastError();
}

}  // namespace sol
