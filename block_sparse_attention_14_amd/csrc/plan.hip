// Work ordering for the fused kernel: outliers first.
//
// The per-query-block budgets of threshold routing vary by two orders of
// magnitude (page "Sol-Attn: Accelerating Video Generation Inference via
// On-the-Fly Attention Sparsification", §1 and §3 "Dynamic threshold
// routing": dynamic, query-dependent budgets). A persistent grid that takes
// items in sequence order ends with a few workgroups finishing the heaviest
// items while the rest idle. These two small kernels estimate every item's
// cost (the size of the union of its two blocks' kept lists) and move the
// outliers of each XCD queue to its front, longest first, so the heavy items
// start early while the rest keep their head-major order.
//
// The estimate uses bf16 MFMA products of the pooled queries and keys: it
// only orders work. The fused kernel routes every item itself, in fp32, and
// nothing here influences which blocks it keeps. Only one count per item is
// written to device memory; no proxy scores or block indices are.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace sol {

namespace {

// Score tiles a wave keeps in registers between the max pass and the count
// pass; tiles beyond these are recomputed in the count pass.
constexpr int kCached = 8;
constexpr int kBatch = 4;  // tiles whose loads are in flight together

// Loads (pass 1) of one 16x16 S^T tile of pooled vectors: lane (g, c16)
// fetches pooled key jt0 + c16, columns 32 ds + 8 g .. +7 (zero past Nk).
template <int D>
__device__ __forceinline__ void tile_load(const float* kp, int Nk, int jt0, int c16, int g, float4 (&x)[D / 16]) {
  const int j = jt0 + c16;
#pragma unroll
  for (int ds = 0; ds < D / 32; ++ds) {
    if (j < Nk) {
      const float4* row = reinterpret_cast<const float4*>(kp + (size_t)j * D + 32 * ds + 8 * g);
      x[2 * ds] = row[0];
      x[2 * ds + 1] = row[1];
    } else {
      x[2 * ds] = x[2 * ds + 1] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
}

// S^T tile = K̄ Q̄^T in bf16 MFMA from the loaded pooled keys.
template <int D>
__device__ __forceinline__ f32x4 tile_mma(const float4 (&x)[D / 16], const bf16x8 (&qop)[D / 32]) {
  f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ds = 0; ds < D / 32; ++ds) {
    const float4 a = x[2 * ds], b = x[2 * ds + 1];
    const uint4 u = make_uint4(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w), pack_bf16x2(b.x, b.y),
                               pack_bf16x2(b.z, b.w));
    s = mfma16x16x32(as_bf16x8(u), qop[ds], s);
  }
  return s;
}

// grid (ceil(Nq / 16), BH), 256 threads. All four waves serve the same 16
// query blocks (lane column c16); wave w takes key tiles w, w + 4, ...
// Pass 1 finds each block's maximum, pass 2 counts, per pair of blocks, the
// key blocks that either block keeps. Both reductions meet in LDS.
template <int D>
__global__ __launch_bounds__(256) void plan_kernel(const float* __restrict__ qpool, const float* __restrict__ kpool,
                                                   unsigned* __restrict__ cost, int Nq, int Nk, float tau,
                                                   float proxy_scale) {
  __shared__ float red[4][16];
  __shared__ unsigned cred[4][16];
  const int bh = blockIdx.y;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int q = 16 * blockIdx.x + c16;  // this lane's query block (column of S^T)
  const float* kp = kpool + (size_t)bh * Nk * D;

  bf16x8 qop[D / 32];
#pragma unroll
  for (int ds = 0; ds < D / 32; ++ds) {
    float4 x0 = make_float4(0.f, 0.f, 0.f, 0.f), x1 = x0;
    if (q < Nq) {
      const float4* row = reinterpret_cast<const float4*>(qpool + ((size_t)bh * Nq + q) * D + 32 * ds + 8 * g);
      x0 = row[0];
      x1 = row[1];
    }
    qop[ds] = as_bf16x8(make_uint4(pack_bf16x2(x0.x, x0.y), pack_bf16x2(x0.z, x0.w), pack_bf16x2(x1.x, x1.y),
                                   pack_bf16x2(x1.z, x1.w)));
  }
  const int njt = (Nk + 15) / 16;
  auto valid = [&](int jt, int i) { return 16 * jt + 4 * g + i < Nk; };

  // pass 1: maxima; the first kCached tiles of this wave stay in registers
  float mx = -INFINITY;
  f32x4 sc[kCached];
#pragma unroll
  for (int c0 = 0; c0 < kCached; c0 += kBatch) {
    float4 x[kBatch][D / 16];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) tile_load<D>(kp, Nk, 16 * (wid + 4 * (c0 + u)), c16, g, x[u]);
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int jt = wid + 4 * (c0 + u);
      sc[c0 + u] = tile_mma<D>(x[u], qop);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (jt < njt && valid(jt, i)) mx = fmaxf(mx, sc[c0 + u][i]);
    }
  }
  for (int jt = wid + 4 * kCached; jt < njt; jt += 4) {
    float4 x[D / 16];
    tile_load<D>(kp, Nk, 16 * jt, c16, g, x);
    const f32x4 s = tile_mma<D>(x, qop);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (valid(jt, i)) mx = fmaxf(mx, s[i]);
  }
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  if (g == 0) red[wid][c16] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0][c16], red[1][c16]), fmaxf(red[2][c16], red[3][c16]));
  const float thr = mx * proxy_scale - tau;

  // pass 2: size of the union of the kept sets of blocks c16 and c16 ^ 1
  unsigned cnt = 0;
  auto count = [&](const f32x4& s, int jt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool keep = q < Nq && jt < njt && valid(jt, i) && s[i] * proxy_scale >= thr;
      const bool other = __shfl_xor((int)keep, 1) != 0;
      cnt += (keep || other) ? 1u : 0u;
    }
  };
#pragma unroll
  for (int c = 0; c < kCached; ++c) count(sc[c], wid + 4 * c);
  for (int jt = wid + 4 * kCached; jt < njt; jt += 4) {
    float4 x[D / 16];
    tile_load<D>(kp, Nk, 16 * jt, c16, g, x);
    count(tile_mma<D>(x, qop), jt);
  }
  cnt += __shfl_xor(cnt, 16);
  cnt += __shfl_xor(cnt, 32);
  if (g == 0) cred[wid][c16] = cnt;
  __syncthreads();
  const int npairs = (Nq + 1) / 2;
  if (wid == 0 && g == 0 && (c16 & 1) == 0 && q < Nq)
    cost[(size_t)bh * npairs + q / 2] = cred[0][c16] + cred[1][c16] + cred[2][c16] + cred[3][c16];
}

// One workgroup per queue. Items whose cost exceeds twice the queue's mean
// go first, by decreasing cost (a counting sort; equal costs in no particular
// order); all other items follow in their natural, head-major order. Taking
// only the outliers out of sequence starts them early enough to keep them off
// the end of the queue, while neighbouring query blocks, whose kept key
// blocks overlap, still run side by side and share those tiles in L2.
__global__ __launch_bounds__(1024) void order_kernel(const unsigned* __restrict__ cost, unsigned* __restrict__ perm,
                                                     int nitems, int Nk) {
  extern __shared__ unsigned hist[];  // [Nk + 1] counts of the outliers, then running offsets
  __shared__ unsigned part[1024];
  __shared__ unsigned long long wsum[16];
  __shared__ unsigned nheavy;
  const int tid = threadIdx.x, nt = blockDim.x;
  const int lo = queue_begin(blockIdx.x, nitems), hi = queue_begin(blockIdx.x + 1, nitems), n = hi - lo;

  // total cost of the queue
  unsigned long long sum = 0;
  for (int i = lo + tid; i < hi; i += nt) sum += cost[i];
  for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
  if ((tid & 63) == 0) wsum[tid >> 6] = sum;
  for (int b = tid; b <= Nk; b += nt) hist[b] = 0u;
  __syncthreads();
  unsigned long long total = 0;
  for (int w = 0; w < nt / 64; ++w) total += wsum[w];
  auto heavy = [&](unsigned c) { return (unsigned long long)c * (unsigned long long)n > 2ull * total; };

  for (int i = lo + tid; i < hi; i += nt) {
    const unsigned c = min(cost[i], (unsigned)Nk);
    if (heavy(c)) atomicAdd(&hist[c], 1u);
  }
  __syncthreads();
  // exclusive offsets with the highest cost first: position p is bucket Nk - p;
  // thread t owns positions [t*C, (t+1)*C)
  const int C = (Nk + 1 + nt - 1) / nt;
  unsigned local = 0;
  for (int k = 0; k < C; ++k) {
    const int pos = tid * C + k;
    if (pos <= Nk) local += hist[Nk - pos];
  }
  part[tid] = local;
  __syncthreads();
  for (int off = 1; off < nt; off <<= 1) {  // inclusive scan of the per-thread sums
    const unsigned v = tid >= off ? part[tid - off] : 0u;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  if (tid == nt - 1) nheavy = part[tid];
  unsigned run = (unsigned)lo + part[tid] - local;  // exclusive, offset to the queue's range
  for (int k = 0; k < C; ++k) {
    const int pos = tid * C + k;
    if (pos <= Nk) {
      const unsigned c = hist[Nk - pos];
      hist[Nk - pos] = run;
      run += c;
    }
  }
  __syncthreads();
  for (int i = lo + tid; i < hi; i += nt) {
    const unsigned c = min(cost[i], (unsigned)Nk);
    if (heavy(c)) perm[atomicAdd(&hist[c], 1u)] = (unsigned)i;
  }

  // the rest in natural order: thread t owns items [lo + t*CI, lo + (t+1)*CI)
  const int CI = (n + nt - 1) / nt;
  const int i0 = lo + tid * CI, i1 = min(hi, i0 + CI);
  unsigned light = 0;
  for (int i = i0; i < i1; ++i) light += heavy(min(cost[i], (unsigned)Nk)) ? 0u : 1u;
  __syncthreads();  // every reader of part is done
  part[tid] = light;
  __syncthreads();
  for (int off = 1; off < nt; off <<= 1) {
    const unsigned v = tid >= off ? part[tid - off] : 0u;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  unsigned dst = (unsigned)lo + nheavy + part[tid] - light;
  for (int i = i0; i < i1; ++i)
    if (!heavy(min(cost[i], (unsigned)Nk))) perm[dst++] = (unsigned)i;
}

__global__ __launch_bounds__(256) void iota_kernel(unsigned* __restrict__ perm, int nitems) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < nitems) perm[i] = (unsigned)i;
}

}  // namespace

hipError_t launch_identity_order(unsigned* perm, int nitems, hipStream_t stream) {
  hipLaunchKernelGGL(iota_kernel, dim3((nitems + 255) / 256), dim3(256), 0, stream, perm, nitems);
  return hipGetLastError();
}

hipError_t launch_plan(const float* qpool, const float* kpool, unsigned* cost, unsigned* perm, int BH, int Nq, int Nk,
                       int d, float tau, float proxy_scale, hipStream_t stream) {
  const dim3 grid((Nq + 15) / 16, BH);
  if (d == 128)
    hipLaunchKernelGGL(plan_kernel<128>, grid, dim3(256), 0, stream, qpool, kpool, cost, Nq, Nk, tau, proxy_scale);
  else
    hipLaunchKernelGGL(plan_kernel<64>, grid, dim3(256), 0, stream, qpool, kpool, cost, Nq, Nk, tau, proxy_scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nitems = forward_items(BH, Nq);
  hipLaunchKernelGGL(order_kernel, dim3(kQueues), dim3(1024), (size_t)(Nk + 1) * sizeof(unsigned), stream, cost,
                     perm, nitems, Nk);
  return hipGetLastError();
}

}  // namespace sol
