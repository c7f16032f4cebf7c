// Pooling pre-pass: per 64-token block, the fp32 mean of q, k and v over the
// block's valid tokens (page "Sol-Attn: Accelerating Video Generation
// Inference via On-the-Fly Attention Sparsification", §2 "Block-Sparse
// Attention": mean-pooled blocks; §3 "Approximate correction": pooled keys and
// summed values, the latter being n_j times the mean stored here), and the
// bf16 operand planes the fused kernel's routing pass reads.
//
// One workgroup per four consecutive blocks of one head and one tensor (see
// pool_kernel below). The pass is a pure HBM stream: every input byte is read
// once.
#include "common.h"
#include "kernels.h"

namespace sol {

// The routing planes (Planes in kernels.h): 16-block tiles stored in the
// order the matrix cores take their operands, so that one 64-lane load of the
// fused kernel reads one contiguous stretch:
//   kh, km, kl [BH][Nkp / 16][D / 8][16][8]: k = kh + km + kl + r, each part
//     rounded to nearest even from the remainder of the parts before it
//     (|r| <= 2^-24 |k| or so), so bf16 products of the parts carry an
//     fp32-grade score; element (j, c) of a head sits in tile j / 16 at
//     8-column chunk c / 8, row j % 16, position c % 8;
//   vt [BH][Nkp / 16][D / 16][4][16][4]: the pooled values in bf16, element
//     (j, c) in tile j / 16 at column tile c / 16, key quarter (j % 16) / 4,
//     column c % 16, position j % 4;
//   vrow [BH][Nk][D] (optional): bf16 pooled values, row-major (per-row
//     correction).
// A workgroup covers four consecutive key blocks, so that a key part's eight
// columns c .. c + 7 of one block and a value column's four blocks j .. j + 3
// are each one contiguous store. Rows Nk .. Nkp - 1 are zero: the fused
// kernel reads them as padding of the last tile.
__device__ __forceinline__ void key_parts(float x, uint16_t& h, uint16_t& m, uint16_t& l) {
  const uint32_t hh = pack_bf16x2(x, 0.f) & 0xffffu;
  const float r1 = x - __uint_as_float(hh << 16);
  const uint32_t mm = pack_bf16x2(r1, 0.f) & 0xffffu;
  const float r2 = r1 - __uint_as_float(mm << 16);
  h = (uint16_t)hh;
  m = (uint16_t)mm;
  l = (uint16_t)(pack_bf16x2(r2, 0.f) & 0xffffu);
}

// Element offsets in the planes of one head: key block jj, column c (a
// multiple of 8 starts eight contiguous columns), and value block jj (a
// multiple of 4 starts four contiguous blocks), column c.
template <int D>
__device__ __forceinline__ size_t key_off(int jj, int c) {
  constexpr int CH = D / 8;
  return ((size_t)((jj >> 4) * CH + (c >> 3)) * 16 + (jj & 15)) * 8 + (c & 7);
}
template <int D>
__device__ __forceinline__ size_t val_off(int jj, int c) {
  constexpr int CT = D / 16;
  return ((size_t)(((jj >> 4) * CT + (c >> 4)) * 4 + ((jj & 15) >> 2)) * 16 + (c & 15)) * 4 + (jj & 3);
}

constexpr int kPoolBlocks = 4;  // key blocks per workgroup of the pooling pass

// One workgroup per four consecutive 64-token blocks of one head and one
// tensor (grid x = head * ngrp + block group, grid y = tensor). Thread t
// streams the 16-byte chunk t % (D / 8) of its rows of all four blocks (every
// load in flight before the first add; rows past the sequence read as zero);
// the partial sums of a column meet across the lanes of a wave (DPP and
// permlane swaps) and across the waves in LDS. The pass is a pure HBM stream:
// every input byte is read once. A workgroup whose tensor has a plane role
// also writes its blocks' entries of the routing planes, from its own means
// or from the caller's pooled keys and values.
template <int D>
__global__ __launch_bounds__(256) void pool_kernel(PoolSet set, int N, int Nk, int ngrp, unsigned* hdr) {
  constexpr int CH = D / 8;      // 16-byte chunks per row
  constexpr int RPP = 256 / CH;  // rows covered per pass of the workgroup
  constexpr int PASSES = kBlk / RPP;
  constexpr int NB = kPoolBlocks;
  __shared__ float part[4][NB][D];  // per wave
  __shared__ float mean[NB][D];

  const int bh = blockIdx.x / ngrp, jg = blockIdx.x - bh * ngrp, which = blockIdx.y;
  const int j0 = NB * jg;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int c = tid % CH, r0 = tid / CH;
  const int rows = min(NB * kBlk, N - j0 * kBlk);  // valid tokens of the group
  const rsrc_t rs = make_rsrc(set.src[which] + ((size_t)bh * N + (size_t)j0 * kBlk) * D, (uint32_t)rows * D * 2);

  uint4 u[NB][PASSES];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int i = 0; i < PASSES; ++i) u[b][i] = ld16(rs, ((b * kBlk + r0 + i * RPP) * D + c * 8) * 2, 0);
  float acc[NB][8];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[b][e] = 0.f;
#pragma unroll
    for (int i = 0; i < PASSES; ++i) {
      acc[b][0] += bf16lo(u[b][i].x); acc[b][1] += bf16hi(u[b][i].x);
      acc[b][2] += bf16lo(u[b][i].y); acc[b][3] += bf16hi(u[b][i].y);
      acc[b][4] += bf16lo(u[b][i].z); acc[b][5] += bf16hi(u[b][i].z);
      acc[b][6] += bf16lo(u[b][i].w); acc[b][7] += bf16hi(u[b][i].w);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[b][e] = colsum_rows<CH>(acc[b][e]);
  }
  if (lane < CH)
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int e = 0; e < 8; ++e) part[wid][b][c * 8 + e] = acc[b][e];
  __syncthreads();
  float* dst = set.dst[which];
  for (int idx = tid; idx < NB * D; idx += 256) {
    const int b = idx / D, col = idx % D, jj = j0 + b;
    float m = 0.f;
    if (jj < Nk) {
      const float sum = (part[0][b][col] + part[1][b][col]) + (part[2][b][col] + part[3][b][col]);
      m = sum / (float)min(kBlk, N - jj * kBlk);
      dst[((size_t)bh * Nk + jj) * D + col] = m;
    }
    mean[b][col] = m;
  }

  const int role = set.role[which];
  if (role != 0) {
    __syncthreads();  // the means are in LDS
    const Planes& pl = set.planes;
    const size_t base = (size_t)bh * pl.Nkp * D;
    const int z0 = NB * ngrp;  // first padding row not covered by a workgroup's own blocks
    if (role & (kRoleKeys | kRoleKeysFromPool)) {
      if (tid < NB * CH) {
        const int b = tid / CH, c8 = 8 * (tid % CH), jj = j0 + b;
        float x[8];
        if (jj >= Nk) {
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = 0.f;
        } else if (role & kRoleKeys) {
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = mean[b][c8 + e];
        } else {
          const float4* kp = reinterpret_cast<const float4*>(pl.kpool + ((size_t)bh * Nk + jj) * D + c8);
          const float4 a = kp[0], a2 = kp[1];
          x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
          x[4] = a2.x; x[5] = a2.y; x[6] = a2.z; x[7] = a2.w;
        }
        uint32_t wh[4], wm[4], wl[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          uint16_t h0, m0, l0, h1, m1, l1;
          key_parts(x[e], h0, m0, l0);
          key_parts(x[e + 1], h1, m1, l1);
          wh[e / 2] = (uint32_t)h0 | ((uint32_t)h1 << 16);
          wm[e / 2] = (uint32_t)m0 | ((uint32_t)m1 << 16);
          wl[e / 2] = (uint32_t)l0 | ((uint32_t)l1 << 16);
        }
        const size_t o = base + key_off<D>(jj, c8);
        *reinterpret_cast<uint4*>(pl.kh + o) = make_uint4(wh[0], wh[1], wh[2], wh[3]);
        *reinterpret_cast<uint4*>(pl.km + o) = make_uint4(wm[0], wm[1], wm[2], wm[3]);
        *reinterpret_cast<uint4*>(pl.kl + o) = make_uint4(wl[0], wl[1], wl[2], wl[3]);
      }
      if (jg == ngrp - 1)
        for (int idx = tid; idx < (pl.Nkp - z0) * CH; idx += 256) {
          const size_t o = base + key_off<D>(z0 + idx / CH, 8 * (idx % CH));
          *reinterpret_cast<uint4*>(pl.kh + o) = make_uint4(0u, 0u, 0u, 0u);
          *reinterpret_cast<uint4*>(pl.km + o) = make_uint4(0u, 0u, 0u, 0u);
          *reinterpret_cast<uint4*>(pl.kl + o) = make_uint4(0u, 0u, 0u, 0u);
        }
    }
    if ((role & (kRoleValues | kRoleValuesFromPool)) && pl.vt) {
      if (tid < D) {
        float x[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const int jj = j0 + b;
          x[b] = jj >= Nk ? 0.f : (role & kRoleValues) ? mean[b][tid] : pl.vmean[((size_t)bh * Nk + jj) * D + tid];
        }
        *reinterpret_cast<uint2*>(pl.vt + base + val_off<D>(j0, tid)) =
            make_uint2(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]));
        if (pl.vrow)
#pragma unroll
          for (int b = 0; b < NB; ++b)
            if (j0 + b < Nk) pl.vrow[((size_t)bh * Nk + j0 + b) * D + tid] = (uint16_t)(pack_bf16x2(x[b], 0.f) & 0xffffu);
      }
      if (jg == ngrp - 1)
        for (int idx = tid; idx < (pl.Nkp - z0) / NB * D; idx += 256)
          *reinterpret_cast<uint2*>(pl.vt + base + val_off<D>(z0 + NB * (idx / D), idx % D)) = make_uint2(0u, 0u);
    }
  }

  if (hdr != nullptr && blockIdx.x == 0 && blockIdx.y == 0)
    for (int w = tid; w < kHdrWords; w += 256) hdr[w] = w == kHdrMin ? 0xffffffffu : 0u;
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

// Pooled-key moments of one head for the Gaussian threshold (page "Sol-Attn:
// Accelerating Video Generation Inference via On-the-Fly Attention
// Sparsification", §3 "Dynamic threshold routing" and App. B "Threshold
// variance derivation": the mean and variance of a proxy row follow from the
// first and second moments of the pooled keys, O(d^2) per head). Grid
// (BH, D / 16): every workgroup forms the mean m (two-level sum over the key
// blocks), then its 16 rows a of the population covariance
// C[a][b] = mean_j (k_ja - m_a)(k_jb - m_b); thread (b, r) accumulates rows
// a0 + r, a0 + r + R, ... of column b.
template <int D>
__global__ __launch_bounds__(256) void kmom_kernel(const float* __restrict__ kpool, float* __restrict__ mom, int Nk) {
  constexpr int P = 256 / D;       // key-block phases of the mean, rows per column group
  constexpr int RPT = 16 / P;      // covariance rows per thread
  __shared__ float part[P][D];
  __shared__ float mean[D];
  const int tid = threadIdx.x, b = tid % D, ph = tid / D;
  const float* kp = kpool + (size_t)blockIdx.x * Nk * D;
  float s = 0.f;
  for (int j = ph; j < Nk; j += P) s += kp[(size_t)j * D + b];
  part[ph][b] = s;
  __syncthreads();
  if (tid < D) {
    float t = 0.f;
#pragma unroll
    for (int q = 0; q < P; ++q) t += part[q][tid];
    mean[tid] = t / (float)Nk;
  }
  __syncthreads();
  const int a0 = 16 * blockIdx.y + ph;  // rows a0 + P r, r = 0 .. RPT - 1
  float acc[RPT];
#pragma unroll
  for (int r = 0; r < RPT; ++r) acc[r] = 0.f;
  const float mb = mean[b];
  float ma[RPT];
#pragma unroll
  for (int r = 0; r < RPT; ++r) ma[r] = mean[a0 + P * r];
  for (int j = 0; j < Nk; ++j) {
    const float* row = kp + (size_t)j * D;
    const float xb = row[b] - mb;
#pragma unroll
    for (int r = 0; r < RPT; ++r) acc[r] += (row[a0 + P * r] - ma[r]) * xb;
  }
  float* out = mom + (size_t)blockIdx.x * (D + 1) * D;
  if (blockIdx.y == 0 && tid < D) out[tid] = mean[tid];
#pragma unroll
  for (int r = 0; r < RPT; ++r) out[(size_t)(1 + a0 + P * r) * D + b] = acc[r] / (float)Nk;
}

hipError_t launch_kmom(const float* kpool, float* mom, int BH, int Nk, int d, hipStream_t stream) {
  if (d == 128)
    hipLaunchKernelGGL(kmom_kernel<128>, dim3(BH, 128 / 16), dim3(256), 0, stream, kpool, mom, Nk);
  else
    hipLaunchKernelGGL(kmom_kernel<64>, dim3(BH, 64 / 16), dim3(256), 0, stream, kpool, mom, Nk);
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
  const int ngrp = (Nk + kPoolBlocks - 1) / kPoolBlocks;
  const dim3 grid((unsigned)(BH * ngrp), (unsigned)set.n), block(256);
  if (d == 128)
    hipLaunchKernelGGL(pool_kernel<128>, grid, block, 0, stream, set, N, Nk, ngrp, hdr);
  else
    hipLaunchKernelGGL(pool_kernel<64>, grid, block, 0, stream, set, N, Nk, ngrp, hdr);
  return hipGetLastError();
}

}  // namespace sol
