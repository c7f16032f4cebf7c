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

// bf16 operand planes of the fused kernel's routing pass, from the fp32
// pooled keys and values, for 64 key blocks per workgroup (grid (Nkp / 64, BH)).
// Both kinds are stored in 16-block tiles laid out in the order the matrix
// cores take their operands, so that one 64-lane load reads one contiguous
// stretch (512 or 1024 bytes) instead of 16-byte pieces of 16 rows:
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
// Key blocks from Nk to Nkp (a multiple of 64) are written as zeros. With vt
// null only the key planes are written.
template <int D>
__global__ __launch_bounds__(256) void prep_kernel(const float* __restrict__ kpool, const float* __restrict__ vmean,
                                                   uint16_t* __restrict__ kh, uint16_t* __restrict__ km,
                                                   uint16_t* __restrict__ kl, uint16_t* __restrict__ vt,
                                                   uint16_t* __restrict__ vrow, int Nk, int Nkp) {
  constexpr int CH = D / 8, CT = D / 16;
  __shared__ float ks[kBlk][D + 1];
  __shared__ float vs[kBlk][D + 1];
  const int bh = blockIdx.y, j0 = blockIdx.x * kBlk, tid = threadIdx.x;
  const size_t rowbase = (size_t)bh * Nk;
  for (int idx = tid; idx < kBlk * D; idx += 256) {
    const int jj = idx / D, c = idx % D, j = j0 + jj;
    float x = 0.f, v = 0.f;
    if (j < Nk) {
      x = kpool[(rowbase + j) * D + c];
      if (vmean) v = vmean[(rowbase + j) * D + c];
      if (vrow) vrow[(rowbase + j) * D + c] = (uint16_t)(pack_bf16x2(v, 0.f) & 0xffffu);
    }
    ks[jj][c] = x;
    vs[jj][c] = v;
  }
  __syncthreads();
  // this workgroup's 64 blocks are four whole tiles: a contiguous stretch of
  // every plane, written in storage order
  const size_t obase = ((size_t)bh * Nkp + j0) * D;
  for (int o = tid; o < kBlk * D; o += 256) {
    const int e8 = o % 8, r = (o / 8) % 16, cc = (o / 128) % CH, t = o / (128 * CH);
    const float x = ks[16 * t + r][8 * cc + e8];
    const uint32_t h = pack_bf16x2(x, 0.f) & 0xffffu;
    const float r1 = x - __uint_as_float(h << 16);
    const uint32_t m = pack_bf16x2(r1, 0.f) & 0xffffu;
    const float r2 = r1 - __uint_as_float(m << 16);
    kh[obase + o] = (uint16_t)h;
    km[obase + o] = (uint16_t)m;
    kl[obase + o] = (uint16_t)(pack_bf16x2(r2, 0.f) & 0xffffu);
  }
  if (vt == nullptr) return;  // the scores' planes only (routing without attention)
  for (int o = tid; o < kBlk * D; o += 256) {
    const int e4 = o % 4, col = (o / 4) % 16, kq = (o / 64) % 4, ci = (o / 256) % CT, t = o / (256 * CT);
    vt[obase + o] = (uint16_t)(pack_bf16x2(vs[16 * t + 4 * kq + e4][16 * ci + col], 0.f) & 0xffffu);
  }
}

hipError_t launch_prep(const float* kpool, const float* vmean, uint16_t* kh, uint16_t* km, uint16_t* kl,
                       uint16_t* vt, uint16_t* vrow, int BH, int Nk, int Nkp, int d, hipStream_t stream) {
  const dim3 grid((unsigned)(Nkp / kBlk), (unsigned)BH);
  if (d == 128)
    hipLaunchKernelGGL(prep_kernel<128>, grid, dim3(256), 0, stream, kpool, vmean, kh, km, kl, vt, vrow, Nk, Nkp);
  else
    hipLaunchKernelGGL(prep_kernel<64>, grid, dim3(256), 0, stream, kpool, vmean, kh, km, kl, vt, vrow, Nk, Nkp);
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
  const dim3 grid((unsigned)(BH * Nk), (unsigned)set.n), block(256);
  if (d == 128)
    hipLaunchKernelGGL(pool_kernel<128>, grid, block, 0, stream, set, N, Nk, hdr);
  else
    hipLaunchKernelGGL(pool_kernel<64>, grid, block, 0, stream, set, N, Nk, hdr);
  return hipGetLastError();
}

}  // namespace sol
