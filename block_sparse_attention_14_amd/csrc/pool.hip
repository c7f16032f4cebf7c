// Pooling pre-pass: per 64-token block, the fp32 mean of q, k and v over the
// block's valid tokens (page "Sol-Attn: Accelerating Video Generation
// Inference via On-the-Fly Attention Sparsification", §2 "Block-Sparse
// Attention": mean-pooled blocks; §3 "Approximate correction": pooled keys and
// summed values, the latter being n_j times the mean stored here), and the
// bf16 operand planes the fused kernel's routing pass reads.
//
// One workgroup per (block j, head) and tensor (grid x = head * Nk + j, grid y
// = tensor). Each thread streams 16-byte chunks of rows, the partial sums meet
// in LDS, and thread c writes column c. The pass is a pure HBM stream: every
// input byte is read once. A workgroup whose tensor has a plane role also
// writes block j's entries of the routing planes, from its own mean or from
// the caller's pooled keys and values.
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
// Thread c of block j's workgroup writes column c of the planes its role
// names, from x (the block's mean) or from the caller's pooled tensors. The
// workgroup of the last block also zeroes rows Nk .. Nkp - 1, which the
// fused kernel reads as padding of the last tile.
__device__ __forceinline__ void key_parts(float x, uint16_t& h, uint16_t& m, uint16_t& l) {
  const uint32_t hh = pack_bf16x2(x, 0.f) & 0xffffu;
  const float r1 = x - __uint_as_float(hh << 16);
  const uint32_t mm = pack_bf16x2(r1, 0.f) & 0xffffu;
  const float r2 = r1 - __uint_as_float(mm << 16);
  h = (uint16_t)hh;
  m = (uint16_t)mm;
  l = (uint16_t)(pack_bf16x2(r2, 0.f) & 0xffffu);
}

template <int D>
__device__ void write_planes(const Planes& pl, int role, float x, int bh, int j, int Nk, int c) {
  constexpr int CH = D / 8, CT = D / 16;
  const size_t base = (size_t)bh * pl.Nkp * D;
  auto koff = [&](int jj) { return base + ((size_t)((jj >> 4) * CH + (c >> 3)) * 16 + (jj & 15)) * 8 + (c & 7); };
  auto voff = [&](int jj) {
    return base + ((size_t)(((jj >> 4) * CT + (c >> 4)) * 4 + ((jj & 15) >> 2)) * 16 + (c & 15)) * 4 + (jj & 3);
  };
  const size_t rowc = ((size_t)bh * Nk + j) * D + c;
  if (role & (kRoleKeys | kRoleKeysFromPool)) {
    const float xk = (role & kRoleKeys) ? x : pl.kpool[rowc];
    uint16_t h, m, l;
    key_parts(xk, h, m, l);
    const size_t o = koff(j);
    pl.kh[o] = h;
    pl.km[o] = m;
    pl.kl[o] = l;
    if (j == Nk - 1)
      for (int jz = Nk; jz < pl.Nkp; ++jz) {
        const size_t oz = koff(jz);
        pl.kh[oz] = pl.km[oz] = pl.kl[oz] = 0;
      }
  }
  if ((role & (kRoleValues | kRoleValuesFromPool)) && pl.vt) {
    const float xv = (role & kRoleValues) ? x : pl.vmean[rowc];
    const uint16_t b = (uint16_t)(pack_bf16x2(xv, 0.f) & 0xffffu);
    pl.vt[voff(j)] = b;
    if (pl.vrow) pl.vrow[rowc] = b;
    if (j == Nk - 1)
      for (int jz = Nk; jz < pl.Nkp; ++jz) pl.vt[voff(jz)] = 0;
  }
}

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
    s /= (float)nj;
    dst[tid] = s;
    const int role = set.role[which];
    if (role != 0) write_planes<D>(set.planes, role, s, bh, j, Nk, tid);
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
  const dim3 grid((unsigned)(BH * Nk), (unsigned)set.n), block(256);
  if (d == 128)
    hipLaunchKernelGGL(pool_kernel<128>, grid, block, 0, stream, set, N, Nk, hdr);
  else
    hipLaunchKernelGGL(pool_kernel<64>, grid, block, 0, stream, set, N, Nk, hdr);
  return hipGetLastError();
}

}  // namespace sol
