// Work ordering for the fused kernel: the tail of each queue heaviest first.
//
// The per-query-block budgets of threshold routing vary by two orders of
// magnitude (page "Sol-Attn: Accelerating Video Generation Inference via
// On-the-Fly Attention Sparsification", §1 and §3 "Dynamic threshold
// routing": dynamic, query-dependent budgets). A persistent grid that takes
// items in sequence order ends with a few workgroups finishing the heaviest
// items while the rest idle. These two small kernels estimate every item's
// cost (the sizes of the unions of its pairs' kept lists) and order each
// XCD queue: head-major first, then its last third heaviest first, so the
// queue ends on light items.
//
// The estimate uses bf16 MFMA products of sampled query means and the pooled
// keys: it only orders work. The fused kernel routes every item itself, in fp32, and
// nothing here influences which blocks it keeps. Only one count per item is
// written to device memory; no proxy scores or block indices are.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace sol {

namespace {

// Score tiles a wave keeps in registers between the max pass and the count
// pass; tiles beyond these are recomputed in the count pass.
constexpr int kCached = 4;
constexpr int kBatch = 2;       // tiles whose loads are in flight together
constexpr int kPlanWaves = 8;   // waves per planning workgroup, splitting the key tiles
constexpr int kPlanQ = 32;      // query blocks per workgroup: two 16-column tiles per wave
constexpr int kSampleStride = 4;  // every 4th row of a query block enters its estimated mean

// Loads of one 16x16 S^T tile of pooled keys: lane (g, c16) fetches pooled
// key jt0 + c16, columns 32 ds + 8 g .. +7. Buffer loads: keys past Nk read
// zero without a branch, so the loads of a batch are all in flight at once.
template <int D>
__device__ __forceinline__ void tile_load(rsrc_t rk, int jt0, int c16, int g, float4 (&x)[D / 16]) {
  const uint32_t off = ((jt0 + c16) * D + 8 * g) * 4;
#pragma unroll
  for (int ds = 0; ds < D / 32; ++ds) {
    x[2 * ds] = ld16f(rk, off + 128 * ds, 0);
    x[2 * ds + 1] = ld16f(rk, off + 128 * ds + 16, 0);
  }
}

// The two S^T column tiles (query blocks 0-15 and 16-31 of the workgroup)
// against one tile of pooled keys, in bf16 MFMA.
template <int D>
__device__ __forceinline__ void tile_mma(const float4 (&x)[D / 16], const bf16x8 (&qop)[2][D / 32], f32x4 (&s)[2]) {
  s[0] = s[1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ds = 0; ds < D / 32; ++ds) {
    const float4 a = x[2 * ds], b = x[2 * ds + 1];
    const bf16x8 k = as_bf16x8(make_uint4(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w), pack_bf16x2(b.x, b.y),
                                          pack_bf16x2(b.z, b.w)));
    s[0] = mfma16x16x32(k, qop[0][ds], s[0]);
    s[1] = mfma16x16x32(k, qop[1][ds], s[1]);
  }
}

// grid (ceil(Nq / 32), BH), 512 threads. The workgroup estimates the pooled
// query of each of its 32 query blocks from every 4th row (a scheduling
// estimate: the forward pools all rows itself), then all eight waves serve
// the same 32 query blocks, wave w taking key tiles w, w + 8, ... Pass 1 finds
// each block's maximum, pass 2 counts, per pair of blocks, the key blocks
// that either block keeps. Both reductions meet in LDS.
template <int D>
__global__ __launch_bounds__(64 * kPlanWaves) void plan_kernel(const uint16_t* __restrict__ q,
                                                                const float* __restrict__ kpool,
                                                   unsigned* __restrict__ cost, int N, int Nq, int Nk, float tau,
                                                   float proxy_scale) {
  constexpr int TPB = 64 * kPlanWaves / kPlanQ;  // threads per query block
  constexpr int CPT = D / TPB;                   // columns per thread
  __shared__ float qs[kPlanQ][D];
  __shared__ float red[kPlanWaves][kPlanQ];
  __shared__ unsigned cred[kPlanWaves][kPlanQ];
  const int bh = blockIdx.y, q0 = kPlanQ * blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform

  // sampled means: thread t covers block t / TPB, columns (t % TPB) * CPT .. +CPT-1;
  // buffer loads over the block's valid rows read zero past them, so all of
  // a thread's loads are issued before the first sum
  {
    const int b = tid / TPB, c0 = (tid % TPB) * CPT, qb = q0 + b;
    const int nb = qb < Nq ? min(kBlk, N - qb * kBlk) : 0;
    float acc[CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) acc[c] = 0.f;
    // one resource per wave (wave-uniform, so no per-lane resource loop) over
    // the rows of its consecutive query blocks, clamped to the sequence
    constexpr int BPW = 64 / TPB;  // query blocks per wave
    const int qw = q0 + wid * BPW;
    const int rows_w = __builtin_amdgcn_readfirstlane(max(0, min(BPW * kBlk, N - qw * kBlk)));
    const rsrc_t rq = make_rsrc(q + ((size_t)bh * N + (size_t)(rows_w > 0 ? qw : 0) * kBlk) * D, (uint32_t)rows_w * D * 2);
    const uint32_t lane_off = (uint32_t)(((b - wid * BPW) * kBlk * D + c0) * 2);
    constexpr int NS = kBlk / kSampleStride;
    if constexpr (CPT == 8) {
      uint4 u[NS];
#pragma unroll
      for (int r = 0; r < NS; ++r) u[r] = ld16(rq, lane_off + (uint32_t)(r * kSampleStride * D * 2), 0);
#pragma unroll
      for (int r = 0; r < NS; ++r) {
        acc[0] += bf16lo(u[r].x); acc[1] += bf16hi(u[r].x);
        acc[2] += bf16lo(u[r].y); acc[3] += bf16hi(u[r].y);
        acc[4] += bf16lo(u[r].z); acc[5] += bf16hi(u[r].z);
        acc[6] += bf16lo(u[r].w); acc[7] += bf16hi(u[r].w);
      }
    } else {
      static_assert(CPT == 4, "8 or 4 columns per thread");
      uint2 u[NS];
#pragma unroll
      for (int r = 0; r < NS; ++r) {
        const auto w = __builtin_amdgcn_raw_buffer_load_b64(rq, (int)(lane_off + r * kSampleStride * D * 2), 0, 0);
        u[r] = make_uint2(w[0], w[1]);
      }
#pragma unroll
      for (int r = 0; r < NS; ++r) {
        acc[0] += bf16lo(u[r].x); acc[1] += bf16hi(u[r].x);
        acc[2] += bf16lo(u[r].y); acc[3] += bf16hi(u[r].y);
      }
    }
    const float inv = nb > 0 ? 1.f / (float)((nb + kSampleStride - 1) / kSampleStride) : 0.f;
#pragma unroll
    for (int c = 0; c < CPT; ++c) qs[b][c0 + c] = acc[c] * inv;
  }
  __syncthreads();

  const int g = lane >> 4, c16 = lane & 15;
  const rsrc_t rk = make_rsrc(kpool + (size_t)bh * Nk * D, (uint32_t)Nk * D * 4);
  bf16x8 qop[2][D / 32];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int ds = 0; ds < D / 32; ++ds) {
      const float* r = &qs[16 * ct + c16][32 * ds + 8 * g];
      qop[ct][ds] = as_bf16x8(make_uint4(pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3]), pack_bf16x2(r[4], r[5]),
                                         pack_bf16x2(r[6], r[7])));
    }
  const int njt = (Nk + 15) / 16;
  auto valid = [&](int jt, int i) { return 16 * jt + 4 * g + i < Nk; };

  // pass 1: maxima; the first kCached tiles of this wave stay in registers
  float mx[2] = {-INFINITY, -INFINITY};
  f32x4 sc[kCached][2];
#pragma unroll
  for (int c0 = 0; c0 < kCached; c0 += kBatch) {
    float4 x[kBatch][D / 16];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) tile_load<D>(rk, 16 * (wid + kPlanWaves * (c0 + u)), c16, g, x[u]);
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int jt = wid + kPlanWaves * (c0 + u);
      tile_mma<D>(x[u], qop, sc[c0 + u]);
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (jt < njt && valid(jt, i)) mx[ct] = fmaxf(mx[ct], sc[c0 + u][ct][i]);
    }
  }
  for (int jt = wid + kPlanWaves * kCached; jt < njt; jt += kPlanWaves) {
    float4 x[D / 16];
    tile_load<D>(rk, 16 * jt, c16, g, x);
    f32x4 s[2];
    tile_mma<D>(x, qop, s);
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (valid(jt, i)) mx[ct] = fmaxf(mx[ct], s[ct][i]);
  }
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    mx[ct] = fmaxf(mx[ct], __shfl_xor(mx[ct], 16));
    mx[ct] = fmaxf(mx[ct], __shfl_xor(mx[ct], 32));
    if (g == 0) red[wid][16 * ct + c16] = mx[ct];
  }
  __syncthreads();
  float thr[2];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int col = 16 * ct + c16;
    float m = red[0][col];
#pragma unroll
    for (int w = 1; w < kPlanWaves; ++w) m = fmaxf(m, red[w][col]);
    thr[ct] = m * proxy_scale - tau;
  }

  // pass 2: size of the union of the kept sets of blocks c16 and c16 ^ 1
  unsigned cnt[2] = {0u, 0u};
  auto count = [&](const f32x4 (&s)[2], int jt) {
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool keep = q0 + 16 * ct + c16 < Nq && jt < njt && valid(jt, i) && s[ct][i] * proxy_scale >= thr[ct];
        const bool other = dpp<kDppXor1>((int)keep) != 0;  // the pair's other block (lane c16 ^ 1)
        cnt[ct] += (keep || other) ? 1u : 0u;
      }
  };
#pragma unroll
  for (int c = 0; c < kCached; ++c) count(sc[c], wid + kPlanWaves * c);
  for (int jt = wid + kPlanWaves * kCached; jt < njt; jt += kPlanWaves) {
    float4 x[D / 16];
    tile_load<D>(rk, 16 * jt, c16, g, x);
    f32x4 s[2];
    tile_mma<D>(x, qop, s);
    count(s, jt);
  }
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    cnt[ct] += __shfl_xor(cnt[ct], 16);
    cnt[ct] += __shfl_xor(cnt[ct], 32);
    if (g == 0) cred[wid][16 * ct + c16] = cnt[ct];
  }
  __syncthreads();
  const int npairs = (Nq + 1) / 2;
  if (tid < kPlanQ && (tid & 1) == 0 && q0 + tid < Nq) {
    unsigned c = 0;
#pragma unroll
    for (int w = 0; w < kPlanWaves; ++w) c += cred[w][tid];
    cost[(size_t)bh * npairs + (q0 + tid) / 2] = c;
  }
}

// One workgroup per queue. The first two thirds of the queue's range keep
// their natural, head-major order, so the workgroups of an XCD work on
// neighbouring query blocks, whose kept key blocks overlap, and share those
// tiles in L2. The last third is sorted by decreasing cost (a counting sort;
// equal costs in no particular order), so the queue ends on its lightest
// items and no workgroup starts a heavy one when the others are about to
// finish.
// An item of G query blocks costs the sum over its G / 2 pairs, bucketed in
// units of G / 2 so that the histogram keeps Nk + 1 buckets.
// The queue is then written out as work units in this order: an item whose
// estimated cost reaches split_cost (so that its routing pass is a small part
// of it) becomes G / 2 units, one per pair, each routing the item again; any
// other item one unit. Unit u = item | (pair + 1) << 28 (pair bits only for
// G >= 4), at units[lo * G / 2 ...], their number in unit_counts[queue].
__global__ __launch_bounds__(1024) void order_kernel(const unsigned* __restrict__ cost, unsigned* __restrict__ perm,
                                                     unsigned* __restrict__ units, unsigned* __restrict__ plan_items,
                                                     int nitems, int Nk, int npairs, int group, int ngroups,
                                                     unsigned split_cost) {
  extern __shared__ unsigned hist[];  // [Nk + 1] counts, then running offsets
  __shared__ unsigned part[1024];
  const int tid = threadIdx.x, nt = blockDim.x;
  const int lo = queue_begin(blockIdx.x, nitems), hi = queue_begin(blockIdx.x + 1, nitems);
  const int t0 = hi - (hi - lo) / 3;  // first item of the sorted tail
  const int hp = group / 2;           // pairs per item
  auto item_cost = [&](int i) {
    const int bh = i / ngroups, p0 = hp * (i - bh * ngroups);
    unsigned c = 0;
    for (int t = 0; t < hp && p0 + t < npairs; ++t) c += cost[(size_t)bh * npairs + p0 + t];
    return c;
  };
  auto bucket = [&](int i) { return min(item_cost(i) / (unsigned)hp, (unsigned)Nk); };
  for (int i = lo + tid; i < t0; i += nt) perm[i] = (unsigned)i;
  for (int b = tid; b <= Nk; b += nt) hist[b] = 0u;
  __syncthreads();
  for (int i = t0 + tid; i < hi; i += nt) atomicAdd(&hist[bucket(i)], 1u);
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
  unsigned run = (unsigned)t0 + part[tid] - local;  // exclusive, offset to the tail's first rank
  for (int k = 0; k < C; ++k) {
    const int pos = tid * C + k;
    if (pos <= Nk) {
      const unsigned c = hist[Nk - pos];
      hist[Nk - pos] = run;
      run += c;
    }
  }
  __syncthreads();
  for (int i = t0 + tid; i < hi; i += nt) perm[atomicAdd(&hist[bucket(i)], 1u)] = (unsigned)i;
  __threadfence_block();
  __syncthreads();  // the queue's order is complete

  // work units in the order's sequence: an exclusive scan of the units per
  // rank, 1024 ranks at a time
  unsigned* out = units + (size_t)lo * hp;
  unsigned base = 0;
  for (int r0 = lo; r0 < hi; r0 += nt) {
    const int r = r0 + tid;
    unsigned it = 0, nu = 0;
    if (r < hi) {
      it = perm[r];
      nu = hp >= 2 && item_cost((int)it) >= split_cost ? (unsigned)hp : 1u;
    }
    part[tid] = nu;
    __syncthreads();
    for (int off = 1; off < nt; off <<= 1) {  // inclusive scan
      const unsigned v = tid >= off ? part[tid - off] : 0u;
      __syncthreads();
      part[tid] += v;
      __syncthreads();
    }
    const unsigned at = base + part[tid] - nu;
    if (nu == 1u)
      out[at] = it;
    else
      for (unsigned k = 0; k < nu; ++k) out[at + k] = it | ((k + 1u) << 28);
    base += part[nt - 1];
    __syncthreads();  // part is rewritten by the next chunk
  }
  if (tid == 0) {
    plan_items[8 + blockIdx.x] = base;
    if (blockIdx.x == 0) *plan_items = (unsigned)nitems;
  }
}

// The identity order as work units: one per item, each queue in sequence.
__global__ __launch_bounds__(256) void iota_kernel(unsigned* __restrict__ units, unsigned* __restrict__ plan_items,
                                                   int nitems, int hp) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i == 0) *plan_items = (unsigned)nitems;
  if (i < kQueues) plan_items[8 + i] = (unsigned)(queue_begin(i + 1, nitems) - queue_begin(i, nitems));
  if (i < nitems) {
    int x = 0;
    while (x + 1 < kQueues && queue_begin(x + 1, nitems) <= i) ++x;
    const int lo = queue_begin(x, nitems);
    units[(size_t)lo * hp + (i - lo)] = (unsigned)i;
  }
}

}  // namespace

hipError_t launch_identity_order(unsigned* units, unsigned* plan_items, int nitems, int group, hipStream_t stream) {
  hipLaunchKernelGGL(iota_kernel, dim3((nitems + 255) / 256), dim3(256), 0, stream, units, plan_items, nitems,
                     group / 2);
  return hipGetLastError();
}

hipError_t launch_plan(const uint16_t* q, const float* kpool, unsigned* cost, unsigned* perm, unsigned* units,
                       unsigned* plan_items, int BH, int N, int Nq, int Nk, int d, float tau, float proxy_scale,
                       int group, unsigned split_cost, hipStream_t stream) {
  const dim3 grid((Nq + kPlanQ - 1) / kPlanQ, BH);
  if (d == 128)
    hipLaunchKernelGGL(plan_kernel<128>, grid, dim3(64 * kPlanWaves), 0, stream, q, kpool, cost, N, Nq, Nk, tau,
                       proxy_scale);
  else
    hipLaunchKernelGGL(plan_kernel<64>, grid, dim3(64 * kPlanWaves), 0, stream, q, kpool, cost, N, Nq, Nk, tau,
                       proxy_scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nitems = forward_items(BH, Nq, group);
  hipLaunchKernelGGL(order_kernel, dim3(kQueues), dim3(1024), (size_t)(Nk + 1) * sizeof(unsigned), stream, cost,
                     perm, units, plan_items, nitems, Nk, (Nq + 1) / 2, group, (Nq + group - 1) / group, split_cost);
  return hipGetLastError();
}

}  // namespace sol
