// Fused Sol-Attn forward for gfx950: routing, exact attention over kept key
// blocks and proxy correction of skipped blocks, in one persistent kernel.
//
// Method (page "Sol-Attn: Accelerating Video Generation Inference via
// On-the-Fly Attention Sparsification", paperlayer.ai summary):
//   §2 "Block-Sparse Attention"      proxy s_ij = mean(q_i).mean(k_j)/sqrt(d)
//   §3 "Dynamic threshold routing"   keep j iff s_ij >= max_j s_ij - tau
//   §3 "On-the-fly sparsification"   the proxy row and the kept list live in
//                                    LDS only; nothing routing-related is
//                                    written to device memory
//   §3 "Approximate correction"      skipped j adds n_j e^{s_ij} mean(v_j) to the
//                                    numerator and n_j e^{s_ij} to the denominator
//   §3 "Unified execution"           one online-softmax state per row holds the
//                                    exact and the corrected terms
//
// Work decomposition. A work item is one 64-row query block (b, h, i). A
// persistent grid of 256-thread workgroups takes items from an atomic ticket
// counter (budgets differ wildly between query blocks, so a static split would
// leave CUs idle). Per item:
//   1. the Q tile is staged through LDS; each wave keeps its 16 rows as the B
//      operand of S^T = K Q^T in registers, and the block mean q̄ is reduced;
//   2. the proxy row s_j (fp32, Nk values) is built in LDS from pooled keys,
//      eight lanes per key block;
//   3. the row max M gives the threshold; a ballot/prefix pass compacts the
//      kept indices (ascending) into LDS and replaces each skipped score by its
//      correction weight n_j e^{s_j - M};
//   4. for every kept block, K (row-major) and V (transposed) tiles go through
//      LDS; each wave computes its 64x16 slice of S^T with 16x16x32 bf16 MFMAs,
//      applies the online softmax in base 2 (one query row per lane, so row
//      statistics need only two cross-lane steps), and accumulates O^T += V^T P^T;
//   5. the correction numerator sum_j w_j mean(v_j) is a GEMV over the pooled
//      values of skipped blocks;
//   6. the exact state and the correction are merged with a common maximum and
//      the normalised rows are stored in fp32.
#include <math.h>

#include <algorithm>
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace sol {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kThreads = 256;
constexpr int kVtStride = kBlk + 4;  // bf16 per row of the transposed V tile

template <int D>
struct Smem {
  uint16_t Ks[kBlk][D + 8];   // K tile, row-major; also stages the Q tile
  uint16_t Vt[D][kVtStride];  // V tile, transposed (key index fastest)
  float qbar[D];              // pooled query of the current block
  float cnum[D];              // correction numerator
  float red[1024];            // reduction scratch
  float wred[8];
  int cnt[4];
  int item;
};

// Global -> register loads of one K tile and one V tile (rows >= nj are zero).
template <int D>
struct KVRegs {
  static constexpr int CH = D / 8;                 // 16-byte chunks per row
  static constexpr int KPER = kBlk * CH / kThreads;  // K chunks per thread
  static constexpr int RG = kBlk * CH / kThreads;    // V rows per thread (same count)
  uint4 k[KPER];
  uint4 v[RG];

  __device__ __forceinline__ void load(const uint16_t* kt, const uint16_t* vt, int nj, int tid) {
#pragma unroll
    for (int u = 0; u < KPER; ++u) {
      const int id = tid + kThreads * u;
      const int r = id / CH, c = id % CH;
      k[u] = r < nj ? *reinterpret_cast<const uint4*>(kt + (size_t)r * D + c * 8) : make_uint4(0, 0, 0, 0);
    }
    const int a = tid / CH, c = tid % CH;
#pragma unroll
    for (int r = 0; r < RG; ++r) {
      const int row = a * RG + r;
      v[r] = row < nj ? *reinterpret_cast<const uint4*>(vt + (size_t)row * D + c * 8) : make_uint4(0, 0, 0, 0);
    }
  }

  __device__ __forceinline__ void store(Smem<D>& sm, int tid) const {
#pragma unroll
    for (int u = 0; u < KPER; ++u) {
      const int id = tid + kThreads * u;
      const int r = id / CH, c = id % CH;
      *reinterpret_cast<uint4*>(&sm.Ks[r][c * 8]) = k[u];
    }
    const int a = tid / CH, c = tid % CH;
    // element e of each of the RG rows -> one contiguous run of Vt[8c + e][RG*a ..]
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint32_t h[RG];
#pragma unroll
      for (int r = 0; r < RG; ++r) {
        const uint32_t w = (e < 2) ? v[r].x : (e < 4) ? v[r].y : (e < 6) ? v[r].z : v[r].w;
        h[r] = (e & 1) ? (w >> 16) : (w & 0xffffu);
      }
      if constexpr (RG == 4) {
        uint2 pk;
        pk.x = h[0] | (h[1] << 16);
        pk.y = h[2] | (h[3] << 16);
        *reinterpret_cast<uint2*>(&sm.Vt[8 * c + e][RG * a]) = pk;
      } else {
        *reinterpret_cast<uint32_t*>(&sm.Vt[8 * c + e][RG * a]) = h[0] | (h[1] << 16);
      }
    }
  }
};

template <int D>
__global__ __launch_bounds__(kThreads, 2) void fwd_kernel(FwdParams p) {
  __shared__ Smem<D> sm;
  extern __shared__ __align__(16) unsigned char dyn[];
  float* wrow = reinterpret_cast<float*>(dyn);                  // [Nk] scores, then weights
  uint16_t* klist = reinterpret_cast<uint16_t*>(dyn + 4 * (size_t)p.Nk);  // [Nk] kept indices

  constexpr int NDS = D / 32;  // k-steps of S^T (d direction)
  constexpr int NDT = D / 16;  // 16-row tiles of O^T (d direction)
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int N = p.N, Nk = p.Nk;

  for (;;) {
    if (tid == 0) sm.item = (int)atomicAdd(p.queue + kQueueTicket, 1u);
    __syncthreads();
    const int item = sm.item;
    if (item >= p.nitems) break;
    const int bh = item / p.Nq;  // head-major: neighbouring query blocks are consecutive tickets
    const int qi = item - bh * p.Nq;
    const size_t hoff = (size_t)bh * N * D;
    const int r0 = qi * kBlk;
    const int ni = min(kBlk, N - r0);

    // ---- 1. Q tile -> LDS, Q^T operands -> registers, pooled query ----
    {
      constexpr int CH = D / 8, PER = kBlk * CH / kThreads;
      const uint16_t* src = p.q + hoff + (size_t)r0 * D;
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int id = tid + kThreads * u;
        const int r = id / CH, c = id % CH;
        *reinterpret_cast<uint4*>(&sm.Ks[r][c * 8]) =
            r < ni ? *reinterpret_cast<const uint4*>(src + (size_t)r * D + c * 8) : make_uint4(0, 0, 0, 0);
      }
    }
    __syncthreads();
    bf16x8 qop[NDS];
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds)
      qop[ds] = as_bf16x8(*reinterpret_cast<const uint4*>(&sm.Ks[16 * wid + c16][32 * ds + 8 * g]));
    {
      constexpr int PARTS = kThreads / D, RP = kBlk / PARTS;
      const int col = tid % D, part = tid / D;
      float s = 0.f;
      for (int r = part * RP; r < part * RP + RP; ++r) s += bf16lo(sm.Ks[r][col]);
      sm.red[part * D + col] = s;
    }
    __syncthreads();
    if (tid < D) {
      float s = 0.f;
#pragma unroll
      for (int part = 0; part < kThreads / D; ++part) s += sm.red[part * D + tid];
      sm.qbar[tid] = s / (float)ni;
    }
    __syncthreads();

    // ---- 2. proxy row s_j = q̄ . k̄_j / sqrt(d) into LDS, and its maximum ----
    {
      constexpr int NV = D / 32;  // float4 per lane; 8 lanes cover one pooled key
      const int sub = tid & 7, jg = tid >> 3;
      float4 qv[NV];
#pragma unroll
      for (int t = 0; t < NV; ++t) qv[t] = *reinterpret_cast<const float4*>(&sm.qbar[4 * (sub + 8 * t)]);
      const float* kp = p.kpool + (size_t)bh * Nk * D;
      float lmax = -INFINITY;
      for (int j0 = 0; j0 < Nk; j0 += kThreads / 8) {
        const int j = j0 + jg;
        float a = 0.f;
        if (j < Nk) {
          const float4* row = reinterpret_cast<const float4*>(kp + (size_t)j * D);
#pragma unroll
          for (int t = 0; t < NV; ++t) {
            const float4 x = row[sub + 8 * t];
            a += qv[t].x * x.x + qv[t].y * x.y + qv[t].z * x.z + qv[t].w * x.w;
          }
        }
        a += __shfl_xor(a, 1);
        a += __shfl_xor(a, 2);
        a += __shfl_xor(a, 4);
        const float sj = a * p.proxy_scale;
        if (j < Nk) {
          if (sub == 0) wrow[j] = sj;
          lmax = fmaxf(lmax, sj);
        }
      }
      lmax = wave_max(lmax);
      if (lane == 0) sm.wred[wid] = lmax;
    }
    __syncthreads();
    const float M = fmaxf(fmaxf(sm.wred[0], sm.wred[1]), fmaxf(sm.wred[2], sm.wred[3]));

    // ---- 3. route: keep iff s_j >= M - tau; skipped scores become weights ----
    const float theta = M - p.tau;
    float wsum = 0.f;
    int nk = 0;
    for (int j0 = 0; j0 < Nk; j0 += kThreads) {
      const int j = j0 + tid;
      bool keep = false;
      if (j < Nk) {
        const float sj = wrow[j];
        keep = sj >= theta;
        float w = 0.f;
        if (!keep) w = (float)min(kBlk, N - j * kBlk) * expf(sj - M);
        wrow[j] = w;
        wsum += w;
      }
      const unsigned long long bal = __ballot(keep);
      if (lane == 0) sm.cnt[wid] = __popcll(bal);
      if (p.bitmap != nullptr && lane == 0) {
        const int w0 = (j0 + 64 * wid) >> 5;
        uint32_t* brow = p.bitmap + (size_t)item * p.nwords;
        if (w0 < p.nwords) brow[w0] = (uint32_t)bal;
        if (w0 + 1 < p.nwords) brow[w0 + 1] = (uint32_t)(bal >> 32);
      }
      __syncthreads();
      int off = nk;
      for (int w2 = 0; w2 < wid; ++w2) off += sm.cnt[w2];
      if (keep) klist[off + __popcll(bal & ((1ull << lane) - 1ull))] = (uint16_t)j;
      nk += sm.cnt[0] + sm.cnt[1] + sm.cnt[2] + sm.cnt[3];
      __syncthreads();
    }
    wsum = wave_sum(wsum);
    if (lane == 0) sm.wred[4 + wid] = wsum;
    __syncthreads();  // klist, wrow and wred complete
    const float cden = (sm.wred[4] + sm.wred[5]) + (sm.wred[6] + sm.wred[7]);

    // ---- 4. exact attention over the kept blocks (online softmax, base 2) ----
    f32x4 acc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, l = 0.f;
    const uint16_t* kh = p.k + hoff;
    const uint16_t* vh = p.v + hoff;
    KVRegs<D> regs;
    if (nk > 0) {
      const int j = klist[0];
      regs.load(kh + (size_t)j * kBlk * D, vh + (size_t)j * kBlk * D, min(kBlk, N - j * kBlk), tid);
    }
    for (int t = 0; t < nk; ++t) {
      const int j = klist[t];
      const int nj = min(kBlk, N - j * kBlk);
      __syncthreads();  // the previous tile is no longer read
      regs.store(sm, tid);
      __syncthreads();
      if (t + 1 < nk) {
        const int jn = klist[t + 1];
        regs.load(kh + (size_t)jn * kBlk * D, vh + (size_t)jn * kBlk * D, min(kBlk, N - jn * kBlk), tid);
      }

      // S^T[kv][q] for kv in 16-row tiles kt, q = this wave's 16 rows
      f32x4 st[4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        st[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) {
          const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(&sm.Ks[16 * kt + c16][32 * ds + 8 * g]));
          st[kt] = mfma16x16x32(a, qop[ds], st[kt]);
        }
      }
      // lane holds S^T[16kt + 4g + e][c16]: one query row, 16 keys
      float bm = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float x = st[kt][e] * p.scale_log2;
          if (16 * kt + 4 * g + e >= nj) x = -INFINITY;
          st[kt][e] = x;
          bm = fmaxf(bm, x);
        }
      bm = fmaxf(bm, __shfl_xor(bm, 16));
      bm = fmaxf(bm, __shfl_xor(bm, 32));
      const float mn = fmaxf(m, bm);
      const float alpha = exp2f(m - mn);
      float ls = 0.f;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float pe = exp2f(st[kt][e] - mn);
          st[kt][e] = pe;
          ls += pe;
        }
      l = l * alpha + ls;
      m = mn;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) acc[dt] *= alpha;

      // P^T operands: k-slots 0-3 = keys 32ks+4g+e, slots 4-7 = keys 32ks+16+4g+e
      bf16x8 pb[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        uint4 u;
        u.x = pack_bf16x2(st[2 * ks][0], st[2 * ks][1]);
        u.y = pack_bf16x2(st[2 * ks][2], st[2 * ks][3]);
        u.z = pack_bf16x2(st[2 * ks + 1][0], st[2 * ks + 1][1]);
        u.w = pack_bf16x2(st[2 * ks + 1][2], st[2 * ks + 1][3]);
        pb[ks] = as_bf16x8(u);
      }
      // O^T[d][q] += V^T[d][kv] P^T[kv][q], same key permutation on both sides
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const uint2 lo = *reinterpret_cast<const uint2*>(&sm.Vt[16 * dt + c16][32 * ks + 4 * g]);
          const uint2 hi = *reinterpret_cast<const uint2*>(&sm.Vt[16 * dt + c16][32 * ks + 16 + 4 * g]);
          acc[dt] = mfma16x16x32(as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y)), pb[ks], acc[dt]);
        }
    }

    // ---- 5. correction numerator: cnum[c] = sum_j w_j vbar_j[c] ----
    {
      constexpr int C4 = D / 4, JG = kThreads / C4;
      const int c4 = tid % C4, jg = tid / C4;
      float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
      if (!p.exact_only && nk < Nk) {
        const float4* vm = reinterpret_cast<const float4*>(p.vmean + (size_t)bh * Nk * D);
        for (int j = jg; j < Nk; j += JG) {
          const float w = wrow[j];
          if (w != 0.f) {
            const float4 x = vm[(size_t)j * C4 + c4];
            a.x += w * x.x; a.y += w * x.y; a.z += w * x.z; a.w += w * x.w;
          }
        }
      }
      *reinterpret_cast<float4*>(&sm.red[jg * D + 4 * c4]) = a;
    }
    __syncthreads();
    if (tid < D) {
      float s = 0.f;
#pragma unroll
      for (int jg = 0; jg < kThreads / (D / 4); ++jg) s += sm.red[jg * D + tid];
      sm.cnum[tid] = s;
    }
    __syncthreads();

    // ---- 6. fold exact and corrected terms, normalise, store ----
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    {
      const float M2 = M * kLog2e;
      const float mf = p.exact_only ? m : fmaxf(m, M2);
      const float fa = exp2f(m - mf);
      const float fc = p.exact_only ? 0.f : exp2f(M2 - mf);
      const float inv = 1.f / (l * fa + cden * fc);
      const int row = 16 * wid + c16;
      if (row < ni) {
        float* orow = p.out + hoff + (size_t)(r0 + row) * D;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const int c = 16 * dt + 4 * g;
          float4 o;
          o.x = (acc[dt][0] * fa + sm.cnum[c + 0] * fc) * inv;
          o.y = (acc[dt][1] * fa + sm.cnum[c + 1] * fc) * inv;
          o.z = (acc[dt][2] * fa + sm.cnum[c + 2] * fc) * inv;
          o.w = (acc[dt][3] * fa + sm.cnum[c + 3] * fc) * inv;
          *reinterpret_cast<float4*>(orow + c) = o;
        }
      }
    }

    if (p.stats != nullptr && tid == 0) {
      unsigned long long kept_tokens = (unsigned long long)nk * kBlk;
      if (nk > 0 && klist[nk - 1] == Nk - 1) kept_tokens -= (unsigned long long)(kBlk - (N - (Nk - 1) * kBlk));
      atomicAdd(&p.stats->kept_blocks, (unsigned long long)nk);
      atomicAdd(&p.stats->total_blocks, (unsigned long long)Nk);
      atomicAdd(&p.stats->kept_pairs, kept_tokens * (unsigned long long)ni);
      atomicMin(&p.stats->min_kept, (unsigned)nk);
      atomicMax(&p.stats->max_kept, (unsigned)nk);
    }
    __syncthreads();  // LDS is rewritten by the next item
  }
}

}  // namespace

size_t forward_dynamic_lds(int Nk) { return ((size_t)Nk * 6 + 15) & ~(size_t)15; }

template <int D>
static hipError_t launch_d(const FwdParams& p, hipStream_t stream) {
  // per-device CU count and occupancy (bucketed by dynamic LDS in 8 KiB steps)
  static std::mutex mu;
  static int cus[64] = {0};
  static int occ_cache[64][8] = {{0}};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  const size_t dyn = forward_dynamic_lds(p.Nk);
  const int bucket = (int)std::min<size_t>(7, dyn / 8192);
  int grid_per_cu = 0, ncu = 0;
  {
    std::lock_guard<std::mutex> lock(mu);
    if (cus[dev] == 0) {
      int n = 0;
      e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
      if (e != hipSuccess) return e;
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(&fwd_kernel<D>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, 96 * 1024);
      if (e != hipSuccess) return e;
      cus[dev] = n;
    }
    if (occ_cache[dev][bucket] == 0) {
      int occ = 0;
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, reinterpret_cast<const void*>(&fwd_kernel<D>),
                                                       kThreads, (size_t)(bucket + 1) * 8192);
      if (e != hipSuccess) return e;
      occ_cache[dev][bucket] = occ < 1 ? 1 : occ;
    }
    ncu = cus[dev];
    grid_per_cu = occ_cache[dev][bucket];
  }
  const int grid = (int)std::min<long long>((long long)ncu * grid_per_cu, p.nitems);
  hipLaunchKernelGGL(fwd_kernel<D>, dim3(grid), dim3(kThreads), dyn, stream, p);
  return hipGetLastError();
}

hipError_t launch_forward(const FwdParams& p, int d, hipStream_t stream) {
  return d == 128 ? launch_d<128>(p, stream) : launch_d<64>(p, stream);
}

}  // namespace sol
