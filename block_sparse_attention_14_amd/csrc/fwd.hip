// Fused Sol-Attn forward for gfx950: routing, exact attention over kept key
// blocks and proxy correction of skipped blocks, in one persistent kernel.
//
// Method (page "Sol-Attn: Accelerating Video Generation Inference via
// On-the-Fly Attention Sparsification", paperlayer.ai summary):
//   §2 "Block-Sparse Attention"      proxy s_ij = mean(q_i).mean(k_j)/sqrt(d)
//   §3 "Dynamic threshold routing"   keep j iff s_ij >= max_j s_ij - tau
//   §3 "On-the-fly sparsification"   proxy rows and kept lists live in LDS
//                                    only; nothing routing-related is written
//                                    to device memory
//   §3 "Approximate correction"      skipped j adds n_j e^{s_ij} mean(v_j) to the
//                                    numerator and n_j e^{s_ij} to the denominator
//   §3 "Unified execution"           one online-softmax state per row holds the
//                                    exact and the corrected terms
//
// Work decomposition. A work item is a PAIR of neighbouring 64-row query
// blocks (b, h, 2p) and (b, h, 2p+1). A persistent grid of 256-thread
// workgroups (two per CU) takes items from atomic ticket counters: per-block
// budgets differ by two orders of magnitude, so a static split would idle CUs.
// There is one queue per XCD, each over a contiguous head-major range of items
// (so an XCD's L2 holds the pooled keys and values of few heads at a time);
// a workgroup whose queue is drained takes from the others. With a plan
// (sol_attn_plan, or the forward's own where it pays) the tickets of a queue
// map to its items through the planned order: the first two thirds in
// sequence, so neighbouring blocks (which keep overlapping key blocks) share
// K/V tiles in L2, the last third heaviest first, so no workgroup starts a
// heavy item late.
// Pairing halves the pooled-key / pooled-value traffic of routing and
// correction (one read serves both rows) and lets one K/V tile in LDS serve
// both blocks whenever both keep it, which neighbours usually do.
//
// Per item:
//   1. both Q tiles arrive through buffer loads (rows past the sequence read
//      as zero) and pass through LDS once to become, per wave, the B operand
//      of S^T = K Q^T (waves 0-1 own block A, waves 2-3 block B, 32 rows
//      each); the pooled queries are summed from the same registers;
//   2. the two fp32 proxy rows are built in LDS from pooled keys, eight lanes
//      per key block (their partial dot products meet through DPP moves), a
//      batch of loads in flight before any use;
//   3. per row: max, threshold (max - tau, or the Gaussian-calibrated
//      mean + beta std of the row, §3 "Dynamic threshold routing"), forced
//      sink blocks (App. A), skipped scores turned into correction weights
//      n_j e^{s_j - M}; a ballot/prefix pass writes the UNION of the two kept
//      lists (ascending, 2-bit owner mask) to LDS;
//   4. the correction numerators sum_j w_j mean(v_j) of both rows, one pass
//      over the pooled values, the next batch of loads in flight while one
//      is used and a batch's weights read from LDS together;
//   5. for every union entry, the K and V tiles stream from HBM straight into
//      LDS (buffer loads with an LDS destination, no registers involved),
//      double-buffered in two stages, one barrier per tile, the copy into
//      one stage issued before the other stage is consumed (the compiler
//      still makes the reads of stage A wait for a copy into stage B; the
//      other workgroup on the CU covers that wait). 16-byte chunks are
//      XOR-swizzled per row through the per-lane source addresses, so both
//      operand reads below are bank-conflict free. Each wave whose block keeps
//      the entry computes its 64x32 S^T with 16x16x32 bf16 MFMAs, the online
//      softmax in base 2 with a lazily raised maximum (one query row per lane:
//      two permlane swaps reduce a row), the row sums as an MFMA against a
//      ones operand, and O^T += V^T P^T with V^T operands read from the
//      row-major V tile by transposing LDS reads (ds_read_b64_tr_b16);
//   6. exact state and correction merge under a common maximum; rows are
//      normalised and stored in fp32 (or rounded to bf16 on request). The
//      next item's ticket is resolved before the stores and the item
//      boundary waits for LDS only, so the stores drain while the next item
//      starts (nothing in the kernel reads the output).
#include <math.h>

#include <algorithm>
#include <mutex>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace sol {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
// Workgroup barrier for LDS reuse only: this wave's LDS operations complete
// (lgkmcnt 0; vmcnt and expcnt left at their maxima), no wait for its global
// stores; the memory clobbers keep the compiler from moving memory accesses
// across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
constexpr int kThreads = 256;
// A row's running max is raised only when a tile's max exceeds it by more than
// this (base-2 units); until then probabilities may reach 2^8, which fp32 and
// bf16 carry as exactly (relatively) as values below 1.
constexpr float kLazyRescale = 8.0f;
constexpr int kMaxKeyWords = (SOL_ATTN_MAX_N / kBlk + 31) / 32;
// max over the four lanes l, l^16, l^32, l^48 that share one query row
__device__ __forceinline__ float rowmax4(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// LDS geometry. A K or V tile is 64 rows of 2d bytes, stored unpadded with
// the 16-byte chunks of each row XOR-swizzled (kslot / vslot below); a stage
// holds one K tile and one V tile. Before the kept loop the two stages also
// hold the staged Q tiles (padded rows), the routing rows and the reduction
// scratch.
template <int D>
struct Geom {
  static constexpr int RB = 2 * D;           // bytes per K / V row
  static constexpr int TILE = kBlk * RB;     // bytes per K or V tile
  static constexpr int STAGE = 2 * TILE;     // K tile, then V tile
  static constexpr int NCH = TILE / 1024;    // 1 KiB DMA chunks per tile
  static constexpr int QS = D + 8;           // staged Q row stride (bf16)
};

// 16-byte slot holding chunk c of row r. K: 16 consecutive rows read at one
// chunk cover every bank group; V: the 8 rows x 2 chunks of one transposing
// read cover every bank group.
template <int D>
__device__ __forceinline__ int kslot(int r, int c) {
  return c ^ (D == 128 ? (r & 15) : ((r >> 1) & 7));
}
template <int D>
__device__ __forceinline__ int vslot(int r, int c) {
  return c ^ (D == 128 ? 2 * (r & 7) : 2 * ((r >> 1) & 3));
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Transposing LDS read: within each 16-lane group, lane j's element e is
// element (j & 3) of the 8 bytes addressed by lane 4e + (j >> 2) of the group.
__device__ __forceinline__ uint2 ld_tr(const unsigned char* p) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  return __builtin_bit_cast(uint2, v);
}

// Issue the asynchronous HBM -> LDS copy of one K tile and one V tile into a
// stage: wave w moves the 1 KiB chunks w, w+4, ... of each tile; rows past the
// resource's size (the ragged last block) arrive as zeros. A lane's source
// offset inside its chunk is the same for every chunk of the wave (the
// swizzles depend on row bits the chunk index does not touch), so only a
// scalar offset changes between the copies.
// One 64-row tile into dst, chunks placed as K rows (kslot) or V rows (vslot).
template <int D, bool KROWS>
__device__ __forceinline__ void dma_one(unsigned char* dst, rsrc_t r, int wid, int lane) {
  using G = Geom<D>;
  constexpr int LPR = G::RB / 16;
  const int row = (1024 * wid) / G::RB + lane / LPR, sl = lane % LPR;
  const uint32_t o = row * G::RB + 16 * (KROWS ? kslot<D>(row, sl) : vslot<D>(row, sl));
#pragma unroll
  for (int u = 0; u < G::NCH / 4; ++u)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(dst + 1024 * (wid + 4 * u)), 16, o, 4096 * u, 0, 0);
}

template <int D>
__device__ __forceinline__ void dma_tile(unsigned char* stage, rsrc_t rk, rsrc_t rv, int wid, int lane) {
  using G = Geom<D>;
  constexpr int LPR = G::RB / 16;  // lanes per row of a chunk
  const int r = (1024 * wid) / G::RB + lane / LPR, sl = lane % LPR;
  const uint32_t ko = r * G::RB + 16 * kslot<D>(r, sl);
  const uint32_t vo = r * G::RB + 16 * vslot<D>(r, sl);
#pragma unroll
  for (int u = 0; u < G::NCH / 4; ++u) {
    const int off = 1024 * (wid + 4 * u);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(stage + off), 16, ko, 4096 * u, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(stage + G::TILE + off), 16, vo, 4096 * u, 0, 0);
  }
}

template <int D>
struct alignas(16) Small {
  float qbar[2][D];  // pooled queries of blocks A and B
  float cnum[2][D];  // correction numerators
  float wred[2][8];
  float gred[2][8];  // row sums, then squared deviations (Gaussian threshold)
  uint32_t kbits[2][kMaxKeyWords];  // kept-block bits of blocks A and B
  float cden[2];
  int cnt[3][4];
  int lastkept[2];
  int item;  // the item of the next iteration (-1: none left)
  int last;  // this workgroup finished last
};

// RC: the per-row (token-to-block) correction replaces the block-level one.
template <int D, bool RC>
__global__ __launch_bounds__(kThreads, 2) void fwd_kernel(FwdParams p) {
  using G = Geom<D>;
  // Two separate LDS objects for the two stages, so that reads of one stage
  // never wait for copies still landing in the other.
  __shared__ __attribute__((aligned(16))) unsigned char stA[G::STAGE];
  __shared__ __attribute__((aligned(16))) unsigned char stB[G::STAGE];
  __shared__ Small<D> sm;
  extern __shared__ __align__(16) unsigned char dyn[];
  uint16_t* ulist = reinterpret_cast<uint16_t*>(dyn);  // [Nk] union of kept lists: j | A<<14 | B<<15
  const int Nk = p.Nk, N = p.N;
  float* wrow0 = reinterpret_cast<float*>(stA);  // [Nk] block A: scores, then weights (before the kept loop)
  float* wrow1 = reinterpret_cast<float*>(stB);  // [Nk] block B

  constexpr int NDS = D / 32;  // k-steps of S^T along d
  constexpr int NDT = D / 16;  // 16-row tiles of O^T along d
  constexpr int CH = D / 8;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int g = lane >> 4, c16 = lane & 15;
  const int qb = wid >> 1;           // which block of the pair this wave serves
  const int qrow0 = 32 * (wid & 1);  // first of its 32 rows in that block
  const int npairs = (p.Nq + 1) >> 1;
  const int nlast = N - (Nk - 1) * kBlk;
  const float csc = p.scale_log2;
  // per-row correction: log2(n_j) of a full and of the ragged last key block
  // in raw dot-product units, formed once (per element they would become a
  // branch around a division)
  const float pbias = RC ? 6.f / csc : 0.f;
  const float pbias_last = RC ? __log2f((float)nlast) / csc : 0.f;

  // Queues: the workgroup starts on its own XCD's queue (workgroups are
  // dispatched to the XCDs round-robin) and, when that is drained, takes
  // from the others in turn. Only thread 0 draws; qcur is its position.
  // ticket() only issues the atomic; take() looks at the result, so the
  // round trip of a ticket drawn early overlaps other work.
  const int home = (int)(blockIdx.x % kQueues);
  int qcur = 0;
  auto ticket = [&]() -> unsigned { return atomicAdd(p.hdr + kHdrQueue + 32 * ((home + qcur) & (kQueues - 1)), 1u); };
  auto take = [&](unsigned t) -> int {
    for (;;) {
      const int x = (home + qcur) & (kQueues - 1);
      const int lo = queue_begin(x, p.nitems), n = queue_begin(x + 1, p.nitems) - lo;
      if (t < (unsigned)n) return lo + (int)t;
      if (++qcur >= kQueues) return -1;
      t = ticket();
    }
  };
  // per-workgroup stats, published once at the end (thread 0's registers)
  unsigned long long st_kept = 0, st_tot = 0, st_pairs = 0;
  unsigned st_min = 0xffffffffu, st_max = 0u;

  // (an order entry out of range, possible only with a workspace that was
  // never planned, ends this workgroup's work instead of being followed)
  auto item_of = [&](int rank) {
    const unsigned it = rank < 0 ? ~0u : (p.perm ? p.perm[rank] : (unsigned)rank);
    return it < (unsigned)p.nitems ? (int)it : -1;
  };
  if (tid == 0) sm.item = item_of(take(ticket()));
  __syncthreads();
  for (;;) {
    const int item = sm.item;
    if (item < 0) break;
    const int bh = item / npairs;  // head-major: neighbouring pairs are consecutive tickets
    const int qA = 2 * (item - bh * npairs);
    const bool hasB = qA + 1 < p.Nq;
    const size_t hoff = (size_t)bh * N * D;
    const int nA = min(kBlk, N - qA * kBlk);
    const int nB = hasB ? min(kBlk, N - (qA + 1) * kBlk) : 0;
    const int nmine = qb ? nB : nA;

    // ---- 1. Q tiles -> LDS -> Q^T operands; pooled queries from the same registers ----
    bf16x8 qop[2][NDS];
    {
      constexpr int PER = kBlk * CH / kThreads, RSTEP = kThreads / CH;
      const uint32_t qoff = ((tid / CH) * D + (tid % CH) * 8) * 2;
      uint4 qr[2][PER];
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        const int nb = blk ? nB : nA;
        const rsrc_t r = make_rsrc(p.q + hoff + (size_t)(qA + blk) * kBlk * D, (uint32_t)nb * D * 2);
#pragma unroll
        for (int u = 0; u < PER; ++u) qr[blk][u] = ld16(r, qoff, u * RSTEP * D * 2);
      }
      float* part = reinterpret_cast<float*>(stA + kBlk * G::QS * 2);  // [4 waves][2][D], past Q tile A
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        uint16_t* qd = reinterpret_cast<uint16_t*>(blk ? stB : stA) + (tid / CH) * G::QS + (tid % CH) * 8;
        float cs[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) cs[e] = 0.f;
#pragma unroll
        for (int u = 0; u < PER; ++u) {
          *reinterpret_cast<uint4*>(qd + u * RSTEP * G::QS) = qr[blk][u];
          const uint4 w = qr[blk][u];
          cs[0] += bf16lo(w.x); cs[1] += bf16hi(w.x); cs[2] += bf16lo(w.y); cs[3] += bf16hi(w.y);
          cs[4] += bf16lo(w.z); cs[5] += bf16hi(w.z); cs[6] += bf16lo(w.w); cs[7] += bf16hi(w.w);
        }
        // lanes l, l ^ 16, l ^ 32, l ^ 48 (and l ^ 8 when a row has 8 chunks)
        // hold the same columns of other rows
#pragma unroll
        for (int e = 0; e < 8; ++e) cs[e] = colsum_rows<CH>(cs[e]);
        if (lane < CH) {
#pragma unroll
          for (int e = 0; e < 8; ++e) part[(wid * 2 + blk) * D + lane * 8 + e] = cs[e];
        }
      }
      __syncthreads();
      if (tid < 2 * D) {
        const int blk = tid / D, col = tid % D;
        const int nb = blk ? nB : nA;
        const float sq = (part[(0 * 2 + blk) * D + col] + part[(1 * 2 + blk) * D + col]) +
                         (part[(2 * 2 + blk) * D + col] + part[(3 * 2 + blk) * D + col]);
        sm.qbar[blk][col] = nb > 0 ? sq / (float)nb : 0.f;
      }
      const uint16_t* qs = reinterpret_cast<const uint16_t*>(qb ? stB : stA) + (qrow0 + c16) * G::QS + 8 * g;
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds)
          qop[qt][ds] = as_bf16x8(*reinterpret_cast<const uint4*>(&qs[16 * qt * G::QS + 32 * ds]));
    }
    __syncthreads();  // qbar complete; the Q tiles may now be overwritten

    // ---- 2. proxy rows s_j = q̄ . k̄_j / sqrt(d), both blocks, into LDS ----
    {
      constexpr int NV = D / 32;  // float4 per lane; 8 lanes cover one pooled key
      constexpr int U = 4;        // key blocks in flight per lane (64 KiB per workgroup at d=128)
      constexpr int JS = kThreads / 8;
      const int sub = tid & 7, jg = tid >> 3;
      float4 qa[NV], qbv[NV];
#pragma unroll
      for (int t = 0; t < NV; ++t) {
        qa[t] = *reinterpret_cast<const float4*>(&sm.qbar[0][4 * (sub + 8 * t)]);
        qbv[t] = *reinterpret_cast<const float4*>(&sm.qbar[1][4 * (sub + 8 * t)]);
      }
      const rsrc_t rk = make_rsrc(p.kpool + (size_t)bh * Nk * D, (uint32_t)Nk * D * 4);
      const uint32_t voff = (jg * D + sub * 4) * 4;
      float mA = -INFINITY, mB = -INFINITY;
      for (int j0 = 0; j0 < Nk; j0 += U * JS) {
        float4 x[U][NV];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int t = 0; t < NV; ++t) x[u][t] = ld16f(rk, voff + t * 128, (uint32_t)(j0 + u * JS) * D * 4);
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int j = j0 + u * JS + jg;
          float a = 0.f, b = 0.f;
#pragma unroll
          for (int t = 0; t < NV; ++t) {
            a += qa[t].x * x[u][t].x + qa[t].y * x[u][t].y + qa[t].z * x[u][t].z + qa[t].w * x[u][t].w;
            b += qbv[t].x * x[u][t].x + qbv[t].y * x[u][t].y + qbv[t].z * x[u][t].z + qbv[t].w * x[u][t].w;
          }
          a = sum8(a);  // the 8 lanes of key block j
          b = sum8(b);
          a *= p.proxy_scale;
          b *= p.proxy_scale;
          if (j < Nk) {
            if (sub == 0) {
              wrow0[j] = a;
              wrow1[j] = b;
            }
            mA = fmaxf(mA, a);
            mB = fmaxf(mB, b);
          }
        }
      }
      mA = wave_max(mA);
      mB = wave_max(mB);
      if (lane == 0) {
        sm.wred[0][wid] = mA;
        sm.wred[1][wid] = mB;
      }
    }
    __syncthreads();
    const float MA = fmaxf(fmaxf(sm.wred[0][0], sm.wred[0][1]), fmaxf(sm.wred[0][2], sm.wred[0][3]));
    const float MB = fmaxf(fmaxf(sm.wred[1][0], sm.wred[1][1]), fmaxf(sm.wred[1][2], sm.wred[1][3]));

    // thresholds: the row max minus tau, or the Gaussian-calibrated mean +
    // beta * std of the row (population statistics over the key blocks; the
    // row is on chip, so both come exactly from it in two passes)
    float thA = MA - p.tau, thB = MB - p.tau;
    if (p.rule == SOL_ROUTE_GAUSS_DIAG) {
      // mean and (diagonal-estimate) variance of the rows from the pooled-key
      // statistics of the head: known without the rows themselves
      float a0 = 0.f, b0 = 0.f, a1 = 0.f, b1 = 0.f;
      if (tid < D) {
        const rsrc_t rs = make_rsrc(p.kstats + (size_t)bh * 2 * D, 2 * D * 4);
        const float mu = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, tid * 4, 0, 0));
        const float var = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, (D + tid) * 4, 0, 0));
        const float x0 = sm.qbar[0][tid], x1 = sm.qbar[1][tid];
        a0 = x0 * mu;
        b0 = x0 * x0 * var;
        a1 = x1 * mu;
        b1 = x1 * x1 * var;
      }
      a0 = wave_sum(a0);
      b0 = wave_sum(b0);
      a1 = wave_sum(a1);
      b1 = wave_sum(b1);
      if (lane == 0) {
        sm.gred[0][wid] = a0;
        sm.gred[0][4 + wid] = b0;
        sm.gred[1][wid] = a1;
        sm.gred[1][4 + wid] = b1;
      }
      __syncthreads();
      const float inv_d = p.proxy_scale * p.proxy_scale;
      thA = ((sm.gred[0][0] + sm.gred[0][1]) + (sm.gred[0][2] + sm.gred[0][3])) * p.proxy_scale +
            p.beta * sqrtf(((sm.gred[0][4] + sm.gred[0][5]) + (sm.gred[0][6] + sm.gred[0][7])) * inv_d);
      thB = ((sm.gred[1][0] + sm.gred[1][1]) + (sm.gred[1][2] + sm.gred[1][3])) * p.proxy_scale +
            p.beta * sqrtf(((sm.gred[1][4] + sm.gred[1][5]) + (sm.gred[1][6] + sm.gred[1][7])) * inv_d);
    } else if (p.rule == SOL_ROUTE_GAUSS) {
      float sA = 0.f, sB = 0.f;
      for (int j = tid; j < Nk; j += kThreads) {
        sA += wrow0[j];
        sB += wrow1[j];
      }
      sA = wave_sum(sA);
      sB = wave_sum(sB);
      if (lane == 0) {
        sm.gred[0][wid] = sA;
        sm.gred[1][wid] = sB;
      }
      __syncthreads();
      const float inv_nk = 1.f / (float)Nk;
      const float muA = ((sm.gred[0][0] + sm.gred[0][1]) + (sm.gred[0][2] + sm.gred[0][3])) * inv_nk;
      const float muB = ((sm.gred[1][0] + sm.gred[1][1]) + (sm.gred[1][2] + sm.gred[1][3])) * inv_nk;
      float vA = 0.f, vB = 0.f;
      for (int j = tid; j < Nk; j += kThreads) {
        const float a = wrow0[j] - muA, b = wrow1[j] - muB;
        vA += a * a;
        vB += b * b;
      }
      vA = wave_sum(vA);
      vB = wave_sum(vB);
      if (lane == 0) {
        sm.gred[0][4 + wid] = vA;
        sm.gred[1][4 + wid] = vB;
      }
      __syncthreads();
      thA = muA + p.beta * sqrtf(((sm.gred[0][4] + sm.gred[0][5]) + (sm.gred[0][6] + sm.gred[0][7])) * inv_nk);
      thB = muB + p.beta * sqrtf(((sm.gred[1][4] + sm.gred[1][5]) + (sm.gred[1][6] + sm.gred[1][7])) * inv_nk);
    }

    // ---- 3. route both rows; weights for skipped blocks; union kept list ----
    int nu = 0, nkA = 0, nkB = 0;
    {
      float wsA = 0.f, wsB = 0.f;
      uint32_t* bmA = p.bitmap ? p.bitmap + (size_t)(bh * p.Nq + qA) * p.nwords : nullptr;
      uint32_t* bmB = (p.bitmap && hasB) ? bmA + p.nwords : nullptr;
      for (int j0 = 0; j0 < Nk; j0 += kThreads) {
        const int j = j0 + tid;
        bool kA = false, kB = false;
        if (j < Nk) {
          const float nj = (float)min(kBlk, N - j * kBlk);
          const float sa = wrow0[j];
          const bool sink = (unsigned)(j - p.sink_lo) < (unsigned)(p.sink_hi - p.sink_lo);
          kA = sa >= thA || sink;
          const float wa = kA ? 0.f : nj * expf(sa - MA);
          wrow0[j] = wa;
          wsA += wa;
          float wb = 0.f;
          if (hasB) {
            const float sb = wrow1[j];
            kB = sb >= thB || sink;
            wb = kB ? 0.f : nj * expf(sb - MB);
            wsB += wb;
          }
          wrow1[j] = wb;
        }
        const unsigned long long bA = __ballot(kA), bB = __ballot(kB), bU = bA | bB;
        if (lane == 0) {
          sm.cnt[0][wid] = __popcll(bU);
          sm.cnt[1][wid] = __popcll(bA);
          sm.cnt[2][wid] = __popcll(bB);
          const int w0 = (j0 + 64 * wid) >> 5;
          if (w0 < kMaxKeyWords) {
            sm.kbits[0][w0] = (uint32_t)bA;
            sm.kbits[1][w0] = (uint32_t)bB;
          }
          if (w0 + 1 < kMaxKeyWords) {
            sm.kbits[0][w0 + 1] = (uint32_t)(bA >> 32);
            sm.kbits[1][w0 + 1] = (uint32_t)(bB >> 32);
          }
          if (bmA) {
            if (w0 < p.nwords) bmA[w0] = (uint32_t)bA;
            if (w0 + 1 < p.nwords) bmA[w0 + 1] = (uint32_t)(bA >> 32);
          }
          if (bmB) {
            if (w0 < p.nwords) bmB[w0] = (uint32_t)bB;
            if (w0 + 1 < p.nwords) bmB[w0 + 1] = (uint32_t)(bB >> 32);
          }
        }
        if (j == Nk - 1) {
          sm.lastkept[0] = kA;
          sm.lastkept[1] = kB;
        }
        __syncthreads();
        int off = nu;
        for (int w2 = 0; w2 < wid; ++w2) off += sm.cnt[0][w2];
        if (kA || kB)
          ulist[off + __popcll(bU & ((1ull << lane) - 1ull))] = (uint16_t)(j | (kA ? 1 << 14 : 0) | (kB ? 1 << 15 : 0));
        nu += sm.cnt[0][0] + sm.cnt[0][1] + sm.cnt[0][2] + sm.cnt[0][3];
        nkA += sm.cnt[1][0] + sm.cnt[1][1] + sm.cnt[1][2] + sm.cnt[1][3];
        nkB += sm.cnt[2][0] + sm.cnt[2][1] + sm.cnt[2][2] + sm.cnt[2][3];
        __syncthreads();
      }
      wsA = wave_sum(wsA);
      wsB = wave_sum(wsB);
      if (lane == 0) {
        sm.wred[0][4 + wid] = wsA;
        sm.wred[1][4 + wid] = wsB;
      }
    }

    // ---- 4. correction numerators cnum[b][c] = sum_j w_bj vbar_j[c] ----
    {
      constexpr int C4 = D / 4, JG = kThreads / C4, U = 8;  // 2 x 32 KiB of pooled values in flight
      const int c4 = tid % C4, jg = tid / C4;
      float4 a0 = make_float4(0.f, 0.f, 0.f, 0.f), a1 = a0;
      if (!RC && !p.exact_only && (nkA < Nk || (hasB && nkB < Nk))) {
        const rsrc_t rv = make_rsrc(p.vmean + (size_t)bh * Nk * D, (uint32_t)Nk * D * 4);
        const uint32_t voff = (jg * U * D + c4 * 4) * 4;
        // two batches of U pooled values per lane (lane group jg takes U
        // consecutive key blocks of each batch): one in flight while the
        // other is used (loads past Nk read zero and are never used)
        auto load = [&](float4 (&x)[U], int j0) {
#pragma unroll
          for (int u = 0; u < U; ++u) x[u] = ld16f(rv, voff, (uint32_t)(j0 + u) * D * 4);
        };
        // all weights of a batch are read before any is used, with no branch
        // in between (four 16-byte LDS reads), so their round trips overlap
        // (blocks past Nk get weight 0; their pooled values read as zero)
        auto use = [&](const float4 (&x)[U], int j0) {
          const int jb = j0 + jg * U;  // (reads up to Nk rounded to 64 stay in the stage)
          float w0[U], w1[U];
#pragma unroll
          for (int u = 0; u < U; u += 4) {
            const float4 a = *reinterpret_cast<const float4*>(&wrow0[jb + u]);
            const float4 b = *reinterpret_cast<const float4*>(&wrow1[jb + u]);
            w0[u] = a.x; w0[u + 1] = a.y; w0[u + 2] = a.z; w0[u + 3] = a.w;
            w1[u] = b.x; w1[u + 1] = b.y; w1[u + 2] = b.z; w1[u + 3] = b.w;
          }
#pragma unroll
          for (int u = 0; u < U; ++u) {
            w0[u] = jb + u < Nk ? w0[u] : 0.f;
            w1[u] = jb + u < Nk ? w1[u] : 0.f;
          }
#pragma unroll
          for (int u = 0; u < U; ++u) {
            a0.x += w0[u] * x[u].x; a0.y += w0[u] * x[u].y; a0.z += w0[u] * x[u].z; a0.w += w0[u] * x[u].w;
            a1.x += w1[u] * x[u].x; a1.y += w1[u] * x[u].y; a1.z += w1[u] * x[u].z; a1.w += w1[u] * x[u].w;
          }
        };
        float4 x0[U], x1[U];
        load(x0, 0);
        for (int j0 = 0; j0 < Nk; j0 += 2 * U * JG) {
          load(x1, j0 + U * JG);
          use(x0, j0);
          if (j0 + U * JG >= Nk) break;
          if (j0 + 2 * U * JG < Nk) load(x0, j0 + 2 * U * JG);
          use(x1, j0 + U * JG);
        }
      }
      __syncthreads();  // weights fully read: their space becomes reduction scratch
      float* red = reinterpret_cast<float*>(stA);  // [2][JG][D]
      *reinterpret_cast<float4*>(&red[(0 * JG + jg) * D + 4 * c4]) = a0;
      *reinterpret_cast<float4*>(&red[(1 * JG + jg) * D + 4 * c4]) = a1;
      __syncthreads();
      if (tid < 2 * D) {
        const int blk = tid / D, col = tid % D;
        float s = 0.f;
#pragma unroll
        for (int r = 0; r < JG; ++r) s += red[(blk * JG + r) * D + col];
        sm.cnum[blk][col] = s;
      }
      if (tid < 2)
        sm.cden[tid] = RC ? 0.f : (sm.wred[tid][4] + sm.wred[tid][5]) + (sm.wred[tid][6] + sm.wred[tid][7]);
      __syncthreads();  // the tile stages are free again
    }


    // ---- 5. exact attention over the union list (online softmax, base 2) ----
    f32x4 acc[2][NDT];
    f32x4 lsum[2];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      lsum[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) acc[qt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float m[2] = {-INFINITY, -INFINITY};
    {
      const bf16x8 ones = as_bf16x8(make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u));
      const uint16_t* kh = p.k + hoff;
      const uint16_t* vh = p.v + hoff;
      const int ownbit = 1 << (14 + qb);
      // K and V tiles of kept key block ulist[t] into one stage
      auto dma = [&](unsigned char* stage, int t) {
        const int j = ulist[t] & 0x3fff;
        const uint32_t bytes = (uint32_t)min(kBlk, N - j * kBlk) * D * 2;
        dma_tile<D>(stage, make_rsrc(kh + (size_t)j * kBlk * D, bytes), make_rsrc(vh + (size_t)j * kBlk * D, bytes),
                    wid, lane);
      };
      // pooled tile c (per-row correction): the two bf16 parts of the pooled
      // keys fill stage A (both as K rows), the pooled values stage B's V half
      auto dma_pooled = [&](int c) {
        const uint32_t bytes = (uint32_t)min(kBlk, Nk - c * kBlk) * D * 2;
        const size_t off = ((size_t)bh * Nk + (size_t)c * kBlk) * D;
        dma_one<D, true>(stA, make_rsrc(p.khi16 + off, bytes), wid, lane);
        dma_one<D, true>(stA + G::TILE, make_rsrc(p.klo16 + off, bytes), wid, lane);
        dma_one<D, false>(stB + G::TILE, make_rsrc(p.vbar16 + off, bytes), wid, lane);
      };
      // per-lane byte offsets of the swizzled operand reads (independent of the key tile kt)
      int koff[NDS];
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) koff[ds] = c16 * G::RB + 16 * kslot<D>(c16, 4 * ds + g);
      // transposing V reads: this lane addresses row 4g + e (+32ks +16h) and the
      // 8 bytes of columns 16dt + 4cc .. +3
      const int ve = (lane >> 2) & 3, vcc = lane & 3, vrow = 4 * g + ve;
      int voff[NDT];
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        voff[dt] = G::TILE + vrow * G::RB + 16 * vslot<D>(vrow, 2 * dt + (vcc >> 1)) + 8 * (vcc & 1);

      auto compute = [&](const unsigned char* stage, int e, auto pooled) {
        constexpr bool kPooled = decltype(pooled)::value;
        if (!kPooled && !(e & ownbit)) return;  // wave-uniform: this wave's block skips the entry
        const int j = e & 0x3fff;
        const int nj = kPooled ? kBlk : min(kBlk, N - j * kBlk);
        // S^T[kv][q]: 4 key tiles x 2 query tiles; each K operand serves both
        f32x4 st[2][4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          st[0][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
          st[1][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        // K operands four steps ahead of the MFMAs that use them (one step
        // ahead leaves each MFMA pair waiting on its LDS read)
        auto kread = [&](int i) {
          return as_bf16x8(*reinterpret_cast<const uint4*>(stage + 16 * (i / NDS) * G::RB + koff[i % NDS]));
        };
        constexpr int KA = 4;
        bf16x8 kop[4 * NDS];
#pragma unroll
        for (int i = 0; i < KA; ++i) kop[i] = kread(i);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
          for (int ds = 0; ds < NDS; ++ds) {
            const int i = kt * NDS + ds;
            const bf16x8 a = kop[i];
            if (i + KA < 4 * NDS) kop[i + KA] = kread(i + KA);
            __builtin_amdgcn_sched_barrier(0);
            st[0][kt] = mfma16x16x32(a, qop[0][ds], st[0][kt]);
            st[1][kt] = mfma16x16x32(a, qop[1][ds], st[1][kt]);
            __builtin_amdgcn_sched_barrier(0);
            if (kPooled) {  // the remainder part of the pooled keys, one tile further on
              const bf16x8 b =
                  as_bf16x8(*reinterpret_cast<const uint4*>(stage + G::TILE + 16 * kt * G::RB + koff[ds]));
              st[0][kt] = mfma16x16x32(b, qop[0][ds], st[0][kt]);
              st[1][kt] = mfma16x16x32(b, qop[1][ds], st[1][kt]);
            }
          }
        }
        // lane holds S^T[16kt + 4g + i][row c16 of query tile qt]
        if (kPooled) {
          // pooled key 64e + 16kt + 4g + i: masked when kept by this wave's
          // block (it is in the exact branch) or past Nk; otherwise its
          // weight n_j enters as log2(n_j) on the base-2 logit, added here in
          // raw dot-product units (n_j = 64 but for the ragged last block)
          const uint32_t* kb = sm.kbits[qb];
          const int valid = Nk - e * kBlk;
          uint64_t off = (uint64_t)kb[2 * e] | ((uint64_t)kb[2 * e + 1] << 32);
          if (valid < kBlk) off |= ~0ull << valid;
          off >>= 4 * g;
          const int last = Nk - 1 - e * kBlk - 4 * g;  // lane position of the last block, if here
#pragma unroll
          for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const bool masked = (off >> (16 * kt + i)) & 1ull;
              const float b = masked ? -INFINITY : 16 * kt + i == last ? pbias_last : pbias;
              st[0][kt][i] += b;
              st[1][kt][i] += b;
            }
        } else if (nj < kBlk) {
#pragma unroll
          for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (16 * kt + 4 * g + i >= nj) {
                st[0][kt][i] = -INFINITY;
                st[1][kt][i] = -INFINITY;
              }
        }
        bool raise = false;
        float mn[2];
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          // two chains of three-input maxima over the lane's 16 scores
          float b0 = fmaxf(fmaxf(st[qt][0][0], st[qt][0][1]), st[qt][0][2]);
          float b1 = fmaxf(fmaxf(st[qt][2][0], st[qt][2][1]), st[qt][2][2]);
          b0 = fmaxf(fmaxf(b0, st[qt][0][3]), st[qt][1][0]);
          b1 = fmaxf(fmaxf(b1, st[qt][2][3]), st[qt][3][0]);
          b0 = fmaxf(fmaxf(b0, st[qt][1][1]), st[qt][1][2]);
          b1 = fmaxf(fmaxf(b1, st[qt][3][1]), st[qt][3][2]);
          b0 = fmaxf(b0, st[qt][1][3]);
          b1 = fmaxf(b1, st[qt][3][3]);
          const float bm = rowmax4(fmaxf(b0, b1)) * csc;
          mn[qt] = bm > m[qt] + kLazyRescale ? bm : m[qt];
          raise = raise || (mn[qt] != m[qt]);
        }
        if (__ballot(raise)) {  // rare: a row's max rose by more than the lazy margin
#pragma unroll
          for (int qt = 0; qt < 2; ++qt) {
            const float alpha = __builtin_amdgcn_exp2f(m[qt] - mn[qt]);
            lsum[qt] *= alpha;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) acc[qt][dt] *= alpha;
            m[qt] = mn[qt];
          }
        }
        // P^T operand slots 0-3 = keys 32ks+4g+i, slots 4-7 = keys 32ks+16+4g+i
        bf16x8 pb[2][2];
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          const float nm = -m[qt];
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            uint32_t w[4];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const f32x4& sv = st[qt][2 * ks + h];
              w[2 * h + 0] = pack_bf16x2(__builtin_amdgcn_exp2f(fmaf(sv[0], csc, nm)),
                                         __builtin_amdgcn_exp2f(fmaf(sv[1], csc, nm)));
              w[2 * h + 1] = pack_bf16x2(__builtin_amdgcn_exp2f(fmaf(sv[2], csc, nm)),
                                         __builtin_amdgcn_exp2f(fmaf(sv[3], csc, nm)));
            }
            pb[qt][ks] = as_bf16x8(make_uint4(w[0], w[1], w[2], w[3]));
          }
          // row sums of the bf16-rounded probabilities: every output row of
          // ones x P^T is the sum over the 32 keys of the step
          lsum[qt] = mfma16x16x32(ones, pb[qt][0], lsum[qt]);
          lsum[qt] = mfma16x16x32(ones, pb[qt][1], lsum[qt]);
        }
        // O^T[d][q] += V^T[d][kv] P^T[kv][q]; the transposing reads of rows
        // 32ks + 4g + e and 32ks + 16 + 4g + e give exactly the keys of the P^T
        // slots; each V^T operand serves both query tiles
        const unsigned char* vstage = kPooled ? stB : stage;
        // V^T operands of the next 16 rows of d read while this slice's MFMAs run
        auto vread = [&](int dt, uint2 (&o)[4]) {
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            o[2 * ks] = ld_tr(vstage + voff[dt] + 32 * ks * G::RB);
            o[2 * ks + 1] = ld_tr(vstage + voff[dt] + (32 * ks + 16) * G::RB);
          }
        };
        uint2 vc[4], vn[4];
        vread(0, vc);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          if (dt + 1 < NDT) vread(dt + 1, vn);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            const bf16x8 a = as_bf16x8(make_uint4(vc[2 * ks].x, vc[2 * ks].y, vc[2 * ks + 1].x, vc[2 * ks + 1].y));
            acc[0][dt] = mfma16x16x32(a, pb[0][ks], acc[0][dt]);
            acc[1][dt] = mfma16x16x32(a, pb[1][ks], acc[1][dt]);
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) vc[e2] = vn[e2];
        }
      };

      // Every barrier below is preceded by an explicit wait for all of this
      // wave's outstanding copies: the copy into one stage is issued in one
      // loop iteration and consumed in the next, a dependency the compiler's
      // own wait insertion does not carry across the loop back-edge.
      if (nu > 0) dma(stA, 0);
      if (nu > 1) dma(stB, 1);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();  // tiles 0 and 1 are in LDS
      for (int t = 0; t < nu; t += 2) {
        compute(stA, ulist[t], std::false_type{});
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();  // tile t+1 has landed in stB; nobody reads stA any more
        if (t + 2 < nu) dma(stA, t + 2);
        if (t + 1 < nu) {
          compute(stB, ulist[t + 1], std::false_type{});
          __builtin_amdgcn_s_waitcnt(0);
          __syncthreads();  // tile t+2 has landed in stA; nobody reads stB any more
          if (t + 3 < nu) dma(stB, t + 3);
        }
      }
      if (RC) {
        // pooled tiles, one at a time: each fills stage A and half of stage B
        const int npool = (Nk + kBlk - 1) / kBlk;
        for (int c = 0; c < npool; ++c) {
          // a tile whose key blocks both rows keep holds only masked pooled
          // keys (all of them, at tau = +inf): skipped, the same decision in
          // every thread (kept bits in LDS), so the barriers stay matched
          const int nv = min(kBlk, Nk - c * kBlk);
          const uint64_t valid = nv >= 64 ? ~0ull : ((1ull << nv) - 1ull);
          const uint64_t ka = (uint64_t)sm.kbits[0][2 * c] | ((uint64_t)sm.kbits[0][2 * c + 1] << 32);
          const uint64_t kb = (uint64_t)sm.kbits[1][2 * c] | ((uint64_t)sm.kbits[1][2 * c + 1] << 32);
          if ((valid & ~ka) == 0 && (!hasB || (valid & ~kb) == 0)) continue;
          dma_pooled(c);
          __builtin_amdgcn_s_waitcnt(0);
          __syncthreads();  // pooled tile c is in LDS
          compute(stA, c, std::true_type{});
          __syncthreads();  // nobody reads the pooled tile any more
        }
      }
    }

    // The next ticket is drawn now, so its round trip overlaps the fold
    // below (it is resolved before this wave's stores); drawing it earlier
    // would tie an item to this workgroup while it may still spend long on
    // this one, which others could have taken.
    unsigned next_ticket = 0;
    if (tid == 0) next_ticket = ticket();

    // ---- 6. fold exact and corrected terms, normalise, store ----
    {
      const float M2 = (qb ? MB : MA) * kLog2e;
      const float cden = sm.cden[qb];
      const int rbase = (qA + qb) * kBlk;
      // with no correction mass (exact-only, the per-row mode, every block
      // kept, or every skipped weight zero) the exact state alone is
      // normalised: a common maximum with M2 could underflow it to zero
      const bool corr = !p.exact_only && cden > 0.f;
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        const float lt = lsum[qt][0];
        const float mf = corr ? fmaxf(m[qt], M2) : m[qt];
        const float fa = __builtin_amdgcn_exp2f(m[qt] - mf);
        const float fc = corr ? __builtin_amdgcn_exp2f(M2 - mf) : 0.f;
        const float inv = 1.f / (lt * fa + cden * fc);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const int c = 16 * dt + 4 * g;
          acc[qt][dt][0] = (acc[qt][dt][0] * fa + sm.cnum[qb][c + 0] * fc) * inv;
          acc[qt][dt][1] = (acc[qt][dt][1] * fa + sm.cnum[qb][c + 1] * fc) * inv;
          acc[qt][dt][2] = (acc[qt][dt][2] * fa + sm.cnum[qb][c + 2] * fc) * inv;
          acc[qt][dt][3] = (acc[qt][dt][3] * fa + sm.cnum[qb][c + 3] * fc) * inv;
        }
      }
      // the next item, resolved before this wave's stores, so that waiting
      // for the ticket never waits for them
      if (tid == 0) sm.item = item_of(take(next_ticket));
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        const int row = qrow0 + 16 * qt + c16;
        if (row < nmine) {
          const size_t orow = hoff + (size_t)(rbase + row) * D;
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) {
            const int c = 16 * dt + 4 * g;
            const f32x4 o = acc[qt][dt];
            if (p.out_bf16)
              *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + orow + c) =
                  make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
            else
              *reinterpret_cast<float4*>(static_cast<float*>(p.out) + orow + c) = make_float4(o[0], o[1], o[2], o[3]);
          }
        }
      }
    }

    if (tid == 0) {
      const unsigned long long tokA = (unsigned long long)nkA * kBlk - (sm.lastkept[0] ? kBlk - nlast : 0);
      st_pairs += tokA * (unsigned long long)nA;
      st_kept += nkA;
      st_tot += Nk;
      st_min = min(st_min, (unsigned)nkA);
      st_max = max(st_max, (unsigned)nkA);
      if (hasB) {
        const unsigned long long tokB = (unsigned long long)nkB * kBlk - (sm.lastkept[1] ? kBlk - nlast : 0);
        st_pairs += tokB * (unsigned long long)nB;
        st_kept += nkB;
        st_tot += Nk;
        st_min = min(st_min, (unsigned)nkB);
        st_max = max(st_max, (unsigned)nkB);
      }
    }
    lds_barrier();  // the next item is in sm.item; LDS is rewritten by it (output stores may still be in flight)
  }

  // Each workgroup adds its stats once; the last one to finish publishes
  // them and leaves the header clean (zero tickets, zero counters) for the
  // next call on this workspace.
  if (tid == 0) {
    unsigned long long* acc64 = reinterpret_cast<unsigned long long*>(p.hdr);
    if (p.stats != nullptr && st_tot != 0) {
      atomicAdd(acc64 + kHdrKept / 2, st_kept);
      atomicAdd(acc64 + kHdrTotal / 2, st_tot);
      atomicAdd(acc64 + kHdrPairs / 2, st_pairs);
      atomicMin(p.hdr + kHdrMin, st_min);
      atomicMax(p.hdr + kHdrMax, st_max);
    }
    __threadfence();
    const unsigned done = atomicAdd(p.hdr + kHdrDone, 1u);
    sm.last = done == gridDim.x - 1;
    if (sm.last) {
      __threadfence();
      if (p.stats != nullptr) {
        p.stats->kept_blocks = __hip_atomic_load(acc64 + kHdrKept / 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        p.stats->total_blocks = __hip_atomic_load(acc64 + kHdrTotal / 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        p.stats->kept_pairs = __hip_atomic_load(acc64 + kHdrPairs / 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        p.stats->min_kept = __hip_atomic_load(p.hdr + kHdrMin, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        p.stats->max_kept = __hip_atomic_load(p.hdr + kHdrMax, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  __syncthreads();
  if (sm.last)
    for (int w = tid; w < kHdrWords; w += kThreads)
      __hip_atomic_store(p.hdr + w, w == kHdrMin ? 0xffffffffu : 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

size_t forward_dynamic_lds(int Nk) { return ((size_t)Nk * 2 + 15) & ~(size_t)15; }

int forward_items(int BH, int Nq) { return BH * ((Nq + 1) / 2); }

int forward_max_blocks(int d) {
  // each fp32 routing row lives in one stage before the kept loop
  return d == 128 ? Geom<128>::STAGE / 4 : Geom<64>::STAGE / 4;
}

template <int D, bool RC>
static hipError_t launch_d(const FwdParams& p, hipStream_t stream) {
  // per-device CU count and occupancy (bucketed by dynamic LDS in 4 KiB steps)
  static std::mutex mu;
  static int cus[64] = {0};
  static int occ_cache[64][8] = {{0}};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  const size_t dyn = forward_dynamic_lds(p.Nk);
  const int bucket = (int)std::min<size_t>(7, dyn / 4096);
  int grid_per_cu = 0, ncu = 0;
  {
    std::lock_guard<std::mutex> lock(mu);
    if (cus[dev] == 0) {
      int n = 0;
      e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
      if (e != hipSuccess) return e;
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(&fwd_kernel<D, RC>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, 32 * 1024);
      if (e != hipSuccess) return e;
      cus[dev] = n;
    }
    if (occ_cache[dev][bucket] == 0) {
      int occ = 0;
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, reinterpret_cast<const void*>(&fwd_kernel<D, RC>),
                                                       kThreads, (size_t)(bucket + 1) * 4096);
      if (e != hipSuccess) return e;
      occ_cache[dev][bucket] = occ < 1 ? 1 : occ;
    }
    ncu = cus[dev];
    grid_per_cu = occ_cache[dev][bucket];
  }
  const int grid = (int)std::min<long long>((long long)ncu * grid_per_cu, p.nitems);
  hipLaunchKernelGGL((fwd_kernel<D, RC>), dim3(grid), dim3(kThreads), dyn, stream, p);
  return hipGetLastError();
}

hipError_t launch_forward(const FwdParams& p, int d, hipStream_t stream) {
  if (p.row_corr) return d == 128 ? launch_d<128, true>(p, stream) : launch_d<64, true>(p, stream);
  return d == 128 ? launch_d<128, false>(p, stream) : launch_d<64, false>(p, stream);
}

}  // namespace sol
