// Fused Sol-Attn forward for gfx950: routing, exact attention over kept key
// blocks and proxy correction of skipped blocks, in one persistent kernel.
//
// Method (page "Sol-Attn: Accelerating Video Generation Inference via
// On-the-Fly Attention Sparsification", paperlayer.ai summary):
//   §2 "Block-Sparse Attention"      proxy s_ij = mean(q_i).mean(k_j)/sqrt(d)
//   §3 "Dynamic threshold routing"   keep j iff s_ij >= max_j s_ij - tau, or the
//                                    Gaussian-calibrated mean + beta std of the
//                                    row, from pooled-key moments
//   §3 "On-the-fly sparsification"   scores are consumed chunk by chunk as
//                                    they are produced; nothing routing-related
//                                    is written to device memory
//   §3 "Approximate correction"      skipped j adds n_j e^{s_ij} mean(v_j) to the
//                                    numerator and n_j e^{s_ij} to the denominator
//   §3 "Unified execution"           one online-softmax state per row holds the
//                                    exact and the corrected terms
//
// Work decomposition. A work item is a GROUP of G consecutive 64-row query
// blocks of one head (G = 2, 4, 6, 8 or 16, chosen by the host so that there are
// enough items to balance the grid). A persistent grid of 256-thread
// workgroups (two per CU) takes items from atomic ticket counters: per-block
// budgets differ by two orders of magnitude, so a static split would idle CUs.
// There is one queue per XCD, each over a contiguous head-major range of items
// (so an XCD's L2 holds the pooled keys and values of few heads at a time); a
// workgroup whose queue is drained takes from the others. With a plan
// (sol_attn_plan, or the forward's own where it pays) the tickets of a queue
// map to its items through the planned order.
//
// Per item:
//   A. the pooled queries of the G blocks (made by the pooling pre-pass) and,
//      for the Gaussian rules, each block's threshold from the head's
//      pooled-key moments (known before any score exists);
//   R. one streaming pass over the head's pooled keys and pooled values (bf16
//      operand planes from the pre-pass: keys in three parts, values in one),
//      in steps of 16 key blocks taken outwards from the group's own blocks;
//      wave w takes steps w, w + 4, ... and streams on its own. Per step:
//        the proxy scores of the G blocks as MFMA products (three-part keys
//        against three-part queries: fp32-grade dot products);
//        per block: the wave's running maximum, the threshold (running
//        maximum - tau, after a first maximum over every wave's first step,
//        or the fixed Gaussian one), keep or skip, the weight n_j e^{s - M}
//        of each skipped block against the running maximum (earlier weights
//        rescaled when it rises), kept bits into LDS;
//        the correction numerators sum_j w_j vbar_j of the G blocks as MFMA
//        products of the pooled values with the weights;
//      so the group reads the pooled keys and values once: G/2 times less
//      than pairs of blocks would, which is what long sequences need;
//   R4. row-max rule only: the steps a wave routed before its maximum reached
//      the row's are routed again against the row's maximum (a block kept
//      against a lower one may move to the correction); the waves' partial
//      sums merge under the row maximum; the group's bits are final;
//   then for each PAIR of blocks of the group:
//   1. both Q tiles through LDS into registers, the B operand of S^T = K Q^T
//      (wave w holds rows 16w .. 16w + 15 of both blocks: query tile 0 of the
//      first block, query tile 1 of the second);
//   2. the union of the two kept lists, walked straight from the kept bits
//      (wave-uniform scalar state, no stored list) in three runs: the key
//      blocks both blocks keep, then those only the first keeps, then those
//      only the second keeps, each run in ascending order with its own copy
//      of the step below (one owner pattern per loop keeps the registers of
//      the three copies apart);
//   3. for every union entry, the K and V tiles stream from HBM straight into
//      LDS (buffer loads with an LDS destination, no registers involved),
//      double-buffered in two stages, one barrier per tile: the copy into one
//      stage runs during the other stage's step (runs of more than 64 entries,
//      dense-like pairs, wait for it before the stage-A step). 16-byte chunks are
//      XOR-swizzled per row through the per-lane source addresses, so both
//      operand reads below are bank-conflict free. Every wave computes the
//      64 x 16 S^T tile of each of its query tiles whose block keeps the
//      entry (so all four waves work on every entry) with 16x16x32 bf16
//      MFMAs, the online
//      softmax in base 2 with a lazily raised maximum (one query row per lane;
//      each lane tests its own scores against the row's limit, and two
//      permlane swaps reduce a row when one passes it), the row sums as an MFMA against a
//      ones operand, and O^T += V^T P^T with V^T operands read from the
//      row-major V tile by transposing LDS reads (ds_read_b64_tr_b16);
//      With the per-row (token-to-block) correction, the pooled tiles follow
//      through the same step: the next tile's key parts are copied during
//      this tile's O^T products, its values during the next score products;
//   4. exact state and correction merge under a common maximum; rows are
//      normalised and stored in fp32 (or rounded to bf16 on request). After
//      the last pair the next item's ticket is resolved before the stores and
//      the item boundary waits for LDS only, so the stores drain while the
//      next item starts (nothing in the kernel reads the output).
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
// Union runs longer than this wait for each stage-B copy before the stage-A
// step (see the kept loop).
constexpr int kLongRun = 64;
// s_waitcnt operand: vmcnt(0), expcnt and lgkmcnt left at their maxima
constexpr int kVmcnt0 = 0x0F70;
// max over the four lanes l, l^16, l^32, l^48 that share one query row
__device__ __forceinline__ float rowmax4(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Words of kept bits per query block: groups of eight or sixteen blocks are
// used up to 2048 key blocks, smaller groups up to the longest supported head.
template <int G>
constexpr int key_words() {
  return G >= 8 ? kMaxKeyBlocksG8 / 32 : (SOL_ATTN_MAX_N / kBlk) / 32;
}

// LDS geometry. A K or V tile is 64 rows of 2d bytes, stored unpadded with
// the 16-byte chunks of each row XOR-swizzled (kslot / vslot below); a stage
// holds one K tile and one V tile. Before the kept loop the two stages also
// hold the routing buffers of the group and the staged Q tiles.
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
// The source is row-major (row r's chunk c at r * RB + 16 c) or, TILED, in
// 16-row tiles stored chunk by chunk (at (r / 16) * 16 RB + (16 c + r % 16) * 16).
template <int D, bool KROWS, bool TILED = false>
__device__ __forceinline__ void dma_one(unsigned char* dst, rsrc_t r, int wid, int lane) {
  using G = Geom<D>;
  constexpr int LPR = G::RB / 16;
  const int row = (1024 * wid) / G::RB + lane / LPR, sl = lane % LPR;
  const int c = KROWS ? kslot<D>(row, sl) : vslot<D>(row, sl);
  const uint32_t o = TILED ? (row >> 4) * 16 * G::RB + (16 * c + (row & 15)) * 16 : row * G::RB + 16 * c;
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

// State of one group that outlives its routing pass (the kept loops of its
// pairs read it), plus the workgroup's small scratch.
template <int D, int G>
struct alignas(16) Small {
  float cnum[G][D];                 // correction numerators
  float cden[G];                    // correction denominators
  float M[G];                       // row maxima of the proxy scores (natural units)
  float theta[G];                   // Gaussian thresholds
  float wmax[4][16];                // per wave and column: maximum over the wave's first step
  float wfin[4][16];                // per wave and column: the wave's final maximum
  float wden[4][16];                // per wave and column: the wave's correction denominator
  uint32_t kbits[G][key_words<G>()];  // kept-block bits
  unsigned long long st64[3];  // this workgroup's stats: kept blocks, total blocks, kept token pairs
  unsigned st32[2];            // fewest and most kept blocks of a query block
  int item;  // the item of the next iteration (-1: none left)
  int pair;  // its one pair to process (-1: all of them)
  int last;  // this workgroup finished last
};

// The k-th step of the outward order that starts at step cs: cs, cs+1,
// cs-1, cs+2, ... (steps outside 0 .. nch-1 are left out).
__device__ __forceinline__ int chunk_at(int k, int cs, int nch) {
  // the k-th valid entry: first the symmetric part, then the longer side
  const int below = cs, above = nch - 1 - cs, sym = min(below, above);
  if (k <= 2 * sym) return k == 0 ? cs : ((k & 1) ? cs + (k + 1) / 2 : cs - k / 2);
  const int rest = k - 2 * sym;  // 1, 2, ... on the longer side
  return above > below ? cs + sym + rest : cs - sym - rest;
}

// RC: the per-row (token-to-block) correction replaces the block-level one.
// RO: routing only (the threshold router): the kernel stops after each
// group's routing pass and writes the kept bits; without the kept loop it
// needs a fraction of the registers and LDS, so four workgroups share a CU.
template <int D, int G, bool RC, bool RO>
__global__ __launch_bounds__(kThreads, RO ? 4 : 2) void fwd_kernel(FwdParams p) {
  using GM = Geom<D>;
  // Two separate LDS objects for the two stages, so that reads of one stage
  // never wait for copies still landing in the other.
  constexpr int kStA = RO ? G * D * 4 : GM::STAGE, kStB = RO ? 4 * G * D * 4 : GM::STAGE;
  __shared__ __attribute__((aligned(16))) unsigned char stA[kStA];
  __shared__ __attribute__((aligned(16))) unsigned char stB[kStB];
  __shared__ Small<D, G> sm;
  constexpr int KW = key_words<G>();
  // routing buffers in the stages (before any pair's kept loop):
  //   stA: qbar[G][D] pooled queries
  //   stB: [4][G][D] per-wave partial sums (pooled queries, Gaussian
  //        statistics, correction numerators)
  static_assert(G * D * 4 <= kStA, "routing buffers exceed stage A");
  static_assert(4 * G * D * 4 <= kStB, "routing buffers exceed stage B");
  float* qbar = reinterpret_cast<float*>(stA);
  float* part = reinterpret_cast<float*>(stB);  // [4 waves][G][D]

  const int Nk = p.Nk, N = p.N, Nq = p.Nq;
  constexpr int NDS = D / 32;  // k-steps of S^T along d
  constexpr int NDT = D / 16;  // 16-row tiles of O^T along d
  constexpr int CH = D / 8;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int g16 = lane >> 4, c16 = lane & 15;
  // wave w serves rows 16w .. 16w + 15 of both blocks of a pair: query tile
  // 0 of the first block, query tile 1 of the second
  const int qrow0 = 16 * wid;
  const int nlast = N - (Nk - 1) * kBlk;
  const float csc = p.scale_log2;
  const bool rowmax = p.rule == SOL_ROUTE_ROWMAX;
  // block-level correction sums are formed (not in the per-row or exact-only modes)
  const bool corr = !RC && !RO && !p.exact_only;
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
  // Work units: an item (all its pairs) or one pair of an item, which is
  // then routed once for each of its pairs taken so (so that the finish of
  // the grid is set by pairs rather than by whole heavy items). With a plan
  // made for this many items, queue x's tickets index its units; a plan made
  // for another group size is ignored and the items go in sequence. A unit
  // past the items, possible only with a workspace that was never planned,
  // ends this workgroup's work instead of being followed. Without a plan,
  // the last split_n items of each queue are handed out pair by pair.
  constexpr int HP = G / 2;  // pairs per item
  const unsigned* units = p.units != nullptr && *p.plan_items == (unsigned)p.nitems ? p.units : nullptr;
  // the item of ticket t (or -1 when every queue is drained) and its pair
  // (-1: all); a split-off pair that the head's last, partial group does not
  // have is passed over
  auto take = [&](unsigned t, int& pair) -> int {
    for (;;) {
      const int x = (home + qcur) & (kQueues - 1);
      const int lo = queue_begin(x, p.nitems), n = queue_begin(x + 1, p.nitems) - lo;
      pair = -1;
      int it = -1;
      bool here = false;
      if (units) {
        if (t < p.plan_items[8 + x]) {
          const unsigned u = units[(size_t)lo * HP + t];
          const unsigned pb = HP >= 2 ? u >> 28 : 0u;
          it = (int)(HP >= 2 ? u & 0x0fffffffu : u);
          pair = (int)pb - 1;
          here = true;
        }
      } else {
        const int a = HP >= 2 && p.split_n > 0 ? max(0, n - p.split_n) : n;  // split ranks [a, n)
        if (t < (unsigned)(a + HP * (n - a))) {
          if (t < (unsigned)a) {
            it = lo + (int)t;
          } else {
            it = lo + a + (int)(t - a) / HP;
            pair = (int)(t - a) % HP;
          }
          here = true;
        }
      }
      if (here) {
        if (it < 0 || it >= p.nitems) {
          pair = -1;
          return -1;
        }
        if (pair >= 0 && G * (it % p.ngroups) + 2 * pair >= p.Nq) {
          t = ticket();
          continue;
        }
        return it;
      }
      if (++qcur >= kQueues) {
        pair = -1;
        return -1;
      }
      t = ticket();
    }
  };
  // per-workgroup stats, published once at the end (thread 0's registers)
  // (in LDS, thread 0's, so that nothing of them is held in registers
  // through the kept loops)
  if (tid == 0) {
    sm.st64[0] = sm.st64[1] = sm.st64[2] = 0ull;
    sm.st32[0] = 0xffffffffu;
    sm.st32[1] = 0u;
  }

  if (tid == 0) {
    int pr = -1;
    sm.item = p.static_grid ? (int)blockIdx.x : take(ticket(), pr);
    sm.pair = pr;
  }
  __syncthreads();
  for (;;) {
    const int item = sm.item;
    if (item < 0) break;
    const int ipair = sm.pair;  // (read before the next item's ticket overwrites it)
    const int bh = item / p.ngroups;  // head-major: neighbouring groups are consecutive tickets
    const int g0 = G * (item - bh * p.ngroups);
    const size_t hoff = (size_t)bh * N * D;
    // The thread index passes through an empty asm statement, so that the
    // per-lane offsets of the routing pass are formed for each item instead
    // of being hoisted out of the item loop and held (or spilled) through the
    // kept loops.
    int tid_i = tid;
    asm volatile("" : "+v"(tid_i));
    const int tid = tid_i, lane = tid_i & 63;

    // routing geometry and the operands of this wave's first step, whose
    // loads are issued before the pooled queries are formed
    constexpr int CT = D / 16;   // 16-column tiles of the pooled values
    constexpr int NQB = D / 32;  // k-steps of a score tile
    // G = 16: every column of a score tile is a block of the group, one
    // product per part of the pooled queries; G = 6 or 8: the queries' third
    // part in a second product; G <= 4: all three parts in one.
    constexpr bool kFull = G == 16;
    constexpr bool kTwoCols = G > 5 && !kFull;
    const int col = lane & 15, kq = lane >> 4;
    const int nst = (Nk + 15) / 16;
    const int cs = min(g0 / 16, nst - 1);
    const bool gval = col < G && g0 + col < Nq;  // this lane's column is a score of a block of the group
    uint16_t* kb16 = reinterpret_cast<uint16_t*>(&sm.kbits[0][0]);  // 16 kept bits per step
    f32x4 accv[CT];
#pragma unroll
    for (int ci = 0; ci < CT; ++ci) accv[ci] = f32x4{0.f, 0.f, 0.f, 0.f};
    float Mw = -INFINITY;  // the wave's running maximum of column col's scores
    float cdl = 0.f;       // this lane's share of the correction denominator
    int nseq = 0;          // steps this wave has routed
    int nlow = 0;          // of them, the ones routed before Mw reached its current value
    // the operand planes of the head: 16-block tiles of 16 * D bf16, stored
    // in operand order (a wave's load is one contiguous stretch)
    const size_t tplane = (size_t)bh * p.Nkp * D;
    const uint32_t tbytes = (uint32_t)p.Nkp * D * 2;
    constexpr uint32_t kTile = 16 * D * 2;
    const rsrc_t rk0 = make_rsrc(p.khi16 + tplane, tbytes);
    const rsrc_t rk1 = make_rsrc(p.klo16 + tplane, tbytes);
    const rsrc_t rk2 = make_rsrc(p.klo2 + tplane, tbytes);
    const rsrc_t rv = make_rsrc(corr ? p.vt + tplane : p.khi16, corr ? tbytes : 0u);
    // operands of a step: the key parts (each k-step's loaded for the next
    // step as soon as this step's products have taken it) and the values
    // (loaded when the step starts; first used after its scores)
    struct StepOps {
      bf16x8 k[3][NQB];  // rows col, 8-column chunks 4 ks + kq of the three key parts
    };
    struct StepVals {
      i16x4 v[CT];  // column 16 ci + col of the values, key blocks 4 kq .. +3
    };
    auto load_ks = [&](StepOps& b, int st, int ks) {
      const int o = st * (int)kTile + 16 * lane + 1024 * ks;
      b.k[0][ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rk0, o, 0, 0));
      b.k[1][ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rk1, o, 0, 0));
      b.k[2][ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rk2, o, 0, 0));
    };
    auto load_step = [&](StepOps& b, int st) {
#pragma unroll
      for (int ks = 0; ks < NQB; ++ks) load_ks(b, st, ks);
    };
    auto load_vals = [&](StepVals& b, int st) {
      if (corr) {
        const int ov = st * (int)kTile + 8 * lane;
#pragma unroll
        for (int ci = 0; ci < CT; ++ci)
          b.v[ci] = __builtin_bit_cast(i16x4, __builtin_amdgcn_raw_buffer_load_b64(rv, ov, 512 * ci, 0));
      }
    };
    const int stEnd = p.Nkp / 16;
    auto step_of = [&](int kk) { return kk < nst ? chunk_at(kk, cs, nst) : stEnd; };

    // ---- A. pooled queries of the G blocks (from the pooling pre-pass); Gaussian thresholds ----
    {
      // routing state of the group
      if (tid < G) sm.M[tid] = -INFINITY;
      for (int w = tid; w < G * KW; w += kThreads) (&sm.kbits[0][0])[w] = 0u;
      for (int idx = tid; idx < G * D; idx += kThreads) {
        const int g = idx / D, c = idx % D;
        qbar[idx] = g0 + g < Nq ? p.qpool[((size_t)bh * Nq + g0 + g) * D + c] : 0.f;
      }
      __syncthreads();  // pooled queries complete

      // Gaussian thresholds theta = mu + beta sigma, known before any score
      // (§3 "Dynamic threshold routing"; App. B): mu = qbar . m_K / sqrt(d),
      // sigma^2 = qbar^T C_K qbar / d (pooled-key covariance, SOL_ROUTE_GAUSS)
      // or sum_c qbar_c^2 v_Kc / d (its diagonal, SOL_ROUTE_GAUSS_DIAG)
      if (!rowmax) {
        float a[G], b[G];
#pragma unroll
        for (int g = 0; g < G; ++g) a[g] = b[g] = 0.f;
        if (tid < D) {
          if (p.rule == SOL_ROUTE_GAUSS_DIAG) {
            const float mu = p.kstats[(size_t)bh * 2 * D + tid];
            const float var = p.kstats[(size_t)bh * 2 * D + D + tid];
#pragma unroll
            for (int g = 0; g < G; ++g) {
              const float x = qbar[g * D + tid];
              a[g] = x * mu;
              b[g] = x * x * var;
            }
          } else {
            const float mu = p.kmom[(size_t)bh * (D + 1) * D + tid];
            // row tid of C_K against every pooled query: y_g = (C_K qbar_g)[tid]
            const float* crow = p.kmom + (size_t)bh * (D + 1) * D + (size_t)(1 + tid) * D;
            float y[G];
#pragma unroll
            for (int g = 0; g < G; ++g) y[g] = 0.f;
            for (int c = 0; c < D; c += 4) {
              const float4 cv = *reinterpret_cast<const float4*>(crow + c);
#pragma unroll
              for (int g = 0; g < G; ++g) {
                const float4 qv = *reinterpret_cast<const float4*>(&qbar[g * D + c]);
                y[g] += cv.x * qv.x + cv.y * qv.y + cv.z * qv.z + cv.w * qv.w;
              }
            }
#pragma unroll
            for (int g = 0; g < G; ++g) {
              const float x = qbar[g * D + tid];
              a[g] = x * mu;
              b[g] = x * y[g];
            }
          }
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
          a[g] = wave_sum(a[g]);
          b[g] = wave_sum(b[g]);
        }
        if (lane == 0) {
#pragma unroll
          for (int g = 0; g < G; ++g) {
            part[(wid * G + g) * 2] = a[g];
            part[(wid * G + g) * 2 + 1] = b[g];
          }
        }
        __syncthreads();
        if (tid < G) {
          float sa = 0.f, sb = 0.f;
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            sa += part[(w * G + tid) * 2];
            sb += part[(w * G + tid) * 2 + 1];
          }
          const float inv_d = p.proxy_scale * p.proxy_scale;
          sm.theta[tid] = sa * p.proxy_scale + p.beta * sqrtf(fmaxf(sb * inv_d, 0.f));
        }
        __syncthreads();
      }
    }

    // ---- R. the routing pass over the pooled keys and values ----
    // Both products run on the matrix cores; lane l = col + 16 kq supplies
    // row col of A and column col of B, and holds rows 4kq .. 4kq+3 of column
    // col of the result:
    //   scores  S^T[j][col] = sum_p kbar_p[j] . B[col] (16x16x32), the pooled
    //           keys as three bf16 parts against the pooled queries as three
    //           parts in the columns of B, [qh | qm | ql] (G <= 4) or [qh | qm]
    //           and [ql | 0] (G = 6 or 8, kh only, the products below 2^-24
    //           left out); a block's score is the sum of its columns, an
    //           fp32-grade dot product;
    //   numerators cnum^T[c][col] = sum_j vbar^T[c][j] W[j][col] (16x16x16),
    //           the pooled values in bf16 against the weights of the skipped
    //           blocks in two parts, columns [wh | wl]. The score tile's result
    //           layout is the weight operand's layout, so the weights never
    //           leave the lanes that form them.
    // The key blocks are cut into 16-block steps, taken outwards from the
    // group's own blocks; wave w takes every fourth step and streams on its own
    // (the next step's operands load while the current one is used), the
    // waves merging at the end. Each wave keeps a running maximum per block
    // and a correction against it (earlier terms rescaled when it rises).
    // Gaussian rules: the threshold is known, so every decision is final when
    // made. Row-max rule: a block is kept while its score is within tau of the
    // running maximum; the maximum over the first step of every wave (the 64
    // key blocks nearest the group's own) is taken before any decision, and
    // once the true maximum is known, the blocks kept before the wave's
    // maximum reached it are checked again (only where it rose after that
    // first step, which the order makes rare) and the ones that fall below
    // move to the correction.
    {
      // score B operands, from the pooled queries in LDS
      bf16x8 qB1[NQB], qB2[NQB], qB3[kFull ? NQB : 1];
      {
        const int qp = kFull ? 0 : col / G;  // which part of the pooled query
        const int g = kFull ? col : col % G;
        const bool on1 = kFull || col < (kTwoCols ? 2 : 3) * G;
        const bool on2 = kFull || (kTwoCols && col < G);
#pragma unroll
        for (int ks = 0; ks < NQB; ++ks) {
          uint32_t w1[4], w2[4], w3[4];
#pragma unroll
          for (int i = 0; i < 8; i += 2) {
            float h[2], m[2], l[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              const float x = qbar[g * D + 32 * ks + 8 * kq + i + e];
              h[e] = __uint_as_float(pack_bf16x2(x, 0.f) << 16);
              const float r1 = x - h[e];
              m[e] = __uint_as_float(pack_bf16x2(r1, 0.f) << 16);
              l[e] = __uint_as_float(pack_bf16x2(r1 - m[e], 0.f) << 16);
            }
            const float* pick = qp == 0 ? h : qp == 1 ? m : l;
            w1[i / 2] = on1 ? pack_bf16x2(pick[0], pick[1]) : 0u;
            w2[i / 2] = on2 ? (kFull ? pack_bf16x2(m[0], m[1]) : pack_bf16x2(l[0], l[1])) : 0u;
            w3[i / 2] = pack_bf16x2(l[0], l[1]);
          }
          qB1[ks] = as_bf16x8(make_uint4(w1[0], w1[1], w1[2], w1[3]));
          qB2[ks] = as_bf16x8(make_uint4(w2[0], w2[1], w2[2], w2[3]));
          if constexpr (kFull) qB3[ks] = as_bf16x8(make_uint4(w3[0], w3[1], w3[2], w3[3]));
        }
      }
      // the step's scores of column col's block, key blocks 16 st + 4 kq + e;
      // the operands of step stn are loaded into b meanwhile (stn = stEnd, a
      // tile past the plane, reads zeros without touching memory)
      auto step_scores = [&](StepOps& b, int st, float (&sc)[4], int stn) {
        f32x4 s1 = {0.f, 0.f, 0.f, 0.f}, s2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NQB; ++ks) {
          s1 = mfma16x16x32(b.k[0][ks], qB1[ks], s1);
          s1 = mfma16x16x32(b.k[1][ks], qB1[ks], s1);
          s1 = mfma16x16x32(b.k[2][ks], qB1[ks], s1);
          if constexpr (kFull) {
            s2 = mfma16x16x32(b.k[0][ks], qB2[ks], s2);
            s2 = mfma16x16x32(b.k[1][ks], qB2[ks], s2);
            s2 = mfma16x16x32(b.k[2][ks], qB2[ks], s2);
            s2 = mfma16x16x32(b.k[0][ks], qB3[ks], s2);
          } else if constexpr (kTwoCols) {
            s2 = mfma16x16x32(b.k[0][ks], qB2[ks], s2);
          }
          load_ks(b, stn, ks);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // lane col g < G gathers its block's columns (g + G and g + 2G, or
          // g + G and column g of the second product; with G = 16 the two
          // products' own column)
          float v = s1[e];
          if constexpr (kFull)
            v += s2[e];
          else if constexpr (kTwoCols)
            v += __shfl_down(s1[e], G, 16) + s2[e];
          else
            v += __shfl_down(s1[e], G, 16) + __shfl_down(s1[e], 2 * G, 16);
          sc[e] = gval && 16 * st + 4 * kq + e < Nk ? v * p.proxy_scale : -INFINITY;
        }
      };
      // correction weights w[e] (relative to Mw) of the step into the
      // numerators, after rescaling them by alpha (per column)
      auto accumulate = [&](const StepVals& b, const float (&w)[4], float alpha) {
        uint32_t hp[2], lp[2];
#pragma unroll
        for (int e = 0; e < 4; e += 2) {
          const float h0 = __uint_as_float(pack_bf16x2(w[e], 0.f) << 16);
          const float h1 = __uint_as_float(pack_bf16x2(w[e + 1], 0.f) << 16);
          hp[e / 2] = pack_bf16x2(h0, h1);
          lp[e / 2] = pack_bf16x2(w[e] - h0, w[e + 1] - h1);
        }
        if constexpr (kFull) {
          // every column is a block: the high parts and the remainders in two
          // products into the same numerators
          const i16x4 wH = __builtin_bit_cast(i16x4, make_uint2(hp[0], hp[1]));
          const i16x4 wL = __builtin_bit_cast(i16x4, make_uint2(lp[0], lp[1]));
          if (__ballot(alpha != 1.f)) {
#pragma unroll
            for (int ci = 0; ci < CT; ++ci) accv[ci] *= alpha;
          }
#pragma unroll
          for (int ci = 0; ci < CT; ++ci) {
            accv[ci] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(b.v[ci], wH, accv[ci], 0, 0, 0);
            accv[ci] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(b.v[ci], wL, accv[ci], 0, 0, 0);
          }
        } else {
          // column col of the weight operand: the high parts of block col
          // (col < G), the remainders of block col - G (G <= col < 2G), else 0
          const uint32_t l0 = __shfl_up(lp[0], G, 16), l1 = __shfl_up(lp[1], G, 16);
          const uint32_t b0 = col < G ? hp[0] : col < 2 * G ? l0 : 0u;
          const uint32_t b1 = col < G ? hp[1] : col < 2 * G ? l1 : 0u;
          const i16x4 wB = __builtin_bit_cast(i16x4, make_uint2(b0, b1));
          if (__ballot(alpha != 1.f)) {
            const float ar = __shfl_up(alpha, G, 16);
            const float al = col < G ? alpha : col < 2 * G ? ar : 1.f;
#pragma unroll
            for (int ci = 0; ci < CT; ++ci) accv[ci] *= al;
          }
#pragma unroll
          for (int ci = 0; ci < CT; ++ci)
            accv[ci] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(b.v[ci], wB, accv[ci], 0, 0, 0);
        }
      };
      // the 16 kept bits of column col's block in the step: OR over its four lanes
      auto or4 = [](uint32_t x) {
        const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
        x = a[0] | a[1];
        const auto c = __builtin_amdgcn_permlane32_swap(x, x, false, false);
        return c[0] | c[1];
      };
      const float thg = !rowmax && col < G ? sm.theta[col] : 0.f;
      // route one step whose scores are sc
      auto route_step = [&](const StepVals& b, int st, const float (&sc)[4]) {
        // (selects rather than branches: every lane evaluates the same
        // instructions, and the exponentials of dropped lanes are discarded)
        const float smax = rowmax4(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])));
        const bool raised = smax > Mw;
        const float alpha = raised ? __builtin_amdgcn_exp2f((Mw - smax) * kLog2e) : 1.f;  // 0 on the first raise from -inf
        Mw = raised ? smax : Mw;
        nlow = raised ? nseq : nlow;
        const float th = rowmax ? Mw - p.tau : thg;
        uint32_t bits = 0u;
        float w[4], wsum = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = 16 * st + 4 * kq + e;
          const bool valid = gval && j < Nk;
          const bool sink = (unsigned)(j - p.sink_lo) < (unsigned)(p.sink_hi - p.sink_lo);
          const bool keep = valid && (sc[e] >= th || sink);
          const float ev = __builtin_amdgcn_exp2f((sc[e] - Mw) * kLog2e);
          w[e] = corr && valid && !keep ? (float)min(kBlk, N - j * kBlk) * ev : 0.f;
          wsum += w[e];
          bits |= (keep ? 1u : 0u) << (4 * kq + e);
        }
        cdl = cdl * alpha + wsum;
        bits = or4(bits);
        if (lane < G && gval) kb16[col * 2 * KW + st] = (uint16_t)bits;
        if (corr) accumulate(b, w, alpha);
        ++nseq;
      };

      // the wave's steps: the scores of the next step (and the loads of the
      // one after) are formed at the end of each iteration
      // (a wave with no step loads the tile past the planes: zeros, no traffic,
      // and scores of -inf)
      float sc[4];
      int k = wid;
      StepOps b;
      StepVals vv;
      load_vals(vv, step_of(k));
      load_step(b, step_of(k));
      step_scores(b, step_of(k), sc, step_of(k + 4));
      if (rowmax) {
        // the maximum over the first step of every wave, before any decision
        const float mx = rowmax4(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])));
        if (lane < 16) sm.wmax[wid][lane] = mx;
        __syncthreads();
        Mw = fmaxf(fmaxf(sm.wmax[0][col], sm.wmax[1][col]), fmaxf(sm.wmax[2][col], sm.wmax[3][col]));
      }
      // (the values of step k + 4 load a whole iteration ahead of their use)
      for (; k < nst; k += 4) {
        StepVals vn;
        if (k + 4 < nst) load_vals(vn, step_of(k + 4));
        route_step(vv, step_of(k), sc);
        if (k + 4 < nst) {
          step_scores(b, step_of(k + 4), sc, step_of(k + 8));
          vv = vn;
        }
      }
      if (lane < 16) sm.wfin[wid][lane] = Mw;
      __syncthreads();  // every wave's maximum is final

      if (rowmax) {
        // blocks kept against a lower maximum than the row's: the steps this
        // wave routed before its maximum reached the row's (all of them if it
        // never did) are routed again against the row's maximum. The scores
        // come out bit for bit as before, so a block is only ever dropped.
        const float M = fmaxf(fmaxf(sm.wfin[0][col], sm.wfin[1][col]), fmaxf(sm.wfin[2][col], sm.wfin[3][col]));
        const int need = gval ? (Mw == M ? nlow : nseq) : 0;
        const int nneed = (int)wave_max((float)need);
        const float thM = M - p.tau;
        for (int i = 0; i < nneed; ++i) {
          const int st = chunk_at(wid + 4 * i, cs, nst);
          const uint32_t old = i < need ? kb16[col * 2 * KW + st] : 0u;
          if (!__ballot(old != 0u)) continue;
          StepOps b;
          StepVals vv;
          load_step(b, st);
          load_vals(vv, st);
          float s2[4];
          step_scores(b, st, s2, stEnd);
          uint32_t drop = 0u;
          float w[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int bit = 4 * kq + e, j = 16 * st + bit;
            const bool sink = (unsigned)(j - p.sink_lo) < (unsigned)(p.sink_hi - p.sink_lo);
            const bool dr = ((old >> bit) & 1u) && !(s2[e] >= thM || sink);
            w[e] = corr && dr ? (float)min(kBlk, N - j * kBlk) * __expf(s2[e] - Mw) : 0.f;
            cdl += w[e];
            drop |= (dr ? 1u : 0u) << bit;
          }
          drop = or4(drop);
          if (lane < G && old != 0u) kb16[col * 2 * KW + st] = (uint16_t)(old & ~drop);
          if (corr) accumulate(vv, w, 1.f);
        }
      }
    }

    // ---- R4. the waves' partial sums merged; the group's routing is final ----
    {
      float cd = cdl;
      cd += __shfl_xor(cd, 16);
      cd += __shfl_xor(cd, 32);
      if (lane < 16) sm.wden[wid][lane] = cd;
    }
    __syncthreads();
    {
      // the group's maximum M of each block, and this wave's factor e^{Mw - M}
      // for its partial sums (0 for a wave that saw none of the block's scores)
      // the block of column col (columns < 2G; with G = 16 the column itself)
      const int gc = kFull || col < G ? col : col - G;
      const float Mg = fmaxf(fmaxf(sm.wfin[0][gc], sm.wfin[1][gc]), fmaxf(sm.wfin[2][gc], sm.wfin[3][gc]));
      const float Mwc = sm.wfin[wid][gc];
      const float f = ((kFull || col < 2 * G) && Mwc > -INFINITY) ? __expf(Mwc - Mg) : 0.f;
      float* partc = reinterpret_cast<float*>(stB);  // [4 waves][G][D]
#pragma unroll
      for (int ci = 0; ci < CT; ++ci) {
        float4 cn;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x = accv[ci][e] * f;
          if constexpr (kFull)
            (&cn.x)[e] = x;
          else
            (&cn.x)[e] = x + __shfl_down(x, G, 16);  // high and remainder columns of block col
        }
        if (col < G) *reinterpret_cast<float4*>(&partc[(wid * G + col) * D + 16 * ci + 4 * kq]) = cn;
      }
      if (tid < G) {
        const float M = fmaxf(fmaxf(sm.wfin[0][tid], sm.wfin[1][tid]), fmaxf(sm.wfin[2][tid], sm.wfin[3][tid]));
        float cd = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float mw = sm.wfin[w][tid];
          cd += mw > -INFINITY ? sm.wden[w][tid] * __expf(mw - M) : 0.f;
        }
        sm.M[tid] = M;
        sm.cden[tid] = corr ? cd : 0.f;
      }
    }
    __syncthreads();
    for (int idx = tid; idx < G * D; idx += kThreads) {
      const int g = idx / D, c = idx % D;
      const float* partc = reinterpret_cast<const float*>(stB);
      sm.cnum[g][c] = corr ? (partc[(0 * G + g) * D + c] + partc[(1 * G + g) * D + c]) +
                                 (partc[(2 * G + g) * D + c] + partc[(3 * G + g) * D + c])
                           : 0.f;
    }
    __syncthreads();
    if (p.bitmap) {
      for (int idx = tid; idx < G * p.nwords; idx += kThreads) {
        const int g = idx / p.nwords, w = idx % p.nwords;
        if (g0 + g < Nq) p.bitmap[((size_t)bh * Nq + g0 + g) * p.nwords + w] = sm.kbits[g][w];
      }
    }
    if constexpr (RO) {
      if (p.static_grid) break;
      __syncthreads();
      if (tid == 0) {
        int pr = -1;
        sm.item = take(ticket(), pr);
        sm.pair = pr;
      }
      __syncthreads();
      continue;
    } else {

    // ---- the pairs of the group: Q tiles, union list, kept loop, fold ----
    const int pr_lo = ipair >= 0 ? ipair : 0, pr_hi = ipair >= 0 ? ipair + 1 : G / 2;
    for (int pr = pr_lo; pr < pr_hi; ++pr) {
      // The lane indices pass through an empty asm statement, so that the
      // kept loop's per-lane offsets are formed here for every pair instead of
      // being hoisted out of the item loop and held in registers through the
      // routing pass.
      int tid_ = tid;
      asm volatile("" : "+v"(tid_));
      const int tid = tid_, lane = tid_ & 63, g16 = lane >> 4, c16 = lane & 15;
      const int qA = g0 + 2 * pr;
      if (qA >= Nq) break;
      const int gA = 2 * pr;
      const bool hasB = qA + 1 < Nq;
      const bool lastpair = pr == pr_hi - 1 || qA + 2 >= Nq;
      const int nA = min(kBlk, N - qA * kBlk);
      const int nB = hasB ? min(kBlk, N - (qA + 1) * kBlk) : 0;

      // ---- 1. Q tiles -> LDS -> Q^T operands ----
      bf16x8 qop[2][NDS];
      {
        constexpr int PER = kBlk * CH / kThreads, RSTEP = kThreads / CH;
        const uint32_t qoff = ((tid / CH) * D + (tid % CH) * 8) * 2;
        uint4 qr[2][PER];
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
          const int nb = blk ? nB : nA;
          const rsrc_t r = make_rsrc(p.q + hoff + (size_t)min(qA + blk, Nq - 1) * kBlk * D, (uint32_t)nb * D * 2);
#pragma unroll
          for (int u = 0; u < PER; ++u) qr[blk][u] = ld16(r, qoff, u * RSTEP * D * 2);
        }
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
          uint16_t* qd = reinterpret_cast<uint16_t*>(blk ? stB : stA) + (tid / CH) * GM::QS + (tid % CH) * 8;
#pragma unroll
          for (int u = 0; u < PER; ++u) *reinterpret_cast<uint4*>(qd + u * RSTEP * GM::QS) = qr[blk][u];
        }
        __syncthreads();
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          const uint16_t* qs = reinterpret_cast<const uint16_t*>(qt ? stB : stA) + (qrow0 + c16) * GM::QS + 8 * g16;
#pragma unroll
          for (int ds = 0; ds < NDS; ++ds) qop[qt][ds] = as_bf16x8(*reinterpret_cast<const uint4*>(&qs[32 * ds]));
        }
      }

      // ---- 2. the union of the two kept lists, walked from the kept bits ----
      // No list is stored: the union is walked in three runs by owner (step
      // 3); at the start of a run every wave holds the run's kept-bit words
      // in its lanes (one word per lane) and a mask of the words that hold
      // entries, and walks them with wave-uniform scalar state. Wave 0
      // counts the pair's kept blocks for the stats.
      int run_len[3];  // union entries kept by both blocks, by the first only, by the second only
      {
        const int nw = (Nk + 31) / 32;
        // the lengths of the three runs (every wave; they pick the copy
        // schedule of each run, step 3)
        {
          int cboth = 0, cfirst = 0, csecond = 0;
          for (int w = lane; w < nw; w += 64) {
            const uint32_t a = sm.kbits[gA][w], b = hasB ? sm.kbits[gA + 1][w] : 0u;
            cboth += __popc(a & b);
            cfirst += __popc(a & ~b);
            csecond += __popc(b & ~a);
          }
          run_len[0] = __builtin_amdgcn_readfirstlane(wave_sum_int(cboth));
          run_len[1] = __builtin_amdgcn_readfirstlane(wave_sum_int(cfirst));
          run_len[2] = __builtin_amdgcn_readfirstlane(wave_sum_int(csecond));
        }
        if (wid == 0) {
          int ca = 0, cb = 0;
          for (int w = lane; w < nw; w += 64) {
            ca += __popc(sm.kbits[gA][w]);
            cb += hasB ? __popc(sm.kbits[gA + 1][w]) : 0;
          }
          const int nkA = wave_sum_int(ca), nkB = wave_sum_int(cb);
          if (lane == 0) {
            // this pair's stats (kept token pairs: the last key block has nlast tokens)
            const int jl = Nk - 1;
            const bool lastA = (sm.kbits[gA][jl >> 5] >> (jl & 31)) & 1u;
            const bool lastB = hasB && ((sm.kbits[gA + 1][jl >> 5] >> (jl & 31)) & 1u);
            const unsigned long long tokA = (unsigned long long)nkA * kBlk - (lastA ? kBlk - nlast : 0);
            const unsigned long long tokB = (unsigned long long)nkB * kBlk - (lastB ? kBlk - nlast : 0);
            sm.st64[0] += (unsigned long long)(nkA + (hasB ? nkB : 0));
            sm.st64[1] += (unsigned long long)Nk * (hasB ? 2 : 1);
            sm.st64[2] += tokA * (unsigned long long)nA + (hasB ? tokB * (unsigned long long)nB : 0ull);
            sm.st32[0] = min(sm.st32[0], hasB ? (unsigned)min(nkA, nkB) : (unsigned)nkA);
            sm.st32[1] = max(sm.st32[1], hasB ? (unsigned)max(nkA, nkB) : (unsigned)nkA);
          }
        }
        __syncthreads();  // every wave holds its Q operands: the stages are free
      }

      // ---- 3. exact attention over the union list (online softmax, base 2) ----
      f32x4 accO[2][NDT];
      f32x4 lsum[2];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        lsum[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) accO[qt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      float m[2] = {-INFINITY, -INFINITY};
      float mlim[2] = {-INFINITY, -INFINITY};  // m + kLazyRescale
      {
        const bf16x8 ones = as_bf16x8(make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u));
        const uint16_t* kh = p.k + hoff;
        const uint16_t* vh = p.v + hoff;
        // K and V tiles of the union entry e (key block e & 0x3fff) into one stage
        // (e < 0, past the end of a run: an empty copy, every load out of range,
        // so that a copy can be issued without a branch around it)
        auto dma = [&](unsigned char* stage, int e) {
          const int j = e < 0 ? 0 : e & 0x3fff;
          const uint32_t bytes = e < 0 ? 0u : (uint32_t)min(kBlk, N - j * kBlk) * D * 2;
          dma_tile<D>(stage, make_rsrc(kh + (size_t)j * kBlk * D, bytes), make_rsrc(vh + (size_t)j * kBlk * D, bytes),
                      wid, lane);
        };
        // pooled tile c (per-row correction): the two bf16 parts of the pooled
        // keys fill stage A (both as K rows), the pooled values stage B's V half
        // pooled tile c (per-row correction): the two bf16 parts of the pooled
        // keys into stage A (both as K rows), the pooled values into stage B's
        // V half. c = npool: empty copies (every load out of range), so that
        // no branch separates a copy from the reads after it.
        const int npool = (Nk + kBlk - 1) / kBlk;
        auto dma_pooled_keys = [&](int c) {
          // (the tiled key planes hold zeros past Nk)
          const bool on = c < npool;
          const size_t toff = ((size_t)bh * p.Nkp + (size_t)(on ? c : 0) * kBlk) * D;
          dma_one<D, true, true>(stA, make_rsrc(p.khi16 + toff, on ? GM::TILE : 0u), wid, lane);
          dma_one<D, true, true>(stA + GM::TILE, make_rsrc(p.klo16 + toff, on ? GM::TILE : 0u), wid, lane);
        };
        auto dma_pooled_vals = [&](int c) {
          // (the row-major values are bounded)
          const bool on = c < npool;
          const uint32_t bytes = on ? (uint32_t)min(kBlk, Nk - c * kBlk) * D * 2 : 0u;
          const size_t off = ((size_t)bh * Nk + (size_t)(on ? c : 0) * kBlk) * D;
          dma_one<D, false>(stB + GM::TILE, make_rsrc(p.vbar16 + off, bytes), wid, lane);
        };
        // per-lane byte offsets of the swizzled operand reads (independent of the key tile kt)
        int koffs[NDS];
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) koffs[ds] = c16 * GM::RB + 16 * kslot<D>(c16, 4 * ds + g16);
        // transposing V reads: this lane addresses row 4g + e (+32ks +16h) and the
        // 8 bytes of columns 16dt + 4cc .. +3
        const int ve = (lane >> 2) & 3, vcc = lane & 3, vrow = 4 * g16 + ve;
        int voffs[NDT];
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
          voffs[dt] = GM::TILE + vrow * GM::RB + 16 * vslot<D>(vrow, 2 * dt + (vcc >> 1)) + 8 * (vcc & 1);

        // QM: the query tiles that take part (bit 0: the first block's, bit
        // 1: the second's), i.e. the blocks of the pair that keep the entry;
        // a tile that does not take part costs nothing
        // mid(): called between the probabilities and the O^T products (the
        // pooled tiles' copy schedule; nothing for the exact tiles)
        auto compute = [&](const unsigned char* stage, int e, auto pooled, auto qmask, auto mid) __attribute__((always_inline)) {
          constexpr bool kPooled = decltype(pooled)::value;
          constexpr int QM = decltype(qmask)::value;
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
            return as_bf16x8(*reinterpret_cast<const uint4*>(stage + 16 * (i / NDS) * GM::RB + koffs[i % NDS]));
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
              if (QM & 1) st[0][kt] = mfma16x16x32(a, qop[0][ds], st[0][kt]);
              if (QM & 2) st[1][kt] = mfma16x16x32(a, qop[1][ds], st[1][kt]);
              __builtin_amdgcn_sched_barrier(0);
              if (kPooled) {  // the remainder part of the pooled keys, one tile further on
                const bf16x8 b =
                    as_bf16x8(*reinterpret_cast<const uint4*>(stage + GM::TILE + 16 * kt * GM::RB + koffs[ds]));
                st[0][kt] = mfma16x16x32(b, qop[0][ds], st[0][kt]);
                st[1][kt] = mfma16x16x32(b, qop[1][ds], st[1][kt]);
              }
            }
          }
          // lane holds S^T[16kt + 4g + i][row c16 of query tile qt]
          if (kPooled) {
            // pooled key 64e + 16kt + 4g + i: masked for a query tile when
            // kept by its block (it is in the exact branch) or past Nk;
            // otherwise its weight n_j enters as log2(n_j) on the base-2 logit,
            // added here in raw dot-product units (n_j = 64 but for the ragged
            // last block)
            const int valid = Nk - e * kBlk;
            const int last = Nk - 1 - e * kBlk - 4 * g16;  // lane position of the last block, if here
#pragma unroll
            for (int qt = 0; qt < 2; ++qt) {
              const uint32_t* kb = sm.kbits[gA + qt];
              uint64_t offb = (uint64_t)kb[2 * e] | ((uint64_t)kb[2 * e + 1] << 32);
              if (valid < kBlk) offb |= ~0ull << valid;
              offb >>= 4 * g16;
#pragma unroll
              for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                  const bool masked = (offb >> (16 * kt + i)) & 1ull;
                  st[qt][kt][i] += masked ? -INFINITY : 16 * kt + i == last ? pbias_last : pbias;
                }
            }
          } else if (nj < kBlk) {
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                if (16 * kt + 4 * g16 + i >= nj) {
                  st[0][kt][i] = -INFINITY;
                  st[1][kt][i] = -INFINITY;
                }
          }
          // The lazily raised maximum: each lane compares the maximum of its own
          // 16 scores with its row's limit m + kLazyRescale (a row's maximum
          // passes the limit iff one of its four lanes' does); the rows' maxima
          // are formed, and the state rescaled, only when some row of the wave
          // passes its limit.
          bool raise = false;
          float lm[2];
#pragma unroll
          for (int qt = 0; qt < 2; ++qt) {
            if (!((QM >> qt) & 1)) continue;
            // two chains of three-input maxima over the lane's 16 scores
            float b0 = fmaxf(fmaxf(st[qt][0][0], st[qt][0][1]), st[qt][0][2]);
            float b1 = fmaxf(fmaxf(st[qt][2][0], st[qt][2][1]), st[qt][2][2]);
            b0 = fmaxf(fmaxf(b0, st[qt][0][3]), st[qt][1][0]);
            b1 = fmaxf(fmaxf(b1, st[qt][2][3]), st[qt][3][0]);
            b0 = fmaxf(fmaxf(b0, st[qt][1][1]), st[qt][1][2]);
            b1 = fmaxf(fmaxf(b1, st[qt][3][1]), st[qt][3][2]);
            b0 = fmaxf(b0, st[qt][1][3]);
            b1 = fmaxf(b1, st[qt][3][3]);
            lm[qt] = fmaxf(b0, b1);
            raise = raise || (lm[qt] * csc > mlim[qt]);
          }
          if (__ballot(raise)) {  // rare: a row's max rose by more than the lazy margin
#pragma unroll
            for (int qt = 0; qt < 2; ++qt) {
              if (!((QM >> qt) & 1)) continue;
              const float bm = rowmax4(lm[qt]) * csc;
              const float mn = bm > mlim[qt] ? bm : m[qt];
              const float alpha = __builtin_amdgcn_exp2f(m[qt] - mn);
              lsum[qt] *= alpha;
#pragma unroll
              for (int dt = 0; dt < NDT; ++dt) accO[qt][dt] *= alpha;
              m[qt] = mn;
              mlim[qt] = mn + kLazyRescale;
            }
          }
          // P^T operand slots 0-3 = keys 32ks+4g+i, slots 4-7 = keys 32ks+16+4g+i
          bf16x8 pb[2][2];
#pragma unroll
          for (int qt = 0; qt < 2; ++qt) {
            if (!((QM >> qt) & 1)) continue;
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
          // slots; each V^T operand serves the query tiles that take part
          const unsigned char* vstage = kPooled ? stB : stage;
          mid();
          // the O^T products in 16 slices t = 16 rows of d (dt = t % NDT) x 32 keys
          // (ks = t / NDT), each accumulator taking its two key steps in order;
          // the V^T operands of slice t + VA are read while slice t's MFMAs run
          auto vread = [&](int t, uint2 (&o)[2]) {
            const int dt = t % NDT, ks = t / NDT;
            o[0] = ld_tr(vstage + voffs[dt] + 32 * ks * GM::RB);
            o[1] = ld_tr(vstage + voffs[dt] + (32 * ks + 16) * GM::RB);
          };
          constexpr int VA = 3;
          constexpr int NT = 2 * NDT;
          uint2 vo[NT][2];
#pragma unroll
          for (int t = 0; t < VA; ++t) vread(t, vo[t]);
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            if (t + VA < NT) vread(t + VA, vo[t + VA]);
            __builtin_amdgcn_sched_barrier(0);
            const int dt = t % NDT, ks = t / NDT;
            const bf16x8 a = as_bf16x8(make_uint4(vo[t][0].x, vo[t][0].y, vo[t][1].x, vo[t][1].y));
            if (QM & 1) accO[0][dt] = mfma16x16x32(a, pb[0][ks], accO[0][dt]);
            if (QM & 2) accO[1][dt] = mfma16x16x32(a, pb[1][ks], accO[1][dt]);
            __builtin_amdgcn_sched_barrier(0);
          }
        };

        // The union in three runs, one per owner pattern (kept by both
        // blocks, by the first only, by the second only), each walked in
        // ascending order with wave-uniform scalar state: the next entry
        // j | A << 14 | B << 15, or -1 past the end. Every value here is the
        // same in all lanes of all waves, so the barriers stay matched.
        using kBoth = std::integral_constant<int, 3>;
        using kFirst = std::integral_constant<int, 1>;
        using kSecond = std::integral_constant<int, 2>;
        auto run = [&](auto qmask) __attribute__((always_inline)) {
          constexpr int QM = decltype(qmask)::value;
          // this run's kept-bit words: lane l holds word l (and word 64 + l in
          // the second register), so the walk takes a word with one lane read
          // and visits only the words that hold entries of this run
          const int nw = (Nk + 31) / 32;
          auto run_word = [&](int w) -> uint32_t {
            if (w >= nw) return 0u;
            const uint32_t a = sm.kbits[gA][w], b = hasB ? sm.kbits[gA + 1][w] : 0u;
            return QM == 3 ? (a & b) : QM == 1 ? (a & ~b) : (b & ~a);
          };
          const uint32_t rw0 = run_word(lane);
          const uint32_t rw1 = KW > 64 ? run_word(64 + lane) : 0u;
          uint64_t m0 = __ballot(rw0 != 0u), m1 = KW > 64 ? __ballot(rw1 != 0u) : 0ull;
          uint32_t rem = 0u;
          int wbase = 0;
          auto next = [&]() __attribute__((always_inline)) -> int {
            if (rem == 0u) {
              const bool lo = m0 != 0ull;
              const uint64_t m = lo ? m0 : m1;
              if (m == 0ull) return -1;
              const int l = (int)__builtin_ctzll(m);
              const uint64_t m2 = m & (m - 1ull);
              m0 = lo ? m2 : 0ull;
              m1 = lo ? m1 : m2;
              rem = (uint32_t)__builtin_amdgcn_readlane((int)(lo ? rw0 : rw1), l);
              wbase = 32 * ((lo ? 0 : 64) + l);
            }
            const int bit = __builtin_ctz(rem);
            rem &= rem - 1u;
            return (wbase + bit) | (QM << 14);
          };
          // Every barrier below is preceded by an explicit wait for all of
          // this wave's outstanding copies: the copy into one stage is issued
          // before the other stage's step and consumed after it. The loop is
          // rotated so that no copy is in flight across its back-edge and each
          // copy sits in the same block as the step after it (the copy past a
          // run's end is an empty one): the compiler's own wait insertion then
          // sees that the step's reads of one stage do not touch the other
          // (with a copy in flight at the loop head it waited for that copy
          // before every step on stage A). Runs longer than kLongRun entries
          // (dense-like pairs) still wait for the stage-B copy before the
          // stage-A step: overlapping every copy there measured 6% slower on
          // dense calls and 3% slower on a layer with diffuse heads, while it
          // pays on the short runs of sparse pairs.
          const bool waitb = run_len[QM == 3 ? 0 : QM == 1 ? 1 : 2] > kLongRun;
          int eA = next();
          int eB = eA >= 0 ? next() : -1;
          if (eA >= 0) dma(stA, eA);
          __builtin_amdgcn_s_waitcnt(0);
          __syncthreads();  // the first tile is in LDS
          while (eA >= 0) {
            // stage A holds entry eA; nothing in flight
            dma(stB, eB);
            if (waitb) __builtin_amdgcn_s_waitcnt(kVmcnt0);
            compute(stA, eA, std::false_type{}, qmask, [] {});
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();  // stage B's tile has landed; nobody reads stage A any more
            if (eB < 0) break;
            eA = next();
            dma(stA, eA);
            compute(stB, eB, std::false_type{}, qmask, [] {});
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();  // stage A's tile has landed; nobody reads stage B any more
            eB = eA >= 0 ? next() : -1;
          }
        };
        run(kBoth{});
        run(kFirst{});
        run(kSecond{});
        if (RC) {
          // Pooled tiles in turn. A tile whose key blocks both rows keep holds
          // only masked pooled keys (all of them, at tau = +inf) and is passed
          // over, the same decision in every thread (kept bits in LDS), so the
          // barriers stay matched. The next tile's key parts are copied once
          // every wave is past this tile's score products (they land during
          // its O^T products), its values once every wave is past this tile's
          // O^T products (they land during the next score products).
          auto needed = [&](int c) -> bool {
            const int nv = min(kBlk, Nk - c * kBlk);
            const uint64_t valid = nv >= 64 ? ~0ull : ((1ull << nv) - 1ull);
            const uint64_t ka = (uint64_t)sm.kbits[gA][2 * c] | ((uint64_t)sm.kbits[gA][2 * c + 1] << 32);
            const uint64_t kb = hasB ? ((uint64_t)sm.kbits[gA + 1][2 * c] | ((uint64_t)sm.kbits[gA + 1][2 * c + 1] << 32))
                                     : valid;
            return (valid & ~ka) != 0 || (valid & ~kb) != 0;
          };
          auto next_tile = [&](int c) {
            while (c < npool && !needed(c)) ++c;
            return c;
          };
          // s_waitcnt operand: all but the last value copy's loads (this
          // wave's loads complete in issue order)
          constexpr int kWaitKeys = kVmcnt0 | (GM::NCH / 4);
          int c = next_tile(0);
          dma_pooled_keys(c);
          dma_pooled_vals(c);
          // (the barriers below wait for LDS work only: each wave first waits
          // explicitly for the copies the next step reads)
          // (the next tile is looked up where no copy is in flight: the
          // compiler would otherwise wait for the copies before its LDS reads)
          while (c < npool) {
            __builtin_amdgcn_s_waitcnt(kWaitKeys);
            lds_barrier();  // tile c's key parts are in LDS
            int cn = npool;
            compute(stA, c, std::true_type{}, kBoth{}, [&] {
              __builtin_amdgcn_s_waitcnt(0);
              lds_barrier();  // tile c's values are in LDS; nobody reads its key parts any more
              cn = next_tile(c + 1);
              dma_pooled_keys(cn);
            });
            lds_barrier();  // nobody reads tile c's values any more
            dma_pooled_vals(cn);
            c = cn;
          }
          __builtin_amdgcn_s_waitcnt(0);  // the empty copies past the last tile
        }
      }

      // After the group's last pair the next ticket is drawn, so its round
      // trip overlaps the fold below (it is resolved before this wave's
      // stores); drawing it earlier would tie an item to this workgroup while
      // it may still spend long on this one, which others could have taken.
      unsigned next_ticket = 0;
      if (lastpair && tid == 0 && !p.static_grid) next_ticket = ticket();

      // ---- 4. fold exact and corrected terms, normalise, store ----
      {
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          const int gm = gA + qt;  // query tile qt holds rows of the pair's block qt
          const float M2 = sm.M[gm] * kLog2e;
          const float cden = sm.cden[gm];
          // with no correction mass (exact-only, the per-row mode, every block
          // kept, or every skipped weight zero) the exact state alone is
          // normalised: a common maximum with M2 could underflow it to zero
          const bool cm = corr && cden > 0.f;
          const float lt = lsum[qt][0];
          const float mf = cm ? fmaxf(m[qt], M2) : m[qt];
          const float fa = __builtin_amdgcn_exp2f(m[qt] - mf);
          const float fc = cm ? __builtin_amdgcn_exp2f(M2 - mf) : 0.f;
          const float inv = 1.f / (lt * fa + cden * fc);
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) {
            const int c = 16 * dt + 4 * g16;
            accO[qt][dt][0] = (accO[qt][dt][0] * fa + sm.cnum[gm][c + 0] * fc) * inv;
            accO[qt][dt][1] = (accO[qt][dt][1] * fa + sm.cnum[gm][c + 1] * fc) * inv;
            accO[qt][dt][2] = (accO[qt][dt][2] * fa + sm.cnum[gm][c + 2] * fc) * inv;
            accO[qt][dt][3] = (accO[qt][dt][3] * fa + sm.cnum[gm][c + 3] * fc) * inv;
          }
        }
        // the next item, resolved before this wave's stores, so that waiting
        // for the ticket never waits for them
        if (lastpair && tid == 0) {
          int pr2 = -1;
          sm.item = p.static_grid ? -1 : take(next_ticket, pr2);
          sm.pair = pr2;
        }
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          const int row = qrow0 + c16;
          if (row < (qt ? nB : nA)) {
            const size_t orow = hoff + (size_t)((qA + qt) * kBlk + row) * D;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
              const int c = 16 * dt + 4 * g16;
              const f32x4 o = accO[qt][dt];
              if (p.out_bf16)
                *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + orow + c) =
                    make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
              else
                *reinterpret_cast<float4*>(static_cast<float*>(p.out) + orow + c) = make_float4(o[0], o[1], o[2], o[3]);
            }
          }
        }
      }

      lds_barrier();  // LDS is rewritten by the next pair or item (output stores may still be in flight)
    }
    }  // !RO
  }
  if (p.static_grid) return;

  // Each workgroup adds its stats once; the last one to finish publishes
  // them and leaves the header clean (zero tickets, zero counters) for the
  // next call on this workspace.
  if (tid == 0) {
    unsigned long long* acc64 = reinterpret_cast<unsigned long long*>(p.hdr);
    if (p.stats != nullptr && sm.st64[1] != 0) {
      atomicAdd(acc64 + kHdrKept / 2, sm.st64[0]);
      atomicAdd(acc64 + kHdrTotal / 2, sm.st64[1]);
      atomicAdd(acc64 + kHdrPairs / 2, sm.st64[2]);
      atomicMin(p.hdr + kHdrMin, sm.st32[0]);
      atomicMax(p.hdr + kHdrMax, sm.st32[1]);
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

int forward_items(int BH, int Nq, int G) { return BH * ((Nq + G - 1) / G); }

template <int D, int G, bool RC, bool RO>
static hipError_t launch_dg(const FwdParams& p, hipStream_t stream) {
  // per-device CU count and occupancy
  static std::mutex mu;
  static int cus[64] = {0};
  static int occ_cache[64] = {0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  int grid_per_cu = 0, ncu = 0;
  {
    std::lock_guard<std::mutex> lock(mu);
    if (cus[dev] == 0) {
      int n = 0;
      e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
      if (e != hipSuccess) return e;
      cus[dev] = n;
    }
    if (occ_cache[dev] == 0) {
      int occ = 0;
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, reinterpret_cast<const void*>(&fwd_kernel<D, G, RC, RO>),
                                                       kThreads, 0);
      if (e != hipSuccess) return e;
      occ_cache[dev] = occ < 1 ? 1 : occ;
    }
    ncu = cus[dev];
    grid_per_cu = occ_cache[dev];
  }
  const int grid = p.static_grid ? p.nitems : (int)std::min<long long>((long long)ncu * grid_per_cu, p.nitems);
  hipLaunchKernelGGL((fwd_kernel<D, G, RC, RO>), dim3(grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <int D, bool RC>
static hipError_t launch_d(const FwdParams& p, hipStream_t stream) {
  switch (p.group) {
    case 16:  // (the routing-only kernel runs groups of at most four)
      return p.route_only ? hipErrorInvalidValue : launch_dg<D, 16, RC, false>(p, stream);
    case 8: return p.route_only ? launch_dg<D, 8, false, true>(p, stream) : launch_dg<D, 8, RC, false>(p, stream);
    case 6:  // (likewise)
      return p.route_only ? hipErrorInvalidValue : launch_dg<D, 6, RC, false>(p, stream);
    case 4: return p.route_only ? launch_dg<D, 4, false, true>(p, stream) : launch_dg<D, 4, RC, false>(p, stream);
    default: return p.route_only ? launch_dg<D, 2, false, true>(p, stream) : launch_dg<D, 2, RC, false>(p, stream);
  }
}

hipError_t launch_forward(const FwdParams& p, int d, hipStream_t stream) {
  if (p.row_corr) return d == 128 ? launch_d<128, true>(p, stream) : launch_d<64, true>(p, stream);
  return d == 128 ? launch_d<128, false>(p, stream) : launch_d<64, false>(p, stream);
}

}  // namespace sol
