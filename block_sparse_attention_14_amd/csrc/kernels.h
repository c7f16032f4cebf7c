// Internal launch interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sol_attn.h"

namespace sol {

// Words at the start of the caller's workspace. The pooling step zeroes them;
// the fused kernel's last workgroup publishes the stats and zeroes them again,
// so a workspace is always clean between calls.
enum {
  kHdrKept = 0,         // u64 kept block pairs
  kHdrTotal = 2,        // u64 block pairs
  kHdrPairs = 4,        // u64 kept query-key pairs
  kHdrMin = 6,          // u32 min kept per query block
  kHdrMax = 7,          // u32 max kept per query block
  kHdrDone = 8,         // workgroups finished
  kHdrQueue = 32,       // ticket counter of queue x at word kHdrQueue + 32 x (own 128-byte line)
  kQueues = 8,          // one queue per XCD
  kHdrWords = kHdrQueue + 32 * kQueues
};

// Queue x owns the items (or, with an order, the ranks) [queue_begin(x),
// queue_begin(x + 1)): a contiguous, head-major range, so the workgroups of one
// XCD share the pooled keys and values of one or two heads in their L2.
__host__ __device__ inline int queue_begin(int x, int nitems) {
  return (int)(((long long)x * nitems) / kQueues);
}

// Longest head (in key blocks) that a work item of eight or sixteen query
// blocks supports: its kept bits must fit the workgroup's LDS.
constexpr int kMaxKeyBlocksG8 = 2048;

struct FwdParams {
  const uint16_t* q;     // bf16 [BH][N][d]
  const uint16_t* k;     // bf16 [BH][N][d]
  const uint16_t* v;     // bf16 [BH][N][d]
  void* out;             // [BH][N][d]: fp32, or bf16 when out_bf16
  const float* kpool;    // fp32 [BH][Nk][d]
  const float* vmean;    // fp32 [BH][Nk][d]
  const unsigned* units;  // nullable: a plan's work units (launch_plan), queue x's at queue_begin(x) * group / 2
  const unsigned* plan_items;  // with units: [0] the item count the plan was made for, [8 + x] queue x's units
  unsigned* hdr;         // workspace header (kHdr*), clean on entry
  sol_attn_stats* stats; // nullable, written by the last workgroup
  uint32_t* bitmap;      // nullable, [BH][Nq][nwords]
  int N, Nq, Nk, nitems, nwords;  // nitems = forward_items(BH, Nq, group)
  int group;             // query blocks per work item: 2, 4, 6, 8 or 16
  int split_n;           // items per queue handed out pair by pair (0: none)
  int ngroups;           // work items per head, ceil(Nq / group)
  int route_only;        // stop after routing (the kept-block bitmap is the only output)
  int static_grid;       // one workgroup per item, no queues, no header, no stats (route_only)
  int rule;              // SOL_ROUTE_ROWMAX or SOL_ROUTE_GAUSS
  float tau;             // ROWMAX: >= 0, may be +inf
  float beta;            // GAUSS: standardized cutoff, finite
  int sink_lo, sink_hi;  // key blocks [sink_lo, sink_hi) are always kept
  float proxy_scale;     // 1/sqrt(d)
  float scale_log2;      // log2(e)/sqrt(d)
  int exact_only;        // skipped blocks dropped instead of corrected
  int row_corr;          // per-row (token-to-block) correction over the pooled tiles below
  int out_bf16;          // store the output rounded to bf16
  const uint16_t* khi16;   // bf16 pooled keys, first part, tiled (Planes kh)
  const uint16_t* klo16;   // bf16 pooled keys, second part, tiled (Planes km)
  const uint16_t* klo2;    // bf16 pooled keys, third part, tiled (Planes kl)
  const uint16_t* vt;      // bf16 pooled values, tiled (Planes vt)
  int Nkp;                 // key blocks per head in the tiled planes: Nk rounded up to 64
  const uint16_t* vbar16;  // bf16 [BH][Nk][d] pooled values (row_corr)
  const float* qpool;      // fp32 [BH][Nq][d] pooled queries
  const float* kstats;     // fp32 [BH][2][d]: mean and variance of the pooled keys (GAUSS_DIAG)
  const float* kmom;       // fp32 [BH][d + 1][d]: mean, then covariance rows of the pooled keys (GAUSS)
};

// Up to three bf16 [BH][N][d] tensors pooled per 64-token block into fp32
// [BH][Nk][d] means.
// The fused kernel's routing planes (layout in pool.hip), written by the
// pooling pre-pass.
struct Planes {
  uint16_t* kh;  // bf16 pooled keys, three parts, [BH][Nkp][d] in 16-block operand tiles
  uint16_t* km;
  uint16_t* kl;
  uint16_t* vt;    // bf16 pooled values, [BH][Nkp][d] in 16-block operand tiles (null: none)
  uint16_t* vrow;  // bf16 pooled values [BH][Nk][d], row-major (null: none)
  const float* kpool;  // the caller's pooled keys (kRoleKeysFromPool)
  const float* vmean;  // the caller's pooled values (kRoleValuesFromPool)
  int Nkp;             // key blocks per head in the tiled planes: Nk rounded up to 64
};
// What a tensor's workgroups write besides its means: the key planes from
// their own means (the tensor is k), the value planes likewise (v), or both
// kinds from the caller's pooled tensors (given to the workgroups of q).
constexpr int kRoleKeys = 1, kRoleValues = 2, kRoleKeysFromPool = 4, kRoleValuesFromPool = 8;

struct PoolSet {
  const uint16_t* src[3];
  float* dst[3];
  int role[3] = {0, 0, 0};
  int n;
  Planes planes = {};
};

// Pools the tensors of `set`; when `hdr` is non-null, also resets the
// workspace header words.
hipError_t launch_pool(const PoolSet& set, int BH, int N, int Nk, int d, unsigned* hdr, hipStream_t stream);

// Routing operand planes from the fp32 pooled keys and values (pool.hip):

// stats[bh][0][c] = mean_j kpool[bh][j][c], stats[bh][1][c] = population
// variance over j (two passes), one workgroup per head.
hipError_t launch_kstats(const float* kpool, float* stats, int BH, int Nk, int d, hipStream_t stream);

// mom[bh][0][c] = m_c = mean_j kpool[bh][j][c]; mom[bh][1 + a][b] = population
// covariance mean_j (kpool[j][a] - m_a)(kpool[j][b] - m_b) (mean first, then
// the centred products).
hipError_t launch_kmom(const float* kpool, float* mom, int BH, int Nk, int d, hipStream_t stream);

// Resets the workspace header words (one small kernel).
hipError_t launch_reset(unsigned* hdr, hipStream_t stream);

// Per-pair cost estimates (union of the kept sets of each pair of query
// blocks, from sampled query means) and the order of each queue's range of
// items of `group` query blocks (an item costs the sum over its pairs):
// head-major, then its last third heaviest first.
// perm[rank] = item, with rank and item in the same queue range (scratch);
// the queue's work units (an item, or one pair of an item whose estimated
// cost reaches split_cost: item | (pair + 1) << 28) at units[queue_begin(x)
// * group / 2 ...]; plan_items[0] = the number of items the order is for,
// plan_items[8 + x] = the number of units of queue x.
hipError_t launch_plan(const uint16_t* q, const float* kpool, unsigned* cost, unsigned* perm, unsigned* units,
                       unsigned* plan_items, int BH, int N, int Nq, int Nk, int d, float tau, float proxy_scale,
                       int group, unsigned split_cost, hipStream_t stream);

// One unit per item, each queue in sequence (the order of a plan that does
// not sort), with the same plan_items words.
hipError_t launch_identity_order(unsigned* units, unsigned* plan_items, int nitems, int group, hipStream_t stream);

// The fused routing + exact + correction kernel (persistent grid).
hipError_t launch_forward(const FwdParams& p, int d, hipStream_t stream);

// The top-k / top-p mask builders (masks.hip).
// map[bh][i][j] = qpool_i . kpool_j * scale (fp32, written to device memory).
hipError_t launch_proxy_map(const float* qpool, const float* kpool, float* map, int BH, int Nq, int Nk, int d,
                            float scale, hipStream_t stream);
// Per-row sort of the map; mode 0 keeps the top `topk`, mode 1 the top-p prefix.
hipError_t launch_sort_mask(const float* map, uint32_t* bitmap, int BH, int Nq, int Nk, int topk, float topp,
                            int mode, hipStream_t stream);

// Number of work items (groups of `group` query blocks) of the fused kernel.
int forward_items(int BH, int Nq, int group);

}  // namespace sol
