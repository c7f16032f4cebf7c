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

struct FwdParams {
  const uint16_t* q;     // bf16 [BH][N][d]
  const uint16_t* k;     // bf16 [BH][N][d]
  const uint16_t* v;     // bf16 [BH][N][d]
  void* out;             // [BH][N][d]: fp32, or bf16 when out_bf16
  const float* kpool;    // fp32 [BH][Nk][d]
  const float* vmean;    // fp32 [BH][Nk][d]
  const unsigned* perm;  // nullable: rank -> item, within each queue's range
  unsigned* hdr;         // workspace header (kHdr*), clean on entry
  sol_attn_stats* stats; // nullable, written by the last workgroup
  uint32_t* bitmap;      // nullable, [BH][Nq][nwords]
  int N, Nq, Nk, nitems, nwords;  // nitems = forward_items(BH, Nq)
  int rule;              // SOL_ROUTE_ROWMAX or SOL_ROUTE_GAUSS
  float tau;             // ROWMAX: >= 0, may be +inf
  float beta;            // GAUSS: standardized cutoff, finite
  int sink_lo, sink_hi;  // key blocks [sink_lo, sink_hi) are always kept
  float proxy_scale;     // 1/sqrt(d)
  float scale_log2;      // log2(e)/sqrt(d)
  int exact_only;        // skipped blocks dropped instead of corrected
  int row_corr;          // per-row (token-to-block) correction over the pooled tiles below
  int out_bf16;          // store the output rounded to bf16
  const uint16_t* khi16;   // bf16 [BH][Nk][d] pooled keys, high part (row_corr)
  const uint16_t* klo16;   // bf16 [BH][Nk][d] pooled keys, the remainder (row_corr)
  const uint16_t* vbar16;  // bf16 [BH][Nk][d] pooled values (row_corr)
  const float* kstats;     // fp32 [BH][2][d]: mean and variance of the pooled keys (GAUSS_DIAG)
};

// Up to three bf16 [BH][N][d] tensors pooled per 64-token block into fp32
// [BH][Nk][d] means.
struct PoolSet {
  const uint16_t* src[3];
  float* dst[3];
  int n;
};

// Pools the tensors of `set`; when `hdr` is non-null, also resets the
// workspace header words.
hipError_t launch_pool(const PoolSet& set, int BH, int N, int Nk, int d, unsigned* hdr, hipStream_t stream);

// a = a_hi + a_lo in two bf16 parts (each rounded to nearest even; the pair
// carries about 16 significant bits) and b16 = bf16(b), for n values each.
hipError_t launch_to_bf16(const float* a, uint16_t* a_hi, uint16_t* a_lo, const float* b, uint16_t* b16, size_t n,
                          hipStream_t stream);

// stats[bh][0][c] = mean_j kpool[bh][j][c], stats[bh][1][c] = population
// variance over j (two passes), one workgroup per head.
hipError_t launch_kstats(const float* kpool, float* stats, int BH, int Nk, int d, hipStream_t stream);

// Resets the workspace header words (one small kernel).
hipError_t launch_reset(unsigned* hdr, hipStream_t stream);

// Per-item cost estimates (union of the kept sets of each pair of query
// blocks, from sampled query means) and the order of each queue's range:
// head-major, then its last third heaviest first.
// perm[rank] = item, with rank and item in the same queue range.
hipError_t launch_plan(const uint16_t* q, const float* kpool, unsigned* cost, unsigned* perm, int BH, int N, int Nq,
                       int Nk, int d, float tau, float proxy_scale, hipStream_t stream);

// perm[i] = i for every item (the order of a plan that does not sort).
hipError_t launch_identity_order(unsigned* perm, int nitems, hipStream_t stream);

// The fused routing + exact + correction kernel (persistent grid).
hipError_t launch_forward(const FwdParams& p, int d, hipStream_t stream);

// The mask builders (masks.hip).
struct MaskParams {
  const uint16_t* q;     // bf16 [BH][N][d]
  const float* kpool;    // fp32 [BH][Nk][d]
  uint32_t* bitmap;      // [BH][Nq][nwords]
  int N, Nq, Nk, nwords;
  int rule;              // SOL_ROUTE_*
  float tau, beta, proxy_scale;
  int sink_lo, sink_hi;
};
// On-chip threshold routing, one workgroup per pair of query blocks.
hipError_t launch_mask_threshold(const MaskParams& p, int d, int BH, hipStream_t stream);
// map[bh][i][j] = qpool_i . kpool_j * scale (fp32, written to device memory).
hipError_t launch_proxy_map(const float* qpool, const float* kpool, float* map, int BH, int Nq, int Nk, int d,
                            float scale, hipStream_t stream);
// Per-row sort of the map; mode 0 keeps the top `topk`, mode 1 the top-p prefix.
hipError_t launch_sort_mask(const float* map, uint32_t* bitmap, int BH, int Nq, int Nk, int topk, float topp,
                            int mode, hipStream_t stream);

// Dynamic LDS bytes the fused kernel needs for the kept list of Nk blocks.
size_t forward_dynamic_lds(int Nk);

// Number of work items (pairs of query blocks) of the fused kernel.
int forward_items(int BH, int Nq);

// Largest Nk whose two fp32 routing rows fit the kernel's LDS tile buffer.
int forward_max_blocks(int d);

}  // namespace sol
