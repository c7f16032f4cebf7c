// Internal launch interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sol_attn.h"

namespace sol {

// Work-queue words at the start of the caller's workspace.
enum { kQueueTicket = 0, kQueueWords = 4 };

struct FwdParams {
  const uint16_t* q;     // bf16 [BH][N][d]
  const uint16_t* k;     // bf16 [BH][N][d]
  const uint16_t* v;     // bf16 [BH][N][d]
  float* out;            // fp32 [BH][N][d]
  const float* kpool;    // fp32 [BH][Nk][d]
  const float* vmean;    // fp32 [BH][Nk][d]
  unsigned* queue;       // ticket counter, zero on entry
  sol_attn_stats* stats; // nullable, reset before the launch
  uint32_t* bitmap;      // nullable, [BH][Nq][nwords]
  int N, Nq, Nk, nitems, nwords;  // nitems = forward_items(BH, Nq)
  float tau;             // >= 0, may be +inf
  float proxy_scale;     // 1/sqrt(d)
  float scale_log2;      // log2(e)/sqrt(d)
  int exact_only;        // skipped blocks dropped instead of corrected
};

// Pools k and v per 64-token block; when `queue` is non-null, also clears the
// forward's queue counter and stats (so the fused kernel that follows on the
// same stream starts from zero).
hipError_t launch_pool(const uint16_t* k, const uint16_t* v, float* kpool, float* vmean,
                       int BH, int N, int Nk, int d, unsigned* queue, sol_attn_stats* stats,
                       hipStream_t stream);

// Clears the queue counter and stats without pooling.
hipError_t launch_reset(unsigned* queue, sol_attn_stats* stats, hipStream_t stream);

// The fused routing + exact + correction kernel (persistent grid).
hipError_t launch_forward(const FwdParams& p, int d, hipStream_t stream);

// Dynamic LDS bytes the fused kernel needs for the kept list of Nk blocks.
size_t forward_dynamic_lds(int Nk);

// Number of work items (pairs of query blocks) of the fused kernel.
int forward_items(int BH, int Nq);

// Largest Nk whose two fp32 routing rows fit the kernel's LDS tile buffer.
int forward_max_blocks(int d);

}  // namespace sol
